"""ctypes binding of libfluxbin.so (include/fluxbin.h): argument marshalling only.

Every function here has the name and argument order of the C entry point it
calls.  Array arguments may be torch CUDA tensors (their data pointers are
passed), raw integer device addresses, or None for NULL.  `stream` defaults to
torch's current stream.  A non-zero status raises FluxbinError.

The library must have been built (``python -m binary_basis_lut_amd.build`` or
``__graft_entry__.build()``); importing this module fails loudly otherwise.
There is no CPU fallback.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "_build" / "libfluxbin.so"
if not LIB_PATH.exists():
    raise ImportError(f"{LIB_PATH} is missing: build the HIP library first (binary_basis_lut_amd/build.py)")

_lib = ctypes.CDLL(str(LIB_PATH))

ABI_VERSION = 8

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
LAYOUT_ROWMAJOR, LAYOUT_TILED = 0, 1
TABLE_F32, TABLE_F16 = 0, 1
DT_I8, DT_F16, DT_BITS = 0, 1, 2

P = ctypes.c_void_p
I64 = ctypes.c_int64
I32 = ctypes.c_int32


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("abi_version", I32), ("g", I32), ("kb", I32), ("ks", I32),
        ("n", I64), ("k", I64), ("s", I64), ("max_batch", I64),
        ("bits_global", P), ("r_global", P), ("c_global", P),
        ("bits_sal", P), ("r_sal", P), ("c_sal", P), ("sal_idx", P),
        ("workspace", P), ("workspace_bytes", ctypes.c_size_t),
        ("chunks_per_block", I32), ("waves_per_block", I32),
        ("row_group", I32), ("sal_group", I32), ("table_precision", I32), ("layout", I32),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("rows_per_block", I32), ("chunks_per_block", I32), ("row_blocks", I32), ("splits", I32),
        ("total_chunks", I32), ("lds_bytes", I32), ("grid", I64), ("banked_tables", I32), ("table_chunks", I32),
        ("threads_per_block", I32),
    ]

    def as_dict(self):
        return {name: getattr(self, name) for name, _ in self._fields_}


class FluxbinError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.fluxbin_last_error().decode(errors="replace")
        super().__init__(f"{where}: {_lib.fluxbin_status_string(status).decode()} ({msg})")


def _decl(name, restype, argtypes):
    fn = getattr(_lib, name)
    fn.restype = restype
    fn.argtypes = argtypes
    return fn


_decl("fluxbin_abi_version", I32, [])
_decl("fluxbin_status_string", ctypes.c_char_p, [ctypes.c_int])
_decl("fluxbin_last_error", ctypes.c_char_p, [])
_decl("fluxbin_tiled_words", I64, [I64, I64])
_decl("fluxbin_pack", ctypes.c_int, [P, I64, I64, I64, I32, P, P, P])
_decl("fluxbin_relayout", ctypes.c_int, [P, I64, I64, I32, I32, P, P])
_decl("fluxbin_tiled_scale_elems", I64, [I64, I64, I64])
_decl("fluxbin_relayout_scales", ctypes.c_int, [P, I64, I64, I64, I32, I32, P, P])
_decl("fluxbin_vcm_gather", ctypes.c_int, [P, I64, P, I64, I64, I32, P, P])
_decl("fluxbin_workspace_size", ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.POINTER(ctypes.c_size_t)])
_decl("fluxbin_create", ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.POINTER(P)])
_decl("fluxbin_destroy", ctypes.c_int, [P])
_decl("fluxbin_get_plan", ctypes.c_int, [P, ctypes.POINTER(PlanInfo)])
_decl("fluxbin_plan_of", ctypes.c_int, [ctypes.POINTER(LayerDesc), ctypes.POINTER(PlanInfo)])
_decl("fluxbin_lut_size", ctypes.c_int, [P, I64, ctypes.POINTER(ctypes.c_size_t)])
_decl("fluxbin_build_lut", ctypes.c_int, [P, P, I64, P, P])
_decl("fluxbin_gemv", ctypes.c_int, [P, P, P, I64, P])
_decl("fluxbin_gemv_timed", ctypes.c_int, [P, P, P, I64, P, P, P])
_decl("fluxbin_gemv_static", ctypes.c_int, [P, P, P, I64, P])
_decl("fluxbin_reset_workspace", ctypes.c_int, [P, P])
_decl("fluxbin_dense_gemv_f16", ctypes.c_int, [P, I64, I64, P, P, I64, P])
_decl("fluxbin_probe_stream_read", ctypes.c_int, [P, I64, I32, I64, ctypes.c_uint32, P, P])
_decl("fluxbin_probe_empty", ctypes.c_int, [I64, I32, P])
_decl("fluxbin_probe_lds_lookup", ctypes.c_int, [I32, I32, I64, I32, ctypes.c_float, P, P])
_decl("fluxbin_probe_lds_lookup_banked", ctypes.c_int, [I32, I64, I32, ctypes.c_float, P, P])
_decl("fluxbin_decomp_workspace_size", ctypes.c_int, [I64, I64, I32, ctypes.POINTER(ctypes.c_size_t)])
_decl("fluxbin_decompose", ctypes.c_int, [P, I64, I64, I32, I32, P, P, P, P, P, P, P, P, ctypes.c_size_t, P])
_decl("fluxbin_decomp_row_scales", ctypes.c_int, [P, I64, I64, I32, I32, P, P, P, P, P, P, ctypes.c_size_t, P])
_decl("fluxbin_decomp_col_scales", ctypes.c_int, [P, I64, I64, I32, I32, P, P, P, P, P, ctypes.c_size_t, P])
_decl("fluxbin_decomp_signs", ctypes.c_int, [P, I64, I64, I32, P, P, P, P])
_decl("fluxbin_decomp_residual_signs", ctypes.c_int, [P, I64, I64, I32, I32, P, P, P, P, P])
_decl("fluxbin_decomp_error", ctypes.c_int, [P, I64, I64, I32, P, P, P, P, P, P, ctypes.c_size_t, P])

SYMBOLS = [
    "fluxbin_abi_version", "fluxbin_status_string", "fluxbin_last_error", "fluxbin_tiled_words", "fluxbin_pack",
    "fluxbin_relayout", "fluxbin_tiled_scale_elems", "fluxbin_relayout_scales", "fluxbin_vcm_gather",
    "fluxbin_workspace_size", "fluxbin_create", "fluxbin_destroy", "fluxbin_get_plan", "fluxbin_plan_of",
    "fluxbin_lut_size",
    "fluxbin_build_lut", "fluxbin_gemv", "fluxbin_gemv_timed", "fluxbin_gemv_static", "fluxbin_reset_workspace", "fluxbin_dense_gemv_f16",
    "fluxbin_probe_stream_read", "fluxbin_probe_empty", "fluxbin_probe_lds_lookup", "fluxbin_probe_lds_lookup_banked",
    "fluxbin_decomp_workspace_size",
    "fluxbin_decompose", "fluxbin_decomp_row_scales", "fluxbin_decomp_col_scales", "fluxbin_decomp_signs",
    "fluxbin_decomp_residual_signs", "fluxbin_decomp_error",
]


def _ptr(a):
    if a is None:
        return None
    if isinstance(a, int):
        return a
    return a.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(st, where):
    if st != OK:
        raise FluxbinError(st, where)


# ------------------------------------------------------------------ entry points

def fluxbin_abi_version() -> int:
    return int(_lib.fluxbin_abi_version())


def fluxbin_status_string(status: int) -> str:
    return _lib.fluxbin_status_string(status).decode()


def fluxbin_last_error() -> str:
    return _lib.fluxbin_last_error().decode(errors="replace")


def fluxbin_tiled_words(rows: int, cols: int) -> int:
    return int(_lib.fluxbin_tiled_words(rows, cols))


def fluxbin_pack(signs, rows, cols, ld, layout, packed, invalid_count=None, stream=None):
    _check(_lib.fluxbin_pack(_ptr(signs), rows, cols, ld, layout, _ptr(packed), _ptr(invalid_count),
                             _stream(stream)), "fluxbin_pack")


def fluxbin_relayout(src, rows, cols, src_layout, dst_layout, dst, stream=None):
    _check(_lib.fluxbin_relayout(_ptr(src), rows, cols, src_layout, dst_layout, _ptr(dst), _stream(stream)),
           "fluxbin_relayout")


def fluxbin_tiled_scale_elems(rows: int, groups: int, groups_per_chunk: int) -> int:
    return int(_lib.fluxbin_tiled_scale_elems(rows, groups, groups_per_chunk))


def fluxbin_relayout_scales(src, rows, groups, groups_per_chunk, src_layout, dst_layout, dst, stream=None):
    _check(_lib.fluxbin_relayout_scales(_ptr(src), rows, groups, groups_per_chunk, src_layout, dst_layout, _ptr(dst),
                                        _stream(stream)), "fluxbin_relayout_scales")


def fluxbin_vcm_gather(idx, s, src, rows, cols, dtype, dst, stream=None):
    _check(_lib.fluxbin_vcm_gather(_ptr(idx), s, _ptr(src), rows, cols, dtype, _ptr(dst), _stream(stream)),
           "fluxbin_vcm_gather")


def fluxbin_workspace_size(desc: LayerDesc) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.fluxbin_workspace_size(ctypes.byref(desc), ctypes.byref(out)), "fluxbin_workspace_size")
    return int(out.value)


def fluxbin_create(desc: LayerDesc) -> int:
    h = P()
    _check(_lib.fluxbin_create(ctypes.byref(desc), ctypes.byref(h)), "fluxbin_create")
    return int(h.value)


def fluxbin_destroy(handle) -> None:
    _check(_lib.fluxbin_destroy(handle), "fluxbin_destroy")


def fluxbin_get_plan(handle) -> dict:
    info = PlanInfo()
    _check(_lib.fluxbin_get_plan(handle, ctypes.byref(info)), "fluxbin_get_plan")
    return info.as_dict()


def fluxbin_plan_of(desc: LayerDesc) -> dict:
    info = PlanInfo()
    _check(_lib.fluxbin_plan_of(ctypes.byref(desc), ctypes.byref(info)), "fluxbin_plan_of")
    return info.as_dict()


def fluxbin_lut_size(handle, batch) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.fluxbin_lut_size(handle, batch, ctypes.byref(out)), "fluxbin_lut_size")
    return int(out.value)


def fluxbin_build_lut(handle, x, batch, lut, stream=None):
    _check(_lib.fluxbin_build_lut(handle, _ptr(x), batch, _ptr(lut), _stream(stream)), "fluxbin_build_lut")


def fluxbin_gemv(handle, x, y, batch, stream=None):
    _check(_lib.fluxbin_gemv(handle, _ptr(x), _ptr(y), batch, _stream(stream)), "fluxbin_gemv")


def fluxbin_gemv_static(handle, x, y, batch, stream=None):
    _check(_lib.fluxbin_gemv_static(handle, _ptr(x), _ptr(y), batch, _stream(stream)), "fluxbin_gemv_static")


def fluxbin_gemv_timed(handle, x, y, batch, start_event, stop_event, stream=None):
    """start_event / stop_event: torch.cuda.Event(enable_timing=True) objects (already created) or raw handles."""
    ev = lambda e: e if isinstance(e, int) else e.cuda_event
    _check(_lib.fluxbin_gemv_timed(handle, _ptr(x), _ptr(y), batch, _stream(stream), ev(start_event),
                                   ev(stop_event)), "fluxbin_gemv_timed")


def fluxbin_reset_workspace(handle, stream=None):
    _check(_lib.fluxbin_reset_workspace(handle, _stream(stream)), "fluxbin_reset_workspace")


def fluxbin_probe_stream_read(buf, nbytes, depth, workgroups, never, sink, stream=None):
    _check(_lib.fluxbin_probe_stream_read(_ptr(buf), nbytes, depth, workgroups, never, _ptr(sink), _stream(stream)),
           "fluxbin_probe_stream_read")


def fluxbin_probe_empty(workgroups, threads, stream=None):
    _check(_lib.fluxbin_probe_empty(workgroups, threads, _stream(stream)), "fluxbin_probe_empty")


def fluxbin_probe_lds_lookup(g, nb, workgroups, iters, never, sink, stream=None):
    _check(_lib.fluxbin_probe_lds_lookup(g, nb, workgroups, iters, never, _ptr(sink), _stream(stream)),
           "fluxbin_probe_lds_lookup")


def fluxbin_probe_lds_lookup_banked(region, workgroups, iters, never, sink, stream=None):
    _check(_lib.fluxbin_probe_lds_lookup_banked(region, workgroups, iters, never, _ptr(sink), _stream(stream)),
           "fluxbin_probe_lds_lookup_banked")


def fluxbin_dense_gemv_f16(w, n, k, x, y, batch, stream=None):
    _check(_lib.fluxbin_dense_gemv_f16(_ptr(w), n, k, _ptr(x), _ptr(y), batch, _stream(stream)),
           "fluxbin_dense_gemv_f16")


def fluxbin_decomp_workspace_size(n, k, kb) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.fluxbin_decomp_workspace_size(n, k, kb, ctypes.byref(out)), "fluxbin_decomp_workspace_size")
    return int(out.value)


def fluxbin_decompose(w, n, k, kb, iters, col_weight, bits, r16, c16, r64, c64, trace, workspace, workspace_bytes,
                      stream=None):
    _check(_lib.fluxbin_decompose(_ptr(w), n, k, kb, iters, _ptr(col_weight), _ptr(bits), _ptr(r16), _ptr(c16),
                                  _ptr(r64), _ptr(c64), _ptr(trace), _ptr(workspace), workspace_bytes,
                                  _stream(stream)), "fluxbin_decompose")


def fluxbin_decomp_row_scales(w, n, k, kb, basis, bits, r, c, col_weight, r_out, workspace, workspace_bytes,
                              stream=None):
    _check(_lib.fluxbin_decomp_row_scales(_ptr(w), n, k, kb, basis, _ptr(bits), _ptr(r), _ptr(c), _ptr(col_weight),
                                          _ptr(r_out), _ptr(workspace), workspace_bytes, _stream(stream)),
           "fluxbin_decomp_row_scales")


def fluxbin_decomp_col_scales(w, n, k, kb, basis, bits, r, c, c_out, workspace, workspace_bytes, stream=None):
    _check(_lib.fluxbin_decomp_col_scales(_ptr(w), n, k, kb, basis, _ptr(bits), _ptr(r), _ptr(c), _ptr(c_out),
                                          _ptr(workspace), workspace_bytes, _stream(stream)),
           "fluxbin_decomp_col_scales")


def fluxbin_decomp_signs(w, n, k, kb, r, c, bits_out, stream=None):
    _check(_lib.fluxbin_decomp_signs(_ptr(w), n, k, kb, _ptr(r), _ptr(c), _ptr(bits_out), _stream(stream)),
           "fluxbin_decomp_signs")


def fluxbin_decomp_residual_signs(w, n, k, kb, basis, bits, r, c, basis_bits_out, stream=None):
    _check(_lib.fluxbin_decomp_residual_signs(_ptr(w), n, k, kb, basis, _ptr(bits), _ptr(r), _ptr(c),
                                              _ptr(basis_bits_out), _stream(stream)), "fluxbin_decomp_residual_signs")


def fluxbin_decomp_error(w, n, k, kb, bits, r, c, col_weight, err_out, workspace, workspace_bytes, stream=None):
    _check(_lib.fluxbin_decomp_error(_ptr(w), n, k, kb, _ptr(bits), _ptr(r), _ptr(c), _ptr(col_weight),
                                     _ptr(err_out), _ptr(workspace), workspace_bytes, _stream(stream)),
           "fluxbin_decomp_error")


def raw_status(name: str, *args) -> int:
    """Call an entry point and return its status instead of raising (error-path tests)."""
    return int(getattr(_lib, name)(*args))


# ------------------------------------------------------------------ device-resident layer

class DeviceLayer:
    """Upload one synthetic layer (binary_basis_lut_amd.inputs.Layer) and create its handle.

    layout=LAYOUT_TILED (default): canonical sign words are copied to the
    device and converted to the tiled layout with fluxbin_relayout, block-wise
    row scales ([basis][n][groups]) to the tiled scale layout with
    fluxbin_relayout_scales.  layout=LAYOUT_ROWMAJOR: the canonical words and
    scales are passed as they are and fluxbin_create converts them into the
    workspace.  Scales, index and workspace are torch CUDA tensors owned by
    this object, which keeps them alive for the handle.
    """

    def __init__(self, layer, max_batch: int = 1, chunks_per_block: int = 0, waves_per_block: int = 0,
                 device="cuda", table_precision: int = TABLE_F32, layout: int = LAYOUT_TILED):
        import numpy as np
        import torch

        self.layer = layer
        self.max_batch = max_batch
        self.table_precision = table_precision
        self.layout = layout
        dev = torch.device(device)

        def up(a, dtype):
            return torch.from_numpy(np.ascontiguousarray(a).view(dtype)).to(dev)

        n, k, s = layer.n, layer.k, layer.s
        rowmajor = layout == LAYOUT_ROWMAJOR
        rgroup = int(getattr(layer, "row_group", 0) or 0)
        self.row_group = rgroup
        self.sal_group = int(getattr(layer, "sal_group", 0) or 0) if layer.ks else 0

        def tiled_bits(canon_np, bases, cols):
            if rowmajor:
                return up(canon_np, np.int32)
            tw = fluxbin_tiled_words(n, cols)
            out = torch.zeros(max(bases * tw, 4), dtype=torch.int32, device=dev)
            canon = up(canon_np, np.int32)
            for b in range(bases):
                fluxbin_relayout(canon[b], n, cols, LAYOUT_ROWMAJOR, LAYOUT_TILED, out[b * tw:(b + 1) * tw])
            return out

        def tiled_scales(r, bases, m):
            """[bases][n][groups] canonical -> concatenated tiled blocks (m groups per chunk)."""
            if rowmajor:
                return up(r, np.int16)
            groups = r.shape[2]
            te = fluxbin_tiled_scale_elems(n, groups, m)
            out = torch.zeros(max(bases * te, 8), dtype=torch.int16, device=dev)
            canon_r = up(r, np.int16)
            for b in range(bases):
                fluxbin_relayout_scales(canon_r[b], n, groups, m, LAYOUT_ROWMAJOR, LAYOUT_TILED,
                                        out[b * te:(b + 1) * te])
            return out

        self.bits_g = tiled_bits(layer.bits_g, layer.kb, k)
        self.r_g = tiled_scales(layer.r_g, layer.kb, 1) if rgroup else up(layer.r_g, np.int16)
        self.c_g = up(layer.c_g, np.int16)
        if layer.ks:
            self.bits_s = tiled_bits(layer.bits_s, layer.ks, s)
            self.r_s = (tiled_scales(layer.r_s, layer.ks, 128 // self.sal_group) if rgroup
                        else up(layer.r_s, np.int16))
            self.c_s = up(layer.c_s, np.int16)
            self.sal_idx = up(layer.sal_idx, np.int32)
        else:
            self.bits_s = self.r_s = self.c_s = self.sal_idx = None
        desc = self.make_desc(chunks_per_block, waves_per_block)
        ws = fluxbin_workspace_size(desc)
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev) if ws else None
        desc.workspace = _ptr(self.workspace)
        desc.workspace_bytes = ws
        self.desc = desc
        torch.cuda.synchronize()
        self.handle = fluxbin_create(desc)
        self.plan = fluxbin_get_plan(self.handle)

    def make_desc(self, chunks_per_block: int = 0, waves_per_block: int = 0) -> LayerDesc:
        L = self.layer
        d = LayerDesc()
        d.abi_version = ABI_VERSION
        d.g, d.kb, d.ks = L.g, L.kb, L.ks
        d.n, d.k, d.s, d.max_batch = L.n, L.k, L.s, self.max_batch
        d.bits_global, d.r_global, d.c_global = _ptr(self.bits_g), _ptr(self.r_g), _ptr(self.c_g)
        d.bits_sal, d.r_sal, d.c_sal, d.sal_idx = (_ptr(self.bits_s), _ptr(self.r_s), _ptr(self.c_s),
                                                   _ptr(self.sal_idx))
        d.chunks_per_block = chunks_per_block
        d.waves_per_block = waves_per_block
        d.row_group = self.row_group
        d.sal_group = self.sal_group
        d.table_precision = self.table_precision
        d.layout = self.layout
        return d

    def gemv(self, x, y, batch=None, stream=None):
        fluxbin_gemv(self.handle, x, y, x.shape[0] if batch is None else batch, stream)

    def reset_workspace(self, stream=None):
        fluxbin_reset_workspace(self.handle, stream)

    def close(self):
        if getattr(self, "handle", None):
            fluxbin_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
