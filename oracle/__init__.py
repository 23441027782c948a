"""fp64 CPU oracle for the FluxBin LUT GEMV -- test infrastructure only.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package.  It shares no code with the GPU library.
"""
