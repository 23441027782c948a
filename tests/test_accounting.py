"""Host-side byte and operation accounting, pinned to the pages' printed storage numbers."""
import json
import os

import pytest

from binary_basis_lut_amd import accounting as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_pages_abw_numbers():
    fx = json.load(open(os.path.join(GOLDEN, "pages_storage_numbers.json")))
    for row in fx["abw_bits"]:
        got = A.pages_abw_bits(row["kb"], row["ks"], row["group"], row["salient_per_group"])
        assert abs(got - row["printed"]) <= 0.005 + 1e-9, row  # printed to two decimals


def test_pages_shared_memory_numbers():
    fx = json.load(open(os.path.join(GOLDEN, "pages_storage_numbers.json")))
    for row in fx["shared_memory_kib"]:
        kib = A.pages_shared_memory_bytes(row["mu"], row["batch"], row["kb"], row["mtile"], row["ktile"]) / 1024
        if row["relation"] == "equal":
            assert kib == row["printed"]
        else:
            assert kib <= row["printed"]


def test_weight_bytes_closed_form():
    # q_proj shape: 2 global bases of 4096x4096 bits, one salient basis of 4096x256 bits
    n = k = 4096
    s = 256
    expect = 2 * n * k // 8 + n * s // 8 + 2 * 3 * n + 2 * (2 * k + s) + 4 * s
    assert A.weight_bytes(n, k, s, 2, 1) == expect == 4_367_872
    # ragged widths round each row up to whole 32-bit words
    assert A.packed_sign_bytes(3, 33, 0, 1, 0) == 3 * 2 * 4


def test_lookup_and_table_counts():
    assert A.lookups(4096, 4096, 256, 2, 1, 4, 1) == 4096 * (2 * 1024 + 64)
    assert A.table_entries(4096, 256, 2, 1, 4, 2) == 2 * 16 * (2 * 1024 + 64)
    assert A.lookups(10, 10, 0, 1, 0, 8, 3) == 3 * 10 * 2
