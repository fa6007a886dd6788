"""Pins of the oracle's byte accounting against the figures the pages print."""
import pytest

import oracle
from conftest import golden


@pytest.mark.parametrize("bits,bpw", [(2, 2.125), (3, 3.125), (4, 4.125), (5, 2.125)])
def test_bits_per_weight(bits, bpw):
    assert oracle.bits_per_weight(bits) == bpw
    for rows, cols in [(1, 128), (512, 512), (7, 1024), (8192, 512)]:
        assert oracle.blob_bytes(bits, 128, rows, cols) * 8 == bpw * rows * cols


def test_needle2_accounting_table():
    g = golden("needle2_accounting.json")
    p2, p4, p16 = g["cq2"]["params"], g["cq4"]["params"], g["fp16"]["params"]
    # every CQ tensor in the archive has an input width that is a multiple of 128, so
    # the bytes of all tensors of one width equal those of one row of all their weights
    assert oracle.blob_bytes(2, g["group"], 1, p2) == g["cq2"]["blob_bytes"]
    assert oracle.blob_bytes(4, g["group"], 1, p4) == g["cq4"]["blob_bytes"]
    assert (p2 + p4) // g["group"] * 2 == g["norm_bytes"]
    assert p2 + p4 + p16 == g["total_numeric_params"]
    assert round((2 * p2 + 4 * p4) / (p2 + p4), 6) == g["code_bits_per_quantised_weight"]
    payload = g["cq2"]["blob_bytes"] + g["cq4"]["blob_bytes"] + g["fp16"]["blob_bytes"]
    assert round(payload * 8 / g["total_numeric_params"], 6) == g["numeric_payload_bpw"]
    assert round(g["file_bytes"] * 8 / g["total_numeric_params"], 6) == g["file_bpw"]
    assert oracle.bits_per_weight(2) == g["pure_cq2_bpw"]
    assert oracle.bits_per_weight(4) == g["pure_cq4_bpw"]


def test_tutorial_length_formula_with_padding():
    # inputPadded = ceil(in/group)*group; rowBytes = inputPadded*bits/8; norms out*inputPadded/group
    assert oracle.padded_cols(130) == 256
    assert oracle.blob_bytes(2, 128, 3, 130) == 3 * (256 * 2 // 8) + 3 * 2 * 2
    assert oracle.blob_bytes(3, 128, 3, 130) == 3 * (256 * 3 // 8) + 3 * 2 * 2
    # ternary rows are 2-bit crumbs: the length uses 2, not the marker 5
    assert oracle.blob_bytes(5, 128, 3, 130) == oracle.blob_bytes(2, 128, 3, 130)
    assert oracle.blob_bytes(2, 128, 0, 512) == 0
    assert oracle.blob_bytes(2, 128, 4, 0) == 0


def test_workload_sizes():
    assert oracle.blob_bytes(2, 128, 65536, 16384) == 285_212_672
    assert oracle.blob_bytes(3, 128, 65536, 16384) == 419_430_400
    assert oracle.blob_bytes(4, 128, 65536, 16384) == 553_648_128
    assert oracle.blob_bytes(5, 128, 65536, 16384) == 285_212_672
    assert oracle.blob_bytes(4, 128, 16384, 16384) == 138_412_032
    assert oracle.blob_bytes(3, 128, 16384, 16384) == 104_857_600
    assert oracle.blob_bytes(2, 128, 512, 512) == 69_632


def test_invalid_parameters():
    for args in [(0, 128, 1, 1), (6, 128, 1, 1), (2, 96, 1, 1), (2, 128, -1, 1)]:
        with pytest.raises(ValueError):
            oracle.blob_bytes(*args)
