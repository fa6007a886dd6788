"""Pins of the oracle's bit layout: hand-derived bytes, agreement of the
8-code word rule (packer) with the per-index read formulas (unpacker), the
bit-position statement of the row bitstream, and the blob layout."""
import numpy as np
import pytest

import oracle
from conftest import golden


def test_hand_derived_examples():
    for ex in golden("packing_examples.json")["examples"]:
        codes = np.array([ex["codes"]], dtype=np.uint8)
        assert oracle.pack_codes(codes, ex["bits"]).ravel().tolist() == ex["bytes"], ex
        got = oracle.unpack_codes(np.array([ex["bytes"]], dtype=np.uint8), ex["bits"], 8)
        assert got.ravel().tolist() == ex["codes"], ex


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_word_rule_agrees_with_per_index_formulas(bits):
    rng = np.random.default_rng(bits)
    b = oracle.storage_bits(bits)
    for k in (8, 128, 384, 1024):
        codes = rng.integers(0, 1 << b, size=(5, k), dtype=np.uint8)
        packed = oracle.pack_codes(codes, bits)
        assert packed.shape == (5, k * b // 8)
        assert np.array_equal(oracle.unpack_codes(packed, bits, k), codes)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_code_k_occupies_bits_kb_to_k1b(bits):
    codes = np.random.default_rng(10 + bits).integers(0, 1 << bits, size=(1, 256), dtype=np.uint8)
    row = oracle.pack_codes(codes, bits)[0]
    stream = int.from_bytes(row.tobytes(), "little")
    for k in range(256):
        assert (stream >> (k * bits)) & ((1 << bits) - 1) == codes[0, k]


def test_three_bit_last_code_stays_inside_its_row():
    codes = np.full((2, 128), 7, dtype=np.uint8)
    packed = oracle.pack_codes(codes, 3)
    for fill in (0x00, 0xFF):
        p = packed.copy()
        p[1, :] = fill
        assert oracle.unpack_codes(p[:1], 3, 128)[0, -1] == 7
        assert np.array_equal(oracle.unpack_codes(p, 3, 128)[0], codes[0])


@pytest.mark.parametrize("bits", [2, 3, 4, 5])
def test_blob_layout_and_length_check(bits):
    rng = np.random.default_rng(bits)
    rows, cols = 3, 200
    kpad, ng = 256, 2
    b = oracle.storage_bits(bits)
    codes = rng.integers(0, 1 << b, size=(rows, kpad), dtype=np.uint8)
    norms = rng.random((rows, ng)).astype(np.float16)
    blob = oracle.make_blob(oracle.pack_codes(codes, bits), norms)
    assert blob.size == oracle.blob_bytes(bits, 128, rows, cols)
    row_bytes = kpad * b // 8
    # norms follow the last packed row, one per (row, group), row-major, little-endian fp16
    tail = blob[rows * row_bytes:]
    assert tail.size == rows * ng * 2
    for r in range(rows):
        for g in range(ng):
            off = 2 * (r * ng + g)
            assert int(tail[off]) | (int(tail[off + 1]) << 8) == int(norms[r, g].view(np.uint16))
    packed, n = oracle.split_blob(blob, bits, rows, cols)
    assert np.array_equal(oracle.unpack_codes(packed, bits, kpad), codes)
    assert np.array_equal(n, norms)
    with pytest.raises(ValueError, match="Inconsistent CQ matrix length"):
        oracle.split_blob(blob[:-1], bits, rows, cols)


def test_pack_rejects_out_of_range_codes():
    with pytest.raises(ValueError):
        oracle.pack_codes(np.full((1, 8), 4, dtype=np.uint8), 2)
