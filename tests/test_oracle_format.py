"""Pins for the oracle's number formats, bit packing and record layout.

Each check compares the oracle with something other than itself: a library
routine (numpy's float16 and packbits), hand-derived fixtures under
tests/golden/, or the record-size figure printed on the gmlx page.
"""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def test_half_conversion_matches_numpy():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.integers(-9, 5, 4000),
        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -24, 2.0 ** -25,
         2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 2.0 ** -14, 1.0 + 2.0 ** -11,
         1.0 + 3 * 2.0 ** -11, 2048.0 + 1.0, 2048.0 + 3.0],
    ])
    mine = oracle.double_to_half(x)
    ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(mine, ref)
    back = oracle.half_to_double(ref)
    assert np.array_equal(back[np.isfinite(back)],
                          ref.view(np.float16).astype(np.float64)[np.isfinite(back)])


def test_all_half_patterns_decode_like_numpy():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = oracle.half_to_double(bits)
    ref = bits.view(np.float16).astype(np.float64)
    finite = np.isfinite(ref)
    assert np.array_equal(mine[finite], ref[finite])
    assert np.array_equal(np.isnan(mine), np.isnan(ref))


@pytest.mark.parametrize("line", _rows("pack_examples.txt"))
def test_pack_golden(line):
    b, codes, packed = [s.strip() for s in line.split("|")]
    b = int(b)
    codes = np.array([int(c) for c in codes.split()], np.uint8)
    packed = np.array([int(x, 16) for x in packed.split()], np.uint8)
    assert np.array_equal(oracle.pack(codes, b), packed)
    assert np.array_equal(oracle.unpack(packed, len(codes), b), codes)


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
def test_pack_matches_numpy_packbits(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, 1000).astype(np.uint8)
    # expand every code into its bits, LSB first, and let numpy pack them
    bitarr = ((codes[:, None] >> np.arange(bits)) & 1).astype(np.uint8).ravel()
    ref = np.packbits(bitarr, bitorder="little")
    assert np.array_equal(oracle.pack(codes, bits), ref)
    assert np.array_equal(oracle.unpack(ref, len(codes), bits), codes)


@pytest.mark.parametrize("line", _rows("record_sizes.txt"))
def test_record_size_and_page_figure(line):
    dtb, per_tok, pct = [s.strip() for s in line.split("|")]
    D, T, b = (int(v) for v in dtb.split())
    rb = oracle.record_bytes(T, D, b)
    assert rb == int(per_tok) * T
    assert abs(100.0 * rb / (2 * D * T) - float(pct)) < 0.01


def test_six_bit_record_is_about_forty_percent():
    # gmlx "The two schemes": at 6 bits a record takes about 40% of fp16.
    frac = oracle.record_bytes(128, 128, 6) / (128 * 128 * 2)
    assert 0.38 < frac < 0.42


def test_record_fields_roundtrip():
    rng = np.random.default_rng(3)
    T, D, b = 64, 128, 4
    x = rng.standard_normal((T, D)).astype(np.float16)
    for cm in (False, True):
        rec, u, lc, lr = oracle.quantize_record(x.view(np.uint16), b, 6, channel_major=cm)
        codes, S, Z, C = oracle.split_record(rec, T, D, b, channel_major=cm)
        exp = np.clip(np.rint(u), 0, 15).astype(np.uint8)
        assert np.array_equal(codes, exp)
        assert np.allclose(C, np.exp(lc), rtol=1e-3)


@pytest.mark.parametrize("T,bits", [(128, 2), (128, 6), (64, 4), (128, 5)])
def test_value_codes_channel_major_in_64_token_blocks(T, bits):
    """Value records keep their codes channel-major in blocks of 64 tokens:
    the code of token t, channel j is element (t // 64) * 64 * D + j * 64 +
    t % 64 of the LSB-first stream (a layout choice the pages leave open; it
    makes the codes of a 64-token block one contiguous run).  Read straight
    from the packed bits and compared with the same tile's key-order record."""
    D = 128
    rng = np.random.default_rng(T + bits)
    x = rng.standard_normal((T, D)).astype(np.float16).view(np.uint16)
    vrec, _, _, _ = oracle.quantize_record(x, bits, 6, channel_major=True)
    krec, _, _, _ = oracle.quantize_record(x, bits, 6, channel_major=False)
    flat = oracle.unpack(vrec[:T * D * bits // 8], T * D, bits)
    tok = oracle.unpack(krec[:T * D * bits // 8], T * D, bits).reshape(T, D)
    t, j = np.meshgrid(np.arange(T), np.arange(D), indexing="ij")
    assert np.array_equal(flat[(t // 64) * 64 * D + j * 64 + t % 64], tok)
    assert np.array_equal(vrec[T * D * bits // 8:], krec[T * D * bits // 8:])
