"""Comparison of HIP results with the oracle, under the path's parity bar:

  codes      identical except for at most 1e-4 of the elements, each of which
             may differ by +-1 only where the oracle's pre-round value lies
             within 1e-3 of a rounding boundary (|frac(u) - 0.5| < 1e-3);
  scales     C and S within 1e-3 relative; Zp within 1e-3 * max(|Zp|, S);
  decode     per (sequence, query head): max_j |o - o_ref| <= 2e-3 * max_j |o_ref|,
             with the oracle run on the HIP path's own records.
"""
import numpy as np

import oracle

CODE_FRAC = 1e-4
BAND = 1e-3
SCALE_RTOL = 1e-3
DECODE_RTOL = 2e-3


class CodeStats:
    def __init__(self):
        self.n = 0
        self.diff = 0
        self.bad = []

    def frac(self):
        return self.diff / max(self.n, 1)


def compare_record(gpu_rec, x16, T, D, bits, n_iters, channel_major, stats, where=""):
    """Quantize the fp16 tile x16 with the oracle and compare with gpu_rec."""
    ref, u, _, _ = oracle.quantize_record(x16, bits, n_iters, channel_major=channel_major)
    gc, gS, gZ, gC = oracle.split_record(gpu_rec, T, D, bits, channel_major)
    rc, rS, rZ, rC = oracle.split_record(ref, T, D, bits, channel_major)
    assert np.all(np.abs(gC - rC) <= SCALE_RTOL * np.abs(rC)), f"{where}: column scales"
    assert np.all(np.abs(gS - rS) <= SCALE_RTOL * np.abs(rS)), f"{where}: token scales"
    assert np.all(np.abs(gZ - rZ) <= SCALE_RTOL * np.maximum(np.abs(rZ), rS)), f"{where}: zero-points"
    d = gc.astype(np.int32) - rc.astype(np.int32)
    nz = d != 0
    stats.n += d.size
    stats.diff += int(nz.sum())
    if nz.any():
        near = np.abs(np.abs(u - np.floor(u)) - 0.5) < BAND
        ok = (np.abs(d) <= 1) & near
        if not np.all(ok[nz]):
            idx = np.argwhere(nz & ~ok)[:5]
            stats.bad.append((where, idx.tolist(), [float(u[tuple(i)]) for i in idx],
                              [int(gc[tuple(i)]) for i in idx], [int(rc[tuple(i)]) for i in idx]))
    return ref


def assert_code_stats(stats):
    assert not stats.bad, f"codes differ away from a rounding boundary: {stats.bad[:3]}"
    assert stats.frac() <= CODE_FRAC, f"{stats.diff} of {stats.n} codes differ ({stats.frac():.2e})"


def decode_rel_err(out, ref):
    """max over rows of max|out - ref| / max|ref| (rows = (b, h))."""
    out = np.asarray(out, np.float64).reshape(-1, out.shape[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, ref.shape[-1])
    den = np.abs(ref).max(axis=1)
    num = np.abs(out - ref).max(axis=1)
    rel = np.where(den > 0, num / np.where(den > 0, den, 1), num)
    return float(rel.max()), int(rel.argmax())


def degenerate_tile(T, D, seed, zero_rows=9):
    """fp16 tile (uint16 bits, [T, D]) with exactly zero token rows and exactly
    zero channels after the rotation: every row is an integer combination of
    half of the +-1 sign patterns s_k(j) = (-1)^popcount(j & k) (the rows of
    the unnormalized Sylvester matrix, mutually orthogonal), so the rotated
    row is zero in every other channel; every zero_rows-th row is zero.  The
    entries are integers of magnitude at most 2 D, exact in fp16.

    Returns (bits, kept channels k)."""
    rng = np.random.default_rng(seed)
    keep = np.sort(rng.choice(D, D // 2, replace=False))
    j = np.arange(D)
    signs = np.array([1 - 2 * (np.unpackbits(np.array([k & jj for jj in j], np.uint16).view(np.uint8))
                                .reshape(D, 16).sum(1) & 1) for k in keep], np.int64)  # [D/2, D]
    coef = rng.integers(-4, 5, (T, D // 2))
    x = coef @ signs
    x[::zero_rows] = 0
    assert np.abs(x).max() <= 2 * D
    return x.astype(np.float16).view(np.uint16), keep


def cancelling_tile(T, D, seed, hi_exp, lo_exp):
    """fp16 tile (uint16 bits, [T, D]) whose exact rotation has channel 0 equal
    to zero in every row while the row's entries span exponents lo_exp ..
    hi_exp: row t holds s*2^hi at channel a, s*k*2^lo at b, -s*(2^hi - m) at c,
    -s*m at d and -s*k*2^lo at e (five distinct channels, random per row,
    s = +-1, k in 1..3, m = 2^(hi - 10)), so its plain sum is exactly 0.  With
    hi_exp - lo_exp below 24 every partial sum of a row is exact in float32;
    above, a float32 rotation can round the small entries away in one partial
    sum and not in another."""
    rng = np.random.default_rng(seed)
    x = np.zeros((T, D), np.float64)
    m = 2.0 ** (hi_exp - 10)
    for t in range(T):
        a, b, c, d, e = rng.choice(D, 5, replace=False)
        s = 1.0 if rng.integers(2) else -1.0
        k = float(rng.integers(1, 4))
        x[t, a] = s * 2.0 ** hi_exp
        x[t, b] = s * k * 2.0 ** lo_exp
        x[t, c] = -s * (2.0 ** hi_exp - m)
        x[t, d] = -s * m
        x[t, e] = -s * k * 2.0 ** lo_exp
    h = x.astype(np.float16)
    assert np.array_equal(h.astype(np.float64), x), "entries must be exact in fp16"
    assert np.all(x.sum(axis=1) == 0.0)
    return h.view(np.uint16)
