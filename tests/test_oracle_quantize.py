"""Pins for the oracle's quantizer: Hadamard rotation, variance
normalization and asymmetric round-to-nearest.

The method (evermx.com KVarN review, method paragraph; gmlx "KV cache
quantization", "The two schemes") is pinned by closed forms, a library
routine (scipy's Hadamard), a textbook algorithm reached by another route
(Sinkhorn-Knopp matrix scaling of the squared tile in linear space), and the
invariants and symmetries the method implies.
"""
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
import parity_util

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tile(T=128, D=128, seed=0, outliers=4, dist="normal"):
    rng = np.random.default_rng(seed)
    if dist == "t3":
        x = rng.standard_t(3, (T, D))
    else:
        x = rng.standard_normal((T, D))
    if outliers:
        x[:, rng.choice(D, outliers, replace=False)] *= 20.0
    return x.astype(np.float16)


# ----------------------------------------------------------------- Hadamard --
def test_hadamard_order4_golden():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "hadamard4.txt"))
            if ln.strip() and not ln.startswith("#")]
    ref = np.array(rows, np.float64) / 2.0
    assert np.array_equal(oracle.hadamard(4), ref)


@pytest.mark.parametrize("D", [2, 4, 8, 16, 32, 64, 128, 256, 512])
def test_hadamard_is_scipy_sylvester_and_orthonormal(D):
    H = oracle.hadamard(D)
    assert np.array_equal(H * np.sqrt(D), scipy.linalg.hadamard(D).astype(np.float64))
    assert np.abs(H @ H.T - np.eye(D)).max() < 1e-13
    assert np.array_equal(H, H.T)


@pytest.mark.parametrize("D", [4, 16, 128])
def test_hadamard_sylvester_recursion(D):
    H, H2 = oracle.hadamard(D), oracle.hadamard(2 * D)
    ref = np.block([[H, H], [H, -H]]) / np.sqrt(2.0)
    assert np.abs(H2 - ref).max() < 1e-15


@pytest.mark.parametrize("D", [128, 256, 512])
def test_rotation_preserves_scores_and_is_self_inverse(D):
    rng = np.random.default_rng(D)
    q = rng.standard_normal((1, D))
    k = rng.standard_normal((5, D))
    Rq, Rk = oracle.rotate(q), oracle.rotate(k)
    assert np.allclose(Rq @ Rk.T, q @ k.T, rtol=1e-12, atol=1e-12)
    assert np.abs(oracle.rotate(Rk) - k).max() < 1e-12
    # a unit vector on channel 0 maps to the constant row 1/sqrt(D)
    e0 = np.zeros((1, D)); e0[0, 0] = 1.0
    assert np.allclose(oracle.rotate(e0), 1.0 / np.sqrt(D), rtol=0, atol=1e-15)


@pytest.mark.parametrize("D", [128, 256, 512])
def test_rotation_is_the_natural_order_matrix_product(D):
    """Y = X . H_D with H_D the natural-order Sylvester matrix (scipy's
    hadamard, scaled by 1/sqrt(D)); a sequency- or Walsh-ordered matrix would
    preserve scores and be self-inverse too, but fails this."""
    rng = np.random.default_rng(100 + D)
    X = rng.standard_normal((7, D)).astype(np.float16).astype(np.float64)
    ref = X @ (scipy.linalg.hadamard(D).astype(np.float64) / np.sqrt(D))
    assert np.abs(oracle.rotate(X) - ref).max() < 1e-12
    # each basis vector e_k maps to row k of the matrix
    E = np.eye(D)[[0, 1, 5, D // 2 + 3, D - 1]]
    assert np.abs(oracle.rotate(E) - scipy.linalg.hadamard(D)[[0, 1, 5, D // 2 + 3, D - 1]] / np.sqrt(D)).max() < 1e-15


@pytest.mark.parametrize("L,T,nq", [(32768, 128, 247), (16384, 64, 238), (65536, 128, 503), (1279, 128, 0),
                                    (1280, 128, 1), (1152, 128, 0), (0, 128, 0), (1407, 128, 1), (1408, 128, 2),
                                    (1216, 64, 1), (1215, 64, 0)])
def test_quantized_page_counts_of_the_workloads(L, T, nq):
    """Region rule with the gmlx defaults (fp16 first 128 and newest 1024
    tokens, "The two schemes"): whole pages after the sink, leaving at least
    the tail.  The 16 x 32K, 64 x 16K (g64) and 64K-context layers quantize
    247, 238 and 503 pages of each sequence."""
    lay = dict(T=T, D=128, k_bits=4, v_bits=2, n_iters=6, sink=128, tail=1024, H=8, mla=0)
    assert oracle.quantized_pages(lay, L) == nq


# ------------------------------------------------------------ normalization --
def _sinkhorn_knopp(A, n):
    """Textbook Sinkhorn-Knopp scaling, columns first, to unit means.
    Returns the accumulated column and row divisors."""
    A = A.copy()
    gc = np.ones(A.shape[1])
    gr = np.ones(A.shape[0])
    for _ in range(n):
        c = A.mean(axis=0)
        A /= c[None, :]
        gc *= c
        r = A.mean(axis=1)
        A /= r[:, None]
        gr *= r
    return gc, gr


@pytest.mark.parametrize("T,D,n", [(128, 128, 6), (64, 128, 6), (128, 256, 3), (16, 8, 10)])
def test_normalization_is_sinkhorn_knopp_on_squares(T, D, n):
    Y = oracle.rotate(tile(T, D, seed=T + D).astype(np.float64))
    lr, lc = oracle.normalize(Y, n)
    gc, gr = _sinkhorn_knopp(Y * Y, n)
    assert np.allclose(np.exp(2 * lc), gc, rtol=1e-12)
    assert np.allclose(np.exp(2 * lr), gr, rtol=1e-12)


def test_rows_unit_after_final_row_step_and_columns_converge():
    Y = oracle.rotate(tile(seed=5).astype(np.float64))
    prev = np.inf
    for n in range(1, 13):
        lr, lc = oracle.normalize(Y, n)
        Z = Y * np.exp(-lr[:, None] - lc[None, :])
        rows = np.sqrt((Z * Z).mean(axis=1))
        cols = np.sqrt((Z * Z).mean(axis=0))
        assert np.abs(rows - 1).max() < 1e-12
        dev = np.abs(cols - 1).max()
        assert dev <= prev * (1 + 1e-9)
        prev = dev
    lr, lc = oracle.normalize(Y, 40)
    Z = Y * np.exp(-lr[:, None] - lc[None, :])
    assert np.abs(np.sqrt((Z * Z).mean(axis=0)) - 1).max() < 1e-10


def test_centred_reading_does_not_converge():
    # Why the root-mean-square reading of "standard deviation" is taken: with
    # the centred deviation, column statistics stall away from 1.
    Y = oracle.rotate(tile(seed=6).astype(np.float64))
    lr, lc = oracle.normalize(Y, 60, sigma_mode=1)
    Z = Y * np.exp(-lr[:, None] - lc[None, :])
    assert np.abs(Z.std(axis=0) - 1).max() > 1e-4


def test_zero_tile_degenerate():
    x = np.zeros((128, 128), np.float16)
    rec, u, lc, lr = oracle.quantize_record(x.view(np.uint16), 4, 6)
    codes, S, Z, C = oracle.split_record(rec, 128, 128, 4)
    assert np.all(codes == 0) and np.all(S == 0) and np.all(Z == 0) and np.all(C == 1)


# ---------------------------------------------------------------------- RTN --
def test_rtn_round_half_even_golden():
    # lc = 0, so W = Y; the row's range 3 at 2 bits gives s = 1, u = W - min.
    Y = np.array([[0.0, 0.5, 1.5, 2.5, 3.0, 1.0, 2.0, 0.49]])
    codes, s, mn, u = oracle.rtn(Y, np.zeros(8), 2)
    assert s[0] == 1.0 and mn[0] == 0.0
    assert codes.tolist() == [[0, 0, 2, 2, 3, 1, 2, 0]]


@pytest.mark.parametrize("bits", [2, 4, 6])
@pytest.mark.parametrize("dist", ["normal", "t3"])
def test_rtn_invariants(bits, dist):
    Y = oracle.rotate(tile(seed=bits, dist=dist).astype(np.float64))
    lr, lc = oracle.normalize(Y, 6)
    codes, s, mn, u = oracle.rtn(Y, lc, bits)
    qmax = (1 << bits) - 1
    assert codes.min() >= 0 and codes.max() <= qmax
    assert np.all(codes.min(axis=1) == 0) and np.all(codes.max(axis=1) == qmax)
    W = Y / np.exp(lc)[None, :]
    err = np.abs(W - (mn[:, None] + s[:, None] * codes))
    assert np.all(err <= s[:, None] / 2 * (1 + 1e-12))


@pytest.mark.parametrize("bits", [2, 4, 6])
def test_last_row_step_changes_no_stored_value(bits):
    # The row log-scale multiplies a token's range and minimum alike, so the
    # per-token round-to-nearest cancels it.
    Y = oracle.rotate(tile(seed=10 + bits).astype(np.float64))
    _, lc_a = oracle.normalize(Y, 6, final_row_step=True)
    _, lc_b = oracle.normalize(Y, 6, final_row_step=False)
    assert np.array_equal(lc_a, lc_b)
    ca, sa, ma, _ = oracle.rtn(Y, lc_a, bits)
    # the row-scaled tile gives the same codes and scales
    lr, _ = oracle.normalize(Y, 6)
    cb, sb, mb, _ = oracle.rtn(Y * np.exp(-lr)[:, None], lc_a, bits)
    assert np.array_equal(ca, cb)
    assert np.allclose(sa * np.exp(-lr), sb, rtol=1e-13)
    assert np.allclose(ma * np.exp(-lr), mb, rtol=1e-13, atol=1e-300)


@pytest.mark.parametrize("k", [-3, 1, 4])
def test_scale_equivariance_bit_exact(k):
    x = tile(seed=21)
    y = (x.astype(np.float64) * 2.0 ** k).astype(np.float16)
    assert np.array_equal(y.astype(np.float64), x.astype(np.float64) * 2.0 ** k)
    ra, _, _, _ = oracle.quantize_record(x.view(np.uint16), 4, 6)
    rb, _, _, _ = oracle.quantize_record(y.view(np.uint16), 4, 6)
    ca, Sa, Za, Ca = oracle.split_record(ra, 128, 128, 4)
    cb, Sb, Zb, Cb = oracle.split_record(rb, 128, 128, 4)
    assert np.array_equal(ca, cb) and np.array_equal(Sa, Sb) and np.array_equal(Za, Zb)
    assert np.array_equal(Cb, Ca * 2.0 ** k)


def test_token_permutation_equivariance():
    x = tile(seed=22)
    perm = np.random.default_rng(0).permutation(128)
    ra, ua, lca, _ = oracle.quantize_record(x.view(np.uint16), 4, 6)
    rb, ub, lcb, _ = oracle.quantize_record(x[perm].copy().view(np.uint16), 4, 6)
    assert np.allclose(lca, lcb, rtol=0, atol=1e-12)
    ca, Sa, Za, _ = oracle.split_record(ra, 128, 128, 4)
    cb, Sb, Zb, _ = oracle.split_record(rb, 128, 128, 4)
    near = np.abs(np.abs(ua[perm] - np.floor(ua[perm])) - 0.5) < 1e-9
    assert np.array_equal(ca[perm][~near], cb[~near])
    assert np.array_equal(Sa[perm], Sb) and np.array_equal(Za[perm], Zb)


@pytest.mark.parametrize("bits", [2, 4, 6])
def test_negation_symmetry(bits):
    x = tile(seed=23)
    qmax = (1 << bits) - 1
    Y = oracle.rotate(x.astype(np.float64))
    _, lc = oracle.normalize(Y, 6)
    ca, sa, ma, ua = oracle.rtn(Y, lc, bits)
    _, lc2 = oracle.normalize(-Y, 6)
    assert np.array_equal(lc, lc2)
    cb, sb, mb, ub = oracle.rtn(-Y, lc2, bits)
    near = np.abs(np.abs(ua - np.floor(ua)) - 0.5) < 1e-9
    assert np.array_equal((qmax - ca)[~near], cb[~near])
    assert np.allclose(sa, sb, rtol=1e-14)
    assert np.allclose(mb, -(ma + sa * qmax), rtol=1e-12, atol=1e-12)


def test_rotation_and_normalization_beat_plain_rtn_on_outliers():
    # Directional check of the pages' motivation (rotation spreads outlier
    # channels): 4-bit reconstruction error, KVarN vs per-token RTN alone.
    x = tile(seed=30)
    rec, _, _, _ = oracle.quantize_record(x.view(np.uint16), 4, 6)
    xh = oracle.dequantize_record(rec, 128, 128, 4)
    X = x.astype(np.float64)
    e_kvarn = np.linalg.norm(xh - X) / np.linalg.norm(X)
    codes, s, mn, _ = oracle.rtn(X, np.zeros(128), 4)
    e_plain = np.linalg.norm(mn[:, None] + s[:, None] * codes - X) / np.linalg.norm(X)
    assert e_kvarn < 0.5 * e_plain


# ------------------------------------------------------- degenerate tiles --
@pytest.mark.parametrize("D", [128, 512])
def test_zero_rows_and_channels_keep_their_scales(D):
    """A token row or a rotated channel that is exactly zero has no spread:
    its log-scale stays at 0 (column scale 1), its codes are those of W = 0
    (a zero row: all 0 with S = Zp = 0; a zero channel: the same code as
    every other zero channel of its row), and every row has the full code
    range."""
    T, bits = 128, 4
    x, keep = parity_util.degenerate_tile(T, D, seed=D)
    Y = oracle.rotate(x.view(np.float16).astype(np.float64))
    zc = np.setdiff1d(np.arange(D), keep)
    assert np.all(Y[:, zc] == 0.0) and np.all(Y[::9] == 0.0)
    rec, u, lc, lr = oracle.quantize_record(x, bits, 6)
    codes, S, Z, C = oracle.split_record(rec, T, D, bits)
    assert np.all(C[zc] == 1.0) and np.all(lc[zc] == 0.0)
    assert np.all(C[keep] != 1.0)
    zr = np.zeros(T, bool)
    zr[::9] = True
    assert np.all(lr[zr] == 0.0)
    assert np.all(codes[zr] == 0) and np.all(S[zr] == 0) and np.all(Z[zr] == 0)
    nz = ~zr
    qmax = (1 << bits) - 1
    assert np.all(codes[nz].min(1) == 0) and np.all(codes[nz].max(1) == qmax)
    assert np.all(codes[nz][:, zc] == codes[nz][:, zc[:1]])
    # the zero channels read back as 0 up to the row's rounding step
    W0 = C[zc][None, :] * (S[nz][:, None] * codes[nz][:, zc] + Z[nz][:, None])
    assert np.all(np.abs(W0) <= 0.5 * S[nz][:, None] * (1 + 1e-2))
