"""CPU oracle for the KVarN quantize and decode-attention path.

TEST INFRASTRUCTURE ONLY.  The functions here wrap ``kvarn_oracle.c`` (plain C,
double precision, no blocking or fusion).  Only ``tests/``, the package's
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may use
this package; the HIP library never imports or links it, and the two share no
code.

Each wrapper names the step of the method it follows; the C source cites the
passages (evermx.com review of KVarN, method paragraph; gmlx documentation
"KV cache quantization", section "The two schemes").

Pinned by ``tests/test_oracle_*.py`` against closed forms, invariants and
special cases.  Exact stored values of a record have no worked example on the
pages: beyond those pins they are "parity unpinned".
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

LAYOUT_FIELDS = ("T", "D", "k_bits", "v_bits", "n_iters", "sink", "tail", "H", "mla")


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _build.LIB
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
        _build.build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.orc_half_to_double.restype = dbl
    lib.orc_half_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_double_to_half.restype = ctypes.c_uint16
    lib.orc_double_to_half.argtypes = [dbl]
    lib.orc_bf16_to_double.restype = dbl
    lib.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_hadamard_matrix.argtypes = [i32, P]
    lib.orc_rotate.argtypes = [i32, i32, P, P]
    lib.orc_normalize.argtypes = [i32, i32, P, i32, i32, i32, P, P]
    lib.orc_rtn.argtypes = [i32, i32, P, P, i32, P, P, P, P]
    lib.orc_pack.argtypes = [P, i64, i32, P]
    lib.orc_unpack.argtypes = [P, i64, i32, P]
    lib.orc_record_bytes.restype = i64
    lib.orc_record_bytes.argtypes = [i32, i32, i32]
    lib.orc_quantize_record.argtypes = [P, i32, i32, i32, i32, i32, P, P, P, P]
    lib.orc_dequantize_record.argtypes = [P, i32, i32, i32, i32, P]
    lib.orc_quantize_pages.argtypes = [P, P, P, P, P, i32, P, P, i32]
    lib.orc_quantized_pages.restype = i32
    lib.orc_quantized_pages.argtypes = [P, i32]
    lib.orc_decode.argtypes = [P, P, P, P, P, P, P, i32, P, i32, i32, dbl, P, i32, P, i32]
    lib.orc_decode_groups.argtypes = [P, P, P, P, P, P, P, i32, P, i32, i32, dbl, P, i32, P, i32]
    lib.orc_decode_mq.argtypes = [P, P, P, P, P, P, P, i32, P, i32, i32, i32, dbl, P, i32, P, i32]
    lib.orc_decode_rope.argtypes = [P, P, P, P, P, i32, P, P, i32, P, i32, i32, i32, i32, dbl, P, i32, P, i32]
    _lib = lib
    return lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- numbers --
def half_to_double(bits):
    """binary16 bit pattern(s) -> float64, from the IEEE-754 definition."""
    lib = _load()
    arr = np.asarray(bits, dtype=np.uint16)
    return np.vectorize(lambda b: lib.orc_half_to_double(int(b)), otypes=[np.float64])(arr)


def double_to_half(x):
    """float64 -> binary16 bit pattern(s), round half to even."""
    lib = _load()
    arr = np.asarray(x, dtype=np.float64)
    return np.vectorize(lambda v: lib.orc_double_to_half(float(v)), otypes=[np.uint16])(arr)


# --------------------------------------------------------------- stages --
def hadamard(D):
    """Natural-order Sylvester Hadamard matrix scaled by 1/sqrt(D)."""
    H = np.empty((D, D), np.float64)
    _load().orc_hadamard_matrix(D, _p(H))
    return H


def rotate(X):
    """Stage 2: Y = X . H_D along channels, for every token row."""
    X = _c(X, np.float64)
    T, D = X.shape
    Y = np.empty_like(X)
    _load().orc_rotate(T, D, _p(X), _p(Y))
    return Y


def normalize(Y, n_iters, final_row_step=True, sigma_mode=0):
    """Stage 3: log-space alternation; returns (lr[T], lc[D])."""
    Y = _c(Y, np.float64)
    T, D = Y.shape
    lr = np.empty(T, np.float64)
    lc = np.empty(D, np.float64)
    _load().orc_normalize(T, D, _p(Y), int(n_iters), int(bool(final_row_step)),
                          int(sigma_mode), _p(lr), _p(lc))
    return lr, lc


def rtn(Y, lc, bits):
    """Stage 4: per-token asymmetric RTN; returns (codes, s, mn, u)."""
    Y = _c(Y, np.float64)
    lc = _c(lc, np.float64)
    T, D = Y.shape
    codes = np.empty((T, D), np.uint8)
    s = np.empty(T, np.float64)
    mn = np.empty(T, np.float64)
    u = np.empty((T, D), np.float64)
    _load().orc_rtn(T, D, _p(Y), _p(lc), int(bits), _p(codes), _p(s), _p(mn), _p(u))
    return codes, s, mn, u


def pack(vals, bits):
    vals = _c(vals, np.uint8).ravel()
    out = np.zeros((vals.size * bits + 7) // 8, np.uint8)
    _load().orc_pack(_p(vals), vals.size, int(bits), _p(out))
    return out


def unpack(buf, n, bits):
    buf = _c(buf, np.uint8)
    vals = np.empty(int(n), np.uint8)
    _load().orc_unpack(_p(buf), int(n), int(bits), _p(vals))
    return vals


def record_bytes(T, D, bits):
    return int(_load().orc_record_bytes(T, D, bits))


def quantize_record(x16, bits, n_iters, channel_major=False):
    """Quantize one fp16 tile (uint16 bits, shape [T, D]).

    Returns (record bytes, u[T, D], lc[D], lr[T])."""
    x16 = _c(x16, np.uint16)
    T, D = x16.shape
    rec = np.zeros(record_bytes(T, D, bits), np.uint8)
    u = np.empty((T, D), np.float64)
    lc = np.empty(D, np.float64)
    lr = np.empty(T, np.float64)
    _load().orc_quantize_record(_p(x16), T, D, int(bits), int(n_iters), int(bool(channel_major)),
                                _p(rec), _p(u), _p(lc), _p(lr))
    return rec, u, lc, lr


def dequantize_record(rec, T, D, bits, channel_major=False):
    rec = _c(rec, np.uint8)
    X = np.empty((T, D), np.float64)
    _load().orc_dequantize_record(_p(rec), T, D, int(bits), int(bool(channel_major)), _p(X))
    return X


def split_record(rec, T, D, bits, channel_major=False):
    """Read the stored fields of a record: codes[T, D] (token, channel order),
    S[T], Zp[T], C[D] as float64 values of the stored fp16."""
    rec = _c(rec, np.uint8)
    nb = T * D * bits // 8
    flat = unpack(rec[:nb], T * D, bits)
    if channel_major:
        # blocks of min(T, 64) tokens, each channel's codes of a block in a row
        TB = min(T, 64)
        codes = flat.reshape(T // TB, D, TB).transpose(0, 2, 1).reshape(T, D).copy()
    else:
        codes = flat.reshape(T, D)
    sz = rec[nb:nb + 4 * T].view(np.uint16).reshape(T, 2)
    C = rec[nb + 4 * T:nb + 4 * T + 2 * D].view(np.uint16)
    f = lambda a: a.view(np.float16).astype(np.float64)
    return codes, f(sz[:, 0].copy()), f(sz[:, 1].copy()), f(C.copy())


# ---------------------------------------------------------- paged cache --
def _cfg(layout):
    return np.array([int(layout[k]) for k in LAYOUT_FIELDS], np.int32)


def quantized_pages(layout, L):
    return int(_load().orc_quantized_pages(_p(_cfg(layout)), int(L)))


def quantize_pages(layout, k16, v16, src, dst, krec, vrec, n_threads=0):
    """Quantize fp16 pages src[i] -> record pages dst[i] (all heads, K and V).

    k16/v16: uint16 pools [n_fpages][H][T][D]; krec/vrec: uint8 pools
    [n_qpages][H][record bytes], written in place."""
    cfg = _cfg(layout)
    src = _c(src, np.int32)
    dst = _c(dst, np.int32)
    for a in (k16, krec) + (() if layout["mla"] else (v16, vrec)):
        assert a.flags["C_CONTIGUOUS"]
    _load().orc_quantize_pages(_p(cfg), _p(k16), _p(v16), _p(src), _p(dst), len(src),
                               _p(krec), _p(vrec), int(n_threads))


def decode(layout, krec, vrec, k16, v16, block_table, seq_lens, q, Hq, sm_scale,
           pairs=None, n_threads=0):
    """Decode attention by its plain definition for the given (b, h) pairs.

    q: float32 [B, Hq, D] or a uint16 array holding bfloat16 bits.
    Returns float64 [n_pairs, D] (or [B, Hq, D] when pairs is None)."""
    cfg = _cfg(layout)
    block_table = _c(block_table, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    B, max_pages = block_table.shape
    is_bf16 = q.dtype == np.uint16
    q = np.ascontiguousarray(q)
    D = int(layout["D"])
    full = pairs is None
    if full:
        pairs = np.array([(b, h) for b in range(B) for h in range(Hq)], np.int32)
    pairs = _c(pairs, np.int32).reshape(-1, 2)
    out = np.zeros((len(pairs), D), np.float64)
    _load().orc_decode(_p(cfg), _p(krec), _p(vrec), _p(k16), _p(v16), _p(block_table),
                       _p(seq_lens), int(max_pages), _p(q), int(is_bf16), int(Hq),
                       float(sm_scale), _p(pairs), len(pairs), _p(out), int(n_threads))
    return out.reshape(B, Hq, D) if full else out


def decode_groups(layout, krec, vrec, k16, v16, block_table, seq_lens, q, Hq, sm_scale,
                  groups=None, n_threads=0):
    """The same definition as decode() for whole (sequence b, KV head g)
    groups: each group's tokens are read back once and attended by its
    G = Hq / H query heads.  Returns float64 [B, Hq, D] when groups is None,
    else [n_groups, G, D]."""
    cfg = _cfg(layout)
    block_table = _c(block_table, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    B, max_pages = block_table.shape
    is_bf16 = q.dtype == np.uint16
    q = np.ascontiguousarray(q)
    D, H = int(layout["D"]), int(layout["H"])
    G = Hq // H
    full = groups is None
    if full:
        groups = np.array([(b, g) for b in range(B) for g in range(H)], np.int32)
    groups = _c(groups, np.int32).reshape(-1, 2)
    out = np.zeros((len(groups), G, D), np.float64)
    _load().orc_decode_groups(_p(cfg), _p(krec), _p(vrec), _p(k16), _p(v16), _p(block_table),
                              _p(seq_lens), int(max_pages), _p(q), int(is_bf16), int(Hq),
                              float(sm_scale), _p(groups), len(groups), _p(out), int(n_threads))
    return out.reshape(B, Hq, D) if full else out


def commit_plan(layout, block_table, seq_lens, n_accept, new_qpages, n_fpages, n_qpages):
    """What one commit step does to a paged cache, stated per sequence from
    the region rule: seq_len L grows by the accepted count a (0 <= a <= T and
    L + a within the page table, else the sequence is left as it was and
    reported -2); if the rule now places one more page in the quantized
    region (whole pages after the fp16 sink, leaving at least `tail` tokens
    in fp16 -- gmlx "KV cache quantization", "The two schemes"), that page,
    every token of which is committed (evermx.com KVarN review, MLA and
    hybrid paragraph), is quantized from its fp16 page into record page
    new_qpages[b], the block table entry is pointed at the record page and
    the fp16 page id is reported (-3 and no change if either id lies outside
    its pool); otherwise -1.

    Returns (block_table', seq_lens', promoted) as new arrays."""
    T, sink = int(layout["T"]), int(layout["sink"])
    bt = np.array(block_table, np.int32, copy=True)
    sl = np.array(seq_lens, np.int32, copy=True)
    B, max_pages = bt.shape
    promoted = np.full(B, -1, np.int32)
    for b in range(B):
        a, L = int(n_accept[b]), int(sl[b])
        if a < 0 or a > T or L < 0 or L + a > max_pages * T:
            promoted[b] = -2
            continue
        n0, n1 = quantized_pages(layout, L), quantized_pages(layout, L + a)
        if n1 > n0:
            p = sink // T + n1 - 1
            src, dst = int(bt[b, p]), int(new_qpages[b])
            if not (0 <= src < n_fpages and 0 <= dst < n_qpages):
                promoted[b] = -3
                continue
            promoted[b] = src
            bt[b, p] = dst
        sl[b] = L + a
    return bt, sl, promoted


def decode_mq(layout, krec, vrec, k16, v16, block_table, seq_lens, q, Hq, sm_scale, rows=None, n_threads=0):
    """Verify-step decode by its plain definition: q [B, M, Hq, D] (float32,
    or uint16 bfloat16 bits), token i of sequence b at position
    seq_lens[b] + i attending every token up to and including itself; the
    quantized region is that of the seq_lens[b] committed tokens.
    Returns float64 [B, M, Hq, D] (rows None) or [n_rows, D] for (b, i, h) rows."""
    cfg = _cfg(layout)
    block_table = _c(block_table, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    B, max_pages = block_table.shape
    is_bf16 = q.dtype == np.uint16
    q = np.ascontiguousarray(q)
    M = int(q.shape[1])
    D = int(layout["D"])
    full = rows is None
    if full:
        rows = np.array([(b, i, h) for b in range(B) for i in range(M) for h in range(Hq)], np.int32)
    rows = _c(rows, np.int32).reshape(-1, 3)
    out = np.zeros((len(rows), D), np.float64)
    _load().orc_decode_mq(_p(cfg), _p(krec), _p(vrec), _p(k16), _p(v16), _p(block_table), _p(seq_lens),
                          int(max_pages), _p(q), int(is_bf16), M, int(Hq), float(sm_scale), _p(rows), len(rows),
                          _p(out), int(n_threads))
    return out.reshape(B, M, Hq, D) if full else out


def decode_rope(layout, krec, k16, rope_q, rope_f, block_table, seq_lens, q, Hq, sm_scale, causal=False,
                rows=None, n_threads=0):
    """MLA decode with a rope sidecar by its plain definition: key t is the
    latent read-back x_t together with the fp16 rope key r_t, the value is
    x_t, and score_t = sm_scale (<q_lat, x_t> + <q_rope, r_t>).  r_t comes
    from rope_q [n_qpages, T, R] (uint16 fp16 bits, indexed like the record
    pool) when t's page is in the quantized region of the seq_lens[b]
    committed tokens, else from rope_f [n_fpages, T, R] (indexed like the
    fp16 pool).  q: [B, M, Hq, D + R] float32 or uint16 bfloat16 bits (M = 1
    when causal is False).  causal: token i of sequence b sits at
    seq_lens[b] + i and attends up to itself (a verify step).
    Returns float64 [B, M, Hq, D] (rows None) or [n_rows, D] for (b, i, h) rows."""
    cfg = _cfg(layout)
    assert int(layout["mla"]) == 1
    block_table = _c(block_table, np.int32)
    seq_lens = _c(seq_lens, np.int32)
    B, max_pages = block_table.shape
    is_bf16 = q.dtype == np.uint16
    q = np.ascontiguousarray(q)
    M = int(q.shape[1])
    D = int(layout["D"])
    R = int(q.shape[3]) - D
    assert causal or M == 1
    rope_q = np.ascontiguousarray(rope_q, dtype=np.uint16)
    rope_f = np.ascontiguousarray(rope_f, dtype=np.uint16)
    assert rope_q.shape[-1] == R and rope_f.shape[-1] == R
    full = rows is None
    if full:
        rows = np.array([(b, i, h) for b in range(B) for i in range(M) for h in range(Hq)], np.int32)
    rows = _c(rows, np.int32).reshape(-1, 3)
    out = np.zeros((len(rows), D), np.float64)
    _load().orc_decode_rope(_p(cfg), _p(krec), _p(k16), _p(rope_q), _p(rope_f), R, _p(block_table), _p(seq_lens),
                            int(max_pages), _p(q), int(is_bf16), M, int(bool(causal)), int(Hq), float(sm_scale),
                            _p(rows), len(rows), _p(out), int(n_threads))
    return out.reshape(B, M, Hq, D) if full else out
