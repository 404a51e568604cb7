"""Pins for the oracle's decode attention over a paged KVarN cache.

The decode oracle is the plain definition (softmax attention over the
read-back cache, double precision).  It is pinned against torch's
scaled_dot_product_attention (a library routine) where the cache is all
fp16, against the special cases the definition implies, and against the
scale-folding identity that the fused path relies on (evermx.com KVarN
review, method paragraph: scales folded back in at read time; the rotation
is orthonormal, so scores are preserved).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from synth.cases import WORKLOADS, make_case


def small(**over):
    w = dict(WORKLOADS["tiny_d128_k4v2"])
    w.update(over)
    return w


def np_case(c):
    g = lambda t: None if t is None else t.cpu().numpy()
    k16 = g(c["k16"]).view(np.uint16)
    v16 = None if c["v16"] is None else g(c["v16"]).view(np.uint16)
    q = c["q"]
    qn = q.view(torch.int16).numpy().view(np.uint16) if q.dtype == torch.bfloat16 else g(q)
    return k16, v16, g(c["block_table"]), g(c["seq_lens"]), qn


def quantized_pools(c):
    lay = c["layout"]
    k16, v16, bt, sl, q = np_case(c)
    H, T, D = lay["H"], lay["T"], lay["D"]
    kb = oracle.record_bytes(T, D, lay["k_bits"])
    vb = oracle.record_bytes(T, D, lay["v_bits"])
    nq = max(c["n_qpages"], 1)
    krec = np.zeros((nq, H, kb), np.uint8)
    vrec = np.zeros((nq, H, vb), np.uint8)
    oracle.quantize_pages(lay, k16, v16, c["src"].numpy(), c["dst"].numpy(), krec, vrec)
    return krec, vrec


def sdpa_reference(Kf, Vf, q, sm):
    """torch SDPA in float64 for one query over fp16 keys/values [L, D]."""
    qt = torch.tensor(q, dtype=torch.float64).view(1, 1, 1, -1)
    kt = torch.tensor(Kf, dtype=torch.float64).view(1, 1, *Kf.shape)
    vt = torch.tensor(Vf, dtype=torch.float64).view(1, 1, *Vf.shape)
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=sm).view(-1).numpy()


def test_fp16_only_cache_matches_sdpa():
    # L <= sink + tail: nothing is quantized, so decode is textbook attention.
    w = small(sink=128, tail=1024, permute=True)
    c = make_case(w, seq_lens=[700, 1, 129], batch=3)
    assert c["n_qpages"] == 0
    k16, v16, bt, sl, q = np_case(c)
    out = oracle.decode(c["layout"], np.zeros(1, np.uint8), np.zeros(1, np.uint8), k16, v16,
                        bt, sl, q, c["Hq"], c["sm_scale"])
    T, D, G = 128, 128, 4
    for b in range(3):
        L = int(sl[b])
        for h in (0, 5, 31):
            g = h // G
            ks = np.concatenate([k16[bt[b, p], g] for p in range(math.ceil(L / T))])[:L]
            vs = np.concatenate([v16[bt[b, p], g] for p in range(math.ceil(L / T))])[:L]
            ref = sdpa_reference(ks.view(np.float16).astype(np.float64),
                                 vs.view(np.float16).astype(np.float64), q[b, h], c["sm_scale"])
            assert np.allclose(out[b, h], ref, rtol=1e-12, atol=1e-12)


def _readback(c, krec, vrec, b, g):
    """Per-token read-back of sequence b, KV head g, via the record fields
    (not via the oracle's decode)."""
    lay = c["layout"]
    T, D = lay["T"], lay["D"]
    k16, v16, bt, sl, _ = np_case(c)
    L = int(sl[b])
    nq = max(0, (L - lay["sink"] - lay["tail"]) // T)
    sp = lay["sink"] // T
    K, V = [], []
    for p in range(math.ceil(L / T)):
        if sp <= p < sp + nq:
            K.append(oracle.dequantize_record(krec[bt[b, p], g], T, D, lay["k_bits"]))
            V.append(oracle.dequantize_record(vrec[bt[b, p], g], T, D, lay["v_bits"], True))
        else:
            K.append(k16[bt[b, p], g].view(np.float16).astype(np.float64))
            V.append(v16[bt[b, p], g].view(np.float16).astype(np.float64))
    return np.concatenate(K)[:L], np.concatenate(V)[:L]


def test_quantized_cache_matches_sdpa_on_readback():
    w = small(sink=128, tail=256, permute=True)
    c = make_case(w, seq_lens=[1024, 777], batch=2)
    krec, vrec = quantized_pools(c)
    k16, v16, bt, sl, q = np_case(c)
    out = oracle.decode(c["layout"], krec, vrec, k16, v16, bt, sl, q, c["Hq"], c["sm_scale"])
    for b in range(2):
        for h in (0, 7, 30):
            K, V = _readback(c, krec, vrec, b, h // 4)
            ref = sdpa_reference(K, V, q[b, h], c["sm_scale"])
            assert np.allclose(out[b, h], ref, rtol=1e-11, atol=1e-12)


def test_scale_folding_identity():
    # <q, k_t> = S_t <qt, code_t> + Zp_t sum(qt), qt = (H q) * C
    rng = np.random.default_rng(4)
    T, D, b = 128, 128, 4
    x = (rng.standard_normal((T, D)) * np.where(rng.random(D) < 0.03, 20, 1)).astype(np.float16)
    rec, _, _, _ = oracle.quantize_record(x.view(np.uint16), b, 6)
    codes, S, Z, C = oracle.split_record(rec, T, D, b)
    q = rng.standard_normal(D)
    K = oracle.dequantize_record(rec, T, D, b)
    qt = (oracle.hadamard(D) @ q) * C
    folded = S * (codes.astype(np.float64) @ qt) + Z * qt.sum()
    assert np.allclose(K @ q, folded, rtol=1e-10, atol=1e-10)


def test_special_cases():
    w = small(sink=0, tail=0, permute=False)
    c = make_case(w, seq_lens=[1024], batch=1)
    krec, vrec = quantized_pools(c)
    k16, v16, bt, sl, q = np_case(c)
    K, V = _readback(c, krec, vrec, 0, 0)
    lay = c["layout"]
    # q = 0: uniform weights, the mean of the read-back values
    out = oracle.decode(lay, krec, vrec, k16, v16, bt, sl, np.zeros_like(q), c["Hq"], 0.125)
    assert np.allclose(out[0, 0], V.mean(axis=0), rtol=1e-11, atol=1e-12)
    # L = 1: the first token's value; a one-token sequence has no whole
    # record, so the token is read from its fp16 page
    out = oracle.decode(lay, krec, vrec, k16, v16, bt, np.array([1], np.int32), q, c["Hq"], 0.125)
    v0 = v16[bt[0, 0], 0, 0].view(np.float16).astype(np.float64)
    assert np.array_equal(out[0, 0], v0)
    # one dominating score: the output is that token's value.  The key of
    # largest norm has the largest inner product with itself; scale q so the
    # gap to every other score is 80 (weights of the rest below e^-80).
    t = int(np.argmax((K * K).sum(1)))
    dots = K @ K[t]
    gap = dots[t] - np.max(np.delete(dots, t))
    assert gap > 0
    qq = q.copy()
    qq[0, 0] = K[t] * (80.0 / gap)
    out = oracle.decode(lay, krec, vrec, k16, v16, bt, sl, qq, c["Hq"], 1.0)
    assert np.allclose(out[0, 0], V[t], rtol=1e-9, atol=1e-9)


def test_page_placement_invariance_and_pairs():
    base = small(sink=128, tail=128)
    outs = []
    for perm in (False, True):
        c = make_case(dict(base, permute=perm), seq_lens=[900, 1024], batch=2)
        krec, vrec = quantized_pools(c)
        k16, v16, bt, sl, q = np_case(c)
        outs.append(oracle.decode(c["layout"], krec, vrec, k16, v16, bt, sl, q, c["Hq"],
                                  c["sm_scale"]))
    assert np.array_equal(outs[0], outs[1])
    pairs = np.array([[1, 3], [0, 31]], np.int32)
    sub = oracle.decode(c["layout"], krec, vrec, k16, v16, bt, sl, q, c["Hq"], c["sm_scale"],
                        pairs=pairs)
    assert np.array_equal(sub[0], outs[1][1, 3]) and np.array_equal(sub[1], outs[1][0, 31])


def test_mla_latent_serves_as_key_and_value():
    w = dict(WORKLOADS["mla_d512_b32_32k_int4"])
    w.update(L=384, sink=128, tail=0, Hq=4)
    c = make_case(w, batch=1)
    lay = c["layout"]
    k16, _, bt, sl, q = np_case(c)
    kb = oracle.record_bytes(128, 512, 4)
    krec = np.zeros((c["n_qpages"], 1, kb), np.uint8)
    oracle.quantize_pages(lay, k16, None, c["src"].numpy(), c["dst"].numpy(), krec, None)
    out = oracle.decode(lay, krec, None, k16, None, bt, sl, q, 4, 1 / math.sqrt(512))
    K = [k16[bt[0, 0], 0].view(np.float16).astype(np.float64)]
    for p in (1, 2):
        K.append(oracle.dequantize_record(krec[bt[0, p], 0], 128, 512, 4))
    K = np.concatenate(K)
    qd = torch.tensor(q.view(np.uint16).astype(np.int32) << 16).view(torch.float32).double()
    for h in range(4):
        ref = sdpa_reference(K, K, qd[0, h].numpy(), 1 / math.sqrt(512))
        assert np.allclose(out[0, h], ref, rtol=1e-11, atol=1e-12)


def _quantized_set(lay, L):
    """Brute force: the pages whose every token lies after the sink and at
    least `tail` tokens before the end, counted one page at a time."""
    T, sink, tail = lay["T"], lay["sink"], lay["tail"]
    out = set()
    p = sink // T
    while (p + 1) * T <= L - tail:
        out.add(p)
        p += 1
    return out


@pytest.mark.parametrize("T,sink,tail", [(64, 64, 96), (128, 128, 1024), (64, 0, 0), (128, 0, 5)])
def test_commit_plan_promotes_exactly_the_pages_entering_the_quantized_region(T, sink, tail):
    lay = dict(T=T, D=128, k_bits=4, v_bits=2, n_iters=6, sink=sink, tail=tail, H=1, mla=0)
    rng = np.random.default_rng(T + sink + tail)
    max_pages = 40
    B = 64
    lens = rng.integers(0, max_pages * T - T, B)
    acc = rng.integers(0, T + 1, B)
    bt = rng.permutation(B * max_pages).reshape(B, max_pages).astype(np.int32)
    newq = np.arange(1000, 1000 + B, dtype=np.int32)
    bt2, sl2, prom = oracle.commit_plan(lay, bt, lens, acc, newq, n_fpages=B * max_pages, n_qpages=2000)
    for b in range(B):
        before, after = _quantized_set(lay, lens[b]), _quantized_set(lay, lens[b] + acc[b])
        new = sorted(after - before)
        assert before <= after and len(new) <= 1
        assert sl2[b] == lens[b] + acc[b]
        if new:
            assert prom[b] == bt[b, new[0]] and bt2[b, new[0]] == newq[b]
            assert np.array_equal(np.delete(bt2[b], new[0]), np.delete(bt[b], new[0]))
        else:
            assert prom[b] == -1 and np.array_equal(bt2[b], bt[b])
    # refusals leave the sequence unchanged
    bad = oracle.commit_plan(lay, bt[:2], [10, 10], [T + 1, -1], newq[:2], B * max_pages, 2000)
    assert list(bad[2]) == [-2, -2] and list(bad[1]) == [10, 10]


def _mq_case(lens, M, **over):
    """Sequences of lens[b] committed tokens plus M appended query tokens:
    the pools hold L + M tokens, the records only the pages of the committed
    length's quantized region (pages that L + M alone would move out of the
    tail stay fp16, as before their commit)."""
    w = small(**over)
    c = make_case(w, seq_lens=[L + M for L in lens], batch=len(lens))
    krec, vrec = quantized_pools(c)
    lay = c["layout"]
    T, sp = lay["T"], lay["sink"] // lay["T"]
    bt = c["block_table"].numpy().copy()
    src = c["src"].numpy()
    base = 0
    for b, L in enumerate(lens):
        n_all, n_com = oracle.quantized_pages(lay, L + M), oracle.quantized_pages(lay, L)
        for i in range(n_com, n_all):
            bt[b, sp + i] = src[base + i]   # back to the fp16 page
        base += n_all
    c["block_table"] = torch.from_numpy(bt)
    c["seq_lens"] = torch.tensor(lens, dtype=torch.int32)
    return c, krec, vrec


def _readback_mq(c, krec, vrec, b, g, Lr, La):
    lay = c["layout"]
    T, D = lay["T"], lay["D"]
    k16, v16, bt, _, _ = np_case(c)
    nq = oracle.quantized_pages(lay, Lr)
    sp = lay["sink"] // T
    K, V = [], []
    for p in range(math.ceil(La / T)):
        if sp <= p < sp + nq:
            K.append(oracle.dequantize_record(krec[bt[b, p], g], T, D, lay["k_bits"]))
            V.append(oracle.dequantize_record(vrec[bt[b, p], g], T, D, lay["v_bits"], True))
        else:
            K.append(k16[bt[b, p], g].view(np.float16).astype(np.float64))
            V.append(v16[bt[b, p], g].view(np.float16).astype(np.float64))
    return np.concatenate(K)[:La], np.concatenate(V)[:La]


@pytest.mark.parametrize("M", [1, 2, 4])
def test_verify_decode_is_causal_attention_over_the_committed_regions(M):
    """gmlx "Speed and speculative decoding": up to four tokens a row are
    verified at once.  Token i attends the first L + i + 1 tokens; the
    records cover only the committed length's quantized region (lengths
    chosen so that L + M crosses a page boundary of the region rule for some
    sequences)."""
    lens = [1024 - 1, 1151, 777, 1279, 1152 - M + 1]
    c, krec, vrec = _mq_case(lens, M, sink=128, tail=256, permute=True)
    lay = c["layout"]
    k16, v16, bt, sl, _ = np_case(c)
    Hq = c["Hq"]
    q = np.random.default_rng(M).standard_normal((len(lens), M, Hq, lay["D"])).astype(np.float32)
    out = oracle.decode_mq(lay, krec, vrec, k16, v16, bt, sl, q, Hq, c["sm_scale"])
    crossing = 0
    for b, L in enumerate(lens):
        crossing += oracle.quantized_pages(lay, L + M) > oracle.quantized_pages(lay, L)
        for i in range(M):
            for h in (0, 13, Hq - 1):
                K, V = _readback_mq(c, krec, vrec, b, h // 4, L, L + i + 1)
                ref = sdpa_reference(K, V, q[b, i, h], c["sm_scale"])
                assert np.allclose(out[b, i, h], ref, rtol=1e-11, atol=1e-12), (b, i, h)
    if M > 1:
        assert crossing >= 1


def test_verify_decode_of_one_token_is_decode_of_one_more_token():
    # where L + 1 moves no page into the quantized region, one verified token
    # is a plain decode step over L + 1 tokens
    lens = [1000, 1200, 1300]
    c, krec, vrec = _mq_case(lens, 1, sink=128, tail=256, permute=True)
    lay = c["layout"]
    assert all(oracle.quantized_pages(lay, L + 1) == oracle.quantized_pages(lay, L) for L in lens)
    k16, v16, bt, sl, _ = np_case(c)
    q = np.random.default_rng(0).standard_normal((3, 1, c["Hq"], lay["D"])).astype(np.float32)
    a = oracle.decode_mq(lay, krec, vrec, k16, v16, bt, sl, q, c["Hq"], c["sm_scale"])
    b = oracle.decode(lay, krec, vrec, k16, v16, bt, sl + 1, q[:, 0], c["Hq"], c["sm_scale"])
    assert np.array_equal(a[:, 0], b)


# ---- MLA with a rope sidecar: the latent (int4 records, the value too) plus
# an fp16 rotary key beside it (evermx.com KVarN review, MLA paragraph: the
# compressed latent is quantized to int4; the rope key stays 16-bit) ----

def _rope_case(lens, Hq=8, M=0, seed=0x2207):
    w = dict(WORKLOADS["mla_d512_b32_32k_int4"])
    w.update(sink=128, tail=256, Hq=Hq, rope=64, seed=seed)
    c = make_case(w, seq_lens=[L + M for L in lens], batch=len(lens))
    lay = c["layout"]
    k16, _, bt, _, q = np_case(c)
    kb = oracle.record_bytes(lay["T"], 512, 4)
    krec = np.zeros((max(c["n_qpages"], 1), 1, kb), np.uint8)
    oracle.quantize_pages(lay, k16, None, c["src"].numpy(), c["dst"].numpy(), krec, None)
    rf = c["rope16"].numpy().view(np.uint16)
    rq = c["rope_q"].numpy().view(np.uint16)
    return c, krec, k16, bt, q, rf, rq


def _latent_and_rope(c, krec, k16, rf, rq, bt, b, Lr, La):
    """Per-token keys (latent read-back, rope key) of sequence b, by page
    region, through the record fields and the pools (not the oracle decode)."""
    lay = c["layout"]
    T = lay["T"]
    nq = oracle.quantized_pages(lay, Lr)
    sp = lay["sink"] // T
    X, Rk = [], []
    for p in range(math.ceil(La / T)):
        if sp <= p < sp + nq:
            X.append(oracle.dequantize_record(krec[bt[b, p], 0], T, 512, 4))
            Rk.append(rq[bt[b, p]].view(np.float16).astype(np.float64))
        else:
            X.append(k16[bt[b, p], 0].view(np.float16).astype(np.float64))
            Rk.append(rf[bt[b, p]].view(np.float16).astype(np.float64))
    return np.concatenate(X)[:La], np.concatenate(Rk)[:La]


def _bf16(q):
    return torch.tensor(q.view(np.uint16).astype(np.int32) << 16).view(torch.float32).double().numpy()


def test_rope_sidecar_is_attention_over_concatenated_keys():
    lens = [1000, 1279, 384]
    c, krec, k16, bt, q, rf, rq = _rope_case(lens)
    assert c["n_qpages"] > 0
    sl = c["seq_lens"].numpy()
    out = oracle.decode_rope(c["layout"], krec, k16, rq, rf, bt, sl, q[:, None], c["Hq"], c["sm_scale"])
    qd = _bf16(q)
    for b, L in enumerate(lens):
        X, Rk = _latent_and_rope(c, krec, k16, rf, rq, bt, b, L, L)
        for h in (0, 5, 7):
            ref = sdpa_reference(np.concatenate([X, Rk], axis=1), X, qd[b, h], c["sm_scale"])
            assert np.allclose(out[b, 0, h], ref, rtol=1e-11, atol=1e-12), (b, h)


def test_rope_sidecar_with_zero_rope_query_is_the_latent_decode():
    lens = [1000, 777]
    c, krec, k16, bt, q, rf, rq = _rope_case(lens)
    sl = c["seq_lens"].numpy()
    q0 = q.copy()
    q0[..., 512:] = 0
    a = oracle.decode_rope(c["layout"], krec, k16, rq, rf, bt, sl, q0[:, None], c["Hq"], c["sm_scale"])
    b = oracle.decode(c["layout"], krec, None, k16, None, bt, sl, np.ascontiguousarray(q0[..., :512]), c["Hq"],
                      c["sm_scale"])
    assert np.array_equal(a[:, 0], b)


def test_rope_sidecar_reads_each_page_rope_key_from_its_region_pool():
    # rope keys a page's region does not use are poisoned: the fp16 pages
    # behind quantized pages (their rope keys were copied out at quantization)
    # and the unused record ids; the result must stay finite and unchanged
    lens = [1000, 1279]
    c, krec, k16, bt, q, rf, rq = _rope_case(lens)
    sl = c["seq_lens"].numpy()
    out = oracle.decode_rope(c["layout"], krec, k16, rq, rf, bt, sl, q[:, None], c["Hq"], c["sm_scale"])
    rf2, rq2 = rf.copy(), np.full((rq.shape[0] + 3,) + rq.shape[1:], 0x7E00, np.uint16)  # NaN
    rq2[:rq.shape[0]] = rq
    rf2[c["src"].numpy()] = 0x7E00
    out2 = oracle.decode_rope(c["layout"], krec, k16, rq2, rf2, bt, sl, q[:, None], c["Hq"], c["sm_scale"])
    assert np.isfinite(out2).all() and np.array_equal(out, out2)


def test_rope_sidecar_dominant_rope_score_selects_its_token():
    lens = [1000]
    c, krec, k16, bt, q, rf, rq = _rope_case(lens, Hq=4)
    sl = c["seq_lens"].numpy()
    L = lens[0]
    X, Rk = _latent_and_rope(c, krec, k16, rf, rq, bt, 0, L, L)
    q2 = np.zeros((1, 1, 4, 576), np.float32)
    toks = (3, 300, 600, 999)   # fp16 sink, quantized (pages 1..4), quantized, fp16 tail
    for h, t in enumerate(toks):
        q2[0, 0, h, 512:] = 4000.0 * Rk[t] / np.linalg.norm(Rk[t])
    out = oracle.decode_rope(c["layout"], krec, k16, rq, rf, bt, sl, q2, 4, c["sm_scale"])
    for h, t in enumerate(toks):
        assert np.allclose(out[0, 0, h], X[t], rtol=1e-9, atol=1e-9), (h, t)


@pytest.mark.parametrize("M", [1, 3])
def test_rope_sidecar_verify_rows_are_causal(M):
    lens = [1023, 1151, 700]
    c, krec, k16, bt, q, rf, rq = _rope_case(lens, M=M)
    lay = c["layout"]
    # committed lengths: pages that only L + M would quantize stay fp16
    sp = lay["sink"] // lay["T"]
    src = c["src"].numpy()
    base = 0
    bt = bt.copy()
    for b, L in enumerate(lens):
        n_all, n_com = oracle.quantized_pages(lay, L + M), oracle.quantized_pages(lay, L)
        for i in range(n_com, n_all):
            bt[b, sp + i] = src[base + i]
        base += n_all
    sl = np.array(lens, np.int32)
    qm = np.random.default_rng(M).standard_normal((len(lens), M, c["Hq"], 576)).astype(np.float32)
    out = oracle.decode_rope(lay, krec, k16, rq, rf, bt, sl, qm, c["Hq"], c["sm_scale"], causal=True)
    for b, L in enumerate(lens):
        for i in range(M):
            X, Rk = _latent_and_rope(c, krec, k16, rf, rq, bt, b, L, L + i + 1)
            for h in (0, 7):
                ref = sdpa_reference(np.concatenate([X, Rk], axis=1), X, qm[b, i, h].astype(np.float64),
                                     c["sm_scale"])
                assert np.allclose(out[b, i, h], ref, rtol=1e-11, atol=1e-12), (b, i, h)
