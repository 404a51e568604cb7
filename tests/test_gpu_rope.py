"""GPU parity of the MLA rope sidecar (through the C ABI): a 64-wide fp16
rope key beside each int4 latent (evermx.com KVarN review, MLA paragraph:
the compressed latent is quantized to int4; the rope key stays 16-bit).

  quantize   copies each page's rope keys to its record page bit for bit and
             leaves the latent records as without a sidecar;
  decode     (and the verify step) per (sequence, token, head):
             max_j |o - o_ref| <= 2e-3 * max_j |o_ref| against the oracle's
             plain definition (oracle.decode_rope) on the HIP path's records;
  append / commit  rope rows land in the rope pool at the token's fp16 page
             and slot; a promoted page's rope keys reach its record page."""
import numpy as np
import pytest
import torch

import kv_cache_quantization_kvarn_amd as kv
import oracle
from gpu_util import device, gpu_case, host_q, host_u16, say, workload
from parity_util import DECODE_RTOL, decode_rel_err
from synth import normal, to_f16

pytestmark = pytest.mark.gpu


def rope_case(lens, Hq=32, T=128, sink=128, tail=256, qd="bf16", seed=0x9100, M=0):
    w = workload("mla_d512_b32_32k_int4", Hq=Hq, T=T, sink=sink, tail=tail, q_dtype=qd, seed=seed, rope=64)
    return gpu_case(w, seq_lens=[L + M for L in lens], batch=len(lens))


def quantize_rope(case):
    L = kv.layout_from_dict(case["layout"])
    nq = max(case["n_qpages"], 1)
    krec = torch.zeros((nq, 1, kv.record_bytes(L, 0)), dtype=torch.uint8, device=device())
    rrec = torch.zeros((nq, case["layout"]["T"], 64), dtype=torch.float16, device=device())
    kv.quantize(L, case["k16"], None, krec, None, case["src"], case["dst"], rope_fp16=case["rope16"],
                rope_records=rrec)
    torch.cuda.synchronize()
    return L, krec, rrec


def oracle_rope(case, krec, rrec, rows=None, causal=False):
    q = host_q(case["q"])
    if q.ndim == 3:
        q = q[:, None]
    return oracle.decode_rope(case["layout"], krec.cpu().numpy(), host_u16(case["k16"]), host_u16(rrec),
                              host_u16(case["rope16"]), case["block_table"].cpu().numpy(),
                              case["seq_lens"].cpu().numpy(), q, case["Hq"], case["sm_scale"], causal=causal,
                              rows=rows)


def test_quantize_copies_rope_pages_and_keeps_latent_records():
    case = rope_case([1500, 1000, 700], Hq=16)
    L, krec, rrec = quantize_rope(case)
    src, dst = case["src"].cpu().numpy(), case["dst"].cpu().numpy()
    r16, rr = host_u16(case["rope16"]), host_u16(rrec)
    assert len(src) > 0
    for s, d in zip(src, dst):
        assert np.array_equal(rr[d], r16[s])
    assert np.array_equal(rr, host_u16(case["rope_q"]))   # the placement the synthetic case states
    L0 = kv.layout_from_dict(dict(case["layout"], rope=0))
    krec0 = torch.zeros_like(krec)
    kv.quantize(L0, case["k16"], None, krec0, None, case["src"], case["dst"])
    torch.cuda.synchronize()
    assert torch.equal(krec, krec0)


ROPE_SHAPES = [
    # Hq, T, lens, sink, tail, q dtype
    (16, 128, [700, 1, 300], 128, 128, "bf16"),
    (32, 64, [900, 129, 64], 64, 100, "f32"),
    (64, 128, [1500, 640], 128, 256, "f16"),
    (128, 128, [1400, 0, 777], 128, 256, "bf16"),
    (128, 64, [1000, 500], 0, 64, "bf16"),
]


@pytest.mark.parametrize("Hq,T,lens,sink,tail,qd", ROPE_SHAPES)
def test_decode_mla_rope_shapes(Hq, T, lens, sink, tail, qd):
    case = rope_case(lens, Hq=Hq, T=T, sink=sink, tail=tail, qd=qd, seed=0x9200 + Hq + T)
    say("mla rope shape", Hq, T, lens, qd)
    L, krec, rrec = quantize_rope(case)
    out = kv.decode_attn(L, krec, None, case["k16"], None, case["block_table"], case["seq_lens"], case["q"],
                         case["sm_scale"], rope_records=rrec, rope_fp16=case["rope16"])
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o))
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(o[b] == 0)
    rows = np.array([(b, 0, h) for b in range(len(lens)) if lens[b] > 0 for h in sorted({0, 5, Hq // 2 + 1, Hq - 1})],
                    np.int32)
    ref = oracle_rope(case, krec, rrec, rows=rows)
    err, where = decode_rel_err(np.stack([o[b, h] for b, _, h in rows]), ref)
    say(f"[parity] mla rope decode Hq{Hq} T{T} {qd}: worst rel err {err:.3e} (row {where})")
    assert err <= DECODE_RTOL


def test_decode_mla_rope_full_size_sampled():
    case = rope_case([32768] * 32, Hq=128, T=128, sink=128, tail=1024, seed=0x1005)
    say("mla rope full size")
    L, krec, rrec = quantize_rope(case)
    out = kv.decode_attn(L, krec, None, case["k16"], None, case["block_table"], case["seq_lens"], case["q"],
                         case["sm_scale"], rope_records=rrec, rope_fp16=case["rope16"])
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o))
    rng = np.random.default_rng(5)
    rows = np.array([(b, 0, h) for b in (0, 13, 31) for h in sorted(rng.choice(128, 6, replace=False))], np.int32)
    ref = oracle_rope(case, krec, rrec, rows=rows)
    err, where = decode_rel_err(np.stack([o[b, h] for b, _, h in rows]), ref)
    say(f"[parity] mla rope full size (32 x 32K, 128 heads), {len(rows)} rows: worst rel err {err:.3e} (row {where})")
    assert err <= DECODE_RTOL


@pytest.mark.parametrize("M", [2, 4])
def test_verify_decode_mla_rope(M):
    lens = [1023, 1151, 700, 0]
    case = rope_case(lens, Hq=32, T=128, sink=128, tail=256, seed=0x9300 + M, M=M)
    L, krec, rrec = quantize_rope(case)
    lay = case["layout"]
    T, sp = lay["T"], lay["sink"] // lay["T"]
    bt = case["block_table"].cpu().numpy()
    src = case["src"].cpu().numpy()
    base = 0
    for b, n in enumerate(lens):   # pages only L + M would quantize stay fp16 (not committed)
        n_all, n_com = oracle.quantized_pages(lay, n + M), oracle.quantized_pages(lay, n)
        for i in range(n_com, n_all):
            bt[b, sp + i] = src[base + i]
        base += n_all
    dev = device()
    case["block_table"] = torch.tensor(bt, device=dev)
    case["seq_lens"] = torch.tensor(lens, dtype=torch.int32, device=dev)
    B, Hq = len(lens), case["Hq"]
    case["q"] = normal(0x9300, 50 + M, B * M * Hq * 576, device=dev).view(B, M, Hq, 576).to(torch.bfloat16)
    out = kv.decode_attn_mq(L, krec, None, case["k16"], None, case["block_table"], case["seq_lens"], case["q"],
                            case["sm_scale"], rope_records=rrec, rope_fp16=case["rope16"])
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o))
    rows = np.array([(b, i, h) for b in range(B) for i in range(M) for h in (0, 17, Hq - 1)], np.int32)
    ref = oracle.decode_rope(lay, krec.cpu().numpy(), host_u16(case["k16"]), host_u16(rrec), host_u16(case["rope16"]),
                             bt, np.array(lens, np.int32), host_q(case["q"]), Hq, case["sm_scale"], causal=True,
                             rows=rows)
    err, where = decode_rel_err(np.stack([o[b, i, h] for b, i, h in rows]), ref)
    say(f"[parity] mla rope verify M={M}: worst rel err {err:.3e} (row {where})")
    assert err <= DECODE_RTOL


def test_decode_mla_rope_noalloc_equals_decode():
    case = rope_case([1400, 333], Hq=64, seed=0x9400)
    L, krec, rrec = quantize_rope(case)
    a = kv.decode_attn(L, krec, None, case["k16"], None, case["block_table"], case["seq_lens"], case["q"],
                       case["sm_scale"], rope_records=rrec, rope_fp16=case["rope16"])
    b = torch.empty_like(a)
    kv.decode_attn_noalloc(L, krec, None, case["k16"], None, case["block_table"], case["seq_lens"], case["q"],
                           case["sm_scale"], b, rope_records=rrec, rope_fp16=case["rope16"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_append_commit_with_rope():
    dev = device()
    T, sink, tail, M = 64, 64, 40, 2
    lay = dict(T=T, D=512, k_bits=4, v_bits=4, n_iters=6, sink=sink, tail=tail, H=1, mla=1, rope=64)
    L = kv.layout_from_dict(lay)
    B, max_pages, Hq = 3, 10, 16
    seed = 0x9500
    rng = np.random.default_rng(seed)
    nf, nqp = B * max_pages + 8, B * max_pages
    k16 = torch.zeros((nf, 1, T, 512), dtype=torch.float16, device=dev)
    r16 = torch.zeros((nf, T, 64), dtype=torch.float16, device=dev)
    krec = torch.zeros((nqp, 1, kv.record_bytes(L, 0)), dtype=torch.uint8, device=dev)
    rrec = torch.zeros((nqp, T, 64), dtype=torch.float16, device=dev)
    ffree, qfree = list(rng.permutation(nf)), list(rng.permutation(nqp))
    bt = np.full((B, max_pages), -1, np.int32)
    lens = np.zeros(B, np.int32)
    bt_d, sl_d = torch.tensor(bt, device=dev), torch.tensor(lens, device=dev)
    hk = np.zeros((nf, 1, T, 512), np.uint16)
    hr = np.zeros((nf, T, 64), np.uint16)
    n_prom = 0
    steps = int(np.ceil((sink + tail + 3.5 * T) / (M / 2)))
    for step in range(steps):
        for b in range(B):
            for pos in range(lens[b], lens[b] + M):
                p = pos // T
                if p < max_pages and bt[b, p] < 0:
                    bt[b, p] = ffree.pop()
                    bt_d[b, p] = int(bt[b, p])
        kn = to_f16(normal(seed, 100 + step, B * M * 576, device=dev)).view(B, M, 1, 576)
        kv.append(L, k16, None, bt_d, sl_d, kn, None, rope_fp16=r16)
        hkn = kn.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        for b in range(B):
            for i in range(M):
                pos = lens[b] + i
                if pos // T < max_pages:
                    hk[bt[b, pos // T], 0, pos % T] = hkn[b, i, 0, :512]
                    hr[bt[b, pos // T], pos % T] = hkn[b, i, 0, 512:]
        acc = rng.integers(0, M + 1, B).astype(np.int32)
        newq = np.array([qfree[-1 - b] for b in range(B)], np.int32)
        prom_d = torch.full((B,), 99, dtype=torch.int32, device=dev)
        kv.commit(L, krec, None, k16, None, bt_d, sl_d, torch.tensor(acc, device=dev), torch.tensor(newq, device=dev),
                  prom_d, rope_records=rrec, rope_fp16=r16)
        torch.cuda.synchronize()
        assert np.array_equal(host_u16(k16), hk) and np.array_equal(host_u16(r16), hr), step
        ebt, esl, eprom = oracle.commit_plan(lay, bt, lens, acc, newq, nf, nqp)
        assert np.array_equal(prom_d.cpu().numpy(), eprom), step
        assert np.array_equal(bt_d.cpu().numpy(), ebt) and np.array_equal(sl_d.cpu().numpy(), esl), step
        rr = host_u16(rrec)
        for b in range(B):
            if eprom[b] >= 0:
                n_prom += 1
                qid = int(newq[b])
                qfree.remove(qid)
                assert np.array_equal(rr[qid], hr[eprom[b]]), (step, b)
                ffree.insert(0, int(eprom[b]))
        bt, lens = ebt, esl
        if step % 60 == 59 or step == steps - 1:
            q = normal(seed, 7 + step, B * Hq * 576, device=dev).view(B, Hq, 576).to(torch.bfloat16)
            sm = 1.0 / np.sqrt(576)
            out = kv.decode_attn(L, krec, None, k16, None, bt_d, sl_d, q, sm, rope_records=rrec, rope_fp16=r16)
            torch.cuda.synchronize()
            ref = oracle.decode_rope(lay, krec.cpu().numpy(), hk, host_u16(rrec), hr, bt, lens, host_q(q)[:, None],
                                     Hq, sm)
            err, _ = decode_rel_err(out.cpu().numpy()[:, None], ref)
            assert err <= DECODE_RTOL, (step, err)
    say(f"append/commit with rope: {steps} steps, {n_prom} pages promoted, lengths {list(lens)}")
    assert n_prom >= 2 * B
