"""GPU parity of the append and commit path (kvarn_append, kvarn_commit,
through the C ABI) over many decode steps: new tokens go to the fp16 pages,
a random number of them is accepted each step, and pages that the region
rule moves out of the fp16 tail are quantized into records.  Every step the
device block table, lengths and per-sequence reports must equal the host
statement of the rule (oracle.commit_plan) bit for bit, every promoted
record must match the oracle's quantize of the same fp16 page under the
quantize bar, and decode on the grown cache must match the oracle."""
import numpy as np
import pytest
import torch

import kv_cache_quantization_kvarn_amd as kv
import oracle
from gpu_util import device, host_q, say
from parity_util import DECODE_RTOL, CodeStats, assert_code_stats, compare_record, decode_rel_err
from synth import normal, to_f16

pytestmark = pytest.mark.gpu

CASES = [
    # D, T, kb, vb, H, Hq, sink, tail, mla, new tokens per step
    (128, 64, 4, 2, 2, 8, 64, 96, 0, 3),
    (256, 128, 6, 6, 1, 4, 128, 60, 0, 4),
    (512, 64, 4, 4, 1, 16, 64, 40, 1, 2),
]


@pytest.mark.parametrize("D,T,kb,vb,H,Hq,sink,tail,mla,M", CASES)
def test_append_commit_steps(D, T, kb, vb, H, Hq, sink, tail, mla, M):
    dev = device()
    lay = dict(T=T, D=D, k_bits=kb, v_bits=vb, n_iters=6, sink=sink, tail=tail, H=H, mla=mla)
    L = kv.layout_from_dict(lay)
    B, max_pages = 3, 16
    seed = 0x6000 + D + T
    rng = np.random.default_rng(seed)
    nf, nqp = B * max_pages + 8, B * max_pages
    # pools: fp16 pages handed out from a free list, record pages likewise
    k16 = torch.zeros((nf, H, T, D), dtype=torch.float16, device=dev)
    v16 = None if mla else torch.zeros_like(k16)
    krec = torch.zeros((nqp, H, kv.record_bytes(L, 0)), dtype=torch.uint8, device=dev)
    vrec = None if mla else torch.zeros((nqp, H, kv.record_bytes(L, 1)), dtype=torch.uint8, device=dev)
    ffree = list(rng.permutation(nf))
    qfree = list(rng.permutation(nqp))
    bt = np.full((B, max_pages), -1, np.int32)
    lens = np.zeros(B, np.int32)
    bt_d = torch.tensor(bt, device=dev)
    sl_d = torch.tensor(lens, device=dev)
    hk = np.zeros((nf, H, T, D), np.uint16)          # host mirror of the fp16 pools
    hv = None if mla else np.zeros_like(hk)
    stats = CodeStats()
    n_prom = 0
    # enough accepted tokens (M / 2 a step on average) for about 3.5 pages past the sink and tail
    steps = int(np.ceil((sink + tail + 3.5 * T) / (M / 2)))
    for step in range(steps):
        # pages for the positions this step writes
        for b in range(B):
            for pos in range(lens[b], lens[b] + M):
                p = pos // T
                if p < max_pages and bt[b, p] < 0:
                    bt[b, p] = ffree.pop()
                    bt_d[b, p] = int(bt[b, p])
        n = B * M * H * D
        kn = to_f16(normal(seed, 100 + 2 * step, n, device=dev)).view(B, M, H, D)
        vn = None if mla else to_f16(normal(seed, 101 + 2 * step, n, device=dev)).view(B, M, H, D)
        kv.append(L, k16, v16, bt_d, sl_d, kn, vn)
        hkn = kn.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        hvn = None if mla else vn.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        for b in range(B):
            for i in range(M):
                pos = lens[b] + i
                if pos // T < max_pages:
                    hk[bt[b, pos // T], :, pos % T] = hkn[b, i]
                    if not mla:
                        hv[bt[b, pos // T], :, pos % T] = hvn[b, i]
        acc = rng.integers(0, M + 1, B).astype(np.int32)
        if step == steps - 3:
            acc[1] = T + 1       # refused: outside [0, T]
        newq = np.array([qfree[-1 - b] for b in range(B)], np.int32)
        if step == steps - 2:
            newq[2] = nqp + 5    # refused if a promotion is due: record id outside the pool
        prom_d = torch.full((B,), 99, dtype=torch.int32, device=dev)
        kv.commit(L, krec, vrec, k16, v16, bt_d, sl_d, torch.tensor(acc, device=dev), torch.tensor(newq, device=dev),
                  prom_d)
        torch.cuda.synchronize()
        ebt, esl, eprom = oracle.commit_plan(lay, bt, lens, acc, newq, nf, nqp)
        assert np.array_equal(prom_d.cpu().numpy(), eprom), (step, prom_d.cpu().numpy(), eprom)
        assert np.array_equal(bt_d.cpu().numpy(), ebt), step
        assert np.array_equal(sl_d.cpu().numpy(), esl), step
        for b in range(B):
            if eprom[b] >= 0:
                n_prom += 1
                qid = int(newq[b])
                qfree.remove(qid)
                for h in range(H):
                    compare_record(krec[qid, h].cpu().numpy(), hk[eprom[b], h], T, D, kb, 6, False, stats,
                                   f"step {step} seq {b} K head {h}")
                    if not mla:
                        compare_record(vrec[qid, h].cpu().numpy(), hv[eprom[b], h], T, D, vb, 6, True, stats,
                                       f"step {step} seq {b} V head {h}")
                ffree.insert(0, int(eprom[b]))   # the fp16 page is free again
        bt, lens = ebt, esl
        if step % 40 == 39 or step == steps - 1:
            q = normal(seed, 7 + step, B * Hq * D, device=dev).view(B, Hq, D)
            q = q.to(torch.bfloat16) if mla else q.to(torch.float32)
            out = kv.decode_attn(L, krec, vrec, k16, v16, bt_d, sl_d, q, 1.0 / np.sqrt(D))
            torch.cuda.synchronize()
            ref = oracle.decode(lay, krec.cpu().numpy(), None if mla else vrec.cpu().numpy(), hk, hv, bt, lens,
                                host_q(q), Hq, 1.0 / np.sqrt(D))
            err, _ = decode_rel_err(out.cpu().numpy(), ref)
            assert err <= DECODE_RTOL, (step, err)
    assert_code_stats(stats)
    say(f"append/commit D{D} T{T} mla{mla}: {steps} steps, {n_prom} pages promoted, lengths {list(lens)}, "
        f"{stats.diff} of {stats.n} codes at a boundary")
    assert n_prom >= 2 * B
