"""GPU parity of the verify-step decode (kvarn_decode_attn_mq, through the C
ABI): M <= 4 query tokens per sequence at positions seq_lens[b] + i, causal
among themselves, against the oracle's plain definition (oracle.decode_mq)
on the HIP path's own records, per (sequence, token, head):
max_j |o - o_ref| <= 2e-3 * max_j |o_ref|."""
import numpy as np
import pytest
import torch

import kv_cache_quantization_kvarn_amd as kv
import oracle
from gpu_util import gpu_case, host_q, host_u16, run_quantize, say, workload
from parity_util import DECODE_RTOL, decode_rel_err

pytestmark = pytest.mark.gpu


def mq_case(w, lens, M):
    """The cache of lens[b] committed tokens plus M appended query tokens:
    pools hold L + M tokens; only the committed length's quantized region is
    in records (pages L + M alone would promote stay fp16)."""
    case = gpu_case(w, seq_lens=[L + M for L in lens], batch=len(lens))
    L_, krec, vrec = run_quantize(case)
    lay = case["layout"]
    T, sp = lay["T"], lay["sink"] // lay["T"]
    bt = case["block_table"].cpu().numpy()
    src = case["src"].cpu().numpy()
    base = 0
    for b, L in enumerate(lens):
        n_all, n_com = oracle.quantized_pages(lay, L + M), oracle.quantized_pages(lay, L)
        for i in range(n_com, n_all):
            bt[b, sp + i] = src[base + i]
        base += n_all
    case["block_table"] = torch.tensor(bt, device=case["q"].device)
    case["seq_lens"] = torch.tensor(lens, dtype=torch.int32, device=case["q"].device)
    B, Hq, D = len(lens), case["Hq"], lay["D"]
    from synth import normal

    qv = normal(w["seed"], 40 + M, B * M * Hq * D, device=case["q"].device).view(B, M, Hq, D)
    case["q"] = qv.to(case["q"].dtype)
    return case, L_, krec, vrec


def check_mq(case, L, krec, vrec, rows=None, name=""):
    out = kv.decode_attn_mq(L, krec, vrec, case["k16"], case["v16"], case["block_table"], case["seq_lens"],
                            case["q"], case["sm_scale"])
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o))
    ref = oracle.decode_mq(case["layout"], krec.cpu().numpy(), None if vrec is None else vrec.cpu().numpy(),
                           host_u16(case["k16"]), host_u16(case["v16"]), case["block_table"].cpu().numpy(),
                           case["seq_lens"].cpu().numpy(), host_q(case["q"]), case["Hq"], case["sm_scale"],
                           rows=rows)
    got = o if rows is None else np.stack([o[b, i, h] for b, i, h in rows])
    err, where = decode_rel_err(got, ref)
    say(f"[parity] verify decode {name}: worst rel err {err:.3e} (row {where})")
    assert err <= DECODE_RTOL
    return out


CASES = [
    # D, T, kb, vb, Hq, H, sink, tail, M, q dtype
    (128, 128, 4, 2, 8, 2, 128, 256, 4, "f32"),
    (128, 64, 4, 2, 8, 2, 128, 100, 3, "bf16"),
    (128, 128, 3, 5, 8, 2, 128, 200, 2, "f32"),
    (256, 128, 6, 6, 8, 2, 128, 256, 4, "f32"),
    (512, 128, 6, 6, 8, 2, 128, 256, 2, "f16"),
    (512, 64, 4, 2, 4, 1, 0, 64, 1, "f32"),
    (128, 64, 4, 2, 32, 4, 64, 128, 4, "bf16"),  # groups of 8 query heads
    (256, 128, 3, 5, 16, 1, 128, 256, 3, "f32"),  # a group of 16
]


@pytest.mark.parametrize("D,T,kb,vb,Hq,H,sink,tail,M,qd", CASES)
def test_verify_decode_shapes(D, T, kb, vb, Hq, H, sink, tail, M, qd):
    w = workload("wide_d256_b8_64k_k6v6", D=D, T=T, k_bits=kb, v_bits=vb, Hq=Hq, H=H, sink=sink, tail=tail,
                 dist="normal", outliers=("per_head", 4), q_dtype=qd, seed=0x8000 + D + T + M)
    # lengths around the region boundaries (L + M crossing one for some)
    base = sink + tail + 3 * T
    lens = [base - 1, base + T - M + 1, 700, 0, 1, base + 5 * T - 2]
    case, L, krec, vrec = mq_case(w, lens, M)
    say("verify decode", D, T, kb, vb, M, qd)
    check_mq(case, L, krec, vrec, name=f"D{D} T{T} k{kb}v{vb} M{M} {qd}")


@pytest.mark.parametrize("Hq,M", [(32, 4), (128, 2), (16, 3)])
def test_verify_decode_mla(Hq, M):
    w = workload("mla_d512_b32_32k_int4", Hq=Hq, T=128, sink=128, tail=256, seed=0x8100 + Hq + M)
    lens = [1500, 128 + 256 + 2 * 128 - M + 1, 300, 0]
    case, L, krec, vrec = mq_case(w, lens, M)
    say("verify decode mla", Hq, M)
    check_mq(case, L, krec, None, name=f"mla Hq{Hq} M{M}")


def test_verify_decode_full_size_m4():
    """The 64 x 16K g64 layer with four query tokens per sequence: every
    query token of every head of four sequences."""
    w = workload("dense8b_b64_16k_k4v2_g64")
    lens = [w["L"] - 4] * w["B"]
    case, L, krec, vrec = mq_case(w, lens, 4)
    rng = np.random.default_rng(3)
    seqs = sorted(set(rng.choice(w["B"] - 1, 3, replace=False).tolist()) | {w["B"] - 1})
    rows = np.array([(b, i, h) for b in seqs for i in range(4) for h in range(w["Hq"])], np.int32)
    say("verify decode full size, M = 4")
    check_mq(case, L, krec, vrec, rows=rows, name="dense8b_b64_16k_k4v2_g64 M4")
