"""GPU parity of kvarn_decode_attn (HIP, through the C ABI) against the
oracle's brute-force attention run on the HIP path's own records.

Per (sequence, query head) the output must satisfy
max_j |o - o_ref| <= 2e-3 * max_j |o_ref|.
"""
import numpy as np
import pytest
import torch

from gpu_util import gpu_case, oracle_decode, run_decode, run_quantize, say, workload
from parity_util import DECODE_RTOL, decode_rel_err

pytestmark = pytest.mark.gpu


def check(case, out, krec, vrec, pairs=None):
    ref = oracle_decode(case, krec, vrec, pairs=pairs)
    o = out.cpu().numpy().astype(np.float64)
    if pairs is not None:
        o = np.stack([o[b, h] for b, h in pairs])
    err, where = decode_rel_err(o, ref)
    say("decode max rel err", f"{err:.3e}", "at row", where)
    assert err <= DECODE_RTOL
    return err


def test_decode_one_layer():
    case = gpu_case(workload("tiny_d128_k4v2"))
    L, krec, vrec = run_quantize(case)
    out = run_decode(case, L, krec, vrec)
    check(case, out, krec, vrec)


def test_decode_ragged_lengths_sink_and_tail():
    lens = [0, 1, 127, 128, 129, 1151, 1152, 1153, 1279, 1280, 1281, 1500, 3000, 4096]
    w = workload("dense8b_b16_32k_k4v2_g128", seed=0x3001)
    case = gpu_case(w, seq_lens=lens, batch=len(lens))
    say("ragged case", case["n_qpages"], "quantized pages")
    L, krec, vrec = run_quantize(case)
    out = run_decode(case, L, krec, vrec)
    o = out.cpu().numpy()
    assert np.all(o[0] == 0)  # empty sequence
    pairs = np.array([(b, h) for b in range(1, len(lens)) for h in (0, 13, 31)], np.int32)
    check(case, out, krec, vrec, pairs)


SHAPES = [
    # D, T, k_bits, v_bits, Hq, H, L, sink, tail
    (128, 64, 4, 2, 8, 2, 1000, 128, 256),
    (128, 128, 6, 6, 8, 2, 1300, 128, 128),
    (256, 128, 6, 6, 8, 2, 1500, 128, 256),
    (256, 64, 4, 6, 4, 1, 900, 64, 100),
    (512, 128, 6, 6, 8, 2, 1400, 128, 256),
    (512, 64, 2, 2, 4, 1, 700, 0, 64),
]


@pytest.mark.parametrize("D,T,kb,vb,Hq,H,Lq,sink,tail", SHAPES)
def test_decode_shapes(D, T, kb, vb, Hq, H, Lq, sink, tail):
    w = workload("wide_d256_b8_64k_k6v6", D=D, T=T, k_bits=kb, v_bits=vb, Hq=Hq, H=H, L=Lq, sink=sink,
                 tail=tail, seed=0x4000 + D + T)
    case = gpu_case(w, seq_lens=[Lq, Lq // 2 + 3, 1], batch=3)
    say("decode shape", D, T, kb, vb, Hq, H, Lq)
    L, krec, vrec = run_quantize(case)
    out = run_decode(case, L, krec, vrec)
    check(case, out, krec, vrec)


def test_decode_zero_query_is_mean_of_values():
    # q = 0: every weight equal, the output is the mean read-back value
    case = gpu_case(workload("tiny_d128_k4v2", L=640))
    case["q"] = torch.zeros_like(case["q"])
    L, krec, vrec = run_quantize(case)
    out = run_decode(case, L, krec, vrec)
    check(case, out, krec, vrec)


FULL = ["dense8b_b16_32k_k4v2_g128", "dense8b_b64_16k_k4v2_g64", "wide_d256_b8_64k_k6v6",
        "wide_d512_b8_64k_k6v6"]


@pytest.mark.parametrize("name", FULL)
def test_decode_full_size_sampled(name):
    case = gpu_case(workload(name))
    say("decode full", name)
    L, krec, vrec = run_quantize(case)
    out = run_decode(case, L, krec, vrec)
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o))
    rng = np.random.default_rng(11)
    B, Hq = case["B"], case["Hq"]
    pairs = np.array([(int(rng.integers(B)), int(rng.integers(Hq))) for _ in range(3)] + [(B - 1, Hq - 1)],
                     np.int32)
    check(case, out, krec, vrec, pairs)


MLA_SHAPES = [
    # Hq, T, lens, sink, tail
    (16, 128, [700, 1, 300], 128, 128),
    (32, 64, [900, 129, 64], 64, 100),
    (64, 128, [1500, 640], 128, 256),
    (128, 128, [1400, 0, 777], 128, 256),
    (128, 64, [1000, 500], 0, 64),
]


@pytest.mark.parametrize("Hq,T,lens,sink,tail", MLA_SHAPES)
def test_decode_mla_shapes(Hq, T, lens, sink, tail):
    w = workload("mla_d512_b32_32k_int4", Hq=Hq, T=T, sink=sink, tail=tail, seed=0x5000 + Hq + T)
    case = gpu_case(w, seq_lens=lens, batch=len(lens))
    say("mla shape", Hq, T, lens)
    L, krec, vrec = run_quantize(case)
    out = run_decode(case, L, krec, vrec)
    o = out.cpu().numpy()
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(o[b] == 0)
    pairs = np.array([(b, h) for b in range(len(lens)) if lens[b] > 0 for h in sorted({0, Hq // 2 + 1, Hq - 1})],
                     np.int32)
    check(case, out, krec, None, pairs)


def test_decode_mla_full_size_sampled():
    case = gpu_case(workload("mla_d512_b32_32k_int4"))
    say("decode full mla")
    L, krec, vrec = run_quantize(case)
    out = run_decode(case, L, krec, vrec)
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o))
    pairs = np.array([(3, 5), (17, 100), (31, 127)], np.int32)
    check(case, out, krec, None, pairs)
