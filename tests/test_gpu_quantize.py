"""GPU parity of kvarn_quantize (HIP, through the C ABI) against the oracle.

Full comparison on the one-layer case and on small cases of every shape;
sampled records at the full sizes of the benchmark workloads, quantized in
the same launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

from gpu_util import device, gpu_case, host_u16, run_quantize, say, workload
from parity_util import CodeStats, assert_code_stats, cancelling_tile, compare_record, degenerate_tile

pytestmark = pytest.mark.gpu


def check_records(case, krec, vrec, idx, heads=None):
    lay = case["layout"]
    T, D, H = lay["T"], lay["D"], lay["H"]
    src = case["src"].cpu().numpy()
    dst = case["dst"].cpu().numpy()
    k16 = case["k16"]
    v16 = case["v16"]
    stats = CodeStats()
    kr = krec.cpu().numpy()
    vr = None if vrec is None else vrec.cpu().numpy()
    for i in idx:
        sp, dp = int(src[i]), int(dst[i])
        hs = range(H) if heads is None else heads
        kt = host_u16(k16[sp])
        vt = None if v16 is None else host_u16(v16[sp])
        for h in hs:
            compare_record(kr[dp, h], kt[h], T, D, lay["k_bits"], lay["n_iters"], False, stats,
                           f"K page {i} head {h}")
            if vr is not None:
                compare_record(vr[dp, h], vt[h], T, D, lay["v_bits"], lay["n_iters"], True, stats,
                               f"V page {i} head {h}")
    assert_code_stats(stats)
    return stats


def test_quantize_one_layer_all_records():
    case = gpu_case(workload("tiny_d128_k4v2"))
    say("quantize tiny_d128_k4v2", case["n_qpages"], "pages")
    L, krec, vrec = run_quantize(case)
    st = check_records(case, krec, vrec, range(case["n_qpages"]))
    say("codes differing:", st.diff, "of", st.n)


SHAPES = [
    # D, T, k_bits, v_bits, mla, dist
    (128, 128, 4, 2, 0, "normal"),
    (128, 64, 4, 2, 0, "normal"),
    (128, 128, 6, 6, 0, "t3"),
    (128, 128, 2, 4, 0, "t3"),
    (256, 128, 6, 6, 0, "t3"),
    (256, 64, 4, 6, 0, "normal"),
    (512, 128, 6, 6, 0, "t3"),
    (512, 64, 2, 2, 0, "normal"),
    (512, 128, 4, 4, 1, "normal"),
]


@pytest.mark.parametrize("D,T,kb,vb,mla,dist", SHAPES)
def test_quantize_shapes(D, T, kb, vb, mla, dist):
    w = workload("tiny_d128_k4v2", D=D, T=T, k_bits=kb, v_bits=vb, mla=mla, H=1 if mla else 2,
                 Hq=16 if mla else 8, L=3 * T, dist=dist, outliers=None if mla else ("per_head", 4),
                 permute=True, seed=0x2000 + D + T + kb)
    case = gpu_case(w, batch=2)
    say("quantize shape", D, T, kb, vb, mla, dist)
    L, krec, vrec = run_quantize(case)
    check_records(case, krec, vrec, range(case["n_qpages"]))


FULL = ["dense8b_b16_32k_k4v2_g128", "dense8b_b64_16k_k4v2_g64", "wide_d256_b8_64k_k6v6",
        "wide_d512_b8_64k_k6v6", "mla_d512_b32_32k_int4"]


@pytest.mark.parametrize("name", FULL)
def test_quantize_full_size_sampled(name):
    """Every head of 32 sampled pages (and the pool's last page) of the full
    workload, quantized in the launch the benchmark times."""
    case = gpu_case(workload(name))
    say("quantize full", name, case["n_qpages"], "pages")
    L, krec, vrec = run_quantize(case)
    rng = np.random.default_rng(7)
    idx = sorted(set(rng.choice(case["n_qpages"], 32, replace=False).tolist()) | {case["n_qpages"] - 1})
    st = check_records(case, krec, vrec, idx)
    say(f"[parity] {name}: {st.diff} of {st.n} codes differ by one at a rounding boundary "
        f"({st.frac():.2e}; bar 1e-4)")


WIDTHS = (2, 3, 4, 5, 6, 8)


@pytest.mark.parametrize("D", [128, 256, 512])
@pytest.mark.parametrize("kb", WIDTHS)
@pytest.mark.parametrize("vb", WIDTHS)
def test_quantize_width_pairs(D, kb, vb):
    """Every pair of key and value widths at each head dim (128- and 64-token
    tiles alternate over the pairs)."""
    T = 64 if (kb + vb) % 4 == 0 else 128
    w = workload("tiny_d128_k4v2", D=D, T=T, k_bits=kb, v_bits=vb, H=2, Hq=8, L=2 * T, dist="t3",
                 outliers=("per_head", 4), permute=True, seed=0x2100 + D + 10 * kb + vb)
    case = gpu_case(w, batch=2)
    say("quantize widths", D, T, kb, vb)
    L, krec, vrec = run_quantize(case)
    check_records(case, krec, vrec, range(case["n_qpages"]))


def test_quantize_deterministic_and_scale_equivariant():
    w = workload("tiny_d128_k4v2", L=512)
    case = gpu_case(w)
    L, k1, v1 = run_quantize(case)
    L, k2, v2 = run_quantize(case)
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    # x -> 2x: codes, S and Zp unchanged, C doubled (bit-exact)
    case2 = dict(case)
    case2["k16"] = case["k16"] * 2
    case2["v16"] = case["v16"] * 2
    L, k3, v3 = run_quantize(case2)
    T, D = 128, 128
    for a, b, bits in ((k1, k3, 4), (v1, v3, 2)):
        cb = T * D * bits // 8
        assert torch.equal(a[..., :cb + 4 * T], b[..., :cb + 4 * T])
        ca = a[..., cb + 4 * T:].contiguous().view(torch.float16).float()
        cc = b[..., cb + 4 * T:].contiguous().view(torch.float16).float()
        assert torch.equal(ca * 2, cc)


def test_quantize_zero_tile_and_invalid_ids():
    w = workload("tiny_d128_k4v2", L=256, H=1, Hq=4)
    case = gpu_case(w)
    case["k16"].zero_()
    L, krec, vrec = run_quantize(case)
    T, D = 128, 128
    cb = T * D * 4 // 8
    rec = krec[0, 0]
    assert int(rec[:cb + 4 * T].abs().sum()) == 0
    C = rec[cb + 4 * T:].contiguous().view(torch.float16).float()
    assert torch.all(C == 1.0)
    # out-of-range page ids are skipped by the kernel: the records stay as they were
    import kv_cache_quantization_kvarn_amd as kv
    before = krec.clone()
    bad_src = torch.tensor([10 ** 6, 0], dtype=torch.int32, device=device())
    bad_dst = torch.tensor([0, -1], dtype=torch.int32, device=device())
    kv.quantize(L, case["k16"], case["v16"], krec, vrec, bad_src, bad_dst)
    torch.cuda.synchronize()
    assert torch.equal(before, krec)


@pytest.mark.parametrize("D,kb,vb,mla", [(128, 4, 2, 0), (256, 6, 6, 0), (512, 2, 6, 0), (512, 4, 4, 1)])
def test_quantize_zero_rows_and_channels(D, kb, vb, mla):
    """Degenerate tiles: head 0 holds rows that are integer combinations of
    half of the Sylvester sign patterns (every other rotated channel exactly
    zero) with every 9th row zero; head 1 random values with every 9th row
    zero.  A zero row or channel has no spread and keeps its scale."""
    T = 128
    w = workload("tiny_d128_k4v2", D=D, T=T, k_bits=kb, v_bits=vb, mla=mla, H=1 if mla else 2,
                 Hq=16 if mla else 8, L=2 * T, seed=0x3000 + D + kb)
    case = gpu_case(w)
    say("quantize degenerate", D, kb, vb, mla)
    H = case["layout"]["H"]
    for name in ("k16", "v16"):
        t = case[name]
        if t is None:
            continue
        host = host_u16(t).copy()
        for i, sp in enumerate(case["src"].cpu().tolist()):
            x, _ = degenerate_tile(T, D, seed=1000 * i + D + (name == "v16"))
            host[sp, 0] = x
            if H > 1:
                host[sp, 1, ::9] = 0
        case[name] = torch.from_numpy(host.view(np.int16)).view(torch.float16).to(device())
    L, krec, vrec = run_quantize(case)
    st = check_records(case, krec, vrec, range(case["n_qpages"]))
    say("codes differing:", st.diff, "of", st.n)


@pytest.mark.parametrize("D,kb,vb,mla", [(128, 4, 2, 0), (256, 6, 6, 0), (512, 4, 2, 0), (512, 4, 4, 1)])
def test_quantize_cancelling_channel_within_float32(D, kb, vb, mla):
    """Tiles whose exact rotation is zero in channel 0 of every row, with
    entries spanning 2^-4 .. 2^9: every partial sum of a row is exact in
    float32, so the kernel's rotation cancels that channel exactly, the
    zero column keeps its scale (C = 1) and its codes match the oracle's."""
    T = 128
    w = workload("tiny_d128_k4v2", D=D, T=T, k_bits=kb, v_bits=vb, mla=mla, H=1 if mla else 2,
                 Hq=16 if mla else 8, L=2 * T, seed=0x3100 + D + kb)
    case = gpu_case(w)
    say("quantize cancelling channel", D, kb, vb, mla)
    H = case["layout"]["H"]
    for name in ("k16", "v16"):
        t = case[name]
        if t is None:
            continue
        host = host_u16(t).copy()
        for i, sp in enumerate(case["src"].cpu().tolist()):
            for h in range(H):
                host[sp, h] = cancelling_tile(T, D, seed=100 * i + 10 * h + (name == "v16"), hi_exp=9, lo_exp=-4)
        case[name] = torch.from_numpy(host.view(np.int16)).view(torch.float16).to(device())
    L, krec, vrec = run_quantize(case)
    st = check_records(case, krec, vrec, range(case["n_qpages"]))
    say("codes differing:", st.diff, "of", st.n)
    # channel 0's column scale stays exactly 1
    import oracle
    for rec, bits, cm in ((krec, kb, False), (vrec, vb, True)):
        if rec is None:
            continue
        for dp in case["dst"].cpu().tolist():
            for h in range(H):
                _, _, _, C = oracle.split_record(rec[dp, h].cpu().numpy(), T, D, bits, cm)
                assert C[0] == 1.0
