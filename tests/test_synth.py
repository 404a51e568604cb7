"""The seeded input generator: published SplitMix64 values, determinism and
the shapes of the synthetic workloads."""
import numpy as np
import torch

import synth
from synth.cases import WORKLOADS, make_case, quantized_page_count


def test_splitmix64_published_sequence():
    # SplitMix64 seeded with 0 (Steele, Lea, Flood 2014; the reference C code
    # by Vigna): first outputs.
    ref = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    got = synth.raw_u64(0, 0, torch.arange(3, dtype=torch.int64)).tolist()
    assert [g & (2 ** 64 - 1) for g in got] == ref


def test_counter_based_offsets_are_consistent():
    a = synth.normal(7, 1, 1000)
    b = synth.normal(7, 1, 400, offset=600)
    assert torch.equal(a[600:], b)
    assert not torch.equal(synth.normal(7, 2, 10), a[:10])


def test_normal_and_t3_moments():
    x = synth.normal(11, 1, 1 << 18).numpy()
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    t = synth.student_t3(11, 2, 1 << 18).numpy()
    # Student-t(3): variance 3, median absolute value ~0.765
    assert abs(np.median(np.abs(t)) - 0.7649) < 0.02


def test_permutation_and_choose():
    p = synth.permutation(3, 6, 1000)
    assert sorted(p.tolist()) == list(range(1000))
    c = synth.choose(3, 4, 128, 4)
    assert len(set(c.tolist())) == 4


def test_case_structure():
    w = dict(WORKLOADS["dense8b_b16_32k_k4v2_g128"])
    c = make_case(w, seq_lens=[2048, 1300, 100], batch=3)
    T = w["T"]
    assert c["max_pages"] == 16
    nqs = [quantized_page_count(L, T, 128, 1024) for L in (2048, 1300, 100)]
    assert nqs == [7, 1, 0] and c["n_qpages"] == 8
    assert len(c["src"]) == 8
    assert sorted(c["dst"].tolist()) == list(range(8))
    bt = c["block_table"]
    assert int(bt[0, 1]) == int(c["dst"][0]) and int(bt[1, 1]) == int(c["dst"][7])
    # outliers: 1% of the 1024 (head, channel) pairs
    k = c["k16"].float()
    big = (k.abs().amax(dim=(0, 2)) > 30).sum().item()
    assert big == 10
