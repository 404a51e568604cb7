"""The benchmark's algorithmic byte and flop counts, checked on every workload
of the suite against counts worked out by hand from the workload shapes and
the region rule (whole T-token pages after the fp16 sink are quantized,
leaving at least `tail` newest tokens in fp16; gmlx "KV cache
quantization", "The two schemes").  These counts are the denominators of
every roofline fraction the benchmark reports.

Per workload: quantize reads the fp16 pages it turns into records (keys and
values; the MLA latent only) and writes the records (T D b / 8 bytes of
codes, 4 T of token scales, 2 D of column scales); the decode reads the
records, the fp16 sink and tail tokens, the queries and writes the fp32
output; its matrix work is one multiply-add per query head, channel and token
for the score and one for the value sum."""
import pytest
import torch

import bench
from synth.cases import WORKLOADS, layout_of, quantized_page_count


def _record(T, D, b):
    return T * D * b // 8 + 4 * T + 2 * D


def _hand_counts():
    # tiny: B 1, L 1024, no sink or tail: 8 pages of 128 tokens, all quantized;
    # K records 8960 B (k4), V records 4864 B (v2), 8 KV heads
    tiny = (1 * 8 * 8 * 128 * 128 * 2 * 2,
            1 * 8 * 8 * (8960 + 4864),
            1 * 8 * 8 * (8960 + 4864) + 1 * 32 * 128 * 4 + 1 * 32 * 128 * 4,
            4 * 32 * 128 * 1024)
    # 16 x 32K, T 128: (32768 - 128 - 1024) // 128 = 247 quantized pages and
    # 32768 - 247 * 128 = 1152 fp16 tokens per sequence
    c2 = (16 * 247 * 8 * 128 * 128 * 2 * 2,
          16 * 247 * 8 * (8960 + 4864),
          16 * 247 * 8 * (8960 + 4864) + 16 * 1152 * 8 * 128 * 2 * 2 + 16 * 32 * 128 * 4 * 2,
          16 * 4 * 32 * 128 * 32768)
    # 64 x 16K, T 64: (16384 - 1152) // 64 = 238 pages, 16384 - 238 * 64 = 1152
    # fp16 tokens; records 4096 + 256 + 256 = 4608 (k4) and 2048 + 512 = 2560 (v2)
    c3 = (64 * 238 * 8 * 64 * 128 * 2 * 2,
          64 * 238 * 8 * (4608 + 2560),
          64 * 238 * 8 * (4608 + 2560) + 64 * 1152 * 8 * 128 * 2 * 2 + 64 * 32 * 128 * 4 * 2,
          64 * 4 * 32 * 128 * 16384)
    # 8 x 64K, T 128: (65536 - 1152) // 128 = 503 pages, 65536 - 503 * 128 = 1152
    # fp16 tokens; k6v6 records 128 D 6 / 8 + 512 + 2 D
    r256, r512 = 128 * 256 * 6 // 8 + 512 + 512, 128 * 512 * 6 // 8 + 512 + 1024
    c4a = (8 * 503 * 4 * 128 * 256 * 2 * 2,
           8 * 503 * 4 * 2 * r256,
           8 * 503 * 4 * 2 * r256 + 8 * 1152 * 4 * 256 * 2 * 2 + 8 * 16 * 256 * 4 * 2,
           8 * 4 * 16 * 256 * 65536)
    c4b = (8 * 503 * 2 * 128 * 512 * 2 * 2,
           8 * 503 * 2 * 2 * r512,
           8 * 503 * 2 * 2 * r512 + 8 * 1152 * 2 * 512 * 2 * 2 + 8 * 8 * 512 * 4 * 2,
           8 * 4 * 8 * 512 * 65536)
    # MLA: 32 x 32K, one 512-wide int4 latent (34304-byte records), bf16 queries
    c5 = (32 * 247 * 128 * 512 * 2,
          32 * 247 * 34304,
          32 * 247 * 34304 + 32 * 1152 * 512 * 2 + 32 * 128 * 512 * 2 + 32 * 128 * 512 * 4,
          32 * 4 * 128 * 512 * 32768)
    return {"tiny_d128_k4v2": tiny, "dense8b_b16_32k_k4v2_g128": c2, "dense8b_b64_16k_k4v2_g64": c3,
            "wide_d256_b8_64k_k6v6": c4a, "wide_d512_b8_64k_k6v6": c4b, "mla_d512_b32_32k_int4": c5}


def _shape_case(w):
    """The fields byte_counts reads, without the pools."""
    lay = layout_of(w)
    lens = [w["L"]] * w["B"]
    qdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w["q_dtype"]]
    return {"layout": lay, "B": w["B"], "Hq": w["Hq"],
            "n_qpages": sum(quantized_page_count(L, w["T"], w["sink"], w["tail"]) for L in lens),
            "seq_lens": torch.tensor(lens, dtype=torch.int32),
            "q": torch.empty(w["B"] * w["Hq"] * w["D"], dtype=qdt)}


def test_hand_records():
    # record sizes used above, from the record layout
    assert _record(128, 128, 4) == 8960 and _record(128, 128, 2) == 4864
    assert _record(64, 128, 4) == 4608 and _record(64, 128, 2) == 2560
    assert _record(128, 512, 4) == 34304


@pytest.mark.parametrize("name", bench.SUITE)
def test_byte_counts(name):
    got = bench.byte_counts(_shape_case(WORKLOADS[name]))
    assert tuple(got) == _hand_counts()[name]
