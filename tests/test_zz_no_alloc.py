"""kvarn_decode_attn_noalloc (workspace in the library's fixed device array)
against kvarn_decode_attn (caller workspace), through the C ABI: two calls in
a row, the second on a smaller batch, for a GQA and an MLA layer; and the
refusal of a shape whose workspace exceeds the array."""
import ctypes

import numpy as np
import pytest
import torch

import kv_cache_quantization_kvarn_amd as kv
from gpu_util import gpu_case, run_quantize, say, workload

pytestmark = pytest.mark.gpu


def _both(case, L, krec, vrec):
    ref = kv.decode_attn(L, krec, vrec, case["k16"], case["v16"], case["block_table"], case["seq_lens"], case["q"],
                         case["sm_scale"])
    out = torch.full_like(ref, float("nan"))
    kv.decode_attn_noalloc(L, krec, vrec, case["k16"], case["v16"], case["block_table"], case["seq_lens"],
                           case["q"], case["sm_scale"], out)
    torch.cuda.synchronize()
    return ref, out


@pytest.mark.parametrize("name,big,small", [
    ("dense8b_b16_32k_k4v2_g128", [4000, 2500, 1300, 600], [1900, 700]),
    ("mla_d512_b32_32k_int4", [3000, 1700, 900], [1500]),
])
def test_noalloc_matches_workspace_entry_point(name, big, small):
    for lens in (big, small):
        w = workload(name, seed=0x7000 + len(lens))
        case = gpu_case(w, seq_lens=lens, batch=len(lens))
        L, krec, vrec = run_quantize(case)
        need = kv.decode_workspace_bytes(L, case["B"], case["Hq"], case["max_pages"])
        say("noalloc", name, lens, "workspace", need, "bytes")
        assert 0 < need <= kv.NOALLOC_SCRATCH_BYTES
        ref, out = _both(case, L, krec, vrec)
        # the same kernels on the same inputs: identical outputs
        assert torch.equal(ref, out)
        assert torch.isfinite(out).all()


def test_noalloc_refuses_a_workspace_beyond_the_array():
    # 128 MLA heads x 512-wide latent, 2048 sequences of 256 pages: far beyond 96 MiB
    L = kv.make_layout(512, 128, 4, 4, num_kv_heads=1, mla=1)
    need = kv.decode_workspace_bytes(L, 2048, 128, 256)
    assert need > kv.NOALLOC_SCRATCH_BYTES
    lib = kv.lib()
    cache = kv.Cache(ctypes.c_void_p(256), None, ctypes.c_void_p(256), None, 1, 1)
    pt = kv.PageTable(ctypes.c_void_p(256), ctypes.c_void_p(256), 2048, 256)
    st = lib.kvarn_decode_attn_noalloc(ctypes.byref(L), ctypes.byref(cache), ctypes.byref(pt), ctypes.c_void_p(256),
                                       kv.KVARN_BF16, 128, ctypes.c_float(0.04), ctypes.c_void_p(256), None)
    assert st == kv.KVARN_EWORKSPACE
    assert "fixed" in lib.kvarn_last_error().decode()
