"""The C-ABI library: it loads without a GPU, exports every function that
include/kvarn.h declares, and validates arguments on the host before any
device work (unsupported shapes are refused with a reason, never given a
fallback -- gmlx "KV cache quantization", "Which layers quantize")."""
import ctypes
import os
import re

import pytest

import kv_cache_quantization_kvarn_amd as kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "kvarn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvarn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return kv.lib()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(kv.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.kvarn_version().decode().startswith("kvarn")


def test_parse_presets():
    L = kv.parse_preset("kvarn_k4v2_g128")
    assert (L.k_bits, L.v_bits, L.tile_tokens, L.n_iters, L.sink_tokens, L.tail_tokens) == (4, 2, 128, 6, 128, 1024)
    L = kv.parse_preset("kvarn_k4v2_g64")
    assert L.tile_tokens == 64
    L = kv.parse_preset("kvarn_k6v6_g128")
    assert (L.k_bits, L.v_bits) == (6, 6)
    L = kv.parse_preset("kvarn_k3v5_g64")
    assert (L.k_bits, L.v_bits, L.tile_tokens) == (3, 5, 64)
    L = kv.parse_preset("kvarn_k8v8_g128")
    assert (L.k_bits, L.v_bits) == (8, 8)
    for bad, st in [("kvarn_k7v2_g128", kv.KVARN_EUNSUPPORTED), ("kvarn_k4v1_g128", kv.KVARN_EUNSUPPORTED),
                    ("kvarn_k4v2_g32", kv.KVARN_EUNSUPPORTED),
                    ("fp8", kv.KVARN_EINVAL), ("kvarn_k4v2_g128x", kv.KVARN_EINVAL)]:
        with pytest.raises(kv.KvarnError) as e:
            kv.parse_preset(bad)
        assert e.value.status == st


def test_head_dim_gate():
    for D in (128, 256, 512):
        assert kv.layout_check(kv.make_layout(D, 128, 4, 2, num_kv_heads=8)) == kv.KVARN_OK
    st = kv.layout_check(kv.make_layout(64, 128, 4, 2, num_kv_heads=8))
    assert st == kv.KVARN_EUNSUPPORTED
    assert "128, 256 and 512" in kv.lib().kvarn_last_error().decode()


@pytest.mark.parametrize("kw,st", [
    (dict(sink_tokens=100), kv.KVARN_EUNSUPPORTED),
    (dict(k_bits=7), kv.KVARN_EUNSUPPORTED),
    (dict(v_bits=1), kv.KVARN_EUNSUPPORTED),
    (dict(v_bits=16), kv.KVARN_EUNSUPPORTED),
    (dict(n_iters=0), kv.KVARN_EINVAL),
    (dict(tail_tokens=-1), kv.KVARN_EINVAL),
    (dict(num_kv_heads=0), kv.KVARN_EINVAL),
    (dict(mla=1, num_kv_heads=1), kv.KVARN_EUNSUPPORTED),  # D=128 latent
])
def test_layout_rejections(kw, st):
    base = dict(head_dim=128, tile_tokens=128, k_bits=4, v_bits=2, num_kv_heads=8)
    base.update(kw)
    assert kv.layout_check(kv.make_layout(**base)) == st


@pytest.mark.parametrize("kb", [2, 3, 4, 5, 6, 8])
def test_every_width_of_the_pages_is_accepted(kb):
    # gmlx "The two schemes": widths 2, 3, 4, 5, 6 and 8, separately for keys and values
    for vb in (2, 3, 4, 5, 6, 8):
        for T in (64, 128):
            for D in (128, 256, 512):
                L = kv.make_layout(D, T, kb, vb, num_kv_heads=2)
                assert kv.layout_check(L) == kv.KVARN_OK
                assert kv.record_bytes(L, 0) == T * D * kb // 8 + 4 * T + 2 * D
                assert kv.record_bytes(L, 0) % 16 == 0 and kv.record_bytes(L, 1) % 16 == 0


def test_record_bytes_and_region_rule():
    L = kv.make_layout(128, 128, 4, 2, num_kv_heads=8)
    assert kv.record_bytes(L, 0) == 128 * 128 * 4 // 8 + 4 * 128 + 2 * 128
    assert kv.record_bytes(L, 1) == 128 * 128 * 2 // 8 + 4 * 128 + 2 * 128
    for Lt, nq in [(0, 0), (1152, 0), (1279, 0), (1280, 1), (32768, 247), (1408, 2)]:
        assert kv.quantized_pages(L, Lt) == nq
    M = kv.make_layout(512, 128, 4, 4, num_kv_heads=1, mla=1)
    assert kv.record_bytes(M, 0) == 128 * 512 // 2 + 512 + 1024
    with pytest.raises(kv.KvarnError):
        kv.record_bytes(M, 1)


def test_quantize_rejects_before_any_device_work():
    L = kv.make_layout(64, 128, 4, 2, num_kv_heads=8)
    cache = kv.Cache(None, None, None, None, 0, 0)
    st = kv.lib().kvarn_quantize(ctypes.byref(L), ctypes.byref(cache), None, None, 4, None)
    assert st == kv.KVARN_EUNSUPPORTED
    L = kv.make_layout(128, 128, 4, 2, num_kv_heads=8)
    st = kv.lib().kvarn_quantize(ctypes.byref(L), ctypes.byref(cache), None, None, 4, None)
    assert st == kv.KVARN_EINVAL
    st = kv.lib().kvarn_quantize(ctypes.byref(L), ctypes.byref(cache), None, None, 0, None)
    assert st == kv.KVARN_OK


def test_decode_rejects_before_any_device_work():
    L = kv.make_layout(128, 128, 4, 2, num_kv_heads=8)
    lib = kv.lib()
    cache = kv.Cache(ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), 1, 1)
    pt = kv.PageTable(ctypes.c_void_p(16), ctypes.c_void_p(16), 2, 4)
    args = lambda hq, ws, wsb, qd=kv.KVARN_F32: (ctypes.byref(L), ctypes.byref(cache), ctypes.byref(pt),
                                                 ctypes.c_void_p(16), qd, hq, ctypes.c_float(0.1),
                                                 ctypes.c_void_p(16), ws, wsb, None)
    need = kv.decode_workspace_bytes(L, 2, 32, 4)
    assert need > 0
    assert lib.kvarn_decode_attn(*args(30, ctypes.c_void_p(256), need)) == kv.KVARN_EINVAL
    # GQA groups: any multiple of 4 query heads per KV head
    assert lib.kvarn_decode_attn(*args(48, ctypes.c_void_p(256), need)) == kv.KVARN_EUNSUPPORTED
    assert lib.kvarn_decode_attn(*args(24, ctypes.c_void_p(256), need)) == kv.KVARN_EUNSUPPORTED
    need8 = kv.decode_workspace_bytes(L, 2, 64, 4)
    assert need8 > need
    assert lib.kvarn_decode_attn(*args(64, ctypes.c_void_p(256), need8 - 1)) == kv.KVARN_EWORKSPACE
    assert lib.kvarn_decode_attn(*args(32, ctypes.c_void_p(256), need - 1)) == kv.KVARN_EWORKSPACE
    assert lib.kvarn_decode_attn(*args(32, None, need)) == kv.KVARN_EWORKSPACE
    assert lib.kvarn_decode_attn(*args(32, ctypes.c_void_p(256), need, qd=7)) == kv.KVARN_EINVAL
    assert lib.kvarn_decode_attn(*args(32, ctypes.c_void_p(260), need)) == kv.KVARN_EINVAL
    # negative pool sizes and batches beyond the grid are refused on the host
    bad = kv.Cache(ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), -1, 1)
    assert lib.kvarn_decode_attn(ctypes.byref(L), ctypes.byref(bad), ctypes.byref(pt), ctypes.c_void_p(16),
                                 kv.KVARN_F32, 32, ctypes.c_float(0.1), ctypes.c_void_p(16), ctypes.c_void_p(256),
                                 need, None) == kv.KVARN_EINVAL
    big = kv.PageTable(ctypes.c_void_p(16), ctypes.c_void_p(16), 40000, 4)
    assert lib.kvarn_decode_attn(ctypes.byref(L), ctypes.byref(cache), ctypes.byref(big), ctypes.c_void_p(16),
                                 kv.KVARN_F32, 32, ctypes.c_float(0.1), ctypes.c_void_p(16), ctypes.c_void_p(256),
                                 1 << 40, None) == kv.KVARN_EUNSUPPORTED
    assert "32767" in lib.kvarn_last_error().decode()


def test_rope_sidecar_gates():
    # a 64-wide rope key beside an MLA latent, or none
    M = kv.make_layout(512, 128, 4, 4, num_kv_heads=1, mla=1, rope_dim=64)
    assert kv.layout_check(M) == kv.KVARN_OK
    assert kv.record_bytes(M, 0) == 128 * 512 // 2 + 4 * 128 + 2 * 512   # the record itself is unchanged
    assert kv.layout_check(kv.make_layout(512, 128, 4, 4, num_kv_heads=1, mla=1, rope_dim=32)) == kv.KVARN_EUNSUPPORTED
    assert kv.layout_check(kv.make_layout(128, 128, 4, 2, num_kv_heads=8, rope_dim=64)) == kv.KVARN_EINVAL
    lib = kv.lib()
    pt = kv.PageTable(ctypes.c_void_p(16), ctypes.c_void_p(16), 2, 4)
    need = kv.decode_workspace_bytes(M, 2, 16, 4)
    assert need > 0

    def decode(cache):
        return lib.kvarn_decode_attn(ctypes.byref(M), ctypes.byref(cache), ctypes.byref(pt), ctypes.c_void_p(16),
                                     kv.KVARN_BF16, 16, ctypes.c_float(0.1), ctypes.c_void_p(16),
                                     ctypes.c_void_p(256), need, None)

    p = ctypes.c_void_p(16)
    assert decode(kv.Cache(p, None, p, None, 1, 1, None, p)) == kv.KVARN_EINVAL        # record-side pool missing
    assert decode(kv.Cache(p, None, p, None, 1, 1, p, None)) == kv.KVARN_EINVAL        # fp16-side pool missing
    assert decode(kv.Cache(p, None, p, None, 1, 1, p, ctypes.c_void_p(24))) == kv.KVARN_EINVAL  # misaligned
    huge = kv.Cache(p, None, p, None, 1, (1 << 32) // (128 * 128) + 1, p, p)           # rope pool of 4 GiB
    assert decode(huge) == kv.KVARN_EUNSUPPORTED
    st = lib.kvarn_quantize(ctypes.byref(M), ctypes.byref(kv.Cache(p, None, p, None, 1, 1, None, p)), p, p, 1, None)
    assert st == kv.KVARN_EINVAL
    st = lib.kvarn_append(ctypes.byref(M), ctypes.byref(kv.Cache(p, None, p, None, 1, 1, p, None)), ctypes.byref(pt),
                          p, None, kv.KVARN_F16, 1, None)
    assert st == kv.KVARN_EINVAL
    assert "rope" in lib.kvarn_last_error().decode()
