"""KVarN hot path on MI355X (gfx950): Python binding of ``libkvarn.so``.

Thin ctypes marshalling over the C ABI declared in ``include/kvarn.h``:
every step of the path runs in the library's HIP kernels.  PyTorch is used
only for device memory and the current HIP stream.  If the library is
missing the import of the functions raises; there is no fallback path.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvarn.so")

KVARN_OK, KVARN_EINVAL, KVARN_EUNSUPPORTED, KVARN_EWORKSPACE, KVARN_EHIP = 0, 1, 2, 3, 4
KVARN_F32, KVARN_F16, KVARN_BF16 = 0, 1, 2

EXPORTS = ("kvarn_parse_preset", "kvarn_layout_check", "kvarn_record_bytes", "kvarn_quantized_pages",
           "kvarn_quantize", "kvarn_decode_workspace_bytes", "kvarn_decode_attn", "kvarn_last_error",
           "kvarn_version", "kvarn_decode_attn_noalloc", "kvarn_append", "kvarn_commit",
           "kvarn_decode_attn_mq", "kvarn_decode_workspace_bytes_mq")


class KvarnError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"kvarn status {status}: {msg}")
        self.status = status


class Layout(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("tile_tokens", ctypes.c_int32), ("k_bits", ctypes.c_int32),
                ("v_bits", ctypes.c_int32), ("n_iters", ctypes.c_int32), ("sink_tokens", ctypes.c_int32),
                ("tail_tokens", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("mla", ctypes.c_int32),
                ("rope_dim", ctypes.c_int32)]


class Cache(ctypes.Structure):
    _fields_ = [("k_records", ctypes.c_void_p), ("v_records", ctypes.c_void_p), ("k_fp16", ctypes.c_void_p),
                ("v_fp16", ctypes.c_void_p), ("n_qpages", ctypes.c_int64), ("n_fpages", ctypes.c_int64),
                ("rope_records", ctypes.c_void_p), ("rope_fp16", ctypes.c_void_p)]


class PageTable(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("max_pages", ctypes.c_int32)]


_lib = None


def lib():
    """Load libkvarn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with kv_cache_quantization_kvarn_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    PL, PC, PT = ctypes.POINTER(Layout), ctypes.POINTER(Cache), ctypes.POINTER(PageTable)
    L.kvarn_parse_preset.argtypes = [ctypes.c_char_p, PL]
    L.kvarn_parse_preset.restype = i32
    L.kvarn_layout_check.argtypes = [PL]
    L.kvarn_layout_check.restype = i32
    L.kvarn_record_bytes.argtypes = [PL, i32]
    L.kvarn_record_bytes.restype = sz
    L.kvarn_quantized_pages.argtypes = [PL, i32]
    L.kvarn_quantized_pages.restype = i32
    L.kvarn_quantize.argtypes = [PL, PC, P, P, i32, P]
    L.kvarn_quantize.restype = i32
    L.kvarn_decode_workspace_bytes.argtypes = [PL, i32, i32, i32]
    L.kvarn_decode_workspace_bytes.restype = sz
    L.kvarn_decode_attn.argtypes = [PL, PC, PT, P, i32, i32, ctypes.c_float, P, P, sz, P]
    L.kvarn_decode_attn.restype = i32
    L.kvarn_decode_attn_noalloc.argtypes = [PL, PC, PT, P, i32, i32, ctypes.c_float, P, P]
    L.kvarn_decode_attn_noalloc.restype = i32
    L.kvarn_decode_workspace_bytes_mq.argtypes = [PL, i32, i32, i32, i32]
    L.kvarn_decode_workspace_bytes_mq.restype = sz
    L.kvarn_decode_attn_mq.argtypes = [PL, PC, PT, P, i32, i32, i32, ctypes.c_float, P, P, sz, P]
    L.kvarn_decode_attn_mq.restype = i32
    L.kvarn_append.argtypes = [PL, PC, PT, P, P, i32, i32, P]
    L.kvarn_append.restype = i32
    L.kvarn_commit.argtypes = [PL, PC, P, P, i32, i32, P, P, P, P]
    L.kvarn_commit.restype = i32
    L.kvarn_last_error.argtypes = []
    L.kvarn_last_error.restype = ctypes.c_char_p
    L.kvarn_version.argtypes = []
    L.kvarn_version.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(st):
    if st != KVARN_OK:
        raise KvarnError(st, lib().kvarn_last_error().decode())


def make_layout(head_dim, tile_tokens, k_bits, v_bits, n_iters=6, sink_tokens=128, tail_tokens=1024,
                num_kv_heads=1, mla=0, rope_dim=0):
    return Layout(head_dim, tile_tokens, k_bits, v_bits, n_iters, sink_tokens, tail_tokens, num_kv_heads, mla,
                  rope_dim)


def layout_from_dict(d):
    """Layout from a dict with keys T, D, k_bits, v_bits, n_iters, sink, tail, H, mla (and rope)."""
    return make_layout(d["D"], d["T"], d["k_bits"], d["v_bits"], d["n_iters"], d["sink"], d["tail"], d["H"],
                       d["mla"], d.get("rope", 0))


def parse_preset(name):
    out = Layout()
    _check(lib().kvarn_parse_preset(name.encode(), ctypes.byref(out)))
    return out


def layout_check(layout):
    return lib().kvarn_layout_check(ctypes.byref(layout))


def record_bytes(layout, which):
    n = lib().kvarn_record_bytes(ctypes.byref(layout), which)
    if n == 0:
        raise KvarnError(KVARN_EINVAL, lib().kvarn_last_error().decode())
    return int(n)


def quantized_pages(layout, seq_len):
    return int(lib().kvarn_quantized_pages(ctypes.byref(layout), int(seq_len)))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_cache(k_records, v_records, k_fp16, v_fp16, rope_records=None, rope_fp16=None):
    """Cache descriptor; rope_records / rope_fp16 (fp16 [n_qpages, T, R] and
    [n_fpages, T, R]) only for an MLA layout with a rope sidecar."""
    nq = 0 if k_records is None else int(k_records.shape[0])
    for t in (rope_records, rope_fp16):
        assert t is None or (t.dtype == torch.float16 and t.is_contiguous())
    return Cache(_ptr(k_records), _ptr(v_records), _ptr(k_fp16), _ptr(v_fp16), nq, int(k_fp16.shape[0]),
                 _ptr(rope_records), _ptr(rope_fp16))


def quantize(layout, k_fp16, v_fp16, k_records, v_records, src, dst, rope_fp16=None, rope_records=None):
    """kvarn_quantize on the current stream.  Pools are device tensors:
    fp16 [n_fpages, H, T, D]; uint8 [n_qpages, H, record bytes]; src/dst int32 [n];
    with a rope sidecar the rope pools fp16 [n_fpages, T, R] and [n_qpages, T, R]."""
    assert src.dtype == torch.int32 and dst.dtype == torch.int32 and src.numel() == dst.numel()
    cache = make_cache(k_records, v_records, k_fp16, v_fp16, rope_records, rope_fp16)
    _check(lib().kvarn_quantize(ctypes.byref(layout), ctypes.byref(cache), _ptr(src), _ptr(dst),
                                int(src.numel()), _stream()))


def decode_workspace_bytes(layout, batch, num_q_heads, max_pages):
    return int(lib().kvarn_decode_workspace_bytes(ctypes.byref(layout), batch, num_q_heads, max_pages))


def alloc_workspace(layout, batch, num_q_heads, max_pages, device="cuda"):
    n = decode_workspace_bytes(layout, batch, num_q_heads, max_pages)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def decode_attn(layout, k_records, v_records, k_fp16, v_fp16, block_table, seq_lens, q, sm_scale, out=None,
                workspace=None, rope_records=None, rope_fp16=None):
    """kvarn_decode_attn on the current stream; q [B, Hq, D] ([B, Hq, D + R]
    with a rope sidecar); returns out [B, Hq, D] fp32."""
    B, Hq = int(q.shape[0]), int(q.shape[1])
    D = layout.head_dim
    assert q.shape[2] == D + layout.rope_dim
    assert block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32
    assert q.is_contiguous() and block_table.is_contiguous()
    qd = {torch.float32: KVARN_F32, torch.bfloat16: KVARN_BF16, torch.float16: KVARN_F16}[q.dtype]
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(layout, B, Hq, block_table.shape[1], q.device)
    cache = make_cache(k_records, v_records, k_fp16, v_fp16, rope_records, rope_fp16)
    pt = PageTable(_ptr(block_table), _ptr(seq_lens), B, int(block_table.shape[1]))
    _check(lib().kvarn_decode_attn(ctypes.byref(layout), ctypes.byref(cache), ctypes.byref(pt), _ptr(q), qd, Hq,
                                   float(sm_scale), _ptr(out), _ptr(workspace), workspace.numel(), _stream()))
    return out


NOALLOC_SCRATCH_BYTES = 96 << 20


def decode_attn_noalloc(layout, k_records, v_records, k_fp16, v_fp16, block_table, seq_lens, q, sm_scale, out,
                        rope_records=None, rope_fp16=None):
    """kvarn_decode_attn_noalloc on the current stream: the workspace is the
    library's fixed device array; out [B, Hq, D] fp32 is caller-provided."""
    B, Hq = int(q.shape[0]), int(q.shape[1])
    assert block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32
    assert q.is_contiguous() and block_table.is_contiguous() and out.is_contiguous()
    qd = {torch.float32: KVARN_F32, torch.bfloat16: KVARN_BF16, torch.float16: KVARN_F16}[q.dtype]
    cache = make_cache(k_records, v_records, k_fp16, v_fp16, rope_records, rope_fp16)
    pt = PageTable(_ptr(block_table), _ptr(seq_lens), B, int(block_table.shape[1]))
    _check(lib().kvarn_decode_attn_noalloc(ctypes.byref(layout), ctypes.byref(cache), ctypes.byref(pt), _ptr(q), qd,
                                           Hq, float(sm_scale), _ptr(out), _stream()))
    return out


def append(layout, k_fp16, v_fp16, block_table, seq_lens, k_new, v_new, rope_fp16=None):
    """kvarn_append on the current stream: k_new / v_new [B, n_new, H, D]
    (MLA: v_new None; with a rope sidecar k_new rows are [D + R]) written
    after each sequence's seq_lens[b] tokens."""
    B, n_new = int(k_new.shape[0]), int(k_new.shape[1])
    assert k_new.is_contiguous() and (v_new is None or v_new.is_contiguous())
    dt = {torch.float32: KVARN_F32, torch.float16: KVARN_F16, torch.bfloat16: KVARN_BF16}[k_new.dtype]
    cache = make_cache(None, None, k_fp16, v_fp16, None, rope_fp16)
    pt = PageTable(_ptr(block_table), _ptr(seq_lens), B, int(block_table.shape[1]))
    _check(lib().kvarn_append(ctypes.byref(layout), ctypes.byref(cache), ctypes.byref(pt), _ptr(k_new), _ptr(v_new),
                              dt, n_new, _stream()))


def commit(layout, k_records, v_records, k_fp16, v_fp16, block_table, seq_lens, n_accept, new_qpages, promoted,
           rope_records=None, rope_fp16=None):
    """kvarn_commit on the current stream; block_table and seq_lens are
    updated in place, promoted [B] receives the per-sequence report."""
    B, max_pages = int(block_table.shape[0]), int(block_table.shape[1])
    for t in (block_table, seq_lens, n_accept, new_qpages, promoted):
        assert t.dtype == torch.int32 and t.is_contiguous()
    cache = make_cache(k_records, v_records, k_fp16, v_fp16, rope_records, rope_fp16)
    _check(lib().kvarn_commit(ctypes.byref(layout), ctypes.byref(cache), _ptr(block_table), _ptr(seq_lens), B,
                              max_pages, _ptr(n_accept), _ptr(new_qpages), _ptr(promoted), _stream()))


def decode_workspace_bytes_mq(layout, batch, num_q_tokens, num_q_heads, max_pages):
    return int(lib().kvarn_decode_workspace_bytes_mq(ctypes.byref(layout), batch, num_q_tokens, num_q_heads,
                                                      max_pages))


def decode_attn_mq(layout, k_records, v_records, k_fp16, v_fp16, block_table, seq_lens, q, sm_scale, out=None,
                   workspace=None, rope_records=None, rope_fp16=None):
    """kvarn_decode_attn_mq on the current stream: q [B, M, Hq, D] (M <= 4
    query tokens at positions seq_lens[b] + i; [B, M, Hq, D + R] with a rope
    sidecar); returns out [B, M, Hq, D] fp32."""
    B, M, Hq = int(q.shape[0]), int(q.shape[1]), int(q.shape[2])
    D = layout.head_dim
    assert q.shape[3] == D + layout.rope_dim
    assert block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32
    assert q.is_contiguous() and block_table.is_contiguous()
    qd = {torch.float32: KVARN_F32, torch.bfloat16: KVARN_BF16, torch.float16: KVARN_F16}[q.dtype]
    if out is None:
        out = torch.empty((B, M, Hq, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        n = decode_workspace_bytes_mq(layout, B, M, Hq, int(block_table.shape[1]))
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)
    cache = make_cache(k_records, v_records, k_fp16, v_fp16, rope_records, rope_fp16)
    pt = PageTable(_ptr(block_table), _ptr(seq_lens), B, int(block_table.shape[1]))
    _check(lib().kvarn_decode_attn_mq(ctypes.byref(layout), ctypes.byref(cache), ctypes.byref(pt), _ptr(q), qd, M, Hq,
                                      float(sm_scale), _ptr(out), _ptr(workspace), workspace.numel(), _stream()))
    return out
