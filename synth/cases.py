"""Synthetic paged-cache workloads for the KVarN path.

Each workload stands in for the structure of the pages' serving workloads
(dense Qwen3-32B and an MLA model on 16K-context bursts; neither weights nor
datasets are used): per-channel outliers that the rotation spreads out,
heavy tails, and contexts of 16K to 64K tokens.

A case holds, on one device:
  k16, v16      fp16 pools [n_fpages][H][T][D]; every logical page of every
                sequence has an fp16 page (the cache before quantization)
  block_table   int32 [B][max_pages]: for each logical page, the id in the
                pool of its region (record pool for quantized pages, fp16
                pool for the sink and tail)
  seq_lens      int32 [B]
  src, dst      int32 [n]: fp16 page id -> record page id, for every page
                that is quantized
  q             [B][Hq][D], float32 or bfloat16 ([B][Hq][D + R] with a rope
                sidecar: the latent query, then the rope query)
  rope16, rope_q  (MLA with a rope sidecar of R = w["rope"] channels) fp16
                rope keys [n_fpages][T][R] placed like k16, and [n_qpages][T][R]
                holding, for every quantized page, the rope keys of its fp16
                page at its record page id (what quantizing the page leaves)

Values are keyed by logical coordinate (b, page, head, token, channel), so
they do not depend on where a page is placed.
"""
import math

import torch

from . import (K_OUT_STREAM, K_STREAM, PAGE_STREAM, Q_STREAM, QPAGE_STREAM, QROPE_STREAM, ROPE_STREAM,
               V_OUT_STREAM, V_STREAM, choose, normal, permutation, student_t3, to_f16)

# fp16 sink (first tokens) and tail (newest tokens) kept unquantized by
# default: 128 and 1024 tokens.
SINK, TAIL = 128, 1024

WORKLOADS = {
    # one layer, 8 KV heads, 1024 tokens, D=128, 4 outlier channels per head x20
    "tiny_d128_k4v2": dict(B=1, H=8, Hq=32, L=1024, D=128, T=128, k_bits=4, v_bits=2,
                           n_iters=6, sink=0, tail=0, mla=0, dist="normal",
                           outliers=("per_head", 4), q_dtype="f32", permute=False,
                           seed=0x1001),
    # dense 8B-like layer: 32 q / 8 KV heads, batch 16, 32K context, 1% outlier channels
    "dense8b_b16_32k_k4v2_g128": dict(B=16, H=8, Hq=32, L=32768, D=128, T=128, k_bits=4,
                                      v_bits=2, n_iters=6, sink=SINK, tail=TAIL, mla=0,
                                      dist="normal", outliers=("frac", 0.01),
                                      q_dtype="f32", permute=True, seed=0x1002),
    # 64-token tiles, batch 64, 16K context
    "dense8b_b64_16k_k4v2_g64": dict(B=64, H=8, Hq=32, L=16384, D=128, T=64, k_bits=4,
                                     v_bits=2, n_iters=6, sink=SINK, tail=TAIL, mla=0,
                                     dist="normal", outliers=("per_head", 4),
                                     q_dtype="f32", permute=True, seed=0x1003),
    # wide heads, 6-bit K and V, Student-t(3) values, 64K context
    "wide_d256_b8_64k_k6v6": dict(B=8, H=4, Hq=16, L=65536, D=256, T=128, k_bits=6,
                                  v_bits=6, n_iters=6, sink=SINK, tail=TAIL, mla=0,
                                  dist="t3", outliers=None, q_dtype="f32", permute=True,
                                  seed=0x1041),
    "wide_d512_b8_64k_k6v6": dict(B=8, H=2, Hq=8, L=65536, D=512, T=128, k_bits=6,
                                  v_bits=6, n_iters=6, sink=SINK, tail=TAIL, mla=0,
                                  dist="t3", outliers=None, q_dtype="f32", permute=True,
                                  seed=0x1042),
    # MLA: one 512-wide latent per token, int4, 128 absorbed query heads (bf16)
    "mla_d512_b32_32k_int4": dict(B=32, H=1, Hq=128, L=32768, D=512, T=128, k_bits=4,
                                  v_bits=4, n_iters=6, sink=SINK, tail=TAIL, mla=1,
                                  dist="normal", outliers=None, q_dtype="bf16",
                                  permute=True, seed=0x1005),
}

LAYOUT_KEYS = ("T", "D", "k_bits", "v_bits", "n_iters", "sink", "tail", "H", "mla")


def layout_of(w):
    d = {k: int(w[k]) for k in LAYOUT_KEYS}
    d["rope"] = int(w.get("rope", 0))
    return d


def quantized_page_count(L, T, sink, tail):
    """Page placement used to build inputs: whole T-token pages after the
    sink, leaving at least `tail` newest tokens unquantized."""
    return max(0, (L - sink - tail) // T)


def _values(w, stream, out_stream, n_pages, device):
    H, T, D = w["H"], w["T"], w["D"]
    n = n_pages * H * T * D
    if w["dist"] == "t3":
        x = student_t3(w["seed"], stream, n, device=device)
    else:
        x = normal(w["seed"], stream, n, device=device)
    x = x.view(n_pages, H, T, D)
    o = w.get("outliers")
    if o is not None:
        if o[0] == "per_head":
            idx = torch.stack([choose(w["seed"], out_stream * 1000 + h, D, o[1], device) + h * D
                               for h in range(H)]).flatten()
        else:
            k = max(1, int(round(o[1] * H * D)))
            idx = choose(w["seed"], out_stream, H * D, k, device)
        scale = torch.ones(H * D, dtype=torch.float64, device=device)
        scale[idx] = 20.0
        x = x * scale.view(1, H, 1, D)
    return to_f16(x)


def make_case(w, device="cpu", seq_lens=None, batch=None, with_v=True):
    """Build the paged case for workload dict w (see WORKLOADS)."""
    B = int(batch if batch is not None else w["B"])
    if seq_lens is None:
        seq_lens = [w["L"]] * B
    seq_lens = [int(x) for x in seq_lens]
    assert len(seq_lens) == B
    T, D, H, Hq = w["T"], w["D"], w["H"], w["Hq"]
    max_pages = max(1, max(math.ceil(L / T) for L in seq_lens))
    n_f = B * max_pages
    mla = bool(w["mla"])

    if w["permute"]:
        fperm = permutation(w["seed"], PAGE_STREAM, n_f, device)
    else:
        fperm = torch.arange(n_f, dtype=torch.int32, device=device)

    def pool(stream, out_stream):
        logical = _values(w, stream, out_stream, n_f, device)
        p = torch.empty_like(logical)
        p[fperm.long()] = logical
        return p

    k16 = pool(K_STREAM, K_OUT_STREAM)
    v16 = pool(V_STREAM, V_OUT_STREAM) if (with_v and not mla) else None

    nqs = [quantized_page_count(L, T, w["sink"], w["tail"]) for L in seq_lens]
    n_q = sum(nqs)
    qperm = (permutation(w["seed"], QPAGE_STREAM, max(n_q, 1), device) if w["permute"]
             else torch.arange(max(n_q, 1), dtype=torch.int32, device=device))
    bt = fperm.view(B, max_pages).clone()
    src, dst = [], []
    sp = w["sink"] // T
    base = 0
    bt_cpu = bt.cpu()
    qperm_cpu = qperm.cpu()
    for b in range(B):
        for i in range(nqs[b]):
            p = sp + i
            src.append(int(bt_cpu[b, p]))
            qid = int(qperm_cpu[base + i])
            dst.append(qid)
            bt_cpu[b, p] = qid
        base += nqs[b]
    bt = bt_cpu.to(device)

    nq_elems = B * Hq * D
    qv = normal(w["seed"], Q_STREAM, nq_elems, device=device).view(B, Hq, D)
    R = int(w.get("rope", 0)) if mla else 0
    rope16 = rope_q = None
    if R > 0:
        logical = to_f16(normal(w["seed"], ROPE_STREAM, n_f * T * R, device=device)).view(n_f, T, R)
        rope16 = torch.empty_like(logical)
        rope16[fperm.long()] = logical
        rope_q = torch.zeros((max(n_q, 1), T, R), dtype=torch.float16, device=device)
        if n_q:
            rope_q[torch.tensor(dst, device=device).long()] = rope16[torch.tensor(src, device=device).long()]
        qr = normal(w["seed"], QROPE_STREAM, B * Hq * R, device=device).view(B, Hq, R)
        qv = torch.cat([qv, qr], dim=2)
    q = qv.to({"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w["q_dtype"]])

    return dict(
        w=w, layout=layout_of(w), B=B, Hq=Hq, seq_lens=torch.tensor(seq_lens, dtype=torch.int32,
                                                                  device=device),
        max_pages=max_pages, n_fpages=n_f, n_qpages=n_q, k16=k16, v16=v16, block_table=bt,
        src=torch.tensor(src, dtype=torch.int32, device=device),
        dst=torch.tensor(dst, dtype=torch.int32, device=device), q=q, R=R, rope16=rope16, rope_q=rope_q,
        sm_scale=1.0 / math.sqrt(D + R))
