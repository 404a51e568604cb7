// C ABI of the KVarN hot path: host-side validation and dispatch.
// Nothing is enqueued unless every argument checks out; a failure returns a
// status and leaves a message for kvarn_last_error() (gmlx "KV cache
// quantization": a cache that cannot use the scheme is refused with a
// reason, never given a different one).
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "kvarn.h"
#include "kvarn_internal.hpp"

namespace {

thread_local char g_err[512] = "";

kvarn_status fail(kvarn_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

kvarn_status ok() {
    g_err[0] = 0;
    return KVARN_OK;
}

// code widths of the gmlx documentation, "The two schemes": 2, 3, 4, 5, 6 and 8
bool width_ok(int b) { return b == 2 || b == 3 || b == 4 || b == 5 || b == 6 || b == 8; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

kvarn_status check_layout(const kvarn_layout* L) {
    if (!L) return fail(KVARN_EINVAL, "layout is NULL");
    if (L->head_dim != 128 && L->head_dim != 256 && L->head_dim != 512)
        return fail(KVARN_EUNSUPPORTED, "head_dim %d: the scheme accepts head dimensions 128, 256 and 512 only",
                    L->head_dim);
    if (L->tile_tokens != 128 && L->tile_tokens != 64)
        return fail(KVARN_EUNSUPPORTED, "tile_tokens %d: supported tiles are 128 (g128) and 64 (g64)",
                    L->tile_tokens);
    if (L->mla != 0 && L->mla != 1) return fail(KVARN_EINVAL, "mla must be 0 or 1");
    if (!width_ok(L->k_bits)) return fail(KVARN_EUNSUPPORTED, "k_bits %d: widths 2, 3, 4, 5, 6 and 8 are implemented", L->k_bits);
    if (L->mla) {
        if (L->head_dim != 512) return fail(KVARN_EUNSUPPORTED, "mla: the latent width must be 512");
        if (L->k_bits != 4) return fail(KVARN_EUNSUPPORTED, "mla: the latent is quantized to int4 (k_bits 4)");
        if (L->num_kv_heads != 1) return fail(KVARN_EINVAL, "mla: num_kv_heads must be 1");
    } else {
        if (!width_ok(L->v_bits))
            return fail(KVARN_EUNSUPPORTED, "v_bits %d: widths 2, 3, 4, 5, 6 and 8 are implemented", L->v_bits);
        if (L->num_kv_heads < 1) return fail(KVARN_EINVAL, "num_kv_heads %d must be >= 1", L->num_kv_heads);
    }
    if (L->n_iters < 1 || L->n_iters > 32) return fail(KVARN_EINVAL, "n_iters %d outside 1..32", L->n_iters);
    if (L->sink_tokens < 0 || L->sink_tokens % L->tile_tokens != 0)
        return fail(KVARN_EUNSUPPORTED, "sink_tokens %d must be a non-negative multiple of tile_tokens %d",
                    L->sink_tokens, L->tile_tokens);
    if (L->tail_tokens < 0) return fail(KVARN_EINVAL, "tail_tokens %d must be >= 0", L->tail_tokens);
    if (L->rope_dim != 0) {
        if (!L->mla) return fail(KVARN_EINVAL, "rope_dim %d: a rope sidecar belongs to MLA layouts only", L->rope_dim);
        if (L->rope_dim != 64)
            return fail(KVARN_EUNSUPPORTED, "rope_dim %d: a 64-wide rope key (or none) is implemented", L->rope_dim);
    }
    return KVARN_OK;
}

// rope pools of a layout with a rope sidecar: present and 16-byte aligned
// (the record-side pool only where record pages exist)
kvarn_status check_rope_pools(const kvarn_layout* L, const kvarn_cache* c, bool need_records) {
    if (L->rope_dim == 0) return KVARN_OK;
    if (!c->rope_fp16 || (need_records && !c->rope_records))
        return fail(KVARN_EINVAL, "rope_dim %d: the rope pools are NULL", L->rope_dim);
    if (!aligned16(c->rope_fp16) || (c->rope_records && !aligned16(c->rope_records)))
        return fail(KVARN_EINVAL, "rope pools must be 16-byte aligned");
    return KVARN_OK;
}

size_t rec_bytes(const kvarn_layout* L, int bits) {
    return (size_t)L->tile_tokens * L->head_dim * bits / 8 + 4 * (size_t)L->tile_tokens + 2 * (size_t)L->head_dim;
}


// Workspace of a decode call with M query tokens per sequence (rows =
// batch x M; a causal call's fp16 tail may hold M more tokens).
size_t decode_workspace(const kvarn_layout* layout, int32_t batch, int32_t M, int causal, int32_t num_q_heads,
                        int32_t max_pages) {
    if (check_layout(layout) != KVARN_OK) return 0;
    if (batch < 1 || num_q_heads < 1 || max_pages < 1) {
        fail(KVARN_EINVAL, "batch, num_q_heads and max_pages must be >= 1");
        return 0;
    }
    const int64_t rows = (int64_t)batch * M;
    if (rows > 0x7fffffff / 2) {
        fail(KVARN_EINVAL, "batch x query tokens too large");
        return 0;
    }
    int ns = 1, pps = 1;
    const int H = layout->num_kv_heads;
    kvarn::decode_plan(layout->head_dim, H, num_q_heads / (H > 0 ? H : 1), layout->mla, (int)rows, max_pages,
                       layout->tile_tokens, layout->k_bits, layout->v_bits, &ns, &pps);
    if (layout->mla) return kvarn::mla_workspace_floats(num_q_heads, (int)rows, ns) * sizeof(float);
    const int nf = kvarn::decode_fp16_slots(layout->tile_tokens, layout->sink_tokens,
                                            layout->tail_tokens + (causal ? M : 0), max_pages);
    return kvarn::decode_workspace_floats(layout->head_dim, num_q_heads, (int)rows, ns, nf) * sizeof(float);
}

kvarn_status decode_common(const kvarn_layout* layout, const kvarn_cache* cache, const kvarn_page_table* pages,
                           const void* q, int32_t q_dtype, int32_t M, int causal, int32_t num_q_heads,
                           float sm_scale, float* out, void* workspace, size_t workspace_bytes, void* stream) {
    kvarn_status st = check_layout(layout);
    if (st != KVARN_OK) return st;
    if (!cache || !pages || !q || !out) return fail(KVARN_EINVAL, "NULL argument");
    if (q_dtype != KVARN_F32 && q_dtype != KVARN_F16 && q_dtype != KVARN_BF16)
        return fail(KVARN_EINVAL, "q_dtype %d: KVARN_F32, KVARN_F16 or KVARN_BF16", q_dtype);
    if (pages->batch < 1 || pages->max_pages < 1 || !pages->block_table || !pages->seq_lens)
        return fail(KVARN_EINVAL, "page table: batch and max_pages must be >= 1, arrays non-NULL");
    const int H = layout->num_kv_heads;
    if (num_q_heads < 1 || num_q_heads % H != 0)
        return fail(KVARN_EINVAL, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads, H);
    const int G = num_q_heads / H;
    if (layout->mla) {
        if (num_q_heads != 16 && num_q_heads != 32 && num_q_heads != 64 && num_q_heads != 128)
            return fail(KVARN_EUNSUPPORTED, "mla: %d query heads; 16, 32, 64 or 128 are implemented", num_q_heads);
    } else if (G % 4 != 0) {
        return fail(KVARN_EUNSUPPORTED, "GQA group %d: groups of a multiple of 4 query heads are implemented", G);
    } else if ((int64_t)H * (G / 4) > 65535) {
        return fail(KVARN_EUNSUPPORTED, "GQA: %d groups of 4 query heads; at most 65535", num_q_heads / 4);
    }
    if (!cache->k_fp16 || (!layout->mla && !cache->v_fp16)) return fail(KVARN_EINVAL, "fp16 pools are NULL");
    if (cache->n_qpages < 0 || cache->n_fpages < 0) return fail(KVARN_EINVAL, "negative pool size");
    const int64_t rows = (int64_t)pages->batch * M;
    // GQA grids carry the query rows (and the fp16 slots of each) in grid z, at most 65535
    if (!layout->mla && rows > 32767)
        return fail(KVARN_EUNSUPPORTED, "batch %d x %d query tokens: at most 32767 query rows per call",
                    pages->batch, M);
    if (layout->mla && rows > (1 << 24))
        return fail(KVARN_EUNSUPPORTED, "mla: at most 2^24 query rows per call");
    if (H > 65535) return fail(KVARN_EUNSUPPORTED, "num_kv_heads %d: at most 65535", H);
    if (cache->n_qpages > 0 && (!cache->k_records || (!layout->mla && !cache->v_records)))
        return fail(KVARN_EINVAL, "record pools are NULL");
    if (!(sm_scale > 0.f) || sm_scale > 1e30f) return fail(KVARN_EINVAL, "sm_scale must be positive and finite");
    st = check_rope_pools(layout, cache, cache->n_qpages > 0);
    if (st != KVARN_OK) return st;
    if (layout->rope_dim) {
        // the MLA kernel streams the rope pools through 32-bit offsets too
        const uint64_t page = (uint64_t)layout->tile_tokens * (uint64_t)layout->rope_dim * 2u;
        if ((uint64_t)cache->n_qpages * page >= (1ull << 32) || (uint64_t)cache->n_fpages * page >= (1ull << 32))
            return fail(KVARN_EUNSUPPORTED, "mla: rope pools below 4 GiB each are implemented");
    }
    if (layout->mla || layout->head_dim == 128) {
        // the MLA and head_dim 128 kernels address each record pool with 32-bit byte offsets
        const uint64_t kb = (uint64_t)cache->n_qpages * (uint64_t)H * kvarn_record_bytes(layout, 0);
        const uint64_t vb = layout->mla ? 0 : (uint64_t)cache->n_qpages * (uint64_t)H * kvarn_record_bytes(layout, 1);
        if (kb >= (1ull << 32) || vb >= (1ull << 32))
            return fail(KVARN_EUNSUPPORTED, "%s: record pools of %llu / %llu bytes; below 4 GiB each is implemented",
                        layout->mla ? "mla" : "head_dim 128", (unsigned long long)kb, (unsigned long long)vb);
        // the MLA kernel also streams its fp16 pool through 32-bit offsets
        const uint64_t fb = (uint64_t)cache->n_fpages * (uint64_t)H * (uint64_t)layout->tile_tokens *
                            (uint64_t)layout->head_dim * 2u;
        if (layout->mla && fb >= (1ull << 32))
            return fail(KVARN_EUNSUPPORTED, "mla: an fp16 pool of %llu bytes; below 4 GiB is implemented",
                        (unsigned long long)fb);
    }
    int ns = 1, pps = 1;
    kvarn::decode_plan(layout->head_dim, H, G, layout->mla, (int)rows, pages->max_pages, layout->tile_tokens,
                       layout->k_bits, layout->v_bits, &ns, &pps);
    const int nf = kvarn::decode_fp16_slots(layout->tile_tokens, layout->sink_tokens,
                                            layout->tail_tokens + (causal ? M : 0), pages->max_pages);
    const size_t need = (layout->mla ? kvarn::mla_workspace_floats(num_q_heads, (int)rows, ns)
                                     : kvarn::decode_workspace_floats(layout->head_dim, num_q_heads, (int)rows, ns,
                                                                      nf)) *
                        sizeof(float);
    if (!workspace || workspace_bytes < need)
        return fail(KVARN_EWORKSPACE, "workspace of %zu bytes is smaller than the %zu bytes required",
                    workspace ? workspace_bytes : (size_t)0, need);
    if (((uintptr_t)workspace & 255u) != 0) return fail(KVARN_EINVAL, "workspace must be 256-byte aligned");
    kvarn::DecodeArgs a{};
    a.D = layout->head_dim;
    a.T = layout->tile_tokens;
    a.k_bits = layout->k_bits;
    a.v_bits = layout->v_bits;
    a.sink = layout->sink_tokens;
    a.tail = layout->tail_tokens;
    a.H = H;
    a.mla = layout->mla;
    a.G = G;
    a.GS = layout->mla ? 1 : G / 4;
    a.B = (int)rows;
    a.M = M;
    a.causal = causal;
    a.Hq = num_q_heads;
    a.max_pages = pages->max_pages;
    a.nsplit = ns;
    a.nfsplit = nf;
    a.pps = pps;
    a.k_records = cache->k_records;
    a.v_records = cache->v_records;
    a.k_fp16 = cache->k_fp16;
    a.v_fp16 = cache->v_fp16;
    a.n_qpages = cache->n_qpages;
    a.n_fpages = cache->n_fpages;
    a.block_table = pages->block_table;
    a.seq_lens = pages->seq_lens;
    a.q = q;
    a.q_dtype = q_dtype;
    a.R = layout->rope_dim;
    a.rope_records = cache->rope_records;
    a.rope_fp16 = cache->rope_fp16;
    a.sm_scale = sm_scale;
    a.out = out;
    a.ws = static_cast<float*>(workspace);
    hipError_t e = kvarn::launch_decode(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KVARN_EHIP, "decode launch failed: %s", hipGetErrorString(e));
    return ok();
}

}  // namespace

namespace kvarn {
kvarn_status set_error(kvarn_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}
}  // namespace kvarn

extern "C" {

kvarn_status kvarn_parse_preset(const char* name, kvarn_layout* out) {
    if (!name || !out) return fail(KVARN_EINVAL, "NULL argument");
    int kb = 0, vb = 0, t = 0;
    char tail = 0;
    if (sscanf(name, "kvarn_k%dv%d_g%d%c", &kb, &vb, &t, &tail) != 3)
        return fail(KVARN_EINVAL, "preset '%s' is not of the form kvarn_k<bits>v<bits>_g<tokens>", name);
    if (!width_ok(kb) || !width_ok(vb))
        return fail(KVARN_EUNSUPPORTED, "preset '%s': widths 2, 3, 4, 5, 6 and 8 are implemented", name);
    if (t != 128 && t != 64) return fail(KVARN_EUNSUPPORTED, "preset '%s': tiles of 128 or 64 tokens", name);
    memset(out, 0, sizeof(*out));
    out->tile_tokens = t;
    out->k_bits = kb;
    out->v_bits = vb;
    out->n_iters = 6;
    out->sink_tokens = 128;
    out->tail_tokens = 1024;
    return ok();
}

kvarn_status kvarn_layout_check(const kvarn_layout* layout) {
    kvarn_status st = check_layout(layout);
    return st == KVARN_OK ? ok() : st;
}

size_t kvarn_record_bytes(const kvarn_layout* layout, int32_t which) {
    if (check_layout(layout) != KVARN_OK) return 0;
    if (which != 0 && which != 1) {
        fail(KVARN_EINVAL, "which must be 0 (keys) or 1 (values)");
        return 0;
    }
    if (which == 1 && layout->mla) {
        fail(KVARN_EINVAL, "mla layouts have no value records");
        return 0;
    }
    return rec_bytes(layout, which == 0 ? layout->k_bits : layout->v_bits);
}

int32_t kvarn_quantized_pages(const kvarn_layout* layout, int32_t seq_len) {
    if (check_layout(layout) != KVARN_OK) return -1;
    if (seq_len < 0) {
        fail(KVARN_EINVAL, "seq_len %d < 0", seq_len);
        return -1;
    }
    const int64_t r = (int64_t)seq_len - layout->sink_tokens - layout->tail_tokens;
    return r >= layout->tile_tokens ? (int32_t)(r / layout->tile_tokens) : 0;
}

kvarn_status kvarn_quantize(const kvarn_layout* layout, const kvarn_cache* cache, const int32_t* src_fpages,
                            const int32_t* dst_qpages, int32_t n, void* stream) {
    kvarn_status st = check_layout(layout);
    if (st != KVARN_OK) return st;
    if (!cache) return fail(KVARN_EINVAL, "cache is NULL");
    if (n < 0) return fail(KVARN_EINVAL, "n %d < 0", n);
    if (n == 0) return ok();
    if (!src_fpages || !dst_qpages) return fail(KVARN_EINVAL, "page lists are NULL");
    if (!cache->k_fp16 || !cache->k_records) return fail(KVARN_EINVAL, "key pools are NULL");
    if (!layout->mla && (!cache->v_fp16 || !cache->v_records)) return fail(KVARN_EINVAL, "value pools are NULL");
    if (!aligned16(cache->k_fp16) || !aligned16(cache->k_records) ||
        (!layout->mla && (!aligned16(cache->v_fp16) || !aligned16(cache->v_records))))
        return fail(KVARN_EINVAL, "pools must be 16-byte aligned");
    if (cache->n_fpages < 1 || cache->n_qpages < 1) return fail(KVARN_EINVAL, "empty pools");
    if ((int64_t)n * layout->num_kv_heads * (layout->mla ? 1 : 2) > 0x7fffffffLL)
        return fail(KVARN_EINVAL, "too many pages in one call: pages x heads x (K, V) must fit one grid");
    st = check_rope_pools(layout, cache, true);
    if (st != KVARN_OK) return st;
    kvarn::QuantizeArgs a{};
    a.D = layout->head_dim;
    a.T = layout->tile_tokens;
    a.k_bits = layout->k_bits;
    a.v_bits = layout->v_bits;
    a.n_iters = layout->n_iters;
    a.H = layout->num_kv_heads;
    a.mla = layout->mla;
    a.k_fp16 = cache->k_fp16;
    a.v_fp16 = cache->v_fp16;
    a.k_records = cache->k_records;
    a.v_records = cache->v_records;
    a.src = src_fpages;
    a.dst = dst_qpages;
    a.n = n;
    a.n_fpages = cache->n_fpages;
    a.n_qpages = cache->n_qpages;
    a.R = layout->rope_dim;
    a.rope_fp16 = cache->rope_fp16;
    a.rope_records = cache->rope_records;
    hipError_t e = kvarn::launch_quantize(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KVARN_EHIP, "quantize launch failed: %s", hipGetErrorString(e));
    return ok();
}

size_t kvarn_decode_workspace_bytes(const kvarn_layout* layout, int32_t batch, int32_t num_q_heads,
                                    int32_t max_pages) {
    return decode_workspace(layout, batch, 1, 0, num_q_heads, max_pages);
}

size_t kvarn_decode_workspace_bytes_mq(const kvarn_layout* layout, int32_t batch, int32_t num_q_tokens,
                                       int32_t num_q_heads, int32_t max_pages) {
    if (num_q_tokens < 1 || num_q_tokens > 4) {
        fail(KVARN_EINVAL, "num_q_tokens %d outside 1..4", num_q_tokens);
        return 0;
    }
    return decode_workspace(layout, batch, num_q_tokens, 1, num_q_heads, max_pages);
}

kvarn_status kvarn_decode_attn(const kvarn_layout* layout, const kvarn_cache* cache, const kvarn_page_table* pages,
                               const void* q, int32_t q_dtype, int32_t num_q_heads, float sm_scale, float* out,
                               void* workspace, size_t workspace_bytes, void* stream) {
    return decode_common(layout, cache, pages, q, q_dtype, 1, 0, num_q_heads, sm_scale, out, workspace,
                         workspace_bytes, stream);
}

kvarn_status kvarn_decode_attn_mq(const kvarn_layout* layout, const kvarn_cache* cache,
                                  const kvarn_page_table* pages, const void* q, int32_t q_dtype,
                                  int32_t num_q_tokens, int32_t num_q_heads, float sm_scale, float* out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    if (num_q_tokens < 1 || num_q_tokens > 4)
        return fail(KVARN_EINVAL, "num_q_tokens %d outside 1..4 (a verify step checks at most four tokens a row)",
                    num_q_tokens);
    return decode_common(layout, cache, pages, q, q_dtype, num_q_tokens, 1, num_q_heads, sm_scale, out, workspace,
                         workspace_bytes, stream);
}

kvarn_status kvarn_append(const kvarn_layout* layout, const kvarn_cache* cache, const kvarn_page_table* pages,
                          const void* k_new, const void* v_new, int32_t dtype, int32_t n_new, void* stream) {
    kvarn_status st = check_layout(layout);
    if (st != KVARN_OK) return st;
    if (!cache || !pages) return fail(KVARN_EINVAL, "NULL argument");
    if (dtype != KVARN_F32 && dtype != KVARN_F16 && dtype != KVARN_BF16)
        return fail(KVARN_EINVAL, "dtype %d: float32, float16 or bfloat16", dtype);
    if (n_new < 0) return fail(KVARN_EINVAL, "n_new %d < 0", n_new);
    if (pages->batch < 1 || pages->max_pages < 1 || !pages->block_table || !pages->seq_lens)
        return fail(KVARN_EINVAL, "page table: batch and max_pages must be >= 1, arrays non-NULL");
    if (n_new == 0) return ok();
    if (!k_new || (!layout->mla && !v_new)) return fail(KVARN_EINVAL, "new key / value arrays are NULL");
    if (!cache->k_fp16 || (!layout->mla && !cache->v_fp16)) return fail(KVARN_EINVAL, "fp16 pools are NULL");
    if (!aligned16(k_new) || (!layout->mla && !aligned16(v_new)) || !aligned16(cache->k_fp16) ||
        (!layout->mla && !aligned16(cache->v_fp16)))
        return fail(KVARN_EINVAL, "new tokens and fp16 pools must be 16-byte aligned");
    if (cache->n_fpages < 1) return fail(KVARN_EINVAL, "empty fp16 pool");
    st = check_rope_pools(layout, cache, false);
    if (st != KVARN_OK) return st;
    const int64_t threads =
        (int64_t)pages->batch * n_new * layout->num_kv_heads * ((layout->head_dim + layout->rope_dim) / 8);
    if (threads > ((int64_t)1 << 40)) return fail(KVARN_EINVAL, "too many new values in one call");
    kvarn::AppendArgs a{};
    a.D = layout->head_dim;
    a.T = layout->tile_tokens;
    a.H = layout->num_kv_heads;
    a.B = pages->batch;
    a.n_new = n_new;
    a.max_pages = pages->max_pages;
    a.dtype = dtype;
    a.R = layout->rope_dim;
    a.rope_fp16 = cache->rope_fp16;
    a.k_new = k_new;
    a.v_new = layout->mla ? nullptr : v_new;
    a.k_fp16 = cache->k_fp16;
    a.v_fp16 = layout->mla ? nullptr : cache->v_fp16;
    a.block_table = pages->block_table;
    a.seq_lens = pages->seq_lens;
    a.n_fpages = cache->n_fpages;
    hipError_t e = kvarn::launch_append(a, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KVARN_EHIP, "append launch failed: %s", hipGetErrorString(e));
    return ok();
}

kvarn_status kvarn_commit(const kvarn_layout* layout, const kvarn_cache* cache, int32_t* block_table,
                          int32_t* seq_lens, int32_t batch, int32_t max_pages, const int32_t* n_accept,
                          const int32_t* new_qpages, int32_t* promoted_fpages, void* stream) {
    kvarn_status st = check_layout(layout);
    if (st != KVARN_OK) return st;
    if (!cache || !block_table || !seq_lens || !n_accept || !new_qpages || !promoted_fpages)
        return fail(KVARN_EINVAL, "NULL argument");
    if (batch < 1 || max_pages < 1) return fail(KVARN_EINVAL, "batch and max_pages must be >= 1");
    if (!cache->k_fp16 || !cache->k_records || (!layout->mla && (!cache->v_fp16 || !cache->v_records)))
        return fail(KVARN_EINVAL, "pools are NULL");
    if (!aligned16(cache->k_fp16) || !aligned16(cache->k_records) ||
        (!layout->mla && (!aligned16(cache->v_fp16) || !aligned16(cache->v_records))))
        return fail(KVARN_EINVAL, "pools must be 16-byte aligned");
    if (cache->n_fpages < 1 || cache->n_qpages < 1) return fail(KVARN_EINVAL, "empty pools");
    if ((int64_t)batch * layout->num_kv_heads * (layout->mla ? 1 : 2) > 0x7fffffffLL)
        return fail(KVARN_EINVAL, "batch x heads x (K, V) must fit one grid");
    st = check_rope_pools(layout, cache, true);
    if (st != KVARN_OK) return st;
    kvarn::CommitArgs c{};
    c.T = layout->tile_tokens;
    c.sink = layout->sink_tokens;
    c.tail = layout->tail_tokens;
    c.B = batch;
    c.max_pages = max_pages;
    c.block_table = block_table;
    c.seq_lens = seq_lens;
    c.n_accept = n_accept;
    c.new_qpages = new_qpages;
    c.promoted = promoted_fpages;
    c.n_fpages = cache->n_fpages;
    c.n_qpages = cache->n_qpages;
    kvarn::QuantizeArgs q{};
    q.D = layout->head_dim;
    q.T = layout->tile_tokens;
    q.k_bits = layout->k_bits;
    q.v_bits = layout->v_bits;
    q.n_iters = layout->n_iters;
    q.H = layout->num_kv_heads;
    q.mla = layout->mla;
    q.k_fp16 = cache->k_fp16;
    q.v_fp16 = cache->v_fp16;
    q.k_records = cache->k_records;
    q.v_records = cache->v_records;
    q.src = promoted_fpages;
    q.dst = new_qpages;
    q.n = batch;
    q.n_fpages = cache->n_fpages;
    q.n_qpages = cache->n_qpages;
    q.R = layout->rope_dim;
    q.rope_fp16 = cache->rope_fp16;
    q.rope_records = cache->rope_records;
    hipError_t e = kvarn::launch_commit(c, q, (hipStream_t)stream);
    if (e != hipSuccess) return fail(KVARN_EHIP, "commit launch failed: %s", hipGetErrorString(e));
    return ok();
}

const char* kvarn_last_error(void) { return g_err; }

const char* kvarn_version(void) { return "kvarn-mi355x 0.1"; }

}  // extern "C"
