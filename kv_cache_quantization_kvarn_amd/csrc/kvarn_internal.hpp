// Internal launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvarn {

// Record a message for kvarn_last_error() on this thread and return st.
int32_t set_error(int32_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

struct QuantizeArgs {
    int D, T, k_bits, v_bits, n_iters, H, mla;
    const void* k_fp16;
    const void* v_fp16;
    void* k_records;
    void* v_records;
    const int32_t* src;
    const int32_t* dst;
    int32_t n;
    int64_t n_fpages, n_qpages;
    int R;                    // MLA rope sidecar width (0: none)
    const void* rope_fp16;    // fp16 [n_fpages][T][R]: rope keys of the fp16 pages
    void* rope_records;       // fp16 [n_qpages][T][R]: rope keys of the record pages
};

// Quantize the pages, and with a rope sidecar copy each page's rope keys to
// its record page.
hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t st);

// One kernel launch for keys and values (HASV) or the MLA latent alone;
// explicitly instantiated per head_dim in quantize_d<D>.hip.
template <int D, int T, int KB, int VB, bool HASV>
hipError_t launch_quantize_shape(const QuantizeArgs& a, hipStream_t st);
// Keys (token-major) or values (channel-major) alone, any width 2..8.
template <int D, int T, int BITS, bool CHMAJOR>
hipError_t launch_quantize_one(const QuantizeArgs& a, hipStream_t st);

struct DecodeArgs {
    int D, T, k_bits, v_bits, sink, tail, H, mla;
    int G;            // query heads per KV head (MLA: all query heads)
    int GS;           // GQA: groups of 4 query heads per KV head (G / 4); one grid row each
    int B, Hq, max_pages;  // B: query rows = sequences x query tokens (row b = sequence b / M, token b % M)
    int M;            // query tokens per sequence (1 for a plain decode step)
    int causal;       // 0: every row attends the seq_lens tokens; 1: token i of a sequence sits at
                      // position seq_lens + i and attends seq_lens + i + 1 tokens (its own included)
    int nsplit;       // splits of each sequence (GQA: over its quantized pages)
    int nfsplit;      // GQA: fp16 slots (64-token parts of fp16 pages) of each sequence, one workgroup each
    int pps;          // pages per split
    const void* k_records;
    const void* v_records;
    const void* k_fp16;
    const void* v_fp16;
    int64_t n_qpages, n_fpages;
    const int32_t* block_table;
    const int32_t* seq_lens;
    const void* q;    // [B][Hq][D + R]
    int q_dtype;      // 0 float32, 1 float16, 2 bfloat16
    int R;            // MLA rope sidecar width (0: none, 64)
    const void* rope_records;  // fp16 [n_qpages][T][R]
    const void* rope_fp16;     // fp16 [n_fpages][T][R]
    float sm_scale;
    float* out;
    float* ws;        // split partials
};

// Attend length of query row b: the region rule uses seq_lens of its sequence
// (committed tokens); a causal row also sees the uncommitted query tokens up
// to and including its own.
__device__ __forceinline__ int attend_len(const DecodeArgs& a, int b, int L, int cap) {
    if (!a.causal) return L;
    const int A = L + (b % a.M) + 1;
    return A < cap ? A : cap;
}

// Split plan shared by the workspace query and the launch.
void decode_plan(int D, int H, int G, int mla, int B, int max_pages, int T, int kb, int vb, int* nsplit,
                 int* pps);
// GQA: the most fp16 (sink and tail) pages a sequence can have.
int decode_fp16_slots(int T, int sink, int tail, int max_pages);
size_t decode_workspace_floats(int D, int Hq, int B, int nsplit, int nfsplit);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);
// GQA with a code width of 3, 5 or 8: the fp16-MFMA split kernel at any head
// dim; instantiated per head dim in decode_gqa_w<D>.hip.
template <int D, int T, int KB, int VB>
hipError_t launch_gqa_wide(const DecodeArgs& a, hipStream_t st);

struct AppendArgs {
    int D, T, H, B, n_new, max_pages, dtype;  // dtype: 0 f32, 1 f16, 2 bf16
    int R;              // MLA rope sidecar width: k_new rows hold D + R values
    const void* k_new;
    const void* v_new;  // NULL for MLA
    void* k_fp16;
    void* v_fp16;       // NULL for MLA
    void* rope_fp16;    // fp16 [n_fpages][T][R] (R > 0)
    const int32_t* block_table;
    const int32_t* seq_lens;
    int64_t n_fpages;
};
hipError_t launch_append(const AppendArgs& a, hipStream_t st);

struct CommitArgs {
    int T, sink, tail, B, max_pages;
    int32_t* block_table;
    int32_t* seq_lens;
    const int32_t* n_accept;
    const int32_t* new_qpages;
    int32_t* promoted;
    int64_t n_fpages, n_qpages;
};
// plan kernel, quantize of the promoted pages (q.src = promoted,
// q.dst = new_qpages, q.n = B), apply kernel
hipError_t launch_commit(const CommitArgs& a, const QuantizeArgs& q, hipStream_t st);

// MLA: fp16 rotated queries [B][Hq][512] then split partials [B][Hq][nsplit][516] fp32.
size_t mla_workspace_floats(int Hq, int B, int nsplit);
hipError_t launch_mla(const DecodeArgs& a, hipStream_t st);

}  // namespace kvarn
