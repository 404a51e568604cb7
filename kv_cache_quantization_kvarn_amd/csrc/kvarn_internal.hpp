// Internal launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvarn {

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
};

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t st);

// One kernel launch for keys and values (HASV) or the MLA latent alone;
// explicitly instantiated per head_dim in quantize_d<D>.hip.
template <int D, int T, int KB, int VB, bool HASV>
hipError_t launch_quantize_shape(const QuantizeArgs& a, hipStream_t st);

struct DecodeArgs {
    int D, T, k_bits, v_bits, sink, tail, H, mla;
    int G;            // query heads per KV head (MLA: all query heads)
    int B, Hq, max_pages;
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
    const void* q;
    int q_bf16;
    float sm_scale;
    float* out;
    float* ws;        // split partials
};

// Split plan shared by the workspace query and the launch.
void decode_plan(int D, int H, int G, int mla, int B, int max_pages, int T, int kb, int vb, int* nsplit,
                 int* pps);
// GQA: the most fp16 (sink and tail) pages a sequence can have.
int decode_fp16_slots(int T, int sink, int tail, int max_pages);
size_t decode_workspace_floats(int D, int Hq, int B, int nsplit, int nfsplit);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);

// MLA: fp16 rotated queries [B][Hq][512] then split partials [B][Hq][nsplit][516] fp32.
size_t mla_workspace_floats(int Hq, int B, int nsplit);
hipError_t launch_mla(const DecodeArgs& a, hipStream_t st);

}  // namespace kvarn
