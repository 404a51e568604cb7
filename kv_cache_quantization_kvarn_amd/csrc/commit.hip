// Append and commit: the serving-side steps around the hot path.
//
// append  writes each decode step's new keys and values (or MLA latents) into
//         the fp16 pages after the sequence's committed tokens; seq_lens is
//         not changed, so tokens that are never accepted simply stay unused
//         and the next append overwrites them.
// commit  advances seq_lens by the accepted counts and, where that moves a
//         page out of the fp16 tail (the region rule: whole pages after the
//         fp16 sink, leaving at least `tail` newest tokens in fp16), quantizes
//         that page into a record page the caller supplies and points the
//         block table at it.  A page is promoted only once every one of its
//         tokens is committed (evermx.com KVarN review, MLA and hybrid
//         paragraph: only fully accepted blocks are quantized; gmlx "KV cache
//         quantization", "The two schemes": the newest tokens stay fp16).
//
// Everything stays on the device: the per-sequence decisions are taken by a
// one-thread-per-sequence kernel, the promoted pages go through the quantize
// kernel (pages with nothing to promote are skipped by its id check), and a
// last kernel writes the block table and the lengths.
#include "kvarn_device.hpp"
#include "kvarn_internal.hpp"

namespace kvarn {
namespace {

// quantized pages of a sequence of L tokens: whole T-token pages after the
// sink leaving at least `tail` tokens
__device__ __forceinline__ int64_t nq_of(int64_t L, int T, int sink, int tail) {
    const int64_t r = L - sink - tail;
    return r >= T ? r / T : 0;
}

// 8 consecutive values of the source dtype -> 8 fp16 (round to nearest even)
template <int DT>
__device__ __forceinline__ uint4 load8_as_f16(const void* src, int64_t e) {
    if constexpr (DT == 1) {  // fp16: a plain copy
        return *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + e);
    } else {
        float f[8];
        if constexpr (DT == 0) {
            const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + e);
            const float4 a = p[0], b = p[1];
            f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w; f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
        } else {  // bf16: the upper half of an fp32
            const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + e);
            const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int k = 0; k < 4; k++) {
                f[2 * k] = __builtin_bit_cast(float, w[k] << 16);
                f[2 * k + 1] = __builtin_bit_cast(float, w[k] & 0xffff0000u);
            }
        }
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; k++) o[k] = float_to_half_bits(f[2 * k]) | (float_to_half_bits(f[2 * k + 1]) << 16);
        return make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// thread = 8 channels of one (sequence b, new token i, head h); with an MLA
// rope sidecar (R > 0, H = 1) a new row holds the D latent channels, then
// the R rope channels, which go to the rope pool
template <int DT>
__global__ void append_kernel(const void* __restrict__ knew, const void* __restrict__ vnew,
                              uint16_t* __restrict__ kpool, uint16_t* __restrict__ vpool, uint16_t* __restrict__ rpool,
                              const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int B,
                              int n_new, int H, int D, int R, int T, int max_pages, int64_t n_fpages) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int per_row = (D + R) / 8;
    const int64_t total = (int64_t)B * n_new * H * per_row;
    if (idx >= total) return;
    const int c8 = (int)(idx % per_row);
    int64_t r = idx / per_row;
    const int h = (int)(r % H);
    r /= H;
    const int i = (int)(r % n_new);
    const int b = (int)(r / n_new);
    const int L = seq_lens[b];
    if (L < 0) return;
    const int64_t pos = (int64_t)L + i;
    const int64_t p = pos / T;
    if (p >= max_pages) return;
    const int id = block_table[(int64_t)b * max_pages + p];
    if (id < 0 || (int64_t)id >= n_fpages) return;
    const int64_t src = (((int64_t)b * n_new + i) * H + h) * (D + R) + 8 * c8;
    if (8 * c8 >= D) {  // rope channels (R > 0: MLA, H = 1)
        const int64_t rdst = ((int64_t)id * T + (pos % T)) * R + (8 * c8 - D);
        *reinterpret_cast<uint4*>(rpool + rdst) = load8_as_f16<DT>(knew, src);
        return;
    }
    const int64_t dst = (((int64_t)id * H + h) * T + (pos % T)) * D + 8 * c8;
    *reinterpret_cast<uint4*>(kpool + dst) = load8_as_f16<DT>(knew, src);
    if (vpool) *reinterpret_cast<uint4*>(vpool + dst) = load8_as_f16<DT>(vnew, src);
}

// per-sequence decision: promoted[b] = the fp16 page id to quantize (>= 0),
// -1 nothing to promote, -2 accepted count outside [0, T] or past the page
// table, -3 a page id outside its pool
__global__ void commit_plan_kernel(const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens,
                                   const int32_t* __restrict__ n_accept, const int32_t* __restrict__ new_qpages,
                                   int32_t* __restrict__ promoted, int B, int max_pages, int T, int sink, int tail,
                                   int64_t n_fpages, int64_t n_qpages) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const int a = n_accept[b];
    const int L = seq_lens[b];
    int out = -1;
    if (a < 0 || a > T || L < 0 || (int64_t)L + a > (int64_t)max_pages * T) {
        out = -2;
    } else {
        const int64_t nq1 = nq_of((int64_t)L + a, T, sink, tail);
        if (nq1 > nq_of(L, T, sink, tail)) {
            const int64_t p = sink / T + nq1 - 1;
            const int src = block_table[(int64_t)b * max_pages + p];
            const int dst = new_qpages[b];
            out = (src < 0 || (int64_t)src >= n_fpages || dst < 0 || (int64_t)dst >= n_qpages) ? -3 : src;
        }
    }
    promoted[b] = out;
}

__global__ void commit_apply_kernel(int32_t* __restrict__ block_table, int32_t* __restrict__ seq_lens,
                                    const int32_t* __restrict__ n_accept, const int32_t* __restrict__ new_qpages,
                                    const int32_t* __restrict__ promoted, int B, int max_pages, int T, int sink,
                                    int tail) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const int st = promoted[b];
    if (st < -1) return;  // refused: the sequence is left as it was
    const int L = seq_lens[b];
    const int a = n_accept[b];
    if (st >= 0) {
        const int64_t p = sink / T + nq_of((int64_t)L + a, T, sink, tail) - 1;
        block_table[(int64_t)b * max_pages + p] = new_qpages[b];
    }
    seq_lens[b] = L + a;
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t st) {
    const int64_t total = (int64_t)a.B * a.n_new * a.H * ((a.D + a.R) / 8);
    if (total == 0) return hipSuccess;
    if (a.R > 0 && (a.H != 1 || a.v_fp16 || !a.rope_fp16)) return hipErrorInvalidValue;
    const int threads = 256;
    const int64_t blocks = (total + threads - 1) / threads;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    auto* kp = static_cast<uint16_t*>(a.k_fp16);
    auto* vp = static_cast<uint16_t*>(a.v_fp16);
    auto* rp = static_cast<uint16_t*>(a.rope_fp16);
#define KVARN_APPEND(DT)                                                                                     \
    hipLaunchKernelGGL(append_kernel<DT>, dim3((unsigned)blocks), dim3(threads), 0, st, a.k_new, a.v_new, kp, vp, \
                       rp, a.block_table, a.seq_lens, a.B, a.n_new, a.H, a.D, a.R, a.T, a.max_pages, a.n_fpages)
    switch (a.dtype) {
        case 0: KVARN_APPEND(0); break;
        case 1: KVARN_APPEND(1); break;
        case 2: KVARN_APPEND(2); break;
        default: return hipErrorInvalidValue;
    }
#undef KVARN_APPEND
    return hipGetLastError();
}

hipError_t launch_commit(const CommitArgs& a, const QuantizeArgs& q, hipStream_t st) {
    const int threads = 256;
    const unsigned blocks = (unsigned)((a.B + threads - 1) / threads);
    hipLaunchKernelGGL(commit_plan_kernel, dim3(blocks), dim3(threads), 0, st, a.block_table, a.seq_lens,
                       a.n_accept, a.new_qpages, a.promoted, a.B, a.max_pages, a.T, a.sink, a.tail, a.n_fpages,
                       a.n_qpages);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_quantize(q, st);  // src = promoted (negative: skipped), dst = new_qpages
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(commit_apply_kernel, dim3(blocks), dim3(threads), 0, st, a.block_table, a.seq_lens,
                       a.n_accept, a.new_qpages, a.promoted, a.B, a.max_pages, a.T, a.sink, a.tail);
    return hipGetLastError();
}

}  // namespace kvarn
