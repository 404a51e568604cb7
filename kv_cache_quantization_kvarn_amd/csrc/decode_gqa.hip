// KVarN paged GQA decode attention for gfx950: split-K partials + combine.
//
// The records are never dequantized to memory (evermx.com KVarN review,
// method paragraph: scales folded back in at read time).  With the rotated
// query q' = H q and, per record, the column scales C, per-token scale S_t
// and zero-point Zp_t:
//   score_t  = <q, k_t> = S_t <q' * C, code_t> + Zp_t * sum(q' * C)
//   sum_t p_t v_t = H ( C_V * ( sum_t (p_t S_t) code_t + sum_t p_t Zp_t ) )
// so each split accumulates the value sum in the rotated basis and the
// combine applies H once.  fp16 sink and tail pages (gmlx "KV cache
// quantization", "The two schemes") are accumulated in the original basis
// into a second sum that the combine adds after the rotation.
//
// Split kernel: one workgroup of four waves per (split, KV head, sequence);
// each wave walks 64-token groups of the split's pages with its own online
// softmax, and the waves are merged through LDS at the end.  Scores use
// lane = token; value sums use lane = channel (channels CPL*lane .. +CPL-1).
#include <math.h>

#include "kvarn_device.hpp"
#include "kvarn_internal.hpp"

namespace kvarn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// code k of a little-endian LSB-first stream held in 32-bit words w[]
template <int B>
__device__ __forceinline__ uint32_t code_at(const uint32_t* w, int k) {
    const int bit = k * B;
    const int wd = bit >> 5, off = bit & 31;
    uint32_t v = w[wd] >> off;
    if (off + B > 32) v |= w[wd + 1] << (32 - off);
    return v & ((1u << B) - 1u);
}

template <int D, int T, int KB, int VB>
__global__ void __launch_bounds__(256) decode_split_kernel(DecodeArgs a) {
    constexpr int G = 4;
    constexpr int NWV = 4;
    constexpr int CPL = D / 64;   // channels per lane in the value sums
    constexpr int GPP = T / 64;   // 64-token groups per page
    constexpr int KCB = T * D * KB / 8;
    constexpr int VCB = T * D * VB / 8;
    constexpr int KREC = KCB + 4 * T + 2 * D;
    constexpr int VREC = VCB + 4 * T + 2 * D;
    constexpr int KROW = D * KB / 8;            // code bytes of one token (token-major K)
    constexpr int SCB = (KB == 6) ? 48 : 16;    // bytes per inner chunk
    constexpr int SCC = SCB * 8 / KB;           // codes per inner chunk
    constexpr int VCH = 64 * VB / 8;            // code bytes of one channel over 64 tokens
    constexpr int WS = 2 * D + 4;

    __shared__ float4 qrot[D];        // rotated query (4 heads per channel)
    __shared__ float4 qpl[D];         // plain query
    __shared__ float4 qt[NWV][D];     // per wave: rotated query times column scales
    __shared__ float4 pp[NWV][64];    // per wave: softmax weights (times S for records)
    __shared__ float mlbuf[NWV][2 * G];
    __shared__ float abuf[2][G][2 * D];

    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Hq = a.Hq;
    const float sm2 = a.sm_scale * kLog2e;   // scores in log2 units

    // ---- query: load 4 heads, rotate (unnormalized butterflies in LDS) ----
    float* qr = reinterpret_cast<float*>(qrot);
    float* qp = reinterpret_cast<float*>(qpl);
    for (int e = tid; e < G * D; e += 256) {
        const int g = e / D, j = e - g * D;
        const int64_t idx = ((int64_t)b * Hq + h * G + g) * D + j;
        float v;
        if (a.q_bf16) v = __builtin_bit_cast(float, ((uint32_t)static_cast<const uint16_t*>(a.q)[idx]) << 16);
        else v = static_cast<const float*>(a.q)[idx];
        qp[j * G + g] = v;
        qr[j * G + g] = v;
    }
    __syncthreads();
    for (int hs = 1; hs < D; hs <<= 1) {
        for (int e = tid; e < G * D / 2; e += 256) {
            const int g = e / (D / 2), k = e - g * (D / 2);
            const int i0 = (k / hs) * 2 * hs + (k % hs), i1 = i0 + hs;
            const float x = qr[i0 * G + g], y = qr[i1 * G + g];
            qr[i0 * G + g] = x + y;
            qr[i1 * G + g] = x - y;
        }
        __syncthreads();
    }
    const float rs = 1.0f / sqrtf((float)D);
    for (int e = tid; e < G * D; e += 256) qr[e] *= rs;
    __syncthreads();

    // ---- walk the split's 64-token groups ----------------------------------
    // a length beyond the page table is clamped to it (never read past a row)
    const int L = min(a.seq_lens[b], a.max_pages * T);
    const int npages = L > 0 ? (L + T - 1) / T : 0;
    const int nq = (L - a.sink - a.tail >= T) ? (L - a.sink - a.tail) / T : 0;
    const int sp = a.sink / T;
    const int pbeg = split * a.pps;
    const int pend = min(pbeg + a.pps, npages);
    const int ngroups = pend > pbeg ? (pend - pbeg) * GPP : 0;

    float m[G], l[G], accr[G][CPL], accp[G][CPL];
#pragma unroll
    for (int g = 0; g < G; g++) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; c++) accr[g][c] = accp[g][c] = 0.f;
    }

    for (int gi = wave; gi < ngroups; gi += NWV) {
        const int page = pbeg + gi / GPP;
        const int half = gi % GPP;
        const int tip = half * 64 + lane;          // token within the page
        const bool valid = page * T + tip < L;
        const bool quant = page >= sp && page < sp + nq;
        const int id = a.block_table[(int64_t)b * a.max_pages + page];
        if (id < 0 || (quant ? (int64_t)id >= a.n_qpages : (int64_t)id >= a.n_fpages)) continue;

        float s[G];
        const uint8_t* rv = nullptr;
        if (quant) {
            const uint8_t* rk = static_cast<const uint8_t*>(a.k_records) + ((int64_t)id * a.H + h) * KREC;
            rv = static_cast<const uint8_t*>(a.v_records) + ((int64_t)id * a.H + h) * VREC;
            // fold the key column scales into the rotated query
            const uint16_t* ck = reinterpret_cast<const uint16_t*>(rk + KCB + 4 * T);
            float sq[G] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < CPL; c++) {
                const int j = CPL * lane + c;
                const float cj = half_bits_to_float(ck[j]);
                const float4 qv = qrot[j];
                const float4 t4 = make_float4(qv.x * cj, qv.y * cj, qv.z * cj, qv.w * cj);
                qt[wave][j] = t4;
                sq[0] += t4.x; sq[1] += t4.y; sq[2] += t4.z; sq[3] += t4.w;
            }
#pragma unroll
            for (int g = 0; g < G; g++) sq[g] = wave_sum_all(sq[g]);
            wave_sync();
            float raw[G] = {0.f, 0.f, 0.f, 0.f};
            const uint8_t* kc = rk + (int64_t)tip * KROW;
#pragma unroll 1
            for (int ch = 0; ch < D / SCC; ch++) {
                uint32_t w[SCB / 4 + 1];
#pragma unroll
                for (int k = 0; k < SCB / 16; k++) {
                    const uint4 v = reinterpret_cast<const uint4*>(kc + ch * SCB)[k];
                    w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
                }
                w[SCB / 4] = 0;
#pragma unroll
                for (int k = 0; k < SCC; k++) {
                    const float cv = (float)code_at<KB>(w, k);
                    const float4 qv = qt[wave][ch * SCC + k];
                    raw[0] = fmaf(qv.x, cv, raw[0]);
                    raw[1] = fmaf(qv.y, cv, raw[1]);
                    raw[2] = fmaf(qv.z, cv, raw[2]);
                    raw[3] = fmaf(qv.w, cv, raw[3]);
                }
            }
            const uint32_t sz = reinterpret_cast<const uint32_t*>(rk + KCB)[tip];
            const float S = half_bits_to_float(sz & 0xffffu), Z = half_bits_to_float(sz >> 16);
#pragma unroll
            for (int g = 0; g < G; g++) s[g] = valid ? sm2 * fmaf(S, raw[g], Z * sq[g]) : -INFINITY;
        } else {
            const uint16_t* kp = static_cast<const uint16_t*>(a.k_fp16) +
                                 (((int64_t)id * a.H + h) * T + tip) * D;
            float raw[G] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
            for (int ch = 0; ch < D / 8; ch++) {
                const uint4 v = reinterpret_cast<const uint4*>(kp)[ch];
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int k = 0; k < 8; k++) {
                    const float kv = half_bits_to_float((w[k >> 1] >> (16 * (k & 1))) & 0xffffu);
                    const float4 qv = qpl[ch * 8 + k];
                    raw[0] = fmaf(qv.x, kv, raw[0]);
                    raw[1] = fmaf(qv.y, kv, raw[1]);
                    raw[2] = fmaf(qv.z, kv, raw[2]);
                    raw[3] = fmaf(qv.w, kv, raw[3]);
                }
            }
#pragma unroll
            for (int g = 0; g < G; g++) s[g] = valid ? sm2 * raw[g] : -INFINITY;
        }

        // ---- online softmax (log2 domain) ----
        float p[G];
#pragma unroll
        for (int g = 0; g < G; g++) {
            const float mx = wave_max_all(s[g]);
            const float mnew = fmaxf(m[g], mx);
            float alpha;
            if (mnew == -INFINITY) {
                alpha = 1.f;
                p[g] = 0.f;
            } else {
                alpha = exp2f(m[g] - mnew);
                p[g] = valid ? exp2f(s[g] - mnew) : 0.f;
            }
            l[g] = fmaf(l[g], alpha, wave_sum_all(p[g]));
            m[g] = mnew;
#pragma unroll
            for (int c = 0; c < CPL; c++) {
                accr[g][c] *= alpha;
                accp[g][c] *= alpha;
            }
        }

        if (quant) {
            const uint32_t szv = reinterpret_cast<const uint32_t*>(rv + VCB)[tip];
            const float Sv = half_bits_to_float(szv & 0xffffu), Zv = half_bits_to_float(szv >> 16);
            float z[G];
#pragma unroll
            for (int g = 0; g < G; g++) z[g] = wave_sum_all(p[g] * Zv);
            pp[wave][lane] = make_float4(p[0] * Sv, p[1] * Sv, p[2] * Sv, p[3] * Sv);
            wave_sync();
            const uint16_t* cvp = reinterpret_cast<const uint16_t*>(rv + VCB + 4 * T);
#pragma unroll
            for (int c = 0; c < CPL; c++) {
                const int j = CPL * lane + c;
                const uint8_t* vc = rv + ((int64_t)j * T + half * 64) * VB / 8;
                uint32_t w[VCH / 4 + 1];
#pragma unroll
                for (int k = 0; k < VCH / 16; k++) {
                    const uint4 v = reinterpret_cast<const uint4*>(vc)[k];
                    w[4 * k] = v.x; w[4 * k + 1] = v.y; w[4 * k + 2] = v.z; w[4 * k + 3] = v.w;
                }
                w[VCH / 4] = 0;
                float ag[G] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int t = 0; t < 64; t++) {
                    const float cv = (float)code_at<VB>(w, t);
                    const float4 pv = pp[wave][t];
                    ag[0] = fmaf(pv.x, cv, ag[0]);
                    ag[1] = fmaf(pv.y, cv, ag[1]);
                    ag[2] = fmaf(pv.z, cv, ag[2]);
                    ag[3] = fmaf(pv.w, cv, ag[3]);
                }
                const float cj = half_bits_to_float(cvp[j]);
#pragma unroll
                for (int g = 0; g < G; g++) accr[g][c] = fmaf(cj, ag[g] + z[g], accr[g][c]);
            }
        } else {
            pp[wave][lane] = make_float4(p[0], p[1], p[2], p[3]);
            wave_sync();
            const uint16_t* vp = static_cast<const uint16_t*>(a.v_fp16) +
                                 (((int64_t)id * a.H + h) * T + half * 64) * D + CPL * lane;
#pragma unroll 4
            for (int t = 0; t < 64; t++) {
                const float4 pv = pp[wave][t];
                float vv[CPL];
                if constexpr (CPL == 2) {
                    const uint32_t w = *reinterpret_cast<const uint32_t*>(vp + (int64_t)t * D);
                    vv[0] = half_bits_to_float(w & 0xffffu);
                    vv[1] = half_bits_to_float(w >> 16);
                } else if constexpr (CPL == 4) {
                    const uint2 w = *reinterpret_cast<const uint2*>(vp + (int64_t)t * D);
                    vv[0] = half_bits_to_float(w.x & 0xffffu); vv[1] = half_bits_to_float(w.x >> 16);
                    vv[2] = half_bits_to_float(w.y & 0xffffu); vv[3] = half_bits_to_float(w.y >> 16);
                } else {
                    const uint4 w = *reinterpret_cast<const uint4*>(vp + (int64_t)t * D);
                    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                    for (int k = 0; k < 8; k++) vv[k] = half_bits_to_float((ww[k >> 1] >> (16 * (k & 1))) & 0xffffu);
                }
#pragma unroll
                for (int c = 0; c < CPL; c++) {
                    accp[0][c] = fmaf(pv.x, vv[c], accp[0][c]);
                    accp[1][c] = fmaf(pv.y, vv[c], accp[1][c]);
                    accp[2][c] = fmaf(pv.z, vv[c], accp[2][c]);
                    accp[3][c] = fmaf(pv.w, vv[c], accp[3][c]);
                }
            }
        }
        wave_sync();
    }

    // ---- merge the four waves ----------------------------------------------
    if (lane == 0) {
#pragma unroll
        for (int g = 0; g < G; g++) {
            mlbuf[wave][g] = m[g];
            mlbuf[wave][G + g] = l[g];
        }
    }
    __syncthreads();
    float M[G], Ls[G];
#pragma unroll
    for (int g = 0; g < G; g++) {
        float mm = -INFINITY;
#pragma unroll
        for (int w = 0; w < NWV; w++) mm = fmaxf(mm, mlbuf[w][g]);
        float ll = 0.f;
        if (mm != -INFINITY) {
#pragma unroll
            for (int w = 0; w < NWV; w++) ll += mlbuf[w][G + g] * exp2f(mlbuf[w][g] - mm);
        }
        M[g] = mm;
        Ls[g] = ll;
        const float sc = (m[g] == -INFINITY) ? 0.f : exp2f(m[g] - mm);
#pragma unroll
        for (int c = 0; c < CPL; c++) {
            accr[g][c] *= sc;
            accp[g][c] *= sc;
        }
    }
    // tree: waves 2,3 -> 0,1; then 1 -> 0
#pragma unroll
    for (int round = 0; round < 2; round++) {
        const int lo = round == 0 ? 2 : 1;
        const int hi = round == 0 ? 4 : 2;
        if (wave >= lo && wave < hi) {
#pragma unroll
            for (int g = 0; g < G; g++)
#pragma unroll
                for (int c = 0; c < CPL; c++) {
                    abuf[wave - lo][g][CPL * lane + c] = accr[g][c];
                    abuf[wave - lo][g][D + CPL * lane + c] = accp[g][c];
                }
        }
        __syncthreads();
        if (wave < lo) {
#pragma unroll
            for (int g = 0; g < G; g++)
#pragma unroll
                for (int c = 0; c < CPL; c++) {
                    accr[g][c] += abuf[wave][g][CPL * lane + c];
                    accp[g][c] += abuf[wave][g][D + CPL * lane + c];
                }
        }
        __syncthreads();
    }
    if (wave == 0) {
#pragma unroll
        for (int g = 0; g < G; g++) {
            float* o = a.ws + (((int64_t)b * Hq + h * G + g) * a.nsplit + split) * WS;
            if (lane == 0) {
                o[0] = M[g];
                o[1] = Ls[g];
            }
#pragma unroll
            for (int c = 0; c < CPL; c++) {
                o[4 + CPL * lane + c] = accr[g][c];
                o[4 + D + CPL * lane + c] = accp[g][c];
            }
        }
    }
}

// One workgroup per (sequence, query head): merge the splits, rotate the
// record part back once, add the fp16 part, normalize.
template <int D>
__global__ void __launch_bounds__(D) decode_combine_kernel(const float* __restrict__ ws, float* __restrict__ out,
                                                            int nsplit) {
    constexpr int WS = 2 * D + 4;
    __shared__ float x[D];
    const int bh = blockIdx.x;
    const int j = threadIdx.x;
    const float* base = ws + (int64_t)bh * nsplit * WS;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; s++) M = fmaxf(M, base[s * WS]);
    float Ls = 0.f, r = 0.f, pl = 0.f;
    if (M != -INFINITY) {
        for (int s = 0; s < nsplit; s++) {
            const float ms = base[s * WS];
            if (ms == -INFINITY) continue;
            const float e = exp2f(ms - M);
            Ls = fmaf(base[s * WS + 1], e, Ls);
            r = fmaf(base[s * WS + 4 + j], e, r);
            pl = fmaf(base[s * WS + 4 + D + j], e, pl);
        }
    }
    x[j] = r;
    __syncthreads();
    for (int hs = 1; hs < D; hs <<= 1) {
        float v = x[j];
        float pv = x[j ^ hs];
        __syncthreads();
        x[j] = (j & hs) ? (pv - v) : (v + pv);
        __syncthreads();
    }
    const float o = Ls > 0.f ? (x[j] * (1.0f / sqrtf((float)D)) + pl) / Ls : 0.f;
    out[(int64_t)bh * D + j] = o;
}

template <int D, int T, int KB, int VB>
hipError_t launch_gqa(const DecodeArgs& a, hipStream_t st) {
    dim3 grid(a.nsplit, a.H, a.B);
    hipLaunchKernelGGL((decode_split_kernel<D, T, KB, VB>), grid, dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(a.B * a.Hq), dim3(D), 0, st, a.ws, a.out, a.nsplit);
    return hipGetLastError();
}

template <int D, int T>
hipError_t gqa_bits(const DecodeArgs& a, hipStream_t st) {
    const int kb = a.k_bits, vb = a.v_bits;
    if (kb == 4 && vb == 2) return launch_gqa<D, T, 4, 2>(a, st);
    if (kb == 4 && vb == 4) return launch_gqa<D, T, 4, 4>(a, st);
    if (kb == 6 && vb == 6) return launch_gqa<D, T, 6, 6>(a, st);
    if (kb == 2 && vb == 2) return launch_gqa<D, T, 2, 2>(a, st);
    if (kb == 6 && vb == 4) return launch_gqa<D, T, 6, 4>(a, st);
    if (kb == 4 && vb == 6) return launch_gqa<D, T, 4, 6>(a, st);
    if (kb == 6 && vb == 2) return launch_gqa<D, T, 6, 2>(a, st);
    if (kb == 2 && vb == 4) return launch_gqa<D, T, 2, 4>(a, st);
    if (kb == 2 && vb == 6) return launch_gqa<D, T, 2, 6>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace

void decode_plan(int D, int H, int G, int mla, int B, int max_pages, int T, int* nsplit, int* pps) {
    (void)D; (void)G; (void)T;
    // GQA: about four 4-wave workgroups per CU.  MLA: one 4-wave workgroup per
    // CU holds 64 heads (its accumulators fill the register file), so up to 128
    // heads take two workgroups per split.
    const int units = mla ? B * ((G + 63) / 64) : B * H;
    const int target = mla ? 256 : 1024;
    int ns = (target + units - 1) / units;
    if (ns < 1) ns = 1;
    if (ns > max_pages) ns = max_pages;
    if (ns < 1) ns = 1;
    int p = (max_pages + ns - 1) / ns;
    if (p < 1) p = 1;
    *pps = p;
    *nsplit = (max_pages + p - 1) / p;
    if (*nsplit < 1) *nsplit = 1;
}

size_t decode_workspace_floats(int D, int Hq, int B, int nsplit) {
    return (size_t)B * Hq * nsplit * (2 * D + 4);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
    if (a.mla) return launch_mla(a, st);
    if (a.D == 128 && a.T == 128) return gqa_bits<128, 128>(a, st);
    if (a.D == 128 && a.T == 64) return gqa_bits<128, 64>(a, st);
    if (a.D == 256 && a.T == 128) return gqa_bits<256, 128>(a, st);
    if (a.D == 256 && a.T == 64) return gqa_bits<256, 64>(a, st);
    if (a.D == 512 && a.T == 128) return gqa_bits<512, 128>(a, st);
    if (a.D == 512 && a.T == 64) return gqa_bits<512, 64>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace kvarn
