// KVarN MLA decode for gfx950: one 512-wide int4 latent record per token
// serves as key and value for all query heads (evermx.com KVarN review,
// paragraph on MLA models: the compressed KV latent is quantized to int4).
//
// The heads share every latent element, so the path is a pair of GEMMs per
// 32-token chunk on the 16x16x32 fp16 MFMA:
//   S[h][t] = q'_h . y_t        O[h][j] += sum_t P[h][t] y_tj
// with q' = H q (rotated once, per sequence and head, by qrot_kernel) and
// y_t the record read back in the rotated basis, y_tj = C_j (S_t c_tj + Zp_t).
// Each chunk is read back once into LDS (fp16) and used by all heads; it never
// goes to HBM.  fp16 sink and tail chunks stay in the original basis (q' . y
// = q . x for the orthonormal H): the plain query meets the stored rows, and
// their value sums form a second partial of the split.  The softmax rescales
// O lazily: only when a head's running maximum grows by more than 2^8, which
// keeps every weight below 256.  The combine applies H once, to the rotated
// partials.
//
// Workgroup: 8 waves (two per SIMD) per (head group of up to 64 heads,
// split, sequence).  Scores: waves 0..3 own one head block (16 heads) each
// while waves 4..7 read the next chunk back; then every wave forms the value
// sums of the previous chunk, so one barrier per chunk separates the stages.
// Value sums: each wave owns 64 of the 512 channels for all the group's
// heads; their operands come from LDS through ds_read_b64_tr_b16 (4 rows x 16
// columns of halves transposed per 16 lanes).
#include <math.h>

#include "decode_combine.hpp"
#include "kvarn_device.hpp"
#include "kvarn_internal.hpp"

namespace kvarn {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int MD = 512;        // latent width
constexpr int CH = 32;         // tokens per chunk
constexpr float kLazy = 8.0f;  // rescale when the maximum grows by more than this (log2 units)
constexpr float kFloor = -1.0e30f;  // finite stand-in for a running maximum of -inf

#define LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

__device__ __forceinline__ h4 tr16(const void* p) {
    s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS(s4, p));
    return __builtin_bit_cast(h4, v);
}

// LDS layout of a read-back chunk: token rows of YROW = 1 KB (512 halves),
// the 16-byte unit u of token t at position u ^ (t & 15) of its row.  The
// gfx950 LDS serves a 128-bit access 16 lanes at a time from 64 banks; the
// swizzle puts the units of 16 consecutive tokens in one column on 16
// different 4-bank groups, so the score operand reads (16 tokens, one unit)
// and the read-back stores (8 tokens, two units 8 apart) are free of bank
// conflicts.  (Padded rows of 1040, 1056 or 1088 bytes measured 1.8x slower
// for the score reads.)
constexpr int YROW = 2 * 512;
__device__ __forceinline__ int yoff(int t, int u) { return t * YROW + 16 * (u ^ (t & 15)); }
// position of piece k (16 bytes) of a token's 256-byte code row in a ring
// slot: the 8 tokens (t & 7) read by 8 lanes for one piece, and the two
// pieces 2 apart of lanes 8 further on, land on 16 different bank groups
__device__ __forceinline__ int cswz(int t) { return (t & 1) | ((t & 6) << 1); }
// 0, as a value the compiler cannot see through.  Taken once per chunk
// (right after a barrier, where the wait the compiler puts before inline asm
// costs nothing) and XOR-ed into the lane keys of the swizzled addresses, it
// makes them chunk-local: each stage forms its few addresses per chunk
// instead of all of them being hoisted out of the chunk loop, one register
// each.
__device__ __forceinline__ int opaque_zero() {
    int z = 0;
    asm volatile("" : "+v"(z));
    return z;
}
// Within a 16-byte unit the eight channels are held in the order
// 0,4,1,5,2,6,3,7 (the order in which packed nibbles unpack to fp16 pairs);
// position p holds channel upos(p).
__device__ __forceinline__ int upos(int p) { return (p >> 1) + 4 * (p & 1); }
// weights: token rows of 160 bytes, with 128 more bytes after every 8 rows
__device__ __forceinline__ int poff(int t) { return t * 160 + (t >> 3) * 128; }
constexpr int PBYTES = 31 * 160 + 3 * 128 + 128;

__device__ __forceinline__ h8 cat(h4 a, h4 b) {
    return h8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// max over the 16 lanes of a row for 4 values: fused v_max_f32_dpp (each
// value's next DPP read comes 4 instructions after its write; s_nop 1 covers
// the write just before the block)
__device__ __forceinline__ void rmax16x4(float (&v)[4]) {
#define KVARN_RMAX4(CTRL)                                                                          \
    "v_max_f32_dpp %0, %0, %0 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
    "v_max_f32_dpp %1, %1, %1 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
    "v_max_f32_dpp %2, %2, %2 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                          \
    "v_max_f32_dpp %3, %3, %3 " CTRL " row_mask:0xf bank_mask:0xf\n\t"
    asm volatile("s_nop 1\n\t" KVARN_RMAX4("row_ror:8") KVARN_RMAX4("row_ror:4") KVARN_RMAX4("row_ror:2")
                     KVARN_RMAX4("row_ror:1")
                 : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
#undef KVARN_RMAX4
}

__device__ __forceinline__ float rsum16(float v) {
    v += i2f(__builtin_amdgcn_update_dpp(0, f2i(v), 0x128, 0xF, 0xF, true));
    v += i2f(__builtin_amdgcn_update_dpp(0, f2i(v), 0x124, 0xF, 0xF, true));
    v += i2f(__builtin_amdgcn_update_dpp(0, f2i(v), 0x122, 0xF, 0xF, true));
    v += i2f(__builtin_amdgcn_update_dpp(0, f2i(v), 0x121, 0xF, 0xF, true));
    return v;
}

// q' = H q / sqrt(D) as fp16, one workgroup per (sequence, head); query rows
// of W elements (the latent query first: W = D, or D + R with a rope sidecar).
__global__ void __launch_bounds__(256) qrot_kernel(const void* __restrict__ q, int q_dtype, int W,
                                                   _Float16* __restrict__ qr) {
    __shared__ float x[MD];
    const int bh = blockIdx.x;
    for (int j = threadIdx.x; j < MD; j += 256) x[j] = q_at(q, q_dtype, (int64_t)bh * W + j);
    __syncthreads();
    for (int hs = 1; hs < MD; hs <<= 1) {
        const int k = threadIdx.x;  // 256 butterflies per stage
        const int i0 = (k / hs) * 2 * hs + (k % hs), i1 = i0 + hs;
        const float a = x[i0], b = x[i1];
        __syncthreads();
        x[i0] = a + b;
        x[i1] = a - b;
        __syncthreads();
    }
    const float rs = 1.0f / sqrtf((float)MD);
    for (int j = threadIdx.x; j < MD; j += 256) qr[(int64_t)bh * MD + j] = (_Float16)(x[j] * rs);
}

// Workgroup of 8 waves, two per SIMD.  Waves 0..3 ("score waves") own one
// head block (16 heads) each: scores over a whole chunk, its softmax and its
// weights.  Waves 4..7 read the next chunk back meanwhile.  All 8 waves form
// the value sums of the chunk before, wave w for channels CPW*w .. CPW*w +
// CPW - 1 of every head.
template <int HB>
struct MlaShape {
    static_assert(HB >= 1 && HB <= 4, "a workgroup holds at most 64 heads");
    static constexpr int NWV = 8;
    static constexpr int NT = NWV * 64;
    static constexpr int CPW = MD / NWV;   // PV channels per wave
    static constexpr int CBW = CPW / 16;   // PV channel blocks per wave
    static constexpr int HQ = HB * 16;
};

// Work of a split: the quantized pages of the sequence are cut into nsplit
// contiguous ranges, and the fp16 pages (sink, then tail) are dealt to the
// splits round-robin, so every split gets the same share of both kinds.
// A split runs its quantized chunks first, software-pipelined (their loads
// stream through an LDS ring; between two barriers chunk c + 1 is read back
// and chunk c scored, and the value sums of chunk c - 1 are formed), then its
// fp16 chunks.  Chunk s (the quantized ones, then the fp16 ones) uses read-back
// buffer s mod 3 (quantized) or 1 and 2 in turn (fp16), weight and rescale
// buffers s mod 2 and rescale flag s mod 3.
//
// ROPE: a 64-wide fp16 rope key beside each latent (DeepSeek-style MLA; the
// latent alone is quantized, evermx.com KVarN review, MLA paragraph) adds
// <q_rope, r_t> to every score.  A chunk's rope keys (4 KB) come by LDS-DMA
// into rbuf[s mod 3] one iteration ahead of its score, one load for each of
// waves 0..3 per chunk (so their fixed wait count rises by one); they take two
// more k-steps per token half of the score MFMAs, with the rope query (fp16,
// natural channel order) as their A operand.
template <int T, int HB, bool ROPE>
__global__ void __launch_bounds__(MlaShape<HB>::NT) mla_split_kernel(DecodeArgs a) {
    using SH = MlaShape<HB>;
    constexpr int NWV = SH::NWV, CPW = SH::CPW, CBW = SH::CBW, HQ = SH::HQ;
    constexpr int KCB = T * MD / 2;                // int4 code bytes of a record
    constexpr int KREC = KCB + 4 * T + 2 * MD;
    constexpr int WS = MD + 4;                     // partial: m, l, pad, pad, O[512]
    constexpr int CPP = T / CH;                    // chunks per page
    static_assert(HQ * 2 <= 160, "weight rows hold at most 64 heads");
    __shared__ __attribute__((aligned(16))) uint8_t ybuf[3][CH * YROW];  // chunks, rotated basis (fp16)
    __shared__ __attribute__((aligned(16))) uint8_t pbuf[2][PBYTES];      // weights [token][head] (fp16)
    __shared__ float alpha[2][HQ];
    __shared__ int rescale_flag[3];
    // ring of chunk slots: codes, token scales (SSC), column scales (SCC)
    constexpr int NR = 4;
    constexpr int SSC = CH * MD / 2, SCC = SSC + 4 * CH, SLOT = SCC + 2 * MD;
    static_assert(SSC == NWV * 1024, "8 KB of codes a chunk: two 1 KB loads for each of waves 0..3");
    __shared__ __attribute__((aligned(16))) uint8_t ring[NR * SLOT];
    __shared__ __attribute__((aligned(16))) uint8_t scratch[16 * NWV];  // targets of the stand-in loads
    // rope keys of a chunk: token rows of RROW bytes, unit u of token t at
    // position u ^ ((t >> 1) & 7) (16 tokens read together lie on 16 bank groups)
    constexpr int RD = ROPE ? 64 : 0, RROW = 2 * RD;
    __shared__ __attribute__((aligned(16))) uint8_t rbuf[ROPE ? 3 : 1][ROPE ? CH * RROW : 16];

    // Workgroup id -> (head group hg, query token m, split, sequence bs).
    // Workgroups are dealt to the 8 XCDs round-robin; the head groups and the
    // query tokens of one (split, sequence) get ids 8 apart, so they run on
    // the same XCD at about the same time and read each latent chunk through
    // that XCD's L2.  Unit v = bs * nsplit + split; ids come in runs of 8 * nhg
    // per (v / 8, m).
    const int nhg = a.Hq / HQ;
    const int units = (a.B / a.M) * a.nsplit;
    const int wid = blockIdx.x;
    const int hg = (wid % (8 * nhg)) / 8;
    const int g8 = wid / (8 * nhg);
    const int mtok = g8 % a.M;
    const int v = (g8 / a.M) * 8 + (wid % 8);
    if (v >= units) return;
    // workgroup-uniform: held in scalar registers
    const int bs = __builtin_amdgcn_readfirstlane(v / a.nsplit);
    const int split = __builtin_amdgcn_readfirstlane(v - bs * a.nsplit);
    const int b = __builtin_amdgcn_readfirstlane(bs * a.M + mtok);  // query row
    const int h0 = __builtin_amdgcn_readfirstlane(hg * HQ);  // first query head of this workgroup
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const float sm2 = a.sm_scale * kLog2e;
    const bool qk_wave = wave < HB;     // score wave with a head block
    const bool rb_wave = wave >= 4;     // read-back wave
    // lane keys of yoff's swizzle: score operands (unit 4 j + g4 of token l16
    // at sk ^ 4 j) and value operands (unit 8 (wave & 1) + (q4 >> 1) of token
    // 8 g4 + (l16 >> 2) at ak)
    const int sk = g4 ^ l16;
    int zk = 0;  // opaque_zero(), renewed per chunk
    const int ak = (8 * (wave & 1) + ((l16 & 3) >> 1)) ^ ((8 * g4 + (l16 >> 2)) & 15);

    // rotated queries of this wave's head block, as QK A operands
    const _Float16* qr = reinterpret_cast<const _Float16*>(a.ws);  // q' at the start of the workspace
    h8 qa[16];
#pragma unroll
    for (int ks = 0; ks < 16; ks++) {
        if (qk_wave) {
            const _Float16* p = qr + ((int64_t)b * a.Hq + h0 + wave * 16 + l16) * MD + 32 * ks + 8 * g4;
            const h8 v = *reinterpret_cast<const h8*>(p);
            qa[ks] = h8{v[0], v[4], v[1], v[5], v[2], v[6], v[3], v[7]};  // unit order
        } else {
            qa[ks] = h8{0, 0, 0, 0, 0, 0, 0, 0};
        }
    }
    // rope query of this wave's head block (natural channel order), as the A
    // operand of two more k-steps: lane head l16, channels 32 kk + 8 g4 ..
    h8 qro[2] = {h8{0, 0, 0, 0, 0, 0, 0, 0}, h8{0, 0, 0, 0, 0, 0, 0, 0}};
    if constexpr (ROPE) {
        if (qk_wave) {
            const int64_t qi = ((int64_t)b * a.Hq + h0 + wave * 16 + l16) * (MD + RD) + MD + 8 * g4;
#pragma unroll
            for (int kk = 0; kk < 2; kk++) {
                float x[8];
                q_load<8>(a.q, a.q_dtype, qi + 32 * kk, x);
                qro[kk] = h8{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3],
                             (_Float16)x[4], (_Float16)x[5], (_Float16)x[6], (_Float16)x[7]};
            }
        }
    }
    if (tid < 3) rescale_flag[tid] = 0;

    f4 O[HB][CBW];
#pragma unroll
    for (int hb = 0; hb < HB; hb++)
#pragma unroll
        for (int c = 0; c < CBW; c++) O[hb][c] = f4{0.f, 0.f, 0.f, 0.f};
    // score waves: running max (log2 units) and per-lane partial sums, heads 16*wave + 4*g4 + i
    float mu[4], lp[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        mu[i] = -INFINITY;
        lp[i] = 0.f;
    }

    // regions by the committed length; the row attends its first A tokens
    const int Lc = min(a.seq_lens[bs], a.max_pages * T);
    const int L = attend_len(a, b, Lc, a.max_pages * T);
    const int npages = L > 0 ? (L + T - 1) / T : 0;
    const int nq = (Lc - a.sink - a.tail >= T) ? (Lc - a.sink - a.tail) / T : 0;
    const int sp = min(a.sink / T, npages);
    const int nf = npages - nq;                           // fp16 pages: sink, then tail
    const int qbeg = sp + (int)(((int64_t)nq * split) / a.nsplit);
    const int nqp = sp + (int)(((int64_t)nq * (split + 1)) / a.nsplit) - qbeg;   // quantized pages of the split
    const int nfp = nf > split ? (nf - split + a.nsplit - 1) / a.nsplit : 0;     // fp16 pages of the split
    auto fpage = [&](int j) {  // page of the split's j-th fp16 page
        const int f = split + j * a.nsplit;
        return f < sp ? f : sp + nq + (f - sp);
    };
    // the split's page ids (128 at most), entry k in lane k & 63 of pid[k >> 6]:
    // quantized pages first, then its fp16 pages; an id outside its pool
    // becomes -1 here, once, so the chunk loops test only the sign
    int pid[2];
#pragma unroll
    for (int r = 0; r < 2; r++) {
        const int k = 64 * r + lane;
        int id = -1;
        if (k < nqp) {
            id = a.block_table[(int64_t)bs * a.max_pages + qbeg + k];
            if ((int64_t)id >= a.n_qpages) id = -1;
        } else if (k < nqp + nfp) {
            id = a.block_table[(int64_t)bs * a.max_pages + fpage(k - nqp)];
            if ((int64_t)id >= a.n_fpages) id = -1;
        }
        pid[r] = id < 0 ? -1 : id;
        asm volatile("" ::"v"(pid[r]));  // loaded before any LDS-DMA load is in flight
    }
    auto page_id = [&](int k) {  // k wave-uniform, < 128
        const int x = __builtin_amdgcn_readlane(pid[0], k & 63), y = __builtin_amdgcn_readlane(pid[1], k & 63);
        return k < 64 ? x : y;
    };
#pragma unroll
    for (int ks = 0; ks < 16; ks++) asm volatile("" ::"v"(qa[ks]));
    asm volatile("" ::"v"(qro[0]), "v"(qro[1]));
    __syncthreads();

    // ---- score waves: scores, softmax and weights of chunk seq, held in yb
    // (32 tokens from sequence position tok0; positions past the sequence end
    // get weight 0).  Sets bit `wave` of rescale_flag[seq % 3] when a
    // running maximum of its head block moves. ----
    auto score = [&](const uint8_t* yb, const uint8_t* rb, int tok0, int seq) {
        // 32 k-steps (token half th = k >> 4, channels 32 (k & 15) ..), the B
        // operand loaded PF steps ahead; two accumulation chains per half
        constexpr int PF = 8;
        // unit 4 (k & 15) + g4 of token 16 (k >> 4) + l16: with yoff's swizzle,
        // 256 ((k & 15) >> 2) + 16 (sk ^ 4 (k & 3)) into the row
        const uint8_t* yrow = yb + l16 * YROW;
        auto ld = [&](int k) {
            const int pos = (sk ^ zk) ^ (4 * (k & 3));
            return *reinterpret_cast<const h8*>(yrow + 16 * pos + (16 * (k >> 4)) * YROW + 256 * ((k & 15) >> 2));
        };
        h8 by[PF];
#pragma unroll
        for (int k = 0; k < PF; k++) by[k] = ld(k);
        f4 acc[2][2] = {{f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}}, {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}}};
#pragma unroll
        for (int k = 0; k < 32; k++) {
            const h8 cur = by[k % PF];
            if (k + PF < 32) by[k % PF] = ld(k + PF);
            acc[k >> 4][k & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[k & 15], cur, acc[k >> 4][k & 1], 0, 0, 0);
        }
        if constexpr (ROPE) {  // unit 4 kk + g4 of token 16 th + l16's rope key, with rbuf's swizzle
            h8 br[2][2];
#pragma unroll
            for (int th = 0; th < 2; th++)
#pragma unroll
                for (int kk = 0; kk < 2; kk++)
                    br[th][kk] = *reinterpret_cast<const h8*>(rb + (16 * th + l16) * RROW +
                                                               16 * ((4 * kk + g4) ^ ((l16 >> 1) & 7)));
#pragma unroll
            for (int th = 0; th < 2; th++)
#pragma unroll
                for (int kk = 0; kk < 2; kk++)
                    acc[th][kk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qro[kk], br[th][kk], acc[th][kk], 0, 0, 0);
        }
        const f4 sacc[2] = {acc[0][0] + acc[0][1], acc[1][0] + acc[1][1]};
        // lane: heads 16*wave + 4*g4 + i, tokens 16*th + l16 of the chunk
        float s[2][4], cmax[4];
        if (tok0 + CH <= L) {  // uniform: every token of the chunk is in the sequence
#pragma unroll
            for (int th = 0; th < 2; th++)
#pragma unroll
                for (int i = 0; i < 4; i++) s[th][i] = sacc[th][i] * sm2;
        } else {
#pragma unroll
            for (int th = 0; th < 2; th++) {
                const bool valid = tok0 + 16 * th + l16 < L;
#pragma unroll
                for (int i = 0; i < 4; i++) s[th][i] = valid ? sacc[th][i] * sm2 : -INFINITY;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; i++) cmax[i] = fmaxf(s[0][i], s[1][i]);
        rmax16x4(cmax);
        bool need = false;
#pragma unroll
        for (int i = 0; i < 4; i++) need |= cmax[i] > mu[i] + kLazy;
        // The heads of a block see the same tokens: either every cmax is
        // finite (and a maximum of -inf, no token yet, moves) or none is.
        // Below, max(mu, kFloor) stands in for mu: with mu = -inf the factors
        // and the weights of the (then all -inf) scores come out as 0 from the
        // bare v_exp_f32.
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float mn = fmaxf(mu[i], cmax[i]);
                const float al = __builtin_amdgcn_exp2f(fmaxf(mu[i], kFloor) - mn);
                lp[i] *= al;
                mu[i] = mn;
                if (l16 == 0) alpha[seq & 1][16 * wave + 4 * g4 + i] = al;
            }
            // one bit per head block: only the blocks whose wave wrote new
            // factors are rescaled (the others' factor slots are stale)
            if (lane == 0) atomicOr(&rescale_flag[seq % 3], 1 << wave);
        }
        float mf[4];
#pragma unroll
        for (int i = 0; i < 4; i++) mf[i] = fmaxf(mu[i], kFloor);
#pragma unroll
        for (int th = 0; th < 2; th++) {
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                p[i] = __builtin_amdgcn_exp2f(s[th][i] - mf[i]);  // s <= mu + kLazy: p <= 256
                lp[i] += p[i];
            }
            const uint2 pk = make_uint2(float_to_half_bits(p[0]) | (float_to_half_bits(p[1]) << 16),
                                        float_to_half_bits(p[2]) | (float_to_half_bits(p[3]) << 16));
            *reinterpret_cast<uint2*>(pbuf[seq & 1] + poff(16 * th + l16) + 32 * wave + 8 * g4) = pk;
        }
    };
    // ---- all waves: O += P Y for this wave's channels, chunk seq held in yb
    // (after its weights are in pbuf[seq & 1]); clears the flag of chunk
    // seq + 2, which no wave reads or sets before the next barrier ----
    auto accumulate = [&](const uint8_t* yb, int seq) {
        const int flags = rescale_flag[seq % 3];
        if (flags) {
#pragma unroll
            for (int hb = 0; hb < HB; hb++) {
                if (!((flags >> hb) & 1)) continue;
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const float al = alpha[seq & 1][16 * hb + 4 * g4 + i];
#pragma unroll
                    for (int c = 0; c < CBW; c++) O[hb][c][i] *= al;
                }
            }
        }
        if (tid == 0) rescale_flag[(seq + 2) % 3] = 0;
        // tr16: lane 4k + q of a 16-lane group reads row k, columns 4q .. 4q+3;
        // lane j receives column j of the 4 rows.  Rows are tokens.
        // unit uu = 8 wave + 2 c + (q4 >> 1) of tokens row and row + 4 (row & 4 = 0):
        // with yoff's swizzle, 16 (wave >> 1) + (ak ^ 2 c ^ 4 h) into row + 4 h
        const int row = 8 * g4 + (l16 >> 2), q4 = l16 & 3;
        static_assert(CPW == 64, "a wave's channels are units 8 wave .. 8 wave + 7");
        const uint8_t* yrow = yb + row * YROW + 8 * (q4 & 1) + 256 * (wave >> 1);
        h8 bv[CBW];  // Y[32 tokens][16 channels]: lane channel l16, tokens 8*g4 .. +7
#pragma unroll
        for (int c = 0; c < CBW; c++) {
            const int p0 = (ak ^ zk) ^ (2 * c), p1 = (ak ^ zk) ^ (2 * c) ^ 4;
            bv[c] = cat(tr16(yrow + 16 * p0), tr16(yrow + 4 * YROW + 16 * p1));
        }
#pragma unroll
        for (int hb = 0; hb < HB; hb++) {
            // P[16 heads][32 tokens]: lane head l16, tokens 8*g4 .. +7
            const uint8_t* pb = pbuf[seq & 1];
            const h8 pa = cat(tr16(pb + poff(row) + 32 * hb + 8 * q4), tr16(pb + poff(row + 4) + 32 * hb + 8 * q4));
#pragma unroll
            for (int c = 0; c < CBW; c++) O[hb][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, bv[c], O[hb][c], 0, 0, 0);
        }
    };

    // ---- quantized chunks: chunk ci is page qbeg + ci / CPP, tokens
    // (ci % CPP) * CH .. +CH.  A ring of NR chunk slots in LDS is filled by
    // LDS-DMA loads: the codes, the token scales and, on a page's first
    // chunk, the column scales.  Waves 0..3 issue every load (2 KB of codes
    // each, then wave 0 the token scales and wave 1 the column scales), the
    // read-back waves none: their issue time would sit on the critical path,
    // while waves 0..3 otherwise wait at the chunk barrier.  Each of waves
    // 0..3 issues exactly three loads per chunk (a one-lane load into a
    // scratch line stands in for a load it has no use for), so a fixed
    // s_waitcnt vmcnt count before the barrier marks a chunk as landed for
    // the whole workgroup. ----
    const int nqc = nqp * CPP;
    auto qchunk = [&](int ci, int& page, int& c0, int& id) {
        page = qbeg + ci / CPP;
        c0 = (ci % CPP) * CH;
        id = page_id(ci / CPP);
    };
    const i32x4 rs = raw_buffer(a.k_records, (uint32_t)(a.n_qpages * KREC));
    const uint32_t ring_lds = lds_address(ring), dummy_lds = lds_address(scratch) + 16 * wave;
    auto issue_chunk = [&](int cj) {
        int page = 0, c0 = 0, id = -1;
        if (cj < nqc) qchunk(cj, page, c0, id);
        const bool q = id >= 0;
        const uint32_t sl = ring_lds + (uint32_t)((cj % NR) * SLOT);
        // byte offsets in the pool (below 4 GiB) as unsigned 32-bit values:
        // the buffer load adds its scalar offset modulo 2^32
        const uint32_t rec = q ? (uint32_t)id * (uint32_t)KREC : 0u;
        // slot piece 64 p + l (p = 2 wave + h, h = 0, 1) holds piece k ^
        // cswz(t) of token t's row (t = piece >> 4, k = piece & 15); both
        // loads under one M0, the second 1 KB further on
        if (q) {
            uint32_t vo[2];
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const int p = 2 * wave + h, pc = 64 * p + lane, t = pc >> 4;
                vo[h] = t * (MD / 2) + 16 * ((pc & 15) ^ cswz(t));
            }
            lds_dma16x2(sl + 2048 * wave, rs, vo[0], vo[1] - 1024u, (int)(rec + (uint32_t)(c0 * (MD / 2))));
        } else if (lane == 0) {
            lds_dma16(dummy_lds, rs, 0, 0);
            lds_dma16(dummy_lds, rs, 0, 0);
        }
        if (q && wave == 0) {
            if (lane < CH / 4) lds_dma16(sl + SSC, rs, 16 * lane, (int)(rec + (uint32_t)(KCB + 4 * c0)));
        } else if (q && wave == 1 && c0 == 0) {
            // unit u at position u ^ ((u >> 3) & 7): the 8 units 8 apart read at once by read_back lie on 8 bank groups
            lds_dma16(sl + SCC, rs, 16 * (lane ^ ((lane >> 3) & 7)), (int)(rec + (uint32_t)(KCB + 4 * T)));
        } else if (lane == 0) {
            lds_dma16(dummy_lds, rs, 0, 0);
        }
    };
    // rope keys of quantized chunk cj -> rbuf[cj % 3]: wave w (0..3) loads
    // tokens 8 w .. 8 w + 7 (position l & 7 of token 8 w + (l >> 3)); a
    // one-lane stand-in load where there is nothing to load
    const i32x4 rrs = raw_buffer(a.rope_records, ROPE ? (uint32_t)(a.n_qpages * T * RROW) : 0u);
    auto issue_rope = [&](int cj) {
        if constexpr (ROPE) {
            int page = 0, c0 = 0, id = -1;
            if (cj < nqc) qchunk(cj, page, c0, id);
            if (id >= 0) {
                const int t = 8 * wave + (lane >> 3);
                lds_dma16(lds_address(rbuf[cj % 3]) + 1024u * wave, rrs, t * RROW + 16 * ((lane & 7) ^ ((t >> 1) & 7)),
                          (int)(((uint32_t)id * (uint32_t)T + (uint32_t)c0) * (uint32_t)RROW));
            } else if (lane == 0) {
                lds_dma16(dummy_lds, rs, 0, 0);
            }
        }
    };
    // read-back waves: chunk ci (landed) -> ybuf[ci % 3], rotated basis, fp16.
    // Lane l of read-back wave 4 + v takes token tt = 8 v + (l & 7), units
    // 8 part .. +8 (channels 64 part ..) with part = l >> 3: the 8 lanes of an
    // 8-lane group hold 8 tokens of one column.  The column scales of a page
    // come from the slot of its first chunk and stay in registers (cvk) for
    // its later chunks: a split's chunks are read back in order.
    const int tt = 8 * ((wave - 4) & 3) + (lane & 7), part = (lane >> 3) & 7;
    uint4 cvk[8];  // column scales of the lane's 8 units, as fp16 pairs in unpacking order
#pragma unroll
    for (int q8 = 0; q8 < 8; q8++) cvk[q8] = make_uint4(0u, 0u, 0u, 0u);
    const int rk = (8 * (part & 1)) ^ (tt & 15);  // read-back store key: unit 8 part + q8 at 16 (part >> 1) + (rk ^ q8)
    auto read_back = [&](int ci) {
        int page, c0, id;
        qchunk(ci, page, c0, id);
        if (id < 0) return;
        const uint8_t* slot = ring + (ci % NR) * SLOT;
        uint8_t* yb = ybuf[ci % 3];
        const uint4* cpg = reinterpret_cast<const uint4*>(slot + SCC);
        uint32_t cw[8];
#pragma unroll
        for (int k = 0; k < 2; k++) {  // pieces 2 part + k of the token's row (see issue_chunk)
            const uint4 v = *reinterpret_cast<const uint4*>(slot + tt * (MD / 2) + 16 * ((2 * part + k) ^ cswz(tt)));
            cw[4 * k] = v.x; cw[4 * k + 1] = v.y; cw[4 * k + 2] = v.z; cw[4 * k + 3] = v.w;
        }
        const uint32_t szw = reinterpret_cast<const uint32_t*>(slot + SSC)[tt];
        // y = C (S c + Zp) in packed fp16: nibbles k and k + 4 of a code word
        // become the pair (1024 + c, 1024 + c') by or-ing in the exponent of 1024
        const h2 S2 = __builtin_bit_cast(h2, (szw & 0xffffu) * 0x10001u);
        const h2 Z2 = __builtin_bit_cast(h2, (szw >> 16) * 0x10001u);
        const h2 k1024 = h2{(_Float16)1024.0f, (_Float16)1024.0f};
        // the nibble mask and the exponent of 1024 in registers (an SGPR and a
        // VGPR), so that the and and the or fuse into one v_and_or_b32
        const uint32_t nmask = (uint32_t)__builtin_amdgcn_readfirstlane(0x000F000F + zk);
        uint32_t e1024 = 0x64006400u;
        asm volatile("" : "+v"(e1024));
        // the 32 pairs of a unit row stage by stage, so that their chains
        // interleave: codes as (1024 + c) pairs, then S c + Zp, then times C
        auto units = [&](const uint4 (&cvs)[8]) {
            h2 y[8][4];
#pragma unroll
            for (int q8 = 0; q8 < 8; q8++)
#pragma unroll
                for (int k = 0; k < 4; k++)
                    y[q8][k] = __builtin_bit_cast(h2, ((cw[q8] >> (4 * k)) & nmask) | e1024) - k1024;
#pragma unroll
            for (int q8 = 0; q8 < 8; q8++)
#pragma unroll
                for (int k = 0; k < 4; k++) y[q8][k] = __builtin_elementwise_fma(y[q8][k], S2, Z2);
#pragma unroll
            for (int q8 = 0; q8 < 8; q8++) {
                const uint32_t cs[4] = {cvs[q8].x, cvs[q8].y, cvs[q8].z, cvs[q8].w};
                uint32_t o[4];
#pragma unroll
                for (int k = 0; k < 4; k++) o[k] = __builtin_bit_cast(uint32_t, y[q8][k] * __builtin_bit_cast(h2, cs[k]));
                // yoff(tt, 8 part + q8) = 16 (part >> 1) + (rk ^ q8) into the row
                *reinterpret_cast<uint4*>(yb + tt * YROW + 256 * (part >> 1) + 16 * ((rk ^ zk) ^ q8)) =
                    make_uint4(o[0], o[1], o[2], o[3]);
            }
        };
        // a page's first chunk brings its column scales (uniform branch); they
        // are all read before the first store, which the compiler cannot tell
        // apart from these reads
        if (c0 == 0) {
#pragma unroll
            for (int q8 = 0; q8 < 8; q8++) {
                const uint4 c = cpg[8 * part + ((part ^ zk) ^ q8)];  // pairs (0,4) (1,5) (2,6) (3,7) of unit 8 part + q8
                cvk[q8] = make_uint4(__builtin_amdgcn_perm(c.z, c.x, 0x05040100u), __builtin_amdgcn_perm(c.z, c.x, 0x07060302u),
                                     __builtin_amdgcn_perm(c.w, c.y, 0x05040100u), __builtin_amdgcn_perm(c.w, c.y, 0x07060302u));
            }
        }
        units(cvk);
    };
    auto chunk_ok = [&](int ci) {
        int page, c0, id;
        qchunk(ci, page, c0, id);
        return id >= 0;
    };

    // loads of waves 0..3 in flight after the ones a wait needs: the codes
    // and scales of the next two chunks (three loads each), and with ROPE the
    // rope keys of the next chunk; the read-back waves have none in flight
    constexpr int VMW = 3 * (NR - 2) + (ROPE ? 1 : 0);
    if (!rb_wave) {
        issue_chunk(0);
        issue_rope(0);
#pragma unroll
        for (int cj = 1; cj < NR - 1; cj++) issue_chunk(cj);
    }
    if (nqc > 0) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(VMW) : "memory");  // chunk 0 has landed
        __syncthreads();
        zk = opaque_zero();
        if (rb_wave) read_back(0);
        __syncthreads();
    }
    // iteration ci: issue chunk ci + NR - 1 into the slot chunk ci - 1 used;
    // score chunk ci while chunk ci + 1 is read back, then the value sums of
    // chunk ci - 1 (iteration nqc only forms those of the last chunk)
    // The loop runs in two copies with the same loads and barriers, one for
    // the score waves and one for the others: the score waves' query operands
    // (qa, qro) are dead in the second, which leaves the read-back the
    // registers to keep its loads and unit chains in flight together.
    auto head = [&](int ci) {
        if (!rb_wave) {
            issue_rope(ci + 1);
            issue_chunk(ci + NR - 1);
        }
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(VMW) : "memory");  // chunk ci + 1 (and rope ci) have landed
        __syncthreads();
        zk = opaque_zero();
    };
    if (qk_wave) {
        for (int ci = 0; ci <= nqc; ci++) {
            head(ci);
            if (ci < nqc) {
                int page, c0, id;
                qchunk(ci, page, c0, id);
                if (id >= 0) score(ybuf[ci % 3], rbuf[ROPE ? ci % 3 : 0], page * T + c0, ci);
            }
            if (ci > 0 && chunk_ok(ci - 1)) accumulate(ybuf[(ci - 1) % 3], ci - 1);
        }
    } else {
        for (int ci = 0; ci <= nqc; ci++) {
            head(ci);
            if (rb_wave && ci + 1 < nqc) read_back(ci + 1);
            if (ci > 0 && chunk_ok(ci - 1)) accumulate(ybuf[(ci - 1) % 3], ci - 1);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may land in LDS after this point
    __syncthreads();

    // ---- partial results: m, l per head; O rows for this wave's channels.
    // Split s writes partial s (quantized chunks, rotated basis, channels in
    // unit order) and partial nsplit + s (fp16 chunks, original basis). ----
    float* wsp = a.ws + (int64_t)a.B * a.Hq * MD / 2;  // partials follow the fp16 queries
    const int64_t brow = (int64_t)b * a.Hq + h0;
    const int np = 2 * a.nsplit;
    auto write_partial = [&](int slot, bool plain) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float lt = rsum16(lp[i]);
            if (qk_wave && l16 == 0) {
                float* o = wsp + ((brow + 16 * wave + 4 * g4 + i) * np + slot) * WS;
                o[0] = mu[i];
                o[1] = lt;
            }
        }
#pragma unroll
        for (int hb = 0; hb < HB; hb++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                float* o = wsp + ((brow + 16 * hb + 4 * g4 + i) * np + slot) * WS + 4;
#pragma unroll
                for (int c = 0; c < CBW; c++)
                    o[CPW * wave + 16 * c + (plain ? l16 : 8 * (l16 >> 3) + upos(l16 & 7))] = O[hb][c][i];
            }
    };
    write_partial(split, false);

    // ---- fp16 chunks, in the original basis (q'.y = q.x): the plain query
    // against the stored rows, value sums into a fresh accumulator.  The 32 KB
    // of a chunk come by LDS-DMA loads one chunk ahead straight into the
    // read-back row layout of ybuf[1] or ybuf[2] (idle now; one 1 KB token
    // row per load, units swizzled as in yoff, channels in natural order
    // within a unit); rows past the sequence end
    // are zeroed instead (their weight is 0 and must not meet NaN). ----
#pragma unroll
    for (int i = 0; i < 4; i++) {
        mu[i] = -INFINITY;
        lp[i] = 0.f;
    }
#pragma unroll
    for (int hb = 0; hb < HB; hb++)
#pragma unroll
        for (int c = 0; c < CBW; c++) O[hb][c] = f4{0.f, 0.f, 0.f, 0.f};
    // the plain query of this wave's head block, natural channel order (set in
    // every wave, so that no earlier value of qa lives through the loop above)
#pragma unroll
    for (int ks = 0; ks < 16; ks++) qa[ks] = h8{0, 0, 0, 0, 0, 0, 0, 0};
    if (qk_wave && nfp > 0) {
        const int64_t qi = ((int64_t)b * a.Hq + h0 + wave * 16 + l16) * (MD + RD) + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < 16; ks++) {
            float x[8];
            q_load<8>(a.q, a.q_dtype, qi + 32 * ks, x);
            qa[ks] = h8{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3],
                        (_Float16)x[4], (_Float16)x[5], (_Float16)x[6], (_Float16)x[7]};
        }
    }
    static_assert(CH * MD * 2 <= CH * YROW, "an fp16 chunk fits a read-back buffer");
    const i32x4 rf = raw_buffer(a.k_fp16, (uint32_t)(a.n_fpages * T * MD * 2));
    const i32x4 rfr = raw_buffer(a.rope_fp16, ROPE ? (uint32_t)(a.n_fpages * T * RROW) : 0u);
    auto fchunks = [&](int j) {  // chunks holding tokens of the split's j-th fp16 page (0: none or a bad id)
        const int page = fpage(j);
        if (page_id(nqp + j) < 0) return 0;
        return (min(L - page * T, T) + CH - 1) / CH;
    };
    struct FChunk {
        int j, cc;
    };
    auto fnext = [&](FChunk f) {  // the split's next fp16 chunk (j == nfp: none)
        f.cc++;
        while (f.j < nfp && f.cc >= fchunks(f.j)) {
            f.j++;
            f.cc = 0;
        }
        return f;
    };
    auto issue_f = [&](FChunk f, int buf) {
        if (f.j >= nfp) return;
        const int id = page_id(nqp + f.j);
        const uint32_t base = ((uint32_t)id * (uint32_t)T + (uint32_t)(f.cc * CH)) * (uint32_t)(MD * 2);
        const int nvalid = min(CH, L - (fpage(f.j) * T + f.cc * CH));  // >= 1
        uint8_t* yb = ybuf[1 + buf];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int t = 4 * wave + i;  // token of the chunk
            // LDS position l of row t holds unit l ^ (t & 15)
            if (t < nvalid) lds_dma16(lds_address(yb) + (uint32_t)(t * YROW), rf, 16 * (lane ^ (t & 15)), (int)(base + 1024u * t));
            else *reinterpret_cast<uint4*>(yb + yoff(t, lane)) = make_uint4(0u, 0u, 0u, 0u);
        }
        if constexpr (ROPE) {  // the chunk's 32 rope keys (rows past the end only meet scores set to -inf)
            if (lane < 32) {
                const int t = 4 * wave + (lane >> 3);
                lds_dma16(lds_address(rbuf[buf]) + 512u * wave, rfr, t * RROW + 16 * ((lane & 7) ^ ((t >> 1) & 7)),
                          (int)(((uint32_t)id * (uint32_t)T + (uint32_t)(f.cc * CH)) * (uint32_t)RROW));
            }
        }
    };
    int fseq = nqc;  // chunk numbering continues from the quantized chunks
    FChunk fc = fnext(FChunk{0, -1});
    int fb = 0;
    issue_f(fc, 0);
    while (fc.j < nfp) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this chunk has landed
        __syncthreads();
        zk = opaque_zero();
        const FChunk fn = fnext(fc);
        issue_f(fn, fb ^ 1);  // the other buffer's last reader finished before the barrier above
        const uint8_t* yb = ybuf[1 + fb];
        if (qk_wave) score(yb, rbuf[ROPE ? fb : 0], fpage(fc.j) * T + fc.cc * CH, fseq);
        __syncthreads();
        accumulate(yb, fseq);
        fseq++;
        fb ^= 1;
        fc = fn;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    write_partial(a.nsplit + split, true);
}

template <int T, int HB>
hipError_t launch_mla_t(const DecodeArgs& a, hipStream_t st) {
    if (a.R != 0 && a.R != 64) return hipErrorInvalidValue;
    hipLaunchKernelGGL(qrot_kernel, dim3(a.B * a.Hq), dim3(256), 0, st, a.q, a.q_dtype, MD + a.R,
                       reinterpret_cast<_Float16*>(a.ws));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nhg = a.Hq / (16 * HB);
    const int units = (a.B / a.M) * a.nsplit;
    const int blocks = ((units + 7) / 8) * 8 * nhg * a.M;
    if (a.R) hipLaunchKernelGGL((mla_split_kernel<T, HB, true>), dim3(blocks), dim3(MlaShape<HB>::NT), 0, st, a);
    else hipLaunchKernelGGL((mla_split_kernel<T, HB, false>), dim3(blocks), dim3(MlaShape<HB>::NT), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // partials s < nsplit: quantized chunks, rotated basis; s >= nsplit: fp16 chunks, original basis
    const float* wsp = a.ws + (int64_t)a.B * a.Hq * MD / 2;
    return launch_split_merge<MD>(wsp, a.out, a.B * a.Hq, a.nsplit, 2 * a.nsplit, st);
}

template <int T>
hipError_t launch_mla_hb(const DecodeArgs& a, hipStream_t st) {
    switch (a.Hq) {
        case 16: return launch_mla_t<T, 1>(a, st);
        case 32: return launch_mla_t<T, 2>(a, st);
        case 64: return launch_mla_t<T, 4>(a, st);
        case 128: return launch_mla_t<T, 4>(a, st);  // two 64-head workgroups
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

size_t mla_workspace_floats(int Hq, int B, int nsplit) {
    // fp16 queries, then two partials per split (quantized and fp16 chunks)
    return (size_t)B * Hq * MD / 2 + (size_t)B * Hq * 2 * nsplit * (MD + 4);
}

hipError_t launch_mla(const DecodeArgs& a, hipStream_t st) {
    if (a.D != MD || a.k_bits != 4) return hipErrorInvalidValue;
    if (a.T == 128) return launch_mla_hb<128>(a, st);
    if (a.T == 64) return launch_mla_hb<64>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace kvarn
