// KVarN paged GQA decode attention: dispatch by head dim, tile and code
// widths; split plan and workspace size.  The kernels are in
// decode_gqa_impl.hpp.
#include "decode_gqa_impl.hpp"

namespace kvarn {
namespace {

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
    // a width of 3, 5 or 8 (instantiated in decode_gqa_w<D>.hip)
    auto even = [](int b) { return b == 2 || b == 4 || b == 6; };
    if (even(kb) && even(vb)) return hipErrorInvalidValue;
    switch (10 * kb + vb) {
#define KVARN_WIDE_CASE(KB, VB) \
    case 10 * KB + VB: return launch_gqa_wide<D, T, KB, VB>(a, st);
#define KVARN_WIDE_CASES_K(KB) \
    KVARN_WIDE_CASE(KB, 2) KVARN_WIDE_CASE(KB, 3) KVARN_WIDE_CASE(KB, 4) KVARN_WIDE_CASE(KB, 5) KVARN_WIDE_CASE(KB, 6) KVARN_WIDE_CASE(KB, 8)
#define KVARN_WIDE_CASES_ODDV(KB) KVARN_WIDE_CASE(KB, 3) KVARN_WIDE_CASE(KB, 5) KVARN_WIDE_CASE(KB, 8)
        KVARN_WIDE_CASES_K(3) KVARN_WIDE_CASES_K(5) KVARN_WIDE_CASES_K(8)
        KVARN_WIDE_CASES_ODDV(2) KVARN_WIDE_CASES_ODDV(4) KVARN_WIDE_CASES_ODDV(6)
#undef KVARN_WIDE_CASES_ODDV
#undef KVARN_WIDE_CASES_K
#undef KVARN_WIDE_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

void decode_plan(int D, int H, int G, int mla, int B, int max_pages, int T, int kb, int vb, int* nsplit,
                 int* pps) {
    (void)T; (void)kb; (void)vb;
    // GQA: as many waves as fit at once: three per SIMD (head_dim 128: 128
    // VGPRs, but the fp16 slots take the fourth; 256 and 512: up to 170 VGPRs,
    // splits of two and four waves).  MLA: one 8-wave workgroup per CU holds 64 heads,
    // so up to 128 heads take two workgroups per split.
    const int units = mla ? B * ((G + 63) / 64) : B * H * (G / 4);  // GQA: one per group of 4 query heads
    // (head_dim 128: 3584 one-wave workgroups, a seventh more than the 3072
    // resident at once, measured best: the splits' lengths vary with the
    // sequence lengths and the fp16 slots fill in behind them)
    const int target = mla ? 256 : (D == 128 ? 3584 : 3072 / (D / 128));  // workgroups
    int ns = (target + units - 1) / units;
    if (ns < 1) ns = 1;
    // MLA: a split holds its page ids in two registers, 128 at most (with the
    // quantized and fp16 pages dealt separately, ceil(max_pages / 126) splits
    // keep every split within that)
    if (mla && ns < (max_pages + 125) / 126) ns = (max_pages + 125) / 126;
    if (ns > max_pages) ns = max_pages;
    if (ns < 1) ns = 1;
    int p = (max_pages + ns - 1) / ns;
    if (p < 1) p = 1;
    *pps = p;
    *nsplit = (max_pages + p - 1) / p;
    if (*nsplit < 1) *nsplit = 1;
}

int decode_fp16_slots(int T, int sink, int tail, int max_pages) {
    // fp16 tokens of a sequence: fewer than sink + tail + T (with quantized
    // pages: sink + tail + T - 1 at most), the sink a whole number of pages;
    // one slot per 64-token part of such a page
    const int n = sink / T + (tail + 2 * T - 2) / T;
    return (n < max_pages ? n : max_pages) * (T / 64);
}

// fp32 rotated queries [B][Hq][D], then split partials
// [B][Hq][nsplit + nfsplit][D + 4] (quantized-page splits with rotated-basis
// value sums, then fp16 slots with original-basis ones)
size_t decode_workspace_floats(int D, int Hq, int B, int nsplit, int nfsplit) {
    return (size_t)B * Hq * D + (size_t)B * Hq * (nsplit + nfsplit) * (D + 4);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
    if (a.mla) return launch_mla(a, st);
    if (a.G < 4 || a.G % 4 != 0 || a.GS != a.G / 4) return hipErrorInvalidValue;
    if (a.D == 128 && a.T == 128) return gqa_bits<128, 128>(a, st);
    if (a.D == 128 && a.T == 64) return gqa_bits<128, 64>(a, st);
    if (a.D == 256 && a.T == 128) return gqa_bits<256, 128>(a, st);
    if (a.D == 256 && a.T == 64) return gqa_bits<256, 64>(a, st);
    if (a.D == 512 && a.T == 128) return gqa_bits<512, 128>(a, st);
    if (a.D == 512 && a.T == 64) return gqa_bits<512, 64>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace kvarn
