/*
 * kvarn.h -- C ABI of the KVarN (variance-normalized KV-cache quantization)
 * hot path on AMD Instinct MI355X (gfx950).
 *
 * Two operations:
 *   kvarn_quantize     turns full fp16 KV pages into KVarN records;
 *   kvarn_decode_attn  one decode step of paged GQA or MLA attention that
 *                      reads the records (and the fp16 sink and tail) directly.
 *
 * Method, as the pages describe it:
 *   - evermx.com review "KVarN vLLM KV-cache quantization", method paragraph:
 *     per fixed-size KV tile -- raw fp16 tile, orthonormal Hadamard rotation
 *     across channels, iterative Sinkhorn-like column/row standard-deviation
 *     normalization in log space, asymmetric round-to-nearest, scales folded
 *     back in at read time; preset kvarn_k4v2_g128 (4-bit K, 2-bit V,
 *     128-token tiles) and a 64-token-tile variant; MLA latent quantized to
 *     int4 (paragraph on MLA and hybrid models).
 *   - gmlx documentation "KV cache quantization", "The two schemes": each head
 *     Hadamard-rotated; records of 128 tokens; the first 128 tokens and the
 *     newest tail tokens (default 1024) stay fp16; widths 2..8.  "Which layers
 *     quantize": only head dimensions 128, 256 and 512; a model that cannot
 *     use the scheme is refused with a reason, never silently given another.
 *
 * Conventions of every entry point:
 *   - Pointers marked "device" are HIP device memory; "host" are host memory.
 *   - The library allocates and frees nothing and never synchronizes: work
 *     is enqueued on `stream` (a hipStream_t; NULL is the default stream) and
 *     runs asynchronously.  The caller owns every buffer and keeps it alive
 *     until the stream has run the work.  The only device state of the
 *     library is the fixed array of kvarn_decode_attn_noalloc.
 *   - Arguments are validated on the host before anything is enqueued.  A
 *     non-zero status means nothing was enqueued; kvarn_last_error() returns
 *     a message (per calling thread) saying why.  Unsupported shapes return
 *     KVARN_EUNSUPPORTED; there is no fallback path.
 *   - Device-side page ids are range-checked by the kernels: an id outside
 *     its pool makes the kernel skip that page (no out-of-bounds access); the
 *     affected outputs are then unspecified.
 *
 * Record format (one quantized page x one KV head x K or V; the latent for
 * MLA), all little-endian, record bytes = T*D*b/8 + 4*T + 2*D (a multiple of
 * 16 for every supported shape):
 *   [0, T*D*b/8)         codes, element e in bits [e*b, e*b+b), LSB first;
 *                        K and the MLA latent token-major (e = t*D + j),
 *                        V channel-major in blocks of TB = min(T, 64) tokens
 *                        (e = (t/TB)*TB*D + j*TB + t%TB: block by block, each
 *                        channel's TB codes in a row)
 *   next 4*T bytes       per token t: fp16 scale S_t, then fp16 zero-point Zp_t
 *   next 2*D bytes       per channel j: fp16 column scale C_j
 * A stored value reads back, in the rotated basis, as
 *   y_tj = C_j * (S_t * code_tj + Zp_t),  and in the original basis x_t = H y_t,
 * with H the natural-order Sylvester Hadamard matrix scaled by 1/sqrt(D).
 *
 * Pools:
 *   record pools  [n_qpages][H][record bytes]   (K and V separately)
 *   fp16 pools    [n_fpages][H][T][D] fp16       (K and V separately)
 *   MLA with a rope sidecar of R = rope_dim channels (the rotary-position key
 *   that DeepSeek-style MLA keeps beside the compressed latent; the latent is
 *   quantized to int4 -- evermx.com review, MLA paragraph -- and the rope key
 *   stays fp16):
 *   rope pools    [n_qpages][T][R] fp16 beside the records (rope_records) and
 *                 [n_fpages][T][R] fp16 beside the fp16 pages (rope_fp16);
 *                 a token's rope key sits in the pool of its page's region,
 *                 at the page id the block table gives for that page.
 *
 * Regions of a sequence of L tokens (page p covers tokens [p*T, p*T+T)):
 *   nq(L) = max(0, floor((L - sink - tail) / T)) quantized pages;
 *   pages p < sink/T                   fp16 sink        (fp16 pool)
 *   sink/T <= p < sink/T + nq(L)       quantized        (record pool)
 *   later pages                        fp16 tail, which keeps between `tail`
 *                                      and tail+T-1 tokens (fp16 pool)
 */
#ifndef KVARN_H
#define KVARN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvarn_status;
#define KVARN_OK 0
#define KVARN_EINVAL 1          /* bad argument (null pointer, negative size, ...) */
#define KVARN_EUNSUPPORTED 2    /* shape or width this library does not implement */
#define KVARN_EWORKSPACE 3      /* workspace missing or smaller than required */
#define KVARN_EHIP 4            /* the HIP runtime reported an error at launch */

#define KVARN_F32 0             /* query dtypes */
#define KVARN_F16 1
#define KVARN_BF16 2

/* Shape and policy of one layer's cache.  Value type, caller-owned. */
typedef struct kvarn_layout {
    int32_t head_dim;      /* D: 128, 256 or 512 (MLA latent: 512) ("Which layers quantize") */
    int32_t tile_tokens;   /* T = page size: 128 (g128) or 64 (g64) */
    int32_t k_bits;        /* key code width: 2, 3, 4, 5, 6 or 8 (gmlx "The two schemes"; MLA latent: 4) */
    int32_t v_bits;        /* value code width: 2, 3, 4, 5, 6 or 8; ignored when mla = 1 */
    int32_t n_iters;       /* normalization iterations (column step + row step), 1..32 */
    int32_t sink_tokens;   /* first tokens kept fp16; a multiple of T (default 128) */
    int32_t tail_tokens;   /* newest tokens kept fp16, >= 0 (default 1024) */
    int32_t num_kv_heads;  /* H >= 1; 1 when mla = 1 */
    int32_t mla;           /* 1: one latent record per token serves as key and value */
    int32_t rope_dim;      /* MLA only: width R of the fp16 rope key kept beside each latent,
                              0 (none) or 64; 0 when mla = 0 */
} kvarn_layout;

/* Device pools of one layer.  Caller-owned; all pointers 16-byte aligned. */
typedef struct kvarn_cache {
    void *k_records;       /* device, [n_qpages][H][kvarn_record_bytes(L, 0)] */
    void *v_records;       /* device, [n_qpages][H][kvarn_record_bytes(L, 1)]; NULL if mla */
    void *k_fp16;          /* device, fp16 [n_fpages][H][T][D] */
    void *v_fp16;          /* device, fp16 [n_fpages][H][T][D]; NULL if mla */
    int64_t n_qpages;      /* pages in each record pool */
    int64_t n_fpages;      /* pages in each fp16 pool */
    void *rope_records;    /* device, fp16 [n_qpages][T][rope_dim]; NULL if rope_dim = 0 */
    void *rope_fp16;       /* device, fp16 [n_fpages][T][rope_dim]; NULL if rope_dim = 0 */
} kvarn_cache;

/* Page table of a decode batch.  Caller-owned device arrays. */
typedef struct kvarn_page_table {
    const int32_t *block_table;  /* device, [batch][max_pages]: logical page -> id in the
                                    pool of that page's region (see "Regions" above) */
    const int32_t *seq_lens;     /* device, [batch]: tokens per sequence, 0..max_pages*T */
    int32_t batch;
    int32_t max_pages;
} kvarn_page_table;

/* Fill *out from a preset name "kvarn_k<kb>v<vb>_g<T>" (e.g. "kvarn_k4v2_g128",
 * "kvarn_k4v2_g64", "kvarn_k6v6_g128", "kvarn_k3v5_g64"), the flag names of the evermx.com
 * review ("--kv-cache-dtype kvarn_k4v2_g128"), with n_iters = 6,
 * sink_tokens = 128, tail_tokens = 1024 (gmlx "The two schemes"), mla = 0,
 * and head_dim = num_kv_heads = 0 for the caller to set.  Host-only. */
kvarn_status kvarn_parse_preset(const char *name, kvarn_layout *out);

/* Check a layout; KVARN_OK or the status and message the operations would
 * return for it.  Host-only. */
kvarn_status kvarn_layout_check(const kvarn_layout *layout);

/* Bytes of one record: which = 0 keys (or the MLA latent), 1 values.
 * 0 for an invalid layout.  Host-only. */
size_t kvarn_record_bytes(const kvarn_layout *layout, int32_t which);

/* nq(L): quantized pages of a sequence of seq_len tokens (see "Regions").
 * -1 for an invalid layout.  Host-only. */
int32_t kvarn_quantized_pages(const kvarn_layout *layout, int32_t seq_len);

/* Quantize n full pages: for i < n, the fp16 page src_fpages[i] (all H heads,
 * keys and values -- or the latent) becomes record page dst_qpages[i] of the
 * record pools.  Per tile of T tokens x D channels and head: rotation
 * Y = X H, n_iters column/row normalization steps on Y (root-mean-square
 * statistics), per-token round-to-nearest with scale = range/(2^b - 1) and
 * zero-point = minimum, codes packed as in the record format.
 * src_fpages, dst_qpages: device int32 [n].  The caller passes only pages
 * that are full and whose every token has been accepted (the commit rule of
 * the evermx.com review, MLA and hybrid paragraph) and distinct dst ids.  n = 0 is a
 * no-op.  Reads cache->k_fp16/v_fp16, writes cache->k_records/v_records; with
 * a rope sidecar also copies rope page src_fpages[i] of rope_fp16 to rope
 * page dst_qpages[i] of rope_records unchanged. */
kvarn_status kvarn_quantize(const kvarn_layout *layout, const kvarn_cache *cache,
                            const int32_t *src_fpages, const int32_t *dst_qpages,
                            int32_t n, void *stream);

/* Workspace bytes kvarn_decode_attn needs for this batch shape (split-K
 * partial results).  0 for invalid arguments.  Host-only. */
size_t kvarn_decode_workspace_bytes(const kvarn_layout *layout, int32_t batch,
                                    int32_t num_q_heads, int32_t max_pages);

/* One decode step: for every sequence b and query head h (KV head
 * h / (num_q_heads / H); MLA: the one latent),
 *   out[b][h] = sum_t softmax_t(sm_scale * <q[b][h], k_t>) v_t
 * over the L = seq_lens[b] tokens, with k_t, v_t read back from the records
 * (quantized region) or the fp16 pages (sink, tail).  The rotation is
 * applied once to q and once (inverse) to the output, and the scales are
 * folded into the score and value sums: no dequantized cache is written.
 * q: device [batch][num_q_heads][D] of q_dtype (KVARN_F32, KVARN_F16 or
 * KVARN_BF16; any other value is KVARN_EINVAL), 16-byte aligned.  MLA with a
 * rope sidecar: q is [batch][num_q_heads][D + R] (the latent query, then the
 * rope query), k_t is the pair (latent read-back, rope key) and
 *   <q, k_t> = <q_latent, latent_t> + <q_rope, rope_t>,
 * the value still the latent alone.
 * out: device fp32 [batch][num_q_heads][D], original basis; a sequence with
 * L = 0 gives zeros.  workspace: device, at least
 * kvarn_decode_workspace_bytes(...) bytes, 256-byte aligned; its contents
 * need no initialisation and are clobbered.  num_q_heads must be a multiple
 * of H (GQA: a group of any multiple of 4 query heads per KV head, at
 * most 65535 groups of 4 in all; MLA: 16, 32, 64 or 128).  With head_dim 128
 * (GQA) and with MLA each record pool, n_qpages * H * record bytes, must be
 * below 4 GiB, and with MLA the fp16 pool and the rope pools too; GQA takes at most 32767
 * sequences per call (KVARN_EUNSUPPORTED otherwise).  Negative pool sizes are
 * KVARN_EINVAL. */
kvarn_status kvarn_decode_attn(const kvarn_layout *layout, const kvarn_cache *cache,
                               const kvarn_page_table *pages, const void *q, int32_t q_dtype,
                               int32_t num_q_heads, float sm_scale, float *out,
                               void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes kvarn_decode_attn_mq needs; 0 for invalid arguments
 * (num_q_tokens outside 1..4 included).  Host-only. */
size_t kvarn_decode_workspace_bytes_mq(const kvarn_layout *layout, int32_t batch, int32_t num_q_tokens,
                                       int32_t num_q_heads, int32_t max_pages);

/* Decode of num_q_tokens (1..4) query tokens per sequence, causal among
 * themselves -- a speculative-decoding verify step, which checks at most
 * four tokens a row (gmlx "KV cache quantization", "Speed and speculative
 * decoding").  The query tokens are the newest tokens of each sequence,
 * appended (kvarn_append) but not committed: token i of sequence b sits at
 * position seq_lens[b] + i, and
 *   out[b][i][h] = sum_{t <= seq_lens[b] + i} softmax_t(sm_scale <q[b][i][h], k_t>) v_t.
 * The regions (see "Regions") follow seq_lens[b], the committed tokens, so
 * the query tokens and every token the causal mask drops lie in fp16 pages
 * (the commit rule keeps uncommitted tokens out of the records).  The
 * records of a sequence are read once for all its query tokens: the
 * workgroups of a sequence's tokens run on one XCD and share its L2.
 * q: device [batch][num_q_tokens][num_q_heads][D] of q_dtype; out: device
 * fp32 [batch][num_q_tokens][num_q_heads][D].  Workspace:
 * kvarn_decode_workspace_bytes_mq(...) bytes.  Everything else as
 * kvarn_decode_attn; batch * num_q_tokens is at most 32767 for GQA. */
kvarn_status kvarn_decode_attn_mq(const kvarn_layout *layout, const kvarn_cache *cache,
                                  const kvarn_page_table *pages, const void *q, int32_t q_dtype,
                                  int32_t num_q_tokens, int32_t num_q_heads, float sm_scale, float *out,
                                  void *workspace, size_t workspace_bytes, void *stream);

/* Append n_new tokens to every sequence of the batch: the keys and values
 * (MLA: latents) of new token i of sequence b go to position seq_lens[b] + i,
 * i.e. slot (pos % T) of fp16 page block_table[b][pos / T] of the fp16
 * pools -- always an fp16 page, since the region rule puts every position
 * at or after seq_lens[b] in the fp16 tail (gmlx "KV cache quantization",
 * "The two schemes": the newest tokens stay fp16).  seq_lens is read, not
 * changed: appended tokens count only once kvarn_commit accepts them, and a
 * later append overwrites tokens that were never accepted.
 * k_new, v_new: device [batch][n_new][H][D] of dtype (KVARN_F32, KVARN_F16
 * or KVARN_BF16; converted to fp16 by round to nearest even, values beyond
 * the fp16 range become infinities), 16-byte aligned; v_new is NULL for MLA.
 * MLA with a rope sidecar: k_new rows are [D + R], the latent (to k_fp16)
 * then the rope key (to rope_fp16, same page and slot).
 * The caller assigns the block-table entries of pages that receive tokens
 * (ids of fp16 pages).  A position past max_pages * T or a page id outside
 * the fp16 pool is skipped.  n_new = 0 is a no-op. */
kvarn_status kvarn_append(const kvarn_layout *layout, const kvarn_cache *cache,
                          const kvarn_page_table *pages, const void *k_new, const void *v_new,
                          int32_t dtype, int32_t n_new, void *stream);

/* Accept n_accept[b] of the appended tokens of every sequence b and keep the
 * quantized region up to date, all on the device:
 *   - seq_lens[b] += n_accept[b];
 *   - when that moves a page out of the fp16 tail (the region rule above:
 *     whole pages after the sink, leaving at least tail_tokens in fp16), the
 *     page -- every token of which is now committed, the commit rule of the
 *     evermx.com review, MLA and hybrid paragraph -- is quantized (as by
 *     kvarn_quantize, rope keys included) from its fp16 page into record page
 *     new_qpages[b], and block_table[b][page] is set to new_qpages[b].
 * promoted_fpages[b] reports, per sequence: the fp16 page id that was
 * quantized (>= 0; the caller may reuse that fp16 page), -1 nothing
 * promoted, -2 n_accept[b] outside [0, T] or seq_lens[b] + n_accept[b] past
 * max_pages * T, -3 the page's fp16 id or new_qpages[b] outside its pool;
 * on -2 and -3 the sequence's length and block table are left unchanged.
 * With n_accept[b] <= T at most one page per sequence is due.
 * block_table [batch][max_pages], seq_lens, n_accept, new_qpages,
 * promoted_fpages [batch]: device int32, caller-owned; new_qpages ids must
 * be distinct and unused (an entry not needed this step stays free). */
kvarn_status kvarn_commit(const kvarn_layout *layout, const kvarn_cache *cache, int32_t *block_table,
                          int32_t *seq_lens, int32_t batch, int32_t max_pages, const int32_t *n_accept,
                          const int32_t *new_qpages, int32_t *promoted_fpages, void *stream);

/* Size of the fixed device array kvarn_decode_attn_noalloc uses as its
 * workspace: 96 MiB, held on every GPU the library runs on until the
 * process ends. */
#define KVARN_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)

/* kvarn_decode_attn without a workspace argument and without allocating:
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * split-K partials go to a fixed device array of KVARN_NOALLOC_SCRATCH_BYTES
 * inside this library instead of a caller buffer; everything else --
 * arguments, layout, outputs, validation and statuses -- is that of
 * kvarn_decode_attn, on the current device (the stream must belong to it).
 * A shape whose workspace (kvarn_decode_workspace_bytes) exceeds the array
 * returns KVARN_EWORKSPACE and enqueues nothing.  The array's address on a
 * device is looked up on the first call there (KVARN_EHIP if that fails).
 * All calls on one GPU share the one array: calls that can overlap on a GPU
 * (other streams, other threads) race on it and must be ordered by the
 * caller.  Nothing in it needs clearing between calls. */
kvarn_status kvarn_decode_attn_noalloc(const kvarn_layout *layout, const kvarn_cache *cache,
                                       const kvarn_page_table *pages, const void *q, int32_t q_dtype,
                                       int32_t num_q_heads, float sm_scale, float *out, void *stream);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *kvarn_last_error(void);

/* Library version string. */
const char *kvarn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVARN_H */
