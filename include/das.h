/*
 * das.h -- split-KV decode attention for AMD Instinct MI355X (gfx950).
 *
 * Single-query (decode-step) softmax attention over a long KV cache, cut
 * along the sequence into splits that run as separate workgroups, followed by
 * a log-sum-exp merge of the per-split partial results.
 *
 * Sources, cited by page title and section:
 *   [FD++]    "FlashDecoding++: 시퀀스 차원 KV 분할 병렬화와 GPU 언더유틸라이제이션 극복을
 *             통한 LLM 서빙 극대화" (TechKnowGenie).  §1: a decode step is one query
 *             token against the N cached K/V rows, a memory-bound vector-matrix
 *             product.  §2: the sequence axis becomes a third grid axis, cut
 *             into chunks.  §3: phase 1 writes, per chunk, the unnormalised
 *             partial output, the chunk max and the chunk exponential sum;
 *             phase 2 rescales every chunk by exp(chunk max - global max),
 *             sums, and divides.  §6 ("chunk size tuning guide"): too small a
 *             chunk inflates phase-2 traffic, too large a chunk leaves
 *             compute units idle; aim for several times more blocks than
 *             compute units.
 *             §4 ("quantisation-friendly kernel fusion"): an FP8 (or INT4) K/V
 *             cache is dequantised on chip, right after it is loaded, back to
 *             16-bit floats for the products, so fewer bytes cross HBM.
 *             §6 (vLLM / TensorRT-LLM integration): serving engines keep K/V
 *             in blocks allocated anywhere in a pool, listed per sequence by a
 *             block table, and map each block onto a slice of a split's chunk.
 *   [SGL-PAR] "병렬 처리 개요 (Parallelism Overview)", SGLang Diffusion docs.
 *             "What happens to the shapes" and "Constraints": partial
 *             attention results over disjoint row sets (ring hops, tail or
 *             replicated parts) are joined by an online-softmax merge that
 *             needs each part's softmax log-sum-exp, so an attention kernel
 *             must export its LSE.
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers to row-major, contiguous arrays,
 *     16-byte aligned.  bf16 means bfloat16 bit patterns (uint16_t storage).
 *   - The caller owns all memory.  The library never allocates, frees,
 *     synchronises the device or copies device memory to the host, so every
 *     call can be recorded into a HIP graph.  It caches only the compute-unit
 *     count of each device it has seen (and, for das_decode_attention_noalloc,
 *     the address of its static workspace on each device).
 *   - Arguments are checked on the host before anything is launched.  On a
 *     failed check the call returns a negative status, launches nothing and
 *     leaves every output untouched.  A launch error returns DAS_ELAUNCH.
 *     No C++ exception crosses this interface.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is
 *     stream-ordered; the call returns without waiting for the GPU.
 *   - Calls are re-entrant.  Concurrent calls must not share a workspace.
 *   - Supported shapes: head dim D in {64, 128}; GQA group G = Hq / Hkv in
 *     {1, 2, 4, 8, 16} (Hq a multiple of Hkv) with every cache format;
 *     1 <= B <= 65535; 1 <= Hkv <= 65535;
 *     1 <= Smax with (Smax + 256) * D * 2 < 2^31 (one sequence's K rows are
 *     addressed with 32-bit byte offsets); num_splits <= DAS_MAX_SPLITS.
 *   - Query head h reads kv-head h / G.
 *   - Device-side precondition (not checked on the host, since reading
 *     seq_lens would need a device-to-host copy): 0 <= seq_lens[b] <= Smax.
 *     Values outside are clamped to [0, Smax].  A sequence of length 0 yields
 *     out = 0 and lse = -inf (the identity of the merge).
 *   - LSE is the natural logarithm of sum_j exp(scale * q.k_j).
 */
#ifndef DAS_H
#define DAS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DAS_OK = 0,
  DAS_EINVAL = -1,     /* bad argument: null pointer, bad shape, bad dtype */
  DAS_ENOTSUP = -2,    /* valid but unsupported: D, G outside the supported set */
  DAS_EWORKSPACE = -3, /* workspace missing or smaller than das_decode_workspace_bytes */
  DAS_ELAUNCH = -4,    /* the HIP runtime refused a launch or a device query */
} das_status;

/* Element types.  Outputs are DAS_F32 or DAS_BF16; a K/V cache is DAS_BF16,
 * DAS_E4M3 (OCP 8-bit floating point, see das_decode_attention_fp8) or
 * DAS_INT4 (4-bit integers with row scales, see das_decode_attention_int4). */
typedef enum { DAS_F32 = 0, DAS_BF16 = 1, DAS_E4M3 = 2, DAS_INT4 = 3 } das_dtype;

/* Page-pool layouts of a paged K/V cache (see das_decode_attention_paged). */
typedef enum {
  DAS_PAGED_HND = 0, /* pool [num_pages][Hkv][page_size][D]: a page's rows of one kv-head contiguous */
  DAS_PAGED_NHD = 1  /* pool [num_pages][page_size][Hkv][D]: a page's rows, all kv-heads per row */
} das_paged_layout;

#define DAS_MAX_SPLITS 4096
/* A workspace begins with this many bytes of arrival counters (see
 * das_decode_attention): zero them before the workspace is first used. */
#define DAS_WORKSPACE_COUNTER_BYTES (65536 * 4)
/* Chunks are whole multiples of this many rows (the per-workgroup quantum). */
#define DAS_CHUNK_QUANTUM 128

/*
 * Split plan ([FD++] §2 grid, §6 tuning guide).  Pure host function.
 *   num_splits == 0: automatic.  The plan picks the number of splits NS so
 *     that the B*Hkv*NS workgroups about fill the chip -- three for every four
 *     compute units, which already saturate HBM (das_plan_kv: every compute
 *     unit for an INT4 cache) -- and the longest sequence into at least five
 *     splits where the chunk bounds allow, with chunk = ceil(Smax/NS) rounded up to
 *     DAS_CHUNK_QUANTUM and kept between a lower bound (partial-result
 *     traffic stays a few percent of the K/V bytes: 256 rows, 512 for G = 8,
 *     1024 for G = 16) and an upper bound (8192 rows).
 *   num_splits == n >= 1: chunk = ceil(Smax/n) rounded up to the quantum;
 *     NS = ceil(Smax/chunk) <= n.
 *   Sequence b uses ceil(seq_lens[b]/chunk) of the NS splits; the rest exit
 *     at once.
 *   num_cus: compute units to plan for; 0 = query the current device (this
 *     is the only device query, cached per device).
 * Outputs *ns_out and *chunk_out.  Returns DAS_OK or a negative status.
 */
int das_plan(int32_t B, int32_t Hkv, int32_t G, int32_t Smax, int32_t D, int32_t num_splits,
             int32_t num_cus, int32_t* ns_out, int32_t* chunk_out);

/*
 * The automatic plan of the one-call entry point for a K/V cache of
 * kv_dtype (DAS_BF16, DAS_E4M3 or DAS_INT4; anything else: DAS_EINVAL).
 * bf16 and E4M3 caches use das_plan's.  An INT4 cache aims for one workgroup
 * on every compute unit instead of three per four: with a quarter of the
 * bytes per row its call is bound by the work per row, not by HBM ([FD++] §2:
 * fill the chip along the sequence axis).  A forced num_splits gives the same
 * plan for every format.  The phase-1-only entry points
 * (das_split_kv_decode*) always use das_plan's plan, which das_lse_combine
 * assumes.  Arguments and outputs as for das_plan.
 */
int das_plan_kv(int32_t kv_dtype, int32_t B, int32_t Hkv, int32_t G, int32_t Smax, int32_t D,
                int32_t num_splits, int32_t num_cus, int32_t* ns_out, int32_t* chunk_out);

/*
 * Workspace bytes das_decode_attention needs for this shape and split
 * request (0 when the plan has a single split).  Layout: first
 * DAS_WORKSPACE_COUNTER_BYTES of arrival counters (one per (b, kv-head)),
 * then the phase-1 partial results of [FD++] §3: per (b, query head, split)
 * an unnormalised output row of D floats, then its max and exponential sum.
 * The size covers the plan of every entry point and cache format for this
 * shape (das_plan and das_plan_kv), so one workspace serves them all.
 * num_cus as in das_plan.  Returns (size_t)-1 on invalid arguments.
 */
size_t das_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t Smax, int32_t D,
                                  int32_t num_splits, int32_t num_cus);

/*
 * Decode attention ([FD++] §1-§3; LSE export per [SGL-PAR] "Constraints").
 *   q        bf16 [B][Hq][D]
 *   k_cache  bf16 [B][Hkv][Smax][D]    rows >= seq_lens[b] are never read
 *   v_cache  bf16 [B][Hkv][Smax][D]
 *   seq_lens int32 [B]                 valid rows per sequence (device memory)
 *   scale    multiplies each dot product q.k (typically 1/sqrt(D))
 *   out      [B][Hq][D], out_dtype DAS_F32 (float) or DAS_BF16 (rounded to
 *            nearest even)
 *   lse_out  float [B][Hq] natural-log LSE, or NULL to skip
 *   num_splits 0 = automatic plan, n >= 1 forces at most n splits (see das_plan)
 *   workspace, workspace_bytes: device scratch of at least
 *            das_decode_workspace_bytes(...) bytes (may be NULL when that is 0)
 *   stream   hipStream_t or NULL
 * One kernel launch: one workgroup per (split, kv-head, batch row) holding
 * the whole GQA group of that kv-head computes its split's partial result
 * (phase 1); the last workgroup of each (b, kv-head) to finish, found with a
 * device-scope arrival counter in the workspace, merges every split of that
 * kv-head (phase 2).  A sequence that uses one split, and every sequence of
 * a single-split plan, is written directly by its workgroup.  When the plan
 * has more than 4 split workgroups per compute unit (B*Hkv*NS > 4*CUs), or
 * more than 65536 (b, kv-head) pairs, phase 2 runs as a second kernel
 * instead (as das_lse_combine).
 * Workspace precondition: its first DAS_WORKSPACE_COUNTER_BYTES must be zero
 * before the workspace is first used (allocate it zero-filled); every
 * completed call leaves them zero again, whatever the shape.  A counter the
 * merge finds at or above the number of splits (a workspace that was never
 * zeroed) turns that (b, kv-head)'s outputs and LSE into NaN; a smaller
 * nonzero count (left by a call that never finished) cannot be told from a
 * valid one and gives wrong outputs.  das_decode_attention_noalloc manages
 * its own workspace.
 */
int das_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                         int32_t Smax, int32_t D, float scale, void* out, int32_t out_dtype,
                         float* lse_out, int32_t num_splits, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Phase 1 alone ([FD++] §3, phase 1): the same arguments and checks as
 * das_decode_attention.  When the plan has more than one split it writes
 * only the partial results into `workspace` and leaves out/lse_out
 * untouched; das_lse_combine with the same shape, num_splits and workspace
 * then finishes the call.  With a single split it writes out/lse_out
 * directly.  It never touches the workspace's arrival counters.
 * das_split_kv_decode + das_lse_combine computes what das_decode_attention
 * computes, with phase 2 as a separate kernel (sums may round differently).
 * Every split slot of the plan is written: the partial of a split that
 * holds rows, or an empty mark (max -inf, sum 0) for one past its sequence.
 */
int das_split_kv_decode(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                        int32_t Smax, int32_t D, float scale, void* out, int32_t out_dtype,
                        float* lse_out, int32_t num_splits, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * Decode attention over an 8-bit floating-point K/V cache ([FD++] §4).  The
 * pages leave the FP8 encoding and its scaling open; this library reads them
 * as OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * subnormals; S.1111.111 is NaN; no infinities) with one fp32 scale per
 * kv-head for K and one for V:
 *   K[b][g][j][d] = k_scale[g] * e4m3(k_cache[b][g][j][d]), V likewise.
 *   k_cache, v_cache  uint8 E4M3 codes [B][Hkv][Smax][D]
 *   k_scale, v_scale  device float [Hkv] (may point to one value repeated)
 * Everything else (q, seq_lens, out, lse_out, num_splits, workspace and its
 * precondition, stream, supported shapes, errors) is as for
 * das_decode_attention; the plan and das_decode_workspace_bytes are shared.
 * The codes are turned into bf16 (exactly) on chip for q.K^T and into fp32
 * for p.V; the K scale multiplies the finished dot product and the V scale
 * the finished p.V sums.  A sequence's rows are addressed with 32-bit byte
 * offsets: (Smax + 256) * D < 2^31.  NULL k_scale or v_scale: DAS_EINVAL.
 */
int das_decode_attention_fp8(const void* q, const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale, const int32_t* seq_lens,
                             int32_t B, int32_t Hq, int32_t Hkv, int32_t Smax, int32_t D,
                             float scale, void* out, int32_t out_dtype, float* lse_out,
                             int32_t num_splits, void* workspace, size_t workspace_bytes,
                             void* stream);

/* Phase 1 alone over an E4M3 K/V cache: das_split_kv_decode with the cache
 * of das_decode_attention_fp8.  Finish with das_lse_combine. */
int das_split_kv_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                            const float* k_scale, const float* v_scale, const int32_t* seq_lens,
                            int32_t B, int32_t Hq, int32_t Hkv, int32_t Smax, int32_t D,
                            float scale, void* out, int32_t out_dtype, float* lse_out,
                            int32_t num_splits, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * Decode attention over a 4-bit integer K/V cache ([FD++] §4 names INT4
 * beside FP8: a quarter of the bf16 bytes, dequantised on chip).  The pages
 * leave the code and its scaling open; this library reads them as
 * two's-complement 4-bit integers (-8 ... 7), two per byte, element 2i in
 * the low nibble and element 2i+1 in the high nibble, with one fp32 scale per
 * cached row (batch row, kv-head, token) for K and one for V:
 *   K[b][g][j][d] = k_scale[b][g][j] * int4(element d of k_cache[b][g][j]),
 *   V likewise.
 *   k_cache, v_cache  uint8 [B][Hkv][Smax][D/2]
 *   k_scale, v_scale  device float [B][Hkv][Smax], 4-byte aligned (only the
 *                     rows j < seq_lens[b] are read)
 * Everything else (q, seq_lens, out, lse_out, num_splits, workspace and its
 * precondition, stream, supported shapes, errors) is as for
 * das_decode_attention, except that the automatic plan is das_plan_kv's for
 * DAS_INT4 (one workgroup per compute unit); das_decode_workspace_bytes covers it.
 * The codes become exact bf16 integers on chip; a row's K scale multiplies its
 * finished dot product and its V scale its softmax weight.  A sequence's rows
 * are addressed with 32-bit byte offsets: (Smax + 256) * D / 2 < 2^31.  NULL
 * or misaligned k_scale or v_scale: DAS_EINVAL.  A paged INT4 cache: see
 * das_decode_attention_paged.
 */
int das_decode_attention_int4(const void* q, const void* k_cache, const void* v_cache,
                              const float* k_scale, const float* v_scale, const int32_t* seq_lens,
                              int32_t B, int32_t Hq, int32_t Hkv, int32_t Smax, int32_t D,
                              float scale, void* out, int32_t out_dtype, float* lse_out,
                              int32_t num_splits, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Phase 1 alone over an INT4 K/V cache: das_split_kv_decode with the cache
 * of das_decode_attention_int4.  Finish with das_lse_combine. */
int das_split_kv_decode_int4(const void* q, const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale, const int32_t* seq_lens,
                             int32_t B, int32_t Hq, int32_t Hkv, int32_t Smax, int32_t D,
                             float scale, void* out, int32_t out_dtype, float* lse_out,
                             int32_t num_splits, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * Decode attention over a paged K/V cache ([FD++] §6).  K and V live in two
 * page pools of num_pages pages of page_size rows; row j of sequence b is
 * row j % page_size of page block_table[b][j / page_size]:
 *   k_pool, v_pool  [num_pages][Hkv][page_size][D] (DAS_PAGED_HND) or
 *                   [num_pages][page_size][Hkv][D] (DAS_PAGED_NHD), elements
 *                   of kv_dtype: DAS_BF16; DAS_E4M3 with k_scale/v_scale
 *                   as in das_decode_attention_fp8; or DAS_INT4, codes as in
 *                   das_decode_attention_int4 (a row is D/2 bytes), with
 *                   k_scale/v_scale pools of fp32 row scales laid out like the
 *                   code pools: [num_pages][Hkv][page_size] (HND) or
 *                   [num_pages][page_size][Hkv] (NHD), 4-byte aligned
 *                   (k_scale/v_scale are ignored for DAS_BF16)
 *   block_table     device int32 [B][max_blocks]; entries of pages a sequence
 *                   does not reach may be read (never outside row b of the
 *                   table) but are never used; an entry outside
 *                   [0, num_pages) is clamped into it on the device (wrong
 *                   rows, never an access outside the pool)
 *   page_size       a power of two, 32 ... 65536 rows (DAS_ENOTSUP otherwise)
 *   seq_lens[b]     device int32, clamped to [0, max_blocks * page_size]
 * Splits cover whole pages: the plan is das_plan_kv's for kv_dtype and Smax =
 * max_blocks * page_size with the chunk rounded up to a multiple of page_size, so a
 * workspace of das_decode_workspace_bytes(B, Hq, Hkv, max_blocks *
 * page_size, D, num_splits, 0) bytes always suffices.  q, out, lse_out,
 * num_splits, the workspace precondition, stream, errors: as for
 * das_decode_attention.  One page is addressed with 32-bit offsets:
 * page_size * Hkv * (bytes of a row of D elements) < 2^31.
 */
int das_decode_attention_paged(const void* q, const void* k_pool, const void* v_pool,
                               int32_t kv_dtype, const float* k_scale, const float* v_scale,
                               const int32_t* block_table, int32_t max_blocks, int32_t page_size,
                               int32_t num_pages, int32_t layout, const int32_t* seq_lens,
                               int32_t B, int32_t Hq, int32_t Hkv, int32_t D, float scale,
                               void* out, int32_t out_dtype, float* lse_out, int32_t num_splits,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Phase 2 alone ([FD++] §3, phase 2): merges the partial results that
 * das_split_kv_decode left in `workspace` (same B, Hq, Hkv, Smax, D,
 * num_splits) into out / lse_out.  Per (b, h): M = max of the split maxima,
 * w_c = exp(m_c - M), out = sum w_c o_c / sum w_c l_c, lse = M + ln(sum w_c
 * l_c).  Phase 1 marks the splits a sequence does not reach as empty (max
 * -inf, sum 0), so seq_lens is checked (non-null, aligned) but not read.  A
 * no-op returning DAS_OK when the plan has a single split.
 */
int das_lse_combine(const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t Smax,
                    int32_t D, int32_t num_splits, const void* workspace,
                    size_t workspace_bytes, void* out, int32_t out_dtype, float* lse_out,
                    void* stream);

/*
 * Merge of two attention states over disjoint row sets ([SGL-PAR] "What
 * happens to the shapes": ring hops merged by online softmax; "Constraints":
 * tail-pad / replicated parts joined by the same merge).  Per row r:
 *   mx = max(lse_a, lse_b); both -inf -> (0, -inf);
 *   lse = mx + ln(exp(lse_a - mx) + exp(lse_b - mx));
 *   o = exp(lse_a - lse) o_a + exp(lse_b - lse) o_b.
 *   o_a, o_b, o_out  [rows][D] in o_dtype (DAS_F32 or DAS_BF16)
 *   lse_a, lse_b, lse_out float [rows]
 * o_out / lse_out may alias the corresponding a or b arrays.  D in {64, 128};
 * rows >= 0 (0 is a no-op).  The formula is symmetric: swapping a and b gives
 * bitwise the same result.
 */
int das_merge_attn_states(const void* o_a, const float* lse_a, const void* o_b,
                          const float* lse_b, void* o_out, float* lse_out, int64_t rows,
                          int32_t D, int32_t o_dtype, void* stream);

/*
 * das_decode_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without workspace and workspace_bytes, the
 * same plan, kernels and results.  Its workspace is a static device array
 * of DAS_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs
 * on until the process ends; the call itself allocates and frees nothing.
 * The first call on a device looks the array up and zeroes its arrival
 * counters (a small fill kernel on `stream`, ahead of the call's kernels).
 *   Returns DAS_EWORKSPACE, launching nothing, when the shape and split
 *   request need more than DAS_NOALLOC_SCRATCH_BYTES of workspace
 *   (das_decode_workspace_bytes tells); otherwise as das_decode_attention.
 *   Every call on one GPU shares that GPU's array, and it keeps the last
 *   call's contents: calls that overlap on one GPU (concurrent streams, or
 *   host threads) race and give wrong results; serialise them.
 */
#define DAS_NOALLOC_SCRATCH_BYTES 67108864 /* 64 MiB */
int das_decode_attention_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                                 int32_t Smax, int32_t D, float scale, void* out,
                                 int32_t out_dtype, float* lse_out, int32_t num_splits,
                                 void* stream);

/* Static, human-readable text for a status code. */
const char* das_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* DAS_H */
