/*
 * bsa.h — block-sparse attention forward for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Every entry point takes plain
 * device pointers and sizes, validates its arguments on the host, enqueues
 * its kernels on the caller's stream and returns without synchronising.
 * The library keeps no state and allocates no memory: every buffer,
 * including scratch ("workspace"), belongs to the caller.  Errors are
 * reported through the returned status; nothing is launched when
 * validation fails.  No exception crosses this interface.
 *
 * Host validation covers shapes, strides, pointers and sizes, not the
 * contents of key patterns (that would need a device round trip).  With the
 * environment variable BSA_DEBUG_CHECKS set to anything but "" or "0", the
 * entry points that take a BLOCK or VS pattern (bsa_fwd, bsa_fwd_partials,
 * bsa_speculative_sparse, bsa_speculative_partials, bsa_bwd) first run the
 * bsa_check_pattern kernel on the caller's stream, wait for it, and return
 * BSA_ERR_INVALID_ARG for a pattern that breaks its rules.  That mode
 * synchronises the stream, cannot be captured in a graph, and keeps its
 * answer in one library-resident int32 pair per device (concurrent debug
 * checks on one device share it).  It is meant for development.
 *
 * Sources of the operations (cited by page title and section):
 *   [IR]   "Sparse FlashAttention with Incremental Repair" (README):
 *          What's in this fork; Usage sections 1 (sparse-only forward),
 *          2 (speculative + sparse decoding with exact combine) and
 *          3 (per-block partials).
 *   [BSFA] "Block Sparse Flash Attention": Abstract; Figure 2 (mechanism).
 *   [SGL]  "Implementation: Sgl project Sglang Sparse Flash Attention":
 *          Description; Signature; I/O Contract.
 *   [FSA]  "FSA: An Alternative Efficient Implementation of Native Sparse
 *          Attention Kernel": Abstract; with the Flash-Sparse-Attention
 *          README page (overview, main features, quick start).
 *
 * Conventions shared by the attention entry points
 * -------------------------------------------------
 * Layouts (element strides, head dim contiguous), as in [IR] Usage 1 and
 * the [SGL] I/O Contract:
 *   q     [B, Sq, Hq, D]       k, v  [B, Sk, Hkv, D]
 *   o     [B, Sq, Hq, D]       lse   [B, Hq, Sq] float32, contiguous
 *   varlen (cu_seqlens given): q [total_q, Hq, D], k/v [total_k, Hkv, D],
 *         o like q, lse [Hq, total_q]; the batch stride is then ignored.
 * Query head h reads key/value head h / (Hq / Hkv).
 * Scores are scale * <q, k> with scale = 1/sqrt(D) unless given
 * ([SGL] I/O Contract, softmax_scale); LSE is the natural-log
 * log-sum-exp of the attended scores.  A row with no attended key gives
 * O = 0 and LSE = -inf, the neutral partial of the combine ([IR] Usage 1).
 * Causal masking is bottom-right aligned: key c is visible to row r iff
 * c <= r + (Sk - Sq) (per sequence in varlen).
 * Inputs q/k/v are bfloat16; o may be bfloat16 or float32.
 * D must be 64 or 128.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The caller's HIP stream (hipStream_t); NULL is the null stream. */
typedef void* bsa_stream;

typedef enum {
  BSA_OK = 0,
  BSA_ERR_INVALID_ARG = 1, /* malformed shape, stride, pointer or size      */
  BSA_ERR_UNSUPPORTED = 2, /* well formed but outside what the kernels cover */
  BSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required    */
  BSA_ERR_HIP = 4          /* a HIP launch failed                           */
} bsa_status;

typedef enum { BSA_BF16 = 0, BSA_F32 = 1 } bsa_dtype;

/* A strided 4-D (or varlen 3-D) tensor view.  Strides are in elements; the
 * last (head-dim) axis is contiguous.  For varlen tensors stride_b is
 * ignored and the token axis is indexed by cu_seqlens[b] + s.  The token
 * stride of q, k, v (and dout) must be non-negative and at most 32 MB in
 * bytes (the kernels address up to 64 tokens from a block's first one with
 * 32-bit offsets); larger ones give BSA_ERR_UNSUPPORTED. */
typedef struct {
  void* ptr;
  int32_t dtype; /* bsa_dtype */
  int64_t stride_b, stride_s, stride_h;
} bsa_tensor;

/* Problem shape.  cu_seqlens_q/k are device int32 arrays of B+1 prefix sums
 * (NULL for fixed length); max_seqlen_q/k bound the per-sequence lengths
 * and must be given for varlen.  softmax_scale <= 0 selects 1/sqrt(D).
 * softcap ([SGL] Signature and I/O Contract; 0 = off): when c > 0 every
 * scaled score x = scale * <q, k> becomes c * tanh(x / c) before masking and
 * the softmax (the usual logit soft-capping; the page gives no formula).
 * Negative, NaN or infinite softcap: BSA_ERR_INVALID_ARG; bsa_fwd_gated
 * rejects softcap > 0 with BSA_ERR_UNSUPPORTED. */
typedef struct {
  int32_t B, Hq, Hkv, Sq, Sk, D;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int32_t max_seqlen_q, max_seqlen_k;
  float softmax_scale;
  int32_t causal;
  float softcap;
} bsa_problem;

typedef enum {
  BSA_PAT_DENSE = 0, /* every key (subject to the causal mask)                */
  BSA_PAT_BLOCK = 1, /* per-query-block lists of key-block ids                */
  BSA_PAT_VS = 2     /* per-query-block key windows plus gathered columns    */
} bsa_pattern_kind;

/* Which keys each query block attends to.
 *
 * BLOCK ([IR] Usage 1): entry j of the list for (b, h_t, query block m) is
 *   the key block [j*block_N, (j+1)*block_N).  Lists are sets (no repeats)
 *   of in-range ids; order does not matter.
 * VS ([SGL] I/O Contract): index holds block_offset — key positions w whose
 *   windows [w, w+block_N) are attended (clipped to the sequence) — and
 *   col_index holds column_index, single key positions; col_count is
 *   column_count.  Windows are disjoint; columns lie outside them.
 *
 * Storage: the list of (b, h_t, m) has count[b*s_b + h_t*s_h + m*s_q]
 * entries at index[(b*s_b + h_t*s_h + m*s_q) * cap + e] (and likewise
 * col_index with col_cap).  Strides of 0 broadcast: s_b = s_h = s_q = 0
 * is the single 1-D table of [IR] Usage 1 shared by every row and head.
 * Ht is the number of list heads: Hq (a list per query head) or Hkv (one
 * list per key/value head, shared by its Hq/Hkv query heads).
 * All arrays are device int32. */
typedef struct {
  int32_t kind; /* bsa_pattern_kind */
  int32_t Ht;
  int32_t block_M, block_N;
  int32_t cap, col_cap;
  const int32_t* count;
  const int32_t* index;
  const int32_t* col_count;
  const int32_t* col_index;
  int64_t s_b, s_h, s_q;
} bsa_pattern;

/* Human-readable name of a status code (static storage); any int32 value is
 * accepted ("unknown status" outside bsa_status). */
const char* bsa_status_string(int32_t status);

/* Checks the contents of a BLOCK or VS pattern on the device: the rules the
 * attention kernels rely on without checking them.  BLOCK ([IR] Usage 1):
 * 0 <= count <= cap; ids j >= 0 with j*block_N below the key length of the
 * list's sequence; no id twice in a list.  VS ([SGL] I/O Contract): window
 * starts in [0, key length), ascending, each at least block_N past the one
 * before (disjoint windows); 0 <= col_count <= col_cap; columns in
 * [0, key length), strictly ascending, none inside a window.
 * Lists checked: every (b, h_t, m) with b < B, h_t < Ht and
 * m < ceil(Sq / block_M) (varlen: the sequence's own query blocks; key
 * length Sk, or the sequence's own length from cu_seqlens_k).
 *   result  device int32[2], written on the stream: result[0] = number of
 *           violating lists, result[1] = the smallest flat list index
 *           (b*Ht + h_t) * nqb + m among them (INT32_MAX if none), where
 *           nqb = ceil(Sq / block_M) (varlen: ceil(max_seqlen_q / block_M)).
 * Asynchronous like the other entry points; the caller reads result after
 * the stream has passed the call.
 * Errors: BSA_ERR_INVALID_ARG for NULL arguments, a DENSE or NULL pattern,
 * or what bsa_fwd rejects in the problem sizes or pattern header;
 * BSA_ERR_HIP on launch failure. */
bsa_status bsa_check_pattern(const bsa_problem* prob, const bsa_pattern* pat, int32_t* result, bsa_stream stream);

/* Bytes of workspace bsa_fwd needs for this problem and pattern (0 when the
 * chosen kernel needs none).  Returns 0 on invalid arguments as well; the
 * subsequent bsa_fwd call reports them. */
size_t bsa_workspace_size(const bsa_problem* prob, const bsa_pattern* pat);

/* Attention restricted to a key pattern, returning (O, LSE).
 * [IR] Usage 1 (sparse-only forward; pattern NULL or DENSE gives ordinary
 * attention, as the speculative pass of [IR] Usage 2 needs).
 *   q, k, v  bf16 inputs (layouts above); k/v may be strided views.
 *   pat      NULL or a pattern; BLOCK needs Sk % block_N == 0 and
 *            block_N in {64, 128}; block_M in {64, 128} (ignored when the
 *            query rows fit one block).  VS: block_M <= block_N, each 64
 *            or 128, fixed length or varlen; with causal == 0 every listed
 *            key is attended ([SGL] Signature: causal defaults to False).
 *   o        output, bf16 or f32; lse float32 output (may be NULL).
 *   ws       device scratch of at least bsa_workspace_size() bytes (may be
 *            NULL when that is 0).  Overwritten; the caller keeps it alive
 *            until the stream has passed this call.
 * Kernels: decode shapes (fixed length, no VS pattern, and the query rows of
 * a kv head's group, G * Sq for dense or kv-head lists, Sq for query-head
 * lists, at most 16) run on the split-KV decode kernel with D 64 or 128;
 * every other shape runs on the tile kernels, which need D == 128
 * (BSA_ERR_UNSUPPORTED for D == 64 there).  VS patterns with 64-row query
 * blocks take two neighbouring query blocks per workgroup, loading the
 * windows both name once; the result is the same attention (up to the order
 * of float32 sums).
 * Errors: BSA_ERR_INVALID_ARG for NULL tensors, non-positive sizes,
 * Hq % Hkv != 0, pattern heads other than Hq/Hkv, Sk % block_N != 0;
 * BSA_ERR_UNSUPPORTED for D or block sizes outside the list above;
 * BSA_ERR_WORKSPACE for a short workspace; BSA_ERR_HIP on launch failure. */
bsa_status bsa_fwd(const bsa_problem* prob, bsa_tensor q, bsa_tensor k, bsa_tensor v,
                   const bsa_pattern* pat, bsa_tensor o, float* lse, void* ws, size_t ws_bytes,
                   bsa_stream stream);

/* (o, lse) partials over consecutive groups of pattern entries.  [IR] Usage 3
 * (per-block partials: entries_per_partial = 1 gives one partial per table
 * entry) and What's in this fork (partials merge exactly with the combine).
 * Entries are the list entries of a BLOCK pattern, or the 64-key blocks
 * [64e, 64e + 64) of a DENSE pattern (pat NULL).  Partial p covers entries
 * [p*E, (p+1)*E) of each list, E = entries_per_partial (E <= 0 lets the
 * library choose, as it does for its own split-KV decode); a partial with no
 * entries is (0, -inf).  The partials of two passes written into one buffer
 * merge with a single bsa_combine.
 *   o_part    float32 [P, B, Sq, Hq, D] contiguous.
 *   lse_part  float32 [P, B, Hq, Sq] contiguous.
 *   P = bsa_num_partials(prob, pat, entries_per_partial).
 * Fixed length only; VS patterns are not accepted.  Errors as for bsa_fwd. */
bsa_status bsa_fwd_partials(const bsa_problem* prob, bsa_tensor q, bsa_tensor k, bsa_tensor v,
                            const bsa_pattern* pat, int32_t entries_per_partial, float* o_part, float* lse_part,
                            bsa_stream stream);

/* Number of partials bsa_fwd_partials writes for these arguments (-1 if invalid). */
int32_t bsa_num_partials(const bsa_problem* prob, const bsa_pattern* pat, int32_t entries_per_partial);

/* Speculative + sparse decoding with exact combine.  [IR] Usage 2: attention
 * over a speculative key/value subset (k_spec, v_spec; Sk_spec keys, causal
 * when causal_spec != 0, bottom-right aligned), attention over the *missed*
 * blocks of the full cache (k, v) listed in `missed` — never masked — and
 * the log-sum-exp combine of the two, so the result equals attention over the
 * union when the sets are disjoint (the caller's precondition).
 *   prob      shapes of q and of the full cache (Sk); prob->causal is ignored.
 *   missed    a BLOCK pattern over (k, v) (Ht = Hq or Hkv).
 *   o, lse    outputs as for bsa_fwd.
 *   ws        at least bsa_speculative_workspace_size() bytes of device
 *             scratch (the float32 partials of both passes).
 * Equivalent to bsa_speculative_partials into ws followed by bsa_combine.
 * Fixed length only.  Errors as for bsa_fwd. */
bsa_status bsa_speculative_sparse(const bsa_problem* prob, bsa_tensor q, bsa_tensor k_spec, bsa_tensor v_spec,
                                  int32_t Sk_spec, int32_t causal_spec, bsa_tensor k, bsa_tensor v,
                                  const bsa_pattern* missed, bsa_tensor o, float* lse, void* ws, size_t ws_bytes,
                                  bsa_stream stream);

/* bsa_speculative_sparse for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, and harnesses that
 * forbid hipMalloc.  Identical result (the same kernels, the same split
 * plan), but the float32 partials of the two passes go to a scratch area
 * that the library keeps in device memory, BSA_NOALLOC_SCRATCH_BYTES per
 * device, held until the process ends, instead of a caller workspace.  The
 * call allocates and frees nothing.  The caller still owns every input and
 * output.  The scratch address is looked up once per device, on the first
 * call made with that device current.
 * Every call on one device shares that device's scratch area: calls that
 * overlap on one GPU (two streams, two threads) race and give undefined
 * results; calls ordered on one stream are safe.  Nothing needs clearing
 * between calls, since every partial a call reads was written by that call.
 * Errors: as bsa_speculative_sparse; BSA_ERR_WORKSPACE when the partials
 * (bsa_speculative_workspace_size bytes) exceed BSA_NOALLOC_SCRATCH_BYTES;
 * BSA_ERR_HIP when the scratch address cannot be obtained. */
#define BSA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
bsa_status bsa_speculative_sparse_noalloc(const bsa_problem* prob, bsa_tensor q, bsa_tensor k_spec,
                                          bsa_tensor v_spec, int32_t Sk_spec, int32_t causal_spec, bsa_tensor k,
                                          bsa_tensor v, const bsa_pattern* missed, bsa_tensor o, float* lse,
                                          bsa_stream stream);

/* The two passes of bsa_speculative_sparse without the combine: P float32
 * partials (o_part [P, B, Sq, Hq, D], lse_part [P, B, Hq, Sq], contiguous),
 * P = bsa_speculative_num_partials().  When the query rows of a kv head fit one
 * decode tile, both passes run in a single launch whose workgroups each take a
 * similar number of 64-key chunks.  [IR] Usage 2 and Usage 3. */
bsa_status bsa_speculative_partials(const bsa_problem* prob, bsa_tensor q, bsa_tensor k_spec, bsa_tensor v_spec,
                                    int32_t Sk_spec, int32_t causal_spec, bsa_tensor k, bsa_tensor v,
                                    const bsa_pattern* missed, float* o_part, float* lse_part, bsa_stream stream);

/* Partial count of bsa_speculative_partials (-1 on invalid arguments). */
int32_t bsa_speculative_num_partials(const bsa_problem* prob, int32_t Sk_spec, const bsa_pattern* missed);

/* Bytes of workspace bsa_speculative_sparse needs (0 on invalid arguments). */
size_t bsa_speculative_workspace_size(const bsa_problem* prob, int32_t Sk_spec, const bsa_pattern* missed);

/* Log-sum-exp combine of P partials.  [IR] What's in this fork (combine
 * identity FA(A u B) == Combine(FA(A), FA(B))) and Usage 2.
 * For each (b, h, s): m = max_p lse_p; if m = -inf the result is (0, -inf);
 * else w_p = exp(lse_p - m), O = sum w_p o_p / sum w_p, LSE = m + ln sum w_p.
 * A partial with lse -inf has weight 0 and its o_p is not used (it may hold
 * anything, NaN included).
 *   o_part    float32 [P, B, Sq, Hq, D] contiguous.
 *   lse_part  float32 [P, B, Hq, Sq] contiguous.
 *   o         output view [B, Sq, Hq, D] (bf16 or f32); lse float32
 *             [B, Hq, Sq] (may be NULL).  o may alias partial 0 only when
 *             it is float32 and contiguous.
 * Errors: BSA_ERR_INVALID_ARG for P < 1 or bad shapes; BSA_ERR_HIP. */
bsa_status bsa_combine(int32_t P, int32_t B, int32_t Hq, int32_t Sq, int32_t D, const float* o_part,
                       const float* lse_part, bsa_tensor o, float* lse, bsa_stream stream);

/* What a skipped tile leaves in the softmax of bsa_fwd_gated.  [BSFA]
 * Figure 2 names what a skipped block avoids (the V_j load and the P V_j
 * product) and nothing else, so the tile's scores, computed for its maximum,
 * may or may not feed the running maximum and normaliser:
 *   BSA_GATE_DROP_SKIPPED   left out altogether: the result is attention over
 *                           the kept tiles only (block-sparse attention on the
 *                           kept set);
 *   BSA_GATE_COUNT_SKIPPED  kept in the maximum and the normaliser, no value:
 *                           attention over every causal key with the value
 *                           rows of skipped tiles taken as zero (LSE is then
 *                           the dense causal LSE). */
typedef enum { BSA_GATE_DROP_SKIPPED = 0, BSA_GATE_COUNT_SKIPPED = 1 } bsa_gate_skipped;

/* BSFA gated causal attention.  [BSFA] Abstract and Figure 2: for query
 * block i and key block j < i the exact tile maximum
 * t(i,j) = max over the tile of scale*<q, k> is computed inside the tile loop
 * and the tile is kept iff t(i,j) >= T[b, h, i] (compared in float32);
 * the diagonal tile always runs; a skipped tile loads no V and does no P V
 * product; its scores enter the softmax or not as `skipped` says.
 *   T          float32 [B, Hq, nQB] thresholds (-inf keeps every tile).
 *   block_M/N  tile sizes; both 128.  Needs Sq == Sk, causal, fixed length,
 *              Sq % 128 == 0.
 *   skipped    bsa_gate_skipped (anything else: BSA_ERR_INVALID_ARG).
 *   keep_mask  optional uint8 [B, Hq, nQB, nKB]: 1 kept, 0 skipped, for
 *              j <= i (entries j > i are not written).
 *   tile_max   optional float32 [B, Hq, nQB, nKB]: t(i, j) for j <= i
 *              (the diagonal tile's maximum over its causal entries).
 * Errors as for bsa_fwd; BSA_ERR_UNSUPPORTED outside the cases above. */
bsa_status bsa_fwd_gated(const bsa_problem* prob, bsa_tensor q, bsa_tensor k, bsa_tensor v, const float* T,
                         int32_t block_M, int32_t block_N, int32_t skipped, bsa_tensor o, float* lse,
                         uint8_t* keep_mask, float* tile_max, bsa_stream stream);

/* Backward of block-sparse attention: dQ, dK, dV.  The pages name a
 * backward pass ([IR] keeps FA's backward; [FSA] and FlagAttention list
 * forward + backward for their sparse kernels) without a formula; this is
 * the plain derivative of bsa_fwd's result over the same key sets: with
 * P = exp(scale Q K^T - LSE) on the key set, D = rowsum(dO * O),
 * dS = P * (dO V^T - D): dV = P^T dO, dQ = scale dS K, dK = scale dS^T Q
 * (summed over the query heads of a kv head).
 *   pat        NULL / dense or BSA_PAT_BLOCK (as bsa_fwd; block_M and block_N
 *              64 or 128); fixed length or variable length (cu_seqlens),
 *              D == 128; with softcap > 0 the gradient goes through the capped
 *              scores (dS times 1 - tanh^2 of the cap's argument).
 *   o, lse     bsa_fwd's output (bf16 or float32) and LSE for the same call
 *              (lse [B, Hq, Sq], or [Hq, total_q] for variable length).
 *   dout       bf16, the layout of q.
 *   dq         device float32 [B, Sq, Hq, D] contiguous; dk, dv float32
 *              [B, Sk, Hkv, D] contiguous (variable length: [total_q, Hq, D]
 *              and [total_k, Hkv, D]); every entry is written.
 *   workspace  bsa_bwd_workspace_size bytes, 256-byte aligned: row dots,
 *              each row's LSE in log2 units (+inf for a row with no keys),
 *              a bitmap of which query blocks name each key block, the
 *              per-64-key-block lists of (query head, query block) pairs,
 *              and room for float32 dK/dV partials of lists split over
 *              several workgroups (64 KB per 128 query slabs of 32 rows, an
 *              upper bound; about 1.4 GB at 32K tokens, 32 heads, 34-entry
 *              lists).
 * A 64-key block's dK and dV come from the workgroups that take its list in
 * chunks of 128 slabs (partials summed in chunk order), dQ from one
 * workgroup per query block: no atomics on the gradients, and the lists are
 * built in a fixed order (by head, then query block), so the gradients are
 * the same bits on every run.
 * Block patterns take at most 2^20 query blocks and 2^11 query heads (a list
 * entry packs both in 32 bits); the workspace size is 0 and the call gives
 * BSA_ERR_UNSUPPORTED beyond them.
 * Errors: as bsa_fwd; BSA_ERR_UNSUPPORTED outside the cases above. */
size_t bsa_bwd_workspace_size(const bsa_problem* prob, const bsa_pattern* pat);
bsa_status bsa_bwd(const bsa_problem* prob, bsa_tensor q, bsa_tensor k, bsa_tensor v, const bsa_pattern* pat,
                   bsa_tensor o, const float* lse, bsa_tensor dout, float* dq, float* dk, float* dv,
                   void* workspace, size_t workspace_bytes, bsa_stream stream);

/* Selected attention: every query token attends to the key blocks it selected.
 * [FSA] Abstract and the Flash-Sparse-Attention README page (main features:
 * a batched query-to-KV kernel, a reduction and an online-softmax pass, no
 * atomics; configuration block_size, topk, varlen cu_seqlens).  Native sparse
 * attention's selection branch: token t of kv head g selected up to topk
 * blocks of block_size keys of its own sequence, shared by the group's query
 * heads; the result is softmax attention over the union of those blocks
 * (clipped to the sequence and, when prob->causal, to keys <= t + Sk - Sq).
 * Computed key-block-outer: the selections are inverted into per-block token
 * lists, each block's K/V tile is loaded once per 128 / G gathered tokens,
 * every (token, slot, head) gets an (o, lse) partial in the workspace, and
 * the combine merges a token's topk partials.
 *   sel        device int32, [B, Sq, Hkv, topk] (fixed length) or
 *              [total_q, Hkv, topk] (varlen); a block index or -1 (unused).
 *              A token's blocks must be distinct (a repeated block is
 *              counted twice).  Blocks past the sequence or with no causally
 *              visible key contribute nothing.
 *   total_q    varlen: rows of q, equal to cu_seqlens_q[B]; ignored for
 *              fixed length.
 *   topk       >= 1.   block_size  64.
 *   o, lse     as bsa_fwd (lse [B, Hq, Sq] or [Hq, total_q]).
 *   workspace  bsa_selected_workspace_size bytes, 256-byte aligned: list
 *              counts and offsets, the inverted lists, and topk float32
 *              partials of every (token, head).
 * Needs D == 128, Hq / Hkv dividing 128 (at most 16), and sequences of at
 * most 8192 key blocks (524288 keys).
 * Errors: as bsa_fwd; BSA_ERR_WORKSPACE for a missing or small workspace. */
size_t bsa_selected_workspace_size(const bsa_problem* prob, int32_t total_q, int32_t topk, int32_t block_size);
bsa_status bsa_fwd_selected(const bsa_problem* prob, bsa_tensor q, bsa_tensor k, bsa_tensor v, const int32_t* sel,
                            int32_t total_q, int32_t topk, int32_t block_size, bsa_tensor o, float* lse,
                            void* workspace, size_t workspace_bytes, bsa_stream stream);

/* BSFA threshold calibration (synthetic, one pass over calibration inputs).
 * [BSFA] Abstract (a one-time calibration learns per-layer, per-head score
 * distributions so that the top-k blocks of each query are kept) and
 * Figure 2 (thresholds T^(k), one per query row, -inf where fewer than k
 * off-diagonal candidates exist).  The page gives no procedure; this one:
 * for each sample b, head h and 128-row query block i, the tile maxima
 * t(i, j) (as bsa_fwd_gated computes them) are written to tile_max and the
 * k_keep-th largest of the off-diagonal ones (j < i) is taken; rows with
 * i < k_keep get -inf; T[h, i] is the mean over the B samples (float32,
 * summed in sample order).  Gating a sample with its own thresholds keeps
 * k_keep off-diagonal tiles per row (ties aside).
 *   q, k       as bsa_fwd_gated (v is not needed): causal self-attention,
 *              fixed length, Sq == Sk, Sq % 128 == 0, D == 128, no softcap.
 *   k_keep     >= 1.
 *   tile_max   device float32 [B, Hq, nQB, nQB], caller-owned; entries
 *              j <= i are written (the diagonal over its causal entries).
 *   T          device float32 [Hq, nQB] output; expand it over the batch
 *              for bsa_fwd_gated's [B, Hq, nQB].
 * Errors: BSA_ERR_INVALID_ARG (NULL, k_keep < 1, shapes, alignment);
 * BSA_ERR_UNSUPPORTED (outside the cases above, nQB > 4096); BSA_ERR_HIP. */
bsa_status bsfa_calibrate(const bsa_problem* prob, bsa_tensor q, bsa_tensor k, int32_t k_keep, float* tile_max,
                          float* T, bsa_stream stream);

/* Vertical-slash index conversion.  [SGL] Description and I/O Contract
 * (convert_vertical_slash_indexes); the conversion rule is this library's
 * own, since the page defers it to a paper that is not among the sources:
 * for query block m of sequence b (rows r0 = m*block_M .. r1-1, d =
 * kv_len - q_len), slash offsets s (key = row + d - s) are walked in the
 * given descending order; each covers keys [max(0, r0+d-s), r1-1+d-s];
 * a frontier f starts at -inf; a range [a, e] opens a window at a when
 * a >= f (f = a + block_N), at f when a < f <= e (f += block_N), and
 * nothing otherwise.  Windows go to block_offset (key positions).  Then
 * the vertical indices v <= r1-1+d, in the given ascending order, that
 * no window contains go to column_index.
 *   q_seqlens, kv_seqlens  device int32 [B].
 *   vertical   device int32 [B, H, nnz_v], ascending, unique.
 *   slash      device int32 [B, H, nnz_s], descending, unique, >= 0.
 *   context_size  rows = cdiv(context_size, block_M) per (b, h); rows past
 *              a sequence's end get counts 0.
 *   outputs    block_count [B,H,rows], block_offset [B,H,rows,nnz_s],
 *              column_count [B,H,rows], column_index [B,H,rows,nnz_v],
 *              device int32; entries past a count are not written.
 * Needs causal != 0 and block_M <= block_N ([SGL] Signature default).
 * Errors: BSA_ERR_INVALID_ARG (NULL, sizes); BSA_ERR_UNSUPPORTED
 * (causal == 0, block_M > block_N); BSA_ERR_HIP. */
bsa_status vs_convert_indexes(const int32_t* q_seqlens, const int32_t* kv_seqlens, const int32_t* vertical,
                              const int32_t* slash, int32_t B, int32_t H, int32_t nnz_v, int32_t nnz_s,
                              int32_t context_size, int32_t block_M, int32_t block_N, int32_t causal,
                              int32_t* block_count, int32_t* block_offset, int32_t* column_count,
                              int32_t* column_index, bsa_stream stream);

/* Vertical-slash conversion with per-head counts of valid indices.
 * [SGL] Description (the merged-head variant takes per-head variable
 * sparsity counts) and Signature.  As vs_convert_indexes, except that head h
 * uses only the first vertical_count[h] entries of each vertical row and the
 * first slash_count[h] entries of each slash row (counts are clamped to
 * [0, nnz_v] and [0, nnz_s]; entries past a count are never read).
 *   vertical_count, slash_count  device int32 [H], shared by every batch entry.
 * Errors as for vs_convert_indexes; BSA_ERR_INVALID_ARG for NULL counts. */
bsa_status vs_convert_indexes_mergehead(const int32_t* q_seqlens, const int32_t* kv_seqlens,
                                        const int32_t* vertical, const int32_t* slash,
                                        const int32_t* vertical_count, const int32_t* slash_count, int32_t B,
                                        int32_t H, int32_t nnz_v, int32_t nnz_s, int32_t context_size,
                                        int32_t block_M, int32_t block_N, int32_t causal, int32_t* block_count,
                                        int32_t* block_offset, int32_t* column_count, int32_t* column_index,
                                        bsa_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
