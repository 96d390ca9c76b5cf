/*
 * sws.h - C ABI of the Sketch&Walk sparse-attention hot path for AMD MI355X
 * (gfx950).
 *
 * The method is the one described on the deep-reading page "Scout Before You
 * Attend: Sketch-and-Walk Sparse Attention for Efficient LLM Inference"
 * (arXiv 2602.07397): Small-World Sketching of Q and K (block means, then a
 * subsampled randomized Hadamard projection d -> k), a walk state carried
 * from layer to layer, top-tau key blocks per query block, and block-sparse
 * attention on the original Q/K/V for prefill and for single-token decode.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer argument is a DEVICE pointer owned by the caller.  The
 *   library never allocates, frees or keeps a pointer after it returns.
 * - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *   enqueues work on it and never synchronises.
 * - Arguments are validated on the host before any launch; on error nothing
 *   is launched and the outputs are untouched.  Device-side offsets and
 *   positions (cu_seqlens, cu_blocks, pos, cur_block) are trusted: they must
 *   be consistent with the host sizes passed alongside them.  Index lists,
 *   their counts, context lengths and page tables are clamped by the kernels
 *   to the ranges the sizes allow, so a malformed one gives a wrong result,
 *   never an access outside the caller's buffers.
 * - Return value: SWS_OK (0) or an sws_status error code.  sws_status_string
 *   names a code; sws_last_error_detail gives a per-thread message for the
 *   most recent failed call.
 * - Activations are token-major and contiguous: X[t][h][e] for token t, head
 *   h, feature e.  A ragged batch packs its sequences one after the other;
 *   cu_seqlens[s] is the first token of sequence s (cu_seqlens[n_seqs] = T)
 *   and cu_blocks[s] its first block (b_s = ceil(n_s / B) blocks; blocks never
 *   straddle sequences).
 * - An empty batch (n_seqs = 0, and then total_blocks = 0) is valid: the
 *   call returns SWS_OK and launches nothing.
 * - GQA: query head h reads KV head h / (hq / hkv).
 * - The library holds no state and no random generator: the Hadamard sign
 *   vector and column subset are inputs.
 */
#ifndef SWS_H
#define SWS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sws_status {
  SWS_OK = 0,
  SWS_ERR_NULL = 1,         /* a required pointer is NULL                        */
  SWS_ERR_SHAPE = 2,        /* inconsistent or out-of-range sizes                */
  SWS_ERR_UNSUPPORTED = 3,  /* a size or dtype the library has no kernel for     */
  SWS_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than required           */
  SWS_ERR_LAUNCH = 5        /* the HIP runtime rejected a kernel launch          */
} sws_status;

typedef enum sws_dtype {
  SWS_F32 = 0,
  SWS_BF16 = 1,
  SWS_FP8_E4M3 = 2  /* KV pages only (sws_sparse_attn_decode_paged): OCP e4m3,
                       value = code * per-tensor scale                        */
} sws_dtype;

/* KV-cache layout flag, OR-ed into the dtype argument of the two decode calls
 * (sws_sparse_attn_decode, sws_sparse_attn_decode_paged).  Without it a cache
 * is token-major ([n_seqs][max_ctx][hkv][d], pages [B][hkv][d]); with it the
 * rows of one KV head are contiguous ([n_seqs][hkv][max_ctx][d], pages
 * [hkv][B][d]), so a selected block is one contiguous run of B rows per head.
 * The result is the same for either layout of the same values. */
enum {
  SWS_KV_HEAD_MAJOR = 0x100
};

/* Walk modes (sws_walk_update_variant, sws_walk_update_row_variant).  The
 * page writes the walk update as R^l = R^(l-1) (A^l)^s and calls s the walk
 * degree; the default reading (mode 0, sws_walk_update) is s hops with the
 * signed sketched scores.  Two other readings are kept behind a mode:
 *   SWS_WALK_POWER    the exponent elementwise: R = rownorm(R_prev T) with
 *                     T[i][j] = M[i][j]^s (j <= i)
 *   SWS_WALK_SOFTMAX  transition probabilities: row i of T is the softmax of
 *                     M[i][0..i]; R = rownorm(R_prev T^s) */
enum {
  SWS_WALK_DEFAULT = 0,
  SWS_WALK_POWER = 1,
  SWS_WALK_SOFTMAX = 2
};

/* Selection flags (sws_select_topk_flags, sws_select_topk_row).  The page
 * leaves the density rule and the GQA treatment open; the default (0) is one
 * budget tau = floor(rho * b / 100) per sequence and one list per query head.
 *   SWS_SELECT_DENSE   every block m <= i (the dense early layers)
 *   SWS_SELECT_ROW_TAU row i keeps tau_i = floor(rho * (i + 1) / 100) earlier
 *                      blocks, the density of its own causal prefix (in decode
 *                      this is the default rule already)
 *   SWS_SELECT_GROUP   one list per KV group: rows are scored by the fp32 sum,
 *                      in ascending head order, of the walk states of the
 *                      group's query heads, and every head of the group gets
 *                      that list */
enum {
  SWS_SELECT_DENSE = 1,
  SWS_SELECT_ROW_TAU = 2,
  SWS_SELECT_GROUP = 4
};

/* Library version (major * 10000 + minor * 100 + patch). */
int sws_version(void);

/* Static string naming a status code. */
const char* sws_status_string(sws_status status);

/* Message describing the most recent failed call on this thread ("" if none). */
const char* sws_last_error_detail(void);

/*
 * sws_sketch - Small-World Sketching of one activation tensor (blog page,
 * section 3.1 block means and section 3.2 Hadamard projection).
 *
 * For every sequence s, block i (tokens [iB, min((i+1)B, n_s))) and head h:
 *   xbar = mean of x[t][h][:] over the tokens the block holds (a partial last
 *          block is averaged over its own token count);
 *   sketch[c] = (1/sqrt(k)) * sum_r signs[r] * H[r][cols[c]] * xbar[r],
 *   with H the natural-order d x d Sylvester-Hadamard matrix, c < k.
 * Called once for Q (n_heads = hq) and once for K (n_heads = hkv).
 *
 *   x           [T][n_heads][d], dtype `dtype` (SWS_F32 or SWS_BF16)
 *   cu_seqlens  [n_seqs + 1] int32, cu_blocks [n_seqs + 1] int32 (device)
 *   total_blocks  host copy of cu_blocks[n_seqs]
 *   d in {64, 128}; B in {64, 128}; 1 <= k <= min(d, 64)
 *   signs       [d] int8 (+1 / -1); cols [k] int32, distinct, < d
 *   sketch_out  fp32; element (h, global block g, c) at h * ld_head + g * k + c,
 *               ld_head >= total_blocks * k
 *   sum_out     optional (NULL to skip) fp32 [n_heads][total_blocks][d]: the
 *               block sums (not divided by the token count)
 */
sws_status sws_sketch(const void* x, int dtype, const int32_t* cu_seqlens, const int32_t* cu_blocks,
                      int32_t n_seqs, int32_t total_blocks, int32_t n_heads, int32_t d, int32_t B,
                      int32_t k, const int8_t* signs, const int32_t* cols, float* sketch_out,
                      int64_t ld_head, float* sum_out, void* stream);

/*
 * sws_sketch_append - decode form of sws_sketch (blog page, section 5: the
 * same block-level sketch for each generated token).  Adds the new token of
 * each sequence to the running sum of its open block and rewrites that
 * block's sketch row, so the row always equals sws_sketch over the tokens the
 * block holds so far.
 *
 *   x_new        [n_seqs][n_heads][d] (the new token of each sequence)
 *   pos          [n_seqs] int32: token index of x_new in its sequence; its
 *                block is c = pos / B; pos % B == 0 restarts the running sum
 *   run_sum      [n_seqs][n_heads][d] fp32, in/out: sum of the open block
 *   sketch_cache [n_seqs][n_heads][b_max][k] fp32: row c is rewritten;
 *                the caller guarantees pos / B < b_max
 */
sws_status sws_sketch_append(const void* x_new, int dtype, const int32_t* pos, int32_t n_seqs,
                             int32_t n_heads, int32_t d, int32_t B, int32_t k, const int8_t* signs,
                             const int32_t* cols, float* run_sum, float* sketch_cache, int32_t b_max,
                             void* stream);

/*
 * sws_sketch_append_qk - sws_sketch_append of a decode step's query and key
 * rows in one launch (the same section: both sketches take the new token
 * each step).  Equal, bit for bit, to sws_sketch_append on (q_new, hq heads,
 * run_sum_q, q_cache) and on (k_new, hkv heads, run_sum_k, k_cache) with the
 * same pos, B, k, signs and cols; dtype applies to both q_new and k_new.
 *   q_new [n_seqs][hq][d], k_new [n_seqs][hkv][d]; run_sum_q [n_seqs][hq][d],
 *   run_sum_k [n_seqs][hkv][d]; q_cache [n_seqs][hq][b_max][k], k_cache
 *   [n_seqs][hkv][b_max][k]; hq + hkv <= 65535
 */
sws_status sws_sketch_append_qk(const void* q_new, const void* k_new, int dtype, const int32_t* pos,
                                int32_t n_seqs, int32_t hq, int32_t hkv, int32_t d, int32_t B,
                                int32_t k, const int8_t* signs, const int32_t* cols, float* run_sum_q,
                                float* run_sum_k, float* q_cache, float* k_cache, int32_t b_max,
                                void* stream);

/*
 * sws_walk_update - the walk state of one layer (blog page, section 4:
 * R^0 = (A^0)^s, R^l = R^(l-1) (A^l)^s), with A = M, the causal sketched
 * block scores M[i][j] = qs_i . ks_j / sqrt(k) for j <= i and 0 for j > i
 * (section 3.2).  s hops per layer; each output row is divided by its largest
 * magnitude (an all-zero row stays zero).  Per sequence and query head:
 *   R_out = rownorm(R_prev * M^s)        (R_prev NULL: the identity)
 * with a finite dynamic range: after every hop, entries smaller in magnitude
 * than 2^-64 times their row's largest magnitude are set to zero (the page
 * fixes no number format; without a floor the walk over many layers keeps
 * entries hundreds of binary orders of magnitude below the row maximum that
 * grow back layers later, so its value would depend on the format).
 *
 *   q_sk  [hq][total_blocks][k] fp32, k_sk [hkv][total_blocks][k] fp32
 *         (sws_sketch output with ld_head = total_blocks * k)
 *   R_prev, R_out  fp32, packed: sequence s starts at element
 *         hq * sum_{s' < s} b_{s'}^2 and holds [hq][b_s][b_s].  R_prev is read
 *         as lower-triangular (entries above the diagonal are ignored).
 *         R_out is written in full (zeros above the diagonal).  R_prev may be
 *         the same buffer as R_out (in-place update).
 *   max_blocks  host: max_s b_s; s >= 1; 1 <= k <= 64
 */
sws_status sws_walk_update(const float* q_sk, const float* k_sk, int32_t hq, int32_t hkv, int32_t k,
                           const int32_t* cu_blocks, int32_t n_seqs, int32_t total_blocks,
                           int32_t max_blocks, int32_t s, const float* R_prev, float* R_out,
                           void* stream);

/*
 * sws_walk_update_row - decode form of sws_walk_update: only the row of the
 * open block c = cur_block[seq] (blog page, section 5).  Equals row c of
 * sws_walk_update over the first c + 1 blocks (same hops, same floor).
 *
 *   q_sk_cache [n_seqs][hq][b_max][k], k_sk_cache [n_seqs][hkv][b_max][k] fp32,
 *              both 16-byte aligned
 *   cur_block  [n_seqs] int32, 0 <= cur_block < b_max; b_max <= 4096
 *   r_prev     NULL (the unit row e_c) or [n_seqs][hq][b_max]; may equal r_out
 *   r_out      [n_seqs][hq][b_max]; entries above cur_block are written 0
 */
sws_status sws_walk_update_row(const float* q_sk_cache, const float* k_sk_cache, int32_t hq,
                               int32_t hkv, int32_t k, int32_t n_seqs, const int32_t* cur_block,
                               int32_t b_max, int32_t s, const float* r_prev, float* r_out,
                               void* stream);

/*
 * sws_walk_update_variant - sws_walk_update with a walk mode (SWS_WALK_*).
 * The variants form the b x b transition matrix T of every (sequence, head)
 * explicitly and multiply lower-triangular matrices in fp32 (cost s b^3 / 3
 * multiply-adds per head for SWS_WALK_SOFTMAX, b^3 / 3 for SWS_WALK_POWER).
 *
 *   same arguments and layouts as sws_walk_update, plus
 *   mode        SWS_WALK_DEFAULT (then ws may be NULL), SWS_WALK_POWER or
 *               SWS_WALK_SOFTMAX, else SWS_ERR_UNSUPPORTED
 *   walk_numel  hq * sum_s b_s^2 (the element count of R)
 *   ws          workspace of sws_walk_variant_workspace_size(walk_numel) bytes
 *               (T and two products, packed like R)
 *   max_blocks <= 4096; R_prev may equal R_out
 */
sws_status sws_walk_update_variant(const float* q_sk, const float* k_sk, int32_t hq, int32_t hkv,
                                   int32_t k, const int32_t* cu_blocks, int32_t n_seqs,
                                   int32_t total_blocks, int32_t max_blocks, int32_t s, int32_t mode,
                                   const float* R_prev, float* R_out, int64_t walk_numel, void* ws,
                                   size_t ws_bytes, void* stream);

/* Workspace bytes of sws_walk_update_variant for walk_numel = hq * sum b_s^2. */
size_t sws_walk_variant_workspace_size(int64_t walk_numel);

/*
 * sws_walk_update_row_variant - decode form of sws_walk_update_variant: row
 * c = cur_block[seq] only, computed with the entries of T formed on the fly
 * from the sketch caches.  Arguments and layouts as sws_walk_update_row, plus
 * mode (SWS_WALK_*; SWS_WALK_DEFAULT runs sws_walk_update_row).
 */
sws_status sws_walk_update_row_variant(const float* q_sk_cache, const float* k_sk_cache, int32_t hq,
                                       int32_t hkv, int32_t k, int32_t n_seqs,
                                       const int32_t* cur_block, int32_t b_max, int32_t s,
                                       int32_t mode, const float* r_prev, float* r_out, void* stream);

/*
 * sws_select_topk - top-tau key blocks per query block (blog page, section
 * 4).  For sequence s, tau_s = floor(rho_percent * b_s / 100).  Row i keeps the
 * tau_s earlier blocks m < i with the largest R[i][m] (ties: lower m first;
 * -0 equals +0), all of them when i <= tau_s, plus the diagonal block i.
 * dense != 0 keeps every block m <= i.  Lists are ascending local block
 * indices.  R must hold no NaN.
 *
 *   R      packed as in sws_walk_update
 *   idx    [hq][total_blocks][width] int32; cnt [hq][total_blocks] int32
 *   width  >= min(max_blocks, floor(rho_percent * max_blocks / 100) + 1),
 *          >= max_blocks when dense
 *   max_blocks <= 4096
 */
sws_status sws_select_topk(const float* R, int32_t hq, const int32_t* cu_blocks, int32_t n_seqs,
                           int32_t total_blocks, int32_t max_blocks, int32_t rho_percent,
                           int32_t dense, int32_t width, int32_t* idx, int32_t* cnt, void* stream);

/*
 * sws_select_topk_flags - sws_select_topk with the selection variants of the
 * SWS_SELECT_* flags; hkv (a divisor of hq) is used by SWS_SELECT_GROUP only.
 * Same layouts, limits and errors as sws_select_topk; with
 * SWS_SELECT_ROW_TAU the width bound is the same (the last row has the
 * largest budget).
 */
sws_status sws_select_topk_flags(const float* R, int32_t hq, int32_t hkv, const int32_t* cu_blocks,
                                 int32_t n_seqs, int32_t total_blocks, int32_t max_blocks,
                                 int32_t rho_percent, int32_t flags, int32_t width, int32_t* idx,
                                 int32_t* cnt, void* stream);

/*
 * sws_select_topk_row - decode form of sws_select_topk for the open block
 * c = cur_block[seq] (b = c + 1 blocks, tau = floor(rho_percent * b / 100)):
 * each decode step keeps the top-tau blocks of the same block-level walk
 * score as prefill (blog page, section 5, decode; section 4, top-tau
 * selection).  It is followed by the union over the query heads of each KV
 * group: the ascending list of blocks that any head of the group keeps, with
 * a bit mask of the heads (bit g = head hkv_group * (hq/hkv) + g) that keep
 * it, so one pass over the cache serves the group (the page lists GQA among
 * the integration costs, section 11.4).
 *
 *   r          [n_seqs][hq][b_max] fp32 (sws_walk_update_row output)
 *   idx, cnt   optional (both NULL or both set): per-head lists
 *              [n_seqs][hq][width] and counts [n_seqs][hq]
 *   union_idx  [n_seqs][hkv][union_width] int32, union_mask same shape uint32,
 *   union_cnt  [n_seqs][hkv] int32
 *   width      >= min(b_max, floor(rho_percent * b_max / 100) + 1)
 *   union_width >= min(b_max, (hq/hkv) * floor(rho_percent * b_max / 100) + 1)
 *   hq / hkv <= 16, b_max <= 4096
 *   flags      SWS_SELECT_* bits (0 or 1 keep the meaning of the former
 *              `dense` argument; SWS_SELECT_ROW_TAU changes nothing here;
 *              with SWS_SELECT_GROUP the union is the group's shared list,
 *              kept by every head)
 */
sws_status sws_select_topk_row(const float* r, int32_t hq, int32_t hkv, int32_t n_seqs,
                               const int32_t* cur_block, int32_t b_max, int32_t rho_percent,
                               int32_t flags, int32_t width, int32_t* idx, int32_t* cnt,
                               int32_t* union_idx, int32_t* union_cnt, uint32_t* union_mask,
                               int32_t union_width, void* stream);

/*
 * sws_sparse_attn_prefill - block-sparse attention over the selected blocks
 * on the original Q, K, V (blog page, sections 4 and 5).  Token t of block i,
 * query head h: softmax over the keys u <= t lying in the blocks of
 * idx[h][g][0 .. cnt[h][g]) (g = global block), scaled by `scale`,
 * renormalised over those keys; out = weights . V.
 *
 *   q [T][hq][d], k and v [T][hkv][d]; out [T][hq][d] (same dtype)
 *   dtype SWS_BF16: bf16 MFMA kernel (q is multiplied by scale * log2(e)
 *   and rounded to bf16 once, so the scores come out in log2 units; fp32
 *   softmax and accumulation; output rounded to nearest even); SWS_F32:
 *   fp32 kernel (no such rounding)
 *   idx, cnt as produced by sws_select_topk; idx == NULL means dense causal
 *   (every block <= i); cnt ignored then
 *   lse  optional [hq][T] fp32: natural-log sum of exp of the scaled scores
 *   ws   workspace of at least sws_prefill_workspace_size(...) bytes (the
 *        bf16 path stages V transposed per block there; may be NULL when the
 *        size is 0)
 *   d in {64, 128}; B in {64, 128}; q, k, v, out and ws 16-byte aligned
 */
sws_status sws_sparse_attn_prefill(const void* q, const void* k, const void* v, int dtype,
                                   const int32_t* cu_seqlens, const int32_t* cu_blocks, int32_t n_seqs,
                                   int32_t total_blocks, int32_t max_blocks, int32_t hq, int32_t hkv,
                                   int32_t d, int32_t B, const int32_t* idx, const int32_t* cnt,
                                   int32_t width, float scale, void* out, float* lse, void* ws,
                                   size_t ws_bytes, void* stream);

/* Workspace bytes sws_sparse_attn_prefill needs (hkv * total_blocks * d * B * 2
 * for SWS_BF16, 0 for SWS_F32). */
size_t sws_prefill_workspace_size(int dtype, int32_t total_blocks, int32_t hkv, int32_t d,
                                  int32_t B);

/*
 * sws_sparse_attn_decode - single-token attention of each sequence over the
 * blocks its query heads kept (blog page, section 5; decode is bound by the
 * KV-cache read, section 8.3).  Split-KV: the union list of every
 * (sequence, KV head) is cut into chunks processed in parallel, then merged
 * with a log-sum-exp combine; the block's KV rows are read once for all the
 * query heads of the group that kept it.
 *
 *   q       [n_seqs][hq][d]; k_cache, v_cache [n_seqs][max_ctx][hkv][d], or
 *           [n_seqs][hkv][max_ctx][d] with SWS_KV_HEAD_MAJOR in dtype
 *   ctx_len [n_seqs] int32: tokens in the cache including the new one
 *           (the new token is the last; its block is the open block)
 *   union_idx / union_cnt / union_mask as produced by sws_select_topk_row
 *   (union_idx NULL: dense, every block of the context for every head)
 *   out     [n_seqs][hq][d] (dtype of q); lse optional [n_seqs][hq] fp32
 *   ws      workspace of at least sws_decode_workspace_size(...) bytes
 *   d in {64, 128}; B in {64, 128}; hq / hkv <= 16; n_seqs * hkv <= 8192
 *   (else SWS_ERR_UNSUPPORTED).  The blocks to read over all pairs are split
 *   evenly across the workgroups, so the cost follows the total number of
 *   blocks, not the largest list.
 */
sws_status sws_sparse_attn_decode(const void* q, const void* k_cache, const void* v_cache, int dtype,
                                  const int32_t* ctx_len, int32_t n_seqs, int32_t max_ctx, int32_t hq,
                                  int32_t hkv, int32_t d, int32_t B, const int32_t* union_idx,
                                  const int32_t* union_cnt, const uint32_t* union_mask,
                                  int32_t union_width, float scale, void* out, float* lse, void* ws,
                                  size_t ws_bytes, void* stream);

/* Size of the fixed device array holding the split-KV records of
 * sws_sparse_attn_decode_noalloc (one copy per GPU the library runs on). */
#define SWS_DECODE_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * sws_sparse_attn_decode_noalloc - sws_sparse_attn_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops
 * that forbid allocation): the same computation and result, bit for bit, with
 * the split-KV records kept in a fixed device array of
 * SWS_DECODE_NOALLOC_SCRATCH_BYTES instead of a workspace argument.
 *
 *   arguments as sws_sparse_attn_decode without ws / ws_bytes; the caller
 *   still passes q, the caches, the lists and out (and lse).
 *   The array of the current device (hipGetDevice) is used: `stream` must
 *   belong to that device.  Its address is looked up once per device, on
 *   the first call there.
 *   Returns SWS_ERR_WORKSPACE when the call needs more than
 *   SWS_DECODE_NOALLOC_SCRATCH_BYTES (sws_decode_workspace_size gives the
 *   need: 4.5 MB for 16 sequences x 8 KV heads x 4 query heads per group,
 *   d = 128).
 *   Every call on one GPU shares that GPU's array and leaves its contents
 *   behind; nothing in it needs to start at any value.  Calls that may run
 *   at the same time on one GPU (on different streams, or from different
 *   threads without ordering) race on the array and give wrong results:
 *   order them on one stream.
 */
sws_status sws_sparse_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                          int dtype, const int32_t* ctx_len, int32_t n_seqs,
                                          int32_t max_ctx, int32_t hq, int32_t hkv, int32_t d,
                                          int32_t B, const int32_t* union_idx,
                                          const int32_t* union_cnt, const uint32_t* union_mask,
                                          int32_t union_width, float scale, void* out, float* lse,
                                          void* stream);

/* Workspace bytes sws_sparse_attn_decode needs for these sizes (a work plan
 * and per-range partial softmax states; union_width does not change it). */
size_t sws_decode_workspace_size(int32_t n_seqs, int32_t hq, int32_t hkv, int32_t d, int32_t B,
                                 int32_t union_width);

/*
 * sws_sparse_attn_decode_paged - sws_sparse_attn_decode over a paged KV cache,
 * with bf16 or fp8 pages.  The deep-reading page lists paged KV caches,
 * continuous batching and mixed precision among what a serving system adds
 * around the method's kernels (section 11.4); this is that layout for the
 * decode step of section 5.  The result is the one sws_sparse_attn_decode
 * gives on the gathered (and, for fp8, dequantised) contiguous cache.
 *
 *   q            [n_seqs][hq][d] bf16
 *   k_pages,     [num_pages][B][hkv][d] ([num_pages][hkv][B][d] with
 *   v_pages      SWS_KV_HEAD_MAJOR in kv_dtype), one page per KV block of B
 *                tokens, dtype kv_dtype: SWS_BF16, or SWS_FP8_E4M3 whose
 *                value is code * k_scale (K) or code * v_scale (V); scales
 *                are ignored for SWS_BF16
 *   block_table  [n_seqs][table_width] int32: page of logical block j of
 *                sequence s.  Sequences come and go between calls
 *                (continuous batching) by rewriting their table rows; pages
 *                may be shared.  The caller guarantees table_width * B >=
 *                ctx_len[s] and 0 <= page < num_pages; entries out of range
 *                are clamped on the device (a wrong result, never a stray
 *                access).
 *   ctx_len, union_idx / union_cnt / union_mask, scale, out, lse: as for
 *                sws_sparse_attn_decode (out is bf16)
 *   ws           workspace of sws_decode_workspace_size(n_seqs, hq, hkv, d,
 *                B, union_width) bytes
 *   Same size limits as sws_sparse_attn_decode; pages 16-byte aligned.
 */
sws_status sws_sparse_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                                        int kv_dtype, float k_scale, float v_scale,
                                        const int32_t* block_table, int32_t table_width,
                                        int32_t num_pages, const int32_t* ctx_len, int32_t n_seqs,
                                        int32_t hq, int32_t hkv, int32_t d, int32_t B,
                                        const int32_t* union_idx, const int32_t* union_cnt,
                                        const uint32_t* union_mask, int32_t union_width, float scale,
                                        void* out, float* lse, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SWS_H */
