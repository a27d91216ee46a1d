/*
 * sparse_attn.h -- C ABI of the gfx950 (MI355X) block-sparse attention library
 * with pooled block routing.
 *
 * The method (three calls, one per stage):
 *
 *   1. sparse_attn_block_pool: cut the N tokens into M = ceil(N/block)
 *      contiguous blocks; per block take the mean query, the mean key and
 *      the sum of the values.  (PISA explainer, kodorricoding.tistory.com/108,
 *      section "how candidate blocks are narrowed" and its routing table;
 *      FlashPrefill summary, gist.science/ko/paper/2603.06199, technical
 *      summary 2(a) "block approximation": average-pooled keys.)
 *
 *   2. sparse_attn_select: score every (query block I, key block J) pair
 *      with the scaled pooled logit s_IJ = scale * qbar_I . kbar_J and keep,
 *      per query block, either every J with s_IJ >= alpha * max_J s_IJ
 *      (FlashPrefill summary 2(b), max-based dynamic threshold, no sort) or
 *      the top-k blocks at a given density (PISA explainer, "minimal
 *      documented usage": density=0.15, block_size=64).  The kept blocks are
 *      written as ascending index lists (FlashPrefill summary 2(c):
 *      index-driven jumping to the selected block coordinates).
 *
 *   3. sparse_attn_fwd: exact softmax attention over the tokens of the
 *      listed blocks, with the running max / sum recurrence of the
 *      FlashAttention tutorial (blog.mna-game.duckdns.org post 22, section 2,
 *      online softmax equation).  With approx=1 every eligible block that is
 *      not listed enters the same running max and sum as one pseudo-key
 *      kbar_J of multiplicity n_J carrying the value sum SigmaV_J -- the
 *      0th-order term exp(q.kbar_J) * (SigmaV_J, n_J) (PISA explainer, routing
 *      table and section "why softmax survives approximating unselected
 *      blocks").  The first-order global-statistic correction mentioned on
 *      the same page is not implemented (the page does not define it).
 *
 * Readings where the pages are silent (both this library and its test oracle
 * follow them):
 *   - scale defaults to 1/sqrt(head_dim) for token and pooled logits;
 *   - alpha mode: if a row's max score m is not positive the threshold is m
 *     itself (only the arg-max blocks are kept); a score equal to the
 *     threshold is kept;
 *   - density mode: k = ceil(density * |E_I| - 1e-9) evaluated in double,
 *     clamped to [1, |E_I|]; equal scores are taken in ascending J;
 *   - causal: key block J is eligible for query block I iff J <= I; inside
 *     the diagonal block a key j is visible to query i iff j <= i.  With
 *     causal=1 and approx=1 the diagonal block is always exact (added to the
 *     list by sparse_attn_select), since its pooled key would mix in later
 *     tokens; the tail covers the unlisted J < I;
 *   - Q head h reads KV head h / (heads_q / heads_kv) (consecutive grouping);
 *   - the last block may be short (n_J < block); pooled means divide by n_J.
 *
 * Data layout (all tensors dense, row-major, 16-byte aligned device memory):
 *   q    [batch, heads_q,  seq_len, head_dim]   element type = dtype
 *   k, v [batch, heads_kv, seq_len, head_dim]   element type = dtype
 *   out  [batch, heads_q,  seq_len, head_dim]   element type = dtype
 *   q_bar [batch, heads_q,  M, head_dim] float32  (block means of q)
 *   k_bar [batch, heads_kv, M, head_dim] float32  (block means of k)
 *   v_sum [batch, heads_kv, M, head_dim] float32  (block sums of v)
 *   tail  bf16 inputs with approx=1 only: [2, batch, heads_kv, M, head_dim]
 *         bfloat16 -- the block means of k, then the block means of v
 *         (v_sum / n_J): the pseudo-keys and their values in the matrix-core
 *         dtype, written once by the pool pass for all query blocks
 *   blk_idx [batch, heads_q, M, M] int32: row (b,h,I) holds blk_cnt[b,h,I]
 *           strictly ascending eligible key-block indices; entries past the
 *           count are left untouched by sparse_attn_select and never read
 *           by sparse_attn_fwd
 *   blk_cnt [batch, heads_q, M] int32, 1 <= count <= M
 *
 * Ownership and threading: the caller allocates and frees every buffer
 * (sizes from sparse_attn_buffer_sizes).  The library never allocates, frees
 * or synchronises and keeps no state between calls, except for the one
 * fixed device array that sparse_attn_bwd_noalloc uses as its scratch (see
 * there: calls of that entry point that overlap on one device race); every
 * other entry point is reentrant.  Each
 * compute call validates its arguments on the host, then enqueues kernels on
 * the caller's HIP stream (`stream`, a hipStream_t; NULL = default stream)
 * and returns without waiting.
 *
 * Errors: argument errors return a non-zero sa_status before anything is
 * enqueued.  SA_ERR_HIP means a launch reported an error (hipGetLastError).
 * Faults inside a kernel surface at the caller's next synchronisation.
 * Caller-supplied block lists (sparse_attn_fwd, sparse_attn_fwd_lse,
 * sparse_attn_bwd) must satisfy the layout above, and with causal=1 and
 * approx=1 every row I must list its diagonal block I (the tail must not
 * take the pooled key of the diagonal block, which holds later tokens).  The
 * compute calls do not check lists (an entry outside [0, M) makes the
 * kernels read and write out of bounds); sparse_attn_check_lists checks
 * them on the device.
 *
 * Supported: head_dim in {64, 128}; block in {64, 128}; M <= 2048;
 * dtype float32 or bfloat16; heads_q a multiple of heads_kv.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPARSE_ATTN_ABI_VERSION 6

typedef enum {
  SA_OK = 0,
  SA_ERR_NULL = 1,         /* a required pointer is NULL                          */
  SA_ERR_SHAPE = 2,        /* a size is out of range or inconsistent               */
  SA_ERR_DTYPE = 3,        /* dtype is not SA_DTYPE_F32 / SA_DTYPE_BF16             */
  SA_ERR_PARAM = 4,        /* alpha / density / select_mode / flags out of range   */
  SA_ERR_ALIGN = 5,        /* a tensor pointer is not 16-byte aligned              */
  SA_ERR_UNSUPPORTED = 6,  /* valid in principle, not built (head_dim, block, M)   */
  SA_ERR_HIP = 7,          /* the HIP runtime reported an error at launch          */
  SA_ERR_SCRATCH = 8       /* the problem needs more than the library's fixed
                              scratch (sparse_attn_bwd_noalloc only)              */
} sa_status;

enum { SA_DTYPE_F32 = 0, SA_DTYPE_BF16 = 1 };
enum { SA_SELECT_ALPHA = 0, SA_SELECT_DENSITY = 1 };

typedef struct {
  int32_t batch;        /* B >= 1                                            */
  int32_t heads_q;      /* Hq >= 1                                           */
  int32_t heads_kv;     /* Hkv >= 1, Hq % Hkv == 0                           */
  int32_t seq_len;      /* N >= 1                                            */
  int32_t head_dim;     /* d: 64 or 128                                      */
  int32_t block;        /* b: tokens per block, 64 or 128                    */
  int32_t dtype;        /* SA_DTYPE_F32 or SA_DTYPE_BF16 (q, k, v, out)      */
  int32_t select_mode;  /* SA_SELECT_ALPHA or SA_SELECT_DENSITY              */
  double alpha;         /* alpha mode: 0 < alpha <= 1                        */
  double density;       /* density mode: 0 < density <= 1                    */
  float scale;          /* logit scale; <= 0 selects 1/sqrt(head_dim)        */
  int32_t causal;       /* 0 or 1                                            */
  int32_t approx;       /* 0 or 1: fold unselected blocks in as 0th order    */
} sa_desc;

typedef struct {        /* bytes of each caller-allocated buffer */
  size_t q_bar, k_bar, v_sum, tail, blk_idx, blk_cnt;
} sa_sizes;

/* Bytes needed for the intermediate buffers of `desc` (host only, no GPU).
 * v_sum is 0 when approx == 0; tail is 0 unless approx == 1 and dtype is
 * bf16.  Errors: SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_DTYPE, SA_ERR_PARAM,
 * SA_ERR_UNSUPPORTED. */
sa_status sparse_attn_buffer_sizes(const sa_desc* desc, sa_sizes* sizes);

/* Stage 1, block pooling: one pass over q, k (and v when approx) writing
 * q_bar, k_bar (block means) and v_sum (block sums), float32, and for bf16
 * inputs with approx the bf16 tail operands.  v, v_sum and tail may be NULL
 * when approx == 0 (then they are ignored); tail may be NULL for float32. */
sa_status sparse_attn_block_pool(const sa_desc* desc, const void* q, const void* k,
                                 const void* v, float* q_bar, float* k_bar, float* v_sum,
                                 void* tail, void* stream);

/* Stage 2, scoring + selection in one kernel: pooled scores (float32, kept
 * on chip, never written), alpha-threshold or top-k selection, compaction of
 * every row into blk_idx / blk_cnt. */
sa_status sparse_attn_select(const sa_desc* desc, const float* q_bar, const float* k_bar,
                             int32_t* blk_idx, int32_t* blk_cnt, void* stream);

/* Stages 1 + 2 in one launch ("fused routing": FlashPrefill summary 2(a),
 * pattern discovery from pooled blocks, and 2(b)-(c), threshold and index
 * lists, without a second launch).  Writes exactly what
 * sparse_attn_block_pool followed by sparse_attn_select writes (same
 * buffers, same values, same arguments and errors as the two calls).  The
 * kernel is launched cooperatively (all its workgroups resident at once, one
 * grid-wide barrier between pooling and scoring); SA_ERR_HIP if the device
 * refuses the cooperative launch.  Kept for callers that want the routing in
 * one launch; the library's own layer does not use it: on MI355X the two
 * separate calls are faster (59 us against 23 + 10 us for the 8K image
 * layer), since the grid-wide barrier, which must flush the pooled vectors
 * out of one XCD's L2 for the other seven, costs more than the launch it
 * saves. */
sa_status sparse_attn_route(const sa_desc* desc, const void* q, const void* k, const void* v,
                            float* q_bar, float* k_bar, float* v_sum, void* tail, int32_t* blk_idx,
                            int32_t* blk_cnt, void* stream);

/* Stage 3, attention: exact online-softmax attention over the listed blocks
 * (+ the 0th-order tail over unlisted eligible blocks when approx == 1),
 * output in dtype.  The tail reads k_bar / v_sum for float32 inputs and
 * `tail` for bf16 inputs; unused ones may be NULL (all three when
 * approx == 0).  The lists may come from sparse_attn_select or from the
 * caller (e.g. every eligible block for dense attention). */
sa_status sparse_attn_fwd(const sa_desc* desc, const void* q, const void* k, const void* v,
                          const float* k_bar, const float* v_sum, const void* tail,
                          const int32_t* blk_idx, const int32_t* blk_cnt, void* out,
                          void* stream);

/* Violation flags of sparse_attn_check_lists (OR-ed over all rows). */
enum {
  SA_LIST_COUNT = 1,        /* blk_cnt outside [1, |E_I|] (|E_I| = M, or I + 1 if causal) */
  SA_LIST_RANGE = 2,        /* an entry outside [0, M)                                   */
  SA_LIST_ORDER = 4,        /* entries not strictly ascending                            */
  SA_LIST_INELIGIBLE = 8,   /* causal: an entry J > I                                     */
  SA_LIST_NO_DIAGONAL = 16  /* causal with approx: the row does not list its block I      */
};

/* Check caller-built block lists on the device, one wave per row, against
 * the layout the attention kernels rely on (the lists of sparse_attn_select
 * always pass).  Writes three uint32 to `result` (device memory, 16-byte
 * aligned): the OR of the SA_LIST_* flags of every bad row (0 = all rows
 * valid), the number of bad rows, and the lowest bad row index
 * ((b * heads_q + h) * M + I; 0xFFFFFFFF if none).  Reads at most M entries
 * per row.  Asynchronous like the other calls: read `result` after the
 * stream has completed.  Errors: as sparse_attn_fwd's argument checks. */
sa_status sparse_attn_check_lists(const sa_desc* desc, const int32_t* blk_idx, const int32_t* blk_cnt,
                                  uint32_t* result, void* stream);

/* ---- Training: gradients of stage 3 (PISA explainer, "minimal documented
 * usage": the simplified 0th-order variant is the one that supports
 * training).  Gradients flow through the listed blocks and through the
 * pooled pseudo-keys of the tail (their block means spread dkbar_J / n_J and
 * dvbar_J / n_J over the block's tokens); the selection is held fixed.
 * bfloat16 inputs only (SA_ERR_UNSUPPORTED for float32). */

/* sparse_attn_fwd that also writes lse [batch, heads_q, seq_len] float32:
 * the natural log of each query row's softmax denominator (exact keys and
 * pooled pseudo-keys with their multiplicity), which sparse_attn_bwd needs. */
sa_status sparse_attn_fwd_lse(const sa_desc* desc, const void* q, const void* k, const void* v,
                              const float* k_bar, const float* v_sum, const void* tail,
                              const int32_t* blk_idx, const int32_t* blk_cnt, void* out, float* lse,
                              void* stream);

typedef struct {        /* bytes of the backward's caller-allocated buffers */
  size_t lse;           /* [B, Hq, N] float32 (written by sparse_attn_fwd_lse)          */
  size_t delta;         /* 2 x [B, Hq, N] float32 scratch: dO . o, then -lse log2 e     */
  size_t sel_bits;      /* [B, Hq, M, ceil(M/32)] uint32 scratch: the selection as bits */
  size_t col_idx;       /* [B, Hkv, M, (Hq/Hkv)*M] int32 scratch: transposed lists      */
  size_t col_cnt;       /* [B, Hkv, M] int32 scratch                                     */
  size_t dk_bar;        /* 16 x [B, Hkv, M, d] float32 partial sums (0 unless approx)   */
  size_t dv_bar;        /* 16 x [B, Hkv, M, d] float32 partial sums (0 unless approx)   */
} sa_bwd_sizes;

/* Bytes of the backward buffers for `desc` (host only). */
sa_status sparse_attn_bwd_buffer_sizes(const sa_desc* desc, sa_bwd_sizes* sizes);

/* Gradients of sum(dout * out) with respect to q, k, v, for the lists the
 * forward used (blk_idx / blk_cnt) and its out and lse.  Writes dq [B, Hq,
 * N, d], dk and dv [B, Hkv, N, d] in bfloat16 (query heads of one KV group
 * add into its dk, dv); uses delta, sel_bits, col_idx, col_cnt and, with
 * approx, dk_bar / dv_bar as scratch (no initial contents needed).  `tail`
 * is the pool pass's bf16 tail operands (approx only).  Lists must be
 * strictly ascending and eligible, as for sparse_attn_fwd.  Errors as for
 * the forward; SA_ERR_UNSUPPORTED for float32 inputs. */
sa_status sparse_attn_bwd(const sa_desc* desc, const void* q, const void* k, const void* v,
                          const void* tail, const int32_t* blk_idx, const int32_t* blk_cnt,
                          const void* out, const float* lse, const void* dout, float* delta,
                          uint32_t* sel_bits, int32_t* col_idx, int32_t* col_cnt, float* dk_bar,
                          float* dv_bar, void* dq, void* dk, void* dv, void* stream);

/* ---- For callers that cannot allocate (code under HIP graph capture,
 * serving loops or harnesses that forbid hipMalloc): sparse_attn_bwd with
 * its scratch taken from a fixed array of device memory that the library
 * owns, instead of caller buffers.  The array holds
 * SPARSE_ATTN_BWD_NOALLOC_SCRATCH_BYTES on each device the entry point runs
 * on, from its first call there until the process ends; the entry point
 * itself calls no allocator.  It runs the same kernels as sparse_attn_bwd and
 * gives the same results.  All calls on one device share its array: calls on
 * one stream are ordered, calls that overlap on one device (several streams
 * or threads) race and must not be made.  `stream` must belong to the
 * current device.  The scratch need is the sum of sparse_attn_bwd_buffer_sizes'
 * delta, sel_bits, col_idx, col_cnt, dk_bar and dv_bar, each rounded up to
 * 256 bytes; beyond the array the call returns SA_ERR_SCRATCH before any
 * launch.  Other errors as for sparse_attn_bwd. */
#define SPARSE_ATTN_BWD_NOALLOC_SCRATCH_BYTES (64u << 20)

/* Scratch bytes `desc` needs (*need) and the array's size (*cap); host only. */
sa_status sparse_attn_bwd_noalloc_scratch(const sa_desc* desc, size_t* need, size_t* cap);

sa_status sparse_attn_bwd_noalloc(const sa_desc* desc, const void* q, const void* k, const void* v,
                                  const void* tail, const int32_t* blk_idx, const int32_t* blk_cnt,
                                  const void* out, const float* lse, const void* dout, void* dq,
                                  void* dk, void* dv, void* stream);

/* Static, human-readable text of a status code. */
const char* sparse_attn_status_string(sa_status status);

/* SPARSE_ATTN_ABI_VERSION of the loaded library. */
int32_t sparse_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
