/*
 * wise.h - C ABI of the WISE working-set attention library (gfx950 / MI355X).
 *
 * WISE ("Attention Routing Stabilizes Early: Working-Set Inference for
 * Recurrent Language Models") runs unrestricted causal attention during the
 * first td recurrent steps, measures how much attention each query block
 * sends to each key block, turns that into a block support once, and then
 * recomputes attention only inside that support in the remaining steps.
 * This library provides the four device operations of that path:
 *
 *   wise_full_attn        dense causal attention (Section 3, Eq. 2)
 *   wise_full_attn_accum  dense causal attention + block mass (Eq. 2 and 5)
 *   wise_select_support   mass -> CSR block support (Section 5.1, Eq. 6)
 *   wise_select_variant   temporal union and early-static controls (Eq. 18-22)
 *   wise_support_mass     retained attention mass of a support (diagnostic)
 *   wise_support_overlap  per-row overlap of two supports (Jaccard, Eq. 24-25)
 *   wise_sparse_attn      attention inside the support (Section 5.2, Eq. 7-8)
 *
 * Conventions shared by every call
 * --------------------------------
 * - Tensors are device pointers owned by the caller; the library allocates
 *   no device memory and keeps no state between calls.
 * - Q, K, V, O are bf16 (raw 16-bit patterns), contiguous, laid out
 *   [batch][heads][seq_len][head_dim] (K and V: [batch][kv_heads][...]).
 *   Q, K and V are read-only; O may not alias them.  All pointers must be
 *   16-byte aligned.
 * - Attention is always causal: key j is admissible for query i iff j <= i
 *   (the mask M of Eq. 2); the descriptor has no switch for it.  Scores are
 *   (q_i . k_j) * scale, scale = 1/sqrt(head_dim) unless
 *   desc->softmax_scale > 0.
 * - The sequence is cut into consecutive blocks of block_size positions
 *   from position 0 (Section 5.1); n_blocks = ceil(seq_len / block_size).
 *   When seq_len is not a multiple of block_size the last block is short:
 *   it holds seq_len - (n_blocks - 1) * block_size positions, and that count
 *   is its |I_q| in Eq. (5).  A "row" is one (batch, head, query block) triple, numbered
 *   r = (b * heads + h) * n_blocks + q; there are batch*heads*n_blocks rows.
 * - Empty calls: batch, heads or seq_len may be 0.  A call with
 *   batch*heads*n_blocks == 0 computes nothing and its tensor pointers may
 *   be NULL; the selection calls still write row_ptr[0] = 0 (row_ptr must
 *   then point at that one entry), every other call launches nothing.
 * - Every call is asynchronous on `stream` (a hipStream_t passed as void*,
 *   so that this header needs no HIP include; NULL = the null stream) and
 *   never synchronises the host.  Arguments are validated on the
 *   host first: on any error nothing is launched and nothing is written.
 * - Results are deterministic: identical inputs give bitwise identical
 *   outputs (no atomics on any value path).
 * - No C++ exception crosses this interface.  The library is thread-safe.
 * - Setting the environment variable WISE_TRACE (to anything but "" or
 *   "0") prints one line per kernel launch on stderr: kernel, grid,
 *   workgroup size, dynamic LDS and the launch parameters.
 *
 * Supported shapes: head_dim in {64, 96, 128}; block_size in {16, 32, 64,
 * 128} (16: the attention calls need seq_len % 32 == 0); seq_len <= 65536;
 * batch*heads*n_blocks < 2^31.
 */
#ifndef WISE_H
#define WISE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WISE_ABI_VERSION 5

typedef enum {
  WISE_OK = 0,
  WISE_ERR_INVALID_ARG = 1,  /* null pointer, bad size, eta outside (0,1], ... */
  WISE_ERR_UNSUPPORTED = 2,  /* valid but not built: head_dim or block_size    */
  WISE_ERR_CAPACITY = 3,     /* col_capacity below wise_select_max_nnz()       */
  WISE_ERR_HIP = 4,          /* the HIP runtime reported a launch error        */
  WISE_ERR_OVERFLOW = 5      /* reserved, never returned: the kernels raise the
                                softmax reference max whenever a score exceeds it
                                by more than 64 (log2 units), so exp terms stay
                                below 2^64 and no fp32 sum can overflow for
                                supported shapes (seq_len <= 65536)           */
} wise_status_t;

/* Shape of one attention call.  All tensors of a call share it. */
typedef struct {
  int32_t batch;       /* >= 0                                         */
  int32_t heads;       /* >= 0 query heads (Q, O, mass and CSR rows)   */
  int32_t seq_len;     /* >= 0; the last block may be short            */
  int32_t head_dim;    /* 64, 96 or 128                                 */
  int32_t block_size;  /* B of Section 5.1: 16, 32, 64 or 128 (16: the
                          attention calls need seq_len % 32 == 0; they run
                          two 16-blocks per 32 x 32 tile)                */
  float softmax_scale; /* <= 0 selects 1/sqrt(head_dim)                 */
  int32_t kv_heads;    /* K/V heads: 0 (= heads) or a divisor of heads;
                          query head h reads K/V head h / (heads / kv_heads)
                          (grouped-query attention)                     */
} wise_attn_desc_t;

/*
 * Dense causal attention, Eq. (2): O = softmax(Q K^T * scale + M) V.
 *
 * q:       bf16 [batch][heads][seq_len][head_dim] (read).
 * k, v:    bf16 [batch][kv_heads][seq_len][head_dim] (read; kv_heads as in
 *          the descriptor, heads when it is 0).
 * o:       bf16, q's layout (written, rounded to nearest even).
 * lse:     optional (NULL to skip) fp32 [batch][heads][seq_len]; receives
 *          the natural-log row normaliser log(sum_j exp(score_ij)).  The sum
 *          is formed from the exp terms rounded to bf16, the same weights
 *          that multiply V (so O is exactly the weighted mean under them);
 *          each term then carries a relative rounding error of at most 2^-9,
 *          and the result differs from the exact log-sum by at most
 *          -log(1 - 2^-9) ~ 2e-3 (in practice a few 1e-4, as the roundings
 *          of many terms cancel).
 * This is the dense baseline that the late steps are compared against.
 */
wise_status_t wise_full_attn(const wise_attn_desc_t* desc, const void* q, const void* k,
                             const void* v, void* o, float* lse, void* stream);

/*
 * Discovery step: dense causal attention (Eq. 2) plus the block mass of
 * Section 5.1, Eq. (5), r_qb = (1/|I_q|) sum_{i in I_q} sum_{j in I_b, j<=i} A_ij
 * (|I_q| = block_size, or the short last block's length), added in place:
 * mass[b][h][q][kb] += r_qb  for kb <= q.
 *
 * q, k, v, o: as in wise_full_attn.
 * mass: fp32 [batch][heads][n_blocks][n_blocks], read-modify-written.  The
 *       caller zeroes it before the first discovery step; calling once per
 *       discovery step leaves the sum of r over those steps.  Entries with
 *       kb > q are never touched.  The mass reduction is fused into the
 *       attention kernel, which never stores the attention matrix: one pass
 *       over the keys while the per-(query, key block) partial sums fit in
 *       on-chip memory, else (long rows) a first pass over the keys for the
 *       row maxima and sums and a second that recomputes the scores.
 */
wise_status_t wise_full_attn_accum(const wise_attn_desc_t* desc, const void* q, const void* k,
                                   const void* v, void* o, float* mass, void* stream);

/*
 * The discovery step of wise_full_attn_accum (the same Eq. 2 output and the
 * same Section 5.1, Eq. (5) block mass, added into mass), with the
 * per-(query, key block) partial sums of Eq. (5) kept in a caller-owned
 * workspace in device memory instead of on chip.  For block sizes 32, 64
 * and 128 this runs the mass launch at the dense kernel's tile size and
 * occupancy in one pass over the keys at every sequence length, where
 * wise_full_attn_accum has to shrink its tiles or walk the keys twice as
 * rows grow (and always walks them twice at block 32).  For block size 16
 * the call is wise_full_attn_accum and the workspace is unused.
 *
 * q, k, v, o, mass: as in wise_full_attn_accum.
 * workspace: device memory of at least
 *       wise_full_attn_accum_workspace_bytes(desc) bytes, 16-byte aligned,
 *       not overlapping any other argument (may be NULL when that size is
 *       0).  Its contents on entry are ignored and on return unspecified:
 *       it is scratch, and calls that share it must not overlap in time.
 * workspace_bytes: its size; WISE_ERR_CAPACITY if it is too small.
 */
wise_status_t wise_full_attn_accum_ws(const wise_attn_desc_t* desc, const void* q, const void* k,
                                      const void* v, void* o, float* mass, void* workspace,
                                      int64_t workspace_bytes, void* stream);

/*
 * wise_full_attn_accum_ws without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  The per-(query, key
 * block) partials live in a fixed buffer of
 * wise_full_attn_accum_noalloc_max_bytes() bytes (64 MiB) that the library
 * holds in each GPU's memory for the life of the process; the call itself
 * allocates nothing.  Same kernels, arguments and results as
 * wise_full_attn_accum_ws (bitwise).
 *
 * Limit: wise_full_attn_accum_workspace_bytes(desc) must not exceed the
 * buffer (for example 32 heads x 4096 keys at block 64 need 32 MiB), else
 * WISE_ERR_CAPACITY with nothing launched.  Block size 16 needs no buffer
 * and runs wise_full_attn_accum.
 * Nothing in the buffer must start at zero: every partial is written before
 * it is read.  All calls on one GPU share its buffer, so two calls that
 * overlap in time on that GPU (on different streams, or from different host
 * threads without ordering) race on it; the caller orders them.  The first
 * call on a device looks up the buffer's device address (no allocation).
 */
wise_status_t wise_full_attn_accum_noalloc(const wise_attn_desc_t* desc, const void* q, const void* k,
                                           const void* v, void* o, float* mass, void* stream);

/* Size in bytes of the fixed buffer of wise_full_attn_accum_noalloc. */
int64_t wise_full_attn_accum_noalloc_max_bytes(void);

/* Workspace bytes wise_full_attn_accum_ws needs for this descriptor:
 * batch * heads * n_blocks^2 * block_size * 4 for block sizes 32, 64 and
 * 128, 0 for 16; -1 for an invalid descriptor. */
int64_t wise_full_attn_accum_workspace_bytes(const wise_attn_desc_t* desc);

/*
 * Working-set selection, Section 5.1, Eq. (6) (Appendix A.1, Eq. 12), once
 * after discovery.  For every row (b, h, q), with mbar_kb = mass[..][kb] /
 * n_steps for the admissible blocks kb = 0..q:
 *   1. rank blocks by mbar descending, ties by lower block index;
 *   2. k* = smallest k whose k leading masses sum to >= eta (float64 sums;
 *      all blocks if the total stays below eta);
 *   3. k  = min(k*, max_blocks) when max_blocks > 0;
 *   4. W  = the k leading blocks, plus the sink block 0 and the diagonal
 *      block q (these two do not count toward eta or the cap).
 * Output is a CSR over rows ("row offsets and active block indices", the
 * format of the paper's Appendix B sparse kernels), column indices
 * ascending within each row:
 *   row_ptr: int32 [n_rows + 1] (written; row_ptr[n_rows] = total nnz),
 *   col_idx: int32 [col_capacity] (the first row_ptr[n_rows] entries written),
 *   nnz:     optional (NULL to skip) int64 on the device, 8-byte aligned;
 *            receives the total entry count row_ptr[n_rows].  It is written
 *            on the stream like the rest: read it after synchronising.
 *
 * mass: fp32 [batch][heads][n_blocks][n_blocks] (read; entries kb > q ignored).
 * n_steps >= 1; eta in (0, 1] as a double (the comparisons are float64;
 * a float eta would move the threshold, e.g. 0.9f = 0.89999998).
 * max_blocks >= 0 (0 = no cap).
 * col_capacity must be >= wise_select_max_nnz(desc, max_blocks), else
 * WISE_ERR_CAPACITY is returned before any launch.  n_blocks <= 2048.
 */
wise_status_t wise_select_support(const wise_attn_desc_t* desc, const float* mass,
                                  int32_t n_steps, double eta, int32_t max_blocks,
                                  int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                  int64_t* nnz, void* stream);

/*
 * Selection variants (same output contract as wise_select_support, no cap):
 * the temporal-union working set of Section 5.1, Eq. (6) left-hand part and
 * Appendix B, Eq. (18), and the early-static controls of Appendix B,
 * Eq. (19)-(22).  They take single-step block masses r^(t) (each row sums to
 * 1; one zeroed mass buffer per step given to wise_full_attn_accum):
 *
 * step_mass: fp32 [n_mass][batch][heads][n_blocks][n_blocks], read; entries
 *            kb > q ignored.
 * kind WISE_SELECT_UNION:        n_mass >= 1 steps (the paper: the last four
 *     discovery steps); W = union over the steps of each step's own
 *     eta-support (Eq. 6 right: smallest highest-mass set reaching eta, ties
 *     to the lower block index).
 * kind WISE_SELECT_STATIC:       n_mass == 1, the first step; W = its
 *     eta-support (Static-95 with eta = 0.95, Eq. 19).
 * kind WISE_SELECT_MASS_MATCHED: n_mass >= 2; step 0 is the first step,
 *     steps 1.. the union window.  m = float64 sum of the first step's masses
 *     over the union; W = smallest first-step-ranked set reaching m
 *     (Eq. 20-21).
 * kind WISE_SELECT_SIZE_MATCHED: n_mass >= 2 as above; W = the |union| blocks
 *     of highest first-step mass (Eq. 22).
 * Every result then gets the sink block 0 and the diagonal block q.
 * eta in (0, 1]; col_capacity >= wise_select_max_nnz(desc, 0), else
 * WISE_ERR_CAPACITY before any launch.  Invalid kind / n_mass ->
 * WISE_ERR_INVALID_ARG.  nnz: as in wise_select_support (optional).
 */
typedef enum {
  WISE_SELECT_UNION = 1,
  WISE_SELECT_STATIC = 2,
  WISE_SELECT_MASS_MATCHED = 3,
  WISE_SELECT_SIZE_MATCHED = 4
} wise_select_kind_t;

wise_status_t wise_select_variant(const wise_attn_desc_t* desc, int32_t kind, const float* step_mass,
                                  int32_t n_mass, double eta, int32_t* row_ptr, int32_t* col_idx,
                                  int64_t col_capacity, int64_t* nnz, void* stream);

/*
 * Reuse step, Section 5.2, Eq. (7)-(8): O = softmax(Q K^T * scale + M + R) V,
 * where R_ij = 0 if key block b(j) is listed in the CSR row of query block
 * q(i) and -inf otherwise.  Only the listed key blocks are read and computed;
 * the causal mask applies inside the diagonal block.
 *
 * q, k, v, o: as in wise_full_attn.
 * row_ptr, col_idx: CSR over rows (as written by wise_select_support).  A
 *          row's entries are read as a set of key blocks: entries outside
 *          [0, q] are ignored, repeated entries count once and their order
 *          does not matter.  A query with no admissible key in its row's
 *          blocks gets a zero output.  The caller keeps every row_ptr
 *          value within [0, length of col_idx]; row r reads col_idx
 *          [row_ptr[r], row_ptr[r+1]).  A negative start is read as 0 and
 *          a row whose end lies below its start as empty, so malformed
 *          pointers cannot make the kernel read before col_idx; a value
 *          past its end can, and is the caller's error.
 */
wise_status_t wise_sparse_attn(const wise_attn_desc_t* desc, const void* q, const void* k,
                               const void* v, const int32_t* row_ptr, const int32_t* col_idx,
                               void* o, void* stream);

/*
 * Diagnostics of the frozen working set (Section 7, "Evaluation metrics";
 * Appendix C.2, Eq. 23-25).  CSR rows are read as sets, as in
 * wise_sparse_attn, with the same reading of malformed pointers (a negative
 * start as 0, an end below the start as an empty row).
 *
 * wise_support_mass: retained[r] = sum over kb in row r's support of
 *   mass[r][kb] (float64 sum in block order, stored fp32).  With the block
 *   masses of an unrestricted step t > td (wise_full_attn_accum into a zeroed
 *   buffer), this is the retained future attention mass of the row; the
 *   method's figure is its mean over rows and late steps.
 *   mass: fp32 [batch][heads][n_blocks][n_blocks] (read);
 *   retained: fp32 [batch * heads * n_blocks] (written).
 *
 * wise_support_overlap: n_inter[r] = |A_r intersect B_r|, n_union[r] =
 *   |A_r union B_r| for two CSRs A and B over the same rows.  The Jaccard
 *   similarity of Eq. (24)/(25) for one batch element is the sum of n_inter
 *   over its rows divided by the sum of n_union.
 *   n_inter, n_union: int32 [batch * heads * n_blocks] (written).
 */
wise_status_t wise_support_mass(const wise_attn_desc_t* desc, const float* mass, const int32_t* row_ptr,
                                const int32_t* col_idx, float* retained, void* stream);
wise_status_t wise_support_overlap(const wise_attn_desc_t* desc, const int32_t* row_ptr_a,
                                   const int32_t* col_idx_a, const int32_t* row_ptr_b, const int32_t* col_idx_b,
                                   int32_t* n_inter, int32_t* n_union, void* stream);

/* Upper bound of the CSR size wise_select_support can write:
 * sum over rows of min(q + 1, max_blocks + 2) (q + 1 when max_blocks == 0).
 * Returns -1 for an invalid descriptor. */
int64_t wise_select_max_nnz(const wise_attn_desc_t* desc, int32_t max_blocks);

/* Static, human-readable name of a status code. */
const char* wise_status_string(wise_status_t status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* wise_last_error(void);

/* WISE_ABI_VERSION of the built library. */
int32_t wise_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* WISE_H */
