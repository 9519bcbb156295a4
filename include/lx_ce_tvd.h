/*
 * lx_ce_tvd.h -- C ABI of the fused cross-entropy + total-variation-distance
 * (CE + TVD) distillation loss for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one the "Liger-Kernel PR #1384 analysis" page
 * (blog.secrett2633.cloud; the analysis of the merged Liger-Kernel pull
 * request "add fused CE + TV distance kernel") describes.  Per token row r of
 * student logits z (length V), teacher logits u and target t = target[r]:
 *
 *   lse_s = log sum_v exp(z_v),  lse_t = log sum_v exp(u_v)
 *                                          (page section "Forward Pass", step 1)
 *   p_v = exp(z_v - lse_s),  q_v = exp(u_v - lse_t)
 *   tvd   = 0.5 * sum_v |p_v - q_v|
 *   sigma = sum_v p_v * sign(p_v - q_v),  sign(0) = 0
 *                                          (page section "Forward Pass", step 2)
 *   ce    = lse_s - z_t                    (same section, the stored outputs)
 *   d(g_ce*ce + g_tvd*tvd)/dz_v =
 *       g_ce * (p_v - [v == t]) + g_tvd * 0.5 * p_v * (sign(p_v - q_v) - sigma)
 *                                          (page section "Backward Pass")
 *
 * Only the O(BT) per-row state (ce, tvd, lse_s, lse_t, sigma) passes from the
 * forward to the backward (page section "Core idea"); no (BT, V) temporary is
 * ever allocated.
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 * - Logits are row-major, shape (BT, V), element type `dt`; student and
 *   teacher share the type.  Row r starts at element r * V (the `_ex` entry
 *   points take a row stride per tensor instead: row r at element r * ld).
 * - All array pointers are DEVICE pointers owned by the caller.  No entry
 *   point allocates device or host memory, and the results of a call depend
 *   on its arguments only; entry points that need scratch memory take a
 *   caller-owned workspace.  The one exception is
 *   lx_ce_tvd_forward_backward_noalloc, whose scratch is a fixed device array
 *   inside the library (its address looked up once per device and kept in a
 *   host table): calls of that entry point that overlap on one device race.
 *   Every other entry point is safe to call from several host threads (on
 *   different or on the same stream).
 * - `stream` is a hipStream_t passed as an opaque pointer; NULL selects the
 *   null stream.  Every call is asynchronous on that stream: the call returns
 *   after enqueueing its kernels.
 * - Arguments are validated on the host before anything is enqueued; a failed
 *   validation returns a status other than LX_OK and enqueues nothing.
 *   LX_ERR_HIP means a kernel launch was rejected by the HIP runtime; call
 *   lx_last_hip_error() for the hipError_t code.
 * - BT == 0 is a no-op returning LX_OK (pointers are not inspected).
 * - Requirements: BT >= 0, 1 <= V <= 2^31 - 1, BT * V * element size fits in
 *   int64; logits pointers aligned to the element size, float arrays to 4
 *   bytes, target to 8 bytes.  Fast 16-byte vector paths are taken when the
 *   logits (and gradient) pointers share their address modulo 16; any other
 *   element-aligned layout runs a slower element-wise path of the same kernels.
 * - Target handling: a row whose target equals ignore_index is IGNORED (tested
 *   first, so an ignore_index inside [0, V) ignores that class): its logits
 *   are never read, its five forward outputs are +0.0 and its gradient row is
 *   +0.0.  A target outside [0, V) that is not ignore_index is a caller error
 *   the device cannot report synchronously: that row's ce and its whole
 *   gradient row are written as NaN.
 * - Logits must be finite.  -inf entries are allowed in a row that has at
 *   least one finite entry (they get probability 0); NaN or +inf entries give
 *   unspecified (NaN) results for their row.
 * - Results are deterministic: the same inputs give bit-identical outputs on
 *   every call.  Identical student and teacher rows give tvd == sigma == 0
 *   exactly and a total-variation gradient of exactly 0.
 */
#ifndef LX_CE_TVD_H
#define LX_CE_TVD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LX_CE_TVD_ABI_VERSION 7

typedef enum lx_status {
  LX_OK = 0,
  LX_ERR_INVALID_ARG = 1,       /* NULL / misaligned pointer, bad size */
  LX_ERR_UNSUPPORTED_DTYPE = 2, /* dt is not LX_F32, LX_BF16 or LX_F16 */
  LX_ERR_ALIAS = 3,             /* an output overlaps an input or another output */
  LX_ERR_WORKSPACE = 4,         /* workspace NULL or smaller than required */
  LX_ERR_HIP = 5,               /* the HIP runtime rejected a launch or a symbol lookup */
  LX_ERR_TOO_LARGE = 6          /* the shape needs more scratch than the static buffer of
                                   lx_ce_tvd_forward_backward_noalloc holds */
} lx_status;

typedef enum lx_dtype {
  LX_F32 = 0,  /* IEEE binary32 logits (and gradient) */
  LX_BF16 = 1, /* bfloat16 logits (and gradient); gradients rounded to nearest-even */
  LX_F16 = 2   /* IEEE binary16 logits (and gradient); gradients rounded to nearest-even
                  (values below the binary16 range become subnormal or zero) */
} lx_dtype;

/* Human-readable name of a status code (static storage, never NULL). */
const char* lx_status_string(lx_status s);

/* LX_CE_TVD_ABI_VERSION of the built library. */
int lx_abi_version(void);

/* hipError_t code (as int) of the last LX_ERR_HIP returned on this host thread; 0 if none. */
int lx_last_hip_error(void);

/*
 * Bytes of device workspace lx_ce_tvd_forward needs for this shape
 * (0 when the shape runs without workspace).  has_teacher: 0 = CE-only mode.
 * Returns 0 for shapes that the forward would reject.
 */
size_t lx_ce_tvd_workspace_bytes(int64_t BT, int64_t V, lx_dtype dt, int has_teacher);

/*
 * Forward pass ("Forward Pass" section of the PR #1384 analysis page).
 *
 * Inputs : student (BT, V) dt; teacher (BT, V) dt or NULL for CE-only mode;
 *          target (BT) int64; ignore_index.
 * Outputs: ce, lse_s: float[BT], required.
 *          tvd, lse_t, sigma: float[BT], required with a teacher; in CE-only
 *          mode they may be NULL and are never written.
 *          All outputs hold fp32 values computed with fp32 accumulation.
 * Workspace: device buffer of at least lx_ce_tvd_workspace_bytes(BT, V, dt,
 *          teacher != NULL) bytes, 256-byte aligned, contents ignored and
 *          clobbered; may be NULL when that size is 0.  It must not be used by
 *          another call that overlaps this one on the device.
 * Errors : LX_ERR_INVALID_ARG, LX_ERR_UNSUPPORTED_DTYPE, LX_ERR_ALIAS (any
 *          output overlapping an input or another output), LX_ERR_WORKSPACE,
 *          LX_ERR_HIP.
 */
lx_status lx_ce_tvd_forward(const void* student, const void* teacher, const int64_t* target,
                            int64_t BT, int64_t V, int64_t ignore_index,
                            float* ce, float* tvd, float* lse_s, float* lse_t, float* sigma,
                            lx_dtype dt, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass ("Backward Pass" section of the PR #1384 analysis page):
 *
 *   grad[r, v] = k * ( g_ce * (p_v - [v == t]) + g_tvd * 0.5 * p_v * (s_v - sigma[r]) )
 *
 * with p, q recomputed from the logits and the forward's lse_s / lse_t,
 * s_v = sign(p_v - q_v) (0 at ties), and k = *g_scale when g_scale is not
 * NULL (a device float, e.g. the inv_n_valid written by
 * lx_ce_tvd_reduce_mean), else 1.  Ignored rows are written +0.0.
 *
 * Inputs : student, teacher (NULL = CE-only: the g_tvd term is absent and
 *          lse_t / sigma may be NULL), target, lse_s, lse_t, sigma as written
 *          by lx_ce_tvd_forward on the same logits; g_ce, g_tvd host scalars.
 * Output : grad (BT, V) dt.  grad may EQUAL student (in place: each element is
 *          read before it is overwritten); any other overlap with an input is
 *          LX_ERR_ALIAS.  bf16 gradients are rounded to nearest-even.
 */
lx_status lx_ce_tvd_backward(void* grad, const void* student, const void* teacher,
                             const int64_t* target, int64_t BT, int64_t V, int64_t ignore_index,
                             const float* lse_s, const float* lse_t, const float* sigma,
                             float g_ce, float g_tvd, const float* g_scale,
                             lx_dtype dt, void* stream);

/*
 * Bytes of device workspace lx_ce_tvd_forward_backward needs for this shape
 * (0 when the shape runs without workspace); otherwise as
 * lx_ce_tvd_workspace_bytes.
 */
size_t lx_ce_tvd_forward_backward_workspace_bytes(int64_t BT, int64_t V, lx_dtype dt, int has_teacher);

/*
 * Forward and backward in one call, for a loss whose upstream gradients are
 * known before the forward runs (the loss is the last node of the graph, and a
 * mean over valid rows needs only their count, see lx_ce_tvd_count_valid).
 * Computes exactly what lx_ce_tvd_forward followed by lx_ce_tvd_backward
 * computes, combining the "Forward Pass" and "Backward Pass" sections of the
 * PR #1384 analysis page into one pass over the logits where the shape allows:
 * for bf16 or binary16 logits (with or without a teacher), V % 8 == 0, V >= 2048 and
 * student, teacher and grad 16-byte aligned, each row is read from HBM once and
 * its gradient written once; any other shape runs the two passes back to back
 * on `stream`.
 *
 * Inputs : as lx_ce_tvd_forward, plus g_ce, g_tvd and g_scale as
 *          lx_ce_tvd_backward (g_scale: optional device float, e.g. the
 *          inv_n_valid written by lx_ce_tvd_count_valid on the same stream).
 * Outputs: ce, tvd, lse_s, lse_t, sigma as lx_ce_tvd_forward; grad (BT, V) dt
 *          as lx_ce_tvd_backward.  grad may EQUAL student (in place: every
 *          logit of a row is read before any gradient of that row is stored);
 *          any other overlap with an input, an output or the workspace is
 *          LX_ERR_ALIAS.  The forward outputs are bit-identical to those of
 *          lx_ce_tvd_forward only when both take the same path; both meet the
 *          same tolerances against the definition.
 * Workspace: at least lx_ce_tvd_forward_backward_workspace_bytes(...) bytes,
 *          256-byte aligned, contents ignored and clobbered.
 * Errors : as lx_ce_tvd_forward and lx_ce_tvd_backward.
 */
lx_status lx_ce_tvd_forward_backward(const void* student, const void* teacher, const int64_t* target,
                                     int64_t BT, int64_t V, int64_t ignore_index,
                                     float* ce, float* tvd, float* lse_s, float* lse_t, float* sigma,
                                     void* grad, float g_ce, float g_tvd, const float* g_scale,
                                     lx_dtype dt, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free variant of lx_ce_tvd_forward_backward, for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments,
 * results and errors as lx_ce_tvd_forward_backward without the workspace: the
 * scratch memory lives in a static device array of the library,
 * LX_NOALLOC_SCRATCH_BYTES per device, held by each device the library runs on
 * until the process ends.  Its device address is looked up once per device, on
 * the first call with that device current (the stream's device), so the first
 * call can return LX_ERR_HIP if the lookup fails.  The call allocates nothing.
 * Shapes whose scratch (lx_ce_tvd_forward_backward_workspace_bytes) exceeds
 * LX_NOALLOC_SCRATCH_BYTES return LX_ERR_TOO_LARGE (e.g. more than about 80000
 * rows of 151936 bf16 logits with a teacher) and enqueue nothing.  Every call on
 * a device shares that device's array (each call re-initialises what it needs),
 * so calls that overlap on one device, on different streams or from different
 * host threads, race: serialise them.
 */
#define LX_NOALLOC_SCRATCH_BYTES (8u << 20)
lx_status lx_ce_tvd_forward_backward_noalloc(const void* student, const void* teacher, const int64_t* target,
                                             int64_t BT, int64_t V, int64_t ignore_index,
                                             float* ce, float* tvd, float* lse_s, float* lse_t, float* sigma,
                                             void* grad, float g_ce, float g_tvd, const float* g_scale,
                                             lx_dtype dt, void* stream);

/*
 * ---------------------------------------------------------------------------
 * Strided rows and per-row upstream gradients.  The page shows contiguous
 * (BT, V) logits and two scalar upstream gradients, grad_ce and grad_tvd
 * (section "Backward Pass"), and is silent on row strides and on unreduced
 * losses.  These entry points extend the three above, with the same
 * arithmetic per row:
 *
 * - ld_student, ld_teacher, ld_grad: elements between the starts of
 *   consecutive rows of each tensor, >= V (V for a contiguous array), e.g.
 *   the logits of a vocabulary padded to a wider lm_head output.  Each array
 *   spans (BT - 1) * ld + V elements for the overlap checks; an in-place
 *   gradient (grad == student) needs ld_grad == ld_student.  The one-pass and
 *   read-once kernels need every row on a 16-byte boundary (base and
 *   ld * element size multiples of 16); other strides run the two-pass
 *   kernels, with 16-byte vectors when all rows of the tensors share their
 *   address modulo 16.
 * - grad_ce_rows, grad_tvd_rows: optional device float[BT] per-row factors of
 *   g_ce and g_tvd (NULL = 1), the upstream gradient of an unreduced
 *   (per-row) loss: row r uses g_ce * grad_ce_rows[r] and
 *   g_tvd * grad_tvd_rows[r], both times *g_scale when given.  Inputs: they
 *   must not overlap the gradient or an output.
 *
 * With ld_* = V and NULL row factors each computes exactly what the
 * entry point without the suffix computes.  Errors: as those, plus
 * LX_ERR_INVALID_ARG for a stride below V or one whose last row end is not
 * addressable.
 */
lx_status lx_ce_tvd_forward_ex(const void* student, int64_t ld_student, const void* teacher, int64_t ld_teacher,
                               const int64_t* target, int64_t BT, int64_t V, int64_t ignore_index,
                               float* ce, float* tvd, float* lse_s, float* lse_t, float* sigma,
                               lx_dtype dt, void* workspace, size_t workspace_bytes, void* stream);

lx_status lx_ce_tvd_backward_ex(void* grad, int64_t ld_grad, const void* student, int64_t ld_student,
                                const void* teacher, int64_t ld_teacher, const int64_t* target,
                                int64_t BT, int64_t V, int64_t ignore_index,
                                const float* lse_s, const float* lse_t, const float* sigma,
                                float g_ce, float g_tvd, const float* grad_ce_rows, const float* grad_tvd_rows,
                                const float* g_scale, lx_dtype dt, void* stream);

/* Workspace: lx_ce_tvd_forward_backward_workspace_bytes (strides do not change it). */
lx_status lx_ce_tvd_forward_backward_ex(const void* student, int64_t ld_student, const void* teacher,
                                        int64_t ld_teacher, const int64_t* target,
                                        int64_t BT, int64_t V, int64_t ignore_index,
                                        float* ce, float* tvd, float* lse_s, float* lse_t, float* sigma,
                                        void* grad, int64_t ld_grad, float g_ce, float g_tvd,
                                        const float* grad_ce_rows, const float* grad_tvd_rows,
                                        const float* g_scale, lx_dtype dt,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Count of the rows whose target is not ignore_index, the only quantity a
 * mean-reduced loss needs before its backward.
 *
 * Inputs : target int64[BT] (may be NULL when BT == 0).
 * Outputs: n_valid int64[1] or NULL; inv_n_valid float[1] or NULL, = 1 / n_valid
 *          (0 when n_valid == 0); at least one of them must be given.
 * Errors : LX_ERR_INVALID_ARG (BT < 0, no output, misaligned pointer),
 *          LX_ERR_ALIAS (outputs overlapping target or each other), LX_ERR_HIP.
 */
lx_status lx_ce_tvd_count_valid(const int64_t* target, int64_t BT, int64_t ignore_index,
                                int64_t* n_valid, float* inv_n_valid, void* stream);

/*
 * Mean reduction over the rows whose target is not ignore_index.
 *
 * Inputs : ce float[BT]; tvd float[BT] or NULL (CE-only); target int64[BT].
 * Outputs: mean_out float[2] = { sum ce / n_valid, sum tvd / n_valid }
 *          (mean_out[1] is written only when tvd is not NULL; 0/0 = NaN when
 *          every row is ignored); n_valid int64[1] or NULL; inv_n_valid
 *          float[1] or NULL, = 1 / n_valid (0 when n_valid == 0), the factor
 *          a mean-reduced loss passes to lx_ce_tvd_backward as g_scale.
 *          Sums are accumulated in float64 in a fixed order (deterministic).
 */
lx_status lx_ce_tvd_reduce_mean(const float* ce, const float* tvd, const int64_t* target,
                                int64_t BT, int64_t ignore_index,
                                float* mean_out, int64_t* n_valid, float* inv_n_valid,
                                void* stream);

/*
 * ---------------------------------------------------------------------------
 * Vocabulary-parallel pieces (a sharded lm_head): each device holds a column
 * shard, columns [v0, v0 + V_shard) of every row of V = sum of the shard
 * widths, as a contiguous (BT, V_shard) array.  The two steps of the page's
 * "Forward Pass" section each become a per-shard partial, an exchange of the
 * partials between devices (which the caller runs, e.g. an all-gather over
 * RCCL), and a merge:
 *
 *   lx_ce_tvd_vp_stats        -> all-gather -> lx_ce_tvd_vp_merge_stats -> ce, lse_s, lse_t
 *   lx_ce_tvd_vp_tv (teacher) -> all-gather -> lx_ce_tvd_vp_merge_tv    -> tvd, sigma
 *
 * and the backward of a shard, lx_ce_tvd_backward_shard, needs no exchange.
 * The merges read the gathered partials as [n_shards][BT][...] in shard order
 * and combine them in that order, so the results do not depend on the order of
 * the exchange; they meet the same tolerances as lx_ce_tvd_forward on the
 * whole rows (page sections "Forward Pass" and "Backward Pass").
 */

/* floats per row of the partials */
#define LX_VP_STATS_FLOATS(has_teacher) ((has_teacher) ? 5 : 3)
#define LX_VP_TV_FLOATS 2

/*
 * Per-shard step 1: for each row, a (m, s) pair of the student (and teacher)
 * with s = sum of exp(x - m) over the shard, so that m + log(s) is the
 * shard's log-sum-exp (m is at most the shard's maximum, or -1e30 when that
 * is lower), and the student's target logit when the
 * target column lies in the shard (else +0).
 *
 * Inputs : student, teacher (NULL = CE-only) (BT, V_shard) dt; target int64[BT]
 *          indexing the WHOLE row; v0 >= 0 the shard's first column.
 * Output : stats float[BT][LX_VP_STATS_FLOATS(teacher != NULL)] =
 *          {m_s, s_s, m_t, s_t, z_t part} (CE-only: {m_s, s_s, z_t part});
 *          ignored rows are all +0.0.  Must not overlap an input.
 * Errors : LX_ERR_INVALID_ARG, LX_ERR_UNSUPPORTED_DTYPE, LX_ERR_ALIAS, LX_ERR_HIP.
 */
lx_status lx_ce_tvd_vp_stats(const void* student, const void* teacher, const int64_t* target,
                             int64_t BT, int64_t V_shard, int64_t v0, int64_t ignore_index,
                             lx_dtype dt, float* stats, void* stream);

/*
 * Merge of the gathered step-1 partials of n_shards shards, in shard order:
 * lse = M + log(sum_n s_n * exp(m_n - M)), ce = lse_s - sum_n (z_t part)_n.
 *
 * Inputs : stats float[n_shards][BT][LX_VP_STATS_FLOATS(has_teacher)];
 *          target int64[BT]; V the whole vocabulary (a target outside [0, V)
 *          that is not ignore_index gives ce = NaN).
 * Outputs: ce, lse_s float[BT]; lse_t float[BT] with a teacher (may be NULL
 *          without).  Ignored rows +0.0.  Outputs must not overlap the inputs
 *          or each other.
 */
lx_status lx_ce_tvd_vp_merge_stats(const float* stats, int64_t n_shards, const int64_t* target,
                                   int64_t BT, int64_t V, int64_t ignore_index, int has_teacher,
                                   float* ce, float* lse_s, float* lse_t, void* stream);

/*
 * Per-shard step 2: for each row, the shard's sum |p - q| and sum p *
 * sign(p - q), p and q formed from the whole-row lse_s and lse_t (as merged).
 *
 * Inputs : student, teacher (BT, V_shard) dt (teacher required); target;
 *          lse_s, lse_t float[BT].
 * Output : tv float[BT][LX_VP_TV_FLOATS]; ignored rows +0.0.  Must not overlap
 *          an input.
 */
lx_status lx_ce_tvd_vp_tv(const void* student, const void* teacher, const int64_t* target,
                          int64_t BT, int64_t V_shard, int64_t ignore_index,
                          const float* lse_s, const float* lse_t, lx_dtype dt, float* tv, void* stream);

/*
 * Merge of the gathered step-2 partials, added in shard order:
 * tvd = 0.5 * sum_n A_n, sigma = sum_n S_n.
 *
 * Inputs : tv float[n_shards][BT][LX_VP_TV_FLOATS]; target int64[BT].
 * Outputs: tvd, sigma float[BT]; ignored rows +0.0; no overlaps.
 */
lx_status lx_ce_tvd_vp_merge_tv(const float* tv, int64_t n_shards, const int64_t* target,
                                int64_t BT, int64_t ignore_index, float* tvd, float* sigma, void* stream);

/*
 * Backward of one column shard: lx_ce_tvd_backward restricted to columns
 * [v0, v0 + V_shard) of rows of V columns, with the whole-row lse_s, lse_t
 * and sigma (as merged).  Only the shard holding the target column subtracts
 * g_ce; a target outside [0, V) that is not ignore_index poisons the row (NaN)
 * in every shard.  Requires 0 <= v0 <= V - V_shard.  grad may EQUAL student.
 */
lx_status lx_ce_tvd_backward_shard(void* grad, const void* student, const void* teacher,
                                   const int64_t* target, int64_t BT, int64_t V_shard, int64_t v0,
                                   int64_t V, int64_t ignore_index,
                                   const float* lse_s, const float* lse_t, const float* sigma,
                                   float g_ce, float g_tvd, const float* g_scale,
                                   lx_dtype dt, void* stream);

/*
 * ---------------------------------------------------------------------------
 * The lm_head product and the loss together.  The aibars.net Liger-Kernel
 * project page lists a fused linear cross-entropy (the lm_head projection and
 * the loss in one operation, so the full logits are never kept); the PR #1384
 * analysis page's CE + TVD loss ("Forward Pass", "Backward Pass") runs here on
 * the logits of student and teacher lm_heads:
 *
 *   z = x_s w_s^T,  u = x_t w_t^T                       (logits, never stored)
 *   ce, tvd, lse_s, lse_t, sigma per row               (as lx_ce_tvd_forward)
 *   G = k * (g_ce * d ce/dz + g_tvd * d tvd/dz)        (as lx_ce_tvd_backward)
 *   grad_x_s = G w_s,  grad_w_s = G^T x_s
 *
 * The products run on the matrix cores (this library's own MFMA kernels:
 * bf16 operands, fp32 accumulation).  Logit tiles are reduced in registers
 * as they are computed: a first pass over all tiles gives each row's
 * log-sum-exps (a per-row dot product gives its target logit), a second (per
 * chunk of chunk_rows rows)
 * recomputes the same tiles, bit for bit, for the total variation and keeps,
 * for the gradient, 2^15 * p as binary16 with the sign of p - q and a tie bit
 * per logit; G is formed from them in bf16 (rounded to nearest even; relative
 * precision 2^-8 + 2^-10, the binary16 p included) and enters the two gradient
 * products.  Nothing is allocated: every byte of scratch is in the caller's
 * workspace.  A target outside [0, V) that is not ignore_index makes its row
 * of G NaN: ce and grad_x_s of that row are NaN, and since grad_w_s sums over
 * the rows, so is every element of grad_w_s.
 */

/*
 * Matrix product on the matrix cores, the contraction step of the path above:
 *
 *   C[m][n] = (accumulate ? C[m][n] : 0) + sum_k A(m, k) * B(n, k)
 *
 * Inputs : A, B bf16 (device), C fp32 (device, row stride ldc >= N).
 *          A(m, k) = A[m * lda + k] when a_k_contiguous, else A[k * lda + m];
 *          B(n, k) = B[n * ldb + k] when b_k_contiguous, else B[k * ldb + n].
 *          The contiguous dimension of A and of B (K, or M for A and N for B)
 *          must be a multiple of 8, lda and ldb multiples of 8 no smaller than
 *          that dimension and at most 2^22, A and B 16-byte aligned, C 4-byte aligned;
 *          1 <= M, N, K <= 2^31 - 1.  C must not overlap A or B.
 * One launch of the library's MFMA kernel (256 x 256 tiles, fp32
 * accumulation); it allocates nothing and keeps no state.  Operands
 * contiguous along M or N are read with the LDS transpose read, at about the
 * speed of K-contiguous ones (the lm_head path uses both).
 * Errors : LX_ERR_INVALID_ARG, LX_ERR_ALIAS, LX_ERR_HIP.
 */
lx_status lx_gemm_bf16(const void* A, int64_t lda, int a_k_contiguous, const void* B, int64_t ldb,
                       int b_k_contiguous, float* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                       int accumulate, void* stream);

/*
 * Bytes of workspace lx_ce_tvd_linear_forward_backward needs (0 when BT == 0 or
 * for arguments it would reject): per-tile partials of every row (20 B per
 * 256 logits with a teacher, 12 without) and of the chunk's rows (8 B per
 * 128 logits), per chunk of rows 2 bytes of binary16 p plus a tie bit per
 * logit (G is formed in place), and for a chunk too short to fill the GPU
 * the split-K partials of its grad_x (at most 8 * chunk_rows * H_s floats).
 * No logit is stored and no operand is copied: at BT = chunk_rows = 8192,
 * V = 151936 that is 2.82 GB.
 */
size_t lx_ce_tvd_linear_workspace_bytes(int64_t BT, int64_t V, int64_t H_s, int has_teacher, int64_t chunk_rows);

/*
 * Inputs : x_s bf16 (BT, H_s) and w_s bf16 (V, H_s), row-major; x_t bf16
 *          (BT, H_t) and w_t bf16 (V, H_t), or both NULL for CE-only mode;
 *          target int64[BT]; H_s, H_t and V multiples of 8, at most 2^22;
 *          all four arrays 16-byte aligned.
 * Outputs: ce, lse_s float[BT]; tvd, lse_t, sigma float[BT] with a teacher
 *          (may be NULL without); grad_x_s float (BT, H_s) and grad_w_s float
 *          (V, H_s), each optional (NULL: not computed), both OVERWRITTEN.
 *          g_ce, g_tvd, g_scale as lx_ce_tvd_backward.  No output may overlap
 *          an input, another output or the workspace.
 * Workspace: at least lx_ce_tvd_linear_workspace_bytes(BT, V, H_s, teacher !=
 *          NULL, chunk_rows) bytes, 256-byte aligned, contents ignored and
 *          clobbered.
 * Errors : LX_ERR_INVALID_ARG (shapes, alignment, chunk_rows < 1),
 *          LX_ERR_ALIAS, LX_ERR_WORKSPACE, LX_ERR_HIP.
 */
lx_status lx_ce_tvd_linear_forward_backward(const void* x_s, const void* w_s, int64_t H_s,
                                            const void* x_t, const void* w_t, int64_t H_t,
                                            const int64_t* target, int64_t BT, int64_t V, int64_t ignore_index,
                                            float* ce, float* tvd, float* lse_s, float* lse_t, float* sigma,
                                            float* grad_x_s, float* grad_w_s,
                                            float g_ce, float g_tvd, const float* g_scale,
                                            int64_t chunk_rows, void* workspace, size_t workspace_bytes,
                                            void* stream);

/*
 * ---------------------------------------------------------------------------
 * Reference streams: the practical HBM ceilings the loss kernels are measured
 * against (not part of the loss).  They move bytes the way the loss kernels
 * do: 16-byte buffer loads and stores with the streamed-once cache policy.
 *
 * lx_stream_read reads `bytes` bytes of src once (the forward's pattern); it
 * may write one uint32 to sink (only to keep the reads alive).
 * lx_stream_read2_write reads a and b and writes out = a XOR b, `bytes` bytes
 * each (the backward's and the one pass's pattern: two tensors in, one out).
 *
 * Inputs : device buffers, 16-byte aligned (sink 4-byte aligned); bytes a
 *          multiple of 16, at most 2^40; 0 is a no-op.
 * Errors : LX_ERR_INVALID_ARG, LX_ERR_ALIAS (out overlapping a or b, sink
 *          overlapping src), LX_ERR_HIP.
 */
lx_status lx_stream_read(const void* src, int64_t bytes, unsigned* sink, void* stream);
lx_status lx_stream_read2_write(const void* a, const void* b, void* out, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LX_CE_TVD_H */
