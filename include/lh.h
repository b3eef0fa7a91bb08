/*
 * lh.h — C ABI of the Lighthouse Attention layer for one MI355X (gfx950) GPU.
 *
 * The layer (aitrends.kr "Lighthouse Attention" summary, sections 방법론 and
 * 기술 상세; techllm.github.io Lighthouse review, section 어떻게 동작하나) runs
 * four steps around a dense attention:
 *   1. pyramid pool: Q, K and V are average-pooled by the same factor p into
 *      levels l = 0..L-1 (level l averages windows of p^l tokens);
 *   2. score and top-K: every token gets a parameter-free score from the l2
 *      norms of its query and key rows; coarser levels take the max of their
 *      children; a stratified, non-differentiable top-K picks k parents at each
 *      level l = 1..L-1;
 *   3. gathered-sequence attention: the whole top level plus the p children of
 *      every selected parent form one causally ordered sub-sequence of length
 *      S = N/p^(L-1) + (L-1)*p*k (techllm review, section 핵심 수식), run
 *      through dense causal softmax attention with scale 1/sqrt(d);
 *   4. scatter-back: every sub-sequence output is added to the tokens of its
 *      causal-safe shifted range R(l, i).
 * The backward holds the selected indices fixed and sends gradients through
 * scatter-back, the attention, the gather and the pooling to Q, K and V.
 *
 * Readings taken where the pages leave a step open (all are fixed behaviour of
 * this library):
 *   - score s_j = sqrt(||q_j||^2) + sqrt(||k_j||^2) in fp32; ||x||^2 of a row
 *     of d values: partial j (j < d/8) is 8 fused multiply-adds over elements
 *     8j..8j+7 in ascending order from +0, then for off = d/16 .. 1 every
 *     partial becomes a_j + a_(j xor off), and the norm is a_0; sqrt is the
 *     correctly rounded fp32 square root;
 *   - stratified top-K: a level of n entries is split into max(1, n/2048)
 *     strata of contiguous entries; stratum c keeps floor(k/C) + [c < k mod C]
 *     entries with the largest score, ties to the lowest index;
 *   - causal order: by the last token an entry covers, coarser entry first
 *     on equal last tokens;
 *   - R(l, i) = tokens (i+1)p^l - 1 .. (i+2)p^l - 2, clipped at N; outputs
 *     that fall in several ranges are summed in fp32, in a fixed order: the
 *     levels a kernel tile shares (the coarse ones) in ascending l first, then
 *     the finer levels from the coarsest of them down to level 0; a token in
 *     no range receives 0.
 *
 * Conventions for every entry point:
 *   - q, k, v, out, dout, dq, dk, dv are DEVICE pointers to [H][N][d]
 *     contiguous arrays (batch folded into H), owned by the caller, 16-byte
 *     aligned. Their element type is `dt` (bf16 or fp32); outputs are written
 *     in the same type.
 *   - ws is a caller-owned DEVICE workspace of at least lh_workspace_bytes()
 *     bytes, 256-byte aligned. The library never allocates device memory.
 *   - stream is a hipStream_t (NULL = the null stream). All work is queued on
 *     it asynchronously; no entry point synchronises or copies to the host.
 *   - Arguments are validated on the host before anything is queued; a bad
 *     argument returns LH_EINVAL / LH_EUNSUPPORTED / LH_EWORKSPACE and queues
 *     nothing. LH_EHIP means a launch failed; faults inside kernels surface at
 *     the caller's next synchronisation, as with any HIP call.
 *   - Results are deterministic and bitwise reproducible: no global-memory
 *     atomics anywhere on the layer's path (the top-K's digit histograms use
 *     LDS integer atomics, whose results do not depend on their order). Calls
 *     on distinct workspaces may run concurrently.
 *   - Inputs must be finite, and so must the logits: |q.k| / sqrt(d) below
 *     2^23 (the softmax keeps its fp32 logits to within one unit, so larger
 *     ones round by more than the probabilities' fp16 range allows).
 *
 * Range. Rows staged in fp16 for the attention (the gathered Q, K, V and
 * dO_sub) carry one power-of-two scale per head and tensor, chosen from the
 * head's largest values, and every result is scaled back exactly, so inputs
 * and gradients may lie far outside fp16's range (pooled rows and gradient
 * sums are fp32). The scales cover a head whose largest |q| and |k| element
 * is below 2^108 and whose value rows and dO_sub rows have norms below 2^64
 * (their squares are summed in fp32, as are those of the norm scores);
 * smaller magnitudes have no lower limit beyond fp16's subnormals, whose
 * absolute error is far below the stated tolerance.
 *
 * Precision. Scores are fp32 in the stated order (bit-exact by design).
 * Pooling sums in fp32. The attention runs on fp16 matrix cores with fp32
 * accumulation: the logits use an fp16 hi/lo pair for the query rows (about
 * 22 significant bits, so pooled rows are not truncated before the softmax)
 * and fp16 key rows, plus the key's lo part for fp32 inputs; with bf16 inputs
 * the query lo product and the dO_sub lo product of dP run on block-scaled
 * fp8 (e4m3) copies with one fixed power-of-two scale per tensor (the
 * per-head staging bounds their magnitudes); P, V, dS and the
 * fp16 hi/lo pair of dO_sub
 * feed the other products; row statistics, Delta = rowsum(dO_sub * O_sub) and
 * all sums are fp32. Outputs are rounded once to the input dtype.
 *
 * Supported shapes: d in {64, 128}; p in {2, 4, 8}; 1 <= L <= 8;
 * 1 <= N <= 2^27, N a multiple of p^(L-1); 1 <= H <= 65535; 0 <= k <= N/p^(L-1);
 * a level of more than 2048 entries must hold a multiple of 2048;
 * (L-1)*k <= 16384; S rounded up to 256, times d, at most 2^30; a
 * workspace (lh_workspace_bytes) of at most 2^46 bytes.
 */
#ifndef LH_H
#define LH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LH_OK = 0,
    LH_EINVAL = 1,       /* a shape or pointer argument is invalid */
    LH_EWORKSPACE = 2,   /* ws is NULL, misaligned or smaller than required */
    LH_EUNSUPPORTED = 3, /* valid for the method, outside what this build supports */
    LH_EHIP = 4          /* a HIP launch returned an error */
} lh_status;

typedef enum {
    LH_BF16 = 0,
    LH_F32 = 1
} lh_dtype;

/* The level-0 score, from nq = sqrt(||q_j||^2) and nk = sqrt(||k_j||^2) (both
 * in the order and rounding stated above), combined in fp32. The pages rank
 * entries by parameter-free query/key l2 norms of more than one kind
 * (aitrends summary, 핵심 기여; techllm review, 한계와 주의할 점: the norm
 * scorer's retrieval differs from the dense baseline's). */
typedef enum {
    LH_SCORE_SUM = 0,     /* nq + nk (lh_forward's score) */
    LH_SCORE_PRODUCT = 1, /* nq * nk */
    LH_SCORE_QUERY = 2,   /* nq */
    LH_SCORE_KEY = 3      /* nk */
} lh_scorer;

/* Human-readable name of a status code (static storage). */
const char *lh_strerror(lh_status s);

/* Validate a shape without touching the GPU. */
lh_status lh_check_shape(int64_t N, int H, int d, int L, int p, int k, lh_dtype dt);

/* Sub-sequence length S = N/p^(L-1) + (L-1)*p*k (techllm review, 핵심 수식);
 * -1 if the shape is invalid. */
int64_t lh_subseq_len(int64_t N, int L, int p, int k);

/* Bytes of device workspace lh_forward + lh_backward need for this shape;
 * 0 if the shape is invalid. The dS tiles the backward stores for its dQ
 * kernel (the causal half of S x S per head, fp16: H * T(T+1)/2 * 2 KiB,
 * T = S_pad/32) are planned only while they fit the dS tile budget (32 GiB
 * unless set otherwise); beyond it the dQ kernel recomputes the logits and
 * dP instead, and the workspace grows as O(H S d) only. */
size_t lh_workspace_bytes(int64_t N, int H, int d, int L, int p, int k, lh_dtype dt);

/* The dS tile budget of every later plan in this process (bytes; 0: always
 * recompute). Sizes and calls must agree: a workspace sized under one budget
 * and used under another may be too small (LH_EWORKSPACE). Thread-safe. */
void lh_set_ds_tile_budget(size_t bytes);
size_t lh_ds_tile_budget(void);

/* Bytes of workspace lh_forward alone needs (a prefix of the layout above):
 * a caller that never runs lh_backward may pass a workspace of this size.
 * 0 if the shape is invalid. */
size_t lh_forward_workspace_bytes(int64_t N, int H, int d, int L, int p, int k, lh_dtype dt);

/*
 * Forward pass: out = Lighthouse(q, k, v). Steps 1-4 above.
 * Leaves in ws the context lh_backward needs (scores, selection, slot maps,
 * gathered rows, sub-sequence output and log-sum-exp); the caller must not
 * modify ws between lh_forward and lh_backward of the same inputs.
 * ws_bytes >= lh_forward_workspace_bytes() suffices for the forward itself.
 */
lh_status lh_forward(const void *q, const void *k, const void *v,
                     int64_t N, int H, int d, int L, int p, int k_sel, lh_dtype dt,
                     void *out, void *ws, size_t ws_bytes, void *stream);

/*
 * lh_forward with the level-0 score chosen by `scorer` (LH_SCORE_*); the rest
 * of the layer is the same, and so are the workspace and the context it
 * leaves for lh_backward. LH_EINVAL for an unknown scorer.
 */
lh_status lh_forward_scored(const void *q, const void *k, const void *v,
                            int64_t N, int H, int d, int L, int p, int k_sel, lh_dtype dt, lh_scorer scorer,
                            void *out, void *ws, size_t ws_bytes, void *stream);

/*
 * lh_forward for calls that no backward follows (evaluation, a loss without
 * gradients). Same arguments, workspace and out; the sub-sequence attention
 * multiplies V by the fp16-rounded probabilities alone, where lh_forward
 * also adds the product with their fp16 residual so that O_sub agrees with
 * the probabilities the backward recomputes (delta = rowsum(dO_sub * O_sub)).
 * Each probability then carries a relative error up to 2^-11 (fp16 rounding)
 * before the fp32 accumulation, so an element (row, c) of one level's O_sub
 * may move by up to 2^-11 times the largest |v[., c]| among the rows it
 * attends, and out by up to L times that. On inputs of unit scale this stays
 * well inside the forward's tolerance; with value rows some 30 times larger
 * it reaches the tolerance's absolute term (lh_forward, with the fp16 pair
 * of P, stays inside it there).
 * The context it leaves differs from lh_forward's only in O_sub; lh_backward
 * on it runs, but its gradients are not covered by the stated tolerance:
 * call lh_forward before a backward.
 */
lh_status lh_forward_nograd(const void *q, const void *k, const void *v,
                            int64_t N, int H, int d, int L, int p, int k_sel, lh_dtype dt,
                            void *out, void *ws, size_t ws_bytes, void *stream);

/*
 * Backward pass with the indices of the preceding lh_forward held fixed
 * (the top-K is non-differentiable; aitrends summary, 핵심 기여): given dout =
 * dLoss/dout, writes dq, dk, dv. Needs only the context lh_forward left in ws,
 * not q, k, v themselves. Same shape arguments as that lh_forward, queued
 * after it (same stream, or ordered by the caller); ws_bytes >=
 * lh_workspace_bytes(). The context is trusted, not checked: on a workspace
 * that no completed lh_forward of this shape filled, or that was modified
 * since, dq, dk and dv hold unspecified values (possibly non-finite). Memory
 * accesses still stay inside ws, dout, dq, dk and dv: every slot-map entry is
 * bounds-checked against S_pad before it addresses a sub-sequence row, and
 * no other value read from ws is used as an address.
 *
 * Departure from the argument list (q, k, v, N, H, d, L, p, k, ...) of the
 * layer's plain call: q, k and v are not passed, because every quantity the
 * gradients need (gathered rows, selection, slot maps, O_sub, log-sum-exp) is
 * part of the context above; passing them again would be an unused argument.
 */
lh_status lh_backward(const void *dout,
                      int64_t N, int H, int d, int L, int p, int k_sel, lh_dtype dt,
                      void *dq, void *dk, void *dv, void *ws, size_t ws_bytes, void *stream);

/*
 * lh_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). The same work as lh_forward, writing the same out;
 * its workspace is a static device array of lh_static_scratch_bytes() bytes
 * (64 MiB) inside the library, one per GPU, held until the process ends.
 * Allocates nothing and calls no allocating routine; the first call on a
 * device looks up that device's array (the device that `stream` belongs to
 * must be current). A shape whose lh_forward_workspace_bytes() exceeds the
 * array returns LH_EWORKSPACE before anything is queued. Every call on a GPU
 * uses that GPU's one array, and the forward writes every part of it that it
 * reads before reading it (no part must start at zero): calls that overlap
 * in time on one GPU (two streams, two threads) race and give undefined
 * results; calls ordered on one stream do not. The array keeps the last
 * call's context, but lh_backward cannot use it (it takes a workspace).
 */
lh_status lh_forward_static(const void *q, const void *k, const void *v,
                            int64_t N, int H, int d, int L, int p, int k_sel, lh_dtype dt,
                            void *out, void *stream);
size_t lh_static_scratch_bytes(void);

/*
 * Timed variants: identical work, and in addition record hipEvent_t handles
 * events[0] before the first kernel and events[i+1] after stage i, on the
 * same stream. `events` holds lh_stage_count(backward)+1 caller-created
 * events. Stage names come from lh_stage_name().
 */
int lh_stage_count(int backward);
const char *lh_stage_name(int backward, int stage);
lh_status lh_forward_timed(const void *q, const void *k, const void *v,
                           int64_t N, int H, int d, int L, int p, int k_sel, lh_dtype dt,
                           void *out, void *ws, size_t ws_bytes, void *stream, void *const *events);
lh_status lh_forward_nograd_timed(const void *q, const void *k, const void *v,
                                  int64_t N, int H, int d, int L, int p, int k_sel, lh_dtype dt,
                                  void *out, void *ws, size_t ws_bytes, void *stream, void *const *events);
lh_status lh_backward_timed(const void *dout,
                            int64_t N, int H, int d, int L, int p, int k_sel, lh_dtype dt,
                            void *dq, void *dk, void *dv, void *ws, size_t ws_bytes, void *stream,
                            void *const *events);

/*
 * The step on either side of the layer, for a training step (aitrends
 * summary, 방법론 item 5: the gradients reach W_Q, W_K and W_V through
 * scatter-back, the gather and the attention): the Q, K and V projections of
 * an input x in, the layer's output out, and the backward to x and to the
 * projection weights.
 *   x      [N][d_model]       (dt), DEVICE, 16-byte aligned rows (d_model % 8 == 0)
 *   w_qkv  [d_model][3 H d]   (dt) row-major, columns [Q head 0..H-1 | K heads | V heads]
 *   out    [H][N][d]          (dt) = Lighthouse(x W_Q, x W_K, x W_V), as lh_forward
 *   dout   [H][N][d]          (dt) dLoss/dout
 *   dx     [N][d_model], dw_qkv [d_model][3 H d]  (dt) the gradients
 * The projections are dense GEMMs run by rocBLAS with fp32 accumulation,
 * atomics disallowed (reproducible), on a rocBLAS workspace inside ws; the
 * projected rows are rounded once to dt and then run through lh_forward /
 * lh_backward exactly as those entry points do. The first call on a device
 * creates that device's rocBLAS handle (rocBLAS may allocate device memory
 * when it creates a handle; every later call allocates nothing). ws holds the
 * projected rows, the layer's workspace, the rocBLAS workspace and the
 * gradients at the projected rows: lh_layer_workspace_bytes, 256-byte
 * aligned, the same ws for the forward and its backward (which does not
 * modify x, w_qkv or dout). After lh_layer_forward, ws begins with the
 * projected rows, [3][H][N][d] in dt (Q, K, V), which lh_layer_backward
 * overwrites; the layer's own workspace follows them at the next multiple of
 * 256 bytes (the base for lh_selection and lh_region_info). Calls from several host threads are serialised
 * around the rocBLAS handle. Errors as for lh_forward; LH_EUNSUPPORTED for
 * d_model not a multiple of 8 or above 65536.
 */
size_t lh_layer_workspace_bytes(int64_t N, int H, int d, int d_model, int L, int p, int k, lh_dtype dt);
lh_status lh_layer_forward(const void *x, const void *w_qkv, int64_t N, int H, int d, int d_model,
                           int L, int p, int k_sel, lh_dtype dt, void *out, void *ws, size_t ws_bytes, void *stream);
lh_status lh_layer_backward(const void *x, const void *w_qkv, const void *dout, int64_t N, int H, int d,
                            int d_model, int L, int p, int k_sel, lh_dtype dt, void *dx, void *dw_qkv,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * Test hook: byte offset and size, inside ws, of one intermediate that
 * lh_forward / lh_backward leave there. Layouts (per head h, heads outermost):
 *   LH_R_SCORES  fp32  [H][sum_l n_l]  level-0 scores, then level 1, ... (n_l = N/p^l);
 *                                      written when L > 1
 *   LH_R_SEL     int32 [L-1][H][k]     selected parents of levels 1..L-1, ascending
 *   LH_R_SLOT    int32 [H][sum_l n_l]  sub-sequence position of entry (l, i), or -1
 *   LH_R_ENT     int32 [H][S_pad]      entry at each position: (i << 3) | l; -1 past S
 *   LH_R_QHI/QLO fp16  [H][S_pad][d]   gathered query rows as an fp16 pair: hi =
 *                                      fp16(x), lo = fp16(x - hi) (pad rows zero);
 *                                      QLO is written for fp32 inputs only (size
 *                                      0 for bf16, whose kernels take the lo
 *                                      part from an internal e4m3 copy)
 *   LH_R_KHI/KLO fp16  [H][S_pad][d]   the same for keys (KLO: fp32 inputs only)
 *   LH_R_V       fp16  [H][S_pad][d]   gathered value rows
 *   LH_R_KHI_T/V_T fp16 [H][d][S_pad]  transposes of KHI and V
 *   LH_R_QHI_T                         size 0: no kernel needs the transpose of
 *                                      QHI (the id stays for compatibility)
 *   LH_R_OSUB    fp32  [H][S_pad][d]   attention output of the sub-sequence
 *   LH_R_LSE     fp32  [H][S_pad]      its row log-sum-exp in the log2 domain:
 *                                      log2 sum_b 2^(log2(e) q.k_b / sqrt(d))
 *                                      (the natural-log value times log2(e))
 *   LH_R_DOSUB   fp32  [H][S_pad][d]   gradient at the sub-sequence output
 *   LH_R_DQSUB/DKSUB/DVSUB fp32 [H][S_pad][d]  gradients at the gathered rows
 *   LH_R_EXP     int32 [4][H]          exponents e of the per-head power-of-two
 *                                      scales 2^e the fp16 rows above are staged
 *                                      with: Q, K and V (the gathered rows are
 *                                      2^e times the pooled rows), dO_sub (its
 *                                      fp16 copy, set by lh_backward)
 * S_pad = S rounded up to a multiple of 256. Returns LH_EINVAL for a bad shape
 * or region id.
 */
typedef enum {
    LH_R_SCORES = 0, LH_R_SEL, LH_R_SLOT, LH_R_ENT,
    LH_R_QHI, LH_R_QLO, LH_R_KHI, LH_R_KLO, LH_R_V,
    LH_R_QHI_T, LH_R_KHI_T, LH_R_V_T,
    LH_R_OSUB, LH_R_LSE, LH_R_DOSUB, LH_R_DQSUB, LH_R_DKSUB, LH_R_DVSUB, LH_R_EXP,
    LH_R_COUNT
} lh_region;
lh_status lh_region_info(int64_t N, int H, int d, int L, int p, int k, lh_dtype dt,
                         lh_region region, size_t *offset, size_t *bytes);
int64_t lh_padded_subseq_len(int64_t N, int L, int p, int k);

/*
 * Test hook for the stratified top-K (techllm review, 한계와 주의할 점: every
 * segment contributes a fixed number of entries; aitrends summary, 핵심 기여:
 * the selection is a non-differentiable top-K): sets *sel_dev to the DEVICE
 * address, inside ws, of the selection lh_forward made at pyramid level
 * `level` (1 <= level <= L-1): an int32 [H][k_sel] array, row h holding head
 * h's k_sel selected parents in ascending order (entries i of level `level`,
 * whose p children at level-1 were gathered). Valid once that lh_forward has
 * completed; the memory belongs to ws. Queues nothing and reads no device
 * memory. The address does not depend on the input type. Returns LH_EINVAL
 * (and sets *sel_dev to NULL when sel_dev is not NULL) for a bad shape, a
 * NULL or misaligned ws, L < 2 or a level outside 1..L-1.
 */
lh_status lh_selection(const void *ws, int64_t N, int H, int d, int L, int p, int k_sel, int level,
                       const int32_t **sel_dev);

/*
 * Test hook for the score's square root: for every fp32 bit pattern b in
 * [first, first + count) that encodes a positive finite value x, checks on
 * the GPU that the device sqrtf(x) used by the scorer is the correctly rounded
 * square root (exact fp64 test against the neighbouring midpoints) and adds
 * the number of failures to *mismatches (a device uint32 the caller zeroes).
 */
lh_status lh_selftest_sqrt(uint32_t first, uint32_t count, uint32_t *mismatches, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* LH_H */
