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
 *     that fall in several ranges are summed (in ascending l); a token in no
 *     range receives 0.
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
 *   - Results are deterministic and bitwise reproducible (no atomics on the
 *     layer's path). Calls on distinct workspaces may run concurrently.
 *   - Inputs must be finite.
 *
 * Precision. Scores are fp32 in the stated order (bit-exact by design).
 * Pooling sums in fp32. The attention runs on fp16 matrix cores with fp32
 * accumulation: the logits use an fp16 hi/lo pair for the query rows (about
 * 22 significant bits, so pooled rows are not truncated before the softmax)
 * and fp16 key rows, plus the key's lo part for fp32 inputs; with bf16 inputs
 * the query lo product and the dO_sub lo product of dP run on block-scaled
 * fp8 (e4m3) copies with one power-of-two scale per head; P, V, dS and the
 * fp16 hi/lo pair of dO_sub
 * feed the other products; row statistics, Delta = rowsum(dO_sub * O_sub) and
 * all sums are fp32. Consequently every input, pooled row, scattered-back
 * gradient sum and attention intermediate must stay within the fp16 range
 * (|x| < 65504); a larger value overflows to inf and shows as a non-finite
 * output. Outputs are rounded once to the input dtype.
 *
 * Supported shapes: d in {64, 128}; p in {2, 4, 8}; 1 <= L <= 8;
 * 1 <= N <= 2^27, N a multiple of p^(L-1); 1 <= H <= 65535; 0 <= k <= N/p^(L-1);
 * a level of more than 2048 entries must hold a multiple of 2048;
 * (L-1)*k <= 16384; S rounded up to 256, times d, at most 2^30.
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

/* Human-readable name of a status code (static storage). */
const char *lh_strerror(lh_status s);

/* Validate a shape without touching the GPU. */
lh_status lh_check_shape(int64_t N, int H, int d, int L, int p, int k, lh_dtype dt);

/* Sub-sequence length S = N/p^(L-1) + (L-1)*p*k (techllm review, 핵심 수식);
 * -1 if the shape is invalid. */
int64_t lh_subseq_len(int64_t N, int L, int p, int k);

/* Bytes of device workspace lh_forward + lh_backward need for this shape;
 * 0 if the shape is invalid. */
size_t lh_workspace_bytes(int64_t N, int H, int d, int L, int p, int k, lh_dtype dt);

/*
 * Forward pass: out = Lighthouse(q, k, v). Steps 1-4 above.
 * Leaves in ws the context lh_backward needs (scores, selection, slot maps,
 * gathered rows, sub-sequence output and log-sum-exp); the caller must not
 * modify ws between lh_forward and lh_backward of the same inputs.
 */
lh_status lh_forward(const void *q, const void *k, const void *v,
                     int64_t N, int H, int d, int L, int p, int k_sel, lh_dtype dt,
                     void *out, void *ws, size_t ws_bytes, void *stream);

/*
 * Backward pass with the indices of the preceding lh_forward held fixed
 * (the top-K is non-differentiable; aitrends summary, 핵심 기여): given dout =
 * dLoss/dout, writes dq, dk, dv. Needs only the context lh_forward left in ws,
 * not q, k, v themselves. Same shape arguments as that lh_forward, queued
 * after it (same stream, or ordered by the caller). The context is trusted,
 * not checked: on a workspace that no completed lh_forward of this shape
 * filled, or that was modified since, the results are undefined and the
 * slot maps read there may address memory outside ws.
 */
lh_status lh_backward(const void *dout,
                      int64_t N, int H, int d, int L, int p, int k_sel, lh_dtype dt,
                      void *dq, void *dk, void *dv, void *ws, size_t ws_bytes, void *stream);

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
lh_status lh_backward_timed(const void *dout,
                            int64_t N, int H, int d, int L, int p, int k_sel, lh_dtype dt,
                            void *dq, void *dk, void *dv, void *ws, size_t ws_bytes, void *stream,
                            void *const *events);

/*
 * Test hook: byte offset and size, inside ws, of one intermediate that
 * lh_forward / lh_backward leave there. Layouts (per head h, heads outermost):
 *   LH_R_SCORES  fp32  [H][sum_l n_l]  level-0 scores, then level 1, ... (n_l = N/p^l);
 *                                      written when L > 1
 *   LH_R_SEL     int32 [H][L-1][k]     selected parents of levels 1..L-1, ascending
 *   LH_R_SLOT    int32 [H][sum_l n_l]  sub-sequence position of entry (l, i), or -1
 *   LH_R_ENT     int32 [H][S_pad]      entry at each position: (i << 3) | l; -1 past S
 *   LH_R_QHI/QLO fp16  [H][S_pad][d]   gathered query rows as an fp16 pair: hi =
 *                                      fp16(x), lo = fp16(x - hi) (pad rows zero)
 *   LH_R_KHI/KLO fp16  [H][S_pad][d]   the same for keys
 *   LH_R_V       fp16  [H][S_pad][d]   gathered value rows
 *   LH_R_QHI_T/KHI_T/V_T fp16 [H][d][S_pad]  transposes of QHI, KHI, V
 *   LH_R_OSUB    fp32  [H][S_pad][d]   attention output of the sub-sequence
 *   LH_R_LSE     fp32  [H][S_pad]      its row log-sum-exp in the log2 domain:
 *                                      log2 sum_b 2^(log2(e) q.k_b / sqrt(d))
 *                                      (the natural-log value times log2(e))
 *   LH_R_DOSUB   fp32  [H][S_pad][d]   gradient at the sub-sequence output
 *   LH_R_DQSUB/DKSUB/DVSUB fp32 [H][S_pad][d]  gradients at the gathered rows
 * S_pad = S rounded up to a multiple of 256. Returns LH_EINVAL for a bad shape
 * or region id.
 */
typedef enum {
    LH_R_SCORES = 0, LH_R_SEL, LH_R_SLOT, LH_R_ENT,
    LH_R_QHI, LH_R_QLO, LH_R_KHI, LH_R_KLO, LH_R_V,
    LH_R_QHI_T, LH_R_KHI_T, LH_R_V_T,
    LH_R_OSUB, LH_R_LSE, LH_R_DOSUB, LH_R_DQSUB, LH_R_DKSUB, LH_R_DVSUB,
    LH_R_COUNT
} lh_region;
lh_status lh_region_info(int64_t N, int H, int d, int L, int p, int k, lh_dtype dt,
                         lh_region region, size_t *offset, size_t *bytes);
int64_t lh_padded_subseq_len(int64_t N, int L, int p, int k);

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
