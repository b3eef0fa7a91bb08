/*
 * Lighthouse Attention oracle: the fp32 token scorer.
 *
 * TEST INFRASTRUCTURE ONLY. This file is part of the CPU oracle that the
 * parity tests, the smoke check and the benchmark's CPU baseline use. It
 * shares no code with the HIP path and the product never calls it.
 *
 * What it computes (aitrends.kr "Lighthouse Attention" summary, section
 * "기술 상세", item 2; techllm.github.io review, "어떻게 동작하나" step 2):
 * every level-0 entry is ranked by a parameter-free score built from the
 * l2 norms of its query row and its key row. The score is
 *
 *     s_j = sqrt(||q_j||^2) + sqrt(||k_j||^2)            (fp32)
 *
 * The pages fix neither the precision nor the reduction order. Selected
 * indices must match the GPU bit for bit, so both sides follow one stated
 * fp32 order for ||x||^2 of a row of d values (d a multiple of 16, d/8 a
 * power of two):
 *   1. partial j, for j in [0, d/8), starts at +0 and accumulates
 *      a_j = fmaf(x_c, x_c, a_j) for c = 8j .. 8j+7 in ascending c;
 *   2. for off = d/16, d/32, ..., 1 every partial is replaced, all at once,
 *      by a_j + a_(j xor off);
 *   3. the result is a_0.
 * sqrt is the IEEE-754 correctly rounded single-precision square root, and
 * the two roots are added in fp32.
 *
 * Variants of the score. The pages rank entries by parameter-free query/key
 * l2 norms and name more than one combination ("QK and KQ l2 norms, etc.",
 * aitrends summary, "핵심 기여"; a norm scorer whose retrieval differs,
 * techllm review, "한계와 주의할 점"). From the same two correctly rounded
 * roots nq = sqrt(||q||^2) and nk = sqrt(||k||^2), in fp32:
 *   0 sum     nq + nk   (the default above)
 *   1 product nq * nk
 *   2 query   nq
 *   3 key     nk
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC (no -ffast-math,
 * so fmaf is a true fused multiply-add and no other operation is fused).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define MAX_PARTIALS 64 /* d <= 512 */

/* ||x||^2 of one row in the order stated above. */
static float row_norm2(const float *x, int d)
{
    float a[MAX_PARTIALS];
    float b[MAX_PARTIALS];
    int parts = d / 8;
    for (int j = 0; j < parts; ++j) {
        float acc = 0.0f;
        for (int c = 8 * j; c < 8 * j + 8; ++c)
            acc = fmaf(x[c], x[c], acc);
        a[j] = acc;
    }
    for (int off = parts / 2; off >= 1; off /= 2) {
        for (int j = 0; j < parts; ++j)
            b[j] = a[j] + a[j ^ off];
        memcpy(a, b, sizeof(float) * (size_t)parts);
    }
    return a[0];
}

static int shape_ok(int d)
{
    if (d < 16 || d > 8 * MAX_PARTIALS || d % 16 != 0)
        return 0;
    int parts = d / 8;
    return (parts & (parts - 1)) == 0;
}

/* out[r] = ||x_r||^2 for n_rows rows of d floats. Returns 0, or -1 on a bad d. */
int oracle_row_norm2(const float *x, int64_t n_rows, int d, float *out)
{
    if (!shape_ok(d))
        return -1;
    for (int64_t r = 0; r < n_rows; ++r)
        out[r] = row_norm2(x + r * (int64_t)d, d);
    return 0;
}

/* s[r] = sqrtf(||q_r||^2) + sqrtf(||k_r||^2). Returns 0, or -1 on a bad d. */
int oracle_token_scores(const float *q, const float *k, int64_t n_rows, int d, float *s)
{
    if (!shape_ok(d))
        return -1;
    for (int64_t r = 0; r < n_rows; ++r) {
        float nq = row_norm2(q + r * (int64_t)d, d);
        float nk = row_norm2(k + r * (int64_t)d, d);
        s[r] = sqrtf(nq) + sqrtf(nk);
    }
    return 0;
}

/* s[r] = the score of variant `scorer` (0 sum, 1 product, 2 query, 3 key) of
 * row r. Returns 0, or -1 on a bad d or scorer. */
int oracle_token_scores_v(const float *q, const float *k, int64_t n_rows, int d, int scorer, float *s)
{
    if (!shape_ok(d) || scorer < 0 || scorer > 3)
        return -1;
    for (int64_t r = 0; r < n_rows; ++r) {
        float nq = sqrtf(row_norm2(q + r * (int64_t)d, d));
        float nk = sqrtf(row_norm2(k + r * (int64_t)d, d));
        switch (scorer) {
        case 0: s[r] = nq + nk; break;
        case 1: s[r] = nq * nk; break;
        case 2: s[r] = nq; break;
        default: s[r] = nk; break;
        }
    }
    return 0;
}
