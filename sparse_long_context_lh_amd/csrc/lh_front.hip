// Front pass of the Lighthouse layer: one streaming read of Q, K and V that
// produces
//   * the token scores s_j = sqrt(||q_j||^2) + sqrt(||k_j||^2) (fp32, fixed
//     order; aitrends summary, 기술 상세 item 2) and their max-pooled values at
//     every coarser level (same passage: coarser levels receive the score by
//     max-pooling);
//   * the average-pooled rows (aitrends summary, 기술 상세 item 1; techllm
//     review, 어떻게 동작하나 step 1) of the levels the host chose to
//     materialise, as fp32 means of an fp32 sum (no rounding to 16 bits, so
//     the attention sees pooled rows at full precision).
//
// Work split: a "lane group" of d/8 lanes owns one row at a time, each lane
// holding 8 consecutive elements (16 B of bf16 or 32 B of fp32). A lane group
// streams a contiguous run of rows that starts on a top-level window
// boundary, so every level's window sum is built in registers by a cascade
// (the level-l sum is pushed into level l+1 when its window ends). No LDS, no
// atomics; each input byte is read once.
#include "lh_device.h"
#include "lh_internal.h"

namespace lh {

// ||x||^2 of a row whose 8-element pieces are spread over LANES lanes of one
// lane group: 8 fused multiply-adds in ascending element order from +0, then
// an xor butterfly with offsets LANES/2 .. 1 (every lane ends with a_0; fp32
// addition is commutative, so both partners of a pair compute the same bits).
template <int LANES>
__device__ __forceinline__ float row_norm2(const float (&x)[8])
{
    float a = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c)
        a = __builtin_fmaf(x[c], x[c], a);
#pragma unroll
    for (int off = LANES / 2; off >= 1; off >>= 1)
        a = a + __shfl_xor(a, off, LANES);
    return a;
}

template <int D, lh_dtype DT, int NL>
__global__ __launch_bounds__(256) void k_front(FrontArgs a)
{
    typedef typename Elem<DT>::T T;
    constexpr int LANES = D / 8;
    constexpr int NLG = 256 / LANES;
    constexpr int NA = NL > 1 ? NL - 1 : 1; // accumulators for levels 1..NL-1
    const int lane = threadIdx.x % LANES;
    const int lg = threadIdx.x / LANES;
    const int64_t run_id = (int64_t)blockIdx.x * NLG + lg;
    if (run_id >= (int64_t)a.H * a.runs_per_head)
        return;
    const int h = (int)(run_id / a.runs_per_head);
    const int64_t t0 = (run_id % a.runs_per_head) * a.run;
    const int64_t row0 = ((int64_t)h * a.N + t0) * D + lane * 8;
    const T *qp = reinterpret_cast<const T *>(a.q) + row0;
    const T *kp = reinterpret_cast<const T *>(a.k) + row0;
    const T *vp = reinterpret_cast<const T *>(a.v) + row0;
    float *sc = a.scores + (int64_t)h * a.lvl_total;
    float *pooled = a.pooled + (int64_t)h * a.mat_rows * D + lane * 8;

    float acc[3][NA][8];
    float smax[NA];
#pragma unroll
    for (int l = 0; l < NA; ++l) {
        smax[l] = 0.0f;
#pragma unroll
        for (int t = 0; t < 3; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[t][l][e] = 0.0f;
    }

    for (int r = 0; r < a.run; r += 4) {
        float xq[4][8], xk[4][8], xv[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (r + u < a.run) {
                load8(qp + (int64_t)(r + u) * D, xq[u]);
                load8(kp + (int64_t)(r + u) * D, xk[u]);
                if (NL > 1)
                    load8(vp + (int64_t)(r + u) * D, xv[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (r + u >= a.run)
                break;
            const int64_t t = t0 + r + u;
            const float s = sqrtf(row_norm2<LANES>(xq[u])) + sqrtf(row_norm2<LANES>(xk[u]));
            if (lane == 0)
                sc[t] = s;
            if constexpr (NL > 1) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    acc[0][0][e] += xq[u][e];
                    acc[1][0][e] += xk[u][e];
                    acc[2][0][e] += xv[u][e];
                }
                smax[0] = fmaxf(smax[0], s);
                // A level-l window ends on token t when p^l divides t+1; the
                // conditions nest, so levels are closed in ascending order.
#pragma unroll
                for (int l = 1; l < NL; ++l) {
                    const int sh = l * a.log2p;
                    if (((t + 1) & ((int64_t(1) << sh) - 1)) == 0) {
                        const int64_t i = t >> sh;
                        if (lane == 0)
                            sc[a.lvl_off[l] + i] = smax[l - 1];
                        if (a.mat_off[l] >= 0) {
                            const float w = 1.0f / (float)(int64_t(1) << sh); // exact: power of two
                            float *dst = pooled + (a.mat_off[l] + i) * D;
#pragma unroll
                            for (int t3 = 0; t3 < 3; ++t3) {
                                float m8[8];
#pragma unroll
                                for (int e = 0; e < 8; ++e)
                                    m8[e] = acc[t3][l - 1][e] * w;
                                store8(dst + t3 * a.tensor_stride, m8);
                            }
                        }
                        if (l + 1 < NL) {
#pragma unroll
                            for (int t3 = 0; t3 < 3; ++t3)
#pragma unroll
                                for (int e = 0; e < 8; ++e)
                                    acc[t3][l][e] += acc[t3][l - 1][e];
                            smax[l] = fmaxf(smax[l], smax[l - 1]);
                        }
#pragma unroll
                        for (int t3 = 0; t3 < 3; ++t3)
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                acc[t3][l - 1][e] = 0.0f;
                        smax[l - 1] = 0.0f;
                    }
                }
            }
        }
    }
}

template <int D, lh_dtype DT>
static hipError_t launch_front_t(const Plan &pl, const FrontArgs &a, hipStream_t s)
{
    constexpr int NLG = 256 / (D / 8);
    const int64_t runs = (int64_t)a.H * a.runs_per_head;
    const dim3 grid((unsigned)((runs + NLG - 1) / NLG));
    switch (pl.L) {
    case 1: hipLaunchKernelGGL((k_front<D, DT, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_front<D, DT, 2>), grid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_front<D, DT, 3>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_front<D, DT, 4>), grid, dim3(256), 0, s, a); break;
    case 5: hipLaunchKernelGGL((k_front<D, DT, 5>), grid, dim3(256), 0, s, a); break;
    case 6: hipLaunchKernelGGL((k_front<D, DT, 6>), grid, dim3(256), 0, s, a); break;
    case 7: hipLaunchKernelGGL((k_front<D, DT, 7>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_front<D, DT, 8>), grid, dim3(256), 0, s, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_front(const Plan &pl, const FrontArgs &a, hipStream_t s)
{
    if (pl.d == 128)
        return pl.dt == LH_BF16 ? launch_front_t<128, LH_BF16>(pl, a, s) : launch_front_t<128, LH_F32>(pl, a, s);
    return pl.dt == LH_BF16 ? launch_front_t<64, LH_BF16>(pl, a, s) : launch_front_t<64, LH_F32>(pl, a, s);
}

// ---------------------------------------------------------------- sqrt self-test
// For x = the fp32 value of bit pattern b (positive, finite), y = sqrtf(x) is
// correctly rounded iff x lies between the squares of the midpoints from y to
// its two fp32 neighbours. Those midpoints have at most 25 significant bits,
// so their squares and the comparison are exact in fp64.
__global__ void k_selftest_sqrt(uint32_t first, uint32_t count, uint32_t *mismatches)
{
    const uint64_t idx = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= count)
        return;
    const uint32_t b = first + (uint32_t)idx;
    if (b == 0u || b >= 0x7f800000u)
        return; // zero, negative, inf and NaN are outside the score's domain
    const float x = __uint_as_float(b);
    const float y = sqrtf(x);
    const uint32_t yb = __float_as_uint(y);
    const double yd = (double)y;
    const double lo = 0.5 * (yd + (double)__uint_as_float(yb - 1u));
    const double hi = 0.5 * (yd + (double)__uint_as_float(yb + 1u));
    const double xd = (double)x;
    if (!(lo * lo <= xd && xd <= hi * hi))
        atomicAdd(mismatches, 1u);
}

hipError_t launch_selftest_sqrt(uint32_t first, uint32_t count, uint32_t *mismatches, hipStream_t s)
{
    const unsigned blocks = (unsigned)(((uint64_t)count + 255) / 256);
    if (blocks == 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_selftest_sqrt, dim3(blocks), dim3(256), 0, s, first, count, mismatches);
    return hipGetLastError();
}

} // namespace lh
