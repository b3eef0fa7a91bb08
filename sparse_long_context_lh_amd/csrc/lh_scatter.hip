// Scatter-back of the Lighthouse layer and the adjoints of the stages around
// the attention.
//
// Scatter-back (aitrends summary, 기술 상세 item 4; techllm review, 어떻게
// 동작하나 step 4): the sub-sequence output of entry (l, i) is added to every
// token of R(l, i) = [(i+1)p^l - 1, (i+2)p^l - 2] (clipped at N). For a token
// j the one level-l entry whose range holds j is i = floor((j+1)/p^l) - 1, so
// the kernel PULLS: O_j = sum over l (ascending) of O_sub[slot_l(i)] for the
// levels where that entry exists and was gathered. No atomics.
//
// Adjoint of scatter-back: with u = j + 1, R(l, i) is the aligned window
// [(i+1)p^l, (i+2)p^l) of u, so dO_sub of entry (l, i) is the sum of dO over
// aligned u-window i+1 of level l. One streaming pass over dO builds all
// levels' window sums in registers (as the front pass does for pooling).
//
// Adjoint of gather(pool(.)): token j receives p^-l times the gradient of
// gathered entry (l, floor(j/p^l)) from every level where that entry was
// gathered (pull again, ascending l).
#include "lh_device.h"
#include "lh_internal.h"

namespace lh {

constexpr int kRowsPerGroup = 4;
constexpr int kPrepTile = 64;

// ---------------------------------------------------------------- scatter-back
template <int D, lh_dtype DT>
__global__ __launch_bounds__(256) void k_scatter(ScatterArgs a)
{
    typedef typename Elem<DT>::T T;
    constexpr int LANES = D / 8, NLG = 256 / LANES;
    const int lane = threadIdx.x % LANES, lg = threadIdx.x / LANES;
    const int64_t rows = (int64_t)a.H * a.N;
    const int64_t r0 = ((int64_t)blockIdx.x * NLG + lg) * kRowsPerGroup;
    for (int rr = 0; rr < kRowsPerGroup; ++rr) {
        const int64_t row = r0 + rr;
        if (row >= rows)
            return;
        const int h = (int)(row / a.N);
        const int64_t j = row - (int64_t)h * a.N;
        const int32_t *slot = a.slot + (int64_t)h * a.lvl_total;
        const float *osub = a.osub + (int64_t)h * a.S_pad * D + lane * 8;
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[e] = 0.0f;
        for (int l = 0; l < a.L; ++l) {
            const int64_t i = ((j + 1) >> (l * a.log2p)) - 1;
            if (i < 0)
                continue;
            const int32_t sl = slot[a.lvl_off[l] + i];
            if ((uint32_t)sl >= (uint32_t)a.S_pad)
                continue; // -1: not gathered
            float x[8];
            load8(osub + (int64_t)sl * D, x);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[e] += x[e];
        }
        store8(reinterpret_cast<T *>(a.out) + row * D + lane * 8, acc);
    }
}

hipError_t launch_scatter(const Plan &pl, const ScatterArgs &a, hipStream_t s)
{
    const int nlg = 256 / (pl.d / 8);
    const int64_t groups = ((int64_t)pl.H * pl.N + kRowsPerGroup - 1) / kRowsPerGroup;
    const dim3 grid((unsigned)((groups + nlg - 1) / nlg));
    if (pl.d == 128) {
        if (pl.dt == LH_BF16)
            hipLaunchKernelGGL((k_scatter<128, LH_BF16>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((k_scatter<128, LH_F32>), grid, dim3(256), 0, s, a);
    } else {
        if (pl.dt == LH_BF16)
            hipLaunchKernelGGL((k_scatter<64, LH_BF16>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((k_scatter<64, LH_F32>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- adjoint of scatter-back
template <int D, lh_dtype DT, int NL>
__global__ __launch_bounds__(256) void k_scatter_bwd(ScatterBwdArgs a)
{
    typedef typename Elem<DT>::T T;
    constexpr int LANES = D / 8, NLG = 256 / LANES;
    constexpr int NA = NL > 1 ? NL - 1 : 1;
    const int lane = threadIdx.x % LANES, lg = threadIdx.x / LANES;
    const int64_t run_id = (int64_t)blockIdx.x * NLG + lg;
    if (run_id >= (int64_t)a.H * a.tiles_per_head)
        return;
    const int h = (int)(run_id / a.tiles_per_head);
    const int64_t u0 = (run_id % a.tiles_per_head) * a.run;
    const T *dout = reinterpret_cast<const T *>(a.dout) + (int64_t)h * a.N * D + lane * 8;
    const int32_t *slot = a.slot + (int64_t)h * a.lvl_total;
    float *dosub = a.dosub + (int64_t)h * a.S_pad * D + lane * 8;

    float acc[NA][8];
#pragma unroll
    for (int l = 0; l < NA; ++l)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[l][e] = 0.0f;

    for (int r = 0; r < a.run; r += 4) {
        float x[4][8];
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) {
            const int64_t j = u0 + r + uu - 1;
            if (r + uu < a.run && j >= 0 && j < a.N) {
                load8(dout + j * D, x[uu]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    x[uu][e] = 0.0f;
            }
        }
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) {
            if (r + uu >= a.run)
                break;
            const int64_t u = u0 + r + uu;
            const int64_t j = u - 1;
            if (j >= 0 && j < a.N) { // level 0: R(0, j) = {j}
                const int32_t sl = slot[a.lvl_off[0] + j];
                if ((uint32_t)sl < (uint32_t)a.S_pad)
                    store8(dosub + (int64_t)sl * D, x[uu]);
            }
            if constexpr (NL > 1) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[0][e] += x[uu][e];
#pragma unroll
                for (int l = 1; l < NL; ++l) {
                    const int sh = l * a.log2p;
                    if (((u + 1) & ((int64_t(1) << sh) - 1)) == 0) {
                        const int64_t i = (u >> sh) - 1;
                        if (i >= 0 && i < (a.N >> sh)) {
                            const int32_t sl = slot[a.lvl_off[l] + i];
                            if ((uint32_t)sl < (uint32_t)a.S_pad)
                                store8(dosub + (int64_t)sl * D, acc[l - 1]);
                        }
                        if (l + 1 < NL) {
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                acc[l][e] += acc[l - 1][e];
                        }
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            acc[l - 1][e] = 0.0f;
                    }
                }
            }
        }
    }
}

template <int D, lh_dtype DT>
static void launch_scatter_bwd_t(const Plan &pl, const ScatterBwdArgs &a, hipStream_t s)
{
    constexpr int NLG = 256 / (D / 8);
    const int64_t runs = (int64_t)a.H * a.tiles_per_head;
    const dim3 grid((unsigned)((runs + NLG - 1) / NLG));
    switch (pl.L) {
    case 1: hipLaunchKernelGGL((k_scatter_bwd<D, DT, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_scatter_bwd<D, DT, 2>), grid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL((k_scatter_bwd<D, DT, 3>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((k_scatter_bwd<D, DT, 4>), grid, dim3(256), 0, s, a); break;
    case 5: hipLaunchKernelGGL((k_scatter_bwd<D, DT, 5>), grid, dim3(256), 0, s, a); break;
    case 6: hipLaunchKernelGGL((k_scatter_bwd<D, DT, 6>), grid, dim3(256), 0, s, a); break;
    case 7: hipLaunchKernelGGL((k_scatter_bwd<D, DT, 7>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_scatter_bwd<D, DT, 8>), grid, dim3(256), 0, s, a); break;
    }
}

hipError_t launch_scatter_bwd(const Plan &pl, const ScatterBwdArgs &a, hipStream_t s)
{
    if (pl.d == 128) {
        if (pl.dt == LH_BF16)
            launch_scatter_bwd_t<128, LH_BF16>(pl, a, s);
        else
            launch_scatter_bwd_t<128, LH_F32>(pl, a, s);
    } else {
        if (pl.dt == LH_BF16)
            launch_scatter_bwd_t<64, LH_BF16>(pl, a, s);
        else
            launch_scatter_bwd_t<64, LH_F32>(pl, a, s);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- backward prep
// fp16 pair of dO_sub (hi = fp16(x), lo = fp16(x - hi)) row-major, the hi part
// transposed (MFMA operands of the attention backward), and
// delta_s = sum_d (hi + lo)[s][d] * O_sub[s][d], the row term of the softmax
// gradient, from the same values the dP products see. Rows past S are zero.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_prep(BwdPrepArgs a)
{
    constexpr int LANES = D / 8, NLG = 256 / LANES, LD = D + 8;
    __shared__ __attribute__((aligned(16))) uint16_t tile[kPrepTile * LD];
    const int h = blockIdx.y;
    const int64_t s0 = (int64_t)blockIdx.x * kPrepTile;
    const int lane = threadIdx.x % LANES, lg = threadIdx.x / LANES;
    for (int r = lg; r < kPrepTile; r += NLG) {
        const int64_t s = s0 + r;
        const int64_t off = ((int64_t)h * a.S_pad + s) * D + lane * 8;
        float x[8], o[8];
        if (s < a.S) {
            load8(a.dosub + off, x);
            load8(a.osub + off, o);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                x[e] = o[e] = 0.0f;
        }
        uint4 hi, lo;
        split8_f16(x, hi, lo);
        float xh[8], xl[8];
        unpack8_f16(hi, xh);
        unpack8_f16(lo, xl);
        float dot = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            dot = __builtin_fmaf(xh[e] + xl[e], o[e], dot);
#pragma unroll
        for (int off2 = LANES / 2; off2 >= 1; off2 >>= 1)
            dot += __shfl_xor(dot, off2, LANES);
        if (lane == 0)
            a.delta[(int64_t)h * a.S_pad + s] = dot;
        *reinterpret_cast<uint4 *>(a.dohi + off) = hi;
        *reinterpret_cast<uint4 *>(a.dolo + off) = lo;
        *reinterpret_cast<uint4 *>(&tile[r * LD + lane * 8]) = hi;
    }
    __syncthreads();
    constexpr int CH = kPrepTile / 8;
    for (int c = threadIdx.x; c < D * CH; c += 256) {
        const int dim = c / CH, sc = c - (c / CH) * CH;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo16 = tile[(sc * 8 + 2 * e) * LD + dim];
            const uint32_t hi16 = tile[(sc * 8 + 2 * e + 1) * LD + dim];
            w[e] = lo16 | (hi16 << 16);
        }
        *reinterpret_cast<uint4 *>(a.dohi_t + ((int64_t)h * D + dim) * a.S_pad + s0 + sc * 8) =
            make_uint4(w[0], w[1], w[2], w[3]);
    }
}

hipError_t launch_bwd_prep(const Plan &pl, const BwdPrepArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)(pl.S_pad / kPrepTile), pl.H);
    if (pl.d == 128)
        hipLaunchKernelGGL((k_bwd_prep<128>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((k_bwd_prep<64>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- adjoint of gather(pool(.))
template <int D, lh_dtype DT>
__global__ __launch_bounds__(256) void k_pool_bwd(PoolBwdArgs a)
{
    typedef typename Elem<DT>::T T;
    constexpr int LANES = D / 8, NLG = 256 / LANES;
    const int lane = threadIdx.x % LANES, lg = threadIdx.x / LANES;
    const int64_t rows = (int64_t)a.H * a.N;
    const int64_t r0 = ((int64_t)blockIdx.x * NLG + lg) * kRowsPerGroup;
    for (int rr = 0; rr < kRowsPerGroup; ++rr) {
        const int64_t row = r0 + rr;
        if (row >= rows)
            return;
        const int h = (int)(row / a.N);
        const int64_t j = row - (int64_t)h * a.N;
        const int32_t *slot = a.slot + (int64_t)h * a.lvl_total;
        float acc[3][8];
#pragma unroll
        for (int t = 0; t < 3; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[t][e] = 0.0f;
        for (int l = 0; l < a.L; ++l) {
            const int sh = l * a.log2p;
            const int32_t sl = slot[a.lvl_off[l] + (j >> sh)];
            if ((uint32_t)sl >= (uint32_t)a.S_pad)
                continue; // -1: not gathered
            const float w = 1.0f / (float)(int64_t(1) << sh); // exact: power of two
            const int64_t off = ((int64_t)h * a.S_pad + sl) * D + lane * 8;
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                float x[8];
                load8(a.dsub[t] + off, x);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc[t][e] += x[e] * w;
            }
        }
#pragma unroll
        for (int t = 0; t < 3; ++t)
            store8(reinterpret_cast<T *>(a.dx[t]) + row * D + lane * 8, acc[t]);
    }
}

hipError_t launch_pool_bwd(const Plan &pl, const PoolBwdArgs &a, hipStream_t s)
{
    const int nlg = 256 / (pl.d / 8);
    const int64_t groups = ((int64_t)pl.H * pl.N + kRowsPerGroup - 1) / kRowsPerGroup;
    const dim3 grid((unsigned)((groups + nlg - 1) / nlg));
    if (pl.d == 128) {
        if (pl.dt == LH_BF16)
            hipLaunchKernelGGL((k_pool_bwd<128, LH_BF16>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((k_pool_bwd<128, LH_F32>), grid, dim3(256), 0, s, a);
    } else {
        if (pl.dt == LH_BF16)
            hipLaunchKernelGGL((k_pool_bwd<64, LH_BF16>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((k_pool_bwd<64, LH_F32>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

} // namespace lh
