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
#include <string.h>

#include <algorithm>

#include "lh_device.h"
#include "lh_internal.h"

namespace lh {

constexpr int kPrepTile = 64;

// ---------------------------------------------------------------- pull kernels
// Scatter-back and the adjoint of gather(pool(.)) have one shape: token t
// receives sum over levels l of w_l * src[slot_l(e_l)] with e_l = (x >> l*log2p)
// - OFF, x = t + OFF, over the levels whose entry e_l exists and was gathered.
// Scatter-back: OFF = 1 (x = u = j + 1), w_l = 1, one tensor. Pool adjoint:
// OFF = 0, w_l = p^-l, three tensors (Q, K, V).
//
// A workgroup owns a tile of T = NLG * R consecutive positions x of one head,
// R = p^NC per lane group. It first copies the slot entries every level needs
// for the tile into LDS (coalesced loads, no dependent index chains). A lane
// group then sums the levels >= NC once for its R positions (they share those
// entries), and walks the positions keeping the partial sums of levels >= l
// (l = NC-1 .. 1) in registers, refreshed when x crosses a p^l boundary; each
// position adds its own level-0 row (if gathered) and is stored.
struct PullArgs {
    const float *src[3];  // [H][S_pad][d]
    void *dst[3];         // [H][N][d] in the input dtype
    const int32_t *slot;  // [H][lvl_total]
    int64_t N, lvl_total, S_pad;
    int64_t lvl_off[kMaxLevels];
    int L, log2p, weighted;
};

constexpr int kPullMaxTile = 512; // positions per workgroup: 32 lane groups x 16

template <int NT>
__device__ __forceinline__ void pull_add(float (&acc)[NT][8], const PullArgs &a, int64_t off, float w)
{
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        float x[8];
        load8(a.src[t] + off, x);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[t][e] = __builtin_fmaf(x[e], w, acc[t][e]);
    }
}

__device__ __forceinline__ int pull_count(int64_t x0, int64_t T, int sh)
{
    return (int)(((x0 + T - 1) >> sh) - (x0 >> sh) + 1);
}

template <int D, lh_dtype DT, int NT, int OFF, int NC>
__global__ __launch_bounds__(256) void k_pull(PullArgs a)
{
    typedef typename Elem<DT>::T T;
    constexpr int LANES = D / 8, NLG = 256 / LANES;
    // level l holds at most T / p^l + 2 entries, so all levels together < 2T + 2L
    __shared__ int32_t s_slot[2 * kPullMaxTile + 2 * kMaxLevels];
    const int lane = threadIdx.x % LANES, lg = threadIdx.x / LANES;
    const int h = blockIdx.y;
    const int lp = a.log2p;
    const int R = 1 << (NC * lp);
    const int64_t tile = (int64_t)NLG * R;
    const int64_t x0 = (int64_t)blockIdx.x * tile;
    const int32_t *slot = a.slot + (int64_t)h * a.lvl_total;

    int b = 0;
    for (int l = 0; l < a.L; ++l) {
        const int sh = l * lp;
        const int cnt = pull_count(x0, tile, sh);
        const int64_t e0 = (x0 >> sh) - OFF, nl = a.N >> sh;
        for (int e = threadIdx.x; e < cnt; e += 256) {
            const int64_t i = e0 + e;
            s_slot[b + e] = (i >= 0 && i < nl) ? slot[a.lvl_off[l] + i] : -1;
        }
        b += cnt;
    }
    __syncthreads();

    const int64_t xg = x0 + (int64_t)lg * R;
    const int64_t rowbase = (int64_t)h * a.S_pad;
    const int col = lane * 8;
    int base[NC > 0 ? NC : 1];
    b = 0;
#pragma unroll
    for (int l = 0; l < NC; ++l) {
        base[l] = b;
        b += pull_count(x0, tile, l * lp);
    }
    float coarse[NT][8]; // levels >= NC, shared by the lane group's R positions
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            coarse[t][e] = 0.0f;
    for (int l = NC; l < a.L; ++l) { // levels shared by the lane group's R positions
        const int sh = l * lp;
        const int sl = s_slot[b + (int)((xg >> sh) - (x0 >> sh))];
        b += pull_count(x0, tile, sh);
        if ((uint32_t)sl < (uint32_t)a.S_pad)
            pull_add<NT>(coarse, a, (rowbase + sl) * D + col, a.weighted ? 1.0f / (float)(1 << sh) : 1.0f);
    }
    if constexpr (NC == 0) { // L = 1: one position per lane group, level 0 already summed
        const int64_t t = xg - OFF;
        if (t >= 0 && t < a.N)
#pragma unroll
            for (int u = 0; u < NT; ++u)
                store8_stream(reinterpret_cast<T *>(a.dst[u]) + ((int64_t)h * a.N + t) * D + col, coarse[u]);
    } else {
        // tensor after tensor (the finer levels' partial sums of one tensor
        // live at a time, which keeps the register count and with it the
        // number of resident workgroups up)
#pragma unroll
        for (int u = 0; u < NT; ++u) {
            float fine[NC][8]; // fine[l]: levels >= l of the current window (l >= 1)
            const float *src = a.src[u];
            T *dst = reinterpret_cast<T *>(a.dst[u]) + (int64_t)h * a.N * D + col;
            for (int r = 0; r < R; ++r) {
                const int64_t x = xg + r;
#pragma unroll
                for (int l = NC - 1; l >= 1; --l) {
                    const int sh = l * lp;
                    if ((r & ((1 << sh) - 1)) == 0) {
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            fine[l][e] = l + 1 < NC ? fine[l + 1 < NC ? l + 1 : 0][e] : coarse[u][e];
                        const int sl = s_slot[base[l] + (int)((x >> sh) - (x0 >> sh))];
                        if ((uint32_t)sl < (uint32_t)a.S_pad) {
                            float y[8];
                            load8(src + (rowbase + sl) * D + col, y);
                            const float w = a.weighted ? 1.0f / (float)(1 << sh) : 1.0f;
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                fine[l][e] = __builtin_fmaf(y[e], w, fine[l][e]);
                        }
                    }
                }
                float o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    o[e] = NC > 1 ? fine[NC > 1 ? 1 : 0][e] : coarse[u][e];
                const int sl = s_slot[base[0] + (int)(x - x0)];
                if ((uint32_t)sl < (uint32_t)a.S_pad) {
                    float y[8];
                    load8(src + (rowbase + sl) * D + col, y);
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        o[e] = __builtin_fmaf(y[e], 1.0f, o[e]);
                }
                const int64_t t = x - OFF;
                if (t >= 0 && t < a.N)
                    store8_stream(dst + t * D, o);
            }
        }
    }
}

// Gathered rows of levels >= nc a position loads on average with runs of
// p^nc positions (a shared level's row once per run; finer levels once per
// window). Level l < L-1 gathers p k of its n_l entries, the top level all.
static double pull_rows_per_position(const Plan &pl, int nc)
{
    double rows = 0.0;
    for (int l = 0; l < pl.L; ++l) {
        const double g = l == pl.L - 1 ? 1.0 : std::min(1.0, (double)pl.p * pl.k / (double)pl.n[l]);
        rows += g / (double)((int64_t)1 << ((l < nc ? l : nc) * pl.log2p));
    }
    return rows;
}

// Levels shared per lane group: a run of R = p^NC positions (8 or 16). The
// three-tensor pool adjoint takes runs of 4 at p = 4 when that keeps its
// row loads low: its smaller tiles write faster (measured: 512K tokens, 0.33
// rows per position, 1.28 -> 1.25 ms), while many shared rows per run make
// it slower (1M tokens, 0.58 rows per position, 1.29 -> 1.56 ms).
static int pull_levels(const Plan &pl, int nt)
{
    int want = pl.log2p == 1 ? 3 : (pl.log2p == 2 ? 2 : 1);
    if (nt == 3 && pl.log2p == 2 && pl.L > 2 && pull_rows_per_position(pl, 1) <= 0.4)
        want = 1;
    return want < pl.L - 1 ? want : pl.L - 1;
}

template <int D, lh_dtype DT, int NT, int OFF>
static hipError_t launch_pull_t(const Plan &pl, const PullArgs &a, hipStream_t s)
{
    constexpr int NLG = 256 / (D / 8);
    const int nc = pull_levels(pl, NT);
    const int64_t tile = (int64_t)NLG << (nc * pl.log2p);
    if (tile > kPullMaxTile)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)((pl.N + OFF + tile - 1) / tile), (unsigned)pl.H);
    switch (nc) {
    case 0: hipLaunchKernelGGL((k_pull<D, DT, NT, OFF, 0>), grid, dim3(256), 0, s, a); break;
    case 1: hipLaunchKernelGGL((k_pull<D, DT, NT, OFF, 1>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((k_pull<D, DT, NT, OFF, 2>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((k_pull<D, DT, NT, OFF, 3>), grid, dim3(256), 0, s, a); break;
    }
    return hipGetLastError();
}

template <int NT, int OFF>
static hipError_t launch_pull(const Plan &pl, const PullArgs &a, hipStream_t s)
{
    if (pl.d == 128)
        return pl.dt == LH_BF16 ? launch_pull_t<128, LH_BF16, NT, OFF>(pl, a, s)
                                : launch_pull_t<128, LH_F32, NT, OFF>(pl, a, s);
    return pl.dt == LH_BF16 ? launch_pull_t<64, LH_BF16, NT, OFF>(pl, a, s)
                            : launch_pull_t<64, LH_F32, NT, OFF>(pl, a, s);
}

hipError_t launch_scatter(const Plan &pl, const ScatterArgs &sa, hipStream_t s)
{
    PullArgs a;
    memset(&a, 0, sizeof(a));
    a.src[0] = sa.osub;
    a.dst[0] = sa.out;
    a.slot = sa.slot;
    a.N = sa.N; a.lvl_total = sa.lvl_total; a.S_pad = sa.S_pad;
    for (int l = 0; l < kMaxLevels; ++l)
        a.lvl_off[l] = sa.lvl_off[l];
    a.L = sa.L; a.log2p = sa.log2p; a.weighted = 0;
    return launch_pull<1, 1>(pl, a, s);
}

// ---------------------------------------------------------------- adjoint of scatter-back
// Row tiles in u-space (u = j + 1; TileShape): a lane group loads R rows of
// dO at once, stores the rows whose level-0 entry was gathered, and sums its
// run level by level (window sums of p child sums in ascending order, from
// 0); run totals meet in LDS for the levels whose windows fit the tile, and
// each coarser level is one small kernel over the window sums of the level
// below. Window m of level l is entry i = m - 1 (window 0 has no entry).
constexpr int cpow(int b, int e) { return e == 0 ? 1 : b * cpow(b, e - 1); }

template <int D, lh_dtype DT, int LP>
__global__ __launch_bounds__(256) void k_scatter_bwd(ScatterBwdArgs a)
{
    typedef typename Elem<DT>::T T;
    typedef TileShape<D, LP, sbwd_nc(LP)> Sh;
    constexpr int LANES = Sh::LANES, NLG = Sh::NLG, NC = Sh::NC, R = Sh::R, P = 1 << LP;
    __shared__ __attribute__((aligned(16))) float s_sum[NLG][D];
    __shared__ int32_t s_slot[2 * Sh::T]; // levels 0..LT: T/p^l windows each
    const int lane = threadIdx.x % LANES, lg = threadIdx.x / LANES, col = lane * 8;
    const int h = blockIdx.y;
    const int64_t x0 = (int64_t)blockIdx.x * Sh::T;
    const int64_t ug = x0 + (int64_t)lg * R;
    const int LT = a.LT;
    const bool keep = LT < a.L - 1;
    const int32_t *slot = a.slot + (int64_t)h * a.lvl_total;
    float *dosub = a.dosub + (int64_t)h * a.S_pad * D + col;
    float *part = a.part + (int64_t)h * a.part_rows * D + col;

    {
        int b = 0;
        for (int l = 0; l <= LT; ++l) {
            const int sh = l * LP, cnt = Sh::T >> sh;
            const int64_t nl = a.N >> sh, e0 = (x0 >> sh) - 1;
            for (int e = threadIdx.x; e < cnt; e += 256) {
                const int64_t i = e0 + e;
                s_slot[b + e] = (i >= 0 && i < nl) ? slot[a.lvl_off[l] + i] : -1;
            }
            b += cnt;
        }
    }
    const T *dout = reinterpret_cast<const T *>(a.dout) + (int64_t)h * a.N * D + col;
    Raw8<DT> rows[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t u = ug + r;
        if (u >= 1 && u <= a.N)
            ld_stream(dout + (u - 1) * D, rows[r]);
        else
            zero_raw(rows[r]);
    }
    __syncthreads();

    // finished window m of level l (l <= LT): to dO_sub if its entry was
    // gathered, and kept for the next level if l is LT and coarser ones exist
    auto put = [&](int l, int64_t m, const float (&acc)[8]) {
        int b = 0;
        for (int q = 0; q < l; ++q)
            b += Sh::T >> (q * LP);
        const int32_t sl = s_slot[b + (int)(m - (x0 >> (l * LP)))];
        if ((uint32_t)sl < (uint32_t)a.S_pad)
            store8(dosub + (int64_t)sl * D, acc);
        if (keep && l == LT)
            store8(part + (a.part_off[l] + m) * D, acc);
    };

    float acc[NC][8], tot[8];
#pragma unroll
    for (int l = 0; l < NC; ++l)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[l][e] = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float x[8];
        unraw(rows[r], x);
        put(0, ug + r, x);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[0][e] += x[e];
#pragma unroll
        for (int l = 1; l <= NC; ++l) {
            if ((r + 1) % cpow(P, l) == 0) {
                if (l <= LT)
                    put(l, (ug >> (l * LP)) + (r + 1) / cpow(P, l) - 1, acc[l - 1]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (l < NC)
                        acc[l < NC ? l : 0][e] += acc[l - 1][e];
                    else
                        tot[e] = acc[l - 1][e];
                    acc[l - 1][e] = 0.0f;
                }
            }
        }
    }

    if (LT > NC) {
        *reinterpret_cast<float4 *>(&s_sum[lg][col]) = make_float4(tot[0], tot[1], tot[2], tot[3]);
        *reinterpret_cast<float4 *>(&s_sum[lg][col + 4]) = make_float4(tot[4], tot[5], tot[6], tot[7]);
        __syncthreads();
        int W = NLG;
        for (int l = NC + 1; l <= LT; ++l) {
            W /= P;
            float res[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                res[e] = 0.0f;
            if (lg < W) {
                for (int c = 0; c < P; ++c) {
                    const float4 lo = *reinterpret_cast<const float4 *>(&s_sum[lg * P + c][col]);
                    const float4 hi = *reinterpret_cast<const float4 *>(&s_sum[lg * P + c][col + 4]);
                    res[0] += lo.x; res[1] += lo.y; res[2] += lo.z; res[3] += lo.w;
                    res[4] += hi.x; res[5] += hi.y; res[6] += hi.z; res[7] += hi.w;
                }
                put(l, (x0 >> (l * LP)) + lg, res);
            }
            __syncthreads();
            if (lg < W) {
                *reinterpret_cast<float4 *>(&s_sum[lg][col]) = make_float4(res[0], res[1], res[2], res[3]);
                *reinterpret_cast<float4 *>(&s_sum[lg][col + 4]) = make_float4(res[4], res[5], res[6], res[7]);
            }
            __syncthreads();
        }
    }
}

// Level l > LT: window m sums windows m*p .. m*p+p-1 of level l-1 (those the
// level below holds; the rest cover no row), one lane group per (head, window).
template <int D>
__global__ __launch_bounds__(256) void k_scatter_bwd_up(ScatterBwdArgs a, int l)
{
    constexpr int LANES = D / 8, NLG = 256 / LANES;
    const int lane = threadIdx.x % LANES, lg = threadIdx.x / LANES, col = lane * 8;
    const int P = 1 << a.log2p;
    const int64_t below = a.part_n[l - 1], ml = (below + P - 1) / P;
    const int64_t item = (int64_t)blockIdx.x * NLG + lg;
    if (item >= (int64_t)a.H * ml)
        return;
    const int h = (int)(item / ml);
    const int64_t m = item - (int64_t)h * ml;
    const float *src = a.part + ((int64_t)h * a.part_rows + a.part_off[l - 1]) * D + col;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        acc[e] = 0.0f;
    for (int c = 0; c < P; ++c) {
        const int64_t mc = m * P + c;
        if (mc < below) {
            float x[8];
            load8(src + mc * D, x);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[e] += x[e];
        }
    }
    const int64_t i = m - 1;
    if (i >= 0 && i < (a.N >> (l * a.log2p))) {
        const int32_t sl = a.slot[(int64_t)h * a.lvl_total + a.lvl_off[l] + i];
        if ((uint32_t)sl < (uint32_t)a.S_pad)
            store8(a.dosub + ((int64_t)h * a.S_pad + sl) * D + col, acc);
    }
    if (l < a.L - 1)
        store8(a.part + ((int64_t)h * a.part_rows + a.part_off[l] + m) * D + col, acc);
}

template <int D, lh_dtype DT, int LP>
static hipError_t launch_scatter_bwd_t(const Plan &pl, const ScatterBwdArgs &a, hipStream_t s)
{
    constexpr int T = TileShape<D, LP, sbwd_nc(LP)>::T, NLG = 256 / (D / 8);
    const dim3 grid((unsigned)((pl.N + 1 + T - 1) / T), (unsigned)pl.H);
    hipLaunchKernelGGL((k_scatter_bwd<D, DT, LP>), grid, dim3(256), 0, s, a);
    for (int l = pl.LTs + 1; l < pl.L; ++l) {
        const int64_t ml = (pl.spart_n[l - 1] + pl.p - 1) / pl.p;
        const int64_t items = (int64_t)pl.H * ml;
        hipLaunchKernelGGL((k_scatter_bwd_up<D>), dim3((unsigned)((items + NLG - 1) / NLG)), dim3(256), 0, s, a, l);
    }
    return hipGetLastError();
}

template <int D, lh_dtype DT>
static hipError_t launch_scatter_bwd_p(const Plan &pl, const ScatterBwdArgs &a, hipStream_t s)
{
    switch (pl.log2p) {
    case 1: return launch_scatter_bwd_t<D, DT, 1>(pl, a, s);
    case 2: return launch_scatter_bwd_t<D, DT, 2>(pl, a, s);
    default: return launch_scatter_bwd_t<D, DT, 3>(pl, a, s);
    }
}

hipError_t launch_scatter_bwd(const Plan &pl, const ScatterBwdArgs &a, hipStream_t s)
{
    if (pl.d == 128)
        return pl.dt == LH_BF16 ? launch_scatter_bwd_p<128, LH_BF16>(pl, a, s)
                                : launch_scatter_bwd_p<128, LH_F32>(pl, a, s);
    return pl.dt == LH_BF16 ? launch_scatter_bwd_p<64, LH_BF16>(pl, a, s)
                            : launch_scatter_bwd_p<64, LH_F32>(pl, a, s);
}

// ---------------------------------------------------------------- backward prep
// fp16 pair of dO_sub (hi = fp16(x), lo = fp16(x - hi)) row-major (MFMA
// operands of the attention backward, which reads the hi part's transpose out
// of LDS), and
// delta_s = sum_d (hi + lo)[s][d] * O_sub[s][d], the row term of the softmax
// gradient, from the same values the dP products see. Rows past S are zero.
// The attention backward works with probabilities scaled by 2^15 (kept out of
// the fp16 underflow range): it reads delta_s * 2^-15 (an exact scaling) and
// the log2-domain LSE minus 15, so that one fma gives the scaled exponent.
// With bf16 inputs it also writes the e4m3 copy of the lo part (operand-order
// 32-row tiles, fixed scale kFp8Exp[3]) for the block-scaled dP products.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_prep(BwdPrepArgs a)
{
    constexpr int LANES = D / 8, NLG = 256 / LANES;
    const int h = blockIdx.y;
    const int64_t s0 = (int64_t)blockIdx.x * kPrepTile;
    const int lane = threadIdx.x % LANES, lg = threadIdx.x / LANES;
    // dO_sub is staged times 2^ex_do; delta then is 2^ex_do delta, and it is
    // kept times 2^(ex_v - 15) (as the dS products see V times 2^ex_v)
    const float sdo = ldexpf(1.0f, a.ex[3 * a.H + h]);
    const float sdelta = ldexpf(1.0f, a.ex[2 * a.H + h] - 15);
    for (int r = lg; r < kPrepTile; r += NLG) {
        const int64_t s = s0 + r;
        const int64_t off = ((int64_t)h * a.S_pad + s) * D + lane * 8;
        float x[8], o[8];
        if (s < a.S) {
            load8(a.dosub + off, x);
            load8(a.osub + off, o);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                x[e] *= sdo;
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
        if (lane == 0) {
            a.delta[(int64_t)h * a.S_pad + s] = dot * sdelta;
            a.lse15[(int64_t)h * a.S_pad + s] = s < a.S ? a.lse[(int64_t)h * a.S_pad + s] - 15.0f : 0.0f;
        }
        *reinterpret_cast<uint4 *>(a.dohi + off) = hi;
        if (a.dolo != nullptr) // fp32 inputs (bf16: the lo part as the e4m3 tile below)
            *reinterpret_cast<uint4 *>(a.dolo + off) = lo;
        if (a.dolo8 != nullptr) {
            const int64_t tile0 = ((int64_t)h * a.S_pad + (s & ~int64_t(31))) * D;
            *reinterpret_cast<uint2 *>(a.dolo8 + tile0 + fp8_tile_offset((int)(s & 31), lane)) =
                pack8_fp8(xl, ldexpf(1.0f, -kFp8Exp[3]));
        }
    }
}

// Largest dO_sub row norm of each 64-row tile of a head (rows past S are
// zero): the per-head staging scale of dO_sub is taken from them.
template <int D>
__global__ __launch_bounds__(256) void k_rowmax(RowMaxArgs a)
{
    constexpr int LANES = D / 8, NLG = 256 / LANES;
    __shared__ float s_m[4];
    const int h = blockIdx.y;
    const int64_t s0 = (int64_t)blockIdx.x * kExpTile;
    const int lane = threadIdx.x % LANES, lg = threadIdx.x / LANES;
    float m = 0.0f;
    for (int r = lg; r < kExpTile; r += NLG) {
        if (s0 + r >= a.S)
            break;
        float x[8], n2 = 0.0f;
        load8(a.src + (((int64_t)h * a.S_pad + s0 + r) * D + lane * 8), x);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            n2 = __builtin_fmaf(x[e], x[e], n2);
#pragma unroll
        for (int o = LANES / 2; o >= 1; o >>= 1) // over the row's lane group
            n2 += __shfl_xor(n2, o, LANES);
        m = fmaxf(m, n2);
    }
    m = sqrtf(m);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        m = fmaxf(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0)
        s_m[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0)
        a.dst[(int64_t)h * (a.S_pad / kExpTile) + blockIdx.x] = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
}

hipError_t launch_rowmax(const Plan &pl, const RowMaxArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)(pl.S_pad / kExpTile), pl.H);
    if (pl.d == 128)
        hipLaunchKernelGGL((k_rowmax<128>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((k_rowmax<64>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
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
hipError_t launch_pool_bwd(const Plan &pl, const PoolBwdArgs &pa, hipStream_t s)
{
    PullArgs a;
    memset(&a, 0, sizeof(a));
    for (int t = 0; t < 3; ++t) {
        a.src[t] = pa.dsub[t];
        a.dst[t] = pa.dx[t];
    }
    a.slot = pa.slot;
    a.N = pa.N; a.lvl_total = pa.lvl_total; a.S_pad = pa.S_pad;
    for (int l = 0; l < kMaxLevels; ++l)
        a.lvl_off[l] = pa.lvl_off[l];
    a.L = pa.L; a.log2p = pa.log2p; a.weighted = 1;
    return launch_pull<3, 0>(pl, a, s);
}

} // namespace lh
