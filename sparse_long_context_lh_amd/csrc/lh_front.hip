// Front pass of the Lighthouse layer: one streaming read of Q, K and V that
// produces
//   * the token scores s_j = sqrt(||q_j||^2) + sqrt(||k_j||^2) (fp32, fixed
//     order; aitrends summary, 기술 상세 item 2) — or a variant built from the
//     same two roots (their product, either one alone; aitrends summary, 핵심
//     기여: query/key l2-norm scores of more than one kind) — and their
//     max-pooled values at every coarser level (same passage: coarser levels
//     receive the score by max-pooling);
//   * the average-pooled rows (aitrends summary, 기술 상세 item 1; techllm
//     review, 어떻게 동작하나 step 1) of the levels the host chose to
//     materialise, as fp32 means of an fp32 sum (no rounding to 16 bits, so
//     the attention sees pooled rows at full precision).
//
// Work split: a "lane group" of d/8 lanes owns a row, each lane holding 8
// consecutive elements (16 B of bf16 or 32 B of fp32). A lane group loads a
// run of R = p^c rows at once (all loads in flight together), computes their
// scores, and sums its run level by level in registers: a level-l window sum
// is the sum of its p level-(l-1) window sums in ascending order, starting
// from 0 (the same tree at every level, so the pooled values do not depend on
// the tiling). A wave's lane groups hold consecutive runs: each wave finishes
// the levels whose windows fit in its rows, and wave 0 those spanning the
// workgroup's tile. Each coarser level is one small kernel over the level
// below: its pooled means times p^l where that level is materialised, else
// the window sums the tile kernel kept for it. No atomics; each input byte is
// read once.
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

// The token score from the two squared norms: both roots correctly rounded,
// then combined in fp32 as `scorer` says (uniform over the launch).
__device__ __forceinline__ float token_score(int scorer, float nq2, float nk2)
{
    const float nq = sqrtf(nq2), nk = sqrtf(nk2);
    switch (scorer) {
    case LH_SCORE_PRODUCT: return nq * nk;
    case LH_SCORE_QUERY: return nq;
    case LH_SCORE_KEY: return nk;
    default: return nq + nk;
    }
}

constexpr int ipow(int b, int e) { return e == 0 ? 1 : b * ipow(b, e - 1); }

template <int D, lh_dtype DT, int LP>
__global__ __launch_bounds__(256) void k_front(FrontArgs a)
{
    typedef typename Elem<DT>::T T;
    typedef TileShape<D, LP, front_nc(LP)> Sh;
    constexpr int LANES = Sh::LANES, NLG = Sh::NLG, NC = Sh::NC, R = Sh::R, P = 1 << LP;
    __shared__ __attribute__((aligned(16))) float s_sum[3][NLG][D];
    // scores of the tile, level after level (T / p^l each): written to memory
    // at the end as whole lines
    __shared__ float s_sc[2 * Sh::T];
    const int lane = threadIdx.x % LANES, lg = threadIdx.x / LANES, col = lane * 8;
    const int h = blockIdx.y;
    const int64_t x0 = (int64_t)blockIdx.x * Sh::T;
    const int64_t j0 = x0 + (int64_t)lg * R;
    const int LT = a.LT;
    const bool keep = LT < a.L - 1; // level LT's window sums feed the next level's kernel
    float *sc = a.scores + (int64_t)h * a.lvl_total;
    float *pooled = a.pooled + (int64_t)h * a.mat_rows * D + col;
    const int64_t pstride = (int64_t)a.H * a.part_rows * D;
    float *part = a.part + (int64_t)h * a.part_rows * D + col;
    float *pmax = a.part + 3 * pstride + (int64_t)h * a.part_rows;

    // A finished level-l window i (i < n_l, l <= LT): the pooled mean of a
    // materialised level, and the sum itself when level LT feeds coarser ones
    // and is not materialised (else the next level reads the means: mean *
    // p^l is the sum, exactly, the scale being a power of two).
    auto put_sum = [&](int t, int l, int64_t i, const float (&acc)[8]) {
        if (a.mat_off[l] >= 0) {
            const float w = 1.0f / (float)(1 << (l * LP)); // exact: power of two
            float m8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                m8[e] = acc[e] * w;
            store8(pooled + t * a.tensor_stride + (a.mat_off[l] + i) * D, m8);
        }
        if (keep && l == LT && a.mat_off[l] < 0)
            store8(part + t * pstride + (a.part_off[l] + i) * D, acc);
    };

    const int64_t in_off = ((int64_t)h * a.N + j0) * D + col;
    const T *qp = reinterpret_cast<const T *>(a.q) + in_off;
    const T *kp = reinterpret_cast<const T *>(a.k) + in_off;
    const T *vp = reinterpret_cast<const T *>(a.v) + in_off;
    Raw8<DT> rq[R], rk[R], rv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (j0 + r < a.N) {
            ld_raw(qp + r * D, rq[r]);
            ld_raw(kp + r * D, rk[r]);
            ld_raw(vp + r * D, rv[r]);
        } else {
            zero_raw(rq[r]);
            zero_raw(rk[r]);
            zero_raw(rv[r]);
        }
    }

    // largest |q| and |k| element and largest v row norm of this wave's rows
    // (the per-head fp16 staging scales of the gather are taken from them)
    {
        float mx[3] = {0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float x[8];
            unraw(rq[r], x);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                mx[0] = fmaxf(mx[0], fabsf(x[e]));
            unraw(rk[r], x);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                mx[1] = fmaxf(mx[1], fabsf(x[e]));
            unraw(rv[r], x);
            mx[2] = fmaxf(mx[2], row_norm2<LANES>(x));
        }
        mx[2] = sqrtf(mx[2]);
#pragma unroll
        for (int t = 0; t < 3; ++t) {
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1)
                mx[t] = fmaxf(mx[t], __shfl_xor(mx[t], o));
        }
        if ((threadIdx.x & 63) == 0) {
#pragma unroll
            for (int t = 0; t < 3; ++t)
                a.xmax[((int64_t)t * a.H + h) * a.nxmax + (int64_t)blockIdx.x * 4 + threadIdx.x / 64] = mx[t];
        }
    }

    // token scores, then their maxima over the run's windows
    float s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float x[8];
        unraw(rq[r], x);
        const float nq = row_norm2<LANES>(x);
        unraw(rk[r], x);
        const float nk = row_norm2<LANES>(x);
        s[r] = token_score(a.scorer, nq, nk);
    }

    // window sums of the run, tensor after tensor
    float tot[3][8];
    auto cascade = [&](int t, const Raw8<DT> (&rows)[R]) {
        float acc[NC][8];
#pragma unroll
        for (int l = 0; l < NC; ++l)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[l][e] = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float x[8];
            unraw(rows[r], x);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[0][e] += x[e];
#pragma unroll
            for (int l = 1; l <= NC; ++l) {
                if ((r + 1) % ipow(P, l) == 0) {
                    const int64_t i = (j0 >> (l * LP)) + (r + 1) / ipow(P, l) - 1;
                    if (l <= LT && i < (a.N >> (l * LP)))
                        put_sum(t, l, i, acc[l - 1]);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if (l < NC)
                            acc[l < NC ? l : 0][e] += acc[l - 1][e];
                        else
                            tot[t][e] = acc[l - 1][e];
                        acc[l - 1][e] = 0.0f;
                    }
                }
            }
        }
    };
    cascade(0, rq);
    cascade(1, rk);
    cascade(2, rv);

    // Levels NC+1 .. LT. A wave's G lane groups hold G consecutive runs, so
    // every level whose windows fit in G runs is finished by that wave alone,
    // in its own rows of LDS (ordered by LDS waits, no workgroup barrier);
    // after one barrier (LDS only: stores in flight are not waited for), wave
    // 0 finishes the levels whose windows span waves. Window sums are the
    // ascending sums of their p children from 0, window scores the maxima of
    // their children (exact, order-free).
    constexpr int G = 64 / LANES;     // lane groups (runs) per wave
    constexpr int WL = clog2(G) / LP; // levels above NC whose windows fit in a wave
    const int wave = threadIdx.x / 64, gl = lg % G, l64 = threadIdx.x & 63;
    auto lds_wave_sync = [] { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); };
    // level-l scores of the tile, in tile order, from s_sc[sb(l)] (T / p^l of them)
    auto sb = [&](int l) {
        int b = 0;
        for (int q = 0; q < l; ++q)
            b += Sh::T >> (q * LP);
        return b;
    };
    auto put_score = [&](int l, int e) {
        const int64_t i = (x0 >> (l * LP)) + e;
        if (i < (a.N >> (l * LP))) {
            const float m = s_sc[sb(l) + e];
            sc[a.lvl_off[l] + i] = m;
            if (keep && l == LT)
                pmax[a.part_off[l] + i] = m;
        }
    };
    // Window sums of level l: W windows, child c of window w at row
    // crow(w P + c) of s_sum, the result to row w0 + w and to memory as window
    // i0 + w of the level; the 3 W (tensor, window) tasks are shared out over
    // nslots lane groups (this one is slot). Reads complete before any write.
    auto sum_level = [&](int l, int W, int i0, int w0, int cbase, int cper, int slot, int nslots) {
        auto crow = [&](int g) { return cbase + (g / cper) * G + g % cper; };
        float res[2][8];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int task = slot + n * nslots;
            if (task < 3 * W) {
                const int t = task / W, w = task - t * W;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    res[n][e] = 0.0f;
                for (int c = 0; c < P; ++c) {
                    const int row = crow(w * P + c);
                    const float4 lo = *reinterpret_cast<const float4 *>(&s_sum[t][row][col]);
                    const float4 hi = *reinterpret_cast<const float4 *>(&s_sum[t][row][col + 4]);
                    res[n][0] += lo.x; res[n][1] += lo.y; res[n][2] += lo.z; res[n][3] += lo.w;
                    res[n][4] += hi.x; res[n][5] += hi.y; res[n][6] += hi.z; res[n][7] += hi.w;
                }
                const int64_t i = (x0 >> (l * LP)) + i0 + w;
                if (i < (a.N >> (l * LP)))
                    put_sum(t, l, i, res[n]);
            }
        }
        lds_wave_sync();
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            const int task = slot + n * nslots;
            if (task < 3 * W) {
                const int t = task / W, w = task - t * W;
                *reinterpret_cast<float4 *>(&s_sum[t][w0 + w][col]) = make_float4(res[n][0], res[n][1], res[n][2], res[n][3]);
                *reinterpret_cast<float4 *>(&s_sum[t][w0 + w][col + 4]) = make_float4(res[n][4], res[n][5], res[n][6], res[n][7]);
            }
        }
        lds_wave_sync();
    };
    // Window scores of level l: entries e0 .. e0 + cnt - 1 (tile order), one
    // per lane of this wave, from level l-1; stored to memory as well.
    auto score_level = [&](int l, int e0, int cnt) {
        if (l64 < cnt) {
            const int e = e0 + l64;
            const float *c = &s_sc[sb(l - 1) + e * P];
            float m = c[0];
#pragma unroll
            for (int q = 1; q < P; ++q)
                m = fmaxf(m, c[q]);
            s_sc[sb(l) + e] = m;
        }
        lds_wave_sync();
        if (l64 < cnt)
            put_score(l, e0 + l64);
    };

    // levels 0 .. NC of the scores: lane e of a run stages entry e of each
    // level (the maxima over the run's windows, in registers)
    {
        float m[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
            m[r] = s[r];
        int cnt = R;
#pragma unroll
        for (int l = 0; l <= NC; ++l) {
            if (l > 0) {
                cnt /= P;
#pragma unroll
                for (int e = 0; e < R / P; ++e)
                    if (e < cnt) {
                        float x = m[e * P];
#pragma unroll
                        for (int c = 1; c < P; ++c)
                            x = fmaxf(x, m[e * P + c]);
                        m[e] = x;
                    }
            }
#pragma unroll
            for (int e = 0; e < R; ++e)
                if (e < cnt && lane == e)
                    s_sc[sb(l) + lg * cnt + e] = m[e];
        }
    }
    if (LT > NC) { // the runs' totals of level NC, one row per lane group
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            *reinterpret_cast<float4 *>(&s_sum[t][lg][col]) = make_float4(tot[t][0], tot[t][1], tot[t][2], tot[t][3]);
            *reinterpret_cast<float4 *>(&s_sum[t][lg][col + 4]) = make_float4(tot[t][4], tot[t][5], tot[t][6], tot[t][7]);
        }
    }
    lds_wave_sync();
    for (int l = 0; l <= NC && l <= LT; ++l) { // this wave's entries of levels 0 .. NC
        const int cnt = (G * R) >> (l * LP);
        if (l64 < cnt)
            put_score(l, wave * cnt + l64);
    }
    // levels inside a wave
    int W = G; // windows of the level below in this wave
    const int lw = LT < NC + WL ? LT : NC + WL;
    for (int l = NC + 1; l <= lw; ++l) {
        W /= P;
        sum_level(l, W, wave * W, wave * G, wave * G, 1 << 30, gl, G);
        score_level(l, wave * W, W);
    }
    // levels spanning waves: wave 0, after one barrier
    if (LT > NC + WL) {
        lds_barrier();
        if (wave == 0) {
            int cper = W; // windows per wave at the level below (rows wave * G + w)
            int Wt = W * 4;
            for (int l = NC + WL + 1; l <= LT; ++l) {
                Wt /= P;
                sum_level(l, Wt, 0, 0, 0, cper, gl, G);
                score_level(l, 0, Wt);
                cper = 1 << 30; // from here on in rows 0 .. Wt - 1
            }
        }
    }
}

// Level l > LT: window i sums the p windows i*p .. i*p+p-1 of level l-1
// (ascending, from 0), one lane group per (head, window). The sums of level
// l-1 are its kept window sums, or, for a materialised level, its pooled
// means times p^(l-1) (exact: a power of two, barring subnormal means).
template <int D>
__global__ __launch_bounds__(256) void k_front_up(FrontArgs a, int l)
{
    constexpr int LANES = D / 8, NLG = 256 / LANES;
    const int lane = threadIdx.x % LANES, lg = threadIdx.x / LANES, col = lane * 8;
    const int64_t nl = a.N >> (l * a.log2p);
    const int64_t item = (int64_t)blockIdx.x * NLG + lg;
    if (item >= (int64_t)a.H * nl)
        return;
    const int h = (int)(item / nl);
    const int64_t i = item - (int64_t)h * nl;
    const int P = 1 << a.log2p;
    const bool keep = l < a.L - 1;
    const int64_t pstride = (int64_t)a.H * a.part_rows * D;
    const bool from_mean = a.mat_off[l - 1] >= 0;
    const float up = (float)(1 << ((l - 1) * a.log2p));
    const float *src = from_mean ? a.pooled + ((int64_t)h * a.mat_rows + a.mat_off[l - 1] + i * P) * D + col
                                 : a.part + ((int64_t)h * a.part_rows + a.part_off[l - 1] + i * P) * D + col;
    const int64_t sstride = from_mean ? a.tensor_stride : pstride;
#pragma unroll
    for (int t = 0; t < 3; ++t) {
        float acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[e] = 0.0f;
        for (int c = 0; c < P; ++c) {
            float x[8];
            load8(src + t * sstride + c * D, x);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[e] += from_mean ? x[e] * up : x[e];
        }
        if (a.mat_off[l] >= 0) {
            const float w = 1.0f / (float)(1 << (l * a.log2p)); // exact: power of two
            float m8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                m8[e] = acc[e] * w;
            store8(a.pooled + t * a.tensor_stride + ((int64_t)h * a.mat_rows + a.mat_off[l] + i) * D + col, m8);
        }
        if (keep && a.mat_off[l] < 0)
            store8(a.part + t * pstride + ((int64_t)h * a.part_rows + a.part_off[l] + i) * D + col, acc);
    }
    if (lane == 0) {
        const float *pm = a.part + 3 * pstride + (int64_t)h * a.part_rows + a.part_off[l - 1] + i * P;
        float m = pm[0];
        for (int c = 1; c < P; ++c)
            m = fmaxf(m, pm[c]);
        a.scores[(int64_t)h * a.lvl_total + a.lvl_off[l] + i] = m;
        if (keep)
            a.part[3 * pstride + (int64_t)h * a.part_rows + a.part_off[l] + i] = m;
    }
}

template <int D, lh_dtype DT, int LP>
static hipError_t launch_front_t(const Plan &pl, const FrontArgs &a, hipStream_t s)
{
    constexpr int T = TileShape<D, LP, front_nc(LP)>::T;
    const dim3 grid((unsigned)((pl.N + T - 1) / T), (unsigned)pl.H);
    hipLaunchKernelGGL((k_front<D, DT, LP>), grid, dim3(256), 0, s, a);
    constexpr int NLG = 256 / (D / 8);
    for (int l = pl.LT + 1; l < pl.L; ++l) {
        const int64_t items = (int64_t)pl.H * pl.n[l];
        hipLaunchKernelGGL((k_front_up<D>), dim3((unsigned)((items + NLG - 1) / NLG)), dim3(256), 0, s, a, l);
    }
    return hipGetLastError();
}

template <int D, lh_dtype DT>
static hipError_t launch_front_p(const Plan &pl, const FrontArgs &a, hipStream_t s)
{
    switch (pl.log2p) {
    case 1: return launch_front_t<D, DT, 1>(pl, a, s);
    case 2: return launch_front_t<D, DT, 2>(pl, a, s);
    default: return launch_front_t<D, DT, 3>(pl, a, s);
    }
}

hipError_t launch_front(const Plan &pl, const FrontArgs &a, hipStream_t s)
{
    if (pl.d == 128)
        return pl.dt == LH_BF16 ? launch_front_p<128, LH_BF16>(pl, a, s) : launch_front_p<128, LH_F32>(pl, a, s);
    return pl.dt == LH_BF16 ? launch_front_p<64, LH_BF16>(pl, a, s) : launch_front_p<64, LH_F32>(pl, a, s);
}

// ---------------------------------------------------------------- fp16 staging scales
// Largest |q| and |k| element and v row norm of each wave's rows when the
// front pass does not run (L = 1), in the front pass's layout: tile T rows
// per workgroup, one value per wave.
template <int D, lh_dtype DT>
__global__ __launch_bounds__(256) void k_absmax(AbsMaxArgs a)
{
    typedef typename Elem<DT>::T T;
    constexpr int LANES = D / 8, G = 64 / LANES; // lane groups per wave
    const int lane = threadIdx.x % LANES, wave = threadIdx.x / 64, gw = (threadIdx.x % 64) / LANES;
    const int h = blockIdx.y;
    const int64_t r0 = (int64_t)blockIdx.x * a.tile, rows = a.tile / 4; // each wave a quarter of the tile
    float mx[3] = {0.0f, 0.0f, 0.0f};
    for (int64_t r = r0 + wave * rows + gw; r < min(r0 + (wave + 1) * rows, a.N); r += G) {
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            Raw8<DT> raw;
            ld_raw(reinterpret_cast<const T *>(a.x[t]) + ((int64_t)h * a.N + r) * D + lane * 8, raw);
            float x[8];
            unraw(raw, x);
            if (t < 2) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    mx[t] = fmaxf(mx[t], fabsf(x[e]));
            } else {
                mx[2] = fmaxf(mx[2], row_norm2<LANES>(x));
            }
        }
    }
    mx[2] = sqrtf(mx[2]);
#pragma unroll
    for (int t = 0; t < 3; ++t) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            mx[t] = fmaxf(mx[t], __shfl_xor(mx[t], o));
    }
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
        for (int t = 0; t < 3; ++t)
            a.xmax[((int64_t)t * a.H + h) * a.nxmax + (int64_t)blockIdx.x * 4 + wave] = mx[t];
    }
}

hipError_t launch_absmax(const Plan &pl, const AbsMaxArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)(pl.nxmax / 4), (unsigned)pl.H);
    if (pl.d == 128) {
        if (pl.dt == LH_BF16)
            hipLaunchKernelGGL((k_absmax<128, LH_BF16>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((k_absmax<128, LH_F32>), grid, dim3(256), 0, s, a);
    } else {
        if (pl.dt == LH_BF16)
            hipLaunchKernelGGL((k_absmax<64, LH_BF16>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((k_absmax<64, LH_F32>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

// Exponent e of a head's staging scale 2^e: the head's largest magnitude m
// times 2^e lies in [2^(t-1), 2^t) (frexp: m = f 2^E, f in [0.5, 1), so
// e = t - E); 0 for a head that is all zeros. One workgroup per (head,
// tensor), four independent maxima per thread so the loads stay in flight.
__global__ __launch_bounds__(1024) void k_head_exp(HeadExpArgs a)
{
    __shared__ float s_m[16];
    const int h = blockIdx.x, t = blockIdx.y, tid = threadIdx.x;
    const float *m = a.m + ((int64_t)t * a.H + h) * a.count;
    float x[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int64_t i = tid;
    for (; i + 3 * 1024 < a.count; i += 4 * 1024) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            x[u] = fmaxf(x[u], m[i + u * 1024]);
    }
    for (; i < a.count; i += 1024)
        x[0] = fmaxf(x[0], m[i]);
    float y = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        y = fmaxf(y, __shfl_xor(y, o));
    if ((tid & 63) == 0)
        s_m[tid >> 6] = y;
    __syncthreads();
    if (tid == 0) {
        float mm = s_m[0];
        for (int w = 1; w < 16; ++w)
            mm = fmaxf(mm, s_m[w]);
        int e = 0;
        if (mm > 0.0f && mm <= 3.0e38f) {
            int E;
            frexpf(mm, &E);
            e = kExpTarget[a.first + t] - E;
            e = e < -96 ? -96 : (e > 96 ? 96 : e);
        }
        a.ex[(a.first + t) * a.H + h] = e;
    }
}

hipError_t launch_head_exp(const HeadExpArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL(k_head_exp, dim3((unsigned)a.H, (unsigned)a.nt), dim3(1024), 0, s, a);
    return hipGetLastError();
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
