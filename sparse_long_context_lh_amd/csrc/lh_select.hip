// Selection of the Lighthouse layer.
//
// k_topk: the stratified top-K of one level (aitrends summary, 핵심 기여 and
// 방법론 item 6: a chunked bitonic top-K, non-differentiable; techllm review,
// 한계와 주의할 점: stratified, every segment contributes a fixed count). One
// workgroup per (head, level, stratum of up to 2048 entries). The pages'
// kernel sorts each chunk with a bitonic network; only the quota-th largest
// key (score, then lower index) is needed, so here a radix select finds the
// quota-th largest score T a byte at a time (per-wave digit histograms in
// LDS) together with how many entries equal to T are kept, and a ballot
// compaction writes the kept entries in ascending index order. It also marks
// the children of every dropped parent as not gathered (slot = -1).
//
// k_index: the causal order of the gathered sub-sequence (techllm review,
// 어떻게 동작하나 step 3: the chosen entries are sorted into causal order).
// Entry (l, i) ends on token t = (i+1) p^l - 1; entries are ordered by t, the
// coarser first on equal t. The position of an entry is the number of
// gathered entries before it, counted level by level with a binary search in
// the sorted selections (the gathered entries of level l are the p children
// of each selected parent of level l+1; the top level is gathered whole).
#include "lh_device.h"
#include "lh_internal.h"

namespace lh {

constexpr int kTopkThreads = 256;
constexpr int kTopkPer = kStratum / kTopkThreads; // entries per thread
constexpr int kTopkWaves = kTopkThreads / 64;
static_assert(kStratum % kTopkThreads == 0, "a stratum fills whole chunks of the workgroup");

__global__ __launch_bounds__(kTopkThreads) void k_topk(TopkArgs a)
{
    constexpr int NW = kTopkWaves, U = kTopkPer;
    // per-wave digit counts (no contention across waves), two buffers: the
    // next pass's is cleared while this pass's is scanned
    __shared__ int hist[2][NW][256];
    __shared__ int s_cnt[U][NW]; // compaction: (above T) << 16 | (equal to T), per chunk and wave
    __shared__ int s_dig, s_need;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = blockIdx.y;
    int l = 1;
    while (l + 1 < a.L && (int)blockIdx.x >= a.strata_before[l + 1])
        ++l;
    const int c = blockIdx.x - a.strata_before[l];
    const int C = a.C[l];
    const int m = (int)(a.n[l] / C);
    const int q = a.k / C + (c < a.k % C ? 1 : 0);
    const int64_t base = (int64_t)c * m;
    const float *s = a.scores + (int64_t)h * a.lvl_total + a.lvl_off[l] + base;

    // Scores are non-negative, so their bit patterns order like the values.
    // Entry tid + 256 u of the stratum (chunk u, ascending index order is
    // chunk, then wave, then lane).
    uint32_t v[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int e = tid + kTopkThreads * u;
        valid[u] = e < m;
        v[u] = valid[u] ? __float_as_uint(s[e]) : 0u;
    }

    // The q-th largest score T, one byte at a time from the top (radix
    // select), and r: how many entries equal to T are kept (the lowest
    // indices among them). Together these keep exactly the q largest keys
    // (score, then lower index).
    uint32_t T = 0u;
    int r = 0;
    if (q > 0) { // (uniform)
        for (int i = tid; i < 2 * NW * 256; i += kTopkThreads)
            (&hist[0][0][0])[i] = 0;
        __syncthreads();
        uint32_t prefix = 0u, mask = 0u;
        int need = q;
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass, b = pass & 1;
            // a thread's entries with equal digits are counted together first:
            // in the first passes most entries share a digit, and LDS atomics
            // to one address serialise
            bool live[U];
            uint32_t dg[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                live[u] = valid[u] && (v[u] & mask) == prefix;
                dg[u] = (v[u] >> shift) & 255u;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (!live[u])
                    continue;
                int n = 1;
#pragma unroll
                for (int u2 = u + 1; u2 < U; ++u2)
                    if (live[u2] && dg[u2] == dg[u]) {
                        ++n;
                        live[u2] = false;
                    }
                atomicAdd(&hist[b][wave][dg[u]], n);
            }
            __syncthreads();
            if (wave == 0) {
                // lane owns digits 4 lane .. 4 lane + 3; suf = entries with a
                // digit >= 4 lane (suffix sum over lanes)
                int cnt[4], tot = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    int x = 0;
#pragma unroll
                    for (int w = 0; w < NW; ++w)
                        x += hist[b][w][4 * lane + j];
                    cnt[j] = x;
                    tot += x;
                }
                int suf = tot;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int y = __shfl_down(suf, o);
                    if (lane + o < 64)
                        suf += y;
                }
                const int above = suf - tot;
                if (above < need && need <= suf) { // the q-th largest has a digit of this lane
                    int acc = above, dsel = 0;
                    for (int j = 3; j >= 0; --j) {
                        if (acc + cnt[j] >= need) {
                            dsel = j;
                            break;
                        }
                        acc += cnt[j];
                    }
                    s_dig = 4 * lane + dsel;
                    s_need = need - acc;
                }
            } else if (pass < 3) {
                // the other buffer was last scanned before the previous barrier
                for (int i = tid - 64; i < NW * 256; i += kTopkThreads - 64)
                    (&hist[b ^ 1][0][0])[i] = 0;
            }
            __syncthreads();
            prefix |= (uint32_t)s_dig << shift;
            mask |= 255u << shift;
            need = s_need;
        }
        T = prefix;
        r = need;
    }

    // Compaction in ascending index order: every entry above T is kept, and
    // the first r entries equal to T. The kept entries before entry e are
    // (entries above T before e) + min(entries equal to T before e, r), so one
    // exchange of per-wave counts places every entry.
    uint64_t ab[U], tb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        ab[u] = __ballot(q > 0 && valid[u] && v[u] > T);
        tb[u] = __ballot(q > 0 && valid[u] && v[u] == T);
        if (lane == 0)
            s_cnt[u][wave] = (__popcll(ab[u]) << 16) | __popcll(tb[u]);
    }
    __syncthreads();
    // selections are stored level-major, [L-1][H][k]
    int32_t *sel = a.sel + ((int64_t)(l - 1) * gridDim.y + h) * a.k + (int64_t)c * (a.k / C) + min(c, a.k % C);
    int32_t *child_slot = a.slot + (int64_t)h * a.lvl_total + a.lvl_off[l - 1];
    const int p = 1 << a.log2p;
    const uint64_t lt = (1ull << lane) - 1ull;
    int run = 0; // packed counts of every (chunk, wave) before this wave's part of chunk u
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int pre = run;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int x = s_cnt[u][w];
            pre += w < wave ? x : 0;
            run += x;
        }
        const int above_before = (pre >> 16) + __popcll(ab[u] & lt);
        const int ties_before = (pre & 0xffff) + __popcll(tb[u] & lt);
        const bool keep = ((ab[u] >> lane) & 1ull) || (((tb[u] >> lane) & 1ull) && ties_before < r);
        const int e = tid + kTopkThreads * u;
        const int pos = above_before + min(ties_before, r); // < q for a kept entry
        if (keep && pos < q)
            sel[pos] = (int32_t)(base + e);
        if (valid[u] && !keep)
            for (int cc = 0; cc < p; ++cc)
                child_slot[((base + e) << a.log2p) + cc] = -1;
    }
}

hipError_t launch_topk(const Plan &pl, const TopkArgs &a, hipStream_t s)
{
    if (pl.L < 2 || pl.strata_total == 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_topk, dim3(pl.strata_total, pl.H), dim3(kTopkThreads), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- causal order
// one position per thread: at 10K-20K positions per head the grid still fills the chip
constexpr int kIndexPerBlock = 256;

__global__ __launch_bounds__(256) void k_index(IndexArgs a)
{
    extern __shared__ int32_t s_sel[]; // [(L-1)][k]: Sel_1 .. Sel_(L-1)
    const int h = blockIdx.y;
    const int tid = threadIdx.x;
    const int nsel = (a.L - 1) * a.k;
    for (int e = tid; e < nsel; e += 256) { // level row r = e / k of the [L-1][H][k] selections
        const int r = e / a.k;
        s_sel[e] = a.sel[((int64_t)r * gridDim.y + h) * a.k + (e - r * a.k)];
    }
    __syncthreads();

    const int L = a.L, k = a.k, log2p = a.log2p;
    const int64_t pmask = (int64_t(1) << log2p) - 1;
    const int64_t n_top = a.n[L - 1];
    const int64_t pk = (int64_t)k << log2p;
    int32_t *slot = a.slot + (int64_t)h * a.lvl_total;
    int32_t *ent = a.ent + (int64_t)h * a.S_pad;
    const int64_t g_end = min((int64_t)(blockIdx.x + 1) * kIndexPerBlock, a.S_pad);
    for (int64_t g = (int64_t)blockIdx.x * kIndexPerBlock + tid; g < g_end; g += 256) {
        if (g >= a.S) {
            ent[g] = -1;
            continue;
        }
        int l;
        int64_t i, rank;
        if (g < n_top) {
            l = L - 1;
            i = g;
            rank = g;
        } else {
            const int64_t gg = g - n_top;
            l = (int)(gg / pk);
            rank = gg - (int64_t)l * pk;
            // children of the j-th selected parent of level l+1 (Sel_(l+1) is row l)
            i = ((int64_t)s_sel[l * k + (rank >> log2p)] << log2p) + (rank & pmask);
        }
        const int64_t e = (i + 1) << (l * log2p); // last covered token + 1
        int64_t pos = rank;                       // gathered entries of level l before i
        for (int lp = 0; lp < L; ++lp) {
            if (lp == l)
                continue;
            // coarser levels count entries ending on or before t, finer levels strictly before
            const int64_t X = lp > l ? (e >> (lp * log2p)) : ((e - 1) >> (lp * log2p));
            if (lp == L - 1) {
                pos += min(X, n_top);
            } else {
                const int32_t *sl = s_sel + lp * k;
                const int64_t A = X >> log2p;
                int lo = 0, hi = k;
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if ((int64_t)sl[mid] < A)
                        lo = mid + 1;
                    else
                        hi = mid;
                }
                pos += ((int64_t)lo << log2p) + ((lo < k && (int64_t)sl[lo] == A) ? (X & pmask) : 0);
            }
        }
        slot[a.lvl_off[l] + i] = (int32_t)pos;
        if (pos >= 0 && pos < a.S)
            ent[pos] = (int32_t)((i << 3) | l);
    }
}

hipError_t launch_index(const Plan &pl, const IndexArgs &a, hipStream_t s)
{
    const unsigned blocks = (unsigned)((pl.S_pad + kIndexPerBlock - 1) / kIndexPerBlock);
    const size_t lds = sizeof(int32_t) * (size_t)(pl.L - 1) * pl.k;
    hipLaunchKernelGGL(k_index, dim3(blocks, pl.H), dim3(256), lds, s, a);
    return hipGetLastError();
}

} // namespace lh
