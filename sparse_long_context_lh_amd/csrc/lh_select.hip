// Selection of the Lighthouse layer.
//
// k_topk: the stratified top-K of one level (aitrends summary, 핵심 기여 and
// 방법론 item 6: a chunked bitonic top-K, non-differentiable; techllm review,
// 한계와 주의할 점: stratified, every segment contributes a fixed count). One
// workgroup per (head, level, stratum of up to 2048 entries): the stratum's
// 64-bit keys (fp32 score bits << 32 | ~index, so larger score first and then
// the lower index) are sorted by a bitonic network in LDS; the quota-th
// largest key is the threshold, and a ballot compaction writes the kept
// entries in ascending index order. It also marks the children of every
// dropped parent as not gathered (slot = -1).
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

__device__ __forceinline__ uint64_t topk_key(float s, int64_t i)
{
    return ((uint64_t)__float_as_uint(s) << 32) | (uint64_t)(0xffffffffu - (uint32_t)i);
}

__global__ __launch_bounds__(1024) void k_topk(TopkArgs a)
{
    __shared__ uint64_t keys[kStratum];
    __shared__ int wave_count[16];
    const int tid = threadIdx.x;
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

    int n2 = 1;
    while (n2 < m)
        n2 <<= 1;
    for (int e = tid; e < n2; e += 1024)
        keys[e] = e < m ? topk_key(s[e], base + e) : 0ull; // pads sort below every real key
    __syncthreads();

    // Bitonic sort, ascending.
    for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int t = tid; t < (n2 >> 1); t += 1024) {
                const int i = ((t & ~(stride - 1)) << 1) | (t & (stride - 1));
                const int j = i + stride;
                const bool up = (i & size) == 0;
                const uint64_t x = keys[i], y = keys[j];
                if ((x > y) == up) {
                    keys[i] = y;
                    keys[j] = x;
                }
            }
            __syncthreads();
        }
    }
    const uint64_t thr = q > 0 ? keys[n2 - q] : ~0ull;

    // Ballot compaction in ascending index order, 1024 entries per pass.
    int32_t *sel = a.sel + ((int64_t)h * (a.L - 1) + (l - 1)) * a.k + (int64_t)c * (a.k / C) + min(c, a.k % C);
    int32_t *child_slot = a.slot + (int64_t)h * a.lvl_total + a.lvl_off[l - 1];
    const int lane = tid & 63, wave = tid >> 6;
    const int p = 1 << a.log2p;
    int done = 0;
    for (int e0 = 0; e0 < m; e0 += 1024) {
        const int e = e0 + tid;
        const bool keep = e < m && topk_key(s[e], base + e) >= thr;
        const uint64_t ball = __ballot(keep);
        if (lane == 0)
            wave_count[wave] = __popcll(ball);
        __syncthreads();
        int before = done;
        for (int w = 0; w < wave; ++w)
            before += wave_count[w];
        int total = 0;
        for (int w = 0; w < 16; ++w)
            total += wave_count[w];
        if (keep)
            sel[before + __popcll(ball & ((1ull << lane) - 1ull))] = (int32_t)(base + e);
        if (e < m && !keep)
            for (int cc = 0; cc < p; ++cc)
                child_slot[((base + e) << a.log2p) + cc] = -1;
        done += total;
        __syncthreads();
    }
}

hipError_t launch_topk(const Plan &pl, const TopkArgs &a, hipStream_t s)
{
    if (pl.L < 2 || pl.strata_total == 0)
        return hipSuccess;
    hipLaunchKernelGGL(k_topk, dim3(pl.strata_total, pl.H), dim3(1024), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------- causal order
constexpr int kIndexPerBlock = 1024;

__global__ __launch_bounds__(256) void k_index(IndexArgs a)
{
    extern __shared__ int32_t s_sel[]; // [(L-1)][k]: Sel_1 .. Sel_(L-1)
    const int h = blockIdx.y;
    const int tid = threadIdx.x;
    const int nsel = (a.L - 1) * a.k;
    for (int e = tid; e < nsel; e += 256)
        s_sel[e] = a.sel[(int64_t)h * nsel + e];
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
