// Gather of the Lighthouse sub-sequence (aitrends summary, 핵심 기여 and
// 기술 상세 item 3: the chosen (Q, K, V) triples form one contiguous
// sub-sequence of S entries).
//
// One workgroup per 64 consecutive positions of one head. For position s it
// reads the entry (l, i) the index kernel placed there and fetches its
// pooled rows: level 0 is the input row itself; a materialised level is
// copied from the front pass (fp32); any other level is averaged here from
// its p^l input rows (fp32 sum). Rows go out as fp16, the layouts the
// attention kernels read as MFMA operands: queries and keys as an fp16 pair
// (hi = fp16(x), lo = fp16(x - hi)) so the logits keep about 22 bits of the
// pooled value, values as one fp16; row-major [S_pad][d] and, through an LDS
// tile, the hi parts transposed [d][S_pad]. Positions past S are zero. Every
// row is staged times its head's power-of-two scale 2^ex (see kExpTarget), so
// that no input scale overflows fp16; the attention kernels undo it.
#include "lh_device.h"
#include "lh_internal.h"

namespace lh {

constexpr int kGatherTile = 64;

template <int D, lh_dtype DT>
__global__ __launch_bounds__(256) void k_gather(GatherArgs a)
{
    typedef typename Elem<DT>::T T;
    constexpr int LANES = D / 8;
    constexpr int NLG = 256 / LANES;
    constexpr int LD = D + 8; // LDS row pitch in bf16 (16 B pad)
    constexpr int CHUNK = 4;  // window rows in flight per tensor
    constexpr int NR = kGatherTile / NLG; // rows per lane group
    constexpr bool F8 = DT == LH_BF16;    // fp8 tiles for the lo products (see lh_device.h)
    __shared__ __attribute__((aligned(16))) uint16_t tile[3][kGatherTile * LD];
    __shared__ int32_t s_ent[kGatherTile];
    __shared__ uint32_t s_amax[3][2]; // [Q lo, K hi, V][32-row tile]: largest magnitude (fp32 bits)
    const int h = blockIdx.y;
    const int64_t s0 = (int64_t)blockIdx.x * kGatherTile;
    const int lane = threadIdx.x % LANES;
    const int lg = threadIdx.x / LANES;
    const T *src[3] = {reinterpret_cast<const T *>(a.q), reinterpret_cast<const T *>(a.k),
                       reinterpret_cast<const T *>(a.v)};
    if (threadIdx.x < kGatherTile)
        s_ent[threadIdx.x] = a.ent[(int64_t)h * a.S_pad + s0 + threadIdx.x];
    if (threadIdx.x < 6)
        s_amax[threadIdx.x >> 1][threadIdx.x & 1] = 0u;
    __syncthreads();

#pragma unroll
    for (int ri = 0; ri < NR; ++ri) {
        const int r = lg + NLG * ri;
        const int64_t s = s0 + r;
        const int32_t en = s_ent[r];
        float x[3][8];
#pragma unroll
        for (int t = 0; t < 3; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                x[t][e] = 0.0f;
        // an entry outside the pyramid (never produced by the index kernel) reads as zeros
        const bool valid = en >= 0 && (en & 7) < a.L && (int64_t)(en >> 3) < a.n[en & 7];
        const int l = en & 7;
        const int64_t i = (int64_t)(en >> 3);
        if (valid && l > 0 && a.mat_off[l] >= 0) {
#pragma unroll
            for (int t = 0; t < 3; ++t)
                load8(a.pooled + t * a.tensor_stride + ((int64_t)h * a.mat_rows + a.mat_off[l] + i) * D + lane * 8,
                      x[t]);
        } else if (valid) {
            // level 0: the input row; other levels: the mean of the p^l input
            // rows, summed in ascending order from 0 (CHUNK rows per round trip)
            const int sh = l * a.log2p;
            const int w = 1 << sh;
            const int64_t row0 = ((int64_t)h * a.N + (i << sh)) * D + lane * 8;
            for (int j = 0; j < w; j += CHUNK) {
                Raw8<DT> y[3][CHUNK];
#pragma unroll
                for (int u = 0; u < CHUNK; ++u)
#pragma unroll
                    for (int t = 0; t < 3; ++t) {
                        if (j + u < w)
                            ld_raw(src[t] + row0 + (int64_t)(j + u) * D, y[t][u]);
                        else
                            zero_raw(y[t][u]);
                    }
#pragma unroll
                for (int u = 0; u < CHUNK; ++u)
#pragma unroll
                    for (int t = 0; t < 3; ++t) {
                        float z[8];
                        unraw(y[t][u], z);
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            x[t][e] += z[e];
                    }
            }
            if (l > 0) {
                const float inv = 1.0f / (float)w; // exact: power of two
#pragma unroll
                for (int t = 0; t < 3; ++t)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        x[t][e] *= inv;
            }
        }
        const int64_t off = ((int64_t)h * a.S_pad + s) * D + lane * 8;
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const float sc = ldexpf(1.0f, a.ex[t * a.H + h]); // exact: a power of two
#pragma unroll
            for (int e = 0; e < 8; ++e)
                x[t][e] *= sc;
            uint4 hi, lo;
            if (t < 2) {
                split8_f16(x[t], hi, lo);
                *reinterpret_cast<uint4 *>(a.lo[t] + off) = lo;
            } else {
                hi = pack8_f16(x[t]);
            }
            if constexpr (F8) { // largest magnitude of the fp16 lo part of Q, of K hi and of V
                float v8[8], m8 = 0.0f;
                unpack8_f16(t == 0 ? lo : hi, v8);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    m8 = fmaxf(m8, fabsf(v8[e]));
#pragma unroll
                for (int o = LANES / 2; o >= 1; o >>= 1) // over the row's lane group
                    m8 = fmaxf(m8, __shfl_xor(m8, o, LANES));
                if (lane == 0 && m8 > 0.0f) // (32-row tile NLG * ri / 32 of row r)
                    atomicMax(&s_amax[t][NLG * ri / 32], __float_as_uint(m8));
            }
            *reinterpret_cast<uint4 *>(a.hi[t] + off) = hi;
            *reinterpret_cast<uint4 *>(&tile[t][r * LD + lane * 8]) = hi;
        }
    }
    __syncthreads();

    // per 32-row tile maxima for the fp8 copies (bf16 inputs; k_lo8 below)
    if (F8 && threadIdx.x < 6)
        a.tmax[threadIdx.x >> 1][(int64_t)h * (a.S_pad / 32) + s0 / 32 + (threadIdx.x & 1)] =
            __uint_as_float(s_amax[threadIdx.x >> 1][threadIdx.x & 1]);

    // Transposed copy: 8 consecutive positions of one dimension per 16-byte store.
    constexpr int CH = kGatherTile / 8;
    for (int c = threadIdx.x; c < 3 * D * CH; c += 256) {
        const int t = c / (D * CH);
        const int rem = c - t * D * CH;
        const int dim = rem / CH;
        const int sc = rem - dim * CH;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t lo = tile[t][(sc * 8 + 2 * e) * LD + dim];
            const uint32_t hi = tile[t][(sc * 8 + 2 * e + 1) * LD + dim];
            w[e] = lo | (hi << 16);
        }
        *reinterpret_cast<uint4 *>(a.hi_t[t] + ((int64_t)h * D + dim) * a.S_pad + s0 + sc * 8) =
            make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// fp8 copies of two fp16 tensors for the block-scaled lo products (bf16
// inputs; see lh_device.h): the gathered Q lo part and K hi part (logits), or
// the dO_sub lo part and V (dP). One scale per head and tensor, from the
// largest magnitude over the head's tile maxima; tiles of 32 rows in operand
// order. One workgroup per 32-row tile of a head.
template <int D, int WHICH> // (0: Q lo / K hi for the logits, 1: dO lo / V for dP; the same work)
__global__ __launch_bounds__(256) void k_lo8(Lo8Args a)
{
    __shared__ float s_m[2][4];
    const int h = blockIdx.y, tile = blockIdx.x, tid = threadIdx.x;
    const int ntile = (int)(a.S_pad / 32);
    float m[2] = {0.0f, 0.0f};
    for (int i = tid; i < ntile; i += 256)
#pragma unroll
        for (int t = 0; t < 2; ++t)
            m[t] = fmaxf(m[t], a.tmax[t][(int64_t)h * ntile + i]);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1)
            m[t] = fmaxf(m[t], __shfl_xor(m[t], o));
        if ((tid & 63) == 0)
            s_m[t][tid >> 6] = m[t];
    }
    __syncthreads();
    int ex[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
        ex[t] = fp8_scale_exp(fmaxf(fmaxf(s_m[t][0], s_m[t][1]), fmaxf(s_m[t][2], s_m[t][3])));
    if (tile == 0 && tid < 2)
        a.sc[tid][h] = 127 + ex[tid]; // every tile computes the same value
    // 32 rows x D elements of each tensor, 8 elements per thread and step
    constexpr int CH = D / 8;
    for (int c = tid; c < 32 * CH; c += 256) {
        const int rr = c / CH, ch = c % CH;
        const int64_t row = (int64_t)h * a.S_pad + 32 * tile + rr;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            float v8[8];
            unpack8_f16(*reinterpret_cast<const uint4 *>(a.src[t] + row * D + 8 * ch), v8);
            uint8_t *tb = a.dst[t] + ((int64_t)h * a.S_pad + 32 * tile) * D;
            *reinterpret_cast<uint2 *>(tb + fp8_tile_offset(rr, ch)) = pack8_fp8(v8, ldexpf(1.0f, -ex[t]));
        }
    }
}

hipError_t launch_lo8(const Plan &pl, const Lo8Args &a, int which, hipStream_t s)
{
    const dim3 grid((unsigned)(pl.S_pad / 32), pl.H);
    if (pl.d == 128) {
        if (which == 0)
            hipLaunchKernelGGL((k_lo8<128, 0>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((k_lo8<128, 1>), grid, dim3(256), 0, s, a);
    } else {
        if (which == 0)
            hipLaunchKernelGGL((k_lo8<64, 0>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((k_lo8<64, 1>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_gather(const Plan &pl, const GatherArgs &a, hipStream_t s)
{
    const dim3 grid((unsigned)(pl.S_pad / kGatherTile), pl.H);
    if (pl.d == 128) {
        if (pl.dt == LH_BF16)
            hipLaunchKernelGGL((k_gather<128, LH_BF16>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((k_gather<128, LH_F32>), grid, dim3(256), 0, s, a);
    } else {
        if (pl.dt == LH_BF16)
            hipLaunchKernelGGL((k_gather<64, LH_BF16>), grid, dim3(256), 0, s, a);
        else
            hipLaunchKernelGGL((k_gather<64, LH_F32>), grid, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

} // namespace lh
