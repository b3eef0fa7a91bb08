// Gather of the Lighthouse sub-sequence (aitrends summary, 핵심 기여 and
// 기술 상세 item 3: the chosen (Q, K, V) triples form one contiguous
// sub-sequence of S entries).
//
// One workgroup per 64 consecutive positions of one head. For position s it
// reads the entry (l, i) the index kernel placed there and fetches its
// pooled rows: level 0 is the input row itself; a materialised level is
// copied from the front pass (fp32); any other level is averaged here from
// its p^l input rows (fp32 sum). Rows go out as fp16, the layouts the
// attention kernels read as MFMA operands: query, key and value rows as fp16
// (hi = fp16(x)), row-major [S_pad][d], and through an LDS tile the key and
// value rows transposed [d][S_pad]. The query's lo part lo = fp16(x - hi)
// keeps the logits at about 22 bits of the pooled value: with fp32 inputs it
// goes out as fp16 (and so does the key's), with bf16 inputs as an e4m3 copy
// in operand-order 32-row tiles (fixed scale kFp8Exp), beside e4m3 copies of
// the key and value rows. Positions past S are zero. Every
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
    constexpr bool F8 = DT == LH_BF16;    // e4m3 tiles for the lo products (see lh_device.h)
    __shared__ __attribute__((aligned(16))) uint16_t tile[2][kGatherTile * LD]; // K hi, V for the transposes
    __shared__ int32_t s_ent[kGatherTile];
    const int h = blockIdx.y;
    const int64_t s0 = (int64_t)blockIdx.x * kGatherTile;
    const int lane = threadIdx.x % LANES;
    const int lg = threadIdx.x / LANES;
    const T *src[3] = {reinterpret_cast<const T *>(a.q), reinterpret_cast<const T *>(a.k),
                       reinterpret_cast<const T *>(a.v)};
    if (threadIdx.x < kGatherTile)
        s_ent[threadIdx.x] = a.ent[(int64_t)h * a.S_pad + s0 + threadIdx.x];
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
            uint4 hi, lo = make_uint4(0u, 0u, 0u, 0u);
            if (t == 0 || (!F8 && t == 1)) {
                split8_f16(x[t], hi, lo);
                if constexpr (!F8) // fp32 inputs: the fp16 lo parts (bf16: Q's lo part as the e4m3 tile below)
                    *reinterpret_cast<uint4 *>(a.lo[t] + off) = lo;
            } else {
                hi = pack8_f16(x[t]);
            }
            if constexpr (F8) { // the e4m3 copy of the Q lo part, of K hi and of V, x * 2^-kFp8Exp[t]
                float v8[8];
                unpack8_f16(t == 0 ? lo : hi, v8);
                const int64_t tile0 = ((int64_t)h * a.S_pad + (s & ~int64_t(31))) * D;
                *reinterpret_cast<uint2 *>(a.t8[t] + tile0 + fp8_tile_offset((int)(s & 31), lane)) =
                    pack8_fp8(v8, ldexpf(1.0f, -kFp8Exp[t]));
            }
            *reinterpret_cast<uint4 *>(a.hi[t] + off) = hi;
            if (t > 0)
                *reinterpret_cast<uint4 *>(&tile[t - 1][r * LD + lane * 8]) = hi;
        }
    }
    __syncthreads();

    // Transposed copies of K hi and V (the dQ kernel's and the forward's P.V
    // operands): 8 consecutive positions of one dimension per 16-byte store.
    constexpr int CH = kGatherTile / 8;
    for (int c = threadIdx.x; c < 2 * D * CH; c += 256) {
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
