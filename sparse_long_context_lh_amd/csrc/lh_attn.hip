// Dense causal softmax attention over the gathered sub-sequence (aitrends
// summary, 핵심 기여 and 기술 상세 item 3: stock FlashAttention on the S
// gathered entries; its default: causal, scale 1/sqrt(d)), forward and
// backward, as fp16 MFMA kernels for gfx950 with fp32 accumulation.
//
// MFMA used: v_mfma_f32_32x32x16_f16. Operand A supplies rows (lane l: row
// l%32, 8 k-values of group l/32), operand B supplies columns the same way,
// and the 32x32 fp32 result leaves row 8*(v/4) + 4*(l/32) + v%4, column l%32
// in register v of lane l. Each lane therefore owns ONE column and 16 rows.
//
// The kernels use this to give every lane one query (forward, dQ) or one key
// (dK/dV) and keep the softmax row statistics in-lane:
//   * forward and dQ compute S^T = K Q^T (keys as rows). The A rows are loaded
//     in a permuted key order kappa(r) so that register v of lane group g holds
//     key 16*(v/8) + 8*g + v%8: two runs of 8 consecutive keys. Those runs are
//     exactly the 8 k-values a lane must supply as operand B of the next
//     product O^T += V^T P^T, so P goes from accumulator to operand without a
//     shuffle, and V^T rows are read as 16-byte runs of 8 keys.
//   * dK/dV computes S = Q K^T with queries permuted the same way.
// Tiles of K/V (forward, dQ) or Q/dO (dK/dV) are staged in LDS with an XOR
// swizzle on 16-byte chunks so that the 32 rows one MFMA operand read touches
// fall in distinct banks.
//
// Precision: a logit is q_hi.k_hi + q_lo.k_hi over the fp16 pair q = hi + lo
// of the gathered query row, plus q_hi.k_lo when the inputs are fp32. With
// bf16 inputs the correction q_lo.k_hi runs on block-scaled fp8 copies of
// q_lo and k_hi (one fixed power-of-two scale per tensor, which the staging
// bounds make safe: see kFp8Exp): it carries the query's low bits, and its own
// error sits about 2^-15 below the largest |q_lo| |k| of the head, far under
// the fp16 hi product's. A
// query's rounding error shifts every logit of its row coherently, so its lo
// part is needed; keys' rounding errors are independent and average out over
// a row, except on the level-0 keys the selection concentrates attention on,
// and those are the bf16 inputs themselves, exact in fp16. The forward and the
// backward form the same logits, so both see the same P. dP uses the pair
// of dO_sub: its hi part in fp16 products, its lo part as fp16 (fp32 inputs)
// or, with bf16 inputs, as a block-scaled fp8 product against an e4m3 copy of
// V (fixed scales again); the forward's P.V uses an fp16 pair of
// P (two products), so O_sub, and with it delta = rowsum(dO_sub * O_sub),
// agree with the P the backward recomputes (dS = P (dP - delta) cancels
// heavily when |dO_sub| is large). dS, V, the backward's P, dO_sub's hi part
// and the query / key hi parts of the gradient products are single fp16
// operands.
//
// The backward is split into a dK/dV kernel (one workgroup per 128 keys) and a
// dQ kernel (one workgroup per block of queries) so that no gradient needs
// atomics and results are bitwise reproducible.
//
// Scale: the gathered rows arrive multiplied by per-head powers of two 2^ex
// (Q, K, V) and dO_sub by 2^ex_do, so that they fit fp16 whatever the inputs'
// scale: the logits' scale is divided by 2^(ex_q + ex_k), and every output
// leaves divided by the scales of the operands that formed it (exact).
//
// Range: probabilities enter fp16 products multiplied by 2^15 (kPScale), so
// the many tiny probabilities of a long, sharply peaked row do not underflow
// fp16 (they would vanish from P.V but stay in the fp32 normaliser, and the
// resulting O_sub error is amplified by delta); the scale cancels against the
// normaliser (forward) or is divided out of dV (backward). The log-sum-exp is
// kept in the log2 domain of the scaled logits, as the backward uses it.
#include "lh_device.h"
#include "lh_internal.h"

namespace lh {

// exp2 offset and factor applied to probabilities before they become fp16
constexpr float kPScaleLog2 = 15.0f;
constexpr float kPScaleInv = 1.0f / 32768.0f;

__device__ __forceinline__ f32x16_t mfma32(uint4 a, uint4 b, f32x16_t c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                  c, 0, 0, 0);
}

__device__ __forceinline__ uint4 pack8h(const float *x)
{
    return make_uint4(pack_f16x2(x[0], x[1]), pack_f16x2(x[2], x[3]), pack_f16x2(x[4], x[5]), pack_f16x2(x[6], x[7]));
}

// Physical 16-byte chunk of logical chunk `ch` in row `row` of an LDS tile
// whose rows hold NCH chunks (16 for 256-byte rows, 8 for 128-byte rows).
template <int NCH>
__device__ __forceinline__ int swz(int row, int ch)
{
    if constexpr (NCH >= 16)
        return ch ^ (row & 15);
    else
        return ch ^ ((row >> 1) & (NCH - 1));
}

__device__ __forceinline__ f32x16_t zero16()
{
    f32x16_t z;
#pragma unroll
    for (int v = 0; v < 16; ++v)
        z[v] = 0.0f;
    return z;
}

__device__ __forceinline__ uint4 ld16(const uint16_t *p) { return *reinterpret_cast<const uint4 *>(p); }

// ============================================================== async staging
// global_load_lds_dwordx4: each lane fetches 16 bytes from its own global
// address and the wave writes them to LDS at M0 + 16 * lane (M0 uniform over
// the wave). A stage is a list of 16-byte LDS chunks; chunk c of a round is
// handled by thread c % 256. The XOR swizzle of a tile is applied by choosing
// which global chunk lands in each physical LDS chunk. No registers hold the
// data, so later stages load while the current one is used.
//
// The transfer is issued from inline assembly: the compiler's own tracking of
// LDS DMA is coarse (it waits for every transfer in flight before any LDS
// read that might alias one, and so does the release fence of
// __syncthreads), which would serialise the rings. The kernels wait
// themselves (s_waitcnt vmcnt, then a plain s_barrier) before reading a
// stage, so a ring can be one LDS array indexed at run time. The address is a wave-uniform 64-bit base in SGPRs plus a 32-bit
// per-lane byte offset (no 64-bit arithmetic per lane). One wait state
// separates the write of M0 from the transfer that reads it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm" // M0 is reserved: nothing else in these kernels keeps it live
__device__ __forceinline__ void dma16(const void *base, uint32_t off_bytes, const uint4 *lds_wave_base)
{
    // the low 32 bits of a generic LDS address are the LDS offset (the shared
    // aperture is 4 GiB aligned); this avoids the null check of an address-space cast
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)lds_wave_base);
    // (readfirstlane yields a signed int: both halves go through uint32_t so
    // that the low word is zero-extended, never sign-extended)
    const uint64_t b = (uint64_t)(size_t)base;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(off_bytes), "s"(sb)
                 : "memory", "m0");
}
// The same with the non-temporal hint, for data read once (the dS tiles).
__device__ __forceinline__ void dma16_nt(const void *base, uint32_t off_bytes, const uint4 *lds_wave_base)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)lds_wave_base);
    const uint64_t b = (uint64_t)(size_t)base;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt" ::"s"(m0), "v"(off_bytes), "s"(sb)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ void wait_async() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }


// Generic swizzle for NCH chunks per row: rows per 256-byte bank window are
// 16/NCH; XOR the chunk with the window index so 16 consecutive rows map the
// same logical chunk to 16 distinct bank groups.
template <int NCH>
__device__ __forceinline__ int swzg(int row, int ch)
{
    return ch ^ ((row / (16 / NCH)) & (NCH - 1));
}

// The dK/dV kernel's row-major Q and dO tiles are read two ways: 16 lanes
// read one chunk of 16 rows (operands of S and dP), and a transposing read
// takes, per half wave, the same 4 consecutive chunks of 4 consecutive rows
// (operands of dV and dK). XOR-ing a row's chunks with a rotation of its
// 256-byte window index (the low bits, which differ between consecutive
// rows, moved to the top) serves both: distinct windows of 16 rows get
// distinct offsets, and 4 consecutive rows send their group of 4 chunks to 4
// different groups, so neither read meets a bank conflict. (NCH: 16 chunks
// per row at d = 128, 8 at d = 64.)
template <int NCH>
__device__ __forceinline__ int swzt(int row, int ch)
{
    constexpr int BITS = NCH == 16 ? 4 : 3, LOW = NCH == 16 ? 2 : 1;
    const int x = (row / (16 / NCH)) & (NCH - 1);
    return ch ^ (((x & ((1 << LOW) - 1)) << (BITS - LOW)) | (x >> LOW));
}

// ============================================================== forward
// One workgroup per 128 queries (32 per wave, Q hi / lo fragments in
// registers); keys stream through LDS 32 at a time in a three-stage ring
// filled asynchronously, two workgroups per CU.
//
// Software pipeline: while the matrix cores form the logits of key block
// j+1, the vector unit turns block j's logits into probabilities, and while
// they accumulate P_j V_j it takes the row maximum of block j+1. An MFMA
// runs in the background of the wave that issued it, so the softmax costs no
// time as long as it is interleaved with independent MFMAs in program order;
// the sched_group_barrier pattern below fixes that order.
template <int D, bool KLO> struct FwdStage {
    static constexpr int BN = 32;
    static constexpr int KCH = D / 8;  // chunks per K row
    static constexpr int VCH = BN / 8; // chunks per V^T row
    static constexpr int KROWS = BN * KCH, VROWS = D * VCH;
    // KL: the K lo tile (fp16, fp32 inputs) or the fp8 K tile (bf16 inputs:
    // 2D chunks, padded to one transfer per thread)
    static constexpr int KH = 0, KL = KROWS, KLSIZE = KLO ? KROWS : 256;
    static constexpr int VT = KROWS + KLSIZE;
    static constexpr int SIZE = VT + VROWS;
    static constexpr int KU = KROWS / 256, VU = VROWS / 256; // load rounds per tile
    static constexpr int NSLOT = 3;
};

// Block-scaled fp8 product (see lh_device.h): A and B are the two 16-byte
// halves of each lane's 32 operand bytes, sa / sb their scales (127 + e).
__device__ __forceinline__ f32x16_t mfma8(uint4 a0, uint4 a1, uint4 b0, uint4 b1, f32x16_t c, int sa, int sb)
{
    typedef int i32x8_t __attribute__((ext_vector_type(8)));
    const i32x8_t a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    const i32x8_t b = {(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// hi = fp16(x), lo = fp16(x - hi) for 8 values. The residual comes from one
// mixed-precision fma per value (fp16 operand, fp32 operand, fp16 result):
// x - hi is exact in fp32, so this rounds exactly as converting it would.
__device__ __forceinline__ void split8_mix(const float *x, uint4 &hi, uint4 &lo)
{
    uint32_t h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = pack_f16x2(x[2 * e], x[2 * e + 1]);
        asm("v_fma_mixlo_f16 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(l[e]) : "v"(h[e]), "v"(x[2 * e]));
        asm("v_fma_mixhi_f16 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
            : "+v"(l[e])
            : "v"(h[e]), "v"(x[2 * e + 1]));
    }
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// pairwise sum of a tile's 16 probabilities
__device__ __forceinline__ float tile_sum(const float *pr)
{
    float t8[8];
#pragma unroll
    for (int v = 0; v < 8; ++v)
        t8[v] = pr[v] + pr[v + 8];
#pragma unroll
    for (int v = 0; v < 4; ++v)
        t8[v] += t8[v + 4];
    return (t8[0] + t8[2]) + (t8[1] + t8[3]);
}

// An LDS address the compiler cannot split into a loop-invariant part per
// access: every fragment read of a stage becomes one base register plus an
// immediate offset instead of one precomputed register per fragment.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef const u32x4_t __attribute__((address_space(3))) *lds_cptr;
__device__ __forceinline__ lds_cptr lane_base(const uint4 *p)
{
    uint32_t off = (uint32_t)(size_t)p; // low word of a generic LDS address = LDS offset
    asm volatile("" : "+v"(off));
    return (lds_cptr)(size_t)off;
}
__device__ __forceinline__ uint4 lds_ld(lds_cptr p, int i) { return __builtin_bit_cast(uint4, p[i]); }

template <int M> struct Mode {
    static constexpr int value = M;
};

template <bool B> struct Flag {
    static constexpr bool value = B;
};

// max over lanes l and l ^ 32 (the two lane groups holding one column)
__device__ __forceinline__ float max_pair(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// BWD = false (calls no backward follows): P.V takes the fp16 P alone. Its
// lo product exists so that O_sub, and with it delta = rowsum(dO_sub *
// O_sub), agrees with the P the backward recomputes (dS = P (dP - delta)
// cancels heavily); O itself needs only the fp16 P (relative rounding error
// up to 2^-11 per probability). The query's lo part stays: without it a few
// outputs of the 64K-token workload leave the stated tolerance.
template <int D, bool KLO, bool BWD>
__global__ __launch_bounds__(256, 1) void k_attn_fwd(AttnFwdArgs a)
{
    typedef FwdStage<D, KLO> St;
    constexpr int BM = 128, BN = St::BN;
    constexpr int NS = D / 16;  // k-steps over d
    constexpr int NT = D / 32;  // 32-dim tiles of the output
    __shared__ uint4 ring[St::NSLOT * St::SIZE];

    const int nqb = (int)((a.S + BM - 1) / BM);
    const int h = blockIdx.x % a.H;
    const int qb = nqb - 1 - (int)(blockIdx.x / a.H); // longest rows first
    const int64_t q0 = (int64_t)qb * BM;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // uniform: LDS bases stay scalar
    const int64_t qw = q0 + wave * 32;
    const int64_t hS = (int64_t)h * a.S_pad;
    const uint16_t *khi = a.khi + hS * D, *klo = a.klo + hS * D;
    const uint8_t *k8 = a.k8 + hS * D;
    const uint16_t *vt = a.vt + (int64_t)h * D * a.S_pad;
    constexpr int NM = D / 64; // fp8 products of the logits' lo part (bf16 inputs)
    constexpr bool Q8 = !KLO; // the logits' lo part as those fp8 products
    // the logits of the staged rows are 2^(ex_q + ex_k) times the true ones
    const float scale_log2 = ldexpf(a.scale_log2, -(a.ex[h] + a.ex[a.H + h]));

    const int64_t kend = min(q0 + BM, a.S);
    const int nkb = (int)((kend + BN - 1) / BN);
    // last key block this wave reads: its diagonal block, or the workgroup's
    // last one for rows past S (their outputs are never read)
    const int jl = (int)min((int64_t)(nkb - 1), qw / BN);

    // byte offsets of this thread's chunks in a stage (the stage moves the base)
    // Operand-order tiles: fragment f of a tile is the 64 x 16 bytes one MFMA
    // operand reads, lane l's chunk at f * 64 + l, so every fragment read is
    // one linear 1 KiB LDS access. The transfer of LDS chunk c = 256u + tid
    // fetches what lane c % 64 of fragment c / 64 needs: for K, k-step
    // s = c / 64 of key row kappa(c % 32); for V^T, dimension row
    // 32 t + c % 32 and keys 16 hh + 8 (c / 32 % 2) .. +7 with
    // (hh, t) = (f / NT, f % NT).
    uint32_t koff[St::KU], voff[St::VU];
#pragma unroll
    for (int u = 0; u < St::KU; ++u) {
        const int f = 4 * u + wave;
        koff[u] = 2u * (uint32_t)(kappa(c32) * D + (2 * f + g) * 8);
    }
#pragma unroll
    for (int u = 0; u < St::VU; ++u) {
        const int f = 4 * u + wave, hh = f / NT, t = f % NT;
        voff[u] = 2u * ((uint32_t)(32 * t + c32) * (uint32_t)a.S_pad + (uint32_t)(16 * hh + 8 * g));
    }
    auto slot = [&](int kb) { return ring + (kb % St::NSLOT) * St::SIZE; };
    auto issue = [&](int kb) {
        if (kb >= nkb)
            return;
        const int64_t k0 = (int64_t)kb * BN;
        const uint4 *base = slot(kb);
#pragma unroll
        for (int u = 0; u < St::KU; ++u) {
            dma16(khi + k0 * D, koff[u], base + St::KH + 256 * u + 64 * wave);
            if constexpr (KLO)
                dma16(klo + k0 * D, koff[u], base + St::KL + 256 * u + 64 * wave);
        }
        if constexpr (Q8) // the fp8 tile is stored in operand order: a linear copy
            dma16(k8 + k0 * D, 16u * (uint32_t)(tid % (2 * D)), base + St::KL + 64 * wave);
#pragma unroll
        for (int u = 0; u < St::VU; ++u)
            dma16(vt + k0, voff[u], base + St::VT + 256 * u + 64 * wave);
    };

    issue(0);
    // Q as MFMA operand B: the fp16 hi part, and the lo part as fp16 (fp32
    // inputs) or as its fp8 tile (bf16 inputs; lane c32 holds query qw + c32,
    // which the tile keeps at lane position kappa(c32) + 32g)
    uint4 qh[NS], ql[KLO ? NS : 1], q8[KLO ? 1 : NM][2];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        qh[s] = ld16(a.qhi + (hS + qw + c32) * D + 16 * s + 8 * g);
        if constexpr (KLO)
            ql[s] = ld16(a.qlo + (hS + qw + c32) * D + 16 * s + 8 * g);
    }
    int qs = 0, ks = 0; // scale bytes of the e4m3 Q lo and K tiles
    if constexpr (Q8) {
        const uint8_t *qt8 = a.qlo8 + (hS + qw) * D + 16 * (kappa(c32) + 32 * g);
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                q8[m][q] = *reinterpret_cast<const uint4 *>(qt8 + 2048 * m + 1024 * q);
        qs = 127 + kFp8Exp[0];
        ks = 127 + kFp8Exp[1];
    }
    // Consume the fragments here: otherwise the compiler waits for them at
    // their first use inside the key loop, in every iteration, and those
    // waits on the memory counter also wait for the ring's transfers in flight.
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        asm volatile("" ::"v"(qh[s].x));
        if constexpr (KLO)
            asm volatile("" ::"v"(ql[s].x));
    }
    if constexpr (Q8) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
            asm volatile("" ::"v"(q8[m][0].x), "v"(q8[m][1].x));
    }
    wait_async(); // stage 0 (its transfers were issued before the fragments)
    issue(1);
    lds_barrier();

    // S^T tile of key block kb (keys as rows, kappa-permuted)
    auto logits = [&](const uint4 *base) __attribute__((always_inline)) {
        f32x16_t st = zero16();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const uint4 kh = base[St::KH + 64 * s + lane];
            st = mfma32(kh, qh[s], st);
            if constexpr (KLO) {
                st = mfma32(base[St::KL + 64 * s + lane], qh[s], st);
                st = mfma32(kh, ql[s], st);
            }
        }
        if constexpr (Q8) {
#pragma unroll
            for (int m = 0; m < NM; ++m)
                st = mfma8(base[St::KL + 128 * m + lane], base[St::KL + 128 * m + 64 + lane], q8[m][0], q8[m][1], st,
                           ks, qs);
        }
        return st;
    };
    auto rowmax = [&](const f32x16_t &st) __attribute__((always_inline)) {
        float mx = st[0];
#pragma unroll
        for (int v = 1; v < 16; ++v)
            mx = fmaxf(mx, st[v]);
        return max_pair(mx);
    };

    f32x16_t o[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        o[t] = zero16();
    float lsum = 0.0f;
    // Running maximum m of the scaled logits y = st * log2(e)/sqrt(d); the
    // maximum is taken on st (a positive scale keeps the order, and rounding
    // is monotonic). Probabilities enter the products as 2^(y - m + 15).
    f32x16_t st = logits(slot(0));
    float m = jl > 0 ? rowmax(st) * scale_log2 : -INFINITY;

    // Probabilities of block st relative to m: the fp16 pair of each run of 8
    // keys, and their sum added to lsum. The tile's 16 probabilities are
    // summed first (pairwise) and then added to the running sum: added one by
    // one, probabilities far below the running sum's half-ulp would all be
    // rounded away, a systematic loss in the normaliser that the backward's
    // dS = P (dP - delta) amplifies.
    // the fp16 pair of 8 probabilities (BWD), or their fp16 values alone
    auto split = [&](const float *x, uint4 &hi, uint4 &lo) __attribute__((always_inline)) {
        if constexpr (BWD)
            split8_mix(x, hi, lo);
        else
            hi = pack8h(x);
    };
    auto probs = [&](const f32x16_t &sv, uint4 (&ph)[2], uint4 (&pl)[2]) __attribute__((always_inline)) {
        const float shift = m - kPScaleLog2; // p * 2^15 <= 2^15: within fp16
        float pr[16];
#pragma unroll
        for (int v = 0; v < 16; ++v)
            pr[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[v], scale_log2, -shift));
        split(pr, ph[0], pl[0]);
        split(pr + 8, ph[1], pl[1]);
        lsum += tile_sum(pr);
    };
    // O^T += V^T P^T for block kb
    auto accumulate = [&](const uint4 *base, const uint4 (&ph)[2], const uint4 (&pl)[2]) __attribute__((always_inline)) {
        const uint4 *sV = base + St::VT;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint4 vv = sV[64 * (hh * NT + t) + lane];
                o[t] = mfma32(vv, ph[hh], o[t]);
                if constexpr (BWD)
                    o[t] = mfma32(vv, pl[hh], o[t]);
            }
    };
    // rescale O and the running sum when some row's maximum moved (a factor
    // of 1 changes nothing)
    auto rescale = [&](float mn) __attribute__((always_inline)) {
        if (__ballot(mn != m) != 0) {
            const float alpha = __builtin_amdgcn_exp2f(m - mn);
            lsum *= alpha;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    o[t][v] *= alpha;
        }
        m = mn;
    };

    // Block j < jl: logits of block j+1 alongside the probabilities of block
    // j, then P_j V_j alongside the row maximum of block j+1 (skipped when
    // block j+1 is the diagonal one: its maximum is taken after masking).
    auto body = [&](int j, auto last) __attribute__((always_inline)) {
        constexpr bool LAST = decltype(last)::value;
        const int dj = j % St::NSLOT - (j + 1) % St::NSLOT; // slot(j) - slot(j + 1), in stages
        const lds_cptr kb = lane_base(slot(j + 1) + lane), vb = kb + (St::VT + dj * St::SIZE);
        // Fragments are read a little ahead of their MFMAs (LDS reads return
        // in order): K of block j+1 two k-steps ahead, V^T of block j during
        // the second half of the logits.
        uint4 kf[NS], kl[KLO ? NS : 1], k8f[KLO ? 1 : NM][2], vf[2 * NT];
        auto read_k = [&](int s) __attribute__((always_inline)) {
            kf[s] = lds_ld(kb, St::KH + 64 * s);
            if constexpr (KLO)
                kl[s] = lds_ld(kb, St::KL + 64 * s);
        };
        auto read_v = [&](int f) __attribute__((always_inline)) { vf[f] = lds_ld(vb, 64 * f); };
        read_k(0);
        read_k(1);
        __builtin_amdgcn_sched_barrier(0);

        // Each group below is its own scheduling region (sched_barrier): the
        // MFMAs first, then vector work that does not depend on them, so the
        // vector unit runs while the matrix core is busy.
        const float shift = m - kPScaleLog2; // p * 2^15 <= 2^15: within fp16
        float pr[16];
        uint4 ph[2], pl[2];
        auto expo = [&](int v0, int v1) __attribute__((always_inline)) {
#pragma unroll
            for (int v = v0; v < v1; ++v)
                pr[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[v], scale_log2, -shift));
        };
        constexpr int HS = NS / 2;
        f32x16_t sn = zero16();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if (s + 2 < NS)
                read_k(s + 2);
            // V^T fragments 0 .. NT-1 over the second half
            if (s >= HS) {
#pragma unroll
                for (int f = (s - HS) * NT / (NS - HS); f < (s - HS + 1) * NT / (NS - HS); ++f)
                    read_v(f);
            }
            if (Q8 && s == NS - 2) {
#pragma unroll
                for (int mm = 0; mm < NM; ++mm) {
                    k8f[mm][0] = lds_ld(kb, St::KL + 128 * mm);
                    k8f[mm][1] = lds_ld(kb, St::KL + 128 * mm + 64);
                }
            }
            sn = mfma32(kf[s], qh[s], sn);
            if constexpr (KLO) {
                sn = mfma32(kl[s], qh[s], sn);
                sn = mfma32(kf[s], ql[s], sn);
            } else if (Q8 && s == NS - 1) { // the lo part, as block-scaled fp8 products
#pragma unroll
                for (int mm = 0; mm < NM; ++mm)
                    sn = mfma8(k8f[mm][0], k8f[mm][1], q8[mm][0], q8[mm][1], sn, ks, qs);
            }
            if (s < HS)
                expo(8 * s / HS, 8 * (s + 1) / HS);
            else if (s == HS)
                split(pr, ph[0], pl[0]);
            else
                expo(8 + 8 * (s - HS - 1) / (NS - HS - 1), 8 + 8 * (s - HS) / (NS - HS - 1));
            __builtin_amdgcn_sched_barrier(0);
        }
        // O^T += V^T P^T: per accumulator the order hi, lo of keys 0-15, then
        // hi, lo of keys 16-31
#pragma unroll
        for (int f = NT; f < 2 * NT; ++f)
            read_v(f);
#pragma unroll
        for (int t = 0; t < NT; ++t)
            o[t] = mfma32(vf[t], ph[0], o[t]);
        split(pr + 8, ph[1], pl[1]);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (BWD) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
                o[t] = mfma32(vf[t], pl[0], o[t]);
        }
        lsum += tile_sum(pr);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < NT; ++t)
            o[t] = mfma32(vf[NT + t], ph[1], o[t]);
        float mn = m;
        if constexpr (!LAST)
            mn = fmaxf(m, rowmax(sn) * scale_log2);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (BWD) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
                o[t] = mfma32(vf[NT + t], pl[1], o[t]);
        }
        st = sn;
        if constexpr (!LAST)
            rescale(mn);
    };
    // Block jl: mask keys after the query (diagonal block), maximum,
    // probabilities, P V.
    auto tail = [&](int j) __attribute__((always_inline)) {
        const int64_t kt0 = (int64_t)j * BN;
        if (kt0 + 31 > qw) {
#pragma unroll
            for (int v = 0; v < 16; ++v)
                if ((int)(kt0 - qw) + 16 * (v >> 3) + 8 * g + (v & 7) > c32)
                    st[v] = -INFINITY;
        }
        rescale(fmaxf(m, rowmax(st) * scale_log2));
        uint4 ph[2], pl[2];
        probs(st, ph, pl);
        accumulate(slot(j), ph, pl);
    };

    // Step j starts by making stage j+1 visible and refilling the slot of
    // stage j-1. Every wave passes the same sequence of barriers; the loops
    // below only split it by what this wave computes in each step.
    auto sync = [&](int j) __attribute__((always_inline)) {
        if (j + 1 < nkb) {
            wait_async(); // stage j+1 (the only one in flight)
            lds_barrier(); // ... visible to all waves; stage j-1's slot is free
            issue(j + 2);
        }
    };
    int j = 0;
    for (; j + 1 < jl; ++j) {
        sync(j);
        body(j, Flag<false>());
    }
    if (jl > 0) {
        sync(j);
        body(j, Flag<true>());
        ++j;
    }
    sync(j);
    tail(j);
    for (++j; j < nkb; ++j)
        sync(j);

    const float ltot = lsum + __shfl_xor(lsum, 32);
    const float inv = ldexpf(1.0f / ltot, -a.ex[2 * a.H + h]); // the staged V is 2^ex_v V
    float *orow = a.o + (hS + qw + c32) * D;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
            *reinterpret_cast<float4 *>(orow + 32 * t + 8 * i4 + 4 * g) =
                make_float4(o[t][4 * i4] * inv, o[t][4 * i4 + 1] * inv, o[t][4 * i4 + 2] * inv, o[t][4 * i4 + 3] * inv);
    if (g == 0)
        a.lse[hS + qw + c32] = m + (__log2f(ltot) - kPScaleLog2); // log2 domain
}

template <int D, bool KLO>
static void launch_fwd_t(const dim3 grid, const AttnFwdArgs &a, hipStream_t s)
{
    if (a.for_bwd)
        hipLaunchKernelGGL((k_attn_fwd<D, KLO, true>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((k_attn_fwd<D, KLO, false>), grid, dim3(256), 0, s, a);
}

hipError_t launch_attn_fwd(const Plan &pl, const AttnFwdArgs &a, hipStream_t s)
{
    const unsigned nqb = (unsigned)((pl.S + 127) / 128);
    const dim3 grid(nqb * pl.H);
    const bool klo = pl.dt == LH_F32; // see the precision note at the top of this file
    if (pl.d == 128) {
        if (klo)
            launch_fwd_t<128, true>(grid, a, s);
        else
            launch_fwd_t<128, false>(grid, a, s);
    } else {
        if (klo)
            launch_fwd_t<64, true>(grid, a, s);
        else
            launch_fwd_t<64, false>(grid, a, s);
    }
    return hipGetLastError();
}

// ============================================================== backward: dK, dV
// One workgroup per 128 keys (32 per wave; K hi, K lo and V rows of the
// lane's key in registers); queries stream through LDS 32 at a time from the
// key block onwards, in a three-deep ring of stages filled asynchronously
// (two stages are in flight while one is used).
// S = Q K^T with queries as (permuted) rows, so a lane owns one key:
//   dV^T += dO^T P,  dP = dO V^T,  dS = P * (dP - delta),  dK^T += Q^T dS.
template <int D>
struct DkdvStage {
    static constexpr int BQ = 32;
    static constexpr int RCH = D / 8;  // chunks per row-major row
    static constexpr int ROWS = BQ * RCH;
    static constexpr int QH = 0, QL = ROWS, DH = 2 * ROWS, DL = 3 * ROWS;
    // row statistics: 64 chunks per wave, the first 4 of them used (wave 0:
    // lse of queries 0-15, 1: lse 16-31, 2: delta 0-15, 3: delta 16-31); a
    // whole wave's transfer fills them, so none is predicated
    static constexpr int LS = 4 * ROWS;
    static constexpr int SIZE = LS + 4 * 64; // in 16-byte chunks
    static constexpr int NBUF = 3;
};

// gfx950's transposing LDS read (16-bit elements): in each group of 16 lanes,
// lane 4R + m supplies 4 consecutive elements a[4R + m][0..3], and lane j
// receives a[4R + j/4][j%4] for R = 0..3 as its 4 elements. With lane 4R + m
// addressing row r_R, columns c + 4m .. c + 4m + 3 of a row-major tile, lane
// j receives column c + j of rows r_0 .. r_3: a column read.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_tr16(const uint4 *tile, uint32_t byte_off)
{
    const uint32_t off = (uint32_t)(size_t)tile + byte_off; // low word of a generic LDS address = LDS offset
    typedef s16x4_t __attribute__((address_space(3))) *ptr_t;
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((ptr_t)(size_t)off));
}

// A 16-byte non-temporal store (the dS tiles: too large to stay cached until
// the dQ kernel reads them, so they should not evict the stream of Q and dO).
__device__ __forceinline__ void store16_stream(uint16_t *p, uint4 v)
{
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, reinterpret_cast<v4u *>(p));
}

// Keeps the compiler from moving instructions across this point: used to
// interleave each matrix product with the LDS read of a later operand.
#define LH_FENCE __builtin_amdgcn_sched_barrier(0)

template <int N>
__device__ __forceinline__ void wait_async_n()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int D, bool KLO>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_attn_bwd_dkdv(AttnBwdArgs a)
{
    typedef DkdvStage<D> St;
    constexpr int BK = 128, BQ = St::BQ, RCH = St::RCH;
    constexpr int NS = D / 16, NT = D / 32;
    constexpr int RU = St::ROWS / 256; // load rounds per tile
    constexpr int NM = D / 64; // fp8 products of the lo parts (bf16 inputs)
    // transfers one wave issues per stage (bf16 inputs: the Q lo and dO lo
    // tiles are fp8 tiles, one transfer per thread each)
    constexpr int LOADS = 2 * RU + 2 * (KLO ? RU : 1) + 1;
    __shared__ uint4 ring[St::NBUF * St::SIZE];

    const int h = blockIdx.x % a.H;
    const int kb = (int)(blockIdx.x / a.H); // early keys see the most queries: run them first
    const int k0 = kb * BK;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // uniform: LDS bases stay scalar
    const int kw = k0 + wave * 32;
    // lane c32 owns key kw + kappa(c32): the lane position the forward's fp8
    // K tile gives that key, so the lane reads its own fragment of it
    const int key = kw + kappa(c32);
    const int S = (int)a.S, S_pad = (int)a.S_pad;
    const int64_t hS = (int64_t)h * S_pad;
    // staged rows: q 2^ex_q, k 2^ex_k, v 2^ex_v, dO_sub 2^ex_do (delta arrives
    // times 2^(ex_do + ex_v)); dS is then 2^(ex_do + ex_v) dS
    const int exq = a.ex[h], exk = a.ex[a.H + h], exv = a.ex[2 * a.H + h], exd = a.ex[3 * a.H + h];
    const float scale_log2 = ldexpf(a.scale_log2, -(exq + exk));

    // Per-lane byte offsets of this thread's chunks inside a stage's tiles
    // (the same for every stage; the stage only moves the uniform base).
    uint32_t roff[RU];
#pragma unroll
    for (int u = 0; u < RU; ++u) {
        const int c = 256 * u + tid, r = c / RCH;
        roff[u] = 2u * (uint32_t)(r * D + swzt<RCH>(r, c % RCH) * 8);
    }
    // Byte offsets of this lane's transposing reads of the row-major Q and dO
    // hi tiles: the operand of dV (dO^T) and dK (Q^T) for dimensions
    // 32t .. 32t+31 and queries 16hh .. 16hh+15 is two reads (queries
    // 16hh + 8g + 4n .. +3, n = 0, 1), lane 16G + 4R + m addressing query
    // 16hh + 8(G/2) + 4n + R, dimensions 32t + 16(G%2) + 4m .. +3.
    uint32_t toff[2][2][NT];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int n = 0; n < 2; ++n)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int G = lane >> 4, R = (lane >> 2) & 3, m = lane & 3;
                const int q = 16 * hh + 8 * (G >> 1) + 4 * n + R, dim = 32 * t + 16 * (G & 1) + 4 * m;
                toff[hh][n][t] = 2u * (uint32_t)(q * D + swzt<RCH>(q, dim >> 3) * 8 + (dim & 7));
            }
    const uint16_t *const rows[4] = {a.qhi, a.qlo, a.dohi, a.dolo};
    // each wave fetches 4 of the 16 lse / delta chunks (lanes 4..63 repeat
    // them), so every wave issues the same number of loads per stage (St::LOADS)
    const float *stat = wave < 2 ? a.lse : a.delta;
    const uint32_t stat_off = 16u * (uint32_t)(4 * (wave & 1) + (lane & 3));

    // A stage's transfers in five parts (the four row-major tiles, then the
    // statistics), issued at spread-out points of the previous stage's math:
    // issued in one burst, their LDS writes stall the operand reads of the
    // products.
    auto issue_rows = [&](int q0, const uint4 *base, int t) {
        if (!KLO && (t == 1 || t == 3)) { // fp8 Q lo / dO lo tile, stored in operand order: a linear copy
            dma16((t == 1 ? a.qlo8 : a.dolo8) + (hS + q0) * D, 16u * (uint32_t)(tid % (2 * D)),
                  base + 64 * wave + (t == 1 ? St::QL : St::DL));
            return;
        }
        const uint16_t *rb = rows[t] + (hS + q0) * D;
#pragma unroll
        for (int u = 0; u < RU; ++u)
            dma16(rb, roff[u], base + 64 * wave + t * St::ROWS + 256 * u);
    };
    auto issue_stats = [&](int q0, const uint4 *base) {
        dma16(stat + hS + q0, stat_off, base + St::LS + 64 * wave);
    };
    auto issue = [&](int q0, const uint4 *base) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
            issue_rows(q0, base, t);
        issue_stats(q0, base);
    };

    uint4 kh[NS], vf[NS], klf[KLO ? NS : 1], k8r[KLO ? 1 : NM][2], v8r[KLO ? 1 : NM][2];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        const int64_t off = (hS + key) * D + 16 * s + 8 * g;
        kh[s] = ld16(a.khi + off);
        if constexpr (KLO)
            klf[s] = ld16(a.klo + off);
        vf[s] = ld16(a.v + off);
    }
    // bf16 inputs: this wave's fp8 K and V tiles as operand B (the tiles keep
    // key kw + kappa(c32) at lane position c32 + 32g: this lane's own position)
    int ks = 0, qs = 0, vs = 0, ds8 = 0; // scale bytes of the e4m3 K, Q lo, V, dO lo tiles
    if constexpr (!KLO) {
        const uint8_t *kt8 = a.k8 + (hS + kw) * D + 16 * lane;
        const uint8_t *vt8 = a.v8 + (hS + kw) * D + 16 * lane;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                k8r[m][q] = *reinterpret_cast<const uint4 *>(kt8 + 2048 * m + 1024 * q);
                v8r[m][q] = *reinterpret_cast<const uint4 *>(vt8 + 2048 * m + 1024 * q);
            }
        qs = 127 + kFp8Exp[0];
        ks = 127 + kFp8Exp[1];
        vs = 127 + kFp8Exp[2];
        ds8 = 127 + kFp8Exp[3];
        // consume them here (see the forward kernel)
#pragma unroll
        for (int m = 0; m < NM; ++m)
            asm volatile("" ::"v"(k8r[m][0].x), "v"(k8r[m][1].x), "v"(v8r[m][0].x), "v"(v8r[m][1].x));
    }
    f32x16_t dvT[NT], dkT[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        dvT[t] = zero16();
        dkT[t] = zero16();
    }
    const int ql = kappa(c32);
    uint16_t *const dst_head = a.dst + (a.dst != nullptr ? (int64_t)h * a.dst_head : 0);
    const int kt = kw / 32; // this wave's key tile
    const int nst = (S - k0 + BQ - 1) / BQ;

    int slot = 0; // ring slot of stage it
    // One stage in four phases, each a group of MFMAs with the vector work
    // that does not depend on them placed behind them (scheduling barriers
    // keep the order): S; dP with P = exp2(...) of the finished S; dV with
    // dS = P (dP - delta); dK with the dS tile store.
    // MODE 0: every query of the stage precedes this wave's keys (nothing to
    // compute); 1: interior stage; 2: masked (diagonal, or reaching past S).
    auto stage = [&](int it, auto mode_flag) __attribute__((always_inline)) {
        constexpr int MODE = decltype(mode_flag)::value;
        const uint4 *base = ring + slot * St::SIZE;
        const uint4 *ahead = ring + (slot == 0 ? 2 : slot - 1) * St::SIZE; // slot of stage it + 2
        const int q0 = k0 + it * BQ;
        // stage it has landed once at most one stage's loads are outstanding
        // (this also waits for the previous stage's dS stores, issued after them:
        // vector memory operations complete in issue order)
        wait_async_n<LOADS>();
        lds_barrier(); // stage it is visible to all waves; stage it-1's slot is free
        // stage it + 2 is loaded during this one; past the last stage, the last
        // stage again (into the free slot, never read): no branch in the stage
        const int q2 = k0 + min(it + 2, nst - 1) * BQ;
        if constexpr (MODE == 0) {
            issue(q2, ahead);
            return;
        }
        const float *sL = reinterpret_cast<const float *>(base + St::LS);
        const float *sDel = sL + 2 * 256; // (waves 2, 3 of the statistics area)
        auto rd = [&](int s, int i) {
            const int at = ql * RCH + swzt<RCH>(ql, 2 * s + g);
            return base[(i == 0 ? St::QH : i == 1 ? St::QL : i == 2 ? St::DH : St::DL) + at];
        };
        // operand of dV (i = 0, 1: dO^T) or dK (i = 2, 3: Q^T), dimensions
        // 32t .. 32t+31, queries 16(i%2) .. +15: transposing reads of the
        // row-major hi tile
        auto gfrag = [&](int t, int i) {
            const uint4 *tile = base + (i < 2 ? St::DH : St::QH);
            const uint2 lo = lds_tr16(tile, toff[i & 1][0][t]), hi = lds_tr16(tile, toff[i & 1][1][t]);
            return make_uint4(lo.x, lo.y, hi.x, hi.y);
        };
        // statistics of 4 queries: register v holds query 16(v/8) + 8g + v%8
        auto stat4 = [&](const float *p, int v0) { // queries 16(v0/8) + 8g + v0%8 .. +3
            return *reinterpret_cast<const float4 *>(p + 256 * (v0 >> 3) + 8 * g + (v0 & 7));
        };
        const int rel = q0 - key; // query - key of register 0's query
        auto ok = [&](int v) {
            const int qi = 16 * (v >> 3) + 8 * g + (v & 7);
            return MODE == 1 || (rel + qi >= 0 && q0 + qi < S);
        };

        // S: the Q operands of k-step s+1 are read under the products of step s
        f32x16_t st = zero16(), dp = zero16();
        float4 lnext;
        uint4 qa[2][2], q8[KLO ? 1 : NM][2];
        qa[0][0] = rd(0, 0);
        if constexpr (KLO)
            qa[0][1] = rd(0, 1);
        LH_FENCE;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if (s % 2 == 1) { // row tiles of stage it + 2, spread over the k-steps
                constexpr int PER = 8 / NS;
#pragma unroll
                for (int t = 0; t < PER; ++t)
                    issue_rows(q2, ahead, (s / 2) * PER + t);
            }
            if (s + 1 < NS) {
                qa[(s + 1) & 1][0] = rd(s + 1, 0);
                if constexpr (KLO)
                    qa[(s + 1) & 1][1] = rd(s + 1, 1);
            }
            if (!KLO && s == NS - 2) {
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    q8[m][0] = base[St::QL + 128 * m + lane];
                    q8[m][1] = base[St::QL + 128 * m + 64 + lane];
                }
            }
            st = mfma32(qa[s & 1][0], kh[s], st);
            if constexpr (KLO) {
                st = mfma32(qa[s & 1][1], kh[s], st);
                st = mfma32(qa[s & 1][0], klf[s], st);
            } else if (s == NS - 1) { // the lo part, as block-scaled fp8 products
#pragma unroll
                for (int m = 0; m < NM; ++m)
                    st = mfma8(q8[m][0], q8[m][1], k8r[m][0], k8r[m][1], st, qs, ks);
            }
            if (s == NS - 1)
                lnext = stat4(sL, 0); // the statistics a piece needs are read a group ahead
            LH_FENCE;
        }
        // dP; behind its products, pr = P * 2^15 (keeps small P out of the fp16
        // underflow range; the statistics arrive as LSE - 15 and delta * 2^-15)
        float pr[16], ds[16];
        uint4 da[2][2], d8[KLO ? 1 : NM][2];
        da[0][0] = rd(0, 2);
        if constexpr (KLO)
            da[0][1] = rd(0, 3);
        LH_FENCE;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if (s + 1 < NS) {
                da[(s + 1) & 1][0] = rd(s + 1, 2);
                if constexpr (KLO)
                    da[(s + 1) & 1][1] = rd(s + 1, 3);
            }
            if (!KLO && s == NS - 2) {
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                    d8[m][0] = base[St::DL + 128 * m + lane];
                    d8[m][1] = base[St::DL + 128 * m + 64 + lane];
                }
            }
            dp = mfma32(da[s & 1][0], vf[s], dp);
            if constexpr (KLO) {
                dp = mfma32(da[s & 1][1], vf[s], dp);
            } else if (s == NS - 1) { // the lo part, as block-scaled fp8 products
#pragma unroll
                for (int m = 0; m < NM; ++m)
                    dp = mfma8(d8[m][0], d8[m][1], v8r[m][0], v8r[m][1], dp, ds8, vs);
            }
#pragma unroll
            for (int i = 4 * s / NS; i < 4 * (s + 1) / NS; ++i) { // values 4i .. 4i+3
                const int v0 = 4 * i;
                const float lq[4] = {lnext.x, lnext.y, lnext.z, lnext.w};
                lnext = i < 3 ? stat4(sL, v0 + 4) : stat4(sDel, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float sv = ok(v0 + e) ? st[v0 + e] : -INFINITY; // masked: P = 0
                    pr[v0 + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv, scale_log2, -lq[e]));
                }
            }
            LH_FENCE;
        }
        const uint4 pb0 = pack8h(pr), pb1 = pack8h(pr + 8);
        // dV; behind it dS = P (dP - delta) (a masked P = 0 gives dS = 0)
        uint4 ga[2][4];
#pragma unroll
        for (int i = 0; i < 2; ++i)
            ga[0][i] = gfrag(0, i);
        issue_stats(q2, ahead);
        LH_FENCE;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t + 1 < NT) {
                ga[(t + 1) & 1][0] = gfrag(t + 1, 0);
                ga[(t + 1) & 1][1] = gfrag(t + 1, 1);
            }
            dvT[t] = mfma32(ga[t & 1][0], pb0, dvT[t]);
            dvT[t] = mfma32(ga[t & 1][1], pb1, dvT[t]);
#pragma unroll
            for (int i = 4 * t / NT; i < 4 * (t + 1) / NT; ++i) {
                const int v0 = 4 * i;
                const float dl[4] = {lnext.x, lnext.y, lnext.z, lnext.w};
                if (i < 3)
                    lnext = stat4(sDel, v0 + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ds[v0 + e] = pr[v0 + e] * __builtin_fmaf(dp[v0 + e], kPScaleInv, -dl[e]);
            }
            LH_FENCE;
        }
        const uint4 db0 = pack8h(ds), db1 = pack8h(ds + 8);
        // dK, with the stage's dS tile (queries q0.., keys kw..) stored for
        // the dQ kernel behind its last products: key-major, the lane's key
        // row of 32 queries is its two fp16 runs (queries 8g.. and 16 + 8g..)
        ga[0][2] = gfrag(0, 2);
        ga[0][3] = gfrag(0, 3);
        LH_FENCE;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t + 1 < NT) {
                ga[(t + 1) & 1][2] = gfrag(t + 1, 2);
                ga[(t + 1) & 1][3] = gfrag(t + 1, 3);
            }
            dkT[t] = mfma32(ga[t & 1][2], db0, dkT[t]);
            dkT[t] = mfma32(ga[t & 1][3], db1, dkT[t]);
            if (t == NT - 1 && a.dst != nullptr) {
                const int qt = q0 / 32;
                uint16_t *row = dst_head + ((int64_t)qt * (qt + 1) / 2 + kt) * 1024 + ql * 32 + 8 * g;
                store16_stream(row, db0);
                store16_stream(row + 16, db1);
            }
            LH_FENCE;
        }
    };
    issue(k0, ring);
    issue(k0 + min(1, nst - 1) * BQ, ring + St::SIZE); // (the only stage again when nst = 1)
    auto next = [&]() { slot = slot == 2 ? 0 : slot + 1; };
    // stages before this wave's keys; the diagonal one; interior ones; the
    // last one when it reaches past S (one code path per loop, so the
    // accumulators stay in place)
    const int last_int = (k0 + nst * BQ > S) ? nst - 1 : nst; // first stage that needs the S mask
    int it = 0;
    for (; it < min(wave, nst); ++it, next())
        stage(it, Mode<0>());
    if (it < nst) {
        stage(it, Mode<2>());
        ++it;
        next();
    }
    for (; it < last_int; ++it, next())
        stage(it, Mode<1>());
    for (; it < nst; ++it, next())
        stage(it, Mode<2>());
    wait_async(); // transfers past the last stage

    float *dk = a.dk + (hS + key) * D;
    float *dv = a.dv + (hS + key) * D;
    const float sk = ldexpf(a.scale, -(exd + exv + exq)), sv = ldexpf(kPScaleInv, -exd);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int dim = 32 * t + 8 * i4 + 4 * g;
            *reinterpret_cast<float4 *>(dk + dim) = make_float4(dkT[t][4 * i4] * sk, dkT[t][4 * i4 + 1] * sk,
                                                                dkT[t][4 * i4 + 2] * sk, dkT[t][4 * i4 + 3] * sk);
            *reinterpret_cast<float4 *>(dv + dim) =
                make_float4(dvT[t][4 * i4] * sv, dvT[t][4 * i4 + 1] * sv, dvT[t][4 * i4 + 2] * sv, dvT[t][4 * i4 + 3] * sv);
        }
}

template <int D>
static void launch_dkdv_t(const dim3 grid, const AttnBwdArgs &a, bool klo, hipStream_t s)
{
    if (klo)
        hipLaunchKernelGGL((k_attn_bwd_dkdv<D, true>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((k_attn_bwd_dkdv<D, false>), grid, dim3(256), 0, s, a);
}

hipError_t launch_attn_bwd_dkdv(const Plan &pl, const AttnBwdArgs &a, hipStream_t s)
{
    const unsigned nkb = (unsigned)((pl.S + 127) / 128);
    const dim3 grid(nkb * pl.H);
    const bool klo = pl.dt == LH_F32; // see the precision note at the top of this file
    if (pl.d == 128)
        launch_dkdv_t<128>(grid, a, klo, s);
    else
        launch_dkdv_t<64>(grid, a, klo, s);
    return hipGetLastError();
}

// ============================================================== backward: dQ
// dQ = scale * dS K from the dS tiles the dK/dV kernel stored (key-major,
// fp16: the values it used itself), so S and dP are not recomputed. One
// workgroup per 256 queries (eight waves of 32, one workgroup per CU): K^T of
// 64 keys per stage, shared by the eight waves, and each wave's own dS tiles
// of the stage go through a three-slot LDS ring with two stages in flight.
// Per 32x32 tile: dQ^T += K^T dS^T, 8 MFMAs, the dS^T operands read down the
// key-major tile's columns.
template <int D>
struct DqStage {
    static constexpr int NW = 8;                  // waves per workgroup
    static constexpr int BN = 64;
    static constexpr int TCH = BN / 8;            // chunks per K^T row
    static constexpr int KT = 0, KSIZE = D * TCH; // K^T [D][BN]
    static constexpr int DS = KSIZE;              // dS: [wave][subtile][32 keys][32 queries]
    static constexpr int DSW = 2 * 32 * 4;        // chunks per wave
    static constexpr int SIZE = KSIZE + NW * DSW;
    static constexpr int KU = KSIZE / (64 * NW);  // K^T load rounds
    static constexpr int LOADS = KU + 4;          // transfers per thread and stage
    static constexpr int NSLOT = 3;
};

template <int D>
__global__ __launch_bounds__(512, 1) void k_attn_bwd_dq(AttnBwdArgs a)
{
    typedef DqStage<D> St;
    constexpr int BM = 32 * St::NW, BN = St::BN, TCH = St::TCH;
    constexpr int NT = D / 32;
    __shared__ uint4 ring[St::NSLOT * St::SIZE];

    const int nqb = (int)((a.S + BM - 1) / BM);
    const int h = blockIdx.x % a.H;
    const int qb = nqb - 1 - (int)(blockIdx.x / a.H); // longest rows first
    const int64_t q0 = (int64_t)qb * BM;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // uniform: LDS bases stay scalar
    const int64_t qw = q0 + wave * 32;
    const int64_t hS = (int64_t)h * a.S_pad;
    const int qt = (int)(qw / 32); // this wave's query tile: key tiles 0..qt
    const bool live = qw < a.S;

    // K^T chunk byte offsets (the stage moves the uniform base)
    uint32_t koff[St::KU];
#pragma unroll
    for (int u = 0; u < St::KU; ++u) {
        const int c = 64 * St::NW * u + tid, dim = c / TCH;
        koff[u] = 2u * ((uint32_t)dim * (uint32_t)a.S_pad + (uint32_t)(swzg<TCH>(dim, c % TCH) * 8));
    }
    const uint16_t *const kht = a.khi_t + (int64_t)h * D * a.S_pad;
    // this wave's dS tiles (qt, kt) are contiguous in kt; lane chunk = 16 B
    const uint16_t *const dsrow = a.dst + (int64_t)h * a.dst_head + (int64_t)qt * (qt + 1) / 2 * 1024;
    // a 32x32 tile is 128 chunks (32 key rows of 64 B): two DMA rounds, in
    // order. The dS^T operand of lane (c32, g) is query c32 of keys 8g .. 8g+7
    // (and 16 + 8g ..): two transposing reads each, lane 4R + m of 16-lane
    // group G addressing key 8g + 4n + R (g = G >> 1), queries 16(G & 1) + 4m
    // .. +3; a half wave reads four whole rows, so no bank is hit twice
    const uint32_t doff0 = 16u * (uint32_t)lane, doff1 = doff0 + 16u * 64u;
    uint32_t troff[2];
#pragma unroll
    for (int n = 0; n < 2; ++n)
        troff[n] = 64u * (uint32_t)(8 * g + 4 * n + ((lane >> 2) & 3)) + 2u * (uint32_t)(16 * ((lane >> 4) & 1) + 4 * (lane & 3));

    const int64_t kend = min(q0 + BM, a.S);
    const int nkb = (int)((kend + BN - 1) / BN);
    auto slot = [&](int kb) { return ring + (kb % St::NSLOT) * St::SIZE; };
    // Every thread issues St::LOADS transfers per stage, so a count of the
    // transfers in flight tells which stage has landed: past the last stage
    // the last one is loaded again, and a wave whose query tile ends before a
    // key tile loads its own diagonal tile (never read) in its place.
    auto issue = [&](int kb) {
        const uint4 *base = slot(kb);
        const int kc = min(kb, nkb - 1);
#pragma unroll
        for (int u = 0; u < St::KU; ++u)
            dma16(kht + (int64_t)kc * BN, koff[u], base + St::KT + 64 * St::NW * u + 64 * wave);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint16_t *tb = dsrow + (int64_t)min(2 * kc + j, qt) * 1024;
            const uint4 *lb = base + St::DS + wave * St::DSW + j * 128;
            dma16_nt(tb, doff0, lb);
            dma16_nt(tb, doff1, lb + 64);
        }
    };

    f32x16_t dqT[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        dqT[t] = zero16();

    issue(0);
    issue(1);
    for (int kb = 0; kb < nkb; ++kb) {
        const uint4 *base = slot(kb);
        wait_async_n<St::LOADS>(); // stage kb has landed (kb + 1 may be in flight)
        lds_barrier();             // ... visible to all waves; stage kb - 1's slot is free
        issue(kb + 2);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int ktile = 2 * kb + j;
            if (!live || ktile > qt)
                break;
            // dS^T operand: query c32, keys 8g.. and 16 + 8g.. of the tile
            const uint4 *dt = base + St::DS + wave * St::DSW + j * 128;
            const uint2 r0 = lds_tr16(dt, troff[0]), r1 = lds_tr16(dt, troff[1]);
            const uint2 r2 = lds_tr16(dt, troff[0] + 1024u), r3 = lds_tr16(dt, troff[1] + 1024u);
            const uint4 ds0 = make_uint4(r0.x, r0.y, r1.x, r1.y), ds1 = make_uint4(r2.x, r2.y, r3.x, r3.y);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int dim = 32 * t + c32;
                dqT[t] = mfma32(base[St::KT + dim * TCH + swzg<TCH>(dim, 4 * j + g)], ds0, dqT[t]);
                dqT[t] = mfma32(base[St::KT + dim * TCH + swzg<TCH>(dim, 4 * j + 2 + g)], ds1, dqT[t]);
            }
        }
    }
    wait_async(); // the transfers past the last stage

    const int64_t query = qw + c32;
    float *dq = a.dq + (hS + query) * D;
    // the tiles hold 2^(ex_do + ex_v) dS, the staged keys 2^ex_k K
    const float sq = ldexpf(a.scale, -(a.ex[3 * a.H + h] + a.ex[2 * a.H + h] + a.ex[a.H + h]));
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
            *reinterpret_cast<float4 *>(dq + 32 * t + 8 * i4 + 4 * g) =
                make_float4(dqT[t][4 * i4] * sq, dqT[t][4 * i4 + 1] * sq, dqT[t][4 * i4 + 2] * sq, dqT[t][4 * i4 + 3] * sq);
}

// ============================================================== backward: dQ, recomputed
// dQ without stored dS tiles (the plan drops them when the causal half of
// S x S per head would take too much of the workspace): the query side of
// the softmax gradient, with S and dP formed again from the gathered rows.
// One workgroup per 256 queries (eight waves of 32, one workgroup per CU);
// keys stream through a three-slot LDS ring 32 at a time, two stages in
// flight, each stage shared by the eight waves. Per key block, as in the
// forward, keys are the rows of every product so that a lane owns one query:
//   S^T = K Q^T (the logits the other kernels form, same operands),
//   P^T = 2^(S^T log2(e)/sqrt(d) - LSE + 15)  (probabilities times 2^15),
//   dP^T = V dO^T (the fp16 pair of dO_sub, as in the dK/dV kernel),
//   dS^T = P^T (dP^T 2^-15 - delta 2^-15)    (delta is per query: per lane),
//   dQ^T += K^T dS^T, with dS^T straight from the accumulator as operand B
// (the kappa row order of K and V puts each lane's keys in runs of 8).
//
// A stage is a list of 64-chunk units (one MFMA operand fragment, or 1 KiB
// of an fp8 tile), unit u at LDS chunk 64 u: K hi rows (NS units, k-step s
// in unit s), V rows (NS), K^T (NS: fragment (hh, t) in unit hh NT + t), then
// the fp8 K and V tiles (NS/2 each, linear copies) for bf16 inputs or the
// fp16 K lo rows (NS) for fp32 inputs. Unit 8 r + w is transferred by wave w
// in round r, so every thread issues the same number of transfers per stage.
template <int D, bool KLO> struct DqrcStage {
    static constexpr int BN = 32, NW = 8;
    static constexpr int NS = D / 16;
    static constexpr int KH = 0, VR = 64 * NS, KT = 128 * NS;  // in chunks
    static constexpr int KL = 192 * NS;                        // fp8 K tile, or K lo rows
    static constexpr int V8 = KL + 32 * NS;                    // fp8 V tile (bf16 inputs)
    static constexpr int UNITS = 4 * NS, SIZE = 64 * UNITS;    // 32 KiB per stage at d = 128
    static constexpr int LOADS = UNITS / NW;                   // transfers per thread and stage
    static constexpr int NSLOT = 3;
    static_assert(UNITS % NW == 0, "whole rounds");
};

template <int D, bool KLO>
__global__ __launch_bounds__(512, 1) void k_attn_bwd_dq_rc(AttnBwdArgs a)
{
    typedef DqrcStage<D, KLO> St;
    constexpr int BM = 32 * St::NW, BN = St::BN;
    constexpr int NS = D / 16, NT = D / 32, NM = D / 64;
    __shared__ uint4 ring[St::NSLOT * St::SIZE];

    const int nqb = (int)((a.S + BM - 1) / BM);
    const int h = blockIdx.x % a.H;
    const int qb = nqb - 1 - (int)(blockIdx.x / a.H); // longest rows first
    const int64_t q0 = (int64_t)qb * BM;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, c32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // uniform: LDS bases stay scalar
    const int64_t qw = q0 + wave * 32;
    const int64_t hS = (int64_t)h * a.S_pad;
    const int64_t kend = min(q0 + BM, a.S);
    const int nkb = (int)((kend + BN - 1) / BN);
    // last key block this wave uses: its diagonal block (rows past S: the
    // workgroup's last one; their results are never read)
    const int jl = (int)min((int64_t)(nkb - 1), qw / BN);

    const uint16_t *khi = a.khi + hS * D, *klo = a.klo + hS * D, *vr = a.v + hS * D;
    const uint8_t *k8 = a.k8 + hS * D, *v8 = a.v8 + hS * D;
    const uint16_t *kt = a.khi_t + (int64_t)h * D * a.S_pad;
    // Round r of this wave: unit 8 r + wave. kind: 0 K hi, 1 V, 2 K^T, 3 K lo
    // rows, 4 fp8 K tile, 5 fp8 V tile (uniform over the wave); off: this
    // lane's source byte offset within the stage's first key.
    int kind[St::LOADS];
    uint32_t off[St::LOADS];
#pragma unroll
    for (int r = 0; r < St::LOADS; ++r) {
        const int u = St::NW * r + wave;
        if (u < 3 * NS) {
            const int f = u % NS;
            kind[r] = u / NS;
            if (kind[r] == 2) { // K^T fragment (hh, t): dimension 32 t + c32, keys 16 hh + 8 g .. +7
                const int hh = f / NT, t = f % NT;
                off[r] = 2u * ((uint32_t)(32 * t + c32) * (uint32_t)a.S_pad + (uint32_t)(16 * hh + 8 * g));
            } else { // row fragment of k-step f: key row kappa(c32), dimensions 16 f + 8 g .. +7
                off[r] = 2u * (uint32_t)(kappa(c32) * D + (2 * f + g) * 8);
            }
        } else if constexpr (KLO) {
            kind[r] = 3;
            off[r] = 2u * (uint32_t)(kappa(c32) * D + (2 * (u - 3 * NS) + g) * 8);
        } else { // fp8 tiles: linear copies
            const int i = u - 3 * NS;
            kind[r] = i < NS / 2 ? 4 : 5;
            off[r] = 16u * (uint32_t)(64 * (i % (NS / 2)) + lane);
        }
    }
    auto slot = [&](int kb) { return ring + (kb % St::NSLOT) * St::SIZE; };
    // Past the last stage the last one is loaded again (never read), so every
    // stage is LOADS transfers per thread and a count of transfers in flight
    // tells which stage has landed.
    auto issue = [&](int kb) {
        const int64_t k0 = (int64_t)min(kb, nkb - 1) * BN;
        const uint4 *base = slot(kb);
#pragma unroll
        for (int r = 0; r < St::LOADS; ++r) {
            const uint4 *dst = base + 64 * (St::NW * r + wave);
            switch (kind[r]) {
            case 0: dma16(khi + k0 * D, off[r], dst); break;
            case 1: dma16(vr + k0 * D, off[r], dst); break;
            case 2: dma16(kt + k0, off[r], dst); break;
            case 3: dma16(klo + k0 * D, off[r], dst); break;
            case 4: dma16(k8 + k0 * D, off[r], dst); break;
            default: dma16(v8 + k0 * D, off[r], dst); break;
            }
        }
    };

    // this lane's query as operand B: Q hi, dO_sub hi, and their lo parts
    // (fp16 for fp32 inputs; the fp8 tiles for bf16 inputs, which keep query
    // qw + c32 at lane position kappa(c32) + 32g)
    const int64_t qrow = (hS + qw + c32) * D;
    uint4 qh[NS], dh[NS], ql[KLO ? NS : 1], dl[KLO ? NS : 1], q8[KLO ? 1 : NM][2], d8[KLO ? 1 : NM][2];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        qh[s] = ld16(a.qhi + qrow + 16 * s + 8 * g);
        dh[s] = ld16(a.dohi + qrow + 16 * s + 8 * g);
        if constexpr (KLO) {
            ql[s] = ld16(a.qlo + qrow + 16 * s + 8 * g);
            dl[s] = ld16(a.dolo + qrow + 16 * s + 8 * g);
        }
    }
    int qs = 0, ks = 0, vs = 0, ds8 = 0;
    if constexpr (!KLO) {
        const int64_t t8 = (hS + qw) * D + 16 * (kappa(c32) + 32 * g);
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                q8[m][q] = *reinterpret_cast<const uint4 *>(a.qlo8 + t8 + 2048 * m + 1024 * q);
                d8[m][q] = *reinterpret_cast<const uint4 *>(a.dolo8 + t8 + 2048 * m + 1024 * q);
            }
        qs = 127 + kFp8Exp[0];
        ks = 127 + kFp8Exp[1];
        vs = 127 + kFp8Exp[2];
        ds8 = 127 + kFp8Exp[3];
    }
    const int exq = a.ex[h], exk = a.ex[a.H + h], exv = a.ex[2 * a.H + h], exd = a.ex[3 * a.H + h];
    const float scale_log2 = ldexpf(a.scale_log2, -(exq + exk)); // staged rows: see the dK/dV kernel
    const float lq = a.lse[hS + qw + c32];   // log2-domain LSE - 15 of this lane's query
    const float dq8 = a.delta[hS + qw + c32]; // delta * 2^-15
    // consume the loads here, before the ring's transfers are in flight (see
    // the forward kernel)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        asm volatile("" ::"v"(qh[s].x), "v"(dh[s].x));
        if constexpr (KLO)
            asm volatile("" ::"v"(ql[s].x), "v"(dl[s].x));
    }
    if constexpr (!KLO) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
            asm volatile("" ::"v"(q8[m][0].x), "v"(q8[m][1].x), "v"(d8[m][0].x), "v"(d8[m][1].x));
        asm volatile("" ::"v"(qs), "v"(ks), "v"(vs), "v"(ds8));
    }
    asm volatile("" ::"v"(lq), "v"(dq8));

    f32x16_t dq[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        dq[t] = zero16();
    issue(0);
    issue(1);
    for (int j = 0; j < nkb; ++j) {
        wait_async_n<St::LOADS>(); // stage j has landed (j + 1 may be in flight)
        lds_barrier();             // ... visible to all waves; stage j - 1's slot is free
        issue(j + 2);
        if (j > jl) // (uniform) keys after every query of this wave
            continue;
        const uint4 *base = slot(j);
        f32x16_t st = zero16(), dp = zero16();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const uint4 kf = base[St::KH + 64 * s + lane];
            st = mfma32(kf, qh[s], st);
            if constexpr (KLO) {
                st = mfma32(base[St::KL + 64 * s + lane], qh[s], st);
                st = mfma32(kf, ql[s], st);
            }
            const uint4 vf = base[St::VR + 64 * s + lane];
            dp = mfma32(vf, dh[s], dp);
            if constexpr (KLO)
                dp = mfma32(vf, dl[s], dp);
        }
        if constexpr (!KLO) {
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                st = mfma8(base[St::KL + 128 * m + lane], base[St::KL + 128 * m + 64 + lane], q8[m][0], q8[m][1], st,
                           ks, qs);
                dp = mfma8(base[St::V8 + 128 * m + lane], base[St::V8 + 128 * m + 64 + lane], d8[m][0], d8[m][1], dp,
                           vs, ds8);
            }
        }
        // register v holds key 16(v/8) + 8g + v%8 of the block; keys after
        // the lane's query (diagonal block) have P = 0, so dS = 0
        const int rel = (int)((int64_t)j * BN - qw); // first key of the block - first query of the wave
        float ds[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const bool ok = rel + 16 * (v >> 3) + 8 * g + (v & 7) <= c32;
            const float pr = ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(st[v], scale_log2, -lq)) : 0.0f;
            ds[v] = pr * __builtin_fmaf(dp[v], kPScaleInv, -dq8);
        }
        const uint4 db0 = pack8h(ds), db1 = pack8h(ds + 8);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            dq[t] = mfma32(base[St::KT + 64 * t + lane], db0, dq[t]);
            dq[t] = mfma32(base[St::KT + 64 * (NT + t) + lane], db1, dq[t]);
        }
    }
    wait_async(); // the transfers past the last stage

    float *dqr = a.dq + qrow;
    const float sq = ldexpf(a.scale, -(exd + exv + exk));
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
            *reinterpret_cast<float4 *>(dqr + 32 * t + 8 * i4 + 4 * g) =
                make_float4(dq[t][4 * i4] * sq, dq[t][4 * i4 + 1] * sq, dq[t][4 * i4 + 2] * sq, dq[t][4 * i4 + 3] * sq);
}

template <int D>
static void launch_dq_t(const Plan &pl, const AttnBwdArgs &a, bool klo, hipStream_t s)
{
    if (pl.ds_tiles) { // 32 * DqStage::NW queries per workgroup
        constexpr int BM = 32 * DqStage<D>::NW;
        const dim3 grid((unsigned)((pl.S + BM - 1) / BM) * pl.H);
        hipLaunchKernelGGL((k_attn_bwd_dq<D>), grid, dim3(64 * DqStage<D>::NW), 0, s, a);
        return;
    }
    constexpr int NW = DqrcStage<D, false>::NW; // 32 queries per wave
    const dim3 grid((unsigned)((pl.S + 32 * NW - 1) / (32 * NW)) * pl.H);
    if (klo)
        hipLaunchKernelGGL((k_attn_bwd_dq_rc<D, true>), grid, dim3(64 * NW), 0, s, a);
    else
        hipLaunchKernelGGL((k_attn_bwd_dq_rc<D, false>), grid, dim3(64 * NW), 0, s, a);
}

hipError_t launch_attn_bwd_dq(const Plan &pl, const AttnBwdArgs &a, hipStream_t s)
{
    const bool klo = pl.dt == LH_F32;
    if (pl.d == 128)
        launch_dq_t<128>(pl, a, klo, s);
    else
        launch_dq_t<64>(pl, a, klo, s);
    return hipGetLastError();
}

} // namespace lh
