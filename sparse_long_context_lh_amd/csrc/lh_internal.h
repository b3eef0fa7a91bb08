// Host-side plan of one Lighthouse layer call and the argument blocks of its
// kernels. Everything here is computed on the host from the shape alone, so
// the launch sequence is static (no device value is ever read back).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/lh.h"

namespace lh {

constexpr int kMaxLevels = 8;       // L <= 8
constexpr int kStratum = 2048;      // entries per top-K stratum
constexpr int kMaxSelTotal = 16384; // (L-1)*k held in LDS by the index kernel
constexpr int kSubseqAlign = 256;   // S is padded to this for the attention tiles
constexpr int64_t kMaxN = int64_t(1) << 27;
constexpr int kMaxHeads = 65535; // heads run along the grid's y dimension
// Default largest workspace share of the backward's stored dS tiles (the
// causal half of S x S per head, fp16; 32 GiB is about a ninth of the card's
// memory, and at 16 heads holds the tiles up to S of about 46K). Above it the
// dQ kernel recomputes S and dP from the gathered rows instead, and the
// workspace stays O(S d). The process-wide value is set with
// lh_set_ds_tile_budget.
constexpr size_t kDsTileBudgetDefault = size_t(32) << 30;
size_t ds_tile_budget();
// Largest workspace a plan may ask for (64 TiB): shapes beyond it are reported
// as unsupported rather than sized.
constexpr size_t kMaxWorkspace = size_t(1) << 46;

// Extra workspace regions that are not exposed through lh_region.
enum InternalRegion {
    IR_POOLED = LH_R_COUNT, // fp32 [3][H][mat_rows][d]: materialized pooled levels
    IR_DOHI,                // fp16 [H][S_pad][d]: hi part of dO_sub
    IR_DOLO,                // fp16 [H][S_pad][d]: lo part of dO_sub
    IR_DELTA,               // fp32 [H][S_pad]: rowsum(dO_sub * O_sub) * 2^-15
    IR_LSE15,               // fp32 [H][S_pad]: log2-domain LSE - 15
    IR_DST,                 // fp16 [H][T(T+1)/2][32][32], T = S_pad/32: dS tiles (key-major), causal half
    IR_FPART,               // fp32 window sums [3][H][fpart_rows][d], then maxima [H][fpart_rows]
    IR_SPART,               // fp32 [H][spart_rows][d]: dO window sums (u-space)
    IR_QLO8,                // e4m3 [H][S_pad/32][32 d] (bf16 inputs): Q lo part, fp8 tiles
    IR_K8,                  // e4m3 [H][S_pad/32][32 d] (bf16 inputs): K hi part, fp8 tiles
    IR_V8,                  // e4m3 [H][S_pad/32][32 d] (bf16 inputs): V, fp8 tiles
    IR_DOLO8,               // e4m3 [H][S_pad/32][32 d] (bf16 inputs): lo part of dO_sub, fp8 tiles
    IR_XMAX,                // fp32 [3][H][nxmax]: largest |q|, |k| element and |v| row norm of each wave's input rows
    IR_DOMAX,               // fp32 [H][S_pad/64]: largest dO_sub row norm of each 64-row tile
    IR_COUNT
};

// Per-head power-of-two scales of the rows staged in fp16 (gathered Q, K, V;
// dO_sub; LH_R_EXP): a head's largest Q or K element, and its largest V or
// dO_sub row norm, is brought into [2^(t-1), 2^t) with t = kExpTarget[...],
// so every value stays inside fp16's range whatever the inputs' scale.
// Scaling by a power of two commutes with rounding, so away from fp16's
// subnormals the products are the same up to that factor. The targets bound
// |dP| = |dO_sub . V| <= 2^9 2^5 and |dS| = |P (dP - delta)| <= 2^15 (fp16
// holds 65504); pooled rows are means, so the inputs' maxima bound them.
constexpr int kExpTarget[4] = {12, 12, 5, 9}; // Q, K (element), V, dO_sub (row norm)

// The e4m3 copies of staged operands (bf16 inputs: the query's lo part, the
// key rows, the value rows, dO_sub's lo part) hold x * 2^-e with a fixed e:
// the staging above bounds each of them, and e takes that bound to 2^8 = 256,
// inside e4m3's largest value 448. A staged query element is below 2^12, so
// its lo part is at most half an fp16 ulp there, 2^0; keys are below 2^12;
// values below 2^5 (their row norm is); dO_sub elements below 2^9, so its lo
// part is at most 2^-3. The MFMA takes 127 + e as the scale byte.
constexpr int kFp8Exp[4] = {kExpTarget[0] - 20, kExpTarget[1] - 8, kExpTarget[2] - 8, kExpTarget[3] - 20};
constexpr int kExpTile = 64;                   // rows per tile of the dO_sub maxima

// Row tiles of the front pass and of the scatter-back adjoint. A lane group
// (d/8 lanes, 8 elements each) owns R = p^NC consecutive rows; a workgroup of
// 256 threads owns NLG * R rows. Levels whose windows fit a tile (p^l divides
// it) are finished inside the tile kernel; coarser ones by one small kernel
// per level over the tile kernel's window sums. The front pass (three
// tensors) runs 4 rows per lane group (8 for p = 8); the scatter-back adjoint
// (one tensor) 16 (8 for p = 8).
constexpr int clog2(int x) { return x <= 1 ? 0 : 1 + clog2(x / 2); }
constexpr int front_nc(int lp) { return lp == 1 ? 2 : 1; }
constexpr int sbwd_nc(int lp) { return lp == 1 ? 4 : (lp == 2 ? 2 : 1); }
template <int D, int LP, int NC_> struct TileShape {
    static constexpr int LANES = D / 8, NLG = 256 / LANES;
    static constexpr int NC = NC_;
    static constexpr int R = 1 << (NC * LP);
    static constexpr int T = NLG * R;
    static constexpr int LMAX = clog2(T) / LP;
};
inline int tile_rows(int d, int log2p, int nc) { return (256 / (d / 8)) << (nc * log2p); }
inline int tile_levels(int d, int log2p, int nc) { return clog2(tile_rows(d, log2p, nc)) / log2p; }

struct Plan {
    int64_t N;
    int H, d, L, p, log2p, k;
    lh_dtype dt;
    int64_t n[kMaxLevels];       // entries at level l
    int64_t lvl_off[kMaxLevels]; // offset of level l inside one head's score / slot block
    int64_t lvl_total;           // sum of n[l]
    int64_t S, S_pad;
    int C[kMaxLevels];           // strata at level l (l >= 1)
    int strata_total;            // sum over l >= 1
    uint32_t mat_mask;           // bit l set: level l pooled rows are written by the front kernel
    int64_t mat_off[kMaxLevels]; // row offset of a materialized level inside one head's pooled block
    int64_t mat_rows;
    int LT;                      // levels 1..LT are finished inside the front pass's row tiles
    int LTs;                     // the same for the scatter-back adjoint's row tiles
    int64_t fpart_off[kMaxLevels]; // row offset of level l's window sums in a head's IR_FPART block
    int64_t fpart_rows;
    int64_t spart_n[kMaxLevels];   // u-space windows of level l kept in IR_SPART (l >= LT)
    int64_t spart_off[kMaxLevels];
    int64_t spart_rows;
    int64_t xmax_tile;           // input rows per front tile (four wave maxima each)
    int64_t nxmax;               // wave maxima per head and tensor
    bool ds_tiles;               // the dK/dV kernel stores dS tiles for the dQ kernel (else dQ recomputes)
    size_t off[IR_COUNT], bytes[IR_COUNT];
    size_t fwd_total;            // end of the regions lh_forward writes
    size_t total;
};

// 32x32 tiles of the causal half of the S_pad x S_pad score matrix (kt <= qt).
inline int64_t dst_tiles(int64_t S_pad)
{
    const int64_t t = S_pad / 32;
    return t * (t + 1) / 2;
}

// Fills `pl` and returns LH_OK, or the validation error.
lh_status make_plan(int64_t N, int H, int d, int L, int p, int k, lh_dtype dt, Plan *pl);

// ---------------------------------------------------------------- kernels
struct FrontArgs {
    const void *q, *k, *v;
    float *scores;           // [H][lvl_total]
    float *pooled;           // [3][H][mat_rows][d]
    int64_t N, lvl_total, mat_rows, tensor_stride; // tensor_stride = H*mat_rows*d
    int64_t lvl_off[kMaxLevels];
    int64_t mat_off[kMaxLevels]; // -1: level not materialized
    float *part;                 // IR_FPART: window sums of levels LT .. L-2, then their maxima
    int64_t part_rows;
    int64_t part_off[kMaxLevels];
    int H, L, log2p, LT;
    int scorer; // lh_scorer
    float *xmax;     // IR_XMAX: largest |q|, |k|, |v| of each wave's rows, [3][H][nxmax]
    int64_t nxmax;
};

struct TopkArgs {
    const float *scores; // [H][lvl_total]
    int32_t *sel;        // [L-1][H][k]
    int32_t *slot;       // [H][lvl_total]
    int64_t lvl_total;
    int64_t lvl_off[kMaxLevels];
    int64_t n[kMaxLevels];
    int C[kMaxLevels];
    int strata_before[kMaxLevels]; // strata of levels 1..l-1
    int L, log2p, k;
};

struct IndexArgs {
    const int32_t *sel;  // [L-1][H][k]
    int32_t *slot;       // [H][lvl_total]
    int32_t *ent;        // [H][S_pad]
    int64_t lvl_total, S, S_pad;
    int64_t lvl_off[kMaxLevels];
    int64_t n[kMaxLevels];
    int L, log2p, k;
};

struct GatherArgs {
    const void *q, *k, *v;     // [H][N][d] inputs
    const float *pooled;       // [3][H][mat_rows][d]
    const int32_t *ent;        // [H][S_pad]
    uint16_t *hi[3];           // fp16 [H][S_pad][d]: Q hi, K hi, V
    uint16_t *lo[2];           // fp32 inputs: fp16 [H][S_pad][d] Q lo, K lo (bf16 inputs: null)
    uint16_t *hi_t[2];         // fp16 [H][d][S_pad]: transposes of K hi and V
    uint8_t *t8[3];            // bf16 inputs: e4m3 tiles of the Q lo part, K hi and V (else null)
    const int32_t *ex;         // LH_R_EXP: the rows are staged as x * 2^ex[t][h]
    int64_t N, S, S_pad, mat_rows, tensor_stride;
    int64_t mat_off[kMaxLevels];
    int64_t n[kMaxLevels];
    int H, L, log2p;
};

struct AttnFwdArgs {
    const uint16_t *qhi, *qlo, *khi, *klo, *vt; // fp16 gathered rows (vt: [H][d][S_pad])
    const uint8_t *qlo8, *k8;                   // bf16 inputs: e4m3 tiles of the Q lo part and of K (kFp8Exp)
    float *o;                           // [H][S_pad][d]
    float *lse;                         // [H][S_pad]
    const int32_t *ex;                  // LH_R_EXP: staged rows are q 2^ex_q, k 2^ex_k, v 2^ex_v
    int64_t S, S_pad;
    int H;
    int for_bwd;      // 1: the lo products the backward's context needs; 0: a call no backward follows
    float scale_log2; // log2(e) / sqrt(d)
};

struct AttnBwdArgs {
    const uint16_t *qhi, *qlo, *khi, *klo, *v;   // fp16 gathered rows [H][S_pad][d]
    const uint8_t *qlo8, *k8, *v8, *dolo8;       // bf16 inputs: e4m3 tiles of the Q lo part, K, V, dO lo part (kFp8Exp)
    const uint16_t *khi_t;                      // fp16 [H][d][S_pad]
    const uint16_t *dohi, *dolo;                // fp16 pair of dO_sub
    const float *lse, *delta;                        // [H][S_pad]: log2 LSE - 15, rowsum(dO o O) * 2^-15
    float *dq, *dk, *dv;                             // [H][S_pad][d]
    uint16_t *dst;     // IR_DST: tile (qt, kt), kt <= qt, at (qt(qt+1)/2 + kt) * 1024 in a head's block
    int64_t dst_head;  // elements per head of IR_DST
    const int32_t *ex; // LH_R_EXP: staged rows are the true rows times 2^ex (Q, K, V, dO_sub)
    int64_t S, S_pad;
    int H;
    float scale_log2; // log2(e) / sqrt(d)
    float scale;      // 1 / sqrt(d)
};

struct ScatterArgs {
    const float *osub;   // [H][S_pad][d]
    const int32_t *slot; // [H][lvl_total]
    void *out;           // [H][N][d] in the input dtype
    int64_t N, lvl_total, S_pad;
    int64_t lvl_off[kMaxLevels];
    int H, L, log2p;
};

struct ScatterBwdArgs {
    const void *dout;    // [H][N][d] in the input dtype
    const int32_t *slot; // [H][lvl_total]
    float *dosub;        // [H][S_pad][d]
    int64_t N, lvl_total, S_pad;
    int64_t lvl_off[kMaxLevels];
    float *part;         // IR_SPART: u-space window sums of levels LT .. L-2
    int64_t part_rows;   // rows of one head's IR_SPART block
    int64_t part_off[kMaxLevels], part_n[kMaxLevels];
    int H, L, log2p, LT;
};

struct BwdPrepArgs {
    const float *dosub, *osub;       // [H][S_pad][d]
    uint16_t *dohi, *dolo;           // fp16 pair (dolo: fp32 inputs; bf16: null, the e4m3 tile instead)
    float *delta;              // [H][S_pad]: rowsum * 2^-15
    const float *lse;          // [H][S_pad]: log2-domain LSE of the forward
    float *lse15;              // [H][S_pad]: lse - 15
    uint8_t *dolo8;            // bf16 inputs: e4m3 tiles of the lo part (kFp8Exp[3]; else null)
    const int32_t *ex;         // LH_R_EXP: dO_sub is staged times 2^ex_do; delta is kept times 2^(ex_do + ex_v)
    int64_t S, S_pad;
    int H;
};

// Largest magnitudes and the per-head exponents of the fp16 staging.
struct AbsMaxArgs {
    const void *x[3];   // [H][N][d] inputs (L = 1: the front pass does not run)
    float *xmax;        // [3][H][nxmax]
    int64_t N, nxmax, tile;
    int H;
};
struct RowMaxArgs {
    const float *src;   // [H][S_pad][d] dO_sub
    float *dst;         // [H][S_pad/64]
    int64_t S, S_pad;
};
struct HeadExpArgs {
    const float *m;     // [nt][H][count] maxima
    int64_t count;
    int nt, H, first;   // exponents go to ex[first + t][h]
    int32_t *ex;        // [4][H]
};

struct PoolBwdArgs {
    const float *dsub[3];  // [H][S_pad][d]: dQ_sub, dK_sub, dV_sub
    const int32_t *slot;   // [H][lvl_total]
    void *dx[3];           // [H][N][d] in the input dtype
    int64_t N, lvl_total, S_pad;
    int64_t lvl_off[kMaxLevels];
    int H, L, log2p;
};

hipError_t launch_front(const Plan &pl, const FrontArgs &a, hipStream_t s);
hipError_t launch_topk(const Plan &pl, const TopkArgs &a, hipStream_t s);
hipError_t launch_index(const Plan &pl, const IndexArgs &a, hipStream_t s);
hipError_t launch_gather(const Plan &pl, const GatherArgs &a, hipStream_t s);
hipError_t launch_attn_fwd(const Plan &pl, const AttnFwdArgs &a, hipStream_t s);
hipError_t launch_scatter(const Plan &pl, const ScatterArgs &a, hipStream_t s);
hipError_t launch_scatter_bwd(const Plan &pl, const ScatterBwdArgs &a, hipStream_t s);
hipError_t launch_bwd_prep(const Plan &pl, const BwdPrepArgs &a, hipStream_t s);
hipError_t launch_attn_bwd_dkdv(const Plan &pl, const AttnBwdArgs &a, hipStream_t s);
hipError_t launch_attn_bwd_dq(const Plan &pl, const AttnBwdArgs &a, hipStream_t s);
hipError_t launch_pool_bwd(const Plan &pl, const PoolBwdArgs &a, hipStream_t s);
hipError_t launch_absmax(const Plan &pl, const AbsMaxArgs &a, hipStream_t s);
hipError_t launch_rowmax(const Plan &pl, const RowMaxArgs &a, hipStream_t s);
hipError_t launch_head_exp(const HeadExpArgs &a, hipStream_t s);
hipError_t launch_selftest_sqrt(uint32_t first, uint32_t count, uint32_t *mismatches, hipStream_t s);

} // namespace lh
