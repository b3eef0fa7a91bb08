// C ABI of the Lighthouse layer (declared in include/lh.h): argument checks,
// the static plan of a call, workspace carving and the launch sequence.
// Nothing here allocates, synchronises or reads device memory.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "lh_internal.h"

namespace lh {

static int ilog2_exact(int p)
{
    for (int b = 0; b < 31; ++b)
        if ((1 << b) == p)
            return b;
    return -1;
}

static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static std::atomic<size_t> g_ds_tile_budget{kDsTileBudgetDefault};
size_t ds_tile_budget() { return g_ds_tile_budget.load(std::memory_order_relaxed); }

// The parts of a plan that depend on N, L, p and k alone: level sizes,
// strata, S and S_pad. Checks the rules of the method on these four.
static lh_status plan_sizes(int64_t N, int L, int p, int k, Plan *pl)
{
    memset(pl, 0, sizeof(*pl));
    if (N < 1 || L < 1 || k < 0)
        return LH_EINVAL;
    if (L > kMaxLevels)
        return LH_EUNSUPPORTED;
    int log2p = 1;
    if (L > 1) {
        if (p < 2)
            return LH_EINVAL;
        log2p = ilog2_exact(p);
        if (log2p < 1 || log2p > 3)
            return LH_EUNSUPPORTED; // p in {2, 4, 8}
        if ((L - 1) * log2p > 27)
            return LH_EUNSUPPORTED;
    }
    if (N > kMaxN)
        return LH_EUNSUPPORTED;
    const int top_shift = (L - 1) * log2p;
    if (L > 1 && (N & ((int64_t(1) << top_shift) - 1)) != 0)
        return LH_EINVAL; // N must be a multiple of p^(L-1)
    pl->N = N; pl->L = L; pl->p = L > 1 ? p : 2; pl->log2p = log2p; pl->k = L > 1 ? k : 0;
    int64_t tot = 0;
    for (int l = 0; l < L; ++l) {
        pl->n[l] = N >> (l * log2p);
        pl->lvl_off[l] = tot;
        tot += pl->n[l];
    }
    pl->lvl_total = tot;
    if (L > 1) {
        if (k > pl->n[L - 1])
            return LH_EINVAL;
        for (int l = 1; l < L; ++l) {
            if (pl->n[l] > kStratum && pl->n[l] % kStratum != 0)
                return LH_EINVAL;
            pl->C[l] = pl->n[l] <= kStratum ? 1 : (int)(pl->n[l] / kStratum);
            pl->strata_total += pl->C[l];
        }
        if ((int64_t)(L - 1) * k > kMaxSelTotal)
            return LH_EUNSUPPORTED;
    }
    pl->S = pl->n[L - 1] + (int64_t)(L - 1) * pl->p * pl->k;
    pl->S_pad = (int64_t)round_up((size_t)pl->S, kSubseqAlign);
    return LH_OK;
}

lh_status make_plan(int64_t N, int H, int d, int L, int p, int k, lh_dtype dt, Plan *pl)
{
    lh_status st = plan_sizes(N, L, p, k, pl);
    if (st != LH_OK)
        return st;
    if (H < 1)
        return LH_EINVAL;
    if (dt != LH_BF16 && dt != LH_F32)
        return LH_EINVAL;
    if (d < 16 || d % 16 != 0)
        return LH_EINVAL;
    if (d != 64 && d != 128)
        return LH_EUNSUPPORTED;
    if (H > kMaxHeads)
        return LH_EUNSUPPORTED;
    pl->H = H; pl->d = d; pl->dt = dt;
    if (pl->S_pad * d > (int64_t(1) << 30))
        return LH_EUNSUPPORTED; // attention kernels address a head's sub-sequence with 32-bit offsets
    const int log2p = pl->log2p;
    const int64_t tot = pl->lvl_total;
    const int64_t pk = (int64_t)pl->p * pl->k;

    // Pooled levels the front pass writes (fp32 rows): the top level (gathered
    // whole) and every middle level whose full write plus the gathered reads
    // moves fewer bytes than averaging the gathered entries' p^l input rows
    // again in the gather.
    for (int l = 0; l < kMaxLevels; ++l)
        pl->mat_off[l] = -1;
    pl->mat_rows = 0;
    const int64_t in_bytes = dt == LH_BF16 ? 2 : 4;
    if (L > 1) {
        for (int l = 1; l < L; ++l) {
            const bool top = l == L - 1;
            const bool cheaper = (pl->n[l] + pk) * 4 < (pk << (l * log2p)) * in_bytes;
            if (top || cheaper) {
                pl->mat_mask |= 1u << l;
                pl->mat_off[l] = pl->mat_rows;
                pl->mat_rows += pl->n[l];
            }
        }
    }
    // Levels finished inside the row tiles; coarser ones keep window sums in
    // IR_FPART (front, entries i of level l) and IR_SPART (scatter-back
    // adjoint, u-space windows m = i + 1, the last tile's tail included).
    {
        const int ltf = tile_levels(d, log2p, front_nc(log2p)), lts = tile_levels(d, log2p, sbwd_nc(log2p));
        pl->LT = L > 1 ? (ltf < L - 1 ? ltf : L - 1) : 0;
        pl->LTs = L > 1 ? (lts < L - 1 ? lts : L - 1) : 0;
    }
    for (int l = 0; l < kMaxLevels; ++l)
        pl->fpart_off[l] = pl->spart_off[l] = pl->spart_n[l] = -1;
    pl->fpart_rows = pl->spart_rows = 0;
    for (int l = pl->LT; l <= L - 2; ++l) {
        pl->fpart_off[l] = pl->fpart_rows;
        pl->fpart_rows += pl->n[l];
    }
    {
        const int64_t T = tile_rows(d, log2p, sbwd_nc(log2p));
        int64_t m = (N + 1 + T - 1) / T * T; // u-space positions the tiles cover
        m >>= pl->LTs * log2p;
        for (int l = pl->LTs; l <= L - 2; ++l) {
            pl->spart_n[l] = m;
            pl->spart_off[l] = pl->spart_rows;
            pl->spart_rows += m;
            m = (m + p - 1) / p;
        }
    }

    // wave maxima of the inputs, for the per-head fp16 staging scales: four
    // per front tile (L = 1: the same tiling, read by k_absmax)
    pl->xmax_tile = tile_rows(d, log2p, front_nc(log2p));
    pl->nxmax = (N + pl->xmax_tile - 1) / pl->xmax_tile * 4;

    // Region sizes. With H <= 2^16, S_pad * d <= 2^30 and N <= 2^27 every
    // product below stays under 2^50; the dS tiles are the one quadratic term
    // and are planned only up to kDsTileBudget bytes (above it the dQ kernel
    // recomputes S and dP instead of reading them).
    const size_t Hs = (size_t)H, Sp = (size_t)pl->S_pad, D = (size_t)d;
    const size_t ds_bytes = 2 * Hs * (size_t)dst_tiles(pl->S_pad) * 1024;
    pl->ds_tiles = ds_bytes <= ds_tile_budget();
    size_t b[IR_COUNT];
    b[LH_R_SCORES] = 4 * Hs * (size_t)tot;
    b[LH_R_SEL] = 4 * Hs * (size_t)(L - 1) * (size_t)pl->k;
    b[LH_R_SLOT] = 4 * Hs * (size_t)tot;
    b[LH_R_ENT] = 4 * Hs * Sp;
    for (int r = LH_R_QHI; r <= LH_R_V_T; ++r)
        b[r] = 2 * Hs * Sp * D;
    // no kernel reads Q^T; with bf16 inputs the lo parts of Q and dO_sub are
    // kept as e4m3 tiles and K's is not used, so their fp16 copies are not made
    b[LH_R_QHI_T] = 0;
    if (pl->dt == LH_BF16)
        b[LH_R_QLO] = b[LH_R_KLO] = 0;
    b[LH_R_OSUB] = 4 * Hs * Sp * D;
    b[LH_R_LSE] = 4 * Hs * Sp;
    b[LH_R_DOSUB] = 4 * Hs * Sp * D;
    b[LH_R_DQSUB] = b[LH_R_DKSUB] = b[LH_R_DVSUB] = 4 * Hs * Sp * D;
    b[IR_POOLED] = 4 * 3 * Hs * (size_t)pl->mat_rows * D;
    b[IR_DOHI] = 2 * Hs * Sp * D;
    b[IR_DOLO] = pl->dt == LH_BF16 ? 0 : 2 * Hs * Sp * D;
    b[IR_DELTA] = 4 * Hs * Sp;
    b[IR_LSE15] = 4 * Hs * Sp;
    b[IR_DST] = pl->ds_tiles ? ds_bytes : 0;
    b[IR_FPART] = 4 * Hs * (size_t)pl->fpart_rows * (3 * D + 1);
    b[IR_SPART] = 4 * Hs * (size_t)pl->spart_rows * D;
    b[IR_QLO8] = b[IR_K8] = b[IR_V8] = b[IR_DOLO8] = Hs * Sp * D;
    b[IR_XMAX] = 4 * 3 * Hs * (size_t)pl->nxmax;
    b[LH_R_EXP] = 4 * 4 * Hs;
    b[IR_DOMAX] = 4 * Hs * (Sp / kExpTile);
    // What lh_forward writes comes first (the context the backward reads and
    // the forward's own scratch), so a forward-only caller can pass a
    // workspace that ends there; the regions only lh_backward writes follow.
    static const int kFwdOrder[] = {LH_R_SCORES, LH_R_SEL, LH_R_SLOT, LH_R_ENT, LH_R_QHI, LH_R_QLO, LH_R_KHI,
                                    LH_R_KLO, LH_R_V, LH_R_QHI_T, LH_R_KHI_T, LH_R_V_T, LH_R_OSUB, LH_R_LSE,
                                    LH_R_EXP, IR_QLO8, IR_K8, IR_V8, IR_POOLED, IR_FPART, IR_XMAX};
    static const int kBwdOrder[] = {LH_R_DOSUB, LH_R_DQSUB, LH_R_DKSUB, LH_R_DVSUB, IR_DOHI, IR_DOLO,
                                    IR_DELTA, IR_LSE15, IR_SPART, IR_DOLO8, IR_DOMAX, IR_DST};
    static_assert(sizeof(kFwdOrder) / sizeof(int) + sizeof(kBwdOrder) / sizeof(int) == IR_COUNT,
                  "every region placed once");
    size_t off = 0;
    for (int r : kFwdOrder) {
        pl->off[r] = off;
        pl->bytes[r] = b[r];
        off = round_up(off + b[r], 256);
    }
    pl->fwd_total = off;
    for (int r : kBwdOrder) {
        pl->off[r] = off;
        pl->bytes[r] = b[r];
        off = round_up(off + b[r], 256);
    }
    pl->total = off;
    if (pl->total > kMaxWorkspace)
        return LH_EUNSUPPORTED;
    return LH_OK;
}

template <typename Tp> static Tp *at(void *ws, const Plan &pl, int r)
{
    return reinterpret_cast<Tp *>(static_cast<char *>(ws) + pl.off[r]);
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

static lh_status check_ws(void *ws, size_t ws_bytes, size_t need)
{
    if (!ws || ((uintptr_t)ws & 255u) != 0 || ws_bytes < need)
        return LH_EWORKSPACE;
    return LH_OK;
}

static void record(void *const *events, int i, hipStream_t s)
{
    if (events)
        (void)hipEventRecord(reinterpret_cast<hipEvent_t>(events[i]), s);
}

static const char *kFwdStages[] = {"front", "topk", "index", "gather", "attn_fwd", "scatter"};
static const char *kBwdStages[] = {"scatter_bwd", "bwd_prep", "attn_bwd_dkdv", "attn_bwd_dq", "pool_bwd"};

static lh_status forward_impl(const void *q, const void *k, const void *v, int64_t N, int H, int d, int L, int p,
                              int k_sel, lh_dtype dt, void *out, void *ws, size_t ws_bytes, hipStream_t s,
                              void *const *events, lh_scorer scorer = LH_SCORE_SUM, bool for_backward = true)
{
    Plan pl;
    lh_status st = make_plan(N, H, d, L, p, k_sel, dt, &pl);
    if (st != LH_OK)
        return st;
    if ((int)scorer < LH_SCORE_SUM || (int)scorer > LH_SCORE_KEY)
        return LH_EINVAL;
    if (!q || !k || !v || !out || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return LH_EINVAL;
    if ((st = check_ws(ws, ws_bytes, pl.fwd_total)) != LH_OK)
        return st;

    float *scores = at<float>(ws, pl, LH_R_SCORES);
    int32_t *sel = at<int32_t>(ws, pl, LH_R_SEL);
    int32_t *slot = at<int32_t>(ws, pl, LH_R_SLOT);
    int32_t *ent = at<int32_t>(ws, pl, LH_R_ENT);
    float *pooled = at<float>(ws, pl, IR_POOLED);
    const int64_t tensor_stride = (int64_t)H * pl.mat_rows * d;

    record(events, 0, s);
    if (L > 1) {
        FrontArgs fa;
        memset(&fa, 0, sizeof(fa));
        fa.q = q; fa.k = k; fa.v = v; fa.scores = scores; fa.pooled = pooled;
        fa.N = N; fa.lvl_total = pl.lvl_total; fa.mat_rows = pl.mat_rows; fa.tensor_stride = tensor_stride;
        for (int l = 0; l < kMaxLevels; ++l) {
            fa.lvl_off[l] = l < L ? pl.lvl_off[l] : 0;
            fa.mat_off[l] = pl.mat_off[l];
        }
        fa.part = at<float>(ws, pl, IR_FPART);
        fa.part_rows = pl.fpart_rows;
        for (int l = 0; l < kMaxLevels; ++l)
            fa.part_off[l] = pl.fpart_off[l];
        fa.H = H; fa.L = L; fa.log2p = pl.log2p; fa.LT = pl.LT;
        fa.scorer = (int)scorer;
        fa.xmax = at<float>(ws, pl, IR_XMAX);
        fa.nxmax = pl.nxmax;
        if (launch_front(pl, fa, s) != hipSuccess)
            return LH_EHIP;
    } else { // no front pass: the inputs' maxima on their own
        AbsMaxArgs ma;
        ma.x[0] = q; ma.x[1] = k; ma.x[2] = v;
        ma.xmax = at<float>(ws, pl, IR_XMAX);
        ma.N = N; ma.nxmax = pl.nxmax; ma.tile = pl.xmax_tile; ma.H = H;
        if (launch_absmax(pl, ma, s) != hipSuccess)
            return LH_EHIP;
    }
    {
        HeadExpArgs ea;
        ea.m = at<float>(ws, pl, IR_XMAX); ea.count = pl.nxmax; ea.nt = 3; ea.H = H; ea.first = 0;
        ea.ex = at<int32_t>(ws, pl, LH_R_EXP);
        if (launch_head_exp(ea, s) != hipSuccess)
            return LH_EHIP;
    }
    record(events, 1, s);
    if (L > 1) {
        TopkArgs ta;
        memset(&ta, 0, sizeof(ta));
        ta.scores = scores; ta.sel = sel; ta.slot = slot; ta.lvl_total = pl.lvl_total;
        int before = 0;
        for (int l = 0; l < kMaxLevels; ++l) {
            ta.lvl_off[l] = l < L ? pl.lvl_off[l] : 0;
            ta.n[l] = l < L ? pl.n[l] : 0;
            ta.C[l] = pl.C[l];
            ta.strata_before[l] = before;
            if (l >= 1 && l < L)
                before += pl.C[l];
        }
        ta.L = L; ta.log2p = pl.log2p; ta.k = pl.k;
        if (launch_topk(pl, ta, s) != hipSuccess)
            return LH_EHIP;
    }
    record(events, 2, s);
    {
        IndexArgs ia;
        memset(&ia, 0, sizeof(ia));
        ia.sel = sel; ia.slot = slot; ia.ent = ent;
        ia.lvl_total = pl.lvl_total; ia.S = pl.S; ia.S_pad = pl.S_pad;
        for (int l = 0; l < kMaxLevels; ++l) {
            ia.lvl_off[l] = l < L ? pl.lvl_off[l] : 0;
            ia.n[l] = l < L ? pl.n[l] : 0;
        }
        ia.L = L; ia.log2p = pl.log2p; ia.k = pl.k;
        if (launch_index(pl, ia, s) != hipSuccess)
            return LH_EHIP;
    }
    record(events, 3, s);
    {
        GatherArgs ga;
        memset(&ga, 0, sizeof(ga));
        ga.q = q; ga.k = k; ga.v = v; ga.pooled = pooled; ga.ent = ent;
        ga.hi[0] = at<uint16_t>(ws, pl, LH_R_QHI);
        ga.hi[1] = at<uint16_t>(ws, pl, LH_R_KHI);
        ga.hi[2] = at<uint16_t>(ws, pl, LH_R_V);
        if (dt == LH_F32) {
            ga.lo[0] = at<uint16_t>(ws, pl, LH_R_QLO);
            ga.lo[1] = at<uint16_t>(ws, pl, LH_R_KLO);
        }
        ga.hi_t[0] = at<uint16_t>(ws, pl, LH_R_KHI_T);
        ga.hi_t[1] = at<uint16_t>(ws, pl, LH_R_V_T);
        if (dt == LH_BF16) { // e4m3 copies for the fp8 products: Q lo and K hi (logits), V (dP)
            ga.t8[0] = at<uint8_t>(ws, pl, IR_QLO8);
            ga.t8[1] = at<uint8_t>(ws, pl, IR_K8);
            ga.t8[2] = at<uint8_t>(ws, pl, IR_V8);
        }
        ga.ex = at<int32_t>(ws, pl, LH_R_EXP);
        ga.N = N; ga.S = pl.S; ga.S_pad = pl.S_pad; ga.mat_rows = pl.mat_rows; ga.tensor_stride = tensor_stride;
        for (int l = 0; l < kMaxLevels; ++l) {
            ga.mat_off[l] = pl.mat_off[l];
            ga.n[l] = l < L ? pl.n[l] : 0;
        }
        ga.H = H; ga.L = L; ga.log2p = pl.log2p;
        if (launch_gather(pl, ga, s) != hipSuccess)
            return LH_EHIP;
    }
    record(events, 4, s);
    {
        AttnFwdArgs aa;
        aa.qhi = at<uint16_t>(ws, pl, LH_R_QHI);
        aa.qlo = dt == LH_F32 ? at<uint16_t>(ws, pl, LH_R_QLO) : nullptr; // fp32 inputs only
        aa.khi = at<uint16_t>(ws, pl, LH_R_KHI);
        aa.klo = dt == LH_F32 ? at<uint16_t>(ws, pl, LH_R_KLO) : nullptr;
        aa.vt = at<uint16_t>(ws, pl, LH_R_V_T);
        aa.qlo8 = at<uint8_t>(ws, pl, IR_QLO8);
        aa.k8 = at<uint8_t>(ws, pl, IR_K8);
        aa.o = at<float>(ws, pl, LH_R_OSUB);
        aa.lse = at<float>(ws, pl, LH_R_LSE);
        aa.ex = at<int32_t>(ws, pl, LH_R_EXP);
        aa.S = pl.S; aa.S_pad = pl.S_pad; aa.H = H;
        aa.for_bwd = for_backward ? 1 : 0;
        aa.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
        if (launch_attn_fwd(pl, aa, s) != hipSuccess)
            return LH_EHIP;
    }
    record(events, 5, s);
    {
        ScatterArgs sa;
        memset(&sa, 0, sizeof(sa));
        sa.osub = at<float>(ws, pl, LH_R_OSUB); sa.slot = slot; sa.out = out;
        sa.N = N; sa.lvl_total = pl.lvl_total; sa.S_pad = pl.S_pad;
        for (int l = 0; l < kMaxLevels; ++l)
            sa.lvl_off[l] = l < L ? pl.lvl_off[l] : 0;
        sa.H = H; sa.L = L; sa.log2p = pl.log2p;
        if (launch_scatter(pl, sa, s) != hipSuccess)
            return LH_EHIP;
    }
    record(events, 6, s);
    return LH_OK;
}

static lh_status backward_impl(const void *dout, int64_t N, int H, int d, int L, int p, int k_sel, lh_dtype dt,
                               void *dq, void *dk, void *dv, void *ws, size_t ws_bytes, hipStream_t s,
                               void *const *events)
{
    Plan pl;
    lh_status st = make_plan(N, H, d, L, p, k_sel, dt, &pl);
    if (st != LH_OK)
        return st;
    if (!dout || !dq || !dk || !dv || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
        return LH_EINVAL;
    if ((st = check_ws(ws, ws_bytes, pl.total)) != LH_OK)
        return st;
    int32_t *slot = at<int32_t>(ws, pl, LH_R_SLOT);
    float *dosub = at<float>(ws, pl, LH_R_DOSUB);

    record(events, 0, s);
    {
        ScatterBwdArgs a;
        memset(&a, 0, sizeof(a));
        a.dout = dout; a.slot = slot; a.dosub = dosub;
        a.N = N; a.lvl_total = pl.lvl_total; a.S_pad = pl.S_pad;
        for (int l = 0; l < kMaxLevels; ++l)
            a.lvl_off[l] = l < L ? pl.lvl_off[l] : 0;
        a.part = at<float>(ws, pl, IR_SPART);
        a.part_rows = pl.spart_rows;
        for (int l = 0; l < kMaxLevels; ++l) {
            a.part_off[l] = pl.spart_off[l];
            a.part_n[l] = pl.spart_n[l];
        }
        a.H = H; a.L = L; a.log2p = pl.log2p; a.LT = pl.LTs;
        if (launch_scatter_bwd(pl, a, s) != hipSuccess)
            return LH_EHIP;
    }
    record(events, 1, s);
    {
        // the per-head staging scale of dO_sub, from its tile maxima
        RowMaxArgs ra;
        ra.src = dosub; ra.dst = at<float>(ws, pl, IR_DOMAX); ra.S = pl.S; ra.S_pad = pl.S_pad;
        if (launch_rowmax(pl, ra, s) != hipSuccess)
            return LH_EHIP;
        HeadExpArgs ea;
        ea.m = ra.dst; ea.count = pl.S_pad / kExpTile; ea.nt = 1; ea.H = H; ea.first = 3;
        ea.ex = at<int32_t>(ws, pl, LH_R_EXP);
        if (launch_head_exp(ea, s) != hipSuccess)
            return LH_EHIP;
    }
    {
        BwdPrepArgs a;
        a.dosub = dosub; a.osub = at<float>(ws, pl, LH_R_OSUB);
        a.dohi = at<uint16_t>(ws, pl, IR_DOHI);
        a.dolo = pl.dt == LH_F32 ? at<uint16_t>(ws, pl, IR_DOLO) : nullptr;
        a.delta = at<float>(ws, pl, IR_DELTA);
        a.lse = at<float>(ws, pl, LH_R_LSE);
        a.lse15 = at<float>(ws, pl, IR_LSE15);
        a.dolo8 = pl.dt == LH_BF16 ? at<uint8_t>(ws, pl, IR_DOLO8) : nullptr; // e4m3 copy of the lo part
        a.ex = at<int32_t>(ws, pl, LH_R_EXP);
        a.S = pl.S; a.S_pad = pl.S_pad; a.H = H;
        if (launch_bwd_prep(pl, a, s) != hipSuccess)
            return LH_EHIP;
    }
    record(events, 2, s);
    AttnBwdArgs ab;
    ab.qhi = at<uint16_t>(ws, pl, LH_R_QHI);
    ab.qlo = pl.dt == LH_F32 ? at<uint16_t>(ws, pl, LH_R_QLO) : nullptr; // fp32 inputs only
    ab.khi = at<uint16_t>(ws, pl, LH_R_KHI);
    ab.klo = pl.dt == LH_F32 ? at<uint16_t>(ws, pl, LH_R_KLO) : nullptr;
    ab.v = at<uint16_t>(ws, pl, LH_R_V);
    ab.qlo8 = at<uint8_t>(ws, pl, IR_QLO8);
    ab.k8 = at<uint8_t>(ws, pl, IR_K8);
    ab.v8 = at<uint8_t>(ws, pl, IR_V8);
    ab.dolo8 = at<uint8_t>(ws, pl, IR_DOLO8);
    ab.khi_t = at<uint16_t>(ws, pl, LH_R_KHI_T);
    ab.dohi = at<uint16_t>(ws, pl, IR_DOHI);
    ab.dolo = pl.dt == LH_F32 ? at<uint16_t>(ws, pl, IR_DOLO) : nullptr;
    ab.lse = at<float>(ws, pl, IR_LSE15);
    ab.delta = at<float>(ws, pl, IR_DELTA);
    ab.dq = at<float>(ws, pl, LH_R_DQSUB);
    ab.dk = at<float>(ws, pl, LH_R_DKSUB);
    ab.dv = at<float>(ws, pl, LH_R_DVSUB);
    ab.dst = pl.ds_tiles ? at<uint16_t>(ws, pl, IR_DST) : nullptr; // none: the dQ kernel recomputes S and dP
    ab.dst_head = dst_tiles(pl.S_pad) * 1024;
    ab.ex = at<int32_t>(ws, pl, LH_R_EXP);
    ab.S = pl.S; ab.S_pad = pl.S_pad; ab.H = H;
    ab.scale = (float)(1.0 / sqrt((double)d));
    ab.scale_log2 = (float)(1.4426950408889634 / sqrt((double)d));
    if (launch_attn_bwd_dkdv(pl, ab, s) != hipSuccess)
        return LH_EHIP;
    record(events, 3, s);
    if (launch_attn_bwd_dq(pl, ab, s) != hipSuccess)
        return LH_EHIP;
    record(events, 4, s);
    {
        PoolBwdArgs a;
        memset(&a, 0, sizeof(a));
        a.dsub[0] = ab.dq; a.dsub[1] = ab.dk; a.dsub[2] = ab.dv;
        a.slot = slot;
        a.dx[0] = dq; a.dx[1] = dk; a.dx[2] = dv;
        a.N = N; a.lvl_total = pl.lvl_total; a.S_pad = pl.S_pad;
        for (int l = 0; l < kMaxLevels; ++l)
            a.lvl_off[l] = l < L ? pl.lvl_off[l] : 0;
        a.H = H; a.L = L; a.log2p = pl.log2p;
        if (launch_pool_bwd(pl, a, s) != hipSuccess)
            return LH_EHIP;
    }
    record(events, 5, s);
    return LH_OK;
}

// ---------------------------------------------------------------- static scratch
// Workspace of lh_forward_static: a file-scope device array. Every GPU the
// library runs on holds its own copy, at its own address, until the process
// ends. In host code `scratch` names a host-side stand-in, never the device
// memory: its device address is looked up once per device with
// hipGetSymbolAddress and only that address reaches the kernels.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_dev[kMaxDevices]; // device address of `scratch` on each device, once looked up

// The current device's copy of `scratch` (looked up on the first call on
// that device; the device must be current, as for any launch).
static lh_status scratch_address(void **out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return LH_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return LH_EHIP;
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return LH_OK;
}

} // namespace lh

using namespace lh;

extern "C" {

const char *lh_strerror(lh_status s)
{
    switch (s) {
    case LH_OK: return "ok";
    case LH_EINVAL: return "invalid argument";
    case LH_EWORKSPACE: return "workspace missing, misaligned or too small";
    case LH_EUNSUPPORTED: return "shape not supported by this build";
    case LH_EHIP: return "HIP launch error";
    }
    return "unknown status";
}

lh_status lh_check_shape(int64_t N, int H, int d, int L, int p, int k, lh_dtype dt)
{
    Plan pl;
    return make_plan(N, H, d, L, p, k, dt, &pl);
}

int64_t lh_subseq_len(int64_t N, int L, int p, int k)
{
    Plan pl;
    if (plan_sizes(N, L, p, k, &pl) != LH_OK)
        return -1;
    return pl.S;
}

int64_t lh_padded_subseq_len(int64_t N, int L, int p, int k)
{
    Plan pl;
    if (plan_sizes(N, L, p, k, &pl) != LH_OK)
        return -1;
    return pl.S_pad;
}

size_t lh_workspace_bytes(int64_t N, int H, int d, int L, int p, int k, lh_dtype dt)
{
    Plan pl;
    if (make_plan(N, H, d, L, p, k, dt, &pl) != LH_OK)
        return 0;
    return pl.total;
}

size_t lh_forward_workspace_bytes(int64_t N, int H, int d, int L, int p, int k, lh_dtype dt)
{
    Plan pl;
    if (make_plan(N, H, d, L, p, k, dt, &pl) != LH_OK)
        return 0;
    return pl.fwd_total;
}

lh_status lh_selection(const void *ws, int64_t N, int H, int d, int L, int p, int k_sel, int level,
                       const int32_t **sel_dev)
{
    if (!sel_dev)
        return LH_EINVAL;
    *sel_dev = nullptr;
    Plan pl;
    // the selection's place depends on N, H, L, p and k only (the first two
    // regions): it is the same for either input type
    lh_status st = make_plan(N, H, d, L, p, k_sel, LH_BF16, &pl);
    if (st != LH_OK)
        return st;
    if (!ws || ((uintptr_t)ws & 255u) != 0 || L < 2 || level < 1 || level > L - 1)
        return LH_EINVAL;
    *sel_dev = reinterpret_cast<const int32_t *>(static_cast<const char *>(ws) + pl.off[LH_R_SEL]) +
               (int64_t)(level - 1) * H * pl.k;
    return LH_OK;
}

lh_status lh_region_info(int64_t N, int H, int d, int L, int p, int k, lh_dtype dt, lh_region region,
                         size_t *offset, size_t *bytes)
{
    Plan pl;
    lh_status st = make_plan(N, H, d, L, p, k, dt, &pl);
    if (st != LH_OK)
        return st;
    if ((int)region < 0 || (int)region >= LH_R_COUNT || !offset || !bytes)
        return LH_EINVAL;
    *offset = pl.off[region];
    *bytes = pl.bytes[region];
    return LH_OK;
}

int lh_stage_count(int backward) { return backward ? 5 : 6; }

const char *lh_stage_name(int backward, int stage)
{
    if (stage < 0 || stage >= lh_stage_count(backward))
        return "";
    return backward ? kBwdStages[stage] : kFwdStages[stage];
}

lh_status lh_forward(const void *q, const void *k, const void *v, int64_t N, int H, int d, int L, int p, int k_sel,
                     lh_dtype dt, void *out, void *ws, size_t ws_bytes, void *stream)
{
    return forward_impl(q, k, v, N, H, d, L, p, k_sel, dt, out, ws, ws_bytes, (hipStream_t)stream, nullptr);
}

lh_status lh_forward_scored(const void *q, const void *k, const void *v, int64_t N, int H, int d, int L, int p,
                            int k_sel, lh_dtype dt, lh_scorer scorer, void *out, void *ws, size_t ws_bytes,
                            void *stream)
{
    return forward_impl(q, k, v, N, H, d, L, p, k_sel, dt, out, ws, ws_bytes, (hipStream_t)stream, nullptr, scorer);
}

lh_status lh_forward_nograd(const void *q, const void *k, const void *v, int64_t N, int H, int d, int L, int p,
                            int k_sel, lh_dtype dt, void *out, void *ws, size_t ws_bytes, void *stream)
{
    return forward_impl(q, k, v, N, H, d, L, p, k_sel, dt, out, ws, ws_bytes, (hipStream_t)stream, nullptr,
                        LH_SCORE_SUM, false);
}

lh_status lh_forward_static(const void *q, const void *k, const void *v, int64_t N, int H, int d, int L, int p,
                            int k_sel, lh_dtype dt, void *out, void *stream)
{
    // shape, pointers and the scratch size first: nothing touches the device
    // before the call is known to fit
    Plan pl;
    lh_status st = make_plan(N, H, d, L, p, k_sel, dt, &pl);
    if (st != LH_OK)
        return st;
    if (!q || !k || !v || !out || !aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return LH_EINVAL;
    if (pl.fwd_total > kStaticScratchBytes)
        return LH_EWORKSPACE;
    void *ws = nullptr;
    if ((st = scratch_address(&ws)) != LH_OK)
        return st;
    return forward_impl(q, k, v, N, H, d, L, p, k_sel, dt, out, ws, kStaticScratchBytes, (hipStream_t)stream,
                        nullptr);
}

size_t lh_static_scratch_bytes(void) { return kStaticScratchBytes; }

void lh_set_ds_tile_budget(size_t bytes) { g_ds_tile_budget.store(bytes, std::memory_order_relaxed); }

size_t lh_ds_tile_budget(void) { return ds_tile_budget(); }

lh_status lh_forward_timed(const void *q, const void *k, const void *v, int64_t N, int H, int d, int L, int p,
                           int k_sel, lh_dtype dt, void *out, void *ws, size_t ws_bytes, void *stream,
                           void *const *events)
{
    if (!events)
        return LH_EINVAL;
    return forward_impl(q, k, v, N, H, d, L, p, k_sel, dt, out, ws, ws_bytes, (hipStream_t)stream, events);
}

lh_status lh_forward_nograd_timed(const void *q, const void *k, const void *v, int64_t N, int H, int d, int L,
                                  int p, int k_sel, lh_dtype dt, void *out, void *ws, size_t ws_bytes, void *stream,
                                  void *const *events)
{
    if (!events)
        return LH_EINVAL;
    return forward_impl(q, k, v, N, H, d, L, p, k_sel, dt, out, ws, ws_bytes, (hipStream_t)stream, events,
                        LH_SCORE_SUM, false);
}

lh_status lh_backward(const void *dout, int64_t N, int H, int d, int L, int p, int k_sel, lh_dtype dt, void *dq,
                      void *dk, void *dv, void *ws, size_t ws_bytes, void *stream)
{
    return backward_impl(dout, N, H, d, L, p, k_sel, dt, dq, dk, dv, ws, ws_bytes, (hipStream_t)stream, nullptr);
}

lh_status lh_backward_timed(const void *dout, int64_t N, int H, int d, int L, int p, int k_sel, lh_dtype dt,
                            void *dq, void *dk, void *dv, void *ws, size_t ws_bytes, void *stream,
                            void *const *events)
{
    if (!events)
        return LH_EINVAL;
    return backward_impl(dout, N, H, d, L, p, k_sel, dt, dq, dk, dv, ws, ws_bytes, (hipStream_t)stream, events);
}

lh_status lh_selftest_sqrt(uint32_t first, uint32_t count, uint32_t *mismatches, void *stream)
{
    if (!mismatches || ((uintptr_t)mismatches & 3u))
        return LH_EINVAL;
    if (launch_selftest_sqrt(first, count, mismatches, (hipStream_t)stream) != hipSuccess)
        return LH_EHIP;
    return LH_OK;
}

} // extern "C"
