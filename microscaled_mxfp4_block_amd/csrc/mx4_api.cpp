// mx4_api.cpp -- the C ABI of include/mx4.h: argument checks, plans, launches.
//
// Every entry point validates its arguments on the host before it touches
// HIP, so an invalid call returns an MX_E* code with nothing enqueued.  The
// library owns no memory and keeps no mutable state.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "../../include/mx4.h"
#include "mx4_internal.h"

using mx4::GemmParams;
using mx4::OperandGeom;
using mx4::Plan;
using mx4::kAmBf16;
using mx4::kAmDirect;
using mx4::kAmLds;
using mx4::kAmPrequant;
using mx4::kAmShared;
using mx4::kAmStream;
using mx4::kAmTile;
static_assert(kAmLds == MX_AMODE_LDS && kAmPrequant == MX_AMODE_PREQUANT && kAmDirect == MX_AMODE_DIRECT &&
                  kAmBf16 == MX_AMODE_BF16 && kAmStream == MX_AMODE_STREAM && kAmShared == MX_AMODE_SHARED &&
                  kAmTile == MX_AMODE_TILE,
              "activation modes of the C ABI and the kernels differ");

namespace {

constexpr int kMaxDim = 1 << 24;

bool aligned(const void* p, uintptr_t a) { return p != nullptr && ((uintptr_t)p % a) == 0; }

int check_operand_shape(int rows, int K) {
    if (rows <= 0 || K <= 0 || rows > kMaxDim || K > kMaxDim || K % mx4::kGroup != 0) return MX_EINVAL;
    const OperandGeom g = mx4::operand_geom(rows, K);
    // the kernels address operands with 32-bit buffer offsets
    if (g.total_bytes >= (1ULL << 31) || (unsigned long long)rows * K * 2 >= (1ULL << 31)) return MX_EINVAL;
    return MX_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MX_OK : MX_EHIP; }

// Plans measured for the five decode-style shapes; other shapes use the model
// in model_plan().
struct TableEntry {
    int M, N, K;
    Plan plan;   // mb, nb, wn, wk, splits, amode, finish
};
const TableEntry kTable[] = {
    {4, 2880, 512, {1, 1, 1, 4, 1, 2, 0}},
    {32, 4096, 512, {1, 1, 1, 4, 1, 2, 0}},
    {32, 2880, 512, {1, 1, 1, 4, 1, 2, 0}},
    {16, 2112, 7168, {1, 1, 3, 4, 7, 5, 0}},
    {64, 7168, 2048, {1, 2, 1, 8, 1, 2, 0}},
    {256, 3072, 1536, {1, 1, 3, 4, 1, 5, 0}},
};

int pow2_floor(int x) {
    int p = 1;
    while (p * 2 <= x) p *= 2;
    return p;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Layout {
    size_t counter_bytes;   // at offset 0 of every non-empty workspace
    size_t aop_offset, aop_bytes;
    size_t partial_offset, partial_bytes;
    size_t total;
    int splits, steps_per_split;
    int mtiles, ntiles;
};

int plan_layout(const Plan& plan, int M, int N, int K, Layout* out) {
    if (!mx4::gemm_plan_supported(plan)) return MX_EPLAN;
    const OperandGeom ga = mx4::operand_geom(M, K);
    const OperandGeom gb = mx4::operand_geom(N, K);
    if (plan.splits > gb.KS) return MX_EPLAN;
    Layout l;
    l.steps_per_split = (gb.KS + plan.splits - 1) / plan.splits;
    // the shared and tile modes' splits start on a scale word (4 steps)
    if (plan.amode == kAmShared || plan.amode == kAmTile) l.steps_per_split = (l.steps_per_split + 3) / 4 * 4;
    l.splits = (gb.KS + l.steps_per_split - 1) / l.steps_per_split;  // every split non-empty
    // The stream mode loops over its K steps; the shared mode's MFMA waves
    // each hold a whole split (its kernels' own budgets, checked when the
    // kernel is resolved); the other modes hold all of a wave's steps in
    // registers at once.
    const bool stream = plan.amode == kAmStream || plan.amode == kAmShared || plan.amode == kAmTile;
    if (plan.amode == kAmShared && !mx4::find_shared_kernel(plan, l.steps_per_split)) return MX_EPLAN;
    // the shared and tile modes' partials go to reduce_kernel
    if ((plan.amode == kAmShared || plan.amode == kAmTile) && plan.finish != 0 && l.splits > 1) return MX_EPLAN;
    if (!stream && (l.steps_per_split + plan.wk - 1) / plan.wk > mx4::kStepsPerWaveMax) return MX_EPLAN;
    // Register budget (no plan may run a kernel that spills).  kAmDirect and
    // kAmBf16 hold the raw bf16 of every fragment of the wave (16 VGPRs per K
    // step and m block) while the weight loads are in flight: at most 128.
    // A 16-wave workgroup leaves each wave 128 VGPRs in all: half that again.
    if (!stream) {
        const int kr = mx4::gemm_kr_for((l.steps_per_split + plan.wk - 1) / plan.wk);
        const bool rega = plan.amode == kAmDirect || plan.amode == kAmBf16;
        const bool waves16 = plan.wn * plan.wk == 16;
        if (rega && plan.mb * kr > (waves16 ? 4 : 8)) return MX_EPLAN;
        // kAmLds also keeps a row of activation loads in flight per lane
        if (!rega && waves16 && plan.mb * plan.nb * kr > (plan.amode == kAmLds ? 4 : 8)) return MX_EPLAN;
    }
    if (mx4::gemm_lds_bytes(plan, l.steps_per_split) > mx4::kLdsBudget) return MX_EPLAN;
    l.mtiles = (ga.RB + plan.mb - 1) / plan.mb;
    // the tile mode's nb counts the workgroup's N blocks, the others' a wave's
    const int nblk = plan.amode == kAmTile ? plan.nb : plan.nb * plan.wn;
    l.ntiles = (gb.RB + nblk - 1) / nblk;
    // grid (N tiles, M tiles, splits): y and z are 16-bit
    if (l.mtiles > 65535 || l.splits > 65535 || l.ntiles > (1 << 30)) return MX_EINVAL;
    if (plan.finish != 0 && plan.finish != 1) return MX_EPLAN;
    if (plan.finish == 1 && l.splits > 1 && (long long)l.mtiles * l.ntiles > mx4::kMaxCounters) return MX_EPLAN;
    l.aop_bytes = mx4::amode_prequantises(plan.amode) ? round_up(ga.total_bytes, 256) : 0;
    l.partial_bytes = l.splits > 1 ? round_up((size_t)l.splits * M * gb.RB * mx4::kRowBlock * sizeof(float), 256) : 0;
    if (l.partial_bytes >= (1ull << 31)) return MX_EPLAN;   // 32-bit buffer offsets
    l.counter_bytes = (l.aop_bytes + l.partial_bytes) > 0 ? mx4::kCounterBytes : 0;
    l.aop_offset = l.counter_bytes;
    l.partial_offset = l.aop_offset + l.aop_bytes;
    l.total = l.counter_bytes + l.aop_bytes + l.partial_bytes;
    *out = l;
    return MX_OK;
}

// Model for shapes without a table entry, fitted to the plan-regret sweep
// over the pages' shape grid (19 (N, K) weight shapes x M = 1 .. 256, up to
// 69 candidate plans each) and to a sweep of M = 256 .. 2048 over six of its
// weight shapes with the tile mode's plans among the candidates:
//   - deep K (more than 32 steps) with one 32-row block of M, or up to four
//     at N <= 2112: the quantiser-wave mode with 4 quantiser waves and K
//     split into pieces of at most 16 steps (7 splits at K = 7168), three
//     MFMA waves when the N blocks divide by 3 and the grid stays within one
//     workgroup per CU (such a workgroup holds about 81 KB of LDS), else
//     four; except at N >= 7168, where one M block of at most 8 rows takes
//     splits of 8 steps (three workgroups fit a CU), 9 .. 32 rows the
//     register mode with 2 splits, and two M blocks the pre-quantisation
//     kernel with 2 splits; the rest of deep K goes on below;
//   - the activation is quantised once per workgroup by quantiser waves for
//     three or four MFMA waves when M has at least eight 32-row blocks (or
//     four, with K <= 512 or N >= 7168; or two, with both) and K is at most
//     24 steps (eight quantiser waves, four for K <= 512 from 12 to 31 M
//     blocks);
//   - else it is quantised in a first kernel when M has four or more 32-row
//     blocks and K more than 8 steps, unless M is exactly four blocks with
//     N < 7168 and K <= 2048: every wave of every N tile would otherwise
//     quantise it again, which costs more vector-ALU time than the launch;
//     there, two M blocks per wave and two waves along N (one for deep K,
//     and from 12 M blocks below N = 7168);
//   - otherwise each wave quantises its own fragments: two N blocks per wave
//     from four M blocks on, from two at N >= 7168, and for deep K;
//   - 8 waves along K (4 for K <= 512), and K split over workgroups only as
//     far as the register budget needs, except that deep K with the register
//     mode takes at least 2 splits: the N tiles alone leave most CUs idle.
//   - the tile mode (activation quantised once, K-looped tiles of both
//     operands), from the sweeps over the grid and M = 256 .. 2048 with its
//     tiles among the candidates: from M = 64; with K > 2048 past M = 64
//     at N >= 1536 (the 64 x 64 tile with its deeper ring on a small grid:
//     11-48 % faster than the other modes at M = 96 .. 192, K = 2560 ..
//     5120, N = 1536 .. 4096, but 25 % slower at M = 64), or at
//     2MNK >= 5 GFLOP with N >= 7168; at K = 2048 from M = 256, or from
//     M = 128 at N >= 7168; with a shorter K from
//     M = 256 at 2MNK >= 3 GFLOP + 0.5 MFLOP per unit of K.  The tile: the
//     largest of 256 x 256, 256 x 128, 128 x 128 and 64 x 64 whose grid has
//     at least 128 workgroups (384 for K <= 512, where a workgroup's few K
//     steps leave it latency-bound), the 128 x 128 tile with eight waves
//     (four for K <= 512).
// A deep-K or tile plan that the layout refuses for a shape (a split count
// past the partials' 32-bit range, say) falls through to the rules after it.
// The shared mode's MFMA waves (N tiles of 3 or 4 N blocks) for a grid of
// RBm x RBn / wn workgroups that runs in one round on the 256 CUs, one a CU:
// three waves when they qualify with no ragged N tile, else four, else four
// with a ragged last N tile, else 0.  Measured at 160 .. 448 rows, K = 1024
// and 1536: a grid that needs a second round costs 1.6x (7.6-7.7 against
// 4.8 us at 288 x 3072 x 1536); from 5 M blocks such a plan was 35-38 %
// faster than the register modes the model took before, and the ragged
// one 11-15 % faster than a second round (288 and 320 x 2880, 384 and
// 448 x 2112).
int shared_round_wn(int RBm, int RBn) {
    for (int wn = 3; wn <= 4; ++wn)
        if (RBn % wn == 0 && (long long)RBm * (RBn / wn) <= 256) return wn;
    return (long long)RBm * ((RBn + 3) / 4) <= 256 ? 4 : 0;
}

Plan model_plan(int M, int N, int K) {
    const OperandGeom ga = mx4::operand_geom(M, K);
    const OperandGeom gb = mx4::operand_geom(N, K);
    const int RBm = ga.RB, RBn = gb.RB, KS = gb.KS;
    const bool deep = KS > 32;   // K past 2048
    Layout l;
    const double flops = 2.0 * M * N * K;
    const bool long_k = K > 2048, mid_k = K == 2048;
    const bool tile =
        M >= 64 && (long_k  ? M >= 256 || (M > 64 && N >= 1536) || (flops >= 5e9 && N >= 7168)
                    : mid_k ? M >= 256 || (M >= 128 && N >= 7168)
                            : M >= 256 && flops >= 3e9 + 0.5e6 * K);
    if (tile) {
        const bool short_k = K <= 512;
        const long long min_wgs = short_k ? 384 : 128;
        // {mb, nb, wn, wk}: wk waves along M, wn along N
        const Plan tiles[4] = {{8, 8, 4, 2, 1, kAmTile, 0},
                               {8, 4, 2, 2, 1, kAmTile, 0},
                               {4, 4, short_k ? 2 : 4, 2, 1, kAmTile, 0},
                               {2, 2, 2, 2, 1, kAmTile, 0}};
        for (int i = 0; i < 4; ++i) {
            const Plan& q = tiles[i];
            const long long wgs = (long long)((RBm + q.mb - 1) / q.mb) * ((RBn + q.nb - 1) / q.nb);
            if ((wgs >= min_wgs || i == 3) && plan_layout(q, M, N, K, &l) == MX_OK) return q;
        }
    }
    // N of at most 32 blocks (off the pages' grid, whose N starts at 2112):
    // the register mode, past K = 2048 with four waves and enough K splits
    // (at most 8) to bring the grid towards 256 workgroups, else unsplit
    // with eight waves (four at most 12 K steps).  Over 40 seeded off-grid
    // shapes the other rules left such grids at 9 .. 26 workgroups (1.12-1.41x
    // the best plan at N = 288 .. 672, K = 2816 .. 6144); at K = 1024 .. 2048
    // the splits' reduction cost more than they saved (1.25-1.52x).
    if (RBn <= 32) {
        Plan q{1, 1, 1, KS > 32 || KS <= 12 ? 4 : 8, 1, kAmDirect, 0};
        if (KS > 32) {
            const long long wgs = (long long)RBm * RBn;
            q.splits = wgs >= 128 ? 1 : wgs >= 64 ? 2 : wgs >= 32 ? 4 : 8;
        }
        while (q.splits < KS && plan_layout(q, M, N, K, &l) != MX_OK) ++q.splits;
        if (plan_layout(q, M, N, K, &l) == MX_OK) return q;
    }
    if (deep && (RBm == 1 || (RBm == 2 && N >= 7168) || (RBm <= 4 && N <= 2112))) {
        Plan q{1, 1, 4, 4, 1, kAmShared, 0};
        if (N >= 7168 && RBm == 2) {
            q = Plan{2, 1, 1, 8, 2, kAmPrequant, 0};
        } else if (N >= 7168 && M > 8) {
            q = Plan{1, 2, 1, 8, 2, kAmDirect, 0};
        } else if (N >= 7168) {
            q.splits = (KS + 7) / 8;
        } else {
            q.splits = (KS + 15) / 16;
            if (RBn % 3 == 0 && (long long)((RBn + 2) / 3) * RBm * q.splits <= 256) q.wn = 3;
        }
        if (plan_layout(q, M, N, K, &l) == MX_OK) return q;
    }
    // quantiser waves for the whole workgroup: at least 8 M blocks, or 4
    // with a short K or a wide N, or 2 with both, or 5 to 7 where the grid
    // fits one round on the 256 CUs with N tiles of 3 or 4 whole N blocks
    // (shared_round_wn), when the split's K fits their budget
    const int round_wn = shared_round_wn(RBm, RBn);
    const bool shared = KS <= 24 && (RBm >= 8 || (RBm >= 5 && round_wn > 0) || (RBm >= 4 && (KS <= 8 || N >= 7168)) ||
                                     (RBm >= 2 && KS <= 8 && N >= 7168));
    const bool pre = !shared && RBm >= 4 && KS > 8 && (RBm > 4 || N >= 7168 || KS > 32);
    Plan p;
    p.finish = 0;
    p.splits = 1;
    // (four waves at 9 .. 12 K steps: 11 % faster than eight at K = 768)
    p.wk = KS <= 8 ? pow2_floor(KS >= 8 ? 4 : (KS + 1) / 2) : KS <= 12 ? 4 : 8;
    if (shared) {
        // the MFMA waves of shared_round_wn, else three when the N blocks
        // divide by 3 (no ragged tile), else four; four quantiser waves for a
        // short K below 32 M blocks from 12, or where the grid runs in more
        // than one round (256 x 7168 x 512: 4 % faster; 255 x 8064 x 512:
        // 14 %)
        p.amode = kAmShared;
        p.mb = 1;
        p.nb = 1;
        p.wn = round_wn > 0 ? round_wn : RBn % 3 == 0 ? 3 : 4;
        const long long grid = (long long)RBm * ((RBn + p.wn - 1) / p.wn);
        p.wk = KS <= 8 && RBm < 32 && (RBm >= 12 || grid > 256) ? 4 : 8;
        return p;
    }
    if (pre) {
        // one N block per wave for deep K, and from 12 M blocks below N = 7168
        p.amode = kAmPrequant;
        p.mb = 2;
        p.nb = 1;
        p.wn = deep || (RBm >= 12 && N < 7168) ? 1 : 2;
    } else {
        p.amode = kAmDirect;
        p.mb = 1;
        p.nb = (RBm >= 4 || (RBm >= 2 && N >= 7168) || deep) ? 2 : 1;
        p.wn = 1;
    }
    while (p.splits < KS && plan_layout(p, M, N, K, &l) != MX_OK) ++p.splits;
    if (deep && !pre && p.splits < 2) p.splits = 2;
    return p;
}

Plan choose_plan(int M, int N, int K) {
    for (const TableEntry& e : kTable)
        if (e.M == M && e.N == N && e.K == K) return e.plan;
    return model_plan(M, N, K);
}

// Plans measured for the a16wfp4 product on the same shapes.
const TableEntry kTableA16w4[] = {
    {4, 2880, 512, {1, 1, 1, 4, 1, 3, 0}},
    {32, 4096, 512, {1, 1, 1, 4, 1, 3, 0}},
    {32, 2880, 512, {1, 1, 1, 4, 1, 3, 0}},
    {16, 2112, 7168, {1, 1, 1, 4, 7, 3, 0}},
    {64, 7168, 2048, {1, 2, 1, 8, 1, 3, 0}},
    {256, 3072, 1536, {1, 2, 2, 8, 1, 3, 0}},
};

// The a16wfp4 product: a measured plan, else the tiling of the MXFP4 plan
// with A left in bf16: one 32-row M block per wave (the raw A registers),
// then the fewest splits that fit the register budget.
Plan choose_plan_a16w4(int M, int N, int K) {
    for (const TableEntry& e : kTableA16w4)
        if (e.M == M && e.N == N && e.K == K) return e.plan;
    Plan p = choose_plan(M, N, K);
    if (p.amode == kAmShared || p.amode == kAmStream || p.amode == kAmTile) {
        // tilings of modes the bf16 kernels do not have: one wave along N,
        // waves along K as the register mode takes them
        const OperandGeom gk = mx4::operand_geom(N, K);
        p.nb = 1;
        p.wn = 1;
        p.wk = gk.KS <= 8 ? pow2_floor(gk.KS >= 8 ? 4 : (gk.KS + 1) / 2) : 8;
        p.splits = 1;
    }
    p.amode = kAmBf16;
    p.mb = 1;
    const OperandGeom gb = mx4::operand_geom(N, K);
    Layout l;
    while (p.splits < gb.KS && plan_layout(p, M, N, K, &l) != MX_OK) ++p.splits;
    return p;
}

// Everything of a call that depends on the shape and plan only: checked
// once, then kept in a small per-thread cache, so that a repeated call only
// checks its pointers, patches them into its copy of the call's GemmParams and
// launches.
struct Prepared {
    int M, N, K, lda, ldc;
    Plan plan;
    Layout lay;
    GemmParams p;            // pointer fields left null
    mx4::GemmLaunch gl;
    bool finish_in_gemm;
};

bool same_key(const Prepared& e, int M, int N, int K, int lda, int ldc, const Plan& pl) {
    return e.M == M && e.N == N && e.K == K && e.lda == lda && e.ldc == ldc && e.plan.mb == pl.mb &&
           e.plan.nb == pl.nb && e.plan.wn == pl.wn && e.plan.wk == pl.wk && e.plan.splits == pl.splits &&
           e.plan.amode == pl.amode && e.plan.finish == pl.finish;
}

int prepare(int M, int N, int K, int lda, int ldc, const Plan& plan, Prepared* out) {
    int rc = check_operand_shape(M, K);
    if (rc) return rc;
    rc = check_operand_shape(N, K);
    if (rc) return rc;
    if (lda < K || lda % 8 != 0 || ldc < N) return MX_EINVAL;
    if ((unsigned long long)M * lda * 2 >= (1ULL << 31)) return MX_EINVAL;
    Layout lay;
    rc = plan_layout(plan, M, N, K, &lay);
    if (rc) return rc;
    const OperandGeom ga = mx4::operand_geom(M, K);
    const OperandGeom gb = mx4::operand_geom(N, K);
    Prepared e;
    memset(&e, 0, sizeof e);
    e.M = M;
    e.N = N;
    e.K = K;
    e.lda = lda;
    e.ldc = ldc;
    e.plan = plan;
    e.lay = lay;
    GemmParams& p = e.p;
    p.lda = lda;
    p.a_bytes = (uint32_t)((size_t)M * lda * 2);
    p.aop_bytes = (uint32_t)ga.total_bytes;
    p.a_code_bytes = (uint32_t)ga.code_bytes;
    p.bp_bytes = (uint32_t)gb.total_bytes;
    p.b_code_bytes = (uint32_t)gb.code_bytes;
    p.KS = gb.KS;
    p.KW = gb.KW;
    p.M = M;
    p.N = N;
    p.K = K;
    p.RBm = ga.RB;
    p.RBn = gb.RB;
    p.mtiles = lay.mtiles;
    p.ntiles = lay.ntiles;
    p.splits = lay.splits;
    p.steps_per_split = lay.steps_per_split;
    p.ldc = ldc;
    p.partial_bytes = (uint32_t)lay.partial_bytes;
    p.ldp = gb.RB * mx4::kRowBlock;
    e.finish_in_gemm = lay.splits > 1 && plan.finish == 1;
    Plan run = plan;
    run.splits = lay.splits;
    if (!mx4::resolve_gemm(run, p, &e.gl)) return MX_EPLAN;
    *out = e;
    return MX_OK;
}

constexpr int kPreparedCache = 4;
thread_local Prepared tl_prepared[kPreparedCache];
thread_local int tl_prepared_count = 0, tl_prepared_next = 0;

int gemm_impl(const void* A, int M, int K, int lda, const void* packed, int N, void* C, int ldc, void* ws,
              size_t ws_bytes, const Plan& plan, void* stream) {
    const Prepared* e = nullptr;
    for (int i = 0; i < tl_prepared_count; ++i)
        if (same_key(tl_prepared[i], M, N, K, lda, ldc, plan)) {
            e = &tl_prepared[i];
            break;
        }
    if (!e) {
        Prepared fresh;
        const int rc = prepare(M, N, K, lda, ldc, plan, &fresh);
        if (rc) return rc;
        Prepared& slot = tl_prepared[tl_prepared_next];
        slot = fresh;
        tl_prepared_next = (tl_prepared_next + 1) % kPreparedCache;
        if (tl_prepared_count < kPreparedCache) ++tl_prepared_count;
        e = &slot;
    }
    if (!aligned(A, 16) || !aligned(packed, 16) || !aligned(C, 2)) return MX_EALIGN;
    const Layout& lay = e->lay;
    if (lay.total > 0) {
        if (!aligned(ws, 256)) return MX_EALIGN;
        if (ws_bytes < lay.total) return MX_ESPACE;
    }
    uint8_t* wsb = (uint8_t*)ws;
    hipStream_t s = (hipStream_t)stream;
    GemmParams p = e->p;
    p.A = (const uint16_t*)A;
    p.aop = mx4::amode_prequantises(plan.amode) ? wsb + lay.aop_offset : nullptr;
    p.bp = (const uint8_t*)packed;
    p.C = (uint16_t*)C;
    p.c_vec = (ldc % 4 == 0 && aligned(C, 8)) ? 1 : 0;
    p.partial = lay.splits > 1 ? (float*)(wsb + lay.partial_offset) : nullptr;
    p.counters = e->finish_in_gemm ? (uint32_t*)wsb : nullptr;

    int rc;
    if (mx4::amode_prequantises(plan.amode)) {
        rc = hip_status(mx4::launch_pack((const uint16_t*)A, M, K, lda, wsb + lay.aop_offset, s));
        if (rc) return rc;
    }
    rc = hip_status(mx4::launch_gemm(e->gl, p, s));
    if (rc) return rc;
    if (lay.splits > 1 && !e->finish_in_gemm) rc = hip_status(mx4::launch_reduce(p, s));
    return rc;
}

}  // namespace

extern "C" {

const char* mx_strerror(int code) {
    switch (code) {
        case MX_OK: return "success";
        case MX_EINVAL: return "invalid shape or leading dimension";
        case MX_EALIGN: return "null or misaligned pointer";
        case MX_ESPACE: return "buffer or workspace too small";
        case MX_EHIP: return "HIP kernel launch failed";
        case MX_EPLAN: return "plan not supported for this shape";
        default: return "unknown error code";
    }
}

int mx_packed_weight_bytes(int N, int K, size_t* bytes_host) {
    if (!bytes_host) return MX_EALIGN;
    int rc = check_operand_shape(N, K);
    if (rc) return rc;
    *bytes_host = mx4::operand_geom(N, K).total_bytes;
    return MX_OK;
}

int mx_pack_weight(const void* B_dev, int N, int K, int ldb, void* packed_dev, size_t packed_bytes, void* stream) {
    int rc = check_operand_shape(N, K);
    if (rc) return rc;
    if (ldb < K || ldb % 8 != 0) return MX_EINVAL;
    if ((unsigned long long)N * ldb * 2 >= (1ULL << 31)) return MX_EINVAL;   // 32-bit buffer offsets
    if (!aligned(B_dev, 16) || !aligned(packed_dev, 16)) return MX_EALIGN;
    if (packed_bytes < mx4::operand_geom(N, K).total_bytes) return MX_ESPACE;
    return hip_status(mx4::launch_pack((const uint16_t*)B_dev, N, K, ldb, (uint8_t*)packed_dev, (hipStream_t)stream));
}

int mx_unpack_weight(const void* packed_dev, int N, int K, void* codes_dev, void* scales_dev, void* stream) {
    int rc = check_operand_shape(N, K);
    if (rc) return rc;
    if (!aligned(packed_dev, 16) || !aligned(codes_dev, 16) || !aligned(scales_dev, 1)) return MX_EALIGN;
    return hip_status(mx4::launch_unpack((const uint8_t*)packed_dev, N, K, (uint8_t*)codes_dev, (uint8_t*)scales_dev,
                                         (hipStream_t)stream));
}

int mx_import_weight(const void* codes_dev, const void* scales_dev, int N, int K, void* packed_dev,
                     size_t packed_bytes, void* stream) {
    int rc = check_operand_shape(N, K);
    if (rc) return rc;
    if (!aligned(codes_dev, 16) || !aligned(scales_dev, 1) || !aligned(packed_dev, 16)) return MX_EALIGN;
    if (packed_bytes < mx4::operand_geom(N, K).total_bytes) return MX_ESPACE;
    return hip_status(mx4::launch_import((const uint8_t*)codes_dev, (const uint8_t*)scales_dev, N, K,
                                         (uint8_t*)packed_dev, (hipStream_t)stream));
}

int mx_quant_act(const void* A_dev, int M, int K, int lda, void* codes_dev, void* scales_dev, void* stream) {
    int rc = check_operand_shape(M, K);
    if (rc) return rc;
    if (lda < K || lda % 8 != 0) return MX_EINVAL;
    if (!aligned(A_dev, 16) || !aligned(codes_dev, 4) || !aligned(scales_dev, 1)) return MX_EALIGN;
    return hip_status(mx4::launch_quant_natural((const uint16_t*)A_dev, M, K, lda, (uint8_t*)codes_dev,
                                                (uint8_t*)scales_dev, (hipStream_t)stream));
}

int mx_gemm_plan(int M, int N, int K, mx_plan* plan_host) {
    if (!plan_host) return MX_EALIGN;
    int rc = check_operand_shape(M, K);
    if (rc) return rc;
    rc = check_operand_shape(N, K);
    if (rc) return rc;
    const Plan p = choose_plan(M, N, K);
    Layout lay;
    rc = plan_layout(p, M, N, K, &lay);
    if (rc) return rc;
    plan_host->mb = p.mb;
    plan_host->nb = p.nb;
    plan_host->wn = p.wn;
    plan_host->wk = p.wk;
    plan_host->splits = lay.splits;
    plan_host->amode = p.amode;
    plan_host->finish = p.finish;
    return MX_OK;
}

int mx_gemm_plan_workspace_bytes(const mx_plan* plan_host, int M, int N, int K, size_t* bytes_host) {
    if (!plan_host || !bytes_host) return MX_EALIGN;
    int rc = check_operand_shape(M, K);
    if (rc) return rc;
    rc = check_operand_shape(N, K);
    if (rc) return rc;
    const Plan p = {plan_host->mb,     plan_host->nb,    plan_host->wn,    plan_host->wk,
                    plan_host->splits, plan_host->amode, plan_host->finish};
    Layout lay;
    rc = plan_layout(p, M, N, K, &lay);
    if (rc) return rc;
    *bytes_host = lay.total;
    return MX_OK;
}

int mx_gemm_workspace_bytes(int M, int N, int K, size_t* bytes_host) {
    mx_plan p;
    int rc = mx_gemm_plan(M, N, K, &p);
    if (rc) return rc;
    return mx_gemm_plan_workspace_bytes(&p, M, N, K, bytes_host);
}

int mx_gemm_with_plan(const void* A_dev, int M, int K, int lda, const void* packed_dev, int N, void* C_dev, int ldc,
                      void* ws_dev, size_t ws_bytes, const mx_plan* plan_host, void* stream) {
    if (!plan_host) return MX_EALIGN;
    const Plan p = {plan_host->mb,     plan_host->nb,    plan_host->wn,    plan_host->wk,
                    plan_host->splits, plan_host->amode, plan_host->finish};
    return gemm_impl(A_dev, M, K, lda, packed_dev, N, C_dev, ldc, ws_dev, ws_bytes, p, stream);
}

int mx_gemm(const void* A_dev, int M, int K, int lda, const void* packed_dev, int N, void* C_dev, int ldc,
            void* ws_dev, size_t ws_bytes, void* stream) {
    return gemm_impl(A_dev, M, K, lda, packed_dev, N, C_dev, ldc, ws_dev, ws_bytes, choose_plan(M, N, K), stream);
}

int mx_gemm_a16w4_plan(int M, int N, int K, mx_plan* plan_host) {
    if (!plan_host) return MX_EALIGN;
    int rc = check_operand_shape(M, K);
    if (rc) return rc;
    rc = check_operand_shape(N, K);
    if (rc) return rc;
    const Plan p = choose_plan_a16w4(M, N, K);
    Layout lay;
    rc = plan_layout(p, M, N, K, &lay);
    if (rc) return rc;
    *plan_host = mx_plan{p.mb, p.nb, p.wn, p.wk, lay.splits, p.amode, p.finish};
    return MX_OK;
}

int mx_gemm_a16w4_workspace_bytes(int M, int N, int K, size_t* bytes_host) {
    mx_plan p;
    int rc = mx_gemm_a16w4_plan(M, N, K, &p);
    if (rc) return rc;
    return mx_gemm_plan_workspace_bytes(&p, M, N, K, bytes_host);
}

int mx_gemm_a16w4(const void* A_dev, int M, int K, int lda, const void* packed_dev, int N, void* C_dev, int ldc,
                  void* ws_dev, size_t ws_bytes, void* stream) {
    return gemm_impl(A_dev, M, K, lda, packed_dev, N, C_dev, ldc, ws_dev, ws_bytes, choose_plan_a16w4(M, N, K),
                     stream);
}

}  // extern "C"
