// mx4_tile.hip -- K-looped, LDS-pipelined block-scaled MXFP4 GEMM for gfx950
// (MI355X) on MFMA-bound shapes: the activation mode MX_AMODE_TILE.
//
//   C[M,N] = bf16_RNE( sum_k deq(A)[m,k] * deq(B)[n,k] )   (fp32 accumulation)
//
// The contraction is the block-scaled dot of the kernelindex.com
// amd-mxfp4-mm pages (tl.dot_scaled(..., "e2m1", ..., "e2m1"), submission
// 748756, kernel_fused_mxfp4_gemm) on v_mfma_scale_f32_32x32x64_f8f6f4.  The
// activation is quantised beforehand by pack_kernel (the rule of submission
// 755056, "Software MXFP4 quant") into the same packed layout as the weight,
// so both operands arrive as 1 KiB MFMA operand tiles and 256-byte scale
// words.
//
// Where M is large the work is MFMA-bound, not weight-bound, and the kernel
// is the classic tiled GEMM: a workgroup owns 32 MB rows x 32 NB columns of
// C over the whole of K and walks K one 64-K step at a time.  Tiles run from
// 64 x 64 to 256 x 256; the small ones give a grid of enough workgroups
// where M or N is short, so the same kernel also serves M from 96 up at
// deep K, re-reading the weight from L2 a few times instead of once.  Each
// step's operand tiles (MB of A, NB of B) and their scale words go straight
// from memory into a ring of S LDS stages (gfx950 buffer loads to LDS,
// issued S steps ahead); its WM x WN waves each read the fragments of their
// TM x TN blocks (TM = MB / WM, TN = NB / WN) from the stage one step ahead,
// into registers, and run TM x TN MFMAs, so every operand tile feeds
// several MFMAs from LDS and a wave's LDS reads overlap its MFMAs.  Every
// wave issues the same number of loads per step (steps past K load from an
// offset past the buffer and read zeros), so the wait for a step is a
// compile-time count.
// One barrier every G steps, with no memory fence (a fence would wait for
// the loads of the steps in flight), tells the waves that every wave's loads
// of the next G steps have landed and that the stages of the steps already
// read are free.
// The epilogue stages each wave's bf16 tiles in the (then dead) ring and
// stores them in 16-byte row chunks.  Where K is split over workgroups
// (grid z), each split walks its own run of steps and writes fp32 partials
// that reduce_kernel sums in split order.
#include "mx4_device.h"
#include <type_traits>

#include "mx4_internal.h"

namespace mx4 {

constexpr int kTileOpBytes = 1024;   // one packed operand tile: 64 lanes x 16 B
constexpr int kTileWordBytes = 256;  // one packed scale word group: 64 lanes x 4 B

// Scale word groups (4 steps each) the ring holds with S tile stages.  The
// words of group h + W are issued with the tiles of step 4 (h + W), after the
// barrier of step 4 (h + W) - S or a later one; group h's words were last
// read from LDS at step 4 h - 1, before the barrier of step 4 h, so W slots
// suffice once 4 W >= S.
__host__ __device__ constexpr int tile_word_slots(int s) { return (s + 3) / 4; }

// LDS of a kernel with S tile stages: S stages of the step's MB + NB operand
// tiles, then tile_word_slots(S) groups of their scale words.
__host__ __device__ constexpr size_t tile_lds_bytes_for(int mb, int nb, int s) {
    return (size_t)(mb + nb) * (s * kTileOpBytes + tile_word_slots(s) * kTileWordBytes);
}

// 4-byte buffer load straight into LDS: lane L's dword lands at lds_base + 4 L.
__device__ __forceinline__ void bload4_lds(Rsrc r, uint8_t* lds_base, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 4, (int)voff, 0, 0,
                                             0);
}

// One block-scaled fp4 MFMA whose scales are byte SEL of each scale register
// (the instruction's op_sel), so the K step's byte needs no shift.
template <int SEL>
__device__ __forceinline__ f32x16 mfma_fp4_sel(const u32x4& a, const u32x4& b, f32x16 acc, uint32_t scale_a,
                                               uint32_t scale_b) {
    i32x8 va = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    i32x8 vb = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc, 4, 4, SEL, (int)scale_a, SEL, (int)scale_b);
}

// The workgroup syncs once every G steps, at the barrier before step t
// (t a multiple of G, t = u mod 4).  Loads of a wave that may still be
// outstanding there once the tiles and words of every step up to t + G have
// landed: the tiles of steps t + G + 1 .. t + S - G (issued at earlier
// barriers) and the word groups whose first step is among them.
__host__ __device__ constexpr int tile_wait_count(int lpw, int s, int g, int u) {
    int groups = 0;
    for (int x = u + g + 1; x <= u + s - g; ++x) groups += (x % 4 == 0);
    return lpw * (s - 2 * g) + lpw * groups;
}

// The same before the first barrier: steps 0 .. S - G issued, step 0 landed.
__host__ __device__ constexpr int tile_prologue_wait(int lpw, int s, int g) {
    int groups = 0;
    for (int x = 1; x <= s - g; ++x) groups += (x % 4 == 0);
    return lpw * (s - g) + lpw * groups;
}

// Scheduling order of one K step after its barrier: the buffer loads, then
// N LDS reads each followed by one MFMA (the rest of the MFMAs follow).
template <int N>
__device__ __forceinline__ void order_reads_between_mfmas() {
    if constexpr (N > 0) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        order_reads_between_mfmas<N - 1>();
    }
}

template <int MB, int NB, int WM, int WN, int S, int G>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_tile_kernel(const void* a_src, const uint8_t* bp, uint16_t* C, float* partial_buf, int lda, int ldc, int M,
                 int N, int K, int steps_arg, uint32_t* counters, int splits, int mtiles) {
    (void)lda;
    (void)counters;
    (void)mtiles;
    constexpr int TM = MB / WM, TN = NB / WN, NW = WM * WN;
    constexpr int OPS = MB + NB;   // operand blocks per step
    static_assert(MB % WM == 0 && NB % WN == 0 && OPS % NW == 0, "whole blocks per wave");
    constexpr int LPW = OPS / NW;  // blocks each wave loads per step
    constexpr int WS = tile_word_slots(S);
    constexpr int TSTAGE = OPS * kTileOpBytes;
    constexpr int WGROUP = OPS * kTileWordBytes;
    constexpr uint32_t kOutOfRange = 0x80000000u;
    static_assert(G >= 1 && 4 % G == 0 && S >= 2 * G, "syncs on a 4-step boundary, two sync intervals in the ring");
    static_assert(tile_prologue_wait(LPW, S, G) < 64, "vmcnt range");

    const OperandGeom ga = operand_geom(M, K), gb = operand_geom(N, K);
    const int KS = gb.KS, KW = gb.KW;
    // steps_arg: the placement code in bits 0..7, the K steps per split (a
    // multiple of 4 when K is split) above them; split z takes steps
    // t0 .. t0 + nsteps - 1 of K
    const int xcd_map = steps_arg & 0xFF;
    const int t0 = (int)blockIdx.z * (steps_arg >> 8);
    const int nsteps = min(KS - t0, steps_arg >> 8);
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    uint8_t* words = lds + (size_t)S * TSTAGE;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int L = tid & 63;
    const int wm = wave / WN, wn = wave % WN;
    // the tile of this workgroup, placed on the XCDs by the placement code
    // (shared_tile_of)
    int mt, nt;
    shared_tile_of((int)blockIdx.x, (int)blockIdx.y, (gb.RB + NB - 1) / NB, (ga.RB + MB - 1) / MB, xcd_map, mt, nt);
    const int rbm0 = mt * MB, rbn0 = nt * NB;
    // Wave w loads blocks q = w LPW .. w LPW + LPW - 1 of a step, q < MB
    // being A block rbm0 + q and the rest B block rbn0 + q - MB: the 1 KiB
    // tile (rb, t) of step t into tile stage t % S and, for the first step of
    // each 4-step group h, the scale word group (rb, h) into word slot
    // h % WS, issued just before that step's tiles (t counts the split's
    // steps: step t is step t0 + t of K, and t0 is a multiple of 4).  Blocks
    // past the operand and steps past the split read zeros.  Each block's
    // resource and offsets are values set up once here.
    Rsrc rsrc[LPW];
    bool rb_live[LPW];
    uint32_t tile_base[LPW], word_base[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int q = wave * LPW + i;
        int rb, rb_end;
        uint32_t word_region;
        if (q < MB) {
            rb = rbm0 + q;
            rb_end = ga.RB;
            word_region = (uint32_t)ga.code_bytes;
            rsrc[i] = make_rsrc(a_src, (uint32_t)ga.total_bytes);
        } else {
            rb = rbn0 + (q - MB);
            rb_end = gb.RB;
            word_region = (uint32_t)gb.code_bytes;
            rsrc[i] = make_rsrc(bp, (uint32_t)gb.total_bytes);
        }
        rb_live[i] = rb < rb_end;
        tile_base[i] = ((uint32_t)(rb * KS + t0) * 64u + (uint32_t)L) * 16u;
        word_base[i] = word_region + ((uint32_t)(rb * KW + (t0 >> 2)) * 64u + (uint32_t)L) * 4u;
    }
    auto issue = [&](int t, int ws) {
        if ((t & 3) == 0) {
#pragma unroll
            for (int i = 0; i < LPW; ++i) {
                const uint32_t woff = rb_live[i] && t < nsteps ? word_base[i] + (uint32_t)(t >> 2) * 256u : kOutOfRange;
                bload4_lds(rsrc[i], words + (size_t)ws * WGROUP + (wave * LPW + i) * kTileWordBytes, woff);
            }
        }
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const uint32_t toff = rb_live[i] && t < nsteps ? tile_base[i] + (uint32_t)t * 1024u : kOutOfRange;
            bload16_lds(rsrc[i], lds + (size_t)(t % S) * TSTAGE + (wave * LPW + i) * kTileOpBytes, toff);
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // a wave's fragments of one step (TM A and TN B tiles, 16 bytes a lane)
    // and the scale words of its 4-step group
    struct Frags {
        u32x4 a[TM], b[TN];
        uint32_t as[TM], bs[TN];
    };
    auto read_tiles = [&](int t, Frags& f) {
        const uint8_t* st = lds + (size_t)(t % S) * TSTAGE;
#pragma unroll
        for (int i = 0; i < TM; ++i) f.a[i] = *(const u32x4*)(st + (wm * TM + i) * kTileOpBytes + 16 * L);
#pragma unroll
        for (int j = 0; j < TN; ++j) f.b[j] = *(const u32x4*)(st + (MB + wn * TN + j) * kTileOpBytes + 16 * L);
    };
    auto read_words = [&](int ws, Frags& f) {
        const uint8_t* wg = words + (size_t)ws * WGROUP;
#pragma unroll
        for (int i = 0; i < TM; ++i) f.as[i] = *(const uint32_t*)(wg + (wm * TM + i) * kTileWordBytes + 4 * L);
#pragma unroll
        for (int j = 0; j < TN; ++j) f.bs[j] = *(const uint32_t*)(wg + (MB + wn * TN + j) * kTileWordBytes + 4 * L);
    };

    // The ring holds S steps; word slot of group h: h % WS (tile_word_slots
    // says why WS slots suffice).  Step t's fragments are read into
    // registers one step ahead, so a wave's LDS reads of step t + 1 overlap
    // its MFMAs of step t.  The workgroup syncs every G steps: the barrier
    // before step t (t a multiple of G) tells every wave that the loads of
    // steps up to t + G have landed everywhere and that every wave has read
    // the steps up to t (its LDS reads completed), whose stages then take
    // steps t + S - G + 1 .. t + S.  The prologue issues steps 0 .. S - G.
    int ws_issue = 0;   // word slot of the next group to issue
#pragma unroll
    for (int t = 0; t <= S - G; ++t) {
        issue(t, ws_issue);
        if ((t & 3) == 0) ws_issue = ws_issue == WS - 1 ? 0 : ws_issue + 1;
    }
    wait_vmcnt<tile_prologue_wait(LPW, S, G)>();   // step 0 and its words have landed
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    Frags cur, nxt;
    read_tiles(0, cur);
    read_words(0, cur);
    int ws_read = 0;    // word slot of the group being read
    const int groups = (nsteps + 3) / 4;
    // one K step at position U of its 4-step group (U fixes the sync, the
    // wait count, the scale byte and whether the next group's words are read)
    auto step = [&](int t, auto uc) {
        constexpr int U = decltype(uc)::value;
        // (scheduling fences keep each step's MFMAs inside the step, on
        // fragments already in registers)
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (U % G == 0) {
            // a wave's loads complete in issue order: at most the loads
            // issued after step t + G's tiles are outstanding
            wait_vmcnt<tile_wait_count(LPW, S, G, U)>();
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < G; ++j) {
                issue(t + S - G + 1 + j, ws_issue);
                if (((U + S - G + 1 + j) & 3) == 0) ws_issue = ws_issue == WS - 1 ? 0 : ws_issue + 1;
            }
        }
        read_tiles(t + 1, nxt);
        if constexpr (U == 3) {
            ws_read = ws_read == WS - 1 ? 0 : ws_read + 1;
            read_words(ws_read, nxt);
        } else {
#pragma unroll
            for (int i = 0; i < TM; ++i) nxt.as[i] = cur.as[i];
#pragma unroll
            for (int j = 0; j < TN; ++j) nxt.bs[j] = cur.bs[j];
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = mfma_fp4_sel<U>(cur.b[j], cur.a[i], acc[i][j], cur.bs[j], cur.as[i]);
        // the loads go out first; the reads of step t + 1 then run under
        // this step's MFMAs
        if constexpr (U % G == 0) __builtin_amdgcn_sched_group_barrier(0x020, 2 * LPW * G, 0);
        order_reads_between_mfmas<(TM + TN < TM * TN ? TM + TN : TM * TN)>();
        __builtin_amdgcn_sched_group_barrier(0x008, TM * TN, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (TM + TN), 0);
        cur = nxt;
    };
    for (int g = 0; g < groups; ++g) {
        step(4 * g + 0, std::integral_constant<int, 0>{});
        step(4 * g + 1, std::integral_constant<int, 1>{});
        step(4 * g + 2, std::integral_constant<int, 2>{});
        step(4 * g + 3, std::integral_constant<int, 3>{});
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mfma_result_fence(acc[i][j]);

    // ---- epilogue: the ring is dead once every wave's loads (including the
    // zero-filling ones issued past K) have landed and every wave has read
    // its last fragments.  Lane L, element e of block (i, j):
    // m = 32 (rbm0 + wm TM + i) + L % 32,
    // n = 32 (rbn0 + wn TN + j) + 8 (e / 4) + 4 (L / 32) + e % 4.
    wait_vmcnt<0>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int m_lane = L & 31;
    const int n_lane = 4 * (L >> 5);
    if (splits > 1) {
        // a split's fp32 partials, [split][m][n] with row stride 32 RB(N)
        // (reduce_kernel sums them in split order): 4 consecutive n a lane
        const int ldp = gb.RB * kRowBlock;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int m = (rbm0 + wm * TM + i) * kRowBlock + m_lane;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int nb = rbn0 + wn * TN + j;
                if (m >= M || nb >= gb.RB) continue;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const f32x4 v = {acc[i][j][4 * r], acc[i][j][4 * r + 1], acc[i][j][4 * r + 2],
                                     acc[i][j][4 * r + 3]};
                    *(f32x4*)(partial_buf + ((size_t)blockIdx.z * M + m) * ldp + nb * kRowBlock + 8 * r + n_lane) = v;
                }
            }
        }
        return;
    }
    constexpr int WC = TN * kRowBlock;   // columns of a wave's row of blocks
    constexpr int WROW = WC + 8;          // bf16 per staged row (16-byte pad)
    static_assert((size_t)NW * kRowBlock * WROW * 2 <= (size_t)S * TSTAGE, "stages fit the ring");
    uint16_t* wst = (uint16_t*)(lds + (size_t)wave * kRowBlock * WROW * 2);
    const int n_base = (rbn0 + wn * TN) * kRowBlock;
    const bool vec16 = ((uintptr_t)C % 16 == 0) && (ldc % 8 == 0);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint2 w;
                w.x = pack_bf16x2(acc[i][j][4 * r], acc[i][j][4 * r + 1]);
                w.y = pack_bf16x2(acc[i][j][4 * r + 2], acc[i][j][4 * r + 3]);
                *(uint2*)(wst + m_lane * WROW + j * kRowBlock + 8 * r + n_lane) = w;
            }
        // the wave reads back its own LDS writes (in order within a wave)
        const int m_base = (rbm0 + wm * TM + i) * kRowBlock;
        static_assert(kRowBlock * WC / 8 % 64 == 0, "whole 16-byte chunks per lane");
#pragma unroll
        for (int k = 0; k < kRowBlock * WC / 8 / 64; ++k) {
            const int c = L + 64 * k;
            const int row = c / (WC / 8), c8 = c % (WC / 8);
            const int m = m_base + row, n = n_base + 8 * c8;
            const u32x4 v = *(const u32x4*)(wst + row * WROW + 8 * c8);
            if (m >= M || n >= N) continue;
            uint16_t* dst = C + (size_t)m * ldc + n;
            if (vec16 && n + 7 < N) {
                __builtin_nontemporal_store(v, (u32x4*)dst);
            } else {
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    if (n + q < N) dst[q] = (uint16_t)(w[q >> 1] >> (16 * (q & 1)));
            }
        }
        // the next row of blocks overwrites the stage: this wave's reads of
        // it have completed
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
}

// ---------------------------------------------------------------------------
// Instantiations.  Plan fields of this mode: mb and nb are the 32-row and
// 32-column blocks of the workgroup tile, wk the waves along M and wn the
// waves along N (splits 1).

constexpr int kTileStages = 8;
constexpr int kTileDeepStages = 16;   // the 64 x 64 tile on a grid of at most one workgroup per CU
constexpr int kTileSync = 2;          // K steps per workgroup barrier

// Ring depth of a tile-mode launch of `wgs` workgroups.  The 64 x 64 tile
// moves only 4 KiB per step, so 8 stages keep too few bytes in flight to
// cover the load latency when a CU holds a single workgroup: there 16 stages
// (68 KiB of LDS, two workgroups per CU) were 10-17 % faster for K >= 4096
// and 2 % at 2048, measured against 8 over grids of 64 .. 256 workgroups.
// With more workgroups than CUs the 8-stage ring's four workgroups per CU
// hide the latency instead, and 16 stages were up to 9 % slower; 24 and 32
// stages were slower than 16 everywhere, and the larger tiles gained nothing.
int tile_stages(const Plan& plan, long long wgs) {
    return plan.mb == 2 && plan.nb == 2 && wgs <= 256 ? kTileDeepStages : kTileStages;
}

GemmKernelFn find_tile_kernel(const Plan& plan, int stages) {
    if (stages == kTileDeepStages)
        return plan.mb == 2 && plan.nb == 2 && plan.wk == 2 && plan.wn == 2
                   ? gemm_tile_kernel<2, 2, 2, 2, kTileDeepStages, kTileSync>
                   : nullptr;
    if (stages != kTileStages) return nullptr;
    if (plan.mb == 8 && plan.nb == 8 && plan.wk == 2 && plan.wn == 4)
        return gemm_tile_kernel<8, 8, 2, 4, kTileStages, kTileSync>;
    if (plan.mb == 4 && plan.nb == 8 && plan.wk == 2 && plan.wn == 2)
        return gemm_tile_kernel<4, 8, 2, 2, kTileStages, kTileSync>;
    if (plan.mb == 8 && plan.nb == 4 && plan.wk == 2 && plan.wn == 2)
        return gemm_tile_kernel<8, 4, 2, 2, kTileStages, kTileSync>;
    if (plan.mb == 4 && plan.nb == 4 && plan.wk == 2 && plan.wn == 2)
        return gemm_tile_kernel<4, 4, 2, 2, kTileStages, kTileSync>;
    if (plan.mb == 4 && plan.nb == 4 && plan.wk == 2 && plan.wn == 4)
        return gemm_tile_kernel<4, 4, 2, 4, kTileStages, kTileSync>;
    if (plan.mb == 2 && plan.nb == 2 && plan.wk == 2 && plan.wn == 2)
        return gemm_tile_kernel<2, 2, 2, 2, kTileStages, kTileSync>;
    return nullptr;
}

GemmKernelFn find_tile_kernel(const Plan& plan) { return find_tile_kernel(plan, kTileStages); }

size_t tile_lds_bytes(const Plan& plan, int stages) { return tile_lds_bytes_for(plan.mb, plan.nb, stages); }

size_t tile_lds_bytes(const Plan& plan) { return tile_lds_bytes(plan, kTileStages); }

}  // namespace mx4
