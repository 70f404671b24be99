// mx4_shared.hip -- block-scaled MXFP4 GEMM for gfx950 (MI355X) with the
// activation quantised once per workgroup by dedicated waves: the activation
// mode MX_AMODE_SHARED.
//
//   C[M,N] = bf16_RNE( sum_k deq(A)[m,k] * deq(B)[n,k] )   (fp32 accumulation)
//
// The contraction is the block-scaled dot of the kernelindex.com
// amd-mxfp4-mm pages (tl.dot_scaled(..., "e2m1", ..., "e2m1"), submission
// 748756, kernel_fused_mxfp4_gemm) on v_mfma_scale_f32_32x32x64_f8f6f4; the
// activation is quantised by the rule of submission 755056, "Software MXFP4
// quant" (mx4_device.h).
//
// A workgroup owns 32 rows of C (one M block) and 32 NB WN columns over one K
// split of at most KR 64-K steps, with two kinds of waves:
//   - WN MFMA waves, each owning NB N blocks over the whole split: at launch
//     each issues the 128-bit non-temporal loads of all its weight fragments
//     and scale words (VGPRs), so the weight stream starts with the kernel
//     (issued right after the activation's: a CU returns its waves' loads
//     roughly in the order it takes them, and the activation must arrive
//     first); after the barrier it reads its activation fragments from LDS
//     and runs the MFMAs.  No two waves
//     share a K range, so there is no cross-wave reduction.
//   - QW quantiser waves, which share out the K steps of the workgroup's
//     activation slice (32 rows x the split's K): each loads its steps'
//     bf16 tiles straight into LDS (whole 128-byte row segments per 8
//     lanes), then every lane quantises one row's 32-element group of a step
//     in registers (amax, scale byte by the bit rule, e2m1 codes by the
//     gfx950 fp4 convert) and writes the MFMA fragment and scale byte into
//     LDS, once for all the MFMA waves; then they join the barrier.
// The two kinds of loads are issued by different waves, so neither waits
// for the other's (a wave's vector-memory counter runs in issue order).  The
// barrier between the two issues orders them and nothing else: it carries no
// memory fence, which would make every quantiser wave wait for its whole
// slice to land (buffer loads to LDS count as LDS writes) before any weight
// load could go out.  Each quantiser wave then waits for its own steps one at
// a time, and the slice barrier waits only for the quantisers' LDS writes, so
// the MFMA waves' weight loads stay in flight across it.
// Workgroups are grouped onto the XCDs (shared_xcd_map): the workgroups the
// dispatcher sends to one XCD (linear id mod 8) take a rectangle of a M tiles
// x b N tiles, chosen so that the activation rows and weight columns that
// one XCD's L2 must fetch are fewest.
// Rows past M are not loaded or read zeros through the buffer bound (zero
// codes, scale byte 0); steps past the split read zeros; a group past K
// (K % 64 == 32) is zeroed explicitly.  After the slice barrier the
// quantiser waves leave; each MFMA wave stages its own bf16 tile in the dead
// raw-tile region and stores it in 16-byte row chunks, with no barrier (a
// wave that finishes early stores early); with K split over workgroups,
// fp32 partials go to the workspace and reduce_kernel sums them in split
// order.
#include "mx4_device.h"
#include "mx4_internal.h"

namespace mx4 {

// LDS: the quantised activation slice, [KR][64 lanes][16 B] codes then the
// scale bytes as [KR / 4][64 lanes] words (byte b: step 4 w + b).
__host__ __device__ constexpr size_t shared_aop_bytes(int kr) { return (size_t)kr * 64 * 17; }
// then the raw bf16 tiles of the slice, one 4 KiB tile per K step; after the
// quantisation the MFMA waves stage their bf16 output tiles there
constexpr int kRawTile = kRowBlock * 128;
__host__ __device__ constexpr size_t shared_raw_offset(int kr) { return (shared_aop_bytes(kr) + 255) / 256 * 256; }
__host__ __device__ constexpr size_t shared_all_bytes(int kr) { return shared_raw_offset(kr) + (size_t)kr * kRawTile; }
__host__ __device__ constexpr int raw_slot(int r, int j) { return r * 128 + ((j ^ ((r >> 1) & 7)) << 4); }

// s_waitcnt for at most RQ m outstanding vector-memory operations (RQ loads
// per step, m later steps; m is a constant after unrolling, so the switch
// folds to one instruction).
template <int RQ>
__device__ __forceinline__ void wait_steps_left(int m) {
    switch (m) {
        case 0: wait_vmcnt<0>(); break;
        case 1: wait_vmcnt<RQ>(); break;
        case 2: wait_vmcnt<2 * RQ>(); break;
        case 3: wait_vmcnt<3 * RQ>(); break;
        case 4: wait_vmcnt<4 * RQ>(); break;
        case 5: wait_vmcnt<5 * RQ>(); break;
        case 6: wait_vmcnt<6 * RQ>(); break;
        case 7: wait_vmcnt<7 * RQ>(); break;
        case 8: wait_vmcnt<8 * RQ>(); break;
        case 9: wait_vmcnt<9 * RQ>(); break;
        case 10: wait_vmcnt<10 * RQ>(); break;
        case 11: wait_vmcnt<11 * RQ>(); break;
        default: wait_vmcnt<0>(); break;
    }
}

// A quantiser wave's share of the activation slice, rows 32 mt ..
// 32 mt + 8 RQ - 1 (RQ of the four 8-row chunks: those holding rows below
// M), split steps tb + s for s = qw, qw + QW, ... (KL of them): each step's
// 32 x 64 bf16 tile goes straight into LDS (gfx950 buffer loads to LDS, RQ
// loads of 1 KiB, 8 lanes per 128-byte row segment, 16-byte column j of row
// r at slot j ^ ((r >> 1) & 7)).  Steps past the split and a group past K
// (K % 64 == 32) read zeros; rows past M read zeros through the buffer
// bound.
template <int KL, int QW, int RQ>
__device__ __forceinline__ void shared_issue_activation(const Rsrc& ra, uint8_t* raw, int mt, int tb, int T, int G,
                                                        int lda, int qw, int L) {
    constexpr uint32_t kOutOfRange = 0x80000000u;
#pragma unroll
    for (int k = 0; k < KL; ++k) {
        const int s = qw + QW * k;
#pragma unroll
        for (int c4 = 0; c4 < RQ; ++c4) {
            const int c = c4 * 64 + L;
            const int r = c >> 3;
            const int j = (c & 7) ^ ((r >> 1) & 7);
            const bool live = s < T && 2 * (tb + s) + (j >> 2) < G;
            const uint32_t off = (uint32_t)(mt * kRowBlock + r) * (uint32_t)lda * 2u + (uint32_t)(tb + s) * 128u +
                                 (uint32_t)j * 16u;
            bload16_lds(ra, raw + (size_t)s * kRawTile + c4 * 1024, live ? off : kOutOfRange);
        }
    }
    asm volatile("" ::: "memory");
}

// The same wave's quantisation: step k has landed once at most the RQ loads
// of each of its KL - 1 - k later steps are outstanding (its only
// vector-memory operations are those loads, and they complete in issue
// order); lane L quantises row L % 32, group L / 32 of the step in registers
// and writes the MFMA fragment (16 bytes) and the scale byte into byte s % 4
// of its word.  Steps past the split quantise zeros (zero codes, scale byte
// 0), and so do the rows of chunks not loaded.
template <int KL, int QW, int RQ>
__device__ __forceinline__ void shared_quantise(const uint8_t* raw, uint8_t* aop, uint8_t* asc, int qw, int L) {
    const bool row_loaded = RQ == 4 || (L & 31) < 8 * RQ;
#pragma unroll
    for (int k = 0; k < KL; ++k) {
        wait_steps_left<RQ>(KL - 1 - k);
        asm volatile("" ::: "memory");
        const int s = qw + QW * k;
        const uint8_t* tile = raw + (size_t)s * kRawTile;
        u32x4 x[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) x[c] = *(const u32x4*)(tile + raw_slot(L & 31, 4 * (L >> 5) + c));
        u32x4 codes;
        uint32_t byte = quant_group32(x, codes);
        if (!row_loaded) {
            codes = u32x4{0u, 0u, 0u, 0u};
            byte = 0u;
        }
        *(u32x4*)(aop + 16 * (s * 64 + L)) = codes;
        asc[((s >> 2) * 64 + L) * 4 + (s & 3)] = (uint8_t)byte;
    }
}

// steps_arg: the steps per K split (at most 24) in bits 0..7, and above them
// the code that places the workgroups' tiles on the XCDs (shared_xcd_map,
// shared_tile_of; 0: tile (blockIdx.y, blockIdx.x)).
template <int NB, int WN, int QW, int KR>
__global__ void __launch_bounds__(64 * (WN + QW))
gemm_shared_kernel(const void* a_src, const uint8_t* bp, uint16_t* C, float* partial_buf, int lda, int ldc, int M,
                   int N, int K, int steps_arg, uint32_t* counters, int splits, int mtiles) {
    (void)counters;
    (void)splits;
    (void)mtiles;
    const int steps_per_split = steps_arg & 0xFF;
    const int xcd_map = steps_arg >> 8;
    constexpr uint32_t kOutOfRange = 0x80000000u;
    const OperandGeom gb = operand_geom(N, K);
    const int KS = gb.KS, KW = gb.KW, RBn = gb.RB;
    const int G = K / kGroup;
    const uint16_t* A = (const uint16_t*)a_src;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    uint8_t* aop = lds;                             // codes, KR * 1 KiB
    uint8_t* asc = lds + (size_t)KR * 1024;         // scale bytes, KR * 64
    uint8_t* raw = lds + shared_raw_offset(KR);      // bf16 tiles, KR * 4 KiB
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int L = tid & 63;

    int mt, nt;
    shared_tile_of((int)blockIdx.x, (int)blockIdx.y, (RBn + WN * NB - 1) / (WN * NB), (M + 31) / 32, xcd_map, mt, nt);
    const int split = blockIdx.z;
    const int tb = split * steps_per_split;
    const int te = min(tb + steps_per_split, KS);
    const int T = te - tb;                          // steps of this split, <= KR
    const bool mfma_wave = wave < WN;
    const int nb0 = (nt * WN + wave) * NB;          // first N block of an MFMA wave

    f32x16 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;

    u32x4 bfrag[KR][NB];
    uint32_t bscale[KR / 4][NB];   // one word per 4 steps (byte b: step 4 w + b when tb % 4 == 0)
    // The activation loads go out before the weight's: a CU returns the loads
    // of its waves roughly in the order it takes them, and the activation
    // (L2-resident) must arrive early for the quantisers, while the weight
    // (HBM) is consumed last.  Quantiser wave qw (0 .. QW - 1) takes the K
    // steps qw, qw + QW, ... of the split.
    constexpr int KL = KR / QW;                      // steps per quantiser wave
    static_assert(KR % QW == 0, "whole steps per quantiser wave");
    static_assert(KL <= 12, "wait_steps_left covers 12 steps per quantiser wave");
    const int qw = wave - WN;
    // The 8-row chunks of this M tile that hold rows below M: 1, 2 or all
    // four (three load all four; the fourth reads zeros through the buffer
    // bound).  The code for each count is straight-line: a branch between
    // the loads would break up their issue.
    const int rows_here = M - mt * kRowBlock;
    const int rq = rows_here > 16 ? 4 : rows_here > 8 ? 2 : 1;
    if (!mfma_wave) {
        const Rsrc ra = make_rsrc(A, (uint32_t)M * (uint32_t)lda * 2u);
        if (rq == 4)
            shared_issue_activation<KL, QW, 4>(ra, raw, mt, tb, T, G, lda, qw, L);
        else if (rq == 2)
            shared_issue_activation<KL, QW, 2>(ra, raw, mt, tb, T, G, lda, qw, L);
        else
            shared_issue_activation<KL, QW, 1>(ra, raw, mt, tb, T, G, lda, qw, L);
    }
    __builtin_amdgcn_s_barrier();   // the activation loads are issued (no fence: see the top)
    if (mfma_wave) {
        // ---- the weight: every fragment and scale word of the split in flight
        // at once (steps past the split read zeros)
        const Rsrc rb = make_rsrc(bp, (uint32_t)gb.total_bytes);
#pragma unroll
        for (int s = 0; s < KR; ++s) {
            const bool on = s < T;
            const int t = on ? tb + s : 0;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const int nb = min(nb0 + j, RBn - 1);   // clamped blocks are never stored
                bfrag[s][j] = bload16<kNonTemporal>(rb, on ? (uint32_t)L * 16u : kOutOfRange,
                                                    (uint32_t)(nb * KS + t) * 1024u);
            }
            // the scale word of steps tb + s .. tb + s + 3 (splits start at
            // multiples of 4 steps, so these share one packed word)
            if (s % 4 == 0) {
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int nb = min(nb0 + j, RBn - 1);
                    bscale[s / 4][j] = bload4(rb, on ? (uint32_t)L * 4u : kOutOfRange,
                                              (uint32_t)gb.code_bytes + (uint32_t)(nb * KW + (t >> 2)) * 256u);
                }
            }
        }
    }
    if (!mfma_wave) {
        if (rq == 4)
            shared_quantise<KL, QW, 4>(raw, aop, asc, qw, L);
        else if (rq == 2)
            shared_quantise<KL, QW, 2>(raw, aop, asc, qw, L);
        else
            shared_quantise<KL, QW, 1>(raw, aop, asc, qw, L);
    }
    // The quantised slice is in LDS: each wave's LDS writes have completed
    // before the barrier.  No vector-memory wait: the MFMA waves' weight
    // loads stay in flight, and each MFMA waits for its own fragment.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (!mfma_wave) return;   // the quantisers are done; no barrier follows
    {
        uint32_t aw = 0;
#pragma unroll
        for (int s = 0; s < KR; ++s) {
            const u32x4 af = *(const u32x4*)(aop + 16 * (s * 64 + L));
            if (s % 4 == 0) aw = *(const uint32_t*)(asc + ((s >> 2) * 64 + L) * 4);
            const int sh = 8 * (s & 3);              // byte of step tb + s in both scale words
#pragma unroll
            for (int j = 0; j < NB; ++j)
                acc[j] = mfma_fp4_32x32x64(bfrag[s][j], af, acc[j], bscale[s / 4][j] >> sh, aw >> sh);
        }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) mfma_result_fence(acc[j]);

    // ---- epilogue, each MFMA wave on its own: lane L, element e of block j:
    // m = 32 mt + L % 32, n = 32 (nb0 + j) + 8 (e / 4) + 4 (L / 32) + e % 4.
    const int m_lane = L & 31;
    const int n_lane = 4 * (L >> 5);
    if (partial_buf != nullptr) {   // K split: fp32 partials, summed by reduce_kernel
        const int ldp = RBn * kRowBlock;
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const f32x4 v = {acc[j][4 * r], acc[j][4 * r + 1], acc[j][4 * r + 2], acc[j][4 * r + 3]};
                const int m = mt * kRowBlock + m_lane;
                const int nb = nb0 + j;
                if (m < M && nb < RBn)
                    *(f32x4*)(partial_buf + ((size_t)split * M + m) * ldp + nb * kRowBlock + 8 * r + n_lane) = v;
            }
        return;
    }
    // The wave's bf16 tile (32 rows x 32 NB columns) goes through its own
    // stage in the raw-tile region, dead since the slice barrier, and leaves
    // in 16-byte row chunks: no barrier, so each wave stores as soon as its
    // MFMAs are done (a wave reads its own LDS writes in order).
    constexpr int WC = NB * kRowBlock;
    constexpr int WROW = WC + 8;   // bf16 per staged row (16-byte pad)
    static_assert((size_t)WN * kRowBlock * WROW * 2 <= (size_t)KR * kRawTile, "stages fit the raw-tile region");
    uint16_t* wst = (uint16_t*)(raw + (size_t)wave * kRowBlock * WROW * 2);
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            uint2 w;
            w.x = pack_bf16x2(acc[j][4 * r], acc[j][4 * r + 1]);
            w.y = pack_bf16x2(acc[j][4 * r + 2], acc[j][4 * r + 3]);
            *(uint2*)(wst + m_lane * WROW + j * kRowBlock + 8 * r + n_lane) = w;
        }
    const int m_base = mt * kRowBlock;
    const int n_base = nb0 * kRowBlock;
    const bool vec16 = ((uintptr_t)C % 16 == 0) && (ldc % 8 == 0);
#pragma unroll
    for (int c = L; c < kRowBlock * WC / 8; c += 64) {
        const int row = c / (WC / 8), c8 = c % (WC / 8);
        const int m = m_base + row, n = n_base + 8 * c8;
        if (m >= M || n >= N) continue;
        const u32x4 v = *(const u32x4*)(wst + row * WROW + 8 * c8);
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
}

// ---------------------------------------------------------------------------
// Instantiations: (NB, WN, QW) in {(1, 2, 2), (1, 3, 4), (1, 3, 8), (1, 4, 4),
// (1, 4, 8), (2, 2, 2), (2, 4, 4)} and KR in {8, 16, 24} (24 with NB = 1).

// The weight registers bound NB * KR (<= 24 fragments per MFMA wave) and LDS
// the slice (KR 4 KiB raw tiles plus the quantised operand: KR <= 24).
template <int NB, int WN, int QW>
static GemmKernelFn shared_pick_kr(int kr) {
    switch (kr) {
        case 8: return gemm_shared_kernel<NB, WN, QW, 8>;
        case 16: return gemm_shared_kernel<NB, WN, QW, 16>;
        case 24: return NB == 1 ? gemm_shared_kernel<1, WN, QW, 24> : nullptr;
        default: return nullptr;
    }
}

int shared_kr_for(int steps) {
    static const int kBudgets[] = {8, 16, 24};
    for (int kr : kBudgets)
        if (steps <= kr) return kr;
    return 0;
}

// Plan fields of this mode: nb N blocks per MFMA wave, wn MFMA waves, wk
// quantiser waves (mb = 1).
GemmKernelFn find_shared_kernel(const Plan& plan, int steps_per_split) {
    if (plan.mb != 1) return nullptr;
    const int kr = shared_kr_for(steps_per_split);
    if (plan.nb == 1 && plan.wn == 2 && plan.wk == 2) return shared_pick_kr<1, 2, 2>(kr);
    if (plan.nb == 1 && plan.wn == 3 && plan.wk == 4) return shared_pick_kr<1, 3, 4>(kr);
    if (plan.nb == 1 && plan.wn == 3 && plan.wk == 8) return shared_pick_kr<1, 3, 8>(kr);
    if (plan.nb == 1 && plan.wn == 4 && plan.wk == 8) return shared_pick_kr<1, 4, 8>(kr);
    if (plan.nb == 1 && plan.wn == 4 && plan.wk == 4) return shared_pick_kr<1, 4, 4>(kr);
    if (plan.nb == 2 && plan.wn == 2 && plan.wk == 2) return shared_pick_kr<2, 2, 2>(kr);
    if (plan.nb == 2 && plan.wn == 4 && plan.wk == 4) return shared_pick_kr<2, 4, 4>(kr);
    return nullptr;
}

size_t shared_lds_bytes(const Plan& plan, int steps_per_split) {
    (void)plan;
    return shared_all_bytes(shared_kr_for(steps_per_split));
}

}  // namespace mx4
