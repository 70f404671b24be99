// mx4_tile.hip -- K-looped, LDS-pipelined block-scaled MXFP4 GEMM for gfx950
// (MI355X) at large M: the activation mode MX_AMODE_TILE.
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
// C over the whole of K and walks K one 64-K step at a time.  Each step's
// operand tiles (MB of A, NB of B) and their scale words go straight from
// memory into a ring of S LDS stages (gfx950 buffer loads to LDS, issued S
// steps ahead); its WM x WN waves each read the fragments of their TM x TN
// blocks (TM = MB / WM, TN = NB / WN) from the stage one step ahead, into
// registers, and run TM x TN MFMAs, so every operand tile feeds several
// MFMAs from LDS and a wave's LDS reads overlap its MFMAs.  Every wave issues the
// same number of loads per step (steps past K load from an offset past the
// buffer and read zeros), so the wait for a step is a compile-time count.
// One barrier per step, with no memory fence (a fence would wait for the
// loads of the steps in flight), tells the waves that every wave's loads of
// the step have landed and that the stage of the previous step is free.
// The epilogue stages each wave's bf16 tiles in the (then dead) ring and
// stores them in 16-byte row chunks.
#include "mx4_device.h"
#include "mx4_internal.h"

namespace mx4 {

constexpr int kTileOpBytes = 1024;   // one packed operand tile: 64 lanes x 16 B
constexpr int kTileWordBytes = 256;  // one packed scale word group: 64 lanes x 4 B

__host__ __device__ constexpr size_t tile_stage_bytes(int mb, int nb) {
    return (size_t)(mb + nb) * (kTileOpBytes + kTileWordBytes);
}

// 4-byte buffer load straight into LDS: lane L's dword lands at lds_base + 4 L.
__device__ __forceinline__ void bload4_lds(Rsrc r, uint8_t* lds_base, uint32_t voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 4, (int)voff, 0, 0,
                                             0);
}

template <int MB, int NB, int WM, int WN, int S>
__global__ void __launch_bounds__(64 * WM * WN)
gemm_tile_kernel(const void* a_src, const uint8_t* bp, uint16_t* C, float* partial_buf, int lda, int ldc, int M,
                 int N, int K, int steps_arg, uint32_t* counters, int splits, int mtiles) {
    (void)partial_buf;
    (void)lda;
    (void)counters;
    (void)splits;
    (void)mtiles;
    constexpr int TM = MB / WM, TN = NB / WN, NW = WM * WN;
    constexpr int OPS = MB + NB;   // operand blocks per step
    static_assert(MB % WM == 0 && NB % WN == 0 && OPS % NW == 0, "whole blocks per wave");
    constexpr int LPW = OPS / NW;  // blocks each wave loads per step (a tile and a word each)
    constexpr int STAGE = (int)tile_stage_bytes(MB, NB);
    constexpr uint32_t kOutOfRange = 0x80000000u;
    static_assert(2 * LPW * (S - 1) < 64, "vmcnt range");

    const OperandGeom ga = operand_geom(M, K), gb = operand_geom(N, K);
    const int KS = gb.KS, KW = gb.KW;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int L = tid & 63;
    const int wm = wave / WN, wn = wave % WN;
    // the tile of this workgroup, placed on the XCDs by the placement code
    // the host passes as steps_arg (shared_tile_of; K's steps come from K)
    int mt, nt;
    shared_tile_of((int)blockIdx.x, (int)blockIdx.y, (gb.RB + NB - 1) / NB, steps_arg, mt, nt);
    const int rbm0 = mt * MB, rbn0 = nt * NB;
    const Rsrc ra = make_rsrc(a_src, (uint32_t)ga.total_bytes);
    const Rsrc rbr = make_rsrc(bp, (uint32_t)gb.total_bytes);

    // The loads of step t into the stage at `st`: wave w takes blocks
    // q = w LPW .. w LPW + LPW - 1 of the step, q < MB being A block rbm0 + q
    // and the rest B block rbn0 + q - MB: the 1 KiB tile (rb, t) and the
    // scale word group (rb, t / 4).  Blocks past the operand and steps past K
    // read zeros.
    auto issue = [&](int t, uint8_t* st) {
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int q = wave * LPW + i;
            const bool is_a = q < MB;
            const int rb = is_a ? rbm0 + q : rbn0 + (q - MB);
            const bool live = t < KS && rb < (is_a ? ga.RB : gb.RB);
            const uint32_t code_bytes = (uint32_t)(is_a ? ga.code_bytes : gb.code_bytes);
            const uint32_t toff = live ? ((uint32_t)(rb * KS + t) * 64u + (uint32_t)L) * 16u : kOutOfRange;
            const uint32_t woff =
                live ? code_bytes + ((uint32_t)(rb * KW + (t >> 2)) * 64u + (uint32_t)L) * 4u : kOutOfRange;
            bload16_lds(is_a ? ra : rbr, st + q * kTileOpBytes, toff);
            bload4_lds(is_a ? ra : rbr, st + OPS * kTileOpBytes + q * kTileWordBytes, woff);
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // this wave's fragments of one step: TM A tiles and TN B tiles (16 bytes
    // a lane) and their scale words
    struct Frags {
        u32x4 a[TM], b[TN];
        uint32_t as[TM], bs[TN];
    };
    auto read_frags = [&](const uint8_t* st, Frags& f) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            f.a[i] = *(const u32x4*)(st + (wm * TM + i) * kTileOpBytes + 16 * L);
            f.as[i] = *(const uint32_t*)(st + OPS * kTileOpBytes + (wm * TM + i) * kTileWordBytes + 4 * L);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            f.b[j] = *(const u32x4*)(st + (MB + wn * TN + j) * kTileOpBytes + 16 * L);
            f.bs[j] = *(const uint32_t*)(st + OPS * kTileOpBytes + (MB + wn * TN + j) * kTileWordBytes + 4 * L);
        }
    };

    // The ring holds S steps in flight.  Step t's fragments are read into
    // registers one step ahead, so a wave's LDS reads of step t + 1 overlap
    // its MFMAs of step t; the barrier before them tells every wave that the
    // loads of step t + 1 have landed everywhere and that every wave has
    // read step t (its LDS reads completed), whose stage then takes step
    // t + S.
#pragma unroll
    for (int t = 0; t < S; ++t) issue(t, lds + (size_t)t * STAGE);
    wait_vmcnt<2 * LPW * (S - 1)>();   // step 0 has landed for this wave
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    Frags cur, nxt;
    read_frags(lds, cur);
    int st_t = 0;   // stage of step t
    for (int t = 0; t < KS; ++t) {
        const int st_n = st_t == S - 1 ? 0 : st_t + 1;   // stage of step t + 1
        // step t + 1 has landed for this wave once at most the loads of
        // steps t + 2 .. t + S - 1 are outstanding (a wave's loads complete
        // in issue order)
        wait_vmcnt<2 * LPW * (S - 2)>();
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        issue(t + S, lds + (size_t)st_t * STAGE);
        read_frags(lds + (size_t)st_n * STAGE, nxt);
        const int sh = 8 * (t & 3);   // byte of step t in the scale words
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = mfma_fp4_32x32x64(cur.b[j], cur.a[i], acc[i][j], cur.bs[j] >> sh, cur.as[i] >> sh);
        cur = nxt;
        st_t = st_n;
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
    constexpr int WC = TN * kRowBlock;   // columns of a wave's row of blocks
    constexpr int WROW = WC + 8;          // bf16 per staged row (16-byte pad)
    static_assert((size_t)NW * kRowBlock * WROW * 2 <= (size_t)S * STAGE, "stages fit the ring");
    uint16_t* wst = (uint16_t*)(lds + (size_t)wave * kRowBlock * WROW * 2);
    const int m_lane = L & 31;
    const int n_lane = 4 * (L >> 5);
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
#pragma unroll
        for (int c = L; c < kRowBlock * WC / 8; c += 64) {
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

constexpr int kTileStages = 6;

GemmKernelFn find_tile_kernel(const Plan& plan) {
    if (plan.mb == 8 && plan.nb == 8 && plan.wk == 2 && plan.wn == 4)
        return gemm_tile_kernel<8, 8, 2, 4, kTileStages>;
    if (plan.mb == 4 && plan.nb == 8 && plan.wk == 2 && plan.wn == 2)
        return gemm_tile_kernel<4, 8, 2, 2, kTileStages>;
    if (plan.mb == 8 && plan.nb == 4 && plan.wk == 2 && plan.wn == 2)
        return gemm_tile_kernel<8, 4, 2, 2, kTileStages>;
    return nullptr;
}

size_t tile_lds_bytes(const Plan& plan) { return (size_t)kTileStages * tile_stage_bytes(plan.mb, plan.nb); }

}  // namespace mx4
