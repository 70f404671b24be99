// mx4_gemm.hip -- block-scaled MXFP4 GEMM for gfx950 (MI355X).
//
//   C[M,N] = bf16_RNE( sum_k deq(A)[m,k] * deq(B)[n,k] )   (fp32 accumulation)
//
// The contraction is what the kernelindex.com amd-mxfp4-mm pages write as
// tl.dot_scaled(a, a_scale, "e2m1", b, b_scale, "e2m1") (e.g. submission
// 748756, kernel_fused_mxfp4_gemm); here it runs directly on
// v_mfma_scale_f32_32x32x64_f8f6f4, whose per-lane e8m0 byte scales that
// lane's 32-element group by 2^(byte-127).
//
// Workgroup = WN x WK waves; a wave owns (32 MBLK) m x (32 NBLK) n outputs,
// the WN waves of a workgroup sit side by side along N and the WK waves
// share the K steps of the workgroup's K split.
//   1. Every wave issues the 128-bit loads of all its weight fragments (its
//      whole share of the split) before anything else: the weight costs one
//      HBM round trip, read exactly once, straight into VGPRs, non-temporal.
//   2. The activation operand, by the plan's activation mode AM:
//      kAmLds     the workgroup quantises its activation slice (its m rows x
//                 its K split) itself into LDS, in MFMA lane order: rows
//                 streamed 1 KB per load instruction, one DPP quad of lanes
//                 per 32-element group (amax across the quad, scale byte by
//                 the bit rule, e2m1 codes by the gfx950 fp4 convert); the
//                 WN waves of the workgroup share it after a barrier;
//      kAmPrequant a first kernel (pack_kernel) quantised A into the packed
//                 operand layout in the workspace; each wave loads its
//                 fragments from there (L2-resident) together with step 1;
//      kAmDirect  every wave loads the rows of exactly the fragments it
//                 feeds to its MFMAs, 128 bytes per 8 lanes, straight into
//                 its own LDS tiles (or through VGPRs into a padded slab when
//                 the tiles of all its K steps do not fit), reads them back
//                 so that each lane holds one row's 32-element group, and
//                 quantises that group in registers:
//                 no workgroup barrier before the MFMAs; waves with the same
//                 m rows and K steps each quantise them;
//      kAmBf16    the a16wfp4 product of the pages (submission 733989,
//                 routing notes): A is not quantised.  Lanes load A as in
//                 kAmDirect; the weight codes are widened to bf16 times
//                 their e8m0 scale by the gfx950 fp4 convert (exact) and
//                 the step runs as four bf16 MFMAs (32x32x16).
//   3. K loop: MFMAs on registers (and 16-byte LDS reads with kAmLds).
//   4. The WK waves add their accumulators through LDS; the result is
//      rounded to bf16, staged in LDS and stored in 16-byte row chunks.
//      When K is split over workgroups, each writes fp32 partials and
//      either reduce_kernel sums them in split order (a second launch), or
//      the last workgroup of a tile to arrive does (one launch): once every
//      wave has waited for its own partial stores to complete, its arrival
//      is counted by an agent-scope atomic on a per-tile counter, the
//      partials are written and read with agent-scope (L2-coherent across
//      XCDs) accesses, and that workgroup returns the counter to zero.
//      Either way the sum runs in split order, so results do not depend on
//      timing.
#include "mx4_device.h"
#include "mx4_internal.h"

namespace mx4 {

// The grid is (N tiles, M tiles, K splits), so the tile indices come straight
// from the workgroup-id SGPRs, with no division.  Workgroups are dispatched
// round-robin over the 8 XCDs by their linear index x + X (y + Y z): when the
// number of N tiles X is a multiple of 8, every M tile of one N tile runs on
// the same XCD, and the M tiles that read the same weight tile share one L2.

// The activation of kAmDirect / kAmBf16 arrives coalesced: each wave loads its
// 32-row x 64-K bf16 tiles a whole 128-byte row segment per 8 lanes into a
// per-wave LDS slab (rows padded to 144 bytes), then every lane reads back
// the 64 bytes of the fragment it quantises.  One wave writes and reads its
// own slab, so LDS ordering within the wave is all the synchronisation; the
// slab holds two K steps at a time and is reused for the next two.  The slabs
// share LDS with the epilogue's buffers, behind a barrier.
constexpr int kSlabRow = 144;
__host__ __device__ constexpr int slab_steps(int kr) { return kr < 2 ? kr : 2; }
__host__ __device__ constexpr size_t gemm_slab_bytes(int waves, int mb, int kr) {
    return (size_t)waves * mb * slab_steps(kr) * kRowBlock * kSlabRow;
}

// When all of a workgroup's K steps fit in LDS at once (waves x MBLK x KR
// tiles of 4 KiB), the coalesced loads skip the VGPRs: each goes straight
// into the wave's LDS tile of its (K step, m block) (gfx950 buffer loads to
// LDS, 16 bytes per lane).  A tile is 32 rows x 128 bytes with 16-byte column
// j of row r at slot j ^ ((r >> 1) & 7): the 16 lanes of each fragment read
// then hit 16 distinct 16-byte bank groups, and each lane still chooses its
// global chunk, so 8 lanes still read one 128-byte row segment.
constexpr int kDmaTile = kRowBlock * 128;
__host__ __device__ constexpr bool gemm_uses_dma(int waves, int mb, int kr) {
    return (size_t)waves * mb * kr * kDmaTile <= kLdsBudget;
}
__host__ __device__ constexpr size_t gemm_dma_bytes(int waves, int mb, int kr) {
    return (size_t)waves * mb * kr * kDmaTile;
}
__host__ __device__ constexpr int dma_slot(int r, int j) { return r * 128 + ((j ^ ((r >> 1) & 7)) << 4); }

// LDS of the WK-reduction buffer and of the staged bf16 output tile.
// The reduction buffer is lane-major: each lane's mb * nb * 16 accumulators
// contiguous, padded by 16 bytes (16-byte writes and reads without bank
// conflicts).
__host__ __device__ constexpr int red_lane_bytes(int mb, int nb) { return mb * nb * 16 * 4 + 16; }
__host__ __device__ constexpr size_t gemm_red_bytes(int wn, int wk, int mb, int nb) {
    return wk > 1 ? (size_t)wn * wk * 64 * red_lane_bytes(mb, nb) : 0;
}
__host__ __device__ constexpr size_t gemm_stage_bytes(int wn, int mb, int nb) {
    return (size_t)mb * kRowBlock * (nb * wn * kRowBlock + 8) * 2;
}

// Four fp32 partials as two 64-bit agent-scope atomic accesses: coherent
// across the XCDs' L2s without a cache-wide write-back or invalidate.
__device__ __forceinline__ void store_partial_agent(float* dst, const float (&v)[4]) {
    const uint64_t lo = (uint64_t)__float_as_uint(v[0]) | ((uint64_t)__float_as_uint(v[1]) << 32);
    const uint64_t hi = (uint64_t)__float_as_uint(v[2]) | ((uint64_t)__float_as_uint(v[3]) << 32);
    __hip_atomic_store((uint64_t*)dst, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store((uint64_t*)dst + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4 load_partial_agent(const float* src) {
    const uint64_t lo = __hip_atomic_load((const uint64_t*)src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load((const uint64_t*)src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return f32x4{__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                 __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32))};
}

// 4 consecutive bf16 outputs (n0..n0+3) of row m, masked at N.  C is written
// once and never read back here, so its stores are non-temporal: they do not
// leave dirty lines in L2 for the end of the kernel to write back.
__device__ __forceinline__ void store_bf16x4(uint16_t* C, int ldc, int N, bool c_vec, int m, int n0,
                                             const float (&v)[4]) {
    uint16_t* dst = C + (size_t)m * ldc + n0;
    if (c_vec && n0 + 3 < N) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        __builtin_nontemporal_store(w, (u32x2*)dst);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (n0 + q < N) dst[q] = (uint16_t)bf16_rne(v[q]);
    }
}

// The leading scalar arguments arrive preloaded in SGPRs (GemmKernelFn); the
// kernel derives both operands' layouts from them with the host's own
// operand_geom.  The last three (counters, splits, mtiles) are read only by
// the last-arrival split-K finish.
// RQ (kAmDirect / kAmBf16 with one 32-row block): how many 8-row chunks of
// the block each K step loads; rows from 8 RQ on are past M, feed only
// outputs that are never stored, and are not loaded (for M <= 8 or <= 16 a
// fourth or a half of the activation traffic).
template <int MBLK, int NBLK, int WN, int WK, int AM, int KR, int RQ>
__global__ void __launch_bounds__(64 * WN * WK) __attribute__((amdgpu_waves_per_eu(2)))
gemm_kernel(const void* a_src, const uint8_t* bp, uint16_t* C, float* partial_buf, int lda, int ldc, int M, int N,
            int K, int steps_per_split, uint32_t* counters, int splits, int mtiles) {
    GemmParams p = {};
    {
        const OperandGeom ga = operand_geom(M, K), gb = operand_geom(N, K);
        if constexpr (AM == kAmPrequant) {
            p.aop = (const uint8_t*)a_src;
            p.aop_bytes = (uint32_t)ga.total_bytes;
            p.a_code_bytes = (uint32_t)ga.code_bytes;
        } else {
            p.A = (const uint16_t*)a_src;
            p.a_bytes = (uint32_t)M * (uint32_t)lda * 2u;
        }
        p.bp = bp;
        p.bp_bytes = (uint32_t)gb.total_bytes;
        p.b_code_bytes = (uint32_t)gb.code_bytes;
        p.C = C;
        p.partial = partial_buf;
        p.lda = lda;
        p.ldc = ldc;
        p.M = M;
        p.N = N;
        p.K = K;
        p.KS = gb.KS;
        p.KW = gb.KW;
        p.RBm = ga.RB;
        p.RBn = gb.RB;
        p.ldp = gb.RB * kRowBlock;
        p.steps_per_split = steps_per_split;
        p.counters = counters;
        p.splits = splits;
        p.mtiles = mtiles;
    }
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    constexpr bool FUSED = AM == kAmLds;
    constexpr bool DIRECT = AM == kAmDirect;
    constexpr bool PREQ = AM == kAmPrequant;
    constexpr bool BF16A = AM == kAmBf16;
    constexpr bool REGA = DIRECT || BF16A;   // activation loaded straight into registers
    constexpr int NT = 64 * WN * WK;
    const int tid = threadIdx.x;
    // wave-uniform values in SGPRs: weight and operand base addresses then
    // stay scalar and each load needs one 32-bit lane offset
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int L = tid & 63;
    const int wn = wave % WN;
    const int wkk = wave / WN;

    // ---- tile of this workgroup
    const int nt = blockIdx.x;
    const int mt = blockIdx.y;
    const int split = blockIdx.z;
    const int mb0 = mt * MBLK;
    const int nb0 = (nt * WN + wn) * NBLK;   // first n block of this wave
    const int tb = split * p.steps_per_split;
    const int te = min(tb + p.steps_per_split, p.KS);
    const int T = te - tb;
    const int per_wave = (T + WK - 1) / WK;
    const int wb = tb + wkk * per_wave;
    const int nsteps = max(min(wb + per_wave, te) - wb, 0);   // <= KR by the planner
    // Steps s >= nsteps are padding: their loads get a lane offset past every
    // buffer's end and read zeros, so the load and MFMA sequences below are
    // the same straight-line code for every wave.
    constexpr uint32_t kOutOfRange = 0x80000000u;

    // ---- 1. operand loads.  kAmLds: the workgroup streams its activation
    // slice (rows 32 mb0 .. 32 (mb0 + MBLK) - 1, K steps tb .. te - 1) a row
    // at a time: wave w takes slice rows w, w + NW, ..., lane l the 16-byte
    // chunks l, l + 64, ... of the row (8 chunks per K step), so each load
    // instruction reads 1 KB of a row.  A DPP quad holds one 32-element group;
    // each lane writes its 8 codes as dword q of the group's slot
    // (i T + t) 64 + row % 32 + 32 (group % 2) of the LDS operand (MFMA lane
    // order), the quad's first lane the scale byte.  The first batch of rows
    // is loaded before the weight: loads complete in issue order, so the
    // quantisation starts while the weight is still in flight.  Rows past M
    // read as zero through the buffer bound (zero codes, scale byte 0); a
    // group past K (K % 64 == 32) is zeroed explicitly.
    const int slots = MBLK * T * 64;
    const int G = p.K / kGroup;
    constexpr int NW = NT / 64;                       // waves of the workgroup
    constexpr int RPW = MBLK * kRowBlock / NW;        // slice rows per wave
    constexpr int CPLM = (WK * KR + 7) / 8;           // most 16-byte chunks per lane per row
    constexpr int BR = (16 / CPLM) < 1 ? 1 : ((16 / CPLM) < RPW ? 16 / CPLM : RPW);   // rows per batch
    const int cpr = 8 * T;                            // 16-byte chunks per slice row
    u32x4 xs[FUSED ? BR : 1][FUSED ? CPLM : 1];
    auto slice_load = [&](int j0) {                   // rows j0 .. j0 + BR - 1 of this wave
        const Rsrc rx_ = make_rsrc(p.A, p.a_bytes);
#pragma unroll
        for (int b = 0; b < BR; ++b) {
            const int sr = wave + NW * (j0 + b);
            const int row = (mb0 + sr / kRowBlock) * kRowBlock + sr % kRowBlock;
            const uint32_t rowoff = (uint32_t)row * (uint32_t)p.lda * 2u + (uint32_t)tb * 128u;
#pragma unroll
            for (int k = 0; k < CPLM; ++k) {
                const int kc = 64 * k + L;
                const bool live = j0 + b < RPW && kc < cpr && 2 * tb + (kc >> 2) < G;
                xs[b][k] = bload16(rx_, live ? rowoff + (uint32_t)kc * 16u : kOutOfRange, 0u);
            }
        }
    };
    auto slice_quant = [&](int j0) {
#pragma unroll
        for (int b = 0; b < BR; ++b) {
            if (j0 + b >= RPW) break;
            const int sr = wave + NW * (j0 + b);
            const int i = sr / kRowBlock, r = sr % kRowBlock;
#pragma unroll
            for (int k = 0; k < CPLM; ++k) {
                const int kc = 64 * k + L;
                if (64 * k >= cpr) break;             // no chunk of this lane group left
                if (kc < cpr) {                       // whole quads (cpr % 8 == 0)
                    uint32_t byte;
                    const uint32_t codes = quad_quant8(xs[b][k], byte);
                    const int t = kc >> 3, h = (kc >> 2) & 1, q = kc & 3;
                    const int u = (i * T + t) * 64 + r + 32 * h;
                    *(uint32_t*)(lds + 16 * u + 4 * q) = codes;
                    if (q == 0) lds[16 * slots + u] = (uint8_t)byte;
                }
            }
        }
    };
    if constexpr (FUSED) slice_load(0);

    // kAmDirect: lane L's fragment of step s, m block i is row
    // 32 (mb0 + i) + L % 32, group 2 (wb + s) + L / 32; padding steps and a
    // group past K read zeros (zero codes, scale byte 0), rows past M read
    // zeros through the buffer bound.
    u32x4 xa[REGA ? KR : 1][MBLK][4];
    constexpr bool DMA = REGA && gemm_uses_dma(NT / 64, MBLK, KR);
    uint8_t* dtile = lds + (size_t)wave * (MBLK * KR * kDmaTile);   // this wave's tiles (DMA)
    if constexpr (REGA) {
        // coalesced: chunk q of lane L is row (64 q + L) / 8 of the tile,
        // 16-byte column (64 q + L) % 8 of its 128-byte K segment -- with
        // DMA, the column whose swizzled slot is (64 q + L) % 8
        const Rsrc rx_ = make_rsrc(p.A, p.a_bytes);
#pragma unroll
        for (int s = 0; s < KR; ++s) {
#pragma unroll
            for (int i = 0; i < MBLK; ++i) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (q >= RQ) {   // rows 8q .. 8q + 7 are past M (resolved at compile time)
                        if constexpr (!DMA) xa[s][i][q] = u32x4{0u, 0u, 0u, 0u};
                        continue;
                    }
                    const int c = q * 64 + L;
                    const int r = c >> 3;
                    const int col = DMA ? (c & 7) ^ ((r >> 1) & 7) : (c & 7);
                    const int g = 2 * (wb + s) + (col >> 2);
                    const bool live = s < nsteps && g < G;
                    const int row = (mb0 + i) * kRowBlock + r;
                    const uint32_t off = live ? (uint32_t)row * (uint32_t)p.lda * 2u + (uint32_t)(wb + s) * 128u +
                                                    (uint32_t)col * 16u
                                              : kOutOfRange;
                    if constexpr (DMA)
                        bload16_lds(rx_, dtile + ((s * MBLK + i) * 4 + q) * 1024, off);
                    else
                        xa[s][i][q] = bload16(rx_, off, 0u);
                }
            }
        }
        // the weight loads below stay behind the DMA loads (vmcnt counts in
        // issue order; the wait before the tiles are read relies on it)
        if constexpr (DMA) asm volatile("" ::: "memory");
    }
    // With 8 or more waves, every wave's activation goes out before any
    // weight load: a CU returns its waves' loads roughly in the order it
    // takes them, so the activation of the last wave to issue no longer waits
    // behind the other waves' weight, and the quantisation overlaps the weight
    // stream (64x7168x2048: -0.09 us; with 4 waves the barrier costs more than
    // it saves).  A bare s_barrier: a fence would wait for the loads to LDS.
    if constexpr (DMA && NT >= 512) __builtin_amdgcn_s_barrier();

    // Weight (and pre-quantised activation) fragments, all in flight.
    // Buffer loads: the wave-uniform part of every offset is a scalar, the
    // lane part one VGPR; steps past the wave's share read as zero.
    const Rsrc rb_ = make_rsrc(p.bp, p.bp_bytes);
    const Rsrc ra_ = make_rsrc(p.aop, p.aop_bytes);
    u32x4 bfrag[KR][NBLK];
    uint32_t bscale[KR][NBLK];
    u32x4 afrag[PREQ ? KR : 1][MBLK];
    uint32_t ascale[PREQ ? KR : 1][MBLK];
#pragma unroll
    for (int s = 0; s < KR; ++s) {
        const bool on = s < nsteps;
        const int t = min(wb + s, p.KS - 1);
        const uint32_t vcode = on ? (uint32_t)L * 16u : kOutOfRange;
        const uint32_t vscale = on ? (uint32_t)L * 4u : kOutOfRange;
#pragma unroll
        for (int j = 0; j < NBLK; ++j) {
            const int nb = min(nb0 + j, p.RBn - 1);   // clamped blocks are never stored
            bfrag[s][j] = bload16<kNonTemporal>(rb_, vcode, (uint32_t)(nb * p.KS + t) * 1024u);
            bscale[s][j] = bload4(rb_, vscale, p.b_code_bytes + (uint32_t)(nb * p.KW + (t >> 2)) * 256u);
        }
        if constexpr (PREQ) {
#pragma unroll
            for (int i = 0; i < MBLK; ++i) {
                const int mb = min(mb0 + i, p.RBm - 1);   // clamped blocks are never stored
                afrag[s][i] = bload16(ra_, vcode, (uint32_t)(mb * p.KS + t) * 1024u);
                ascale[s][i] = bload4(ra_, vscale, p.a_code_bytes + (uint32_t)(mb * p.KW + (t >> 2)) * 256u);
            }
        }
    }

    // ---- 2. (FUSED) quantise the activation slice into LDS.
    if constexpr (FUSED) {
        slice_quant(0);
        for (int j0 = BR; j0 < RPW; j0 += BR) {
            slice_load(j0);
            slice_quant(j0);
        }
        __syncthreads();
    }

    // ---- 2b. (kAmDirect / kAmBf16) the coalesced activation chunks go through
    // this wave's LDS tiles or slab into fragment order: lane L then holds the
    // 64 bytes of row 32 (mb0 + i) + L % 32, group 2 (wb + s) + L / 32.
    if constexpr (DMA) {
        // every weight load is issued; wait until at most those are still
        // outstanding, i.e. every DMA load has landed
        asm volatile("" ::: "memory");
        wait_vmcnt<2 * KR * NBLK>();
#pragma unroll
        for (int s = 0; s < KR; ++s)
#pragma unroll
            for (int i = 0; i < MBLK; ++i)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    xa[s][i][c] = *(const u32x4*)(dtile + (s * MBLK + i) * kDmaTile +
                                                  dma_slot(L & 31, 4 * (L >> 5) + c));
    } else if constexpr (REGA) {
        constexpr int SR = slab_steps(KR);
        uint8_t* slab = lds + (size_t)wave * (MBLK * SR * kRowBlock * kSlabRow);
#pragma unroll
        for (int s0 = 0; s0 < KR; s0 += SR) {
#pragma unroll
            for (int ds = 0; ds < SR; ++ds)
#pragma unroll
                for (int i = 0; i < MBLK; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (s0 + ds >= KR) continue;   // odd KR: the last pass holds one step
                        const int c = q * 64 + L;
                        *(u32x4*)(slab + ((i * SR + ds) * kRowBlock + (c >> 3)) * kSlabRow + (c & 7) * 16) =
                            xa[s0 + ds][i][q];
                    }
#pragma unroll
            for (int ds = 0; ds < SR; ++ds)
#pragma unroll
                for (int i = 0; i < MBLK; ++i)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        if (s0 + ds >= KR) continue;
                        xa[s0 + ds][i][c] = *(const u32x4*)(slab + ((i * SR + ds) * kRowBlock + (L & 31)) * kSlabRow +
                                                            (L >> 5) * 64 + c * 16);
                    }
        }
    }

    // ---- 2c. (kAmDirect) quantise every step of the wave before the first
    // MFMA: the MFMA of a step waits for that step's weight fragment, and a
    // quantisation placed after it would wait too (-0.04 to -0.11 us).
    u32x4 afq[DIRECT ? KR : 1][MBLK];
    uint32_t asq[DIRECT ? KR : 1][MBLK];
    if constexpr (DIRECT) {
#pragma unroll
        for (int s = 0; s < KR; ++s)
#pragma unroll
            for (int i = 0; i < MBLK; ++i)
                asq[s][i] = quant_group32(xa[s][i], afq[s][i]);   // xa already in fragment order (see the slab pass)
    }

    // ---- 3. K loop over the wave's steps
    f32x16 acc[MBLK][NBLK];
#pragma unroll
    for (int i = 0; i < MBLK; ++i)
#pragma unroll
        for (int j = 0; j < NBLK; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
#pragma unroll
    for (int s = 0; s < KR; ++s) {
        const int t = wb + s;
        const int sh = 8 * (t & 3);
        u32x4 af[MBLK];
        uint32_t as[MBLK];
#pragma unroll
        for (int i = 0; i < MBLK; ++i) {
            if constexpr (FUSED) {
                const bool on = s < nsteps;
                const int u = (i * T + min(t - tb, T - 1)) * 64 + L;
                const u32x4 a = *(const u32x4*)(lds + 16 * u);
                af[i] = on ? a : u32x4{0u, 0u, 0u, 0u};
                as[i] = lds[16 * MBLK * T * 64 + u];
            } else if constexpr (DIRECT) {
                af[i] = afq[s][i];
                as[i] = asq[s][i];
            } else if constexpr (BF16A) {
                af[i] = u32x4{0u, 0u, 0u, 0u};   // unused: the bf16 MFMAs read xa
                as[i] = 0u;
            } else {
                af[i] = afrag[s][i];
                as[i] = ascale[s][i] >> sh;
            }
        }
        if constexpr (BF16A) {
            // 16-K chunk c of the step: lane L's codes 8c..8c+7 (dword c of
            // its fragment) against A elements 8c..8c+7 of the same group.
#pragma unroll
            for (int j = 0; j < NBLK; ++j) {
                const float bsc = scale_operand((bscale[s][j] >> sh) & 0xFFu);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const bf16x8 bv = widen8_fp4(bfrag[s][j][c], bsc);
#pragma unroll
                    for (int i = 0; i < MBLK; ++i)
                        acc[i][j] = mfma_bf16_32x32x16(bv, __builtin_bit_cast(bf16x8, xa[s][i][c]), acc[i][j]);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < NBLK; ++j) {
                const uint32_t bs = bscale[s][j] >> sh;
#pragma unroll
                for (int i = 0; i < MBLK; ++i)
                    acc[i][j] = mfma_fp4_32x32x64(bfrag[s][j], af[i], acc[i][j], bs, as[i]);
            }
        }
    }

    // The epilogue reads the accumulators right after the last MFMA; pad the
    // MFMA-result-to-VALU distance explicitly (the asm names every
    // accumulator, so it stays after the MFMAs and before the first read).
#pragma unroll
    for (int i = 0; i < MBLK; ++i)
#pragma unroll
        for (int j = 0; j < NBLK; ++j) mfma_result_fence(acc[i][j]);

    // ---- 4. epilogue
    // lane L, element e of tile (i, j): m = 32 (mb0 + i) + L % 32,
    // n = 32 nb + 8 (e / 4) + 4 (L / 32) + e % 4.
    const int m_lane = L & 31;
    const int n_lane = 4 * (L >> 5);
    constexpr int TR = MBLK * kRowBlock;      // rows of the workgroup tile
    constexpr int TC = NBLK * WN * kRowBlock; // columns of the workgroup tile
    constexpr int SROW = TC + 8;              // bf16 per staged row (16-byte pad)
    uint16_t* stage = (uint16_t*)(lds + gemm_red_bytes(WN, WK, MBLK, NBLK));
    const bool partial = p.partial != nullptr;   // K is split over workgroups
    const bool finish_here = partial && p.counters != nullptr;
    __shared__ uint32_t last_arrival;
    if constexpr (FUSED || REGA) __syncthreads();   // every wave is done with the activation in LDS
    constexpr int RL = red_lane_bytes(MBLK, NBLK);
    // four consecutive accumulators (from float index idx) of lane `lane` of wave w2
    auto red4 = [&](int w2, int lane, int idx) -> f32x4 {
        return *(const f32x4*)(lds + (size_t)(w2 * 64 + lane) * RL + idx * 4);
    };
    if constexpr (WK > 1) {
        uint8_t* mine = lds + (size_t)(wave * 64 + L) * RL;
#pragma unroll
        for (int i = 0; i < MBLK; ++i)
#pragma unroll
            for (int j = 0; j < NBLK; ++j)
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const f32x4 v4 = {acc[i][j][4 * e4], acc[i][j][4 * e4 + 1], acc[i][j][4 * e4 + 2],
                                      acc[i][j][4 * e4 + 3]};
                    *(f32x4*)(mine + ((i * NBLK + j) * 16 + 4 * e4) * 4) = v4;
                }
        __syncthreads();
    }
    // groups of 4 consecutive n per (i, j, r); the WK waves of column wn share
    // them.  Split-K partials go straight to the workspace as fp32; bf16
    // results are staged in LDS as a row-major tile first.
    auto stage4 = [&](int i, int j, int r, const float (&v)[4]) {
        const int row = i * kRowBlock + m_lane;
        const int col = (wn * NBLK + j) * kRowBlock + 8 * r + n_lane;
        uint2 w;
        w.x = pack_bf16x2(v[0], v[1]);
        w.y = pack_bf16x2(v[2], v[3]);
        *(uint2*)(stage + row * SROW + col) = w;
    };
    auto emit = [&](int i, int j, int r, const float (&v)[4]) {
        if (partial) {
            const int m = (mb0 + i) * kRowBlock + m_lane;
            const int nb = nb0 + j;
            const int n0 = nb * kRowBlock + 8 * r + n_lane;
            if (m >= p.M || nb >= p.RBn) return;
            float* dst = p.partial + ((size_t)split * p.M + m) * p.ldp + n0;
            if (finish_here) {
                store_partial_agent(dst, v);
            } else {
                const f32x4 pv = {v[0], v[1], v[2], v[3]};
                *(f32x4*)dst = pv;
            }
        } else {
            stage4(i, j, r, v);
        }
    };
    // The last arrival's sum of one group over the splits, in split order.
    auto finish = [&](int i, int j, int r) {
        const int m = (mb0 + i) * kRowBlock + m_lane;
        const int nb = nb0 + j;
        const int n0 = nb * kRowBlock + 8 * r + n_lane;
        float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (m < p.M && nb < p.RBn) {
            const float* src = p.partial + (size_t)m * p.ldp + n0;
            f32x4 acc4 = load_partial_agent(src);
            for (int k0 = 1; k0 < p.splits; k0 += 4) {   // 4 splits' loads in flight, then add in order
                f32x4 x[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (k0 + q < p.splits) x[q] = load_partial_agent(src + (size_t)(k0 + q) * p.M * p.ldp);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (k0 + q < p.splits) acc4 += x[q];
            }
            v[0] = acc4.x;
            v[1] = acc4.y;
            v[2] = acc4.z;
            v[3] = acc4.w;
        }
        stage4(i, j, r, v);
    };
    if constexpr (WK == 1) {
#pragma unroll
        for (int i = 0; i < MBLK; ++i)
#pragma unroll
            for (int j = 0; j < NBLK; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float v[4] = {acc[i][j][4 * r], acc[i][j][4 * r + 1], acc[i][j][4 * r + 2],
                                        acc[i][j][4 * r + 3]};
                    emit(i, j, r, v);
                }
    } else {
        constexpr int GPW = MBLK * NBLK * 4;
        for (int gi = wkk; gi < GPW; gi += WK) {
            const int ij = gi >> 2, r = gi & 3;
            const int i = ij / NBLK, j = ij % NBLK;
            f32x4 s4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int w2 = 0; w2 < WK; ++w2) s4 += red4(w2 * WN + wn, L, (i * NBLK + j) * 16 + 4 * r);
            const float v[4] = {s4.x, s4.y, s4.z, s4.w};
            emit(i, j, r, v);
        }
    }
    if (partial) {
        if (!finish_here) return;   // reduce_kernel sums the partials
        // A workgroup barrier does not wait for vector memory: every wave
        // first waits until its own partial stores have completed (vmcnt
        // counts stores on gfx9; they are agent-scope, so complete means
        // visible to every XCD), then the barrier, then one atomic per
        // workgroup counts the arrival at this tile.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) {
            uint32_t* counter = p.counters + (nt * p.mtiles + mt);
            const uint32_t before = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last_arrival = before == (uint32_t)(p.splits - 1);
            if (last_arrival) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (!last_arrival) return;
        if constexpr (WK == 1) {
#pragma unroll
            for (int i = 0; i < MBLK; ++i)
#pragma unroll
                for (int j = 0; j < NBLK; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) finish(i, j, r);
        } else {
            constexpr int GPW = MBLK * NBLK * 4;
            for (int gi = wkk; gi < GPW; gi += WK) {
                const int ij = gi >> 2, r = gi & 3;
                finish(ij / NBLK, ij % NBLK, r);
            }
        }
    }
    __syncthreads();
    // the staged tile leaves in 16-byte row chunks: consecutive lanes write
    // consecutive bytes of a row of C, non-temporal (C is not read again
    // here; the split-K partials above stay cached for their reader)
    const int m_base = mb0 * kRowBlock;
    const int n_base = nt * WN * NBLK * kRowBlock;
    const bool vec16 = ((uintptr_t)p.C % 16 == 0) && (p.ldc % 8 == 0);
    for (int c = tid; c < TR * TC / 8; c += NT) {
        const int row = c / (TC / 8), c8 = c % (TC / 8);
        const int m = m_base + row, n = n_base + 8 * c8;
        if (m >= p.M || n >= p.N) continue;
        const u32x4 v = *(const u32x4*)(stage + row * SROW + 8 * c8);
        uint16_t* dst = p.C + (size_t)m * p.ldc + n;
        if (vec16 && n + 7 < p.N) {
            __builtin_nontemporal_store(v, (u32x4*)dst);
        } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (n + q < p.N) dst[q] = (uint16_t)(w[q >> 1] >> (16 * (q & 1)));
        }
    }
}

// ---------------------------------------------------------------------------
// Instantiation table.  This file is compiled once per K-step budget KR
// (-DMX4_KR=1, 2, 3, 4 or 8); each object instantiates MBLK, NBLK in {1, 2},
// WN in {1, 2}, WK in {1, 2, 4, 8, 16} (at most 16 waves) and the four
// activation modes with all four row chunks (RQ = 4), and the register modes
// with MBLK = WN = 1 also with RQ = 1 and 2.

#ifndef MX4_KR
#error "compile with -DMX4_KR=<K steps per wave>"
#endif

typedef GemmKernelFn GemmFn;

template <int MBLK, int NBLK, int WN, int AM, int RQ>
static GemmFn pick_wk(int wk) {
    constexpr int KR = MX4_KR;
    switch (wk) {
        case 1: return gemm_kernel<MBLK, NBLK, WN, 1, AM, KR, RQ>;
        case 2: return gemm_kernel<MBLK, NBLK, WN, 2, AM, KR, RQ>;
        case 4: return gemm_kernel<MBLK, NBLK, WN, 4, AM, KR, RQ>;
        case 8: return gemm_kernel<MBLK, NBLK, WN, 8, AM, KR, RQ>;
        case 16: return WN == 1 ? gemm_kernel<MBLK, NBLK, WN, (WN == 1 ? 16 : 8), AM, KR, RQ> : nullptr;
        default: return nullptr;
    }
}

template <int MBLK, int NBLK, int AM>
static GemmFn pick_wn(int wn, int wk) {
    switch (wn) {
        case 1: return pick_wk<MBLK, NBLK, 1, AM, 4>(wk);
        case 2: return pick_wk<MBLK, NBLK, 2, AM, 4>(wk);
        default: return nullptr;
    }
}

template <int AM>
static GemmFn pick_tile(const Plan& plan) {
    if (plan.mb == 1 && plan.nb == 1) return pick_wn<1, 1, AM>(plan.wn, plan.wk);
    if (plan.mb == 1 && plan.nb == 2) return pick_wn<1, 2, AM>(plan.wn, plan.wk);
    if (plan.mb == 2 && plan.nb == 1) return pick_wn<2, 1, AM>(plan.wn, plan.wk);
    if (plan.mb == 2 && plan.nb == 2) return pick_wn<2, 2, AM>(plan.wn, plan.wk);
    return nullptr;
}

// The RQ < 4 kernels (register modes, MBLK = WN = 1).
template <int AM, int RQ>
static GemmFn pick_rows(const Plan& plan) {
    if (plan.nb == 1) return pick_wk<1, 1, 1, AM, RQ>(plan.wk);
    if (plan.nb == 2) return pick_wk<1, 2, 1, AM, RQ>(plan.wk);
    return nullptr;
}

#define MX4_CAT2(a, b) a##b
#define MX4_CAT(a, b) MX4_CAT2(a, b)
GemmFn MX4_CAT(find_gemm_kr, MX4_KR)(const Plan& plan, int rq) {
    const bool reg = plan.amode == kAmDirect || plan.amode == kAmBf16;
    if (rq < 4 && reg && plan.mb == 1 && plan.wn == 1) {
        if (plan.amode == kAmDirect) return rq == 1 ? pick_rows<kAmDirect, 1>(plan) : pick_rows<kAmDirect, 2>(plan);
        return rq == 1 ? pick_rows<kAmBf16, 1>(plan) : pick_rows<kAmBf16, 2>(plan);
    }
    switch (plan.amode) {
        case kAmLds: return pick_tile<kAmLds>(plan);
        case kAmPrequant: return pick_tile<kAmPrequant>(plan);
        case kAmDirect: return pick_tile<kAmDirect>(plan);
        case kAmBf16: return pick_tile<kAmBf16>(plan);
        default: return nullptr;
    }
}

#if MX4_KR == 1
// The split-K reduction and the launch helpers live in one object only.
// Grid (ceil(N / 4 / 64), rows) of one-wave workgroups: one thread per 4
// consecutive n of row m (rows past 65535 are walked by the y workgroups).
// Small workgroups spread the loads over more CUs: at M = 16, N = 2112 the
// 144 one-wave workgroups finish 0.15 us sooner than 48 four-wave ones.  The partials of each
// batch of 8 splits are all loaded before the first add (padding splits read
// zeros through the buffer bound), then added in split order.  Its arguments
// are ten scalars (48 bytes, preloaded in SGPRs; the row stride of the y
// workgroups is one of them, so no hidden arguments), which keeps the host's
// launch cheap.
constexpr int kReduceBatch = 8;
constexpr int kReduceThreads = 64;
__global__ void __launch_bounds__(kReduceThreads)
reduce_kernel(const float* partial, uint16_t* C, uint32_t partial_bytes, int M, int N, int ldp, int ldc, int splits,
              int c_vec, int mstep) {
    const int n0 = 4 * (int)(blockIdx.x * (unsigned)kReduceThreads + threadIdx.x);
    if (n0 >= N) return;
    const Rsrc rp_ = make_rsrc(partial, partial_bytes);
    const uint32_t split_stride = (uint32_t)M * (uint32_t)ldp * 4u;
    for (int m = blockIdx.y; m < M; m += mstep) {
        const uint32_t base = ((uint32_t)m * (uint32_t)ldp + (uint32_t)n0) * 4u;
        f32x4 s = __builtin_bit_cast(f32x4, bload16(rp_, base, 0u));
        for (int k0 = 1; k0 < splits; k0 += kReduceBatch) {
            u32x4 x[kReduceBatch];
#pragma unroll
            for (int q = 0; q < kReduceBatch; ++q)
                x[q] = bload16(rp_, k0 + q < splits ? base + (uint32_t)(k0 + q) * split_stride : 0x80000000u, 0u);
#pragma unroll
            for (int q = 0; q < kReduceBatch; ++q)
                if (k0 + q < splits) s += __builtin_bit_cast(f32x4, x[q]);
        }
        const float v[4] = {s.x, s.y, s.z, s.w};
        store_bf16x4(C, ldc, N, c_vec != 0, m, n0, v);
    }
}

GemmFn find_gemm_kr2(const Plan& plan, int rq);
GemmFn find_gemm_kr3(const Plan& plan, int rq);
GemmFn find_gemm_kr4(const Plan& plan, int rq);
GemmFn find_gemm_kr8(const Plan& plan, int rq);

// The smallest compiled K-step budget that holds a wave's steps (3 steps per
// wave -- 24 K steps over 8 waves -- would otherwise run a padding step).
int gemm_kr_for(int steps_per_wave) {
    static const int kBudgets[] = {1, 2, 3, 4, 8};
    for (int kr : kBudgets)
        if (steps_per_wave <= kr) return kr;
    return 0;
}

static GemmFn find_kernel(const Plan& plan, int kr, int rq = 4) {
    switch (kr) {
        case 1: return find_gemm_kr1(plan, rq);
        case 2: return find_gemm_kr2(plan, rq);
        case 3: return find_gemm_kr3(plan, rq);
        case 4: return find_gemm_kr4(plan, rq);
        case 8: return find_gemm_kr8(plan, rq);
        default: return nullptr;
    }
}

// Row chunks a call needs loaded (the kernels' RQ): with a single M tile of
// one 32-row block, the chunks that hold rows below M; else all four.
static int row_chunks(const Plan& plan, const GemmParams& p) {
    if (p.RBm != 1 || plan.mb != 1) return 4;
    return p.M <= 8 ? 1 : p.M <= 16 ? 2 : 4;
}

size_t gemm_lds_bytes(const Plan& plan, int steps_per_split) {
    if (plan.amode == kAmStream) return stream_lds_bytes(plan);
    if (plan.amode == kAmShared) return shared_lds_bytes(plan, steps_per_split);
    if (plan.amode == kAmTile) return tile_lds_bytes(plan);
    const size_t a_op = plan.amode == kAmLds ? (size_t)plan.mb * steps_per_split * 64 * 17 : 0;
    size_t out = gemm_red_bytes(plan.wn, plan.wk, plan.mb, plan.nb) + gemm_stage_bytes(plan.wn, plan.mb, plan.nb);
    if (plan.amode == kAmDirect || plan.amode == kAmBf16) {   // tiles or slabs alias the epilogue's buffers
        const int nw = plan.wn * plan.wk;
        const int kr = gemm_kr_for((steps_per_split + plan.wk - 1) / plan.wk);
        const size_t slab =
            gemm_uses_dma(nw, plan.mb, kr) ? gemm_dma_bytes(nw, plan.mb, kr) : gemm_slab_bytes(nw, plan.mb, kr);
        out = slab > out ? slab : out;
    }
    return a_op > out ? a_op : out;
}

bool gemm_plan_supported(const Plan& plan) {
    if (plan.amode == kAmStream) return plan.splits >= 1 && find_stream_kernel(plan, 4) != nullptr;
    if (plan.amode == kAmShared) return plan.splits >= 1 && find_shared_kernel(plan, 8) != nullptr;
    if (plan.amode == kAmTile) return plan.splits >= 1 && find_tile_kernel(plan) != nullptr;
    return plan.splits >= 1 && find_kernel(plan, 1) != nullptr;
}

bool resolve_gemm(const Plan& plan, const GemmParams& p, GemmLaunch* out) {
    const int per_wave = (p.steps_per_split + plan.wk - 1) / plan.wk;
    const int stages = plan.amode == kAmTile ? tile_stages(plan, (long long)p.mtiles * p.ntiles * p.splits) : 0;
    GemmFn fn = plan.amode == kAmStream   ? find_stream_kernel(plan, row_chunks(plan, p))
              : plan.amode == kAmShared ? find_shared_kernel(plan, p.steps_per_split)
              : plan.amode == kAmTile   ? find_tile_kernel(plan, stages)
                                        : find_kernel(plan, gemm_kr_for(per_wave), row_chunks(plan, p));
    if (!fn) return false;
    const size_t lds = plan.amode == kAmTile ? tile_lds_bytes(plan, stages) : gemm_lds_bytes(plan, p.steps_per_split);
    // the shared mode's workgroup is wn MFMA waves plus wk quantiser waves
    const int waves = plan.amode == kAmShared ? plan.wn + plan.wk : plan.wn * plan.wk;
    // the shared kernels take their tile placement in bits 8 and up of the
    // steps-per-split argument (at most 24 steps); the tile kernels take the
    // placement code in bits 0..7 (XCD placement for one split only) and the
    // steps per split above it
    const double kbytes = p.K / 2.0 + p.K / 32.0;   // packed bytes of one row over K
    const int steps_arg =
        plan.amode == kAmShared
            ? p.steps_per_split |
                  (shared_xcd_map(p.mtiles, p.ntiles, p.splits, 64.0 * p.K, 32.0 * plan.nb * plan.wn * kbytes) << 8)
        : plan.amode == kAmTile
            ? (p.splits == 1 ? tile_xcd_map(p.mtiles, p.ntiles, 32.0 * plan.mb * kbytes, 32.0 * plan.nb * kbytes,
                                            tile_wgs_per_xcd(lds, waves), tile_runs_policy(plan.mb, plan.nb, p.K))
                             : 0) |
                  (p.steps_per_split << 8)
            : p.steps_per_split;
    *out = GemmLaunch{fn, (unsigned)p.ntiles, (unsigned)p.mtiles, (unsigned)p.splits, (unsigned)(64 * waves), lds,
                      amode_prequantises(plan.amode), steps_arg};
    return true;
}

hipError_t launch_gemm(const GemmLaunch& gl, const GemmParams& p, hipStream_t s) {
    const void* a_src = gl.prequant ? (const void*)p.aop : (const void*)p.A;
    return launch_kernel(gl.fn, dim3(gl.gx, gl.gy, gl.gz), dim3(gl.block), gl.lds, s, a_src, p.bp, p.C, p.partial,
                         p.lda, p.ldc, p.M, p.N, p.K, gl.steps_arg, p.counters, p.splits, p.mtiles);
}

hipError_t launch_reduce(const GemmParams& p, hipStream_t s) {
    const unsigned gx = (unsigned)(((p.N + 3) / 4 + kReduceThreads - 1) / kReduceThreads);
    const unsigned gy = (unsigned)(p.M < 65535 ? p.M : 65535);
    return launch_kernel(reduce_kernel, dim3(gx, gy), dim3(kReduceThreads), 0, s, (const float*)p.partial, p.C,
                         p.partial_bytes, p.M, p.N, p.ldp, p.ldc, p.splits, p.c_vec, (int)gy);
}
#endif

}  // namespace mx4
