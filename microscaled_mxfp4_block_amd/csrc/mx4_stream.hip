// mx4_stream.hip -- K-looped block-scaled MXFP4 GEMM for gfx950 (MI355X):
// the activation mode MX_AMODE_STREAM.
//
//   C[M,N] = bf16_RNE( sum_k deq(A)[m,k] * deq(B)[n,k] )   (fp32 accumulation)
//
// The contraction is the block-scaled dot that the kernelindex.com
// amd-mxfp4-mm pages write as tl.dot_scaled(a, a_scale, "e2m1", b, b_scale,
// "e2m1") (submission 748756, kernel_fused_mxfp4_gemm), on
// v_mfma_scale_f32_32x32x64_f8f6f4; the activation is quantised by the rule
// of submission 755056, "Software MXFP4 quant" (mx4_device.h).
//
// A workgroup owns 32 rows of C (one M block) and 32 NB columns (NB N blocks)
// over one K split; its WK waves take the split's 64-K steps in turn (wave w:
// steps w, w + WK, w + 2 WK, ...), so at any moment the waves of a workgroup
// read neighbouring pieces of the weight and of the activation.  Each wave
// walks its steps through a ring of D slots:
//   - a slot holds the step's NB weight fragments and scale words in VGPRs
//     (128-bit and 32-bit non-temporal buffer loads of the packed layout:
//     one fully coalesced load per lane per fragment) and its 32 x 64 bf16
//     activation tile in the wave's LDS (gfx950 buffer loads straight to LDS,
//     8 lanes per 128-byte row segment, RQ of the 4 eight-row chunks, the
//     16-byte column j of row r at slot j ^ ((r >> 1) & 7) so that the
//     fragment reads below hit distinct bank groups);
//   - the loads of D steps are in flight at once; the weight's are issued
//     first in each step, so the HBM stream starts with the kernel;
//   - for each step the wave waits until at most the (D - 1) later steps'
//     loads are outstanding (vector-memory operations of a wave complete in
//     issue order), reads back the 64 bytes of its lane's 32-element group,
//     quantises it in registers (scale byte by the bit rule, e2m1 codes by
//     the gfx950 fp4 convert), runs NB MFMAs and refills the slot with the
//     step D ahead.
// Steps past the split (and a group past K when K % 64 == 32) are loaded
// from an offset past the buffer, read zeros (zero codes, scale byte 0) and
// add nothing; the load count per step stays fixed, so every wait count is a
// compile-time constant.  Rows past M read zeros through the buffer bound,
// or are not loaded at all (RQ < 4) and feed only outputs that are never
// stored.
//
// Epilogue as in mx4_gemm.hip: the WK waves add their accumulators through
// LDS, the sum is rounded to bf16 (v_cvt_pk_bf16_f32), staged in LDS and
// stored in 16-byte row chunks; with K split over workgroups, fp32 partials
// go to the workspace and reduce_kernel (or the last workgroup to arrive at
// the tile) sums them in split order.
#include "mx4_device.h"
#include "mx4_internal.h"

namespace mx4 {

constexpr int kRingTile = kRowBlock * 128;   // 32 rows x 64 K of bf16

// Ring depth: as many steps in flight per wave as 128 KiB of LDS rings hold
// (8 for up to 4 waves, 4 at 8 waves, 2 at 16), and at most 63 loads
// outstanding (the vmcnt counter's range).
__host__ __device__ constexpr int stream_ring_cap(int wk) { return wk <= 4 ? 8 : wk <= 8 ? 4 : 2; }
__host__ __device__ constexpr int stream_ring_depth(int wk, int lps) {
    return stream_ring_cap(wk) < 1 + 63 / lps ? stream_ring_cap(wk) : 1 + 63 / lps;
}
__host__ __device__ constexpr int ring_slot(int r, int j) { return r * 128 + ((j ^ ((r >> 1) & 7)) << 4); }
__host__ __device__ constexpr size_t stream_ring_bytes(int wk) {
    return (size_t)wk * stream_ring_cap(wk) * kRingTile;
}
// Reduction buffer, lane-major (each lane's NB x 16 accumulators contiguous,
// 16 bytes of padding), then the staged bf16 tile (rows padded by 8).
__host__ __device__ constexpr int stream_red_lane(int nb) { return nb * 16 * 4 + 16; }
__host__ __device__ constexpr size_t stream_red_bytes(int wk, int nb) {
    return wk > 1 ? (size_t)wk * 64 * stream_red_lane(nb) : 0;
}
__host__ __device__ constexpr size_t stream_stage_bytes(int nb) {
    return (size_t)kRowBlock * (nb * kRowBlock + 8) * 2;
}

__device__ __forceinline__ void store_partial_agent4(float* dst, float v0, float v1, float v2, float v3) {
    const uint64_t lo = (uint64_t)__float_as_uint(v0) | ((uint64_t)__float_as_uint(v1) << 32);
    const uint64_t hi = (uint64_t)__float_as_uint(v2) | ((uint64_t)__float_as_uint(v3) << 32);
    __hip_atomic_store((uint64_t*)dst, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store((uint64_t*)dst + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4 load_partial_agent4(const float* src) {
    const uint64_t lo = __hip_atomic_load((const uint64_t*)src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load((const uint64_t*)src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return f32x4{__uint_as_float((uint32_t)lo), __uint_as_float((uint32_t)(lo >> 32)),
                 __uint_as_float((uint32_t)hi), __uint_as_float((uint32_t)(hi >> 32))};
}

// The call arrives as the same thirteen scalars as gemm_kernel's
// (GemmKernelFn; the first ten preloaded in SGPRs).
template <int NB, int WK, int RQ>
__global__ void __launch_bounds__(64 * WK)
gemm_stream_kernel(const void* a_src, const uint8_t* bp, uint16_t* C, float* partial_buf, int lda, int ldc, int M,
                   int N, int K, int steps_per_split, uint32_t* counters, int splits, int mtiles) {
    constexpr int LPS = RQ + 2 * NB;             // vector-memory loads per step
    constexpr int D = stream_ring_depth(WK, LPS);
    constexpr uint32_t kOutOfRange = 0x80000000u;
    const OperandGeom gb = operand_geom(N, K);
    const int KS = gb.KS, KW = gb.KW, RBn = gb.RB;
    const int G = K / kGroup;
    const uint16_t* A = (const uint16_t*)a_src;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int L = tid & 63;

    const int nt = blockIdx.x;
    const int mt = blockIdx.y;
    const int split = blockIdx.z;
    const int nb0 = nt * NB;
    const int tb = split * steps_per_split;
    const int te = min(tb + steps_per_split, KS);
    const int S = (te - tb - wave + WK - 1) / WK;   // this wave's steps (may be 0)
    const int S_all = (te - tb + WK - 1) / WK;      // the most any wave of the workgroup has

    uint8_t* ring = lds + (size_t)wave * (D * kRingTile);
    const Rsrc ra = make_rsrc(A, (uint32_t)M * (uint32_t)lda * 2u);
    const Rsrc rb = make_rsrc(bp, (uint32_t)gb.total_bytes);
    const uint32_t b_code_bytes = (uint32_t)gb.code_bytes;

    // Activation chunk q of a step: lane L loads tile row r = (64 q + L) / 8,
    // the 16-byte column j whose swizzled slot is (64 q + L) % 8.
    uint32_t a_lane[RQ];
    int a_col[RQ];
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
        const int c = q * 64 + L;
        const int r = c >> 3;
        const int j = (c & 7) ^ ((r >> 1) & 7);
        a_col[q] = j;
        a_lane[q] = (uint32_t)(mt * kRowBlock + r) * (uint32_t)lda * 2u + (uint32_t)j * 16u;
    }

    u32x4 bq[D][NB];
    uint32_t bs[D][NB];
    // Loads of this wave's step i into ring slot `slot` (a compile-time index).
    auto issue = [&](int i, int slot) {
        const int t = tb + wave + WK * i;
        const bool on = i < S;
        const int tc = on ? t : 0;
        const uint32_t vcode = on ? (uint32_t)L * 16u : kOutOfRange;
        const uint32_t vscale = on ? (uint32_t)L * 4u : kOutOfRange;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int nb = min(nb0 + j, RBn - 1);   // clamped blocks are never stored
            bq[slot][j] = bload16<kNonTemporal>(rb, vcode, (uint32_t)(nb * KS + tc) * 1024u);
            bs[slot][j] = bload4(rb, vscale, b_code_bytes + (uint32_t)(nb * KW + (tc >> 2)) * 256u);
        }
#pragma unroll
        for (int q = 0; q < RQ; ++q) {
            const bool live = on && 2 * t + (a_col[q] >> 2) < G;
            bload16_lds(ra, ring + slot * kRingTile + q * 1024,
                        live ? a_lane[q] + (uint32_t)t * 128u : kOutOfRange);
        }
    };

    f32x16 acc[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;

    // the first D steps, in step order (the waits below count on it)
#pragma unroll
    for (int d = 0; d < D; ++d) {
        issue(d, d);
        asm volatile("" ::: "memory");
    }

    const int rounds = (S_all + D - 1) / D;
    for (int rr = 0; rr < rounds; ++rr) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int i = rr * D + d;
            if (i >= S_all) break;   // uniform over the workgroup
            // step i has landed when at most the loads of steps i+1 .. i+D-1
            // are outstanding (issued after it, each issue() a fixed LPS)
            asm volatile("" ::: "memory");
            wait_vmcnt<(D - 1) * LPS>();
            asm volatile("" ::: "memory");
            u32x4 x[4];
            const uint8_t* tile = ring + d * kRingTile;
#pragma unroll
            for (int c = 0; c < 4; ++c) x[c] = *(const u32x4*)(tile + ring_slot(L & 31, 4 * (L >> 5) + c));
            u32x4 af;
            const uint32_t as = quant_group32(x, af);
            const int sh = 8 * ((tb + wave + WK * i) & 3);
            // The MFMAs take the slot's weight registers before their refill
            // is issued, so the refill can load into the same registers (no
            // copies between rounds, which would wait for the loads).
#pragma unroll
            for (int j = 0; j < NB; ++j) acc[j] = mfma_fp4_32x32x64(bq[d][j], af, acc[j], bs[d][j] >> sh, as);
            // the slot's LDS reads have completed before its refill is issued
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            issue(i + D, d);
            asm volatile("" ::: "memory");
        }
    }
    // the ring's last refills (past the split: zeros) land before its LDS is reused
    wait_vmcnt<0>();
#pragma unroll
    for (int j = 0; j < NB; ++j) mfma_result_fence(acc[j]);

    // ---- epilogue
    // lane L, element e of block j: m = 32 mt + L % 32,
    // n = 32 (nb0 + j) + 8 (e / 4) + 4 (L / 32) + e % 4.
    constexpr int TC = NB * kRowBlock;
    constexpr int SROW = TC + 8;
    constexpr int RL = stream_red_lane(NB);
    const int m_lane = L & 31;
    const int n_lane = 4 * (L >> 5);
    uint16_t* stage = (uint16_t*)(lds + stream_red_bytes(WK, NB));
    const bool part = partial_buf != nullptr;
    const bool finish_here = part && counters != nullptr;
    const int ldp = RBn * kRowBlock;
    __shared__ uint32_t last_arrival;
    __syncthreads();   // every wave is done with its ring
    if constexpr (WK > 1) {
        uint8_t* mine = lds + (size_t)(wave * 64 + L) * RL;
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const f32x4 v4 = {acc[j][4 * e4], acc[j][4 * e4 + 1], acc[j][4 * e4 + 2], acc[j][4 * e4 + 3]};
                *(f32x4*)(mine + (j * 16 + 4 * e4) * 4) = v4;
            }
        __syncthreads();
    }
    auto stage4 = [&](int j, int r, const f32x4& v) {
        const int col = j * kRowBlock + 8 * r + n_lane;
        uint2 w;
        w.x = pack_bf16x2(v.x, v.y);
        w.y = pack_bf16x2(v.z, v.w);
        *(uint2*)(stage + m_lane * SROW + col) = w;
    };
    auto emit = [&](int j, int r, const f32x4& v) {
        if (part) {
            const int m = mt * kRowBlock + m_lane;
            const int nb = nb0 + j;
            if (m >= M || nb >= RBn) return;
            float* dst = partial_buf + ((size_t)split * M + m) * ldp + nb * kRowBlock + 8 * r + n_lane;
            if (finish_here)
                store_partial_agent4(dst, v.x, v.y, v.z, v.w);
            else
                *(f32x4*)dst = v;
        } else {
            stage4(j, r, v);
        }
    };
    auto finish = [&](int j, int r) {
        const int m = mt * kRowBlock + m_lane;
        const int nb = nb0 + j;
        f32x4 s4 = {0.0f, 0.0f, 0.0f, 0.0f};
        if (m < M && nb < RBn) {
            const float* src = partial_buf + (size_t)m * ldp + nb * kRowBlock + 8 * r + n_lane;
            s4 = load_partial_agent4(src);
            for (int k0 = 1; k0 < splits; k0 += 4) {   // 4 splits' loads in flight, added in order
                f32x4 x[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (k0 + q < splits) x[q] = load_partial_agent4(src + (size_t)(k0 + q) * M * ldp);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (k0 + q < splits) s4 += x[q];
            }
        }
        stage4(j, r, s4);
    };
    if constexpr (WK == 1) {
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const f32x4 v = {acc[j][4 * r], acc[j][4 * r + 1], acc[j][4 * r + 2], acc[j][4 * r + 3]};
                emit(j, r, v);
            }
    } else {
        for (int gi = wave; gi < NB * 4; gi += WK) {
            const int j = gi >> 2, r = gi & 3;
            f32x4 s4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int w2 = 0; w2 < WK; ++w2)
                s4 += *(const f32x4*)(lds + (size_t)(w2 * 64 + L) * RL + (j * 16 + 4 * r) * 4);
            emit(j, r, s4);
        }
    }
    if (part) {
        if (!finish_here) return;   // reduce_kernel sums the partials
        // every wave's partial stores complete (agent scope: visible to every
        // XCD) before the barrier that precedes the arrival atomic
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0) {
            uint32_t* counter = counters + (nt * mtiles + mt);
            const uint32_t before = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last_arrival = before == (uint32_t)(splits - 1);
            if (last_arrival) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        if (!last_arrival) return;
        for (int gi = wave; gi < NB * 4; gi += WK) finish(gi >> 2, gi & 3);
    }
    __syncthreads();
    // the staged tile leaves in 16-byte row chunks, non-temporal
    const int m_base = mt * kRowBlock;
    const int n_base = nb0 * kRowBlock;
    const bool vec16 = ((uintptr_t)C % 16 == 0) && (ldc % 8 == 0);
    for (int c = tid; c < kRowBlock * TC / 8; c += 64 * WK) {
        const int row = c / (TC / 8), c8 = c % (TC / 8);
        const int m = m_base + row, n = n_base + 8 * c8;
        if (m >= M || n >= N) continue;
        const u32x4 v = *(const u32x4*)(stage + row * SROW + 8 * c8);
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
// Instantiations: NB in {1, 2, 4}, WK in {1, 2, 4, 8, 16} (NB <= 2 at 16
// waves), RQ in {1, 2, 4}.

template <int NB, int RQ>
static GemmKernelFn stream_pick_wk(int wk) {
    switch (wk) {
        case 1: return gemm_stream_kernel<NB, 1, RQ>;
        case 2: return gemm_stream_kernel<NB, 2, RQ>;
        case 4: return gemm_stream_kernel<NB, 4, RQ>;
        case 8: return gemm_stream_kernel<NB, 8, RQ>;
        case 16: return NB <= 2 ? gemm_stream_kernel<(NB <= 2 ? NB : 2), 16, RQ> : nullptr;
        default: return nullptr;
    }
}

template <int RQ>
static GemmKernelFn stream_pick_nb(int nb, int wk) {
    switch (nb) {
        case 1: return stream_pick_wk<1, RQ>(wk);
        case 2: return stream_pick_wk<2, RQ>(wk);
        case 4: return stream_pick_wk<4, RQ>(wk);
        default: return nullptr;
    }
}

GemmKernelFn find_stream_kernel(const Plan& plan, int rq) {
    if (plan.mb != 1 || plan.wn != 1) return nullptr;
    switch (rq) {
        case 1: return stream_pick_nb<1>(plan.nb, plan.wk);
        case 2: return stream_pick_nb<2>(plan.nb, plan.wk);
        case 4: return stream_pick_nb<4>(plan.nb, plan.wk);
        default: return nullptr;
    }
}

size_t stream_lds_bytes(const Plan& plan) {
    const size_t ring = stream_ring_bytes(plan.wk);
    const size_t epi = stream_red_bytes(plan.wk, plan.nb) + stream_stage_bytes(plan.nb);
    return ring > epi ? ring : epi;
}

}  // namespace mx4
