// mx4_gemm.hip -- single-launch MXFP4 GEMM for gfx950 (MI355X).
//
//   C[M,N] = bf16_RNE( sum_k deq(A)[m,k] * deq(B)[n,k] )   (fp32 accumulation)
//
// One kernel does the whole call: activation quantisation, the block-scaled
// fp4 contraction and (for split-K) the reduction of the K partials.  The
// contraction is what the kernelindex.com amd-mxfp4-mm pages write as
// tl.dot_scaled(a, a_scale, "e2m1", b, b_scale, "e2m1") (e.g. submission
// 748756, kernel_fused_mxfp4_gemm); here it runs directly on
// v_mfma_scale_f32_32x32x64_f8f6f4, whose per-lane e8m0 byte scales that
// lane's 32-element group by 2^(byte-127).
//
// Workgroup = WN x WK waves; workgroup tile = (32 MBLK) m x (32 NBLK WN) n
// over one K split of `steps_per_split` steps of 64.
//   1. Every wave issues the 128-bit loads of all its weight fragments for
//      its share of the split (WK waves share the split's K steps) before
//      anything else, so the one HBM round trip of the weight overlaps the
//      activation work below.  Weight bytes are read exactly once, straight
//      into VGPRs (non-temporal: they are never reused).
//   2. The workgroup quantises the activation slice it needs (its m rows x
//      its K split) once: one lane per 32-element group, amax is a per-lane
//      max, scale byte by the bit rule, e2m1 codes by the gfx950 fp4 convert.
//      The codes land in LDS in MFMA operand order, shared by the WN waves
//      that use them.
//   3. K loop: 16-byte LDS reads of the activation fragments, MFMAs against
//      the weight fragments already in registers.
//   4. The WK waves add their accumulators through LDS.  With one split the
//      result is rounded to bf16 and stored.  With several splits each
//      workgroup writes its fp32 partial tile, then counts itself in on the
//      tile's arrival counter; the last one to arrive sums the partials of all
//      splits in split order (deterministic) and stores bf16, and resets the
//      counter to zero for the next call.
#include "mx4_device.h"
#include "mx4_internal.h"

namespace mx4 {

// Workgroups are dispatched round-robin over the 8 XCDs (blockIdx i runs on
// XCD i % 8).  Remap so that consecutive logical tile indices share an XCD:
// the M tiles that read the same weight tiles, placed next to each other,
// then share one L2.
__device__ __forceinline__ int xcd_linear(int i, int G) {
    const int q = G / 8, r = G % 8, x = i % 8;
    return x * q + (x < r ? x : r) + i / 8;
}

// Activation operand in LDS: codes [MBLK][T][64 lanes][16 B], then scale
// bytes [MBLK][T][64 lanes]; T = K steps of the split.
__device__ __forceinline__ uint32_t lds_code_off(int mb, int tl, int lane, int T) {
    return (uint32_t)(((mb * T + tl) * 64 + lane) * 16);
}
__device__ __forceinline__ uint32_t lds_scale_off(int mb, int tl, int lane, int T, int mblk) {
    return (uint32_t)(mblk * T * 64 * 16 + (mb * T + tl) * 64 + lane);
}

// 4 consecutive bf16 outputs (n0..n0+3) of row m, masked at N.
__device__ __forceinline__ void store_bf16x4(const GemmParams& p, int m, int n0, const float (&v)[4]) {
    uint16_t* dst = p.C + (size_t)m * p.ldc + n0;
    if (p.c_vec && n0 + 3 < p.N) {
        uint2 w;
        w.x = pack_bf16x2(v[0], v[1]);
        w.y = pack_bf16x2(v[2], v[3]);
        *(uint2*)dst = w;
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (n0 + q < p.N) dst[q] = (uint16_t)bf16_rne(v[q]);
    }
}

template <int MBLK, int NBLK, int WN, int WK>
__global__ void __launch_bounds__(64 * WN * WK) gemm_kernel(GemmParams p) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ int last_flag;
    constexpr int NT = 64 * WN * WK;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int L = tid & 63;
    const int wn = wave % WN;
    const int wkk = wave / WN;

    // ---- tile of this workgroup
    const int lin = xcd_linear(blockIdx.x, gridDim.x);
    const int mt = lin % p.mtiles;
    const int rest = lin / p.mtiles;
    const int split = rest % p.splits;
    const int nt = rest / p.splits;
    const int mb0 = mt * MBLK;
    const int nb0 = (nt * WN + wn) * NBLK;   // first n block of this wave
    const int tb = split * p.steps_per_split;
    const int te = min(tb + p.steps_per_split, p.KS);
    const int T = te - tb;
    const int per_wave = (T + WK - 1) / WK;
    const int wb = tb + wkk * per_wave;
    const int we = min(wb + per_wave, te);
    const int nsteps = max(we - wb, 0);      // <= kStepsPerWaveMax by the planner

    // ---- 1. weight fragments of this wave, all in flight at once
    u32x4 bfrag[kStepsPerWaveMax][NBLK];
    uint32_t bscale[kStepsPerWaveMax][NBLK];
#pragma unroll
    for (int s = 0; s < kStepsPerWaveMax; ++s) {
        if (s < nsteps) {
            const int t = wb + s;
#pragma unroll
            for (int j = 0; j < NBLK; ++j) {
                const int nb = min(nb0 + j, p.RBn - 1);   // clamped blocks are never stored
                bfrag[s][j] = load16_nt(p.bp + ((size_t)(nb * p.KS + t) * 64 + L) * 16);
                bscale[s][j] = *(const uint32_t*)(p.bp + p.b_code_bytes +
                                                  ((size_t)(nb * p.KW + (t >> 2)) * 64 + L) * 4);
            }
        }
    }

    // ---- 2. quantise the activation slice into LDS
    const int row0 = mb0 * kRowBlock;
    const int rows = min(p.M - row0, MBLK * kRowBlock);   // >= 1
    const int G = p.K / kGroup;
    const int g0 = 2 * tb;
    const int g1 = min(2 * te, G);
    const int Gw = g1 - g0;
    if (rows < MBLK * kRowBlock || g1 < 2 * te) {
        // padding rows / the missing last group: zero codes and zero scale bytes
        const int words = MBLK * T * 64 * 17 / 4;
        for (int i = tid; i < words; i += NT) ((uint32_t*)lds)[i] = 0u;
        __syncthreads();
    }
    {
        const int units = rows * Gw;
        constexpr int QREG = 4;   // units per thread whose loads are issued together
        for (int u0 = 0; u0 < units; u0 += NT * QREG) {
            u32x4 x[QREG][4];
#pragma unroll
            for (int q = 0; q < QREG; ++q) {
                const int u = u0 + q * NT + tid;
                if (u < units) {
                    const int r = u / Gw, g = g0 + u % Gw;
                    const uint16_t* src = p.A + (size_t)(row0 + r) * p.lda + (size_t)g * kGroup;
#pragma unroll
                    for (int c = 0; c < 4; ++c) x[q][c] = load16(src + 8 * c);
                }
            }
#pragma unroll
            for (int q = 0; q < QREG; ++q) {
                const int u = u0 + q * NT + tid;
                if (u < units) {
                    const int r = u / Gw, g = g0 + u % Gw;
                    u32x4 codes;
                    const uint32_t byte = quant_group32(x[q], codes);
                    const int mb = r >> 5, tl = (g >> 1) - tb, lane = (r & 31) + 32 * (g & 1);
                    *(u32x4*)(lds + lds_code_off(mb, tl, lane, T)) = codes;
                    lds[lds_scale_off(mb, tl, lane, T, MBLK)] = (uint8_t)byte;
                }
            }
        }
    }
    __syncthreads();

    // ---- 3. K loop over the wave's steps
    f32x16 acc[MBLK][NBLK];
#pragma unroll
    for (int i = 0; i < MBLK; ++i)
#pragma unroll
        for (int j = 0; j < NBLK; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
#pragma unroll
    for (int s = 0; s < kStepsPerWaveMax; ++s) {
        if (s < nsteps) {
            const int t = wb + s;
            const int tl = t - tb;
            const int sh = 8 * (t & 3);
            u32x4 af[MBLK];
            uint32_t as[MBLK];
#pragma unroll
            for (int i = 0; i < MBLK; ++i) {
                af[i] = *(const u32x4*)(lds + lds_code_off(i, tl, L, T));
                as[i] = lds[lds_scale_off(i, tl, L, T, MBLK)];
            }
#pragma unroll
            for (int j = 0; j < NBLK; ++j) {
                const uint32_t bs = bscale[s][j] >> sh;
#pragma unroll
                for (int i = 0; i < MBLK; ++i)
                    acc[i][j] = mfma_fp4_32x32x64(bfrag[s][j], af[i], acc[i][j], bs, as[i]);
            }
        }
    }

    // ---- 4. epilogue
    // lane L, element e of tile (i, j): m = 32 (mb0 + i) + L % 32,
    // n = 32 nb + 8 (e / 4) + 4 (L / 32) + e % 4.
    const int m_lane = L & 31;
    const int n_lane = 4 * (L >> 5);
    constexpr int E = MBLK * NBLK * 16;       // accumulator floats per lane
    float* red = (float*)lds;
    if constexpr (WK > 1) {
        __syncthreads();   // every wave is done with the activation operand
#pragma unroll
        for (int i = 0; i < MBLK; ++i)
#pragma unroll
            for (int j = 0; j < NBLK; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) red[((wave * E) + (i * NBLK + j) * 16 + e) * 64 + L] = acc[i][j][e];
        __syncthreads();
    }
    // groups of 4 consecutive n per (i, j, r); the WK waves of column wn share them
    constexpr int GPW = MBLK * NBLK * 4;
    const bool partial = p.splits > 1;
    for (int gi = wkk; gi < GPW; gi += WK) {
        const int ij = gi >> 2, r = gi & 3;
        const int i = ij / NBLK, j = ij % NBLK;
        float v[4];
        if constexpr (WK > 1) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float s = 0.0f;
#pragma unroll
                for (int w2 = 0; w2 < WK; ++w2)
                    s += red[(((w2 * WN + wn) * E) + (i * NBLK + j) * 16 + 4 * r + q) * 64 + L];
                v[q] = s;
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = acc[i][j][4 * r + q];
        }
        const int m = (mb0 + i) * kRowBlock + m_lane;
        const int nb = nb0 + j;
        const int n0 = nb * kRowBlock + 8 * r + n_lane;
        if (m >= p.M || nb >= p.RBn) continue;
        if (partial) {
            const f32x4 pv = {v[0], v[1], v[2], v[3]};
            *(f32x4*)(p.partial + ((size_t)split * p.M + m) * p.ldp + n0) = pv;
        } else {
            store_bf16x4(p, m, n0, v);
        }
    }
    if (!partial) return;

    // ---- split-K finish: the last workgroup of this tile to arrive reduces it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");   // publish this wave's partial stores
    __syncthreads();
    const int tile = nt * p.mtiles + mt;
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(p.counters + tile, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_flag = (old == p.splits - 1);
    }
    __syncthreads();
    if (!last_flag) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const int m_base = mb0 * kRowBlock;
    const int n_base = nt * WN * NBLK * kRowBlock;
    constexpr int TW4 = WN * NBLK * kRowBlock / 4;   // float4 groups per tile row
    for (int g = tid; g < MBLK * kRowBlock * TW4; g += NT) {
        const int m = m_base + g / TW4;
        const int n0 = n_base + 4 * (g % TW4);
        if (m >= p.M || n0 >= p.RBn * kRowBlock) continue;
        f32x4 s = *(const f32x4*)(p.partial + (size_t)m * p.ldp + n0);
        for (int k = 1; k < p.splits; ++k) {
            const f32x4 x = *(const f32x4*)(p.partial + ((size_t)k * p.M + m) * p.ldp + n0);
            s.x += x.x;
            s.y += x.y;
            s.z += x.z;
            s.w += x.w;
        }
        const float v[4] = {s.x, s.y, s.z, s.w};
        store_bf16x4(p, m, n0, v);
    }
    if (tid == 0) __hip_atomic_store(p.counters + tile, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Instantiation table: MBLK, NBLK in {1, 2}; WN in {1, 2, 4}; WK in {1, 2, 4, 8}
// with at most 16 waves (1024 lanes) per workgroup.

typedef void (*GemmFn)(GemmParams);

template <int MBLK, int NBLK, int WN>
GemmFn pick_wk(int wk) {
    switch (wk) {
        case 1: return gemm_kernel<MBLK, NBLK, WN, 1>;
        case 2: return gemm_kernel<MBLK, NBLK, WN, 2>;
        case 4: return gemm_kernel<MBLK, NBLK, WN, 4>;
        case 8: return WN <= 2 ? gemm_kernel<MBLK, NBLK, WN, (WN <= 2 ? 8 : 4)> : nullptr;
        default: return nullptr;
    }
}

template <int MBLK, int NBLK>
GemmFn pick_wn(int wn, int wk) {
    switch (wn) {
        case 1: return pick_wk<MBLK, NBLK, 1>(wk);
        case 2: return pick_wk<MBLK, NBLK, 2>(wk);
        case 4: return pick_wk<MBLK, NBLK, 4>(wk);
        default: return nullptr;
    }
}

static GemmFn find_kernel(const Plan& plan) {
    if (plan.mb == 1 && plan.nb == 1) return pick_wn<1, 1>(plan.wn, plan.wk);
    if (plan.mb == 1 && plan.nb == 2) return pick_wn<1, 2>(plan.wn, plan.wk);
    if (plan.mb == 2 && plan.nb == 1) return pick_wn<2, 1>(plan.wn, plan.wk);
    if (plan.mb == 2 && plan.nb == 2) return pick_wn<2, 2>(plan.wn, plan.wk);
    return nullptr;
}

size_t gemm_lds_bytes(const Plan& plan, int steps_per_split) {
    const size_t a_op = (size_t)plan.mb * steps_per_split * 64 * 17;
    const size_t red = plan.wk > 1 ? (size_t)plan.wn * plan.wk * plan.mb * plan.nb * 16 * 64 * 4 : 0;
    return a_op > red ? a_op : red;
}

bool gemm_plan_supported(const Plan& plan) {
    return plan.splits >= 1 && find_kernel(plan) != nullptr;
}

hipError_t launch_gemm(const Plan& plan, const GemmParams& p, hipStream_t s) {
    GemmFn fn = find_kernel(plan);
    if (!fn) return hipErrorInvalidValue;
    const long long grid = (long long)p.mtiles * p.ntiles * p.splits;
    const size_t lds = gemm_lds_bytes(plan, p.steps_per_split);
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(64 * plan.wn * plan.wk), lds, s, p);
    return hipGetLastError();
}

}  // namespace mx4
