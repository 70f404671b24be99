// mx4_internal.h -- host-side declarations shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <utility>
#include <vector>

#include "mx4_layout.h"

namespace mx4 {

// Largest number of K steps one wave holds in registers (its whole share of
// a split); the planner splits K further when a shape needs more.
constexpr int kStepsPerWaveMax = 8;
// Largest dynamic LDS block the planner gives a workgroup (gfx950: 160 KiB
// per CU, less a little for the kernel's static LDS).
constexpr size_t kLdsBudget = 160 * 1024 - 256;

// Kernel launch straight through hipLaunchKernel, with the argument array
// built here; each argument is first converted to the kernel's parameter
// type.  The triple-chevron form costs about 0.14 us more host time per launch
// (it pushes and pops a launch configuration), and the status comes back
// directly, with no hipGetLastError call.
template <typename... P>
struct KernelCall {
    static hipError_t go(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s, P... args) {
        void* argv[] = {(void*)&args...};
        return hipLaunchKernel((const void*)kernel, grid, block, argv, lds, s);
    }
};
template <typename... P, typename... A>
inline hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, size_t lds, hipStream_t s, A&&... args) {
    return KernelCall<P...>::go(kernel, grid, block, lds, s, std::forward<A>(args)...);
}

// Per-tile arrival counters sit at the start of every non-empty workspace,
// whatever the shape, so that a workspace reused across shapes never has
// partials or activation codes written over a counter.
constexpr size_t kCounterBytes = 16384;
constexpr int kMaxCounters = (int)(kCounterBytes / 4);

// Everything a GEMM call needs: its pointers, shape and derived layout.  The
// host builds it once per prepared call; the launches pass the kernels the
// few scalars they take from it, and the GEMM kernel rebuilds the rest from
// those scalars in a local copy.  The MFMA's first operand is the weight tile
// (rows = N), the second the activation tile (rows = M), so each lane's 16
// outputs are runs of 4 consecutive n for one m.
struct GemmParams {
    const uint16_t* A;        // bf16 activations [M, lda] (quantised in the GEMM when fused)
    int lda;
    uint32_t a_bytes;         // bytes of A a buffer load may touch: M * lda * 2
    const uint8_t* aop;       // activations quantised into the packed layout (not fused)
    uint32_t aop_bytes;
    uint32_t a_code_bytes;
    const uint8_t* bp;        // packed weight
    uint32_t bp_bytes;
    uint32_t b_code_bytes;
    int KS, KW;               // K steps of 64 and scale words of 4 steps (A and B alike)
    int M, N, K;
    int RBm, RBn;             // 32-row blocks of M and N
    int mtiles, ntiles;       // workgroup tiles along M and N
    int splits;               // workgroups along K
    int steps_per_split;      // K steps per split
    uint16_t* C;              // bf16 output [M, ldc]
    int ldc;
    int c_vec;                // 1 when rows of C are 8-byte aligned (ldc % 4 == 0)
    float* partial;           // fp32 partials [splits, M, ldp] when splits > 1, else null
    uint32_t partial_bytes;   // bytes of that region (< 2^31)
    int ldp;
    uint32_t* counters;       // per-tile arrival counters (zero between calls) when the
                              // last-arriving workgroup sums the partials, else null
};

// mb: 32-row M blocks per wave; nb: 32-row N blocks per wave; wn x wk waves
// per workgroup (wn along N, wk along K); splits along K; amode: where the
// activation is quantised (kAm*, the same values as the public MX_AMODE_*);
// finish: with splits > 1, 1 = the last workgroup to arrive at a tile sums
// the partials, 0 = reduce_kernel does.
struct Plan {
    int mb, nb, wn, wk, splits, amode, finish;
};
constexpr int kAmLds = 0;        // by the workgroup, into LDS
constexpr int kAmPrequant = 1;   // by pack_kernel, into the workspace
constexpr int kAmDirect = 2;     // by each wave, in registers
constexpr int kAmBf16 = 3;       // not at all: bf16 A x dequantised B (the a16wfp4 product)
constexpr int kAmStream = 4;     // by each wave, in registers, in a K loop (gemm_stream_kernel)
constexpr int kAmShared = 5;     // by quantiser waves into LDS, for MFMA waves (gemm_shared_kernel)
constexpr int kAmTile = 6;       // by pack_kernel, into the workspace; K-looped LDS-tiled GEMM (gemm_tile_kernel)
// the modes whose GEMM reads A pre-quantised by pack_kernel
constexpr bool amode_prequantises(int amode) { return amode == kAmPrequant || amode == kAmTile; }

bool gemm_plan_supported(const Plan& p);
int gemm_kr_for(int steps_per_wave);   // K-step budget KR of the kernel for that many steps (0: none)
size_t gemm_lds_bytes(const Plan& plan, int steps_per_split);
// The GEMM kernels take the call as thirteen scalar arguments (72 bytes of
// argument segment): the activation source (A, or the pre-quantised operand
// in the workspace), bp, C, partial, lda, ldc, M, N, K, steps_per_split --
// the first 14 SGPRs -- then what only the last-arrival split-K finish reads:
// counters, splits, mtiles.  The kernel sources are compiled with
// -amdgpu-kernarg-preload-count=14, so the dispatcher places the first ten in
// SGPRs at wave launch and the first loads wait on no scalar-memory round
// trip to the argument segment; everything else the kernel needs is derived
// from them.  A short argument segment also keeps the host's launch cheap:
// the runtime writes it to device memory on every launch.
typedef void (*GemmKernelFn)(const void*, const uint8_t*, uint16_t*, float*, int, int, int, int, int, int, uint32_t*,
                             int, int);

// A resolved GEMM launch: kernel, grid, block and dynamic LDS for a plan.
struct GemmLaunch {
    GemmKernelFn fn;
    unsigned gx, gy, gz, block;
    size_t lds;
    bool prequant;   // the activation source is the pre-quantised operand
    int steps_arg;   // the kernel's steps-per-split argument (with the shared mode's placement code)
};
bool resolve_gemm(const Plan& plan, const GemmParams& p, GemmLaunch* out);
// The K-looped kernels of the stream mode (mx4_stream.hip): one M block and
// one wave along N per workgroup (mb = wn = 1), nb in {1, 2, 4}, wk in
// {1, 2, 4, 8, 16} (nb <= 2 at 16 waves), rq activation row chunks per step.
GemmKernelFn find_stream_kernel(const Plan& plan, int rq);
size_t stream_lds_bytes(const Plan& plan);
// The kernels of the shared mode (mx4_shared.hip): plan.wn MFMA waves of
// plan.nb N blocks each and plan.wk quantiser waves per workgroup (mb = 1),
// (nb, wn, wk) in {(1, 2, 2), (1, 3, 4), (1, 3, 8), (1, 4, 4), (1, 4, 8),
// (2, 2, 2), (2, 4, 4)}, at most 24
// K steps per split (16 with nb = 2); no last-arrival finish.
GemmKernelFn find_shared_kernel(const Plan& plan, int steps_per_split);
size_t shared_lds_bytes(const Plan& plan, int steps_per_split);
// The K-looped tiled kernels of the tile mode (mx4_tile.hip): a workgroup
// tile of plan.mb x plan.nb blocks over the whole of K, plan.wk waves along
// M and plan.wn along N, (mb, nb, wk, wn) in {(8, 8, 2, 4), (4, 8, 2, 2),
// (8, 4, 2, 2), (4, 4, 2, 2), (4, 4, 2, 4), (2, 2, 2, 2)}; splits 1.  The
// ring has 8 stages, or 16 for the 64 x 64 tile on a grid of at most 256
// workgroups (tile_stages); the one-argument forms are the 8-stage kernels.
int tile_stages(const Plan& plan, long long wgs);
GemmKernelFn find_tile_kernel(const Plan& plan, int stages);
GemmKernelFn find_tile_kernel(const Plan& plan);
size_t tile_lds_bytes(const Plan& plan, int stages);
size_t tile_lds_bytes(const Plan& plan);
// Tile-mode workgroups one XCD runs at once: its 32 CUs each hold as many
// as their 160 KiB of LDS and 32 wave slots allow (one 256 x 256 or
// 256 x 128 tile, two 128 x 128, four 64 x 64).
inline int tile_wgs_per_xcd(size_t lds_bytes, int waves) {
    const int by_lds = (int)((160u * 1024u) / (lds_bytes > 0 ? lds_bytes : 1));
    const int by_waves = 32 / (waves > 0 ? waves : 1);
    const int per_cu = by_lds < by_waves ? by_lds : by_waves;
    return 32 * (per_cu > 1 ? per_cu : 1);
}

// Placement of the shared kernel's tiles on the 8 XCDs.  The dispatcher
// hands the workgroups of a grid, in x-major order, to XCD (linear id mod 8),
// and each XCD's L2 fetches every activation row block and weight column
// block its workgroups touch.  A one-split grid of mtiles x ntiles
// workgroups is laid out so that the workgroups of one XCD take a rectangle
// of a M tiles x b N tiles (a b = tiles / 8), the rectangle that costs the
// fewest fetched bytes: a * a_tile_bytes of activation plus b * b_tile_bytes
// of weight (the shared mode: 32 bf16 rows, 64 K bytes, and `cols` packed
// weight columns, cols (K / 2 + K / 32) bytes; the tile mode: packed
// operands on both sides).  a and mtiles / a are powers of two (the kernel
// decodes with shifts).
// shared_xcd_map returns the placement code: 0 when no rectangle fits (the
// dispatcher's order), else 1 + la + 16 lmg with a = 2^la M tiles per XCD
// and 2^lmg groups of M tiles.  It reaches the kernel in bits 8 and up of
// its steps-per-split argument (a shared-mode split has at most 24 steps),
// which is among the preloaded arguments: the first loads' addresses wait
// on no argument-segment read.
// With conc > 0, an XCD runs at most conc workgroups at once, in rounds of
// conc consecutive ones: its rectangle is then scored by the fetches of its
// rounds, each round covering min(a, conc) M tiles x ceil(conc / a) N tiles
// (the decode below walks M fastest).
inline int shared_xcd_map(int mtiles, int ntiles, int splits, double a_bytes, double b_bytes, int conc = 0) {
    if (splits != 1 || mtiles < 1 || ntiles < 1 || ((long long)mtiles * ntiles) % 8 != 0) return 0;
    int best = 0;
    double best_cost = 0.0;
    for (int lmg = 0; lmg <= 3; ++lmg) {
        const int mg = 1 << lmg, ng = 8 >> lmg;   // M groups x N groups = 8 XCDs
        if (mtiles % mg != 0 || ntiles % ng != 0) continue;
        const int a = mtiles / mg, b = ntiles / ng;
        if ((a & (a - 1)) != 0) continue;
        int la = 0;
        while ((1 << la) < a) ++la;
        double cost = a * a_bytes + b * b_bytes;
        if (conc > 0 && (long long)a * b > conc) {
            const double rounds = (double)a * b / conc;
            const int ra = a < conc ? a : conc, rb = (conc + a - 1) / a;
            cost = rounds * (ra * a_bytes + rb * b_bytes);
        }
        if (best == 0 || cost < best_cost) {
            best = 1 + la + 16 * lmg;
            best_cost = cost;
        }
    }
    return best;
}

// The tile mode adds one more placement, which fits any grid: XCD x takes a
// run of consecutive tiles in M-fastest order (tile t being M tile
// t mod mtiles, N tile t / mtiles), runs of ceil or floor of tiles / 8 in XCD
// order.  It wins where the tile count does not split into good rectangles
// (33 N tiles of 64 columns at N = 2112 leave only 1 x 33 per XCD, every XCD
// reading all of the weight).
constexpr int kXcdRuns = 128;   // placement code of the runs

// Tile (mt, nt) of workgroup (bx, by) of an ntiles x mtiles grid under
// placement code xcd_map (for the runs: T = mtiles ntiles tiles, q = T / 8,
// r = T mod 8; XCD x = lin mod 8 starts its run at tile x q + min(x, r) and
// takes tile j = lin / 8 of it); for the rectangles:
// the workgroups with linear id lin = bx + ntiles by, x = lin mod 8 and
// j = lin / 8 take M tile (x mod 2^lmg) 2^la + (j mod 2^la) and N tile
// (x / 2^lmg) b + j / 2^la, b = ntiles / 2^(3 - lmg) N tiles per XCD.
__host__ __device__ inline void shared_tile_of(int bx, int by, int ntiles, int mtiles, int xcd_map, int& mt,
                                               int& nt) {
    if (xcd_map == 0) {
        mt = by;
        nt = bx;
        return;
    }
    if (xcd_map == kXcdRuns) {
        const int lin = bx + ntiles * by, tiles = ntiles * mtiles;
        const int x = lin & 7, q = tiles >> 3, r = tiles & 7;
        const int t = x * q + (x < r ? x : r) + (lin >> 3);
        mt = t % mtiles;
        nt = t / mtiles;
        return;
    }
    const int la = (xcd_map - 1) & 15, lmg = (xcd_map - 1) >> 4;
    const int lin = bx + ntiles * by;
    const int x = lin & 7, j = lin >> 3;
    const int b = ntiles >> (3 - lmg);
    mt = ((x & ((1 << lmg) - 1)) << la) + (j & ((1 << la) - 1));
    nt = (x >> lmg) * b + (j >> la);
}

// Fetches of a placement, counted: over each XCD's workgroups in dispatch
// order, in rounds of conc (all of them when conc is 0), the distinct M tiles
// of a round times a_bytes plus its distinct N tiles times b_bytes.
inline double xcd_fetch_cost(int mtiles, int ntiles, int xcd_map, int conc, double a_bytes, double b_bytes) {
    const int tiles = mtiles * ntiles;
    std::vector<long long> seen_m((size_t)mtiles, -1), seen_n((size_t)ntiles, -1);
    double cost = 0.0;
    for (int x = 0; x < 8; ++x)
        for (int lin = x, j = 0; lin < tiles; lin += 8, ++j) {
            const long long stamp = (long long)x * tiles + (conc > 0 ? j / conc : 0);
            int mt, nt;
            shared_tile_of(lin % ntiles, lin / ntiles, ntiles, mtiles, xcd_map, mt, nt);
            if (seen_m[mt] != stamp) cost += a_bytes, seen_m[mt] = stamp;
            if (seen_n[nt] != stamp) cost += b_bytes, seen_n[nt] = stamp;
        }
    return cost;
}

// When the tile mode may place runs: never (0), in place of the dispatcher's
// order or of a rectangle (1), or only in place of a rectangle (2).  Measured
// in one process against the same library without the runs, over 112
// tile-mode shapes whose placement they change, the runs were 7 % faster
// on average (geometric mean) on the 64 x 64 tile at K = 2048, 6 % at 4096,
// 2 % at 7168, with single shapes up to 13 % slower at 7168 where they
// replaced the dispatcher's order; on the 128 x 128 tile 2 % faster at
// K = 2048 and neutral past it; on the larger tiles neutral to 5 % slower.
enum { kRunsNever = 0, kRunsAny = 1, kRunsForRect = 2 };
inline int tile_runs_policy(int mb, int nb, int K) {
    if (mb == 2 && nb == 2) return K <= 4096 ? kRunsAny : kRunsForRect;
    return mb == 4 && nb == 4 && K <= 2048 ? kRunsAny : kRunsNever;
}

// The tile mode's placement code: the best rectangle (shared_xcd_map), or the
// runs where the policy allows them and they fetch less.  Up to 2^16 tiles
// both are counted by xcd_fetch_cost; past that the runs are taken only where
// no rectangle fits (and the policy allows that).
inline int tile_xcd_map(int mtiles, int ntiles, double a_bytes, double b_bytes, int conc, int policy) {
    if (mtiles < 1 || ntiles < 1) return 0;
    const int rect = shared_xcd_map(mtiles, ntiles, 1, a_bytes, b_bytes, conc);
    if (policy == kRunsNever || (policy == kRunsForRect && rect == 0)) return rect;
    const long long tiles = (long long)mtiles * ntiles;
    if (tiles <= (1 << 16))
        return xcd_fetch_cost(mtiles, ntiles, kXcdRuns, conc, a_bytes, b_bytes) <
                       xcd_fetch_cost(mtiles, ntiles, rect, conc, a_bytes, b_bytes)
                   ? kXcdRuns
                   : rect;
    return rect == 0 ? kXcdRuns : rect;
}

hipError_t launch_gemm(const GemmLaunch& gl, const GemmParams& p, hipStream_t s);
hipError_t launch_reduce(const GemmParams& p, hipStream_t s);

hipError_t launch_quant_natural(const uint16_t* x, int rows, int K, int ld, uint8_t* codes, uint8_t* scales,
                                hipStream_t s);
hipError_t launch_pack(const uint16_t* x, int rows, int K, int ld, uint8_t* packed, hipStream_t s);
hipError_t launch_import(const uint8_t* codes, const uint8_t* scales, int rows, int K, uint8_t* packed,
                         hipStream_t s);
hipError_t launch_unpack(const uint8_t* packed, int rows, int K, uint8_t* codes, uint8_t* scales, hipStream_t s);

}  // namespace mx4
