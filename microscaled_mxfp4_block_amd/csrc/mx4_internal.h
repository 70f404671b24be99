// mx4_internal.h -- host-side declarations shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mx4_layout.h"

namespace mx4 {

// Largest number of K steps one wave holds in registers (its whole share of
// a split); the planner splits K further when a shape needs more.
constexpr int kStepsPerWaveMax = 8;
// Largest LDS block the planner gives a workgroup.
constexpr size_t kLdsBudget = 64 * 1024;
// The workspace starts with a fixed region of per-tile arrival counters that
// no shape ever uses for anything else, so counters left at zero by one call
// are zero for the next call whatever its shape; split-K plans are limited to
// this many output tiles.
constexpr size_t kCounterRegionBytes = 64 * 1024;
constexpr int kMaxSplitTiles = (int)(kCounterRegionBytes / sizeof(int));

// Arguments of the GEMM kernel.  The MFMA's first operand is the weight tile
// (rows = N), the second the activation tile (rows = M), so each lane's 16
// outputs are runs of 4 consecutive n for one m.
struct GemmParams {
    const uint16_t* A;        // bf16 activations [M, lda], quantised in the kernel
    int lda;
    const uint8_t* bp;        // packed weight
    size_t b_code_bytes;
    int KS, KW;               // K steps of 64 and scale words of 4 steps
    int M, N, K;
    int RBm, RBn;             // 32-row blocks of M and N
    int mtiles, ntiles;       // workgroup tiles along M and N
    int splits;               // workgroups along K
    int steps_per_split;      // K steps per split
    uint16_t* C;              // bf16 output [M, ldc]
    int ldc;
    int c_vec;                // 1 when rows of C are 8-byte aligned (ldc % 4 == 0)
    float* partial;           // fp32 partials [splits, M, ldp] when splits > 1
    int ldp;
    int* counters;            // per-tile arrival counters (zero between calls)
};

// mb: 32-row M blocks per workgroup; nb: 32-row N blocks per wave;
// wn x wk waves per workgroup (wn along N, wk along K); splits along K.
struct Plan {
    int mb, nb, wn, wk, splits;
};

bool gemm_plan_supported(const Plan& p);
size_t gemm_lds_bytes(const Plan& plan, int steps_per_split);
hipError_t launch_gemm(const Plan& plan, const GemmParams& p, hipStream_t s);

hipError_t launch_quant_natural(const uint16_t* x, int rows, int K, int ld, uint8_t* codes, uint8_t* scales,
                                hipStream_t s);
hipError_t launch_pack(const uint16_t* x, int rows, int K, int ld, uint8_t* packed, hipStream_t s);
hipError_t launch_unpack(const uint8_t* packed, int rows, int K, uint8_t* codes, uint8_t* scales, hipStream_t s);

}  // namespace mx4
