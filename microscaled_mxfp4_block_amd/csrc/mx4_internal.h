// mx4_internal.h -- host-side declarations shared by the library's sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "mx4_layout.h"

namespace mx4 {

// Arguments of the GEMM kernel.  Operands follow the packed layout of
// mx4_layout.h: the MFMA's first operand is the weight tile (rows = N), the
// second the activation tile (rows = M), so each lane's 16 outputs are runs
// of 4 consecutive n for one m.
struct GemmParams {
    const uint16_t* A;        // bf16 activations [M, lda] (quantised in-kernel)
    int lda;
    const uint8_t* aop;       // quantised activations in packed layout (no in-kernel quant)
    size_t a_code_bytes;
    const uint8_t* bp;        // packed weight
    size_t b_code_bytes;
    int KS, KW;               // K steps of 64 and scale words of 4 steps (shared by A and B)
    int M, N, K;
    int RBm, RBn;             // 32-row blocks of M and N
    int mtiles, ntiles;       // tiles of MBLK / NBLK row blocks
    int splits;               // workgroups along K
    int steps_per_split;      // K steps per split
    uint16_t* C;              // bf16 output [M, ldc]
    int ldc;
    int c_vec;                // 1 when rows of C are 8-byte aligned (ldc % 4 == 0)
    float* partial;           // fp32 partials [splits, M, ldp] when splits > 1
    int ldp;
};

struct Plan {
    int mb, nb, wk, splits, fuse;
};

// Returns false when no kernel is instantiated for this plan.
bool gemm_plan_supported(const Plan& p);
hipError_t launch_gemm(const Plan& plan, const GemmParams& p, hipStream_t s);
hipError_t launch_reduce(const float* partial, int splits, int M, int N, int ldp, uint16_t* C, int ldc,
                         int c_vec, hipStream_t s);

hipError_t launch_quant_natural(const uint16_t* x, int rows, int K, int ld, uint8_t* codes, uint8_t* scales,
                                hipStream_t s);
hipError_t launch_pack(const uint16_t* x, int rows, int K, int ld, uint8_t* packed, hipStream_t s);
hipError_t launch_unpack(const uint8_t* packed, int rows, int K, uint8_t* codes, uint8_t* scales, hipStream_t s);

}  // namespace mx4
