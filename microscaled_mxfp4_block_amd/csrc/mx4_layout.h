// mx4_layout.h -- geometry of the packed MXFP4 operand layout (host and device).
//
// The GEMM contracts on the gfx950 block-scaled MFMA
// v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in e2m1 (fp4).  For that
// instruction one operand tile is 32 rows x 64 K: lane L (0..63) supplies row
// L % 32 and the 32-element K group L / 32 of the step, as 16 bytes (two
// codes per byte, even k in the low nibble), plus one e8m0 byte for its group.
//
// The packed layout stores every operand tile as the exact 1 KiB its wave
// loads -- lane L's 16 bytes at offset 16 * L -- so a wave fetches a tile with
// one fully coalesced 128-bit load per lane and never permutes in registers:
//
//   codes : tile (rb, t) at ((rb * KS + t) * 64 + L) * 16 bytes
//           rb = row block (32 rows), t = K step (64 K), L = lane;
//           lane L holds row 32 rb + L % 32, group g = 2 t + L / 32.
//   scales: word (rb, w) at codes_bytes + ((rb * KW + w) * 64 + L) * 4,
//           byte b (0..3) of the word is the e8m0 byte of row 32 rb + L % 32
//           in K step t = 4 w + b (group 2 t + L / 32).
//
// Rows past the matrix and K groups past K are zero codes with scale byte 0
// (2^-127), as are the scale bytes of steps past the last one in its word.
// The same layout carries the packed weight B (rows = N) and the quantised
// activation operand A (rows = M) in the workspace.
#pragma once

#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define MX4_HD __host__ __device__
#else
#define MX4_HD
#endif

namespace mx4 {

constexpr int kGroup = 32;        // elements per e8m0 scale
constexpr int kStepK = 64;        // K per MFMA step (two groups)
constexpr int kRowBlock = 32;     // rows per operand tile
constexpr int kTileBytes = 1024;  // 64 lanes x 16 bytes
constexpr int kStepsPerWord = 4;  // K steps sharing one scale word per lane

struct OperandGeom {
    int rows;        // logical rows (N for B, M for A)
    int K;           // logical K (multiple of 32)
    int RB;          // row blocks of 32
    int KS;          // K steps of 64
    int KW;          // scale words per lane per row block
    size_t code_bytes;
    size_t scale_bytes;
    size_t total_bytes;
};

MX4_HD inline OperandGeom operand_geom(int rows, int K) {
    OperandGeom g;
    g.rows = rows;
    g.K = K;
    g.RB = (rows + kRowBlock - 1) / kRowBlock;
    g.KS = (K + kStepK - 1) / kStepK;
    g.KW = (g.KS + kStepsPerWord - 1) / kStepsPerWord;
    g.code_bytes = (size_t)g.RB * g.KS * kTileBytes;
    g.scale_bytes = (size_t)g.RB * g.KW * 64 * 4;
    g.total_bytes = g.code_bytes + g.scale_bytes;
    return g;
}

}  // namespace mx4
