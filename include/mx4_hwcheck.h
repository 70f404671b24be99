/*
 * mx4_hwcheck.h -- one-wave checks of the gfx950 instructions the MXFP4 path
 * is built on (libmx4hw.so).  Test infrastructure only: the product library
 * libmx4.so does not contain or call these.  Each kernel goes through the
 * same device wrappers as the GEMM and quantisation kernels, so a test can
 * compare the instructions' results with a host model element by element.
 *
 * Except in mxhw_xcd_map (host only), all pointers are device pointers; each
 * call enqueues one launch on `stream` (a hipStream_t, NULL for the default
 * stream) and returns 0, or -1 for a bad size or null pointer, -2 for a
 * misaligned pointer, -4 when the launch failed.  Nothing is allocated.
 */
#ifndef MX4_HWCHECK_H
#define MX4_HWCHECK_H

#ifdef __cplusplus
extern "C" {
#endif

/* e2m1 codes of n bf16 values (n % 8 == 0, finite, x_dev 16-byte aligned)
 * under the scale operand of every scale byte 0 .. bytes-1 (bytes <= 255):
 * codes_dev receives bytes * n / 2 bytes, row b holding the codes of x under
 * byte b, two per byte with element 2j in the low nibble -- the conversion
 * (v_cvt_scalef32_pk_fp4_bf16) the quantisers of the MXFP4 rule use. */
int mxhw_cvt_fp4(const void* x_dev, int n, int bytes, void* codes_dev, void* stream);

/* All 16 e2m1 codes widened to bf16 times 2^(byte-127) for every scale
 * byte 0 .. bytes-1 (v_cvt_scalef32_pk_bf16_fp4, as the a16wfp4 product
 * widens its weight): out_dev receives bytes x 16 bf16, 16-byte aligned. */
int mxhw_widen_fp4(int bytes, void* out_dev, void* stream);

/* One block-scaled fp4 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, both
 * operands e2m1) from a zero accumulator on one wave: lane L passes the 16
 * bytes a_dev[16L..16L+15] and b_dev[16L..16L+15] as its first and second
 * operand fragments and the 32-bit words sa_dev[L] and sb_dev[L] as its
 * scale registers; out_dev[16L + e] receives element e of lane L's
 * accumulator (fp32, 64 x 16). */
int mxhw_mfma_fp4(const void* a_dev, const void* b_dev, const void* sa_dev, const void* sb_dev,
                  void* out_dev, void* stream);

/* Measurement reference, no arithmetic: `wgs` workgroups of `waves` waves;
 * workgroup g reads bytes [g*stride, g*stride + chunk) of buf_dev (clipped at
 * `bytes`, < 2^31; chunk > 0, chunk % 16 == 0) with 128-bit non-temporal
 * buffer loads, lpl (1, 2, 4, 8 or 16) in flight per lane, starting at byte
 * (g*rot) % chunk of its piece and wrapping (rot % 16 == 0), and stores one
 * xor dword per wave to out_dev[g*waves + wave].  stride = chunk streams
 * disjoint pieces (HBM); stride = 0 has every workgroup read the same piece
 * (L2). */
int mxhw_stream_read(const void* buf_dev, unsigned bytes, int wgs, int waves, int lpl,
                     unsigned chunk, unsigned stride, unsigned rot, void* out_dev, void* stream);

/* Host only, no GPU call: the placement of the GEMM's workgroup tiles on
 * the 8 XCDs (shared and tile modes), by the library's own code.  For a
 * one-split grid of mtiles x ntiles workgroups (at most 2^20) whose M tile
 * costs an XCD's L2 a_tile_bytes of fetch and whose N tile b_tile_bytes,
 * with at most `conc` workgroups of an XCD running at once (0: all of them),
 * and with runs = 0 (the shared mode), 1 or 2 for whether each XCD may
 * instead take a run of consecutive tiles in M-fastest order (placement code
 * 128): never, in place of the dispatcher's order or of a rectangle, or only
 * in place of a rectangle (the tile mode picks 1 or 2 by tile and K),
 * *map_out receives the placement code the kernel gets, and
 * mt_out[lin] and nt_out[lin] (host arrays of mtiles * ntiles ints) the M and
 * N tile of the workgroup with linear id lin = bx + ntiles * by.  Returns 0,
 * or -1 for a bad size, byte count, runs value or null pointer. */
int mxhw_xcd_map(int mtiles, int ntiles, int splits, double a_tile_bytes, double b_tile_bytes, int conc, int runs,
                 int* map_out, int* mt_out, int* nt_out);

#ifdef __cplusplus
}
#endif

#endif /* MX4_HWCHECK_H */
