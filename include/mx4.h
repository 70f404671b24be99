/*
 * mx4.h -- C ABI of an MI355X (gfx950) MXFP4 GEMM library.
 *
 *   C[M,N] (bf16) = A[M,K] (bf16, quantised per call to MXFP4) x B[N,K]^T
 *                   (bf16, quantised once to MXFP4 and packed).
 *
 * MXFP4 here is the block format of the kernelindex.com amd-mxfp4-mm pages
 * (MI355X leaderboard submissions 748756, 721672, 754569, 755056, 733989):
 * 32 consecutive K elements of one row share one e8m0 scale byte, each element
 * is a 4-bit e2m1 code.  The quantisation rule is the one of submission 755056,
 * section "Software MXFP4 quant":
 *   amax = max |x| of the group (fp32);
 *   R    = (bits(amax) + 0x00200000) & 0xFF800000   (power of two);
 *   s    = clamp(E(R) - 129, -127, 127), scale byte = s + 127;
 *   code = e2m1(x * 2^-s), round to nearest even, |q| >= 6 -> 6, sign kept.
 * Natural layouts (as in submission 721672, "Quant kernel for Triton/splitK
 * path"): codes [rows, K/2] bytes, element 2j in the low nibble of byte j;
 * scales [rows, K/32] bytes, group g covers k in [32g, 32g+32).
 *
 * Conventions for every entry point (those of the C launcher on submission
 * 755056's page, quant_and_ck_gemm: an int status, buffers and scratch owned
 * by the caller, work launched asynchronously on the caller's queue):
 *   - bf16 is passed as raw 16-bit patterns; matrices are row-major with an
 *     explicit leading dimension in elements.
 *   - Pointers named *_dev are device pointers (hipMalloc or torch CUDA
 *     tensors); *_host pointers are host memory.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     synchronises; each call only enqueues work on `stream` (a hipStream_t,
 *     NULL for the default stream) and returns.  (mx_gemm_noalloc, for
 *     callers that cannot allocate, uses a static device array of the
 *     library instead of a caller's workspace.)
 *   - Arguments are validated on the host before any HIP call; on error the
 *     call returns a negative MX_E* code, enqueues nothing and writes nothing.
 *   - Device pointers read with 128-bit loads must be 16-byte aligned (bf16
 *     inputs A and B, with lda / ldb multiples of 8), the packed weight
 *     16-byte aligned, the workspace 256-byte aligned, C 2-byte aligned (C is
 *     written with 16-byte stores when it is 16-byte aligned and ldc % 8 == 0,
 *     with narrower stores otherwise).
 *   - Inputs must be finite; NaN or Inf inputs give unspecified codes.
 *   - Calls on different streams with disjoint output and workspace buffers
 *     may run concurrently, from any threads.  The library's only state is a
 *     small per-thread cache of prepared calls (shape, plan, kernel and grid;
 *     no buffers), so a repeated mx_gemm call only checks its pointers and
 *     launches.
 */
#ifndef MX4_H
#define MX4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MX_OK = 0,
    MX_EINVAL = -1,   /* bad shape or leading dimension (M, N, K <= 0, K % 32 != 0, ld too small) */
    MX_EALIGN = -2,   /* null or misaligned pointer */
    MX_ESPACE = -3,   /* output, packed or workspace buffer too small */
    MX_EHIP = -4,     /* a HIP launch failed (the status hipLaunchKernel returned) */
    MX_EPLAN = -5     /* an explicit plan that the library cannot run for this shape */
};

/* Version of the packed-weight layout written by mx_pack_weight. */
#define MX_PACKED_LAYOUT_VERSION 1

/* Message for an MX_* code; never NULL. */
const char* mx_strerror(int code);

/* Size in bytes of the packed weight for an N x K matrix (host only, no HIP call).
 * The packed buffer is opaque: e2m1 codes in the GEMM's 32-row x 64-K operand
 * tiles (1 KiB, one 16-byte fragment per MFMA lane) followed by the e8m0
 * scales in 4-byte words per lane (4 K steps per word); rows are padded to a
 * multiple of 32 and K to a multiple of 64 with zero codes. */
int mx_packed_weight_bytes(int N, int K, size_t* bytes_host);

/* One-time weight packing: the MXFP4 rule above applied to B along K (the
 * weight is quantised the same way as the activation; on the pages the
 * harness hands B over already quantised and shuffled), written into the
 * GEMM's tile layout.
 *   B_dev       bf16 [N, K], row stride ldb elements (ldb >= K, ldb % 8 == 0,
 *               N * ldb * 2 < 2^31)
 *   packed_dev  output, packed_bytes >= mx_packed_weight_bytes(N, K), 16-B aligned */
int mx_pack_weight(const void* B_dev, int N, int K, int ldb,
                   void* packed_dev, size_t packed_bytes, void* stream);

/* Inverse view of a packed weight in the natural layouts (for tests and
 * export): codes_dev [N, K/2] bytes and scales_dev [N, K/32] bytes. */
int mx_unpack_weight(const void* packed_dev, int N, int K,
                     void* codes_dev, void* scales_dev, void* stream);

/* Import of a weight quantised elsewhere by the same MXFP4 rule: natural
 * e2m1 codes [N, K/2] (two per byte, even k in the low nibble; codes_dev
 * 16-byte aligned) and e8m0 scales [N, K/32] are moved unchanged into the
 * packed layout, with no re-quantisation; the exact inverse of
 * mx_unpack_weight on the bytes it covers.
 *   packed_dev  output, packed_bytes >= mx_packed_weight_bytes(N, K), 16-B aligned */
int mx_import_weight(const void* codes_dev, const void* scales_dev, int N, int K,
                     void* packed_dev, size_t packed_bytes, void* stream);

/* Stand-alone activation quantisation to the natural layouts (the rule
 * above; the standalone quantiser of submission 755056's page writes the
 * same codes and scales, in a shuffled scale layout).
 *   A_dev       bf16 [M, K], row stride lda (lda >= K, lda % 8 == 0)
 *   codes_dev   [M, K/2] bytes, scales_dev [M, K/32] bytes (dense) */
int mx_quant_act(const void* A_dev, int M, int K, int lda,
                 void* codes_dev, void* scales_dev, void* stream);

/* Workspace bytes mx_gemm needs for this shape under the library's plan
 * (0 when A is quantised inside the GEMM and K is not split).  A non-empty
 * workspace holds, in this order, 16 KiB of per-tile arrival counters, the
 * quantised activation operand and the fp32 partial sums of the K splits.
 * The counters must be zero before a workspace's first use (allocate it
 * zero-filled, or clear it once); every completed call leaves them zero, so
 * one workspace can serve any sequence of shapes on one stream. */
int mx_gemm_workspace_bytes(int M, int N, int K, size_t* bytes_host);

/* C = A x B^T with A quantised on the fly (quantisation, block-scaled MFMA
 * contraction with fp32 accumulation, split-K reduction when planned, bf16
 * round-to-nearest-even epilogue).  The contraction is the block-scaled dot
 * the pages write as tl.dot_scaled(a, a_scale, "e2m1", b, b_scale, "e2m1")
 * (submission 748756, kernel_fused_mxfp4_gemm): every product of two e2m1
 * values carries 2^(sa-127) * 2^(sb-127) of its two 32-element groups, and
 * the sum runs over all of K; here it runs on the gfx950 scaled MFMA
 * (v_mfma_scale_f32_32x32x64_f8f6f4).  The call only validates (host),
 * enqueues and returns; results land when the stream reaches them.  Errors:
 * MX_EINVAL (shape, lda or ldc), MX_EALIGN, MX_ESPACE (workspace too small),
 * MX_EHIP (a launch failed; earlier launches of the call may be enqueued).
 *   A_dev      bf16 [M, K], lda >= K, lda % 8 == 0, M * lda * 2 < 2^31
 *   packed_dev weight packed by mx_pack_weight for (N, K)
 *   C_dev      bf16 [M, N] output, ldc >= N
 *   ws_dev     workspace of ws_bytes >= mx_gemm_workspace_bytes(M, N, K),
 *              256-byte aligned (may be NULL when that is 0), zero-filled
 *              before its first use (see mx_gemm_workspace_bytes).  Calls
 *              that overlap in time (other streams) need separate
 *              workspaces.
 * Launches per call: 1 (A quantised inside the GEMM), +1 for the quantisation
 * kernel when the plan's amode is MX_AMODE_PREQUANT or MX_AMODE_TILE, +1 for the split-K
 * reduction when splits > 1 and the plan's finish is MX_FINISH_KERNEL.
 * Either split-K finish sums the partials in split order: results do not
 * depend on timing. */
int mx_gemm(const void* A_dev, int M, int K, int lda,
            const void* packed_dev, int N,
            void* C_dev, int ldc,
            void* ws_dev, size_t ws_bytes, void* stream);

/* A launch plan: how mx_gemm tiles the problem.  Exposed so that callers can
 * inspect the plan chosen for a shape and tests can force alternatives.
 * A workgroup of wn x wk waves owns 32*mb rows of C and 32*nb*wn columns,
 * over K / splits of the reduction; its wk waves share that K range. */
typedef struct mx_plan {
    int mb;          /* 32-row blocks of M per wave (1 or 2); in
                        MX_AMODE_TILE per workgroup */
    int nb;          /* 32-column blocks of N per wave (1 or 2; 1, 2 or 4 in
                        MX_AMODE_STREAM); in MX_AMODE_TILE per workgroup */
    int wn;          /* waves along N per workgroup (1 or 2; up to 4 in
                        MX_AMODE_SHARED and MX_AMODE_TILE) */
    int wk;          /* waves along K per workgroup (1, 2, 4, 8 or 16; wn*wk <= 16);
                        in MX_AMODE_SHARED the quantiser waves, in
                        MX_AMODE_TILE the waves along M */
    int splits;      /* workgroups along K; > 1 adds a reduction kernel
                        unless finish is MX_FINISH_LAST_ARRIVAL */
    int amode;       /* where A is quantised: one of MX_AMODE_* */
    int finish;      /* who sums the split-K partials: one of MX_FINISH_* */
} mx_plan;

/* Activation modes of a plan. */
enum {
    MX_AMODE_LDS = 0,       /* each GEMM workgroup quantises its slice of A into
                               LDS, shared by its waves */
    MX_AMODE_PREQUANT = 1,  /* a first kernel quantises A into the workspace */
    MX_AMODE_DIRECT = 2,    /* each wave loads the A rows of the fragments it
                               consumes (through its own LDS tiles) and
                               quantises them in registers; no workgroup
                               barrier before the MFMAs */
    MX_AMODE_BF16 = 3,      /* A is NOT quantised: the a16wfp4 product of
                               mx_gemm_a16w4 (a different result) */
    MX_AMODE_STREAM = 4,    /* as MX_AMODE_DIRECT, but each wave loops over its
                               K steps with the loads of several steps in
                               flight (any K per wave; mb = wn = 1,
                               nb in {1, 2, 4}) */
    MX_AMODE_SHARED = 5,    /* wk quantiser waves per workgroup quantise its
                               32-row activation slice once into LDS for wn
                               MFMA waves of nb N blocks each, which hold the
                               weight of the whole K split in registers and
                               need no cross-wave reduction (mb = 1;
                               (nb, wn, wk) in {(1,2,2), (1,3,4), (1,3,8),
                               (1,4,4), (1,4,8), (2,2,2), (2,4,4)}; at most
                               24 K steps per split, 16 with nb = 2;
                               finish 0) */
    MX_AMODE_TILE = 6       /* a first kernel quantises A into the workspace;
                               the GEMM workgroup owns 32*mb x 32*nb of C over
                               its K split and loops over K with both
                               operands staged in LDS, wk waves along M and
                               wn along N (the MFMA-bound regime, M from
                               64 up; (mb, nb, wk, wn) in {(8,8,2,4),
                               (4,8,2,2), (8,4,2,2), (4,4,2,2), (4,4,2,4),
                               (2,2,2,2)}; splits start on a multiple of 4
                               K steps; finish 0) */
};

/* Split-K finishes of a plan (no effect when splits == 1). */
enum {
    MX_FINISH_KERNEL = 0,       /* a second kernel sums the partials */
    MX_FINISH_LAST_ARRIVAL = 1  /* the last GEMM workgroup to finish a tile
                                   sums them (at most 4096 output tiles) */
};

/* The plan mx_gemm uses for (M, N, K) (host only). */
int mx_gemm_plan(int M, int N, int K, mx_plan* plan_host);

/* Workspace bytes for an explicit plan. */
int mx_gemm_plan_workspace_bytes(const mx_plan* plan_host, int M, int N, int K,
                                 size_t* bytes_host);

/* mx_gemm under an explicit plan (MX_EPLAN when the plan is not supported). */
int mx_gemm_with_plan(const void* A_dev, int M, int K, int lda,
                      const void* packed_dev, int N,
                      void* C_dev, int ldc,
                      void* ws_dev, size_t ws_bytes,
                      const mx_plan* plan_host, void* stream);

/* The a16wfp4 product (the pages' route for small M: submission 733989,
 * routing notes, "bf16 A x fp4 B"): C = A x dequant(B)^T with A's bf16
 * values used as they are, B packed by mx_pack_weight (or imported), fp32
 * accumulation of exact bf16 x bf16 products on bf16 MFMAs, bf16
 * round-to-nearest-even.  This is a different function from mx_gemm, which
 * also quantises A.  Arguments, alignment, workspace rules and return codes
 * are those of mx_gemm; the plan has amode MX_AMODE_BF16. */
int mx_gemm_a16w4_plan(int M, int N, int K, mx_plan* plan_host);
int mx_gemm_a16w4_workspace_bytes(int M, int N, int K, size_t* bytes_host);
int mx_gemm_a16w4(const void* A_dev, int M, int K, int lda,
                  const void* packed_dev, int N,
                  void* C_dev, int ldc,
                  void* ws_dev, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * product, plan, arguments and return codes as mx_gemm, but with no
 * workspace argument: the workspace lives in a static device array of
 * MX_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends.  The call allocates and frees nothing.  On its first call on
 * a device (the one current on the calling thread, which must be the
 * stream's) it looks up that device's copy of the array and enqueues one
 * small kernel that zeroes its arrival counters.
 *   Returns MX_ESPACE when the shape's workspace (mx_gemm_workspace_bytes)
 * exceeds MX_NOALLOC_SCRATCH_BYTES, before any HIP call.
 *   Every call on one GPU shares that GPU's array, which keeps the last
 * call's contents: calls that may overlap in time on one GPU (other streams,
 * other threads) race on it and must be serialised by the caller. */
#define MX_NOALLOC_SCRATCH_BYTES (8u << 20)
int mx_gemm_noalloc(const void* A_dev, int M, int K, int lda,
                    const void* packed_dev, int N,
                    void* C_dev, int ldc, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MX4_H */
