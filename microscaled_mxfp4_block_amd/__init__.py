"""MI355X-native MXFP4 GEMM: C[M,N] (bf16) = A[M,K] x B[N,K]^T with on-the-fly
activation quantisation, behind the C ABI declared in include/mx4.h."""
