// mamba_gemm.h -- bf16 MFMA GEMM for gfx950 used by the projections of a Mamba block.
//
// C[b] (M x N) = A (M x K) * B[b] (K x N), bf16 inputs, fp32 accumulation, bf16 outputs
// (round to nearest even).  A is row-major with K contiguous (a weight matrix).  B is either
// K-contiguous (B(k, n) at B[n*ldb + k]: token-major activations) or N-contiguous
// (B(k, n) at B[k*ldb + n]: channel-major activations).  Output rows are routed to up to three
// destinations by row range, each stored row-major or transposed, so a projection can write
// exactly the layouts its consumers read.
#pragma once
#include "mamba_common.h"

namespace mamba {

struct GemmDest {
  uint16_t* ptr;     // bf16 output; NULL: rows [m0, m1) are not stored
  int64_t m0, m1;    // rows [m0, m1) of C go here (row index taken relative to m0)
  int64_t ld;        // leading dimension in elements
  int64_t bstride;   // batch stride in elements
  int32_t trans;     // 0: C(m, n) at (m - m0) * ld + n;  1: at n * ld + (m - m0)
};

struct GemmArgs {
  const uint16_t* A;
  const uint16_t* B;
  int64_t lda, ldb, b_bstride;
  int64_t M, N, K;
  int32_t mtiles, ntiles, ndst;
  int64_t batch;
  GemmDest dst[3];
  // split-K (register-staged kernel only): workgroup s of ksplit covers K range
  // [s kchunk, min(K, (s + 1) kchunk)) and writes fp32 partials to part (ksplit, batch, M, N);
  // ksplit <= 1: one pass, bf16 results straight to the destinations
  int32_t ksplit;
  int64_t kchunk;
  float* part;
};

// Shape rules the kernels rely on (gemm_check, on the host): M % 16 == 0, N % 8 == 0,
// K % 8 == 0, lda and ldb multiples of 8, A and B 16-byte aligned, destination row ranges on
// multiples of 16; a transposed destination needs ld % 4 == 0 and an 8-byte aligned pointer
// (it stores 4 consecutive rows as one 8-byte word).
__attribute__((visibility("hidden"))) int gemm_check(const GemmArgs& a);
__attribute__((visibility("hidden"))) int launch_gemm(const GemmArgs& a, bool b_kcontig,
                                                      int64_t batch, hipStream_t s);
// Split-K for calls with too few output tiles to fill the GPU (long K, small M x N): the number
// of splits launch_gemm_split will use, the fp32 workspace it needs, and the launch (the split
// pass, then a deterministic reduction that sums the splits in order, rounds to bf16 and routes
// rows to the destinations).  Falls back to launch_gemm when one split is chosen.
__attribute__((visibility("hidden"))) int gemm_split_factor(const GemmArgs& a, int64_t batch);
__attribute__((visibility("hidden"))) size_t gemm_split_bytes(const GemmArgs& a, int64_t batch);
__attribute__((visibility("hidden"))) int launch_gemm_split(const GemmArgs& a, bool b_kcontig,
                                                            int64_t batch, float* part,
                                                            size_t part_bytes, hipStream_t s);

}  // namespace mamba
