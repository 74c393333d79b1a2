// tile_fp32.h -- float32 4 x 4 register tiles of 64 x 64 products with
// operands in LDS or global memory (256 threads: thread t owns rows
// t/16 + 16 r and columns t%16 + 16 s).  Used by the prefill alignment and
// the backward pass, whose per-chunk algebra runs in float32 on the vector
// units.
#pragma once

namespace pathattn {

// acc[r][s] += sum_k A(r0 + 16 r, k) B(k, c0 + 16 s) over k < K for one
// thread's 4 x 4 tile of a 64 x 64 output block, operands in LDS with
// arbitrary row / column strides (so transposed reads need no copy).  Rows of
// the tile are 16 apart and columns 16 apart: a wave's lanes read 4 distinct
// A addresses and 16 consecutive B addresses per instruction.
template <int K>
__device__ __forceinline__ void tile_mm(float (&acc)[4][4], const float *A, int a_rs, int a_cs,
                                        const float *B, int b_rs, int b_cs, int r0, int c0) {
  for (int kk = 0; kk < K; ++kk) {
    float a[4], b[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = A[(r0 + 16 * r) * a_rs + kk * a_cs];
#pragma unroll
    for (int c = 0; c < 4; ++c) b[c] = B[kk * b_rs + (c0 + 16 * c) * b_cs];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[r][c] = __builtin_fmaf(a[r], b[c], acc[r][c]);
  }
}

__device__ __forceinline__ void tile_zero(float (&acc)[4][4]) {
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;
}

}  // namespace pathattn
