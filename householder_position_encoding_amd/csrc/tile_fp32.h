// tile_fp32.h -- float32 products of 64 x 64 blocks for 256-thread blocks:
// 4 x 4 register tiles on the vector units (thread t owns rows t/16 + 16 r
// and columns t%16 + 16 s), and 32 x 32 tiles on the float32 matrix cores with
// operands staged through LDS panels; plus the blocked unit-triangular
// inverse of the chunk algebra.  Used by the prefill alignment and the
// backward pass, whose per-chunk algebra runs in float32.
#pragma once

#include "path_attn_internal.h"

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

namespace pathattn {

// ---------------------------------------------------------------------------
// float32 matrix-core products of 64 x 64 blocks (v_mfma_f32_32x32x2f32) with
// both operands staged through LDS panels, for 256-thread blocks: wave w owns
// the 32 x 32 output tile (w >> 1, w & 1).  In a tile, lane l register r
// holds row 8*(r/4) + 4*(l/32) + r%4 and column l%32 (acc_row).

// Floats of one panel: a 64 x K block or a K x 64 block (K <= KMAX), each
// stored with pitch (columns + 1) so row and column reads are conflict-free.
__host__ __device__ constexpr int panel_floats(int kmax) { return kmax * 65 > 64 * (kmax + 1) ? kmax * 65 : 64 * (kmax + 1); }

__device__ __forceinline__ void load4(const float *p, float (&v)[4]) {
  const float4 x = *reinterpret_cast<const float4 *>(p);
  v[0] = x.x;
  v[1] = x.y;
  v[2] = x.z;
  v[3] = x.w;
}
__device__ __forceinline__ void load4(const __bf16 *p, float (&v)[4]) {
  const bf16x4 x = *reinterpret_cast<const bf16x4 *>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (float)x[e];
}

// dst[r][c] = src[r * ld + c] (times rscale[r] if given) for a ROWS x COLS
// block (rows 16-byte aligned for float, 8-byte for bf16; COLS % 4 == 0):
// every thread issues its vector loads before its LDS stores.
template <int ROWS, int COLS, typename T>
__device__ __forceinline__ void load_panel(float *dst, const T *src, int ld, const float *rscale,
                                           int tid) {
  constexpr int CV = COLS / 4, PER = ROWS * CV / 256;
  static_assert(ROWS * CV % 256 == 0, "panel must split evenly over 256 threads");
  float v[PER][4];
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int vi = tid + 256 * it, r = vi / CV, c4 = 4 * (vi % CV);
    load4(src + (size_t)r * ld + c4, v[it]);
  }
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int vi = tid + 256 * it, r = vi / CV, c4 = 4 * (vi % CV);
    const float sc = rscale ? rscale[r] : 1.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[r * (COLS + 1) + c4 + e] = sc * v[it][e];
  }
}

// acc += op(X)[64 x K] op(Y)[K x 64] for this wave's tile, X and Y row-major
// in global memory:  op(X) = X (a 64 x K block) or, with TX, X^T (X a K x 64
// block); op(Y) = Y (a K x 64 block) or, with TY, Y^T (Y a 64 x K block).
// yscale (optional, not with TY) multiplies row k of Y.  Starts and ends with
// the block-wide barriers that make the panels (and earlier global writes of
// the block) safe to reuse.
template <int K, bool TX, bool TY, typename TXe, typename TYe>
__device__ __forceinline__ void gmm(f32x16 &acc, const TXe *X, int ldx, const TYe *Y, int ldy,
                                    float *PX, float *PY, int tid,
                                    const float *yscale = nullptr) {
  __syncthreads();
  if (TX) load_panel<K, 64>(PX, X, ldx, nullptr, tid);
  else load_panel<64, K>(PX, X, ldx, nullptr, tid);
  if (TY) load_panel<64, K>(PY, Y, ldy, nullptr, tid);
  else load_panel<K, 64>(PY, Y, ldy, yscale, tid);
  __syncthreads();
  const int lane = tid & 63, wv = tid >> 6, i = lane & 31, k0 = lane >> 5;
  constexpr int a_rs = TX ? 1 : K + 1, a_cs = TX ? 65 : 1;
  constexpr int b_rs = TY ? 1 : 65, b_cs = TY ? K + 1 : 1;
  const float *pa = PX + (32 * (wv >> 1) + i) * a_rs + k0 * a_cs;
  const float *pb = PY + k0 * b_rs + (32 * (wv & 1) + i) * b_cs;
#pragma unroll 8
  for (int k = 0; k < K; k += 2)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(pa[k * a_cs], pb[k * b_rs], acc, 0, 0, 0);
}

__device__ __forceinline__ void zero16(f32x16 &a) {
#pragma unroll
  for (int r = 0; r < 16; ++r) a[r] = 0.f;
}

// f(row, col, r) for each of this wave's 16 tile elements (acc[r] is element
// (row, col) of the 64 x 64 block).
template <typename F>
__device__ __forceinline__ void tile_each(int tid, F f) {
  const int lane = tid & 63, wv = tid >> 6;
  const int col = 32 * (wv & 1) + (lane & 31), g = lane >> 5, row0 = 32 * (wv >> 1);
#pragma unroll
  for (int r = 0; r < 16; ++r) f(row0 + acc_row(r, g), col, r);
}

// X = (I + N)^{-1} for a strictly lower triangular 64 x 64 N (LDS, pitch 65),
// written in full to Xs (pitch 65), by blocked forward substitution on 16 x 16
// blocks: diagonal blocks by substitution, then X_pq = -X_pp sum_{r=q}^{p-1}
// N_pr X_rq one block diagonal at a time.  tmp: 768 floats of LDS.
__device__ __forceinline__ void unit_lower_inverse(const float *Ns, float *Xs, float *tmp,
                                                   int tid) {
  constexpr int P = 65;
  for (int idx = tid; idx < 64 * 64; idx += 256) {
    const int i = idx >> 6, j = idx & 63;
    if ((i >> 4) < (j >> 4)) Xs[i * P + j] = 0.f;
  }
  if (tid < 64) {
    const int base = 16 * (tid >> 4), j = tid & 15;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float a = i == j ? 1.f : 0.f;
#pragma unroll
      for (int t = 0; t < i; ++t) a = __builtin_fmaf(-Ns[(base + i) * P + base + t], x[t], a);
      x[i] = a;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) Xs[(base + i) * P + base + j] = x[i];
  }
  __syncthreads();
  for (int lev = 1; lev < 4; ++lev) {
    const int nb = 4 - lev;
    for (int idx = tid; idx < nb * 256; idx += 256) {
      const int q = idx >> 8, e = idx & 255, i = e >> 4, j = e & 15, p = q + lev;
      float y = 0.f;
      for (int t = 16 * q; t < 16 * p; ++t) y = __builtin_fmaf(Ns[(16 * p + i) * P + t], Xs[t * P + 16 * q + j], y);
      tmp[idx] = y;
    }
    __syncthreads();
    for (int idx = tid; idx < nb * 256; idx += 256) {
      const int q = idx >> 8, e = idx & 255, i = e >> 4, j = e & 15, p = q + lev;
      float x = 0.f;
#pragma unroll
      for (int t = 0; t < 16; ++t) x = __builtin_fmaf(-Xs[(16 * p + i) * P + 16 * p + t], tmp[(q << 8) + t * 16 + j], x);
      Xs[(16 * p + i) * P + 16 * q + j] = x;
    }
    __syncthreads();
  }
}

}  // namespace pathattn
