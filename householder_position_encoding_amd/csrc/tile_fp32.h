// tile_fp32.h -- float32 products of 64 x 64 blocks for 256-thread blocks:
// 4 x 4 register tiles on the vector units (thread t owns rows t/16 + 16 r
// and columns t%16 + 16 s), and 32 x 32 tiles on the float32 matrix cores with
// operands staged through LDS panels (or, for bf16 inputs, on the bf16
// matrix cores with float32 operands split into hi/lo pairs); plus the
// blocked unit-triangular inverse of the chunk algebra.  Used by the prefill
// alignment and the backward pass, whose per-chunk algebra runs in float32.
#pragma once

#include <type_traits>

#include "path_attn_internal.h"

namespace pathattn {

// acc[r][s] += sum_k A(r0 + 16 r, k) B(k, c0 + 16 s) over k < K for one
// thread's 4 x 4 tile of a 64 x 64 output block, operands in LDS with
// arbitrary row / column strides (so transposed reads need no copy).  Rows of
// the tile are 16 apart and columns 16 apart: a wave's lanes read 4 distinct
// A addresses and 16 consecutive B addresses per instruction.  Operands are
// float or bf16 (widened exactly).
template <int K, typename TA, typename TB>
__device__ __forceinline__ void tile_mm(float (&acc)[4][4], const TA *A, int a_rs, int a_cs,
                                        const TB *B, int b_rs, int b_cs, int r0, int c0) {
  for (int kk = 0; kk < K; ++kk) {
    float a[4], b[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = (float)A[(r0 + 16 * r) * a_rs + kk * a_cs];
#pragma unroll
    for (int c = 0; c < 4; ++c) b[c] = (float)B[kk * b_rs + (c0 + 16 * c) * b_cs];
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
  asm volatile("" : "+v"(tid));   // as in gmm_hilo: addresses computed here
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

// ---------------------------------------------------------------------------
// The same products on the bf16 matrix cores (v_mfma_f32_32x32x16_bf16), for
// blocks whose inputs are bf16: each float32 operand x is split into
// hi = bf16(x) and lo = bf16(x - hi), and the product is hi hi + hi lo + lo hi
// (about 16 significant bits, float32 accumulation; the lo lo term, below
// 2^-16 of the product, is left out).  An operand that is a bf16 input is
// exact in bf16: it has no lo part, and its lo products are left out.  The
// output tile has the layout of gmm's.

// Floats of LDS for one operand's hi and lo planes: 64 rows (the operand's
// non-contracted index) of K + 8 bf16, the contraction index contiguous, so a
// lane's 8 contraction values are one 16-byte read and the rows of a 16-lane
// group fall in distinct banks.
__host__ __device__ constexpr int planes_floats(int kmax) { return 64 * (kmax + 8); }
// LDS floats of a panel that serves either form.
__host__ __device__ constexpr int panel_floats_any(int kmax) {
  return panel_floats(kmax) > planes_floats(kmax) ? panel_floats(kmax) : planes_floats(kmax);
}

__device__ __forceinline__ void split8(const float (&x)[8], bf16x8 &h, bf16x8 &l) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    h[e] = (__bf16)x[e];
    l[e] = (__bf16)(x[e] - (float)h[e]);
  }
}

// plane[r][k] = kscale[k] * S(r, k) for r < 64, k < K, as hi (and, unless
// EXACT, lo) bf16 planes at P (hi) and P + 64 (K + 8) (lo); S(r, k) =
// src[r * ld + k] with KMAJ, else src[k * ld + r].  Every thread issues its
// global loads before its LDS stores.
template <int K, bool KMAJ, bool EXACT, typename T>
__device__ __forceinline__ void stage_planes(__bf16 *P, const T *src, int ld, const float *kscale,
                                             int tid) {
  constexpr int PK = K + 8, ITEMS = 64 * K / 8, PER = ITEMS / 256;
  static_assert(ITEMS % 256 == 0, "items split evenly over 256 threads");
  float v[PER][8];
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int vi = tid + 256 * it;
    // KMAJ: 8 consecutive k of row r; else row r = lane order (coalesced
    // scalar loads down the contraction index)
    const int r = KMAJ ? vi / (K / 8) : vi % 64, k8 = 8 * (KMAJ ? vi % (K / 8) : vi / 64);
    if constexpr (KMAJ) {
      if constexpr (std::is_same<T, __bf16>::value) {
        const bf16x8 x = *reinterpret_cast<const bf16x8 *>(src + (size_t)r * ld + k8);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[it][e] = (float)x[e];
      } else {
        const float4 a = *reinterpret_cast<const float4 *>(src + (size_t)r * ld + k8);
        const float4 b = *reinterpret_cast<const float4 *>(src + (size_t)r * ld + k8 + 4);
        v[it][0] = a.x, v[it][1] = a.y, v[it][2] = a.z, v[it][3] = a.w;
        v[it][4] = b.x, v[it][5] = b.y, v[it][6] = b.z, v[it][7] = b.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[it][e] = (float)src[(size_t)(k8 + e) * ld + r];
    }
  }
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int vi = tid + 256 * it;
    const int r = KMAJ ? vi / (K / 8) : vi % 64, k8 = 8 * (KMAJ ? vi % (K / 8) : vi / 64);
    if (kscale)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[it][e] *= kscale[k8 + e];
    bf16x8 h, l;
    split8(v[it], h, l);
    *reinterpret_cast<bf16x8 *>(P + r * PK + k8) = h;
    if (!EXACT) *reinterpret_cast<bf16x8 *>(P + 64 * PK + r * PK + k8) = l;
  }
}

// gmm's product on the bf16 matrix cores (same operands, flags and output
// layout; PX, PY hold planes_floats(K) floats).  yscale multiplies row k of
// Y (not with TY).
template <int K, bool TX, bool TY, typename TXe, typename TYe>
__device__ __forceinline__ void gmm_hilo(f32x16 &acc, const TXe *X, int ldx, const TYe *Y,
                                         int ldy, float *PX, float *PY, int tid,
                                         const float *yscale = nullptr) {
  constexpr bool XE = std::is_same<TXe, __bf16>::value, YB = std::is_same<TYe, __bf16>::value;
  constexpr int PK = K + 8;
  __bf16 *A = reinterpret_cast<__bf16 *>(PX), *B = reinterpret_cast<__bf16 *>(PY);
  const bool ye = YB && !yscale;   // Y exact in bf16
  // the thread index re-derived here: otherwise the compiler computes the
  // addresses of every product of the kernel up front and keeps them live
  // (spilled to accumulation registers)
  asm volatile("" : "+v"(tid));
  __syncthreads();
  // A[r][k] = op(X)(r, k); B[c][k] = op(Y)(k, c)
  stage_planes<K, !TX, XE>(A, X, ldx, nullptr, tid);
  if (ye) stage_planes<K, TY, true>(B, Y, ldy, nullptr, tid);
  else stage_planes<K, TY, false>(B, Y, ldy, yscale, tid);
  __syncthreads();
  const int lane = tid & 63, wv = tid >> 6, i = lane & 31, kg = lane >> 5;
  const __bf16 *pa = A + (32 * (wv >> 1) + i) * PK + 8 * kg;
  const __bf16 *pb = B + (32 * (wv & 1) + i) * PK + 8 * kg;
  auto run = [&](auto yexact) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < K / 16; ++s) {
      const bf16x8 ah = *reinterpret_cast<const bf16x8 *>(pa + 16 * s);
      const bf16x8 bh = *reinterpret_cast<const bf16x8 *>(pb + 16 * s);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh, acc, 0, 0, 0);
      if constexpr (!decltype(yexact)::value) {
        const bf16x8 bl = *reinterpret_cast<const bf16x8 *>(pb + 64 * PK + 16 * s);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl, acc, 0, 0, 0);
      }
      if constexpr (!XE) {
        const bf16x8 al = *reinterpret_cast<const bf16x8 *>(pa + 64 * PK + 16 * s);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh, acc, 0, 0, 0);
      }
    }
  };
  if (ye) run(std::true_type{});
  else run(std::false_type{});
}

// The block product of a kernel whose inputs have type E: the bf16 form for
// bf16 inputs, float32 matrix cores otherwise.
template <typename E, int K, bool TX, bool TY, typename TXe, typename TYe>
__device__ __forceinline__ void gmm_e(f32x16 &acc, const TXe *X, int ldx, const TYe *Y, int ldy,
                                      float *PX, float *PY, int tid,
                                      const float *yscale = nullptr) {
  if constexpr (std::is_same<E, __bf16>::value)
    gmm_hilo<K, TX, TY>(acc, X, ldx, Y, ldy, PX, PY, tid, yscale);
  else
    gmm<K, TX, TY>(acc, X, ldx, Y, ldy, PX, PY, tid, yscale);
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
