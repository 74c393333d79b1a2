// backward.hip -- gradients of PaTH attention (q, k, v, w, beta, log f).
//
// The pages time forward plus backward ([R]'s latency table) but describe
// only the forward kernel; the backward here is this library's blockwise
// derivation of the exact gradients, built on the forward's chunk algebra
// (PaTH slides for arXiv:2505.16381v2, frames "A triangular representation
// makes paths computable", "A right-to-left scan accumulates cross-block
// paths", "Backup: fix orientation before implementing UT products") and on
// the decoding view of frame "Decoding updates historical keys in place".
//
// Per 64-token chunk c the forward's UT quantities are Qa = <-Q_c, Kb = ->K_c,
// M_c and the diagonal logits Al_c.  The keys of every chunk before c,
// aligned to the start of chunk c ("key level" c), satisfy
//     Khat[c+1] = [ Khat[c] (I - M_c)^T ; Kb_c ],
// and the cross logits of query chunk c are Qa_c Khat[c]^T.  With the
// forward's lse the weights P = exp(s - lse) are known, so the gradient of the
// raw logits is g = scale * P o (dO V^T - rowdot(dO, O) + dlse).  Then, for
// c = N-1 down to 1 (one launch per chunk, one block per earlier key chunk):
//     dQa_c  = g Khat[c]                       (partials reduced per chunk)
//     dV    += P^T dO_c,   dLambda_j -= colsum(dS)
//     Gamma += g^T Qa_c                        (gradient of Khat[c])
//     dKb_{c-1} = Gamma[chunk c-1],  dM_{c-1} = -Gamma[< c-1]^T Khat[c-1],
//     Gamma <- Gamma[< c-1] (I - M_{c-1}).
// The diagonal blocks give dAl and start dV; a per-chunk adjoint of the UT
// formulas maps (dQa, dKb, dM, dAl) to dq, dk, dw, dbeta; suffix sums of
// dLambda give d log f.  All arithmetic is float32; the key levels of a head
// take 64*d*N(N-1)/2 floats of workspace.
#include <type_traits>

#include "path_attn_internal.h"
#include "tile_fp32.h"

namespace pathattn {

namespace {

constexpr int C = kChunk;
constexpr int NT = 256;

template <typename E>
__device__ __forceinline__ float ld(const E *p) { return (float)*p; }

// 16 bytes of a row as floats: 8 bf16 or 4 float32 elements (p 16-byte aligned).
template <typename E>
struct Row16;
template <>
struct Row16<__bf16> {
  static constexpr int N = 8;
  __device__ static __forceinline__ void load(float (&x)[N], const __bf16 *p) {
    const bf16x8 v = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int t = 0; t < N; ++t) x[t] = (float)v[t];
  }
};
template <>
struct Row16<float> {
  static constexpr int N = 4;
  __device__ static __forceinline__ void load(float (&x)[N], const float *p) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
    for (int t = 0; t < N; ++t) x[t] = v[t];
  }
};

// ------------------------------------------------------------ chunk prep

// Per-chunk float32 matrices kept from the preparation for the adjoint:
// X = (I + N)^{-1}, U, A = lower(Q W^T), B = strictLower(W K^T), T2 = U B
// (64 x 64 each) and U W (64 x D).
__host__ __device__ constexpr size_t saved_floats(int D) { return 5 * 4096 + 64 * (size_t)D; }
// Per-chunk adjoint intermediates: dA, dT2, dX, Y, dN, dB (64 x 64) and dUW (64 x D).
__host__ __device__ constexpr size_t adj_floats(int D) { return 6 * 4096 + 64 * (size_t)D; }

// One block per (bh, chunk), float32 matrix cores: Kb ([T][D]), M
// ([N][D][D]), Al ([N][64][64], zero above the diagonal) and the saved
// matrices of the chunk; for the matrix-core sweep Qa and -M in the input
// dtype (Qa rows [T][D], -M per chunk), and either the bf16 d = 64 operand
// images or Qa^T and -M^T per chunk for the general kernel.  SAVED_ONLY:
// only the saved matrices (their bytes are shared with the sweep's buffers,
// so they are computed again, the same bits, after the sweep).
template <typename E, int D, bool SAVED_ONLY = false>
__global__ __launch_bounds__(256) void bwd_prep_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ w,
    const float *__restrict__ beta, float *__restrict__ kb,
    float *__restrict__ m, float *__restrict__ al, float *__restrict__ saved, E *__restrict__ qae,
    E *__restrict__ qat, E *__restrict__ nm, E *__restrict__ nmt, E *__restrict__ qimg,
    E *__restrict__ mimg, int T) {
  constexpr bool IMG = std::is_same<E, __bf16>::value && D == 64;
  __shared__ float PX[panel_floats_any(D)], PY[panel_floats_any(D)];
  __shared__ float tmp[768], bs[C];
  const int N = T / C;
  const int chunk = blockIdx.x, bh = chunk / N, c = chunk % N;
  const size_t row0 = (size_t)bh * T + (size_t)c * C;
  const int tid = threadIdx.x;
  const E *Q = q + row0 * D, *K = k + row0 * D, *W = w + row0 * D;
  float *Xg = saved + (size_t)chunk * saved_floats(D);
  float *Ug = Xg + 4096, *Ag = Ug + 4096, *Bg = Ag + 4096, *T2g = Bg + 4096, *UWg = T2g + 4096;
  float *kb_c = kb + row0 * D;
  float *m_c = m + (size_t)chunk * D * D, *al_c = al + (size_t)chunk * C * C;
  if (tid < C) bs[tid] = beta[row0 + tid];
  f32x16 acc, acc2;

  zero16(acc);   // G = W W^T -> N = strictLower(D G) -> X -> U
  gmm_e<E, D, false, true>(acc, W, D, W, D, PX, PY, tid);
  __syncthreads();
  tile_each(tid, [&](int i, int j, int r) { PX[i * 65 + j] = j < i ? bs[i] * acc[r] : 0.f; });
  __syncthreads();
  unit_lower_inverse(PX, PY, tmp, tid);
  for (int idx = tid; idx < 4096; idx += NT) {
    const int i = idx >> 6, j = idx & 63;
    const float x = PY[i * 65 + j];
    Xg[idx] = x;
    Ug[idx] = j <= i ? x * bs[j] : 0.f;
  }
#pragma unroll
  for (int nb = 0; nb < D / 64; ++nb) {   // U W
    zero16(acc);
    gmm_e<E, 64, false, false>(acc, Ug, 64, W + 64 * nb, D, PX, PY, tid);
    tile_each(tid, [&](int i, int j, int r) { UWg[i * D + 64 * nb + j] = acc[r]; });
  }
#pragma unroll
  for (int ma = 0; ma < D / 64; ++ma)   // M = W^T (U W)
#pragma unroll
    for (int nb = 0; nb < D / 64 && !SAVED_ONLY; ++nb) {
      zero16(acc);
      gmm_e<E, 64, true, false>(acc, W + 64 * ma, D, UWg + 64 * nb, D, PX, PY, tid);
      tile_each(tid, [&](int i, int j, int r) {
        const int a = 64 * ma + i, b = 64 * nb + j;
        m_c[(size_t)a * D + b] = acc[r];
        nm[(size_t)chunk * D * D + (size_t)a * D + b] = (E)(-acc[r]);
        if (!IMG) nmt[(size_t)chunk * D * D + (size_t)b * D + a] = (E)(-acc[r]);
        if (IMG) mimg[(size_t)chunk * kMImgElems + mimg_index(a, b)] = (E)(-acc[r]);
      });
    }
  zero16(acc);   // A = lower(Q W^T)
  gmm_e<E, D, false, true>(acc, Q, D, W, D, PX, PY, tid);
  tile_each(tid, [&](int i, int j, int r) { Ag[i * 64 + j] = j <= i ? acc[r] : 0.f; });
#pragma unroll
  for (int nb = 0; nb < D / 64 && !SAVED_ONLY; ++nb) {   // <-Q = Q - A (U W)
    zero16(acc);
    gmm_e<E, 64, false, false>(acc, Ag, 64, UWg + 64 * nb, D, PX, PY, tid);
    tile_each(tid, [&](int i, int j, int r) {
      const int d = 64 * nb + j;
      const float x = (float)Q[i * D + d] - acc[r];
      qae[(row0 + i) * D + d] = (E)x;
      if (!IMG) qat[(size_t)chunk * D * C + (size_t)d * C + i] = (E)x;
      if (IMG) {
        E *img = qimg + (size_t)chunk * kQImgElems;
        img[i * kImgPitch + d] = (E)x;                  // rows
        img[64 * kImgPitch + mimg_index(i, d)] = (E)x;  // fragment order
      }
    });
  if (IMG && !SAVED_ONLY)   // zero padding of the image rows
    for (int idx = tid; idx < 64 * (kImgPitch - 64); idx += NT)
      qimg[(size_t)chunk * kQImgElems + (idx / (kImgPitch - 64)) * kImgPitch + 64 +
           idx % (kImgPitch - 64)] = (E)0.f;
  }
  zero16(acc);   // B = strictLower(W K^T)
  gmm_e<E, D, false, true>(acc, W, D, K, D, PX, PY, tid);
  tile_each(tid, [&](int i, int j, int r) { Bg[i * 64 + j] = j < i ? acc[r] : 0.f; });
  zero16(acc);   // T2 = U B
  gmm_e<E, 64, false, false>(acc, Ug, 64, Bg, 64, PX, PY, tid);
  tile_each(tid, [&](int i, int j, int r) { T2g[i * 64 + j] = acc[r]; });
  if constexpr (SAVED_ONLY) return;
#pragma unroll
  for (int nb = 0; nb < D / 64; ++nb) {   // ->K = K - T2^T W
    zero16(acc);
    gmm_e<E, 64, true, false>(acc, T2g, 64, W + 64 * nb, D, PX, PY, tid);
    tile_each(tid, [&](int i, int j, int r) {
      kb_c[i * D + 64 * nb + j] = (float)K[i * D + 64 * nb + j] - acc[r];
    });
  }
  zero16(acc);   // Al = lower(Q K^T) - A T2
  gmm_e<E, D, false, true>(acc, Q, D, K, D, PX, PY, tid);
  zero16(acc2);
  gmm_e<E, 64, false, false>(acc2, Ag, 64, T2g, 64, PX, PY, tid);
  tile_each(tid, [&](int i, int j, int r) { al_c[i * 64 + j] = j <= i ? acc[r] - acc2[r] : 0.f; });
}

// Lambda_t = sum_{1<=s<=t} log f_s in float64, rounded once: one block per
// head, each thread a contiguous segment, then a scan of the segment totals.
__global__ __launch_bounds__(256) void bwd_gate_kernel(const float *__restrict__ logf,
                                                       float *__restrict__ lam, int T) {
  __shared__ double tot[NT];
  const size_t base = (size_t)blockIdx.x * T;
  const int tid = threadIdx.x, seg = (T + NT - 1) / NT;
  const int lo = tid * seg, hi = lo + seg < T ? lo + seg : T;
  double s = 0.0;
  for (int t = lo > 1 ? lo : 1; t < hi; ++t) s += (double)logf[base + t];
  tot[tid] = s;
  __syncthreads();
  double before = 0.0;
  for (int u = 0; u < tid; ++u) before += tot[u];
  for (int t = lo; t < hi; ++t) {
    if (t >= 1) before += (double)logf[base + t];
    lam[base + t] = (float)before;
  }
}

// ------------------------------------------------------------ diagonal blocks

// One block per (bh, chunk): rowdot(dO, O), the diagonal block's weights and
// gradients; starts dV (P^T dO) and, with the gate, dLambda (row sums minus
// column sums of dS) of the chunk.  The row sums of dS equal dlse in exact
// arithmetic, but taking them from the computed dS makes the rounding of
// rowdot(dO, O) cancel in the suffix sums of dLambda: what remains of it in
// d log f_t is weighted by the softmax mass on keys before t.
template <typename E, int D, bool FOX>
__global__ __launch_bounds__(256) void bwd_diag_kernel(
    const float *__restrict__ al, const E *__restrict__ v, const E *__restrict__ o,
    const E *__restrict__ dout, const float *__restrict__ lse, const float *__restrict__ dlse,
    const float *__restrict__ lam, float scale, float *__restrict__ dal,
    float *__restrict__ dv, float *__restrict__ dlam, float *__restrict__ dvec,
    E *__restrict__ dot, E *__restrict__ oimg, float4 *__restrict__ qst, int T) {
  constexpr bool IMG = std::is_same<E, __bf16>::value && D == 64;
  // dO and V rows in LDS in the input dtype (bf16 widens exactly); pitch D + 1
  // floats or D + 2 bf16 (column reads by 16 lanes fall in 16 banks)
  constexpr int DP = std::is_same<E, __bf16>::value ? D + 2 : D + 1, CP = C + 1;
  __shared__ E Os[C * DP];
  __shared__ E Vs[C * DP];
  __shared__ float Ps[C * CP];
  __shared__ float rl[C], rd[C], rg[C], rdl[C];
  const int N = T / C;
  const int bh = blockIdx.x / N, c = blockIdx.x % N;
  const size_t row0 = (size_t)bh * T + (size_t)c * C;
  int tid = threadIdx.x;
  // dO and V rows to LDS as floats, 16 bytes per load
  using RV = Row16<E>;
  constexpr int VPR = D / RV::N;   // 16-byte loads per row
  for (int vi = tid; vi < C * VPR; vi += NT) {
    const int r = vi / VPR, e0 = RV::N * (vi % VPR);
    float xo[RV::N], xv[RV::N];
    RV::load(xo, dout + (row0 + r) * D + e0);
    RV::load(xv, v + (row0 + r) * D + e0);
#pragma unroll
    for (int t = 0; t < RV::N; ++t) {
      Os[r * DP + e0 + t] = (E)xo[t];
      Vs[r * DP + e0 + t] = (E)xv[t];
    }
  }
  {   // rowdot(dO, O): four threads per row, each a quarter of the columns
    static_assert(NT == 4 * C, "four threads per row");
    const int r = tid >> 2, part = tid & 3;
    const E *pd = dout + (row0 + r) * D + part * (D / 4), *po = o + (row0 + r) * D + part * (D / 4);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < D / 4; e += RV::N) {
      float xd[RV::N], xo[RV::N];
      RV::load(xd, pd + e);
      RV::load(xo, po + e);
#pragma unroll
      for (int t = 0; t < RV::N; ++t) s = __builtin_fmaf(xd[t], xo[t], s);
    }
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    if (part == 0) {
      rd[r] = s;
      dvec[row0 + r] = s;
      rl[r] = lse[row0 + r];
      rg[r] = FOX ? lam[row0 + r] : 0.f;
      rdl[r] = dlse ? dlse[row0 + r] : 0.f;
    }
  }
  __syncthreads();
  if (!IMG)
    for (int idx = tid; idx < C * D; idx += NT)   // dO^T of the chunk, [D][64]
      dot[((size_t)bh * N + c) * C * D + idx] = (E)Os[(idx % C) * DP + idx / C];
  if (IMG) {   // bf16, d = 64: 16-byte stores of 8 values each
    E *img = oimg + ((size_t)bh * N + c) * kQImgElems;
    for (int vi = tid; vi < 64 * (kImgPitch / 8); vi += NT) {   // dO rows, zero padded
      const int r = vi / (kImgPitch / 8), c8 = 8 * (vi % (kImgPitch / 8));
      bf16x8 x;
#pragma unroll
      for (int t = 0; t < 8; ++t) x[t] = c8 < 64 ? (E)Os[r * DP + c8 + t] : (E)0.f;
      *reinterpret_cast<bf16x8 *>(img + r * kImgPitch + c8) = x;
    }
    // dO in fragment order: blob (mt, s), lane l holds the 8 values
    // dO[frag_row(s, l/32, t)][32 mt + l%32], t < 8, contiguously
    for (int vi = tid; vi < 8 * 64; vi += NT) {
      const int blob = vi / 64, l = vi % 64, mt = blob / 4, sI = blob % 4;
      bf16x8 x;
#pragma unroll
      for (int t = 0; t < 8; ++t)
        x[t] = (E)Os[frag_row(sI, l / 32, t, 8) * DP + 32 * mt + l % 32];
      *reinterpret_cast<bf16x8 *>(img + 64 * kImgPitch + (blob * 64 + l) * 8) = x;
    }
    if (tid < C) qst[row0 + tid] = make_float4(rl[tid], rd[tid], rdl[tid], rg[tid]);
  }
  // the thread index re-derived: the products' addresses are computed here,
  // not kept live from the kernel's start
  asm volatile("" : "+v"(tid));
  const int r0 = tid / 16, c0 = tid % 16;
  const float *al_c = al + ((size_t)bh * N + c) * C * C;
  float p[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int i = r0 + 16 * r, j = c0 + 16 * s;
      p[r][s] = j <= i ? __expf(scale * al_c[i * C + j] + rg[i] - rg[j] - rl[i]) : 0.f;
      Ps[i * CP + j] = p[r][s];
    }
  __syncthreads();
  float acc[4][4];
#pragma unroll
  for (int h = 0; h < D / 64; ++h) {   // dV_c = P^T dO
    tile_zero(acc);
    tile_mm<C>(acc, Ps, 1, CP, Os + 64 * h, DP, 1, r0, c0);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int s = 0; s < 4; ++s)
        dv[(row0 + r0 + 16 * r) * D + 64 * h + c0 + 16 * s] = acc[r][s];
  }
  tile_zero(acc);   // dP = dO V^T, dS = P (dP - D + dlse)
  tile_mm<D>(acc, Os, DP, 1, Vs, 1, DP, r0, c0);
  __syncthreads();
  float *dal_c = dal + ((size_t)bh * N + c) * C * C;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int i = r0 + 16 * r, j = c0 + 16 * s;
      const float ds = p[r][s] * (acc[r][s] - rd[i] + rdl[i]);
      Ps[i * CP + j] = ds;
      dal_c[i * C + j] = scale * ds;
    }
  __syncthreads();
  if (FOX && tid < C) {   // dLambda_t = sum_j dS_tj - sum_i dS_it over the diagonal block
    float cs = 0.f, rs = 0.f;
    for (int i = 0; i < C; ++i) {
      cs += Ps[i * CP + tid];
      rs += Ps[tid * CP + i];
    }
    dlam[row0 + tid] = rs - cs;
  }
}

// ------------------------------------------------------------ local adjoint

// One block per (bh, chunk), float32 matrix cores: gradients of the chunk's
// inputs from those of its UT quantities (dQa, dKb, dM, dAl), with
// A = lower(Q W^T), B = strictLower(W K^T), T2 = U B, N = strictLower(D G),
// G = W W^T, D = diag(beta), X = (I + N)^{-1}, U = X D:
//   dA   = lower(-dQa (UW)^T - dAl T2^T)
//   dUW  = -A^T dQa + W dM
//   dT2  = -W dKb^T - A^T dAl
//   dU   = lower(dUW W^T + dT2 B^T),  dB = strictLower(U^T dT2)
//   dX   = dU D,  dbeta_j += sum_i X_ij dU_ij
//   dN   = strictLower(-X^T dX X^T)
//   dG   = D dN,  dbeta_i += sum_j dN_ij G_ij = w_i . (dN W)_i
//   dQ   = dQa + dAl K + dA W
//   dK   = dKb + dAl^T Q + dB^T W
//   dW   = -T2 dKb + UW dM^T + U^T dUW + dA^T Q + dB K + dG W + dG^T W
template <typename E, int D>
__global__ __launch_bounds__(256) void bwd_local_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ w,
    const float *__restrict__ beta, const float *__restrict__ dqa,
    const float *__restrict__ dkb, const float *__restrict__ dm, const float *__restrict__ dal,
    const float *__restrict__ saved, float *__restrict__ adj, E *__restrict__ dq,
    E *__restrict__ dk, E *__restrict__ dw, float *__restrict__ dbeta, int T) {
  __shared__ float PX[panel_floats_any(D)], PY[panel_floats_any(D)];
  // dbeta's two sums, reduced in a fixed order (no atomics, so the same bits
  // on every call): [half of the block's waves][token]
  __shared__ float bs[C], dbx[2][C], dbn[2][C];
  const int N = T / C;
  const int chunk = blockIdx.x, bh = chunk / N, c = chunk % N;
  const size_t row0 = (size_t)bh * T + (size_t)c * C;
  const int tid = threadIdx.x;
  const E *Q = q + row0 * D, *K = k + row0 * D, *W = w + row0 * D;
  const float *dQa = dqa + row0 * D, *dKb = dkb + row0 * D;
  const float *dM = dm + (size_t)chunk * D * D, *dAl = dal + (size_t)chunk * C * C;
  const float *Xg = saved + (size_t)chunk * saved_floats(D);
  const float *Ug = Xg + 4096, *Ag = Ug + 4096, *Bg = Ag + 4096, *T2g = Bg + 4096, *UWg = T2g + 4096;
  float *dAg = adj + (size_t)chunk * adj_floats(D);
  float *dT2g = dAg + 4096, *dXg = dT2g + 4096, *Yg = dXg + 4096, *dNg = Yg + 4096, *dBg = dNg + 4096;
  float *dUWg = dBg + 4096;
  if (tid < C) bs[tid] = beta[row0 + tid];
  f32x16 acc, acc2;

  zero16(acc);   // dA
  gmm_e<E, D, false, true>(acc, dQa, D, UWg, D, PX, PY, tid);
  gmm_e<E, 64, false, true>(acc, dAl, 64, T2g, 64, PX, PY, tid);
  tile_each(tid, [&](int i, int j, int r) { dAg[i * 64 + j] = j <= i ? -acc[r] : 0.f; });
#pragma unroll
  for (int nb = 0; nb < D / 64; ++nb) {   // dUW
    zero16(acc);
    gmm_e<E, D, false, false>(acc, W, D, dM + 64 * nb, D, PX, PY, tid);
    zero16(acc2);
    gmm_e<E, 64, true, false>(acc2, Ag, 64, dQa + 64 * nb, D, PX, PY, tid);
    tile_each(tid, [&](int i, int j, int r) { dUWg[i * D + 64 * nb + j] = acc[r] - acc2[r]; });
  }
  zero16(acc);   // dT2
  gmm_e<E, D, false, true>(acc, W, D, dKb, D, PX, PY, tid);
  gmm_e<E, 64, true, false>(acc, Ag, 64, dAl, 64, PX, PY, tid);
  tile_each(tid, [&](int i, int j, int r) { dT2g[i * 64 + j] = -acc[r]; });
  zero16(acc);   // dU -> dX, dbeta_j
  gmm_e<E, D, false, true>(acc, dUWg, D, W, D, PX, PY, tid);
  gmm_e<E, 64, false, true>(acc, dT2g, 64, Bg, 64, PX, PY, tid);
  {
    float part = 0.f;
    int col = 0;
    tile_each(tid, [&](int i, int j, int r) {
      const float du = j <= i ? acc[r] : 0.f;
      part = __builtin_fmaf(Xg[i * 64 + j], du, part);
      col = j;
      dXg[i * 64 + j] = du * bs[j];
    });
    // the column's 32 rows of this wave: both halves of the lane set
    part += __shfl_xor(part, 32);
    if ((tid & 63) < 32) dbx[tid >> 7][col] = part;
  }
  zero16(acc);   // dB
  gmm_e<E, 64, true, false>(acc, Ug, 64, dT2g, 64, PX, PY, tid);
  tile_each(tid, [&](int i, int j, int r) { dBg[i * 64 + j] = j < i ? acc[r] : 0.f; });
  zero16(acc);   // Y = dX X^T
  gmm_e<E, 64, false, true>(acc, dXg, 64, Xg, 64, PX, PY, tid);
  tile_each(tid, [&](int i, int j, int r) { Yg[i * 64 + j] = acc[r]; });
  zero16(acc);   // dN = strictLower(-X^T Y)
  gmm_e<E, 64, true, false>(acc, Xg, 64, Yg, 64, PX, PY, tid);
  tile_each(tid, [&](int i, int j, int r) { dNg[i * 64 + j] = j < i ? -acc[r] : 0.f; });
#pragma unroll
  for (int nb = 0; nb < D / 64; ++nb) {   // dQ
    zero16(acc);
    gmm_e<E, 64, false, false>(acc, dAl, 64, K + 64 * nb, D, PX, PY, tid);
    gmm_e<E, 64, false, false>(acc, dAg, 64, W + 64 * nb, D, PX, PY, tid);
    tile_each(tid, [&](int i, int j, int r) {
      const size_t o = (size_t)i * D + 64 * nb + j;
      dq[row0 * D + o] = (E)(dQa[o] + acc[r]);
    });
  }
#pragma unroll
  for (int nb = 0; nb < D / 64; ++nb) {   // dK
    zero16(acc);
    gmm_e<E, 64, true, false>(acc, dAl, 64, Q + 64 * nb, D, PX, PY, tid);
    gmm_e<E, 64, true, false>(acc, dBg, 64, W + 64 * nb, D, PX, PY, tid);
    tile_each(tid, [&](int i, int j, int r) {
      const size_t o = (size_t)i * D + 64 * nb + j;
      dk[row0 * D + o] = (E)(dKb[o] + acc[r]);
    });
  }
  float rn[16];   // w_i . (dN W)_i over this wave's columns, per tile row
#pragma unroll
  for (int r = 0; r < 16; ++r) rn[r] = 0.f;
#pragma unroll
  for (int nb = 0; nb < D / 64; ++nb) {   // dW
    f32x16 accn;
    zero16(accn);   // dN W
    gmm_e<E, 64, false, false>(accn, dNg, 64, W + 64 * nb, D, PX, PY, tid);
    zero16(acc2);   // T2 dKb
    gmm_e<E, 64, false, false>(acc2, T2g, 64, dKb + 64 * nb, D, PX, PY, tid);
    zero16(acc);
    gmm_e<E, 64, true, false>(acc, dNg, 64, W + 64 * nb, D, PX, PY, tid, bs);   // dG^T W
    gmm_e<E, D, false, true>(acc, UWg, D, dM + (size_t)64 * nb * D, D, PX, PY, tid);   // UW dM^T
    gmm_e<E, 64, true, false>(acc, Ug, 64, dUWg + 64 * nb, D, PX, PY, tid);   // U^T dUW
    gmm_e<E, 64, true, false>(acc, dAg, 64, Q + 64 * nb, D, PX, PY, tid);     // dA^T Q
    gmm_e<E, 64, false, false>(acc, dBg, 64, K + 64 * nb, D, PX, PY, tid);    // dB K
    tile_each(tid, [&](int i, int j, int r) {
      const size_t o = (size_t)i * D + 64 * nb + j;
      const float wv = (float)W[o];
      rn[r] = __builtin_fmaf(wv, accn[r], rn[r]);
      dw[row0 * D + o] = (E)(acc[r] - acc2[r] + bs[i] * accn[r]);
    });
  }
  {   // each tile row's 32 columns of this wave (the lanes of one half)
    const int lane = tid & 63, g = lane >> 5, wv = tid >> 6;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = rn[r];
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) x += __shfl_xor(x, o);
      if ((lane & 31) == 0) dbn[wv & 1][32 * (wv >> 1) + acc_row(r, g)] = x;
    }
  }
  __syncthreads();
  if (tid < C) dbeta[row0 + tid] = (dbx[0][tid] + dbx[1][tid]) + (dbn[0][tid] + dbn[1][tid]);
}

// dv = dV in the input dtype (grid-stride over all heads).
template <typename E>
__global__ __launch_bounds__(256) void bwd_cast_kernel(const float *__restrict__ src,
                                                       E *__restrict__ dst, size_t n) {
  for (size_t i = (size_t)blockIdx.x * NT + threadIdx.x; i < n; i += (size_t)gridDim.x * NT)
    dst[i] = (E)src[i];
}

// d log f_t = sum_{i >= t} dLambda_i for t >= 1, d log f_0 = 0: one block
// per head, float64 suffix sums (each thread a contiguous segment, then a
// scan of the segment totals).
__global__ __launch_bounds__(256) void bwd_gate_grad_kernel(const float *__restrict__ dlam,
                                                            float *__restrict__ dlogf, int T) {
  __shared__ double tot[NT];
  const size_t base = (size_t)blockIdx.x * T;
  const int tid = threadIdx.x, seg = (T + NT - 1) / NT;
  const int lo = tid * seg, hi = lo + seg < T ? lo + seg : T;
  double s = 0.0;
  for (int t = lo; t < hi; ++t) s += (double)dlam[base + t];
  tot[tid] = s;
  __syncthreads();
  double after = 0.0;   // sum of the segments to the right
  for (int u = tid + 1; u < NT; ++u) after += tot[u];
  for (int t = hi - 1; t >= lo; --t) {
    after += (double)dlam[base + t];
    if (t >= 1) dlogf[base + t] = (float)after;
  }
  if (tid == 0) dlogf[base] = 0.f;
}

}  // namespace

BwdLayout bwd_layout(int B, int H, int T, int D, int dtype, int window) {
  const size_t BH = (size_t)B * H, N = (size_t)T / C;
  const size_t esize = dtype == 1 ? 2 : 4;
  BwdLayout L;
  size_t off = 0;
  auto take = [&](size_t floats) {
    const size_t o = off;
    off = align256(off + floats * sizeof(float));
    return o;
  };
  const BwdPlan P = bwd_plan(T, window);
  const bool img = dtype == 1 && D == 64;   // bf16, d = 64: operand images, no transposed levels
  const size_t lev_elems = BH * P.win_blocks * C * D;
  L.kb = take(BH * T * D);
  L.m = take(BH * N * D * D);
  L.al = take(BH * N * C * C);
  L.lam = take(BH * T);
  L.dvec = take(BH * T);
  // the sweep's buffers, whose bytes the adjoint scratch reuses afterwards
  const size_t sweep0 = off;
  L.levels = take((lev_elems * esize + 3) / 4);
  L.levt = take(img ? 0 : (lev_elems * esize + 3) / 4);
  L.dmpart = take(bwd_dmpart_floats(dtype, (int)BH, T, D, window));
  L.ckpt = take(BH * P.ckpt_blocks * C * D);
  L.gstate = take(P.nwin > 1 ? BH * T * D : 0);
  L.kn2 = take(BH * P.win_blocks * 2);   // level row norms for the forget-gate skip
  L.zhi = take(BH * (N + 1));             // skipped dM partials per group; a flag per head
  // after the sweep the same bytes hold the adjoint scratch and, with
  // windows, the saved per-chunk matrices, computed again for the adjoint
  // (bwd_t); one window (the fast, large workspace) keeps them in bytes of
  // their own
  const size_t adj_bytes = align256(BH * N * adj_floats(D) * sizeof(float));
  const size_t saved_bytes = align256(BH * N * saved_floats(D) * sizeof(float));
  L.saved_kept = P.nwin == 1;
  const size_t shared = adj_bytes + (L.saved_kept ? 0 : saved_bytes);
  L.adj = sweep0;
  L.saved = sweep0 + adj_bytes;
  off = sweep0 + (off - sweep0 > shared ? off - sweep0 : shared);
  if (L.saved_kept) L.saved = take(BH * N * saved_floats(D));
  L.dv = take(BH * T * D);
  L.dlam = take(BH * T);
  L.dqa = take(BH * T * D);
  L.dkb = take(BH * T * D);
  L.dm = take(BH * N * D * D);
  L.dal = take(BH * N * C * C);
  auto take_e = [&](size_t elems) { return take((elems * esize + 3) / 4); };
  const bool general = !(dtype == 1 && D == 64);   // the general dk kernel's operands
  L.qae = take_e(BH * T * D);
  L.qat = take_e(general ? BH * T * D : 0);
  L.nm = take_e(BH * N * D * D);
  L.nmt = take_e(general ? BH * N * D * D : 0);
  L.dot = take_e(general ? BH * T * D : 0);
  L.qimg = take_e(img ? BH * N * kQImgElems : 0);
  L.oimg = take_e(img ? BH * N * kQImgElems : 0);
  L.mimg = take_e(img ? BH * N * kMImgElems : 0);
  L.qst = take(img ? BH * T * 4 : 0);
  L.qagg = take(BH * N * 2);
  L.kmin = take(BH * N * 2);
  L.total = off;
  return L;
}

template <typename E, int D, bool FOX>
hipError_t bwd_t(const BwdArgs &a, char *ws, int dtype, hipStream_t s) {
  const BwdLayout L = bwd_layout(a.B, a.H, a.T, D, dtype, a.window);
  const int BH = a.B * a.H, T = a.T, N = T / C;
  auto f = [&](size_t off) { return reinterpret_cast<float *>(ws + off); };
  const E *q = (const E *)a.q, *k = (const E *)a.k, *v = (const E *)a.v, *w = (const E *)a.w;
  auto e = [&](size_t off) { return reinterpret_cast<E *>(ws + off); };
  hipLaunchKernelGGL((bwd_prep_kernel<E, D>), dim3(BH * N), dim3(NT), 0, s, q, k, w, a.beta,
                     f(L.kb), f(L.m), f(L.al), f(L.saved), e(L.qae), e(L.qat), e(L.nm),
                     e(L.nmt), e(L.qimg), e(L.mimg), T);
  if (FOX) hipLaunchKernelGGL(bwd_gate_kernel, dim3(BH), dim3(NT), 0, s, a.logf, f(L.lam), T);
  hipLaunchKernelGGL((bwd_diag_kernel<E, D, FOX>), dim3(BH * N), dim3(NT), 0, s, f(L.al), v,
                     (const E *)a.out, (const E *)a.dout, a.lse, a.dlse, f(L.lam), a.scale, f(L.dal),
                     f(L.dv), f(L.dlam), f(L.dvec), e(L.dot), e(L.oimg),
                     reinterpret_cast<float4 *>(ws + L.qst), T);
  SweepArgs sa{};
  sa.qae = ws + L.qae;
  sa.qat = ws + L.qat;
  sa.nm = ws + L.nm;
  sa.nmt = ws + L.nmt;
  sa.dot = ws + L.dot;
  sa.levt = ws + L.levt;
  sa.qimg = ws + L.qimg;
  sa.oimg = ws + L.oimg;
  sa.mimg = ws + L.mimg;
  sa.qst = ws + L.qst;
  sa.kb = f(L.kb);
  sa.m = f(L.m);
  sa.dout = a.dout;
  sa.v = a.v;
  sa.lse = a.lse;
  sa.dlse = a.dlse;
  sa.dvec = f(L.dvec);
  sa.lam = f(L.lam);
  sa.levels = ws + L.levels;
  sa.dmpart = f(L.dmpart);
  sa.dqa = f(L.dqa);
  sa.dkb = f(L.dkb);
  sa.dv = f(L.dv);
  sa.dlam = f(L.dlam);
  sa.dm = f(L.dm);
  sa.ckpt = f(L.ckpt);
  sa.gstate = f(L.gstate);
  sa.kn2 = f(L.kn2);
  sa.qagg = reinterpret_cast<const float2 *>(ws + L.qagg);
  sa.kmin = f(L.kmin);
  sa.zhi = reinterpret_cast<int *>(ws + L.zhi);
  sa.skip = a.skip;
  sa.scale = a.scale;
  sa.BH = BH;
  sa.T = T;
  sa.window = a.window;
  if (launch_bwd_sweep(dtype, D, FOX, sa, s) != hipSuccess) return hipGetLastError();
  // with windows the sweep has reused the saved matrices' bytes: compute
  // them again
  if (!L.saved_kept)
    hipLaunchKernelGGL((bwd_prep_kernel<E, D, true>), dim3(BH * N), dim3(NT), 0, s, q, k, w,
                       a.beta, f(L.kb), f(L.m), f(L.al), f(L.saved), e(L.qae), e(L.qat), e(L.nm),
                       e(L.nmt), e(L.qimg), e(L.mimg), T);
  hipLaunchKernelGGL((bwd_local_kernel<E, D>), dim3(BH * N), dim3(NT), 0, s, q, k, w, a.beta,
                     f(L.dqa), f(L.dkb), f(L.dm), f(L.dal), f(L.saved), f(L.adj), (E *)a.dq,
                     (E *)a.dk, (E *)a.dw, a.dbeta, T);
  const size_t nv = (size_t)BH * T * D;
  const size_t cb = (nv + NT - 1) / NT;
  hipLaunchKernelGGL((bwd_cast_kernel<E>), dim3((unsigned)(cb < 8192 ? cb : 8192)), dim3(NT), 0, s,
                     f(L.dv), (E *)a.dv, nv);
  if (FOX) hipLaunchKernelGGL(bwd_gate_grad_kernel, dim3(BH), dim3(NT), 0, s, f(L.dlam), a.dlogf, T);
  return hipGetLastError();
}

hipError_t launch_bwd(int dtype, int D, const BwdArgs &a, void *workspace, hipStream_t s) {
  char *ws = static_cast<char *>(workspace);
  const bool fox = a.logf != nullptr;
  if (dtype == 1) {
    if (D == 64)
      return fox ? bwd_t<__bf16, 64, true>(a, ws, dtype, s) : bwd_t<__bf16, 64, false>(a, ws, dtype, s);
    return fox ? bwd_t<__bf16, 128, true>(a, ws, dtype, s) : bwd_t<__bf16, 128, false>(a, ws, dtype, s);
  }
  if (D == 64)
    return fox ? bwd_t<float, 64, true>(a, ws, dtype, s) : bwd_t<float, 64, false>(a, ws, dtype, s);
  return fox ? bwd_t<float, 128, true>(a, ws, dtype, s) : bwd_t<float, 128, false>(a, ws, dtype, s);
}

}  // namespace pathattn
