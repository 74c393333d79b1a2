// prep.hip -- forget-gate prefix sum and per-chunk UT preparation (float32).
//
// Chunk preparation follows the PaTH discussion slides for arXiv:2505.16381v2,
// frames "A triangular representation makes paths computable" and "Backup: fix
// orientation before implementing UT products" (paper Secs. 3.1-3.3).  For one
// chunk of C = 64 tokens with rows w_t^T stacked in W and D = diag(beta):
//
//   U   = (I + strictLower(D W W^T))^{-1} D           lower triangular
//   <-Q = Q - lower(Q W^T) U W        row i: (H_first ... H_i q_i)^T
//   ->K = K - (U strictLower(W K^T))^T W   row j: (H_last ... H_{j+1} k_j)^T
//   M   = W^T U W                     H_first ... H_last = I - M^T
//   Al  = lower(Q K^T) - lower(Q W^T) U strictLower(W K^T)
//
// Everything is computed in float32: the pages report bf16 arithmetic to be
// unstable for beta near 2 (author-response page, on the range of beta), so
// only the operands handed to the bf16 matrix cores are rounded, once, at the
// end.
#include "path_attn_internal.h"

namespace pathattn {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
template <typename E>
__device__ __forceinline__ E from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

template <typename E>
struct Kpl;
template <>
struct Kpl<__bf16> { static constexpr int value = 8; };
template <>
struct Kpl<float> { static constexpr int value = 1; };

// a_t = -log2(e) * sum_{1<=s<=t} log f_s for one (b, h) per block; the running
// sum is kept in float64 and rounded once.  The gate of a logit (i, j) is
// sum_{s=j+1..i} log f_s = Lambda_i - Lambda_j, so f_0 never enters; leaving it
// out of the prefix keeps the result bitwise independent of it.
__global__ __launch_bounds__(256) void gate_prefix_kernel(
    const float *__restrict__ logf, float *__restrict__ gate, int T) {
  __shared__ double part[256];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const float *f = logf + (size_t)bh * T;
  float *a = gate + (size_t)bh * T;
  const int per = (T + 255) / 256;
  const int t0 = min(T, tid * per), t1 = min(T, t0 + per);
  double s = 0.0;
  for (int t = max(t0, 1); t < t1; ++t) s += (double)f[t];
  part[tid] = s;
  __syncthreads();
  if (tid == 0) {
    double run = 0.0;
    for (int i = 0; i < 256; ++i) {
      const double x = part[i];
      part[i] = run;
      run += x;
    }
  }
  __syncthreads();
  double run = part[tid];
  for (int t = t0; t < t1; ++t) {
    if (t > 0) run += (double)f[t];
    a[t] = (float)(-1.4426950408889634 * run);
  }
}

// One block of 256 threads per (bh, chunk).  LDS: W and U W (64 x D, padded),
// U, P1 = lower(Q W^T) and T2 = U strictLower(W K^T) (64 x 64, padded).
template <typename E, int D>
__global__ __launch_bounds__(256) void prep_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const E *__restrict__ w, const float *__restrict__ beta,
    float *__restrict__ qa, E *__restrict__ kvm, float *__restrict__ al,
    int T) {
  constexpr int C = kChunk, DP = D + 1, CP = C + 1, NT = 256;
  constexpr int KPL = Kpl<E>::value, KSTEP = 2 * KPL;
  __shared__ float Ws[C * DP];
  __shared__ float UWs[C * DP];
  __shared__ float Us[C * CP];
  __shared__ float P1s[C * CP];
  __shared__ float T2s[C * CP];
  __shared__ float bs[C];

  const int N = T / C;
  const int bh = blockIdx.x / N, c = blockIdx.x % N;
  const size_t row0 = (size_t)bh * T + (size_t)c * C;  // first token row
  const int tid = threadIdx.x;
  const E *qc = q + row0 * D;
  const E *kc = k + row0 * D;
  const E *vc = v + row0 * D;
  const E *wc = w + row0 * D;

  for (int idx = tid; idx < C * D; idx += NT)
    Ws[(idx / D) * DP + idx % D] = to_f32(wc[idx]);
  if (tid < C) bs[tid] = beta[row0 + tid];
  __syncthreads();

  // N[i][j] = beta_i (w_i . w_j) for j < i, else 0.
  for (int idx = tid; idx < C * C; idx += NT) {
    const int i = idx / C, j = idx % C;
    float s = 0.f;
    if (j < i) {
      for (int t = 0; t < D; ++t) s += Ws[i * DP + t] * Ws[j * DP + t];
      s *= bs[i];
    }
    Us[i * CP + j] = s;
  }
  __syncthreads();

  // Forward substitution for X = (I + N)^{-1} (unit lower triangular), one
  // column per lane of wave 0:  X[i][j] = -N[i][j] - sum_{j<t<i} N[i][t] X[t][j].
  // N stays in Us (read only); X goes to T2s.  A lane only reads the column it
  // writes itself, so no synchronisation is needed inside the solve.
  if (tid < C) {
    const int j = tid;
    for (int i = j + 1; i < C; ++i) {
      float x = -Us[i * CP + j];
      for (int t = j + 1; t < i; ++t) x -= Us[i * CP + t] * T2s[t * CP + j];
      T2s[i * CP + j] = x;
    }
  }
  __syncthreads();
  // U = X D:  U[i][j] = X[i][j] beta_j (j < i), beta_i (j == i), 0 above.
  for (int idx = tid; idx < C * C; idx += NT) {
    const int i = idx / C, j = idx % C;
    Us[i * CP + j] = j < i ? T2s[i * CP + j] * bs[j] : (j == i ? bs[i] : 0.f);
  }
  __syncthreads();

  // UW = U W  (C x D) and SK = strictLower(W K^T) into P1s (temporary).
  for (int idx = tid; idx < C * D; idx += NT) {
    const int s = idx / D, col = idx % D;
    float acc = 0.f;
    for (int t = 0; t <= s; ++t) acc += Us[s * CP + t] * Ws[t * DP + col];
    UWs[s * DP + col] = acc;
  }
  for (int idx = tid; idx < C * C; idx += NT) {
    const int t = idx / C, j = idx % C;
    float acc = 0.f;
    if (t > j) {
      const E *kr = kc + (size_t)j * D;
      for (int e = 0; e < D; ++e) acc += Ws[t * DP + e] * to_f32(kr[e]);
    }
    P1s[t * CP + j] = acc;
  }
  __syncthreads();

  // T2 = U SK:  T2[s][j] = sum_{j<t<=s} U[s][t] SK[t][j]  (zero unless s > j).
  for (int idx = tid; idx < C * C; idx += NT) {
    const int s = idx / C, j = idx % C;
    float acc = 0.f;
    for (int t = j + 1; t <= s; ++t) acc += Us[s * CP + t] * P1s[t * CP + j];
    T2s[s * CP + j] = acc;
  }
  __syncthreads();

  // P1 = lower(Q W^T):  P1[i][t] = q_i . w_t for t <= i.
  for (int idx = tid; idx < C * C; idx += NT) {
    const int i = idx / C, t = idx % C;
    float acc = 0.f;
    if (t <= i) {
      const E *qr = qc + (size_t)i * D;
      for (int e = 0; e < D; ++e) acc += to_f32(qr[e]) * Ws[t * DP + e];
    }
    P1s[i * CP + t] = acc;
  }
  __syncthreads();

  // <-Q = Q - P1 UW  (float32, natural layout).
  float *qa_c = qa + row0 * D;
  for (int idx = tid; idx < C * D; idx += NT) {
    const int i = idx / D, col = idx % D;
    float acc = to_f32(qc[idx]);
    for (int t = 0; t <= i; ++t) acc -= P1s[i * CP + t] * UWs[t * DP + col];
    qa_c[idx] = acc;
  }

  // Al = lower(Q K^T) - P1 T2  (raw logits of the diagonal block; 0 above).
  float *al_c = al + ((size_t)bh * N + c) * C * C;
  for (int idx = tid; idx < C * C; idx += NT) {
    const int i = idx / C, j = idx % C;
    float acc = 0.f;
    if (j <= i) {
      const E *qr = qc + (size_t)i * D, *kr = kc + (size_t)j * D;
      for (int e = 0; e < D; ++e) acc += to_f32(qr[e]) * to_f32(kr[e]);
      for (int t = j + 1; t <= i; ++t) acc -= P1s[i * CP + t] * T2s[t * CP + j];
    }
    al_c[idx] = acc;
  }

  // Matrix-core operands in fragment order (see path_attn_internal.h).
  E *kf = kvm + ((size_t)bh * N + c) * kvm_elems(D);
  E *vf = kf + C * D;
  E *mf = vf + C * D;
  // KF: X[key][dcol] = ->K[key][dcol] = K[key][dcol] - sum_{s>key} T2[s][key] W[s][dcol]
  {
    constexpr int NS = D / KSTEP, ITEMS = 2 * NS * 64;
    for (int it = tid; it < ITEMS; it += NT) {
      const int blob = it / 64, lane = it % 64;
      const int mb = blob / NS, s = blob % NS, g = lane / 32;
      const int key = 32 * mb + lane % 32;
      E vals[KPL];
#pragma unroll
      for (int t = 0; t < KPL; ++t) {
        const int dcol = frag_row(s, g, t, KPL);
        float acc = to_f32(kc[(size_t)key * D + dcol]);
        for (int r = key + 1; r < C; ++r) acc -= T2s[r * CP + key] * Ws[r * DP + dcol];
        vals[t] = from_f32<E>(acc);
      }
#pragma unroll
      for (int t = 0; t < KPL; ++t) kf[(size_t)blob * 64 * KPL + lane * KPL + t] = vals[t];
    }
  }
  // VF: X[dd][key] = V[key][dd]
  {
    constexpr int NS = C / KSTEP, ITEMS = (D / 32) * NS * 64;
    for (int it = tid; it < ITEMS; it += NT) {
      const int blob = it / 64, lane = it % 64;
      const int mb = blob / NS, s = blob % NS, g = lane / 32;
      const int dd = 32 * mb + lane % 32;
#pragma unroll
      for (int t = 0; t < KPL; ++t)
        vf[(size_t)blob * 64 * KPL + lane * KPL + t] =
            vc[(size_t)frag_row(s, g, t, KPL) * D + dd];
    }
  }
  // MF: X[b][a] = -M[a][b] = -sum_s W[s][a] UW[s][b]
  {
    constexpr int NS = D / KSTEP, ITEMS = (D / 32) * NS * 64;
    for (int it = tid; it < ITEMS; it += NT) {
      const int blob = it / 64, lane = it % 64;
      const int mb = blob / NS, s = blob % NS, g = lane / 32;
      const int b = 32 * mb + lane % 32;
      E vals[KPL];
#pragma unroll
      for (int t = 0; t < KPL; ++t) {
        const int a = frag_row(s, g, t, KPL);
        float acc = 0.f;
        for (int r = 0; r < C; ++r) acc += Ws[r * DP + a] * UWs[r * DP + b];
        vals[t] = from_f32<E>(-acc);
      }
#pragma unroll
      for (int t = 0; t < KPL; ++t) mf[(size_t)blob * 64 * KPL + lane * KPL + t] = vals[t];
    }
  }
}

// Debug unpack of the workspace into natural float32 layouts.
template <typename E, int D>
__global__ __launch_bounds__(256) void unpack_kernel(
    const float *__restrict__ qa_ws, const E *__restrict__ kvm,
    const float *__restrict__ al_ws, const float *__restrict__ gate,
    float *__restrict__ qa, float *__restrict__ kb, float *__restrict__ m,
    float *__restrict__ al, float *__restrict__ lam, int T) {
  constexpr int C = kChunk, KPL = Kpl<E>::value, KSTEP = 2 * KPL;
  const int N = T / C;
  const int bh = blockIdx.x / N, c = blockIdx.x % N;
  const size_t row0 = (size_t)bh * T + (size_t)c * C;
  const int tid = threadIdx.x;
  if (qa)
    for (int idx = tid; idx < C * D; idx += 256) qa[row0 * D + idx] = qa_ws[row0 * D + idx];
  if (al) {
    const size_t o = ((size_t)bh * N + c) * C * C;
    for (int idx = tid; idx < C * C; idx += 256) al[o + idx] = al_ws[o + idx];
  }
  if (lam && gate)
    for (int idx = tid; idx < C; idx += 256)
      lam[row0 + idx] = -0.69314718055994531f * gate[row0 + idx];
  const E *kf = kvm + ((size_t)bh * N + c) * kvm_elems(D);
  const E *mf = kf + 2 * C * D;
  if (kb) {
    constexpr int NS = D / KSTEP;
    for (int e = tid; e < C * D; e += 256) {
      const int blob = e / (64 * KPL), lane = (e / KPL) % 64, t = e % KPL;
      const int mb = blob / NS, s = blob % NS;
      kb[(row0 + 32 * mb + lane % 32) * D + frag_row(s, lane / 32, t, KPL)] = to_f32(kf[e]);
    }
  }
  if (m) {
    constexpr int NS = D / KSTEP;
    float *mc = m + ((size_t)bh * N + c) * D * D;
    for (int e = tid; e < D * D; e += 256) {
      const int blob = e / (64 * KPL), lane = (e / KPL) % 64, t = e % KPL;
      const int mb = blob / NS, s = blob % NS;
      const int b = 32 * mb + lane % 32, a = frag_row(s, lane / 32, t, KPL);
      mc[(size_t)a * D + b] = -to_f32(mf[e]);
    }
  }
}

template <typename E, int D>
hipError_t launch_prep_t(const void *q, const void *k, const void *v,
                         const void *w, const float *beta, float *qa, void *kvm,
                         float *al, int BH, int T, hipStream_t stream) {
  const int blocks = BH * (T / kChunk);
  hipLaunchKernelGGL((prep_kernel<E, D>), dim3(blocks), dim3(256), 0, stream,
                     (const E *)q, (const E *)k, (const E *)v, (const E *)w,
                     beta, qa, (E *)kvm, al, T);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_unpack_t(const float *qa_ws, const void *kvm,
                           const float *al_ws, const float *gate, float *qa,
                           float *kb, float *m, float *al, float *lam, int BH,
                           int T, hipStream_t stream) {
  const int blocks = BH * (T / kChunk);
  hipLaunchKernelGGL((unpack_kernel<E, D>), dim3(blocks), dim3(256), 0, stream,
                     qa_ws, (const E *)kvm, al_ws, gate, qa, kb, m, al, lam, T);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_prefix(const float *logf, float *gate, int BH, int T,
                              hipStream_t stream) {
  hipLaunchKernelGGL(gate_prefix_kernel, dim3(BH), dim3(256), 0, stream, logf,
                     gate, T);
  return hipGetLastError();
}

hipError_t launch_prep(int dtype, int D, const void *q, const void *k,
                       const void *v, const void *w, const float *beta,
                       float *qa, void *kvm, float *al, int BH, int T,
                       hipStream_t stream) {
  if (dtype == 1) {
    if (D == 64) return launch_prep_t<__bf16, 64>(q, k, v, w, beta, qa, kvm, al, BH, T, stream);
    return launch_prep_t<__bf16, 128>(q, k, v, w, beta, qa, kvm, al, BH, T, stream);
  }
  if (D == 64) return launch_prep_t<float, 64>(q, k, v, w, beta, qa, kvm, al, BH, T, stream);
  return launch_prep_t<float, 128>(q, k, v, w, beta, qa, kvm, al, BH, T, stream);
}

hipError_t launch_unpack(int dtype, int D, const float *qa_ws, const void *kvm,
                         const float *al_ws, const float *gate, float *qa,
                         float *kb, float *m, float *al, float *lam, int BH,
                         int T, hipStream_t stream) {
  if (dtype == 1) {
    if (D == 64)
      return launch_unpack_t<__bf16, 64>(qa_ws, kvm, al_ws, gate, qa, kb, m, al, lam, BH, T, stream);
    return launch_unpack_t<__bf16, 128>(qa_ws, kvm, al_ws, gate, qa, kb, m, al, lam, BH, T, stream);
  }
  if (D == 64)
    return launch_unpack_t<float, 64>(qa_ws, kvm, al_ws, gate, qa, kb, m, al, lam, BH, T, stream);
  return launch_unpack_t<float, 128>(qa_ws, kvm, al_ws, gate, qa, kb, m, al, lam, BH, T, stream);
}

}  // namespace pathattn
