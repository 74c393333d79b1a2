// prep.hip -- forget-gate prefix sum and per-chunk UT preparation.
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
// The triangular solve and every intermediate are kept in float32 precision:
// the pages report bf16 arithmetic to be unstable for beta near 2
// (author-response page, on the range of beta).  Two kernels compute the same
// quantities:
//   * prep_bf16_kernel (bf16 inputs): all products on bf16 matrix cores with
//     float32 accumulation.  Products of the bf16 inputs (W W^T, Q W^T, W K^T,
//     K Q^T) are exact before the float32 sums; a float32 intermediate x enters
//     a product as the pair hi = bf16(x), lo = bf16(x - hi) (about 16
//     significant bits), with hi*hi + hi*lo + lo*hi for two such operands.
//     The triangular inverse is a blocked float32 computation on the vector
//     units.
//   * prep_f32_kernel (float32 inputs): plain float32 arithmetic on the vector
//     units.
// Only the operands handed to the streaming kernel's matrix cores (->K, V,
// -M^T) are rounded to the storage type, once, at the end.
#include "path_attn_internal.h"

namespace pathattn {

namespace {

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

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

// ---------------------------------------------------------------- bf16 path

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  return z;
}

// acc += A[0..32)[0..K) * Bt[0..32)[0..K)^T on one wave: A and Bt are bf16 in
// LDS with the contraction index contiguous (row pitches PA, PB elements).
template <int K>
__device__ __forceinline__ void tile_mma(f32x16 &acc, const __bf16 *A, int PA,
                                         const __bf16 *Bt, int PB, int lane) {
  const __bf16 *a = A + (lane & 31) * PA + 8 * (lane >> 5);
  const __bf16 *b = Bt + (lane & 31) * PB + 8 * (lane >> 5);
#pragma unroll
  for (int ks = 0; ks < K / 16; ++ks)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        *reinterpret_cast<const bf16x8 *>(a + 16 * ks),
        *reinterpret_cast<const bf16x8 *>(b + 16 * ks), acc, 0, 0, 0);
}

__device__ __forceinline__ void store_split(__bf16 *hi, __bf16 *lo, int idx, float x) {
  const __bf16 h = (__bf16)x;
  hi[idx] = h;
  lo[idx] = (__bf16)(x - (float)h);
}

// X_pq = -X_pp * sum_{t=16q}^{16p-1} N[16p+i][t] X[t][16q+j] for the blocks
// (p, q) = (q + dist, q), q = 0 .. 3-dist, of the blocked unit-lower-triangular
// inverse X = (I + N)^{-1} (16 x 16 blocks).  Ys holds 256 floats per block.
template <int DIST>
__device__ __forceinline__ void solve_band(const float *Ns, float *Xs, float *Ys,
                                           int tid) {
  constexpr int PN = 65, NB = 4 - DIST;
  for (int o = tid; o < NB * 256; o += 256) {
    const int q = o >> 8, i = (o >> 4) & 15, j = o & 15, p = q + DIST;
    float y = 0.f;
    for (int t = 16 * q; t < 16 * p; ++t) y += Ns[(16 * p + i) * PN + t] * Xs[t * PN + 16 * q + j];
    Ys[o] = y;
  }
  __syncthreads();
  for (int o = tid; o < NB * 256; o += 256) {
    const int q = o >> 8, i = (o >> 4) & 15, j = o & 15, p = q + DIST;
    float x = 0.f;
#pragma unroll
    for (int t = 0; t < 16; ++t) x -= Xs[(16 * p + i) * PN + 16 * p + t] * Ys[q * 256 + t * 16 + j];
    Xs[(16 * p + i) * PN + 16 * q + j] = x;
  }
  __syncthreads();
}

// One block of 4 waves per (bh, chunk).  Every 64x64 product is split in four
// 32x32 output tiles, one per wave (tile (w>>1, w&1)); products with a d-sized
// output dimension give each wave several tiles (tile index w + 4u).
template <int D>
__global__ __launch_bounds__(256) void prep_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k,
    const __bf16 *__restrict__ v, const __bf16 *__restrict__ w,
    const float *__restrict__ beta, float *__restrict__ qa,
    __bf16 *__restrict__ kvm, float *__restrict__ al, int T) {
  constexpr int C = kChunk, PD = D + 8, P64 = 72, PN = 65;
  constexpr int NDB = D / 32, NSD = D / 16, NSK = C / 16;
  constexpr int TPW = D / 64;  // d x 64 output tiles per wave
  constexpr int A_BYTES = (3 * C * PD * 2 > 4 * C * P64 * 2) ? 3 * C * PD * 2 : 4 * C * P64 * 2;
  constexpr int B_SOLVE = 2 * C * PN * 4 + 768 * 4;
  constexpr int B_BYTES = (B_SOLVE > 2 * D * P64 * 2) ? B_SOLVE : 2 * D * P64 * 2;
  constexpr int C_BYTES = 4 * C * P64 * 2 + D * P64 * 2 + C * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[A_BYTES + B_BYTES + C_BYTES];
  // region A: W, Q, K (inputs), later U and T2^T (hi/lo planes)
  __bf16 *Ws = reinterpret_cast<__bf16 *>(smem);
  __bf16 *Qs = Ws + C * PD;
  __bf16 *Ks = Qs + C * PD;
  __bf16 *Uh = reinterpret_cast<__bf16 *>(smem);
  __bf16 *Ul = Uh + C * P64;
  __bf16 *T2h = Ul + C * P64;
  __bf16 *T2l = T2h + C * P64;
  // region B: the solve (N, X, scratch), later (U W)^T (hi/lo planes)
  float *Ns = reinterpret_cast<float *>(smem + A_BYTES);
  float *Xs = Ns + C * PN;
  float *Ys = Xs + C * PN;
  __bf16 *UWh = reinterpret_cast<__bf16 *>(smem + A_BYTES);
  __bf16 *UWl = UWh + D * P64;
  // region C: lower(Q W^T), strictLower(W K^T)^T (hi/lo planes), W^T, beta
  __bf16 *P1h = reinterpret_cast<__bf16 *>(smem + A_BYTES + B_BYTES);
  __bf16 *P1l = P1h + C * P64;
  __bf16 *SKh = P1l + C * P64;
  __bf16 *SKl = SKh + C * P64;
  __bf16 *Wt = SKl + C * P64;
  float *bs = reinterpret_cast<float *>(Wt + D * P64);

  const int N = T / C;
  const int bh = blockIdx.x / N, c = blockIdx.x % N;
  const size_t row0 = (size_t)bh * T + (size_t)c * C;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, n = lane & 31;
  const int mt = wv >> 1, nt = wv & 1;
  const __bf16 *qc = q + row0 * D;
  const __bf16 *kc = k + row0 * D;
  const __bf16 *vc = v + row0 * D;
  const __bf16 *wc = w + row0 * D;
  __bf16 *kf = kvm + ((size_t)bh * N + c) * kvm_elems(D);
  __bf16 *vf = kf + C * D;
  __bf16 *mf = vf + C * D;

  // VF: X[dd][key] = V[key][dd] in fragment order (global to global).
  for (int item = tid; item < NDB * NSK * 64; item += 256) {
    const int blob = item >> 6, mb = blob / NSK, s = blob % NSK;
    const int dd = 32 * mb + n;
    bf16x8 x;
#pragma unroll
    for (int t = 0; t < 8; ++t) x[t] = vc[(size_t)frag_row(s, g, t, 8) * D + dd];
    *reinterpret_cast<bf16x8 *>(vf + blob * 512 + lane * 8) = x;
  }
  // W, Q, K into LDS (natural layout, padded rows), beta.
  for (int idx = tid; idx < C * D / 8; idx += 256) {
    const int row = idx / (D / 8), c8 = idx % (D / 8);
    *reinterpret_cast<bf16x8 *>(Ws + row * PD + 8 * c8) = *reinterpret_cast<const bf16x8 *>(wc + row * D + 8 * c8);
    *reinterpret_cast<bf16x8 *>(Qs + row * PD + 8 * c8) = *reinterpret_cast<const bf16x8 *>(qc + row * D + 8 * c8);
    *reinterpret_cast<bf16x8 *>(Ks + row * PD + 8 * c8) = *reinterpret_cast<const bf16x8 *>(kc + row * D + 8 * c8);
  }
  if (tid < C) bs[tid] = beta[row0 + tid];
  __syncthreads();

  // ---- phase 1: products of the inputs (contraction over d) ----
  f32x16 gacc = zero16(), p1acc = zero16(), skacc = zero16(), kq = zero16();
  tile_mma<D>(gacc, Ws + 32 * mt * PD, PD, Ws + 32 * nt * PD, PD, lane);   // W W^T
  tile_mma<D>(p1acc, Qs + 32 * mt * PD, PD, Ws + 32 * nt * PD, PD, lane);  // Q W^T
  tile_mma<D>(skacc, Ks + 32 * mt * PD, PD, Ws + 32 * nt * PD, PD, lane);  // K W^T
  tile_mma<D>(kq, Ks + 32 * mt * PD, PD, Qs + 32 * nt * PD, PD, lane);     // K Q^T
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 32 * mt + acc_row(r, g), col = 32 * nt + n;
    Ns[row * PN + col] = col < row ? bs[row] * gacc[r] : 0.f;          // N = strictLower(D W W^T)
    store_split(P1h, P1l, row * P64 + col, col <= row ? p1acc[r] : 0.f);  // lower(Q W^T)[i][t]
    store_split(SKh, SKl, row * P64 + col, col > row ? skacc[r] : 0.f);   // strictLower(W K^T)^T[j][t]
  }
  // Initial values of the <-Q^T and ->K^T tiles: Q^T and K^T.
  f32x16 qinit[TPW], kinit[TPW];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tau = wv + 4 * u, eb = tau >> 1, xb = tau & 1;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int e0 = 32 * eb + 8 * r4 + 4 * g, x = 32 * xb + n;
      const bf16x4 qv = *reinterpret_cast<const bf16x4 *>(Qs + x * PD + e0);
      const bf16x4 kv = *reinterpret_cast<const bf16x4 *>(Ks + x * PD + e0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qinit[u][4 * r4 + e] = (float)qv[e];
        kinit[u][4 * r4 + e] = (float)kv[e];
      }
    }
  }
  // W^T (rows e, contraction index t contiguous).
  for (int idx = tid; idx < C * D; idx += 256) {
    const int t = idx & 63, e = idx >> 6;
    Wt[e * P64 + t] = Ws[t * PD + e];
  }
  __syncthreads();

  // ---- phase 2: U = (I + N)^{-1} D, blocked (16 x 16 blocks), float32 ----
  if (wv == 0) {
    // diagonal blocks by forward substitution: lane = (block b, column j)
    const int b = lane >> 4, j = lane & 15, base = 16 * b;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = i == j ? 1.f : 0.f;
#pragma unroll
      for (int t = 0; t < i; ++t) acc -= Ns[(base + i) * PN + base + t] * x[t];
      x[i] = acc;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) Xs[(base + i) * PN + base + j] = x[i];
  }
  __syncthreads();
  solve_band<1>(Ns, Xs, Ys, tid);
  solve_band<2>(Ns, Xs, Ys, tid);
  solve_band<3>(Ns, Xs, Ys, tid);
  for (int idx = tid; idx < C * C; idx += 256) {
    const int i = idx >> 6, j = idx & 63;
    const float x = j < i ? Xs[i * PN + j] : (j == i ? 1.f : 0.f);
    store_split(Uh, Ul, i * P64 + j, x * bs[j]);
  }
  __syncthreads();

  // ---- phase 3: (U W)^T and T2^T = (U strictLower(W K^T))^T ----
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tau = wv + 4 * u, eb = tau >> 1, sb = tau & 1;
    f32x16 acc = zero16();
    tile_mma<C>(acc, Wt + 32 * eb * P64, P64, Uh + 32 * sb * P64, P64, lane);
    tile_mma<C>(acc, Wt + 32 * eb * P64, P64, Ul + 32 * sb * P64, P64, lane);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      store_split(UWh, UWl, (32 * eb + acc_row(r, g)) * P64 + 32 * sb + n, acc[r]);
  }
  {
    f32x16 acc = zero16();
    tile_mma<C>(acc, SKh + 32 * mt * P64, P64, Uh + 32 * nt * P64, P64, lane);
    tile_mma<C>(acc, SKh + 32 * mt * P64, P64, Ul + 32 * nt * P64, P64, lane);
    tile_mma<C>(acc, SKl + 32 * mt * P64, P64, Uh + 32 * nt * P64, P64, lane);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      store_split(T2h, T2l, (32 * mt + acc_row(r, g)) * P64 + 32 * nt + n, acc[r]);
  }
  __syncthreads();

  // ---- phase 4: outputs ----
  float *qa_c = qa + ((size_t)bh * N + c) * qa_floats(D);
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int tau = wv + 4 * u, eb = tau >> 1, ib = tau & 1;
    // <-Q^T = Q^T - (U W)^T lower(Q W^T)^T
    f32x16 acc = zero16();
    tile_mma<C>(acc, UWh + 32 * eb * P64, P64, P1h + 32 * ib * P64, P64, lane);
    tile_mma<C>(acc, UWh + 32 * eb * P64, P64, P1l + 32 * ib * P64, P64, lane);
    tile_mma<C>(acc, UWl + 32 * eb * P64, P64, P1h + 32 * ib * P64, P64, lane);
    float *dst = qa_c + ((ib * NDB + eb) * 64 + lane) * 16;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = qinit[u][4 * r4 + e] - acc[4 * r4 + e];
      *reinterpret_cast<f32x4 *>(dst + 4 * r4) = x;
    }
    // ->K^T = K^T - W^T T2 (tile (eb, jb = ib)), into KF fragment blobs
    f32x16 kacc = zero16();
    tile_mma<C>(kacc, Wt + 32 * eb * P64, P64, T2h + 32 * ib * P64, P64, lane);
    tile_mma<C>(kacc, Wt + 32 * eb * P64, P64, T2l + 32 * ib * P64, P64, lane);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 x;
#pragma unroll
      for (int t = 0; t < 8; ++t) x[t] = (__bf16)(kinit[u][8 * h + t] - kacc[8 * h + t]);
      *reinterpret_cast<bf16x8 *>(kf + ((ib * NSD + 2 * eb + h) * 64 + lane) * 8) = x;
    }
  }
  // -M^T in MF fragment blobs: M = W^T (U W), tiles (ab, bb).
#pragma unroll
  for (int u = 0; u < NDB * NDB / 4; ++u) {
    const int tau = wv + 4 * u, ab = tau / NDB, bb = tau % NDB;
    f32x16 acc = zero16();
    tile_mma<C>(acc, Wt + 32 * ab * P64, P64, UWh + 32 * bb * P64, P64, lane);
    tile_mma<C>(acc, Wt + 32 * ab * P64, P64, UWl + 32 * bb * P64, P64, lane);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 x;
#pragma unroll
      for (int t = 0; t < 8; ++t) x[t] = (__bf16)(-acc[8 * h + t]);
      *reinterpret_cast<bf16x8 *>(mf + ((bb * NSD + 2 * ab + h) * 64 + lane) * 8) = x;
    }
  }
  // Al^T = K Q^T - T2^T lower(Q W^T)^T, tile (jb = mt, ib = nt); the tile with
  // keys 32..63 and queries 0..31 lies above the diagonal and is not stored.
  if (!(mt == 1 && nt == 0)) {
    f32x16 acc = zero16();
    tile_mma<C>(acc, T2h + 32 * mt * P64, P64, P1h + 32 * nt * P64, P64, lane);
    tile_mma<C>(acc, T2h + 32 * mt * P64, P64, P1l + 32 * nt * P64, P64, lane);
    tile_mma<C>(acc, T2l + 32 * mt * P64, P64, P1h + 32 * nt * P64, P64, lane);
    float *dst = al + ((size_t)bh * N + c) * al_floats() + (al_tile(nt, mt) * 64 + lane) * 16;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = kq[4 * r4 + e] - acc[4 * r4 + e];
      *reinterpret_cast<f32x4 *>(dst + 4 * r4) = x;
    }
  }
}

// ---------------------------------------------------------------- fp32 path

// One block of 256 threads per (bh, chunk), plain float32 on the vector units.
// LDS: W and U W (64 x D, padded), U, P1 = lower(Q W^T) and T2 = U
// strictLower(W K^T) (64 x 64, padded).
template <int D>
__global__ __launch_bounds__(256) void prep_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k,
    const float *__restrict__ v, const float *__restrict__ w,
    const float *__restrict__ beta, float *__restrict__ qa,
    float *__restrict__ kvm, float *__restrict__ al, int T) {
  constexpr int C = kChunk, DP = D + 1, CP = C + 1, NT = 256;
  constexpr int KPL = 1, KSTEP = 2;
  __shared__ float Ws[C * DP];
  __shared__ float UWs[C * DP];
  __shared__ float Us[C * CP];
  __shared__ float P1s[C * CP];
  __shared__ float T2s[C * CP];
  __shared__ float bs[C];

  const int N = T / C;
  const int bh = blockIdx.x / N, c = blockIdx.x % N;
  const size_t row0 = (size_t)bh * T + (size_t)c * C;
  const int tid = threadIdx.x;
  const float *qc = q + row0 * D;
  const float *kc = k + row0 * D;
  const float *vc = v + row0 * D;
  const float *wc = w + row0 * D;

  for (int idx = tid; idx < C * D; idx += NT) Ws[(idx / D) * DP + idx % D] = wc[idx];
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
  // Forward substitution for X = (I + N)^{-1}, one column per lane of wave 0:
  // X[i][j] = -N[i][j] - sum_{j<t<i} N[i][t] X[t][j].  N stays in Us (read
  // only); X goes to T2s.  A lane only reads the column it writes itself.
  if (tid < C) {
    const int j = tid;
    for (int i = j + 1; i < C; ++i) {
      float x = -Us[i * CP + j];
      for (int t = j + 1; t < i; ++t) x -= Us[i * CP + t] * T2s[t * CP + j];
      T2s[i * CP + j] = x;
    }
  }
  __syncthreads();
  for (int idx = tid; idx < C * C; idx += NT) {
    const int i = idx / C, j = idx % C;
    Us[i * CP + j] = j < i ? T2s[i * CP + j] * bs[j] : (j == i ? bs[i] : 0.f);
  }
  __syncthreads();
  // UW = U W and SK = strictLower(W K^T) (into P1s for now).
  for (int idx = tid; idx < C * D; idx += NT) {
    const int s = idx / D, col = idx % D;
    float acc = 0.f;
    for (int t = 0; t <= s; ++t) acc += Us[s * CP + t] * Ws[t * DP + col];
    UWs[s * DP + col] = acc;
  }
  for (int idx = tid; idx < C * C; idx += NT) {
    const int t = idx / C, j = idx % C;
    float acc = 0.f;
    if (t > j)
      for (int e = 0; e < D; ++e) acc += Ws[t * DP + e] * kc[(size_t)j * D + e];
    P1s[t * CP + j] = acc;
  }
  __syncthreads();
  // T2 = U SK: T2[s][j] = sum_{j<t<=s} U[s][t] SK[t][j].
  for (int idx = tid; idx < C * C; idx += NT) {
    const int s = idx / C, j = idx % C;
    float acc = 0.f;
    for (int t = j + 1; t <= s; ++t) acc += Us[s * CP + t] * P1s[t * CP + j];
    T2s[s * CP + j] = acc;
  }
  __syncthreads();
  // P1 = lower(Q W^T).
  for (int idx = tid; idx < C * C; idx += NT) {
    const int i = idx / C, t = idx % C;
    float acc = 0.f;
    if (t <= i)
      for (int e = 0; e < D; ++e) acc += qc[(size_t)i * D + e] * Ws[t * DP + e];
    P1s[i * CP + t] = acc;
  }
  __syncthreads();

  // <-Q = Q - P1 UW, register image [w][mb][lane][r].
  float *qa_c = qa + ((size_t)bh * N + c) * qa_floats(D);
  for (int idx = tid; idx < C * D; idx += NT) {
    const int r = idx & 15, lane = (idx >> 4) & 63, blk = idx >> 10;
    const int wq = blk / (D / 32), mb = blk % (D / 32);
    const int i = 32 * wq + (lane & 31), col = 32 * mb + acc_row(r, lane >> 5);
    float acc = qc[(size_t)i * D + col];
    for (int t = 0; t <= i; ++t) acc -= P1s[i * CP + t] * UWs[t * DP + col];
    qa_c[idx] = acc;
  }
  // Al = lower(Q K^T) - P1 T2, register image of the three stored tiles.
  float *al_c = al + ((size_t)bh * N + c) * al_floats();
  for (int idx = tid; idx < al_floats(); idx += NT) {
    const int r = idx & 15, lane = (idx >> 4) & 63, tile = idx >> 10;
    const int wq = tile == 0 ? 0 : 1, mb = tile == 2 ? 1 : 0;
    const int i = 32 * wq + (lane & 31), j = 32 * mb + acc_row(r, lane >> 5);
    float acc = 0.f;
    if (j <= i) {
      for (int e = 0; e < D; ++e) acc += qc[(size_t)i * D + e] * kc[(size_t)j * D + e];
      for (int t = j + 1; t <= i; ++t) acc -= P1s[i * CP + t] * T2s[t * CP + j];
    }
    al_c[idx] = acc;
  }

  // Matrix-core operands in fragment order.
  float *kf = kvm + ((size_t)bh * N + c) * kvm_elems(D);
  float *vf = kf + C * D;
  float *mf = vf + C * D;
  {  // KF: ->K[key][dcol] = K[key][dcol] - sum_{s>key} T2[s][key] W[s][dcol]
    constexpr int NS = D / KSTEP;
    for (int it = tid; it < 2 * NS * 64; it += NT) {
      const int blob = it / 64, lane = it % 64, mb = blob / NS, s = blob % NS;
      const int key = 32 * mb + lane % 32, dcol = frag_row(s, lane / 32, 0, KPL);
      float acc = kc[(size_t)key * D + dcol];
      for (int r = key + 1; r < C; ++r) acc -= T2s[r * CP + key] * Ws[r * DP + dcol];
      kf[it] = acc;
    }
  }
  {  // VF: X[dd][key] = V[key][dd]
    constexpr int NS = C / KSTEP;
    for (int it = tid; it < (D / 32) * NS * 64; it += NT) {
      const int blob = it / 64, lane = it % 64, mb = blob / NS, s = blob % NS;
      vf[it] = vc[(size_t)frag_row(s, lane / 32, 0, KPL) * D + 32 * mb + lane % 32];
    }
  }
  {  // MF: X[b][a] = -M[a][b] = -sum_s W[s][a] UW[s][b]
    constexpr int NS = D / KSTEP;
    for (int it = tid; it < (D / 32) * NS * 64; it += NT) {
      const int blob = it / 64, lane = it % 64, mb = blob / NS, s = blob % NS;
      const int b = 32 * mb + lane % 32, a = frag_row(s, lane / 32, 0, KPL);
      float acc = 0.f;
      for (int r = 0; r < C; ++r) acc += Ws[r * DP + a] * UWs[r * DP + b];
      mf[it] = -acc;
    }
  }
}

// ---------------------------------------------------------------- unpack

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
  if (qa) {
    const float *src = qa_ws + ((size_t)bh * N + c) * qa_floats(D);
    for (int idx = tid; idx < C * D; idx += 256) {
      const int r = idx & 15, lane = (idx >> 4) & 63, blk = idx >> 10;
      const int wq = blk / (D / 32), mb = blk % (D / 32);
      qa[(row0 + 32 * wq + (lane & 31)) * D + 32 * mb + acc_row(r, lane >> 5)] = src[idx];
    }
  }
  if (al) {
    const float *src = al_ws + ((size_t)bh * N + c) * al_floats();
    float *dst = al + ((size_t)bh * N + c) * C * C;
    for (int idx = tid; idx < C * C; idx += 256) {  // tile above the diagonal
      const int i = idx / C, j = idx % C;
      if (i < 32 && j >= 32) dst[idx] = 0.f;
    }
    for (int idx = tid; idx < al_floats(); idx += 256) {
      const int r = idx & 15, lane = (idx >> 4) & 63, tile = idx >> 10;
      const int wq = tile == 0 ? 0 : 1, mb = tile == 2 ? 1 : 0;
      dst[(32 * wq + (lane & 31)) * C + 32 * mb + acc_row(r, lane >> 5)] = src[idx];
    }
  }
  if (lam && gate)
    for (int idx = tid; idx < C; idx += 256)
      lam[row0 + idx] = -0.69314718055994531f * gate[row0 + idx];
  const E *kf = kvm + ((size_t)bh * N + c) * kvm_elems(D);
  const E *mf = kf + 2 * C * D;
  constexpr int NS = D / KSTEP;
  if (kb) {
    for (int e = tid; e < C * D; e += 256) {
      const int blob = e / (64 * KPL), lane = (e / KPL) % 64, t = e % KPL;
      const int mb = blob / NS, s = blob % NS;
      kb[(row0 + 32 * mb + lane % 32) * D + frag_row(s, lane / 32, t, KPL)] = to_f32(kf[e]);
    }
  }
  if (m) {
    float *mc = m + ((size_t)bh * N + c) * D * D;
    for (int e = tid; e < D * D; e += 256) {
      const int blob = e / (64 * KPL), lane = (e / KPL) % 64, t = e % KPL;
      const int mb = blob / NS, s = blob % NS;
      const int b = 32 * mb + lane % 32, a = frag_row(s, lane / 32, t, KPL);
      mc[(size_t)a * D + b] = -to_f32(mf[e]);
    }
  }
}

template <int D>
hipError_t launch_prep_bf16(const void *q, const void *k, const void *v,
                            const void *w, const float *beta, float *qa,
                            void *kvm, float *al, int BH, int T,
                            hipStream_t stream) {
  hipLaunchKernelGGL((prep_bf16_kernel<D>), dim3(BH * (T / kChunk)), dim3(256), 0,
                     stream, (const __bf16 *)q, (const __bf16 *)k,
                     (const __bf16 *)v, (const __bf16 *)w, beta, qa,
                     (__bf16 *)kvm, al, T);
  return hipGetLastError();
}

template <int D>
hipError_t launch_prep_f32(const void *q, const void *k, const void *v,
                           const void *w, const float *beta, float *qa,
                           void *kvm, float *al, int BH, int T,
                           hipStream_t stream) {
  hipLaunchKernelGGL((prep_f32_kernel<D>), dim3(BH * (T / kChunk)), dim3(256), 0,
                     stream, (const float *)q, (const float *)k,
                     (const float *)v, (const float *)w, beta, qa,
                     (float *)kvm, al, T);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_unpack_t(const float *qa_ws, const void *kvm,
                           const float *al_ws, const float *gate, float *qa,
                           float *kb, float *m, float *al, float *lam, int BH,
                           int T, hipStream_t stream) {
  hipLaunchKernelGGL((unpack_kernel<E, D>), dim3(BH * (T / kChunk)), dim3(256), 0,
                     stream, qa_ws, (const E *)kvm, al_ws, gate, qa, kb, m, al,
                     lam, T);
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
    if (D == 64) return launch_prep_bf16<64>(q, k, v, w, beta, qa, kvm, al, BH, T, stream);
    return launch_prep_bf16<128>(q, k, v, w, beta, qa, kvm, al, BH, T, stream);
  }
  if (D == 64) return launch_prep_f32<64>(q, k, v, w, beta, qa, kvm, al, BH, T, stream);
  return launch_prep_f32<128>(q, k, v, w, beta, qa, kvm, al, BH, T, stream);
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
