// bwd_sweep.hip -- the quadratic part of the backward pass on matrix cores.
//
// Notation as in backward.hip: per 64-token chunk c the forward's UT
// quantities Qa_c = <-Q_c, Kb_c = ->K_c, M_c; key level c holds the keys of
// every chunk c' < c aligned to the start of chunk c,
//     Khat[c]_{c'} = Kb_{c'} (I - M_{c'+1})^T ... (I - M_{c-1})^T,
// and the cross logits of query chunk c against key chunk c' are
// Qa_c Khat[c]_{c'}^T (PaTH slides for arXiv:2505.16381v2, frames "A
// right-to-left scan accumulates cross-block paths" and "Decoding updates
// historical keys in place").  With the forward's lse, P = exp(s - lse) and
// g = scale * P o (dO V^T - rowdot(dO, O) + dlse).  Three kernels:
//
//   levels  one block per key chunk c' walks c upward, Khat[c+1] =
//           Khat[c] - Khat[c] M_c^T, and stores every level in the input dtype
//           (float32 running value, the product taken on the rounded value,
//           as the forward scan does for its running query tile).
//   dq      one block per query chunk c: dQa_c = sum_{c'<c} g Khat[c]_{c'},
//           and the row sums of dS for the forget-gate gradient.
//   dk      one block per group of G key chunks walks c downward keeping,
//           per key chunk c', Gamma (the gradient of its level-c keys) and dV
//           in registers:  dV += P^T dO_c,  Gamma += g^T Qa_c;  crossing
//           chunk m = c-1 (if m > c'):  dM_m -= Gamma^T Khat[m]_{c'} (one
//           partial per (m, group), summed by dm_reduce), Gamma <- Gamma
//           (I - M_m);  at c = c'+1, dKb_{c'} = Gamma.  Also the column sums
//           of dS for the gate.
//
// Matrix products are 32 x 32 tiles: v_mfma_f32_32x32x16_bf16 for bf16
// inputs (operands rounded to bf16, float32 accumulation, as in the forward),
// v_mfma_f32_32x32x2f32 for float32 inputs.  Operands are read from LDS or
// global memory as rows with the contraction index contiguous (bf16: 8
// values, one 16-byte load, per lane); LDS copies are padded against bank
// conflicts.  In a 32 x 32 accumulator tile, lane l register r holds row
// acc_row(r, l/32) and column l%32.
#include <type_traits>

#include "path_attn_internal.h"

namespace pathattn {

namespace {

constexpr int C = kChunk;

template <typename E>
struct MM;

template <>
struct MM<__bf16> {
  static constexpr int KPL = 8;   // contraction values per lane per instruction
  static constexpr int PAD = 8;   // LDS row padding (elements): keeps 16-byte alignment
  using frag = bf16x8;
  __device__ static __forceinline__ frag ld(const __bf16 *p, int) {
    return *reinterpret_cast<const bf16x8 *>(p);
  }
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct MM<float> {
  static constexpr int KPL = 1;
  static constexpr int PAD = 1;
  using frag = float;
  __device__ static __forceinline__ frag ld(const float *p, int) { return *p; }
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// acc(i, j) += sum_{k<K} A(i, k) B(j, k) for i, j < 32, with
// A(i, k) = A[i*ars + k*acs] and B(j, k) = B[j*brs + k*bcs].  For bf16 the
// contraction index must be contiguous (acs = bcs = 1).
template <typename E, int K>
__device__ __forceinline__ void mma_tile(f32x16 &acc, const E *A, int ars, int acs, const E *B,
                                         int brs, int bcs, int lane) {
  constexpr int KPL = MM<E>::KPL;
  const int i = lane & 31, k0 = KPL * (lane >> 5);
  const E *pa = A + i * ars + k0 * acs;
  const E *pb = B + i * brs + k0 * bcs;
#pragma unroll
  for (int k = 0; k < K; k += 2 * KPL)
    acc = MM<E>::mma(MM<E>::ld(pa + k * acs, acs), MM<E>::ld(pb + k * bcs, bcs), acc);
}

__device__ __forceinline__ void zero16(f32x16 &a) {
#pragma unroll
  for (int r = 0; r < 16; ++r) a[r] = 0.f;
}

// dst[i*rs + j*cs] = acc(i, j) rounded to E, for this lane's 16 elements.
template <typename E>
__device__ __forceinline__ void st_tile(E *dst, int rs, int cs, const f32x16 &a, int lane) {
  const int g = lane >> 5, j = lane & 31;
  if constexpr (std::is_same<E, __bf16>::value) {
    if (rs == 1) {   // rows r%4 = 0..3 are consecutive: one 8-byte store per quad
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)a[4 * q + e];
        *reinterpret_cast<bf16x4 *>(dst + (8 * q + 4 * g) + j * cs) = v;
      }
      return;
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) dst[acc_row(r, g) * rs + j * cs] = (E)a[r];
}

// ------------------------------------------------------------------ levels

__host__ __device__ inline size_t lev_off(int c, int cp, int D) {
  return ((size_t)c * (c - 1) / 2 + cp) * (size_t)C * D;
}

// One block of 2 waves (32 keys each) per (key chunk c' < N-1, bh).
template <typename E, int D>
__global__ __launch_bounds__(128) void levels_kernel(const float *__restrict__ kb,
                                                     const float *__restrict__ m,
                                                     E *__restrict__ levels, int T, int BH) {
  constexpr int P = D + MM<E>::PAD;
  __shared__ __attribute__((aligned(16))) E Xs[C * P];
  __shared__ __attribute__((aligned(16))) E Ms[D * P];
  const int N = T / C;
  const int cp = blockIdx.x / BH, bh = blockIdx.x % BH;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 5, col = lane & 31;
  f32x16 x[D / 32];
  const float *src = kb + ((size_t)bh * T + (size_t)cp * C + 32 * wv) * D;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) x[t][r] = src[acc_row(r, g) * D + 32 * t + col];
  E *head = levels + (size_t)bh * lev_off(N, 0, D);
  for (int c = cp + 1; c < N; ++c) {
    E *dst = head + lev_off(c, cp, D) + (size_t)32 * wv * D;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) st_tile(dst + 32 * t, D, 1, x[t], lane);
    if (c + 1 >= N) break;
    __syncthreads();
    const float *mc = m + ((size_t)bh * N + c) * D * D;
    for (int idx = tid; idx < D * D; idx += 128) Ms[(idx / D) * P + idx % D] = (E)(-mc[idx]);
#pragma unroll
    for (int t = 0; t < D / 32; ++t) st_tile(Xs + 32 * wv * P + 32 * t, P, 1, x[t], lane);
    __syncthreads();
    // Khat[c+1] = Khat[c] + round(Khat[c]) (-M_c)^T
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
      mma_tile<E, D>(x[t], Xs + 32 * wv * P, P, 1, Ms + 32 * t * P, P, 1, lane);
  }
}

// ------------------------------------------------------------------ dq

// One block of 4 waves per (bh, query chunk c): wave (qh, kh) = (w & 1, w >> 1)
// takes queries 32 qh.. and, at each key chunk, keys 32 kh...  Chunk 0 has no
// earlier keys: its dQa is zero.
template <typename E, int D, bool FOX>
__global__ __launch_bounds__(256) void dq_kernel(
    const float *__restrict__ qa, const E *__restrict__ dout, const float *__restrict__ lse,
    const float *__restrict__ dlse, const float *__restrict__ dvec, const float *__restrict__ lam,
    const E *__restrict__ levels, const E *__restrict__ v, float scale, float *__restrict__ dqa,
    float *__restrict__ dlam, int T, int BH) {
  constexpr bool BF = std::is_same<E, __bf16>::value;
  constexpr int PQ = D + MM<E>::PAD;          // Qs, Os: [64 q][D]
  constexpr int PK = C + MM<E>::PAD;          // Kt: [D][64 keys] (bf16) ; float: Khat rows [64][D]
  constexpr int PKF = D + MM<E>::PAD;
  constexpr int PG = 32 + MM<E>::PAD;         // Gs: per wave [32 q][32 keys]
  __shared__ __attribute__((aligned(16))) E Qs[C * PQ];
  __shared__ __attribute__((aligned(16))) E Os[C * PQ];
  __shared__ __attribute__((aligned(16))) E Kt[BF ? D * PK : C * PKF];
  __shared__ __attribute__((aligned(16))) E Gs[4 * 32 * PG];
  __shared__ float red[2 * 32 * (D + 1)];
  __shared__ float lamk[C];
  const int N = T / C;
  const int bh = blockIdx.x % BH, c = N - 1 - blockIdx.x / BH;   // longest walks first
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 5, col = lane & 31;
  const int qh = wv & 1, kh = wv >> 1;
  const size_t qrow = (size_t)bh * T + (size_t)c * C;
  if (c == 0) {
    for (int idx = tid; idx < C * D; idx += 256) dqa[qrow * D + idx] = 0.f;
    return;
  }
  for (int idx = tid; idx < C * D; idx += 256) {
    Qs[(idx / D) * PQ + idx % D] = (E)qa[qrow * D + idx];
    Os[(idx / D) * PQ + idx % D] = dout[qrow * D + idx];
  }
  const int myq = 32 * qh + col;
  const float q_lse = lse[qrow + myq], q_d = dvec[qrow + myq];
  const float q_dl = dlse ? dlse[qrow + myq] : 0.f;
  const float q_lam = FOX ? lam[qrow + myq] : 0.f;
  f32x16 dq[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) zero16(dq[t]);
  float rowsum = 0.f;
  const E *lev_c = levels + (size_t)bh * lev_off(N, 0, D) + lev_off(c, 0, D);
  E *Gw = Gs + wv * 32 * PG;
  for (int cp = c - 1; cp >= 0; --cp) {
    const E *kh_rows = lev_c + (size_t)cp * C * D;   // Khat[c]_{c'}: [64 keys][D]
    const size_t krow = (size_t)bh * T + (size_t)cp * C;
    __syncthreads();
    for (int idx = tid; idx < C * D; idx += 256) {
      const int key = idx / D, d = idx % D;
      if constexpr (BF) Kt[d * PK + key] = kh_rows[idx];
      else Kt[key * PKF + d] = kh_rows[idx];
    }
    if (FOX && tid < C) lamk[tid] = lam[krow + tid];
    __syncthreads();
    // S^T and dP^T tiles: rows = keys 32 kh.., columns = queries 32 qh..
    f32x16 s, dp;
    zero16(s);
    zero16(dp);
    mma_tile<E, D>(s, kh_rows + 32 * kh * D, D, 1, Qs + 32 * qh * PQ, PQ, 1, lane);
    mma_tile<E, D>(dp, v + (krow + 32 * kh) * D, D, 1, Os + 32 * qh * PQ, PQ, 1, lane);
    f32x16 gt;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 32 * kh + acc_row(r, g);
      const float kl = FOX ? lamk[key] : 0.f;
      const float p = __expf(scale * s[r] + q_lam - kl - q_lse);
      const float ds = p * (dp[r] - q_d + q_dl);
      rowsum += ds;
      gt[r] = scale * ds;
    }
    st_tile(Gw, 1, PG, gt, lane);   // Gw[q][key] = g(q, key)
    __syncthreads();
    // dQa^T(d, q) += sum_key Khat(key, d) g(q, key)
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      if constexpr (BF)
        mma_tile<E, 32>(dq[t], Kt + 32 * t * PK + 32 * kh, PK, 1, Gw, PG, 1, lane);
      else
        mma_tile<E, 32>(dq[t], Kt + 32 * kh * PKF + 32 * t, 1, PKF, Gw, PG, 1, lane);
    }
  }
  // combine the two key halves, then store dQa rows
  __syncthreads();
  float *rq = red + qh * 32 * (D + 1);
  if (kh == 1) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) rq[col * (D + 1) + 32 * t + acc_row(r, g)] = dq[t][r];
  }
  rowsum += __shfl_xor(rowsum, 32);
  if (kh == 1 && g == 0) lamk[32 * qh + col] = rowsum;
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * t + acc_row(r, g);
        dqa[(qrow + myq) * D + d] = dq[t][r] + rq[col * (D + 1) + d];
      }
    if (FOX && g == 0) dlam[qrow + myq] += rowsum + lamk[myq];
  }
}

// ------------------------------------------------------------------ dk

// Staging sizes (elements of E) of the dk kernel.
template <typename E, int D, int G>
struct DkLds {
  static constexpr bool BF = std::is_same<E, __bf16>::value;
  static constexpr int PAD = MM<E>::PAD;
  static constexpr int PQ = D + PAD;              // Qs, Os rows [64 q][D]
  static constexpr int PQT = C + PAD;             // Qt, Ot rows [D][64 q] (bf16 only)
  static constexpr int PP = C + PAD;              // per-wave P^T, g^T rows [32 keys][64 q]
  static constexpr int KG = 64 * G;               // keys of a group
  static constexpr int PGT = KG + PAD;            // crossing: Gamma^T, Khat^T rows [D][KG] (bf16)
  static constexpr int PGN = D + PAD;             // crossing (float): Gamma, Khat rows [KG][D]
  static constexpr int PM = D + PAD;              // -M^T rows [D][D] (bf16 only)
  static constexpr int STAGE = BF ? 2 * C * PQ + 2 * D * PQT : 2 * C * PQ;
  static constexpr int CROSS = BF ? 2 * D * PGT : 2 * KG * PGN;
  static constexpr int AREA1 = STAGE > CROSS ? STAGE : CROSS;
  static constexpr int WAVES = 2 * G;
  static constexpr int PERWAVE = 2 * 32 * PP;     // P^T and g^T
  static constexpr int GR = 32 * PGN;             // rounded Gamma rows (bf16 transition)
  static constexpr int AREA2 = WAVES * (PERWAVE > GR ? PERWAVE : GR);
  static constexpr int MS = BF ? D * PM : 0;
};

// One block of 2G waves per (group of G key chunks, bh); wave w takes keys
// 32 (w & 1).. of chunk c' = G*group + (w >> 1).
template <typename E, int D, int G, bool FOX>
__global__ __launch_bounds__(128 * G) void dk_kernel(
    const float *__restrict__ qa, const E *__restrict__ dout, const float *__restrict__ lse,
    const float *__restrict__ dlse, const float *__restrict__ dvec, const float *__restrict__ lam,
    const E *__restrict__ levels, const E *__restrict__ v, const float *__restrict__ m,
    float scale, float *__restrict__ dkb, float *__restrict__ dv, float *__restrict__ dlam,
    float *__restrict__ dmpart, int T, int BH) {
  using L = DkLds<E, D, G>;
  constexpr bool BF = L::BF;
  constexpr int NW = L::WAVES, NTH = 64 * NW;
  __shared__ __attribute__((aligned(16))) E area1[L::AREA1];
  __shared__ __attribute__((aligned(16))) E area2[L::AREA2];
  __shared__ __attribute__((aligned(16))) E Ms[L::MS > 0 ? L::MS : 1];
  __shared__ float4 qst[C];
  const int N = T / C, NG = (N + G - 1) / G;
  const int grp = blockIdx.x / BH, bh = blockIdx.x % BH;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 5, col = lane & 31;
  const int kh = wv & 1, cp = G * grp + (wv >> 1);
  const size_t head = (size_t)bh * T;
  const size_t krow = head + (size_t)cp * C + 32 * kh;   // first key row of this wave
  const bool member = cp < N;
  // staging views
  E *Qs = area1, *Os = area1 + C * L::PQ;
  E *Qt = area1 + 2 * C * L::PQ, *Ot = Qt + D * L::PQT;   // bf16 only
  E *PT = area2 + wv * L::PERWAVE, *GT = PT + 32 * L::PP;
  E *GR = area2 + wv * L::GR;                             // aliases P^T / g^T at crossings
  E *Gx = area1, *Kx = area1 + (BF ? D * L::PGT : L::KG * L::PGN);   // crossing staging
  const E *lev_head = levels + (size_t)bh * lev_off(N, 0, D);

  f32x16 gam[D / 32], dva[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    zero16(gam[t]);
    zero16(dva[t]);
  }
  float colsum = 0.f;
  const float my_lam = (FOX && member) ? lam[krow + col] : 0.f;
  const int c_low = G * grp + 1;   // last query chunk the group visits
  for (int c = N - 1; c >= c_low; --c) {
    const bool active = member && c > cp;
    const size_t qrow = head + (size_t)c * C;
    __syncthreads();
    for (int idx = tid; idx < C * D; idx += NTH) {
      const int q = idx / D, d = idx % D;
      const E a = (E)qa[qrow * D + idx], o = dout[qrow * D + idx];
      Qs[q * L::PQ + d] = a;
      Os[q * L::PQ + d] = o;
      if constexpr (BF) {
        Qt[d * L::PQT + q] = a;
        Ot[d * L::PQT + q] = o;
      }
    }
    if (tid < C)
      qst[tid] = make_float4(lse[qrow + tid], dvec[qrow + tid], dlse ? dlse[qrow + tid] : 0.f,
                             FOX ? lam[qrow + tid] : 0.f);
    const bool crossing = c - 1 > G * grp;   // some chunk of the group crosses m = c-1
    if constexpr (BF) {
      if (crossing) {
        const float *mm = m + (head / T * N + (size_t)(c - 1)) * D * D;
        for (int idx = tid; idx < D * D; idx += NTH) {
          const int d = idx / D, dp = idx % D;   // M[d][d'] -> Ms[d'][d] = -M[d][d']
          Ms[dp * L::PM + d] = (E)(-mm[idx]);
        }
      }
    }
    __syncthreads();
    const E *kl = lev_head + lev_off(c, cp < c ? cp : 0, D) + (size_t)32 * kh * D;   // Khat[c] rows
    if (active) {
      f32x16 s[2], dp[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        zero16(s[qt]);
        zero16(dp[qt]);
        mma_tile<E, D>(s[qt], Qs + 32 * qt * L::PQ, L::PQ, 1, kl, D, 1, lane);
        mma_tile<E, D>(dp[qt], Os + 32 * qt * L::PQ, L::PQ, 1, v + krow * D, D, 1, lane);
      }
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float4 st = qst[32 * qt + acc_row(r, g)];
          const float p = __expf(scale * s[qt][r] + st.w - my_lam - st.x);
          const float ds = p * (dp[qt][r] - st.y + st.z);
          colsum += ds;
          s[qt][r] = p;
          dp[qt][r] = scale * ds;
        }
        // P^T[key][q], g^T[key][q]
        st_tile(PT + 32 * qt, 1, L::PP, s[qt], lane);
        st_tile(GT + 32 * qt, 1, L::PP, dp[qt], lane);
      }
    }
    __syncthreads();
    if (active) {
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        if constexpr (BF) {
          mma_tile<E, C>(dva[t], PT, L::PP, 1, Ot + 32 * t * L::PQT, L::PQT, 1, lane);
          mma_tile<E, C>(gam[t], GT, L::PP, 1, Qt + 32 * t * L::PQT, L::PQT, 1, lane);
        } else {
          mma_tile<E, C>(dva[t], PT, L::PP, 1, Os + 32 * t, 1, L::PQ, lane);
          mma_tile<E, C>(gam[t], GT, L::PP, 1, Qs + 32 * t, 1, L::PQ, lane);
        }
      }
      if (c == cp + 1) {   // chunk c' is done: dKb = Gamma
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            dkb[(krow + acc_row(r, g)) * D + 32 * t + col] = gam[t][r];
      }
    }
    if (!crossing) continue;
    // ---- crossing of chunk m = c-1 by the group's chunks c' < m
    const int mch = c - 1;
    const bool crosses = member && cp < mch;
    __syncthreads();
    {
      const E *km = lev_head + lev_off(mch, crosses ? cp : 0, D) + (size_t)32 * kh * D;
      const int kbase = 64 * (wv >> 1) + 32 * kh;   // this wave's keys within the group
      if constexpr (BF) {
        // Gx = Gamma^T [D][KG], Kx = Khat[m]^T [D][KG]; GR = round(Gamma) rows
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          f32x16 z = gam[t];
          if (!crosses) zero16(z);
          st_tile(Gx + 32 * t * L::PGT + kbase, 1, L::PGT, z, lane);
          st_tile(GR + 32 * t, L::PGN, 1, z, lane);
        }
        for (int e = lane; e < 32 * D; e += 64) {
          const int key = e / D, d = e % D;
          Kx[d * L::PGT + kbase + key] = crosses ? km[e] : (E)0.f;
        }
      } else {
        // float: Gx = Gamma rows [KG][D] (also the transition operand), Kx = Khat[m] rows
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          f32x16 z = gam[t];
          if (!crosses) zero16(z);
          st_tile(Gx + kbase * L::PGN + 32 * t, L::PGN, 1, z, lane);
        }
        for (int e = lane; e < 32 * D; e += 64) {
          const int key = e / D, d = e % D;
          Kx[(kbase + key) * L::PGN + d] = crosses ? km[e] : (E)0.f;
        }
      }
    }
    __syncthreads();
    // dM_m partial of the group: -sum_keys Gamma(key, d) Khat[m](key, d')
    {
      constexpr int TILES = (D / 32) * (D / 32);
      float *dst = dmpart + (((size_t)bh * N + mch) * NG + grp) * D * D;
      for (int tI = wv; tI < TILES; tI += NW) {
        const int ta = tI / (D / 32), tb = tI % (D / 32);
        f32x16 acc;
        zero16(acc);
        if constexpr (BF)
          mma_tile<E, L::KG>(acc, Gx + 32 * ta * L::PGT, L::PGT, 1, Kx + 32 * tb * L::PGT,
                             L::PGT, 1, lane);
        else
          mma_tile<E, L::KG>(acc, Gx + 32 * ta, 1, L::PGN, Kx + 32 * tb, 1, L::PGN, lane);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dst[(size_t)(32 * ta + acc_row(r, g)) * D + 32 * tb + col] = -acc[r];
      }
    }
    if (crosses) {   // Gamma <- Gamma + round(Gamma) (-M_m)
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        if constexpr (BF) {
          mma_tile<E, D>(gam[t], GR, L::PGN, 1, Ms + 32 * t * L::PM, L::PM, 1, lane);
        } else {
          // B(d', d) = -M[d][d'] read from global memory
          const float *mm = m + ((size_t)bh * N + mch) * D * D;
          f32x16 acc;
          zero16(acc);
          mma_tile<E, D>(acc, Gx + (64 * (wv >> 1) + 32 * kh) * L::PGN, L::PGN, 1, mm + 32 * t,
                         1, D, lane);
#pragma unroll
          for (int r = 0; r < 16; ++r) gam[t][r] -= acc[r];
        }
      }
    }
  }
  if (!member) return;
  if (cp == N - 1) {   // no later query chunk: dKb = 0
    for (int e = lane; e < 32 * D; e += 64) dkb[krow * D + e] = 0.f;
    return;
  }
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dv[(krow + acc_row(r, g)) * D + 32 * t + col] += dva[t][r];
  if (FOX) {
    colsum += __shfl_xor(colsum, 32);
    if (g == 0) dlam[krow + col] -= colsum;
  }
}

// dM_m = sum over the groups that cross m (m in [1, N-2]); 0 otherwise.
// One block per (bh, m) and slice of DD / XB elements (XB blocks per matrix).
template <int G>
__global__ __launch_bounds__(256) void dm_reduce_kernel(const float *__restrict__ dmpart,
                                                        float *__restrict__ dm, int N, int DD,
                                                        int XB) {
  const int NG = (N + G - 1) / G;
  const size_t bm = blockIdx.x / XB;   // bh * N + m
  const int xb = blockIdx.x % XB;
  const int mch = (int)(bm % N);
  const int ng = (mch >= 1 && mch <= N - 2) ? (mch + G - 1) / G : 0;
  for (int e = xb * 256 + threadIdx.x; e < DD; e += XB * 256) {
    float s = 0.f;
    for (int gi = 0; gi < ng; ++gi) s += dmpart[(bm * NG + gi) * DD + e];
    dm[bm * DD + e] = s;
  }
}

template <typename E, int D>
constexpr int group_of() {
  return std::is_same<E, __bf16>::value ? (D == 64 ? 4 : 2) : (D == 64 ? 2 : 1);
}

}  // namespace

size_t bwd_levels_elems(int BH, int T, int D) { return (size_t)BH * lev_off(T / C, 0, D); }

size_t bwd_dmpart_floats(int dtype, int BH, int T, int D) {
  const int N = T / C;
  const int G = dtype == 1 ? (D == 64 ? 4 : 2) : (D == 64 ? 2 : 1);
  return (size_t)BH * N * ((N + G - 1) / G) * D * D;
}

template <typename E, int D, bool FOX>
static hipError_t sweep_t(const SweepArgs &a, hipStream_t s) {
  const int BH = a.BH, T = a.T, N = T / C;
  constexpr int G = group_of<E, D>();
  E *lev = static_cast<E *>(a.levels);
  if (N > 1)
    hipLaunchKernelGGL((levels_kernel<E, D>), dim3(BH * (N - 1)), dim3(128), 0, s, a.kb, a.m, lev,
                       T, BH);
  hipLaunchKernelGGL((dq_kernel<E, D, FOX>), dim3(BH * N), dim3(256), 0, s, a.qa,
                     (const E *)a.dout, a.lse, a.dlse, a.dvec, a.lam, lev, (const E *)a.v, a.scale,
                     a.dqa, a.dlam, T, BH);
  const int NG = (N + G - 1) / G;
  hipLaunchKernelGGL((dk_kernel<E, D, G, FOX>), dim3(BH * NG), dim3(128 * G), 0, s, a.qa,
                     (const E *)a.dout, a.lse, a.dlse, a.dvec, a.lam, lev, (const E *)a.v, a.m,
                     a.scale, a.dkb, a.dv, a.dlam, a.dmpart, T, BH);
  constexpr int XB = D * D / 256;
  hipLaunchKernelGGL((dm_reduce_kernel<G>), dim3(BH * N * XB), dim3(256), 0, s, a.dmpart, a.dm, N,
                     D * D, XB);
  return hipGetLastError();
}

hipError_t launch_bwd_sweep(int dtype, int D, bool fox, const SweepArgs &a, hipStream_t s) {
  if (dtype == 1) {
    if (D == 64) return fox ? sweep_t<__bf16, 64, true>(a, s) : sweep_t<__bf16, 64, false>(a, s);
    return fox ? sweep_t<__bf16, 128, true>(a, s) : sweep_t<__bf16, 128, false>(a, s);
  }
  if (D == 64) return fox ? sweep_t<float, 64, true>(a, s) : sweep_t<float, 64, false>(a, s);
  return fox ? sweep_t<float, 128, true>(a, s) : sweep_t<float, 128, false>(a, s);
}

}  // namespace pathattn
