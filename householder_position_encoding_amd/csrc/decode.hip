// decode.hip -- PaTH decoding with in-place key refinement.
//
// PaTH discussion slides for arXiv:2505.16381v2, frame "Decoding updates
// historical keys in place" (paper Sec. 3.4, Eq. (1)): when token t arrives,
// every cached key is reflected by H_t = I - beta_t w_t w_t^T,
//
//     k_j <- k_j - beta_t w_t (w_t . k_j),    j < t,
//
// after which k_j . q_t is the path logit k_j^T H_{j+1} ... H_t q_t and the
// readout is ordinary softmax attention over the refined keys and the new key
// k_t.  Before decoding, the cache of a prompt of length L must hold every key
// aligned to the prompt end: k~_j = H_{L-1} ... H_{j+1} k_j.
//
// Prefill alignment.  Per 64-token chunk c the chunk algebra of the forward
// pass gives ->K_c (row j: H_last ... H_{j+1} k_j) and M_c = W^T U W (H_last
// ... H_first = I - M_c).  With G_c the transpose of the product of the
// transforms of all later chunks, G_{N-1} = I and G_{c-1} = G_c - M_c^T G_c,
// the aligned rows of chunk c are ->K_c G_c.  The right-to-left recurrence
// runs per (batch, head); every column of G evolves on its own, so a head's
// columns are split over several blocks.  Everything is float32.
//
// Decode step (flash-decoding with the refinement fused in): the cached keys
// 0..t-1 are split over blocks; each block reflects its keys by H_t, writes
// them back, forms the logits with q_t and keeps an online-softmax partial
// (max, sum, weighted values) in log2 units.  A combine kernel merges the
// partials with the new key k_t (whose logit has an empty path) and appends
// k_t, v_t and the gate prefix to the caches.
//
// With the forget gate the logit of (t, j) gains Lambda_t - Lambda_j with
// Lambda_t = sum_{1<=s<=t} log f_s, kept in float64 in the gate cache so that
// the running sum does not drift over long decodes (PaTH slides, frame "FoX
// adds a separate mechanism for forgetting").
#include <type_traits>

#include "path_attn_internal.h"
#include "tile_fp32.h"

namespace pathattn {

namespace {

constexpr float kLog2eD = 1.4426950408889634f;
constexpr float kLn2D = 0.69314718055994531f;

template <typename E>
__device__ __forceinline__ float to_f(E x) { return (float)x; }
template <typename E>
__device__ __forceinline__ E from_f(float x) { return (E)x; }   // RNE for bf16

// ------------------------------------------------------------ prefill: chunks

// acc(i, j) += sum_{k < K} A(i, k) B(k, j) for this wave's 32 x 32 output tile
// on the float32 matrix cores (v_mfma_f32_32x32x2f32: lane l supplies A(l%32,
// l/32) and B(l/32, l%32) per instruction), operands in LDS addressed through
// row / column strides (A(i, k) = A[i*ars + k*acs], B(k, j) = B[k*brs +
// j*bcs], already offset to the tile), so transposed operands need no copy.
// With an odd pitch (65) row and column reads are both free of bank conflicts.
template <int K>
__device__ __forceinline__ void lds_mm(f32x16 &acc, const float *A, int ars, int acs,
                                       const float *B, int brs, int bcs, int lane) {
  const int i = lane & 31, k0 = lane >> 5;
  const float *pa = A + i * ars + k0 * acs;
  const float *pb = B + k0 * brs + i * bcs;
#pragma unroll 8
  for (int k = 0; k < K; k += 2)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(pa[k * acs], pb[k * brs], acc, 0, 0, 0);
}

// One block of 256 threads per (bh, chunk): ->K_c and M_c in float32, natural
// layouts kb[bh][L][D] and m[bh][N][D][D] (M[a][b]).
// U = (I + strictLower(D W W^T))^{-1} D (blocked unit-lower inverse),
// T2 = U strictLower(W K^T), ->K = K - T2^T W, M = W^T (U W).
// Every product is a 64 x 64 (or 64 x D, D x D) block of float32
// matrix-core products on LDS operands; wave w owns the 32 x 32 tile
// (w >> 1, w & 1) of every 64 x 64 output block.
template <typename E, int D>
__global__ __launch_bounds__(256) void align_prep_kernel(
    const E *__restrict__ k, const E *__restrict__ w, const float *__restrict__ beta,
    float *__restrict__ kb, float *__restrict__ m, int L) {
  constexpr int C = kChunk, DP = D + 1, CP = C + 1, NT = 256;
  // LDS: W; N, then U, then T2 (Bs); X, then strictLower(W K^T) (Xs); U W,
  // later K (UWs)
  __shared__ float Ws[C * DP];
  __shared__ float UWs[C * DP];
  __shared__ float Bs[C * CP];
  __shared__ float Xs[C * CP];
  __shared__ float bs[C];
  __shared__ float tmp[768];
  float *Ks = UWs;
  const int N = L / C;
  const int bh = blockIdx.x / N, c = blockIdx.x % N;
  const size_t row0 = (size_t)bh * L + (size_t)c * C;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int tr = 32 * (wv >> 1), tc = 32 * (wv & 1);   // this wave's tile of a 64 x 64 block
  const E *kc = k + row0 * D;
  const E *wc = w + row0 * D;
  f32x16 acc;

  for (int idx = tid; idx < C * D; idx += NT) Ws[(idx / D) * DP + idx % D] = to_f(wc[idx]);
  if (tid < C) bs[tid] = beta[row0 + tid];
  __syncthreads();
  // N[i][j] = beta_i (w_i . w_j) for j < i (into Bs)
  zero16(acc);
  lds_mm<D>(acc, Ws + tr * DP, DP, 1, Ws + tc * DP, 1, DP, lane);
  tile_each(tid, [&](int i, int j, int r) { Bs[i * CP + j] = j < i ? acc[r] * bs[i] : 0.f; });
  __syncthreads();
  // X = (I + N)^{-1}: blocked unit-lower inverse (16 x 16 diagonal blocks by
  // substitution, the off-diagonal blocks level by level with the whole block)
  unit_lower_inverse(Bs, Xs, tmp, tid);
  __syncthreads();
  // U = X D (unit diagonal of X times beta), zero above the diagonal (into Bs)
  for (int idx = tid; idx < C * C; idx += NT) {
    const int i = idx / C, j = idx % C;
    Bs[i * CP + j] = j < i ? Xs[i * CP + j] * bs[j] : (j == i ? bs[i] : 0.f);
  }
  __syncthreads();
  // UW = U W (64 x D)
#pragma unroll
  for (int h = 0; h < D / 64; ++h) {
    zero16(acc);
    lds_mm<C>(acc, Bs + tr * CP, CP, 1, Ws + 64 * h + tc, DP, 1, lane);
    tile_each(tid, [&](int i, int j, int r) { UWs[i * DP + 64 * h + j] = acc[r]; });
  }
  __syncthreads();
  // M[a][b] = sum_s W[s][a] UW[s][b]
  float *m_c = m + ((size_t)bh * N + c) * D * D;
#pragma unroll
  for (int ha = 0; ha < D / 64; ++ha)
#pragma unroll
    for (int hb = 0; hb < D / 64; ++hb) {
      zero16(acc);
      lds_mm<C>(acc, Ws + 64 * ha + tr, 1, DP, UWs + 64 * hb + tc, DP, 1, lane);
      tile_each(tid, [&](int a, int b, int r) {
        m_c[(size_t)(64 * ha + a) * D + 64 * hb + b] = acc[r];
      });
    }
  __syncthreads();   // U W is no longer read: its buffer takes K
  for (int idx = tid; idx < C * D; idx += NT) Ks[(idx / D) * DP + idx % D] = to_f(kc[idx]);
  __syncthreads();
  // SK[t][j] = w_t . k_j for t > j, else 0 (into Xs)
  zero16(acc);
  lds_mm<D>(acc, Ws + tr * DP, DP, 1, Ks + tc * DP, 1, DP, lane);
  tile_each(tid, [&](int t, int j, int r) { Xs[t * CP + j] = t > j ? acc[r] : 0.f; });
  __syncthreads();
  // T2 = U SK (both triangular, dense product), written over U once every
  // wave has read it
  zero16(acc);
  lds_mm<C>(acc, Bs + tr * CP, CP, 1, Xs + tc, CP, 1, lane);
  __syncthreads();
  tile_each(tid, [&](int sr, int j, int r) { Bs[sr * CP + j] = acc[r]; });
  __syncthreads();
  // ->K[j][col] = K[j][col] - sum_s T2[s][j] W[s][col]  (T2[s][j] = 0 for s <= j)
  float *kb_c = kb + row0 * D;
#pragma unroll
  for (int h = 0; h < D / 64; ++h) {
    zero16(acc);
    lds_mm<C>(acc, Bs + tr, 1, CP, Ws + 64 * h + tc, DP, 1, lane);
    tile_each(tid, [&](int j, int col, int r) {
      kb_c[(size_t)j * D + 64 * h + col] = Ks[j * DP + 64 * h + col] - acc[r];
    });
  }
}

// ------------------------------------------------------------ prefill: scan

// acc(i, j) += sum_{k < K} A(i, k) B(k, j) for this wave's 16 x 16 output
// tile on the float32 matrix cores (v_mfma_f32_16x16x4f32: lane l supplies
// A(l%16, l/16) and B(l/16, l%16) per instruction; result lane l register r
// holds row 4 (l/16) + r, column l%16), operands in LDS through strides as
// for lds_mm.
template <int K>
__device__ __forceinline__ void lds_mm16(f32x4 &acc, const float *A, int ars, int acs,
                                         const float *B, int brs, int bcs, int lane) {
  const int i = lane & 15, k0 = lane >> 4;
  const float *pa = A + i * ars + k0 * acs;
  const float *pb = B + k0 * brs + i * bcs;
#pragma unroll 8
  for (int k = 0; k < K; k += 4)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k * acs], pb[k * brs], acc, 0, 0, 0);
}

// One block of 8 waves per (bh, slice of 16 columns of G).  Chunk by chunk
// from the last: ->K_c and M_c are staged in LDS (loaded into registers one
// chunk ahead); the aligned rows ->K_c G_c of this column slice (64 x 16:
// four 16 x 16 tiles) are written and G <- G - M_c^T G (D x 16: D/16 tiles)
// is formed, one 16 x 16 tile per wave at a time, on the float32 matrix
// cores.  G's slice lives in LDS.  The chain of dependent chunk steps is what
// bounds the kernel, so the tiles are small: each step costs a wave at most
// two D-deep chains of 16 x 16 x 4 products.
template <typename KC, int D>
__global__ __launch_bounds__(512) void align_scan_kernel(
    const float *__restrict__ kb, const float *__restrict__ m, KC *__restrict__ kcache,
    int L, int T_cap, int BH) {
  constexpr int C = kChunk, NT = 512, NW = 8, DP = D + 1, SW = 16, SP = SW + 1;
  constexpr int NSL = D / SW;                                   // column slices per head
  constexpr int NK4 = C * D / 4 / NT, NM4 = D * D / 4 / NT;    // float4 loads per thread
  constexpr int NRT = C / 16, NGT = D / 16, NTILE = NRT + NGT;  // row tiles, G tiles
  constexpr int TPW = (NTILE + NW - 1) / NW;                    // tiles per wave
  static_assert(C * D % (4 * NT) == 0 && D * D % (4 * NT) == 0, "loads split evenly");
  __shared__ float Ks[C * DP];
  __shared__ float Ms[D * DP];
  __shared__ float Gs[D * SP];
  const int N = L / C;
  // Blocks are dealt to the 8 XCDs round robin: block 8 (NSL g + sl) + r is
  // slice sl of head 8 g + r, so every slice of a head runs on one XCD and
  // the head's ->K and M are fetched into that XCD's L2 once.
  const int grp8 = blockIdx.x / (8 * NSL), rem = blockIdx.x % (8 * NSL);
  const int sl = rem / 8, bh = 8 * grp8 + rem % 8;
  if (bh >= BH) return;   // the last group of eight heads may be partial
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, q4 = lane >> 4, cl = lane & 15;

  f32x4 kreg[NK4], mreg[NM4];
  auto fetch = [&](int c) {       // chunk c's ->K and M into registers
    const f32x4 *kb_c = reinterpret_cast<const f32x4 *>(kb + ((size_t)bh * L + (size_t)c * C) * D);
    const f32x4 *m_c = reinterpret_cast<const f32x4 *>(m + ((size_t)bh * N + c) * D * D);
#pragma unroll
    for (int i = 0; i < NK4; ++i) kreg[i] = kb_c[tid + NT * i];
#pragma unroll
    for (int i = 0; i < NM4; ++i) mreg[i] = m_c[tid + NT * i];
  };
  auto park = [&]() {             // registers into LDS (padded rows)
#pragma unroll
    for (int i = 0; i < NK4; ++i) {
      const int idx = 4 * (tid + NT * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) Ks[((idx + e) / D) * DP + (idx + e) % D] = kreg[i][e];
    }
#pragma unroll
    for (int i = 0; i < NM4; ++i) {
      const int idx = 4 * (tid + NT * i);
#pragma unroll
      for (int e = 0; e < 4; ++e) Ms[((idx + e) / D) * DP + (idx + e) % D] = mreg[i][e];
    }
  };

  for (int idx = tid; idx < D * SW; idx += NT) {
    const int a = idx / SW, b = idx % SW;
    Gs[a * SP + b] = a == SW * sl + b ? 1.f : 0.f;
  }
  if (N > 0) fetch(N - 1);
  for (int c = N - 1; c >= 0; --c) {
    __syncthreads();   // previous chunk's reads of Ks/Ms/Gs are done
    park();
    __syncthreads();
    if (c > 0) fetch(c - 1);   // in flight while chunk c is computed
    f32x4 gn[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = wv + NW * u;
      if (t < NGT) {
        // G <- G - M_c^T G, rows 16 t.. of the slice: (M^T G)[a][b] = sum_r M[r][a] G[r][b]
        f32x4 prod = {0.f, 0.f, 0.f, 0.f};
        lds_mm16<D>(prod, Ms + 16 * t, 1, DP, Gs, SP, 1, lane);
#pragma unroll
        for (int r = 0; r < 4; ++r) gn[u][r] = Gs[(16 * t + 4 * q4 + r) * SP + cl] - prod[r];
      } else if (t < NTILE) {
        // aligned rows 16 (t - NGT).. of chunk c: (->K_c G_c)[j][col]
        const int rt = t - NGT;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        lds_mm16<D>(acc, Ks + 16 * rt * DP, DP, 1, Gs, SP, 1, lane);
        KC *dst = kcache + ((size_t)bh * T_cap + (size_t)c * C + 16 * rt + 4 * q4) * D + SW * sl + cl;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(size_t)r * D] = from_f<KC>(acc[r]);
      }
    }
    __syncthreads();   // all reads of the old G are done
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int t = wv + NW * u;
      if (t < NGT)
#pragma unroll
        for (int r = 0; r < 4; ++r) Gs[(16 * t + 4 * q4 + r) * SP + cl] = gn[u][r];
    }
  }
}

// Values of the prompt into the value cache: vcache[bh][j] = v[bh][j], j < L.
template <typename E>
__global__ __launch_bounds__(256) void copy_rows_kernel(const E *__restrict__ v, E *__restrict__ vcache,
                                                        int L, int T_cap, int D) {
  const size_t per_head = (size_t)L * D;
  const size_t bh = blockIdx.y;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < per_head; i += (size_t)gridDim.x * 256)
    vcache[bh * (size_t)T_cap * D + i] = v[bh * per_head + i];
}

// Gate cache of the prompt: Lambda_j = sum_{1<=s<=j} log f_s in float64 (f_0
// never enters a logit), one block of 256 threads per (b, h): each thread sums
// its segment, the segment sums are prefixed, and each thread writes its
// segment's running sums.
__global__ __launch_bounds__(256) void gate_cache_kernel(const float *__restrict__ logf,
                                                         double *__restrict__ gcache, int L,
                                                         int T_cap) {
  __shared__ double part[256];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const float *f = logf + (size_t)bh * L;
  const int per = (L + 255) / 256;
  const int t0 = min(L, tid * per), t1 = min(L, t0 + per);
  double s = 0.0;
  for (int t = t0 < 1 ? 1 : t0; t < t1; ++t) s += (double)f[t];
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
    if (t >= 1) run += (double)f[t];
    gcache[(size_t)bh * T_cap + t] = run;
  }
}

// ------------------------------------------------------------ decode step

template <typename T>
struct Vec16;   // 16 bytes of T
template <>
struct Vec16<float> {
  static constexpr int n = 4;
  typedef float type __attribute__((ext_vector_type(4)));
};
template <>
struct Vec16<__bf16> {
  static constexpr int n = 8;
  typedef __bf16 type __attribute__((ext_vector_type(8)));
};

// Load / store n consecutive elements as floats.
template <typename T, int n>
__device__ __forceinline__ void load_f(const T *p, float (&x)[n]) {
  if constexpr (std::is_same<T, float>::value && n == 4) {
    const f32x4 v = *reinterpret_cast<const f32x4 *>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = v[e];
  } else if constexpr (std::is_same<T, __bf16>::value && n == 8) {
    const bf16x8 v = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
  } else if constexpr (std::is_same<T, __bf16>::value && n == 4) {
    const bf16x4 v = *reinterpret_cast<const bf16x4 *>(p);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (float)v[e];
  } else {
    static_assert(std::is_same<T, float>::value && n == 8, "unsupported vector");
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = a[e];
      x[4 + e] = b[e];
    }
  }
}
template <typename T, int n>
__device__ __forceinline__ void store_f(T *p, const float (&x)[n]) {
  if constexpr (std::is_same<T, float>::value && n == 4) {
    *reinterpret_cast<f32x4 *>(p) = f32x4{x[0], x[1], x[2], x[3]};
  } else {
    static_assert(std::is_same<T, __bf16>::value && n == 8, "unsupported vector");
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)x[e];
    *reinterpret_cast<bf16x8 *>(p) = v;
  }
}

// Sum over the LPK lanes of a key group (aligned groups of LPK lanes).
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int off = LPK / 2; off >= 1; off /= 2) x += __shfl_xor(x, off);
  return x;
}

constexpr int kKeysPerSplit = 512;
constexpr int kUnroll = 4;

// Partials per (bh, split): m, l (log2 units, max and sum), then o[D].
template <int D>
__host__ __device__ constexpr int partial_floats() { return D + 2; }

// Decode workspace: the partials of up to ceil(T_cap / 512) splits per head.
inline size_t decode_partials_size(int BH, int T_cap, int D) {
  const size_t nsplit = ((size_t)T_cap + kKeysPerSplit - 1) / kKeysPerSplit;
  return (size_t)BH * (nsplit > 0 ? nsplit : 1) * (D + 2) * sizeof(float);
}

// The merge, one block of 256 threads per head in a kernel of its own after
// the split kernel (the kernel boundary orders the partials' stores before
// the merge's loads):
// the split partials and the new key k_t (logit scale * q_t . k_t, no gate
// term) give o_t and lse_t; k_t, v_t and Lambda_t are appended to the caches.  The merge is an online softmax over
// batches of up to 64 splits: each batch's partials are copied into LDS in
// one coalesced pass, its max and weights come from one wave's shuffles, and
// the running (M, l, o) is rescaled once per batch.  It starts from the new
// key itself: M = x_new, l = 1, o = v_t.
constexpr int kMergeBatch = 64;   // splits per merge batch

template <int D>
struct MergeLds {
  float sp[kMergeBatch * partial_floats<D>()];   // partials of the batch
  float wsp[kMergeBatch];                        // weight of each split of the batch
  float bc[4];                                   // broadcast: x_new, batch max, batch l
};

template <typename E, typename KC, int D, bool FOX>
__device__ __forceinline__ void merge_head(
    MergeLds<D> &sm, int bh, const E *__restrict__ q, const E *__restrict__ k,
    const E *__restrict__ v, const float *__restrict__ logf, KC *__restrict__ kcache,
    E *__restrict__ vcache, double *__restrict__ gcache, const float *part, E *__restrict__ out,
    float *__restrict__ lse, int t, int T_cap, int nsplit, float sl2) {
  constexpr int PF = partial_floats<D>();
  constexpr int NT = 256, SB = kMergeBatch;
  float *sp = sm.sp, *wsp = sm.wsp, *bc = sm.bc;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float *ph = part + (size_t)bh * nsplit * PF;
  // every global read the merge needs is issued up front (first batch of
  // partials into registers, q, k, v), so the kernel waits on memory once
  constexpr int PER = (SB * PF + NT - 1) / NT;
  float pre[PER];
  const int ns0 = min(SB, nsplit);
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int i = tid + r * NT;
    pre[r] = i < ns0 * PF ? ph[i] : 0.f;
  }
  const float vt = tid < D ? to_f(v[(size_t)bh * D + tid]) : 0.f;
  const float kt = tid < D ? to_f(k[(size_t)bh * D + tid]) : 0.f;
  float qk = 0.f;
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < D / 64; ++i)
      qk = __builtin_fmaf(to_f(q[(size_t)bh * D + lane + 64 * i]),
                          to_f(k[(size_t)bh * D + lane + 64 * i]), qk);
  }
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int i = tid + r * NT;
    if (i < ns0 * PF) sp[i] = pre[r];
  }
  // logit of the new key: wave 0, D / 64 elements per lane
  if (wave == 0) {
#pragma unroll
    for (int off = 32; off >= 1; off /= 2) qk += __shfl_xor(qk, off);
    if (lane == 0) bc[0] = qk * sl2;
  }
  __syncthreads();
  float M = bc[0], l = 1.f;
  float o = vt;
  for (int s0 = 0; s0 < nsplit; s0 += SB) {
    const int ns = min(SB, nsplit - s0);
    if (s0 > 0) {
      __syncthreads();   // the previous batch is consumed
      for (int i = tid; i < ns * PF; i += NT) sp[i] = ph[(size_t)s0 * PF + i];
      __syncthreads();
    }
    if (wave == 0) {
      const float ms = lane < ns ? sp[lane * PF] : -INFINITY;
      float mc = ms;
#pragma unroll
      for (int off = 32; off >= 1; off /= 2) mc = fmaxf(mc, __shfl_xor(mc, off));
      const float Mn = fmaxf(M, mc);
      const float f = ms > -INFINITY ? __builtin_amdgcn_exp2f(ms - Mn) : 0.f;
      wsp[lane] = f;
      float lb = lane < ns ? f * sp[lane * PF + 1] : 0.f;
#pragma unroll
      for (int off = 32; off >= 1; off /= 2) lb += __shfl_xor(lb, off);
      if (lane == 0) {
        bc[1] = Mn;
        bc[2] = lb;
      }
    }
    __syncthreads();
    const float Mn = bc[1];
    const float alpha = __builtin_amdgcn_exp2f(M - Mn);   // M finite: it includes x_new
    l = __builtin_fmaf(l, alpha, bc[2]);
    if (tid < D) {
      float acc = o * alpha;
      for (int sidx = 0; sidx < ns; ++sidx) {
        const float f = wsp[sidx];
        if (f != 0.f) acc = __builtin_fmaf(f, sp[sidx * PF + 2 + tid], acc);
      }
      o = acc;
    }
    M = Mn;
  }
  if (tid < D) {
    out[(size_t)bh * D + tid] = from_f<E>(o / l);
    kcache[((size_t)bh * T_cap + t) * D + tid] = from_f<KC>(kt);
    vcache[((size_t)bh * T_cap + t) * D + tid] = from_f<E>(vt);
  }
  if (tid == 0) {
    lse[bh] = kLn2D * (M + __builtin_amdgcn_logf(l));
    if (FOX)
      gcache[(size_t)bh * T_cap + t] =
          t >= 1 ? gcache[(size_t)bh * T_cap + t - 1] + (double)logf[bh] : 0.0;
  }
}

// One block of 256 threads per (split, bh): keys [split*KPS, min(t, +KPS))
// (an empty range when t == 0: the step then has one block with no keys).
// A key row is spread over LPK lanes with EPL consecutive elements each
// (16-byte loads of the key cache); a wave covers KPW = 64 / LPK keys at once.
template <typename E, typename KC, int D, bool FOX>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const E *__restrict__ w, const float *__restrict__ beta, const float *__restrict__ logf,
    KC *__restrict__ kcache, E *__restrict__ vcache, double *__restrict__ gcache,
    float *__restrict__ part, int t, int T_cap, int nsplit, float sl2) {
  constexpr int EPL = Vec16<KC>::n;
  constexpr int LPK = D / EPL;
  constexpr int KPW = 64 / LPK;
  constexpr int NW = 4;
  constexpr int STRIDE = NW * KPW;          // keys per block iteration
  constexpr int PF = partial_floats<D>();
  __shared__ float red_m[NW * KPW], red_l[NW * KPW];
  __shared__ float red_o[NW * KPW][D];

  const int split = blockIdx.x, bh = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane / LPK, e0 = (lane % LPK) * EPL;
  const int j_begin = split * kKeysPerSplit;
  const int j_end = min(t, j_begin + kKeysPerSplit);

  float qv[EPL], wv[EPL];
  load_f<E, EPL>(q + (size_t)bh * D + e0, qv);
  load_f<E, EPL>(w + (size_t)bh * D + e0, wv);
  const float bt = beta[bh];
  double lam_t = 0.0;
  if (FOX) lam_t = (t >= 1 ? gcache[(size_t)bh * T_cap + t - 1] : 0.0) + (t >= 1 ? (double)logf[bh] : 0.0);
  KC *kc_h = kcache + (size_t)bh * T_cap * D;
  const E *vc_h = vcache + (size_t)bh * T_cap * D;
  const double *gc_h = FOX ? gcache + (size_t)bh * T_cap : nullptr;

  float m_run = -INFINITY, l_run = 0.f, o_run[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o_run[e] = 0.f;

  for (int base = j_begin + wave * KPW + grp; base < j_end; base += kUnroll * STRIDE) {
    float kk[kUnroll][EPL], vv[kUnroll][EPL], x[kUnroll];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = base + u * STRIDE;
      ok[u] = j < j_end;
      if (ok[u]) {
        load_f<KC, EPL>(kc_h + (size_t)j * D + e0, kk[u]);
        load_f<E, EPL>(vc_h + (size_t)j * D + e0, vv[u]);
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) kk[u][e] = vv[u][e] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      // k_j <- k_j - beta_t w_t (w_t . k_j), written back in place
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) a = __builtin_fmaf(wv[e], kk[u][e], a);
      a = group_sum<LPK>(a) * bt;
#pragma unroll
      for (int e = 0; e < EPL; ++e) kk[u][e] = __builtin_fmaf(-a, wv[e], kk[u][e]);
      const int j = base + u * STRIDE;
      if (ok[u]) store_f<KC, EPL>(kc_h + (size_t)j * D + e0, kk[u]);
      // the logit uses the key as stored (rounded to the cache type)
      float kr[EPL];
      if constexpr (std::is_same<KC, float>::value) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) kr[e] = kk[u][e];
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) kr[e] = (float)(__bf16)kk[u][e];
      }
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) s = __builtin_fmaf(qv[e], kr[e], s);
      s = group_sum<LPK>(s);
      float xv = s * sl2;
      if (FOX && ok[u]) xv += (float)((lam_t - gc_h[j]) * (double)kLog2eD);
      x[u] = ok[u] ? xv : -INFINITY;
    }
    float mx = m_run;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) mx = fmaxf(mx, x[u]);
    if (mx > -INFINITY) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - mx);
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o_run[e] *= alpha;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const float p = __builtin_amdgcn_exp2f(x[u] - mx);
        l_run += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o_run[e] = __builtin_fmaf(p, vv[u][e], o_run[e]);
      }
      m_run = mx;
    }
  }

  // combine the KPW key groups of every wave and the NW waves: slot
  // (wave, grp) in LDS, then the first KPW*NW... reduced by wave 0
  const int slot = wave * KPW + grp;
  if (lane % LPK == 0) {
    red_m[slot] = m_run;
    red_l[slot] = l_run;
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) red_o[slot][e0 + e] = o_run[e];
  __syncthreads();
  float *dst = part + ((size_t)bh * nsplit + split) * PF;
  if (threadIdx.x < D) {
    float M = -INFINITY;
    for (int s = 0; s < NW * KPW; ++s) M = fmaxf(M, red_m[s]);
    float l = 0.f, o = 0.f;
    if (M > -INFINITY) {
      for (int s = 0; s < NW * KPW; ++s) {
        const float f = __builtin_amdgcn_exp2f(red_m[s] - M);
        l = __builtin_fmaf(f, red_l[s], l);
        o = __builtin_fmaf(f, red_o[s][threadIdx.x], o);
      }
    }
    dst[2 + threadIdx.x] = o;
    if (threadIdx.x == 0) {
      dst[0] = M;
      dst[1] = l;
    }
  }
}

// The merge of one head's split partials (see merge_head).
template <typename E, typename KC, int D, bool FOX>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const E *__restrict__ q, const E *__restrict__ k, const E *__restrict__ v,
    const float *__restrict__ logf, KC *__restrict__ kcache, E *__restrict__ vcache,
    double *__restrict__ gcache, const float *__restrict__ part, E *__restrict__ out,
    float *__restrict__ lse, int t, int T_cap, int nsplit, float sl2) {
  __shared__ MergeLds<D> msm;
  merge_head<E, KC, D, FOX>(msm, (int)blockIdx.x, q, k, v, logf, kcache, vcache, gcache, part,
                            out, lse, t, T_cap, nsplit, sl2);
}

template <typename E, typename KC, int D>
hipError_t prefill_t(const void *k, const void *v, const void *w, const float *beta,
                     const float *logf, void *kcache, void *vcache, double *gcache, float *ws_kb,
                     float *ws_m, int BH, int L, int T_cap, hipStream_t stream) {
  const int N = L / kChunk;
  if (N > 0) {
    hipLaunchKernelGGL((align_prep_kernel<E, D>), dim3(BH * N), dim3(256), 0, stream,
                       (const E *)k, (const E *)w, beta, ws_kb, ws_m, L);
    hipLaunchKernelGGL((align_scan_kernel<KC, D>), dim3((BH + 7) / 8 * 8 * (D / 16)), dim3(512), 0, stream,
                       ws_kb, ws_m, (KC *)kcache, L, T_cap, BH);
    const int gx = min(1024, (int)(((size_t)L * D + 255) / 256));
    hipLaunchKernelGGL((copy_rows_kernel<E>), dim3(gx, BH), dim3(256), 0, stream, (const E *)v,
                       (E *)vcache, L, T_cap, D);
    if (logf)
      hipLaunchKernelGGL(gate_cache_kernel, dim3(BH), dim3(256), 0, stream, logf, gcache, L, T_cap);
  }
  return hipGetLastError();
}

template <typename E, typename KC, int D, bool FOX>
hipError_t decode_t(const void *q, const void *k, const void *v, const void *w,
                    const float *beta, const float *logf, void *kcache, void *vcache,
                    double *gcache, void *out, float *lse, float *part, int BH, int t,
                    int T_cap, float sl2, hipStream_t stream) {
  const int nsplit = t > 0 ? (t + kKeysPerSplit - 1) / kKeysPerSplit : 1;
  hipLaunchKernelGGL((decode_split_kernel<E, KC, D, FOX>), dim3(nsplit, BH), dim3(256), 0, stream,
                     (const E *)q, (const E *)k, (const E *)v, (const E *)w, beta, logf,
                     (KC *)kcache, (E *)vcache, gcache, part, t, T_cap, nsplit, sl2);
  hipLaunchKernelGGL((decode_merge_kernel<E, KC, D, FOX>), dim3(BH), dim3(256), 0, stream,
                     (const E *)q, (const E *)k, (const E *)v, logf, (KC *)kcache, (E *)vcache,
                     gcache, (const float *)part, (E *)out, lse, t, T_cap, nsplit, sl2);
  return hipGetLastError();
}

template <typename E, typename KC>
hipError_t prefill_d(int D, const void *k, const void *v, const void *w, const float *beta,
                     const float *logf, void *kcache, void *vcache, double *gcache,
                     float *ws_kb, float *ws_m, int BH, int L, int T_cap, hipStream_t s) {
  if (D == 64)
    return prefill_t<E, KC, 64>(k, v, w, beta, logf, kcache, vcache, gcache, ws_kb, ws_m, BH, L,
                                T_cap, s);
  return prefill_t<E, KC, 128>(k, v, w, beta, logf, kcache, vcache, gcache, ws_kb, ws_m, BH, L,
                               T_cap, s);
}

template <typename E, typename KC>
hipError_t decode_d(int D, const void *q, const void *k, const void *v, const void *w,
                    const float *beta, const float *logf, void *kcache, void *vcache,
                    double *gcache, void *out, float *lse, float *part, int BH, int t,
                    int T_cap, float sl2, hipStream_t s) {
  if (D == 64) {
    if (logf)
      return decode_t<E, KC, 64, true>(q, k, v, w, beta, logf, kcache, vcache, gcache, out, lse,
                                       part, BH, t, T_cap, sl2, s);
    return decode_t<E, KC, 64, false>(q, k, v, w, beta, logf, kcache, vcache, gcache, out, lse,
                                      part, BH, t, T_cap, sl2, s);
  }
  if (logf)
    return decode_t<E, KC, 128, true>(q, k, v, w, beta, logf, kcache, vcache, gcache, out, lse,
                                      part, BH, t, T_cap, sl2, s);
  return decode_t<E, KC, 128, false>(q, k, v, w, beta, logf, kcache, vcache, gcache, out, lse,
                                     part, BH, t, T_cap, sl2, s);
}

}  // namespace

size_t decode_partial_bytes(int BH, int T_cap, int D) {
  return decode_partials_size(BH, T_cap, D);
}

hipError_t launch_prefill_cache(int dtype, int kc_dtype, int D, const void *k, const void *v,
                                const void *w, const float *beta, const float *logf,
                                void *kcache, void *vcache, double *gcache, float *ws_kb,
                                float *ws_m, int BH, int L, int T_cap, hipStream_t s) {
  if (dtype == 1) {
    if (kc_dtype == 1)
      return prefill_d<__bf16, __bf16>(D, k, v, w, beta, logf, kcache, vcache, gcache, ws_kb,
                                       ws_m, BH, L, T_cap, s);
    return prefill_d<__bf16, float>(D, k, v, w, beta, logf, kcache, vcache, gcache, ws_kb, ws_m,
                                     BH, L, T_cap, s);
  }
  if (kc_dtype == 1)
    return prefill_d<float, __bf16>(D, k, v, w, beta, logf, kcache, vcache, gcache, ws_kb, ws_m,
                                    BH, L, T_cap, s);
  return prefill_d<float, float>(D, k, v, w, beta, logf, kcache, vcache, gcache, ws_kb, ws_m, BH,
                                 L, T_cap, s);
}

hipError_t launch_decode_step(int dtype, int kc_dtype, int D, const void *q, const void *k,
                              const void *v, const void *w, const float *beta,
                              const float *logf, void *kcache, void *vcache, double *gcache,
                              void *out, float *lse, float *part, int BH, int t, int T_cap,
                              float sl2, hipStream_t s) {
  if (dtype == 1) {
    if (kc_dtype == 1)
      return decode_d<__bf16, __bf16>(D, q, k, v, w, beta, logf, kcache, vcache, gcache, out,
                                      lse, part, BH, t, T_cap, sl2, s);
    return decode_d<__bf16, float>(D, q, k, v, w, beta, logf, kcache, vcache, gcache, out, lse,
                                   part, BH, t, T_cap, sl2, s);
  }
  if (kc_dtype == 1)
    return decode_d<float, __bf16>(D, q, k, v, w, beta, logf, kcache, vcache, gcache, out, lse,
                                   part, BH, t, T_cap, sl2, s);
  return decode_d<float, float>(D, q, k, v, w, beta, logf, kcache, vcache, gcache, out, lse,
                                part, BH, t, T_cap, sl2, s);
}

}  // namespace pathattn
