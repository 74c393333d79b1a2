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
//     The triangular inverse is blocked (16 x 16): diagonal blocks by
//     substitution on the vector units, off-diagonal blocks on float32 matrix
//     cores.  Transposed copies (W^T, V^T in fragment order) are exact
//     identity products on the matrix cores.
//   * prep_f32_kernel (float32 inputs): plain float32 arithmetic on the vector
//     units.
// Only the operands handed to the streaming kernel's matrix cores (->K, V,
// -M^T) are rounded to the storage type, once, at the end.
#include "path_attn_internal.h"
#include <algorithm>
#include <atomic>

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
    const float *__restrict__ logf, float *__restrict__ gate, int T, int H, TokStrides sf) {
  __shared__ double part[256];
  const int bh = blockIdx.x, tid = threadIdx.x;
  // log f_t of head (b, h) at f[t * sf.t]
  const float *f0 = logf + (long long)(bh / H) * sf.b + (long long)(bh % H) * sf.h;
  auto f = [&](int t) { return f0[(long long)t * sf.t]; };
  float *a = gate + (size_t)bh * T;
  const int per = (T + 255) / 256;
  const int t0 = min(T, tid * per), t1 = min(T, t0 + per);
  double s = 0.0;
  for (int t = max(t0, 1); t < t1; ++t) s += (double)f(t);
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
    if (t > 0) run += (double)f(t);
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

__device__ __forceinline__ f32x16 mma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// One 32x32x(16*KS) product on a wave from bf16 rows with the contraction
// index contiguous: lane l supplies row l%32, elements 8*(l/32) + 16*ks ...
template <int KS>
__device__ __forceinline__ void load_rows(bf16x8 (&f)[KS], const __bf16 *rows, int pitch, int lane) {
  const __bf16 *p = rows + (lane & 31) * pitch + 8 * (lane >> 5);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) f[ks] = *reinterpret_cast<const bf16x8 *>(p + 16 * ks);
}
// Inputs of one chunk staged in LDS at d = 64: a 64 x 64 bf16 tile, rows of
// 128 bytes, the 16-byte column cc of row r stored at slot cc ^ (r & 7), so
// eight consecutive rows of one column fall in eight different slots (the
// fragment reads below are free of bank conflicts).
__device__ __forceinline__ int sw_off(int r, int cc) { return r * 128 + ((cc ^ (r & 7)) << 4); }
// load_rows from a staged tile: rows row0 + l%32, columns 8*(l/32) + 16*ks.
template <int KS>
__device__ __forceinline__ void load_rows_sw(bf16x8 (&f)[KS], const unsigned char *tile, int row0,
                                             int lane) {
  const int r = row0 + (lane & 31);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    f[ks] = *reinterpret_cast<const bf16x8 *>(tile + sw_off(r, (lane >> 5) + 2 * ks));
}

template <int KS>
__device__ __forceinline__ void mma_rows(f32x16 &acc, const bf16x8 (&a)[KS], const bf16x8 (&b)[KS]) {
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) acc = mma32(a[ks], b[ks], acc);
}

// acc += A[0..32)[0..K) * Bt[0..32)[0..K)^T with both operands in LDS.
template <int K>
__device__ __forceinline__ void tile_mma(f32x16 &acc, const __bf16 *A, int PA,
                                         const __bf16 *Bt, int PB, int lane) {
  bf16x8 a[K / 16], b[K / 16];
  load_rows<K / 16>(a, A, PA, lane);
  load_rows<K / 16>(b, Bt, PB, lane);
  mma_rows<K / 16>(acc, a, b);
}

// Identity B operand for the exact MFMA transpose of a 32-column block:
// k-step h of the block holds 1 where contraction index 16h + 8g + t equals
// the lane's column l%32.
__device__ __forceinline__ bf16x8 eye_frag(int h, int lane) {
  bf16x8 f;
  const int t0 = (lane & 31) - 16 * h - 8 * (lane >> 5);
#pragma unroll
  for (int t = 0; t < 8; ++t) f[t] = (__bf16)(t == t0 ? 1.f : 0.f);
  return f;
}

// Store 4 accumulator values (rows acc_row(4*r4 + 0..3, g), consecutive) as
// hi/lo bf16 pairs at dst_hi/dst_lo + offset (4 contiguous elements).
__device__ __forceinline__ void store4_split(__bf16 *hi, __bf16 *lo, int off, f32x4 x) {
  bf16x4 h, l;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    h[e] = (__bf16)x[e];
    l[e] = (__bf16)(x[e] - (float)h[e]);
  }
  *reinterpret_cast<bf16x4 *>(hi + off) = h;
  *reinterpret_cast<bf16x4 *>(lo + off) = l;
}

// f[idx] for a wave-uniform runtime idx without dynamic register indexing.
template <int KS>
__device__ __forceinline__ bf16x8 pick(const bf16x8 (&f)[KS], int idx) {
  bf16x8 r = f[0];
#pragma unroll
  for (int i = 1; i < KS; ++i)
    if (i == idx) r = f[i];
  return r;
}

__device__ __forceinline__ f32x4 quad(const f32x16 &a, int r4) {
  return f32x4{a[4 * r4], a[4 * r4 + 1], a[4 * r4 + 2], a[4 * r4 + 3]};
}

__device__ __forceinline__ f32x4 mma16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Off-diagonal block (p, q) of X = (I + N)^{-1}, 16 x 16 blocks, one wave, on
// fp32 matrix cores:  X_pq = -X_pp * sum_{r=q}^{p-1} N_pr X_rq.
// Xs holds N (strictly lower blocks), X_pp over the diagonal blocks and X_pq
// (p > q) transposed in the upper block (q, p), which N leaves unused.
// MFMA 16x16x4 layouts: A lane l -> A[l%16][k = l/16], B lane l ->
// B[k = l/16][l%16], D lane l register r -> D[4*(l/16) + r][l%16].
template <int PX>
__device__ __forceinline__ void solve_block(float *Xs, int p, int q, int lane) {
  const int m = lane & 15, g16 = lane >> 4;
  f32x4 y = {0.f, 0.f, 0.f, 0.f};
  for (int r = q; r < p; ++r) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int k = 4 * s + g16;
      const float a = Xs[(16 * p + m) * PX + 16 * r + k];                      // N[16p+m][16r+k]
      const float b = r == q ? Xs[(16 * q + k) * PX + 16 * q + m]               // X_qq[k][m]
                             : Xs[(16 * q + m) * PX + 16 * r + k];              // X_rq[k][m], transposed
      y = mma16(a, b, y);
    }
  }
  // X_pq = X_pp * (-Y): lane holds Y rows 4*g16 + s; contraction slot
  // 4*s + g16 of the MFMA maps to physical row 4*g16 + s.
  f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s)
    x = mma16(Xs[(16 * p + m) * PX + 16 * p + 4 * g16 + s], -y[s], x);
  // D rows i = 4*g16 + e, column j = m: stored transposed at (16q + j, 16p + i).
  *reinterpret_cast<f32x4 *>(Xs + (16 * q + m) * PX + 16 * p + 4 * g16) = x;
}

// One block of 4 waves per (bh, chunk).  Every 64x64 product is split in four
// 32x32 output tiles, one per wave, tile (mt, nt) = (w>>1, w&1); products with
// a d-sized dimension give each wave D/64 tiles.  Products whose result goes
// to LDS are computed in the orientation where a lane's fixed column is the
// destination row, so each lane stores 4 contiguous elements at a time.
// DP: the leading coordinates the factors act on (D; or D / 2 for partial
// PaTH, where w is not read beyond them: every product with W contracts over
// DP coordinates only, U W and M vanish outside them, and <-Q, ->K equal Q, K
// there).
template <int D, int DP>
__global__ __launch_bounds__(256, 2) void prep_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k,
    const __bf16 *__restrict__ v, const __bf16 *__restrict__ w,
    const float *__restrict__ beta, float *__restrict__ qa,
    __bf16 *__restrict__ kvm, float *__restrict__ al, int T, int total, FwdIo io,
    __bf16 *__restrict__ klo) {
  constexpr int C = kChunk, P = 72, PX = 72;
  constexpr int NDB = D / 32, NSD = D / 16, NSK = C / 16, KSD = D / 16, KSC = C / 16;
  constexpr int TPW = D / 64;                       // d x 64 tiles per wave
  constexpr int KSDP = DP / 16, NDBP = DP / 32, NSDP = DP / 16;
  static_assert(DP == D || 2 * DP == D, "path coordinates: all, or the leading half");
  constexpr int PLANE = C * P * 2;                  // one 64 x 72 bf16 plane (bytes)
  constexpr int SLOT = 2 * PLANE;                   // 18432 B: hi/lo planes or 64 x 72 fp32
  constexpr int WT_BYTES = D * P * 2;
  __shared__ __attribute__((aligned(16))) unsigned char smem[3 * SLOT + WT_BYTES + C * 4];
  // slot 0: N / X (fp32), then T2^T (hi/lo)
  // slot 1: lower(Q W^T) (hi/lo)
  // slot 2: strictLower(W K^T)^T (hi/lo), then (U W)^T (hi/lo) for 64 of the
  // d columns at a time (d = 128: two halves, the second kept in registers
  // meanwhile, so that two blocks fit a CU)
  float *Xs = reinterpret_cast<float *>(smem);
  __bf16 *T2h = reinterpret_cast<__bf16 *>(smem), *T2l = T2h + C * P;
  __bf16 *P1h = reinterpret_cast<__bf16 *>(smem + SLOT), *P1l = P1h + C * P;
  __bf16 *SKh = reinterpret_cast<__bf16 *>(smem + 2 * SLOT), *SKl = SKh + C * P;
  __bf16 *UWh = SKh, *UWl = UWh + C * P;
  __bf16 *Wt = reinterpret_cast<__bf16 *>(smem + 3 * SLOT);
  float *bs = reinterpret_cast<float *>(smem + 3 * SLOT + WT_BYTES);

  const int N = T / C;
  const int sq = (int)io.q.t, sk = (int)io.k.t, sv = (int)io.v.t, sw = (int)io.w.t;
  // the first row of chunk c of head bh in a tensor with token strides st
  auto first_of = [&](int bh, int c, const TokStrides &st) {
    return (long long)(bh / io.H) * st.b + (long long)(bh % io.H) * st.h + (long long)c * C * st.t;
  };

  // d = 64: q, k, v, w of a chunk (32 KiB) are staged in slots 0 and 1, rows
  // swizzled as in sw_off, and every wave reads its operands from there.  The
  // blocks are persistent: each walks chunks blockIdx.x, + gridDim.x, ... and
  // holds the next chunk's inputs (eight 16-byte pieces and beta per thread)
  // in registers while the current chunk is computed, so the load latency is
  // paid once per block.  Piece i of a thread is tensor i / 2 (q, k, v, w),
  // rows 8 ch.. with ch = wv + 4 (i % 2), column piece cc of row r at slot
  // cc ^ (r % 8).  d = 128 reads its operands from global memory, one chunk
  // per block.
  constexpr bool STAGE = D == 64;
  bf16x8 pre[8];
  float bpre = 0.f;
  auto fetch = [&](int blk) {
    const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    const int fbh = blk / N, fc = blk % N;
    const __bf16 *src[4] = {q + first_of(fbh, fc, io.q), k + first_of(fbh, fc, io.k),
                            v + first_of(fbh, fc, io.v), w + first_of(fbh, fc, io.w)};
    const int pitch[4] = {sq, sk, sv, sw};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = i >> 1, ch = wv + 4 * (i & 1);
      const int r = 8 * ch + (lane >> 3), cc = (lane & 7) ^ (r & 7);
      pre[i] = *reinterpret_cast<const bf16x8 *>(src[t] + (long long)r * pitch[t] + cc * 8);
    }
    bpre = tid < C ? beta[first_of(fbh, fc, io.beta) + (long long)tid * io.beta.t] : 0.f;
  };
  if constexpr (STAGE) fetch(blockIdx.x);

  const int blk_end = STAGE ? total : (int)blockIdx.x + 1;   // d = 128: one chunk per block
  for (int blk = blockIdx.x; blk < blk_end; blk += gridDim.x) {
  // The thread index is taken afresh in each chunk (through an empty asm the
  // compiler cannot move out of the loop), so that the many addresses derived
  // from it are not hoisted and kept live across the loop.
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wv = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, n = lane & 31;
  const int mt = wv >> 1, nt = wv & 1;
  const int bh = blk / N, c = blk % N;
  auto first = [&](const TokStrides &st) { return first_of(bh, c, st); };
  float bval;
  if constexpr (STAGE) {
    __syncthreads();   // the previous chunk's reads of slots 0 and 1 are done
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = i >> 1, ch = wv + 4 * (i & 1);
      *reinterpret_cast<bf16x8 *>(smem + (t >> 1) * SLOT + (t & 1) * 8192 + ch * 1024 + lane * 16) =
          pre[i];
    }
    bval = bpre;
    if (blk + (int)gridDim.x < total) fetch(blk + gridDim.x);
  } else {
    bval = tid < C ? beta[first(io.beta) + (long long)tid * io.beta.t] : 0.f;
  }
  const __bf16 *qc = q + first(io.q);
  const __bf16 *kc = k + first(io.k);
  const __bf16 *vc = v + first(io.v);
  const __bf16 *wc = w + first(io.w);
  __bf16 *kf = kvm + ((size_t)bh * N + c) * kvm_elems(D, DP);
  __bf16 *vf = kf + C * D;
  __bf16 *mf = vf + C * D;

  // ---- phase 1: products of the inputs, operands straight from global ----
  // All global reads of this phase are issued before the first use of any of
  // them, so their latencies overlap.
  f32x16 kq = zero16();
  f32x16 qinit[TPW], kinit[TPW];
  const unsigned char *st_q = smem, *st_k = smem + 8192;
  const unsigned char *st_v = smem + SLOT, *st_w = smem + SLOT + 8192;
  {
    bf16x8 wm[KSD], wn[KSD], qn[KSD], kn[KSD], km[KSD];
    // <-Q^T and ->K^T start from Q^T and K^T: tiles (eb, xb) = (tau>>1, tau&1)
    bf16x4 qv[TPW][4], kv[TPW][4];
    if constexpr (STAGE) {
      __syncthreads();   // the staged inputs have landed
      load_rows_sw<KSD>(wm, st_w, 32 * mt, lane);
      load_rows_sw<KSD>(wn, st_w, 32 * nt, lane);
      load_rows_sw<KSD>(qn, st_q, 32 * nt, lane);
      load_rows_sw<KSD>(kn, st_k, 32 * nt, lane);
      load_rows_sw<KSD>(km, st_k, 32 * mt, lane);
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int tau = wv + 4 * u, eb = tau >> 1, xb = tau & 1;
        const int r = 32 * xb + n;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int off = sw_off(r, 4 * eb + r4) + 8 * g;
          qv[u][r4] = *reinterpret_cast<const bf16x4 *>(st_q + off);
          kv[u][r4] = *reinterpret_cast<const bf16x4 *>(st_k + off);
        }
      }
    } else {
      load_rows<KSD>(wm, wc + 32 * mt * (long long)sw, sw, lane);
      load_rows<KSD>(wn, wc + 32 * nt * (long long)sw, sw, lane);
      load_rows<KSD>(qn, qc + 32 * nt * (long long)sq, sq, lane);
      load_rows<KSD>(kn, kc + 32 * nt * (long long)sk, sk, lane);
      load_rows<KSD>(km, kc + 32 * mt * (long long)sk, sk, lane);
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int tau = wv + 4 * u, eb = tau >> 1, xb = tau & 1;
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int cidx = 32 * eb + 8 * r4 + 4 * g, r = 32 * xb + n;
          qv[u][r4] = *reinterpret_cast<const bf16x4 *>(qc + (long long)r * sq + cidx);
          kv[u][r4] = *reinterpret_cast<const bf16x4 *>(kc + (long long)r * sk + cidx);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          qinit[u][4 * r4 + e] = (float)qv[u][r4][e];
          kinit[u][4 * r4 + e] = (float)kv[u][r4][e];
        }
    f32x16 gacc = zero16(), p1acc = zero16(), skacc = zero16();
#pragma unroll
    for (int ks = 0; ks < KSDP; ++ks) {   // products with W: path coordinates only
      gacc = mma32(wm[ks], wn[ks], gacc);     // [j][s]  = w_j . w_s
      p1acc = mma32(wm[ks], qn[ks], p1acc);   // [t][i]  = w_t . q_i
      skacc = mma32(wm[ks], kn[ks], skacc);   // [t][j]  = w_t . k_j
    }
    mma_rows<KSD>(kq, km, qn);      // [j][i]  = k_j . q_i  (kept for the diagonal logits)
    // W^T by exact identity products: tile (t block mt, e block eb)
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int eb = nt + 2 * u;
      if (eb >= NDBP) continue;   // W^T is read only over the path coordinates
      f32x16 acc = zero16();
      acc = mma32(pick(wm, 2 * eb), eye_frag(0, lane), acc);
      acc = mma32(pick(wm, 2 * eb + 1), eye_frag(1, lane), acc);
      const int e = 32 * eb + n;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (__bf16)acc[4 * r4 + i];
        *reinterpret_cast<bf16x4 *>(Wt + e * P + 32 * mt + 8 * r4 + 4 * g) = x;
      }
    }
    // V^T in fragment order by exact identity products: tile (key block mt,
    // d block db); register group h of the tile is blob (db, 2*mt + h).
    {
      bf16x8 vm[KSD];
      if constexpr (STAGE)
        load_rows_sw<KSD>(vm, st_v, 32 * mt, lane);
      else
        load_rows<KSD>(vm, vc + 32 * mt * (long long)sv, sv, lane);
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int db = nt + 2 * u;
        f32x16 acc = zero16();
        acc = mma32(pick(vm, 2 * db), eye_frag(0, lane), acc);
        acc = mma32(pick(vm, 2 * db + 1), eye_frag(1, lane), acc);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x8 x;
#pragma unroll
          for (int t = 0; t < 8; ++t) x[t] = (__bf16)acc[8 * h + t];
          *reinterpret_cast<bf16x8 *>(vf + ((db * NSK + 2 * mt + h) * 64 + lane) * 8) = x;
        }
      }
    }
    if (tid < C) bs[tid] = bval;
    __syncthreads();   // beta visible
    // N = strictLower(D W W^T) (fp32), lower(Q W^T), strictLower(W K^T)^T.
    // Lane column = destination row (s, i or j); 4 consecutive rows of the
    // accumulator = 4 contiguous destination columns.
    const int col = 32 * nt + n;
    const float bcol = bs[col];
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int r0 = 32 * mt + 8 * r4 + 4 * g;
      f32x4 nv, pv, sv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        nv[e] = r0 + e < col ? bcol * gacc[4 * r4 + e] : 0.f;   // N[s = col][j = r0 + e]
        pv[e] = r0 + e <= col ? p1acc[4 * r4 + e] : 0.f;        // P1[i = col][t]
        sv[e] = r0 + e > col ? skacc[4 * r4 + e] : 0.f;         // SK^T[j = col][t]
      }
      *reinterpret_cast<f32x4 *>(Xs + col * PX + r0) = nv;
      store4_split(P1h, P1l, col * P + r0, pv);
      store4_split(SKh, SKl, col * P + r0, sv);
    }
  }
  __syncthreads();

  // ---- phase 2: X = (I + N)^{-1}, 16 x 16 blocks; U = X D ----
  if (wv == 0) {
    // diagonal blocks by forward substitution: lane = (block b, column j)
    const int b = lane >> 4, j = lane & 15, base = 16 * b;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = i == j ? 1.f : 0.f;
#pragma unroll
      for (int t4 = 0; t4 < 4; ++t4) {
        if (4 * t4 < i) {
          const f32x4 nr = *reinterpret_cast<const f32x4 *>(Xs + (base + i) * PX + base + 4 * t4);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * t4 + e < i) acc -= nr[e] * x[4 * t4 + e];
        }
      }
      x[i] = acc;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) Xs[(base + i) * PX + base + j] = x[i];
  }
  __syncthreads();
  if (wv < 3) solve_block<PX>(Xs, wv + 1, wv, lane);       // blocks (1,0) (2,1) (3,2)
  __syncthreads();
  if (wv < 2) solve_block<PX>(Xs, wv + 2, wv, lane);       // blocks (2,0) (3,1)
  __syncthreads();
  if (wv == 0) solve_block<PX>(Xs, 3, 0, lane);            // block (3,0)
  __syncthreads();
  // ---- phase 3: T2 = U strictLower(W K^T) and U W, stored transposed ----
  // uw[u] holds (U W)^T tile (e block nt + 2u, s block mt): u = 0 is the
  // first 64 d columns, u = 1 (d = 128) the second.
  f32x16 uw[TPW];
  {
    // This wave's A fragments of U = X D as hi/lo pairs, straight from X:
    // U[i][s] = X[i][s] beta_s (s < i), beta_i (s == i), 0 (s > i).  Lane l
    // takes row i = 32 mt + l%32 and the 8 columns s0.. = 8 (l/32) + 16 ks,
    // which lie in one 16-block: the diagonal block of X is stored in rows,
    // the blocks below it transposed.
    bf16x8 uh[KSC], ul[KSC];
    {
      const int i = 32 * mt + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < KSC; ++ks) {
        const int s0 = 8 * (lane >> 5) + 16 * ks;
        const bool diag = (s0 >> 4) == (i >> 4);
        const f32x4 r0 = *reinterpret_cast<const f32x4 *>(Xs + i * PX + s0);
        const f32x4 r1 = *reinterpret_cast<const f32x4 *>(Xs + i * PX + s0 + 4);
        const f32x4 b0 = *reinterpret_cast<const f32x4 *>(bs + s0);
        const f32x4 b1 = *reinterpret_cast<const f32x4 *>(bs + s0 + 4);
        float xt[8];   // read whether used or not: no branch per element
#pragma unroll
        for (int t = 0; t < 8; ++t) xt[t] = Xs[(s0 + t) * PX + i];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int sc = s0 + t;
          const float xr = t < 4 ? r0[t] : r1[t - 4];
          const float x = diag ? xr : xt[t];
          const float b = t < 4 ? b0[t] : b1[t - 4];
          const float u = sc < i ? x * b : (sc == i ? b : 0.f);
          const __bf16 h = (__bf16)u;
          uh[ks][t] = h;
          ul[ks][t] = (__bf16)(u - (float)h);
        }
      }
    }
    f32x16 t2 = zero16();
    {
      bf16x8 sh[KSC], sl[KSC];
      load_rows<KSC>(sh, SKh + 32 * nt * P, P, lane);
      load_rows<KSC>(sl, SKl + 32 * nt * P, P, lane);
      mma_rows<KSC>(t2, uh, sh);
      mma_rows<KSC>(t2, uh, sl);
      mma_rows<KSC>(t2, ul, sh);
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      uw[u] = zero16();
      if (nt + 2 * u >= NDBP) continue;   // U W vanishes beyond the path coordinates
      bf16x8 wt[KSC];
      load_rows<KSC>(wt, Wt + 32 * (nt + 2 * u) * P, P, lane);
      mma_rows<KSC>(uw[u], uh, wt);
      mma_rows<KSC>(uw[u], ul, wt);
    }
    __syncthreads();   // X and strictLower(W K^T)^T are dead
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int s0 = 32 * mt + 8 * r4 + 4 * g;
      store4_split(T2h, T2l, (32 * nt + n) * P + s0, quad(t2, r4));         // T2^T[j][s]
      store4_split(UWh, UWl, (32 * nt + n) * P + s0, quad(uw[0], r4));      // (UW)^T[e][s], e < 64
    }
  }
  __syncthreads();

  // ---- phase 4: outputs, in TPW passes over 64 d columns of (U W)^T ----
  float *qa_c = qa + ((size_t)bh * N + c) * qa_floats(D);
  constexpr int MPP = NDB * NDB / 4 / TPW;   // -M tiles per wave and pass
#pragma unroll
  for (int h = 0; h < TPW; ++h) {
    if (h > 0) {   // the next 64 columns of (U W)^T replace the previous ones
      __syncthreads();
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        store4_split(UWh, UWl, (32 * nt + n) * P + 32 * mt + 8 * r4 + 4 * g, quad(uw[h], r4));
      __syncthreads();
    }
    // tile tau = wv + 4h: d block eb (in this pass's columns), query / key block ib
    const int tau = wv + 4 * h, eb = tau >> 1, ib = tau & 1, ebl = eb - 2 * h;
    {
      // <-Q^T = Q^T - (U W)^T lower(Q W^T)^T (= Q^T beyond the path coordinates)
      f32x16 acc = zero16();
      if (eb < NDBP) {
        tile_mma<C>(acc, UWh + 32 * ebl * P, P, P1h + 32 * ib * P, P, lane);
        tile_mma<C>(acc, UWh + 32 * ebl * P, P, P1l + 32 * ib * P, P, lane);
        tile_mma<C>(acc, UWl + 32 * ebl * P, P, P1h + 32 * ib * P, P, lane);
      }
      float *dst = qa_c + ((ib * NDB + eb) * 64 + lane) * 16;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = qinit[h][4 * r4 + e] - acc[4 * r4 + e];
        *reinterpret_cast<f32x4 *>(dst + 4 * r4) = x;
      }
      // ->K^T = K^T - W^T T2 (tile (eb, jb = ib)), into KF fragment blobs
      // (= K^T beyond the path coordinates)
      f32x16 kacc = zero16();
      if (eb < NDBP) {
        tile_mma<C>(kacc, Wt + 32 * eb * P, P, T2h + 32 * ib * P, P, lane);
        tile_mma<C>(kacc, Wt + 32 * eb * P, P, T2l + 32 * ib * P, P, lane);
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x8 x, xl;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float y = kinit[h][8 * hh + t] - kacc[8 * hh + t];
          x[t] = (__bf16)y;
          xl[t] = (__bf16)(y - (float)x[t]);
        }
        const size_t o = ((ib * NSD + 2 * eb + hh) * 64 + lane) * 8;
        *reinterpret_cast<bf16x8 *>(kf + o) = x;
        if (klo) *reinterpret_cast<bf16x8 *>(klo + ((size_t)bh * N + c) * C * D + o) = xl;
      }
    }
    // -M^T in MF fragment blobs: M = W^T (U W), tile (ab, bb) = (tau % NDB,
    // tau / NDB) for tau = wv + 4u, so this pass's columns bb are 2h, 2h + 1.
    // With DP < D (then DP <= 64) the DP x DP block is done in pass 0.
#pragma unroll
    for (int v = 0; v < (DP == D ? MPP : (NDBP * NDBP + 3) / 4); ++v) {
      if (DP < D && (h > 0 || wv + 4 * v >= NDBP * NDBP)) continue;
      const int tm = DP == D ? wv + 4 * (h * MPP + v) : wv + 4 * v;
      const int ab = tm % NDBP, bb = tm / NDBP, bbl = bb - 2 * h;
      f32x16 acc = zero16();
      tile_mma<C>(acc, Wt + 32 * ab * P, P, UWh + 32 * bbl * P, P, lane);
      tile_mma<C>(acc, Wt + 32 * ab * P, P, UWl + 32 * bbl * P, P, lane);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x8 x;
#pragma unroll
        for (int t = 0; t < 8; ++t) x[t] = (__bf16)(-acc[8 * hh + t]);
        *reinterpret_cast<bf16x8 *>(mf + ((bb * NSDP + 2 * ab + hh) * 64 + lane) * 8) = x;
      }
    }
  }
  // Al^T = K Q^T - T2^T lower(Q W^T)^T, tile (jb = mt, ib = nt); the tile with
  // keys 32..63 and queries 0..31 lies above the diagonal and is not stored.
  if (!(mt == 1 && nt == 0)) {
    f32x16 acc = zero16();
    tile_mma<C>(acc, T2h + 32 * mt * P, P, P1h + 32 * nt * P, P, lane);
    tile_mma<C>(acc, T2h + 32 * mt * P, P, P1l + 32 * nt * P, P, lane);
    tile_mma<C>(acc, T2l + 32 * mt * P, P, P1h + 32 * nt * P, P, lane);
    float *dst = al + ((size_t)bh * N + c) * al_floats() + (al_tile(nt, mt) * 64 + lane) * 16;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = kq[4 * r4 + e] - acc[4 * r4 + e];
      *reinterpret_cast<f32x4 *>(dst + 4 * r4) = x;
    }
  }
  }   // chunks of this block
}

// ---------------------------------------------------------------- fp32 path

// One block of 256 threads per (bh, chunk), plain float32 on the vector units.
// LDS: W and U W (64 x D, padded), U, P1 = lower(Q W^T) and T2 = U
// strictLower(W K^T) (64 x 64, padded).
template <int D, int DP>
__global__ __launch_bounds__(256) void prep_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k,
    const float *__restrict__ v, const float *__restrict__ w,
    const float *__restrict__ beta, float *__restrict__ qa,
    float *__restrict__ kvm, float *__restrict__ al, int T) {
  constexpr int C = kChunk, DPW = D + 1, CP = C + 1, NT = 256;
  constexpr int KPL = 1, KSTEP = 2;
  __shared__ float Ws[C * DPW];
  __shared__ float UWs[C * DPW];
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

  // w beyond the path coordinates is not read (taken as zero)
  for (int idx = tid; idx < C * D; idx += NT)
    Ws[(idx / D) * DPW + idx % D] = idx % D < DP ? wc[idx] : 0.f;
  if (tid < C) bs[tid] = beta[row0 + tid];
  __syncthreads();

  // N[i][j] = beta_i (w_i . w_j) for j < i, else 0.
  for (int idx = tid; idx < C * C; idx += NT) {
    const int i = idx / C, j = idx % C;
    float s = 0.f;
    if (j < i) {
      for (int t = 0; t < DP; ++t) s += Ws[i * DPW + t] * Ws[j * DPW + t];
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
    for (int t = 0; t <= s; ++t) acc += Us[s * CP + t] * Ws[t * DPW + col];
    UWs[s * DPW + col] = acc;
  }
  for (int idx = tid; idx < C * C; idx += NT) {
    const int t = idx / C, j = idx % C;
    float acc = 0.f;
    if (t > j)
      for (int e = 0; e < DP; ++e) acc += Ws[t * DPW + e] * kc[(size_t)j * D + e];
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
      for (int e = 0; e < DP; ++e) acc += qc[(size_t)i * D + e] * Ws[t * DPW + e];
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
    for (int t = 0; t <= i; ++t) acc -= P1s[i * CP + t] * UWs[t * DPW + col];
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
  float *kf = kvm + ((size_t)bh * N + c) * kvm_elems(D, DP);
  float *vf = kf + C * D;
  float *mf = vf + C * D;
  {  // KF: ->K[key][dcol] = K[key][dcol] - sum_{s>key} T2[s][key] W[s][dcol]
    constexpr int NS = D / KSTEP;
    for (int it = tid; it < 2 * NS * 64; it += NT) {
      const int blob = it / 64, lane = it % 64, mb = blob / NS, s = blob % NS;
      const int key = 32 * mb + lane % 32, dcol = frag_row(s, lane / 32, 0, KPL);
      float acc = kc[(size_t)key * D + dcol];
      for (int r = key + 1; r < C; ++r) acc -= T2s[r * CP + key] * Ws[r * DPW + dcol];
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
  {  // MF: X[b][a] = -M[a][b] = -sum_s W[s][a] UW[s][b], a, b < DP
    constexpr int NS = DP / KSTEP;
    for (int it = tid; it < (DP / 32) * NS * 64; it += NT) {
      const int blob = it / 64, lane = it % 64, mb = blob / NS, s = blob % NS;
      const int b = 32 * mb + lane % 32, a = frag_row(s, lane / 32, 0, KPL);
      float acc = 0.f;
      for (int r = 0; r < C; ++r) acc += Ws[r * DPW + a] * UWs[r * DPW + b];
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

// Compute units of the device that a stream runs on, cached per device.
hipError_t cu_count(hipStream_t stream, int *out) {
  static std::atomic<int> cache[64];
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < 64;
  int c = cached ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (c <= 0) {
    e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    c = c > 0 ? c : 1;
    if (cached) cache[dev].store(c, std::memory_order_relaxed);
  }
  *out = c;
  return hipSuccess;
}

template <int D, int DP>
hipError_t launch_prep_bf16(const void *q, const void *k, const void *v,
                            const void *w, const float *beta, float *qa,
                            void *kvm, float *al, int BH, int T, const FwdIo &io,
                            hipStream_t stream, void *klo) {
  const int total = BH * (T / kChunk);
  // d = 64: persistent blocks, two per compute unit (the LDS of one block is
  // 63 KiB), each walking total / grid chunks.
  int grid = total;
  if (D == 64) {
    int cus = 0;
    const hipError_t e = cu_count(stream, &cus);
    if (e != hipSuccess) return e;
    grid = std::min(total, 2 * cus);
  }
  hipLaunchKernelGGL((prep_bf16_kernel<D, DP>), dim3(grid), dim3(256), 0,
                     stream, (const __bf16 *)q, (const __bf16 *)k,
                     (const __bf16 *)v, (const __bf16 *)w, beta, qa,
                     (__bf16 *)kvm, al, T, total, io, (__bf16 *)klo);
  return hipGetLastError();
}

template <int D, int DP>
hipError_t launch_prep_f32(const void *q, const void *k, const void *v,
                           const void *w, const float *beta, float *qa,
                           void *kvm, float *al, int BH, int T,
                           hipStream_t stream) {
  hipLaunchKernelGGL((prep_f32_kernel<D, DP>), dim3(BH * (T / kChunk)), dim3(256), 0,
                     stream, (const float *)q, (const float *)k,
                     (const float *)v, (const float *)w, beta, qa,
                     (float *)kvm, al, T);
  return hipGetLastError();
}

// Per key chunk, the two inputs of the exact block skip of the streaming scan
// (forget gate only): the largest gate value a_t of the chunk and the largest
// squared norm of its ->K rows as stored for the scan (bf16 values squared
// exactly, summed in float32).  One wave per chunk, four chunks per block.
// A non-finite value makes its bound +inf, so that no block is skipped on it.
template <typename E, int D, int DP>
__global__ __launch_bounds__(256) void chunk_bounds_kernel(
    const E *__restrict__ kvm, const float *__restrict__ gate,
    float2 *__restrict__ bnd, int n_chunks, int T) {
  constexpr int C = kChunk, KPL = Kpl<E>::value, NS = D / (2 * KPL);
  const int lane = threadIdx.x & 63;
  const int ci = blockIdx.x * 4 + (threadIdx.x >> 6);   // bh * N + c
  if (ci >= n_chunks) return;
  const int N = T / C;
  const int bh = ci / N, c = ci % N;
  float amax = gate[(size_t)bh * T + (size_t)c * C + lane];
  if (!(amax <= 3.0e38f)) amax = INFINITY;   // NaN or +inf
  // fragment order: in every blob of key block mb, lane l holds KPL values of
  // row 32*mb + l%32
  const E *kf = kvm + (size_t)ci * kvm_elems(D, DP);
  float kmax2 = 0.f;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int t = 0; t < KPL; ++t) {
        const float x = to_f32(kf[((mb * NS + s) * 64 + lane) * KPL + t]);
        ss = __builtin_fmaf(x, x, ss);
      }
    ss += __shfl_xor(ss, 32);
    if (!(ss <= 3.0e38f)) ss = INFINITY;
    kmax2 = fmaxf(kmax2, ss);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    amax = fmaxf(amax, __shfl_xor(amax, o));
    kmax2 = fmaxf(kmax2, __shfl_xor(kmax2, o));
  }
  if (lane == 0) bnd[ci] = make_float2(amax, kmax2);
}

template <typename E, int D, int DP>
hipError_t launch_chunk_bounds_t(const void *kvm, const float *gate, float2 *bnd,
                                 int BH, int T, hipStream_t stream) {
  const int n = BH * (T / kChunk);
  hipLaunchKernelGGL((chunk_bounds_kernel<E, D, DP>), dim3((n + 3) / 4), dim3(256), 0, stream,
                     (const E *)kvm, gate, bnd, n, T);
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

hipError_t launch_gate_prefix(const float *logf, float *gate, int BH, int T, const FwdIo &io,
                              hipStream_t stream) {
  hipLaunchKernelGGL(gate_prefix_kernel, dim3(BH), dim3(256), 0, stream, logf,
                     gate, T, io.H, io.logf);
  return hipGetLastError();
}

// float32 inputs are always read in the padded dense layout (io unused).
hipError_t launch_prep(int dtype, int D, int DP, const void *q, const void *k,
                       const void *v, const void *w, const float *beta,
                       float *qa, void *kvm, float *al, int BH, int T,
                       const FwdIo &io, hipStream_t stream, void *klo) {
  const bool half = DP != D;
  if (dtype == 1) {
    if (D == 64)
      return half ? launch_prep_bf16<64, 32>(q, k, v, w, beta, qa, kvm, al, BH, T, io, stream, klo)
                  : launch_prep_bf16<64, 64>(q, k, v, w, beta, qa, kvm, al, BH, T, io, stream, klo);
    return half ? launch_prep_bf16<128, 64>(q, k, v, w, beta, qa, kvm, al, BH, T, io, stream, klo)
                : launch_prep_bf16<128, 128>(q, k, v, w, beta, qa, kvm, al, BH, T, io, stream, klo);
  }
  if (D == 64)
    return half ? launch_prep_f32<64, 32>(q, k, v, w, beta, qa, kvm, al, BH, T, stream)
                : launch_prep_f32<64, 64>(q, k, v, w, beta, qa, kvm, al, BH, T, stream);
  return half ? launch_prep_f32<128, 64>(q, k, v, w, beta, qa, kvm, al, BH, T, stream)
              : launch_prep_f32<128, 128>(q, k, v, w, beta, qa, kvm, al, BH, T, stream);
}

hipError_t launch_chunk_bounds(int dtype, int D, int DP, const void *kvm,
                               const float *gate, float2 *bnd, int BH, int T,
                               hipStream_t stream) {
  const bool half = DP != D;
  if (dtype == 1) {
    if (D == 64)
      return half ? launch_chunk_bounds_t<__bf16, 64, 32>(kvm, gate, bnd, BH, T, stream)
                  : launch_chunk_bounds_t<__bf16, 64, 64>(kvm, gate, bnd, BH, T, stream);
    return half ? launch_chunk_bounds_t<__bf16, 128, 64>(kvm, gate, bnd, BH, T, stream)
                : launch_chunk_bounds_t<__bf16, 128, 128>(kvm, gate, bnd, BH, T, stream);
  }
  if (D == 64)
    return half ? launch_chunk_bounds_t<float, 64, 32>(kvm, gate, bnd, BH, T, stream)
                : launch_chunk_bounds_t<float, 64, 64>(kvm, gate, bnd, BH, T, stream);
  return half ? launch_chunk_bounds_t<float, 128, 64>(kvm, gate, bnd, BH, T, stream)
              : launch_chunk_bounds_t<float, 128, 128>(kvm, gate, bnd, BH, T, stream);
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
