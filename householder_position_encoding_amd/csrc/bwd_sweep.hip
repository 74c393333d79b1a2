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
//   levels  one block per key chunk c' (bf16: per four key chunks, which
//           share each -M_c through LDS) walks c upward,
//           Khat[c+1] = Khat[c] - Khat[c] M_c^T, and stores every level in the
//           input dtype (float32 running value, the product taken on the
//           rounded value, as the forward scan does for its running query
//           tile).
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

template <typename E>
constexpr int KPL_OF() { return MM<E>::KPL; }

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

// Wave-scope ordering of LDS accesses: a wave's later reads see its earlier
// writes (other lanes included) and its later writes follow its earlier reads.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;
typedef __attribute__((address_space(1))) void *gbl_ptr_t;

// Wait until at most n vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14; expcnt, lgkmcnt at maxima).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Block barrier that completes the wave's LDS accesses but leaves its global
// loads (the next step's operand copies) in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


// ------------------------------------------------------------------ levels

__host__ __device__ inline size_t lev_off(int c, int cp, int D) {
  return ((size_t)c * (c - 1) / 2 + cp) * (size_t)C * D;
}

// One window of query chunks [lo, hi): its level buffer holds Khat[c]_{c'}
// for c in [lo - 1, hi), c' < c, at lev_off(c, c') - base in each head's
// slice of `head` elements.
struct Win {
  int lo, hi;
  size_t base, head;
};
__device__ __forceinline__ size_t lev_at(const Win &w, int bh, int c, int cp, int D) {
  return (size_t)bh * w.head + lev_off(c, cp, D) - w.base;
}
// Float32 level checkpoints: level k W of key chunk c' < k W (k = 1 .. nwin-2,
// the levels lo - 1 of the windows between the first and the last) at block
// W k (k-1) / 2 + c' of each head's slice of `head` floats.
struct Ckpt {
  float *p;
  size_t head;
  int W;
};
__device__ __forceinline__ float *ck_at(const Ckpt &k, int bh, int c, int cp, int D) {
  const int kk = c / k.W;
  return k.p + (size_t)bh * k.head + ((size_t)k.W * kk * (kk - 1) / 2 + cp) * (size_t)C * D;
}
// A wave's 32 x D running level (tiles t, rows acc_row) to or from a checkpoint.
template <int D>
__device__ __forceinline__ void ck_store(float *dst, const f32x16 (&x)[D / 32], int lane) {
  const int g = lane >> 5, col = lane & 31;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dst[acc_row(r, g) * D + 32 * t + col] = x[t][r];
}
template <int D>
__device__ __forceinline__ void ck_load(f32x16 (&x)[D / 32], const float *src, int lane) {
  const int g = lane >> 5, col = lane & 31;
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) x[t][r] = src[acc_row(r, g) * D + 32 * t + col];
}

// float32 inputs: each wave walks the levels of 32 keys of one key chunk c'
// (blocks of 2 waves, one per key half) and stores level c in rows [64
// keys][D] and transposed [D][64 keys] (both at lev_at(c, c')).  The product
// takes -M_c straight from global memory (shared by every block of the head)
// and the level from its LDS copy; the row layout is written from that copy
// too.  Window pass (ck_pass = 0): levels [max(lo - 1, c' + 1), hi), from the
// checkpoint at lo - 1 when c' < lo - 1.  First pass (ck_pass = 1, with the
// last window): the whole walk [c' + 1, hi), storing the checkpoint levels
// below the window and the window's levels.
template <int D>
__global__ __launch_bounds__(128) void levels_f32_kernel(const float *__restrict__ kb,
                                                         const float *__restrict__ nm,
                                                         float *__restrict__ levels,
                                                         float *__restrict__ levt, int T, int BH,
                                                         Win win, Ckpt ck, int ck_pass) {
  using E = float;
  constexpr int EPV = 4;            // elements per 16-byte vector
  constexpr int P = D + EPV;        // rows stay 16-byte aligned
  __shared__ __attribute__((aligned(16))) E Xs[2 * 32 * P];
  const int N = T / C;
  const int cp = blockIdx.x / BH, bh = blockIdx.x % BH;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  E *Xw = Xs + wv * 32 * P;
  f32x16 x[D / 32];
  const bool from_ck = !ck_pass && cp < win.lo - 1;
  const int c0 = from_ck ? win.lo - 1 : cp + 1;
  const int c_end = win.hi;
  if (from_ck)
    ck_load<D>(x, ck_at(ck, bh, win.lo - 1, cp, D) + (size_t)32 * wv * D, lane);
  else
    ck_load<D>(x, kb + ((size_t)bh * T + (size_t)cp * C + 32 * wv) * D, lane);
  for (int c = c0; c < c_end; ++c) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t) st_tile(Xw + 32 * t, P, 1, x[t], lane);
    const bool in_win = c >= win.lo - 1;
    if (!in_win) {   // first pass below the window: checkpoints only
      if (c % ck.W == 0) ck_store<D>(ck_at(ck, bh, c, cp, D) + (size_t)32 * wv * D, x, lane);
    } else {
      const size_t off = lev_at(win, bh, c, cp, D);
#pragma unroll
      for (int t = 0; t < D / 32; ++t) st_tile(levt + off + (size_t)32 * t * C + 32 * wv, 1, C, x[t], lane);
    }
    wave_sync();
    if (in_win) {   // level rows from the LDS copy, 16 bytes per lane
      E *dst = levels + lev_at(win, bh, c, cp, D) + (size_t)32 * wv * D;
#pragma unroll
      for (int j = 0; j < 32 * D / EPV / 64; ++j) {
        const int vi = j * 64 + lane, row = vi / (D / EPV), c16 = EPV * (vi % (D / EPV));
        *reinterpret_cast<uint4 *>(dst + (size_t)row * D + c16) =
            *reinterpret_cast<const uint4 *>(Xw + row * P + c16);
      }
    }
    if (c + 1 < c_end) {   // Khat[c+1] = Khat[c] + Khat[c] (-M_c)^T
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
        mma_tile<E, D>(x[t], Xw, P, 1, nm + ((size_t)bh * N + c) * D * D + (size_t)32 * t * D, D,
                       1, lane);
    }
    wave_sync();
  }
}

// The same walk for bf16 inputs, four key chunks c' = 4 grp + j per block
// (8 waves, a wave per 32 keys), walking the levels together so that each
// -M_c is fetched once per block instead of once per wave.  Each wave loads
// one eighth of -M_c (D / 64 16-byte pieces per lane) into registers two
// levels ahead and writes it into an LDS double buffer one level ahead, where
// it is the B operand of every wave's product; one barrier per level
// publishes it and frees the other buffer.  Row r of -M_c keeps its 16-byte
// piece p at position p ^ (r & 7), so a fragment read (32 rows, one piece
// each) touches every bank once.  The per-level sequence of global loads and
// stores is the same in every iteration of the walk (the fetch index is
// clamped at the last chunk), so the compiler's wait for a fetched piece
// covers only operations issued two levels back: the walk's warm-up levels,
// in which the later chunks of the group have not started, are peeled off
// and end with every memory operation complete.  d = 128 also stores each
// level transposed ([D][64 keys], for its dq and dk kernels), straight from
// the register tiles.
template <int D>
__global__ __launch_bounds__(512) void levels_shared_kernel(const float *__restrict__ kb,
                                                            const __bf16 *__restrict__ nm,
                                                            __bf16 *__restrict__ levels,
                                                            __bf16 *__restrict__ levt, int T,
                                                            int BH, Win win, Ckpt ck,
                                                            int ck_pass, float *__restrict__ kn2,
                                                            int *__restrict__ zbad) {
  using E = __bf16;
  constexpr int G = 4, P = D + 8, WARM = G - 1;
  constexpr bool WT = D != 64;            // transposed copy
  constexpr int NP = D * D / 8 / 512;     // 16-byte pieces of -M_c per lane
  constexpr int RV = 32 * D / 8 / 64;     // 16-byte row-store vectors per lane
  // d = 128 keeps 256 registers and spills a few (44 bytes) even so, but two
  // sets of pieces in flight beat one (level walk of B4 H8 T8192: 2.36
  // against 2.60 ms; the per-wave walk took 3.48 ms)
  __shared__ __attribute__((aligned(16))) E ring[2][D * D];
  __shared__ __attribute__((aligned(16))) E Xs[2 * G * 32 * P];
  const int N = T / C;
  const int grp = blockIdx.x / BH, bh = blockIdx.x % BH;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, col = lane & 31;
  // the wave index as a scalar: member-dependent branches stay wave-uniform
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kh = wv & 1, cp = G * grp + (wv >> 1);
  // levels [c_lo, c_end): the window's (from its checkpoint at lo - 1 for
  // chunks below it), or in the first pass (the last window) every level,
  // storing the checkpoints below the window
  const int c_end = win.hi;
  const bool member = cp < c_end - 1;   // a level of this chunk lies in the range
  const int c_lo = ck_pass ? G * grp + 1 : max(win.lo - 1, G * grp + 1);
  E *Xw = Xs + wv * 32 * P;
  f32x16 x[D / 32];
  if (member && !ck_pass && cp < win.lo - 1)
    ck_load<D>(x, ck_at(ck, bh, win.lo - 1, cp, D) + (size_t)32 * kh * D, lane);
  else
    ck_load<D>(x, kb + ((size_t)bh * T + (size_t)(member ? cp : 0) * C + 32 * kh) * D, lane);
  const E *nmh = nm + (size_t)bh * N * D * D;
  // piece i of this wave: row pr(i) of -M_c, 16-byte piece pp(i) of the row
  auto pr = [&](int i) __attribute__((always_inline)) { return ((wv * NP + i) * 64 + lane) / (D / 8); };
  auto pp = [&](int i) __attribute__((always_inline)) { return ((wv * NP + i) * 64 + lane) % (D / 8); };
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  using Pieces = u32x4[NP];
  auto fetch = [&](int c, Pieces &u) __attribute__((always_inline)) {
    c = c < N - 1 ? c : N - 1;
#pragma unroll
    for (int i = 0; i < NP; ++i)
      u[i] = *reinterpret_cast<const u32x4 *>(nmh + (size_t)c * D * D + pr(i) * D + 8 * pp(i));
  };
  auto put = [&](int b, const Pieces &u) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NP; ++i)
      *reinterpret_cast<u32x4 *>(&ring[b][pr(i) * D + 8 * (pp(i) ^ (pr(i) & 7))]) = u[i];
  };
  // level c: store it; step to level c + 1 with -M_c from ring[b]; publish
  // -M_{c+1} (in nx) into ring[b ^ 1] and fetch -M_{c+3} into nx
  auto level = [&](int c, bool active, Pieces &nx) __attribute__((always_inline)) {
    const int b = (c - c_lo) & 1;
    __syncthreads();
    if (active) {
      if (c < win.lo - 1) {   // first pass below the window: checkpoints only
#pragma unroll
        for (int t = 0; t < D / 32; ++t) st_tile(Xw + 32 * t, P, 1, x[t], lane);
        if (c % ck.W == 0) ck_store<D>(ck_at(ck, bh, c, cp, D) + (size_t)32 * kh * D, x, lane);
        wave_sync();
      } else {
        const size_t off = lev_at(win, bh, c, cp, D);
#pragma unroll
        for (int t = 0; t < D / 32; ++t) {
          if constexpr (WT) st_tile(levt + off + (size_t)32 * t * C + 32 * kh, 1, C, x[t], lane);
          st_tile(Xw + 32 * t, P, 1, x[t], lane);
        }
        wave_sync();
        E *dst = levels + off + (size_t)32 * kh * D;
        float nmax = 0.f;   // with kn2: the largest squared row norm of the stored level
#pragma unroll
        for (int j = 0; j < RV; ++j) {
          const int vi = j * 64 + lane, row = vi / (D / 8), c16 = 8 * (vi % (D / 8));
          const uint4 val = *reinterpret_cast<const uint4 *>(Xw + row * P + c16);
          *reinterpret_cast<uint4 *>(dst + (size_t)row * D + c16) = val;
          if (kn2) {
            bf16x8 x;
            __builtin_memcpy(&x, &val, 16);
            float ss = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) ss = __builtin_fmaf((float)x[t], (float)x[t], ss);
#pragma unroll
            for (int o = 1; o < D / 8; o <<= 1) ss += __shfl_xor(ss, o);   // the row's D / 8 lanes
            nmax = fmaxf(nmax, ss <= 3.0e38f ? ss : INFINITY);   // NaN or inf: never skip
          }
        }
        if (kn2) {
          nmax = fmaxf(nmax, __shfl_xor(nmax, 16));
          nmax = fmaxf(nmax, __shfl_xor(nmax, 32));
          if (D == 64) nmax = fmaxf(nmax, __shfl_xor(nmax, 8));
          if (lane == 0) {
            kn2[off / ((size_t)C * D) * 2 + kh] = nmax;
            if (!(nmax <= 3.0e38f)) zbad[bh] = 1;   // a level that is not finite
          }
        }
      }
      if (c + 1 < c_end) {   // Khat[c+1] = Khat[c] + round(Khat[c]) (-M_c)^T
        const E *pa = Xw + col * P + 8 * g;
        const unsigned char *mb = reinterpret_cast<const unsigned char *>(ring[b]);
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks)
            x[t] = MM<E>::mma(
                *reinterpret_cast<const bf16x8 *>(pa + 16 * ks),
                *reinterpret_cast<const bf16x8 *>(mb + (32 * t + col) * 2 * D +
                                                  (((2 * ks + g) ^ (col & 7)) << 4)),
                x[t]);
      }
    }
    put(b ^ 1, nx);
    fetch(c + 3, nx);
  };
  Pieces na, nb;
  {
    Pieces n0;
    fetch(c_lo, n0);
    put(0, n0);
  }
  fetch(c_lo + 1, na);
  fetch(c_lo + 2, nb);
  // warm-up: chunk c' = c_lo - 1 + j starts at level c_lo + j (register sets
  // named at compile time, so that both stay in registers)
  static_assert(WARM == 3, "three warm-up levels");
  if (c_lo < c_end) level(c_lo, member && c_lo > cp, na);
  if (c_lo + 1 < c_end) level(c_lo + 1, member && c_lo + 1 > cp, nb);
  if (c_lo + 2 < c_end) level(c_lo + 2, member && c_lo + 2 > cp, na);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  // steady state: level c_lo + WARM on takes the register set (c - c_lo) & 1
  auto walk = [&](auto stores) __attribute__((always_inline)) {
    int c = c_lo + WARM;
    for (; c + 1 < c_end; c += 2) {   // no exit between the halves: one wait per piece
      level(c, decltype(stores)::value, nb);
      level(c + 1, decltype(stores)::value, na);
    }
    if (c < c_end) level(c, decltype(stores)::value, nb);
  };
  if (member) walk(std::true_type{});
  else walk(std::false_type{});
}

// ------------------------------------------------------------------ skip bounds

// Exact forget-gate skip.  A logit of query q against key j in the sweep is
//     scale * Qa_q . Khat_j + Lambda_q - Lambda_j,
// and its weight exp(logit - lse_q) underflows to exactly zero in float32
// once logit - lse_q < -112 (e^-112 is below the smallest denormal).  With
// |Qa_q . Khat_j| <= |Qa_q| |Khat_j| (the bf16 values the products take,
// float32 sums: the factor 1.01 covers their rounding), a block of query
// chunk c and 32 keys (key half h of chunk c') is all zeros when
//     scale sqrt(max_q |Qa_q|^2 * max_j |Khat_j|^2) * 1.01
//         + max_q (Lambda_q - lse_q) - min_j Lambda_j + 1 < -112;
// its dS is then exactly zero and leaving out its products changes no bit
// (the level walk still crosses it).  This kernel gives the per-chunk query
// terms and the per-half key terms; the level walk gives max |Khat_j|^2.
constexpr float kBwdSkipBelow = -112.f;
// Key chunks a dq wave can list (its query chunk's index, at most): the
// host enables the skip only for N <= kBwdSkipList.
constexpr int kBwdSkipList = 2048;

__device__ __forceinline__ bool bwd_block_vanishes(float scale, float2 qa, float kn2, float kmin) {
  const float b = __builtin_fmaf(scale * __builtin_sqrtf(qa.x * kn2), 1.01f, qa.y - kmin + 1.f);
  return b < kBwdSkipBelow;   // false for NaN: such blocks are computed
}

// One wave per (bh, chunk): lane t is token t of the chunk.
template <typename E, int D>
__global__ __launch_bounds__(64) void bwd_skip_stats_kernel(const E *__restrict__ qae,
                                                             const float *__restrict__ lam,
                                                             const float *__restrict__ lse,
                                                             float2 *__restrict__ qagg,
                                                             float *__restrict__ kmin,
                                                             int *__restrict__ zbad, int T) {
  const int N = T / C;
  const int chunk = blockIdx.x, bh = chunk / N, c = chunk % N, lane = threadIdx.x;
  if (c == 0 && lane == 0) zbad[bh] = 0;   // set by the level walk
  const size_t row = (size_t)bh * T + (size_t)c * C + lane;
  float n2 = 0.f;
  const E *qr = qae + row * D;
  constexpr int V = 16 / (int)sizeof(E);   // elements per 16-byte load
#pragma unroll
  for (int d = 0; d < D; d += V) {
    E x[V];
    __builtin_memcpy(x, qr + d, 16);
#pragma unroll
    for (int t = 0; t < V; ++t) n2 = __builtin_fmaf((float)x[t], (float)x[t], n2);
  }
  float g = lam[row] - lse[row], l = lam[row];
  if (!(n2 <= 3.0e38f)) n2 = INFINITY;   // NaN or inf: never skip
  if (!(g <= 3.0e38f)) g = INFINITY;
  if (!(l >= -3.0e38f)) l = -INFINITY;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    n2 = fmaxf(n2, __shfl_xor(n2, o));
    g = fmaxf(g, __shfl_xor(g, o));
    if (o < 32) l = fminf(l, __shfl_xor(l, o));   // per half of 32 keys
  }
  if (lane == 0) qagg[chunk] = make_float2(n2, g);
  if ((lane & 31) == 0) kmin[(size_t)chunk * 2 + lane / 32] = l;
}

// ------------------------------------------------------------------ dq

// One block of 4 waves per (bh, query chunk c): wave (qh, kh) = (w & 1, w >> 1)
// takes queries 32 qh.. and, at each key chunk, keys 32 kh..; the block
// synchronises only to stage its queries and to combine the key halves.
// Chunk 0 has no earlier keys: its dQa is zero.
template <typename E, int D, bool FOX>
__global__ __launch_bounds__(256, (std::is_same<E, __bf16>::value ? 2 : 1)) void dq_kernel(
    const E *__restrict__ qae, const E *__restrict__ dout, const float *__restrict__ lse,
    const float *__restrict__ dlse, const float *__restrict__ dvec, const float *__restrict__ lam,
    const E *__restrict__ levels, const E *__restrict__ levt, const E *__restrict__ v,
    float scale, float *__restrict__ dqa, float *__restrict__ dlam, int T, int BH, Win win,
    const float *__restrict__ kn2, const float2 *__restrict__ qagg, const float *__restrict__ kmin,
    int skip) {
  constexpr int PQ = D + MM<E>::PAD;          // Qs, Os: [64 q][D]
  constexpr int PG = 32 + MM<E>::PAD;         // Gs: per wave [32 q][32 keys]
  __shared__ __attribute__((aligned(16))) E Qs[C * PQ];
  __shared__ __attribute__((aligned(16))) E Os[C * PQ];
  __shared__ __attribute__((aligned(16))) E Gs[4 * 32 * PG];
  // bf16, d = 64: per wave, the key block transposed [D][32 keys]
  __shared__ __attribute__((aligned(16))) E KtS[(KPL_OF<E>() > 1 && D == 64) ? 4 * D * PG : 1];
  __shared__ float red[2 * 32 * (D + 1)];
  __shared__ float rsum[C];
  const int bh = blockIdx.x % BH, c = win.hi - 1 - blockIdx.x / BH;   // longest walks first
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 5, col = lane & 31;
  const int qh = wv & 1, kh = wv >> 1;
  const size_t qrow = (size_t)bh * T + (size_t)c * C;
  if (c == 0) {
    for (int idx = tid; idx < C * D; idx += 256) dqa[qrow * D + idx] = 0.f;
    return;
  }
  {
    constexpr int EPV = 16 / sizeof(E);
    static_assert(PQ % EPV == 0 || !std::is_same<E, __bf16>::value, "16-byte LDS rows");
    if constexpr (std::is_same<E, __bf16>::value) {
      for (int vi = tid; vi < C * D / EPV; vi += 256) {
        const int r = vi / (D / EPV), c8 = EPV * (vi % (D / EPV));
        *reinterpret_cast<uint4 *>(Qs + r * PQ + c8) = *reinterpret_cast<const uint4 *>(qae + (qrow + r) * D + c8);
        *reinterpret_cast<uint4 *>(Os + r * PQ + c8) = *reinterpret_cast<const uint4 *>(dout + (qrow + r) * D + c8);
      }
    } else {
      for (int idx = tid; idx < C * D; idx += 256) {
        Qs[(idx / D) * PQ + idx % D] = qae[qrow * D + idx];
        Os[(idx / D) * PQ + idx % D] = dout[qrow * D + idx];
      }
    }
  }
  const int myq = 32 * qh + col;
  const float q_lse = lse[qrow + myq], q_d = dvec[qrow + myq];
  const float q_dl = dlse ? dlse[qrow + myq] : 0.f;
  const float q_lam = FOX ? lam[qrow + myq] : 0.f;
  f32x16 dq[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) zero16(dq[t]);
  float rowsum = 0.f;
  const size_t lev_c = lev_at(win, bh, c, 0, D);
  E *Gw = Gs + wv * 32 * PG;
  __syncthreads();
  // Matrix-core A operands of one key chunk for this wave: Khat[c]_{c'} rows
  // (keys 32 kh..), V rows, Khat[c]_{c'}^T rows (d, contraction over keys
  // 32 kh..); bf16 with d = 64 fetches the next key chunk's one step ahead.
  using frag = typename MM<E>::frag;
  constexpr int KPL = MM<E>::KPL, KSD = D / (2 * KPL), KSK = 32 / (2 * KPL);
  constexpr bool PF = KPL > 1 && D == 64;
  struct Frags {
    frag k[PF ? KSD : 1], v[PF ? KSD : 1];
  };
  auto fetch = [&](int cp, Frags &f) {
    if constexpr (PF) {
      const size_t blk = lev_c + (size_t)cp * C * D;
      const size_t krow = (size_t)bh * T + (size_t)cp * C + 32 * kh;
      const E *pk = levels + blk + (size_t)(32 * kh + col) * D + KPL * g;
      const E *pv = v + (krow + col) * D + KPL * g;
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        f.k[ks] = MM<E>::ld(pk + 2 * KPL * ks, 1);
        f.v[ks] = MM<E>::ld(pv + 2 * KPL * ks, 1);
      }
    }
  };
  const E *qb = Qs + (32 * qh + col) * PQ + KPL * g, *ob = Os + (32 * qh + col) * PQ + KPL * g;
  auto step = [&](int cp, Frags &fc, Frags &fn) {
    const size_t blk = lev_c + (size_t)cp * C * D;   // Khat[c]_{c'}
    const size_t krow = (size_t)bh * T + (size_t)cp * C + 32 * kh;
    if (PF && cp >= 1) fetch(cp - 1, fn);
    // S^T and dP^T tiles: rows = keys 32 kh.., columns = queries 32 qh..
    f32x16 s, dp;
    zero16(s);
    zero16(dp);
    if constexpr (PF) {
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        s = MM<E>::mma(fc.k[ks], MM<E>::ld(qb + 2 * KPL * ks, 1), s);
        dp = MM<E>::mma(fc.v[ks], MM<E>::ld(ob + 2 * KPL * ks, 1), dp);
      }
    } else {
      mma_tile<E, D>(s, levels + blk + (size_t)32 * kh * D, D, 1, Qs + 32 * qh * PQ, PQ, 1, lane);
      mma_tile<E, D>(dp, v + krow * D, D, 1, Os + 32 * qh * PQ, PQ, 1, lane);
    }
    f32x16 gt;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float kl = FOX ? lam[krow + acc_row(r, g)] : 0.f;
      const float p = __expf(scale * s[r] + q_lam - kl - q_lse);
      const float ds = p * (dp[r] - q_d + q_dl);
      rowsum += ds;
      gt[r] = scale * ds;
    }
    st_tile(Gw, 1, PG, gt, lane);   // Gw[q][key] = g(q, key)
    if constexpr (PF) {   // this wave's key block transposed: Kt[d][key]
      E *kt = KtS + wv * D * PG;
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
        for (int t = 0; t < KPL; ++t) kt[(KPL * g + 2 * KPL * ks + t) * PG + col] = fc.k[ks][t];
    }
    wave_sync();
    // dQa^T(d, q) += sum_key Khat(key, d) g(q, key)
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      if constexpr (PF) {
        const E *gb = Gw + col * PG + KPL * g;
        const E *ka = KtS + wv * D * PG + (32 * t + col) * PG + KPL * g;
#pragma unroll
        for (int ks = 0; ks < KSK; ++ks)
          dq[t] = MM<E>::mma(MM<E>::ld(ka + 2 * KPL * ks, 1), MM<E>::ld(gb + 2 * KPL * ks, 1), dq[t]);
      } else {
        mma_tile<E, 32>(dq[t], levt + blk + (size_t)32 * t * C + 32 * kh, C, 1, Gw, PG, 1, lane);
      }
    }
    wave_sync();
  };
  if constexpr (KPL > 1 && D == 128) {
    // bf16, d = 128: the key chunk's level rows and V rows are loaded one
    // key chunk ahead into one register set, right after the products that
    // read them are issued; its gate values and transposed level rows (A
    // operands of the dQa product) are loaded before the next chunk's, ahead
    // of the softmax.  No operand is read from global memory inside a
    // product.
    frag kf[KSD], vf[KSD], lt[D / 32][KSK];
    float kl[16];
    auto fetch_kv = [&](int cp) __attribute__((always_inline)) {
      const size_t blk = lev_c + (size_t)cp * C * D;
      const size_t krow = (size_t)bh * T + (size_t)cp * C + 32 * kh;
      const E *pk = levels + blk + (size_t)(32 * kh + col) * D + KPL * g;
      const E *pv = v + (krow + col) * D + KPL * g;
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        kf[ks] = MM<E>::ld(pk + 2 * KPL * ks, 1);
        vf[ks] = MM<E>::ld(pv + 2 * KPL * ks, 1);
      }
    };
    auto fetch_kl = [&](int cp) __attribute__((always_inline)) {
      const size_t krow = (size_t)bh * T + (size_t)cp * C + 32 * kh;
#pragma unroll
      for (int r = 0; r < 16; ++r) kl[r] = FOX ? lam[krow + acc_row(r, g)] : 0.f;
    };
    const E *qb = Qs + (32 * qh + col) * PQ + KPL * g, *ob = Os + (32 * qh + col) * PQ + KPL * g;
    // one key chunk cp; the next one in the walk is cpn
    auto step128 = [&](int cp, int cpn) __attribute__((always_inline)) {
      const size_t blk = lev_c + (size_t)cp * C * D;
      f32x16 s, dp;
      zero16(s);
      zero16(dp);
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) {
        s = MM<E>::mma(kf[ks], MM<E>::ld(qb + 2 * KPL * ks, 1), s);
        dp = MM<E>::mma(vf[ks], MM<E>::ld(ob + 2 * KPL * ks, 1), dp);
      }
      __builtin_amdgcn_sched_barrier(0);
      // this key chunk's gate values and transposed rows, then the next key
      // chunk's operands
      if constexpr (FOX) fetch_kl(cp);
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int ks = 0; ks < KSK; ++ks)
          lt[t][ks] = MM<E>::ld(levt + blk + (size_t)(32 * t + col) * C + 32 * kh + KPL * g + 2 * KPL * ks, 1);
      fetch_kv(cpn);
      __builtin_amdgcn_sched_barrier(0);
      f32x16 gt;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __expf(scale * s[r] + q_lam - (FOX ? kl[r] : 0.f) - q_lse);
        const float ds = p * (dp[r] - q_d + q_dl);
        rowsum += ds;
        gt[r] = scale * ds;
      }
      st_tile(Gw, 1, PG, gt, lane);   // Gw[q][key] = g(q, key)
      wave_sync();
      // dQa^T(d, q) += sum_key Khat(key, d) g(q, key)
      const E *gb = Gw + col * PG + KPL * g;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int ks = 0; ks < KSK; ++ks)
          dq[t] = MM<E>::mma(lt[t][ks], MM<E>::ld(gb + 2 * KPL * ks, 1), dq[t]);
      wave_sync();
    };
    static_assert(2 * 32 * (D + 1) >= 4 * kBwdSkipList, "skip lists fit the reduction area");
    if (FOX && skip) {
      // the key chunks whose block with this chunk's queries and this wave's
      // key half does not vanish (bwd_block_vanishes), descending, listed in
      // the reduction area (free until the end); the host enables the skip
      // only when they fit
      int *lst = reinterpret_cast<int *>(red) + wv * kBwdSkipList;
      const float2 qa = qagg[(size_t)bh * (T / C) + c];
      int cnt = 0;
      for (int base = c - 1; base >= 0; base -= 64) {
        const int cp = base - lane;
        bool keep = cp >= 0;
        if (keep)
          keep = !bwd_block_vanishes(scale, qa, kn2[lev_at(win, bh, c, cp, D) / ((size_t)C * D) * 2 + kh],
                                     kmin[((size_t)bh * (T / C) + cp) * 2 + kh]);
        const unsigned long long m = __ballot(keep);
        if (keep) lst[cnt + __popcll(m & ((1ull << lane) - 1ull))] = cp;
        cnt += __popcll(m);
      }
      wave_sync();
      if (cnt > 0) {
        fetch_kv(__builtin_amdgcn_readfirstlane(lst[0]));
        for (int i = 0; i < cnt; ++i) {
          const int cp = __builtin_amdgcn_readfirstlane(lst[i]);
          const int cpn = __builtin_amdgcn_readfirstlane(lst[i + 1 < cnt ? i + 1 : i]);
          step128(cp, cpn);
        }
      }
    } else {
      fetch_kv(c - 1);
      for (int cp = c - 1; cp >= 0; --cp) step128(cp, cp > 0 ? cp - 1 : 0);
    }
  } else {
    Frags fa, fb;
    fetch(c - 1, fa);
    for (int cp = c - 1; cp >= 0; cp -= 2) {
      step(cp, fa, fb);
      if (cp - 1 < 0) break;
      step(cp - 1, fb, fa);
    }
  }
  // combine the two key halves, then store dQa rows; the barrier keeps a wave
  // that is done from overwriting the key lists the others still walk
  __syncthreads();
  float *rq = red + qh * 32 * (D + 1);
  rowsum += __shfl_xor(rowsum, 32);
  if (kh == 1) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) rq[col * (D + 1) + 32 * t + acc_row(r, g)] = dq[t][r];
    if (g == 0) rsum[myq] = rowsum;
  }
  __syncthreads();
  if (kh == 0) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int d = 32 * t + acc_row(r, g);
        dqa[(qrow + myq) * D + d] = dq[t][r] + rq[col * (D + 1) + d];
      }
    if (FOX && g == 0) dlam[qrow + myq] += rowsum + rsum[myq];
  }
}

// bf16, d = 64: one block of 4 waves per (bh, query chunk c); wave (st, kh)
// = (w >> 1, w & 1) takes keys 32 kh.. of the key chunks c' = c-1-st,
// c-3-st, ... against all 64 queries, so each level block is read from HBM
// once and a window's few query chunks still fill the chip.  The key block's
// fragments (for S^T) are fetched one key chunk ahead and transposed on chip
// for the dQa product; the four partial dQa are summed through LDS.
template <bool FOX>
__global__ __launch_bounds__(256) void dq64_kernel(
    const __bf16 *__restrict__ qae, const __bf16 *__restrict__ dout,
    const float *__restrict__ lse, const float *__restrict__ dlse,
    const float *__restrict__ dvec, const float *__restrict__ lam,
    const __bf16 *__restrict__ levels, const __bf16 *__restrict__ v, float scale,
    float *__restrict__ dqa, float *__restrict__ dlam, int T, int BH, Win win) {
  using E = __bf16;
  constexpr int D = 64, PQ = D + 8, PG = 32 + 8, KS = D / 16;
  __shared__ __attribute__((aligned(16))) E Qs[C * PQ];
  __shared__ __attribute__((aligned(16))) E Os[C * PQ];
  // per wave g[q][key] and Khat^T[d][key]; at the end the reduction
  __shared__ __attribute__((aligned(16))) E pool[4 * C * PG + 4 * D * PG];
  __shared__ float rsum[2][C];
  E *Gs = pool, *KtS = pool + 4 * C * PG;
  const int bh = blockIdx.x % BH, c = win.hi - 1 - blockIdx.x / BH;   // longest walks first
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 5, col = lane & 31;
  const int kh = wv & 1, st = wv >> 1;
  const size_t qrow = (size_t)bh * T + (size_t)c * C;
  if (c == 0) {
    for (int idx = tid; idx < C * D; idx += 256) dqa[qrow * D + idx] = 0.f;
    return;
  }
  for (int vi = tid; vi < C * D / 8; vi += 256) {
    const int r = vi / (D / 8), c8 = 8 * (vi % (D / 8));
    *reinterpret_cast<uint4 *>(Qs + r * PQ + c8) = *reinterpret_cast<const uint4 *>(qae + (qrow + r) * D + c8);
    *reinterpret_cast<uint4 *>(Os + r * PQ + c8) = *reinterpret_cast<const uint4 *>(dout + (qrow + r) * D + c8);
  }
  float q_lse[2], q_d[2], q_dl[2], q_lam[2], rowsum[2] = {0.f, 0.f};
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int q = 32 * qt + col;
    q_lse[qt] = lse[qrow + q];
    q_d[qt] = dvec[qrow + q];
    q_dl[qt] = dlse ? dlse[qrow + q] : 0.f;
    q_lam[qt] = FOX ? lam[qrow + q] : 0.f;
  }
  f32x16 dq[D / 32][2];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    zero16(dq[t][0]);
    zero16(dq[t][1]);
  }
  const size_t lev_c = lev_at(win, bh, c, 0, D);
  E *Gw = Gs + wv * C * PG, *Kt = KtS + wv * D * PG;
  __syncthreads();
  // one key chunk's operands: level rows and V rows (B operands) and, with the
  // gate, Lambda of the wave's keys
  struct Frags {
    bf16x8 k[KS], v[KS];
    float kl[FOX ? 16 : 1];
  };
  // The fetch index is clamped at chunk 0 and every step fetches, so the
  // sequence of loads is the same in every step and the compiler's wait for
  // a step's operands leaves the next step's loads in flight.
  auto fetch = [&](int cp, Frags &f) {
    cp = cp > 0 ? cp : 0;
    const E *pk = levels + lev_c + (size_t)cp * C * D + (size_t)(32 * kh + col) * D + 8 * g;
    const E *pv = v + ((size_t)bh * T + (size_t)cp * C + 32 * kh + col) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      f.k[ks] = *reinterpret_cast<const bf16x8 *>(pk + 16 * ks);
      f.v[ks] = *reinterpret_cast<const bf16x8 *>(pv + 16 * ks);
    }
    if constexpr (FOX) {
      const float *pl = lam + (size_t)bh * T + (size_t)cp * C + 32 * kh;
#pragma unroll
      for (int r = 0; r < 16; ++r) f.kl[r] = pl[acc_row(r, g)];
    }
  };
  auto step = [&](int cp, Frags &fc, Frags &fn) {
    fetch(cp - 2, fn);
    __builtin_amdgcn_sched_barrier(0);   // issue the loads before this step's products
    float kl[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) kl[r] = FOX ? fc.kl[r] : 0.f;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      // S^T and dP^T: rows = this wave's 32 keys, columns = queries 32 qt..
      f32x16 s, dp;
      zero16(s);
      zero16(dp);
      const E *qb = Qs + (32 * qt + col) * PQ + 8 * g, *ob = Os + (32 * qt + col) * PQ + 8 * g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = MM<E>::mma(fc.k[ks], *reinterpret_cast<const bf16x8 *>(qb + 16 * ks), s);
        dp = MM<E>::mma(fc.v[ks], *reinterpret_cast<const bf16x8 *>(ob + 16 * ks), dp);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __expf(scale * s[r] + q_lam[qt] - kl[r] - q_lse[qt]);
        const float ds = p * (dp[r] - q_d[qt] + q_dl[qt]);
        rowsum[qt] += ds;
        s[r] = scale * ds;
      }
      st_tile(Gw + 32 * qt * PG, 1, PG, s, lane);   // Gw[q][key] = g(q, key)
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)   // Kt[d][key]
#pragma unroll
      for (int t = 0; t < 8; ++t) Kt[(8 * g + 16 * ks + t) * PG + col] = fc.k[ks][t];
    wave_sync();
    // dQa^T(d, q) += sum_key Khat(key, d) g(q, key)
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      const E *ka = Kt + (32 * t + col) * PG + 8 * g;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const E *gb = Gw + (32 * qt + col) * PG + 8 * g;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          dq[t][qt] = MM<E>::mma(*reinterpret_cast<const bf16x8 *>(ka + 16 * ks),
                                 *reinterpret_cast<const bf16x8 *>(gb + 16 * ks), dq[t][qt]);
      }
    }
    wave_sync();
  };
  Frags fa, fb;
  int cp = c - 1 - st;
  fetch(cp, fa);
  for (; cp >= 2; cp -= 4) {   // no exit between the halves
    step(cp, fa, fb);
    step(cp - 2, fb, fa);
  }
  if (cp >= 0) step(cp, fa, fb);
  // sum the four partials through LDS (over Gs and KtS): first stream 1 onto
  // stream 0 (per key half), then key half 1 onto key half 0
  float *red = reinterpret_cast<float *>(pool);   // [2][64 q][D + 1] floats
  static_assert(2 * C * (D + 1) * 4 <= (4 * C * PG + 4 * D * PG) * 2, "reduction area");
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) rowsum[qt] += __shfl_xor(rowsum[qt], 32);
  auto put = [&](float *r, float *rs) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int i = 0; i < 16; ++i) r[(32 * qt + col) * (D + 1) + 32 * t + acc_row(i, g)] = dq[t][qt][i];
    if (g == 0) {
      rs[col] = rowsum[0];
      rs[32 + col] = rowsum[1];
    }
  };
  auto add = [&](const float *r, const float *rs) {
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int i = 0; i < 16; ++i) dq[t][qt][i] += r[(32 * qt + col) * (D + 1) + 32 * t + acc_row(i, g)];
    rowsum[0] += rs[col];
    rowsum[1] += rs[32 + col];
  };
  __syncthreads();
  if (st == 1) put(red + kh * C * (D + 1), rsum[kh]);
  __syncthreads();
  if (st == 0) add(red + kh * C * (D + 1), rsum[kh]);
  __syncthreads();
  if (wv == 1) put(red, rsum[0]);
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int q = 32 * qt + col;
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d0 = 32 * t + 8 * r4 + 4 * g;
          float4 o;
          o.x = dq[t][qt][4 * r4] + red[q * (D + 1) + d0];
          o.y = dq[t][qt][4 * r4 + 1] + red[q * (D + 1) + d0 + 1];
          o.z = dq[t][qt][4 * r4 + 2] + red[q * (D + 1) + d0 + 2];
          o.w = dq[t][qt][4 * r4 + 3] + red[q * (D + 1) + d0 + 3];
          *reinterpret_cast<float4 *>(dqa + (qrow + q) * D + d0) = o;
        }
      if (FOX && g == 0) dlam[qrow + q] += rowsum[qt] + rsum[0][q];
    }
  }
}

// ------------------------------------------------------------------ dk

// LDS layout (elements of E) of the dk kernel.
template <typename E, int D, int G>
struct DkLds {
  static constexpr bool BF = std::is_same<E, __bf16>::value;
  static constexpr int PAD = MM<E>::PAD;
  static constexpr int PQ = D + PAD;              // Qs, Os rows [64 q][D]
  static constexpr int PQT = C + PAD;             // Qt, Ot rows [D][64 q] (bf16 only)
  static constexpr int PP = C + PAD;              // per-wave P^T, g^T rows [32 keys][64 q]
  static constexpr int KG = 64 * G;               // keys of a group
  static constexpr int PGT = KG + PAD;            // Gamma^T rows [D][KG] (bf16)
  static constexpr int PGN = D + PAD;             // Gamma rows [KG][D] (float); rounded Gamma rows (bf16)
  static constexpr int STAGE = BF ? 2 * C * PQ + 2 * D * PQT : 2 * C * PQ;
  static constexpr int GX = BF ? D * PGT : KG * PGN;
  static constexpr int WAVES = 2 * G;
  static constexpr int PERWAVE = 2 * 32 * PP;     // P^T and g^T; rounded Gamma rows at crossings
  static_assert(32 * PGN <= PERWAVE, "rounded Gamma rows must fit the wave's P/g area");
};

// One block of 2G waves per (group of G key chunks, bh); wave w takes keys
// 32 (w & 1).. of chunk c' = G*group + (w >> 1).
template <typename E, int D, int G, bool FOX>
__global__ __launch_bounds__(128 * G) void dk_kernel(
    const E *__restrict__ qae, const E *__restrict__ qat, const E *__restrict__ dout,
    const E *__restrict__ dot, const float *__restrict__ lse, const float *__restrict__ dlse,
    const float *__restrict__ dvec, const float *__restrict__ lam, const E *__restrict__ levels,
    const E *__restrict__ levt, const E *__restrict__ v, const E *__restrict__ nmt,
    float scale, float *__restrict__ dkb, float *__restrict__ dv, float *__restrict__ dlam,
    float *__restrict__ dmpart, int T, int BH, Win win, int slots, float *__restrict__ gstate,
    const float *__restrict__ kn2, const float2 *__restrict__ qagg, const float *__restrict__ kmin,
    int skip, int *__restrict__ zhi) {
  using L = DkLds<E, D, G>;
  constexpr bool BF = L::BF;
  constexpr int NW = L::WAVES, NTH = 64 * NW;
  __shared__ __attribute__((aligned(16))) E stage[L::STAGE];
  __shared__ __attribute__((aligned(16))) E gx[L::GX];
  __shared__ __attribute__((aligned(16))) E pw[NW * L::PERWAVE];
  __shared__ float4 qst[C];
  const int N = T / C, NG = (N + G - 1) / G;
  const int grp = blockIdx.x / BH, bh = blockIdx.x % BH;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, g = lane >> 5, col = lane & 31;
  const int kh = wv & 1, cp = G * grp + (wv >> 1);
  const size_t head = (size_t)bh * T;
  const size_t krow = head + (size_t)cp * C + 32 * kh;   // first key row of this wave
  const bool member = cp < N;
  E *Qs = stage, *Os = stage + C * L::PQ;
  E *Qt = stage + 2 * C * L::PQ, *Ot = Qt + D * L::PQT;   // bf16 only
  E *PT = pw + wv * L::PERWAVE, *GT = PT + 32 * L::PP;
  E *GR = PT;                                             // rounded Gamma rows at crossings
  const int kbase = 64 * (wv >> 1) + 32 * kh;             // this wave's keys within the group
  const int c_low = G * grp + 1;   // last query chunk the group visits
  // this window's steps: query chunks top down to bottom
  const int top = win.hi - 1, bottom = max(win.lo, c_low);
  const bool has_work = member && cp < top;

  f32x16 gam[D / 32], dva[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    zero16(gam[t]);
    zero16(dva[t]);
  }
  if (has_work && win.hi < N)   // Gamma as the window above left it
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) gam[t][r] = gstate[(krow + acc_row(r, g)) * D + 32 * t + col];
  float colsum = 0.f;
  const float my_lam = (FOX && member) ? lam[krow + col] : 0.f;
  // bf16: the next step's global reads are in flight during the current
  // step: its query-side copies (into registers, stored to LDS at the top of
  // the next step) and this wave's level rows Khat[c-1]_{c'} (B operands of
  // S); the wave's V rows (B operands of dP) stay in registers for the whole
  // walk.  Each step issues these loads before any other global access, so
  // the waits of the step's later loads (crossing operands) do not wait for
  // anything issued later.
  using frag = typename MM<E>::frag;
  constexpr int KPL = MM<E>::KPL, KSD = BF ? D / (2 * KPL) : 1;
  constexpr int NV = BF ? C * D / 8 / NTH : 1;      // 16-byte copies per thread and tensor
  static_assert(!BF || C * D / 8 % NTH == 0, "copies split evenly over the block");
  bf16x8 cq[BF ? NV : 1], co[BF ? NV : 1], cqt[BF ? NV : 1], cot[BF ? NV : 1];
  float4 cst = make_float4(0.f, 0.f, 0.f, 0.f);
  frag vfr[KSD], kfr[KSD];
  // bf16: -M_{c-1}^T of the step's crossing, prefetched with the level rows
  // and parked in the staging area (free once the step's products are done)
  // next to Khat[c-1]^T, so that the crossing's products read only LDS
  constexpr int NM = BF ? D * D / 8 / NTH : 1;      // 16-byte pieces of -M^T per thread
  constexpr int PMT = D + L::PAD;                   // -M^T rows [D][D] in LDS
  static_assert(!BF || D * L::PGT + D * PMT <= L::STAGE, "crossing operands fit the staging area");
  bf16x8 mreg[NM];
  E *KX = stage, *MT = stage + D * L::PGT;          // crossing: Khat[m]^T [D][KG], -M_m^T [D][D]
  auto fetch_mt = [&](int mm) __attribute__((always_inline)) {
    if constexpr (BF) {
      const E *src = nmt + ((size_t)bh * N + mm) * D * D;
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        const int vi = tid + NTH * i;
        mreg[i] = *reinterpret_cast<const bf16x8 *>(src + (size_t)vi * 8);
      }
    }
  };
  auto fetch_copy = [&](int cc) __attribute__((always_inline)) {
    if constexpr (BF) {
      const size_t qr = head + (size_t)cc * C;
      const E *sq = qae + qr * D, *so = dout + qr * D;
      const E *sqt = qat + qr * D, *sot = dot + qr * D;   // chunk block [D][64]
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int vi = tid + NTH * i, r = vi / (D / 8), c8 = 8 * (vi % (D / 8));
        const int rt = vi / (C / 8), ct = 8 * (vi % (C / 8));
        cq[i] = *reinterpret_cast<const bf16x8 *>(sq + r * D + c8);
        co[i] = *reinterpret_cast<const bf16x8 *>(so + r * D + c8);
        cqt[i] = *reinterpret_cast<const bf16x8 *>(sqt + rt * C + ct);
        cot[i] = *reinterpret_cast<const bf16x8 *>(sot + rt * C + ct);
      }
      if (tid < C)
        cst = make_float4(lse[qr + tid], dvec[qr + tid], dlse ? dlse[qr + tid] : 0.f,
                          FOX ? lam[qr + tid] : 0.f);
    }
  };
  // exact forget-gate skip (bf16): this wave's block against query chunk c
  // vanishes when bwd_block_vanishes; its bound's inputs for the next step
  // are loaded with the level rows
  const bool do_skip = BF && FOX && skip && member;
  const float my_kmin = do_skip ? kmin[((size_t)bh * N + cp) * 2 + kh] : 0.f;
  float nx_kn2 = 0.f;
  float2 nx_qa = make_float2(0.f, 0.f);
  auto fetch_bound = [&](int cc) __attribute__((always_inline)) {
    if (do_skip && cc > cp) {
      nx_kn2 = kn2[lev_at(win, bh, cc, cp, D) / ((size_t)C * D) * 2 + kh];
      nx_qa = qagg[(size_t)bh * N + cc];
    }
  };
  auto fetch_level = [&](int cc) __attribute__((always_inline)) {
    if constexpr (BF) {   // rows Khat[cc]_{c'} of this wave's keys, B-operand fragments
      const E *kl = levels + lev_at(win, bh, cc, cp, D) + (size_t)(32 * kh + col) * D + KPL * g;
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) kfr[ks] = MM<E>::ld(kl + 2 * KPL * ks, 1);
    }
  };
  // Whole steps.  Gamma starts at zero (at the top of the walk, or as the
  // window above left it) and stays exactly zero while every block of the
  // group vanishes: such a step adds nothing, and its crossing only zeros
  // (Gamma (I - M) and the dM partial, for finite levels and M; a level or
  // an M that is not finite shows in the stored levels, which turns this off
  // for the head).  The walk starts at the highest step of the window where
  // a block of the group does not vanish; dm_reduce leaves out the group's
  // partials of the transitions above it.
  int cs = top;
  if (BF && FOX && skip) {
    __shared__ int zw[NW];
    int hw = top;   // this wave's highest step with work
    bool gz = true;
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) gz = gz && gam[t][r] == 0.f;
    if (!zhi[(size_t)BH * N + bh] && __ballot(!gz) == 0ull) {
      hw = bottom - 1;
      if (member)
        for (int base = top; base >= bottom; base -= 64) {
          const int cc = base - lane;
          bool work = false;
          if (cc >= bottom && cc > cp)
            work = !bwd_block_vanishes(scale, qagg[(size_t)bh * N + cc],
                                       kn2[lev_at(win, bh, cc, cp, D) / ((size_t)C * D) * 2 + kh],
                                       my_kmin);
          const unsigned long long m = __ballot(work);
          if (m) {   // the lowest such lane has the highest step
            hw = base - (__ffsll((long long)m) - 1);
            break;
          }
        }
    }
    if (lane == 0) zw[wv] = hw;
    __syncthreads();
    cs = bottom - 1;
#pragma unroll
    for (int i = 0; i < NW; ++i) cs = max(cs, zw[i]);
    if (tid == 0) zhi[(size_t)bh * NG + grp] = cs < top ? cs : 0x7fffffff;
    // a chunk whose last step is among the skipped ones: dKb = Gamma = 0
    if (member && cp + 1 > cs && cp + 1 <= top && cp + 1 >= bottom)
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) dkb[(krow + acc_row(r, g)) * D + 32 * t + col] = gam[t][r];
  }
  if constexpr (BF) {
    if (member) {
      const E *vr = v + (krow + col) * D + KPL * g;
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) vfr[ks] = MM<E>::ld(vr + 2 * KPL * ks, 1);
      if (cs >= bottom && cs > cp) fetch_level(cs);
      if (cs >= bottom) fetch_bound(cs);
    }
    if (cs >= bottom) fetch_copy(cs);
  }
  for (int c = cs; c >= bottom; --c) {
    const bool active = member && c > cp;
    const size_t qrow = head + (size_t)c * C;
    __syncthreads();
    if constexpr (BF) {   // the prefetched copies of Qa, dO (rows) and Qa^T, dO^T
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int vi = tid + NTH * i, r = vi / (D / 8), c8 = 8 * (vi % (D / 8));
        const int rt = vi / (C / 8), ct = 8 * (vi % (C / 8));
        *reinterpret_cast<bf16x8 *>(Qs + r * L::PQ + c8) = cq[i];
        *reinterpret_cast<bf16x8 *>(Os + r * L::PQ + c8) = co[i];
        *reinterpret_cast<bf16x8 *>(Qt + rt * L::PQT + ct) = cqt[i];
        *reinterpret_cast<bf16x8 *>(Ot + rt * L::PQT + ct) = cot[i];
      }
      if (tid < C) qst[tid] = cst;
    } else {
      for (int idx = tid; idx < C * D; idx += NTH) {
        Qs[(idx / D) * L::PQ + idx % D] = qae[qrow * D + idx];
        Os[(idx / D) * L::PQ + idx % D] = dout[qrow * D + idx];
      }
      if (tid < C)
        qst[tid] = make_float4(lse[qrow + tid], dvec[qrow + tid], dlse ? dlse[qrow + tid] : 0.f,
                               FOX ? lam[qrow + tid] : 0.f);
    }
    __syncthreads();
    frag kcur[KSD];
    const bool vanish = do_skip && active && bwd_block_vanishes(scale, nx_qa, nx_kn2, my_kmin);
    if constexpr (BF) {
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks) kcur[ks] = kfr[ks];
      fetch_bound(c - 1);
      // next step's operands: level rows first, then this step's -M^T for the
      // crossing, then the copies
      if (member && c - 1 > cp) fetch_level(c - 1);
      if (c - 1 > G * grp) fetch_mt(c - 1);
      if (c - 1 >= bottom) fetch_copy(c - 1);
    }
    if (active && !vanish) {
      const E *kl = levels + lev_at(win, bh, c, cp, D) + (size_t)32 * kh * D;   // Khat[c] rows
      f32x16 s[2], dp[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        zero16(s[qt]);
        zero16(dp[qt]);
        if constexpr (BF) {
          const E *qa_r = Qs + (32 * qt + col) * L::PQ + KPL * g;
          const E *do_r = Os + (32 * qt + col) * L::PQ + KPL * g;
#pragma unroll
          for (int ks = 0; ks < KSD; ++ks) {
            s[qt] = MM<E>::mma(MM<E>::ld(qa_r + 2 * KPL * ks, 1), kcur[ks], s[qt]);
            dp[qt] = MM<E>::mma(MM<E>::ld(do_r + 2 * KPL * ks, 1), vfr[ks], dp[qt]);
          }
        } else {
          mma_tile<E, D>(s[qt], Qs + 32 * qt * L::PQ, L::PQ, 1, kl, D, 1, lane);
          mma_tile<E, D>(dp[qt], Os + 32 * qt * L::PQ, L::PQ, 1, v + krow * D, D, 1, lane);
        }
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
        st_tile(PT + 32 * qt, 1, L::PP, s[qt], lane);   // P^T[key][q]
        st_tile(GT + 32 * qt, 1, L::PP, dp[qt], lane);  // g^T[key][q]
      }
      wave_sync();
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
    }
    if (active && c == cp + 1) {   // chunk c' is done: dKb = Gamma
#pragma unroll
      for (int t = 0; t < D / 32; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dkb[(krow + acc_row(r, g)) * D + 32 * t + col] = gam[t][r];
    }
    const int mch = c - 1;
    if (!(mch > G * grp)) continue;   // no chunk of the group crosses m = c-1
    // ---- crossing of chunk m = c-1 by the group's chunks c' < m
    const bool crosses = member && cp < mch;
    wave_sync();   // this wave's reads of P^T / g^T are done before GR overwrites them
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      f32x16 z = gam[t];
      if (!crosses) zero16(z);
      if constexpr (BF) {
        st_tile(gx + 32 * t * L::PGT + kbase, 1, L::PGT, z, lane);   // Gamma^T [D][KG]
        st_tile(GR + 32 * t, L::PGN, 1, z, lane);                    // round(Gamma) rows
      } else {
        st_tile(gx + kbase * L::PGN + 32 * t, L::PGN, 1, z, lane);   // Gamma rows [KG][D]
      }
    }
    __syncthreads();
    if constexpr (BF) {   // every wave is past its products: the staging area is free
      // Khat[m]^T [D][KG] from this wave's next-level rows (lane = key), and -M_m^T
#pragma unroll
      for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
        for (int t = 0; t < KPL; ++t)
          KX[(KPL * g + 2 * KPL * ks + t) * L::PGT + kbase + col] = crosses ? kfr[ks][t] : (E)0.f;
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        const int vi = tid + NTH * i, r = vi / (D / 8), c8 = 8 * (vi % (D / 8));
        *reinterpret_cast<bf16x8 *>(MT + r * PMT + c8) = mreg[i];
      }
      __syncthreads();
    }
    // dM_m partial of the group: -sum_keys Gamma(key, d) Khat[m](key, d'), over
    // the chunks c' < m of the group
    {
      constexpr int TILES = (D / 32) * (D / 32);
      const int nch = mch - G * grp < G ? mch - G * grp : G;
      float *dst = dmpart + (((size_t)bh * slots + mch - (win.lo - 1)) * NG + grp) * D * D;
      const size_t lm = lev_at(win, bh, mch, G * grp, D);   // chunk blocks are consecutive
      for (int tI = wv; tI < TILES; tI += NW) {
        const int ta = tI / (D / 32), tb = tI % (D / 32);
        f32x16 acc;
        zero16(acc);
        for (int j = 0; j < nch; ++j) {
          if constexpr (BF) {
            mma_tile<E, C>(acc, gx + 32 * ta * L::PGT + 64 * j, L::PGT, 1,
                           KX + 32 * tb * L::PGT + 64 * j, L::PGT, 1, lane);
          } else {
            const E *kt = levt + lm + (size_t)j * C * D + (size_t)32 * tb * C;   // [d'][64 keys]
            mma_tile<E, C>(acc, gx + 64 * j * L::PGN + 32 * ta, 1, L::PGN, kt, C, 1, lane);
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dst[(size_t)(32 * ta + acc_row(r, g)) * D + 32 * tb + col] = -acc[r];
      }
    }
    if (crosses) {   // Gamma <- Gamma + round(Gamma) (-M_m): B(d', d) = -M_m[d][d'] = (-M^T)[d'][d]
      const E *nb = nmt + ((size_t)bh * N + mch) * D * D;
#pragma unroll
      for (int t = 0; t < D / 32; ++t) {
        if constexpr (BF)
          mma_tile<E, D>(gam[t], GR, L::PGN, 1, MT + 32 * t * PMT, PMT, 1, lane);
        else
          mma_tile<E, D>(gam[t], gx + kbase * L::PGN, L::PGN, 1, nb + 32 * t * D, D, 1, lane);
      }
    }
  }
  if (!member) return;
  if (cp == N - 1) {   // no later query chunk: dKb = 0
    if (win.hi == N)
      for (int e = lane; e < 32 * D; e += 64) dkb[krow * D + e] = 0.f;
    return;
  }
  if (!has_work) return;
  // this window's share of dV and of the gate's column sums; Gamma for the
  // window below when the walk goes on there
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) dv[(krow + acc_row(r, g)) * D + 32 * t + col] += dva[t][r];
  if (FOX) {
    colsum += __shfl_xor(colsum, 32);
    if (g == 0) dlam[krow + col] -= colsum;
  }
  if (bottom > cp + 1)
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) gstate[(krow + acc_row(r, g)) * D + 32 * t + col] = gam[t][r];
}

// ------------------------------------------------------------------ dk, bf16, d = 64

// Same walk as dk_kernel for bf16 inputs and d = 64, G = 4 key chunks per
// block (8 waves).  The query-side operands of step c (Qa and dO as rows and
// in fragment order, -M_{c-1}^T in fragment order, per-query statistics: 43
// KiB of per-chunk images) are copied straight into one of two LDS buffers one
// step ahead (global_load_lds); V and the level rows Khat[c]_{c'} are
// matrix-core B operands held in registers, the latter loaded one step ahead.
// dV, Gamma and the S, dP tiles keep one key per lane (dV, Gamma transposed:
// d x keys), so the products that contract over queries (dV^T += dO^T P,
// Gamma^T += Qa^T g) and the transition Gamma^T <- Gamma^T + (-M^T)
// round(Gamma^T) take their B operands straight from the accumulators (the
// contraction index permuted as frag_row, matched by the fragment-order
// images).
template <bool FOX>
__global__ __launch_bounds__(512) void dk64_kernel(
    const __bf16 *__restrict__ qimg, const __bf16 *__restrict__ oimg,
    const __bf16 *__restrict__ mimg, const float4 *__restrict__ qstat,
    const float *__restrict__ lam, const __bf16 *__restrict__ levels,
    const __bf16 *__restrict__ levt, const __bf16 *__restrict__ v, float scale,
    float *__restrict__ dkb, float *__restrict__ dv, float *__restrict__ dlam,
    float *__restrict__ dmpart, int T, int BH, Win win, int slots, float *__restrict__ gstate) {
  using E = __bf16;
  constexpr int D = 64, G = 4, NW = 8, P = kImgPitch, KG = 64 * G, PGT = KG + 8;
  constexpr int QB = kQImgElems * 2, MB = kMImgElems * 2, SB = 64 * 16;   // bytes
  constexpr int BUF = 2 * QB + MB + SB;                                   // 43 KiB
  constexpr int NCOPY = BUF / 1024;
  static_assert(BUF % 1024 == 0, "whole 1 KiB copies");
  __shared__ __attribute__((aligned(16))) unsigned char sbuf[2 * BUF];
  __shared__ __attribute__((aligned(16))) E gx[D * PGT];   // Gamma^T [d][KG] at crossings
  __shared__ __attribute__((aligned(16))) E kx[D * PGT];   // Khat[m]^T [d][KG] at crossings
  const int N = T / C, NG = (N + G - 1) / G;
  const int grp = blockIdx.x / BH, bh = blockIdx.x % BH;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, col = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar: uniform branches
  const int kh = wv & 1, cp = G * grp + (wv >> 1);
  const size_t head = (size_t)bh * T;
  const size_t krow = head + (size_t)cp * C + 32 * kh;
  const bool member = cp < N;
  const int kbase = 64 * (wv >> 1) + 32 * kh;
  const int c_low = G * grp + 1;
  // this window's steps: query chunks top down to bottom
  const int top = win.hi - 1, bottom = max(win.lo, c_low);
  const bool has_work = member && cp < top;

  auto stage = [&](int c, int b) {
    const size_t ch = (size_t)bh * N + c;
    const unsigned char *q = reinterpret_cast<const unsigned char *>(qimg + ch * kQImgElems);
    const unsigned char *o = reinterpret_cast<const unsigned char *>(oimg + ch * kQImgElems);
    const unsigned char *mm = reinterpret_cast<const unsigned char *>(mimg + (ch - 1) * kMImgElems);
    const unsigned char *st = reinterpret_cast<const unsigned char *>(qstat + ch * C);
    for (int j = wv; j < NCOPY; j += NW) {
      const unsigned char *src = j < QB / 1024 ? q + j * 1024
                                 : j < 2 * QB / 1024 ? o + (j - QB / 1024) * 1024
                                 : j < (2 * QB + MB) / 1024 ? mm + (j - 2 * QB / 1024) * 1024
                                                            : st;
      copy16_to_lds(src + lane * 16, lds_addr(sbuf + b * BUF + j * 1024));
    }
  };
  auto load_rows = [&](bf16x8 (&f)[D / 16], const E *rows) {   // B operand: this wave's 32 rows
    const E *p = rows + (size_t)col * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) f[ks] = *reinterpret_cast<const bf16x8 *>(p + 16 * ks);
  };

  f32x16 gamT[D / 32], dvT[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    zero16(gamT[t]);
    zero16(dvT[t]);
  }
  if (has_work && win.hi < N)   // Gamma^T as the window above left it (lane = key)
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 x = *reinterpret_cast<const float4 *>(gstate + (krow + col) * D + 32 * t + 8 * q4 + 4 * g);
        gamT[t][4 * q4] = x.x;
        gamT[t][4 * q4 + 1] = x.y;
        gamT[t][4 * q4 + 2] = x.z;
        gamT[t][4 * q4 + 3] = x.w;
      }
  float colsum = 0.f;
  const float my_lam = (FOX && member) ? lam[krow + col] : 0.f;
  bf16x8 vf[D / 16], kf[D / 16];
  if (member) load_rows(vf, v + krow * D);
  if (top >= bottom) {
    stage(top, top & 1);
    if (member && top > cp) load_rows(kf, levels + lev_at(win, bh, top, cp, D) + (size_t)32 * kh * D);
  }
  // one step: query chunk c with level fragments kf; the next step's go to kn
  auto step = [&](int c, bf16x8 (&kf)[D / 16], bf16x8 (&kn)[D / 16]) {
    const bool active = member && c > cp;
    const int b = c & 1;
    wait_vmcnt<0>();
    lds_barrier();
    if (c - 1 >= bottom) stage(c - 1, b ^ 1);
    // the next level's rows (the next step's S operand, and Khat[c-1] at the
    // crossing below, also after the window's last step: level lo - 1 is in
    // the window); every step loads (a valid block when there is no next
    // level), so the sequence of loads is the same in every step
    const bool next_active = member && c - 1 > cp;
    load_rows(kn, levels + (next_active ? lev_at(win, bh, c - 1, cp, D) : (size_t)bh * win.head) +
                      (size_t)32 * kh * D);
    const E *Qs = reinterpret_cast<const E *>(sbuf + b * BUF), *QF = Qs + 64 * P;
    const E *Os = reinterpret_cast<const E *>(sbuf + b * BUF + QB), *OF = Os + 64 * P;
    const E *Ms = reinterpret_cast<const E *>(sbuf + b * BUF + 2 * QB);
    const float4 *qs = reinterpret_cast<const float4 *>(sbuf + b * BUF + 2 * QB + MB);
    if (active) {
      f32x16 s[2], dp[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        zero16(s[qt]);
        zero16(dp[qt]);
        const E *qa = Qs + (32 * qt + col) * P + 8 * g, *oa = Os + (32 * qt + col) * P + 8 * g;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          s[qt] = MM<E>::mma(*reinterpret_cast<const bf16x8 *>(qa + 16 * ks), kf[ks], s[qt]);
          dp[qt] = MM<E>::mma(*reinterpret_cast<const bf16x8 *>(oa + 16 * ks), vf[ks], dp[qt]);
        }
      }
      bf16x8 pf[4], gf[4];   // P and g as B operands: k-step s covers queries frag_row(s, g, .)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float4 st = qs[32 * qt + acc_row(r, g)];
          const float p = __expf(scale * s[qt][r] + st.w - my_lam - st.x);
          const float ds = p * (dp[qt][r] - st.y + st.z);
          colsum += ds;
          pf[2 * qt + r / 8][r % 8] = (E)p;
          gf[2 * qt + r / 8][r % 8] = (E)(scale * ds);
        }
      }
      // dV^T(d, key) += sum_q dO(q, d) P(q, key);  Gamma^T(d, key) += sum_q Qa(q, d) g(q, key)
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
        for (int sI = 0; sI < 4; ++sI) {
          dvT[mt] = MM<E>::mma(*reinterpret_cast<const bf16x8 *>(OF + (mt * 4 + sI) * 512 + lane * 8),
                               pf[sI], dvT[mt]);
          gamT[mt] = MM<E>::mma(*reinterpret_cast<const bf16x8 *>(QF + (mt * 4 + sI) * 512 + lane * 8),
                                gf[sI], gamT[mt]);
        }
      if (c == cp + 1) {   // chunk c' is done: dKb = Gamma
#pragma unroll
        for (int t = 0; t < D / 32; ++t)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4)
            *reinterpret_cast<float4 *>(dkb + (krow + col) * D + 32 * t + 8 * q4 + 4 * g) =
                make_float4(gamT[t][4 * q4], gamT[t][4 * q4 + 1], gamT[t][4 * q4 + 2],
                            gamT[t][4 * q4 + 3]);
      }
    }
    const int mch = c - 1;
    if (!(mch > G * grp)) return;
    // ---- crossing of chunk m = c-1 by the group's chunks c' < m
    const bool crosses = member && cp < mch;
    // Khat[m]^T [d][KG] from the next step's level fragments (lane = key)
    E *Kx = kx;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
      f32x16 z = gamT[t];
      if (!crosses) zero16(z);
      st_tile(gx + 32 * t * PGT + kbase, PGT, 1, z, lane);   // Gamma^T [d][KG]
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
      for (int t = 0; t < 8; ++t)
        Kx[(8 * g + 16 * ks + t) * PGT + kbase + col] = crosses ? kn[ks][t] : (E)0.f;
    lds_barrier();
    {
      constexpr int TILES = (D / 32) * (D / 32);
      const int nch = mch - G * grp < G ? mch - G * grp : G;
      float *dst = dmpart + (((size_t)bh * slots + mch - (win.lo - 1)) * NG + grp) * D * D;
      for (int tI = wv; tI < TILES; tI += NW) {
        const int ta = tI / (D / 32), tb = tI % (D / 32);
        f32x16 acc;
        zero16(acc);
        for (int j = 0; j < nch; ++j)
          mma_tile<E, C>(acc, gx + 32 * ta * PGT + 64 * j, PGT, 1, Kx + 32 * tb * PGT + 64 * j,
                         PGT, 1, lane);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          dst[(size_t)(32 * ta + acc_row(r, g)) * D + 32 * tb + col] = -acc[r];
      }
    }
    if (crosses) {   // Gamma^T <- Gamma^T + (-M_m^T) round(Gamma^T)
      bf16x8 bfr[D / 16];
#pragma unroll
      for (int sI = 0; sI < D / 16; ++sI)
#pragma unroll
        for (int t = 0; t < 8; ++t) bfr[sI][t] = (E)gamT[sI / 2][8 * (sI % 2) + t];
#pragma unroll
      for (int mt = 0; mt < D / 32; ++mt)
#pragma unroll
        for (int sI = 0; sI < D / 16; ++sI)
          gamT[mt] = MM<E>::mma(
              *reinterpret_cast<const bf16x8 *>(Ms + (mt * (D / 16) + sI) * 512 + lane * 8),
              bfr[sI], gamT[mt]);
    }
  };
  bf16x8 kf2[D / 16];
  for (int c = top; c >= bottom; c -= 2) {
    step(c, kf, kf2);
    if (c - 1 < bottom) break;
    step(c - 1, kf2, kf);
  }
  if (!member) return;
  if (cp == N - 1) {   // no later query chunk: dKb = 0
    if (win.hi == N)
      for (int e = lane; e < 32 * D; e += 64) dkb[krow * D + e] = 0.f;
    return;
  }
  if (!has_work) return;
  if (bottom > cp + 1)   // Gamma^T for the window below
#pragma unroll
    for (int t = 0; t < D / 32; ++t)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<float4 *>(gstate + (krow + col) * D + 32 * t + 8 * q4 + 4 * g) =
            make_float4(gamT[t][4 * q4], gamT[t][4 * q4 + 1], gamT[t][4 * q4 + 2], gamT[t][4 * q4 + 3]);
#pragma unroll
  for (int t = 0; t < D / 32; ++t)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {   // dV^T tile: this lane's key row, 4 consecutive d
      float4 *p4 = reinterpret_cast<float4 *>(dv + (krow + col) * D + 32 * t + 8 * q4 + 4 * g);
      float4 x = *p4;
      x.x += dvT[t][4 * q4];
      x.y += dvT[t][4 * q4 + 1];
      x.z += dvT[t][4 * q4 + 2];
      x.w += dvT[t][4 * q4 + 3];
      *p4 = x;
    }
  if (FOX) {
    colsum += __shfl_xor(colsum, 32);
    if (g == 0) dlam[krow + col] -= colsum;
  }
}

// dM_m = sum over the groups that cross m (m in [1, N-2]); 0 otherwise, for
// the nm chunks m = m0 .. m0 + nm - 1 of one window (partial slot m - m0).
// One block per (bh, m) and slice of 1024 elements (DD / 1024 blocks per
// matrix), four consecutive elements per thread; the partials are summed in
// group order, eight loads in flight.
template <int G>
__global__ __launch_bounds__(256) void dm_reduce_kernel(const float4 *__restrict__ dmpart,
                                                        float4 *__restrict__ dm, int N, int DD,
                                                        int XB, int m0, int nm, int slots,
                                                        const int *__restrict__ zhi) {
  constexpr int U = 8;
  const int NG = (N + G - 1) / G, DD4 = DD / 4;
  const int bmi = blockIdx.x / XB;   // bh * nm + (m - m0)
  const int bh = bmi / nm, mi = bmi % nm, mch = m0 + mi;
  const int e = (blockIdx.x % XB) * 256 + threadIdx.x;
  const int ng = (mch >= 1 && mch <= N - 2) ? (mch + G - 1) / G : 0;
  const size_t bm = (size_t)bh * N + mch;
  const float4 *src = dmpart + ((size_t)bh * slots + mi) * NG * DD4 + e;
  // with the whole-step skip, group gi wrote no partial for m >= zhi[gi]:
  // those are zero (adding them changes no bit of the sum)
  const int *zh = zhi ? zhi + (size_t)bh * NG : nullptr;
  auto part = [&](int gi) __attribute__((always_inline)) {
    return !zh || mch < zh[gi] ? src[(size_t)gi * DD4] : make_float4(0.f, 0.f, 0.f, 0.f);
  };
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  int gi = 0;
  for (; gi + U <= ng; gi += U) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = part(gi + u);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      acc.x += v[u].x;
      acc.y += v[u].y;
      acc.z += v[u].z;
      acc.w += v[u].w;
    }
  }
  for (; gi < ng; ++gi) {
    const float4 v = part(gi);
    acc.x += v.x;
    acc.y += v.y;
    acc.z += v.z;
    acc.w += v.w;
  }
  dm[bm * DD4 + e] = acc;
}

template <typename E, int D>
constexpr int group_of() {
  return std::is_same<E, __bf16>::value ? (D == 64 ? 4 : 2) : (D == 64 ? 2 : 1);
}

}  // namespace

BwdPlan bwd_plan(int T, int window) {
  BwdPlan p{};
  p.N = T / C;
  const int nq = p.N - 1 > 1 ? p.N - 1 : 1;   // query chunks with earlier keys
  p.W = window > 0 ? (window < nq ? window : nq) : (nq <= 2 * kBwdWindowMin ? nq : kBwdWindowMin);
  p.nwin = (nq + p.W - 1) / p.W;
  p.win_blocks = 0;
  p.slots = 0;
  for (int w = 0; w < p.nwin; ++w) {
    const int lo = 1 + w * p.W, hi = p.N < lo + p.W ? p.N : lo + p.W;
    const size_t blk = (size_t)hi * (hi - 1) / 2 - (size_t)(lo - 1) * (lo - 2) / 2;
    p.win_blocks = blk > p.win_blocks ? blk : p.win_blocks;
    p.slots = hi - lo + 1 > p.slots ? hi - lo + 1 : p.slots;
  }
  p.ckpt_blocks = p.nwin > 2 ? (size_t)p.W * (p.nwin - 1) * (p.nwin - 2) / 2 : 0;
  return p;
}

size_t bwd_dmpart_floats(int dtype, int BH, int T, int D, int window) {
  const int N = T / C;
  const int G = dtype == 1 ? (D == 64 ? 4 : 2) : (D == 64 ? 2 : 1);
  return (size_t)BH * bwd_plan(T, window).slots * ((N + G - 1) / G) * D * D;
}

template <typename E, int D, bool FOX>
static hipError_t sweep_t(const SweepArgs &a, hipStream_t s) {
  const int BH = a.BH, T = a.T, N = T / C;
  constexpr int G = group_of<E, D>();
  constexpr bool BF = std::is_same<E, __bf16>::value;
  const BwdPlan P = bwd_plan(T, a.window);
  const int NG = (N + G - 1) / G;
  E *lev = static_cast<E *>(a.levels), *levt = static_cast<E *>(a.levt);
  const E *qae = (const E *)a.qae, *dout = (const E *)a.dout, *v = (const E *)a.v;
  const Ckpt ck{a.ckpt, P.ckpt_blocks * C * D, P.W};
  // exact forget-gate skip: bf16 at d = 128 (dq_kernel's key lists bound N)
  const int skip = FOX && BF && D == 128 && a.skip && N <= kBwdSkipList ? 1 : 0;
  float *kn2 = skip ? a.kn2 : nullptr;
  if (skip)
    hipLaunchKernelGGL((bwd_skip_stats_kernel<E, D>), dim3(BH * N), dim3(64), 0, s, qae, a.lam,
                       a.lse, const_cast<float2 *>(a.qagg), const_cast<float *>(a.kmin),
                       a.zhi + (size_t)BH * N, T);
  constexpr int XB = D * D / 1024;
  static_assert(D * D % 1024 == 0, "whole 1024-element slices");
  // windows of query chunks, the last first (Gamma flows down); the last
  // window's level pass is the whole walk, which also leaves the checkpoints
  for (int w = P.nwin - 1; w >= 0; --w) {
    const int lo = 1 + w * P.W, hi = N < lo + P.W ? N : lo + P.W;
    const Win win{lo, hi, lev_off(lo - 1, 0, D), P.win_blocks * C * D};
    const int first = w == P.nwin - 1;
    if (hi - 1 > 0) {   // levels [lo - 1, hi) of the key chunks c' < hi - 1
      if constexpr (BF)
        hipLaunchKernelGGL((levels_shared_kernel<D>), dim3(BH * ((hi - 1 + 3) / 4)), dim3(512), 0,
                           s, a.kb, (const E *)a.nm, lev, levt, T, BH, win, ck, first, kn2,
                           a.zhi + (size_t)BH * N);
      else
        hipLaunchKernelGGL((levels_f32_kernel<D>), dim3(BH * (hi - 1)), dim3(128), 0, s, a.kb,
                           (const float *)a.nm, lev, levt, T, BH, win, ck, first);
    }
    const int nq = hi - (w == 0 ? 0 : lo);   // query chunks of the window (chunk 0 in the first)
    if constexpr (BF && D == 64)
      hipLaunchKernelGGL((dq64_kernel<FOX>), dim3(BH * nq), dim3(256), 0, s, qae, dout, a.lse,
                         a.dlse, a.dvec, a.lam, lev, v, a.scale, a.dqa, a.dlam, T, BH, win);
    else
      hipLaunchKernelGGL((dq_kernel<E, D, FOX>), dim3(BH * nq), dim3(256), 0, s, qae, dout, a.lse,
                         a.dlse, a.dvec, a.lam, lev, levt, v, a.scale, a.dqa, a.dlam, T, BH, win,
                         kn2, a.qagg, a.kmin, skip);
    // groups with a step in the window (G grp + 1 <= hi - 1); the last window
    // also runs the rest, which store dKb = 0 for chunk N - 1
    const int ngw = hi == N ? NG : (hi - 2) / G + 1 < NG ? (hi - 2) / G + 1 : NG;
    if constexpr (BF && D == 64) {
      static_assert(G == 4, "dk64_kernel takes groups of 4 key chunks");
      hipLaunchKernelGGL((dk64_kernel<FOX>), dim3(BH * ngw), dim3(512), 0, s, (const E *)a.qimg,
                         (const E *)a.oimg, (const E *)a.mimg, (const float4 *)a.qst, a.lam, lev,
                         levt, v, a.scale, a.dkb, a.dv, a.dlam, a.dmpart, T, BH, win, P.slots,
                         a.gstate);
    } else {
      hipLaunchKernelGGL((dk_kernel<E, D, G, FOX>), dim3(BH * ngw), dim3(128 * G), 0, s, qae,
                         (const E *)a.qat, dout, (const E *)a.dot, a.lse, a.dlse, a.dvec, a.lam,
                         lev, levt, v, (const E *)a.nmt, a.scale, a.dkb, a.dv, a.dlam, a.dmpart, T,
                         BH, win, P.slots, a.gstate, kn2, a.qagg, a.kmin, skip, a.zhi);
    }
    // dM_m for m in [lo - 1, hi - 1), and m = N - 1 with the last window
    const int nm = hi - lo + (hi == N ? 1 : 0);
    hipLaunchKernelGGL((dm_reduce_kernel<G>), dim3(BH * nm * XB), dim3(256), 0, s,
                       (const float4 *)a.dmpart, (float4 *)a.dm, N, D * D, XB, lo - 1, nm,
                       P.slots, skip ? a.zhi : nullptr);
  }
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
