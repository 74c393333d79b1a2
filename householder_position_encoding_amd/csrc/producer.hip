// producer.hip -- the w / beta producer: the inputs of the transitions from
// the hidden states (bf16).
//
// From the PaTH slides, frame "PaTH inserts a learned transformation along
// every path" (beta_t = 2 sigmoid(u^T x_t + b), ||w_t||_2 = 1, w_t from a
// low-rank projection, a convolution of width 3 and an L2 normalisation), and
// the discussion page's section "Model Architecture Details" (the
// normalisation per head, the projection low-rank):
//
//     z_t    = Wu (Wd x_t)                              Wd: [R][Dm], Wu: [H d][R]
//     z'_t   = cw[., 0] z_{t-2} + cw[., 1] z_{t-1} + cw[., 2] z_t   (per channel)
//     w_t[h] = z'_t[h d .. h d + d) / || . ||_2         (0 for a zero vector)
//     beta_t[h] = 2 sigmoid(u[h] . x_t + ub[h])        u: [H][Dm]
//
// One block of four waves per (batch, 62 tokens).  Its 64-row tile starts two
// tokens early, so that the convolution's earlier tokens are in the tile (2
// of 64 rows computed twice).  Phase 1: the tile of x times [Wd; u]^T on the
// bf16 matrix cores (x, Wd and u are bf16 inputs, exact; float32
// accumulation): the first R columns are y = Wd x, kept in LDS as bf16 hi/lo
// planes for the second product; the next H columns are beta's logits,
// finished straight from the accumulators.  Phase 2, one head at a time:
// z = y Wu_h^T (hi and lo parts of y against the exact bf16 Wu), the head's
// tile through LDS, then per token the three-tap convolution, the norm over
// the head's d channels (d / 16 threads per token) and the bf16 store of w.
// Both phases keep two register sets of operands in flight (chunks k + 1 and
// k + 2, heads h + 1 and h + 2), and every thread issues the same memory
// operations in every step, so that a wait for one set never waits for the
// other or for stores issued before it.
#include <hip/hip_runtime.h>

#include "path_attn_internal.h"
#include "tile_fp32.h"

namespace pathattn {
namespace {

constexpr int kTileRows = 64, kTileOut = kTileRows - 2;   // two halo tokens

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 ld8(const __bf16 *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

__device__ __forceinline__ f32x16 mma16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D, int RMAX>
__global__ __launch_bounds__(256, D == 128 && RMAX == 128 ? 1 : 2) void wbeta_kernel(
    const __bf16 *__restrict__ x, const __bf16 *__restrict__ wd, const __bf16 *__restrict__ wu,
    const float *__restrict__ cw, const __bf16 *__restrict__ u, const float *__restrict__ ub,
    __bf16 *__restrict__ w, float *__restrict__ beta, int T, int Dm, int R, int H, int ntile) {
  constexpr int PR = RMAX + 8, PZ = D + 4;   // PZ: 16-byte rows for the z reads
  constexpr int KC = 64, PK = KC + 8, CG = 128;   // phase 1: k chunk, output column group
  // LDS: the y planes (hi, then lo) [64][PR], kept from phase 1 to phase 2;
  // then phase 1's staged chunk of x [64][PK] and of [Wd; u] [CG][PK], whose
  // bytes phase 2 reuses for one head's z tile [64][PZ], its Wu rows [D][PR]
  // and the taps of two heads [2][D][3]
  constexpr int YP = 2 * kTileRows * PR * 2;
  constexpr int ST1 = (kTileRows + CG) * PK * 2;
  constexpr int ST2 = kTileRows * PZ * 4 + D * PR * 2 + 2 * D * 3 * 4;
  __shared__ __attribute__((aligned(16))) unsigned char smem[YP + (ST1 > ST2 ? ST1 : ST2)];
  __bf16 *yp = reinterpret_cast<__bf16 *>(smem);
  __bf16 *xs = reinterpret_cast<__bf16 *>(smem + YP), *ws = xs + kTileRows * PK;
  float *zs = reinterpret_cast<float *>(smem + YP);
  __bf16 *wub = reinterpret_cast<__bf16 *>(smem + YP + kTileRows * PZ * 4);
  float *cwl = reinterpret_cast<float *>(smem + YP + kTileRows * PZ * 4 + D * PR * 2);
  const int b = blockIdx.x / ntile, tile = blockIdx.x % ntile;
  const int t0 = tile * kTileOut - 2;   // token of tile row 0
  int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6, g = lane >> 5, n = lane & 31;
  // the head's Wu rows and taps: R / 8 16-byte pieces per row, 3 D taps
  const int wpieces = D * (R / 8);
  constexpr int WPT = D * (RMAX / 8) / 256, CPT = (3 * D + 255) / 256;   // per thread, at most
  // Two register sets of a head's operands: the head after next is fetched
  // while this one is finished.  Every thread issues the same loads (indices
  // clamped, the surplus unused), so that waiting for them never waits for
  // stores issued before them on another control path.
  bf16x8 wpa[WPT], wpb[WPT];
  float cpa[CPT], cpb[CPT];
  auto fetch_head = [&](int h, bf16x8 (&wp)[WPT], float (&cp)[CPT]) __attribute__((always_inline)) {
    h = min(h, H - 1);
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const int pi = min(tid + 256 * j, wpieces - 1);
      const int row = pi / (R / 8), c8 = 8 * (pi % (R / 8));
      wp[j] = ld8(wu + ((size_t)h * D + row) * R + c8);
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) cp[j] = cw[(size_t)h * D * 3 + min(tid + 256 * j, 3 * D - 1)];
  };
  auto put_head = [&](int h, const bf16x8 (&wp)[WPT], const float (&cp)[CPT]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const int pi = tid + 256 * j;
      if (pi < wpieces) {
        const int row = pi / (R / 8), c8 = 8 * (pi % (R / 8));
        *reinterpret_cast<bf16x8 *>(wub + row * PR + c8) = wp[j];
      }
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int e = tid + 256 * j;
      if (e < 3 * D) cwl[(h & 1) * 3 * D + e] = cp[j];
    }
  };

  // ---- phase 1: [y | logits] = X [Wd; u]^T, 64 x NC (NC = R + H, rounded up
  // to 32), in groups of up to CG output columns; each group walks Dm in
  // chunks of KC staged in LDS (16-byte pieces, whole rows), the next chunk
  // loaded into registers while the current one is multiplied
  const int NC = (R + H + 31) / 32 * 32;
  constexpr int XPT = kTileRows * (KC / 8) / 256, WPC = CG * (KC / 8) / 256;   // pieces per thread
  for (int cg = 0; cg < NC; cg += CG) {
    const int ncg = NC - cg < CG ? NC - cg : CG, ntl = 2 * (ncg / 32);
    // two register sets of staged chunks: chunk k + 2 is loaded while chunk
    // k is multiplied; the loads of a chunk past Dm re-read the last one
    // (unused), so every step issues the same memory operations
    bf16x8 xa[XPT], wa[WPC], xb[XPT], wb[WPC];
    // Pieces outside the matrices (rows of x before token 0 or past T,
    // columns past R + H) are loaded from a valid row and replaced by zeros
    // when staged: zeroing the loaded register itself would make the wave
    // wait for the load right after issuing it.
    bool xok[XPT], wok[WPC];
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int tok = t0 + (tid + 256 * j) / (KC / 8);
      xok[j] = tok >= 0 && tok < T;
    }
#pragma unroll
    for (int j = 0; j < WPC; ++j) {
      const int row = (tid + 256 * j) / (KC / 8);
      wok[j] = cg + row < R + H && row < ncg;
    }
    auto load_chunk = [&](int k0, bf16x8 (&xr)[XPT], bf16x8 (&wr)[WPC]) __attribute__((always_inline)) {
      k0 = min(k0, Dm - KC);
#pragma unroll
      for (int j = 0; j < XPT; ++j) {
        const int pi = tid + 256 * j, row = pi / (KC / 8), c8 = 8 * (pi % (KC / 8));
        const int tok = min(max(t0 + row, 0), T - 1);
        xr[j] = ld8(x + ((size_t)b * T + tok) * Dm + k0 + c8);
      }
#pragma unroll
      for (int j = 0; j < WPC; ++j) {
        const int pi = tid + 256 * j, row = pi / (KC / 8), c8 = 8 * (pi % (KC / 8));
        const int col = min(cg + row, R + H - 1);   // output column: Wd row or u row
        const __bf16 *src = col < R ? wd + (size_t)col * Dm : u + (size_t)(col - R) * Dm;
        wr[j] = ld8(src + k0 + c8);
      }
    };
    f32x16 acc[2];
    zero16(acc[0]);
    zero16(acc[1]);
    // one chunk: stage the set, reload it with chunk k0 + 2 KC, multiply
    // (the product only when chunk k0 exists)
    auto chunk_step = [&](int k0, bf16x8 (&xr)[XPT], bf16x8 (&wr)[WPC]) __attribute__((always_inline)) {
      __syncthreads();   // the previous chunk's fragments are read
#pragma unroll
      for (int j = 0; j < XPT; ++j) {
        const int pi = tid + 256 * j;
        *reinterpret_cast<bf16x8 *>(xs + (pi / (KC / 8)) * PK + 8 * (pi % (KC / 8))) = xok[j] ? xr[j] : bf16x8{};
      }
#pragma unroll
      for (int j = 0; j < WPC; ++j) {
        const int pi = tid + 256 * j;
        *reinterpret_cast<bf16x8 *>(ws + (pi / (KC / 8)) * PK + 8 * (pi % (KC / 8))) = wok[j] ? wr[j] : bf16x8{};
      }
      __syncthreads();
      load_chunk(k0 + 2 * KC, xr, wr);
      if (k0 < Dm) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int ti = wv + 4 * j;
          if (ti < ntl) {
            const int mh = ti & 1, nb = ti >> 1;
            const __bf16 *pa = xs + (32 * mh + n) * PK + 8 * g, *pb = ws + (32 * nb + n) * PK + 8 * g;
#pragma unroll
            for (int s2 = 0; s2 < KC / 16; ++s2) acc[j] = mma16(ld8(pa + 16 * s2), ld8(pb + 16 * s2), acc[j]);
          }
        }
      }
    };
    load_chunk(0, xa, wa);
    // set a's loads ahead of set b's, as in every step, so that the wait for
    // set a at the top of the loop leaves set b in flight
    __builtin_amdgcn_sched_barrier(0);
    load_chunk(KC, xb, wb);
    for (int k0 = 0; k0 < Dm; k0 += 2 * KC) {
      chunk_step(k0, xa, wa);
      chunk_step(k0 + KC, xb, wb);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int ti = wv + 4 * j;
      if (ti >= ntl) continue;
      const int mh = ti & 1, col = cg + 32 * (ti >> 1) + n;
      if (col < R) {   // y: hi / lo planes, row = tile row, column = col
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * mh + acc_row(r, g);
          const __bf16 hi = (__bf16)acc[j][r];
          yp[row * PR + col] = hi;
          yp[kTileRows * PR + row * PR + col] = (__bf16)(acc[j][r] - (float)hi);
        }
      } else if (col < R + H) {   // beta of head col - R for the tile's output rows
        const int h = col - R;
        const float bh = ub[h];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * mh + acc_row(r, g), t = t0 + row;
          if (row >= 2 && t < T)
            beta[((size_t)b * H + h) * T + t] = 2.f / (1.f + __expf(-(acc[j][r] + bh)));
        }
      }
    }
  }
  fetch_head(0, wpa, cpa);
  fetch_head(1, wpb, cpb);
  __syncthreads();   // phase 1's staging bytes are free
  put_head(0, wpa, cpa);
  __syncthreads();

  // ---- phase 2, per head: z = y Wu_h^T, convolution, normalisation.  Head
  // h's Wu rows and taps are in LDS, head h + 1's in one register set (wn,
  // cn), and head h + 2's are fetched into the other (wf, cf) while head h
  // is finished.
  auto head_step = [&](int h, const bf16x8 (&wn)[WPT], const float (&cn)[CPT], bf16x8 (&wf)[WPT],
                       float (&cf)[CPT]) __attribute__((always_inline)) {
    // the thread index re-derived per head, so that the addresses below are
    // not computed for all heads up front and kept live
    asm volatile("" : "+v"(tid));
    for (int ti = wv; ti < 2 * (D / 32); ti += 4) {
      const int mh = ti & 1, nb = ti >> 1;
      const __bf16 *ya = yp + (32 * mh + n) * PR + 8 * g;
      const __bf16 *wb = wub + (32 * nb + n) * PR + 8 * g;
      f32x16 acc;
      zero16(acc);
#pragma unroll
      for (int s = 0; s < RMAX / 16; ++s)
        if (s < R / 16) {
          const bf16x8 bw = ld8(wb + 16 * s);
          acc = mma16(ld8(ya + 16 * s), bw, acc);                    // y hi
          acc = mma16(ld8(ya + kTileRows * PR + 16 * s), bw, acc);   // y lo
        }
#pragma unroll
      for (int r = 0; r < 16; ++r) zs[(32 * mh + acc_row(r, g)) * PZ + 32 * nb + n] = acc[r];
    }
    fetch_head(h + 2, wf, cf);   // clamped past the last head: the same loads every step
    __syncthreads();   // the head's z tile is complete, and every wave is done with wub
    // the convolution, the norm over the head's d channels and the store of
    // w: TPR threads per token (d = 64: four, 16 consecutive channels each;
    // d = 128: eight, channel runs 8 q .. and 64 + 8 q ..), so that a wave's
    // reads of a row of z fall in distinct banks (pitch D + 1)
    constexpr int TPR = D / 16, RPP = 256 / TPR;   // threads per token, rows per pass
    // w rows of this tile's output tokens t0 + 2 .. as a buffer range: every
    // thread stores; the halo rows (offset 2^31) and the rows past T (past
    // the range) are dropped by the range check, so the stores are
    // unconditional and the next head's loads can be waited for alone
    const int nout = min(kTileOut, T - (t0 + 2));
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
        w + (((size_t)b * H + h) * T + t0 + 2) * D, (short)0, nout * D * 2, 0x00020000);
#pragma unroll
    for (int pass = 0; pass < kTileRows / RPP; ++pass) {
      const int i = tid / TPR + RPP * pass, q = tid % TPR;
      // channel e of this thread (e < 16): d = 64, one run of 16 channels at
      // 16 q; d = 128, two runs of 8 at 8 q and 64 + 8 q
      constexpr int RUN = D == 64 ? 16 : 8;
      auto chan = [&](int e) __attribute__((always_inline)) {
        return D == 64 ? 16 * q + e : (e < 8 ? 8 * q + e : 64 + 8 * q + e - 8);
      };
      // rows i - 2, i - 1 clamped at the tile's first row: rows 0 and 1 are
      // the halo, whose w is not stored, so their values do not matter
      const float *z0r = zs + max(i - 2, 0) * PZ, *z1r = zs + max(i - 1, 0) * PZ, *z2r = zs + i * PZ;
      const float *tw = cwl + (h & 1) * 3 * D;
      float v[16];
      float ss = 0.f;
#pragma unroll
      for (int e4 = 0; e4 < 16; e4 += 4) {   // four channels: 16-byte reads of z and of the taps
        const int c4 = chan(e4);               // e4 .. e4 + 3 lie in one run
        const f32x4 a = *reinterpret_cast<const f32x4 *>(z0r + c4);
        const f32x4 bz = *reinterpret_cast<const f32x4 *>(z1r + c4);
        const f32x4 cz = *reinterpret_cast<const f32x4 *>(z2r + c4);
        f32x4 t[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) t[k] = *reinterpret_cast<const f32x4 *>(tw + 3 * c4 + 4 * k);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int o = 3 * e;   // taps of channel c4 + e: t[o / 4][o % 4] ..
          const float y = t[o / 4][o % 4] * a[e] + t[(o + 1) / 4][(o + 1) % 4] * bz[e] +
                          t[(o + 2) / 4][(o + 2) % 4] * cz[e];
          v[e4 + e] = y;
          ss = __builtin_fmaf(y, y, ss);
        }
      }
      static_assert(RUN % 4 == 0, "runs of whole 16-byte pieces");
#pragma unroll
      for (int o = 1; o < TPR; o <<= 1) ss += __shfl_xor(ss, o);   // the token's d channels
      {
        const float inv = ss > 0.f ? 1.f / __builtin_sqrtf(ss) : 0.f;
#pragma unroll
        for (int r8 = 0; r8 < 2; ++r8) {
          bf16x8 o;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = (__bf16)(v[8 * r8 + e] * inv);
          const int off = i >= 2 ? ((i - 2) * D + chan(8 * r8)) * 2 : (int)0x80000000;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), wrs, off, 0, 0);
        }
      }
    }
    if (h + 1 < H) put_head(h + 1, wn, cn);   // wub is free; the taps go to the other buffer
    __syncthreads();   // the z tile is read, and the next head's operands are in place
  };
  int h = 0;
  for (; h + 1 < H; h += 2) {   // pairs of heads: the register sets alternate
    head_step(h, wpb, cpb, wpa, cpa);
    head_step(h + 1, wpa, cpa, wpb, cpb);
  }
  if (h < H) head_step(h, wpb, cpb, wpa, cpa);
}

}  // namespace

int wbeta_tiles(int T) { return (T + kTileOut - 1) / kTileOut; }

hipError_t launch_wbeta(const WbetaArgs &a, hipStream_t s) {
  const int ntile = wbeta_tiles(a.T);
  const dim3 grid((unsigned)a.B * ntile), block(256);
  const auto *x = static_cast<const __bf16 *>(a.x), *wd = static_cast<const __bf16 *>(a.wd);
  const auto *wu = static_cast<const __bf16 *>(a.wu), *u = static_cast<const __bf16 *>(a.u);
  auto *w = static_cast<__bf16 *>(a.w);
  // the LDS is sized for R <= 64 or R <= 128
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, s, x, wd, wu, a.cw, u, a.ub, w, a.beta, a.T, a.Dm,
                       a.R, a.H, ntile);
  };
  if (a.d == 64) {
    if (a.R <= 64) go(wbeta_kernel<64, 64>);
    else go(wbeta_kernel<64, 128>);
  } else {
    if (a.R <= 64) go(wbeta_kernel<128, 64>);
    else go(wbeta_kernel<128, 128>);
  }
  return hipGetLastError();
}

}  // namespace pathattn
