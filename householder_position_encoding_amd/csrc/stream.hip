// stream.hip -- right-to-left streaming scan of PaTH attention on matrix cores.
//
// PaTH discussion slides for arXiv:2505.16381v2, frame "A right-to-left scan
// accumulates cross-block paths" (paper Sec. 3.3): for query chunk b, the
// diagonal block uses the local (UT) logits; then Q_work = <-Q_b and for
// c = b-1, ..., 0 the logits against key chunk c are Q_work ->K_c^T, fed to an
// online softmax and the value sum, after which the tile crosses chunk c's
// transition, Q_work <- Q_work F_c^T = Q_work (I - M_c).  Query chunks run in
// parallel; the attention matrix never leaves registers.
//
// Work decomposition.  A block takes NQC consecutive query chunks of one
// (batch, head), two waves per chunk, 32 queries per wave.  The block walks
// key chunks c from its top chunk down to 0; at step c every wave whose chunk
// lies above c does a cross step, the waves of chunk c do their diagonal
// block, the others wait.  All of them share one staged copy of key chunk c's
// operands (->K, V^T, -M^T: one contiguous block of the workspace), which is
// loaded straight into LDS (global_load_lds) one step ahead into the other of
// two buffers, so each step needs a single barrier.  Blocks are numbered so
// that the groups with the most key chunks start first, and all blocks of one
// (batch, head) fall on the same XCD (block index = group * B*H + head).
//
// Register layout (transposed orientation, see path_attn_internal.h): the
// running query tile Q_work^T (D x 32), the scores S^T (64 keys x 32) and the
// output O^T (D x 32) are float32 MFMA accumulators; lane l holds query l%32.
// Q_work^T and P^T become the B operands of the next MFMAs in registers, so
// the serial chain S = K Q, Q <- Q - M^T Q, O += V^T P never touches LDS.
// The running tile keeps a float32 master copy; the transform is applied as
// Q + (-M^T) round(Q), so the identity part of F_c is exact.
#include "path_attn_internal.h"

namespace pathattn {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

typedef __attribute__((address_space(3))) void *lds_ptr_t;
typedef __attribute__((address_space(1))) void *gbl_ptr_t;

template <typename E>
struct Mfma;

// bf16 inputs: v_mfma_f32_32x32x16_bf16, 8 contraction values per lane.
template <>
struct Mfma<__bf16> {
  static constexpr int KPL = 8;
  using frag = bf16x8;
  __device__ static __forceinline__ f32x16 run(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // B operand from accumulator registers rg = s*KPL .. s*KPL+7.
  template <int NB>
  __device__ static __forceinline__ frag pack(const f32x16 (&acc)[NB], int s) {
    frag f;
#pragma unroll
    for (int t = 0; t < 8; ++t) f[t] = (__bf16)acc[(s * 8 + t) / 16][(s * 8 + t) % 16];
    return f;
  }
  __device__ static __forceinline__ frag load(const __bf16 *p) {
    return *reinterpret_cast<const frag *>(p);
  }
  __device__ static __forceinline__ void store4(__bf16 *p, f32x4 x) {
    bf16x4 y;
    y[0] = (__bf16)x[0];
    y[1] = (__bf16)x[1];
    y[2] = (__bf16)x[2];
    y[3] = (__bf16)x[3];
    *reinterpret_cast<bf16x4 *>(p) = y;
  }
};

// float32 inputs: v_mfma_f32_32x32x2_f32, one contraction value per lane.
template <>
struct Mfma<float> {
  static constexpr int KPL = 1;
  using frag = float;
  __device__ static __forceinline__ f32x16 run(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  template <int NB>
  __device__ static __forceinline__ frag pack(const f32x16 (&acc)[NB], int s) {
    return acc[s / 16][s % 16];
  }
  __device__ static __forceinline__ frag load(const float *p) { return *p; }
  __device__ static __forceinline__ void store4(float *p, f32x4 x) {
    *reinterpret_cast<f32x4 *>(p) = x;
  }
};

__device__ __forceinline__ void wait_all_memory() { __builtin_amdgcn_s_waitcnt(0); }

// NQC query chunks per block; NBUF = 2 double-buffers the staged operands
// (NBUF = 1 is used only where two copies do not fit in LDS).
template <typename E, int D, bool FOX, int NQC, int NBUF>
__global__ __launch_bounds__(NQC * 128) void stream_kernel(
    const float *__restrict__ qa, const E *__restrict__ kvm,
    const float *__restrict__ al, const float *__restrict__ gate,
    E *__restrict__ out, float *__restrict__ lse, int BH, int T, float sl2) {
  using MF = Mfma<E>;
  using frag = typename MF::frag;
  constexpr int C = kChunk, KPL = MF::KPL, KSTEP = 2 * KPL;
  constexpr int NDB = D / 32;           // 32-row blocks over d
  constexpr int NSD = D / KSTEP;        // k-steps of a contraction over d
  constexpr int NSK = C / KSTEP;        // k-steps of a contraction over keys
  constexpr int KVM = kvm_elems(D);
  constexpr int KVM_BYTES = KVM * (int)sizeof(E);
  constexpr int FRAG = 64 * KPL;        // elements of one A-operand fragment
  constexpr int NW = NQC * 2;           // waves per block
  static_assert(KVM_BYTES % 1024 == 0, "operand block must be whole 1 KiB pieces");
  __shared__ __attribute__((aligned(16))) unsigned char lds[NBUF * KVM_BYTES];

  const int N = T / C;
  const int NG = (N + NQC - 1) / NQC;
  const int bh = (int)(blockIdx.x % BH);
  const int qc0 = (NG - 1 - (int)(blockIdx.x / BH)) * NQC;   // longest groups first
  const int c_top = min(qc0 + NQC, N) - 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int qcw = qc0 + (wave >> 1);    // this wave's query chunk
  const int half = wave & 1;            // queries 32*half .. 32*half+31 of it
  const bool valid = qcw < N;
  const int qloc = half * 32 + n;
  const E *kvm_h = kvm + (size_t)bh * N * KVM;
  const float *gate_h = FOX ? gate + (size_t)bh * T : nullptr;

  // Copy key chunk c's operand block into LDS buffer `buf`: 1 KiB per wave
  // instruction, lane l's 16 bytes landing at offset 16*l.
  auto stage = [&](int c, int buf) {
    const unsigned char *src = reinterpret_cast<const unsigned char *>(kvm_h + (size_t)c * KVM);
    unsigned char *dst = lds + buf * KVM_BYTES;
    for (int j = wave; j < KVM_BYTES / 1024; j += NW)
      __builtin_amdgcn_global_load_lds((gbl_ptr_t)(src + j * 1024 + lane * 16),
                                       (lds_ptr_t)(dst + j * 1024), 16, 0, 0);
  };

  f32x16 qw[NDB], o[NDB], sc[2];
  float m_run = -INFINITY, l_run = 0.f;
#pragma unroll
  for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mb][r] = 0.f;
  if (valid) {  // running query tile, from the register image of <-Q
    const float *src = qa + ((size_t)bh * N + qcw) * qa_floats(D) + (size_t)half * NDB * 1024 + lane * 16;
#pragma unroll
    for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 x = *reinterpret_cast<const f32x4 *>(src + mb * 1024 + 4 * r4);
#pragma unroll
        for (int e = 0; e < 4; ++e) qw[mb][4 * r4 + e] = x[e];
      }
  }

  stage(c_top, NBUF == 2 ? (c_top & 1) : 0);
  wait_all_memory();
  __syncthreads();

  for (int c = c_top; c >= 0; --c) {
    const int buf = NBUF == 2 ? (c & 1) : 0;
    if (NBUF == 2 && c > 0) stage(c - 1, (c - 1) & 1);
    const E *kf_l = reinterpret_cast<const E *>(lds + buf * KVM_BYTES);
    const E *vf_l = kf_l + C * D;
    const E *mf_l = vf_l + C * D;

    if (valid && c == qcw) {
      // ---- diagonal block: register image of its logits; the key block
      // above the diagonal of the first half (keys 32..63, queries 0..31) is
      // wholly masked.
      const float *al_c = al + ((size_t)bh * N + qcw) * al_floats() + lane * 16;
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int key0 = 32 * mb + 8 * r4 + 4 * g;
          f32x4 x = {0.f, 0.f, 0.f, 0.f};
          if (mb <= half) x = *reinterpret_cast<const f32x4 *>(al_c + al_tile(half, mb) * 1024 + 4 * r4);
          f32x4 a = {0.f, 0.f, 0.f, 0.f};
          if (FOX) a = *reinterpret_cast<const f32x4 *>(gate_h + (size_t)c * C + key0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float s = key0 + e <= qloc ? __builtin_fmaf(x[e], sl2, a[e]) : -INFINITY;
            sc[mb][4 * r4 + e] = s;
            mx = fmaxf(mx, s);
          }
        }
      m_run = fmaxf(mx, __shfl_xor(mx, 32));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(sc[mb][r] - m_run);
          sc[mb][r] = p;
          l_run += p;
        }
#pragma unroll
      for (int s = 0; s < NSK; ++s) {
        const frag pb = MF::pack(sc, s);
#pragma unroll
        for (int mb = 0; mb < NDB; ++mb)
          o[mb] = MF::run(MF::load(vf_l + (mb * NSK + s) * FRAG + lane * KPL), pb, o[mb]);
      }
    } else if (valid && c < qcw) {
      // ---- cross step against key chunk c ----
      frag qb[NSD];
#pragma unroll
      for (int s = 0; s < NSD; ++s) qb[s] = MF::pack(qw, s);
      // S^T = ->K_c Q_work^T
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[mb][r] = 0.f;
#pragma unroll
        for (int s = 0; s < NSD; ++s)
          sc[mb] = MF::run(MF::load(kf_l + (mb * NSD + s) * FRAG + lane * KPL), qb[s], sc[mb]);
      }
      // Q_work^T <- Q_work^T - M_c^T round(Q_work^T): cross chunk c's transition.
      if (c > 0) {
#pragma unroll
        for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
          for (int s = 0; s < NSD; ++s)
            qw[mb] = MF::run(MF::load(mf_l + (mb * NSD + s) * FRAG + lane * KPL), qb[s], qw[mb]);
      }
      // Online softmax in log2 units: logit x = S * scale * log2(e) (+ a_j).
      float mx = -INFINITY;
      if (FOX) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(gate_h + (size_t)c * C + 32 * mb + 8 * r4 + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float s = __builtin_fmaf(sc[mb][4 * r4 + e], sl2, a[e]);
              sc[mb][4 * r4 + e] = s;
              mx = fmaxf(mx, s);
            }
          }
      } else {
        // the scale is positive: take the max of the raw scores, scale once
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[mb][r]);
        mx *= sl2;
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      if (__any(m_new > m_run)) {   // wave-uniform: rescale only when a max grew
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[mb][r] *= alpha;
        m_run = m_new;
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(
              FOX ? sc[mb][r] - m_run : __builtin_fmaf(sc[mb][r], sl2, -m_run));
          sc[mb][r] = p;
          l_run += p;
        }
      // O^T += V_c^T P^T
#pragma unroll
      for (int s = 0; s < NSK; ++s) {
        const frag pb = MF::pack(sc, s);
#pragma unroll
        for (int mb = 0; mb < NDB; ++mb)
          o[mb] = MF::run(MF::load(vf_l + (mb * NSK + s) * FRAG + lane * KPL), pb, o[mb]);
      }
    }

    if (NBUF == 2) {
      wait_all_memory();   // this wave's share of chunk c-1 has landed
      __syncthreads();     // ... and everyone's; buffer c is free again
    } else {
      __syncthreads();
      if (c > 0) {
        stage(c - 1, 0);
        wait_all_memory();
      }
      __syncthreads();
    }
  }

  // ---- epilogue: o_i = O_i / l_i, lse_i = ln 2 (m + log2 l - a_i) ----
  if (!valid) return;
  const size_t qtok = (size_t)bh * T + (size_t)qcw * C + qloc;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  E *out_r = out + qtok * D;
#pragma unroll
  for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = o[mb][4 * r4 + e] * inv;
      MF::store4(out_r + 32 * mb + 8 * r4 + 4 * g, x);
    }
  if (g == 0) {
    const float a_i = FOX ? gate_h[(size_t)qcw * C + qloc] : 0.f;
    lse[qtok] = kLn2 * (m_run - a_i + __builtin_amdgcn_logf(l_tot));
  }
}

// Launch shapes: query chunks per block and staging buffers per (dtype, d).
template <typename E, int D>
struct Shape;
template <>
struct Shape<__bf16, 64> { static constexpr int NQC = 2, NBUF = 2; };
template <>
struct Shape<__bf16, 128> { static constexpr int NQC = 4, NBUF = 2; };
template <>
struct Shape<float, 64> { static constexpr int NQC = 2, NBUF = 2; };
template <>
struct Shape<float, 128> { static constexpr int NQC = 2, NBUF = 1; };

template <typename E, int D, bool FOX>
hipError_t launch_stream_t(const float *qa, const void *kvm, const float *al,
                           const float *gate, void *out, float *lse, int BH,
                           int T, hipStream_t stream) {
  constexpr int NQC = Shape<E, D>::NQC, NBUF = Shape<E, D>::NBUF;
  const int N = T / kChunk;
  const int blocks = BH * ((N + NQC - 1) / NQC);
  const float sl2 = kLog2e / sqrtf((float)D);
  hipLaunchKernelGGL((stream_kernel<E, D, FOX, NQC, NBUF>), dim3(blocks),
                     dim3(NQC * 128), 0, stream, qa, (const E *)kvm, al, gate,
                     (E *)out, lse, BH, T, sl2);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_stream_d(bool fox, const float *qa, const void *kvm,
                           const float *al, const float *gate, void *out,
                           float *lse, int BH, int T, hipStream_t stream) {
  if (fox) return launch_stream_t<E, D, true>(qa, kvm, al, gate, out, lse, BH, T, stream);
  return launch_stream_t<E, D, false>(qa, kvm, al, gate, out, lse, BH, T, stream);
}

}  // namespace

hipError_t launch_stream(int dtype, int D, bool fox, const float *qa,
                         const void *kvm, const float *al, const float *gate,
                         void *out, float *lse, int BH, int T,
                         hipStream_t stream) {
  if (dtype == 1) {
    if (D == 64) return launch_stream_d<__bf16, 64>(fox, qa, kvm, al, gate, out, lse, BH, T, stream);
    return launch_stream_d<__bf16, 128>(fox, qa, kvm, al, gate, out, lse, BH, T, stream);
  }
  if (D == 64) return launch_stream_d<float, 64>(fox, qa, kvm, al, gate, out, lse, BH, T, stream);
  return launch_stream_d<float, 128>(fox, qa, kvm, al, gate, out, lse, BH, T, stream);
}

}  // namespace pathattn
