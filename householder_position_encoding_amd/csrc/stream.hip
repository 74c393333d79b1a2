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
// Work decomposition: one block of 2 waves per (batch*head, query chunk); each
// wave owns 32 queries.  Blocks are numbered so that the chunks with the most
// key blocks start first.  Per key chunk, the block stages that chunk's ->K,
// V^T and -M^T operands (one contiguous block of the workspace) in LDS.
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
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
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

template <typename E, int D, bool FOX>
__global__ __launch_bounds__(128) void stream_kernel(
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
  constexpr int FRAG = 64 * KPL;        // elements of one A-operand fragment
  __shared__ __attribute__((aligned(16))) E lds[KVM];
  const E *kf_l = lds;
  const E *vf_l = lds + C * D;
  const E *mf_l = lds + 2 * C * D;

  const int N = T / C;
  const int qc = N - 1 - (int)(blockIdx.x / BH);   // longest chunks first
  const int bh = (int)(blockIdx.x % BH);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int qloc = wave * 32 + n;                  // query row inside the chunk
  const size_t qtok = (size_t)bh * T + (size_t)qc * C + qloc;
  const E *kvm_h = kvm + (size_t)bh * N * KVM;
  const float *gate_h = FOX ? gate + (size_t)bh * T : nullptr;

  // Stage one chunk's operands in LDS (16-byte copies).
  auto stage = [&](int c) {
    const uint4 *src = reinterpret_cast<const uint4 *>(kvm_h + (size_t)c * KVM);
    uint4 *dst = reinterpret_cast<uint4 *>(lds);
    constexpr int NV = KVM * (int)sizeof(E) / 16;
    for (int i = tid; i < NV; i += 128) dst[i] = src[i];
  };

  // Running query tile, from the register image of <-Q of this chunk.
  f32x16 qw[NDB];
  {
    const float *src = qa + ((size_t)bh * N + qc) * qa_floats(D) + (size_t)wave * NDB * 1024 + lane * 16;
#pragma unroll
    for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 x = *reinterpret_cast<const f32x4 *>(src + mb * 1024 + 4 * r4);
#pragma unroll
        for (int e = 0; e < 4; ++e) qw[mb][4 * r4 + e] = x[e];
      }
  }

  f32x16 o[NDB];
#pragma unroll
  for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[mb][r] = 0.f;
  f32x16 sc[2];
  float m_run, l_run;   // running max (log2 units) and this lane's partial sum

  // ---- diagonal block ----
  stage(qc);
  {
    // Register image of the diagonal-block logits; the key block above the
    // diagonal of wave 0 (keys 32..63, queries 0..31) is wholly masked.
    const float *al_c = al + ((size_t)bh * N + qc) * al_floats() + lane * 16;
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int key0 = 32 * mb + 8 * r4 + 4 * g;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (mb <= wave) x = *reinterpret_cast<const f32x4 *>(al_c + al_tile(wave, mb) * 1024 + 4 * r4);
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
        if (FOX) a = *reinterpret_cast<const f32x4 *>(gate_h + (size_t)qc * C + key0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float s = key0 + e <= qloc ? x[e] * sl2 + a[e] : -INFINITY;
          sc[mb][4 * r4 + e] = s;
          mx = fmaxf(mx, s);
        }
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    m_run = mx;
    l_run = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(sc[mb][r] - m_run);
        sc[mb][r] = p;
        l_run += p;
      }
  }
  __syncthreads();
#pragma unroll
  for (int s = 0; s < NSK; ++s) {
    const frag pb = MF::pack(sc, s);
#pragma unroll
    for (int mb = 0; mb < NDB; ++mb)
      o[mb] = MF::run(MF::load(vf_l + (mb * NSK + s) * FRAG + lane * KPL), pb, o[mb]);
  }

  // ---- earlier key chunks, right to left ----
  for (int c = qc - 1; c >= 0; --c) {
    __syncthreads();
    stage(c);
    __syncthreads();

    frag qb[NSD];
#pragma unroll
    for (int s = 0; s < NSD; ++s) qb[s] = MF::pack(qw, s);

    // S^T = ->K_c Q_work^T
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int s = 0; s < NSD; ++s)
        acc = MF::run(MF::load(kf_l + (mb * NSD + s) * FRAG + lane * KPL), qb[s], acc);
      sc[mb] = acc;
    }
    // Q_work^T <- Q_work^T - M_c^T round(Q_work^T): cross chunk c's transition.
    if (c > 0) {
#pragma unroll
      for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
        for (int s = 0; s < NSD; ++s)
          qw[mb] = MF::run(MF::load(mf_l + (mb * NSD + s) * FRAG + lane * KPL), qb[s], qw[mb]);
    }

    // Online softmax in log2 units.
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
        if (FOX) a = *reinterpret_cast<const f32x4 *>(gate_h + (size_t)c * C + 32 * mb + 8 * r4 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float s = sc[mb][4 * r4 + e] * sl2 + a[e];
          sc[mb][4 * r4 + e] = s;
          mx = fmaxf(mx, s);
        }
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
        const float p = __builtin_amdgcn_exp2f(sc[mb][r] - m_run);
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

  // ---- epilogue: o_i = O_i / l_i, lse_i = ln 2 (m + log2 l - a_i) ----
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
    const float a_i = FOX ? gate_h[(size_t)qc * C + qloc] : 0.f;
    lse[qtok] = kLn2 * (m_run - a_i + __builtin_amdgcn_logf(l_tot));
  }
}

template <typename E, int D, bool FOX>
hipError_t launch_stream_t(const float *qa, const void *kvm, const float *al,
                           const float *gate, void *out, float *lse, int BH,
                           int T, hipStream_t stream) {
  const int blocks = BH * (T / kChunk);
  const float sl2 = kLog2e / sqrtf((float)D);
  hipLaunchKernelGGL((stream_kernel<E, D, FOX>), dim3(blocks), dim3(128), 0,
                     stream, qa, (const E *)kvm, al, gate, (E *)out, lse, BH,
                     T, sl2);
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
