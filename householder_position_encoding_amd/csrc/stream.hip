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
#include <type_traits>

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
  // The rounding remainder of pack(acc, s): acc - hi, rounded to bf16.
  template <int NB>
  __device__ static __forceinline__ frag pack_lo(const f32x16 (&acc)[NB], int s, frag hi) {
    frag f;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      f[t] = (__bf16)(acc[(s * 8 + t) / 16][(s * 8 + t) % 16] - (float)hi[t]);
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

// Workgroup barrier for the LDS operand ring.  __syncthreads() (and a
// workgroup fence, even one restricted to LDS, since copies into LDS count as
// LDS writes) waits for every outstanding global load of the wave, which would
// drain the operand prefetch at each step.  Here the wave's own LDS reads are
// completed (lgkmcnt 0, so a buffer can be refilled after the barrier), the
// copies are waited for explicitly (vmcnt) by the caller, and the empty asm
// statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt at maxima
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most n vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their maxima so they impose no wait).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Exact block skip with the forget gate.  For query i and key chunk c every
// logit of the block obeys (log2 units, without the row constant -a_i)
//     x_ij = scale*log2(e) * bf16(Q_work_i) . k~_j + a_j
//         <= scale*log2(e) * |Q_work_i| * max_j |k~_j| * (1 + 2^-9 + ...) + max_j a_j,
// with b = (max_j a_j, max_j |k~_j|^2) per chunk from the chunk preparation.
// When this bound lies more than kSkipBelow under the running max for every
// query of the wave, every weight 2^(x - m_ref) (m_ref >= m_run) of the block
// is below 2^-160, i.e. exactly 0 in float32, the max does not move and l and
// O would only add zeros: skipping S, the softmax and P.V of that block leaves
// every result bit unchanged.  The transition of chunk c is still applied.
constexpr float kSkipBelow = 160.f;

__device__ __forceinline__ float logit_bound(float qn2, float2 b, float sl2) {
  // 1.01 covers the bf16 rounding of the query tile, the float32 accumulation
  // of the products and of the squared norms; +1 covers the gate's rounding.
  return __builtin_fmaf(sl2 * __builtin_sqrtf(qn2 * b.y), 1.01f, b.x + 1.f);
}

// NQC query chunks per block, two waves per chunk.  Operand blocks are
// prefetched PD key chunks ahead into a ring of PD + 1 LDS buffers (PD = 0:
// one buffer, loaded synchronously, for shapes where two copies do not fit).
// DP: the leading coordinates the chunk transitions act on (D, or D / 2 for
// partial PaTH: -M^T is DP x DP and the transition product touches only the
// first DP rows of the running tile).
// PREC (bf16): the S product takes the running query tile and ->K_c as bf16
// hi + lo pairs (Q_hi K_hi + Q_lo K_hi + Q_hi K_lo), so neither rounding
// enters the logits; ->K_c's remainders (klo, same blob order) are staged
// after the operand block.
template <typename E, int D, int DP, bool FOX, int NQC, int PD, bool PREC = false>
__global__ __launch_bounds__(NQC * 128) void stream_kernel(
    const float *__restrict__ qa, const E *__restrict__ kvm,
    const float *__restrict__ al, const float *__restrict__ gate,
    const float2 *__restrict__ bnd, int skip, unsigned long long *__restrict__ skipped,
    E *__restrict__ out, float *__restrict__ lse, int BH, int T, float sl2, int H,
    TokStrides so, TokStrides sl, const E *__restrict__ klo) {
  using MF = Mfma<E>;
  using frag = typename MF::frag;
  constexpr int C = kChunk, KPL = MF::KPL, KSTEP = 2 * KPL;
  constexpr int NDB = D / 32;           // 32-row blocks over d
  constexpr int NSD = D / KSTEP;        // k-steps of a contraction over d
  constexpr int NDBP = DP / 32;         // the same over the path coordinates
  constexpr int NSDP = DP / KSTEP;
  constexpr int NSK = C / KSTEP;        // k-steps of a contraction over keys
  constexpr int KVM = kvm_elems(D, DP);
  constexpr int KVM_BYTES = KVM * (int)sizeof(E);
  constexpr int FRAG = 64 * KPL;        // elements of one A-operand fragment
  constexpr int NW = NQC * 2;           // waves per block
  constexpr int NBUF = PD + 1;
  constexpr int NBLK = KVM_BYTES / 1024;          // 1 KiB copy instructions per chunk
  constexpr int NL = (NBLK + NW - 1) / NW;        // per wave (the last round partly)
  static_assert(KVM_BYTES % 1024 == 0, "operand block in whole KiB");
  static_assert(PD < 2 || NBLK % NW == 0, "deep prefetch counts copies per wave");
  constexpr int KLO_BYTES = PREC ? C * D * (int)sizeof(E) : 0;   // ->K remainders
  constexpr int BUFB = KVM_BYTES + KLO_BYTES;                      // one LDS buffer
  constexpr int NBLO = KLO_BYTES / 1024, NLL = (NBLO + NW - 1) / NW;
  static_assert(!PREC || (PD < 2 && std::is_same<E, __bf16>::value), "precise: bf16, PD <= 1");
  __shared__ __attribute__((aligned(16))) unsigned char lds[NBUF * BUFB];
  __shared__ __attribute__((aligned(16))) float gate_l[FOX ? NBUF * C : 1];

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
  // With the forget gate, wave 0 first copies the chunk's 64 gate values
  // (4 bytes per lane) into the matching slot of a small LDS ring.
  auto stage = [&](int c, int buf) {
    if (FOX && wave == 0)
      copy4_to_lds(gate_h + (size_t)c * C + lane, lds_addr(gate_l + buf * C));
    const unsigned char *src = reinterpret_cast<const unsigned char *>(kvm_h + (size_t)c * KVM);
    unsigned char *dst = lds + buf * BUFB;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int j = wave + i * NW;
      if (NBLK % NW == 0 || j < NBLK) copy16_to_lds(src + j * 1024 + lane * 16, lds_addr(dst + j * 1024));
    }
    if constexpr (PREC) {
      const unsigned char *slo =
          reinterpret_cast<const unsigned char *>(klo + ((size_t)bh * N + c) * C * D);
#pragma unroll
      for (int i = 0; i < NLL; ++i) {
        const int j = wave + i * NW;
        if (j < NBLO) copy16_to_lds(slo + j * 1024 + lane * 16, lds_addr(dst + KVM_BYTES + j * 1024));
      }
    }
  };

  f32x16 qw[NDB], o[NDB], sc[2];
  float m_run = -INFINITY, l_run = 0.f;
  unsigned n_skip = 0;
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

  // Online softmax in log2 units (logit x = S * scale * log2(e) + a_j), lazy
  // rescale: O and l are rescaled only when the wave-wide max grew.
  auto softmax_pv = [&](f32x16 (&s_in)[2], const float *gb, const E *vb, bool scaled) {
    float mx = -INFINITY;
    if (scaled) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_in[mb][r]);
    } else if (FOX) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 a = *reinterpret_cast<const f32x4 *>(gb + 32 * mb + 8 * r4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = __builtin_fmaf(s_in[mb][4 * r4 + e], sl2, a[e]);
            s_in[mb][4 * r4 + e] = x;
            mx = fmaxf(mx, x);
          }
        }
    } else {
      // the scale is positive: take the max of the raw scores, scale once
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s_in[mb][r]);
      mx *= sl2;
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__any(mx > m_run)) {   // wave-uniform
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[mb][r] *= alpha;
      m_run = m_new;
    }
    const bool raw = !scaled && !FOX;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(
            raw ? __builtin_fmaf(s_in[mb][r], sl2, -m_run) : s_in[mb][r] - m_run);
        s_in[mb][r] = pr;
        l_run += pr;
      }
#pragma unroll
    for (int s = 0; s < NSK; ++s) {
      const frag pb = MF::pack(s_in, s);
#pragma unroll
      for (int mb = 0; mb < NDB; ++mb)
        o[mb] = MF::run(MF::load(vb + (mb * NSK + s) * FRAG + lane * KPL), pb, o[mb]);
    }
  };

  for (int p = 0; p <= (PD > 0 ? PD - 1 : 0); ++p)
    if (c_top - p >= 0) stage(c_top - p, (c_top - p) % NBUF);
  wait_all_memory();
  lds_barrier();

  for (int c = c_top; c >= 0; --c) {
    const int buf = c % NBUF;
    if (PD > 0 && c - PD >= 0) stage(c - PD, (c - PD) % NBUF);
    const E *kf_l = reinterpret_cast<const E *>(lds + buf * BUFB);
    const E *vf_l = kf_l + C * D;
    const E *kl_l = reinterpret_cast<const E *>(lds + buf * BUFB + KVM_BYTES);   // PREC
    const E *mf_l = vf_l + C * D;
    const float *ga = gate_l + buf * C + 4 * g;

    if (valid && c == qcw) {
      // ---- diagonal block: register image of its logits; the key block
      // above the diagonal of the first half (keys 32..63, queries 0..31) is
      // wholly masked.
      const float *al_c = al + ((size_t)bh * N + qcw) * al_floats() + lane * 16;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int key0 = 32 * mb + 8 * r4 + 4 * g;
          f32x4 x = {0.f, 0.f, 0.f, 0.f};
          if (mb <= half) x = *reinterpret_cast<const f32x4 *>(al_c + al_tile(half, mb) * 1024 + 4 * r4);
          f32x4 a = {0.f, 0.f, 0.f, 0.f};
          if (FOX) a = *reinterpret_cast<const f32x4 *>(ga + 32 * mb + 8 * r4);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sc[mb][4 * r4 + e] = key0 + e <= qloc ? __builtin_fmaf(x[e], sl2, a[e]) : -INFINITY;
        }
      softmax_pv(sc, ga, vf_l, true);
    } else if (valid && c < qcw) {
      // ---- cross step against key chunk c ----
      bool skip_blk = false;
      if (FOX && skip) {
        float qn2 = 0.f;
#pragma unroll
        for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) qn2 = __builtin_fmaf(qw[mb][r], qw[mb][r], qn2);
        qn2 += __shfl_xor(qn2, 32);
        skip_blk = __all(logit_bound(qn2, bnd[(size_t)bh * N + c], sl2) < m_run - kSkipBelow);
        n_skip += skip_blk;
      }
      frag qb[NSD];
#pragma unroll
      for (int s = 0; s < NSD; ++s) qb[s] = MF::pack(qw, s);
      if (!skip_blk) {
        // S^T = ->K_c Q_work^T
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[mb][r] = 0.f;
        if constexpr (PREC) {
          // one lo fragment live at a time
#pragma unroll
          for (int s = 0; s < NSD; ++s) {
            const frag lo = MF::pack_lo(qw, s, qb[s]);
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) {
              const frag a = MF::load(kf_l + (mb * NSD + s) * FRAG + lane * KPL);
              const frag al = MF::load(kl_l + (mb * NSD + s) * FRAG + lane * KPL);
              sc[mb] = MF::run(a, qb[s], sc[mb]);
              sc[mb] = MF::run(a, lo, sc[mb]);
              sc[mb] = MF::run(al, qb[s], sc[mb]);
            }
          }
        } else {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int s = 0; s < NSD; ++s)
              sc[mb] = MF::run(MF::load(kf_l + (mb * NSD + s) * FRAG + lane * KPL), qb[s], sc[mb]);
        }
      }
      // Q_work^T <- Q_work^T - M_c^T round(Q_work^T): crossing chunk c's
      // transition (after chunk 0 the tile is not used)
      if (c > 0) {
#pragma unroll
        for (int mb = 0; mb < NDBP; ++mb)
#pragma unroll
          for (int s = 0; s < NSDP; ++s)
            qw[mb] = MF::run(MF::load(mf_l + (mb * NSDP + s) * FRAG + lane * KPL), qb[s], qw[mb]);
      }
      if (!skip_blk) softmax_pv(sc, ga, vf_l, false);
    }

    if (PD == 0) {
      lds_barrier();
      if (c > 0) {
        stage(c - 1, 0);
        wait_all_memory();
      }
      lds_barrier();
    } else {
      // This wave's share of chunk c-1 has landed once at most the copies of
      // the chunks issued after it (c-2 .. c-PD, those that exist) are
      // outstanding (wave 0 also copies the gate: one more operation per
      // chunk); the barrier then makes everyone's share visible and frees
      // buffer c for the next prefetch.
      if (PD >= 2 && c - 2 >= 0) {
        if (FOX && wave == 0)
          wait_vmcnt<(PD >= 2 ? NL + 1 : 0)>();
        else
          wait_vmcnt<(PD >= 2 ? NL : 0)>();
      } else {
        wait_all_memory();
      }
      lds_barrier();
    }
  }

  // ---- epilogue: o_i = O_i / l_i, lse_i = ln 2 (m + log2 l - a_i) ----
  if (!valid) return;
  if (FOX && skipped && lane == 0 && n_skip) atomicAdd(skipped, (unsigned long long)n_skip);
  const long long tq = (long long)qcw * C + qloc;
  const long long ob = (long long)(bh / H) * so.b + (long long)(bh % H) * so.h;
  const long long lb = (long long)(bh / H) * sl.b + (long long)(bh % H) * sl.h;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  E *out_r = out + ob + tq * so.t;
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
    lse[lb + tq * sl.t] = kLn2 * (m_run - a_i + __builtin_amdgcn_logf(l_tot));
  }
}

// Wide variant for bf16 operands: one wave holds a whole 64-query chunk as two
// 32-query column blocks j = 0, 1, so every A fragment read from LDS (->K,
// -M^T, V^T) feeds two matrix instructions.  This halves the LDS operand reads
// and the staging per unit of work; the price is about 250 registers per lane
// (running tile, output and scores for 64 queries), i.e. two waves per SIMD.
// Without the gate, a cross step exponentiates against the running max m_run
// with no max pass over the block: the lane's sum of the weights bounds every
// weight, and if it exceeds 2^11 (or is not finite) the block is redone
// against m_ref = max(m_run, block max - 8) after rescaling O and l.  This is
// the usual online softmax with another choice of reference (any reference
// gives the same normalised result); the bound keeps every weight below 2^11,
// far inside float32 and bf16 range.  With the gate (and on the diagonal) the
// block max is taken first and the reference is max(m_run, mx - 8), so
// p <= 2^8 and the rare rescale comes after the exponentials.  The row sums
// are taken from the bf16-rounded weights that the P.V products use (dot with
// (1, 1)), so numerator and denominator match.
template <int D, int DP, bool FOX, int NQC, int PD>
__global__ __launch_bounds__(NQC * 64, 2) void stream_wide_kernel(
    const float *__restrict__ qa, const __bf16 *__restrict__ kvm,
    const float *__restrict__ al, const float *__restrict__ gate,
    const float2 *__restrict__ bnd, int skip, unsigned long long *__restrict__ skipped,
    __bf16 *__restrict__ out, float *__restrict__ lse, int BH, int T, float sl2, int H,
    TokStrides so, TokStrides sl) {
  using E = __bf16;
  using MF = Mfma<E>;
  using frag = typename MF::frag;
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  constexpr int C = kChunk, KPL = MF::KPL, KSTEP = 2 * KPL;
  constexpr int NDB = D / 32;
  constexpr int NSD = D / KSTEP;
  constexpr int NDBP = DP / 32;
  constexpr int NSDP = DP / KSTEP;
  constexpr int NSK = C / KSTEP;
  constexpr int KVM = kvm_elems(D, DP);
  constexpr int KVM_BYTES = KVM * (int)sizeof(E);
  constexpr int FRAG = 64 * KPL;
  constexpr int NW = NQC;               // one wave per query chunk
  constexpr int NBUF = PD + 1;
  constexpr int NBLK = KVM_BYTES / 1024;
  constexpr int NL = (NBLK + NW - 1) / NW;
  static_assert(PD >= 1, "the wide kernel always prefetches");
  static_assert(KVM_BYTES % 1024 == 0, "operand block in whole KiB");
  static_assert(PD < 2 || NBLK % NW == 0, "deep prefetch counts copies per wave");
  __shared__ __attribute__((aligned(16))) unsigned char lds[NBUF * KVM_BYTES];
  __shared__ __attribute__((aligned(16))) float gate_l[FOX ? NBUF * C : 1];

  const int N = T / C;
  const int NG = (N + NQC - 1) / NQC;
  const int bh = (int)(blockIdx.x % BH);
  const int qc0 = (NG - 1 - (int)(blockIdx.x / BH)) * NQC;   // longest groups first
  const int c_top = min(qc0 + NQC, N) - 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, g = lane >> 5;
  const int qcw = qc0 + wave;
  const bool valid = qcw < N;
  const E *kvm_h = kvm + (size_t)bh * N * KVM;
  const float *gate_h = FOX ? gate + (size_t)bh * T : nullptr;

  auto stage = [&](int c, int buf) {
    if (FOX && wave == 0)
      copy4_to_lds(gate_h + (size_t)c * C + lane, lds_addr(gate_l + buf * C));
    const unsigned char *src = reinterpret_cast<const unsigned char *>(kvm_h + (size_t)c * KVM);
    unsigned char *dst = lds + buf * KVM_BYTES;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int jb = wave + i * NW;
      if (NBLK % NW == 0 || jb < NBLK) copy16_to_lds(src + jb * 1024 + lane * 16, lds_addr(dst + jb * 1024));
    }
  };

  f32x16 qw[2][NDB], o[2][NDB], sc[2][2];
  float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
  unsigned n_skip = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[j][mb][r] = 0.f;
  if (valid) {
    const float *src = qa + ((size_t)bh * N + qcw) * qa_floats(D) + lane * 16;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 x = *reinterpret_cast<const f32x4 *>(src + (j * NDB + mb) * 1024 + 4 * r4);
#pragma unroll
          for (int e = 0; e < 4; ++e) qw[j][mb][4 * r4 + e] = FOX ? x[e] : x[e] * sl2;
        }
  }

  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  // p = 2^(x - m), packed to the bf16 B operands of P.V; returns the lane's
  // partial sum of the packed weights.
  // x is already in log2 units when mul == 1 (diagonal, gated scores),
  // raw scores with mul = scale * log2(e) otherwise.  REL: x is already
  // x - m (the cross steps without the gate), mul and m are not used, and
  // the weights are summed onto l0 in one chain (the caller keeps l0).
  auto exp_pack = [&](const f32x16 (&x)[2], float mul, float m, frag (&pb)[NSK],
                      auto rel, float l0 = 0.f) -> float {
    constexpr bool REL = decltype(rel)::value;
    float part[4] = {REL ? l0 : 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NSK; ++s) {
      f32x16 pr[2];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int rg = s * 8 + t;
        const float xv = x[rg / 16][rg % 16];
        pr[rg / 16][rg % 16] = __builtin_amdgcn_exp2f(REL ? xv : __builtin_fmaf(xv, mul, -m));
      }
      pb[s] = MF::pack(pr, s);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const bf16x2 pair = {pb[s][2 * h], pb[s][2 * h + 1]};
        part[REL ? 0 : h] = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, part[REL ? 0 : h], false);
      }
    }
    return REL ? part[0] : (part[0] + part[1]) + (part[2] + part[3]);
  };
  auto pv = [&](const frag (&pb)[2][NSK], const E *vb) {
#pragma unroll
    for (int s = 0; s < NSK; ++s)
#pragma unroll
      for (int mb = 0; mb < NDB; ++mb) {
        const frag a = MF::load(vb + (mb * NSK + s) * FRAG + lane * KPL);
#pragma unroll
        for (int j = 0; j < 2; ++j) o[j][mb] = MF::run(a, pb[j][s], o[j][mb]);
      }
  };

  for (int p = 0; p < PD; ++p)
    if (c_top - p >= 0) stage(c_top - p, (c_top - p) % NBUF);
  wait_all_memory();
  lds_barrier();

  for (int c = c_top; c >= 0; --c) {
    const int buf = c % NBUF;
    if (c - PD >= 0) stage(c - PD, (c - PD) % NBUF);
    const E *kf_l = reinterpret_cast<const E *>(lds + buf * KVM_BYTES);
    const E *vf_l = kf_l + C * D;
    const E *mf_l = vf_l + C * D;
    const float *ga = gate_l + buf * C + 4 * g;

    if (valid && c == qcw) {
      // ---- diagonal block: logits from the register image; key block 1 of
      // query block 0 lies wholly above the diagonal.
      const float *al_c = al + ((size_t)bh * N + qcw) * al_floats() + lane * 16;
      frag pb[2][NSK];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int key0 = 32 * kb + 8 * r4 + 4 * g;
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            if (kb <= j) x = *reinterpret_cast<const f32x4 *>(al_c + al_tile(j, kb) * 1024 + 4 * r4);
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
            if (FOX) a = *reinterpret_cast<const f32x4 *>(ga + 32 * kb + 8 * r4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float sv = key0 + e <= 32 * j + n ? __builtin_fmaf(x[e], sl2, a[e]) : -INFINITY;
              sc[j][kb][4 * r4 + e] = sv;
              mx = fmaxf(mx, sv);
            }
          }
        m_run[j] = fmaxf(mx, __shfl_xor(mx, 32));
        l_run[j] = exp_pack(sc[j], 1.f, m_run[j], pb[j], std::false_type{});
      }
      pv(pb, vf_l);
    } else if (valid && c < qcw) {
      // ---- cross step against key chunk c ----
      bool skip_blk = false;
      if (FOX && skip) {   // exact block skip, see logit_bound
        bool below = true;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          float qn2 = 0.f;
#pragma unroll
          for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) qn2 = __builtin_fmaf(qw[j][mb][r], qw[j][mb][r], qn2);
          qn2 += __shfl_xor(qn2, 32);
          below = below && logit_bound(qn2, bnd[(size_t)bh * N + c], sl2) < m_run[j] - kSkipBelow;
        }
        skip_blk = __all(below);
        n_skip += skip_blk;
      }
      frag qb[2][NSD];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int s = 0; s < NSD; ++s) qb[j][s] = MF::pack(qw[j], s);
      // S^T = ->K_c Q_work^T for both column blocks.  Without the gate the
      // tile is pre-scaled by scale * log2(e) and the products start from
      // -m_run, so the scores come out as x - m_run in log2 units
#pragma unroll
      for (int kb = 0; kb < 2 && !skip_blk; ++kb) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[j][kb][r] = FOX ? 0.f : -m_run[j];
#pragma unroll
        for (int s = 0; s < NSD; ++s) {
          const frag a = MF::load(kf_l + (kb * NSD + s) * FRAG + lane * KPL);
#pragma unroll
          for (int j = 0; j < 2; ++j) sc[j][kb] = MF::run(a, qb[j][s], sc[j][kb]);
        }
      }
      // Q_work^T <- Q_work^T - M_c^T round(Q_work^T) (unused after chunk 0)
      if (c > 0) {
#pragma unroll
        for (int mb = 0; mb < NDBP; ++mb)
#pragma unroll
          for (int s = 0; s < NSDP; ++s) {
            const frag a = MF::load(mf_l + (mb * NSDP + s) * FRAG + lane * KPL);
#pragma unroll
            for (int j = 0; j < 2; ++j) qw[j][mb] = MF::run(a, qb[j][s], qw[j][mb]);
          }
      }
      if (!skip_blk) {
      if (!FOX) {
        // weights against the running max without a max pass (the scores
        // are x - m_run already); a chunk whose weights exceed 2^11 (or are
        // not finite) is redone against max(m_run, chunk max - 8) after
        // rescaling O and l
        frag pb[2][NSK];
        float lnew[2];
        bool big = false;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          lnew[j] = exp_pack(sc[j], 1.f, 0.f, pb[j], std::true_type{}, l_run[j]);
          big = big || !(lnew[j] - l_run[j] <= 2048.f);
        }
        if (__any(big)) {   // wave-uniform, rare
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
              for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[j][kb][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float up = fmaxf(0.f, mx - 8.f);   // m_new - m_run
            const float alpha = __builtin_amdgcn_exp2f(-up);
            l_run[j] *= alpha;
#pragma unroll
            for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
              for (int r = 0; r < 16; ++r) o[j][mb][r] *= alpha;
            m_run[j] += up;
            lnew[j] = l_run[j] + exp_pack(sc[j], 1.f, up, pb[j], std::false_type{});
          }
        }
        l_run[0] = lnew[0];
        l_run[1] = lnew[1];
        pv(pb, vf_l);
      } else {
      // online softmax in log2 units, x = S * scale * log2(e) + a_key; the
      // gate of a key is read once and applied to both column blocks
      float mx[2] = {-INFINITY, -INFINITY};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 a = {0.f, 0.f, 0.f, 0.f};
          if (FOX) a = *reinterpret_cast<const f32x4 *>(ga + 32 * kb + 8 * r4);
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float x = sc[j][kb][4 * r4 + e];
              if (FOX) {
                x = __builtin_fmaf(x, sl2, a[e]);
                sc[j][kb][4 * r4 + e] = x;
              }
              mx[j] = fmaxf(mx[j], x);
            }
        }
      float m_ref[2];
      bool grow = false;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        // without the gate the max is taken on the raw scores (scale > 0)
        const float mj = FOX ? mx[j] : mx[j] * sl2;
        m_ref[j] = fmaxf(m_run[j], fmaxf(mj, __shfl_xor(mj, 32)) - 8.f);
        grow = grow || m_ref[j] > m_run[j];
      }
      frag pb[2][NSK];
      float lsum[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) lsum[j] = exp_pack(sc[j], FOX ? 1.f : sl2, m_ref[j], pb[j], std::false_type{});
      if (__any(grow)) {   // wave-uniform
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float alpha = __builtin_amdgcn_exp2f(m_run[j] - m_ref[j]);
          l_run[j] *= alpha;
#pragma unroll
          for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[j][mb][r] *= alpha;
          m_run[j] = m_ref[j];
        }
      }
      l_run[0] += lsum[0];
      l_run[1] += lsum[1];
      pv(pb, vf_l);
      }
      }
    }

    // chunk c-1 must have landed (this wave's share: at most the copies of
    // chunks c-2 .. c-PD outstanding); the barrier then publishes every
    // wave's share and frees buffer c for the next prefetch.
    // (wave 0 also copies the gate: one more operation per chunk)
    if (PD >= 2 && c - 2 >= 0) {
      if (FOX && wave == 0)
        wait_vmcnt<(PD >= 2 ? NL + 1 : 0)>();
      else
        wait_vmcnt<(PD >= 2 ? NL : 0)>();
    } else {
      wait_all_memory();
    }
    lds_barrier();
  }

  // ---- epilogue ----
  if (!valid) return;
  if (FOX && skipped && lane == 0 && n_skip) atomicAdd(skipped, (unsigned long long)n_skip);
  const long long ob = (long long)(bh / H) * so.b + (long long)(bh % H) * so.h;
  const long long lb = (long long)(bh / H) * sl.b + (long long)(bh % H) * sl.h;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int qloc = 32 * j + n;
    const long long tq = (long long)qcw * C + qloc;
    const float l_tot = l_run[j] + __shfl_xor(l_run[j], 32);
    const float inv = 1.f / l_tot;
    E *out_r = out + ob + tq * so.t;
#pragma unroll
    for (int mb = 0; mb < NDB; ++mb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = o[j][mb][4 * r4 + e] * inv;
        MF::store4(out_r + 32 * mb + 8 * r4 + 4 * g, x);
      }
    if (g == 0) {
      const float a_i = FOX ? gate_h[(size_t)qcw * C + qloc] : 0.f;
      lse[lb + tq * sl.t] = kLn2 * (m_run[j] - a_i + __builtin_amdgcn_logf(l_tot));
    }
  }
}

// Launch shapes: query chunks per block (NQC) and prefetch distance (PD) of
// the narrow kernel per (dtype, d); bf16 d = 64 runs the wide kernel.
#ifndef PATH_ATTN_WIDE_BF16_64
#define PATH_ATTN_WIDE_BF16_64 1
#endif
#ifndef PATH_ATTN_WIDE_PD
#define PATH_ATTN_WIDE_PD 1
#endif
#ifndef PATH_ATTN_NQC_BF16_128
#define PATH_ATTN_NQC_BF16_128 4
#endif
#ifndef PATH_ATTN_PD_BF16_128
#define PATH_ATTN_PD_BF16_128 1
#endif
template <typename E, int D>
struct Shape;
template <>
struct Shape<__bf16, 64> { static constexpr int NQC = 2, PD = 1; };
template <>
struct Shape<__bf16, 128> { static constexpr int NQC = PATH_ATTN_NQC_BF16_128, PD = PATH_ATTN_PD_BF16_128; };
template <>
struct Shape<float, 64> { static constexpr int NQC = 2, PD = 1; };
template <>
struct Shape<float, 128> { static constexpr int NQC = 2, PD = 0; };

template <typename E, int D, int DP, bool FOX>
hipError_t launch_stream_t(const StreamArgs &a, hipStream_t stream) {
  const int N = a.T / kChunk;
  const float sl2 = a.sl2;
  if constexpr (std::is_same<E, __bf16>::value) {
    if (a.klo) {   // precise: the narrow kernel with hi/lo operands in S
      // two buffers of 32 KiB at d = 64; one of 80 KiB at d = 128
      constexpr int NQC = D == 64 ? 2 : 4, PD = D == 64 ? 1 : 0;
      const int blocks = a.BH * ((N + NQC - 1) / NQC);
      hipLaunchKernelGGL((stream_kernel<E, D, DP, FOX, NQC, PD, true>), dim3(blocks),
                         dim3(NQC * 128), 0, stream, a.qa, (const E *)a.kvm, a.al, a.gate, a.bnd,
                         a.skip, a.skipped, (E *)a.out, a.lse, a.BH, a.T, sl2, a.H, a.so, a.sl,
                         (const E *)a.klo);
      return hipGetLastError();
    }
  }
  if constexpr (std::is_same<E, __bf16>::value && D == 64 && PATH_ATTN_WIDE_BF16_64) {
    // A block runs as long as its longest wave, and wave j of query group g
    // walks NQC g + j + 1 key chunks.  Eight chunks per block share each staged
    // operand block among twice the queries of four, but at N <= 64 chunks the
    // shorter waves of each block idle 10 % of the time or more: four chunks
    // per block (two blocks per CU) are faster there (B16 H16 T2048: 0.258 ->
    // 0.242 ms), eight above (B2 H16 T16384: 1.462 against 1.475 ms).
    constexpr int PD = PATH_ATTN_WIDE_PD;
    auto go = [&](auto nqc) {
      constexpr int NQC = decltype(nqc)::value;
      const int blocks = a.BH * ((N + NQC - 1) / NQC);
      hipLaunchKernelGGL((stream_wide_kernel<D, DP, FOX, NQC, PD>), dim3(blocks), dim3(NQC * 64), 0,
                         stream, a.qa, (const __bf16 *)a.kvm, a.al, a.gate, a.bnd, a.skip,
                         a.skipped, (__bf16 *)a.out, a.lse, a.BH, a.T, sl2, a.H, a.so, a.sl);
      return hipGetLastError();
    };
    if (N <= 64) return go(std::integral_constant<int, 4>{});
    return go(std::integral_constant<int, 8>{});
  }
  constexpr int NQC = Shape<E, D>::NQC, PD = Shape<E, D>::PD;
  const int blocks = a.BH * ((N + NQC - 1) / NQC);
  hipLaunchKernelGGL((stream_kernel<E, D, DP, FOX, NQC, PD>), dim3(blocks), dim3(NQC * 128), 0,
                     stream, a.qa, (const E *)a.kvm, a.al, a.gate, a.bnd, a.skip, a.skipped,
                     (E *)a.out, a.lse, a.BH, a.T, sl2, a.H, a.so, a.sl, (const E *)nullptr);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t launch_stream_d(int DP, bool fox, const StreamArgs &a, hipStream_t stream) {
  if (DP == D) {
    if (fox) return launch_stream_t<E, D, D, true>(a, stream);
    return launch_stream_t<E, D, D, false>(a, stream);
  }
  if (fox) return launch_stream_t<E, D, D / 2, true>(a, stream);
  return launch_stream_t<E, D, D / 2, false>(a, stream);
}

}  // namespace

hipError_t launch_stream(int dtype, int D, int DP, bool fox, const StreamArgs &a,
                         hipStream_t stream) {
  if (dtype == 1) {
    if (D == 64) return launch_stream_d<__bf16, 64>(DP, fox, a, stream);
    return launch_stream_d<__bf16, 128>(DP, fox, a, stream);
  }
  if (D == 64) return launch_stream_d<float, 64>(DP, fox, a, stream);
  return launch_stream_d<float, 128>(DP, fox, a, stream);
}

}  // namespace pathattn
