// path_attn_internal.h -- shared definitions of the libpath_attn kernels.
//
// Data layout in HBM (the caller's workspace), per (batch*head) bh and 64-token
// chunk c (N = T/64 chunks per head):
//
//   qa   float [BH][T][D]        boundary-adjusted queries <-Q (row i holds
//                                H_first...H_i q_i), the starting value of the
//                                streaming kernel's running query tile.
//   kvm  elem  [BH][N][KVM(D)]   per chunk, three matrix-core A operands stored
//                                back to back in "fragment order" (below):
//                                  KF: ->K   (64 keys x D, contraction over D)
//                                  VF: V^T   (D x 64 keys, contraction over keys)
//                                  MF: -M^T  (D x D, contraction over D),
//                                      M = W^T U W, the chunk transform
//   al   float [BH][N][64][64]   diagonal-block raw logits (row = query)
//   gate float [BH][T]           a_t = -log2(e) * sum_{1<=s<=t} log f_s (FoX only)
//
// Fragment order.  The streaming kernel keeps its running query tile, scores
// and output in MFMA accumulators laid out as X^T (rows = d or key index,
// columns = the wave's 32 queries) and feeds an accumulator straight back as
// the B operand of the next MFMA.  For a 32x32 accumulator block, lane l
// (g = l/32) register r holds row 8*(r/4) + 4*g + r%4 of column l%32.  Taking
// KPL consecutive accumulator registers per k-step as the B operand makes the
// k-th contraction slot of lane group g correspond to the physical row
//
//     frag_row(s, g, t) = 32*(rg/16) + 8*((rg%16)/4) + 4*g + rg%4,
//     rg = s*KPL + t,   t in [0, KPL),
//
// where KPL = 8 for bf16 MFMA 32x32x16 and 1 for fp32 MFMA 32x32x2.  The A
// operand must use the same permutation of its contraction index, so the
// chunk-prep kernel writes A operands pre-permuted: blob (mb, s) of an operand
// X[R][Kc] holds, for lane l, the KPL values X[32*mb + l%32][frag_row(s,l/32,t)]
// contiguously; blob index = mb * (Kc / (2*KPL)) + s.  A wave then reads one
// A fragment as one contiguous 64*KPL-element block (conflict-free LDS reads).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pathattn {

constexpr int kChunk = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__host__ __device__ constexpr int frag_row(int s, int g, int t, int kpl) {
  return 32 * ((s * kpl + t) / 16) + 8 * (((s * kpl + t) % 16) / 4) + 4 * g +
         ((s * kpl + t) % 4);
}

// Elements of one chunk's kvm block.
__host__ __device__ constexpr int kvm_elems(int D) { return 2 * kChunk * D + D * D; }

struct Layout {
  size_t qa, kvm, al, gate, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline Layout make_layout(int B, int H, int T, int D, size_t esize) {
  const size_t BH = (size_t)B * H, N = (size_t)T / kChunk;
  Layout L;
  size_t off = 0;
  L.qa = off;
  off = align256(off + BH * T * D * sizeof(float));
  L.kvm = off;
  off = align256(off + BH * N * kvm_elems(D) * esize);
  L.al = off;
  off = align256(off + BH * N * kChunk * kChunk * sizeof(float));
  L.gate = off;
  off = align256(off + BH * T * sizeof(float));
  L.total = off;
  return L;
}

// Launchers (return hipGetLastError() after the launch).
hipError_t launch_gate_prefix(const float *logf, float *gate, int BH, int T,
                              hipStream_t stream);
hipError_t launch_prep(int dtype, int D, const void *q, const void *k,
                       const void *v, const void *w, const float *beta,
                       float *qa, void *kvm, float *al, int BH, int T,
                       hipStream_t stream);
hipError_t launch_stream(int dtype, int D, bool fox, const float *qa,
                         const void *kvm, const float *al, const float *gate,
                         void *out, float *lse, int BH, int T,
                         hipStream_t stream);
hipError_t launch_unpack(int dtype, int D, const float *qa_ws, const void *kvm,
                         const float *al_ws, const float *gate, float *qa,
                         float *kb, float *m, float *al, float *lam, int BH,
                         int T, hipStream_t stream);

}  // namespace pathattn
