// path_attn_internal.h -- shared definitions of the libpath_attn kernels.
//
// Register image.  The streaming kernel keeps its running query tile, its
// scores and its output in MFMA 32x32 accumulators in transposed orientation
// (rows = d or key index, columns = the wave's 32 queries).  In a 32x32
// accumulator block, lane l (g = l/32) register r (0..15) holds
//
//     row acc_row(r, g) = 8*(r/4) + 4*g + r%4,   column l%32.
//
// Taking KPL consecutive accumulator registers per k-step as the B operand of
// the next MFMA makes the k-th contraction slot of lane group g correspond to
// the physical row
//
//     frag_row(s, g, t) = 32*(rg/16) + acc_row(rg%16, g),  rg = s*KPL + t,
//
// with KPL = 8 for bf16 MFMA 32x32x16 and 1 for fp32 MFMA 32x32x2.  A operands
// therefore carry the same permutation of their contraction index; the chunk
// preparation writes them pre-permuted ("fragment order"): blob (mb, s) of an
// operand X[R][Kc] holds, for lane l, the KPL values
// X[32*mb + l%32][frag_row(s, l/32, t)] contiguously, blob index
// mb * (Kc / (2*KPL)) + s.  A fragment is then one contiguous 64*KPL-element
// block (conflict-free LDS reads, 16-byte global loads).
//
// Data layout in HBM (the caller's workspace), per (batch*head) bh and 64-token
// chunk c (N = T/64 chunks per head):
//
//   qa   float [BH][N][2][D/32][64][16]   boundary-adjusted queries <-Q
//        (row i: H_first...H_i q_i) as register image: [query block w]
//        [d block mb][lane][r] = <-Q[32w + lane%32][32mb + acc_row(r, lane/32)]
//   kvm  elem  [BH][N][KVM(D, DP)]   three A operands in fragment order:
//          KF: ->K   (64 keys x D, contraction over D)
//          VF: V^T   (D x 64 keys, contraction over keys)
//          MF: -M^T  (DP x DP, contraction over DP),  M = W^T U W
//        DP = D, or the leading DP coordinates that the factors act on with
//        partial PaTH (M vanishes outside its leading DP x DP block)
//   al   float [BH][N][3][64][16]  diagonal-block raw logits as register image
//        of the scores S^T: tiles (query block w, key block mb) = (0,0),
//        (1,0), (1,1) (tile (0,1) lies wholly above the diagonal):
//        [tile][lane][r] = Al[32w + lane%32][32mb + acc_row(r, lane/32)]
//   gate float [BH][T]          a_t = -log2(e) * sum_{1<=s<=t} log f_s (FoX)
//   bnd  float2 [BH][N]         per key chunk, with the gate: (max_t a_t,
//        max_j |k~_j|^2 of the bf16 (or float32) ->K rows the scan reads),
//        inputs of the exact block skip; +inf where an input is not finite
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pathattn {

constexpr int kChunk = 64;
constexpr int kAlTiles = 3;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__host__ __device__ constexpr int acc_row(int r, int g) {
  return 8 * (r / 4) + 4 * g + (r % 4);
}

__host__ __device__ constexpr int frag_row(int s, int g, int t, int kpl) {
  return 32 * ((s * kpl + t) / 16) + acc_row((s * kpl + t) % 16, g);
}

// Elements of one chunk's kvm block (DP: the coordinates the factors act on).
__host__ __device__ constexpr int kvm_elems(int D, int DP) { return 2 * kChunk * D + DP * DP; }
__host__ __device__ constexpr int kvm_elems(int D) { return kvm_elems(D, D); }
// Floats of one chunk's register images.
__host__ __device__ constexpr int qa_floats(int D) { return kChunk * D; }
__host__ __device__ constexpr int al_floats() { return kAlTiles * 64 * 16; }
// Tile index of the diagonal-block image for (query block w, key block mb),
// mb <= w.
__host__ __device__ constexpr int al_tile(int w, int mb) { return w + mb; }

// Copies from global memory straight into LDS (lane l's bytes landing at
// lds + size * l, lds wave-uniform), written as assembly so that the compiler,
// which does not see them, places no wait for them before the wave's later LDS
// reads: through the intrinsic it waits for every outstanding copy before the
// first read it cannot tell apart from a copy's destination, which for a
// double buffer with a runtime index is every read of the other buffer.  The
// caller waits for its copies itself (vmcnt) and publishes them with a
// barrier before any wave reads them.  The compiler's own waits stay correct,
// only more conservative: it counts fewer outstanding operations than there
// are.  M0 (the LDS address) is a register the compiler reserves; the kernels
// that use these make no other use of M0 (no LDS copy intrinsics, messages or
// indexed register moves), as their generated code shows.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void copy16_to_lds(const void *gsrc, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void copy4_to_lds(const void *gsrc, unsigned lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gsrc), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop
// The LDS address of a pointer into shared memory, as a wave-uniform scalar.
__device__ __forceinline__ unsigned lds_addr(const void *p) {
  typedef __attribute__((address_space(3))) const void *lds_cptr;
  return __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)(lds_cptr)(p));
}

// Element strides over (batch, head, token) of a [B, H, T, row] tensor that
// a kernel reads or writes in place; the flat head index is bh = b * H + h.
struct TokStrides {
  long long b, h, t;
};
inline TokStrides dense_strides(int H, int T, int row) {
  return TokStrides{(long long)H * T * row, (long long)T * row, row};
}
// The forward's tensors as its kernels address them: inputs q, k, v, w, beta,
// logf and outputs out, lse.
struct FwdIo {
  int H;
  TokStrides q, k, v, w, beta, logf, out, lse;
};
inline FwdIo dense_io(int H, int T, int d) {
  const TokStrides vec = dense_strides(H, T, d), sca = dense_strides(H, T, 1);
  return FwdIo{H, vec, vec, vec, vec, sca, sca, vec, sca};
}

struct Layout {
  size_t qa, kvm, al, gate, bnd, klo, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline Layout make_layout(int B, int H, int T, int D, size_t esize, int DP) {
  const size_t BH = (size_t)B * H, N = (size_t)T / kChunk;
  Layout L;
  size_t off = 0;
  L.qa = off;
  off = align256(off + BH * N * qa_floats(D) * sizeof(float));
  L.kvm = off;
  off = align256(off + BH * N * kvm_elems(D, DP) * esize);
  L.al = off;
  off = align256(off + BH * N * al_floats() * sizeof(float));
  L.gate = off;
  off = align256(off + BH * T * sizeof(float));
  L.bnd = off;
  off = align256(off + BH * N * 2 * sizeof(float));
  // bf16: the rounding remainder of ->K (same blob order as ->K in the
  // operand block), written only for the precise scan
  L.klo = off;
  off = align256(off + (esize == 2 ? BH * T * D * esize : 0));
  L.total = off;
  return L;
}

// Launchers (return hipGetLastError() after the launch).
// io: how the inputs are addressed (the padded dense layout, or the caller's
// views when they are read in place: bf16 with whole chunks only).
hipError_t launch_gate_prefix(const float *logf, float *gate, int BH, int T, const FwdIo &io,
                              hipStream_t stream);
// DP: the leading coordinates the factors act on (D for PaTH on every
// coordinate; D / 2 for partial PaTH, whose w is not read beyond them).
// klo (bf16, may be null): also store ->K's rounding remainders there.
hipError_t launch_prep(int dtype, int D, int DP, const void *q, const void *k,
                       const void *v, const void *w, const float *beta,
                       float *qa, void *kvm, float *al, int BH, int T,
                       const FwdIo &io, hipStream_t stream, void *klo = nullptr);
hipError_t launch_chunk_bounds(int dtype, int D, int DP, const void *kvm,
                               const float *gate, float2 *bnd, int BH, int T,
                               hipStream_t stream);

// Arguments of the streaming scan.  skip != 0 enables the exact block skip
// with the gate (bnd must then hold the chunk bounds); skipped, if not null,
// receives += the number of (wave, key chunk) steps skipped.
struct StreamArgs {
  const float *qa;
  const void *kvm;
  const float *al;
  const float *gate;
  const float2 *bnd;
  int skip;
  unsigned long long *skipped;
  void *out;
  float *lse;
  int BH, T;
  float sl2;   // softmax scale times log2(e)
  int H;                // bh = b * H + h
  TokStrides so, sl;    // out and lse row (b, h, t) at b so.b + h so.h + t so.t
  const void *klo;      // bf16: ->K's rounding remainders; set: the precise scan
};
hipError_t launch_stream(int dtype, int D, int DP, bool fox, const StreamArgs &a,
                         hipStream_t stream);
hipError_t launch_unpack(int dtype, int D, const float *qa_ws, const void *kvm,
                         const float *al_ws, const float *gate, float *qa,
                         float *kb, float *m, float *al, float *lam, int BH,
                         int T, hipStream_t stream);

// A caller's [B, H, T, row] tensor as a view (pad.hip): row (b, h, t) starts at
// element (off_b + t) * s_tok + b * s_b + h * s_h, off_b = cu ? cu[b] : 0, and
// exists for t < (cu ? cu[b+1] - cu[b] : T).  cu is a device array of B + 1
// sequence starts (packed batches) or null.
struct RowView {
  const int *cu;
  long long s_b, s_h, s_tok;
};
// The view of a dense [B, H, T, row] tensor, row_elems elements per row.
inline RowView dense_view(int H, int T, int row_elems) {
  return RowView{nullptr, (long long)H * T * row_elems, (long long)T * row_elems, row_elems};
}
// gather: dst[b][h][t] (padded layout, Tp rows per head) = view row (b, h, t),
// zero beyond the row's sequence; scatter: view row (b, h, t) = src[b][h][t]
// for the rows that exist.  Rows are row_bytes bytes, copied in 16-byte words
// where view_rows_vec16 holds, else 4-byte words.
bool view_rows_vec16(const void *base, const RowView &view, int esize, int row_bytes);
hipError_t launch_view_rows(bool gather, const void *src, void *dst, const RowView &view, int B,
                            int H, int T, int Tp, int esize, int row_bytes, hipStream_t stream);

// Decoding with in-place key refinement (decode.hip).
size_t decode_partial_bytes(int BH, int T_cap, int D);
hipError_t launch_prefill_cache(int dtype, int kc_dtype, int D, const void *k, const void *v,
                                const void *w, const float *beta, const float *logf,
                                void *kcache, void *vcache, double *gcache, float *ws_kb,
                                float *ws_m, int BH, int L, int T_cap, hipStream_t s);
hipError_t launch_decode_step(int dtype, int kc_dtype, int D, const void *q, const void *k,
                              const void *v, const void *w, const float *beta,
                              const float *logf, void *kcache, void *vcache, double *gcache,
                              void *out, float *lse, float *part, int BH, int t, int T_cap,
                              float sl2, hipStream_t s);

// Backward pass (backward.hip, bwd_sweep.hip).
//
// The quadratic sweep runs over windows of query chunks, the last window
// first: window w holds query chunks [lo, hi) with lo = 1 + w*W and
// hi = min(N, lo + W), and the key levels c in [lo - 1, hi) of every earlier
// key chunk.  The last window's level pass is the whole walk, which also
// keeps float32 checkpoints at the levels lo - 1 of the other windows (but
// the first); each of those walks its own levels from there, so a head holds
// one window of levels instead of all N(N-1)/2 of them.  Up to 33 chunks run
// as one window (no checkpoints) by default; a caller that gives the
// backward more workspace gets longer windows (window > 0: that many query
// chunks, at most N - 1; window <= 0: the default).
constexpr int kBwdWindowMin = 16;
struct BwdPlan {
  int N, W, nwin;          // chunks, window length (query chunks), windows
  size_t win_blocks;       // 64-key level blocks of the largest window, per head
  size_t ckpt_blocks;      // float32 64-key checkpoint blocks per head
  int slots;               // dM partial slots per head: window length + 1
};
BwdPlan bwd_plan(int T, int window);
// Workspace offsets in bytes.  adj (the per-chunk adjoint scratch, used only
// after the sweep) shares its bytes with the sweep's buffers (levels, levt,
// ckpt, dmpart, gstate).
struct BwdLayout {
  size_t kb, m, al, lam, dvec, levels, dmpart, dv, dlam, dqa, dkb, dm, dal, saved, adj, qae, qat,
      nm, nmt, dot, levt, qimg, oimg, mimg, qst, ckpt, gstate, kn2, zhi, qagg, kmin, total;
  // the saved per-chunk matrices have bytes of their own (one window), so
  // they need not be computed again after the sweep
  bool saved_kept;
};
BwdLayout bwd_layout(int B, int H, int T, int D, int dtype, int window);
size_t bwd_dmpart_floats(int dtype, int BH, int T, int D, int window);

// The quadratic part (bwd_sweep.hip): key levels, dQa (+ dLambda row sums),
// dKb, dV (+= onto the diagonal part), dLambda column sums, dM.
struct SweepArgs {
  const float *kb, *m;
  const void *qae, *qat, *nm, *nmt, *dot;   // input-dtype copies: Qa rows, Qa^T, -M, -M^T, dO^T
  void *levt;                               // key levels transposed, [D][64] per (level, chunk)
  // bf16, d = 64 only: per-chunk LDS images of the dk kernel's operands
  const void *qimg, *oimg, *mimg, *qst;
  const void *dout, *v;
  const float *lse, *dlse, *dvec, *lam;
  void *levels;
  float *dmpart, *dqa, *dkb, *dv, *dlam, *dm;
  float *ckpt, *gstate;                     // level checkpoints, Gamma between windows
  // exact forget-gate skip (bf16, d = 128): a block of 32 keys against a query
  // chunk whose weights exp(s - lse) all underflow to zero is left out
  float *kn2;          // per level block and key half: max row |Khat|^2 (bf16 values)
  const float2 *qagg;  // per query chunk: (max |Qa_q|^2, max (Lambda_q - lse_q))
  const float *kmin;   // per key chunk half: min Lambda over its 32 keys
  // per (head, group of key chunks): dM partials of the transitions m >= zhi
  // are zero and not written (the dk walk skipped those steps whole); then,
  // at zbad = zhi + BH * N, per head: 1 if a stored level is not finite
  int *zhi;
  int skip;
  float scale;
  int BH, T, window;
};
hipError_t launch_bwd_sweep(int dtype, int D, bool fox, const SweepArgs &a, hipStream_t s);

// LDS images of the bf16 d = 64 dk kernel, per 64-token chunk.  A 64 x 64
// matrix X in "fragment order" is the matrix-core A operand of a product that
// contracts X's row index against accumulator registers: blob (mt, s) of 64
// lanes x 8 values, lane l holding X[frag_row(s, l/32, t)][32 mt + l%32], t < 8
// (mimg_index below).  qimg: Qa rows [64 q][64 d] padded to kImgPitch, then
// Qa in fragment order; oimg: the same for dO; mimg: -M^T in fragment order
// (X = -M, i.e. lane l holds -M[frag_row(s, l/32, t)][32 mt + l%32]); qst:
// float4 (lse, rowdot(dO, O), dlse, Lambda) per query.
constexpr int kImgPitch = 72;
constexpr int kQImgElems = 64 * kImgPitch + 64 * 64;
constexpr int kMImgElems = 64 * 64;
// Position of X[a][b] (64 x 64) in the fragment-order image.
__host__ __device__ inline int mimg_index(int a, int b) {
  const int u = a / 32, w = a % 32;
  const int r = 4 * (w / 8) + (w % 4), g = (w / 4) & 1;
  const int rg = 16 * u + r, s = rg >> 3, t = rg & 7;
  const int lane = 32 * g + (b % 32), mt = b / 32;
  return (mt * 4 + s) * 512 + lane * 8 + t;
}

struct BwdArgs {
  const void *q, *k, *v, *w;
  const float *beta, *logf;
  const void *out;
  const float *lse;
  const void *dout;
  const float *dlse;
  void *dq, *dk, *dv, *dw;
  float *dbeta, *dlogf;
  int B, H, T;
  float scale;
  int window;   // query chunks per window of the sweep (bwd_plan)
  int skip;     // exact forget-gate skip allowed (not PATH_ATTN_NO_SKIP)
};
hipError_t launch_bwd(int dtype, int D, const BwdArgs &a, void *workspace, hipStream_t s);

// The w / beta producer (producer.hip), bf16: x [B][T][Dm], Wd [R][Dm],
// Wu [H d][R], cw [H d][3] (float32, oldest tap first), u [H][Dm], ub [H]
// (float32) -> w [B][H][T][d] (bf16), beta [B][H][T] (float32).
struct WbetaArgs {
  const void *x, *wd, *wu, *u;
  const float *cw, *ub;
  void *w;
  float *beta;
  int B, T, Dm, R, H, d;
};
int wbeta_tiles(int T);   // blocks per batch row
hipError_t launch_wbeta(const WbetaArgs &a, hipStream_t s);

}  // namespace pathattn
