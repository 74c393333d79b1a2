// api.hip -- the C ABI of libpath_attn (see include/path_attn.h).
//
// Host side only: argument validation (before any HIP call), workspace
// carving, and the in-order launches on the caller's stream.
#include <atomic>
#include <mutex>

#include "path_attn.h"
#include "path_attn_internal.h"

using namespace pathattn;

namespace {

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

size_t elem_size(int dtype) { return dtype == PATH_ATTN_BF16 ? 2 : 4; }

// Lengths are padded to whole 64-token chunks (see pad.hip).
int padded(int T) { return (T + kChunk - 1) / kChunk * kChunk; }

// Shape/dtype checks shared by every entry point.
int check_shape(int B, int H, int T, int d, int dtype) {
  if (B <= 0 || H <= 0 || T <= 0 || d <= 0) return PATH_ATTN_EINVAL;
  if (dtype != PATH_ATTN_F32 && dtype != PATH_ATTN_BF16) return PATH_ATTN_EINVAL;
  if (d != 64 && d != 128) return PATH_ATTN_EUNSUPPORTED;
  const unsigned long long elems = (unsigned long long)B * H * padded(T) * d;
  if (elems >= (1ull << 31)) return PATH_ATTN_EUNSUPPORTED;
  // grid size of one block per (b, h, chunk) must fit in a 32-bit launch
  if ((unsigned long long)B * H * (padded(T) / kChunk) >= (1ull << 31)) return PATH_ATTN_EUNSUPPORTED;
  return PATH_ATTN_OK;
}

// Workspace: the per-chunk layout at the padded length, then, when T is not a
// multiple of 64 or the tensors are general views, zero-padded staging copies
// of the inputs and outputs.
struct FullLayout {
  Layout base;
  bool staged;
  size_t q, k, v, w, beta, logf, out, lse, total;
};

// dp: the coordinates the factors act on (d, or d / 2 for partial PaTH); the
// layout with dp = d is the largest.
FullLayout full_layout(int B, int H, int T, int d, int dtype, bool views = false, int dp = 0) {
  const int Tp = padded(T);
  const size_t e = elem_size(dtype);
  FullLayout F{};
  F.base = make_layout(B, H, Tp, d, e, dp > 0 ? dp : d);
  F.staged = views || Tp != T;
  size_t off = F.base.total;
  if (F.staged) {
    const size_t rows = (size_t)B * H * Tp;
    size_t *vecs[] = {&F.q, &F.k, &F.v, &F.w};
    for (size_t *o : vecs) {
      *o = off;
      off = align256(off + rows * d * e);
    }
    F.beta = off;
    off = align256(off + rows * 4);
    F.logf = off;
    off = align256(off + rows * 4);
    F.out = off;
    off = align256(off + rows * d * e);
    F.lse = off;
    off = align256(off + rows * 4);
  }
  F.total = off;
  return F;
}

// Views of the forward tensors, in the order q, k, v, w, out, beta, logf, lse.
struct FwdViews {
  RowView v[8];
};

TokStrides tok_strides(const RowView &v) { return TokStrides{v.s_b, v.s_h, v.s_tok}; }

FwdViews dense_fwd_views(int H, int T, int d) {
  FwdViews V;
  for (int i = 0; i < 8; ++i) V.v[i] = dense_view(H, T, i < 5 ? d : 1);
  return V;
}

int check_inputs(const void *q, const void *k, const void *v, const void *w,
                 const float *beta, const float *logf, void *workspace,
                 size_t workspace_bytes, int B, int H, int T, int d,
                 int dtype) {
  const int st = check_shape(B, H, T, d, dtype);
  if (st != PATH_ATTN_OK) return st;
  if (!q || !k || !v || !w || !beta || !workspace) return PATH_ATTN_EINVAL;
  const void *ptrs[] = {q, k, v, w, beta};
  for (const void *p : ptrs)
    if (!aligned(p, 16)) return PATH_ATTN_EINVAL;
  if (logf && !aligned(logf, 16)) return PATH_ATTN_EINVAL;
  if (!aligned(workspace, 256)) return PATH_ATTN_EINVAL;
  if (workspace_bytes < full_layout(B, H, T, d, dtype).total) return PATH_ATTN_EINVAL;
  return PATH_ATTN_OK;
}

// scale > 0 is used as given, 0 selects 1/sqrt(d); anything else is invalid
// (the scan takes the block max on the raw scores, which needs scale > 0).
bool scale_ok(float scale) { return scale == 0.f || (scale > 0.f && scale < INFINITY); }
float scale_of(float scale, int d) { return scale > 0.f ? scale : 1.f / sqrtf((float)d); }

struct Carved {
  float *qa;
  void *kvm;
  float *al;
  float *gate;
  float2 *bnd;
  char *base;
  FullLayout F;
  int dp;
  void *klo;   // ->K remainders for the precise scan (bf16 with PATH_ATTN_PRECISE), else null
};

Carved carve(void *workspace, int B, int H, int T, int d, int dtype, bool views = false,
             int dp = 0, unsigned flags = 0) {
  const FullLayout F = full_layout(B, H, T, d, dtype, views, dp);
  char *base = static_cast<char *>(workspace);
  const bool precise = dtype == PATH_ATTN_BF16 && (flags & PATH_ATTN_PRECISE);
  return Carved{reinterpret_cast<float *>(base + F.base.qa), base + F.base.kvm,
                reinterpret_cast<float *>(base + F.base.al),
                reinterpret_cast<float *>(base + F.base.gate),
                reinterpret_cast<float2 *>(base + F.base.bnd), base, F, dp > 0 ? dp : d,
                precise ? base + F.base.klo : nullptr};
}

// The streaming scan at the padded length; with staging into the staging
// outputs, then each existing row written to the caller's out and lse views.
int run_stream(const Carved &ws, bool gate, unsigned flags,
               unsigned long long *skipped, void *out, float *lse, int B, int H,
               int T, int d, int dtype, float scale, const FwdViews &views, hipStream_t s,
               bool in_place = false) {
  const int Tp = padded(T);
  StreamArgs a;
  a.qa = ws.qa;
  a.kvm = ws.kvm;
  a.al = ws.al;
  a.gate = ws.gate;
  a.bnd = ws.bnd;
  a.skip = gate && !(flags & PATH_ATTN_NO_SKIP);
  a.skipped = skipped;
  a.klo = ws.klo;
  const bool staged = ws.F.staged && !in_place;
  a.out = staged ? static_cast<void *>(ws.base + ws.F.out) : out;
  a.lse = staged ? reinterpret_cast<float *>(ws.base + ws.F.lse) : lse;
  a.BH = B * H;
  a.T = Tp;
  a.sl2 = 1.4426950408889634f * scale_of(scale, d);
  a.H = H;
  a.so = in_place ? tok_strides(views.v[4]) : dense_strides(H, Tp, d);
  a.sl = in_place ? tok_strides(views.v[7]) : dense_strides(H, Tp, 1);
  if (launch_stream(dtype, d, ws.dp, gate, a, s) != hipSuccess) return PATH_ATTN_EHIP;
  if (staged) {
    const int e = (int)elem_size(dtype);
    if (launch_view_rows(false, a.out, out, views.v[4], B, H, T, Tp, e, d * e, s) != hipSuccess ||
        launch_view_rows(false, a.lse, lse, views.v[7], B, H, T, Tp, 4, 4, s) != hipSuccess)
      return PATH_ATTN_EHIP;
  }
  return PATH_ATTN_OK;
}

// Enqueue the gate prefix (if any) and the chunk preparation, at the padded
// length (inputs first gathered into the zero-padded staging when staged).
int run_prep(const void *q, const void *k, const void *v, const void *w,
             const float *beta, const float *logf, const Carved &ws, int B, int H,
             int T, int d, int dtype, const FwdViews &views, hipStream_t s,
             bool in_place = false) {
  const int Tp = padded(T), BH = B * H;
  FwdIo io = dense_io(H, Tp, d);
  if (in_place) {   // the kernels address the caller's views directly
    io.q = tok_strides(views.v[0]);
    io.k = tok_strides(views.v[1]);
    io.v = tok_strides(views.v[2]);
    io.w = tok_strides(views.v[3]);
    io.out = tok_strides(views.v[4]);
    io.beta = tok_strides(views.v[5]);
    io.logf = tok_strides(views.v[6]);
    io.lse = tok_strides(views.v[7]);
  } else if (ws.F.staged) {
    const int e = (int)elem_size(dtype);
    char *b = ws.base;
    const void *src[] = {q, k, v, w};
    const size_t dst[] = {ws.F.q, ws.F.k, ws.F.v, ws.F.w};
    for (int i = 0; i < 4; ++i)
      if (launch_view_rows(true, src[i], b + dst[i], views.v[i], B, H, T, Tp, e, d * e, s) !=
          hipSuccess)
        return PATH_ATTN_EHIP;
    if (launch_view_rows(true, beta, b + ws.F.beta, views.v[5], B, H, T, Tp, 4, 4, s) !=
        hipSuccess)
      return PATH_ATTN_EHIP;
    if (logf &&
        launch_view_rows(true, logf, b + ws.F.logf, views.v[6], B, H, T, Tp, 4, 4, s) !=
            hipSuccess)
      return PATH_ATTN_EHIP;
    q = b + ws.F.q;
    k = b + ws.F.k;
    v = b + ws.F.v;
    w = b + ws.F.w;
    beta = reinterpret_cast<const float *>(b + ws.F.beta);
    if (logf) logf = reinterpret_cast<const float *>(b + ws.F.logf);
  }
  if (logf && launch_gate_prefix(logf, ws.gate, BH, Tp, io, s) != hipSuccess)
    return PATH_ATTN_EHIP;
  if (launch_prep(dtype, d, ws.dp, q, k, v, w, beta, ws.qa, ws.kvm, ws.al, BH, Tp, io, s,
                  ws.klo) != hipSuccess)
    return PATH_ATTN_EHIP;
  if (logf &&
      launch_chunk_bounds(dtype, d, ws.dp, ws.kvm, ws.gate, ws.bnd, BH, Tp, s) != hipSuccess)
    return PATH_ATTN_EHIP;
  return PATH_ATTN_OK;
}

}  // namespace

extern "C" size_t path_attn_workspace_bytes(int B, int H, int T, int d, int dtype) {
  if (check_shape(B, H, T, d, dtype) != PATH_ATTN_OK) return 0;
  return full_layout(B, H, T, d, dtype).total;
}

extern "C" int path_attn_fwd_ex(const void *q, const void *k, const void *v,
                                const void *w, const float *beta, const float *logf,
                                void *out, float *lse, int B, int H, int T, int d,
                                int dtype, float scale, unsigned flags, void *workspace,
                                size_t workspace_bytes, void *stream) {
  int st = check_inputs(q, k, v, w, beta, logf, workspace, workspace_bytes, B,
                        H, T, d, dtype);
  if (st != PATH_ATTN_OK) return st;
  if (!out || !lse) return PATH_ATTN_EINVAL;
  if (!aligned(out, 16) || !aligned(lse, 16)) return PATH_ATTN_EINVAL;
  if (!scale_ok(scale) || (flags & ~(unsigned)(PATH_ATTN_NO_SKIP | PATH_ATTN_PRECISE))) return PATH_ATTN_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Carved ws = carve(workspace, B, H, T, d, dtype, false, 0, flags);
  const FwdViews views = dense_fwd_views(H, T, d);
  st = run_prep(q, k, v, w, beta, logf, ws, B, H, T, d, dtype, views, s);
  if (st != PATH_ATTN_OK) return st;
  return run_stream(ws, logf != nullptr, flags, nullptr, out, lse, B, H, T, d, dtype, scale,
                    views, s);
}

extern "C" int path_attn_fwd(const void *q, const void *k, const void *v,
                             const void *w, const float *beta, const float *logf,
                             void *out, float *lse, int B, int H, int T, int d,
                             int dtype, void *workspace, size_t workspace_bytes,
                             void *stream) {
  return path_attn_fwd_ex(q, k, v, w, beta, logf, out, lse, B, H, T, d, dtype, 0.f, 0u,
                          workspace, workspace_bytes, stream);
}

extern "C" int path_attn_fwd_partial(const void *q, const void *k, const void *v,
                                     const void *w, const float *beta, const float *logf,
                                     void *out, float *lse, int B, int H, int T, int d,
                                     int d_path, int dtype, float scale, unsigned flags,
                                     void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_shape(B, H, T, d, dtype);
  if (st != PATH_ATTN_OK) return st;
  if (d_path <= 0 || d_path > d) return PATH_ATTN_EINVAL;
  if (d_path != d && 2 * d_path != d) return PATH_ATTN_EUNSUPPORTED;
  if (!q || !k || !v || !w || !beta || !out || !lse || !workspace) return PATH_ATTN_EINVAL;
  const void *ptrs[] = {q, k, v, w, beta, out, lse};
  for (const void *p : ptrs)
    if (!aligned(p, 16)) return PATH_ATTN_EINVAL;
  if (logf && !aligned(logf, 16)) return PATH_ATTN_EINVAL;
  if (!aligned(workspace, 256) ||
      workspace_bytes < full_layout(B, H, T, d, dtype, false, d_path).total)
    return PATH_ATTN_EINVAL;
  if (!scale_ok(scale) || (flags & ~(unsigned)(PATH_ATTN_NO_SKIP | PATH_ATTN_PRECISE))) return PATH_ATTN_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Carved ws = carve(workspace, B, H, T, d, dtype, false, d_path, flags);
  const FwdViews views = dense_fwd_views(H, T, d);
  st = run_prep(q, k, v, w, beta, logf, ws, B, H, T, d, dtype, views, s);
  if (st != PATH_ATTN_OK) return st;
  return run_stream(ws, logf != nullptr, flags, nullptr, out, lse, B, H, T, d, dtype, scale,
                    views, s);
}

// ---- the forward without a caller workspace ----------------------------------
//
// Its workspace is `scratch`, a fixed array in the library's device memory.
// In host code the name `scratch` stands for a host-side shadow, not a device
// address; the device address of each GPU's copy is looked up once per device
// with hipGetSymbolAddress and only that address is handed to kernels.  No
// part of the forward's workspace has to start at zero (every region a call
// reads is written earlier in the same call, padded staging rows included), so
// nothing is cleared between calls.

namespace {

__device__ __align__(256) unsigned char scratch[PATH_ATTN_NOALLOC_MAX_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on `dev` (looked up on first use, with that
// device current, and kept for the life of the process).
int scratch_address(int dev, void **addr) {
  if (dev < 0 || dev >= kMaxDevices) return PATH_ATTN_EUNSUPPORTED;
  void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      int cur = -1;
      if (hipGetDevice(&cur) != hipSuccess) return PATH_ATTN_EHIP;
      if (cur != dev && hipSetDevice(dev) != hipSuccess) return PATH_ATTN_EHIP;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (cur != dev && hipSetDevice(cur) != hipSuccess) return PATH_ATTN_EHIP;
      if (e != hipSuccess || !p) return PATH_ATTN_EHIP;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *addr = p;
  return PATH_ATTN_OK;
}

}  // namespace

extern "C" int path_attn_fwd_noalloc(const void *q, const void *k, const void *v,
                                     const void *w, const float *beta, const float *logf,
                                     void *out, float *lse, int B, int H, int T, int d,
                                     int dtype, float scale, unsigned flags, void *stream) {
  // argument checks first, before any HIP call
  int st = check_shape(B, H, T, d, dtype);
  if (st != PATH_ATTN_OK) return st;
  if (full_layout(B, H, T, d, dtype).total > (size_t)PATH_ATTN_NOALLOC_MAX_BYTES)
    return PATH_ATTN_EINVAL;
  if (!q || !k || !v || !w || !beta || !out || !lse) return PATH_ATTN_EINVAL;
  const void *ptrs[] = {q, k, v, w, beta, out, lse};
  for (const void *p : ptrs)
    if (!aligned(p, 16)) return PATH_ATTN_EINVAL;
  if (logf && !aligned(logf, 16)) return PATH_ATTN_EINVAL;
  if (!scale_ok(scale) || (flags & ~(unsigned)(PATH_ATTN_NO_SKIP | PATH_ATTN_PRECISE))) return PATH_ATTN_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = -1;
  if (s ? hipStreamGetDevice(s, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
    return PATH_ATTN_EHIP;
  void *ws_addr = nullptr;
  st = scratch_address(dev, &ws_addr);
  if (st != PATH_ATTN_OK) return st;
  const Carved ws = carve(ws_addr, B, H, T, d, dtype, false, 0, flags);
  const FwdViews views = dense_fwd_views(H, T, d);
  st = run_prep(q, k, v, w, beta, logf, ws, B, H, T, d, dtype, views, s);
  if (st != PATH_ATTN_OK) return st;
  return run_stream(ws, logf != nullptr, flags, nullptr, out, lse, B, H, T, d, dtype, scale,
                    views, s);
}

namespace {

// A caller-described view: a row start at a 4-byte boundary for every row
// (base pointer and each stride in bytes multiples of 4), strides >= 0 and
// below 2^40 elements.  The strides of an absent (null) optional tensor are
// not read.
bool view_ok(const void *p, const long long *st, size_t esize) {
  if (!p) return true;
  if (!aligned(p, 4)) return false;
  for (int i = 0; i < 3; ++i)
    if (st[i] < 0 || st[i] >= (1ll << 40) || (st[i] * (long long)esize) % 4 != 0) return false;
  return true;
}

RowView make_view(const long long *st, const int *cu) { return RowView{cu, st[0], st[1], st[2]}; }

// Whether the forward can address the views in place, without staging: bf16
// (its chunk preparation reads rows through the view strides; float32 does
// not), no packed sequences and whole chunks (no row needs zero padding), and
// every vector row (q, k, v, w, out) starting at a 16-byte boundary with a
// token pitch below 2^31 elements.  ptrs and strides in the order q, k, v, w,
// out, beta, logf, lse; the scalar views are already known to be usable.
bool in_place_ok(const void *const *ptrs, const long long *strides, const int *cu, int T,
                 int dtype) {
  if (cu || T % kChunk != 0 || dtype != 1) return false;
  for (int i = 0; i < 5; ++i) {
    if (!aligned(ptrs[i], 16)) return false;
    for (int j = 0; j < 3; ++j)
      if ((strides[3 * i + j] * 2) % 16 != 0) return false;
    if (strides[3 * i + 2] >= (1ll << 31)) return false;
  }
  return true;
}

}  // namespace

extern "C" size_t path_attn_varlen_workspace_bytes(int B, int H, int T, int d, int dtype) {
  if (check_shape(B, H, T, d, dtype) != PATH_ATTN_OK) return 0;
  return full_layout(B, H, T, d, dtype, true).total;
}

extern "C" int path_attn_fwd_varlen(const void *q, const void *k, const void *v, const void *w,
                                    const float *beta, const float *logf, void *out, float *lse,
                                    const long long *strides, const int *cu_seqlens, int B,
                                    int H, int T, int d, int dtype, float scale, unsigned flags,
                                    void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_shape(B, H, T, d, dtype);
  if (st != PATH_ATTN_OK) return st;
  if (!q || !k || !v || !w || !beta || !out || !lse || !strides || !workspace)
    return PATH_ATTN_EINVAL;
  if (!scale_ok(scale) || (flags & ~(unsigned)(PATH_ATTN_NO_SKIP | PATH_ATTN_PRECISE))) return PATH_ATTN_EINVAL;
  if (cu_seqlens && !aligned(cu_seqlens, 4)) return PATH_ATTN_EINVAL;
  const void *ptrs[] = {q, k, v, w, out, beta, logf, lse};
  const size_t e = elem_size(dtype);
  for (int i = 0; i < 8; ++i)
    if (!view_ok(ptrs[i], strides + 3 * i, i < 5 ? e : 4)) return PATH_ATTN_EINVAL;
  if (!aligned(workspace, 256) || workspace_bytes < full_layout(B, H, T, d, dtype, true).total)
    return PATH_ATTN_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Carved ws = carve(workspace, B, H, T, d, dtype, true, 0, flags);
  FwdViews views;
  for (int i = 0; i < 8; ++i) views.v[i] = make_view(strides + 3 * i, cu_seqlens);
  const bool direct = in_place_ok(ptrs, strides, cu_seqlens, T, dtype);
  st = run_prep(q, k, v, w, beta, logf, ws, B, H, T, d, dtype, views, s, direct);
  if (st != PATH_ATTN_OK) return st;
  return run_stream(ws, logf != nullptr, flags, nullptr, out, lse, B, H, T, d, dtype, scale,
                    views, s, direct);
}

extern "C" int path_attn_prepare(const void *q, const void *k, const void *v,
                                 const void *w, const float *beta,
                                 const float *logf, int B, int H, int T, int d,
                                 int dtype, void *workspace,
                                 size_t workspace_bytes, void *stream) {
  const int st = check_inputs(q, k, v, w, beta, logf, workspace,
                              workspace_bytes, B, H, T, d, dtype);
  if (st != PATH_ATTN_OK) return st;
  const Carved ws = carve(workspace, B, H, T, d, dtype);
  return run_prep(q, k, v, w, beta, logf, ws, B, H, T, d, dtype, dense_fwd_views(H, T, d),
                  static_cast<hipStream_t>(stream));
}

extern "C" int path_attn_stream_ex(const void *workspace, size_t workspace_bytes,
                                   int use_gate, float scale, unsigned flags,
                                   unsigned long long *skipped, void *out,
                                   float *lse, int B, int H, int T, int d,
                                   int dtype, void *stream) {
  const int st = check_shape(B, H, T, d, dtype);
  if (st != PATH_ATTN_OK) return st;
  if (!workspace || !out || !lse) return PATH_ATTN_EINVAL;
  if (use_gate != 0 && use_gate != 1) return PATH_ATTN_EINVAL;
  if (!scale_ok(scale)) return PATH_ATTN_EINVAL;
  // PATH_ATTN_PRECISE needs ->K's remainders, which only the one-shot calls write
  if (flags & ~(unsigned)PATH_ATTN_NO_SKIP) return PATH_ATTN_EINVAL;
  if (!aligned(workspace, 256) || !aligned(out, 16) || !aligned(lse, 16))
    return PATH_ATTN_EINVAL;
  if (skipped && !aligned(skipped, 8)) return PATH_ATTN_EINVAL;
  if (workspace_bytes < full_layout(B, H, T, d, dtype).total) return PATH_ATTN_EINVAL;
  const Carved ws = carve(const_cast<void *>(workspace), B, H, T, d, dtype);
  return run_stream(ws, use_gate == 1, flags, skipped, out, lse, B, H, T, d, dtype, scale,
                    dense_fwd_views(H, T, d), static_cast<hipStream_t>(stream));
}

extern "C" int path_attn_stream(const void *workspace, size_t workspace_bytes,
                                int use_gate, void *out, float *lse, int B,
                                int H, int T, int d, int dtype, void *stream) {
  return path_attn_stream_ex(workspace, workspace_bytes, use_gate, 0.f, 0u, nullptr,
                             out, lse, B, H, T, d, dtype, stream);
}

extern "C" int path_attn_chunk_prep(const void *q, const void *k, const void *v,
                                    const void *w, const float *beta,
                                    const float *logf, float *qa, float *kb,
                                    float *m, float *al, float *lam, int B,
                                    int H, int T, int d, int dtype,
                                    void *workspace, size_t workspace_bytes,
                                    void *stream) {
  int st = check_inputs(q, k, v, w, beta, logf, workspace, workspace_bytes, B,
                        H, T, d, dtype);
  if (st != PATH_ATTN_OK) return st;
  if (T % kChunk != 0) return PATH_ATTN_EUNSUPPORTED;   // whole chunks only
  float *outs[] = {qa, kb, m, al, lam};
  for (float *p : outs)
    if (p && !aligned(p, 16)) return PATH_ATTN_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const Carved ws = carve(workspace, B, H, T, d, dtype);
  const int BH = B * H;
  st = run_prep(q, k, v, w, beta, logf, ws, B, H, T, d, dtype, dense_fwd_views(H, T, d), s);
  if (st != PATH_ATTN_OK) return st;
  if (launch_unpack(dtype, d, ws.qa, ws.kvm, ws.al, logf ? ws.gate : nullptr,
                    qa, kb, m, al, logf ? lam : nullptr, BH, T, s) != hipSuccess)
    return PATH_ATTN_EHIP;
  return PATH_ATTN_OK;
}

// ---------------------------------------------------------------- backward

namespace {

// Backward workspace: the layout at the padded length, then, when T is not a
// multiple of 64 or the tensors are general views, zero-padded staging rows:
// q, k, v, w, out, dout and dq, dk, dv, dw (input dtype), beta, logf, lse,
// dlse and dbeta, dlogf (fp32).  Padded tokens have identity factors and zero
// q, k, v, dout, dlse and gate, and lse = 0: their logits are <= 0, so
// exp(s - lse) stays finite, and every gradient contribution they make is
// exactly zero.
struct BwdFull {
  size_t vec[10], sca[6], total;
  bool staged;
  int window;
};

BwdFull bwd_full(int B, int H, int T, int d, int dtype, bool views, int window) {
  const int Tp = padded(T);
  BwdFull F{};
  F.window = window;
  size_t off = bwd_layout(B, H, Tp, d, dtype, window).total;
  F.staged = views || Tp != T;
  if (F.staged) {
    const size_t rows = (size_t)B * H * Tp;
    for (size_t &o : F.vec) {
      o = off;
      off = align256(off + rows * d * elem_size(dtype));
    }
    for (size_t &o : F.sca) {
      o = off;
      off = align256(off + rows * 4);
    }
  }
  F.total = off;
  return F;
}

// The layout for a workspace of `bytes`: the sweep in one window when that
// fits, else in the longest windows of 128, 64, 32 or 16 query chunks that
// fit (total = 0 when not even the default fits).
BwdFull bwd_fit(int B, int H, int T, int d, int dtype, bool views, size_t bytes) {
  const int nq = padded(T) / kChunk - 1 > 1 ? padded(T) / kChunk - 1 : 1;
  const int cand[] = {nq, 128, 64, 32, kBwdWindowMin};
  for (int w : cand) {
    if (w > nq) continue;
    const BwdFull F = bwd_full(B, H, T, d, dtype, views, w);
    if (F.total <= bytes) return F;
  }
  const BwdFull F = bwd_full(B, H, T, d, dtype, views, 0);
  if (F.total <= bytes) return F;
  BwdFull none{};
  return none;
}

// Everything after argument checks: stage (gather) the inputs when staged,
// run the backward at the padded length, scatter the gradients.  views holds
// the 16 tensors in the order q, k, v, w, out, dout, dq, dk, dv, dw, beta,
// logf, lse, dlse, dbeta, dlogf.
int run_bwd(const void *q, const void *k, const void *v, const void *w, const float *beta,
            const float *logf, const void *out, const float *lse, const void *dout,
            const float *dlse, void *dq, void *dk, void *dv, void *dw, float *dbeta,
            float *dlogf, int B, int H, int T, int d, int dtype, float scale,
            const RowView *views, const BwdFull &F, void *workspace, hipStream_t s,
            unsigned flags = 0) {
  const int Tp = padded(T);
  char *ws = static_cast<char *>(workspace);
  BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.w = w;
  a.beta = beta;
  a.logf = logf;
  a.out = out;
  a.lse = lse;
  a.dout = dout;
  a.dlse = dlse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dw = dw;
  a.dbeta = dbeta;
  a.dlogf = logf ? dlogf : nullptr;
  a.B = B;
  a.H = H;
  a.T = Tp;
  a.scale = scale_of(scale, d);
  a.window = F.window;
  a.skip = (flags & PATH_ATTN_NO_SKIP) ? 0 : 1;
  const int e = (int)elem_size(dtype), row = d * e;
  if (F.staged) {   // gather the inputs at the padded length
    const void *vin[] = {q, k, v, w, out, dout};
    const void **vdst[] = {&a.q, &a.k, &a.v, &a.w, &a.out, &a.dout};
    for (int i = 0; i < 6; ++i) {
      if (launch_view_rows(true, vin[i], ws + F.vec[i], views[i], B, H, T, Tp, e, row, s) !=
          hipSuccess)
        return PATH_ATTN_EHIP;
      *vdst[i] = ws + F.vec[i];
    }
    const float *sin[] = {beta, logf, lse, dlse};
    const float **sdst[] = {&a.beta, &a.logf, &a.lse, &a.dlse};
    for (int i = 0; i < 4; ++i) {
      if (!sin[i]) continue;
      if (launch_view_rows(true, sin[i], ws + F.sca[i], views[10 + i], B, H, T, Tp, 4, 4, s) !=
          hipSuccess)
        return PATH_ATTN_EHIP;
      *sdst[i] = reinterpret_cast<const float *>(ws + F.sca[i]);
    }
    a.dq = ws + F.vec[6];
    a.dk = ws + F.vec[7];
    a.dv = ws + F.vec[8];
    a.dw = ws + F.vec[9];
    a.dbeta = reinterpret_cast<float *>(ws + F.sca[4]);
    if (logf) a.dlogf = reinterpret_cast<float *>(ws + F.sca[5]);
  }
  if (launch_bwd(dtype, d, a, workspace, s) != hipSuccess) return PATH_ATTN_EHIP;
  if (F.staged) {   // scatter the gradients of the rows that exist
    void *vout[] = {dq, dk, dv, dw};
    for (int i = 0; i < 4; ++i)
      if (launch_view_rows(false, ws + F.vec[6 + i], vout[i], views[6 + i], B, H, T, Tp, e, row,
                           s) != hipSuccess)
        return PATH_ATTN_EHIP;
    if (launch_view_rows(false, ws + F.sca[4], dbeta, views[14], B, H, T, Tp, 4, 4, s) !=
        hipSuccess)
      return PATH_ATTN_EHIP;
    if (logf && launch_view_rows(false, ws + F.sca[5], dlogf, views[15], B, H, T, Tp, 4, 4, s) !=
                    hipSuccess)
      return PATH_ATTN_EHIP;
  }
  return PATH_ATTN_OK;
}

}  // namespace

extern "C" size_t path_attn_bwd_workspace_bytes(int B, int H, int T, int d, int dtype) {
  if (check_shape(B, H, T, d, dtype) != PATH_ATTN_OK) return 0;
  return bwd_full(B, H, T, d, dtype, false, 0).total;
}

extern "C" size_t path_attn_bwd_workspace_bytes_window(int B, int H, int T, int d, int dtype,
                                                       int window) {
  if (check_shape(B, H, T, d, dtype) != PATH_ATTN_OK) return 0;
  const int nq = padded(T) / kChunk - 1 > 1 ? padded(T) / kChunk - 1 : 1;
  return bwd_full(B, H, T, d, dtype, false, window > 0 ? window : nq).total;
}

extern "C" size_t path_attn_bwd_varlen_workspace_bytes(int B, int H, int T, int d, int dtype) {
  if (check_shape(B, H, T, d, dtype) != PATH_ATTN_OK) return 0;
  return bwd_full(B, H, T, d, dtype, true, 0).total;
}

extern "C" int path_attn_bwd_ex(const void *q, const void *k, const void *v, const void *w,
                                const float *beta, const float *logf, const void *out,
                                const float *lse, const void *dout, const float *dlse, void *dq,
                                void *dk, void *dv, void *dw, float *dbeta, float *dlogf, int B,
                                int H, int T, int d, int dtype, float scale, unsigned flags,
                                void *workspace, size_t workspace_bytes, void *stream) {
  const int st = check_shape(B, H, T, d, dtype);
  if (st != PATH_ATTN_OK) return st;
  if (!scale_ok(scale) || (flags & ~(unsigned)PATH_ATTN_NO_SKIP)) return PATH_ATTN_EINVAL;
  const void *need[] = {q, k, v, w, beta, out, lse, dout, dq, dk, dv, dw, dbeta, workspace};
  for (const void *p : need)
    if (!p) return PATH_ATTN_EINVAL;
  if (logf && !dlogf) return PATH_ATTN_EINVAL;
  const void *all[] = {q, k, v, w, beta, logf, out, lse, dout, dlse, dq, dk, dv, dw, dbeta, dlogf};
  for (const void *p : all)
    if (p && !aligned(p, 16)) return PATH_ATTN_EINVAL;
  const BwdFull F = bwd_fit(B, H, T, d, dtype, false, workspace_bytes);
  if (!aligned(workspace, 256) || F.total == 0) return PATH_ATTN_EINVAL;
  RowView views[16];
  for (int i = 0; i < 16; ++i) views[i] = dense_view(H, T, i < 10 ? d : 1);
  return run_bwd(q, k, v, w, beta, logf, out, lse, dout, dlse, dq, dk, dv, dw, dbeta, dlogf, B,
                 H, T, d, dtype, scale, views, F, workspace, static_cast<hipStream_t>(stream),
                 flags);
}

extern "C" int path_attn_bwd(const void *q, const void *k, const void *v, const void *w,
                             const float *beta, const float *logf, const void *out,
                             const float *lse, const void *dout, const float *dlse, void *dq,
                             void *dk, void *dv, void *dw, float *dbeta, float *dlogf, int B,
                             int H, int T, int d, int dtype, float scale, void *workspace,
                             size_t workspace_bytes, void *stream) {
  return path_attn_bwd_ex(q, k, v, w, beta, logf, out, lse, dout, dlse, dq, dk, dv, dw, dbeta,
                          dlogf, B, H, T, d, dtype, scale, 0u, workspace, workspace_bytes, stream);
}

extern "C" int path_attn_bwd_varlen(const void *q, const void *k, const void *v, const void *w,
                                    const float *beta, const float *logf, const void *out,
                                    const float *lse, const void *dout, const float *dlse,
                                    void *dq, void *dk, void *dv, void *dw, float *dbeta,
                                    float *dlogf, const long long *strides,
                                    const int *cu_seqlens, int B, int H, int T, int d, int dtype,
                                    float scale, void *workspace, size_t workspace_bytes,
                                    void *stream) {
  const int st = check_shape(B, H, T, d, dtype);
  if (st != PATH_ATTN_OK) return st;
  if (!scale_ok(scale)) return PATH_ATTN_EINVAL;
  const void *need[] = {q, k, v, w, beta, out, lse, dout, dq, dk, dv, dw, dbeta, workspace,
                        strides};
  for (const void *p : need)
    if (!p) return PATH_ATTN_EINVAL;
  if (logf && !dlogf) return PATH_ATTN_EINVAL;
  if (cu_seqlens && !aligned(cu_seqlens, 4)) return PATH_ATTN_EINVAL;
  const void *all[] = {q, k, v, w, out, dout, dq, dk, dv, dw,
                       beta, logf, lse, dlse, dbeta, dlogf};
  const size_t e = elem_size(dtype);
  for (int i = 0; i < 16; ++i)
    if (!view_ok(all[i], strides + 3 * i, i < 10 ? e : 4)) return PATH_ATTN_EINVAL;
  const BwdFull F = bwd_fit(B, H, T, d, dtype, true, workspace_bytes);
  if (!aligned(workspace, 256) || F.total == 0) return PATH_ATTN_EINVAL;
  RowView views[16];
  for (int i = 0; i < 16; ++i) views[i] = make_view(strides + 3 * i, cu_seqlens);
  return run_bwd(q, k, v, w, beta, logf, out, lse, dout, dlse, dq, dk, dv, dw, dbeta, dlogf, B,
                 H, T, d, dtype, scale, views, F, workspace, static_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------- decoding

namespace {

int check_decode_shape(int B, int H, int T_cap, int d, int dtype, int kc_dtype) {
  if (B <= 0 || H <= 0 || T_cap <= 0 || d <= 0) return PATH_ATTN_EINVAL;
  if ((dtype != PATH_ATTN_F32 && dtype != PATH_ATTN_BF16) ||
      (kc_dtype != PATH_ATTN_F32 && kc_dtype != PATH_ATTN_BF16))
    return PATH_ATTN_EINVAL;
  if (d != 64 && d != 128) return PATH_ATTN_EUNSUPPORTED;
  if ((unsigned long long)B * H * T_cap * d >= (1ull << 31)) return PATH_ATTN_EUNSUPPORTED;
  if ((unsigned long long)B * H >= 65536ull) return PATH_ATTN_EUNSUPPORTED;
  return PATH_ATTN_OK;
}

struct PrefillLayout {
  size_t kb, m, total;
};

PrefillLayout prefill_layout(int B, int H, int L, int d) {
  const size_t BH = (size_t)B * H, N = (size_t)L / kChunk;
  PrefillLayout P;
  P.kb = 0;
  P.m = align256(BH * L * d * sizeof(float));
  P.total = P.m + align256(BH * N * d * d * sizeof(float));
  return P;
}

}  // namespace

extern "C" size_t path_attn_prefill_workspace_bytes(int B, int H, int L, int d) {
  if (B <= 0 || H <= 0 || L < 0 || (d != 64 && d != 128) || L % kChunk != 0) return 0;
  return prefill_layout(B, H, L, d).total;
}

extern "C" int path_attn_prefill_cache(const void *k, const void *v, const void *w,
                                       const float *beta, const float *logf, void *kcache,
                                       void *vcache, double *gcache, int B, int H, int L,
                                       int T_cap, int d, int dtype, int kc_dtype,
                                       void *workspace, size_t workspace_bytes, void *stream) {
  int st = check_decode_shape(B, H, T_cap, d, dtype, kc_dtype);
  if (st != PATH_ATTN_OK) return st;
  if (L < 0 || L > T_cap) return PATH_ATTN_EINVAL;
  if (L % kChunk != 0) return PATH_ATTN_EUNSUPPORTED;
  if (!kcache || !vcache) return PATH_ATTN_EINVAL;
  if (logf && !gcache) return PATH_ATTN_EINVAL;
  if (L > 0 && (!k || !v || !w || !beta)) return PATH_ATTN_EINVAL;
  const void *ptrs[] = {k, v, w, beta, logf, kcache, vcache, gcache};
  for (const void *p : ptrs)
    if (p && !aligned(p, 16)) return PATH_ATTN_EINVAL;
  const PrefillLayout P = prefill_layout(B, H, L, d);
  if (L > 0 && (!workspace || !aligned(workspace, 256) || workspace_bytes < P.total))
    return PATH_ATTN_EINVAL;
  if (L == 0) return PATH_ATTN_OK;
  char *base = static_cast<char *>(workspace);
  return launch_prefill_cache(dtype, kc_dtype, d, k, v, w, beta, logf, kcache, vcache, gcache,
                              reinterpret_cast<float *>(base + P.kb),
                              reinterpret_cast<float *>(base + P.m), B * H, L, T_cap,
                              static_cast<hipStream_t>(stream)) == hipSuccess
             ? PATH_ATTN_OK
             : PATH_ATTN_EHIP;
}

extern "C" size_t path_attn_decode_workspace_bytes(int B, int H, int T_cap, int d) {
  if (B <= 0 || H <= 0 || T_cap <= 0 || (d != 64 && d != 128)) return 0;
  return align256(decode_partial_bytes(B * H, T_cap, d));
}

extern "C" int path_attn_decode_step(const void *q, const void *k, const void *v, const void *w,
                                     const float *beta, const float *logf, void *kcache,
                                     void *vcache, double *gcache, int t, void *out, float *lse,
                                     int B, int H, int T_cap, int d, int dtype, int kc_dtype,
                                     float scale, void *workspace, size_t workspace_bytes,
                                     void *stream) {
  int st = check_decode_shape(B, H, T_cap, d, dtype, kc_dtype);
  if (st != PATH_ATTN_OK) return st;
  if (!scale_ok(scale)) return PATH_ATTN_EINVAL;
  if (t < 0 || t >= T_cap) return PATH_ATTN_EINVAL;
  if (!q || !k || !v || !w || !beta || !kcache || !vcache || !out || !lse || !workspace)
    return PATH_ATTN_EINVAL;
  if (logf && !gcache) return PATH_ATTN_EINVAL;
  // vectors are read 16 bytes at a time; the per-head scalars one at a time
  const void *vecs[] = {q, k, v, w, kcache, vcache, gcache, out};
  for (const void *p : vecs)
    if (p && !aligned(p, 16)) return PATH_ATTN_EINVAL;
  const void *scalars[] = {beta, logf, lse};
  for (const void *p : scalars)
    if (p && !aligned(p, 4)) return PATH_ATTN_EINVAL;
  if (!aligned(workspace, 256) ||
      workspace_bytes < path_attn_decode_workspace_bytes(B, H, T_cap, d))
    return PATH_ATTN_EINVAL;
  return launch_decode_step(dtype, kc_dtype, d, q, k, v, w, beta, logf, kcache, vcache, gcache,
                            out, lse, static_cast<float *>(workspace), B * H, t, T_cap,
                            1.4426950408889634f * scale_of(scale, d),
                            static_cast<hipStream_t>(stream)) == hipSuccess
             ? PATH_ATTN_OK
             : PATH_ATTN_EHIP;
}

extern "C" int path_attn_wbeta(const void *x, const void *wd, const void *wu, const float *cw,
                               const void *u, const float *ub, void *w, float *beta, int B,
                               int T, int Dm, int R, int H, int d, int dtype, void *stream) {
  if (B <= 0 || T <= 0 || Dm <= 0 || R <= 0 || H <= 0 || d <= 0) return PATH_ATTN_EINVAL;
  if (dtype != PATH_ATTN_F32 && dtype != PATH_ATTN_BF16) return PATH_ATTN_EINVAL;
  if (dtype != PATH_ATTN_BF16 || (d != 64 && d != 128)) return PATH_ATTN_EUNSUPPORTED;
  if (Dm % 64 != 0 || R % 16 != 0 || R > 128) return PATH_ATTN_EUNSUPPORTED;
  // int element offsets of a row stay below 2^31; one block per 62 tokens
  if ((unsigned long long)B * T * Dm >= (1ull << 40) || (unsigned long long)B * H * T * d >= (1ull << 40) ||
      (unsigned long long)B * wbeta_tiles(T) >= (1ull << 31) || (unsigned long long)H * d * R >= (1ull << 31))
    return PATH_ATTN_EUNSUPPORTED;
  const void *ptrs[] = {x, wd, wu, cw, u, ub, w, beta};
  for (const void *p : ptrs)
    if (!p) return PATH_ATTN_EINVAL;
  const void *vecs[] = {x, wd, wu, cw, u, w};   // 16-byte loads and stores
  for (const void *p : vecs)
    if (!aligned(p, 16)) return PATH_ATTN_EINVAL;
  if (!aligned(ub, 4) || !aligned(beta, 4)) return PATH_ATTN_EINVAL;
  WbetaArgs a{x, wd, wu, u, cw, ub, w, beta, B, T, Dm, R, H, d};
  return launch_wbeta(a, static_cast<hipStream_t>(stream)) == hipSuccess ? PATH_ATTN_OK
                                                                          : PATH_ATTN_EHIP;
}

extern "C" const char *path_attn_strerror(int status) {
  switch (status) {
    case PATH_ATTN_OK: return "ok";
    case PATH_ATTN_EINVAL:
      return "invalid argument (null or misaligned pointer, non-positive size, "
             "unknown dtype or flag, scale not positive, or workspace too small)";
    case PATH_ATTN_EUNSUPPORTED:
      return "unsupported shape (d must be 64 or 128, B*H*T*d < 2^31 with T "
             "rounded up to a multiple of 64; prefill lengths and the chunk "
             "unpack need whole 64-token chunks)";
    case PATH_ATTN_EHIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

extern "C" const char *path_attn_version(void) { return "libpath_attn 0.1.0 (gfx950)"; }
