// pad.hip -- staging between the caller's tensors and whole 64-token chunks.
//
// The chunked algorithm needs whole chunks (the authors' reference listing
// also requires L % BT == 0).  A length T is padded to Tp = 64*ceil(T/64) with
// tokens whose factor is the identity (beta = 0, w = 0) and whose query, key,
// value and gate are zero.  Padded tokens come after every real token, so they
// never enter the path H_{j+1} ... H_i of a real query i < T, and the causal
// mask keeps them out of its softmax; the rows of padded queries are computed
// and dropped.
//
// The same row copy serves strided and packed (variable-length) batches: a
// caller's tensor is any view whose rows (d elements, or one float32 scalar)
// are contiguous, addressed by element strides over (batch, head, token) and,
// for packed batches, by each sequence's first token.  Each sequence of a
// packed batch becomes one padded [Tp]-row head of the staging layout, so its
// path and its gate prefix start at its own first token.
#include "path_attn_internal.h"

namespace pathattn {

namespace {

// Row gather / scatter between a view and the padded layout [B][H][Tp][row]
// (row = `words` words of type W).  View row (b, h, t) starts at element
//     (off_b + t) * s_tok + b * s_b + h * s_h
// of the view (elements of esize bytes), off_b = cu ? cu[b] : 0, and exists
// for t < len_b = cu ? cu[b+1] - cu[b] : T, clamped to [0, T].  Gather fills
// the rows at t >= len_b with zeros; scatter writes only the rows t < len_b.
template <bool GATHER, typename W>
__global__ __launch_bounds__(256) void view_rows_kernel(const unsigned char *__restrict__ src,
                                                        unsigned char *__restrict__ dst,
                                                        const int *__restrict__ cu, int H, int T,
                                                        int Tp, long long s_b, long long s_h,
                                                        long long s_tok, int esize, int words,
                                                        size_t total) {
  const size_t per_head = (size_t)Tp * words;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (size_t)gridDim.x * 256) {
    const size_t bh = i / per_head, rem = i % per_head;
    const int t = (int)(rem / words), wd = (int)(rem % words);
    const int b = (int)(bh / H), h = (int)(bh % H);
    long long off_b = 0;
    int len = T;
    if (cu) {
      off_b = cu[b];
      len = cu[b + 1] - cu[b];
      len = len < 0 ? 0 : (len > T ? T : len);
    }
    const long long view_byte =
        ((off_b + t) * s_tok + (long long)b * s_b + (long long)h * s_h) * esize +
        (long long)wd * (long long)sizeof(W);
    if (GATHER) {
      W val{};
      if (t < len) val = *reinterpret_cast<const W *>(src + view_byte);
      reinterpret_cast<W *>(dst)[i] = val;
    } else if (t < len) {
      *reinterpret_cast<W *>(dst + view_byte) = reinterpret_cast<const W *>(src)[i];
    }
  }
}

template <bool GATHER, typename W>
hipError_t launch_rows(const void *src, void *dst, const RowView &view, int B, int H, int T,
                       int Tp, int esize, int row_bytes, hipStream_t stream) {
  const int words = row_bytes / (int)sizeof(W);
  const size_t total = (size_t)B * H * Tp * words;
  size_t blocks = (total + 255) / 256;
  blocks = blocks < 1 ? 1 : (blocks > 8192 ? 8192 : blocks);
  hipLaunchKernelGGL((view_rows_kernel<GATHER, W>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const unsigned char *>(src), static_cast<unsigned char *>(dst),
                     view.cu, H, T, Tp, view.s_b, view.s_h, view.s_tok, esize, words, total);
  return hipGetLastError();
}

}  // namespace

bool view_rows_vec16(const void *base, const RowView &view, int esize, int row_bytes) {
  const long long e = esize;
  return (uintptr_t)base % 16 == 0 && row_bytes % 16 == 0 && (view.s_b * e) % 16 == 0 &&
         (view.s_h * e) % 16 == 0 && (view.s_tok * e) % 16 == 0;
}

hipError_t launch_view_rows(bool gather, const void *src, void *dst, const RowView &view, int B,
                            int H, int T, int Tp, int esize, int row_bytes, hipStream_t stream) {
  const void *user = gather ? src : static_cast<const void *>(dst);
  if (view_rows_vec16(user, view, esize, row_bytes))
    return gather ? launch_rows<true, uint4>(src, dst, view, B, H, T, Tp, esize, row_bytes, stream)
                  : launch_rows<false, uint4>(src, dst, view, B, H, T, Tp, esize, row_bytes,
                                              stream);
  return gather ? launch_rows<true, uint32_t>(src, dst, view, B, H, T, Tp, esize, row_bytes, stream)
                : launch_rows<false, uint32_t>(src, dst, view, B, H, T, Tp, esize, row_bytes,
                                               stream);
}

}  // namespace pathattn
