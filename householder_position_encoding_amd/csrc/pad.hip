// pad.hip -- sequence lengths that are not a multiple of the 64-token chunk.
//
// The chunked algorithm needs whole chunks (the authors' reference listing
// also requires L % BT == 0).  A length T is padded to Tp = 64*ceil(T/64) with
// tokens whose factor is the identity (beta = 0, w = 0) and whose query, key,
// value and gate are zero.  Padded tokens come after every real token, so they
// never enter the path H_{j+1} ... H_i of a real query i < T, and the causal
// mask keeps them out of its softmax; the rows of padded queries are computed
// and dropped.  This file holds the row copy that moves [BH][T][row] arrays
// into and out of the padded staging buffers.
#include "path_attn_internal.h"

namespace pathattn {

namespace {

// dst[bh][t] = t < n_copy ? src[bh][t] : 0 for t < dst_rows; rows are `words`
// 4-byte words; src has src_rows rows per head.
__global__ __launch_bounds__(256) void copy_pad_kernel(const uint32_t *__restrict__ src,
                                                       uint32_t *__restrict__ dst, int BH,
                                                       int src_rows, int dst_rows, int n_copy,
                                                       int words) {
  const size_t per_head = (size_t)dst_rows * words;
  const size_t total = per_head * BH;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (size_t)gridDim.x * 256) {
    const size_t bh = i / per_head, rem = i % per_head;
    const size_t t = rem / words, wd = rem % words;
    dst[i] = t < (size_t)n_copy ? src[(bh * src_rows + t) * words + wd] : 0u;
  }
}

}  // namespace

hipError_t launch_copy_pad(const void *src, void *dst, int BH, int src_rows, int dst_rows,
                           int n_copy, int row_bytes, hipStream_t stream) {
  const int words = row_bytes / 4;
  const size_t total = (size_t)BH * dst_rows * words;
  const int blocks = (int)((total + 255) / 256 < 8192 ? (total + 255) / 256 : 8192);
  hipLaunchKernelGGL(copy_pad_kernel, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, stream,
                     static_cast<const uint32_t *>(src), static_cast<uint32_t *>(dst), BH,
                     src_rows, dst_rows, n_copy, words);
  return hipGetLastError();
}

}  // namespace pathattn
