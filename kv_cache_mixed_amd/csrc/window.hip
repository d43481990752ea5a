// window.hip -- the copy kernel of the unpacked token window.
//
// PM-KVQ page (Training strategy and Related work): as in KIVI, the first
// token and the most recent tokens stay at 16-bit precision while the rest of
// the cache is packed.  kvq_window_append (kvq_api.cpp) keeps those tokens in
// a window buffer per stream and hands every full 128-token group to the
// quantizer; this kernel moves appended token rows into the window.
//
// A pure copy: one 16-byte chunk per thread, rows of 128 elements (256 or 512
// bytes), K in grid row 0 and V in grid row 1.
#include "kvq_device.h"

namespace kvq {

__global__ __launch_bounds__(256) void window_copy_kernel(const uint8_t* __restrict__ k,
                                                          const uint8_t* __restrict__ v,
                                                          int64_t ksb, int64_t ksh, int64_t kst,
                                                          int64_t vsb, int64_t vsh, int64_t vst,
                                                          uint8_t* __restrict__ wk,
                                                          uint8_t* __restrict__ wv, int H, int m,
                                                          int64_t n_chunks, int row_bytes, int slot0) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_chunks) return;
  const int cpr = row_bytes >> 4;                 // 16-byte chunks per row
  const int64_t r = i / cpr;
  const int c = (int)(i - r * cpr);
  const int64_t bh = r / m;                       // stream b * H + h
  const int t = (int)(r - bh * m);
  const int64_t b = bh / H, h = bh - (bh / H) * H;
  const bool is_v = blockIdx.y != 0;
  const uint8_t* src = is_v ? v + b * vsb + h * vsh + (int64_t)t * vst
                            : k + b * ksb + h * ksh + (int64_t)t * kst;
  uint8_t* dst = (is_v ? wv : wk) + (bh * KVQ_WINDOW_ROWS + slot0 + t) * row_bytes;
  *(uint4*)(dst + 16 * c) = *(const uint4*)(src + 16 * c);
}

hipError_t launch_window_copy(const void* k, const void* v, const int64_t ks[3], const int64_t vs[3],
                              int elt_bytes, void* wk, void* wv, int B, int H, int m, int slot0,
                              hipStream_t st) {
  if (m <= 0) return hipSuccess;
  // the rows must lie inside the window (the caller's plan guarantees it)
  if (slot0 < 0 || slot0 + m > KVQ_WINDOW_ROWS || (elt_bytes != 2 && elt_bytes != 4))
    return hipErrorInvalidValue;
  const int row_bytes = 128 * elt_bytes;
  const int64_t n_chunks = (int64_t)B * H * m * (row_bytes / 16);
  const dim3 grid((unsigned)((n_chunks + 255) / 256), 2), block(256);
  // strides in bytes
  hipLaunchKernelGGL(window_copy_kernel, grid, block, 0, st, (const uint8_t*)k, (const uint8_t*)v,
                     ks[0] * elt_bytes, ks[1] * elt_bytes, ks[2] * elt_bytes, vs[0] * elt_bytes,
                     vs[1] * elt_bytes, vs[2] * elt_bytes, (uint8_t*)wk, (uint8_t*)wv, H, m, n_chunks,
                     row_bytes, slot0);
  return hipGetLastError();
}

}  // namespace kvq
