// shrink.hip -- Equivalent Right Shift of whole packed tiles, in place.
//
// PM-KVQ page, Key design 1 (ERS equation): a 2b-bit code X becomes
//   X_b = ((2^(2b) - 2^b + 1) * (X + 2^(b-1))) >> 3b,
// the zero point is kept and the scale becomes (2^b + 1) * S.  The product
// stays below 2^32 for b <= 8, so the arithmetic is unsigned 32-bit.
// The same page's ablation compares it with a direct right shift (keep the
// high b bits: X_b = X >> b) and a "modified" right shift, which it does not
// define; here that is the rounded shift min((X + 2^(b-1)) >> b, 2^b - 1).
// Both keep the zero point and scale by 2^b.
//
// A uniform-width key tile is a stream of 16384 codes whose order the shrink
// keeps.  A value tile's word planes depend on the width: output word
// (w, c, a) at b bits is made of input words (2w, c, a) and (2w+1, c, a) at 2b
// bits.  One workgroup of 256 threads owns one tile: every thread loads the
// input words it needs into registers, the workgroup synchronises, and only
// then writes the b-bit result into the first half of the tile.  No
// workgroup touches another tile, so in-place is race-free.
// Threads 0..127 also rescale the tile's 128 scales (key: per channel of this
// tile; value: per token of this tile).
#pragma clang fp contract(off)

#include "kvq_device.h"

namespace kvq {

// one 2B-bit code -> B bits by method M (KVQ_SHIFT_ERS / _DIRECT / _MODIFIED)
template <int B, int M>
__device__ __forceinline__ uint32_t shift_code(uint32_t x) {
  constexpr uint32_t HALF = 1u << (B - 1);
  if constexpr (M == KVQ_SHIFT_DIRECT) {
    return x >> B;
  } else if constexpr (M == KVQ_SHIFT_MODIFIED) {
    return min((x + HALF) >> B, (1u << B) - 1u);
  } else {
    constexpr uint32_t C = (1u << (2 * B)) - (1u << B) + 1u;
    return (C * (x + HALF)) >> (3 * B);
  }
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// n codes of 2B bits in the low bits of w (LSB first) -> n codes of B bits
template <int B, int M, int N>
__device__ __forceinline__ uint32_t shift_word(uint32_t w) {
  constexpr uint32_t MASK = (2 * B == 32) ? 0xffffffffu : ((1u << (2 * B)) - 1u);
  if constexpr (M == KVQ_SHIFT_ERS && B <= 4 && N == 16 / B) {
    // ERS in 16-bit halves: C * (X + 2^(b-1)) <= 241 * 263 < 2^16 for b <= 4.
    // Pair i holds code i in the low half and code N/2 + i in the high half;
    // the results land at bits B*i and 16 + B*i and are folded to 16 bits.
    constexpr unsigned short C = (unsigned short)((1u << (2 * B)) - (1u << B) + 1u);
    constexpr unsigned short CH = (unsigned short)(C * (1u << (B - 1)));
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < N / 2; i++) {
      const u16x2 x = __builtin_bit_cast(u16x2, (w >> (i * 2 * B)) & (MASK | (MASK << 16)));
      const u16x2 y = (x * (u16x2){C, C} + (u16x2){CH, CH}) >> (u16x2){3 * B, 3 * B};
      acc |= __builtin_bit_cast(uint32_t, y) << (i * B);
    }
    return (acc & 0xffu) | ((acc >> 8) & 0xff00u);
  }
  uint32_t o = 0;
#pragma unroll
  for (int i = 0; i < N; i++) o |= shift_code<B, M>((w >> (i * 2 * B)) & MASK) << (i * B);
  return o;
}

template <int B, int PDT, int M>
__global__ __launch_bounds__(256) void shrink_kernel(Geo g) {
  constexpr int IN_WORDS = 4 * B;             // per thread: 64 codes * 2B bits / 32
  constexpr int OUT_WORDS = 2 * B;            // per thread: 64 codes * B bits / 32
  const int tile = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / g.H, h = bh % g.H;
  const bool is_v = blockIdx.z != 0;
  uint8_t* base = is_v ? g.v_codes + v_tile_offset(g, b, h, tile)
                       : g.k_codes + k_tile_offset(g, b, h, tile);
  uint32_t w[IN_WORDS];
  if (!is_v) {
    // key tile: a flat stream of codes; output word o = t + 256k is made of
    // input words 2o and 2o + 1 (one 8-byte load, consecutive across lanes)
    const uint2* in = (const uint2*)base;
#pragma unroll
    for (int k = 0; k < OUT_WORDS; k++) {
      const uint2 v = in[threadIdx.x + 256 * k];
      w[2 * k] = v.x;
      w[2 * k + 1] = v.y;
    }
  } else {
    // value tile: output word o = wp*512 + r (r: position inside the word
    // plane, the same function of (channel, lane group) at every width) takes
    // its low half from input word o + wp*512 (plane 2wp, same r) and its high
    // half from o + (wp+1)*512 (plane 2wp+1)
    const uint32_t* in = (const uint32_t*)base;
#pragma unroll
    for (int k = 0; k < OUT_WORDS; k++) {
      const int o = threadIdx.x + 256 * k;
      const int wp = o >> 9;
      w[2 * k] = in[o + wp * 512];
      w[2 * k + 1] = in[o + (wp + 1) * 512];
    }
  }
  void* sarr = is_v ? g.v_scale : g.k_scale;
  const int64_t pbase = is_v ? v_param_base(g, b, h, (int64_t)tile * 128)
                             : k_param_base(g, b, h, tile);
  float s_new = 0.0f;
  if (threadIdx.x < 128) {
    const float s_old = Param<PDT>::load(sarr, pbase + threadIdx.x);
    // (2^b + 1) * S is exact for 16/8/4-bit significands; 2^b * S is exact
    const float f = (M == KVQ_SHIFT_ERS) ? (float)((1u << B) + 1u) : (float)(1u << B);
    s_new = f * s_old;
  }
  __syncthreads();   // every code of the tile is in registers before any write

  uint32_t* out = (uint32_t*)base;
  if (!is_v) {
    // 2 input words (2 * 16/B codes each) -> 1 output word
#pragma unroll
    for (int k = 0; k < OUT_WORDS; k++)
      out[threadIdx.x + 256 * k] =
          shift_word<B, M, 16 / B>(w[2 * k]) | (shift_word<B, M, 16 / B>(w[2 * k + 1]) << 16);
  } else {
#pragma unroll
    for (int k = 0; k < OUT_WORDS; k++)
      out[threadIdx.x + 256 * k] =
          shift_word<B, M, 16 / B>(w[2 * k]) | (shift_word<B, M, 16 / B>(w[2 * k + 1]) << 16);
  }
  if (threadIdx.x < 128) Param<PDT>::store(sarr, pbase + threadIdx.x, s_new);
}

template <int PDT, int M>
static hipError_t launch_shrink_m(const Geo& g, int to_bits, hipStream_t st) {
  dim3 grid(g.n_tiles, g.B * g.H, 2), block(256);
  switch (to_bits) {
    case 8: hipLaunchKernelGGL((shrink_kernel<8, PDT, M>), grid, block, 0, st, g); break;
    case 4: hipLaunchKernelGGL((shrink_kernel<4, PDT, M>), grid, block, 0, st, g); break;
    case 2: hipLaunchKernelGGL((shrink_kernel<2, PDT, M>), grid, block, 0, st, g); break;
    case 1: hipLaunchKernelGGL((shrink_kernel<1, PDT, M>), grid, block, 0, st, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int PDT>
static hipError_t launch_shrink_pdt(const Geo& g, int to_bits, int method, hipStream_t st) {
  switch (method) {
    case KVQ_SHIFT_ERS: return launch_shrink_m<PDT, KVQ_SHIFT_ERS>(g, to_bits, st);
    case KVQ_SHIFT_DIRECT: return launch_shrink_m<PDT, KVQ_SHIFT_DIRECT>(g, to_bits, st);
    case KVQ_SHIFT_MODIFIED: return launch_shrink_m<PDT, KVQ_SHIFT_MODIFIED>(g, to_bits, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_shrink(const Geo& g, int to_bits, int method, hipStream_t st) {
  if (g.n_tiles == 0) return hipSuccess;
  switch (g.pdt) {
    case KVQ_F32: return launch_shrink_pdt<KVQ_F32>(g, to_bits, method, st);
    case KVQ_F16: return launch_shrink_pdt<KVQ_F16>(g, to_bits, method, st);
    case KVQ_BF16: return launch_shrink_pdt<KVQ_BF16>(g, to_bits, method, st);
    case KVQ_E4M3: return launch_shrink_pdt<KVQ_E4M3>(g, to_bits, method, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
