// shrink.hip -- Equivalent Right Shift of whole packed tiles, in place.
//
// PM-KVQ page, Key design 1 (ERS equation): a 2b-bit code X becomes
//   X_b = ((2^(2b) - 2^b + 1) * (X + 2^(b-1))) >> 3b,
// the zero point is kept and the scale becomes (2^b + 1) * S.  The product
// stays below 2^32 for b <= 8, so the arithmetic is unsigned 32-bit.
//
// A uniform-width tile is a stream of 16384 codes (keys token-major, values
// channel-major); the shrink keeps the code order, so key and value tiles use
// the same kernel.  One workgroup of 256 threads owns one tile: every thread
// loads its 64 codes (16*b bytes at 2b bits) into registers, the workgroup
// synchronises, and only then writes the 8*b-byte result into the first half
// of the tile.  No workgroup touches another tile, so in-place is race-free.
// Threads 0..127 also rescale the tile's 128 scales (key: per channel of this
// tile; value: per token of this tile).
#pragma clang fp contract(off)

#include "kvq_device.h"

namespace kvq {

template <int B, int PDT>
__global__ __launch_bounds__(256) void shrink_kernel(Geo g) {
  constexpr int IN_BITS = 2 * B;
  constexpr int IN_WORDS = 4 * B;             // 64 codes * 2B bits / 32
  constexpr int OUT_WORDS = 2 * B;            // 64 codes * B bits / 32
  constexpr uint32_t C = (1u << (2 * B)) - (1u << B) + 1u;
  constexpr uint32_t HALF = 1u << (B - 1);
  constexpr uint32_t IN_MASK = (IN_BITS == 32) ? 0xffffffffu : ((1u << IN_BITS) - 1u);

  const int tile = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / g.H, h = bh % g.H;
  const bool is_v = blockIdx.z != 0;
  uint8_t* base = is_v ? g.v_codes + v_tile_offset(g, b, h, tile)
                       : g.k_codes + k_tile_offset(g, b, h, tile);
  uint32_t* in = (uint32_t*)base + threadIdx.x * IN_WORDS;
  uint32_t w[IN_WORDS];
#pragma unroll
  for (int i = 0; i < IN_WORDS; i++) w[i] = in[i];

  void* sarr = is_v ? g.v_scale : g.k_scale;
  const int64_t pbase = is_v ? v_param_base(g, b, h, (int64_t)tile * 128)
                             : k_param_base(g, b, h, tile);
  float s_new = 0.0f;
  if (threadIdx.x < 128) {
    const float s_old = Param<PDT>::load(sarr, pbase + threadIdx.x);
    s_new = (float)((1u << B) + 1u) * s_old;        // exact for 16/8/4-bit significands
  }
  __syncthreads();   // every code of the tile is in registers before any write

  uint32_t o[OUT_WORDS];
#pragma unroll
  for (int i = 0; i < OUT_WORDS; i++) o[i] = 0u;
#pragma unroll
  for (int k = 0; k < 64; k++) {
    const int ib = k * IN_BITS;
    const uint32_t x = (w[ib >> 5] >> (ib & 31)) & IN_MASK;
    const uint32_t y = (C * (x + HALF)) >> (3 * B);
    const int ob = k * B;
    o[ob >> 5] |= y << (ob & 31);
  }
  uint32_t* out = (uint32_t*)base + threadIdx.x * OUT_WORDS;
#pragma unroll
  for (int i = 0; i < OUT_WORDS; i++) out[i] = o[i];
  if (threadIdx.x < 128) Param<PDT>::store(sarr, pbase + threadIdx.x, s_new);
}

template <int PDT>
static hipError_t launch_shrink_pdt(const Geo& g, int to_bits, hipStream_t st) {
  dim3 grid(g.n_tiles, g.B * g.H, 2), block(256);
  switch (to_bits) {
    case 8: hipLaunchKernelGGL((shrink_kernel<8, PDT>), grid, block, 0, st, g); break;
    case 4: hipLaunchKernelGGL((shrink_kernel<4, PDT>), grid, block, 0, st, g); break;
    case 2: hipLaunchKernelGGL((shrink_kernel<2, PDT>), grid, block, 0, st, g); break;
    case 1: hipLaunchKernelGGL((shrink_kernel<1, PDT>), grid, block, 0, st, g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_shrink(const Geo& g, int to_bits, hipStream_t st) {
  if (g.n_tiles == 0) return hipSuccess;
  switch (g.pdt) {
    case KVQ_F32: return launch_shrink_pdt<KVQ_F32>(g, to_bits, st);
    case KVQ_F16: return launch_shrink_pdt<KVQ_F16>(g, to_bits, st);
    case KVQ_BF16: return launch_shrink_pdt<KVQ_BF16>(g, to_bits, st);
    case KVQ_E4M3: return launch_shrink_pdt<KVQ_E4M3>(g, to_bits, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
