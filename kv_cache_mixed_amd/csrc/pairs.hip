// pairs.hip -- pair-granular key widths from RoPE pair norms.
//
// PN-Mix page (abstract): the quantization error of a RoPE channel pair moves
// the attention logit in proportion to the product of the query's and the
// key's norms over that pair, so the pairs with the largest query-key
// pair-norm products get the higher widths; they are picked once from prefill
// statistics and kept for the whole decode.  Pair p of a 128-channel head is
// channels (p, p + 64), the rotate-half pairing of the RoPE in use.
//
// kvq_pair_norms sums the pair norms over batch, tokens and the heads of a
// group (an HBM-bound reduction); kvq_pair_slot_map turns per-pair scores into
// the slot order of the mixed key tile, both channels of a pair in one class,
// so the mixed quantize and decode kernels serve the pair-granular maps as
// they are.
#pragma clang fp contract(off)

#include <algorithm>
#include <cmath>

#include "kvq_device.h"

namespace kvq {

constexpr int PAIR_TOKENS = 256;   // tokens per workgroup

// workgroup (token chunk, head, batch): thread (j, p) takes pair p of tokens
// t0 + j, t0 + j + 4, ...; both halves of a token row are read by coalesced
// 256-byte loads
template <int IN>
__global__ __launch_bounds__(256) void pair_norm_kernel(const void* __restrict__ x, int64_t sb, int64_t sh,
                                                        int64_t st, int T, int group,
                                                        float* __restrict__ out) {
  const int p = threadIdx.x & 63, j = threadIdx.x >> 6;
  const int h = blockIdx.y, b = blockIdx.z;
  const int t0 = blockIdx.x * PAIR_TOKENS;
  const int t1 = min(T, t0 + PAIR_TOKENS);
  const int64_t base = (int64_t)b * sb + (int64_t)h * sh + p;
  float acc = 0.0f;
#pragma unroll 8
  for (int t = t0 + j; t < t1; t += 4) {
    float a, c;
    if constexpr (IN == KVQ_F32) {
      a = __builtin_nontemporal_load((const float*)x + base + (int64_t)t * st);
      c = __builtin_nontemporal_load((const float*)x + base + (int64_t)t * st + 64);
    } else {
      a = bf16_bits_to_f32(((const uint16_t*)x)[base + (int64_t)t * st]);
      c = bf16_bits_to_f32(((const uint16_t*)x)[base + (int64_t)t * st + 64]);
    }
    acc += __builtin_sqrtf(a * a + c * c);
  }
  __shared__ float red[4][64];
  red[j][p] = acc;
  __syncthreads();
  if (j == 0) atomicAdd(out + (int64_t)(h / group) * 64 + p, (red[0][p] + red[1][p]) + (red[2][p] + red[3][p]));
}

}  // namespace kvq

extern "C" kvq_status kvq_pair_norms(const void* x, kvq_dtype in_dtype, const int64_t strides[3], int32_t batch,
                                     int32_t n_heads, int32_t n_tokens, int32_t group, float* out,
                                     hipStream_t stream) {
  if (!out || !strides) return KVQ_EINVAL;
  if (in_dtype != KVQ_F32 && in_dtype != KVQ_BF16) return KVQ_EINVAL;
  if (batch < 1 || n_heads < 1 || n_tokens < 0 || group < 1 || n_heads % group) return KVQ_EINVAL;
  if (strides[0] < 0 || strides[1] < 0 || strides[2] < 128) return KVQ_EINVAL;
  if (n_tokens == 0) return KVQ_OK;   // x is not read
  if (!x) return KVQ_EINVAL;
  const dim3 grid((n_tokens + kvq::PAIR_TOKENS - 1) / kvq::PAIR_TOKENS, n_heads, batch), block(256);
  if (in_dtype == KVQ_F32)
    hipLaunchKernelGGL(kvq::pair_norm_kernel<KVQ_F32>, grid, block, 0, stream, x, strides[0], strides[1],
                       strides[2], n_tokens, group, out);
  else
    hipLaunchKernelGGL(kvq::pair_norm_kernel<KVQ_BF16>, grid, block, 0, stream, x, strides[0], strides[1],
                       strides[2], n_tokens, group, out);
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EHIP;
}

extern "C" kvq_status kvq_pair_slot_map(const float* score, int32_t n_kv_heads, int16_t* slot_chan) {
  if (!score || !slot_chan || n_kv_heads < 1) return KVQ_EINVAL;
  for (int64_t i = 0; i < (int64_t)n_kv_heads * 64; i++)
    if (!std::isfinite(score[i])) return KVQ_EINVAL;
  for (int h = 0; h < n_kv_heads; h++) {
    const float* s = score + (int64_t)h * 64;
    int rank[64];
    for (int p = 0; p < 64; p++) rank[p] = p;
    // descending score, equal scores by ascending pair index
    std::stable_sort(rank, rank + 64, [&](int a, int b) { return s[a] > s[b]; });
    // classes of the mixed key tile: 4 pairs (8 channels) each at 4, 3 and
    // 1 bits, the 52 others at 2 bits
    int c4[8], c3[8], c1[8], c2[104];
    int n4 = 0, n3 = 0, n1 = 0, n2 = 0;
    for (int r = 0; r < 64; r++) {
      for (int c : {rank[r], rank[r] + 64}) {
        if (r < 4) c4[n4++] = c;
        else if (r < 8) c3[n3++] = c;
        else if (r >= 60) c1[n1++] = c;
        else c2[n2++] = c;
      }
    }
    std::sort(c4, c4 + 8);
    std::sort(c3, c3 + 8);
    std::sort(c1, c1 + 8);
    std::sort(c2, c2 + 104);
    int16_t* o = slot_chan + (int64_t)h * 128;
    for (int i = 0; i < 8; i++) {
      o[i] = (int16_t)c4[i];
      o[8 + 2 * i] = (int16_t)c3[i];
      o[9 + 2 * i] = (int16_t)c1[i];
    }
    for (int i = 0; i < 104; i++) o[24 + i] = (int16_t)c2[i];
  }
  return KVQ_OK;
}
