// kvq_device.h -- device-side numerics and cache addressing shared by the
// libkvq kernels (gfx950).  Not part of the public ABI.
//
// Number formats are written from their definitions (IEEE 754 binary16,
// bfloat16, OCP FP8 E4M3): narrowing is round-to-nearest-even on the bit
// pattern, with no dependence on the hardware rounding or denormal mode.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

// ---------------------------------------------------------------------------
// binary32 helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float u2f(uint32_t x) { return __builtin_bit_cast(float, x); }

// 2^k as a binary32 for k in [-126, 127]
__device__ __forceinline__ float exp2i(int k) {
  k = k < -126 ? -126 : (k > 127 ? 127 : k);
  return u2f((uint32_t)(k + 127) << 23);
}

// Lane swaps of gfx950.  v_permlane32_swap / v_permlane16_swap of a register
// with a copy of itself leave in every lane its own value (r0) and that of
// lane l ^ 32 / l ^ 16 (r1).  Written as inline assembly: through the
// builtins the compiler has been seen to use the first result for both
// (a min or sum of the pair then silently became the lane's own value).  The
// leading s_nop covers the VALU-write-to-permlane-read wait states.
__device__ __forceinline__ void lane_swap32(uint32_t x, uint32_t& r0, uint32_t& r1) {
  uint32_t a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 0" : "+v"(a), "+v"(b));
  r0 = a;
  r1 = b;
}
__device__ __forceinline__ void lane_swap16(uint32_t x, uint32_t& r0, uint32_t& r1) {
  uint32_t a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 0" : "+v"(a), "+v"(b));
  r0 = a;
  r1 = b;
}

// unbiased exponent field of a non-negative binary32 (-127 for zero/subnormal)
__device__ __forceinline__ int expo(float x) { return (int)((f2u(x) >> 23) & 0xffu) - 127; }

// round-to-nearest-even right shift of an unsigned significand by s >= 1 bits
__device__ __forceinline__ uint32_t rne_shift(uint32_t m, uint32_t s) {
  if (s >= 32) return 0;
  uint32_t q = m >> s;
  uint32_t rem = m & ((1u << s) - 1u);
  uint32_t half = 1u << (s - 1);
  if (rem > half || (rem == half && (q & 1u))) q += 1;
  return q;
}

// ---------------------------------------------------------------------------
// IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits; subnormal
// quantum 2^-24; |x| >= 65520 overflows to infinity.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  uint32_t x = f2u(f);
  uint32_t sign = (x >> 16) & 0x8000u;
  uint32_t a = x & 0x7fffffffu;
  if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u);          // NaN
  if (a >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);         // >= 65520 -> inf
  uint32_t e = a >> 23;
  if (e >= 113) {                                                   // normal binary16
    uint32_t r = rne_shift(a - (112u << 23), 13);                   // rebias, carry ok
    return (uint16_t)(sign | r);
  }
  // subnormal binary16: value = m * 2^-24 with m = round(a_value * 2^24)
  if (e == 0) return (uint16_t)sign;                                // binary32 subnormal: < 2^-126
  uint32_t mant = (a & 0x7fffffu) | 0x800000u;                      // value = mant * 2^(e-150)
  uint32_t s = 126u - e;                                            // shift into 2^-24 units
  return (uint16_t)(sign | rne_shift(mant, s));
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  uint32_t sign = (h & 0x8000u) << 16;
  uint32_t e = (h >> 10) & 31u, m = h & 1023u;
  float v;
  if (e == 0) v = (float)m * 5.9604644775390625e-08f;               // m * 2^-24, exact
  else if (e == 31) v = u2f(0x7f800000u | (m << 13));
  else v = u2f(((e + 112u) << 23) | (m << 13));
  return u2f(f2u(v) | sign);
}

// ---------------------------------------------------------------------------
// bfloat16: the upper half of a binary32, round to nearest even.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t x = f2u(f);
  if ((x & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((x >> 16) | 0x40u);
  return (uint16_t)((x + 0x7fffu + ((x >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return u2f(h << 16); }

// ---------------------------------------------------------------------------
// OCP FP8 E4M3: 1 sign, 4 exponent (bias 7), 3 fraction bits, no infinities,
// S.1111.111 = NaN, largest finite 448; subnormal quantum 2^-9.  Narrowing
// rounds to nearest even and saturates finite overflow to +-448.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint8_t f32_to_e4m3_bits(float f) {
  uint32_t x = f2u(f);
  uint32_t sign = (x >> 24) & 0x80u;
  uint32_t a = x & 0x7fffffffu;
  if (a > 0x7f800000u) return (uint8_t)(sign | 0x7fu);
  if (a >= 0x43e00000u) return (uint8_t)(sign | 0x7eu);            // >= 448 -> 448
  uint32_t e = a >> 23;
  if (e >= 121) {                                                   // normal e4m3 (>= 2^-6)
    uint32_t r = rne_shift(a - (120u << 23), 20);
    if (r > 0x7eu) r = 0x7eu;                                       // [448, 464) rounds to 448
    return (uint8_t)(sign | r);
  }
  if (e == 0) return (uint8_t)sign;
  uint32_t mant = (a & 0x7fffffu) | 0x800000u;                      // value = mant * 2^(e-150)
  uint32_t s = 141u - e;                                            // into 2^-9 units
  return (uint8_t)(sign | rne_shift(mant, s));
}

__device__ __forceinline__ float e4m3_bits_to_f32(uint32_t c) {
  uint32_t sign = (c & 0x80u) << 24;
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v;
  if (e == 0) v = (float)m * 0.001953125f;                          // m * 2^-9
  else if (e == 15 && m == 7) v = u2f(0x7fc00000u);
  else v = u2f(((e + 120u) << 23) | (m << 20));
  return u2f(f2u(v) | sign);
}

// ---------------------------------------------------------------------------
// parameter arrays (raw values of param dtype)
// ---------------------------------------------------------------------------
template <int PDT>
struct Param;
template <>
struct Param<KVQ_F32> {
  static constexpr int bytes = 4;
  __device__ static float load(const void* p, int64_t i) { return ((const float*)p)[i]; }
  __device__ static float narrow(float x) { return x; }
  __device__ static void store(void* p, int64_t i, float x) { ((float*)p)[i] = x; }
  __device__ static float dec(uint32_t raw) { return u2f(raw); }
};
template <>
struct Param<KVQ_F16> {
  // hardware conversions: v_cvt_f16_f32 rounds to nearest even with IEEE
  // overflow to infinity and keeps binary16 subnormals (the kernels run with
  // denormals enabled); v_cvt_f32_f16 is exact
  static constexpr int bytes = 2;
  __device__ static float load(const void* p, int64_t i) {
    return (float)((const _Float16*)p)[i];
  }
  __device__ static float narrow(float x) { return (float)(_Float16)x; }
  __device__ static void store(void* p, int64_t i, float x) { ((_Float16*)p)[i] = (_Float16)x; }
  __device__ static float dec(uint32_t raw) { return (float)__builtin_bit_cast(_Float16, (uint16_t)raw); }
};
template <>
struct Param<KVQ_BF16> {
  static constexpr int bytes = 2;
  __device__ static float load(const void* p, int64_t i) {
    return bf16_bits_to_f32(((const uint16_t*)p)[i]);
  }
  __device__ static float narrow(float x) { return bf16_bits_to_f32(f32_to_bf16_bits(x)); }
  __device__ static void store(void* p, int64_t i, float x) { ((uint16_t*)p)[i] = f32_to_bf16_bits(x); }
  __device__ static float dec(uint32_t raw) { return bf16_bits_to_f32(raw); }
};
template <>
struct Param<KVQ_E4M3> {
  static constexpr int bytes = 1;
  __device__ static float load(const void* p, int64_t i) {
    return e4m3_bits_to_f32(((const uint8_t*)p)[i]);
  }
  __device__ static float narrow(float x) { return e4m3_bits_to_f32(f32_to_e4m3_bits(x)); }
  __device__ static void store(void* p, int64_t i, float x) { ((uint8_t*)p)[i] = f32_to_e4m3_bits(x); }
  __device__ static float dec(uint32_t raw) { return e4m3_bits_to_f32(raw); }
};

// ---------------------------------------------------------------------------
// cache geometry passed to kernels by value
// ---------------------------------------------------------------------------
struct Geo {
  int32_t B, H, max_tiles, n_tiles;
  int32_t k_bits, v_bits, pdt;
  uint8_t* k_codes;
  uint8_t* v_codes;
  const int64_t* k_off;
  const int64_t* v_off;
  int64_t k_stride, v_stride;
  void* k_scale;
  void* k_zero;
  void* v_scale;
  void* v_zero;
  const int16_t* slot_chan;
  int32_t max_tokens;
  const int16_t* v_slot_chan;   // mixed values: channel of value slot j per head
};

// The offset tables are read through the constant address space (they never
// change while a kernel runs), so a wave-uniform index becomes a scalar load.
typedef const __attribute__((address_space(4))) int64_t* const_i64_ptr;
__device__ __forceinline__ int64_t k_tile_offset(const Geo& g, int b, int h, int tile) {
  if (g.k_off) return ((const_i64_ptr)g.k_off)[((int64_t)tile * g.B + b) * g.H + h];
  return (((int64_t)b * g.H + h) * g.max_tiles + tile) * g.k_stride;
}
__device__ __forceinline__ int64_t v_tile_offset(const Geo& g, int b, int h, int tile) {
  if (g.v_off) return ((const_i64_ptr)g.v_off)[((int64_t)tile * g.B + b) * g.H + h];
  return (((int64_t)b * g.H + h) * g.max_tiles + tile) * g.v_stride;
}
// first parameter index of key tile (b, h, tile); value token (b, h, t)
__device__ __forceinline__ int64_t k_param_base(const Geo& g, int b, int h, int tile) {
  return (((int64_t)b * g.H + h) * g.max_tiles + tile) * 128;
}
__device__ __forceinline__ int64_t v_param_base(const Geo& g, int b, int h, int64_t t) {
  return ((int64_t)b * g.H + h) * (int64_t)g.max_tokens + t;
}
// mixed values: parameter of class k (0..3) of token t, class-major per stream
__device__ __forceinline__ int64_t vm_param_index(const Geo& g, int b, int h, int k, int64_t t) {
  return (((int64_t)b * g.H + h) * 4 + k) * (int64_t)g.max_tokens + t;
}

// mixed-width value slots: 0..15 4-bit, 16..31 3-bit, 32..47 1-bit,
// 48..127 2-bit (classes 0..3); blocks of 16 slots, the codes of block m in
// fields of 4 bits (m < 2) or 2 bits (m >= 2)
__host__ __device__ constexpr int vmixed_class_bits(int k) { return k == 0 ? 4 : (k == 1 ? 3 : (k == 2 ? 1 : 2)); }
__host__ __device__ constexpr int vmixed_block_class(int m) { return m < 3 ? m : 3; }
__host__ __device__ constexpr int vmixed_block_field(int m) { return m < 2 ? 4 : 2; }
// first 32-bit word of block m in the 5120-byte tile
__host__ __device__ constexpr int vmixed_block_word(int m) { return m < 2 ? 256 * m : 512 + 128 * (m - 2); }

// mixed-width key slots: 0..7 4-bit, 8..23 alternating 3/1-bit, 24..127 2-bit
__host__ __device__ constexpr int mixed_slot_bits(int j) {
  return j < 8 ? 4 : (j < 24 ? ((j & 1) ? 1 : 3) : 2);
}

}  // namespace kvq

// launchers (host side), implemented in the .hip files
namespace kvq {
// tok (device [B][H][n_new] int32, or null): new token t of stream (b, h) is
// input row tok[(b * H + h) * n_new + t], clamped to [0, n_src)
hipError_t launch_quantize(const Geo& g, const void* k, const void* v, int in_dtype,
                           const int64_t* ks, const int64_t* vs, int t0, int n_new,
                           hipStream_t st, const int32_t* tok = nullptr, int n_src = 0);
hipError_t launch_shrink(const Geo& g, int to_bits, int method, hipStream_t st);
// copy m token rows of every stream (b, h) of k and v (element strides ks / vs
// of batch, kv head, token; channel stride 1; elt_bytes 2 or 4) into rows
// slot0 .. slot0 + m - 1 of the window buffers wk / wv
// ([B][H][KVQ_WINDOW_ROWS][128] elements)
hipError_t launch_window_copy(const void* k, const void* v, const int64_t ks[3], const int64_t vs[3],
                              int elt_bytes, void* wk, void* wv, int B, int H, int m, int slot0,
                              hipStream_t st);
// partial slots per stream: up to KVQ_MAX_CHUNKS packed chunks, then one per
// KVQ_RES_CHUNK residual tokens; the combine kernel takes at most 128
constexpr int KVQ_RES_CHUNK = 32;
constexpr int KVQ_MAX_RES_SLOTS = KVQ_MAX_RESIDUAL / KVQ_RES_CHUNK;
constexpr int KVQ_MAX_CHUNKS = 128 - KVQ_MAX_RES_SLOTS;
constexpr int KVQ_MAX_SLOTS = KVQ_MAX_CHUNKS + KVQ_MAX_RES_SLOTS;
struct DecodePlan {
  int ns, n_groups, n_chunks, tpc;
};
DecodePlan decode_plan(int BH, int G, int k_bits, int v_bits, int pdt, int n_tiles,
                       int max_chunks = KVQ_MAX_CHUNKS);
// decode over two caches of the same streams (tokens split between them)
constexpr int KVQ_SPLIT_MAX_CHUNKS = 64;
hipError_t launch_decode_split(const Geo& ga, const Geo& gb, const void* q, int G, float scale, float* out,
                               void* ws, hipStream_t st);
size_t decode_split_workspace_bytes(int B, int H, int G);
size_t decode_workspace_needed(int BH, int G, const DecodePlan& p);
size_t decode_workspace_bytes(int B, int H, int G, int max_tiles);
// residual segment of a decode call (R = 0: none)
struct ResArgs {
  const void* k;
  const void* v;
  int64_t ks[3], vs[3];   // element strides of (batch, kv head, token); channel stride 1
  int R;
};
hipError_t launch_decode(const Geo& g, const void* q, int G, float scale, float* out, void* ws,
                         const ResArgs& res, int res_dtype, hipStream_t st);
// the two phases of launch_decode (packed cache only) as separate launches:
// the chunk partials (always written to ws, also for a single chunk), and the
// combine of n_slots slots of that layout into out
hipError_t launch_decode_partials(const Geo& g, const void* q, int G, float scale, void* ws, int* n_slots,
                                  int* tiles_per_slot, hipStream_t st);
hipError_t launch_decode_combine(const void* ws, int B, int H, int G, int n_slots, float* out, hipStream_t st);
// bytes of n_slots partial slots per stream (the (m, l) array rounded up to
// 256 bytes, then the outputs)
size_t decode_partials_bytes(int BH, int G, int n_slots);
// allocation-free decode: the device address of the current device's copy
// of the library's scratch array (KVQ_DECODE_SCRATCH_BYTES)
hipError_t decode_scratch_acquire(void** ptr);
bool decode_supported(int k_bits, int v_bits, int pdt);
}  // namespace kvq
