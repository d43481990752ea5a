// decode_attn.hip -- decode attention over the packed cache (gfx950).
//
// ChanMix page, Overall framework / Key design 3: at decode time the packed
// cache is read, dequantized (x^ = S' * q + Z') and fed to ordinary
// (FlashAttention-style) attention.  Here the dequantization never
// materialises: the key parameters are folded into the query and the value
// parameters into the softmax weights, so the two contractions run on the raw
// integer codes with MFMA.
//
// Work decomposition.  Grid = (chunk, b * Hkv).  A workgroup of 4 waves owns
// one chunk of 128-token tiles of one (batch, kv head) stream and all G query
// heads of that kv head; wave w takes tiles w, w+4, ... of the chunk.  Per tile
// a wave computes, with the G heads padded to the 16 columns of a
// 16x16x32 f16 MFMA:
//   S^T[t][n] = sum_c K[t][c] * u[n][c],   u = q * S_K * 2^k (per tile, f16)
//   logit_n(t) = sigma * (S^T / 2^k + sum_c q[n][c] Z_K[c])
//   online softmax in the log2 domain (running max per head, shared by the
//   four lane groups through cross-lane max)
//   O^T[c][n] += sum_t V[c][t] * P[t][n],  P = e^(logit - m) * S_V[t] * 2^k'
//   zsum_n    += sum_t e^(logit - m) * Z_V[t]
// The workgroup merges its four wave partials in LDS and writes one partial
// (m, l, o[128]) per head; a second kernel combines the chunks of a stream:
// o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
//
// MFMA operand layout (16x16x32 f16): lane l = 16*g + n holds, for A, row n and
// k-slice g (8 values), for B, column n and k-slice g, and receives D rows
// 4g..4g+3 of column n.  Row r of the key block j maps to token
//   tau(j, r) = 32*(r/4) + 4*j + (r%4)
// so lane group g of the D output holds tokens 32g + 4j + i, i.e. exactly the
// 32 tokens whose value codes the same lane group loads for the PV product.
// Each lane therefore reads 4b contiguous bytes per key row and per value row.
//
// Codes become f16 operands without conversion instructions: a b-bit field at
// bit position p (p + b <= 10) of both 16-bit halves of a loaded word, masked in
// place, is the f16 subnormal code * 2^(p - 24), which MFMA multiplies exactly.
// The power-of-two field weights (2^-p, and 2^8 for the high byte of 16-bit
// codes) are folded into the other operand.  That operand (u for keys, P for
// values) is split into f16 hi + lo parts (two MFMAs), so the products carry
// about 22 significant bits and the sums accumulate in binary32.
//
// Softmax uses a lazy running max: the reference m only moves when a logit
// exceeds it by more than TAU (log2 units), so e = 2^(logit - m) <= 2^TAU and
// the output accumulator is rescaled only when some head's reference moved.
#include "kvq_device.h"
// waves of the decode kernel resident per SIMD (register budget 512 / n)
// A nonzero KVQ_DECODE_WAVES_PER_SIMD forces every decode instance to that
// occupancy (tuning builds); 0 uses the per-instance table decode_occ().
#ifndef KVQ_DECODE_WAVES_PER_SIMD
#define KVQ_DECODE_WAVES_PER_SIMD 0
#endif
// most sub-tiles a 128-token tile is cut into (4, 2 or 1)
#ifndef KVQ_DECODE_NSUB_MAX
#define KVQ_DECODE_NSUB_MAX 4
#endif
// most kv streams one decode wave packs into its MFMA columns
#ifndef KVQ_DECODE_NS_MAX
#define KVQ_DECODE_NS_MAX 3
#endif
// wave priority from the tiles a wave has left (1) or the default (0)
#ifndef KVQ_DECODE_PRIO
#define KVQ_DECODE_PRIO 1
#endif
// streams split into at least this many chunks are combined inside the decode
// kernel by the workgroup that finishes the last chunk of a stream group;
// fewer chunks are combined by a second kernel.  Measured: a second kernel is
// cheaper at the 16-32 chunks of batched layers, where the combine work of the
// last workgroups at the tail costs more than the launch; the in-kernel
// combine wins for the 64 chunks of single-sequence long contexts.
#ifndef KVQ_DECODE_FUSED_MIN_CHUNKS
#define KVQ_DECODE_FUSED_MIN_CHUNKS 48
#endif
// cache-policy bits of the code loads (sc0 = 1, nt = 2, sc1 = 16) and of the
// parameter loads.  Codes are read once: non-temporal loads measured 6-11%
// faster at every width but 16-bit, where they are 15% slower.
#ifndef KVQ_DECODE_CPOL_CODES
#define KVQ_DECODE_CPOL_CODES 2
#endif
#ifndef KVQ_DECODE_CPOL_PARAMS
#define KVQ_DECODE_CPOL_PARAMS 0
#endif
// workgroups one decode launch aims at per wave-per-SIMD of the instance
#ifndef KVQ_DECODE_WG_PER_OCC
#define KVQ_DECODE_WG_PER_OCC 256
#endif

namespace kvq {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// A bit field of a loaded 32-bit word that becomes one f16x2 operand register:
// word index, right shift before masking, bit position and width inside each
// 16-bit half, lane-local code index of the low and high half, log2 weight.
struct Fld {
  int w, sh, pos, wid, lo, hi, wexp;
};

// Uniform b-bit row segment of 32 codes (b words).  Codes in the low half of a
// word pair with codes of the high half; fields that would reach bit 10 are
// shifted down first.
template <int B>
__host__ __device__ constexpr Fld ufield(int i) {
  if (B == 16) { const int w = i / 2, hb = i % 2; return {w, hb ? 8 : 0, 0, 8, 2 * w, 2 * w + 1, hb ? 8 : 0}; }
  if (B == 8) { const int w = i / 2, k = i % 2; return {w, k ? 8 : 0, 0, 8, 4 * w + k, 4 * w + 2 + k, 0}; }
  if (B == 4) { const int w = i / 4, k = i % 4; return {w, k >= 2 ? 8 : 0, (k % 2) * 4, 4, 8 * w + k, 8 * w + 4 + k, 0}; }
  if (B == 2) {
    const int w = i / 8, k = i % 8;
    return {w, k >= 5 ? 10 : 0, k >= 5 ? 2 * (k - 5) : 2 * k, 2, 16 * w + k, 16 * w + 8 + k, 0};
  }
  const int w = i / 16, k = i % 16;
  return {w, k >= 10 ? 10 : 0, k >= 10 ? k - 10 : k, 1, 32 * w + k, 32 * w + 16 + k, 0};
}

// Mixed key layout, lane group 0: word 0 = slots 0..7 (4-bit), word 1 = slots
// 8..23 ((3,1)-bit pairs), word 2 = slots 120..127 (2-bit) spread so that
// slots 120..123 sit in the low half and 124..127 in the high half.  Lane-local
// index = slot for slots 0..23, 24 + (slot - 120) for the others.
__host__ __device__ constexpr Fld mfield0(int i) {
  if (i < 4) { const int k = i; return {0, k >= 2 ? 8 : 0, (k % 2) * 4, 4, k, 4 + k, 0}; }
  if (i < 12) {
    const int k = i - 4, kk = k % 4;
    return {1, k >= 4 ? 8 : 0, (kk / 2) * 4 + (kk % 2) * 3, (kk % 2) ? 1 : 3, 8 + k, 16 + k, 0};
  }
  const int k = i - 12;
  return {2, 0, 2 * k, 2, 24 + k, 28 + k, 0};
}





__device__ __forceinline__ f32x4 mfma(const uint32_t* a, const uint32_t* b, f32x4 c) {
  const f16x8 av = __builtin_bit_cast(f16x8, (u32x4){a[0], a[1], a[2], a[3]});
  const f16x8 bv = __builtin_bit_cast(f16x8, (u32x4){b[0], b[1], b[2], b[3]});
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, c, 0, 0, 0);
}

// Reductions over the four lane groups (lanes n, n+16, n+32, n+48) with the
// gfx950 lane-swap instructions: after v_permlane32_swap (v_permlane16_swap)
// of a register with itself, each lane holds its own value and that of lane
// l ^ 32 (l ^ 16) in the two results.
__device__ __forceinline__ float wave_max16x4(float v) {
  uint32_t r0, r1;
  lane_swap32(f2u(v), r0, r1);
  v = u2f(r0) > u2f(r1) ? u2f(r0) : u2f(r1);
  lane_swap16(f2u(v), r0, r1);
  return u2f(r0) > u2f(r1) ? u2f(r0) : u2f(r1);
}
// maximum of non-negative binary32 values, as bit patterns
__device__ __forceinline__ uint32_t wave_maxu16x4(uint32_t v) {
  uint32_t r0, r1;
  lane_swap32(v, r0, r1);
  v = max(r0, r1);
  lane_swap16(v, r0, r1);
  return max(r0, r1);
}
__device__ __forceinline__ float wave_sum16x4(float v) {
  uint32_t r0, r1;
  lane_swap32(f2u(v), r0, r1);
  v = u2f(r0) + u2f(r1);
  lane_swap16(f2u(v), r0, r1);
  return u2f(r0) + u2f(r1);
}

// Load 8 consecutive parameters starting at element e into f32.
template <int PDT>
__device__ __forceinline__ void load_params8(const void* base, int64_t e, float* out) {
  if constexpr (PDT == KVQ_E4M3) {
    // v_cvt_f32_fp8 converts OCP E4M3 on gfx950 (exact: every e4m3 value is a
    // binary32 value)
    const u32x2 v = *(const u32x2*)((const uint8_t*)base + e);
    out[0] = __builtin_amdgcn_cvt_f32_fp8((int)v[0], 0);
    out[1] = __builtin_amdgcn_cvt_f32_fp8((int)v[0], 1);
    out[2] = __builtin_amdgcn_cvt_f32_fp8((int)v[0], 2);
    out[3] = __builtin_amdgcn_cvt_f32_fp8((int)v[0], 3);
    out[4] = __builtin_amdgcn_cvt_f32_fp8((int)v[1], 0);
    out[5] = __builtin_amdgcn_cvt_f32_fp8((int)v[1], 1);
    out[6] = __builtin_amdgcn_cvt_f32_fp8((int)v[1], 2);
    out[7] = __builtin_amdgcn_cvt_f32_fp8((int)v[1], 3);
  } else if constexpr (PDT == KVQ_F32) {
    const u32x4 a = *(const u32x4*)((const float*)base + e);
    const u32x4 b = *(const u32x4*)((const float*)base + e + 4);
#pragma unroll
    for (int i = 0; i < 4; i++) { out[i] = u2f(a[i]); out[4 + i] = u2f(b[i]); }
  } else {
    const u32x4 v = *(const u32x4*)((const uint16_t*)base + e);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const uint32_t raw = (v[i / 2] >> (16 * (i % 2))) & 0xffffu;
      out[i] = (PDT == KVQ_F16) ? (float)__builtin_bit_cast(_Float16, (uint16_t)raw)
                                : bf16_bits_to_f32(raw);
    }
  }
}

struct DecodeArgs {
  Geo g;
  const uint16_t* q;  // bf16 [B][Hq][128]
  float* out;         // [B][Hq][128]
  float* part_ml;     // [BH][n_slots][G][2]   (running max in log2 units, sum)
  float* part_o;      // [BH][n_slots][G][128] (unnormalised output)
  int G, n_chunks, tpc, n_groups;
  int n_slots;        // partial slots per stream: n_chunks + residual slots
  unsigned* counters; // [n_groups] finished chunks per stream group: zero on
                      // entry, left zero (chunk combine inside the kernel)
  int fused;          // chunks combined inside the kernel (1) or by a second kernel (0)
  float sl2;          // softmax_scale * log2(e)
  // residual segment run by extra workgroups of this launch (grid rows past
  // n_groups), n_res blocks of 32 tokens per stream, partial slots
  // n_chunks .. n_chunks + n_res - 1; n_res = 0: none (or a separate launch)
  ResArgs res;
  int res_dtype, n_res;
};

// Operand registers per 32 codes and row words per lane for width B.
template <int B>
struct UInfo {
  static constexpr int NF = (B == 16) ? 32 : 16;
  static constexpr int NW = B;
};

// -1.0f in an SGPR that the compiler cannot see through: fma(h, -1, x) with
// a literal -1 is rewritten into a subtraction, which then needs the half
// widened first
__device__ __forceinline__ float opaque_m1() {
  uint32_t b;
  asm("s_mov_b32 %0, 0xbf800000" : "=s"(b));
  return __builtin_bit_cast(float, b);
}

// f16 split of a pair: hi = f16 truncation of x (one v_cvt_pkrtz for both),
// lo = f16 of the binary32 residual x - hi, which is exact (hi is x with low
// significand bits cleared); the residual reads hi's halves directly
// (v_fma_mix_f32 with m1 = -1), so the pair costs two conversions and two
// mixed fmas.
__device__ __forceinline__ void split_pack(float xl, float xh, uint32_t& hi, uint32_t& lo, float m1) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(xl, xh);
  hi = __builtin_bit_cast(uint32_t, h);
  const float rl = __builtin_fmaf((float)h[0], m1, xl);
  const float rh = __builtin_fmaf((float)h[1], m1, xh);
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(rl, rh));
}

// binary16 half i of a raw word array, widened exactly
__device__ __forceinline__ float half_at(const uint32_t* w, int i) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)((w[i >> 1] >> (16 * (i & 1))) & 0xffffu));
}
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
// larger of each 16-bit half (v_pk_max_u16)
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                __builtin_bit_cast(u16x2, b)));
}

// Value field weights.  Token i of a sub-tile (lane-local index) has its codes
// in field F of ufield<VB>, whose MFMA operand carries code * 2^(pos - 24);
// the probability operand carries 2^W(i), W = wexp - pos, to make up for it.
// 16-bit codes span two fields (low byte W = 0, high byte W = 8): W(i) is the
// first one's.
template <int VB, int FVS>
__host__ __device__ constexpr int tok_w(int i) {
  for (int ff = 0; ff < FVS; ff++) {
    const Fld F = ufield<VB>(ff);
    if (F.lo == i || F.hi == i) return F.wexp - F.pos;
  }
  return 0;
}
// class of a field weight (W is 0, -1 .. -9, or 8 for the high byte of 16-bit
// codes) and the weight of a class
__host__ __device__ constexpr int w_class(int w) { return w > 0 ? 1 : -w; }
template <int VB>
__host__ __device__ constexpr int class_w(int k) { return (VB == 16 && k == 1) ? 8 : -k; }
template <int VB, int FVS, int TPS>
__host__ __device__ constexpr bool class_used(int k) {
  for (int i = 0; i < TPS; i++)
    if (w_class(tok_w<VB, FVS>(i)) == k) return true;
  return false;
}

// device-scope store (written through the XCD's L2)
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// buffer resource over [base, base + bytes): raw buffer loads take a 32-bit
// lane offset plus SGPR/immediate offsets and return 0 beyond `bytes`
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// The field as an f16x2 operand register holding code * 2^(pos - 24) in each
// half: f16 subnormals are the integers times 2^-24, so masking the field in
// place is the whole conversion (MFMA consumes subnormal f16 exactly).
template <class F>
__device__ __forceinline__ uint32_t field_subnormal(uint32_t word, F f) {
  const uint32_t m = ((1u << f.wid) - 1u) << f.pos;
  const uint32_t x = f.sh ? (word >> f.sh) : word;
  return x & (m | (m << 16));
}





// binary32 of parameter I (compile-time) of a raw parameter-word array
template <int PDT, int I>
__device__ __forceinline__ float praw(const uint32_t* w) {
  if constexpr (PDT == KVQ_E4M3) {
    return __builtin_amdgcn_cvt_f32_fp8((int)w[I / 4], I % 4);   // OCP E4M3 on gfx950
  } else if constexpr (PDT == KVQ_F32) {
    return u2f(w[I]);
  } else if constexpr (PDT == KVQ_F16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)((w[I / 2] >> (16 * (I % 2))) & 0xffffu));
  } else {
    return u2f((I % 2) ? (w[I / 2] & 0xffff0000u) : (w[I / 2] << 16));
  }
}
// parameter i of a raw parameter-word array, i a constant after unrolling
template <int PDT>
__device__ __forceinline__ float pget(const uint32_t* w, int i) {
  if constexpr (PDT == KVQ_E4M3) {
    const int x = (int)w[i / 4];
    switch (i & 3) {
      case 0: return __builtin_amdgcn_cvt_f32_fp8(x, 0);
      case 1: return __builtin_amdgcn_cvt_f32_fp8(x, 1);
      case 2: return __builtin_amdgcn_cvt_f32_fp8(x, 2);
      default: return __builtin_amdgcn_cvt_f32_fp8(x, 3);
    }
  } else if constexpr (PDT == KVQ_F32) {
    return u2f(w[i]);
  } else if constexpr (PDT == KVQ_F16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)((w[i / 2] >> (16 * (i % 2))) & 0xffffu));
  } else {
    return u2f((i % 2) ? (w[i / 2] & 0xffff0000u) : (w[i / 2] << 16));
  }
}
template <int PDT, int N>
__device__ __forceinline__ void praw_unpack(const uint32_t* w, float* out) {
  if constexpr (N > 0) {
    praw_unpack<PDT, N - 1>(w, out);
    out[N - 1] = praw<PDT, N - 1>(w);
  }
}
// raw 32-bit words holding N parameters
template <int PDT, int N>
struct PW {
  static constexpr int W = (N * (PDT == KVQ_F32 ? 4 : (PDT == KVQ_E4M3 ? 1 : 2))) / 4;
};
// load N consecutive parameters (N * bytes a multiple of 4, offset aligned)
template <int PDT, int N>
__device__ __forceinline__ void pload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                      uint32_t* w) {
  constexpr int W = PW<PDT, N>::W;
  if constexpr (W % 4 == 0) {
#pragma unroll
    for (int i = 0; i < W; i += 4) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 4 * i, soff, KVQ_DECODE_CPOL_PARAMS);
      w[i] = v[0]; w[i + 1] = v[1]; w[i + 2] = v[2]; w[i + 3] = v[3];
    }
  } else if constexpr (W == 2) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, KVQ_DECODE_CPOL_PARAMS);
    w[0] = v[0]; w[1] = v[1];
  } else {
    static_assert(W == 1, "parameter group");
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, KVQ_DECODE_CPOL_PARAMS);
  }
}

// Waves per SIMD a decode instance is compiled for.  Two (two workgroups of 4
// waves per CU) wherever the instance fits in 256 registers per lane with at
// most a few spilled words -- the stream counts of ns_cap() are chosen for
// that; measured, a second resident wave hides more latency than any
// register-hungry schedule of a single one.  16-bit codes and mixed keys with
// 1-bit values need the full register file.
// waves per SIMD of three-stream 4-bit instances (they fit 256 registers).
// Three streams (15 of 16 columns for G = 5) measured no faster than two at
// two waves per SIMD, and 1.8x slower at one; 2-bit ones spill at two.
#ifndef KVQ_DECODE_NS3_OCC
#define KVQ_DECODE_NS3_OCC 1
#endif
constexpr int decode_occ(int kb, int vb, int pdt, int ns) {
  (void)pdt;
  if (KVQ_DECODE_WAVES_PER_SIMD) return KVQ_DECODE_WAVES_PER_SIMD;
  if (kb == 16 || (kb == 0 && vb == 1) || ns >= 4) return 1;
  if (ns == 3) return kb == 4 ? KVQ_DECODE_NS3_OCC : 1;
  return 2;
}

// KB: 16/8/4/2/1 or 0 (mixed keys).  VB: 16/8/4/2/1.  NS: kv streams packed
// into the 16 MFMA columns (column n serves stream n / G, head n % G).
//
// Main loop: the wave walks its tiles in sub-tiles of TPS tokens per lane
// group.  Sub-tile operands (key blocks, value words, value parameters) are
// double buffered in registers: the loads of the next sub-tile are issued
// before the current one is computed.  All loads are raw buffer loads with an
// SGPR base per (stream, tile) and lane offsets fixed for the whole kernel.
// The folded query u = q * S_K * 2^k (split into f16 hi + lo) lives in LDS,
// one 4-register group per k-step, computed once per tile.  Lanes of columns
// that serve no head have q = 0, so their operands are harmless and never
// masked.
// Residual segment: R tokens per stream that are not packed (the first and
// recent tokens the caller keeps at 16-bit or full precision), attended in
// binary32.  Workgroup (rc, bh) takes tokens [32 rc, 32 rc + 32) of stream bh
// and emits one more partial (m, l, o) per head in slot slot0 + rc -- or, when
// it is the only partial of the stream, the normalised row straight into
// `out`.  Every thread issues all its 16-byte loads (query, keys, values)
// before the first use, so a workgroup costs one memory round trip; logits,
// softmax and the value product then run out of LDS, the values taking the
// keys' place once the logits are formed (27 KB).  The same block runs as its
// own kernel or as extra workgroups of a decode launch (in the decode
// kernel's LDS), where the dispatcher starts it as decode workgroups retire.
template <int IN>
__device__ __forceinline__ float res_elem(uint4 w, int j) {
  if constexpr (IN == KVQ_F32) {
    return u2f(j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w);
  } else {
    const uint32_t x = (j >> 1) == 0 ? w.x : (j >> 1) == 1 ? w.y : (j >> 1) == 2 ? w.z : w.w;
    const uint32_t hbits = (j & 1) ? (x >> 16) : (x & 0xffffu);
    if constexpr (IN == KVQ_F16) return (float)__builtin_bit_cast(_Float16, (uint16_t)hbits);
    else return bf16_bits_to_f32(hbits);
  }
}

// LDS floats of a residual block: query [16][129], keys then values
// [32][129], weights [32][16], per-head (max, sum) [16][2]
constexpr int RES_LDS_FLOATS = 16 * 129 + KVQ_RES_CHUNK * 129 + KVQ_RES_CHUNK * 16 + 32;

template <int IN>
__device__ __forceinline__ void residual_block(const ResArgs& r, const uint16_t* __restrict__ q, int H, int G,
                                               float sl2, float* __restrict__ part_ml,
                                               float* __restrict__ part_o, int n_slots, int slot0,
                                               float* __restrict__ out, int rc, int bh, float* smem) {
  constexpr int RC = KVQ_RES_CHUNK;
  constexpr int VW = IN == KVQ_F32 ? 4 : 8;                 // elements per 16-byte load
  constexpr int NV = RC * 128 / VW / 256;                   // loads per thread per operand
  static_assert(RC == 32 && NV >= 1, "one token per half wave in the softmax");
  float (*qv)[129] = (float (*)[129])smem;                  // padded rows: conflict-free across tokens
  float (*kv)[129] = (float (*)[129])(smem + 16 * 129);     // keys, then values
  float (*sp)[16] = (float (*)[16])(smem + 16 * 129 + RC * 129);   // [token][head]: logits, then weights
  float (*sm)[2] = (float (*)[2])(smem + 16 * 129 + RC * 129 + RC * 16);   // per head: max, sum
  const int tid = threadIdx.x;
  const int b = bh / H, h = bh - (bh / H) * H;
  const int lane = tid & 63, wave = tid >> 6;
  const int t0 = rc * RC, n = min(RC, r.R - t0);
  const int64_t kb = (int64_t)b * r.ks[0] + (int64_t)h * r.ks[1] + (int64_t)t0 * r.ks[2];
  const int64_t vb = (int64_t)b * r.vs[0] + (int64_t)h * r.vs[1] + (int64_t)t0 * r.vs[2];
  const int esz = IN == KVQ_F32 ? 4 : 2;
  uint4 qw = make_uint4(0u, 0u, 0u, 0u);
  if (tid < G * 16) qw = ((const uint4*)(q + ((int64_t)b * H * G + (int64_t)h * G) * 128))[tid];
  // rows past n repeat row n - 1 (in bounds, never used): the loads need no branch
  uint4 kw[NV], vw[NV];
#pragma unroll
  for (int i = 0; i < NV; i++) {
    const int j = tid + 256 * i, t = min(j / (128 / VW), n - 1), c = (j % (128 / VW)) * VW;
    kw[i] = *(const uint4*)((const uint8_t*)r.k + (kb + (int64_t)t * r.ks[2] + c) * esz);
    vw[i] = *(const uint4*)((const uint8_t*)r.v + (vb + (int64_t)t * r.vs[2] + c) * esz);
  }
  if (tid < G * 16) {
#pragma unroll
    for (int e = 0; e < 8; e++) qv[tid >> 4][(tid & 15) * 8 + e] = res_elem<KVQ_BF16>(qw, e);
  }
#pragma unroll
  for (int i = 0; i < NV; i++) {
    const int j = tid + 256 * i, t = j / (128 / VW), c = (j % (128 / VW)) * VW;
#pragma unroll
    for (int e = 0; e < VW; e++) kv[t][c + e] = res_elem<IN>(kw[i], e);
  }
  __syncthreads();
  // logits: thread i takes head i / n, token i % n
  for (int i = tid; i < n * G; i += 256) {
    const int hh = i / n, t = i - (i / n) * n;
    float d = 0.0f;
#pragma unroll 16
    for (int c = 0; c < 128; c++) d = fmaf(qv[hh][c], kv[t][c], d);
    sp[t][hh] = d * sl2;
  }
  __syncthreads();
  // the values take the keys' place (read again only after the next barrier)
#pragma unroll
  for (int i = 0; i < NV; i++) {
    const int j = tid + 256 * i, t = j / (128 / VW), c = (j % (128 / VW)) * VW;
#pragma unroll
    for (int e = 0; e < VW; e++) kv[t][c + e] = res_elem<IN>(vw[i], e);
  }
  // softmax: each wave takes two heads at a time, one per half wave (lane & 31 = token)
  for (int hp = wave; 2 * hp < G; hp += 4) {
    const int hh = 2 * hp + (lane >> 5), t = lane & 31;
    const bool ok = hh < G && t < n;
    const float s = ok ? sp[t][hh] : -INFINITY;
    float m = s;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    const float e = ok ? exp2f(s - m) : 0.0f;
    float l = e;
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);
    if (hh < G) {
      sp[t][hh] = e;                              // 0 for the rows past n
      if (t == 0) { sm[hh][0] = m; sm[hh][1] = l; }
    }
  }
  __syncthreads();
  // values: thread takes channel tid & 127 and heads 8 hb .. 8 hb + 7 (hb =
  // tid >> 7, uniform per wave); the sums of heads >= G are never stored
  const int c = tid & 127, hb = tid >> 7;
  if (8 * hb >= G) return;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; j++) acc[j] = 0.0f;
#pragma unroll 4
  for (int t = 0; t < n; t++) {
    const float x = kv[t][c];
    const float4 w0 = *(const float4*)&sp[t][8 * hb];
    const float4 w1 = *(const float4*)&sp[t][8 * hb + 4];
    acc[0] = fmaf(w0.x, x, acc[0]);
    acc[1] = fmaf(w0.y, x, acc[1]);
    acc[2] = fmaf(w0.z, x, acc[2]);
    acc[3] = fmaf(w0.w, x, acc[3]);
    acc[4] = fmaf(w1.x, x, acc[4]);
    acc[5] = fmaf(w1.y, x, acc[5]);
    acc[6] = fmaf(w1.z, x, acc[6]);
    acc[7] = fmaf(w1.w, x, acc[7]);
  }
#pragma unroll
  for (int j = 0; j < 8; j++) {
    const int hh = 8 * hb + j;
    if (hh >= G) break;
    if (out) {
      out[((int64_t)b * H * G + (int64_t)h * G + hh) * 128 + c] = acc[j] / sm[hh][1];
    } else {
      const int64_t row = ((int64_t)bh * n_slots + slot0 + rc) * G + hh;
      if (c == 0) { part_ml[2 * row] = sm[hh][0]; part_ml[2 * row + 1] = sm[hh][1]; }
      part_o[row * 128 + c] = acc[j];
    }
  }
}

template <int IN>
__global__ __launch_bounds__(256) void decode_residual_kernel(ResArgs r, const uint16_t* __restrict__ q,
                                                              int H, int G, float sl2,
                                                              float* __restrict__ part_ml,
                                                              float* __restrict__ part_o, int n_slots,
                                                              int slot0, float* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) float smem[RES_LDS_FLOATS];
  residual_block<IN>(r, q, H, G, sl2, part_ml, part_o, n_slots, slot0, out, blockIdx.x, blockIdx.y, smem);
}

template <int KB, int VB, int PDT, int NS>
__global__ __launch_bounds__(256, decode_occ(KB, VB, PDT, NS)) void decode_kernel(DecodeArgs a) {
  constexpr bool MIXED = (KB == 0);
  constexpr int NFK = MIXED ? 16 : UInfo<KB>::NF;    // key operand registers per token
  constexpr int NWK = MIXED ? 3 : UInfo<KB>::NW;     // key words per lane per token
  constexpr int NKK = NFK / 4;                       // key k-steps
  constexpr int NFV = UInfo<VB>::NF;
  constexpr int NWV = UInfo<VB>::NW;
  constexpr int NSUB0 = (VB == 1) ? 1 : ((VB == 2) ? 2 : 4);
  constexpr int NSUB = NSUB0 < KVQ_DECODE_NSUB_MAX ? NSUB0 : KVQ_DECODE_NSUB_MAX;  // sub-tiles per tile
  constexpr int TPS = 32 / NSUB;                     // tokens per lane per sub-tile
  constexpr int JB = 8 / NSUB;                       // key blocks per sub-tile
  constexpr int FVS = NFV / NSUB;                    // value fields per sub-tile
  constexpr int WVS = NWV / NSUB;                    // value words per sub-tile
  constexpr int KSV = FVS / 4;                       // value k-steps per sub-tile
  constexpr int PB = (PDT == KVQ_F32) ? 4 : ((PDT == KVQ_E4M3) ? 1 : 2);
  constexpr int PWV = PW<PDT, TPS>::W;               // value-parameter words per sub-tile
  constexpr int PWK = PW<PDT, 8>::W;                 // key-parameter words per 8 slots
  constexpr int KPA = 32 * PB;                       // words per 128 key parameters
  constexpr int KPL = (PB == 4) ? 2 : 1;             // of which one lane loads
  // Headroom exponents keep every f16 operand below 2^15: |u| < 2^(KH+2) and
  // P = e * S_V * 2^(VH - E) < 2^(VH + 1 + TAU), times the field weights.
  constexpr int TAU = 8;                             // lazy-max slack (log2 units)
  constexpr int KH = (KB == 16) ? 4 : 12;
  constexpr int VH = (VB == 16) ? -2 : 6;
  // largest probability shift: e * 2^ps * 2^W stays below 2^(TAU + PSMAX + 8)
  // and its sums over a chunk below 2^127
  constexpr int PSMAX = 96;
  constexpr int ROW_K = MIXED ? 8 : 16 * KB;
  constexpr int LDS_WAVE = NFK * 2 * 64;             // u32 words of folded query per wave
  constexpr int CPOL = (KB == 16) ? 0 : KVQ_DECODE_CPOL_CODES;
  static_assert(KSV >= 1 && WVS >= 1, "sub-tile must hold whole value k-steps");
  static_assert(LDS_WAVE >= 16 * 128 && TPS % 8 == 0, "layout assumptions");

  // folded query (per wave) during the loop; the wave partial afterwards
  __shared__ __attribute__((aligned(16))) uint32_t lds[4][LDS_WAVE];
  // key scales / zeros of the current tile of each stream, per wave
  __shared__ __attribute__((aligned(16))) uint32_t kst[4][NS][2][KPA];
  // query heads of the group in slot order
  __shared__ __attribute__((aligned(16))) uint16_t qs[16][128];

  const Geo& g = a.g;
  if (blockIdx.y >= (unsigned)a.n_groups) {
    // a residual workgroup: block r of the grid rows past the stream groups
    const int r = (blockIdx.y - a.n_groups) * gridDim.x + blockIdx.x;
    const int BHr = g.B * g.H;
    if (r >= a.n_res * BHr) return;
    static_assert(sizeof(lds) >= RES_LDS_FLOATS * sizeof(float), "residual block fits the decode LDS");
    float* smem = (float*)&lds[0][0];
    const int rc = r % a.n_res, bh = r / a.n_res;
    if (a.res_dtype == KVQ_F32)
      residual_block<KVQ_F32>(a.res, a.q, g.H, a.G, a.sl2, a.part_ml, a.part_o, a.n_slots, a.n_chunks, nullptr,
                              rc, bh, smem);
    else if (a.res_dtype == KVQ_F16)
      residual_block<KVQ_F16>(a.res, a.q, g.H, a.G, a.sl2, a.part_ml, a.part_o, a.n_slots, a.n_chunks, nullptr,
                              rc, bh, smem);
    else
      residual_block<KVQ_BF16>(a.res, a.q, g.H, a.G, a.sl2, a.part_ml, a.part_o, a.n_slots, a.n_chunks,
                               nullptr, rc, bh, smem);
    return;
  }
  // the wave index is uniform: keep it (and everything derived) in SGPRs
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, lg = lane >> 4;
  // consecutive workgroup ids (which the dispatcher deals out to the XCDs in
  // turn) walk the chunks of one stream group
  const int grp = blockIdx.y;
  const int chunk = blockIdx.x;
  const int G = a.G;
  const int BH = g.B * g.H;
  const int own = n / G;
  const int bh_own = grp * NS + own;
  const bool real = (own < NS) && (bh_own < BH);
  // the chunk's tiles, numbered k = 0 .. t_count-1: tile = t_base + k
  const int t_count = min(a.tpc, g.n_tiles - chunk * a.tpc);
  const int t_base = chunk * a.tpc;

  auto kslot = [&](int li) -> int {
    if constexpr (MIXED) return lg == 0 ? (li < 24 ? li : 96 + li) : 32 * lg - 8 + li;
    else return 32 * lg + li;
  };

  // ---- lane offsets, fixed for the whole kernel
  // key block j row r = 32*(n/4) + 4j + n%4; the lane reads its lane group's
  // 4*KB bytes of the row (mixed: its plane's 8 bytes, lane group 0 also the
  // 2 plane-4 bytes)
  const uint32_t row0 = 32 * (n >> 2) + (n & 3);
  const uint32_t koff = MIXED ? (uint32_t)((lg == 0 ? 0 : 1024 * lg) + 8 * row0)
                              : (uint32_t)(row0 * ROW_K + 4 * KB * lg);
  const uint32_t koff4 = 4096 + 2 * row0;                       // mixed plane 4
  const uint32_t voff4 = (uint32_t)(4 * n + lg) * 16;           // value words (w, h, n, lg, 0..3)
  // parameter arrays from the group's first stream on (offsets stay below 2^32:
  // the host bounds max_tokens)
  const int64_t s0 = (int64_t)grp * NS;
  const int own_c = real ? own : 0;
  const uint32_t vpoff = (uint32_t)(((int64_t)own_c * g.max_tokens + 32 * lg) * PB);
  const __amdgpu_buffer_rsrc_t r_vs = rsrc((const uint8_t*)g.v_scale + s0 * g.max_tokens * PB, 0xffffffffu);
  const __amdgpu_buffer_rsrc_t r_vz = rsrc((const uint8_t*)g.v_zero + s0 * g.max_tokens * PB, 0xffffffffu);
  const __amdgpu_buffer_rsrc_t r_ks = rsrc((const uint8_t*)g.k_scale + s0 * g.max_tokens * PB, 0xffffffffu);
  const __amdgpu_buffer_rsrc_t r_kz = rsrc((const uint8_t*)g.k_zero + s0 * g.max_tokens * PB, 0xffffffffu);
  // key parameters: lane l loads word l (and l + 64) of the tile's 128 (e4m3:
  // lanes 32.. repeat words 0..31)
  const uint32_t kloff = (uint32_t)((PB == 1) ? (lane & 31) : lane) * 4;

  float m_run = -INFINITY, l_run = 0.0f, z_run = 0.0f;
  int e_run = -1000;
  const float m1 = opaque_m1();
  float ak = 0.0f, bk0 = 0.0f;
  // output accumulators, shared by the packed streams (the probabilities are
  // masked per stream)
  f32x4 acc_o[8];
#pragma unroll
  for (int cb = 0; cb < 8; cb++) acc_o[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  uint32_t* my_lds = lds[wave];

  // one sub-tile of raw operands; value words travel outside the prefetch
  // buffers: they are loaded at the start of their own sub-tile (in flight
  // during its key product and softmax)
  struct Buf {
    uint32_t kw[NS][JB][NWK];
    uint32_t vs[PWV], vz[PWV];
    uint32_t kp[NS][2][KPL];   // next tile's key scales / zeros (sub-tile 0 only)
  };

  // value word planes: word (w, c = 64h + 16q + n, a) at word index
  // w*512 + ((h*16 + n)*4 + a)*4 + q, so lane (n, lg) finds the words of its
  // channels n, 16+n, 32+n, 48+n (h = 0) and 64+n, ... (h = 1) as 16
  // contiguous bytes: two 16-byte loads per plane, 1 KB per wave each
  auto load_vw = [&](uint32_t* vw, __amdgpu_buffer_rsrc_t rv, int sub) {
#pragma unroll
    for (int w = 0; w < WVS; w++)
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const u32x4 v4 = __builtin_amdgcn_raw_buffer_load_b128(rv, voff4, (uint32_t)(sub * WVS + w) * 2048 + 1024 * h, CPOL);
#pragma unroll
        for (int q = 0; q < 4; q++) vw[(4 * h + q) * WVS + w] = v4[q];
      }
  };
  auto v_rsrc = [&](int s, int tile) {
    const int bh = min(grp * NS + s, BH - 1);
    return rsrc(g.v_codes + v_tile_offset(g, bh / g.H, bh % g.H, tile), 2048 * VB);
  };

  // sub-tile `sub` (a constant after unrolling) of the chunk's tile k: key
  // blocks (and, for sub-tile 0, the tile's key parameters) ...
  auto load_k = [&](Buf& bf, int k, int sub) {
    const int tile = t_base + k;
#pragma unroll
    for (int s = 0; s < NS; s++) {
      const int bh = min(grp * NS + s, BH - 1);   // a missing stream re-reads a valid one
      const int bs = bh / g.H, hs = bh % g.H;
      const __amdgpu_buffer_rsrc_t rk =
          rsrc(g.k_codes + k_tile_offset(g, bs, hs, tile), MIXED ? KVQ_MIXED_TILE_BYTES : 2048 * KB);
#pragma unroll
      for (int jj = 0; jj < JB; jj++) {
        const uint32_t soff = (uint32_t)(sub * JB) * 4 * ROW_K;       // rows 4j apart
        if constexpr (MIXED) {
          const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rk, koff + jj * 32, soff, CPOL);
          const uint32_t w2 = __builtin_amdgcn_raw_buffer_load_b16(rk, koff4 + jj * 8, soff / 4, CPOL);
          bf.kw[s][jj][0] = v[0];
          bf.kw[s][jj][1] = v[1];
          bf.kw[s][jj][2] = (w2 & 0xffu) | ((w2 & 0xff00u) << 8);
        } else if constexpr (NWK >= 4) {
#pragma unroll
          for (int w = 0; w < NWK; w += 4) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rk, koff + jj * 4 * ROW_K + 4 * w, soff, CPOL);
            bf.kw[s][jj][w] = v[0]; bf.kw[s][jj][w + 1] = v[1];
            bf.kw[s][jj][w + 2] = v[2]; bf.kw[s][jj][w + 3] = v[3];
          }
        } else if constexpr (NWK == 2) {
          const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rk, koff + jj * 4 * ROW_K, soff, CPOL);
          bf.kw[s][jj][0] = v[0]; bf.kw[s][jj][1] = v[1];
        } else {
          bf.kw[s][jj][0] = __builtin_amdgcn_raw_buffer_load_b32(rk, koff + jj * 4 * ROW_K, soff, CPOL);
        }
      }
    }
    if (sub == 0) {
#pragma unroll
      for (int s = 0; s < NS; s++) {
        const int bh = min(grp * NS + s, BH - 1);
        const uint32_t soff = (uint32_t)((((int64_t)(bh - grp * NS)) * g.max_tiles + tile) * 128 * PB);
#pragma unroll
        for (int j = 0; j < KPL; j++) {
          bf.kp[s][0][j] = __builtin_amdgcn_raw_buffer_load_b32(r_ks, kloff + 256 * j, soff, KVQ_DECODE_CPOL_PARAMS);
          bf.kp[s][1][j] = __builtin_amdgcn_raw_buffer_load_b32(r_kz, kloff + 256 * j, soff, KVQ_DECODE_CPOL_PARAMS);
        }
      }
    }
  };
  // ... and the own stream's value scales / zeros of the lane's TPS tokens
  auto load_p = [&](Buf& bf, int k, int sub) {
    const int tile = t_base + k;
    const uint32_t psoff = (uint32_t)(tile * 128 + sub * TPS) * PB;
    pload<PDT, TPS>(r_vs, vpoff, psoff, bf.vs);
    pload<PDT, TPS>(r_vz, vpoff, psoff, bf.vz);
  };
  auto load = [&](Buf& bf, int k, int sub) {
    load_k(bf, k, sub);
    load_p(bf, k, sub);
  };

  // the first sub-tile's loads are in flight while the query is staged
  Buf b0, b1;
  // wave w takes the chunk's tiles k = w, w + 4, ...; the queue holds its next four
  int q0 = wave, q1, q2, q3;
  // ---- the query heads of the group in slot order, [column][slot] bf16 in
  // LDS (column n = stream n / G, head n % G; zero for columns without a
  // head).  Column cn is query row grp * NS * G + cn of q (rows are
  // (batch, kv head, head) in order), valid while cn < NS * G and the row is
  // inside q.  The query loads go out before the first tile's loads, so they
  // are not queued behind them when every workgroup starts at once.
  // a negative softmax scale is folded into the staged query (bf16 sign
  // flips are exact), so ak >= 0 and a lane's largest logit always comes from
  // its largest raw sum
  const uint32_t qflip = (a.sl2 < 0.0f) ? 0x80008000u : 0u;
  if constexpr (!MIXED) {
    // uniform widths: slot = channel, one 16-byte load per thread
    const int cn = threadIdx.x >> 4, part = threadIdx.x & 15;
    const int64_t row = (int64_t)grp * NS * G + cn;
    u32x4 v = (u32x4){0u, 0u, 0u, 0u};
    if (cn < NS * G && row < (int64_t)BH * G) v = *(const u32x4*)(a.q + row * 128 + 8 * part);
    v ^= (u32x4)qflip;
    if (q0 < t_count) load(b0, q0, 0);
    *(u32x4*)&qs[cn][8 * part] = v;
  } else {
    // mixed widths: slot j holds channel slot_chan[kv head][j]
    uint16_t qv[8];
#pragma unroll
    for (int r = 0; r < 8; r++) {
      const int i = threadIdx.x + 256 * r;
      const int cn = i >> 7, j = i & 127;
      const int cs = cn / G;
      const int cbh = grp * NS + cs;
      qv[r] = 0;
      if (cs < NS && cbh < BH) {
        const int chh = cbh % g.H;
        qv[r] = a.q[((int64_t)grp * NS * G + cn) * 128 + g.slot_chan[chh * 128 + j]] ^ (uint16_t)qflip;
      }
    }
    if (q0 < t_count) load(b0, q0, 0);
#pragma unroll
    for (int r = 0; r < 8; r++) {
      const int i = threadIdx.x + 256 * r;
      qs[i >> 7][i & 127] = qv[r];
    }
  }
  __syncthreads();
  // the lane's 32 query values (slots kslot(0..31)) as bf16 pairs
  auto load_q = [&](uint32_t* qw) {
#pragma unroll
    for (int c = 0; c < 4; c++) {
      const u32x4 v = *(const u32x4*)&qs[n][kslot(8 * c)];
      qw[4 * c] = v[0]; qw[4 * c + 1] = v[1]; qw[4 * c + 2] = v[2]; qw[4 * c + 3] = v[3];
    }
  };
  auto qget = [](const uint32_t* qw, int li) -> float {
    return (li & 1) ? u2f(qw[li >> 1] & 0xffff0000u) : u2f(qw[li >> 1] << 16);
  };
  int eq;
  {
    uint32_t qw[16];
    load_q(qw);
    uint32_t qmax = 0;
#pragma unroll
    for (int li = 0; li < 32; li++) qmax = max(qmax, f2u(qget(qw, li)) & 0x7fffffffu);
    eq = expo(u2f(wave_maxu16x4(qmax)));
  }

  // fold the key scales of `tile` into the query: u = q * S * 2^k as f16 hi/lo
  // operand registers in LDS; logit constants ak, bk0
  auto fold_query = [&](const Buf& bf) {
    // stage the tile's key parameters in LDS, then read the own stream's 32
    // slots (four runs of 8 consecutive slots)
#pragma unroll
    for (int s = 0; s < NS; s++)
#pragma unroll
      for (int a2 = 0; a2 < 2; a2++)
#pragma unroll
        for (int j = 0; j < KPL; j++) kst[wave][s][a2][(kloff >> 2) + 64 * j] = bf.kp[s][a2][j];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // raw words of the lane's 32 key parameters (four runs of 8 slots)
    auto load_kp = [&](int which, uint32_t* pw) {
#pragma unroll
      for (int s4 = 0; s4 < 4; s4++) {
        const int wo = kslot(8 * s4) * PB / 4;
#pragma unroll
        for (int i = 0; i < PWK; i++) pw[s4 * PWK + i] = kst[wave][own_c][which][wo + i];
      }
    };
    uint32_t qw[16];
    load_q(qw);
    // beta in four independent chains (a single chain of 32 fmas is latency bound)
    float beta;
    {
      uint32_t zw[4 * PWK];
      load_kp(1, zw);
      float bc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int li = 0; li < 32; li++) bc[li & 3] = fmaf(qget(qw, li), pget<PDT>(zw, li), bc[li & 3]);
      beta = (bc[0] + bc[1]) + (bc[2] + bc[3]);
    }
    uint32_t sw[4 * PWK];
    load_kp(0, sw);
    uint32_t smax = 0;
    if constexpr (PDT == KVQ_F16) {
      // scales are >= +0, so their binary16 patterns order like the values
      uint32_t m2 = sw[0];
#pragma unroll
      for (int i = 1; i < 4 * PWK; i++) m2 = pk_max_u16(m2, sw[i]);
      smax = f2u((float)__builtin_bit_cast(_Float16, (uint16_t)max(m2 & 0xffffu, m2 >> 16)));
    } else {
#pragma unroll
      for (int li = 0; li < 32; li++) smax = max(smax, f2u(pget<PDT>(sw, li)));   // scales are >= +0
    }
    // eq + es is bounded below so that kf * 2^(field weight) stays finite when
    // a tile's scales are all zero (codes then 0, u = 0)
    const int eqs = max(eq + expo(u2f(wave_maxu16x4(smax))), -100);
    beta = wave_sum16x4(beta);
    const float kf = exp2i(KH - eqs);
    // q * S; a binary16 scale is read by a mixed fma (+0 addend: the product
    // itself, up to the sign of a zero)
    auto uval = [&](int li) -> float {
      if constexpr (PDT == KVQ_F16) return __builtin_fmaf(qget(qw, li), pget<PDT>(sw, li), 0.0f);
      else return qget(qw, li) * pget<PDT>(sw, li);
    };
#pragma unroll
    for (int f = 0; f < NFK; f++) {
      float ul, uh, w;
      if constexpr (MIXED) {
        const Fld F0 = mfield0(f), F1 = ufield<2>(f);
        ul = (lg == 0) ? uval(F0.lo) : uval(F1.lo);
        uh = (lg == 0) ? uval(F0.hi) : uval(F1.hi);
        w = kf * ((lg == 0) ? exp2i(F0.wexp - F0.pos) : exp2i(F1.wexp - F1.pos));
      } else {
        const Fld F = ufield<KB>(f);
        ul = uval(F.lo);
        uh = uval(F.hi);
        w = kf * exp2i(F.wexp - F.pos);
      }
      uint32_t hi, lo;
      split_pack(ul * w, uh * w, hi, lo, m1);
      // [k-step][hi/lo][lane][4]: one ds_read_b128 per operand group
      my_lds[(((f >> 2) * 2 + 0) * 64 + lane) * 4 + (f & 3)] = hi;
      my_lds[(((f >> 2) * 2 + 1) * 64 + lane) * 4 + (f & 3)] = lo;
    }
    ak = __builtin_fabsf(a.sl2) * exp2i(24 - KH + eqs);
    bk0 = __builtin_fabsf(a.sl2) * beta;
  };

  // compute sub-tile sub of the chunk's tile ti from bf; with the two-ahead
  // prefetch, bf is refilled with sub-tile (ti2, sub2) as soon as each part has
  // been read
  auto issue_v = [&](uint32_t* vw, int k, int sub) {
#pragma unroll
    for (int s = 0; s < NS; s++) load_vw(vw + s * 8 * WVS, v_rsrc(s, t_base + k), sub);
  };
  auto compute = [&](Buf& bf, int ti, int sub, int ti2, int sub2) {
    uint32_t vjit[NS * 8 * WVS];
    issue_v(vjit, ti, sub);
    const uint32_t* vwp = vjit;
    if (sub == 0) fold_query(bf);
    // ---- logits: k-step-major over all (stream, block) accumulators
    f32x4 acc[NS][JB];
#pragma unroll
    for (int s = 0; s < NS; s++)
#pragma unroll
      for (int jj = 0; jj < JB; jj++) acc[s][jj] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NKK; k++) {
      const u32x4 bhv = *(const u32x4*)(my_lds + ((k * 2 + 0) * 64 + lane) * 4);
      const u32x4 blv = *(const u32x4*)(my_lds + ((k * 2 + 1) * 64 + lane) * 4);
      const uint32_t bh4[4] = {bhv[0], bhv[1], bhv[2], bhv[3]};
      const uint32_t bl4[4] = {blv[0], blv[1], blv[2], blv[3]};
      uint32_t av[NS][JB][4];
#pragma unroll
      for (int s = 0; s < NS; s++)
#pragma unroll
        for (int jj = 0; jj < JB; jj++)
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const int f = 4 * k + r;
            if constexpr (MIXED) {
              const uint32_t x0 = field_subnormal(bf.kw[s][jj][mfield0(f).w], mfield0(f));
              const uint32_t x1 = field_subnormal(bf.kw[s][jj][ufield<2>(f).w], ufield<2>(f));
              av[s][jj][r] = (lg == 0) ? x0 : x1;
            } else {
              av[s][jj][r] = field_subnormal(bf.kw[s][jj][ufield<KB>(f).w], ufield<KB>(f));
            }
          }
#pragma unroll
      for (int s = 0; s < NS; s++)
#pragma unroll
        for (int jj = 0; jj < JB; jj++) acc[s][jj] = mfma(av[s][jj], bh4, acc[s][jj]);
#pragma unroll
      for (int s = 0; s < NS; s++)
#pragma unroll
        for (int jj = 0; jj < JB; jj++) acc[s][jj] = mfma(av[s][jj], bl4, acc[s][jj]);
    }
    load_k(bf, ti2, sub2);
    // ---- logits l = ak * v + bk0 (v the column's own raw sum) and an online
    // softmax with a lazy running max: the reference m_run only moves when a
    // logit exceeds it by more than TAU (so e <= 2^TAU), and the accumulator
    // is rescaled only when some column's reference moved
    float lv[TPS];
#pragma unroll
    for (int jj = 0; jj < JB; jj++) {
      f32x4 v = acc[0][jj];
#pragma unroll
      for (int s = 1; s < NS; s++)
        if (own == s) v = acc[s][jj];
#pragma unroll
      for (int i = 0; i < 4; i++) lv[4 * jj + i] = v[i];
    }
    // the lane's largest logit (ak >= 0: from its largest raw sum)
    float vx = lv[0];
#pragma unroll
    for (int i = 1; i < TPS; i++) vx = fmaxf(vx, lv[i]);
    const float lmax = fmaf(ak, vx, bk0);
    // value parameters of the sub-tile; binary16 ones stay raw and are read
    // by mixed-precision fmas.  smx: the lane's largest value scale as a
    // binary32 bit pattern (scales are >= +0, so patterns order like values)
    constexpr bool MIX = (PDT == KVQ_F16);
    uint32_t rvs[PWV], rvz[PWV];
    float vs[MIX ? 1 : TPS], vz[MIX ? 1 : TPS];
    uint32_t smx;
    if constexpr (MIX) {
#pragma unroll
      for (int w = 0; w < PWV; w++) { rvs[w] = bf.vs[w]; rvz[w] = bf.vz[w]; }
      uint32_t m2 = rvs[0];
#pragma unroll
      for (int w = 1; w < PWV; w++) m2 = pk_max_u16(m2, rvs[w]);
      smx = f2u((float)__builtin_bit_cast(_Float16, (uint16_t)max(m2 & 0xffffu, m2 >> 16)));
    } else {
      praw_unpack<PDT, TPS>(bf.vs, vs);
      praw_unpack<PDT, TPS>(bf.vz, vz);
      smx = 0;
#pragma unroll
      for (int i = 0; i < TPS; i++) smx = max(smx, f2u(vs[i]));
    }
    load_p(bf, ti2, sub2);
    // A column's reference max moves only when one of its logits exceeds it
    // by more than TAU, and its value-scale exponent e_run only when a larger
    // scale arrives.  Both need the reductions over the four lane groups, so
    // they (and the rescale of the running sums and accumulators) run only
    // when some lane of the wave sees such a logit or scale.
    if (__builtin_amdgcn_ballot_w64(lmax > m_run + (float)TAU || expo(u2f(smx)) > e_run) != 0) {
      const float tmax = wave_max16x4(lmax);
      const int ev = expo(u2f(wave_maxu16x4(smx)));
      const float m_new = (tmax > m_run + (float)TAU) ? tmax : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // v_exp_f32, 0 for -inf
      const int e_new = max(e_run, ev);
      // the probabilities carry 2^ps, ps = VH - e_run (capped so the scaled
      // sums stay finite), which keeps the value operand below 2^15
      const int ps_old = min(VH - e_run, PSMAX), ps_new = min(VH - e_new, PSMAX);
      const float rescale = alpha * exp2i(ps_new - ps_old);
      m_run = m_new;
      e_run = e_new;
      l_run *= rescale;
      z_run *= rescale;
#pragma unroll
      for (int cb = 0; cb < 8; cb++) acc_o[cb] *= rescale;
    }
    // e''(i) = e(i) * 2^ps * 2^W(i) straight from the exponent; the running
    // sums l_run, z_run are kept in units of 2^ps
    const float c0 = bk0 - m_run + (float)min(VH - e_run, PSMAX);
    float p[TPS];
    float lsum = 0.0f;
    float zc[10];
#pragma unroll
    for (int k = 0; k < 10; k++) zc[k] = 0.0f;
#pragma unroll
    for (int i = 0; i < TPS; i++) {
      const int W = tok_w<VB, FVS>(i);
      const float e = __builtin_amdgcn_exp2f(fmaf(ak, lv[i], c0 + (float)W));
      lsum = fmaf(e, exp2i(-W), lsum);
      if constexpr (MIX) {
        zc[w_class(W)] = fmaf(e, half_at(rvz, i), zc[w_class(W)]);
        p[i] = fmaf(e, half_at(rvs, i), 0.0f);
      } else {
        zc[w_class(W)] = fmaf(e, vz[i], zc[w_class(W)]);
        p[i] = e * vs[i];
      }
    }
    float zsum = zc[0];
#pragma unroll
    for (int k = 1; k < 10; k++)
      if (class_used<VB, FVS, TPS>(k)) zsum = fmaf(zc[k], exp2i(-class_w<VB>(k)), zsum);
    l_run += lsum;
    z_run += zsum;

    // ---- P operand (split hi/lo) and PV; every sub-tile has the field
    // layout of sub-tile 0, shifted by WVS words and TPS tokens
    uint32_t bvh[FVS], bvl[FVS];
#pragma unroll
    for (int ff = 0; ff < FVS; ff++) {
      // a token whose codes span two fields (the bytes of a 16-bit code)
      // carries the weight of its first field; the other gets the difference
      const Fld F = ufield<VB>(ff);
      const float dw = exp2i((F.wexp - F.pos) - tok_w<VB, FVS>(F.lo));
      split_pack(p[F.lo] * dw, p[F.hi] * dw, bvh[ff], bvl[ff], m1);
    }
#pragma unroll
    for (int s = 0; s < NS; s++) {
      uint32_t bsh[FVS], bsl[FVS];
#pragma unroll
      for (int ff = 0; ff < FVS; ff++) {
        const bool sel = (NS == 1) || (own == s);
        bsh[ff] = sel ? bvh[ff] : 0u;
        bsl[ff] = sel ? bvl[ff] : 0u;
      }
      f32x4* ao = acc_o;
#pragma unroll
      for (int k = 0; k < KSV; k++) {
        uint32_t av[8][4];
#pragma unroll
        for (int cb = 0; cb < 8; cb++)
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const Fld F = ufield<VB>(4 * k + r);
            av[cb][r] = field_subnormal(vwp[(s * 8 + cb) * WVS + F.w], F);
          }
#pragma unroll
        for (int cb = 0; cb < 8; cb++) ao[cb] = mfma(av[cb], bsh + 4 * k, ao[cb]);
#pragma unroll
        for (int cb = 0; cb < 8; cb++) ao[cb] = mfma(av[cb], bsl + 4 * k, ao[cb]);
      }
    }
  };

  // ---- software-pipelined main loop (two register buffers).  One iteration
  // covers U sub-tiles (a whole tile, or two one-sub-tile tiles) unrolled, so
  // the fold and every buffer choice are compile-time; the prefetch of the
  // sub-tile after the wave's last one re-reads that last one (harmless, in
  // bounds) instead of branching.
  constexpr int U = NSUB >= 2 ? NSUB : 2;
  constexpr int TPI = U / NSUB;   // tiles per iteration (2 for one-sub-tile tiles)
  q1 = q0 + 4; q2 = q0 + 8; q3 = q0 + 12;
  // the queue entry for sub-tile offset d (d = 0..3 tiles ahead), a valid tile
  // when it lies past the chunk (such prefetches are never consumed)
  auto qk = [&](int d) -> int {
    const int v = d == 0 ? q0 : (d == 1 ? q1 : (d == 2 ? q2 : q3));
    return v < t_count ? v : q0;
  };
  // the second buffer: loads run two sub-tiles ahead of the computation
  if (q0 < t_count) load(b1, qk(1 / NSUB), 1 % NSUB);
#pragma unroll 1
  while (q0 < t_count) {
    if constexpr (KVQ_DECODE_PRIO != 0) {
      // The two workgroups sharing a CU have equal work, but the hardware
      // issues the older wave first when both are ready, so the older one
      // would finish early and leave its SIMDs half idle.  The wave with more
      // tiles left runs at the higher priority instead.
      const int rem = (t_count - q0 + 3) / 4 - 1;
      if (rem >= 3) __builtin_amdgcn_s_setprio(3);
      else if (rem == 2) __builtin_amdgcn_s_setprio(2);
      else if (rem == 1) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      if constexpr (NSUB == 1) {
        if (u == 1 && q1 >= t_count) break;
      }
      compute((u % 2 == 0) ? b0 : b1, qk(u / NSUB), u % NSUB, qk((u + 2) / NSUB), (u + 2) % NSUB);
    }
    if constexpr (TPI == 1) {
      q0 = q1; q1 = q2; q2 = q3;
      q3 = q3 + 4;
    } else {
      q0 = q2; q1 = q3;
      q2 = q2 + 8;
      q3 = q3 + 8;
    }
  }

  // ---- wave partial -> LDS -> workgroup partial (per column = stream, head);
  // each wave overwrites only its own LDS region, which it no longer reads
  __shared__ float sh_ml[4][16][2];
  // wave w's partial [16][128] sits at the start of ITS OWN region lds[w]
  // (regions are LDS_WAVE words apart, more than 16*128 for 16-bit codes)
  auto sh_o = [&](int w, int col, int c) -> float& { return ((float*)&lds[w][0])[col * 128 + c]; };
  static_assert(sizeof(lds[0]) >= sizeof(float) * 16 * 128, "partial fits the wave region");
  const int ps = min(VH - e_run, PSMAX);
  const float unps = exp2i(-ps);
  const float l_tot = wave_sum16x4(l_run) * unps;
  const float z_tot = wave_sum16x4(z_run) * unps;
  const float of = exp2i(24 - ps);           // acc_o * 2^24 / 2^ps
  if (lg == 0) {
    sh_ml[wave][n][0] = m_run;
    sh_ml[wave][n][1] = l_tot;
  }
#pragma unroll
  for (int cb = 0; cb < 8; cb++)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float a = acc_o[cb][i];
      sh_o(wave, n, 16 * cb + 4 * lg + i) = (m_run == -INFINITY) ? 0.0f : a * of + z_tot;
    }
  __syncthreads();

  const int ncol = NS * G;
  const bool single = (a.n_slots == 1);
  // per column: the workgroup max M, the weight 2^(m_w - M) of each wave's
  // partial, the sum and the destination row -- the output row
  // (batch, query head) = grp * NS * G + col when this is the stream's only
  // partial, else the partial row of this chunk (-1: no head in the column)
  __shared__ float sh_cw[16][4];
  __shared__ float sh_cd[16][2];
  __shared__ int sh_row[16];
  __shared__ int sh_orow[16];
  if (threadIdx.x < ncol) {
    const int col = threadIdx.x;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; w++) M = fmaxf(M, sh_ml[w][col][0]);
    float den = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; w++) {
      const float mw = sh_ml[w][col][0];
      const float sc = (mw == -INFINITY) ? 0.0f : exp2f(mw - M);
      sh_cw[col][w] = sc;
      den += sc * sh_ml[w][col][1];
    }
    sh_cd[col][0] = M;
    sh_cd[col][1] = den;
    const int s = col / G, hh = col - s * G;
    const int bh = grp * NS + s;
    sh_row[col] = bh >= BH ? -1 : (single ? bh * G + hh : (bh * a.n_slots + chunk) * G + hh);
    sh_orow[col] = bh * G + hh;
  }
  __syncthreads();
  // four consecutive channels per thread
  for (int idx = threadIdx.x; idx < ncol * 32; idx += 256) {
    const int col = idx >> 5, c4 = (idx & 31) * 4;
    const int row = sh_row[col];
    if (row < 0) continue;
    f32x4 num = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; w++) num += sh_cw[col][w] * *(const f32x4*)&sh_o(w, col, c4);
    if (single) {
      *(f32x4*)(a.out + (int64_t)row * 128 + c4) = num / sh_cd[col][1];
    } else {
      if (a.fused) {
        // device-scope stores: they pass the XCD's own L2, so the workgroup
        // that combines (on any XCD) reads them without a cache write-back
        if (c4 == 0) {
          st_dev(a.part_ml + 2 * (int64_t)row, sh_cd[col][0]);
          st_dev(a.part_ml + 2 * (int64_t)row + 1, sh_cd[col][1]);
        }
#pragma unroll
        for (int k = 0; k < 4; k++) st_dev(a.part_o + (int64_t)row * 128 + c4 + k, num[k]);
      } else {
        if (c4 == 0) { a.part_ml[2 * (int64_t)row] = sh_cd[col][0]; a.part_ml[2 * (int64_t)row + 1] = sh_cd[col][1]; }
        *(f32x4*)(a.part_o + (int64_t)row * 128 + c4) = num;
      }
    }
  }
  if (a.fused) {
    if (single) return;
    // ---- chunk combine by the workgroup that completes the stream group:
    // once this workgroup's partial stores are complete it counts itself in
    // the group's counter; the one that brings the count to n_chunks reads
    // every partial slot of the group's streams back (the chunks and any
    // residual slots), writes o = sum_k 2^(m_k - M) o_k / sum_k 2^(m_k - M) l_k
    // and resets the counter for the next call.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    __shared__ int s_last;
    if (threadIdx.x == 0)
      s_last = __hip_atomic_fetch_add(a.counters + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               (unsigned)(a.n_chunks - 1);
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const int ns = a.n_slots;
    constexpr int KR = 16;   // slots whose outputs are loaded before the weights are known
    // items: four consecutive channels of one column, two per thread
    f32x4 ov[2][KR];
    int icol[2], ic4[2], irow[2];
#pragma unroll
    for (int it = 0; it < 2; it++) {
      const int idx = threadIdx.x + 256 * it;
      icol[it] = min(idx >> 5, 15);
      ic4[it] = (idx & 31) * 4;
      irow[it] = idx < ncol * 32 ? sh_row[icol[it]] : -1;
      // partial row of slot k = irow + (k - chunk) * G
      const int64_t r0 = (int64_t)irow[it] - (int64_t)chunk * G;
#pragma unroll
      for (int k = 0; k < KR; k++) {
        ov[it][k] = (f32x4){0.f, 0.f, 0.f, 0.f};
        if (irow[it] >= 0 && k < ns) ov[it][k] = *(const f32x4*)(a.part_o + (r0 + (int64_t)k * G) * 128 + ic4[it]);
      }
    }
    // (m, l) of every (column, slot), then the weights, in the free LDS
    float* sml = (float*)&lds[0][0];                 // [16][ns][2]
    float* sden = sml + 16 * 2 * KVQ_MAX_SLOTS;      // [16]
    for (int i = threadIdx.x; i < ncol * ns; i += 256) {
      const int col = i / ns, k = i - (i / ns) * ns;
      float m = -INFINITY, l = 0.0f;
      if (sh_row[col] >= 0) {
        const int64_t r = (int64_t)sh_row[col] + (int64_t)(k - chunk) * G;
        m = a.part_ml[2 * r];
        l = a.part_ml[2 * r + 1];
      }
      sml[2 * (col * ns + k)] = m;
      sml[2 * (col * ns + k) + 1] = l;
    }
    __syncthreads();
    if (threadIdx.x < ncol) {
      const int col = threadIdx.x;
      float M = -INFINITY;
      for (int k = 0; k < ns; k++) M = fmaxf(M, sml[2 * (col * ns + k)]);
      float den = 0.0f;
      for (int k = 0; k < ns; k++) {
        const float mk = sml[2 * (col * ns + k)];
        const float w = (mk == -INFINITY) ? 0.0f : exp2f(mk - M);
        den += w * sml[2 * (col * ns + k) + 1];
        sml[2 * (col * ns + k)] = w;
      }
      sden[col] = den;
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 2; it++) {
      if (irow[it] < 0) continue;
      const int col = icol[it];
      const float* wk = sml + 2 * col * ns;
      f32x4 num = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KR; k++)
        if (k < ns) num += wk[2 * k] * ov[it][k];
      const int64_t r0 = (int64_t)irow[it] - (int64_t)chunk * G;
      for (int k = KR; k < ns; k++) num += wk[2 * k] * *(const f32x4*)(a.part_o + (r0 + (int64_t)k * G) * 128 + ic4[it]);
      *(f32x4*)(a.out + (int64_t)sh_orow[col] * 128 + ic4[it]) = num / sden[col];
    }
    if (threadIdx.x == 0) __hip_atomic_store(a.counters + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}


// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// kv streams per wave: as many query groups as fit the 16 MFMA columns,
// capped per width so the kernel keeps two waves per SIMD without spilling.
// streams per wave allowed for 4- and 2-bit codes (see KVQ_DECODE_NS3_OCC)
#ifndef KVQ_DECODE_NS_CAP_LOW
#define KVQ_DECODE_NS_CAP_LOW 2
#endif
// a plan packing several streams per wave falls back to one stream when its
// chunks would hold fewer tiles than this
#ifndef KVQ_DECODE_NS_MIN_TPC
#define KVQ_DECODE_NS_MIN_TPC 16
#endif
// measured: two mixed-key streams per wave 30% slower, three 2x slower
#ifndef KVQ_DECODE_NS_CAP_MIXED2
#define KVQ_DECODE_NS_CAP_MIXED2 1
#endif
constexpr int ns_cap(int kb, int vb) {
  if (kb == 0) return vb == 4 ? 2 : (vb == 2 ? KVQ_DECODE_NS_CAP_MIXED2 : 1);
  return (kb == 4 || kb == 2) ? KVQ_DECODE_NS_CAP_LOW : 1;
}

// Launch plan (shared by workspace sizing, validation and launch): NS streams
// per wave, n_groups = ceil(BH / NS) stream groups, and the token tiles of a
// group cut into n_chunks chunks of tpc tiles, aiming at one round of
// resident workgroups (256 CUs x waves per SIMD) with 4..64 tiles per chunk and
// at most KVQ_MAX_CHUNKS chunks.
static DecodePlan plan_for(int BH, int ns, int k_bits, int v_bits, int pdt, int n_tiles) {
  DecodePlan p;
  p.ns = ns;
  p.n_groups = (BH + ns - 1) / ns;
  const long total = (long)p.n_groups * n_tiles;
  // about one round of resident workgroups
  const long wg_target = (long)KVQ_DECODE_WG_PER_OCC * decode_occ(k_bits, v_bits, pdt, ns);
  int tpc = (int)((total + wg_target - 1) / wg_target);
  tpc = ((tpc + 3) / 4) * 4;
  if (tpc < 4) tpc = 4;
  if (tpc > 64) tpc = 64;
  const int tmin = (n_tiles + KVQ_MAX_CHUNKS - 1) / KVQ_MAX_CHUNKS;
  if (tpc < tmin) tpc = tmin;
  p.n_chunks = (n_tiles + tpc - 1) / tpc;
  p.tpc = (n_tiles + p.n_chunks - 1) / p.n_chunks;   // balanced, every chunk non-empty
  return p;
}

// As many streams per wave as the columns and ns_cap() allow -- unless that
// leaves a wave fewer than four tiles, where a single stream per wave (twice
// the tiles, the prologue and partial write amortised over more work) is
// faster.
DecodePlan decode_plan(int BH, int G, int k_bits, int v_bits, int pdt, int n_tiles) {
  const int cap = ns_cap(k_bits, v_bits);
  int ns = 16 / G;
  if (ns > KVQ_DECODE_NS_MAX) ns = KVQ_DECODE_NS_MAX;
  ns = ns > cap ? cap : (ns < 1 ? 1 : ns);
  DecodePlan p = plan_for(BH, ns, k_bits, v_bits, pdt, n_tiles);
  if (ns > 1 && p.tpc < KVQ_DECODE_NS_MIN_TPC) p = plan_for(BH, 1, k_bits, v_bits, pdt, n_tiles);
  return p;
}

// Chunk combine, a separate launch so that the partials are visible without
// device-scope fences.  One wave per output row (batch, query head):
//   o = sum_k 2^(m_k - M) o_k / sum_k 2^(m_k - M) l_k,  M = max_k m_k.
// Lane k holds the (m, l) of chunks k and k + 64; each lane owns two channels
// of o and walks the chunks with the weight broadcast from its owner lane.
__global__ __launch_bounds__(256) void decode_combine_kernel(const float* __restrict__ part_ml,
                                                             const float* __restrict__ part_o,
                                                             float* __restrict__ out, int BH, int H,
                                                             int G, int nck) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);   // bh * G + hh
  if (row >= BH * G) return;
  const int bh = row / G, hh = row - (row / G) * G;
  const int64_t r0 = (int64_t)bh * nck * G + hh;         // partial row of chunk 0
  float m0 = -INFINITY, m1 = -INFINITY, l0 = 0.0f, l1 = 0.0f;
  if (lane < nck) { m0 = part_ml[2 * (r0 + (int64_t)lane * G)]; l0 = part_ml[2 * (r0 + (int64_t)lane * G) + 1]; }
  if (lane + 64 < nck) {
    m1 = part_ml[2 * (r0 + (int64_t)(lane + 64) * G)];
    l1 = part_ml[2 * (r0 + (int64_t)(lane + 64) * G) + 1];
  }
  // the first 16 chunk outputs are loaded before the weights are known, so a
  // typical combine costs one memory round trip
  const float* po = part_o + r0 * 128 + 2 * lane;
  const int64_t step = (int64_t)G * 128;
  float2 v[16];
#pragma unroll
  for (int k = 0; k < 16; k++) v[k] = (k < nck) ? *(const float2*)(po + step * k) : make_float2(0.f, 0.f);
  float M = fmaxf(m0, m1);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  const float w0 = exp2f(m0 - M), w1 = exp2f(m1 - M);   // 0 for absent chunks
  float den = w0 * l0 + w1 * l1;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o, 64);
  float n0 = 0.0f, n1 = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; k++) {
    const float w = u2f(__builtin_amdgcn_readlane(f2u(w0), k));   // 0 beyond nck
    n0 = fmaf(w, v[k].x, n0);
    n1 = fmaf(w, v[k].y, n1);
  }
  for (int k = 16; k < nck; k++) {
    const float w = u2f(__builtin_amdgcn_readlane(f2u(k < 64 ? w0 : w1), k & 63));
    const float2 x = *(const float2*)(po + step * k);
    n0 = fmaf(w, x.x, n0);
    n1 = fmaf(w, x.y, n1);
  }
  const float inv = 1.0f / den;
  const int bo = bh / H, ho = bh - (bh / H) * H;
  *(float2*)(out + ((int64_t)bo * H * G + (int64_t)ho * G + hh) * 128 + 2 * lane) = make_float2(n0 * inv, n1 * inv);
}

static size_t ml_bytes(int BH, int n_chunks, int G) {
  return ((size_t)BH * n_chunks * G * 2 * 4 + 255) / 256 * 256;
}
// per-stream-group counters of the in-kernel combine, at the start of the
// workspace (at most one group per stream)
static size_t cnt_bytes(int BH) { return ((size_t)BH * 4 + 255) / 256 * 256; }

// partial slots: every chunk plus the most a residual segment can add
size_t decode_workspace_needed(int BH, int G, const DecodePlan& p) {
  const int slots = p.n_chunks + KVQ_MAX_RES_SLOTS;
  return cnt_bytes(BH) + ml_bytes(BH, slots, G) + (size_t)BH * slots * G * 128 * 4;
}

size_t decode_workspace_bytes(int B, int H, int G, int max_tiles) {
  // upper bound over every n_tokens <= max_tokens and every packing: a chunk
  // holds at least 4 tiles and there are at most KVQ_MAX_CHUNKS of them
  const int BH = B * H;
  int nc = (max_tiles + 3) / 4;
  if (nc > KVQ_MAX_CHUNKS) nc = KVQ_MAX_CHUNKS;
  DecodePlan p;
  p.n_chunks = nc;
  return decode_workspace_needed(BH, G, p);
}

bool decode_supported(int k_bits, int v_bits, int pdt) {
  (void)pdt;
  if (k_bits == 0) return v_bits == 1 || v_bits == 2 || v_bits == 4;
  return k_bits == v_bits && (k_bits == 1 || k_bits == 2 || k_bits == 4 || k_bits == 8 || k_bits == 16);
}

template <int KB, int VB, int PDT>
static hipError_t launch_ns(const DecodeArgs& a0, hipStream_t st) {
  constexpr int CAP = ns_cap(KB, VB);
  DecodeArgs a = a0;
  const DecodePlan p = decode_plan(a.g.B * a.g.H, a.G, KB, VB, PDT, a.g.n_tiles);
  a.n_groups = p.n_groups;
  a.n_chunks = p.n_chunks;
  a.tpc = p.tpc;
  a.n_slots = p.n_chunks + a.n_slots;   // residual slots on entry
  a.fused = a.n_slots > 1 && p.n_chunks >= KVQ_DECODE_FUSED_MIN_CHUNKS;
  // residual workgroups ride along only when a second kernel combines
  if (a.fused && a.n_res) return hipErrorInvalidValue;
  const int res_rows = a.n_res ? (a.n_res * a.g.B * a.g.H + a.n_chunks - 1) / a.n_chunks : 0;
  const dim3 grid(a.n_chunks, a.n_groups + res_rows), block(256);
  if (p.ns == 1) {
    hipLaunchKernelGGL((decode_kernel<KB, VB, PDT, 1>), grid, block, 0, st, a);
  } else if (p.ns == 2) {
    if constexpr (CAP >= 2) hipLaunchKernelGGL((decode_kernel<KB, VB, PDT, 2>), grid, block, 0, st, a);
  } else if (p.ns == 3) {
    if constexpr (CAP >= 3) hipLaunchKernelGGL((decode_kernel<KB, VB, PDT, 3>), grid, block, 0, st, a);
  } else {
    if constexpr (CAP >= 4) hipLaunchKernelGGL((decode_kernel<KB, VB, PDT, 4>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

template <int PDT>
static hipError_t launch_decode_pdt(const DecodeArgs& a, hipStream_t st) {
  const int kb = a.g.k_bits, vb = a.g.v_bits;
#define KVQ_DEC(KBV, VBV) \
  if (kb == KBV && vb == VBV) return launch_ns<KBV, VBV, PDT>(a, st);
  KVQ_DEC(16, 16) KVQ_DEC(8, 8) KVQ_DEC(4, 4) KVQ_DEC(2, 2) KVQ_DEC(1, 1)
  KVQ_DEC(0, 1) KVQ_DEC(0, 2) KVQ_DEC(0, 4)
#undef KVQ_DEC
  return hipErrorInvalidValue;
}

namespace {
hipError_t launch_residual(const ResArgs& res, int res_dtype, dim3 grid, const void* q, int H, int G,
                           float sl2, float* part_ml, float* part_o, int n_slots, int slot0,
                           float* direct, hipStream_t st) {
  if (res_dtype == KVQ_F32)
    hipLaunchKernelGGL(decode_residual_kernel<KVQ_F32>, grid, dim3(256), 0, st, res, (const uint16_t*)q,
                       H, G, sl2, part_ml, part_o, n_slots, slot0, direct);
  else if (res_dtype == KVQ_F16)
    hipLaunchKernelGGL(decode_residual_kernel<KVQ_F16>, grid, dim3(256), 0, st, res, (const uint16_t*)q,
                       H, G, sl2, part_ml, part_o, n_slots, slot0, direct);
  else
    hipLaunchKernelGGL(decode_residual_kernel<KVQ_BF16>, grid, dim3(256), 0, st, res, (const uint16_t*)q,
                       H, G, sl2, part_ml, part_o, n_slots, slot0, direct);
  return hipGetLastError();
}
}  // namespace

// Packed cache (when it holds tokens) and residual segment (res.R > 0), then
// the chunk combine when a stream has more than one partial slot.  All on the
// caller's stream.  With the separate combine kernel the residual blocks are
// extra workgroups of the decode launch: the dispatcher starts them as decode
// workgroups retire, so they fill the decode kernel's tail instead of taking
// a launch of their own.
hipError_t launch_decode(const Geo& g, const void* q, int G, float scale, float* out, void* ws,
                         const ResArgs& res, int res_dtype, hipStream_t st) {
  const int BH = g.B * g.H;
  const float sl2 = scale * 1.4426950408889634f;
  const bool has_packed = g.n_tiles > 0;
  const int n_res = (res.R + KVQ_RES_CHUNK - 1) / KVQ_RES_CHUNK;
  DecodePlan p;
  p.n_chunks = 0;
  if (has_packed) p = decode_plan(BH, G, g.k_bits, g.v_bits, g.pdt, g.n_tiles);
  const int n_slots = p.n_chunks + n_res;
  unsigned* counters = (unsigned*)ws;
  float* part_ml = (float*)((uint8_t*)ws + cnt_bytes(BH));
  float* part_o = (float*)((uint8_t*)part_ml + ml_bytes(BH, n_slots, G));
  hipError_t e = hipSuccess;
  // with a second combine kernel the residual blocks ride along as extra
  // workgroups of the decode launch; otherwise (in-kernel combine, or no
  // packed tokens) they run first as their own kernel
  const bool res_inline = has_packed && n_res > 0 && p.n_chunks < KVQ_DECODE_FUSED_MIN_CHUNKS;
  if (n_res > 0 && !res_inline) {
    e = launch_residual(res, res_dtype, dim3(n_res, BH), q, g.H, G, sl2, part_ml, part_o, n_slots,
                        p.n_chunks, n_slots == 1 ? out : nullptr, st);
    if (e != hipSuccess) return e;
  }
  if (has_packed) {
    DecodeArgs a;
    a.g = g;
    a.q = (const uint16_t*)q;
    a.out = out;
    a.part_ml = part_ml;
    a.part_o = part_o;
    a.G = G;
    a.sl2 = sl2;
    a.n_chunks = a.tpc = a.n_groups = 0;
    a.n_slots = n_res;
    a.counters = counters;
    a.fused = 0;   // set by the launch from the plan
    a.res = res;
    a.res_dtype = res_dtype;
    a.n_res = res_inline ? n_res : 0;
    switch (g.pdt) {
      case KVQ_F32: e = launch_decode_pdt<KVQ_F32>(a, st); break;
      case KVQ_F16: e = launch_decode_pdt<KVQ_F16>(a, st); break;
      case KVQ_BF16: e = launch_decode_pdt<KVQ_BF16>(a, st); break;
      case KVQ_E4M3: e = launch_decode_pdt<KVQ_E4M3>(a, st); break;
      default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
  }
  if (n_slots > 1 && (!has_packed || p.n_chunks < KVQ_DECODE_FUSED_MIN_CHUNKS)) {
    const int rows = BH * G;
    hipLaunchKernelGGL(decode_combine_kernel, dim3((rows + 3) / 4), dim3(256), 0, st, (const float*)part_ml,
                       (const float*)part_o, out, BH, g.H, G, n_slots);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace kvq
