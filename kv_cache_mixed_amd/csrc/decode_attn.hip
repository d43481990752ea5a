// decode_attn.hip -- decode attention over the packed cache (gfx950).
//
// ChanMix page, Overall framework / Key design 3: at decode time the packed
// cache is read, dequantized (x^ = S' * q + Z') and fed to ordinary
// (FlashAttention-style) attention.  Here the dequantization never
// materialises: the key parameters are folded into the query and the value
// parameters into the softmax weights, so the two contractions run on the raw
// integer codes with MFMA.
//
// Work decomposition.  Grid = (chunk, stream group).  A workgroup of 4 waves
// owns one chunk of 128-token tiles of NS (batch, kv head) streams and all G
// query heads of each (NS * G <= 16 columns); wave w takes tiles w, w+4, ...
// of the chunk.  Per tile a wave computes, with the heads padded to the 16
// columns of a 16x16x32 f16 MFMA:
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
// codes) are folded into the other operand.  For keys that operand (u) is
// split into f16 hi + lo parts (two MFMAs), so the products carry about 22
// significant bits; for values P is one rounded binary16 per token, and its
// rounding residual times the codes' midpoint is added back exactly through
// the zero-point sum.  The sums accumulate in binary32.
//
// Mixed-width keys (4/3/1/2-bit slots in five byte planes) and mixed-width
// values (4/3/1/2-bit slot classes in 4- and 2-bit fields, one probability
// operand and one zero-point sum per class) use the same loop with their own
// field extraction.
//
// Softmax uses a lazy running max: the reference m only moves when a logit
// exceeds it by more than TAU (log2 units), so e = 2^(logit - m) <= 2^TAU and
// the output accumulator is rescaled only when some head's reference moved.
//
// Compacted softmax (one stream per wave with G <= 8 or G <= 4 heads, 1/2 or
// 3/4 of the 16 columns without a head): the CMP lane parts of an MFMA row
// share each head's work.  DPP row shifts spread the column's logits over the
// parts (each takes the tokens of its share of the probability registers),
// every part runs the softmax, the value-parameter loads and the zero-point
// sums on its tokens and folds its share of the query slots, and DPP row
// shifts bring the probability and folded-query registers back to the lanes
// of the head columns for the two products.
#include "kvq_device.h"

#include <mutex>
// waves of the decode kernel resident per SIMD (register budget 512 / n)
// A nonzero KVQ_DECODE_WAVES_PER_SIMD forces every decode instance to that
// occupancy (tuning builds); 0 uses the per-instance table decode_occ().
#ifndef KVQ_DECODE_WAVES_PER_SIMD
#define KVQ_DECODE_WAVES_PER_SIMD 0
#endif
// Operand prefetch: some instances load the next sub-tile's operands into a
// single buffer (one sub-tile ahead), the others into two (two ahead); see
// pf1_instance().  1: that choice; 0: two buffers everywhere.
#ifndef KVQ_DECODE_PF1
#define KVQ_DECODE_PF1 1
#endif
// uniform 2-bit codes: most streams per wave, and waves per SIMD of
// three-stream instances (three streams spill even with one buffer)
#ifndef KVQ_DECODE_NS_CAP_2BIT
#define KVQ_DECODE_NS_CAP_2BIT 2
#endif
#ifndef KVQ_DECODE_NS3_OCC_2BIT
#define KVQ_DECODE_NS3_OCC_2BIT 1
#endif
// folded query operand kept in registers across a tile's sub-tiles (1) or
// staged in the wave's LDS region (0)
#ifndef KVQ_DECODE_QREG
#define KVQ_DECODE_QREG 1
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
// cache-policy bits of the code loads (sc0 = 1, nt = 2, sc1 = 16) and of the
// parameter loads.  Codes are read once: non-temporal loads measured 6-11%
// faster at every width but 16-bit, where they are 15% slower.
#ifndef KVQ_DECODE_CPOL_CODES
#define KVQ_DECODE_CPOL_CODES 2
#endif
#ifndef KVQ_DECODE_CPOL_PARAMS
#define KVQ_DECODE_CPOL_PARAMS 0
#endif
// value words of the compacted one-stream instances loaded one sub-tile ahead
// in two alternating buffers (1) or at the start of their own sub-tile (0)
#ifndef KVQ_DECODE_VPF
#define KVQ_DECODE_VPF 1
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
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

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

// Mixed key tile, lane group g (every group has the same class mix): the
// lane's words are D0 = plane g bytes 0..3 (a 4-bit pair, a (3,1,3,1) group,
// two 2-bit quads), D1 = plane g bytes 4..7 (four 2-bit quads) and N = the
// group's nibble of plane 4 (two 2-bit slots) at bits 0..3.  Operand register
// f (two fields, one per 16-bit half) and its halves' bit positions:
//   f0  D0 & (0xF,  0x3 <<16)  lo 4-bit @0  hi 2-bit @0
//   f1  D0 & (0xF0, 0xC <<16)  lo 4-bit @4  hi 2-bit @2
//   f2..f5  (D0 >> 8): lo 3/1/3/1-bit @0/3/4/7, hi 2-bit @0/2/4/6
//   f6  D0 & (0x3 << 20) | N & 0x3   lo 2-bit @0  hi 2-bit @4
//   f7  D0 & (0xC << 20) | N & 0xC   lo 2-bit @2  hi 2-bit @6
//   f8..f15  D1 as a uniform 2-bit word (ufield<2>)
// Lane-local index li = 2f + half; mixed_lane_slot gives its slot.
__host__ __device__ constexpr int mixed_pos(int f, int half) {
  constexpr int lo[8] = {0, 4, 0, 3, 4, 7, 0, 2};
  constexpr int hi[8] = {0, 2, 0, 2, 4, 6, 4, 6};
  if (f >= 8) return 2 * ((f - 8) < 5 ? (f - 8) : (f - 8) - 5);
  return half ? hi[f] : lo[f];
}
__host__ __device__ constexpr int mixed_lane_slot(int g, int li) {
  const int f = li >> 1, h = li & 1;
  if (f >= 8) return 32 + 24 * g + (f - 8) + 8 * h;
  // high halves of f0..f7 hold 2-bit slots 24 + 24g + {0, 1, 4, 5, 6, 7, 2, 3}
  if (h) return 24 + 24 * g + (f < 2 ? f : (f < 6 ? f + 2 : f - 4));
  if (f < 2) return 2 * g + f;
  if (f < 6) return 8 + 4 * g + (f - 2);
  return 120 + 2 * g + (f - 6);
}
// inverse: the lane-order position 32 g + li of slot j
__host__ __device__ constexpr int mixed_slot_lpos(int j) {
  if (j < 8) return 32 * (j >> 1) + 2 * (j & 1);
  if (j < 24) return 32 * ((j - 8) >> 2) + 2 * (2 + ((j - 8) & 3));
  if (j >= 120) return 32 * ((j - 120) >> 1) + 2 * (6 + ((j - 120) & 1));
  const int m = j - 24, g = m / 24, i = m % 24;
  if (i < 8) return 32 * g + 2 * (i < 2 ? i : (i < 4 ? i + 4 : i - 2)) + 1;
  return 32 * g + 2 * (8 + ((i - 8) & 7)) + ((i - 8) >> 3);
}
__device__ __forceinline__ uint32_t mixed_field(const uint32_t* kw, int f) {
  const uint32_t d0 = kw[0], d1 = kw[1], nn = kw[2];
  switch (f) {
    case 0: return d0 & 0x0003000Fu;
    case 1: return d0 & 0x000C00F0u;
    case 2: return (d0 >> 8) & 0x00030007u;
    case 3: return (d0 >> 8) & 0x000C0008u;
    case 4: return (d0 >> 8) & 0x00300070u;
    case 5: return (d0 >> 8) & 0x00C00080u;
    case 6: return (d0 & 0x00300000u) | (nn & 0x3u);
    case 7: return (d0 & 0x00C00000u) | (nn & 0xCu);
    default: {
      const Fld F = ufield<2>(f - 8);
      const uint32_t m = ((1u << F.wid) - 1u) << F.pos;
      return (F.sh ? (d1 >> F.sh) : d1) & (m | (m << 16));
    }
  }
}
// the compacted softmax's token runs and field weights (2-bit value words):
// register k pairs tokens k and 8 + k at bit position 2k (k < 5) or 2(k - 5)
namespace cmp_check {
constexpr bool ok() {
  for (int k = 0; k < 8; k++) {
    const Fld F = ufield<2>(k);
    if (F.w != 0 || F.lo != k || F.hi != 8 + k || F.wexp != 0 || F.pos != (k < 5 ? 2 * k : 2 * (k - 5))) return false;
  }
  return true;
}
static_assert(ok(), "2-bit value field map");
}  // namespace cmp_check

// Compacted-softmax geometry.  Value side: part pa of a row owns probability
// registers pa * RPL .. pa * RPL + RPL - 1 of a sub-tile; slot sl < RPL of
// the part is the low-half token of register pa * RPL + sl, slot RPL + r the
// high-half token of register pa * RPL + r.
template <int VB, int RPL>
__host__ __device__ constexpr int cmp_tok(int pa, int sl) {
  return sl < RPL ? ufield<VB>(pa * RPL + sl).lo : ufield<VB>(pa * RPL + sl - RPL).hi;
}
// Key side (the fold): part pa computes folded-query registers pa * NFP ..;
// register f's halves hold the lane-order slots kslot_lo(f), kslot_hi(f)
// (mixed keys: 2f and 2f + 1).
template <int KB>
__host__ __device__ constexpr int kslot_lo(int f) { return KB == 0 ? 2 * f : ufield<KB == 0 ? 2 : KB>(f).lo; }
template <int KB>
__host__ __device__ constexpr int kslot_hi(int f) { return KB == 0 ? 2 * f + 1 : ufield<KB == 0 ? 2 : KB>(f).hi; }
namespace cmp_check {
// every part's low and high tokens are two runs of RPL consecutive tokens
template <int VB, int CMP, int FVS>
constexpr bool vruns() {
  constexpr int RPL = FVS / CMP;
  for (int pa = 0; pa < CMP; pa++)
    for (int r = 0; r < RPL; r++)
      if (cmp_tok<VB, RPL>(pa, r) != cmp_tok<VB, RPL>(pa, 0) + r ||
          cmp_tok<VB, RPL>(pa, RPL + r) != cmp_tok<VB, RPL>(pa, RPL) + r)
        return false;
  return true;
}
static_assert(vruns<2, 2, 8>() && vruns<2, 4, 8>() && vruns<4, 2, 4>() && vruns<4, 4, 4>() && vruns<8, 2, 4>() &&
              vruns<8, 4, 4>(), "value token runs");
// a part's slot offsets from its first slot do not depend on the part
template <int KB, int CMP>
constexpr bool kshift() {
  constexpr int NFP = 16 / CMP;
  for (int pa = 0; pa < CMP; pa++)
    for (int j = 0; j < NFP; j++)
      if (kslot_lo<KB>(pa * NFP + j) - kslot_lo<KB>(pa * NFP) != kslot_lo<KB>(j) - kslot_lo<KB>(0) ||
          kslot_hi<KB>(pa * NFP + j) - kslot_lo<KB>(pa * NFP) != kslot_hi<KB>(j) - kslot_lo<KB>(0))
        return false;
  return true;
}
static_assert(kshift<0, 2>() && kshift<0, 4>() && kshift<2, 2>() && kshift<2, 4>() && kshift<4, 2>() &&
              kshift<4, 4>() && kshift<8, 2>() && kshift<8, 4>(), "key slot offsets");
}  // namespace cmp_check
// whether a part's 2 NFP key slots form one run (else: low halves j, then
// high halves at kslot_hi(0) - kslot_lo(0) + j)
template <int KB, int CMP>
__host__ __device__ constexpr bool kslot_run1() {
  constexpr int NFP = 16 / CMP;
  for (int t = 0; t < 2 * NFP; t++) {
    bool found = false;
    for (int j = 0; j < NFP; j++)
      if (kslot_lo<KB>(j) - kslot_lo<KB>(0) == t || kslot_hi<KB>(j) - kslot_lo<KB>(0) == t) found = true;
    if (!found) return false;
  }
  return true;
}
namespace cmp_check {
template <int KB, int CMP>
constexpr bool krun2() {   // two runs: lows are j, highs HIOFF + j
  constexpr int NFP = 16 / CMP;
  for (int j = 0; j < NFP; j++)
    if (kslot_lo<KB>(j) - kslot_lo<KB>(0) != j || kslot_hi<KB>(j) - kslot_hi<KB>(0) != j) return false;
  return true;
}
static_assert((kslot_run1<0, 2>() || krun2<0, 2>()) && (kslot_run1<0, 4>() || krun2<0, 4>()) &&
              (kslot_run1<2, 2>() || krun2<2, 2>()) && (kslot_run1<2, 4>() || krun2<2, 4>()) &&
              (kslot_run1<4, 2>() || krun2<4, 2>()) && (kslot_run1<4, 4>() || krun2<4, 4>()) &&
              (kslot_run1<8, 2>() || krun2<8, 2>()) && (kslot_run1<8, 4>() || krun2<8, 4>()), "key slot runs");
}  // namespace cmp_check
namespace mixed_check {
// the lane map is a bijection of the 128 slots and its inverse is exact
constexpr bool ok() {
  for (int g = 0; g < 4; g++)
    for (int li = 0; li < 32; li++) {
      const int j = mixed_lane_slot(g, li);
      if (j < 0 || j > 127 || mixed_slot_lpos(j) != 32 * g + li) return false;
    }
  return true;
}
static_assert(ok(), "mixed lane map");
}  // namespace mixed_check





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
  int n_slots;        // partial slots per stream: n_chunks + residual slots (+ another cache's)
  int slot0;          // slot of this launch's chunk 0 (0, or after another cache's chunks)
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

// Row-local DPP moves (rows are 16 lanes, banks 4 lanes of a row).  The lanes
// of the banks in BANKS take src from the lane SH below (shr) or above (shl)
// in their row; every other lane keeps old.  ror rotates the whole row.
template <int SH, int BANKS>
__device__ __forceinline__ uint32_t dpp_shr(uint32_t old, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, 0x110 + SH, 0xF, BANKS, false);
}
template <int SH, int BANKS>
__device__ __forceinline__ uint32_t dpp_shl(uint32_t old, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, 0x100 + SH, 0xF, BANKS, false);
}
template <int SH>
__device__ __forceinline__ uint32_t dpp_ror(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x120 + SH, 0xF, 0xF, false);
}
// Reductions over the CMP parts of a row (lanes n, n + 16/CMP, ... of one
// column, see the compacted softmax of decode_kernel); every lane gets the result.
template <int CMP>
__device__ __forceinline__ float part_max(float v) {
  if constexpr (CMP >= 2) { const float o = u2f(dpp_ror<8>(f2u(v))); v = o > v ? o : v; }
  if constexpr (CMP >= 4) { const float o = u2f(dpp_ror<4>(f2u(v))); v = o > v ? o : v; }
  return v;
}
template <int CMP>
__device__ __forceinline__ uint32_t part_maxu(uint32_t v) {
  if constexpr (CMP >= 2) v = max(v, dpp_ror<8>(v));
  if constexpr (CMP >= 4) v = max(v, dpp_ror<4>(v));
  return v;
}
template <int CMP>
__device__ __forceinline__ float part_sum(float v) {
  if constexpr (CMP >= 2) v += u2f(dpp_ror<8>(f2u(v)));
  if constexpr (CMP >= 4) v += u2f(dpp_ror<4>(f2u(v)));
  return v;
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
// two runs of N consecutive parameters (at voff_lo and voff_hi) as one array
// of 2N: the token slots of a compacted softmax lane
template <int PDT, int N>
__device__ __forceinline__ void pload_runs(__amdgpu_buffer_rsrc_t r, uint32_t voff_lo, uint32_t voff_hi,
                                           uint32_t soff, uint32_t* w) {
  constexpr int RB = N * (PDT == KVQ_F32 ? 4 : (PDT == KVQ_E4M3 ? 1 : 2));
  if constexpr (RB >= 4) {
    pload<PDT, N>(r, voff_lo, soff, w);
    pload<PDT, N>(r, voff_hi, soff, w + RB / 4);
  } else if constexpr (RB == 2) {
    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(r, voff_lo, soff, KVQ_DECODE_CPOL_PARAMS);
    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(r, voff_hi, soff, KVQ_DECODE_CPOL_PARAMS);
    w[0] = lo | (hi << 16);
  } else {
    static_assert(RB == 1, "parameter run");
    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b8(r, voff_lo, soff, KVQ_DECODE_CPOL_PARAMS);
    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b8(r, voff_hi, soff, KVQ_DECODE_CPOL_PARAMS);
    w[0] = lo | (hi << 8);
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
// waves per SIMD of the 16-bit instances and of mixed values.  At two, the
// 16-bit instances fit 256 registers without spills but measured no faster
// (32K and 8K layers), and mixed values spill 32 registers and run 7-140%
// slower.
#ifndef KVQ_DECODE_OCC16
#define KVQ_DECODE_OCC16 1
#endif
#ifndef KVQ_DECODE_OCC_VMIX
#define KVQ_DECODE_OCC_VMIX 1
#endif
// waves per SIMD of mixed keys with 1-bit values: two, with one prefetch
// buffer, fit 256 registers without spills (binary32 parameters aside, which
// stay at one) and run 29-35% faster than one (128K sequence, batched 32K)
#ifndef KVQ_DECODE_OCC_MIXED1
#define KVQ_DECODE_OCC_MIXED1 2
#endif
// Instances that prefetch through a single buffer, one sub-tile ahead
// (settled A/B against two buffers): two-stream 2-bit codes 18-20% faster
// (with two buffers they spill), mixed values 21%, mixed keys 2-8% with 1-,
// 2- and 4-bit values (and two streams with 2-bit values fit only so), 2-bit
// with one stream 2%, 8-bit 1-2%, 1-bit 1.5%.  4-bit codes measured mixed
// (+2.7% on the 7B-shaped layer, -1.7% on the 32B-shaped one, -3% on a 128K
// sequence; at three waves per SIMD 6% slower) and 16-bit neutral: they
// keep two buffers.
constexpr bool pf1_instance(int kb, int vb, int ns) {
  (void)vb;
  (void)ns;
  if (KVQ_DECODE_PF1 == 0) return false;
  return kb != 4 && kb != 16;
}

// Instances with a compacted-softmax variant (one stream per wave, 2-bit
// values): with G <= 4 heads (8), each column's logits are spread over four
// (two) lanes of its row instead of leaving 12 (8) of a row's 16 softmax lanes
// on columns without a head.  0 switches the variants off (tuning builds).
#ifndef KVQ_DECODE_CMP
#define KVQ_DECODE_CMP 1
#endif
constexpr bool cmp_instance(int kb, int vb) {
  return (vb == 2 && (kb == 0 || kb == 2)) || (kb == 0 && vb == 0) || (kb == vb && (vb == 4 || vb == 8));
}
// the compaction a launch of ns streams per wave with G heads per stream uses
constexpr int cmp_for(int kb, int vb, int ns, int G) {
  if (!KVQ_DECODE_CMP || ns != 1 || !cmp_instance(kb, vb)) return 1;
  return G <= 4 ? 4 : (G <= 8 ? 2 : 1);
}
// waves per SIMD of mixed values with the four-part compacted softmax: its
// registers fit 256 per lane, and two waves per SIMD ran 17% faster than
// one (128K sequence, G = 4: 42.9 -> 35.6 us per call)
#ifndef KVQ_DECODE_OCC_VMIX_CMP4
#define KVQ_DECODE_OCC_VMIX_CMP4 2
#endif

constexpr int decode_occ(int kb, int vb, int pdt, int ns, int cmp = 1) {
  if (KVQ_DECODE_WAVES_PER_SIMD) return KVQ_DECODE_WAVES_PER_SIMD;
  if (kb == 16) return KVQ_DECODE_OCC16;
  if (kb == 0 && vb == 0) return cmp == 4 ? KVQ_DECODE_OCC_VMIX_CMP4 : KVQ_DECODE_OCC_VMIX;
  if (kb == 0 && vb == 1) return pdt == KVQ_F32 ? 1 : KVQ_DECODE_OCC_MIXED1;
  if (ns >= 4) return 1;
  if (ns == 3) return kb == 4 ? KVQ_DECODE_NS3_OCC : (kb == 2 ? KVQ_DECODE_NS3_OCC_2BIT : 1);
  return 2;
}

// KB: 16/8/4/2/1 or 0 (mixed keys).  VB: 16/8/4/2/1.  NS: kv streams packed
// into the 16 MFMA columns (column n serves stream n / G, head n % G).
//
// Main loop: the wave walks its tiles in sub-tiles of TPS tokens per lane
// group.  Sub-tile operands (key blocks, key and value parameters) are
// double buffered in registers and loaded two sub-tiles ahead, or single
// buffered and loaded one sub-tile ahead where that measured faster
// (pf1_instance: it mostly keeps instances out of spills); value words arrive
// at the start of their own sub-tile.  All
// loads are raw buffer loads with an
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

template <int KB, int VB, int PDT, int NS, int CMP>
__global__ __launch_bounds__(256, decode_occ(KB, VB, PDT, NS, CMP)) void decode_kernel(DecodeArgs a) {
  constexpr bool MIXED = (KB == 0);
  constexpr bool VMIX = (VB == 0);                   // mixed-width values
  constexpr int NFK = MIXED ? 16 : UInfo<KB>::NF;    // key operand registers per token
  constexpr int NWK = MIXED ? 3 : UInfo<KB>::NW;     // key words per lane per token
  constexpr int NKK = NFK / 4;                       // key k-steps
  // mixed values: every slot block has 16 operand registers per tile (four
  // 4-bit-field words or two 2-bit-field words); WVS below is then unused
  constexpr int NFV = VMIX ? 16 : UInfo<VB>::NF;
  constexpr int NWV = VMIX ? 2 : UInfo<VB>::NW;
  constexpr int NSUB0 = VMIX ? 2 : ((VB == 1) ? 1 : ((VB == 2) ? 2 : 4));
  constexpr int NSUB = NSUB0 < KVQ_DECODE_NSUB_MAX ? NSUB0 : KVQ_DECODE_NSUB_MAX;  // sub-tiles per tile
  constexpr int TPS = 32 / NSUB;                     // tokens per lane per sub-tile
  constexpr int JB = 8 / NSUB;                       // key blocks per sub-tile
  constexpr int FVS = NFV / NSUB;                    // value fields per sub-tile
  constexpr int WVS = NWV / NSUB;                    // value words per sub-tile
  constexpr int KSV = FVS / 4;                       // value k-steps per sub-tile
  constexpr int PB = (PDT == KVQ_F32) ? 4 : ((PDT == KVQ_E4M3) ? 1 : 2);
  // Compacted softmax (CMP = 2 or 4, one stream of G <= 16 / CMP heads): the
  // columns that hold heads are the first CPW = 16 / CMP of each row, so the
  // logits of column c are spread over lanes c, c + CPW, ... (part a of the
  // row takes the tokens of probability registers a * RPL .. a * RPL + RPL - 1)
  // and the probability registers go back to lane c for the value product.
  static_assert(CMP == 1 || ((CMP == 2 || CMP == 4) && NS <= 2 && (VB == 2 || VB == 4 || VB == 8 || VMIX)),
                "compaction: 2-, 4-, 8-bit or mixed values");
  constexpr int CPW = 16 / CMP;                      // lanes per part
  constexpr int RPL = FVS / CMP;                     // probability registers per lane (compacted)
  constexpr int NL = CMP > 1 ? 2 * RPL : TPS;        // tokens per lane in the softmax
  constexpr int PWV = CMP > 1 ? (NL * PB + 3) / 4 : PW<PDT, TPS>::W;   // value-parameter words per sub-tile (and class)
  constexpr int NCV = VMIX ? 4 : 1;                  // value parameter classes
  constexpr int NVW = VMIX ? 10 : 8 * WVS;           // value words per stream per sub-tile
  // mixed values: the sub-tile's value parameters (4 classes, 32 registers
  // per buffer with e4m3) are loaded with its value words instead of two
  // sub-tiles ahead (measured 7% faster with binary16 parameters, equal with
  // e4m3, at one wave per SIMD; two waves per SIMD spill even so)
  constexpr bool PJIT = VMIX;
  // one prefetch buffer (operands one sub-tile ahead instead of two)
  constexpr bool PF1 = pf1_instance(KB, VB, NS);
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
  static_assert(!VMIX || (NS == 1 && TPS == 16), "mixed values: one stream, 16 tokens per sub-tile");
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
  // (compacted softmax: lanes of every part work for column n % CPW)
  const int own = (CMP > 1 ? n % CPW : n) / G;
  const int bh_own = grp * NS + own;
  const bool real = (own < NS) && (bh_own < BH);
  // the chunk's tiles, numbered k = 0 .. t_count-1: tile = t_base + k
  const int t_count = min(a.tpc, g.n_tiles - chunk * a.tpc);
  const int t_base = chunk * a.tpc;

  auto kslot = [&](int li) -> int {
    return 32 * lg + li;   // query and key parameters are staged in lane order
  };

  // ---- lane offsets, fixed for the whole kernel
  // key block j row r = 32*(n/4) + 4j + n%4; the lane reads its lane group's
  // 4*KB bytes of the row (mixed: its plane's 8 bytes, lane group 0 also the
  // 2 plane-4 bytes)
  const uint32_t row0 = 32 * (n >> 2) + (n & 3);
  const uint32_t koff = MIXED ? (uint32_t)(1024 * lg + 8 * row0)
                              : (uint32_t)(row0 * ROW_K + 4 * KB * lg);
  const uint32_t koff4 = 4096 + 2 * row0;                       // mixed plane 4
  const uint32_t voff4 = (uint32_t)(4 * n + lg) * 16;           // value words (w, h, n, lg, 0..3)
  const uint32_t voffm = (uint32_t)(16 * n + 4 * lg);            // mixed value words (w, n, lg)
  // parameter arrays from the group's first stream on (offsets stay below 2^32:
  // the host bounds max_tokens)
  const int64_t s0 = (int64_t)grp * NS;
  const int own_c = real ? own : 0;
  const uint32_t vpoff = (uint32_t)(((int64_t)own_c * NCV * g.max_tokens + 32 * lg) * PB);
  // compacted softmax: the lane's part and the column it serves; its tokens
  // are the two runs (low and high halves of its probability registers) of
  // RPL tokens at ufield offsets cpart * RPL and ufield<VB>(0).hi + cpart * RPL
  const int cpart = n / CPW, ccol = n % CPW;
  constexpr int VBF = VB == 0 ? 2 : VB;   // mixed values: the 2-bit container's token order
  int ctl = 0, cth = 0;   // first low / high token of the lane's part
  // field weights of the lane's probability registers: W = wexp - pos
  float cw[CMP > 1 ? RPL : 1], ciw[CMP > 1 ? RPL : 1], cew[CMP > 1 ? RPL : 1];
  if constexpr (CMP > 1) {
#pragma unroll
    for (int pa = 0; pa < CMP; pa++)
      if (cpart == pa) { ctl = cmp_tok<VBF, RPL>(pa, 0); cth = cmp_tok<VBF, RPL>(pa, RPL); }
#pragma unroll
    for (int r = 0; r < RPL; r++) {
      int w = 0;
#pragma unroll
      for (int pa = 0; pa < CMP; pa++)
        if (cpart == pa) w = ufield<VBF>(pa * RPL + r).wexp - ufield<VBF>(pa * RPL + r).pos;
      cw[r] = (float)w;
      ciw[r] = exp2i(-w);
      cew[r] = exp2i(w);
    }
  }
  const uint32_t vpoff_lo = vpoff + (uint32_t)(ctl * PB);
  const uint32_t vpoff_hi = vpoff + (uint32_t)(cth * PB);
  const __amdgpu_buffer_rsrc_t r_vs = rsrc((const uint8_t*)g.v_scale + s0 * NCV * g.max_tokens * PB, 0xffffffffu);
  const __amdgpu_buffer_rsrc_t r_vz = rsrc((const uint8_t*)g.v_zero + s0 * NCV * g.max_tokens * PB, 0xffffffffu);
  const __amdgpu_buffer_rsrc_t r_ks = rsrc((const uint8_t*)g.k_scale + s0 * g.max_tokens * PB, 0xffffffffu);
  const __amdgpu_buffer_rsrc_t r_kz = rsrc((const uint8_t*)g.k_zero + s0 * g.max_tokens * PB, 0xffffffffu);
  // key parameters: lane l loads word l (and l + 64) of the tile's 128 (e4m3:
  // lanes 32.. repeat words 0..31)
  const uint32_t kloff = (uint32_t)((PB == 1) ? (lane & 31) : lane) * 4;
  // mixed keys: lane-order positions of the parameters this lane stages
  // (its word j holds slots (kloff / PB) + 256 j / PB + e)
  int mlpos[4 / PB * KPL > 0 ? 4 / PB * KPL : 1];
  if constexpr (MIXED) {
#pragma unroll
    for (int j = 0; j < KPL; j++)
#pragma unroll
      for (int e = 0; e < 4 / PB; e++) mlpos[j * (4 / PB) + e] = mixed_slot_lpos((int)(kloff / PB) + 256 * j / PB + e);
  }

  float m_run = -INFINITY, l_run = 0.0f, z_run = 0.0f;
  float zm_run[NCV];   // mixed values: zero-point sums per class
#pragma unroll
  for (int k = 0; k < NCV; k++) zm_run[k] = 0.0f;
  int e_run = -1000;
  const float m1 = opaque_m1();
  float ak = 0.0f, bk0 = 0.0f;
  // output accumulators, shared by the packed streams (the probabilities are
  // masked per stream)
  f32x4 acc_o[8];
#pragma unroll
  for (int cb = 0; cb < 8; cb++) acc_o[cb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  uint32_t* my_lds = lds[wave];
  // the folded query operand of the current tile, [k-step][hi/lo][4]: in
  // registers (QREG), or in the wave's LDS region where its 32 registers
  // would spill: 16-bit keys (64 registers), 1-bit codes, two streams of
  // 2-bit codes (measured 9% slower there, 3-5% faster at 4 bits) or of mixed
  // keys with 2-bit values (5% slower there), and binary32 parameters (twice
  // the parameter registers)
  constexpr bool QREG = KVQ_DECODE_QREG && KB != 16 && KB != 1 && !(KB == 2 && NS >= 2) &&
                        !(MIXED && VB == 2 && NS >= 2) && PDT != KVQ_F32 && !VMIX;
  uint32_t qop[QREG ? NKK : 1][2][4];

  // one sub-tile of raw operands; value words travel outside the prefetch
  // buffers: they are loaded at the start of their own sub-tile (in flight
  // during its key product and softmax)
  struct Buf {
    uint32_t kw[NS][JB][NWK];
    uint32_t vs[PJIT ? 1 : NCV * PWV], vz[PJIT ? 1 : NCV * PWV];
    uint32_t kp[NS][2][KPL];   // next tile's key scales / zeros (sub-tile 0 only)
  };

  // value word planes: word (w, c = 64h + 16q + n, a) at word index
  // w*512 + ((h*16 + n)*4 + a)*4 + q, so lane (n, lg) finds the words of its
  // channels n, 16+n, 32+n, 48+n (h = 0) and 64+n, ... (h = 1) as 16
  // contiguous bytes: two 16-byte loads per plane, 1 KB per wave each
  auto load_vw = [&](uint32_t* vw, __amdgpu_buffer_rsrc_t rv, int sub) {
    if constexpr (VMIX) {
      // mixed values: block m's word (w, n, lg) at 4 * (block word + 64 w) +
      // voffm; the sub-tile's 16 tokens are planes 2 sub, 2 sub + 1 of the
      // 4-bit-field blocks 0, 1 (vw[2m + 0..1]) and plane sub of the
      // 2-bit-field blocks 2..7 (vw[2 + m])
#pragma unroll
      for (int m = 0; m < 2; m++)
#pragma unroll
        for (int w = 0; w < 2; w++)
          vw[2 * m + w] = __builtin_amdgcn_raw_buffer_load_b32(
              rv, voffm, (uint32_t)(vmixed_block_word(m) + 64 * (2 * sub + w)) * 4, CPOL);
#pragma unroll
      for (int m = 2; m < 8; m++)
        vw[2 + m] = __builtin_amdgcn_raw_buffer_load_b32(rv, voffm, (uint32_t)(vmixed_block_word(m) + 64 * sub) * 4,
                                                         CPOL);
      return;
    }
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
    return rsrc(g.v_codes + v_tile_offset(g, bh / g.H, bh % g.H, tile), VMIX ? KVQ_VMIXED_TILE_BYTES : 2048 * VB);
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
          bf.kw[s][jj][2] = (uint32_t)w2 >> (4 * lg);   // the lane group's nibble at bits 0..3
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
  auto load_p_to = [&](uint32_t* ps, uint32_t* pz, int k, int sub) {
    const int tile = t_base + k;
    const uint32_t psoff = (uint32_t)(tile * 128 + sub * TPS) * PB;
    if constexpr (CMP > 1) {
#pragma unroll
      for (int c = 0; c < NCV; c++) {   // mixed values: class c's parameters c * max_tokens further
        const uint32_t co = psoff + (uint32_t)(c * g.max_tokens * PB);
        pload_runs<PDT, RPL>(r_vs, vpoff_lo, vpoff_hi, co, ps + c * PWV);
        pload_runs<PDT, RPL>(r_vz, vpoff_lo, vpoff_hi, co, pz + c * PWV);
      }
      return;
    }
#pragma unroll
    for (int c = 0; c < NCV; c++) {   // mixed values: class c's parameters c * max_tokens further
      pload<PDT, TPS>(r_vs, vpoff, psoff + (uint32_t)(c * g.max_tokens * PB), ps + c * PWV);
      pload<PDT, TPS>(r_vz, vpoff, psoff + (uint32_t)(c * g.max_tokens * PB), pz + c * PWV);
    }
  };
  auto load_p = [&](Buf& bf, int k, int sub) {
    if constexpr (!PJIT) load_p_to(bf.vs, bf.vz, k, sub);
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
    // mixed widths: lane-order position p = 32 lane group + li holds slot
    // mixed_lane_slot(p / 32, p % 32), i.e. channel slot_chan[kv head][slot].
    // The raw query rows (one 16-byte load per thread) and the group's slot
    // maps go to LDS together -- one memory round trip instead of a map load
    // followed by a gather that depends on it -- and the permutation runs in
    // LDS (the raw rows sit in wave 0's folded-query region, unused until the
    // first fold, after the barrier below).
    uint16_t* qraw = (uint16_t*)&lds[0][0];     // [16][128], channel order
    int16_t* smap = (int16_t*)(qraw + 16 * 128);   // [NS][128] slot -> channel
    static_assert(sizeof(lds[0]) >= (16 * 128 + NS * 128) * 2, "raw query rows and slot maps fit");
    {
      const int cn = threadIdx.x >> 4, part = threadIdx.x & 15;
      const int64_t row = (int64_t)grp * NS * G + cn;
      u32x4 v = (u32x4){0u, 0u, 0u, 0u};
      if (cn < NS * G && row < (int64_t)BH * G) v = *(const u32x4*)(a.q + row * 128 + 8 * part);
      int16_t sm[(NS * 128 + 255) / 256];
#pragma unroll
      for (int e = 0; e < (NS * 128 + 255) / 256; e++) {
        const int idx = threadIdx.x + 256 * e, cs = idx >> 7;
        sm[e] = (idx < NS * 128 && grp * NS + cs < BH) ? g.slot_chan[((grp * NS + cs) % g.H) * 128 + (idx & 127)] : 0;
      }
      v ^= (u32x4)qflip;
      if (q0 < t_count) load(b0, q0, 0);
      *(u32x4*)&qraw[cn * 128 + 8 * part] = v;
#pragma unroll
      for (int e = 0; e < (NS * 128 + 255) / 256; e++) {
        const int idx = threadIdx.x + 256 * e;
        if (idx < NS * 128) smap[idx] = sm[e];
      }
    }
    __syncthreads();
    uint16_t qv[8];
#pragma unroll
    for (int r = 0; r < 8; r++) {
      const int i = threadIdx.x + 256 * r;
      const int cn = i >> 7, pp = i & 127;
      const int cs = cn / G;
      qv[r] = 0;
      if (cs < NS && grp * NS + cs < BH)
        qv[r] = qraw[cn * 128 + (smap[cs * 128 + mixed_lane_slot(pp >> 5, pp & 31)] & 127)];
    }
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
      const u32x4 v = *(const u32x4*)&qs[CMP > 1 ? ccol : n][kslot(8 * c)];
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
  // Compacted fold (CMP > 1): part a of the row computes registers
  // a * NFP .. a * NFP + NFP - 1 of its column's folded query, from the
  // part's 2 NFP slots (lane-order positions cpbase + offset; register j's
  // halves at offsets foff(j, 0), foff(j, 1)), whose query values stay in
  // registers; DPP row shifts gather the registers back to lane ccol.
  constexpr int NFP = NFK / CMP;
  // the part's 2 NFP slots: one run from cpbase, or (2-bit keys with four
  // parts) two runs of NFP, the low halves and the high halves HIOFF slots
  // further.  foff: register j's halves as indices into the part's parameter
  // array, fli: such an index as a slot offset from cpbase
  constexpr bool FRUN2 = !kslot_run1<KB, CMP>();
  constexpr int HIOFF = kslot_hi<KB>(0) - kslot_lo<KB>(0);
  auto foff = [](int j, int half) -> int {
    return FRUN2 ? j + half * NFP : (half ? kslot_hi<KB>(j) : kslot_lo<KB>(j)) - kslot_lo<KB>(0);
  };
  auto fli = [](int off) -> int { return FRUN2 ? (off < NFP ? off : HIOFF + off - NFP) : off; };
  int cpbase = 0;
  if constexpr (CMP > 1) {
#pragma unroll
    for (int pa = 0; pa < CMP; pa++)
      if (cpart == pa) cpbase = kslot_lo<KB>(pa * NFP);
  }
  float qv[CMP > 1 ? 2 * NFP : 1];
  int fwl[CMP > 1 ? NFP : 1], fwh[CMP > 1 ? NFP : 1];   // field weight exponents of register j's halves
  if constexpr (CMP > 1) {
#pragma unroll
    for (int off = 0; off < 2 * NFP; off++)
      qv[off] = u2f((uint32_t)qs[ccol][kslot(cpbase + fli(off))] << 16);
#pragma unroll
    for (int j = 0; j < NFP; j++) {
      int el = 0, eh = 0;
#pragma unroll
      for (int pa = 0; pa < CMP; pa++) {
        const int f = pa * NFP + j;
        int l0, h0;
        if constexpr (MIXED) {
          l0 = -mixed_pos(f, 0);
          h0 = -mixed_pos(f, 1);
        } else {
          const Fld F = ufield<MIXED ? 2 : KB>(f);
          l0 = h0 = F.wexp - F.pos;
        }
        if (cpart == pa) { el = l0; eh = h0; }
      }
      fwl[j] = el;
      fwh[j] = eh;
    }
  }

  // fold the key scales of `tile` into the query: u = q * S * 2^k as f16 hi/lo
  // operand registers in LDS; logit constants ak, bk0
  auto fold_query = [&](const Buf& bf) {
    // stage the tile's key parameters in LDS, then read the own stream's 32
    // slots (four runs of 8 consecutive slots).  Mixed keys: each parameter
    // goes to its slot's lane-order position
    if constexpr (!MIXED) {
#pragma unroll
      for (int s = 0; s < NS; s++)
#pragma unroll
        for (int a2 = 0; a2 < 2; a2++)
#pragma unroll
          for (int j = 0; j < KPL; j++) kst[wave][s][a2][(kloff >> 2) + 64 * j] = bf.kp[s][a2][j];
    } else {
#pragma unroll
      for (int s = 0; s < NS; s++)
#pragma unroll
        for (int a2 = 0; a2 < 2; a2++) {
          uint8_t* dst = (uint8_t*)&kst[wave][s][a2][0];
#pragma unroll
          for (int j = 0; j < KPL; j++)
#pragma unroll
            for (int e = 0; e < 4 / PB; e++) {
              const int pi = j * (4 / PB) + e;
              const uint32_t v = bf.kp[s][a2][j] >> (8 * PB * e);
              if constexpr (PB == 1) {
                if (lane < 32) dst[mlpos[pi]] = (uint8_t)v;
              } else if constexpr (PB == 2) {
                *(uint16_t*)(dst + 2 * mlpos[pi]) = (uint16_t)v;
              } else {
                *(uint32_t*)(dst + 4 * mlpos[pi]) = v;
              }
            }
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if constexpr (CMP > 1) {
      // the part's 2 NFP key parameters, in offset order
      constexpr int RW = (FRUN2 ? NFP : 2 * NFP) * PB / 4;   // words per run
      auto load_kpp = [&](int which, uint32_t* pw) {
        const uint32_t* src = &kst[wave][own_c][which][0];
        const int w0 = kslot(cpbase) * PB / 4;
#pragma unroll
        for (int i = 0; i < RW; i++) pw[i] = src[w0 + i];
        if constexpr (FRUN2) {
#pragma unroll
          for (int i = 0; i < RW; i++) pw[RW + i] = src[w0 + HIOFF * PB / 4 + i];
        }
      };
      constexpr int PWP = (FRUN2 ? 2 : 1) * RW;
      uint32_t zw[PWP], sw[PWP];
      load_kpp(1, zw);
      load_kpp(0, sw);
      float bc[2] = {0.0f, 0.0f};
#pragma unroll
      for (int t = 0; t < 2 * NFP; t++) bc[t & 1] = fmaf(qv[t], pget<PDT>(zw, t), bc[t & 1]);
      float beta = bc[0] + bc[1];
      uint32_t smax = 0;
      if constexpr (PDT == KVQ_F16) {
        uint32_t m2 = sw[0];
#pragma unroll
        for (int i = 1; i < PWP; i++) m2 = pk_max_u16(m2, sw[i]);
        smax = f2u((float)__builtin_bit_cast(_Float16, (uint16_t)max(m2 & 0xffffu, m2 >> 16)));
      } else {
#pragma unroll
        for (int t = 0; t < 2 * NFP; t++) smax = max(smax, f2u(pget<PDT>(sw, t)));
      }
      const int eqs = max(eq + expo(u2f(part_maxu<CMP>(wave_maxu16x4(smax)))), -100);
      beta = part_sum<CMP>(wave_sum16x4(beta));
      const float kf = exp2i(KH - eqs);
      auto uval = [&](int t) -> float {
        if constexpr (PDT == KVQ_F16) return __builtin_fmaf(qv[t], pget<PDT>(sw, t), 0.0f);
        else return qv[t] * pget<PDT>(sw, t);
      };
      uint32_t oh[NFP], ol[NFP];
#pragma unroll
      for (int j = 0; j < NFP; j++)
        split_pack(uval(foff(j, 0)) * (kf * exp2i(fwl[j])), uval(foff(j, 1)) * (kf * exp2i(fwh[j])), oh[j], ol[j], m1);
      // register f of part 0's lane from part f / NFP of its row
      constexpr int P0 = CMP == 4 ? 0x1 : 0x3;
      auto to0 = [&](uint32_t x, int pa) -> uint32_t {
        if (pa == 1) return dpp_shl<CPW, P0>(x, x);
        if constexpr (CMP == 4) {
          if (pa == 2) return dpp_shl<2 * CPW, P0>(x, x);
          if (pa == 3) return dpp_shl<3 * CPW, P0>(x, x);
        }
        return x;
      };
#pragma unroll
      for (int f = 0; f < NFK; f++) {
        const uint32_t hi = to0(oh[f % NFP], f / NFP), lo = to0(ol[f % NFP], f / NFP);
        if constexpr (QREG) {
          qop[f >> 2][0][f & 3] = hi;
          qop[f >> 2][1][f & 3] = lo;
        } else {
          my_lds[(((f >> 2) * 2 + 0) * 64 + lane) * 4 + (f & 3)] = hi;
          my_lds[(((f >> 2) * 2 + 1) * 64 + lane) * 4 + (f & 3)] = lo;
        }
      }
      ak = __builtin_fabsf(a.sl2) * exp2i(24 - KH + eqs);
      bk0 = __builtin_fabsf(a.sl2) * beta;
      return;
    }
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
      float wh;
      if constexpr (MIXED) {
        // lane order: register f holds li = 2f (low half) and 2f + 1 (high half)
        ul = uval(2 * f);
        uh = uval(2 * f + 1);
        w = kf * exp2i(-mixed_pos(f, 0));
        wh = kf * exp2i(-mixed_pos(f, 1));
      } else {
        const Fld F = ufield<KB>(f);
        ul = uval(F.lo);
        uh = uval(F.hi);
        w = kf * exp2i(F.wexp - F.pos);
        wh = w;
      }
      uint32_t hi, lo;
      split_pack(ul * w, uh * wh, hi, lo, m1);
      // [k-step][hi/lo][lane][4]: one ds_read_b128 per operand group
      if constexpr (QREG) {
        qop[f >> 2][0][f & 3] = hi;
        qop[f >> 2][1][f & 3] = lo;
      } else {
        my_lds[(((f >> 2) * 2 + 0) * 64 + lane) * 4 + (f & 3)] = hi;
        my_lds[(((f >> 2) * 2 + 1) * 64 + lane) * 4 + (f & 3)] = lo;
      }
    }
    ak = __builtin_fabsf(a.sl2) * exp2i(24 - KH + eqs);
    bk0 = __builtin_fabsf(a.sl2) * beta;
  };

  // compute sub-tile sub of the chunk's tile ti from bf; with the two-ahead
  // prefetch, bf is refilled with sub-tile (ti2, sub2) as soon as each part has
  // been read
  auto issue_v = [&](uint32_t* vw, int k, int sub) {
#pragma unroll
    for (int s = 0; s < NS; s++) load_vw(vw + s * NVW, v_rsrc(s, t_base + k), sub);
  };
  // Value words one sub-tile ahead in two alternating buffers (VPF), for
  // the compacted one-stream instances with 2-bit values: with few tiles per
  // wave their waves otherwise wait on each sub-tile's value words, which
  // are only in flight during its own key product and softmax.  Measured
  // 2-2.4% faster per call there (128K mixed keys, B = 8 x 32K 2-bit codes),
  // neutral for mixed values and 4.7% slower for 4-bit codes, which keep
  // loading them at the start of their sub-tile.
  constexpr bool VPF = KVQ_DECODE_VPF && CMP > 1 && VB == 2;
  uint32_t vwbuf[VPF ? 2 : 1][VPF ? NS * NVW : 1];
  // (VPF) value words of sub-tile (tn, subn), the next one, go to the other
  // buffer at the start of each sub-tile; vbi (the sub-tile's parity) picks
  // the buffer holding the current one
  auto compute = [&](Buf& bf, int ti, int sub, int ti2, int sub2, int tn, int subn, int vbi) {
    uint32_t vjit[VPF ? 1 : NS * NVW];
    if constexpr (VPF) {
      if (tn >= 0) issue_v(vwbuf[vbi ^ 1], tn, subn);   // nothing past the wave's last tile
    } else {
      issue_v(vjit, ti, sub);
    }
    // (PJIT) the sub-tile's value parameters, loaded with its value words
    uint32_t pjs[PJIT ? NCV * PWV : 1], pjz[PJIT ? NCV * PWV : 1];
    if constexpr (PJIT) load_p_to(pjs, pjz, ti, sub);
    const uint32_t* vwp = VPF ? vwbuf[vbi] : vjit;
    if (sub == 0) fold_query(bf);
    // ---- logits: k-step-major over all (stream, block) accumulators
    f32x4 acc[NS][JB];
#pragma unroll
    for (int s = 0; s < NS; s++)
#pragma unroll
      for (int jj = 0; jj < JB; jj++) acc[s][jj] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < NKK; k++) {
      uint32_t bh4[4], bl4[4];
      if constexpr (QREG) {
#pragma unroll
        for (int r = 0; r < 4; r++) { bh4[r] = qop[k][0][r]; bl4[r] = qop[k][1][r]; }
      } else {
        const u32x4 bhv = *(const u32x4*)(my_lds + ((k * 2 + 0) * 64 + lane) * 4);
        const u32x4 blv = *(const u32x4*)(my_lds + ((k * 2 + 1) * 64 + lane) * 4);
#pragma unroll
        for (int r = 0; r < 4; r++) { bh4[r] = bhv[r]; bl4[r] = blv[r]; }
      }
      uint32_t av[NS][JB][4];
#pragma unroll
      for (int s = 0; s < NS; s++)
#pragma unroll
        for (int jj = 0; jj < JB; jj++)
#pragma unroll
          for (int r = 0; r < 4; r++) {
            const int f = 4 * k + r;
            if constexpr (MIXED) {
              av[s][jj][r] = mixed_field(bf.kw[s][jj], f);
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
    if (ti2 >= 0) load_k(bf, ti2, sub2);   // nothing to prefetch past the wave's last tile
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
    // compacted softmax: slot s of part a is token ufield(a * RPL + s).lo for
    // s < RPL, ufield(a * RPL + s - RPL).hi above, fetched from lane ccol of
    // the row (part 0 keeps its own)
    float lc[NL];
    if constexpr (CMP > 1) {
      auto tok = [](int pa, int sl) -> int { return cmp_tok<VBF, RPL>(pa, sl); };
#pragma unroll
      for (int sl = 0; sl < NL; sl++) {
        uint32_t x = f2u(lv[tok(0, sl)]);
        if constexpr (CMP == 2) {
          x = dpp_shr<8, 0xC>(x, f2u(lv[tok(1, sl)]));
        } else {
          x = dpp_shr<4, 0x2>(x, f2u(lv[tok(1, sl)]));
          x = dpp_shr<8, 0x4>(x, f2u(lv[tok(2, sl)]));
          x = dpp_shr<12, 0x8>(x, f2u(lv[tok(3, sl)]));
        }
        lc[sl] = u2f(x);
      }
    } else {
#pragma unroll
      for (int i = 0; i < TPS; i++) lc[i] = lv[i];
    }
    // the lane's largest logit (ak >= 0: from its largest raw sum)
    float vx = lc[0];
#pragma unroll
    for (int i = 1; i < NL; i++) vx = fmaxf(vx, lc[i]);
    const float lmax = fmaf(ak, vx, bk0);
    // value parameters of the sub-tile; binary16 ones stay raw and are read
    // by mixed-precision fmas.  smx: the lane's largest value scale as a
    // binary32 bit pattern (scales are >= +0, so patterns order like values)
    constexpr bool MIX = (PDT == KVQ_F16);
    uint32_t rvs[NCV * PWV], rvz[NCV * PWV];
    float vs[(MIX || VMIX) ? 1 : NL], vz[(MIX || VMIX) ? 1 : NL];
    uint32_t smx;
    if constexpr (VMIX) {
      // raw words only; the largest scale straight from the patterns (scales
      // are >= +0, so binary16 and e4m3 patterns order like their values)
      static_assert(!VMIX || PDT == KVQ_F16 || PDT == KVQ_E4M3, "mixed values: binary16 or e4m3 parameters");
#pragma unroll
      for (int w = 0; w < NCV * PWV; w++) {
        if constexpr (PJIT) {
          rvs[w] = pjs[w];
          rvz[w] = pjz[w];
        } else {
          rvs[w] = bf.vs[w];
          rvz[w] = bf.vz[w];
        }
      }
      if constexpr (MIX) {
        uint32_t m2 = rvs[0];
#pragma unroll
        for (int w = 1; w < NCV * PWV; w++) m2 = pk_max_u16(m2, rvs[w]);
        smx = f2u((float)__builtin_bit_cast(_Float16, (uint16_t)max(m2 & 0xffffu, m2 >> 16)));
      } else {
        // bytes 1 and 3 of each word lead their 16-bit halves, so the halves'
        // maxima of the words carry the largest byte 1 / byte 3 in their high
        // bytes; the words shifted left by 8 do the same for bytes 0 and 2
        uint32_t hi = rvs[0], lo = rvs[0] << 8;
#pragma unroll
        for (int w = 1; w < NCV * PWV; w++) {
          hi = pk_max_u16(hi, rvs[w]);
          lo = pk_max_u16(lo, rvs[w] << 8);
        }
        const uint32_t m2 = pk_max_u16(hi, lo);
        smx = f2u(__builtin_amdgcn_cvt_f32_fp8((int)max((m2 >> 8) & 0xffu, m2 >> 24), 0));
      }
    } else if constexpr (MIX) {
#pragma unroll
      for (int w = 0; w < PWV; w++) { rvs[w] = bf.vs[w]; rvz[w] = bf.vz[w]; }
      uint32_t m2 = rvs[0];
#pragma unroll
      for (int w = 1; w < PWV; w++) m2 = pk_max_u16(m2, rvs[w]);
      smx = f2u((float)__builtin_bit_cast(_Float16, (uint16_t)max(m2 & 0xffffu, m2 >> 16)));
    } else {
      praw_unpack<PDT, NL>(bf.vs, vs);
      praw_unpack<PDT, NL>(bf.vz, vz);
      smx = 0;
#pragma unroll
      for (int i = 0; i < NL; i++) smx = max(smx, f2u(vs[i]));
    }
    if (ti2 >= 0) load_p(bf, ti2, sub2);
    // A column's reference max moves only when one of its logits exceeds it
    // by more than TAU, and its value-scale exponent e_run only when a larger
    // scale arrives.  Both need the reductions over the four lane groups, so
    // they (and the rescale of the running sums and accumulators) run only
    // when some lane of the wave sees such a logit or scale.
    if (__builtin_amdgcn_ballot_w64(lmax > m_run + (float)TAU || expo(u2f(smx)) > e_run) != 0) {
      // (compacted: over the lanes of the column in every part too)
      const float tmax = part_max<CMP>(wave_max16x4(lmax));
      const int ev = expo(u2f(part_maxu<CMP>(wave_maxu16x4(smx))));
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
      for (int k = 0; k < NCV; k++) zm_run[k] *= rescale;
#pragma unroll
      for (int cb = 0; cb < 8; cb++) acc_o[cb] *= rescale;
    }
    if constexpr (VMIX) {
      // Mixed-width values.  e(i) = 2^(logit - m) * 2^ps without field
      // weight; class k's probability operand is P_k(i) = e(i) * S_k(i) *
      // 2^W(i), W(i) the weight of token i's field in the class's container
      // (4-bit fields for classes 0, 1, 2-bit fields for classes 2, 3).
      // Each class keeps its own zero-point sum, with the rounding of its
      // binary16 P~ made up at the class's code midpoint as for uniform
      // widths; the residual sums read P~ * 2^-W exactly through fdot2.
      const float c0 = bk0 - m_run + (float)min(VH - e_run, PSMAX);
      if constexpr (CMP > 1) {
        // compacted (slot sl of the lane: token parity sl % 2, probability
        // register sl % RPL of its 2-bit field): per class the lane's NL
        // binary16 operands as pairs Q[m] = (slot 2m, slot 2m + 1), then the
        // registers of part 0's lane.  4-bit container register ff pairs
        // tokens t and t + 4 (t = 8 (ff / 4) + ff % 4), held by parts p and
        // p + CMP / 2 of the row at the same slot; 2-bit container register
        // a * RPL + r pairs slots r and RPL + r of part a.
        float e[NL];
        float lsum = 0.0f;
#pragma unroll
        for (int sl = 0; sl < NL; sl++) {
          e[sl] = __builtin_amdgcn_exp2f(fmaf(ak, lc[sl], c0));
          lsum += e[sl];
        }
        l_run += lsum;
        constexpr int P0 = CMP == 4 ? 0x1 : 0x3;
#pragma unroll
        for (int k = 0; k < 4; k++) {
          const float vmid = 0.5f * (float)((1u << vmixed_class_bits(k)) - 1u);
          const uint32_t* ks = rvs + k * PWV;
          const uint32_t* kz = rvz + k * PWV;
          float zc = 0.0f, zr = 0.0f;
          float p[NL];
#pragma unroll
          for (int sl = 0; sl < NL; sl++) {
            const float ew = e[sl] * (k < 2 ? ((sl & 1) ? 0.0625f : 1.0f) : cew[sl % RPL]);
            if constexpr (MIX) {
              zc = fmaf(e[sl], __builtin_fmaf(vmid, half_at(ks, sl), half_at(kz, sl)), zc);
              p[sl] = fmaf(ew, half_at(ks, sl), 0.0f);
            } else {
              const float sk = pget<PDT>(ks, sl);
              zc = fmaf(e[sl], fmaf(vmid, sk, pget<PDT>(kz, sl)), zc);
              p[sl] = ew * sk;
            }
          }
          uint32_t qp[NL / 2];
#pragma unroll
          for (int m = 0; m < NL / 2; m++) {
            const f16x2 h = __builtin_convertvector((f32x2){p[2 * m], p[2 * m + 1]}, f16x2);
            qp[m] = __builtin_bit_cast(uint32_t, h);
          }
          uint32_t bv[FVS];
          if (k < 2) {
            // 2^-W of the 4-bit fields: 1 (even tokens), 16 (odd)
#pragma unroll
            for (int m = 0; m < NL / 2; m++)
              zr = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, qp[m]), (f16x2){1.0f16, 16.0f16}, zr, false);
#pragma unroll
            for (int ff = 0; ff < FVS; ff++) {
              uint32_t lo, hi;   // the pair's halves: parts pl (low token) and pl + CMP / 2
              int m;
              if constexpr (CMP == 4) {
                m = ff / 4;
                const int pl = (ff % 4) / 2;
                lo = pl == 0 ? qp[m] : dpp_shl<4, P0>(qp[m], qp[m]);
                hi = pl == 0 ? dpp_shl<8, P0>(qp[m], qp[m]) : dpp_shl<12, P0>(qp[m], qp[m]);
              } else {
                m = ff / 2;
                lo = qp[m];
                hi = dpp_shl<8, P0>(qp[m], qp[m]);
              }
              (void)m;
              bv[ff] = (ff & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u) : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
            }
          } else {
            uint32_t pr[RPL];
#pragma unroll
            for (int r = 0; r < RPL; r++) {
              const uint32_t a0 = qp[r / 2], a1 = qp[(RPL + r) / 2];
              pr[r] = (r & 1) ? __builtin_amdgcn_perm(a1, a0, 0x07060302u) : __builtin_amdgcn_perm(a1, a0, 0x05040100u);
              const _Float16 iw = (_Float16)ciw[r];
              zr = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pr[r]), (f16x2){iw, iw}, zr, false);
            }
#pragma unroll
            for (int r = 0; r < RPL; r++) {
              bv[r] = pr[r];
              if constexpr (CMP == 2) {
                bv[RPL + r] = dpp_shl<8, 0x3>(pr[r], pr[r]);
              } else {
                bv[RPL + r] = dpp_shl<4, 0x1>(pr[r], pr[r]);
                bv[2 * RPL + r] = dpp_shl<8, 0x1>(pr[r], pr[r]);
                bv[3 * RPL + r] = dpp_shl<12, 0x1>(pr[r], pr[r]);
              }
            }
          }
          zm_run[k] += fmaf(-vmid, zr, zc);
#pragma unroll
          for (int cb = 0; cb < 8; cb++) {
            if (vmixed_block_class(cb) != k) continue;
#pragma unroll
            for (int kk = 0; kk < KSV; kk++) {
              uint32_t av[4];
#pragma unroll
              for (int r = 0; r < 4; r++) {
                const Fld F = cb < 2 ? ufield<4>(4 * kk + r) : ufield<2>(4 * kk + r);
                av[r] = field_subnormal(cb < 2 ? vwp[2 * cb + F.w] : vwp[2 + cb], F);
              }
              acc_o[cb] = mfma(av, bv + 4 * kk, acc_o[cb]);
            }
          }
        }
      } else {
        float e[TPS];
        float lsum = 0.0f;
  #pragma unroll
        for (int i = 0; i < TPS; i++) {
          e[i] = __builtin_amdgcn_exp2f(fmaf(ak, lv[i], c0));
          lsum += e[i];
        }
        l_run += lsum;
        // one class at a time: its operand, its zero-point sum, then the value
        // products of its slot blocks (block k for k < 3, blocks 3..7 for k = 3)
  #pragma unroll
        for (int k = 0; k < 4; k++) {
          const float vmid = 0.5f * (float)((1u << vmixed_class_bits(k)) - 1u);
          const uint32_t* ks = rvs + k * PWV;
          const uint32_t* kz = rvz + k * PWV;
          float zc = 0.0f, zr = 0.0f;
          float p[TPS];
  #pragma unroll
          for (int i = 0; i < TPS; i++) {
            const float ew = e[i] * exp2i(k < 2 ? tok_w<4, FVS>(i) : tok_w<2, FVS>(i));
            if constexpr (MIX) {
              zc = fmaf(e[i], __builtin_fmaf(vmid, half_at(ks, i), half_at(kz, i)), zc);
              p[i] = fmaf(ew, half_at(ks, i), 0.0f);
            } else {
              const float sk = pget<PDT>(ks, i);
              zc = fmaf(e[i], fmaf(vmid, sk, pget<PDT>(kz, i)), zc);
              p[i] = ew * sk;
            }
          }
          uint32_t bv[FVS];
  #pragma unroll
          for (int ff = 0; ff < FVS; ff++) {
            const Fld F = k < 2 ? ufield<4>(ff) : ufield<2>(ff);
            const f16x2 h = __builtin_convertvector((f32x2){p[F.lo], p[F.hi]}, f16x2);
            bv[ff] = __builtin_bit_cast(uint32_t, h);
            const _Float16 iw = (_Float16)exp2i(F.pos - F.wexp);   // 2^-W: 1 .. 256, exact
            zr = __builtin_amdgcn_fdot2(h, (f16x2){iw, iw}, zr, false);
          }
          zm_run[k] += fmaf(-vmid, zr, zc);
  #pragma unroll
          for (int cb = 0; cb < 8; cb++) {
            if (vmixed_block_class(cb) != k) continue;
  #pragma unroll
            for (int kk = 0; kk < KSV; kk++) {
              uint32_t av[4];
  #pragma unroll
              for (int r = 0; r < 4; r++) {
                const Fld F = cb < 2 ? ufield<4>(4 * kk + r) : ufield<2>(4 * kk + r);
                av[r] = field_subnormal(cb < 2 ? vwp[2 * cb + F.w] : vwp[2 + cb], F);
              }
              acc_o[cb] = mfma(av, bv + 4 * kk, acc_o[cb]);
            }
          }
        }
      }
    } else {
      // e''(i) = e(i) * 2^ps * 2^W(i) straight from the exponent; the running
      // sums l_run, z_run are kept in units of 2^ps.
      // The probability operand of PV is one binary16 per token (P~ = rne(P)).
      // Its rounding residual r = P - P~ meets every code of the token; the
      // part r * VMID (VMID = the codes' midpoint (2^VB - 1) / 2) is added back
      // exactly through the zero-point sum -- e * (Z + VMID * S) - VMID * P~ --
      // and only r * (code - VMID), which has no common sign, is left out.
      constexpr float VMID = 0.5f * (float)((1u << VB) - 1u);
      const float c0 = bk0 - m_run + (float)min(VH - e_run, PSMAX);
      uint32_t bvh[FVS];
      if constexpr (CMP > 1) {
        // compacted: the lane's NL slots (one column, two runs of RPL tokens),
        // then its RPL probability registers (slot r low, slot RPL + r high)
        // back to lane ccol of part 0 as registers cpart * RPL + r
        float p[NL];
        float lsum = 0.0f;
        float zc[RPL], zr[RPL];
#pragma unroll
        for (int r = 0; r < RPL; r++) { zc[r] = 0.0f; zr[r] = 0.0f; }
#pragma unroll
        for (int sl = 0; sl < NL; sl++) {
          const int r = sl % RPL;
          const float e = __builtin_amdgcn_exp2f(fmaf(ak, lc[sl], c0 + cw[r]));
          lsum = fmaf(e, ciw[r], lsum);
          if constexpr (MIX) {
            zc[r] = fmaf(e, __builtin_fmaf(VMID, half_at(rvs, sl), half_at(rvz, sl)), zc[r]);
            p[sl] = fmaf(e, half_at(rvs, sl), 0.0f);
          } else {
            zc[r] = fmaf(e, fmaf(VMID, vs[sl], vz[sl]), zc[r]);
            p[sl] = e * vs[sl];
          }
        }
        l_run += lsum;
        uint32_t pr[RPL];
        float zsum = 0.0f;
#pragma unroll
        for (int r = 0; r < RPL; r++) {
          const f16x2 h = __builtin_convertvector((f32x2){p[r], p[RPL + r]}, f16x2);
          pr[r] = __builtin_bit_cast(uint32_t, h);
          zr[r] = __builtin_amdgcn_fdot2(h, (f16x2){1.0f16, 1.0f16}, zr[r], false);
          zsum = fmaf(fmaf(-VMID, zr[r], zc[r]), ciw[r], zsum);
        }
        z_run += zsum;
#pragma unroll
        for (int r = 0; r < RPL; r++) {
          bvh[r] = pr[r];
          if constexpr (CMP == 2) {
            bvh[RPL + r] = dpp_shl<8, 0x3>(pr[r], pr[r]);
          } else {
            bvh[RPL + r] = dpp_shl<4, 0x1>(pr[r], pr[r]);
            bvh[2 * RPL + r] = dpp_shl<8, 0x1>(pr[r], pr[r]);
            bvh[3 * RPL + r] = dpp_shl<12, 0x1>(pr[r], pr[r]);
          }
        }
      } else {
        float p[TPS];
        float lsum = 0.0f;
        float zc[10], zr[10];
    #pragma unroll
        for (int k = 0; k < 10; k++) { zc[k] = 0.0f; zr[k] = 0.0f; }
    #pragma unroll
        for (int i = 0; i < TPS; i++) {
          const int W = tok_w<VB, FVS>(i);
          const float e = __builtin_amdgcn_exp2f(fmaf(ak, lv[i], c0 + (float)W));
          lsum = fmaf(e, exp2i(-W), lsum);
          if constexpr (MIX) {
            zc[w_class(W)] = fmaf(e, __builtin_fmaf(VMID, half_at(rvs, i), half_at(rvz, i)), zc[w_class(W)]);
            p[i] = fmaf(e, half_at(rvs, i), 0.0f);
          } else {
            zc[w_class(W)] = fmaf(e, fmaf(VMID, vs[i], vz[i]), zc[w_class(W)]);
            p[i] = e * vs[i];
          }
        }
        l_run += lsum;

        // ---- P operand and PV; every sub-tile has the field layout of sub-tile
        // 0, shifted by WVS words and TPS tokens
    #pragma unroll
        for (int ff = 0; ff < FVS; ff++) {
          // a token whose codes span two fields (the bytes of a 16-bit code)
          // carries the weight of its first field; the other gets the difference
          const Fld F = ufield<VB>(ff);
          const int dwe = (F.wexp - F.pos) - tok_w<VB, FVS>(F.lo);
          const f16x2 h = __builtin_convertvector((f32x2){p[F.lo] * exp2i(dwe), p[F.hi] * exp2i(dwe)}, f16x2);
          bvh[ff] = __builtin_bit_cast(uint32_t, h);
          // the tokens' first field: P~ of both tokens into the residual sums
          if (dwe == 0) zr[w_class(tok_w<VB, FVS>(F.lo))] = __builtin_amdgcn_fdot2(h, (f16x2){1.0f16, 1.0f16},
                                                                                   zr[w_class(tok_w<VB, FVS>(F.lo))], false);
        }
        float zsum = fmaf(-VMID, zr[0], zc[0]);
    #pragma unroll
        for (int k = 1; k < 10; k++)
          if (class_used<VB, FVS, TPS>(k)) zsum = fmaf(fmaf(-VMID, zr[k], zc[k]), exp2i(-class_w<VB>(k)), zsum);
        z_run += zsum;
      }
  #pragma unroll
      for (int s = 0; s < NS; s++) {
        uint32_t bsh[FVS];
  #pragma unroll
        for (int ff = 0; ff < FVS; ff++) {
          const bool sel = (NS == 1) || (own == s);
          bsh[ff] = sel ? bvh[ff] : 0u;
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
        }
      }
    }
  };

  // ---- software-pipelined main loop (two register buffers).  One iteration
  // covers U sub-tiles (a whole tile, or two one-sub-tile tiles) unrolled, so
  // the fold and every buffer choice are compile-time; past the wave's last
  // tile the prefetches are skipped (a wave-uniform branch).  Re-reading the
  // last tile instead measured 6% more DRAM reads than the algorithmic bytes
  // (non-temporal code loads miss on the re-read).
  constexpr int U = NSUB >= 2 ? NSUB : 2;
  constexpr int TPI = U / NSUB;   // tiles per iteration (2 for one-sub-tile tiles)
  q1 = q0 + 4; q2 = q0 + 8; q3 = q0 + 12;
  // the queue entry for sub-tile offset d (d = 0..3 tiles ahead), or -1 when
  // it lies past the chunk
  auto qk = [&](int d) -> int {
    const int v = d == 0 ? q0 : (d == 1 ? q1 : (d == 2 ? q2 : q3));
    return v < t_count ? v : -1;
  };
  // the second buffer: loads run two sub-tiles ahead of the computation (one
  // ahead, in the single buffer, for PF1 instances)
  if constexpr (!PF1)
    if (q0 < t_count && qk(1 / NSUB) >= 0) load(b1, qk(1 / NSUB), 1 % NSUB);
  if constexpr (VPF)
    if (q0 < t_count) issue_v(vwbuf[0], q0, 0);   // the first sub-tile's value words
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
      if constexpr (PF1)
        compute(b0, qk(u / NSUB), u % NSUB, qk((u + 1) / NSUB), (u + 1) % NSUB, qk((u + 1) / NSUB), (u + 1) % NSUB,
                u % 2);
      else
        compute((u % 2 == 0) ? b0 : b1, qk(u / NSUB), u % NSUB, qk((u + 2) / NSUB), (u + 2) % NSUB,
                qk((u + 1) / NSUB), (u + 1) % NSUB, u % 2);
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
  // (compacted: the column's sums are spread over the parts of its row)
  const float l_tot = part_sum<CMP>(wave_sum16x4(l_run)) * unps;
  const float z_tot = part_sum<CMP>(wave_sum16x4(z_run)) * unps;
  float zm_tot[NCV];
#pragma unroll
  for (int k = 0; k < NCV; k++) zm_tot[k] = VMIX ? part_sum<CMP>(wave_sum16x4(zm_run[k])) * unps : 0.0f;
  const float of = exp2i(24 - ps);           // acc_o * 2^24 / 2^ps
  if (lg == 0) {
    sh_ml[wave][n][0] = m_run;
    sh_ml[wave][n][1] = l_tot;
  }
  // output row 16 cb + 4 lg + i is value slot 16 cb + 4 lg + i: channel
  // v_slot_chan[kv head][slot] for mixed values (low 7 bits, so a map that
  // is not a permutation scatters within the row), the slot itself otherwise
  const int16_t* vsc = VMIX ? g.v_slot_chan + (int64_t)((real ? bh_own : 0) % g.H) * 128 : nullptr;
#pragma unroll
  for (int cb = 0; cb < 8; cb++)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float a = acc_o[cb][i];
      const int slot = 16 * cb + 4 * lg + i;
      const int ch = VMIX ? ((int)vsc[slot] & 127) : slot;
      const float zt = VMIX ? zm_tot[vmixed_block_class(cb)] : z_tot;
      sh_o(wave, n, ch) = (m_run == -INFINITY) ? 0.0f : a * of + zt;
    }
  __syncthreads();

  const int ncol = NS * G;
  const bool single = (a.n_slots == 1) && a.out != nullptr;   // no out: partials only
  // per column: the workgroup max M, the weight 2^(m_w - M) of each wave's
  // partial, the sum and the destination row -- the output row
  // (batch, query head) = grp * NS * G + col when this is the stream's only
  // partial, else the partial row of this chunk (-1: no head in the column)
  __shared__ float sh_cw[16][4];
  __shared__ float sh_cd[16][2];
  __shared__ int sh_row[16];
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
    sh_row[col] = bh >= BH ? -1 : (single ? bh * G + hh : (bh * a.n_slots + a.slot0 + chunk) * G + hh);
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
      if (c4 == 0) { a.part_ml[2 * (int64_t)row] = sh_cd[col][0]; a.part_ml[2 * (int64_t)row + 1] = sh_cd[col][1]; }
      *(f32x4*)(a.part_o + (int64_t)row * 128 + c4) = num;
    }
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
// streams per wave for mixed keys with 2-bit values.  Two, with one
// prefetch buffer (PF1) and the folded query in LDS, fit two waves per SIMD
// without spills: 12-18% faster than one stream on batched 32K and 128K
// mixed-key layers (G = 4), the same at B = 4 x 128K; single sequences keep
// one stream (too few tiles per chunk, KVQ_DECODE_NS_MIN_TPC).  With two
// buffers they spilled and ran 30% slower; three streams 2x slower.
#ifndef KVQ_DECODE_NS_CAP_MIXED2
#define KVQ_DECODE_NS_CAP_MIXED2 2
#endif
constexpr int ns_cap(int kb, int vb) {
  if (kb == 0) return vb == 4 ? 2 : (vb == 2 ? KVQ_DECODE_NS_CAP_MIXED2 : 1);
  return kb == 4 ? KVQ_DECODE_NS_CAP_LOW : (kb == 2 ? KVQ_DECODE_NS_CAP_2BIT : 1);
}

// Launch plan (shared by workspace sizing, validation and launch): NS streams
// per wave, n_groups = ceil(BH / NS) stream groups, and the token tiles of a
// group cut into n_chunks chunks of tpc tiles, aiming at one round of
// resident workgroups (256 CUs x waves per SIMD) with 4..64 tiles per chunk and
// at most KVQ_MAX_CHUNKS chunks.
static DecodePlan plan_for(int BH, int ns, int k_bits, int v_bits, int pdt, int n_tiles, int max_chunks, int G) {
  DecodePlan p;
  p.ns = ns;
  p.n_groups = (BH + ns - 1) / ns;
  const long total = (long)p.n_groups * n_tiles;
  // about one round of resident workgroups
  const long wg_target = (long)KVQ_DECODE_WG_PER_OCC * decode_occ(k_bits, v_bits, pdt, ns, cmp_for(k_bits, v_bits, ns, G));
  int tpc = (int)((total + wg_target - 1) / wg_target);
  tpc = ((tpc + 3) / 4) * 4;
  if (tpc < 4) tpc = 4;
  if (tpc > 64) tpc = 64;
  const int tmin = (n_tiles + max_chunks - 1) / max_chunks;
  if (tpc < tmin) tpc = tmin;
  p.n_chunks = (n_tiles + tpc - 1) / tpc;
  p.tpc = (n_tiles + p.n_chunks - 1) / p.n_chunks;   // balanced, every chunk non-empty
  return p;
}

// As many streams per wave as the columns and ns_cap() allow -- unless that
// leaves a wave fewer than four tiles, where a single stream per wave (twice
// the tiles, the prologue and partial write amortised over more work) is
// faster.
DecodePlan decode_plan(int BH, int G, int k_bits, int v_bits, int pdt, int n_tiles, int max_chunks) {
  // (binary32 parameters of mixed keys with 2-bit values: one stream, two spill)
  const int cap = (k_bits == 0 && v_bits == 2 && pdt == KVQ_F32) ? 1 : ns_cap(k_bits, v_bits);
  int ns = 16 / G;
  if (ns > KVQ_DECODE_NS_MAX) ns = KVQ_DECODE_NS_MAX;
  ns = ns > cap ? cap : (ns < 1 ? 1 : ns);
  DecodePlan p = plan_for(BH, ns, k_bits, v_bits, pdt, n_tiles, max_chunks, G);
  if (ns > 1 && p.tpc < KVQ_DECODE_NS_MIN_TPC) p = plan_for(BH, 1, k_bits, v_bits, pdt, n_tiles, max_chunks, G);
  return p;
}

// Chunk combine, a separate launch so that the partials are visible without
// device-scope fences.  One wave per output row (batch, query head):
//   o = sum_k 2^(m_k - M) o_k / sum_k 2^(m_k - M) l_k,  M = max_k m_k.
// Lane k holds the (m, l) of chunks k and k + 64; each lane owns two channels
// of o and walks the chunks with the weight broadcast from its owner lane.
// output rows (one wave each) per combine workgroup.  One: the rows spread
// over as many CUs as there are rows, which measured 2% faster per call on
// a single 128K sequence (32 rows) than four rows per workgroup, and the same
// on the batched layers.
#ifndef KVQ_COMBINE_WAVES
#define KVQ_COMBINE_WAVES 1
#endif
template <int KP>
__global__ __launch_bounds__(64 * KVQ_COMBINE_WAVES) void decode_combine_kernel(const float* __restrict__ part_ml,
                                                             const float* __restrict__ part_o,
                                                             float* __restrict__ out, int BH, int H,
                                                             int G, int nck) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * KVQ_COMBINE_WAVES + (threadIdx.x >> 6);   // bh * G + hh
  if (row >= BH * G) return;
  const int bh = row / G, hh = row - (row / G) * G;
  const int64_t r0 = (int64_t)bh * nck * G + hh;         // partial row of chunk 0
  float m0 = -INFINITY, m1 = -INFINITY, l0 = 0.0f, l1 = 0.0f;
  if (lane < nck) { m0 = part_ml[2 * (r0 + (int64_t)lane * G)]; l0 = part_ml[2 * (r0 + (int64_t)lane * G) + 1]; }
  if (lane + 64 < nck) {
    m1 = part_ml[2 * (r0 + (int64_t)(lane + 64) * G)];
    l1 = part_ml[2 * (r0 + (int64_t)(lane + 64) * G) + 1];
  }
  // the first KP (>= nck up to 64) chunk outputs are loaded before the
  // weights are known, so the combine costs one memory round trip
  const float* po = part_o + r0 * 128 + 2 * lane;
  const int64_t step = (int64_t)G * 128;
  float2 v[KP];
#pragma unroll
  for (int k = 0; k < KP; k++) v[k] = (k < nck) ? *(const float2*)(po + step * k) : make_float2(0.f, 0.f);
  float M = fmaxf(m0, m1);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  const float w0 = exp2f(m0 - M), w1 = exp2f(m1 - M);   // 0 for absent chunks
  float den = w0 * l0 + w1 * l1;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) den += __shfl_xor(den, o, 64);
  float n0 = 0.0f, n1 = 0.0f;
#pragma unroll
  for (int k = 0; k < KP; k++) {
    const float w = u2f(__builtin_amdgcn_readlane(f2u(w0), k));   // 0 beyond nck
    n0 = fmaf(w, v[k].x, n0);
    n1 = fmaf(w, v[k].y, n1);
  }
  // slots past 64 in batches of 16 independent loads (a
  // batch past the last slot re-reads that slot, at weight 0)
  for (int k0 = KP; k0 < nck; k0 += 16) {
    float2 x[16];
#pragma unroll
    for (int k = 0; k < 16; k++) x[k] = *(const float2*)(po + step * min(k0 + k, nck - 1));
#pragma unroll
    for (int k = 0; k < 16; k++) {
      const int kk = k0 + k;
      const float w = u2f(__builtin_amdgcn_readlane(f2u(kk < 64 ? w0 : w1), kk & 63));   // 0 beyond nck
      n0 = fmaf(w, x[k].x, n0);
      n1 = fmaf(w, x[k].y, n1);
    }
  }
  const float inv = 1.0f / den;
  const int bo = bh / H, ho = bh - (bh / H) * H;
  *(float2*)(out + ((int64_t)bo * H * G + (int64_t)ho * G + hh) * 128 + 2 * lane) = make_float2(n0 * inv, n1 * inv);
}

// the combine instance that preloads every slot up to 64
static hipError_t launch_combine(const float* part_ml, const float* part_o, float* out, int BH, int H, int G,
                                 int n_slots, hipStream_t st) {
  const int rows = BH * G;
  const dim3 grid((rows + KVQ_COMBINE_WAVES - 1) / KVQ_COMBINE_WAVES), block(64 * KVQ_COMBINE_WAVES);
  if (n_slots <= 16)
    hipLaunchKernelGGL(decode_combine_kernel<16>, grid, block, 0, st, part_ml, part_o, out, BH, H, G, n_slots);
  else if (n_slots <= 32)
    hipLaunchKernelGGL(decode_combine_kernel<32>, grid, block, 0, st, part_ml, part_o, out, BH, H, G, n_slots);
  else
    hipLaunchKernelGGL(decode_combine_kernel<64>, grid, block, 0, st, part_ml, part_o, out, BH, H, G, n_slots);
  return hipGetLastError();
}

static size_t ml_bytes(int BH, int n_chunks, int G) {
  return ((size_t)BH * n_chunks * G * 2 * 4 + 255) / 256 * 256;
}
// partial slots: every chunk plus the most a residual segment can add
size_t decode_workspace_needed(int BH, int G, const DecodePlan& p) {
  const int slots = p.n_chunks + KVQ_MAX_RES_SLOTS;
  return ml_bytes(BH, slots, G) + (size_t)BH * slots * G * 128 * 4;
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
  if (k_bits == 0) return v_bits == 1 || v_bits == 2 || v_bits == 4 || (v_bits == 0 && (pdt == KVQ_E4M3 || pdt == KVQ_F16));
  return k_bits == v_bits && (k_bits == 1 || k_bits == 2 || k_bits == 4 || k_bits == 8 || k_bits == 16);
}

// a0 carries n_slots, slot0 and the residual rows; the plan gives the
// grid (the same plan the caller validated the workspace against)
template <int KB, int VB, int PDT>
static hipError_t launch_ns(const DecodeArgs& a0, const DecodePlan& p, hipStream_t st) {
  constexpr int CAP = ns_cap(KB, VB);
  DecodeArgs a = a0;
  a.n_groups = p.n_groups;
  a.n_chunks = p.n_chunks;
  a.tpc = p.tpc;
  const int res_rows = a.n_res ? (a.n_res * a.g.B * a.g.H + a.n_chunks - 1) / a.n_chunks : 0;
  const dim3 grid(a.n_chunks, a.n_groups + res_rows), block(256);
  if (p.ns == 1) {
    // one stream: a compacted softmax where the heads fill at most a half or
    // a quarter of the MFMA columns (with two streams per wave it measured no
    // faster: B = 8 x 32K mixed keys and B = 16 x 32K 2-bit codes, G = 4)
    if constexpr (cmp_instance(KB, VB)) {
      const int cmp = cmp_for(KB, VB, 1, a.G);
      if (cmp == 4) {
        hipLaunchKernelGGL((decode_kernel<KB, VB, PDT, 1, 4>), grid, block, 0, st, a);
        return hipGetLastError();
      }
      if (cmp == 2) {
        hipLaunchKernelGGL((decode_kernel<KB, VB, PDT, 1, 2>), grid, block, 0, st, a);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((decode_kernel<KB, VB, PDT, 1, 1>), grid, block, 0, st, a);
  } else if (p.ns == 2) {
    if constexpr (CAP >= 2) hipLaunchKernelGGL((decode_kernel<KB, VB, PDT, 2, 1>), grid, block, 0, st, a);
  } else if (p.ns == 3) {
    if constexpr (CAP >= 3) hipLaunchKernelGGL((decode_kernel<KB, VB, PDT, 3, 1>), grid, block, 0, st, a);
  } else {
    if constexpr (CAP >= 4) hipLaunchKernelGGL((decode_kernel<KB, VB, PDT, 4, 1>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

template <int PDT>
static hipError_t launch_decode_pdt(const DecodeArgs& a, const DecodePlan& p, hipStream_t st) {
  const int kb = a.g.k_bits, vb = a.g.v_bits;
#define KVQ_DEC(KBV, VBV) \
  if (kb == KBV && vb == VBV) return launch_ns<KBV, VBV, PDT>(a, p, st);
  KVQ_DEC(16, 16) KVQ_DEC(8, 8) KVQ_DEC(4, 4) KVQ_DEC(2, 2) KVQ_DEC(1, 1)
  KVQ_DEC(0, 1) KVQ_DEC(0, 2) KVQ_DEC(0, 4)
  if constexpr (PDT == KVQ_E4M3 || PDT == KVQ_F16) {
    KVQ_DEC(0, 0)
  }
#undef KVQ_DEC
  return hipErrorInvalidValue;
}

static hipError_t launch_decode_any(const DecodeArgs& a, const DecodePlan& p, hipStream_t st) {
  switch (a.g.pdt) {
    case KVQ_F32: return launch_decode_pdt<KVQ_F32>(a, p, st);
    case KVQ_F16: return launch_decode_pdt<KVQ_F16>(a, p, st);
    case KVQ_BF16: return launch_decode_pdt<KVQ_BF16>(a, p, st);
    case KVQ_E4M3: return launch_decode_pdt<KVQ_E4M3>(a, p, st);
  }
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
  float* part_ml = (float*)ws;
  float* part_o = (float*)((uint8_t*)part_ml + ml_bytes(BH, n_slots, G));
  hipError_t e = hipSuccess;
  // the residual blocks ride along as extra workgroups of the decode launch;
  // with no packed tokens they run as their own kernel
  const bool res_inline = has_packed && n_res > 0;
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
    a.n_slots = n_slots;
    a.slot0 = 0;
    a.res = res;
    a.res_dtype = res_dtype;
    a.n_res = res_inline ? n_res : 0;
    e = launch_decode_any(a, p, st);
    if (e != hipSuccess) return e;
  }
  if (n_slots > 1) e = launch_combine(part_ml, part_o, out, BH, g.H, G, n_slots, st);
  return e;
}

// First phase alone: the packed cache's chunk partials, written to the
// workspace even when the plan has a single chunk (out = null tells the
// kernel so); the plan's slot count and tiles per slot go to the caller.
hipError_t launch_decode_partials(const Geo& g, const void* q, int G, float scale, void* ws, int* n_slots,
                                  int* tiles_per_slot, hipStream_t st) {
  const int BH = g.B * g.H;
  const DecodePlan p = decode_plan(BH, G, g.k_bits, g.v_bits, g.pdt, g.n_tiles);
  DecodeArgs a;
  a.g = g;
  a.q = (const uint16_t*)q;
  a.out = nullptr;
  a.part_ml = (float*)ws;
  a.part_o = (float*)((uint8_t*)ws + ml_bytes(BH, p.n_chunks, G));
  a.G = G;
  a.sl2 = scale * 1.4426950408889634f;
  a.n_chunks = a.tpc = a.n_groups = 0;
  a.n_slots = p.n_chunks;
  a.slot0 = 0;
  a.res = ResArgs{};
  a.res.R = 0;
  a.res_dtype = KVQ_F32;
  a.n_res = 0;
  *n_slots = p.n_chunks;
  *tiles_per_slot = p.tpc;
  return launch_decode_any(a, p, st);
}

// Second phase alone: the combine over n_slots partial slots laid out as the
// first phase writes them.
hipError_t launch_decode_combine(const void* ws, int B, int H, int G, int n_slots, float* out, hipStream_t st) {
  const int BH = B * H;
  const float* part_ml = (const float*)ws;
  const float* part_o = (const float*)((const uint8_t*)ws + ml_bytes(BH, n_slots, G));
  return launch_combine(part_ml, part_o, out, BH, H, G, n_slots, st);
}

size_t decode_partials_bytes(int BH, int G, int n_slots) {
  return ml_bytes(BH, n_slots, G) + (size_t)BH * n_slots * G * 128 * 4;
}

// Decode over the tokens of two caches of the same streams (each cache's
// chunks in its own range of partial slots: cache a's chunks first), then one
// combine over all slots.  Plans capped at KVQ_SPLIT_MAX_CHUNKS chunks each,
// so the combine sees at most 128 slots.
hipError_t launch_decode_split(const Geo& ga, const Geo& gb, const void* q, int G, float scale, float* out,
                               void* ws, hipStream_t st) {
  const int BH = ga.B * ga.H;
  const float sl2 = scale * 1.4426950408889634f;
  const Geo* gs[2] = {&ga, &gb};
  DecodePlan ps[2];
  int n_slots = 0;
  for (int i = 0; i < 2; i++) {
    ps[i].n_chunks = 0;
    if (gs[i]->n_tiles > 0)
      ps[i] = decode_plan(BH, G, gs[i]->k_bits, gs[i]->v_bits, gs[i]->pdt, gs[i]->n_tiles, KVQ_SPLIT_MAX_CHUNKS);
    n_slots += ps[i].n_chunks;
  }
  if (n_slots < 1 || n_slots > KVQ_MAX_SLOTS) return hipErrorInvalidValue;
  float* part_ml = (float*)ws;
  float* part_o = (float*)((uint8_t*)part_ml + ml_bytes(BH, n_slots, G));
  int slot0 = 0;
  for (int i = 0; i < 2; i++) {
    if (ps[i].n_chunks == 0) continue;
    DecodeArgs a;
    a.g = *gs[i];
    a.q = (const uint16_t*)q;
    a.out = out;
    a.part_ml = part_ml;
    a.part_o = part_o;
    a.G = G;
    a.sl2 = sl2;
    a.n_chunks = a.tpc = a.n_groups = 0;
    a.n_slots = n_slots;
    a.slot0 = slot0;
    a.res = ResArgs{};
    a.res.R = 0;
    a.res_dtype = KVQ_F32;
    a.n_res = 0;
    hipError_t e = launch_decode_any(a, ps[i], st);
    if (e != hipSuccess) return e;
    slot0 += ps[i].n_chunks;
  }
  if (n_slots > 1) return launch_combine(part_ml, part_o, out, BH, ga.H, G, n_slots, st);
  return hipSuccess;
}

size_t decode_split_workspace_bytes(int B, int H, int G) {
  DecodePlan p;
  p.n_chunks = 2 * KVQ_SPLIT_MAX_CHUNKS - KVQ_MAX_RES_SLOTS;   // the bound adds the residual slots
  return decode_workspace_needed(B * H, G, p);
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free decode: the chunk partials that a caller's
// workspace holds otherwise, in a file-scope device array (one copy per GPU,
// kept until the process ends).  Host code never passes the array's name to
// a kernel: its device address comes from hipGetSymbolAddress, once per
// device, with that device current.
// ---------------------------------------------------------------------------
static __device__ __attribute__((aligned(256))) uint8_t scratch[KVQ_DECODE_SCRATCH_BYTES];

namespace {
constexpr int SCRATCH_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[SCRATCH_DEVICES];   // device address of each GPU's copy of `scratch`
}  // namespace

hipError_t decode_scratch_acquire(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= SCRATCH_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = p;
  }
  *ptr = scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace kvq
