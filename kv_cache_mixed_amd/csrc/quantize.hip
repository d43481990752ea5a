// quantize.hip -- quantize-and-pack kernels for one or more 128-token tiles.
//
// Keys are quantized channel-wise (one group = one channel, or one slot of the
// mixed layout, over the 128 tokens of a tile), values token-wise (one group =
// the 128 channels of one token), following the key-channel / value-token
// convention described on the ChanMix page (Background, Overall framework).
// The quantizer is the asymmetric uniform one of the ChanMix page (Key design 1:
// S = (max - min) / (2^b - 1), zero point = min) with parameters narrowed to
// the stored dtype before the codes are computed from them.
//
// Bit-exactness: every step is one IEEE binary32 operation (no contraction),
// division is correctly rounded (HIP default) -- the code quotient is formed
// with a reciprocal and re-done by division wherever that could round
// differently (quant_code) --, rounding of the quotient is round-half-even
// (v_rndne_f32), narrowing rounds to nearest even (binary16: v_cvt_f16_f32
// with denormals kept; bfloat16 and e4m3: on the bit pattern).
//
// One workgroup (256 threads) per (tile, kv head, batch).  The input tile is
// read once with coalesced loads; key codes are staged in LDS as uint16 and
// written as packed rows with coalesced 32-bit stores, value codes are packed
// into words in registers and written through LDS as 16-byte stores.
#pragma clang fp contract(off)

#include "kvq_device.h"

namespace kvq {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int IN>  // KVQ_F32 or KVQ_BF16
__device__ __forceinline__ float load_in(const void* p, int64_t i) {
  if constexpr (IN == KVQ_F32) return __builtin_nontemporal_load((const float*)p + i);
  else return bf16_bits_to_f32(((const uint16_t*)p)[i]);
}

// Codes of N members of one group given the stored (narrowed) S', Z'.
//
// A code is rint(fl32(d / S')), d = fl32(x - Z'), clamped to [0, levels].  It
// is formed from r = d * rsp, rsp = v_rcp_f32(S') (within 1 ulp of 1/S'): r is
// within |d/S'| * 2^-22 of fl32(d / S') (one ulp of the reciprocal, one
// rounding of the product, one of the division), so both round to the same
// integer unless r lies within that distance of a half-integer.  When any
// lane of the wave has a member with r within |r| * 2^-19 of a half-integer
// (or r not finite, or S' so large that its reciprocal is subnormal), the
// wave redoes the N quotients with the correctly rounded division -- members
// away from a half-integer get the same codes either way.  Widths above
// 8 bits (quotients up to 65535, where that window would catch a large share)
// always divide.  S' = 0 gives code 0.
template <bool FAST, int N>
__device__ __forceinline__ void quant_codes(const float* x, float sp, float zp, float levels, uint32_t* q) {
  float d[N], rr[N];
  bool redo = !FAST;
#pragma unroll
  for (int k = 0; k < N; k++) d[k] = x[k] - zp;
  if constexpr (FAST) {
    const float rsp = __builtin_amdgcn_rcpf(sp);
    bool near = !(sp < 0x1p125f);
#pragma unroll
    for (int k = 0; k < N; k++) {
      const float r = d[k] * rsp;
      rr[k] = __builtin_rintf(r);
      // distance of r from its nearest half-integer: 0.5 - |r - rint(r)|
      near |= !(__builtin_fabsf(r - rr[k]) < __builtin_fmaf(__builtin_fabsf(r), -0x1p-19f, 0.5f));
    }
    redo = __builtin_amdgcn_ballot_w64(near && sp != 0.0f) != 0;
  }
  if (redo) {
#pragma unroll
    for (int k = 0; k < N; k++) rr[k] = __builtin_rintf(d[k] / sp);
  }
#pragma unroll
  for (int k = 0; k < N; k++) {
    float c = rr[k] > 0.0f ? rr[k] : 0.0f;   // also maps NaN to 0
    c = c < levels ? c : levels;
    q[k] = sp == 0.0f ? 0u : (uint32_t)c;
  }
}

// Pack codes[row][elem] (LDS, uint16, row pitch PITCH) into 128 rows of
// 16*BITS bytes; each thread writes whole 32-bit words.
template <int BITS, int PITCH = 128>
__device__ __forceinline__ void pack_rows_store(const uint16_t* codes, uint8_t* tile) {
  constexpr int WORDS_PER_ROW = 4 * BITS;        // 16*BITS bytes
  constexpr int PER_WORD = 32 / BITS;            // codes in one 32-bit word (BITS<=16)
  uint32_t* out = (uint32_t*)tile;
  for (int w = threadIdx.x; w < 128 * WORDS_PER_ROW; w += blockDim.x) {
    int row = w / WORDS_PER_ROW;
    int e0 = (w % WORDS_PER_ROW) * PER_WORD;
    const uint16_t* src = codes + row * PITCH + e0;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < PER_WORD; i++) word |= (uint32_t)src[i] << (i * BITS);
    out[w] = word;
  }
}

// Logical byte b (0..33) of a token's mixed row from its slot codes:
// bytes 0..3 hold 4-bit pairs (slots 2b, 2b+1), bytes 4..7 (3,1,3,1)
// groups (slots 8+4m .. 11+4m), bytes 8..33 2-bit quads (slots 24+4m ..).
__device__ __forceinline__ uint32_t mixed_logical_byte(const uint16_t* c, int b) {
  if (b < 4) return (uint32_t)c[2 * b] | ((uint32_t)c[2 * b + 1] << 4);
  if (b < 8) {
    const uint16_t* p = c + 8 + 4 * (b - 4);
    return (uint32_t)p[0] | ((uint32_t)p[1] << 3) | ((uint32_t)p[2] << 4) | ((uint32_t)p[3] << 7);
  }
  const uint16_t* p = c + 24 + 4 * (b - 8);
  return (uint32_t)p[0] | ((uint32_t)p[1] << 2) | ((uint32_t)p[2] << 4) | ((uint32_t)p[3] << 6);
}

// Mixed key tile: codes[t][slot]; five planes (see include/kvq.h): plane g
// holds logical bytes g, 4+g, 8+6g .. 13+6g, plane 4 bytes 32, 33.
__device__ __forceinline__ void pack_mixed_store(const uint16_t* codes, uint8_t* tile) {
  // planes 0..3: 8 bytes per token = 2 words; 1024 words in total
  uint32_t* out = (uint32_t*)tile;
  for (int w = threadIdx.x; w < 1024; w += blockDim.x) {
    const int plane = w >> 8, t = (w >> 1) & 127, half = w & 1;
    const uint16_t* c = codes + t * 128;
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const int i = 4 * half + k;                                   // byte of the plane row
      const int b = i == 0 ? plane : (i == 1 ? 4 + plane : 8 + 6 * plane + (i - 2));
      word |= mixed_logical_byte(c, b) << (8 * k);
    }
    out[w] = word;
  }
  // plane 4: logical bytes 32..33 = slots 120..127, 2 bytes per token
  uint16_t* out4 = (uint16_t*)(tile + 4096);
  for (int t = threadIdx.x; t < 128; t += blockDim.x) {
    const uint16_t* c = codes + t * 128 + 120;
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) v |= (uint32_t)c[i] << (2 * i);
    out4[t] = (uint16_t)v;
  }
}

// ---------------------------------------------------------------------------
// Keys: thread (slot j = tid & 127, half = tid >> 7) scans 64 tokens.
// KB = 0 selects the mixed layout (slot j holds channel slot_chan[h][j]).
// ---------------------------------------------------------------------------
// Gathered tokens (GATHER): new token t of stream (b, h) is input row
// tok[(b * H + h) * n_new + t], clamped to [0, n_src).
struct TokIdx {
  const int32_t* tok;
  int n_new, n_src;
};
__device__ __forceinline__ int64_t src_row(const TokIdx& ti, int b, int h, int H, int t) {
  int r = ti.tok[((int64_t)b * H + h) * ti.n_new + t];
  r = r < 0 ? 0 : (r >= ti.n_src ? ti.n_src - 1 : r);
  return r;
}

template <int KB, int PDT, int IN, bool GATHER>
__global__ __launch_bounds__(256) void quantize_k_kernel(Geo g, const void* __restrict__ kin,
                                                         int64_t sb, int64_t sh, int64_t st,
                                                         int t0, TokIdx ti) {
  __shared__ uint16_t codes[128 * 128];
  __shared__ float red_mn[2][128], red_mx[2][128];
  __shared__ int64_t rows[GATHER ? 128 : 1];
  __shared__ uint8_t slot_of[KB == 0 ? 128 : 1];
  const int tile_local = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tile = t0 / 128 + tile_local;
  // thread (j, half) reads channel j, so a wave's loads cover whole rows
  // whatever the slot map; mixed keys quantize channel j as the slot the map
  // gives it (the inverse of slot -> channel, built in LDS; entries are used
  // through their low 7 bits, so a map that is not a permutation leaves some
  // slots unspecified but every access inside the tile and its parameters)
  const int j = threadIdx.x & 127, half = threadIdx.x >> 7;
  const int chan = j;

  float x[64];
  if constexpr (GATHER) {
    if (threadIdx.x < 128) rows[threadIdx.x] = src_row(ti, b, h, g.H, tile_local * 128 + threadIdx.x) * st;
    __syncthreads();
    const int64_t base = (int64_t)b * sb + (int64_t)h * sh + chan;
#pragma unroll
    for (int i = 0; i < 64; i++) x[i] = load_in<IN>(kin, base + rows[half * 64 + i]);
  } else {
    const int64_t base = (int64_t)b * sb + (int64_t)h * sh + (int64_t)(tile_local * 128) * st + chan;
#pragma unroll
    for (int i = 0; i < 64; i++) x[i] = load_in<IN>(kin, base + (int64_t)(half * 64 + i) * st);
  }
  // (the slot map is read while the tile's loads are in flight)
  int slot = j;
  if constexpr (KB == 0) {
    if (threadIdx.x < 128) slot_of[(int)g.slot_chan[h * 128 + threadIdx.x] & 127] = (uint8_t)threadIdx.x;
    __syncthreads();
    slot = slot_of[j] & 127;
  }
  const int bits = (KB == 0) ? mixed_slot_bits(slot) : KB;
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int i = 1; i < 64; i++) {
    mn = x[i] < mn ? x[i] : mn;
    mx = x[i] > mx ? x[i] : mx;
  }
  red_mn[half][j] = mn;
  red_mx[half][j] = mx;
  __syncthreads();
  mn = red_mn[0][j] < red_mn[1][j] ? red_mn[0][j] : red_mn[1][j];
  mx = red_mx[0][j] > red_mx[1][j] ? red_mx[0][j] : red_mx[1][j];
  mn = mn + 0.0f;   // -0 and +0 are one value: keep +0 whatever the reduction order
  mx = mx + 0.0f;
  const float levels = (float)((1u << bits) - 1u);
  const float s = (mx - mn) / levels;
  const float sp = Param<PDT>::narrow(s);
  const float zp = Param<PDT>::narrow(mn);
  if (half == 0) {
    const int64_t pi = k_param_base(g, b, h, tile) + slot;
    Param<PDT>::store(g.k_scale, pi, s);
    Param<PDT>::store(g.k_zero, pi, mn);
  }
#pragma unroll
  for (int i = 0; i < 64; i += 8) {
    uint32_t q[8];
    quant_codes<KB <= 8, 8>(&x[i], sp, zp, levels, q);
#pragma unroll
    for (int k = 0; k < 8; k++) codes[(half * 64 + i + k) * 128 + slot] = (uint16_t)q[k];
  }
  __syncthreads();
  uint8_t* dst = g.k_codes + k_tile_offset(g, b, h, tile);
  if constexpr (KB == 0) pack_mixed_store(codes, dst);
  else pack_rows_store<KB>(codes, dst);
}

// ---------------------------------------------------------------------------
// Values: wave a handles tokens [32a, 32a+32) of the tile.  Row r of the wave
// (16 lanes) takes tokens 32a + 8r + i, i = 0..7, one per step; lane j of the
// row holds channels 4j..4j+3 and 64+4j..64+4j+3 of it, so one load
// instruction covers four whole token rows, and all 16 loads of a lane are
// issued before any reduction.  The min/max of a token is a reduction inside
// its row (four DPP steps).  Each lane packs the codes of its 8 channels for
// the row's 8 tokens into value words in registers: a row fills whole words
// at b >= 4; at b = 2 (1) two (four) rows share a word and are merged by lane
// swaps.  The finished words pass through LDS only to leave as 16-byte stores
// in tile order.  VEC: the input allows 16-byte (F32) / 8-byte (BF16) loads
// of 4 channels.
// ---------------------------------------------------------------------------
// min / max over each 16-lane row of the wave, result in every lane:
// quad_perm xor 1 and xor 2, row_half_mirror, row_mirror (DPP, fused into the
// min / max)
template <bool MAX>
__device__ __forceinline__ float row_reduce(float v) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : fminf(a, b); };
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));
  v = op(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)));
  return v;
}

template <int IN, bool VEC>
__device__ __forceinline__ void load4(const void* p, int64_t i, float* x) {
  if constexpr (VEC && IN == KVQ_F32) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    const f4 v = __builtin_nontemporal_load((const f4*)((const float*)p + i));
    x[0] = v[0]; x[1] = v[1]; x[2] = v[2]; x[3] = v[3];
  } else if constexpr (VEC && IN == KVQ_BF16) {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    const u2 v = *(const u2*)((const uint16_t*)p + i);
    x[0] = bf16_bits_to_f32(v[0] & 0xffffu); x[1] = bf16_bits_to_f32(v[0] >> 16);
    x[2] = bf16_bits_to_f32(v[1] & 0xffffu); x[3] = bf16_bits_to_f32(v[1] >> 16);
  } else {
#pragma unroll
    for (int k = 0; k < 4; k++) x[k] = load_in<IN>(p, i + k);
  }
}

template <int VB, int PDT, int IN, bool VEC, bool GATHER>
__global__ __launch_bounds__(256) void quantize_v_kernel(Geo g, const void* __restrict__ vin,
                                                         int64_t sb, int64_t sh, int64_t st,
                                                         int t0, TokIdx ti) {
  // word W[w][c][a] holds channel c of the tokens 32a + w*PW + i (i < PW,
  // code i at bits [i*VB, (i+1)*VB)); token 32a + 8r + i (step i of row r)
  // lands in word (8r + i) / PW at slot (8r + i) % PW
  constexpr int PW = 32 / VB;                    // codes per word
  constexpr int RW = (8 * VB + 31) / 32;         // words per channel a row fills (one when shared)
  const int tile_local = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tile = t0 / 128 + tile_local;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = lane >> 4, j = lane & 15;
  const float levels = (float)((1u << VB) - 1u);
  const int64_t base = (int64_t)b * sb + (int64_t)h * sh + (GATHER ? 0 : (int64_t)(tile_local * 128) * st) + 4 * j;
  float x[8][8];   // [step][channel slot k: channel 64 * (k / 4) + 4j + k % 4]
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int t = wave * 32 + 8 * row + i;
    const int64_t r = GATHER ? src_row(ti, b, h, g.H, tile_local * 128 + t) : (int64_t)t;
    load4<IN, VEC>(vin, base + r * st, &x[i][0]);
    load4<IN, VEC>(vin, base + r * st + 64, &x[i][4]);
  }
  uint32_t wd[8][RW];
#pragma unroll
  for (int k = 0; k < 8; k++)
#pragma unroll
    for (int w = 0; w < RW; w++) wd[k][w] = 0u;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int t = wave * 32 + 8 * row + i;
    float mn = x[i][0], mx = x[i][0];
#pragma unroll
    for (int k = 1; k < 8; k++) {
      mn = fminf(mn, x[i][k]);
      mx = fmaxf(mx, x[i][k]);
    }
    mn = row_reduce<false>(mn);
    mx = row_reduce<true>(mx);
    mn = mn + 0.0f;   // -0 and +0 are one value: keep +0 whatever the reduction order
    mx = mx + 0.0f;
    const float s = (mx - mn) / levels;
    const float sp = Param<PDT>::narrow(s);
    const float zp = Param<PDT>::narrow(mn);
    if (j == 0) {
      const int64_t pi = v_param_base(g, b, h, (int64_t)tile * 128 + t);
      Param<PDT>::store(g.v_scale, pi, s);
      Param<PDT>::store(g.v_zero, pi, mn);
    }
    // word of the row (b >= 4: i / PW; shared words: the row's part of word 0)
    const int lw = (VB >= 4) ? i / PW : 0;
    const uint32_t sh = (VB >= 4) ? (uint32_t)((i % PW) * VB) : (uint32_t)(((8 * row + i) % PW) * VB);
    uint32_t qc[8];
    quant_codes<VB <= 8, 8>(x[i], sp, zp, levels, qc);
#pragma unroll
    for (int k = 0; k < 8; k++) wd[k][lw] |= qc[k] << sh;
  }
  // rows sharing a word: merge rows (0, 1) and (2, 3), then (0-1, 2-3)
  if constexpr (VB <= 2) {
#pragma unroll
    for (int k = 0; k < 8; k++) {
      uint32_t r0, r1;
      lane_swap16(wd[k][0], r0, r1);
      wd[k][0] = r0 | r1;
      if constexpr (VB == 1) {
        lane_swap32(wd[k][0], r0, r1);
        wd[k][0] = r0 | r1;
      }
    }
  }
  const bool writer = (VB >= 4) || (VB == 2 ? (row & 1) == 0 : row == 0);
  // the words go to LDS at their tile positions, then out with 16-byte
  // stores that cover the tile in order (storing each word from its register
  // scatters a wave's stores over the tile: 4.5% slower at 4 and 2 bits)
  constexpr int TW = 32 * VB * 16;   // words per tile (2048 * VB bytes / 4)
  __shared__ __attribute__((aligned(16))) uint32_t tw[TW];
  if (writer) {
#pragma unroll
    for (int k = 0; k < 8; k++) {
      // channel c = 64 hh + 16 q + n
      const int hh = k >> 2, q = j >> 2, n = 4 * (j & 3) + (k & 3);
#pragma unroll
      for (int lw = 0; lw < RW; lw++) {
        const int w = (VB >= 4) ? (8 * row) / PW + lw : (8 * row) / PW;
        tw[w * 512 + ((hh * 16 + n) * 4 + wave) * 4 + q] = wd[k][lw];
      }
    }
  }
  __syncthreads();
  {
    uint32_t* out = (uint32_t*)(g.v_codes + v_tile_offset(g, b, h, tile));
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int o = threadIdx.x * 4; o < TW; o += 1024) *(u4*)(out + o) = *(const u4*)(tw + o);
  }
}

// ---------------------------------------------------------------------------
// Values with mixed channel widths: for every token, the slots of each width
// class (4, 3, 1, 2 bits; slot j holds channel v_slot_chan[h][j]) form one
// group with its own S', Z'.  Every thread issues its loads of the whole tile
// first (16 x 16 bytes); the inputs then pass through LDS in two halves of
// 64 tokens (binary32, row pitch 129 words, so a wave reading one channel of
// 64 tokens hits 32 banks).  Wave w quantizes slot blocks w and
// w + 4 (16 slots each; the block's class, and so its width, is uniform over
// the wave) of the half's 64 tokens, one token per lane: block minima and
// maxima go through LDS so the five blocks of the 2-bit class share one
// group.  Codes are staged as bytes [slot][token] and packed into the tile's
// 32-bit words at the end, one word per thread and step, in tile order.
// ---------------------------------------------------------------------------
template <int PDT, int IN, bool VEC, bool GATHER>
__global__ __launch_bounds__(256) void quantize_vmixed_kernel(Geo g, const void* __restrict__ vin,
                                                              int64_t sb, int64_t sh, int64_t st,
                                                              int t0, TokIdx ti) {
  __shared__ float xs[64][129];
  __shared__ __attribute__((aligned(16))) uint8_t codes[128][128];   // [slot][token]
  __shared__ float bmn[8][64], bmx[8][64];                            // [block][token]
  const int tile_local = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tile = t0 / 128 + tile_local;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), r = threadIdx.x & 63;
  const int64_t base = (int64_t)b * sb + (int64_t)h * sh + (GATHER ? 0 : (int64_t)(tile_local * 128) * st);
  // item i of half hf = token row 64 hf + i / 32, channels 4 (i % 32) ..
  float xin[2][8][4];
#pragma unroll
  for (int hf = 0; hf < 2; hf++)
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const int i = threadIdx.x + 256 * k;
      const int t = hf * 64 + (i >> 5);
      const int64_t row = GATHER ? src_row(ti, b, h, g.H, tile_local * 128 + t) : (int64_t)t;
      load4<IN, VEC>(vin, base + row * st + (i & 31) * 4, xin[hf][k]);
    }
  // the channels of the wave's two slot blocks (the same for every lane:
  // scalar registers)
  int chan[2][16];
#pragma unroll
  for (int u = 0; u < 2; u++)
#pragma unroll
    for (int j = 0; j < 16; j++) chan[u][j] = (int)g.v_slot_chan[h * 128 + 16 * (wave + 4 * u) + j] & 127;
#pragma unroll
  for (int half = 0; half < 2; half++) {
#pragma unroll
    for (int k = 0; k < 8; k++) {
      const int i = threadIdx.x + 256 * k;
      const int tr = i >> 5, c4 = (i & 31) * 4;
#pragma unroll
      for (int e = 0; e < 4; e++) xs[tr][c4 + e] = xin[half][k][e];
    }
    __syncthreads();
    float x[2][16];
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int m = wave + 4 * u;
      float mn, mx;
#pragma unroll
      for (int j = 0; j < 16; j++) {
        x[u][j] = xs[r][chan[u][j]];
        mn = j ? fminf(mn, x[u][j]) : x[u][j];
        mx = j ? fmaxf(mx, x[u][j]) : x[u][j];
      }
      bmn[m][r] = mn;
      bmx[m][r] = mx;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int m = wave + 4 * u;
      const int k = vmixed_block_class(m);
      float mn = bmn[m][r], mx = bmx[m][r];
      if (k == 3) {
#pragma unroll
        for (int m2 = 3; m2 < 8; m2++) {
          mn = fminf(mn, bmn[m2][r]);
          mx = fmaxf(mx, bmx[m2][r]);
        }
      }
      mn = mn + 0.0f;   // -0 and +0 are one value: keep +0 whatever the reduction order
      mx = mx + 0.0f;
      const float levels = (float)((1u << vmixed_class_bits(k)) - 1u);
      const float s = (mx - mn) / levels;
      const float sp = Param<PDT>::narrow(s);
      const float zp = Param<PDT>::narrow(mn);
      if (m < 4) {   // the class's first block stores its parameters
        const int64_t pi = vm_param_index(g, b, h, k, (int64_t)tile * 128 + half * 64 + r);
        Param<PDT>::store(g.v_scale, pi, s);
        Param<PDT>::store(g.v_zero, pi, mn);
      }
#pragma unroll
      for (int j = 0; j < 16; j += 8) {
        uint32_t q[8];
        quant_codes<true, 8>(&x[u][j], sp, zp, levels, q);
#pragma unroll
        for (int e = 0; e < 8; e++) codes[16 * m + j + e][half * 64 + r] = (uint8_t)q[e];
      }
    }
    __syncthreads();   // xs and the block extremes are reused by the next half
  }
  // word wi of the tile: block m, inside it word (w * 16 + n) * 4 + a holds
  // slot 16m + n for the 32/f tokens 32a + w * (32/f) + i, code i at bits
  // [i*f, i*f + f)
  uint32_t* out = (uint32_t*)(g.v_codes + v_tile_offset(g, b, h, tile));
#pragma unroll
  for (int k = 0; k < 5; k++) {
    const int wi = threadIdx.x + 256 * k;
    const bool wide = wi < 512;
    const int m = wide ? (wi >> 8) : 2 + ((wi - 512) >> 7);
    const int li = wide ? (wi & 255) : ((wi - 512) & 127);
    const int a = li & 3, n = (li >> 2) & 15, w = li >> 6;
    const uint8_t* src = &codes[16 * m + n][0];
    uint32_t word = 0;
    if (wide) {
      const u32x2 c = *(const u32x2*)(src + 32 * a + 8 * w);
#pragma unroll
      for (int i = 0; i < 8; i++) word |= ((c[i / 4] >> (8 * (i % 4))) & 0xFu) << (4 * i);
    } else {
      const u32x4 c = *(const u32x4*)(src + 32 * a + 16 * w);
#pragma unroll
      for (int i = 0; i < 16; i++) word |= ((c[i / 4] >> (8 * (i % 4))) & 0x3u) << (2 * i);
    }
    out[wi] = word;
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
template <int PDT, int IN>
static hipError_t launch_k(const Geo& g, const void* k, const int64_t* s, int t0, int n_new,
                           const TokIdx& ti, hipStream_t stm) {
  dim3 grid(n_new / 128, g.H, g.B), block(256);
#define KVQ_QK(KBV)                                                                            \
  case KBV:                                                                                    \
    if (ti.tok)                                                                                \
      hipLaunchKernelGGL((quantize_k_kernel<KBV, PDT, IN, true>), grid, block, 0, stm, g, k,   \
                         s[0], s[1], s[2], t0, ti);                                            \
    else                                                                                       \
      hipLaunchKernelGGL((quantize_k_kernel<KBV, PDT, IN, false>), grid, block, 0, stm, g, k,  \
                         s[0], s[1], s[2], t0, ti);                                            \
    break;
  switch (g.k_bits) {
    KVQ_QK(0) KVQ_QK(1) KVQ_QK(2) KVQ_QK(4) KVQ_QK(8) KVQ_QK(16)
    default: return hipErrorInvalidValue;
  }
#undef KVQ_QK
  return hipGetLastError();
}

template <int PDT, int IN>
static hipError_t launch_v(const Geo& g, const void* v, const int64_t* s, int t0, int n_new,
                           const TokIdx& ti, hipStream_t stm) {
  dim3 grid(n_new / 128, g.H, g.B), block(256);
  const int eb = (IN == KVQ_F32) ? 4 : 2;
  const bool vec = ((uintptr_t)v % (4 * eb) == 0) && (s[0] % 4 == 0) && (s[1] % 4 == 0) &&
                   (s[2] % 4 == 0);
#define KVQ_QV(VBV)                                                                                   \
  case VBV:                                                                                           \
    if (ti.tok)                                                                                       \
      hipLaunchKernelGGL((quantize_v_kernel<VBV, PDT, IN, false, true>), grid, block, 0, stm, g, v,   \
                         s[0], s[1], s[2], t0, ti);                                                   \
    else if (vec)                                                                                     \
      hipLaunchKernelGGL((quantize_v_kernel<VBV, PDT, IN, true, false>), grid, block, 0, stm, g, v,   \
                         s[0], s[1], s[2], t0, ti);                                                   \
    else                                                                                              \
      hipLaunchKernelGGL((quantize_v_kernel<VBV, PDT, IN, false, false>), grid, block, 0, stm, g, v,  \
                         s[0], s[1], s[2], t0, ti);                                                   \
    break;
  switch (g.v_bits) {
    case 0:
      if (ti.tok)
        hipLaunchKernelGGL((quantize_vmixed_kernel<PDT, IN, false, true>), grid, block, 0, stm, g, v, s[0], s[1],
                           s[2], t0, ti);
      else if (vec)
        hipLaunchKernelGGL((quantize_vmixed_kernel<PDT, IN, true, false>), grid, block, 0, stm, g, v, s[0], s[1],
                           s[2], t0, ti);
      else
        hipLaunchKernelGGL((quantize_vmixed_kernel<PDT, IN, false, false>), grid, block, 0, stm, g, v, s[0], s[1],
                           s[2], t0, ti);
      break;
    KVQ_QV(1) KVQ_QV(2) KVQ_QV(4) KVQ_QV(8) KVQ_QV(16)
    default: return hipErrorInvalidValue;
  }
#undef KVQ_QV
  return hipGetLastError();
}

template <int PDT>
static hipError_t launch_pdt(const Geo& g, const void* k, const void* v, int in_dtype,
                             const int64_t* ks, const int64_t* vs, int t0, int n_new,
                             const TokIdx& ti, hipStream_t st) {
  hipError_t e = hipSuccess;
  if (in_dtype == KVQ_F32) {
    if (k) e = launch_k<PDT, KVQ_F32>(g, k, ks, t0, n_new, ti, st);
    if (e == hipSuccess && v) e = launch_v<PDT, KVQ_F32>(g, v, vs, t0, n_new, ti, st);
  } else {
    if (k) e = launch_k<PDT, KVQ_BF16>(g, k, ks, t0, n_new, ti, st);
    if (e == hipSuccess && v) e = launch_v<PDT, KVQ_BF16>(g, v, vs, t0, n_new, ti, st);
  }
  return e;
}

hipError_t launch_quantize(const Geo& g, const void* k, const void* v, int in_dtype,
                           const int64_t* ks, const int64_t* vs, int t0, int n_new,
                           hipStream_t st, const int32_t* tok, int n_src) {
  TokIdx ti;
  ti.tok = tok;
  ti.n_new = n_new;
  ti.n_src = n_src;
  switch (g.pdt) {
    case KVQ_F32: return launch_pdt<KVQ_F32>(g, k, v, in_dtype, ks, vs, t0, n_new, ti, st);
    case KVQ_F16: return launch_pdt<KVQ_F16>(g, k, v, in_dtype, ks, vs, t0, n_new, ti, st);
    case KVQ_BF16: return launch_pdt<KVQ_BF16>(g, k, v, in_dtype, ks, vs, t0, n_new, ti, st);
    case KVQ_E4M3: return launch_pdt<KVQ_E4M3>(g, k, v, in_dtype, ks, vs, t0, n_new, ti, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kvq
