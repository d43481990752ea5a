/*
 * kvq.h -- C ABI of libkvq: low-bit, mixed-precision KV-cache quantization,
 * the Equivalent Right Shift bit-width shrink, and decode attention over the
 * packed cache, for AMD Instinct MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [PMKVQ]   "PM-KVQ: Progressive Mixed-Precision KV Cache Quantization for
 *              Long-CoT LLMs" (papernotes.org summary).
 *   [CHANMIX] "Channel-Aware Mixed-Precision Quantization for Efficient
 *              Long-Context Inference" (papernotes.org summary).
 *   [PNMIX]   "PN-Mix: Pair-Norm Guided Mixed-Precision Key Cache
 *              Quantization" (shd-paper.top summary, abstract).
 *   [SEMKV]   "SemKV: Semantic Mixed-Precision KV Cache Quantization Guided
 *              by the Quality Cliff for Long-Context LLM Inference"
 *              (paperdance.org, abstract).
 *
 * ------------------------------------------------------------------------
 * Conventions
 *   - Every buffer is owned by the caller.  Pointers named "device" are HIP
 *     device memory; the library never allocates or frees device memory.
 *   - The kvq_cache struct is host memory and is read during the call only;
 *     kvq_quantize, kvq_shrink, kvq_append and kvq_window_append update its
 *     n_tokens / k_bits / v_bits fields (and the window's counts) as
 *     documented.
 *   - All device work is enqueued on the given stream; calls return before it
 *     completes.  Every argument is validated on the host first: any status
 *     other than KVQ_OK / KVQ_EHIP means no device work was enqueued.
 *     KVQ_EHIP means a HIP call failed (work already enqueued may be partial).
 *   - No exceptions cross the ABI.  The library holds no global mutable
 *     state; calls on different caches are independent.  Calls that touch the
 *     same cache or workspace must be ordered by the caller (same stream).
 *
 * ------------------------------------------------------------------------
 * The quantizer ([CHANMIX] Key design 1; [PMKVQ] Training strategy)
 *   A group is a set of real values x.  With mn = min x, mx = max x (a zero
 *   extreme is +0 whatever the signs of the zeros in the group):
 *     S  = (mx - mn) / (2^b - 1)      (binary32: one subtraction, one division)
 *     S' = narrow(S),  Z' = narrow(mn)   (round to nearest even to the
 *                                         parameter dtype; e4m3 saturates)
 *     q  = clamp(rne((x - Z') / S'), 0, 2^b - 1)   (binary32), or 0 if S' == 0
 *   and the reconstruction is x^ = S' * q + Z'.  Inputs must be finite and
 *   small enough that S' and Z' are finite in the parameter dtype.
 *   Keys are grouped channel-wise: one group = one channel (slot) over one
 *   128-token tile.  Values are grouped token-wise: one group = the 128
 *   channels of one token, or for mixed values the channels of one width
 *   class of one token ([CHANMIX] Background; [PMKVQ] related work on KIVI).
 *   Bit widths: 16, 8, 4, 2, 1 ("16-bit" is an integer code, not fp16).
 *
 * Equivalent Right Shift ([PMKVQ] Key design 1, ERS equation), per code:
 *     X_b = ((2^(2b) - 2^b + 1) * (X_2b + 2^(b-1))) >> 3b   (unsigned 32-bit)
 *     Z'_b = Z'_2b,   S'_b = narrow((2^b + 1) * S'_2b)       (binary32 product)
 *
 * ------------------------------------------------------------------------
 * Packed layouts
 *   Tokens of a (batch b, kv head h) stream are cut into tiles of 128 tokens;
 *   tile g holds tokens [128g, 128g + 128).
 *
 *   Packed row: a little-endian bit string -- bit i of the row is bit (i mod 8)
 *   of byte (i div 8); element e of a b-bit row occupies bits [e*b, e*b + b),
 *   least significant code bit first.
 *
 *   Key tile, uniform width b (2048*b bytes): 128 rows of 16*b bytes; row t is
 *     token 128g + t, element c is channel c.
 *   Value tile, width b (2048*b bytes): 32-bit little-endian words W[w][c][a]
 *     for w in [0, b), c in [0, 128), a in [0, 4).  Word W[w][c][a] holds
 *     channel c of the 32/b tokens 128g + 32a + w*(32/b) + i,
 *     i = 0 .. 32/b - 1, code i at bits [i*b, i*b + b).  Writing
 *     c = 64h + 16q + n (h in [0, 2), q in [0, 4), n in [0, 16)), the word sits
 *     at word index w*512 + ((h*16 + n)*4 + a)*4 + q.  (Every channel's 128
 *     tokens are split into b word planes of 512 words; inside a plane, the
 *     four words of channels 16q + n, q = 0..3, for one token slice a are
 *     contiguous.)
 *   Key tile, mixed width (k_bits == KVQ_KMIXED, 4352 bytes) ([CHANMIX] Key
 *     design 3: 4/3/2/1-bit channel classes, as many 1-bit as 3-bit channels,
 *     channels reordered so every byte holds exactly 8 code bits):
 *     slot j of a token holds channel k_slot_chan[h][j]; slots 0..7 are 4-bit,
 *     slots 8..23 alternate 3-bit (even j) and 1-bit (odd j), slots 24..127 are
 *     2-bit.  A token's logical 34-byte row is the packed row of its 128 slot
 *     codes in slot order (widths as listed), so bytes 0..3 hold 4-bit pairs,
 *     bytes 4..7 hold (3,1,3,1)-bit groups, bytes 8..33 hold 2-bit quads.  The
 *     tile stores these rows as five column planes.  Plane g (g < 4) sits at
 *     tile offset 1024*g with 8 bytes per token: logical bytes g, 4+g,
 *     8+6g, 9+6g, 10+6g, 11+6g, 12+6g, 13+6g in that order (so every plane
 *     holds two 4-bit, two 3-bit, two 1-bit and 24 2-bit slots).  Plane 4
 *     sits at tile offset 4096 with 2 bytes per token: logical bytes 32, 33.
 *     Tokens are in order inside a plane.
 *
 *   Value tile, mixed width (v_bits == KVQ_VMIXED, 5120 bytes) (the [CHANMIX]
 *     Key design 3 channel classes read for values: token-wise groups, one
 *     per class of each token): slot j of a token holds channel
 *     v_slot_chan[h][j]; slots 0..15 are 4-bit, 16..31 3-bit, 32..47 1-bit,
 *     48..127 2-bit (class k = 0, 1, 2, 3 in that order; 2.25 code bits per
 *     value).  The tile is eight blocks of 16 slots, block m = slots
 *     16m .. 16m + 15, stored at byte 1024*m (m < 2) or 2048 + 512*(m - 2)
 *     (m >= 2).  Block m keeps its codes in fields of f = 4 bits (m < 2; the
 *     3-bit codes of block 1 in the field's low bits) or f = 2 bits (m >= 2;
 *     the 1-bit codes of block 2 in the field's low bit), so every code stays
 *     inside one 32-bit word: inside the block, 32-bit word
 *     (w * 16 + n) * 4 + a (w < f, n < 16, a < 4) holds slot 16m + n of the
 *     32/f tokens 128g + 32a + w*(32/f) + i, code i at bits [i*f, i*f + f).
 *
 *   Tile placement: tile g of stream (b, h) starts at
 *     k_codes + k_tile_off[(g * batch + b) * n_kv_heads + h]   if k_tile_off,
 *     k_codes + ((b * n_kv_heads + h) * max_tiles + g) * k_tile_stride   else,
 *   (same for values) with max_tiles = max_tokens / 128.  Offsets and strides
 *   are multiples of 256 bytes; a stride is at least the current tile size.
 *   kvq_shrink rewrites every tile in place: the narrower tile occupies the
 *   first half of the bytes the wider one used, at the same offset (key codes
 *   keep their order; value codes move to the word planes of the new width).
 *
 *   Parameters (S', Z' raw values of param_dtype):
 *     k_scale, k_zero: [batch][n_kv_heads][max_tiles][128]  (per tile, per slot;
 *                      for uniform keys slot j is channel j)
 *     v_scale, v_zero: [batch][n_kv_heads][max_tokens]       (per token), or
 *                      [batch][n_kv_heads][4][max_tokens]    (mixed values:
 *                      per class k and token, class-major)
 *
 * ------------------------------------------------------------------------
 * Decode attention ([CHANMIX] Overall framework and Key design 3: read the
 * packed cache, dequantize to full precision, FlashAttention-style decode)
 *   For batch b and query head hq, with G = n_q_heads / n_kv_heads and kv head
 *   h = hq / G (query heads of one kv head are contiguous):
 *     s_t = softmax_scale * sum_c q[b][hq][c] * K^[b][h][t][c],  t < n_tokens
 *     out[b][hq][c] = sum_t softmax(s)_t * V^[b][h][t][c]
 *   where K^, V^ are the reconstructions S' * q + Z' of the stored codes.
 *   q is bfloat16 [batch][n_q_heads][128]; out is float32, same shape.
 *   Widths decoded: k_bits == v_bits in {16, 8, 4, 2, 1}; mixed keys with
 *   4-, 2- or 1-bit values; mixed keys with mixed values when param_dtype
 *   is KVQ_E4M3 or KVQ_F16.  Other pairs return KVQ_EUNSUPPORTED.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVQ_OK = 0,
    KVQ_EINVAL = 1,        /* invalid argument (null pointer, bad size, bad width ...) */
    KVQ_EUNSUPPORTED = 2,  /* valid request the library does not implement */
    KVQ_EBUDGET = 3,       /* kvq_append / kvq_window_append / kvq_allocate_bits: the budget or the pool cannot hold it */
    KVQ_EWORKSPACE = 4,    /* workspace pointer null or smaller than required */
    KVQ_EHIP = 5           /* a HIP runtime call or kernel launch failed */
} kvq_status;

typedef enum {
    KVQ_F32 = 0,
    KVQ_F16 = 1,   /* IEEE binary16 */
    KVQ_BF16 = 2,  /* bfloat16 */
    KVQ_E4M3 = 3   /* OCP FP8 E4M3 (bias 7, max 448, no infinities), saturating */
} kvq_dtype;

#define KVQ_HEAD_DIM 128
#define KVQ_GROUP 128
#define KVQ_KMIXED 0          /* k_bits value selecting the mixed-width key tile */
#define KVQ_VMIXED 0          /* v_bits value selecting the mixed-width value tile */
/* Largest per-stream capacity (2^26 tokens): device offsets into the
 * per-stream parameter arrays are 32-bit. */
#define KVQ_MAX_TOKENS (1 << 26)
/* Most residual (unquantized) tokens one decode call attends per stream. */
#define KVQ_MAX_RESIDUAL 512
#define KVQ_MIXED_TILE_BYTES 4352
#define KVQ_VMIXED_TILE_BYTES 5120

typedef struct kvq_cache {
    int32_t batch;            /* B >= 1 */
    int32_t n_kv_heads;       /* Hkv >= 1 */
    int32_t head_dim;         /* must be 128 */
    int32_t group;            /* must be 128 */
    int32_t max_tokens;       /* capacity per stream, multiple of 128, <= KVQ_MAX_TOKENS */
    int32_t n_tokens;         /* tokens stored per stream, multiple of 128 */
    int32_t k_bits;           /* 16, 8, 4, 2, 1, or KVQ_KMIXED */
    int32_t v_bits;           /* 16, 8, 4, 2, 1, or KVQ_VMIXED */
    int32_t param_dtype;      /* kvq_dtype of S' and Z': F32, F16, BF16 or E4M3 */
    int32_t reserved0;        /* must be 0 */
    void *k_codes;            /* device: key tiles */
    void *v_codes;            /* device: value tiles */
    const int64_t *k_tile_off;  /* device [max_tiles][B][Hkv] byte offsets, or NULL */
    const int64_t *v_tile_off;  /* device [max_tiles][B][Hkv] byte offsets, or NULL */
    int64_t k_tile_stride;    /* bytes between tiles when k_tile_off is NULL */
    int64_t v_tile_stride;    /* bytes between tiles when v_tile_off is NULL */
    void *k_scale;            /* device [B][Hkv][max_tiles][128] */
    void *k_zero;             /* device [B][Hkv][max_tiles][128] */
    void *v_scale;            /* device [B][Hkv][max_tokens] ([B][Hkv][4][max_tokens] mixed) */
    void *v_zero;             /* device, as v_scale */
    const int16_t *k_slot_chan; /* device [Hkv][128]: channel held by slot j
                                   (mixed keys only, a permutation per head;
                                   the kernels use only its low 7 bits, so a
                                   map that is not a permutation gives wrong
                                   or unspecified codes for some slots but no
                                   access outside a row, a tile or its
                                   parameters) */
    const int16_t *v_slot_chan; /* device [Hkv][128]: channel held by value
                                   slot j (mixed values only; same rules) */
} kvq_cache;

/* Human-readable name of a status code (static string). */
const char *kvq_strerror(kvq_status status);

/* Bytes of one packed tile at width `bits` (KVQ_KMIXED: the mixed key tile);
 * 0 for an invalid width.  kvq_value_tile_bytes: the same for value tiles
 * (KVQ_VMIXED: the mixed value tile). */
size_t kvq_tile_bytes(int32_t bits);
size_t kvq_value_tile_bytes(int32_t bits);

/* Memory of a cache holding n_tokens tokens per stream at the given widths,
 * as the progressive schedule counts it ([PMKVQ] Key design 2: total KV
 * memory within the budget): key codes + value codes + every stored scale and
 * zero point, over all B * Hkv streams.  k_bits may be KVQ_KMIXED, v_bits
 * KVQ_VMIXED (four value scales and zero points per token).  Returns -1
 * for invalid arguments. */
int64_t kvq_cache_bytes(const kvq_cache *cache, int32_t n_tokens, int32_t k_bits, int32_t v_bits);

/* Quantize and pack tokens [t0, t0 + n_new) of every stream at the cache's
 * current widths (keys channel-wise per tile, values token-wise), writing the
 * tiles and their S', Z'.  k / v: device inputs of logical shape
 * [B][Hkv][n_new][128]; element (b, h, t, c) is at base + b*s[0] + h*s[1] +
 * t*s[2] + c (strides in elements, channel stride 1).  in_dtype: KVQ_F32 or
 * KVQ_BF16.  Either k or v may be NULL to skip that side.  t0 and n_new are
 * multiples of 128, n_new >= 128, t0 + n_new <= max_tokens.  On success
 * n_tokens becomes max(n_tokens, t0 + n_new). */
kvq_status kvq_quantize(kvq_cache *cache, const void *k, const void *v, kvq_dtype in_dtype,
                        const int64_t k_strides[3], const int64_t v_strides[3],
                        int32_t t0, int32_t n_new, hipStream_t stream);

/* kvq_quantize of gathered tokens ([SEMKV] abstract: every token is kept; the
 * tokens of a stream, ranked by a model-internal score, go to one of two
 * caches of adjacent precisions).  New token i of stream (b, h) is input row
 * r = tok[(b * n_kv_heads + h) * n_new + i] of that stream: element
 * (b, h, r, c) at base + b*s[0] + h*s[1] + r*s[2] + c.  tok: device int32
 * [B][Hkv][n_new]; values outside [0, n_src) are clamped into it (a wrong
 * index reads another row of the input, never outside it; n_src >= 1 is the
 * number of input rows per stream).  Otherwise as kvq_quantize (same
 * checks, layout and effect on n_tokens). */
kvq_status kvq_quantize_tokens(kvq_cache *cache, const void *k, const void *v, kvq_dtype in_dtype,
                               const int64_t k_strides[3], const int64_t v_strides[3],
                               const int32_t *tok, int32_t n_src, int32_t t0, int32_t n_new,
                               hipStream_t stream);

/* kvq_rank_tokens (host; [SEMKV] abstract: tokens ranked by a model-internal
 * score, the top-ranked at the higher of two precisions).  score: host
 * [n_streams][n_tokens] finite binary32.  order: host [n_streams][n_tokens]
 * output; per stream, the first n_high entries are the tokens with the
 * n_high largest scores (equal scores: the earlier token ranks first) in
 * ascending token order, the other n_tokens - n_high entries the remaining
 * tokens in ascending order.  KVQ_EINVAL for NULL pointers, sizes out of
 * range or a score that is not finite (order then unwritten). */
kvq_status kvq_rank_tokens(const float *score, int32_t n_streams, int32_t n_tokens, int32_t n_high,
                           int32_t *order);

/* Equivalent Right Shift of the whole cache ([PMKVQ] Key design 1): every
 * stored key and value tile of every stream goes from 2*to_bits to to_bits
 * bits in place, scales become narrow((2^b + 1) * S'), zero points stay.
 * Requires k_bits == v_bits == 2 * to_bits (uniform keys), to_bits in
 * {8, 4, 2, 1}.  On success k_bits = v_bits = to_bits. */
kvq_status kvq_shrink(kvq_cache *cache, int32_t to_bits, hipStream_t stream);

/* Bit-width halving rules compared in [PMKVQ]'s ablation (Key design 1 and
 * the ablation table): the Equivalent Right Shift above; the direct right
 * shift, which keeps the high b bits (X_b = X_2b >> b, S_b = 2^b * S_2b); and
 * the modified right shift, which the page names but does not define -- read
 * here as the rounded shift X_b = min((X_2b + 2^(b-1)) >> b, 2^b - 1),
 * S_b = 2^b * S_2b.  Zero points stay in every case; scales are narrowed to
 * the parameter dtype after the exact binary32 product. */
typedef enum { KVQ_SHIFT_ERS = 0, KVQ_SHIFT_DIRECT = 1, KVQ_SHIFT_MODIFIED = 2 } kvq_shift;

/* kvq_shrink with the halving rule chosen by method (kvq_shrink is
 * method = KVQ_SHIFT_ERS).  Same requirements, layout and effect on k_bits /
 * v_bits; KVQ_EINVAL for an unknown method. */
kvq_status kvq_shrink_shift(kvq_cache *cache, int32_t to_bits, kvq_shift method, hipStream_t stream);

/* Workspace bytes kvq_decode_attn needs for this cache geometry (sized for
 * max_tokens, so it stays valid as the cache grows).  0 on invalid input. */
size_t kvq_decode_workspace_bytes(const kvq_cache *cache, int32_t n_q_heads);

/* Decode attention of one query token per sequence over the n_tokens stored
 * tokens (see "Decode attention" above).  q: device bfloat16
 * [B][n_q_heads][128]; out: device float32 [B][n_q_heads][128]; n_q_heads a
 * multiple of n_kv_heads with 1 <= n_q_heads / n_kv_heads <= 16; n_tokens >= 128.
 * workspace: device buffer of at least kvq_decode_workspace_bytes() bytes,
 * 256-byte aligned, no initial contents needed: it holds the per-chunk
 * partials (max, sum, weighted values per head).  When the tokens are split
 * over several chunks, the partials are combined into out by a second kernel
 * on the same stream.  Concurrent calls must not share a workspace. */
kvq_status kvq_decode_attn(const kvq_cache *cache, const void *q, int32_t n_q_heads,
                           float softmax_scale, float *out, void *workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Decode attention in its two phases, as separate calls.  kvq_decode_attn
 * is the same two launches back to back.  The split is the one of
 * FlashAttention-style decoding (attention over token ranges, then a
 * rescaled sum), applied to the attention over the reconstructed cache of
 * [CHANMIX] Overall framework.  It serves callers that combine partials from
 * several sources (for example one sequence's tokens held on several
 * devices: each runs the first phase over its share, the partial slots are
 * gathered into one array, and one combine finishes), and callers that time
 * the phases apart.
 *
 * kvq_decode_attn_partials: the first phase over the packed cache.  The
 * stored tiles of every stream are cut into *n_slots chunks of
 * *tiles_per_slot consecutive tiles (the last may hold fewer); slot s covers
 * tokens [128 * s * tiles_per_slot, min(128 * (s + 1) * tiles_per_slot,
 * n_tokens)).  For stream bh = b * n_kv_heads + h, slot s and query head
 * j < G of the stream (query head h * G + j), with row r = (bh * n_slots + s)
 * * G + j and x_t = softmax_scale * log2(e) * (q . k^_t) over the slot's
 * tokens t (k^, v^ the reconstructions S' * q + Z'), it writes
 *   float ml[r][2] = {m, l},  l = sum_t 2^(x_t - m)
 *   float o[r][128]          = sum_t 2^(x_t - m) * v^_t  (not normalised)
 * where m is a reference the kernel picks (m <= max_t x_t <= m + 8 up to
 * rounding; the combine takes any finite m).  ml starts at byte 0 of
 * the workspace, o at byte round_up(8 * B * n_kv_heads * n_slots * G, 256)
 * (kvq_decode_partials_bytes gives the total).  Always written as partials,
 * also when n_slots is 1.  Requirements, workspace (at least
 * kvq_decode_workspace_bytes()) and errors as for kvq_decode_attn;
 * n_slots and tiles_per_slot: host pointers, written on success.
 *
 * kvq_decode_combine: the second phase.  For every (b, query head) it reads
 * n_slots partial rows in the layout above and writes
 *   out[b][hq][c] = sum_s 2^(m_s - M) o_s[c] / sum_s 2^(m_s - M) l_s,
 *   M = max_s m_s
 * (out: device float32 [B][n_q_heads][128], 16-byte aligned).  1 <= n_slots
 * <= 128, else KVQ_EINVAL; workspace 256-byte aligned with at least
 * kvq_decode_partials_bytes(batch, n_kv_heads, n_q_heads, n_slots) bytes,
 * else KVQ_EWORKSPACE; n_q_heads a multiple of n_kv_heads, at most 16 query
 * heads per kv head. */
kvq_status kvq_decode_attn_partials(const kvq_cache *cache, const void *q, int32_t n_q_heads,
                                    float softmax_scale, void *workspace, size_t workspace_bytes,
                                    int32_t *n_slots, int32_t *tiles_per_slot, hipStream_t stream);
size_t kvq_decode_partials_bytes(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads, int32_t n_slots);
kvq_status kvq_decode_combine(const void *workspace, size_t workspace_bytes, int32_t batch,
                              int32_t n_kv_heads, int32_t n_q_heads, int32_t n_slots, float *out,
                              hipStream_t stream);

/* Decode attention over the tokens of two caches of the same streams
 * ([SEMKV] abstract: every token kept, each stream's tokens split by rank
 * between two adjacent precisions).  For batch b and query head hq the
 * attended set is the union of cache a's and cache b's stored tokens of
 * stream (b, hq / G) (attention does not depend on the order of the tokens,
 * so the split need not follow positions).  The caches must have the same
 * batch and n_kv_heads; widths, parameter dtypes and capacities may differ;
 * either may hold no tokens, but together at least 128.  Each cache's chunks
 * leave partials (max, sum, weighted values) per head in one workspace and
 * one combine kernel merges them into out.  workspace: at least
 * kvq_decode_split_workspace_bytes(a, b, n_q_heads) bytes, 256-byte aligned,
 * no initial contents needed.  Other arguments and errors as for
 * kvq_decode_attn. */
size_t kvq_decode_split_workspace_bytes(const kvq_cache *a, const kvq_cache *b, int32_t n_q_heads);
kvq_status kvq_decode_attn_split(const kvq_cache *a, const kvq_cache *b, const void *q, int32_t n_q_heads,
                                 float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* Allocation-free decode attention, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  Same computation, arguments and errors as
 * kvq_decode_attn, without a caller workspace: the chunk partials live in
 * a library-owned device array of KVQ_DECODE_SCRATCH_BYTES
 * per GPU (static storage, held until the process ends; never allocated or
 * freed by the call).  The array of the current device is used, so the
 * stream must belong to the current device.  A call whose launch plan needs
 * more scratch than the array holds returns KVQ_EWORKSPACE before any device
 * work (about 520 * (n_chunks + 16) * batch * n_q_heads bytes; the Qwen2.5-7B- and
 * 32B-shaped layers at 32K tokens need under 8 MiB).  The array keeps the
 * last call's contents, which no call reads before writing them.  All calls
 * on one GPU share the array: calls that may overlap in time (on
 * different streams without ordering between them) race -- order them. */
#define KVQ_DECODE_SCRATCH_BYTES (32u << 20)
kvq_status kvq_decode_attn_noalloc(const kvq_cache *cache, const void *q, int32_t n_q_heads,
                                   float softmax_scale, float *out, hipStream_t stream);

/* Decode attention over the packed cache together with a residual segment
 * of res_len tokens per stream that are not packed ([PMKVQ] Training
 * strategy and Related work: as in KIVI, the first token and the most recent
 * tokens are kept at 16-bit precision instead of the low-bit codes).  The
 * caller holds those tokens -- the first token, and the recent tokens of the
 * 128-token group not yet quantized -- in res_k / res_v.  For batch b and
 * query head hq (kv head h = hq / G) the attended set is the n_tokens stored
 * tokens (reconstructions S' * q + Z') and the residual tokens
 * t = 0 .. res_len-1 with keys res_k[b][h][t][0..128) and values
 * res_v[b][h][t][0..128), read exactly (res_dtype KVQ_F32, KVQ_F16 or
 * KVQ_BF16) at element offsets b*s[0] + h*s[1] + t*s[2] + c
 * (s = res_k_strides / res_v_strides, channel stride 1; res_k and res_v
 * 16-byte aligned and every stride a multiple of 16 bytes, else
 * KVQ_EINVAL).  Attention does not
 * depend on the order of the tokens (positions are already applied to the
 * keys), so the residual tokens may be in any order.
 * 0 <= res_len <= KVQ_MAX_RESIDUAL; n_tokens may be 0 when res_len >= 1;
 * res_len = 0 is kvq_decode_attn.  Logits and weights of the residual tokens
 * are formed in binary32 and merged with the packed part through one more
 * partial (max, sum, weighted values) per head.  Other arguments, the
 * workspace and errors as for kvq_decode_attn. */
kvq_status kvq_decode_attn_residual(const kvq_cache *cache, const void *q, int32_t n_q_heads,
                                    float softmax_scale, const void *res_k, const void *res_v,
                                    kvq_dtype res_dtype, const int64_t res_k_strides[3],
                                    const int64_t res_v_strides[3], int32_t res_len, float *out,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Progressive schedule ([PMKVQ] Overall framework and Key design 1: each
 * block's cache starts at 16 bits; when its memory budget is full, the whole
 * cache drops one width, 16 -> 8 -> 4 -> 2, down to the block's target).
 *
 * A kvq_pool is a host-side tile allocator over a caller-owned device code
 * buffer of pool_bytes bytes that serves as both k_codes and v_codes; it
 * writes the device offset tables k_tile_off_dev / v_tile_off_dev (each
 * [max_tiles][B][Hkv] int64, caller-owned) and keeps a host copy.  After a
 * shrink, the second half of every tile returns to the pool; new tiles are
 * carved from freed halves first.  The cache must use these tables (its
 * k_tile_off / v_tile_off pointers equal the two device pointers).
 */
typedef struct kvq_pool kvq_pool;

kvq_status kvq_pool_create(const kvq_cache *cache, int64_t pool_bytes, int64_t *k_tile_off_dev,
                           int64_t *v_tile_off_dev, kvq_pool **out);
void kvq_pool_destroy(kvq_pool *pool);
/* Bytes of the pool currently holding tiles, and its high-water mark. */
int64_t kvq_pool_used_bytes(const kvq_pool *pool);
int64_t kvq_pool_high_water(const kvq_pool *pool);

/* Append n_new tokens (multiple of 128) to every stream of a uniform-width
 * cache under a memory budget: while kvq_cache_bytes(n_tokens + n_new) at the
 * current width exceeds budget_bytes, halve the width with kvq_shrink (never
 * below floor_bits); then allocate the new tiles (from `pool`, or at the
 * contiguous placement when pool is NULL) and kvq_quantize them at the
 * resulting width.  If the group does not fit even at floor_bits, or the
 * pool has no free extents left for the new tiles (after the halvings'
 * releases), returns KVQ_EBUDGET before any work, the pool unchanged.
 * *n_shrinks (may be NULL) receives the number of halvings performed.  Input
 * arguments as for kvq_quantize. */
kvq_status kvq_append(kvq_cache *cache, kvq_pool *pool, int64_t budget_bytes, int32_t floor_bits,
                      const void *k, const void *v, kvq_dtype in_dtype,
                      const int64_t k_strides[3], const int64_t v_strides[3], int32_t n_new,
                      hipStream_t stream, int32_t *n_shrinks);

/* ------------------------------------------------------------------------
 * Token-granular append ([PMKVQ] Training strategy and Related work: as in
 * KIVI, the first token and the most recent tokens stay at 16-bit precision
 * while the rest of the cache is packed).
 *
 * A kvq_window holds, for every stream of one cache, the tokens not packed:
 * row 0 the sequence's first token (when keep_first is set, for the whole
 * sequence), rows 1 .. n_recent the recent tokens that have not yet formed a
 * 128-token group.  k and v are caller-owned device buffers of
 * [batch][n_kv_heads][KVQ_WINDOW_ROWS][128] elements of `dtype`, 16-byte
 * aligned; their contents need no initialisation.  The caller zero-fills
 * n_first and n_recent for a new sequence; the library maintains them.
 *
 * Decode over cache + window: kvq_decode_attn_residual with
 * res_k = k + (1 - n_first) * 128 elements (likewise res_v), res_len =
 * n_first + n_recent, strides {n_kv_heads * KVQ_WINDOW_ROWS * 128,
 * KVQ_WINDOW_ROWS * 128, 128} and res_dtype = dtype.  The order of the
 * window rows is not token order, which attention does not depend on.
 */
#define KVQ_WINDOW_ROWS 129

typedef struct kvq_window {
    int32_t batch;            /* equal to the cache's batch */
    int32_t n_kv_heads;       /* equal to the cache's n_kv_heads */
    int32_t dtype;            /* kvq_dtype of the window and of appended tokens: F32 or BF16 */
    int32_t keep_first;       /* 1: the first token stays unpacked in row 0; 0: it is packed */
    void *k;                  /* device [B][Hkv][KVQ_WINDOW_ROWS][128] */
    void *v;                  /* device [B][Hkv][KVQ_WINDOW_ROWS][128] */
    int32_t n_first;          /* 0 or 1: row 0 holds the first token */
    int32_t n_recent;         /* 0 .. 128: rows 1 .. n_recent hold recent tokens */
} kvq_window;

/* Append n_new >= 0 tokens to every stream, in order: k[b][h][t][0..128) and
 * v[b][h][t][0..128) at element offsets b*s[0] + h*s[1] + t*s[2] + c of
 * w->dtype (16-byte aligned, strides multiples of 16 bytes).
 *   - With keep_first, the first token of an empty sequence (no packed
 *     tokens, an empty window) goes to row 0.
 *   - Every other token joins the recent rows.  When a token arrives while
 *     128 recent tokens are held, those 128 are packed as the cache's next
 *     group first (so after a call 1 .. 128 recent tokens are held, unless
 *     no token reached the recent rows).  Runs of more than 128 tokens that
 *     arrive with no recent tokens held are packed straight from k / v,
 *     leaving the last 1 .. 128 for the window.
 * Groups are packed by kvq_append under budget_bytes / floor_bits (with
 * `pool`; uniform widths only) when budget_bytes >= 0, one group per call in
 * token order, so the packed cache depends on the token sequence only and
 * not on how it was split into calls; or by kvq_quantize at the cache's
 * widths when budget_bytes < 0 (pool and the cache's tile tables must then
 * be NULL: groups go to the contiguous placement).  The cache's
 * n_tokens (and k_bits / v_bits after halvings) and the window's n_first /
 * n_recent are updated; *n_shrinks (may be NULL) counts the halvings.
 * Arguments, capacity (max_tokens), the budget at floor_bits for the final
 * token count and (with a pool) a replay of the group appends on a copy of
 * the pool's free extents are checked before any device work: any status
 * but KVQ_OK / KVQ_EHIP leaves the cache, the pool and the window as they
 * were.  After KVQ_EHIP the structs describe the work enqueued so far.  All work is on `stream`; calls on one window must use one
 * stream (or be ordered by the caller). */
kvq_status kvq_window_append(kvq_window *w, kvq_cache *cache, kvq_pool *pool, int64_t budget_bytes,
                             int32_t floor_bits, const void *k, const void *v,
                             const int64_t k_strides[3], const int64_t v_strides[3], int32_t n_new,
                             hipStream_t stream, int32_t *n_shrinks);

/* ------------------------------------------------------------------------
 * Block-wise bit-width allocation ([PMKVQ] Key design 2: each transformer
 * block gets one width, minimising the summed sensitivity s_{i,b} with the
 * blocks' total KV-cache memory within the budget M).  Host-only; the
 * sensitivities are the caller's (the page derives them from loss
 * gradients).
 *
 * sens: host [n_blocks][n_choices] finite binary64; bytes: host
 * [n_blocks][n_choices] cache bytes of block i at choice j (> 0, at most
 * 2^50).  Finds choice[i] in [0, n_choices) minimising
 *   s[0][c0] + (s[1][c1] + ( ... + s[n-1][c_{n-1}]))   (binary64, that order)
 * subject to sum_i bytes[i][c_i] <= budget_bytes, exactly (dynamic
 * programming over the costs divided by their greatest common divisor);
 * among minimal allocations the lexicographically smallest choice vector.
 * *cost (may be NULL) receives the minimum.  KVQ_EBUDGET if even the
 * cheapest choices exceed the budget; KVQ_EUNSUPPORTED if the table would
 * exceed KVQ_ALLOC_MAX_STATES entries (n_blocks + 1) * (budget / gcd + 1);
 * KVQ_EINVAL for bad arguments.  choice is written only on KVQ_OK. */
#define KVQ_ALLOC_MAX_CHOICES 16
#define KVQ_ALLOC_MAX_STATES ((int64_t)1 << 26)
kvq_status kvq_allocate_bits(int32_t n_blocks, int32_t n_choices, const double *sens,
                             const int64_t *bytes, int64_t budget_bytes, int32_t *choice,
                             double *cost);

/* ------------------------------------------------------------------------
 * Pair-granular key widths ([PNMIX] abstract: the quantization error of a
 * RoPE channel pair moves the attention logit in proportion to the product of
 * the query's and the key's norms over that pair, so the pairs with the
 * largest query-key pair-norm products get the higher widths, chosen once
 * from prefill statistics and kept through the decode).  Pair p (0 <= p < 64)
 * of a head is channels (p, p + 64), the rotate-half RoPE pairing.
 *
 * kvq_pair_norms: adds to out[h / group][p] (device binary32
 * [n_heads / group][64]) the sum over b < batch, over the heads h of each
 * group of `group` consecutive heads and over t < n_tokens of
 *   sqrt(x[b][h][t][p]^2 + x[b][h][t][p + 64]^2)
 * for x device [batch][n_heads][n_tokens][128] in in_dtype (KVQ_F32 or
 * KVQ_BF16), element strides (b, h, t) as given (token stride >= 128) and
 * unit channel stride.  Keys: group = 1 (one row per kv head); queries:
 * group = G folds the query heads of each kv head.  out is accumulated into
 * (zero it before the first call; calls over successive prefill chunks add
 * up), with device atomics, so the order of the binary32 sums is
 * unspecified.  With n_tokens == 0 nothing is read or enqueued (x may be
 * NULL).  Enqueued on `stream`; KVQ_EINVAL for bad arguments (nothing
 * enqueued), KVQ_EHIP if the launch fails. */
kvq_status kvq_pair_norms(const void *x, kvq_dtype in_dtype, const int64_t strides[3], int32_t batch,
                          int32_t n_heads, int32_t n_tokens, int32_t group, float *out,
                          hipStream_t stream);

/* kvq_pair_slot_map (host): the mixed key tile's slot order
 * (k_slot_chan, see the mixed layout above) from per-pair saliency scores,
 * score host [n_kv_heads][64] finite binary32 (e.g. the product of the
 * prefill queries' and keys' kvq_pair_norms).  Per kv head the pairs are
 * ranked by score, descending, equal scores by ascending pair index; the
 * first 4 pairs fill the eight 4-bit slots, the next 4 the eight 3-bit slots,
 * the last 4 the eight 1-bit slots and the other 52 the 104 2-bit slots, so
 * both channels of a pair share a width; inside each class the channels are
 * in ascending order.  slot_chan: host [n_kv_heads][128] output, written only
 * on KVQ_OK; KVQ_EINVAL for NULL pointers, n_kv_heads < 1 or a score that is
 * not finite. */
kvq_status kvq_pair_slot_map(const float *score, int32_t n_kv_heads, int16_t *slot_chan);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
