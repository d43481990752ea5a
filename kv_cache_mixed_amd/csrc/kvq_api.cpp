// kvq_api.cpp -- the C ABI of libkvq (include/kvq.h): argument validation on
// the host, kernel launches, and the progressive-schedule runtime (tile pool
// and budget-driven append).
//
// Every entry point validates all of its arguments before enqueuing any device
// work, and never lets a C++ exception cross the ABI.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <map>
#include <new>
#include <vector>

#include "kvq.h"
#include "kvq_device.h"

namespace {

bool valid_bits(int b) { return b == 1 || b == 2 || b == 4 || b == 8 || b == 16; }
bool valid_kbits(int b) { return b == KVQ_KMIXED || valid_bits(b); }
bool valid_vbits(int b) { return b == KVQ_VMIXED || valid_bits(b); }
bool valid_pdt(int p) { return p == KVQ_F32 || p == KVQ_F16 || p == KVQ_BF16 || p == KVQ_E4M3; }
int param_bytes(int p) { return p == KVQ_F32 ? 4 : (p == KVQ_E4M3 ? 1 : 2); }
int64_t tile_bytes(int bits) {
  return bits == KVQ_KMIXED ? (int64_t)KVQ_MIXED_TILE_BYTES : (int64_t)2048 * bits;
}
int64_t vtile_bytes(int bits) {
  return bits == KVQ_VMIXED ? (int64_t)KVQ_VMIXED_TILE_BYTES : (int64_t)2048 * bits;
}
// value scales (and zero points) per token
int vparams_per_token(int bits) { return bits == KVQ_VMIXED ? 4 : 1; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Structural checks shared by every call.  `bits_ok` lets callers validate
// widths themselves.
kvq_status check_cache(const kvq_cache* c) {
  if (!c) return KVQ_EINVAL;
  if (c->batch < 1 || c->n_kv_heads < 1) return KVQ_EINVAL;
  if (c->head_dim != KVQ_HEAD_DIM || c->group != KVQ_GROUP) return KVQ_EUNSUPPORTED;
  if (c->max_tokens < 128 || c->max_tokens % 128 || c->max_tokens > KVQ_MAX_TOKENS) return KVQ_EINVAL;
  if (c->n_tokens < 0 || c->n_tokens % 128 || c->n_tokens > c->max_tokens) return KVQ_EINVAL;
  if (!valid_kbits(c->k_bits) || !valid_vbits(c->v_bits)) return KVQ_EINVAL;
  if (!valid_pdt(c->param_dtype) || c->reserved0 != 0) return KVQ_EINVAL;
  if (!c->k_codes || !c->v_codes || !c->k_scale || !c->k_zero || !c->v_scale || !c->v_zero)
    return KVQ_EINVAL;
  if (!aligned(c->k_codes, 256) || !aligned(c->v_codes, 256)) return KVQ_EINVAL;
  if (!aligned(c->k_scale, 16) || !aligned(c->k_zero, 16) || !aligned(c->v_scale, 16) ||
      !aligned(c->v_zero, 16))
    return KVQ_EINVAL;
  if (c->k_bits == KVQ_KMIXED && !c->k_slot_chan) return KVQ_EINVAL;
  if (c->v_bits == KVQ_VMIXED && !c->v_slot_chan) return KVQ_EINVAL;
  if (!c->k_tile_off) {
    if (c->k_tile_stride < tile_bytes(c->k_bits) || c->k_tile_stride % 256) return KVQ_EINVAL;
  }
  if (!c->v_tile_off) {
    if (c->v_tile_stride < vtile_bytes(c->v_bits) || c->v_tile_stride % 256) return KVQ_EINVAL;
  }
  return KVQ_OK;
}

kvq::Geo make_geo(const kvq_cache* c) {
  kvq::Geo g;
  g.B = c->batch;
  g.H = c->n_kv_heads;
  g.max_tiles = c->max_tokens / 128;
  g.n_tiles = c->n_tokens / 128;
  g.max_tokens = c->max_tokens;
  g.k_bits = c->k_bits;
  g.v_bits = c->v_bits;
  g.pdt = c->param_dtype;
  g.k_codes = (uint8_t*)c->k_codes;
  g.v_codes = (uint8_t*)c->v_codes;
  g.k_off = c->k_tile_off;
  g.v_off = c->v_tile_off;
  g.k_stride = c->k_tile_stride;
  g.v_stride = c->v_tile_stride;
  g.k_scale = c->k_scale;
  g.k_zero = c->k_zero;
  g.v_scale = c->v_scale;
  g.v_zero = c->v_zero;
  g.slot_chan = c->k_slot_chan;
  g.v_slot_chan = c->v_slot_chan;
  return g;
}

}  // namespace

extern "C" {

const char* kvq_strerror(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_EINVAL: return "invalid argument";
    case KVQ_EUNSUPPORTED: return "unsupported configuration";
    case KVQ_EBUDGET: return "memory budget exceeded even at the floor bit width";
    case KVQ_EWORKSPACE: return "workspace missing or too small";
    case KVQ_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

size_t kvq_tile_bytes(int32_t bits) {
  if (!valid_kbits(bits)) return 0;
  return (size_t)tile_bytes(bits);
}

size_t kvq_value_tile_bytes(int32_t bits) {
  if (!valid_vbits(bits)) return 0;
  return (size_t)vtile_bytes(bits);
}

int64_t kvq_cache_bytes(const kvq_cache* c, int32_t n_tokens, int32_t k_bits, int32_t v_bits) {
  if (!c || c->batch < 1 || c->n_kv_heads < 1 || !valid_pdt(c->param_dtype)) return -1;
  if (n_tokens < 0 || n_tokens % 128 || !valid_kbits(k_bits) || !valid_vbits(v_bits)) return -1;
  const int64_t groups = n_tokens / 128;
  const int64_t pb = param_bytes(c->param_dtype);
  const int64_t per_group = tile_bytes(k_bits) + vtile_bytes(v_bits) + 2 * 128 * pb  // key S,Z
                            + 2 * 128 * pb * vparams_per_token(v_bits);              // value S,Z
  return (int64_t)c->batch * c->n_kv_heads * groups * per_group;
}

kvq_status kvq_quantize(kvq_cache* c, const void* k, const void* v, kvq_dtype in_dtype,
                        const int64_t k_strides[3], const int64_t v_strides[3], int32_t t0,
                        int32_t n_new, hipStream_t stream) {
  try {
    kvq_status s = check_cache(c);
    if (s != KVQ_OK) return s;
    if (!k && !v) return KVQ_EINVAL;
    if (in_dtype != KVQ_F32 && in_dtype != KVQ_BF16) return KVQ_EINVAL;
    if ((k && !k_strides) || (v && !v_strides)) return KVQ_EINVAL;
    if (t0 < 0 || t0 % 128 || n_new < 128 || n_new % 128) return KVQ_EINVAL;
    if ((int64_t)t0 + n_new > c->max_tokens) return KVQ_EINVAL;
    if ((int64_t)n_new / 128 > 65535 || c->n_kv_heads > 65535 || c->batch > 65535)
      return KVQ_EUNSUPPORTED;
    const int64_t zero[3] = {0, 0, 0};
    kvq::Geo g = make_geo(c);
    hipError_t e = kvq::launch_quantize(g, k, v, in_dtype, k ? k_strides : zero,
                                        v ? v_strides : zero, t0, n_new, stream);
    if (e != hipSuccess) return KVQ_EHIP;
    c->n_tokens = std::max(c->n_tokens, t0 + n_new);
    return KVQ_OK;
  } catch (...) {
    return KVQ_EHIP;
  }
}

kvq_status kvq_quantize_tokens(kvq_cache* c, const void* k, const void* v, kvq_dtype in_dtype,
                               const int64_t k_strides[3], const int64_t v_strides[3],
                               const int32_t* tok, int32_t n_src, int32_t t0, int32_t n_new,
                               hipStream_t stream) {
  try {
    kvq_status s = check_cache(c);
    if (s != KVQ_OK) return s;
    if (!tok || n_src < 1) return KVQ_EINVAL;
    if (!k && !v) return KVQ_EINVAL;
    if (in_dtype != KVQ_F32 && in_dtype != KVQ_BF16) return KVQ_EINVAL;
    if ((k && !k_strides) || (v && !v_strides)) return KVQ_EINVAL;
    if (t0 < 0 || t0 % 128 || n_new < 128 || n_new % 128) return KVQ_EINVAL;
    if ((int64_t)t0 + n_new > c->max_tokens) return KVQ_EINVAL;
    if ((int64_t)n_new / 128 > 65535 || c->n_kv_heads > 65535 || c->batch > 65535)
      return KVQ_EUNSUPPORTED;
    const int64_t zero[3] = {0, 0, 0};
    kvq::Geo g = make_geo(c);
    hipError_t e = kvq::launch_quantize(g, k, v, in_dtype, k ? k_strides : zero, v ? v_strides : zero, t0,
                                        n_new, stream, tok, n_src);
    if (e != hipSuccess) return KVQ_EHIP;
    c->n_tokens = std::max(c->n_tokens, t0 + n_new);
    return KVQ_OK;
  } catch (...) {
    return KVQ_EHIP;
  }
}

kvq_status kvq_rank_tokens(const float* score, int32_t n_streams, int32_t n_tokens, int32_t n_high,
                           int32_t* order) {
  try {
    if (!score || !order || n_streams < 1 || n_tokens < 1 || n_high < 0 || n_high > n_tokens)
      return KVQ_EINVAL;
    const int64_t n = (int64_t)n_streams * n_tokens;
    for (int64_t i = 0; i < n; i++)
      if (!std::isfinite(score[i])) return KVQ_EINVAL;
    std::vector<int32_t> idx(n_tokens), out((size_t)n);
    for (int32_t sidx = 0; sidx < n_streams; sidx++) {
      const float* sc = score + (int64_t)sidx * n_tokens;
      for (int32_t t = 0; t < n_tokens; t++) idx[t] = t;
      // the n_high largest scores (equal scores: the earlier token first)
      std::stable_sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) { return sc[a] > sc[b]; });
      std::sort(idx.begin(), idx.begin() + n_high);
      std::sort(idx.begin() + n_high, idx.end());
      std::copy(idx.begin(), idx.end(), out.begin() + (int64_t)sidx * n_tokens);
    }
    std::copy(out.begin(), out.end(), order);
    return KVQ_OK;
  } catch (...) {
    return KVQ_EHIP;
  }
}

kvq_status kvq_shrink(kvq_cache* c, int32_t to_bits, hipStream_t stream) {
  return kvq_shrink_shift(c, to_bits, KVQ_SHIFT_ERS, stream);
}

kvq_status kvq_shrink_shift(kvq_cache* c, int32_t to_bits, kvq_shift method, hipStream_t stream) {
  try {
    kvq_status s = check_cache(c);
    if (s != KVQ_OK) return s;
    if (method != KVQ_SHIFT_ERS && method != KVQ_SHIFT_DIRECT && method != KVQ_SHIFT_MODIFIED)
      return KVQ_EINVAL;
    if (to_bits != 8 && to_bits != 4 && to_bits != 2 && to_bits != 1) return KVQ_EINVAL;
    if (c->k_bits == KVQ_KMIXED) return KVQ_EUNSUPPORTED;
    if (c->k_bits != 2 * to_bits || c->v_bits != 2 * to_bits) return KVQ_EINVAL;
    if ((int64_t)c->batch * c->n_kv_heads > 65535) return KVQ_EUNSUPPORTED;
    kvq::Geo g = make_geo(c);
    hipError_t e = kvq::launch_shrink(g, to_bits, (int)method, stream);
    if (e != hipSuccess) return KVQ_EHIP;
    c->k_bits = to_bits;
    c->v_bits = to_bits;
    return KVQ_OK;
  } catch (...) {
    return KVQ_EHIP;
  }
}

size_t kvq_decode_workspace_bytes(const kvq_cache* c, int32_t n_q_heads) {
  if (!c || c->batch < 1 || c->n_kv_heads < 1 || c->max_tokens < 128 || c->max_tokens % 128)
    return 0;
  if (n_q_heads < 1 || n_q_heads % c->n_kv_heads) return 0;
  const int G = n_q_heads / c->n_kv_heads;
  if (G > 16) return 0;
  return kvq::decode_workspace_bytes(c->batch, c->n_kv_heads, G, c->max_tokens / 128);
}

// Shared by kvq_decode_attn and kvq_decode_attn_residual: validate everything
// on the host, then launch.
static kvq_status decode_common(const kvq_cache* c, const void* q, int32_t n_q_heads,
                                float softmax_scale, const kvq::ResArgs& res, int res_dtype,
                                float* out, void* workspace, size_t workspace_bytes,
                                hipStream_t stream, bool use_scratch = false) {
  kvq_status s = check_cache(c);
  if (s != KVQ_OK) return s;
  if (!q || !out) return KVQ_EINVAL;
  if (!aligned(q, 16) || !aligned(out, 16)) return KVQ_EINVAL;
  if (n_q_heads < 1 || n_q_heads % c->n_kv_heads) return KVQ_EINVAL;
  const int G = n_q_heads / c->n_kv_heads;
  if (G > 16) return KVQ_EUNSUPPORTED;
  if (res.R < 0 || res.R > KVQ_MAX_RESIDUAL) return KVQ_EINVAL;
  if (res.R == 0 && c->n_tokens < 128) return KVQ_EINVAL;   // nothing to attend
  if (res.R > 0) {
    if (!res.k || !res.v) return KVQ_EINVAL;
    if (res_dtype != KVQ_F32 && res_dtype != KVQ_F16 && res_dtype != KVQ_BF16) return KVQ_EINVAL;
    // rows are read with 16-byte loads: aligned bases, strides in whole 16-byte units
    const int64_t vw = res_dtype == KVQ_F32 ? 4 : 8;
    if (!aligned(res.k, 16) || !aligned(res.v, 16)) return KVQ_EINVAL;
    for (int i = 0; i < 3; i++)
      if (res.ks[i] < 0 || res.vs[i] < 0 || res.ks[i] % vw || res.vs[i] % vw) return KVQ_EINVAL;
  }
  if (!(softmax_scale == softmax_scale) || softmax_scale == INFINITY ||
      softmax_scale == -INFINITY)
    return KVQ_EINVAL;
  if (c->n_tokens > 0 && !kvq::decode_supported(c->k_bits, c->v_bits, c->param_dtype))
    return KVQ_EUNSUPPORTED;
  if ((int64_t)c->batch * c->n_kv_heads > 65535) return KVQ_EUNSUPPORTED;
  if (use_scratch) {
    // allocation-free variant: this call's own plan must fit the library's
    // scratch array
    kvq::DecodePlan plan;
    plan.n_chunks = 0;
    if (c->n_tokens > 0) {
      plan = kvq::decode_plan(c->batch * c->n_kv_heads, G, c->k_bits, c->v_bits, c->param_dtype,
                              c->n_tokens / 128);
      if (plan.n_chunks > kvq::KVQ_MAX_CHUNKS || plan.n_chunks * plan.tpc < c->n_tokens / 128)
        return KVQ_EWORKSPACE;
    }
    if (kvq::decode_workspace_needed(c->batch * c->n_kv_heads, G, plan) > (size_t)KVQ_DECODE_SCRATCH_BYTES)
      return KVQ_EWORKSPACE;
    hipError_t e = kvq::decode_scratch_acquire(&workspace);
    if (e != hipSuccess) return KVQ_EHIP;
    kvq::Geo g = make_geo(c);
    e = kvq::launch_decode(g, q, G, softmax_scale, out, workspace, res, res_dtype, stream);
    return e == hipSuccess ? KVQ_OK : KVQ_EHIP;
  }
  const size_t need = kvq::decode_workspace_bytes(c->batch, c->n_kv_heads, G, c->max_tokens / 128);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return KVQ_EWORKSPACE;
  if (c->n_tokens > 0) {
    // the plan of this call must fit the workspace (guaranteed by the bound
    // above; checked so a sizing mistake can never turn into stray writes)
    const kvq::DecodePlan plan = kvq::decode_plan(c->batch * c->n_kv_heads, G, c->k_bits, c->v_bits,
                                                  c->param_dtype, c->n_tokens / 128);
    if (kvq::decode_workspace_needed(c->batch * c->n_kv_heads, G, plan) > workspace_bytes ||
        plan.n_chunks > kvq::KVQ_MAX_CHUNKS || plan.n_chunks * plan.tpc < c->n_tokens / 128)
      return KVQ_EWORKSPACE;
  }
  kvq::Geo g = make_geo(c);
  hipError_t e = kvq::launch_decode(g, q, G, softmax_scale, out, workspace, res, res_dtype, stream);
  return e == hipSuccess ? KVQ_OK : KVQ_EHIP;
}

kvq_status kvq_decode_attn(const kvq_cache* c, const void* q, int32_t n_q_heads,
                           float softmax_scale, float* out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  try {
    kvq::ResArgs res{};
    res.R = 0;
    return decode_common(c, q, n_q_heads, softmax_scale, res, KVQ_F32, out, workspace,
                         workspace_bytes, stream);
  } catch (...) {
    return KVQ_EHIP;
  }
}

kvq_status kvq_decode_attn_partials(const kvq_cache* c, const void* q, int32_t n_q_heads, float softmax_scale,
                                    void* workspace, size_t workspace_bytes, int32_t* n_slots,
                                    int32_t* tiles_per_slot, hipStream_t stream) {
  try {
    kvq_status s = check_cache(c);
    if (s != KVQ_OK) return s;
    if (!q || !n_slots || !tiles_per_slot || !aligned(q, 16)) return KVQ_EINVAL;
    if (n_q_heads < 1 || n_q_heads % c->n_kv_heads) return KVQ_EINVAL;
    const int G = n_q_heads / c->n_kv_heads;
    if (G > 16) return KVQ_EUNSUPPORTED;
    if (c->n_tokens < 128) return KVQ_EINVAL;   // nothing to attend
    if (!(softmax_scale == softmax_scale) || softmax_scale == INFINITY || softmax_scale == -INFINITY)
      return KVQ_EINVAL;
    if (!kvq::decode_supported(c->k_bits, c->v_bits, c->param_dtype)) return KVQ_EUNSUPPORTED;
    if ((int64_t)c->batch * c->n_kv_heads > 65535) return KVQ_EUNSUPPORTED;
    const int BH = c->batch * c->n_kv_heads;
    const size_t need = kvq::decode_workspace_bytes(c->batch, c->n_kv_heads, G, c->max_tokens / 128);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return KVQ_EWORKSPACE;
    const kvq::DecodePlan plan =
        kvq::decode_plan(BH, G, c->k_bits, c->v_bits, c->param_dtype, c->n_tokens / 128);
    if (plan.n_chunks < 1 || plan.n_chunks > kvq::KVQ_MAX_CHUNKS || plan.n_chunks * plan.tpc < c->n_tokens / 128 ||
        kvq::decode_partials_bytes(BH, G, plan.n_chunks) > workspace_bytes)
      return KVQ_EWORKSPACE;
    int ns = 0, tps = 0;
    hipError_t e = kvq::launch_decode_partials(make_geo(c), q, G, softmax_scale, workspace, &ns, &tps, stream);
    if (e != hipSuccess) return KVQ_EHIP;
    *n_slots = ns;
    *tiles_per_slot = tps;
    return KVQ_OK;
  } catch (...) {
    return KVQ_EHIP;
  }
}

size_t kvq_decode_partials_bytes(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads, int32_t n_slots) {
  if (batch < 1 || n_kv_heads < 1 || n_q_heads < 1 || n_q_heads % n_kv_heads) return 0;
  const int G = n_q_heads / n_kv_heads;
  if (G > 16 || n_slots < 1 || n_slots > kvq::KVQ_MAX_SLOTS) return 0;
  if ((int64_t)batch * n_kv_heads > 65535) return 0;
  return kvq::decode_partials_bytes(batch * n_kv_heads, G, n_slots);
}

kvq_status kvq_decode_combine(const void* workspace, size_t workspace_bytes, int32_t batch, int32_t n_kv_heads,
                              int32_t n_q_heads, int32_t n_slots, float* out, hipStream_t stream) {
  try {
    if (batch < 1 || n_kv_heads < 1 || n_q_heads < 1 || n_q_heads % n_kv_heads) return KVQ_EINVAL;
    const int G = n_q_heads / n_kv_heads;
    if (G > 16 || (int64_t)batch * n_kv_heads > 65535) return KVQ_EUNSUPPORTED;
    if (n_slots < 1 || n_slots > kvq::KVQ_MAX_SLOTS) return KVQ_EINVAL;
    if (!out || !aligned(out, 16)) return KVQ_EINVAL;
    if (!workspace || !aligned(workspace, 256) ||
        workspace_bytes < kvq::decode_partials_bytes(batch * n_kv_heads, G, n_slots))
      return KVQ_EWORKSPACE;
    hipError_t e = kvq::launch_decode_combine(workspace, batch, n_kv_heads, G, n_slots, out, stream);
    return e == hipSuccess ? KVQ_OK : KVQ_EHIP;
  } catch (...) {
    return KVQ_EHIP;
  }
}

size_t kvq_decode_split_workspace_bytes(const kvq_cache* a, const kvq_cache* b, int32_t n_q_heads) {
  if (check_cache(a) != KVQ_OK || check_cache(b) != KVQ_OK) return 0;
  if (a->batch != b->batch || a->n_kv_heads != b->n_kv_heads) return 0;
  if (n_q_heads < a->n_kv_heads || n_q_heads % a->n_kv_heads) return 0;
  return kvq::decode_split_workspace_bytes(a->batch, a->n_kv_heads, n_q_heads / a->n_kv_heads);
}

kvq_status kvq_decode_attn_split(const kvq_cache* a, const kvq_cache* b, const void* q, int32_t n_q_heads,
                                 float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  try {
    const kvq_cache* cs[2] = {a, b};
    for (const kvq_cache* c : cs) {
      kvq_status s = check_cache(c);
      if (s != KVQ_OK) return s;
      if (c->n_tokens > 0 && !kvq::decode_supported(c->k_bits, c->v_bits, c->param_dtype))
        return KVQ_EUNSUPPORTED;
    }
    if (a->batch != b->batch || a->n_kv_heads != b->n_kv_heads) return KVQ_EINVAL;
    if (!q || !out) return KVQ_EINVAL;
    if (n_q_heads < a->n_kv_heads || n_q_heads % a->n_kv_heads) return KVQ_EINVAL;
    const int G = n_q_heads / a->n_kv_heads;
    if (G > 16) return KVQ_EUNSUPPORTED;
    if (a->n_tokens + (int64_t)b->n_tokens < 128) return KVQ_EINVAL;   // nothing to attend
    if (!(softmax_scale == softmax_scale) || softmax_scale == INFINITY || softmax_scale == -INFINITY)
      return KVQ_EINVAL;
    if ((int64_t)a->batch * a->n_kv_heads > 65535) return KVQ_EUNSUPPORTED;
    const size_t need = kvq::decode_split_workspace_bytes(a->batch, a->n_kv_heads, G);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return KVQ_EWORKSPACE;
    const int BH = a->batch * a->n_kv_heads;
    int slots = 0;
    for (const kvq_cache* c : cs) {
      if (c->n_tokens == 0) continue;
      const kvq::DecodePlan p = kvq::decode_plan(BH, G, c->k_bits, c->v_bits, c->param_dtype, c->n_tokens / 128,
                                                 kvq::KVQ_SPLIT_MAX_CHUNKS);
      if (p.n_chunks > kvq::KVQ_SPLIT_MAX_CHUNKS || p.n_chunks * p.tpc < c->n_tokens / 128) return KVQ_EWORKSPACE;
      slots += p.n_chunks;
    }
    kvq::DecodePlan pall;
    pall.n_chunks = slots - kvq::KVQ_MAX_RES_SLOTS;
    if (slots > kvq::KVQ_MAX_SLOTS || (pall.n_chunks > 0 && kvq::decode_workspace_needed(BH, G, pall) > workspace_bytes))
      return KVQ_EWORKSPACE;
    hipError_t e = kvq::launch_decode_split(make_geo(a), make_geo(b), q, G, softmax_scale, out, workspace, stream);
    return e == hipSuccess ? KVQ_OK : KVQ_EHIP;
  } catch (...) {
    return KVQ_EHIP;
  }
}

kvq_status kvq_decode_attn_noalloc(const kvq_cache* c, const void* q, int32_t n_q_heads,
                                   float softmax_scale, float* out, hipStream_t stream) {
  try {
    kvq::ResArgs res{};
    res.R = 0;
    return decode_common(c, q, n_q_heads, softmax_scale, res, KVQ_F32, out, nullptr, 0, stream, true);
  } catch (...) {
    return KVQ_EHIP;
  }
}

kvq_status kvq_decode_attn_residual(const kvq_cache* c, const void* q, int32_t n_q_heads,
                                    float softmax_scale, const void* res_k, const void* res_v,
                                    kvq_dtype res_dtype, const int64_t res_k_strides[3],
                                    const int64_t res_v_strides[3], int32_t res_len, float* out,
                                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  try {
    if (res_len > 0 && (!res_k_strides || !res_v_strides)) return KVQ_EINVAL;
    kvq::ResArgs res{};
    res.k = res_k;
    res.v = res_v;
    res.R = res_len;
    for (int i = 0; i < 3; i++) {
      res.ks[i] = res_len > 0 ? res_k_strides[i] : 0;
      res.vs[i] = res_len > 0 ? res_v_strides[i] : 0;
    }
    return decode_common(c, q, n_q_heads, softmax_scale, res, (int)res_dtype, out, workspace,
                         workspace_bytes, stream);
  } catch (...) {
    return KVQ_EHIP;
  }
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Tile pool: power-of-two extents of one device buffer.  Every tile at width b
// is 2048*b bytes; after a halving the second half of each tile is returned.
// Allocation takes the smallest free extent that fits (splitting larger ones)
// before growing the high-water mark, so freed halves are always reused first.
// ---------------------------------------------------------------------------
// The extent state (free lists, high-water mark, bytes in use) is its own
// value type, so a call can plan its releases and allocations on a copy and
// commit them only once every allocation has succeeded.
struct PoolExtents {
  int64_t capacity = 0;
  int64_t high = 0;
  int64_t used = 0;
  std::map<int64_t, std::vector<int64_t>> free_by_size;

  bool alloc(int64_t size, int64_t* off) {
    auto it = free_by_size.lower_bound(size);
    while (it != free_by_size.end() && it->second.empty()) ++it;
    if (it != free_by_size.end()) {
      int64_t ext = it->first, o = it->second.back();
      it->second.pop_back();
      // split: keep the first `size` bytes, return the rest as power-of-two pieces
      int64_t piece = size;
      while (piece < ext) {
        free_by_size[piece].push_back(o + piece);
        piece *= 2;
      }
      *off = o;
      used += size;
      return true;
    }
    if (high + size > capacity) return false;
    *off = high;
    high += size;
    used += size;
    return true;
  }
  void release(int64_t off, int64_t size) {
    free_by_size[size].push_back(off);
    used -= size;
  }
};

struct kvq_pool {
  int B, H, max_tiles;
  int64_t* k_dev;
  int64_t* v_dev;
  std::vector<int64_t> k_host, v_host;   // [max_tiles][B][H]
  PoolExtents ext;
};

extern "C" {

kvq_status kvq_pool_create(const kvq_cache* c, int64_t pool_bytes, int64_t* k_dev, int64_t* v_dev,
                           kvq_pool** out) {
  try {
    if (!out) return KVQ_EINVAL;
    *out = nullptr;
    kvq_status s = check_cache(c);
    if (s != KVQ_OK) return s;
    if (!k_dev || !v_dev || pool_bytes < 2048 || pool_bytes % 256) return KVQ_EINVAL;
    if (c->k_tile_off != k_dev || c->v_tile_off != v_dev) return KVQ_EINVAL;
    if (c->k_codes != c->v_codes) return KVQ_EINVAL;
    if (c->n_tokens != 0) return KVQ_EINVAL;
    kvq_pool* p = new (std::nothrow) kvq_pool();
    if (!p) return KVQ_EINVAL;
    p->B = c->batch;
    p->H = c->n_kv_heads;
    p->max_tiles = c->max_tokens / 128;
    p->ext.capacity = pool_bytes;
    p->k_dev = k_dev;
    p->v_dev = v_dev;
    const size_t n = (size_t)p->max_tiles * p->B * p->H;
    p->k_host.assign(n, -1);
    p->v_host.assign(n, -1);
    *out = p;
    return KVQ_OK;
  } catch (...) {
    return KVQ_EINVAL;
  }
}

void kvq_pool_destroy(kvq_pool* p) { delete p; }
int64_t kvq_pool_used_bytes(const kvq_pool* p) { return p ? p->ext.used : -1; }
int64_t kvq_pool_high_water(const kvq_pool* p) { return p ? p->ext.high : -1; }

kvq_status kvq_append(kvq_cache* c, kvq_pool* pool, int64_t budget, int32_t floor_bits,
                      const void* k, const void* v, kvq_dtype in_dtype, const int64_t k_strides[3],
                      const int64_t v_strides[3], int32_t n_new, hipStream_t stream,
                      int32_t* n_shrinks) {
  try {
    if (n_shrinks) *n_shrinks = 0;
    kvq_status s = check_cache(c);
    if (s != KVQ_OK) return s;
    if (!k || !v || !k_strides || !v_strides) return KVQ_EINVAL;
    if (in_dtype != KVQ_F32 && in_dtype != KVQ_BF16) return KVQ_EINVAL;
    if (c->k_bits == KVQ_KMIXED || c->k_bits != c->v_bits) return KVQ_EUNSUPPORTED;
    if (!valid_bits(floor_bits) || floor_bits > c->k_bits) return KVQ_EINVAL;
    if (n_new < 128 || n_new % 128 || (int64_t)c->n_tokens + n_new > c->max_tokens)
      return KVQ_EINVAL;
    if (pool && (pool->B != c->batch || pool->H != c->n_kv_heads ||
                 pool->max_tiles != c->max_tokens / 128 || c->k_tile_off != pool->k_dev ||
                 c->v_tile_off != pool->v_dev))
      return KVQ_EINVAL;
    if (!pool && (c->k_tile_off || c->v_tile_off)) return KVQ_EINVAL;
    // the launch limits of kvq_shrink and kvq_quantize, checked before any shrink
    if ((int64_t)c->batch * c->n_kv_heads > 65535 || n_new / 128 > 65535) return KVQ_EUNSUPPORTED;
    // plan the halvings first: fail with no work done if the floor cannot hold it
    int bits = c->k_bits, halvings = 0;
    const int32_t target = c->n_tokens + n_new;
    while (kvq_cache_bytes(c, target, bits, bits) > budget) {
      if (bits == 1 || bits / 2 < floor_bits) return KVQ_EBUDGET;
      bits /= 2;
      halvings++;
    }
    // the pool's side of the halvings (each frees the second half of every
    // stored tile) and of the new tiles, planned on a copy of its extents:
    // running out of free extents fails here, before any device work
    const size_t per = (size_t)c->batch * c->n_kv_heads;
    const int t_first = c->n_tokens / 128, t_last = target / 128;
    std::vector<int64_t> new_k, new_v;
    PoolExtents plan;
    if (pool) {
      plan = pool->ext;
      int w = c->k_bits;
      for (int i = 0; i < halvings; i++) {
        w /= 2;
        const int64_t half = tile_bytes(w);              // the halved tile size
        for (size_t idx = 0; idx < (size_t)t_first * per; idx++) {
          plan.release(pool->k_host[idx] + half, half);
          plan.release(pool->v_host[idx] + half, half);
        }
      }
      const int64_t sz = tile_bytes(w);
      new_k.resize((size_t)(t_last - t_first) * per);
      new_v.resize(new_k.size());
      for (size_t i = 0; i < new_k.size(); i++)
        if (!plan.alloc(sz, &new_k[i]) || !plan.alloc(sz, &new_v[i])) return KVQ_EBUDGET;
    }
    for (int i = 0; i < halvings; i++) {
      s = kvq_shrink(c, c->k_bits / 2, stream);
      if (s != KVQ_OK) return s;
      if (n_shrinks) (*n_shrinks)++;
    }
    if (pool) {
      pool->ext = std::move(plan);
      const size_t first = (size_t)t_first * per, count = (size_t)(t_last - t_first) * per;
      std::copy(new_k.begin(), new_k.end(), pool->k_host.begin() + first);
      std::copy(new_v.begin(), new_v.end(), pool->v_host.begin() + first);
      if (hipMemcpyAsync(pool->k_dev + first, pool->k_host.data() + first, count * 8,
                         hipMemcpyHostToDevice, stream) != hipSuccess)
        return KVQ_EHIP;
      if (hipMemcpyAsync(pool->v_dev + first, pool->v_host.data() + first, count * 8,
                         hipMemcpyHostToDevice, stream) != hipSuccess)
        return KVQ_EHIP;
    }
    return kvq_quantize(c, k, v, in_dtype, k_strides, v_strides, c->n_tokens, n_new, stream);
  } catch (...) {
    return KVQ_EHIP;
  }
}


// Token-granular append: the window of unpacked tokens (first token + recent
// tokens) and the hand-over of full 128-token groups to the packed cache.

// Replays n_groups one-group kvq_append calls (halvings from the byte count,
// the pool's releases and allocations in kvq_append's order) on a copy of the
// pool's extents; false if an allocation would fail.  Offsets of the tiles
// placed during the replay are tracked so that later halvings release their
// halves too.
static bool pool_replay_ok(const kvq_cache* c, const kvq_pool* pool, int64_t budget, int32_t floor_bits,
                           int64_t n_groups) {
  PoolExtents ext = pool->ext;
  std::map<size_t, int64_t> k_new, v_new;
  const size_t per = (size_t)c->batch * c->n_kv_heads;
  auto off = [&](const std::map<size_t, int64_t>& placed, const std::vector<int64_t>& host, size_t idx) {
    const auto it = placed.find(idx);
    return it != placed.end() ? it->second : host[idx];
  };
  int32_t n = c->n_tokens;
  int bits = c->k_bits;
  for (int64_t g = 0; g < n_groups; g++) {
    const int32_t target = n + 128;
    while (kvq_cache_bytes(c, target, bits, bits) > budget) {
      if (bits == 1 || bits / 2 < floor_bits) return false;
      bits /= 2;
      const int64_t half = tile_bytes(bits);
      for (size_t idx = 0; idx < (size_t)(n / 128) * per; idx++) {
        ext.release(off(k_new, pool->k_host, idx) + half, half);
        ext.release(off(v_new, pool->v_host, idx) + half, half);
      }
    }
    const int64_t sz = tile_bytes(bits);
    for (size_t idx = (size_t)(n / 128) * per; idx < (size_t)(target / 128) * per; idx++) {
      int64_t ko, vo;
      if (!ext.alloc(sz, &ko) || !ext.alloc(sz, &vo)) return false;
      k_new[idx] = ko;
      v_new[idx] = vo;
    }
    n = target;
  }
  return true;
}

kvq_status kvq_window_append(kvq_window* w, kvq_cache* c, kvq_pool* pool, int64_t budget,
                             int32_t floor_bits, const void* k, const void* v, const int64_t ks[3],
                             const int64_t vs[3], int32_t n_new, hipStream_t stream,
                             int32_t* n_shrinks) {
  try {
    if (n_shrinks) *n_shrinks = 0;
    kvq_status s = check_cache(c);
    if (s != KVQ_OK) return s;
    if (!w || w->batch != c->batch || w->n_kv_heads != c->n_kv_heads) return KVQ_EINVAL;
    if (w->dtype != KVQ_F32 && w->dtype != KVQ_BF16) return KVQ_EINVAL;
    if ((w->keep_first != 0 && w->keep_first != 1) || (w->n_first != 0 && w->n_first != 1) ||
        (w->n_first && !w->keep_first))
      return KVQ_EINVAL;
    if (w->n_recent < 0 || w->n_recent > 128) return KVQ_EINVAL;
    if (!w->k || !w->v || !aligned(w->k, 16) || !aligned(w->v, 16)) return KVQ_EINVAL;
    if (n_new < 0) return KVQ_EINVAL;
    if (n_new == 0) return KVQ_OK;
    if (!k || !v || !ks || !vs || !aligned(k, 16) || !aligned(v, 16)) return KVQ_EINVAL;
    const int elt = w->dtype == KVQ_F32 ? 4 : 2;
    for (int i = 0; i < 3; i++)
      if (ks[i] < 0 || vs[i] < 0 || (ks[i] * elt) % 16 || (vs[i] * elt) % 16) return KVQ_EINVAL;
    if ((int64_t)c->batch * c->n_kv_heads > 65535) return KVQ_EUNSUPPORTED;
    if (budget >= 0) {
      // the checks kvq_append makes, so that no group hand-over can fail on them later
      if (c->k_bits == KVQ_KMIXED || c->k_bits != c->v_bits) return KVQ_EUNSUPPORTED;
      if (!valid_bits(floor_bits) || floor_bits > c->k_bits) return KVQ_EINVAL;
      if (pool && (pool->B != c->batch || pool->H != c->n_kv_heads ||
                   pool->max_tiles != c->max_tokens / 128 || c->k_tile_off != pool->k_dev ||
                   c->v_tile_off != pool->v_dev))
        return KVQ_EINVAL;
      if (!pool && (c->k_tile_off || c->v_tile_off)) return KVQ_EINVAL;
    } else if (pool || c->k_tile_off || c->v_tile_off) {
      // without a budget the groups go to kvq_quantize at the contiguous
      // placement: tile tables (which a pool fills only when it allocates)
      // could name tiles that were never placed
      return KVQ_EINVAL;
    }

    // plan: the first token, filling the recent rows, groups packed from the
    // window (one each time a token arrives with 128 held) or straight from
    // the input (runs longer than 128 arriving with no recent token held),
    // and the rest into the recent rows
    const int first = (w->keep_first && !w->n_first && c->n_tokens == 0 && w->n_recent == 0) ? 1 : 0;
    int64_t packed = 0, direct = 0;
    {
      int64_t r = n_new - first;
      int recent = w->n_recent;
      if (r > 0 && recent == 128) { packed += 128; recent = 0; }
      if (r > 0 && recent > 0) {
        const int64_t fill = std::min<int64_t>(r, 128 - recent);
        r -= fill;
        if (r > 0) packed += 128;
      }
      if (r > 128) { direct = (r - 1) / 128 * 128; packed += direct; }
    }
    if ((int64_t)c->n_tokens + packed > c->max_tokens) return KVQ_EINVAL;
    if (direct / 128 > 65535) return KVQ_EUNSUPPORTED;
    if (budget >= 0 && packed > 0 &&
        kvq_cache_bytes(c, (int32_t)(c->n_tokens + packed), floor_bits, floor_bits) > budget)
      return KVQ_EBUDGET;
    // under a budget the groups go to kvq_append one at a time: replay them
    // on the pool first, so that running out of extents fails before any work
    if (budget >= 0 && pool && packed > 0 && !pool_replay_ok(c, pool, budget, floor_bits, packed / 128))
      return KVQ_EBUDGET;

    const int64_t wst[3] = {(int64_t)c->n_kv_heads * KVQ_WINDOW_ROWS * 128, KVQ_WINDOW_ROWS * 128, 128};
    const uint8_t* wk_row1 = (const uint8_t*)w->k + 128 * elt;
    const uint8_t* wv_row1 = (const uint8_t*)w->v + 128 * elt;
    auto at = [&](const void* p, const int64_t* st, int64_t t) { return (const uint8_t*)p + t * st[2] * elt; };
    auto copy = [&](int64_t t, int m, int slot0) -> kvq_status {
      hipError_t e = kvq::launch_window_copy(at(k, ks, t), at(v, vs, t), ks, vs, elt, w->k, w->v,
                                             c->batch, c->n_kv_heads, m, slot0, stream);
      return e == hipSuccess ? KVQ_OK : KVQ_EHIP;
    };
    auto pack = [&](const void* pk, const void* pv, const int64_t* sk, const int64_t* sv, int n) {
      if (budget < 0)
        return kvq_quantize(c, pk, pv, (kvq_dtype)w->dtype, sk, sv, c->n_tokens, n, stream);
      int32_t ns = 0;
      const kvq_status e = kvq_append(c, pool, budget, floor_bits, pk, pv, (kvq_dtype)w->dtype, sk, sv, n,
                                      stream, &ns);
      if (n_shrinks) *n_shrinks += ns;
      return e;
    };

    int64_t t = 0;
    if (first) {
      if ((s = copy(0, 1, 0)) != KVQ_OK) return s;
      w->n_first = 1;
      t = 1;
    }
    if (t < n_new && w->n_recent == 128) {
      if ((s = pack(wk_row1, wv_row1, wst, wst, 128)) != KVQ_OK) return s;
      w->n_recent = 0;
    }
    if (t < n_new && w->n_recent > 0) {
      const int fill = (int)std::min<int64_t>(n_new - t, 128 - w->n_recent);
      if ((s = copy(t, fill, 1 + w->n_recent)) != KVQ_OK) return s;
      w->n_recent += fill;
      t += fill;
      if (t < n_new) {
        if ((s = pack(wk_row1, wv_row1, wst, wst, 128)) != KVQ_OK) return s;
        w->n_recent = 0;
      }
    }
    if (n_new - t > 128) {
      // under a budget one group at a time, as if the tokens had come one by
      // one (a halving decided for several groups at once would quantize the
      // earlier ones at the narrower width instead of shrinking them)
      const int d = (int)((n_new - t - 1) / 128 * 128);
      const int step = budget >= 0 ? 128 : d;
      for (int done = 0; done < d; done += step) {
        if ((s = pack(at(k, ks, t), at(v, vs, t), ks, vs, step)) != KVQ_OK) return s;
        t += step;
      }
    }
    if (t < n_new) {
      if ((s = copy(t, (int)(n_new - t), 1)) != KVQ_OK) return s;
      w->n_recent = (int)(n_new - t);
    }
    return KVQ_OK;
  } catch (...) {
    return KVQ_EHIP;
  }
}

}  // extern "C"
