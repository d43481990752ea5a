"""C-ABI contract checks that need no GPU: the library loads, exports every
function include/kvq.h declares, and rejects invalid arguments on the host
before any launch (no call here reaches the device)."""
import ctypes
import os
import re

import pytest

from kv_cache_mixed_amd import kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def _lib():
    if not os.path.exists(kvq.LIB_PATH):
        pytest.skip("libkvq.so not built")
    return kvq.load()


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    L = _lib()
    names = _declared()
    assert set(names) == set(kvq.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_pure_host_helpers():
    L = _lib()
    assert kvq.tile_bytes(4) == 8192 and kvq.tile_bytes(0) == 4352 and kvq.tile_bytes(3) == 0
    assert kvq.strerror(kvq.EBUDGET).startswith("memory budget")
    s = _fake_struct(16, 4, 32768, 4, 4)
    s.n_tokens = 32768
    assert L.kvq_cache_bytes(ctypes.byref(s), 32768, 4, 4) == 285212672
    assert L.kvq_cache_bytes(ctypes.byref(s), 100, 4, 4) == -1
    s4 = _fake_struct(1, 8, 131072, 0, 2, kvq.E4M3)
    assert L.kvq_cache_bytes(ctypes.byref(s4), 131072, 0, 2) == 73400320
    ws = L.kvq_decode_workspace_bytes(ctypes.byref(s), 28)
    assert ws > 0 and ws % 4 == 0
    assert L.kvq_decode_workspace_bytes(ctypes.byref(s), 30) == 0      # not a multiple of Hkv
    assert L.kvq_decode_workspace_bytes(ctypes.byref(s), 4 * 17) == 0  # G > 16


FAKE = 0x10000000  # never dereferenced: every call below fails validation first


def _fake_struct(B, H, T, kb, vb, pdt=kvq.F16):
    s = kvq.KvqCacheStruct()
    s.batch, s.n_kv_heads, s.head_dim, s.group = B, H, 128, 128
    s.max_tokens, s.n_tokens, s.k_bits, s.v_bits = T, 0, kb, vb
    s.param_dtype, s.reserved0 = pdt, 0
    s.k_codes = s.v_codes = FAKE
    s.k_tile_off = s.v_tile_off = None
    s.k_tile_stride = kvq.tile_bytes(kb)
    s.v_tile_stride = kvq.value_tile_bytes(vb)
    s.k_scale = s.k_zero = s.v_scale = s.v_zero = FAKE
    s.k_slot_chan = FAKE if kb == 0 else None
    s.v_slot_chan = FAKE if vb == 0 else None
    return s


def test_validation_rejects_before_launch():
    L = _lib()
    st3 = (ctypes.c_int64 * 3)(0, 0, 128)
    vp = ctypes.c_void_p
    s = _fake_struct(2, 2, 1024, 4, 4)
    P = ctypes.byref
    # quantize
    assert L.kvq_quantize(None, vp(FAKE), vp(FAKE), kvq.F32, st3, st3, 0, 128, None) == kvq.EINVAL
    assert L.kvq_quantize(P(s), None, None, kvq.F32, st3, st3, 0, 128, None) == kvq.EINVAL
    assert L.kvq_quantize(P(s), vp(FAKE), vp(FAKE), kvq.F32, st3, st3, 64, 128, None) == kvq.EINVAL
    assert L.kvq_quantize(P(s), vp(FAKE), vp(FAKE), kvq.F32, st3, st3, 0, 100, None) == kvq.EINVAL
    assert L.kvq_quantize(P(s), vp(FAKE), vp(FAKE), kvq.F32, st3, st3, 896, 256, None) == kvq.EINVAL
    assert L.kvq_quantize(P(s), vp(FAKE), vp(FAKE), kvq.E4M3, st3, st3, 0, 128, None) == kvq.EINVAL
    assert L.kvq_quantize(P(s), vp(FAKE), None, kvq.F32, None, None, 0, 128, None) == kvq.EINVAL
    bad = _fake_struct(2, 2, 1024, 4, 4)
    bad.head_dim = 64
    assert L.kvq_quantize(P(bad), vp(FAKE), vp(FAKE), kvq.F32, st3, st3, 0, 128, None) == kvq.EUNSUPPORTED
    bad = _fake_struct(2, 2, 1000, 4, 4)
    assert L.kvq_quantize(P(bad), vp(FAKE), vp(FAKE), kvq.F32, st3, st3, 0, 128, None) == kvq.EINVAL
    bad = _fake_struct(2, 2, 1024, 3, 4)
    assert L.kvq_quantize(P(bad), vp(FAKE), vp(FAKE), kvq.F32, st3, st3, 0, 128, None) == kvq.EINVAL
    bad = _fake_struct(2, 2, 1024, 4, 4)
    bad.k_tile_stride = 1000
    assert L.kvq_quantize(P(bad), vp(FAKE), vp(FAKE), kvq.F32, st3, st3, 0, 128, None) == kvq.EINVAL
    bad = _fake_struct(2, 2, 1024, 0, 2)
    bad.k_slot_chan = None
    assert L.kvq_quantize(P(bad), vp(FAKE), vp(FAKE), kvq.F32, st3, st3, 0, 128, None) == kvq.EINVAL
    bad = _fake_struct(2, 2, 1024, 4, 4)
    bad.k_codes = FAKE + 4                                   # misaligned code buffer
    assert L.kvq_quantize(P(bad), vp(FAKE), vp(FAKE), kvq.F32, st3, st3, 0, 128, None) == kvq.EINVAL
    # shrink with an unknown halving rule, or a known one at a wrong width
    s2m = _fake_struct(2, 2, 1024, 4, 4)
    assert L.kvq_shrink_shift(P(s2m), 2, 3, None) == kvq.EINVAL
    assert L.kvq_shrink_shift(P(s2m), 2, -1, None) == kvq.EINVAL
    assert L.kvq_shrink_shift(P(s2m), 1, kvq.SHIFT_DIRECT, None) == kvq.EINVAL
    assert s2m.k_bits == 4 and s2m.v_bits == 4
    # shrink
    s2 = _fake_struct(2, 2, 1024, 4, 4)
    assert L.kvq_shrink(P(s2), 4, None) == kvq.EINVAL        # 4 -> 4 is not a halving
    assert L.kvq_shrink(P(s2), 1, None) == kvq.EINVAL        # 4 -> 1 skips a width
    assert L.kvq_shrink(P(s2), 3, None) == kvq.EINVAL
    sm = _fake_struct(1, 1, 1024, 0, 2)
    assert L.kvq_shrink(P(sm), 1, None) == kvq.EUNSUPPORTED  # mixed keys
    assert s2.k_bits == 4                                    # untouched on failure
    # decode
    s3 = _fake_struct(2, 2, 1024, 4, 4)
    s3.n_tokens = 512
    ws = L.kvq_decode_workspace_bytes(P(s3), 8)
    assert L.kvq_decode_attn(P(s3), vp(FAKE), 8, 0.088, vp(FAKE), None, ws, None) == kvq.EWORKSPACE
    assert L.kvq_decode_attn(P(s3), vp(FAKE), 8, 0.088, vp(FAKE), vp(FAKE), ws - 4, None) == kvq.EWORKSPACE
    assert L.kvq_decode_attn(P(s3), vp(FAKE), 7, 0.088, vp(FAKE), vp(FAKE), ws, None) == kvq.EINVAL
    assert L.kvq_decode_attn(P(s3), vp(FAKE), 2 * 17, 0.088, vp(FAKE), vp(FAKE), ws, None) == kvq.EUNSUPPORTED
    assert L.kvq_decode_attn(P(s3), None, 8, 0.088, vp(FAKE), vp(FAKE), ws, None) == kvq.EINVAL
    assert L.kvq_decode_attn(P(s3), vp(FAKE), 8, float("nan"), vp(FAKE), vp(FAKE), ws, None) == kvq.EINVAL
    s4 = _fake_struct(2, 2, 1024, 4, 2)                      # K4/V2 is not built
    s4.n_tokens = 512
    assert L.kvq_decode_attn(P(s4), vp(FAKE), 8, 0.088, vp(FAKE), vp(FAKE), ws, None) == kvq.EUNSUPPORTED
    s5 = _fake_struct(2, 2, 1024, 4, 4)                      # empty cache
    assert L.kvq_decode_attn(P(s5), vp(FAKE), 8, 0.088, vp(FAKE), vp(FAKE), ws, None) == kvq.EINVAL


def test_mixed_value_sizes_and_validation():
    """Mixed-width values (v_bits = KVQ_VMIXED): a 5120-byte tile (16 x 4 +
    16 x 4 + 16 x 2 + 80 x 2 bits per token: 3-bit codes in 4-bit fields,
    1-bit codes in 2-bit fields), four scales and zero points per token, a
    required slot map, no halving and no budgeted append."""
    L = _lib()
    P = ctypes.byref
    vp = ctypes.c_void_p
    st3 = (ctypes.c_int64 * 3)(0, 0, 128)
    assert kvq.value_tile_bytes(0) == 5120 and kvq.value_tile_bytes(4) == 8192
    assert kvq.value_tile_bytes(3) == 0 and kvq.tile_bytes(0) == 4352
    s = _fake_struct(1, 8, 131072, 0, 0, kvq.E4M3)
    # per 128-token group and stream: 4352 + 5120 code bytes, 2 x 128 key
    # parameters and 2 x 4 x 128 value parameters of one byte
    assert L.kvq_cache_bytes(P(s), 131072, 0, 0) == 8 * 1024 * (4352 + 5120 + 256 + 1024)
    f = _fake_struct(1, 8, 131072, 0, 0, kvq.F16)
    assert L.kvq_cache_bytes(P(f), 128, 0, 0) == 8 * (4352 + 5120 + 512 + 2048)
    assert L.kvq_cache_bytes(P(f), 128, 4, 0) == 8 * (8192 + 5120 + 512 + 2048)
    bad = _fake_struct(2, 2, 1024, 0, 0)
    bad.v_slot_chan = None
    assert L.kvq_quantize(P(bad), vp(FAKE), vp(FAKE), kvq.F32, st3, st3, 0, 128, None) == kvq.EINVAL
    bad = _fake_struct(2, 2, 1024, 0, 0)
    bad.v_tile_stride = 4352                                 # below the mixed value tile
    assert L.kvq_quantize(P(bad), vp(FAKE), vp(FAKE), kvq.F32, st3, st3, 0, 128, None) == kvq.EINVAL
    sm = _fake_struct(1, 1, 1024, 0, 0)
    assert L.kvq_shrink(P(sm), 1, None) == kvq.EUNSUPPORTED
    # decode: mixed keys with mixed values need e4m3 or binary16 parameters,
    # and uniform keys with mixed values are not built
    for kb, pdt, want in ((0, kvq.BF16, kvq.EUNSUPPORTED), (0, kvq.F32, kvq.EUNSUPPORTED),
                          (4, kvq.E4M3, kvq.EUNSUPPORTED)):
        d = _fake_struct(2, 2, 1024, kb, 0, pdt)
        d.n_tokens = 512
        ws = L.kvq_decode_workspace_bytes(P(d), 8)
        assert L.kvq_decode_attn(P(d), vp(FAKE), 8, 0.088, vp(FAKE), vp(FAKE), ws, None) == want


def test_append_budget_rejected_before_work():
    L = _lib()
    st3 = (ctypes.c_int64 * 3)(0, 0, 128)
    vp = ctypes.c_void_p
    s = _fake_struct(8, 4, 32768, 16, 16)
    s.n_tokens = 30720
    s.k_bits = s.v_bits = 2
    s.k_tile_stride = s.v_tile_stride = 2048 * 16
    n = ctypes.c_int32(-1)
    # 2-bit, floor 2: 30720 + 2048 tokens need 73.7 MiB > 70 MiB
    r = L.kvq_append(ctypes.byref(s), None, 70 * 2 ** 20, 2, vp(FAKE), vp(FAKE), kvq.F32, st3, st3,
                     2048, None, ctypes.byref(n))
    assert r == kvq.EBUDGET and n.value == 0 and s.k_bits == 2 and s.n_tokens == 30720
    # floor above the current width
    s.k_bits = s.v_bits = 4
    r = L.kvq_append(ctypes.byref(s), None, 1 << 40, 8, vp(FAKE), vp(FAKE), kvq.F32, st3, st3,
                     128, None, None)
    assert r == kvq.EINVAL


def test_residual_validation_rejects_before_launch():
    L = _lib()
    m = re.search(r"#define KVQ_MAX_RESIDUAL (\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == kvq.MAX_RESIDUAL
    vp = ctypes.c_void_p
    P = ctypes.byref
    rs = (ctypes.c_int64 * 3)(2 * 40 * 128, 40 * 128, 128)
    neg = (ctypes.c_int64 * 3)(2 * 40 * 128, -128, 128)
    s = _fake_struct(2, 2, 1024, 4, 4)
    s.n_tokens = 512
    ws = L.kvq_decode_workspace_bytes(P(s), 8)
    F = vp(FAKE)

    def call(st, rk, rv, rdt, ks, vs, R, w=F, wb=ws):
        return L.kvq_decode_attn_residual(P(st), F, 8, 0.088, rk, rv, rdt, ks, vs, R, F, w, wb, None)

    assert call(s, F, F, kvq.F32, rs, rs, kvq.MAX_RESIDUAL + 1) == kvq.EINVAL
    assert call(s, F, F, kvq.F32, rs, rs, -1) == kvq.EINVAL
    assert call(s, None, F, kvq.F32, rs, rs, 5) == kvq.EINVAL
    assert call(s, F, None, kvq.BF16, rs, rs, 5) == kvq.EINVAL
    assert call(s, F, F, kvq.F32, None, rs, 5) == kvq.EINVAL
    assert call(s, F, F, kvq.E4M3, rs, rs, 5) == kvq.EINVAL       # residual: f32, f16 or bf16
    assert call(s, F, F, kvq.F32, rs, neg, 5) == kvq.EINVAL
    odd = (ctypes.c_int64 * 3)(2 * 40 * 128, 40 * 128, 130)        # rows not 16-byte multiples
    assert call(s, F, F, kvq.F32, odd, rs, 5) == kvq.EINVAL
    assert call(s, F, F, kvq.BF16, rs, (ctypes.c_int64 * 3)(0, 0, 132), 5) == kvq.EINVAL
    assert call(s, F, F, kvq.F32, (ctypes.c_int64 * 3)(0, 0, 132), rs, 5, None) == kvq.EWORKSPACE
    assert call(s, vp(FAKE + 8), F, kvq.F32, rs, rs, 5) == kvq.EINVAL  # misaligned base
    assert call(s, F, F, kvq.F32, rs, rs, 5, None) == kvq.EWORKSPACE
    # empty cache: a residual segment alone is a valid request (reaches the
    # workspace check); with no residual there is nothing to attend
    e = _fake_struct(2, 2, 1024, 4, 4)
    assert call(e, F, F, kvq.F32, rs, rs, 0) == kvq.EINVAL
    assert call(e, F, F, kvq.F32, rs, rs, 3, None) == kvq.EWORKSPACE
    # a width pair the packed decode does not build is only an error when
    # the cache holds packed tokens
    u = _fake_struct(2, 2, 1024, 4, 2)
    assert call(u, F, F, kvq.F32, rs, rs, 3, None) == kvq.EWORKSPACE
    u.n_tokens = 128
    assert call(u, F, F, kvq.F32, rs, rs, 3, None) == kvq.EUNSUPPORTED


def test_decode_workspace_bytes_cover_the_partials():
    """The workspace bound holds the partials (max, sum: 8 B; weighted values:
    512 B per head) of every chunk a plan can make (at most 112, of at least 4
    tiles each) plus the 16 residual slots, and grows with the query heads."""
    L = _lib()
    for B, H, T in [(1, 1, 4096), (16, 4, 32768), (1, 8, 131072), (64, 4, 512), (3, 5, 2048)]:
        s = _fake_struct(B, H, T, 4, 4)
        for G in (1, 7, 16):
            chunks = min((T // 128 + 3) // 4, 112)
            need = B * H * G * (chunks + 16) * (8 + 512)
            got = L.kvq_decode_workspace_bytes(ctypes.byref(s), G * H)
            assert need <= got <= need + 512, (B, H, T, G, got, need)


def test_two_phase_decode_sizes_and_validation():
    """kvq_decode_partials_bytes: the (max, sum) pairs rounded up to 256
    bytes, then 512 bytes per head and slot; the partials and combine calls
    reject bad arguments on the host."""
    L = _lib()
    vp, P = ctypes.c_void_p, ctypes.byref
    for B, H, Hq, n in [(16, 4, 28, 16), (1, 8, 32, 64), (3, 5, 5, 1), (2, 2, 32, 128)]:
        BH, G = B * H, Hq // H
        want = (8 * BH * n * G + 255) // 256 * 256 + 512 * BH * n * G
        assert L.kvq_decode_partials_bytes(B, H, Hq, n) == want
    assert L.kvq_decode_partials_bytes(16, 4, 28, 0) == 0       # no slot
    assert L.kvq_decode_partials_bytes(16, 4, 28, 129) == 0     # past the combine's 128
    assert L.kvq_decode_partials_bytes(16, 4, 30, 16) == 0      # not a multiple of the kv heads
    assert L.kvq_decode_partials_bytes(1, 1, 17, 16) == 0       # G > 16
    comb = L.kvq_decode_combine
    need = L.kvq_decode_partials_bytes(2, 2, 8, 16)
    assert comb(vp(FAKE), need, 2, 2, 8, 0, vp(FAKE), None) == kvq.EINVAL
    assert comb(vp(FAKE), need, 2, 2, 8, 129, vp(FAKE), None) == kvq.EINVAL
    assert comb(vp(FAKE), need, 2, 2, 7, 16, vp(FAKE), None) == kvq.EINVAL
    assert comb(vp(FAKE), need, 2, 2, 8, 16, None, None) == kvq.EINVAL
    assert comb(vp(FAKE), need, 2, 2, 8, 16, vp(FAKE + 4), None) == kvq.EINVAL     # out not 16-byte aligned
    assert comb(None, need, 2, 2, 8, 16, vp(FAKE), None) == kvq.EWORKSPACE
    assert comb(vp(FAKE), need - 4, 2, 2, 8, 16, vp(FAKE), None) == kvq.EWORKSPACE
    assert comb(vp(FAKE + 128), need, 2, 2, 8, 16, vp(FAKE), None) == kvq.EWORKSPACE  # not 256-byte aligned
    assert comb(vp(FAKE), need, 1, 1, 17, 16, vp(FAKE), None) == kvq.EUNSUPPORTED
    part = L.kvq_decode_attn_partials
    s = _fake_struct(2, 2, 1024, 4, 4)
    s.n_tokens = 512
    ws = L.kvq_decode_workspace_bytes(P(s), 8)
    ns, tps = ctypes.c_int32(-1), ctypes.c_int32(-1)
    assert part(P(s), vp(FAKE), 8, 0.088, None, ws, P(ns), P(tps), None) == kvq.EWORKSPACE
    assert part(P(s), vp(FAKE), 8, 0.088, vp(FAKE), ws - 4, P(ns), P(tps), None) == kvq.EWORKSPACE
    assert part(P(s), vp(FAKE), 8, 0.088, vp(FAKE), ws, None, P(tps), None) == kvq.EINVAL
    assert part(P(s), vp(FAKE), 8, 0.088, vp(FAKE), ws, P(ns), None, None) == kvq.EINVAL
    assert part(P(s), vp(FAKE), 7, 0.088, vp(FAKE), ws, P(ns), P(tps), None) == kvq.EINVAL
    assert part(P(s), vp(FAKE), 8, float("inf"), vp(FAKE), ws, P(ns), P(tps), None) == kvq.EINVAL
    assert part(P(s), vp(FAKE), 2 * 17, 0.088, vp(FAKE), ws, P(ns), P(tps), None) == kvq.EUNSUPPORTED
    s4 = _fake_struct(2, 2, 1024, 4, 2)                      # K4/V2 is not built
    s4.n_tokens = 512
    assert part(P(s4), vp(FAKE), 8, 0.088, vp(FAKE), ws, P(ns), P(tps), None) == kvq.EUNSUPPORTED
    s5 = _fake_struct(2, 2, 1024, 4, 4)                      # empty cache
    assert part(P(s5), vp(FAKE), 8, 0.088, vp(FAKE), ws, P(ns), P(tps), None) == kvq.EINVAL
    assert ns.value == -1 and tps.value == -1                # untouched on failure


def _fake_window(s, dtype=kvq.BF16, keep_first=1):
    w = kvq.KvqWindowStruct()
    w.batch, w.n_kv_heads, w.dtype, w.keep_first = s.batch, s.n_kv_heads, dtype, keep_first
    w.k, w.v = FAKE, FAKE + 1024
    w.n_first = w.n_recent = 0
    return w


def test_window_validation_rejects_before_launch():
    """kvq_window_append checks arguments, capacity and the budget for the
    whole call before its first copy or group (no call here reaches the
    device), and leaves both structs unchanged on rejection."""
    L = _lib()
    m = re.search(r"#define KVQ_WINDOW_ROWS (\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == kvq.WINDOW_ROWS
    vp = ctypes.c_void_p
    P = ctypes.byref
    F = vp(FAKE)
    st = (ctypes.c_int64 * 3)(2 * 1000 * 128, 1000 * 128, 128)

    def call(w, s, n, budget=-1, floor=1, k=F, v=F, ks=st, vs=st, pool=None):
        return L.kvq_window_append(P(w), P(s), pool, budget, floor, k, v, ks, vs, n, None, None)

    s = _fake_struct(2, 2, 1024, 4, 4)
    w = _fake_window(s)
    assert call(w, s, 0) == kvq.OK                              # nothing to do
    assert call(w, s, -1) == kvq.EINVAL
    assert L.kvq_window_append(None, P(s), None, -1, 1, F, F, st, st, 5, None, None) == kvq.EINVAL
    for field, bad in (("batch", 3), ("n_kv_heads", 1), ("dtype", kvq.F16), ("keep_first", 2),
                       ("n_first", 2), ("n_recent", 129), ("n_recent", -1), ("k", 0), ("v", FAKE + 8)):
        w = _fake_window(s)
        setattr(w, field, bad)
        assert call(w, s, 5) == kvq.EINVAL, field
    w = _fake_window(s, keep_first=0)
    w.n_first = 1                                               # a first row without keep_first
    assert call(w, s, 5) == kvq.EINVAL
    w = _fake_window(s)
    assert call(w, s, 5, k=None) == kvq.EINVAL
    assert call(w, s, 5, ks=None) == kvq.EINVAL
    assert call(w, s, 5, v=vp(FAKE + 8)) == kvq.EINVAL           # misaligned input
    assert call(w, s, 5, ks=(ctypes.c_int64 * 3)(0, 0, 132)) == kvq.EINVAL   # 264-byte rows: not 16-byte units
    assert call(w, s, 5, vs=(ctypes.c_int64 * 3)(0, -128, 128)) == kvq.EINVAL
    # capacity: 1 first token + 1024 packed + 128 recent > 1024 + 129 held
    assert call(w, s, 1 + 1024 + 129) == kvq.EINVAL
    # budget for the final count at the floor width: 4 streams x 8 groups at
    # 1 bit with fp16 parameters, (2048 + 2048 + 4 * 128 * 2) B per group
    s16 = _fake_struct(2, 2, 1024, 16, 16)
    need = L.kvq_cache_bytes(P(s16), 1024, 1, 1)
    assert need == 2 * 2 * 8 * (2048 + 2048 + 4 * 128 * 2)
    w = _fake_window(s16)
    assert call(w, s16, 1 + 1024 + 1, budget=need - 1, floor=1) == kvq.EBUDGET
    assert call(w, s16, 1 + 1024 + 1, budget=1 << 40, floor=32) == kvq.EINVAL    # floor not a width
    tabled = _fake_struct(2, 2, 1024, 16, 16)
    tabled.k_tile_off = tabled.v_tile_off = FAKE                # tile tables without their pool
    assert call(_fake_window(tabled), tabled, 300, budget=1 << 40) == kvq.EINVAL
    # without a budget the groups go to the contiguous placement: tile tables
    # (a pool's, unfilled past its tiles) are rejected before any work
    assert call(_fake_window(tabled), tabled, 300, budget=-1) == kvq.EINVAL
    assert call(_fake_window(tabled), tabled, 5, budget=-1) == kvq.EINVAL
    mixed = _fake_struct(2, 2, 1024, kvq.KMIXED, 2)
    assert call(_fake_window(mixed), mixed, 300, budget=1 << 40) == kvq.EUNSUPPORTED  # budget: uniform widths
    assert w.n_first == 0 and w.n_recent == 0 and s16.n_tokens == 0 and s16.k_bits == 16


def test_append_pool_exhausted_before_work():
    """A pool without room for the new tiles fails kvq_append with
    KVQ_EBUDGET before any device work: the cache and the pool's counters are
    unchanged (the offset tables are never written, so fake pointers do)."""
    L = _lib()
    P = ctypes.byref
    vp = ctypes.c_void_p
    st3 = (ctypes.c_int64 * 3)(0, 0, 128)
    s = _fake_struct(1, 2, 1024, 16, 16)
    s.k_tile_off = s.v_tile_off = FAKE + 4096
    s.k_tile_stride = s.v_tile_stride = 0
    pool = vp()
    # 64 KiB: two 32 KiB 16-bit tiles, while 128 tokens of 2 streams need four
    assert L.kvq_pool_create(P(s), 64 << 10, vp(FAKE + 4096), vp(FAKE + 4096), P(pool)) == kvq.OK
    try:
        n = ctypes.c_int32(-1)
        r = L.kvq_append(P(s), pool, 1 << 40, 16, vp(FAKE), vp(FAKE), kvq.F32, st3, st3, 128, None, P(n))
        assert r == kvq.EBUDGET and n.value == 0
        assert s.n_tokens == 0 and s.k_bits == 16
        assert L.kvq_pool_used_bytes(pool) == 0 and L.kvq_pool_high_water(pool) == 0
    finally:
        L.kvq_pool_destroy(pool)


def test_window_pool_exhausted_before_work():
    """kvq_window_append under a budget replays its group appends on the
    pool first: a pool without room for them fails with KVQ_EBUDGET before
    the first copy, leaving cache, pool and window unchanged."""
    L = _lib()
    P = ctypes.byref
    vp = ctypes.c_void_p
    st = (ctypes.c_int64 * 3)(2 * 1000 * 128, 1000 * 128, 128)
    s = _fake_struct(1, 2, 1024, 16, 16)
    s.k_tile_off = s.v_tile_off = FAKE + 4096
    s.k_tile_stride = s.v_tile_stride = 0
    pool = vp()
    # 192 KiB: room for the 16-bit tiles of one group of 2 streams (4 x 32 KiB), not of two
    assert L.kvq_pool_create(P(s), 192 << 10, vp(FAKE + 4096), vp(FAKE + 4096), P(pool)) == kvq.OK
    try:
        w = _fake_window(s)
        n = ctypes.c_int32(-1)
        # first token + 300: two groups packed straight from the input, 43 held
        r = L.kvq_window_append(P(w), P(s), pool, 1 << 40, 16, vp(FAKE), vp(FAKE), st, st, 301, None, P(n))
        assert r == kvq.EBUDGET and n.value == 0
        assert (w.n_first, w.n_recent, s.n_tokens, s.k_bits) == (0, 0, 0, 16)
        assert L.kvq_pool_used_bytes(pool) == 0 and L.kvq_pool_high_water(pool) == 0
    finally:
        L.kvq_pool_destroy(pool)
