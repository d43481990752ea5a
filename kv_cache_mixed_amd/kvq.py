"""ctypes binding of libkvq (C ABI in include/kvq.h).

Argument marshalling only: every step of quantize / shrink / decode attention
runs in the HIP kernels of libkvq.so.  torch supplies device memory and the
current HIP stream.  There is no fallback: if the library is missing, load()
raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

F32, F16, BF16, E4M3 = 0, 1, 2, 3
PARAM_BYTES = {F32: 4, F16: 2, BF16: 2, E4M3: 1}
KMIXED = 0
VMIXED = 0                 # v_bits selecting the mixed-width value tile
MIXED_TILE_BYTES = 4352
VMIXED_TILE_BYTES = 5120
OK, EINVAL, EUNSUPPORTED, EBUDGET, EWORKSPACE, EHIP = range(6)
SHIFT_ERS, SHIFT_DIRECT, SHIFT_MODIFIED = range(3)   # kvq_shift of the header
MAX_RESIDUAL = 512          # KVQ_MAX_RESIDUAL of the header


class KvqCacheStruct(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("group", ctypes.c_int32),
        ("max_tokens", ctypes.c_int32), ("n_tokens", ctypes.c_int32),
        ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32),
        ("param_dtype", ctypes.c_int32), ("reserved0", ctypes.c_int32),
        ("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
        ("k_tile_off", ctypes.c_void_p), ("v_tile_off", ctypes.c_void_p),
        ("k_tile_stride", ctypes.c_int64), ("v_tile_stride", ctypes.c_int64),
        ("k_scale", ctypes.c_void_p), ("k_zero", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p), ("v_zero", ctypes.c_void_p),
        ("k_slot_chan", ctypes.c_void_p),
        ("v_slot_chan", ctypes.c_void_p),
    ]


WINDOW_ROWS = 129          # KVQ_WINDOW_ROWS of the header


class KvqWindowStruct(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("keep_first", ctypes.c_int32),
        ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("n_first", ctypes.c_int32), ("n_recent", ctypes.c_int32),
    ]


class KvqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, strerror(status), status))


_lib = None

EXPORTS = ["kvq_strerror", "kvq_tile_bytes", "kvq_value_tile_bytes", "kvq_cache_bytes", "kvq_quantize", "kvq_shrink",
           "kvq_shrink_shift", "kvq_decode_workspace_bytes", "kvq_decode_attn", "kvq_decode_attn_noalloc",
           "kvq_decode_attn_residual", "kvq_quantize_tokens", "kvq_rank_tokens",
           "kvq_decode_split_workspace_bytes", "kvq_decode_attn_split",
           "kvq_decode_attn_partials", "kvq_decode_partials_bytes", "kvq_decode_combine",
           "kvq_pool_create", "kvq_pool_destroy", "kvq_pool_used_bytes", "kvq_pool_high_water",
           "kvq_append", "kvq_window_append", "kvq_allocate_bits", "kvq_pair_norms", "kvq_pair_slot_map"]


def load():
    """Load libkvq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libkvq.so not built at %s (run __graft_entry__.build())" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(KvqCacheStruct)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.kvq_strerror.restype = ctypes.c_char_p
    L.kvq_strerror.argtypes = [ctypes.c_int]
    L.kvq_tile_bytes.restype = ctypes.c_size_t
    L.kvq_tile_bytes.argtypes = [i32]
    L.kvq_value_tile_bytes.restype = ctypes.c_size_t
    L.kvq_value_tile_bytes.argtypes = [i32]
    L.kvq_cache_bytes.restype = i64
    L.kvq_cache_bytes.argtypes = [P, i32, i32, i32]
    L.kvq_quantize.restype = ctypes.c_int
    L.kvq_quantize.argtypes = [P, vp, vp, ctypes.c_int, vp, vp, i32, i32, vp]
    L.kvq_shrink.restype = ctypes.c_int
    L.kvq_shrink.argtypes = [P, i32, vp]
    L.kvq_shrink_shift.restype = ctypes.c_int
    L.kvq_shrink_shift.argtypes = [P, i32, ctypes.c_int, vp]
    L.kvq_decode_workspace_bytes.restype = ctypes.c_size_t
    L.kvq_decode_workspace_bytes.argtypes = [P, i32]
    L.kvq_decode_attn.restype = ctypes.c_int
    L.kvq_decode_attn.argtypes = [P, vp, i32, ctypes.c_float, vp, vp, ctypes.c_size_t, vp]
    L.kvq_quantize_tokens.restype = ctypes.c_int
    L.kvq_quantize_tokens.argtypes = [P, vp, vp, ctypes.c_int, vp, vp, vp, i32, i32, i32, vp]
    L.kvq_rank_tokens.restype = ctypes.c_int
    L.kvq_rank_tokens.argtypes = [vp, i32, i32, i32, vp]
    L.kvq_decode_split_workspace_bytes.restype = ctypes.c_size_t
    L.kvq_decode_split_workspace_bytes.argtypes = [P, P, i32]
    L.kvq_decode_attn_split.restype = ctypes.c_int
    L.kvq_decode_attn_split.argtypes = [P, P, vp, i32, ctypes.c_float, vp, vp, ctypes.c_size_t, vp]
    L.kvq_decode_attn_noalloc.restype = ctypes.c_int
    L.kvq_decode_attn_noalloc.argtypes = [P, vp, i32, ctypes.c_float, vp, vp]
    L.kvq_decode_attn_partials.restype = ctypes.c_int
    L.kvq_decode_attn_partials.argtypes = [P, vp, i32, ctypes.c_float, vp, ctypes.c_size_t,
                                           ctypes.POINTER(i32), ctypes.POINTER(i32), vp]
    L.kvq_decode_partials_bytes.restype = ctypes.c_size_t
    L.kvq_decode_partials_bytes.argtypes = [i32, i32, i32, i32]
    L.kvq_decode_combine.restype = ctypes.c_int
    L.kvq_decode_combine.argtypes = [vp, ctypes.c_size_t, i32, i32, i32, i32, vp, vp]
    L.kvq_decode_attn_residual.restype = ctypes.c_int
    L.kvq_decode_attn_residual.argtypes = [P, vp, i32, ctypes.c_float, vp, vp, ctypes.c_int, vp, vp,
                                           i32, vp, vp, ctypes.c_size_t, vp]
    L.kvq_allocate_bits.restype = ctypes.c_int
    L.kvq_allocate_bits.argtypes = [i32, i32, vp, vp, i64, vp, ctypes.POINTER(ctypes.c_double)]
    L.kvq_pair_norms.restype = ctypes.c_int
    L.kvq_pair_norms.argtypes = [vp, ctypes.c_int, ctypes.POINTER(ctypes.c_int64), i32, i32, i32, i32, vp, vp]
    L.kvq_pair_slot_map.restype = ctypes.c_int
    L.kvq_pair_slot_map.argtypes = [vp, i32, vp]
    L.kvq_pool_create.restype = ctypes.c_int
    L.kvq_pool_create.argtypes = [P, i64, vp, vp, ctypes.POINTER(vp)]
    L.kvq_pool_destroy.restype = None
    L.kvq_pool_destroy.argtypes = [vp]
    L.kvq_pool_used_bytes.restype = i64
    L.kvq_pool_used_bytes.argtypes = [vp]
    L.kvq_pool_high_water.restype = i64
    L.kvq_pool_high_water.argtypes = [vp]
    L.kvq_append.restype = ctypes.c_int
    L.kvq_append.argtypes = [P, vp, i64, i32, vp, vp, ctypes.c_int, vp, vp, i32, vp,
                             ctypes.POINTER(i32)]
    L.kvq_window_append.restype = ctypes.c_int
    L.kvq_window_append.argtypes = [ctypes.POINTER(KvqWindowStruct), P, vp, i64, i32, vp, vp, vp, vp, i32, vp,
                                    ctypes.POINTER(i32)]
    _lib = L
    return L


def strerror(status: int) -> str:
    return load().kvq_strerror(status).decode()


def _check(status: int, what: str):
    if status != OK:
        raise KvqError(status, what)


def _stream_ptr(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _strides3(t):
    """(b, h, t) element strides of a [B][H][T][128] tensor with unit channel stride."""
    assert t.dim() == 4 and t.shape[-1] == 128 and t.stride(-1) == 1
    return (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))


def pair_norms(x, group=1, out=None, stream=None):
    """kvq_pair_norms: x [B][H][T][128] float32 / bfloat16 device tensor with
    unit channel stride -> out [H // group][64] float32 (added to when given,
    else a fresh zero tensor)."""
    import torch
    in_dtype = {torch.float32: F32, torch.bfloat16: BF16}[x.dtype]
    B, H, T, _ = x.shape
    if out is None:
        out = torch.zeros((H // group, 64), dtype=torch.float32, device=x.device)
    assert out.dtype == torch.float32 and out.is_contiguous() and out.shape == (H // group, 64)
    st = load().kvq_pair_norms(_ptr(x), in_dtype, _strides3(x), B, H, T, group, _ptr(out), _stream_ptr(stream))
    _check(st, "kvq_pair_norms")
    return out


def pair_slot_map(score):
    """kvq_pair_slot_map: score [Hkv][64] (host, float32) -> slot_chan
    [Hkv][128] int16 (the mixed key tile's slot order)."""
    import numpy as np
    s = np.ascontiguousarray(score, dtype=np.float32)
    assert s.ndim == 2 and s.shape[1] == 64
    out = np.empty((s.shape[0], 128), dtype=np.int16)
    _check(load().kvq_pair_slot_map(s.ctypes.data, s.shape[0], out.ctypes.data), "kvq_pair_slot_map")
    return out


def allocate_bits(sens, nbytes, budget_bytes):
    """kvq_allocate_bits: sens [n_blocks][n_choices] (float64), nbytes
    [n_blocks][n_choices] (int64) host arrays -> (choice indices, minimum)."""
    import numpy as np
    s = np.ascontiguousarray(sens, dtype=np.float64)
    w = np.ascontiguousarray(nbytes, dtype=np.int64)
    assert s.ndim == 2 and s.shape == w.shape
    choice = np.zeros(s.shape[0], dtype=np.int32)
    cost = ctypes.c_double(0.0)
    st = load().kvq_allocate_bits(s.shape[0], s.shape[1], s.ctypes.data, w.ctypes.data, int(budget_bytes),
                                  choice.ctypes.data, ctypes.byref(cost))
    _check(st, "kvq_allocate_bits")
    return choice, cost.value


def rank_tokens(score, n_high):
    """kvq_rank_tokens: score [n_streams][n_tokens] float32 (host) -> order
    [n_streams][n_tokens] int32: per stream the n_high highest-scoring tokens
    (ascending), then the others (ascending)."""
    import numpy as np
    sc = np.ascontiguousarray(score, dtype=np.float32)
    assert sc.ndim == 2
    order = np.empty(sc.shape, dtype=np.int32)
    _check(load().kvq_rank_tokens(sc.ctypes.data, sc.shape[0], sc.shape[1], int(n_high), order.ctypes.data),
           "kvq_rank_tokens")
    return order


def split_workspace(cache_a, cache_b, n_q_heads):
    """device workspace for decode_attn_split (uint8 tensor)"""
    import torch
    n = int(load().kvq_decode_split_workspace_bytes(ctypes.byref(cache_a.s), ctypes.byref(cache_b.s), n_q_heads))
    if n == 0:
        raise KvqError(EINVAL, "kvq_decode_split_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=cache_a.device)


def decode_attn_split(cache_a, cache_b, q, softmax_scale, out=None, workspace=None, stream=None):
    """kvq_decode_attn_split: attention over the union of two caches' tokens
    (same batch and kv heads)."""
    import torch
    assert q.dtype == torch.bfloat16 and q.is_contiguous()
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    ws = workspace if workspace is not None else split_workspace(cache_a, cache_b, q.shape[1])
    st = load().kvq_decode_attn_split(ctypes.byref(cache_a.s), ctypes.byref(cache_b.s), _ptr(q), q.shape[1],
                                      float(softmax_scale), _ptr(out), _ptr(ws), ws.numel(), _stream_ptr(stream))
    _check(st, "kvq_decode_attn_split")
    return out


def partials_bytes(batch, n_kv_heads, n_q_heads, n_slots):
    """kvq_decode_partials_bytes: bytes of n_slots partial slots per stream
    (0 for invalid arguments)."""
    return int(load().kvq_decode_partials_bytes(batch, n_kv_heads, n_q_heads, n_slots))


def partials_views(ws, batch, n_kv_heads, n_q_heads, n_slots):
    """(ml, o) float32 views of a partials workspace: ml [B*Hkv][n_slots][G][2],
    o [B*Hkv][n_slots][G][128]."""
    import torch
    G = n_q_heads // n_kv_heads
    BH = batch * n_kv_heads
    n_ml = BH * n_slots * G * 2
    o_off = (n_ml * 4 + 255) // 256 * 256
    f = ws[:partials_bytes(batch, n_kv_heads, n_q_heads, n_slots)]
    ml = f[:n_ml * 4].view(torch.float32).view(BH, n_slots, G, 2)
    o = f[o_off:o_off + BH * n_slots * G * 128 * 4].view(torch.float32).view(BH, n_slots, G, 128)
    return ml, o


def decode_combine(ws, batch, n_kv_heads, n_q_heads, n_slots, out=None, stream=None):
    """kvq_decode_combine: the partial slots in ws -> out [B][Hq][128] float32."""
    import torch
    if out is None:
        out = torch.empty((batch, n_q_heads, 128), dtype=torch.float32, device=ws.device)
    st = load().kvq_decode_combine(_ptr(ws), ws.numel(), batch, n_kv_heads, n_q_heads, n_slots, _ptr(out),
                                   _stream_ptr(stream))
    _check(st, "kvq_decode_combine")
    return out


def tile_bytes(bits: int) -> int:
    return int(load().kvq_tile_bytes(bits))


def value_tile_bytes(bits: int) -> int:
    return int(load().kvq_value_tile_bytes(bits))


class PackedCache:
    """Device buffers of one block's packed cache plus the kvq_cache struct.

    layout="contiguous": tiles at ((b*H + h)*max_tiles + g) * stride (stride =
    tile size at the initial widths); layout="pool": one code pool of
    pool_bytes with per-tile offset tables managed by a kvq_pool.
    """

    def __init__(self, batch, n_kv_heads, max_tokens, k_bits, v_bits, param_dtype=F16,
                 slot_chan=None, device="cuda", layout="contiguous", pool_bytes=None, v_slot_chan=None):
        import torch
        load()
        self.device = torch.device(device)
        self.B, self.H, self.max_tokens = batch, n_kv_heads, max_tokens
        self.max_tiles = max_tokens // 128
        self.pdt = param_dtype
        pb = PARAM_BYTES[param_dtype]
        u8 = dict(dtype=torch.uint8, device=self.device)
        s = KvqCacheStruct()
        s.batch, s.n_kv_heads, s.head_dim, s.group = batch, n_kv_heads, 128, 128
        s.max_tokens, s.n_tokens = max_tokens, 0
        s.k_bits, s.v_bits, s.param_dtype, s.reserved0 = k_bits, v_bits, param_dtype, 0
        n_streams = batch * n_kv_heads
        self.layout = layout
        self.pool = None
        if layout == "contiguous":
            self.k_stride = tile_bytes(k_bits)
            self.v_stride = value_tile_bytes(v_bits)
            self.k_codes = torch.zeros(n_streams * self.max_tiles * self.k_stride, **u8)
            self.v_codes = torch.zeros(n_streams * self.max_tiles * self.v_stride, **u8)
            s.k_codes, s.v_codes = self.k_codes.data_ptr(), self.v_codes.data_ptr()
            s.k_tile_off = s.v_tile_off = None
            s.k_tile_stride, s.v_tile_stride = self.k_stride, self.v_stride
            self.k_off = self.v_off = None
        elif layout == "pool":
            assert pool_bytes is not None
            self.k_codes = torch.zeros(pool_bytes, **u8)
            self.v_codes = self.k_codes
            s.k_codes = s.v_codes = self.k_codes.data_ptr()
            self.k_off = torch.full((self.max_tiles * n_streams,), -1, dtype=torch.int64,
                                    device=self.device)
            self.v_off = torch.full_like(self.k_off, -1)
            s.k_tile_off, s.v_tile_off = self.k_off.data_ptr(), self.v_off.data_ptr()
            s.k_tile_stride = s.v_tile_stride = 0
        else:
            raise ValueError(layout)
        self.k_scale = torch.zeros(n_streams * self.max_tiles * 128 * pb, **u8)
        self.k_zero = torch.zeros_like(self.k_scale)
        self.v_classes = 4 if v_bits == VMIXED else 1
        self.v_scale = torch.zeros(n_streams * self.v_classes * max_tokens * pb, **u8)
        self.v_zero = torch.zeros_like(self.v_scale)
        s.k_scale, s.k_zero = self.k_scale.data_ptr(), self.k_zero.data_ptr()
        s.v_scale, s.v_zero = self.v_scale.data_ptr(), self.v_zero.data_ptr()
        self.slot_chan = None
        if slot_chan is not None:
            self.slot_chan = torch.as_tensor(np.ascontiguousarray(slot_chan, dtype=np.int16),
                                             device=self.device)
            s.k_slot_chan = self.slot_chan.data_ptr()
        else:
            s.k_slot_chan = None
        self.v_slot_chan = None
        s.v_slot_chan = None
        if v_slot_chan is not None:
            self.v_slot_chan = torch.as_tensor(np.ascontiguousarray(v_slot_chan, dtype=np.int16),
                                               device=self.device)
            s.v_slot_chan = self.v_slot_chan.data_ptr()
        self.s = s
        self._ws = {}
        if layout == "pool":
            h = ctypes.c_void_p()
            _check(load().kvq_pool_create(ctypes.byref(s), pool_bytes, _ptr(self.k_off),
                                          _ptr(self.v_off), ctypes.byref(h)), "kvq_pool_create")
            self.pool = h

    def __del__(self):
        try:
            if self.pool is not None and _lib is not None:
                _lib.kvq_pool_destroy(self.pool)
                self.pool = None
        except Exception:
            pass

    def clone(self):
        """A copy of the cache's device contents and widths, for decode only
        (e.g. to rotate cold copies): a pool-layout clone keeps the tile
        tables but no pool, so appends to it are rejected."""
        import torch
        c = PackedCache.__new__(PackedCache)
        c.device, c.B, c.H, c.max_tokens = self.device, self.B, self.H, self.max_tokens
        c.max_tiles, c.pdt, c.layout, c.pool, c._ws = self.max_tiles, self.pdt, self.layout, None, {}
        c.v_classes = self.v_classes
        s = KvqCacheStruct()
        ctypes.pointer(s)[0] = self.s
        c.k_codes = self.k_codes.clone()
        c.v_codes = c.k_codes if self.v_codes is self.k_codes else self.v_codes.clone()
        s.k_codes, s.v_codes = c.k_codes.data_ptr(), c.v_codes.data_ptr()
        if self.layout == "contiguous":
            c.k_stride, c.v_stride = self.k_stride, self.v_stride
            c.k_off = c.v_off = None
        else:
            c.k_off, c.v_off = self.k_off.clone(), self.v_off.clone()
            s.k_tile_off, s.v_tile_off = c.k_off.data_ptr(), c.v_off.data_ptr()
        for name in ("k_scale", "k_zero", "v_scale", "v_zero"):
            setattr(c, name, getattr(self, name).clone())
        s.k_scale, s.k_zero = c.k_scale.data_ptr(), c.k_zero.data_ptr()
        s.v_scale, s.v_zero = c.v_scale.data_ptr(), c.v_zero.data_ptr()
        c.slot_chan = None if self.slot_chan is None else self.slot_chan.clone()
        s.k_slot_chan = None if c.slot_chan is None else c.slot_chan.data_ptr()
        c.v_slot_chan = None if self.v_slot_chan is None else self.v_slot_chan.clone()
        s.v_slot_chan = None if c.v_slot_chan is None else c.v_slot_chan.data_ptr()
        c.s = s
        return c

    # -- state ----------------------------------------------------------------
    @property
    def n_tokens(self):
        return self.s.n_tokens

    @property
    def k_bits(self):
        return self.s.k_bits

    @property
    def v_bits(self):
        return self.s.v_bits

    def cache_bytes(self, n_tokens=None, k_bits=None, v_bits=None):
        return int(load().kvq_cache_bytes(ctypes.byref(self.s),
                                          self.n_tokens if n_tokens is None else n_tokens,
                                          self.k_bits if k_bits is None else k_bits,
                                          self.v_bits if v_bits is None else v_bits))

    def pool_used(self):
        return int(load().kvq_pool_used_bytes(self.pool))

    def pool_high_water(self):
        return int(load().kvq_pool_high_water(self.pool))

    # -- operations -----------------------------------------------------------
    def quantize(self, k, v, t0=0, stream=None):
        """k, v: [B][H][n_new][128] float32 or bfloat16 device tensors (either may be None)."""
        import torch
        ref = k if k is not None else v
        in_dtype = {torch.float32: F32, torch.bfloat16: BF16}[ref.dtype]
        n_new = ref.shape[2]
        st = load().kvq_quantize(ctypes.byref(self.s), _ptr(k), _ptr(v), in_dtype,
                                 _strides3(k) if k is not None else None,
                                 _strides3(v) if v is not None else None,
                                 t0, n_new, _stream_ptr(stream))
        _check(st, "kvq_quantize")

    def shrink(self, to_bits, stream=None, method=SHIFT_ERS):
        if method == SHIFT_ERS:
            _check(load().kvq_shrink(ctypes.byref(self.s), to_bits, _stream_ptr(stream)), "kvq_shrink")
        else:
            _check(load().kvq_shrink_shift(ctypes.byref(self.s), to_bits, method, _stream_ptr(stream)),
                   "kvq_shrink_shift")

    def append(self, k, v, budget_bytes, floor_bits, stream=None):
        import torch
        in_dtype = {torch.float32: F32, torch.bfloat16: BF16}[k.dtype]
        n = ctypes.c_int32(0)
        st = load().kvq_append(ctypes.byref(self.s), self.pool, budget_bytes, floor_bits,
                               _ptr(k), _ptr(v), in_dtype, _strides3(k), _strides3(v),
                               k.shape[2], _stream_ptr(stream), ctypes.byref(n))
        _check(st, "kvq_append")
        return n.value

    def workspace_bytes(self, n_q_heads):
        return int(load().kvq_decode_workspace_bytes(ctypes.byref(self.s), n_q_heads))

    def workspace(self, n_q_heads):
        import torch
        if n_q_heads not in self._ws:
            nb = self.workspace_bytes(n_q_heads)
            if nb == 0:
                raise KvqError(EINVAL, "kvq_decode_workspace_bytes")
            self._ws[n_q_heads] = torch.zeros(nb, dtype=torch.uint8, device=self.device)
        return self._ws[n_q_heads]

    def decode_attn(self, q, softmax_scale, out=None, workspace=None, stream=None, res_k=None,
                    res_v=None):
        """q: [B][Hq][128] bfloat16 device tensor -> out [B][Hq][128] float32.
        res_k, res_v: optional residual segment [B][Hkv][R][128] (float32,
        float16 or bfloat16, unit channel stride) attended with the packed
        tokens."""
        import torch
        assert q.dtype == torch.bfloat16 and q.is_contiguous()
        Hq = q.shape[1]
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        ws = workspace if workspace is not None else self.workspace(Hq)
        if res_k is None:
            st = load().kvq_decode_attn(ctypes.byref(self.s), _ptr(q), Hq, float(softmax_scale),
                                        _ptr(out), _ptr(ws), ws.numel(), _stream_ptr(stream))
            _check(st, "kvq_decode_attn")
            return out
        assert res_v is not None and res_k.dtype == res_v.dtype and res_k.shape == res_v.shape
        rdt = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}[res_k.dtype]
        st = load().kvq_decode_attn_residual(ctypes.byref(self.s), _ptr(q), Hq, float(softmax_scale),
                                             _ptr(res_k), _ptr(res_v), rdt, _strides3(res_k),
                                             _strides3(res_v), res_k.shape[2], _ptr(out), _ptr(ws),
                                             ws.numel(), _stream_ptr(stream))
        _check(st, "kvq_decode_attn_residual")
        return out

    def decode_partials(self, q, softmax_scale, workspace=None, stream=None):
        """kvq_decode_attn_partials: the chunk partials of the packed cache in
        workspace -> (n_slots, tiles_per_slot)."""
        import torch
        assert q.dtype == torch.bfloat16 and q.is_contiguous()
        ws = workspace if workspace is not None else self.workspace(q.shape[1])
        ns, tps = ctypes.c_int32(0), ctypes.c_int32(0)
        st = load().kvq_decode_attn_partials(ctypes.byref(self.s), _ptr(q), q.shape[1], float(softmax_scale),
                                             _ptr(ws), ws.numel(), ctypes.byref(ns), ctypes.byref(tps),
                                             _stream_ptr(stream))
        _check(st, "kvq_decode_attn_partials")
        return ns.value, tps.value

    def quantize_tokens(self, k, v, tok, t0=0, stream=None):
        """kvq_quantize_tokens: k, v [B][H][n_src][128] float32 / bfloat16
        device tensors, tok [B][H][n_new] int32 device tensor of input rows."""
        import torch
        ref = k if k is not None else v
        in_dtype = {torch.float32: F32, torch.bfloat16: BF16}[ref.dtype]
        assert tok.dtype == torch.int32 and tok.is_contiguous() and tok.shape[:2] == (self.B, self.H)
        st = load().kvq_quantize_tokens(ctypes.byref(self.s), _ptr(k), _ptr(v), in_dtype,
                                        _strides3(k) if k is not None else None,
                                        _strides3(v) if v is not None else None,
                                        _ptr(tok), ref.shape[2], t0, tok.shape[2], _stream_ptr(stream))
        _check(st, "kvq_quantize_tokens")

    def decode_attn_noalloc(self, q, softmax_scale, out=None, stream=None):
        """kvq_decode_attn_noalloc: decode attention with the library's own
        scratch array instead of a workspace (nothing is allocated by the
        call; out must be given to avoid the allocation here as well)."""
        import torch
        assert q.dtype == torch.bfloat16 and q.is_contiguous()
        if out is None:
            out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
        st = load().kvq_decode_attn_noalloc(ctypes.byref(self.s), _ptr(q), q.shape[1], float(softmax_scale),
                                            _ptr(out), _stream_ptr(stream))
        _check(st, "kvq_decode_attn_noalloc")
        return out

    # -- host views for tests --------------------------------------------------
    def k_tile(self, b, h, g):
        """bytes of key tile (b, h, g) at the current width (host numpy)."""
        n = tile_bytes(self.k_bits)
        off = self._tile_off(self.k_off, self.k_stride if self.layout == "contiguous" else 0,
                             b, h, g)
        return self.k_codes[off:off + n].cpu().numpy()

    def v_tile(self, b, h, g):
        n = value_tile_bytes(self.v_bits)
        off = self._tile_off(self.v_off, self.v_stride if self.layout == "contiguous" else 0,
                             b, h, g)
        return self.v_codes[off:off + n].cpu().numpy()

    def _tile_off(self, table, stride, b, h, g):
        if table is None:
            return ((b * self.H + h) * self.max_tiles + g) * stride
        return int(table[(g * self.B + b) * self.H + h].item())

    def k_params(self, b, h):
        """(S raw, Z raw) of stream (b, h) for stored tiles: [n_tiles, 128] numpy."""
        pb = PARAM_BYTES[self.pdt]
        nt = self.n_tokens // 128
        base = ((b * self.H + h) * self.max_tiles) * 128 * pb
        npdt = {F32: np.float32, F16: np.uint16, BF16: np.uint16, E4M3: np.uint8}[self.pdt]
        sl = slice(base, base + nt * 128 * pb)
        return (self.k_scale[sl].cpu().numpy().view(npdt).reshape(nt, 128),
                self.k_zero[sl].cpu().numpy().view(npdt).reshape(nt, 128))

    def v_params(self, b, h):
        """(S raw, Z raw) of stream (b, h)'s stored tokens: [n_tokens] numpy,
        or [4][n_tokens] (class-major) for mixed values."""
        pb = PARAM_BYTES[self.pdt]
        nc, T = self.v_classes, self.max_tokens
        npdt = {F32: np.float32, F16: np.uint16, BF16: np.uint16, E4M3: np.uint8}[self.pdt]
        out = []
        for arr in (self.v_scale, self.v_zero):
            base = (b * self.H + h) * nc * T * pb
            a = arr[base:base + nc * T * pb].cpu().numpy().view(npdt).reshape(nc, T)[:, :self.n_tokens]
            out.append(a if nc > 1 else a[0])
        return tuple(out)


class Window:
    """The unpacked tokens of every stream of one cache (kvq_window of the
    header): row 0 the first token (keep_first), rows 1..n_recent the recent
    tokens not yet packed.  append() hands every full 128-token group to the
    cache; residual() gives the views decode_attn attends with the cache."""

    def __init__(self, cache, dtype=None, keep_first=True):
        import torch
        load()
        dtype = torch.bfloat16 if dtype is None else dtype
        self.cache = cache
        self.dtype = dtype
        shape = (cache.B, cache.H, WINDOW_ROWS, 128)
        self.k = torch.zeros(shape, dtype=dtype, device=cache.device)
        self.v = torch.zeros_like(self.k)
        w = KvqWindowStruct()
        w.batch, w.n_kv_heads = cache.B, cache.H
        w.dtype = {torch.float32: F32, torch.bfloat16: BF16}[dtype]
        w.keep_first = 1 if keep_first else 0
        w.k, w.v = self.k.data_ptr(), self.v.data_ptr()
        w.n_first = w.n_recent = 0
        self.w = w

    @property
    def n_first(self):
        return self.w.n_first

    @property
    def n_recent(self):
        return self.w.n_recent

    def append(self, k, v, budget_bytes=-1, floor_bits=1, stream=None):
        """k, v: [B][H][n][128] device tensors of the window's dtype, unit
        channel stride.  budget_bytes < 0: groups are packed at the cache's
        widths; otherwise under the budget (progressive halvings, returned)."""
        assert k.dtype == self.dtype and v.dtype == self.dtype and k.shape == v.shape
        n = ctypes.c_int32(0)
        c = self.cache
        if budget_bytes < 0 and c.layout == "pool":
            # the pool's offset tables hold no tiles for the new groups
            raise ValueError("a pool-layout cache takes groups under a budget")
        st = load().kvq_window_append(ctypes.byref(self.w), ctypes.byref(c.s),
                                      c.pool if budget_bytes >= 0 else None, budget_bytes, floor_bits,
                                      _ptr(k), _ptr(v), _strides3(k), _strides3(v), k.shape[2],
                                      _stream_ptr(stream), ctypes.byref(n))
        _check(st, "kvq_window_append")
        return n.value

    def residual(self):
        """(res_k, res_v) views over the held rows, for decode_attn."""
        lo = 1 - self.w.n_first
        hi = 1 + self.w.n_recent
        return self.k[:, :, lo:hi], self.v[:, :, lo:hi]

