"""CPU oracle for packed KV quantization, ERS shrink and decode attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` import this package.  The product library never
loads it and shares no code with it; the two meet only through the seeded
input generators and the layout text of the public header.

The arithmetic lives in ``kvq_oracle.c`` (plain C, single-threaded, binary32
quantizer with one rounding per operation, binary64 attention).  This module
builds it with gcc, loads it with ctypes and offers numpy-level wrappers that
work on one (batch, kv-head) stream at a time.

Sources, cited by page title and section:
  * "PM-KVQ: Progressive Mixed-Precision KV Cache Quantization for Long-CoT
    LLMs" (papernotes.org summary) -- Key design 1 (ERS equation, progressive
    16->8->4->2 schedule), Training strategy (asymmetric groups of 128).
  * "Channel-Aware Mixed-Precision Quantization for Efficient Long-Context
    Inference" (papernotes.org summary) -- Background (key channel-wise, value
    token-wise), Key design 1 (S = (Cmax - Cmin)/(2^b - 1), Emax = S/2), Key
    design 3 (4/3/2/1-bit classes in 8-bit-aligned blocks, fp8 parameters).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_kvq_oracle.so")

F32, F16, BF16, E4M3 = 0, 1, 2, 3
PARAM_NP = {F32: np.float32, F16: np.uint16, BF16: np.uint16, E4M3: np.uint8}
PARAM_BYTES = {F32: 4, F16: 2, BF16: 2, E4M3: 1}
MIXED_TILE_BYTES = 4352
VMIXED_TILE_BYTES = 5120

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build()
            L = ctypes.CDLL(_LIB_PATH)
            vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
            L.orc_f32_to_f16.restype = ctypes.c_uint16
            L.orc_f32_to_f16.argtypes = [ctypes.c_float]
            L.orc_f32_to_e4m3.restype = ctypes.c_uint8
            L.orc_f32_to_e4m3.argtypes = [ctypes.c_float]
            L.orc_ers.restype = ctypes.c_uint32
            L.orc_ers.argtypes = [ctypes.c_uint32, i32]
            L.orc_narrow_array.argtypes = [vp, i64, i32, vp]
            L.orc_decode_array.argtypes = [vp, i64, i32, vp]
            L.orc_ers_array.argtypes = [vp, i64, i32, vp]
            L.orc_quantize_group.argtypes = [vp, i64, i32, i32, i32, vp, i64, vp, vp, i64]
            L.orc_pack_rows.argtypes = [vp, i32, vp]
            L.orc_unpack_rows.argtypes = [vp, i32, vp]
            L.orc_pack_vtile.argtypes = [vp, i32, vp]
            L.orc_unpack_vtile.argtypes = [vp, i32, vp]
            L.orc_shrink_vtile.argtypes = [vp, i32]
            L.orc_pack_mixed.argtypes = [vp, vp]
            L.orc_unpack_mixed.argtypes = [vp, vp]
            L.orc_mixed_slot_bits.restype = i32
            L.orc_mixed_slot_bits.argtypes = [i32]
            L.orc_quantize_k.argtypes = [vp, i64, i32, i32, i32, vp, i64, vp, vp]
            L.orc_quantize_k_mixed.argtypes = [vp, i64, i32, i32, vp, vp, i64, vp, vp]
            L.orc_quantize_v.argtypes = [vp, i64, i32, i32, i32, vp, i64, vp, vp]
            L.orc_shrink_tile.argtypes = [vp, i32]
            L.orc_shrink_scales.argtypes = [vp, i64, i32, i32]
            L.orc_shrink_tile_m.argtypes = [vp, i32, i32]
            L.orc_shrink_vtile_m.argtypes = [vp, i32, i32]
            L.orc_shrink_scales_m.argtypes = [vp, i64, i32, i32, i32]
            L.orc_shift_array.argtypes = [vp, i64, i32, i32, vp]
            L.orc_decode_attn.restype = i32
            L.orc_pack_vmixed.argtypes = [vp, vp]
            L.orc_unpack_vmixed.argtypes = [vp, vp]
            L.orc_vmixed_slot_bits.restype = i32
            L.orc_vmixed_slot_bits.argtypes = [i32]
            L.orc_quantize_v_mixed.argtypes = [vp, i64, i32, i32, vp, vp, i64, vp, vp]
            L.orc_decode_attn.argtypes = [vp, i64, vp, vp, i32, vp, vp, i64, vp, vp, i32, vp,
                                          i32, i32, vp, i32, ctypes.c_float, vp]
            L.orc_block_bytes.restype = i64
            L.orc_block_bytes.argtypes = [i32, i32, i64, i32, i32, i32]
            L.orc_schedule.restype = i32
            L.orc_schedule.argtypes = [i32, i32, i64, i32, i32, i32, i64, vp, i32]
            _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"] or a.ndim == 0
    return ctypes.c_void_p(a.ctypes.data)


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------
def narrow(x: np.ndarray, pdt: int) -> np.ndarray:
    """binary32 -> raw bits of the parameter dtype (RNE; e4m3 saturates)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=PARAM_NP[pdt])
    lib().orc_narrow_array(_p(x), x.size, pdt, _p(out))
    return out


def decode(raw: np.ndarray, pdt: int) -> np.ndarray:
    """raw bits of a parameter dtype -> exact float64 values."""
    raw = np.ascontiguousarray(raw, dtype=PARAM_NP[pdt])
    out = np.empty(raw.shape, dtype=np.float64)
    lib().orc_decode_array(_p(raw), raw.size, pdt, _p(out))
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """binary32 -> bfloat16 raw bits (RNE)."""
    return narrow(x, BF16)


SHIFT_ERS, SHIFT_DIRECT, SHIFT_MODIFIED = 0, 1, 2


def shift(x: np.ndarray, b: int, method: int) -> np.ndarray:
    """2b-bit codes -> b bits by a halving rule of the ablation (0 ERS, 1
    direct right shift, 2 modified (rounded, clamped) right shift)."""
    x = np.ascontiguousarray(x, dtype=np.uint32)
    out = np.empty_like(x)
    lib().orc_shift_array(_p(x), x.size, b, method, _p(out))
    return out


def ers(x: np.ndarray, b: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint32)
    out = np.empty_like(x)
    lib().orc_ers_array(_p(x), x.size, b, _p(out))
    return out


# --------------------------------------------------------------------------
# quantizer, packing
# --------------------------------------------------------------------------
def quantize_group(x: np.ndarray, bits: int, pdt: int):
    """One group -> (codes uint16, S raw, Z raw)."""
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    codes = np.empty(x.size, dtype=np.uint16)
    s = np.empty(1, dtype=PARAM_NP[pdt])
    z = np.empty(1, dtype=PARAM_NP[pdt])
    lib().orc_quantize_group(_p(x), 1, x.size, bits, pdt, _p(codes), 1, _p(s), _p(z), 0)
    return codes, s[0], z[0]


def pack_rows(codes: np.ndarray, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint16).reshape(128, 128)
    tile = np.zeros(16 * bits * 128, dtype=np.uint8)
    lib().orc_pack_rows(_p(codes), bits, _p(tile))
    return tile


def unpack_rows(tile: np.ndarray, bits: int) -> np.ndarray:
    tile = np.ascontiguousarray(tile, dtype=np.uint8)
    assert tile.size >= 16 * bits * 128
    codes = np.empty((128, 128), dtype=np.uint16)
    lib().orc_unpack_rows(_p(tile), bits, _p(codes))
    return codes


def pack_vtile(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes[c][t] -> value tile (word planes W[w][c][a])"""
    codes = np.ascontiguousarray(codes, dtype=np.uint16).reshape(128, 128)
    tile = np.zeros(16 * bits * 128, dtype=np.uint8)
    lib().orc_pack_vtile(_p(codes), bits, _p(tile))
    return tile


def unpack_vtile(tile: np.ndarray, bits: int) -> np.ndarray:
    tile = np.ascontiguousarray(tile, dtype=np.uint8)
    assert tile.size >= 16 * bits * 128
    codes = np.empty((128, 128), dtype=np.uint16)
    lib().orc_unpack_vtile(_p(tile), bits, _p(codes))
    return codes


def pack_mixed(codes: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint16).reshape(128, 128)
    tile = np.zeros(MIXED_TILE_BYTES, dtype=np.uint8)
    lib().orc_pack_mixed(_p(codes), _p(tile))
    return tile


def unpack_mixed(tile: np.ndarray) -> np.ndarray:
    tile = np.ascontiguousarray(tile, dtype=np.uint8)
    assert tile.size >= MIXED_TILE_BYTES
    codes = np.empty((128, 128), dtype=np.uint16)
    lib().orc_unpack_mixed(_p(tile), _p(codes))
    return codes


def pack_vmixed(codes: np.ndarray) -> np.ndarray:
    """codes[slot][t] (128 x 128) -> 5120-byte mixed-width value tile"""
    codes = np.ascontiguousarray(codes, dtype=np.uint16).reshape(128, 128)
    tile = np.zeros(VMIXED_TILE_BYTES, dtype=np.uint8)
    lib().orc_pack_vmixed(_p(codes), _p(tile))
    return tile


def unpack_vmixed(tile: np.ndarray) -> np.ndarray:
    tile = np.ascontiguousarray(tile, dtype=np.uint8)
    assert tile.size >= VMIXED_TILE_BYTES
    codes = np.empty((128, 128), dtype=np.uint16)
    lib().orc_unpack_vmixed(_p(tile), _p(codes))
    return codes


def vmixed_slot_bits() -> np.ndarray:
    return np.array([lib().orc_vmixed_slot_bits(j) for j in range(128)], dtype=np.int32)


def mixed_slot_bits() -> np.ndarray:
    return np.array([lib().orc_mixed_slot_bits(j) for j in range(128)], dtype=np.int32)


def tile_bytes(bits: int) -> int:
    """bytes of one packed tile; bits == 0 selects the mixed-bit key tile"""
    return MIXED_TILE_BYTES if bits == 0 else 2048 * bits


# --------------------------------------------------------------------------
# one (batch, kv-head) stream
# --------------------------------------------------------------------------
class Stream:
    """Packed cache of one (batch, kv-head) stream, as the oracle builds it.

    k_tiles: [n_tiles, tile_bytes(k_bits)] uint8, ks/kz: [n_tiles, 128] raw
    v_tiles: [n_tiles, 2048*v_bits] uint8, vs/vz: [n_tok] raw
    """

    def __init__(self, k_bits, v_bits, pdt, k_tiles, ks, kz, v_tiles, vs, vz, slot_chan=None, v_slot_chan=None):
        self.v_slot_chan = v_slot_chan
        self.k_bits, self.v_bits, self.pdt = k_bits, v_bits, pdt
        self.k_tiles, self.ks, self.kz = k_tiles, ks, kz
        self.v_tiles, self.vs, self.vz = v_tiles, vs, vz
        self.slot_chan = slot_chan

    @property
    def n_tok(self):
        return self.k_tiles.shape[0] * 128


def quantize_stream(k: np.ndarray, v: np.ndarray, k_bits: int, v_bits: int, pdt: int,
                    slot_chan: np.ndarray | None = None, v_slot_chan: np.ndarray | None = None) -> Stream:
    """k, v: [T, 128] float32 (T multiple of 128).  k_bits == 0 -> mixed keys."""
    k = np.ascontiguousarray(k, dtype=np.float32)
    v = np.ascontiguousarray(v, dtype=np.float32)
    T = k.shape[0]
    assert k.shape == (T, 128) and v.shape == (T, 128) and T % 128 == 0
    nt = T // 128
    L = lib()
    kt = np.zeros((nt, tile_bytes(k_bits)), dtype=np.uint8)
    ks = np.empty((nt, 128), dtype=PARAM_NP[pdt])
    kz = np.empty((nt, 128), dtype=PARAM_NP[pdt])
    if k_bits == 0:
        sc = np.ascontiguousarray(slot_chan, dtype=np.int16)
        assert sc.shape == (128,) and sorted(sc.tolist()) == list(range(128))
        L.orc_quantize_k_mixed(_p(k), 128, T, pdt, _p(sc), _p(kt), kt.shape[1], _p(ks), _p(kz))
    else:
        sc = None
        L.orc_quantize_k(_p(k), 128, T, k_bits, pdt, _p(kt), kt.shape[1], _p(ks), _p(kz))
    if v_bits == 0:
        # value channel classes (4/3/1/2 bits), one group per (token, class)
        vsc = np.ascontiguousarray(v_slot_chan, dtype=np.int16)
        assert vsc.shape == (128,) and sorted(vsc.tolist()) == list(range(128))
        vt = np.zeros((nt, VMIXED_TILE_BYTES), dtype=np.uint8)
        vs = np.empty((4, T), dtype=PARAM_NP[pdt])      # [class][token]
        vz = np.empty((4, T), dtype=PARAM_NP[pdt])
        L.orc_quantize_v_mixed(_p(v), 128, T, pdt, _p(vsc), _p(vt), vt.shape[1], _p(vs), _p(vz))
        return Stream(k_bits, v_bits, pdt, kt, ks, kz, vt, vs, vz, sc, vsc)
    vt = np.zeros((nt, tile_bytes(v_bits)), dtype=np.uint8)
    vs = np.empty(T, dtype=PARAM_NP[pdt])
    vz = np.empty(T, dtype=PARAM_NP[pdt])
    L.orc_quantize_v(_p(v), 128, T, v_bits, pdt, _p(vt), vt.shape[1], _p(vs), _p(vz))
    return Stream(k_bits, v_bits, pdt, kt, ks, kz, vt, vs, vz, sc)


def shrink_stream(st: Stream, to_bits: int, method: int = SHIFT_ERS) -> Stream:
    """2b -> b of every tile of a uniform-width stream (returns a new Stream);
    method: 0 ERS, 1 direct right shift, 2 modified right shift."""
    assert st.k_bits == 2 * to_bits and st.v_bits == 2 * to_bits
    L = lib()
    out = []
    for tiles, fn in ((st.k_tiles, L.orc_shrink_tile_m), (st.v_tiles, L.orc_shrink_vtile_m)):
        t2 = np.array(tiles, copy=True)
        for i in range(t2.shape[0]):
            row = np.ascontiguousarray(t2[i])
            fn(_p(row), to_bits, method)
            t2[i] = row
        out.append(np.ascontiguousarray(t2[:, : tile_bytes(to_bits)]))
    ks = np.array(st.ks, copy=True)
    vs = np.array(st.vs, copy=True)
    L.orc_shrink_scales_m(_p(ks), ks.size, to_bits, st.pdt, method)
    L.orc_shrink_scales_m(_p(vs), vs.size, to_bits, st.pdt, method)
    return Stream(to_bits, to_bits, st.pdt, out[0], ks, st.kz.copy(), out[1], vs, st.vz.copy(),
                  st.slot_chan)


def dequant_k(st: Stream) -> np.ndarray:
    """[T, 128] float64 keys (channel order) reconstructed from the stream."""
    nt = st.k_tiles.shape[0]
    S = decode(st.ks, st.pdt)
    Z = decode(st.kz, st.pdt)
    out = np.empty((nt * 128, 128), dtype=np.float64)
    for g in range(nt):
        if st.k_bits == 0:
            codes = unpack_mixed(st.k_tiles[g]).astype(np.float64)  # [t][slot]
            val = codes * S[g][None, :] + Z[g][None, :]
            blk = np.empty_like(val)
            blk[:, st.slot_chan.astype(np.int64)] = val
        else:
            codes = unpack_rows(st.k_tiles[g], st.k_bits).astype(np.float64)  # [t][c]
            blk = codes * S[g][None, :] + Z[g][None, :]
        out[g * 128:(g + 1) * 128] = blk
    return out


def dequant_v(st: Stream) -> np.ndarray:
    nt = st.v_tiles.shape[0]
    S = decode(st.vs, st.pdt)
    Z = decode(st.vz, st.pdt)
    out = np.empty((nt * 128, 128), dtype=np.float64)
    if st.v_bits == 0:
        cls = np.array([0] * 16 + [1] * 16 + [2] * 16 + [3] * 80)
        for g in range(nt):
            codes = unpack_vmixed(st.v_tiles[g]).astype(np.float64)         # [slot][t]
            Sg, Zg = S[:, g * 128:(g + 1) * 128].T, Z[:, g * 128:(g + 1) * 128].T   # [t][class]
            val = codes.T * Sg[:, cls] + Zg[:, cls]                         # [t][slot]
            out[g * 128:(g + 1) * 128][:, st.v_slot_chan.astype(np.int64)] = val
        return out
    for g in range(nt):
        codes = unpack_vtile(st.v_tiles[g], st.v_bits).astype(np.float64)  # [c][t]
        out[g * 128:(g + 1) * 128] = codes.T * S[g * 128:(g + 1) * 128, None] + \
            Z[g * 128:(g + 1) * 128, None]
    return out


def decode_attn(st: Stream, q_bf16: np.ndarray, scale: float) -> np.ndarray:
    """q_bf16: [G, 128] uint16 raw bfloat16 -> [G, 128] float64."""
    q = np.ascontiguousarray(q_bf16, dtype=np.uint16)
    G = q.shape[0]
    out = np.empty((G, 128), dtype=np.float64)
    sc = st.slot_chan if st.slot_chan is not None else np.zeros(128, dtype=np.int16)
    sc = np.ascontiguousarray(sc, dtype=np.int16)
    vsc = st.v_slot_chan if st.v_slot_chan is not None else np.zeros(128, dtype=np.int16)
    vsc = np.ascontiguousarray(vsc, dtype=np.int16)
    kt = np.ascontiguousarray(st.k_tiles)
    vt = np.ascontiguousarray(st.v_tiles)
    rc = lib().orc_decode_attn(_p(kt), kt.shape[1], _p(np.ascontiguousarray(st.ks)),
                               _p(np.ascontiguousarray(st.kz)), st.k_bits, _p(sc),
                               _p(vt), vt.shape[1], _p(np.ascontiguousarray(st.vs)),
                               _p(np.ascontiguousarray(st.vz)), st.v_bits, _p(vsc), st.pdt, st.n_tok,
                               _p(q), G, ctypes.c_float(scale), _p(out))
    if rc != 0:
        raise RuntimeError("orc_decode_attn failed: %d" % rc)
    return out


def decode_attn_residual(st, q_bf16: np.ndarray, scale: float, res_k: np.ndarray,
                         res_v: np.ndarray) -> np.ndarray:
    """Attention of the G query heads over the packed stream's reconstructed
    tokens followed by residual tokens kept at full precision (PM-KVQ page,
    Training strategy and Related work: first / recent tokens not quantized).
    Written as its plain definition in float64: dequantize, concatenate,
    softmax(sigma * q K^T) V.  st may be None (no packed tokens).
    res_k, res_v: [R, 128] real values (bfloat16 inputs are widened exactly by
    the caller)."""
    qf = decode(np.ascontiguousarray(q_bf16, dtype=np.uint16), BF16)
    parts_k, parts_v = [], []
    if st is not None and st.n_tok > 0:
        parts_k.append(dequant_k(st))
        parts_v.append(dequant_v(st))
    parts_k.append(np.asarray(res_k, dtype=np.float64))
    parts_v.append(np.asarray(res_v, dtype=np.float64))
    K = np.concatenate(parts_k)
    V = np.concatenate(parts_v)
    sigma = float(np.float32(scale))
    s = sigma * (qf @ K.T)                                           # [G, T]
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ V


# --------------------------------------------------------------------------
# per-token split between two precisions ("SemKV: Semantic Mixed-Precision KV
# Cache Quantization ...", abstract: every token is kept; tokens are ranked by
# a model-internal score and given one of two adjacent precisions)
# --------------------------------------------------------------------------
def rank_tokens(score, n_high: int) -> np.ndarray:
    """score [S][T] -> order [S][T]: per stream, the n_high tokens with the
    largest scores (a larger score ranks first; equal scores, the earlier
    token first) in ascending token order, then the other tokens in
    ascending order.  Plain Python sort on (-score, token)."""
    out = []
    for sc in np.asarray(score, dtype=np.float32):
        ranked = sorted(range(len(sc)), key=lambda t: (-float(sc[t]), t))
        out.append(sorted(ranked[:n_high]) + sorted(ranked[n_high:]))
    return np.array(out, dtype=np.int64)


def decode_attn_union(streams, q_bf16: np.ndarray, scale: float) -> np.ndarray:
    """Attention of the G query heads over the union of several packed
    streams' reconstructed tokens (the same kv head's tokens split between
    caches).  Written as its plain definition in float64: dequantize every
    stream, concatenate, softmax(sigma * q K^T) V.  Streams holding no tokens
    may be None."""
    qf = decode(np.ascontiguousarray(q_bf16, dtype=np.uint16), BF16)
    ks = [dequant_k(st) for st in streams if st is not None and st.n_tok > 0]
    vs = [dequant_v(st) for st in streams if st is not None and st.n_tok > 0]
    K = np.concatenate(ks)
    V = np.concatenate(vs)
    sigma = float(np.float32(scale))
    s = sigma * (qf @ K.T)
    s -= s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    return p @ V


# --------------------------------------------------------------------------
# schedule accounting
# --------------------------------------------------------------------------
def block_bytes(B, H, n_tok, k_bits, v_bits, pdt) -> int:
    return int(lib().orc_block_bytes(B, H, n_tok, k_bits, v_bits, pdt))


def schedule(B, H, n_total, start_bits, floor_bits, pdt, budget):
    """-> list of (tokens stored before the append that triggered it, new width)"""
    ev = np.zeros(64, dtype=np.int64)
    n = lib().orc_schedule(B, H, n_total, start_bits, floor_bits, pdt, budget, _p(ev), 32)
    if n < 0:
        return None
    return [(int(ev[2 * i]), int(ev[2 * i + 1])) for i in range(n)]


# --------------------------------------------------------------------------
# block-wise bit-width allocation (PM-KVQ Key design 2), by enumeration
# --------------------------------------------------------------------------
def allocate_bits_bruteforce(sens, nbytes, budget_bytes):
    """Every choice vector in lexicographic order; the objective is the sum
    s[0][c0] + (s[1][c1] + (... + s[n-1][c_{n-1}])) in binary64 (Python
    float) under sum_i nbytes[i][c_i] <= budget_bytes; the first vector with
    the smallest sum wins.  None if no vector fits.  Small instances only."""
    import itertools
    n, m = len(sens), len(sens[0])
    best, best_cost = None, None
    for cv in itertools.product(range(m), repeat=n):
        if sum(int(nbytes[i][cv[i]]) for i in range(n)) > budget_bytes:
            continue
        c = 0.0
        for i in reversed(range(n)):
            c = float(sens[i][cv[i]]) + c
        if best_cost is None or c < best_cost:
            best, best_cost = cv, c
    return (None, None) if best is None else (list(best), best_cost)



# --------------------------------------------------------------------------
# pair-granular key widths ("PN-Mix: Pair-Norm Guided Mixed-Precision Key
# Cache Quantization ...", abstract: RoPE channel pairs ranked by the product
# of query and key pair norms; the salient pairs get the higher widths)
# --------------------------------------------------------------------------
def pair_norms(x: np.ndarray, group: int = 1) -> np.ndarray:
    """x [B][H][T][128] -> [H // group][64]: for pair p = channels (p, p + 64)
    (rotate-half RoPE pairing), the sum over batch, tokens and the `group`
    consecutive heads of each row of the Euclidean norm of the pair, in
    binary64."""
    x = np.asarray(x, dtype=np.float64)
    B, H, T, D = x.shape
    assert D == 128 and H % group == 0
    norms = np.sqrt(x[..., :64] ** 2 + x[..., 64:] ** 2)        # [B][H][T][64]
    per_head = norms.sum(axis=(0, 2))                            # [H][64]
    return per_head.reshape(H // group, group, 64).sum(axis=1)


def pair_slot_map(score: np.ndarray) -> np.ndarray:
    """score [Hkv][64] -> slot_chan [Hkv][128] int16.  Per kv head, the pairs
    in order of decreasing score (ties: the lower pair index first); the four
    most salient pairs take the 4-bit class, the next four the 3-bit class, the
    four least salient the 1-bit class and the rest the 2-bit class, both
    channels of a pair together.  Slots follow the mixed key layout: 0..7 the
    4-bit channels, 8, 10, .., 22 the 3-bit ones, 9, 11, .., 23 the 1-bit ones,
    24..127 the 2-bit ones, ascending channel order inside each class."""
    score = np.asarray(score, dtype=np.float32)
    out = np.empty((score.shape[0], 128), dtype=np.int16)
    for h in range(score.shape[0]):
        order = sorted(range(64), key=lambda p: (-float(score[h, p]), p))
        classes = {4: [], 3: [], 1: [], 2: []}
        for r, p in enumerate(order):
            width = 4 if r < 4 else (3 if r < 8 else (1 if r >= 60 else 2))
            classes[width] += [p, p + 64]
        c4, c3, c1, c2 = (sorted(classes[w]) for w in (4, 3, 1, 2))
        out[h, 0:8] = c4
        out[h, 8:24:2] = c3
        out[h, 9:24:2] = c1
        out[h, 24:] = c2
    return out
