"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds no quantization, shrink or attention arithmetic: it only
draws keys, values, queries and channel-class maps.  Both the HIP path and the
CPU oracle consume exactly what it returns.

Recipes (stand-ins for real model activations; no dataset or weights are used):
  tiny     1 x 1 kv head x 1 query head, 512 tokens; K, V ~ N(0,1) with key
           channels 3 and 77 scaled x10, then RoPE on K at positions 0..511.
  layer    Qwen2.5-7B-shaped (B=16, Hkv=4, Hq=28, T=32768) and the other GQA
           layers: K ~ N(0,1) pre-RoPE with 4 fixed outlier channels per kv head
           scaled x8, RoPE at the true positions; V ~ N(0,1); q ~ N(0,1) bf16.
  mixed    Llama-3.1-8B-shaped long context (B=1, Hkv=8, Hq=32, T=131072): per kv
           head a seeded permutation picks 8 channels at 4 bits, 8 at 3 bits,
           8 at 1 bit, the other 104 at 2 bits; K ~ N(0,1) with the 3/4-bit
           channels x6 and the 1-bit channels x0.2, no RoPE; V ~ N(0,1).
  pairs    the mixed shape with RoPE-pair saliency: per kv head a seeded
           permutation of the 64 RoPE pairs scales both channels of 4 pairs x8
           and of 4 more x4, and of 4 pairs x0.2; K ~ N(0,1) otherwise, then
           RoPE (which keeps every pair's norm); V ~ N(0,1); the decode query
           and 64 prefill query tokens per head ~ N(0,1) (the prefill queries
           with RoPE at positions 0..63).
RoPE here is rotate-half over channel pairs (i, i+64), theta_i = 1e4^(-2i/128),
angle = position * theta_i, evaluated in float64 and stored as float32.
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 128
ROPE_THETA = 10000.0


def rope_inv_freq(head_dim: int = HEAD_DIM, theta: float = ROPE_THETA) -> np.ndarray:
    i = np.arange(head_dim // 2, dtype=np.float64)
    return theta ** (-2.0 * i / head_dim)


def apply_rope(x: np.ndarray, pos0: int = 0) -> np.ndarray:
    """x: [..., T, 128] float32 -> rotated float32 (rotate-half pairs)."""
    T = x.shape[-2]
    ang = np.arange(pos0, pos0 + T, dtype=np.float64)[:, None] * rope_inv_freq()[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a = x[..., :64].astype(np.float64)
    b = x[..., 64:].astype(np.float64)
    out = np.empty(x.shape, dtype=np.float32)
    out[..., :64] = a * c - b * s
    out[..., 64:] = a * s + b * c
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 raw bits, round to nearest even (input recipe only:
    the query is drawn in float32 and handed to both sides as bfloat16)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


def tiny(seed: int = 0):
    """-> dict(k [1,1,512,128] f32, v, q_bf16 [1,1,128] uint16)"""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((512, HEAD_DIM), dtype=np.float32)
    v = rng.standard_normal((512, HEAD_DIM), dtype=np.float32)
    q = rng.standard_normal(HEAD_DIM, dtype=np.float32)
    k[:, 3] *= 10.0
    k[:, 77] *= 10.0
    k = apply_rope(k, 0)
    return dict(k=k[None, None], v=v[None, None], q_bf16=to_bf16_bits(q)[None, None])


def layer(B: int, Hkv: int, Hq: int, T: int, seed: int, n_outliers: int = 4,
          outlier_scale: float = 8.0, rope: bool = True, pos0: int = 0):
    """GQA layer inputs.  -> dict(k, v [B,Hkv,T,128] f32, q_bf16 [B,Hq,128] uint16,
    outliers [Hkv, n_outliers])"""
    rng = np.random.default_rng(seed)
    outl = np.stack([rng.choice(HEAD_DIM, n_outliers, replace=False) for _ in range(Hkv)])
    k = rng.standard_normal((B, Hkv, T, HEAD_DIM), dtype=np.float32)
    for h in range(Hkv):
        k[:, h, :, outl[h]] *= np.float32(outlier_scale)
    if rope:
        for b in range(B):
            for h in range(Hkv):
                k[b, h] = apply_rope(k[b, h], pos0)
    v = rng.standard_normal((B, Hkv, T, HEAD_DIM), dtype=np.float32)
    q = rng.standard_normal((B, Hq, HEAD_DIM), dtype=np.float32)
    return dict(k=k, v=v, q_bf16=to_bf16_bits(q), outliers=outl)


def mixed_class_map(Hkv: int, seed: int):
    """Per kv head: a seeded permutation assigns 8 channels to 4 bits, the next
    8 to 3 bits, the next 8 to 1 bit and the rest to 2 bits.  Returns
    slot_chan [Hkv,128] int16 in the mixed key layout's slot order (slots 0..7:
    4-bit channels; slots 8,10,..,22: 3-bit channels; slots 9,11,..,23: 1-bit
    channels; slots 24..127: 2-bit channels; ascending channel order inside
    every class) and the class sets."""
    rng = np.random.default_rng(seed)
    slot_chan = np.empty((Hkv, HEAD_DIM), dtype=np.int16)
    classes = []
    for h in range(Hkv):
        perm = rng.permutation(HEAD_DIM)
        c4, c3, c1, c2 = (np.sort(perm[:8]), np.sort(perm[8:16]), np.sort(perm[16:24]),
                          np.sort(perm[24:]))
        slot_chan[h, 0:8] = c4
        slot_chan[h, 8:24:2] = c3
        slot_chan[h, 9:24:2] = c1
        slot_chan[h, 24:] = c2
        classes.append(dict(b4=c4, b3=c3, b1=c1, b2=c2))
    return slot_chan, classes


def mixed_layer(B: int, Hkv: int, Hq: int, T: int, seed: int):
    """Channel-class key generator (no RoPE).  -> dict(k, v, q_bf16, slot_chan)"""
    slot_chan, classes = mixed_class_map(Hkv, seed + 1)
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, Hkv, T, HEAD_DIM), dtype=np.float32)
    for h in range(Hkv):
        big = np.concatenate([classes[h]["b4"], classes[h]["b3"]])
        k[:, h, :, big] *= np.float32(6.0)
        k[:, h, :, classes[h]["b1"]] *= np.float32(0.2)
    v = rng.standard_normal((B, Hkv, T, HEAD_DIM), dtype=np.float32)
    q = rng.standard_normal((B, Hq, HEAD_DIM), dtype=np.float32)
    return dict(k=k, v=v, q_bf16=to_bf16_bits(q), slot_chan=slot_chan)


VMIXED_CLASS_SCALES = (3.0, 2.0, 0.25, 1.0)   # value channel scale per class (4, 3, 1, 2 bits)


def vmixed_class_map(Hkv: int, seed: int):
    """Per kv head: a seeded permutation picks 16 value channels for 4 bits,
    the next 16 for 3 bits, the next 16 for 1 bit and the other 80 for 2 bits
    (ascending channel order inside every class).  Returns v_slot_chan
    [Hkv,128] int16 in the mixed value layout's slot order and the
    per-channel value scale [Hkv,128] float32 (VMIXED_CLASS_SCALES by class:
    wider classes get the wider channels)."""
    rng = np.random.default_rng(seed)
    vsc = np.empty((Hkv, HEAD_DIM), dtype=np.int16)
    scale = np.empty((Hkv, HEAD_DIM), dtype=np.float32)
    for h in range(Hkv):
        perm = rng.permutation(HEAD_DIM)
        parts = (np.sort(perm[:16]), np.sort(perm[16:32]), np.sort(perm[32:48]), np.sort(perm[48:]))
        vsc[h] = np.concatenate(parts)
        for cls, ch in enumerate(parts):
            scale[h, ch] = VMIXED_CLASS_SCALES[cls]
    return vsc, scale


def mixed_kv_layer(B: int, Hkv: int, Hq: int, T: int, seed: int):
    """mixed_layer() plus value channel classes: values scaled per channel by
    their class.  -> dict(k, v, q_bf16, slot_chan, v_slot_chan)"""
    d = mixed_layer(B, Hkv, Hq, T, seed)
    vsc, vscale = vmixed_class_map(Hkv, seed + 2)
    d["v"] = (d["v"] * vscale[None, :, None, :]).astype(np.float32)
    d["v_slot_chan"] = vsc
    return d


def mixed_kv_layer_device(B: int, Hkv: int, Hq: int, T: int, seed: int, device):
    """mixed_layer_device() plus value channel classes (same class map as
    mixed_kv_layer())."""
    import torch
    d = mixed_layer_device(B, Hkv, Hq, T, seed, device)
    vsc, vscale = vmixed_class_map(Hkv, seed + 2)
    d["v"] *= torch.as_tensor(vscale, device=device)[None, :, None, :]
    d["v_slot_chan"] = vsc
    return d


def layer_sensitivities(n_layers: int = 64, widths=(2, 4, 8), seed: int = 0) -> np.ndarray:
    """Synthetic per-block sensitivities s[l][j] of block l at width widths[j]
    ([n_layers][len(widths)] float64), standing in for PM-KVQ's
    gradient-based ones (Key design 2), which need a trained model.  A block's
    importance a_l grows with depth (1 + 3 l / (n_layers - 1)), block 0 is
    weighted 500x (the first block's cache is the most sensitive), times a
    seeded log-normal factor (sigma 0.5); s[l][j] = a_l / (2^b - 1)^2, the
    rounding-error variance of a b-bit uniform code relative to the squared
    group range."""
    rng = np.random.default_rng(seed)
    a = (1.0 + 3.0 * np.arange(n_layers) / max(n_layers - 1, 1)) * np.exp(rng.normal(0.0, 0.5, n_layers))
    a[0] *= 500.0
    return np.array([[a[l] / float((1 << b) - 1) ** 2 for b in widths] for l in range(n_layers)])


def layer_device(B: int, Hkv: int, Hq: int, T: int, seed: int, device, n_outliers: int = 4,
                 outlier_scale: float = 8.0):
    """Same recipe as layer() drawn with torch on a device (used where the
    host draw is too slow, e.g. 64 layers of B=16, Hkv=8, T=32768).  The draw
    differs from layer()'s numpy stream but follows the same distribution."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    outl = torch.stack([torch.randperm(HEAD_DIM, generator=g, device=device)[:n_outliers]
                        for _ in range(Hkv)])
    k = torch.randn((B, Hkv, T, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
    scale = torch.ones((Hkv, HEAD_DIM), device=device, dtype=torch.float32)
    for h in range(Hkv):
        scale[h, outl[h]] = outlier_scale
    k *= scale[None, :, None, :]
    inv = torch.tensor(rope_inv_freq(), device=device, dtype=torch.float64)
    pos = torch.arange(T, device=device, dtype=torch.float64)
    ang = pos[:, None] * inv[None, :]
    c, s = torch.cos(ang), torch.sin(ang)
    for b in range(B):
        a = k[b, :, :, :64].double()
        bb = k[b, :, :, 64:].double()
        k[b, :, :, :64] = (a * c - bb * s).float()
        k[b, :, :, 64:] = (a * s + bb * c).float()
    v = torch.randn((B, Hkv, T, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
    q = torch.randn((B, Hq, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
    return dict(k=k, v=v, q=q.to(torch.bfloat16))


def mixed_layer_device(B: int, Hkv: int, Hq: int, T: int, seed: int, device):
    """Same recipe as mixed_layer() drawn with torch on a device (class map from
    the same seeded permutation; the normal draws differ from numpy's stream)."""
    import torch
    slot_chan, classes = mixed_class_map(Hkv, seed + 1)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    k = torch.randn((B, Hkv, T, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
    scale = torch.ones((Hkv, HEAD_DIM), device=device, dtype=torch.float32)
    for h in range(Hkv):
        big = np.concatenate([classes[h]["b4"], classes[h]["b3"]])
        scale[h, torch.as_tensor(big, device=device)] = 6.0
        scale[h, torch.as_tensor(classes[h]["b1"], device=device)] = 0.2
    k *= scale[None, :, None, :]
    v = torch.randn((B, Hkv, T, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
    q = torch.randn((B, Hq, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
    return dict(k=k, v=v, q=q.to(torch.bfloat16), slot_chan=slot_chan)


PAIR_SCALES = ((4, 8.0), (4, 4.0), (4, 0.2))   # (pairs, factor) after the seeded permutation


def pair_scales(Hkv: int, seed: int) -> np.ndarray:
    """[Hkv][64] per-pair key scale of the pairs recipe (1 for the unscaled pairs)."""
    rng = np.random.default_rng(seed)
    sc = np.ones((Hkv, 64), dtype=np.float32)
    for h in range(Hkv):
        perm = rng.permutation(64)
        i = 0
        for n, f in PAIR_SCALES:
            sc[h, perm[i:i + n]] = f
            i += n
    return sc


def pair_layer(B: int, Hkv: int, Hq: int, T: int, seed: int, Tq: int = 64):
    """RoPE-pair saliency generator.  -> dict(k, v [B,Hkv,T,128] f32,
    q_bf16 [B,Hq,128] uint16, q_prefill [B,Hq,Tq,128] f32, pair_scale [Hkv,64])"""
    sc = pair_scales(Hkv, seed + 1)
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, Hkv, T, HEAD_DIM), dtype=np.float32)
    full = np.concatenate([sc, sc], axis=1)                      # both channels of a pair
    k *= full[None, :, None, :]
    for b in range(B):
        for h in range(Hkv):
            k[b, h] = apply_rope(k[b, h], 0)
    v = rng.standard_normal((B, Hkv, T, HEAD_DIM), dtype=np.float32)
    q = rng.standard_normal((B, Hq, HEAD_DIM), dtype=np.float32)
    qp = rng.standard_normal((B, Hq, Tq, HEAD_DIM), dtype=np.float32)
    for b in range(B):
        for h in range(Hq):
            qp[b, h] = apply_rope(qp[b, h], 0)
    return dict(k=k, v=v, q_bf16=to_bf16_bits(q), q_prefill=qp, pair_scale=sc)


def pair_layer_device(B: int, Hkv: int, Hq: int, T: int, seed: int, device, Tq: int = 64):
    """Same recipe as pair_layer() drawn with torch on a device (pair scales from
    the same seeded permutation; the normal draws differ from numpy's stream)."""
    import torch
    sc = pair_scales(Hkv, seed + 1)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    k = torch.randn((B, Hkv, T, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
    full = torch.as_tensor(np.concatenate([sc, sc], axis=1), device=device)
    k *= full[None, :, None, :]
    inv = torch.tensor(rope_inv_freq(), device=device, dtype=torch.float64)

    def rope(x):
        pos = torch.arange(x.shape[-2], device=device, dtype=torch.float64)
        ang = pos[:, None] * inv[None, :]
        c, s = torch.cos(ang), torch.sin(ang)
        for b in range(x.shape[0]):
            a = x[b, :, :, :64].double()
            bb = x[b, :, :, 64:].double()
            x[b, :, :, :64] = (a * c - bb * s).float()
            x[b, :, :, 64:] = (a * s + bb * c).float()
    rope(k)
    v = torch.randn((B, Hkv, T, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
    q = torch.randn((B, Hq, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
    qp = torch.randn((B, Hq, Tq, HEAD_DIM), generator=g, device=device, dtype=torch.float32)
    rope(qp)
    return dict(k=k, v=v, q=q.to(torch.bfloat16), q_prefill=qp, pair_scale=sc)
