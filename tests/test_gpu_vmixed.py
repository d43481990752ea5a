"""GPU parity of mixed-width values (the ChanMix page's Key design 3 channel
classes read for values: 16 x 4-bit, 16 x 3-bit, 16 x 1-bit and 80 x 2-bit
value slots, one group per class of each token).

Quantize-and-pack is bit-exact against the oracle (tile bytes and the
class-major scales / zero points); decode attention over mixed keys and mixed
values meets the per-row bound ||o - o_ref||_inf / ||o_ref||_inf <= 2e-3
against the float64 oracle (dequantize, then ordinary attention), over
several tiles, every GQA group size class, both parameter dtypes the decode
path takes, a negative softmax scale, all-zero queries, one-hot softmaxes,
gathered tokens, the two-cache split and a residual segment.
"""
import math

import numpy as np
import pytest

import oracle
from kv_cache_mixed_amd import kvq, synth
from tests.gpu_helpers import (PDT_ORACLE, REL_TOL, SCALE, assert_stream_bytes_equal, q_to_dev,
                               rel_err_rows, to_dev)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    oracle.build(force=False)
    kvq.load()


def _stream(inp, b, h, pdt):
    return oracle.quantize_stream(inp["k"][b, h], inp["v"][b, h], kvq.KMIXED, kvq.VMIXED, PDT_ORACLE[pdt],
                                  inp["slot_chan"][h], inp["v_slot_chan"][h])


def _cache(inp, T, pdt, max_tokens=None):
    B, H = inp["k"].shape[:2]
    c = kvq.PackedCache(B, H, max_tokens or T, kvq.KMIXED, kvq.VMIXED, pdt, slot_chan=inp["slot_chan"],
                        v_slot_chan=inp["v_slot_chan"])
    return c


def _attn_err(out, inp, q_bits, pdt, scale, streams=None):
    B, H = inp["k"].shape[:2]
    G = q_bits.shape[1] // H
    worst = 0.0
    for b in range(B):
        for h in range(H):
            st = streams[b][h] if streams is not None else _stream(inp, b, h, pdt)
            ref = oracle.decode_attn(st, q_bits[b, h * G:(h + 1) * G], scale)
            worst = max(worst, rel_err_rows(out[b, h * G:(h + 1) * G], ref).max())
    return worst


@pytest.mark.parametrize("pdt", [kvq.E4M3, kvq.F16, kvq.F32, kvq.BF16])
def test_quantize_bytes_bit_exact(pdt):
    inp = synth.mixed_kv_layer(2, 2, 8, 512, seed=600 + pdt)
    print("vmixed quantize pdt=%d" % pdt, flush=True)
    c = _cache(inp, 640, pdt)
    c.quantize(to_dev(inp["k"], torch), to_dev(inp["v"], torch), 0)
    torch.cuda.synchronize()
    for b in range(2):
        for h in range(2):
            assert_stream_bytes_equal(c, _stream(inp, b, h, pdt), b, h, "vmixed pdt=%d" % pdt)


def test_quantize_bf16_input_and_offset():
    """bfloat16 inputs at a tile offset t0 (second call) with strided rows."""
    inp = synth.mixed_kv_layer(1, 3, 3, 256, seed=610)
    k16 = torch.from_numpy(inp["k"]).to(torch.bfloat16)
    v16 = torch.from_numpy(inp["v"]).to(torch.bfloat16)
    kf = k16.float().numpy()
    vf = v16.float().numpy()
    print("vmixed quantize bf16 offset", flush=True)
    c = _cache(inp, 512, kvq.E4M3)
    c.quantize(k16[:, :, :128].cuda(), v16[:, :, :128].cuda(), 0)
    big = torch.zeros((1, 3, 128, 256), dtype=torch.bfloat16)
    big[..., :128] = v16[:, :, 128:]
    c.quantize(k16[:, :, 128:].cuda(), big.cuda()[..., :128], 128)
    torch.cuda.synchronize()
    assert c.n_tokens == 256
    for h in range(3):
        st = oracle.quantize_stream(kf[0, h], vf[0, h], kvq.KMIXED, kvq.VMIXED, oracle.E4M3,
                                    inp["slot_chan"][h], inp["v_slot_chan"][h])
        assert_stream_bytes_equal(c, st, 0, h, "bf16 offset")


def test_quantize_tokens_gathered():
    """kvq_quantize_tokens with mixed values: rows picked by a token list."""
    inp = synth.mixed_kv_layer(1, 2, 4, 384, seed=620)
    rng = np.random.default_rng(621)
    tok = np.stack([np.sort(rng.permutation(384)[:256]) for _ in range(2)])[None].astype(np.int32)
    print("vmixed gathered quantize", flush=True)
    c = _cache(inp, 256, kvq.E4M3)
    c.quantize_tokens(to_dev(inp["k"], torch), to_dev(inp["v"], torch), torch.from_numpy(tok).cuda())
    torch.cuda.synchronize()
    for h in range(2):
        rows = tok[0, h]
        st = oracle.quantize_stream(inp["k"][0, h][rows], inp["v"][0, h][rows], kvq.KMIXED, kvq.VMIXED,
                                    oracle.E4M3, inp["slot_chan"][h], inp["v_slot_chan"][h])
        assert_stream_bytes_equal(c, st, 0, h, "gathered")


@pytest.mark.parametrize("pdt", [kvq.E4M3, kvq.F16])
@pytest.mark.parametrize("B,H,G,T", [(1, 2, 4, 1280), (2, 2, 1, 640), (1, 1, 16, 896), (2, 3, 7, 384)])
def test_decode_parity(pdt, B, H, G, T):
    inp = synth.mixed_kv_layer(B, H, H * G, T, seed=630 + B + H + G + T // 128)
    print("vmixed decode pdt=%d B=%d H=%d G=%d T=%d" % (pdt, B, H, G, T), flush=True)
    c = _cache(inp, T, pdt)
    c.quantize(to_dev(inp["k"], torch), to_dev(inp["v"], torch), 0)
    out = c.decode_attn(q_to_dev(inp["q_bf16"], torch), SCALE).cpu().numpy()
    assert np.all(np.isfinite(out))
    err = _attn_err(out, inp, inp["q_bf16"], pdt, SCALE)
    assert err <= REL_TOL, "max row relative error %.3e" % err


def test_decode_long_fused_combine():
    """A single long stream group cut into 64 chunks."""
    inp = synth.mixed_kv_layer(1, 1, 4, 16384, seed=640)
    print("vmixed decode long", flush=True)
    c = _cache(inp, 16384, kvq.E4M3)
    c.quantize(to_dev(inp["k"], torch), to_dev(inp["v"], torch), 0)
    out = c.decode_attn(q_to_dev(inp["q_bf16"], torch), SCALE).cpu().numpy()
    err = _attn_err(out, inp, inp["q_bf16"], kvq.E4M3, SCALE)
    assert err <= REL_TOL, "max row relative error %.3e" % err


def test_decode_negative_scale_and_zero_queries():
    inp = synth.mixed_kv_layer(2, 2, 12, 768, seed=650)
    q = inp["q_bf16"].copy()
    q[0, 1] = 0
    q[1, 6:12] = 0
    print("vmixed decode negative scale / zero queries", flush=True)
    c = _cache(inp, 768, kvq.E4M3)
    c.quantize(to_dev(inp["k"], torch), to_dev(inp["v"], torch), 0)
    for sc in (-SCALE, SCALE):
        out = c.decode_attn(q_to_dev(q, torch), sc).cpu().numpy()
        err = _attn_err(out, inp, q, kvq.E4M3, sc)
        assert err <= REL_TOL, "scale %g: max row relative error %.3e" % (sc, err)


def test_decode_dominant_key():
    """sigma x 1000 with one planted key along the query: the output is that
    token's reconstructed value row (every class's parameters of one token)."""
    inp = synth.mixed_kv_layer(1, 2, 8, 1024, seed=660)
    k = inp["k"].copy()
    rng = np.random.default_rng(661)
    qf = rng.standard_normal((1, 8, 128)).astype(np.float32)
    for h in range(2):
        k[0, h, 500 + 200 * h] = 4.0 * qf[0, 4 * h] / np.linalg.norm(qf[0, 4 * h]) * math.sqrt(128)
    inp = dict(inp, k=k)
    q = synth.to_bf16_bits(qf)
    print("vmixed decode dominant key", flush=True)
    c = _cache(inp, 1024, kvq.E4M3)
    c.quantize(to_dev(k, torch), to_dev(inp["v"], torch), 0)
    out = c.decode_attn(q_to_dev(q, torch), 1000 * SCALE).cpu().numpy()
    err = _attn_err(out, inp, q, kvq.E4M3, 1000 * SCALE)
    assert err <= REL_TOL, "max row relative error %.3e" % err


def test_decode_residual_segment():
    """Mixed cache plus 70 residual (bfloat16) tokens per stream."""
    inp = synth.mixed_kv_layer(1, 2, 8, 640, seed=670)
    rng = np.random.default_rng(671)
    rk = rng.standard_normal((1, 2, 70, 128)).astype(np.float32)
    rv = rng.standard_normal((1, 2, 70, 128)).astype(np.float32)
    rk16, rv16 = torch.from_numpy(rk).to(torch.bfloat16), torch.from_numpy(rv).to(torch.bfloat16)
    print("vmixed decode residual", flush=True)
    c = _cache(inp, 640, kvq.F16)
    c.quantize(to_dev(inp["k"], torch), to_dev(inp["v"], torch), 0)
    out = c.decode_attn(q_to_dev(inp["q_bf16"], torch), SCALE, res_k=rk16.cuda(), res_v=rv16.cuda()).cpu().numpy()
    worst = 0.0
    for h in range(2):
        st = _stream(inp, 0, h, kvq.F16)
        K = np.concatenate([oracle.dequant_k(st), rk16.float().numpy()[0, h].astype(np.float64)])
        V = np.concatenate([oracle.dequant_v(st), rv16.float().numpy()[0, h].astype(np.float64)])
        qq = synth.bf16_bits_to_f32(inp["q_bf16"][0, 4 * h:4 * h + 4]).astype(np.float64)
        s = SCALE * qq @ K.T
        p = np.exp(s - s.max(axis=1, keepdims=True))
        ref = (p / p.sum(axis=1, keepdims=True)) @ V
        worst = max(worst, rel_err_rows(out[0, 4 * h:4 * h + 4], ref).max())
    assert worst <= REL_TOL, "max row relative error %.3e" % worst


def test_decode_split_mixed_and_uniform():
    """Two caches of the same streams, one with mixed values and one at
    uniform 4-bit widths: attention over the union of their tokens."""
    inp = synth.mixed_kv_layer(1, 2, 8, 768, seed=680)
    print("vmixed split decode", flush=True)
    a = _cache({**inp, "k": inp["k"][:, :, :512], "v": inp["v"][:, :, :512]}, 512, kvq.E4M3)
    a.quantize(to_dev(inp["k"][:, :, :512], torch), to_dev(inp["v"][:, :, :512], torch), 0)
    bc = kvq.PackedCache(1, 2, 256, 4, 4, kvq.E4M3)
    bc.quantize(to_dev(inp["k"][:, :, 512:], torch), to_dev(inp["v"][:, :, 512:], torch), 0)
    out = kvq.decode_attn_split(a, bc, q_to_dev(inp["q_bf16"], torch), SCALE).cpu().numpy()
    worst = 0.0
    for h in range(2):
        sa = oracle.quantize_stream(inp["k"][0, h, :512], inp["v"][0, h, :512], kvq.KMIXED, kvq.VMIXED,
                                    oracle.E4M3, inp["slot_chan"][h], inp["v_slot_chan"][h])
        sb = oracle.quantize_stream(inp["k"][0, h, 512:], inp["v"][0, h, 512:], 4, 4, oracle.E4M3)
        ref = oracle.decode_attn_union([sa, sb], inp["q_bf16"][0, 4 * h:4 * h + 4], SCALE)
        worst = max(worst, rel_err_rows(out[0, 4 * h:4 * h + 4], ref).max())
    assert worst <= REL_TOL, "max row relative error %.3e" % worst


def test_decode_noalloc_equals_workspace_call():
    """The allocation-free entry point on a mixed K+V cache gives the same
    bits as the workspace entry point."""
    inp = synth.mixed_kv_layer(1, 2, 8, 2048, seed=690)
    print("vmixed noalloc", flush=True)
    c = _cache(inp, 2048, kvq.E4M3)
    c.quantize(to_dev(inp["k"], torch), to_dev(inp["v"], torch), 0)
    q = q_to_dev(inp["q_bf16"], torch)
    a = c.decode_attn(q, SCALE)
    b = c.decode_attn_noalloc(q, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_window_append_and_residual_decode():
    """Token-granular append into a mixed K+V cache (first token and recent
    tokens held in bfloat16, full groups packed at the mixed widths), then
    decode over cache + window against the oracle's attention over (packed
    tokens, held tokens)."""
    B, H, G, T = 1, 2, 4, 300
    inp = synth.mixed_kv_layer(B, H, H * G, T, seed=700)
    k16 = torch.from_numpy(inp["k"]).to(torch.bfloat16)
    v16 = torch.from_numpy(inp["v"]).to(torch.bfloat16)
    kf, vf = k16.float().numpy(), v16.float().numpy()
    print("vmixed window append", flush=True)
    c = _cache(inp, 512, kvq.E4M3)
    win = kvq.Window(c, torch.bfloat16, keep_first=True)
    for a, b in ((0, 1), (1, 130), (130, 131), (131, 300)):
        win.append(k16[:, :, a:b].contiguous().cuda(), v16[:, :, a:b].contiguous().cuda())
    torch.cuda.synchronize()
    # token 0 in row 0, tokens 1..256 packed (two groups), 257..299 held
    assert (win.w.n_first, win.w.n_recent, c.n_tokens) == (1, 43, 256)
    held = [0] + list(range(257, 300))
    rk, rv = win.residual()
    out = c.decode_attn(q_to_dev(inp["q_bf16"], torch), SCALE, res_k=rk, res_v=rv).cpu().numpy()
    worst = 0.0
    for h in range(H):
        st = oracle.quantize_stream(kf[0, h, 1:257], vf[0, h, 1:257], kvq.KMIXED, kvq.VMIXED, oracle.E4M3,
                                    inp["slot_chan"][h], inp["v_slot_chan"][h])
        assert_stream_bytes_equal(c, st, 0, h, "window")
        ref = oracle.decode_attn_residual(st, inp["q_bf16"][0, h * G:(h + 1) * G], SCALE, kf[0, h, held],
                                          vf[0, h, held])
        worst = max(worst, rel_err_rows(out[0, h * G:(h + 1) * G], ref).max())
    assert worst <= REL_TOL, "max row relative error %.3e" % worst
