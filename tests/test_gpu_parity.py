"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Integer codes, packed bytes, scales/zeros and ERS output must be bit-exact;
attention must agree within max relative error 2e-3 per output row
(||o - o_ref||_inf / ||o_ref||_inf, float64 oracle).
"""
import numpy as np
import pytest

import oracle
from kv_cache_mixed_amd import kvq, synth
from tests.gpu_helpers import (PDT_ORACLE, REL_TOL, SCALE, assert_stream_bytes_equal, oracle_attn,
                               oracle_stream, q_to_dev, rel_err_rows, to_dev)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    oracle.build(force=False)
    kvq.load()


def _quantized(B, H, Hq, T, k_bits, v_bits, pdt, seed, mixed=False):
    if mixed:
        inp = synth.mixed_layer(B, H, Hq, T, seed)
        slot_chan = inp["slot_chan"]
    else:
        inp = synth.layer(B, H, Hq, T, seed)
        slot_chan = None
    cache = kvq.PackedCache(B, H, T, k_bits, v_bits, pdt,
                            slot_chan=slot_chan if mixed else None)
    cache.quantize(to_dev(inp["k"], torch), to_dev(inp["v"], torch), 0)
    torch.cuda.synchronize()
    return inp, cache


@pytest.mark.parametrize("bits", [16, 8, 4, 2, 1])
@pytest.mark.parametrize("pdt", [kvq.F16, kvq.E4M3, kvq.BF16, kvq.F32])
def test_quantize_bitexact(bits, pdt):
    print("case quantize bits=%d pdt=%d" % (bits, pdt), flush=True)
    inp, cache = _quantized(2, 2, 4, 384, bits, bits, pdt, seed=10 + bits + 17 * pdt)
    for b in range(2):
        for h in range(2):
            st = oracle_stream(inp, b, h, bits, bits, pdt)
            assert_stream_bytes_equal(cache, st, b, h, "bits=%d pdt=%d" % (bits, pdt))


@pytest.mark.parametrize("pdt", [kvq.F16, kvq.E4M3])
def test_quantize_mixed_bitexact(pdt):
    print("case quantize mixed pdt=%d" % pdt, flush=True)
    inp, cache = _quantized(1, 3, 6, 512, kvq.KMIXED, 2, pdt, seed=5, mixed=True)
    for h in range(3):
        st = oracle_stream(inp, 0, h, 0, 2, pdt, inp["slot_chan"][h])
        assert_stream_bytes_equal(cache, st, 0, h, "mixed pdt=%d" % pdt)


def test_quantize_bf16_input_and_offset_t0():
    """bfloat16 inputs, quantizing into a later tile range with strided input."""
    inp = synth.layer(1, 2, 2, 512, 77)
    kb = torch.from_numpy(inp["k"]).to(torch.bfloat16)
    vb = torch.from_numpy(inp["v"]).to(torch.bfloat16)
    cache = kvq.PackedCache(1, 2, 1024, 4, 4, kvq.F16)
    big_k = torch.zeros(1, 2, 640, 128, dtype=torch.bfloat16)
    big_k[:, :, 64:576] = kb
    kd = big_k.cuda()[:, :, 64:576]                 # non-contiguous view, stride(2) = 128
    cache.quantize(kd, vb.cuda(), t0=256)
    cache.quantize(kd[:, :, :256], vb.cuda()[:, :, :256], t0=0)
    torch.cuda.synchronize()
    assert cache.n_tokens == 768
    kf = np.concatenate([kb.float().numpy()[:, :, :256], kb.float().numpy()], axis=2)
    vf = np.concatenate([vb.float().numpy()[:, :, :256], vb.float().numpy()], axis=2)
    for h in range(2):
        st = oracle.quantize_stream(kf[0, h], vf[0, h], 4, 4, oracle.F16)
        assert_stream_bytes_equal(cache, st, 0, h, "bf16 input")


@pytest.mark.parametrize("to_bits", [8, 4, 2, 1])
@pytest.mark.parametrize("pdt", [kvq.F16, kvq.E4M3])
def test_shrink_bitexact(to_bits, pdt):
    print("case shrink to=%d pdt=%d" % (to_bits, pdt), flush=True)
    inp, cache = _quantized(2, 2, 4, 384, 2 * to_bits, 2 * to_bits, pdt, seed=30 + to_bits)
    cache.shrink(to_bits)
    torch.cuda.synchronize()
    assert cache.k_bits == to_bits and cache.v_bits == to_bits
    for b in range(2):
        for h in range(2):
            st = oracle.shrink_stream(oracle_stream(inp, b, h, 2 * to_bits, 2 * to_bits, pdt), to_bits)
            assert_stream_bytes_equal(cache, st, b, h, "shrink to %d" % to_bits)


@pytest.mark.parametrize("to_bits", [8, 4, 2, 1])
@pytest.mark.parametrize("method", [kvq.SHIFT_DIRECT, kvq.SHIFT_MODIFIED])
def test_shrink_other_rules_bitexact(to_bits, method):
    """The ablation's direct and modified right shifts, bytes and scales
    against the oracle; decode over the shrunk cache within tolerance."""
    print("case shrink rule=%d to=%d" % (method, to_bits), flush=True)
    inp, cache = _quantized(2, 2, 8, 384, 2 * to_bits, 2 * to_bits, kvq.F16, seed=40 + to_bits + 7 * method)
    cache.shrink(to_bits, method=method)
    torch.cuda.synchronize()
    assert cache.k_bits == to_bits and cache.v_bits == to_bits
    out = cache.decode_attn(q_to_dev(inp["q_bf16"], torch), SCALE).cpu().numpy()
    for b in range(2):
        for h in range(2):
            st = oracle.shrink_stream(oracle_stream(inp, b, h, 2 * to_bits, 2 * to_bits, kvq.F16), to_bits, method)
            assert_stream_bytes_equal(cache, st, b, h, "shrink rule %d to %d" % (method, to_bits))
            ref = oracle_attn(st, inp["q_bf16"][b, h * 4:(h + 1) * 4])
            assert rel_err_rows(out[b, h * 4:(h + 1) * 4], ref).max() <= REL_TOL


def _decode_case(B, H, Hq, T, k_bits, v_bits, pdt, seed, mixed=False, pairs=None):
    inp, cache = _quantized(B, H, Hq, T, k_bits, v_bits, pdt, seed, mixed)
    q = q_to_dev(inp["q_bf16"], torch)
    out = cache.decode_attn(q, SCALE).cpu().numpy()
    G = Hq // H
    worst = 0.0
    for (b, h) in (pairs or [(b, h) for b in range(B) for h in range(H)]):
        st = oracle_stream(inp, b, h, k_bits, v_bits, pdt,
                           inp["slot_chan"][h] if mixed else None)
        ref = oracle_attn(st, inp["q_bf16"][b, h * G:(h + 1) * G])
        err = rel_err_rows(out[b, h * G:(h + 1) * G], ref).max()
        worst = max(worst, err)
    assert np.all(np.isfinite(out))
    assert worst <= REL_TOL, "max row relative error %.3e" % worst
    return worst


@pytest.mark.parametrize("bits", [4, 2, 8, 1, 16])
@pytest.mark.parametrize("pdt", [kvq.F16, kvq.E4M3])
def test_decode_uniform(bits, pdt):
    print("case decode bits=%d pdt=%d" % (bits, pdt), flush=True)
    _decode_case(2, 2, 14, 1152, bits, bits, pdt, seed=40 + bits)


@pytest.mark.parametrize("bits", [16, 8])
def test_decode_several_tiles_per_wave(bits):
    """Regression: with several tiles per wave (B=8, Hkv=4, T=8192 -> 2 tiles per
    wave) the wide-code instances must not let one wave's partial overwrite the
    folded query another wave is still reading (LDS regions of 16 KB)."""
    print("case decode several tiles per wave bits=%d" % bits, flush=True)
    _decode_case(8, 4, 28, 8192, bits, bits, kvq.F16, seed=140 + bits,
                 pairs=[(0, 0), (2, 1), (5, 2), (7, 3)])


@pytest.mark.parametrize("v_bits", [2, 4, 1])
def test_decode_mixed(v_bits):
    print("case decode mixed v=%d" % v_bits, flush=True)
    _decode_case(1, 2, 8, 1280, kvq.KMIXED, v_bits, kvq.E4M3, seed=60 + v_bits, mixed=True)


@pytest.mark.parametrize("G", [1, 5, 16])
def test_decode_group_sizes(G):
    print("case decode G=%d" % G, flush=True)
    _decode_case(1, 2, 2 * G, 640, 4, 4, kvq.F16, seed=70 + G)


@pytest.mark.parametrize("T", [128, 384, 8192])
def test_decode_lengths(T):
    """one tile, a ragged chunk (fewer tiles than waves), many chunks."""
    print("case decode T=%d" % T, flush=True)
    _decode_case(2, 1, 4, T, 4, 4, kvq.F16, seed=80 + T // 128)


@pytest.mark.parametrize("pdt", [kvq.BF16, kvq.F32])
def test_decode_other_param_dtypes(pdt):
    _decode_case(1, 2, 8, 512, 4, 4, pdt, seed=90 + pdt)


def test_decode_repeat_and_workspace_reuse():
    """Repeated calls give identical output, and the workspace needs no
    initial contents (garbage, NaN bit patterns included, gives the same
    bits)."""
    inp, cache = _quantized(2, 2, 8, 4096, 4, 4, kvq.F16, seed=95)
    q = q_to_dev(inp["q_bf16"], torch)
    o1 = cache.decode_attn(q, SCALE).cpu().numpy()
    o2 = cache.decode_attn(q, SCALE).cpu().numpy()
    ws = cache.workspace(8)
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, generator=torch.Generator().manual_seed(7)))
    ws[:64].fill_(0xff)
    o3 = cache.decode_attn(q, SCALE, workspace=ws).cpu().numpy()
    o4 = cache.decode_attn(q, SCALE, workspace=ws).cpu().numpy()
    assert np.array_equal(o1, o2) and np.array_equal(o2, o3) and np.array_equal(o3, o4)


def test_tiny_config():
    """1 kv head, 1 query head, 512 tokens: 4-bit quantize, ERS 4->2, decode on both."""
    inp = synth.tiny(0)
    cache = kvq.PackedCache(1, 1, 512, 4, 4, kvq.F16)
    cache.quantize(to_dev(inp["k"], torch), to_dev(inp["v"], torch))
    q = q_to_dev(inp["q_bf16"], torch)
    o4 = cache.decode_attn(q, SCALE).cpu().numpy()
    st4 = oracle_stream(inp, 0, 0, 4, 4, kvq.F16)
    assert_stream_bytes_equal(cache, st4, 0, 0, "tiny 4-bit")
    assert rel_err_rows(o4[0], oracle_attn(st4, inp["q_bf16"][0])).max() <= REL_TOL
    cache.shrink(2)
    o2 = cache.decode_attn(q, SCALE).cpu().numpy()
    st2 = oracle.shrink_stream(st4, 2)
    assert_stream_bytes_equal(cache, st2, 0, 0, "tiny 2-bit")
    assert rel_err_rows(o2[0], oracle_attn(st2, inp["q_bf16"][0])).max() <= REL_TOL


def test_pool_layout_decode():
    """Tiles placed through a kvq_pool (offset tables) decode like the contiguous layout."""
    B, H, Hq, T = 2, 2, 8, 1024
    inp = synth.layer(B, H, Hq, T, 99)
    pool_bytes = B * H * (T // 128) * 2 * 2048 * 4
    cache = kvq.PackedCache(B, H, T, 4, 4, kvq.F16, layout="pool", pool_bytes=pool_bytes)
    kd, vd = to_dev(inp["k"], torch), to_dev(inp["v"], torch)
    for t0 in range(0, T, 256):
        cache.append(kd[:, :, t0:t0 + 256], vd[:, :, t0:t0 + 256], budget_bytes=1 << 40,
                     floor_bits=4)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            assert_stream_bytes_equal(cache, oracle_stream(inp, b, h, 4, 4, kvq.F16), b, h, "pool")
    out = cache.decode_attn(q_to_dev(inp["q_bf16"], torch), SCALE).cpu().numpy()
    G = Hq // H
    for b in range(B):
        for h in range(H):
            ref = oracle_attn(oracle_stream(inp, b, h, 4, 4, kvq.F16), inp["q_bf16"][b, h * G:(h + 1) * G])
            assert rel_err_rows(out[b, h * G:(h + 1) * G], ref).max() <= REL_TOL


@pytest.mark.parametrize("B,H,Hq,T", [(64, 4, 28, 8192), (16, 4, 28, 4096), (1, 8, 32, 4096)])
def test_workspace_and_output_guard_bytes(B, H, Hq, T):
    """Regression: the workspace must hold every chunk the launch plan uses
    (a plan with several kv streams per wave has more chunks).  Guard bytes
    after the workspace and after the output must stay untouched."""
    print("case guard B=%d H=%d Hq=%d T=%d" % (B, H, Hq, T), flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(B + T)
    cache = kvq.PackedCache(B, H, T, 4, 4, kvq.F16)
    for t0 in range(0, T, 2048):
        k = torch.randn((B, H, 2048, 128), generator=g, device="cuda")
        v = torch.randn((B, H, 2048, 128), generator=g, device="cuda")
        cache.quantize(k, v, t0)
    q = torch.randn((B, Hq, 128), generator=g, device="cuda").to(torch.bfloat16)
    nb = cache.workspace_bytes(Hq)
    GUARD = 1 << 20
    ws_full = torch.zeros(nb + GUARD, dtype=torch.uint8, device="cuda")
    ws_full[nb:] = 0xA5
    out_full = torch.full((B * Hq * 128 + 4096,), 7.0, dtype=torch.float32, device="cuda")
    out = out_full[:B * Hq * 128].view(B, Hq, 128)
    for _ in range(2):
        cache.decode_attn(q, SCALE, out=out, workspace=ws_full[:nb])
    torch.cuda.synchronize()
    assert bool((ws_full[nb:] == 0xA5).all()), "workspace overrun"
    assert bool((out_full[B * Hq * 128:] == 7.0).all()), "output overrun"
    assert bool(torch.isfinite(out).all())


@pytest.mark.parametrize("pdt", [kvq.F16, kvq.E4M3])
def test_quantize_edge_groups(pdt):
    """Constant groups (S' = 0), groups of signed zeros, ranges so small that
    S' is subnormal or flushes to zero, one huge outlier, exact integers."""
    print("case edge groups pdt=%d" % pdt, flush=True)
    rng = np.random.default_rng(123)
    T = 512
    k = rng.standard_normal((1, 2, T, 128)).astype(np.float32)
    v = rng.standard_normal((1, 2, T, 128)).astype(np.float32)
    k[0, 0, 0:128, 5] = 1.25                       # constant key group
    k[0, 0, 0:128, 6] = np.where(np.arange(128) % 2, -0.0, 0.0).astype(np.float32)
    k[0, 0, 128:256, 7] = 1.0 + rng.standard_normal(128).astype(np.float32) * 1e-6
    k[0, 1, 256:384, 9] *= 1e-7                     # subnormal-range scale
    k[0, 1, 384:512, 11][17] = 300.0 if pdt == kvq.E4M3 else 5000.0   # huge outlier
    v[0, 0, 3, :] = -2.5                            # constant value group
    v[0, 0, 4, :] = np.where(np.arange(128) % 3, 0.0, -0.0)
    v[0, 1, 5, :] = np.arange(128, dtype=np.float32)  # exact integers
    v[0, 1, 6, :] *= 1e-6
    inp = dict(k=k, v=v)
    for bits in (4, 2, 8):
        cache = kvq.PackedCache(1, 2, T, bits, bits, pdt)
        cache.quantize(to_dev(k, torch), to_dev(v, torch), 0)
        torch.cuda.synchronize()
        for h in range(2):
            st = oracle_stream(inp, 0, h, bits, bits, pdt)
            assert_stream_bytes_equal(cache, st, 0, h, "edge bits=%d pdt=%d" % (bits, pdt))


def _near_tie_values(lo, S, levels, n, rng):
    """n float32 values whose quotients (x - lo) / S lie on, or a few ulps off,
    half-integers k + 1/2 (lo and S exact in the parameter dtype)."""
    k = rng.integers(0, levels, n)
    x = (np.float32(lo) + (k + 0.5).astype(np.float32) * np.float32(S)).astype(np.float32)
    steps = rng.integers(-3, 4, n)
    for i in range(n):
        for _ in range(abs(int(steps[i]))):
            x[i] = np.nextafter(x[i], np.float32(np.inf if steps[i] > 0 else -np.inf))
    return x


@pytest.mark.parametrize("pdt", [kvq.F16, kvq.E4M3])
def test_quantize_near_half_integer_quotients(pdt):
    """Groups whose code quotients (x - Z')/S' sit exactly on, or within three
    ulps of, half-integers, with S' = 0.375 (an inexact reciprocal): the codes
    the kernels form from a reciprocal must equal those of the correctly
    rounded division, ties to even."""
    print("case near ties pdt=%d" % pdt, flush=True)
    rng = np.random.default_rng(321)
    T, lo, S = 256, -1.5, 0.375
    for bits in (8, 4, 2):
        levels = (1 << bits) - 1
        hi = lo + levels * S
        k = np.empty((1, 1, T, 128), np.float32)
        v = np.empty((1, 1, T, 128), np.float32)
        for t in range(T):                          # value groups: one token
            v[0, 0, t, 0], v[0, 0, t, 1] = lo, hi
            v[0, 0, t, 2:] = _near_tie_values(lo, S, levels, 126, rng)
        for c in range(128):                        # key groups: one channel of a tile
            for g in range(T // 128):
                k[0, 0, 128 * g, c], k[0, 0, 128 * g + 1, c] = lo, hi
                k[0, 0, 128 * g + 2:128 * g + 128, c] = _near_tie_values(lo, S, levels, 126, rng)
        q = (v[0, 0, :, 2:] - np.float32(lo)) / np.float32(S)
        assert np.mean(q == np.floor(q) + 0.5) > 0.05   # the construction hits exact ties
        cache = kvq.PackedCache(1, 1, T, bits, bits, pdt)
        cache.quantize(to_dev(k, torch), to_dev(v, torch), 0)
        torch.cuda.synchronize()
        st = oracle_stream(dict(k=k, v=v), 0, 0, bits, bits, pdt)
        assert_stream_bytes_equal(cache, st, 0, 0, "near ties bits=%d pdt=%d" % (bits, pdt))


# ---------------------------------------------------------------------------
# decode with a residual segment of unquantized tokens
# ---------------------------------------------------------------------------
def _residual_case(B, H, Hq, T, R, bits, pdt, res_dtype, seed, mixed=False):
    """Tokens [0, T) quantized into the cache, tokens [T, T+R) handed over as the
    residual segment (float32 or bfloat16); every stream against the oracle."""
    G = Hq // H
    if mixed:
        inp = synth.mixed_layer(B, H, Hq, T + R, seed)
    else:
        inp = synth.layer(B, H, Hq, T + R, seed)
    sc = inp["slot_chan"] if mixed else None
    cache = kvq.PackedCache(B, H, max(T, 128), kvq.KMIXED if mixed else bits, bits, pdt, slot_chan=sc)
    if T:
        cache.quantize(to_dev(inp["k"][:, :, :T], torch), to_dev(inp["v"][:, :, :T], torch), 0)
    rk = to_dev(inp["k"][:, :, T:], torch).to(res_dtype)
    rv = to_dev(inp["v"][:, :, T:], torch).to(res_dtype)
    out = cache.decode_attn(q_to_dev(inp["q_bf16"], torch), SCALE, res_k=rk, res_v=rv).cpu().numpy()
    assert np.all(np.isfinite(out))
    rk_h, rv_h = rk.float().cpu().numpy(), rv.float().cpu().numpy()   # exact widening
    worst = 0.0
    for b in range(B):
        for h in range(H):
            st = None
            if T:
                st = oracle.quantize_stream(inp["k"][b, h, :T], inp["v"][b, h, :T],
                                            0 if mixed else bits, bits, PDT_ORACLE[pdt],
                                            None if sc is None else sc[h])
            ref = oracle.decode_attn_residual(st, inp["q_bf16"][b, h * G:(h + 1) * G], SCALE,
                                              rk_h[b, h], rv_h[b, h])
            worst = max(worst, rel_err_rows(out[b, h * G:(h + 1) * G], ref).max())
    assert worst <= REL_TOL, "max row relative error %.3e" % worst
    return worst


@pytest.mark.parametrize("T,R", [(128, 1), (1152, 77), (4096, 128), (384, 512), (0, 1), (0, 200),
                                 (0, 512)])
@pytest.mark.parametrize("res_dtype", ["f32", "f16", "bf16"])
def test_decode_residual(T, R, res_dtype):
    print("case decode residual T=%d R=%d %s" % (T, R, res_dtype), flush=True)
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[res_dtype]
    _residual_case(2, 2, 14, T, R, 4, kvq.F16, dt, seed=900 + T + R)


@pytest.mark.parametrize("bits,G", [(2, 4), (8, 7), (16, 16), (1, 1)])
def test_decode_residual_widths_and_groups(bits, G):
    print("case decode residual bits=%d G=%d" % (bits, G), flush=True)
    _residual_case(2, 2, 2 * G, 1024, 100, bits, kvq.E4M3 if bits == 2 else kvq.F16,
                   torch.bfloat16, seed=950 + bits)


def test_decode_residual_mixed_keys():
    print("case decode residual mixed", flush=True)
    _residual_case(1, 3, 12, 2048, 64, 2, kvq.E4M3, torch.float32, seed=960, mixed=True)


def test_decode_residual_strided_views_and_garbage_workspace():
    """Residual segment read through strided views of a larger ring buffer
    (element strides of a [B][H][512][128] buffer, window starting at 40);
    workspace filled with garbage; result equals the contiguous call."""
    B, H, Hq, T, R = 2, 2, 8, 640, 90
    inp = synth.layer(B, H, Hq, T + R, 961)
    cache = kvq.PackedCache(B, H, 1024, 4, 4, kvq.F16)
    cache.quantize(to_dev(inp["k"][:, :, :T], torch), to_dev(inp["v"][:, :, :T], torch), 0)
    ring_k = torch.full((B, H, 512, 128), float("nan"), device="cuda")
    ring_v = torch.full((B, H, 512, 128), float("nan"), device="cuda")
    ring_k[:, :, 40:40 + R] = to_dev(inp["k"][:, :, T:], torch)
    ring_v[:, :, 40:40 + R] = to_dev(inp["v"][:, :, T:], torch)
    q = q_to_dev(inp["q_bf16"], torch)
    ws = cache.workspace(Hq)
    ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda"))
    a = cache.decode_attn(q, SCALE, res_k=ring_k[:, :, 40:40 + R], res_v=ring_v[:, :, 40:40 + R])
    b = cache.decode_attn(q, SCALE, res_k=ring_k[:, :, 40:40 + R].contiguous(),
                          res_v=ring_v[:, :, 40:40 + R].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    G = Hq // H
    out = a.cpu().numpy()
    for bb in range(B):
        for h in range(H):
            st = oracle.quantize_stream(inp["k"][bb, h, :T], inp["v"][bb, h, :T], 4, 4, oracle.F16)
            ref = oracle.decode_attn_residual(st, inp["q_bf16"][bb, h * G:(h + 1) * G], SCALE,
                                              inp["k"][bb, h, T:], inp["v"][bb, h, T:])
            assert rel_err_rows(out[bb, h * G:(h + 1) * G], ref).max() <= REL_TOL


def test_decode_streaming_with_residual():
    """Decode as generation runs, with the first-token + recent-token window
    ([PMKVQ] Training strategy): a bfloat16 window buffer per stream holds the
    first token in row 0 for good and the most recent 1..128 tokens after it.
    When a token arrives with 128 recent tokens already held, those 128 become
    one packed group (kvq_append reads them straight from the window) and the
    new token starts the next window.  Every step's output matches the oracle
    over (packed tokens, window tokens)."""
    B, H, Hq, N = 1, 2, 8, 3 * 128 + 46
    G = Hq // H
    inp = synth.layer(B, H, Hq, N, 962)
    cache = kvq.PackedCache(B, H, 512, 4, 4, kvq.F16)
    kd = to_dev(inp["k"], torch).to(torch.bfloat16)
    vd = to_dev(inp["v"], torch).to(torch.bfloat16)
    kf, vf = kd.float().cpu().numpy(), vd.float().cpu().numpy()
    win_k = torch.zeros((B, H, 129, 128), dtype=torch.bfloat16, device="cuda")
    win_v = torch.zeros_like(win_k)
    q = q_to_dev(inp["q_bf16"], torch)
    streams = [None] * H
    first_recent = 1             # token index held in window row 1
    for t in range(N):           # token t arrives
        if t == 0:
            win_k[:, :, 0] = kd[:, :, 0]
            win_v[:, :, 0] = vd[:, :, 0]
            n_win = 1
        else:
            if n_win == 129:     # 128 recent tokens held: pack them, restart the window
                assert cache.append(win_k[:, :, 1:129], win_v[:, :, 1:129], budget_bytes=1 << 40,
                                    floor_bits=4) == 0
                first_recent += 128
                n_win = 1
                for h in range(H):
                    streams[h] = oracle.quantize_stream(kf[0, h, 1:first_recent],
                                                        vf[0, h, 1:first_recent], 4, 4, oracle.F16)
            win_k[:, :, n_win] = kd[:, :, t]
            win_v[:, :, n_win] = vd[:, :, t]
            n_win += 1
        assert cache.n_tokens == first_recent - 1
        out = cache.decode_attn(q, SCALE, res_k=win_k[:, :, :n_win],
                                res_v=win_v[:, :, :n_win]).cpu().numpy()
        idx = np.r_[0, first_recent:t + 1]           # the window's tokens
        for h in range(H):
            ref = oracle.decode_attn_residual(streams[h], inp["q_bf16"][0, h * G:(h + 1) * G],
                                              SCALE, kf[0, h, idx], vf[0, h, idx])
            err = rel_err_rows(out[0, h * G:(h + 1) * G], ref).max()
            assert err <= REL_TOL, "token %d (packed %d, window %d): %.3e" % (
                t, cache.n_tokens, n_win, err)
    assert cache.n_tokens == 384


@pytest.mark.parametrize("B,H,Hq,T,bits,R", [(1, 1, 7, 32768, 4, 0), (2, 2, 8, 32768, 2, 100),
                                              (1, 2, 8, 24576, 8, 0)])
def test_decode_many_chunks(B, H, Hq, T, bits, R):
    """Few streams over many tokens: the plan cuts each stream into 48 or more
    chunks (the combine kernel's preload of 64 slots, residual slots past them
    when R > 0).  Against the oracle; repeated calls give identical bits."""
    print("case many chunks B=%d H=%d Hq=%d T=%d bits=%d R=%d" % (B, H, Hq, T, bits, R), flush=True)
    if R:
        _residual_case(B, H, Hq, T, R, bits, kvq.F16, torch.bfloat16, seed=970 + T % 97)
        return
    inp, cache = _quantized(B, H, Hq, T, bits, bits, kvq.F16, seed=971 + bits)
    q = q_to_dev(inp["q_bf16"], torch)
    o1 = cache.decode_attn(q, SCALE)
    o2 = cache.decode_attn(q, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    out = o1.cpu().numpy()
    G = Hq // H
    for b in range(B):
        for h in range(H):
            ref = oracle_attn(oracle_stream(inp, b, h, bits, bits, kvq.F16), inp["q_bf16"][b, h * G:(h + 1) * G])
            assert rel_err_rows(out[b, h * G:(h + 1) * G], ref).max() <= REL_TOL
