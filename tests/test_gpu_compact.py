"""GPU parity of the compacted-softmax decode instances.

With one kv stream per wave whose heads fill at most half (a quarter) of the
16 MFMA columns, the decode kernel spreads each head's logits and query fold
over two (four) lanes of its MFMA row and gathers the operands back for the
two products (2-, 4- and 8-bit values with keys of the same width, 2-bit or
mixed values with mixed-width keys).  The cases below
force that plan (few streams and tiles) for every group size, every
parameter dtype, a softmax whose reference max moves inside tiles (the rescale
branch and its reductions over the lane parts), a negative scale and ragged
chunk splits; each is gated against the float64 oracle at the per-row
relative error of 2e-3 (ChanMix page, Overall framework: dequantize, then
ordinary attention).
"""
import numpy as np
import pytest

import oracle
from kv_cache_mixed_amd import kvq, synth
from tests.gpu_helpers import PDT_ORACLE, REL_TOL, SCALE, q_to_dev, rel_err_rows, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    oracle.build(force=False)
    kvq.load()


def _check(k, v, q_bits, kb, pdt, scale, slot_chan=None, what="", vb=2):
    B, H, T, _ = k.shape
    G = q_bits.shape[1] // H
    print("case %s B=%d H=%d G=%d T=%d kb=%d vb=%d pdt=%d scale=%g" % (what, B, H, G, T, kb, vb, pdt, scale), flush=True)
    cache = kvq.PackedCache(B, H, T, kb, vb, pdt, slot_chan=slot_chan)
    cache.quantize(to_dev(k, torch), to_dev(v, torch), 0)
    out = cache.decode_attn(q_to_dev(q_bits, torch), scale).cpu().numpy()
    assert np.all(np.isfinite(out)), what
    worst = 0.0
    for b in range(B):
        for h in range(H):
            st = oracle.quantize_stream(k[b, h], v[b, h], kb, vb, PDT_ORACLE[pdt],
                                        None if slot_chan is None else slot_chan[h])
            ref = oracle.decode_attn(st, q_bits[b, h * G:(h + 1) * G], scale)
            worst = max(worst, rel_err_rows(out[b, h * G:(h + 1) * G], ref).max())
    assert worst <= REL_TOL, "%s: max row relative error %.3e" % (what, worst)


@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 7, 8])
@pytest.mark.parametrize("pdt", [kvq.E4M3, kvq.F16, kvq.BF16, kvq.F32])
def test_mixed_keys_compacted(G, pdt):
    inp = synth.mixed_layer(1, 2, 2 * G, 2944, seed=300 + 10 * G + pdt)
    _check(inp["k"], inp["v"], inp["q_bf16"], kvq.KMIXED, pdt, SCALE, inp["slot_chan"], what="mixed G=%d" % G)


@pytest.mark.parametrize("G", [1, 3, 4, 6, 8])
@pytest.mark.parametrize("pdt", [kvq.F16, kvq.E4M3, kvq.BF16, kvq.F32])
def test_two_bit_compacted(G, pdt):
    inp = synth.layer(2, 1, G, 3200, seed=400 + 10 * G + pdt)
    _check(inp["k"], inp["v"], inp["q_bf16"], 2, pdt, SCALE, what="2-bit G=%d" % G)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("G", [1, 3, 4, 6, 8])
@pytest.mark.parametrize("pdt", [kvq.F16, kvq.E4M3, kvq.BF16, kvq.F32])
def test_wider_codes_compacted(bits, G, pdt):
    """4- and 8-bit codes: sub-tiles of 8 tokens per lane group, so a part
    holds one (four parts) or two (two parts) probability registers."""
    inp = synth.layer(2, 1, G, 2944, seed=800 + 10 * G + pdt + bits)
    _check(inp["k"], inp["v"], inp["q_bf16"], bits, pdt, SCALE, what="%d-bit G=%d" % (bits, G), vb=bits)


@pytest.mark.parametrize("kb,G", [(2, 4), (2, 7), (kvq.KMIXED, 4), (kvq.KMIXED, 6), (4, 3), (4, 7), (8, 4), (8, 8)])
def test_compacted_climbing_logits(kb, G):
    """Keys ramped along each head's query: logits climb by ~40 log2 units
    inside every tile and across tiles, so the per-column reference moves
    (reductions over the lane parts of a row) in most sub-tiles."""
    rng = np.random.default_rng(500 + G + (kb or 50))
    B, H, T = 1, 2, 4096
    k = rng.standard_normal((B, H, T, 128)).astype(np.float32)
    v = rng.standard_normal((B, H, T, 128)).astype(np.float32)
    q = rng.standard_normal((B, H * G, 128)).astype(np.float32)
    t = np.arange(T)
    ramp = (t % 128) / 127.0 * 3.0 + (t // 128) / (T // 128)
    for h in range(H):
        d = q[0, h * G] / np.linalg.norm(q[0, h * G])
        k[0, h] += (ramp[:, None] * d[None, :] * 10.0).astype(np.float32)
    slot_chan = None
    if kb == kvq.KMIXED:
        slot_chan = synth.mixed_layer(1, H, H * G, 128, seed=510)["slot_chan"]
    vb = 2 if kb in (2, kvq.KMIXED) else kb
    _check(k, v, synth.to_bf16_bits(q), kb, kvq.F16, SCALE, slot_chan, what="climbing kb=%d G=%d" % (kb, G), vb=vb)
    _check(k, v, synth.to_bf16_bits(q), kb, kvq.E4M3, -SCALE, slot_chan, what="climbing, negative kb=%d G=%d" % (kb, G),
           vb=vb)


def test_compacted_128k_sequence_sampled():
    """A single 128K-token sequence of mixed keys (the long-context layer's
    launch: one stream per wave, 64 chunk partials), checked on sampled heads."""
    B, H, G, T = 1, 2, 4, 131072
    inp = synth.mixed_layer(B, H, H * G, T, seed=520)
    cache = kvq.PackedCache(B, H, T, kvq.KMIXED, 2, kvq.E4M3, slot_chan=inp["slot_chan"])
    cache.quantize(to_dev(inp["k"], torch), to_dev(inp["v"], torch), 0)
    out = cache.decode_attn(q_to_dev(inp["q_bf16"], torch), SCALE).cpu().numpy()
    for h in range(H):
        st = oracle.quantize_stream(inp["k"][0, h], inp["v"][0, h], kvq.KMIXED, 2, PDT_ORACLE[kvq.E4M3],
                                    inp["slot_chan"][h])
        ref = oracle.decode_attn(st, inp["q_bf16"][0, h * G:(h + 1) * G], SCALE)
        assert rel_err_rows(out[0, h * G:(h + 1) * G], ref).max() <= REL_TOL


@pytest.mark.parametrize("kb,B,H,G,T", [(2, 16, 8, 4, 32768), (2, 16, 8, 2, 32768), (kvq.KMIXED, 4, 8, 2, 65536)],
                         ids=["2bit_g4", "2bit_g2", "mixed_g2"])
def test_compacted_two_streams_sampled(kb, B, H, G, T):
    """Layers with chunks long enough for two streams per wave whose heads
    fill half (G = 4) or a quarter (G = 2) of the MFMA columns (these keep
    the uncompacted softmax): sampled streams, both members of a stream pair
    among them, and the two decode phases reproduce the call bit for bit."""
    Hq = H * G
    print("case two streams kb=%d B=%d H=%d G=%d T=%d" % (kb, B, H, G, T), flush=True)
    if kb == kvq.KMIXED:
        dev = synth.mixed_layer_device(B, H, Hq, T, seed=530 + G, device="cuda")
        cache = kvq.PackedCache(B, H, T, kb, 2, kvq.E4M3, slot_chan=dev["slot_chan"])
        pdt = kvq.E4M3
    else:
        dev = synth.layer_device(B, H, Hq, T, seed=540 + G, device="cuda")
        cache = kvq.PackedCache(B, H, T, kb, 2, kvq.F16)
        pdt = kvq.F16
    cache.quantize(dev["k"], dev["v"], 0)
    out = cache.decode_attn(dev["q"], SCALE).cpu().numpy()
    assert np.isfinite(out).all()
    ws = cache.workspace(Hq)
    n, tps = cache.decode_partials(dev["q"], SCALE, workspace=ws)
    assert n * tps >= T // 128 and (n - 1) * tps < T // 128
    two = kvq.decode_combine(ws, B, H, Hq, n).cpu().numpy()
    assert np.array_equal(two.view(np.uint32), out.view(np.uint32))
    q_bits = dev["q"].view(torch.int16).cpu().numpy().view(np.uint16)
    for b, h in [(0, 0), (0, 1), (B // 2, 5), (B - 1, 6), (B - 1, 7)]:
        k = dev["k"][b, h].cpu().numpy()
        v = dev["v"][b, h].cpu().numpy()
        sc = None if kb != kvq.KMIXED else np.asarray(dev["slot_chan"])[h]
        st = oracle.quantize_stream(k, v, kb, 2, PDT_ORACLE[pdt], sc)
        ref = oracle.decode_attn(st, q_bits[b, h * G:(h + 1) * G], SCALE)
        err = rel_err_rows(out[b, h * G:(h + 1) * G], ref).max()
        assert err <= REL_TOL, "stream (%d,%d) rel err %.3e" % (b, h, err)


@pytest.mark.parametrize("G", [2, 3, 4, 5, 8])
@pytest.mark.parametrize("pdt", [kvq.E4M3, kvq.F16])
def test_mixed_values_compacted(G, pdt):
    """Mixed-width keys and values (4/3/1/2-bit value classes in 4- and 2-bit
    field containers, whose probability registers pair tokens differently)."""
    inp = synth.mixed_kv_layer(1, 2, 2 * G, 2432, seed=700 + 10 * G + pdt)
    print("case mixed K+V G=%d pdt=%d" % (G, pdt), flush=True)
    cache = kvq.PackedCache(1, 2, 2432, kvq.KMIXED, kvq.VMIXED, pdt, slot_chan=inp["slot_chan"],
                            v_slot_chan=inp["v_slot_chan"])
    cache.quantize(to_dev(inp["k"], torch), to_dev(inp["v"], torch), 0)
    for scale in (SCALE, -SCALE):
        out = cache.decode_attn(q_to_dev(inp["q_bf16"], torch), scale).cpu().numpy()
        assert np.all(np.isfinite(out))
        for h in range(2):
            st = oracle.quantize_stream(inp["k"][0, h], inp["v"][0, h], kvq.KMIXED, kvq.VMIXED, PDT_ORACLE[pdt],
                                        inp["slot_chan"][h], inp["v_slot_chan"][h])
            ref = oracle.decode_attn(st, inp["q_bf16"][0, h * G:(h + 1) * G], scale)
            err = rel_err_rows(out[0, h * G:(h + 1) * G], ref).max()
            assert err <= REL_TOL, "mixed K+V G=%d scale=%g head %d: %.3e" % (G, scale, h, err)


@pytest.mark.parametrize("G", [4, 7])
def test_mixed_values_compacted_climbing(G):
    """Mixed K+V with keys ramped along each head's query (the rescale of the
    four per-class zero-point sums across the lane parts)."""
    T = 4096
    inp = synth.mixed_kv_layer(1, 2, 2 * G, T, seed=750 + G)
    k = inp["k"].copy()
    q = synth.bf16_bits_to_f32(inp["q_bf16"])
    t = np.arange(T)
    ramp = (t % 128) / 127.0 * 3.0 + (t // 128) / (T // 128)
    for h in range(2):
        d = q[0, h * G] / np.linalg.norm(q[0, h * G])
        k[0, h] += (ramp[:, None] * d[None, :] * 10.0).astype(np.float32)
    cache = kvq.PackedCache(1, 2, T, kvq.KMIXED, kvq.VMIXED, kvq.E4M3, slot_chan=inp["slot_chan"],
                            v_slot_chan=inp["v_slot_chan"])
    cache.quantize(to_dev(k, torch), to_dev(inp["v"], torch), 0)
    out = cache.decode_attn(q_to_dev(inp["q_bf16"], torch), SCALE).cpu().numpy()
    for h in range(2):
        st = oracle.quantize_stream(k[0, h], inp["v"][0, h], kvq.KMIXED, kvq.VMIXED, PDT_ORACLE[kvq.E4M3],
                                    inp["slot_chan"][h], inp["v_slot_chan"][h])
        ref = oracle.decode_attn(st, inp["q_bf16"][0, h * G:(h + 1) * G], SCALE)
        err = rel_err_rows(out[0, h * G:(h + 1) * G], ref).max()
        assert err <= REL_TOL, "mixed K+V climbing G=%d head %d: %.3e" % (G, h, err)
