"""GPU parity of the per-token split between two precisions (SemKV page,
abstract: every token is kept; tokens ranked by a model-internal score go to
one of two adjacent precisions): the gathered quantize (kvq_quantize_tokens)
bit-exact against the oracle quantizing the same rows, and the decode over
both caches (kvq_decode_attn_split) within the 2e-3 row gate of the oracle's
attention over the union of the reconstructed tokens."""
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


def _split_case(B, H, G, T, n_high, hi, lo, seed, pdt=kvq.F16, pairs=None, what=""):
    """hi / lo: (k_bits, v_bits) of the two caches; k_bits 0 = mixed keys"""
    print("case split %s B=%d H=%d G=%d T=%d n_high=%d hi=%s lo=%s" % (what, B, H, G, T, n_high, hi, lo), flush=True)
    if 0 in (hi[0], lo[0]):
        inp = synth.mixed_layer(B, H, H * G, T, seed)
    else:
        inp = synth.layer(B, H, H * G, T, seed)
    sc = np.linalg.norm(inp["k"], axis=-1).reshape(B * H, T).astype(np.float32)   # key norm as the score
    order = kvq.rank_tokens(sc, n_high)
    assert np.array_equal(order, oracle.rank_tokens(sc, n_high))
    order = order.reshape(B, H, T)
    kd, vd = to_dev(inp["k"], torch), to_dev(inp["v"], torch)
    caches, sets = [], []
    for (kb, vb), sel in ((hi, order[:, :, :n_high]), (lo, order[:, :, n_high:])):
        n = sel.shape[2]
        slot = inp.get("slot_chan") if kb == 0 else None
        c = kvq.PackedCache(B, H, max(n, 128), kb, vb, pdt, slot_chan=slot)
        if n:
            c.quantize_tokens(kd, vd, to_dev(np.ascontiguousarray(sel, dtype=np.int32), torch))
        caches.append(c)
        sets.append(sel)
    torch.cuda.synchronize()
    q = q_to_dev(inp["q_bf16"], torch)
    out = kvq.decode_attn_split(caches[0], caches[1], q, SCALE).cpu().numpy()
    assert np.all(np.isfinite(out))
    worst = 0.0
    for (b, h) in (pairs or [(b, h) for b in range(B) for h in range(H)]):
        sts = []
        for (kb, vb), sel, c in zip((hi, lo), sets, caches):
            if sel.shape[2] == 0:
                sts.append(None)
                continue
            rows = sel[b, h]
            st = oracle.quantize_stream(inp["k"][b, h][rows], inp["v"][b, h][rows], kb, vb, PDT_ORACLE[pdt],
                                        inp["slot_chan"][h] if kb == 0 else None)
            assert_stream_bytes_equal(c, st, b, h, "split %s" % what)
            sts.append(st)
        ref = oracle.decode_attn_union(sts, inp["q_bf16"][b, h * G:(h + 1) * G], SCALE)
        worst = max(worst, rel_err_rows(out[b, h * G:(h + 1) * G], ref).max())
    assert worst <= REL_TOL, "%s: max row relative error %.3e" % (what, worst)
    return worst


def test_split_4_and_2_bits():
    _split_case(2, 2, 4, 1024, 256, (4, 4), (2, 2), seed=400, what="4/2")


def test_split_8_and_4_bits_e4m3_groups_of_7():
    _split_case(1, 2, 7, 768, 384, (8, 8), (4, 4), seed=401, pdt=kvq.E4M3, what="8/4 e4m3")


def test_split_one_side_empty():
    _split_case(1, 2, 4, 512, 0, (4, 4), (2, 2), seed=402, what="empty high side")
    _split_case(1, 2, 4, 512, 512, (4, 4), (2, 2), seed=403, what="empty low side")


def test_split_mixed_keys_low_side():
    _split_case(1, 2, 4, 768, 256, (4, 4), (0, 2), seed=404, pdt=kvq.E4M3, what="4-bit / mixed keys")


def test_split_long_context_many_chunks():
    _split_case(1, 4, 4, 32768, 8192, (4, 4), (2, 2), seed=405, pairs=[(0, 0), (0, 3)], what="long")


def test_split_same_width_equals_one_cache():
    """Two caches at the same width holding tiles of one stream's tokens in
    position order give the single-cache decode's result (both within the
    gate of the oracle, and within 1e-5 of each other)."""
    B, H, G, T = 1, 2, 4, 1024
    inp = synth.layer(B, H, H * G, T, seed=406)
    kd, vd = to_dev(inp["k"], torch), to_dev(inp["v"], torch)
    whole = kvq.PackedCache(B, H, T, 4, 4, kvq.F16)
    whole.quantize(kd, vd, 0)
    parts = []
    for lo_t, hi_t in ((0, 384), (384, T)):
        c = kvq.PackedCache(B, H, hi_t - lo_t, 4, 4, kvq.F16)
        tok = np.broadcast_to(np.arange(lo_t, hi_t, dtype=np.int32), (B, H, hi_t - lo_t))
        c.quantize_tokens(kd, vd, to_dev(np.ascontiguousarray(tok), torch))
        parts.append(c)
    q = q_to_dev(inp["q_bf16"], torch)
    a = whole.decode_attn(q, SCALE).cpu().numpy()
    b = kvq.decode_attn_split(parts[0], parts[1], q, SCALE).cpu().numpy()
    assert rel_err_rows(b, a).max() <= 1e-5


def test_gather_clamps_out_of_range_rows():
    """Indices below 0 read row 0 and indices past the input read its last
    row (bytes equal to the oracle quantizing the clamped rows)."""
    B, H, T = 1, 1, 256
    inp = synth.layer(B, H, 4, T, seed=407)
    kd, vd = to_dev(inp["k"], torch), to_dev(inp["v"], torch)
    tok = np.arange(128, dtype=np.int32)[None, None, :].copy()
    tok[0, 0, :10] = -5
    tok[0, 0, 10:20] = T + 3
    c = kvq.PackedCache(B, H, 128, 4, 4, kvq.F16)
    c.quantize_tokens(kd, vd, to_dev(tok, torch))
    rows = np.clip(tok[0, 0], 0, T - 1)
    st = oracle.quantize_stream(inp["k"][0, 0][rows], inp["v"][0, 0][rows], 4, 4, oracle.F16)
    assert_stream_bytes_equal(c, st, 0, 0, "clamped gather")
