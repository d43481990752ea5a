"""GPU parity of the two-phase decode (kvq_decode_attn_partials, then
kvq_decode_combine) through the C ABI.

- The two phases back to back give kvq_decode_attn's output (bit for bit
  when the plan has several chunks: the same kernels run on the same plan).
- Every partial slot means what the header states: o / l is the attention
  over the slot's own tokens and m + log2(l) their log2-sum of 2^x, both
  against the oracle's reconstructed keys and values in float64.
- Partials of two caches that hold the two halves of each sequence, gathered
  into one array and combined, give the attention over the whole sequence
  (the token-split use of the combine).
"""
import math

import numpy as np
import pytest

import oracle
from kv_cache_mixed_amd import kvq, synth
from tests.gpu_helpers import PDT_ORACLE, REL_TOL, SCALE, oracle_attn, oracle_stream, q_to_dev, rel_err_rows, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LOG2E = 1.0 / math.log(2.0)


@pytest.fixture(scope="module", autouse=True)
def _setup():
    oracle.build(force=False)
    kvq.load()


def _cache(inp, B, H, T, kb, vb, pdt, t_lo=0, t_hi=None):
    """cache of tokens [t_lo, t_hi) of every stream of inp (multiples of 128)"""
    t_hi = T if t_hi is None else t_hi
    kw = {}
    if kb == kvq.KMIXED:
        kw["slot_chan"] = inp["slot_chan"]
    if vb == kvq.VMIXED:
        kw["v_slot_chan"] = inp["v_slot_chan"]
    c = kvq.PackedCache(B, H, t_hi - t_lo, kb, vb, pdt, **kw)
    c.quantize(to_dev(inp["k"][:, :, t_lo:t_hi], torch), to_dev(inp["v"][:, :, t_lo:t_hi], torch), 0)
    return c


def _inputs(B, H, Hq, T, kb, vb, seed):
    if vb == kvq.VMIXED:
        return synth.mixed_kv_layer(B, H, Hq, T, seed)
    if kb == kvq.KMIXED:
        return synth.mixed_layer(B, H, Hq, T, seed)
    return synth.layer(B, H, Hq, T, seed)


def _stream(inp, b, h, kb, vb, pdt):
    if vb == kvq.VMIXED:
        return oracle.quantize_stream(inp["k"][b, h], inp["v"][b, h], kb, vb, PDT_ORACLE[pdt],
                                      inp["slot_chan"][h], inp["v_slot_chan"][h])
    return oracle_stream(inp, b, h, kb, vb, pdt, inp["slot_chan"][h] if kb == kvq.KMIXED else None)


CASES = [
    # B, H, Hq, T, k_bits, v_bits, pdt
    (2, 2, 14, 4096, 4, 4, kvq.F16),
    (1, 2, 8, 8192, 2, 2, kvq.F16),
    (1, 2, 8, 4096, kvq.KMIXED, 2, kvq.E4M3),
    (1, 2, 8, 4096, kvq.KMIXED, kvq.VMIXED, kvq.E4M3),
    (2, 1, 5, 384, 8, 8, kvq.F16),
    (1, 1, 1, 128, 4, 4, kvq.E4M3),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%d_H%d_Hq%d_T%d_k%d_v%d" % c[:6])
def test_two_phases_give_decode_attn(case):
    B, H, Hq, T, kb, vb, pdt = case
    print("case two-phase", case, flush=True)
    inp = _inputs(B, H, Hq, T, kb, vb, seed=300 + T // 128 + kb)
    c = _cache(inp, B, H, T, kb, vb, pdt)
    q = q_to_dev(inp["q_bf16"], torch)
    ref = c.decode_attn(q, SCALE).clone()
    ws = torch.full((c.workspace_bytes(Hq),), 0xA5, dtype=torch.uint8, device="cuda")   # garbage contents
    n, tps = c.decode_partials(q, SCALE, workspace=ws)
    assert 1 <= n <= 128 and (n - 1) * tps < T // 128 <= n * tps
    out = kvq.decode_combine(ws, B, H, Hq, n)
    torch.cuda.synchronize()
    got, want = out.cpu().numpy(), ref.cpu().numpy()
    assert np.all(np.isfinite(got))
    if n > 1:
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    G = Hq // H
    worst = 0.0
    for b in range(B):
        for h in range(H):
            st = _stream(inp, b, h, kb, vb, pdt)
            r = oracle_attn(st, inp["q_bf16"][b, h * G:(h + 1) * G])
            worst = max(worst, rel_err_rows(got[b, h * G:(h + 1) * G], r).max())
    assert worst <= REL_TOL, worst


@pytest.mark.parametrize("case", CASES[:4], ids=lambda c: "B%d_H%d_Hq%d_T%d_k%d_v%d" % c[:6])
def test_partial_slots_mean_what_the_header_says(case):
    B, H, Hq, T, kb, vb, pdt = case
    print("case partial semantics", case, flush=True)
    inp = _inputs(B, H, Hq, T, kb, vb, seed=500 + T // 128 + kb)
    c = _cache(inp, B, H, T, kb, vb, pdt)
    q = q_to_dev(inp["q_bf16"], torch)
    ws = c.workspace(Hq)
    n, tps = c.decode_partials(q, SCALE, workspace=ws)
    torch.cuda.synchronize()
    ml, o = kvq.partials_views(ws, B, H, Hq, n)
    ml, o = ml.cpu().numpy().astype(np.float64), o.cpu().numpy().astype(np.float64)
    G = Hq // H
    sigma = float(np.float32(SCALE))
    for b in range(B):
        for h in range(H):
            st = _stream(inp, b, h, kb, vb, pdt)
            K, V = oracle.dequant_k(st), oracle.dequant_v(st)
            qf = oracle.decode(np.ascontiguousarray(inp["q_bf16"][b, h * G:(h + 1) * G]), oracle.BF16)
            x = sigma * LOG2E * (qf @ K.T)                                     # [G, T] log2 units
            bh = b * H + h
            for s in range(n):
                t0, t1 = 128 * s * tps, min(128 * (s + 1) * tps, T)
                xs = x[:, t0:t1]
                xmax = xs.max(axis=1)
                w = np.exp2(xs - xmax[:, None])
                lse = xmax + np.log2(w.sum(axis=1))                          # log2 sum_t 2^x_t
                attn = (w @ V[t0:t1]) / w.sum(axis=1)[:, None]
                m, l = ml[bh, s, :, 0], ml[bh, s, :, 1]
                assert np.all(m <= xmax + 1e-2) and np.all(m >= xmax - 8.0 - 1e-2), (b, h, s, m, xmax)
                assert np.all(np.abs(m + np.log2(l) - lse) <= 3e-3), (b, h, s)
                err = rel_err_rows(o[bh, s] / l[:, None], attn).max()
                assert err <= REL_TOL, (b, h, s, err)


@pytest.mark.parametrize("case", [(2, 2, 14, 4096, 4, 4, kvq.F16), (1, 2, 8, 4096, kvq.KMIXED, 2, kvq.E4M3)],
                         ids=["uniform4", "mixed_keys"])
def test_gathered_partials_of_two_token_shares(case):
    """Tokens [0, T/2) of every stream in one cache and [T/2, T) in another
    (as two devices would hold a split sequence): each cache's partials, the
    slots gathered per stream into one array, one combine."""
    B, H, Hq, T, kb, vb, pdt = case
    print("case gathered partials", case, flush=True)
    inp = _inputs(B, H, Hq, T, kb, vb, seed=700 + kb)
    half = T // 2
    ca = _cache(inp, B, H, T, kb, vb, pdt, 0, half)
    cb = _cache(inp, B, H, T, kb, vb, pdt, half, T)
    q = q_to_dev(inp["q_bf16"], torch)
    wa, wb = ca.workspace(Hq), cb.workspace(Hq)
    na, _ = ca.decode_partials(q, SCALE, workspace=wa)
    nb, _ = cb.decode_partials(q, SCALE, workspace=wb)
    n = na + nb
    ws = torch.empty(kvq.partials_bytes(B, H, Hq, n), dtype=torch.uint8, device="cuda")
    mla, oa = kvq.partials_views(wa, B, H, Hq, na)
    mlb, ob = kvq.partials_views(wb, B, H, Hq, nb)
    ml, o = kvq.partials_views(ws, B, H, Hq, n)
    ml[:, :na].copy_(mla)
    ml[:, na:].copy_(mlb)
    o[:, :na].copy_(oa)
    o[:, na:].copy_(ob)
    out = kvq.decode_combine(ws, B, H, Hq, n).cpu().numpy()
    G = Hq // H
    worst = 0.0
    for b in range(B):
        for h in range(H):
            st = _stream(inp, b, h, kb, vb, pdt)
            r = oracle_attn(st, inp["q_bf16"][b, h * G:(h + 1) * G])
            worst = max(worst, rel_err_rows(out[b, h * G:(h + 1) * G], r).max())
    assert worst <= REL_TOL, worst
