"""Pair-granular key widths (PN-Mix page, abstract): the oracle's pair norms and
slot map pinned to closed forms, brute force and invariants, and the host
slot-map builder of the library against the oracle (host logic, no GPU)."""
import ctypes

import numpy as np
import pytest

import oracle
from kv_cache_mixed_amd import kvq, synth


def _widths(slot_chan_row):
    """channel -> width of one slot map row (mixed key layout slot classes)."""
    bits = oracle.mixed_slot_bits()
    return {int(c): int(bits[j]) for j, c in enumerate(slot_chan_row)}


# ---------------------------------------------------------------------------
# pair norms
# ---------------------------------------------------------------------------
def test_pair_norms_closed_form():
    """Pairs (3, 4) -> 5 per token; sums over batch, tokens and grouped heads."""
    B, H, T = 2, 4, 5
    x = np.zeros((B, H, T, 128), np.float32)
    x[..., :64] = 3.0
    x[..., 64:] = 4.0
    x[:, 1, :, 10] = 0.0          # pair 10 of head 1: |(0, 4)| = 4
    x[:, 1, :, 74] = 4.0
    n1 = oracle.pair_norms(x, 1)
    assert n1.shape == (4, 64)
    assert np.all(n1[[0, 2, 3]] == 5.0 * B * T)
    assert n1[1, 10] == 4.0 * B * T and np.all(np.delete(n1[1], 10) == 5.0 * B * T)
    n2 = oracle.pair_norms(x, 2)
    assert n2.shape == (2, 64)
    assert np.allclose(n2, n1[0::2] + n1[1::2], rtol=0, atol=0)


def test_pair_norms_bruteforce():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 3, 7, 128)).astype(np.float32)
    ref = np.zeros((3, 64))
    for b in range(2):
        for h in range(3):
            for t in range(7):
                for p in range(64):
                    a, c = float(x[b, h, t, p]), float(x[b, h, t, p + 64])
                    ref[h, p] += (a * a + c * c) ** 0.5
    assert np.allclose(oracle.pair_norms(x, 1), ref, rtol=1e-13, atol=0)


def test_pair_norms_are_rope_invariant():
    """The pairs are the RoPE rotation's planes: rotating every token leaves
    every pair norm unchanged (pairing (2i, 2i+1) or a transposed index would
    not)."""
    rng = np.random.default_rng(6)
    x = rng.standard_normal((1, 2, 300, 128)).astype(np.float32)
    xr = np.stack([synth.apply_rope(x[0, h], 1000) for h in range(2)])[None]
    a, b = oracle.pair_norms(x, 1), oracle.pair_norms(xr, 1)
    assert np.allclose(a, b, rtol=1e-6, atol=0)
    # a different pairing is not invariant
    perm = np.concatenate([np.arange(0, 128, 2), np.arange(1, 128, 2)])
    assert not np.allclose(oracle.pair_norms(x[..., perm], 1), oracle.pair_norms(xr[..., perm], 1), rtol=1e-3)


# ---------------------------------------------------------------------------
# slot map
# ---------------------------------------------------------------------------
def test_slot_map_hand_example():
    """score(p) = p: pairs 63..60 are the 4-bit class, 59..56 the 3-bit class,
    0..3 the 1-bit class."""
    s = np.arange(64, dtype=np.float32)[None]
    m = oracle.pair_slot_map(s)[0]
    assert list(m[0:8]) == [60, 61, 62, 63, 124, 125, 126, 127]
    assert list(m[8:24:2]) == [56, 57, 58, 59, 120, 121, 122, 123]
    assert list(m[9:24:2]) == [0, 1, 2, 3, 64, 65, 66, 67]
    rest = sorted(set(range(4, 56)) | set(range(68, 120)))
    assert list(m[24:]) == rest


def _check_map(score, m):
    for h in range(score.shape[0]):
        row = m[h]
        assert sorted(row.tolist()) == list(range(128))
        w = _widths(row)
        for p in range(64):
            assert w[p] == w[p + 64], "pair %d split across widths" % p
        counts = {b: sum(1 for c in w if w[c] == b) for b in (4, 3, 2, 1)}
        assert counts == {4: 8, 3: 8, 2: 104, 1: 8}
        for lo, hi in ((0, 8), (24, 128)):
            assert list(row[lo:hi]) == sorted(row[lo:hi])
        assert list(row[8:24:2]) == sorted(row[8:24:2]) and list(row[9:24:2]) == sorted(row[9:24:2])
        rank = {4: 0, 3: 1, 2: 2, 1: 3}
        for p in range(64):
            for q in range(64):
                if rank[w[p]] < rank[w[q]]:       # p in a higher class than q
                    assert score[h, p] > score[h, q] or (score[h, p] == score[h, q] and p < q)


def test_slot_map_properties():
    rng = np.random.default_rng(7)
    for i in range(20):
        s = rng.standard_normal((3, 64)).astype(np.float32)
        if i % 3 == 0:
            s = np.round(s)                  # many ties
        _check_map(s, oracle.pair_slot_map(s))


def test_slot_map_library_matches_oracle():
    kvq.load()
    rng = np.random.default_rng(8)
    for i in range(200):
        s = rng.standard_normal((4, 64)).astype(np.float32)
        if i % 4 == 0:
            s = np.round(s * 2) / 2
        if i % 7 == 0:
            s[:, ::3] = 0.0
            s[:, 1::5] = -0.0
        assert np.array_equal(kvq.pair_slot_map(s), oracle.pair_slot_map(s))


def test_slot_map_validation():
    L = kvq.load()
    out = np.zeros((1, 128), np.int16)
    for bad in (np.nan, np.inf, -np.inf):
        s = np.zeros((1, 64), np.float32)
        s[0, 5] = bad
        assert L.kvq_pair_slot_map(s.ctypes.data, 1, out.ctypes.data) == kvq.EINVAL
    s = np.zeros((1, 64), np.float32)
    assert L.kvq_pair_slot_map(s.ctypes.data, 0, out.ctypes.data) == kvq.EINVAL
    assert L.kvq_pair_slot_map(None, 1, out.ctypes.data) == kvq.EINVAL
    assert np.all(out == 0)                  # untouched on error


def test_pair_norms_argument_validation():
    """Rejected before any launch (no GPU needed)."""
    L = kvq.load()
    st = (ctypes.c_int64 * 3)(4 * 8 * 128, 8 * 128, 128)
    buf = ctypes.c_void_p(16)               # never dereferenced: validation fails first
    assert L.kvq_pair_norms(buf, kvq.F16, st, 1, 4, 8, 1, buf, None) == kvq.EINVAL     # dtype
    assert L.kvq_pair_norms(buf, kvq.F32, st, 1, 4, 8, 3, buf, None) == kvq.EINVAL     # group
    bad = (ctypes.c_int64 * 3)(4 * 8 * 128, 8 * 128, 64)
    assert L.kvq_pair_norms(buf, kvq.F32, bad, 1, 4, 8, 1, buf, None) == kvq.EINVAL    # token stride
    assert L.kvq_pair_norms(None, kvq.F32, st, 1, 4, 8, 1, buf, None) == kvq.EINVAL
    assert L.kvq_pair_norms(None, kvq.F32, st, 1, 4, 0, 1, buf, None) == kvq.OK        # nothing to read
    assert L.kvq_pair_norms(buf, kvq.F32, st, 0, 4, 8, 1, buf, None) == kvq.EINVAL


def test_pairs_recipe_classes_recovered():
    """On the pairs recipe the map from prefill query and key pair norms puts
    the x8 pairs at 4 bits, the x4 pairs at 3 bits and the x0.2 pairs at 1 bit."""
    d = synth.pair_layer(1, 3, 12, 512, 11)
    score = (oracle.pair_norms(d["q_prefill"], 4) * oracle.pair_norms(d["k"], 1)).astype(np.float32)
    m = oracle.pair_slot_map(score)
    want = {np.float32(8.0): 4, np.float32(4.0): 3, np.float32(0.2): 1, np.float32(1.0): 2}
    for h in range(3):
        w = _widths(m[h])
        for p in range(64):
            assert w[p] == want[np.float32(d["pair_scale"][h, p])], (h, p)
