"""Per-token split between two precisions (SemKV page, abstract: every token
is kept; tokens ranked by a model-internal score get one of two adjacent
precisions).  CPU pins of the oracle's ranking and union attention, and the
library's host ranking against the oracle."""
import math

import numpy as np
import pytest

import oracle
from kv_cache_mixed_amd import kvq


@pytest.fixture(scope="module", autouse=True)
def _build():
    oracle.build(force=False)


def test_rank_tokens_brute_force():
    """Top set: every chosen token scores at least as high as every other;
    among equal scores the earlier tokens are chosen (brute force over all
    pairs, with many ties); each part ascending; a permutation of 0..T-1."""
    rng = np.random.default_rng(3)
    for trial in range(20):
        S, T = 3, int(rng.integers(1, 40))
        sc = rng.integers(0, 4, (S, T)).astype(np.float32) if trial % 2 else rng.standard_normal((S, T)).astype(np.float32)
        n_high = int(rng.integers(0, T + 1))
        order = oracle.rank_tokens(sc, n_high)
        for s in range(S):
            hi, lo = list(order[s, :n_high]), list(order[s, n_high:])
            assert sorted(hi + lo) == list(range(T))
            assert hi == sorted(hi) and lo == sorted(lo)
            for a in hi:
                for b in lo:
                    assert sc[s, a] > sc[s, b] or (sc[s, a] == sc[s, b] and a < b)


def test_rank_tokens_library_matches_oracle():
    try:
        kvq.load()
    except RuntimeError as e:
        pytest.skip(str(e))
    rng = np.random.default_rng(4)
    for T, n_high in ((1, 0), (1, 1), (37, 5), (256, 128), (1000, 333)):
        sc = rng.integers(0, 6, (4, T)).astype(np.float32) * np.float32(0.25)
        sc[1] = rng.standard_normal(T).astype(np.float32)
        assert np.array_equal(kvq.rank_tokens(sc, n_high), oracle.rank_tokens(sc, n_high))
    with pytest.raises(kvq.KvqError):
        kvq.rank_tokens(np.array([[1.0, np.nan]], np.float32), 1)
    with pytest.raises(kvq.KvqError):
        kvq.rank_tokens(np.zeros((1, 4), np.float32), 5)


def _stream(k, v, bits):
    return oracle.quantize_stream(k, v, bits, bits, oracle.F16)


def test_union_of_a_split_at_a_tile_boundary_equals_the_whole_stream():
    """Tokens [0, 256) in one stream and [256, 640) in another, at the same
    width: their tiles are the whole stream's tiles, so the union attention
    equals the single-stream oracle (two-pass, in C) on all 640 tokens."""
    rng = np.random.default_rng(5)
    k = rng.standard_normal((640, 128)).astype(np.float32)
    v = rng.standard_normal((640, 128)).astype(np.float32)
    q = oracle.narrow(rng.standard_normal((4, 128)).astype(np.float32), oracle.BF16)
    scale = 1 / math.sqrt(128)
    for bits in (4, 2):
        whole = oracle.decode_attn(_stream(k, v, bits), q, scale)
        a, b = _stream(k[:256], v[:256], bits), _stream(k[256:], v[256:], bits)
        assert np.allclose(oracle.decode_attn_union([a, b], q, scale), whole, rtol=1e-12, atol=1e-14)
        assert np.allclose(oracle.decode_attn_union([b, a], q, scale), whole, rtol=1e-12, atol=1e-14)
        assert np.allclose(oracle.decode_attn_union([None, a], q, scale), oracle.decode_attn(a, q, scale),
                           rtol=1e-12, atol=1e-14)


def test_union_equal_keys_is_the_mean_of_values():
    """Every key equal: all logits equal, so the output is the plain mean of
    the reconstructed values of both streams (different widths)."""
    rng = np.random.default_rng(6)
    kr = rng.standard_normal(128).astype(np.float32)
    k = np.tile(kr, (384, 1))
    v = rng.standard_normal((384, 128)).astype(np.float32)
    a, b = _stream(k[:128], v[:128], 4), _stream(k[128:], v[128:], 2)
    q = oracle.narrow(rng.standard_normal((2, 128)).astype(np.float32), oracle.BF16)
    mean = np.concatenate([oracle.dequant_v(a), oracle.dequant_v(b)]).mean(axis=0)
    out = oracle.decode_attn_union([a, b], q, 1 / math.sqrt(128))
    assert np.allclose(out, mean[None, :], rtol=1e-12, atol=1e-14)
