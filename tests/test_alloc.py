"""Block-wise bit-width allocation (PM-KVQ Key design 2): the library's exact
dynamic programme (host code of libkvq.so) against enumeration, and the
enumeration against cases whose answer is known in closed form."""
import ctypes

import numpy as np
import pytest

import oracle
from kv_cache_mixed_amd import kvq


def _lib_or_skip():
    try:
        return kvq.load()
    except RuntimeError as e:
        pytest.skip(str(e))


def test_bruteforce_closed_forms():
    """Enumeration pinned by cases with a known answer: an unbounded budget
    lets every block take its own least-sensitive choice; the tightest budget
    forces the cheapest choice of every block; a hand-worked 3-block case."""
    rng = np.random.default_rng(3)
    s = rng.random((5, 3))
    w = np.array([[1, 2, 4]] * 5) * 1000
    ch, c = oracle.allocate_bits_bruteforce(s, w, 10 ** 9)
    assert ch == list(np.argmin(s, axis=1))
    ch, c = oracle.allocate_bits_bruteforce(s, w, 5000)
    assert ch == [0] * 5
    assert oracle.allocate_bits_bruteforce(s, w, 4999) == (None, None)
    # 3 blocks, widths {2, 4} costing 2 / 4 units, sensitivities (2-bit, 4-bit):
    # block 0 (5, 1), block 1 (3, 2), block 2 (9, 0); budget 8 units: one block
    # can be 4-bit -> block 2 (saves 9) ; budget 10: blocks 2 and 0 (saves 9 + 4)
    s3 = [[5.0, 1.0], [3.0, 2.0], [9.0, 0.0]]
    w3 = [[2, 4]] * 3
    assert oracle.allocate_bits_bruteforce(s3, w3, 8) == ([0, 0, 1], 8.0)
    assert oracle.allocate_bits_bruteforce(s3, w3, 10) == ([1, 0, 1], 4.0)
    assert oracle.allocate_bits_bruteforce(s3, w3, 12) == ([1, 1, 1], 3.0)
    # ties: equal sums, the lexicographically smallest vector
    assert oracle.allocate_bits_bruteforce([[1.0, 1.0], [1.0, 1.0]], [[1, 1], [1, 1]], 2) == ([0, 0], 2.0)


@pytest.mark.parametrize("seed", range(12))
def test_dp_matches_enumeration(seed):
    _lib_or_skip()
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 7))
    m = int(rng.integers(1, 5))
    unit = int(rng.choice([1, 7, 4096, 33554432]))
    w = rng.integers(1, 9, size=(n, m)) * unit
    if seed % 3 == 0:
        s = rng.integers(0, 4, size=(n, m)).astype(np.float64)     # many ties
    else:
        s = rng.random((n, m)) * 10.0 ** rng.integers(-3, 4)
    lo, hi = int(w.min(axis=1).sum()), int(w.max(axis=1).sum())
    for budget in (lo, (lo + hi) // 2, hi, hi + 3 * unit):
        want, want_cost = oracle.allocate_bits_bruteforce(s, w, budget)
        got, got_cost = kvq.allocate_bits(s, w, budget)
        assert got.tolist() == want and got_cost == want_cost, (n, m, budget)


def test_dp_errors():
    L = _lib_or_skip()
    s = np.zeros((2, 2))
    w = np.array([[2, 4], [2, 4]], dtype=np.int64)
    ch = np.zeros(2, dtype=np.int32)
    P = lambda a: a.ctypes.data
    assert L.kvq_allocate_bits(2, 2, P(s), P(w), 3, P(ch), None) == kvq.EBUDGET
    assert L.kvq_allocate_bits(0, 2, P(s), P(w), 8, P(ch), None) == kvq.EINVAL
    assert L.kvq_allocate_bits(2, 17, P(s), P(w), 8, P(ch), None) == kvq.EINVAL
    assert L.kvq_allocate_bits(2, 2, None, P(w), 8, P(ch), None) == kvq.EINVAL
    bad = np.array([[2, 0], [2, 4]], dtype=np.int64)
    assert L.kvq_allocate_bits(2, 2, P(s), P(bad), 8, P(ch), None) == kvq.EINVAL
    nan = np.array([[0.0, float("nan")], [0.0, 0.0]])
    assert L.kvq_allocate_bits(2, 2, P(nan), P(w), 8, P(ch), None) == kvq.EINVAL
    coprime = np.array([[1 << 30, (1 << 30) + 1], [1 << 30, (1 << 30) + 1]], dtype=np.int64)
    assert L.kvq_allocate_bits(2, 2, P(s), P(coprime), 1 << 40, P(ch), None) == kvq.EUNSUPPORTED


def test_more_sensitive_blocks_get_more_bits():
    """64 blocks, widths {2, 4, 8, 16} with the Qwen2.5-32B-shaped layer's
    cache bytes, s_{i,b} = a_i * 4^-b (synthetic: deeper blocks and block 0
    more sensitive, as the page reports), budget = 2.84 bits on average.  With
    equal bytes per block and a separable s, an exchange argument says widths
    never decrease with a_i; the budget is met and nearly used."""
    _lib_or_skip()
    L, widths = 64, [2, 4, 8, 16]
    a = 1.0 + 2.0 * np.arange(L) / (L - 1)
    a[0] = 4.0
    s = a[:, None] * np.array([4.0 ** -b for b in widths])[None, :]
    per_tok = np.array([32 * b + 8 for b in widths], dtype=np.int64)     # codes K+V + fp16 S/Z
    w = np.tile(16 * 8 * 32768 * per_tok, (L, 1))
    budget = int(16 * 8 * 32768 * (32 * 2.84 + 8) * L)
    ch, cost = kvq.allocate_bits(s, w, budget)
    got_bits = np.array(widths)[ch]
    order = np.argsort(a, kind="stable")
    assert np.all(np.diff(got_bits[order]) >= 0)
    used = int(w[np.arange(L), ch].sum())
    assert used <= budget and budget - used < int(w[0, 1] - w[0, 0])
    assert got_bits[0] == got_bits.max()           # block 0 is the most sensitive here


def _step_instance(L, B=16, H=8, T=32768):
    from kv_cache_mixed_amd import synth
    widths = (2, 4, 8)
    sens = synth.layer_sensitivities(L, widths, seed=0)
    per = [B * H * T * (128 * b // 8 * 2 + 4 * 2) for b in widths]
    nbytes = np.array([per] * L, dtype=np.int64)
    budget = int(0.195 * L * B * H * T * 128 * 2 * 2)
    return widths, sens, nbytes, budget


def test_step_widths_reduced_instance_matches_enumeration():
    """The allocation that drives the 64-layer step's widths, on a reduced
    instance of the same recipe (10 layers, the same budget fraction): the
    library's table equals the oracle's enumeration of all 3^10 tables."""
    _lib_or_skip()
    widths, sens, nbytes, budget = _step_instance(10)
    want, want_cost = oracle.allocate_bits_bruteforce(sens, nbytes, budget)
    got, got_cost = kvq.allocate_bits(sens, nbytes, budget)
    assert got.tolist() == want and got_cost == want_cost


def test_step_widths_full_instance():
    """64 layers at 19.5% of the 16-bit size: the table fits the budget, the
    first block takes 8 bits, deeper blocks hold more of the 4-bit widths,
    and no single swap of two blocks' widths (same bytes) or move of one block
    to a cheaper width lowers the objective."""
    _lib_or_skip()
    import bench
    widths, sens, nbytes, budget = _step_instance(64)
    bits, M, obj = bench.step_width_table(kvq, __import__("kv_cache_mixed_amd.synth").synth)
    assert M == budget
    ch = [widths.index(b) for b in bits]
    assert sum(int(nbytes[i][c]) for i, c in enumerate(ch)) <= budget
    assert bits[0] == 8 and 2.7 < np.mean(bits) < 3.0
    assert sum(b == 4 for b in bits[32:]) > sum(b == 4 for b in bits[1:32])
    total = sum(int(nbytes[i][c]) for i, c in enumerate(ch))
    base = sum(sens[i][c] for i, c in enumerate(ch))
    for i in range(64):
        for j in range(64):
            if ch[i] != ch[j]:
                alt = base - sens[i][ch[i]] - sens[j][ch[j]] + sens[i][ch[j]] + sens[j][ch[i]]
                assert alt >= base - 1e-12 * abs(base)
        for c in range(3):
            if total - nbytes[i][ch[i]] + nbytes[i][c] <= budget:
                assert base - sens[i][ch[i]] + sens[i][c] >= base - 1e-12 * abs(base)
