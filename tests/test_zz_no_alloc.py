"""The allocation-free decode entry point (kvq_decode_attn_noalloc) against
kvq_decode_attn on the same caches: two calls in a row, the second with a
smaller input, through the C ABI; each output equals the workspace entry
point's bit for bit (same kernels, same launch plan) and both are within the
2e-3 row gate of the float64 oracle on sampled streams.  Also a call whose
plan needs more scratch than the library's array is rejected before any
device work."""
import numpy as np
import pytest

import oracle
from kv_cache_mixed_amd import kvq, synth
from tests.gpu_helpers import REL_TOL, SCALE, oracle_attn, oracle_stream, q_to_dev, rel_err_rows, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    oracle.build(force=False)
    kvq.load()


def _case(B, H, Hq, T, bits, seed):
    inp = synth.layer(B, H, Hq, T, seed)
    cache = kvq.PackedCache(B, H, T, bits, bits, kvq.F16)
    cache.quantize(to_dev(inp["k"], torch), to_dev(inp["v"], torch), 0)
    return inp, cache


def _check(inp, cache, bits, pairs):
    B, H = cache.B, cache.H
    q = q_to_dev(inp["q_bf16"], torch)
    G = q.shape[1] // H
    ref_out = cache.decode_attn(q, SCALE).cpu().numpy()
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=q.device)
    cache.decode_attn_noalloc(q, SCALE, out=out)
    got = out.cpu().numpy()
    assert np.array_equal(got, ref_out)
    for b, h in pairs:
        st = oracle_stream(inp, b, h, bits, bits, kvq.F16)
        ref = oracle_attn(st, inp["q_bf16"][b, h * G:(h + 1) * G])
        assert rel_err_rows(got[b, h * G:(h + 1) * G], ref).max() <= REL_TOL


def test_noalloc_matches_workspace_entry_point_two_calls():
    # first call: a single long stream group cut into 64 chunks, then a
    # batched layer, then a smaller input
    print("case noalloc 1x1x7 T=32768 4-bit", flush=True)
    inp, cache = _case(1, 1, 7, 32768, 4, seed=301)
    _check(inp, cache, 4, [(0, 0)])
    print("case noalloc 4x4x28 T=4096 2-bit", flush=True)
    inp, cache = _case(4, 4, 28, 4096, 2, seed=302)
    _check(inp, cache, 2, [(0, 0), (3, 3)])
    print("case noalloc 1x2x8 T=640 4-bit", flush=True)
    inp, cache = _case(1, 2, 8, 640, 4, seed=303)
    _check(inp, cache, 4, [(0, 0), (0, 1)])
    # the long stream again, over the partials the earlier calls left
    print("case noalloc 1x1x7 T=32768 4-bit again", flush=True)
    inp, cache = _case(1, 1, 7, 32768, 4, seed=304)
    _check(inp, cache, 4, [(0, 0)])


def test_noalloc_rejects_plans_beyond_the_scratch():
    """512 streams of 16 query heads at 32K tokens need more partials than
    the scratch holds: KVQ_EWORKSPACE, nothing launched (fake device
    pointers are never touched)."""
    import ctypes
    s = kvq.KvqCacheStruct()
    s.batch, s.n_kv_heads, s.head_dim, s.group = 64, 8, 128, 128
    s.max_tokens, s.n_tokens, s.k_bits, s.v_bits, s.param_dtype = 32768, 32768, 4, 4, kvq.F16
    fake = 1 << 40
    for name in ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero"):
        setattr(s, name, fake)
    s.k_tile_stride = s.v_tile_stride = kvq.tile_bytes(4)
    L = kvq.load()
    st = L.kvq_decode_attn_noalloc(ctypes.byref(s), ctypes.c_void_p(fake), 8 * 16, 0.1,
                                   ctypes.c_void_p(fake), None)
    assert st == kvq.EWORKSPACE
