"""GPU parity of the pair-granular key widths (PN-Mix page, abstract): the
pair-norm reduction against the oracle's binary64 sums, and the whole chain
(prefill pair norms -> slot map -> mixed-width quantize -> decode) against the
oracle on the pairs recipe."""
import numpy as np
import pytest

import oracle
from kv_cache_mixed_amd import kvq, synth
from tests.gpu_helpers import (REL_TOL, SCALE, assert_stream_bytes_equal, oracle_attn, oracle_stream,
                               q_to_dev, rel_err_rows, to_dev)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

# binary32 sums of up to a few thousand norms per (row, pair), in any order,
# against binary64
NORM_RTOL = 2e-5


@pytest.fixture(scope="module", autouse=True)
def _setup():
    oracle.build(force=False)
    kvq.load()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("group", [1, 4])
def test_pair_norms(dtype, group):
    print("case pair norms %s group=%d" % (dtype, group), flush=True)
    rng = np.random.default_rng(40 + group)
    x = rng.standard_normal((2, 8, 700, 128)).astype(np.float32) * 3.0
    xd = to_dev(x, torch)
    if dtype == "bf16":
        xd = xd.to(torch.bfloat16)
        x = xd.float().cpu().numpy()                 # the values the kernel reads
    out = kvq.pair_norms(xd, group)
    ref = oracle.pair_norms(x, group)
    assert np.allclose(out.cpu().numpy(), ref, rtol=NORM_RTOL, atol=0)


def test_pair_norms_strided_and_accumulated():
    """A token window of a larger tensor (non-contiguous), in two calls that
    add into the same output, plus a ragged last workgroup."""
    print("case pair norms strided", flush=True)
    rng = np.random.default_rng(44)
    big = rng.standard_normal((1, 4, 1200, 128)).astype(np.float32)
    bd = to_dev(big, torch)
    out = torch.zeros((4, 64), dtype=torch.float32, device="cuda")
    kvq.pair_norms(bd[:, :, 100:613], 1, out=out)
    kvq.pair_norms(bd[:, :, 613:1100], 1, out=out)
    ref = oracle.pair_norms(big[:, :, 100:1100], 1)
    assert np.allclose(out.cpu().numpy(), ref, rtol=NORM_RTOL, atol=0)
    # no tokens: nothing added
    kvq.pair_norms(bd[:, :, :0], 1, out=out)
    assert np.allclose(out.cpu().numpy(), ref, rtol=NORM_RTOL, atol=0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_pair_norms_unaligned_rows(dtype):
    """Token rows 130 elements apart and a base 2 elements into the buffer
    (no alignment beyond the element)."""
    print("case pair norms unaligned %s" % dtype, flush=True)
    rng = np.random.default_rng(46)
    big = rng.standard_normal((1, 3, 300, 130)).astype(np.float32)
    bd = to_dev(big, torch)
    if dtype == "bf16":
        bd = bd.to(torch.bfloat16)
        big = bd.float().cpu().numpy()
    view = bd[:, :, :, 2:]                      # [1][3][300][128], row stride 130
    out = kvq.pair_norms(view, 1)
    ref = oracle.pair_norms(big[:, :, :, 2:], 1)
    assert np.allclose(out.cpu().numpy(), ref, rtol=NORM_RTOL, atol=0)


@pytest.mark.parametrize("v_bits", [2, 4])
def test_pn_mix_chain(v_bits):
    """Pairs recipe: scores from the GPU pair norms of the prefill queries and
    keys, the library's slot map (equal to the oracle's map of the oracle's
    scores: the recipe separates the salient pairs far beyond rounding), then
    mixed-width quantize (bit-exact) and decode (within the attention
    tolerance) with that map."""
    print("case pn-mix chain v=%d" % v_bits, flush=True)
    B, H, Hq, T = 2, 2, 8, 1024
    G = Hq // H
    d = synth.pair_layer(B, H, Hq, T, 21)
    kd, vd = to_dev(d["k"], torch), to_dev(d["v"], torch)
    score = (kvq.pair_norms(to_dev(d["q_prefill"], torch), G) * kvq.pair_norms(kd, 1)).cpu().numpy()
    ref_score = (oracle.pair_norms(d["q_prefill"], G) * oracle.pair_norms(d["k"], 1)).astype(np.float32)
    assert np.allclose(score, ref_score, rtol=5e-5, atol=0)
    slot_chan = kvq.pair_slot_map(score)
    assert np.array_equal(slot_chan, oracle.pair_slot_map(ref_score))
    cache = kvq.PackedCache(B, H, T, kvq.KMIXED, v_bits, kvq.E4M3, slot_chan=slot_chan)
    cache.quantize(kd, vd, 0)
    torch.cuda.synchronize()
    out = cache.decode_attn(q_to_dev(d["q_bf16"], torch), SCALE).cpu().numpy()
    worst = 0.0
    for b in range(B):
        for h in range(H):
            st = oracle_stream(d, b, h, 0, v_bits, kvq.E4M3, slot_chan[h])
            assert_stream_bytes_equal(cache, st, b, h, "pn-mix b=%d h=%d" % (b, h))
            ref = oracle_attn(st, d["q_bf16"][b, h * G:(h + 1) * G])
            worst = max(worst, rel_err_rows(out[b, h * G:(h + 1) * G], ref).max())
    assert worst <= REL_TOL, "max row relative error %.3e" % worst
