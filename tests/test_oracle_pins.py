"""Pins of the CPU oracle to facts fixed outside it (CPU only).

Each test checks the oracle against something independent of the oracle's own
code: exhaustive enumeration against exact rational arithmetic, closed forms,
library conversions (numpy/torch), brute force, invariants, and the numbers
the pages print (tests/golden/pages_constants.json).  Chosen so that a dropped
term, a wrong sign or index, or a transposed operand in the oracle fails one.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")


@pytest.fixture(scope="module", autouse=True)
def _build():
    oracle.build(force=False)


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------
def _fp16_probe_values():
    rng = np.random.default_rng(1)
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    finite = allh[np.isfinite(allh)].astype(np.float32)
    vals = [finite]
    # midpoints of consecutive positive binary16 values, and one binary32 ulp either side
    pos = np.sort(np.unique(np.abs(finite.astype(np.float64))))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    vals += [mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0)),
             -mids]
    vals.append(rng.standard_normal(300000).astype(np.float32) *
                np.exp2(rng.integers(-30, 18, 300000)).astype(np.float32))
    vals.append(np.array([65504, 65519.99, 65520, 65536, 1e30, 2.0 ** -24, 2.0 ** -25,
                          1.5 * 2.0 ** -25, 2.0 ** -26, 0.0, -0.0], dtype=np.float32))
    return np.concatenate(vals).astype(np.float32)


def test_f16_narrowing_matches_numpy():
    x = _fp16_probe_values()
    ours = oracle.narrow(x, oracle.F16)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref), np.flatnonzero(ours != ref)[:10]


def test_f16_decode_matches_numpy():
    raw = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode(raw, oracle.F16)
    ref = raw.view(np.float16).astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))


def test_bf16_narrowing_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(2)
    x = np.concatenate([
        rng.standard_normal(400000).astype(np.float32) *
        np.exp2(rng.integers(-140, 120, 400000)).astype(np.float32),
        # exact midpoints between bfloat16 neighbours and one ulp off
        (np.arange(1 << 16, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        (np.arange(1 << 16, dtype=np.uint32) << 16 | 0x7FFF).view(np.float32),
        (np.arange(1 << 16, dtype=np.uint32) << 16 | 0x8001).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    ours = oracle.narrow(x, oracle.BF16)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ok = ours == ref
    # torch maps overflow to inf, as IEEE rounding does; both must agree everywhere
    assert ok.all(), (x[~ok][:5], ours[~ok][:5], ref[~ok][:5])


def _e4m3_closed_form(c):
    s, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
    if e == 15 and m == 7:
        return math.nan
    v = (2.0 ** -6) * m / 8 if e == 0 else 2.0 ** (e - 7) * (1 + m / 8)
    return -v if s else v


def test_e4m3_decode_all_codes_closed_form():
    raw = np.arange(256, dtype=np.uint8)
    ours = oracle.decode(raw, oracle.E4M3)
    for c in range(256):
        ref = _e4m3_closed_form(c)
        if math.isnan(ref):
            assert math.isnan(ours[c])
        else:
            assert ours[c] == ref, c
    assert np.nanmax(ours) == 448.0


def test_e4m3_encode_roundtrip_ties_saturation():
    raw = np.arange(256, dtype=np.uint8)
    vals = oracle.decode(raw, oracle.E4M3)
    fin = np.isfinite(vals)
    back = oracle.narrow(vals[fin].astype(np.float32), oracle.E4M3)
    assert np.array_equal(back, raw[fin])
    # every midpoint of consecutive positive values rounds to the even code
    pos = np.unique(vals[fin & (vals >= 0)])
    for a, b in zip(pos[:-1], pos[1:]):
        mid = np.float32((a + b) / 2)
        code = oracle.narrow(np.array([mid]), oracle.E4M3)[0]
        ca = oracle.narrow(np.array([a], dtype=np.float32), oracle.E4M3)[0]
        cb = oracle.narrow(np.array([b], dtype=np.float32), oracle.E4M3)[0]
        assert code == (ca if ca % 2 == 0 else cb)
    big = oracle.narrow(np.array([449.0, 464.0, 1e6, -1e9], dtype=np.float32), oracle.E4M3)
    assert list(oracle.decode(big, oracle.E4M3)) == [448.0, 448.0, 448.0, -448.0]


def test_e4m3_matches_torch_in_range():
    torch = pytest.importorskip("torch")
    if not hasattr(torch, "float8_e4m3fn"):
        pytest.skip("torch without float8_e4m3fn")
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-12, 8, 200000))).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ours = oracle.narrow(x, oracle.E4M3)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------------------
# Equivalent Right Shift (PM-KVQ Key design 1)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_ers_equals_requantization_exhaustive(b):
    """ERS(X) must equal round((x^ - Z) / S_b) with x^ = S X + Z and
    S_b = (2^b + 1) S, Z_b = Z, in exact rationals, for every X in [0, 2^2b)."""
    X = np.arange(1 << (2 * b), dtype=np.uint32)
    got = oracle.ers(X, b)
    S, Z = Fraction(3, 7), Fraction(-5, 3)   # arbitrary positive scale, any offset
    Sb = (2 ** b + 1) * S
    for x in range(1 << (2 * b)):
        xhat = S * x + Z
        r = (xhat - Z) / Sb
        fl = math.floor(r)
        frac = r - fl
        assert frac != Fraction(1, 2)               # 2^b + 1 is odd: never an exact tie
        want = fl + (1 if frac > Fraction(1, 2) else 0)
        want = min(max(want, 0), 2 ** b - 1)
        assert got[x] == want, (b, x, got[x], want)


@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_ers_invariants(b):
    X = np.arange(1 << (2 * b), dtype=np.uint32)
    Y = oracle.ers(X, b).astype(np.int64)
    assert Y[0] == 0 and Y[-1] == 2 ** b - 1
    assert np.all(np.diff(Y) >= 0)                                   # monotone
    err = np.abs((2 ** b + 1) * Y - X.astype(np.int64))
    assert err.max() <= 2 ** (b - 1)                                 # |x^_b - x^_2b| <= 2^(b-1) S
    counts = np.bincount(Y, minlength=2 ** b)
    assert counts[0] == 2 ** (b - 1) + 1 and counts[-1] == 2 ** (b - 1) + 1
    assert np.all(counts[1:-1] == 2 ** b + 1)
    # the unsigned 32-bit product of the library never overflows
    cmax = (2 ** (2 * b) - 2 ** b + 1) * (2 ** (2 * b) - 1 + 2 ** (b - 1))
    assert cmax < 2 ** 32


def test_ers_near_ties():
    """Near-ties (X mod (2^b+1) in {2^(b-1), 2^(b-1)+1}) round down then up.
    Hand-derived lists for b = 1, 2 and the counts 2 / 6 / 30 / 510."""
    expect_lists = {1: [1, 2], 2: [2, 3, 7, 8, 12, 13]}
    for b, n_expect in [(1, 2), (2, 6), (4, 30), (8, 510)]:
        X = np.arange(1 << (2 * b), dtype=np.int64)
        r = X % (2 ** b + 1)
        near = X[(r == 2 ** (b - 1)) | (r == 2 ** (b - 1) + 1)]
        assert len(near) == n_expect
        if b in expect_lists:
            assert near.tolist() == expect_lists[b]
        Y = oracle.ers(near.astype(np.uint32), b).astype(np.int64)
        q = near // (2 ** b + 1)
        down = (near % (2 ** b + 1)) == 2 ** (b - 1)
        assert np.all(Y[down] == q[down]) and np.all(Y[~down] == q[~down] + 1)


def test_ers_identity_sum_of_cubes():
    for b in range(1, 9):
        assert (2 ** b + 1) * (2 ** (2 * b) - 2 ** b + 1) == 2 ** (3 * b) + 1


def test_ers_scale_update_exact():
    """S_b = narrow((2^b+1) S): the binary32 product is exact for binary16/e4m3 S."""
    rng = np.random.default_rng(4)
    s = oracle.narrow(np.abs(rng.standard_normal(1000)).astype(np.float32), oracle.F16)
    for b in (8, 4, 2, 1):
        st = oracle.Stream(2 * b, 2 * b, oracle.F16, None, s.reshape(-1, 8), s.reshape(-1, 8),
                           None, s, s)
        # shrink_scales via the C routine on a copy
        arr = s.copy()
        oracle.lib().orc_shrink_scales(oracle._p(arr), arr.size, b, oracle.F16)
        exact = oracle.decode(s, oracle.F16) * (2 ** b + 1)
        want = exact.astype(np.float32).astype(np.float16).view(np.uint16)
        assert np.array_equal(arr, want)
        del st


# ---------------------------------------------------------------------------
# Halving rules of the ablation (PM-KVQ Key design 1 and the ablation table):
# direct right shift (keep the high b bits) and the modified right shift, read
# as the rounded, clamped shift
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_direct_shift_keeps_high_bits_exhaustive(b):
    """Direct right shift = the high b bits of the 2b-bit code, taken from its
    binary string; every X in [0, 2^2b)."""
    X = np.arange(1 << (2 * b), dtype=np.uint32)
    got = oracle.shift(X, b, oracle.SHIFT_DIRECT)
    want = [int(format(int(x), "0%db" % (2 * b))[:b], 2) for x in X]
    assert got.tolist() == want


@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_modified_shift_rounds_and_clamps_exhaustive(b):
    """Modified right shift: the nearest integer to X / 2^b (halves up, in exact
    rationals), clamped to 2^b - 1; every X in [0, 2^2b)."""
    X = np.arange(1 << (2 * b), dtype=np.uint32)
    got = oracle.shift(X, b, oracle.SHIFT_MODIFIED)
    for x in range(1 << (2 * b)):
        r = Fraction(x, 2 ** b)
        want = min(math.floor(r + Fraction(1, 2)), 2 ** b - 1)
        assert got[x] == want, (b, x)
    # the clamp is hit exactly by the top 2^(b-1) codes
    clamped = (X.astype(np.int64) + 2 ** (b - 1)) >= 2 ** (2 * b)
    assert clamped.sum() == 2 ** (b - 1) and np.all(got[clamped] == 2 ** b - 1)


@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_halving_rule_reconstruction_errors(b):
    """Reconstruction x^_b - x^_2b in units of S_2b, over every 2b-bit code:
    ERS  |e| <= 2^(b-1), mean exactly 0 (the rule is symmetric);
    direct  -(2^b - 1) <= e <= 0, mean exactly -(2^b - 1)/2 (truncation);
    modified  |e| <= 2^(b-1) below the clamp, e = 2^b(2^b - 1) - X above it,
    down to -(2^b - 1) at the top code."""
    X = np.arange(1 << (2 * b), dtype=np.int64)
    n = X.size
    e_ers = (2 ** b + 1) * oracle.shift(X.astype(np.uint32), b, oracle.SHIFT_ERS).astype(np.int64) - X
    e_dir = 2 ** b * oracle.shift(X.astype(np.uint32), b, oracle.SHIFT_DIRECT).astype(np.int64) - X
    e_mod = 2 ** b * oracle.shift(X.astype(np.uint32), b, oracle.SHIFT_MODIFIED).astype(np.int64) - X
    assert np.abs(e_ers).max() <= 2 ** (b - 1) and Fraction(int(e_ers.sum()), n) == 0
    assert e_dir.max() == 0 and e_dir.min() == -(2 ** b - 1)
    assert Fraction(int(e_dir.sum()), n) == Fraction(-(2 ** b - 1), 2)
    top = X + 2 ** (b - 1) >= 2 ** (2 * b)
    assert np.abs(e_mod[~top]).max() <= 2 ** (b - 1)
    assert np.array_equal(e_mod[top], 2 ** b * (2 ** b - 1) - X[top]) and e_mod[-1] == -(2 ** b - 1)


def test_halving_rules_on_a_stream():
    """shrink_stream with each rule on a quantized stream: zero points kept,
    scales narrow((2^b + 1) S) for ERS and 2^b S (exact) for the shifts, and
    the codes are the rule applied to the 4-bit codes."""
    from kv_cache_mixed_amd import synth
    inp = synth.layer(1, 1, 1, 256, seed=61)
    st4 = oracle.quantize_stream(inp["k"][0, 0], inp["v"][0, 0], 4, 4, oracle.F16)
    c4k = np.concatenate([oracle.unpack_rows(t, 4) for t in st4.k_tiles]).ravel()
    for m in (oracle.SHIFT_ERS, oracle.SHIFT_DIRECT, oracle.SHIFT_MODIFIED):
        st2 = oracle.shrink_stream(st4, 2, m)
        assert np.array_equal(st2.kz, st4.kz) and np.array_equal(st2.vz, st4.vz)
        f = 5.0 if m == oracle.SHIFT_ERS else 4.0
        want = (oracle.decode(st4.ks, oracle.F16) * f).astype(np.float32).astype(np.float16).view(np.uint16)
        assert np.array_equal(st2.ks, want)
        c2k = np.concatenate([oracle.unpack_rows(t, 2) for t in st2.k_tiles]).ravel()
        assert np.array_equal(c2k, oracle.shift(c4k.astype(np.uint32), 2, m))


# ---------------------------------------------------------------------------
# quantizer (ChanMix Key design 1; PM-KVQ Training strategy)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("bits", [1, 2, 4, 8, 16])
def test_quantizer_math_mode_bound(bits):
    """With binary32 parameters (no narrowing): q(min) = 0, q(max) = 2^b - 1
    and |x - x^| <= S/2 up to binary32 rounding."""
    rng = np.random.default_rng(10 + bits)
    for trial in range(50):
        x = (rng.standard_normal(128) * rng.uniform(0.01, 20)).astype(np.float32)
        codes, s, z = oracle.quantize_group(x, bits, oracle.F32)
        S = float(s)
        assert float(z) == float(x.min())
        assert codes[np.argmin(x)] == 0 and codes[np.argmax(x)] == 2 ** bits - 1
        xhat = S * codes.astype(np.float64) + float(z)
        slack = 4 * np.finfo(np.float32).eps * (np.abs(x).max() + S * 2 ** bits)
        assert np.abs(x - xhat).max() <= S / 2 + slack


@pytest.mark.parametrize("pdt", [oracle.F16, oracle.E4M3, oracle.BF16])
@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8, 16])
def test_quantizer_picks_nearest_level(bits, pdt):
    """Brute force: every code is the level S'q + Z' nearest to x (exact
    arithmetic), except where two levels are within binary32 rounding of a tie;
    values outside the level range clamp to the end code."""
    rng = np.random.default_rng(100 + bits + 7 * pdt)
    scale = 1.0 if pdt != oracle.E4M3 else 0.5
    for trial in range(20):
        x = (rng.standard_normal(128) * scale * rng.uniform(0.1, 3)).astype(np.float32)
        codes, s, z = oracle.quantize_group(x, bits, pdt)
        S = Fraction(float(oracle.decode(np.array([s]), pdt)[0]))
        Z = Fraction(float(oracle.decode(np.array([z]), pdt)[0]))
        if S == 0:
            assert np.all(codes == 0)
            continue
        for xi, qi in zip(x.tolist(), codes.tolist()):
            xf = Fraction(xi)
            exact = (xf - Z) / S
            best = min(max(round(exact), 0), 2 ** bits - 1)     # nearest level (clamped)
            if qi != best:
                # only allowed at a near-tie: two binary32 roundings ((x - Z'), then
                # the division) move the quotient by at most ~2^-23 of its size
                tol = max(abs(exact), Fraction(1)) / 2 ** 21
                assert abs(abs(exact - math.floor(exact)) - Fraction(1, 2)) < tol, \
                    (bits, pdt, xi, qi, best, float(exact))
                assert abs(qi - best) == 1


def test_quantizer_constant_group_and_storage_bound():
    codes, s, z = oracle.quantize_group(np.full(128, 1.2345, np.float32), 4, oracle.F16)
    assert np.all(codes == 0) and oracle.decode(np.array([s]), oracle.F16)[0] == 0.0
    rng = np.random.default_rng(7)
    for bits in (2, 4, 8):
        x = rng.standard_normal(128).astype(np.float32) * 3
        codes, s, z = oracle.quantize_group(x, bits, oracle.F16)
        S = oracle.decode(np.array([s]), oracle.F16)[0]
        Z = oracle.decode(np.array([z]), oracle.F16)[0]
        xhat = S * codes + Z
        mn, mx = float(x.min()), float(x.max())
        bound = max(S / 2, Z - mn, mx - Z - (2 ** bits - 1) * S) + 1e-6
        assert np.abs(x - xhat).max() <= bound


# ---------------------------------------------------------------------------
# packed layouts (header layout text)
# ---------------------------------------------------------------------------
def test_pack_bit_positions_by_hand():
    c = np.zeros((128, 128), np.uint16)
    c[0, 0], c[0, 1], c[0, 5] = 0xA, 0x5, 0x3          # 4-bit row 0
    c[2, 127] = 0xF
    t = oracle.pack_rows(c, 4)
    assert t[0] == 0x5A and t[2] == 0x30 and t[2 * 64 + 63] == 0xF0
    c2 = np.zeros((128, 128), np.uint16)
    c2[1, 2], c2[1, 3] = 0x2, 0x1                       # 2-bit: row 1 starts at byte 32
    assert oracle.pack_rows(c2, 2)[32] == (0x2 << 4) | (0x1 << 6)
    c16 = np.zeros((128, 128), np.uint16)
    c16[0, 1] = 0xBEEF
    t16 = oracle.pack_rows(c16, 16)
    assert t16[2] == 0xEF and t16[3] == 0xBE
    c1 = np.zeros((128, 128), np.uint16)
    c1[0, 9] = 1
    assert oracle.pack_rows(c1, 1)[1] == 0x02


def test_value_tile_positions_by_hand():
    """Value word planes W[w][c][a] (header layout text), positions worked out
    by hand: 4-bit -> 8 tokens per word; with c = 64h + 16q + n the word index
    is w*512 + ((h*16 + n)*4 + a)*4 + q."""
    c = np.zeros((128, 128), np.uint16)          # [channel][token]
    c[0, 0] = 0x3                                # w=0,c=0,a=0,i=0 -> byte 0 low nibble
    c[0, 9] = 0x5                                # t=9: a=0, w=1, i=1 -> word 512, bits 4..7
    c[2, 33] = 0xF                               # t=33: a=1, w=0, i=1; n=2 -> word (2*4+1)*4 = 36
    c[20, 0] = 0x7                               # c=20: h=0, q=1, n=4 -> word (4*4)*4 + 1 = 65
    c[64, 0] = 0x9                               # c=64: h=1, q=0, n=0 -> word (16*4)*4 = 256
    c[127, 127] = 0x6                            # h=1,q=3,n=15, a=3, w=3, i=7 -> word 2047, bits 28..31
    t = oracle.pack_vtile(c, 4)
    assert t[0] == 0x03
    assert t[4 * 512] == 0x50
    assert t[4 * 36] == 0xF0
    assert t[4 * 65] == 0x07
    assert t[4 * 256] == 0x09
    assert t[4 * 2047 + 3] == 0x60
    assert int(np.count_nonzero(t)) == 6
    c1 = np.zeros((128, 128), np.uint16)
    c1[5, 40] = 1                                # 1-bit: w=0, a=1, i=8; n=5 -> word (5*4+1)*4 = 84, bit 8
    assert oracle.pack_vtile(c1, 1)[4 * 84 + 1] == 0x01
    c16 = np.zeros((128, 128), np.uint16)
    c16[1, 3] = 0xBEEF                           # 16-bit: 2 tokens per word; t=3: w=1, i=1; n=1
    t16 = oracle.pack_vtile(c16, 16)
    wi = 512 + (1 * 4 + 0) * 4
    assert t16[4 * wi + 2] == 0xEF and t16[4 * wi + 3] == 0xBE
    for bits in (1, 2, 4, 8, 16):
        r = np.random.default_rng(bits).integers(0, 2 ** bits, (128, 128)).astype(np.uint16)
        assert np.array_equal(oracle.unpack_vtile(oracle.pack_vtile(r, bits), bits), r)


def test_mixed_pack_by_hand():
    """Byte positions worked out by hand from the header's mixed layout text:
    plane g holds logical bytes g, 4+g, 8+6g .. 13+6g at plane bytes 0..7."""
    c = np.zeros((128, 128), np.uint16)
    c[0, 0] = 0x9                 # 4-bit slot 0 -> logical byte 0 low nibble -> plane 0 byte 0
    c[0, 7] = 0xA                 # 4-bit slot 7 -> logical byte 3 high nibble -> plane 3 byte 0
    c[0, 8], c[0, 9] = 5, 1       # 3-bit slot 8, 1-bit slot 9 -> logical byte 4 = 0b1101
    c[0, 10], c[0, 11] = 7, 0     # -> high nibble of logical byte 4 = 0b0111; plane 0 byte 1
    c[3, 24] = 3                  # first 2-bit slot -> logical byte 8 of token 3 -> plane 0 byte 2
    c[1, 77] = 2                  # slot 77 -> logical byte 21 bits 2-3 -> plane 2 byte 3
    c[2, 119] = 1                 # slot 119 -> logical byte 31 bits 6-7 -> plane 3 byte 7
    c[5, 127] = 2                 # last 2-bit slot -> logical byte 33 of token 5 (plane 4)
    t = oracle.pack_mixed(c)
    assert t[0] == 0x09
    assert t[3072 + 0] == 0xA0
    assert t[1] == 0x7D
    assert t[8 * 3 + 2] == 0x03
    assert t[2048 + 8 * 1 + 3] == 0x08
    assert t[3072 + 8 * 2 + 7] == 0x40
    assert t[4096 + 2 * 5 + 1] == 0x80
    assert int(np.count_nonzero(t)) == 7
    assert list(oracle.mixed_slot_bits()[:12]) == [4] * 8 + [3, 1, 3, 1]
    assert oracle.mixed_slot_bits().sum() == 272        # 34 bytes, 8 bits per byte


@pytest.mark.parametrize("bits", [1, 2, 4, 8, 16])
def test_pack_roundtrip(bits):
    rng = np.random.default_rng(bits)
    c = rng.integers(0, 2 ** bits, (128, 128)).astype(np.uint16)
    assert np.array_equal(oracle.unpack_rows(oracle.pack_rows(c, bits), bits), c)
    w = oracle.mixed_slot_bits()
    cm = (rng.integers(0, 1 << 16, (128, 128)) % (1 << w)[None, :]).astype(np.uint16)
    assert np.array_equal(oracle.unpack_mixed(oracle.pack_mixed(cm)), cm)


def test_stream_k_channelwise_v_tokenwise():
    """Keys: one group per channel over 128 tokens; values: one per token."""
    rng = np.random.default_rng(5)
    k = rng.standard_normal((256, 128)).astype(np.float32)
    v = rng.standard_normal((256, 128)).astype(np.float32)
    st = oracle.quantize_stream(k, v, 4, 4, oracle.F16)
    ks = oracle.decode(st.ks, oracle.F16)
    kz = oracle.decode(st.kz, oracle.F16)
    assert np.allclose(kz[1, 7], k[128:256, 7].min(), rtol=1e-3)
    assert np.allclose(ks[1, 7], (k[128:256, 7].max() - k[128:256, 7].min()) / 15, rtol=1e-3)
    vz = oracle.decode(st.vz, oracle.F16)
    assert np.allclose(vz[130], v[130].min(), rtol=1e-3)
    K = oracle.dequant_k(st)
    V = oracle.dequant_v(st)
    assert np.abs(K - k).max() <= ks.max() / 2 + 2e-3 * np.abs(k).max()
    assert np.abs(V - v).max() <= oracle.decode(st.vs, oracle.F16).max() / 2 + 2e-3 * np.abs(v).max()


# ---------------------------------------------------------------------------
# decode attention (fp64, two-pass)
# ---------------------------------------------------------------------------
def _stream(T, seed, kb=4, vb=4, pdt=oracle.F16, mixed=False):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((T, 128)).astype(np.float32)
    v = rng.standard_normal((T, 128)).astype(np.float32)
    sc = None
    if mixed:
        sc = rng.permutation(128).astype(np.int16)
        kb = 0
    return oracle.quantize_stream(k, v, kb, vb, pdt, sc), rng


def _bf16(x):
    return oracle.narrow(np.asarray(x, np.float32), oracle.BF16)


@pytest.mark.parametrize("mixed", [False, True])
def test_attention_matches_numpy_softmax(mixed):
    st, rng = _stream(384, 11, mixed=mixed, pdt=oracle.E4M3 if mixed else oracle.F16)
    q = _bf16(rng.standard_normal((3, 128)))
    scale = 1 / math.sqrt(128)
    out = oracle.decode_attn(st, q, scale)
    K = oracle.dequant_k(st)
    V = oracle.dequant_v(st)
    qd = oracle.decode(q, oracle.BF16)
    s = (qd @ K.T) * float(np.float32(scale))
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    assert np.allclose(out, p @ V, rtol=1e-12, atol=1e-12)


def test_attention_special_cases():
    st, rng = _stream(256, 12)
    V = oracle.dequant_v(st)
    K = oracle.dequant_k(st)
    # q = 0: uniform weights -> mean of the value rows
    out0 = oracle.decode_attn(st, _bf16(np.zeros((1, 128))), 0.088)
    assert np.allclose(out0[0], V.mean(axis=0), atol=1e-12)
    # one dominant logit: q aligned with one key, huge scale -> that key's value row
    t_star = int(np.argmax(np.linalg.norm(K, axis=1)))
    q = _bf16(K[t_star][None, :])
    outd = oracle.decode_attn(st, q, 1e4)
    assert np.allclose(outd[0], V[t_star], atol=1e-9)
    # equal query heads -> equal outputs
    qq = _bf16(np.repeat(rng.standard_normal((1, 128)), 4, axis=0))
    oq = oracle.decode_attn(st, qq, 0.088)
    assert np.all(oq == oq[0])
    # swapping whole tiles (keeps every quantization group) leaves the output unchanged
    sw = oracle.Stream(st.k_bits, st.v_bits, st.pdt, st.k_tiles[::-1].copy(), st.ks[::-1].copy(),
                       st.kz[::-1].copy(), st.v_tiles[::-1].copy(),
                       np.concatenate([st.vs[128:], st.vs[:128]]),
                       np.concatenate([st.vz[128:], st.vz[:128]]))
    qr = _bf16(rng.standard_normal((2, 128)))
    assert np.allclose(oracle.decode_attn(sw, qr, 0.1), oracle.decode_attn(st, qr, 0.1),
                       rtol=1e-12, atol=1e-13)


def test_attention_single_tile_of_one_repeated_token():
    """Every token equal -> the output is that token's reconstruction."""
    rng = np.random.default_rng(13)
    row = rng.standard_normal(128).astype(np.float32)
    k = np.repeat(row[None], 128, axis=0)
    v = np.repeat(rng.standard_normal(128).astype(np.float32)[None], 128, axis=0)
    st = oracle.quantize_stream(k, v, 4, 4, oracle.F16)
    out = oracle.decode_attn(st, _bf16(rng.standard_normal((1, 128))), 0.1)
    assert np.allclose(out[0], oracle.dequant_v(st)[0], atol=1e-12)


def test_split_softmax_combine_equals_two_pass():
    """Flash-decoding identity used by the kernel's split + combine."""
    st, rng = _stream(512, 14)
    q = _bf16(rng.standard_normal((2, 128)))
    ref = oracle.decode_attn(st, q, 0.088)
    K, V = oracle.dequant_k(st), oracle.dequant_v(st)
    s = (oracle.decode(q, oracle.BF16) @ K.T) * float(np.float32(0.088))
    parts = []
    for c0 in range(0, 512, 96):
        sc = s[:, c0:c0 + 96]
        m = sc.max(axis=1)
        e = np.exp(sc - m[:, None])
        parts.append((m, e.sum(axis=1), e @ V[c0:c0 + 96]))
    M = np.max([p[0] for p in parts], axis=0)
    num = sum(np.exp(p[0] - M)[:, None] * p[2] for p in parts)
    den = sum(np.exp(p[0] - M) * p[1] for p in parts)
    assert np.allclose(num / den[:, None], ref, rtol=1e-12, atol=1e-13)


def _first_tiles(st, n):
    """the stream's first n tiles (n*128 tokens) as a stream of their own"""
    return oracle.Stream(st.k_bits, st.v_bits, st.pdt, st.k_tiles[:n].copy(), st.ks[:n].copy(),
                         st.kz[:n].copy(), st.v_tiles[:n].copy(), st.vs[:n * 128].copy(),
                         st.vz[:n * 128].copy(), st.slot_chan)


@pytest.mark.parametrize("mixed", [False, True])
def test_residual_segment_of_reconstructed_tokens_equals_packed(mixed):
    """A residual segment holding exactly the reconstructions of the last tile
    gives the C oracle's attention over the whole packed stream (numpy float64
    path against the C path)."""
    st, rng = _stream(384, 21, mixed=mixed, pdt=oracle.E4M3 if mixed else oracle.F16)
    q = _bf16(rng.standard_normal((4, 128)))
    full = oracle.decode_attn(st, q, 0.09)
    head = _first_tiles(st, 2)
    res = oracle.decode_attn_residual(head, q, 0.09, oracle.dequant_k(st)[256:],
                                      oracle.dequant_v(st)[256:])
    assert np.allclose(res, full, rtol=1e-12, atol=1e-13)
    # and the other way round: no packed tokens, every token residual
    allres = oracle.decode_attn_residual(None, q, 0.09, oracle.dequant_k(st), oracle.dequant_v(st))
    assert np.allclose(allres, full, rtol=1e-12, atol=1e-13)


def test_residual_segment_special_cases():
    rng = np.random.default_rng(22)
    k = rng.standard_normal((37, 128))
    v = rng.standard_normal((37, 128))
    # q = 0: uniform weights -> the mean of the value rows
    out0 = oracle.decode_attn_residual(None, _bf16(np.zeros((1, 128))), 0.1, k, v)
    assert np.allclose(out0[0], v.mean(axis=0), atol=1e-13)
    # a single residual token gets all the weight
    one = oracle.decode_attn_residual(None, _bf16(rng.standard_normal((3, 128))), 0.1, k[:1], v[:1])
    assert np.array_equal(one, np.repeat(v[:1], 3, axis=0))
    # one dominant residual key overrides a whole packed stream
    st, _ = _stream(256, 23)
    kd = np.zeros((2, 128))
    kd[1, 5] = 1000.0   # logit 1e7, far above any packed key (|k| < 10)
    q = np.zeros((1, 128), np.float32)
    q[0, 5] = 1.0
    outd = oracle.decode_attn_residual(st, _bf16(q), 1e4, kd, v[:2])
    assert np.allclose(outd[0], v[1], atol=1e-9)


def test_residual_merge_identity():
    """packed part and residual part combined through their (max, sum,
    weighted sum) partials equal one softmax over both: the merge the decode
    kernels use for the residual slot."""
    st, rng = _stream(512, 24)
    q = _bf16(rng.standard_normal((3, 128)))
    rk = rng.standard_normal((77, 128))
    rv = rng.standard_normal((77, 128))
    ref = oracle.decode_attn_residual(st, q, 0.088, rk, rv)
    qd = oracle.decode(q, oracle.BF16)
    sig = float(np.float32(0.088))
    parts = []
    for K, V in ((oracle.dequant_k(st), oracle.dequant_v(st)), (rk, rv)):
        s = sig * (qd @ K.T)
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        parts.append((m, e.sum(axis=1), e @ V))
    M = np.maximum(parts[0][0], parts[1][0])
    num = sum(np.exp(p[0] - M)[:, None] * p[2] for p in parts)
    den = sum(np.exp(p[0] - M) * p[1] for p in parts)
    assert np.allclose(num / den[:, None], ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# shrink on a stream, schedule, sizes
# ---------------------------------------------------------------------------
def test_shrink_stream_matches_requantized_codes():
    st, _ = _stream(256, 15, kb=4, vb=4)
    st2 = oracle.shrink_stream(st, 2)
    for g in range(2):
        c4 = oracle.unpack_rows(st.k_tiles[g], 4).astype(np.int64)
        c2 = oracle.unpack_rows(st2.k_tiles[g], 2).astype(np.int64)
        assert np.array_equal(c2, np.floor(c4 / 5 + 0.5).astype(np.int64))
        v4 = oracle.unpack_vtile(st.v_tiles[g], 4).astype(np.int64)
        v2 = oracle.unpack_vtile(st2.v_tiles[g], 2).astype(np.int64)
        assert np.array_equal(v2, np.floor(v4 / 5 + 0.5).astype(np.int64))
    assert st2.k_tiles.shape[1] == st.k_tiles.shape[1] // 2
    # error after one shrink is within S'_4/2 + 2 S'_4
    K2 = oracle.dequant_k(st2)
    K4 = oracle.dequant_k(st)
    s4 = oracle.decode(st.ks, oracle.F16).max()
    assert np.abs(K2 - K4).max() <= 2 * s4 + 1e-2 * s4 * 5


def test_schedule_trigger_points():
    """Progressive schedule at B=8, Hkv=4, 128 MiB per layer (25% of the
    16-bit size of 32768 tokens): halvings fire when the next 128-token group
    would not fit -- derived by hand from the byte counts 66560 / 33792 / 17408
    / 9216 per group per stream at 16 / 8 / 4 / 2 bits."""
    B, H, T = 8, 4, 32768
    fp16_bytes = B * H * T * 128 * 2 * 2
    budget = fp16_bytes // 4
    assert budget == 128 * 2 ** 20
    per = {b: oracle.block_bytes(1, 1, 128, b, b, oracle.F16) for b in (16, 8, 4, 2)}
    assert per == {16: 66560, 8: 33792, 4: 17408, 2: 9216}
    ev = oracle.schedule(B, H, T, 16, 2, oracle.F16, budget)
    assert ev == [(8064, 8), (15872, 4), (30720, 2)]
    per_stream = budget // (B * H)
    for t, b in ev:
        prev = 2 * b
        assert (t // 128) * per[prev] <= per_stream < (t // 128 + 1) * per[prev]
    assert oracle.schedule(B, H, T, 16, 4, oracle.F16, budget) is None   # floor 4 cannot fit


def test_sizes_against_pages():
    with open(GOLDEN) as f:
        g = json.load(f)
    # 64 layers, 8 kv heads, head_dim 128, K and V, 2 bytes, 32768 tokens, batch 16
    fp16 = 64 * 8 * 128 * 2 * 2 * 32768 * 16
    assert fp16 == g["kv_cache_gb_32b_32k_batch16"]["value"] * 2 ** 30
    # packed attention read set of the 7B layer at 4 bits with binary16 S/Z
    assert oracle.block_bytes(16, 4, 32768, 4, 4, oracle.F16) == 285212672
    # 128K mixed layer: 34-byte keys, 2-bit values, e4m3 S/Z
    per_tile = oracle.tile_bytes(0) + oracle.tile_bytes(2) + 512 * 1
    assert 8 * 1024 * per_tile == 73400320


def test_rope_period_against_pages():
    from kv_cache_mixed_amd import synth
    with open(GOLDEN) as f:
        g = json.load(f)
    inv = synth.rope_inv_freq()
    period = 2 * math.pi / inv[-1]
    assert round(period) == g["rope_lowest_freq_period_tokens"]["value"]
    # rotation preserves each pair's norm
    rng = np.random.default_rng(0)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    y = synth.apply_rope(x, 1000)
    nx = np.hypot(x[:, :64].astype(np.float64), x[:, 64:])
    ny = np.hypot(y[:, :64].astype(np.float64), y[:, 64:])
    assert np.allclose(nx, ny, rtol=1e-6)


# ---------------------------------------------------------------------------
# mixed-width keys: the oracle's quantizer against an independent build
# ---------------------------------------------------------------------------
# Class widths of the mixed key tile, written here from the channel classes of
# "Channel-Aware Mixed-Precision Quantization ..." (Key design 3: 4-bit
# retrieval channels, 3-bit outlier channels paired with as many 1-bit
# sub-normal channels, 2-bit for the rest, packed so that every byte holds 8
# code bits) and the slot order of the header's mixed layout text: 8 slots of
# 4 bits, then 8 (3-bit, 1-bit) pairs, then 104 slots of 2 bits.
_MIXED_WIDTHS = [4] * 8 + [3, 1] * 8 + [2] * 104


def _narrow_ref(x, pdt):
    """binary32 -> exact value of its narrowing, by library routines (numpy
    binary16, torch float8_e4m3fn), not by the oracle"""
    import torch
    x = np.float32(x)
    if pdt == oracle.F16:
        return float(np.float16(x))
    assert pdt == oracle.E4M3 and abs(float(x)) <= 448.0
    return float(torch.tensor([float(x)], dtype=torch.float32).to(torch.float8_e4m3fn).float()[0])


def _mixed_row_bytes(codes_row):
    """34-byte logical row of one token: little-endian bit string of the slot
    codes in slot order at the class widths (header layout text)"""
    bits = 0
    pos = 0
    for j, w in enumerate(_MIXED_WIDTHS):
        assert 0 <= codes_row[j] < (1 << w)
        bits |= int(codes_row[j]) << pos
        pos += w
    assert pos == 272
    return bits.to_bytes(34, "little")


def _mixed_tile_bytes(codes):
    """[128 tokens][128 slots] -> 4352-byte tile: plane g (g < 4) at 1024g + 8t
    holds logical bytes g, 4+g, 8+6g .. 13+6g; bytes 32, 33 at 4096 + 2t
    (header text)"""
    tile = bytearray(4352)
    for t in range(128):
        row = _mixed_row_bytes(codes[t])
        for g in range(4):
            plane = [row[g], row[4 + g]] + [row[8 + 6 * g + i] for i in range(6)]
            tile[1024 * g + 8 * t: 1024 * g + 8 * t + 8] = bytes(plane)
        tile[4096 + 2 * t: 4096 + 2 * t + 2] = row[32:34]
    return np.frombuffer(bytes(tile), dtype=np.uint8)


@pytest.mark.parametrize("pdt", [oracle.E4M3, oracle.F16])
def test_mixed_key_quantizer_against_independent_build(pdt):
    """Every slot j of the oracle's mixed key tile quantizes channel
    slot_chan[j] of the tile's 128 tokens at its class width: Z'_j is the
    narrowed channel minimum, S'_j the narrowed (max - min) / (2^b_j - 1),
    codes 0 and 2^b_j - 1 sit at that channel's argmin and argmax, every code
    is the nearest level S'q + Z' (brute force, exact rationals; only near-ties
    may differ by one) and the bytes equal an independent packing of the
    header's layout text.  Channels get distinct ranges and the permutation is
    not the identity, so a slot that reads the wrong channel or uses the wrong
    width fails."""
    rng = np.random.default_rng(1234 + pdt)
    T = 256
    chan_scale = np.exp(rng.uniform(-1.5, 1.5, 128)).astype(np.float32)
    chan_shift = rng.uniform(-1.0, 1.0, 128).astype(np.float32)
    k = (rng.standard_normal((T, 128)).astype(np.float32) * chan_scale + chan_shift).astype(np.float32)
    if pdt == oracle.E4M3:
        k = (k * np.float32(0.5)).astype(np.float32)
    v = rng.standard_normal((T, 128)).astype(np.float32)
    slot_chan = rng.permutation(128).astype(np.int16)
    assert (slot_chan != np.arange(128)).sum() > 100
    st = oracle.quantize_stream(k, v, 0, 2, pdt, slot_chan)
    S_raw = oracle.decode(st.ks, pdt)
    Z_raw = oracle.decode(st.kz, pdt)
    for g in range(T // 128):
        codes = oracle.unpack_mixed(st.k_tiles[g]).astype(np.int64)      # [token][slot]
        exp_codes = np.zeros((128, 128), np.int64)
        for j in range(128):
            b = _MIXED_WIDTHS[j]
            x = k[128 * g: 128 * g + 128, slot_chan[j]]
            mn, mx = np.float32(x.min()), np.float32(x.max())
            s32 = np.float32(np.float32(mx - mn) / np.float32(2 ** b - 1))
            S, Z = _narrow_ref(s32, pdt), _narrow_ref(mn, pdt)
            assert S_raw[g, j] == S and Z_raw[g, j] == Z, (g, j)
            assert codes[np.argmin(x), j] == 0
            if S > 0 and (mx - Z) / S > (2 ** b - 1) - 0.5:
                assert codes[np.argmax(x), j] == 2 ** b - 1
            Sf, Zf = Fraction(S), Fraction(Z)
            for t in range(128):
                if S == 0:
                    best = 0
                else:
                    ex = (Fraction(float(x[t])) - Zf) / Sf
                    best = min(max(round(ex), 0), 2 ** b - 1)
                    if codes[t, j] != best:
                        tol = max(abs(ex), Fraction(1)) / 2 ** 21
                        assert abs(abs(ex - math.floor(ex)) - Fraction(1, 2)) < tol, (g, j, t)
                        best = int(codes[t, j])
                exp_codes[t, j] = best
            xhat = S * codes[:, j].astype(np.float64) + Z
            bound = max(S / 2, Z - float(mn), float(mx) - Z - (2 ** b - 1) * S)
            assert np.abs(x - xhat).max() <= bound * (1 + 1e-6) + 1e-7
        assert np.array_equal(st.k_tiles[g], _mixed_tile_bytes(exp_codes))


# ---------------------------------------------------------------------------
# mixed-width values: the oracle's tile and quantizer against independent builds
# ---------------------------------------------------------------------------
# Value slot classes (header layout text; ChanMix Key design 3's classes read
# for values with one group per token and class): 16 x 4-bit, 16 x 3-bit,
# 16 x 1-bit, 80 x 2-bit; stored fields 4 bits for slots 0..31, 2 bits after.
_VMIXED_WIDTHS = [4] * 16 + [3] * 16 + [1] * 16 + [2] * 80
_VMIXED_CLASS = [0] * 16 + [1] * 16 + [2] * 16 + [3] * 80


def _vmixed_bitpos(j, t):
    """bit position of (value slot j, token t) in the 5120-byte tile, from the
    header text: block b = j // 16 at word 64 * (4b) (b < 2) or 64 * (8 + 2(b-2));
    word (w * 16 + n) * 4 + a holds 32 / cw tokens 32a + w * (32/cw) + i"""
    b, n = divmod(j, 16)
    cw = 4 if b < 2 else 2
    base = 64 * (4 * b if b < 2 else 8 + 2 * (b - 2))
    a, r = divmod(t, 32)
    w, i = divmod(r, 32 // cw)
    return (base + (w * 16 + n) * 4 + a) * 32 + i * cw, cw


def test_vmixed_tile_positions_by_hand():
    c = np.zeros((128, 128), np.uint16)      # [slot][token]
    c[0, 0] = 0x9                            # block 0, word 0, bits 0..3
    c[17, 9] = 0x5                           # 3-bit slot 17, token 9: word 256 + 17*4 = 324, bits 4..7
    c[33, 40] = 1                            # 1-bit slot 33, token 40: word 512 + 4 + 1 = 517, bit 16
    c[127, 127] = 3                          # last slot and token: word 1279, bits 30..31
    t = oracle.pack_vmixed(c)
    assert t.size == 5120
    assert t[0] == 0x09
    assert t[4 * 324] == 0x50
    assert t[4 * 517 + 2] == 0x01
    assert t[4 * 1279 + 3] == 0xC0
    assert int(np.count_nonzero(t)) == 4
    assert list(oracle.vmixed_slot_bits()) == _VMIXED_WIDTHS
    r = np.random.default_rng(9).integers(0, 1 << 16, (128, 128))
    r = (r % (1 << np.array(_VMIXED_WIDTHS))[:, None]).astype(np.uint16)
    assert np.array_equal(oracle.unpack_vmixed(oracle.pack_vmixed(r)), r)


@pytest.mark.parametrize("pdt", [oracle.E4M3, oracle.F16])
def test_mixed_value_quantizer_against_independent_build(pdt):
    """Every token's value slots of one class form one group: Z' is the
    narrowed minimum of the class's channels (slot -> channel through the
    map), S' the narrowed range / (2^b - 1) at the class width, every code the
    nearest level (brute force, exact rationals), and the bytes equal an
    independent packing of the header's layout text; params are [class][token]."""
    rng = np.random.default_rng(4321 + pdt)
    T = 128
    chan_scale = np.exp(rng.uniform(-1.5, 1.5, 128)).astype(np.float32)
    v = (rng.standard_normal((T, 128)).astype(np.float32) * chan_scale).astype(np.float32)
    if pdt == oracle.E4M3:
        v = (v * np.float32(0.5)).astype(np.float32)
    k = rng.standard_normal((T, 128)).astype(np.float32)
    vsc = rng.permutation(128).astype(np.int16)
    st = oracle.quantize_stream(k, v, 4, 0, pdt, None, vsc)
    S = oracle.decode(st.vs, pdt).T          # params are [class][token]
    Z = oracle.decode(st.vz, pdt).T
    assert S.shape == (T, 4)
    exp_codes = np.zeros((128, T), np.int64)
    first = [0, 16, 32, 48, 128]
    for t in range(T):
        for cls in range(4):
            slots = list(range(first[cls], first[cls + 1]))
            b = _VMIXED_WIDTHS[first[cls]]
            x = v[t, vsc[slots]]
            mn, mx = np.float32(x.min()), np.float32(x.max())
            s32 = np.float32(np.float32(mx - mn) / np.float32(2 ** b - 1))
            Sx, Zx = _narrow_ref(s32, pdt), _narrow_ref(mn, pdt)
            assert S[t, cls] == Sx and Z[t, cls] == Zx, (t, cls)
            for j, xv in zip(slots, x.tolist()):
                if Sx == 0:
                    exp_codes[j, t] = 0
                    continue
                ex = (Fraction(xv) - Fraction(Zx)) / Fraction(Sx)
                exp_codes[j, t] = min(max(round(ex), 0), 2 ** b - 1)
    got = oracle.unpack_vmixed(st.v_tiles[0]).astype(np.int64)
    diff = np.argwhere(got != exp_codes)
    for j, t in diff:          # near-ties only (two binary32 roundings)
        b = _VMIXED_WIDTHS[j]
        cls = _VMIXED_CLASS[j]
        ex = (Fraction(float(v[t, vsc[j]])) - Fraction(float(Z[t, cls]))) / Fraction(float(S[t, cls]))
        assert abs(abs(ex - math.floor(ex)) - Fraction(1, 2)) < max(abs(ex), Fraction(1)) / 2 ** 21
        assert abs(int(got[j, t]) - int(exp_codes[j, t])) == 1
        exp_codes[j, t] = got[j, t]
    bits = 0
    for j in range(128):
        for t in range(T):
            pos, cw = _vmixed_bitpos(j, t)
            bits |= int(exp_codes[j, t]) << pos
    assert np.array_equal(st.v_tiles[0], np.frombuffer(bits.to_bytes(5120, "little"), np.uint8))
    # reconstruction within the storage-mode bound of each (token, class):
    # max(S'/2, Z' - min, max - Z' - (2^b - 1) S')
    V = oracle.dequant_v(st)
    for cls in range(4):
        ch = vsc[first[cls]:first[cls + 1]].astype(np.int64)
        b = _VMIXED_WIDTHS[first[cls]]
        err = np.abs(V[:, ch] - v[:, ch]).max(axis=1)
        mn, mx = v[:, ch].min(axis=1), v[:, ch].max(axis=1)
        bound = np.maximum.reduce([S[:, cls] / 2, Z[:, cls] - mn, mx - Z[:, cls] - (2 ** b - 1) * S[:, cls]])
        assert np.all(err <= bound + 1e-6)


def test_mixed_value_attention_c_matches_numpy():
    """The C two-pass attention reading the mixed value tile (its own unpack
    and slot -> channel scatter) equals the numpy path (dequant_v, softmax)."""
    rng = np.random.default_rng(77)
    k = rng.standard_normal((384, 128)).astype(np.float32)
    v = rng.standard_normal((384, 128)).astype(np.float32)
    q = oracle.narrow(rng.standard_normal((4, 128)).astype(np.float32), oracle.BF16)
    for kb, sc in ((4, None), (0, rng.permutation(128).astype(np.int16))):
        st = oracle.quantize_stream(k, v, kb, 0, oracle.E4M3, sc, rng.permutation(128).astype(np.int16))
        a = oracle.decode_attn(st, q, 1 / math.sqrt(128))
        b = oracle.decode_attn_union([st], q, 1 / math.sqrt(128))
        assert np.allclose(a, b, rtol=1e-11, atol=1e-13)
