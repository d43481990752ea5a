"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and the CPU oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import math

import numpy as np

import oracle
from kv_cache_mixed_amd import kvq, synth

PDT_ORACLE = {kvq.F32: oracle.F32, kvq.F16: oracle.F16, kvq.BF16: oracle.BF16,
              kvq.E4M3: oracle.E4M3}
SCALE = 1.0 / math.sqrt(128.0)
REL_TOL = 2e-3   # max over rows of ||o - o_ref||_inf / ||o_ref||_inf


def to_dev(x, torch):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def q_to_dev(q_bits, torch):
    return torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).cuda().view(torch.bfloat16)


def oracle_stream(inp, b, h, k_bits, v_bits, pdt, slot_chan=None):
    return oracle.quantize_stream(inp["k"][b, h], inp["v"][b, h], k_bits, v_bits,
                                  PDT_ORACLE[pdt], slot_chan)


def assert_stream_bytes_equal(cache, st, b, h, what=""):
    """Bit-exact comparison of every stored tile and parameter of stream (b, h)."""
    nt = cache.n_tokens // 128
    for g in range(nt):
        kt = cache.k_tile(b, h, g)
        assert np.array_equal(kt, st.k_tiles[g]), "%s key tile (b=%d,h=%d,g=%d) differs at bytes %s" % (
            what, b, h, g, np.flatnonzero(kt != st.k_tiles[g])[:8])
        vt = cache.v_tile(b, h, g)
        assert np.array_equal(vt, st.v_tiles[g]), "%s value tile (b=%d,h=%d,g=%d) differs at %s" % (
            what, b, h, g, np.flatnonzero(vt != st.v_tiles[g])[:8])
    ks, kz = cache.k_params(b, h)
    vs, vz = cache.v_params(b, h)
    assert np.array_equal(ks.view(np.uint8), np.ascontiguousarray(st.ks).view(np.uint8)), what + " key scales"
    assert np.array_equal(kz.view(np.uint8), np.ascontiguousarray(st.kz).view(np.uint8)), what + " key zeros"
    assert np.array_equal(vs.view(np.uint8), np.ascontiguousarray(st.vs).view(np.uint8)), what + " value scales"
    assert np.array_equal(vz.view(np.uint8), np.ascontiguousarray(st.vz).view(np.uint8)), what + " value zeros"


def rel_err_rows(out, ref):
    """per-row ||out - ref||_inf / ||ref||_inf"""
    num = np.abs(out - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return num / np.maximum(den, 1e-300)


def oracle_attn(st, q_bits_rows):
    return oracle.decode_attn(st, q_bits_rows, SCALE)
