"""Pins for the oracle's iq1c and iq1s (IQ1_M and IQ1_S codebook forms) decoders and partials.

llama.cpp PR #304 describes an IQ1_M value as d*(2s+1)*(g+delta) where the ternary g of
eight values come from one grid entry named by an 11-bit index, with a 3-bit sub-scale s
per 16 values and a delta sign per 8. The grid itself is not on the pages; the workloads
use a self-generated one (gen.IQ1C_GRID), which is an input of both the oracle and the
library's repack.

* A hand-assembled golden super-block with a hand-made codebook (tests/golden/
  weight_blocks.json) pins both decoders (C and NumPy) to the byte layout and the value
  formula.
* The same g, s, delta and d written in the iq1t layout (whose decoders are pinned by
  their own golden block) decode to the same values and give the same integer partials.
* With d = 8 every value is an integer, so the folded per-32 partials are an integer
  matmul per block (library routine: NumPy int64 @).
* The generated codebook holds 2048 distinct valid entries; an invalid code is rejected.
* iq1s (IQ1_S: the same 11-bit index per 8 values, but one s and one delta sign per 32
  values) has its own golden block, and re-laid as iq1t (s and delta repeated over the
  block's halves and groups) decodes to the same values.
"""
import json
import os

import numpy as np
import pytest

import gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden_grid(closed_form):
    return np.array([sum(int(eval(closed_form, {}, {"e": e, "j": j})) << (2 * j) for j in range(8))
                     for e in range(2048)], np.uint16)


@pytest.mark.parametrize("fmt,nbytes", [("iq1c", 56), ("iq1s", 50)])
def test_golden_block_decodes(orc, fmt, nbytes):
    with open(os.path.join(GOLD, "weight_blocks.json")) as f:
        g = json.load(f)[fmt]
    grid = _golden_grid(g["grid_closed_form"])
    raw = np.frombuffer(bytes.fromhex(g["hex"].replace(" ", "")), np.uint8)
    assert raw.size == nbytes
    expect = np.array([eval(g["closed_form"], {}, {"i": i}) for i in range(256)], np.float64)
    for k, v in g["spot"].items():
        assert expect[int(k)] == v, k
    wh = orc.dequant_weights(fmt, raw[None, :], 1, 256, grid=grid)[0]
    assert np.array_equal(wh, expect)
    wq, wd, wm, mult = orc.decode_row_c(fmt, raw, 256, grid=grid)
    assert np.array_equal(np.repeat(wd.astype(np.float64), 16) * wq, expect)
    assert np.all(wm == 0)
    s_of_half = np.arange(16) % 8 if fmt == "iq1c" else np.arange(16) // 2
    assert np.array_equal(mult, 2 * s_of_half + 1)


def _as_iq1t(raw_c, N, K, grid):
    """Re-lay iq1c rows in the iq1t byte layout (2-bit codes, s bits, sign bits, d): a byte
    re-layout of the same fields, so both formats must decode to the same values."""
    b = raw_c.reshape(N, K // 256, 56)
    qh = np.stack([b[..., 32:48] & 0xF, b[..., 32:48] >> 4], axis=-1).reshape(N, K // 256, 32)
    idx = b[..., 0:32].astype(np.int64) | ((qh & 7).astype(np.int64) << 8)
    codes = np.stack([(grid[idx] >> (2 * j)) & 3 for j in range(8)], axis=-1).reshape(N, K // 256, 256)
    c4 = codes.astype(np.uint8).reshape(N, K // 256, 64, 4)
    t = np.empty((N, K // 256, 76), np.uint8)
    t[..., 0:64] = c4[..., 0] | (c4[..., 1] << 2) | (c4[..., 2] << 4) | (c4[..., 3] << 6)
    t[..., 64:70] = b[..., 48:54]
    sgn = (qh >> 3).astype(np.uint8).reshape(N, K // 256, 4, 8)
    t[..., 70:74] = np.packbits(sgn, axis=-1, bitorder="little")[..., 0]
    t[..., 74:76] = b[..., 54:56]
    return t.reshape(N, -1)


def test_same_fields_as_iq1t_decode_and_fold_identically(orc):
    N, K, M = 9, 768, 4
    grid = gen.IQ1C_GRID
    raw = gen.weights_iq1c(N, K, seed=4, cfg=81)
    raw_t = _as_iq1t(raw, N, K, grid)
    assert np.array_equal(orc.dequant_weights("iq1c", raw, N, K, grid=grid),
                          orc.dequant_weights("iq1t", raw_t, N, K))
    for n in range(N):
        a = orc.decode_row_c("iq1c", raw[n], K, grid=grid)
        t = orc.decode_row_c("iq1t", raw_t[n], K)
        for u, v in zip(a, t):
            assert np.array_equal(u, v)
    xq = np.random.default_rng(2).integers(-128, 128, size=(M, K), dtype=np.int8)
    assert np.array_equal(orc.partials("iq1c", raw, N, K, xq, grid=grid),
                          orc.partials("iq1t", raw_t, N, K, xq))


def test_folded_partials_are_integer_matmul_with_d8(orc):
    # d = 8: each value is the integer (2s+1)(8g+sigma) and the folded per-32 partial is the
    # block's integer matmul
    M, N, K = 5, 11, 512
    grid = gen.IQ1C_GRID
    raw = gen.weights_iq1c(N, K, seed=6, cfg=82).reshape(N, K // 256, 56)
    raw[..., 54:56] = np.array([np.float16(8.0)]).view(np.uint8)
    raw = raw.reshape(N, -1)
    w_int = orc.dequant_weights("iq1c", raw, N, K, grid=grid)
    assert np.array_equal(w_int, np.rint(w_int))
    xq = np.random.default_rng(3).integers(-128, 128, size=(M, K), dtype=np.int8)
    P = orc.partials("iq1c", raw, N, K, xq, grid=grid)
    for b in range(K // 32):
        ref = xq[:, 32 * b:32 * b + 32].astype(np.int64) @ w_int[:, 32 * b:32 * b + 32].astype(np.int64).T
        assert np.array_equal(P[..., b], ref)


@pytest.mark.parametrize("M", [1, 4])
def test_per_block_oracle_matches_f64_definition(orc, M):
    N, K = 13, 512
    grid = gen.IQ1C_GRID
    raw = gen.weights_iq1c(N, K, seed=2, cfg=83)
    x = gen.act_f32(M, K, seed=2, cfg=83, outlier_rate=0.01)
    xq, xs, xsum = orc.quantize_q8_1(x)
    ref = orc.gemm_f64("iq1c", raw, N, K, xq, xs, grid=grid)
    got = orc.gemm_c("iq1c", raw, N, K, xq, xs, xsum, grid=grid)
    assert np.max(np.abs(got - ref)) <= 4e-7 * np.abs(ref).max()


def test_generated_grid_and_weights():
    g = gen.IQ1C_GRID
    assert g.shape == (2048,) and g.dtype == np.uint16
    assert len(np.unique(g)) == 2048
    codes = np.stack([(g >> (2 * j)) & 3 for j in range(8)], axis=-1)
    assert codes.max() <= 2
    frac = np.bincount(codes.ravel(), minlength=3) / codes.size
    assert np.all(np.abs(frac - 1 / 3) < 0.02)
    raw = gen.weights_iq1c(64, 4096, seed=0, cfg=5).reshape(64, 16, 56)
    assert raw.shape[-1] * 8 == 7 * 64             # 56 B per 256 values = 1.75 bits per value
    assert np.all(raw[..., 54:56].copy().view(np.float16) == np.float16(0.005))
    qh = np.stack([raw[..., 32:48] & 0xF, raw[..., 32:48] >> 4], axis=-1)
    idx = raw[..., 0:32].astype(np.int64) | ((qh.reshape(64, 16, 32) & 7).astype(np.int64) << 8)
    assert idx.max() <= 2047 and len(np.unique(idx)) > 1900


def test_invalid_grid_code_is_rejected(orc):
    grid = gen.IQ1C_GRID.copy()
    raw = gen.weights_iq1c(1, 256, seed=1, cfg=84)
    first = int(raw[0, 0]) | ((int(raw[0, 32]) & 7) << 8)   # group 0's index
    grid[first] |= 3                                          # value 0's code becomes 3
    with pytest.raises(ValueError):
        orc.decode_row_c("iq1c", raw[0], 256, grid=grid)
    with pytest.raises(ValueError):
        orc.dequant_weights("iq1c", raw, 1, 256, grid=grid)
    with pytest.raises(ValueError):
        orc.partials("iq1c", raw, 1, 256, np.ones((1, 256), np.int8), grid=grid)


def _iq1s_as_iq1t(raw_s, N, K, grid):
    """The same g, s, delta and d in the iq1t byte layout: s and the delta sign of each 32-value
    block repeated over its two halves and four groups (a re-layout of fields)."""
    b = raw_s.reshape(N, K // 256, 50)
    qh = (b[..., 34:50:2].astype(np.int64) | (b[..., 35:50:2].astype(np.int64) << 8))
    hi = np.stack([(qh >> (3 * j)) & 7 for j in range(4)], axis=-1)
    idx = b[..., 2:34].astype(np.int64).reshape(N, K // 256, 8, 4) | (hi << 8)
    codes = np.stack([(grid[idx] >> (2 * j)) & 3 for j in range(8)], axis=-1).reshape(N, K // 256, 256)
    c4 = codes.astype(np.uint8).reshape(N, K // 256, 64, 4)
    t = np.empty((N, K // 256, 76), np.uint8)
    t[..., 0:64] = c4[..., 0] | (c4[..., 1] << 2) | (c4[..., 2] << 4) | (c4[..., 3] << 6)
    s16 = np.repeat((qh >> 12) & 7, 2, axis=-1).astype(np.uint64)            # [N, sb, 16]
    word = np.zeros((N, K // 256), np.uint64)
    for h in range(16):
        word |= s16[..., h] << np.uint64(3 * h)
    for k in range(6):
        t[..., 64 + k] = ((word >> np.uint64(8 * k)) & np.uint64(0xFF)).astype(np.uint8)
    sg = np.repeat((qh >> 15) & 1, 4, axis=-1).astype(np.uint8).reshape(N, K // 256, 4, 8)
    t[..., 70:74] = np.packbits(sg, axis=-1, bitorder="little")[..., 0]
    t[..., 74:76] = b[..., 0:2]
    return t.reshape(N, -1)


def test_iq1s_same_fields_as_iq1t(orc):
    N, K, M = 7, 768, 3
    grid = gen.IQ1C_GRID
    raw = gen.weights_iq1s(N, K, seed=4, cfg=89)
    raw_t = _iq1s_as_iq1t(raw, N, K, grid)
    assert np.array_equal(orc.dequant_weights("iq1s", raw, N, K, grid=grid),
                          orc.dequant_weights("iq1t", raw_t, N, K))
    xq = np.random.default_rng(5).integers(-128, 128, size=(M, K), dtype=np.int8)
    assert np.array_equal(orc.partials("iq1s", raw, N, K, xq, grid=grid),
                          orc.partials("iq1t", raw_t, N, K, xq))
    x = gen.act_f32(M, K, seed=4, cfg=89)
    q, xs, xsum = orc.quantize_q8_1(x)
    ref = orc.gemm_f64("iq1s", raw, N, K, q, xs, grid=grid)
    assert np.max(np.abs(orc.gemm_c("iq1s", raw, N, K, q, xs, xsum, grid=grid) - ref)) <= 4e-7 * np.abs(ref).max()
    assert raw.shape[1] * 8 == K * 1.5625                 # 50 B per 256 values
