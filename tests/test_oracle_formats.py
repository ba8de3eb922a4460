"""Pins for the oracle's weight decoders and the IQ1_M fold.

* Hand-assembled golden blocks (tests/golden/weight_blocks.json) pin both of the
  oracle's decoders (the C one used for integer partials and the NumPy f64 one
  used for the definition) to the value formulas: q8_0 d*q, q4_0 d*(nib-8)
  (minfer R1 section 1), Q4_K d*sc*nib - dmin*m (minfer R1 section 2.2),
  IQ1_M-style d*(2s+1)*(g+delta) (llama.cpp PR #304 description), q6_K d*sc_h*(q-32)
  with an int8 scale per 16 values (minfer R1 sections 2.2 and 3.3).
* The IQ1_M fold 8(g+delta) = 8g+-1 with per-16 scale d(2s+1)/8 (PR #304) is
  checked exhaustively for exactness in f64 and f32.
* The seeded generators are checked to encode what they claim (round trip
  within half a quantisation step), which pins generator and decoder together.
"""
import json
import os

import numpy as np
import pytest

import gen

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLD, "weight_blocks.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0", "q4_K", "q6_K", "iq1t"])
def test_golden_block_decodes(orc, fmt):
    g = _golden()[fmt]
    raw = np.frombuffer(bytes.fromhex(g["hex"].replace(" ", "")), np.uint8)
    K = gen.VALUES_PER_BLOCK[fmt]
    expect = np.array([eval(g["closed_form"], {}, {"i": i}) for i in range(K)], np.float64)
    for k, v in g["spot"].items():               # the hand-worked spot values
        assert expect[int(k)] == v, (fmt, k)
    wh = orc.dequant_weights(fmt, raw[None, :], 1, K)[0]
    assert np.array_equal(wh, expect)
    wq, wd, wm, _ = orc.decode_row_c(fmt, raw, K)
    wc = np.repeat(wd.astype(np.float64), 16) * wq + np.repeat(wm.astype(np.float64), 32)
    assert np.array_equal(wc, expect)


def test_q4_K_sixbit_fields_round_trip_every_value(orc):
    # every 6-bit value in every sub-block slot, scale and min, decoded back
    K = 256
    rows = []
    for base in range(0, 64, 8):
        blk = np.zeros(144, np.uint8)
        blk[0:2] = np.array([np.float16(1.0)]).view(np.uint8)
        blk[2:4] = np.array([np.float16(1.0)]).view(np.uint8)
        vals = np.arange(base, base + 8)
        for off, field in ((4, vals), (10, 63 - vals)):
            word = 0
            for j, v in enumerate(field):
                word |= int(v) << (6 * j)
            blk[off:off + 6] = np.frombuffer(word.to_bytes(6, "little"), np.uint8)
        blk[16:] = 0x11                           # nib = 1 everywhere
        rows.append(blk)
        wq, wd, wm, _ = orc.decode_row_c("q4_K", blk, K)
        assert np.array_equal(wd[::2], vals.astype(np.float32))
        assert np.array_equal(wm, -(63 - vals).astype(np.float32))
    wh = orc.dequant_weights("q4_K", np.stack(rows), len(rows), K)
    # w = d*sc*nib - dmin*m with d = dmin = nib = 1: sc - m = 2*sc - 63
    expect = np.stack([np.repeat(2.0 * np.arange(b, b + 8) - 63, 32) for b in range(0, 64, 8)])
    assert np.array_equal(wh, expect)


def test_iq1_fold_is_exact():
    # PR #304: d(2s+1)(g+delta) == (d(2s+1)/8) * (8g + sigma), delta = sigma/8, for every
    # g in {-1,0,1}, sigma in {+1,-1}, s in 0..7, and many f16 d - exactly in f64 and f32.
    r = np.random.default_rng(5)
    d16 = np.concatenate([r.standard_normal(10000).astype(np.float16),
                          np.array([6.1e-5, 65504, 1.0, 0.005], np.float16)])
    d16 = d16[np.isfinite(d16.astype(np.float32))]
    for dt in (np.float64, np.float32):
        d = d16.astype(dt)
        for g in (-1, 0, 1):
            for sig in (1, -1):
                for s in range(8):
                    lhs = d * dt(2 * s + 1) * (dt(g) + dt(sig) / dt(8))
                    rhs = (d * dt(2 * s + 1) / dt(8)) * dt(8 * g + sig)
                    assert np.array_equal(lhs, rhs), (dt, g, sig, s)
    # the folded integers are exactly the set the PR lists
    assert sorted({8 * g + s for g in (-1, 0, 1) for s in (1, -1)}) == [-9, -7, -1, 1, 7, 9]


def test_iq1_c_decoder_uses_fold_and_matches_definition(orc):
    K, N = 512, 5
    raw = gen.weights_iq1t(N, K, seed=3, cfg=99)
    wh = orc.dequant_weights("iq1t", raw, N, K)
    for n in range(N):
        wq, wd, wm, _ = orc.decode_row_c("iq1t", raw[n], K)
        assert set(np.unique(wq)) <= {-9, -7, -1, 1, 7, 9}
        assert np.array_equal(np.repeat(wd.astype(np.float64), 16) * wq, wh[n])
        assert np.all(wm == 0)


# ------------------------------------------------------------ generators

def test_q8_0_generator_round_trip(orc):
    N, K = 17, 256
    raw = gen.weights_q8_0(N, K, seed=0, cfg=1)
    w = gen._normal_weights(N, K, 0, 1, gen.T_WEIGHT, 0.02).astype(np.float64)
    wh = orc.dequant_weights("q8_0", raw, N, K)
    d = wh.reshape(N, K // 32, 32)
    step = np.abs(w).reshape(N, K // 32, 32).max(axis=2, keepdims=True) / 127
    assert np.all(np.abs(d - w.reshape(N, K // 32, 32)) <= 0.5 * step * 1.01 + 1e-12)


def test_q4_0_generator_round_trip(orc):
    N, K = 9, 512
    raw = gen.weights_q4_0(N, K, seed=0, cfg=2)
    w = gen._normal_weights(N, K, 0, 2, gen.T_WEIGHT, 0.02).astype(np.float64).reshape(N, K // 32, 32)
    wh = orc.dequant_weights("q4_0", raw, N, K).reshape(N, K // 32, 32)
    peak = np.take_along_axis(w, np.abs(w).argmax(axis=2)[..., None], axis=2)
    d = np.abs(peak) / 8
    qs = raw.reshape(N, K // 32, 18)[..., 2:]
    nib = np.concatenate([qs & 0xF, qs >> 4], axis=-1)
    err = np.abs(wh - w)
    # unclipped values round to the nearest step; values of the sign opposite to the peak can
    # clip at nib 15 (value 7*d instead of 8*d), so their error is below one step
    assert np.all(err[nib < 15] <= 0.5 * np.broadcast_to(d, err.shape)[nib < 15] * 1.01 + 1e-12)
    assert np.all(err <= d * 1.01 + 1e-12)
    # the peak itself sits on nib 0 (d = peak/-8)
    assert np.all(np.take_along_axis(nib, np.abs(w).argmax(axis=2)[..., None], axis=2) == 0)


def test_q4_K_generator_round_trip(orc):
    N, K = 7, 512
    raw = gen.weights_q4_K(N, K, seed=0, cfg=3)
    w = gen._normal_weights(N, K, 0, 3, gen.T_WEIGHT, 0.02).astype(np.float64)
    wh = orc.dequant_weights("q4_K", raw, N, K)
    # Q4_K is coarse (4-bit steps with 6-bit scales); error stays well under the per-block range/15
    rng_ = (w.reshape(N, -1, 32).max(axis=2) - np.minimum(w.reshape(N, -1, 32).min(axis=2), 0))
    err = np.abs(wh - w).reshape(N, -1, 32).max(axis=2)
    assert np.all(err <= rng_ / 15 * 1.5 + 1e-6)


def test_iq1t_generator_distribution(orc):
    N, K = 64, 4096
    raw = gen.weights_iq1t(N, K, seed=0, cfg=5)
    b = raw.reshape(N, K // 256, 76)
    codes = np.stack([(b[..., :64] >> (2 * j)) & 3 for j in range(4)], -1)
    assert codes.max() <= 2                       # code 3 never generated
    frac = np.bincount(codes.ravel(), minlength=3) / codes.size
    assert np.all(np.abs(frac - 1 / 3) < 0.01)
    d = b[..., 74:76].copy().view(np.float16)
    assert np.all(d == np.float16(0.005))


def test_q6_K_generator_round_trip(orc):
    N, K = 7, 512
    raw = gen.weights_q6_K(N, K, seed=0, cfg=6)
    w = gen._normal_weights(N, K, 0, 6, gen.T_WEIGHT, 0.02).astype(np.float64).reshape(N, K // 16, 16)
    wh = orc.dequant_weights("q6_K", raw, N, K).reshape(N, K // 16, 16)
    b = raw.reshape(N, K // 256, 210)
    sc = b[..., 192:208].view(np.int8).astype(np.float64).reshape(N, K // 16, 1)
    d = b[..., 208:210].copy().view(np.float16).astype(np.float64).reshape(N, K // 256, 1, 1)
    step = np.abs(np.broadcast_to(d, (N, K // 256, 16, 1)).reshape(N, K // 16, 1) * sc)
    err = np.abs(wh - w)
    # values inside the grid round to the nearest step (d*sc); only values beyond it clip at
    # q = 0 or 63 (the step is the rounded w_peak/-32, so the far side can exceed 31 steps)
    ratio = w / np.where(step != 0, np.sign(sc) * step, 1)
    inside = (ratio >= -32.5) & (ratio <= 31.5)
    assert np.all(err[inside] <= 0.5 * np.broadcast_to(step, err.shape)[inside] * (1 + 1e-6) + 1e-12)
    assert inside.mean() > 0.95
    assert np.median(err / np.maximum(step, 1e-12)) < 0.3
    assert np.any(sc < 0) and np.any(sc > 0)      # both signs of sub-scale occur


def test_i8_rows_generator(orc):
    q, s = gen.i8_rows(33, 4096, seed=0, cfg=4)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert np.all(np.abs(q.astype(np.int32)).max(axis=1) == 127)


def test_moe_ids_distinct():
    ids = gen.moe_ids(512, 8, 64, seed=0, cfg=5)
    assert ids.shape == (512, 8) and ids.dtype == np.int32
    assert all(len(set(r)) == 8 for r in ids)
    assert ids.min() >= 0 and ids.max() < 64
    counts = np.bincount(ids.ravel(), minlength=64)
    assert counts.sum() == 4096 and 30 < counts.mean() < 100
