"""CPU checks of the GPU tests' output bars (tests/parity.py) and of the oracle's term
magnitudes (oracle.gemm_abs): the bars accept an f32 evaluation that adds the per-block terms
one at a time (what the kernels do), and reject a scale-path defect far below the pages' 1e-3
gate - q4_K with the low half of its exact f16 split of d*sc dropped (an error of up to 2^-12
per term)."""
import numpy as np
import pytest

import gen
import parity


def _blocks(orc, fmt, N, K, seed):
    raw = gen.weights(fmt, N, K, seed=seed, cfg=120)
    x = gen.act_f32(9, K, seed=seed, cfg=120, outlier_rate=1e-2)
    xq, xs, xsum = orc.quantize_q8_1(x)
    P16 = orc.partials16(fmt, raw, N, K, xq).astype(np.float64)           # [M, N, K/16]
    dec = [orc.decode_row_c(fmt, raw[n], K) for n in range(N)]
    wd = np.stack([d[1] for d in dec]).astype(np.float64)                  # [N, K/16]
    wm = np.stack([d[2] for d in dec]).astype(np.float64)                  # [N, K/32]
    return raw, xq, xs, xsum, P16, wd, wm


def _f32_accumulate(terms):
    """terms [M, N, T] in f64, each exact: acc = f32(acc + t) in order (one rounding per term)."""
    acc = np.zeros(terms.shape[:2], np.float32)
    for i in range(terms.shape[2]):
        acc = (acc.astype(np.float64) + terms[..., i]).astype(np.float32)
    return acc


def _terms(xs, xsum, P16, wd, wm, split_hi_only=False):
    M, N, H = P16.shape
    xs2 = np.repeat(xs.astype(np.float64), 2, axis=1)                      # [M, K/16]
    w = wd
    if split_hi_only:
        w = w.astype(np.float32).astype(np.float16).astype(np.float64)     # keep only the hi half
    t = xs2[:, None, :] * w[None, :, :] * P16                              # per half-block
    tm = xs.astype(np.float64)[:, None, :] * wm[None, :, :] * xsum.astype(np.float64)[:, None, :]
    return np.concatenate([t, tm], axis=2)


@pytest.mark.parametrize("fmt", ["q4_K", "q4_0", "q6_K"])
def test_bars_accept_an_f32_evaluation(orc, fmt):
    N, K = 40, 1024
    raw, xq, xs, xsum, P16, wd, wm = _blocks(orc, fmt, N, K, seed=1)
    got = _f32_accumulate(_terms(xs, xsum, P16, wd, wm))
    r1, r2 = parity.check_f32(orc, got, fmt, raw, N, K, xq, xs, xsum)
    assert r1 < 1e-6 and r2 < 1e-6


def test_bars_reject_a_dropped_split_half(orc):
    N, K = 40, 1024
    raw, xq, xs, xsum, P16, wd, wm = _blocks(orc, "q4_K", N, K, seed=2)
    bad = _f32_accumulate(_terms(xs, xsum, P16, wd, wm, split_hi_only=True))
    ref = orc.gemm_f64("q4_K", raw, N, K, xq, xs)
    assert parity.rel(bad, ref) <= parity.PAGES_GATE          # the pages' gate alone passes it
    with pytest.raises(AssertionError):
        parity.check_f32(orc, bad, "q4_K", raw, N, K, xq, xs, xsum)


def test_gemm_abs_pins(orc):
    # magnitudes bound the result, equal it when every term has one sign, and scale linearly
    N, K = 24, 512
    raw = gen.weights("q4_0", N, K, seed=3, cfg=121)
    x = gen.act_f32(5, K, seed=3, cfg=121)
    xq, xs, xsum = orc.quantize_q8_1(x)
    out = orc.gemm_c("q4_0", raw, N, K, xq, xs, xsum).astype(np.float64)
    a = orc.gemm_abs("q4_0", raw, N, K, xq, xs, xsum)
    assert np.all(a >= np.abs(out) * (1 - 1e-6))
    assert np.array_equal(orc.gemm_abs("q4_0", raw, N, K, xq, 2 * xs, xsum), 2 * a)
    # one sign: q8_0 weights all >= 0 (d > 0, q >= 0) against activations all >= 0
    w = gen.weights("q8_0", N, K, seed=4, cfg=121).reshape(N, K // 32, 34).copy()
    w[..., 2:] = np.abs(w[..., 2:].view(np.int8)).astype(np.uint8)
    d = w[..., 0:2].copy().view(np.float16)
    w[..., 0:2] = np.abs(d).view(np.uint8)
    w = w.reshape(N, -1)
    xq2, xs2, xsum2 = orc.quantize_q8_1(np.abs(x))
    o2 = orc.gemm_c("q8_0", w, N, K, xq2, xs2, xsum2).astype(np.float64)
    a2 = orc.gemm_abs("q8_0", w, N, K, xq2, xs2, xsum2)
    assert np.allclose(a2, o2, rtol=1e-7, atol=0)
