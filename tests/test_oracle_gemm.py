"""Pins for the oracle's integer partials, f32 output, W8A8 and MoE paths.

The contraction is out[m,n] = sum over 32-blocks b of (xs[m,b]*wd[n,b]) *
sum_{k in b} xq[m,k]*wq[n,k] ("A Negative Result on int8 Tensor-Core MMQ",
section 2; minfer R1 section 2.1). Pins used here, none of which retypes the
oracle's own loops:

* special cases that reduce to a library routine: with every weight scale set
  to 1 (and d = 8 for iq1t) the block partials are an exact integer matmul of
  each 32-column block, computed with NumPy int64 '@';
* brute force on tiny inputs: the per-block C oracle against the f64
  definition (dequantise both sides, one f64 matmul);
* closed forms: K = 32 (one block), M = 1 (a matvec), the int32 worst cases of
  the pages' bounds;
* W8A8 with unit scales is an integer matmul; its bf16 rounding is checked
  against PyTorch's conversion;
* MoE reduces, pair by pair, to the dense definition and is equivariant under
  token permutation.
"""
import numpy as np
import pytest

import gen


def _set_scale(raw, fmt, N, K, value, field=0):
    """Overwrite every block's f16 scale field (field 0 = d, 1 = dmin for q4_K) with value."""
    raw = raw.copy().reshape(N, -1)
    bits = np.array([np.float16(value)]).view(np.uint8)
    if fmt in ("q8_0", "q4_0"):
        bs = 34 if fmt == "q8_0" else 18
        b = raw.reshape(N, K // 32, bs)
        b[..., 0:2] = bits
    elif fmt == "q4_K":
        b = raw.reshape(N, K // 256, 144)
        b[..., 2 * field:2 * field + 2] = bits
    elif fmt == "iq1t":
        b = raw.reshape(N, K // 256, 76)
        b[..., 74:76] = bits
    return raw.reshape(N, -1)


def _block_int_matmul(xq, w_int, K):
    """sum over each 32-column block of xq @ w_int.T, with NumPy int64 matmul."""
    M, N = xq.shape[0], w_int.shape[0]
    out = np.empty((M, N, K // 32), np.int64)
    for b in range(K // 32):
        out[..., b] = xq[:, 32 * b:32 * b + 32].astype(np.int64) @ w_int[:, 32 * b:32 * b + 32].astype(np.int64).T
    return out


def _xq(M, K, seed):
    r = np.random.default_rng(seed)
    return r.integers(-128, 128, size=(M, K)).astype(np.int8)


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_partials_unit_scale_equal_block_int_matmul(orc, fmt):
    M, N, K = 7, 11, 256
    raw = _set_scale(gen.weights(fmt, N, K, seed=1, cfg=50), fmt, N, K, 1.0)
    w_int = orc.dequant_weights(fmt, raw, N, K)           # d = 1: the integers themselves
    assert np.array_equal(w_int, np.rint(w_int))
    xq = _xq(M, K, 6)
    P = orc.partials(fmt, raw, N, K, xq)
    assert np.array_equal(P, _block_int_matmul(xq, w_int, K))


def test_partials_q4_K_unsigned_nibbles(orc):
    M, N, K = 5, 9, 512
    raw = _set_scale(gen.weights_q4_K(N, K, seed=1, cfg=51), "q4_K", N, K, 1.0, field=0)
    raw = _set_scale(raw, "q4_K", N, K, 0.0, field=1)       # dmin = 0 -> w = sc * nib
    b = raw.reshape(N, K // 256, 144)
    b[..., 4:10] = np.frombuffer(sum(1 << (6 * j) for j in range(8)).to_bytes(6, "little"), np.uint8)  # sc = 1
    raw = b.reshape(N, -1)
    nib = orc.dequant_weights("q4_K", raw, N, K)            # = nib exactly
    assert nib.min() >= 0 and nib.max() <= 15
    xq = _xq(M, K, 7)
    P = orc.partials("q4_K", raw, N, K, xq)
    assert np.array_equal(P, _block_int_matmul(xq, nib, K))


def test_partials_iq1t_folded_is_integer_matmul_with_d8(orc):
    # with d = 8 the dequantised value is (2s+1)(8g+sigma), an integer: the folded per-32
    # partial sum_h (2s_h+1) P16_h is the integer matmul of each block
    M, N, K = 6, 10, 512
    raw = _set_scale(gen.weights_iq1t(N, K, seed=1, cfg=52), "iq1t", N, K, 8.0)
    w_int = orc.dequant_weights("iq1t", raw, N, K)
    assert np.array_equal(w_int, np.rint(w_int))
    xq = _xq(M, K, 8)
    assert np.array_equal(orc.partials("iq1t", raw, N, K, xq), _block_int_matmul(xq, w_int, K))
    # and the unfolded per-16 partials with s forced to 0 (2s+1 = 1) are the 16-column matmuls
    b = raw.reshape(N, K // 256, 76)
    b[..., 64:70] = 0
    raw0 = b.reshape(N, -1)
    v = orc.dequant_weights("iq1t", raw0, N, K)              # = 8g + sigma
    P16 = orc.partials16_iq1t(raw0, N, K, xq)
    for h in range(K // 16):
        ref = xq[:, 16 * h:16 * h + 16].astype(np.int64) @ v[:, 16 * h:16 * h + 16].astype(np.int64).T
        assert np.array_equal(P16[..., h], ref)


def test_partials16_q6_K_are_half_block_int_matmuls(orc):
    # minfer R1 sections 2.2 and 3.3: each 32-value q6_K block is two 16-value halves with
    # separate integer sums of xq*(q-32). With d = 1 and every sc = 1 the dequantised value is
    # the integer q-32, so each per-16 partial is the 16-column integer matmul.
    M, N, K = 6, 9, 512
    raw = gen.weights_q6_K(N, K, seed=3, cfg=55).reshape(N, K // 256, 210)
    raw[..., 192:208] = 1
    raw[..., 208:210] = np.array([np.float16(1.0)]).view(np.uint8)
    raw = raw.reshape(N, -1)
    v = orc.dequant_weights("q6_K", raw, N, K)
    assert np.array_equal(v, np.rint(v)) and v.min() >= -32 and v.max() <= 31
    xq = _xq(M, K, 9)
    P16 = orc.partials16("q6_K", raw, N, K, xq)
    for h in range(K // 16):
        ref = xq[:, 16 * h:16 * h + 16].astype(np.int64) @ v[:, 16 * h:16 * h + 16].astype(np.int64).T
        assert np.array_equal(P16[..., h], ref)
    # worst case of one half: all q = 0 (value -32) against xq = -128 -> 16 * 32 * 128
    raw0 = raw.reshape(N, K // 256, 210).copy()
    raw0[..., 0:192] = 0
    P16w = orc.partials16("q6_K", raw0.reshape(N, -1), N, K, np.full((1, K), -128, np.int8))
    assert np.all(P16w == 16 * 32 * 128)


def test_partials_int32_worst_cases(orc):
    # the bounds behind the exact int32 accumulation (minfer R1 section 2.1; PR #304's per-16 bound
    # 16*9*127 = 18288, garbled on the page): worst blocks hit exactly these values.
    K = 256
    xq = np.full((1, K), -128, np.int8)
    # q8_0: all q = -128 -> 32 * 128 * 128
    raw = gen.weights_q8_0(1, K, seed=0, cfg=53).reshape(1, K // 32, 34)
    raw[..., 2:] = np.uint8(0x80)
    assert orc.partials("q8_0", raw.reshape(1, -1), 1, K, xq)[0, 0, 0] == 32 * 128 * 128
    # q4_0: all nib = 0 -> value -8
    raw = gen.weights_q4_0(1, K, seed=0, cfg=53).reshape(1, K // 32, 18)
    raw[..., 2:] = 0
    assert orc.partials("q4_0", raw.reshape(1, -1), 1, K, xq)[0, 0, 0] == 32 * 8 * 128
    # iq1t: every value -9 (g=-1, sign -), s = 7 -> per-16 |P16| = 16*9*128, folded 2*15*16*9*128
    raw = gen.weights_iq1t(1, K, seed=0, cfg=53).reshape(1, 1, 76)
    raw[..., :64] = 0                                        # c = 0 -> g = -1
    raw[..., 64:70] = 0xFF                                   # s = 7
    raw[..., 70:74] = 0xFF                                   # delta = -1/8
    raw = raw.reshape(1, -1)
    xq127 = np.full((1, K), 127, np.int8)
    P16 = orc.partials16_iq1t(raw, 1, K, xq127)
    assert np.all(P16 == -16 * 9 * 127) and 16 * 9 * 127 == 18288
    assert np.all(orc.partials("iq1t", raw, 1, K, xq127) == -2 * 15 * 16 * 9 * 127)


@pytest.mark.parametrize("fmt,K", [("q8_0", 32), ("q8_0", 256), ("q4_0", 96), ("q4_K", 256),
                                   ("q4_K", 512), ("iq1t", 256), ("iq1t", 768), ("q6_K", 256),
                                   ("q6_K", 768)])
@pytest.mark.parametrize("M", [1, 5])
def test_per_block_oracle_matches_f64_definition(orc, fmt, K, M):
    # brute force: the per-block integer oracle (C) against the f64 definition sum_k x_hat*w_hat
    N = 13
    raw = gen.weights(fmt, N, K, seed=2, cfg=54)
    x = gen.act_f32(M, K, seed=2, cfg=54, outlier_rate=0.01)
    xq, xs, xsum = orc.quantize_q8_1(x)
    ref = orc.gemm_f64(fmt, raw, N, K, xq, xs)
    got = orc.gemm_c(fmt, raw, N, K, xq, xs, xsum)
    tol = 4e-7 * np.abs(ref).max() + 1e-30
    assert np.max(np.abs(got - ref)) <= tol


def test_single_block_by_hand(orc):
    # K = 32: one block; q8_0 with d = 0.5 and activations with amax = 127 (xs = 1)
    K = 32
    xrow = np.zeros((1, K), np.float32)
    xrow[0, :4] = [127, -3, 2, 5]
    xq, xs, xsum = orc.quantize_q8_1(xrow)
    assert xq[0, :4].tolist() == [127, -3, 2, 5] and xs[0, 0] == 1.0 and xsum[0, 0] == 131
    raw = np.zeros((1, 34), np.uint8)
    raw[0, 0:2] = np.array([np.float16(0.5)]).view(np.uint8)
    raw[0, 2:6] = np.array([1, 2, -4, 10], np.int8).view(np.uint8)
    # P = 127*1 + (-3)*2 + 2*(-4) + 5*10 = 163; out = 1 * 0.5 * 163 = 81.5
    assert orc.partials("q8_0", raw, 1, K, xq)[0, 0, 0] == 163
    assert orc.gemm_c("q8_0", raw, 1, K, xq, xs, xsum)[0, 0] == np.float32(81.5)
    assert orc.gemm_f64("q8_0", raw, 1, K, xq, xs)[0, 0] == 81.5


def test_q4_K_min_term_uses_block_sum(orc):
    # minfer R1 section 2.2: sum(w*q) = ds*sum(nib*q) - dmin*sum(q); with nib = 0 everywhere the
    # output is exactly -dmin*m*xs*xsum per block
    K, N = 256, 2
    raw = gen.weights_q4_K(N, K, seed=3, cfg=55).reshape(N, 1, 144)
    raw[..., 16:] = 0
    raw = raw.reshape(N, -1)
    x = gen.act_f32(3, K, seed=3, cfg=55)
    xq, xs, xsum = orc.quantize_q8_1(x)
    wh = orc.dequant_weights("q4_K", raw, N, K).reshape(N, 8, 32)
    mins = -wh[..., 0]                                       # dmin*m_j per sub-block
    ref = -(xs.astype(np.float64) * xsum) @ mins.T
    got = orc.gemm_c("q4_K", raw, N, K, xq, xs, xsum)
    assert np.allclose(got, ref, rtol=1e-6, atol=0)


def test_w8a8_unit_scales_is_integer_matmul(orc):
    M, N, K = 9, 14, 320
    r = np.random.default_rng(9)
    a = r.integers(-128, 128, (M, K)).astype(np.int8)
    w = r.integers(-127, 128, (N, K)).astype(np.int8)
    out, acc = orc.gemm_w8a8(a, np.ones(M, np.float32), w, np.ones(N, np.float32), want_acc=True)
    ref = a.astype(np.int64) @ w.astype(np.int64).T
    assert np.array_equal(acc, ref)


def test_w8a8_bf16_epilogue_matches_torch_rounding(orc):
    import torch
    M, N, K = 6, 10, 256
    a, sa = gen.i8_rows(M, K, seed=4, cfg=56, tensor=0)
    w, sw = gen.i8_rows(N, K, seed=4, cfg=56, tensor=1)
    out, acc = orc.gemm_w8a8(a, sa, w, sw, want_acc=True)
    t = (torch.from_numpy(acc.astype(np.float32)) * torch.from_numpy(sa)[:, None]) * torch.from_numpy(sw)[None, :]
    ref = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, ref)


def test_w8a8_worst_case_accumulator_fits_int32(orc):
    K = 4096
    a = np.full((1, K), -128, np.int8)
    w = np.full((1, K), -127, np.int8)
    _, acc = orc.gemm_w8a8(a, np.ones(1, np.float32), w, np.ones(1, np.float32), want_acc=True)
    assert acc[0, 0] == 4096 * 128 * 127


def test_moe_reduces_to_dense_and_is_permutation_equivariant(orc):
    E, N, K, T, top_k = 6, 16, 256, 10, 3
    raw = np.stack([gen.weights_iq1t(N, K, seed=5, cfg=57, tensor=10 + e) for e in range(E)])
    ids = gen.moe_ids(T, top_k, E, seed=5, cfg=57)
    x = gen.act_f32(T, K, seed=5, cfg=57)
    xq, xs, xsum = orc.quantize_q8_1(x)
    out = orc.moe_f64("iq1t", raw, E, N, K, xq, xs, ids)
    for t in range(T):
        for j in range(top_k):
            dense = orc.gemm_f64("iq1t", raw[ids[t, j]], N, K, xq[t:t + 1], xs[t:t + 1])[0]
            assert np.array_equal(out[t, j], dense)
    perm = np.random.default_rng(0).permutation(T)
    out_p = orc.moe_f64("iq1t", raw, E, N, K, xq[perm], xs[perm], ids[perm])
    assert np.array_equal(out_p, out[perm])
    pairs = [(0, 0), (3, 2), (9, 1)]
    assert np.array_equal(orc.moe_f64("iq1t", raw, E, N, K, xq, xs, ids, pairs=pairs),
                          np.stack([out[t, j] for t, j in pairs]))
