"""Pins for the oracle's scalar conversions and activation quantisers.

The q8_1 quantiser follows minfer "08 . R1 - int8 MMQ prefill GEMM", section 3.2
(the parity test's CPU reference) and section 2.2 (the block sum). Its pins:
hand-worked golden blocks (tests/golden/q8_1_blocks.json), closed forms, and
invariants that any correct quantiser satisfies. The f16 / bf16 rounding
helpers are pinned against NumPy's and PyTorch's own conversions.
"""
import json
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ scalars

def test_half_to_float_all_bit_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32)
    ref = bits.astype(np.uint16).view(np.float16).astype(np.float32)
    got = np.array([orc.half_to_float(int(b)) for b in bits], dtype=np.float32)
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite].view(np.uint32), ref[finite].view(np.uint32))
    assert np.all(np.isnan(got[np.isnan(ref)]))
    assert np.array_equal(got[np.isinf(ref)], ref[np.isinf(ref)])


def test_float_to_half_matches_numpy_rne():
    import oracle as orc
    r = np.random.default_rng(1)
    # random magnitudes across the whole f16 range, subnormals, exact ties and overflow edge
    x = np.concatenate([
        (r.standard_normal(20000) * np.exp(r.uniform(-20, 11, 20000))).astype(np.float32),
        np.float32(2.0) ** np.arange(-26, 16, dtype=np.float32),
        # exact midpoints between adjacent f16 values (ties): 1 + (2k+1)/2048
        (1 + (2 * np.arange(0, 1024, 37) + 1) / 2048).astype(np.float32),
        np.array([65504, 65519, 65520, 6.1e-5, 5.96e-8, 2.98e-8, 2.99e-8, 0.0, -0.0], np.float32),
    ])
    ref = x.astype(np.float16).view(np.uint16)
    got = np.array([orc.float_to_half_bits(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_float_to_bf16_matches_torch_rne():
    import torch
    import oracle as orc
    r = np.random.default_rng(2)
    x = np.concatenate([
        (r.standard_normal(20000) * np.exp(r.uniform(-30, 30, 20000))).astype(np.float32),
        # exact bf16 ties: low 16 bits == 0x8000, with even and odd kept lsb
        (np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x40490000 | 0x8000], np.uint32)).view(np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([orc.float_to_bf16_bits(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)


# ------------------------------------------------------------------ q8_1

def _golden_blocks():
    with open(os.path.join(GOLD, "q8_1_blocks.json")) as f:
        return json.load(f)["blocks"]


def test_q8_1_golden_blocks(orc):
    blocks = _golden_blocks()
    x = np.array([b["x"] for b in blocks], dtype=np.float32).reshape(1, -1)   # one row, 5 blocks
    xq, xs, xsum = orc.quantize_q8_1(x)
    for i, b in enumerate(blocks):
        assert xq[0, 32 * i:32 * (i + 1)].tolist() == b["q"], b["name"]
        assert float(xs[0, i]) == b["xs"], b["name"]
        assert int(xsum[0, i]) == b["xsum"], b["name"]


def test_q8_1_golden_blocks_as_rows(orc):
    # the same blocks laid out one per row: row layout must not matter
    blocks = _golden_blocks()
    x = np.array([b["x"] for b in blocks], dtype=np.float32)
    xq, xs, xsum = orc.quantize_q8_1(x)
    assert xq.tolist() == [b["q"] for b in blocks]
    assert xs[:, 0].tolist() == [b["xs"] for b in blocks]
    assert xsum[:, 0].tolist() == [b["xsum"] for b in blocks]


@pytest.mark.parametrize("val", [1e-3, 0.37, -2.5, 7.0, -123.456, 3.0e4])
@pytest.mark.parametrize("pos", [0, 13, 31])
def test_q8_1_single_nonzero_gives_full_scale(orc, val, pos):
    x = np.zeros((1, 64), np.float32)
    x[0, 32 + pos] = val
    xq, xs, xsum = orc.quantize_q8_1(x)
    expect = np.zeros(64, np.int8)
    expect[32 + pos] = 127 if val > 0 else -127
    assert np.array_equal(xq[0], expect)
    assert xs[0, 0] == 0 and xsum[0, 0] == 0
    assert xsum[0, 1] == expect[32 + pos]
    d = np.float32(abs(np.float32(val))) / np.float32(127)
    assert xs[0, 1] == np.float32(np.float16(d))


@pytest.mark.parametrize("dpow", [-6, -1, 0, 1, 3])
def test_q8_1_exact_multiples_of_power_of_two_scale(orc, dpow):
    # amax = 127 * 2^p makes d = 2^p and 1/d exact, so x = k*d quantises to exactly k
    r = np.random.default_rng(dpow + 10)
    k = r.integers(-127, 128, size=(8, 32)).astype(np.float32)
    k[:, 0] = 127
    x = k * np.float32(2.0 ** dpow)
    xq, xs, xsum = orc.quantize_q8_1(x.reshape(4, 64))
    assert np.array_equal(xq.reshape(8, 32), k.astype(np.int8))
    assert np.all(xs == np.float32(2.0 ** dpow))
    assert np.array_equal(xsum.reshape(8), k.sum(axis=1).astype(np.int32))


def test_q8_1_invariants_random(orc):
    r = np.random.default_rng(3)
    x = (r.standard_normal((37, 256)) * np.exp(r.uniform(-8, 8, (37, 1)))).astype(np.float32)
    x[5, 32:64] = 0
    xq, xs, xsum = orc.quantize_q8_1(x)
    M, K = x.shape
    xb = x.reshape(M, K // 32, 32).astype(np.float64)
    q = xq.reshape(M, K // 32, 32).astype(np.int64)
    assert np.array_equal(q.sum(axis=2), xsum)
    assert np.abs(q).max() <= 127
    amax = np.abs(xb).max(axis=2)
    # the element of largest magnitude always lands on +-127
    assert np.all(np.abs(q).max(axis=2)[amax > 0] == 127)
    # reconstruction with the unrounded f32 d is within half a step (plus the 1/d rounding)
    d = (amax / 127.0)[..., None]
    assert np.all(np.abs(xb - d * q) <= d * (0.5 + 1e-5) + 1e-30)
    # stored scale is d rounded to f16
    assert np.array_equal(xs, (amax / 127.0).astype(np.float32).astype(np.float16).astype(np.float32))
    assert np.all(q[5, 1] == 0) and xs[5, 1] == 0


def test_q8_1_is_blockwise_and_row_stride_free(orc):
    r = np.random.default_rng(4)
    x = r.standard_normal((6, 128)).astype(np.float32)
    a = orc.quantize_q8_1(x)
    # permuting whole 32-blocks permutes the outputs the same way
    perm = np.array([2, 0, 3, 1])
    xp = x.reshape(6, 4, 32)[:, perm].reshape(6, 128)
    b = orc.quantize_q8_1(xp)
    assert np.array_equal(b[0].reshape(6, 4, 32), a[0].reshape(6, 4, 32)[:, perm])
    assert np.array_equal(b[1], a[1][:, perm])
    assert np.array_equal(b[2], a[2][:, perm])


# ------------------------------------------------------------------ per-token int8

def test_i8_token_closed_forms(orc):
    x = np.zeros((3, 96), np.float32)
    x[0, :] = np.arange(96) - 40          # amax 55 at the end
    x[1, 7] = -254.0                      # d = 2, 1/d exact
    x[1, 8] = 5.0                         # 2.5 -> 2 (ties to even)
    x[1, 9] = 7.0                         # 3.5 -> 4
    a, sa = orc.quantize_i8_token(x)
    assert sa[2] == 0 and np.all(a[2] == 0)
    assert sa[1] == np.float32(2.0)
    assert a[1, 7] == -127 and a[1, 8] == 2 and a[1, 9] == 4
    assert sa[0] == np.float32(55) / np.float32(127)
    assert a[0, 95] == 127 and a[0, 40] == 0


def test_i8_token_scale_not_rounded_to_half(orc):
    x = np.full((1, 32), 0.3, np.float32)
    x[0, 0] = 1.0
    a, sa = orc.quantize_i8_token(x)
    assert sa[0] == np.float32(1.0) / np.float32(127)            # f32, not f16-rounded
    assert sa[0] != np.float32(np.float16(np.float32(1.0) / np.float32(127)))
    xq, xs, _ = orc.quantize_q8_1(x)
    assert xs[0, 0] == np.float32(np.float16(np.float32(1.0) / np.float32(127)))


def test_q8_1_tiny_blocks_closed_forms(orc):
    """Blocks whose amax is so small that d = amax/127 is subnormal, and 1/d may overflow f32.
    The pages leave that open; the reading taken (mmq.h) is di = FLT_MAX where 1/d overflows,
    so zeros stay 0 and no value leaves [-127, 127]. Hand-derived values:
      amax = 1e-37: d ~ 7.9e-40, 1/d overflows, 1e-37 * 3.4028235e38 = 34.03 -> 34;
      amax = 1e-36: d ~ 7.9e-39 (subnormal), 1/d ~ 1.27e38 is finite -> the peak maps to 127;
      amax = 1e-39: 1/d overflows, 1e-39 * 3.4028235e38 = 0.034 -> 0.
    In every case f16(d) = 0, so the stored scale is 0."""
    x = np.zeros((1, 128), np.float32)
    x[0, 0], x[0, 5] = 1e-37, -1e-37
    x[0, 32 + 9] = 1e-36
    x[0, 64 + 31] = -1e-39
    x[0, 96 + 3], x[0, 96 + 4] = 1e-37, 5e-38          # 5e-38 * FLT_MAX = 17.01 -> 17
    xq, xs, xsum = orc.quantize_q8_1(x)
    expect = np.zeros(128, np.int8)
    expect[0], expect[5] = 34, -34
    expect[32 + 9] = 127
    expect[96 + 3], expect[96 + 4] = 34, 17
    assert np.array_equal(xq[0], expect)
    assert np.all(xs == 0)
    assert xsum[0].tolist() == [0, 127, 0, 51]
