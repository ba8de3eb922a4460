"""GPU parity of the dense 128 x 128 configuration on ragged shapes, through the C ABI.

The library picks 128 weight rows x 128 token rows per workgroup once that gives about two
workgroups per CU (448 or more); smaller problems run 128 x 32. The other parity shapes are too
small to reach it, and the full-size workloads have no ragged tails. Here M = 1999 and N = 3937
(16 x 31 = 496 workgroups, neither a multiple of 32) exercise its masked token and weight tails
and several double-buffered stages. Outputs are checked against the f64 definition within
max|gpu - ref| / max|ref| <= 1e-3 (minfer R1 section 4) on every column of sampled rows (the last
row among them). The int32 block partials of the same configuration, the debug output, are
checked bit-exact against the per-block integer oracle.
"""
import numpy as np
import pytest

import gen
import parity

pytestmark = pytest.mark.gpu

GATE = 1e-3
M, N = 1999, 3937


@pytest.fixture(scope="module")
def env():
    import torch
    import block_quantized_int8_amd as mmq
    import oracle
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mmq.lib()
    oracle.build()
    return torch, mmq, oracle


def _rel(got, ref):
    return float(np.max(np.abs(got.astype(np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-300))


def _grid_is_128x128():
    return -(-N // 128) * -(-M // 128) >= 448


def _prepare(env, fmt, K, seed):
    torch, mmq, orc = env
    dev = torch.device("cuda:0")
    print(f"[case] large grid {fmt} M={M} N={N} K={K} seed={seed}", flush=True)
    raw = gen.weights(fmt, N, K, seed=seed, cfg=95)
    x = gen.act_f32(M, K, seed=seed, cfg=95, outlier_rate=1e-2)
    act = mmq.quantize_act(torch.from_numpy(x).to(dev), "q8_1")
    packed = mmq.repack_weights(fmt, torch.from_numpy(raw).to(dev), N, K)
    return raw, x, act, packed


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0", "q4_K", "iq1t"])
def test_dense_128x128_ragged_output(env, fmt):
    torch, mmq, orc = env
    assert _grid_is_128x128()
    K = 512
    raw, x, act, packed = _prepare(env, fmt, K, seed=41)
    out = mmq.gemm(fmt, packed, act, M, N, K, "f32")
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    r = np.random.default_rng(5)
    rows = np.sort(np.concatenate([[0, 127, 128, M - 33, M - 1], r.choice(M, 11, replace=False)]))
    rq, rs, rsum = orc.quantize_q8_1(x)
    r1, r2 = parity.check_f32(orc, got[rows], fmt, raw, N, K, rq, rs, rsum, rows=rows, what=fmt)
    print(f"  rel err {r1:.3e} (definition), {r2:.3e} (C oracle) on {len(rows)} full rows", flush=True)


@pytest.mark.parametrize("fmt", ["q4_0", "q4_K"])
def test_dense_128x128_ragged_partials(env, fmt):
    torch, mmq, orc = env
    assert _grid_is_128x128()
    K = 256
    raw, x, act, packed = _prepare(env, fmt, K, seed=43)
    parts = mmq.gemm(fmt, packed, act, M, N, K, "i32_partials")
    torch.cuda.synchronize()
    rq, _, _ = orc.quantize_q8_1(x)
    assert np.array_equal(parts.cpu().numpy(), orc.partials(fmt, raw, N, K, rq))
