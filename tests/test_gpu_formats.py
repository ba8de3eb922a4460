"""GPU parity of the Q4_K and IQ1T (IQ1_M-style ternary) paths against the CPU oracle,
through the C ABI: q8_1 activations bit-exact, int32 block partials bit-exact (Q4_K: the
unsigned-nibble dots; IQ1T: the folded sum_h (2s_h+1) * sum_16 xq*(8g+-1), llama.cpp PR #304),
f32 outputs within max|gpu - ref| / max|ref| <= 1e-3 of the f64 definition (minfer R1
section 4) and within the rounding bound of tests/parity.py of the per-block C oracle. Shapes have K a multiple of 256 (one super-block) with ragged M and N tails,
plus the Q4_K workload sizes (M = 512; K x N = 4096 x 14336 and 14336 x 4096) checked on
sampled rows and columns in the launch configuration the bench times."""
import numpy as np
import pytest

import gen
import parity

pytestmark = pytest.mark.gpu


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


SHAPES = [(1, 32, 256), (17, 33, 256), (64, 256, 512), (65, 97, 768), (130, 300, 512),
          (33, 129, 2048), (256, 256, 1024)]


@pytest.mark.parametrize("fmt", ["q4_K", "iq1t"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_super_block_formats(env, fmt, M, N, K):
    torch, mmq, orc = env
    dev = torch.device("cuda:0")
    seed = 3 * M + N + K
    print(f"[case] {fmt} M={M} N={N} K={K} seed={seed}", flush=True)
    raw = gen.weights(fmt, N, K, seed=seed, cfg=72)
    x = gen.act_f32(M, K, seed=seed, cfg=72, outlier_rate=1e-2)
    act = mmq.quantize_act(torch.from_numpy(x).to(dev), "q8_1")
    packed = mmq.repack_weights(fmt, torch.from_numpy(raw).to(dev), N, K)
    out = mmq.gemm(fmt, packed, act, M, N, K, "f32")
    parts = mmq.gemm(fmt, packed, act, M, N, K, "i32_partials")
    torch.cuda.synchronize()
    rq, rs, rsum = orc.quantize_q8_1(x)
    xq, xs, xsum = mmq.act_to_host(act.cpu().numpy(), M, K)
    assert np.array_equal(xq, rq) and np.array_equal(xsum, rsum)
    assert np.array_equal(xs.view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(parts.cpu().numpy(), orc.partials(fmt, raw, N, K, rq))
    r1, r2 = parity.check_f32(orc, out.cpu().numpy(), fmt, raw, N, K, rq, rs, rsum, what=(fmt, M, N, K))
    print(f"  rel err {r1:.3e} (definition), {r2:.3e} (C oracle)")


@pytest.mark.parametrize("fmt", ["q4_K", "iq1t"])
def test_extreme_weights(env, fmt):
    # the largest partials the formats allow: Q4_K nibbles all 15 with max scales and mins;
    # IQ1T all |g| = 1 with s = 7 against xq = +-127 (the folded bound 16*9*127 per 16)
    torch, mmq, orc = env
    dev = torch.device("cuda:0")
    M, N, K = 64, 64, 512
    raw = gen.weights(fmt, N, K, seed=5, cfg=73).copy()
    rb = raw.reshape(N, K // 256, -1)
    if fmt == "q4_K":
        rb[:, :, 4:16] = 0xFF                    # every 6-bit scale and min = 63
        rb[:, :, 16:144] = 0xFF                  # every nibble = 15
    else:
        rb[:, :, 0:64] = 0b10101010              # every code c = 2 -> g = +1
        rb[:, :, 64:70] = 0xFF                   # every sub-scale s = 7
        rb[:, 1::2, 70:74] = 0xFF                # odd super-blocks: every sign -1/8
    x = np.ones((M, K), np.float32)
    x[1::2] *= -1
    x[:, ::3] *= 0.5
    act = mmq.quantize_act(torch.from_numpy(x).to(dev), "q8_1")
    packed = mmq.repack_weights(fmt, torch.from_numpy(raw).to(dev), N, K)
    out = mmq.gemm(fmt, packed, act, M, N, K, "f32")
    parts = mmq.gemm(fmt, packed, act, M, N, K, "i32_partials")
    torch.cuda.synchronize()
    rq, rs, rsum = orc.quantize_q8_1(x)
    assert np.array_equal(parts.cpu().numpy(), orc.partials(fmt, raw, N, K, rq))
    parity.check_f32(orc, out.cpu().numpy(), fmt, raw, N, K, rq, rs, rsum, what=fmt)


@pytest.mark.parametrize("name", ["q4_K_m512_n14336_k4096", "q4_K_m512_n4096_k14336"])
def test_q4_K_full_size_sampled(env, name):
    torch, mmq, orc = env
    c = gen.CONFIGS[name]
    M, N, K = c["M"], c["N"], c["K"]
    print(f"[case] {name} M={M} N={N} K={K}", flush=True)
    dev = torch.device("cuda:0")
    raw = gen.weights("q4_K", N, K, seed=0, cfg=c["cfg"])
    x = gen.act_f32(M, K, seed=0, cfg=c["cfg"])
    act = mmq.quantize_act(torch.from_numpy(x).to(dev), "q8_1")
    packed = mmq.repack_weights("q4_K", torch.from_numpy(raw).to(dev), N, K)
    out = mmq.gemm("q4_K", packed, act, M, N, K, "f32")
    torch.cuda.synchronize()
    r = np.random.default_rng(11)
    rows = np.sort(np.concatenate([r.choice(M, 24, replace=False), [0, M - 1]]))
    cols = np.sort(np.concatenate([r.choice(N, 384, replace=False), [0, N - 1]]))
    rq, rs, rsum = orc.quantize_q8_1(x[rows])
    got = out.cpu().numpy()[np.ix_(rows, cols)]
    r1, r2 = parity.check_f32(orc, got, "q4_K", raw, N, K, rq, rs, rsum, cols=cols, what=name)
    print(f"  rel err {r1:.3e} (definition), {r2:.3e} (C oracle) on {len(rows)}x{len(cols)} samples")
    # the first rows through both oracles on every column
    xq, xs, xsum = orc.quantize_q8_1(x[:4])
    parity.check_f32(orc, out.cpu().numpy()[:4], "q4_K", raw, N, K, xq, xs, xsum, what=name)
