"""A dense GEMM whose operand regions pass 2 GiB, so the library splits it into several launches
over weight-tile and token-tile ranges (the kernels address each region with 32-bit offsets).

q4_0, K = 2^23 (262144 blocks per row: one 32-row tile of fragments is 256 MiB of activation
values, so 7 such tiles fit below 2 GiB): M = 256 token rows (2 GiB of int8 values: the token
tiles are cut 7 + 1) against N = 160 weight rows (the weight tiles are cut 4 + 1 by the
128-row workgroups). The act buffer is written on the host in the documented q8_1 layout from
the oracle's quantisation (a 2 GiB region from an 8 GiB f32 input would not add anything to
this test). Checked: sampled rows on both sides of the token cut, against every weight row
(the C oracle's rounding bound) and on columns on both sides of the weight cut (the f64
definition)."""
import numpy as np
import pytest

import gen
import parity

pytestmark = pytest.mark.gpu

M, N, K = 256, 160, 1 << 23


def test_dense_gemm_past_the_2gib_split():
    import torch
    import block_quantized_int8_amd as mmq
    import oracle as orc
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"[case] split q4_0 M={M} N={N} K={K}", flush=True)
    # inputs in row chunks (seeded per chunk) to bound host memory
    raw = np.concatenate([gen.weights_q4_0(32, K, seed=i, cfg=128) for i in range(N // 32)])
    xq = np.empty((M, K), np.int8)
    xs = np.empty((M, K // 32), np.float32)
    xsum = np.empty((M, K // 32), np.int32)
    for i in range(M // 32):
        q = orc.quantize_q8_1(gen.act_f32(32, K, seed=i, cfg=129, outlier_rate=1e-3))
        xq[32 * i:32 * i + 32], xs[32 * i:32 * i + 32], xsum[32 * i:32 * i + 32] = q
    print("  inputs ready", flush=True)
    dev = torch.device("cuda:0")
    act = torch.from_numpy(mmq.act_q8_1_pack_host(xq, xs)).to(dev)
    packed = mmq.repack_weights("q4_0", torch.from_numpy(raw).to(dev), N, K)
    out = mmq.gemm("q4_0", packed, act, M, N, K, "f32")
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    print("  gemm done", flush=True)
    rows = np.array([0, 100, 223, 224, 255])          # token tiles 0-6 | 7
    cols = np.array([0, 31, 127, 128, 159])           # weight tiles 0-3 | 4
    r1, r2 = parity.check_f32(orc, got[np.ix_(rows, cols)], "q4_0", raw, N, K, xq, xs, xsum, rows=rows,
                              cols=cols, what="split")
    parity.check_tight(got[rows], orc.gemm_c("q4_0", raw, N, K, xq[rows], xs[rows], xsum[rows]),
                       orc.gemm_abs("q4_0", raw, N, K, xq[rows], xs[rows], xsum[rows]), K, "split rows")
    print(f"  rel err {r1:.3e} (definition), {r2:.3e} (C oracle)", flush=True)
