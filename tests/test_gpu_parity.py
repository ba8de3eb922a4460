"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars (the pages' parity gate and its reading, see the oracle's header):
* q8_1 activations (xq, xs, xsum): bit-exact; padded rows / blocks are zero.
* int32 per-block partials: bit-exact.
* f32 outputs: max|gpu - ref| / max|ref| <= 1e-3 against the f64 definition
  (minfer R1 section 4: max diff < 1e-3; the integer dots are exact, so only the f32
  rescale order can differ), and the rounding bound of tests/parity.py against the
  per-block C oracle (per output, plus a 1e-5 normwise gate).
* W8A8: int32 accumulators and bf16 outputs bit-exact (metainfer section 3.1:
  mismatch 0, max_abs_error 0.0).
Shapes span several tiles with ragged M, N and K tails (llama.cpp PR #304 review: sizes
like 17, 33, 65, 97 reach every tile edge), plus the full workload sizes, checked on
sampled outputs in the exact launch configuration the bench times.
"""
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


def _run(env, fmt, M, N, K, seed, x=None, outlier=0.0):
    torch, mmq, orc = env
    dev = torch.device("cuda:0")
    raw = gen.weights(fmt, N, K, seed=seed, cfg=70)
    if x is None:
        x = gen.act_f32(M, K, seed=seed, cfg=70, outlier_rate=outlier)
    print(f"[case] {fmt} M={M} N={N} K={K} seed={seed}", flush=True)
    xd = torch.from_numpy(x).to(dev)
    act = mmq.quantize_act(xd, "q8_1")
    packed = mmq.repack_weights(fmt, torch.from_numpy(raw).to(dev), N, K)
    out = mmq.gemm(fmt, packed, act, M, N, K, "f32")
    torch.cuda.synchronize()
    return raw, x, act, packed, out


SHAPES = [(64, 256, 256), (1, 32, 32), (17, 33, 96), (65, 97, 256), (130, 300, 544), (33, 129, 1024),
          (97, 65, 4096), (256, 256, 512)]


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_block_formats_quantize_partials_output(env, fmt, M, N, K):
    torch, mmq, orc = env
    raw, x, act, packed, out = _run(env, fmt, M, N, K, seed=M + N + K, outlier=1e-2)
    host = act.cpu().numpy()
    xq, xs, xsum = mmq.act_to_host(host, M, K)
    rq, rs, rsum = orc.quantize_q8_1(x)
    assert np.array_equal(xq, rq)
    assert np.array_equal(xs.view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(xsum, rsum)
    # the 8-value group sums (region 3) are the integer sums of the oracle's q
    G = mmq.act_groups_host(host, M, K)[:M, :K // 32]
    assert np.array_equal(G, rq.reshape(M, K // 32, 4, 8).astype(np.int64).sum(axis=3))
    assert np.all(mmq.act_padding_host(host, M, K) == 0)
    lo, hi, xsx = mmq.act_derived_host(host, M, K)
    full_s = np.zeros(lo.shape, np.float32)
    full_s[:M, :K // 32] = rs
    full_x = np.zeros(lo.shape, np.float32)
    full_x[:M, :K // 32] = rs * rsum.astype(np.float32)
    assert np.array_equal(lo, full_s) and np.array_equal(hi, full_s)
    assert np.array_equal(xsx, full_x)
    parts = mmq.gemm(fmt, packed, act, M, N, K, "i32_partials")
    torch.cuda.synchronize()
    assert np.array_equal(parts.cpu().numpy(), orc.partials(fmt, raw, N, K, rq))
    r1, r2 = parity.check_f32(orc, out.cpu().numpy(), fmt, raw, N, K, rq, rs, rsum, what=(fmt, M, N, K))
    print(f"  rel err {r1:.3e} (definition), {r2:.3e} (C oracle)")


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_edge_activations(env, fmt):
    # zero rows, a single huge outlier, tiny magnitudes, exact ties, and an all-negative block
    torch, mmq, orc = env
    M, N, K = 40, 64, 256
    x = gen.act_f32(M, K, seed=3, cfg=71)
    x[0] = 0
    x[1, 7] = 3.0e4
    x[2] *= np.float32(1e-30)
    x[3, :32] = np.arange(32, dtype=np.float32) - 15.5 + 127 * 0  # ties after scaling
    x[3, 0] = 127.0
    x[4, 32:64] = -np.abs(x[4, 32:64])
    x[5] *= np.float32(1e-3)          # amax/127 below 2^-14: the f16 block scale is subnormal
    # blocks whose d = amax/127 is an f32 subnormal, with zeros among the values: 1/d overflows
    # for amax 1e-37 and 1e-39 (di is then the largest finite f32), not for 1e-36
    x[6] = 0
    x[6, :32] = gen.act_f32(1, 32, seed=4, cfg=71)[0] * np.float32(1e-37 / 3)
    x[6, 3] = 0
    x[6, 32 + 9], x[6, 64 + 1], x[6, 96 + 31] = 1e-36, -1e-39, 5e-38
    x[7, ::2] = 0
    x[7] *= np.float32(1e-36)
    raw, x, act, packed, out = _run(env, fmt, M, N, K, seed=5, x=x)
    xq, xs, xsum = mmq.act_to_host(act.cpu().numpy(), M, K)
    rq, rs, rsum = orc.quantize_q8_1(x)
    assert np.array_equal(xq, rq) and np.array_equal(xs.view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(xsum, rsum)
    got = out.cpu().numpy()
    assert np.all(got[0] == 0)
    # per-row gates (rows differ in magnitude by 1e30)
    parity.check_f32(orc, got, fmt, raw, N, K, rq, rs, rsum, what=fmt, per_row=True)


def test_ldo_wider_than_n_leaves_padding_untouched(env):
    torch, mmq, orc = env
    M, N, K, ldo = 33, 40, 128, 52
    raw = gen.weights("q4_0", N, K, seed=9, cfg=72)
    x = gen.act_f32(M, K, seed=9, cfg=72)
    dev = torch.device("cuda:0")
    act = mmq.quantize_act(torch.from_numpy(x).to(dev))
    packed = mmq.repack_weights("q4_0", torch.from_numpy(raw).to(dev), N, K)
    out = torch.full((M, ldo), 7.0, dtype=torch.float32, device=dev)
    mmq.gemm("q4_0", packed, act, M, N, K, "f32", out=out, ldo=ldo)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[:, N:] == 7.0)
    rq, rs, rsum = orc.quantize_q8_1(x)
    parity.check_f32(orc, o[:, :N], "q4_0", raw, N, K, rq, rs, rsum)


def test_deterministic_and_stream_ordered(env):
    torch, mmq, orc = env
    M, N, K = 200, 320, 1024
    raw, x, act, packed, out = _run(env, "q4_0", M, N, K, seed=11)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        act2 = mmq.quantize_act(torch.from_numpy(x).to("cuda"))
        out2 = mmq.gemm("q4_0", packed, act2, M, N, K)
    s.synchronize()
    assert torch.equal(out, out2)
    assert torch.equal(act, act2)


def test_graph_capture_replay_with_changed_contents(env):
    # metainfer section 3.1: graph capture and changed-contents replay must pass
    torch, mmq, orc = env
    M, N, K = 96, 128, 512
    dev = torch.device("cuda:0")
    raw = gen.weights("q8_0", N, K, seed=13, cfg=73)
    packed = mmq.repack_weights("q8_0", torch.from_numpy(raw).to(dev), N, K)
    xbuf = torch.zeros((M, K), dtype=torch.float32, device=dev)
    act = torch.empty(mmq.act_bytes("q8_1", M, K), dtype=torch.uint8, device=dev)
    out = torch.empty((M, N), dtype=torch.float32, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                    # warm up outside capture
        mmq.quantize_act(xbuf, out=act)
        mmq.gemm("q8_0", packed, act, M, N, K, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mmq.quantize_act(xbuf, out=act)
        mmq.gemm("q8_0", packed, act, M, N, K, out=out)
    for rep in range(3):
        x = gen.act_f32(M, K, seed=100 + rep, cfg=73)
        xbuf.copy_(torch.from_numpy(x))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = mmq.gemm("q8_0", packed, mmq.quantize_act(torch.from_numpy(x).to(dev)), M, N, K)
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
        rq, rs, rsum = orc.quantize_q8_1(x)
        parity.check_f32(orc, out.cpu().numpy(), "q8_0", raw, N, K, rq, rs, rsum, what=rep)


# ------------------------------------------------------------------ W8A8

def _w8a8_case(env, M, N, K, seed, sample_rows=None):
    torch, mmq, orc = env
    dev = torch.device("cuda:0")
    a, sa = gen.i8_rows(M, K, seed=seed, cfg=74, tensor=0)
    w, sw = gen.i8_rows(N, K, seed=seed, cfg=74, tensor=1)
    print(f"[case] w8a8 M={M} N={N} K={K}", flush=True)
    act = torch.from_numpy(mmq.act_i8_pack_host(a, sa)).to(dev)
    packed = mmq.repack_weights("i8_row", torch.from_numpy(w).to(dev), N, K, row_scale=torch.from_numpy(sw).to(dev))
    out = mmq.gemm("i8_row", packed, act, M, N, K, "bf16")
    acc = mmq.gemm("i8_row", packed, act, M, N, K, "i32_partials")
    torch.cuda.synchronize()
    rows = (0, M) if sample_rows is None else sample_rows
    ref_bf, ref_acc = orc.gemm_w8a8(a, sa, w, sw, rows=rows, want_acc=True)
    got_bf = out.view(torch.int16).cpu().numpy().view(np.uint16)[rows[0]:rows[1]]
    got_acc = acc.cpu().numpy()[rows[0]:rows[1]]
    assert np.array_equal(got_acc, ref_acc)
    assert np.array_equal(got_bf, ref_bf)


@pytest.mark.parametrize("M,N,K", [(1, 32, 32), (17, 33, 96), (65, 97, 256), (130, 260, 544), (300, 128, 4096)])
def test_w8a8_bit_exact(env, M, N, K):
    _w8a8_case(env, M, N, K, seed=M + N)


def test_w8a8_full_size_sampled(env):
    # the tensor-parallel share M=3072, K=4096, N=1536, in the bench's launch configuration
    _w8a8_case(env, 3072, 1536, 4096, seed=0, sample_rows=(3000, 3072))


# ------------------------------------------------------------------ full-size q4_0

@pytest.mark.parametrize("N", [4096, 11008])
def test_q4_0_full_size_sampled(env, N):
    torch, mmq, orc = env
    cfg = gen.CONFIGS["q4_0_m2048_n4096_k4096"]
    M, K = cfg["M"], cfg["K"]
    raw, x, act, packed, out = _run(env, "q4_0", M, N, K, seed=0, outlier=cfg["outlier_rate"])
    xq, xs, xsum = mmq.act_to_host(act.cpu().numpy(), M, K)
    rq, rs, rsum = orc.quantize_q8_1(x)
    assert np.array_equal(xq, rq) and np.array_equal(xs.view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(xsum, rsum)
    got = out.cpu().numpy()
    r = np.random.default_rng(N)
    rows = np.concatenate([[0, M - 1], r.choice(M, 62, replace=False)])
    cols = np.concatenate([[0, N - 1], r.choice(N, 62, replace=False)])
    parity.check_f32(orc, got[rows[:8]], "q4_0", raw, N, K, rq, rs, rsum, rows=rows[:8])   # 8 full rows
    parity.check_f32(orc, got[np.ix_(rows, cols)], "q4_0", raw, N, K, rq, rs, rsum, rows=rows,
                     cols=cols)                                                          # 64 x 64 sample


# ------------------------------------------------------------------ per-token quantiser

@pytest.mark.parametrize("M,K", [(1, 32), (5, 96), (37, 4096), (3, 14336)])
def test_quantize_i8_token_bit_exact(env, M, K):
    torch, mmq, orc = env
    x = gen.act_f32(M, K, seed=M, cfg=75, outlier_rate=1e-2)
    x[0, :] = 0 if M > 1 else x[0, :]
    print(f"[case] i8_token M={M} K={K}", flush=True)
    act = mmq.quantize_act(torch.from_numpy(x).to("cuda"), "i8_token")
    torch.cuda.synchronize()
    host = act.cpu().numpy()
    a, sa = mmq.act_i8_to_host(host, M, K)
    ra, rsa = orc.quantize_i8_token(x)
    assert np.array_equal(a, ra)
    assert np.array_equal(sa.view(np.uint32), rsa.view(np.uint32))
    full, sap = mmq.act_i8_to_host(host, M, K, padded=True)      # padding rows/blocks are zero
    assert not full[M:].any() and not full[:, K:].any() and not sap[M:].any()
