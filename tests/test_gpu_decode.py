"""GPU parity of the decode (small-batch) path against the CPU oracle, through the C ABI.

mmq_gemm sends batches of M <= 16 token rows (f32 out for the block formats, bf16 for W8A8)
to the split-K matrix-vector kernel, and up to 128 rows as batches of 16 while ceil(M/16) x
ceil(N/16) stays within 8 rounds of the compute units; more go to the prefill tiles. The bars are the
prefill ones: f32 outputs within max|gpu - ref| / max|ref| <= 1e-3 of the f64 definition
(minfer R1 section 4) and within the rounding bound of tests/parity.py of the per-block C
oracle, W8A8 bf16 outputs bit-exact (metainfer section 3.1). Cases cover every
live-register count (M = 1, 2, 3, 4 and M > 4), the largest batch (16), ragged N (a last
16-row group that is partly or wholly padding), K whose block count is not a multiple of the
kernel's 4-block chunk or of the 16 waves' share, ldo > N, and the full decode shapes the
bench times, on sampled outputs.
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


def _case(env, fmt, M, N, K, seed, ldo=None, cfg=80, outlier=1e-2):
    torch, mmq, orc = env
    dev = torch.device("cuda:0")
    print(f"[case] decode {fmt} M={M} N={N} K={K} ldo={ldo} seed={seed}", flush=True)
    raw = gen.weights(fmt, N, K, seed=seed, cfg=cfg)
    x = gen.act_f32(M, K, seed=seed, cfg=cfg, outlier_rate=outlier)
    act = mmq.quantize_act(torch.from_numpy(x).to(dev))
    packed = mmq.repack_weights(fmt, torch.from_numpy(raw).to(dev), N, K)
    L = ldo or N
    out = torch.full((M, L), 7.0, dtype=torch.float32, device=dev)
    mmq.gemm(fmt, packed, act, M, N, K, "f32", out=out, ldo=L)
    torch.cuda.synchronize()
    rq, rs, rsum = orc.quantize_q8_1(x)
    return raw, (rq, rs, rsum), out.cpu().numpy(), (packed, act, out)


# (N, K): K = 256 (8 blocks: two chunks, only two waves busy), 416 (13 blocks padded to 16),
# 768 (24 blocks), 4096 (128 blocks: one 8-block share per wave); N with a ragged last group
SMALL = [(32, 256), (48, 416), (33, 768), (300, 4096), (129, 1024)]
SUPER = [(32, 256), (33, 768), (300, 4096), (129, 1024)]


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 13, 16])
@pytest.mark.parametrize("fmt", ["q8_0", "q4_0", "q4_K", "iq1t"])
def test_decode_block_formats(env, fmt, M):
    torch, mmq, orc = env
    shapes = SMALL if fmt in ("q8_0", "q4_0") else SUPER
    for i, (N, K) in enumerate(shapes):
        raw, q, got, _ = _case(env, fmt, M, N, K, seed=100 * M + i)
        r1, r2 = parity.check_f32(orc, got, fmt, raw, N, K, *q, what=(fmt, M, N, K))
        print(f"  rel err {r1:.3e} (definition), {r2:.3e} (C oracle)", flush=True)


@pytest.mark.parametrize("fmt", ["q4_0", "q4_K"])
def test_decode_crossover_and_ldo(env, fmt):
    # M = 16 (one decode batch), 17 (two, the second with one token), 128 (eight, the most)
    # and 129 (the prefill tiles) on the same weights agree with the oracle; ldo > N leaves the
    # row padding untouched
    torch, mmq, orc = env
    N, K, ldo = 80, 512, 100
    for M in (16, 17, 128, 129):
        raw, q, got, _ = _case(env, fmt, M, N, K, seed=7, ldo=ldo)
        assert np.all(got[:, N:] == 7.0)
        parity.check_f32(orc, got[:, :N], fmt, raw, N, K, *q, what=M)


def test_decode_zero_and_padded_rows(env):
    # a zero activation row gives exact zeros; the other rows keep the gate per row
    torch, mmq, orc = env
    M, N, K = 6, 64, 1024
    dev = torch.device("cuda:0")
    raw = gen.weights("q4_0", N, K, seed=3, cfg=81)
    x = gen.act_f32(M, K, seed=3, cfg=81)
    x[2] = 0
    x[4] *= np.float32(1e-30)
    act = mmq.quantize_act(torch.from_numpy(x).to(dev))
    packed = mmq.repack_weights("q4_0", torch.from_numpy(raw).to(dev), N, K)
    out = mmq.gemm("q4_0", packed, act, M, N, K, "f32")
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    rq, rs, rsum = orc.quantize_q8_1(x)
    assert np.all(got[2] == 0)
    parity.check_f32(orc, got, "q4_0", raw, N, K, rq, rs, rsum, per_row=True)


def test_decode_deterministic(env):
    # the 16 waves' partial sums are added in a fixed order: repeated calls are bit-identical
    torch, mmq, orc = env
    raw, q, got, (packed, act, out) = _case(env, "q4_K", 9, 200, 4096, seed=11)
    for _ in range(3):
        again = mmq.gemm("q4_K", packed, act, 9, 200, 4096, "f32")
        torch.cuda.synchronize()
        assert np.array_equal(again.cpu().numpy(), got)


@pytest.mark.parametrize("M,N,K", [(1, 32, 32), (3, 33, 96), (8, 97, 256), (16, 130, 544), (5, 64, 4096)])
def test_decode_w8a8_bit_exact(env, M, N, K):
    torch, mmq, orc = env
    dev = torch.device("cuda:0")
    a, sa = gen.i8_rows(M, K, seed=M + N, cfg=82, tensor=0)
    w, sw = gen.i8_rows(N, K, seed=M + N, cfg=82, tensor=1)
    print(f"[case] decode w8a8 M={M} N={N} K={K}", flush=True)
    act = torch.from_numpy(mmq.act_i8_pack_host(a, sa)).to(dev)
    packed = mmq.repack_weights("i8_row", torch.from_numpy(w).to(dev), N, K,
                                row_scale=torch.from_numpy(sw).to(dev))
    out = mmq.gemm("i8_row", packed, act, M, N, K, "bf16")
    torch.cuda.synchronize()
    ref_bf, _ = orc.gemm_w8a8(a, sa, w, sw, rows=(0, M), want_acc=True)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, ref_bf)


@pytest.mark.parametrize("name", ["dec_q4_0_m1_n4096_k4096", "dec_q4_0_m8_n4096_k4096", "dec_q4_0_m16_n4096_k4096", "dec_q4_0_m8_n11008_k4096", "dec_q8_0_m8_n4096_k4096",
                                  "dec_q4_K_m8_n14336_k4096", "dec_q4_K_m8_n4096_k14336", "dec_iq1t_m8_n2048_k4096"])
def test_decode_full_size(env, name):
    # the decode workloads in the bench's launch configuration: every token row in full
    # against the f64 definition on 512 sampled weight rows (plus the first and last)
    torch, mmq, orc = env
    c = gen.CONFIGS[name]
    fmt, M, N, K = c["fmt"], c["M"], c["N"], c["K"]
    dev = torch.device("cuda:0")
    print(f"[case] {name}: {fmt} M={M} N={N} K={K}", flush=True)
    raw = gen.weights(fmt, N, K, seed=0, cfg=c["cfg"])
    x = gen.act_f32(M, K, seed=0, cfg=c["cfg"], outlier_rate=c.get("outlier_rate", 0.0))
    act = mmq.quantize_act(torch.from_numpy(x).to(dev))
    packed = mmq.repack_weights(fmt, torch.from_numpy(raw).to(dev), N, K)
    out = mmq.gemm(fmt, packed, act, M, N, K, "f32")
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    rq, rs, rsum = orc.quantize_q8_1(x)
    cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(N + M).choice(N, 512, replace=False)]))
    r1, r2 = parity.check_f32(orc, got[:, cols], fmt, raw, N, K, rq, rs, rsum, cols=cols, what=name)
    print(f"  rel err {r1:.3e} (definition), {r2:.3e} (C oracle)", flush=True)


def test_decode_w8a8_full_size(env):
    torch, mmq, orc = env
    c = gen.CONFIGS["dec_w8a8_m8_n1536_k4096"]
    M, N, K = c["M"], c["N"], c["K"]
    dev = torch.device("cuda:0")
    a, sa = gen.i8_rows(M, K, seed=0, cfg=c["cfg"], tensor=gen.T_ACT)
    w, sw = gen.i8_rows(N, K, seed=0, cfg=c["cfg"], tensor=gen.T_WEIGHT)
    print(f"[case] dec_w8a8_m8_n1536_k4096 M={M} N={N} K={K}", flush=True)
    act = torch.from_numpy(mmq.act_i8_pack_host(a, sa)).to(dev)
    packed = mmq.repack_weights("i8_row", torch.from_numpy(w).to(dev), N, K,
                                row_scale=torch.from_numpy(sw).to(dev))
    out = mmq.gemm("i8_row", packed, act, M, N, K, "bf16")
    torch.cuda.synchronize()
    ref_bf, _ = orc.gemm_w8a8(a, sa, w, sw, rows=(0, M), want_acc=True)
    assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), ref_bf)


@pytest.mark.parametrize("fmt,M,N,K", [("q4_0", 17, 4096, 4096), ("q4_K", 64, 4096, 4096),
                                        ("iq1t", 128, 2048, 4096), ("q8_0", 40, 300, 1024),
                                        ("q6_K", 33, 4096, 11008), ("iq1c", 97, 2048, 4096)])
def test_decode_batches_of_16(env, fmt, M, N, K):
    # 17..128 token rows as batches of 16 on the decode kernel (units = batches x 16-row groups;
    # each batch reads its own token tile and row offset): the last batch ragged (17, 33, 97),
    # whole (64, 128: the most batches) and a ragged N; every row in full against the f64
    # definition on sampled weight rows
    torch, mmq, orc = env
    dev = torch.device("cuda:0")
    seed = M + N
    print(f"[case] decode batches {fmt} M={M} N={N} K={K} seed={seed}", flush=True)
    gridded = fmt in ("iq1c", "iq1s")
    grid_np = gen.IQ1C_GRID if gridded else None
    raw = gen.weights(fmt, N, K, seed=seed, cfg=81)
    x = gen.act_f32(M, K, seed=seed, cfg=81, outlier_rate=1e-2)
    act = mmq.quantize_act(torch.from_numpy(x).to(dev))
    packed = mmq.repack_weights(fmt, torch.from_numpy(raw).to(dev), N, K,
                                grid=torch.from_numpy(grid_np.view(np.int16)).to(dev) if gridded else None)
    out = mmq.gemm(fmt, packed, act, M, N, K, "f32")
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    rq, rs, rsum = orc.quantize_q8_1(x)
    cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(seed).choice(N, min(N, 256), replace=False)]))
    r1, r2 = parity.check_f32(orc, got[:, cols], fmt, raw, N, K, rq, rs, rsum, cols=cols, grid=grid_np,
                              what=(fmt, M, N, K))
    print(f"  rel err {r1:.3e} (definition), {r2:.3e} (C oracle)", flush=True)


def test_decode_batches_admission_boundary(env):
    # 128 tokens are 8 batches: N = 16 x the CU count is the widest matrix the decode kernel
    # takes (8 units per CU); one more row sends the call to the prefill tiles. Both agree with
    # the oracle, every output checked
    torch, mmq, orc = env
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    K = 512
    for N in (16 * cus, 16 * cus + 1):
        raw, q, got, _ = _case(env, "q4_0", 128, N, K, seed=N)
        r1, r2 = parity.check_f32(orc, got, "q4_0", raw, N, K, *q, what=N)
        print(f"  N={N}: rel err {r1:.3e} (definition), {r2:.3e} (C oracle)", flush=True)


def test_decode_w8a8_batches_of_16(env):
    # W8A8 at 64 and 45 tokens on the decode kernel: bf16 outputs bit-exact
    torch, mmq, orc = env
    N, K = 1536, 4096
    dev = torch.device("cuda:0")
    for M in (64, 45):
        print(f"[case] w8a8 batches M={M} N={N} K={K}", flush=True)
        a, sa = gen.i8_rows(M, K, seed=M, cfg=82, tensor=gen.T_ACT)
        w, sw = gen.i8_rows(N, K, seed=M, cfg=82, tensor=gen.T_WEIGHT)
        act = torch.from_numpy(mmq.act_i8_pack_host(a, sa)).to(dev)
        packed = mmq.repack_weights("i8_row", torch.from_numpy(w).to(dev), N, K,
                                    row_scale=torch.from_numpy(sw).to(dev))
        out = mmq.gemm("i8_row", packed, act, M, N, K, "bf16")
        torch.cuda.synchronize()
        ref_bf, _ = orc.gemm_w8a8(a, sa, w, sw, rows=(0, M), want_acc=True)
        assert np.array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), ref_bf)


@pytest.mark.parametrize("fmt", ["q4_0", "q4_K", "iq1t", "q8_0"])
@pytest.mark.parametrize("M", [1, 7])
def test_decode_persistent_groups(env, fmt, M):
    # more 16-row groups than workgroups (N > 16 x compute units): workgroups loop over groups
    # with loads running ahead across group boundaries; K = 768 leaves most waves without a
    # chunk (they only reduce), K = 4352 gives waves unequal chunk counts (34 chunks, 16 waves).
    # A wave's item count (groups x chunks) is then 1, 2, 3, 4 or 6: the item loop runs zero to
    # two whole triples and leaves zero, one or two items after them
    torch, mmq, orc = env
    for K in (768, 4352):
        N = 16 * 256 + 53
        raw, q, got, _ = _case(env, fmt, M, N, K, seed=M + K)
        cols = np.unique(np.concatenate([np.arange(0, 64), np.arange(N - 80, N),
                                         np.random.default_rng(K).choice(N, 256, replace=False)]))
        r1, r2 = parity.check_f32(orc, got[:, cols], fmt, raw, N, K, *q, cols=cols, what=K)
        print(f"  K={K} rel err {r1:.3e} (definition), {r2:.3e} (C oracle)", flush=True)


@pytest.mark.parametrize("fmt,M", [("q4_0", 3), ("q4_K", 12)])
def test_decode_graph_capture_replay_with_changed_contents(env, fmt, M):
    # the decode launch captured with its quantiser in a hipGraph and replayed after the input
    # changed: every replay equals the eager result and passes the gate
    torch, mmq, orc = env
    N, K = 160, 1024
    dev = torch.device("cuda:0")
    raw = gen.weights(fmt, N, K, seed=17, cfg=83)
    packed = mmq.repack_weights(fmt, torch.from_numpy(raw).to(dev), N, K)
    xbuf = torch.zeros((M, K), dtype=torch.float32, device=dev)
    act = torch.empty(mmq.act_bytes("q8_1", M, K), dtype=torch.uint8, device=dev)
    out = torch.empty((M, N), dtype=torch.float32, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mmq.quantize_act(xbuf, out=act)
        mmq.gemm(fmt, packed, act, M, N, K, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mmq.quantize_act(xbuf, out=act)
        mmq.gemm(fmt, packed, act, M, N, K, out=out)
    for rep in range(3):
        x = gen.act_f32(M, K, seed=200 + rep, cfg=83)
        xbuf.copy_(torch.from_numpy(x))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = mmq.gemm(fmt, packed, mmq.quantize_act(torch.from_numpy(x).to(dev)), M, N, K)
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
        rq, rs, rsum = orc.quantize_q8_1(x)
        parity.check_f32(orc, out.cpu().numpy(), fmt, raw, N, K, rq, rs, rsum, what=rep)
