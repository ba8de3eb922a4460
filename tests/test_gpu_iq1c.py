"""GPU parity of the IQ1_M and IQ1_S codebook forms (iq1c, iq1s) against the CPU oracle,
through the C ABI.

iq1c and iq1s rows carry an 11-bit grid index per 8 values (llama.cpp PR #304 description;
the grid is the self-generated gen.IQ1C_GRID, an input of the repack); iq1c has s per 16 and
the delta sign per 8 values, iq1s both per 32. The repack keeps the indices: one dword per
fragment lane (two indices and the lane's s and signs), d per (row, 4-block group) and the grid
itself, which the GEMMs look up in LDS. The checks are:

* the packed buffer equals, byte for byte, tests/packmodel.py's model of that layout;
* the same values written in the iq1t layout give bit-identical f32 outputs (both forms feed
  the same matrix-core fold), dense and decode;
* dense prefill: q8_1 bit-exact, the folded int32 block partials bit-exact, f32 within
  max|gpu - ref| / max|ref| <= 1e-3 of the f64 definition (minfer R1 section 4), on shapes
  with ragged M and N tails;
* decode batches (M <= 16, the small-batch kernel, and up to 128 rows as batches of 16) within the same gate;
* MUL_MAT_ID at small sizes (every output row) and at the 64-expert workload size on sampled
  pairs and columns in the launch configuration the bench times, plus a decode-size MoE.
"""
import numpy as np
import pytest

import gen
import packmodel
import parity

pytestmark = pytest.mark.gpu

GATE = 1e-3
SENTINEL = np.float32(-12345.0)


@pytest.fixture(scope="module")
def env():
    import torch
    import block_quantized_int8_amd as mmq
    import oracle
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mmq.lib()
    oracle.build()
    grid = torch.from_numpy(gen.IQ1C_GRID.view(np.int16)).to("cuda:0")
    return torch, mmq, oracle, grid


def _rel(got, ref):
    return float(np.max(np.abs(got.astype(np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-300))


def _as_iq1t(raw_c, N, K, grid):
    """The same g, s, delta and d in the iq1t byte layout (a re-layout of fields)."""
    b = raw_c.reshape(N, K // 256, 56)
    qh = np.stack([b[..., 32:48] & 0xF, b[..., 32:48] >> 4], axis=-1).reshape(N, K // 256, 32)
    idx = b[..., 0:32].astype(np.int64) | ((qh & 7).astype(np.int64) << 8)
    codes = np.stack([(grid[idx] >> (2 * j)) & 3 for j in range(8)], axis=-1).reshape(N, K // 256, 256)
    c4 = codes.astype(np.uint8).reshape(N, K // 256, 64, 4)
    t = np.empty((N, K // 256, 76), np.uint8)
    t[..., 0:64] = c4[..., 0] | (c4[..., 1] << 2) | (c4[..., 2] << 4) | (c4[..., 3] << 6)
    t[..., 64:70] = b[..., 48:54]
    t[..., 70:74] = np.packbits((qh >> 3).astype(np.uint8).reshape(N, K // 256, 4, 8), axis=-1,
                                bitorder="little")[..., 0]
    t[..., 74:76] = b[..., 54:56]
    return t.reshape(N, -1)


def _iq1s_as_iq1t(raw_s, N, K, grid):
    """iq1s fields in the iq1t layout: the block's s and delta sign repeated per half / group."""
    b = raw_s.reshape(N, K // 256, 50)
    qh = (b[..., 34:50:2].astype(np.int64) | (b[..., 35:50:2].astype(np.int64) << 8))
    hi = np.stack([(qh >> (3 * j)) & 7 for j in range(4)], axis=-1)
    idx = b[..., 2:34].astype(np.int64).reshape(N, K // 256, 8, 4) | (hi << 8)
    codes = np.stack([(grid[idx] >> (2 * j)) & 3 for j in range(8)], axis=-1).reshape(N, K // 256, 256)
    c4 = codes.astype(np.uint8).reshape(N, K // 256, 64, 4)
    t = np.empty((N, K // 256, 76), np.uint8)
    t[..., 0:64] = c4[..., 0] | (c4[..., 1] << 2) | (c4[..., 2] << 4) | (c4[..., 3] << 6)
    s16 = np.repeat((qh >> 12) & 7, 2, axis=-1).astype(np.uint64)
    word = np.zeros((N, K // 256), np.uint64)
    for h in range(16):
        word |= s16[..., h] << np.uint64(3 * h)
    for k in range(6):
        t[..., 64 + k] = ((word >> np.uint64(8 * k)) & np.uint64(0xFF)).astype(np.uint8)
    sg = np.repeat((qh >> 15) & 1, 4, axis=-1).astype(np.uint8).reshape(N, K // 256, 4, 8)
    t[..., 70:74] = np.packbits(sg, axis=-1, bitorder="little")[..., 0]
    t[..., 74:76] = b[..., 0:2]
    return t.reshape(N, -1)


AS_IQ1T = {"iq1c": _as_iq1t, "iq1s": _iq1s_as_iq1t}
FMTS = ["iq1c", "iq1s"]


def _pack(env, raw, N, K, fmt="iq1c"):
    torch, mmq, _, grid = env
    return mmq.repack_weights(fmt, torch.from_numpy(np.ascontiguousarray(raw)).to("cuda:0"), N, K,
                              grid=grid)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("N,K", [(32, 256), (33, 768), (300, 512), (64, 4096)])
def test_packed_matches_the_layout_model(env, fmt, N, K):
    torch, mmq, _, grid = env
    print(f"[case] {fmt} repack N={N} K={K}", flush=True)
    raw = gen.weights(fmt, N, K, seed=N + K, cfg=85)
    out = torch.full((mmq.packed_bytes(fmt, N, K),), 0xA5, dtype=torch.uint8, device="cuda:0")
    mmq.repack_weights(fmt, torch.from_numpy(np.ascontiguousarray(raw)).to("cuda:0"), N, K, grid=grid, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = packmodel.pack(fmt, raw, N, K, row_scale=gen.IQ1C_GRID, fill=0xA5)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (fmt, N, K, int(bad.size), int(bad[0]) if bad.size else None)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", [(130, 300, 512), (4, 97, 4096), (1, 33, 768)])
def test_same_values_as_iq1t_same_outputs(env, fmt, M, N, K):
    torch, mmq, _, _ = env
    dev = torch.device("cuda:0")
    print(f"[case] {fmt} vs iq1t M={M} N={N} K={K}", flush=True)
    raw = gen.weights(fmt, N, K, seed=M + N + K, cfg=89)
    x = gen.act_f32(M, K, seed=M + N, cfg=89, outlier_rate=1e-2)
    act = mmq.quantize_act(torch.from_numpy(x).to(dev), "q8_1")
    pc = _pack(env, raw, N, K, fmt)
    pt = mmq.repack_weights("iq1t", torch.from_numpy(AS_IQ1T[fmt](raw, N, K, gen.IQ1C_GRID)).to(dev), N, K)
    oc = mmq.gemm(fmt, pc, act, M, N, K, "f32")
    ot = mmq.gemm("iq1t", pt, act, M, N, K, "f32")
    torch.cuda.synchronize()
    assert np.array_equal(oc.cpu().numpy().view(np.uint32), ot.cpu().numpy().view(np.uint32))


SHAPES = [(1, 32, 256), (17, 33, 256), (65, 97, 768), (130, 300, 512), (256, 256, 1024)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_dense_prefill(env, fmt, M, N, K):
    torch, mmq, orc, _ = env
    dev = torch.device("cuda:0")
    seed = 5 * M + N + K
    print(f"[case] {fmt} M={M} N={N} K={K} seed={seed}", flush=True)
    raw = gen.weights(fmt, N, K, seed=seed, cfg=86)
    x = gen.act_f32(M, K, seed=seed, cfg=86, outlier_rate=1e-2)
    act = mmq.quantize_act(torch.from_numpy(x).to(dev), "q8_1")
    packed = _pack(env, raw, N, K, fmt)
    out = mmq.gemm(fmt, packed, act, M, N, K, "f32")
    parts = mmq.gemm(fmt, packed, act, M, N, K, "i32_partials")
    torch.cuda.synchronize()
    rq, rs, rsum = orc.quantize_q8_1(x)
    xq, xs, xsum = mmq.act_to_host(act.cpu().numpy(), M, K)
    assert np.array_equal(xq, rq) and np.array_equal(xsum, rsum)
    assert np.array_equal(parts.cpu().numpy(), orc.partials(fmt, raw, N, K, rq, grid=gen.IQ1C_GRID))
    r1, r2 = parity.check_f32(orc, out.cpu().numpy(), fmt, raw, N, K, rq, rs, rsum, grid=gen.IQ1C_GRID,
                              what=(fmt, M, N, K))
    print(f"  rel err {r1:.3e} (definition), {r2:.3e} (C oracle)")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 4, 8, 16])
def test_decode_batches(env, fmt, M):
    torch, mmq, orc, _ = env
    dev = torch.device("cuda:0")
    N, K = 300, 4096
    print(f"[case] {fmt} decode M={M} N={N} K={K}", flush=True)
    raw = gen.weights(fmt, N, K, seed=M, cfg=87)
    x = gen.act_f32(M, K, seed=M, cfg=87, outlier_rate=1e-2)
    act = mmq.quantize_act(torch.from_numpy(x).to(dev), "q8_1")
    out = mmq.gemm(fmt, _pack(env, raw, N, K, fmt), act, M, N, K, "f32")
    torch.cuda.synchronize()
    rq, rs, rsum = orc.quantize_q8_1(x)
    parity.check_f32(orc, out.cpu().numpy(), fmt, raw, N, K, rq, rs, rsum, grid=gen.IQ1C_GRID, what=(fmt, M))


def _moe(env, E, T, top_k, N, K, ids, seed, cfg=88, fmt="iq1c"):
    torch, mmq, orc, _ = env
    dev = torch.device("cuda:0")
    print(f"[case] moe {fmt} E={E} T={T} top_k={top_k} N={N} K={K} seed={seed}", flush=True)
    raw = gen.moe_weights(fmt, E, N, K, seed=seed, cfg=cfg)
    x = gen.act_f32(T, K, seed=seed, cfg=cfg, outlier_rate=1e-3)
    act = mmq.quantize_act(torch.from_numpy(x).to(dev), "q8_1")
    pb = mmq.packed_bytes(fmt, N, K)
    packed = torch.empty(E * pb, dtype=torch.uint8, device=dev)
    for e in range(E):
        packed[e * pb:(e + 1) * pb] = _pack(env, raw[e], N, K, fmt)
    out = torch.full((T, top_k, N), float(SENTINEL), dtype=torch.float32, device=dev)
    mmq.gemm_id(fmt, packed, E, act, torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to(dev),
                T, top_k, N, K, out=out)
    torch.cuda.synchronize()
    rq, rs, _ = orc.quantize_q8_1(x)
    return raw, rq, rs, out.cpu().numpy()


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("T", [2, 8, 9, 37, 150])
def test_moe_every_row(env, fmt, T):
    # up to 8 tokens the decode kernel (each workgroup groups the pairs itself), from 9 the
    # routing launch and the prefill gather
    _, _, orc, _ = env
    E, top_k, N, K = 8, 3, 97, 512
    ids = gen.moe_ids(T, top_k, E, seed=T, cfg=88)
    raw, rq, rs, got = _moe(env, E, T, top_k, N, K, ids, seed=T, fmt=fmt)
    ref = orc.moe_f64(fmt, raw.reshape(E * N, -1), E, N, K, rq, rs, ids, grid=gen.IQ1C_GRID)
    rel = _rel(got, ref)
    r2 = parity.check_moe(orc, got, fmt, raw, N, K, rq, rs, parity.block_sums(rq), ids, grid=gen.IQ1C_GRID)
    print(f"  rel err {rel:.3e} (definition), {r2:.3e} (C oracle)")
    assert rel <= GATE


@pytest.mark.parametrize("name", ["moe_iq1c_e64_t512_top8_n2048_k4096", "moe_iq1s_e64_t512_top8_n2048_k4096"])
def test_moe_full_size_sampled(env, name):
    _, _, orc, _ = env
    c = gen.CONFIGS[name]
    E, T, top_k, N, K = c["E"], c["M"], c["top_k"], c["N"], c["K"]
    ids = gen.moe_ids(T, top_k, E, seed=0, cfg=c["cfg"])
    raw, rq, rs, got = _moe(env, E, T, top_k, N, K, ids, seed=0, cfg=c["cfg"], fmt=c["fmt"])
    assert np.all(np.isfinite(got))
    r = np.random.default_rng(13)
    cols = np.sort(np.concatenate([r.choice(N, 192, replace=False), [0, N - 1]]))
    worst = 0.0
    experts = r.choice(E, 10, replace=False)
    for e in experts:
        tt, jj = np.nonzero(ids == e)
        ref = orc.gemm_f64(c["fmt"], raw[e], N, K, rq[tt], rs[tt], cols=cols, grid=gen.IQ1C_GRID)
        worst = max(worst, _rel(got[tt, jj][:, cols], ref))
    r2 = parity.check_moe(orc, got[:, :, cols], c["fmt"], raw, N, K, rq, rs, parity.block_sums(rq), ids,
                          grid=gen.IQ1C_GRID, experts=experts, cols=cols)
    print(f"  rel err {worst:.3e} (definition), {r2:.3e} (C oracle)")
    assert worst <= GATE
