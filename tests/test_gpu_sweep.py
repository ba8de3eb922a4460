"""GPU parity over the shape sweep of llama.cpp PR #304's test-backend-ops loop (Design: every
quantised type at k in {256, 1024, 4096, 5376}, batch sizes from one token to several tiles,
and MUL_MAT_ID with many experts), through the C ABI, for every block format.

K = 5376 (168 blocks, 21 super-blocks) is the one K of that loop that is not a power of two:
its block count is not a multiple of the kernels' 4-block stage group times the split-K
chunking, so the last stage and the last decode chunk are partly padding. M = 1 and 9 run the
small-batch kernel, M = 67 the prefill tiles with a ragged token tail; N = 80 leaves a ragged
weight-row tail. The MoE cases use 128 experts, above the 64 of the bench workload: with
T*top_k = 512 pairs most experts hold a handful of pairs, so nearly every unit is a tail unit;
and a decode batch (T = 2) over the same 128 experts. Checks: int32 partials bit-exact against
the oracle (per 32-value block; q6_K per 16-value half), and both output bars of
tests/parity.py (the pages' 1e-3 and the rounding bound against the per-block C oracle)."""
import numpy as np
import pytest

import gen
import parity

pytestmark = pytest.mark.gpu

FMTS = ["q8_0", "q4_0", "q4_K", "q6_K", "iq1t", "iq1c", "iq1s"]
GRIDDED = ("iq1c", "iq1s")
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


def _grid(fmt):
    return gen.IQ1C_GRID if fmt in GRIDDED else None


def _pack(env, fmt, raw, N, K, out=None):
    torch, mmq, _, grid = env
    return mmq.repack_weights(fmt, torch.from_numpy(np.ascontiguousarray(raw)).to("cuda:0"), N, K,
                              grid=grid if fmt in GRIDDED else None, out=out)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("K", [256, 1024, 4096, 5376])
@pytest.mark.parametrize("M", [1, 9, 67])
def test_dense_sweep(env, fmt, K, M):
    torch, mmq, orc, _ = env
    dev = torch.device("cuda:0")
    N = 80
    seed = M + K + FMTS.index(fmt)
    print(f"[case] sweep {fmt} M={M} N={N} K={K} seed={seed}", flush=True)
    raw = gen.weights(fmt, N, K, seed=seed, cfg=140)
    x = gen.act_f32(M, K, seed=seed, cfg=140, outlier_rate=1e-2)
    act = mmq.quantize_act(torch.from_numpy(x).to(dev), "q8_1")
    packed = _pack(env, fmt, raw, N, K)
    out = mmq.gemm(fmt, packed, act, M, N, K, "f32")
    parts = mmq.gemm(fmt, packed, act, M, N, K, "i32_partials")
    torch.cuda.synchronize()
    rq, rs, rsum = orc.quantize_q8_1(x)
    xq, _, xsum = mmq.act_to_host(act.cpu().numpy(), M, K)
    assert np.array_equal(xq, rq) and np.array_equal(xsum, rsum)
    # q6_K: the two half-block dots of every block (its scale changes every 16 values)
    ref_parts = orc.partials16(fmt, raw, N, K, rq) if fmt == "q6_K" else orc.partials(fmt, raw, N, K, rq, grid=_grid(fmt))
    assert np.array_equal(parts.cpu().numpy(), ref_parts)
    r1, r2 = parity.check_f32(orc, out.cpu().numpy(), fmt, raw, N, K, rq, rs, rsum, grid=_grid(fmt),
                              what=(fmt, M, N, K))
    print(f"  rel err {r1:.3e} (definition), {r2:.3e} (C oracle)")


@pytest.mark.parametrize("fmt", ["q4_0", "q4_K", "iq1c"])
@pytest.mark.parametrize("T", [2, 64])
def test_moe_128_experts(env, fmt, T):
    torch, mmq, orc, _ = env
    dev = torch.device("cuda:0")
    E, top_k, N, K = 128, 8, 96, 1024
    seed = T + FMTS.index(fmt)
    print(f"[case] moe {fmt} E={E} T={T} top_k={top_k} N={N} K={K} seed={seed}", flush=True)
    raw = gen.moe_weights(fmt, E, N, K, seed=seed, cfg=141)
    x = gen.act_f32(T, K, seed=seed, cfg=141, outlier_rate=1e-3)
    ids = gen.moe_ids(T, top_k, E, seed=seed, cfg=141)
    act = mmq.quantize_act(torch.from_numpy(x).to(dev), "q8_1")
    pb = mmq.packed_bytes(fmt, N, K)
    packed = torch.empty(E * pb, dtype=torch.uint8, device=dev)
    for e in range(E):
        _pack(env, fmt, raw[e], N, K, out=packed[e * pb:(e + 1) * pb])
    out = torch.full((T, top_k, N), float(SENTINEL), dtype=torch.float32, device=dev)
    mmq.gemm_id(fmt, packed, E, act, torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to(dev),
                T, top_k, N, K, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    rq, rs, _ = orc.quantize_q8_1(x)
    ref = orc.moe_f64(fmt, raw.reshape(E * N, -1), E, N, K, rq, rs, ids, grid=_grid(fmt))
    rel = parity.rel(got, ref)
    r2 = parity.check_moe(orc, got, fmt, raw, N, K, rq, rs, parity.block_sums(rq), ids, grid=_grid(fmt))
    print(f"  rel err {rel:.3e} (definition), {r2:.3e} (C oracle)")
    assert rel <= parity.PAGES_GATE


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0", "q4_K", "q6_K", "iq1t", "iq1c"])
def test_moe_ragged_weight_units(env, fmt):
    """N = 300 spans two 256-row MUL_MAT_ID units (q8_0 and q6_K: three 128-row units) whose last
    one is mostly past the matrix: its clamped weight tiles, and for IQ1C the second d chunk of
    an eight-tile unit, must not leak into the stored rows. 300 tokens at top-2 of 8 experts
    give ~75 pairs per expert, so units of both kinds (64-pair full units and tails) occur."""
    torch, mmq, orc, _ = env
    dev = torch.device("cuda:0")
    E, T, top_k, N, K = 8, 300, 2, 300, 512
    seed = 7 + FMTS.index(fmt)
    print(f"[case] moe ragged {fmt} E={E} T={T} top_k={top_k} N={N} K={K} seed={seed}", flush=True)
    raw = gen.moe_weights(fmt, E, N, K, seed=seed, cfg=142)
    x = gen.act_f32(T, K, seed=seed, cfg=142, outlier_rate=1e-3)
    ids = gen.moe_ids(T, top_k, E, seed=seed, cfg=142)
    act = mmq.quantize_act(torch.from_numpy(x).to(dev), "q8_1")
    pb = mmq.packed_bytes(fmt, N, K)
    packed = torch.empty(E * pb, dtype=torch.uint8, device=dev)
    for e in range(E):
        _pack(env, fmt, raw[e], N, K, out=packed[e * pb:(e + 1) * pb])
    out = torch.full((T, top_k, N), float(SENTINEL), dtype=torch.float32, device=dev)
    mmq.gemm_id(fmt, packed, E, act, torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to(dev),
                T, top_k, N, K, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert not np.any(got == SENTINEL)
    rq, rs, _ = orc.quantize_q8_1(x)
    ref = orc.moe_f64(fmt, raw.reshape(E * N, -1), E, N, K, rq, rs, ids, grid=_grid(fmt))
    rel = parity.rel(got, ref)
    r2 = parity.check_moe(orc, got, fmt, raw, N, K, rq, rs, parity.block_sums(rq), ids, grid=_grid(fmt))
    print(f"  rel err {rel:.3e} (definition), {r2:.3e} (C oracle)")
    assert rel <= parity.PAGES_GATE


@pytest.mark.parametrize("fmt,E,T", [("q8_0", 3000, 200), ("iq1c", 3000, 200), ("iq1c", 4096, 3),
                                     ("q4_0", 65, 40), ("iq1t", 4096, 16)])
def test_moe_thousands_of_experts(env, fmt, E, T):
    """More experts than the routing workgroup has threads (3000: three experts per thread, the
    last thread's range ragged; most experts empty or with one pair, so nearly every unit is a
    tail), and the most experts the call accepts (4096) at a decode batch, where each decode
    workgroup ranks the pairs by expert itself (keys up to 4096 << 8). Past 64 experts a gather
    workgroup finds its unit's expert in two ballot rounds over the unit offsets (every st-th
    offset, then st of them): 65 experts is the smallest such case (st = 2), 4096 at 16 tokens
    the largest (st = 64) on the gather path."""
    torch, mmq, orc, _ = env
    dev = torch.device("cuda:0")
    top_k, N, K = 8, 64, 256
    seed = 40 + FMTS.index(fmt)
    print(f"[case] moe many experts {fmt} E={E} T={T} top_k={top_k} N={N} K={K} seed={seed}", flush=True)
    raw = gen.moe_weights(fmt, E, N, K, seed=seed, cfg=143)
    x = gen.act_f32(T, K, seed=seed, cfg=143)
    ids = gen.moe_ids(T, top_k, E, seed=seed, cfg=143)
    act = mmq.quantize_act(torch.from_numpy(x).to(dev), "q8_1")
    pb = mmq.packed_bytes(fmt, N, K)
    packed = torch.empty(E * pb, dtype=torch.uint8, device=dev)
    for e in range(E):
        _pack(env, fmt, raw[e], N, K, out=packed[e * pb:(e + 1) * pb])
    out = torch.full((T, top_k, N), float(SENTINEL), dtype=torch.float32, device=dev)
    mmq.gemm_id(fmt, packed, E, act, torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to(dev),
                T, top_k, N, K, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert not np.any(got == SENTINEL)
    rq, rs, _ = orc.quantize_q8_1(x)
    ref = orc.moe_f64(fmt, raw.reshape(E * N, -1), E, N, K, rq, rs, ids, grid=_grid(fmt))
    rel = parity.rel(got, ref)
    r2 = parity.check_moe(orc, got, fmt, raw, N, K, rq, rs, parity.block_sums(rq), ids, grid=_grid(fmt))
    print(f"  rel err {rel:.3e} (definition), {r2:.3e} (C oracle)")
    assert rel <= parity.PAGES_GATE
