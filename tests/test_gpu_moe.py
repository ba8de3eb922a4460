"""GPU parity of MUL_MAT_ID (expert-routed MoE through the MMQ kernel, llama.cpp PR #304)
against the oracle's out[t, j, :] = dense(W_{ids[t,j]}, x[t]), through the C ABI.

Covers: uniform top-k routing with ragged N, an expert holding more tokens than one tile
unit (several units per expert), empty experts, ids outside [0, E) (those output rows must
stay untouched), every block format, repeated calls with one workspace (the device-side
grouping is rebuilt each call), and the IQ1T MoE workload (64 experts of 2048 x 4096, 512
tokens, top-8) on sampled pairs and columns in the launch configuration the bench times."""
import numpy as np
import pytest

import gen
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
    return torch, mmq, oracle


def _rel(got, ref):
    return float(np.max(np.abs(got.astype(np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-300))


def _moe(env, fmt, E, T, top_k, N, K, ids, seed, out=None, ws=None):
    torch, mmq, orc = env
    dev = torch.device("cuda:0")
    print(f"[case] moe {fmt} E={E} T={T} top_k={top_k} N={N} K={K} seed={seed}", flush=True)
    raw = gen.moe_weights(fmt, E, N, K, seed=seed, cfg=74)
    x = gen.act_f32(T, K, seed=seed, cfg=74, outlier_rate=1e-3)
    act = mmq.quantize_act(torch.from_numpy(x).to(dev), "q8_1")
    pb = mmq.packed_bytes(fmt, N, K)
    packed = torch.empty(E * pb, dtype=torch.uint8, device=dev)
    for e in range(E):
        mmq.repack_weights(fmt, torch.from_numpy(np.ascontiguousarray(raw[e])).to(dev), N, K,
                           out=packed[e * pb:(e + 1) * pb])
    if out is None:
        out = torch.full((T, top_k, N), float(SENTINEL), dtype=torch.float32, device=dev)
    ids_d = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(dev)
    mmq.gemm_id(fmt, packed, E, act, ids_d, T, top_k, N, K, out=out, workspace=ws)
    torch.cuda.synchronize()
    rq, rs, _ = orc.quantize_q8_1(x)
    return raw, rq, rs, out.cpu().numpy()


def _check_full(env, fmt, E, N, K, ids, raw, rq, rs, got):
    _, _, orc = env
    valid = (ids >= 0) & (ids < E)
    ref = orc.moe_f64(fmt, raw.reshape(E * N, -1), E, N, K, rq, rs, np.where(valid, ids, -1))
    assert np.all(got[~valid] == SENTINEL)
    if valid.any():
        rel = _rel(got[valid], ref[valid])
        r2 = parity.check_moe(orc, got, fmt, raw, N, K, rq, rs, parity.block_sums(rq), np.where(valid, ids, -1))
        print(f"  rel err {rel:.3e} (definition), {r2:.3e} (C oracle)")
        assert rel <= GATE


@pytest.mark.parametrize("fmt", ["iq1t", "q4_0", "q8_0", "q4_K"])
def test_moe_uniform_routing(env, fmt):
    E, T, top_k, N, K = 8, 37, 3, 97, 512
    ids = gen.moe_ids(T, top_k, E, seed=1, cfg=74)
    raw, rq, rs, got = _moe(env, fmt, E, T, top_k, N, K, ids, seed=1)
    _check_full(env, fmt, E, N, K, ids, raw, rq, rs, got)


def test_moe_hot_expert_empty_experts_and_invalid_ids(env):
    # 300 tokens: slot 0 always expert 2 (four 64-pair units and a tail), slot 1 spread over experts
    # 5..7, experts 0, 1, 3, 4 empty; a few ids out of range in both directions
    E, T, top_k, N, K = 8, 300, 2, 160, 256
    r = np.random.default_rng(7)
    ids = np.empty((T, top_k), np.int32)
    ids[:, 0] = 2
    ids[:, 1] = r.integers(5, 8, T)
    ids[3, 1] = -1
    ids[10, 0] = E
    ids[299, 1] = 1 << 30
    raw, rq, rs, got = _moe(env, "iq1t", E, T, top_k, N, K, ids, seed=2)
    _check_full(env, "iq1t", E, N, K, ids, raw, rq, rs, got)


def test_moe_all_ids_invalid_writes_nothing(env):
    E, T, top_k, N, K = 4, 9, 2, 64, 256
    ids = np.full((T, top_k), -3, np.int32)
    _, _, _, got = _moe(env, "q4_0", E, T, top_k, N, K, ids, seed=3)
    assert np.all(got == SENTINEL)


def test_moe_workspace_reuse_and_determinism(env):
    torch, mmq, _ = env
    E, T, top_k, N, K = 16, 200, 4, 128, 512
    ws = torch.empty(mmq.gemm_id_workspace_bytes(E, T, top_k), dtype=torch.uint8, device="cuda:0")
    ids1 = gen.moe_ids(T, top_k, E, seed=4, cfg=74)
    ids2 = gen.moe_ids(T, top_k, E, seed=5, cfg=74)
    raw, rq, rs, a = _moe(env, "iq1t", E, T, top_k, N, K, ids1, seed=4, ws=ws)
    _, _, _, b = _moe(env, "iq1t", E, T, top_k, N, K, ids2, seed=4, ws=ws)
    _, _, _, c = _moe(env, "iq1t", E, T, top_k, N, K, ids1, seed=4, ws=ws)
    assert np.array_equal(a.view(np.uint32), c.view(np.uint32))      # bitwise repeatable
    _check_full(env, "iq1t", E, N, K, ids2, raw, rq, rs, b)


@pytest.mark.parametrize("fmt", ["q4_0", "iq1t"])
def test_moe_unit_boundaries(env, fmt):
    # per-expert pair counts on both sides of the gather unit sizes (64-pair full units, tails
    # of at most 32): a tail of 1, 31, 32; one full unit of 33, 63, 64; a full unit plus a tail
    # (65, 96); two full units (97, 128); and an empty expert. top_k = 2, shuffled pairs
    counts = [0, 1, 31, 32, 33, 63, 64, 65, 96, 97, 128]
    E, top_k, N, K = len(counts), 2, 160, 256
    flat = np.repeat(np.arange(E, dtype=np.int32), counts)
    assert flat.size % top_k == 0
    np.random.default_rng(11).shuffle(flat)
    T = flat.size // top_k
    ids = flat.reshape(T, top_k)
    raw, rq, rs, got = _moe(env, fmt, E, T, top_k, N, K, ids, seed=11)
    _check_full(env, fmt, E, N, K, ids, raw, rq, rs, got)


def test_moe_matches_dense_per_expert(env):
    # each pair's row equals the dense MMQ of its token against its expert, bit for bit; 150
    # tokens keep the dense call on the tile kernel (up to 128 it takes the decode kernel, whose
    # split-K sums in another order)
    torch, mmq, _ = env
    E, T, top_k, N, K = 4, 150, 2, 96, 512
    ids = gen.moe_ids(T, top_k, E, seed=6, cfg=74)
    raw, _, _, got = _moe(env, "q4_K", E, T, top_k, N, K, ids, seed=6)
    dev = torch.device("cuda:0")
    x = gen.act_f32(T, K, seed=6, cfg=74, outlier_rate=1e-3)
    act = mmq.quantize_act(torch.from_numpy(x).to(dev), "q8_1")
    for e in range(E):
        packed = mmq.repack_weights("q4_K", torch.from_numpy(np.ascontiguousarray(raw[e])).to(dev), N, K)
        dense = mmq.gemm("q4_K", packed, act, T, N, K, "f32").cpu().numpy()
        tt, jj = np.nonzero(ids == e)
        assert np.array_equal(got[tt, jj].view(np.uint32), dense[tt].view(np.uint32))


def test_moe_full_size_sampled(env):
    torch, mmq, orc = env
    c = gen.CONFIGS["moe_iq1t_e64_t512_top8_n2048_k4096"]
    E, T, top_k, N, K = c["E"], c["M"], c["top_k"], c["N"], c["K"]
    print(f"[case] moe_iq1t_e64_t512_top8_n2048_k4096 E={E} T={T} top_k={top_k} N={N} K={K}", flush=True)
    dev = torch.device("cuda:0")
    raw = gen.moe_weights("iq1t", E, N, K, seed=0, cfg=c["cfg"])
    x = gen.act_f32(T, K, seed=0, cfg=c["cfg"])
    ids = gen.moe_ids(T, top_k, E, seed=0, cfg=c["cfg"])
    act = mmq.quantize_act(torch.from_numpy(x).to(dev), "q8_1")
    pb = mmq.packed_bytes("iq1t", N, K)
    packed = torch.empty(E * pb, dtype=torch.uint8, device=dev)
    for e in range(E):
        mmq.repack_weights("iq1t", torch.from_numpy(np.ascontiguousarray(raw[e])).to(dev), N, K,
                           out=packed[e * pb:(e + 1) * pb])
    out = mmq.gemm_id("iq1t", packed, E, act, torch.from_numpy(ids).to(dev), T, top_k, N, K)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    rq, rs, _ = orc.quantize_q8_1(x)
    r = np.random.default_rng(12)
    cols = np.sort(np.concatenate([r.choice(N, 192, replace=False), [0, N - 1]]))
    worst = 0.0
    experts = r.choice(E, 12, replace=False)
    for e in experts:
        tt, jj = np.nonzero(ids == e)
        ref = orc.gemm_f64("iq1t", raw[e], N, K, rq[tt], rs[tt], cols=cols)
        worst = max(worst, _rel(got[tt, jj][:, cols], ref))
    r2 = parity.check_moe(orc, got[:, :, cols], "iq1t", raw, N, K, rq, rs, parity.block_sums(rq), ids,
                          experts=experts, cols=cols)
    print(f"  rel err {worst:.3e} (definition), {r2:.3e} (C oracle)")
    assert worst <= GATE
