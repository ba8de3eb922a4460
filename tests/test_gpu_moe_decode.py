"""GPU parity of MUL_MAT_ID at decode batch sizes, through the C ABI.

With at most 10 tokens (and at most 256 (token, slot) pairs) mmq_gemm_id runs its expert
grouping and then the decode kernel over (batch of up to 8 of one expert's pairs, 16-row group)
units instead of the prefill gather tiles; past 8 tokens a workgroup stages 16 token rows, so K
is then at most 4096. 11 tokens, 257 pairs or 9 tokens at K > 4096 go back to the gather (both
sides of each crossover are checked). Bars: each pair's f32 row
within max|gpu - ref| / max|ref| <= 1e-3 of the f64 definition (minfer R1 section 4), rows of
invalid ids untouched, and each pair's row bit-identical to the dense decode product of its token
against its expert (the same per-block integer dots, scales and summation order).
"""
import numpy as np
import pytest

import gen
import parity

pytestmark = pytest.mark.gpu

GATE = 1e-3
SENTINEL = -12345.0


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


def _packed(env, fmt, raw, E, N, K):
    torch, mmq, _ = env
    dev = torch.device("cuda:0")
    pb = mmq.packed_bytes(fmt, N, K)
    packed = torch.empty(E * pb, dtype=torch.uint8, device=dev)
    for e in range(E):
        mmq.repack_weights(fmt, torch.from_numpy(np.ascontiguousarray(raw[e])).to(dev), N, K,
                           out=packed[e * pb:(e + 1) * pb])
    return packed


def _case(env, fmt, E, T, top_k, N, K, ids, seed, cfg=84):
    torch, mmq, orc = env
    dev = torch.device("cuda:0")
    print(f"[case] moe decode {fmt} E={E} T={T} top_k={top_k} N={N} K={K} seed={seed}", flush=True)
    raw = gen.moe_weights(fmt, E, N, K, seed=seed, cfg=cfg)
    x = gen.act_f32(T, K, seed=seed, cfg=cfg, outlier_rate=1e-2)
    act = mmq.quantize_act(torch.from_numpy(x).to(dev))
    packed = _packed(env, fmt, raw, E, N, K)
    out = torch.full((T, top_k, N), SENTINEL, dtype=torch.float32, device=dev)
    ids_d = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(dev)
    mmq.gemm_id(fmt, packed, E, act, ids_d, T, top_k, N, K, out=out)
    torch.cuda.synchronize()
    rq, rs, _ = orc.quantize_q8_1(x)
    return raw, rq, rs, act, packed, out.cpu().numpy()


def _check(env, fmt, E, N, K, ids, raw, rq, rs, got):
    _, _, orc = env
    valid = (ids >= 0) & (ids < E)
    ref = orc.moe_f64(fmt, raw.reshape(E * N, -1), E, N, K, rq, rs, np.where(valid, ids, -1))
    assert np.all(got[~valid] == SENTINEL)
    if valid.any():
        rel = _rel(got[valid], ref[valid])
        r2 = parity.check_moe(orc, got, fmt, raw, N, K, rq, rs, parity.block_sums(rq), np.where(valid, ids, -1))
        print(f"  rel err {rel:.3e} (definition), {r2:.3e} (C oracle)", flush=True)
        assert rel <= GATE


@pytest.mark.parametrize("T", [1, 2, 4, 5, 8, 9, 10, 11])
@pytest.mark.parametrize("fmt", ["q8_0", "q4_0", "q4_K", "iq1t"])
def test_moe_decode_formats(env, fmt, T):
    E, top_k, N, K = 32, 4, 160, 512
    ids = gen.moe_ids(T, top_k, E, seed=T, cfg=84)
    raw, rq, rs, _, _, got = _case(env, fmt, E, T, top_k, N, K, ids, seed=T)
    _check(env, fmt, E, N, K, ids, raw, rq, rs, got)


@pytest.mark.parametrize("T", [4, 10])
def test_moe_decode_matches_dense_decode_per_expert(env, T):
    # each pair's row equals the dense decode product of its token against its expert, bit for
    # bit (10 tokens: 16 staged token rows, tokens 8 and 9 read from the second group of 8)
    torch, mmq, _ = env
    E, top_k, N, K = 6, 3, 96, 1024
    ids = gen.moe_ids(T, top_k, E, seed=21, cfg=84)
    raw, _, _, act, packed, got = _case(env, "q4_K", E, T, top_k, N, K, ids, seed=21)
    dev = torch.device("cuda:0")
    for e in range(E):
        pe = mmq.repack_weights("q4_K", torch.from_numpy(np.ascontiguousarray(raw[e])).to(dev), N, K)
        dense = mmq.gemm("q4_K", pe, act, T, N, K, "f32").cpu().numpy()
        tt, jj = np.nonzero(ids == e)
        assert np.array_equal(got[tt, jj].view(np.uint32), dense[tt].view(np.uint32)), e


@pytest.mark.parametrize("K", [4096, 4128])
def test_moe_decode_16_rows_k_limit(env, K):
    # past 8 tokens the decode kernel stages 16 token rows, which fit up to K = 4096 (128 blocks);
    # one more block sends the call to the gather tiles. Both agree with the oracle
    E, T, top_k, N = 16, 9, 4, 96
    ids = gen.moe_ids(T, top_k, E, seed=K, cfg=84)
    raw, rq, rs, _, _, got = _case(env, "q4_0", E, T, top_k, N, K, ids, seed=K)
    _check(env, "q4_0", E, N, K, ids, raw, rq, rs, got)


def test_moe_decode_invalid_ids_and_shared_expert(env):
    # invalid ids leave their rows untouched; all tokens on one expert next to experts with one
    # pair
    T, top_k, E, N, K = 4, 3, 10, 64, 256
    ids = np.empty((T, top_k), np.int32)
    ids[:, 0] = 4                       # every token: expert 4
    ids[:, 1] = np.arange(T) % 9 + (np.arange(T) % 9 >= 4)     # spread over the others
    ids[:, 2] = -1
    ids[3, 2], ids[1, 1] = E, 123       # out of range
    raw, rq, rs, _, _, got = _case(env, "iq1t", E, T, top_k, N, K, ids, seed=22)
    _check(env, "iq1t", E, N, K, ids, raw, rq, rs, got)


@pytest.mark.parametrize("top_k", [64, 65])
def test_moe_decode_pair_limit_crossover(env, top_k):
    # 4 tokens x 64 slots = 256 pairs runs the decode kernel, 65 slots the prefill gather
    T, E, N, K = 4, 80, 96, 256
    ids = gen.moe_ids(T, top_k, E, seed=23, cfg=84)
    raw, rq, rs, _, _, got = _case(env, "q4_0", E, T, top_k, N, K, ids, seed=23)
    _check(env, "q4_0", E, N, K, ids, raw, rq, rs, got)


@pytest.mark.parametrize("T", [1, 4, 8, 10])
def test_moe_decode_full_shape_sampled(env, T):
    # the MoE workload's expert shape (64 experts x IQ1T 2048 x 4096, top-8) at decode batches
    # (10 tokens: 16 staged token rows); every pair row in full against the f64 definition on
    # 256 sampled columns
    torch, mmq, orc = env
    c = gen.CONFIGS["moe_iq1t_e64_t512_top8_n2048_k4096"]
    E, top_k, N, K = c["E"], c["top_k"], c["N"], c["K"]
    ids = gen.moe_ids(T, top_k, E, seed=T, cfg=c["cfg"])
    raw, rq, rs, _, _, got = _case(env, "iq1t", E, T, top_k, N, K, ids, seed=T, cfg=c["cfg"])
    cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(T).choice(N, 254, replace=False)]))
    for t in range(T):
        for j in range(top_k):
            e = ids[t, j]
            ref = orc.gemm_f64("iq1t", raw[e], N, K, rq[t:t + 1], rs[t:t + 1], cols=cols)
            assert _rel(got[t, j][cols][None, :], ref) <= GATE, (t, j)
    parity.check_moe(orc, got[:, :, cols], "iq1t", raw, N, K, rq, rs, parity.block_sums(rq), ids, cols=cols)


def test_moe_decode_repeated_expert_in_a_token(env):
    # ids need not be distinct within a token: expert 0 named by four slots of each of 3 tokens
    # holds 12 pairs, more than the 8 staged token rows of a 3-token batch (two batches);
    # experts 4-7 stay unused
    T, top_k, E, N, K = 3, 8, 8, 80, 512
    ids = np.tile(np.array([0, 0, 0, 0, 1, 1, 2, 3], np.int32), (T, 1))
    raw, rq, rs, _, _, got = _case(env, "q4_0", E, T, top_k, N, K, ids, seed=24)
    _check(env, "q4_0", E, N, K, ids, raw, rq, rs, got)
