"""GPU parity of q6_K against the CPU oracle, through the C ABI.

q6_K values are a 6-bit grid moved to the signed domain by -32 with an int8 scale per 16
values; a 32-value block is two half-block integer sums with separate accumulators, each
rescaled by its own d*sc (minfer R1 sections 2.2 and 3.3). The checks:

* the repack's scale split: the two f16 halves of every packed scale dword add up to d*sc_h
  exactly (read back at the documented packed offsets);
* prefill: q8_1 bit-exact, the per-16 int32 partials (two per block) bit-exact, f32 within
  max|gpu - ref| / max|ref| <= 1e-3 of the f64 definition (minfer R1 section 4) and within the
  rounding bound of tests/parity.py of the per-block C oracle, on shapes with
  ragged M and N tails and both signs of sub-scale, plus worst-case blocks;
* small batches (M <= 16, and batches of 16 up to 128 rows: the decode kernel, two half-block
  MFMAs per block), MUL_MAT_ID
  (prefill gather and, for at most 10 tokens, the decode kernel), and the 7B
  ffn_down shape (M = 2048, N = 4096, K = 11008) on sampled rows and columns in the launch
  configuration the bench times.
"""
import numpy as np
import pytest

import gen
import parity

pytestmark = pytest.mark.gpu

GATE = 1e-3


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


def _run(env, raw, x, M, N, K, partials=True):
    torch, mmq, orc = env
    dev = torch.device("cuda:0")
    act = mmq.quantize_act(torch.from_numpy(x).to(dev), "q8_1")
    packed = mmq.repack_weights("q6_K", torch.from_numpy(np.ascontiguousarray(raw)).to(dev), N, K)
    out = mmq.gemm("q6_K", packed, act, M, N, K, "f32")
    parts = mmq.gemm("q6_K", packed, act, M, N, K, "i32_partials") if partials else None
    torch.cuda.synchronize()
    return act, packed, out.cpu().numpy(), None if parts is None else parts.cpu().numpy()


@pytest.mark.parametrize("N,K", [(32, 256), (45, 768)])
def test_repack_scale_split_is_exact(env, N, K):
    torch, mmq, _ = env
    raw = gen.weights_q6_K(N, K, seed=N, cfg=61)
    _, packed, _, _ = _run(env, raw, np.zeros((1, K), np.float32), 1, N, K, partials=False)
    buf = packed.cpu().numpy()
    Np, KB = (N + 31) // 32 * 32, K // 32
    KBp = (KB + 7) // 8 * 8
    scale_off = (Np // 32 * KBp * 1024 + 255) // 256 * 256
    min_off = scale_off + (Np * KBp * 4 + 255) // 256 * 256
    assert buf.size == min_off + (Np * KBp * 4 + 255) // 256 * 256 == mmq.packed_bytes("q6_K", N, K)
    b = raw.reshape(N, K // 256, 210)
    d = b[..., 208:210].copy().view(np.float16)[..., 0].astype(np.float64)          # [N, K/256]
    sc = b[..., 192:208].view(np.int8).astype(np.float64)
    for off, half in ((scale_off, 0), (min_off, 1)):
        words = buf[off:off + Np * KBp * 4].view(np.uint32).reshape(Np // 32, KBp, 32)
        words = words.transpose(0, 2, 1).reshape(Np, KBp)[:N, :KB]
        hi = (words & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
        lo = (words >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
        ds = np.repeat(d, 8, axis=1) * sc[..., half::2].reshape(N, KB)
        assert np.array_equal(hi + lo, ds)


SHAPES = [(1, 32, 256), (17, 33, 256), (40, 97, 768), (130, 300, 512), (256, 256, 1024), (33, 129, 2304)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_prefill(env, M, N, K):
    _, mmq, orc = env
    seed = 7 * M + N + K
    print(f"[case] q6_K M={M} N={N} K={K} seed={seed}", flush=True)
    raw = gen.weights_q6_K(N, K, seed=seed, cfg=62)
    x = gen.act_f32(M, K, seed=seed, cfg=62, outlier_rate=1e-2)
    act, _, out, parts = _run(env, raw, x, M, N, K)
    rq, rs, rsum = orc.quantize_q8_1(x)
    xq, xs, xsum = mmq.act_to_host(act.cpu().numpy(), M, K)
    assert np.array_equal(xq, rq) and np.array_equal(xsum, rsum)
    assert np.array_equal(parts, orc.partials16("q6_K", raw, N, K, rq))
    r1, r2 = parity.check_f32(orc, out, "q6_K", raw, N, K, rq, rs, rsum, what=(M, N, K))
    print(f"  rel err {r1:.3e} (definition), {r2:.3e} (C oracle)")


def test_extreme_blocks(env):
    # every value -32 (q = 0) with sc = -128 / 127 against xq = +-127: the largest half-block
    # dots (16 * 32 * 127) and scaled products the format allows
    M, N, K = 64, 64, 512
    raw = gen.weights_q6_K(N, K, seed=3, cfg=63).reshape(N, K // 256, 210).copy()
    raw[..., 0:192] = 0
    raw[0::2, :, 192:208] = np.uint8(0x80)        # sc = -128
    raw[1::2, :, 192:208] = np.uint8(0x7F)        # sc = 127
    raw = raw.reshape(N, -1)
    x = np.ones((M, K), np.float32)
    x[1::2] *= -1
    _, mmq, orc = env
    _, _, out, parts = _run(env, raw, x, M, N, K)
    rq, rs, rsum = orc.quantize_q8_1(x)
    P16 = orc.partials16("q6_K", raw, N, K, rq)
    assert np.abs(P16).max() == 16 * 32 * 127
    assert np.array_equal(parts, P16)
    parity.check_f32(orc, out, "q6_K", raw, N, K, rq, rs, rsum)


# small batches run the decode kernel: token rows staged in LDS (K up to 448 blocks for M <= 8,
# 128 for M > 8) or loaded per wave (longer K), every live-register count, ragged N
@pytest.mark.parametrize("M,K", [(1, 2304), (3, 2304), (8, 2304), (16, 2304), (2, 11008), (8, 11008),
                                 (13, 11008)])
def test_small_batches(env, M, K):
    _, _, orc = env
    N = 300
    print(f"[case] q6_K decode M={M} N={N} K={K}", flush=True)
    raw = gen.weights_q6_K(N, K, seed=M, cfg=64)
    x = gen.act_f32(M, K, seed=M, cfg=64)
    _, _, out, _ = _run(env, raw, x, M, N, K, partials=False)
    rq, rs, rsum = orc.quantize_q8_1(x)
    parity.check_f32(orc, out, "q6_K", raw, N, K, rq, rs, rsum, what=(M, K))


def test_small_batch_matches_prefill_tiles(env):
    # M = 16 (decode kernel) against M = 129 (prefill tiles; from 129 rows mmq_gemm leaves the
    # decode kernel's batches) on the same first 16 rows: both are the same per-half
    # contraction, so they agree to f32 rounding order
    torch, mmq, _ = env
    N, K = 200, 1024
    raw = gen.weights_q6_K(N, K, seed=5, cfg=66)
    x = gen.act_f32(129, K, seed=5, cfg=66)
    _, _, o129, _ = _run(env, raw, x, 129, N, K, partials=False)
    _, _, o16, _ = _run(env, raw, x[:16], 16, N, K, partials=False)
    assert _rel(o16, o129[:16].astype(np.float64)) <= 1e-5


def test_moe(env):
    torch, mmq, orc = env
    dev = torch.device("cuda:0")
    E, T, top_k, N, K = 8, 90, 3, 97, 512
    ids = gen.moe_ids(T, top_k, E, seed=9, cfg=65)
    raw = gen.moe_weights("q6_K", E, N, K, seed=9, cfg=65)
    x = gen.act_f32(T, K, seed=9, cfg=65, outlier_rate=1e-3)
    act = mmq.quantize_act(torch.from_numpy(x).to(dev), "q8_1")
    pb = mmq.packed_bytes("q6_K", N, K)
    packed = torch.empty(E * pb, dtype=torch.uint8, device=dev)
    for e in range(E):
        mmq.repack_weights("q6_K", torch.from_numpy(np.ascontiguousarray(raw[e])).to(dev), N, K,
                           out=packed[e * pb:(e + 1) * pb])
    out = mmq.gemm_id("q6_K", packed, E, act, torch.from_numpy(ids).to(dev), T, top_k, N, K)
    torch.cuda.synchronize()
    rq, rs, rsum = orc.quantize_q8_1(x)
    ref = orc.moe_f64("q6_K", raw.reshape(E * N, -1), E, N, K, rq, rs, ids)
    assert _rel(out.cpu().numpy(), ref) <= GATE
    parity.check_moe(orc, out.cpu().numpy(), "q6_K", raw, N, K, rq, rs, rsum, ids)


@pytest.mark.parametrize("T", [1, 4, 8, 10])
def test_moe_decode(env, T):
    # MUL_MAT_ID with at most 10 tokens runs the decode kernel per expert
    torch, mmq, orc = env
    dev = torch.device("cuda:0")
    E, top_k, N, K = 16, 8, 160, 1024
    print(f"[case] q6_K moe decode T={T}", flush=True)
    ids = gen.moe_ids(T, top_k, E, seed=T, cfg=67)
    raw = gen.moe_weights("q6_K", E, N, K, seed=T, cfg=67)
    x = gen.act_f32(T, K, seed=T, cfg=67)
    act = mmq.quantize_act(torch.from_numpy(x).to(dev), "q8_1")
    pb = mmq.packed_bytes("q6_K", N, K)
    packed = torch.empty(E * pb, dtype=torch.uint8, device=dev)
    for e in range(E):
        mmq.repack_weights("q6_K", torch.from_numpy(np.ascontiguousarray(raw[e])).to(dev), N, K,
                           out=packed[e * pb:(e + 1) * pb])
    out = mmq.gemm_id("q6_K", packed, E, act, torch.from_numpy(ids).to(dev), T, top_k, N, K)
    torch.cuda.synchronize()
    rq, rs, rsum = orc.quantize_q8_1(x)
    ref = orc.moe_f64("q6_K", raw.reshape(E * N, -1), E, N, K, rq, rs, ids)
    assert _rel(out.cpu().numpy(), ref) <= GATE
    parity.check_moe(orc, out.cpu().numpy(), "q6_K", raw, N, K, rq, rs, rsum, ids, what=T)


def test_ffn_down_full_size_sampled(env):
    c = gen.CONFIGS["q6_K_m2048_n4096_k11008"]
    M, N, K = c["M"], c["N"], c["K"]
    print(f"[case] q6_K_m2048_n4096_k11008 M={M} N={N} K={K}", flush=True)
    _, _, orc = env
    raw = gen.weights_q6_K(N, K, seed=0, cfg=c["cfg"])
    x = gen.act_f32(M, K, seed=0, cfg=c["cfg"], outlier_rate=c["outlier_rate"])
    _, _, out, _ = _run(env, raw, x, M, N, K, partials=False)
    r = np.random.default_rng(14)
    rows = np.sort(np.concatenate([r.choice(M, 16, replace=False), [0, M - 1]]))
    cols = np.sort(np.concatenate([r.choice(N, 256, replace=False), [0, N - 1]]))
    rq, rs, rsum = orc.quantize_q8_1(x[rows])
    r1, r2 = parity.check_f32(orc, out[np.ix_(rows, cols)], "q6_K", raw, N, K, rq, rs, rsum, cols=cols)
    print(f"  rel err {r1:.3e} (definition), {r2:.3e} (C oracle)")
