"""mmq_gemm_id_noalloc (the allocation-free MUL_MAT_ID for callers that cannot allocate:
graph capture, serving loops) against mmq_gemm_id with a caller workspace, through the C ABI.

Both run the same kernels, so the outputs must agree bit for bit: two calls in a row on the
shared static scratch, the second with a smaller problem (fewer experts, tokens and pairs), so
stale contents of the first call would show; then a decode-sized call (the small-batch path)
and the oracle's rounding bound on the last prefill-sized result."""
import numpy as np
import pytest

import gen
import parity

pytestmark = pytest.mark.gpu

SENTINEL = np.float32(-777.0)


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


def _problem(env, fmt, E, T, top_k, N, K, seed):
    torch, mmq, _ = env
    dev = torch.device("cuda:0")
    raw = gen.moe_weights(fmt, E, N, K, seed=seed, cfg=130)
    x = gen.act_f32(T, K, seed=seed, cfg=130, outlier_rate=1e-3)
    ids = gen.moe_ids(T, top_k, E, seed=seed, cfg=130)
    pb = mmq.packed_bytes(fmt, N, K)
    packed = torch.empty(E * pb, dtype=torch.uint8, device=dev)
    for e in range(E):
        mmq.repack_weights(fmt, torch.from_numpy(np.ascontiguousarray(raw[e])).to(dev), N, K,
                           out=packed[e * pb:(e + 1) * pb])
    act = mmq.quantize_act(torch.from_numpy(x).to(dev))
    return raw, x, ids, packed, act, torch.from_numpy(ids).to(dev)


def _both(env, fmt, E, T, top_k, N, K, seed):
    torch, mmq, _ = env
    print(f"[case] noalloc {fmt} E={E} T={T} top_k={top_k} N={N} K={K}", flush=True)
    raw, x, ids, packed, act, ids_d = _problem(env, fmt, E, T, top_k, N, K, seed)
    ref = torch.full((T, top_k, N), float(SENTINEL), dtype=torch.float32, device="cuda:0")
    got = torch.full((T, top_k, N), float(SENTINEL), dtype=torch.float32, device="cuda:0")
    mmq.gemm_id(fmt, packed, E, act, ids_d, T, top_k, N, K, out=ref)
    mmq.gemm_id_noalloc(fmt, packed, E, act, ids_d, T, top_k, N, K, out=got)
    torch.cuda.synchronize()
    g, r = got.cpu().numpy(), ref.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), r.view(np.uint32))
    return raw, x, ids, g


def test_noalloc_matches_the_workspace_entry_point(env):
    torch, mmq, orc = env
    assert mmq.gemm_id_noalloc_max_workspace_bytes() == 1 << 20
    _both(env, "iq1t", 64, 300, 8, 256, 512, seed=1)          # fills a large part of the scratch
    raw, x, ids, g = _both(env, "q4_0", 8, 37, 3, 97, 256, seed=2)   # smaller: stale entries would show
    rq, rs, rsum = orc.quantize_q8_1(x)
    parity.check_moe(orc, g, "q4_0", raw, 97, 256, rq, rs, rsum, ids)
    _both(env, "q4_K", 16, 3, 8, 160, 512, seed=3)            # decode batch: the small-batch kernel
