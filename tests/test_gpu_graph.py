"""hipGraph capture and replay of the prefill and MUL_MAT_ID paths, through the C ABI.

The bench times every workload as graph replays, and a caller may capture the path (the pages'
W8A8 contract asks for a graph-safe pack and GEMM: metainfer "INT8 W8A8 GEMM - Prefill",
section 3.2). Each test captures quantise + GEMM (or the expert-routed GEMM with its device-side
grouping) once, then replays the graph several times with new input contents copied into the
captured buffers, with eager work and synchronisations between replays; every replay must equal
the eager launches bit for bit and pass the oracle gate.
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


def _capture(torch, fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                  # warm outside capture
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


@pytest.mark.parametrize("fmt,M,N,K", [("q4_0", 300, 384, 1024), ("q4_K", 96, 4096, 512), ("q6_K", 70, 256, 768)])
def test_prefill_graph_replay_with_changed_inputs(env, fmt, M, N, K):
    torch, mmq, orc = env
    dev = torch.device("cuda:0")
    print(f"[case] graph prefill {fmt} M={M} N={N} K={K}", flush=True)
    raw = gen.weights(fmt, N, K, seed=31, cfg=91)
    packed = mmq.repack_weights(fmt, torch.from_numpy(raw).to(dev), N, K)
    xbuf = torch.zeros((M, K), dtype=torch.float32, device=dev)
    act = torch.empty(mmq.act_bytes("q8_1", M, K), dtype=torch.uint8, device=dev)
    out = torch.empty((M, N), dtype=torch.float32, device=dev)

    def path():
        mmq.quantize_act(xbuf, out=act)
        mmq.gemm(fmt, packed, act, M, N, K, out=out)
    g = _capture(torch, path)
    for rep in range(3):
        x = gen.act_f32(M, K, seed=300 + rep, cfg=91, outlier_rate=1e-2)
        xbuf.copy_(torch.from_numpy(x))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = mmq.gemm(fmt, packed, mmq.quantize_act(torch.from_numpy(x).to(dev)), M, N, K)
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
        rq, rs, rsum = orc.quantize_q8_1(x)
        parity.check_f32(orc, out.cpu().numpy(), fmt, raw, N, K, rq, rs, rsum, what=(fmt, rep))


def test_w8a8_graph_replay_with_changed_inputs(env):
    torch, mmq, orc = env
    dev = torch.device("cuda:0")
    M, N, K = 200, 320, 1024
    w, sw = gen.i8_rows(N, K, seed=32, cfg=92, tensor=gen.T_WEIGHT)
    packed = mmq.repack_weights("i8_row", torch.from_numpy(w).to(dev), N, K, row_scale=torch.from_numpy(sw).to(dev))
    xbuf = torch.zeros((M, K), dtype=torch.float32, device=dev)
    act = torch.empty(mmq.act_bytes("i8_token", M, K), dtype=torch.uint8, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def path():
        mmq.quantize_act(xbuf, "i8_token", out=act)
        mmq.gemm("i8_row", packed, act, M, N, K, "bf16", out=out)
    g = _capture(torch, path)
    for rep in range(3):
        x = gen.act_f32(M, K, seed=400 + rep, cfg=92)
        xbuf.copy_(torch.from_numpy(x))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a, sa = orc.quantize_i8_token(x)
        ref = orc.gemm_w8a8(a, sa, w, sw)
        assert np.array_equal(out.cpu().view(torch.int16).numpy().view(np.uint16), ref), rep


def test_moe_graph_replay_with_changed_routing(env):
    # the device-side grouping runs inside the graph: new ids between replays regroup the pairs
    torch, mmq, orc = env
    dev = torch.device("cuda:0")
    E, T, top_k, N, K = 16, 120, 4, 160, 512
    raw = gen.moe_weights("iq1t", E, N, K, seed=33, cfg=93)
    pb = mmq.packed_bytes("iq1t", N, K)
    packed = torch.empty(E * pb, dtype=torch.uint8, device=dev)
    for e in range(E):
        mmq.repack_weights("iq1t", torch.from_numpy(np.ascontiguousarray(raw[e])).to(dev), N, K,
                           out=packed[e * pb:(e + 1) * pb])
    xbuf = torch.zeros((T, K), dtype=torch.float32, device=dev)
    ids_buf = torch.zeros((T, top_k), dtype=torch.int32, device=dev)
    act = torch.empty(mmq.act_bytes("q8_1", T, K), dtype=torch.uint8, device=dev)
    out = torch.empty((T, top_k, N), dtype=torch.float32, device=dev)
    ws = torch.empty(mmq.gemm_id_workspace_bytes(E, T, top_k), dtype=torch.uint8, device=dev)
    ids_buf.copy_(torch.from_numpy(gen.moe_ids(T, top_k, E, seed=0, cfg=93)))

    def path():
        mmq.quantize_act(xbuf, out=act)
        mmq.gemm_id("iq1t", packed, E, act, ids_buf, T, top_k, N, K, out=out, workspace=ws)
    g = _capture(torch, path)
    for rep in range(3):
        x = gen.act_f32(T, K, seed=500 + rep, cfg=93)
        ids = gen.moe_ids(T, top_k, E, seed=1 + rep, cfg=93)
        xbuf.copy_(torch.from_numpy(x))
        ids_buf.copy_(torch.from_numpy(ids))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = mmq.gemm_id("iq1t", packed, E, mmq.quantize_act(torch.from_numpy(x).to(dev)),
                            torch.from_numpy(ids).to(dev), T, top_k, N, K)
        torch.cuda.synchronize()
        assert torch.equal(out, eager), rep
        rq, rs, rsum = orc.quantize_q8_1(x)
        ref = orc.moe_f64("iq1t", raw.reshape(E * N, -1), E, N, K, rq, rs, ids)
        assert _rel(out.cpu().numpy(), ref) <= GATE
        parity.check_moe(orc, out.cpu().numpy(), "iq1t", raw.reshape(E, N, -1), N, K, rq, rs, rsum, ids, what=rep)
