"""Byte-exact check of the GPU repack against tests/packmodel.py, a NumPy model of the
documented panel layout (metainfer "INT8 W8A8 GEMM - Prefill", section 3.2: packs are
validated by exact comparison with a simulation of the index map; a mis-vectorised transpose
there produced 16.8 M mismatches). Every byte of every region, padding rows and blocks
included, must match; the output buffer is prefilled so that bytes outside the regions show
whether the repack wrote there. Together with the model's CPU pins (test_packmodel.py) this
also fixes the q4_K and q6_K scale splits: each packed pair hi | lo is the f16 rounding of
d*sc and the f16 rounding of the remainder, and hi + lo == d*sc exactly."""
import numpy as np
import pytest

import gen
import packmodel

pytestmark = pytest.mark.gpu

SHAPES = [(32, 256), (45, 768), (70, 512), (129, 2048)]


@pytest.fixture(scope="module")
def env():
    import torch
    import block_quantized_int8_amd as mmq
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mmq.lib()
    return torch, mmq


def _gpu_pack(env, fmt, raw, N, K, row_scale=None):
    torch, mmq = env
    dev = torch.device("cuda:0")
    out = torch.full((mmq.packed_bytes(fmt, N, K),), 0xA5, dtype=torch.uint8, device=dev)
    rs = None if row_scale is None else torch.from_numpy(row_scale).to(dev)
    mmq.repack_weights(fmt, torch.from_numpy(np.ascontiguousarray(raw)).to(dev), N, K, row_scale=rs, out=out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0", "q4_K", "iq1t", "q6_K"])
@pytest.mark.parametrize("N,K", SHAPES)
def test_repack_matches_the_layout_model(env, fmt, N, K):
    print(f"[case] panels {fmt} N={N} K={K}", flush=True)
    raw = gen.weights(fmt, N, K, seed=3 * N + K, cfg=124)
    got = _gpu_pack(env, fmt, raw, N, K)
    want = packmodel.pack(fmt, raw, N, K, fill=0xA5)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (fmt, N, K, int(bad.size), int(bad[0]) if bad.size else None)


@pytest.mark.parametrize("N,K", [(40, 96), (33, 4096), (129, 544)])
def test_repack_i8_row_matches_the_layout_model(env, N, K):
    w, sw = gen.i8_rows(N, K, seed=N, cfg=125)
    got = _gpu_pack(env, "i8_row", w, N, K, row_scale=sw)
    want = packmodel.pack("i8_row", w, N, K, row_scale=sw, fill=0xA5)
    assert np.array_equal(got, want)


def test_repack_extreme_scales(env):
    # q4_K and q6_K scale products at the edges of the f16 split: the largest d*sc below
    # 65504, f16-subnormal d, and negative q6_K sub-scales
    N, K = 32, 512
    for fmt in ("q4_K", "q6_K"):
        raw = gen.weights(fmt, N, K, seed=9, cfg=126).reshape(N, K // 256, -1).copy()
        if fmt == "q4_K":
            raw[0::4, :, 0:2] = np.array([1000.0], np.float16).view(np.uint8)   # d*63 = 63000
            raw[1::4, :, 0:2] = np.array([3e-7], np.float16).view(np.uint8)     # subnormal d
            raw[2::4, :, 4:10] = 0xFF                                            # every sc = 63
        else:
            raw[0::4, :, 208:210] = np.array([500.0], np.float16).view(np.uint8)  # |d*sc| <= 64000
            raw[1::4, :, 208:210] = np.array([3e-7], np.float16).view(np.uint8)
            raw[2::4, :, 192:208] = np.uint8(0x80)                                # sc = -128
        raw = raw.reshape(N, -1)
        got = _gpu_pack(env, fmt, raw, N, K)
        assert np.array_equal(got, packmodel.pack(fmt, raw, N, K, fill=0xA5)), fmt
