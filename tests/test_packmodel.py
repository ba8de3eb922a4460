"""CPU pins of tests/packmodel.py, the NumPy model of the packed weight layout that the GPU
repack is compared with byte for byte: decoding the model's panels back gives exactly the
values and scales the oracle's own decoder reads from the raw rows, and the model's buffer
size is the library's mmq_packed_bytes."""
import numpy as np
import pytest

import gen
import packmodel

SHAPES = [(32, 256), (45, 768), (70, 512)]


def _f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0", "q4_K", "iq1t", "q6_K"])
@pytest.mark.parametrize("N,K", SHAPES)
def test_model_decodes_to_the_oracle(orc, fmt, N, K):
    raw = gen.weights(fmt, N, K, seed=N + K, cfg=122)
    buf = packmodel.pack(fmt, raw, N, K)
    vals = packmodel.unpack_values(fmt, buf, N, K)
    s1 = packmodel.scale_dwords(fmt, buf, N, K, 1)
    s2 = packmodel.scale_dwords(fmt, buf, N, K, 2) if fmt in ("q4_K", "q6_K") else None
    for n in range(N):
        wq, wd, wm, mult = orc.decode_row_c(fmt, raw[n], K)
        wd = wd.astype(np.float64)
        if fmt == "iq1t":
            meta = np.stack([(s1[n] >> 16) & 0xFF, (s1[n] >> 24) & 0xFF], axis=1).reshape(-1)   # per 16
            sig = np.stack([(meta >> 3) & 1, (meta >> 4) & 1], axis=1).reshape(-1)              # per 8
            v = 8 * (vals[n] - 1) + np.where(np.repeat(sig, 8) == 1, -1, 1)
            assert np.array_equal(v, wq), n
            d = _f16(s1[n] & 0xFFFF)
            assert np.array_equal(np.repeat(d, 2) * (2 * (meta & 7) + 1) / 8, wd), n
            assert np.array_equal(2 * (meta & 7) + 1, mult), n
            continue
        assert np.array_equal(vals[n], wq), n
        if fmt in ("q8_0", "q4_0"):
            assert np.all(s1[n] >> 16 == 0)
            assert np.array_equal(np.repeat(_f16(s1[n] & 0xFFFF), 2), wd), n
        elif fmt == "q4_K":
            hi, lo = _f16(s1[n] & 0xFFFF), _f16(s1[n] >> 16)
            assert np.array_equal(np.repeat(hi + lo, 2), wd), n        # hi + lo == d*sc exactly
            assert np.array_equal(s2[n].view(np.float32).astype(np.float64), wm), n
        else:                                                          # q6_K: per-16 halves
            for reg, h in ((s1, 0), (s2, 1)):
                assert np.array_equal(_f16(reg[n] & 0xFFFF) + _f16(reg[n] >> 16), wd[h::2]), (n, h)


@pytest.mark.parametrize("N,K", [(40, 96), (33, 4096)])
def test_model_i8_row(N, K):
    w, sw = gen.i8_rows(N, K, seed=N, cfg=123)
    buf = packmodel.pack("i8_row", w, N, K, row_scale=sw)
    assert np.array_equal(packmodel.unpack_values("i8_row", buf, N, K), w)
    so, _, _ = packmodel.offsets("i8_row", N, K)
    assert np.array_equal(buf[so:so + 4 * N].view(np.float32), sw)


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0", "q4_K", "iq1t", "q6_K", "i8_row"])
def test_model_size_is_the_library_size(fmt):
    import block_quantized_int8_amd as mmq
    for N, K in [(32, 256), (45, 768), (300, 4096)]:
        assert packmodel.offsets(fmt, N, K)[2] == mmq.packed_bytes(fmt, N, K), (N, K)


@pytest.mark.parametrize("fmt", ["iq1c", "iq1s"])
@pytest.mark.parametrize("N,K", [(32, 256), (45, 768), (70, 512)])
def test_model_grid_index_panels_decode_to_the_oracle(orc, fmt, N, K):
    """The grid-index panels: each lane dword names the grid entries of its two 8-value groups
    and carries the half's s and signs; with the spread grid of region 2 and d of region 1
    they give the oracle's values 8g +- 1, per-16 factors (2s+1) and scales d(2s+1)/8."""
    raw = gen.weights(fmt, N, K, seed=N + K, cfg=127)
    buf = packmodel.pack(fmt, raw, N, K, row_scale=gen.IQ1C_GRID)
    W, dbits = packmodel.gridded_words(fmt, buf, N, K)
    mo = packmodel.offsets(fmt, N, K)[1]
    gtab = np.asarray(buf[mo:mo + 8192]).copy().view(np.uint32)
    assert np.array_equal(gtab, packmodel.spread(gen.IQ1C_GRID))
    for n in range(N):
        wq, wd, wm, mult = orc.decode_row_c(fmt, raw[n], K, grid=gen.IQ1C_GRID)
        w = W[n].reshape(-1)                                   # per 16-value half
        ia, ib, meta = (w >> 2) & 0x7FF, (w >> 20) & 0x7FF, (w >> 13) & 0x1F
        assert np.all((w & 3) == 0) and np.all((w >> 18) & 3 == 0) and np.all(w >> 31 == 0)
        codes = np.stack([(gen.IQ1C_GRID[ia] >> (2 * j)) & 3 for j in range(8)] +
                         [(gen.IQ1C_GRID[ib] >> (2 * j)) & 3 for j in range(8)], axis=1).reshape(-1)
        sig = np.stack([(meta >> 3) & 1, (meta >> 4) & 1], axis=1).reshape(-1)
        assert np.array_equal(8 * (codes.astype(np.int64) - 1) + np.where(np.repeat(sig, 8) == 1, -1, 1), wq), n
        d = np.repeat(dbits[n].view(np.float16).astype(np.float64), 16)
        assert np.array_equal(d * (2 * (meta & 7) + 1) / 8, wd), n
