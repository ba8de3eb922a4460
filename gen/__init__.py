"""Seeded synthetic inputs for the MMQ path (shared by tests, bench and smoke).

This module only draws random numbers and lays the draws out in the raw
block formats' byte layouts. It holds none of the method's arithmetic: no
activation quantisation, no dot products, no per-block scale application.
Both the oracle and the HIP path consume what it returns; neither is imported
here.

Every tensor uses NumPy's PCG64 seeded with SeedSequence([seed, cfg, tensor]),
so each tensor of each configuration is an independent, reproducible stream.

Raw weight formats (little-endian; one row of a weight matrix is K/32 or
K/256 consecutive blocks):

* q8_0  - 34 B per 32 values: f16 d, then 32 int8 q.          w = d*q
* q4_0  - 18 B per 32 values: f16 d, then 16 bytes qs; value j is
          qs[j] & 0xF and value j+16 is qs[j] >> 4.           w = d*(nib-8)
* q4_K  - 144 B per 256 values: f16 d, f16 dmin, 12 bytes of 6-bit sub-block
          scales (bytes 0..5) and mins (bytes 6..11) packed LSB-first, then
          128 bytes qs; sub-block j uses qs[16j..16j+15], low nibble = value
          32j+i, high nibble = value 32j+16+i.       w = d*sc_j*nib - dmin*m_j
* iq1t  - 76 B per 256 values (an IQ1_M-style ternary format): 64 bytes of
          2-bit codes c = g+1 (4 per byte, LSB first), 6 bytes of 3-bit
          sub-scales s (one per 16 values, LSB-first bit stream), 4 bytes of
          sign bits (one per 8 values; 0 -> delta=+1/8, 1 -> delta=-1/8),
          then f16 d.                             w = d*(2s+1)*(g+delta)
* iq1c  - 56 B per 256 values (the IQ1_M codebook form, 1.75 bits per value):
          32 bytes qs (low 8 bits of each 8-value group's 11-bit grid index),
          16 bytes qh (byte j: groups 2j and 2j+1 in its low and high nibble;
          nibble bits 0-2 = index bits 8-10, bit 3 = that group's delta sign),
          6 bytes of 3-bit sub-scales s (one per 16 values, LSB-first), f16 d.
          The grid is a table of 2048 uint16 entries, each eight 2-bit codes
          c = g+1 (value j at bits 2j..2j+1).     w = d*(2s+1)*(g+delta)
* iq1s  - 50 B per 256 values (the IQ1_S codebook form, 1.5625 bits per value):
          f16 d, 32 bytes qs (low 8 bits of each 8-value group's 11-bit grid index),
          8 uint16 qh, one per 32 values: bits 3j..3j+2 = index bits 8-10 of the
          block's group j (j < 4), bits 12-14 = the block's sub-scale s, bit 15 =
          its delta sign. Same grid as iq1c.        w = d*(2s+1)*(g+delta)
* q6_K  - 210 B per 256 values: 128 bytes ql, 64 bytes qh, 16 int8 sub-scales
          sc (one per 16 values), f16 d. In 32-value block j, value 32j+i
          (i < 16) has its low 4 bits in the low nibble of ql[16j+i] and value
          32j+16+i in the high nibble; the high 2 bits of value 32j+8t+i
          (t < 4, i < 8) are bits 2t..2t+1 of qh[8j+i].  w = d*sc_h*(q-32)
* i8_row - int8 [N][K] plus one f32 scale per row.            w = sw[n]*q

The shapes and value distributions follow the five workloads the MMQ pages
are measured on (7B-like dense prefill in q8_0/q4_0/Q4_K, a per-channel W8A8
tensor-parallel share, and a 64-expert 1-bit MoE up projection).
"""
from __future__ import annotations

import numpy as np

QK = 32          # values per quantisation block
QK_SUPER = 256   # values per K-quant / iq1t super-block

ROW_BYTES_PER_BLOCK = {"q8_0": 34, "q4_0": 18, "q4_K": 144, "iq1t": 76, "iq1c": 56, "iq1s": 50, "q6_K": 210}
VALUES_PER_BLOCK = {"q8_0": 32, "q4_0": 32, "q4_K": 256, "iq1t": 256, "iq1c": 256, "iq1s": 256, "q6_K": 256}

# tensor ids inside a configuration's seed sequence
T_ACT, T_WEIGHT, T_IDS, T_OUTLIER, T_GRID = 0, 1, 2, 3, 4
GRID_SIZE = 2048        # iq1c codebook entries (11-bit index)
GRID_CFG = 90           # the codebook's own seed-sequence slot


def rng(seed: int, cfg: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg, tensor])))


def row_bytes(fmt: str, K: int) -> int:
    vpb = VALUES_PER_BLOCK[fmt]
    if K % vpb:
        raise ValueError(f"K={K} is not a multiple of {vpb} for {fmt}")
    return K // vpb * ROW_BYTES_PER_BLOCK[fmt]


def _f16_bits(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float16).view(np.uint16)


def act_f32(M: int, K: int, *, seed: int = 0, cfg: int = 0, outlier_rate: float = 0.0,
            outlier_scale: float = 20.0) -> np.ndarray:
    """Activations ~ N(0,1) in f32; optionally a Bernoulli(outlier_rate) mask scaled by outlier_scale."""
    x = rng(seed, cfg, T_ACT).standard_normal((M, K), dtype=np.float32)
    if outlier_rate > 0:
        mask = rng(seed, cfg, T_OUTLIER).random((M, K)) < outlier_rate
        x[mask] *= np.float32(outlier_scale)
    return x


def _normal_weights(N: int, K: int, seed: int, cfg: int, tensor: int, std: float) -> np.ndarray:
    return (rng(seed, cfg, tensor).standard_normal((N, K), dtype=np.float32) * np.float32(std))


def weights_q8_0(N: int, K: int, *, seed: int = 0, cfg: int = 0, tensor: int = T_WEIGHT,
                 std: float = 0.02) -> np.ndarray:
    """q8_0 rows from N(0,std): per block d = f16(max|w|/127), q = clip(rint(w/d), -127, 127)."""
    w = _normal_weights(N, K, seed, cfg, tensor, std).reshape(N, K // QK, QK)
    amax = np.abs(w).max(axis=2)
    d16 = (amax / np.float32(127)).astype(np.float16)
    d = d16.astype(np.float32)[..., None]
    q = np.where(d > 0, np.clip(np.rint(w / np.where(d > 0, d, 1)), -127, 127), 0).astype(np.int8)
    out = np.empty((N, K // QK, 34), dtype=np.uint8)
    out[..., 0:2] = d16.view(np.uint8).reshape(N, K // QK, 2)
    out[..., 2:34] = q.view(np.uint8)
    return out.reshape(N, -1)


def weights_q4_0(N: int, K: int, *, seed: int = 0, cfg: int = 0, tensor: int = T_WEIGHT,
                 std: float = 0.02) -> np.ndarray:
    """q4_0 rows from N(0,std): d = f16(w_peak / -8) where w_peak is the first value of largest
    magnitude (sign kept); nib = clip(rint(w/d) + 8, 0, 15)."""
    w = _normal_weights(N, K, seed, cfg, tensor, std).reshape(N, K // QK, QK)
    idx = np.abs(w).argmax(axis=2)
    peak = np.take_along_axis(w, idx[..., None], axis=2)[..., 0]
    d16 = (peak / np.float32(-8)).astype(np.float16)
    d = d16.astype(np.float32)[..., None]
    nib = np.where(d != 0, np.clip(np.rint(w / np.where(d != 0, d, 1)) + 8, 0, 15), 8).astype(np.uint8)
    out = np.empty((N, K // QK, 18), dtype=np.uint8)
    out[..., 0:2] = d16.view(np.uint8).reshape(N, K // QK, 2)
    out[..., 2:18] = nib[..., :16] | (nib[..., 16:] << 4)
    return out.reshape(N, -1)


def _pack6(v: np.ndarray) -> np.ndarray:
    """Pack 8 six-bit values per row (last axis) LSB-first into 6 bytes."""
    v = v.astype(np.uint64)
    word = np.zeros(v.shape[:-1], dtype=np.uint64)
    for j in range(8):
        word |= v[..., j] << np.uint64(6 * j)
    return np.stack([(word >> np.uint64(8 * b)) & np.uint64(0xFF) for b in range(6)], axis=-1).astype(np.uint8)


def weights_q4_K(N: int, K: int, *, seed: int = 0, cfg: int = 0, tensor: int = T_WEIGHT,
                 std: float = 0.02) -> np.ndarray:
    """Q4_K-style super-blocks from N(0,std): per 32-sub-block min/max give a step sc_f and an
    offset m_f; d = f16(max sc_f / 63), dmin = f16(max m_f / 63); sc, m are 6-bit; nibbles
    nib = clip(rint((w + dmin*m) / (d*sc)), 0, 15)."""
    nsb = K // QK_SUPER
    w = _normal_weights(N, K, seed, cfg, tensor, std).reshape(N, nsb, 8, QK)
    wmin = w.min(axis=3)
    wmax = w.max(axis=3)
    m_f = np.maximum(-wmin, 0)
    sc_f = (wmax + m_f) / np.float32(15)
    d16 = (sc_f.max(axis=2) / np.float32(63)).astype(np.float16)
    dm16 = (m_f.max(axis=2) / np.float32(63)).astype(np.float16)
    d = d16.astype(np.float32)[..., None]
    dm = dm16.astype(np.float32)[..., None]
    sc = np.where(d > 0, np.clip(np.rint(sc_f / np.where(d > 0, d, 1)), 0, 63), 0).astype(np.uint8)
    mm = np.where(dm > 0, np.clip(np.rint(m_f / np.where(dm > 0, dm, 1)), 0, 63), 0).astype(np.uint8)
    step = (d * sc.astype(np.float32))[..., None]
    off = (dm * mm.astype(np.float32))[..., None]
    nib = np.where(step > 0, np.clip(np.rint((w + off) / np.where(step > 0, step, 1)), 0, 15), 0)
    nib = nib.astype(np.uint8)
    out = np.empty((N, nsb, 144), dtype=np.uint8)
    out[..., 0:2] = d16.view(np.uint8).reshape(N, nsb, 2)
    out[..., 2:4] = dm16.view(np.uint8).reshape(N, nsb, 2)
    out[..., 4:10] = _pack6(sc)
    out[..., 10:16] = _pack6(mm)
    qs = nib[..., :16] | (nib[..., 16:] << 4)          # [N, nsb, 8, 16]
    out[..., 16:144] = qs.reshape(N, nsb, 128)
    return out.reshape(N, -1)


def pack_q6_K(q: np.ndarray, sc: np.ndarray, d16: np.ndarray) -> np.ndarray:
    """Lay out 6-bit values q [N, nsb, 256] (0..63), int8 sub-scales sc [N, nsb, 16] and f16 d
    [N, nsb] in the q6_K byte layout described above."""
    N, nsb = q.shape[:2]
    q = q.astype(np.uint8).reshape(N, nsb, 8, 32)
    out = np.empty((N, nsb, 210), dtype=np.uint8)
    lo = q & 0xF
    out[..., 0:128] = (lo[..., :16] | (lo[..., 16:] << 4)).reshape(N, nsb, 128)
    hi = (q >> 4).reshape(N, nsb, 8, 4, 8)                       # [.., j, t, i]
    out[..., 128:192] = (hi[..., 0, :] | (hi[..., 1, :] << 2) | (hi[..., 2, :] << 4) |
                         (hi[..., 3, :] << 6)).reshape(N, nsb, 64)
    out[..., 192:208] = sc.astype(np.int8).view(np.uint8)
    out[..., 208:210] = np.asarray(d16, np.float16).view(np.uint8).reshape(N, nsb, 2)
    return out.reshape(N, -1)


def weights_q6_K(N: int, K: int, *, seed: int = 0, cfg: int = 0, tensor: int = T_WEIGHT,
                 std: float = 0.02) -> np.ndarray:
    """q6_K-style super-blocks from N(0,std): per 16 values a signed step sf = w_peak / -32
    (w_peak: the first value of largest magnitude, sign kept); d = f16(max|sf| / 127);
    sc = clip(rint(sf / d), -127, 127); q = clip(rint(w / (d*sc)) + 32, 0, 63)."""
    nsb = K // QK_SUPER
    w = _normal_weights(N, K, seed, cfg, tensor, std).reshape(N, nsb, 16, 16)
    idx = np.abs(w).argmax(axis=3)
    peak = np.take_along_axis(w, idx[..., None], axis=3)[..., 0]
    sf = peak / np.float32(-32)
    d16 = (np.abs(sf).max(axis=2) / np.float32(127)).astype(np.float16)
    d = d16.astype(np.float32)[..., None]
    sc = np.where(d > 0, np.clip(np.rint(sf / np.where(d > 0, d, 1)), -127, 127), 0).astype(np.int8)
    step = (d * sc.astype(np.float32))[..., None]
    q = np.where(step != 0, np.clip(np.rint(w / np.where(step != 0, step, 1)) + 32, 0, 63), 32)
    return pack_q6_K(q.reshape(N, nsb, 256), sc, d16)


def weights_iq1t(N: int, K: int, *, seed: int = 0, cfg: int = 0, tensor: int = T_WEIGHT,
                 d_value: float = 0.02 / 4) -> np.ndarray:
    """IQ1_M-style ternary rows: g uniform in {-1,0,1}, s uniform in 0..7 per 16 values,
    delta sign uniform per 8 values, d = f16(d_value) for every super-block."""
    nsb = K // QK_SUPER
    r = rng(seed, cfg, tensor)
    out = np.empty((N, nsb, 76), dtype=np.uint8)
    code = r.integers(0, 3, size=(N, nsb, 256), dtype=np.uint8)          # c = g + 1
    c4 = code.reshape(N, nsb, 64, 4)
    out[..., 0:64] = c4[..., 0] | (c4[..., 1] << 2) | (c4[..., 2] << 4) | (c4[..., 3] << 6)
    s = r.integers(0, 8, size=(N, nsb, 16), dtype=np.uint64)
    word = np.zeros((N, nsb), dtype=np.uint64)
    for h in range(16):
        word |= s[..., h] << np.uint64(3 * h)
    for b in range(6):
        out[..., 64 + b] = ((word >> np.uint64(8 * b)) & np.uint64(0xFF)).astype(np.uint8)
    sgn = r.integers(0, 2, size=(N, nsb, 32), dtype=np.uint8).reshape(N, nsb, 4, 8)
    out[..., 70:74] = np.packbits(sgn, axis=-1, bitorder="little")[..., 0]
    out[..., 74:76] = np.full((N, nsb), np.float16(d_value)).view(np.uint8).reshape(N, nsb, 2)
    return out.reshape(N, -1)


def iq1c_grid(seed: int = 0) -> np.ndarray:
    """The iq1c codebook: 2048 distinct ternary 8-vectors drawn uniformly without replacement
    from all 3^8 = 6561, each stored as eight 2-bit codes c = g+1 (value j at bits 2j..2j+1).
    The pages name an 11-bit grid index per 8 values but do not print the grid, so this one is
    self-generated; it is an input of the repack and of the oracle alike."""
    pick = rng(seed, GRID_CFG, T_GRID).choice(3 ** 8, size=GRID_SIZE, replace=False)
    codes = np.zeros(GRID_SIZE, dtype=np.uint16)
    v = pick.copy()
    for j in range(8):
        codes |= ((v % 3).astype(np.uint16) << np.uint16(2 * j))
        v //= 3
    return codes


IQ1C_GRID = iq1c_grid()


def weights_iq1c(N: int, K: int, *, seed: int = 0, cfg: int = 0, tensor: int = T_WEIGHT,
                 d_value: float = 0.02 / 4) -> np.ndarray:
    """IQ1_M codebook rows: per 8 values a grid index uniform in 0..2047 and a delta sign
    uniform in {0, 1}; s uniform in 0..7 per 16 values; d = f16(d_value) per super-block."""
    nsb = K // QK_SUPER
    r = rng(seed, cfg, tensor)
    out = np.empty((N, nsb, 56), dtype=np.uint8)
    idx = r.integers(0, GRID_SIZE, size=(N, nsb, 32), dtype=np.uint16)
    sgn = r.integers(0, 2, size=(N, nsb, 32), dtype=np.uint8)
    s = r.integers(0, 8, size=(N, nsb, 16), dtype=np.uint64)
    out[..., 0:32] = (idx & 0xFF).astype(np.uint8)
    nib = ((idx >> 8) & 7).astype(np.uint8) | (sgn << 3)                  # one nibble per group
    out[..., 32:48] = nib[..., 0::2] | (nib[..., 1::2] << 4)
    word = np.zeros((N, nsb), dtype=np.uint64)
    for h in range(16):
        word |= s[..., h] << np.uint64(3 * h)
    for b in range(6):
        out[..., 48 + b] = ((word >> np.uint64(8 * b)) & np.uint64(0xFF)).astype(np.uint8)
    out[..., 54:56] = np.full((N, nsb), np.float16(d_value)).view(np.uint8).reshape(N, nsb, 2)
    return out.reshape(N, -1)


def weights_iq1s(N: int, K: int, *, seed: int = 0, cfg: int = 0, tensor: int = T_WEIGHT,
                  d_value: float = 0.02 / 4) -> np.ndarray:
    """IQ1_S codebook rows: per 8 values a grid index uniform in 0..2047; per 32 values s
    uniform in 0..7 and a delta sign uniform in {0, 1}; d = f16(d_value) per super-block."""
    nsb = K // QK_SUPER
    r = rng(seed, cfg, tensor)
    out = np.empty((N, nsb, 50), dtype=np.uint8)
    idx = r.integers(0, GRID_SIZE, size=(N, nsb, 8, 4), dtype=np.uint16)
    s = r.integers(0, 8, size=(N, nsb, 8), dtype=np.uint16)
    sgn = r.integers(0, 2, size=(N, nsb, 8), dtype=np.uint16)
    out[..., 0:2] = np.full((N, nsb), np.float16(d_value)).view(np.uint8).reshape(N, nsb, 2)
    out[..., 2:34] = (idx & 0xFF).astype(np.uint8).reshape(N, nsb, 32)
    hi = (idx >> 8) & 7
    qh = hi[..., 0] | (hi[..., 1] << 3) | (hi[..., 2] << 6) | (hi[..., 3] << 9) | (s << 12) | (sgn << 15)
    out[..., 34:50] = qh.astype(np.uint16).view(np.uint8).reshape(N, nsb, 16)
    return out.reshape(N, -1)


def i8_rows(R: int, K: int, *, seed: int = 0, cfg: int = 0, tensor: int = T_WEIGHT):
    """Per-row int8: v ~ N(0,1), scale = max|v|/127 (f32), q = clip(rint(v/scale), -127, 127)."""
    v = rng(seed, cfg, tensor).standard_normal((R, K), dtype=np.float32)
    scale = (np.abs(v).max(axis=1) / np.float32(127)).astype(np.float32)
    q = np.clip(np.rint(v / scale[:, None]), -127, 127).astype(np.int8)
    return q, scale


def weights(fmt: str, N: int, K: int, **kw):
    if fmt == "q8_0":
        return weights_q8_0(N, K, **kw)
    if fmt == "q4_0":
        return weights_q4_0(N, K, **kw)
    if fmt == "q4_K":
        return weights_q4_K(N, K, **kw)
    if fmt == "iq1t":
        return weights_iq1t(N, K, **kw)
    if fmt == "iq1c":
        return weights_iq1c(N, K, **kw)
    if fmt == "iq1s":
        return weights_iq1s(N, K, **kw)
    if fmt == "q6_K":
        return weights_q6_K(N, K, **kw)
    if fmt == "i8_row":
        return i8_rows(N, K, **kw)
    raise ValueError(fmt)


def moe_weights(fmt: str, E: int, N: int, K: int, *, seed: int = 0, cfg: int = 5) -> np.ndarray:
    """E expert matrices of N raw rows each, drawn as one (E*N)-row matrix: [E, N, row bytes]."""
    return weights(fmt, E * N, K, seed=seed, cfg=cfg).reshape(E, N, -1)


def moe_ids(T: int, top_k: int, E: int, *, seed: int = 0, cfg: int = 5) -> np.ndarray:
    """Each token picks top_k distinct experts uniformly at random (without replacement)."""
    u = rng(seed, cfg, T_IDS).random((T, E))
    return np.argsort(u, axis=1)[:, :top_k].astype(np.int32)


# The five measured workloads. 'name' is used by tests and the bench.
CONFIGS = {
    "q8_0_m64_n256_k256": dict(cfg=1, fmt="q8_0", M=64, N=256, K=256, out="f32"),
    "q4_0_m2048_n4096_k4096": dict(cfg=2, fmt="q4_0", M=2048, N=4096, K=4096, out="f32", outlier_rate=1e-3),
    "q4_0_m2048_n11008_k4096": dict(cfg=2, fmt="q4_0", M=2048, N=11008, K=4096, out="f32", outlier_rate=1e-3),
    "q4_K_m512_n14336_k4096": dict(cfg=3, fmt="q4_K", M=512, N=14336, K=4096, out="f32"),
    "q4_K_m512_n4096_k14336": dict(cfg=3, fmt="q4_K", M=512, N=4096, K=14336, out="f32"),
    # q6_K carries a 7B model's ffn_down (and lm_head) in q4_k_m files: the down projection
    "q6_K_m2048_n4096_k11008": dict(cfg=6, fmt="q6_K", M=2048, N=4096, K=11008, out="f32", outlier_rate=1e-3),
    "w8a8_m3072_n1536_k4096": dict(cfg=4, fmt="i8_row", M=3072, N=1536, K=4096, out="bf16"),
    "moe_iq1t_e64_t512_top8_n2048_k4096": dict(cfg=5, fmt="iq1t", M=512, N=2048, K=4096, out="f32", E=64, top_k=8),
    # the same MoE with the IQ1_M codebook form of the weights (1.75 bits per value)
    "moe_iq1c_e64_t512_top8_n2048_k4096": dict(cfg=5, fmt="iq1c", M=512, N=2048, K=4096, out="f32", E=64, top_k=8),
    # and with the IQ1_S codebook form (1.5625 bits per value)
    "moe_iq1s_e64_t512_top8_n2048_k4096": dict(cfg=5, fmt="iq1s", M=512, N=2048, K=4096, out="f32", E=64, top_k=8),
    # decode batches (a few tokens) on the same weight shapes: the small-M path
    "dec_q4_0_m1_n4096_k4096": dict(cfg=2, fmt="q4_0", M=1, N=4096, K=4096, out="f32", outlier_rate=1e-3),
    "dec_q4_0_m8_n4096_k4096": dict(cfg=2, fmt="q4_0", M=8, N=4096, K=4096, out="f32", outlier_rate=1e-3),
    "dec_q4_0_m16_n4096_k4096": dict(cfg=2, fmt="q4_0", M=16, N=4096, K=4096, out="f32", outlier_rate=1e-3),
    "dec_q4_0_m8_n11008_k4096": dict(cfg=2, fmt="q4_0", M=8, N=11008, K=4096, out="f32", outlier_rate=1e-3),
    "dec_q4_0_m32_n4096_k4096": dict(cfg=2, fmt="q4_0", M=32, N=4096, K=4096, out="f32", outlier_rate=1e-3),
    "dec_q4_0_m64_n4096_k4096": dict(cfg=2, fmt="q4_0", M=64, N=4096, K=4096, out="f32", outlier_rate=1e-3),
    "dec_q4_K_m64_n4096_k4096": dict(cfg=3, fmt="q4_K", M=64, N=4096, K=4096, out="f32"),
    "dec_q8_0_m8_n4096_k4096": dict(cfg=1, fmt="q8_0", M=8, N=4096, K=4096, out="f32"),
    "dec_q4_K_m8_n14336_k4096": dict(cfg=3, fmt="q4_K", M=8, N=14336, K=4096, out="f32"),
    "dec_q4_K_m8_n4096_k14336": dict(cfg=3, fmt="q4_K", M=8, N=4096, K=14336, out="f32"),
    "dec_iq1t_m8_n2048_k4096": dict(cfg=5, fmt="iq1t", M=8, N=2048, K=4096, out="f32"),
    "dec_iq1c_m8_n2048_k4096": dict(cfg=5, fmt="iq1c", M=8, N=2048, K=4096, out="f32"),
    "dec_q6_K_m8_n4096_k11008": dict(cfg=6, fmt="q6_K", M=8, N=4096, K=11008, out="f32"),
    "dec_w8a8_m8_n1536_k4096": dict(cfg=4, fmt="i8_row", M=8, N=1536, K=4096, out="bf16"),
    "dec_moe_iq1t_e64_t1_top8_n2048_k4096": dict(cfg=5, fmt="iq1t", M=1, N=2048, K=4096, out="f32", E=64, top_k=8),
    "dec_moe_iq1t_e64_t4_top8_n2048_k4096": dict(cfg=5, fmt="iq1t", M=4, N=2048, K=4096, out="f32", E=64, top_k=8),
    "dec_moe_iq1t_e64_t10_top8_n2048_k4096": dict(cfg=5, fmt="iq1t", M=10, N=2048, K=4096, out="f32", E=64, top_k=8),
}
