"""CPU oracle for the prefill MMQ contraction - TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may
import this package. The HIP library and its Python binding never do, and
this package imports nothing from them. The only code both sides share is
the seeded input generator module `gen` (which holds none of the method's
arithmetic).

Two independent parts:

(i) `liborc` - a plain C implementation (mmq_oracle.c) of the per-block
    integer structure: the q8_1 quantiser, the exact int32 block partials,
    the f32 output accumulated in double, the W8A8 bf16 epilogue. It is the
    bit-exact reference for quantised activations, partials and bf16 outputs,
    and it is the timed CPU baseline.

(ii) the NumPy f64 definition in this file: dequantise both operands with the
    formats' defining formulas and take one f64 matmul,
        out[m,n] = sum_k (xs*xq)[m,k] * w_hat[n,k],
    which is what the method reaches up to f32 rounding order ("A Negative
    Result on int8 Tensor-Core MMQ", section 2; minfer R1 sections 2.1 and 4).

Function-by-function citations are in the docstrings. No function here is
"parity unpinned": each is pinned by tests/test_oracle_*.py against closed
forms, hand-derived golden blocks, library routines or brute force.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mmq_oracle.c")
_LIB = os.path.join(_HERE, "liborc.so")

FMT_ID = {"q8_0": 0, "q4_0": 1, "q4_K": 2, "iq1t": 3, "iq1c": 4, "q6_K": 5, "iq1s": 6}


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                        "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        L.orc_half_to_float.argtypes = [ctypes.c_uint16]
        L.orc_half_to_float.restype = ctypes.c_float
        L.orc_float_to_half.argtypes = [ctypes.c_float]
        L.orc_float_to_half.restype = ctypes.c_uint16
        L.orc_float_to_bf16.argtypes = [ctypes.c_float]
        L.orc_float_to_bf16.restype = ctypes.c_uint16
        L.orc_quantize_q8_1.argtypes = [P, I, I, I, P, P, P]
        L.orc_quantize_i8_token.argtypes = [P, I, I, I, P, P]
        L.orc_decode_row.argtypes = [ctypes.c_int, P, I, P, P, P, P, P]
        L.orc_decode_row.restype = ctypes.c_int
        L.orc_partials.argtypes = [ctypes.c_int, P, I, I, P, P, I, P]
        L.orc_partials.restype = ctypes.c_int
        L.orc_partials16.argtypes = [ctypes.c_int, P, I, I, P, P, I, P]
        L.orc_gemm_rows.argtypes = [ctypes.c_int, P, I, I, P, P, P, P, I, I, P, I]
        L.orc_gemm_rows.restype = ctypes.c_int
        L.orc_gemm_abs_rows.argtypes = [ctypes.c_int, P, I, I, P, P, P, P, I, I, P]
        L.orc_gemm_abs_rows.restype = ctypes.c_int
        L.orc_gemm.argtypes = [ctypes.c_int, P, I, I, P, P, P, P, I, P]
        L.orc_gemm.restype = ctypes.c_int
        L.orc_gemm_w8a8.argtypes = [P, P, I, P, P, I, I, P, P, I, I]
        L.orc_gemm_w8a8.restype = ctypes.c_int
        L.orc_num_threads.restype = ctypes.c_int
        L.orc_set_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ----------------------------------------------------------------- scalars

def half_to_float(bits: int) -> float:
    return float(lib().orc_half_to_float(int(bits)))


def float_to_half_bits(x: float) -> int:
    return int(lib().orc_float_to_half(float(x)))


def float_to_bf16_bits(x: float) -> int:
    return int(lib().orc_float_to_bf16(float(x)))


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_threads(n: int) -> None:
    """OpenMP thread count of later calls (timing only; results do not depend on it)."""
    lib().orc_set_threads(int(n))


# -------------------------------------------------------------- quantisers

def quantize_q8_1(x: np.ndarray):
    """q8_1 activations per minfer R1 section 3.2 (the parity test's CPU reference) and
    section 2.2 (block sum kept with the block). Returns (xq int8 [M,K], xs f32 [M,K/32],
    xsum int32 [M,K/32]) in plain row-major order."""
    x = _c(x, np.float32)
    M, K = x.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    xq = np.empty((M, K), np.int8)
    xs = np.empty((M, K // 32), np.float32)
    xsum = np.empty((M, K // 32), np.int32)
    lib().orc_quantize_q8_1(_p(x), M, K, K, _p(xq), _p(xs), _p(xsum))
    return xq, xs, xsum


def quantize_i8_token(x: np.ndarray):
    """Per-token int8 activations (metainfer W8A8 section 1: int8 A with a per-token f32 scale);
    the q8_1 steps with one block per row and the scale kept in f32."""
    x = _c(x, np.float32)
    M, K = x.shape
    a = np.empty((M, K), np.int8)
    sa = np.empty((M,), np.float32)
    lib().orc_quantize_i8_token(_p(x), M, K, K, _p(a), _p(sa))
    return a, sa


# ------------------------------------------------------------ C decode / partials

def _grid_arg(fmt: str, grid):
    """The codebook as a contiguous uint16 [2048] array (required for iq1c and iq1s only)."""
    if fmt not in ("iq1c", "iq1s"):
        return None
    if grid is None:
        raise ValueError(f"{fmt} needs its grid (uint16 [2048])")
    g = _c(grid, np.uint16)
    if g.shape != (2048,):
        raise ValueError("the iq1c grid has 2048 entries")
    return g


def decode_row_c(fmt: str, raw_row: np.ndarray, K: int, grid=None):
    """C decoder for one row: (wq int16 [K], wd f32 [K/16], wm f32 [K/32], mult int16 [K/16])."""
    raw_row = _c(raw_row, np.uint8)
    g = _grid_arg(fmt, grid)
    wq = np.empty(K, np.int16)
    wd = np.empty(K // 16, np.float32)
    wm = np.empty(K // 32, np.float32)
    mult = np.empty(K // 16, np.int16)
    rc = lib().orc_decode_row(FMT_ID[fmt], _p(raw_row), K, None if g is None else _p(g), _p(wq), _p(wd),
                              _p(wm), _p(mult))
    if rc != 0:
        raise ValueError("invalid iq1c grid code (3)")
    return wq, wd, wm, mult


def partials(fmt: str, raw: np.ndarray, N: int, K: int, xq: np.ndarray, grid=None) -> np.ndarray:
    """Exact int32 block partials P[m,n,b] (iq1t, iq1c: the folded per-32 integer
    sum_h (2s_h+1)*P16_h, PR #304's fold)."""
    raw = _c(raw, np.uint8)
    xq = _c(xq, np.int8)
    g = _grid_arg(fmt, grid)
    M = xq.shape[0]
    P = np.empty((M, N, K // 32), np.int32)
    rc = lib().orc_partials(FMT_ID[fmt], _p(raw), N, K, None if g is None else _p(g), _p(xq), M, _p(P))
    if rc == -2:
        raise ValueError("invalid iq1c grid code (3)")
    if rc != 0:
        raise OverflowError("a block partial left int32")
    return P


def partials16(fmt: str, raw: np.ndarray, N: int, K: int, xq: np.ndarray, grid=None) -> np.ndarray:
    """Exact int32 per-16 partials P16[m,n,h] = sum over half-block h of xq*wq (iq1t/iq1c:
    before the (2s+1) fold; q6_K: the two separate half-block sums of each 32-value block,
    minfer R1 sections 2.2 and 3.3)."""
    raw = _c(raw, np.uint8)
    xq = _c(xq, np.int8)
    g = _grid_arg(fmt, grid)
    M = xq.shape[0]
    P = np.empty((M, N, K // 16), np.int32)
    lib().orc_partials16(FMT_ID[fmt], _p(raw), N, K, None if g is None else _p(g), _p(xq), M, _p(P))
    return P


def partials16_iq1t(raw: np.ndarray, N: int, K: int, xq: np.ndarray) -> np.ndarray:
    return partials16("iq1t", raw, N, K, xq)


def gemm_c(fmt: str, raw: np.ndarray, N: int, K: int, xq, xs, xsum, rows=None, grid=None) -> np.ndarray:
    """Per-block C oracle output (double accumulation, one f32 rounding). rows=(m0,m1)
    restricts to a row range."""
    raw = _c(raw, np.uint8)
    xq = _c(xq, np.int8)
    xs = _c(xs, np.float32)
    xsum = _c(xsum, np.int32)
    g = _grid_arg(fmt, grid)
    M = xq.shape[0]
    m0, m1 = (0, M) if rows is None else rows
    out = np.empty((m1 - m0, N), np.float32)
    rc = lib().orc_gemm_rows(FMT_ID[fmt], _p(raw), N, K, None if g is None else _p(g), _p(xq), _p(xs),
                             _p(xsum), m0, m1, _p(out), N)
    if rc != 0:
        raise ValueError("invalid iq1c grid code (3)")
    return out


def gemm_abs(fmt: str, raw: np.ndarray, N: int, K: int, xq, xs, xsum, rows=None, grid=None) -> np.ndarray:
    """f64 [M, N]: the sum of the magnitudes of the per-block (per-half) terms the contraction
    adds for each output, sum_b sum_h |xs*wd_h*P16_h| + |xs*wm*xsum|: the scale of the rounding
    error of any evaluation that adds those terms in f32."""
    raw = _c(raw, np.uint8)
    xq = _c(xq, np.int8)
    xs = _c(xs, np.float32)
    xsum = _c(xsum, np.int32)
    g = _grid_arg(fmt, grid)
    M = xq.shape[0]
    m0, m1 = (0, M) if rows is None else rows
    out = np.empty((m1 - m0, N), np.float64)
    rc = lib().orc_gemm_abs_rows(FMT_ID[fmt], _p(raw), N, K, None if g is None else _p(g), _p(xq), _p(xs),
                                 _p(xsum), m0, m1, _p(out))
    if rc != 0:
        raise ValueError("invalid iq1c grid code (3)")
    return out


def gemm_w8a8(a, sa, w, sw, rows=None, want_acc: bool = False):
    """W8A8 per metainfer section 1: exact int32 accumulation, epilogue
    bf16_rne((f32(acc)*sa[m])*sw[n]). Returns bf16 bits (uint16) [and int32 acc]."""
    a = _c(a, np.int8)
    w = _c(w, np.int8)
    sa = _c(sa, np.float32)
    sw = _c(sw, np.float32)
    M, K = a.shape
    N = w.shape[0]
    m0, m1 = (0, M) if rows is None else rows
    out = np.empty((m1 - m0, N), np.uint16)
    acc = np.empty((m1 - m0, N), np.int32) if want_acc else None
    rc = lib().orc_gemm_w8a8(_p(a), _p(sa), M, _p(w), _p(sw), N, K,
                             _p(acc) if want_acc else None, _p(out), m0, m1)
    if rc != 0:
        raise OverflowError("a W8A8 accumulator left int32")
    return (out, acc) if want_acc else out


# ------------------------------------------------------ NumPy f64 definition

def _f16(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def dequant_weights(fmt: str, raw: np.ndarray, N: int, K: int, grid=None) -> np.ndarray:
    """w_hat [N,K] in f64 from each format's defining formula (independent of the C decoder):
    q8_0 d*q; q4_0 d*(nib-8); q4_K d*sc*nib - dmin*m (minfer R1 section 2.2);
    q6_K d*sc_h*(q-32) with one int8 sc per 16 values (minfer R1 sections 2.2 and 3.3);
    iq1t, iq1c and iq1s d*(2s+1)*(g+delta) (PR #304 description; iq1c and iq1s take the eight
    g of a group from the grid entry its 11-bit index names; iq1s has s and delta per 32)."""
    raw = np.asarray(raw, dtype=np.uint8).reshape(N, -1)
    if fmt == "q8_0":
        b = raw.reshape(N, K // 32, 34)
        d = _f16(b[..., 0].astype(np.uint16) | (b[..., 1].astype(np.uint16) << 8))
        q = b[..., 2:].view(np.int8).astype(np.float64)
        return (d[..., None] * q).reshape(N, K)
    if fmt == "q4_0":
        b = raw.reshape(N, K // 32, 18)
        d = _f16(b[..., 0].astype(np.uint16) | (b[..., 1].astype(np.uint16) << 8))
        qs = b[..., 2:]
        nib = np.concatenate([qs & 0xF, qs >> 4], axis=-1).astype(np.float64)
        return (d[..., None] * (nib - 8.0)).reshape(N, K)
    if fmt == "q4_K":
        b = raw.reshape(N, K // 256, 144)
        d = _f16(b[..., 0].astype(np.uint16) | (b[..., 1].astype(np.uint16) << 8))
        dmin = _f16(b[..., 2].astype(np.uint16) | (b[..., 3].astype(np.uint16) << 8))
        bits_sc = np.unpackbits(b[..., 4:10], axis=-1, bitorder="little").reshape(N, K // 256, 8, 6)
        bits_m = np.unpackbits(b[..., 10:16], axis=-1, bitorder="little").reshape(N, K // 256, 8, 6)
        weights6 = (1 << np.arange(6)).astype(np.float64)
        sc = bits_sc @ weights6
        mm = bits_m @ weights6
        qs = b[..., 16:].reshape(N, K // 256, 8, 16)
        nib = np.concatenate([qs & 0xF, qs >> 4], axis=-1).astype(np.float64)   # [N, sb, 8, 32]
        w = d[..., None, None] * sc[..., None] * nib - dmin[..., None, None] * mm[..., None]
        return w.reshape(N, K)
    if fmt == "iq1t":
        b = raw.reshape(N, K // 256, 76)
        codes = np.stack([(b[..., :64] >> (2 * j)) & 3 for j in range(4)], axis=-1).reshape(N, K // 256, 256)
        g = codes.astype(np.float64) - 1.0
        s_bits = np.unpackbits(b[..., 64:70], axis=-1, bitorder="little")[..., :48].reshape(N, K // 256, 16, 3)
        s = s_bits @ np.array([1.0, 2.0, 4.0])
        sgn = np.unpackbits(b[..., 70:74], axis=-1, bitorder="little").reshape(N, K // 256, 32)
        delta = np.where(sgn == 1, -0.125, 0.125)
        d = _f16(b[..., 74].astype(np.uint16) | (b[..., 75].astype(np.uint16) << 8))
        w = (d[..., None] * np.repeat(2.0 * s + 1.0, 16, axis=-1)) * (g + np.repeat(delta, 8, axis=-1))
        return w.reshape(N, K)
    if fmt == "iq1c":
        table = _grid_arg(fmt, grid)
        gvals = np.stack([(table >> (2 * j)) & 3 for j in range(8)], axis=-1).astype(np.int64)
        if np.any(gvals == 3):
            raise ValueError("invalid iq1c grid code (3)")
        b = raw.reshape(N, K // 256, 56)
        qh = np.stack([b[..., 32:48] & 0xF, b[..., 32:48] >> 4], axis=-1).reshape(N, K // 256, 32)
        idx = b[..., 0:32].astype(np.int64) + 256 * (qh & 7).astype(np.int64)
        g = gvals[idx].astype(np.float64) - 1.0                                # [N, sb, 32, 8]
        delta = np.where((qh >> 3) == 1, -0.125, 0.125)
        s_bits = np.unpackbits(b[..., 48:54], axis=-1, bitorder="little")[..., :48].reshape(N, K // 256, 16, 3)
        s = s_bits @ np.array([1.0, 2.0, 4.0])
        d = _f16(b[..., 54].astype(np.uint16) | (b[..., 55].astype(np.uint16) << 8))
        w = (d[..., None] * np.repeat(2.0 * s + 1.0, 16, axis=-1)) * (g + delta[..., None]).reshape(N, K // 256, 256)
        return w.reshape(N, K)
    if fmt == "iq1s":
        table = _grid_arg(fmt, grid)
        gvals = np.stack([(table >> (2 * j)) & 3 for j in range(8)], axis=-1).astype(np.int64)
        if np.any(gvals == 3):
            raise ValueError("invalid iq1s grid code (3)")
        b = raw.reshape(N, K // 256, 50)
        d = _f16(b[..., 0].astype(np.uint16) | (b[..., 1].astype(np.uint16) << 8))
        qh = (b[..., 34:50:2].astype(np.int64) | (b[..., 35:50:2].astype(np.int64) << 8))   # [N, sb, 8]
        hi = np.stack([(qh >> (3 * j)) & 7 for j in range(4)], axis=-1)                    # [N, sb, 8, 4]
        idx = b[..., 2:34].astype(np.int64).reshape(N, K // 256, 8, 4) + 256 * hi
        g = gvals[idx].astype(np.float64) - 1.0                                            # [N, sb, 8, 4, 8]
        s = ((qh >> 12) & 7).astype(np.float64)
        delta = np.where(((qh >> 15) & 1) == 1, -0.125, 0.125)
        w = d[..., None, None, None] * (2.0 * s + 1.0)[..., None, None] * (g + delta[..., None, None])
        return w.reshape(N, K)
    if fmt == "q6_K":
        b = raw.reshape(N, K // 256, 210)
        ql = b[..., 0:128].reshape(N, K // 256, 8, 16)
        lo = np.concatenate([ql & 0xF, ql >> 4], axis=-1)                      # [N, sb, 8, 32]
        qh = b[..., 128:192].reshape(N, K // 256, 8, 1, 8)
        hi = ((qh >> (2 * np.arange(4)[:, None])) & 3).reshape(N, K // 256, 8, 32)
        q = (lo.astype(np.int64) | (hi.astype(np.int64) << 4)).reshape(N, K // 256, 256)
        sc = b[..., 192:208].view(np.int8).astype(np.float64)
        d = _f16(b[..., 208].astype(np.uint16) | (b[..., 209].astype(np.uint16) << 8))
        w = d[..., None] * np.repeat(sc, 16, axis=-1) * (q - 32).astype(np.float64)
        return w.reshape(N, K)
    raise ValueError(fmt)


def dequant_act(xq: np.ndarray, xs: np.ndarray) -> np.ndarray:
    """x_hat = xs * xq per 32-block, in f64."""
    M, K = xq.shape
    return (xq.reshape(M, K // 32, 32).astype(np.float64) * xs.astype(np.float64)[..., None]).reshape(M, K)


def gemm_f64(fmt: str, raw: np.ndarray, N: int, K: int, xq: np.ndarray, xs: np.ndarray,
             rows=None, cols=None, grid=None) -> np.ndarray:
    """The definition: out[m,n] = sum_k x_hat[m,k] * w_hat[n,k] in f64 (optionally on a
    subset of rows / weight rows, for sampled checks of large shapes)."""
    xh = dequant_act(xq if rows is None else xq[rows], xs if rows is None else xs[rows])
    raw2 = np.asarray(raw, np.uint8).reshape(N, -1)
    if cols is not None:
        raw2 = raw2[cols]
    wh = dequant_weights(fmt, raw2, raw2.shape[0], K, grid=grid)
    return xh @ wh.T


def moe_f64(fmt: str, raw_experts: np.ndarray, E: int, N: int, K: int, xq, xs, ids,
            pairs=None, grid=None) -> np.ndarray:
    """MUL_MAT_ID: out[t, j, :] = dense(W_{ids[t,j]}, x[t]) (PR #304: MUL_MAT_ID routes each
    token's rows through the selected experts). pairs: optional list of (t, j) to evaluate;
    returns [T, top_k, N] (NaN where not evaluated) or [len(pairs), N]."""
    raw_experts = np.asarray(raw_experts, np.uint8).reshape(E, N, -1)
    T, top_k = ids.shape
    if pairs is None:
        out = np.zeros((T, top_k, N), np.float64)
        for e in range(E):
            tt, jj = np.nonzero(ids == e)
            if len(tt) == 0:
                continue
            out[tt, jj] = gemm_f64(fmt, raw_experts[e], N, K, xq[tt], xs[tt], grid=grid)
        return out
    res = np.zeros((len(pairs), N), np.float64)
    for i, (t, j) in enumerate(pairs):
        e = int(ids[t, j])
        res[i] = gemm_f64(fmt, raw_experts[e], N, K, xq[t:t + 1], xs[t:t + 1], grid=grid)[0]
    return res


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)
