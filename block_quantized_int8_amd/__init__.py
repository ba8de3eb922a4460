"""Python binding for libmmq.so, the MI355X (gfx950) prefill MMQ library.

Argument marshalling only: every step of the path (activation quantisation, weight repack,
the MMQ contraction, MoE grouping) runs in the library's HIP kernels. PyTorch provides device
memory and the stream. There is no CPU fallback: if the library is missing, every call raises.

The functions mirror include/mmq.h one to one (same names without the `mmq_` prefix):

    act_bytes, act_region_offsets, quantize_act, packed_bytes, repack_weights, gemm,
    gemm_id_workspace_bytes, gemm_id, gemm_id_noalloc, gemm_id_noalloc_max_workspace_bytes,
    status_string

plus host-side encoders/decoders of the documented act layouts (`act_to_host`,
`act_q8_1_pack_host` and friends for q8_1, `act_i8_pack_host` / `act_i8_to_host` for the
per-token int8 form), used by tests and the bench to fill or read act buffers.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmmq.so")

# enums (include/mmq.h)
MMQ_OK, MMQ_EINVAL, MMQ_EUNSUPPORTED, MMQ_EALIGN, MMQ_EWORKSPACE, MMQ_EHIP = range(6)
WTYPE = {"q8_0": 0, "q4_0": 1, "q4_K": 2, "iq1t": 3, "i8_row": 4, "iq1c": 5, "q6_K": 6, "iq1s": 7}
ATYPE = {"q8_1": 0, "i8_token": 1}
OTYPE = {"f32": 0, "bf16": 1, "i32_partials": 2}


class MMQError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {status_string(code)} ({code})")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmmq.so (built in-tree by __graft_entry__.build()); raise if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    P, I, S = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    e = ctypes.c_int
    L.mmq_status_string.argtypes = [e]
    L.mmq_status_string.restype = ctypes.c_char_p
    L.mmq_act_bytes.argtypes = [e, I, I]
    L.mmq_act_bytes.restype = S
    L.mmq_act_region_offsets.argtypes = [e, I, I, ctypes.POINTER(S)]
    L.mmq_act_region_offsets.restype = e
    L.mmq_quantize_act.argtypes = [e, P, I, I, I, P, P]
    L.mmq_quantize_act.restype = e
    L.mmq_packed_bytes.argtypes = [e, I, I]
    L.mmq_packed_bytes.restype = S
    L.mmq_repack_weights.argtypes = [e, P, P, I, I, P, P]
    L.mmq_repack_weights.restype = e
    L.mmq_gemm.argtypes = [e, P, P, I, I, I, e, P, I, P]
    L.mmq_gemm.restype = e
    L.mmq_gemm_id_workspace_bytes.argtypes = [I, I, I]
    L.mmq_gemm_id_workspace_bytes.restype = S
    L.mmq_gemm_id.argtypes = [e, P, I, P, P, I, I, I, I, e, P, P, S, P]
    L.mmq_gemm_id.restype = e
    L.mmq_gemm_id_noalloc.argtypes = [e, P, I, P, P, I, I, I, I, e, P, P]
    L.mmq_gemm_id_noalloc.restype = e
    L.mmq_gemm_id_noalloc_max_workspace_bytes.argtypes = []
    L.mmq_gemm_id_noalloc_max_workspace_bytes.restype = S
    _lib = L
    return L


def status_string(code: int) -> str:
    return lib().mmq_status_string(int(code)).decode()


def _check(fn: str, code: int):
    if code != MMQ_OK:
        raise MMQError(fn, code)


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def _stream(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _wt(w) -> int:
    return WTYPE[w] if isinstance(w, str) else int(w)


def _at(a) -> int:
    return ATYPE[a] if isinstance(a, str) else int(a)


def _ot(o) -> int:
    return OTYPE[o] if isinstance(o, str) else int(o)


# -------------------------------------------------------------------------- sizes

def act_bytes(atype, M: int, K: int) -> int:
    return int(lib().mmq_act_bytes(_at(atype), M, K))


def act_region_offsets(atype, M: int, K: int) -> tuple[int, int, int, int, int]:
    arr = (ctypes.c_size_t * 5)()
    _check("mmq_act_region_offsets", lib().mmq_act_region_offsets(_at(atype), M, K, arr))
    return tuple(int(v) for v in arr)


def packed_bytes(wtype, N: int, K: int) -> int:
    return int(lib().mmq_packed_bytes(_wt(wtype), N, K))


def gemm_id_workspace_bytes(E: int, T: int, top_k: int) -> int:
    return int(lib().mmq_gemm_id_workspace_bytes(E, T, top_k))


# -------------------------------------------------------------------------- calls

def quantize_act(x, atype="q8_1", out=None, stream=None):
    """x: CUDA float32 [M, K] (row stride x.stride(0)); returns the act buffer (uint8)."""
    import torch
    assert x.is_cuda and x.dtype == torch.float32 and x.dim() == 2 and x.stride(1) == 1
    M, K = x.shape
    nbytes = act_bytes(atype, M, K)
    if nbytes == 0:
        raise MMQError("mmq_act_bytes", MMQ_EINVAL)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    _check("mmq_quantize_act", lib().mmq_quantize_act(_at(atype), _ptr(x), M, K, x.stride(0),
                                                       _ptr(out), _stream(stream)))
    return out


def repack_weights(wtype, raw, N: int, K: int, row_scale=None, out=None, stream=None, grid=None):
    """raw: CUDA tensor holding the raw rows (uint8 bytes, or int8 [N,K] for i8_row).
    The repack's auxiliary input `aux` is row_scale (CUDA f32 [N]) for i8_row and grid (CUDA
    uint16/int16 [2048], the codebook) for iq1c and iq1s."""
    import torch
    nbytes = packed_bytes(wtype, N, K)
    if nbytes == 0:
        raise MMQError("mmq_packed_bytes", MMQ_EINVAL)
    if row_scale is not None and grid is not None:
        raise ValueError("pass row_scale (i8_row) or grid (iq1c, iq1s), not both")
    aux = row_scale if row_scale is not None else grid
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=raw.device)
    _check("mmq_repack_weights", lib().mmq_repack_weights(_wt(wtype), _ptr(raw), _ptr(aux), N, K,
                                                           _ptr(out), _stream(stream)))
    return out


def gemm(wtype, packed, act, M: int, N: int, K: int, otype="f32", out=None, ldo=None, stream=None):
    import torch
    o = _ot(otype)
    if out is None:
        if o == OTYPE["f32"]:
            out = torch.empty((M, N), dtype=torch.float32, device=packed.device)
        elif o == OTYPE["bf16"]:
            out = torch.empty((M, N), dtype=torch.bfloat16, device=packed.device)
        else:
            w = _wt(wtype)
            shape = (M, N) if w == WTYPE["i8_row"] else (M, N, K // 16) if w == WTYPE["q6_K"] else (M, N, K // 32)
            out = torch.empty(shape, dtype=torch.int32, device=packed.device)
    if ldo is None:
        ldo = out.stride(0) if out.dim() == 2 else N
    _check("mmq_gemm", lib().mmq_gemm(_wt(wtype), _ptr(packed), _ptr(act), M, N, K, o, _ptr(out), ldo,
                                       _stream(stream)))
    return out


def gemm_id(wtype, packed, E: int, act, ids, T: int, top_k: int, N: int, K: int, out=None,
            workspace=None, stream=None):
    import torch
    if out is None:
        out = torch.empty((T, top_k, N), dtype=torch.float32, device=packed.device)
    ws = gemm_id_workspace_bytes(E, T, top_k)
    if workspace is None:
        workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=packed.device)
    _check("mmq_gemm_id", lib().mmq_gemm_id(_wt(wtype), _ptr(packed), E, _ptr(act), _ptr(ids), T, top_k, N, K,
                                             OTYPE["f32"], _ptr(out), _ptr(workspace), workspace.numel(),
                                             _stream(stream)))
    return out


def gemm_id_noalloc_max_workspace_bytes() -> int:
    return int(lib().mmq_gemm_id_noalloc_max_workspace_bytes())


def gemm_id_noalloc(wtype, packed, E: int, act, ids, T: int, top_k: int, N: int, K: int, out, stream=None):
    """mmq_gemm_id without a workspace argument: the library's static per-GPU scratch is used.
    `out` must be given (the call allocates nothing)."""
    _check("mmq_gemm_id_noalloc", lib().mmq_gemm_id_noalloc(_wt(wtype), _ptr(packed), E, _ptr(act), _ptr(ids), T,
                                                             top_k, N, K, OTYPE["f32"], _ptr(out), _stream(stream)))
    return out


# -------------------------------------------------------------------------- host helpers

def _act_dims(M: int, K: int):
    Mp = (M + 31) // 32 * 32
    KB = K // 32
    KBp = (KB + 7) // 8 * 8
    return Mp, KB, KBp, Mp // 32


def _act_regions(act_bytes_host: np.ndarray, M: int, K: int):
    """All four q8_1 regions, padding included, as row-major arrays: xq int8 [Mp, KBp*32],
    xs2 uint32 [Mp, KBp], xsx f32 [Mp, KBp], xg uint32 [Mp, KBp, 2] (the dword of half h of each
    block; all stored tiled, transposed back here)."""
    o = act_region_offsets("q8_1", M, K)
    Mp, KB, KBp, MT = _act_dims(M, K)
    buf = np.asarray(act_bytes_host, dtype=np.uint8)
    t = buf[o[0]:o[0] + MT * KBp * 1024].view(np.int8).reshape(MT, KBp, 2, 32, 16)   # [mt, b, h, r, 16]
    xq = t.transpose(0, 3, 1, 2, 4).reshape(Mp, KBp * 32)
    cells = Mp * KBp
    def tile_major(region, dt):
        return buf[region:region + 4 * cells].view(dt).reshape(MT, KBp, 32).transpose(0, 2, 1).reshape(Mp, KBp)
    xs2 = tile_major(o[1], np.uint32)
    xsx = tile_major(o[2], np.float32)
    xg = buf[o[3]:o[3] + 8 * cells].view(np.uint32).reshape(MT, KBp, 2, 32).transpose(0, 3, 1, 2).reshape(Mp, KBp, 2)
    return xq, xs2, xsx, xg


def _half_bits(v):
    return np.asarray(v, np.uint32).astype(np.uint16).view(np.float16).astype(np.float32)


def act_groups_host(act_bytes_host: np.ndarray, M: int, K: int):
    """Region 3 decoded: the integer 8-value group sums G as int32 [Mp, KBp, 4], padding
    included (G_j * 2^-13 is stored as f16, so G_j = f16 value * 2^13 exactly)."""
    _, _, _, xg = _act_regions(act_bytes_host, M, K)
    g = np.stack([_half_bits(xg & 0xFFFF), _half_bits(xg >> 16)], axis=-1).reshape(xg.shape[0], xg.shape[1], 4)
    return (g.astype(np.float64) * 8192.0).astype(np.int32)


def act_to_host(act_bytes_host: np.ndarray, M: int, K: int):
    """Decode a q8_1 act buffer (copied to host as uint8) into plain row-major
    (xq int8 [M,K], xs f32 [M,K/32], xsum int32 [M,K/32]) following the documented layout:
    xs is the low f16 half of region 1, xsum the sum of the four group sums of region 3."""
    xq, xs2, _, _ = _act_regions(act_bytes_host, M, K)
    KB = K // 32
    xs = _half_bits(xs2 & 0xFFFF)
    xsum = act_groups_host(act_bytes_host, M, K).sum(axis=2).astype(np.int32)
    return (np.ascontiguousarray(xq[:M, :K]), np.ascontiguousarray(xs[:M, :KB]),
            np.ascontiguousarray(xsum[:M, :KB]))


def act_derived_host(act_bytes_host: np.ndarray, M: int, K: int):
    """Regions 1 and 2 decoded to f32 [Mp, KBp] each (padding included): the low and high f16
    halves of xs2, and xsx. They must equal xs, xs and xs * xsum exactly."""
    _, xs2, xsx, _ = _act_regions(act_bytes_host, M, K)
    return _half_bits(xs2 & 0xFFFF), _half_bits(xs2 >> 16), xsx.copy()


def act_padding_host(act_bytes_host: np.ndarray, M: int, K: int):
    """The padded rows (m >= M) and padded blocks (b >= K/32) of every region of a q8_1 act
    buffer, as one flat array that must be all zero."""
    xq, xs2, xsx, xg = _act_regions(act_bytes_host, M, K)
    KB = K // 32
    pads = [xq[M:].ravel(), xq[:, K:].ravel()]
    for r in (xs2, xsx, xg):
        pads += [r[M:].ravel(), r[:, KB:].ravel()]
    return np.concatenate([p.astype(np.float64) for p in pads])


def act_q8_1_pack_host(xq: np.ndarray, xs: np.ndarray) -> np.ndarray:
    """Encode q8_1 activations (xq int8 [M, K], xs f32 [M, K/32], the f16-exact block scales)
    into the documented MMQ_ACT_Q8_1 layout (uint8 buffer of act_bytes("q8_1", M, K) bytes);
    xsum and the group sums are taken from xq."""
    xq = np.asarray(xq, dtype=np.int8)
    M, K = xq.shape
    o = act_region_offsets("q8_1", M, K)
    Mp, KB, KBp, MT = _act_dims(M, K)
    buf = np.zeros(act_bytes("q8_1", M, K), np.uint8)
    full = np.zeros((Mp, KBp * 32), np.int8)
    full[:M, :K] = xq
    buf[o[0]:o[0] + MT * KBp * 1024] = full.reshape(MT, 32, KBp, 2, 16).transpose(0, 2, 3, 1, 4).reshape(-1).view(np.uint8)
    g = full.reshape(Mp, KBp, 4, 8).astype(np.int64).sum(axis=3)                      # [Mp, KBp, 4]
    s = np.zeros((Mp, KBp), np.float32)
    s[:M, :KB] = xs
    h = s.astype(np.float16).view(np.uint16).astype(np.uint32)
    def tm(a):
        return a.reshape(MT, 32, KBp).transpose(0, 2, 1).reshape(-1)
    buf[o[1]:o[1] + 4 * Mp * KBp] = tm(h | (h << 16)).view(np.uint8)
    buf[o[2]:o[2] + 4 * Mp * KBp] = tm((s * g.sum(axis=2).astype(np.float32)).astype(np.float32)).view(np.uint8)
    gh = (g.astype(np.float32) * np.float32(2.0 ** -13)).astype(np.float16).view(np.uint16).astype(np.uint32)
    pair = gh[..., 0::2] | (gh[..., 1::2] << 16)                                      # [Mp, KBp, 2 halves]
    buf[o[3]:o[3] + 8 * Mp * KBp] = pair.reshape(MT, 32, KBp, 2).transpose(0, 2, 3, 1).reshape(-1).view(np.uint8)
    return buf


def act_i8_pack_host(a: np.ndarray, sa: np.ndarray) -> np.ndarray:
    """Encode int8 activations a [M, K] and per-token scales sa [M] into the documented
    MMQ_ACT_I8_TOKEN layout (uint8 buffer of act_bytes("i8_token", M, K) bytes)."""
    a = np.asarray(a, dtype=np.int8)
    M, K = a.shape
    o = act_region_offsets("i8_token", M, K)
    Mp, KB, KBp, MT = _act_dims(M, K)
    buf = np.zeros(act_bytes("i8_token", M, K), np.uint8)
    full = np.zeros((Mp, KBp * 32), np.int8)
    full[:M, :K] = a
    t = full.reshape(MT, 32, KBp, 2, 16).transpose(0, 2, 3, 1, 4)          # [mt, b, h, r, 16]
    buf[o[0]:o[0] + MT * KBp * 1024] = t.reshape(-1).view(np.uint8)
    sp = np.zeros(Mp, np.float32)
    sp[:M] = np.asarray(sa, dtype=np.float32)
    buf[o[1]:o[1] + 4 * Mp] = sp.view(np.uint8)
    return buf


def act_i8_to_host(act_bytes_host: np.ndarray, M: int, K: int, padded: bool = False):
    """Decode an MMQ_ACT_I8_TOKEN buffer (copied to host as uint8) into (a int8 [M, K],
    sa f32 [M]), or with padded=True into ([Mp, KBp*32], [Mp]) including the zero padding."""
    o = act_region_offsets("i8_token", M, K)
    Mp, KB, KBp, MT = _act_dims(M, K)
    buf = np.asarray(act_bytes_host, dtype=np.uint8)
    t = buf[o[0]:o[0] + MT * KBp * 1024].view(np.int8).reshape(MT, KBp, 2, 32, 16)
    full = t.transpose(0, 3, 1, 2, 4).reshape(Mp, KBp * 32)
    sa = buf[o[1]:o[1] + 4 * Mp].view(np.float32)
    if padded:
        return full.copy(), sa.copy()
    return np.ascontiguousarray(full[:M, :K]), sa[:M].copy()
