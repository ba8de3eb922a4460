"""Host-side tests of the C ABI (no GPU needed): the library loads, exports every entry point
include/mmq.h declares, sizes its buffers as documented, and rejects bad arguments on the
host before touching the device (every call here returns before any HIP call)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mmq.h")


@pytest.fixture(scope="module")
def mmq():
    import block_quantized_int8_amd as m
    if not os.path.exists(m.LIB_PATH):
        from block_quantized_int8_amd import build
        build.build()
    m.lib()
    return m


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mmq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_path_calls():
    names = _declared_functions()
    for fn in ["mmq_quantize_act", "mmq_repack_weights", "mmq_gemm", "mmq_gemm_id"]:
        assert fn in names


def test_library_exports_every_declared_symbol(mmq):
    L = mmq.lib()
    for fn in _declared_functions():
        assert hasattr(L, fn), fn


def test_status_strings(mmq):
    for code in range(6):
        assert mmq.status_string(code).startswith("MMQ_")
    assert "unknown" in mmq.status_string(99)


def test_act_bytes_and_offsets(mmq):
    M, K = 70, 96                      # Mp = 96, KB = 3, KBp = 8
    o = mmq.act_region_offsets("q8_1", M, K)
    cells = 96 * 8                     # (row, block) entries of a scale region
    assert o[0] == 0
    assert o[1] == 3 * 8 * 1024        # xq region: MT * KBp * 1 KB
    assert o[2] == o[1] + 4 * cells    # xs2 f16 pair
    assert o[3] == o[2] + 4 * cells    # xsx f32
    assert o[4] == 0
    assert mmq.act_bytes("q8_1", M, K) == o[3] + 8 * cells   # xg: two f16 pairs per (row, block)
    assert all(v % 256 == 0 for v in o)
    # i8_token: Mp=32, KBp=8 -> one 8 KB tile region, then sa f32 [Mp]
    oi = mmq.act_region_offsets("i8_token", 3, 64)
    assert oi == (0, 8192, 0, 0, 0)
    assert mmq.act_bytes("i8_token", 3, 64) == 8192 + 256
    assert mmq.act_bytes("q8_1", 4, 33) == 0         # K not a multiple of 32
    assert mmq.act_bytes("q8_1", 0, 64) == 0
    assert mmq.act_bytes(7, 4, 64) == 0


def test_packed_bytes(mmq):
    # q4_0: NT=2 (Np=64), KBp=8 -> 2*8*512 B fragments + 64*8 scale dwords
    assert mmq.packed_bytes("q4_0", 40, 64) == 2 * 8 * 512 + 64 * 8 * 4
    assert mmq.packed_bytes("q8_0", 32, 256) == 8 * 1024 + 32 * 8 * 4
    # q4_K: + a row-major f32 min region; iq1t: 256 B code fragments
    assert mmq.packed_bytes("q4_K", 32, 256) == 8 * 512 + 2 * 32 * 8 * 4
    assert mmq.packed_bytes("iq1t", 32, 256) == 8 * 256 + 32 * 8 * 4
    assert mmq.packed_bytes("i8_row", 33, 32) == 2 * 8 * 1024 + 256
    assert mmq.packed_bytes("q4_K", 32, 128) == 0      # Q4_K needs K % 256 == 0
    assert mmq.packed_bytes("iq1t", 32, 200) == 0
    # iq1c / iq1s grid-index panels (K % 256 required): 256 B index fragments per (tile,
    # block), f16 d per (row, 4-block group), then the 8 KiB grid; iq1s the same layout
    assert mmq.packed_bytes("iq1c", 40, 512) == 2 * 16 * 256 + 64 * 4 * 2 + 8192   # Np = 64, KBp = 16
    assert mmq.packed_bytes("iq1c", 32, 288) == 0
    assert mmq.packed_bytes("iq1s", 40, 512) == mmq.packed_bytes("iq1c", 40, 512)
    # q6_K: int8 fragments plus two scale-dword regions (one per 16-value half)
    assert mmq.packed_bytes("q6_K", 32, 256) == 8 * 1024 + 2 * 32 * 8 * 4
    assert mmq.packed_bytes("q6_K", 32, 224) == 0
    assert mmq.packed_bytes(9, 32, 64) == 0


def test_validation_rejects_before_any_launch(mmq):
    L = mmq.lib()
    BAD = ctypes.c_void_p(0x1001)      # misaligned, never dereferenced
    GOOD = ctypes.c_void_p(0x10000)    # aligned, never dereferenced (validation fails first)
    # null pointers
    assert L.mmq_quantize_act(0, None, 4, 64, 64, GOOD, None) == mmq.MMQ_EINVAL
    assert L.mmq_gemm(0, None, GOOD, 4, 32, 64, 0, GOOD, 32, None) == mmq.MMQ_EINVAL
    # sizes / strides / enums
    assert L.mmq_quantize_act(0, GOOD, 4, 48, 48, GOOD, None) == mmq.MMQ_EINVAL      # K % 32
    assert L.mmq_quantize_act(0, GOOD, 4, 64, 32, GOOD, None) == mmq.MMQ_EINVAL      # ldx < K
    assert L.mmq_quantize_act(5, GOOD, 4, 64, 64, GOOD, None) == mmq.MMQ_EINVAL      # atype
    assert L.mmq_gemm(0, GOOD, GOOD, 4, 32, 64, 0, GOOD, 16, None) == mmq.MMQ_EINVAL   # ldo < N
    assert L.mmq_gemm(2, GOOD, GOOD, 4, 32, 128, 0, GOOD, 32, None) == mmq.MMQ_EINVAL  # q4_K K
    assert L.mmq_gemm(0, GOOD, GOOD, 0, 32, 64, 0, GOOD, 32, None) == mmq.MMQ_EINVAL   # M = 0
    assert L.mmq_gemm(0, GOOD, GOOD, 4, 32, 64, 3, GOOD, 32, None) == mmq.MMQ_EINVAL   # otype
    assert L.mmq_gemm(0, GOOD, GOOD, 4, 32, 64, 2, GOOD, 40, None) == mmq.MMQ_EINVAL   # partials ldo
    assert L.mmq_gemm(6, GOOD, GOOD, 4, 32, 128, 0, GOOD, 32, None) == mmq.MMQ_EINVAL  # q6_K K
    assert L.mmq_gemm(8, GOOD, GOOD, 4, 32, 256, 0, GOOD, 32, None) == mmq.MMQ_EINVAL  # wtype
    # unsupported combinations
    assert L.mmq_gemm(0, GOOD, GOOD, 4, 32, 64, 1, GOOD, 32, None) == mmq.MMQ_EUNSUPPORTED  # q8_0 bf16
    assert L.mmq_gemm(4, GOOD, GOOD, 4, 32, 64, 0, GOOD, 32, None) == mmq.MMQ_EUNSUPPORTED  # i8 f32
    # alignment
    assert L.mmq_quantize_act(0, BAD, 4, 64, 64, GOOD, None) == mmq.MMQ_EALIGN
    assert L.mmq_quantize_act(0, GOOD, 4, 64, 66, GOOD, None) == mmq.MMQ_EALIGN     # ldx % 4
    assert L.mmq_gemm(0, GOOD, BAD, 4, 32, 64, 0, GOOD, 32, None) == mmq.MMQ_EALIGN
    assert L.mmq_repack_weights(1, BAD, None, 32, 64, GOOD, None) == mmq.MMQ_EALIGN
    # the auxiliary input: row scales with i8_row, the grid with iq1c, NULL otherwise
    assert L.mmq_repack_weights(1, GOOD, GOOD, 32, 64, GOOD, None) == mmq.MMQ_EINVAL
    assert L.mmq_repack_weights(4, GOOD, None, 32, 64, GOOD, None) == mmq.MMQ_EINVAL
    assert L.mmq_repack_weights(5, GOOD, None, 32, 256, GOOD, None) == mmq.MMQ_EINVAL
    assert L.mmq_repack_weights(3, GOOD, GOOD, 32, 256, GOOD, None) == mmq.MMQ_EINVAL
    assert L.mmq_repack_weights(5, GOOD, GOOD, 32, 128, GOOD, None) == mmq.MMQ_EINVAL   # K % 256
    assert L.mmq_repack_weights(5, GOOD, BAD, 32, 256, GOOD, None) == mmq.MMQ_EALIGN
    assert L.mmq_repack_weights(7, GOOD, None, 32, 256, GOOD, None) == mmq.MMQ_EINVAL   # iq1s grid


def test_gemm_id_validation(mmq):
    L = mmq.lib()
    GOOD = ctypes.c_void_p(0x10000)
    ws = mmq.gemm_id_workspace_bytes(64, 512, 8)
    assert ws > 0 and ws % 256 == 0
    assert mmq.gemm_id_workspace_bytes(4, 10, 5) == 0           # top_k > E
    args = lambda wsz, ids=GOOD: (3, GOOD, 64, GOOD, ids, 512, 8, 2048, 4096, 0, GOOD, GOOD, wsz, None)
    assert L.mmq_gemm_id(*args(ws - 1)) == mmq.MMQ_EWORKSPACE
    assert L.mmq_gemm_id(*args(ws, None)) == mmq.MMQ_EINVAL
    assert L.mmq_gemm_id(4, GOOD, 64, GOOD, GOOD, 512, 8, 2048, 4096, 0, GOOD, GOOD, ws, None) == mmq.MMQ_EUNSUPPORTED
    assert L.mmq_gemm_id(3, GOOD, 64, GOOD, GOOD, 512, 8, 2048, 4096, 1, GOOD, GOOD, ws, None) == mmq.MMQ_EUNSUPPORTED


def test_act_q8_1_layout_codec(mmq):
    """Build a q8_1 act image byte by byte from the header's formulas, check that the host
    encoder produces the same bytes and that the decoders give the values back."""
    M, K = 40, 96
    o = mmq.act_region_offsets("q8_1", M, K)
    KB, KBp = 3, 8
    buf = np.zeros(mmq.act_bytes("q8_1", M, K), np.uint8)
    r = np.random.default_rng(0)
    xq = r.integers(-128, 128, (M, K)).astype(np.int8)
    xs = r.random((M, KB)).astype(np.float16).astype(np.float32)
    xsum = xq.reshape(M, KB, 32).astype(np.int64).sum(axis=2).astype(np.int32)
    for m in range(M):
        for k in range(K):
            mt, b, kk = m // 32, k // 32, k % 32
            buf[o[0] + (mt * KBp + b) * 1024 + ((kk // 16) * 32 + m % 32) * 16 + kk % 16] = xq[m, k].view(np.uint8)
        for b in range(KB):
            tdx = 4 * (((m // 32) * KBp + b) * 32 + m % 32)          # regions 1, 2: tile-major
            h = int(np.float16(xs[m, b]).view(np.uint16))
            buf[o[1] + tdx:o[1] + tdx + 4] = np.frombuffer(np.uint32(h | (h << 16)).tobytes(), np.uint8)
            buf[o[2] + tdx:o[2] + tdx + 4] = np.frombuffer(np.float32(xs[m, b] * xsum[m, b]).tobytes(), np.uint8)
            for hh in range(2):                                      # region 3: one dword per half
                g = [int(xq[m, 32 * b + 8 * j:32 * b + 8 * j + 8].astype(np.int64).sum()) for j in (2 * hh, 2 * hh + 1)]
                f = [int(np.float16(np.float32(v) * np.float32(2.0 ** -13)).view(np.uint16)) for v in g]
                gdx = 4 * (((m // 32) * KBp + b) * 64 + hh * 32 + m % 32)
                buf[o[3] + gdx:o[3] + gdx + 4] = np.frombuffer(np.uint32(f[0] | (f[1] << 16)).tobytes(), np.uint8)
    assert np.array_equal(mmq.act_q8_1_pack_host(xq, xs), buf)
    a, s, u = mmq.act_to_host(buf, M, K)
    assert np.array_equal(a, xq) and np.array_equal(s, xs) and np.array_equal(u, xsum)
    G = mmq.act_groups_host(buf, M, K)
    assert np.array_equal(G[:M, :KB], xq.reshape(M, KB, 4, 8).astype(np.int64).sum(axis=3))
    lo, hi, xsx = mmq.act_derived_host(buf, M, K)
    assert np.array_equal(lo[:M, :KB], xs) and np.array_equal(hi[:M, :KB], xs)
    assert np.array_equal(xsx[:M, :KB], xs * xsum)
    assert np.all(mmq.act_padding_host(buf, M, K) == 0)


def test_product_path_does_not_import_oracle():
    # the HIP path and the oracle share no code: no import of oracle/ from the package
    pkg = os.path.join(ROOT, "block_quantized_int8_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "mmq_oracle" not in text, f
    # and the oracle does not import the package
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c")):
            text = open(os.path.join(ROOT, "oracle", f)).read()
            assert "block_quantized_int8_amd" not in text, f


def test_act_i8_layout_roundtrip(mmq):
    """The host encoder of the per-token int8 act layout places value (m, k) where the header
    says: ((m/32)*KBp + k/32)*1024 + (((k%32)/16)*32 + m%32)*16 + k%16, and the decoder
    inverts it; padding rows/blocks and scales are zero."""
    M, K = 37, 96
    rng = np.random.default_rng(3)
    a = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    sa = rng.random(M, dtype=np.float32) + 0.5
    buf = mmq.act_i8_pack_host(a, sa)
    assert buf.size == mmq.act_bytes("i8_token", M, K)
    o = mmq.act_region_offsets("i8_token", M, K)
    KBp = 8
    for m, k in [(0, 0), (5, 17), (31, 95), (32, 0), (36, 63), (33, 40)]:
        pos = o[0] + ((m // 32) * KBp + k // 32) * 1024 + (((k % 32) // 16) * 32 + m % 32) * 16 + k % 16
        assert buf[pos].view(np.int8) == a[m, k]
    a2, sa2 = mmq.act_i8_to_host(buf, M, K)
    assert np.array_equal(a2, a) and np.array_equal(sa2, sa)
    full, sap = mmq.act_i8_to_host(buf, M, K, padded=True)
    assert full.shape == (64, KBp * 32) and not full[M:].any() and not full[:, K:].any()
    assert not sap[M:].any()


def test_binding_fails_loudly_without_the_library(monkeypatch):
    # no CPU fallback: with libmmq.so absent every call raises instead of computing elsewhere
    import block_quantized_int8_amd as mmq
    monkeypatch.setattr(mmq, "LIB_PATH", "/nonexistent/libmmq.so")
    monkeypatch.setattr(mmq, "_lib", None)
    with pytest.raises(RuntimeError):
        mmq.lib()
    with pytest.raises(RuntimeError):
        mmq.packed_bytes("q4_0", 32, 64)


def test_size_limits_rejected_before_any_launch(mmq):
    """Every size the kernels cannot address is refused on the host with MMQ_EINVAL (the pointers
    here are never dereferenced: validation returns first)."""
    L = mmq.lib()
    G = ctypes.c_void_p(0x10000)
    EINVAL = mmq.MMQ_EINVAL
    # K above 2^23 (any format, any call)
    assert L.mmq_gemm(0, G, G, 4, 32, (1 << 23) + 32, 0, G, 32, None) == EINVAL
    assert L.mmq_quantize_act(0, G, 4, (1 << 23) + 32, (1 << 23) + 32, G, None) == EINVAL
    assert mmq.act_bytes("q8_1", 4, (1 << 23) + 32) == 0
    assert mmq.packed_bytes("q4_0", 32, (1 << 23) + 32) == 0
    # M, N above 2^24
    assert L.mmq_gemm(1, G, G, (1 << 24) + 1, 32, 64, 0, G, 32, None) == EINVAL
    assert L.mmq_gemm(1, G, G, 4, (1 << 24) + 1, 64, 0, G, (1 << 24) + 1, None) == EINVAL
    # W8A8: the int32 accumulator over all of K needs K < 2^17 (prefill and decode sizes)
    assert L.mmq_gemm(4, G, G, 64, 32, 1 << 17, 1, G, 32, None) == EINVAL
    assert L.mmq_gemm(4, G, G, 4, 32, 1 << 17, 1, G, 32, None) == EINVAL
    assert L.mmq_gemm(4, G, G, 64, 32, 1 << 17, 2, G, 32, None) == EINVAL
    # debug partials: at most 2^31 values; the largest sizes must not overflow the check
    assert L.mmq_gemm(1, G, G, 1 << 12, 1 << 12, 1 << 17, 2, G, 1 << 12, None) == EINVAL
    assert L.mmq_gemm(1, G, G, 1 << 24, 1 << 24, 1 << 23, 2, G, 1 << 24, None) == EINVAL
    assert L.mmq_gemm(4, G, G, 1 << 16, 1 << 16, 64, 2, G, 1 << 16, None) == EINVAL
    # MUL_MAT_ID gather path: one expert's fragments (q8_0 N*K = 2^31 values), or the act
    # values of all T tokens (T*K = 2^31), at 2 GiB or more
    big = ctypes.c_size_t(1 << 40)
    assert L.mmq_gemm_id(0, G, 1, G, G, 8, 1, 1 << 17, 1 << 14, 0, G, G, big, None) == EINVAL
    assert L.mmq_gemm_id(0, G, 1, G, G, 1 << 17, 1, 32, 1 << 14, 0, G, G, big, None) == EINVAL
    # T * top_k above 2^24
    assert L.mmq_gemm_id(0, G, 8, G, G, 1 << 22, 8, 32, 64, 0, G, G, big, None) == EINVAL
    assert mmq.gemm_id_workspace_bytes(8, 1 << 22, 8) == 0


def test_noalloc_gemm_id_refuses_problems_beyond_its_scratch(mmq):
    """mmq_gemm_id_noalloc takes its workspace from a 1 MiB static array: a problem that needs
    more is refused with MMQ_EWORKSPACE before anything is enqueued (no device is touched)."""
    L = mmq.lib()
    G = ctypes.c_void_p(0x10000)
    assert mmq.gemm_id_noalloc_max_workspace_bytes() == 1 << 20
    assert mmq.gemm_id_workspace_bytes(64, 40000, 8) > 1 << 20
    assert L.mmq_gemm_id_noalloc(3, G, 64, G, G, 40000, 8, 256, 512, 0, G, None) == mmq.MMQ_EWORKSPACE
    # argument errors come first, as in mmq_gemm_id
    assert L.mmq_gemm_id_noalloc(3, None, 64, G, G, 512, 8, 256, 512, 0, G, None) == mmq.MMQ_EINVAL
    assert L.mmq_gemm_id_noalloc(4, G, 64, G, G, 512, 8, 256, 512, 0, G, None) == mmq.MMQ_EUNSUPPORTED
