"""A NumPy model of the packed weight layout that mmq_repack_weights documents (include/mmq.h
for the raw formats; the panel layout: 32-row tiles, one fragment per (tile, 32-value block)
in the int8 matrix-core operand order, one scale dword per (row, block), tile-major). Test code
only: the GPU tests compare the library's repack with this model byte for byte (metainfer
"INT8 W8A8 GEMM - Prefill", section 3.2: packs validated by exact comparison against a
simulation of the index map), and tests/test_packmodel.py pins the model on the CPU by
decoding it back and comparing with the oracle's decoder.

Layout, with Np = N rounded up to 32, NT = Np/32, KB = K/32, KBp = KB rounded up to 8:
  region 0 (offset 0): fragments [NT][KBp][FB]; lane L = 32h + r (r < 32, h < 2) of fragment
      (nt, b) holds row n = 32nt + r, values k = 16h..16h+15 of block b:
        q8_0, i8_row, q6_K  FB = 1024: 16 int8 per lane (q6_K: q - 32)
        q4_0                FB = 512: dwords X0, X1; byte i of X0 has value 16h+i in its high
                            nibble and 16h+4+i in its low nibble (X1: 16h+8+i, 16h+12+i), each
                            stored as nib ^ 8 (the 4-bit two's complement of nib - 8)
        q4_K                FB = 512: as q4_0 with unsigned nibbles and the halves swapped
                            (byte i of X0: low nibble 16h+i, high 16h+4+i)
        iq1t                FB = 256: one dword, value i of the lane at bits 8(i%4) + 2(i/4),
                            the 2-bit code c = g+1
        iq1c, iq1s          FB = 256: one dword W = ia << 2 | meta << 13 | ib << 20, ia and ib the
                            11-bit grid indices of the lane's 8-value groups 2h and 2h+1, meta =
                            s | sigma_a << 3 | sigma_b << 4 (iq1s: its per-32 s and sign twice)
  region 1 (256-aligned, after region 0): one dword per (row n, block b) at
      ((nt*KBp + b)*32 + r)*4; i8_row instead: f32 sw[n] for n < Np
        q8_0, q4_0   f16 d | 0
        q4_K         hi | lo << 16 with hi = f16(d*sc) (nearest even), lo = f16(d*sc - hi)
        q6_K         the same split of d*sc for the block's first 16 values
        iq1t         f16 d | meta0 << 16 | meta1 << 24, meta_h = s_h | sigma_a << 3 | sigma_b << 4
                     for the block's 16-value half h (its sub-scale and its two 8-value groups'
                     sign bits)
        iq1c, iq1s   instead f16 d of the row's super-block per (row n, 4-block group g = b/4)
                     at ((nt*(KBp/4) + g)*32 + r)*2
  region 2 (q4_K, q6_K; 256-aligned, after region 1), indexed like region 1:
        q4_K         f32 -dmin*m
        q6_K         the hi | lo split of d*sc for the block's last 16 values
        iq1c, iq1s   the grid: 2048 dwords, entry i = the 8 codes of index i with code j at bits
                     8(j%4) + 2(j/4)
  Every byte of a padding row (n >= N) or padding block (b >= KB) is zero.
"""
import numpy as np

FB = {"q8_0": 1024, "q4_0": 512, "q4_K": 512, "iq1t": 256, "q6_K": 1024, "i8_row": 1024, "iq1c": 256,
      "iq1s": 256}
GRIDDED = ("iq1c", "iq1s")


def _ru(a, b):
    return (a + b - 1) // b * b


def dims(N, K):
    Np = _ru(N, 32)
    KB = K // 32
    return Np, Np // 32, KB, _ru(KB, 8)


def offsets(fmt, N, K):
    Np, NT, KB, KBp = dims(N, K)
    scale = _ru(NT * KBp * FB[fmt], 256)
    sb = Np * 4 if fmt == "i8_row" else Np * (KBp // 4) * 2 if fmt in GRIDDED else Np * KBp * 4
    mn = scale + _ru(sb, 256)
    total = mn + (_ru(Np * KBp * 4, 256) if fmt in ("q4_K", "q6_K") else 2048 * 4 if fmt in GRIDDED else 0)
    return scale, mn, total


def spread(entry):
    """A grid entry's 8 codes (value j at bits 2j) moved to bits 8(j%4) + 2(j/4)."""
    e = np.asarray(entry, np.uint32)
    w = np.zeros(e.shape, np.uint32)
    for j in range(8):
        w |= ((e >> np.uint32(2 * j)) & np.uint32(3)) << np.uint32(8 * (j & 3) + 2 * (j >> 2))
    return w


def _gridded(fmt, raw, N, K):
    """Per (n, block, half): W; per (n, super-block): d bits."""
    raw = np.asarray(raw, np.uint8).reshape(N, -1)
    SB = K // 256
    if fmt == "iq1c":
        b = raw.reshape(N, SB, 56)
        qh = np.stack([b[..., 32:48] & 0xF, b[..., 32:48] >> 4], axis=-1).reshape(N, SB, 32).astype(np.uint32)
        idx = b[..., 0:32].astype(np.uint32) | ((qh & 7) << 8)                            # [N, SB, 32 groups]
        sg = qh >> 3
        sbits = np.unpackbits(b[..., 48:54], axis=-1, bitorder="little")[..., :48].reshape(N, SB, 16, 3)
        s16 = (sbits.astype(np.uint32) * np.array([1, 2, 4], np.uint32)).sum(-1)         # [N, SB, 16 halves]
        d = (b[..., 54].astype(np.uint32) | (b[..., 55].astype(np.uint32) << 8))
    else:
        b = raw.reshape(N, SB, 50)
        qh = (b[..., 34:50:2].astype(np.uint32) | (b[..., 35:50:2].astype(np.uint32) << 8))   # [N, SB, 8]
        hi = np.stack([(qh >> (3 * j)) & 7 for j in range(4)], axis=-1)                      # [N, SB, 8, 4]
        idx = (b[..., 2:34].astype(np.uint32).reshape(N, SB, 8, 4) | (hi << 8)).reshape(N, SB, 32)
        sg = np.repeat((qh >> 15) & 1, 4, axis=-1)
        s16 = np.repeat((qh >> 12) & 7, 2, axis=-1)
        d = (b[..., 0].astype(np.uint32) | (b[..., 1].astype(np.uint32) << 8))
    meta = s16 | (sg[..., 0::2] << 3) | (sg[..., 1::2] << 4)                              # per half
    W = (idx[..., 0::2] << 2) | (meta << 13) | (idx[..., 1::2] << 20)                     # [N, SB, 16 halves]
    return W.reshape(N, K // 32, 2), d


def _f16_bits(v):
    return np.asarray(v, np.float32).astype(np.float16).view(np.uint16).astype(np.uint32)


def _split(ds):
    """exact f16 pair of an f32 value: hi = f16(ds), lo = f16(ds - hi)"""
    ds = np.asarray(ds, np.float32)
    hi = ds.astype(np.float16)
    lo = (ds - hi.astype(np.float32)).astype(np.float16)
    return hi.view(np.uint16).astype(np.uint32) | (lo.view(np.uint16).astype(np.uint32) << 16)


def _values(fmt, raw, N, K):
    """Per (n, k) the lane value the layout stores (q8_0 q, q4_0 / q4_K nib, iq1t code,
    q6_K q - 32) and per (n, block) the scale dword(s) / min."""
    KB = K // 32
    raw = np.asarray(raw, np.uint8).reshape(N, -1)
    sc1 = np.zeros((N, KB), np.uint32)
    sc2 = np.zeros((N, KB), np.uint32)
    if fmt == "q8_0":
        b = raw.reshape(N, KB, 34)
        v = b[..., 2:].astype(np.int64)
        sc1 = (b[..., 0].astype(np.uint32) | (b[..., 1].astype(np.uint32) << 8))
        return v.reshape(N, K), sc1, sc2
    if fmt == "q4_0":
        b = raw.reshape(N, KB, 18)
        qs = b[..., 2:].astype(np.int64)
        v = np.concatenate([qs & 15, qs >> 4], axis=-1)
        sc1 = (b[..., 0].astype(np.uint32) | (b[..., 1].astype(np.uint32) << 8))
        return v.reshape(N, K), sc1, sc2
    if fmt == "q4_K":
        b = raw.reshape(N, K // 256, 144)
        d = b[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float32)
        dmin = b[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float32)
        scw = np.zeros(b.shape[:2], np.uint64)
        mw = np.zeros(b.shape[:2], np.uint64)
        for i in range(6):
            scw |= b[..., 4 + i].astype(np.uint64) << np.uint64(8 * i)
            mw |= b[..., 10 + i].astype(np.uint64) << np.uint64(8 * i)
        j = np.arange(8, dtype=np.uint64)
        sc = ((scw[..., None] >> (np.uint64(6) * j)) & np.uint64(63)).astype(np.float32)
        mm = ((mw[..., None] >> (np.uint64(6) * j)) & np.uint64(63)).astype(np.float32)
        qs = b[..., 16:].reshape(N, K // 256, 8, 16).astype(np.int64)
        v = np.concatenate([qs & 15, qs >> 4], axis=-1).reshape(N, K)
        sc1 = _split((d[..., None] * sc).reshape(N, KB))
        sc2 = (-(dmin[..., None] * mm)).astype(np.float32).reshape(N, KB).view(np.uint32)
        return v, sc1, sc2
    if fmt == "iq1t":
        b = raw.reshape(N, K // 256, 76)
        codes = np.stack([(b[..., :64] >> (2 * j)) & 3 for j in range(4)], axis=-1).reshape(N, K // 256, 256)
        sbits = np.unpackbits(b[..., 64:70], axis=-1, bitorder="little")[..., :48].reshape(N, K // 256, 16, 3)
        s = (sbits.astype(np.uint32) * np.array([1, 2, 4], np.uint32)).sum(-1)          # [N, sb, 16]
        sgn = np.unpackbits(b[..., 70:74], axis=-1, bitorder="little").reshape(N, K // 256, 32).astype(np.uint32)
        d = (b[..., 74].astype(np.uint32) | (b[..., 75].astype(np.uint32) << 8))
        meta = s | (sgn[..., 0::2] << 3) | (sgn[..., 1::2] << 4)                          # per 16: groups 2h', 2h'+1
        meta = meta.reshape(N, K // 256, 8, 2)
        sc1 = (d[..., None] | (meta[..., 0] << 16) | (meta[..., 1] << 24)).reshape(N, KB)
        return codes.reshape(N, K).astype(np.int64), sc1, sc2
    if fmt == "q6_K":
        b = raw.reshape(N, K // 256, 210)
        ql = b[..., 0:128].reshape(N, K // 256, 8, 16).astype(np.int64)
        lo = np.concatenate([ql & 15, ql >> 4], axis=-1)
        qh = b[..., 128:192].reshape(N, K // 256, 8, 1, 8).astype(np.int64)
        hi = ((qh >> (2 * np.arange(4)[:, None])) & 3).reshape(N, K // 256, 8, 32)
        v = ((lo | (hi << 4)) - 32).reshape(N, K)
        sc = b[..., 192:208].view(np.int8).astype(np.float32).reshape(N, K // 256, 8, 2)
        d = b[..., 208:210].copy().view(np.float16)[..., 0].astype(np.float32)
        sc1 = _split((d[..., None] * sc[..., 0]).reshape(N, KB))
        sc2 = _split((d[..., None] * sc[..., 1]).reshape(N, KB))
        return v, sc1, sc2
    raise ValueError(fmt)


def _lane_bytes(fmt, lanes):
    """lanes [..., 16] int64 lane values -> [..., FB/64] bytes"""
    if fmt in ("q8_0", "q6_K", "i8_row"):
        return (lanes & 0xFF).astype(np.uint8)
    if fmt in ("q4_0", "q4_K"):
        t = (lanes ^ 8) if fmt == "q4_0" else lanes
        out = np.zeros(lanes.shape[:-1] + (8,), np.uint8)
        for i in range(4):
            for x in range(2):                       # X0 (values 0-7), X1 (values 8-15)
                a, c = t[..., 8 * x + i], t[..., 8 * x + 4 + i]
                out[..., 4 * x + i] = ((a << 4) | c) if fmt == "q4_0" else (a | (c << 4))
        return out
    if fmt == "iq1t":
        w = np.zeros(lanes.shape[:-1], np.uint32)
        for i in range(16):
            w |= (lanes[..., i].astype(np.uint32) & 3) << np.uint32(8 * (i & 3) + 2 * (i >> 2))
        return w[..., None].view(np.uint8).reshape(lanes.shape[:-1] + (4,))
    raise ValueError(fmt)


def pack(fmt, raw, N, K, row_scale=None, fill=0):
    """The packed buffer (uint8) the layout above prescribes for raw weight rows (row_scale:
    the f32 row scales of i8_row, the grid of iq1c / iq1s). The alignment gaps between regions
    (not written by the repack) hold `fill`."""
    Np, NT, KB, KBp = dims(N, K)
    scale_off, min_off, total = offsets(fmt, N, K)
    buf = np.full(total, fill, np.uint8)
    if fmt in GRIDDED:
        W, d = _gridded(fmt, raw, N, K)
        full = np.zeros((Np, KBp, 2), np.uint32)
        full[:N, :KB] = W
        buf[:NT * KBp * 256] = full.reshape(NT, 32, KBp, 2).transpose(0, 2, 3, 1).reshape(-1).view(np.uint8)
        dd = np.zeros((Np, KBp // 4), np.uint16)
        dd[:N, :KB // 4] = np.repeat(d, 2, axis=1)
        buf[scale_off:scale_off + Np * (KBp // 4) * 2] = dd.reshape(NT, 32, KBp // 4).transpose(0, 2, 1).reshape(-1).view(np.uint8)
        buf[min_off:min_off + 8192] = spread(row_scale).view(np.uint8)         # row_scale: the grid
        return buf
    if fmt == "i8_row":
        v = np.asarray(raw, np.int8).reshape(N, K).astype(np.int64)
        sc1 = sc2 = None
    else:
        v, sc1, sc2 = _values(fmt, raw, N, K)
    full = np.zeros((Np, KBp * 32), np.int64)
    full[:N, :K] = v
    lanes = full.reshape(NT, 32, KBp, 2, 16).transpose(0, 2, 3, 1, 4)        # [nt, b, h, r, 16]
    fb = _lane_bytes(fmt, lanes)
    live = np.zeros((Np, KBp * 32), bool)
    live[:N, :K] = True
    lv = live.reshape(NT, 32, KBp, 2, 16).transpose(0, 2, 3, 1, 4)[..., 0]
    fb = fb * lv[..., None]
    buf[:NT * KBp * FB[fmt]] = fb.reshape(-1)
    if fmt == "i8_row":
        sw = np.zeros(Np, np.float32)
        sw[:N] = np.asarray(row_scale, np.float32)
        buf[scale_off:scale_off + 4 * Np] = sw.view(np.uint8)
        return buf

    def tile_major(a):
        f = np.zeros((Np, KBp), np.uint32)
        f[:N, :KB] = a
        return f.reshape(NT, 32, KBp).transpose(0, 2, 1).reshape(-1).view(np.uint8)
    buf[scale_off:scale_off + Np * KBp * 4] = tile_major(sc1)
    if fmt in ("q4_K", "q6_K"):
        buf[min_off:min_off + Np * KBp * 4] = tile_major(sc2)
    return buf


def unpack_values(fmt, buf, N, K):
    """Inverse of the fragment map: the lane values [N, K] a packed buffer holds (q4_0 back to
    nib - 8, q4_K nib, iq1t 8g +- 1 needs the signs, so iq1t returns the codes c)."""
    Np, NT, KB, KBp = dims(N, K)
    fbytes = np.asarray(buf, np.uint8)[:NT * KBp * FB[fmt]].reshape(NT, KBp, 2, 32, FB[fmt] // 64)
    if fmt in ("q8_0", "q6_K", "i8_row"):
        lanes = fbytes.view(np.int8).astype(np.int64)
    elif fmt in ("q4_0", "q4_K"):
        lanes = np.zeros(fbytes.shape[:-1] + (16,), np.int64)
        for i in range(4):
            for x in range(2):
                byte = fbytes[..., 4 * x + i].astype(np.int64)
                hi_n, lo_n = byte >> 4, byte & 15
                if fmt == "q4_0":
                    lanes[..., 8 * x + i], lanes[..., 8 * x + 4 + i] = (hi_n ^ 8) - 8, (lo_n ^ 8) - 8
                else:
                    lanes[..., 8 * x + i], lanes[..., 8 * x + 4 + i] = lo_n, hi_n
    else:
        w = fbytes.copy().view(np.uint32)[..., 0].astype(np.int64)
        lanes = np.stack([(w >> (8 * (i & 3) + 2 * (i >> 2))) & 3 for i in range(16)], axis=-1)
    full = lanes.transpose(0, 3, 1, 2, 4).reshape(Np, KBp * 32)
    return full[:N, :K]


def scale_dwords(fmt, buf, N, K, region=1):
    """Region 1 (or 2) as uint32 [N, KB] (row-major)."""
    Np, NT, KB, KBp = dims(N, K)
    scale_off, min_off, _ = offsets(fmt, N, K)
    off = scale_off if region == 1 else min_off
    a = np.asarray(buf, np.uint8)[off:off + Np * KBp * 4].copy().view(np.uint32)
    return a.reshape(NT, KBp, 32).transpose(0, 2, 1).reshape(Np, KBp)[:N, :KB]


def gridded_words(fmt, buf, N, K):
    """iq1c / iq1s: the lane dwords W as uint32 [N, K/32, 2] and the d bits [N, K/256] (the
    copies of each super-block's d in its two 4-block groups must agree)."""
    Np, NT, KB, KBp = dims(N, K)
    scale_off, _, _ = offsets(fmt, N, K)
    b = np.asarray(buf, np.uint8)
    W = b[:NT * KBp * 256].copy().view(np.uint32).reshape(NT, KBp, 2, 32).transpose(0, 3, 1, 2).reshape(Np, KBp, 2)
    d = b[scale_off:scale_off + Np * (KBp // 4) * 2].copy().view(np.uint16).reshape(NT, KBp // 4, 32)
    d = d.transpose(0, 2, 1).reshape(Np, KBp // 4)[:N, :KB // 4]
    assert np.array_equal(d[:, 0::2], d[:, 1::2])            # both 4-block groups of a super-block
    return W[:N, :KB], d[:, 0::2]
