"""Shared output checks of the GPU parity tests (a helper module, not a test file).

Two bars for every f32 output of the block-scaled contraction:

1. The pages' parity gate (minfer R1 section 4: max diff < 1e-3), read as
   max|gpu - ref| / max|ref| <= 1e-3 against the f64 definition (`oracle.gemm_f64`: both
   operands dequantised with the formats' defining formulas, one f64 matmul).

2. A rounding bound derived from the arithmetic, against the per-block C oracle
   (`oracle.gemm_c`, double accumulation rounded once to f32). Every per-block integer dot is
   exact on both sides and every scale product is exact or rounded once, so the GPU may
   differ only by rounding the per-block terms t into its f32 accumulators: each of the at
   most A additions rounds with a relative error of at most u = 2^-24 of a partial sum, and
   every partial sum is bounded by abs = sum |t| (`oracle.gemm_abs`). Hence, per output,
       |gpu - ref| <= (A + 4) * u * abs + u * |ref| + A * 2^-124,
   with A = 2 * K/32 + 16 (one FMA per block, or per half-block for q6_K; the q4_K min term
   adds at most one rounding per block; the small-batch kernel adds up to 16 wave partial
   sums), +4 for a scale product rounded once or twice (q4_K / q6_K: d*sc as two f16 halves
   times xs), u * |ref| for the oracle's own final rounding, and the last term for
   accumulators that fall into the f32 subnormal range (2^-150 per rounding, times the
   largest power-of-two scale, 2^26, the kernels apply in the epilogue). On top, the
   normwise error must stay within max(1e-5, 2 u sqrt(K/32)) (the kernels reach ~1e-7 at
   K of a few thousand; rounding errors of a sequential f32 sum of K/32 terms drift like
   u sqrt(K/32) relative to its result, 1.3e-5 measured at K = 2^23): a defect of the scale
   path well below the pages' 1e-3 - for instance dropping the low half of q4_K's exact
   f16 split of d*sc, an error of up to 2^-12 per term - fails one of the two.
"""
import numpy as np

PAGES_GATE = 1e-3
NORMWISE_GATE = 1e-5
U = 2.0 ** -24


def rel(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-300))


def normwise_gate(K):
    return max(NORMWISE_GATE, 2 * U * np.sqrt(K // 32))


def rounding_bound(ref_c, absum, K):
    A = 2 * (K // 32) + 16
    return (A + 4) * U * absum + U * np.abs(np.asarray(ref_c, np.float64)) + A * 2.0 ** -124


def check_tight(got, ref_c, absum, K, what="", per_row=False):
    """Bar 2 on outputs `got` against the C oracle's `ref_c` and the magnitudes `absum`
    (arrays of one shape). per_row: the normwise gate per row (rows of very different scale)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref_c, np.float64)
    err = np.abs(got - ref)
    bound = rounding_bound(ref, absum, K)
    bad = err > bound
    assert not bad.any(), (what, int(bad.sum()), float(err[bad].max()), float(bound[bad].min()))
    if per_row:
        for i in range(got.shape[0]):
            r = rel(got[i], ref[i]) if np.any(ref[i]) else float(np.max(err[i]))
            assert r <= normwise_gate(K), (what, i, r)
        return
    r = rel(got, ref)
    assert r <= normwise_gate(K), (what, r)
    return r


def check_f32(orc, got, fmt, raw, N, K, xq, xs, xsum, rows=None, cols=None, grid=None, what="",
              per_row=False):
    """Both bars on `got` = outputs for activation rows `rows` (all if None) and weight rows
    `cols` (all if None) of the dense product act x W^T. xq, xs, xsum: the oracle's q8_1 of
    all rows. Returns (pages' relative error, normwise error vs the C oracle)."""
    got = np.asarray(got, np.float64)
    ref = orc.gemm_f64(fmt, raw, N, K, xq if rows is None else xq[rows], xs if rows is None else xs[rows],
                       cols=cols, grid=grid)
    r1 = rel(got, ref) if not per_row else max(
        rel(got[i], ref[i]) if np.any(ref[i]) else 0.0 for i in range(got.shape[0]))
    assert r1 <= PAGES_GATE, (what, r1)
    sel = slice(None) if rows is None else rows
    xq2, xs2, xsum2 = np.ascontiguousarray(xq[sel]), np.ascontiguousarray(xs[sel]), np.ascontiguousarray(xsum[sel])
    ref_c = orc.gemm_c(fmt, raw, N, K, xq2, xs2, xsum2, grid=grid).astype(np.float64)
    absum = orc.gemm_abs(fmt, raw, N, K, xq2, xs2, xsum2, grid=grid)
    if cols is not None:
        ref_c, absum = ref_c[:, cols], absum[:, cols]
    r2 = check_tight(got, ref_c, absum, K, what, per_row=per_row)
    return r1, r2


def check_moe(orc, got, fmt, raw_e, N, K, xq, xs, xsum, ids, grid=None, experts=None, cols=None, what=""):
    """Bar 2 on MUL_MAT_ID outputs got [T, top_k, N] (columns `cols` if given, then got is
    [T, top_k, len(cols)]): every pair (t, j) with a valid id is the dense product of token t
    with expert ids[t, j]; all pairs of each expert (or of the experts listed) are checked
    against the per-block C oracle. Returns the normwise error over the checked pairs."""
    raw_e = np.asarray(raw_e, np.uint8)
    E = raw_e.shape[0]
    g_all, r_all = [], []
    for e in (range(E) if experts is None else experts):
        tt, jj = np.nonzero(ids == e)
        if len(tt) == 0:
            continue
        q = (np.ascontiguousarray(xq[tt]), np.ascontiguousarray(xs[tt]), np.ascontiguousarray(xsum[tt]))
        ref_c = orc.gemm_c(fmt, raw_e[e], N, K, *q, grid=grid).astype(np.float64)
        absum = orc.gemm_abs(fmt, raw_e[e], N, K, *q, grid=grid)
        if cols is not None:
            ref_c, absum = ref_c[:, cols], absum[:, cols]
        g = np.asarray(got[tt, jj], np.float64)
        err = np.abs(g - ref_c)
        bound = rounding_bound(ref_c, absum, K)
        bad = err > bound
        assert not bad.any(), (what, e, int(bad.sum()), float(err[bad].max()))
        g_all.append(g)
        r_all.append(ref_c)
    r = rel(np.concatenate(g_all), np.concatenate(r_all))
    assert r <= normwise_gate(K), (what, r)
    return r


def block_sums(xq):
    """xsum of a q8_1 activation from its values: the integer sum of every 32-value block."""
    xq = np.asarray(xq)
    return xq.reshape(xq.shape[0], -1, 32).astype(np.int64).sum(axis=2).astype(np.int32)
