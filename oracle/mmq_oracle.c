/*
 * mmq_oracle.c - plain, slow CPU oracle for the prefill MMQ contraction.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path (the HIP library and
 * its Python binding) may include, link, load or call this file. Only the
 * tests, the smoke check and the bench's CPU-baseline leg use it.
 *
 * It shares no code, header, table or constant with the GPU path. Every
 * function below is a direct transcription of a definition from the MMQ
 * pages, restated in this project's own words:
 *
 *  - "08 . R1 - int8 MMQ prefill GEMM" (minfer), section 3.2, the CPU
 *    reference of the parity test: per 32-value block, d = max|x|/127 in f32,
 *    the stored scale is d rounded to f16, q = round-half-even(x * (1/d))
 *    clamped to [-128,127], and the block's integer sum is kept. Section 2.2
 *    gives the rank-1 min term: sum(w*q) = ds*sum(nib*q) - dmin*sum(q).
 *  - "A Negative Result on int8 Tensor-Core MMQ" (Hanzo), section 2: the
 *    contraction out[m,n] = sum over 32-blocks of (xs*wd) * sum(xq*wq).
 *  - llama.cpp PR #304 "CUDA: add IQ1_M to MMQ", description: an IQ1_M value
 *    is d*(2s+1)*(g+delta); 8(g+delta) = 8g +- 1 and the per-16 scale becomes
 *    d(2s+1)/8. In the codebook forms the ternary g of 8 values come from one
 *    grid entry named by an 11-bit index (the grid itself is an input here):
 *    IQ1_M with s per 16 and delta per 8 values, IQ1_S with both per 32.
 *  - minfer R1 sections 2.2 and 3.3: q6_K values are a 6-bit grid 0..63 moved
 *    to the signed domain by -32, with an int8 scale per 16 values; a 32-value
 *    block is two 16-value halves with separate integer sums, each rescaled by
 *    its own d*sc.
 *  - "INT8 W8A8 GEMM - Prefill" (metainfer), section 1: int8 activations with
 *    a per-token f32 scale, int8 weights with a per-channel f32 scale, int32
 *    accumulation, epilogue fragment -> scale -> bf16, no bias.
 *
 * The raw weight byte layouts are this project's own (the pages give
 * semantics, not bytes); they are documented in gen/__init__.py.
 *
 * Precision: the quantiser works in f32 because the pages fix it; integer
 * partial sums are exact (int64, checked to fit int32); the f32 outputs are
 * accumulated in double; the W8A8 epilogue is the pages' f32 two-multiply
 * order rounded to bf16 (round-to-nearest-even).
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_Q8_0 0
#define ORC_Q4_0 1
#define ORC_Q4_K 2
#define ORC_IQ1T 3
#define ORC_IQ1C 4
#define ORC_Q6_K 5
#define ORC_IQ1S 6

/* ---------------------------------------------------------------- scalars */

/* IEEE binary16 -> binary32, exact (handles zero, subnormal, inf, nan). */
float orc_half_to_float(uint16_t h) {
    uint32_t sign = (uint32_t)(h >> 15) & 1u;
    uint32_t expo = (uint32_t)(h >> 10) & 0x1Fu;
    uint32_t mant = (uint32_t)h & 0x3FFu;
    float mag;
    if (expo == 0) {
        mag = ldexpf((float)mant, -24);                 /* subnormal or zero */
    } else if (expo == 31) {
        mag = mant ? NAN : INFINITY;
    } else {
        mag = ldexpf((float)(mant | 0x400u), (int)expo - 25);
    }
    return sign ? -mag : mag;
}

/* binary32 -> binary16 with round-to-nearest-even (finite inputs; overflow -> inf). */
uint16_t orc_float_to_half(float f) {
    uint32_t sign = signbit(f) ? 0x8000u : 0u;
    double a = fabs((double)f);
    if (isnan(f)) return (uint16_t)(sign | 0x7E00u);
    if (a == 0.0) return (uint16_t)sign;
    int e;
    (void)frexp(a, &e);                                /* a = m * 2^e, m in [0.5,1) */
    int ulp_exp = e - 11;                              /* 11 significant bits */
    if (ulp_exp < -24) ulp_exp = -24;                  /* subnormal spacing */
    double units = a / ldexp(1.0, ulp_exp);            /* exact: a has 24 bits */
    double r = nearbyint(units);                       /* default mode: ties to even */
    double v = r * ldexp(1.0, ulp_exp);
    if (v >= 65520.0) return (uint16_t)(sign | 0x7C00u);
    /* re-encode v exactly */
    if (v < ldexp(1.0, -14)) {                         /* subnormal (or rounds up to min normal) */
        uint32_t m = (uint32_t)(v / ldexp(1.0, -24));
        return (uint16_t)(sign | m);                   /* m == 1024 encodes 2^-14 correctly */
    }
    int ve;
    double vm = frexp(v, &ve);                         /* v = vm * 2^ve, vm in [0.5,1) */
    uint32_t expo = (uint32_t)(ve - 1 + 15);
    uint32_t mant = (uint32_t)(vm * 2048.0) - 1024u;
    return (uint16_t)(sign | (expo << 10) | mant);
}

/* binary32 -> bfloat16 with round-to-nearest-even (finite inputs). */
uint16_t orc_float_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x40u);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* ------------------------------------------------------ activation quantiser */

/* q8_1 (the activation format of the contraction).
 *
 * Definition (minfer R1 section 3.2 gives it as the parity test's CPU reference; section 2.2
 * adds the block sum). For a block B of 32 values:
 *     d(B)   = max_{i in B} |x_i| / 127                       (one f32 division)
 *     inv(B) = 0 if d(B) = 0, else 1/d(B) in f32, taken as the largest finite f32 when it
 *              overflows (d(B) below 2^-128): the pages leave that case open, and this keeps
 *              0 * inv = 0 and |x * inv| <= 127 (1 + 2^-23) for every x of the block
 *     q_i    = the integer nearest x_i * inv(B) (ties to even), limited to [-128, 127]
 *     xs(B)  = d(B) rounded to f16 (nearest even), carried as f32;  xsum(B) = sum of the q_i.
 * Computed below in three passes over each row: the block scales, then every value, then the
 * per-block sums. Outputs are row-major: xq [M][K], xs [M][K/32], xsum [M][K/32]. */
static float q8_block_amax(const float* v) {
    float a = 0.0f;
    for (int i = 0; i < 32; ++i) a = fmaxf(a, fabsf(v[i]));
    return a;
}

static float q8_inverse(float d) {
    if (d == 0.0f) return 0.0f;
    const float r = 1.0f / d;
    return isinf(r) ? FLT_MAX : r;
}

static int8_t q8_value(float x, float inv) {
    const float t = nearbyintf(x * inv);            /* default rounding: ties to even */
    return (int8_t)(t > 127.0f ? 127 : t < -128.0f ? -128 : (int)t);
}

void orc_quantize_q8_1(const float* x, int64_t M, int64_t K, int64_t ldx,
                       int8_t* xq, float* xs, int32_t* xsum) {
    const int64_t KB = K / 32;
#pragma omp parallel
    {
        float* dk = (float*)malloc(sizeof(float) * (size_t)(KB > 0 ? KB : 1));
#pragma omp for schedule(static)
        for (int64_t m = 0; m < M; ++m) {
            const float* row = x + m * ldx;
            for (int64_t b = 0; b < KB; ++b) dk[b] = q8_block_amax(row + 32 * b) / 127.0f;
            for (int64_t k = 0; k < K; ++k) xq[m * K + k] = q8_value(row[k], q8_inverse(dk[k / 32]));
            for (int64_t b = 0; b < KB; ++b) {
                int32_t total = 0;
                for (int64_t k = 32 * b; k < 32 * b + 32; ++k) total += xq[m * K + k];
                xsum[m * KB + b] = total;
                xs[m * KB + b] = orc_half_to_float(orc_float_to_half(dk[b]));
            }
        }
        free(dk);
    }
}

/* Per-token int8 (W8A8 activations): the same steps with the block being the
 * whole row and the scale kept in f32 (not rounded to f16).                  */
void orc_quantize_i8_token(const float* x, int64_t M, int64_t K, int64_t ldx,
                           int8_t* a, float* sa) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const float* row = x + m * ldx;
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float v = fabsf(row[k]);
            if (v > amax) amax = v;
        }
        float d = amax / 127.0f;
        float inv = q8_inverse(d);
        for (int64_t k = 0; k < K; ++k) a[m * K + k] = q8_value(row[k], inv);
        sa[m] = d;
    }
}

/* ------------------------------------------------------------ weight decode */

/* Decode one weight row into:
 *   wq[K]      - the integer that enters the int8 dot for each value
 *                (q8_0: q; q4_0: nib-8; q4_K: nib (unsigned); iq1t/iq1c: 8g+sigma;
 *                q6_K: q-32)
 *   wd[K/16]   - the f32 scale multiplying each 16-value half of the dot
 *                (q8_0/q4_0: d; q4_K: d*sc; iq1t/iq1c: d*(2s+1)/8; q6_K: d*sc_h)
 *   wm[K/32]   - the f32 coefficient of the activation block sum
 *                (q4_K: -dmin*m, others 0)
 *   mult[K/16] - the integer factor of each half in the folded block partial
 *                (iq1t/iq1c: 2s+1, others 1)
 * Every scale here is exact in f32 (an f16 times a small integer, or /8).
 * grid: the iq1c codebook (2048 entries of eight 2-bit codes), else unused.
 * Returns 0, or -1 if an iq1c grid entry holds the invalid code 3.          */
static int decode_row(int fmt, const uint8_t* row, int64_t K, const uint16_t* grid,
                      int16_t* wq, float* wd, float* wm, int16_t* mult) {
    const int64_t KB = K / 32;
    int bad = 0;
    for (int64_t b = 0; b < KB; ++b) wm[b] = 0.0f;
    for (int64_t h = 0; h < K / 16; ++h) mult[h] = 1;
    if (fmt == ORC_Q8_0) {
        for (int64_t b = 0; b < KB; ++b) {
            const uint8_t* blk = row + b * 34;
            float d = orc_half_to_float(rd16(blk));
            for (int i = 0; i < 32; ++i) wq[b * 32 + i] = (int8_t)blk[2 + i];
            wd[2 * b] = d;
            wd[2 * b + 1] = d;
        }
    } else if (fmt == ORC_Q4_0) {
        for (int64_t b = 0; b < KB; ++b) {
            const uint8_t* blk = row + b * 18;
            float d = orc_half_to_float(rd16(blk));
            for (int j = 0; j < 16; ++j) {
                wq[b * 32 + j] = (int16_t)((blk[2 + j] & 0xF) - 8);
                wq[b * 32 + 16 + j] = (int16_t)((blk[2 + j] >> 4) - 8);
            }
            wd[2 * b] = d;
            wd[2 * b + 1] = d;
        }
    } else if (fmt == ORC_Q4_K) {
        for (int64_t sb = 0; sb < K / 256; ++sb) {
            const uint8_t* blk = row + sb * 144;
            float d = orc_half_to_float(rd16(blk));
            float dmin = orc_half_to_float(rd16(blk + 2));
            uint64_t scw = 0, mw = 0;
            for (int i = 0; i < 6; ++i) {
                scw |= (uint64_t)blk[4 + i] << (8 * i);
                mw |= (uint64_t)blk[10 + i] << (8 * i);
            }
            const uint8_t* qs = blk + 16;
            for (int j = 0; j < 8; ++j) {
                int sc = (int)((scw >> (6 * j)) & 63u);
                int mm = (int)((mw >> (6 * j)) & 63u);
                int64_t b = sb * 8 + j;
                for (int i = 0; i < 16; ++i) {
                    wq[b * 32 + i] = (int16_t)(qs[16 * j + i] & 0xF);
                    wq[b * 32 + 16 + i] = (int16_t)(qs[16 * j + i] >> 4);
                }
                wd[2 * b] = d * (float)sc;
                wd[2 * b + 1] = d * (float)sc;
                wm[b] = -(dmin * (float)mm);
            }
        }
    } else if (fmt == ORC_IQ1T) {
        for (int64_t sb = 0; sb < K / 256; ++sb) {
            const uint8_t* blk = row + sb * 76;
            float d = orc_half_to_float(rd16(blk + 74));
            uint64_t sw = 0;
            for (int i = 0; i < 6; ++i) sw |= (uint64_t)blk[64 + i] << (8 * i);
            for (int e = 0; e < 256; ++e) {
                int c = (blk[e / 4] >> (2 * (e % 4))) & 3;
                int g = c - 1;
                int sgn = (blk[70 + e / 64] >> ((e / 8) % 8)) & 1;
                wq[sb * 256 + e] = (int16_t)(8 * g + (sgn ? -1 : 1));
            }
            for (int h = 0; h < 16; ++h) {
                int s = (int)((sw >> (3 * h)) & 7u);
                wd[sb * 16 + h] = d * (float)(2 * s + 1) / 8.0f;
                mult[sb * 16 + h] = (int16_t)(2 * s + 1);
            }
        }
    } else if (fmt == ORC_IQ1C) {
        /* group q (values 8q..8q+7): index = qs[q] | (index bits 8-10 from the nibble of
         * qh[q/2] selected by q%2), delta sign = bit 3 of that nibble; the grid entry gives
         * the eight codes c = g+1. */
        for (int64_t sb = 0; sb < K / 256; ++sb) {
            const uint8_t* blk = row + sb * 56;
            float d = orc_half_to_float(rd16(blk + 54));
            uint64_t sw = 0;
            for (int i = 0; i < 6; ++i) sw |= (uint64_t)blk[48 + i] << (8 * i);
            for (int q = 0; q < 32; ++q) {
                int nib = (blk[32 + q / 2] >> (4 * (q % 2))) & 15;
                int idx = blk[q] | ((nib & 7) << 8);
                int sgn = (nib >> 3) & 1;
                uint16_t entry = grid[idx];
                for (int j = 0; j < 8; ++j) {
                    int c = (entry >> (2 * j)) & 3;
                    if (c == 3) bad = 1;
                    wq[sb * 256 + 8 * q + j] = (int16_t)(8 * (c - 1) + (sgn ? -1 : 1));
                }
            }
            for (int h = 0; h < 16; ++h) {
                int s = (int)((sw >> (3 * h)) & 7u);
                wd[sb * 16 + h] = d * (float)(2 * s + 1) / 8.0f;
                mult[sb * 16 + h] = (int16_t)(2 * s + 1);
            }
        }
    } else if (fmt == ORC_IQ1S) {
        /* block b (values 32b..32b+31) of a super-block: its uint16 qh word holds index bits
         * 8-10 of group j (values 32b+8j..+7) at bits 3j..3j+2, s at bits 12-14 and the delta
         * sign at bit 15; the low index bytes are qs[4b+j]. */
        for (int64_t sb = 0; sb < K / 256; ++sb) {
            const uint8_t* blk = row + sb * 50;
            float d = orc_half_to_float(rd16(blk));
            for (int b = 0; b < 8; ++b) {
                uint16_t qh = rd16(blk + 34 + 2 * b);
                int s = (qh >> 12) & 7;
                int sgn = (qh >> 15) & 1;
                for (int j = 0; j < 4; ++j) {
                    int idx = blk[2 + 4 * b + j] | (((qh >> (3 * j)) & 7) << 8);
                    uint16_t entry = grid[idx];
                    for (int i = 0; i < 8; ++i) {
                        int c = (entry >> (2 * i)) & 3;
                        if (c == 3) bad = 1;
                        wq[sb * 256 + 32 * b + 8 * j + i] = (int16_t)(8 * (c - 1) + (sgn ? -1 : 1));
                    }
                }
                for (int h = 0; h < 2; ++h) {
                    wd[sb * 16 + 2 * b + h] = d * (float)(2 * s + 1) / 8.0f;
                    mult[sb * 16 + 2 * b + h] = (int16_t)(2 * s + 1);
                }
            }
        }
    } else if (fmt == ORC_Q6_K) {
        /* 32-value block j of a super-block: value 32j+i (i < 16) has its low 4 bits in the
         * low nibble of ql[16j+i], value 32j+16+i in the high nibble; value 32j+8t+i (t < 4,
         * i < 8) has its high 2 bits at bits 2t..2t+1 of qh[8j+i]. */
        for (int64_t sb = 0; sb < K / 256; ++sb) {
            const uint8_t* blk = row + sb * 210;
            float d = orc_half_to_float(rd16(blk + 208));
            for (int j = 0; j < 8; ++j) {
                for (int u = 0; u < 32; ++u) {
                    int lo = (blk[16 * j + (u % 16)] >> (4 * (u / 16))) & 15;
                    int hi = (blk[128 + 8 * j + (u % 8)] >> (2 * (u / 8))) & 3;
                    wq[sb * 256 + 32 * j + u] = (int16_t)((lo | (hi << 4)) - 32);
                }
            }
            for (int h = 0; h < 16; ++h) wd[sb * 16 + h] = d * (float)(int8_t)blk[192 + h];
        }
    }
    return bad ? -1 : 0;
}

/* Expose the decoder (one row) for the oracle's own tests. */
int orc_decode_row(int fmt, const uint8_t* row, int64_t K, const uint16_t* grid,
                   int16_t* wq, float* wd, float* wm, int16_t* mult) {
    return decode_row(fmt, row, K, grid, wq, wd, wm, mult);
}

static int64_t raw_row_bytes(int fmt, int64_t K) {
    switch (fmt) {
        case ORC_Q8_0: return K / 32 * 34;
        case ORC_Q4_0: return K / 32 * 18;
        case ORC_Q4_K: return K / 256 * 144;
        case ORC_IQ1C: return K / 256 * 56;
        case ORC_Q6_K: return K / 256 * 210;
        case ORC_IQ1S: return K / 256 * 50;
        default:       return K / 256 * 76;
    }
}

/* ----------------------------------------------------------- integer partials */

/* P[m][n][b] = the exact integer dot of block b:
 *   q8_0, q4_0: sum xq*wq;  q4_K: sum xq*nib (unsigned nibbles);
 *   iq1t, iq1c: the folded per-32 form sum_h (2s_h+1) * sum_{16 in half h} xq*(8g+sigma).
 * Returns 0, -1 if any partial falls outside int32, -2 on an invalid grid code. */
int orc_partials(int fmt, const uint8_t* raw, int64_t N, int64_t K, const uint16_t* grid,
                 const int8_t* xq, int64_t M, int32_t* P) {
    const int64_t KB = K / 32, rb = raw_row_bytes(fmt, K);
    int bad = 0, badgrid = 0;
#pragma omp parallel
    {
        int16_t* wq = (int16_t*)malloc(sizeof(int16_t) * K);
        float* wd = (float*)malloc(sizeof(float) * (K / 16));
        float* wm = (float*)malloc(sizeof(float) * KB);
        int16_t* mult = (int16_t*)malloc(sizeof(int16_t) * (K / 16));
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            if (decode_row(fmt, raw + n * rb, K, grid, wq, wd, wm, mult) != 0) badgrid = 1;
            for (int64_t m = 0; m < M; ++m) {
                for (int64_t b = 0; b < KB; ++b) {
                    int64_t total = 0;
                    for (int half = 0; half < 2; ++half) {
                        int64_t s16 = 0;
                        for (int i = 0; i < 16; ++i) {
                            int64_t k = b * 32 + half * 16 + i;
                            s16 += (int64_t)xq[m * K + k] * (int64_t)wq[k];
                        }
                        total += (int64_t)mult[2 * b + half] * s16;
                    }
                    if (total > INT32_MAX || total < INT32_MIN) bad = 1;
                    P[(m * N + n) * KB + b] = (int32_t)total;
                }
            }
        }
        free(wq); free(wd); free(wm); free(mult);
    }
    return badgrid ? -2 : bad ? -1 : 0;
}

/* Per-16 partials P16[m][n][h] = sum over the 16 values of half-block h of
 * xq * wq (iq1t/iq1c: wq = 8g+sigma, before the (2s+1) fold; q6_K: wq = q-32,
 * the two separate half-block sums of each 32-value block).                  */
void orc_partials16(int fmt, const uint8_t* raw, int64_t N, int64_t K, const uint16_t* grid,
                    const int8_t* xq, int64_t M, int32_t* P16) {
    const int64_t KH = K / 16, rb = raw_row_bytes(fmt, K);
#pragma omp parallel
    {
        int16_t* wq = (int16_t*)malloc(sizeof(int16_t) * K);
        float* wd = (float*)malloc(sizeof(float) * KH);
        float* wm = (float*)malloc(sizeof(float) * (K / 32));
        int16_t* mult = (int16_t*)malloc(sizeof(int16_t) * KH);
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            decode_row(fmt, raw + n * rb, K, grid, wq, wd, wm, mult);
            for (int64_t m = 0; m < M; ++m)
                for (int64_t h = 0; h < KH; ++h) {
                    int32_t s = 0;
                    for (int i = 0; i < 16; ++i) s += (int32_t)xq[m * K + h * 16 + i] * wq[h * 16 + i];
                    P16[(m * N + n) * KH + h] = s;
                }
        }
        free(wq); free(wd); free(wm); free(mult);
    }
}

/* ------------------------------------------------------------ f32 output */

/* out[m*ldo + n] = sum over blocks b of xs[m,b] * ( sum_half wd*P16 + wm*xsum[m,b] ),
 * accumulated in double and rounded to f32 once. Rows m0 <= m < m1 only (the
 * bench times a bounded sample of rows with this). Returns -2 on an invalid
 * iq1c grid code, else 0.                                                    */
int orc_gemm_rows(int fmt, const uint8_t* raw, int64_t N, int64_t K, const uint16_t* grid,
                  const int8_t* xq, const float* xs, const int32_t* xsum,
                  int64_t m0, int64_t m1, float* out, int64_t ldo) {
    const int64_t KB = K / 32, rb = raw_row_bytes(fmt, K);
    int badgrid = 0;
    int16_t* wq_all = (int16_t*)malloc(sizeof(int16_t) * (size_t)(N * K));
    float* wd_all = (float*)malloc(sizeof(float) * (size_t)(N * (K / 16)));
    float* wm_all = (float*)malloc(sizeof(float) * (size_t)(N * KB));
    int16_t* mult_all = (int16_t*)malloc(sizeof(int16_t) * (size_t)(N * (K / 16)));
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        if (decode_row(fmt, raw + n * rb, K, grid, wq_all + n * K, wd_all + n * (K / 16), wm_all + n * KB,
                       mult_all + n * (K / 16)) != 0)
            badgrid = 1;
#pragma omp parallel for schedule(static)
    for (int64_t m = m0; m < m1; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            const int16_t* wq = wq_all + n * K;
            const float* wd = wd_all + n * (K / 16);
            const float* wm = wm_all + n * KB;
            double acc = 0.0;
            for (int64_t b = 0; b < KB; ++b) {
                double blockval = 0.0;
                for (int half = 0; half < 2; ++half) {
                    int32_t s16 = 0;
                    for (int i = 0; i < 16; ++i) {
                        int64_t k = b * 32 + half * 16 + i;
                        s16 += (int32_t)xq[m * K + k] * (int32_t)wq[k];
                    }
                    blockval += (double)wd[2 * b + half] * (double)s16;
                }
                blockval += (double)wm[b] * (double)xsum[m * KB + b];
                acc += (double)xs[m * KB + b] * blockval;
            }
            out[(m - m0) * ldo + n] = (float)acc;
        }
    }
    free(wq_all); free(wd_all); free(wm_all); free(mult_all);
    return badgrid ? -2 : 0;
}

/* The magnitude of what the contraction adds up, per output: abs[m*N + n] = sum over blocks
 * b and halves h of |xs[m,b] * wd_h * P16_h| + |xs[m,b] * wm_b * xsum[m,b]| (in double).
 * A floating-point evaluation that adds the per-block terms one at a time in f32 makes an
 * error of at most (number of f32 additions) * 2^-24 * abs (each rounding is relative to a
 * partial sum, and every partial sum is bounded by abs), so this is the yardstick of the
 * tests' rounding bound for f32 outputs. Rows m0 <= m < m1. Returns -2 on an invalid grid
 * code, else 0. */
int orc_gemm_abs_rows(int fmt, const uint8_t* raw, int64_t N, int64_t K, const uint16_t* grid,
                      const int8_t* xq, const float* xs, const int32_t* xsum,
                      int64_t m0, int64_t m1, double* absout) {
    const int64_t KB = K / 32, rb = raw_row_bytes(fmt, K);
    int badgrid = 0;
#pragma omp parallel
    {
        int16_t* wq = (int16_t*)malloc(sizeof(int16_t) * K);
        float* wd = (float*)malloc(sizeof(float) * (K / 16));
        float* wm = (float*)malloc(sizeof(float) * KB);
        int16_t* mult = (int16_t*)malloc(sizeof(int16_t) * (K / 16));
#pragma omp for schedule(static)
        for (int64_t n = 0; n < N; ++n) {
            if (decode_row(fmt, raw + n * rb, K, grid, wq, wd, wm, mult) != 0) badgrid = 1;
            for (int64_t m = m0; m < m1; ++m) {
                double a = 0.0;
                for (int64_t h = 0; h < K / 16; ++h) {
                    int32_t s16 = 0;
                    for (int i = 0; i < 16; ++i) s16 += (int32_t)xq[m * K + h * 16 + i] * (int32_t)wq[h * 16 + i];
                    a += fabs((double)xs[m * KB + h / 2] * (double)wd[h] * (double)s16);
                }
                for (int64_t b = 0; b < KB; ++b)
                    a += fabs((double)xs[m * KB + b] * (double)wm[b] * (double)xsum[m * KB + b]);
                absout[(m - m0) * N + n] = a;
            }
        }
        free(wq); free(wd); free(wm); free(mult);
    }
    return badgrid ? -2 : 0;
}

int orc_gemm(int fmt, const uint8_t* raw, int64_t N, int64_t K, const uint16_t* grid,
             const int8_t* xq, const float* xs, const int32_t* xsum, int64_t M, float* out) {
    return orc_gemm_rows(fmt, raw, N, K, grid, xq, xs, xsum, 0, M, out, N);
}

/* ---------------------------------------------------------------- W8A8 */

/* acc[m][n] = sum_k a[m,k]*w[n,k] (exact int32); out = bf16_rne((f32(acc)*sa[m])*sw[n]),
 * two separate f32 multiplies in that order. acc may be NULL. Returns -1 if an
 * accumulator leaves int32.                                                    */
int orc_gemm_w8a8(const int8_t* a, const float* sa, int64_t M, const int8_t* w, const float* sw,
                  int64_t N, int64_t K, int32_t* acc, uint16_t* out, int64_t m0, int64_t m1) {
    int bad = 0;
#pragma omp parallel for schedule(static)
    for (int64_t m = m0; m < m1; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k) s += (int64_t)a[m * K + k] * (int64_t)w[n * K + k];
            if (s > INT32_MAX || s < INT32_MIN) bad = 1;
            volatile float t = (float)(int32_t)s * sa[m];
            volatile float u = t * sw[n];
            if (acc) acc[(m - m0) * N + n] = (int32_t)s;
            out[(m - m0) * N + n] = orc_float_to_bf16(u);
        }
    }
    return bad ? -1 : 0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count for the timed baseline only (no effect on any result). */
void orc_set_threads(int n) {
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}
