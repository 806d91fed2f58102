/*
 * attn_oracle.c -- plain fp64 CPU oracle for the fused attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle, not the product: only the
 * test-suite, the smoke check and the CPU-baseline leg of the benchmark load the
 * library built from it.  It shares no code, header, table or helper with the
 * HIP path, and the HIP path never calls it.
 *
 * What it computes.  The page "A Thread-Register Decoupled GPU Execution Model
 * for Efficient Tensor Computation" (introduction) names multi-head attention,
 * "Equ. 1", as the core of a transformer block and the FlashAttention series as
 * its fused implementation.  The text of Equ. 1 did not survive extraction; it
 * is read here as standard scaled dot-product attention applied per head:
 *
 *     s_ij  = scale * sum_d Q[i,d] * K[j,d]           for every visible key j
 *     m_i   = max_j s_ij
 *     l_i   = sum_j exp(s_ij - m_i)
 *     O_i   = sum_j exp(s_ij - m_i) * V[j,:] / l_i
 *     LSE_i = m_i + ln(l_i)
 *
 * FlashAttention reaches the same result (up to rounding order) with a tiled
 * pass and an online softmax; the oracle does not tile, does not fuse and keeps
 * the plain two-pass softmax per row, all in fp64.
 *
 * Readings where the pages are silent (each one listed in the design notes):
 *   - layout: q, o are [B][Hq][Sq][D]; k, v are [B][Hkv][Sk][D]; lse is [B][Hq][Sq];
 *     all contiguous, D fastest.
 *   - grouped heads (the evaluation's GQA/MQA variants, with groups of eight query heads):
 *     query head h reads key/value head h / (Hq / Hkv), i.e. consecutive groups.
 *   - causal mask with Sq != Sk: aligned bottom-right, key j is visible from query
 *     i iff j <= i + (Sk - Sq); a query with no visible key gets O = 0, LSE = -inf.
 *   - LSE is the natural logarithm of the sum of exponentials of the scaled scores.
 *   - inputs arrive already rounded to their storage type (bf16, fp16, fp32 or
 *     fp64) and are widened exactly to fp64 before any arithmetic.
 *
 * Parity status: every function here is pinned by the CPU tests (closed forms,
 * invariants, 50-digit brute force on tiny inputs, an independent library
 * routine; the gradients also by central differences of the forward; the rotary
 * embedding by complex multiplication, exact rotations, the relative-position
 * property and independent roundings); the pages print no attention values to
 * pin against.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* storage-type codes accepted by the oracle (its own numbering) */
enum { ORACLE_BF16 = 0, ORACLE_FP16 = 1, ORACLE_FP32 = 2, ORACLE_FP64 = 3 };

/* Widen one bfloat16 bit pattern: bf16 is the top half of an IEEE binary32. */
static double widen_bf16(uint16_t bits) {
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* Widen one IEEE-754 binary16 bit pattern from its definition:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double widen_fp16(uint16_t bits) {
    int sign = (bits >> 15) & 1;
    int expo = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double mag;
    if (expo == 0)
        mag = ldexp((double)frac, -24);               /* subnormal: frac * 2^-14 * 2^-10 */
    else if (expo == 31)
        mag = frac ? NAN : INFINITY;
    else
        mag = ldexp((double)(frac | 0x400), expo - 25); /* (1024 + frac) * 2^(e-15-10) */
    return sign ? -mag : mag;
}

static double load_elem(const void* base, int dtype, size_t idx) {
    switch (dtype) {
    case ORACLE_BF16: return widen_bf16(((const uint16_t*)base)[idx]);
    case ORACLE_FP16: return widen_fp16(((const uint16_t*)base)[idx]);
    case ORACLE_FP32: return (double)((const float*)base)[idx];
    default:          return ((const double*)base)[idx];
    }
}

/* Widen n elements of a storage-typed array into fp64 (test helper). */
int oracle_widen(const void* src, int dtype, int64_t n, double* dst) {
    if (!src || !dst || n < 0 || dtype < ORACLE_BF16 || dtype > ORACLE_FP64) return 1;
    for (int64_t i = 0; i < n; ++i) dst[i] = load_elem(src, dtype, (size_t)i);
    return 0;
}

/* One query row of one head: scores, two-pass softmax, weighted sum of V. */
static void one_row(const void* q, const void* k, const void* v, int dtype,
                    int Hq, int Hkv, int Sq, int Sk, int D, double scale, int causal,
                    int64_t row, double* qrow, double* s, double* o_out, double* lse_out) {
    const int64_t i  = row % Sq;
    const int64_t bh = row / Sq;
    const int64_t h  = bh % Hq;
    const int64_t b  = bh / Hq;
    const int64_t kvh = h / (Hq / Hkv);

    const size_t q_off  = (size_t)row * (size_t)D;
    const size_t kv_off = ((size_t)b * (size_t)Hkv + (size_t)kvh) * (size_t)Sk * (size_t)D;

    /* visible keys: 0 .. last (inclusive) */
    int64_t last = Sk - 1;
    if (causal) {
        int64_t lim = i + ((int64_t)Sk - (int64_t)Sq);
        if (lim < last) last = lim;
    }
    if (last < 0) {                      /* no visible key */
        for (int d = 0; d < D; ++d) o_out[d] = 0.0;
        *lse_out = -INFINITY;
        return;
    }

    for (int d = 0; d < D; ++d) qrow[d] = load_elem(q, dtype, q_off + (size_t)d);

    /* pass 1: scaled scores and their maximum */
    double m = -INFINITY;
    for (int64_t j = 0; j <= last; ++j) {
        double dot = 0.0;
        const size_t kr = kv_off + (size_t)j * (size_t)D;
        for (int d = 0; d < D; ++d) dot += qrow[d] * load_elem(k, dtype, kr + (size_t)d);
        s[j] = scale * dot;
        if (s[j] > m) m = s[j];
    }

    /* pass 2: exponentials relative to the maximum, their sum, and the V mix */
    double l = 0.0;
    for (int d = 0; d < D; ++d) o_out[d] = 0.0;
    for (int64_t j = 0; j <= last; ++j) {
        const double w = exp(s[j] - m);
        l += w;
        const size_t vr = kv_off + (size_t)j * (size_t)D;
        for (int d = 0; d < D; ++d) o_out[d] += w * load_elem(v, dtype, vr + (size_t)d);
    }
    for (int d = 0; d < D; ++d) o_out[d] /= l;
    *lse_out = m + log(l);
}

/*
 * Attention forward for a list of query rows (or all rows when rows == NULL).
 *   row index r = (b * Hq + h) * Sq + i
 *   o   : nrows x D doubles, row-major, in the order of `rows`
 *   lse : nrows doubles (may be NULL)
 *   nthreads <= 0 uses the OpenMP default.
 * Returns 0 on success, 1 on an invalid argument (nothing written).
 */
int oracle_attn_rows(const void* q, const void* k, const void* v, int dtype,
                     int B, int Hq, int Hkv, int Sq, int Sk, int D,
                     double scale, int causal,
                     const int64_t* rows, int64_t nrows,
                     double* o, double* lse, int nthreads) {
    if (!q || !k || !v || !o) return 1;
    if (dtype < ORACLE_BF16 || dtype > ORACLE_FP64) return 1;
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || D < 1) return 1;
    if (Hq % Hkv != 0) return 1;
    const int64_t total = (int64_t)B * Hq * Sq;
    if (rows == NULL && nrows != total) return 1;
    if (nrows < 0) return 1;
    if (rows)
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= total) return 1;

    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
        double* s    = (double*)malloc(sizeof(double) * (size_t)Sk);
        double  lse_dummy;
        if (!qrow || !s) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 8)
            for (int64_t r = 0; r < nrows; ++r) {
                const int64_t row = rows ? rows[r] : r;
                one_row(q, k, v, dtype, Hq, Hkv, Sq, Sk, D, scale, causal, row, qrow, s,
                        o + (size_t)r * (size_t)D, lse ? lse + r : &lse_dummy);
            }
        }
        free(qrow);
        free(s);
    }
    return bad ? 2 : 0;
}

/*
 * Gradients of the attention forward above (the FlashAttention backward the FIBER
 * page evaluates as its training workload), written from the chain rule of
 *     s_ij = scale q_i.k_j,  P_ij = exp(s_ij - LSE_i),  O_i = sum_j P_ij v_j
 * for a loss whose gradient with respect to O is dO:
 *     dv_j  = sum_i P_ij dO_i
 *     dP_ij = dO_i . v_j
 *     dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)
 *     dq_i  = scale sum_j dS_ij k_j,   dk_j = scale sum_i dS_ij q_i
 * over visible pairs only; a key/value head's dk, dv sum over the query heads that
 * read it.  P is recomputed in fp64 from the inputs (two-pass softmax per row).
 *   q, dout : [B][Hq][Sq][D]   k, v : [B][Hkv][Sk][D]   (storage type `dtype`)
 *   dq      : [B][Hq][Sq][D]   dk, dv : [B][Hkv][Sk][D]  (fp64, fully written)
 * One thread per (batch, key/value head): no two threads touch the same output,
 * and every sum runs in a fixed order.  Returns 0, 1 (invalid argument) or 2.
 */
int oracle_attn_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype,
                    int B, int Hq, int Hkv, int Sq, int Sk, int D, double scale, int causal,
                    double* dq, double* dk, double* dv, int nthreads) {
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return 1;
    if (dtype < ORACLE_BF16 || dtype > ORACLE_FP64) return 1;
    if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 1 || D < 1) return 1;
    if (Hq % Hkv != 0) return 1;
    const int64_t groups = (int64_t)B * Hkv;
    const int R = Hq / Hkv;
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel
    {
        double* qrow = (double*)malloc(sizeof(double) * (size_t)D);
        double* grow = (double*)malloc(sizeof(double) * (size_t)D);
        double* p    = (double*)malloc(sizeof(double) * (size_t)Sk);
        double* dp   = (double*)malloc(sizeof(double) * (size_t)Sk);
        if (!qrow || !grow || !p || !dp) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t gi = 0; gi < groups; ++gi) {
                const int64_t b = gi / Hkv, g = gi % Hkv;
                const size_t kv_off = (size_t)gi * (size_t)Sk * (size_t)D;
                for (size_t x = 0; x < (size_t)Sk * (size_t)D; ++x) {
                    dk[kv_off + x] = 0.0;
                    dv[kv_off + x] = 0.0;
                }
                for (int r = 0; r < R; ++r) {
                    const int64_t h = g * R + r;
                    for (int64_t i = 0; i < Sq; ++i) {
                        const size_t row = (size_t)((b * Hq + h) * Sq + i);
                        const size_t q_off = row * (size_t)D;
                        double* dqi = dq + q_off;
                        for (int d = 0; d < D; ++d) dqi[d] = 0.0;
                        int64_t last = Sk - 1;
                        if (causal) {
                            const int64_t diag = i + ((int64_t)Sk - (int64_t)Sq);
                            if (diag < last) last = diag;
                        }
                        if (last < 0) continue;                 /* no visible key: no gradient */
                        for (int d = 0; d < D; ++d) {
                            qrow[d] = load_elem(q, dtype, q_off + (size_t)d);
                            grow[d] = load_elem(dout, dtype, q_off + (size_t)d);
                        }
                        /* scores, their max, and the normalised weights */
                        double m = -INFINITY;
                        for (int64_t j = 0; j <= last; ++j) {
                            double dot = 0.0;
                            const size_t koff = kv_off + (size_t)j * (size_t)D;
                            for (int d = 0; d < D; ++d) dot += qrow[d] * load_elem(k, dtype, koff + (size_t)d);
                            p[j] = scale * dot;
                            if (p[j] > m) m = p[j];
                        }
                        double l = 0.0;
                        for (int64_t j = 0; j <= last; ++j) {
                            p[j] = exp(p[j] - m);
                            l += p[j];
                        }
                        for (int64_t j = 0; j <= last; ++j) p[j] /= l;
                        /* dP = dO . v and the row's sum of P dP */
                        double pdp = 0.0;
                        for (int64_t j = 0; j <= last; ++j) {
                            double dot = 0.0;
                            const size_t voff = kv_off + (size_t)j * (size_t)D;
                            for (int d = 0; d < D; ++d) dot += grow[d] * load_elem(v, dtype, voff + (size_t)d);
                            dp[j] = dot;
                            pdp += p[j] * dot;
                        }
                        for (int64_t j = 0; j <= last; ++j) {
                            const double ds = p[j] * (dp[j] - pdp);
                            const size_t koff = kv_off + (size_t)j * (size_t)D;
                            for (int d = 0; d < D; ++d) {
                                dqi[d] += scale * ds * load_elem(k, dtype, koff + (size_t)d);
                                dk[koff + (size_t)d] += scale * ds * qrow[d];
                                dv[koff + (size_t)d] += p[j] * grow[d];
                            }
                        }
                    }
                }
            }
        }
        free(qrow);
        free(grow);
        free(p);
        free(dp);
    }
    return bad ? 2 : 0;
}

/* ---- Rotary position embedding (RoPE) -------------------------------------
 *
 * The FIBER page names RoPE among the vector operations that sit between the
 * GEMMs of a transformer block (background; evaluation set-up, "Workloads"),
 * and the VDCores page evaluates QKV projection fused with RoPE (evaluation,
 * "dynamic fusion", Fig. 12).  Neither page writes the rotation out; it is read
 * as the rotary embedding of the RoPE paper the FIBER page cites: the D features
 * of a row form D/2 pairs, and pair i of the row at position p is turned through
 * an angle whose cosine and sine the caller tabulates as cos_tab[p][i] and
 * sin_tab[p][i]:
 *
 *     a' = a * c - b * s,      b' = a * s + b * c.
 *
 * Pairs are features (2i, 2i+1) (layout 1, the RoPE paper's arrangement) or
 * (i, i + D/2) (layout 2, the split-halves arrangement).  Row s of a head sits at
 * position s + pos_offset.  Each rotated value is computed in fp64 (both products
 * are exact there for 16-bit inputs and fp32 table entries, so only the
 * difference or sum rounds) and is then rounded once, to nearest with ties to
 * even, into the storage type: the same result a separate RoPE step writing
 * 16-bit tensors would give. */

/* Round v to the nearest value of a binary format with `mant` fraction bits and
 * normal exponents emin..emax (ties to an even last fraction bit), from the
 * format's definition: below 2^emin the spacing is fixed at 2^(emin - mant)
 * (subnormals); at or beyond 2^(emax + 1) after rounding the result is infinite. */
static double round_to_format(double v, int mant, int emin, int emax) {
    if (v != v || v == 0.0 || isinf(v)) return v;
    int e;
    (void)frexp(fabs(v), &e);          /* |v| = f * 2^e, f in [0.5, 1): exponent e - 1 */
    int ex = e - 1;
    if (ex < emin) ex = emin;
    const double quantum = ldexp(1.0, ex - mant);
    const double scaled = v / quantum;  /* exact: division by a power of two */
    double r = floor(scaled);
    const double frac = scaled - r;     /* exact: scaled has at most 53 bits */
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    const double out = copysign(r * quantum, v);   /* a value rounded to zero keeps its sign */
    if (fabs(out) >= ldexp(1.0, emax + 1)) return v > 0 ? INFINITY : -INFINITY;
    return out;
}

/* Encode a value already representable in the storage type as its bit pattern. */
static uint16_t encode16(double r, int dtype) {
    if (dtype == ORACLE_BF16) {
        const float f = (float)r;       /* exact: every bf16 value is a binary32 value */
        uint32_t w;
        memcpy(&w, &f, sizeof w);
        if (r != r) return 0x7fc0;
        return (uint16_t)(w >> 16);
    }
    /* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits */
    uint16_t sign = signbit(r) ? 0x8000 : 0;
    double a = fabs(r);
    if (r != r) return 0x7e00;
    if (isinf(a)) return sign | 0x7c00;
    if (a < ldexp(1.0, -14))            /* subnormal or zero: a = frac * 2^-24 */
        return sign | (uint16_t)(a * ldexp(1.0, 24));
    int e = ilogb(a);
    uint16_t frac = (uint16_t)((ldexp(a, -e) - 1.0) * 1024.0);
    return sign | (uint16_t)((e + 15) << 10) | frac;
}

static double round_to_storage(double v, int dtype) {
    return dtype == ORACLE_BF16 ? round_to_format(v, 7, -126, 127)
                                : round_to_format(v, 10, -14, 15);
}

/* Round n fp64 values to the 16-bit storage type (test helper for the pins). */
int oracle_round16(const double* src, int dtype, int64_t n, uint16_t* dst) {
    if (!src || !dst || n < 0 || (dtype != ORACLE_BF16 && dtype != ORACLE_FP16)) return 1;
    for (int64_t i = 0; i < n; ++i) dst[i] = encode16(round_to_storage(src[i], dtype), dtype);
    return 0;
}

/* Rotate every row of x ([nheads][S][D], 16-bit storage type) by the tabulated
 * angles of its position; writes the unrounded fp64 result (may be NULL) and the
 * rounded storage bits (may be NULL).  Tables are [ntab][D/2] fp32; a position
 * outside 0..ntab-1 is an error. */
int oracle_rope(const void* x, int dtype, int64_t nheads, int S, int D,
                const float* cos_tab, const float* sin_tab, int ntab, int pos_offset,
                int layout, double* out_f64, uint16_t* out_bits) {
    if (!x || !cos_tab || !sin_tab || nheads < 0 || S < 0 || D < 2 || D % 2)
        return 1;
    if (dtype != ORACLE_BF16 && dtype != ORACLE_FP16) return 1;
    if (layout != 1 && layout != 2) return 1;
    if (S > 0 && (pos_offset < 0 || pos_offset + S - 1 >= ntab)) return 2;
    const int half = D / 2;
    for (int64_t hs = 0; hs < nheads * (int64_t)S; ++hs) {
        const int pos = (int)(hs % S) + pos_offset;
        const size_t row = (size_t)hs * (size_t)D;
        for (int i = 0; i < half; ++i) {
            const int ia = layout == 1 ? 2 * i : i;
            const int ib = layout == 1 ? 2 * i + 1 : i + half;
            const double a = load_elem(x, dtype, row + (size_t)ia);
            const double b = load_elem(x, dtype, row + (size_t)ib);
            const double c = (double)cos_tab[(size_t)pos * half + i];
            const double sn = (double)sin_tab[(size_t)pos * half + i];
            const double ra = a * c - b * sn;
            const double rb = a * sn + b * c;
            if (out_f64) {
                out_f64[row + (size_t)ia] = ra;
                out_f64[row + (size_t)ib] = rb;
            }
            if (out_bits) {
                out_bits[row + (size_t)ia] = encode16(round_to_storage(ra, dtype), dtype);
                out_bits[row + (size_t)ib] = encode16(round_to_storage(rb, dtype), dtype);
            }
        }
    }
    return 0;
}

/* Number of threads an OpenMP parallel region here would use. */
int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
