/*
 * oracle.c -- plain fp64 CPU oracle for block-sparse masked softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the yardstick the GPU path is checked
 * against; it is never part of the product path.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark load it.  It shares no code,
 * header, table or helper with the HIP library.
 *
 * What it computes (the operation the pages define):
 *   "Writing Pallas Kernels for JAX" (rajatpandit.com), section "Writing the Kernel
 *   Logic: Load, Compute, Store": scores are the scaled dot products of query rows
 *   with key rows; where the block mask is 0 the score is pushed to -inf before a
 *   row softmax; the softmax weights multiply V.  "Pallas-Triton kernels and kernel
 *   auto-tuning" (robertdyro.com), section "Flash Attention": the tiled method
 *   computes that operator exactly, so the oracle is the plain definition, not
 *   the tiled algorithm.
 *
 * Readings (where the pages leave a step open):
 *   - The softmax is over the whole row of keys, not per tile.  The per-tile
 *     softmax printed in the Pallas kernel listing is not attention; the oracle
 *     follows the exact operator.
 *   - The mask is block level: mask[b][h][qi][kj] != 0 activates the key block
 *     kj (keys kj*block_k .. kj*block_k+block_k-1) for every query in query block
 *     qi (queries qi*block_q .. qi*block_q+block_q-1).
 *   - A row with no active key has out = 0 and lse = -inf (a literal softmax over
 *     an all -inf row is undefined).
 *   - lse is the natural logarithm of the row's sum of exp(score).
 *   - Inputs are widened exactly to double; scale is the caller's fp32 value
 *     widened, applied as scale * (q . k).  Inputs may be fp32, bf16, fp64 or fp8
 *     (e4m3, OCP form: "JAX Pallas and Blackwell", section "What the Tutorial
 *     Covers", keeps fp32 accumulators and fp8 data); the method is the same on
 *     the widened values.
 *
 * Two passes per row, with no online rescaling and no tiling:
 *   pass 1: s_j = scale * sum_d q[r][d] * k[j][d]   (d ascending, j ascending over
 *           the active keys), m = max_j s_j;
 *   pass 2: e_j = exp(s_j - m), l = sum_j e_j, out[r][:] = sum_j e_j v[j][:] / l,
 *           lse[r] = m + log(l).
 * Skipping inactive keys equals the literal -inf form exactly: those terms add
 * exact zeros and never change the max.
 *
 * Compaction (the block-list form of the mask): for each mask row in (b, h, qi)
 * row-major order, the ascending list of kj with mask != 0; row_ptr[0] = 0 and
 * row_ptr[r+1] = row_ptr[r] + count of row r.
 *
 * Element-level masks (the *_elem entry points).  The mask the pages load per
 * (query block, key block) is an element tile: "Writing Pallas Kernels for JAX",
 * section "Writing the Kernel Logic: Load, Compute, Store", keeps a score where
 * the mask tile is set and pushes it to -inf elsewhere.  Reading: a block of the
 * block mask is empty (0: every element masked), full (1: every element kept) or
 * partial (any other value: element (i, j) of the block is kept iff bit j % 32 of
 * word j / 32 of row i of bit tile pidx[block] is set, the tiles being
 * pbits[n_tiles][block_q][block_k / 32]).  Everything else is as above, with the
 * kept elements in place of the active keys; a row with no kept element has
 * out = 0 and lse = -inf.
 *
 * Backward (oracle_bwd, oracle_bwd_sample).  "Writing Pallas Kernels for JAX",
 * section "The Empathy of the Void": a hand-written kernel gets no automatic
 * gradient, its author supplies one.  The
 * gradient of the forward above is fixed by the chain rule.  For an upstream
 * gradient dout = dL/dout, with P[r][j] = exp(s[r][j] - lse[r]) over the active
 * keys of row r (0 elsewhere):
 *   dv[j]    = sum_r P[r][j] dout[r]
 *   dP[r][j] = dout[r] . v[j]
 *   delta[r] = sum_j P[r][j] dP[r][j]
 *   dS[r][j] = P[r][j] (dP[r][j] - delta[r])
 *   dq[r]    = scale sum_j dS[r][j] k[j]
 *   dk[j]    = scale sum_r dS[r][j] q[r]
 * lse and delta of every row come from the oracle's own two-pass forward (never
 * from the caller).  Pass A walks each query row (its scores, lse, P, dP, delta,
 * dq); pass B walks each key row over the query rows that see its block and
 * accumulates dk and dv.  Sums run over ascending j, r and d.  Rows with no active
 * key have dq = 0 and add nothing to any dk or dv.
 *
 * Ragged dot (oracle_ragged_dot): "Pallas-Triton kernels and kernel auto-tuning",
 * section "Ragged Dot (Group Matrix Multiplication)": the right-hand side is a
 * stack of G expert matrices rhs[g][K][N]; the rows of lhs[M][K] are assigned to
 * the experts in order, group g taking the next group_sizes[g] rows, and output
 * row i is lhs row i times the matrix of its group.  Readings: rows past the sum of
 * the group sizes belong to no group and are 0; a negative size or a sum above M
 * is a bad argument.  out[i][n] = sum over k ascending of lhs[i][k] * rhs[g][k][n],
 * in fp64 from the exactly widened inputs.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F64 = 2, ORC_FP8 = 3 };

typedef struct {
    const void* q;
    const void* k;
    const void* v;
    int dtype;
    const uint8_t* mask;
    int64_t B, H, S, D;
    int64_t block_q, block_k, n_q, n_k;
    double scale;
    /* element-level masks: NULL pidx means the block mask alone decides */
    const int32_t* pidx;
    const uint32_t* pbits;
    int64_t n_tiles;
} problem;

/* Exact widening of one element to double.  bf16 is the top 16 bits of an fp32.
 * fp8 is e4m3 in the OCP form: sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * exponent 0 is subnormal (m/8 * 2^-6), no infinities, S.1111.111 is NaN. */
static double widen(const void* base, int dtype, int64_t idx) {
    if (dtype == ORC_F32) return (double)((const float*)base)[idx];
    if (dtype == ORC_FP8) {
        const uint8_t b = ((const uint8_t*)base)[idx];
        const int sgn = b >> 7, e = (b >> 3) & 15, m = b & 7;
        if (e == 15 && m == 7) return NAN;
        const double mag = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
        return sgn ? -mag : mag;
    }
    if (dtype == ORC_BF16) {
        uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return (double)f;
    }
    return ((const double*)base)[idx];
}

static int check(const problem* p) {
    if (!p->q || !p->k || !p->v || !p->mask) return 1;
    if (p->B <= 0 || p->H <= 0 || p->S <= 0 || p->D <= 0) return 2;
    if (p->block_q <= 0 || p->block_k <= 0) return 2;
    if (p->S % p->block_q != 0 || p->S % p->block_k != 0) return 2;
    if (p->dtype < ORC_F32 || p->dtype > ORC_FP8) return 3;
    if (p->pidx) {
        if (!p->pbits || p->n_tiles < 0 || p->block_k % 32 != 0) return 4;
        /* every partial block must name an existing tile */
        const int64_t nb = p->B * p->H * p->n_q * p->n_k;
        for (int64_t i = 0; i < nb; ++i)
            if (p->mask[i] > 1 && (p->pidx[i] < 0 || p->pidx[i] >= p->n_tiles)) return 4;
    }
    return 0;
}

/* Is key j kept for query s?  blk is the mask value of (s's query block, j's key
 * block), bi that block's flat index. */
static int kept(const problem* p, uint8_t blk, int64_t bi, int64_t s, int64_t j) {
    if (blk == 0) return 0;
    if (!p->pidx || blk == 1) return 1;
    const int64_t i = s % p->block_q, c = j % p->block_k;
    const uint32_t w = p->pbits[((int64_t)p->pidx[bi] * p->block_q + i) * (p->block_k / 32) + c / 32];
    return (int)((w >> (c % 32)) & 1u);
}

/* One query row: bh = b*H + h, s = query position.  sbuf holds S doubles,
 * acc holds D doubles. */
static void oracle_row(const problem* p, int64_t bh, int64_t s, double* out_row,
                       double* lse_out, double* sbuf, double* acc) {
    const int64_t D = p->D;
    const int64_t qi = s / p->block_q;
    const uint8_t* mrow = p->mask + (bh * p->n_q + qi) * p->n_k;
    const int64_t qbase = (bh * p->S + s) * D;

    const int64_t brow = (bh * p->n_q + qi) * p->n_k;

    /* pass 1: scores of the active keys, ascending, and their max */
    int64_t n = 0;
    double m = -INFINITY;
    for (int64_t kj = 0; kj < p->n_k; ++kj) {
        if (!mrow[kj]) continue;
        for (int64_t j = kj * p->block_k; j < (kj + 1) * p->block_k; ++j) {
            if (!kept(p, mrow[kj], brow + kj, s, j)) continue;
            const int64_t kbase = (bh * p->S + j) * D;
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d)
                dot += widen(p->q, p->dtype, qbase + d) * widen(p->k, p->dtype, kbase + d);
            const double sj = p->scale * dot;
            sbuf[n++] = sj;
            if (sj > m) m = sj;
        }
    }
    if (n == 0) {
        for (int64_t d = 0; d < D; ++d) out_row[d] = 0.0;
        *lse_out = -INFINITY;
        return;
    }

    /* pass 2: exponentials, their sum, and the weighted sum of V rows */
    double l = 0.0;
    for (int64_t t = 0; t < n; ++t) {
        sbuf[t] = exp(sbuf[t] - m);
        l += sbuf[t];
    }
    for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
    int64_t t = 0;
    for (int64_t kj = 0; kj < p->n_k; ++kj) {
        if (!mrow[kj]) continue;
        for (int64_t j = kj * p->block_k; j < (kj + 1) * p->block_k; ++j) {
            if (!kept(p, mrow[kj], brow + kj, s, j)) continue;
            const int64_t vbase = (bh * p->S + j) * D;
            const double e = sbuf[t++];
            for (int64_t d = 0; d < D; ++d) acc[d] += e * widen(p->v, p->dtype, vbase + d);
        }
    }
    for (int64_t d = 0; d < D; ++d) out_row[d] = acc[d] / l;
    *lse_out = m + log(l);
}

/* Thread count of the next parallel region: nthreads if positive, else the
 * process's default (OMP_NUM_THREADS or all cores), so that one call with an
 * explicit count does not change the calls after it. */
static int default_threads(void) {
#ifdef _OPENMP
    static int n = 0;
    if (n == 0) n = omp_get_max_threads();  /* taken before any call sets a count */
    return n;
#else
    return 1;
#endif
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    omp_set_num_threads(nthreads > 0 ? nthreads : default_threads());
#else
    (void)nthreads;
#endif
}

static problem make_problem(const void* q, const void* k, const void* v, int dtype,
                            const uint8_t* mask, int64_t B, int64_t H, int64_t S, int64_t D,
                            int64_t block_q, int64_t block_k, float scale) {
    problem p;
    p.q = q; p.k = k; p.v = v; p.dtype = dtype; p.mask = mask;
    p.B = B; p.H = H; p.S = S; p.D = D;
    p.block_q = block_q; p.block_k = block_k;
    p.n_q = block_q > 0 ? S / block_q : 0;
    p.n_k = block_k > 0 ? S / block_k : 0;
    p.scale = (double)scale;
    p.pidx = NULL;
    p.pbits = NULL;
    p.n_tiles = 0;
    return p;
}

/* Full forward: out is double[B][H][S][D], lse is double[B][H][S].
 * Returns 0 on success, nonzero on a bad argument (nothing written). */
static int run_fwd(const problem* pp, double* out, double* lse, int nthreads) {
    const problem p = *pp;
    const int64_t S = p.S, D = p.D;
    int rc = check(&p);
    if (rc) return rc;
    if (!out || !lse) return 1;
    set_threads(nthreads);
    const int64_t rows = p.B * p.H * S;
    int failed = 0;
#pragma omp parallel
    {
        double* sbuf = (double*)malloc(sizeof(double) * (size_t)S);
        double* acc = (double*)malloc(sizeof(double) * (size_t)D);
        if (!sbuf || !acc) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < rows; ++r)
                oracle_row(&p, r / S, r % S, out + r * D, lse + r, sbuf, acc);
        }
        free(sbuf);
        free(acc);
    }
    return failed ? 9 : 0;
}

int oracle_fwd(const void* q, const void* k, const void* v, int dtype, const uint8_t* mask,
               int64_t B, int64_t H, int64_t S, int64_t D, int64_t block_q, int64_t block_k,
               float scale, double* out, double* lse, int nthreads) {
    problem p = make_problem(q, k, v, dtype, mask, B, H, S, D, block_q, block_k, scale);
    return run_fwd(&p, out, lse, nthreads);
}

/* Element-level masks: mask holds block states (0 empty, 1 full, else partial),
 * pidx[B][H][n_q][n_k] the bit tile of each partial block, pbits the tiles. */
int oracle_fwd_elem(const void* q, const void* k, const void* v, int dtype, const uint8_t* mask,
                    const int32_t* pidx, const uint32_t* pbits, int64_t n_tiles, int64_t B,
                    int64_t H, int64_t S, int64_t D, int64_t block_q, int64_t block_k, float scale,
                    double* out, double* lse, int nthreads) {
    problem p = make_problem(q, k, v, dtype, mask, B, H, S, D, block_q, block_k, scale);
    if (!pidx) return 1;
    p.pidx = pidx;
    p.pbits = pbits;
    p.n_tiles = n_tiles;
    return run_fwd(&p, out, lse, nthreads);
}

/* Selected rows only: rows[i] is a flat row index (b*H + h)*S + s.
 * out_rows is double[n_rows][D], lse_rows is double[n_rows]. */
static int run_rows(const problem* pp, const int64_t* rows, int64_t n_rows, double* out_rows,
                    double* lse_rows, int nthreads) {
    const problem p = *pp;
    const int64_t S = p.S, D = p.D;
    int rc = check(&p);
    if (rc) return rc;
    if (!rows || !out_rows || !lse_rows) return 1;
    for (int64_t i = 0; i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= p.B * p.H * S) return 2;
    set_threads(nthreads);
    int failed = 0;
#pragma omp parallel
    {
        double* sbuf = (double*)malloc(sizeof(double) * (size_t)S);
        double* acc = (double*)malloc(sizeof(double) * (size_t)D);
        if (!sbuf || !acc) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < n_rows; ++i)
                oracle_row(&p, rows[i] / S, rows[i] % S, out_rows + i * D, lse_rows + i, sbuf, acc);
        }
        free(sbuf);
        free(acc);
    }
    return failed ? 9 : 0;
}

int oracle_fwd_rows(const void* q, const void* k, const void* v, int dtype, const uint8_t* mask,
                    int64_t B, int64_t H, int64_t S, int64_t D, int64_t block_q, int64_t block_k,
                    float scale, const int64_t* rows, int64_t n_rows, double* out_rows,
                    double* lse_rows, int nthreads) {
    problem p = make_problem(q, k, v, dtype, mask, B, H, S, D, block_q, block_k, scale);
    return run_rows(&p, rows, n_rows, out_rows, lse_rows, nthreads);
}

int oracle_fwd_rows_elem(const void* q, const void* k, const void* v, int dtype,
                         const uint8_t* mask, const int32_t* pidx, const uint32_t* pbits,
                         int64_t n_tiles, int64_t B, int64_t H, int64_t S, int64_t D,
                         int64_t block_q, int64_t block_k, float scale, const int64_t* rows,
                         int64_t n_rows, double* out_rows, double* lse_rows, int nthreads) {
    problem p = make_problem(q, k, v, dtype, mask, B, H, S, D, block_q, block_k, scale);
    if (!pidx) return 1;
    p.pidx = pidx;
    p.pbits = pbits;
    p.n_tiles = n_tiles;
    return run_rows(&p, rows, n_rows, out_rows, lse_rows, nthreads);
}

/* ---- backward ---------------------------------------------------------- */

/* Pass A for one query row: lse and delta of the row, and (if dq_row) its dq.
 * sbuf holds S doubles, pbuf S doubles. */
static void bwd_row(const problem* p, const void* dout, int64_t bh, int64_t s, double* lse_out,
                    double* delta_out, double* dq_row, double* sbuf, double* pbuf) {
    const int64_t D = p->D;
    const int64_t qi = s / p->block_q;
    const uint8_t* mrow = p->mask + (bh * p->n_q + qi) * p->n_k;
    const int64_t qbase = (bh * p->S + s) * D;
    const int64_t brow = (bh * p->n_q + qi) * p->n_k;
    int64_t n = 0;
    double m = -INFINITY;
    for (int64_t kj = 0; kj < p->n_k; ++kj) {
        if (!mrow[kj]) continue;
        for (int64_t j = kj * p->block_k; j < (kj + 1) * p->block_k; ++j) {
            if (!kept(p, mrow[kj], brow + kj, s, j)) continue;
            const int64_t kbase = (bh * p->S + j) * D;
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d)
                dot += widen(p->q, p->dtype, qbase + d) * widen(p->k, p->dtype, kbase + d);
            sbuf[n] = p->scale * dot;
            if (sbuf[n] > m) m = sbuf[n];
            ++n;
        }
    }
    if (dq_row)
        for (int64_t d = 0; d < D; ++d) dq_row[d] = 0.0;
    if (n == 0) {
        *lse_out = -INFINITY;
        *delta_out = 0.0;
        return;
    }
    double l = 0.0;
    for (int64_t t = 0; t < n; ++t) l += exp(sbuf[t] - m);
    const double lse = m + log(l);
    /* P and dP of the active keys; delta */
    double delta = 0.0;
    int64_t t = 0;
    for (int64_t kj = 0; kj < p->n_k; ++kj) {
        if (!mrow[kj]) continue;
        for (int64_t j = kj * p->block_k; j < (kj + 1) * p->block_k; ++j) {
            if (!kept(p, mrow[kj], brow + kj, s, j)) continue;
            const int64_t vbase = (bh * p->S + j) * D;
            double dp = 0.0;
            for (int64_t d = 0; d < D; ++d)
                dp += widen(dout, p->dtype, qbase + d) * widen(p->v, p->dtype, vbase + d);
            sbuf[t] = exp(sbuf[t] - lse); /* P */
            pbuf[t] = dp;                  /* dP */
            delta += sbuf[t] * dp;
            ++t;
        }
    }
    *lse_out = lse;
    *delta_out = delta;
    if (!dq_row) return;
    t = 0;
    for (int64_t kj = 0; kj < p->n_k; ++kj) {
        if (!mrow[kj]) continue;
        for (int64_t j = kj * p->block_k; j < (kj + 1) * p->block_k; ++j) {
            if (!kept(p, mrow[kj], brow + kj, s, j)) continue;
            const int64_t kbase = (bh * p->S + j) * D;
            const double ds = sbuf[t] * (pbuf[t] - delta);
            for (int64_t d = 0; d < D; ++d) dq_row[d] += ds * widen(p->k, p->dtype, kbase + d);
            ++t;
        }
    }
    for (int64_t d = 0; d < D; ++d) dq_row[d] *= p->scale;
}

/* Pass B for one key row j of head bh: dk and dv from the query rows whose block
 * sees j's block.  lse and delta are the head's per-row values from pass A. */
static void bwd_key(const problem* p, const void* dout, int64_t bh, int64_t j, const double* lse,
                    const double* delta, double* dk_row, double* dv_row) {
    const int64_t D = p->D, kj = j / p->block_k;
    const int64_t kbase = (bh * p->S + j) * D;
    for (int64_t d = 0; d < D; ++d) dk_row[d] = dv_row[d] = 0.0;
    for (int64_t qi = 0; qi < p->n_q; ++qi) {
        const int64_t bi = (bh * p->n_q + qi) * p->n_k + kj;
        if (!p->mask[bi]) continue;
        for (int64_t r = qi * p->block_q; r < (qi + 1) * p->block_q; ++r) {
            if (!kept(p, p->mask[bi], bi, r, j)) continue;
            const int64_t qbase = (bh * p->S + r) * D;
            double dot = 0.0, dp = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                dot += widen(p->q, p->dtype, qbase + d) * widen(p->k, p->dtype, kbase + d);
                dp += widen(dout, p->dtype, qbase + d) * widen(p->v, p->dtype, kbase + d);
            }
            const double P = exp(p->scale * dot - lse[r]);
            const double ds = P * (dp - delta[r]);
            for (int64_t d = 0; d < D; ++d) {
                dv_row[d] += P * widen(dout, p->dtype, qbase + d);
                dk_row[d] += ds * widen(p->q, p->dtype, qbase + d);
            }
        }
    }
    for (int64_t d = 0; d < D; ++d) dk_row[d] *= p->scale;
}

/* Pass A over every query row of the heads flagged in want (NULL = all heads):
 * lse and delta into [B*H*S] arrays. */
static int bwd_stats(const problem* p, const void* dout, const uint8_t* want, double* lse,
                     double* delta) {
    const int64_t S = p->S, rows = p->B * p->H * S;
    int failed = 0;
#pragma omp parallel
    {
        double* sbuf = (double*)malloc(sizeof(double) * (size_t)S);
        double* pbuf = (double*)malloc(sizeof(double) * (size_t)S);
        if (!sbuf || !pbuf) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < rows; ++r)
                if (!want || want[r / S]) bwd_row(p, dout, r / S, r % S, lse + r, delta + r, NULL, sbuf, pbuf);
        }
        free(sbuf);
        free(pbuf);
    }
    return failed;
}

/* Full backward: dq, dk, dv are double[B][H][S][D]. */
static int run_bwd(const problem* pp, const void* dout, double* dq, double* dk, double* dv, int nthreads) {
    const problem p = *pp;
    const int64_t B = p.B, H = p.H, S = p.S, D = p.D;
    int rc = check(&p);
    if (rc) return rc;
    if (!dout || !dq || !dk || !dv) return 1;
    set_threads(nthreads);
    const int64_t rows = B * H * S;
    double* lse = (double*)malloc(sizeof(double) * (size_t)rows);
    double* delta = (double*)malloc(sizeof(double) * (size_t)rows);
    int failed = !lse || !delta;
    if (!failed) {
#pragma omp parallel
        {
            double* sbuf = (double*)malloc(sizeof(double) * (size_t)S);
            double* pbuf = (double*)malloc(sizeof(double) * (size_t)S);
            if (!sbuf || !pbuf) {
#pragma omp atomic write
                failed = 1;
            } else {
#pragma omp for schedule(dynamic, 16)
                for (int64_t r = 0; r < rows; ++r)
                    bwd_row(&p, dout, r / S, r % S, lse + r, delta + r, dq + r * D, sbuf, pbuf);
            }
            free(sbuf);
            free(pbuf);
        }
    }
    if (!failed) {
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t r = 0; r < rows; ++r) {
            const int64_t bh = r / S;
            bwd_key(&p, dout, bh, r % S, lse + bh * S, delta + bh * S, dk + r * D, dv + r * D);
        }
    }
    free(lse);
    free(delta);
    return failed ? 9 : 0;
}

int oracle_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype,
               const uint8_t* mask, int64_t B, int64_t H, int64_t S, int64_t D, int64_t block_q,
               int64_t block_k, float scale, double* dq, double* dk, double* dv, int nthreads) {
    problem p = make_problem(q, k, v, dtype, mask, B, H, S, D, block_q, block_k, scale);
    return run_bwd(&p, dout, dq, dk, dv, nthreads);
}

/* The backward with an element-level mask (block states, pidx, bit tiles as in
 * oracle_fwd_elem): the same formulas over the kept (query, key) pairs only. */
int oracle_bwd_elem(const void* q, const void* k, const void* v, const void* dout, int dtype,
                    const uint8_t* mask, const int32_t* pidx, const uint32_t* pbits, int64_t n_tiles,
                    int64_t B, int64_t H, int64_t S, int64_t D, int64_t block_q, int64_t block_k,
                    float scale, double* dq, double* dk, double* dv, int nthreads) {
    problem p = make_problem(q, k, v, dtype, mask, B, H, S, D, block_q, block_k, scale);
    if (!pidx) return 1;
    p.pidx = pidx;
    p.pbits = pbits;
    p.n_tiles = n_tiles;
    return run_bwd(&p, dout, dq, dk, dv, nthreads);
}

/* Sampled backward: dq of the flat query rows q_rows[i] = (b*H + h)*S + s into
 * dq_rows[n_q_rows][D]; dk and dv of the flat key rows k_rows[i] into
 * dk_rows / dv_rows [n_k_rows][D].  Pass A runs only over the heads that hold a
 * sampled key row. */
static int run_bwd_sample(const problem* pp, const void* dout, const int64_t* q_rows, int64_t n_q_rows,
                          double* dq_rows, const int64_t* k_rows, int64_t n_k_rows, double* dk_rows,
                          double* dv_rows, int nthreads) {
    const problem p = *pp;
    const int64_t B = p.B, H = p.H, S = p.S, D = p.D;
    int rc = check(&p);
    if (rc) return rc;
    if (!dout || (n_q_rows > 0 && (!q_rows || !dq_rows)) ||
        (n_k_rows > 0 && (!k_rows || !dk_rows || !dv_rows)))
        return 1;
    const int64_t rows = B * H * S;
    for (int64_t i = 0; i < n_q_rows; ++i)
        if (q_rows[i] < 0 || q_rows[i] >= rows) return 2;
    for (int64_t i = 0; i < n_k_rows; ++i)
        if (k_rows[i] < 0 || k_rows[i] >= rows) return 2;
    set_threads(nthreads);
    int failed = 0;
#pragma omp parallel
    {
        double* sbuf = (double*)malloc(sizeof(double) * (size_t)S);
        double* pbuf = (double*)malloc(sizeof(double) * (size_t)S);
        if (!sbuf || !pbuf) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t i = 0; i < n_q_rows; ++i) {
                double lse, delta;
                bwd_row(&p, dout, q_rows[i] / S, q_rows[i] % S, &lse, &delta, dq_rows + i * D, sbuf, pbuf);
            }
        }
        free(sbuf);
        free(pbuf);
    }
    if (failed || n_k_rows == 0) return failed ? 9 : 0;
    uint8_t* want = (uint8_t*)calloc((size_t)(B * H), 1);
    double* lse = (double*)malloc(sizeof(double) * (size_t)rows);
    double* delta = (double*)malloc(sizeof(double) * (size_t)rows);
    failed = !want || !lse || !delta;
    if (!failed) {
        for (int64_t i = 0; i < n_k_rows; ++i) want[k_rows[i] / S] = 1;
        failed = bwd_stats(&p, dout, want, lse, delta);
    }
    if (!failed) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t i = 0; i < n_k_rows; ++i) {
            const int64_t bh = k_rows[i] / S;
            bwd_key(&p, dout, bh, k_rows[i] % S, lse + bh * S, delta + bh * S, dk_rows + i * D,
                    dv_rows + i * D);
        }
    }
    free(want);
    free(lse);
    free(delta);
    return failed ? 9 : 0;
}

int oracle_bwd_sample(const void* q, const void* k, const void* v, const void* dout, int dtype,
                      const uint8_t* mask, int64_t B, int64_t H, int64_t S, int64_t D,
                      int64_t block_q, int64_t block_k, float scale, const int64_t* q_rows,
                      int64_t n_q_rows, double* dq_rows, const int64_t* k_rows, int64_t n_k_rows,
                      double* dk_rows, double* dv_rows, int nthreads) {
    problem p = make_problem(q, k, v, dtype, mask, B, H, S, D, block_q, block_k, scale);
    return run_bwd_sample(&p, dout, q_rows, n_q_rows, dq_rows, k_rows, n_k_rows, dk_rows, dv_rows, nthreads);
}

int oracle_bwd_sample_elem(const void* q, const void* k, const void* v, const void* dout, int dtype,
                           const uint8_t* mask, const int32_t* pidx, const uint32_t* pbits, int64_t n_tiles,
                           int64_t B, int64_t H, int64_t S, int64_t D, int64_t block_q, int64_t block_k,
                           float scale, const int64_t* q_rows, int64_t n_q_rows, double* dq_rows,
                           const int64_t* k_rows, int64_t n_k_rows, double* dk_rows, double* dv_rows,
                           int nthreads) {
    problem p = make_problem(q, k, v, dtype, mask, B, H, S, D, block_q, block_k, scale);
    if (!pidx) return 1;
    p.pidx = pidx;
    p.pbits = pbits;
    p.n_tiles = n_tiles;
    return run_bwd_sample(&p, dout, q_rows, n_q_rows, dq_rows, k_rows, n_k_rows, dk_rows, dv_rows, nthreads);
}

/* Dense probability matrix P[b][h][s][j] (zero where masked), for tiny shapes:
 * the row softmax weights exp(s_j - m)/l of the definition above.  An empty row
 * is all zeros. */
int oracle_probs(const void* q, const void* k, const void* v, int dtype, const uint8_t* mask,
                 int64_t B, int64_t H, int64_t S, int64_t D, int64_t block_q, int64_t block_k,
                 float scale, double* P) {
    problem p = make_problem(q, k, v, dtype, mask, B, H, S, D, block_q, block_k, scale);
    int rc = check(&p);
    if (rc) return rc;
    if (!P) return 1;
    double* sbuf = (double*)malloc(sizeof(double) * (size_t)S);
    if (!sbuf) return 9;
    for (int64_t bh = 0; bh < B * H; ++bh) {
        for (int64_t s = 0; s < S; ++s) {
            double* prow = P + (bh * S + s) * S;
            for (int64_t j = 0; j < S; ++j) prow[j] = 0.0;
            const int64_t qi = s / block_q;
            const uint8_t* mrow = mask + (bh * p.n_q + qi) * p.n_k;
            const int64_t qbase = (bh * S + s) * D;
            double m = -INFINITY;
            int64_t n = 0;
            for (int64_t j = 0; j < S; ++j) {
                sbuf[j] = -INFINITY;
                if (!mrow[j / block_k]) continue;
                const int64_t kbase = (bh * S + j) * D;
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += widen(q, dtype, qbase + d) * widen(k, dtype, kbase + d);
                sbuf[j] = p.scale * dot;
                if (sbuf[j] > m) m = sbuf[j];
                ++n;
            }
            if (n == 0) continue;
            double l = 0.0;
            for (int64_t j = 0; j < S; ++j)
                if (mrow[j / block_k]) l += exp(sbuf[j] - m);
            for (int64_t j = 0; j < S; ++j)
                if (mrow[j / block_k]) prow[j] = exp(sbuf[j] - m) / l;
        }
    }
    free(sbuf);
    return 0;
}

/* Compaction of a block mask with n_rows rows of n_k bytes into CSR.
 * row_ptr holds n_rows+1 entries; col_idx must hold n_rows*n_k entries.
 * Returns the number of active blocks (nnz), or -1 on a bad argument. */
int64_t oracle_compact(const uint8_t* mask, int64_t n_rows, int64_t n_k, int32_t* row_ptr,
                       int32_t* col_idx) {
    if (!mask || !row_ptr || !col_idx || n_rows < 0 || n_k <= 0) return -1;
    int64_t nnz = 0;
    row_ptr[0] = 0;
    for (int64_t r = 0; r < n_rows; ++r) {
        for (int64_t kj = 0; kj < n_k; ++kj)
            if (mask[r * n_k + kj]) col_idx[nnz++] = (int32_t)kj;
        row_ptr[r + 1] = (int32_t)nnz;
    }
    return nnz;
}

int oracle_max_threads(void) { return default_threads(); }

/* Ragged dot: out is double[M][N].  Returns 0 on success, nonzero on a bad
 * argument (nothing written).
 *
 * Group sizes the page leaves open (it assumes sizes that tile the rows):
 * group g takes the next rows in order; a negative size counts as 0 rows, and
 * a group takes at most the rows that remain (so the sizes never reach past
 * row M - 1); rows after the last group's are 0. */
int oracle_ragged_dot(const void* lhs, const void* rhs, int dtype, const int32_t* group_sizes,
                      int64_t G, int64_t M, int64_t K, int64_t N, double* out, int nthreads) {
    if (!lhs || !rhs || !group_sizes || !out) return 1;
    if (G <= 0 || M < 0 || K <= 0 || N <= 0) return 2;
    if (dtype < ORC_F32 || dtype > ORC_FP8) return 3;
    set_threads(nthreads);
    int64_t start = 0;
    for (int64_t g = 0; g < G; ++g) {
        int64_t rows = group_sizes[g] < 0 ? 0 : (int64_t)group_sizes[g];
        if (rows > M - start) rows = M - start;
        const int64_t end = start + rows;
#pragma omp parallel for schedule(static)
        for (int64_t i = start; i < end; ++i)
            for (int64_t n = 0; n < N; ++n) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    acc += widen(lhs, dtype, i * K + k) * widen(rhs, dtype, (g * K + k) * N + n);
                out[i * N + n] = acc;
            }
        start = end;
    }
    for (int64_t i = start; i < M; ++i)
        for (int64_t n = 0; n < N; ++n) out[i * N + n] = 0.0;
    return 0;
}
