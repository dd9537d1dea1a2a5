/*
 * CPU oracle for D = alpha * A * B + beta * C   (TEST INFRASTRUCTURE ONLY)
 *
 * A plain, slow, obviously correct fp64 implementation of the general matrix
 * multiply with the fused bias / activation epilogue. Only the test-suite, the smoke check
 * and the benchmark's CPU-baseline leg load this library; the GPU library
 * never links or calls it, and it shares no code with the GPU library.
 *
 * What it follows on the pages:
 *   - "CUTLASS Python 接口全解析" (gsyq.cn), section 2: plan.run computes
 *     D = A * B + C; section 2.1: element_A/B/C/D/accumulator are separate
 *     types bound to the plan, layouts RowMajor/ColumnMajor; section 2.3:
 *     an elementwise activation (ReLU) fused into the epilogue.
 *   - "CUTLASS Python接口" (kwkr.cn), section 3.3: D = alpha * A * B + beta * C
 *     with fp32 accumulation; section 5.2: the activation is applied to the
 *     result of the linear combination.
 *   - "Python packages associated with CUTLASS", Current functionality:
 *     GEMM, fused elementwise epilogue, grouped GEMM (independent problems).
 *   - "Generating State-of-the-Art GEMMs with TorchInductor's CuteDSL backend",
 *     section 5.1: FP8 GEMM as a scaled mm (per-tensor scales here);
 *     section 7: the epilogue-fusion kernels take activations ReLU, Sigmoid
 *     and Tanh.
 *   - "CUTLASS Python接口" (kwkr.cn), the fused BiasAdd-ReLU GEMM example:
 *     Output = Activation(Input * Weight + Bias), Bias a length-N vector
 *     added to every row.
 *   - "Generating State-of-the-Art GEMMs with TorchInductor's CuteDSL
 *     backend", section 7 (epilogue fusion): the fusion kernels load and
 *     store auxiliary tensors and apply elementwise add, multiply, subtract
 *     and divide besides the activations.
 *   - "Generating State-of-the-Art GEMMs with TorchInductor's CuteDSL
 *     backend", sections 5.1 (feature list: the scaled mm family for MXFP8,
 *     with its own scale type, block size and layout) and 5.2 (MXFP8
 *     results). The pages name the format only; its definition is taken from
 *     the OCP Microscaling (MX) specification v1.0: 32 consecutive elements
 *     along K share one E8M0 scale (an 8-bit biased power of two, bias 127,
 *     0xFF = NaN), the elements are e4m3.
 *
 * Definition computed, for each selected output (i, j):
 *   acc     = sum_{k=0}^{K-1} a(i,k) * b(k,j)            fp64, increasing k
 *             MX: each product also times X_A(i, k/32) * X_B(j, k/32), the
 *             decoded E8M0 scales of A's row i and B's column j for the
 *             32-element block holding k
 *   acc     = acc * s_A * s_B                             (scales; 1 unless fp8)
 *   v       = alpha * acc + (beta != 0 ? beta * c(i,j) : 0) + bias(j)
 *             (bias(j) = 0 without a bias vector)
 *   act     : identity; ReLU: v > 0 ? v : +0; Sigmoid: 1/(1+e^-v);
 *             Tanh: tanh(v)  (all in fp64)
 *   without an auxiliary tensor: D = act(v)
 *   with an auxiliary M x N tensor X (element_C, layout_C) and an
 *   elementwise op in {add, sub, mul, div} (y op x = y + x, y - x, y * x,
 *   y / x):
 *             before the activation: z = v op X(i,j),  D = act(z)
 *             after the activation:  z = v,            D = act(v) op X(i,j)
 *             and the auxiliary store Z(i,j) = z (the activation's input),
 *             rounded once to element_D; without X, z = v
 *   ref     = D                                           (fp64, unrounded)
 *   d_exact = D rounded once, to nearest even, to element_D
 *   S       = |alpha * s_A * s_B| * sum_k |a(i,k) * b(k,j)|  (tolerance scale;
 *             MX: the scaled products); a mul multiplies it by |X(i,j)|, a
 *             div divides it by |X(i,j)| -- for D, and for Z when the op
 *             comes before the activation
 * Operands are decoded exactly from their storage bits by this file's own
 * decoders; products of fp32/fp16/bf16/e4m3 values are exact in fp64.
 * Layouts: RowMajor X[r][c] = base[r*cols + c]; ColumnMajor X[r][c] =
 * base[r + c*rows] (packed operands, leading dimension implied).
 * MX scales: X_A is [M][K/32] and X_B is [N][K/32] bytes, row-major, whatever
 * the layouts of A and B.
 * MXFP4 ("Generating State-of-the-Art GEMMs with TorchInductor's CuteDSL
 * backend", section 5.1 lists MXF4 beside MXFP8 in the scaled mm family): the
 * elements are OCP FP4 E2M1 (OCP MX v1.0: sign, 2 exponent bits with bias 1,
 * 1 fraction bit; values 0, 1/2, 1, 3/2, 2, 3, 4, 6 and their negatives), two
 * per byte in the operand's storage order, element 2t in the low nibble of
 * byte t; the same E8M0 block scales as MXFP8.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_F8E4M3 = 3, DT_E8M0 = 4, DT_F4E2M1 = 5 };
enum { LAYOUT_ROW = 0, LAYOUT_COL = 1 };
enum { ACT_IDENTITY = 0, ACT_RELU = 1, ACT_SIGMOID = 2, ACT_TANH = 3 };
enum { AUX_ADD = 0, AUX_SUB = 1, AUX_MUL = 2, AUX_DIV = 3 };
enum { AUX_BEFORE_ACT = 0, AUX_AFTER_ACT = 1 };

/* ---- exact decoders, one per storage format (sign, exponent, fraction) ---- */

static double dec_f32(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double dec_f16(uint32_t u) {
    int s = (u >> 15) & 1, e = (u >> 10) & 31, m = u & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);
    return s ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
static double dec_bf16(uint32_t u) {
    int s = (u >> 15) & 1, e = (u >> 7) & 255, m = u & 127;
    double v;
    if (e == 0) v = ldexp((double)m, -133);
    else if (e == 255) v = m ? NAN : INFINITY;
    else v = ldexp((double)(128 + m), e - 134);
    return s ? -v : v;
}

/* OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent (bias 7), 3 fraction bits;
 * no infinities, S.1111.111 is NaN, largest finite 448. */
static double dec_e4m3(uint32_t u) {
    int s = (u >> 7) & 1, e = (u >> 3) & 15, m = u & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* OCP MX FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 fraction bit; exponent
 * field 0 holds the subnormals 0 and 1/2; no infinities and no NaN, the
 * largest magnitude is 6. */
static double dec_e2m1(uint32_t u) {
    int s = (u >> 3) & 1, e = (u >> 1) & 3, m = u & 1;
    double v = (e == 0) ? ldexp((double)m, -1) : ldexp((double)(2 + m), e - 2);
    return s ? -v : v;
}

/* OCP MX E8M0 scale: 8 exponent bits (bias 127), no sign, no fraction;
 * 0xFF is NaN, 0x00 is 2^-127. */
static double dec_e8m0(uint32_t u) {
    u &= 255u;
    return u == 255u ? NAN : ldexp(1.0, (int)u - 127);
}

double oracle_decode(int dtype, uint32_t bits) {
    switch (dtype) {
    case DT_F32: return dec_f32(bits);
    case DT_F16: return dec_f16(bits);
    case DT_BF16: return dec_bf16(bits);
    case DT_F8E4M3: return dec_e4m3(bits);
    case DT_E8M0: return dec_e8m0(bits);
    case DT_F4E2M1: return dec_e2m1(bits);
    }
    return NAN;
}

/* ---- one rounding, to nearest even, from fp64 into fp32 / fp16 / bf16 ---- */

uint32_t oracle_encode(int dtype, double v) {
    int p, emin, emax, bias, ebits;
    switch (dtype) {
    case DT_F32: p = 24; emin = -126; emax = 127; bias = 127; ebits = 8; break;
    case DT_F16: p = 11; emin = -14; emax = 15; bias = 15; ebits = 5; break;
    case DT_BF16: p = 8; emin = -126; emax = 127; bias = 127; ebits = 8; break;
    default: return 0xFFFFFFFFu;
    }
    const int fbits = p - 1;
    const uint32_t sign = signbit(v) ? (1u << (ebits + fbits)) : 0u;
    const uint32_t exp_all = ((1u << ebits) - 1u) << fbits;
    if (isnan(v)) return exp_all | (1u << (fbits - 1));      /* quiet NaN */
    double a = fabs(v);
    if (isinf(a)) return sign | exp_all;
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);                 /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;                /* a in [2^E, 2^(E+1)) */
    if (E < emin) E = emin;        /* subnormal range shares emin's quantum */
    double m = ldexp(a, fbits - E);            /* exact: power-of-two scale */
    double mr = nearbyint(m);                  /* ties to even (default mode) */
    if (mr >= ldexp(1.0, p)) { E += 1; mr = ldexp(1.0, fbits); }
    if (E > emax) return sign | exp_all;       /* overflow -> infinity */
    uint32_t mant = (uint32_t)mr;
    if (mant < (1u << fbits)) return sign | mant;   /* subnormal (or zero) */
    return sign | ((uint32_t)(E + bias) << fbits) | (mant - (1u << fbits));
}

/* ---- storage access -------------------------------------------------------- */

static uint32_t load_bits(const void *base, int dtype, int64_t idx) {
    switch (dtype) {
    case DT_F32: return ((const uint32_t *)base)[idx];
    case DT_F16:
    case DT_BF16: return ((const uint16_t *)base)[idx];
    case DT_F8E4M3: return ((const uint8_t *)base)[idx];
    case DT_F4E2M1: {   /* two per byte: element 2t in the low nibble of byte t */
        const uint8_t b = ((const uint8_t *)base)[idx >> 1];
        return (idx & 1) ? (uint32_t)(b >> 4) : (uint32_t)(b & 15u);
    }
    }
    return 0;
}

/* Element (r, c) of a rows x cols operand stored packed in `layout`. */
static double elem(const void *base, int dtype, int layout, int64_t rows,
                   int64_t cols, int64_t r, int64_t c) {
    int64_t idx = (layout == LAYOUT_ROW) ? r * cols + c : r + c * rows;
    return oracle_decode(dtype, load_bits(base, dtype, idx));
}

static int valid_dtype(int d) { return (d >= DT_F32 && d <= DT_F8E4M3) || d == DT_F4E2M1; }

/* MX block size along K (OCP MX v1.0). */
#define MX_BLOCK 32

/* X(r, k/32) of an MX scale array [rows][K/32], or 1 without one. */
static double mx_scale(const uint8_t *x, int64_t K, int64_t r, int64_t k) {
    return x ? oracle_decode(DT_E8M0, x[r * (K / MX_BLOCK) + k / MX_BLOCK]) : 1.0;
}

/* MX needs e4m3 or e2m1 elements (the same for A and B) and whole blocks;
 * both arrays or neither. e2m1 exists only as MX elements. */
static int mx_ok(const uint8_t *xa, const uint8_t *xb, int dtA, int dtB, int64_t K) {
    if (!xa && !xb) return dtA != DT_F4E2M1 && dtB != DT_F4E2M1;
    return xa && xb && dtA == dtB && (dtA == DT_F8E4M3 || dtA == DT_F4E2M1) &&
           K % MX_BLOCK == 0;
}

/* The activation of the epilogue, in fp64. */
static double activate(double v, int act) {
    switch (act) {
    case ACT_RELU: return (v > 0.0) ? v : 0.0;
    case ACT_SIGMOID: return 1.0 / (1.0 + exp(-v));
    case ACT_TANH: return tanh(v);
    default: return v;
    }
}

/* y op x for the auxiliary elementwise op. */
static double aux_apply(double y, double x, int op) {
    switch (op) {
    case AUX_SUB: return y - x;
    case AUX_MUL: return y * x;
    case AUX_DIV: return y / x;
    default: return y + x;
    }
}

/* How the op scales an error already in y (the tolerance scale). */
static double aux_scale(double s, double x, int op) {
    if (op == AUX_MUL) return s * fabs(x);
    if (op == AUX_DIV) return s / fabs(x);
    return s;
}

/* Everything an output's epilogue needs besides its own accumulator. */
typedef struct {
    double sab, alpha, beta;
    int act;
    const void *aux;      /* X, or NULL */
    int aux_op, aux_pos;
} epi_t;

/* Epilogue of one output: scales, linear combination, bias, then the
 * auxiliary op on its side of the activation. Returns D's value; *z gets the
 * activation's input; *sd and *sz the tolerance scales of D and Z, starting
 * from the accumulator's s_acc. */
static double finish(const epi_t *e, double acc, double s_acc, double c,
                     double bias, double x, double *z, double *sd, double *sz) {
    double v = e->alpha * (acc * e->sab);
    if (e->beta != 0.0) v += e->beta * c;
    v += bias;
    double s = s_acc;
    if (e->aux && e->aux_pos == AUX_BEFORE_ACT) {
        v = aux_apply(v, x, e->aux_op);
        s = aux_scale(s, x, e->aux_op);
    }
    *z = v;
    *sz = s;
    double d = activate(v, e->act);
    if (e->aux && e->aux_pos == AUX_AFTER_ACT) {
        d = aux_apply(d, x, e->aux_op);
        s = aux_scale(s, x, e->aux_op);
    }
    *sd = s;
    return d;
}

/* bias(j): element j of the length-N vector in element type dtype, or 0. */
static double bias_at(const void *bias, int dtype, int64_t j) {
    return bias ? oracle_decode(dtype, load_bits(bias, dtype, j)) : 0.0;
}

/* Outputs of one (i, j): D's fp64 value, scale and bits; Z's likewise. */
typedef struct {
    double *ref, *S, *z_ref, *z_S;
    uint32_t *d_bits, *z_bits;
} out_t;

static void put(const out_t *o, int dtD, int64_t t, double d, double sd,
                double z, double sz) {
    o->ref[t] = d;
    if (o->S) o->S[t] = sd;
    if (o->d_bits) o->d_bits[t] = oracle_encode(dtD, d);
    if (o->z_ref) o->z_ref[t] = z;
    if (o->z_S) o->z_S[t] = sz;
    if (o->z_bits) o->z_bits[t] = oracle_encode(dtD, z);
}

static int args_ok(int dtA, int dtB, int dtC, int dtD, int act, int64_t M,
                   int64_t N, int64_t K, const uint8_t *xa, const uint8_t *xb,
                   int aux_op, int aux_pos) {
    return valid_dtype(dtA) && valid_dtype(dtB) && valid_dtype(dtC) &&
           valid_dtype(dtD) && M >= 0 && N >= 0 && K >= 0 &&
           act >= ACT_IDENTITY && act <= ACT_TANH && mx_ok(xa, xb, dtA, dtB, K) &&
           aux_op >= AUX_ADD && aux_op <= AUX_DIV &&
           (aux_pos == AUX_BEFORE_ACT || aux_pos == AUX_AFTER_ACT);
}

/*
 * Rows mode: computes every column j of each row i listed in `rows`
 * (rows == NULL selects all M rows in order). Outputs are dense row-major
 * [n_rows][N]: ref (fp64), S (fp64, optional), d_bits (element_D bits,
 * optional), and for the auxiliary store z_ref, z_S, z_bits (optional).
 * aux (M x N, element_C, layout_C) may be NULL. Returns 0 on success, -1 on
 * bad arguments.
 */
int oracle_gemm_rows(int dtA, int dtB, int dtC, int dtD, int la, int lb,
                     int lc, int act, int64_t M, int64_t N, int64_t K,
                     const void *A, const void *B, const void *C,
                     const void *bias, const uint8_t *xa, const uint8_t *xb,
                     const void *aux, int aux_op, int aux_pos,
                     float alpha, float beta, float scale_a, float scale_b,
                     const int64_t *rows, int64_t n_rows, double *ref,
                     double *S, uint32_t *d_bits, double *z_ref, double *z_S,
                     uint32_t *z_bits) {
    if (!ref || !args_ok(dtA, dtB, dtC, dtD, act, M, N, K, xa, xb, aux_op, aux_pos))
        return -1;
    if (rows == NULL) n_rows = M;
    const epi_t e = {(double)scale_a * (double)scale_b, (double)alpha, (double)beta,
                     act, aux, aux_op, aux_pos};
    const out_t o = {ref, S, z_ref, z_S, d_bits, z_bits};
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t i = rows ? rows[r] : r;
        if (i < 0 || i >= M) { bad = 1; continue; }
        double *acc = (double *)calloc((size_t)(N ? N : 1), sizeof(double));
        double *sab_abs = (double *)calloc((size_t)(N ? N : 1), sizeof(double));
        for (int64_t k = 0; k < K; ++k) {
            double a = elem(A, dtA, la, M, K, i, k) * mx_scale(xa, K, i, k);
            for (int64_t j = 0; j < N; ++j) {
                double p = a * (elem(B, dtB, lb, K, N, k, j) * mx_scale(xb, K, j, k));
                acc[j] += p;
                sab_abs[j] += fabs(p);
            }
        }
        for (int64_t j = 0; j < N; ++j) {
            double c = (e.beta != 0.0) ? elem(C, dtC, lc, M, N, i, j) : 0.0;
            double x = aux ? elem(aux, dtC, lc, M, N, i, j) : 0.0;
            double z, sd, sz;
            double d = finish(&e, acc[j], fabs(e.alpha * e.sab) * sab_abs[j], c,
                              bias_at(bias, dtC, j), x, &z, &sd, &sz);
            put(&o, dtD, r * N + j, d, sd, z, sz);
        }
        free(acc);
        free(sab_abs);
    }
    return bad ? -1 : 0;
}

/*
 * Entries mode: computes the n listed outputs (ii[t], jj[t]) one by one.
 * Outputs ref[t], S[t], d_bits[t], z_ref[t], z_S[t], z_bits[t] (all but ref
 * optional).
 */
int oracle_gemm_entries(int dtA, int dtB, int dtC, int dtD, int la, int lb,
                        int lc, int act, int64_t M, int64_t N, int64_t K,
                        const void *A, const void *B, const void *C,
                        const void *bias, const uint8_t *xa, const uint8_t *xb,
                        const void *aux, int aux_op, int aux_pos,
                        float alpha, float beta, float scale_a, float scale_b,
                        const int64_t *ii, const int64_t *jj, int64_t n,
                        double *ref, double *S, uint32_t *d_bits, double *z_ref,
                        double *z_S, uint32_t *z_bits) {
    if (!ref || !ii || !jj ||
        !args_ok(dtA, dtB, dtC, dtD, act, M, N, K, xa, xb, aux_op, aux_pos))
        return -1;
    const epi_t e = {(double)scale_a * (double)scale_b, (double)alpha, (double)beta,
                     act, aux, aux_op, aux_pos};
    const out_t o = {ref, S, z_ref, z_S, d_bits, z_bits};
    int bad = 0;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < n; ++t) {
        int64_t i = ii[t], j = jj[t];
        if (i < 0 || i >= M || j < 0 || j >= N) { bad = 1; continue; }
        double acc = 0.0, sabs = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = (elem(A, dtA, la, M, K, i, k) * mx_scale(xa, K, i, k)) *
                       (elem(B, dtB, lb, K, N, k, j) * mx_scale(xb, K, j, k));
            acc += p;
            sabs += fabs(p);
        }
        double c = (e.beta != 0.0) ? elem(C, dtC, lc, M, N, i, j) : 0.0;
        double x = aux ? elem(aux, dtC, lc, M, N, i, j) : 0.0;
        double z, sd, sz;
        double d = finish(&e, acc, fabs(e.alpha * e.sab) * sabs, c,
                          bias_at(bias, dtC, j), x, &z, &sd, &sz);
        put(&o, dtD, t, d, sd, z, sz);
    }
    return bad ? -1 : 0;
}

/* Vector helpers for the tests: decode / encode n values. */
void oracle_decode_n(int dtype, const uint32_t *bits, int64_t n, double *out) {
    for (int64_t t = 0; t < n; ++t) out[t] = oracle_decode(dtype, bits[t]);
}

void oracle_encode_n(int dtype, const double *v, int64_t n, uint32_t *out) {
    for (int64_t t = 0; t < n; ++t) out[t] = oracle_encode(dtype, v[t]);
}
