/*
 * Oracle for the multi-adapter LoRA-linear layer.  TEST INFRASTRUCTURE ONLY:
 * tests, the smoke check and the benchmark's CPU-baseline leg call it; the
 * product library never links, loads or calls it.
 *
 * What it computes, for every requested row t and output column n:
 *
 *   y[t,n] = sum_k x[t,k] * W0[n,k]
 *          + [a(t) != none] * (alpha_a / r_a) * sum_j B_a[j,n] * ( sum_k x[t,k] * A_a[j,k] )
 *
 * This is the LoRA forward pass y = W0 x + (alpha / r) B A x of
 * "S-LoRA: Serving Thousands of Concurrent Adapters in 2026" (section "The
 * Three Core Pillars of Multi-LoRA Serving", first pillar), applied per row
 * with the row's own adapter as in "Multi-LoRA serving: S-LoRA, Punica and
 * adapter batching" (section "How the kernels work": shrink v = A x, expand
 * y += gamma B v) and with rows that name no adapter left at the base output
 * (the demo's Step 2, where the adapter id None means the un-adapted base).
 * W0 is stored [d_out][d_in] (the demo's base_weight layout); A_a is r rows of
 * length d_in; B_a is stored as r rows of length d_out (row j holds the j-th
 * column of the page's d_out x r matrix B).
 *
 * Plain loops in double precision: row t outer; the shrink sum for each j is
 * formed once per row; then each output column.  No blocking, no BLAS, no
 * reordering beyond that.  Inputs are bf16 bit patterns or fp32 values, read
 * exactly into double.  gamma = alpha / r is formed in double.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double load_elem(const void* base, int bf16, int64_t i) {
    if (bf16) {
        uint32_t u = (uint32_t)((const uint16_t*)base)[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return (double)((const float*)base)[i];
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * x        [T][d_in]     input rows
 * w0       [d_out][d_in] base weight, or NULL for a zero base term (delta only)
 * row_adapter [T]        index into the adapter arrays, or -1 for none
 * rank, alpha [n_adapters]
 * a_off, b_off [n_adapters]  element offsets of A_a in A_all and of B_a in B_all
 * rows     [n_rows]      which rows of y to compute (NULL: rows 0..n_rows-1)
 * y        [n_rows][d_out] output, double
 * returns 0, or -1 on a malformed argument (nothing written then).
 */
int oracle_lora_linear(int bf16, int64_t T, int64_t d_in, int64_t d_out,
                       const void* x, const void* w0, const int32_t* row_adapter,
                       int32_t n_adapters, const int32_t* rank, const double* alpha,
                       const int64_t* a_off, const int64_t* b_off,
                       const void* A_all, const void* B_all,
                       const int64_t* rows, int64_t n_rows, double* y) {
    if (T < 0 || d_in < 0 || d_out < 0 || n_rows < 0) return -1;
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t t = rows ? rows[i] : i;
        if (t < 0 || t >= T) return -1;
        int32_t a = row_adapter[t];
        if (a < -1 || a >= n_adapters) return -1;
        if (a >= 0 && rank[a] < 1) return -1;
    }
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t t = rows ? rows[i] : i;
        const int64_t xo = t * d_in;
        double* yrow = y + i * d_out;
        /* base term, one dense product over the whole batch */
        for (int64_t n = 0; n < d_out; ++n) {
            double s = 0.0;
            if (w0) {
                for (int64_t k = 0; k < d_in; ++k)
                    s += load_elem(x, bf16, xo + k) * load_elem(w0, bf16, n * d_in + k);
            }
            yrow[n] = s;
        }
        int32_t a = row_adapter[t];
        if (a < 0) continue; /* no adapter: the base output stands */
        const int32_t r = rank[a];
        const double gamma = alpha[a] / (double)r;
        double* v = (double*)malloc(sizeof(double) * (size_t)r);
        if (!v) {
#pragma omp atomic write
            err = 1;
            continue;
        }
        /* shrink: v_j = sum_k A_a[j,k] x[t,k] */
        for (int32_t j = 0; j < r; ++j) {
            double s = 0.0;
            for (int64_t k = 0; k < d_in; ++k)
                s += load_elem(A_all, bf16, a_off[a] + (int64_t)j * d_in + k) * load_elem(x, bf16, xo + k);
            v[j] = s;
        }
        /* expand: y[t,n] += gamma * sum_j B_a[j,n] v_j */
        for (int64_t n = 0; n < d_out; ++n) {
            double s = 0.0;
            for (int32_t j = 0; j < r; ++j)
                s += load_elem(B_all, bf16, b_off[a] + (int64_t)j * d_out + n) * v[j];
            yrow[n] += gamma * s;
        }
        free(v);
    }
    return err ? -1 : 0;
}

/*
 * FP8 base.  A quantized base with 16-bit adapters ("Multi-LoRA serving:
 * S-LoRA, Punica and adapter batching", section "Interaction with how the
 * adapters were trained": the base may be served quantized, e.g. in FP8,
 * while the adapters stay 16-bit).  Reading of what the page leaves open: the
 * base weight is stored as 8-bit E4M3 floating-point codes (1 sign bit, 4
 * exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
 * subnormals m * 2^-9; the code with all exponent and mantissa bits set is
 * NaN and there are no infinities) times one fp32 scale per output channel:
 *
 *   W0[n,k] = scale[n] * e4m3(code[n,k])
 *
 * x and the adapters are bf16, as in oracle_lora_linear; the delta is the
 * same.  Plain loops in double precision.
 */
static double e4m3_value(uint8_t code) {
    const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) {
        v = 0.0 / 0.0; /* NaN */
    } else if (e == 0) {
        v = m * (1.0 / 512.0); /* subnormal: m * 2^-9 */
    } else {
        v = (1.0 + m / 8.0);
        for (int i = 7; i < e; ++i) v *= 2.0; /* 2^(e - 7) */
        for (int i = e; i < 7; ++i) v *= 0.5;
    }
    return sign ? -v : v;
}

double oracle_e4m3_value(int code) { return e4m3_value((uint8_t)code); }

/*
 * As oracle_lora_linear (bf16 x and adapters), with the base term
 *   sum_k x[t,k] * scale[n] * e4m3(w0_code[n,k]).
 * w0_code [d_out][d_in] bytes, w0_scale [d_out] fp32 (read exactly).
 */
int oracle_lora_linear_fp8base(int64_t T, int64_t d_in, int64_t d_out,
                               const void* x, const uint8_t* w0_code, const float* w0_scale,
                               const int32_t* row_adapter, int32_t n_adapters, const int32_t* rank,
                               const double* alpha, const int64_t* a_off, const int64_t* b_off,
                               const void* A_all, const void* B_all,
                               const int64_t* rows, int64_t n_rows, double* y) {
    if (T < 0 || d_in < 0 || d_out < 0 || n_rows < 0 || !w0_code || !w0_scale) return -1;
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t t = rows ? rows[i] : i;
        if (t < 0 || t >= T) return -1;
        int32_t a = row_adapter[t];
        if (a < -1 || a >= n_adapters) return -1;
        if (a >= 0 && rank[a] < 1) return -1;
    }
    double table[256];
    for (int c = 0; c < 256; ++c) table[c] = e4m3_value((uint8_t)c);
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t t = rows ? rows[i] : i;
        const int64_t xo = t * d_in;
        double* out = y + i * d_out;
        /* base term: the decoded base weight times its channel's scale */
        for (int64_t n = 0; n < d_out; ++n) {
            const double sc = (double)w0_scale[n];
            double acc = 0.0;
            for (int64_t k = 0; k < d_in; ++k)
                acc += load_elem(x, 1, xo + k) * (sc * table[w0_code[n * d_in + k]]);
            out[n] = acc;
        }
        const int32_t ad = row_adapter[t];
        if (ad == -1) continue; /* no adapter: the base output stands */
        const int32_t rk = rank[ad];
        const double scale_ad = alpha[ad] / (double)rk;
        double* vv = (double*)malloc(sizeof(double) * (size_t)rk);
        if (!vv) {
#pragma omp atomic write
            err = 1;
            continue;
        }
        /* shrink, then expand, as in oracle_lora_linear */
        for (int32_t jj = 0; jj < rk; ++jj) {
            double acc = 0.0;
            for (int64_t kk = 0; kk < d_in; ++kk)
                acc += load_elem(x, 1, xo + kk) * load_elem(A_all, 1, a_off[ad] + jj * d_in + kk);
            vv[jj] = acc;
        }
        for (int64_t nn = 0; nn < d_out; ++nn) {
            double acc = 0.0;
            for (int32_t jj = 0; jj < rk; ++jj)
                acc += vv[jj] * load_elem(B_all, 1, b_off[ad] + jj * d_out + nn);
            out[nn] += scale_ad * acc;
        }
        free(vv);
    }
    return err ? -1 : 0;
}
