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
