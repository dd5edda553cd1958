/*
 * CPU oracle for single-query decode attention and for merging partial states.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library. The product path
 * (the HIP library) never calls it and shares no code with it.
 *
 * Everything here is the plain definition, evaluated in float64 with no
 * chunking, no tiling and no merge operator:
 *
 *   s_j   = (sum_c q[c] * K[j][c]) / sqrt(d)                 for each token j
 *   M     = max_j s_j
 *   Z     = sum_j exp(s_j - M)                               (token order)
 *   lse   = M + ln Z                                         (natural log)
 *   out[c]= (sum_j exp(s_j - M) * V[j][c]) / Z
 *
 * Sources:
 *  - softmax with a global maximum to avoid overflow: "Tree Attention Guide:
 *    Topology-Aware LLM Decoding", section "Core Innovation 2: Mathematical
 *    Formulation of Online Softmax on Trees" (the Softmax(S)_j formula);
 *  - the 1/sqrt(d) scale and the single-query product against K and V: the
 *    same page, section "Step-by-Step Implementation: Building a Tree
 *    Attention Worker in PyTorch" (its local attention method);
 *  - the final output o/l and the log-sum-exp m + ln l that a partial state
 *    carries: the same page, "Core Innovation 1" step 2 and "Core Innovation 2"
 *    (the final normalisation at the root).
 *
 * Inputs are exactly widened from their stored type: float32 directly,
 * bfloat16 by placing its 16 bits at the top of a float32.
 *
 * Parity pins for this file: brute force at 50 digits, a library attention
 * routine in float64, closed forms and the chunking/tree invariance of the
 * merge operator (all in the CPU test suite).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

static double load_elem(const void* base, int dtype, int64_t i) {
    if (dtype == ORACLE_F32) return (double)((const float*)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the number of OpenMP threads later calls use (for timing; results do not
   depend on it). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Exact decode attention for selected (batch, query head) rows.
 *
 *   q        [B, Hq, d]       contiguous, dtype f32 or bf16 bits
 *   k, v     [B, Hkv, N, d]   contiguous, same dtype
 *   seqlens  int32 [B] or NULL (NULL: every sequence has N tokens); clamped to [0, N]
 *   t_begin, t_end: the token window [t_begin, t_end) intersected with
 *            [0, seqlens[b]); t_end < 0 means "to the end of the sequence"
 *   sel      n_sel flat row ids b*Hq + h, or NULL for all B*Hq rows in order
 *   out      [n_rows, d] float64, lse [n_rows] float64
 *
 * Query head h reads KV head h / (Hq / Hkv). An empty window yields out = 0
 * and lse = -inf (the value of a sum over no tokens).
 * Returns 0, or -1 on a bad argument, -2 when memory runs out.
 */
int oracle_decode(const void* q, const void* k, const void* v, int dtype,
                  int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t d,
                  const int32_t* seqlens, int64_t t_begin, int64_t t_end,
                  const int64_t* sel, int64_t n_sel, double* out, double* lse) {
    if (!q || !k || !v || !out || !lse) return -1;
    if (dtype != ORACLE_F32 && dtype != ORACLE_BF16) return -1;
    if (B < 0 || Hq <= 0 || Hkv <= 0 || N < 0 || d <= 0 || Hq % Hkv != 0) return -1;
    const int64_t rows = sel ? n_sel : B * Hq;
    const int64_t group = Hq / Hkv;
    const double scale = 1.0 / sqrt((double)d);
    int status = 0;

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        const int64_t row = sel ? sel[r] : r;
        double* o = out + r * d;
        if (row < 0 || row >= B * Hq) {
#pragma omp atomic write
            status = -1;
            continue;
        }
        const int64_t b = row / Hq, h = row % Hq, g = h / group;
        int64_t n = seqlens ? (int64_t)seqlens[b] : N;
        if (n < 0) n = 0;
        if (n > N) n = N;
        int64_t t0 = t_begin < 0 ? 0 : t_begin;
        int64_t t1 = t_end < 0 ? n : t_end;
        if (t1 > n) t1 = n;
        if (t0 > t1) t0 = t1;
        for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
        if (t1 == t0) {
            lse[r] = -INFINITY;
            continue;
        }
        const int64_t qoff = (b * Hq + h) * d;
        const int64_t kvoff = (b * Hkv + g) * N * d;
        double* s = (double*)malloc(sizeof(double) * (size_t)(t1 - t0));
        double* qd = (double*)malloc(sizeof(double) * (size_t)d);
        if (!s || !qd) {
            free(s);
            free(qd);
#pragma omp atomic write
            status = -2;
            continue;
        }
        for (int64_t c = 0; c < d; ++c) qd[c] = load_elem(q, dtype, qoff + c);

        /* pass 1: every logit, and their maximum */
        double M = -INFINITY;
        for (int64_t j = t0; j < t1; ++j) {
            double acc = 0.0;
            for (int64_t c = 0; c < d; ++c) acc += qd[c] * load_elem(k, dtype, kvoff + j * d + c);
            s[j - t0] = acc * scale;
            if (s[j - t0] > M) M = s[j - t0];
        }
        /* pass 2: sum of exponentials and the weighted sum of value rows */
        double Z = 0.0;
        for (int64_t j = t0; j < t1; ++j) {
            const double w = exp(s[j - t0] - M);
            Z += w;
            for (int64_t c = 0; c < d; ++c) o[c] += w * load_elem(v, dtype, kvoff + j * d + c);
        }
        for (int64_t c = 0; c < d; ++c) o[c] /= Z;
        lse[r] = M + log(Z);
        free(s);
        free(qd);
    }
    return status;
}

/*
 * Merge of normalised partial states, by definition.
 *
 * Row r holds n_parts states (o_i[d], lse_i), each the softmax-weighted mean
 * of V over a token set T_i and the log-sum-exp of the logits over T_i. The
 * state of the union of disjoint sets is
 *
 *   LSE = ln sum_i exp(lse_i)            (evaluated as L + ln sum_i exp(lse_i - L),
 *                                         L = max_i lse_i)
 *   out = sum_i exp(lse_i - LSE) * o_i
 *
 * which is what the pages' pairwise merge (Core Innovation 2, the merge
 * operator, then the final normalisation at the root) reaches for any tree.
 * States with lse_i = -inf (no tokens) carry zero weight; if every state is
 * empty the result is out = 0, lse = -inf.
 *
 *   partial_o   float32 [rows, n_parts, d], partial_lse float32 [rows, n_parts]
 *   out         float64 [rows, d],          lse float64 [rows]
 */
int oracle_combine(const float* partial_o, const float* partial_lse, int64_t rows,
                   int64_t n_parts, int64_t d, double* out, double* lse) {
    if (!partial_o || !partial_lse || !out || !lse || rows < 0 || n_parts < 0 || d <= 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float* po = partial_o + r * n_parts * d;
        const float* pl = partial_lse + r * n_parts;
        double* o = out + r * d;
        for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
        double L = -INFINITY;
        for (int64_t i = 0; i < n_parts; ++i)
            if ((double)pl[i] > L) L = (double)pl[i];
        if (L == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double S = 0.0;
        for (int64_t i = 0; i < n_parts; ++i) S += exp((double)pl[i] - L);
        const double LSE = L + log(S);
        for (int64_t i = 0; i < n_parts; ++i) {
            const double w = exp((double)pl[i] - LSE);
            if (w == 0.0) continue;
            for (int64_t c = 0; c < d; ++c) o[c] += w * (double)po[i * d + c];
        }
        lse[r] = LSE;
    }
    return 0;
}
