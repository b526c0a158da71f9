/*
 * CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code with the HIP path.
 *
 * What it computes (token-by-token, fp64 throughout), following the recurrence
 * stated on the FlashQLA PR #1 page ("Fused recurrent GDN decode + SGLang DFlash
 * verify kernel", core decode-kernel commit: decay -> kS -> v_new -> rank-1 -> o,
 * post-update read, raw per-token g):
 *
 *   for each sequence n (tokens cu[n] .. cu[n+1]-1) and value head h,
 *   with key/query head hk = h / (HV / HK) (the "h // grp" GQA mapping of the
 *   same page's review commit):
 *       S[V][K] = initial state (zeros when absent)
 *       for each token t:
 *           S[v][c] *= exp(g[t,h])            (scalar gate, GDN)
 *           S[v][c] *= exp(gk[t,h,c])         (per-key-channel gate, KDA)
 *           kS[v]    = sum_c S[v][c] k[t,hk,c]
 *           nu[v]    = beta[t,h] (v[t,h,v] - kS[v])
 *           S[v][c] += nu[v] k[t,hk,c]
 *           o[t,h,v] = scale sum_c S[v][c] q[t,hk,c]     (post-update read)
 *       final state = S
 *
 * Row v of S only ever reads row v, so the work is split into independent
 * (sequence, head, row) tasks for OpenMP.  Nothing else is reordered.
 *
 * All arrays are contiguous, row-major float64:
 *   q, k [T, HK, K]; v [T, HV, V]; g [T, HV] or gk [T, HV, K]; beta [T, HV];
 *   initial_state / final_state [N, HV, V, K]; o [T, HV, V];
 *   states (optional) [T, HV, V, K]: the post-update state after every token.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int gdr_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int gdr_oracle_recurrent(int64_t T, int32_t N, const int32_t* cu_seqlens,
                         int32_t HK, int32_t HV, int32_t K, int32_t V,
                         int32_t per_k_gate, double scale,
                         const double* q, const double* k, const double* v,
                         const double* g, const double* beta,
                         const double* initial_state,
                         double* o, double* final_state, double* states,
                         int32_t num_threads) {
    if (N < 0 || HK <= 0 || HV <= 0 || K <= 0 || V <= 0 || HV % HK != 0) return 1;
    (void)T;
    const int32_t grp = HV / HK;
    const int64_t tasks = (int64_t)N * HV * V;
    int nt = num_threads > 0 ? num_threads : 1;
    (void)nt;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t task = 0; task < tasks; ++task) {
        const int32_t n = (int32_t)(task / ((int64_t)HV * V));
        const int32_t h = (int32_t)((task / V) % HV);
        const int32_t row = (int32_t)(task % V);
        const int32_t hk = h / grp;
        double* S = (double*)malloc(sizeof(double) * (size_t)K);
        const int64_t sidx = (((int64_t)n * HV + h) * V + row) * K;
        for (int32_t c = 0; c < K; ++c) S[c] = initial_state ? initial_state[sidx + c] : 0.0;
        const int64_t bos = cu_seqlens[n], eos = cu_seqlens[n + 1];
        for (int64_t t = bos; t < eos; ++t) {
            const double* kt = k + (t * HK + hk) * K;
            const double* qt = q + (t * HK + hk) * K;
            /* decay */
            if (per_k_gate) {
                const double* gt = g + (t * HV + h) * K;
                for (int32_t c = 0; c < K; ++c) S[c] *= exp(gt[c]);
            } else {
                const double a = exp(g[t * HV + h]);
                for (int32_t c = 0; c < K; ++c) S[c] *= a;
            }
            /* read: kS = S k */
            double ks = 0.0;
            for (int32_t c = 0; c < K; ++c) ks += S[c] * kt[c];
            /* delta-rule correction and rank-1 write */
            const double nu = beta[t * HV + h] * (v[(t * HV + h) * V + row] - ks);
            for (int32_t c = 0; c < K; ++c) S[c] += nu * kt[c];
            /* post-update output read */
            double acc = 0.0;
            for (int32_t c = 0; c < K; ++c) acc += S[c] * qt[c];
            o[(t * HV + h) * V + row] = scale * acc;
            if (states) memcpy(states + ((t * HV + h) * (int64_t)V + row) * K, S, sizeof(double) * (size_t)K);
        }
        if (final_state) memcpy(final_state + sidx, S, sizeof(double) * (size_t)K);
        free(S);
    }
    return 0;
}
