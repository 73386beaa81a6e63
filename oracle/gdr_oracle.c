/*
 * Float64 token-by-token oracle for the Gated Delta Rule.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The GPU library shares
 * no code, header, table or helper with it.
 *
 * What it computes, per batch entry b and value head h (key/query head
 * kh = h / (Nv/Nk), the repeat-interleave grouping of the Gated DeltaNet blog
 * post, "GQA repeat_interleave" step), for each valid token t in order:
 *
 *   S <- S * exp(g_t)                        decay; with a per-key gate, row i
 *                                            of S is also scaled by exp(gk_t[i])
 *   kv <- S^T k_t                            read memory (length Dv)
 *   delta <- beta_t * (v_t - kv)
 *   S <- S + k_t delta^T                     rank-1 delta write
 *   o_t <- scale * S^T q_t
 *
 * Sources: lite_boost.ops.recurrent_gated_delta_rule (MindSpore Lite API
 * page), algorithm section (decay, memory read, delta update, output, and the
 * per-key gate gk); lite_boost.ops.chunk_gated_delta_rule, formula section
 * (g omitted means alpha = 1); the blog post's torch_recurrent_gated_delta_rule
 * (decay before the memory read, outer product k delta^T); inferencelayer
 * deltanet.rs, delta_step (state S is Dk x Dv, row-major S[i*Dv + j]).
 *
 * The state is kept in double throughout and no intermediate is rounded.
 * Inputs arrive already widened (exactly) to double by the caller.
 *
 * Integer semantics (the readings of the operator pages used throughout):
 *   L_b  = clamp(actual_seq_lengths[b], 0, S)       (NULL lengths: L_b = S)
 *   decode: n_b = num_accepted_tokens[b] (NULL: L_b); the entering state is
 *           read from slot idx[b*S + n_b - 1]; after each valid token t the
 *           state is written to slot idx[b*S + t]. A sequence with L_b == 0,
 *           n_b outside [1, S] or a read slot outside [0, slots) produces zero
 *           outputs and writes nothing; a write slot outside [0, slots) skips
 *           that one write.
 *   prefill: the state enters as initial_state[b, h] (NULL: zeros) and the
 *           state after token L_b - 1 leaves as final_state[b, h].
 *   Both: outputs at t >= L_b are exactly zero.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* One token of the recurrence on one value head. S is Dk x Dv row-major.
 * alpha = exp(g_t) (1 when g is absent); gk is NULL or the Dk per-key log
 * gates of this token. kv is caller scratch of length Dv. */
static void gdr_token(double *S, int Dk, int Dv, const double *q, const double *k,
                      const double *v, double beta, double g, int has_g,
                      const double *gk, double scale, double *o, double *kv)
{
    const double alpha = has_g ? exp(g) : 1.0;
    for (int i = 0; i < Dk; ++i) {
        const double f = gk ? alpha * exp(gk[i]) : alpha;
        for (int j = 0; j < Dv; ++j) S[(size_t)i * Dv + j] *= f;
    }
    for (int j = 0; j < Dv; ++j) kv[j] = 0.0;
    for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j) kv[j] += S[(size_t)i * Dv + j] * k[i];
    for (int j = 0; j < Dv; ++j) kv[j] = beta * (v[j] - kv[j]); /* kv now holds delta */
    for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j) S[(size_t)i * Dv + j] += k[i] * kv[j];
    for (int j = 0; j < Dv; ++j) o[j] = 0.0;
    for (int i = 0; i < Dk; ++i)
        for (int j = 0; j < Dv; ++j) o[j] += S[(size_t)i * Dv + j] * q[i];
    for (int j = 0; j < Dv; ++j) o[j] *= scale;
}

static int clamp_len(int32_t x, int S)
{
    if (x < 0) return 0;
    if (x > S) return S;
    return (int)x;
}

int gdr_oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * One sequence on one head, strided views. Used by both operators and
 * exported for sampled checks of single (b, h) units.
 *   q, k: L rows of Dk at row stride ldq/ldk; v, out: rows of Dv at ldv/ldo;
 *   beta, g: stride 1 (g may be NULL); gk: NULL or L rows of Dk (stride Dk).
 *   S: Dk*Dv state, in/out. out rows t >= L are NOT touched here.
 */
int gdr_oracle_sequence(int L, int Dk, int Dv, const double *q, int64_t ldq,
                        const double *k, int64_t ldk, const double *v, int64_t ldv,
                        const double *beta, const double *g, const double *gk,
                        double scale, double *S, double *out, int64_t ldo)
{
    double *kv = (double *)malloc(sizeof(double) * (size_t)Dv);
    if (!kv) return 1;
    for (int t = 0; t < L; ++t)
        gdr_token(S, Dk, Dv, q + t * ldq, k + t * ldk, v + t * ldv, beta[t],
                  g ? g[t] : 0.0, g != NULL, gk ? gk + (size_t)t * Dk : NULL, scale,
                  out + t * ldo, kv);
    free(kv);
    return 0;
}

/*
 * Chunked-prefill operator semantics (lite_boost.ops.chunk_gated_delta_rule:
 * parameters and returns), evaluated token by token.
 * Shapes (row-major): q,k (B,Nk,S,Dk); v,out (B,Nv,S,Dv); beta (B,Nv,S);
 * g (B,Nv,S) or NULL; init (B,Nv,Dk,Dv) or NULL; lens (B) or NULL;
 * final (B,Nv,Dk,Dv). Returns 0 on success.
 */
int gdr_oracle_prefill(int B, int Nk, int Nv, int S, int Dk, int Dv, const double *q,
                       const double *k, const double *v, const double *beta,
                       const double *g, const double *init, const int32_t *lens,
                       double scale, double *out, double *final_state, int nthreads)
{
    if (B < 0 || Nk <= 0 || Nv <= 0 || S < 0 || Dk <= 0 || Dv <= 0 || Nv % Nk) return 2;
    const int rep = Nv / Nk;
    const int64_t units = (int64_t)B * Nv;
    int err = 0;
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads())
#endif
    for (int64_t u = 0; u < units; ++u) {
        const int b = (int)(u / Nv), h = (int)(u % Nv), kh = h / rep;
        const int L = lens ? clamp_len(lens[b], S) : S;
        const size_t qk_off = ((size_t)b * Nk + kh) * S * Dk;
        const size_t v_off = ((size_t)b * Nv + h) * S * Dv;
        const size_t bg_off = ((size_t)b * Nv + h) * S;
        double *St = final_state + ((size_t)b * Nv + h) * Dk * Dv;
        if (init)
            memcpy(St, init + ((size_t)b * Nv + h) * Dk * Dv, sizeof(double) * Dk * Dv);
        else
            memset(St, 0, sizeof(double) * Dk * Dv);
        if (gdr_oracle_sequence(L, Dk, Dv, q + qk_off, Dk, k + qk_off, Dk, v + v_off, Dv,
                                beta + bg_off, g ? g + bg_off : NULL, NULL, scale, St,
                                out + v_off, Dv))
            err = 1;
        for (int t = L; t < S; ++t) memset(out + v_off + (size_t)t * Dv, 0, sizeof(double) * Dv);
    }
    return err;
}

/*
 * Recurrent-decode operator semantics (lite_boost.ops.recurrent_gated_delta_rule:
 * parameters and returns), with the indexed state pool.
 * Shapes: q,k (B,Nk,S,Dk); v,out (B,Nv,S,Dv); beta,g (B,Nv,S) (g may be NULL);
 * gk (B,Nv,S,Dk) or NULL; lens (B); n_acc (B) or NULL; idx (B*S);
 * pool_in (slots,Nv,Dk,Dv) read-only; pool_out must hold a copy of pool_in on
 * entry and receives the writes. Entering states are read from pool_in, so the
 * result does not depend on the order in which units are processed.
 * Writes by different sequences to one slot are undefined by the operator;
 * here the highest b wins among them (sequential order over b within a head).
 */
int gdr_oracle_decode(int B, int Nk, int Nv, int S, int Dk, int Dv, int slots,
                      const double *q, const double *k, const double *v, const double *beta,
                      const double *g, const double *gk, const int32_t *lens,
                      const int32_t *n_acc, const int32_t *idx, double scale,
                      const double *pool_in, double *pool_out, double *out, int nthreads)
{
    if (B < 0 || Nk <= 0 || Nv <= 0 || S <= 0 || Dk <= 0 || Dv <= 0 || Nv % Nk || slots < 0)
        return 2;
    const int rep = Nv / Nk;
    const size_t hs = (size_t)Dk * Dv;
    int err = 0;
    /* Heads are independent; within a head, sequences run in order of b. */
#ifdef _OPENMP
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads > 0 ? nthreads : omp_get_max_threads())
#endif
    for (int h = 0; h < Nv; ++h) {
        double *St = (double *)malloc(sizeof(double) * hs);
        double *kv = (double *)malloc(sizeof(double) * (size_t)Dv);
        if (!St || !kv) { err = 1; free(St); free(kv); continue; }
        const int kh = h / rep;
        for (int b = 0; b < B; ++b) {
            const int L = clamp_len(lens[b], S);
            const int n = n_acc ? n_acc[b] : L;
            const size_t v_off = ((size_t)b * Nv + h) * S * Dv;
            for (int t = 0; t < S; ++t) memset(out + v_off + (size_t)t * Dv, 0, sizeof(double) * Dv);
            if (L == 0 || n < 1 || n > S) continue;
            const int32_t r = idx[(size_t)b * S + n - 1];
            if (r < 0 || r >= slots) continue;
            memcpy(St, pool_in + ((size_t)r * Nv + h) * hs, sizeof(double) * hs);
            const size_t qk_off = ((size_t)b * Nk + kh) * S * Dk;
            const size_t bg_off = ((size_t)b * Nv + h) * S;
            for (int t = 0; t < L; ++t) {
                gdr_token(St, Dk, Dv, q + qk_off + (size_t)t * Dk, k + qk_off + (size_t)t * Dk,
                          v + v_off + (size_t)t * Dv, beta[bg_off + t],
                          g ? g[bg_off + t] : 0.0, g != NULL,
                          gk ? gk + (bg_off + t) * Dk : NULL, scale,
                          out + v_off + (size_t)t * Dv, kv);
                const int32_t w = idx[(size_t)b * S + t];
                if (w >= 0 && w < slots)
                    memcpy(pool_out + ((size_t)w * Nv + h) * hs, St, sizeof(double) * hs);
            }
        }
        free(St);
        free(kv);
    }
    return err;
}
