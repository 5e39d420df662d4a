/*
 * fp64 CPU oracle for the Mamba-2 decode recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path may link,
 * load or call this file; only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the HIP
 * path.
 *
 * Source: "ReplaySSM: Rethinking State Storage for Faster Hybrid-Model
 * Decoding" (NVIDIA Developer blog), section "Why SSM layers can become a
 * decoding bottleneck".  The page decodes one token of a Mamba-2 layer by
 * decaying the state with a data-dependent factor, adding a rank-1 update built
 * from the token's inputs and reading the output with C; the formula itself
 * was lost in extraction.  Written out per sequence b and head h (group g(h)):
 *
 *     a     = exp(dt_t[b,h] * A[h])
 *     H    <- a * H + dt_t[b,h] * x_t[b,h,:] (outer) B_t[b,g,:]   (headdim x dstate)
 *     y_t[b,h,i] = sum_j H[i,j] * C_t[b,g,j] + D[h] * x_t[b,h,i]
 *
 * Readings taken where the page is silent:
 *   - the output of token t reads the state that already includes token t;
 *   - D is one skip scalar per head;
 *   - dt arrives after the softplus and is used as given;
 *   - heads map to groups in contiguous blocks: g(h) = h / (nheads/ngroups).
 *
 * ReplaySSM (same page, section "How ReplaySSM represents the state") states
 * that its outputs match this step-by-step decoding up to floating-point
 * differences, so this plain recurrence is the oracle for decode, flush (the
 * state after the buffered tokens) and draft verification (the outputs of the
 * drafts stepped one by one).
 *
 * Everything is fp64 with plain loops; OpenMP only splits independent
 * (sequence, head) pairs across threads.
 *
 * Array layouts (all row-major, double):
 *   H  [batch][nheads][headdim][dstate]      in/out
 *   x  [steps][batch][nheads][headdim]
 *   B  [steps][batch][ngroups][dstate]
 *   C  [steps][batch][ngroups][dstate]
 *   dt [steps][batch][nheads]
 *   A, D [nheads]
 *   y  [steps][batch][nheads][headdim]       out (may be NULL)
 *   nsteps [batch]: tokens to apply to sequence b (NULL: all `steps`)
 */
#include <math.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static int head_group(int h, int nheads, int ngroups)
{
    return h / (nheads / ngroups);
}

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int orc_conventional(int batch, int nheads, int headdim, int dstate, int ngroups,
                     int steps, const int *nsteps,
                     double *H, const double *x, const double *B, const double *C,
                     const double *dt, const double *A, const double *D,
                     double *y, int nthreads)
{
    if (batch < 0 || nheads <= 0 || headdim <= 0 || dstate <= 0 || ngroups <= 0 ||
        steps < 0 || nheads % ngroups != 0)
        return -1;
    if (!H || (steps > 0 && (!x || !B || !C || !dt)) || !A || !D)
        return -1;
    if (nsteps)
        for (int b = 0; b < batch; ++b)
            if (nsteps[b] < 0 || nsteps[b] > steps)
                return -1;
    if (nthreads <= 0)
        nthreads = orc_num_threads();

    const long pairs = (long)batch * nheads;
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
    for (long p = 0; p < pairs; ++p) {
        const int b = (int)(p / nheads);
        const int h = (int)(p % nheads);
        const int g = head_group(h, nheads, ngroups);
        double *Hbh = H + (size_t)p * headdim * dstate;
        const int n = nsteps ? nsteps[b] : steps;
        for (int t = 0; t < n; ++t) {
            const size_t tb = (size_t)t * batch + b;
            const double *xt = x + (tb * nheads + h) * headdim;
            const double *Bt = B + (tb * ngroups + g) * dstate;
            const double *Ct = C + (tb * ngroups + g) * dstate;
            const double dtv = dt[tb * nheads + h];
            const double decay = exp(dtv * A[h]);

            /* state update: decay, then the rank-1 input term */
            for (int i = 0; i < headdim; ++i)
                for (int j = 0; j < dstate; ++j)
                    Hbh[i * dstate + j] = decay * Hbh[i * dstate + j] + dtv * xt[i] * Bt[j];

            /* output read from the updated state, plus the skip term */
            if (y) {
                double *yt = y + (tb * nheads + h) * headdim;
                for (int i = 0; i < headdim; ++i) {
                    double acc = 0.0;
                    for (int j = 0; j < dstate; ++j)
                        acc += Hbh[i * dstate + j] * Ct[j];
                    yt[i] = acc + D[h] * xt[i];
                }
            }
        }
    }
    return 0;
}
