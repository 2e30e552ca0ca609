/*
 * ssd_oracle.c -- fp64 CPU oracle for the scalar-decay state space model (SSD).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load
 * this file: only the test suite, the smoke check and the benchmark's CPU
 * baseline use it. It shares no code with the HIP library.
 *
 * What it computes is the plain definition of the layer, written out token by
 * token (the SSD path reaches exactly this result up to rounding order):
 *
 *   h_t = a_t * h_{t-1} + B_t x_t^T        (state, N x P per head)
 *   y_t = C_t^T h_t                        (output, P per head)
 *
 * with a_t = exp(log_a_t) one scalar per (token, head).
 * Sources: "Transformers are SSMs" paper card (wikillm.com/papers/2405.21060),
 * Method 1 (selective SSM as a matrix, paper sections 2-3) and Method 2
 * (scalar-identity case A_t = a_t I, paper section 5.1); the same recurrence
 * is the step rule of the state-space explainer page "State-space sequence
 * models (S4, Mamba, Mamba-2)", glossary entry "recurrence".
 *
 * Readings where the pages are silent (each one is listed in the design doc):
 *  - The state is stored per head as [P][N], element (p, n) = h[n][p].
 *  - B and C are shared by groups of H/G consecutive heads: head h reads
 *    group h / (H/G).
 *  - A segment [begin, end) of one row starts from a zero state (or from
 *    the given initial state); packed variable-length sequences are segments.
 *
 * Layouts (all row-major, fp64):
 *   X  [rows][T][H][P]    la [rows][T][H]    B, C [rows][T][G][N]
 *   Y  [rows][T][H][P]    states [*][H][P][N]
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Mutants exist only so the test suite can show that its pins catch plausible
 * mistakes; 0 is the oracle itself. */
enum {
  MUT_NONE = 0,
  MUT_DECAY_AFTER_INPUT = 1, /* h_t = a_t (h_{t-1} + B_t x_t^T)             */
  MUT_OUTPUT_BEFORE_UPDATE = 2, /* y_t = C_t^T h_{t-1}                       */
  MUT_SWAP_B_C = 3,          /* roles of B and C exchanged                    */
  MUT_DECAY_SIGN = 4,        /* a_t = exp(-log_a_t)                           */
  MUT_NO_DECAY = 5,          /* a_t = 1                                       */
  MUT_GROUP_MOD = 6,         /* head h reads group h % G                      */
  MUT_DECAY_NEXT_TOKEN = 7,  /* uses log_a of token t+1 (0 past the end)      */
  MUT_STATE_TRANSPOSE = 8,   /* reads out h[p][n] instead of h[n][p] (P == N) */
};

/* One (segment, head) pair: run the recurrence over [t0, t1) of row `row`. */
static void run_pair(int T, int H, int G, int P, int N,
                     const double* X, const double* la, const double* B,
                     const double* C, int row, int t0, int t1, int h,
                     const double* init /* [P][N] or NULL */,
                     double* Y, double* final_state /* [P][N] or NULL */,
                     const int* snap_slot, double* snaps, int mutant,
                     double* hs /* scratch [N][P] */, double* y /* [P] */) {
  const int heads_per_group = H / G;
  int g = h / heads_per_group;
  if (mutant == MUT_GROUP_MOD) g = h % G;

  /* hs[n][p] holds h[n][p]; the input state is given as [P][N]. */
  if (init) {
    for (int p = 0; p < P; ++p)
      for (int n = 0; n < N; ++n) hs[(size_t)n * P + p] = init[(size_t)p * N + n];
  } else {
    memset(hs, 0, sizeof(double) * (size_t)N * P);
  }

  for (int t = t0; t < t1; ++t) {
    const size_t tok = (size_t)row * T + t;
    double lat = la[tok * H + h];
    if (mutant == MUT_DECAY_NEXT_TOKEN) lat = (t + 1 < t1) ? la[(tok + 1) * H + h] : 0.0;
    double alpha = exp(lat);
    if (mutant == MUT_DECAY_SIGN) alpha = exp(-lat);
    if (mutant == MUT_NO_DECAY) alpha = 1.0;

    const double* x = X + (tok * H + h) * P;
    const double* b = B + (tok * G + g) * N;
    const double* c = C + (tok * G + g) * N;
    if (mutant == MUT_SWAP_B_C) {
      const double* tmp = b;
      b = c;
      c = tmp;
    }

    if (mutant == MUT_OUTPUT_BEFORE_UPDATE) {
      for (int p = 0; p < P; ++p) y[p] = 0.0;
      for (int n = 0; n < N; ++n) {
        const double* hn = hs + (size_t)n * P;
        for (int p = 0; p < P; ++p) y[p] += c[n] * hn[p];
      }
    }

    /* h_t = a_t h_{t-1} + B_t x_t^T */
    for (int n = 0; n < N; ++n) {
      double* hn = hs + (size_t)n * P;
      const double bn = b[n];
      if (mutant == MUT_DECAY_AFTER_INPUT) {
        for (int p = 0; p < P; ++p) hn[p] = alpha * (hn[p] + bn * x[p]);
      } else {
        for (int p = 0; p < P; ++p) hn[p] = alpha * hn[p] + bn * x[p];
      }
    }

    /* y_t = C_t^T h_t, summed over n in increasing order */
    if (mutant != MUT_OUTPUT_BEFORE_UPDATE) {
      for (int p = 0; p < P; ++p) y[p] = 0.0;
      if (mutant == MUT_STATE_TRANSPOSE) {
        for (int p = 0; p < P; ++p)
          for (int n = 0; n < N; ++n) y[p] += c[n] * hs[(size_t)p * P + n];
      } else {
        for (int n = 0; n < N; ++n) {
          const double* hn = hs + (size_t)n * P;
          const double cn = c[n];
          for (int p = 0; p < P; ++p) y[p] += cn * hn[p];
        }
      }
    }
    if (Y) memcpy(Y + (tok * H + h) * P, y, sizeof(double) * (size_t)P);

    if (snap_slot && snap_slot[tok] >= 0) {
      double* dst = snaps + ((size_t)snap_slot[tok] * H + h) * (size_t)P * N;
      for (int p = 0; p < P; ++p)
        for (int n = 0; n < N; ++n) dst[(size_t)p * N + n] = hs[(size_t)n * P + p];
    }
  }

  if (final_state) {
    for (int p = 0; p < P; ++p)
      for (int n = 0; n < N; ++n) final_state[(size_t)p * N + n] = hs[(size_t)n * P + p];
  }
}

/*
 * Run the recurrence over `nseg` segments; segment s is seg[3s..3s+2] =
 * (row, begin, end). Each segment starts from init[s] (or zero when init is
 * NULL) and leaves its state in final_state[s] (when not NULL). Y entries of
 * tokens outside every segment are not written. When snap_slot is not NULL,
 * snap_slot[row*T + t] >= 0 stores the state after token t into
 * snaps[snap_slot[...]]. nthreads <= 0 uses the OpenMP default.
 * Returns 0, or -1 on an argument error.
 */
int ssd_oracle_scan(int rows, int T, int H, int G, int P, int N,
                    const double* X, const double* la, const double* B,
                    const double* C, int nseg, const int* seg,
                    const double* init, double* Y, double* final_state,
                    const int* snap_slot, double* snaps, int nthreads,
                    int mutant) {
  if (rows <= 0 || T < 0 || H <= 0 || G <= 0 || P <= 0 || N <= 0 || H % G) return -1;
  if (nseg < 0 || (nseg > 0 && !seg)) return -1;
  for (int s = 0; s < nseg; ++s) {
    int r = seg[3 * s], b = seg[3 * s + 1], e = seg[3 * s + 2];
    if (r < 0 || r >= rows || b < 0 || e < b || e > T) return -1;
  }
  if (snap_slot && !snaps) return -1;
  const long npairs = (long)nseg * H;
  int status = 0;
#ifdef _OPENMP
  if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
  for (long w = 0; w < npairs; ++w) {
    const int s = (int)(w / H), h = (int)(w % H);
    const size_t pn = (size_t)P * N;
    double* hs = (double*)malloc(sizeof(double) * (pn + (size_t)P));
    if (!hs) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      status = -1;
      continue;
    }
    run_pair(T, H, G, P, N, X, la, B, C, seg[3 * s], seg[3 * s + 1], seg[3 * s + 2], h,
             init ? init + ((size_t)s * H + h) * pn : NULL, Y,
             final_state ? final_state + ((size_t)s * H + h) * pn : NULL, snap_slot, snaps,
             mutant, hs, hs + pn);
    free(hs);
  }
  return status;
}

int ssd_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
