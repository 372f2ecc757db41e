/*
 * h3conv_oracle.c -- plain, slow, fp64 CPU oracle for the causal SSM long
 * convolution of H3 / FlashConv.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the correctness reference that the
 * GPU library is checked against.  Only the test suite, the package smoke
 * check and the CPU-baseline leg of the benchmark may load it.  It shares no
 * code, header, table or helper with the GPU library and includes nothing
 * from it.
 *
 * Every function computes the plain *definition* of what the method reaches,
 * not the method's fast algorithm:
 *
 *   - "Hungry Hungry Hippos: Towards Language Modeling with State Space
 *     Models" (paperlayer.ai summary), section 2 Background, "Convolutional
 *     view": with a zero initial state the SSM output is exactly a linear
 *     convolution of the input with a filter plus a residual term D*u.
 *   - same page, Appendix C.1 "Backward Pass": signals are zero-padded to
 *     length 2L and the first N entries are kept, i.e. the convolution is the
 *     causal *linear* one, never circular.
 *   - deep-paper.org blog on the paper, section "The Convolution Connection":
 *     the filter is f = [CB, CAB, CA^2B, ...].
 *   - same blog, section "Background: What Are State Space Models?": the state
 *     x_i is updated from x_{i-1} with the current input u_i and the output is
 *     read from the state (y_i = C x_i + D u_i, section 2 of the summary page).
 *   - summary page, section 4 FlashConv, "Correctness": state passing returns
 *     exactly the output of the full-length SSM, so the full-length recurrence
 *     below is the oracle for chunked state passing.
 *   - blog, section "The Solution, Part 1": H3 computes
 *     Q (.) SSM_diag( SSM_shift(K) (.) V ), the shift SSM having a shift
 *     matrix as its A (so it is a short causal FIR filter).
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes of the repository):
 *   - index convention x_t = Abar x_{t-1} + Bbar u_t, y_t = 2 Re(C.x_t) + D u_t,
 *     so f_0 = 2 Re(sum_j C_j Bbar_j): the current input passes through f_0;
 *   - discretisation Abar_j = exp(dt A_j), Bbar_j = dt B_j; the S complex
 *     modes carry no explicit conjugate partners, the real part is doubled;
 *   - the shift-SSM tap w[d,0] multiplies k_t, w[d,i] multiplies k_{t-i},
 *     values before t = 0 are zero, and the shift SSM has no residual term.
 *
 * All arithmetic is IEEE fp64 in program order (built without fast-math).
 * Loops over independent rows are spread over OpenMP threads; each output is
 * still computed by one thread in the order written here.
 */
#include <complex.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* Number of OpenMP threads this library will use (1 without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the OpenMP thread count (ignored without OpenMP). */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Causal linear convolution with residual, one filter per channel:
 *   y[b,h,t] = sum_{k=0..t} f[h,t-k] * u[b,h,k]  +  D[h] * u[b,h,t]
 * u, y: [B,H,N] row-major; f: [H,N]; D: [H].  O(N^2) per row.
 * Source: summary page section 2 "Convolutional view" (linear convolution
 * plus residual) and Appendix C.1 (zero-pad to 2L, keep the first N).
 */
void oracle_causal_conv(const double *u, const double *f, const double *D,
                        double *y, int64_t B, int64_t H, int64_t N)
{
    int64_t rows = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t h = r % H;
        const double *ur = u + r * N;
        const double *fh = f + h * N;
        double *yr = y + r * N;
        for (int64_t t = 0; t < N; ++t) {
            double acc = 0.0;
            for (int64_t k = 0; k <= t; ++k)
                acc += fh[t - k] * ur[k];
            yr[t] = acc + D[h] * ur[t];
        }
    }
}

/*
 * Multi-head H3 mixing, head dimension dh, channel-last [B,N,Dm], Dm = heads*dh.
 * For head h (model channels h*dh .. h*dh+dh-1), step t:
 *   s[t,i]   = sum_{l<L, l<=t} w[h*dh+i, l] k[t-l, h*dh+i]    shift SSM on each key channel
 *   m[t,i,j] = s[t,i] * v[t, h*dh+j]                          outer product of key and value
 *   z[t,i,j] = sum_{tau<=t} f[c, t-tau] m[tau,i,j] + D[c] m[t,i,j],  c = (h*dh+i)*dh + j
 *   out[t, h*dh+j] = sum_i q[t, h*dh+i] z[t,i,j]
 * q, k, v, out: [B,N,Dm]; w: [Dm,L]; f: [Dm*dh,N]; D: [Dm*dh].
 * Source: summary page section 3 (cost O(d^2 N + d N log N) when the head
 * dimension is O(1)) and Appendix C "H3 Model to Solve Lambda" (keys in
 * separate heads); blog "The Solution, Part 1" (Q gate on the diagonal SSM
 * of shift(K) gate V).  Readings: the gates become the outer product
 * shift(K)^T V per head and the contraction with Q, one long filter and one
 * D per state entry (i, j); dh = 1 is oracle_h3_mix.
 * `scratch` must hold (2*dh*dh + dh) * N doubles per OpenMP thread.
 */
void oracle_h3_mix_mh(const double *q, const double *k, const double *v,
                      const double *w, const double *f, const double *D,
                      double *out, int64_t B, int64_t N, int64_t Dm,
                      int64_t dh, int64_t L, double *scratch)
{
    int64_t heads = Dm / dh;
    int64_t items = B * heads;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t it = 0; it < items; ++it) {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        double *m = scratch + (int64_t)tid * (2 * dh * dh + dh) * N; /* [dh*dh][N] */
        double *z = m + dh * dh * N;                                  /* [dh*dh][N] */
        double *sk = z + dh * dh * N;                                 /* [dh][N] */
        int64_t b = it / heads, h = it % heads;
        const int64_t base = b * N * Dm; /* element (t, d) at base + t*Dm + d */
        for (int64_t i = 0; i < dh; ++i) {
            int64_t d = h * dh + i;
            for (int64_t t = 0; t < N; ++t) {
                double s = 0.0;
                for (int64_t l = 0; l < L && l <= t; ++l)
                    s += w[d * L + l] * k[base + (t - l) * Dm + d];
                sk[i * N + t] = s;
            }
        }
        for (int64_t i = 0; i < dh; ++i)
            for (int64_t j = 0; j < dh; ++j)
                for (int64_t t = 0; t < N; ++t)
                    m[(i * dh + j) * N + t] = sk[i * N + t] * v[base + t * Dm + h * dh + j];
        for (int64_t i = 0; i < dh; ++i)
            for (int64_t j = 0; j < dh; ++j) {
                int64_t c = (h * dh + i) * dh + j;
                const double *mr = m + (i * dh + j) * N;
                double *zr = z + (i * dh + j) * N;
                for (int64_t t = 0; t < N; ++t) {
                    double acc = 0.0;
                    for (int64_t tau = 0; tau <= t; ++tau)
                        acc += f[c * N + t - tau] * mr[tau];
                    zr[t] = acc + D[c] * mr[t];
                }
            }
        for (int64_t j = 0; j < dh; ++j)
            for (int64_t t = 0; t < N; ++t) {
                double acc = 0.0;
                for (int64_t i = 0; i < dh; ++i)
                    acc += q[base + t * Dm + h * dh + i] * z[(i * dh + j) * N + t];
                out[base + t * Dm + h * dh + j] = acc;
            }
    }
}

/*
 * Bidirectional long convolution with residual: a causal copy with filter f
 * and an anti-causal copy with filter g over the same input, summed,
 *   y[b,h,t] = sum_{k=0..t} f[h,t-k] u[b,h,k] + sum_{k=t..N-1} g[h,k-t] u[b,h,k]
 *              + D[h] u[b,h,t]
 * u, y: [B,H,N]; f, g: [H,N]; D: [H].  O(N^2) per row.
 * Source: summary page, E.4 "LRA evaluation" (the layer used as bidirectional
 * copies) with the convolution of section 2; the anti-causal copy is the
 * causal convolution of the time-reversed input, reversed back.  Reading:
 * the two copies' outputs are summed and share one residual D u.
 */
void oracle_bidir_conv(const double *u, const double *f, const double *g,
                       const double *D, double *y, int64_t B, int64_t H,
                       int64_t N)
{
    int64_t rows = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t h = r % H;
        const double *ur = u + r * N;
        const double *fh = f + h * N;
        const double *gh = g + h * N;
        double *yr = y + r * N;
        for (int64_t t = 0; t < N; ++t) {
            double acc = 0.0;
            for (int64_t k = 0; k <= t; ++k)
                acc += fh[t - k] * ur[k];
            for (int64_t k = t; k < N; ++k)
                acc += gh[k - t] * ur[k];
            yr[t] = acc + D[h] * ur[t];
        }
    }
}

/*
 * Gradients (reverse mode) of the causal convolution with residual above,
 * for an upstream gradient dy of y:
 *   du[b,h,k] = sum_{t=k..N-1} f[h,t-k] * dy[b,h,t]  +  D[h] * dy[b,h,k]
 *   df[h,s]   = sum_b sum_{t=s..N-1} dy[b,h,t] * u[b,h,t-s]
 *   dD[h]     = sum_b sum_t dy[b,h,t] * u[b,h,t]
 * u, dy, du: [B,H,N]; f, df: [H,N]; D, dD: [H].  O(N^2) per row.
 * Source: summary page Appendix C.1 "Backward Pass": the gradients of u, f
 * and D are the transposed (correlation) convolutions of the forward one,
 * with D*dy entering du, derived from the Toeplitz form of the causal
 * convolution (signals padded to 2L, the first N entries kept).  Each sum
 * runs in the order written (b outer, t inner).
 */
void oracle_causal_conv_bwd(const double *u, const double *f, const double *D,
                            const double *dy, double *du, double *df,
                            double *dD, int64_t B, int64_t H, int64_t N)
{
    int64_t rows = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t h = r % H;
        const double *dyr = dy + r * N;
        const double *fh = f + h * N;
        double *dur = du + r * N;
        for (int64_t k = 0; k < N; ++k) {
            double acc = 0.0;
            for (int64_t t = k; t < N; ++t)
                acc += fh[t - k] * dyr[t];
            dur[k] = acc + D[h] * dyr[k];
        }
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t h = 0; h < H; ++h) {
        for (int64_t s = 0; s < N; ++s) {
            double acc = 0.0;
            for (int64_t b = 0; b < B; ++b) {
                const double *ur = u + (b * H + h) * N;
                const double *dyr = dy + (b * H + h) * N;
                for (int64_t t = s; t < N; ++t)
                    acc += dyr[t] * ur[t - s];
            }
            df[h * N + s] = acc;
        }
        double d = 0.0;
        for (int64_t b = 0; b < B; ++b) {
            const double *ur = u + (b * H + h) * N;
            const double *dyr = dy + (b * H + h) * N;
            for (int64_t t = 0; t < N; ++t)
                d += dyr[t] * ur[t];
        }
        dD[h] = d;
    }
}

/*
 * Filter of a diagonal complex SSM (S modes per channel):
 *   f[h,k] = 2 Re( sum_j C[h,j] * exp(dt[h] * A[h,j] * k) * dt[h] * B[h,j] )
 * Complex arrays are interleaved (re, im) pairs: A, Bm, C are [H,S,2].
 * Each power of Abar is evaluated directly as exp(dt*A*k), never by repeated
 * multiplication, so the oracle does not share the recurrence's rounding.
 * Source: blog section "The Convolution Connection" (f = [CB, CAB, ...]) with
 * the discretisation reading stated in the file header.
 */
void oracle_ssm_filter(const double *A, const double *Bm, const double *C,
                       const double *dt, double *f, int64_t H, int64_t S,
                       int64_t N)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t h = 0; h < H; ++h) {
        for (int64_t k = 0; k < N; ++k) {
            double complex acc = 0.0;
            for (int64_t j = 0; j < S; ++j) {
                const int64_t o = 2 * (h * S + j);
                double complex a = A[o] + I * A[o + 1];
                double complex b = Bm[o] + I * Bm[o + 1];
                double complex c = C[o] + I * C[o + 1];
                acc += c * cexp(dt[h] * a * (double)k) * (dt[h] * b);
            }
            f[h * N + k] = 2.0 * creal(acc);
        }
    }
}

/*
 * Step-by-step recurrence of the diagonal complex SSM, one state per row:
 *   Abar_j = exp(dt A_j),  Bbar_j = dt B_j
 *   x_j <- Abar_j x_j + Bbar_j u_t        (t = 0 .. N-1)
 *   y_t  = 2 Re( sum_j C_j x_j ) + D u_t
 * u, y: [B,H,N]; A, Bm, C: [H,S,2]; dt, D: [H];
 * x_in, x_out: [B,H,S,2] (x_in NULL means a zero initial state, x_out NULL
 * means the final state is not returned).  O(N*S) per row.
 * Source: blog section "Background: What Are State Space Models?" and summary
 * page section 2 (y_i = C x_i + D u_i); section 4 "Correctness" makes this
 * the reference for chunked state passing.
 */
void oracle_ssm_recurrence(const double *u, const double *A, const double *Bm,
                           const double *C, const double *dt, const double *D,
                           const double *x_in, double *y, double *x_out,
                           int64_t B, int64_t H, int64_t N, int64_t S)
{
    int64_t rows = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t h = r % H;
        const double *ur = u + r * N;
        double *yr = y + r * N;
        double complex x[256];
        double complex abar[256], bbar[256], c[256];
        for (int64_t j = 0; j < S; ++j) {
            const int64_t o = 2 * (h * S + j);
            abar[j] = cexp(dt[h] * (A[o] + I * A[o + 1]));
            bbar[j] = dt[h] * (Bm[o] + I * Bm[o + 1]);
            c[j] = C[o] + I * C[o + 1];
            if (x_in)
                x[j] = x_in[2 * (r * S + j)] + I * x_in[2 * (r * S + j) + 1];
            else
                x[j] = 0.0;
        }
        for (int64_t t = 0; t < N; ++t) {
            double complex acc = 0.0;
            for (int64_t j = 0; j < S; ++j) {
                x[j] = abar[j] * x[j] + bbar[j] * ur[t];
                acc += c[j] * x[j];
            }
            yr[t] = 2.0 * creal(acc) + D[h] * ur[t];
        }
        if (x_out) {
            for (int64_t j = 0; j < S; ++j) {
                x_out[2 * (r * S + j)] = creal(x[j]);
                x_out[2 * (r * S + j) + 1] = cimag(x[j]);
            }
        }
    }
}

/*
 * H3 mixing with head dimension 1, channel-last layout [B,N,Dm]:
 *   s_t = sum_{i<L, i<=t} w[d,i] * k_{t-i}          (shift SSM, short FIR)
 *   m_t = s_t * v_t                                   (first gate)
 *   z_t = sum_{tau<=t} f[d,t-tau] * m_tau + D[d] m_t  (diagonal SSM, long conv)
 *   out_t = q_t * z_t                                 (second gate)
 * q, k, v, out: [B,N,Dm]; w: [Dm,L]; f: [Dm,N]; D: [Dm].
 * Source: blog section "The Solution, Part 1" (shift SSM on K, gate with V,
 * diagonal SSM, gate with Q) and summary page section 3 (head dimension O(1)).
 * `scratch` must hold 2*N doubles per OpenMP thread (m and z of one column).
 */
void oracle_h3_mix(const double *q, const double *k, const double *v,
                   const double *w, const double *f, const double *D,
                   double *out, int64_t B, int64_t N, int64_t Dm, int64_t L,
                   double *scratch)
{
    int64_t cols = B * Dm;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t cidx = 0; cidx < cols; ++cidx) {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        double *m = scratch + (int64_t)tid * 2 * N;
        double *z = m + N;
        int64_t b = cidx / Dm, d = cidx % Dm;
        const int64_t base = b * N * Dm + d; /* element t at base + t*Dm */
        for (int64_t t = 0; t < N; ++t) {
            double s = 0.0;
            for (int64_t i = 0; i < L && i <= t; ++i)
                s += w[d * L + i] * k[base + (t - i) * Dm];
            m[t] = s * v[base + t * Dm];
        }
        for (int64_t t = 0; t < N; ++t) {
            double acc = 0.0;
            for (int64_t tau = 0; tau <= t; ++tau)
                acc += f[d * N + t - tau] * m[tau];
            z[t] = acc + D[d] * m[t];
        }
        for (int64_t t = 0; t < N; ++t)
            out[base + t * Dm] = q[base + t * Dm] * z[t];
    }
}
