/*
 * h3conv.h -- C ABI of the MI355X (gfx950) causal SSM long-convolution library.
 *
 * The operations follow "Hungry Hungry Hippos: Towards Language Modeling with
 * State Space Models" as summarised on the paperlayer.ai page (sections 2, 3,
 * 4 and Appendix C) and the deep-paper.org blog on the same paper (sections
 * "The Convolution Connection", "The Solution, Part 1" and "Part 2:
 * FLASHCONV").
 *
 * Conventions shared by every entry point
 *   - All tensor arguments are DEVICE pointers to contiguous row-major memory
 *     on the current HIP device, at least 16-byte aligned.  Complex arrays are
 *     interleaved (re, im) fp32 pairs.
 *   - The caller owns every buffer.  No entry point allocates or frees device
 *     memory, and none keeps per-call state; workspace is passed in.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns without synchronising.
 *   - Arguments are validated on the host before any HIP call.  Outputs must
 *     not overlap any input.  Errors are reported only through the returned
 *     status; nothing aborts or throws.
 *   - `io` selects the element type of the activations (u, y, q, k, v, out):
 *     H3CONV_F32, H3CONV_F16 or H3CONV_BF16.  Filters, SSM parameters, states
 *     and the residual D are always fp32.  Outputs are rounded to nearest-even.
 *   - A call with a zero-sized batch, channel or length dimension is a no-op
 *     returning H3CONV_OK (pointers may then be NULL).
 *   - Calls may be made from several host threads; the library holds no
 *     mutable global state after the first successful call on a device.
 */
#ifndef H3CONV_H
#define H3CONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    H3CONV_OK = 0,
    H3CONV_ERR_INVALID_ARG = 1, /* null/misaligned pointer, negative size, aliasing */
    H3CONV_ERR_UNSUPPORTED = 2, /* well-formed but outside the supported sizes       */
    H3CONV_ERR_NO_DEVICE = 3,   /* no usable gfx950 HIP device                        */
    H3CONV_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed         */
    H3CONV_ERR_WORKSPACE = 5    /* workspace missing or smaller than required         */
} h3conv_status;

typedef enum { H3CONV_F32 = 0, H3CONV_F16 = 1, H3CONV_BF16 = 2 } h3conv_dtype;

typedef enum {
    H3CONV_OP_FFT_CONV = 0,
    H3CONV_OP_STATE_PASS = 1,
    H3CONV_OP_H3_MIX = 2,
    H3CONV_OP_H3_MIX_MH = 3
} h3conv_op;

/* Largest sequence length handled by one fused FFT block (2N <= 16384 points),
 * for every activation type and operation. */
#define H3CONV_MAX_FUSED_N 8192
/* Largest for h3conv_fft_conv and h3conv_fft_conv_bidir with 16-bit
 * activations (2N = 32768 points: one 128 KiB signal in a compute unit's
 * LDS). */
#define H3CONV_MAX_FUSED_N_16BIT 16384
/* Largest number of diagonal-SSM modes per channel. */
#define H3CONV_MAX_STATE 64

/*
 * Causal long convolution with residual, one filter per channel:
 *     y[b,h,t] = sum_{k=0..t} f[h,t-k] * u[b,h,k] + D[h] * u[b,h,t]
 * computed through an FFT of the zero-padded sequence (2*N points, first N
 * outputs kept), fused in one kernel per channel.
 * Defined on the paperlayer.ai summary, section 2 "Convolutional view"
 * (linear convolution plus residual, computed by FFT, pointwise product and
 * inverse FFT), section 4 (fused FFT convolution up to 8K) and Appendix C.1
 * (zero-padding to 2L, first N entries kept).
 *
 *   u  [B,H,N]  io dtype     input
 *   f  [H,N]    fp32         filter
 *   D  [H]      fp32         residual weight
 *   y  [B,H,N]  io dtype     output (must not overlap u, f or D)
 * Supported: 1 <= N <= H3CONV_MAX_FUSED_N for fp32 activations and
 * N <= H3CONV_MAX_FUSED_N_16BIT for fp16 / bf16 (any N; longer inputs use
 * h3conv_state_pass), B*H < 2^31, and for 16-bit activations with N > 128
 * (the matrix-core engine, whose row offsets within one launch are 32-bit)
 * (2*SIG + 4) * 2*H*N < 2^32 bytes, SIG being the complex signals per round
 * of that transform size: 8 for 2N = 512, 4 for 1024 and 2048, 2 for 4096,
 * 1 for 8192, 16384 and 32768 (so at N = 8192, H <= 43690).  Larger batches B are
 * split by the library.  Otherwise H3CONV_ERR_UNSUPPORTED, before any HIP call.
 * Rows are transformed two at a time as one complex signal; each row has a
 * scale of its own, so its error is set by its own magnitude, and a row of
 * zeros gives exact zeros (16-bit activations).  With fp32 activations a
 * row's rounding error also holds a part of about 2^-22 times its partner
 * row's magnitude.
 */
h3conv_status h3conv_fft_conv(const void *u, const float *f, const float *D, void *y,
                              int64_t B, int64_t H, int64_t N, int io, void *stream);

/*
 * Bidirectional copies of the convolution (the paperlayer.ai summary, E.4
 * "LRA evaluation": the layer used as bidirectional copies), one residual:
 *     y[b,h,t] = sum_{k<=t} f[h,t-k] u[b,h,k] + sum_{k>=t} g[h,k-t] u[b,h,k]
 *                + D[h] u[b,h,t]
 * i.e. a causal copy with filter f and an anti-causal copy with filter g
 * (the causal convolution of the time-reversed input, reversed back),
 * computed as one fused transform per row pair with the two-sided filter.
 *
 *   u, y [B,H,N] io dtype;  f, g [H,N] fp32;  D [H] fp32
 * Supported sizes and errors: as h3conv_fft_conv (N up to
 * H3CONV_MAX_FUSED_N_16BIT for 16-bit activations).
 */
h3conv_status h3conv_fft_conv_bidir(const void *u, const float *f, const float *g, const float *D,
                                    void *y, int64_t B, int64_t H, int64_t N, int io, void *stream);

/*
 * Backward pass of h3conv_fft_conv: for an upstream gradient dy of y,
 *     du[b,h,k] = sum_{t=k..N-1} f[h,t-k] dy[b,h,t] + D[h] dy[b,h,k]
 *     df[h,s]   = sum_b sum_{t=s..N-1} dy[b,h,t] u[b,h,t-s]
 *     dD[h]     = sum_b sum_t dy[b,h,t] u[b,h,t]
 * i.e. the correlations of dy with the filter and with the input, computed
 * through the same zero-padded 2N-point transforms (the paperlayer.ai
 * summary, Appendix C.1 "Backward Pass": gradients of u, f and D through
 * (inverse) FFTs of the conjugated spectra, D dy entering du).
 *
 *   u, dy   [B,H,N]  io dtype   forward input and upstream gradient
 *   f [H,N], D [H]   fp32       forward filter and residual weight
 *   du      [B,H,N]  io dtype   output
 *   df [H,N], dD [H] fp32       outputs, summed over the batch (written, not
 *                               accumulated into)
 * Outputs must not overlap any input or each other.  B == 0 writes zeros
 * to df and dD.  Supported sizes: those of h3conv_fft_conv with
 * N <= H3CONV_MAX_FUSED_N.
 * Precision with fp16 / bf16 activations: the transforms run in fp16 on the
 * matrix cores; du scales every row on its own (as h3conv_fft_conv); df
 * sums fp16 spectrum products in fp32, the two rows of a row pair sharing
 * one exact power-of-two weight, so a row whose u-dy product is far below
 * its partner's is carried to about 2^-11 of the partner's (not of its own).
 */
h3conv_status h3conv_fft_conv_bwd(const void *u, const float *f, const float *D, const void *dy,
                                  void *du, float *df, float *dD, int64_t B, int64_t H, int64_t N,
                                  int io, void *stream);

/*
 * Filter of a diagonal complex SSM with S modes per channel:
 *     f[h,k] = 2 Re( sum_j C[h,j] * exp(dt[h] * A[h,j] * k) * dt[h] * Bm[h,j] ),  k < N
 * i.e. f = [C Bbar, C Abar Bbar, C Abar^2 Bbar, ...] with Abar = exp(dt A),
 * Bbar = dt B (the blog's section "The Convolution Connection"; the
 * discretisation Abar = exp(dt A), Bbar = dt B and the doubled real part are
 * this library's reading where the pages give no formula).
 *
 *   A, Bm, C [H,S] complex (interleaved fp32)   dt [H] fp32   f [H,N] fp32 output
 * Supported: 1 <= S <= H3CONV_MAX_STATE, N >= 1.
 */
h3conv_status h3conv_ssm_filter(const float *A, const float *Bm, const float *C, const float *dt,
                                float *f, int64_t H, int64_t S, int64_t N, void *stream);

/*
 * Chunked state passing for sequences longer than one fused block (the
 * paperlayer.ai summary, section 4 "Long-sequence computation" and
 * "Correctness"; Appendix C "State Passing" for the update matrix M_ux).
 * The output equals the full-length diagonal SSM
 *     x_t = Abar x_{t-1} + Bbar u_t,   y_t = 2 Re(C . x_t) + D u_t
 * with Abar = exp(dt A), Bbar = dt B and x_{-1} = x_in (zero if NULL).
 * Between chunks of T samples the state is carried as
 *     x_c = Abar^T x_{c-1} + sum_k Abar^{T-1-k} Bbar u_{c,k}
 * and chunk c adds 2 Re(sum_j C_j Abar_j^{t+1} x_{c-1,j}) at offset t to its
 * own convolution with the length-T filter.  fp32 activations convolve each
 * chunk by FFT.  16-bit activations pass the state at every block of 64
 * samples, a refinement of any chunk grid T (so the result is the same for
 * every valid T): each block's own convolution (a 64 x 64 Toeplitz product),
 * its contribution and its correction are matrix-core products, and y is
 * written once.
 *
 *   u      [B,H,N]  io dtype      input
 *   A,Bm,C [H,S]    complex fp32  SSM parameters
 *   dt, D  [H]      fp32
 *   x_in   [B,H,S]  complex fp32  initial state, or NULL for zero
 *   x_out  [B,H,S]  complex fp32  final state after sample N-1, or NULL
 *   y      [B,H,N]  io dtype      output (must not overlap any input)
 *   ws, ws_bytes    workspace of at least h3conv_workspace_size(H3CONV_OP_STATE_PASS, ...)
 * Supported: T a power of two, 64 <= T <= H3CONV_MAX_FUSED_N, N % T == 0,
 * 1 <= S <= H3CONV_MAX_STATE, B <= 65535, H <= 65535.  N == 0 writes x_in
 * (or zeros) to x_out and nothing else.
 * 16-bit activations require stable or neutral modes, |exp(dt A_j)| <= 1
 * (Re(dt A_j) <= 0), as every SSM of the pages is: the powers of Abar that
 * the projections use are then fp16 operands in [-1, 1].  Modes with
 * |Abar| > 1 overflow them (the results are then undefined); fp32
 * activations have no such limit.
 */
h3conv_status h3conv_state_pass(const void *u, const float *A, const float *Bm, const float *C,
                                const float *dt, const float *D, const float *x_in, float *x_out,
                                void *y, int64_t B, int64_t H, int64_t N, int64_t S, int64_t T,
                                int io, void *ws, size_t ws_bytes, void *stream);

/*
 * h3conv_state_pass without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same operation, arguments (less ws and
 * ws_bytes), kernels and results as h3conv_state_pass; the workspace is the
 * library's own static device array of H3CONV_NOALLOC_WORKSPACE_BYTES per
 * device (part of its device code, held until the process ends).  No call
 * allocates or frees anything.
 * Sizes whose workspace, h3conv_workspace_size(H3CONV_OP_STATE_PASS, ...) for
 * this activation type, exceeds the array return H3CONV_ERR_WORKSPACE before
 * any HIP call (16-bit activations: about 33 KiB of channel tables per
 * channel whatever B, N and T, so up to about 3900 channels; fp32
 * activations: the chunk filter, power tables and per-chunk contributions,
 * which grow with T and with B * N / T).
 * All calls on one device share that device's array: calls that overlap in
 * time on one device (several streams, or several host threads) race and
 * must be serialised by the caller, e.g. by issuing them on one stream.
 * Nothing in the array needs to start zeroed; each call writes what it reads.
 */
#define H3CONV_NOALLOC_WORKSPACE_BYTES (128u * 1024u * 1024u)
h3conv_status h3conv_state_pass_noalloc(const void *u, const float *A, const float *Bm,
                                        const float *C, const float *dt, const float *D,
                                        const float *x_in, float *x_out, void *y, int64_t B,
                                        int64_t H, int64_t N, int64_t S, int64_t T, int io,
                                        void *stream);

/*
 * Recurrent generation: K steps of the diagonal SSM per row from its current
 * state, the state updated in place (the recurrent view of the blog's
 * section "Background: What Are State Space Models?" and of the
 * paperlayer.ai summary, section 2; cheap generation, summary section 5):
 *     x_j <- Abar_j x_j + Bbar_j u_t,   y_t = 2 Re(sum_j C_j x_j) + D u_t
 * for t = 0 .. K-1, Abar = exp(dt A), Bbar = dt B: the recurrence and state
 * layout of h3conv_state_pass, so x_out of a state-passing prefix continues
 * here token by token.
 *
 *   u      [B,H,K]  io dtype      the next K inputs of every row
 *   A,Bm,C [H,S]    complex fp32  SSM parameters
 *   dt, D  [H]      fp32
 *   x      [B,H,S]  complex fp32  state: read, then overwritten with the
 *                                 state after the K steps
 *   y      [B,H,K]  io dtype      outputs (must not overlap any input or x)
 * Supported: 1 <= S <= H3CONV_MAX_STATE, H * ceil(B/4) < 2^26 (one wave
 * per channel and four batch rows; about 2^28 rows), else
 * H3CONV_ERR_UNSUPPORTED.  The recurrence runs in fp32.
 */
h3conv_status h3conv_ssm_step(const void *u, const float *A, const float *Bm, const float *C,
                              const float *dt, const float *D, float *x, void *y, int64_t B, int64_t H,
                              int64_t K, int64_t S, int io, void *stream);

/*
 * H3 mixing with head dimension 1 (the blog's section "The Solution, Part 1";
 * paperlayer.ai summary section 3), channel-last layout:
 *     s_t   = sum_{i<L, i<=t} w[d,i] * k_{t-i}     shift SSM = short causal FIR
 *     m_t   = s_t * v_t                           first multiplicative gate
 *     z_t   = sum_{tau<=t} f[d,t-tau] m_tau + D[d] m_t   diagonal-SSM long conv
 *     out_t = q_t * z_t                           second multiplicative gate
 *
 *   q, k, v [B,N,Dm] io dtype   w [Dm,L] fp32   f [Dm,N] fp32   D [Dm] fp32
 *   out     [B,N,Dm] io dtype (must not overlap any input)
 *   ws, ws_bytes  for H3CONV_F16 / H3CONV_BF16: workspace of at least
 *             h3conv_workspace_size(H3CONV_OP_H3_MIX, B, Dm, N, 0, 0) bytes,
 *             16-byte aligned, overlapping nothing else (m and z are staged
 *             there channel-major, as bf16); ignored for H3CONV_F32 (may be
 *             NULL).  Too small or NULL: H3CONV_ERR_WORKSPACE.
 * Supported: 1 <= N <= H3CONV_MAX_FUSED_N, 1 <= L <= 4, B*Dm < 2^31; for
 * 16-bit activations also B <= 65535 and the h3conv_fft_conv limit with
 * H = Dm.  Otherwise H3CONV_ERR_UNSUPPORTED, before any HIP call.
 */
h3conv_status h3conv_h3_mix(const void *q, const void *k, const void *v, const float *w,
                            const float *f, const float *D, void *out, int64_t B, int64_t N,
                            int64_t Dm, int64_t L, int io, void *ws, size_t ws_bytes,
                            void *stream);

/*
 * Multi-head H3 mixing, head dimension dh (model width Dm = heads * dh),
 * channel-last layout.  The summary page's section 3 (cost O(d^2 N + d N
 * log N) for an O(1) head dimension) and Appendix C "H3 Model to Solve
 * Lambda" (keys in separate heads), with the blog's "The Solution, Part 1";
 * the readings (the gates as an outer product and a contraction, one filter
 * per state entry) are this library's.  For head h, channels h*dh + (0..dh-1):
 *     s[t,i]   = sum_{l<L, l<=t} w[h*dh+i, l] k[t-l, h*dh+i]   shift SSM on keys
 *     m[t,i,j] = s[t,i] v[t, h*dh+j]                          outer product
 *     z[.,i,j] = (f[c] * m[.,i,j])[:N] + D[c] m[.,i,j],  c = (h*dh+i)*dh + j
 *     out[t, h*dh+j] = sum_i q[t, h*dh+i] z[t,i,j]
 * dh = 1 is h3conv_h3_mix.
 *
 *   q, k, v, out [B,N,Dm] io dtype;  w [Dm,L] fp32;  f [Dm*dh, N] fp32;
 *   D [Dm*dh] fp32
 *   ws, ws_bytes  workspace: the state entries staged channel-major twice,
 *                 2 * B*N*Dm*dh elements of bf16 (16-bit activations; this
 *                 is h3conv_workspace_size(H3CONV_OP_H3_MIX_MH, B, Dm, N, dh,
 *                 0)) or fp32 (fp32 activations, twice that), 16-byte
 *                 aligned, overlapping nothing else.
 * Supported: dh a power of two <= 32 dividing Dm, 1 <= L <= 4,
 * 1 <= N <= H3CONV_MAX_FUSED_N, B <= 65535, and the h3conv_fft_conv limits
 * for B x (Dm*dh) rows.
 */
h3conv_status h3conv_h3_mix_mh(const void *q, const void *k, const void *v, const float *w,
                               const float *f, const float *D, void *out, int64_t B, int64_t N,
                               int64_t Dm, int64_t dh, int64_t L, int io, void *ws, size_t ws_bytes,
                               void *stream);

/*
 * Workspace bytes an operation needs for the given sizes (0 if none).
 * `op` is an h3conv_op; unused size arguments are ignored.  For
 * H3CONV_OP_H3_MIX, H is the model width Dm and the size is that of the
 * 16-bit activation path (the fp32 path needs none).  For
 * H3CONV_OP_H3_MIX_MH, H is Dm and S the head dimension dh; the size is that
 * of the 16-bit activation path (fp32 activations need twice as much).  Returns (size_t)-1 for
 * sizes the operation does not support.
 */
size_t h3conv_workspace_size(int op, int64_t B, int64_t H, int64_t N, int64_t S, int64_t T);

/* Static, NUL-terminated description of a status code. */
const char *h3conv_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int h3conv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* H3CONV_H */
