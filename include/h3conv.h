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

typedef enum { H3CONV_OP_FFT_CONV = 0, H3CONV_OP_STATE_PASS = 1, H3CONV_OP_H3_MIX = 2 } h3conv_op;

/* Largest sequence length handled by one fused FFT block (2N <= 16384 points). */
#define H3CONV_MAX_FUSED_N 8192
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
 * Supported: 1 <= N <= H3CONV_MAX_FUSED_N (any N; longer inputs use
 * h3conv_state_pass), B*H < 2^31.  Otherwise H3CONV_ERR_UNSUPPORTED.
 */
h3conv_status h3conv_fft_conv(const void *u, const float *f, const float *D, void *y,
                              int64_t B, int64_t H, int64_t N, int io, void *stream);

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
 * Each chunk of T samples is convolved with the length-T SSM filter by FFT;
 * between chunks the state is carried as
 *     x_c = Abar^T x_{c-1} + sum_k Abar^{T-1-k} Bbar u_{c,k}
 * and chunk c adds 2 Re(sum_j C_j Abar_j^{t+1} x_{c-1,j}) at offset t.
 *
 *   u      [B,H,N]  io dtype      input
 *   A,Bm,C [H,S]    complex fp32  SSM parameters
 *   dt, D  [H]      fp32
 *   x_in   [B,H,S]  complex fp32  initial state, or NULL for zero
 *   x_out  [B,H,S]  complex fp32  final state after sample N-1, or NULL
 *   y      [B,H,N]  io dtype      output (must not overlap any input)
 *   ws, ws_bytes    workspace of at least h3conv_workspace_size(H3CONV_OP_STATE_PASS, ...)
 * Supported: T a power of two, 64 <= T <= H3CONV_MAX_FUSED_N, N % T == 0,
 * 1 <= S <= H3CONV_MAX_STATE.
 */
h3conv_status h3conv_state_pass(const void *u, const float *A, const float *Bm, const float *C,
                                const float *dt, const float *D, const float *x_in, float *x_out,
                                void *y, int64_t B, int64_t H, int64_t N, int64_t S, int64_t T,
                                int io, void *ws, size_t ws_bytes, void *stream);

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
 * Supported: 1 <= N <= H3CONV_MAX_FUSED_N, 1 <= L <= 4, B*Dm < 2^31.
 */
h3conv_status h3conv_h3_mix(const void *q, const void *k, const void *v, const float *w,
                            const float *f, const float *D, void *out, int64_t B, int64_t N,
                            int64_t Dm, int64_t L, int io, void *ws, size_t ws_bytes,
                            void *stream);

/*
 * Workspace bytes an operation needs for the given sizes (0 if none).
 * `op` is an h3conv_op; unused size arguments are ignored.  For
 * H3CONV_OP_H3_MIX, H is the model width Dm and the size is that of the
 * 16-bit activation path (the fp32 path needs none).  Returns (size_t)-1 for
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
