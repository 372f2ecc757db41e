// h3conv_internal.h -- launchers shared between the C-ABI shim and the kernel
// translation units.  Every launcher assumes its arguments were validated by
// the shim (sizes in range, pointers non-null and aligned) and only enqueues
// work on `stream`; it returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>

namespace h3c {

// Enqueue kernel `k` on `s` and return the status of this launch itself
// (hipLaunchKernel's own return value, never an error left on the thread by
// an earlier, unrelated call).  The arguments are converted to the kernel's
// parameter types before their addresses are taken.
template <class... P, class... A>
inline hipError_t launch(void (*k)(P...), dim3 grid, dim3 block, size_t shmem, hipStream_t s, A &&...a) {
    static_assert(sizeof...(P) == sizeof...(A), "one argument per kernel parameter");
    std::tuple<P...> args(static_cast<P>(a)...);
    return std::apply(
        [&](P &...v) {
            void *ptrs[] = {(void *)&v..., nullptr};
            return hipLaunchKernel((const void *)k, grid, block, ptrs, shmem, s);
        },
        args);
}

// Whether the fused 16-bit convolution of rows of N samples over H channels
// keeps every row byte offset of one launch within 32 bits (the launcher
// slices the batch, but one slice must hold at least a few rows).  Always
// true for fp32 activations and for the small transforms of the fp32 engine.
bool fft_conv_rows_fit(int64_t H, int64_t N, int io);

// Padded length 2*Np of the fused transform for a sequence of N samples:
// Np = max(32, next power of two >= N).
int fused_log2m(int64_t N);

hipError_t launch_fft_conv(const void *u, const float *f, const float *D, void *y, int B, int H,
                           int N, int io, hipStream_t s);

// Multi-head H3 mixing (head dimension dh); workspace bytes for io.
hipError_t launch_h3_mix_mh(const void *q, const void *k, const void *v, const float *w, const float *f,
                            const float *D, void *out, int B, int N, int Dm, int dh, int L, int io, void *ws,
                            hipStream_t s);
size_t h3_mix_mh_workspace(int64_t B, int64_t N, int64_t Dm, int64_t dh, int io);

// Bidirectional copies: causal convolution with f plus anti-causal with g.
hipError_t launch_fft_bidir(const void *u, const float *f, const float *g, const float *D, void *y, int B, int H,
                            int N, int io, hipStream_t s);

// Gradients du, df, dD of the causal convolution for an upstream dy.
hipError_t launch_fft_conv_bwd(const void *u, const float *f, const float *D, const void *dy, void *du,
                               float *df, float *dD, int B, int H, int N, int io, hipStream_t s);

hipError_t launch_h3_mix(const void *q, const void *k, const void *v, const float *w,
                         const float *f, const float *D, void *out, int B, int N, int Dm, int L,
                         int io, void *ws, hipStream_t s);
size_t h3_mix_workspace(int64_t B, int64_t N, int64_t Dm);

hipError_t launch_ssm_filter(const float *A, const float *Bm, const float *C, const float *dt,
                             float *f, int H, int S, int64_t N, hipStream_t s);

// Workspace bytes of state passing: for any activation type (the larger of
// the two paths' layouts), and for one activation type.
size_t state_pass_workspace(int64_t B, int64_t H, int64_t N, int64_t S, int64_t T);
size_t state_pass_workspace_io(int64_t B, int64_t H, int64_t N, int64_t S, int64_t T, int io);

// x_out = x_in (or zero when x_in is NULL), n complex values: the final
// state of a state passing over zero samples.
hipError_t launch_state_copy(const float *x_in, float *x_out, int64_t n, hipStream_t s);

hipError_t launch_state_pass(const void *u, const float *A, const float *Bm, const float *C,
                             const float *dt, const float *D, const float *x_in, float *x_out,
                             void *y, int B, int H, int64_t N, int S, int T, int io, void *ws,
                             hipStream_t s);

// K steps of the recurrence per row from the state x (updated in place).
// Whether the generation step's grid for B x H rows fits one dispatch.
bool ssm_step_fits(int64_t B, int64_t H);
hipError_t launch_ssm_step(const void *u, const float *A, const float *Bm, const float *C, const float *dt,
                           const float *D, float *x, void *y, int64_t B, int64_t H, int64_t K, int S, int io,
                           hipStream_t s);

}  // namespace h3c
