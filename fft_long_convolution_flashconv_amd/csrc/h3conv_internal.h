// h3conv_internal.h -- launchers shared between the C-ABI shim and the kernel
// translation units.  Every launcher assumes its arguments were validated by
// the shim (sizes in range, pointers non-null and aligned) and only enqueues
// work on `stream`; it returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace h3c {

// Padded length 2*Np of the fused transform for a sequence of N samples:
// Np = max(32, next power of two >= N).
int fused_log2m(int64_t N);

hipError_t launch_fft_conv(const void *u, const float *f, const float *D, void *y, int B, int H,
                           int N, int io, hipStream_t s);

hipError_t launch_h3_mix(const void *q, const void *k, const void *v, const float *w,
                         const float *f, const float *D, void *out, int B, int N, int Dm, int L,
                         int io, void *ws, hipStream_t s);
size_t h3_mix_workspace(int64_t B, int64_t N, int64_t Dm);

hipError_t launch_ssm_filter(const float *A, const float *Bm, const float *C, const float *dt,
                             float *f, int H, int S, int64_t N, hipStream_t s);

size_t state_pass_workspace(int64_t B, int64_t H, int64_t N, int64_t S, int64_t T);

hipError_t launch_state_pass(const void *u, const float *A, const float *Bm, const float *C,
                             const float *dt, const float *D, const float *x_in, float *x_out,
                             void *y, int B, int H, int64_t N, int S, int T, int io, void *ws,
                             hipStream_t s);

}  // namespace h3c
