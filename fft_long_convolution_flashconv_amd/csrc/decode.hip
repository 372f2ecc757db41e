// decode.hip -- recurrent single-step generation of the diagonal SSM.
//
// The recurrent view of the SSM (the deep-paper.org blog on "Hungry Hungry
// Hippos", section "Background: What Are State Space Models?": the state is
// updated from the previous state with the current input, and the output is
// read from the state; the paperlayer.ai summary, section 2): one new token
// per step costs O(S) per channel, independent of the sequence length, which
// is what makes generation cheap (summary page, section 5).  Per row (b, h)
// and step t:
//   x_j <- Abar_j x_j + Bbar_j u_t,   y_t = 2 Re(sum_j C_j x_j) + D u_t
// with Abar = exp(dt A), Bbar = dt B: the same recurrence, state layout
// ([B, H, S] complex fp32) and readings as h3conv_state_pass, so a prefix run
// by state passing continues here token by token.
//
// One wave per row, lane j holding mode j; K steps run in order, the inputs
// of 64 steps loaded by the wave at once and the outputs stored the same way.
#include <hip/hip_runtime.h>

#include "h3conv_device.h"
#include "h3conv_internal.h"

namespace h3c {

__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

template <int IO>
__global__ __launch_bounds__(256) void k_ssm_step(const typename io_elem<IO>::T *__restrict__ u,
                                                 const float *__restrict__ A, const float *__restrict__ Bm,
                                                 const float *__restrict__ C, const float *__restrict__ dt,
                                                 const float *__restrict__ D, float *__restrict__ x,
                                                 typename io_elem<IO>::T *__restrict__ y, int64_t rows, int H,
                                                 int64_t K, int S) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;  // (the whole wave)
    const int h = (int)(r % H);
    // this lane's mode: Abar = exp(dt A), Bbar = dt B.  The phase dt Im A
    // (up to ~1e2 rad) is formed exactly in fp64 and reduced by whole turns
    // there; the fp32 sine, cosine and exponential of the reduced values are
    // then accurate to about one ulp.
    cf ab = mk(0.f, 0.f), bb = mk(0.f, 0.f), cc = mk(0.f, 0.f), xs = mk(0.f, 0.f);
    if (lane < S) {
        const size_t o = ((size_t)h * S + lane) * 2;
        const double dth = (double)dt[h];
        constexpr double kTwoPi = 6.283185307179586232;
        const double ph = dth * (double)A[o + 1];
        const float phr = (float)fma(-rint(ph * (1.0 / kTwoPi)), kTwoPi, ph);
        float sn, cs;
        sincosf(phr, &sn, &cs);
        const float m = expf((float)(dth * (double)A[o]));
        ab = mk(m * cs, m * sn);
        bb = mk((float)(dth * (double)Bm[o]), (float)(dth * (double)Bm[o + 1]));
        cc = mk(C[o], C[o + 1]);
        xs = mk(x[((size_t)r * S + lane) * 2], x[((size_t)r * S + lane) * 2 + 1]);
    }
    const float dh = D[h];
    const typename io_elem<IO>::T *ur = u + r * K;
    typename io_elem<IO>::T *yr = y + r * K;
    for (int64_t t0 = 0; t0 < K; t0 += 64) {
        const int nt = (int)((K - t0) < 64 ? (K - t0) : 64);
        const float uv = lane < nt ? ld_io<IO>(ur + t0 + lane) : 0.f;
        float yv = 0.f;
        for (int k = 0; k < nt; ++k) {
            const float ut = __shfl(uv, k, 64);
            xs = cadd(cmul(ab, xs), cscale(bb, ut));
            const float s = wave_sum64(2.f * fmaf(cc.x, xs.x, -cc.y * xs.y));
            if (lane == k) yv = fmaf(dh, ut, s);
        }
        if (lane < nt) st_io<IO>(yr + t0 + lane, yv);
    }
    if (lane < S) {
        x[((size_t)r * S + lane) * 2] = xs.x;
        x[((size_t)r * S + lane) * 2 + 1] = xs.y;
    }
}

hipError_t launch_ssm_step(const void *u, const float *A, const float *Bm, const float *C, const float *dt,
                           const float *D, float *x, void *y, int64_t B, int64_t H, int64_t K, int S, int io,
                           hipStream_t s) {
    const int64_t rows = B * H;
    const dim3 grid((unsigned)((rows + 3) / 4));
    switch (io) {
        case IO_F32:
            return launch(k_ssm_step<IO_F32>, grid, dim3(256), 0, s, (const float *)u, A, Bm, C, dt, D, x,
                          (float *)y, rows, (int)H, K, S);
        case IO_F16:
            return launch(k_ssm_step<IO_F16>, grid, dim3(256), 0, s, (const _Float16 *)u, A, Bm, C, dt, D, x,
                          (_Float16 *)y, rows, (int)H, K, S);
        case IO_BF16:
            return launch(k_ssm_step<IO_BF16>, grid, dim3(256), 0, s, (const uint16_t *)u, A, Bm, C, dt, D, x,
                          (uint16_t *)y, rows, (int)H, K, S);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace h3c
