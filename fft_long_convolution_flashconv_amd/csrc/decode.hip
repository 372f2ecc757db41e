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
// One wave per channel and group of batch rows, lane j holding mode j of
// each row; K steps run in order, the inputs of 64 steps loaded by the wave
// at once and the outputs stored the same way.
#include <hip/hip_runtime.h>

#include "h3conv_device.h"
#include "h3conv_internal.h"

namespace h3c {

// Sum over the 64 lanes of a wave with DPP row operations (pairs, quads,
// half-row and row mirrors, then the row broadcasts), no LDS round trips;
// the total is read from lane 63 (wave-uniform).
template <int CTRL, int RMASK>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, RMASK, 0xf, false));
}
__device__ __forceinline__ float wave_sum64(float v) {
    v = dpp_add<0xb1, 0xf>(v);   // quad_perm [1,0,3,2]
    v = dpp_add<0x4e, 0xf>(v);   // quad_perm [2,3,0,1]
    v = dpp_add<0x141, 0xf>(v);  // row_half_mirror
    v = dpp_add<0x140, 0xf>(v);  // row_mirror
    v = dpp_add<0x142, 0xa>(v);  // row_bcast:15 (rows 1, 3)
    v = dpp_add<0x143, 0xc>(v);  // row_bcast:31 (rows 2, 3)
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Rows per wave: one wave takes one channel h for kRowsPerWave batch rows
// (rows b*H + h), so the channel's Abar, Bbar and C are formed once per wave
// and shared; the rows' loads are issued together and their steps interleave,
// which keeps several independent chains in flight.
constexpr int kRowsPerWave = 4;

template <int IO>
__global__ __launch_bounds__(256) void k_ssm_step(const typename io_elem<IO>::T *__restrict__ u,
                                                 const float *__restrict__ A, const float *__restrict__ Bm,
                                                 const float *__restrict__ C, const float *__restrict__ dt,
                                                 const float *__restrict__ D, float *__restrict__ x,
                                                 typename io_elem<IO>::T *__restrict__ y, int64_t Bn, int H,
                                                 int64_t K, int S) {
    constexpr int RW = kRowsPerWave;
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int h = (int)(w % H);
    const int64_t b0 = (w / H) * RW;
    if (b0 >= Bn) return;  // (the whole wave)
    const float dh = D[h];
    cf ab = mk(0.f, 0.f), bb = ab, cc = ab;
    if (lane < S) {
        // this lane's mode: Abar = exp(dt A), Bbar = dt B.  The phase dt Im A
        // (up to ~1e2 rad) is formed exactly in fp64 and reduced by whole
        // turns there; the fp32 sine, cosine and exponential of the reduced
        // values are then accurate to about one ulp.
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
    }
    int64_t row[RW];
    bool ok[RW];
    cf xs[RW];
#pragma unroll
    for (int q = 0; q < RW; ++q) {
        ok[q] = b0 + q < Bn;
        row[q] = (b0 + q) * H + h;
        xs[q] = mk(0.f, 0.f);
        if (ok[q] && lane < S)
            xs[q] = mk(x[((size_t)row[q] * S + lane) * 2], x[((size_t)row[q] * S + lane) * 2 + 1]);
    }
    for (int64_t t0 = 0; t0 < K; t0 += 64) {
        const int nt = (int)((K - t0) < 64 ? (K - t0) : 64);
        float uv[RW], yv[RW];
#pragma unroll
        for (int q = 0; q < RW; ++q) {
            uv[q] = (ok[q] && lane < nt) ? ld_io<IO>(u + row[q] * K + t0 + lane) : 0.f;
            yv[q] = 0.f;
        }
        for (int k = 0; k < nt; ++k) {
#pragma unroll
            for (int q = 0; q < RW; ++q) {
                const float ut = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, uv[q]), k));
                xs[q] = cadd(cmul(ab, xs[q]), cscale(bb, ut));
                const float sm = wave_sum64(2.f * fmaf(cc.x, xs[q].x, -cc.y * xs[q].y));
                if (lane == k) yv[q] = fmaf(dh, ut, sm);
            }
        }
#pragma unroll
        for (int q = 0; q < RW; ++q)
            if (ok[q] && lane < nt) st_io<IO>(y + row[q] * K + t0 + lane, yv[q]);
    }
#pragma unroll
    for (int q = 0; q < RW; ++q) {
        if (ok[q] && lane < S) {
            x[((size_t)row[q] * S + lane) * 2] = xs[q].x;
            x[((size_t)row[q] * S + lane) * 2 + 1] = xs[q].y;
        }
    }
}

bool ssm_step_fits(int64_t B, int64_t H) {
    // the launch's work-item count (waves x 64, in blocks of 256) must fit
    // the 32-bit grid size of a dispatch
    if (B <= 0 || H <= 0) return true;
    const int64_t groups = (B + kRowsPerWave - 1) / kRowsPerWave;
    return H <= (int64_t(1) << 26) && groups <= (int64_t(1) << 26) && H * groups <= (int64_t(1) << 26) - 4;
}

hipError_t launch_ssm_step(const void *u, const float *A, const float *Bm, const float *C, const float *dt,
                           const float *D, float *x, void *y, int64_t B, int64_t H, int64_t K, int S, int io,
                           hipStream_t s) {
    // waves: H channels x ceil(B / kRowsPerWave) batch groups, four per block
    const int64_t waves = H * ((B + kRowsPerWave - 1) / kRowsPerWave);
    const dim3 grid((unsigned)((waves + 3) / 4));
    switch (io) {
        case IO_F32:
            return launch(k_ssm_step<IO_F32>, grid, dim3(256), 0, s, (const float *)u, A, Bm, C, dt, D, x,
                          (float *)y, B, (int)H, K, S);
        case IO_F16:
            return launch(k_ssm_step<IO_F16>, grid, dim3(256), 0, s, (const _Float16 *)u, A, Bm, C, dt, D, x,
                          (_Float16 *)y, B, (int)H, K, S);
        case IO_BF16:
            return launch(k_ssm_step<IO_BF16>, grid, dim3(256), 0, s, (const uint16_t *)u, A, Bm, C, dt, D, x,
                          (uint16_t *)y, B, (int)H, K, S);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace h3c
