// h3mh.hip -- multi-head H3 mixing (head dimension dh > 1).
//
// After the paperlayer.ai summary of "Hungry Hungry Hippos", section 3 (cost
// O(d^2 N + d N log N) for an O(1) head dimension) and Appendix C "H3 Model
// to Solve Lambda" (keys in separate heads), and the deep-paper.org blog,
// "The Solution, Part 1" (Q gate on the diagonal SSM of shift(K) gate V).
// For head h and step t, with s = shift SSM of the keys:
//   m[t,i,j] = s[t,i] v[t,j]                     outer product per head
//   z[.,i,j] = (f_(i,j) * m[.,i,j])[:N] + D_(i,j) m[.,i,j]
//   out[t,j] = sum_i q[t,i] z[t,i,j]
// Three launches: gate-in writes the state entries as channel-major rows
// [B, Dm*dh, N] (row (h dh + i) dh + j), the fused convolution kernels run
// over those rows with one filter per row, and gate-out contracts them with
// the queries back to channel-last [B, N, Dm].  The intermediates are bf16
// for 16-bit activations (fp32 range, so no product overflows them) and fp32
// for fp32 activations.  A tile covers 32 steps and 256 state rows, i.e.
// 256 / dh model channels: whole heads.
#include <hip/hip_runtime.h>

#include "h3conv_device.h"
#include "h3conv_internal.h"

namespace h3c {

constexpr int MH_TT = 32, MH_ROWS = 256;

template <class MT>
__device__ __forceinline__ MT mh_put(float x) {
    if constexpr (sizeof(MT) == 4) return x;
    else return f32_to_bf16_rne(x);
}
template <class MT>
__device__ __forceinline__ float mh_get(MT x) {
    if constexpr (sizeof(MT) == 4) return x;
    else return __uint_as_float((uint32_t)x << 16);
}

template <int IO, class MT>
__global__ __launch_bounds__(256) void k_h3mh_gate_in(const typename io_elem<IO>::T *__restrict__ k,
                                                     const typename io_elem<IO>::T *__restrict__ v,
                                                     const float *__restrict__ w, MT *__restrict__ mT, int N,
                                                     int Dm, int dh, int L) {
    const int TD = MH_ROWS / dh;  // model channels of the tile
    __shared__ float ks[(MH_TT + 3) * (MH_ROWS + 1)];
    __shared__ float vs[MH_TT * (MH_ROWS + 1)];
    const int tid = threadIdx.x;
    const int d0 = blockIdx.x * TD, t0 = blockIdx.y * MH_TT, b = blockIdx.z;
    const size_t base = (size_t)b * N * Dm;
    // k at steps t0 - 3 .. t0 + TT - 1 (the shift's history), v at t0 .. t0 + TT - 1
    for (int e = tid; e < (MH_TT + 3) * TD; e += 256) {
        const int r = e / TD, c = e % TD, t = t0 - 3 + r, d = d0 + c;
        ks[r * (MH_ROWS + 1) + c] = (t >= 0 && t < N && d < Dm) ? ld_io<IO>(k + base + (size_t)t * Dm + d) : 0.f;
    }
    for (int e = tid; e < MH_TT * TD; e += 256) {
        const int r = e / TD, c = e % TD, t = t0 + r, d = d0 + c;
        vs[r * (MH_ROWS + 1) + c] = (t < N && d < Dm) ? ld_io<IO>(v + base + (size_t)t * Dm + d) : 0.f;
    }
    __syncthreads();
    // items: (state row rl of the tile, chunk of 8 steps)
    for (int e = tid; e < MH_ROWS * (MH_TT / 8); e += 256) {
        const int rl = e / (MH_TT / 8), ck = e % (MH_TT / 8);
        const int kc = rl / dh, j = rl % dh, vc = (kc / dh) * dh + j;
        const int d = d0 + kc;
        if (d >= Dm) continue;
        float wt[4];
#pragma unroll
        for (int l = 0; l < 4; ++l) wt[l] = l < L ? w[(size_t)d * L + l] : 0.f;
        MT *row = mT + ((size_t)b * Dm * dh + (size_t)d0 * dh + rl) * N;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int tl = 8 * ck + q, t = t0 + tl;
            if (t >= N) break;
            float s = 0.f;
#pragma unroll
            for (int l = 0; l < 4; ++l) s = fmaf(wt[l], ks[(tl + 3 - l) * (MH_ROWS + 1) + kc], s);
            row[t] = mh_put<MT>(s * vs[tl * (MH_ROWS + 1) + vc]);
        }
    }
}

template <int IO, class MT>
__global__ __launch_bounds__(256) void k_h3mh_gate_out(const typename io_elem<IO>::T *__restrict__ q,
                                                      const MT *__restrict__ zT,
                                                      typename io_elem<IO>::T *__restrict__ out, int N, int Dm,
                                                      int dh) {
    const int TD = MH_ROWS / dh;
    __shared__ float zs[MH_ROWS * (MH_TT + 1)];
    __shared__ float qs[MH_TT * (MH_ROWS + 1)];
    const int tid = threadIdx.x;
    const int d0 = blockIdx.x * TD, t0 = blockIdx.y * MH_TT, b = blockIdx.z;
    const size_t base = (size_t)b * N * Dm;
    for (int e = tid; e < MH_ROWS * MH_TT; e += 256) {
        const int rl = e / MH_TT, tl = e % MH_TT, t = t0 + tl;
        const bool ok = t < N && d0 + rl / dh < Dm;
        zs[rl * (MH_TT + 1) + tl] = ok ? mh_get<MT>(zT[((size_t)b * Dm * dh + (size_t)d0 * dh + rl) * N + t]) : 0.f;
    }
    for (int e = tid; e < MH_TT * TD; e += 256) {
        const int tl = e / TD, c = e % TD, t = t0 + tl, d = d0 + c;
        qs[tl * (MH_ROWS + 1) + c] = (t < N && d < Dm) ? ld_io<IO>(q + base + (size_t)t * Dm + d) : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < MH_TT * TD; e += 256) {
        const int tl = e / TD, c = e % TD, t = t0 + tl, d = d0 + c;
        if (t >= N || d >= Dm) continue;
        const int h0 = (c / dh) * dh, j = c % dh;  // first model channel of the head, value index
        float acc = 0.f;
        for (int i = 0; i < dh; ++i)
            acc = fmaf(qs[tl * (MH_ROWS + 1) + h0 + i], zs[((h0 + i) * dh + j) * (MH_TT + 1) + tl], acc);
        st_io<IO>(out + base + (size_t)t * Dm + d, acc);
    }
}

size_t h3_mix_mh_workspace(int64_t B, int64_t N, int64_t Dm, int64_t dh, int io) {
    const size_t one = ((size_t)(B * N * Dm * dh) * (io == IO_F32 ? 4 : 2) + 255) & ~(size_t)255;
    return 2 * one;
}

template <int IO, class MT>
static hipError_t mh_run(const void *q, const void *k, const void *v, const float *w, const float *f, const float *D,
                         void *out, int B, int N, int Dm, int dh, int L, void *ws, hipStream_t s) {
    using T = typename io_elem<IO>::T;
    const size_t one = h3_mix_mh_workspace(B, N, Dm, dh, IO) / 2;
    MT *mT = (MT *)ws;
    MT *zT = (MT *)((char *)ws + one);
    const int TD = MH_ROWS / dh;
    const dim3 grid((Dm + TD - 1) / TD, (N + MH_TT - 1) / MH_TT, B);
    hipError_t e = launch(k_h3mh_gate_in<IO, MT>, grid, dim3(256), 0, s, (const T *)k, (const T *)v, w, mT, N, Dm, dh,
                          L);
    if (e != hipSuccess) return e;
    // the convolution over the B x (Dm dh) state rows, one filter per row
    e = launch_fft_conv(mT, f, D, zT, B, Dm * dh, N, sizeof(MT) == 4 ? IO_F32 : IO_BF16, s);
    if (e != hipSuccess) return e;
    return launch(k_h3mh_gate_out<IO, MT>, grid, dim3(256), 0, s, (const T *)q, (const MT *)zT, (T *)out, N, Dm, dh);
}

hipError_t launch_h3_mix_mh(const void *q, const void *k, const void *v, const float *w, const float *f,
                            const float *D, void *out, int B, int N, int Dm, int dh, int L, int io, void *ws,
                            hipStream_t s) {
    switch (io) {
        case IO_F32: return mh_run<IO_F32, float>(q, k, v, w, f, D, out, B, N, Dm, dh, L, ws, s);
        case IO_F16: return mh_run<IO_F16, uint16_t>(q, k, v, w, f, D, out, B, N, Dm, dh, L, ws, s);
        case IO_BF16: return mh_run<IO_BF16, uint16_t>(q, k, v, w, f, D, out, B, N, Dm, dh, L, ws, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace h3c
