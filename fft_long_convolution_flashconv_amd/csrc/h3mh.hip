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
// 256 / dh model channels: whole heads (dh <= 32, so a tile spans at least 8
// model channels, one 16-byte access).
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

// 8 consecutive elements of type T at p (n of them valid, the rest zero) as
// floats; one 16-byte access when `vec` (16-bit T) allows it
template <int IO>
__device__ __forceinline__ void mh_load8(const typename io_elem<IO>::T *p, int n, bool vec, float (&o)[8]) {
    using T = typename io_elem<IO>::T;
    if constexpr (sizeof(T) == 2) {
        if (vec && n >= 8) {
            const uint4 v = *(const uint4 *)p;
            const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint16_t lo = (uint16_t)(w4[e] & 0xffffu), hi = (uint16_t)(w4[e] >> 16);
                o[2 * e] = ld_io<IO>((const T *)&lo);
                o[2 * e + 1] = ld_io<IO>((const T *)&hi);
            }
            return;
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = e < n ? ld_io<IO>(p + e) : 0.f;
}

template <int IO, class MT>
__global__ __launch_bounds__(256) void k_h3mh_gate_in(const typename io_elem<IO>::T *__restrict__ k,
                                                     const typename io_elem<IO>::T *__restrict__ v,
                                                     const float *__restrict__ w, MT *__restrict__ mT, int N,
                                                     int Dm, int dh, int L, int vec) {
    const int TD = MH_ROWS / dh;  // model channels of the tile (whole heads)
    constexpr int P = MH_ROWS + 1;
    __shared__ float ks[(MH_TT + 3) * P];
    __shared__ float vs[MH_TT * P];
    const int tid = threadIdx.x;
    const int d0 = blockIdx.x * TD, t0 = blockIdx.y * MH_TT, b = blockIdx.z;
    const size_t base = (size_t)b * N * Dm;
    // k at steps t0 - 3 .. t0 + TT - 1 (the shift's history), v at t0 ..
    // t0 + TT - 1, 8 channels per access
    const int CR = TD / 8;
    for (int e = tid; e < (MH_TT + 3) * CR; e += 256) {
        const int r = e / CR, c = 8 * (e % CR), t = t0 - 3 + r, d = d0 + c;
        float x[8];
        if (t >= 0 && t < N && d < Dm) mh_load8<IO>(k + base + (size_t)t * Dm + d, Dm - d, vec, x);
        else for (int q = 0; q < 8; ++q) x[q] = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) ks[r * P + c + q] = x[q];
    }
    for (int e = tid; e < MH_TT * CR; e += 256) {
        const int r = e / CR, c = 8 * (e % CR), t = t0 + r, d = d0 + c;
        float x[8];
        if (t < N && d < Dm) mh_load8<IO>(v + base + (size_t)t * Dm + d, Dm - d, vec, x);
        else for (int q = 0; q < 8; ++q) x[q] = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) vs[r * P + c + q] = x[q];
    }
    __syncthreads();
    // items: (state row rl of the tile, chunk of 8 steps): one 16-byte store
    // of bf16 (8 steps) or two of fp32 (4 steps each)
    for (int e = tid; e < MH_ROWS * (MH_TT / 8); e += 256) {
        const int rl = e / (MH_TT / 8), ck = e % (MH_TT / 8);
        const int kc = rl / dh, j = rl % dh, vc = (kc / dh) * dh + j;
        const int d = d0 + kc;
        if (d >= Dm) continue;
        float wt[4];
#pragma unroll
        for (int l = 0; l < 4; ++l) wt[l] = l < L ? w[(size_t)d * L + l] : 0.f;
        MT o[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int tl = 8 * ck + q;
            float sh = 0.f;
#pragma unroll
            for (int l = 0; l < 4; ++l) sh = fmaf(wt[l], ks[(tl + 3 - l) * P + kc], sh);
            o[q] = mh_put<MT>(sh * vs[tl * P + vc]);
        }
        MT *row = mT + ((size_t)b * Dm * dh + (size_t)d0 * dh + rl) * N + t0 + 8 * ck;
        const int nt = N - (t0 + 8 * ck);
        if (vec && nt >= 8) {
            if constexpr (sizeof(MT) == 2) {
                uint4 u;
                u.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16); u.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
                u.z = (uint32_t)o[4] | ((uint32_t)o[5] << 16); u.w = (uint32_t)o[6] | ((uint32_t)o[7] << 16);
                *(uint4 *)row = u;
            } else {
                *(float4 *)row = make_float4(o[0], o[1], o[2], o[3]);
                *(float4 *)(row + 4) = make_float4(o[4], o[5], o[6], o[7]);
            }
        } else {
            for (int q = 0; q < 8 && q < nt; ++q) row[q] = o[q];
        }
    }
}

template <int IO, class MT>
__global__ __launch_bounds__(256) void k_h3mh_gate_out(const typename io_elem<IO>::T *__restrict__ q,
                                                      const MT *__restrict__ zT,
                                                      typename io_elem<IO>::T *__restrict__ out, int N, int Dm,
                                                      int dh, int vec) {
    using T = typename io_elem<IO>::T;
    const int TD = MH_ROWS / dh;
    constexpr int PZ = MH_TT + 1, PQ = MH_ROWS + 1;
    __shared__ float zs[MH_ROWS * PZ];
    __shared__ float qs[MH_TT * PQ];
    const int tid = threadIdx.x;
    const int d0 = blockIdx.x * TD, t0 = blockIdx.y * MH_TT, b = blockIdx.z;
    const size_t base = (size_t)b * N * Dm;
    // z rows of the tile, 8 steps per access
    for (int e = tid; e < MH_ROWS * (MH_TT / 8); e += 256) {
        const int rl = e / (MH_TT / 8), tl = 8 * (e % (MH_TT / 8)), t = t0 + tl;
        float x[8];
        const bool ok = t < N && d0 + rl / dh < Dm;
        const MT *src = zT + ((size_t)b * Dm * dh + (size_t)d0 * dh + rl) * N + t;
        if (ok && vec && N - t >= 8) {
            if constexpr (sizeof(MT) == 2) {
                const uint4 u = *(const uint4 *)src;
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[2 * i] = mh_get<MT>((MT)(w4[i] & 0xffffu));
                    x[2 * i + 1] = mh_get<MT>((MT)(w4[i] >> 16));
                }
            } else {
                const float4 a = *(const float4 *)src, c = *(const float4 *)(src + 4);
                x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = (ok && t + i < N) ? mh_get<MT>(src[i]) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) zs[rl * PZ + tl + i] = x[i];
    }
    const int CR = TD / 8;
    for (int e = tid; e < MH_TT * CR; e += 256) {
        const int tl = e / CR, c = 8 * (e % CR), t = t0 + tl, d = d0 + c;
        float x[8];
        if (t < N && d < Dm) mh_load8<IO>(q + base + (size_t)t * Dm + d, Dm - d, vec, x);
        else for (int i = 0; i < 8; ++i) x[i] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) qs[tl * PQ + c + i] = x[i];
    }
    __syncthreads();
    // outputs: (step, 8 consecutive channels), one 16-byte store (16-bit)
    for (int e = tid; e < MH_TT * CR; e += 256) {
        const int tl = e / CR, c0 = 8 * (e % CR), t = t0 + tl, d = d0 + c0;
        if (t >= N || d >= Dm) continue;
        float o[8];
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
            const int c = c0 + cc, h0 = (c / dh) * dh, j = c % dh;
            float acc = 0.f;
            for (int i = 0; i < dh; ++i) acc = fmaf(qs[tl * PQ + h0 + i], zs[((h0 + i) * dh + j) * PZ + tl], acc);
            o[cc] = acc;
        }
        T *dst = out + base + (size_t)t * Dm + d;
        if constexpr (sizeof(T) == 2) {
            if (vec && Dm - d >= 8) {
                uint16_t hv[8];
#pragma unroll
                for (int cc = 0; cc < 8; ++cc) {
                    T tmp;
                    st_io<IO>(&tmp, o[cc]);
                    hv[cc] = __builtin_bit_cast(uint16_t, tmp);
                }
                uint4 u;
                u.x = (uint32_t)hv[0] | ((uint32_t)hv[1] << 16); u.y = (uint32_t)hv[2] | ((uint32_t)hv[3] << 16);
                u.z = (uint32_t)hv[4] | ((uint32_t)hv[5] << 16); u.w = (uint32_t)hv[6] | ((uint32_t)hv[7] << 16);
                *(uint4 *)dst = u;
                continue;
            }
        }
        for (int cc = 0; cc < 8 && d + cc < Dm; ++cc) st_io<IO>(dst + cc, o[cc]);
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
    // 16-byte accesses along the contiguous dimension when sizes and
    // pointers allow (else element by element)
    const uintptr_t al = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)ws;
    const int vec = (N % 8 == 0 && Dm % 8 == 0 && (al & 15) == 0 && (one & 15) == 0) ? 1 : 0;
    hipError_t e = launch(k_h3mh_gate_in<IO, MT>, grid, dim3(256), 0, s, (const T *)k, (const T *)v, w, mT, N, Dm, dh,
                          L, vec);
    if (e != hipSuccess) return e;
    // the convolution over the B x (Dm dh) state rows, one filter per row
    e = launch_fft_conv(mT, f, D, zT, B, Dm * dh, N, sizeof(MT) == 4 ? IO_F32 : IO_BF16, s);
    if (e != hipSuccess) return e;
    return launch(k_h3mh_gate_out<IO, MT>, grid, dim3(256), 0, s, (const T *)q, (const MT *)zT, (T *)out, N, Dm, dh,
                  vec);
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
