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
// for fp32 activations.  A tile covers the state rows of mh_td(dh) model
// channels (whole heads, at least 8 channels: one 16-byte access) over one
// 128-byte line of steps (fewer steps past 256 state rows); the gates' LDS
// is sized per launch for those channels, and the shift of each key channel
// is computed once per tile.  Head dimension 1 runs the H3 mix kernels (the
// same formula).
#include <hip/hip_runtime.h>

#include "h3conv_device.h"
#include "h3conv_internal.h"

namespace h3c {

// Model channels per gate tile: 128 state rows (at least 8 channels, one
// 16-byte access, and at least one whole head), so that several workgroups
// share a compute unit while their tiles load.
__host__ __device__ constexpr int mh_td(int dh) {
    const int c = 128 / dh > 8 ? 128 / dh : 8;  // 128 state rows, at least 8 channels
    return c > dh ? c : dh;                      // and at least one whole head
}

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

// Steps per gate tile: one 128-byte line of a state row of the
// intermediate (64 bf16 or 32 fp32 values), so every state-row access of
// the gates moves whole lines.
// (Tiles of more than 256 state rows, wide heads, take proportionally fewer
// steps, so that the output gate's z tile stays within 64 KiB of LDS.)
template <class MT>
__host__ __device__ constexpr int mh_tt(int dh) {
    return mh_td(dh) * dh <= 256 ? 128 / (int)sizeof(MT) : 128 / (int)sizeof(MT) * 256 / (mh_td(dh) * dh);
}

// LDS of the gates, sized per launch for the tile's TD = mh_td(dh) model
// channels (rows padded by one element against bank conflicts); activation
// tiles are kept in the activation type.
template <int IO, class MT>
static size_t mh_in_lds(int dh) {
    const int TD = mh_td(dh), TT = mh_tt<MT>(dh);
    return (size_t)(2 * TT + 3) * (TD + 1) * sizeof(typename io_elem<IO>::T);
}
template <int IO, class MT>
static size_t mh_out_lds(int dh) {
    const int TD = mh_td(dh), TT = mh_tt<MT>(dh);
    return (((size_t)TD * dh * (TT + 2) * sizeof(MT) + 15) & ~(size_t)15) +
           (size_t)TT * (TD + 1) * sizeof(typename io_elem<IO>::T);
}

// 8 consecutive activations at p (n of them valid, the rest zero) into LDS
// as they are, one 16-byte access when `vec` allows it
template <int IO>
__device__ __forceinline__ void mh_copy8(const typename io_elem<IO>::T *p, int n, bool vec,
                                         typename io_elem<IO>::T *dst) {
    using T = typename io_elem<IO>::T;
    if constexpr (sizeof(T) == 2) {
        if (vec && n >= 8) {
            const uint4 u = *(const uint4 *)p;
            const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint16_t lo = (uint16_t)(w4[e] & 0xffffu), hi = (uint16_t)(w4[e] >> 16);
                dst[2 * e] = __builtin_bit_cast(T, lo);
                dst[2 * e + 1] = __builtin_bit_cast(T, hi);
            }
            return;
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = e < n ? p[e] : T{};
}

template <int IO, class MT>
__global__ __launch_bounds__(256) void k_h3mh_gate_in(const typename io_elem<IO>::T *__restrict__ k,
                                                     const typename io_elem<IO>::T *__restrict__ v,
                                                     const float *__restrict__ w, MT *__restrict__ mT, int N,
                                                     int Dm, int dh, int L, int vec) {
    using T = typename io_elem<IO>::T;
    const int TT = mh_tt<MT>(dh);
    const int TD = mh_td(dh);  // model channels of the tile (whole heads)
    const int P = TD + 1;
    extern __shared__ __attribute__((aligned(16))) unsigned char mh_lds[];
    T *ks = (T *)mh_lds;         // [TT + 3][P]: k at steps t0 - 3 .. t0 + TT - 1
    T *vs = ks + (TT + 3) * P;   // [TT][P]: v
    const int tid = threadIdx.x;
    const int d0 = blockIdx.x * TD, t0 = blockIdx.y * TT, b = blockIdx.z;
    const size_t base = (size_t)b * N * Dm;
    // 8 channels per access (k with the shift's history of 3 steps)
    const int CR = TD / 8;
    for (int e = tid; e < (TT + 3) * CR; e += 256) {
        const int r = e / CR, c = 8 * (e % CR), t = t0 - 3 + r, d = d0 + c;
        if (t >= 0 && t < N && d < Dm) mh_copy8<IO>(k + base + (size_t)t * Dm + d, Dm - d, vec, ks + r * P + c);
        else for (int q = 0; q < 8; ++q) ks[r * P + c + q] = T{};
    }
    for (int e = tid; e < TT * CR; e += 256) {
        const int r = e / CR, c = 8 * (e % CR), t = t0 + r, d = d0 + c;
        if (t < N && d < Dm) mh_copy8<IO>(v + base + (size_t)t * Dm + d, Dm - d, vec, vs + r * P + c);
        else for (int q = 0; q < 8; ++q) vs[r * P + c + q] = T{};
    }
    __syncthreads();
    // items: (key channel kc, chunk of 8 steps): shift(k) once for the 8
    // steps, then the dh state rows kc dh + j, one 16-byte store each (bf16,
    // or two of fp32); 8 consecutive items fill one line of a row
    for (int e = tid; e < TD * (TT / 8); e += 256) {
        const int kc = e / (TT / 8), ck = e % (TT / 8), d = d0 + kc;
        if (d >= Dm) continue;
        float sh[8];
        float wt[4];
#pragma unroll
        for (int l = 0; l < 4; ++l) wt[l] = l < L ? w[(size_t)d * L + l] : 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int tl = 8 * ck + q;
            float a = 0.f;
#pragma unroll
            for (int l = 0; l < 4; ++l) a = fmaf(wt[l], ld_io<IO>(ks + (tl + 3 - l) * P + kc), a);
            sh[q] = a;
        }
        const int h0 = (kc / dh) * dh;
        const int nt = N - (t0 + 8 * ck);
        for (int j = 0; j < dh; ++j) {
            MT o[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) o[q] = mh_put<MT>(sh[q] * ld_io<IO>(vs + (8 * ck + q) * P + h0 + j));
            MT *row = mT + ((size_t)b * Dm * dh + (size_t)(d0 + kc) * dh + j) * N + t0 + 8 * ck;
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
}

template <int IO, class MT>
__global__ __launch_bounds__(256) void k_h3mh_gate_out(const typename io_elem<IO>::T *__restrict__ q,
                                                      const MT *__restrict__ zT,
                                                      typename io_elem<IO>::T *__restrict__ out, int N, int Dm,
                                                      int dh, int vec) {
    using T = typename io_elem<IO>::T;
    const int TT = mh_tt<MT>(dh);
    const int PZ = TT + 2;  // (even, so a row of 16-bit values stays 4-byte aligned)
    const int TD = mh_td(dh), ROWS = TD * dh;
    const int PQ = TD + 1;
    extern __shared__ __attribute__((aligned(16))) unsigned char mh_lds[];
    MT *zs = (MT *)mh_lds;  // [ROWS][PZ], as stored (bf16 bits or fp32)
    T *qs = (T *)(mh_lds + (((size_t)ROWS * PZ * sizeof(MT) + 15) & ~(size_t)15));  // [TT][PQ]
    const int tid = threadIdx.x;
    const int d0 = blockIdx.x * TD, t0 = blockIdx.y * TT, b = blockIdx.z;
    const size_t base = (size_t)b * N * Dm;
    // z rows of the tile, 8 steps per access (8 consecutive threads read one
    // line of a row)
    for (int e = tid; e < ROWS * (TT / 8); e += 256) {
        const int rl = e / (TT / 8), tl = 8 * (e % (TT / 8)), t = t0 + tl;
        const bool ok = t < N && d0 + rl / dh < Dm;
        const MT *src = zT + ((size_t)b * Dm * dh + (size_t)d0 * dh + rl) * N + t;
        MT *dst = zs + rl * PZ + tl;
        if (ok && vec && N - t >= 8) {
            if constexpr (sizeof(MT) == 2) {
                const uint4 u = *(const uint4 *)src;
                uint32_t *d4 = (uint32_t *)dst;
                d4[0] = u.x; d4[1] = u.y; d4[2] = u.z; d4[3] = u.w;
            } else {
                const float4 a = *(const float4 *)src, c = *(const float4 *)(src + 4);
                dst[0] = a.x; dst[1] = a.y; dst[2] = a.z; dst[3] = a.w;
                dst[4] = c.x; dst[5] = c.y; dst[6] = c.z; dst[7] = c.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) dst[i] = (ok && t + i < N) ? src[i] : (MT)0;
        }
    }
    const int CR = TD / 8;
    for (int e = tid; e < TT * CR; e += 256) {
        const int tl = e / CR, c = 8 * (e % CR), t = t0 + tl, d = d0 + c;
        if (t < N && d < Dm) mh_copy8<IO>(q + base + (size_t)t * Dm + d, Dm - d, vec, qs + tl * PQ + c);
        else for (int i = 0; i < 8; ++i) qs[tl * PQ + c + i] = T{};
    }
    __syncthreads();
    // outputs: (step, 8 consecutive channels), one 16-byte store (16-bit)
    for (int e = tid; e < TT * CR; e += 256) {
        const int tl = e / CR, c0 = 8 * (e % CR), t = t0 + tl, d = d0 + c0;
        if (t >= N || d >= Dm) continue;
        float o[8];
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
            const int c = c0 + cc, h0 = (c / dh) * dh, j = c % dh;
            float acc = 0.f;
            for (int i = 0; i < dh; ++i)
                acc = fmaf(ld_io<IO>(qs + tl * PQ + h0 + i), mh_get<MT>(zs[((h0 + i) * dh + j) * PZ + tl]), acc);
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
    const int TD = mh_td(dh), TT = mh_tt<MT>(dh);
    const dim3 grid((Dm + TD - 1) / TD, (N + TT - 1) / TT, B);
    // 16-byte accesses along the contiguous dimension when sizes and
    // pointers allow (else element by element)
    const uintptr_t al = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)ws;
    const int vec = (N % 8 == 0 && Dm % 8 == 0 && (al & 15) == 0 && (one & 15) == 0) ? 1 : 0;
    hipError_t e = launch(k_h3mh_gate_in<IO, MT>, grid, dim3(256), mh_in_lds<IO, MT>(dh), s, (const T *)k, (const T *)v, w,
                          mT, N, Dm, dh, L, vec);
    if (e != hipSuccess) return e;
    // the convolution over the B x (Dm dh) state rows, one filter per row
    e = launch_fft_conv(mT, f, D, zT, B, Dm * dh, N, sizeof(MT) == 4 ? IO_F32 : IO_BF16, s);
    if (e != hipSuccess) return e;
    return launch(k_h3mh_gate_out<IO, MT>, grid, dim3(256), mh_out_lds<IO, MT>(dh), s, (const T *)q, (const MT *)zT,
                  (T *)out, N, Dm, dh, vec);
}

hipError_t launch_h3_mix_mh(const void *q, const void *k, const void *v, const float *w, const float *f,
                            const float *D, void *out, int B, int N, int Dm, int dh, int L, int io, void *ws,
                            hipStream_t s) {
    // head dimension 1 is the H3 mix itself (its workspace is this one's)
    if (dh == 1) return launch_h3_mix(q, k, v, w, f, D, out, B, N, Dm, L, io, ws, s);
    switch (io) {
        case IO_F32: return mh_run<IO_F32, float>(q, k, v, w, f, D, out, B, N, Dm, dh, L, ws, s);
        case IO_F16: return mh_run<IO_F16, uint16_t>(q, k, v, w, f, D, out, B, N, Dm, dh, L, ws, s);
        case IO_BF16: return mh_run<IO_BF16, uint16_t>(q, k, v, w, f, D, out, B, N, Dm, dh, L, ws, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace h3c
