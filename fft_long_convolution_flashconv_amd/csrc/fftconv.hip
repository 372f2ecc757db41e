// fftconv.hip -- fused FFT long convolution kernels (fp32 VALU engine) for
// h3conv_fft_conv and h3conv_h3_mix.
//
// One workgroup owns one channel.  It first transforms the channel's filter
// (with the residual weight D folded into tap 0, since D*u is the convolution
// of u with D*delta) and keeps the spectrum in registers; it then walks over
// the batch two rows at a time, packing row 2s into the real part and row
// 2s+1 into the imaginary part of one complex signal.  Because the filter is
// real, the inverse transform of (spectrum of the pair) x (filter spectrum)
// returns the two convolutions in the real and imaginary parts, so one
// complex transform pair serves two rows.
//
// Method: paperlayer.ai summary of "Hungry Hungry Hippos", section 2
// "Convolutional view" (FFT, pointwise product, inverse FFT), section 4
// ("fuses FFT, pointwise multiplication, and inverse FFT"), Appendix C.1
// (zero-pad to 2L, keep the first N).
#include "h3conv_device.h"
#include "h3conv_internal.h"
#include "mfma_engine.h"

namespace h3c {

int fused_log2m(int64_t N) {
    int l = 5;  // Np >= 32
    while ((int64_t(1) << l) < N) ++l;
    return l + 1;
}

template <int LOG2M, int IO>
__global__ __launch_bounds__(Plan<LOG2M>::NT) void k_fft_conv(
    const typename io_elem<IO>::T *__restrict__ u, const float *__restrict__ f,
    const float *__restrict__ D, typename io_elem<IO>::T *__restrict__ y, int B, int H, int N) {
    using T = typename io_elem<IO>::T;
    __shared__ cf lds[Plan<LOG2M>::LDS_ELEMS];
    const int tid = threadIdx.x;
    const int h = blockIdx.x;
    const float *fh = f + (size_t)h * N;
    const float dh = D[h];

    FiltReg<LOG2M> F;
    auto ldf = [&](int pos) -> cf {
        float v = (pos < N) ? fh[pos] : 0.f;
        if (pos == 0) v += dh;
        return mk(v, 0.f);
    };
    filter_spectrum<LOG2M>(lds, tid, ldf, F);

    const int nsig = (B + 1) / 2;
    for (int s = 0; s < nsig; ++s) {
        const int b0 = 2 * s;
        const bool has1 = (b0 + 1) < B;
        const T *u0 = u + ((size_t)b0 * H + h) * N;
        const T *u1 = u0 + (size_t)H * N;
        T *y0 = y + ((size_t)b0 * H + h) * N;
        T *y1 = y0 + (size_t)H * N;
        auto ld = [&](int pos) -> cf {
            if (pos >= N) return mk(0.f, 0.f);
            return mk(ld_io<IO>(u0 + pos), has1 ? ld_io<IO>(u1 + pos) : 0.f);
        };
        auto st = [&](int pos, cf v) {
            if (pos < N) {
                st_io<IO>(y0 + pos, v.x);
                if (has1) st_io<IO>(y1 + pos, v.y);
            }
        };
        conv_signal<LOG2M>(lds, tid, F, ld, st);
    }
}

// H3 mix (head dimension 1), channel-last [B,N,Dm]: the loader forms
// m_t = (sum_{i<L} w_i k_{t-i}) * v_t, the store applies out_t = q_t * z_t.
template <int LOG2M, int IO>
__global__ __launch_bounds__(Plan<LOG2M>::NT) void k_h3_mix(
    const typename io_elem<IO>::T *__restrict__ q, const typename io_elem<IO>::T *__restrict__ k,
    const typename io_elem<IO>::T *__restrict__ v, const float *__restrict__ w,
    const float *__restrict__ f, const float *__restrict__ D, typename io_elem<IO>::T *__restrict__ out,
    int B, int N, int Dm, int L) {
    using T = typename io_elem<IO>::T;
    __shared__ cf lds[Plan<LOG2M>::LDS_ELEMS];
    const int tid = threadIdx.x;
    const int d = blockIdx.x;
    const float *fd = f + (size_t)d * N;
    const float dd = D[d];
    float wd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wd[i] = (i < L) ? w[(size_t)d * L + i] : 0.f;

    FiltReg<LOG2M> F;
    auto ldf = [&](int pos) -> cf {
        float x = (pos < N) ? fd[pos] : 0.f;
        if (pos == 0) x += dd;
        return mk(x, 0.f);
    };
    filter_spectrum<LOG2M>(lds, tid, ldf, F);

    const size_t rowstride = (size_t)N * Dm;
    const int nsig = (B + 1) / 2;
    for (int s = 0; s < nsig; ++s) {
        const int b0 = 2 * s;
        const bool has1 = (b0 + 1) < B;
        const size_t o0 = (size_t)b0 * rowstride + d;
        const size_t o1 = o0 + rowstride;
        auto mval = [&](size_t o, int t) -> float {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (i < L && i <= t) acc = fmaf(wd[i], ld_io<IO>(k + o + (size_t)(t - i) * Dm), acc);
            return acc * ld_io<IO>(v + o + (size_t)t * Dm);
        };
        auto ld = [&](int t) -> cf {
            if (t >= N) return mk(0.f, 0.f);
            return mk(mval(o0, t), has1 ? mval(o1, t) : 0.f);
        };
        auto st = [&](int t, cf z) {
            if (t < N) {
                const size_t a0 = o0 + (size_t)t * Dm;
                st_io<IO>(out + a0, ld_io<IO>(q + a0) * z.x);
                if (has1) {
                    const size_t a1 = o1 + (size_t)t * Dm;
                    st_io<IO>(out + a1, ld_io<IO>(q + a1) * z.y);
                }
            }
        };
        conv_signal<LOG2M>(lds, tid, F, ld, st);
    }
}


// ---------------------------------------------------------------- MFMA block-FFT variants
// fp16 / bf16 activations, 2N >= 256: same per-channel structure, transforms on
// the matrix cores (see mfma_engine.h).

template <int LOG2M, int IO>
__global__ __launch_bounds__(mf::Shape<LOG2M>::NT) __attribute__((amdgpu_waves_per_eu(mf::Shape<LOG2M>::WPE))) void k_fft_conv_mfma(
    const typename io_elem<IO>::T *__restrict__ u, const float *__restrict__ f,
    const float *__restrict__ D, typename io_elem<IO>::T *__restrict__ y, int B, int H, int N) {
    using T = typename io_elem<IO>::T;
    using SH = mf::Shape<LOG2M>;
    constexpr int KIND = IO == IO_F16 ? mf::IN_F16 : mf::IN_BF16;
    __shared__ __attribute__((aligned(16))) uint32_t smem[SH::LDS_DWORDS];
    mf::Engine<LOG2M, KIND> E(smem);
    E.init();
    const int h = blockIdx.x;
    const float *fh = f + (size_t)h * N;
    const float dh = D[h];
    // bytes between batch rows; every row offset of a launch fits 32 bits
    // (the launcher splits larger batches), so a row's address is one 32-bit
    // product and one 64-bit add
    const uint32_t rsb = mf::opaque_u32(2u * (uint32_t)H * (uint32_t)N);
    const char *uh = (const char *)(u + (size_t)h * N);
    char *yh = (char *)(y + (size_t)h * N);
    const int hb = mf::half_bits(N);
    // complex signal `sig` = batch rows 2 sig (real part), 2 sig + 1
    // (imaginary); rows past B get empty resources
    auto rows = [&](int sig) -> mf::RowBufs {
        const uint32_t o = (uint32_t)(2 * sig) * rsb;
        const int nb0 = (2 * sig < B) ? 2 * N : 0;
        const int nb1 = (2 * sig + 1 < B) ? 2 * N : 0;
        return {mf::row_rsrc(uh + o, nb0), mf::row_rsrc(uh + o + rsb, nb1), mf::row_rsrc(yh + o, nb0),
                mf::row_rsrc(yh + o + rsb, nb1)};
    };
    E.run_raw(mf::row_rsrc(fh, 4 * N), dh, rows, (B + 1) / 2, hb);
}

template <int LOG2M, int IO>
static hipError_t launch_fc_mfma(const void *u, const float *f, const float *D, void *y, int B,
                                 int H, int N, hipStream_t s) {
    using T = typename io_elem<IO>::T;
    // Row byte offsets inside one launch are 32-bit, including the empty rows
    // a last partial round addresses (up to 2 SIG + 2 past the batch): larger
    // batches go in slices of an even number of rows.
    const uint64_t rowb = 2ull * (uint64_t)H * (uint64_t)N;
    const uint64_t pad = 2 * mf::Shape<LOG2M>::SIG + 2;
    if ((pad + 2) * rowb >= (1ull << 32)) return hipErrorInvalidValue;
    const int bmax = (int)std::min<uint64_t>((uint64_t)B, (((1ull << 32) - 1) / rowb - pad) & ~1ull);
    for (int b0 = 0; b0 < B; b0 += bmax) {
        const size_t o = (size_t)b0 * H * N;
        hipLaunchKernelGGL((k_fft_conv_mfma<LOG2M, IO>), dim3(H), dim3(mf::Shape<LOG2M>::NT), 0, s,
                           (const T *)u + o, f, D, (T *)y + o, std::min(bmax, B - b0), H, N);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int LOG2M, int IO>
static hipError_t launch_fc(const void *u, const float *f, const float *D, void *y, int B, int H,
                            int N, hipStream_t s) {
    using T = typename io_elem<IO>::T;
    hipLaunchKernelGGL((k_fft_conv<LOG2M, IO>), dim3(H), dim3(Plan<LOG2M>::NT), 0, s,
                       (const T *)u, f, D, (T *)y, B, H, N);
    return hipGetLastError();
}

template <int IO>
static hipError_t fc_dispatch(int log2m, const void *u, const float *f, const float *D, void *y,
                              int B, int H, int N, hipStream_t s) {
    if constexpr (IO != IO_F32) {
        switch (log2m) {
            case 9: return launch_fc_mfma<9, IO>(u, f, D, y, B, H, N, s);
            case 10: return launch_fc_mfma<10, IO>(u, f, D, y, B, H, N, s);
            case 11: return launch_fc_mfma<11, IO>(u, f, D, y, B, H, N, s);
            case 12: return launch_fc_mfma<12, IO>(u, f, D, y, B, H, N, s);
            case 13: return launch_fc_mfma<13, IO>(u, f, D, y, B, H, N, s);
            case 14: return launch_fc_mfma<14, IO>(u, f, D, y, B, H, N, s);
            default: break;
        }
    }
    switch (log2m) {
        case 6: return launch_fc<6, IO>(u, f, D, y, B, H, N, s);
        case 7: return launch_fc<7, IO>(u, f, D, y, B, H, N, s);
        case 8: return launch_fc<8, IO>(u, f, D, y, B, H, N, s);
        case 9: return launch_fc<9, IO>(u, f, D, y, B, H, N, s);
        case 10: return launch_fc<10, IO>(u, f, D, y, B, H, N, s);
        case 11: return launch_fc<11, IO>(u, f, D, y, B, H, N, s);
        case 12: return launch_fc<12, IO>(u, f, D, y, B, H, N, s);
        case 13: return launch_fc<13, IO>(u, f, D, y, B, H, N, s);
        case 14: return launch_fc<14, IO>(u, f, D, y, B, H, N, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fft_conv(const void *u, const float *f, const float *D, void *y, int B, int H,
                           int N, int io, hipStream_t s) {
    const int l = fused_log2m(N);
    switch (io) {
        case IO_F32: return fc_dispatch<IO_F32>(l, u, f, D, y, B, H, N, s);
        case IO_F16: return fc_dispatch<IO_F16>(l, u, f, D, y, B, H, N, s);
        case IO_BF16: return fc_dispatch<IO_BF16>(l, u, f, D, y, B, H, N, s);
        default: return hipErrorInvalidValue;
    }
}

template <int LOG2M, int IO>
static hipError_t launch_hm(const void *q, const void *k, const void *v, const float *w,
                            const float *f, const float *D, void *out, int B, int N, int Dm, int L,
                            hipStream_t s) {
    using T = typename io_elem<IO>::T;
    hipLaunchKernelGGL((k_h3_mix<LOG2M, IO>), dim3(Dm), dim3(Plan<LOG2M>::NT), 0, s, (const T *)q,
                       (const T *)k, (const T *)v, w, f, D, (T *)out, B, N, Dm, L);
    return hipGetLastError();
}

template <int IO>
static hipError_t hm_dispatch(int log2m, const void *q, const void *k, const void *v,
                              const float *w, const float *f, const float *D, void *out, int B,
                              int N, int Dm, int L, hipStream_t s) {
    switch (log2m) {
        case 6: return launch_hm<6, IO>(q, k, v, w, f, D, out, B, N, Dm, L, s);
        case 7: return launch_hm<7, IO>(q, k, v, w, f, D, out, B, N, Dm, L, s);
        case 8: return launch_hm<8, IO>(q, k, v, w, f, D, out, B, N, Dm, L, s);
        case 9: return launch_hm<9, IO>(q, k, v, w, f, D, out, B, N, Dm, L, s);
        case 10: return launch_hm<10, IO>(q, k, v, w, f, D, out, B, N, Dm, L, s);
        case 11: return launch_hm<11, IO>(q, k, v, w, f, D, out, B, N, Dm, L, s);
        case 12: return launch_hm<12, IO>(q, k, v, w, f, D, out, B, N, Dm, L, s);
        case 13: return launch_hm<13, IO>(q, k, v, w, f, D, out, B, N, Dm, L, s);
        case 14: return launch_hm<14, IO>(q, k, v, w, f, D, out, B, N, Dm, L, s);
        default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------- H3 mix, 16-bit activations
// Channel-last activations [B, N, Dm] are transposed to channel-major rows on
// the way in and back on the way out, so the long convolution runs on
// contiguous rows in the matrix-core block-FFT engine:
//   gate-in  m_T[b, d, t] = v[b, t, d] * sum_{i < L, i <= t} w[d, i] k[b, t - i, d]
//   conv     z_T = (f_d * m_T)[:N] + D[d] m_T                  (fft conv, in ws)
//   gate-out out[b, t, d] = q[b, t, d] * z_T[b, d, t]
// The intermediates are bf16 (fp32 range, so no product can overflow them).
// A block covers 64 channels x 64 steps of one batch row; thread (d, tg)
// owns 16 consecutive steps of one channel, so channel-last accesses are
// coalesced across the 64 channels of a wave and channel-major ones are
// 32 contiguous bytes per thread.
constexpr int HM_TD = 64, HM_TT = 64, HM_TR = 16;

template <int IO>
__global__ __launch_bounds__(256) void k_h3_gate_in(const typename io_elem<IO>::T *__restrict__ k,
                                                   const typename io_elem<IO>::T *__restrict__ v,
                                                   const float *__restrict__ w, uint16_t *__restrict__ mT,
                                                   int N, int Dm, int L) {
    const int d = blockIdx.y * HM_TD + (threadIdx.x & 63);
    const int t0 = blockIdx.x * HM_TT + (threadIdx.x >> 6) * HM_TR;
    const int b = blockIdx.z;
    if (d >= Dm || t0 >= N) return;
    float wd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wd[i] = (i < L) ? w[(size_t)d * L + i] : 0.f;
    const size_t base = (size_t)b * N * Dm + d;
    float kk[HM_TR + 3];
#pragma unroll
    for (int r = 0; r < HM_TR + 3; ++r) {
        const int t = t0 + r - 3;
        kk[r] = (t >= 0 && t < N) ? ld_io<IO>(k + base + (size_t)t * Dm) : 0.f;
    }
    uint16_t mo[HM_TR];
#pragma unroll
    for (int r = 0; r < HM_TR; ++r) {
        const int t = t0 + r;
        float m = 0.f;
        if (t < N) {
            const float sh = fmaf(wd[0], kk[r + 3], fmaf(wd[1], kk[r + 2], fmaf(wd[2], kk[r + 1], wd[3] * kk[r])));
            m = sh * ld_io<IO>(v + base + (size_t)t * Dm);
        }
        mo[r] = __builtin_bit_cast(uint16_t, (__bf16)m);
    }
    uint16_t *dst = mT + ((size_t)b * Dm + d) * N + t0;
    if (t0 + HM_TR <= N && (N & 7) == 0) {
        mf::u32x4 lo, hi;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            lo[q] = (uint32_t)mo[2 * q] | ((uint32_t)mo[2 * q + 1] << 16);
            hi[q] = (uint32_t)mo[8 + 2 * q] | ((uint32_t)mo[8 + 2 * q + 1] << 16);
        }
        *(mf::u32x4 *)dst = lo;
        *(mf::u32x4 *)(dst + 8) = hi;
    } else {
#pragma unroll
        for (int r = 0; r < HM_TR; ++r)
            if (t0 + r < N) dst[r] = mo[r];
    }
}

template <int IO>
__global__ __launch_bounds__(256) void k_h3_gate_out(const typename io_elem<IO>::T *__restrict__ q,
                                                    const uint16_t *__restrict__ zT,
                                                    typename io_elem<IO>::T *__restrict__ out, int N, int Dm) {
    const int d = blockIdx.y * HM_TD + (threadIdx.x & 63);
    const int t0 = blockIdx.x * HM_TT + (threadIdx.x >> 6) * HM_TR;
    const int b = blockIdx.z;
    if (d >= Dm || t0 >= N) return;
    const uint16_t *src = zT + ((size_t)b * Dm + d) * N + t0;
    float z[HM_TR];
    if (t0 + HM_TR <= N && (N & 7) == 0) {
        const mf::u32x4 lo = *(const mf::u32x4 *)src, hi = *(const mf::u32x4 *)(src + 8);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t a = lo[c], e = hi[c];
            z[2 * c] = __uint_as_float(a << 16);
            z[2 * c + 1] = __uint_as_float(a & 0xffff0000u);
            z[8 + 2 * c] = __uint_as_float(e << 16);
            z[8 + 2 * c + 1] = __uint_as_float(e & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int r = 0; r < HM_TR; ++r) z[r] = (t0 + r < N) ? __uint_as_float((uint32_t)src[r] << 16) : 0.f;
    }
    const size_t base = (size_t)b * N * Dm + d;
#pragma unroll
    for (int r = 0; r < HM_TR; ++r) {
        const int t = t0 + r;
        if (t < N) {
            const size_t o = base + (size_t)t * Dm;
            st_io<IO>(out + o, ld_io<IO>(q + o) * z[r]);
        }
    }
}

size_t h3_mix_workspace(int64_t B, int64_t N, int64_t Dm) {
    const size_t one = ((size_t)(B * N * Dm) * 2 + 255) & ~(size_t)255;
    return 2 * one;
}

template <int IO>
static hipError_t hm_16bit(const void *q, const void *k, const void *v, const float *w, const float *f,
                           const float *D, void *out, int B, int N, int Dm, int L, void *ws, hipStream_t s) {
    using T = typename io_elem<IO>::T;
    const size_t one = h3_mix_workspace(B, N, Dm) / 2;
    uint16_t *mT = (uint16_t *)ws;
    uint16_t *zT = (uint16_t *)((char *)ws + one);
    const dim3 grid((N + HM_TT - 1) / HM_TT, (Dm + HM_TD - 1) / HM_TD, B);
    hipLaunchKernelGGL((k_h3_gate_in<IO>), grid, dim3(256), 0, s, (const T *)k, (const T *)v, w, mT, N, Dm, L);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = fc_dispatch<IO_BF16>(fused_log2m(N), mT, f, D, zT, B, Dm, N, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_h3_gate_out<IO>), grid, dim3(256), 0, s, (const T *)q, (const uint16_t *)zT, (T *)out,
                       N, Dm);
    return hipGetLastError();
}

hipError_t launch_h3_mix(const void *q, const void *k, const void *v, const float *w,
                         const float *f, const float *D, void *out, int B, int N, int Dm, int L,
                         int io, void *ws, hipStream_t s) {
    switch (io) {
        case IO_F32: return hm_dispatch<IO_F32>(fused_log2m(N), q, k, v, w, f, D, out, B, N, Dm, L, s);
        case IO_F16: return hm_16bit<IO_F16>(q, k, v, w, f, D, out, B, N, Dm, L, ws, s);
        case IO_BF16: return hm_16bit<IO_BF16>(q, k, v, w, f, D, out, B, N, Dm, L, ws, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace h3c
