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

// CORR: correlation with the filter instead of convolution (the conjugated
// filter spectrum; the backward pass's du).
template <int LOG2M, int IO, bool CORR>
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
    if constexpr (CORR) {
#pragma unroll
        for (int i = 0; i < FiltReg<LOG2M>::NBT; ++i)
#pragma unroll
            for (int k = 0; k < FiltReg<LOG2M>::R; ++k) F.v[i][k].y = -F.v[i][k].y;
    }

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


// Backward pass of the causal convolution with residual (the paperlayer.ai
// summary of "Hungry Hungry Hippos", Appendix C.1: the gradients of u, f and
// D are correlations computed through the same zero-padded transforms, D dy
// entering du):
//   du[b] = IDFT(DY_b conj(F))[:N] with F = DFT(f + D delta): the correlation
//           of dy with the filter, D dy included by tap 0;
//   df    = Re IDFT(sum_pairs conj(Z_u) Z_dy)[:N], Z = row 2s + i row 2s+1:
//           the real part of the correlation of the complex pair signals is
//           the sum of the two rows' correlations of u with dy (the spectrum
//           summed over the batch and inverted once);
//   dD    = df[0] (the gradient of tap 0, which D shares).
// The zero padding to 2N keeps every correlation lag in [0, N) free of wrap.
// Kernels: 16-bit activations at 2N = 512, 1024, 2048 run all three in one
// (k_fft_bwd_mfma); at 2N = 4096, 8192, 16384 du runs as the convolution
// kernel with the conjugated filter spectrum (CORR) and df, dD as
// k_fft_df_mfma;
// fp32 activations and the remaining sizes take CORR and k_fft_corr_df
// below (one workgroup per channel, fp32 transforms).
template <int LOG2M, int IO>
__global__ __launch_bounds__(Plan<LOG2M>::NT) void k_fft_corr_df(
    const typename io_elem<IO>::T *__restrict__ u, const typename io_elem<IO>::T *__restrict__ dy,
    float *__restrict__ df, float *__restrict__ dD, int B, int H, int N) {
    using T = typename io_elem<IO>::T;
    using FR = FiltReg<LOG2M>;
    __shared__ cf lds[Plan<LOG2M>::LDS_ELEMS];
    const int tid = threadIdx.x;
    const int h = blockIdx.x;
    FR acc;
#pragma unroll
    for (int i = 0; i < FR::NBT; ++i)
#pragma unroll
        for (int k = 0; k < FR::R; ++k) acc.v[i][k] = mk(0.f, 0.f);
    const int nsig = (B + 1) / 2;
    for (int s = 0; s < nsig; ++s) {
        const int b0 = 2 * s;
        const bool has1 = (b0 + 1) < B;
        const size_t o0 = ((size_t)b0 * H + h) * N, o1 = o0 + (size_t)H * N;
        auto ldp = [&](const T *x) {
            return [=](int pos) -> cf {
                if (pos >= N) return mk(0.f, 0.f);
                return mk(ld_io<IO>(x + o0 + pos), has1 ? ld_io<IO>(x + o1 + pos) : 0.f);
            };
        };
        FR Sd, Su;
        spectrum<LOG2M>(lds, tid, ldp(dy), Sd, 1.f);
        spectrum<LOG2M>(lds, tid, ldp(u), Su, 1.f);
#pragma unroll
        for (int i = 0; i < FR::NBT; ++i)
#pragma unroll
            for (int k = 0; k < FR::R; ++k) {
                const cf a = Su.v[i][k], d = Sd.v[i][k];  // += conj(a) d
                acc.v[i][k] = cadd(acc.v[i][k], mk(fmaf(a.x, d.x, a.y * d.y), fmaf(a.x, d.y, -a.y * d.x)));
            }
    }
    constexpr float SC = 1.0f / (float)Plan<LOG2M>::M;
#pragma unroll
    for (int i = 0; i < FR::NBT; ++i)
#pragma unroll
        for (int k = 0; k < FR::R; ++k) acc.v[i][k] = cscale(acc.v[i][k], SC);
    inverse_regs<LOG2M>(lds, tid, acc, [&](int pos, cf v) {
        if (pos < N) {
            df[(size_t)h * N + pos] = v.x;
            if (pos == 0) dD[h] = v.x;
        }
    });
}

template <int LOG2M, int IO>
static hipError_t launch_df(const void *u, const void *dy, float *df, float *dD, int B, int H, int N,
                            hipStream_t s) {
    using T = typename io_elem<IO>::T;
    return launch(k_fft_corr_df<LOG2M, IO>, dim3(H), dim3(Plan<LOG2M>::NT), 0, s, (const T *)u, (const T *)dy, df,
                  dD, B, H, N);
}

// The same gradient on the matrix-core engine for 16-bit activations (2N =
// 4096, 8192; smaller sizes take the fused backward kernel): see
// Engine::run_df.  One workgroup per channel; rounds alternate
// between SIG row pairs of u and the same pairs of dy.  Rows are addressed
// with 64-bit offsets, so no batch is split (the sum runs over all of it).
// Waves per SIMD the gradient kernel's registers are set for: it holds a
// round of last-pass values and the fp32 sum besides the transform's own,
// so it runs fewer workgroups per compute unit than the convolution.
template <int LOG2M> struct DfOcc { static constexpr int WPE = 4; };
// 2N = 512: a two-wave workgroup carries eight signals a round, so each lane
// holds twice the values of the larger sizes (166 registers, no spills at
// three waves per SIMD; 64 spilled at four)
template <> struct DfOcc<9> { static constexpr int WPE = 3; };
// 2N = 16384: the sum alone is 64 registers a lane; at two waves per SIMD
// (one workgroup per compute unit) the kernel holds 196 without spilling,
// where four waves per SIMD would spill 68
template <> struct DfOcc<14> { static constexpr int WPE = 2; };

template <int LOG2M, int IO>
__global__ __launch_bounds__(mf::Shape<LOG2M>::NT) __attribute__((amdgpu_waves_per_eu(DfOcc<LOG2M>::WPE))) void k_fft_df_mfma(
    const typename io_elem<IO>::T *__restrict__ u, const typename io_elem<IO>::T *__restrict__ dy,
    float *__restrict__ df, float *__restrict__ dD, int B, int H, int N) {
    using SH = mf::Shape<LOG2M>;
    constexpr int KIND = IO == IO_F16 ? mf::IN_F16 : mf::IN_BF16;
    constexpr int SIG = SH::SIG;
    __shared__ __attribute__((aligned(16))) uint32_t smem[SH::LDS_DWORDS];
    mf::Engine<LOG2M, KIND> E(smem);
    E.init();
    const int h = blockIdx.x;
    const size_t rowb = (size_t)H * (size_t)N * 2;
    const char *uh = (const char *)(u + (size_t)h * N);
    const char *dh = (const char *)(dy + (size_t)h * N);
    const int np = (B + 1) / 2;
    const int nround = 2 * ((np + SIG - 1) / SIG);
    // virtual signal v = round * SIG + s: pair (round / 2) * SIG + s of u
    // (even rounds) or dy (odd rounds); rows past B get empty resources
    auto rows = [&](int v) -> mf::RowBufs {
        const int r = v / SIG, p = (r >> 1) * SIG + v % SIG;
        const char *p0 = ((r & 1) ? dh : uh) + (size_t)(2 * p) * rowb;
        const int nb0 = (2 * p < B) ? 2 * N : 0;
        const int nb1 = (2 * p + 1 < B) ? 2 * N : 0;
        return {mf::row_rsrc(p0, nb0), mf::row_rsrc(p0 + rowb, nb1), mf::row_rsrc(p0, 0), mf::row_rsrc(p0, 0)};
    };
    const __amdgpu_buffer_rsrc_t drs = mf::row_rsrc(df + (size_t)h * N, 4 * N);
    float *dDh = dD + h;
    E.run_df(rows, nround, mf::half_bits(N), [&](int pos, float v) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), drs, 4 * pos, 0, 0);
        if (pos == 0) *dDh = v;
    });
}

// The whole backward pass in one kernel (Engine::run_bwd): du, df and dD
// from one read of u and dy.  One workgroup per channel; rounds alternate
// between SIG row pairs of dy (with du as output) and the same pairs of u.
template <int LOG2M, int IO>
__global__ __launch_bounds__(mf::Shape<LOG2M>::NT) __attribute__((amdgpu_waves_per_eu(DfOcc<LOG2M>::WPE))) void k_fft_bwd_mfma(
    const typename io_elem<IO>::T *__restrict__ u, const float *__restrict__ f, const float *__restrict__ D,
    const typename io_elem<IO>::T *__restrict__ dy, typename io_elem<IO>::T *__restrict__ du,
    float *__restrict__ df, float *__restrict__ dD, int B, int H, int N) {
    using SH = mf::Shape<LOG2M>;
    constexpr int KIND = IO == IO_F16 ? mf::IN_F16 : mf::IN_BF16;
    constexpr int SIG = SH::SIG;
    __shared__ __attribute__((aligned(16))) uint32_t smem[SH::LDS_DWORDS];
    mf::Engine<LOG2M, KIND> E(smem);
    E.init();
    const int h = blockIdx.x;
    const size_t rowb = (size_t)H * (size_t)N * 2;
    const char *uh = (const char *)(u + (size_t)h * N);
    const char *dyh = (const char *)(dy + (size_t)h * N);
    char *duh = (char *)(du + (size_t)h * N);
    const int np = (B + 1) / 2;
    const int nround = 2 * ((np + SIG - 1) / SIG);
    // virtual signal v = round * SIG + s: pair (round / 2) * SIG + s of dy
    // with du as output (even rounds) or of u (odd rounds); rows past B get
    // empty resources
    auto rows = [&](int v) -> mf::RowBufs {
        const int r = v / SIG, p = (r >> 1) * SIG + v % SIG;
        const size_t o = (size_t)(2 * p) * rowb;
        const int nb0 = (2 * p < B) ? 2 * N : 0;
        const int nb1 = (2 * p + 1 < B) ? 2 * N : 0;
        if (r & 1)
            return {mf::row_rsrc(uh + o, nb0), mf::row_rsrc(uh + o + rowb, nb1), mf::row_rsrc(uh, 0), mf::row_rsrc(uh, 0)};
        return {mf::row_rsrc(dyh + o, nb0), mf::row_rsrc(dyh + o + rowb, nb1), mf::row_rsrc(duh + o, nb0),
                mf::row_rsrc(duh + o + rowb, nb1)};
    };
    const __amdgpu_buffer_rsrc_t drs = mf::row_rsrc(df + (size_t)h * N, 4 * N);
    float *dDh = dD + h;
    E.template run_bwd<mf::kNT>(mf::row_rsrc(f + (size_t)h * N, 4 * N), D[h], rows, nround, mf::half_bits(N),
                                [&](int pos, float v) {
                                    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), drs, 4 * pos, 0, 0);
                                    if (pos == 0) *dDh = v;
                                });
}

template <int LOG2M, int IO>
static hipError_t launch_bwd_mfma(const void *u, const float *f, const float *D, const void *dy, void *du, float *df,
                                  float *dD, int B, int H, int N, hipStream_t s) {
    using T = typename io_elem<IO>::T;
    return launch(k_fft_bwd_mfma<LOG2M, IO>, dim3(H), dim3(mf::Shape<LOG2M>::NT), 0, s, (const T *)u, f, D,
                  (const T *)dy, (T *)du, df, dD, B, H, N);
}

template <int LOG2M, int IO>
static hipError_t launch_df_mfma(const void *u, const void *dy, float *df, float *dD, int B, int H, int N,
                                 hipStream_t s) {
    using T = typename io_elem<IO>::T;
    return launch(k_fft_df_mfma<LOG2M, IO>, dim3(H), dim3(mf::Shape<LOG2M>::NT), 0, s, (const T *)u, (const T *)dy,
                  df, dD, B, H, N);
}

template <int IO>
static hipError_t df_dispatch(int log2m, const void *u, const void *dy, float *df, float *dD, int B, int H, int N,
                              hipStream_t s) {
    if constexpr (IO != IO_F32) {
        // (2N = 512, 1024, 2048: the fused backward kernel)
        switch (log2m) {
            case 12: return launch_df_mfma<12, IO>(u, dy, df, dD, B, H, N, s);
            case 13: return launch_df_mfma<13, IO>(u, dy, df, dD, B, H, N, s);
            case 14: return launch_df_mfma<14, IO>(u, dy, df, dD, B, H, N, s);
            default: break;
        }
    }
    switch (log2m) {
        case 6: return launch_df<6, IO>(u, dy, df, dD, B, H, N, s);
        case 7: return launch_df<7, IO>(u, dy, df, dD, B, H, N, s);
        case 8: return launch_df<8, IO>(u, dy, df, dD, B, H, N, s);
        case 9: return launch_df<9, IO>(u, dy, df, dD, B, H, N, s);
        case 10: return launch_df<10, IO>(u, dy, df, dD, B, H, N, s);
        case 11: return launch_df<11, IO>(u, dy, df, dD, B, H, N, s);
        case 12: return launch_df<12, IO>(u, dy, df, dD, B, H, N, s);
        case 13: return launch_df<13, IO>(u, dy, df, dD, B, H, N, s);
        case 14: return launch_df<14, IO>(u, dy, df, dD, B, H, N, s);
        default: return hipErrorInvalidValue;
    }
}

// ---------------------------------------------------------------- MFMA block-FFT variants
// fp16 / bf16 activations, 2N >= 256: same per-channel structure, transforms on
// the matrix cores (see mfma_engine.h).

// SPOL: cache policy of the output stores (non-temporal unless the output
// is read again right away); V: the engine's shape variant (1: half the
// signals per round, for batches that fill at most half a round)
template <int LOG2M, int IO, int SPOL, bool CORR = false, int V = 0>
__global__ __launch_bounds__((mf::Shape<LOG2M, V>::NT)) __attribute__((amdgpu_waves_per_eu(mf::Shape<LOG2M, V>::WPE))) void k_fft_conv_mfma(
    const typename io_elem<IO>::T *__restrict__ u, const float *__restrict__ f,
    const float *__restrict__ D, typename io_elem<IO>::T *__restrict__ y, int B, int H, int N) {
    using T = typename io_elem<IO>::T;
    using SH = mf::Shape<LOG2M, V>;
    constexpr int KIND = IO == IO_F16 ? mf::IN_F16 : mf::IN_BF16;
    __shared__ __attribute__((aligned(16))) uint32_t smem[SH::LDS_DWORDS];
    mf::Engine<LOG2M, KIND, V> E(smem);
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
    E.template run_raw<SPOL, CORR>(mf::row_rsrc(fh, 4 * N), dh, rows, (B + 1) / 2, hb);
}

// Bidirectional copies of the layer (the paperlayer.ai summary, E.4 "LRA
// evaluation"): y = causal (f * u) + anti-causal (g * u) + D u, one
// transform per row pair with the spectrum F + conj(G) of the two-sided
// filter (g's taps sit at negative lags, which the zero padding to 2N keeps
// apart from f's).
template <int LOG2M, int IO>
__global__ __launch_bounds__(Plan<LOG2M>::NT) void k_fft_bidir(
    const typename io_elem<IO>::T *__restrict__ u, const float *__restrict__ f, const float *__restrict__ g,
    const float *__restrict__ D, typename io_elem<IO>::T *__restrict__ y, int B, int H, int N) {
    using T = typename io_elem<IO>::T;
    using FR = FiltReg<LOG2M>;
    __shared__ cf lds[Plan<LOG2M>::LDS_ELEMS];
    const int tid = threadIdx.x;
    const int h = blockIdx.x;
    const float *fh = f + (size_t)h * N, *gh = g + (size_t)h * N;
    const float dh = D[h];
    FR F, G;
    filter_spectrum<LOG2M>(lds, tid, [&](int pos) -> cf {
        float v = (pos < N) ? fh[pos] : 0.f;
        if (pos == 0) v += dh;
        return mk(v, 0.f);
    }, F);
    filter_spectrum<LOG2M>(lds, tid, [&](int pos) -> cf { return mk(pos < N ? gh[pos] : 0.f, 0.f); }, G);
#pragma unroll
    for (int i = 0; i < FR::NBT; ++i)
#pragma unroll
        for (int k = 0; k < FR::R; ++k) F.v[i][k] = mk(F.v[i][k].x + G.v[i][k].x, F.v[i][k].y - G.v[i][k].y);
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

template <int LOG2M, int IO>
__global__ __launch_bounds__(mf::Shape<LOG2M>::NT) __attribute__((amdgpu_waves_per_eu(mf::Shape<LOG2M>::WPE))) void k_fft_bidir_mfma(
    const typename io_elem<IO>::T *__restrict__ u, const float *__restrict__ f, const float *__restrict__ g,
    const float *__restrict__ D, typename io_elem<IO>::T *__restrict__ y, int B, int H, int N) {
    using SH = mf::Shape<LOG2M>;
    constexpr int KIND = IO == IO_F16 ? mf::IN_F16 : mf::IN_BF16;
    __shared__ __attribute__((aligned(16))) uint32_t smem[SH::LDS_DWORDS];
    mf::Engine<LOG2M, KIND> E(smem);
    E.init();
    const int h = blockIdx.x;
    const uint32_t rsb = mf::opaque_u32(2u * (uint32_t)H * (uint32_t)N);
    const char *uh = (const char *)(u + (size_t)h * N);
    char *yh = (char *)(y + (size_t)h * N);
    auto rows = [&](int sig) -> mf::RowBufs {
        const uint32_t o = (uint32_t)(2 * sig) * rsb;
        const int nb0 = (2 * sig < B) ? 2 * N : 0;
        const int nb1 = (2 * sig + 1 < B) ? 2 * N : 0;
        return {mf::row_rsrc(uh + o, nb0), mf::row_rsrc(uh + o + rsb, nb1), mf::row_rsrc(yh + o, nb0),
                mf::row_rsrc(yh + o + rsb, nb1)};
    };
    E.run_raw_bidir(mf::row_rsrc(f + (size_t)h * N, 4 * N), D[h], mf::row_rsrc(g + (size_t)h * N, 4 * N), rows,
                    (B + 1) / 2, mf::half_bits(N));
}

// Row byte offsets inside one launch of the 16-bit engine are 32-bit,
// including the empty rows a last partial round addresses (up to 2 SIG + 2
// past the batch): larger batches go in slices of an even number of rows,
// and a slice must hold at least two.
template <int LOG2M>
static constexpr uint64_t fc_row_pad() { return 2 * mf::Shape<LOG2M>::SIG + 2; }

static uint64_t fc_pad_for(int log2m) {
    switch (log2m) {
        case 9: return fc_row_pad<9>();
        case 10: return fc_row_pad<10>();
        case 11: return fc_row_pad<11>();
        case 12: return fc_row_pad<12>();
        case 13: return fc_row_pad<13>();
        case 14: return fc_row_pad<14>();
        case 15: return fc_row_pad<15>();
        default: return 0;  // fp32 engine: 64-bit offsets
    }
}

bool fft_conv_rows_fit(int64_t H, int64_t N, int io) {
    if (io == IO_F32 || H <= 0 || N <= 0) return true;
    const uint64_t pad = fc_pad_for(fused_log2m(N));
    if (pad == 0) return true;
    const uint64_t rowb = 2ull * (uint64_t)H * (uint64_t)N;
    return (pad + 2) * rowb < (1ull << 32);
}

template <int LOG2M, int IO, int SPOL, bool CORR>
static hipError_t launch_fc_mfma(const void *u, const float *f, const float *D, void *y, int B,
                                 int H, int N, hipStream_t s) {
    using T = typename io_elem<IO>::T;
    const uint64_t rowb = 2ull * (uint64_t)H * (uint64_t)N;
    const uint64_t pad = fc_row_pad<LOG2M>();
    if ((pad + 2) * rowb >= (1ull << 32)) return hipErrorInvalidValue;  // refused by the API first
    const int bmax = (int)std::min<uint64_t>((uint64_t)B, (((1ull << 32) - 1) / rowb - pad) & ~1ull);
    // batches of at most half a round's signals: the half shape (2N <= 4096)
    constexpr bool HALF = LOG2M <= 12;
    if (HALF && (B + 1) / 2 <= mf::Shape<LOG2M>::SIG / 2)
        return launch(k_fft_conv_mfma<LOG2M, IO, SPOL, CORR, HALF ? 1 : 0>, dim3(H), dim3(mf::Shape<LOG2M, HALF ? 1 : 0>::NT),
                      0, s, (const T *)u, f, D, (T *)y, B, H, N);
    for (int b0 = 0; b0 < B; b0 += bmax) {
        const size_t o = (size_t)b0 * H * N;
        const hipError_t e = launch(k_fft_conv_mfma<LOG2M, IO, SPOL, CORR>, dim3(H), dim3(mf::Shape<LOG2M>::NT), 0, s,
                                    (const T *)u + o, f, D, (T *)y + o, std::min(bmax, B - b0), H, N);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int LOG2M, int IO, bool CORR>
static hipError_t launch_fc(const void *u, const float *f, const float *D, void *y, int B, int H,
                            int N, hipStream_t s) {
    using T = typename io_elem<IO>::T;
    return launch(k_fft_conv<LOG2M, IO, CORR>, dim3(H), dim3(Plan<LOG2M>::NT), 0, s, (const T *)u, f, D, (T *)y,
                  B, H, N);
}

template <int IO, int SPOL = mf::kNT, bool CORR = false>
static hipError_t fc_dispatch(int log2m, const void *u, const float *f, const float *D, void *y,
                              int B, int H, int N, hipStream_t s) {
    if constexpr (IO != IO_F32) {
        switch (log2m) {
            case 9: return launch_fc_mfma<9, IO, SPOL, CORR>(u, f, D, y, B, H, N, s);
            case 10: return launch_fc_mfma<10, IO, SPOL, CORR>(u, f, D, y, B, H, N, s);
            case 11: return launch_fc_mfma<11, IO, SPOL, CORR>(u, f, D, y, B, H, N, s);
            case 12: return launch_fc_mfma<12, IO, SPOL, CORR>(u, f, D, y, B, H, N, s);
            case 13: return launch_fc_mfma<13, IO, SPOL, CORR>(u, f, D, y, B, H, N, s);
            case 14: return launch_fc_mfma<14, IO, SPOL, CORR>(u, f, D, y, B, H, N, s);
            case 15: return launch_fc_mfma<15, IO, SPOL, CORR>(u, f, D, y, B, H, N, s);
            default: break;
        }
    }
    switch (log2m) {
        case 6: return launch_fc<6, IO, CORR>(u, f, D, y, B, H, N, s);
        case 7: return launch_fc<7, IO, CORR>(u, f, D, y, B, H, N, s);
        case 8: return launch_fc<8, IO, CORR>(u, f, D, y, B, H, N, s);
        case 9: return launch_fc<9, IO, CORR>(u, f, D, y, B, H, N, s);
        case 10: return launch_fc<10, IO, CORR>(u, f, D, y, B, H, N, s);
        case 11: return launch_fc<11, IO, CORR>(u, f, D, y, B, H, N, s);
        case 12: return launch_fc<12, IO, CORR>(u, f, D, y, B, H, N, s);
        case 13: return launch_fc<13, IO, CORR>(u, f, D, y, B, H, N, s);
        case 14: return launch_fc<14, IO, CORR>(u, f, D, y, B, H, N, s);
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
static hipError_t launch_bidir(const void *u, const float *f, const float *g, const float *D, void *y, int B, int H,
                               int N, hipStream_t s) {
    using T = typename io_elem<IO>::T;
    if constexpr (IO != IO_F32 && LOG2M >= 9) {
        const uint64_t rowb = 2ull * (uint64_t)H * (uint64_t)N;
        const uint64_t pad = fc_row_pad<LOG2M>();
        if ((pad + 2) * rowb >= (1ull << 32)) return hipErrorInvalidValue;  // refused by the API first
        const int bmax = (int)std::min<uint64_t>((uint64_t)B, (((1ull << 32) - 1) / rowb - pad) & ~1ull);
        for (int b0 = 0; b0 < B; b0 += bmax) {
            const size_t o = (size_t)b0 * H * N;
            const hipError_t e = launch(k_fft_bidir_mfma<LOG2M, IO>, dim3(H), dim3(mf::Shape<LOG2M>::NT), 0, s,
                                        (const T *)u + o, f, g, D, (T *)y + o, std::min(bmax, B - b0), H, N);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    } else if constexpr (LOG2M <= 14) {
        return launch(k_fft_bidir<LOG2M, IO>, dim3(H), dim3(Plan<LOG2M>::NT), 0, s, (const T *)u, f, g, D, (T *)y, B,
                      H, N);
    } else {
        return hipErrorInvalidValue;  // fp32 activations: up to 2N = 16384 (refused by the API first)
    }
}

template <int IO>
static hipError_t bidir_dispatch(int log2m, const void *u, const float *f, const float *g, const float *D, void *y,
                                 int B, int H, int N, hipStream_t s) {
    switch (log2m) {
        case 6: return launch_bidir<6, IO>(u, f, g, D, y, B, H, N, s);
        case 7: return launch_bidir<7, IO>(u, f, g, D, y, B, H, N, s);
        case 8: return launch_bidir<8, IO>(u, f, g, D, y, B, H, N, s);
        case 9: return launch_bidir<9, IO>(u, f, g, D, y, B, H, N, s);
        case 10: return launch_bidir<10, IO>(u, f, g, D, y, B, H, N, s);
        case 11: return launch_bidir<11, IO>(u, f, g, D, y, B, H, N, s);
        case 12: return launch_bidir<12, IO>(u, f, g, D, y, B, H, N, s);
        case 13: return launch_bidir<13, IO>(u, f, g, D, y, B, H, N, s);
        case 14: return launch_bidir<14, IO>(u, f, g, D, y, B, H, N, s);
        case 15: return launch_bidir<15, IO>(u, f, g, D, y, B, H, N, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_fft_bidir(const void *u, const float *f, const float *g, const float *D, void *y, int B, int H,
                            int N, int io, hipStream_t s) {
    const int l = fused_log2m(N);
    switch (io) {
        case IO_F32: return bidir_dispatch<IO_F32>(l, u, f, g, D, y, B, H, N, s);
        case IO_F16: return bidir_dispatch<IO_F16>(l, u, f, g, D, y, B, H, N, s);
        case IO_BF16: return bidir_dispatch<IO_BF16>(l, u, f, g, D, y, B, H, N, s);
        default: return hipErrorInvalidValue;
    }
}

template <int IO>
static hipError_t bwd_fused(int log2m, const void *u, const float *f, const float *D, const void *dy, void *du,
                            float *df, float *dD, int B, int H, int N, hipStream_t s, bool *done) {
    *done = true;
    switch (log2m) {
        case 9: return launch_bwd_mfma<9, IO>(u, f, D, dy, du, df, dD, B, H, N, s);
        case 10: return launch_bwd_mfma<10, IO>(u, f, D, dy, du, df, dD, B, H, N, s);
        case 11: return launch_bwd_mfma<11, IO>(u, f, D, dy, du, df, dD, B, H, N, s);
        // (2N = 4096, 8192: the registers of the fused kernel would spill at
        //  two workgroups per compute unit; two kernels instead)
        default: *done = false; return hipSuccess;
    }
}

hipError_t launch_fft_conv_bwd(const void *u, const float *f, const float *D, const void *dy, void *du,
                               float *df, float *dD, int B, int H, int N, int io, hipStream_t s) {
    const int l = fused_log2m(N);
    hipError_t e;
    bool done = false;
    // 16-bit activations with 2N = 512, 1024, 2048: one kernel for all three
    // gradients; otherwise the correlation kernel for du, then df and dD
    if (io == IO_F16) e = bwd_fused<IO_F16>(l, u, f, D, dy, du, df, dD, B, H, N, s, &done);
    else if (io == IO_BF16) e = bwd_fused<IO_BF16>(l, u, f, D, dy, du, df, dD, B, H, N, s, &done);
    if (done) return e;
    switch (io) {
        case IO_F32:
            e = fc_dispatch<IO_F32, mf::kNT, true>(l, dy, f, D, du, B, H, N, s);
            return e != hipSuccess ? e : df_dispatch<IO_F32>(l, u, dy, df, dD, B, H, N, s);
        case IO_F16:
            e = fc_dispatch<IO_F16, mf::kNT, true>(l, dy, f, D, du, B, H, N, s);
            return e != hipSuccess ? e : df_dispatch<IO_F16>(l, u, dy, df, dD, B, H, N, s);
        case IO_BF16:
            e = fc_dispatch<IO_BF16, mf::kNT, true>(l, dy, f, D, du, B, H, N, s);
            return e != hipSuccess ? e : df_dispatch<IO_BF16>(l, u, dy, df, dD, B, H, N, s);
        default: return hipErrorInvalidValue;
    }
}

template <int LOG2M, int IO>
static hipError_t launch_hm(const void *q, const void *k, const void *v, const float *w,
                            const float *f, const float *D, void *out, int B, int N, int Dm, int L,
                            hipStream_t s) {
    using T = typename io_elem<IO>::T;
    return launch(k_h3_mix<LOG2M, IO>, dim3(Dm), dim3(Plan<LOG2M>::NT), 0, s, (const T *)q, (const T *)k,
                  (const T *)v, w, f, D, (T *)out, B, N, Dm, L);
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
// Both gates transpose a tile of HM_TT steps x HM_TD channels of one batch
// row through LDS, so every global access is 16 bytes per lane along the
// contiguous dimension; the channel tile is the fastest grid index, so the
// workgroups in flight together cover whole channel-last rows.  `vec` (set
// by the launcher when N, Dm and the pointers allow 16-byte accesses) picks
// the vector accesses; otherwise, and at ragged tile edges, they go element
// by element.
constexpr int HM_TT = 64, HM_TD = 128;

template <int IO>
__device__ __forceinline__ float hm_f(uint16_t x) {
    if constexpr (IO == IO_F16) return (float)__builtin_bit_cast(_Float16, x);
    else return __uint_as_float((uint32_t)x << 16);
}
template <int IO>
__device__ __forceinline__ uint16_t hm_h(float x) {
    if constexpr (IO == IO_F16) return __builtin_bit_cast(uint16_t, (_Float16)x);
    else return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// 8 consecutive 16-bit values at p (n of them valid), zero-filled
// NTA: non-temporal access.  The block's own inputs (q, k, v) and output
// are touched once, and non-temporal stores of the output leave no dirty L2
// lines behind; the bf16 intermediates m_T and z_T keep the default policy.
template <bool NTA>
__device__ __forceinline__ mf::u32x4 hm_load8(const uint16_t *p, int n, bool vec) {
    if (vec && n >= 8) {
        if constexpr (NTA) return __builtin_nontemporal_load((const mf::u32x4 *)p);
        else return *(const mf::u32x4 *)p;
    }
    uint16_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = i < n ? p[i] : (uint16_t)0;
    mf::u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (uint32_t)e[2 * i] | ((uint32_t)e[2 * i + 1] << 16);
    return r;
}
template <bool NTA>
__device__ __forceinline__ void hm_store8(uint16_t *p, int n, bool vec, const uint16_t (&e)[8]) {
    if (vec && n >= 8) {
        mf::u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = (uint32_t)e[2 * i] | ((uint32_t)e[2 * i + 1] << 16);
        if constexpr (NTA) __builtin_nontemporal_store(r, (mf::u32x4 *)p);
        else *(mf::u32x4 *)p = r;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < n) p[i] = e[i];
    }
}

template <int IO>
__global__ __launch_bounds__(256) void k_h3_gate_in(const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
                                                   const float *__restrict__ w, uint16_t *__restrict__ mT,
                                                   int N, int Dm, int L, int vec) {
    // LDS row stride (16-bit units): rows 4-byte aligned, and 8 rows apart
    // land 8 banks apart, so the reads below spread over the banks
    constexpr int PD = HM_TD + 2;
    __shared__ __attribute__((aligned(16))) uint16_t ks[(HM_TT + 3) * PD];
    __shared__ __attribute__((aligned(16))) uint16_t vs[HM_TT * PD];
    auto put = [&](uint16_t *row, const mf::u32x4 &x) {
#pragma unroll
        for (int e = 0; e < 4; ++e) ((uint32_t *)row)[e] = x[e];
    };
    const int tid = threadIdx.x;
    const int d0 = blockIdx.x * HM_TD, t0 = blockIdx.y * HM_TT, b = blockIdx.z;
    const uint16_t *kb = k + (size_t)b * N * Dm, *vb = v + (size_t)b * N * Dm;
    // rows t0 - 3 .. t0 + TT - 1 of k (the short filter's history) and
    // t0 .. t0 + TT - 1 of v, 16 chunks of 8 channels per row; every load of
    // the tile is issued before the first LDS write
    constexpr int CR = HM_TD / 8, NKC = (HM_TT + 3) * CR, NVC = HM_TT * CR;
    constexpr int NK = (NKC + 255) / 256, NV = (NVC + 255) / 256;
    mf::u32x4 xk[NK], xv[NV];
#pragma unroll
    for (int j = 0; j < NK; ++j) {
        const int ci = tid + 256 * j, r = ci / CR, c = ci % CR;
        const int t = t0 - 3 + r, d = d0 + 8 * c;
        xk[j] = mf::u32x4{0u, 0u, 0u, 0u};
        if (ci < NKC && t >= 0 && t < N && d < Dm) xk[j] = hm_load8<true>(kb + (size_t)t * Dm + d, Dm - d, vec);
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int ci = tid + 256 * j, r = ci / CR, c = ci % CR;
        const int t = t0 + r, d = d0 + 8 * c;
        xv[j] = mf::u32x4{0u, 0u, 0u, 0u};
        if (ci < NVC && t < N && d < Dm) xv[j] = hm_load8<true>(vb + (size_t)t * Dm + d, Dm - d, vec);
    }
#pragma unroll
    for (int j = 0; j < NK; ++j) {
        const int ci = tid + 256 * j;
        if (ci < NKC) put(&ks[(ci / CR) * PD + 8 * (ci % CR)], xk[j]);
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
        const int ci = tid + 256 * j;
        if (ci < NVC) put(&vs[(ci / CR) * PD + 8 * (ci % CR)], xv[j]);
    }
    // thread: steps 8 c .. 8 c + 7 of channels dl0, dl0 + DS, ...; the 8
    // lanes of a channel write one contiguous 128-byte run of its m_T row.
    // The short-filter taps are loaded before the barrier too.
    constexpr int DS = 256 / (HM_TT / 8), ND = HM_TD / DS;
    const int c = tid % (HM_TT / 8), dl0 = tid / (HM_TT / 8);
    float wt[ND][4];
#pragma unroll
    for (int j = 0; j < ND; ++j) {
        const int d = d0 + dl0 + DS * j;
#pragma unroll
        for (int i = 0; i < 4; ++i) wt[j][i] = (i < L && d < Dm) ? w[(size_t)d * L + i] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < ND; ++j) {
        const int dl = dl0 + DS * j, d = d0 + dl;
        if (d >= Dm) break;
        const float(&wd)[4] = wt[j];
        // k at t - 1, t - 2, t - 3 for t = t0 + 8 c (tile row r + 3 holds step t0 + r)
        float k1 = hm_f<IO>(ks[(8 * c + 2) * PD + dl]), k2 = hm_f<IO>(ks[(8 * c + 1) * PD + dl]),
              k3 = hm_f<IO>(ks[(8 * c) * PD + dl]);
        uint16_t mo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int r = 8 * c + e;
            const float k0 = hm_f<IO>(ks[(r + 3) * PD + dl]);
            const float sh = fmaf(wd[0], k0, fmaf(wd[1], k1, fmaf(wd[2], k2, wd[3] * k3)));
            mo[e] = __builtin_bit_cast(uint16_t, (__bf16)(sh * hm_f<IO>(vs[r * PD + dl])));
            k3 = k2;
            k2 = k1;
            k1 = k0;
        }
        const int nt = N - (t0 + 8 * c);
        if (nt > 0) hm_store8<false>(mT + ((size_t)b * Dm + d) * N + t0 + 8 * c, nt, vec, mo);
    }
}

template <int IO>
__global__ __launch_bounds__(256) void k_h3_gate_out(const uint16_t *__restrict__ q, const uint16_t *__restrict__ zT,
                                                    uint16_t *__restrict__ out, int N, int Dm, int vec) {
    constexpr int PZ = HM_TT + 1;  // odd row stride: the transposed reads spread over the banks
    __shared__ uint16_t zs[HM_TD * PZ];
    const int tid = threadIdx.x;
    const int d0 = blockIdx.x * HM_TD, t0 = blockIdx.y * HM_TT, b = blockIdx.z;
    // rows d0 .. d0 + TD - 1 of z_T, 8 chunks of 8 steps per row, all
    // loaded before the first LDS write
    constexpr int CT = HM_TT / 8, NZ = HM_TD * CT / 256;
    static_assert(HM_TD * CT % 256 == 0, "whole chunks per thread");
    mf::u32x4 xz[NZ];
#pragma unroll
    for (int j = 0; j < NZ; ++j) {
        const int ci = tid + 256 * j, r = ci / CT, c = ci % CT;
        const int d = d0 + r, t = t0 + 8 * c;
        xz[j] = mf::u32x4{0u, 0u, 0u, 0u};
        if (d < Dm && t < N) xz[j] = hm_load8<false>(zT + ((size_t)b * Dm + d) * N + t, N - t, vec);
    }
#pragma unroll
    for (int j = 0; j < NZ; ++j) {
        const int ci = tid + 256 * j, r = ci / CT, c = ci % CT;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            zs[r * PZ + 8 * c + 2 * e] = (uint16_t)(xz[j][e] & 0xffffu);
            zs[r * PZ + 8 * c + 2 * e + 1] = (uint16_t)(xz[j][e] >> 16);
        }
    }
    // thread: 8 channels 8 c .. 8 c + 7, steps tl, tl + 16, ...; its q
    // loads are issued before the barrier
    constexpr int TS = 256 / (HM_TD / 8), NQ = HM_TT / TS;
    const int c = tid % (HM_TD / 8), d = d0 + 8 * c, tl0 = tid / (HM_TD / 8);
    const uint16_t *qb = q + (size_t)b * N * Dm;
    uint16_t *ob = out + (size_t)b * N * Dm;
    mf::u32x4 xq[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const int t = t0 + tl0 + TS * j;
        xq[j] = mf::u32x4{0u, 0u, 0u, 0u};
        if (d < Dm && t < N) xq[j] = hm_load8<true>(qb + (size_t)t * Dm + d, Dm - d, vec);
    }
    __syncthreads();
    if (d >= Dm) return;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const int tl = tl0 + TS * j, t = t0 + tl;
        if (t >= N) break;
        const size_t o = (size_t)t * Dm + d;
        uint16_t r[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint16_t qe = (uint16_t)((e & 1) ? (xq[j][e >> 1] >> 16) : (xq[j][e >> 1] & 0xffffu));
            const float z = __uint_as_float((uint32_t)zs[(8 * c + e) * PZ + tl] << 16);
            r[e] = hm_h<IO>(hm_f<IO>(qe) * z);
        }
        hm_store8<true>(ob + o, Dm - d, vec, r);
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
    const dim3 grid((Dm + HM_TD - 1) / HM_TD, (N + HM_TT - 1) / HM_TT, B);
    const uintptr_t al = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)ws;
    const int vec = (N % 8 == 0 && Dm % 8 == 0 && (al & 15) == 0 && (one & 15) == 0) ? 1 : 0;
    hipError_t e = launch(k_h3_gate_in<IO>, grid, dim3(256), 0, s, (const uint16_t *)k, (const uint16_t *)v, w,
                          mT, N, Dm, L, vec);
    if (e != hipSuccess) return e;
    // z_T is read back by the output gate right away: its stores keep the
    // default cache policy
    e = fc_dispatch<IO_BF16, 0>(fused_log2m(N), mT, f, D, zT, B, Dm, N, s);
    if (e != hipSuccess) return e;
    return launch(k_h3_gate_out<IO>, grid, dim3(256), 0, s, (const uint16_t *)q, (const uint16_t *)zT,
                  (uint16_t *)out, N, Dm, vec);
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
