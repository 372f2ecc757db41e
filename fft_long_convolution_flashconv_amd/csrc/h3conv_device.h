// h3conv_device.h -- device-side building blocks of the gfx950 long-convolution
// kernels: complex arithmetic, activation dtype I/O, in-register radix-2^r DFTs
// and the fused FFT-convolution engine (VALU, fp32, LDS-resident).
//
// The engine computes, for one channel, the causal linear convolution of the
// paperlayer.ai summary of "Hungry Hungry Hippos" (section 2 "Convolutional
// view": FFT of filter and input, pointwise product, inverse FFT; Appendix
// C.1: zero-pad to 2L and keep the first N).  Transform, product and inverse
// are fused in one kernel as in section 4 ("kernel fusion reduces memory
// reads and writes"), with the signal resident in LDS between passes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3c {

// ---------------------------------------------------------------- complex

struct __attribute__((aligned(8))) cf {
    float x, y;
};

__device__ __forceinline__ cf mk(float a, float b) { cf r; r.x = a; r.y = b; return r; }
__device__ __forceinline__ cf cadd(cf a, cf b) { return mk(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ cf csub(cf a, cf b) { return mk(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ cf cmul(cf a, cf b) {
    return mk(fmaf(a.x, b.x, -a.y * b.y), fmaf(a.x, b.y, a.y * b.x));
}
__device__ __forceinline__ cf cscale(cf a, float s) { return mk(a.x * s, a.y * s); }

// Multiply by w16^e where w16 = exp(-2 pi i / 16) (forward) or its conjugate
// (INV).  `e` is a compile-time constant once the calling loops are unrolled,
// so the switch folds and quarter turns cost no multiplies.
template <bool INV>
__device__ __forceinline__ cf mul_w16(cf z, int e) {
    constexpr float C1 = 0.923879532511286756f;  // cos(pi/8)
    constexpr float C2 = 0.707106781186547524f;  // cos(pi/4)
    constexpr float C3 = 0.382683432365089772f;  // cos(3pi/8)
    e &= 15;
    if (INV) e = (16 - e) & 15;
    // w = cos(2 pi e/16) - i sin(2 pi e/16)
    float c, s;
    switch (e) {
        case 0: return z;
        case 4: return mk(z.y, -z.x);     // * (-i)
        case 8: return mk(-z.x, -z.y);    // * (-1)
        case 12: return mk(-z.y, z.x);    // * (+i)
        case 1: c = C1; s = -C3; break;
        case 2: c = C2; s = -C2; break;
        case 3: c = C3; s = -C1; break;
        case 5: c = -C3; s = -C1; break;
        case 6: c = -C2; s = -C2; break;
        case 7: c = -C1; s = -C3; break;
        case 9: c = -C1; s = C3; break;
        case 10: c = -C2; s = C2; break;
        case 11: c = -C3; s = C1; break;
        case 13: c = C3; s = C1; break;
        case 14: c = C2; s = C2; break;
        default: c = C1; s = C3; break;   // 15
    }
    return mk(fmaf(z.x, c, -z.y * s), fmaf(z.x, s, z.y * c));
}

// In-register DFT of size R (2, 4, 8 or 16), natural order in and out:
//   X[k] = sum_m x[m] w_R^{m k},  w_R = exp(-2 pi i / R)  (conjugate if INV).
// Radix-2 decimation in frequency followed by a compile-time bit reversal.
template <int R, bool INV>
__device__ __forceinline__ void dft(cf (&a)[R]) {
#pragma unroll
    for (int half = R / 2; half >= 1; half >>= 1) {
#pragma unroll
        for (int start = 0; start < R; start += 2 * half) {
#pragma unroll
            for (int j = 0; j < half; ++j) {
                cf x = a[start + j], y = a[start + j + half];
                a[start + j] = cadd(x, y);
                // twiddle w_{2 half}^j = w_16^{j * 16 / (2 half)}
                a[start + j + half] = mul_w16<INV>(csub(x, y), j * (16 / (2 * half)));
            }
        }
    }
    // bit-reverse permutation
#pragma unroll
    for (int i = 0; i < R; ++i) {
        int r = 0;
#pragma unroll
        for (int b = 1, t = i; b < R; b <<= 1, t >>= 1) r = (r << 1) | (t & 1);
        if (r > i) { cf t = a[i]; a[i] = a[r]; a[r] = t; }
    }
}

// Multiply x[k] by w_L^{n k} (conjugated if INV), k = 1..R-1.  w_L^n comes from
// one accurate sincospi; higher powers by successive products (at most R-2
// roundings), keeping only two complex temporaries live.
template <int R, bool INV>
__device__ __forceinline__ void apply_twiddles(cf (&x)[R], int n, float inv_L) {
    float s, c;
    sincospif(2.0f * (float)n * inv_L, &s, &c);
    const cf w1 = mk(c, INV ? s : -s);
    cf w = w1;
#pragma unroll
    for (int k = 1; k < R; ++k) {
        x[k] = cmul(x[k], w);
        if (k + 1 < R) w = cmul(w, w1);
    }
}

// ---------------------------------------------------------------- dtype I/O

enum IoType { IO_F32 = 0, IO_F16 = 1, IO_BF16 = 2 };

template <int IO> struct io_elem;
template <> struct io_elem<IO_F32> { using T = float; };
template <> struct io_elem<IO_F16> { using T = _Float16; };
template <> struct io_elem<IO_BF16> { using T = uint16_t; };

template <int IO>
__device__ __forceinline__ float ld_io(const typename io_elem<IO>::T *p) {
    if constexpr (IO == IO_F32) return *p;
    else if constexpr (IO == IO_F16) return (float)(*p);
    else return __uint_as_float(((uint32_t)(*p)) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u)            // inf or nan
        return (uint16_t)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <int IO>
__device__ __forceinline__ void st_io(typename io_elem<IO>::T *p, float v) {
    if constexpr (IO == IO_F32) *p = v;
    else if constexpr (IO == IO_F16) *p = (_Float16)v;
    else *p = f32_to_bf16_rne(v);
}

// ---------------------------------------------------------------- FFT plan

// Transform size M = 2^LOG2M (64 .. 16384).  Passes use radix 16 while at
// least 4 bits remain, then one pass of radix 2, 4 or 8.
template <int LOG2M>
struct Plan {
    static constexpr int M = 1 << LOG2M;
    static constexpr int NT = (M / 16 < 64) ? 64 : (M / 16 > 512 ? 512 : M / 16);  // threads per block
    static constexpr int NPASS = (LOG2M + 3) / 4;
    __host__ __device__ static constexpr int log2r(int p) {
        return (p < LOG2M / 4) ? 4 : (LOG2M - 4 * (LOG2M / 4));
    }
    __host__ __device__ static constexpr int radix(int p) { return 1 << log2r(p); }
    // sub-problem length L_p = M / (R_0 ... R_{p-1})
    __host__ __device__ static constexpr int L(int p) {
        int l = LOG2M;
        for (int i = 0; i < p; ++i) l -= log2r(i);
        return 1 << l;
    }
    static constexpr int LDS_ELEMS = M + M / 16;  // padded
};

__device__ __forceinline__ int pad(int i) { return i + (i >> 4); }

// One DIF pass p (not the first, not the last) over LDS: for every butterfly
// (block, n) read R points at stride s = L/R, DFT, multiply X_k by w_L^{n k},
// write back in place.
template <int LOG2M, int P>
__device__ __forceinline__ void dif_pass(cf *lds, int tid) {
    using PL = Plan<LOG2M>;
    constexpr int R = PL::radix(P), L = PL::L(P), S = L / R, NB = PL::M / R;
    constexpr float INV_L = 1.0f / (float)L;
#pragma unroll 1
    for (int beta = tid; beta < NB; beta += PL::NT) {
        const int blk = beta / S, n = beta % S, base = blk * L + n;
        cf x[R];
#pragma unroll
        for (int m = 0; m < R; ++m) x[m] = lds[pad(base + m * S)];
        dft<R, false>(x);
        apply_twiddles<R, false>(x, n, INV_L);
#pragma unroll
        for (int k = 0; k < R; ++k) lds[pad(base + k * S)] = x[k];
    }
    __syncthreads();
}

// One DIT pass p (inverse of dif_pass<P>, up to a factor R).
template <int LOG2M, int P>
__device__ __forceinline__ void dit_pass(cf *lds, int tid) {
    using PL = Plan<LOG2M>;
    constexpr int R = PL::radix(P), L = PL::L(P), S = L / R, NB = PL::M / R;
    constexpr float INV_L = 1.0f / (float)L;
#pragma unroll 1
    for (int beta = tid; beta < NB; beta += PL::NT) {
        const int blk = beta / S, n = beta % S, base = blk * L + n;
        cf x[R];
#pragma unroll
        for (int k = 0; k < R; ++k) x[k] = lds[pad(base + k * S)];
        apply_twiddles<R, true>(x, n, INV_L);
        dft<R, true>(x);
#pragma unroll
        for (int m = 0; m < R; ++m) lds[pad(base + m * S)] = x[m];
    }
    __syncthreads();
}

template <int LOG2M, int P>
__device__ __forceinline__ void dif_middle(cf *lds, int tid) {
    if constexpr (P >= 1 && P < Plan<LOG2M>::NPASS - 1) {
        dif_pass<LOG2M, P>(lds, tid);
        dif_middle<LOG2M, P + 1>(lds, tid);
    }
}

template <int LOG2M, int P>
__device__ __forceinline__ void dit_middle(cf *lds, int tid) {
    if constexpr (P >= 1 && P < Plan<LOG2M>::NPASS - 1) {
        dit_pass<LOG2M, P>(lds, tid);
        dit_middle<LOG2M, P - 1>(lds, tid);
    }
}

// Register-resident spectrum of the filter at the positions this thread
// covers in the last pass (already scaled by 1/M).
template <int LOG2M>
struct FiltReg {
    using PL = Plan<LOG2M>;
    static constexpr int P = PL::NPASS - 1;
    static constexpr int R = PL::radix(P);
    static constexpr int NBT = (PL::M / R + PL::NT - 1) / PL::NT;  // butterflies / thread
    cf v[NBT][R];
};

// First DIF pass: reads the zero-padded input through `ld(pos)` (only
// positions < M/2 can be non-zero, so the upper half of every butterfly is
// skipped), DFT, twiddle, write to LDS.
template <int LOG2M, class LD>
__device__ __forceinline__ void first_pass(cf *lds, int tid, const LD &ld) {
    using PL = Plan<LOG2M>;
    constexpr int R = PL::radix(0), L = PL::M, S = L / R, NB = PL::M / R;
    constexpr float INV_L = 1.0f / (float)L;
#pragma unroll 1
    for (int beta = tid; beta < NB; beta += PL::NT) {
        const int n = beta;
        cf x[R];
#pragma unroll
        for (int m = 0; m < R; ++m) x[m] = (m < R / 2) ? ld(n + m * S) : mk(0.f, 0.f);
        dft<R, false>(x);
        apply_twiddles<R, false>(x, n, INV_L);
#pragma unroll
        for (int k = 0; k < R; ++k) lds[pad(n + k * S)] = x[k];
    }
    __syncthreads();
}

// Last DIT pass: conjugate twiddle, inverse DFT, hand the first half of every
// butterfly (positions < M/2) to `st(pos, value)`.
template <int LOG2M, class ST>
__device__ __forceinline__ void final_pass(cf *lds, int tid, const ST &st) {
    using PL = Plan<LOG2M>;
    constexpr int R = PL::radix(0), L = PL::M, S = L / R, NB = PL::M / R;
    constexpr float INV_L = 1.0f / (float)L;
#pragma unroll 1
    for (int beta = tid; beta < NB; beta += PL::NT) {
        const int n = beta;
        cf x[R];
#pragma unroll
        for (int k = 0; k < R; ++k) x[k] = lds[pad(n + k * S)];
        apply_twiddles<R, true>(x, n, INV_L);
        dft<R, true>(x);
#pragma unroll
        for (int m = 0; m < R / 2; ++m) st(n + m * S, x[m]);
    }
}

// Spectrum of a zero-padded signal (positions < M/2 loaded by `ld`) into
// registers: S = DFT_M(x || 0) * sc, digit-reversed, at the positions the
// last pass of this thread covers.
template <int LOG2M, class LD>
__device__ __forceinline__ void spectrum(cf *lds, int tid, const LD &ld, FiltReg<LOG2M> &S, float sc) {
    using PL = Plan<LOG2M>;
    using FR = FiltReg<LOG2M>;
    constexpr int R = FR::R, NB = PL::M / R;
    first_pass<LOG2M>(lds, tid, ld);
    dif_middle<LOG2M, 1>(lds, tid);
#pragma unroll
    for (int i = 0; i < FR::NBT; ++i) {
        const int beta = tid + i * PL::NT;
        if (beta < NB) {
            cf x[R];
#pragma unroll
            for (int m = 0; m < R; ++m) x[m] = lds[pad(beta * R + m)];
            dft<R, false>(x);
#pragma unroll
            for (int k = 0; k < R; ++k) S.v[i][k] = cscale(x[k], sc);
        }
    }
    __syncthreads();
}

// Spectrum of a zero-padded real filter into registers: F = DFT_M(f || 0)/M.
template <int LOG2M, class LD>
__device__ __forceinline__ void filter_spectrum(cf *lds, int tid, const LD &ld, FiltReg<LOG2M> &F) {
    spectrum<LOG2M>(lds, tid, ld, F, 1.0f / (float)Plan<LOG2M>::M);
}

// Inverse transform (unnormalised) of a spectrum held in registers in the
// FiltReg layout: the inverse last-pass DFT into LDS, the inverse DIT
// passes, and st(pos, value) for the first M/2 positions.
template <int LOG2M, class ST>
__device__ __forceinline__ void inverse_regs(cf *lds, int tid, const FiltReg<LOG2M> &Y, const ST &st) {
    using PL = Plan<LOG2M>;
    using FR = FiltReg<LOG2M>;
    constexpr int R = FR::R, NB = PL::M / R;
#pragma unroll
    for (int i = 0; i < FR::NBT; ++i) {
        const int beta = tid + i * PL::NT;
        if (beta < NB) {
            cf x[R];
#pragma unroll
            for (int k = 0; k < R; ++k) x[k] = Y.v[i][k];
            dft<R, true>(x);
#pragma unroll
            for (int m = 0; m < R; ++m) lds[pad(beta * R + m)] = x[m];
        }
    }
    __syncthreads();
    dit_middle<LOG2M, PL::NPASS - 2>(lds, tid);
    final_pass<LOG2M>(lds, tid, st);
    __syncthreads();  // LDS is reused by the next transform
}

// Full fused convolution of one complex signal with the filter spectrum:
// forward DIF passes, pointwise product with F fused into the last pass
// together with the first inverse pass, inverse DIT passes, store.
template <int LOG2M, class LD, class ST>
__device__ __forceinline__ void conv_signal(cf *lds, int tid, const FiltReg<LOG2M> &F, const LD &ld,
                                            const ST &st) {
    using PL = Plan<LOG2M>;
    using FR = FiltReg<LOG2M>;
    constexpr int R = FR::R, NB = PL::M / R;
    first_pass<LOG2M>(lds, tid, ld);
    dif_middle<LOG2M, 1>(lds, tid);
#pragma unroll
    for (int i = 0; i < FR::NBT; ++i) {
        const int beta = tid + i * PL::NT;
        if (beta < NB) {
            cf x[R];
#pragma unroll
            for (int m = 0; m < R; ++m) x[m] = lds[pad(beta * R + m)];
            dft<R, false>(x);
#pragma unroll
            for (int k = 0; k < R; ++k) x[k] = cmul(x[k], F.v[i][k]);
            dft<R, true>(x);
#pragma unroll
            for (int m = 0; m < R; ++m) lds[pad(beta * R + m)] = x[m];
        }
    }
    __syncthreads();
    dit_middle<LOG2M, PL::NPASS - 2>(lds, tid);
    final_pass<LOG2M>(lds, tid, st);
    __syncthreads();  // LDS is reused by the next signal
}

}  // namespace h3c
