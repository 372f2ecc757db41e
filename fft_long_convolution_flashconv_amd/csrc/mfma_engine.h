// mfma_engine.h -- fused block-FFT convolution engine for fp16/bf16 activations
// on gfx950: radix-16 DFT blocks as dense matrix products on the matrix cores
// (v_mfma_f32_16x16x32_f16, fp16 operands, fp32 accumulation), twiddles and
// the pointwise product on the vector ALUs, the signal resident in LDS as
// packed fp16 complex between passes.
//
// Method: the paperlayer.ai summary of "Hungry Hungry Hippos", section 4
// (FlashConv: fused FFT, pointwise product and inverse FFT; the block FFT
// rewrites the FFT as small matrix multiplications so it runs on matrix
// units, possibly with more FLOPs), section 2 "Convolutional view" and
// Appendix C.1 (zero-pad to 2L, keep the first N).
//
// Transform of size M = 2^LOG2M = V * 16^NM (V = 2..16):
//   pass 0      VALU radix-V decimation-in-frequency on the zero-padded input
//               (read from HBM, only the first V/2 points of each butterfly
//               are non-zero), twiddle, to LDS;
//   pass 1..NM  radix-16 DIF passes; the 16x16 complex DFT is a 32x32 real
//               matrix [[Re W, -Im W], [Im W, Re W]] applied by two MFMAs to
//               16 butterflies (columns) at a time;
//   last pass   (L = 16) keeps the spectrum in registers, multiplies by the
//               filter spectrum, and feeds the product straight into the
//               inverse radix-16 MFMA (the accumulator layout is reused as the
//               next operand layout, no LDS round trip);
//   inverse     the same passes in reverse order (decimation in time), the
//               last one on the VALU writes only the first N outputs.
// Spectra stay in digit-reversed order; the filter spectrum is produced by
// the same forward passes, so the pointwise product needs no reordering.
//
// Range: activations are scaled by a power of two chosen from max|u| per
// round of signals so that no fp16 intermediate can overflow
// (|U| <= N max|u| s < 2^15), and the spectrum product is rescaled the same
// way from its own maximum before the inverse; all scales are powers of two
// and are undone exactly at the output.
#pragma once

#include "h3conv_device.h"

namespace h3c {
namespace mf {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- packed fp16 complex

// Packed fp16 complex helpers, written as plain vector code: the compiler
// emits v_cvt_pk_f16_f32 (round to nearest even) and v_pk_mul_f16 /
// v_pk_fma_f16 with op_sel / neg modifiers, and it knows their hazards
// against the matrix-core results they consume.
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));

// (re, im) -> one dword, round to nearest even.
__device__ __forceinline__ uint32_t pk(float re, float im) {
    const f2 v = {re, im};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
}
__device__ __forceinline__ float h_lo(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}
__device__ __forceinline__ float h_hi(uint32_t v) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}
__device__ __forceinline__ cf unpk(uint32_t v) { return mk(h_lo(v), h_hi(v)); }

// x * w on packed fp16 complex.
__device__ __forceinline__ uint32_t cmulh(uint32_t xx, uint32_t ww) {
    const h2 x = __builtin_bit_cast(h2, xx), w = __builtin_bit_cast(h2, ww);
    const h2 t = x.xx * w;
    const h2 nw = {-w.y, w.x};
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(x.yy, nw, t));
}
// x * conj(w) on packed fp16 complex.
__device__ __forceinline__ uint32_t cmulh_conj(uint32_t xx, uint32_t ww) {
    const h2 x = __builtin_bit_cast(h2, xx), w = __builtin_bit_cast(h2, ww);
    const h2 cw = {w.x, -w.y};
    const h2 t = x.xx * cw;
    const h2 sw = {w.y, w.x};
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(x.yy, sw, t));
}
// both halves times the same packed factor
__device__ __forceinline__ uint32_t pkmul(uint32_t xx, uint32_t ss) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, xx) * __builtin_bit_cast(h2, ss));
}

__device__ __forceinline__ half8 as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    u4 v = {a, b, c, d};
    return __builtin_bit_cast(half8, v);
}

// One real entry of the 32x32 real form of the complex 16-point DFT:
// output (k, part p) from input (m, part q), W = exp(-+2 pi i k m / 16).
// v_cos_f32 / v_sin_f32 take revolutions; their error (~1e-7) is far below
// the fp16 rounding the entry gets anyway.
__device__ __forceinline__ float dft_entry(int k, int p, int m, int q, bool inv) {
    const float r = (float)((k * m) & 15) * 0.0625f;
    const float wr = __builtin_amdgcn_cosf(r), s = __builtin_amdgcn_sinf(r);
    const float wi = inv ? s : -s;
    if (p == 0) return q == 0 ? wr : -wi;
    return q == 0 ? wi : wr;
}

// Shared-memory index swizzle for packed-complex dwords: bits 4-5 are XORed
// with a fold of bits 6 and up, so 16-dword groups stay contiguous (b128
// reads) while strided MFMA operand gathers spread over the 64 banks.  The
// map is linear over XOR, so phys(a + b) = phys(a) ^ phys(b) whenever a and
// b have disjoint bits; addresses are split that way into per-lane and
// compile-time parts.
__host__ __device__ constexpr int phys(int i) {
    int x = i >> 6;
    x = (x ^ (x >> 2) ^ (x >> 4) ^ (x >> 6)) & 3;
    return i ^ (x << 4);
}

// Workgroup shape per transform size: SIG signals in flight, NW waves.
template <int LOG2M> struct Cfg;
template <> struct Cfg<9> { static constexpr int SIG = 8, NW = 2; };
template <> struct Cfg<10> { static constexpr int SIG = 4, NW = 4; };
template <> struct Cfg<11> { static constexpr int SIG = 4, NW = 8; };
template <> struct Cfg<12> { static constexpr int SIG = 2, NW = 8; };
template <> struct Cfg<13> { static constexpr int SIG = 1, NW = 16; };
template <> struct Cfg<14> { static constexpr int SIG = 1, NW = 16; };

// M = 16 * 16^K * R (R = 2, 4, 8 or 16): pass 0 is a zero-padded radix-16
// pass, then K radix-16 passes, then the last pass of radix R.
template <int LOG2M>
struct Shape {
    static constexpr int M = 1 << LOG2M;
    static constexpr int K = (LOG2M - 5) / 4;          // middle radix-16 passes
    static constexpr int LR = LOG2M - 4 - 4 * K;       // log2 of the last radix
    static constexpr int R = 1 << LR;
    static constexpr int S0 = M / 16;                  // pass-0 stride (= butterflies)
    static constexpr int SIG = Cfg<LOG2M>::SIG, NW = Cfg<LOG2M>::NW, NT = 64 * NW;
    static constexpr int T0 = SIG * S0 / 32;           // pass-0 tiles (32 butterflies) per round
    static constexpr int T0W = T0 / NW;
    static constexpr int TI = SIG * S0 / 16;           // inverse pass-0 tiles (16 butterflies)
    static constexpr int TIW = TI / NW;
    static constexpr int TM = M / 256;                 // middle-pass tiles per signal
    static constexpr int TPW = TM / NW;
    static constexpr int TL8 = M / 128;                // radix-8 last-pass tiles per signal
    static constexpr int T8W = TL8 / NW;
    static constexpr int NBL = M / R;                  // radix-2/4 last-pass butterflies per signal
    static constexpr int NSL = (NBL > NT) ? NBL / NT : 1;            // distinct positions per thread
    static constexpr int BPTL = (SIG * NBL + NT - 1) / NT;           // butterflies per thread
    static constexpr int DATA = SIG * M;
    static constexpr int LDS_DWORDS = SIG * M + 64;
    static constexpr int DELTA = 256 * NW;             // butterfly-base step between a wave's tiles
    static_assert(T0 % NW == 0 && TI % NW == 0, "pass-0 tiles must split evenly over waves");
    static_assert(K == 0 || TM % NW == 0, "middle tiles must split evenly over waves");
    static_assert(R != 8 || TL8 % NW == 0, "radix-8 tiles must split evenly over waves");
    static_assert(R > 4 || NBL % NT == 0 || NT % NBL == 0, "radix-2/4 butterflies must tile the threads");
    static_assert(M <= 256 * 16 * NW, "a lane must see one butterfly offset per middle pass");
    __host__ __device__ static constexpr int L(int p) { return M >> (4 * p); }  // p = 1..K
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Power-of-two scale 2^(8 - e - hb) where amax < 2^e: after a transform that
// can grow magnitudes by at most 2^(2 hb), values stay below 2^(8 + hb).
__device__ __forceinline__ float pow2_scale(float amax, int hb) {
    int e = 0;
    if (amax > 0.f) (void)frexpf(amax, &e);
    return ldexpf(1.f, 8 - e - hb);
}

// max(|re|, |im|) of a packed fp16 complex, as fp32
__device__ __forceinline__ float habs_max(uint32_t v) {
    const h2 a = __builtin_elementwise_abs(__builtin_bit_cast(h2, v));
    return (float)__builtin_elementwise_max(a.x, a.y);
}

// opaque copy: keeps lane-derived indices from being hoisted (and held in
// registers) across the whole kernel
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));

// How a round's inputs arrive: RAW_F16 / RAW_BF16 = two 16-bit activations
// packed in a dword (row 2s low half, row 2s+1 high half); FP32 = a complex
// value already in fp32 (used when the loader computes its input).
enum InKind { IN_FP32 = 0, IN_F16 = 1, IN_BF16 = 2 };
template <int KIND> struct InT { using T = cf; };
template <> struct InT<IN_F16> { using T = uint32_t; };
template <> struct InT<IN_BF16> { using T = uint32_t; };

template <int KIND>
__device__ __forceinline__ float in_amax(const typename InT<KIND>::T &x) {
    if constexpr (KIND == IN_F16) return habs_max(x);
    else if constexpr (KIND == IN_BF16)
        return fmaxf(fabsf(__uint_as_float(x << 16)), fabsf(__uint_as_float(x & 0xffff0000u)));
    else return fmaxf(fabsf(x.x), fabsf(x.y));
}
// scaled packed fp16 operand value; `sh` is the scale as a packed fp16 pair
template <int KIND>
__device__ __forceinline__ uint32_t in_scaled(const typename InT<KIND>::T &x, float s, uint32_t sh) {
    if constexpr (KIND == IN_F16) return pkmul(x, sh);
    else if constexpr (KIND == IN_BF16) return pk(__uint_as_float(x << 16) * s, __uint_as_float(x & 0xffff0000u) * s);
    else return pk(x.x * s, x.y * s);
}

// Row pointers of one complex signal (two activation rows) for the 16-bit
// activation kinds: in0/out0 carry the real part, in1/out1 (may be null) the
// imaginary part.
struct RowPtrs {
    const uint16_t *in0, *in1;
    uint16_t *out0, *out1;
};

template <int LOG2M, int KIND>
struct Engine {
    using SH = Shape<LOG2M>;
    using IT = typename InT<KIND>::T;
    static constexpr int M = SH::M, K = SH::K, R = SH::R, S0 = SH::S0, SIG = SH::SIG, NW = SH::NW,
                         NT = SH::NT, T0W = SH::T0W, TIW = SH::TIW, TPW = SH::TPW, T8W = SH::T8W,
                         NBL = SH::NBL, NSL = SH::NSL, BPTL = SH::BPTL, DELTA = SH::DELTA;
    static_assert(S0 >= 32, "pass-0 tiles must lie within one signal");
    static constexpr int KM = K > 0 ? K : 1;          // array sizes
    static constexpr int FN = R == 16 ? TPW * 4 : (R == 8 ? T8W * 2 : NSL * R);  // filter values / lane
    // distinct butterfly offsets a lane meets in pass 0 (32-column tiles) and
    // in its inverse (16-column tiles)
    static constexpr int ND0 = S0 > 32 * NW ? S0 / (32 * NW) : 1;
    static constexpr int NDI = S0 > 16 * NW ? S0 / (16 * NW) : 1;

    uint32_t *data;  // [SIG][M] packed complex (swizzled)
    float *red;      // [2][NW] reduction slots
    int tid, w, lane, j, g;
    half8 A0;                               // pass 0: 32x32x16, zero-padded DFT-16
    half8 Af0, Af1, Ai0, Ai1, Ac0, Ac1;     // 16x16x32: forward, inverse, chained inverse
    half4 A8f, A8i;                         // 16x16x16: radix-8 forward and inverse
    uint32_t F[FN];                         // filter spectrum * cF (packed fp16)
    uint32_t twf[KM][4], twi[KM][4];        // middle pass p: w_L^{n k} (write / read slots)
    uint32_t tw0[ND0][8];                   // pass 0:  w_M^{n q}, q = this lane's 8 outputs
    uint32_t tu0[NDI][4];                   // inverse pass 0: w_M^{n k}, k = 4g .. 4g+3
    float cF;
    IT pin[T0W][4], pnx[T0W][4];            // pass-0 operands: this round, next round
    int rbank = 0;

    __device__ Engine(uint32_t *smem) {
        data = smem;
        red = (float *)(smem + SH::DATA);
        tid = threadIdx.x;
        w = tid >> 6;
        lane = tid & 63;
        j = lane & 15;
        g = lane >> 4;
    }

    __device__ static uint32_t tw_m(int t) {  // w_M^t = exp(-2 pi i t / M), t in [0, M)
        const float r = (float)(t & (M - 1)) * (1.0f / (float)M);
        return pk(__builtin_amdgcn_cosf(r), -__builtin_amdgcn_sinf(r));
    }
    // output q of accumulator pair v (v even) in the 32x32 layout, lane half h
    __device__ static __forceinline__ int q32(int v, int h) { return 4 * (v >> 2) + 2 * h + ((v & 3) >> 1); }

    template <int P>
    __device__ void init_mid() {
        if constexpr (P <= K) {
            constexpr int L = SH::L(P), S = L / 16, SHF = LOG2M - __builtin_ctz(L);
            const int n = (16 * w + j) % S;
            twf[P - 1][0] = tw_m((n * (2 * g)) << SHF);
            twf[P - 1][1] = tw_m((n * (2 * g + 1)) << SHF);
            twf[P - 1][2] = tw_m((n * (8 + 2 * g)) << SHF);
            twf[P - 1][3] = tw_m((n * (9 + 2 * g)) << SHF);
#pragma unroll
            for (int e = 0; e < 4; ++e) twi[P - 1][e] = tw_m((n * (4 * g + e)) << SHF);
            init_mid<P + 1>();
        }
    }

    __device__ void init() {
        const int p = j & 1, kk = j >> 1;
        const int i32 = lane & 31, g32 = lane >> 5;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // 16x16x32 natural K order: slot (g, e) <-> input m = 4g + e/2, part e%2
            const int m = 4 * g + (e >> 1), q = e & 1;
            Af0[e] = (_Float16)dft_entry(kk, p, m, q, false);
            Af1[e] = (_Float16)dft_entry(kk + 8, p, m, q, false);
            Ai0[e] = (_Float16)dft_entry(kk, p, m, q, true);
            Ai1[e] = (_Float16)dft_entry(kk + 8, p, m, q, true);
            // chained K order: slot (g, e) <-> k = 8 (e/4) + 2g + (e%4)/2, part e%2
            const int kc = 8 * (e >> 2) + 2 * g + ((e & 3) >> 1);
            Ac0[e] = (_Float16)dft_entry(kk, p, kc, q, true);
            Ac1[e] = (_Float16)dft_entry(kk + 8, p, kc, q, true);
            // 32x32x16: row i32 -> output (i32/2, i32%2); slot (g32, e) -> input
            // m = 4 g32 + e/2 (inputs 8..15 are the zero padding)
            A0[e] = (_Float16)dft_entry(i32 >> 1, i32 & 1, 4 * g32 + (e >> 1), q, false);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            // 16x16x16 (radix 8): row j -> output (j/2, j%2); slot (g, e) -> m = 2g + e/2
            const int m = 2 * g + (e >> 1), q = e & 1;
            const float r = (float)((kk * m) & 7) * 0.125f;
            const float wr = __builtin_amdgcn_cosf(r), ws = __builtin_amdgcn_sinf(r);
            A8f[e] = (_Float16)(p == 0 ? (q == 0 ? wr : ws) : (q == 0 ? -ws : wr));
            A8i[e] = (_Float16)(p == 0 ? (q == 0 ? wr : -ws) : (q == 0 ? ws : wr));
        }
#pragma unroll
        for (int d = 0; d < ND0; ++d) {
            const int n = (32 * (w + d * NW) + i32) % S0;
#pragma unroll
            for (int v = 0; v < 16; v += 2) tw0[d][v >> 1] = tw_m(n * q32(v, g32));
        }
#pragma unroll
        for (int d = 0; d < NDI; ++d) {
            const int n = (16 * (w + d * NW) + j) % S0;
#pragma unroll
            for (int e = 0; e < 4; ++e) tu0[d][e] = tw_m(n * (4 * g + e));
        }
        init_mid<1>();
    }

    // Workgroup max (SUM = false) or sum (SUM = true).  Two alternating slot
    // banks: a wave can only write a bank again after the next reduction's
    // barrier, which every wave reaches only after reading that bank.
    template <bool SUM>
    __device__ float block_reduce(float v) {
        v = SUM ? wave_sum(v) : wave_max(v);
        float *r = red + rbank * NW;
        rbank ^= 1;
        if (lane == 0) r[w] = v;
        __syncthreads();
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) m = SUM ? m + r[i] : fmaxf(m, r[i]);
        return m;
    }
    __device__ float block_max(float v) { return block_reduce<false>(v); }

    __device__ __forceinline__ uint32_t &at(int s, int pi) { return data[s * M + pi]; }

    // ---------------------------------------------------------- pass 0
    // Operand gather: tile i of this wave covers butterflies (columns)
    // c = 32 (w + i NW) + lane%32 of signal s = 32 (w + i NW) / S0 (uniform
    // over the tile), offset n = c % S0; lane half h = lane/32 holds inputs
    // m = 4h .. 4h+3 at n + m S0.
    __device__ __forceinline__ int tile_sig(int i) { return (32 * (w + i * NW)) / S0; }
    __device__ __forceinline__ int tile_n(int i) { return (32 * (w + i * NW)) % S0 + (lane & 31); }

    // 16-bit activations through row pointers; `nval` valid samples per row.
    template <class RP>
    __device__ __forceinline__ void fetch_raw(const RP &rows, int sig0, int nsig, int nval, uint32_t (&buf)[T0W][4]) {
        const int h = lane >> 5;
        const bool full = nval >= M / 2;
#pragma unroll
        for (int i = 0; i < T0W; ++i) {
            const int s = __builtin_amdgcn_readfirstlane(tile_sig(i));
            const int off = tile_n(i) + 4 * h * S0;
            if (s < nsig) {
                const RowPtrs rp = rows(sig0 + s);
                if (full) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t lo = rp.in0[off + e * S0];
                        const uint32_t hi = rp.in1 ? (uint32_t)rp.in1[off + e * S0] : 0u;
                        buf[i][e] = lo | (hi << 16);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int pos = off + e * S0;
                        const bool ok = pos < nval;
                        const uint32_t lo = ok ? (uint32_t)rp.in0[pos] : 0u;
                        const uint32_t hi = (ok && rp.in1) ? (uint32_t)rp.in1[pos] : 0u;
                        buf[i][e] = lo | (hi << 16);
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) buf[i][e] = 0u;
            }
        }
    }

    // generic fp32 inputs: ld(sig, pos) -> cf, zero past the sequence
    template <class LD>
    __device__ __forceinline__ void fetch_fp32(const LD &ld, int sig0, int nsig, cf (&buf)[T0W][4]) {
        const int h = lane >> 5;
#pragma unroll
        for (int i = 0; i < T0W; ++i) {
            const int s = tile_sig(i);
            const int off = tile_n(i) + 4 * h * S0;
#pragma unroll
            for (int e = 0; e < 4; ++e) buf[i][e] = (s < nsig) ? ld(sig0 + s, off + e * S0) : mk(0.f, 0.f);
        }
    }

    // zero-padded radix-16 DIF pass: DFT on the matrix cores, twiddle w_M^{n q},
    // to LDS.  `op(i, e)` yields the packed scaled operand.  The matrix-core
    // pass runs for every tile (operands of absent signals are zero); results
    // land in that signal's slot of LDS, which no later pass reads.
    template <class OP>
    __device__ void pass0(const OP &op) {
        const int h = lane >> 5;
        const int pq = phys(2 * h * S0);  // q = const(v) + 2h, disjoint bits
#pragma unroll
        for (int i = 0; i < T0W; ++i) {
            const int s = tile_sig(i);
            const int pn = phys(tile_n(i)) ^ pq;
            const half8 b = as_half8(op(i, 0), op(i, 1), op(i, 2), op(i, 3));
            f16v z = {};
            const f16v d = __builtin_amdgcn_mfma_f32_32x32x16_f16(A0, b, z, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 16; v += 2) {
                const int qc = 4 * (v >> 2) + ((v & 3) >> 1);  // q = qc + 2h
                at(s, pn ^ phys(qc * S0)) = cmulh(pk(d[v], d[v + 1]), tw0[i % ND0][v >> 1]);
            }
        }
        __syncthreads();
    }

    // inverse pass 0: conjugate twiddle, inverse DFT-16 on the matrix cores
    // keeping outputs m < 8; out(s, n, m, re, im) for m = 2g, 2g+1.
    template <class OUT>
    __device__ void pass0_inv(const OUT &out, int nsig) {
        const int pk4 = phys(4 * g * S0);
        const int s_stride = (16 * NW) / S0;  // signals per tile step (0 if a signal spans steps)
        (void)s_stride;
#pragma unroll
        for (int i = 0; i < TIW; ++i) {
            const int s = __builtin_amdgcn_readfirstlane((16 * (w + i * NW)) / S0);
            const int n = (16 * (w + i * NW)) % S0 + j;
            if (s < nsig) {
                const int pn = phys(n) ^ pk4;
                uint32_t x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = cmulh_conj(at(s, pn ^ phys(e * S0)), tu0[i % NDI][e]);
                f4 z = {0.f, 0.f, 0.f, 0.f};
                const f4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ai0, as_half8(x[0], x[1], x[2], x[3]), z, 0, 0, 0);
                out(s, n, 2 * g, d[0], d[1]);
                out(s, n, 2 * g + 1, d[2], d[3]);
            }
        }
    }

    // ---------------------------------------------------------- middle passes
    template <int P>
    __device__ __forceinline__ int base0() {
        constexpr int L = SH::L(P), S = L / 16;
        const int b = 16 * opaque(w) + opaque(j);
        return (b / S) * L + (b % S);
    }

    template <int P>
    __device__ void fwd_pass(int nsig) {
        constexpr int L = SH::L(P), S = L / 16;
        const int b0 = base0<P>();
        const int pr = phys(b0) ^ phys(4 * g * S);   // read  slots m = 4g + e
        const int pw = phys(b0) ^ phys(2 * g * S);   // write slots k = 2g + {0, 1, 8, 9}
        for (int s = 0; s < nsig; ++s) {
#pragma unroll
            for (int ti = 0; ti < TPW; ++ti) {
                const int ct = phys(ti * DELTA);
                const half8 b = as_half8(at(s, pr ^ ct ^ phys(0 * S)), at(s, pr ^ ct ^ phys(1 * S)),
                                         at(s, pr ^ ct ^ phys(2 * S)), at(s, pr ^ ct ^ phys(3 * S)));
                f4 z = {0.f, 0.f, 0.f, 0.f};
                const f4 d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Af0, b, z, 0, 0, 0);
                const f4 d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Af1, b, z, 0, 0, 0);
                at(s, pw ^ ct ^ phys(0 * S)) = cmulh(pk(d0[0], d0[1]), twf[P - 1][0]);
                at(s, pw ^ ct ^ phys(1 * S)) = cmulh(pk(d0[2], d0[3]), twf[P - 1][1]);
                at(s, pw ^ ct ^ phys(8 * S)) = cmulh(pk(d1[0], d1[1]), twf[P - 1][2]);
                at(s, pw ^ ct ^ phys(9 * S)) = cmulh(pk(d1[2], d1[3]), twf[P - 1][3]);
            }
        }
        __syncthreads();
    }

    template <int P>
    __device__ void inv_pass(int nsig) {
        constexpr int L = SH::L(P), S = L / 16;
        const int b0 = base0<P>();
        const int pr = phys(b0) ^ phys(4 * g * S);
        const int pw = phys(b0) ^ phys(2 * g * S);
        for (int s = 0; s < nsig; ++s) {
#pragma unroll
            for (int ti = 0; ti < TPW; ++ti) {
                const int ct = phys(ti * DELTA);
                uint32_t x[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) x[e] = cmulh_conj(at(s, pr ^ ct ^ phys(e * S)), twi[P - 1][e]);
                f4 z = {0.f, 0.f, 0.f, 0.f};
                const half8 b = as_half8(x[0], x[1], x[2], x[3]);
                const f4 d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ai0, b, z, 0, 0, 0);
                const f4 d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ai1, b, z, 0, 0, 0);
                at(s, pw ^ ct ^ phys(0 * S)) = pk(d0[0], d0[1]);
                at(s, pw ^ ct ^ phys(1 * S)) = pk(d0[2], d0[3]);
                at(s, pw ^ ct ^ phys(8 * S)) = pk(d1[0], d1[1]);
                at(s, pw ^ ct ^ phys(9 * S)) = pk(d1[2], d1[3]);
            }
        }
        __syncthreads();
    }

    template <int P>
    __device__ void fwd_middle(int nsig) {
        if constexpr (P <= K) {
            fwd_pass<P>(nsig);
            fwd_middle<P + 1>(nsig);
        }
    }
    template <int P>
    __device__ void inv_middle(int nsig) {
        if constexpr (P >= 1) {
            inv_pass<P>(nsig);
            inv_middle<P - 1>(nsig);
        }
    }

    // ---------------------------------------------------------- last pass
    static constexpr int NV = R == 16 ? 4 : (R == 8 ? 2 : R);
    static constexpr int NLS = R == 16 ? TPW : (R == 8 ? T8W : BPTL);  // slots per round
    static constexpr int NU = R >= 8 ? SIG * NLS : NLS;                 // (signal, slot) units

    __device__ __forceinline__ int lpos(int slot, int &s) {
        // physical base of the slot's butterfly (R consecutive positions)
        if constexpr (R == 16) {
            s = -1;
            return phys(16 * (16 * opaque(w) + opaque(j))) ^ phys(16 * slot * 16 * NW);
        } else if constexpr (R == 8) {
            s = -1;
            return phys(8 * (16 * opaque(w) + opaque(j))) ^ phys(8 * slot * 16 * NW);
        } else {
            const int beta = opaque(tid) + slot * NT;
            s = beta / NBL;
            return phys(R * (beta % NBL));
        }
    }

    // forward last-pass DFT of this slot (packed fp16 results)
    __device__ __forceinline__ void last_fwd(int s, int pb, uint32_t (&y)[NV]) {
        if constexpr (R == 16) {
            typedef uint32_t u4 __attribute__((ext_vector_type(4)));
            const u4 v = *(const u4 *)&at(s, pb ^ (4 * g));
            f4 z = {0.f, 0.f, 0.f, 0.f};
            const f4 d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Af0, __builtin_bit_cast(half8, v), z, 0, 0, 0);
            const f4 d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Af1, __builtin_bit_cast(half8, v), z, 0, 0, 0);
            y[0] = pk(d0[0], d0[1]);
            y[1] = pk(d0[2], d0[3]);
            y[2] = pk(d1[0], d1[1]);
            y[3] = pk(d1[2], d1[3]);
        } else if constexpr (R == 8) {
            typedef uint32_t u2 __attribute__((ext_vector_type(2)));
            const u2 v = *(const u2 *)&at(s, pb ^ (2 * g));
            f4 z = {0.f, 0.f, 0.f, 0.f};
            const f4 d = __builtin_amdgcn_mfma_f32_16x16x16f16(A8f, __builtin_bit_cast(half4, v), z, 0, 0, 0);
            y[0] = pk(d[0], d[1]);
            y[1] = pk(d[2], d[3]);
        } else if constexpr (R == 4) {
            // (vector elements are copied to scalars before the bit casts:
            //  bit-casting an element expression directly reads element 0)
            typedef uint32_t u4 __attribute__((ext_vector_type(4)));
            const u4 v = *(const u4 *)&at(s, pb);
            const uint32_t v0 = v.x, v1 = v.y, v2 = v.z, v3 = v.w;
            const h2 a = __builtin_bit_cast(h2, v0), b = __builtin_bit_cast(h2, v1),
                     c = __builtin_bit_cast(h2, v2), d = __builtin_bit_cast(h2, v3);
            const h2 s0 = a + c, d0 = a - c, s1 = b + d, d1 = b - d;
            const h2 d1mi = {d1.y, -d1.x};  // (b - d) * (-i)
            y[0] = __builtin_bit_cast(uint32_t, s0 + s1);
            y[1] = __builtin_bit_cast(uint32_t, d0 + d1mi);
            y[2] = __builtin_bit_cast(uint32_t, s0 - s1);
            y[3] = __builtin_bit_cast(uint32_t, d0 - d1mi);
        } else {
            typedef uint32_t u2 __attribute__((ext_vector_type(2)));
            const u2 v = *(const u2 *)&at(s, pb);
            const uint32_t v0 = v.x, v1 = v.y;
            const h2 a = __builtin_bit_cast(h2, v0), b = __builtin_bit_cast(h2, v1);
            y[0] = __builtin_bit_cast(uint32_t, a + b);
            y[1] = __builtin_bit_cast(uint32_t, a - b);
        }
    }

    // inverse last-pass DFT of the (scaled) spectrum product, written in place
    __device__ __forceinline__ void last_inv(int s, int pb, const uint32_t (&y)[NV]) {
        if constexpr (R == 16) {
            f4 z = {0.f, 0.f, 0.f, 0.f};
            const half8 b = as_half8(y[0], y[1], y[2], y[3]);
            const f4 d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ac0, b, z, 0, 0, 0);
            const f4 d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ac1, b, z, 0, 0, 0);
            typedef uint32_t u2 __attribute__((ext_vector_type(2)));
            u2 lo = {pk(d0[0], d0[1]), pk(d0[2], d0[3])};
            u2 hi = {pk(d1[0], d1[1]), pk(d1[2], d1[3])};
            *(u2 *)&at(s, pb ^ (2 * g)) = lo;
            *(u2 *)&at(s, pb ^ (8 + 2 * g)) = hi;
        } else if constexpr (R == 8) {
            typedef uint32_t u2 __attribute__((ext_vector_type(2)));
            const u2 yy = {y[0], y[1]};
            f4 z = {0.f, 0.f, 0.f, 0.f};
            const f4 d = __builtin_amdgcn_mfma_f32_16x16x16f16(A8i, __builtin_bit_cast(half4, yy), z, 0, 0, 0);
            u2 o = {pk(d[0], d[1]), pk(d[2], d[3])};
            *(u2 *)&at(s, pb ^ (2 * g)) = o;
        } else if constexpr (R == 4) {
            const h2 a = __builtin_bit_cast(h2, y[0]), b = __builtin_bit_cast(h2, y[1]),
                     c = __builtin_bit_cast(h2, y[2]), d = __builtin_bit_cast(h2, y[3]);
            const h2 s0 = a + c, d0 = a - c, s1 = b + d, d1 = b - d;
            const h2 d1pi = {-d1.y, d1.x};  // (b - d) * (+i)
            typedef uint32_t u4 __attribute__((ext_vector_type(4)));
            u4 o = {__builtin_bit_cast(uint32_t, s0 + s1), __builtin_bit_cast(uint32_t, d0 + d1pi),
                    __builtin_bit_cast(uint32_t, s0 - s1), __builtin_bit_cast(uint32_t, d0 - d1pi)};
            *(u4 *)&at(s, pb) = o;
        } else {
            const h2 a = __builtin_bit_cast(h2, y[0]), b = __builtin_bit_cast(h2, y[1]);
            typedef uint32_t u2 __attribute__((ext_vector_type(2)));
            u2 o = {__builtin_bit_cast(uint32_t, a + b), __builtin_bit_cast(uint32_t, a - b)};
            *(u2 *)&at(s, pb) = o;
        }
    }

    __device__ __forceinline__ int fslot(int slot) {
        if constexpr (R >= 8) return slot * NV;
        else return (slot % NSL) * NV;
    }
    __device__ __forceinline__ bool slot_ok(int slot, int s, int nsig) {
        if constexpr (R >= 8) return true;
        else return slot * NT + tid < SIG * NBL && s < nsig;
    }

    // ---------------------------------------------------------- filter
    // Filter spectrum, kept in registers as packed fp16: F = DFT(f) * cF with
    // cF = 2^-e where sum |f| < 2^e.  Every partial sum of the transform is
    // bounded by sum |f|, so inputs scaled by 2^(14 - e) keep the whole
    // transform below 2^14 and F below 1, without a reduction over the
    // spectrum itself.
    template <class LDF>
    __device__ void filter(const LDF &ldf, int nf) {
        cf fin[T0W][4];
        fetch_fp32([&](int, int pos) -> cf { return mk(pos < nf ? ldf(pos) : 0.f, 0.f); }, 0, 1, fin);
        float asum = 0.f;
#pragma unroll
        for (int i = 0; i < T0W; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) asum += fabsf(fin[i][e].x);
        asum = block_reduce<true>(asum);
        int ef = 0;
        if (asum > 0.f) (void)frexpf(asum, &ef);
        const float sf = ldexpf(1.f, 14 - ef);
        cF = ldexpf(1.f, -ef);
        const uint32_t ch = pk(1.0f / 16384.0f, 1.0f / 16384.0f);
        pass0([&](int i, int e) -> uint32_t { return pk(fin[i][e].x * sf, 0.f); });
        fwd_middle<1>(1);
#pragma unroll
        for (int slot = 0; slot < NLS; ++slot) {
            if (R >= 8 || slot < NSL) {
                int s;
                const int pb = lpos(slot, s);
                uint32_t y[NV];
                last_fwd(0, pb, y);
#pragma unroll
                for (int q = 0; q < NV; ++q) F[fslot(slot) + q] = pkmul(y[q], ch);
            }
        }
    }

    // ---------------------------------------------------------- conv round
    template <class OUT>
    __device__ void conv_round(const OUT &out, int nsig, int hb) {
        float amax;
        if constexpr (KIND == IN_F16) {
            h2 am = {(_Float16)0.f, (_Float16)0.f};
#pragma unroll
            for (int i = 0; i < T0W; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    am = __builtin_elementwise_max(am, __builtin_elementwise_abs(__builtin_bit_cast(h2, pin[i][e])));
            amax = fmaxf((float)am.x, (float)am.y);
        } else {
            amax = 0.f;
#pragma unroll
            for (int i = 0; i < T0W; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) amax = fmaxf(amax, in_amax<KIND>(pin[i][e]));
        }
        // fp16 inputs are scaled in fp16, so the scale must be an fp16 power of two
        const float su0 = pow2_scale(block_max(amax), hb);
        const float su = (KIND == IN_F16) ? fminf(su0, 16384.0f) : su0;
        const uint32_t suh = pk(su, su);
        pass0([&](int i, int e) -> uint32_t { return in_scaled<KIND>(pin[i][e], su, suh); });
        fwd_middle<1>(nsig);
        // last pass: spectrum x filter spectrum, held in registers; its maximum
        // sets the scale of the inverse
        uint32_t P[NU][NV];
        float ymax = 0.f;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int slot = u % NLS, s0 = u / NLS;
            int s;
            const int pb = lpos(slot, s);
            if (R >= 8) s = s0;
            if ((R >= 8 && s < nsig) || (R < 8 && slot_ok(slot, s, nsig))) {
                uint32_t y[NV];
                last_fwd(s, pb, y);
#pragma unroll
                for (int q = 0; q < NV; ++q) {
                    P[u][q] = cmulh(y[q], F[fslot(slot) + q]);
                    ymax = fmaxf(ymax, habs_max(P[u][q]));
                }
            }
        }
        // Scale of the inverse: a power of two that keeps every inverse partial
        // sum below 2^15; applied to the fp16 product, so clamped to fp16's exact
        // powers of two (max|Y| < 2^16 bounds it below by 2^-15).
        const float sy = fminf(fmaxf(pow2_scale(block_max(ymax), (LOG2M + 1) / 2), 1.0f / 32768.0f), 16384.0f);
        const uint32_t syh = pk(sy, sy);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int slot = u % NLS, s0 = u / NLS;
            int s;
            const int pb = lpos(slot, s);
            if (R >= 8) s = s0;
            if ((R >= 8 && s < nsig) || (R < 8 && slot_ok(slot, s, nsig))) {
                uint32_t y[NV];
#pragma unroll
                for (int q = 0; q < NV; ++q) y[q] = pkmul(P[u][q], syh);
                last_inv(s, pb, y);
            }
        }
        __syncthreads();
        inv_middle<K>(nsig);
        const float os = 1.0f / ((float)M * su * sy * cF);
        pass0_inv([&](int s, int n, int m, float re, float im) { out(s, n, m, re * os, im * os); }, nsig);
    }

    // A whole channel of 16-bit activations: the filter spectrum, then
    // ceil(nsig / SIG) rounds of complex signals.  ldf(pos) gives the real
    // filter (nf taps); rows(sig) the row pointers of signal `sig`; nval the
    // sequence length.  The inputs of each round are fetched while the
    // previous round (or the filter) is being transformed.
    template <class LDF, class RP>
    __device__ void run_raw(const LDF &ldf, int nf, const RP &rows, int nsig, int nval, int hb) {
        static_assert(KIND == IN_F16 || KIND == IN_BF16, "16-bit activations");
        fetch_raw(rows, 0, min(SIG, nsig), nval, pnx);
        filter(ldf, nf);
        for (int r0 = 0; r0 < nsig; r0 += SIG) {
            const int nr = min(SIG, nsig - r0);
#pragma unroll
            for (int i = 0; i < T0W; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) pin[i][e] = pnx[i][e];
            if (r0 + SIG < nsig) fetch_raw(rows, r0 + SIG, min(SIG, nsig - r0 - SIG), nval, pnx);
            auto out = [&](int s, int n, int m, float re, float im) {
                const int pos = n + m * S0;
                if (pos < nval) {
                    const RowPtrs rp = rows(r0 + s);
                    if constexpr (KIND == IN_F16) {
                        const h2 hv = __builtin_convertvector((f2){re, im}, h2);
                        const _Float16 hre = hv.x, him = hv.y;
                        rp.out0[pos] = __builtin_bit_cast(uint16_t, hre);
                        if (rp.out1) rp.out1[pos] = __builtin_bit_cast(uint16_t, him);
                    } else {
                        rp.out0[pos] = f32_to_bf16_rne(re);
                        if (rp.out1) rp.out1[pos] = f32_to_bf16_rne(im);
                    }
                }
            };
            conv_round(out, nr, hb);
        }
    }

    // Same for fp32 inputs from a loader ld(sig, pos) (zero past the
    // sequence) and a store st(sig, pos, re, im).
    template <class LDF, class LD, class ST>
    __device__ void run_fp32(const LDF &ldf, int nf, const LD &ld, const ST &st, int nsig, int nval, int hb) {
        static_assert(KIND == IN_FP32, "fp32 inputs");
        fetch_fp32(ld, 0, min(SIG, nsig), pnx);
        filter(ldf, nf);
        for (int r0 = 0; r0 < nsig; r0 += SIG) {
            const int nr = min(SIG, nsig - r0);
#pragma unroll
            for (int i = 0; i < T0W; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) pin[i][e] = pnx[i][e];
            if (r0 + SIG < nsig) fetch_fp32(ld, r0 + SIG, min(SIG, nsig - r0 - SIG), pnx);
            auto out = [&](int s, int n, int m, float re, float im) {
                const int pos = n + m * S0;
                if (pos < nval) st(r0 + s, pos, re, im);
            };
            conv_round(out, nr, hb);
        }
    }
};

// ceil(log2(n) / 2) for n >= 1
__device__ __forceinline__ int half_bits(int n) {
    int b = 0;
    while ((1 << b) < n) ++b;
    return (b + 1) / 2;
}

}  // namespace mf
}  // namespace h3c
