// mfma_engine.h -- fused block-FFT convolution engine for fp16/bf16 activations
// on gfx950: the radix-16 (and radix-8) DFT blocks of the transform run as
// dense matrix products on the matrix cores (fp16 operands, fp32
// accumulation); twiddles, scaling and the pointwise product run on the
// vector ALUs in packed fp16; between passes the signal lives in LDS as
// packed fp16 complex.
//
// Method: the paperlayer.ai summary of "Hungry Hungry Hippos", section 4
// (FlashConv: FFT, pointwise product and inverse FFT fused in one kernel; the
// FFT rewritten as small dense matrix products so that it runs on matrix
// units, at the price of more FLOPs), section 2 "Convolutional view" and
// Appendix C.1 (zero-pad to 2N, keep the first N outputs).
//
// Transform of size M = 2^LOG2M = 16 * 16^K * R (R = 2, 4, 8 or 16):
//   pass 0      radix-16 decimation-in-frequency pass on the zero-padded
//               input straight from HBM (only the first 8 points of each
//               16-point column are non-zero): one 32x32x16 MFMA per 32
//               columns, twiddle, to LDS;
//   pass 1..K   radix-16 DIF passes, two 16x16x32 MFMAs per 16 columns, each
//               lane reading and writing back the same four LDS slots;
//   last pass   radix-R DFT of contiguous groups, product with the filter
//               spectrum (held in registers), and the inverse of the same
//               radix straight from registers;
//   inverse     passes K..1 and the inverse of pass 0 (decimation in time),
//               which writes only the first N outputs.
// Spectra stay in digit-reversed order; the filter spectrum goes through the
// same passes, so the pointwise product needs no reordering.  Inverse DFTs use
// the forward matrices: IDFT(x) = conj(DFT(conj(x))); the inverse passes keep
// the signal conjugated, so the conjugations between them cancel and only the
// first (in the product with the filter spectrum) and the last (in the output
// scaling) remain, both free as instruction modifiers.
//
// Range: the activations of each round of signals are scaled by a power of
// two chosen from their maximum so that no fp16 intermediate can overflow
// (|U| <= N max|u| s < 2^15); the filter is scaled from sum |f|, which bounds
// every partial sum of its transform; the spectrum product is rescaled from
// its own maximum before the inverse.  All scales are powers of two and are
// undone exactly at the output.
#pragma once

#include "h3conv_device.h"

namespace h3c {
namespace mf {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ================================================================ constant tables
// DFT matrices and per-thread twiddles are evaluated at compile time (cosine
// and sine from their Taylor series on the first octant, extended by
// symmetry) and stored as packed fp16 (round to nearest even) in read-only
// device memory; a workgroup loads its share with a few coalesced 16-byte
// loads instead of evaluating them.
namespace tab {

constexpr double kPi = 3.14159265358979323846;
constexpr int kBaseLog = 15;
constexpr int kBaseM = 1 << kBaseLog;  // finest root of unity: exp(-2 pi i / 32768)

// cos x and sin x for 0 <= x <= pi/4 (Taylor terms up to x^29)
constexpr void cos_sin_small(double x, double &c, double &s) {
    const double x2 = x * x;
    double tc = 1.0, ts = x;
    c = 0.0;
    s = 0.0;
    for (int n = 0; n < 15; ++n) {
        c += tc;
        s += ts;
        tc *= -x2 / (double)((2 * n + 1) * (2 * n + 2));
        ts *= -x2 / (double)((2 * n + 2) * (2 * n + 3));
    }
}

struct Octant {
    double c[kBaseM / 8 + 1], s[kBaseM / 8 + 1];  // cos, sin of 2 pi r / kBaseM, r <= kBaseM / 8
};
constexpr Octant make_octant() {
    Octant o{};
    for (int r = 0; r <= kBaseM / 8; ++r) cos_sin_small(2.0 * kPi * (double)r / (double)kBaseM, o.c[r], o.s[r]);
    return o;
}
constexpr Octant kOct = make_octant();

constexpr uint32_t pk16(double re, double im) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)re) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)im) << 16);
}

// exp(-2 pi i r / kBaseM) for 0 <= r <= kBaseM / 4, packed fp16 (re low, im high)
struct Quadrant {
    uint32_t v[kBaseM / 4 + 1];
};
constexpr Quadrant make_quadrant() {
    Quadrant t{};
    for (int r = 0; r <= kBaseM / 4; ++r) {
        // cos and sin of the angle from the first octant by symmetry
        const bool lo = r <= kBaseM / 8;
        const int o = lo ? r : kBaseM / 4 - r;
        const double c = lo ? kOct.c[o] : kOct.s[o], s = lo ? kOct.s[o] : kOct.c[o];
        t.v[r] = pk16(c, -s + 0.0);
    }
    return t;
}
constexpr Quadrant kQuad = make_quadrant();

// packed fp16 complex times -i: (re, im) -> (im, -re), exact on the bits
constexpr uint32_t times_neg_i(uint32_t x) {
    uint32_t nre = (x & 0xffffu) ^ 0x8000u;
    if ((nre & 0x7fffu) == 0) nre = 0;  // no negative zero
    return (x >> 16) | (nre << 16);
}

// exp(-2 pi i t / m), packed fp16, for m a power of two dividing kBaseM
constexpr uint32_t wpk(long t, long m) {
    const long u = (t % m + m) % m * (kBaseM / m);  // in [0, kBaseM)
    uint32_t x = kQuad.v[u % (kBaseM / 4)];
    for (long q = u / (kBaseM / 4); q > 0; --q) x = times_neg_i(x);
    return x;
}
// the same, unpacked (exact fp16 values, for the matrix entries)
constexpr void root(long t, long m, double &re, double &im) {
    const uint32_t x = wpk(t, m);
    re = (double)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xffffu));
    im = (double)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
}

// Entry of the real 2R x 2R form of the forward R-point DFT, W = exp(-2 pi i/R):
// output (k, part p) from input (m, part q); parts 0 = re, 1 = im.
constexpr double dft_real(int r, int k, int p, int m, int q) {
    double wr = 0.0, wi = 0.0;
    root((long)k * m, r, wr, wi);
    if (p == 0) return q == 0 ? wr : -wi;
    return q == 0 ? wi : wr;
}

// Chained slot order of a 16-point column in the 16x16x32 layouts: lane
// group g (= lane / 16) holds points 2g + {0, 1, 8, 9}, which is also where
// that group's accumulator rows land, so a pass reads and writes the same
// slots and results feed the next product without reordering.
constexpr int kChain[4] = {0, 1, 8, 9};
constexpr int chain(int g, int t) { return 2 * g + kChain[t]; }
// output point of accumulator pair v (v even) in the 32x32x16 layout, lane half h
constexpr int q32(int v, int h) { return 4 * (v >> 2) + 2 * h + ((v & 3) >> 1); }

// Per-lane matrix operands, as quads [4][64 lanes][4 dwords]:
//   0: 32x32x16 A, zero-padded forward DFT-16: row l%32 -> output (l%32 / 2,
//      part l%2); K slot (l/32, e) -> input 4 (l/32) + e/2, part e%2
//   1, 2: 16x16x32 A, forward DFT-16 outputs 0..7 / 8..15 (row l%16 ->
//      output l%16/2 (+8), part l%2) in chained K order (slot (l/16, e) ->
//      input chain(l/16, e/2), part e%2)
//   3: 16x16x16 A, forward DFT-8 (row l%16 -> output l%16/2, part l%2; slot
//      (l/16, e) -> input 2 (l/16) + e/2, part e%2), dwords 2, 3 zero
struct MatTab {
    uint32_t q[4][64][4];
};
constexpr MatTab make_mat() {
    MatTab t{};
    for (int l = 0; l < 64; ++l) {
        const int i32 = l & 31, g32 = l >> 5, j = l & 15, g = l >> 4;
        for (int e = 0; e < 8; e += 2) {
            double a[2] = {0.0, 0.0}, c0[2] = {0.0, 0.0}, c1[2] = {0.0, 0.0};
            for (int h = 0; h < 2; ++h) {
                const int q = (e + h) & 1;
                a[h] = dft_real(16, i32 >> 1, i32 & 1, 4 * g32 + ((e + h) >> 1), q);
                const int mc = chain(g, (e + h) >> 1);
                c0[h] = dft_real(16, j >> 1, j & 1, mc, q);
                c1[h] = dft_real(16, 8 + (j >> 1), j & 1, mc, q);
            }
            t.q[0][l][e / 2] = pk16(a[0], a[1]);
            t.q[1][l][e / 2] = pk16(c0[0], c0[1]);
            t.q[2][l][e / 2] = pk16(c1[0], c1[1]);
        }
        for (int e = 0; e < 4; e += 2) {
            const int m = 2 * g + (e >> 1);
            t.q[3][l][e / 2] = pk16(dft_real(8, j >> 1, j & 1, m, 0), dft_real(8, j >> 1, j & 1, m, 1));
        }
    }
    return t;
}
__device__ const MatTab kMat = make_mat();

}  // namespace tab

// ================================================================ packed fp16 complex
// Written as plain vector code: the compiler emits v_cvt_pk_f16_f32 (round
// to nearest even) and v_pk_mul_f16 / v_pk_fma_f16 with op_sel / neg
// modifiers, and it knows their hazards against the matrix-core results they
// consume.

__device__ __forceinline__ uint32_t pk(float re, float im) {
    const f2 v = {re, im};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
}
// x * w and conj(x) * w on packed fp16 complex, two instructions each with
// the half selection and negation in op_sel / neg modifiers.  Written as
// instructions so that the twiddle operand stays as it is: as plain vector
// code the compiler hoists the swapped copy of a loop-invariant twiddle out
// of every loop and keeps both copies in registers.  Their operands are
// never matrix-core results directly (those pass through a compiler-emitted
// conversion first).  conj(x) * w feeds matrix-core operands, and the
// compiler does not insert the wait states between a vector write and a
// matrix-core read for an instruction it did not emit, so that variant works
// on a whole operand at once and ends with its own.
__device__ __forceinline__ uint32_t cmulh(uint32_t x, uint32_t w) {
    uint32_t t, r;
    asm("v_pk_mul_f16 %0, %1, %2 op_sel_hi:[0,1]" : "=v"(t) : "v"(x), "v"(w));
    asm("v_pk_fma_f16 %0, %1, %2, %3 op_sel:[1,1,0] op_sel_hi:[1,0,1] neg_lo:[1,0,0]"
        : "=v"(r) : "v"(x), "v"(w), "v"(t));
    return r;
}
// conj(x[i]) * w[i] for the N operand dwords of one matrix-core product, in
// one block so that the wait states at its end cover every result.
template <int N>
__device__ __forceinline__ void cmulh_cx_n(uint32_t (&x)[N], const uint32_t (&w)[N]) {
    static_assert(N == 2 || N == 4, "two or four operand dwords");
    uint32_t t[N];
    if constexpr (N == 4) {
        asm("v_pk_mul_f16 %4, %0, %8 op_sel_hi:[0,1]\n\t"
            "v_pk_mul_f16 %5, %1, %9 op_sel_hi:[0,1]\n\t"
            "v_pk_mul_f16 %6, %2, %10 op_sel_hi:[0,1]\n\t"
            "v_pk_mul_f16 %7, %3, %11 op_sel_hi:[0,1]\n\t"
            "v_pk_fma_f16 %0, %0, %8, %4 op_sel:[1,1,0] op_sel_hi:[1,0,1] neg_hi:[1,0,0]\n\t"
            "v_pk_fma_f16 %1, %1, %9, %5 op_sel:[1,1,0] op_sel_hi:[1,0,1] neg_hi:[1,0,0]\n\t"
            "v_pk_fma_f16 %2, %2, %10, %6 op_sel:[1,1,0] op_sel_hi:[1,0,1] neg_hi:[1,0,0]\n\t"
            "v_pk_fma_f16 %3, %3, %11, %7 op_sel:[1,1,0] op_sel_hi:[1,0,1] neg_hi:[1,0,0]\n\t"
            "s_nop 4"
            : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3])
            : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]));
    } else {
        asm("v_pk_mul_f16 %2, %0, %4 op_sel_hi:[0,1]\n\t"
            "v_pk_mul_f16 %3, %1, %5 op_sel_hi:[0,1]\n\t"
            "v_pk_fma_f16 %0, %0, %4, %2 op_sel:[1,1,0] op_sel_hi:[1,0,1] neg_hi:[1,0,0]\n\t"
            "v_pk_fma_f16 %1, %1, %5, %3 op_sel:[1,1,0] op_sel_hi:[1,0,1] neg_hi:[1,0,0]\n\t"
            "s_nop 4"
            : "+v"(x[0]), "+v"(x[1]), "=&v"(t[0]), "=&v"(t[1])
            : "v"(w[0]), "v"(w[1]));
    }
}
// x[i] * w[i] for the N operand dwords of one matrix-core product (the same
// layout and closing wait states as above).
template <int N>
__device__ __forceinline__ void cmulh_n(uint32_t (&x)[N], const uint32_t (&w)[N]) {
    static_assert(N == 2 || N == 4, "two or four operand dwords");
    uint32_t t[N];
    if constexpr (N == 4) {
        asm("v_pk_mul_f16 %4, %0, %8 op_sel_hi:[0,1]\n\t"
            "v_pk_mul_f16 %5, %1, %9 op_sel_hi:[0,1]\n\t"
            "v_pk_mul_f16 %6, %2, %10 op_sel_hi:[0,1]\n\t"
            "v_pk_mul_f16 %7, %3, %11 op_sel_hi:[0,1]\n\t"
            "v_pk_fma_f16 %0, %0, %8, %4 op_sel:[1,1,0] op_sel_hi:[1,0,1] neg_lo:[1,0,0]\n\t"
            "v_pk_fma_f16 %1, %1, %9, %5 op_sel:[1,1,0] op_sel_hi:[1,0,1] neg_lo:[1,0,0]\n\t"
            "v_pk_fma_f16 %2, %2, %10, %6 op_sel:[1,1,0] op_sel_hi:[1,0,1] neg_lo:[1,0,0]\n\t"
            "v_pk_fma_f16 %3, %3, %11, %7 op_sel:[1,1,0] op_sel_hi:[1,0,1] neg_lo:[1,0,0]\n\t"
            "s_nop 4"
            : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3])
            : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]));
    } else {
        asm("v_pk_mul_f16 %2, %0, %4 op_sel_hi:[0,1]\n\t"
            "v_pk_mul_f16 %3, %1, %5 op_sel_hi:[0,1]\n\t"
            "v_pk_fma_f16 %0, %0, %4, %2 op_sel:[1,1,0] op_sel_hi:[1,0,1] neg_lo:[1,0,0]\n\t"
            "v_pk_fma_f16 %1, %1, %5, %3 op_sel:[1,1,0] op_sel_hi:[1,0,1] neg_lo:[1,0,0]\n\t"
            "s_nop 4"
            : "+v"(x[0]), "+v"(x[1]), "=&v"(t[0]), "=&v"(t[1])
            : "v"(w[0]), "v"(w[1]));
    }
}
// both halves times the matching halves of a packed factor
__device__ __forceinline__ uint32_t pkmul(uint32_t xx, uint32_t ss) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, xx) * __builtin_bit_cast(h2, ss));
}
__device__ __forceinline__ half8 as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const u32x4 v = {a, b, c, d};
    return __builtin_bit_cast(half8, v);
}
__device__ __forceinline__ half4 as_half4(uint32_t a, uint32_t b) {
    const u32x2 v = {a, b};
    return __builtin_bit_cast(half4, v);
}
// max(|re|, |im|) of a packed fp16 complex, as fp32
__device__ __forceinline__ float habs_max(uint32_t v) {
    const h2 a = __builtin_elementwise_abs(__builtin_bit_cast(h2, v));
    return (float)__builtin_elementwise_max(a.x, a.y);
}

// Shared-memory index swizzle for packed-complex dwords, per transform size:
// bit p >= 6 of an index, when set, flips the bits kSwz[LOG2M][p - 6] among
// bits 1..5, and bit 5 flips the bits kSwz5[LOG2M] among bits 1..4, so
// strided operand gathers and the contiguous last-pass groups spread over the
// banks (masks chosen by a search over this engine's access patterns, every
// wave of a workgroup, against 32- and 64-bank models; bit 0, and bit 1 where
// the last pass reads four dwords at once, are never flipped, so the groups a
// lane reads with one access stay contiguous).  Indices below 32 map to
// themselves: a lane's column within a 32-column tile is used as is.  The map is linear over XOR, so
// phys(a ^ b) = phys(a) ^ phys(b); addresses are split that way into
// per-lane and compile-time parts.
constexpr int kSwz[16][9] = {
    {}, {}, {}, {}, {}, {}, {}, {}, {},
    {48, 18, 16},                        // 9
    {4, 48, 16, 32},                     // 10
    {4, 8, 48, 32, 16},                  // 11
    {24, 4, 16, 48, 16, 32},             // 12
    {16, 34, 16, 32, 48, 32, 16},        // 13
    {4, 48, 16, 32, 16, 48, 16, 32},     // 14
    {4, 48, 16, 32, 16, 48, 16, 32, 48}, // 15 (the 2^14 pattern, one bit more)
};
constexpr int kSwz5[16] = {0, 0, 0, 0, 0, 0, 0, 0, 0, 8, 0, 0, 16, 8, 0, 0};
template <int LOG2M>
__host__ __device__ constexpr int phys(int i) {
    int r = (i >> 5) & 1 ? i ^ kSwz5[LOG2M] : i;
    for (int p = 6; p < LOG2M; ++p)
        if ((i >> p) & 1) r ^= kSwz[LOG2M][p - 6];
    return r;
}

// Workgroup shape per transform size: SIG signals in flight, NW waves.
template <int LOG2M> struct Cfg;
// OCC = workgroups per compute unit the register budget is set for; BD =
// most dwords a lane reads from LDS ahead of the first write in a pass.
template <> struct Cfg<9> { static constexpr int SIG = 8, NW = 2, OCC = 4, BD = 16; };
template <> struct Cfg<10> { static constexpr int SIG = 4, NW = 4, OCC = 4, BD = 16; };
template <> struct Cfg<11> { static constexpr int SIG = 4, NW = 8, OCC = 3, BD = 8; };
template <> struct Cfg<12> { static constexpr int SIG = 2, NW = 8, OCC = 2, BD = 16; };
template <> struct Cfg<13> { static constexpr int SIG = 1, NW = 8, OCC = 2, BD = 16; };
template <> struct Cfg<14> { static constexpr int SIG = 1, NW = 8, OCC = 2, BD = 16; };
// 2N = 32768 (sequences up to 16K in one fused block): one signal of 128 KiB
// in LDS per workgroup, one workgroup per compute unit
template <> struct Cfg<15> { static constexpr int SIG = 1, NW = 8, OCC = 1, BD = 16; };

// Shape variant V = 1 (2N <= 4096): half the signals per round with half the
// waves, about twice the workgroups per compute unit (the same work per
// wave), for batches that fill at most half a round.  At 2N = 2048 a wave
// of the half shape holds 8 more registers (its share of the filter
// spectrum and of the inverse twiddles doubles), so it is set for 5
// workgroups (20 waves) rather than 6.
template <int LOG2M, int V> struct CfgV {
    static_assert(V == 0 || (Cfg<LOG2M>::SIG >= 2 && Cfg<LOG2M>::NW >= 2), "no half shape for this size");
    static constexpr int SIG = V ? Cfg<LOG2M>::SIG / 2 : Cfg<LOG2M>::SIG;
    static constexpr int NW = V ? Cfg<LOG2M>::NW / 2 : Cfg<LOG2M>::NW;
    static constexpr int OCC = V ? (LOG2M == 11 ? 5 : 2 * Cfg<LOG2M>::OCC) : Cfg<LOG2M>::OCC;
    static constexpr int BD = Cfg<LOG2M>::BD;
};

template <int LOG2M, int V = 0>
struct Shape {
    static constexpr int M = 1 << LOG2M;
    static constexpr int K = (LOG2M - 5) / 4;          // middle radix-16 passes
    static constexpr int LR = LOG2M - 4 - 4 * K;       // log2 of the last radix
    static constexpr int R = 1 << LR;
    static constexpr int S0 = M / 16;                  // pass-0 columns per signal
    static constexpr int SIG = CfgV<LOG2M, V>::SIG, NW = CfgV<LOG2M, V>::NW, NT = 64 * NW, OCC = CfgV<LOG2M, V>::OCC;
    static constexpr int BD = CfgV<LOG2M, V>::BD;
    static constexpr int WPE = (OCC * NW + 3) / 4;     // waves per SIMD at that occupancy
    static constexpr int T0 = SIG * S0 / 32;           // pass-0 tiles (32 columns) per round
    static constexpr int T0W = T0 / NW;
    static constexpr int TI = SIG * S0 / 16;           // inverse pass-0 tiles (16 columns)
    static constexpr int TIW = TI / NW;
    static constexpr int TM = M / 256;                 // middle-pass tiles per signal
    static constexpr int TPW = TM / NW;
    static constexpr int TL8 = M / 128;                // radix-8 last-pass tiles per signal
    static constexpr int T8W = TL8 / NW;
    static constexpr int NBL = M / R;                  // radix-2/4 last-pass butterflies per signal
    static constexpr int NSL = (NBL > NT) ? NBL / NT : 1;            // distinct positions per thread
    static constexpr int BPTL = (SIG * NBL + NT - 1) / NT;           // butterflies per thread
    // The filter is transformed together with the first round's signals, in
    // a signal slot of its own, when that slot fits the LDS budget of OCC
    // workgroups per compute unit (160 KiB); otherwise it is transformed on
    // its own first, in the signals' slots.
    static constexpr int PAD = 16;                     // dwords after each signal slot
    static constexpr bool FUSEF = ((SIG + 1) * (M + PAD) + 64) * 4 * OCC <= 160 * 1024;
    static constexpr int DATA = (SIG + (FUSEF ? 1 : 0)) * (M + PAD);
    // Reduction slots (after the signal data, two alternating banks): per
    // round, the per-signal input maxima (one slot per pass-0 tile, or per
    // wave when a round holds one signal) and the filter sums of the waves.
    static constexpr int NSLOT = SIG == 1 ? NW : T0;
    static constexpr int RBK = ((NSLOT + NW > 2 * NW ? NSLOT + NW : 2 * NW) + 3) / 4 * 4;  // 16-byte banks
    static_assert(2 * RBK <= 64, "two reduction banks fit the 64 slots");
    // With several signals per round, the pass-0 tiles of one wave belong to
    // different signals (32 NW columns >= one signal's S0 columns).
    static_assert(SIG == 1 || 32 * NW >= S0, "a wave's pass-0 tiles cover distinct signals");
    static constexpr int LDS_DWORDS = DATA + 64;
    static constexpr int DELTA = 256 * NW;             // butterfly-base step between a wave's tiles
    // distinct column offsets a thread meets in pass 0 (32-column tiles) and
    // in its inverse (16-column tiles)
    static constexpr int ND0 = S0 > 32 * NW ? S0 / (32 * NW) : 1;
    static constexpr int NDI = S0 > 16 * NW ? S0 / (16 * NW) : 1;
    // per-thread twiddle quads: pass 0 (2 per offset), inverse pass 0, middle passes
    static constexpr int Q_TU = 2 * ND0, Q_MID = 2 * ND0 + NDI, NQ = 2 * ND0 + NDI + K;
    static constexpr bool TWREG = 4 * NQ <= 24;        // twiddles held in registers
    static_assert(S0 >= 32, "pass-0 tiles must lie within one signal");
    static_assert(K >= 1, "the inverse scale is applied by the first inverse middle pass");
    static_assert(T0 % NW == 0 && TI % NW == 0, "pass-0 tiles must split evenly over waves");
    static_assert(K == 0 || TM % NW == 0, "middle tiles must split evenly over waves");
    static_assert(R != 8 || TL8 % NW == 0, "radix-8 tiles must split evenly over waves");
    static_assert(R > 4 || NBL % NT == 0 || NT % NBL == 0, "radix-2/4 butterflies must tile the threads");
    static_assert(M <= 256 * 16 * NW, "a lane must see one column offset per middle pass");
    __host__ __device__ static constexpr int L(int p) { return M >> (4 * p); }  // p = 1..K
};

namespace tab {
// Per-thread twiddles of one transform size, as quads [NQ][NT][4]:
//   2d, 2d+1   pass 0, offset d: w_M^(n q) for this lane's 8 outputs q = q32(v, h)
//   Q_TU + d   inverse pass 0, offset d: w_M^(n k), k = chain(g, 0..3)
//   Q_MID + p  middle pass p+1 (length L, stride S = L/16): w_L^(n k), k = chain(g, 0..3)
template <int LOG2M, int V>
struct TwTab {
    uint32_t q[Shape<LOG2M, V>::NQ][Shape<LOG2M, V>::NT][4];
};
template <int LOG2M, int V>
constexpr TwTab<LOG2M, V> make_tw() {
    using SH = Shape<LOG2M, V>;
    TwTab<LOG2M, V> t{};
    for (int tid = 0; tid < SH::NT; ++tid) {
        const int w = tid >> 6, lane = tid & 63, j = lane & 15, g = lane >> 4;
        for (int d = 0; d < SH::ND0; ++d) {
            const long n = (32 * (w + d * SH::NW) + (lane & 31)) % SH::S0;
            for (int v = 0; v < 16; v += 2)
                t.q[2 * d + (v >> 3)][tid][(v >> 1) & 3] = wpk(n * q32(v, lane >> 5), SH::M);
        }
        for (int d = 0; d < SH::NDI; ++d) {
            const long n = (16 * (w + d * SH::NW) + j) % SH::S0;
            for (int c = 0; c < 4; ++c) t.q[SH::Q_TU + d][tid][c] = wpk(n * chain(g, c), SH::M);
        }
        for (int p = 1; p <= SH::K; ++p) {
            const int L = SH::L(p), S = L / 16;
            const long n = (16 * w + j) % S;
            for (int c = 0; c < 4; ++c) t.q[SH::Q_MID + p - 1][tid][c] = wpk(n * chain(g, c), L);
        }
    }
    return t;
}
template <int LOG2M, int V = 0>
__device__ const TwTab<LOG2M, V> kTw = make_tw<LOG2M, V>();
}  // namespace tab

// ================================================================ helpers

// Wave-wide max (SUM = false) or sum of a non-negative value with DPP row
// operations (no LDS round trips): pairs and quads, half-row and row
// mirrors, then the row broadcasts; the result is in lane 63.  The max works
// on the bit patterns as integers (the same order for non-negative floats),
// with 0 as the identity, so that the full-row steps become one max
// instruction with a DPP source operand.
template <int CTRL, int RMASK>
__device__ __forceinline__ int dpp_max_step(int x) {
    return max(x, __builtin_amdgcn_update_dpp(0, x, CTRL, RMASK, 0xf, false));
}
template <int CTRL, int RMASK>
__device__ __forceinline__ float dpp_sum_step(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, RMASK, 0xf, false));
}
template <bool SUM>
__device__ __forceinline__ float wave_reduce(float v) {
    // quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror,
    // row_bcast:15 (rows 1, 3), row_bcast:31 (rows 2, 3)
    if constexpr (SUM) {
        v = dpp_sum_step<0xb1, 0xf>(v);
        v = dpp_sum_step<0x4e, 0xf>(v);
        v = dpp_sum_step<0x141, 0xf>(v);
        v = dpp_sum_step<0x140, 0xf>(v);
        v = dpp_sum_step<0x142, 0xa>(v);
        v = dpp_sum_step<0x143, 0xc>(v);
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
    } else {
        int x = __builtin_bit_cast(int, v);
        x = dpp_max_step<0xb1, 0xf>(x);
        x = dpp_max_step<0x4e, 0xf>(x);
        x = dpp_max_step<0x141, 0xf>(x);
        x = dpp_max_step<0x140, 0xf>(x);
        x = dpp_max_step<0x142, 0xa>(x);
        x = dpp_max_step<0x143, 0xc>(x);
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(x, 63));
    }
}
__device__ __forceinline__ float wave_max(float v) { return wave_reduce<false>(v); }
__device__ __forceinline__ float wave_sum(float v) { return wave_reduce<true>(v); }

// Max of two pairs of 16-bit magnitudes, half by half.  The bit patterns of
// non-negative fp16 or bf16 values order like the values themselves, so the
// pairs are compared as unsigned 16-bit integers.
__device__ __forceinline__ uint32_t pkmax_u16(uint32_t a, uint32_t b) {
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, a), __builtin_bit_cast(us2, b)));
}
template <int CTRL, int RMASK>
__device__ __forceinline__ uint32_t dpp_pkmax_step(uint32_t x) {
    return pkmax_u16(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, RMASK, 0xf, false));
}
// wave-wide half-by-half max of packed 16-bit magnitudes (same DPP steps as
// wave_reduce; 0 is the identity), wave-uniform result
__device__ __forceinline__ uint32_t wave_pkmax(uint32_t x) {
    x = dpp_pkmax_step<0xb1, 0xf>(x);
    x = dpp_pkmax_step<0x4e, 0xf>(x);
    x = dpp_pkmax_step<0x141, 0xf>(x);
    x = dpp_pkmax_step<0x140, 0xf>(x);
    x = dpp_pkmax_step<0x142, 0xa>(x);
    x = dpp_pkmax_step<0x143, 0xc>(x);
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Power-of-two scale 2^(8 - e - hb) where amax < 2^e: after a transform that
// can grow magnitudes by at most 2^(2 hb), values stay below 2^(8 + hb).
__device__ __forceinline__ float pow2_scale(float amax, int hb) {
    int e = 0;
    if (amax > 0.f) (void)frexpf(amax, &e);
    return ldexpf(1.f, 8 - e - hb);
}

// opaque copy: keeps lane-derived indices from being hoisted (and held in
// registers) across the whole kernel
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// opaque copy of a wave-uniform value (kept in scalar registers)
__device__ __forceinline__ uint32_t opaque_u32(uint32_t x) {
    asm volatile("" : "+s"(x));
    return x;
}

// ceil(log2(n) / 2) for n >= 1
__device__ __forceinline__ int half_bits(int n) {
    int b = 0;
    while ((1 << b) < n) ++b;
    return (b + 1) / 2;
}

// How a round's inputs arrive: IN_F16 / IN_BF16 = two 16-bit activations
// packed in a dword (real part low half, imaginary part high half); IN_FP32 =
// a complex value in fp32 (used when the loader computes its input).
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
// scaled packed fp16 operand value: the real half times s.x, the imaginary
// half times s.y; `sh` is the same pair as packed fp16
template <int KIND>
__device__ __forceinline__ uint32_t in_scaled(const typename InT<KIND>::T &x, f2 s, uint32_t sh) {
    if constexpr (KIND == IN_F16) return pkmul(x, sh);
    else if constexpr (KIND == IN_BF16) return pk(__uint_as_float(x << 16) * s.x, __uint_as_float(x & 0xffff0000u) * s.y);
    else return pk(x.x * s.x, x.y * s.y);
}

// Rows of one complex signal for the 16-bit activation kinds, as raw buffer
// resources (base in scalar registers, 32-bit per-lane offsets): in0/out0
// carry the real part, in1/out1 the imaginary part.  The byte extent of each
// resource is the valid part of its row, so loads past it return zero (the
// zero padding of the transform) and stores past it are dropped; a signal
// with one row gets empty in1/out1.
// Cache policy of the activation loads and stores: non-temporal (each value
// is read or written once), so they do not displace the tables and filters
// in L2 and leave no dirty lines in it for the end of the kernel to write back.
constexpr int kNT = 2;

// Wave priorities (s_setprio).  The instruction arbiter otherwise favours
// the oldest waves, so the workgroups sharing a compute unit run one after
// the other: the last one works alone at the end, too few waves to keep the
// unit busy.  A wave runs at kPrioLoad from its start (through the filter
// transform, where that comes first) or the start of a round until pass 0
// has consumed the round's inputs, then at kPrioWork:
// a younger workgroup gets its loads out and its first pass done ahead of
// the older ones' later passes, and the workgroups of a unit stay closer
// together.
constexpr int kPrioLoad = 3, kPrioWork = 2;
struct RowBufs {
    __amdgpu_buffer_rsrc_t in0, in1, out0, out1;
};
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void *p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, 0x00020000);
}

// ================================================================ engine

template <int LOG2M, int KIND, int VAR = 0>
struct Engine {
    using SH = Shape<LOG2M, VAR>;
    using IT = typename InT<KIND>::T;
    static constexpr int M = SH::M, K = SH::K, R = SH::R, S0 = SH::S0, SIG = SH::SIG, NW = SH::NW,
                         NT = SH::NT, T0W = SH::T0W, TIW = SH::TIW, TPW = SH::TPW, T8W = SH::T8W,
                         NBL = SH::NBL, NSL = SH::NSL, BPTL = SH::BPTL, DELTA = SH::DELTA,
                         ND0 = SH::ND0, NDI = SH::NDI;
    static constexpr bool TWREG = SH::TWREG;
    static constexpr int KM = K > 0 ? K : 1;
    static constexpr int FN = R == 16 ? TPW * 4 : (R == 8 ? T8W * 2 : NSL * R);  // filter values / lane
    static constexpr int NV = R == 16 ? 4 : (R == 8 ? 2 : R);                     // values per last-pass slot
    static constexpr int NLS = R == 16 ? TPW : (R == 8 ? T8W : BPTL);            // slots per round
    static constexpr int NU = R >= 8 ? SIG * NLS : NLS;                           // (signal, slot) units

    uint32_t *data;  // [SIG][M] packed complex (swizzled)
    float *red;      // [2][NW] reduction slots
    int tid, w, lane, j, g;
    __amdgpu_buffer_rsrc_t twr;             // the twiddle table
    int two;                                // this thread's byte offset in it
    half8 A0, C0, C1;                       // DFT-16: zero-padded 32x32x16; chained 16x16x32
    half4 A8;                               // DFT-8: 16x16x16
    uint32_t tw0[TWREG ? ND0 : 1][8];       // pass-0 twiddles (when held in registers)
    uint32_t tu0[TWREG ? NDI : 1][4];       // inverse pass-0 twiddles
    // middle-pass twiddles: always in registers (4 K dwords; each is used by
    // a forward and an inverse pass, and a table load at a pass's start
    // would put its latency on the critical path)
    static constexpr bool MIDREG = true;
    uint32_t twm[KM][4];
    uint32_t F[FN];                         // filter spectrum * cF (packed fp16)
    float cF;
    // Inputs of the next round are fetched during the current one, unless
    // twiddles come from the table: loads retire in order, so every table
    // load would then also wait for the whole prefetch.
    static constexpr bool PREFETCH = TWREG;
    IT pin[T0W][4];  // pass-0 operands of the current (or, prefetched, the next) round
    int rbank = 0;

    __device__ Engine(uint32_t *smem) {
        data = smem;
        red = (float *)(smem + SH::DATA);
        tid = threadIdx.x;
        // (masked so the compiler knows w < NW: with the launch's NT threads it
        //  changes nothing, and tile-to-signal maps become compile-time)
        w = __builtin_amdgcn_readfirstlane(tid >> 6) & (NW - 1);
        lane = tid & 63;
        j = lane & 15;
        g = lane >> 4;
    }

    // Quad c of this thread's twiddles.  The offset goes through an opaque
    // copy so that a load stays where it is used: the table is the same for
    // every round, and the compiler would otherwise hoist the loads out of
    // the round loop and hold (or spill) all of them throughout.
    __device__ __forceinline__ u32x4 tq(int c) const {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(twr, opaque(two), c * NT * 16, 0));
    }

    __device__ void init() {
        const u32x4 *mt = (const u32x4 *)&tab::kMat.q[0][0][0];
        A0 = __builtin_bit_cast(half8, mt[lane]);
        C0 = __builtin_bit_cast(half8, mt[64 + lane]);
        C1 = __builtin_bit_cast(half8, mt[128 + lane]);
        if constexpr (R == 8) {
            const u32x4 a = mt[192 + lane];
            const uint32_t a0 = a.x, a1 = a.y;
            A8 = as_half4(a0, a1);
        }
        twr = row_rsrc(&tab::kTw<LOG2M, VAR>.q[0][0][0], (int)sizeof(tab::TwTab<LOG2M, VAR>));
        two = tid * 16;
        if constexpr (TWREG) {
#pragma unroll
            for (int d = 0; d < ND0; ++d) {
                const u32x4 a = tq(2 * d), b = tq(2 * d + 1);
                tw0[d][0] = a.x; tw0[d][1] = a.y; tw0[d][2] = a.z; tw0[d][3] = a.w;
                tw0[d][4] = b.x; tw0[d][5] = b.y; tw0[d][6] = b.z; tw0[d][7] = b.w;
            }
#pragma unroll
            for (int d = 0; d < NDI; ++d) {
                const u32x4 a = tq(SH::Q_TU + d);
                tu0[d][0] = a.x; tu0[d][1] = a.y; tu0[d][2] = a.z; tu0[d][3] = a.w;
            }
        }
        if constexpr (MIDREG) {
#pragma unroll
            for (int p = 0; p < K; ++p) {
                const u32x4 a = tq(SH::Q_MID + p);
                twm[p][0] = a.x; twm[p][1] = a.y; twm[p][2] = a.z; twm[p][3] = a.w;
            }
        }
    }

    // twiddle accessors (registers, or the table in read-only memory)
    __device__ __forceinline__ void get_tw0(int d, uint32_t (&t)[8]) const {
        if constexpr (TWREG) {
#pragma unroll
            for (int v = 0; v < 8; ++v) t[v] = tw0[d][v];
        } else {
            const u32x4 a = tq(2 * d), b = tq(2 * d + 1);
            t[0] = a.x; t[1] = a.y; t[2] = a.z; t[3] = a.w;
            t[4] = b.x; t[5] = b.y; t[6] = b.z; t[7] = b.w;
        }
    }
    __device__ __forceinline__ void get_tu0(int d, uint32_t (&t)[4]) const {
        if constexpr (TWREG) {
#pragma unroll
            for (int c = 0; c < 4; ++c) t[c] = tu0[d][c];
        } else {
            const u32x4 a = tq(SH::Q_TU + d);
            t[0] = a.x; t[1] = a.y; t[2] = a.z; t[3] = a.w;
        }
    }
    __device__ __forceinline__ void get_twm(int p, uint32_t (&t)[4]) const {
        if constexpr (MIDREG) {
#pragma unroll
            for (int c = 0; c < 4; ++c) t[c] = twm[p][c];
        } else {
            const u32x4 a = tq(SH::Q_MID + p);
            t[0] = a.x; t[1] = a.y; t[2] = a.z; t[3] = a.w;
        }
    }

    // Workgroup max (SUM = false) or sum (SUM = true).  Two alternating slot
    // banks (of 2 NW floats, room for the joint reduction below): a wave can
    // only write a bank again after the next reduction's barrier, which every
    // wave reaches only after reading that bank.
    static constexpr int NSLOT = SH::NSLOT, RBK = SH::RBK;

    template <bool SUM>
    __device__ float block_reduce(float v) {
        v = SUM ? wave_sum(v) : wave_max(v);
        float *r = red + rbank * RBK;
        rbank ^= 1;
        if (lane == 0) r[w] = v;
        __syncthreads();
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) m = SUM ? m + r[i] : fmaxf(m, r[i]);
        return m;
    }

    // Workgroup sum of a and max of b with one barrier (same bank scheme).
    __device__ f2 block_reduce_sm(float a, float b) {
        a = wave_sum(a);
        b = wave_max(b);
        float *r = red + rbank * RBK;
        rbank ^= 1;
        if (lane == 0) {
            r[w] = a;
            r[NW + w] = b;
        }
        __syncthreads();
        float sa = 0.f, mb = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            sa += r[i];
            mb = fmaxf(mb, r[NW + i]);
        }
        return f2{sa, mb};
    }

    // Input scales of a round, one per row: each signal's real and imaginary
    // halves are different rows.  round_exps (below) reduces the per-half
    // maxima of the round's inputs (as 16-bit bit patterns) with one barrier;
    // exps_of then gives kp[i] = scale exponents (real, imaginary half) of
    // the signal of pass-0 tile i and kq[i] those of inverse pass-0 tile i
    // (see scale_exp).
    __device__ __forceinline__ void exps_of(uint32_t kpk, int (&kp)[T0W][2], int (&kq)[TIW][2]) {
        auto get = [&](int (&k)[2], int sg) {
            const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)kpk, sg);
            k[0] = lo16(v);
            k[1] = hi16(v);
        };
#pragma unroll
        for (int i = 0; i < T0W; ++i) get(kp[i], SIG == 1 ? 0 : tile_sig(i));
#pragma unroll
        for (int i = 0; i < TIW; ++i) get(kq[i], SIG == 1 ? 0 : (16 * (w + i * NW)) / S0);
    }
    __device__ __forceinline__ static int lo16(uint32_t v) { return (int)(int16_t)(uint16_t)(v & 0xffffu); }
    __device__ __forceinline__ static int hi16(uint32_t v) { return (int)v >> 16; }

    // The reduction behind the round scales: returns, in lane l < SIG, the two
    // scale exponents of signal l (real half in the low 16 bits, imaginary
    // half in the high 16 bits); with FILT, fs (the filter's |f| of this
    // thread) becomes the workgroup's sum.  The exponents are read from the
    // slots right after the barrier, so the bank can be written again two
    // reductions later.
    template <bool FILT>
    __device__ uint32_t round_exps(float &fs, int hb) {
        uint32_t tm[T0W];
#pragma unroll
        for (int i = 0; i < T0W; ++i) {
            uint32_t m = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) m = pkmax_u16(m, pin[i][e] & 0x7fff7fffu);
            tm[i] = m;
        }
        if constexpr (SIG == 1) {
#pragma unroll
            for (int i = 1; i < T0W; ++i) tm[0] = pkmax_u16(tm[0], tm[i]);
        }
        constexpr int NR = SIG == 1 ? 1 : T0W;
#pragma unroll
        for (int i = 0; i < NR; ++i) tm[i] = wave_pkmax(tm[i]);
        if constexpr (FILT) fs = wave_sum(fs);
        uint32_t *r = (uint32_t *)(red + rbank * RBK);
        rbank ^= 1;
        if (lane == 0) {
            // slot of tile i of wave w: its pass-0 tile index w + i NW, whose
            // signal is 32 (w + i NW) / S0 (with one signal: the wave)
#pragma unroll
            for (int i = 0; i < NR; ++i) r[SIG == 1 ? w : w + i * NW] = tm[i];
            if constexpr (FILT) ((float *)r)[NSLOT + w] = fs;
        }
        __syncthreads();
        // lane l < SIG: the maximum of signal l over its slots and its two
        // scale exponents (all signals at once), packed as two 16-bit fields;
        // each tile then takes its signal's pair with one readlane
        constexpr int PER = NSLOT / SIG;
        uint32_t m = 0;
        {
            const uint32_t *q = r + (lane < SIG ? lane : 0) * PER;
            if constexpr (PER % 4 == 0) {
#pragma unroll
                for (int k = 0; k < PER; k += 4) {
                    const u32x4 v = *(const u32x4 *)(q + k);
                    const uint32_t v0 = v.x, v1 = v.y, v2 = v.z, v3 = v.w;
                    m = pkmax_u16(m, pkmax_u16(pkmax_u16(v0, v1), pkmax_u16(v2, v3)));
                }
            } else {
#pragma unroll
                for (int k = 0; k < PER; ++k) m = pkmax_u16(m, q[k]);
            }
        }
        const uint32_t kpk = ((uint32_t)scale_exp(m & 0xffffu, hb) & 0xffffu) | ((uint32_t)scale_exp(m >> 16, hb) << 16);
        if constexpr (FILT) {
            float sa = 0.f;
#pragma unroll
            for (int k = 0; k < NW; ++k) sa += ((const float *)r)[NSLOT + k];
            fs = sa;
        }
        return kpk;
    }

    // Scale exponents.  For a 16-bit magnitude pattern m > 0 of the input
    // type, mag_exp(m) = e with 2^(e-1) <= |x| < 2^e (normal and subnormal
    // fp16 / bf16; an inf or NaN pattern counts as 2^129).  The input scale of
    // a row is 2^k with k = 8 - e - hb (the old float form of this was
    // pow2_scale), limited to the fp16 range for fp16 inputs (which are
    // scaled in fp16) and to the normal fp32 range otherwise; an all-zero row
    // gets kZero, which the output stage writes as zeros.  All of it is
    // integer arithmetic on wave-uniform values.
    static constexpr int kZero = 0x4000;  // (fits a signed 16-bit field)
    __device__ __forceinline__ static int mag_exp(uint32_t m) {
        if constexpr (KIND == IN_F16) {
            const int E = (int)(m >> 10);
            return E ? E - 14 : (32 - __builtin_clz(m)) - 24;
        } else {
            const int E = (int)(m >> 7);
            return E ? E - 126 : (32 - __builtin_clz(m)) - 133;
        }
    }
    __device__ __forceinline__ static int scale_exp(uint32_t m, int hb) {
        const int k = 8 - mag_exp(m | (m == 0 ? 1u : 0u)) - hb;
        const int kc = (KIND == IN_F16) ? min(max(k, -24), 14) : min(max(k, -126), 127);
        return m ? kc : kZero;
    }
    // 2^k as fp32 bits (k in [-126, 127]; kZero gives 1, the scale is unused)
    __device__ __forceinline__ static float exp2i(int k) {
        return __uint_as_float((uint32_t)((k == kZero ? 0 : k) + 127) << 23);
    }
    // 2^k as fp16 bits, k in [-24, 15] (kZero gives 1)
    __device__ __forceinline__ static uint32_t exp2h(int k) {
        if (k == kZero) return 0x3c00u;
        return k >= -14 ? (uint32_t)(k + 15) << 10 : 1u << (k + 24);
    }
    // LDS access by byte address.  Addresses are built as a per-lane base,
    // laundered once per pass (so the compiler does not keep one register per
    // tile and slot alive across the whole kernel), XORed with compile-time or
    // wave-uniform parts; a compile-time signal offset is added last and folds
    // into the instruction's offset field.
    template <class V = uint32_t>
    __device__ __forceinline__ V &lds(int b) { return *(V *)((char *)data + b); }
    // Bytes per signal slot: M points and PAD more dwords, so that the same
    // point of two slots falls in different banks (the compiler merges such
    // pairs of reads into one two-address instruction, whose two dwords a
    // power-of-two slot stride would put in one bank).  The slot offset is
    // added after every XOR of the swizzle.
    static constexpr int SB = (M + SH::PAD) * 4;

    // ---------------------------------------------------------- pass 0
    // Tile i of this wave covers columns c = 32 (w + i NW) + lane%32 of
    // signal s = 32 (w + i NW) / S0 (uniform over the tile), offset n = c % S0;
    // lane half h = lane/32 holds inputs m = 4h .. 4h+3 at n + m S0.
    __device__ __forceinline__ int tile_sig(int i) const { return (32 * (w + i * NW)) / S0; }
    __device__ __forceinline__ int tile_n(int i) const { return (32 * (w + i * NW)) % S0 + (lane & 31); }

    // 16-bit activations through the rows' buffer resources (zero past each
    // row's valid length; a row that does not exist has an empty resource,
    // so a round is always SIG signals, the missing ones all zero).  The
    // compile-time part of the offset goes in the scalar offset, which gfx950
    // includes in the range check of a raw buffer access (checked on the
    // device: a load whose per-lane offset is in range but whose total offset
    // is not returns zero).
    template <class RB>
    __device__ __forceinline__ void fetch_raw(const RB &rows, int sig0, uint32_t (&buf)[T0W][4]) {
        const int h = lane >> 5;
#pragma unroll
        for (int i = 0; i < T0W; ++i) {
            const int off = 2 * (tile_n(i) + 4 * h * S0);
            const RowBufs rb = rows(sig0 + tile_sig(i));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rb.in0, off, 2 * e * S0, kNT);
                const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rb.in1, off, 2 * e * S0, kNT);
                buf[i][e] = lo | (hi << 16);
            }
        }
    }

    // Zero-padded radix-16 DIF pass over the first NS signals: DFT on the
    // matrix cores, twiddle w_M^{n q}, to LDS.  `op(i, e)` yields the packed
    // scaled operand of tile i.  With FILT, the tiles of signal 0's columns
    // are also done for the filter operand fop(i, e), into slot SIG.
    template <int NS, bool FILT = false, class OP, class FOP>
    __device__ void pass0(const OP &op, const FOP &fop) {
        const int h = lane >> 5;
        // lane part of the column (lane % 32) and of the output q = qc + 2h
        const int lb = opaque(((lane & 31) ^ phys<LOG2M>(2 * h * S0)) << 2);
        auto tile = [&](int i, int s, const half8 b) {
            uint32_t tw[8];
            get_tw0(i % ND0, tw);
            const int pn = lb ^ (phys<LOG2M>((32 * (w + i * NW)) % S0) << 2);
            const f16v z = {};
            const f16v d = __builtin_amdgcn_mfma_f32_32x32x16_f16(A0, b, z, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 16; v += 2) {
                const int qc = 4 * (v >> 2) + ((v & 3) >> 1);  // q = qc + 2h
                lds((pn ^ (phys<LOG2M>(qc * S0) << 2)) + s * SB) = cmulh(pk(d[v], d[v + 1]), tw[v >> 1]);
            }
        };
#pragma unroll
        for (int i = 0; i < T0W; ++i) {
            const int s = tile_sig(i);
            if (NS == SIG || s < NS) tile(i, s, as_half8(op(i, 0), op(i, 1), op(i, 2), op(i, 3)));
        }
        if constexpr (FILT) {
#pragma unroll
            for (int i = 0; i < T0W; ++i)
                if (tile_sig(i) == 0) tile(i, SIG, as_half8(fop(i, 0), fop(i, 1), fop(i, 2), fop(i, 3)));
        }
        __syncthreads();
    }

    // Inverse of pass 0 keeping outputs m < 8.  The inverse passes keep the
    // signal conjugated in LDS (IDFT(x) = conj(DFT(conj(x))), and the
    // conjugations between consecutive passes cancel), so this pass is the
    // twiddle times the stored value, forward DFT-16 rows 0..7, and the one
    // remaining conjugation in the output, scaled by os and converted to
    // the activation type; st(s, n, m, v) stores the packed pair v (row 2s
    // in the low half, row 2s + 1 in the high half) of output m = 2g, 2g+1.
    template <class ST>
    __device__ void pass0_inv(const ST &st, const int (&kq)[TIW][2], float ob) {
        const int lb = opaque((j ^ phys<LOG2M>(2 * g * S0)) << 2);
        // All twiddles and products first, then all stores: loads and stores
        // retire in order, so a table load behind a store would wait for it.
        // The LDS reads go in batches of BD / 4 tiles (an empty asm with a
        // memory clobber keeps a batch's reads from moving up into the
        // previous one, where they would only hold registers).
        // (twiddles from the table: per batch, issued with its LDS reads)
        constexpr int NTA = TWREG ? NDI : 1;
        uint32_t tua[NTA][4];
        if constexpr (TWREG) {
#pragma unroll
            for (int d = 0; d < NDI; ++d) get_tu0(d, tua[d]);
        }
        constexpr int BI = TIW < SH::BD / 4 ? TIW : SH::BD / 4;
        static_assert(TIW % BI == 0, "inverse pass-0 tiles split into equal batches");
        uint32_t ov[TIW][2];
        // output scale of each tile's signal, ob 2^-k: real half (row 2s),
        // imaginary half (row 2s + 1); zero for a row of zeros
        f2 os[TIW];
#pragma unroll
        for (int i = 0; i < TIW; ++i)
            os[i] = f2{kq[i][0] == kZero ? 0.f : ldexpf(ob, -kq[i][0]), kq[i][1] == kZero ? 0.f : ldexpf(ob, -kq[i][1])};
        auto cv = [&](float re, float im, f2 o) -> uint32_t {
            const f2 v = {re * o.x, im * o.y};
            if constexpr (KIND == IN_BF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2));
            else return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
        };
#pragma unroll
        for (int i0 = 0; i0 < TIW; i0 += BI) {
            uint32_t xb[BI][4], tb[TWREG ? 1 : BI][4];
            if constexpr (!TWREG) {
#pragma unroll
                for (int k = 0; k < BI; ++k) get_tu0((i0 + k) % NDI, tb[k]);
            }
#pragma unroll
            for (int k = 0; k < BI; ++k) {
                const int i = i0 + k;
                const int s = (16 * (w + i * NW)) / S0;
                const int n0 = (16 * (w + i * NW)) % S0;
                const int pn = lb ^ (phys<LOG2M>(n0) << 2);
#pragma unroll
                for (int t = 0; t < 4; ++t) xb[k][t] = lds((pn ^ (phys<LOG2M>(tab::kChain[t] * S0) << 2)) + s * SB);
            }
#pragma unroll
            for (int k = 0; k < BI; ++k) {
                const int i = i0 + k;
                uint32_t tu[4], x[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    tu[t] = TWREG ? tua[i % NTA][t] : tb[TWREG ? 0 : k][t];
                    x[t] = xb[k][t];
                }
                cmulh_n(x, tu);
                const f4 z = {0.f, 0.f, 0.f, 0.f};
                const f4 r = __builtin_amdgcn_mfma_f32_16x16x32_f16(C0, as_half8(x[0], x[1], x[2], x[3]), z, 0, 0, 0);
                ov[i][0] = cv(r[0], -r[1], os[i]);
                ov[i][1] = cv(r[2], -r[3], os[i]);
            }
            asm volatile("" ::: "memory");
        }
#pragma unroll
        for (int i = 0; i < TIW; ++i) {
            const int s = (16 * (w + i * NW)) / S0;
            const int n = (16 * (w + i * NW)) % S0 + j;
            st(s, n, 2 * g, ov[i][0]);
            st(s, n, 2 * g + 1, ov[i][1]);
        }
    }

    // ---------------------------------------------------------- middle passes
    template <int P>
    __device__ __forceinline__ int base0() {
        constexpr int L = SH::L(P), S = L / 16;
        const int b = 16 * w + j;
        return (b / S) * L + (b % S);
    }

    // INV = false: DIF pass, y_k = tw_k * sum_m W^{km} x_m.
    // INV = true:  its inverse (up to the factor 16) on conjugated data:
    // conj(x) = DFT(conj(y) tw), i.e. twiddle first, then the forward DFT.
    // Each lane reads and writes back the slots k = chain(g, 0..3) of its
    // tiles (signal s < NS, tile ti < TPW).  The reads of a batch of tiles
    // are all issued before its first write: the compiler cannot tell that
    // one tile's writes never touch another's slots, so it would otherwise
    // wait out every tile's read latency in turn.
    template <int P, bool INV, int NS>
    __device__ void mid_pass(uint32_t pre = 0u) {
        constexpr int L = SH::L(P), S = L / 16;
        constexpr int NTL = NS * TPW, BT = NTL < SH::BD / 4 ? NTL : SH::BD / 4;
        const int pb = opaque((phys<LOG2M>(base0<P>()) ^ phys<LOG2M>(2 * g * S)) << 2);
        uint32_t tw[4];
        get_twm(P - 1, tw);
        auto addr = [&](int tile, int t) {
            const int s = tile / TPW, ti = tile % TPW;
            return ((pb ^ (phys<LOG2M>(ti * DELTA) << 2)) ^ (phys<LOG2M>(tab::kChain[t] * S) << 2)) + s * SB;
        };
#pragma unroll
        for (int b0 = 0; b0 < NTL; b0 += BT) {
            uint32_t xb[BT][4];
#pragma unroll
            for (int k = 0; k < BT; ++k)
                if (b0 + k < NTL) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) xb[k][t] = lds(addr(b0 + k, t));
                }
#pragma unroll
            for (int k = 0; k < BT; ++k) {
                if (b0 + k >= NTL) break;
                int a[4];
                uint32_t x[4];
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    a[t] = addr(b0 + k, t);
                    x[t] = xb[k][t];
                    if (INV && P == K) x[t] = pkmul(x[t], pre);  // scale set after the last pass
                }
                if (INV) cmulh_n(x, tw);
                const half8 b = as_half8(x[0], x[1], x[2], x[3]);
                const f4 z = {0.f, 0.f, 0.f, 0.f};
                const f4 d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(C0, b, z, 0, 0, 0);
                const f4 d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(C1, b, z, 0, 0, 0);
                if (!INV) {
                    lds(a[0]) = cmulh(pk(d0[0], d0[1]), tw[0]);
                    lds(a[1]) = cmulh(pk(d0[2], d0[3]), tw[1]);
                    lds(a[2]) = cmulh(pk(d1[0], d1[1]), tw[2]);
                    lds(a[3]) = cmulh(pk(d1[2], d1[3]), tw[3]);
                } else {
                    lds(a[0]) = pk(d0[0], d0[1]);
                    lds(a[1]) = pk(d0[2], d0[3]);
                    lds(a[2]) = pk(d1[0], d1[1]);
                    lds(a[3]) = pk(d1[2], d1[3]);
                }
            }
        }
        __syncthreads();
    }

    template <int P, int NS>
    __device__ void fwd_middle() {
        if constexpr (P <= K) {
            mid_pass<P, false, NS>();
            fwd_middle<P + 1, NS>();
        }
    }
    template <int P, int NS = SIG>
    __device__ void inv_middle(uint32_t pre) {
        if constexpr (P >= 1) {
            mid_pass<P, true, NS>(pre);
            inv_middle<P - 1, NS>(pre);
        }
    }

    // ---------------------------------------------------------- last pass
    // Unit u of a lane covers one group of R consecutive points.  lbase() is
    // the lane's byte base (laundered by the caller), lpos(u) the unit's
    // compile-time XOR part, lsig(u) its signal.  For R = 16 / 8 the base
    // already points at the lane's first slot 2g; R <= 4 needs NBL >= NT.
    __device__ __forceinline__ int lbase() const {
        if constexpr (R == 16) return (phys<LOG2M>(16 * (16 * w + j)) ^ (2 * g)) << 2;
        else if constexpr (R == 8) return (phys<LOG2M>(8 * (16 * w + j)) ^ (2 * g)) << 2;
        else return phys<LOG2M>(R * tid) << 2;
    }
    static constexpr int lpos(int u) {
        if constexpr (R == 16) return phys<LOG2M>(16 * (u % NLS) * 16 * NW) << 2;
        else if constexpr (R == 8) return phys<LOG2M>(8 * (u % NLS) * 16 * NW) << 2;
        else return phys<LOG2M>(R * ((u % NSL) * NT)) << 2;
    }
    static constexpr int lsig(int u) { return R >= 8 ? u / NLS : u / NSL; }
    static_assert(R >= 8 || NBL % NT == 0, "radix-2/4 last pass: butterflies must be a multiple of the threads");

    // dwords a lane reads for one last-pass unit
    static constexpr int NVD = (R == 16 || R == 4) ? 4 : 2;
    // read one unit (pb = byte address of the unit including its signal offset)
    __device__ __forceinline__ void last_load(int pb, uint32_t (&v)[NVD]) {
        // (elements go through scalars: bit-casting an element expression of
        //  an ext_vector directly reads element 0)
        if constexpr (R == 16) {
            const u32x2 lo = lds<u32x2>(pb);
            const u32x2 hi = lds<u32x2>(pb ^ 32);  // slots 8 + 2g, 9 + 2g
            const uint32_t v0 = lo.x, v1 = lo.y, v2 = hi.x, v3 = hi.y;
            v[0] = v0; v[1] = v1; v[2] = v2; v[3] = v3;
        } else if constexpr (R == 4) {
            const u32x4 a = lds<u32x4>(pb);
            const uint32_t v0 = a.x, v1 = a.y, v2 = a.z, v3 = a.w;
            v[0] = v0; v[1] = v1; v[2] = v2; v[3] = v3;
        } else {
            const u32x2 a = lds<u32x2>(pb);
            const uint32_t v0 = a.x, v1 = a.y;
            v[0] = v0; v[1] = v1;
        }
    }
    // forward last-pass DFT of one unit's values (packed fp16 results,
    // chained order for R = 16, natural for R = 8)
    __device__ __forceinline__ void last_fwd(const uint32_t (&v)[NVD], uint32_t (&y)[NV]) {
        if constexpr (R == 16) {
            const half8 b = as_half8(v[0], v[1], v[2], v[3]);
            const f4 z = {0.f, 0.f, 0.f, 0.f};
            const f4 d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(C0, b, z, 0, 0, 0);
            const f4 d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(C1, b, z, 0, 0, 0);
            y[0] = pk(d0[0], d0[1]);
            y[1] = pk(d0[2], d0[3]);
            y[2] = pk(d1[0], d1[1]);
            y[3] = pk(d1[2], d1[3]);
        } else if constexpr (R == 8) {
            const f4 z = {0.f, 0.f, 0.f, 0.f};
            const f4 d = __builtin_amdgcn_mfma_f32_16x16x16f16(A8, as_half4(v[0], v[1]), z, 0, 0, 0);
            y[0] = pk(d[0], d[1]);
            y[1] = pk(d[2], d[3]);
        } else if constexpr (R == 4) {
            const h2 a = __builtin_bit_cast(h2, v[0]), b = __builtin_bit_cast(h2, v[1]),
                     c = __builtin_bit_cast(h2, v[2]), d = __builtin_bit_cast(h2, v[3]);
            const h2 s0 = a + c, d0 = a - c, s1 = b + d, d1 = b - d;
            const h2 d1mi = {d1.y, -d1.x};  // (b - d) * (-i)
            y[0] = __builtin_bit_cast(uint32_t, s0 + s1);
            y[1] = __builtin_bit_cast(uint32_t, d0 + d1mi);
            y[2] = __builtin_bit_cast(uint32_t, s0 - s1);
            y[3] = __builtin_bit_cast(uint32_t, d0 - d1mi);
        } else {
            const h2 a = __builtin_bit_cast(h2, v[0]), b = __builtin_bit_cast(h2, v[1]);
            y[0] = __builtin_bit_cast(uint32_t, a + b);
            y[1] = __builtin_bit_cast(uint32_t, a - b);
        }
    }
    __device__ __forceinline__ void last_fwd(int pb, uint32_t (&y)[NV]) {
        uint32_t v[NVD];
        last_load(pb, v);
        last_fwd(v, y);
    }

    // Inverse last-pass DFT, written back in place conjugated (the inverse
    // passes work on conjugated data): `y` holds conj(Y) and the forward DFT
    // gives conj(IDFT(Y)) R.  Returns the largest magnitude of a real or
    // imaginary part written.
    __device__ __forceinline__ float last_inv(int pb, const uint32_t (&y)[NV]) {
        if constexpr (R == 16) {
            const half8 b = as_half8(y[0], y[1], y[2], y[3]);
            const f4 z = {0.f, 0.f, 0.f, 0.f};
            const f4 d0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(C0, b, z, 0, 0, 0);
            const f4 d1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(C1, b, z, 0, 0, 0);
            const u32x2 lo = {pk(d0[0], d0[1]), pk(d0[2], d0[3])};
            const u32x2 hi = {pk(d1[0], d1[1]), pk(d1[2], d1[3])};
            lds<u32x2>(pb) = lo;
            lds<u32x2>(pb ^ 32) = hi;
            return fmaxf(fmaxf(habs_max(lo.x), habs_max(lo.y)), fmaxf(habs_max(hi.x), habs_max(hi.y)));
        } else if constexpr (R == 8) {
            const f4 z = {0.f, 0.f, 0.f, 0.f};
            const f4 d = __builtin_amdgcn_mfma_f32_16x16x16f16(A8, as_half4(y[0], y[1]), z, 0, 0, 0);
            const u32x2 o = {pk(d[0], d[1]), pk(d[2], d[3])};
            lds<u32x2>(pb) = o;
            return fmaxf(habs_max(o.x), habs_max(o.y));
        } else if constexpr (R == 4) {
            const h2 a = __builtin_bit_cast(h2, y[0]), b = __builtin_bit_cast(h2, y[1]),
                     c = __builtin_bit_cast(h2, y[2]), d = __builtin_bit_cast(h2, y[3]);
            const h2 s0 = a + c, d0 = a - c, s1 = b + d, d1 = b - d;
            const h2 d1mi = {d1.y, -d1.x};  // (b - d) * (-i)
            const h2 o0 = s0 + s1, o1 = d0 + d1mi, o2 = s0 - s1, o3 = d0 - d1mi;
            const u32x4 o = {__builtin_bit_cast(uint32_t, o0), __builtin_bit_cast(uint32_t, o1),
                             __builtin_bit_cast(uint32_t, o2), __builtin_bit_cast(uint32_t, o3)};
            lds<u32x4>(pb) = o;
            const h2 m = __builtin_elementwise_max(
                __builtin_elementwise_max(__builtin_elementwise_abs(o0), __builtin_elementwise_abs(o1)),
                __builtin_elementwise_max(__builtin_elementwise_abs(o2), __builtin_elementwise_abs(o3)));
            return fmaxf((float)m.x, (float)m.y);
        } else {
            const h2 a = __builtin_bit_cast(h2, y[0]), b = __builtin_bit_cast(h2, y[1]);
            const h2 o0 = a + b, o1 = a - b;
            const u32x2 o = {__builtin_bit_cast(uint32_t, o0), __builtin_bit_cast(uint32_t, o1)};
            lds<u32x2>(pb) = o;
            const h2 m = __builtin_elementwise_max(__builtin_elementwise_abs(o0), __builtin_elementwise_abs(o1));
            return fmaxf((float)m.x, (float)m.y);
        }
    }

    __device__ __forceinline__ int fslot(int slot) const {
        if constexpr (R >= 8) return slot * NV;
        else return (slot % NSL) * NV;
    }
    // ---------------------------------------------------------- filter
    // Filter spectrum, kept in registers as packed fp16: conj(F) = conj(DFT(f))
    // * cF / R with cF = 2^-e where sum |f| < 2^e.  Every
    // partial sum of the transform is bounded by sum |f|, so inputs scaled by
    // 2^(14 - e) keep the whole transform below 2^14 and |F| below 1 / R,
    // without a reduction over the spectrum itself.
    // Issue the loads of the real filter into this lane's pass-0 slots, kept
    // apart from the transform so the activation loads can be issued behind
    // them.  `frs` covers the filter's taps (reads past them return zero:
    // the padding); d0 is added to tap 0 (the skip term D u folded in).
    __device__ __forceinline__ void filter_fetch(__amdgpu_buffer_rsrc_t frs, float d0, float (&fin)[T0W][4]) {
        const int h = lane >> 5;
#pragma unroll
        for (int i = 0; i < T0W; ++i) {
            const int off = tile_n(i) + 4 * h * S0;
            if (tile_sig(i) == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    fin[i][e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(frs, 4 * off, 4 * e * S0, 0));
                if (off == 0) fin[i][0] += d0;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) fin[i][e] = 0.f;
            }
        }
    }

    __device__ __forceinline__ float filter_asum(const float (&fin)[T0W][4]) const {
        float asum = 0.f;
#pragma unroll
        for (int i = 0; i < T0W; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) asum += fabsf(fin[i][e]);
        return asum;
    }
    // input scale of the filter from the workgroup's sum |f|; sets cF
    __device__ __forceinline__ float filter_scale(float asum) {
        int ef = 0;
        if (asum > 0.f) (void)frexpf(asum, &ef);
        cF = ldexpf(1.f, -ef);
        return ldexpf(1.f, 14 - ef);
    }
    // last pass of the filter transform (signal slot `s`): the spectrum into
    // F, conjugated (the products take conj(X) conj(F) = conj(X F)), or as
    // it is with CORR (conj(X) F = conj(X conj(F)): correlation)
    // ACC: added to the spectrum already in F (both at the same scale).
    template <bool CORR, bool ACC = false>
    __device__ __forceinline__ void filter_last(int s) {
        constexpr float c = 1.0f / (16384.0f * R);
        const uint32_t ch = CORR ? pk(c, c) : pk(c, -c);
        const int lb = opaque(lbase());
#pragma unroll
        for (int slot = 0; slot < NLS; ++slot) {
            if (R >= 8 || slot < NSL) {
                uint32_t y[NV];
                last_fwd((lb ^ lpos(slot)) + s * SB, y);
#pragma unroll
                for (int q = 0; q < NV; ++q) {
                    const uint32_t v = pkmul(y[q], ch);
                    F[fslot(slot) + q] = ACC ? __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, F[fslot(slot) + q]) +
                                                                               __builtin_bit_cast(h2, v))
                                             : v;
                }
            }
        }
    }
    // the filter on its own, in signal slot 0
    template <bool CORR>
    __device__ void filter(const float (&fin)[T0W][4]) {
        const float sf = filter_scale(block_reduce<true>(filter_asum(fin)));
        auto fop = [&](int i, int e) -> uint32_t { return pk(fin[i][e] * sf, 0.f); };
        pass0<1>(fop, fop);
        fwd_middle<1, 1>();
        filter_last<CORR>(0);
    }

    // ---------------------------------------------------------- conv round
    // One round of SIG signals from pin.  FILT: the filter (fin) is
    // transformed alongside, in slot SIG, and its spectrum taken into F
    // before the products.  prefetch() is called once pin has been consumed.
    template <bool FILT, bool CORR, class OUT, class PF>
    __device__ void conv_round(const OUT &out, int hb, const float (&fin)[T0W][4], const PF &prefetch) {
        conv_round<FILT, CORR>(out, hb, fin, prefetch, [](uint32_t) {}, [](int, const uint32_t(&)[NV]) {});
    }
    // With hooks: onexp(e) receives the round's row exponents (lane s <
    // SIG: signal s's pair, as round_exps returns them), onfwd(u, y) the
    // forward last-pass values of unit u before the product.
    template <bool FILT, bool CORR, class OUT, class PF, class OE, class OF>
    __device__ void conv_round(const OUT &out, int hb, const float (&fin)[T0W][4], const PF &prefetch,
                               const OE &onexp, const OF &onfwd) {
        static_assert(KIND == IN_F16 || KIND == IN_BF16, "16-bit activations");
        __builtin_amdgcn_s_setprio(kPrioLoad);
        // Every row gets a scale of its own: a signal's real and imaginary
        // halves are different rows, and one scale for both would leave a
        // small row with rounding errors of the size of its partner's values.
        int kp[T0W][2], kq[TIW][2];
        float sf = 0.f;
        {
            float fa = FILT ? filter_asum(fin) : 0.f;
            const uint32_t kpk = round_exps<FILT>(fa, hb);
            onexp(kpk);
            exps_of(kpk, kp, kq);
            if constexpr (FILT) sf = filter_scale(fa);
        }
        f2 sut[T0W] = {};
        uint32_t suh[T0W] = {};
#pragma unroll
        for (int i = 0; i < T0W; ++i) {
            if constexpr (KIND == IN_F16) suh[i] = exp2h(kp[i][0]) | (exp2h(kp[i][1]) << 16);
            else sut[i] = f2{exp2i(kp[i][0]), exp2i(kp[i][1])};
        }
        pass0<SIG, FILT>([&](int i, int e) -> uint32_t { return in_scaled<KIND>(pin[i][e], sut[i], suh[i]); },
                         [&](int i, int e) -> uint32_t { return pk(fin[i][e] * sf, 0.f); });
        prefetch();
        __builtin_amdgcn_s_setprio(kPrioWork);
        fwd_middle<1, SIG + (FILT ? 1 : 0)>();
        if constexpr (FILT) filter_last<CORR>(SIG);
        // Last pass, in place: forward DFT-R, product with the filter spectrum
        // (stored as conj(F) cF / R, so no product can overflow the inverse
        // DFT-R), inverse DFT-R on conjugated values.  The maximum of what it
        // writes sets the scale sy applied by the next inverse pass.
        uint32_t Fr[FN];
#pragma unroll
        for (int i = 0; i < FN; ++i) Fr[i] = F[i];
        // Units go in batches whose reads are all issued before the first
        // write (as in the middle passes).
        float vmax = 0.f;
        const int lb = opaque(lbase());
        constexpr int UB = NU * NVD <= SH::BD ? NU : SH::BD / NVD;
        static_assert(NU % UB == 0, "last-pass units split into equal batches");
#pragma unroll
        for (int u0 = 0; u0 < NU; u0 += UB) {
            uint32_t vb[UB][NVD];
#pragma unroll
            for (int k = 0; k < UB; ++k) last_load((lb ^ lpos(u0 + k)) + lsig(u0 + k) * SB, vb[k]);
#pragma unroll
            for (int k = 0; k < UB; ++k) {
                const int u = u0 + k, slot = u % NLS;
                const int pb = (lb ^ lpos(u)) + lsig(u) * SB;
                uint32_t y[NV], fr[NV];
                last_fwd(vb[k], y);
                onfwd(u, y);
#pragma unroll
                for (int q = 0; q < NV; ++q) fr[q] = Fr[fslot(slot) + q];
                cmulh_cx_n(y, fr);  // conj(Y) = conj(X) conj(F)
                vmax = fmaxf(vmax, last_inv(pb, y));
            }
        }
        // The remaining inverse passes grow magnitudes by at most M / R: scale
        // to keep every partial sum below 2^14, as an exact fp16 power of two.
        const float vm = block_reduce<false>(vmax);
        int ev = 0;
        if (vm > 0.f) (void)frexpf(vm, &ev);
        const float sy = fminf(fmaxf(ldexpf(1.f, 14 - ev - (LOG2M - SH::LR)), 1.0f / 16384.0f), 32768.0f);
        inv_middle<K>(pk(sy, sy));
        // output scales R / (M su sy cF), su = 2^k per row (rows of zeros
        // are written as zeros)
        pass0_inv(out, kq, (float)R / ((float)M * sy * cF));
    }

    // A whole channel of 16-bit activations: the filter spectrum, then
    // ceil(nsig / SIG) rounds of complex signals.  `frs` covers the real
    // filter's taps and d0 is added to tap 0; rows(sig) gives the buffer
    // resources of signal `sig`, empty ones for the rows past the last (a
    // round always transforms SIG signals).  The inputs of each round are
    // fetched while the previous round (or the filter) is being transformed.
    // SPOL: cache policy of the output stores.
    // Bidirectional copies: the convolution with the two-sided filter whose
    // causal taps are f (with d0 added to tap 0, the residual) and whose
    // anti-causal taps are g, i.e. the spectrum F + conj(G): both filters are
    // transformed on their own (f, then g, in signal slot 0) with one input
    // scale from sum |f| + sum |g|, which bounds every partial sum of either
    // transform and of the combined spectrum; the stored conjugate is
    // conj(F) + G.  Then the rounds, as in run_raw.
    template <int SPOL = kNT, class RB>
    __device__ void run_raw_bidir(__amdgpu_buffer_rsrc_t frs, float d0, __amdgpu_buffer_rsrc_t grs, const RB &rows,
                                  int nsig, int hb) {
        static_assert(KIND == IN_F16 || KIND == IN_BF16, "16-bit activations");
        float fin[T0W][4];
        __builtin_amdgcn_s_setprio(kPrioLoad);
        {
            // g is loaded twice: for its sum |g| now, and for its transform
            // after f's (kept in registers through f's transform, it would
            // spill)
            float gs;
            {
                float gin[T0W][4];
                filter_fetch(frs, d0, fin);
                filter_fetch(grs, 0.f, gin);
                gs = filter_asum(gin);
            }
            const float sf = filter_scale(block_reduce<true>(filter_asum(fin) + gs));
            auto fop = [&](int i, int e) -> uint32_t { return pk(fin[i][e] * sf, 0.f); };
            pass0<1>(fop, fop);
            float gin[T0W][4];
            filter_fetch(grs, 0.f, gin);
            fwd_middle<1, 1>();
            filter_last<false>(0);
            __syncthreads();  // slot 0 has been read; the second transform writes it
            auto gop = [&](int i, int e) -> uint32_t { return pk(gin[i][e] * sf, 0.f); };
            pass0<1>(gop, gop);
            if constexpr (PREFETCH) fetch_raw(rows, 0, pin);
            fwd_middle<1, 1>();
            filter_last<true, true>(0);
        }
        auto store = [&](int r0, int s, int n, int m, uint32_t hv) {
            const RowBufs rb = rows(r0 + s);
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)hv, rb.out0, 2 * (n + m * S0), 0, SPOL);
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(hv >> 16), rb.out1, 2 * (n + m * S0), 0, SPOL);
        };
        auto prefetch = [&](int r0) {
            if (PREFETCH && r0 + SIG < nsig) fetch_raw(rows, r0 + SIG, pin);
        };
        for (int r0 = 0; r0 < nsig; r0 += SIG) {
            __builtin_amdgcn_s_setprio(kPrioLoad);
            if (!PREFETCH) fetch_raw(rows, r0, pin);
            conv_round<false, false>([&](int s, int n, int m, uint32_t hv) { store(r0, s, n, m, hv); }, hb, fin,
                                     [&]() { prefetch(r0); });
        }
    }

    // CORR: correlation with the filter (its conjugated spectrum) instead of
    // convolution.
    template <int SPOL = kNT, bool CORR = false, class RB>
    __device__ void run_raw(__amdgpu_buffer_rsrc_t frs, float d0, const RB &rows, int nsig, int hb) {
        static_assert(KIND == IN_F16 || KIND == IN_BF16, "16-bit activations");
        float fin[T0W][4];
        __builtin_amdgcn_s_setprio(kPrioLoad);
        filter_fetch(frs, d0, fin);
        if constexpr (PREFETCH || SH::FUSEF) fetch_raw(rows, 0, pin);
        // output of round r0: packed pair v of rows 2 (r0 + s), 2 (r0 + s) + 1
        auto store = [&](int r0, int s, int n, int m, uint32_t hv) {
            const RowBufs rb = rows(r0 + s);
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)hv, rb.out0, 2 * (n + m * S0), 0, SPOL);
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(hv >> 16), rb.out1, 2 * (n + m * S0), 0, SPOL);
        };
        // with PREFETCH, the next round's inputs are loaded into pin as soon
        // as pass 0 has consumed this round's
        auto prefetch = [&](int r0) {
            if (PREFETCH && r0 + SIG < nsig) fetch_raw(rows, r0 + SIG, pin);
        };
        int r1 = 0;
        if constexpr (SH::FUSEF) {
            // first round with the filter alongside
            conv_round<true, CORR>([&](int s, int n, int m, uint32_t hv) { store(0, s, n, m, hv); }, hb, fin,
                                   [&]() { prefetch(0); });
            r1 = SIG;
        } else {
            filter<CORR>(fin);
        }
        for (int r0 = r1; r0 < nsig; r0 += SIG) {
            __builtin_amdgcn_s_setprio(kPrioLoad);
            if (!PREFETCH && (!SH::FUSEF || r0 > 0)) fetch_raw(rows, r0, pin);
            conv_round<false, CORR>([&](int s, int n, int m, uint32_t hv) { store(r0, s, n, m, hv); }, hb, fin,
                                    [&]() { prefetch(r0); });
        }
    }

    // ---------------------------------------------------------- filter gradient
    // Inverse of pass 0 for signal 0 alone, real part only, in fp32:
    // st(p, v) receives output point p = n + m S0 (m < 8) times ob.
    template <class ST>
    __device__ void pass0_inv_real(const ST &st, float ob) {
        constexpr int TI0 = S0 / 16;  // signal 0's inverse pass-0 tiles
        static_assert(TI0 % NW == 0, "signal 0's inverse tiles split evenly over the waves");
        constexpr int TW0 = TI0 / NW;
        const int lb = opaque((j ^ phys<LOG2M>(2 * g * S0)) << 2);
#pragma unroll
        for (int i = 0; i < TW0; ++i) {
            const int n0 = 16 * (w + i * NW);
            const int pn = lb ^ (phys<LOG2M>(n0) << 2);
            uint32_t x[4], tu[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) x[t] = lds(pn ^ (phys<LOG2M>(tab::kChain[t] * S0) << 2));
            get_tu0(i % NDI, tu);
            cmulh_n(x, tu);
            const f4 z = {0.f, 0.f, 0.f, 0.f};
            const f4 r = __builtin_amdgcn_mfma_f32_16x16x32_f16(C0, as_half8(x[0], x[1], x[2], x[3]), z, 0, 0, 0);
            st(n0 + j + 2 * g * S0, r[0] * ob);
            st(n0 + j + (2 * g + 1) * S0, r[2] * ob);
        }
    }

    // Filter gradient of a causal convolution: Re IDFT(sum_p conj(U_p)
    // DY_p)[:M/2] with U_p = DFT(u_2p + i u_2p+1) and DY_p the same of dy;
    // the real part is the sum over the rows of the correlations of u with
    // dy (the cross terms of a pair are imaginary).  Rounds come in twos
    // over the same SIG row pairs: the first keeps its forward last-pass
    // values in registers, with each row at its own scale 2^k_x; the second
    // ("tied") scales row x of the other tensor by 2^(K - k_x), K = min over
    // the pair's rows of k_x + k'_x (k'_x = that row's own exponent), so both
    // rows' products carry the one factor 2^K, removed exactly as they are
    // added, in fp32, to this lane's points of the sum.  A row scaled below
    // its own exponent holds a product at most 2^(K - k_x - k'_x) of the
    // pair's largest.  Rows of zeros take no part.
    static constexpr int kDrop = -0x4000;  // input exponent of a row left out (ldexp to zero)
    static constexpr int UBL = NU * NVD <= SH::BD ? NU : SH::BD / NVD;  // last-pass units per batch of reads
    static_assert(NU % UBL == 0, "last-pass units split into equal batches");

    // The kept round of a pair (run_df: u rows at their own scales): forward
    // passes, last-pass values into yk; returns the row exponents.
    template <class RB>
    __device__ __forceinline__ uint32_t keep_round(const RB &rows, int r, int nround, int hb,
                                                   uint32_t (&yk)[NU][NV]) {
        __builtin_amdgcn_s_setprio(kPrioLoad);
        if (!PREFETCH && r > 0) fetch_raw(rows, r * SIG, pin);
        float fs = 0.f;
        const uint32_t kpk = round_exps<false>(fs, hb);
        f2 sut[T0W] = {};
        uint32_t suh[T0W] = {};
#pragma unroll
        for (int i = 0; i < T0W; ++i) {
            const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)kpk, SIG == 1 ? 0 : tile_sig(i));
            if constexpr (KIND == IN_F16) suh[i] = exp2h(lo16(v)) | (exp2h(hi16(v)) << 16);
            else sut[i] = f2{exp2i(lo16(v)), exp2i(hi16(v))};
        }
        auto op = [&](int i, int e) -> uint32_t { return in_scaled<KIND>(pin[i][e], sut[i], suh[i]); };
        pass0<SIG>(op, op);
        if (PREFETCH && r + 1 < nround) fetch_raw(rows, (r + 1) * SIG, pin);
        __builtin_amdgcn_s_setprio(kPrioWork);
        fwd_middle<1, SIG>();
        const int lb = opaque(lbase());
#pragma unroll
        for (int u0 = 0; u0 < NU; u0 += UBL) {
            uint32_t vb[UBL][NVD];
#pragma unroll
            for (int k = 0; k < UBL; ++k) last_load((lb ^ lpos(u0 + k)) + lsig(u0 + k) * SB, vb[k]);
#pragma unroll
            for (int k = 0; k < UBL; ++k) last_fwd(vb[k], yk[u0 + k]);
        }
        return kpk;
    }

    // The tied round of a pair: scales tied to the kept round's exponents
    // kpk, products with the kept values yk added to acc.  CONJ_CUR: the
    // sum takes conj(this round's values) (u in this round), else conj(yk).
    template <bool CONJ_CUR, class RB>
    __device__ __forceinline__ void tied_round(const RB &rows, int r, int nround, int hb, uint32_t kpk,
                                               const uint32_t (&yk)[NU][NV], float (&acc)[FN][2]) {
        __builtin_amdgcn_s_setprio(kPrioLoad);
        if (!PREFETCH) fetch_raw(rows, r * SIG, pin);
        float fs = 0.f;
        const uint32_t kpo = round_exps<false>(fs, hb);
        // lane s < SIG: this round's input exponents for signal s, and K
        const int ka = lo16(kpk), kb = hi16(kpk), oa = lo16(kpo), ob = hi16(kpo);
        const bool va = ka != kZero && oa != kZero, vb = kb != kZero && ob != kZero;
        int kk = va ? ka + oa : (vb ? kb + ob : 0);
        if (va && vb) kk = min(kk, kb + ob);
        const int ea = va ? kk - ka : kDrop, eb = vb ? kk - kb : kDrop;
        const uint32_t kpe = ((uint32_t)ea & 0xffffu) | ((uint32_t)eb << 16);
        int eia[T0W], eib[T0W];
#pragma unroll
        for (int i = 0; i < T0W; ++i) {
            const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)kpe, SIG == 1 ? 0 : tile_sig(i));
            eia[i] = lo16(v);
            eib[i] = hi16(v);
        }
        auto op = [&](int i, int e) -> uint32_t {
            const uint32_t x = pin[i][e];
            float a, b;
            if constexpr (KIND == IN_F16) {
                const h2 hv = __builtin_bit_cast(h2, x);
                a = (float)hv.x;
                b = (float)hv.y;
            } else {
                a = __uint_as_float(x << 16);
                b = __uint_as_float(x & 0xffff0000u);
            }
            return pk(ldexpf(a, eia[i]), ldexpf(b, eib[i]));
        };
        pass0<SIG>(op, op);
        if (PREFETCH && r + 1 < nround) fetch_raw(rows, (r + 1) * SIG, pin);
        __builtin_amdgcn_s_setprio(kPrioWork);
        fwd_middle<1, SIG>();
        int nk[SIG];
#pragma unroll
        for (int sg = 0; sg < SIG; ++sg) nk[sg] = -__builtin_amdgcn_readlane(kk, sg);
        const int lb = opaque(lbase());
#pragma unroll
        for (int u0 = 0; u0 < NU; u0 += UBL) {
            uint32_t vb2[UBL][NVD];
#pragma unroll
            for (int k = 0; k < UBL; ++k) last_load((lb ^ lpos(u0 + k)) + lsig(u0 + k) * SB, vb2[k]);
#pragma unroll
            for (int k = 0; k < UBL; ++k) {
                const int u = u0 + k;
                uint32_t y[NV];
                last_fwd(vb2[k], y);
#pragma unroll
                for (int q = 0; q < NV; ++q) {
                    // acc += conj(a) d 2^-K
                    const h2 a = __builtin_bit_cast(h2, CONJ_CUR ? y[q] : yk[u][q]);
                    const h2 d = __builtin_bit_cast(h2, CONJ_CUR ? yk[u][q] : y[q]);
                    const float ar = (float)a.x, ai = (float)a.y, dr = (float)d.x, di = (float)d.y;
                    const float re = fmaf(ar, dr, ai * di), im = fmaf(ar, di, -ai * dr);
                    const int ix = fslot(u % NLS) + q;
                    acc[ix][0] += ldexpf(re, nk[lsig(u)]);
                    acc[ix][1] += ldexpf(im, nk[lsig(u)]);
                }
            }
        }
    }

    // After the last pair: the sum scaled so that |values| < 2^(14 - LR)
    // (its DFT-R, the first inverse step, then stays below 2^14), inverted
    // as in a convolution round (on conjugated values) for signal 0 alone,
    // real part stored through st(p, v).
    template <class ST>
    __device__ __forceinline__ void df_finish(const float (&acc)[FN][2], const ST &st) {
        float am = 0.f;
#pragma unroll
        for (int i = 0; i < FN; ++i) am = fmaxf(am, fmaxf(fabsf(acc[i][0]), fabsf(acc[i][1])));
        const float vm0 = block_reduce<false>(am);
        int ea0 = 0;
        if (vm0 > 0.f) (void)frexpf(vm0, &ea0);
        const int ec = 14 - SH::LR - ea0;
        float vmax = 0.f;
        {
            const int lb = opaque(lbase());
            constexpr int NU0 = R >= 8 ? NLS : NSL;  // signal 0's units
#pragma unroll
            for (int u = 0; u < NU0; ++u) {
                uint32_t y[NV];
#pragma unroll
                for (int q = 0; q < NV; ++q) {
                    const int ix = fslot(u % NLS) + q;
                    y[q] = pk(ldexpf(acc[ix][0], ec), -ldexpf(acc[ix][1], ec));
                }
                vmax = fmaxf(vmax, last_inv(lb ^ lpos(u), y));
            }
        }
        const float vm = block_reduce<false>(vmax);
        int ev = 0;
        if (vm > 0.f) (void)frexpf(vm, &ev);
        const float sy = fminf(fmaxf(ldexpf(1.f, 14 - ev - (LOG2M - SH::LR)), 1.0f / 16384.0f), 32768.0f);
        inv_middle<K, 1>(pk(sy, sy));
        // the output chain multiplied the sum by M sy 2^ec
        pass0_inv_real(st, ldexpf(1.0f / ((float)M * sy), -ec));
    }

    // The filter gradient alone.  rows(v): the buffers of virtual signal v =
    // round * SIG + s (u rows in even rounds, dy rows in odd ones).
    template <class RB, class ST>
    __device__ void run_df(const RB &rows, int nround, int hb, const ST &st) {
        static_assert(KIND == IN_F16 || KIND == IN_BF16, "16-bit activations");
        float acc[FN][2];
#pragma unroll
        for (int i = 0; i < FN; ++i) acc[i][0] = acc[i][1] = 0.f;
        uint32_t yk[NU][NV];
        __builtin_amdgcn_s_setprio(kPrioLoad);
        fetch_raw(rows, 0, pin);
        for (int r = 0; r < nround; r += 2) {
            const uint32_t kpk = keep_round(rows, r, nround, hb, yk);
            tied_round<false>(rows, r + 1, nround, hb, kpk, yk, acc);
        }
        df_finish(acc, st);
    }

    // The whole backward pass of a causal convolution with residual, one
    // read of u and dy: in each pair of rounds, the dy round is a
    // correlation round (CORR: du = the correlation of dy with the filter,
    // D dy by tap 0, dy rows at their own scales) whose forward last-pass
    // values are kept; the u round that follows (the same row pairs) is
    // tied to dy's exponents and adds conj(U) DY to the sum; df_finish then
    // gives df.  rows(v): dy rows (du as output) in even rounds, u rows in
    // odd ones.  `frs` covers the filter's taps, d0 is added to tap 0.
    template <int SPOL, class RB, class ST>
    __device__ void run_bwd(__amdgpu_buffer_rsrc_t frs, float d0, const RB &rows, int nround, int hb, const ST &st) {
        static_assert(KIND == IN_F16 || KIND == IN_BF16, "16-bit activations");
        float acc[FN][2];
#pragma unroll
        for (int i = 0; i < FN; ++i) acc[i][0] = acc[i][1] = 0.f;
        uint32_t yk[NU][NV];
        uint32_t kpd = 0;
        float fin[T0W][4];
        __builtin_amdgcn_s_setprio(kPrioLoad);
        filter_fetch(frs, d0, fin);
        fetch_raw(rows, 0, pin);
        auto store = [&](int r0, int s, int n, int m, uint32_t hv) {
            const RowBufs rb = rows(r0 + s);
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)hv, rb.out0, 2 * (n + m * S0), 0, SPOL);
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(hv >> 16), rb.out1, 2 * (n + m * S0), 0, SPOL);
        };
        auto onexp = [&](uint32_t e) { kpd = e; };
        auto onfwd = [&](int u, const uint32_t (&y)[NV]) {
#pragma unroll
            for (int q = 0; q < NV; ++q) yk[u][q] = y[q];
        };
        // (with B = 0 the first pair still runs, on empty rows: no stores,
        //  a zero sum)
        int r = 0;
        if constexpr (SH::FUSEF) {
            // the first dy round with the filter alongside
            auto pf = [&]() {
                if (PREFETCH) fetch_raw(rows, SIG, pin);
            };
            conv_round<true, true>([&](int s, int n, int m, uint32_t hv) { store(0, s, n, m, hv); }, hb, fin, pf,
                                   onexp, onfwd);
            tied_round<true>(rows, 1, nround, hb, kpd, yk, acc);
            r = 2;
        } else {
            filter<true>(fin);
        }
        for (; r < nround; r += 2) {
            const int r0 = r * SIG;
            auto pf = [&]() {
                if (PREFETCH) fetch_raw(rows, r0 + SIG, pin);
            };
            __builtin_amdgcn_s_setprio(kPrioLoad);
            if (!PREFETCH && r > 0) fetch_raw(rows, r0, pin);
            conv_round<false, true>([&](int s, int n, int m, uint32_t hv) { store(r0, s, n, m, hv); }, hb, fin, pf,
                                    onexp, onfwd);
            tied_round<true>(rows, r + 1, nround, hb, kpd, yk, acc);
        }
        df_finish(acc, st);
    }
};

}  // namespace mf
}  // namespace h3c
