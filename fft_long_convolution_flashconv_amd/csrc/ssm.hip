// ssm.hip -- diagonal-SSM filter generation and chunked state passing.
//
// Filter: f_k = 2 Re(sum_j C_j Abar_j^k Bbar_j), the blog's "The Convolution
// Connection" (f = [CB, CAB, CA^2B, ...]), with Abar = exp(dt A), Bbar = dt B.
// Powers are factored as Abar^k = Abar^(64 i) * Abar^l (k = 64 i + l), two
// small tables per mode built from exact exponentials in fp64, so the filter
// is a sum of products of table entries and no power is accumulated by long
// chains of multiplications.
//
// State passing: paperlayer.ai summary, section 4 "Long-sequence
// computation" (chunks sized to on-chip memory, an extra state vector carried
// between chunks, only chunk-size FFTs) and Appendix C "State Passing" (the
// update matrix M_ux = [Abar^{T-1} B, ..., Abar B, B]).  Per chunk c:
//   y_c = (f[:T] * u_c) + D u_c + 2 Re(sum_j C_j Abar_j^{t+1} x_{c-1,j})
//   x_c = Abar^T x_{c-1} + sum_k Abar^{T-1-k} Bbar u_{c,k}
// The chunk convolutions run on the fused FFT engine; the two projections use
// the same factored power tables.
#include <algorithm>
#include <atomic>

#include "h3conv_device.h"
#include "h3conv_internal.h"
#include "mfma_engine.h"

namespace h3c {

// Abar^n = exp(n dt A) in fp64.  dt Re A and dt Im A are exact products of
// fp32 values.  The phase n dt Im A reaches ~1e5 rad, so it is first reduced
// by whole turns with a two-part 2 pi (the residual keeps the absolute error
// of the fp64 product, ~1e-11 rad) and the sine and cosine then take their
// short-argument path.
__device__ __forceinline__ void apow64(double are, double aim, double n, double &re, double &im) {
    constexpr double kTwoPiHi = 6.283185307179586232;   // 2 pi rounded to fp64
    constexpr double kTwoPiLo = 2.4492935982947064e-16; // 2 pi - kTwoPiHi
    const double ph = aim * n;
    const double k = rint(ph * (1.0 / kTwoPiHi));
    const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, ph));
    double sn, cs;
    sincos(r, &sn, &cs);
    const double m = exp(are * n);
    re = m * cs;
    im = m * sn;
}
__device__ __forceinline__ cf abar_pow(double are, double aim, double n) {
    double re, im;
    apow64(are, aim, n, re, im);
    return mk((float)re, (float)im);
}

// ---------------------------------------------------------------- filter

// One workgroup per channel, 8 waves.  With k = 64 i + l the filter is the
// real part of a complex matrix product,
//   f[64 i + l] = 2 sum_j Re(W[j][l] G[j][i]),  W[j][l] = w_j Abar_j^l,
//   G[j][i] = Abar_j^(64 i)                    (w_j = C_j Bbar_j),
// i.e. the real product of [Gr | Gi] (i x 2S) and [Wr ; -Wi] (2S x l), run on
// the matrix cores in fp32 (16x16x4 products; K = 128 with modes j >= S
// zeroed).  W is built once; G for 64 values of i at a time (4096 outputs).
// LDS rows are 72 floats apart, so the four rows one operand read touches
// fall 8 banks apart and the 64 lanes of a read cover every bank twice (and
// two workgroups of 8 waves fit a compute unit).
constexpr int FILT_PR = 72;
constexpr int FILT_LDS = 4 * 64 * FILT_PR;  // floats: Wr, Wn, Gr, Gi

__device__ __forceinline__ double2 dmul(double2 x, double2 y) {
    return double2{x.x * y.x - x.y * y.y, x.x * y.y + x.y * y.x};
}

// The fp64 exponentials per mode of channel h, one wave each (waves 0..3):
// pw[0..3][j] = Abar_j^1, ^16, ^64, ^1024 (zero for j >= S).  Every power
// the filter and the state-passing tables use is a short product of these
// (a handful of fp64 complex products: relative error ~1e-16 each).  The
// caller synchronises before reading pw.
__device__ __forceinline__ void ssm_powers(const float *__restrict__ A, double dth, int S, int h,
                                           double2 (*pw)[64]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (w < 4) {
        constexpr double kPow[4] = {1.0, 16.0, 64.0, 1024.0};
        double re = 0.0, im = 0.0;
        if (lane < S) {
            const float *a = A + ((size_t)h * S + lane) * 2;
            apow64(dth * (double)a[0], dth * (double)a[1], kPow[w], re, im);
        }
        pw[w][lane] = double2{re, im};
    }
}

// The filter of channel h (512 threads) from its powers pw; lds holds
// FILT_LDS floats.
__device__ __forceinline__ void ssm_filter_body(const float *__restrict__ Bm, const float *__restrict__ C, double dth,
                                const float *__restrict__ D, float *__restrict__ f, int S, int64_t N, int64_t ldf,
                                int h, const double2 (*pw)[64], float *lds) {
    typedef float f4v __attribute__((ext_vector_type(4)));
    float *const Wr = lds, *const Wn = lds + 64 * FILT_PR;  // W[j][l]: real part, minus imaginary part
    float *const Gr = lds + 2 * 64 * FILT_PR, *const Gi = lds + 3 * 64 * FILT_PR;  // G[j][i - i0]
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

    // W: runs of 16 powers per (mode, quarter) from Abar^(16 q), step Abar;
    // modes j >= S are zero
    for (int e = tid; e < 64 * 4; e += 512) {
        const int j = e >> 2, q = e & 3;
        if (j < S) {
            const float *b = Bm + ((size_t)h * S + j) * 2;
            const float *c = C + ((size_t)h * S + j) * 2;
            const cf wj = cmul(mk(c[0], c[1]), mk((float)(dth * b[0]), (float)(dth * b[1])));
            double2 p = double2{1.0, 0.0};
            for (int r = 0; r < q; ++r) p = dmul(p, pw[1][j]);
            const double2 st = pw[0][j];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const cf v = cmul(wj, mk((float)p.x, (float)p.y));
                Wr[j * FILT_PR + 16 * q + k] = v.x;
                Wn[j * FILT_PR + 16 * q + k] = -v.y;
                p = dmul(p, st);
            }
        } else {
#pragma unroll
            for (int k = 0; k < 16; ++k) Wr[j * FILT_PR + 16 * q + k] = Wn[j * FILT_PR + 16 * q + k] = 0.f;
        }
    }
    const int64_t ntot = (N + 63) / 64;  // values of i
    // this wave's output tiles: i in [16 (w / 2), +16), l-tiles 2 (w % 2) + {0, 1}
    const int it = w >> 1, lt0 = 2 * (w & 1);
    // G run (j, q) of the block at i0 starts at Abar^(64 (i0 + 16 q)): from
    // (Abar^1024)^q, advanced by Abar^4096 from one block to the next
    // (threads e < 256 keep their run across the blocks)
    double2 gs = double2{1.0, 0.0}, gadv = double2{1.0, 0.0}, gst = double2{1.0, 0.0};
    if (tid < 256 && (tid >> 2) < S) {
        const int j = tid >> 2, q = tid & 3;
        for (int r = 0; r < q; ++r) gs = dmul(gs, pw[3][j]);
        gadv = dmul(pw[3][j], pw[3][j]);
        gadv = dmul(gadv, gadv);
        gst = pw[2][j];
    }
    for (int64_t i0 = 0; i0 < ntot; i0 += 64) {
        __syncthreads();  // the previous block of G has been read
        for (int e = tid; e < 64 * 4; e += 512) {
            const int j = e >> 2, q = e & 3;
            if (j < S) {
                double2 p = gs;
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    Gr[j * FILT_PR + 16 * q + k] = (float)p.x;
                    Gi[j * FILT_PR + 16 * q + k] = (float)p.y;
                    p = dmul(p, gst);
                }
                gs = dmul(gs, gadv);
            } else {
#pragma unroll
                for (int k = 0; k < 16; ++k) Gr[j * FILT_PR + 16 * q + k] = Gi[j * FILT_PR + 16 * q + k] = 0.f;
            }
        }
        __syncthreads();
        // out[i][l] over K = 128 in steps of 4: lane holds A[i = lane % 16][k = lane / 16]
        // and B[k = lane / 16][l = lane % 16]
        f4v acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        const int col = lane & 15, kr = lane >> 4;
#pragma unroll 8
        for (int k0 = 0; k0 < 64; k0 += 4) {
            const int j = k0 + kr;
            const float ar = Gr[j * FILT_PR + 16 * it + col];
            const float b0 = Wr[j * FILT_PR + 16 * lt0 + col], b1 = Wr[j * FILT_PR + 16 * (lt0 + 1) + col];
            acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(ar, b0, acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(ar, b1, acc[1], 0, 0, 0);
        }
#pragma unroll 8
        for (int k0 = 0; k0 < 64; k0 += 4) {
            const int j = k0 + kr;
            const float ai = Gi[j * FILT_PR + 16 * it + col];
            const float b0 = Wn[j * FILT_PR + 16 * lt0 + col], b1 = Wn[j * FILT_PR + 16 * (lt0 + 1) + col];
            acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(ai, b0, acc[0], 0, 0, 0);
            acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(ai, b1, acc[1], 0, 0, 0);
        }
        // accumulator v of tile t: i = i0 + 16 it + 4 (lane / 16) + v, l = 16 (lt0 + t) + lane % 16
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t k = 64 * (i0 + 16 * it + 4 * kr + v) + 16 * (lt0 + t) + col;
                if (k < N) {
                    float val = 2.f * acc[t][v];
                    if (D != nullptr && k == 0) val += D[h];
                    f[(size_t)h * ldf + k] = val;
                }
            }
    }
}

__global__ __launch_bounds__(512) void k_ssm_filter(const float *__restrict__ A,
                                                   const float *__restrict__ Bm,
                                                   const float *__restrict__ C,
                                                   const float *__restrict__ dt,
                                                   const float *__restrict__ D, float *__restrict__ f,
                                                   int S, int64_t N, int64_t ldf) {
    __shared__ float lds[FILT_LDS];
    __shared__ double2 pw[4][64];
    const int h = blockIdx.x;
    const double dth = (double)dt[h];
    ssm_powers(A, dth, S, h, pw);
    __syncthreads();
    ssm_filter_body(Bm, C, dth, D, f, S, N, ldf, h, pw, lds);
}

hipError_t launch_ssm_filter(const float *A, const float *Bm, const float *C, const float *dt,
                             float *f, int H, int S, int64_t N, hipStream_t s) {
    return launch(k_ssm_filter, dim3(H), dim3(512), 0, s, A, Bm, C, dt, (const float *)nullptr, f, S, N, N);
}

// ---------------------------------------------------------------- state passing

// Workspace layout (256-byte aligned blocks), by path.  Both start with
//   fT  [H, T]            chunk filter with D folded into tap 0            fp32
// fp32 activations (vector-ALU projections) then hold
//   E   [H, S, 65]        Abar^l, l = 0..64                                complex
//   G   [H, S, T/64 + 1]  Abar^(64 i), i = 0..T/64                         complex
//   sc  [B, H, C, 64]     per-chunk state contributions                    complex
// and 16-bit activations (matrix-core projections, modes padded to 64)
//   Et  [H, 128, 64]      row 2j+p, column l: part p of Abar_j^(63-l)      fp16
//   Rt  [H, 64, 128]      row l, column 2j+p: 2 Re / -2 Im of C_j Abar_j^(l+1)  fp16
//   Pc  [H, 64, 8]        Bbar_j Abar_j^(1024 (NCT-1-ih))                  complex
//   Qc  [H, 64, 16]       Abar_j^(64 (TL-1-il)), zero for il >= TL         complex
//   Px  [H, 64, 8]        Abar_j^(1024 ih)                                 complex
//   Qx  [H, 64, 16]       Abar_j^(64 il), zero for il >= TL                complex
//   aT  [H, 64]           Abar_j^T                                         complex
// with T2 = T/64 columns i = 16 ih + il, NCT = ceil(T2/16), TL = min(T2, 16).
// The workspace size the API reports is the larger of the two.
struct SpLayout {
    size_t fT, E, G, sc, Et, Rt, Pc, Qc, Px, Qx, aT, total;
};

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

static SpLayout sp_layout(int64_t B, int64_t H, int64_t N, int64_t S, int64_t T, bool f32) {
    SpLayout L{};
    const int64_t C = N / T, T2 = T / 64;
    size_t o = 0;
    L.fT = o; o += al256((size_t)H * T * 4);
    if (f32) {
        L.E = o; o += al256((size_t)H * S * 65 * 8);
        L.G = o; o += al256((size_t)H * S * (T2 + 1) * 8);
        L.sc = o; o += al256((size_t)B * H * C * 64 * 8);
    } else {
        L.Et = o; o += al256((size_t)H * 128 * 64 * 2);
        L.Rt = o; o += al256((size_t)H * 64 * 128 * 2);
        L.Pc = o; o += al256((size_t)H * 64 * 8 * 8);
        L.Qc = o; o += al256((size_t)H * 64 * 16 * 8);
        L.Px = o; o += al256((size_t)H * 64 * 8 * 8);
        L.Qx = o; o += al256((size_t)H * 64 * 16 * 8);
        L.aT = o; o += al256((size_t)H * 64 * 8);
    }
    L.total = o;
    return L;
}

size_t state_pass_workspace(int64_t B, int64_t H, int64_t N, int64_t S, int64_t T) {
    return std::max(sp_layout(B, H, N, S, T, true).total, sp_layout(B, H, N, S, T, false).total);
}

size_t state_pass_workspace_io(int64_t B, int64_t H, int64_t N, int64_t S, int64_t T, int io) {
    return sp_layout(B, H, N, S, T, io == IO_F32).total;
}

__global__ __launch_bounds__(256) void k_sp_tables(const float *__restrict__ A,
                                                  const float *__restrict__ dt, cf *__restrict__ E,
                                                  cf *__restrict__ G, int S, int T2) {
    const int h = blockIdx.x;
    const double dth = (double)dt[h];
    const int per = 65 + T2 + 1;
    for (int e = threadIdx.x; e < S * per; e += 256) {
        const int j = e / per, r = e % per;
        const float *a = A + ((size_t)h * S + j) * 2;
        const double are = dth * (double)a[0], aim = dth * (double)a[1];
        if (r < 65) E[((size_t)h * S + j) * 65 + r] = abar_pow(are, aim, (double)r);
        else G[((size_t)h * S + j) * (T2 + 1) + (r - 65)] = abar_pow(are, aim, 64.0 * (r - 65));
    }
}

// Chunk convolution: one workgroup per channel; rows are the B*C chunk-rows
// (b, c) of that channel, paired two by two into complex signals.
template <int LOG2M, int IO>
__global__ __launch_bounds__(Plan<LOG2M>::NT) void k_sp_chunk_conv(
    const typename io_elem<IO>::T *__restrict__ u, const float *__restrict__ fT,
    typename io_elem<IO>::T *__restrict__ y, int B, int H, int64_t N, int T) {
    using T_ = typename io_elem<IO>::T;
    __shared__ cf lds[Plan<LOG2M>::LDS_ELEMS];
    const int tid = threadIdx.x;
    const int h = blockIdx.x;
    const int C = (int)(N / T);
    const float *fh = fT + (size_t)h * T;

    FiltReg<LOG2M> F;
    auto ldf = [&](int pos) -> cf { return mk(pos < T ? fh[pos] : 0.f, 0.f); };
    filter_spectrum<LOG2M>(lds, tid, ldf, F);

    const int rows = B * C;
    for (int r0 = 0; r0 < rows; r0 += 2) {
        const bool has1 = (r0 + 1) < rows;
        const int b0 = r0 / C, c0 = r0 % C, b1 = (r0 + 1) / C, c1 = (r0 + 1) % C;
        const size_t o0 = ((size_t)b0 * H + h) * N + (size_t)c0 * T;
        const size_t o1 = ((size_t)b1 * H + h) * N + (size_t)c1 * T;
        auto ld = [&](int pos) -> cf {
            if (pos >= T) return mk(0.f, 0.f);
            return mk(ld_io<IO>(u + o0 + pos), has1 ? ld_io<IO>(u + o1 + pos) : 0.f);
        };
        auto st = [&](int pos, cf v) {
            if (pos < T) {
                st_io<IO>(y + o0 + pos, v.x);
                if (has1) st_io<IO>(y + o1 + pos, v.y);
            }
        };
        conv_signal<LOG2M>(lds, tid, F, ld, st);
    }
}

// State contribution of one chunk-row (b, h, c):
//   s_j = Bbar_j sum_i Abar_j^{64 (T2-1-i)} sum_l Abar_j^{63-l} u[c T + 64 i + l]
// (= M_ux u_c with Abar^{T-1-k} split as Abar^{64(T2-1-i)} Abar^{63-l}).
template <int IO>
__global__ __launch_bounds__(256) void k_sp_contrib(const typename io_elem<IO>::T *__restrict__ u,
                                                   const float *__restrict__ Bm,
                                                   const float *__restrict__ dt,
                                                   const cf *__restrict__ E, const cf *__restrict__ G,
                                                   cf *__restrict__ sc, int B, int H, int64_t N, int S,
                                                   int T) {
    extern __shared__ float smem[];
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int C = gridDim.x, T2 = T / 64;
    float *us = smem;                       // [T]
    cf *Er = (cf *)(smem + T);              // [64][64]: Er[l][j] = Abar_j^{63-l}
    cf *part = Er + 64 * 64;                // [4][64]
    const int tid = threadIdx.x;
    const size_t ou = ((size_t)b * H + h) * N + (size_t)c * T;
    for (int e = tid; e < T; e += 256) us[e] = ld_io<IO>(u + ou + e);
    for (int e = tid; e < 64 * 64; e += 256) {
        const int l = e >> 6, j = e & 63;
        Er[e] = (j < S) ? E[((size_t)h * S + j) * 65 + (63 - l)] : mk(0.f, 0.f);
    }
    __syncthreads();
    const int j = tid & 63, q = tid >> 6;
    cf acc = mk(0.f, 0.f);
    if (j < S) {
        const cf *Gj = G + ((size_t)h * S + j) * (T2 + 1);
        for (int i = q; i < T2; i += 4) {
            cf v = mk(0.f, 0.f);
            const float *ui = us + 64 * i;
#pragma unroll 8
            for (int l = 0; l < 64; ++l) {
                const cf e = Er[l * 64 + j];
                const float x = ui[l];
                v.x = fmaf(e.x, x, v.x);
                v.y = fmaf(e.y, x, v.y);
            }
            acc = cadd(acc, cmul(Gj[T2 - 1 - i], v));
        }
    }
    part[q * 64 + j] = acc;
    __syncthreads();
    if (tid < S) {
        cf s = cadd(cadd(part[tid], part[64 + tid]), cadd(part[128 + tid], part[192 + tid]));
        const float *bb = Bm + ((size_t)h * S + tid) * 2;
        const float d = dt[h];
        s = cmul(s, mk(d * bb[0], d * bb[1]));
        sc[(((size_t)b * H + h) * C + c) * 64 + tid] = s;
    }
}

// Carry the state into chunk c and add its free response:
//   x_{c-1} = Abar^T x_{c-2} + s_{c-1}  (scan from x_in, or zero)
//   y[c T + 64 i + l] += 2 Re(sum_j C_j Abar_j^{l+1} Abar_j^{64 i} x_{c-1,j})
// The last chunk also writes x_out = Abar^T x_{C-2} + s_{C-1}.
template <int IO>
__global__ __launch_bounds__(256) void k_sp_correct(typename io_elem<IO>::T *__restrict__ y,
                                                   const float *__restrict__ Cc,
                                                   const cf *__restrict__ E, const cf *__restrict__ G,
                                                   const cf *__restrict__ sc,
                                                   const float *__restrict__ x_in,
                                                   float *__restrict__ x_out, int B, int H, int64_t N,
                                                   int S, int T) {
    extern __shared__ float smem[];
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int C = gridDim.x, T2 = T / 64;
    cf *Rt = (cf *)smem;              // [64 j][64 l]: C_j Abar_j^{l+1}
    cf *X = Rt + 64 * 64;             // [64 j][T2]:  Abar_j^{64 i} x_j
    __shared__ int any_state;
    const int tid = threadIdx.x;
    const size_t orow = ((size_t)b * H + h);
    if (tid == 0) any_state = 0;
    __syncthreads();
    if (tid < 64) {
        const int j = tid;
        cf x = mk(0.f, 0.f);
        if (j < S) {
            if (x_in) x = mk(x_in[(orow * S + j) * 2], x_in[(orow * S + j) * 2 + 1]);
            const cf aT = G[((size_t)h * S + j) * (T2 + 1) + T2];
            for (int cc = 0; cc < c; ++cc) x = cadd(cmul(aT, x), sc[(orow * C + cc) * 64 + j]);
            if (c == C - 1 && x_out) {
                const cf xo = cadd(cmul(aT, x), sc[(orow * C + c) * 64 + j]);
                x_out[(orow * S + j) * 2] = xo.x;
                x_out[(orow * S + j) * 2 + 1] = xo.y;
            }
            if (x.x != 0.f || x.y != 0.f) atomicOr(&any_state, 1);
        }
        // stash the state in X[j][0] temporarily via registers below
        for (int l = 0; l < 64; ++l) {
            cf r = mk(0.f, 0.f);
            if (j < S) {
                const cf cj = mk(Cc[((size_t)h * S + j) * 2], Cc[((size_t)h * S + j) * 2 + 1]);
                r = cmul(cj, E[((size_t)h * S + j) * 65 + l + 1]);
            }
            Rt[j * 64 + l] = r;
        }
        for (int i = 0; i < T2; ++i)
            X[j * T2 + i] = (j < S) ? cmul(G[((size_t)h * S + j) * (T2 + 1) + i], x) : mk(0.f, 0.f);
    }
    __syncthreads();
    if (!any_state) return;
    const int l = tid & 63, iq = tid >> 6;
    typename io_elem<IO>::T *yr = y + orow * N + (size_t)c * T;
    for (int i = iq; i < T2; i += 4) {
        float acc = 0.f;
        for (int j = 0; j < S; ++j) {
            const cf r = Rt[j * 64 + l], xv = X[j * T2 + i];
            acc = fmaf(r.x, xv.x, fmaf(-r.y, xv.y, acc));
        }
        const int t = 64 * i + l;
        st_io<IO>(yr + t, ld_io<IO>(yr + t) + 2.f * acc);
    }
}

// ---------------------------------------------------------------- matrix-core projections
// For 16-bit activations both projections of the state passing run as small
// dense products on the matrix cores (fp16 operands, fp32 accumulation), with
// the chunk index split as k = 64 i + l and i = 16 ih + il:
//   s_j    = sum_ih Pc[j][ih] sum_il Qc[j][il] V[j][16 ih + il],
//   V[j][i] = sum_l Abar_j^(63-l) u[64 i + l]                    (Et x U, K = l)
//   corr[64 i + l] = sum_(j,p) Rt[l][2j+p] X[2j+p][i],           (Rt x X, K = 2j+p)
//   X[j][i] = Abar_j^(64 i) x_j = Px[j][ih] Qx[j][il] x_j.
// The operands of each product are scaled by a power of two into fp16 range
// and the scale is undone on the fp32 results.


// fp64 -> fp32 -> fp16 with the two hardware conversions (the empty asm keeps
// the compiler from fusing them into one software-rounded fp64 -> fp16
// conversion, about forty instructions)
__device__ __forceinline__ uint16_t f16bits(double x) {
    float f = (float)x;
    asm volatile("" : "+v"(f));
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// The tables of channel h from its powers pw (ssm_powers), by the workgroup's
// NT threads: eight runs of powers per mode (the modes past S are written as
// zeros):
//   runs 0..3  Abar^p, p = 16 q .. 16 q + 15 -> Et (l = 63 - p), Rt (l = p - 1)
//   run 4      Abar^64                      -> Rt (l = 63)
//   run 5      Abar^(64 k), k < 16         -> Qx[k], Qc[TL - 1 - k]
//   run 6      Abar^(1024 k), k < 8        -> Px[k], Pc[NCT - 1 - k] (times Bbar)
//   run 7      Abar^T                      -> aT
constexpr int SP_EST = 66;                                // Et row stride in LDS (16-bit units)
constexpr int SP_TAB_LDS = 128 * SP_EST * 2 + 64 * 128 * 2;  // bytes: Et, then Rt

template <int NT>
__device__ __forceinline__ void sp_tables_body(const float *__restrict__ Bm, const float *__restrict__ Cc, double dth,
                               uint16_t *__restrict__ Et, uint16_t *__restrict__ Rt, cf *__restrict__ Pc,
                               cf *__restrict__ Qc, cf *__restrict__ Px, cf *__restrict__ Qx, cf *__restrict__ aT,
                               int S, int T, int h, const double2 (*pw)[64], uint16_t *lds) {
    const int T2 = T / 64, NCT = (T2 + 15) / 16, TL = T2 < 16 ? T2 : 16;
    // Et and Rt are built in LDS and written out with 16-byte stores.  The
    // lanes of a wave take 64 modes of one run, so the runs' different code
    // paths never diverge within a wave; Et rows are padded to 66 entries so
    // those lanes' writes spread over the banks.
    constexpr int EST = SP_EST;
    uint16_t *const Eh = lds, *const Rh = lds + 128 * EST;
    // cnt powers st^k times p, k < cnt
    auto run_ = [&](double2 p, double2 st, int cnt, auto &&emit) {
        for (int k = 0; k < cnt; ++k) {
            emit(k, p.x, p.y);
            p = dmul(p, st);
        }
    };
    for (int e = threadIdx.x; e < 64 * 8; e += NT) {
        const int j = e & 63, run = e >> 6;
        const bool on = j < S;
        double br = 0.0, bi = 0.0, cr = 0.0, ci = 0.0;
        if (on) {
            const size_t o = ((size_t)h * S + j) * 2;
            br = dth * (double)Bm[o];
            bi = dth * (double)Bm[o + 1];
            cr = (double)Cc[o];
            ci = (double)Cc[o + 1];
        }
        // modes past S: all-zero tables (the power run is evaluated and masked)
        const double on_d = on ? 1.0 : 0.0;
        auto et_rt = [&](int p, double pr, double pi) {
            pr *= on_d;
            pi *= on_d;
            if (p <= 63) {
                Eh[(2 * j) * EST + (63 - p)] = f16bits(pr);
                Eh[(2 * j + 1) * EST + (63 - p)] = f16bits(pi);
            }
            if (p >= 1) {
                const int l = p - 1;
                const double zr = cr * pr - ci * pi, zi = cr * pi + ci * pr;
                Rh[l * 128 + 2 * j] = f16bits(2.0 * zr);
                Rh[l * 128 + 2 * j + 1] = f16bits(-2.0 * zi);
            }
        };
        const double2 one = double2{1.0, 0.0};
        if (run < 4) {
            double2 p = one;
            for (int r = 0; r < run; ++r) p = dmul(p, pw[1][j]);
            run_(p, pw[0][j], 16, [&](int k, double pr, double pi) { et_rt(16 * run + k, pr, pi); });
        } else if (run == 4) {
            et_rt(64, pw[2][j].x, pw[2][j].y);
        } else if (run == 5) {
            run_(one, pw[2][j], 16, [&](int k, double pr, double pi) {
                const bool ok = on && k < TL;
                const cf v = ok ? mk((float)pr, (float)pi) : mk(0.f, 0.f);
                Qx[((size_t)h * 64 + j) * 16 + k] = v;
                Qc[((size_t)h * 64 + j) * 16 + (k < TL ? TL - 1 - k : k)] = v;
            });
        } else if (run == 6) {
            run_(one, pw[3][j], 8, [&](int k, double pr, double pi) {
                const bool ok = on && k < NCT;
                Px[((size_t)h * 64 + j) * 8 + k] = ok ? mk((float)pr, (float)pi) : mk(0.f, 0.f);
                Pc[((size_t)h * 64 + j) * 8 + (k < NCT ? NCT - 1 - k : k)] =
                    ok ? mk((float)(br * pr - bi * pi), (float)(br * pi + bi * pr)) : mk(0.f, 0.f);
            });
        } else {
            // Abar^T, T = 64 2^m: squarings of Abar^64
            double2 p = pw[2][j];
            for (int t = 64; t < T; t <<= 1) p = dmul(p, p);
            aT[(size_t)h * 64 + j] = on ? mk((float)p.x, (float)p.y) : mk(0.f, 0.f);
        }
    }
    __syncthreads();
    using u32x4 = mf::u32x4;
    u32x4 *eo = (u32x4 *)(Et + (size_t)h * 128 * 64), *ro = (u32x4 *)(Rt + (size_t)h * 64 * 128);
    for (int e = threadIdx.x; e < 128 * 64 / 8; e += NT) {
        const uint32_t *er = (const uint32_t *)(Eh + (e >> 3) * EST + 8 * (e & 7));
        eo[e] = u32x4{er[0], er[1], er[2], er[3]};
        ro[e] = ((const u32x4 *)Rh)[e];
    }
}

// The per-channel parameters of the 16-bit state passing in one launch, one
// workgroup of 8 waves per channel: the powers, the chunk filter (with D
// folded into tap 0) and then, in the same LDS, the projection tables.
__global__ __launch_bounds__(512) void k_sp_params(const float *__restrict__ A, const float *__restrict__ Bm,
                                                  const float *__restrict__ Cc, const float *__restrict__ dt,
                                                  const float *__restrict__ D, float *__restrict__ fT,
                                                  uint16_t *__restrict__ Et, uint16_t *__restrict__ Rt,
                                                  cf *__restrict__ Pc, cf *__restrict__ Qc, cf *__restrict__ Px,
                                                  cf *__restrict__ Qx, cf *__restrict__ aT, int S, int T) {
    static_assert(SP_TAB_LDS <= FILT_LDS * 4, "the tables fit the filter's LDS");
    __shared__ __attribute__((aligned(16))) float lds[FILT_LDS];
    __shared__ double2 pw[4][64];
    const int h = blockIdx.x;
    const double dth = (double)dt[h];
    ssm_powers(A, dth, S, h, pw);
    __syncthreads();
    ssm_filter_body(Bm, Cc, dth, D, fT, S, (int64_t)T, (int64_t)T, h, pw, lds);
    __syncthreads();  // (the filter's operands have been read)
    sp_tables_body<512>(Bm, Cc, dth, Et, Rt, Pc, Qc, Px, Qx, aT, S, T, h, pw, (uint16_t *)lds);
}

__device__ __forceinline__ float sp_wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Both projections of one (batch row b, channel h), walking its chunks in
// order; every wave carries its own copy of the state (lane l: mode l), so
// the state update needs no barrier of its own.  Eight waves; for each chunk
// c (the correction goes first, so that its stores are issued before the
// next chunk's loads and are long complete when those are waited for):
//   1. the chunk's activations are staged in LDS as fp16 (bf16 inputs scaled
//      by a power of two into fp16 range);
//   2. contribution: wave w owns modes 8w .. 8w+7 (Et row tile w) and all
//      column tiles, so its Et operands stay in registers;
//   3. correction with the state carried into the chunk,
//        y[64 i + l] += 2 Re sum_j (C_j Abar_j^(l+1) x_j) Abar_j^(64 i):
//      the power table G = Abar^(64 i) is the B operand, built once in LDS;
//      wave w owns output rows l = 16 (w % 4) .. +15 and column tiles
//      4 (w / 4) .. +3, scales its Rt operands (in registers) by the state,
//      and updates y in place;
//   4. x <- Abar^T x + s, in every wave at the top of the next chunk (the
//      contributions s are complete at the chunk's last barrier).
// Two barriers per chunk: after staging, and after the contribution.  The
// next chunk's activations are loaded while the current one is used.
constexpr int SP_USTR = 72;   // staged chunk: 64 samples per row i, padded (bank spread)
constexpr int SP_XSTR = 136;  // G operand: 128 (mode, part) entries per column i, padded

template <int IO>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void k_sp_proj_mfma(const typename io_elem<IO>::T *__restrict__ u,
                                                     typename io_elem<IO>::T *__restrict__ y,
                                                     const uint16_t *__restrict__ Et,
                                                     const uint16_t *__restrict__ Rt,
                                                     const cf *__restrict__ Pc, const cf *__restrict__ Qc,
                                                     const cf *__restrict__ Px, const cf *__restrict__ Qx,
                                                     const cf *__restrict__ aT, const float *__restrict__ x_in,
                                                     float *__restrict__ x_out, int H, int64_t N, int S, int T) {
    using namespace mf;
    using T_ = typename io_elem<IO>::T;
    constexpr int NWV = 8;
    const int h = blockIdx.x, b = blockIdx.y;
    const int C = (int)(N / T), T2 = T >> 6, NCT = (T2 + 15) >> 4;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, il = lane & 15, g = lane >> 4;
    const int lr = w & 3, ch = w >> 2;  // correction rows 16 lr .., column tiles 4 ch ..
    __shared__ __attribute__((aligned(16))) uint16_t us[128 * SP_USTR];
    __shared__ __attribute__((aligned(16))) uint16_t xs[128 * SP_XSTR];
    __shared__ cf pcs[64 * 8], pxs[64 * 8], qxs[64 * 16];
    __shared__ cf xw[NWV][64], sst[64];
    __shared__ float red[NWV], rmax[NWV];
    const size_t orow = (size_t)b * H + h;
    // tables and the initial state
    for (int e = tid; e < 64 * 8; e += 512) {
        pcs[e] = Pc[(size_t)h * 512 + e];
        pxs[e] = Px[(size_t)h * 512 + e];
    }
    for (int e = tid; e < 64 * 16; e += 512) qxs[e] = Qx[(size_t)h * 1024 + e];
    // rows i >= T2 of both operands stay zero, so the column-tile loops need
    // no tests (the tables are zero past the chunk's tiles as well)
    for (int e = tid; e < 128 * SP_USTR / 8; e += 512) ((u32x4 *)us)[e] = u32x4{0u, 0u, 0u, 0u};
    for (int e = tid; e < 128 * SP_XSTR / 8; e += 512) ((u32x4 *)xs)[e] = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
    // G[(j, part)][i] = Abar_j^(64 i) as fp16 (|G| <= 1 for stable modes)
    for (int e = tid; e < 64 * T2; e += 512) {
        const int j = e & 63, i = e >> 6;
        const cf X = cmul(pxs[j * 8 + (i >> 4)], qxs[j * 16 + (i & 15)]);
        *(uint32_t *)(xs + i * SP_XSTR + 2 * j) = pk(X.x, X.y);
    }
    // every wave carries its own copy of the state: lane l holds mode l
    cf xl = mk(0.f, 0.f);
    if (x_in && lane < S) xl = mk(x_in[(orow * S + lane) * 2], x_in[(orow * S + lane) * 2 + 1]);
    // matrix operands in registers
    const uint16_t *Eh = Et + (size_t)h * 128 * 64, *Rh = Rt + (size_t)h * 64 * 128;
    half8 Ea[2], Ra[4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
        Ea[ks] = __builtin_bit_cast(half8, *(const u32x4 *)(Eh + (16 * w + il) * 64 + 32 * ks + 8 * g));
    const int j0 = 8 * w + 2 * g;  // modes of this lane's accumulator pairs: j0, j0 + 1
    const cf qc0 = Qc[((size_t)h * 64 + j0) * 16 + il], qc1 = Qc[((size_t)h * 64 + j0 + 1) * 16 + il];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        Ra[ks] = __builtin_bit_cast(half8, *(const u32x4 *)(Rh + (16 * lr + il) * 128 + 32 * ks + 8 * g));
    const cf aTl = aT[(size_t)h * 64 + lane];
    // max |Rt entry| < 2^er over the workgroup (sets the state scale below)
    int er = 0;
    {
        float m = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf((float)Ra[ks][e]));
        m = sp_wave_max(m);
        if (lane == 0) rmax[w] = m;
        __syncthreads();
        m = 0.f;
#pragma unroll
        for (int k = 0; k < NWV; ++k) m = fmaxf(m, rmax[k]);
        if (m > 0.f) (void)frexpf(m, &er);
    }
    // chunk loads: T / 8 groups of 8 activations (at most 2 per thread), and
    // the 4 outputs per column tile this lane corrects (read-modify-write).
    const int nq = T >> 3;
    u32x4 pre[2];
    u32x2 ypre[4];
    // Loads go through buffer resources: a chunk past the last (the loads
    // issued during the last chunk) or outputs that no correction will use
    // (chunk 0 without x_in) get an empty resource, whose loads read zero and
    // touch no memory, with no branch around them.
    auto load_chunk = [&](int c, bool uv, bool yv) {
        const __amdgpu_buffer_rsrc_t ur = row_rsrc(u + orow * N + (size_t)c * T, uv ? 2 * T : 0);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int q = tid + 512 * k;
            if (q < nq) pre[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ur, 16 * q, 0, 0));
        }
        const __amdgpu_buffer_rsrc_t yrs = row_rsrc(y + orow * N + (size_t)c * T, yv ? 2 * T : 0);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            const int ct = 4 * ch + c4, i = 16 * ct + il;
            if (ct < NCT && i < T2)
                ypre[c4] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(yrs, 2 * (64 * i + 16 * lr + 4 * g), 0, 0));
        }
    };
    load_chunk(0, true, x_in != nullptr);
    __syncthreads();
    for (int c = 0; c < C; ++c) {
        // 1. stage (fp16, scaled for bf16 inputs)
        float su = 1.f;
        if constexpr (IO == IO_BF16) {
            float m = 0.f;
#pragma unroll
            for (int k = 0; k < 2; ++k)
                if (tid + 512 * k < nq) {
                    const uint32_t d4[4] = {pre[k].x, pre[k].y, pre[k].z, pre[k].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        m = fmaxf(m, fmaxf(fabsf(__uint_as_float(d4[e] << 16)), fabsf(__uint_as_float(d4[e] & 0xffff0000u))));
                }
            m = sp_wave_max(m);
            if (lane == 0) red[w] = m;
            __syncthreads();
            m = 0.f;
#pragma unroll
            for (int k = 0; k < NWV; ++k) m = fmaxf(m, red[k]);
            int ex = 0;
            if (m > 0.f) (void)frexpf(m, &ex);
            su = ldexpf(1.f, 14 - ex);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int q = tid + 512 * k;
            if (q < nq) {
                u32x4 v = pre[k];
                if constexpr (IO == IO_BF16) {
                    const uint32_t d4[4] = {v.x, v.y, v.z, v.w};
                    uint32_t o4[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o4[e] = pk(__uint_as_float(d4[e] << 16) * su, __uint_as_float(d4[e] & 0xffff0000u) * su);
                    v = u32x4{o4[0], o4[1], o4[2], o4[3]};
                }
                *(u32x4 *)(us + (q >> 3) * SP_USTR + 8 * (q & 7)) = v;
            }
        }
        // (taken into registers of their own here, at the top of the pass,
        //  so that no later use waits behind the stores issued meanwhile)
        u32x2 ycur[4];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            ycur[c4] = ypre[c4];
            asm volatile("" : "+v"(ycur[c4]));
        }
        // correction operand: this wave's Rt rows times the state carried in,
        // (2 Re R, -2 Im R) (x) -> (2 Re (R x), -2 Im (R x)), with x scaled by
        // sx = 2^(14 - e - er), max |x| < 2^e, so every product stays below 2^14
        // 4. (for the previous chunk) x <- Abar^T x + s, in every wave; the
        //    contributions s were completed at the previous chunk's last barrier
        if (c > 0) xl = cadd(cmul(aTl, xl), sst[lane]);
        const float xm = sp_wave_max(fmaxf(fabsf(xl.x), fabsf(xl.y)));
        xw[w][lane] = xl;
        const bool corr = xm > 0.f;
        float sx = 1.f;
        half8 Rx[4];
        if (corr) {
            int ex = 0;
            (void)frexpf(xm, &ex);
            sx = ldexpf(1.f, 14 - ex - er);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const u32x4 r4 = __builtin_bit_cast(u32x4, Ra[ks]);
                uint32_t o4[4] = {r4.x, r4.y, r4.z, r4.w}, xc[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const cf x = xw[w][16 * ks + 4 * g + q];  // mode of slot pair q
                    xc[q] = pk(x.x * sx, -x.y * sx);
                }
                // (a + i b) conj(x sx) with (a, b) = (2 Re R, -2 Im R); the
                // results are matrix-core operands (the helper ends with the
                // wait states that needs)
                cmulh_n(o4, xc);
                Rx[ks] = __builtin_bit_cast(half8, u32x4{o4[0], o4[1], o4[2], o4[3]});
            }
        }
        __syncthreads();
        // 3. correction: y += 2 Re(C Abar^(t+1) x), rows l = 16 lr + 4 g + v
        if (corr) {
            const float inv = 1.0f / sx;
            T_ *yr = y + orow * N + (size_t)c * T;
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                const int ct = 4 * ch + c4, i = 16 * ct + il;
                {
                    f4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        d = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            Rx[ks], __builtin_bit_cast(half8, *(const u32x4 *)(xs + i * SP_XSTR + 32 * ks + 8 * g)), d, 0, 0, 0);
                    if (i < T2) {
                        T_ *p = yr + 64 * i + 16 * lr + 4 * g;
                        const uint32_t y01 = ycur[c4].x, y23 = ycur[c4].y;
                        const T_ *yv = (const T_ *)&y01;
                        const T_ *yw = (const T_ *)&y23;
                        T_ o[4];
                        o[0] = yv[0]; o[1] = yv[1]; o[2] = yw[0]; o[3] = yw[1];
#pragma unroll
                        for (int v = 0; v < 4; ++v) st_io<IO>(o + v, ld_io<IO>(o + v) + d[v] * inv);
                        const uint32_t a = *(const uint32_t *)&o[0], bb = *(const uint32_t *)&o[2];
                        *(u32x2 *)p = u32x2{a, bb};
                    }
                }
            }
        }
        // next chunk's loads (issued on every pass, with empty resources on
        // the last: in a branch of their own they end up after the barrier)
        load_chunk(c + 1 < C ? c + 1 : c, c + 1 < C, c + 1 < C);
        // 2. contribution (column tiles unrolled, so their reads and products
        //    overlap; the per-lane factor qc is applied once at the end)
        cf acc0 = mk(0.f, 0.f), acc1 = mk(0.f, 0.f);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
            const int i = 16 * ct + il;
            half8 Bop[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                Bop[ks] = __builtin_bit_cast(half8, *(const u32x4 *)(us + i * SP_USTR + 32 * ks + 8 * g));
            const f4 z = {0.f, 0.f, 0.f, 0.f};
            f4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ea[0], Bop[0], z, 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ea[1], Bop[1], d, 0, 0, 0);
            acc0 = cadd(acc0, cmul(pcs[j0 * 8 + ct], mk(d[0], d[1])));
            acc1 = cadd(acc1, cmul(pcs[(j0 + 1) * 8 + ct], mk(d[2], d[3])));
        }
        acc0 = cmul(qc0, acc0);
        acc1 = cmul(qc1, acc1);
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            acc0.x += __shfl_xor(acc0.x, o, 64);
            acc0.y += __shfl_xor(acc0.y, o, 64);
            acc1.x += __shfl_xor(acc1.x, o, 64);
            acc1.y += __shfl_xor(acc1.y, o, 64);
        }
        if (il == 0) {
            const float inv = 1.0f / su;
            sst[j0] = cscale(acc0, inv);
            sst[j0 + 1] = cscale(acc1, inv);
        }
        __syncthreads();
    }
    if (x_out && w == 0) {
        xl = cadd(cmul(aTl, xl), sst[lane]);
        if (lane < S) {
            x_out[(orow * S + lane) * 2] = xl.x;
            x_out[(orow * S + lane) * 2 + 1] = xl.y;
        }
    }
}

// Same chunk convolution on the MFMA block-FFT engine (fp16 / bf16 I/O).
template <int LOG2M, int IO>
__global__ __launch_bounds__(mf::Shape<LOG2M>::NT) __attribute__((amdgpu_waves_per_eu(mf::Shape<LOG2M>::WPE))) void k_sp_chunk_conv_mfma(
    const typename io_elem<IO>::T *__restrict__ u, const float *__restrict__ fT,
    typename io_elem<IO>::T *__restrict__ y, int B, int H, int64_t N, int T) {
    using SH = mf::Shape<LOG2M>;
    constexpr int KIND = IO == IO_F16 ? mf::IN_F16 : mf::IN_BF16;
    __shared__ __attribute__((aligned(16))) uint32_t smem[SH::LDS_DWORDS];
    mf::Engine<LOG2M, KIND> E(smem);
    E.init();
    const int h = blockIdx.x;
    const int C = (int)(N / T);
    const float *fh = fT + (size_t)h * T;
    const int hb = mf::half_bits(T);
    const int rows = B * C;
    auto off = [&](int r) -> size_t {
        const int b = r / C, c = r % C;
        return ((size_t)b * H + h) * N + (size_t)c * T;
    };
    // complex signal `sig` = row chunks 2 sig (real part), 2 sig + 1
    // (imaginary); chunks past the last get empty resources
    auto rowp = [&](int sig) -> mf::RowBufs {
        const int r = 2 * sig;
        const int nb0 = (r < rows) ? 2 * T : 0;
        const int nb1 = (r + 1 < rows) ? 2 * T : 0;
        const uint16_t *ub = (const uint16_t *)u;
        uint16_t *yb = (uint16_t *)y;
        const size_t o0 = (r < rows) ? off(r) : 0;
        const size_t o1 = (r + 1 < rows) ? off(r + 1) : o0;
        return {mf::row_rsrc(ub + o0, nb0), mf::row_rsrc(ub + o1, nb1), mf::row_rsrc(yb + o0, nb0),
                mf::row_rsrc(yb + o1, nb1)};
    };
    E.run_raw(mf::row_rsrc(fh, 4 * T), 0.f, rowp, (rows + 1) / 2, hb);
}

template <int LOG2M, int IO>
static hipError_t sp_conv(const void *u, const float *fT, void *y, int B, int H, int64_t N, int T,
                          hipStream_t s) {
    using T_ = typename io_elem<IO>::T;
    if constexpr (IO != IO_F32 && LOG2M >= 9) {
        return launch(k_sp_chunk_conv_mfma<LOG2M, IO>, dim3(H), dim3(mf::Shape<LOG2M>::NT), 0, s, (const T_ *)u,
                      fT, (T_ *)y, B, H, N, T);
    } else {
        return launch(k_sp_chunk_conv<LOG2M, IO>, dim3(H), dim3(Plan<LOG2M>::NT), 0, s, (const T_ *)u, fT,
                      (T_ *)y, B, H, N, T);
    }
}

// Dynamic LDS limits of the fp32 projection kernels, set once per device
// (for the largest chunk, T = 8192) with the status of the calls kept.
template <int IO>
static hipError_t sp_f32_attributes() {
    constexpr int kDev = 64;
    static std::atomic<int> state[kDev];  // 0 unset, 1 set, else -(hipError_t)
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kDev) return hipErrorInvalidDevice;
    const int st = state[dev].load(std::memory_order_acquire);
    if (st == 1) return hipSuccess;
    if (st < 0) return (hipError_t)(-st);
    const int sm_c = 8192 * 4 + 64 * 64 * 8 + 4 * 64 * 8;
    const int sm_x = 64 * 64 * 8 + 64 * (8192 / 64) * 8;
    e = hipFuncSetAttribute((const void *)k_sp_contrib<IO>, hipFuncAttributeMaxDynamicSharedMemorySize, sm_c);
    if (e == hipSuccess)
        e = hipFuncSetAttribute((const void *)k_sp_correct<IO>, hipFuncAttributeMaxDynamicSharedMemorySize, sm_x);
    state[dev].store(e == hipSuccess ? 1 : -(int)e, std::memory_order_release);
    return e;
}

__global__ __launch_bounds__(256) void k_state_copy(const float *__restrict__ x_in, float *__restrict__ x_out,
                                                   int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < 2 * n; i += (int64_t)gridDim.x * 256)
        x_out[i] = x_in ? x_in[i] : 0.f;
}

hipError_t launch_state_copy(const float *x_in, float *x_out, int64_t n, hipStream_t s) {
    const int64_t blocks = std::min<int64_t>((2 * n + 255) / 256, 65535);
    return launch(k_state_copy, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, s, x_in, x_out, n);
}

template <int IO>
static hipError_t sp_run(const void *u, const float *A, const float *Bm, const float *C,
                         const float *dt, const float *D, const float *x_in, float *x_out, void *y,
                         int B, int H, int64_t N, int S, int T, void *ws, hipStream_t s) {
    using T_ = typename io_elem<IO>::T;
    const SpLayout L = sp_layout(B, H, N, S, T, IO == IO_F32);
    char *w = (char *)ws;
    float *fT = (float *)(w + L.fT);
    cf *E = (cf *)(w + L.E);
    cf *G = (cf *)(w + L.G);
    cf *sc = (cf *)(w + L.sc);
    const int C_ = (int)(N / T), T2 = T / 64;

    hipError_t e;
    if constexpr (IO != IO_F32) {
        e = launch(k_sp_params, dim3(H), dim3(512), 0, s, A, Bm, C, dt, D, fT, (uint16_t *)(w + L.Et),
                   (uint16_t *)(w + L.Rt), (cf *)(w + L.Pc), (cf *)(w + L.Qc), (cf *)(w + L.Px), (cf *)(w + L.Qx),
                   (cf *)(w + L.aT), S, T);
    } else {
        e = launch(k_ssm_filter, dim3(H), dim3(512), 0, s, A, Bm, C, dt, D, fT, S, (int64_t)T, (int64_t)T);
        if (e != hipSuccess) return e;
        e = launch(k_sp_tables, dim3(H), dim3(256), 0, s, A, dt, E, G, S, T2);
    }
    if (e != hipSuccess) return e;
    switch (fused_log2m(T)) {
        case 7: e = sp_conv<7, IO>(u, fT, y, B, H, N, T, s); break;
        case 8: e = sp_conv<8, IO>(u, fT, y, B, H, N, T, s); break;
        case 9: e = sp_conv<9, IO>(u, fT, y, B, H, N, T, s); break;
        case 10: e = sp_conv<10, IO>(u, fT, y, B, H, N, T, s); break;
        case 11: e = sp_conv<11, IO>(u, fT, y, B, H, N, T, s); break;
        case 12: e = sp_conv<12, IO>(u, fT, y, B, H, N, T, s); break;
        case 13: e = sp_conv<13, IO>(u, fT, y, B, H, N, T, s); break;
        case 14: e = sp_conv<14, IO>(u, fT, y, B, H, N, T, s); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    if constexpr (IO != IO_F32) {
        return launch(k_sp_proj_mfma<IO>, dim3(H, B), dim3(512), 0, s, (const T_ *)u, (T_ *)y,
                      (const uint16_t *)(w + L.Et), (const uint16_t *)(w + L.Rt), (const cf *)(w + L.Pc),
                      (const cf *)(w + L.Qc), (const cf *)(w + L.Px), (const cf *)(w + L.Qx),
                      (const cf *)(w + L.aT), x_in, x_out, H, N, S, T);
    } else {
        const size_t sm_c = (size_t)T * 4 + 64 * 64 * 8 + 4 * 64 * 8;
        const size_t sm_x = 64 * 64 * 8 + (size_t)64 * T2 * 8;
        // the dynamic LDS limits are set once per device, for the largest
        // chunk length (T = 8192), and their status is checked
        if ((e = sp_f32_attributes<IO>()) != hipSuccess) return e;
        e = launch(k_sp_contrib<IO>, dim3(C_, H, B), dim3(256), sm_c, s, (const T_ *)u, Bm, dt, E, G, sc, B, H,
                   N, S, T);
        if (e != hipSuccess) return e;
        return launch(k_sp_correct<IO>, dim3(C_, H, B), dim3(256), sm_x, s, (T_ *)y, C, E, G, sc, x_in, x_out,
                      B, H, N, S, T);
    }
}

hipError_t launch_state_pass(const void *u, const float *A, const float *Bm, const float *C,
                             const float *dt, const float *D, const float *x_in, float *x_out,
                             void *y, int B, int H, int64_t N, int S, int T, int io, void *ws,
                             hipStream_t s) {
    switch (io) {
        case IO_F32: return sp_run<IO_F32>(u, A, Bm, C, dt, D, x_in, x_out, y, B, H, N, S, T, ws, s);
        case IO_F16: return sp_run<IO_F16>(u, A, Bm, C, dt, D, x_in, x_out, y, B, H, N, S, T, ws, s);
        case IO_BF16: return sp_run<IO_BF16>(u, A, Bm, C, dt, D, x_in, x_out, y, B, H, N, S, T, ws, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace h3c
