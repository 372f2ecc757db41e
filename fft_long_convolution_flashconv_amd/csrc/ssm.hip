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
// fp32 activations: the chunk convolutions run on the fp32 FFT engine, the
// two projections on the vector ALUs.  16-bit activations: the same update
// with chunks of 64 samples in one pass over the row (k_sp_block below),
// every product on the matrix cores.
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
// Abar^n for the fp16 tables: the phase n dt Im A is formed and reduced by
// whole turns in fp64, then the fp32 sine, cosine and exponential of the
// reduced values (about one ulp of fp32 each)
__device__ __forceinline__ cf apow_f32(double are, double aim, double n) {
    constexpr double kTwoPi = 6.283185307179586232;
    const double ph = aim * n;
    const float phr = (float)fma(-rint(ph * (1.0 / kTwoPi)), kTwoPi, ph);
    float sn, cs;
    sincosf(phr, &sn, &cs);
    const float m = expf((float)(are * n));
    return mk(m * cs, m * sn);
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

// Workspace layout (256-byte aligned blocks), by path.  fp32 activations
// (FFT chunk convolutions, vector-ALU projections):
//   fT  [H, T]            chunk filter with D folded into tap 0            fp32
//   E   [H, S, 65]        Abar^l, l = 0..64                                complex
//   G   [H, S, T/64 + 1]  Abar^(64 i), i = 0..T/64                         complex
//   sc  [B, H, C, 64]     per-chunk state contributions                    complex
// 16-bit activations (block state passing): fb, Eb, Rb, ab, ak, sb as
// described above k_spb_params.  The workspace size the API reports is the
// larger of the two.
struct SpLayout {
    size_t fT, E, G, sc, fb, Eb, Rb, ab, sb, total;
};

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

static SpLayout sp_layout(int64_t B, int64_t H, int64_t N, int64_t S, int64_t T, bool f32) {
    SpLayout L{};
    const int64_t C = N / T, T2 = T / 64;
    size_t o = 0;
    if (f32) {
        L.fT = o; o += al256((size_t)H * T * 4);
        L.E = o; o += al256((size_t)H * S * 65 * 8);
        L.G = o; o += al256((size_t)H * S * (T2 + 1) * 8);
        L.sc = o; o += al256((size_t)B * H * C * 64 * 8);
    } else {
        L.fb = o; o += al256((size_t)H * 64 * 4);
        L.Eb = o; o += al256((size_t)H * 128 * 64 * 2);
        L.Rb = o; o += al256((size_t)H * 64 * 128 * 2);
        L.ab = o; o += al256((size_t)H * 64 * 8);
        L.sb = o; o += al256((size_t)H * 2 * 4);
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

// ---------------------------------------------------------------- block state passing (16-bit)
//
// The state is passed at every block of Q = 64 samples, a refinement of any
// chunk grid T (64 <= T, T | N) the caller names, so output and final state
// are those of the chunked form for every such T.  For block c of a row (the
// 0-based offset t < 64 inside it),
//   y[64 c + t] = sum_{k <= t} f_{t-k} u[64 c + k] + D u[64 c + t]
//               + 2 Re sum_j C_j Abar_j^(t+1) x_{c-1,j}
//   x_c = Abar^64 x_{c-1} + s_c,   s_{c,j} = sum_k Abar_j^(63-k) Bbar_j u[64 c + k]
// i.e. the pages' state passing with chunks of 64: the chunk's own
// convolution is a 64 x 64 lower-triangular Toeplitz product (f_0 .. f_63,
// D folded into f_0), the contribution is M_ux u_c and the correction the
// projection of the carried state; the three are dense products on the
// matrix cores (16x16x32, fp16 operands, fp32 accumulate) over the 16 blocks
// a wave holds at once, and only the state recurrence itself,
// x_c = Abar^64 x_{c-1} + s_c, runs on the vector ALUs in fp32.  Against a
// 2T-point FFT per chunk this costs 64 multiply-adds per sample for the
// block's own convolution and 2 x 2S for the projections, all of it dense
// matrix-core work, and it reads u and writes y exactly once.
//
// Workspace of 16-bit activations (per channel h):
//   fb  [H, 64]       taps f_0 .. f_63, D folded into f_0                       fp32
//   Eb  [H, 128, 64]  row 2j+p, column k: part p of Abar_j^(63-k) Bbar_j / sB  fp16
//   Rb  [H, 64, 128]  row t, columns 2j, 2j+1: 2 Re, -2 Im of C_j Abar_j^(t+1) / sC   fp16
//   ab  [H, 64]       Abar_j^64                                                 complex
//   sb  [H, 2]        sB, sC: powers of two with |Bbar_j| < sB and 2 |C_j| < sC fp32
// (modes j >= S are zero in every table).

// The tables of one channel per workgroup of eight waves: wave r, lane j
// takes the powers Abar_j^(8 r) .. Abar_j^(8 r + 7), the first from an exact
// fp64 phase reduction and fp32 sine, cosine and exponential, the rest
// stepped by Abar in fp32 (7 steps: relative error ~1e-6, far below the fp16
// tables' 2^-11; Abar^64 itself, which the scan applies once per block, is
// an fp64 exponential), and writes their table entries
// straight to memory: two 16-byte pieces of Eb (one per part) and, per
// power, 4 bytes of a row of Rb (the wave's lanes fill the row).  The
// filter's 64 taps are sums over the modes in fp64, in mode order (so the
// result does not depend on the schedule), of fp32 terms staged in LDS.
__global__ __launch_bounds__(512) void k_spb_params(const float *__restrict__ A, const float *__restrict__ Bm,
                                                   const float *__restrict__ Cc, const float *__restrict__ dt,
                                                   const float *__restrict__ D, float *__restrict__ fb,
                                                   uint16_t *__restrict__ Eb, uint16_t *__restrict__ Rb,
                                                   cf *__restrict__ ab, float *__restrict__ sb, int S) {
    __shared__ __attribute__((aligned(16))) float Ft[64][65];  // Ft[k][j] = 2 Re(C_j Bbar_j Abar_j^k)
    const int h = blockIdx.x, tid = threadIdx.x, j = tid & 63, r = tid >> 6;
    const double dth = (double)dt[h];
    const bool on = j < S;
    double br = 0.0, bi = 0.0, cr = 0.0, ci = 0.0, are = 0.0, aim = 0.0;
    if (on) {
        const size_t o = ((size_t)h * S + j) * 2;
        br = dth * (double)Bm[o];
        bi = dth * (double)Bm[o + 1];
        cr = (double)Cc[o];
        ci = (double)Cc[o + 1];
        are = dth * (double)A[o];
        aim = dth * (double)A[o + 1];
    }
    // scales: the largest |Bbar_j| and 2 |C_j| over the modes (lane = mode)
    const float mb = mf::wave_max((float)sqrt(br * br + bi * bi));
    const float mc = mf::wave_max((float)(2.0 * sqrt(cr * cr + ci * ci)));
    int eb = 0, ec = 0;
    if (mb > 0.f) (void)frexpf(mb, &eb);
    if (mc > 0.f) (void)frexpf(mc, &ec);
    const double rB = ldexp(1.0, -eb), rC2 = ldexp(2.0, -ec);  // 1 / sB, 2 / sC (exact powers of two)
    const float fbr = (float)(br * rB), fbi = (float)(bi * rB);  // Bbar_j / sB
    const float fcr = (float)(cr * rC2), fci = (float)(ci * rC2);  // 2 C_j / sC
    const float fwr = (float)(2.0 * (cr * br - ci * bi)), fwi = (float)(2.0 * (cr * bi + ci * br));  // 2 C_j Bbar_j
    cf p = on ? apow_f32(are, aim, 8.0 * r) : mk(0.f, 0.f);
    const cf st = apow_f32(are, aim, 1.0);
    uint16_t er[8], ei[8];
    uint16_t *const rh = Rb + (size_t)h * 8192;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int pp = 8 * r + k;
        er[7 - k] = __builtin_bit_cast(uint16_t, (_Float16)(p.x * fbr - p.y * fbi));
        ei[7 - k] = __builtin_bit_cast(uint16_t, (_Float16)(p.x * fbi + p.y * fbr));
        Ft[pp][j] = p.x * fwr - p.y * fwi;
        if (pp >= 1) {
            const uint16_t zr = __builtin_bit_cast(uint16_t, (_Float16)(fcr * p.x - fci * p.y));
            const uint16_t zi = __builtin_bit_cast(uint16_t, (_Float16)(-(fcr * p.y + fci * p.x)));
            *(uint32_t *)(rh + (pp - 1) * 128 + 2 * j) = (uint32_t)zr | ((uint32_t)zi << 16);
        }
        p = cmul(p, st);
    }
    // Eb row 2j (+1), columns 56 - 8 r .. 63 - 8 r hold Abar^(8 r + 7) .. Abar^(8 r)
    using u32x4 = mf::u32x4;
    auto pack = [](const uint16_t (&v)[8]) -> u32x4 {
        return u32x4{(uint32_t)v[0] | ((uint32_t)v[1] << 16), (uint32_t)v[2] | ((uint32_t)v[3] << 16),
                     (uint32_t)v[4] | ((uint32_t)v[5] << 16), (uint32_t)v[6] | ((uint32_t)v[7] << 16)};
    };
    uint16_t *const eh = Eb + (size_t)h * 8192;
    *(u32x4 *)(eh + (2 * j) * 64 + 56 - 8 * r) = pack(er);
    *(u32x4 *)(eh + (2 * j + 1) * 64 + 56 - 8 * r) = pack(ei);
    if (r == 0) {
        // Abar^64 (the block step) and its correction row t = 63
        double qr, qi;
        apow64(are, aim, 64.0, qr, qi);
        const cf q = on ? mk((float)qr, (float)qi) : mk(0.f, 0.f);
        ab[(size_t)h * 64 + j] = q;
        const uint16_t zr = __builtin_bit_cast(uint16_t, (_Float16)(fcr * q.x - fci * q.y));
        const uint16_t zi = __builtin_bit_cast(uint16_t, (_Float16)(-(fcr * q.y + fci * q.x)));
        *(uint32_t *)(rh + 63 * 128 + 2 * j) = (uint32_t)zr | ((uint32_t)zi << 16);
        if (j == 0) {
            sb[2 * h] = ldexpf(1.f, eb);
            sb[2 * h + 1] = ldexpf(1.f, ec);
        }
    }
    __syncthreads();
    // taps: wave r sums modes 8 r .. 8 r + 7 of tap k = lane, then tap k sums
    // the eight partial sums (fixed order throughout)
    {
        double part = 0.0;
#pragma unroll
        for (int q = 0; q < 8; ++q) part += (double)Ft[j][8 * r + q];
        __syncthreads();  // (every term has been read)
        ((double *)&Ft[0][0])[r * 64 + j] = part;
        __syncthreads();
        if (tid < 64) {
            double acc = tid == 0 ? (double)D[h] : 0.0;
#pragma unroll
            for (int q = 0; q < 8; ++q) acc += ((const double *)&Ft[0][0])[q * 64 + tid];
            fb[(size_t)h * 64 + tid] = (float)acc;
        }
    }
}

// x * a + s on complex values, as four fused multiply-adds
__device__ __forceinline__ cf cfma(cf a, cf x, cf s) {
    return mk(fmaf(a.x, x.x, fmaf(-a.y, x.y, s.x)), fmaf(a.x, x.y, fmaf(a.y, x.x, s.y)));
}
__device__ __forceinline__ mf::f4 mfma16(mf::half8 a, mf::half8 b, mf::f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// two outputs rounded to the activation type (nearest even), packed
template <int IO>
__device__ __forceinline__ uint32_t spb_pk(float a, float b) {
    if constexpr (IO == IO_BF16) {
        const mf::f2 v = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, mf::bf2));
    } else {
        return mf::pk(a, b);
    }
}
// orders this lane's LDS writes before the reads of the other lanes of its
// wave that follow (LDS requests of one wave complete in order)
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int SPB_SS = 66;   // LDS row of one block: 64 modes (complex) and a pad
constexpr int SPB_XS = 136;  // the same row read as the fp16 states entering the block

// One wave per (batch row b, channel h), two waves per SIMD (232 registers:
// the contribution and correction operands, 32 KiB of the channel's tables,
// stay in registers for the whole row), walking the row in steps of 16
// blocks (1024 samples).  The blocks are the 16 columns of its matrix-core
// products (the B operand, read straight from HBM one step ahead: lane
// (n, g) loads samples 32 ks + 8 g .. + 7 of block n).  Per step:
//   1. contributions S[(j, part)][n] = Eb . U (8 row tiles) -> LDS (one row
//      per block), read back with lane = mode j;
//   2. from the state carried into the step, the state entering each block
//      (x <- Abar^64 x + s, fp32), and the state carried out of the step;
//      the entering states are scaled by a power of two into fp16 range and
//      written back to LDS in the B-operand layout (over the contributions);
//   3. the blocks' own convolutions Y = L . U (the Toeplitz tiles depend only
//      on their distance from the diagonal: 4 distinct tiles, 6 products)
//      and Y += Rb . X (the correction), in fp32;
//   4. y rounded once and stored once.
// A row's steps are sequential; the rows (2048 at B = 2, H = 1024) fill the
// GPU at two waves per SIMD, with no barrier and no exchange between waves.
template <int IO>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void k_sp_block(
    const typename io_elem<IO>::T *__restrict__ u, typename io_elem<IO>::T *__restrict__ y,
    const float *__restrict__ fb, const uint16_t *__restrict__ Eb, const uint16_t *__restrict__ Rb,
    const cf *__restrict__ ab, const float *__restrict__ sb, const float *__restrict__ x_in,
    float *__restrict__ x_out, int H, int64_t N, int S) {
    using namespace mf;
    using T_ = typename io_elem<IO>::T;
    const int h = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x, col = lane & 15, g = lane >> 4;
    __shared__ __attribute__((aligned(16))) cf Sw[16 * SPB_SS];
    uint16_t *const Xw = (uint16_t *)Sw;
    const size_t row = (size_t)b * H + h;
    // contribution operands (A): rows 16 rt + col (mode 8 rt + col / 2, part
    // col % 2), columns 32 ks + 8 g ..
    half8 Ea[8][2];
    {
        const uint16_t *eh = Eb + (size_t)h * 8192;
#pragma unroll
        for (int rt = 0; rt < 8; ++rt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                Ea[rt][ks] = __builtin_bit_cast(half8, *(const u32x4 *)(eh + (16 * rt + col) * 64 + 32 * ks + 8 * g));
    }
    // correction operands (A): rows t = 16 rt + col, columns 32 ks + 8 g ..
    half8 Ra[4][4];
    {
        const uint16_t *rh = Rb + (size_t)h * 8192;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                Ra[rt][ks] = __builtin_bit_cast(half8, *(const u32x4 *)(rh + (16 * rt + col) * 128 + 32 * ks + 8 * g));
    }
    // Toeplitz tiles (A): tile d holds f[16 d + col - 8 g - e] (zero below index 0)
    half8 La[4];
    {
        const float *fh = fb + (size_t)h * 64;
#pragma unroll
        for (int d = 0; d < 4; ++d)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int i = 16 * d + col - 8 * g - e;
                const float v = fh[i < 0 ? 0 : i];
                La[d][e] = (_Float16)(i < 0 ? 0.f : v);
            }
    }
    const cf a = ab[(size_t)h * 64 + lane];
    const float sB = sb[2 * h], sC = sb[2 * h + 1];
    // state carried into the step (lane = mode), in units of sB
    cf X = mk(0.f, 0.f);
    if (x_in && lane < S) {
        const float r = 1.f / sB;
        X = mk(x_in[(row * S + lane) * 2] * r, x_in[(row * S + lane) * 2 + 1] * r);
    }
    const int64_t nch = N / 64;
    const int nst = (int)((nch + 15) / 16);
    const T_ *urow = u + row * N;
    T_ *yrow = y + row * N;
    // the step's window of the row as a buffer resource (empty past the end:
    // its loads return zeros and its stores are dropped)
    auto window = [&](const void *base, int st) -> __amdgpu_buffer_rsrc_t {
        const int64_t s0 = (int64_t)st * 1024, rem = N - s0;
        const int bytes = rem <= 0 ? 0 : (int)(2 * (rem < 1024 ? rem : 1024));
        return row_rsrc((const char *)base + 2 * (rem > 0 ? s0 : 0), bytes);
    };
    const int uoff = col * 128 + 16 * g;
    auto load = [&](int st, u32x4 (&v)[2]) {
        const __amdgpu_buffer_rsrc_t rs = window(urow, st);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            v[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, uoff + 64 * ks, 0, 0));
    };
    u32x4 cur[2], nxt[2];
    load(0, cur);
    asm volatile("" : "+v"(cur[0]), "+v"(cur[1]));  // (complete before the loop: see below)
    const f4 z4 = {0.f, 0.f, 0.f, 0.f};
    // a step's packed outputs, kept live into the next step: a store's data
    // registers may not be reused before the store completes, so reusing
    // them at the top of the next step would wait for every store of this one
    u32x2 opk[4] = {};
    for (int st = 0; st < nst; ++st) {
        load(st + 1, nxt);
        // B operands in fp16: bf16 activations are scaled by a power of two
        // into fp16 range (largest magnitude of the step's 1024 samples
        // below 2^14), then converted exactly but for fp16's subnormals
        half8 U0, U1;
        float isu = 1.f;
        if constexpr (IO == IO_BF16) {
            uint32_t mx = 0;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                mx = pkmax_u16(mx, cur[ks].x & 0x7fff7fffu);
                mx = pkmax_u16(mx, cur[ks].y & 0x7fff7fffu);
                mx = pkmax_u16(mx, cur[ks].z & 0x7fff7fffu);
                mx = pkmax_u16(mx, cur[ks].w & 0x7fff7fffu);
            }
            const uint32_t mh = (mx & 0xffffu) > (mx >> 16) ? (mx & 0xffffu) : (mx >> 16);
            const float mu = wave_max(__uint_as_float(mh << 16));
            int eu = 0;
            if (mu > 0.f) (void)frexpf(mu, &eu);
            eu = eu < -100 ? -100 : eu;
            const float su = ldexpf(1.f, 14 - eu);
            isu = ldexpf(1.f, eu - 14);
            uint32_t o8[2][4];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const uint32_t d4[4] = {cur[ks].x, cur[ks].y, cur[ks].z, cur[ks].w};
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    o8[ks][q] = pk(__uint_as_float(d4[q] << 16) * su, __uint_as_float(d4[q] & 0xffff0000u) * su);
            }
            U0 = __builtin_bit_cast(half8, u32x4{o8[0][0], o8[0][1], o8[0][2], o8[0][3]});
            U1 = __builtin_bit_cast(half8, u32x4{o8[1][0], o8[1][1], o8[1][2], o8[1][3]});
        } else {
            U0 = __builtin_bit_cast(half8, cur[0]);
            U1 = __builtin_bit_cast(half8, cur[1]);
        }
        // 1. contributions: rows 16 rt + 4 g + v of tile rt are (mode 8 rt + 2 g + v / 2, part v % 2)
#pragma unroll
        for (int rt = 0; rt < 8; ++rt) {
            f4 s = mfma16(Ea[rt][0], U0, z4);
            s = mfma16(Ea[rt][1], U1, s);
            *(f4 *)(Sw + col * SPB_SS + 8 * rt + 2 * g) = s;
        }
        wave_lds_sync();
        // 2. lane = mode j: the states entering the blocks, and the largest
        //    of their parts (a step that ends the row early holds the state
        //    after its last block)
        const int64_t rem = nch - (int64_t)st * 16;
        const int nv = rem >= 16 ? 16 : (int)rem;
        cf xin[16];
        float m = 0.f;
        {
            cf x = X;
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                xin[c] = x;
                m = fmaxf(m, fmaxf(fabsf(x.x), fabsf(x.y)));
                const cf sc = cscale(Sw[c * SPB_SS + lane], isu);
                if (nv == 16 || c < nv) x = cfma(a, x, sc);
            }
            X = x;
        }
        asm volatile("" : "+v"(opk[0]), "+v"(opk[1]), "+v"(opk[2]), "+v"(opk[3]));
        m = wave_max(m);
        int ex = 0;
        if (m > 0.f) (void)frexpf(m, &ex);
        ex = ex < -100 ? -100 : ex;
        const float sx = ldexpf(1.f, 14 - ex);  // |x sx| < 2^14
        wave_lds_sync();  // (the contributions have been read)
#pragma unroll
        for (int c = 0; c < 16; ++c) *(uint32_t *)(Xw + c * SPB_XS + 2 * lane) = pk(xin[c].x * sx, xin[c].y * sx);
        wave_lds_sync();
        half8 Xo[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) Xo[ks] = __builtin_bit_cast(half8, *(const u32x4 *)(Xw + col * SPB_XS + 32 * ks + 8 * g));
        const float inv = ldexpf(sB * sC, ex - 14);  // sB sC / sx
        // The next step's activations are taken here, before this step's
        // stores: loads and stores share one counter whose events can
        // complete out of order, so a wait for loads issued before stores
        // would also wait for the stores.
        asm volatile("" : "+v"(nxt[0]), "+v"(nxt[1]));
        const __amdgpu_buffer_rsrc_t yrs = window(yrow, st);
        // 3. the blocks' own convolutions (Toeplitz tiles on and below the diagonal)
        f4 Y[4];
        Y[0] = mfma16(La[0], U0, z4);
        Y[1] = mfma16(La[1], U0, z4);
        Y[2] = mfma16(La[0], U1, mfma16(La[2], U0, z4));
        Y[3] = mfma16(La[1], U1, mfma16(La[3], U0, z4));
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            f4 cc = z4;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) cc = mfma16(Ra[rt][ks], Xo[ks], cc);
            const f4 o = Y[rt] * isu + cc * inv;
            // 4. rows t = 16 rt + 4 g .. + 3 of block col
            opk[rt] = u32x2{spb_pk<IO>(o[0], o[1]), spb_pk<IO>(o[2], o[3])};
            __builtin_amdgcn_raw_buffer_store_b64(opk[rt], yrs, col * 128 + 2 * (16 * rt + 4 * g), 0, 0);
        }
        cur[0] = nxt[0];
        cur[1] = nxt[1];
    }
    if (x_out && lane < S) {
        x_out[(row * S + lane) * 2] = X.x * sB;
        x_out[(row * S + lane) * 2 + 1] = X.y * sB;
    }
}

template <int LOG2M, int IO>
static hipError_t sp_conv(const void *u, const float *fT, void *y, int B, int H, int64_t N, int T,
                          hipStream_t s) {
    using T_ = typename io_elem<IO>::T;
    return launch(k_sp_chunk_conv<LOG2M, IO>, dim3(H), dim3(Plan<LOG2M>::NT), 0, s, (const T_ *)u, fT, (T_ *)y,
                  B, H, N, T);
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

// fp32 activations: chunk filter and power tables, FFT chunk convolutions,
// then the contributions and corrections of every chunk.
static hipError_t sp_run_f32(const void *u, const float *A, const float *Bm, const float *C,
                             const float *dt, const float *D, const float *x_in, float *x_out, void *y,
                             int B, int H, int64_t N, int S, int T, void *ws, hipStream_t s) {
    constexpr int IO = IO_F32;
    using T_ = float;
    const SpLayout L = sp_layout(B, H, N, S, T, true);
    char *w = (char *)ws;
    float *fT = (float *)(w + L.fT);
    cf *E = (cf *)(w + L.E);
    cf *G = (cf *)(w + L.G);
    cf *sc = (cf *)(w + L.sc);
    const int C_ = (int)(N / T), T2 = T / 64;

    hipError_t e = launch(k_ssm_filter, dim3(H), dim3(512), 0, s, A, Bm, C, dt, D, fT, S, (int64_t)T, (int64_t)T);
    if (e != hipSuccess) return e;
    e = launch(k_sp_tables, dim3(H), dim3(256), 0, s, A, dt, E, G, S, T2);
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
    const size_t sm_c = (size_t)T * 4 + 64 * 64 * 8 + 4 * 64 * 8;
    const size_t sm_x = 64 * 64 * 8 + (size_t)64 * T2 * 8;
    // the dynamic LDS limits are set once per device, for the largest
    // chunk length (T = 8192), and their status is checked
    if ((e = sp_f32_attributes<IO>()) != hipSuccess) return e;
    e = launch(k_sp_contrib<IO>, dim3(C_, H, B), dim3(256), sm_c, s, (const T_ *)u, Bm, dt, E, G, sc, B, H, N,
               S, T);
    if (e != hipSuccess) return e;
    return launch(k_sp_correct<IO>, dim3(C_, H, B), dim3(256), sm_x, s, (T_ *)y, C, E, G, sc, x_in, x_out, B,
                  H, N, S, T);
}

// 16-bit activations: the channel tables, then one pass of the block state
// passing over every row (the result does not depend on T).
template <int IO>
static hipError_t sp_run_block(const void *u, const float *A, const float *Bm, const float *C,
                               const float *dt, const float *D, const float *x_in, float *x_out, void *y,
                               int B, int H, int64_t N, int S, int T, void *ws, hipStream_t s) {
    using T_ = typename io_elem<IO>::T;
    const SpLayout L = sp_layout(B, H, N, S, T, false);
    char *w = (char *)ws;
    hipError_t e = launch(k_spb_params, dim3(H), dim3(512), 0, s, A, Bm, C, dt, D, (float *)(w + L.fb),
                          (uint16_t *)(w + L.Eb), (uint16_t *)(w + L.Rb), (cf *)(w + L.ab),
                          (float *)(w + L.sb), S);
    if (e != hipSuccess) return e;
    return launch(k_sp_block<IO>, dim3(H, B), dim3(64), 0, s, (const T_ *)u, (T_ *)y, (const float *)(w + L.fb),
                  (const uint16_t *)(w + L.Eb), (const uint16_t *)(w + L.Rb), (const cf *)(w + L.ab),
                  (const float *)(w + L.sb), x_in, x_out, H, N, S);
}

hipError_t launch_state_pass(const void *u, const float *A, const float *Bm, const float *C,
                             const float *dt, const float *D, const float *x_in, float *x_out,
                             void *y, int B, int H, int64_t N, int S, int T, int io, void *ws,
                             hipStream_t s) {
    switch (io) {
        case IO_F32: return sp_run_f32(u, A, Bm, C, dt, D, x_in, x_out, y, B, H, N, S, T, ws, s);
        case IO_F16: return sp_run_block<IO_F16>(u, A, Bm, C, dt, D, x_in, x_out, y, B, H, N, S, T, ws, s);
        case IO_BF16: return sp_run_block<IO_BF16>(u, A, Bm, C, dt, D, x_in, x_out, y, B, H, N, S, T, ws, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace h3c
