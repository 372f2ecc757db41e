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
#include "h3conv_device.h"
#include "h3conv_internal.h"
#include "mfma_engine.h"

namespace h3c {

// Abar^n = exp(n dt A) in fp64 (dt*Re A and dt*Im A are exact products of
// fp32 values; the library's fp64 sincos reduces large phases accurately).
__device__ __forceinline__ cf abar_pow(double are, double aim, double n) {
    double s, c;
    sincos(aim * n, &s, &c);
    const double m = exp(are * n);
    return mk((float)(m * c), (float)(m * s));
}

// ---------------------------------------------------------------- filter

constexpr int FILT_SEG = 8192;  // outputs per table segment (128 x 64)

// One workgroup per channel.  LDS: WE[j][l] = w_j Abar_j^l (w_j = C_j Bbar_j),
// G[j][i] = Abar_j^(seg + 64 i).  Each thread computes a 2 x 4 tile (two l,
// four i) of outputs per step so a pair of table loads feeds several products.
__global__ __launch_bounds__(256) void k_ssm_filter(const float *__restrict__ A,
                                                   const float *__restrict__ Bm,
                                                   const float *__restrict__ C,
                                                   const float *__restrict__ dt,
                                                   const float *__restrict__ D, float *__restrict__ f,
                                                   int S, int64_t N, int64_t ldf) {
    __shared__ cf WE[64][65];
    __shared__ cf G[64][129];
    const int tid = threadIdx.x;
    const int h = blockIdx.x;
    const double dth = (double)dt[h];

    // WE table
    for (int e = tid; e < S * 64; e += 256) {
        const int j = e >> 6, l = e & 63;
        const float *a = A + ((size_t)h * S + j) * 2;
        const float *b = Bm + ((size_t)h * S + j) * 2;
        const float *c = C + ((size_t)h * S + j) * 2;
        const cf p = abar_pow(dth * (double)a[0], dth * (double)a[1], (double)l);
        const cf w = cmul(mk(c[0], c[1]), mk((float)(dth * b[0]), (float)(dth * b[1])));
        WE[j][l] = cmul(w, p);
    }
    for (int64_t seg = 0; seg < N; seg += FILT_SEG) {
        const int nseg = (int)((N - seg < FILT_SEG) ? (N - seg) : FILT_SEG);
        const int ni = (nseg + 63) / 64;
        __syncthreads();
        for (int e = tid; e < S * ni; e += 256) {
            const int j = e / ni, i = e % ni;
            const float *a = A + ((size_t)h * S + j) * 2;
            G[j][i] = abar_pow(dth * (double)a[0], dth * (double)a[1], (double)(seg + 64 * i));
        }
        __syncthreads();
        // tiles: l in {2 lp, 2 lp + 1}, i in {4 ip .. 4 ip + 3}
        const int ntile = 32 * ((ni + 3) / 4);
        for (int t = tid; t < ntile; t += 256) {
            const int lp = t & 31, ip = t >> 5;
            float acc[2][4] = {};
            for (int j = 0; j < S; ++j) {
                const cf e0 = WE[j][2 * lp], e1 = WE[j][2 * lp + 1];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int i = 4 * ip + q;
                    const cf g = G[j][i < ni ? i : 0];
                    acc[0][q] = fmaf(e0.x, g.x, fmaf(-e0.y, g.y, acc[0][q]));
                    acc[1][q] = fmaf(e1.x, g.x, fmaf(-e1.y, g.y, acc[1][q]));
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int k = 64 * (4 * ip + q) + 2 * lp + r;
                    if (k < nseg) {
                        float v = 2.f * acc[r][q];
                        if (D != nullptr && seg + k == 0) v += D[h];
                        f[(size_t)h * ldf + seg + k] = v;
                    }
                }
            }
        }
    }
}

hipError_t launch_ssm_filter(const float *A, const float *Bm, const float *C, const float *dt,
                             float *f, int H, int S, int64_t N, hipStream_t s) {
    hipLaunchKernelGGL(k_ssm_filter, dim3(H), dim3(256), 0, s, A, Bm, C, dt, (const float *)nullptr,
                       f, S, N, N);
    return hipGetLastError();
}

// ---------------------------------------------------------------- state passing

// Workspace layout (all fp32, 256-byte aligned blocks):
//   fT  [H, T]            chunk filter with D folded into tap 0
//   E   [H, S, 65]        Abar^l, l = 0..64            (complex)
//   G   [H, S, T/64 + 1]  Abar^(64 i), i = 0..T/64     (complex)
//   sc  [B, H, C, S]      per-chunk state contributions (complex)
struct SpLayout {
    size_t fT, E, G, sc, total;
};

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

static SpLayout sp_layout(int64_t B, int64_t H, int64_t N, int64_t S, int64_t T) {
    SpLayout L;
    const int64_t C = N / T, T2 = T / 64;
    size_t o = 0;
    L.fT = o; o += al256((size_t)H * T * 4);
    L.E = o; o += al256((size_t)H * S * 65 * 8);
    L.G = o; o += al256((size_t)H * S * (T2 + 1) * 8);
    L.sc = o; o += al256((size_t)B * H * C * S * 8);
    L.total = o;
    return L;
}

size_t state_pass_workspace(int64_t B, int64_t H, int64_t N, int64_t S, int64_t T) {
    return sp_layout(B, H, N, S, T).total;
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
        sc[(((size_t)b * H + h) * C + c) * S + tid] = s;
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
            for (int cc = 0; cc < c; ++cc) x = cadd(cmul(aT, x), sc[(orow * C + cc) * S + j]);
            if (c == C - 1 && x_out) {
                const cf xo = cadd(cmul(aT, x), sc[(orow * C + c) * S + j]);
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

// Same chunk convolution on the MFMA block-FFT engine (fp16 / bf16 I/O).
template <int LOG2M, int IO>
__global__ __launch_bounds__(mf::Shape<LOG2M>::NT) void k_sp_chunk_conv_mfma(
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
    // complex signal `sig` = row chunks 2 sig (real part), 2 sig + 1 (imaginary)
    auto rowp = [&](int sig) -> mf::RowPtrs {
        const int r = 2 * sig;
        const bool two = r + 1 < rows;
        const uint16_t *ub = (const uint16_t *)u;
        uint16_t *yb = (uint16_t *)y;
        return {ub + off(r), two ? ub + off(r + 1) : nullptr, yb + off(r), two ? yb + off(r + 1) : nullptr};
    };
    E.run_raw([&](int pos) -> float { return fh[pos]; }, T, rowp, (rows + 1) / 2, T, hb);
}

template <int LOG2M, int IO>
static hipError_t sp_conv(const void *u, const float *fT, void *y, int B, int H, int64_t N, int T,
                          hipStream_t s) {
    using T_ = typename io_elem<IO>::T;
    if constexpr (IO != IO_F32 && LOG2M >= 9) {
        hipLaunchKernelGGL((k_sp_chunk_conv_mfma<LOG2M, IO>), dim3(H), dim3(mf::Shape<LOG2M>::NT), 0, s,
                           (const T_ *)u, fT, (T_ *)y, B, H, N, T);
    } else {
        hipLaunchKernelGGL((k_sp_chunk_conv<LOG2M, IO>), dim3(H), dim3(Plan<LOG2M>::NT), 0, s,
                           (const T_ *)u, fT, (T_ *)y, B, H, N, T);
    }
    return hipGetLastError();
}

template <int IO>
static hipError_t sp_run(const void *u, const float *A, const float *Bm, const float *C,
                         const float *dt, const float *D, const float *x_in, float *x_out, void *y,
                         int B, int H, int64_t N, int S, int T, void *ws, hipStream_t s) {
    using T_ = typename io_elem<IO>::T;
    const SpLayout L = sp_layout(B, H, N, S, T);
    char *w = (char *)ws;
    float *fT = (float *)(w + L.fT);
    cf *E = (cf *)(w + L.E);
    cf *G = (cf *)(w + L.G);
    cf *sc = (cf *)(w + L.sc);
    const int C_ = (int)(N / T), T2 = T / 64;

    hipLaunchKernelGGL(k_ssm_filter, dim3(H), dim3(256), 0, s, A, Bm, C, dt, D, fT, S, (int64_t)T,
                       (int64_t)T);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_sp_tables, dim3(H), dim3(256), 0, s, A, dt, E, G, S, T2);
    if ((e = hipGetLastError()) != hipSuccess) return e;
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
    hipFuncSetAttribute((const void *)k_sp_contrib<IO>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)sm_c);
    hipFuncSetAttribute((const void *)k_sp_correct<IO>, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)sm_x);
    hipLaunchKernelGGL((k_sp_contrib<IO>), dim3(C_, H, B), dim3(256), sm_c, s, (const T_ *)u, Bm, dt,
                       E, G, sc, B, H, N, S, T);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((k_sp_correct<IO>), dim3(C_, H, B), dim3(256), sm_x, s, (T_ *)y, C, E, G, sc,
                       x_in, x_out, B, H, N, S, T);
    return hipGetLastError();
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
