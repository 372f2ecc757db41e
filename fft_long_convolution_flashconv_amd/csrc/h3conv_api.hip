// h3conv_api.hip -- the C ABI: argument validation (host only, before any HIP
// call), device check, dispatch to the kernel launchers.  See include/h3conv.h
// for the contract of every entry point.
#include <atomic>
#include <cstring>
#include <mutex>

#include "../../include/h3conv.h"
#include "h3conv_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_ok[kMaxDevices];  // 0 unknown, 1 usable gfx950, -1 not usable

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t esize(int io) { return io == H3CONV_F32 ? 4 : 2; }

bool valid_io(int io) { return io == H3CONV_F32 || io == H3CONV_F16 || io == H3CONV_BF16; }

// [p, p + n) and [q, q + m) overlap?
bool overlap(const void *p, size_t n, const void *q, size_t m) {
    if (!p || !q || n == 0 || m == 0) return false;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return a < b + m && b < a + n;
}

bool mul_ok(int64_t a, int64_t b, int64_t lim) { return a >= 0 && b >= 0 && (a == 0 || b <= lim / a); }

h3conv_status device_check() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return H3CONV_ERR_NO_DEVICE;
    if (dev >= kMaxDevices) return H3CONV_ERR_NO_DEVICE;
    int st = g_dev_ok[dev].load(std::memory_order_acquire);
    if (st == 0) {
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) return H3CONV_ERR_NO_DEVICE;
        st = (std::strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
        g_dev_ok[dev].store(st, std::memory_order_release);
    }
    return st == 1 ? H3CONV_OK : H3CONV_ERR_NO_DEVICE;
}

h3conv_status from_hip(hipError_t e) { return e == hipSuccess ? H3CONV_OK : H3CONV_ERR_HIP; }

// Scratch memory of h3conv_state_pass_noalloc: one array per device, part of
// the library's device code (allocated when the code is loaded on a device,
// held until the process ends).  Host code never passes `scratch` itself to
// a kernel (on the host it is only a stand-in for the symbol); the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current.
static __device__ __align__(256) unsigned char scratch[H3CONV_NOALLOC_WORKSPACE_BYTES];
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

h3conv_status scratch_ptr(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return H3CONV_ERR_NO_DEVICE;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lk(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_acquire);
        if (!p) {
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !p) return H3CONV_ERR_HIP;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return H3CONV_OK;
}

// Status meaning "arguments valid, sizes non-empty: run it" (never returned
// to a caller; within the enum's value range, above every real status).
constexpr h3conv_status SP_RUN = (h3conv_status)7;

// Host-side validation shared by the state-passing entry points (everything
// but the workspace).  Returns SP_RUN when the call has work to do; a
// zero-length call (N == 0) with x_out is completed here (x_out = x_in or 0).
h3conv_status sp_validate(const void *u, const float *A, const float *Bm, const float *C,
                          const float *dt, const float *D, const float *x_in, float *x_out,
                          void *y, int64_t B, int64_t H, int64_t N, int64_t S, int64_t T, int io,
                          void *stream) {
    if (B < 0 || H < 0 || N < 0 || S < 1 || T < 1 || !valid_io(io)) return H3CONV_ERR_INVALID_ARG;
    if (B == 0 || H == 0) return H3CONV_OK;
    if (N == 0) {
        // no samples: the final state is the initial one (zero without x_in)
        if (!x_out) return H3CONV_OK;
        if (S > H3CONV_MAX_STATE || !mul_ok(B * H, S, INT64_MAX / 16)) return H3CONV_ERR_UNSUPPORTED;
        if (!aligned16(x_out) || (x_in && !aligned16(x_in))) return H3CONV_ERR_INVALID_ARG;
        const size_t nx = (size_t)(B * H * S) * 8;
        if (overlap(x_out, nx, x_in, nx)) return H3CONV_ERR_INVALID_ARG;
        h3conv_status st = device_check();
        if (st != H3CONV_OK) return st;
        return from_hip(h3c::launch_state_copy(x_in, x_out, B * H * S, (hipStream_t)stream));
    }
    if (S > H3CONV_MAX_STATE || T < 64 || T > H3CONV_MAX_FUSED_N || (T & (T - 1)) != 0 || N % T != 0)
        return H3CONV_ERR_UNSUPPORTED;
    if (!u || !A || !Bm || !C || !dt || !D || !y) return H3CONV_ERR_INVALID_ARG;
    const void *ptrs[] = {u, A, Bm, C, dt, D, y, x_in, x_out};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return H3CONV_ERR_INVALID_ARG;
    if (B > 65535 || H > 65535 || N / T > INT32_MAX || !mul_ok(B * H, N, INT64_MAX / 4))
        return H3CONV_ERR_UNSUPPORTED;
    const size_t ny = (size_t)(B * H * N) * esize(io), np = (size_t)(H * S) * 8,
                 nx = (size_t)(B * H * S) * 8, nh = (size_t)H * 4;
    // outputs (y, x_out) must not overlap the inputs or each other
    struct R { const void *p; size_t n; } ins[] = {{u, ny}, {A, np}, {Bm, np}, {C, np},
                                                   {dt, nh}, {D, nh}, {x_in, nx}};
    struct R outs[] = {{y, ny}, {x_out, nx}};
    for (auto &o : outs)
        for (auto &i : ins)
            if (overlap(o.p, o.n, i.p, i.n)) return H3CONV_ERR_INVALID_ARG;
    if (overlap(y, ny, x_out, nx)) return H3CONV_ERR_INVALID_ARG;
    return SP_RUN;
}

}  // namespace

extern "C" {

int h3conv_version(void) { return 100; }

const char *h3conv_status_string(int status) {
    switch (status) {
        case H3CONV_OK: return "ok";
        case H3CONV_ERR_INVALID_ARG: return "invalid argument";
        case H3CONV_ERR_UNSUPPORTED: return "unsupported size or configuration";
        case H3CONV_ERR_NO_DEVICE: return "no usable gfx950 device";
        case H3CONV_ERR_HIP: return "HIP runtime or launch failure";
        case H3CONV_ERR_WORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

size_t h3conv_workspace_size(int op, int64_t B, int64_t H, int64_t N, int64_t S, int64_t T) {
    switch (op) {
        case H3CONV_OP_FFT_CONV: return 0;
        case H3CONV_OP_H3_MIX:
            if (B < 0 || H < 0 || N < 0) return (size_t)-1;
            return h3c::h3_mix_workspace(B, N, H);
        case H3CONV_OP_H3_MIX_MH:
            // H = Dm, S = head dimension; the 16-bit activation path (bf16
            // intermediates); fp32 activations need twice this
            if (B < 0 || H < 0 || N < 0 || S < 1 || H % S != 0) return (size_t)-1;
            return h3c::h3_mix_mh_workspace(B, N, H, S, H3CONV_BF16);
        case H3CONV_OP_STATE_PASS:
            if (B < 0 || H < 0 || N < 0 || S < 1 || S > H3CONV_MAX_STATE || T < 64 ||
                T > H3CONV_MAX_FUSED_N || (T & (T - 1)) != 0 || N % T != 0)
                return (size_t)-1;
            return h3c::state_pass_workspace(B, H, N, S, T);
        default: return (size_t)-1;
    }
}

h3conv_status h3conv_fft_conv(const void *u, const float *f, const float *D, void *y, int64_t B,
                              int64_t H, int64_t N, int io, void *stream) {
    if (B < 0 || H < 0 || N < 0 || !valid_io(io)) return H3CONV_ERR_INVALID_ARG;
    if (B == 0 || H == 0 || N == 0) return H3CONV_OK;
    if (!u || !f || !D || !y) return H3CONV_ERR_INVALID_ARG;
    if (!aligned16(u) || !aligned16(f) || !aligned16(D) || !aligned16(y)) return H3CONV_ERR_INVALID_ARG;
    if (N > (io == H3CONV_F32 ? H3CONV_MAX_FUSED_N : H3CONV_MAX_FUSED_N_16BIT)) return H3CONV_ERR_UNSUPPORTED;
    if (!mul_ok(B, H, INT32_MAX) || !mul_ok(B * H, N, INT64_MAX / 4)) return H3CONV_ERR_UNSUPPORTED;
    if (!h3c::fft_conv_rows_fit(H, N, io)) return H3CONV_ERR_UNSUPPORTED;
    const size_t ny = (size_t)(B * H * N) * esize(io);
    if (overlap(y, ny, u, ny) || overlap(y, ny, f, (size_t)(H * N) * 4) ||
        overlap(y, ny, D, (size_t)H * 4))
        return H3CONV_ERR_INVALID_ARG;
    h3conv_status st = device_check();
    if (st != H3CONV_OK) return st;
    return from_hip(h3c::launch_fft_conv(u, f, D, y, (int)B, (int)H, (int)N, io,
                                         (hipStream_t)stream));
}

h3conv_status h3conv_fft_conv_bidir(const void *u, const float *f, const float *g, const float *D,
                                    void *y, int64_t B, int64_t H, int64_t N, int io, void *stream) {
    if (B < 0 || H < 0 || N < 0 || !valid_io(io)) return H3CONV_ERR_INVALID_ARG;
    if (B == 0 || H == 0 || N == 0) return H3CONV_OK;
    if (!u || !f || !g || !D || !y) return H3CONV_ERR_INVALID_ARG;
    if (!aligned16(u) || !aligned16(f) || !aligned16(g) || !aligned16(D) || !aligned16(y))
        return H3CONV_ERR_INVALID_ARG;
    if (N > (io == H3CONV_F32 ? H3CONV_MAX_FUSED_N : H3CONV_MAX_FUSED_N_16BIT)) return H3CONV_ERR_UNSUPPORTED;
    if (!mul_ok(B, H, INT32_MAX) || !mul_ok(B * H, N, INT64_MAX / 4)) return H3CONV_ERR_UNSUPPORTED;
    if (!h3c::fft_conv_rows_fit(H, N, io)) return H3CONV_ERR_UNSUPPORTED;
    const size_t ny = (size_t)(B * H * N) * esize(io), nf = (size_t)(H * N) * 4;
    if (overlap(y, ny, u, ny) || overlap(y, ny, f, nf) || overlap(y, ny, g, nf) ||
        overlap(y, ny, D, (size_t)H * 4))
        return H3CONV_ERR_INVALID_ARG;
    h3conv_status st = device_check();
    if (st != H3CONV_OK) return st;
    return from_hip(h3c::launch_fft_bidir(u, f, g, D, y, (int)B, (int)H, (int)N, io, (hipStream_t)stream));
}

h3conv_status h3conv_fft_conv_bwd(const void *u, const float *f, const float *D, const void *dy,
                                  void *du, float *df, float *dD, int64_t B, int64_t H, int64_t N,
                                  int io, void *stream) {
    if (B < 0 || H < 0 || N < 0 || !valid_io(io)) return H3CONV_ERR_INVALID_ARG;
    if (H == 0 || N == 0) return H3CONV_OK;
    if (!f || !D || !df || !dD || (B > 0 && (!u || !dy || !du))) return H3CONV_ERR_INVALID_ARG;
    const void *ptrs[] = {u, f, D, dy, du, df, dD};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return H3CONV_ERR_INVALID_ARG;
    if (N > H3CONV_MAX_FUSED_N) return H3CONV_ERR_UNSUPPORTED;
    if (!mul_ok(B, H, INT32_MAX) || !mul_ok(B * H, N, INT64_MAX / 4) || H > INT32_MAX)
        return H3CONV_ERR_UNSUPPORTED;
    if (!h3c::fft_conv_rows_fit(H, N, io)) return H3CONV_ERR_UNSUPPORTED;
    const size_t na = (size_t)(B * H * N) * esize(io), nf = (size_t)(H * N) * 4, nh = (size_t)H * 4;
    struct R { const void *p; size_t n; } ins[] = {{u, na}, {f, nf}, {D, nh}, {dy, na}};
    struct R outs[] = {{du, na}, {df, nf}, {dD, nh}};
    for (auto &o : outs)
        for (auto &i : ins)
            if (overlap(o.p, o.n, i.p, i.n)) return H3CONV_ERR_INVALID_ARG;
    if (overlap(du, na, df, nf) || overlap(du, na, dD, nh) || overlap(df, nf, dD, nh))
        return H3CONV_ERR_INVALID_ARG;
    h3conv_status st = device_check();
    if (st != H3CONV_OK) return st;
    return from_hip(h3c::launch_fft_conv_bwd(u, f, D, dy, du, df, dD, (int)B, (int)H, (int)N, io,
                                             (hipStream_t)stream));
}

h3conv_status h3conv_ssm_filter(const float *A, const float *Bm, const float *C, const float *dt,
                                float *f, int64_t H, int64_t S, int64_t N, void *stream) {
    if (H < 0 || N < 0 || S < 1) return H3CONV_ERR_INVALID_ARG;
    if (H == 0 || N == 0) return H3CONV_OK;
    if (!A || !Bm || !C || !dt || !f) return H3CONV_ERR_INVALID_ARG;
    if (!aligned16(A) || !aligned16(Bm) || !aligned16(C) || !aligned16(dt) || !aligned16(f))
        return H3CONV_ERR_INVALID_ARG;
    if (S > H3CONV_MAX_STATE || H > INT32_MAX || !mul_ok(H, N, INT64_MAX / 4))
        return H3CONV_ERR_UNSUPPORTED;
    const size_t nf = (size_t)(H * N) * 4, np = (size_t)(H * S) * 8;
    if (overlap(f, nf, A, np) || overlap(f, nf, Bm, np) || overlap(f, nf, C, np) ||
        overlap(f, nf, dt, (size_t)H * 4))
        return H3CONV_ERR_INVALID_ARG;
    h3conv_status st = device_check();
    if (st != H3CONV_OK) return st;
    return from_hip(h3c::launch_ssm_filter(A, Bm, C, dt, f, (int)H, (int)S, N, (hipStream_t)stream));
}

h3conv_status h3conv_state_pass(const void *u, const float *A, const float *Bm, const float *C,
                                const float *dt, const float *D, const float *x_in, float *x_out,
                                void *y, int64_t B, int64_t H, int64_t N, int64_t S, int64_t T,
                                int io, void *ws, size_t ws_bytes, void *stream) {
    h3conv_status st = sp_validate(u, A, Bm, C, dt, D, x_in, x_out, y, B, H, N, S, T, io, stream);
    if (st != SP_RUN) return st;
    const size_t need = h3c::state_pass_workspace_io(B, H, N, S, T, io);
    if (!ws || ws_bytes < need) return H3CONV_ERR_WORKSPACE;
    if (!aligned16(ws)) return H3CONV_ERR_INVALID_ARG;
    // the workspace must not overlap any input or output
    const size_t ny = (size_t)(B * H * N) * esize(io), np = (size_t)(H * S) * 8,
                 nx = (size_t)(B * H * S) * 8, nh = (size_t)H * 4;
    struct R { const void *p; size_t n; } bufs[] = {{u, ny}, {A, np}, {Bm, np}, {C, np}, {dt, nh},
                                                    {D, nh}, {x_in, nx}, {y, ny}, {x_out, nx}};
    for (auto &b : bufs)
        if (overlap(ws, need, b.p, b.n)) return H3CONV_ERR_INVALID_ARG;
    st = device_check();
    if (st != H3CONV_OK) return st;
    return from_hip(h3c::launch_state_pass(u, A, Bm, C, dt, D, x_in, x_out, y, (int)B, (int)H, N,
                                           (int)S, (int)T, io, ws, (hipStream_t)stream));
}

h3conv_status h3conv_state_pass_noalloc(const void *u, const float *A, const float *Bm,
                                        const float *C, const float *dt, const float *D,
                                        const float *x_in, float *x_out, void *y, int64_t B,
                                        int64_t H, int64_t N, int64_t S, int64_t T, int io,
                                        void *stream) {
    h3conv_status st = sp_validate(u, A, Bm, C, dt, D, x_in, x_out, y, B, H, N, S, T, io, stream);
    if (st != SP_RUN) return st;
    if (h3c::state_pass_workspace_io(B, H, N, S, T, io) > (size_t)H3CONV_NOALLOC_WORKSPACE_BYTES)
        return H3CONV_ERR_WORKSPACE;
    st = device_check();
    if (st != H3CONV_OK) return st;
    void *ws = nullptr;
    st = scratch_ptr(&ws);
    if (st != H3CONV_OK) return st;
    return from_hip(h3c::launch_state_pass(u, A, Bm, C, dt, D, x_in, x_out, y, (int)B, (int)H, N,
                                           (int)S, (int)T, io, ws, (hipStream_t)stream));
}

h3conv_status h3conv_ssm_step(const void *u, const float *A, const float *Bm, const float *C,
                              const float *dt, const float *D, float *x, void *y, int64_t B, int64_t H,
                              int64_t K, int64_t S, int io, void *stream) {
    if (B < 0 || H < 0 || K < 0 || S < 1 || !valid_io(io)) return H3CONV_ERR_INVALID_ARG;
    if (B == 0 || H == 0 || K == 0) return H3CONV_OK;
    if (S > H3CONV_MAX_STATE) return H3CONV_ERR_UNSUPPORTED;
    if (!u || !A || !Bm || !C || !dt || !D || !x || !y) return H3CONV_ERR_INVALID_ARG;
    const void *ptrs[] = {u, A, Bm, C, dt, D, x, y};
    for (const void *p : ptrs)
        if (!aligned16(p)) return H3CONV_ERR_INVALID_ARG;
    if (H > INT32_MAX || !h3c::ssm_step_fits(B, H) || !mul_ok(B * H, K, INT64_MAX / 4) ||
        !mul_ok(B * H, S, INT64_MAX / 16))
        return H3CONV_ERR_UNSUPPORTED;
    const size_t ny = (size_t)(B * H * K) * esize(io), np = (size_t)(H * S) * 8,
                 nx = (size_t)(B * H * S) * 8, nh = (size_t)H * 4;
    // outputs (y, and x, read and written in place) must not overlap the
    // inputs or each other
    struct R { const void *p; size_t n; } ins[] = {{u, ny}, {A, np}, {Bm, np}, {C, np}, {dt, nh}, {D, nh}};
    for (auto &i : ins)
        if (overlap(y, ny, i.p, i.n) || overlap(x, nx, i.p, i.n)) return H3CONV_ERR_INVALID_ARG;
    if (overlap(y, ny, x, nx)) return H3CONV_ERR_INVALID_ARG;
    h3conv_status st = device_check();
    if (st != H3CONV_OK) return st;
    return from_hip(h3c::launch_ssm_step(u, A, Bm, C, dt, D, x, y, B, H, K, (int)S, io, (hipStream_t)stream));
}

h3conv_status h3conv_h3_mix_mh(const void *q, const void *k, const void *v, const float *w,
                               const float *f, const float *D, void *out, int64_t B, int64_t N,
                               int64_t Dm, int64_t dh, int64_t L, int io, void *ws, size_t ws_bytes,
                               void *stream) {
    if (B < 0 || N < 0 || Dm < 0 || dh < 1 || L < 1 || !valid_io(io)) return H3CONV_ERR_INVALID_ARG;
    if (B == 0 || N == 0 || Dm == 0) return H3CONV_OK;
    if (L > 4 || N > H3CONV_MAX_FUSED_N || dh > 32 || (dh & (dh - 1)) != 0 || Dm % dh != 0)
        return H3CONV_ERR_UNSUPPORTED;
    if (!q || !k || !v || !w || !f || !D || !out || !ws) return !ws ? H3CONV_ERR_WORKSPACE : H3CONV_ERR_INVALID_ARG;
    const void *ptrs[] = {q, k, v, w, f, D, out, ws};
    for (const void *p : ptrs)
        if (!aligned16(p)) return H3CONV_ERR_INVALID_ARG;
    if (B > 65535 || !mul_ok(B, Dm * dh, INT32_MAX) || !mul_ok(B * Dm * dh, N, INT64_MAX / 8) ||
        (N + 31) / 32 > 65535)
        return H3CONV_ERR_UNSUPPORTED;
    // the convolution over the state rows: its row-offset limit with H = Dm dh
    if (!h3c::fft_conv_rows_fit(Dm * dh, N, io == H3CONV_F32 ? H3CONV_F32 : H3CONV_BF16))
        return H3CONV_ERR_UNSUPPORTED;
    const size_t need = h3c::h3_mix_mh_workspace(B, N, Dm, dh, io);
    if (ws_bytes < need) return H3CONV_ERR_WORKSPACE;
    const size_t n = (size_t)(B * N * Dm) * esize(io), nf = (size_t)(Dm * dh * N) * 4;
    struct R { const void *p; size_t n; } ins[] = {{q, n}, {k, n}, {v, n}, {w, (size_t)(Dm * L) * 4}, {f, nf},
                                                   {D, (size_t)(Dm * dh) * 4}};
    for (auto &i : ins)
        if (overlap(out, n, i.p, i.n) || overlap(ws, need, i.p, i.n)) return H3CONV_ERR_INVALID_ARG;
    if (overlap(out, n, ws, need)) return H3CONV_ERR_INVALID_ARG;
    h3conv_status st = device_check();
    if (st != H3CONV_OK) return st;
    return from_hip(h3c::launch_h3_mix_mh(q, k, v, w, f, D, out, (int)B, (int)N, (int)Dm, (int)dh, (int)L, io,
                                          ws, (hipStream_t)stream));
}

h3conv_status h3conv_h3_mix(const void *q, const void *k, const void *v, const float *w,
                            const float *f, const float *D, void *out, int64_t B, int64_t N,
                            int64_t Dm, int64_t L, int io, void *ws, size_t ws_bytes, void *stream) {
    if (B < 0 || N < 0 || Dm < 0 || L < 1 || !valid_io(io)) return H3CONV_ERR_INVALID_ARG;
    if (B == 0 || N == 0 || Dm == 0) return H3CONV_OK;
    if (L > 4 || N > H3CONV_MAX_FUSED_N) return H3CONV_ERR_UNSUPPORTED;
    if (!q || !k || !v || !w || !f || !D || !out) return H3CONV_ERR_INVALID_ARG;
    const void *ptrs[] = {q, k, v, w, f, D, out};
    for (const void *p : ptrs)
        if (!aligned16(p)) return H3CONV_ERR_INVALID_ARG;
    if (!mul_ok(B, Dm, INT32_MAX) || !mul_ok(B * Dm, N, INT64_MAX / 4)) return H3CONV_ERR_UNSUPPORTED;
    // 16-bit path: one gate workgroup row per batch row (grid z <= 65535),
    // and the channel-major convolution rows within 32-bit slice offsets
    if (io != H3CONV_F32 && (B > 65535 || !h3c::fft_conv_rows_fit(Dm, N, H3CONV_BF16)))
        return H3CONV_ERR_UNSUPPORTED;
    const size_t n = (size_t)(B * N * Dm) * esize(io);
    if (overlap(out, n, q, n) || overlap(out, n, k, n) || overlap(out, n, v, n) ||
        overlap(out, n, w, (size_t)(Dm * L) * 4) || overlap(out, n, f, (size_t)(Dm * N) * 4) ||
        overlap(out, n, D, (size_t)Dm * 4))
        return H3CONV_ERR_INVALID_ARG;
    if (io != H3CONV_F32) {
        const size_t need = h3c::h3_mix_workspace(B, N, Dm);
        if (!ws || ws_bytes < need) return H3CONV_ERR_WORKSPACE;
        if (!aligned16(ws)) return H3CONV_ERR_INVALID_ARG;
        const void *ins[] = {q, k, v, out};
        for (const void *p : ins)
            if (overlap(ws, need, p, n)) return H3CONV_ERR_INVALID_ARG;
        if (overlap(ws, need, w, (size_t)(Dm * L) * 4) || overlap(ws, need, f, (size_t)(Dm * N) * 4) ||
            overlap(ws, need, D, (size_t)Dm * 4))
            return H3CONV_ERR_INVALID_ARG;
    }
    h3conv_status st = device_check();
    if (st != H3CONV_OK) return st;
    return from_hip(h3c::launch_h3_mix(q, k, v, w, f, D, out, (int)B, (int)N, (int)Dm, (int)L, io, ws,
                                       (hipStream_t)stream));
}

}  // extern "C"
