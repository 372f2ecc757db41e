// h3conv_api.hip -- the C ABI: argument validation (host only, before any HIP
// call), device check, dispatch to the kernel launchers.  See include/h3conv.h
// for the contract of every entry point.
#include <atomic>
#include <cstring>

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
    if (N > H3CONV_MAX_FUSED_N) return H3CONV_ERR_UNSUPPORTED;
    if (!mul_ok(B, H, INT32_MAX) || !mul_ok(B * H, N, INT64_MAX / 4)) return H3CONV_ERR_UNSUPPORTED;
    const size_t ny = (size_t)(B * H * N) * esize(io);
    if (overlap(y, ny, u, ny) || overlap(y, ny, f, (size_t)(H * N) * 4) ||
        overlap(y, ny, D, (size_t)H * 4))
        return H3CONV_ERR_INVALID_ARG;
    h3conv_status st = device_check();
    if (st != H3CONV_OK) return st;
    return from_hip(h3c::launch_fft_conv(u, f, D, y, (int)B, (int)H, (int)N, io,
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
    if (B < 0 || H < 0 || N < 0 || S < 1 || T < 1 || !valid_io(io)) return H3CONV_ERR_INVALID_ARG;
    if (B == 0 || H == 0) return H3CONV_OK;
    if (S > H3CONV_MAX_STATE || T < 64 || T > H3CONV_MAX_FUSED_N || (T & (T - 1)) != 0 ||
        N == 0 || N % T != 0)
        return N == 0 ? H3CONV_OK : H3CONV_ERR_UNSUPPORTED;
    if (!u || !A || !Bm || !C || !dt || !D || !y) return H3CONV_ERR_INVALID_ARG;
    const void *ptrs[] = {u, A, Bm, C, dt, D, y, x_in, x_out, ws};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return H3CONV_ERR_INVALID_ARG;
    if (B > 65535 || H > 65535 || N / T > INT32_MAX || !mul_ok(B * H, N, INT64_MAX / 4))
        return H3CONV_ERR_UNSUPPORTED;
    const size_t ny = (size_t)(B * H * N) * esize(io), np = (size_t)(H * S) * 8,
                 nx = (size_t)(B * H * S) * 8, nh = (size_t)H * 4;
    const size_t need = h3c::state_pass_workspace(B, H, N, S, T);
    if (!ws || ws_bytes < need) return H3CONV_ERR_WORKSPACE;
    // outputs (y, x_out, ws) must not overlap inputs or each other
    struct R { const void *p; size_t n; } ins[] = {{u, ny}, {A, np}, {Bm, np}, {C, np},
                                                   {dt, nh}, {D, nh}, {x_in, nx}};
    struct R outs[] = {{y, ny}, {x_out, nx}, {ws, need}};
    for (auto &o : outs) {
        for (auto &i : ins)
            if (overlap(o.p, o.n, i.p, i.n)) return H3CONV_ERR_INVALID_ARG;
    }
    if (overlap(y, ny, x_out, nx) || overlap(y, ny, ws, need) || overlap(x_out, nx, ws, need))
        return H3CONV_ERR_INVALID_ARG;
    h3conv_status st = device_check();
    if (st != H3CONV_OK) return st;
    return from_hip(h3c::launch_state_pass(u, A, Bm, C, dt, D, x_in, x_out, y, (int)B, (int)H, N,
                                           (int)S, (int)T, io, ws, (hipStream_t)stream));
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
