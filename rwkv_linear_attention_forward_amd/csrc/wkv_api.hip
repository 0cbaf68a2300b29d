// wkv_api.hip -- the C ABI of librwkv_wkv (declared in include/rwkv_wkv.h).
//
// Host-side only: argument validation (before any HIP call), the gfx950 check, workspace
// layout, kernel dispatch and error reporting. No C++ exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/rwkv_wkv.h"
#include "wkv_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int fail_hip(hipError_t e, const char *what) {
    return fail(WKV_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

constexpr int64_t kMaxC = int64_t(1) << 24;  // keeps per-row byte strides of a chunk in 31 bits
constexpr int64_t kMaxElems = int64_t(1) << 62;

bool dims_ok(int64_t B, int64_t T, int64_t C, const char *fn) {
    if (B < 0 || T < 0 || C < 0) {
        fail(WKV_ERR_INVALID_ARG, "%s: negative dimension (B=%lld, T=%lld, C=%lld)", fn,
             (long long)B, (long long)T, (long long)C);
        return false;
    }
    if (C > kMaxC) {
        fail(WKV_ERR_INVALID_ARG, "%s: C=%lld exceeds the supported maximum %lld", fn,
             (long long)C, (long long)kMaxC);
        return false;
    }
    if (B > 0 && T > 0 && C > 0) {
        if (T > kMaxElems / B || B * T > kMaxElems / C) {
            fail(WKV_ERR_INVALID_ARG, "%s: B*T*C overflows int64", fn);
            return false;
        }
        if (B * ((C + 63) / 64) > INT32_MAX) {
            fail(WKV_ERR_INVALID_ARG, "%s: B*ceil(C/64)=%lld workgroups exceed 2^31-1", fn,
                 (long long)(B * ((C + 63) / 64)));
            return false;
        }
    }
    return true;
}

bool nonnull(const void *p, const char *name, const char *fn) {
    if (p == nullptr) {
        fail(WKV_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);
        return false;
    }
    return true;
}

bool aligned(const void *p, size_t a, const char *name, const char *fn) {
    if (reinterpret_cast<uintptr_t>(p) % a != 0) {
        fail(WKV_ERR_INVALID_ARG, "%s: %s is not %zu-byte aligned", fn, name, a);
        return false;
    }
    return true;
}

// Byte ranges [p, p+n) and [q, q+m) overlap?
bool overlap(const void *p, size_t n, const void *q, size_t m) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
    return n > 0 && m > 0 && a < b + m && b < a + n;
}

// gfx950 check, cached per device id.
std::mutex g_arch_mu;
int g_arch[256];  // 0 unknown, 1 gfx950, 2 other

int check_device(const char *fn) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, fn);
    if (dev < 0 || dev >= 256) return fail(WKV_ERR_UNSUPPORTED, "%s: device id %d", fn, dev);
    {
        std::lock_guard<std::mutex> lk(g_arch_mu);
        if (g_arch[dev] == 0) {
            hipDeviceProp_t prop;
            e = hipGetDeviceProperties(&prop, dev);
            if (e != hipSuccess) return fail_hip(e, fn);
            g_arch[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
            if (g_arch[dev] == 2)
                fail(WKV_ERR_UNSUPPORTED, "%s: device %d is %s, not gfx950", fn, dev,
                     prop.gcnArchName);
        }
        if (g_arch[dev] != 1) {
            if (g_err[0] == '\0') fail(WKV_ERR_UNSUPPORTED, "%s: device %d is not gfx950", fn, dev);
            return WKV_ERR_UNSUPPORTED;
        }
    }
    return WKV_OK;
}

int64_t nsave_of(int64_t T) { return (T + wkvdev::kSaveStride - 1) / wkvdev::kSaveStride; }

size_t saved_bytes_of(int64_t B, int64_t T, int64_t C) {
    return (size_t)B * (size_t)nsave_of(T) * (size_t)C * 16u;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

extern "C" {

int wkv_version(void) { return 100; }  // 0.1.0

const char *wkv_status_string(int status) {
    switch (status) {
    case WKV_OK: return "ok";
    case WKV_ERR_INVALID_ARG: return "invalid argument";
    case WKV_ERR_UNSUPPORTED: return "unsupported device";
    case WKV_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char *wkv_last_error(void) { return g_err; }

size_t wkv_saved_size(int64_t B, int64_t T, int64_t C) {
    if (B < 0 || T < 0 || C < 0 || C > kMaxC) return 0;
    if (B > 0 && T > 0 && C > 0 && (T > kMaxElems / B || B * T > kMaxElems / C)) return 0;
    return saved_bytes_of(B, T, C);
}

int wkv_forward(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                const float *k, const float *v, float *y, void *saved, size_t saved_bytes,
                void *stream) {
    static const char *fn = "wkv_forward";
    g_err[0] = '\0';
    if (!dims_ok(B, T, C, fn)) return WKV_ERR_INVALID_ARG;
    if (B == 0 || T == 0 || C == 0) return WKV_OK;
    if (!nonnull(w, "w", fn) || !nonnull(u, "u", fn) || !nonnull(k, "k", fn) ||
        !nonnull(v, "v", fn) || !nonnull(y, "y", fn))
        return WKV_ERR_INVALID_ARG;
    if (!aligned(w, 4, "w", fn) || !aligned(u, 4, "u", fn) || !aligned(k, 4, "k", fn) ||
        !aligned(v, 4, "v", fn) || !aligned(y, 4, "y", fn))
        return WKV_ERR_INVALID_ARG;
    const size_t nb = (size_t)(B * T * C) * 4u;
    if (overlap(y, nb, k, nb) || overlap(y, nb, v, nb) || overlap(y, nb, w, C * 4u) ||
        overlap(y, nb, u, C * 4u))
        return fail(WKV_ERR_INVALID_ARG, "%s: y overlaps an input", fn);
    float *sva = nullptr, *svb = nullptr;
    double *svP = nullptr;
    if (saved != nullptr) {
        const size_t need = saved_bytes_of(B, T, C);
        if (saved_bytes < need)
            return fail(WKV_ERR_INVALID_ARG, "%s: saved buffer has %zu bytes, needs %zu", fn,
                        saved_bytes, need);
        if (!aligned(saved, 8, "saved", fn)) return WKV_ERR_INVALID_ARG;
        if (overlap(saved, need, y, nb) || overlap(saved, need, k, nb) || overlap(saved, need, v, nb))
            return fail(WKV_ERR_INVALID_ARG, "%s: saved overlaps a tensor", fn);
        const size_t n = (size_t)B * (size_t)nsave_of(T) * (size_t)C;
        sva = static_cast<float *>(saved);
        svb = sva + n;
        svP = reinterpret_cast<double *>(svb + n);
    }
    int rc = check_device(fn);
    if (rc != WKV_OK) return rc;
    hipError_t e = wkvdev::launch_forward(B, T, C, w, u, k, v, y, sva, svb, svP,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip(e, fn);
    return WKV_OK;
}

size_t wkv_backward_workspace_size(int64_t B, int64_t T, int64_t C, int have_saved) {
    if (B < 0 || T < 0 || C < 0 || C > kMaxC) return 0;
    if (B > 0 && T > 0 && C > 0 && (T > kMaxElems / B || B * T > kMaxElems / C)) return 0;
    size_t ws = round_up((size_t)B * (size_t)C * 16u, 256);
    if (!have_saved) ws += round_up(saved_bytes_of(B, T, C), 256);
    return ws;
}

int wkv_backward(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                 const float *k, const float *v, const float *dy, const void *saved,
                 float *dk, float *dv, float *dw, float *du, void *workspace,
                 size_t workspace_bytes, void *stream) {
    static const char *fn = "wkv_backward";
    g_err[0] = '\0';
    (void)w; (void)u; (void)k; (void)v; (void)dy; (void)saved; (void)dk; (void)dv;
    (void)dw; (void)du; (void)workspace; (void)workspace_bytes; (void)stream;
    if (!dims_ok(B, T, C, fn)) return WKV_ERR_INVALID_ARG;
    return fail(WKV_ERR_UNSUPPORTED, "%s: not built in this version", fn);
}

int wkv_decode_step(int64_t B, int64_t C, const float *w, const float *u, const float *k,
                    const float *v, float *a, float *b, float *p, float *y, void *stream) {
    static const char *fn = "wkv_decode_step";
    g_err[0] = '\0';
    if (B < 0 || C < 0) return fail(WKV_ERR_INVALID_ARG, "%s: negative dimension", fn);
    if (C > kMaxC) return fail(WKV_ERR_INVALID_ARG, "%s: C exceeds %lld", fn, (long long)kMaxC);
    if (B > (int64_t(1) << 40) / (C > 0 ? C : 1))
        return fail(WKV_ERR_INVALID_ARG, "%s: B*C exceeds 2^40", fn);
    if (B == 0 || C == 0) return WKV_OK;
    if (!nonnull(w, "w", fn) || !nonnull(u, "u", fn) || !nonnull(k, "k", fn) ||
        !nonnull(v, "v", fn) || !nonnull(a, "a", fn) || !nonnull(b, "b", fn) ||
        !nonnull(p, "p", fn) || !nonnull(y, "y", fn))
        return WKV_ERR_INVALID_ARG;
    const void *ptrs[8] = {w, u, k, v, a, b, p, y};
    const char *names[8] = {"w", "u", "k", "v", "a", "b", "p", "y"};
    for (int i = 0; i < 8; ++i)
        if (!aligned(ptrs[i], 4, names[i], fn)) return WKV_ERR_INVALID_ARG;
    const size_t nb = (size_t)(B * C) * 4u;
    const size_t sizes[8] = {(size_t)C * 4u, (size_t)C * 4u, nb, nb, nb, nb, nb, nb};
    for (int i = 4; i < 8; ++i)      // written: a, b, p, y
        for (int j = 0; j < 8; ++j)  // against everything else
            if (j != i && overlap(ptrs[i], sizes[i], ptrs[j], sizes[j]))
                return fail(WKV_ERR_INVALID_ARG, "%s: %s overlaps %s", fn, names[i], names[j]);
    int rc = check_device(fn);
    if (rc != WKV_OK) return rc;
    hipError_t e = wkvdev::launch_decode(B, C, w, u, k, v, a, b, p, y,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip(e, fn);
    return WKV_OK;
}

}  // extern "C"
