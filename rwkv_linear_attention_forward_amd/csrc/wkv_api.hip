// wkv_api.hip -- the C ABI of librwkv_wkv (declared in include/rwkv_wkv.h).
//
// Host-side only: argument validation (before any HIP call), the gfx950 check, workspace
// layout, kernel dispatch and error reporting. No C++ exception crosses the ABI.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <atomic>
#include <chrono>
#include <cstring>
#include <mutex>
#include <random>
#include <unordered_map>

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

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int64_t nseg_of(int64_t T) { return (T + wkvdev::kFwdWindow - 1) / wkvdev::kFwdWindow; }
int64_t bseg_of(int64_t T) { return (T + wkvdev::kBwdWindow - 1) / wkvdev::kBwdWindow; }

// Forward workspace: the stamp, flags, aggregates, inclusive carries, chunk carries, the
// carry entering token 0 and the final state (see wkv_launch.h).
size_t fwd_ws_bytes(int64_t B, int64_t T, int64_t C) {
    const size_t nseg = (size_t)nseg_of(T), ngrp = (size_t)((C + 63) / 64);
    const size_t nbc = (size_t)B * (size_t)C;
    const size_t recs = nbc * nseg * (wkvdev::kRecFields * sizeof(double));
    const size_t cin = recs * (size_t)wkvdev::kCinCarries;
    return wkvdev::kWsHeaderBytes + round_up((size_t)B * ngrp * nseg * 8u, 256) +
           2 * round_up(recs, 256) + round_up(cin, 256) +
           round_up(nbc * (wkvdev::kRecFields * sizeof(double)), 256) +
           round_up(nbc * 3 * sizeof(float), 256);
}

// The compact scan layout of a forward that keeps nothing and takes no state: the stamp,
// the flags, and agg, incl with the three fields (a, b, P) such a forward stores.
constexpr size_t kScanFields = 3;
size_t fwd_scan_bytes(int64_t B, int64_t T, int64_t C) {
    const size_t nseg = (size_t)nseg_of(T), ngrp = (size_t)((C + 63) / 64);
    const size_t recs = (size_t)B * nseg * (size_t)C * (kScanFields * sizeof(double));
    return wkvdev::kWsHeaderBytes + round_up((size_t)B * ngrp * nseg * 8u, 256) +
           2 * round_up(recs, 256);
}

wkvdev::FwdLayout scan_layout(int64_t B, int64_t T, int64_t C, void *ws) {
    wkvdev::FwdLayout L;
    const size_t nseg = (size_t)nseg_of(T), ngrp = (size_t)((C + 63) / 64);
    const size_t recs = (size_t)B * nseg * (size_t)C * (kScanFields * sizeof(double));
    char *p = static_cast<char *>(ws);
    L.nseg = (int64_t)nseg;
    L.hdr = reinterpret_cast<uint64_t *>(p);
    p += wkvdev::kWsHeaderBytes;
    L.flags = reinterpret_cast<uint64_t *>(p);
    p += round_up((size_t)B * ngrp * nseg * 8u, 256);
    L.agg = reinterpret_cast<double *>(p);
    p += round_up(recs, 256);
    L.incl = reinterpret_cast<double *>(p);
    L.cin = nullptr;
    L.init = nullptr;
    L.fin = nullptr;
    return L;
}

wkvdev::FwdLayout fwd_layout(int64_t B, int64_t T, int64_t C, void *ws) {
    wkvdev::FwdLayout L;
    const size_t nseg = (size_t)nseg_of(T), ngrp = (size_t)((C + 63) / 64);
    const size_t recs = (size_t)B * nseg * (size_t)C * (wkvdev::kRecFields * sizeof(double));
    char *p = static_cast<char *>(ws);
    L.nseg = (int64_t)nseg;
    L.hdr = reinterpret_cast<uint64_t *>(p);
    p += wkvdev::kWsHeaderBytes;
    L.flags = reinterpret_cast<uint64_t *>(p);
    p += round_up((size_t)B * ngrp * nseg * 8u, 256);
    L.agg = reinterpret_cast<double *>(p);
    p += round_up(recs, 256);
    L.incl = reinterpret_cast<double *>(p);
    p += round_up(recs, 256);
    L.cin = reinterpret_cast<double *>(p);
    p += round_up(recs * (size_t)wkvdev::kCinCarries, 256);
    L.init = reinterpret_cast<double *>(p);
    p += round_up((size_t)B * (size_t)C * (wkvdev::kRecFields * sizeof(double)), 256);
    L.fin = reinterpret_cast<float *>(p);
    return L;
}

// Backward workspace: flags, reverse aggregates, reverse inclusive carries, per-window dw/du
// partials, then (without a forward workspace) a forward workspace of its own.
size_t bwd_own_bytes(int64_t B, int64_t T, int64_t C) {
    const size_t nseg = (size_t)bseg_of(T), ngrp = (size_t)((C + 63) / 64);
    const size_t n = (size_t)B * nseg * (size_t)C;
    return round_up((size_t)B * ngrp * nseg * 8u, 256) +
           2 * round_up(n * (wkvdev::kRevFields * sizeof(double)), 256) +
           round_up(n * 2 * sizeof(double), 256) +
           round_up((size_t)B * (size_t)C * (wkvdev::kRevFields * sizeof(double)), 256);
}

wkvdev::BwdLayout bwd_layout(int64_t B, int64_t T, int64_t C, void *ws) {
    wkvdev::BwdLayout L;
    const size_t nseg = (size_t)bseg_of(T), ngrp = (size_t)((C + 63) / 64);
    const size_t n = (size_t)B * nseg * (size_t)C;
    char *p = static_cast<char *>(ws);
    L.nseg = (int64_t)nseg;
    L.flags = reinterpret_cast<uint64_t *>(p);
    p += round_up((size_t)B * ngrp * nseg * 8u, 256);
    L.ragg = reinterpret_cast<double *>(p);
    p += round_up(n * (wkvdev::kRevFields * sizeof(double)), 256);
    L.rincl = reinterpret_cast<double *>(p);
    p += round_up(n * (wkvdev::kRevFields * sizeof(double)), 256);
    L.part = reinterpret_cast<double *>(p);
    p += round_up(n * 2 * sizeof(double), 256);
    L.tail = reinterpret_cast<double *>(p);
    return L;
}

// Publication epochs: unique per call, seeded randomly per process so that flags left in a
// reused buffer by another process or an earlier call never match.
std::atomic<uint64_t> g_epoch{0};
std::once_flag g_epoch_once;

uint64_t next_epoch() {
    std::call_once(g_epoch_once, [] {
        std::random_device rd;
        const uint64_t t =
            (uint64_t)std::chrono::high_resolution_clock::now().time_since_epoch().count();
        const uint64_t seed =
            (((uint64_t)rd() << 32) ^ (uint64_t)rd() ^ (t * 0x9E3779B97F4A7C15ull));
        g_epoch.store(seed & ((uint64_t(1) << 60) - 1));
    });
    return (g_epoch.fetch_add(1) + 1) & ((uint64_t(1) << 61) - 1);
}

// What this process last left in each forward workspace it filled (by address): whether the
// states a backward reads were kept, and for which (B, T, C). A backward given a workspace
// that an inference forward filled, or one filled for other sizes, is refused here; the
// device-side stamp (checked when dw, du are summed) catches what this map cannot see.
struct WsRecord {
    int64_t B, T, C;
    bool kept;
};
std::mutex g_ws_mu;
std::unordered_map<uintptr_t, WsRecord> g_ws;

void note_workspace(const void *ws, int64_t B, int64_t T, int64_t C, bool kept) {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    if (g_ws.size() >= 4096) g_ws.clear();  // bounded; a forgotten entry only skips this check
    g_ws[reinterpret_cast<uintptr_t>(ws)] = WsRecord{B, T, C, kept};
}

bool workspace_usable(const void *ws, int64_t B, int64_t T, int64_t C, const char *fn) {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    const auto it = g_ws.find(reinterpret_cast<uintptr_t>(ws));
    if (it == g_ws.end()) return true;
    const WsRecord &r = it->second;
    if (!r.kept) {
        fail(WKV_ERR_INVALID_ARG,
             "%s: fwd_workspace was last filled by wkv_forward_infer, which keeps no states "
             "for a backward", fn);
        return false;
    }
    if (r.B != B || r.T != T || r.C != C) {
        fail(WKV_ERR_INVALID_ARG,
             "%s: fwd_workspace was last filled for B=%lld T=%lld C=%lld, not B=%lld T=%lld "
             "C=%lld", fn, (long long)r.B, (long long)r.T, (long long)r.C, (long long)B,
             (long long)T, (long long)C);
        return false;
    }
    return true;
}

// The storage format of a dtype code (WKV_F32, WKV_BF16, WKV_F16).
bool io_of(int dtype, const char *fn, wkvdev::Io *out) {
    switch (dtype) {
    case WKV_F32: *out = wkvdev::Io::F32; return true;
    case WKV_BF16: *out = wkvdev::Io::BF16; return true;
    case WKV_F16: *out = wkvdev::Io::F16; return true;
    default: fail(WKV_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype); return false;
    }
}

bool grid_ok(int64_t B, int64_t T, int64_t C, const char *fn) {
    const int64_t units = B * ((C + 63) / 64) * nseg_of(T);
    if (units > INT32_MAX) {
        fail(WKV_ERR_INVALID_ARG, "%s: %lld workgroups exceed 2^31-1", fn, (long long)units);
        return false;
    }
    return true;
}

// The backward's grid: B * ceil(C/64) * ceil(T / window) workgroups.
bool bwd_grid_ok(int64_t B, int64_t T, int64_t C, const char *fn) {
    const int64_t units = B * ((C + 63) / 64) * bseg_of(T);
    if (units > INT32_MAX) {
        fail(WKV_ERR_INVALID_ARG, "%s: %lld workgroups exceed 2^31-1", fn, (long long)units);
        return false;
    }
    return grid_ok(B, T, C, fn);
}

}  // namespace

namespace wkvdev {

static std::atomic<int> g_poll_limit{kPollTries};

int poll_limit() { return g_poll_limit.load(std::memory_order_relaxed); }

}  // namespace wkvdev

extern "C" {

int wkv_version(void) { return 100; }  // 0.1.0

int wkv_set_poll_limit(int tries) {
    g_err[0] = '\0';
    if (tries < 0) return fail(WKV_ERR_INVALID_ARG, "wkv_set_poll_limit: negative count %d", tries);
    wkvdev::g_poll_limit.store(tries, std::memory_order_relaxed);
    return WKV_OK;
}

int wkv_poll_limit(void) { return wkvdev::poll_limit(); }

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

size_t wkv_forward_workspace_size(int64_t B, int64_t T, int64_t C) {
    if (B < 0 || T < 0 || C < 0 || C > kMaxC) return 0;
    if (B > 0 && T > 0 && C > 0 && (T > kMaxElems / B || B * T > kMaxElems / C)) return 0;
    return fwd_ws_bytes(B, T, C);
}

}  // extern "C"

namespace {

// wkv_forward, wkv_forward_state and wkv_forward_gated: sa, sb, sp are the state arrays of
// the second (all three non-null) or null, r the gate of the third or null.
// With validate_only the arguments are checked (workspace included) and nothing is launched.
int forward_call(const char *fn, int64_t B, int64_t T, int64_t C, wkvdev::Io fmt,
                 const float *w, const float *u, const void *k, const void *v, const void *r,
                 void *y, float *sa, float *sb, float *sp, void *workspace,
                 size_t workspace_bytes, void *stream, bool keep = true,
                 bool validate_only = false) {
    g_err[0] = '\0';
    if (!dims_ok(B, T, C, fn)) return WKV_ERR_INVALID_ARG;
    if (B == 0 || T == 0 || C == 0) return WKV_OK;
    if (!grid_ok(B, T, C, fn)) return WKV_ERR_INVALID_ARG;
    if (!nonnull(w, "w", fn) || !nonnull(u, "u", fn) || !nonnull(k, "k", fn) ||
        !nonnull(v, "v", fn) || !nonnull(y, "y", fn) || !nonnull(workspace, "workspace", fn))
        return WKV_ERR_INVALID_ARG;
    const size_t es = fmt == wkvdev::Io::F32 ? 4u : 2u;
    if (!aligned(w, 4, "w", fn) || !aligned(u, 4, "u", fn) || !aligned(k, es, "k", fn) ||
        !aligned(v, es, "v", fn) || !aligned(y, es, r ? "out" : "y", fn) ||
        !aligned(workspace, 16, "workspace", fn))
        return WKV_ERR_INVALID_ARG;
    const size_t nb = (size_t)(B * T * C) * es;
    const size_t need = validate_only ? workspace_bytes : fwd_ws_bytes(B, T, C);
    if (workspace_bytes < need)
        return fail(WKV_ERR_INVALID_ARG, "%s: workspace has %zu bytes, needs %zu", fn,
                    workspace_bytes, need);
    if (overlap(y, nb, k, nb) || overlap(y, nb, v, nb) || overlap(y, nb, w, C * 4u) ||
        overlap(y, nb, u, C * 4u) || (r != nullptr && overlap(y, nb, r, nb)))
        return fail(WKV_ERR_INVALID_ARG, "%s: %s overlaps an input", fn, r ? "out" : "y");
    if (r != nullptr) {
        if (!aligned(r, es, "r", fn)) return WKV_ERR_INVALID_ARG;
        if (overlap(workspace, need, r, nb))
            return fail(WKV_ERR_INVALID_ARG, "%s: workspace overlaps r", fn);
    }
    if (overlap(workspace, need, y, nb) || overlap(workspace, need, k, nb) ||
        overlap(workspace, need, v, nb) || overlap(workspace, need, w, C * 4u) ||
        overlap(workspace, need, u, C * 4u))
        return fail(WKV_ERR_INVALID_ARG, "%s: workspace overlaps a tensor", fn);
    if (sa != nullptr) {
        const size_t ns = (size_t)(B * C) * 4u;
        float *st[3] = {sa, sb, sp};
        const char *sn[3] = {"a", "b", "p"};
        for (int i = 0; i < 3; ++i) {
            if (!aligned(st[i], 4, sn[i], fn)) return WKV_ERR_INVALID_ARG;
            if (overlap(st[i], ns, k, nb) || overlap(st[i], ns, v, nb) ||
                overlap(st[i], ns, y, nb) || overlap(st[i], ns, w, C * 4u) ||
                overlap(st[i], ns, u, C * 4u) || overlap(st[i], ns, workspace, need))
                return fail(WKV_ERR_INVALID_ARG, "%s: state %s overlaps another tensor", fn,
                            sn[i]);
            for (int j = 0; j < i; ++j)
                if (overlap(st[i], ns, st[j], ns))
                    return fail(WKV_ERR_INVALID_ARG, "%s: state %s overlaps state %s", fn,
                                sn[i], sn[j]);
        }
    }
    if (validate_only) return WKV_OK;
    int rc = check_device(fn);
    if (rc != WKV_OK) return rc;
    hipError_t e = wkvdev::launch_forward(B, T, C, fmt, w, u, k, v, r, y, sa, sb, sp,
                                          fwd_layout(B, T, C, workspace), next_epoch(), keep,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip(e, fn);
    note_workspace(workspace, B, T, C, keep);
    return WKV_OK;
}

}  // namespace

extern "C" {

int wkv_forward_train(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                      const float *k, const float *v, float *y, void *workspace,
                      size_t workspace_bytes, void *stream) {
    return forward_call("wkv_forward_train", B, T, C, wkvdev::Io::F32, w, u, k, v, nullptr, y,
                        nullptr, nullptr, nullptr, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Scratch of wkv_forward_noalloc: one copy per GPU, held from the library's load to the end
// of the process. Host code never uses this name as an address (on the host it is only a
// stand-in); it uses the device address that hipGetSymbolAddress returns for the current
// device, looked up once per device.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[256];  // per device id; null until looked up

int scratch_address(const char *fn, void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail_hip(e, fn);
    if (dev < 0 || dev >= 256) return fail(WKV_ERR_UNSUPPORTED, "%s: device id %d", fn, dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return fail_hip(e, "wkv_forward_noalloc: scratch address");
        if (p == nullptr)
            return fail(WKV_ERR_HIP, "%s: scratch address of device %d is null", fn, dev);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return WKV_OK;
}

}  // namespace

extern "C" {

size_t wkv_forward_noalloc_max_scratch(void) { return kNoAllocScratchBytes; }

size_t wkv_forward_noalloc_scratch_bytes(int64_t B, int64_t T, int64_t C) {
    if (B < 0 || T < 0 || C < 0 || C > kMaxC) return 0;
    if (B > 0 && T > 0 && C > 0 && (T > kMaxElems / B || B * T > kMaxElems / C)) return 0;
    return fwd_scan_bytes(B, T, C);
}

int wkv_forward_noalloc(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                        const float *k, const float *v, float *y, void *stream) {
    static const char *fn = "wkv_forward_noalloc";
    g_err[0] = '\0';
    if (!dims_ok(B, T, C, fn)) return WKV_ERR_INVALID_ARG;
    if (B == 0 || T == 0 || C == 0) return WKV_OK;
    const size_t need = fwd_scan_bytes(B, T, C);
    if (need > kNoAllocScratchBytes)
        return fail(WKV_ERR_INVALID_ARG,
                    "%s: B=%lld T=%lld C=%lld needs %zu bytes of scratch, more than the %zu the "
                    "library holds per GPU (use wkv_forward or wkv_forward_infer)", fn,
                    (long long)B, (long long)T, (long long)C, need, kNoAllocScratchBytes);
    void *const probe = reinterpret_cast<void *>(uintptr_t(1) << 62);
    int rc = forward_call(fn, B, T, C, wkvdev::Io::F32, w, u, k, v, nullptr, y, nullptr,
                          nullptr, nullptr, probe, need, nullptr, false, true);
    if (rc != WKV_OK) return rc;
    rc = check_device(fn);
    if (rc != WKV_OK) return rc;
    void *ws = nullptr;
    rc = scratch_address(fn, &ws);
    if (rc != WKV_OK) return rc;
    // the flags carry a per-call epoch, so what an earlier call left in the array is never
    // taken for this call's: nothing needs clearing
    hipError_t e = wkvdev::launch_forward(B, T, C, wkvdev::Io::F32, w, u, k, v, nullptr, y,
                                          nullptr, nullptr, nullptr, scan_layout(B, T, C, ws),
                                          next_epoch(), false, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip(e, fn);
    return WKV_OK;
}

int wkv_forward(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                const float *k, const float *v, float *y, void *stream) {
    static const char *fn = "wkv_forward";
    g_err[0] = '\0';
    if (!dims_ok(B, T, C, fn)) return WKV_ERR_INVALID_ARG;
    if (B == 0 || T == 0 || C == 0) return WKV_OK;
    // the look-back's records live in memory taken from the device's stream-ordered pool for
    // the duration of the call (allocated and released on `stream`); validation happens
    // before that, on a placeholder address that overlaps nothing
    void *const probe = reinterpret_cast<void *>(uintptr_t(1) << 62);
    const size_t need = fwd_scan_bytes(B, T, C);
    int rc = forward_call(fn, B, T, C, wkvdev::Io::F32, w, u, k, v, nullptr, y, nullptr,
                          nullptr, nullptr, probe, need, nullptr, false, true);
    if (rc != WKV_OK) return rc;
    rc = check_device(fn);
    if (rc != WKV_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    void *ws = nullptr;
    hipError_t e = hipMallocAsync(&ws, need, st);
    if (e != hipSuccess) return fail_hip(e, "wkv_forward: scratch from the stream-ordered pool");
    e = wkvdev::launch_forward(B, T, C, wkvdev::Io::F32, w, u, k, v, nullptr, y, nullptr,
                               nullptr, nullptr, scan_layout(B, T, C, ws), next_epoch(), false,
                               st);
    const hipError_t e2 = hipFreeAsync(ws, st);
    if (e != hipSuccess) return fail_hip(e, fn);
    if (e2 != hipSuccess) return fail_hip(e2, "wkv_forward: releasing its scratch");
    return WKV_OK;
}

int wkv_forward_state(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                      const float *k, const float *v, float *y, float *a, float *b, float *p,
                      void *workspace, size_t workspace_bytes, void *stream) {
    static const char *fn = "wkv_forward_state";
    if (B > 0 && T > 0 && C > 0) {
        g_err[0] = '\0';
        if (!nonnull(a, "a", fn) || !nonnull(b, "b", fn) || !nonnull(p, "p", fn))
            return WKV_ERR_INVALID_ARG;
    }
    return forward_call(fn, B, T, C, wkvdev::Io::F32, w, u, k, v, nullptr, y, a, b, p,
                        workspace, workspace_bytes, stream);
}

int wkv_forward_infer(int dtype, int64_t B, int64_t T, int64_t C, const float *w,
                      const float *u, const void *k, const void *v, const void *r, void *y,
                      float *a, float *b, float *p, void *workspace, size_t workspace_bytes,
                      void *stream) {
    static const char *fn = "wkv_forward_infer";
    g_err[0] = '\0';
    wkvdev::Io fmt;
    if (!io_of(dtype, fn, &fmt)) return WKV_ERR_INVALID_ARG;
    const int given = (a != nullptr) + (b != nullptr) + (p != nullptr);
    if (given != 0 && given != 3)
        return fail(WKV_ERR_INVALID_ARG, "%s: give all of a, b, p or none", fn);
    return forward_call(fn, B, T, C, fmt, w, u, k, v, r, y, a, b, p, workspace,
                        workspace_bytes, stream, false);
}

int wkv_forward_state_typed(int dtype, int64_t B, int64_t T, int64_t C, const float *w,
                            const float *u, const void *k, const void *v, const void *r,
                            void *y, float *a, float *b, float *p, void *workspace,
                            size_t workspace_bytes, void *stream) {
    static const char *fn = "wkv_forward_state_typed";
    g_err[0] = '\0';
    wkvdev::Io fmt;
    if (!io_of(dtype, fn, &fmt)) return WKV_ERR_INVALID_ARG;
    const int given = (a != nullptr) + (b != nullptr) + (p != nullptr);
    if (given != 0 && given != 3)
        return fail(WKV_ERR_INVALID_ARG, "%s: give all of a, b, p or none", fn);
    return forward_call(fn, B, T, C, fmt, w, u, k, v, r, y, a, b, p, workspace,
                        workspace_bytes, stream, true);
}

int wkv_forward_gated(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                      const float *k, const float *v, const float *r, float *out,
                      void *workspace, size_t workspace_bytes, void *stream) {
    static const char *fn = "wkv_forward_gated";
    if (B > 0 && T > 0 && C > 0) {
        g_err[0] = '\0';
        if (!nonnull(r, "r", fn)) return WKV_ERR_INVALID_ARG;
    }
    return forward_call(fn, B, T, C, wkvdev::Io::F32, w, u, k, v, r, out, nullptr, nullptr,
                        nullptr, workspace, workspace_bytes, stream);
}

int wkv_forward_typed(int dtype, int64_t B, int64_t T, int64_t C, const float *w,
                      const float *u, const void *k, const void *v, const void *r, void *y,
                      void *workspace, size_t workspace_bytes, void *stream) {
    static const char *fn = "wkv_forward_typed";
    wkvdev::Io fmt;
    if (!io_of(dtype, fn, &fmt)) return WKV_ERR_INVALID_ARG;
    return forward_call(fn, B, T, C, fmt, w, u, k, v, r, y, nullptr, nullptr, nullptr,
                        workspace, workspace_bytes, stream);
}

size_t wkv_backward_workspace_size_ex(int64_t B, int64_t T, int64_t C,
                                      int have_fwd_workspace) {
    if (B < 0 || T < 0 || C < 0 || C > kMaxC) return 0;
    if (B > 0 && T > 0 && C > 0 && (T > kMaxElems / B || B * T > kMaxElems / C)) return 0;
    size_t ws = bwd_own_bytes(B, T, C);
    if (!have_fwd_workspace) ws += fwd_ws_bytes(B, T, C);
    return ws;
}

size_t wkv_backward_workspace_size(int64_t B, int64_t T, int64_t C) {
    return wkv_backward_workspace_size_ex(B, T, C, 0);
}

size_t wkv_backward_train_workspace_size(int64_t B, int64_t T, int64_t C) {
    return wkv_backward_workspace_size_ex(B, T, C, 1);
}

}  // extern "C"

namespace {

// wkv_backward and wkv_backward_gated: r and dr are the gate and its gradient of the latter
// (both non-null) or null for the former.
int backward_call(const char *fn, int64_t B, int64_t T, int64_t C, wkvdev::Io fmt,
                  const float *w, const float *u, const void *k, const void *v, const void *dy,
                  const void *r, const void *fwd_workspace, void *dk, void *dv, void *dr,
                  float *dw, float *du, void *workspace, size_t workspace_bytes, void *stream,
                  float *ga = nullptr, float *gb = nullptr, float *gp = nullptr,
                  const float *dfa = nullptr, const float *dfb = nullptr) {
    g_err[0] = '\0';
    if (!dims_ok(B, T, C, fn)) return WKV_ERR_INVALID_ARG;
    if (C == 0) return WKV_OK;
    if (!nonnull(dw, "dw", fn) || !nonnull(du, "du", fn)) return WKV_ERR_INVALID_ARG;
    if (!aligned(dw, 4, "dw", fn) || !aligned(du, 4, "du", fn)) return WKV_ERR_INVALID_ARG;
    if (overlap(dw, C * 4u, du, C * 4u)) return fail(WKV_ERR_INVALID_ARG, "%s: dw overlaps du", fn);
    if (B == 0 || T == 0) {
        int rc = check_device(fn);
        if (rc != WKV_OK) return rc;
        hipError_t e = wkvdev::launch_zero2(dw, du, C, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fail_hip(e, fn);
        return WKV_OK;
    }
    if (!bwd_grid_ok(B, T, C, fn)) return WKV_ERR_INVALID_ARG;
    const bool gated = r != nullptr || dr != nullptr;
    const char *gname = gated ? "dout" : "dy";
    const void *ptrs[10] = {w, u, k, v, dy, dk, dv, workspace, r, dr};
    const char *names[10] = {"w", "u", "k", "v", gname, "dk", "dv", "workspace", "r", "dr"};
    for (int i = 0; i < (gated ? 10 : 8); ++i)
        if (!nonnull(ptrs[i], names[i], fn)) return WKV_ERR_INVALID_ARG;
    const size_t es = fmt == wkvdev::Io::F32 ? 4u : 2u;
    for (int i = 0; i < (gated ? 10 : 8); ++i)
        if (i != 7 && !aligned(ptrs[i], i < 2 ? 4u : es, names[i], fn))
            return WKV_ERR_INVALID_ARG;
    if (!aligned(workspace, 16, "workspace", fn)) return WKV_ERR_INVALID_ARG;
    if (fwd_workspace != nullptr && !aligned(fwd_workspace, 16, "fwd_workspace", fn))
        return WKV_ERR_INVALID_ARG;
    const size_t need = wkv_backward_workspace_size_ex(B, T, C, fwd_workspace != nullptr);
    if (workspace_bytes < need)
        return fail(WKV_ERR_INVALID_ARG, "%s: workspace has %zu bytes, needs %zu", fn,
                    workspace_bytes, need);
    const size_t nb = (size_t)(B * T * C) * es, nc = (size_t)C * 4u;
    const size_t ns = ga ? (size_t)(B * C) * 4u : 0;
    if (ga != nullptr && (!aligned(ga, 4, "da", fn) || !aligned(gb, 4, "db", fn) ||
                          !aligned(gp, 4, "dp", fn)))
        return WKV_ERR_INVALID_ARG;
    const void *outs[9] = {dk, dv, dw, du, workspace, dr, ga, gb, gp};
    const size_t osz[9] = {nb, nb, nc, nc, need, dr ? nb : 0, ns, ns, ns};
    if (dfa != nullptr && (!aligned(dfa, 4, "dfa", fn) || !aligned(dfb, 4, "dfb", fn)))
        return WKV_ERR_INVALID_ARG;
    const size_t nf = dfa ? (size_t)(B * C) * 4u : 0;
    const void *ins[9] = {w, u, k, v, dy, fwd_workspace, r, dfa, dfb};
    const size_t isz[9] = {nc, nc, nb, nb, nb, fwd_workspace ? fwd_ws_bytes(B, T, C) : 0,
                           r ? nb : 0, nf, nf};
    for (int i = 0; i < 9; ++i) {
        for (int j = 0; j < 9; ++j)
            if (overlap(outs[i], osz[i], ins[j], isz[j]))
                return fail(WKV_ERR_INVALID_ARG, "%s: an output overlaps an input", fn);
        for (int j = i + 1; j < 9; ++j)
            if (overlap(outs[i], osz[i], outs[j], osz[j]))
                return fail(WKV_ERR_INVALID_ARG, "%s: two outputs overlap", fn);
    }
    if (fwd_workspace != nullptr && !workspace_usable(fwd_workspace, B, T, C, fn))
        return WKV_ERR_INVALID_ARG;
    int rc = check_device(fn);
    if (rc != WKV_OK) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    wkvdev::FwdLayout F;
    char *own = static_cast<char *>(workspace);
    if (fwd_workspace != nullptr) {
        F = fwd_layout(B, T, C, const_cast<void *>(fwd_workspace));
    } else {
        F = fwd_layout(B, T, C, own + bwd_own_bytes(B, T, C));
        hipError_t e = wkvdev::launch_forward(B, T, C, fmt, w, u, k, v, nullptr, nullptr,
                                              nullptr, nullptr, nullptr, F, next_epoch(), true,
                                              st);
        if (e != hipSuccess) return fail_hip(e, fn);
    }
    hipError_t e = wkvdev::launch_backward(B, T, C, fmt, w, u, k, v, dy, r, F, dk, dv, dr, dw,
                                           du, ga, gb, gp, dfa, dfb,
                                           bwd_layout(B, T, C, own), next_epoch(), st);
    if (e != hipSuccess) return fail_hip(e, fn);
    return WKV_OK;
}

}  // namespace

extern "C" {

int wkv_backward(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                 const float *k, const float *v, const float *dy, float *dk, float *dv,
                 float *dw, float *du, void *workspace, size_t workspace_bytes, void *stream) {
    return backward_call("wkv_backward", B, T, C, wkvdev::Io::F32, w, u, k, v, dy, nullptr,
                         nullptr, dk, dv, nullptr, dw, du, workspace, workspace_bytes, stream);
}

int wkv_backward_train(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                       const float *k, const float *v, const float *dy,
                       const void *fwd_workspace, float *dk, float *dv, float *dw, float *du,
                       void *workspace, size_t workspace_bytes, void *stream) {
    static const char *fn = "wkv_backward_train";
    if (B > 0 && T > 0 && C > 0) {
        g_err[0] = '\0';
        if (!nonnull(fwd_workspace, "fwd_workspace", fn)) return WKV_ERR_INVALID_ARG;
    }
    return backward_call(fn, B, T, C, wkvdev::Io::F32, w, u, k, v, dy, nullptr, fwd_workspace,
                         dk, dv, nullptr, dw, du, workspace, workspace_bytes, stream);
}

namespace {

int backward_state_call(const char *fn, wkvdev::Io fmt, int64_t B, int64_t T, int64_t C,
                        const float *w, const float *u, const void *k, const void *v,
                        const void *dy, const void *r, const float *dfa, const float *dfb,
                        const void *fwd_workspace, void *dk, void *dv, void *dr, float *dw,
                        float *du, float *da, float *db, float *dp, void *workspace,
                        size_t workspace_bytes, void *stream) {
    g_err[0] = '\0';
    if (!dims_ok(B, T, C, fn)) return WKV_ERR_INVALID_ARG;
    if (B > 0 && C > 0) {
        if (!nonnull(fwd_workspace, "fwd_workspace", fn) || !nonnull(da, "da", fn) ||
            !nonnull(db, "db", fn) || !nonnull(dp, "dp", fn))
            return WKV_ERR_INVALID_ARG;
        if ((dfa == nullptr) != (dfb == nullptr))
            return fail(WKV_ERR_INVALID_ARG, "%s: give both of dfa, dfb or neither", fn);
        if (T == 0 && dfa != nullptr)
            return fail(WKV_ERR_INVALID_ARG,
                        "%s: T = 0 records no state; the final state's cotangent is the "
                        "initial state's", fn);
        if (!aligned(da, 4, "da", fn) || !aligned(db, 4, "db", fn) || !aligned(dp, 4, "dp", fn))
            return WKV_ERR_INVALID_ARG;
        const size_t ns = (size_t)(B * C) * 4u;
        if (overlap(da, ns, db, ns) || overlap(da, ns, dp, ns) || overlap(db, ns, dp, ns))
            return fail(WKV_ERR_INVALID_ARG, "%s: two outputs overlap", fn);
        if (T == 0) {
            // no token: the state passes through unchanged, and L does not depend on it
            int rc = check_device(fn);
            if (rc != WKV_OK) return rc;
            hipStream_t st = static_cast<hipStream_t>(stream);
            hipError_t e = wkvdev::launch_zero2(da, db, B * C, st);
            if (e == hipSuccess) e = wkvdev::launch_zero2(dp, da, B * C, st);  // da again
            if (e != hipSuccess) return fail_hip(e, fn);
        }
    }
    return backward_call(fn, B, T, C, fmt, w, u, k, v, dy, r, fwd_workspace, dk, dv, dr, dw, du,
                         workspace, workspace_bytes, stream, da, db, dp, dfa, dfb);
}

}  // namespace

int wkv_backward_state(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                       const float *k, const float *v, const float *dy, const float *dfa,
                       const float *dfb, const void *fwd_workspace, float *dk, float *dv,
                       float *dw, float *du, float *da, float *db, float *dp,
                       void *workspace, size_t workspace_bytes, void *stream) {
    return backward_state_call("wkv_backward_state", wkvdev::Io::F32, B, T, C, w, u, k, v, dy,
                               nullptr, dfa, dfb, fwd_workspace, dk, dv, nullptr, dw, du, da, db,
                               dp, workspace, workspace_bytes, stream);
}

int wkv_backward_state_typed(int dtype, int64_t B, int64_t T, int64_t C, const float *w,
                             const float *u, const void *k, const void *v, const void *dy,
                             const void *r, const float *dfa, const float *dfb,
                             const void *fwd_workspace, void *dk, void *dv, void *dr,
                             float *dw, float *du, float *da, float *db, float *dp,
                             void *workspace, size_t workspace_bytes, void *stream) {
    static const char *fn = "wkv_backward_state_typed";
    g_err[0] = '\0';
    wkvdev::Io fmt;
    if (!io_of(dtype, fn, &fmt)) return WKV_ERR_INVALID_ARG;
    if ((r == nullptr) != (dr == nullptr) && B > 0 && T > 0 && C > 0)
        return fail(WKV_ERR_INVALID_ARG, "%s: r and dr must be given together", fn);
    return backward_state_call(fn, fmt, B, T, C, w, u, k, v, dy, r, dfa, dfb, fwd_workspace, dk,
                               dv, dr, dw, du, da, db, dp, workspace, workspace_bytes, stream);
}

int wkv_backward_gated(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                       const float *k, const float *v, const float *r, const float *dout,
                       const void *fwd_workspace, float *dk, float *dv, float *dr, float *dw,
                       float *du, void *workspace, size_t workspace_bytes, void *stream) {
    static const char *fn = "wkv_backward_gated";
    if (B > 0 && T > 0 && C > 0) {
        g_err[0] = '\0';
        if (!nonnull(r, "r", fn) || !nonnull(dr, "dr", fn)) return WKV_ERR_INVALID_ARG;
    }
    return backward_call(fn, B, T, C, wkvdev::Io::F32, w, u, k, v, dout, r, fwd_workspace, dk,
                         dv, dr, dw, du, workspace, workspace_bytes, stream);
}

int wkv_backward_typed(int dtype, int64_t B, int64_t T, int64_t C, const float *w,
                       const float *u, const void *k, const void *v, const void *dy,
                       const void *r, const void *fwd_workspace, void *dk, void *dv, void *dr,
                       float *dw, float *du, void *workspace, size_t workspace_bytes,
                       void *stream) {
    static const char *fn = "wkv_backward_typed";
    wkvdev::Io fmt;
    if (!io_of(dtype, fn, &fmt)) return WKV_ERR_INVALID_ARG;
    if ((r == nullptr) != (dr == nullptr) && B > 0 && T > 0 && C > 0)
        return fail(WKV_ERR_INVALID_ARG, "%s: r and dr must be given together", fn);
    return backward_call(fn, B, T, C, fmt, w, u, k, v, dy, r, fwd_workspace, dk, dv, dr, dw, du,
                         workspace, workspace_bytes, stream);
}

namespace {

int decode_call(const char *fn, wkvdev::Io fmt, int64_t B, int64_t C, const float *w,
                const float *u, const void *k, const void *v, float *a, float *b, float *p,
                void *y, void *stream) {
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
    const size_t es = fmt == wkvdev::Io::F32 ? 4u : 2u;
    const void *ptrs[8] = {w, u, k, v, a, b, p, y};
    const char *names[8] = {"w", "u", "k", "v", "a", "b", "p", "y"};
    const size_t align[8] = {4, 4, es, es, 4, 4, 4, es};
    for (int i = 0; i < 8; ++i)
        if (!aligned(ptrs[i], align[i], names[i], fn)) return WKV_ERR_INVALID_ARG;
    const size_t nb = (size_t)(B * C) * 4u, ne = (size_t)(B * C) * es;
    const size_t sizes[8] = {(size_t)C * 4u, (size_t)C * 4u, ne, ne, nb, nb, nb, ne};
    for (int i = 4; i < 8; ++i)      // written: a, b, p, y
        for (int j = 0; j < 8; ++j)  // against everything else
            if (j != i && overlap(ptrs[i], sizes[i], ptrs[j], sizes[j]))
                return fail(WKV_ERR_INVALID_ARG, "%s: %s overlaps %s", fn, names[i], names[j]);
    int rc = check_device(fn);
    if (rc != WKV_OK) return rc;
    hipError_t e = wkvdev::launch_decode(B, C, fmt, w, u, k, v, a, b, p, y,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip(e, fn);
    return WKV_OK;
}

}  // namespace

int wkv_decode_step(int64_t B, int64_t C, const float *w, const float *u, const float *k,
                    const float *v, float *a, float *b, float *p, float *y, void *stream) {
    return decode_call("wkv_decode_step", wkvdev::Io::F32, B, C, w, u, k, v, a, b, p, y,
                       stream);
}

int wkv_decode_step_typed(int dtype, int64_t B, int64_t C, const float *w, const float *u,
                          const void *k, const void *v, float *a, float *b, float *p, void *y,
                          void *stream) {
    static const char *fn = "wkv_decode_step_typed";
    g_err[0] = '\0';
    wkvdev::Io fmt;
    if (!io_of(dtype, fn, &fmt)) return WKV_ERR_INVALID_ARG;
    return decode_call(fn, fmt, B, C, w, u, k, v, a, b, p, y, stream);
}

namespace {

// Written buffers (the first nout of ptrs) must not overlap any other non-null buffer.
bool disjoint(const void *const *ptrs, const size_t *sizes, const char *const *names, int n,
              int nout, const char *fn) {
    for (int i = 0; i < nout; ++i)
        for (int j = 0; j < n; ++j)
            if (j != i && ptrs[i] != nullptr && ptrs[j] != nullptr &&
                overlap(ptrs[i], sizes[i], ptrs[j], sizes[j])) {
                fail(WKV_ERR_INVALID_ARG, "%s: %s overlaps %s", fn, names[i], names[j]);
                return false;
            }
    return true;
}

bool shift_dims_ok(int64_t B, int64_t T, int64_t C, const char *fn) {
    if (!dims_ok(B, T, C, fn)) return false;
    const int64_t waves = B * ((T + 63) / 64) * ((C + 63) / 64);
    if (waves / 4 + 1 > INT32_MAX) {
        fail(WKV_ERR_INVALID_ARG, "%s: too many workgroups", fn);
        return false;
    }
    return true;
}

}  // namespace

int wkv_token_shift(int64_t B, int64_t T, int64_t C, const float *x, const float *x_prev,
                    const float *mu, float *out_r, float *out_k, float *out_v, float *x_last,
                    void *stream) {
    static const char *fn = "wkv_token_shift";
    g_err[0] = '\0';
    if (!shift_dims_ok(B, T, C, fn)) return WKV_ERR_INVALID_ARG;
    if (B == 0 || T == 0 || C == 0) return WKV_OK;
    if (!nonnull(x, "x", fn) || !nonnull(mu, "mu", fn) || !nonnull(out_r, "out_r", fn) ||
        !nonnull(out_k, "out_k", fn) || !nonnull(out_v, "out_v", fn))
        return WKV_ERR_INVALID_ARG;
    const size_t nb = (size_t)(B * T * C) * 4u, ns = (size_t)(B * C) * 4u, nm = (size_t)C * 12u;
    const void *ptrs[7] = {out_r, out_k, out_v, x_last, x, x_prev, mu};
    const size_t sizes[7] = {nb, nb, nb, ns, nb, ns, nm};
    const char *names[7] = {"out_r", "out_k", "out_v", "x_last", "x", "x_prev", "mu"};
    for (int i = 0; i < 7; ++i)
        if (ptrs[i] != nullptr && !aligned(ptrs[i], 4, names[i], fn)) return WKV_ERR_INVALID_ARG;
    if (!disjoint(ptrs, sizes, names, 7, 4, fn)) return WKV_ERR_INVALID_ARG;
    int rc = check_device(fn);
    if (rc != WKV_OK) return rc;
    hipError_t e = wkvdev::launch_shift(B, T, C, x, x_prev, mu, out_r, out_k, out_v, x_last,
                                        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip(e, fn);
    return WKV_OK;
}

size_t wkv_token_shift_backward_workspace_size(int64_t B, int64_t T, int64_t C) {
    if (B < 0 || T < 0 || C < 0 || C > kMaxC) return 0;
    if (B > 0 && T > 0 && C > 0 && (T > kMaxElems / B || B * T > kMaxElems / C)) return 0;
    return round_up((size_t)3 * (size_t)B * (size_t)wkvdev::shift_chunks(T) * (size_t)C * 8u,
                    256);
}

int wkv_token_shift_backward(int64_t B, int64_t T, int64_t C, const float *x,
                             const float *x_prev, const float *mu, const float *dout_r,
                             const float *dout_k, const float *dout_v, float *dx, float *dx_prev,
                             float *dmu, void *workspace, size_t workspace_bytes, void *stream) {
    static const char *fn = "wkv_token_shift_backward";
    g_err[0] = '\0';
    if (!shift_dims_ok(B, T, C, fn)) return WKV_ERR_INVALID_ARG;
    if (C == 0) return WKV_OK;
    if (!nonnull(dmu, "dmu", fn) || !aligned(dmu, 4, "dmu", fn)) return WKV_ERR_INVALID_ARG;
    if (B == 0 || T == 0) {
        int rc = check_device(fn);
        if (rc != WKV_OK) return rc;
        // dmu = 0 over its 3C entries
        hipError_t e = wkvdev::launch_zero2(dmu, dmu + C, C, static_cast<hipStream_t>(stream));
        if (e == hipSuccess)
            e = wkvdev::launch_zero2(dmu + 2 * C, dmu + 2 * C, C, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return fail_hip(e, fn);
        if (dx_prev != nullptr && B > 0) {
            // no token: nothing flows to the previous token's input
            e = wkvdev::launch_zero2(dx_prev, dx_prev, B * C, static_cast<hipStream_t>(stream));
            if (e != hipSuccess) return fail_hip(e, fn);
        }
        return WKV_OK;
    }
    if (!nonnull(x, "x", fn) || !nonnull(mu, "mu", fn) || !nonnull(dout_r, "dout_r", fn) ||
        !nonnull(dout_k, "dout_k", fn) || !nonnull(dout_v, "dout_v", fn) ||
        !nonnull(dx, "dx", fn) || !nonnull(workspace, "workspace", fn))
        return WKV_ERR_INVALID_ARG;
    const size_t need = wkv_token_shift_backward_workspace_size(B, T, C);
    if (workspace_bytes < need)
        return fail(WKV_ERR_INVALID_ARG, "%s: workspace has %zu bytes, needs %zu", fn,
                    workspace_bytes, need);
    if (!aligned(workspace, 16, "workspace", fn)) return WKV_ERR_INVALID_ARG;
    const size_t nb = (size_t)(B * T * C) * 4u, ns = (size_t)(B * C) * 4u, nm = (size_t)C * 12u;
    const void *ptrs[10] = {dx, dx_prev, dmu, workspace, x, x_prev, mu, dout_r, dout_k, dout_v};
    const size_t sizes[10] = {nb, ns, nm, need, nb, ns, nm, nb, nb, nb};
    const char *names[10] = {"dx", "dx_prev", "dmu", "workspace", "x", "x_prev", "mu",
                             "dout_r", "dout_k", "dout_v"};
    for (int i = 0; i < 10; ++i)
        if (i != 3 && ptrs[i] != nullptr && !aligned(ptrs[i], 4, names[i], fn))
            return WKV_ERR_INVALID_ARG;
    if (!disjoint(ptrs, sizes, names, 10, 4, fn)) return WKV_ERR_INVALID_ARG;
    int rc = check_device(fn);
    if (rc != WKV_OK) return rc;
    hipError_t e = wkvdev::launch_shift_backward(B, T, C, x, x_prev, mu, dout_r, dout_k, dout_v,
                                                 dx, dx_prev, dmu,
                                                 static_cast<double *>(workspace),
                                                 static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail_hip(e, fn);
    return WKV_OK;
}

}  // extern "C"
