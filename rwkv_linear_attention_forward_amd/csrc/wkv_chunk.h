// wkv_chunk.h -- chunk-level device helpers shared by the forward and backward kernels:
// streaming a lane's CH-token chunk, the chunk frame and forward summary, and publishing
// and reading per-window records between workgroups (device scope).
#pragma once

#include "wkv_device.h"
#include "wkv_launch.h"

namespace wkvdev {

// Load a CH-token chunk of one lane's channel starting at token t0 (rows past T are 0).
template <int CH>
__device__ __forceinline__ void load_chunk(float (&kc)[CH], float (&vc)[CH],
                                           const float *__restrict__ k,
                                           const float *__restrict__ v, int64_t row0,
                                           int64_t t0, int64_t T, int64_t C, int voff) {
    if (t0 >= T) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            kc[j] = 0.0f;
            vc[j] = 0.0f;
        }
        return;
    }
    const rsrc_t rk = make_rsrc(k + (row0 + t0) * C);
    const rsrc_t rv = make_rsrc(v + (row0 + t0) * C);
    const int stride = (int)(C * 4);
    const int Lv = (int)(T - t0 < CH ? T - t0 : CH);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        if (j < Lv) {
            kc[j] = bload(rk, voff, j * stride);
            vc[j] = bload(rv, voff, j * stride);
        } else {
            kc[j] = 0.0f;
            vc[j] = 0.0f;
        }
    }
}

// Summary of one lane's chunk from the empty state: (S, Z) at scale 2^sc, in the fast
// form, which leaves e_j in kc (and e_j v_j in vc unless KEEPV). Returns true
// (wave-uniform) if the exact form is needed instead (forced, or the fixed frame underflows
// for some lane); the caller then reloads the raw chunk and uses exact_summary.
template <int CH, bool KEEPV = false>
__device__ __forceinline__ bool chunk_summary(float (&kc)[CH], float (&vc)[CH], int Lv,
                                              float ref, bool force_exact, const Decay &dc,
                                              float &S, float &Z, double &sc) {
    const float ref2 = ref * kLog2e;
    S = 0.0f;
    Z = 0.0f;
    sc = (double)ref2;
    if (force_exact) return true;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const float e = (j < Lv) ? ex2(fmaf(kc[j], kLog2e, -ref2)) : 0.0f;
        const float ev = e * vc[j];
        kc[j] = e;
        if (!KEEPV) vc[j] = ev;
        S = fmaf(S, dc.dwf, ev);
        Z = fmaf(Z, dc.dwf, e);
    }
    return wave_any(Lv > 0 && !(Z >= kTinyDen));
}

// Load one tensor's CH-token chunk (rows past T are 0).
template <int CH>
__device__ __forceinline__ void load_chunk1(float (&gc)[CH], const float *__restrict__ g,
                                            int64_t row0, int64_t t0, int64_t T, int64_t C,
                                            int voff) {
    if (t0 >= T) {
#pragma unroll
        for (int j = 0; j < CH; ++j) gc[j] = 0.0f;
        return;
    }
    const rsrc_t rg = make_rsrc(g + (row0 + t0) * C);
    const int stride = (int)(C * 4);
    const int Lv = (int)(T - t0 < CH ? T - t0 : CH);
#pragma unroll
    for (int j = 0; j < CH; ++j) gc[j] = (j < Lv) ? bload(rg, voff, j * stride) : 0.0f;
}

// Valid tokens of the chunk starting at t0.
__device__ __forceinline__ int chunk_len(int64_t t0, int64_t T, int CH) {
    return (int)(t0 >= T ? 0 : (T - t0 < CH ? T - t0 : CH));
}

template <int CH>
__device__ __forceinline__ void exact_summary(const float (&kc)[CH], const float (&vc)[CH],
                                              int Lv, float ref, const Decay &dc, float &S,
                                              float &Z, double &sc) {
    Rs s{0.0f, 0.0f, kNegBig};
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        if (j < Lv)
            rs_push(s, kc[j] - ref, vc[j], dc);
        else
            s.p -= dc.w;
    }
    S = s.a;
    Z = s.b;
    sc = (double)(ref * kLog2e) + (double)s.p * kLog2eD;
}

template <int CH>
__device__ __forceinline__ float chunk_ref(const float (&kc)[CH], int Lv) {
    float ref = kNegBig;
#pragma unroll
    for (int j = 0; j < CH; ++j)
        if (j < Lv) ref = fmaxf(ref, kc[j]);
    return ref;
}

// ---- publication records (device-scope, see wkv_launch.h for the layout) ----
__device__ __forceinline__ void put_rec(Rec *r, const Carry &c) {
    const uint64_t ab = ((uint64_t)__builtin_bit_cast(uint32_t, c.b) << 32) |
                        (uint64_t)__builtin_bit_cast(uint32_t, c.a);
    __hip_atomic_store(&r->ab, ab, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&r->P, __builtin_bit_cast(uint64_t, c.P), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ Carry get_rec(const Rec *r) {
    const uint64_t ab = __hip_atomic_load(&r->ab, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t P = __hip_atomic_load(&r->P, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    Carry c;
    c.a = __builtin_bit_cast(float, (uint32_t)(ab & 0xffffffffu));
    c.b = __builtin_bit_cast(float, (uint32_t)(ab >> 32));
    c.P = __builtin_bit_cast(double, P);
    return c;
}
__device__ __forceinline__ void put_flag(uint64_t *f, uint64_t epoch, uint64_t status) {
    __hip_atomic_store(f, (epoch << 2) | status, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}
// Publish `status` unless a higher status of this call is already there (a helper that
// recomputed an aggregate must not hide the owner's inclusive carry).
__device__ __forceinline__ void raise_flag(uint64_t *f, uint64_t epoch, uint64_t status) {
    __hip_atomic_fetch_max(f, (epoch << 2) | status, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// Status of a unit's publication for this call: 1 aggregate, 2 inclusive carry, or 0 if
// nothing was published within `tries` polls (the caller then recomputes; no unit ever
// waits without bound).
__device__ __forceinline__ int poll_flag(const uint64_t *f, uint64_t epoch, int tries) {
    for (int i = 0;; ++i) {
        const uint64_t x = __hip_atomic_load(f, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
        if ((x >> 2) == epoch && (x & 3u) != 0u) return (int)(x & 3u);
        if (i >= tries) return 0;
        __builtin_amdgcn_s_sleep(4);
    }
}

// c <- fold of a carry and a summary (the summary follows c in time, length `len` tokens).
__device__ __forceinline__ Carry follow(Carry c, const Carry &sum, double len_w2) {
    fold(c, sum.a, sum.b, sum.P, len_w2);
    return c;
}

}  // namespace wkvdev
