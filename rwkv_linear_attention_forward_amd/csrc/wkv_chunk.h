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

// Summary of one lane's chunk from the empty state, in the chunk frame: with
// ref = max_j k_j and e_j = 2^{(k_j - ref) log2 e} <= 1 (fp64), the sums A, B, A', B'
// after the CH tokens, at scale 2^{ref log2 e}. Horner from the first token:
//   A'_{j+1} = e^{-w} (A'_j + A_j),   A_{j+1} = e^{-w} A_j + e_j v_j   (B, B' alike).
// Unless KEEPK, kc receives e_j rounded to fp32 (for outputs that need only fp32). Returns
// true (wave-uniform) if the exact form is needed instead (forced, or the fixed frame
// underflows for some lane); the caller then uses exact_summary on the raw chunk.
template <int CH, bool KEEPK>
__device__ __forceinline__ bool chunk_summary(float (&kc)[CH], const float (&vc)[CH], int Lv,
                                              float ref, bool force_exact, double dwf,
                                              Carry &sum) {
    const double refd = (double)ref;
    sum = Carry{0.0, 0.0, 0.0, 0.0, refd * kLog2eD};
    if (force_exact) return true;
    double S = 0.0, Z = 0.0, Sp = 0.0, Zp = 0.0;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const double e = (j < Lv) ? exp2_64(((double)kc[j] - refd) * kLog2eD) : 0.0;
        if (!KEEPK) kc[j] = (float)e;
        Sp = dwf * (Sp + S);
        Zp = dwf * (Zp + Z);
        S = fma(S, dwf, e * (double)vc[j]);
        Z = fma(Z, dwf, e);
    }
    sum.a = S;
    sum.b = Z;
    sum.ap = Sp;
    sum.bp = Zp;
    return wave_any(Lv > 0 && !(Z >= (double)kTinyDen));
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

// Per-token rescaled state in fp64, natural log-scale relative to the chunk frame e^{ref}:
// A = a e^p, B = b e^p, A' = a' e^p, B' = b' e^p. Used where the fixed frame would under-
// or overflow. Its sums feed carries and the gradients, which need the weights
// e^{k_i - ...} to agree with one another to far better than fp32 (dw cancels heavily),
// hence fp64 throughout.
struct Rs64 {
    double a, b, ap, bp, p;
};

// Advance by token (kr = k - ref, v): A' <- e^{-w} (A' + A), A <- e^{-w} A + e^{kr} v, and
// B', B alike. The larger of p - w and kr becomes the new scale.
__device__ __forceinline__ void rs64_push(Rs64 &s, double kr, double v, double w) {
    const double pw = s.p - w;
    const double m = fmax(pw, kr);
    const double f1 = exp(pw - m), f2 = exp(kr - m);
    s.ap = (s.ap + s.a) * f1;
    s.bp = (s.bp + s.b) * f1;
    s.a = fma(f1, s.a, f2 * v);
    s.b = fma(f1, s.b, f2);
    s.p = m;
}

// A token past the sequence end: decay only.
__device__ __forceinline__ void rs64_skip(Rs64 &s, double w) {
    s.ap += s.a;
    s.bp += s.b;
    s.p -= w;
}

// Chunk summary in the per-token form (fp64), same meaning as chunk_summary's.
template <int CH>
__device__ __forceinline__ void exact_summary(const float (&kc)[CH], const float (&vc)[CH],
                                              int Lv, float ref, double w, Carry &sum) {
    const double refd = (double)ref;
    Rs64 s{0.0, 0.0, 0.0, 0.0, kNegBigD};
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        if (j < Lv)
            rs64_push(s, (double)kc[j] - refd, (double)vc[j], w);
        else
            rs64_skip(s, w);
    }
    // A = a e^{p + ref}; the carry scale is base 2: 2^{P} = e^{p + ref}
    sum = Carry{s.a, s.b, s.ap, s.bp, (s.p + refd) * kLog2eD};
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
__device__ __forceinline__ void put_u64(uint64_t *p, double x) {
    __hip_atomic_store(p, __builtin_bit_cast(uint64_t, x), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double get_u64(const uint64_t *p) {
    return __builtin_bit_cast(double,
                              __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void put_rec(Rec *r, const Carry &c) {
    put_u64(&r->a, c.a);
    put_u64(&r->b, c.b);
    put_u64(&r->ap, c.ap);
    put_u64(&r->bp, c.bp);
    put_u64(&r->P, c.P);
}
__device__ __forceinline__ Carry get_rec(const Rec *r) {
    return Carry{get_u64(&r->a), get_u64(&r->b), get_u64(&r->ap), get_u64(&r->bp),
                 get_u64(&r->P)};
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

// c <- fold of a carry and a summary (the summary follows c in time, `len` tokens,
// len_w2 = len w log2 e).
__device__ __forceinline__ Carry follow(Carry c, const Carry &sum, double len_w2, double len) {
    fold(c, sum, len_w2, len);
    return c;
}

}  // namespace wkvdev
