// wkv_device.h -- device helpers shared by the WKV kernels (gfx950, wave64).
//
// Two state representations are used:
//
//   Carry (a, b, a', b', P): the two sums of the recursive form of formula (8)
//     ("RWKV解读：在Transformer的时代的新RNN", section 二.3),
//       A_t = sum_{i<t} e^{-(t-1-i)w + k_i} v_i,   B_t = sum_{i<t} e^{-(t-1-i)w + k_i},
//     and their age-weighted versions, held as A = a 2^P etc. with the base-2 log-scale P,
//     all fp64. Carries move between 32-token chunks and across whole sequences; in fp64
//     their rounding cannot build up over thousands of folds, and dw (a sum whose terms
//     cancel heavily) needs them, and the weights e^{k_i - ref} inside them, far more
//     accurate than fp32.
//
//   Rs (a, b, p): the same sums per token, A = a e^p, B = b e^p, fp32, natural log-scale.
//     Used by the decode step (whose state the public API exposes) and by the exact
//     per-token path that chunks fall back to when their fixed frame would under- or
//     overflow. Its update keeps p fixed while older mass dominates and applies the decay
//     to a and b with a single rounding per step, so p carries no drift over long decode
//     runs. The decay factor itself must be exact to a few 1e-8 relative: for small w it is
//     applied as a - a (1 - e^{-w}) in one fma (1 - e^{-w} = -expm1(-w) is accurate, while
//     e^{-w} rounded to fp32 is off by up to 3e-8 per step, which compounds); for large w
//     as a e^{-w} (1 - fp32(1 - e^{-w}) would lose the small factor to cancellation).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wkv_launch.h"

namespace wkvdev {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr double kLog2eD = 1.44269504088896340736;
constexpr double kLn2D = 0.69314718055994530942;
constexpr float kNegBig = -1e30f;   // "no mass yet" log-scale: finite, so no inf - inf
constexpr double kNegBigD = -1e30;
constexpr float kTinyDen = 0x1p-100f;  // smallest in-frame denominator the fast path accepts
constexpr float kCarryGap = 64.0f;     // largest log2 gap (carry above chunk frame) accepted
constexpr double kTinySum = 0x1p-900;  // smallest fp64 chunk summary the fast path accepts
constexpr float kFaintGap = 87.0f;     // key gap below the chunk's largest whose weight
                                       // e^{-87} ~ 2^{-125.5} nears the fp32 subnormals
constexpr float kRenorm = 0x1p-40f;    // Rs renormalization threshold on b
constexpr float kRenormUp = 0x1p40f;
constexpr float kRenormLn = 27.725887222397812f;  // 40 ln 2

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcpf(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float expn(float x) { return ex2(x * kLog2e); }
__device__ __forceinline__ bool wave_any(bool pred) { return __ballot(pred) != 0ull; }
// The logistic gate 1 / (1 + e^{-x}) in fp32 (0 and 1 at the extremes, no NaN).
__device__ __forceinline__ float sigmoidf_(float x) { return rcpf(1.0f + ex2(-x * kLog2e)); }

// ---- raw buffer access: per-lane byte offset in a VGPR, per-row offset in an SGPR ----
using rsrc_t = __amdgpu_buffer_rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base) {
    // stride 0, maximal record count; word 3 = 0x00020000 selects the 32-bit raw format
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff,
                                             0x00020000);
}
// A resource of 0 records: every access through it is out of range (loads return 0,
// stores are dropped), whatever the offsets.
__device__ __forceinline__ rsrc_t make_rsrc_empty(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0, 0x00020000);
}
__device__ __forceinline__ float bload(rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 2));
}
__device__ __forceinline__ void bstore(rsrc_t r, float x, int voff, int soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), r, voff, soff, 2);
}

// ---------------------------------------------------------------------------------
// Storage formats of the [B][T][C] tensors at the boundary. Whatever the format, values are
// widened to fp32 on load and all arithmetic (and every carry and state) stays fp32/fp64;
// outputs are rounded to the format on store (round to nearest even).
// ---------------------------------------------------------------------------------
template <Io F> struct IoType;
template <> struct IoType<Io::F32> { using T = float; };
template <> struct IoType<Io::BF16> { using T = uint16_t; };
template <> struct IoType<Io::F16> { using T = uint16_t; };
template <Io F> using io_t = typename IoType<F>::T;
template <Io F> constexpr int kIoBytes = F == Io::F32 ? 4 : 2;

template <Io F> __device__ __forceinline__ float io_widen(io_t<F> x) {
    if constexpr (F == Io::F32) {
        return x;
    } else if constexpr (F == Io::BF16) {
        return __builtin_bit_cast(float, (unsigned)x << 16);
    } else {
        return (float)__builtin_bit_cast(_Float16, x);
    }
}
template <Io F> __device__ __forceinline__ io_t<F> io_narrow(float x) {
    if constexpr (F == Io::F32) {
        return x;
    } else if constexpr (F == Io::BF16) {
        // round to nearest even (a NaN stays a NaN) with gfx950's conversion instruction
        // (v_cvt_pk_bf16_f32: one instruction where the integer rounding took five; the
        // bf16 forward 196 -> 187 us, the backward 312 -> 297 us on the 3B-class shape, with
        // bitwise the same outputs). The fp32 value is materialized first, as for fp16.
        asm volatile("" : "+v"(x));
        return __builtin_bit_cast(uint16_t, (__bf16)x);
    } else {
        // the fp32 value is materialized first, so that the rounding to 16 bits is always of
        // the fp32 result (the compiler would otherwise fold a final product into a
        // mixed-precision multiply-add that rounds once, straight to 16 bits)
        asm volatile("" : "+v"(x));
        return __builtin_bit_cast(uint16_t, (_Float16)x);
    }
}
// Element i of a tensor in format F, widened (plain load, for the rare per-token paths).
template <Io F> __device__ __forceinline__ float io_ld(const io_t<F> *p, int64_t i) {
    return io_widen<F>(p[i]);
}
template <Io F> __device__ __forceinline__ void io_st(io_t<F> *p, int64_t i, float x) {
    p[i] = io_narrow<F>(x);
}
// Buffer load/store of one element per lane; voff, soff in bytes.
template <Io F> __device__ __forceinline__ float bload_io(rsrc_t r, int voff, int soff) {
    if constexpr (F == Io::F32)
        return bload(r, voff, soff);
    else
        return io_widen<F>((uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 2));
}
template <Io F> __device__ __forceinline__ void bstore_io(rsrc_t r, float x, int voff, int soff) {
    if constexpr (F == Io::F32)
        bstore(r, x, voff, soff);
    else
        __builtin_amdgcn_raw_buffer_store_b16(io_narrow<F>(x), r, voff, soff, 2);
}

// ---------------------------------------------------------------------------------
// fp64 power of two.
// ---------------------------------------------------------------------------------
// 2^x in fp64 for x <= 1023 (arguments below -1100, -inf included, give 0). x = n + f with
// n = rint(x), |f| <= 1/2; 2^f by a degree-7 polynomial fitted for relative error on
// [-1/2, 1/2] (weighted least squares with Lawson reweighting toward the minimax fit;
// max relative error 4.0e-11, checked against extended-precision 2^f), then the exponent
// n is applied exactly. That is ~1500 times finer than fp32 rounding, which is what the
// carries and gradients need the weights e^{k - ref} for.
__device__ __forceinline__ double exp2_64(double x) {
    x = fmax(x, -1100.0);
    const double n = rint(x);
    const double f = x - n;  // exact
    double p = 1.5201917955622472e-05;
    p = fma(p, f, 1.5469291108814392e-04);
    p = fma(p, f, 1.3333922579229899e-03);
    p = fma(p, f, 9.6180272537891073e-03);
    p = fma(p, f, 5.5504103534287648e-02);
    p = fma(p, f, 2.4022651198156497e-01);
    p = fma(p, f, 6.9314718072845216e-01);
    p = fma(p, f, 9.9999999996168176e-01);
    return ldexp(p, (int)n);
}

// ---------------------------------------------------------------------------------
// Carry (a, b, a', b', P), base 2, fp64.
// ---------------------------------------------------------------------------------
// Besides A and B the carry holds the age-weighted sums that w's gradient needs,
//   A'_t = sum_{i<t} (t-1-i) e^{-(t-1-i)w + k_i} v_i,   B'_t likewise without v_i,
// which advance as A'_{t+1} = e^{-w} (A'_t + A_t). All four share the scale 2^P.
struct Carry {
    double a, b, ap, bp;
    double P;
};

// c <- c advanced over `len` tokens (decay 2^{-dec}, dec = len w log2 e) plus the summary
// s of those tokens taken from the empty state. The larger of the two scales becomes the
// new one, so every factor applied is <= 1.
__device__ __forceinline__ void fold(Carry &c, const Carry &s, double dec, double len) {
    const double Pd = c.P - dec;
    const double d = s.P - Pd;
    const double f = exp2_64(-fabs(d));
    const bool up = d >= 0.0;
    const double ca = up ? f : 1.0;
    const double cs = up ? 1.0 : f;
    const double a = c.a, b = c.b;
    c.a = fma(a, ca, s.a * cs);
    c.b = fma(b, ca, s.b * cs);
    c.ap = fma(fma(len, a, c.ap), ca, s.ap * cs);
    c.bp = fma(fma(len, b, c.bp), ca, s.bp * cs);
    c.P = up ? s.P : Pd;
}

__device__ __forceinline__ Carry carry_empty() { return Carry{0.0, 0.0, 0.0, 0.0, kNegBigD}; }

// Move a carry's scale so that b lies in [1, 2) (exact: a power-of-two rescale), so that
// the scale P says how large the mass is. Empty carries are left alone.
__device__ __forceinline__ void normalize(Carry &c) {
    if (c.b > 0.0) {
        const int e = __builtin_amdgcn_frexp_exp(c.b) - 1;
        c.a = ldexp(c.a, -e);
        c.b = ldexp(c.b, -e);
        c.ap = ldexp(c.ap, -e);
        c.bp = ldexp(c.bp, -e);
        c.P += (double)e;
    }
}

// 1/x in fp64 from the fp32 reciprocal and one Newton step (relative error ~1e-14 for x
// in the fp32 normal range, which the callers guarantee).
__device__ __forceinline__ double rcpd(double x) {
    const double r0 = (double)rcpf((float)x);
    return fma(r0, fma(-x, r0, 1.0), r0);
}

// The logistic gate in fp64, 1 / (1 + 2^{-x log2 e}) (exp2_64 and rcpd; the argument is
// capped so that a very negative x gives 0 rather than inf/inf).
__device__ __forceinline__ double sigmoid64(float x) {
    return rcpd(1.0 + exp2_64(fmin(-(double)x * kLog2eD, 200.0)));
}

// ---------------------------------------------------------------------------------
// Rs (a, b, p), natural log-scale, per token.
// ---------------------------------------------------------------------------------
struct Rs {
    float a, b, p;
};

// Output for token (k, v) from the state before it:
//   y = (e^p a + e^{u+k} v) / (e^p b + e^{u+k}), evaluated with the larger exponent as 0.
// The quotient is taken as a product with the hardware reciprocal (about 1 ulp; the
// denominator is at least 1 whenever the state holds any mass, and e2 = 1 otherwise).
__device__ __forceinline__ float rs_out(const Rs &s, float k, float v, float u) {
    const float uk = u + k;
    const float d = s.p - uk;
    const float e = expn(-fabsf(d));
    const bool sp = d >= 0.0f;
    const float e1 = sp ? 1.0f : e;
    const float e2 = sp ? e : 1.0f;
    return fmaf(e1, s.a, e2 * v) * rcpf(fmaf(e1, s.b, e2));
}

// Per-channel decay constants for rs_push.
struct Decay {
    float w;      // the rate
    float dwf;    // e^{-w}
    float omw;    // 1 - e^{-w}, accurate for small w
    bool small;   // apply the decay as a - a*omw (small w) or a*dwf (large w)
};

__device__ __forceinline__ Decay make_decay(float w) {
    Decay d;
    d.w = w;
    d.dwf = expf(-w);
    d.omw = -expm1f(-w);
    d.small = w < 0.5f;
    return d;
}

// Advance the state by token (k, v): A <- e^{-w} A + e^k v, B <- e^{-w} B + e^k.
// If k <= p the scale stays and the old sums are decayed in place; otherwise the scale
// moves to k and the old sums are scaled by e^{p-w-k} <= 1.
__device__ __forceinline__ void rs_push(Rs &s, float k, float v, const Decay &dc) {
    const float d = k - s.p;
    const bool keep = d <= 0.0f;
    const float e = expn(keep ? d : -(d + dc.w));
    const float ka = dc.small ? fmaf(-s.a, dc.omw, s.a) : s.a * dc.dwf;
    const float kb = dc.small ? fmaf(-s.b, dc.omw, s.b) : s.b * dc.dwf;
    const float ad = keep ? ka : s.a * e;
    const float bd = keep ? kb : s.b * e;
    const float f = keep ? e : 1.0f;
    s.a = fmaf(v, f, ad);
    s.b = bd + f;
    s.p = keep ? s.p : k;
    if (s.b < kRenorm) {
        s.a *= kRenormUp;
        s.b *= kRenormUp;
        s.p -= kRenormLn;
    }
}

}  // namespace wkvdev
