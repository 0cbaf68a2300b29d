// wkv_shift.hip -- the token-shift mix that produces the inputs of the R, K, V projections.
//
// "RWKV解读：在Transformer的时代的新RNN", section 二.3, formula (7): the input from which R, K and
// V are computed is a weighted sum of the current and the previous token's input, with a
// trained per-channel weight for each of the three:
//     out_m[t] = mu_m x[t] + (1 - mu_m) x[t-1],   m = r, k, v,
// x[-1] being the previous call's last token (0 for a fresh sequence). The projections are
// matrix products and not part of this.
//
// Elementwise and HBM-bound: x is read once and the three mixes written (16 B per element;
// the backward reads the three cotangents and x and writes dx, 20 B). One lane per channel
// (or per 4 channels, with 16-byte accesses) and one wave per kShiftTokens tokens of one
// sequence: the wave's loads are issued together, then the tokens are walked in order with
// the previous token carried in registers, so x[t-1] is never read twice.
#include <initializer_list>

#include "wkv_device.h"

namespace wkvdev {

constexpr int kShiftTokens = 32;

// VEC consecutive channels per lane (4 when C % 4 == 0 and every pointer is 16-byte aligned:
// 16-byte accesses, 1 KB per wave per row; else 1). A wave covers 64 * VEC channels.
template <int VEC> struct VecT;
template <> struct VecT<1> { using T = float; };
template <> struct VecT<4> { using T = float4; };
template <int VEC> __device__ __forceinline__ float lane_of(const typename VecT<VEC>::T &x, int i) {
    if constexpr (VEC == 1) {
        return x;
    } else {
        return i == 0 ? x.x : i == 1 ? x.y : i == 2 ? x.z : x.w;
    }
}
template <int VEC> __device__ __forceinline__ void set_lane(typename VecT<VEC>::T &x, int i, float v) {
    if constexpr (VEC == 1) {
        x = v;
    } else {
        if (i == 0) x.x = v; else if (i == 1) x.y = v; else if (i == 2) x.z = v; else x.w = v;
    }
}
template <int VEC>
__device__ __forceinline__ typename VecT<VEC>::T vload(const float *p) {
    return *reinterpret_cast<const typename VecT<VEC>::T *>(p);
}
template <int VEC>
__device__ __forceinline__ void vstore(float *p, const typename VecT<VEC>::T &x) {
    *reinterpret_cast<typename VecT<VEC>::T *>(p) = x;
}

template <int VEC>
__global__ __launch_bounds__(256) void wkv_shift_kernel(
    int64_t T, int64_t C, int ngrp, int64_t nchunk, int64_t nwaves,
    const float *__restrict__ x, const float *__restrict__ x_prev,
    const float *__restrict__ mu, float *__restrict__ o_r, float *__restrict__ o_k,
    float *__restrict__ o_v, float *__restrict__ x_last) {
    using V = typename VecT<VEC>::T;
    const int lane = threadIdx.x & 63;
    const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wv >= nwaves) return;  // whole waves only
    const int64_t g = wv % ngrp, rest = wv / ngrp;
    const int64_t chunk = rest % nchunk, b = rest / nchunk;
    const int64_t c = (g * 64 + lane) * VEC;  // first channel of the lane
    const bool cval = c < C;                   // C % VEC == 0 when VEC > 1
    const int64_t cl = cval ? c : C - VEC;
    const int64_t t0 = chunk * kShiftTokens;
    const int64_t t1 = t0 + kShiftTokens < T ? t0 + kShiftTokens : T;
    const V mr = vload<VEC>(mu + cl), mk = vload<VEC>(mu + C + cl), mv = vload<VEC>(mu + 2 * C + cl);
    V prev;
    if (t0 > 0) {
        prev = vload<VEC>(x + ((b * T) + t0 - 1) * C + cl);
    } else if (x_prev != nullptr) {
        prev = vload<VEC>(x_prev + b * C + cl);
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) set_lane<VEC>(prev, i, 0.0f);
    }
    // the wave's tokens loaded together (a token past t1 repeats the last), then walked
    const int n = (int)(t1 - t0);
    V xs[kShiftTokens];
#pragma unroll
    for (int j = 0; j < kShiftTokens; ++j)
        xs[j] = vload<VEC>(x + (b * T + t0 + (j < n ? j : n - 1)) * C + cl);
#pragma unroll
    for (int j = 0; j < kShiftTokens; ++j) {
        if (j < n) {
            const int64_t i0 = (b * T + t0 + j) * C + cl;
            const V xt = xs[j];
            V a, bk, cv;
#pragma unroll
            for (int i = 0; i < VEC; ++i) {
                const float xi = lane_of<VEC>(xt, i), pi = lane_of<VEC>(prev, i);
                const float r = lane_of<VEC>(mr, i), k = lane_of<VEC>(mk, i), v = lane_of<VEC>(mv, i);
                set_lane<VEC>(a, i, fmaf(r, xi, (1.0f - r) * pi));
                set_lane<VEC>(bk, i, fmaf(k, xi, (1.0f - k) * pi));
                set_lane<VEC>(cv, i, fmaf(v, xi, (1.0f - v) * pi));
            }
            if (cval) {
                vstore<VEC>(o_r + i0, a);
                vstore<VEC>(o_k + i0, bk);
                vstore<VEC>(o_v + i0, cv);
            }
            prev = xt;
        }
    }
    if (x_last != nullptr && t1 == T && cval) vstore<VEC>(x_last + b * C + c, prev);
}

// Backward of L = sum_m sum dout_m * out_m, walking the tokens backwards:
//   dx[t]    = sum_m mu_m d_m[t] + sum_m (1 - mu_m) d_m[t+1]   (the second sum is 0 at T-1)
//   dx_prev  = sum_m (1 - mu_m) d_m[0]
//   dmu_m    = sum_{b,t} (x[t] - x[t-1]) d_m[t]   (fp64; a partial per wave, then summed)
// One lane per channel; the wave's tokens in batches of kShiftBatch, the last batch first,
// each batch's loads (three cotangents and x[t-1] per token) issued together before the
// batch is walked, so that a wave keeps 32 loads in flight (a batch of 8 measured
// 321 us on the 3B-class shape, 16 tokens 329, the whole 32 at once 375, one token at a
// time with the loop unrolled twice 366).
constexpr int kShiftBatch = 8;

__global__ __launch_bounds__(256) void wkv_shift_backward_kernel(
    int64_t T, int64_t C, int ngrp, int64_t nchunk, int64_t nwaves,
    const float *__restrict__ x, const float *__restrict__ x_prev,
    const float *__restrict__ mu, const float *__restrict__ d_r,
    const float *__restrict__ d_k, const float *__restrict__ d_v, float *__restrict__ dx,
    float *__restrict__ dx_prev, double *__restrict__ part) {
    const int lane = threadIdx.x & 63;
    const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wv >= nwaves) return;
    const int64_t g = wv % ngrp, rest = wv / ngrp;
    const int64_t chunk = rest % nchunk, b = rest / nchunk;
    const int64_t c = g * 64 + lane;
    const bool cval = c < C;
    const int64_t cl = cval ? c : C - 1;
    const int voff = (int)(cl * 4);
    const int stride = (int)(C * 4);
    const int64_t t0 = chunk * kShiftTokens;
    const int64_t t1 = t0 + kShiftTokens < T ? t0 + kShiftTokens : T;
    const float mr = mu[cl], mk = mu[C + cl], mv = mu[2 * C + cl];
    const float nr = 1.0f - mr, nk = 1.0f - mk, nv = 1.0f - mv;
    float next = 0.0f;  // sum_m (1 - mu_m) d_m[t+1]
    if (t1 < T) {
        const int64_t i0 = (b * T + t1) * C + cl;
        next = fmaf(nr, d_r[i0], fmaf(nk, d_k[i0], nv * d_v[i0]));
    }
    float xt = x[(b * T + t1 - 1) * C + cl];
    // x[-1] of the sequence: the previous call's last token, or 0
    const float xfirst = (t0 == 0 && x_prev != nullptr) ? x_prev[b * C + cl] : 0.0f;
    double sr = 0.0, sk = 0.0, sv = 0.0;
    for (int64_t hi = t1; hi > t0; hi -= kShiftBatch) {
        const int n = (int)(hi - t0 < kShiftBatch ? hi - t0 : kShiftBatch);  // wave-uniform
        const int64_t tb = hi - n;                                            // first token
        const int64_t row = (b * T + tb) * C;
        const rsrc_t rr = make_rsrc(d_r + row), rk = make_rsrc(d_k + row),
                     rv = make_rsrc(d_v + row), rd = make_rsrc(dx + row);
        // x[t-1] for t = tb + i: row tb - 1 + i; at tb == 0 the token t = 0 reads row 0 and
        // takes xfirst instead
        const rsrc_t rx = make_rsrc(x + (tb > 0 ? row - C : row));
        float ga[kShiftBatch], gb[kShiftBatch], gc[kShiftBatch], xp[kShiftBatch];
#pragma unroll
        for (int j = 0; j < kShiftBatch; ++j) {
            const int i = j < n ? n - 1 - j : 0;  // token tb + i, the last of the batch first
            const int ix = tb > 0 ? i : (i > 0 ? i - 1 : 0);
            ga[j] = bload(rr, voff, i * stride);
            gb[j] = bload(rk, voff, i * stride);
            gc[j] = bload(rv, voff, i * stride);
            xp[j] = bload(rx, voff, ix * stride);
        }
#pragma unroll
        for (int j = 0; j < kShiftBatch; ++j) {
            if (j < n) {
                const int i = n - 1 - j;
                const float xpj = (tb == 0 && i == 0) ? xfirst : xp[j];
                const float o = fmaf(mr, ga[j], fmaf(mk, gb[j], fmaf(mv, gc[j], next)));
                const double diff = (double)xt - (double)xpj;
                sr = fma(diff, (double)ga[j], sr);
                sk = fma(diff, (double)gb[j], sk);
                sv = fma(diff, (double)gc[j], sv);
                next = fmaf(nr, ga[j], fmaf(nk, gb[j], nv * gc[j]));
                xt = xpj;
                if (cval) bstore(rd, o, voff, i * stride);
            }
        }
    }
    if (cval) {
        if (t0 == 0 && dx_prev != nullptr) dx_prev[b * C + c] = next;
        const int64_t npart = nwaves / ngrp, pr = b * nchunk + chunk;
        part[pr * C + c] = sr;
        part[(npart + pr) * C + c] = sk;
        part[(2 * npart + pr) * C + c] = sv;
    }
}

// out[f][c] = sum of part[f][i][c] over the npart rows, in a fixed order (f = 0, 1, 2): as
// the dw/du reduction, 16 channels x 32 row slices per workgroup.
__global__ __launch_bounds__(512) void wkv_shift_reduce_kernel(int64_t npart, int64_t C,
                                                               const double *__restrict__ part,
                                                               float *__restrict__ out) {
    constexpr int CH = 16, RS = 32;
    __shared__ double acc[3][RS][CH];
    const int ch = (int)threadIdx.x % CH, sl = (int)threadIdx.x / CH;
    const int64_t c = (int64_t)blockIdx.x * CH + ch;
    const int64_t cl = c < C ? c : C - 1;
    double s[3] = {0.0, 0.0, 0.0};
    for (int64_t i = sl; i < npart; i += RS)
#pragma unroll
        for (int f = 0; f < 3; ++f) s[f] += part[(f * npart + i) * C + cl];
#pragma unroll
    for (int f = 0; f < 3; ++f) acc[f][sl][ch] = s[f];
    __syncthreads();
    if (sl == 0 && c < C) {
#pragma unroll
        for (int f = 0; f < 3; ++f) {
            double t = 0.0;
            for (int r = 0; r < RS; ++r) t += acc[f][r][ch];
            out[f * C + c] = (float)t;
        }
    }
}

int64_t shift_chunks(int64_t T) { return (T + kShiftTokens - 1) / kShiftTokens; }

// 4 channels per lane when C % 4 == 0 and every pointer is 16-byte aligned.
static bool vec4_ok(int64_t C, std::initializer_list<const void *> ptrs) {
    if (C % 4 != 0) return false;
    for (const void *p : ptrs)
        if (p != nullptr && reinterpret_cast<uintptr_t>(p) % 16 != 0) return false;
    return true;
}

hipError_t launch_shift(int64_t B, int64_t T, int64_t C, const float *x, const float *x_prev,
                        const float *mu, float *o_r, float *o_k, float *o_v, float *x_last,
                        hipStream_t stream) {
    const bool v4 = vec4_ok(C, {x, x_prev, mu, mu + C, o_r, o_k, o_v, x_last});
    const int vec = v4 ? 4 : 1;
    const int ngrp = (int)((C / vec + 63) / 64);
    const int64_t nchunk = shift_chunks(T), nwaves = B * nchunk * ngrp;
    const dim3 grid((unsigned)((nwaves + 3) / 4)), block(256);
    if (v4)
        hipLaunchKernelGGL(wkv_shift_kernel<4>, grid, block, 0, stream, T, C, ngrp, nchunk,
                           nwaves, x, x_prev, mu, o_r, o_k, o_v, x_last);
    else
        hipLaunchKernelGGL(wkv_shift_kernel<1>, grid, block, 0, stream, T, C, ngrp, nchunk,
                           nwaves, x, x_prev, mu, o_r, o_k, o_v, x_last);
    return hipGetLastError();
}

hipError_t launch_shift_backward(int64_t B, int64_t T, int64_t C, const float *x,
                                 const float *x_prev, const float *mu, const float *d_r,
                                 const float *d_k, const float *d_v, float *dx, float *dx_prev,
                                 float *dmu, double *part, hipStream_t stream) {
    // one channel per lane: 4 per lane with 16-byte accesses measured slower here, unlike
    // the forward
    const int ngrp = (int)((C + 63) / 64);
    const int64_t nchunk = shift_chunks(T), nwaves = B * nchunk * ngrp;
    hipLaunchKernelGGL(wkv_shift_backward_kernel, dim3((unsigned)((nwaves + 3) / 4)),
                       dim3(256), 0, stream, T, C, ngrp, nchunk, nwaves, x, x_prev, mu, d_r, d_k,
                       d_v, dx, dx_prev, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(wkv_shift_reduce_kernel, dim3((unsigned)((C + 15) / 16)), dim3(512), 0,
                       stream, B * nchunk, C, part, dmu);
    return hipGetLastError();
}

}  // namespace wkvdev
