// wkv_forward.hip -- WKV forward on gfx950: chunked time scan, one lane per (b, c).
//
// Operator: "RWKV解读：在Transformer的时代的新RNN", section 二.3, formula (8), evaluated
// through its recursive form (same section) as an associative scan over time, which is
// possible because the decay w does not depend on the data ("RWKV についての調査記録",
// section "Trainingについて").
//
// Work decomposition. A workgroup owns 64 channels of one sequence and NW waves; it walks
// the sequence in windows of NW*CH tokens, wave q taking the q-th CH-token chunk of each
// window. Each lane streams its channel's k and v rows (one dword per token, 256 B per
// wave per token, coalesced along C) into registers, so k and v are read from HBM exactly
// once and y is written exactly once: 12 bytes per element.
//
// Per chunk, with frame ref = max_j k_j of the lane's chunk and e_j = e^{k_j - ref} <= 1:
//   phase 1  summary from the empty state: S = sum_j e^{-(CH-1-j)w} e_j v_j, Z likewise
//            without v (Horner with the fp32 factor e^{-w}; at most CH steps, so its
//            rounding cannot compound); the chunk adds S 2^{ref log2 e} to A and Z to B.
//   scan     summaries go to LDS; after one barrier every wave folds the NW summaries of
//            the window into the window's incoming carry in order, keeping its own
//            incoming carry on the way (identical arithmetic in every wave, so the
//            window's outgoing carry needs no second barrier). Carries keep their
//            log-scale in fp64 (see wkv_device.h).
//   phase 3  outputs from the incoming carry put into the chunk frame:
//            y_j = (S_j + e^u e_j v_j) / (Z_j + e^u e_j),  S_{j+1} = e^{-w} S_j + e_j v_j.
// One exp2 per element in each phase, one reciprocal in phase 3.
//
// The fixed frame is exact in real arithmetic but can underflow when k varies by more
// than ~70 inside one chunk, or overflow when the incoming carry exceeds the chunk frame
// by 2^64. Such chunks (rare; only far outside the training distributions) are detected
// per wave and recomputed with the per-token rescaled recursion (Rs in wkv_device.h),
// which is safe for any finite k.
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
    if (t0 + CH <= T) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            kc[j] = bload(rk, voff, j * stride);
            vc[j] = bload(rv, voff, j * stride);
        }
    } else {
        const int Lv = (int)(T - t0);
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
}

template <int NW, int CH>
__global__ __launch_bounds__(NW * 64) void wkv_forward_kernel(
    int64_t T, int64_t C, int ngrp, const float *__restrict__ w, const float *__restrict__ u,
    const float *__restrict__ k, const float *__restrict__ v, float *__restrict__ y,
    float *__restrict__ sva, float *__restrict__ svb, double *__restrict__ svP) {
    constexpr int WIN = NW * CH;
    static_assert(kSaveStride % WIN == 0, "window must divide the carry save stride");
    __shared__ float s_al[2][NW][64];
    __shared__ float s_be[2][NW][64];
    __shared__ double s_sc[2][NW][64];

    const int lane = threadIdx.x & 63;
    const int q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t bidx = blockIdx.x / ngrp;
    const int grp = (int)(blockIdx.x - bidx * ngrp);
    const int64_t c = (int64_t)grp * 64 + lane;
    const bool cval = c < C;
    const int cl = (int)(cval ? c : C - 1);
    const int voff = cl * 4;

    const float wc = w[cl];
    const float uc = u[cl];
    const Decay dc = make_decay(wc);
    const float dwf = dc.dwf;
    const float eu = expf(uc);
    const double dec = (double)CH * ((double)wc * kLog2eD);
    const bool slow_lane = !(fabsf(uc) <= 60.0f);
    const bool slow_wave = wave_any(slow_lane);

    const int64_t row0 = bidx * T;
    const int64_t nwin = (T + WIN - 1) / WIN;
    const int64_t nsave = (T + kSaveStride - 1) / kSaveStride;

    Carry carry{0.0f, 0.0f, kNegBigD};
    float kc[CH], vc[CH];
    load_chunk<CH>(kc, vc, k, v, row0, (int64_t)q * CH, T, C, voff);
    int buf = 0;

    for (int64_t win = 0; win < nwin; ++win) {
        const int64_t tw = win * WIN;
        const int64_t t0 = tw + (int64_t)q * CH;
        const int Lv = (int)(t0 >= T ? 0 : (T - t0 < CH ? T - t0 : CH));

        if (svP != nullptr && q == 0 && cval && (tw % kSaveStride) == 0) {
            const int64_t si = (bidx * nsave + tw / kSaveStride) * C + c;
            sva[si] = carry.a;
            svb[si] = carry.b;
            svP[si] = carry.P;
        }

        float kn[CH], vn[CH];
        const bool more = win + 1 < nwin;
        if (more) load_chunk<CH>(kn, vn, k, v, row0, t0 + WIN, T, C, voff);

        // ---- phase 1: frame and summary of this chunk ----
        float ref = kNegBig;
#pragma unroll
        for (int j = 0; j < CH; ++j)
            if (j < Lv) ref = fmaxf(ref, kc[j]);
        const float ref2 = ref * kLog2e;
        bool exact = slow_wave;
        float S = 0.0f, Z = 0.0f;
        double sc = (double)ref2;
        if (!exact) {
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const float e = (j < Lv) ? ex2(fmaf(kc[j], kLog2e, -ref2)) : 0.0f;
                const float ev = e * vc[j];
                kc[j] = e;
                vc[j] = ev;
                S = fmaf(S, dwf, ev);
                Z = fmaf(Z, dwf, e);
            }
            exact = wave_any(Lv > 0 && !(Z >= kTinyDen));
            if (exact) load_chunk<CH>(kc, vc, k, v, row0, t0, T, C, voff);
        }
        if (exact) {
            Rs s{0.0f, 0.0f, kNegBig};
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                if (j < Lv)
                    rs_push(s, kc[j] - ref, vc[j], dc);
                else
                    s.p -= wc;
            }
            S = s.a;
            Z = s.b;
            sc = (double)ref2 + (double)s.p * kLog2eD;
        }

        // ---- scan over the window's chunks ----
        s_al[buf][q][lane] = S;
        s_be[buf][q][lane] = Z;
        s_sc[buf][q][lane] = sc;
        __syncthreads();
        Carry mine = carry;
#pragma unroll
        for (int qq = 0; qq < NW; ++qq) {
            if (qq == q) mine = carry;
            fold(carry, s_al[buf][qq][lane], s_be[buf][qq][lane], s_sc[buf][qq][lane], dec);
        }
        buf ^= 1;

        // ---- phase 3: outputs ----
        if (!exact) {
            const float gap = (float)(mine.P - (double)ref2);
            bool bad = gap > kCarryGap;
            const float s0 = ex2(gap);
            float Sx = mine.a * s0, Zx = mine.b * s0;
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                const float e = kc[j], ev = vc[j];
                const float num = fmaf(eu, ev, Sx);
                const float den = fmaf(eu, e, Zx);
                if (j < Lv) bad |= !(den >= kTinyDen);
                kc[j] = num * rcpf(den);
                Sx = fmaf(Sx, dwf, ev);
                Zx = fmaf(Zx, dwf, e);
            }
            exact = wave_any(bad);
            if (exact) load_chunk<CH>(kc, vc, k, v, row0, t0, T, C, voff);
        }
        if (exact) {
            Rs s{mine.a, mine.b, (float)((mine.P - (double)ref2) * kLn2D)};
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                if (j < Lv) {
                    const float kr = kc[j] - ref;
                    const float yj = rs_out(s, kr, vc[j], uc);
                    rs_push(s, kr, vc[j], dc);
                    kc[j] = yj;
                }
            }
        }

        // ---- store y ----
        if (Lv > 0 && cval) {
            const rsrc_t ry = make_rsrc(y + (row0 + t0) * C);
            const int stride = (int)(C * 4);
#pragma unroll
            for (int j = 0; j < CH; ++j)
                if (j < Lv) bstore(ry, kc[j], voff, j * stride);
        }

        if (more) {
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                kc[j] = kn[j];
                vc[j] = vn[j];
            }
        }
    }
}

hipError_t launch_forward(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                          const float *k, const float *v, float *y, float *sva, float *svb,
                          double *svP, hipStream_t stream) {
    constexpr int NW = 8, CH = 32;
    const int ngrp = (int)((C + 63) / 64);
    const int64_t nblk = B * ngrp;
    hipLaunchKernelGGL((wkv_forward_kernel<NW, CH>), dim3((unsigned)nblk), dim3(NW * 64), 0,
                       stream, T, C, ngrp, w, u, k, v, y, sva, svb, svP);
    return hipGetLastError();
}

}  // namespace wkvdev
