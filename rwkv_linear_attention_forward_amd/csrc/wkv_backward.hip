// wkv_backward.hip -- WKV backward on gfx950: dk, dv, dw, du of L = sum dy * y.
//
// Gradients of the operator of "RWKV解读：在Transformer的时代的新RNN", section 二.3,
// formula (8); "RWKV についての調査記録", section "Trainingについて" (all parameters are
// trained by gradient descent, w and u being per-channel vectors).
//
// With D_t the denominator of y_t, s_t = dy_t / D_t, and the future sums
//   G_i = sum_{t>i} e^{-(t-1-i)w} s_t,   H_i = same with s_t y_t,
//   G'_i = sum_{t>i} (t-1-i) e^{-(t-1-i)w} s_t,   H'_i = same with s_t y_t,
// the gradients are
//   dv_i = s_i e^{u+k_i} + e^{k_i} G_i
//   dk_i = s_i e^{u+k_i} (v_i - y_i) + e^{k_i} (v_i G_i - H_i)
//   du   = sum_i s_i e^{u+k_i} (v_i - y_i)
//   dw   = -sum_i e^{k_i} (v_i G'_i - H'_i)
// (the O(T^2) softmax form gives the same sums term by term).
//
// Work decomposition as in the forward (64 channels x one 256-token window per workgroup,
// one CH-token chunk per wave), with units numbered from the last window backwards so that
// the future of a unit was launched first. Each unit reads k, v, dy once and writes dk, dv
// once: 20 bytes per element. The forward state entering the window is read from the
// forward's workspace, so no extra pass over k and v is needed.
//
// Per chunk, in the forward pass's chunk frame (ref = max k, e_j = e^{k_j - ref}):
//   F1/F3  recompute y_j and den_j exactly as the forward does; sigma_j = dy_j / den_j is
//          s_t expressed in the frame.
//   R1     reverse summary of the chunk from a zero future, by Horner from the chunk end:
//          R_{j-1} = e^{-w} R_j + sigma_j, Q likewise with sigma_j y_j,
//          X_{j-1} = e^{-w} (X_j + R_j), Y likewise with Q (the age-weighted sums).
//   scan   reverse summaries are folded through LDS and across windows (decoupled
//          look-back toward later windows) into the future sums at each chunk's end.
//   R3     the same recursion from the incoming future sums gives, per token,
//          e^{k_i} G_i = e_i R_i etc., hence dv, dk, and the dw, du contributions.
// The fixed frame needs no exponential in R1/R3 at all. Chunks whose frame would under- or
// overflow are redone with a per-token rescaled recursion (exact_chunk_bwd).
#include "wkv_chunk.h"

namespace wkvdev {

// Future sums (G, H, G', H') = (g, h, gp, hp) 2^r.
struct RevCarry {
    float g, h, gp, hp;
    double r;
};

__device__ __forceinline__ RevCarry rev_zero() { return RevCarry{0.f, 0.f, 0.f, 0.f, kNegBigD}; }

// c <- the future seen from `len` tokens earlier, where `sum` summarizes those `len` tokens
// (from a zero future) and c was the future beyond them:
//   G <- e^{-len w} G + sum.G,   G' <- e^{-len w} (G' + len G) + sum.G'   (H, H' alike).
__device__ __forceinline__ void rfold(RevCarry &c, const RevCarry &sum, double len_w2,
                                      float len) {
    const double rd = c.r - len_w2;
    const float d = (float)(sum.r - rd);
    const float f = ex2(-fabsf(d));
    const bool up = d >= 0.0f;
    const float ca = up ? f : 1.0f;
    const float cs = up ? 1.0f : f;
    const float g = c.g, h = c.h;
    c.g = fmaf(g, ca, sum.g * cs);
    c.h = fmaf(h, ca, sum.h * cs);
    c.gp = fmaf(fmaf(len, g, c.gp), ca, sum.gp * cs);
    c.hp = fmaf(fmaf(len, h, c.hp), ca, sum.hp * cs);
    c.r = up ? sum.r : rd;
}

__device__ __forceinline__ RevCarry rfollow(RevCarry c, const RevCarry &sum, double len_w2,
                                            float len) {
    rfold(c, sum, len_w2, len);
    return c;
}

// Rescale so that the largest |mantissa| lies in [1, 2) (exact), making r the magnitude.
__device__ __forceinline__ void rnormalize(RevCarry &c) {
    const float m = fmaxf(fmaxf(fabsf(c.g), fabsf(c.h)), fmaxf(fabsf(c.gp), fabsf(c.hp)));
    if (m > 0.0f && m <= 3.0e38f) {
        const int e = __builtin_amdgcn_frexp_expf(m) - 1;
        c.g = ldexpf(c.g, -e);
        c.h = ldexpf(c.h, -e);
        c.gp = ldexpf(c.gp, -e);
        c.hp = ldexpf(c.hp, -e);
        c.r += (double)e;
    }
}

__device__ __forceinline__ uint64_t pack2(float x, float y) {
    return ((uint64_t)__builtin_bit_cast(uint32_t, y) << 32) |
           (uint64_t)__builtin_bit_cast(uint32_t, x);
}
__device__ __forceinline__ float lo32(uint64_t v) {
    return __builtin_bit_cast(float, (uint32_t)(v & 0xffffffffu));
}
__device__ __forceinline__ float hi32(uint64_t v) {
    return __builtin_bit_cast(float, (uint32_t)(v >> 32));
}

__device__ __forceinline__ void put_rrec(RevRec *p, const RevCarry &c) {
    __hip_atomic_store(&p->gh, pack2(c.g, c.h), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p->gphp, pack2(c.gp, c.hp), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&p->r, __builtin_bit_cast(uint64_t, c.r), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ RevCarry get_rrec(const RevRec *p) {
    const uint64_t gh = __hip_atomic_load(&p->gh, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t gphp = __hip_atomic_load(&p->gphp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t r = __hip_atomic_load(&p->r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return RevCarry{lo32(gh), hi32(gh), lo32(gphp), hi32(gphp), __builtin_bit_cast(double, r)};
}

// ---------------------------------------------------------------------------------
// Exact per-token backward of one lane's chunk (tokens [0, Lv)), for chunks whose fixed
// frame would under- or overflow. On entry kc, vc, gc hold the raw k, v, dy; they and yc
// are clobbered. `fin` is the forward carry entering the chunk, `rin` the future sums at
// the chunk's nominal end (CH tokens after its start). The chunk is done in two halves:
// the forward recursion is rerun from `fin` for each half and its per-token quantities
// (k - ref, v, y, dy / den, log-scale of D) are kept only for that half, which is then
// swept backwards. With OUT, dk and dv are stored and the du, dw contributions added.
// Returns the future sums at the chunk start.
// ---------------------------------------------------------------------------------
struct RevState {  // (R, Q, X, Y) = (g, h, gp, hp) e^r, natural scale relative to e^{ref}
    float g, h, gp, hp, r;
};

template <int CH, int J0, int J1, bool STORE>
__device__ __forceinline__ void exact_fwd_steps(float (&kc)[CH], float (&vc)[CH],
                                                float (&gc)[CH], float (&yc)[CH], int Lv,
                                                float ref, float uc, const Decay &dc, Rs &st) {
    constexpr int H = CH / 2;
#pragma unroll
    for (int j = J0; j < J1; ++j) {
        if (j < Lv) {
            const float kr = kc[j] - ref;
            const float vv = vc[j];
            if (STORE) {
                const float uk = uc + kr;
                const float d = st.p - uk;
                const float e = expn(-fabsf(d));
                const bool sp = d >= 0.0f;
                const float e1 = sp ? 1.0f : e;
                const float e2 = sp ? e : 1.0f;
                const float den = fmaf(e1, st.b, e2);
                kc[j] = kr;
                yc[j] = fmaf(e1, st.a, e2 * vv) / den;
                gc[j] = gc[j] / den;
                yc[(j + H) % CH] = sp ? st.p : uk;
            }
            rs_push(st, kr, vv, dc);
        }
    }
}

template <int CH, int J0, int J1, bool OUT>
__device__ __forceinline__ void exact_rev_steps(const float (&kc)[CH], const float (&vc)[CH],
                                                const float (&gc)[CH], const float (&yc)[CH],
                                                int Lv, float uc, const Decay &dc, RevState &rs,
                                                rsrc_t rdk, rsrc_t rdv, int voff, int stride,
                                                bool st_ok, float &du_acc, float &dw_acc) {
    constexpr int H = CH / 2;
#pragma unroll
    for (int j = J1 - 1; j >= J0; --j) {
        if (j < Lv) {
            const float kr = kc[j], vv = vc[j], yy = yc[j], sg = gc[j];
            const float M = yc[(j + H) % CH];
            if (OUT) {
                const float ekr = expn(kr + rs.r);
                const float cpi = sg * expn(uc + kr - M);
                const float dd = vv - yy;
                if (st_ok) {
                    bstore(rdv, fmaf(ekr, rs.g, cpi), voff, j * stride);
                    bstore(rdk, fmaf(cpi, dd, ekr * fmaf(vv, rs.g, -rs.h)), voff, j * stride);
                }
                du_acc = fmaf(cpi, dd, du_acc);
                dw_acc = fmaf(ekr, fmaf(vv, rs.gp, -rs.hp), dw_acc);
            }
            const float a = rs.r - dc.w;
            const float b = -M;
            const float e = expn(-fabsf(a - b));
            const bool keep = a >= b;
            const float fa = keep ? 1.0f : e;
            const float fb = keep ? e : 1.0f;
            rs.gp = (rs.gp + rs.g) * fa;
            rs.hp = (rs.hp + rs.h) * fa;
            rs.g = fmaf(rs.g, fa, sg * fb);
            rs.h = fmaf(rs.h, fa, sg * yy * fb);
            rs.r = keep ? a : b;
        } else {
            rs.gp = rs.gp + rs.g;  // a padded token past T: pure decay (its s is 0)
            rs.hp = rs.hp + rs.h;
            rs.r -= dc.w;
        }
    }
}

template <int CH, bool OUT>
__device__ RevCarry exact_chunk_bwd(float (&kc)[CH], float (&vc)[CH], float (&gc)[CH],
                                    float (&yc)[CH], int Lv, float ref, const Carry &fin,
                                    const RevCarry &rin, float uc, const Decay &dc, rsrc_t rdk,
                                    rsrc_t rdv, int voff, int stride, bool st_ok, float &du_acc,
                                    float &dw_acc) {
    constexpr int H = CH / 2;
    const double ref2 = (double)(ref * kLog2e);
    const Rs st0{fin.a, fin.b, (float)((fin.P - ref2) * kLn2D)};
    RevState rs{rin.g, rin.h, rin.gp, rin.hp, (float)((rin.r + ref2) * kLn2D)};
    // second half: forward to the middle, then forward over the half keeping its tokens
    {
        Rs st = st0;
        exact_fwd_steps<CH, 0, H, false>(kc, vc, gc, yc, Lv, ref, uc, dc, st);
        exact_fwd_steps<CH, H, CH, true>(kc, vc, gc, yc, Lv, ref, uc, dc, st);
        exact_rev_steps<CH, H, CH, OUT>(kc, vc, gc, yc, Lv, uc, dc, rs, rdk, rdv, voff, stride,
                                        st_ok, du_acc, dw_acc);
    }
    // first half
    {
        Rs st = st0;
        exact_fwd_steps<CH, 0, H, true>(kc, vc, gc, yc, Lv, ref, uc, dc, st);
        exact_rev_steps<CH, 0, H, OUT>(kc, vc, gc, yc, Lv, uc, dc, rs, rdk, rdv, voff, stride,
                                       st_ok, du_acc, dw_acc);
    }
    return RevCarry{rs.g, rs.h, rs.gp, rs.hp, (double)rs.r * kLog2eD - ref2};
}

// LDS staging shared by the waves of a backward unit (forward summaries use a, b, r).
template <int NW>
struct BwdShared {
    float a[NW][64];
    float b[NW][64];
    float c[NW][64];
    float d[NW][64];
    double r[NW][64];
    int status[2];
};

// Everything a unit needs about one lane's chunk of window jw, up to its reverse summary:
// the forward recomputation (F1/F3) and the reverse summary from a zero future (R1).
// Called by all waves of the workgroup together (it contains a barrier; the caller makes
// sure nobody still reads the staging arrays). On return with exact == false, kc, vc, gc,
// yc hold e_j, v_j, sigma_j, y_j; with exact == true they are clobbered and the chunk must
// take the per-token path again from raw data. Deterministic: the owner of a window and
// a helper recomputing it get identical bits.
template <int NW, int CH>
__device__ __forceinline__ RevCarry chunk_pass(
    BwdShared<NW> &sh, int64_t jw, int q, int lane, int64_t T, int64_t C, int64_t nseg,
    int64_t bidx, int64_t row0, int cl, int voff, int stride, const float *__restrict__ k,
    const float *__restrict__ v, const float *__restrict__ dy, const Rec *__restrict__ fincl,
    const Decay &dc, float uc, float eu, double w2, bool slow_wave, float (&kc)[CH],
    float (&vc)[CH], float (&gc)[CH], float (&yc)[CH], bool &exact, Carry &mine, float &ref,
    int &Lv) {
    const int64_t t0 = jw * (int64_t)(NW * CH) + (int64_t)q * CH;
    Lv = chunk_len(t0, T, CH);
    load_chunk<CH>(kc, vc, k, v, row0, t0, T, C, voff);
    load_chunk1<CH>(gc, dy, row0, t0, T, C, voff);

    // F1: forward summary of the chunk, and the carry entering it
    ref = chunk_ref<CH>(kc, Lv);
    const float ref2 = ref * kLog2e;
    float S, Z;
    double sc;
    exact = chunk_summary<CH, true>(kc, vc, Lv, ref, slow_wave, dc, S, Z, sc);
    if (exact) {
        load_chunk<CH>(kc, vc, k, v, row0, t0, T, C, voff);
        exact_summary<CH>(kc, vc, Lv, ref, dc, S, Z, sc);
    }
    sh.a[q][lane] = S;
    sh.b[q][lane] = Z;
    sh.r[q][lane] = sc;
    __syncthreads();
    mine = Carry{0.0f, 0.0f, kNegBigD};
    if (jw > 0) {
        const Rec *fr = fincl + (bidx * nseg + (jw - 1)) * C + cl;
        mine.a = lo32(fr->ab);
        mine.b = hi32(fr->ab);
        mine.P = __builtin_bit_cast(double, fr->P);
    }
    for (int qq = 0; qq < q; ++qq)
        fold(mine, sh.a[qq][lane], sh.b[qq][lane], sh.r[qq][lane], (double)CH * w2);
    normalize(mine);

    // F3: y and sigma = dy / den in the chunk frame
    if (!exact) {
        const float gap = (float)(mine.P - (double)ref2);
        bool bad = gap > kCarryGap;
        const float s0 = ex2(gap);
        float Sx = mine.a * s0, Zx = mine.b * s0;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const float e = kc[j];
            const float ev = e * vc[j];
            const float num = fmaf(eu, ev, Sx);
            const float den = fmaf(eu, e, Zx);
            const float r = rcpf(den);
            if (j < Lv) {
                bad |= !(den >= kTinyDen);
                yc[j] = num * r;
                gc[j] = gc[j] * r;
            } else {
                yc[j] = 0.0f;
                gc[j] = 0.0f;
            }
            Sx = fmaf(Sx, dc.dwf, ev);
            Zx = fmaf(Zx, dc.dwf, e);
        }
        exact = wave_any(bad);
    }

    // R1: reverse summary of the chunk from a zero future
    if (!exact) {
        const float dwf = dc.dwf;
        float R = 0.f, Q = 0.f, X = 0.f, Y = 0.f;
#pragma unroll
        for (int j = CH - 1; j >= 0; --j) {
            X = dwf * (X + R);
            Y = dwf * (Y + Q);
            R = fmaf(R, dwf, gc[j]);
            Q = fmaf(Q, dwf, gc[j] * yc[j]);
        }
        return RevCarry{R, Q, X, Y, -(double)ref2};
    }
    load_chunk<CH>(kc, vc, k, v, row0, t0, T, C, voff);
    load_chunk1<CH>(gc, dy, row0, t0, T, C, voff);
    float d0 = 0.f, d1 = 0.f;
    const rsrc_t none = make_rsrc(dy);
    return exact_chunk_bwd<CH, false>(kc, vc, gc, yc, Lv, ref, mine, rev_zero(), uc, dc, none,
                                      none, voff, stride, false, d0, d1);
}

// Stage this wave's chunk reverse summary and fold the window's NW summaries (last chunk
// first) from a zero future: `agg` is the window's reverse aggregate, `lfut` the part of it
// that lies after this wave's chunk. Contains barriers (all waves call it together).
template <int NW, int CH>
__device__ __forceinline__ void window_rev_fold(BwdShared<NW> &sh, const RevCarry &rsum, int q,
                                                int lane, double w2, RevCarry &agg,
                                                RevCarry &lfut) {
    __syncthreads();
    sh.a[q][lane] = rsum.g;
    sh.b[q][lane] = rsum.h;
    sh.c[q][lane] = rsum.gp;
    sh.d[q][lane] = rsum.hp;
    sh.r[q][lane] = rsum.r;
    __syncthreads();
    agg = rev_zero();
    lfut = agg;
#pragma unroll
    for (int qq = NW - 1; qq >= 0; --qq) {
        if (qq == q) lfut = agg;
        const RevCarry sm{sh.a[qq][lane], sh.b[qq][lane], sh.c[qq][lane], sh.d[qq][lane],
                          sh.r[qq][lane]};
        rfold(agg, sm, (double)CH * w2, (float)CH);
    }
}

template <int NW, int CH>
__global__ __launch_bounds__(NW * 64) void wkv_backward_kernel(
    int64_t T, int64_t C, int ngrp, int64_t nbg, int64_t nseg, uint64_t epoch,
    const float *__restrict__ w, const float *__restrict__ u, const float *__restrict__ k,
    const float *__restrict__ v, const float *__restrict__ dy, const Rec *__restrict__ fincl,
    float *__restrict__ dk, float *__restrict__ dv, uint64_t *__restrict__ flags,
    RevRec *__restrict__ ragg, RevRec *__restrict__ rincl, double *__restrict__ part) {
    constexpr int WIN = NW * CH;
    static_assert(WIN == kFwdWindow, "backward windows must match the forward's carries");
    __shared__ BwdShared<NW> sh;

    const int lane = threadIdx.x & 63;
    const int q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t sidx = (int64_t)blockIdx.x / nbg;
    const int64_t s = nseg - 1 - sidx;
    const int64_t bg = (int64_t)blockIdx.x - sidx * nbg;
    const int64_t bidx = bg / ngrp;
    const int grp = (int)(bg - bidx * ngrp);
    const int64_t c = (int64_t)grp * 64 + lane;
    const bool cval = c < C;
    const int cl = (int)(cval ? c : C - 1);
    const int voff = cl * 4;
    const int stride = (int)(C * 4);

    const float wc = w[cl];
    const float uc = u[cl];
    const Decay dc = make_decay(wc);
    const float dwf = dc.dwf;
    const float eu = expf(uc);
    const double w2 = (double)wc * kLog2eD;
    const bool slow_wave = wave_any(!(fabsf(uc) <= 60.0f));
    const int64_t row0 = bidx * T;
    const int64_t t0 = s * WIN + (int64_t)q * CH;

    float kc[CH], vc[CH], gc[CH], yc[CH];
    bool exact;
    Carry mine;
    float ref;
    int Lv;
    RevCarry rsum = chunk_pass<NW, CH>(sh, s, q, lane, T, C, nseg, bidx, row0, cl, voff, stride,
                                       k, v, dy, fincl, dc, uc, eu, w2, slow_wave, kc, vc, gc,
                                       yc, exact, mine, ref, Lv);
    RevCarry agg, lfut;
    window_rev_fold<NW, CH>(sh, rsum, q, lane, w2, agg, lfut);
    const int64_t rec = (bidx * nseg + s) * C + cl;
    uint64_t *myflag = flags + sidx * nbg + bg;
    if (q == 0) {
        if (cval) put_rrec(ragg + rec, agg);
        put_flag(myflag, epoch, kAggregate);
    }

    // ---- look-back toward later windows: future sums at this window's end ----
    // Walk forward in time to the nearest window whose inclusive future sums are
    // published (or past the sequence end), making sure every window in between has its
    // reverse aggregate in memory, then fold those back in order: bitwise the sequential
    // chain rincl[s] = rfold(rincl[s+1], ragg[s]) whatever the timing.
    RevCarry fut = rev_zero();
    if (s < nseg - 1) {
        int64_t j = s + 1;
        int it = 0;
        bool redo_own = false;
        for (;;) {
            if (q == 0) {
                const int st = poll_flag(flags + (nseg - 1 - j) * nbg + bg, epoch, kPollTries);
                if (lane == 0) sh.status[it & 1] = st;
            }
            __syncthreads();
            const int st = sh.status[it & 1];
            ++it;
            if (st == (int)kInclusive) break;
            if (st != (int)kAggregate) {
                // not published in time: recompute window j's reverse aggregate here and
                // publish it (bitwise what unit j itself publishes)
                bool ex_j;
                Carry m_j;
                float r_j;
                int L_j;
                const RevCarry rs_j = chunk_pass<NW, CH>(
                    sh, j, q, lane, T, C, nseg, bidx, row0, cl, voff, stride, k, v, dy, fincl,
                    dc, uc, eu, w2, slow_wave, kc, vc, gc, yc, ex_j, m_j, r_j, L_j);
                RevCarry agg_j, lf_j;
                window_rev_fold<NW, CH>(sh, rs_j, q, lane, w2, agg_j, lf_j);
                if (q == 0) {
                    if (cval) put_rrec(ragg + (bidx * nseg + j) * C + cl, agg_j);
                    raise_flag(flags + (nseg - 1 - j) * nbg + bg, epoch, kAggregate);
                }
                __syncthreads();
                redo_own = true;
            }
            if (j == nseg - 1) {
                j = nseg;
                break;
            }
            ++j;
        }
        if (j < nseg) fut = get_rrec(rincl + (bidx * nseg + j) * C + cl);
        for (int64_t m = j - 1; m > s; --m)
            fut = rfollow(fut, get_rrec(ragg + (bidx * nseg + m) * C + cl), (double)WIN * w2,
                          (float)WIN);
        if (redo_own) {
            __syncthreads();
            chunk_pass<NW, CH>(sh, s, q, lane, T, C, nseg, bidx, row0, cl, voff, stride, k, v,
                               dy, fincl, dc, uc, eu, w2, slow_wave, kc, vc, gc, yc, exact,
                               mine, ref, Lv);
        }
    }
    if (q == 0) {
        if (cval) put_rrec(rincl + rec, rfollow(fut, agg, (double)WIN * w2, (float)WIN));
        put_flag(myflag, epoch, kInclusive);
    }

    // ---- R3: gradients of this chunk ----
    const rsrc_t rdk = make_rsrc(dk + (row0 + (t0 < T ? t0 : 0)) * C);
    const rsrc_t rdv = make_rsrc(dv + (row0 + (t0 < T ? t0 : 0)) * C);
    float du_acc = 0.0f, dw_acc = 0.0f;
    RevCarry rc = rfollow(fut, lfut, (double)((NW - 1 - q) * CH) * w2, (float)((NW - 1 - q) * CH));
    rnormalize(rc);
    const float ref2 = ref * kLog2e;
    const float rgap = (float)((double)ref2 + rc.r);
    if (!exact) exact = wave_any(rgap > kCarryGap);
    if (!exact) {
        const float fr = ex2(rgap);
        float R = rc.g * fr, Q = rc.h * fr, X = rc.gp * fr, Y = rc.hp * fr;
#pragma unroll
        for (int j = CH - 1; j >= 0; --j) {
            const float e = kc[j], vv = vc[j], sg = gc[j], yy = yc[j];
            const float cs = eu * sg;
            const float t1 = cs * (vv - yy);
            const float dvj = e * (cs + R);
            const float dkj = e * (t1 + fmaf(vv, R, -Q));
            du_acc = fmaf(t1, e, du_acc);
            dw_acc = fmaf(e, fmaf(vv, X, -Y), dw_acc);
            if (j < Lv && cval) {
                bstore(rdv, dvj, voff, j * stride);
                bstore(rdk, dkj, voff, j * stride);
            }
            X = dwf * (X + R);
            Y = dwf * (Y + Q);
            R = fmaf(R, dwf, sg);
            Q = fmaf(Q, dwf, sg * yy);
        }
    } else {
        load_chunk<CH>(kc, vc, k, v, row0, t0, T, C, voff);
        load_chunk1<CH>(gc, dy, row0, t0, T, C, voff);
        exact_chunk_bwd<CH, true>(kc, vc, gc, yc, Lv, ref, mine, rc, uc, dc, rdk, rdv, voff,
                                  stride, cval, du_acc, dw_acc);
    }

    // ---- dw, du partials of this window, summed over its chunks in a fixed order ----
    __syncthreads();
    sh.r[q][lane] = (double)du_acc;
    __syncthreads();
    if (q == 0) {
        double su = 0.0;
        for (int qq = 0; qq < NW; ++qq) su += sh.r[qq][lane];
        if (cval) part[rec * 2 + 1] = su;
    }
    __syncthreads();
    sh.r[q][lane] = -(double)dw_acc;
    __syncthreads();
    if (q == 0) {
        double sw = 0.0;
        for (int qq = 0; qq < NW; ++qq) sw += sh.r[qq][lane];
        if (cval) part[rec * 2] = sw;
    }
}

// dw[c], du[c] = sums of the per-window partials over b and windows, in a fixed order.
__global__ __launch_bounds__(256) void wkv_reduce_kernel(int64_t n_bs, int64_t C,
                                                         const double *__restrict__ part,
                                                         float *__restrict__ dw,
                                                         float *__restrict__ du) {
    const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (c >= C) return;
    double sw = 0.0, su = 0.0;
    for (int64_t i = 0; i < n_bs; ++i) {
        sw += part[(i * C + c) * 2];
        su += part[(i * C + c) * 2 + 1];
    }
    dw[c] = (float)sw;
    du[c] = (float)su;
}

__global__ __launch_bounds__(256) void wkv_zero2_kernel(float *__restrict__ a,
                                                        float *__restrict__ b, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) {
        a[i] = 0.0f;
        b[i] = 0.0f;
    }
}

hipError_t launch_backward(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                           const float *k, const float *v, const float *dy, const Rec *fincl,
                           float *dk, float *dv, float *dw, float *du, const BwdLayout &L,
                           uint64_t epoch, hipStream_t stream) {
    const int ngrp = (int)((C + 63) / 64);
    const int64_t nbg = B * ngrp;
    const int64_t units = nbg * L.nseg;
    hipLaunchKernelGGL((wkv_backward_kernel<kFwdWaves, kFwdChunk>), dim3((unsigned)units),
                       dim3(kFwdWaves * 64), 0, stream, T, C, ngrp, nbg, L.nseg, epoch, w, u,
                       k, v, dy, fincl, dk, dv, L.flags, L.ragg, L.rincl, L.part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(wkv_reduce_kernel, dim3((unsigned)((C + 255) / 256)), dim3(256), 0,
                       stream, B * L.nseg, C, L.part, dw, du);
    return hipGetLastError();
}

hipError_t launch_zero2(float *dw, float *du, int64_t C, hipStream_t stream) {
    hipLaunchKernelGGL(wkv_zero2_kernel, dim3((unsigned)((C + 255) / 256)), dim3(256), 0, stream,
                       dw, du, C);
    return hipGetLastError();
}

}  // namespace wkvdev
