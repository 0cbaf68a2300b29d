// wkv_backward.hip -- WKV backward on gfx950: dk, dv, dw, du of L = sum dy * y.
//
// Gradients of the operator of "RWKV解读：在Transformer的时代的新RNN", section 二.3,
// formula (8); "RWKV についての調査記録", section "Trainingについて" (all parameters are
// trained by gradient descent, w and u being per-channel vectors).
//
// With D_t the denominator of y_t, s_t = dy_t / D_t, the past sums A_t, B_t of the
// recursive form and their age-weighted versions A'_t = sum_{i<t} (t-1-i) e^{-(t-1-i)w+k_i}
// v_i, B'_t likewise (dA_t/dw = -A'_t), and the future sums
//   G_i = sum_{t>i} e^{-(t-1-i)w} s_t,   H_i = same with s_t y_t,
// the gradients are
//   dv_i = s_i e^{u+k_i} + e^{k_i} G_i
//   dk_i = s_i e^{u+k_i} (v_i - y_i) + e^{k_i} (v_i G_i - H_i)
//   du   = sum_t s_t e^{u+k_t} (v_t - y_t)
//   dw   = -sum_t s_t (A'_t - y_t B'_t)
// (the O(T^2) softmax form gives the same sums term by term). dw and du are thus sums over
// the forward direction, formed where y_t and D_t are computed; only dk and dv need the
// future sums.
//
// Work decomposition as in the forward (64 channels x one 256-token window per workgroup,
// one CH-token chunk per wave), with units numbered from the last window backwards so that
// the future of a unit was launched first. Each unit reads k, v, dy once and writes dk, dv
// once: 20 bytes per element. The forward state entering the window (with A', B') is read
// from the forward's workspace, so no extra pass over k and v is needed.
//
// Per chunk, in the forward pass's chunk frame (ref = max k, e_j = e^{k_j - ref}):
//   F1     forward summary of the chunk (fp64, as the forward computes it); the window's
//          summaries are folded through LDS into the carry entering each chunk.
//   F3     y_j, den_j, sigma_j = dy_j / den_j (s_t in the frame) and the dw, du terms,
//          all in fp64 from fp64 weights e_j: dw is a sum over B*T tokens whose terms
//          cancel by factors of 10^4 on some channels (and its per-sequence parts cancel
//          again over the batch), so any fp32 rounding of e_j, y_j or sigma_j inside it
//          shows up. e_j, y_j, sigma_j are then kept in fp32 for dk, dv.
//   R1     reverse summary of the chunk from a zero future, by Horner from the chunk end:
//          R_{j-1} = e^{-w} R_j + sigma_j, Q likewise with sigma_j y_j (fp64).
//   scan   reverse summaries are folded through LDS and across windows (decoupled
//          look-back toward later windows) into the future sums at each chunk's end.
//   R3     the same recursion from the incoming future sums gives, per token,
//          e^{k_i} G_i = e_i R_i and e^{k_i} H_i = e_i Q_i, hence dv and dk.
// Chunks whose frame would under- or overflow are redone with a per-token rescaled
// recursion in fp64 (exact_chunk).
#include "wkv_chunk.h"

namespace wkvdev {

// Future sums (G, H) = (g, h) 2^r.
struct RevCarry {
    double g, h;
    double r;
};

__device__ __forceinline__ RevCarry rev_zero() { return RevCarry{0.0, 0.0, kNegBigD}; }

// c <- the future seen from `len` tokens earlier (len_w2 = len w log2 e), where `sum`
// summarizes those tokens from a zero future and c was the future beyond them:
//   G <- e^{-len w} G + sum.G   (H alike).
__device__ __forceinline__ void rfold(RevCarry &c, const RevCarry &sum, double len_w2) {
    const double rd = c.r - len_w2;
    const double d = sum.r - rd;
    const double f = exp2_64(-fabs(d));
    const bool up = d >= 0.0;
    const double ca = up ? f : 1.0;
    const double cs = up ? 1.0 : f;
    c.g = fma(c.g, ca, sum.g * cs);
    c.h = fma(c.h, ca, sum.h * cs);
    c.r = up ? sum.r : rd;
}

__device__ __forceinline__ RevCarry rfollow(RevCarry c, const RevCarry &sum, double len_w2) {
    rfold(c, sum, len_w2);
    return c;
}

// Rescale so that the larger |mantissa| lies in [1, 2) (exact), making r the magnitude.
__device__ __forceinline__ void rnormalize(RevCarry &c) {
    const double m = fmax(fabs(c.g), fabs(c.h));
    if (m > 0.0 && m <= 1.0e300) {
        const int e = __builtin_amdgcn_frexp_exp(m) - 1;
        c.g = ldexp(c.g, -e);
        c.h = ldexp(c.h, -e);
        c.r += (double)e;
    }
}

__device__ __forceinline__ void put_rrec(RevRec *p, const RevCarry &c) {
    put_u64(&p->g, c.g);
    put_u64(&p->h, c.h);
    put_u64(&p->r, c.r);
}
__device__ __forceinline__ RevCarry get_rrec(const RevRec *p) {
    return RevCarry{get_u64(&p->g), get_u64(&p->h), get_u64(&p->r)};
}

// ---------------------------------------------------------------------------------
// Exact per-token backward of one lane's chunk (tokens [0, Lv)), for chunks whose fixed
// frame would under- or overflow (a dominant key next to much smaller ones, extreme u).
// Everything is fp64 with library exponentials. On entry kc, vc, gc hold the raw k, v,
// dy; gc and yc are clobbered. `fin` is the forward carry entering the chunk, `rin` the
// future sums at the chunk's nominal end. The chunk is swept in quarters from the last
// one: for each quarter the forward recursion is rerun from `fin` (adding the dw, du
// terms of the quarter's tokens if FG) and that quarter's per-token y and log-scale of D
// (each as a float pair, about 48 bits) and dy / den are kept in yc and gc; then the
// quarter is swept backwards (storing dk, dv if OUT). Returns the future sums at the
// chunk start.
// ---------------------------------------------------------------------------------
struct RevState64 {  // (G, H) = (g, h) e^{r - ref}
    double g, h, r;
};

template <int CH, int QS, bool OUT, bool FG>
__device__ __forceinline__ void exact_quarter(const float (&kc)[CH], const float (&vc)[CH],
                                              float (&gc)[CH], float (&yc)[CH], int Lv,
                                              double ref, double uc, double wc,
                                              const Rs64 &st0, RevState64 &rs, rsrc_t rdk,
                                              rsrc_t rdv, int voff, int stride, bool st_ok,
                                              double &du_acc, double &dw_acc) {
    constexpr int Q = CH / 4;  // tokens per quarter
    constexpr int J0 = QS * Q;
    static_assert(4 * Q <= CH, "yc holds y and M of one quarter, each as a float pair");
    Rs64 st = st0;
#pragma unroll
    for (int j = 0; j < J0; ++j)
        if (j < Lv) rs64_push(st, (double)kc[j] - ref, (double)vc[j], wc);
#pragma unroll
    for (int j = J0; j < J0 + Q; ++j) {
        if (j < Lv) {
            const double kr = (double)kc[j] - ref, vv = (double)vc[j];
            const double uk = uc + kr;
            const double m = fmax(st.p, uk);
            const double e1 = exp(st.p - m), e2 = exp(uk - m);
            const double rden = 1.0 / fma(e1, st.b, e2);
            const double yv = fma(e1, st.a, e2 * vv) * rden;
            const double sg = (double)gc[j] * rden;  // dy / D in units of e^{-(m + ref)}
            if (FG) {
                // s (A' - y B') and s e^{u+k} (v - y), with A' = a' e^{p+ref}
                dw_acc = fma(sg * e1, fma(-yv, st.bp, st.ap), dw_acc);
                du_acc = fma(sg * e2, vv - yv, du_acc);
            }
            const float yh = (float)yv;
            yc[j - J0] = yh;
            yc[3 * Q + j - J0] = (float)(yv - (double)yh);
            gc[j] = (float)sg;
            const float mh = (float)m;
            yc[Q + j - J0] = mh;
            yc[2 * Q + j - J0] = (float)(m - (double)mh);
            rs64_push(st, kr, vv, wc);
        }
    }
#pragma unroll
    for (int j = J0 + Q - 1; j >= J0; --j) {
        if (j < Lv) {
            const double kr = (double)kc[j] - ref, vv = (double)vc[j];
            const double yy = (double)yc[j - J0] + (double)yc[3 * Q + j - J0];
            const double sg = (double)gc[j];
            const double M = (double)yc[Q + j - J0] + (double)yc[2 * Q + j - J0];
            if (OUT) {
                const double ekr = exp(kr + rs.r);
                const double cpi = sg * exp(uc + kr - M);
                if (st_ok) {
                    bstore(rdv, (float)fma(ekr, rs.g, cpi), voff, j * stride);
                    bstore(rdk, (float)fma(cpi, vv - yy, ekr * fma(vv, rs.g, -rs.h)), voff,
                           j * stride);
                }
            }
            const double a = rs.r - wc, b = -M;
            const double rn = fmax(a, b);
            const double fa = exp(a - rn), fb = exp(b - rn);
            rs.g = fma(rs.g, fa, sg * fb);
            rs.h = fma(rs.h, fa, sg * yy * fb);
            rs.r = rn;
        } else {
            rs.r -= wc;  // a padded token past T: pure decay (its s is 0)
        }
    }
}

template <int CH, bool OUT, bool FG>
__device__ RevCarry exact_chunk(const float (&kc)[CH], const float (&vc)[CH], float (&gc)[CH],
                                float (&yc)[CH], int Lv, float ref, const Carry &fin,
                                RevCarry rin, float uc, float wc, rsrc_t rdk, rsrc_t rdv,
                                int voff, int stride, bool st_ok, double &du_acc,
                                double &dw_acc) {
    const double refd = (double)ref;
    const double ref2 = refd * kLog2eD;  // the frame 2^{ref2} the carries refer to
    rnormalize(rin);
    // the carries are relative to 2^{ref2}; the per-token path works relative to e^{ref}
    const double shift = ref2 * kLn2D - refd;
    const Rs64 st0{fin.a, fin.b, fin.ap, fin.bp, (fin.P - ref2) * kLn2D + shift};
    RevState64 rs{rin.g, rin.h, (rin.r + ref2) * kLn2D - shift};
    const double u = (double)uc, w = (double)wc;
    exact_quarter<CH, 3, OUT, FG>(kc, vc, gc, yc, Lv, refd, u, w, st0, rs, rdk, rdv, voff,
                                  stride, st_ok, du_acc, dw_acc);
    exact_quarter<CH, 2, OUT, FG>(kc, vc, gc, yc, Lv, refd, u, w, st0, rs, rdk, rdv, voff,
                                  stride, st_ok, du_acc, dw_acc);
    exact_quarter<CH, 1, OUT, FG>(kc, vc, gc, yc, Lv, refd, u, w, st0, rs, rdk, rdv, voff,
                                  stride, st_ok, du_acc, dw_acc);
    exact_quarter<CH, 0, OUT, FG>(kc, vc, gc, yc, Lv, refd, u, w, st0, rs, rdk, rdv, voff,
                                  stride, st_ok, du_acc, dw_acc);
    // G = g e^{r - ref} at the chunk start
    return RevCarry{rs.g, rs.h, (rs.r - refd) * kLog2eD};
}

// LDS staging shared by the waves of a backward unit (forward summaries use all five
// arrays, reverse summaries three, the dw, du partials two).
template <int NW>
struct BwdShared {
    double a[NW][64];
    double b[NW][64];
    double c[NW][64];
    double d[NW][64];
    double r[NW][64];
    int status[2];
};

// Per-channel constants of a backward lane.
struct BwdConst {
    double w;       // the decay rate
    double dwf;     // e^{-w}
    double eu;      // e^{u}
    double w2;      // w log2 e
    float uc;
    bool slow_wave; // some lane has |u| > 60: exact path throughout
};

// Everything a unit needs about one lane's chunk of window jw, up to its reverse summary:
// the forward recomputation with the chunk's dw, du terms (F1/F3) and the reverse summary
// from a zero future (R1). Called by all waves of the workgroup together (it contains a
// barrier; the caller makes sure nobody still reads the staging arrays). On return with
// fx == false, kc, vc, gc, yc hold e_j, v_j, sigma_j, y_j; with fx == true (the forward
// frame failed) they are clobbered and the chunk must take the per-token path again from
// raw data. Deterministic: the owner of a window and a helper recomputing it get identical
// bits.
template <int NW, int CH>
__device__ __forceinline__ RevCarry chunk_pass(
    BwdShared<NW> &sh, int64_t jw, int q, int lane, int64_t T, int64_t C, int64_t nseg,
    int64_t bidx, int64_t row0, int cl, int voff, int stride, const float *__restrict__ k,
    const float *__restrict__ v, const float *__restrict__ dy, const Rec *__restrict__ fincl,
    const BwdConst &K, float (&kc)[CH], float (&vc)[CH], float (&gc)[CH], float (&yc)[CH],
    bool &fx, Carry &mine, float &ref, int &Lv, double &du_acc, double &dw_acc) {
    const int64_t t0 = jw * (int64_t)(NW * CH) + (int64_t)q * CH;
    Lv = chunk_len(t0, T, CH);
    load_chunk<CH>(kc, vc, k, v, row0, t0, T, C, voff);
    load_chunk1<CH>(gc, dy, row0, t0, T, C, voff);

    // F1: forward summary of the chunk, and the carry entering it
    ref = chunk_ref<CH>(kc, Lv);
    const double refd = (double)ref;
    const double ref2 = refd * kLog2eD;
    Carry sum;
    fx = chunk_summary<CH, true>(kc, vc, Lv, ref, K.slow_wave, K.dwf, sum);
    if (fx) exact_summary<CH>(kc, vc, Lv, ref, K.w, sum);
    sh.a[q][lane] = sum.a;
    sh.b[q][lane] = sum.b;
    sh.c[q][lane] = sum.ap;
    sh.d[q][lane] = sum.bp;
    sh.r[q][lane] = sum.P;
    __syncthreads();
    mine = carry_empty();
    if (jw > 0) mine = get_rec(fincl + (bidx * nseg + (jw - 1)) * C + cl);
    for (int qq = 0; qq < q; ++qq)
        fold(mine, Carry{sh.a[qq][lane], sh.b[qq][lane], sh.c[qq][lane], sh.d[qq][lane],
                         sh.r[qq][lane]},
             (double)CH * K.w2, (double)CH);
    normalize(mine);

    // F3: y, sigma = dy / den and the dw, du terms in the chunk frame (fp64)
    du_acc = 0.0;
    dw_acc = 0.0;
    if (!fx) {
        const double gap = mine.P - ref2;
        bool bad = gap > (double)kCarryGap;
        const double s0 = exp2_64(gap);
        double Sx = mine.a * s0, Zx = mine.b * s0, Spx = mine.ap * s0, Zpx = mine.bp * s0;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const double e = (j < Lv) ? exp2_64(((double)kc[j] - refd) * kLog2eD) : 0.0;
            const double vv = (double)vc[j];
            const double ev = e * vv;
            const double num = fma(K.eu, ev, Sx);
            const double den = fma(K.eu, e, Zx);
            if (j < Lv) {
                bad |= !(den >= (double)kTinyDen);
                const double r = rcpd(den);
                const double yv = num * r;
                const double sg = (double)gc[j] * r;
                dw_acc = fma(sg, fma(-yv, Zpx, Spx), dw_acc);
                du_acc = fma(sg * (K.eu * e), vv - yv, du_acc);
                kc[j] = (float)e;
                yc[j] = (float)yv;
                gc[j] = (float)sg;
            } else {
                kc[j] = 0.0f;
                yc[j] = 0.0f;
                gc[j] = 0.0f;
            }
            Spx = K.dwf * (Spx + Sx);
            Zpx = K.dwf * (Zpx + Zx);
            Sx = fma(Sx, K.dwf, ev);
            Zx = fma(Zx, K.dwf, e);
        }
        fx = wave_any(bad);
    }

    // R1: reverse summary of the chunk from a zero future
    if (!fx) {
        double R = 0.0, Q = 0.0;
#pragma unroll
        for (int j = CH - 1; j >= 0; --j) {
            const double sg = (double)gc[j];
            R = fma(R, K.dwf, sg);
            Q = fma(Q, K.dwf, sg * (double)yc[j]);
        }
        return RevCarry{R, Q, -ref2};
    }
    load_chunk<CH>(kc, vc, k, v, row0, t0, T, C, voff);
    load_chunk1<CH>(gc, dy, row0, t0, T, C, voff);
    du_acc = 0.0;
    dw_acc = 0.0;
    const rsrc_t none = make_rsrc(dy);
    return exact_chunk<CH, false, true>(kc, vc, gc, yc, Lv, ref, mine, rev_zero(), K.uc,
                                        (float)K.w, none, none, voff, stride, false, du_acc,
                                        dw_acc);
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
    sh.r[q][lane] = rsum.r;
    __syncthreads();
    agg = rev_zero();
    lfut = agg;
#pragma unroll
    for (int qq = NW - 1; qq >= 0; --qq) {
        if (qq == q) lfut = agg;
        rfold(agg, RevCarry{sh.a[qq][lane], sh.b[qq][lane], sh.r[qq][lane]}, (double)CH * w2);
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
    BwdConst K;
    K.uc = u[cl];
    K.w = (double)wc;
    K.dwf = exp(-K.w);
    K.eu = exp((double)K.uc);
    K.w2 = K.w * kLog2eD;
    K.slow_wave = wave_any(!(fabsf(K.uc) <= 60.0f));
    const int64_t row0 = bidx * T;
    const int64_t t0 = s * WIN + (int64_t)q * CH;

    float kc[CH], vc[CH], gc[CH], yc[CH];
    bool fx;
    Carry mine;
    float ref;
    int Lv;
    double du_acc, dw_acc;
    RevCarry rsum = chunk_pass<NW, CH>(sh, s, q, lane, T, C, nseg, bidx, row0, cl, voff, stride,
                                       k, v, dy, fincl, K, kc, vc, gc, yc, fx, mine, ref, Lv,
                                       du_acc, dw_acc);
    RevCarry agg, lfut;
    window_rev_fold<NW, CH>(sh, rsum, q, lane, K.w2, agg, lfut);
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
                bool fx_j;
                Carry m_j;
                float r_j;
                int L_j;
                double du_j, dw_j;
                const RevCarry rs_j = chunk_pass<NW, CH>(
                    sh, j, q, lane, T, C, nseg, bidx, row0, cl, voff, stride, k, v, dy, fincl,
                    K, kc, vc, gc, yc, fx_j, m_j, r_j, L_j, du_j, dw_j);
                RevCarry agg_j, lf_j;
                window_rev_fold<NW, CH>(sh, rs_j, q, lane, K.w2, agg_j, lf_j);
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
            fut = rfollow(fut, get_rrec(ragg + (bidx * nseg + m) * C + cl), (double)WIN * K.w2);
        if (redo_own) {
            __syncthreads();
            chunk_pass<NW, CH>(sh, s, q, lane, T, C, nseg, bidx, row0, cl, voff, stride, k, v,
                               dy, fincl, K, kc, vc, gc, yc, fx, mine, ref, Lv, du_acc, dw_acc);
        }
    }
    if (q == 0) {
        if (cval) put_rrec(rincl + rec, rfollow(fut, agg, (double)WIN * K.w2));
        put_flag(myflag, epoch, kInclusive);
    }

    // ---- R3: dk, dv of this chunk ----
    const rsrc_t rdk = make_rsrc(dk + (row0 + (t0 < T ? t0 : 0)) * C);
    const rsrc_t rdv = make_rsrc(dv + (row0 + (t0 < T ? t0 : 0)) * C);
    RevCarry rc = rfollow(fut, lfut, (double)((NW - 1 - q) * CH) * K.w2);
    rnormalize(rc);
    const double rgap = (double)ref * kLog2eD + rc.r;
    const bool rx = fx || wave_any(rgap > (double)kCarryGap);
    if (!rx) {
        const double fr = exp2_64(rgap);
        const double dwf = K.dwf;
        double R = rc.g * fr, Q = rc.h * fr;
#pragma unroll
        for (int j = CH - 1; j >= 0; --j) {
            const double e = (double)kc[j], vv = (double)vc[j], sg = (double)gc[j];
            const double yy = (double)yc[j];
            const double cs = K.eu * sg;
            if (j < Lv && cval) {
                bstore(rdv, (float)(e * (cs + R)), voff, j * stride);
                bstore(rdk, (float)(e * fma(cs, vv - yy, fma(vv, R, -Q))), voff, j * stride);
            }
            R = fma(R, dwf, sg);
            Q = fma(Q, dwf, sg * yy);
        }
    } else {
        load_chunk<CH>(kc, vc, k, v, row0, t0, T, C, voff);
        load_chunk1<CH>(gc, dy, row0, t0, T, C, voff);
        double d0 = 0.0, d1 = 0.0;
        exact_chunk<CH, true, false>(kc, vc, gc, yc, Lv, ref, mine, rc, K.uc, wc, rdk, rdv,
                                     voff, stride, cval, d0, d1);
    }

    // ---- dw, du partials of this window, summed over its chunks in a fixed order ----
    __syncthreads();
    sh.a[q][lane] = du_acc;
    sh.b[q][lane] = -dw_acc;
    __syncthreads();
    if (q == 0) {
        double su = 0.0, sw = 0.0;
        for (int qq = 0; qq < NW; ++qq) {
            su += sh.a[qq][lane];
            sw += sh.b[qq][lane];
        }
        if (cval) {
            part[rec * 2] = sw;
            part[rec * 2 + 1] = su;
        }
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
