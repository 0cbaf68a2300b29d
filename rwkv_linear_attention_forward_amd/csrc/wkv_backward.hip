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
// Work decomposition as in the forward (64 channels x one 64-token window per workgroup,
// one 32-token chunk per wave), with units numbered from the last window backwards so that
// the future of a unit was launched first. Each unit reads k, v, dy once and writes dk, dv
// once: 20 bytes per element. The forward state entering each chunk (with A', B') is read
// from the forward's workspace, so no extra pass over k and v is needed.
//
// Per chunk, in the forward pass's chunk frame (ref = max k, e_j = e^{k_j - ref}):
//   F1     the carry entering the chunk: the previous window's inclusive carry or the
//          window's kept chunk carry, from the forward's workspace.
//   F3     y_j, den_j, sigma_j = dy_j / den_j (s_t in the frame) and the dw, du terms,
//          all in fp64 from fp64 weights e_j: dw is a sum over B*T tokens whose terms
//          cancel by factors of 10^4 on some channels (and its per-sequence parts cancel
//          again over the batch), so any fp32 rounding of e_j, y_j or sigma_j inside it
//          shows up. e_j and sigma_j are then kept in fp32 registers and sigma_j y_j in
//          LDS for dk, dv.
//   R1     reverse summary of the chunk from a zero future, by Horner from the chunk end:
//          R_{j-1} = e^{-w} R_j + sigma_j, Q likewise with sigma_j y_j (fp64).
//   scan   reverse summaries are folded through LDS and across windows (decoupled
//          look-back toward later windows) into the future sums at each chunk's end.
//   R3     the same recursion from the incoming future sums gives, per token,
//          e^{k_i} G_i = e_i R_i and e^{k_i} H_i = e_i Q_i, hence dv and dk.
// Chunks whose frame would under- or overflow, or that hold a key more than 87 below their
// largest (an fp32 weight without full precision), are redone with a per-token rescaled
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

// Reverse record i of n (fields g, h, r at stride n).
__device__ __forceinline__ void put_rrec(double *p, int64_t n, int64_t i, const RevCarry &c) {
    put_u64(p + i, c.g);
    put_u64(p + n + i, c.h);
    put_u64(p + 2 * n + i, c.r);
}
__device__ __forceinline__ RevCarry get_rrec(const double *p, int64_t n, int64_t i) {
    return RevCarry{get_u64(p + i), get_u64(p + n + i), get_u64(p + 2 * n + i)};
}

// ---------------------------------------------------------------------------------
// Exact per-token backward of one lane's chunk (tokens [0, Lv) from t0), for chunks whose
// fixed frame would under- or overflow (a dominant key next to much smaller ones, extreme
// u). Everything is fp64 with library exponentials. It reads k, v, dy straight from
// memory in loops that are not unrolled (per-token values of the forward sweep go to
// private arrays), so that this rare path holds few registers of its own. `fin` is the
// forward carry entering the chunk, `rin` the future sums at the chunk's nominal end (CH
// tokens on). The forward sweep sums the chunk's dw, du terms if FG; the reverse sweep
// stores dk, dv if OUT. With `r` the cotangent is gated (dy = dout sigma(r), dout read from
// `dy`), and with `dr` the forward sweep also stores dr = dout sigma(r) (1 - sigma(r)) y.
// Returns the future sums at the chunk start and the dw, du terms.
// ---------------------------------------------------------------------------------
struct RevState64 {  // (G, H) = (g, h) e^{r - ref}
    double g, h, r;
};

// What exact_chunk returns: the future sums at the chunk start and (FG) the chunk's du, dw
// terms. (Results are returned, not written through references, so that the function needs
// no stack object when it is not inlined.)
struct ExactResult {
    RevCarry fut;
    double du, dw;
};

template <int CH, bool OUT, bool FG, Io IO>
__device__ __noinline__ ExactResult exact_chunk(
    const io_t<IO> *__restrict__ k, const io_t<IO> *__restrict__ v,
    const io_t<IO> *__restrict__ dy, io_t<IO> *__restrict__ dk, io_t<IO> *__restrict__ dv,
    int64_t row0, int64_t t0, int Lv,
    int64_t C, int cl, bool st_ok, float ref, const Carry fin, RevCarry rin, float uc,
    float wc, const io_t<IO> *__restrict__ r = nullptr, io_t<IO> *__restrict__ dr = nullptr) {
    double du_acc = 0.0, dw_acc = 0.0;
    const double refd = (double)ref;
    const double ref2 = refd * kLog2eD;  // the frame 2^{ref2} the carries refer to
    // the carries are relative to 2^{ref2}; the per-token path works relative to e^{ref}
    const double shift = ref2 * kLn2D - refd;
    const double u = (double)uc, w = (double)wc;
    double ys[CH], ss[CH], ms[CH];
    Rs64 st{fin.a, fin.b, fin.ap, fin.bp, (fin.P - ref2) * kLn2D + shift};
#pragma unroll 1
    for (int j = 0; j < Lv; ++j) {
        const int64_t i = (row0 + t0 + j) * C + cl;
        const double kr = (double)io_ld<IO>(k, i) - refd, vv = (double)io_ld<IO>(v, i);
        const double uk = u + kr;
        const double m = fmax(st.p, uk);
        const double e1 = exp(st.p - m), e2 = exp(uk - m);
        const double rden = 1.0 / fma(e1, st.b, e2);
        const double yv = fma(e1, st.a, e2 * vv) * rden;
        double g = (double)io_ld<IO>(dy, i);
        if (r != nullptr) {
            const double sr = sigmoid64(io_ld<IO>(r, i));
            g *= sr;  // the gated cotangent, in fp64 (dw, du cancel too much for fp32)
            if (FG && dr != nullptr) io_st<IO>(dr, i, (float)(g * (1.0 - sr) * yv));
        }
        const double sg = g * rden;  // dy / D in units of e^{-(m + ref)}
        if (FG) {
            // s (A' - y B') and s e^{u+k} (v - y), with A' = a' e^{p+ref}
            dw_acc = fma(sg * e1, fma(-yv, st.bp, st.ap), dw_acc);
            du_acc = fma(sg * e2, vv - yv, du_acc);
        }
        ys[j] = yv;
        ss[j] = sg;
        ms[j] = m;
        rs64_push(st, kr, vv, w);
    }
    rnormalize(rin);
    RevState64 rs{rin.g, rin.h, (rin.r + ref2) * kLn2D - shift};
    rs.r -= (double)(CH - Lv) * w;  // padded tokens past T: pure decay (their s is 0)
#pragma unroll 1
    for (int j = Lv - 1; j >= 0; --j) {
        const int64_t i = (row0 + t0 + j) * C + cl;
        const double kr = (double)io_ld<IO>(k, i) - refd, vv = (double)io_ld<IO>(v, i);
        const double yy = ys[j], sg = ss[j], M = ms[j];
        if (OUT) {
            const double ekr = exp(kr + rs.r);
            const double cpi = sg * exp(u + kr - M);
            if (st_ok) {
                io_st<IO>(dv, i, (float)fma(ekr, rs.g, cpi));
                io_st<IO>(dk, i, (float)fma(cpi, vv - yy, ekr * fma(vv, rs.g, -rs.h)));
            }
        }
        const double a = rs.r - w, b = -M;
        const double rn = fmax(a, b);
        const double fa = exp(a - rn), fb = exp(b - rn);
        rs.g = fma(rs.g, fa, sg * fb);
        rs.h = fma(rs.h, fa, sg * yy * fb);
        rs.r = rn;
    }
    // G = g e^{r - ref} at the chunk start
    return ExactResult{RevCarry{rs.g, rs.h, (rs.r - refd) * kLog2eD}, du_acc, dw_acc};
}

// LDS of a backward unit: staging for the window's reverse summaries and the dw/du
// partials, and each wave's per-token sigma_j y_j from F3 until its reverse sweep (sigma_j
// itself stays in the registers that held dy_j: half the LDS of staging both).
template <int NW, int CH>
struct BwdShared {
    double a[NW][64];
    double b[NW][64];
    double r[NW][64];
    double pu[NW][64], pw[NW][64];  // each wave's du, dw terms
    float sy[NW][CH][64];
    float ref[NW][64];  // each lane's chunk frame, kept here across the look-back
    int status[2];
};

// Per-channel constants of a backward lane.
struct BwdConst {
    double dwf;      // e^{-w}
    double eu;       // e^{u}
    float wc;        // the decay rate
    float uc;
    bool slow_wave;  // some lane has |u| > 60: exact path throughout
    // w log2 e, recomputed where used (the asm keeps it from being held across the kernel)
    __device__ __forceinline__ double w2() const {
        float x = wc;
        asm volatile("" : "+v"(x));
        return (double)x * kLog2eD;
    }
};

// Register budget. The plain backward runs at three waves per SIMD (at most 168 VGPRs; its
// hot path needs ~162), which only holds if the chunk's 96 registers (kc, vc, gc) are not
// also live inside the rare paths: the per-token path and the look-back's recomputation of
// another window are functions that are not inlined (their stack and registers are touched
// only when they run), and after either the chunk's registers are redefined here, so that
// the compiler sees their old values die before the call. A chunk that took the per-token
// path takes it for dk, dv too; a look-back that recomputed a window reloads and recomputes
// the unit's own chunk afterwards (bitwise the same).
template <int CH>
__device__ __forceinline__ void kill_chunk(float (&kc)[CH], float (&vc)[CH], float (&gc)[CH]) {
#pragma unroll
    for (int j = 0; j < CH; ++j) kc[j] = vc[j] = gc[j] = 0.0f;
}

// One lane's chunk ci (tokens t0 = ci*CH ...): the forward recomputation from the chunk's
// entering carry (read from the forward's workspace) and, in the same sweep, the chunk's
// reverse summary from a zero future (R1):
//   R = sum_j e^{-j w} sigma_j,  Q = sum_j e^{-j w} sigma_j y_j   (future sums at the
// chunk start, in the chunk frame).
// Also the chunk's dw, du terms; e_j, v_j, sigma_j are left in kc, vc, gc and sigma_j y_j in
// `sy` (fp32) for the reverse sweep, unless fx (the fixed frame failed for some lane of the
// wave; the chunk then takes the per-token path). helper_summary repeats the summary
// arithmetic op for op, so a helper publishes the bits the owner would (every fused
// multiply-add is written out; the build does not contract).
template <int CH, bool GATE, Io IO>
__device__ __forceinline__ RevCarry chunk_pass(
    int64_t ci, int64_t T, int64_t C, const FwdCarries &F, int64_t bidx, int64_t row0,
    int cl, bool cval, int voff, int stride, const io_t<IO> *__restrict__ rgate,
    io_t<IO> *__restrict__ dr, const io_t<IO> *__restrict__ k, const io_t<IO> *__restrict__ v,
    const io_t<IO> *__restrict__ dy,
    const BwdConst &K, float (&kc)[CH], float (&vc)[CH], float (&gc)[CH],
    float (*__restrict__ sy)[64], int lane, bool &fx, float &ref, int &Lv, double &du_acc,
    double &dw_acc) {
    const int64_t t0 = ci * CH;
    Lv = chunk_len(t0, T, CH);
    load_chunk<CH, IO>(kc, vc, k, v, row0, t0, T, C, voff);
    load_chunk1<CH, IO>(gc, dy, row0, t0, T, C, voff);
    if constexpr (GATE) {
        // r's chunk goes straight into the LDS rows that sigma y takes over token by token in
        // the sweep (a dword per lane, a 16-bit format zero-extended), holding no registers
        if (Lv > 0) load_chunk_lds<CH, IO>(sy, rgate, row0, t0, Lv, C, voff);
    }
    ref = chunk_ref<CH>(kc, Lv);
    const double refd = (double)ref;
    const double ref2 = refd * kLog2eD;
    du_acc = 0.0;
    dw_acc = 0.0;
    if (Lv == 0) {  // past the sequence end
        fx = false;
        return rev_zero();
    }
    const Carry fin = chunk_carry(F, bidx, ci, C, cl);
    const double gap = fin.P - ref2;
    fx = K.slow_wave || wave_any(gap > (double)kCarryGap || chunk_has_faint_key<CH>(kc, Lv, ref));
    double R = 0.0, Q = 0.0;
    if (!fx) {
        if constexpr (GATE) lds_load_fence();
        // dr's stores carry no branch: a token past the sequence end (or a call without dr)
        // stores through a record of size 0, which drops them; a lane past C repeats the
        // store of the lane for channel C-1 (the same value: it computes the same inputs)
        const rsrc_t rnull = make_rsrc_empty(dy);
        const rsrc_t rdr = GATE && dr != nullptr ? make_rsrc(dr + (row0 + t0) * C) : rnull;
        const double s0 = exp2_64(gap);
        double Sx = fin.a * s0, Zx = fin.b * s0;
        // A'_j = d P_j with P_{j+1} = d P_j + A_j (d = e^{-w}; A'_{j+1} = d (A'_j + A_j));
        // the dw terms are summed without the common factor d, applied at the end
        double Ps = 0.0, Pz = 0.0;
        if (K.dwf > 0.0) {
            Ps = fin.ap * s0 / K.dwf;
            Pz = fin.bp * s0 / K.dwf;
        }
        double pw = 1.0;
        bool tiny = false;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            // padded tokens (k = -inf, v = dy = 0) contribute e = sigma = 0; the clamp on den
            // keeps 1/den finite where a padded token's den (the decayed carry alone) falls
            // below the fp32 range, so that its sigma is 0 and not NaN. Their den enters the
            // test too: at worst a ragged last chunk takes the per-token path.
            const double e = exp2_64(fma((double)kc[j], kLog2eD, -ref2));
            const double vv = (double)vc[j];
            const double ev = e * vv;
            const double num = fma(K.eu, ev, Sx);
            const double den = fma(K.eu, e, Zx);
            tiny = tiny || !(den >= (double)kTinyDen);
            const double r = rcpd(fmax(den, 0x1p-120));
            const double yv = num * r;
            double gd = (double)gc[j];
            if constexpr (GATE) {
                // the gated cotangent dout sigma(r) in fp64, and dr = dout sigma (1 - sigma) y,
                // stored now (a chunk that then takes the per-token path stores it again)
                const double sr = sigmoid64(lds_widen<IO>(sy[j][lane]));
                gd *= sr;
                bstore_io<IO>(j < Lv ? rdr : rnull, (float)(gd * (1.0 - sr) * yv), voff,
                              j * stride);
            }
            const double sg = gd * r;
            const double sgy = sg * yv;
            // dw term s (A' - y B') / d and du term s e^{k} (v - y), both in the frame; the
            // common factors d and e^u are applied after the loop
            dw_acc = fma(sg, fma(-yv, Pz, Ps), dw_acc);
            du_acc = fma(sg, fma(-e, yv, ev), du_acc);
            R = fma(pw, sg, R);
            Q = fma(pw, sgy, Q);
            kc[j] = (float)e;
            gc[j] = (float)sg;
            sy[j][lane] = (float)sgy;
            pw *= K.dwf;
            Ps = fma(Ps, K.dwf, Sx);
            Pz = fma(Pz, K.dwf, Zx);
            Sx = fma(Sx, K.dwf, ev);
            Zx = fma(Zx, K.dwf, e);
        }
        dw_acc *= K.dwf;
        du_acc *= K.eu;
        fx = wave_any(tiny);
    }
    if (!fx) return RevCarry{R, Q, -ref2};
    const ExactResult xr = exact_chunk<CH, false, true, IO>(
        k, v, dy, nullptr, nullptr, row0, t0, Lv, C, cl, false, ref, fin, rev_zero(), K.uc,
        K.wc, GATE ? rgate : nullptr, GATE && cval ? dr : nullptr);
    du_acc = xr.du;
    dw_acc = xr.dw;
    kill_chunk<CH>(kc, vc, gc);
    return xr.fut;
}

// Reverse summary of another unit's chunk, for the look-back's recomputation of a window
// whose aggregate was not published in time: the summary arithmetic of chunk_pass, op
// for op and in the same order, the per-token-path decision included (so the bits are those
// the owner publishes), streaming k, v, dy from memory in a loop that is not unrolled.
template <int CH, Io IO>
__device__ __noinline__ RevCarry helper_summary(
    int64_t ci, int64_t T, int64_t C, const FwdCarries F, int64_t bidx, int64_t row0,
    int cl, const io_t<IO> *__restrict__ k, const io_t<IO> *__restrict__ v,
    const io_t<IO> *__restrict__ dy, const io_t<IO> *__restrict__ rg,
    const BwdConst K) {
    const int64_t t0 = ci * CH;
    const int Lv = chunk_len(t0, T, CH);
    if (Lv == 0) return rev_zero();
    const io_t<IO> *kp = k + (row0 + t0) * C + cl;
    const io_t<IO> *vp = v + (row0 + t0) * C + cl;
    const io_t<IO> *gp = dy + (row0 + t0) * C + cl;
    float ref = kNegBig, kmin = __builtin_inff();
#pragma unroll 1
    for (int j = 0; j < Lv; ++j) {
        const float kj = io_ld<IO>(kp, (int64_t)j * C);
        ref = fmaxf(ref, kj);
        kmin = fminf(kmin, kj);
    }
    const double refd = (double)ref;
    const double ref2 = refd * kLog2eD;
    const Carry fin = chunk_carry(F, bidx, ci, C, cl);
    const double gap = fin.P - ref2;
    // the owner's tests, in the same order: carry gap, faint key (chunk_has_faint_key)
    bool fx = K.slow_wave || wave_any(gap > (double)kCarryGap || ref - kmin > kFaintGap);
    if (!fx) {
        const double s0 = exp2_64(gap);
        double Sx = fin.a * s0, Zx = fin.b * s0;
        double pw = 1.0, R = 0.0, Q = 0.0;
        bool tiny = false;
#pragma unroll 1
        for (int j = 0; j < CH; ++j) {
            const bool in = j < Lv;
            const float kj = in ? io_ld<IO>(kp, (int64_t)j * C) : -__builtin_inff();
            const double e = exp2_64(fma((double)kj, kLog2eD, -ref2));
            const double vv = in ? (double)io_ld<IO>(vp, (int64_t)j * C) : 0.0;
            const double ev = e * vv;
            const double num = fma(K.eu, ev, Sx);
            const double den = fma(K.eu, e, Zx);
            tiny = tiny || !(den >= (double)kTinyDen);  // padded tokens too, as the owner
            const double r = rcpd(fmax(den, 0x1p-120));
            const double yv = num * r;
            double g = in ? (double)io_ld<IO>(gp, (int64_t)j * C) : 0.0;
            if (rg != nullptr) g *= sigmoid64(in ? io_ld<IO>(rg, (row0 + t0 + j) * C + cl) : 0.0f);
            const double sg = g * r;
            const double sgy = sg * yv;
            R = fma(pw, sg, R);
            Q = fma(pw, sgy, Q);
            pw *= K.dwf;
            Sx = fma(Sx, K.dwf, ev);
            Zx = fma(Zx, K.dwf, e);
        }
        fx = wave_any(tiny);
        if (!fx) return RevCarry{R, Q, -ref2};
    }
    return exact_chunk<CH, false, false, IO>(k, v, dy, nullptr, nullptr, row0, t0, Lv, C, cl,
                                             false, ref, fin, rev_zero(), K.uc, K.wc, rg)
        .fut;
}

// Stage this wave's chunk reverse summary for window_rev_sums. Contains barriers (all waves
// call it together).
template <int NW, int CH>
__device__ __forceinline__ void window_rev_stage(BwdShared<NW, CH> &sh, const RevCarry &rsum,
                                                 int q, int lane) {
    __syncthreads();
    sh.a[q][lane] = rsum.g;
    sh.b[q][lane] = rsum.h;
    sh.r[q][lane] = rsum.r;
    __syncthreads();
}

// Fold the window's NW staged summaries (last chunk first) from a zero future: `agg` is the
// window's reverse aggregate, `lfut` the part of it that lies after this wave's chunk. (Cheap
// enough to redo from the staged values rather than hold 12 registers across the look-back.)
template <int NW, int CH>
__device__ __forceinline__ void window_rev_sums(const BwdShared<NW, CH> &sh, int q, int lane,
                                                double w2, RevCarry &agg, RevCarry &lfut) {
    agg = rev_zero();
    lfut = agg;
#pragma unroll
    for (int qq = NW - 1; qq >= 0; --qq) {
        if (qq == q) lfut = agg;
        rfold(agg, RevCarry{sh.a[qq][lane], sh.b[qq][lane], sh.r[qq][lane]}, (double)CH * w2);
    }
}

// GATE: the output was sigma(r) * y; `dy` holds the cotangent of that gated output, and dr
// is written too. IO: the storage format of k, v, dy, r, dk, dv and dr. `tries`: polls
// before a missing window is recomputed.
template <int NW, int CH, bool GATE, Io IO>
__global__ __launch_bounds__(NW * 64, 3) void wkv_backward_kernel(
    int64_t B, int64_t T, int64_t C, int ngrp, int64_t nbg, int64_t nseg,
    uint64_t epoch, int tries, const float *__restrict__ w, const float *__restrict__ u,
    const io_t<IO> *__restrict__ k, const io_t<IO> *__restrict__ v,
    const io_t<IO> *__restrict__ dy, const io_t<IO> *__restrict__ r, const FwdCarries F,
    io_t<IO> *__restrict__ dk, io_t<IO> *__restrict__ dv, io_t<IO> *__restrict__ dr,
    float *__restrict__ dw,
    float *__restrict__ du,
    uint64_t *__restrict__ flags, double *__restrict__ ragg, double *__restrict__ rincl,
    double *__restrict__ part) {
    constexpr int WIN = NW * CH;
    __shared__ BwdShared<NW, CH> sh;

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
    const int voff = cl * kIoBytes<IO>;
    const int stride = (int)(C * kIoBytes<IO>);

    const float wc = w[cl];
    BwdConst K;
    K.uc = u[cl];
    K.wc = wc;
    K.dwf = exp(-(double)wc);
    K.eu = exp((double)K.uc);
    K.slow_wave = wave_any(!(fabsf(K.uc) <= 60.0f));
    const int64_t row0 = bidx * T;
    const int64_t ci = s * NW + q;
    const int64_t t0 = ci * CH;

    float kc[CH], vc[CH], gc[CH];
    bool fx;
    float ref;
    int Lv;
    double du_acc, dw_acc;
    RevCarry rsum = chunk_pass<CH, GATE, IO>(ci, T, C, F, bidx, row0, cl, cval, voff, stride, r,
                                         dr, k, v, dy, K, kc, vc, gc, sh.sy[q], lane, fx, ref,
                                         Lv, du_acc, dw_acc);
    // the dw, du terms and the frame are staged with the reverse summaries (the fold's
    // barrier covers them)
    sh.pu[q][lane] = du_acc;
    sh.pw[q][lane] = dw_acc;
    sh.ref[q][lane] = ref;
    window_rev_stage<NW, CH>(sh, rsum, q, lane);
    const int64_t nrec = B * nseg * C;
    uint64_t *myflag = flags + sidx * nbg + bg;
    // the next window's flag is read before this unit's flag store, so that one wait
    // covers the aggregate's stores and that read
    uint64_t next = 0;
    if (q == 0) {
        if (cval) {
            const int64_t rec = (bidx * nseg + s) * C + cl;
            RevCarry agg, lf;
            window_rev_sums<NW, CH>(sh, q, lane, K.w2(), agg, lf);
            put_rrec(ragg, nrec, rec, agg);
            // this window's dw, du partial: its chunks' terms summed in a fixed order
            double su = 0.0, sw = 0.0;
            for (int qq = 0; qq < NW; ++qq) {
                su += sh.pu[qq][lane];
                sw += sh.pw[qq][lane];
            }
            part[rec] = -sw;
            part[nrec + rec] = su;
        }
        if (s < nseg - 1) next = peek_flag(myflag - nbg);
        put_flag(myflag, epoch, kAggregate);
    }

    // ---- look-back toward later windows: future sums at this window's end ----
    // Walk forward in time to the nearest window whose inclusive future sums are
    // published (or past the sequence end), making sure every window in between has its
    // reverse aggregate in memory, then fold those back in order: bitwise the sequential
    // chain rincl[s] = rfold(rincl[s+1], ragg[s]) whatever the timing.
    // beyond the last window the future is zero, or what a cotangent of the final state puts
    // there (as sums at the window end, F.tail)
    auto beyond = [&]() {
        return F.tail != nullptr ? get_rrec(F.tail, F.nrec / F.nseg, bidx * C + cl) : rev_zero();
    };
    RevCarry fut = rev_zero();
    if (s == nseg - 1) fut = beyond();
    if (s < nseg - 1) {
        int64_t j = s + 1;
        int it = 0;
        bool redo = false;
        for (;;) {
            if (q == 0) {
                int st = it == 0 ? flag_status(next, epoch) : 0;
                if (st != 0)
                    consume_fence();
                else
                    st = poll_flag(flags + (nseg - 1 - j) * nbg + bg, epoch, tries);
                if (lane == 0) sh.status[it & 1] = st;
            }
            __syncthreads();
            const int st = sh.status[it & 1];
            ++it;
            if (st == (int)kInclusive) break;
            if (st != (int)kAggregate) {
                // not published in time: recompute window j's reverse aggregate here and
                // publish it (bitwise what unit j itself publishes)
                const RevCarry rs_j = helper_summary<CH, IO>(j * NW + q, T, C, F, bidx, row0, cl,
                                                         k, v, dy, GATE ? r : nullptr, K);
                RevCarry agg_j, lf_j;
                window_rev_stage<NW, CH>(sh, rs_j, q, lane);
                window_rev_sums<NW, CH>(sh, q, lane, K.w2(), agg_j, lf_j);
                if (q == 0) {
                    if (cval) put_rrec(ragg, nrec, (bidx * nseg + j) * C + cl, agg_j);
                    raise_flag(flags + (nseg - 1 - j) * nbg + bg, epoch, kAggregate);
                }
                // the unit's own chunk and staged summaries are redone after the walk
                kill_chunk<CH>(kc, vc, gc);
                redo = true;
            }
            if (j == nseg - 1) {
                j = nseg;
                break;
            }
            ++j;
        }
        if (redo) {  // the same for every wave of the unit (the status is shared)
            double du_x, dw_x;
            float ref_x;
            const RevCarry rs2 = chunk_pass<CH, GATE, IO>(ci, T, C, F, bidx, row0, cl, cval, voff,
                                                          stride, r, dr, k, v, dy, K, kc, vc, gc,
                                                          sh.sy[q], lane, fx, ref_x, Lv, du_x,
                                                          dw_x);
            window_rev_stage<NW, CH>(sh, rs2, q, lane);
        }
        fut = j < nseg ? get_rrec(rincl, nrec, (bidx * nseg + j) * C + cl) : beyond();
        for (int64_t m = j - 1; m > s; --m)
            fut = rfollow(fut, get_rrec(ragg, nrec, (bidx * nseg + m) * C + cl),
                          (double)WIN * K.w2());
    }
    RevCarry agg, lfut;
    window_rev_sums<NW, CH>(sh, q, lane, K.w2(), agg, lfut);
    if (q == 0 && cval)
        put_rrec(rincl, nrec, (bidx * nseg + s) * C + cl, rfollow(fut, agg, (double)WIN * K.w2()));

    // ---- R3: dk, dv of this chunk ----
    const rsrc_t rdk = make_rsrc(dk + (row0 + (t0 < T ? t0 : 0)) * C);
    const rsrc_t rdv = make_rsrc(dv + (row0 + (t0 < T ? t0 : 0)) * C);
    RevCarry rc = rfollow(fut, lfut, (double)((NW - 1 - q) * CH) * K.w2());
    rnormalize(rc);
    ref = sh.ref[q][lane];
    const double rgap = (double)ref * kLog2eD + rc.r;
    const bool rx = fx || wave_any(rgap > (double)kCarryGap);
    // The sweep's arithmetic runs before wave 0 stores the inclusive flag, so that the wait
    // for the record's stores overlaps it; dv, dk replace e, v in kc, vc and are stored
    // after the flag.
    if (Lv != 0 && !rx) {
        const double fr = exp2_64(rgap);
        const double dwf = K.dwf;
        double R = rc.g * fr, Q = rc.h * fr;
#pragma unroll
        for (int j = CH - 1; j >= 0; --j) {
            // dv = e (e^u s + R),  dk = e (e^u s (v - y) + v R - Q) = v dv - e (e^u s y + Q)
            const double e = (double)kc[j], vv = (double)vc[j];
            const double sg = (double)gc[j], sgy = (double)sh.sy[q][j][lane];
            const double dvv = e * fma(K.eu, sg, R);
            const double dkk = fma(vv, dvv, -(e * fma(K.eu, sgy, Q)));
            kc[j] = (float)dvv;
            vc[j] = (float)dkk;
            R = fma(R, dwf, sg);
            Q = fma(Q, dwf, sgy);
        }
    }
    if (q == 0) put_flag(myflag, epoch, kInclusive);
    if (Lv == 0) {
        // past the sequence end: nothing to store
    } else if (!rx) {
        if (cval) {
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                if (j < Lv) {
                    bstore_io<IO>(rdv, kc[j], voff, j * stride);
                    bstore_io<IO>(rdk, vc[j], voff, j * stride);
                }
            }
        }
    } else {
        const Carry fin = chunk_carry(F, bidx, ci, C, cl);
        exact_chunk<CH, true, false, IO>(k, v, dy, dk, dv, row0, t0, Lv, C, cl, cval, ref, fin, rc,
                                         K.uc, wc, GATE ? r : nullptr);
    }
}

// dw[c], du[c]: the sums of the B * nseg window partials of each channel, in a fixed order.
// A workgroup takes kReduceCh channels (one 128-byte row segment of each partial array) and
// kReduceSlices row slices: thread (slice r, channel) sums partials r, r + RS, r + 2 RS, ...
// (loads issued in batches), then slice 0 adds the RS slice sums in order. ceil(C/16)
// workgroups: enough to spread the 16 B per window and channel over the whole chip.
constexpr int kReduceCh = 16;      // channels of a workgroup: one 128-byte row of fp64
constexpr int kReduceSlices = 32;  // row slices of a workgroup

// The forward workspace's stamp must show a launch that kept the backward's states for the
// same (B, T, C); otherwise dw and du are set to NaN (the host refuses such a call when it
// can tell; this catches what it cannot, e.g. a workspace filled by another process).
__global__ __launch_bounds__(kReduceCh * kReduceSlices) void wkv_reduce_kernel(
    int64_t npart, int64_t C, const double *__restrict__ part, float *__restrict__ dw,
    float *__restrict__ du, const uint64_t *__restrict__ hdr, int64_t B, int64_t T) {
    constexpr int RS = kReduceSlices, RB = 8;
    __shared__ double sw_[RS][kReduceCh], su_[RS][kReduceCh];
    // uniform across the launch: read once, up front
    const bool stamped = hdr[0] == (kWsTag | kWsKept) && hdr[1] == (uint64_t)B &&
                         hdr[2] == (uint64_t)T && hdr[3] == (uint64_t)C;
    const int ch = (int)threadIdx.x % kReduceCh;
    const int sl = (int)threadIdx.x / kReduceCh;
    const int64_t c = (int64_t)blockIdx.x * kReduceCh + ch;
    const int64_t cl = c < C ? c : C - 1;
    const int64_t nrec = npart * C;
    double sw = 0.0, su = 0.0;
    for (int64_t i0 = sl; i0 < npart; i0 += (int64_t)RS * RB) {
        double a[RB], b[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            const int64_t i = i0 + (int64_t)r * RS;
            const int64_t ic = i < npart ? i : npart - 1;
            a[r] = part[ic * C + cl];
            b[r] = part[nrec + ic * C + cl];
        }
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            if (i0 + (int64_t)r * RS < npart) {
                sw += a[r];
                su += b[r];
            }
        }
    }
    sw_[sl][ch] = sw;
    su_[sl][ch] = su;
    __syncthreads();
    if (sl == 0 && c < C) {
        double tw = 0.0, tu = 0.0;
        for (int r = 0; r < RS; ++r) {
            tw += sw_[r][ch];
            tu += su_[r][ch];
        }
        dw[c] = stamped ? (float)tw : __builtin_nanf("");
        du[c] = stamped ? (float)tu : __builtin_nanf("");
    }
}

__global__ __launch_bounds__(256) void wkv_zero2_kernel(float *__restrict__ a,
                                                        float *__restrict__ b, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) {
        a[i] = 0.0f;
        b[i] = 0.0f;
    }
}

template <Io IO>
static void launch_backward_io(int64_t units, hipStream_t stream, int64_t B, int64_t T,
                               int64_t C, int ngrp, int64_t nbg, const BwdLayout &L,
                               uint64_t epoch, const float *w, const float *u, const void *k,
                               const void *v, const void *dy, const void *r,
                               const FwdCarries &fc, void *dk, void *dv, void *dr, float *dw,
                               float *du) {
    using E = io_t<IO>;
    const E *kk = static_cast<const E *>(k), *vv = static_cast<const E *>(v),
            *gg = static_cast<const E *>(dy), *rr = static_cast<const E *>(r);
    E *ddk = static_cast<E *>(dk), *ddv = static_cast<E *>(dv), *ddr = static_cast<E *>(dr);
    if (r != nullptr)
        hipLaunchKernelGGL((wkv_backward_kernel<kBwdWaves, kCinChunk, true, IO>),
                           dim3((unsigned)units), dim3(kBwdWaves * 64), 0, stream, B, T, C, ngrp,
                           nbg, L.nseg, epoch, poll_limit(), w, u, kk, vv, gg, rr, fc, ddk, ddv,
                           ddr, dw, du, L.flags, L.ragg, L.rincl, L.part);
    else
        hipLaunchKernelGGL((wkv_backward_kernel<kBwdWaves, kCinChunk, false, IO>),
                           dim3((unsigned)units), dim3(kBwdWaves * 64), 0, stream, B, T, C, ngrp,
                           nbg, L.nseg, epoch, poll_limit(), w, u, kk, vv, gg, rr, fc, ddk, ddv,
                           ddr, dw, du, L.flags, L.ragg, L.rincl, L.part);
}

// Cotangent of the final state. With (a_T, b_T, p_T) the state the forward returned after
// token T-1 (A_T = a_T e^{p_T}, B_T = b_T e^{p_T}) and da_T, db_T the gradient of L with
// respect to a_T, b_T: dL/dA_T = da_T e^{-p_T} (B alike). A_T = sum_i e^{-(T-1-i) w} e^{k_i}
// v_i + e^{-T w} A_0 is what a token at T would see, so the cotangent acts as one more
// token at T with s_T = dA_T and s_T y_T = -dB_T in the future sums G, H of every earlier
// token (and of the state before token 0): dk, dv and da, db, dp take it in through the
// backward's reverse scan, which starts the last window from it. As sums at that window's
// end (nseg * 64 tokens, d = nseg * 64 - T tokens past T): (G, H) = (dA_T, -dB_T) e^{d w}.
__global__ __launch_bounds__(256) void wkv_tail_kernel(int64_t n, int64_t T, int64_t C,
                                                       int64_t nseg,
                                                       const float *__restrict__ w,
                                                       const float *__restrict__ dfa,
                                                       const float *__restrict__ dfb,
                                                       const float *__restrict__ fin,
                                                       double *__restrict__ tail) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int64_t c = i % C;
    const double d = (double)(nseg * kBwdWindow - T);
    RevCarry t{(double)dfa[i], -(double)dfb[i],
               (d * (double)w[c] - (double)fin[2 * n + i]) * kLog2eD};
    if (t.g == 0.0 && t.h == 0.0) t = rev_zero();
    rnormalize(t);
    put_rrec(tail, n, i, t);
}

// ... and dw: the extra token's term -s_T (A'_T - y_T B'_T) = -(dA_T A'_T + dB_T B'_T), with
// the age-weighted sums A'_T, B'_T after token T-1: from the forward's carry entering the
// last 32-token chunk, the chunk's tokens are folded in one at a time (fp64, rescaled at
// every token) and the term is added to the last window's dw partial. One lane per (b, c).
template <Io IO>
__global__ __launch_bounds__(256) void wkv_tail_dw_kernel(
    int64_t B, int64_t T, int64_t C, int64_t nseg, const FwdCarries F,
    const float *__restrict__ w, const io_t<IO> *__restrict__ k, const io_t<IO> *__restrict__ v,
    const float *__restrict__ dfa, const float *__restrict__ dfb,
    const float *__restrict__ fin, double *__restrict__ part) {
    const int64_t n = B * C;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int64_t b = i / C, c = i - b * C;
    const int64_t ci = (T - 1) / kCinChunk, t0 = ci * kCinChunk;
    const int Lv = (int)(T - t0);
    float kc[kCinChunk], vc[kCinChunk];  // the chunk's tokens, all loads issued first
#pragma unroll
    for (int j = 0; j < kCinChunk; ++j) {
        const int64_t x = (b * T + t0 + (j < Lv ? j : Lv - 1)) * C + c;
        kc[j] = io_ld<IO>(k, x);
        vc[j] = io_ld<IO>(v, x);
    }
    Carry st = chunk_carry(F, b, ci, C, (int)c);
    const double w2 = (double)w[c] * kLog2eD;
#pragma unroll
    for (int j = 0; j < kCinChunk; ++j) {
        if (j >= Lv) break;
        const double kx = (double)kc[j] * kLog2eD, vx = (double)vc[j];
        const double pd = st.P - w2;
        const double m = fmax(pd, kx);
        const double fa = exp2_64(pd - m), fx = exp2_64(kx - m);
        st.ap = (st.ap + st.a) * fa;
        st.bp = (st.bp + st.b) * fa;
        st.a = fma(st.a, fa, fx * vx);
        st.b = fma(st.b, fa, fx);
        st.P = m;
    }
    const double sc = exp2_64(st.P - (double)fin[2 * n + i] * kLog2eD);
    const double term = -fma((double)dfa[i], st.ap, (double)dfb[i] * st.bp) * sc;
    part[(b * nseg + nseg - 1) * C + c] += term;
}

// Gradient with respect to the state before token 0. That state holds A0 = a e^p and
// B0 = b e^p, which reach token t as e^{-t w} A0 and e^{-t w} B0, so dL/dA0 = G_{-1} and
// dL/dB0 = -H_{-1}: the future sums over the whole sequence (a cotangent of the final state
// included), which the backward leaves as window 0's reverse inclusive record. With the
// state (a, b, 2^P = e^p) as the forward recorded it: da = G e^p, db = -H e^p,
// dp = (a G - b H) e^p. One lane per (b, c).
__global__ __launch_bounds__(256) void wkv_state_grad_kernel(
    int64_t n, int64_t C, int64_t nseg, const double *__restrict__ init,
    const double *__restrict__ rincl, float *__restrict__ ga, float *__restrict__ gb,
    float *__restrict__ gp) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int64_t b = i / C, c = i - b * C;
    const RevCarry fut = get_rrec(rincl, n * nseg, b * nseg * C + c);
    const Carry st = get_cin(init, n, i);
    const double sc = exp2_64(fut.r + st.P);
    ga[i] = (float)(fut.g * sc);
    gb[i] = (float)(-fut.h * sc);
    gp[i] = (float)(fma(st.a, fut.g, -st.b * fut.h) * sc);
}

hipError_t launch_backward(int64_t B, int64_t T, int64_t C, Io fmt, const float *w,
                           const float *u, const void *k, const void *v, const void *dy,
                           const void *r, const FwdLayout &F, void *dk, void *dv, void *dr,
                           float *dw, float *du, float *ga, float *gb, float *gp,
                           const float *dfa, const float *dfb, const BwdLayout &L,
                           uint64_t epoch, hipStream_t stream) {
    const int ngrp = (int)((C + 63) / 64);
    const int64_t nbg = B * ngrp;
    const int64_t units = nbg * L.nseg;
    const FwdCarries fc{F.incl, F.cin, F.init, dfa != nullptr ? L.tail : nullptr,
                        B * F.nseg * C, F.nseg};
    const int64_t n = B * C;
    const dim3 nb((unsigned)((n + 255) / 256));
    if (dfa != nullptr) {
        hipLaunchKernelGGL(wkv_tail_kernel, nb, dim3(256), 0, stream, n, T, C, L.nseg, w, dfa,
                           dfb, F.fin, L.tail);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (fmt == Io::BF16)
        launch_backward_io<Io::BF16>(units, stream, B, T, C, ngrp, nbg, L, epoch, w, u, k, v, dy,
                                     r, fc, dk, dv, dr, dw, du);
    else if (fmt == Io::F16)
        launch_backward_io<Io::F16>(units, stream, B, T, C, ngrp, nbg, L, epoch, w, u, k, v, dy,
                                    r, fc, dk, dv, dr, dw, du);
    else
        launch_backward_io<Io::F32>(units, stream, B, T, C, ngrp, nbg, L, epoch, w, u, k, v, dy,
                                    r, fc, dk, dv, dr, dw, du);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (dfa != nullptr) {
        if (fmt == Io::BF16)
            hipLaunchKernelGGL(wkv_tail_dw_kernel<Io::BF16>, nb, dim3(256), 0, stream, B, T, C,
                               L.nseg, fc, w, static_cast<const io_t<Io::BF16> *>(k),
                               static_cast<const io_t<Io::BF16> *>(v), dfa, dfb, F.fin, L.part);
        else if (fmt == Io::F16)
            hipLaunchKernelGGL(wkv_tail_dw_kernel<Io::F16>, nb, dim3(256), 0, stream, B, T, C,
                               L.nseg, fc, w, static_cast<const io_t<Io::F16> *>(k),
                               static_cast<const io_t<Io::F16> *>(v), dfa, dfb, F.fin, L.part);
        else
            hipLaunchKernelGGL(wkv_tail_dw_kernel<Io::F32>, nb, dim3(256), 0, stream, B, T, C,
                               L.nseg, fc, w, static_cast<const float *>(k),
                               static_cast<const float *>(v), dfa, dfb, F.fin, L.part);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(wkv_reduce_kernel, dim3((unsigned)((C + kReduceCh - 1) / kReduceCh)),
                       dim3(kReduceCh * kReduceSlices), 0,
                       stream, B * L.nseg, C, L.part, dw, du, F.hdr, B, T);
    e = hipGetLastError();
    if (e != hipSuccess || ga == nullptr) return e;
    hipLaunchKernelGGL(wkv_state_grad_kernel, nb, dim3(256), 0, stream, n, C, L.nseg, F.init,
                       L.rincl, ga, gb, gp);
    return hipGetLastError();
}

hipError_t launch_zero2(float *dw, float *du, int64_t C, hipStream_t stream) {
    hipLaunchKernelGGL(wkv_zero2_kernel, dim3((unsigned)((C + 255) / 256)), dim3(256), 0, stream,
                       dw, du, C);
    return hipGetLastError();
}

}  // namespace wkvdev
