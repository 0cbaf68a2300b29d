// wkv_forward.hip -- WKV forward on gfx950: time-split chunked scan with decoupled look-back.
//
// Operator: "RWKV解读：在Transformer的时代的新RNN", section 二.3, formula (8), evaluated
// through its recursive form (same section) as an associative scan over time, which is
// possible because the decay w does not depend on the data ("RWKV についての調査記録",
// section "Trainingについて").
//
// Work decomposition. One workgroup = one unit = 64 channels x one window of WIN = NW*CH
// tokens of one sequence; wave q owns the q-th CH-token chunk of the window, one lane per
// channel. Units are numbered window-major (all units of window 0 first), so a unit's
// predecessor in time was launched earlier; there are B * ceil(C/64) * ceil(T/WIN) units,
// many more than CUs, which keeps all 256 CUs evenly busy even when B*C is small.
// k and v are streamed once with non-temporal loads (one dword per lane per token, 256 B
// per wave per token, coalesced along C) and y is written once: 12 bytes per element.
//
// Per chunk, with frame ref = max_j k_j of the lane's chunk and e_j = e^{k_j - ref} <= 1:
//   phase 1  summary from the empty state: S = sum_j e^{-(CH-1-j)w} e_j v_j, Z likewise
//            without v, and the age-weighted S', Z' (Horner, fp64, e_j from an fp64 exp2:
//            the carries also serve the backward pass, whose dw needs them that exact);
//            the chunk adds S 2^{ref log2 e} to A, Z to B and S', Z' to A', B'.
//   window   summaries go to LDS; after one barrier every wave folds the NW summaries in
//            order from the empty state (identical arithmetic in every wave), giving its own
//            chunk's local incoming carry and the window aggregate. Carries keep their
//            log-scale in fp64 (see wkv_device.h).
//   look-back  the aggregate is published; the carry entering the window is then the fold
//            of the nearest predecessor's published inclusive carry and the aggregates in
//            between (a predecessor that has not published within a bounded wait has its
//            aggregate recomputed from k, v here, so no unit ever blocks on another). The
//            window's inclusive carry is published for its successors and kept for the
//            backward pass.
//   phase 3  outputs from the incoming carry put into the chunk frame, in fp32:
//            y_j = (S_j + e^u e_j v_j) / (Z_j + e^u e_j),  S_{j+1} = e^{-w} S_j + e_j v_j.
// One fp64 exp2 per element in phase 1, one fp32 reciprocal per element in phase 3.
//
// The fixed frame is exact in real arithmetic, but its fp32 weights e^{k - ref} keep full
// precision only for keys within ~87 of the chunk's largest (the fp64 summaries to ~600),
// and the incoming carry must not exceed the frame by more than 2^64. A chunk outside
// either bound, or on a wave with a bonus |u| > 60, is detected per wave and computed with
// the per-token rescaled recursion in fp64 instead, which is safe for any finite k (rare:
// only far outside the training distributions).
#include "wkv_chunk.h"

namespace wkvdev {

// Outputs of one lane's chunk by the per-token rescaled recursion, in fp64 with library
// exponentials, from the carry entering the chunk; for chunks whose fixed frame would under-
// or overflow (keys hundreds apart, extreme u). fp64 throughout: with a key of 1000 setting
// the frame, k - ref alone would carry 6e-5 of fp32 rounding into every weight. Reads k, v
// (and r) straight from memory in a loop that is not unrolled: few registers.
template <int CH, Io F>
__device__ __forceinline__ void exact_outputs(const io_t<F> *__restrict__ k,
                                           const io_t<F> *__restrict__ v,
                                           const io_t<F> *__restrict__ r, io_t<F> *__restrict__ y,
                                           int64_t row0, int64_t t0, int Lv, int64_t C, int cl,
                                           float ref, const Carry &mine, float uc, double w) {
    const double refd = (double)ref, u = (double)uc;
    // A = a e^{p + ref}, B = b e^{p + ref}
    double a = mine.a, b = mine.b, p = (mine.P - refd * kLog2eD) * kLn2D;
#pragma unroll 1
    for (int j = 0; j < Lv; ++j) {
        const int64_t i = (row0 + t0 + j) * C + cl;
        const double kr = (double)io_ld<F>(k, i) - refd, vv = (double)io_ld<F>(v, i);
        const double uk = u + kr;
        const double m = fmax(p, uk);
        const double e1 = exp(p - m), e2 = exp(uk - m);
        const float o = (float)(fma(e1, a, e2 * vv) / fma(e1, b, e2));
        io_st<F>(y, i, r != nullptr ? o * sigmoidf_(io_ld<F>(r, i)) : o);
        const double pw = p - w;
        const double m2 = fmax(pw, kr);
        const double f1 = exp(pw - m2), f2 = exp(kr - m2);
        a = fma(f1, a, f2 * vv);
        b = fma(f1, b, f2);
        p = m2;
    }
}

// The final state in the decode convention (fp32 a, b, p with A = a e^p, B = b e^p) from
// sums S, Z at scale 2^P: p is rounded to fp32 first and a, b rescaled by the rounding, so
// that the fp32 triple holds A and B to fp32 accuracy.
__device__ __forceinline__ void store_state(double S, double Z, double P, float *__restrict__ fin,
                                            int64_t n, int64_t i) {
    const float p32 = (float)(P * kLn2D);
    const double sc = exp2_64(P - (double)p32 * kLog2eD);
    fin[i] = (float)(S * sc);
    fin[n + i] = (float)(Z * sc);
    fin[2 * n + i] = p32;
}

// State after token T-1 = t0 + Lv - 1, from the fp64 carry entering that token's chunk and
// the chunk's weights e_j (fp32, in the chunk frame 2^{ref log2 e}) and values still in
// registers: the recursion over the chunk's Lv tokens, accumulated in fp64 at the larger of
// the two scales. One wave per sequence and channel group runs it.
template <int CH>
__device__ __forceinline__ void final_state(const float (&ec)[CH], const float (&vc)[CH], int Lv,
                                         float ref, const Carry &mine, double dwf,
                                         float *__restrict__ fin, int64_t n, int64_t i) {
    const double ref2 = (double)ref * kLog2eD;
    const double P = fmax(ref2, mine.P);
    const double sc = exp2_64(mine.P - P), sk = exp2_64(ref2 - P);
    double S = mine.a * sc, Z = mine.b * sc;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        if (j < Lv) {
            const double e = (double)ec[j] * sk;
            S = fma(S, dwf, e * (double)vc[j]);
            Z = fma(Z, dwf, e);
        }
    }
    store_state(S, Z, P, fin, n, i);
}

// The same for a chunk that took the per-token path (its weights are not in registers):
// the rescaled recursion in fp64 with k and v read again from memory.
template <int CH, Io F>
__device__ __forceinline__ void final_state_exact(const io_t<F> *__restrict__ k,
                                               const io_t<F> *__restrict__ v, int64_t row0,
                                               int64_t t0, int Lv, int64_t C, int cl,
                                               const Carry &mine, double w,
                                               float *__restrict__ fin, int64_t n, int64_t i) {
    double a = mine.a, b = mine.b, p = mine.P * kLn2D;
#pragma unroll 1
    for (int j = 0; j < Lv; ++j) {
        const int64_t x = (row0 + t0 + j) * C + cl;
        const double kk = (double)io_ld<F>(k, x), vv = (double)io_ld<F>(v, x);
        const double pw = p - w;
        const double m = fmax(pw, kk);
        const double f1 = exp(pw - m), f2 = exp(kk - m);
        a = fma(f1, a, f2 * vv);
        b = fma(f1, b, f2);
        p = m;
    }
    store_state(a, b, p * kLog2eD, fin, n, i);
}

// Window staging of chunk summaries (one per wave) for the in-window fold.
template <int NW>
struct FwdShared {
    double a[NW][64], b[NW][64], ap[NW][64], bp[NW][64], P[NW][64];
    int status[2];
    int depth;
};

template <int NW>
__device__ __forceinline__ void stage(FwdShared<NW> &sh, int q, int lane, const Carry &c) {
    sh.a[q][lane] = c.a;
    sh.b[q][lane] = c.b;
    sh.ap[q][lane] = c.ap;
    sh.bp[q][lane] = c.bp;
    sh.P[q][lane] = c.P;
}

template <int NW>
__device__ __forceinline__ Carry staged(const FwdShared<NW> &sh, int q, int lane) {
    return Carry{sh.a[q][lane], sh.b[q][lane], sh.ap[q][lane], sh.bp[q][lane], sh.P[q][lane]};
}

// Aggregate of window j (its NW chunk summaries folded from the empty state), for the
// look-back's recomputation of a window whose aggregate was not published in time. Called
// by all waves together (it contains barriers). Each wave streams its chunk from memory in
// a loop that is not unrolled, repeating chunk_summary's arithmetic op for op and in the
// same order (bitwise what unit j computes itself), so the unit's own chunk stays in
// registers.
template <int NW, int CH, Io F>
__device__ __forceinline__ Carry window_aggregate(FwdShared<NW> &sh, int64_t j, int q, int lane,
                                                  int64_t T, int64_t C, int64_t row0, int cl,
                                                  const io_t<F> *__restrict__ k,
                                                  const io_t<F> *__restrict__ v, bool slow_wave,
                                                  double dwfd, double wd, double cw2) {
    const int64_t tj = j * (NW * CH) + (int64_t)q * CH;
    const int Lj = chunk_len(tj, T, CH);
    Carry sj = carry_empty();
    if (Lj > 0) {
        const io_t<F> *kp = k + (row0 + tj) * C + cl;
        const io_t<F> *vp = v + (row0 + tj) * C + cl;
        float rj = kNegBig;
#pragma unroll 1
        for (int i = 0; i < Lj; ++i) rj = fmaxf(rj, io_ld<F>(kp, (int64_t)i * C));
        const double refd = (double)rj;
        sj.P = refd * kLog2eD;
        if (slow_wave) {
            sj = exact_summary<CH, F>(k, v, row0, tj, Lj, C, cl, rj, wd);
        } else {
            double S = 0.0, Z = 0.0, Qs = 0.0, Qz = 0.0;
#pragma unroll 1
            for (int i = 0; i < CH; ++i) {
                const bool in = i < Lj;
                const float ki = in ? io_ld<F>(kp, (int64_t)i * C) : -__builtin_inff();
                const double e = exp2_64(fma((double)ki, kLog2eD, -sj.P));
                const double vi = in ? (double)io_ld<F>(vp, (int64_t)i * C) : 0.0;
                Qs = fma(Qs, dwfd, S);
                Qz = fma(Qz, dwfd, Z);
                S = fma(S, dwfd, e * vi);
                Z = fma(Z, dwfd, e);
            }
            sj.a = S;
            sj.b = Z;
            sj.ap = dwfd * Qs;
            sj.bp = dwfd * Qz;
            if (wave_any(!(Z >= kTinySum)))
                sj = exact_summary<CH, F>(k, v, row0, tj, Lj, C, cl, rj, wd);
        }
    }
    __syncthreads();
    stage(sh, q, lane, sj);
    __syncthreads();
    Carry X = carry_empty();
#pragma unroll
    for (int qq = 0; qq < NW; ++qq) fold(X, staged(sh, qq, lane), cw2, (double)CH);
    __syncthreads();
    return X;
}

// The workspace stamp (see wkv_launch.h), written by one thread of the first unit; kept out of
// line so that it costs the kernel no registers.
__device__ __noinline__ void stamp_workspace(uint64_t *hdr, bool keep, int64_t B, int64_t T,
                                             int64_t C) {
    hdr[0] = kWsTag | (keep ? kWsKept : kWsInfer);
    hdr[1] = (uint64_t)B;
    hdr[2] = (uint64_t)T;
    hdr[3] = (uint64_t)C;
}

// GATE: the output is sigma(r) * y (r [B][T][C]) instead of y. F: the storage format of k,
// v, r and y. KEEP: the workspace keeps what the backward reads (the age-weighted fields of
// the records, the carry entering each window's second chunk and token 0); without it the
// records hold a, b, P only, and the sums they would have come from are never formed.
template <int NW, int CH, bool GATE, Io F, bool KEEP>
__global__ __launch_bounds__(NW * 64) void wkv_forward_kernel(
    int64_t T, int64_t C, int ngrp, int64_t nbg, int64_t nseg, uint64_t epoch, int tries,
    const float *__restrict__ w, const float *__restrict__ u, const io_t<F> *__restrict__ k,
    const io_t<F> *__restrict__ v, const io_t<F> *__restrict__ r, io_t<F> *__restrict__ y,
    uint64_t *__restrict__ flags,
    double *__restrict__ agg, double *__restrict__ incl, int64_t nrec, double *__restrict__ cin,
    const float *__restrict__ sa, const float *__restrict__ sb, const float *__restrict__ sp,
    double *__restrict__ init, float *__restrict__ fin, uint64_t *__restrict__ hdr,
    int64_t B) {
    constexpr int WIN = NW * CH;
    __shared__ FwdShared<NW> sh;

    const int lane = threadIdx.x & 63;
    const int q = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t s = (int64_t)blockIdx.x / nbg;
    const int64_t bg = (int64_t)blockIdx.x - s * nbg;
    const int64_t bidx = bg / ngrp;
    const int grp = (int)(bg - bidx * ngrp);
    const int64_t c = (int64_t)grp * 64 + lane;
    const bool cval = c < C;
    const int cl = (int)(cval ? c : C - 1);
    const int voff = cl * kIoBytes<F>;
    auto put_r = [&](double *base, int64_t i, const Carry &x) {
        if constexpr (KEEP)
            put_rec(base, nrec, i, x);
        else
            put_rec3(base, nrec, i, x);
    };
    auto get_r = [&](const double *base, int64_t i) {
        if constexpr (KEEP)
            return get_rec(base, nrec, i);
        else
            return get_rec3(base, nrec, i);
    };

    const float wc = w[cl];
    const float uc = u[cl];
    const Decay dc = make_decay(wc);
    const double wd = (double)wc;
    const double dwfd = exp(-wd);
    const float eu = expf(uc);
    const double cw2 = (double)CH * wd * kLog2eD;
    const double ww2 = (double)WIN * wd * kLog2eD;
    const bool slow_wave = wave_any(!(fabsf(uc) <= 60.0f));

    const int64_t row0 = bidx * T;
    const int64_t t0 = s * WIN + (int64_t)q * CH;
    const int Lv = chunk_len(t0, T, CH);

    // ---- phase 1: frame and summary of this wave's chunk ----
    float kc[CH], vc[CH];
    load_chunk<CH, F>(kc, vc, k, v, row0, t0, T, C, voff);
    const float ref = chunk_ref<CH>(kc, Lv);
    // for the outputs (phase 3); wave-uniform, so it holds no vector register meanwhile
    const bool faint = wave_any(chunk_has_faint_key<CH>(kc, Lv, ref));
    Carry sum;
    bool exact = chunk_summary<CH, false>(kc, vc, Lv, ref, slow_wave, dwfd, sum);
    if (exact) sum = exact_summary<CH, F>(k, v, row0, t0, Lv, C, cl, ref, wd);

    // ---- window: local carries and aggregate ----
    stage(sh, q, lane, sum);
    __syncthreads();
    Carry run = carry_empty();
    Carry lexcl = run;
#pragma unroll
    for (int qq = 0; qq < NW; ++qq) {
        if (qq == q) lexcl = run;
        fold(run, staged(sh, qq, lane), cw2, (double)CH);
    }
    const int64_t rec = (bidx * nseg + s) * C + cl;
    uint64_t *myflag = flags + s * nbg + bg;
    // the flags of the previous kPeekDepth windows are read before this unit's flag store,
    // so that one wait covers the aggregate's stores and those reads
    if (q == 0) {
        if (cval) put_r(agg, rec, run);
        uint64_t pk = 0;
        if (lane < kPeekDepth && lane < s) pk = peek_flag(myflag - (int64_t)(lane + 1) * nbg);
        put_flag(myflag, epoch, kAggregate);
        if (s > 0) {
            const int d = peek_depth(pk, epoch, lane, s);
            if (lane == 0) sh.depth = d;
        }
    }

    // ---- look-back: carry entering this window ----
    // Walk back to the nearest window whose inclusive carry is published (or the sequence
    // start), making sure every window in between has its aggregate in memory; then fold
    // those aggregates forward in order. The result is bitwise the sequential chain
    // incl[s] = fold(incl[s-1], agg[s]) whatever the timing, so every run is deterministic.
    // the carry before token 0: the empty carry, or the given state (A = a e^p)
    auto start_carry = [&]() {
        if (sa == nullptr) return carry_empty();
        const int64_t ic = bidx * C + cl;
        return Carry{(double)sa[ic], (double)sb[ic], 0.0, 0.0, (double)sp[ic] * kLog2eD};
    };
    Carry prefix = s == 0 ? start_carry() : carry_empty();
    if (s > 0) {
        __syncthreads();
        const int d = sh.depth;
        int64_t j = s - d;  // settled by the batch of peeks when d > 0
        if (d == 0) {
            j = s - 1;
            int it = 0;
            for (;;) {
                if (q == 0) {
                    const int st = poll_flag(flags + j * nbg + bg, epoch, tries);
                    if (lane == 0) sh.status[it & 1] = st;
                }
                __syncthreads();
                const int st = sh.status[it & 1];
                ++it;
                if (st == (int)kInclusive) break;
                if (st != (int)kAggregate) {
                    // not published in time: compute window j's aggregate here and publish
                    // it (bitwise what unit j itself publishes)
                    const Carry X = window_aggregate<NW, CH, F>(sh, j, q, lane, T, C, row0, cl, k,
                                                             v, slow_wave, dwfd, wd, cw2);
                    if (q == 0) {
                        if (cval) put_r(agg, (bidx * nseg + j) * C + cl, X);
                        raise_flag(flags + j * nbg + bg, epoch, kAggregate);
                    }
                }
                if (j == 0) {
                    j = -1;
                    break;
                }
                --j;
            }
        }
        // j is the window with a published inclusive carry, or -1; the records are read
        // two at a time so that their round trips overlap
        prefix = j >= 0 ? get_r(incl, (bidx * nseg + j) * C + cl) : start_carry();
        int64_t m = j + 1;
        for (; m + 1 < s; m += 2) {
            const Carry a0 = get_r(agg, (bidx * nseg + m) * C + cl);
            const Carry a1 = get_r(agg, (bidx * nseg + m + 1) * C + cl);
            prefix = follow(follow(prefix, a0, ww2, (double)WIN), a1, ww2, (double)WIN);
        }
        if (m < s)
            prefix = follow(prefix, get_r(agg, (bidx * nseg + m) * C + cl), ww2, (double)WIN);
    }
    // The inclusive record and its flag are published now, before the output sweep: a
    // successor that finds the flag stops its walk here. (Deferring the flag past the sweep,
    // so that the wait for the record's stores overlapped it, made the successors of shapes
    // with few units per window walk deeper: the long-context forward 121 -> 125 us, the
    // 3B-class forward 226 -> 230 us.)
    if (q == 0) {
        if (cval) put_r(incl, rec, follow(prefix, run, ww2, (double)WIN));
        put_flag(myflag, epoch, kInclusive);
    }
    // ---- the carry entering this wave's chunk, kept for the backward pass ----
    Carry mine = follow(prefix, lexcl, (double)(q * CH) * wd * kLog2eD, (double)(q * CH));
    normalize(mine);
    {
        // the carry entering each kCinChunk-token chunk of the window but its first (that
        // one is the previous window's inclusive carry) is kept
        constexpr int CPC = kCinChunk / CH;
        const int r = q / CPC;
        if (KEEP && Lv > 0 && cval && q % CPC == 0 && r > 0)
            put_cin(cin, nrec * kCinCarries, ((bidx * nseg + s) * kCinCarries + r - 1) * C + cl,
                    mine);
    }
    // the carry entering token 0 is kept too, as given (the backward's first chunk starts
    // from it, normalized; the gradient with respect to a given state needs its p)
    if (KEEP && s == 0 && q == 0 && cval) put_cin(init, nrec / nseg, bidx * C + cl, prefix);
    // the wave that holds token T-1 gives the state after it, when asked for
    if (fin != nullptr && t0 < T && T <= t0 + CH && cval) {
        if (exact)
            final_state_exact<CH, F>(k, v, row0, t0, Lv, C, cl, mine, wd, fin, nrec / nseg,
                                  bidx * C + cl);
        else
            final_state<CH>(kc, vc, Lv, ref, mine, dwfd, fin, nrec / nseg, bidx * C + cl);
    }
    // stamp the workspace with what this launch leaves in it (a backward checks it)
    if (blockIdx.x == 0 && threadIdx.x == 0) stamp_workspace(hdr, KEEP, B, T, C);
    if (y == nullptr || Lv == 0) return;

    // ---- phase 3: outputs ----
    const double ref2 = (double)ref * kLog2eD;
    float rc[GATE ? CH : 1];  // r of the chunk, loaded while the sweep runs
    if constexpr (GATE) {
        if (!exact) load_chunk1<CH, F>(rc, r, row0, t0, T, C, voff);
    }
    if (!exact) {
        const double gap = mine.P - ref2;
        bool bad = gap > (double)kCarryGap || faint;
        float dmin = __builtin_inff();
        const double s0 = exp2_64(gap);
        float Sx = (float)(mine.a * s0), Zx = (float)(mine.b * s0);
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const float e = kc[j], ev = e * vc[j];
            const float num = fmaf(eu, ev, Sx);
            const float den = fmaf(eu, e, Zx);
            dmin = fminf(dmin, den);  // padded tokens too: at worst a ragged last chunk
            kc[j] = num * rcpf(den);     // goes the per-token way (its decayed carry is tiny)
            Sx = fmaf(Sx, dc.dwf, ev);
            Zx = fmaf(Zx, dc.dwf, e);
        }
        exact = wave_any(bad || !(dmin >= kTinyDen));
    }
    if (exact) {
        if (cval)
            exact_outputs<CH, F>(k, v, GATE ? r : nullptr, y, row0, t0, Lv, C, cl, ref, mine, uc,
                                 wd);
        return;
    }
    if (cval) {
        const rsrc_t ry = make_rsrc(y + (row0 + t0) * C);
        const int stride = (int)(C * kIoBytes<F>);
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            if (j < Lv) {
                float o = kc[j];
                if constexpr (GATE) o *= sigmoidf_(rc[j]);
                bstore_io<F>(ry, o, voff, j * stride);
            }
        }
    }
}

// The state after the last token, from the forward's workspace into the caller's arrays.
__global__ __launch_bounds__(256) void wkv_state_out_kernel(const float *__restrict__ fin,
                                                            float *__restrict__ a,
                                                            float *__restrict__ b,
                                                            float *__restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) {
        a[i] = fin[i];
        b[i] = fin[n + i];
        p[i] = fin[2 * n + i];
    }
}

template <Io F, bool KEEP>
static void launch_forward_io(int64_t units, hipStream_t stream, int64_t T, int64_t C, int ngrp,
                              int64_t nbg, uint64_t epoch, const float *w, const float *u,
                              const void *k, const void *v, const void *r, void *y, float *sa,
                              float *sb, float *sp, float *fin, const FwdLayout &L, int64_t B) {
    const io_t<F> *kk = static_cast<const io_t<F> *>(k), *vv = static_cast<const io_t<F> *>(v),
                  *rr = static_cast<const io_t<F> *>(r);
    io_t<F> *yy = static_cast<io_t<F> *>(y);
    if (r != nullptr)
        hipLaunchKernelGGL((wkv_forward_kernel<kFwdWaves, kFwdChunk, true, F, KEEP>),
                           dim3((unsigned)units), dim3(kFwdWaves * 64), 0, stream, T, C, ngrp,
                           nbg, L.nseg, epoch, poll_limit(), w, u, kk, vv, rr, yy, L.flags, L.agg,
                           L.incl, B * L.nseg * C, L.cin, sa, sb, sp, L.init, fin, L.hdr, B);
    else
        hipLaunchKernelGGL((wkv_forward_kernel<kFwdWaves, kFwdChunk, false, F, KEEP>),
                           dim3((unsigned)units), dim3(kFwdWaves * 64), 0, stream, T, C, ngrp,
                           nbg, L.nseg, epoch, poll_limit(), w, u, kk, vv, rr, yy, L.flags, L.agg,
                           L.incl, B * L.nseg * C, L.cin, sa, sb, sp, L.init, fin, L.hdr, B);
}

template <Io F>
static void launch_forward_fmt(bool keep, int64_t units, hipStream_t stream, int64_t T,
                               int64_t C, int ngrp, int64_t nbg, uint64_t epoch, const float *w,
                               const float *u, const void *k, const void *v, const void *r,
                               void *y, float *sa, float *sb, float *sp, float *fin,
                               const FwdLayout &L, int64_t B) {
    if (keep)
        launch_forward_io<F, true>(units, stream, T, C, ngrp, nbg, epoch, w, u, k, v, r, y, sa, sb,
                                   sp, fin, L, B);
    else
        launch_forward_io<F, false>(units, stream, T, C, ngrp, nbg, epoch, w, u, k, v, r, y, sa,
                                    sb, sp, fin, L, B);
}

hipError_t launch_forward(int64_t B, int64_t T, int64_t C, Io fmt, const float *w,
                          const float *u, const void *k, const void *v, const void *r, void *y,
                          float *sa, float *sb, float *sp, const FwdLayout &L, uint64_t epoch,
                          bool keep, hipStream_t stream) {
    const int ngrp = (int)((C + 63) / 64);
    const int64_t nbg = B * ngrp;
    const int64_t units = nbg * L.nseg;
    float *fin = sa != nullptr ? L.fin : nullptr;
    if (fmt == Io::BF16)
        launch_forward_fmt<Io::BF16>(keep, units, stream, T, C, ngrp, nbg, epoch, w, u, k, v, r,
                                     y, sa, sb, sp, fin, L, B);
    else if (fmt == Io::F16)
        launch_forward_fmt<Io::F16>(keep, units, stream, T, C, ngrp, nbg, epoch, w, u, k, v, r, y,
                                    sa, sb, sp, fin, L, B);
    else
        launch_forward_fmt<Io::F32>(keep, units, stream, T, C, ngrp, nbg, epoch, w, u, k, v, r, y,
                                    sa, sb, sp, fin, L, B);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || sa == nullptr) return e;
    const int64_t n = B * C;
    hipLaunchKernelGGL(wkv_state_out_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       stream, L.fin, sa, sb, sp, n);
    return hipGetLastError();
}

}  // namespace wkvdev
