/*
 * wkv_oracle.c -- plain fp64 CPU oracle for the RWKV-4 time-mixing WKV operator.
 *
 * TEST INFRASTRUCTURE ONLY. It exists to check the GPU library, never to stand in
 * for it: only the test suite, the package smoke check and the CPU-baseline leg of
 * the benchmark may load it. It shares no code, header or constant with the GPU path.
 *
 * Operator (one batch row b, one channel c, 0-based time t; k, v: [B][T][C]; w, u: [C]):
 *
 *     logit_{t,i} = k_i - (t-1-i) * w      for i < t   (older tokens decay with distance)
 *     logit_{t,t} = u + k_t                            (bonus u on the current token)
 *     y_t         = sum_{i<=t} softmax_i(logit_{t,.}) * v_i
 *
 * i.e. y_t = (sum_{i<t} e^{-(t-1-i)w+k_i} v_i + e^{u+k_t} v_t)
 *          / (sum_{i<t} e^{-(t-1-i)w+k_i}     + e^{u+k_t}).
 *
 * Sources (the formula bodies of the first page were lost in extraction; the prose fixes
 * the structure):
 *   - "RWKV解读：在Transformer的时代的新RNN", section 二.3 "RWKV的网络架构", formula (8):
 *     the absolute-position bias of AFT is replaced by a relative-position decay with a
 *     single trained vector w, the current position gets its own parameter u, and (8) can
 *     be written in recursive form. Same section: W is channel-wise.
 *   - "RWKV についての調査記録", section 【wkvとは】: wkv is a weighted average of v with
 *     k-dependent weights, the current v gets a bonus u, past v decay the further back they
 *     are, one decay vector w is shared, all channels are computed independently.
 *   - same page, section "RWKVとは？": at inference RWKV runs as an RNN that takes a token
 *     and a state and returns the new state (the recurrent routines below).
 *   - same page, section "Trainingについて": the gradients of all parameters are computed
 *     (the backward routines below; w and u are per-channel parameters, so dw and du are
 *     summed over batch rows and time).
 *
 * Every routine takes fp64 arrays; callers upcast fp32 inputs exactly.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define IDX(b, t, c) (((int64_t)(b) * T + (t)) * C + (c))

int wkv_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------------------
 * 1. Direct O(T^2) forward: the definition written out. For every output position the
 *    logits of all contributing tokens are formed, their maximum is subtracted (which
 *    leaves the softmax unchanged) and the weighted average of v is taken.
 * ------------------------------------------------------------------------------- */
void wkv_oracle_forward_direct(int64_t B, int64_t T, int64_t C, const double *w,
                               const double *u, const double *k, const double *v,
                               double *y) {
    int64_t n = B * C;
#pragma omp parallel
    {
        double *lg = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
#pragma omp for schedule(static)
        for (int64_t bc = 0; bc < n; ++bc) {
            int64_t b = bc / C, c = bc % C;
            for (int64_t t = 0; t < T; ++t) {
                double mx = -INFINITY;
                for (int64_t i = 0; i <= t; ++i) {
                    double l = (i < t) ? k[IDX(b, i, c)] - (double)(t - 1 - i) * w[c]
                                       : u[c] + k[IDX(b, t, c)];
                    lg[i] = l;
                    if (l > mx) mx = l;
                }
                double num = 0.0, den = 0.0;
                for (int64_t i = 0; i <= t; ++i) {
                    double e = exp(lg[i] - mx);
                    num += e * v[IDX(b, i, c)];
                    den += e;
                }
                y[IDX(b, t, c)] = num / den;
            }
        }
        free(lg);
    }
}

/* ---------------------------------------------------------------------------------
 * 2. Plain recurrent forward (the recursive form of formula (8)), no rescaling:
 *        y_t     = (A + e^{u+k_t} v_t) / (Bs + e^{u+k_t})
 *        A      <- e^{-w} A  + e^{k_t} v_t
 *        Bs     <- e^{-w} Bs + e^{k_t}
 *    starting from A = Bs = 0. Valid while the exponentials stay inside fp64 range;
 *    returns 1 (and writes nothing) when max|k| + max|u| >= 600.
 * ------------------------------------------------------------------------------- */
static int range_ok(int64_t nk, const double *k, int64_t C, const double *u) {
    double mk = 0.0, mu = 0.0;
    for (int64_t i = 0; i < nk; ++i) {
        double a = fabs(k[i]);
        if (!(a <= 1e300)) return 0; /* inf / nan */
        if (a > mk) mk = a;
    }
    for (int64_t c = 0; c < C; ++c) {
        double a = fabs(u[c]);
        if (!(a <= 1e300)) return 0;
        if (a > mu) mu = a;
    }
    return mk + mu < 600.0;
}

int wkv_oracle_forward_recurrent(int64_t B, int64_t T, int64_t C, const double *w,
                                 const double *u, const double *k, const double *v,
                                 double *y) {
    if (!range_ok(B * T * C, k, C, u)) return 1;
    int64_t n = B * C;
#pragma omp parallel for schedule(static)
    for (int64_t bc = 0; bc < n; ++bc) {
        int64_t b = bc / C, c = bc % C;
        double decay = exp(-w[c]);
        double A = 0.0, Bs = 0.0;
        for (int64_t t = 0; t < T; ++t) {
            double kk = k[IDX(b, t, c)], vv = v[IDX(b, t, c)];
            double cur = exp(u[c] + kk);
            y[IDX(b, t, c)] = (A + cur * vv) / (Bs + cur);
            double ek = exp(kk);
            A = decay * A + ek * vv;
            Bs = decay * Bs + ek;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------------
 * 3. Rescaled recurrent forward with an explicit state (a, b, p), meaning
 *        A = a e^p,  Bs = b e^p
 *    so that no exponential argument is positive and any finite k is safe:
 *        m  = max(p, u+k_t);          y_t = (e^{p-m} a + e^{u+k_t-m} v_t)
 *                                          / (e^{p-m} b + e^{u+k_t-m})
 *        m' = max(p-w, k_t);          a <- e^{p-w-m'} a + e^{k_t-m'} v_t
 *                                     b <- e^{p-w-m'} b + e^{k_t-m'};  p <- m'
 *    The state arrays ([B][C]) are read as the initial state and overwritten with the
 *    final one; pass NULL for all three to start from the empty state (a = b = 0,
 *    p = -1e38) and discard the final state. With T = 1 this is one decode step.
 * ------------------------------------------------------------------------------- */
void wkv_oracle_forward_rescaled(int64_t B, int64_t T, int64_t C, const double *w,
                                 const double *u, const double *k, const double *v,
                                 double *y, double *sa, double *sb, double *sp) {
    int64_t n = B * C;
#pragma omp parallel for schedule(static)
    for (int64_t bc = 0; bc < n; ++bc) {
        int64_t b = bc / C, c = bc % C;
        double a = 0.0, bb = 0.0, p = -1e38;
        if (sa) {
            a = sa[bc];
            bb = sb[bc];
            p = sp[bc];
        }
        for (int64_t t = 0; t < T; ++t) {
            double kk = k[IDX(b, t, c)], vv = v[IDX(b, t, c)];
            double uk = u[c] + kk;
            double m = p > uk ? p : uk;
            double e1 = exp(p - m), e2 = exp(uk - m);
            y[IDX(b, t, c)] = (e1 * a + e2 * vv) / (e1 * bb + e2);
            double pw = p - w[c];
            double m2 = pw > kk ? pw : kk;
            double f1 = exp(pw - m2), f2 = exp(kk - m2);
            a = f1 * a + f2 * vv;
            bb = f1 * bb + f2;
            p = m2;
        }
        if (sa) {
            sa[bc] = a;
            sb[bc] = bb;
            sp[bc] = p;
        }
    }
}

/* One decode step for B sequences: the recurrent form applied to a single token, the
 * state updated in place, y [B][C] computed from the state before the update. */
void wkv_oracle_decode_step(int64_t B, int64_t C, const double *w, const double *u,
                            const double *k, const double *v, double *sa, double *sb,
                            double *sp, double *y) {
    wkv_oracle_forward_rescaled(B, 1, C, w, u, k, v, y, sa, sb, sp);
}

/* ---------------------------------------------------------------------------------
 * 4. Direct O(T^2) backward of L = sum_t dy_t * y_t, from the softmax form.
 *    With P_{t,i} = softmax_i(logit_{t,.}) and g = dy:
 *        dy_t/dlogit_{t,i} = P_{t,i} (v_i - y_t),   dy_t/dv_i = P_{t,i}
 *        dlogit_{t,i}/dk_i = 1,  dlogit_{t,t}/du = 1,  dlogit_{t,i}/dw = -(t-1-i) (i<t)
 *    so
 *        dv_i = sum_{t>=i} g_t P_{t,i}
 *        dk_i = sum_{t>=i} g_t P_{t,i} (v_i - y_t)
 *        du   = sum_{b,t} g_t P_{t,t} (v_t - y_t)
 *        dw   = -sum_{b,t} sum_{i<t} (t-1-i) g_t P_{t,i} (v_i - y_t)
 *    dw and du ([C]) are summed over b in a fixed order.
 * ------------------------------------------------------------------------------- */
void wkv_oracle_backward_direct(int64_t B, int64_t T, int64_t C, const double *w,
                                const double *u, const double *k, const double *v,
                                const double *dy, double *dk, double *dv, double *dw,
                                double *du) {
    int64_t n = B * C;
    double *pw = (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
    double *pu = (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
#pragma omp parallel
    {
        double *lg = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
#pragma omp for schedule(static)
        for (int64_t bc = 0; bc < n; ++bc) {
            int64_t b = bc / C, c = bc % C;
            for (int64_t t = 0; t < T; ++t) {
                dk[IDX(b, t, c)] = 0.0;
                dv[IDX(b, t, c)] = 0.0;
            }
            double sw = 0.0, su = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                double mx = -INFINITY;
                for (int64_t i = 0; i <= t; ++i) {
                    double l = (i < t) ? k[IDX(b, i, c)] - (double)(t - 1 - i) * w[c]
                                       : u[c] + k[IDX(b, t, c)];
                    lg[i] = l;
                    if (l > mx) mx = l;
                }
                double den = 0.0, num = 0.0;
                for (int64_t i = 0; i <= t; ++i) {
                    lg[i] = exp(lg[i] - mx);
                    den += lg[i];
                    num += lg[i] * v[IDX(b, i, c)];
                }
                double yt = num / den, g = dy[IDX(b, t, c)];
                for (int64_t i = 0; i <= t; ++i) {
                    double P = lg[i] / den;
                    double vi = v[IDX(b, i, c)];
                    dv[IDX(b, i, c)] += g * P;
                    dk[IDX(b, i, c)] += g * P * (vi - yt);
                    if (i < t)
                        sw -= (double)(t - 1 - i) * g * P * (vi - yt);
                    else
                        su += g * P * (vi - yt);
                }
            }
            pw[bc] = sw;
            pu[bc] = su;
        }
        free(lg);
    }
    for (int64_t c = 0; c < C; ++c) {
        double sw = 0.0, su = 0.0;
        for (int64_t b = 0; b < B; ++b) {
            sw += pw[b * C + c];
            su += pu[b * C + c];
        }
        dw[c] = sw;
        du[c] = su;
    }
    free(pw);
    free(pu);
}

/* ---------------------------------------------------------------------------------
 * 5. Linear-time backward with plain (unscaled) fp64 carries.
 *    Forward sweep, with D_t = Bs_t + e^{u+k_t} and s_t = g_t / D_t:
 *        du += s_t e^{u+k_t} (v_t - y_t)
 *        dw -= s_t (A'_t - y_t B'_t)
 *    where A'_t = sum_{i<t} (t-1-i) e^{-(t-1-i)w+k_i} v_i (B'_t likewise without v),
 *    updated as A' <- e^{-w} (A' + A) before A itself is advanced.
 *    Reverse sweep, with G_i = sum_{t>i} e^{-(t-1-i)w} s_t and H_i the same with s_t y_t:
 *        dv_i = s_i e^{u+k_i} + e^{k_i} G_i
 *        dk_i = s_i e^{u+k_i} (v_i - y_i) + e^{k_i} (v_i G_i - H_i)
 *        G_{i-1} = e^{-w} G_i + s_i,   H_{i-1} = e^{-w} H_i + s_i y_i.
 *    Returns 1 (and writes nothing) when max|k| + max|u| >= 600.
 * ------------------------------------------------------------------------------- */
int wkv_oracle_backward_recurrent(int64_t B, int64_t T, int64_t C, const double *w,
                                  const double *u, const double *k, const double *v,
                                  const double *dy, double *dk, double *dv, double *dw,
                                  double *du) {
    if (!range_ok(B * T * C, k, C, u)) return 1;
    int64_t n = B * C;
    double *pw = (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
    double *pu = (double *)calloc((size_t)(n > 0 ? n : 1), sizeof(double));
#pragma omp parallel
    {
        double *ys = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
        double *ss = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
#pragma omp for schedule(static)
        for (int64_t bc = 0; bc < n; ++bc) {
            int64_t b = bc / C, c = bc % C;
            double decay = exp(-w[c]);
            double A = 0.0, Bs = 0.0, Ap = 0.0, Bp = 0.0, sw = 0.0, su = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                double kk = k[IDX(b, t, c)], vv = v[IDX(b, t, c)];
                double cur = exp(u[c] + kk);
                double D = Bs + cur;
                double yt = (A + cur * vv) / D;
                double s = dy[IDX(b, t, c)] / D;
                ys[t] = yt;
                ss[t] = s;
                su += s * cur * (vv - yt);
                sw -= s * (Ap - yt * Bp);
                Ap = decay * (Ap + A);
                Bp = decay * (Bp + Bs);
                double ek = exp(kk);
                A = decay * A + ek * vv;
                Bs = decay * Bs + ek;
            }
            double G = 0.0, H = 0.0;
            for (int64_t i = T - 1; i >= 0; --i) {
                double kk = k[IDX(b, i, c)], vv = v[IDX(b, i, c)];
                double cur = exp(u[c] + kk), ek = exp(kk);
                dv[IDX(b, i, c)] = ss[i] * cur + ek * G;
                dk[IDX(b, i, c)] = ss[i] * cur * (vv - ys[i]) + ek * (vv * G - H);
                G = decay * G + ss[i];
                H = decay * H + ss[i] * ys[i];
            }
            pw[bc] = sw;
            pu[bc] = su;
        }
        free(ys);
        free(ss);
    }
    for (int64_t c = 0; c < C; ++c) {
        double sw = 0.0, su = 0.0;
        for (int64_t b = 0; b < B; ++b) {
            sw += pw[b * C + c];
            su += pu[b * C + c];
        }
        dw[c] = sw;
        du[c] = su;
    }
    free(pw);
    free(pu);
    return 0;
}
