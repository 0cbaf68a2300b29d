// wkv_launch.h -- kernel launchers and workspace layouts behind the C ABI (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkvdev {

// Storage formats of the [B][T][C] tensors at the boundary (the state and all arithmetic
// stay fp32/fp64 whatever the format).
enum class Io { F32, BF16, F16 };

// Forward geometry: a unit is 64 channels x one window of kFwdWaves * kFwdChunk tokens.
constexpr int kFwdWaves = 2;
constexpr int kFwdChunk = 32;
constexpr int kFwdWindow = kFwdWaves * kFwdChunk;

// The backward starts each kCinChunk-token chunk from the forward carry entering it: a
// chunk that opens a forward window starts from the previous window's inclusive carry
// (published anyway), the other kCinCarries chunks of a window from a carry the forward
// keeps for them.
constexpr int kCinChunk = 32;
static_assert(kCinChunk % kFwdChunk == 0 && kFwdWindow % kCinChunk == 0,
              "carry chunks must be whole forward chunks and tile the forward window");
constexpr int kCinCarries = kFwdWindow / kCinChunk - 1;

// Publication status of a unit (low 2 bits of its flag; the high bits hold the call epoch).
constexpr uint64_t kAggregate = 1;
constexpr uint64_t kInclusive = 2;
constexpr int kPollTries = 2000;  // bounded wait before a missing aggregate is recomputed

// The polls of a predecessor's flag a look-back makes before it recomputes that window's
// aggregate itself (kPollTries unless changed through wkv_set_poll_limit).
int poll_limit();

// Published carries and summaries are stored one fp64 array per field (field f of
// record i at f * n + i, n records), so that a wave's 64 channels write and read 512
// contiguous bytes per field. A forward record has the fields (a, b, a', b', P):
// A = a 2^P, B = b 2^P and the age-weighted A' = a' 2^P, B' = b' 2^P.
constexpr int kRecFields = 5;

// Forward workspace, carved out of the caller's buffer (see wkv_api.hip):
//   hdr[32]                 uint64 stamp written by the forward that filled it:
//                           hdr[0] = kWsTag | kWsKept (states kept for a backward) or
//                           kWsTag | kWsInfer (inference: nothing kept), hdr[1..3] = B, T, C
//   flags[nseg][B * ngrp]   uint64 publication flags
//   agg[5][B][nseg][C]      window aggregates (from the empty state)
//   incl[5][B][nseg][C]     inclusive carries: the state after window s, i.e. entering s+1
//   cin[5][B][nseg][kCinCarries][C]  the carry entering each kCinChunk-token chunk of a
//                           window but its first, normalized, one fp64 array per field
//                           (a, b, a', b', P) so that a wave's 64 channels read and write
//                           512 contiguous bytes per field.
//   init[5][B][C]           the carry entering token 0 as the forward used it (normalized)
//   fin[3][B][C]            fp32 state (a, b, p) after the last token, when one is asked for
// A forward that keeps nothing for a backward and takes no state (the plain wkv_forward)
// needs only the stamp, the flags and agg, incl with three fields each (a, b, P): the
// compact scan layout (cin, init, fin null).
constexpr uint64_t kWsTag = 0x574b5657534b0000ull;  // "WKVWSK" in the high bytes
constexpr uint64_t kWsKept = 1;
constexpr uint64_t kWsInfer = 2;
constexpr size_t kWsHeaderBytes = 256;
struct FwdLayout {
    int64_t nseg;
    uint64_t *hdr;
    uint64_t *flags;
    double *agg;
    double *incl;
    double *cin;
    double *init;
    float *fin;
};

// A reverse record has the fields (g, h, r): the future sums
//   G = sum_{t>=t0} e^{-(t-t0)w} s_t,  H = same with s_t y_t   (s_t = dy_t / D_t)
// held as (g, h) 2^r.
constexpr int kRevFields = 3;

// Backward geometry: a unit is 64 channels x kBwdWaves chunks of kCinChunk tokens (each
// starts from the carry the forward kept for it).
constexpr int kBwdWaves = 2;
constexpr int kBwdWindow = kBwdWaves * kCinChunk;

// Backward workspace:
//   flags[nseg][B * ngrp]    uint64 publication flags (reverse direction)
//   ragg[3][B][nseg][C]      reverse window aggregates (from a zero future)
//   rincl[3][B][nseg][C]     reverse inclusive carries: the future sums entering window s
//   part[2][B][nseg][C]      per-window dw, du partials (fp64), summed by a second kernel
//   tail[3][B][C]            the future sums beyond the last window, when the final state
//                            has a cotangent (otherwise unused: that future is zero)
struct BwdLayout {
    int64_t nseg;
    uint64_t *flags;
    double *ragg;
    double *rincl;
    double *part;
    double *tail;
};

// `sa`, `sb`, `sp` ([B][C], all three or none) hold the state before token 0 in the decode
// convention (A = a e^p, B = b e^p); when given, they are overwritten with the state after
// token T-1 (through L.fin, by a second kernel, so that no workgroup can read a state that
// another has already replaced). Without them the scan starts from the empty state.
// `r` ([B][T][C]) or null: with it the output is sigma(r) * y, the receptance gate. k, v, r
// and y are in storage format `fmt` (the state sa, sb, sp stays fp32). `keep`: the workspace
// is left with the states the backward reads (otherwise only what the scan itself needs).
hipError_t launch_forward(int64_t B, int64_t T, int64_t C, Io fmt, const float *w,
                          const float *u, const void *k, const void *v, const void *r, void *y,
                          float *sa, float *sb, float *sp, const FwdLayout &L, uint64_t epoch,
                          bool keep, hipStream_t stream);

// `F` is the forward workspace filled for the same inputs (its chunk carries are read).
// With `r` (and `dr`) the forward output was sigma(r) * y and `dy` is its cotangent. k, v,
// dy, r, dk, dv, dr are in storage format `fmt`; dw, du are fp32.
// With `ga`, `gb`, `gp` ([B][C], all three or none) it also gives the gradient with respect
// to the state (a, b, p) the forward started from (F's record of the carry before token 0).
// With `dfa`, `dfb` ([B][C] fp32, both or none) L also has the terms
// dfa * a_T + dfb * b_T of the final state F.fin the forward returned (p_T held fixed).
hipError_t launch_backward(int64_t B, int64_t T, int64_t C, Io fmt, const float *w,
                           const float *u, const void *k, const void *v, const void *dy,
                           const void *r, const FwdLayout &F, void *dk, void *dv, void *dr,
                           float *dw, float *du, float *ga, float *gb, float *gp,
                           const float *dfa, const float *dfb, const BwdLayout &L,
                           uint64_t epoch, hipStream_t stream);

// dw = du = 0 over C channels (backward of an empty batch or sequence).
hipError_t launch_zero2(float *dw, float *du, int64_t C, hipStream_t stream);

// Token-shift mix (out_m = mu_m x[t] + (1 - mu_m) x[t-1], m = r, k, v) and its backward;
// `part` holds 3 * B * shift_chunks(T) * C fp64 partials of dmu.
int64_t shift_chunks(int64_t T);
hipError_t launch_shift(int64_t B, int64_t T, int64_t C, const float *x, const float *x_prev,
                        const float *mu, float *o_r, float *o_k, float *o_v, float *x_last,
                        hipStream_t stream);
hipError_t launch_shift_backward(int64_t B, int64_t T, int64_t C, const float *x,
                                 const float *x_prev, const float *mu, const float *d_r,
                                 const float *d_k, const float *d_v, float *dx, float *dx_prev,
                                 float *dmu, double *part, hipStream_t stream);

// k, v, y ([B][C]) in storage format `fmt`; the state a, b, p stays fp32.
hipError_t launch_decode(int64_t B, int64_t C, Io fmt, const float *w, const float *u,
                         const void *k, const void *v, float *a, float *b, float *p, void *y,
                         hipStream_t stream);

}  // namespace wkvdev
