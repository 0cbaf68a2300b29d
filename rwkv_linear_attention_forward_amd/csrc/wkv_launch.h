// wkv_launch.h -- kernel launchers and workspace layouts behind the C ABI (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkvdev {

// Forward geometry: a unit is 64 channels x one window of kFwdWaves * kFwdChunk tokens.
constexpr int kFwdWaves = 4;
constexpr int kFwdChunk = 32;
constexpr int kFwdWindow = kFwdWaves * kFwdChunk;

// Publication status of a unit (low 2 bits of its flag; the high bits hold the call epoch).
constexpr uint64_t kAggregate = 1;
constexpr uint64_t kInclusive = 2;
constexpr int kPollTries = 2000;  // bounded wait before a missing aggregate is recomputed

// A carry or window summary as published: A = a 2^P, B = b 2^P and the age-weighted
// A' = a' 2^P, B' = b' 2^P (fp64 bits each).
struct Rec {
    uint64_t a, b, ap, bp;
    uint64_t P;
};

// Forward workspace, carved out of the caller's buffer (see wkv_api.hip):
//   flags[nseg][B * ngrp]   uint64 publication flags
//   agg[B][nseg][C]         window aggregates (from the empty state)
//   incl[B][nseg][C]        inclusive carries: the state after window s, i.e. entering s+1
//   cin[5][B][nchunk][C]    the carry entering every kFwdChunk-token chunk, normalized,
//                           one fp64 array per field (a, b, a', b', P) so that a wave's
//                           64 channels read and write 512 contiguous bytes per field;
//                           the backward pass starts each of its chunks from these.
struct FwdLayout {
    int64_t nseg;
    int64_t nchunk;
    uint64_t *flags;
    Rec *agg;
    Rec *incl;
    double *cin;
};

// A reverse carry or reverse window summary as published: the future sums
//   G = sum_{t>=t0} e^{-(t-t0)w} s_t,  H = same with s_t y_t
// (s_t = dy_t / D_t), held as (g, h) 2^r (fp64 bits each).
struct RevRec {
    uint64_t g, h;
    uint64_t r;
};

// Backward geometry: a unit is 64 channels x kBwdWaves chunks of kFwdChunk tokens (the
// chunks must coincide with the forward's, whose entering carries they start from).
constexpr int kBwdWaves = 4;
constexpr int kBwdWindow = kBwdWaves * kFwdChunk;

// Backward workspace:
//   flags[nseg][B * ngrp]    uint64 publication flags (reverse direction)
//   ragg[B][nseg][C]         reverse window aggregates (from a zero future)
//   rincl[B][nseg][C]        reverse inclusive carries: the future sums entering window s
//   part[B][nseg][C][2]      per-window dw, du partials (fp64)
//   ctr[ngrp]                per channel group: arrivals of this call's units, tagged with
//                            the call epoch; the last unit to arrive sums the partials
struct BwdLayout {
    int64_t nseg;
    uint64_t *flags;
    RevRec *ragg;
    RevRec *rincl;
    uint64_t *part;  // fp64 bits
    uint64_t *ctr;
};

// Units per channel group (B * nseg) must fit the arrival counter's 24-bit count.
constexpr int kCountBits = 24;

hipError_t launch_forward(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                          const float *k, const float *v, float *y, const FwdLayout &L,
                          uint64_t epoch, hipStream_t stream);

// `F` is the forward workspace filled for the same inputs (its chunk carries are read).
hipError_t launch_backward(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                           const float *k, const float *v, const float *dy, const FwdLayout &F,
                           float *dk, float *dv, float *dw, float *du, const BwdLayout &L,
                           uint64_t epoch, hipStream_t stream);

// dw = du = 0 over C channels (backward of an empty batch or sequence).
hipError_t launch_zero2(float *dw, float *du, int64_t C, hipStream_t stream);

hipError_t launch_decode(int64_t B, int64_t C, const float *w, const float *u, const float *k,
                         const float *v, float *a, float *b, float *p, float *y,
                         hipStream_t stream);

}  // namespace wkvdev
