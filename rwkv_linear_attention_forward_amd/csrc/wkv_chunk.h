// wkv_chunk.h -- chunk-level device helpers shared by the forward and backward kernels:
// streaming a lane's CH-token chunk, the chunk frame and forward summary, and publishing
// and reading per-window records between workgroups (device scope).
#pragma once

#include "wkv_device.h"
#include "wkv_launch.h"

namespace wkvdev {

// Load a CH-token chunk of one lane's channel starting at token t0. Tokens past T are
// padding: k = -inf (weight e^{k - ref} = 0 in every frame), v = 0. The loads carry no
// branches (a padded token re-reads the last valid row), so the unrolled chunk stays in
// straight-line code.
template <int CH, Io F = Io::F32>
__device__ __forceinline__ void load_chunk(float (&kc)[CH], float (&vc)[CH],
                                           const io_t<F> *__restrict__ k,
                                           const io_t<F> *__restrict__ v, int64_t row0,
                                           int64_t t0, int64_t T, int64_t C, int voff) {
    if (t0 >= T) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            kc[j] = -__builtin_inff();
            vc[j] = 0.0f;
        }
        return;
    }
    const rsrc_t rk = make_rsrc(k + (row0 + t0) * C);
    const rsrc_t rv = make_rsrc(v + (row0 + t0) * C);
    const int stride = (int)(C * kIoBytes<F>);
    const int last = (int)(T - t0 < CH ? T - t0 : CH) - 1;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const int soff = (j < last ? j : last) * stride;
        kc[j] = bload_io<F>(rk, voff, soff);
        vc[j] = bload_io<F>(rv, voff, soff);
    }
    if (last < CH - 1) {
#pragma unroll
        for (int j = 1; j < CH; ++j) {
            if (j > last) {
                kc[j] = -__builtin_inff();
                vc[j] = 0.0f;
            }
        }
    }
}

// Summary of one lane's chunk from the empty state, in the chunk frame: with
// ref = max_j k_j and e_j = 2^{(k_j - ref) log2 e} <= 1 (fp64), the sums A, B, A', B'
// after the CH tokens, at scale 2^{ref log2 e}. Horner from the first token,
//   A_{j+1} = d A_j + e_j v_j   (d = e^{-w}),
// and A' = d dA/dd by the derivative recursion Q_{j+1} = d Q_j + A_j, A' = d Q (one fused
// multiply-add per token; A'_{j+1} = d (A'_j + A_j) term by term). B, B' alike.
// Padded tokens (k = -inf) have e_j = 0. Unless KEEPK, kc receives e_j rounded to fp32
// (for outputs that need only fp32). Returns true (wave-uniform) if the exact form is
// needed instead (forced, or the fp64 sums would underflow for some lane, which takes keys
// some 600 apart within one chunk); the caller then uses exact_summary.
template <int CH, bool KEEPK>
__device__ __forceinline__ bool chunk_summary(float (&kc)[CH], const float (&vc)[CH], int Lv,
                                              float ref, bool force_exact, double dwf,
                                              Carry &sum) {
    const double refd = (double)ref;
    const double ref2 = refd * kLog2eD;
    sum = Carry{0.0, 0.0, 0.0, 0.0, ref2};
    if (Lv == 0) {
        sum.P = kNegBigD;
        return false;
    }
    if (force_exact) return true;
    double S = 0.0, Z = 0.0, Qs = 0.0, Qz = 0.0;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
        const double e = exp2_64(fma((double)kc[j], kLog2eD, -ref2));
        if (!KEEPK) kc[j] = (float)e;
        Qs = fma(Qs, dwf, S);
        Qz = fma(Qz, dwf, Z);
        S = fma(S, dwf, e * (double)vc[j]);
        Z = fma(Z, dwf, e);
    }
    sum.a = S;
    sum.b = Z;
    sum.ap = dwf * Qs;
    sum.bp = dwf * Qz;
    return wave_any(!(Z >= kTinySum));
}

// Load one tensor's CH-token chunk (tokens past T are 0), branch-free as load_chunk.
template <int CH, Io F = Io::F32>
__device__ __forceinline__ void load_chunk1(float (&gc)[CH], const io_t<F> *__restrict__ g,
                                            int64_t row0, int64_t t0, int64_t T, int64_t C,
                                            int voff) {
    if (t0 >= T) {
#pragma unroll
        for (int j = 0; j < CH; ++j) gc[j] = 0.0f;
        return;
    }
    const rsrc_t rg = make_rsrc(g + (row0 + t0) * C);
    const int stride = (int)(C * kIoBytes<F>);
    const int last = (int)(T - t0 < CH ? T - t0 : CH) - 1;
#pragma unroll
    for (int j = 0; j < CH; ++j) gc[j] = bload_io<F>(rg, voff, (j < last ? j : last) * stride);
    if (last < CH - 1) {
#pragma unroll
        for (int j = 1; j < CH; ++j)
            if (j > last) gc[j] = 0.0f;
    }
}

// Load one tensor's CH-token chunk straight into LDS: row j of `dst` ([CH][64] dwords, the
// wave's own) gets token j's value of each lane's channel (a 16-bit format zero-extended in
// the low half), tokens past the Lv valid ones repeating the last valid row. No registers
// hold the data; lds_load_fence() must come before `dst` is read.
template <int CH, Io F>
__device__ __forceinline__ void load_chunk_lds(float (*dst)[64], const io_t<F> *__restrict__ g,
                                               int64_t row0, int64_t t0, int Lv, int64_t C,
                                               int voff) {
    const rsrc_t rg = make_rsrc(g + (row0 + t0) * C);
    const int stride = (int)(C * kIoBytes<F>);
#pragma unroll
    for (int j = 0; j < CH; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rg, (__attribute__((address_space(3))) void *)dst[j], kIoBytes<F>, voff,
            (j < Lv ? j : Lv - 1) * stride, 0, 2);
}
// Wait for this wave's direct-to-LDS loads (and every other load it has in flight).
__device__ __forceinline__ void lds_load_fence() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
// A value that load_chunk_lds left in a dword, widened to fp32.
template <Io F>
__device__ __forceinline__ float lds_widen(float x) {
    if constexpr (F == Io::F32) {
        return x;
    } else if constexpr (F == Io::BF16) {
        return __builtin_bit_cast(float, __builtin_bit_cast(unsigned, x) << 16);
    } else {
        return (float)__builtin_bit_cast(_Float16,
                                         (unsigned short)(__builtin_bit_cast(unsigned, x)));
    }
}

// Valid tokens of the chunk starting at t0.
__device__ __forceinline__ int chunk_len(int64_t t0, int64_t T, int CH) {
    return (int)(t0 >= T ? 0 : (T - t0 < CH ? T - t0 : CH));
}

// Per-token rescaled state in fp64, natural log-scale relative to the chunk frame e^{ref}:
// A = a e^p, B = b e^p, A' = a' e^p, B' = b' e^p. Used where the fixed frame would under-
// or overflow. Its sums feed carries and the gradients, which need the weights
// e^{k_i - ...} to agree with one another to far better than fp32 (dw cancels heavily),
// hence fp64 throughout.
struct Rs64 {
    double a, b, ap, bp, p;
};

// Advance by token (kr = k - ref, v): A' <- e^{-w} (A' + A), A <- e^{-w} A + e^{kr} v, and
// B', B alike. The larger of p - w and kr becomes the new scale.
__device__ __forceinline__ void rs64_push(Rs64 &s, double kr, double v, double w) {
    const double pw = s.p - w;
    const double m = fmax(pw, kr);
    const double f1 = exp(pw - m), f2 = exp(kr - m);
    s.ap = (s.ap + s.a) * f1;
    s.bp = (s.bp + s.b) * f1;
    s.a = fma(f1, s.a, f2 * v);
    s.b = fma(f1, s.b, f2);
    s.p = m;
}

// A token past the sequence end: decay only.
__device__ __forceinline__ void rs64_skip(Rs64 &s, double w) {
    s.ap += s.a;
    s.bp += s.b;
    s.p -= w;
}

// Chunk summary in the per-token form (fp64), same meaning as chunk_summary's, for the
// rare chunks the fixed frame cannot take. Reads k, v straight from memory in a loop that
// is not unrolled: few registers wherever it is inlined.
template <int CH, Io F = Io::F32>
__device__ __forceinline__ Carry exact_summary(const io_t<F> *__restrict__ k,
                                            const io_t<F> *__restrict__ v, int64_t row0,
                                            int64_t t0, int Lv, int64_t C, int cl, float ref,
                                            double w) {
    const double refd = (double)ref;
    Rs64 s{0.0, 0.0, 0.0, 0.0, kNegBigD};
#pragma unroll 1
    for (int j = 0; j < CH; ++j) {
        if (j < Lv) {
            const int64_t i = (row0 + t0 + j) * C + cl;
            rs64_push(s, (double)io_ld<F>(k, i) - refd, (double)io_ld<F>(v, i), w);
        } else {
            rs64_skip(s, w);
        }
    }
    // A = a e^{p + ref}; the carry scale is base 2: 2^{P} = e^{p + ref}
    return Carry{s.a, s.b, s.ap, s.bp, (s.p + refd) * kLog2eD};
}

// Frame of a chunk: its largest key (padding is -inf; a chunk of padding only gets kNegBig).
template <int CH>
__device__ __forceinline__ float chunk_ref(const float (&kc)[CH], int Lv) {
    float ref = kNegBig;
#pragma unroll
    for (int j = 0; j < CH; ++j) ref = fmaxf(ref, kc[j]);
    return ref;
}

// True when some valid key of the chunk lies more than 87 below the chunk's largest (ref):
// its in-frame weight e^{k - ref} is then below the fp32 normal range and would carry only a
// few significant bits in the fp32 sweeps, which matters where a large bonus e^u lifts it
// into the denominator. Such chunks take the per-token path (the test is per chunk, ahead of
// the sweeps, so it costs the unrolled loops nothing).
template <int CH>
__device__ __forceinline__ bool chunk_has_faint_key(const float (&kc)[CH], int Lv, float ref) {
    float kmin = __builtin_inff();
#pragma unroll
    for (int j = 0; j < CH; ++j) kmin = j < Lv ? fminf(kmin, kc[j]) : kmin;
    return ref - kmin > kFaintGap;
}

// ---- publication records (device-scope, see wkv_launch.h for the layout) ----
// Everything one workgroup publishes for another (records, flags, partials) is written
// and read only with device-scope atomic loads and stores (sc1: coherent across the XCDs'
// separate L2 caches without flushing them). Ordering is explicit: a producer waits for
// its record stores to complete before it stores the flag (publish_fence), and a consumer
// issues its record loads only after the flag value it polled has returned. A C++
// release/acquire would instead write back or invalidate the whole L2 of the XCD
// (buffer_wbl2 / buffer_inv), which costs microseconds per publication here.
__device__ __forceinline__ void publish_fence() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void consume_fence() { asm volatile("" ::: "memory"); }
__device__ __forceinline__ void put_u64(double *p, double x) {
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), __builtin_bit_cast(uint64_t, x),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double get_u64(const double *p) {
    return __builtin_bit_cast(double, __hip_atomic_load(reinterpret_cast<const uint64_t *>(p),
                                                        __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT));
}
// Forward record i of n (fields a, b, a', b', P at stride n).
__device__ __forceinline__ void put_rec(double *r, int64_t n, int64_t i, const Carry &c) {
    put_u64(r + i, c.a);
    put_u64(r + n + i, c.b);
    put_u64(r + 2 * n + i, c.ap);
    put_u64(r + 3 * n + i, c.bp);
    put_u64(r + 4 * n + i, c.P);
}
__device__ __forceinline__ Carry get_rec(const double *r, int64_t n, int64_t i) {
    return Carry{get_u64(r + i), get_u64(r + n + i), get_u64(r + 2 * n + i),
                 get_u64(r + 3 * n + i), get_u64(r + 4 * n + i)};
}
// The same records without the age-weighted fields, for a forward whose states no backward
// will use: a, b and P in the first three field slots (a', b' read back as 0), so that such
// a forward's record arrays need only 3 * n doubles each.
__device__ __forceinline__ void put_rec3(double *r, int64_t n, int64_t i, const Carry &c) {
    put_u64(r + i, c.a);
    put_u64(r + n + i, c.b);
    put_u64(r + 2 * n + i, c.P);
}
__device__ __forceinline__ Carry get_rec3(const double *r, int64_t n, int64_t i) {
    return Carry{get_u64(r + i), get_u64(r + n + i), 0.0, 0.0, get_u64(r + 2 * n + i)};
}
__device__ __forceinline__ void put_flag(uint64_t *f, uint64_t epoch, uint64_t status) {
    publish_fence();
    __hip_atomic_store(f, (epoch << 2) | status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Publish `status` unless a higher status of this call is already there (a helper that
// recomputed an aggregate must not hide the owner's inclusive carry).
__device__ __forceinline__ void raise_flag(uint64_t *f, uint64_t epoch, uint64_t status) {
    publish_fence();
    __hip_atomic_fetch_max(f, (epoch << 2) | status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One relaxed read of a flag, not yet interpreted: a unit issues it before its own
// publish_fence, so that the wait for its record stores also covers this read's round
// trip (the loads and stores of a wave complete in order).
__device__ __forceinline__ uint64_t peek_flag(const uint64_t *f) {
    return __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// The status a peeked flag value shows for this call (0 if none).
__device__ __forceinline__ int flag_status(uint64_t x, uint64_t epoch) {
    return (x >> 2) == epoch ? (int)(x & 3u) : 0;
}

// Look-back read in one batch: lane i < kPeekDepth of the publishing wave peeks the flag of
// the unit i+1 places before its own in scan order (position p-1-i for a unit at position
// p of its chain), all lanes in one load instruction.
constexpr int kPeekDepth = 8;

// Depth d >= 1 when the unit d places back holds an inclusive carry (or d == p: the chain
// start, an empty carry) and every unit in between has published at least its aggregate;
// 0 when the batch does not settle the walk (the caller then polls unit by unit). Called
// by a whole wave, lane i holding the value it peeked.
__device__ __forceinline__ int peek_depth(uint64_t x, uint64_t epoch, int lane, int64_t p) {
    const int n = p < kPeekDepth ? (int)p : kPeekDepth;
    const int st = lane < n ? flag_status(x, epoch) : 0;
    uint64_t incl = __ballot(st == (int)kInclusive);
    if (p <= kPeekDepth) incl |= 1ull << p;
    const uint64_t ok = __ballot(st != 0);
    if (incl == 0) return 0;
    const int i = __builtin_ctzll(incl);
    const uint64_t below = (1ull << i) - 1;
    return (ok & below) == below ? i + 1 : 0;
}

// Status of a unit's publication for this call: 1 aggregate, 2 inclusive carry, or 0 if
// nothing was published within `tries` polls (the caller then recomputes; no unit ever
// waits without bound).
__device__ __forceinline__ int poll_flag(const uint64_t *f, uint64_t epoch, int tries) {
    for (int i = 0;; ++i) {
        const uint64_t x = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((x >> 2) == epoch && (x & 3u) != 0u) {
            consume_fence();
            return (int)(x & 3u);
        }
        if (i >= tries) return 0;
        __builtin_amdgcn_s_sleep(4);
    }
}

// Chunk carries, one fp64 array per field (stride n between fields).
__device__ __forceinline__ void put_cin(double *f, int64_t n, int64_t i, const Carry &c) {
    f[i] = c.a;
    f[n + i] = c.b;
    f[2 * n + i] = c.ap;
    f[3 * n + i] = c.bp;
    f[4 * n + i] = c.P;
}
__device__ __forceinline__ Carry get_cin(const double *f, int64_t n, int64_t i) {
    return Carry{f[i], f[n + i], f[2 * n + i], f[3 * n + i], f[4 * n + i]};
}

// Where the backward finds the forward carries: the inclusive records (nrec = B*nseg*C of
// them per field) and the kept chunk carries of a finished forward launch.
struct FwdCarries {
    const double *incl;
    const double *cin;
    const double *init;  // [5][B][C]: the carry before token 0
    const double *tail;  // [3][B][C] or null: the future sums beyond the last window
    int64_t nrec;
    int64_t nseg;
};

// The forward carry entering kCinChunk-token chunk ci of sequence bidx, channel cl: for a
// chunk that opens forward window s, the inclusive carry of window s-1 normalized (for
// s = 0 the carry before token 0, normalized) -- bitwise the carry the forward computed for
// that chunk, since
// folding in an empty summary over no tokens leaves a carry unchanged -- else the carry
// the forward kept (plain loads: the records come from an earlier launch).
__device__ __forceinline__ Carry chunk_carry(const FwdCarries &F, int64_t bidx, int64_t ci,
                                             int64_t C, int cl) {
    constexpr int CPW = kCinCarries + 1;
    const int64_t s = ci / CPW;
    const int r = (int)(ci - s * CPW);
    if (r == 0) {
        Carry c = s == 0 ? get_cin(F.init, F.nrec / F.nseg, bidx * C + cl)
                         : get_cin(F.incl, F.nrec, (bidx * F.nseg + s - 1) * C + cl);
        normalize(c);
        return c;
    }
    return get_cin(F.cin, F.nrec * kCinCarries,
                   ((bidx * F.nseg + s) * kCinCarries + (r - 1)) * C + cl);
}

// c <- fold of a carry and a summary (the summary follows c in time, `len` tokens,
// len_w2 = len w log2 e).
__device__ __forceinline__ Carry follow(Carry c, const Carry &sum, double len_w2, double len) {
    fold(c, sum, len_w2, len);
    return c;
}

}  // namespace wkvdev
