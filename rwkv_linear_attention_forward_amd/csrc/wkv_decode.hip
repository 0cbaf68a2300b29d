// wkv_decode.hip -- one recurrent step of the WKV operator for a batch of sequences.
//
// The recursive form of formula (8) ("RWKV解读：在Transformer的时代的新RNN", section 二.3):
// the model takes a token and a state and returns the output and the new state ("RWKV
// についての調査記録", section "RWKVとは？"), so the per-token cost does not depend on how
// many tokens came before ("介绍RWKV – 具有Transformer优势的RNN", section
// "RWKV作为RNN和transformer的结合体"). Purely elementwise over (b, c): 36 bytes of HBM
// traffic per element (read k, v, a, b, p; write y, a, b, p), no reuse, so the kernel is
// a coalesced stream with one lane per element. With k, v, y stored in 16 bits, 30 bytes.
#include "wkv_device.h"
#include "wkv_launch.h"

namespace wkvdev {

// Grid: x over 256-channel blocks, y over groups of kDecodeRows sequences (strided when there
// are more groups than a grid's y extent). A lane owns one channel c and kDecodeRows
// sequences b0 .. b0 + kDecodeRows - 1: the channel's constants (w, u and the decay factors
// of the rescaled update) are formed once per lane, and the rows go through a two-stage
// pipeline, row r + 1's loads issued before row r's arithmetic and stores, so that a wave's
// loads and stores overlap. No division or remainder in the index math. On the 256 x 5120
// decode workload the grid is 20 x 64 workgroups of four waves: 5,120 waves, all resident at
// once.
#ifndef WKV_DECODE_ROWS
#define WKV_DECODE_ROWS 4
#endif
constexpr int kDecodeRows = WKV_DECODE_ROWS;
constexpr int64_t kDecodeMaxGroups = 65535;

// One group of kDecodeRows sequences for the lane's channel c (vf, vio: its byte offsets
// in fp32 and in format IO), rows b0 .. b0 + rows - 1.
template <Io IO>
__device__ __forceinline__ void decode_group(int64_t b0, int rows, int64_t C, int vf, int vio,
                                             const float *__restrict__ w,
                                             const float *__restrict__ u,
                                             const io_t<IO> *__restrict__ k,
                                             const io_t<IO> *__restrict__ v, float *__restrict__ a,
                                             float *__restrict__ b, float *__restrict__ p,
                                             io_t<IO> *__restrict__ y) {
    // one buffer resource per tensor at the group's first row (scalar registers), the lane's
    // channel as a 32-bit byte offset, the row as a scalar offset
    const int64_t base = b0 * C;
    const rsrc_t ra = make_rsrc(a + base), rb = make_rsrc(b + base), rp = make_rsrc(p + base);
    const rsrc_t rk = make_rsrc(k + base), rv = make_rsrc(v + base), ry = make_rsrc(y + base);
    // row r's scalar byte offsets (a row past B reads the group's first row: in bounds)
    auto sf = [&](int r) { return (int)((r < rows ? r : 0) * C * 4); };
    auto sio = [&](int r) { return (int)((r < rows ? r : 0) * C * kIoBytes<IO>); };
    const Rs s0{bload(ra, vf, 0), bload(rb, vf, 0), bload(rp, vf, 0)};
    const float k0 = bload_io<IO>(rk, vio, 0), v0 = bload_io<IO>(rv, vio, 0);
    // the channel's constants, read after the first row's loads are issued, so that their
    // round trip overlaps the row's instead of preceding it (the empty statement keeps the
    // compiler from moving memory accesses across it)
    asm volatile("" ::: "memory");
    const float uc = bload(make_rsrc(u), vf, 0);
    const Decay dc = make_decay(bload(make_rsrc(w), vf, 0));
    Rs s = s0;
    float kk = k0, vv = v0;
#pragma unroll
    for (int r = 0; r < kDecodeRows; ++r) {
        Rs sn{0.0f, 0.0f, 0.0f};
        float kn = 0.0f, vn = 0.0f;
        if (r + 1 < kDecodeRows) {
            // row r + 1's loads go out before row r's stores. A row past B takes the first
            // row's inputs as loaded before any store (its own load of that row may see the
            // row already updated) and so stores the first row's results again, the same
            // values at the same addresses: every row is computed and stored branch-free and
            // the compiler cannot sink a row's loads behind a condition.
            const bool dup = r + 1 >= rows;
            const Rs sl{bload(ra, vf, sf(r + 1)), bload(rb, vf, sf(r + 1)),
                        bload(rp, vf, sf(r + 1))};
            const float kl = bload_io<IO>(rk, vio, sio(r + 1));
            const float vl = bload_io<IO>(rv, vio, sio(r + 1));
            sn = dup ? s0 : sl;
            kn = dup ? k0 : kl;
            vn = dup ? v0 : vl;
        }
        bstore_io<IO>(ry, rs_out(s, kk, vv, uc), vio, sio(r));
        rs_push(s, kk, vv, dc);
        bstore(ra, s.a, vf, sf(r));
        bstore(rb, s.b, vf, sf(r));
        bstore(rp, s.p, vf, sf(r));
        s = sn;
        kk = kn;
        vv = vn;
    }
}

// LOOP: more row groups than the grid's y extent, taken in strides of gridDim.y; otherwise
// one group per workgroup row.
template <bool LOOP, Io IO>
__global__ __launch_bounds__(256) void wkv_decode_kernel(
    int64_t B, int64_t C, int64_t ngroups, const float *__restrict__ w, const float *__restrict__ u,
    const io_t<IO> *__restrict__ k, const io_t<IO> *__restrict__ v, float *__restrict__ a,
    float *__restrict__ b, float *__restrict__ p, io_t<IO> *__restrict__ y) {
    const int c = (int)(blockIdx.x * 256 + threadIdx.x);
    // the arguments are read into scalar registers before the channel guard, in one round
    // trip (the compiler would otherwise read the size first, branch, then read the pointers:
    // two dependent round trips ahead of every wave's first load; 4-5% of the decode's time)
    asm volatile("" ::"s"(B), "s"(C), "s"(ngroups), "s"(w), "s"(u), "s"(k), "s"(v), "s"(a),
                 "s"(b), "s"(p), "s"(y));
    if (c >= C) return;
    const int vf = c * 4, vio = c * kIoBytes<IO>;
    for (int64_t g = blockIdx.y; g < ngroups; g += gridDim.y) {
        const int64_t b0 = g * kDecodeRows;
        const int rows = (int)(B - b0 < kDecodeRows ? B - b0 : kDecodeRows);
        decode_group<IO>(b0, rows, C, vf, vio, w, u, k, v, a, b, p, y);
        if (!LOOP) break;
    }
}

template <Io IO>
static hipError_t launch_decode_io(int64_t B, int64_t C, const float *w, const float *u,
                                   const void *k, const void *v, float *a, float *b, float *p,
                                   void *y, hipStream_t stream) {
    using E = io_t<IO>;
    const E *kk = static_cast<const E *>(k), *vv = static_cast<const E *>(v);
    E *yy = static_cast<E *>(y);
    const int64_t ngroups = (B + kDecodeRows - 1) / kDecodeRows;
    const dim3 grid((unsigned)((C + 255) / 256),
                    (unsigned)(ngroups < kDecodeMaxGroups ? ngroups : kDecodeMaxGroups));
    if (ngroups <= kDecodeMaxGroups)
        hipLaunchKernelGGL((wkv_decode_kernel<false, IO>), grid, dim3(256), 0, stream, B, C,
                           ngroups, w, u, kk, vv, a, b, p, yy);
    else
        hipLaunchKernelGGL((wkv_decode_kernel<true, IO>), grid, dim3(256), 0, stream, B, C,
                           ngroups, w, u, kk, vv, a, b, p, yy);
    return hipGetLastError();
}

hipError_t launch_decode(int64_t B, int64_t C, Io fmt, const float *w, const float *u,
                         const void *k, const void *v, float *a, float *b, float *p, void *y,
                         hipStream_t stream) {
    if (fmt == Io::BF16)
        return launch_decode_io<Io::BF16>(B, C, w, u, k, v, a, b, p, y, stream);
    if (fmt == Io::F16)
        return launch_decode_io<Io::F16>(B, C, w, u, k, v, a, b, p, y, stream);
    return launch_decode_io<Io::F32>(B, C, w, u, k, v, a, b, p, y, stream);
}

}  // namespace wkvdev
