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

// k, v, y in storage format IO (widened on load, rounded on store); the state stays fp32.
template <Io IO>
__device__ __forceinline__ void decode_elem(int64_t i, int64_t C, const float *__restrict__ w,
                                            const float *__restrict__ u,
                                            const io_t<IO> *__restrict__ k,
                                            const io_t<IO> *__restrict__ v,
                                            float *__restrict__ a, float *__restrict__ b,
                                            float *__restrict__ p, io_t<IO> *__restrict__ y) {
    const int64_t c = i % C;
    const float wc = w[c], uc = u[c];
    Rs s{a[i], b[i], p[i]};
    const float kk = io_ld<IO>(k, i), vv = io_ld<IO>(v, i);
    io_st<IO>(y, i, rs_out(s, kk, vv, uc));
    rs_push(s, kk, vv, make_decay(wc));
    a[i] = s.a;
    b[i] = s.b;
    p[i] = s.p;
}

// Two elements per lane, 256 apart (both accesses coalesced; the two loads of each tensor are
// in flight together). Past kDecodeMaxBlocks workgroups (2^29 elements) the grid is capped and
// lanes loop (LOOP). Measured on the 256 x 5120 decode workload: 11.0 us per call, against
// 11.2 with one element per lane and 11.5 with four per lane in 16-byte accesses.
constexpr int kDecodeEpt = 2;
constexpr int64_t kDecodeMaxBlocks = int64_t(1) << 20;

template <bool LOOP, Io IO>
__global__ __launch_bounds__(256) void wkv_decode_kernel(
    int64_t n, int64_t C, const float *__restrict__ w, const float *__restrict__ u,
    const io_t<IO> *__restrict__ k, const io_t<IO> *__restrict__ v, float *__restrict__ a,
    float *__restrict__ b, float *__restrict__ p, io_t<IO> *__restrict__ y) {
    const int64_t span = (int64_t)256 * kDecodeEpt;
    const int64_t step = LOOP ? (int64_t)gridDim.x * span : n;
    for (int64_t i0 = (int64_t)blockIdx.x * span + threadIdx.x; i0 < n; i0 += step) {
#pragma unroll
        for (int e = 0; e < kDecodeEpt; ++e) {
            const int64_t i = i0 + e * 256;
            if (i < n) decode_elem<IO>(i, C, w, u, k, v, a, b, p, y);
        }
    }
}

template <Io IO>
static hipError_t launch_decode_io(int64_t B, int64_t C, const float *w, const float *u,
                                   const void *k, const void *v, float *a, float *b, float *p,
                                   void *y, hipStream_t stream) {
    using E = io_t<IO>;
    const E *kk = static_cast<const E *>(k), *vv = static_cast<const E *>(v);
    E *yy = static_cast<E *>(y);
    const int64_t n = B * C;
    const int64_t nblk = (n + 256 * kDecodeEpt - 1) / (256 * kDecodeEpt);
    if (nblk <= kDecodeMaxBlocks)
        hipLaunchKernelGGL((wkv_decode_kernel<false, IO>), dim3((unsigned)nblk), dim3(256), 0,
                           stream, n, C, w, u, kk, vv, a, b, p, yy);
    else
        hipLaunchKernelGGL((wkv_decode_kernel<true, IO>), dim3((unsigned)kDecodeMaxBlocks),
                           dim3(256), 0, stream, n, C, w, u, kk, vv, a, b, p, yy);
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
