// wkv_decode.hip -- one recurrent step of the WKV operator for a batch of sequences.
//
// The recursive form of formula (8) ("RWKV解读：在Transformer的时代的新RNN", section 二.3):
// the model takes a token and a state and returns the output and the new state ("RWKV
// についての調査記録", section "RWKVとは？"), so the per-token cost does not depend on how
// many tokens came before ("介绍RWKV – 具有Transformer优势的RNN", section
// "RWKV作为RNN和transformer的结合体"). Purely elementwise over (b, c): 36 bytes of HBM
// traffic per element (read k, v, a, b, p; write y, a, b, p), no reuse, so the kernel is
// a coalesced stream with one lane per element.
#include "wkv_device.h"
#include "wkv_launch.h"

namespace wkvdev {

__device__ __forceinline__ void decode_elem(int64_t i, int64_t C, const float *__restrict__ w,
                                            const float *__restrict__ u,
                                            const float *__restrict__ k,
                                            const float *__restrict__ v, float *__restrict__ a,
                                            float *__restrict__ b, float *__restrict__ p,
                                            float *__restrict__ y) {
    const int64_t c = i % C;
    const float wc = w[c], uc = u[c];
    Rs s{a[i], b[i], p[i]};
    const float kk = k[i], vv = v[i];
    y[i] = rs_out(s, kk, vv, uc);
    rs_push(s, kk, vv, make_decay(wc));
    a[i] = s.a;
    b[i] = s.b;
    p[i] = s.p;
}

// One lane per element. Past kDecodeMaxBlocks workgroups (2^28 elements) the grid is capped
// and lanes loop (LOOP); below, one pass without the loop's overhead (~1% of the call).
// Four elements per lane with 16-byte accesses measured slower on the 256 x 5120 decode
// workload (11.5 vs 11.2 us per call).
constexpr int64_t kDecodeMaxBlocks = int64_t(1) << 20;

template <bool LOOP>
__global__ __launch_bounds__(256) void wkv_decode_kernel(
    int64_t n, int64_t C, const float *__restrict__ w, const float *__restrict__ u,
    const float *__restrict__ k, const float *__restrict__ v, float *__restrict__ a,
    float *__restrict__ b, float *__restrict__ p, float *__restrict__ y) {
    const int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if constexpr (LOOP) {
        for (int64_t i = i0; i < n; i += (int64_t)gridDim.x * 256)
            decode_elem(i, C, w, u, k, v, a, b, p, y);
    } else if (i0 < n) {
        decode_elem(i0, C, w, u, k, v, a, b, p, y);
    }
}

hipError_t launch_decode(int64_t B, int64_t C, const float *w, const float *u, const float *k,
                         const float *v, float *a, float *b, float *p, float *y,
                         hipStream_t stream) {
    const int64_t n = B * C;
    const int64_t nblk = (n + 255) / 256;
    if (nblk <= kDecodeMaxBlocks)
        hipLaunchKernelGGL(wkv_decode_kernel<false>, dim3((unsigned)nblk), dim3(256), 0, stream,
                           n, C, w, u, k, v, a, b, p, y);
    else
        hipLaunchKernelGGL(wkv_decode_kernel<true>, dim3((unsigned)kDecodeMaxBlocks), dim3(256),
                           0, stream, n, C, w, u, k, v, a, b, p, y);
    return hipGetLastError();
}

}  // namespace wkvdev
