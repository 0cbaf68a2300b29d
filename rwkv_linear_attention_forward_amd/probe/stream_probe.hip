// stream_probe.hip -- the streaming ceiling of a workgroup layout, for the benchmark (not
// part of the operator's library; built into its own librwkv_stream_probe.so).
//
// A workgroup of STRIPS x CHUNKS waves; wave (strip s, chunk c) reads 32 rows x 64 channels
// of k and v ([R][C] fp32, C fastest; one dword per lane per row, non-temporal) and writes
// y = k + v: the same bytes per element as the forward (12) and no other arithmetic. The
// strips of a workgroup are adjacent in the channels (STRIPS x 256 bytes of each row), its
// chunks adjacent in the rows; workgroups are numbered with the channel groups fastest.
// STRIPS = 1, CHUNKS = 2 is the layout of the forward's and backward's units (two waves
// over one 64-channel strip and 64 consecutive rows). Dynamic LDS (unused) sets the number
// of workgroups a CU holds, i.e. the occupancy.
//
// wkv_stream_probe_decode is the same measure for the decode step: the decode's 36 bytes per
// element (read k, v, a, b, p; write y, a, b, p) in the decode kernel's layout, with a
// minimum of arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kRows = 32;

template <int STRIPS, int CHUNKS>
__global__ __launch_bounds__(STRIPS * CHUNKS * 64) void stream_kernel(int64_t C,
                                                                      const float *__restrict__ k,
                                                                      const float *__restrict__ v,
                                                                      float *__restrict__ y) {
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int s = w % STRIPS, c = w / STRIPS;
    const int64_t ngrp = C / (64 * STRIPS);
    const int64_t g = blockIdx.x % ngrp, win = blockIdx.x / ngrp;
    const int64_t row0 = (win * CHUNKS + c) * kRows;
    const int64_t base = row0 * C + (g * STRIPS + s) * 64 + lane;
    float kk[kRows], vv[kRows];
#pragma unroll
    for (int j = 0; j < kRows; ++j) {
        kk[j] = __builtin_nontemporal_load(k + base + j * C);
        vv[j] = __builtin_nontemporal_load(v + base + j * C);
    }
#pragma unroll
    for (int j = 0; j < kRows; ++j) __builtin_nontemporal_store(kk[j] + vv[j], y + base + j * C);
}

template <int STRIPS, int CHUNKS>
hipError_t launch(int64_t R, int64_t C, const float *k, const float *v, float *y, int lds,
                  hipStream_t st) {
    const int64_t nwg = (R / (kRows * CHUNKS)) * (C / (64 * STRIPS));
    hipLaunchKernelGGL((stream_kernel<STRIPS, CHUNKS>), dim3((unsigned)nwg),
                       dim3(STRIPS * CHUNKS * 64), lds, st, C, k, v, y);
    return hipGetLastError();
}

// Decode layout: a lane owns one channel and kDecRows consecutive sequences of [B][C] fp32
// tensors; the grid is x over 256-channel blocks, y over groups of kDecRows sequences. All
// rows' loads are issued first; then y = k + v, a + k, b + v and p + 1 are stored in place
// (non-temporal, as the decode's accesses).
constexpr int kDecRows = 4;

__global__ __launch_bounds__(256) void decode_stream_kernel(int64_t C, const float *__restrict__ k,
                                                            const float *__restrict__ v,
                                                            float *__restrict__ a,
                                                            float *__restrict__ b,
                                                            float *__restrict__ p,
                                                            float *__restrict__ y) {
    const int64_t base = (int64_t)blockIdx.y * kDecRows * C + blockIdx.x * 256 + threadIdx.x;
    float ka[kDecRows], va[kDecRows], aa[kDecRows], ba[kDecRows], pa[kDecRows];
#pragma unroll
    for (int r = 0; r < kDecRows; ++r) {
        const int64_t i = base + r * C;
        ka[r] = __builtin_nontemporal_load(k + i);
        va[r] = __builtin_nontemporal_load(v + i);
        aa[r] = __builtin_nontemporal_load(a + i);
        ba[r] = __builtin_nontemporal_load(b + i);
        pa[r] = __builtin_nontemporal_load(p + i);
    }
#pragma unroll
    for (int r = 0; r < kDecRows; ++r) {
        const int64_t i = base + r * C;
        __builtin_nontemporal_store(ka[r] + va[r], y + i);
        __builtin_nontemporal_store(aa[r] + ka[r], a + i);
        __builtin_nontemporal_store(ba[r] + va[r], b + i);
        __builtin_nontemporal_store(pa[r] + 1.0f, p + i);
    }
}

}  // namespace

// y = k + v over [R][C] in the layout (strips, chunks) with `lds_bytes` of dynamic LDS per
// workgroup. Returns 0, 1 for a shape the layout does not tile (C must be a multiple of
// 64 * strips and R of 32 * chunks, R * C < 2^40) or an unsupported layout (strips x chunks
// in {1x2, 2x2, 4x1}, lds_bytes <= 65536), 2 for a launch error.
extern "C" int wkv_stream_probe(int64_t R, int64_t C, const float *k, const float *v, float *y,
                                int strips, int chunks, int lds_bytes, void *stream) {
    if (R <= 0 || C <= 0 || strips <= 0 || chunks <= 0 || C % (64 * strips) != 0 ||
        R % (kRows * chunks) != 0 || R > (int64_t(1) << 40) / C || lds_bytes < 0 ||
        lds_bytes > 65536 || k == nullptr || v == nullptr || y == nullptr)
        return 1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (strips == 1 && chunks == 2)
        e = launch<1, 2>(R, C, k, v, y, lds_bytes, st);
    else if (strips == 2 && chunks == 2)
        e = launch<2, 2>(R, C, k, v, y, lds_bytes, st);
    else if (strips == 4 && chunks == 1)
        e = launch<4, 1>(R, C, k, v, y, lds_bytes, st);
    else
        return 1;
    return e == hipSuccess ? 0 : 2;
}

// The decode's traffic over [B][C] fp32 tensors in the decode kernel's layout: y = k + v,
// a += k, b += v, p += 1 (in place). Returns 0, 1 for a shape the layout does not tile (C a
// multiple of 256, B of 4 with B / 4 <= 65535, B * C < 2^40) or a null pointer, 2 for a
// launch error.
extern "C" int wkv_stream_probe_decode(int64_t B, int64_t C, const float *k, const float *v,
                                       float *a, float *b, float *p, float *y, void *stream) {
    if (B <= 0 || C <= 0 || C % 256 != 0 || B % kDecRows != 0 || B / kDecRows > 65535 ||
        B > (int64_t(1) << 40) / C || k == nullptr || v == nullptr || a == nullptr ||
        b == nullptr || p == nullptr || y == nullptr)
        return 1;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(decode_stream_kernel, dim3((unsigned)(C / 256), (unsigned)(B / kDecRows)),
                       dim3(256), 0, st, C, k, v, a, b, p, y);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
