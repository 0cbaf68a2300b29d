// wkv_launch.h -- kernel launchers behind the C ABI (internal to librwkv_wkv).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wkvdev {

// Tokens between two carries saved by the forward for the backward. Every kernel window
// divides it, and the saved-carry layout is [B][ceil(T / kSaveStride)][C] for each of
// a (fp32), b (fp32) and P (fp64), in that order in one buffer.
constexpr int kSaveStride = 256;

hipError_t launch_forward(int64_t B, int64_t T, int64_t C, const float *w, const float *u,
                          const float *k, const float *v, float *y, float *sva, float *svb,
                          double *svP, hipStream_t stream);

hipError_t launch_decode(int64_t B, int64_t C, const float *w, const float *u, const float *k,
                         const float *v, float *a, float *b, float *p, float *y,
                         hipStream_t stream);

}  // namespace wkvdev
