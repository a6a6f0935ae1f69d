// Phase-1 backward kernels for bf16 source rows and bf16 G rows.
#include "backward_p1.h"

namespace attnres {

hipError_t launch_p1b_bf16(int n, int64_t T, int d, const void* src, int64_t stride, int S, const float* w, const float* kg,
             float eps, const void* gin, int64_t gstride, const float* c_in, const float* gp_in, float* dsrc,
             int64_t dstride, int accumulate, float* dw, float* dkg, float* ws, hipStream_t stream) {
  return pick_p1b<bf16_t, bf16_t>(n, T, d, src, stride, S, w, kg, eps, gin, gstride, c_in, gp_in, dsrc, dstride, accumulate,
                          dw, dkg, ws, stream);
}

}  // namespace attnres
