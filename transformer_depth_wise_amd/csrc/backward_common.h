// Private to the backward kernels of libattnres: fixed-order team
// reductions and the per-team weight-gradient reduction shared by the site,
// phase-2 and phase-1 backward passes.
#pragma once
#include <type_traits>

#include "attnres_device.h"
#include "attnres_launch.h"

namespace attnres {

constexpr int kBwdMax = 32;   // sources per site
constexpr int kBwdBatch = 4;  // rows loaded per batch

// Fixed-order sum of v[0..NV) over the team (NW waves): DPP wave sums, then
// the waves in index order through LDS.  `buf` holds NW * NV floats of LDS,
// alternated by the caller between consecutive reductions.  Unused entries
// are zeros and cost a few instructions, not branches.
template <int NW, int NV>
__device__ __forceinline__ void team_reduce(float (&v)[NV], float* buf, int wv, int lane) {
#pragma unroll
  for (int i = 0; i < NV; ++i) v[i] = wave_sum_dpp(v[i]);
  if (NW > 1) {
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < NV; ++i) buf[wv * NV + i] = v[i];
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float s = buf[i];
#pragma unroll
      for (int k = 1; k < NW; ++k) s += buf[k * NV + i];
      v[i] = s;
    }
  }
}

// OUT: how dL/du_i leaves -- stored in the storage type (kOutStore), added to
// fp32 rows (kOutAdd) or stored as fp32 rows (kOutF32).
constexpr int kOutStore = 0, kOutAdd = 1, kOutF32 = 2;


constexpr int kRedWaves = 16;  // waves of the fixed-order per-team sum reduction

// dw = g (.) A, dg = w (.) A, dgamma = G from the per-team partials
// part[slot][0..1][d], summed over `slots` in a fixed order (added to the
// outputs with `add`).
hipError_t launch_wgrad_reduce(int64_t slots, int d, const float* part, const float* w, const float* kg, float* dw,
                               float* dkg, float* dgamma, int add, hipStream_t stream);

// Threads per team of the site backward for rows of d channels.
int backward_team(int d);

// Waves of the phase-1 backward's weight-gradient pass (a fixed count, so the
// workspace size and the summation order do not depend on the device).
constexpr int kWgradWaves = 2048;

// The phase-1 backward of a block for one pair of row types: bf16 sources and
// G, fp32 sources and G, or fp32 sources with bf16 G.
#define ATTNRES_P1B_ARGS                                                                                        \
  int n, int64_t T, int d, const void *src, int64_t stride, int S, const float *w, const float *kg, float eps, \
      const void *gin, int64_t gstride, const float *c_in, const float *gp_in, float *dsrc, int64_t dstride,   \
      int accumulate, float *dw, float *dkg, float *ws, hipStream_t stream
hipError_t launch_p1b_bf16(ATTNRES_P1B_ARGS);
hipError_t launch_p1b_f32(ATTNRES_P1B_ARGS);
hipError_t launch_p1b_f32src(ATTNRES_P1B_ARGS);
#undef ATTNRES_P1B_ARGS

}  // namespace attnres
