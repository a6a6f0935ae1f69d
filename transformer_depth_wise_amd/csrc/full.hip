// Phase 2 of the grouped two-phase Full AttnRes on gfx950.
//
// Full AttnRes keeps every sublayer output as its own depth source
// ("Attention Residuals" notes, section 7).  The two-phase schedule of the
// reading notes (static queries, two-phase computation) and of the notes'
// section 10 groups consecutive sublayers: phase 1 scores, for all queries of
// a group at once, the sources completed before the group and returns the
// normalised output o and its log-sum-exp lse; phase 2, once per sublayer,
// adds the k outputs produced inside the group so far, each as a separate
// source with its own score:
//     z_i = w^T (g (.) u_i / r(u_i)),  M = max(lse, z_1..z_k),
//     h = (e^{lse-M} o + sum_i e^{z_i-M} u_i) / (e^{lse-M} + sum_i e^{z_i-M}),
// and applies the consuming sublayer's PreNorm, x = gamma (.) h / r(h).
//
// One team of threads per token row (a wave for d <= 2048, the 256-thread
// workgroup above that), each thread owning CPL chunks of 8 channels.  Pass 1
// loads o and the k rows (in batches of kBatch rows, every load unconditional)
// and accumulates per-thread partial sums of u_i^2 and (w (.) g) . u_i; the
// 2k partials are reduced over the team in one batch (wave shuffles, then one
// LDS exchange for 256-thread teams).  Pass 2 re-reads the k rows (they were
// just read by the same threads) to form h, then the PreNorm reduction and
// the stores.  HBM sees each row once.
#include "attnres_device.h"
#include "attnres_launch.h"

namespace attnres {

constexpr int kMultiMax = 16;  // in-group sources per call
constexpr int kBatch = 4;      // rows loaded per batch

template <typename St, int TEAM, int CPL>
__global__ __launch_bounds__(256) void k_merge_multi(int64_t T, int d, const St* __restrict__ o1,
                                                     const float* __restrict__ lse1, const St* __restrict__ src,
                                                     int k, int64_t stride, const float* __restrict__ w,
                                                     const float* __restrict__ kg,
                                                     const float* __restrict__ gamma, float eps,
                                                     St* __restrict__ h_out, St* __restrict__ x_out) {
  constexpr int TPW = 256 / TEAM;
  constexpr int NW = TEAM / kWave;  // waves per team
  // per team-wave partial sums of the batched reduction, two buffers
  __shared__ float red[2][TPW * NW][2 * kMultiMax + 1];
  const int team = threadIdx.x / TEAM;
  const int tl = threadIdx.x % TEAM;
  const int wv = tl / kWave;  // wave within the team
  const int lane = threadIdx.x & (kWave - 1);
  const int C = d >> 3;
  const float inv_d = 1.0f / (float)d;
  // w and g are loaded (clamped, unconditionally) and multiplied where the
  // first row needs them, so no wait precedes the first token's loads
  float wr[CPL][8], gk[CPL][8];
#pragma unroll
  for (int c8 = 0; c8 < CPL; ++c8) {
    const int c0 = tl + TEAM * c8;
    const int c = c0 < C ? c0 : C - 1;
    if (k > 0) {
      load8(w + c * 8, wr[c8]);
      if (kg) {
        load8(kg + c * 8, gk[c8]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) gk[c8][e] = 1.f;
      }
    } else {
      zero8(wr[c8]);
      zero8(gk[c8]);
    }
  }
  int parity = 0;
  const int64_t step = (int64_t)gridDim.x * TPW;
  for (int64_t tok = (int64_t)blockIdx.x * TPW + team; tok - team < T; tok += step) {
    // every team of the workgroup runs the same number of iterations (the
    // reductions below synchronise the whole workgroup); tokens past T use a
    // clamped row and store nothing
    const bool live = tok < T;
    const int64_t tc = live ? tok : T - 1;
    bool ok[CPL];
    int cc[CPL];
#pragma unroll
    for (int c8 = 0; c8 < CPL; ++c8) {
      const int c0 = tl + TEAM * c8;
      ok[c8] = c0 < C;
      cc[c8] = ok[c8] ? c0 : C - 1;
    }
    // ---- pass 1: o and the per-row partial sums
    float h[CPL][8];
#pragma unroll
    for (int c8 = 0; c8 < CPL; ++c8) {
      Chunk<St> ch;
      ch.load(o1 + tc * d + cc[c8] * 8);
      ch.unpack(h[c8]);
    }
    float part[2 * kMultiMax];
#pragma unroll
    for (int i = 0; i < 2 * kMultiMax; ++i) part[i] = 0.f;
#pragma unroll
    for (int b0 = 0; b0 < kMultiMax; b0 += kBatch) {
      if (b0 < k) {  // uniform
        Chunk<St> u[kBatch][CPL];
#pragma unroll
        for (int r = 0; r < kBatch; ++r) {
          const int i = b0 + r < k ? b0 + r : k - 1;  // clamped: always a valid row
#pragma unroll
          for (int c8 = 0; c8 < CPL; ++c8) u[r][c8].load(src + (int64_t)i * stride + tc * d + cc[c8] * 8);
        }
#pragma unroll
        for (int r = 0; r < kBatch; ++r) {
          float ss = 0.f, dot = 0.f;
#pragma unroll
          for (int c8 = 0; c8 < CPL; ++c8) {
            float f[8];
            u[r][c8].unpack(f);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float v = ok[c8] ? f[e] : 0.f;
              ss = fmaf(v, v, ss);
              dot = fmaf(wr[c8][e] * gk[c8][e], v, dot);
            }
          }
          part[2 * (b0 + r)] = ss;
          part[2 * (b0 + r) + 1] = dot;
        }
      }
    }
    // ---- batched team reduction of the 2k partial sums
    float z[kMultiMax];
    {
      float* buf = &red[parity][0][0];
      parity ^= 1;
#pragma unroll
      for (int i = 0; i < 2 * kMultiMax; ++i)
        if (i < 2 * k) part[i] = wave_sum(part[i]);
      if (NW > 1) {
        if (lane == 0) {
#pragma unroll
          for (int i = 0; i < 2 * kMultiMax; ++i)
            if (i < 2 * k) buf[(team * NW + wv) * (2 * kMultiMax + 1) + i] = part[i];
        }
        lds_barrier();
        const float* tb = buf + team * NW * (2 * kMultiMax + 1);
#pragma unroll
        for (int i = 0; i < 2 * kMultiMax; ++i)
          if (i < 2 * k) {
            constexpr int S1 = 2 * kMultiMax + 1;
            part[i] = NW == 4 ? (tb[i] + tb[S1 + i]) + (tb[2 * S1 + i] + tb[3 * S1 + i]) : tb[i];
          }
      }
#pragma unroll
      for (int i = 0; i < kMultiMax; ++i)
        z[i] = i < k ? part[2 * i + 1] / sqrtf(part[2 * i] * inv_d + eps) : 0.f;
    }
    // ---- softmax weights of the k + 1 partitions
    const float lse = lse1[tc];
    float M = lse;
#pragma unroll
    for (int i = 0; i < kMultiMax; ++i)
      if (i < k) M = fmaxf(M, z[i]);
    float den = expf(lse - M);
    float a[kMultiMax];
#pragma unroll
    for (int i = 0; i < kMultiMax; ++i) {
      a[i] = i < k ? expf(z[i] - M) : 0.f;
      den += a[i];
    }
    const float inv = 1.0f / den;
    const float ao = expf(lse - M) * inv;
    // ---- pass 2: h = ao o + sum_i a_i u_i (rows re-read by the same threads)
#pragma unroll
    for (int c8 = 0; c8 < CPL; ++c8)
#pragma unroll
      for (int e = 0; e < 8; ++e) h[c8][e] *= ao;
#pragma unroll
    for (int b0 = 0; b0 < kMultiMax; b0 += kBatch) {
      if (b0 < k) {
        Chunk<St> u[kBatch][CPL];
#pragma unroll
        for (int r = 0; r < kBatch; ++r) {
          const int i = b0 + r < k ? b0 + r : k - 1;
#pragma unroll
          for (int c8 = 0; c8 < CPL; ++c8) u[r][c8].load(src + (int64_t)i * stride + tc * d + cc[c8] * 8);
        }
#pragma unroll
        for (int r = 0; r < kBatch; ++r) {
          if (b0 + r < k) {
            const float ar = a[b0 + r] * inv;
#pragma unroll
            for (int c8 = 0; c8 < CPL; ++c8) {
              float f[8];
              u[r][c8].unpack(f);
#pragma unroll
              for (int e = 0; e < 8; ++e) h[c8][e] = fmaf(ar, f[e], h[c8][e]);
            }
          }
        }
      }
    }
    // ---- PreNorm and stores
    float sh = 0.f;
#pragma unroll
    for (int c8 = 0; c8 < CPL; ++c8)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (!ok[c8]) h[c8][e] = 0.f;
        sh = fmaf(h[c8][e], h[c8][e], sh);
      }
    float rinv = 1.f;
    if (x_out) {
      float* buf = &red[parity][0][0];
      parity ^= 1;
      sh = wave_sum(sh);
      if (NW > 1) {
        if (lane == 0) buf[(team * NW + wv) * (2 * kMultiMax + 1)] = sh;
        lds_barrier();
        const float* tb = buf + team * NW * (2 * kMultiMax + 1);
        constexpr int S1 = 2 * kMultiMax + 1;
        sh = NW == 4 ? (tb[0] + tb[S1]) + (tb[2 * S1] + tb[3 * S1]) : tb[0];
      }
      rinv = 1.0f / sqrtf(sh * inv_d + eps);
    }
    if (live) {
#pragma unroll
      for (int c8 = 0; c8 < CPL; ++c8) {
        if (!ok[c8]) continue;
        const int64_t off = tok * d + cc[c8] * 8;
        if (h_out) store8(h_out + off, h[c8]);
        if (x_out) {
          float gm[8], x[8];
          if (gamma) {
            load8(gamma + cc[c8] * 8, gm);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) gm[e] = 1.f;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = gm[e] * (h[c8][e] * rinv);
          store8(x_out + off, x);
        }
      }
    }
  }
}

template <typename St, int TEAM, int CPL>
static hipError_t run_multi_merge(int64_t T, int d, const void* o1, const float* lse1, const void* src, int k,
                                  int64_t stride, const float* w, const float* kg, const float* gamma, float eps,
                                  void* h_out, void* x_out, hipStream_t stream) {
  constexpr int TPW = 256 / TEAM;
  const int64_t wgs = (T + TPW - 1) / TPW;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  hipLaunchKernelGGL((k_merge_multi<St, TEAM, CPL>), dim3((unsigned)(wgs < cap ? wgs : cap)), dim3(256), 0, stream,
                     T, d, static_cast<const St*>(o1), lse1, static_cast<const St*>(src), k, stride, w, kg, gamma,
                     eps, static_cast<St*>(h_out), static_cast<St*>(x_out));
  return hipGetLastError();
}

template <typename St>
static hipError_t pick_multi(int64_t T, int d, const void* o1, const float* lse1, const void* src, int k,
                             int64_t stride, const float* w, const float* kg, const float* gamma, float eps,
                             void* h_out, void* x_out, hipStream_t stream) {
  const int C = d >> 3;
#define ATTNRES_RUN(TEAM_, CPL_) \
  return run_multi_merge<St, TEAM_, CPL_>(T, d, o1, lse1, src, k, stride, w, kg, gamma, eps, h_out, x_out, stream)
  if (C <= 64) ATTNRES_RUN(64, 1);
  if (C <= 128) ATTNRES_RUN(64, 2);
  if (C <= 256) ATTNRES_RUN(64, 4);
  if (C <= 512) ATTNRES_RUN(256, 2);
  if (C <= 1024) ATTNRES_RUN(256, 4);
  ATTNRES_RUN(256, 8);
#undef ATTNRES_RUN
}

hipError_t launch_merge_multi(Dtype dt, int64_t T, int d, const void* o1, const float* lse1, const void* src,
                              int k, int64_t stride, const float* w, const float* kg, const float* gamma, float eps,
                              void* h_out, void* x_out, hipStream_t stream) {
  if (dt == kBF16) return pick_multi<bf16_t>(T, d, o1, lse1, src, k, stride, w, kg, gamma, eps, h_out, x_out, stream);
  return pick_multi<float>(T, d, o1, lse1, src, k, stride, w, kg, gamma, eps, h_out, x_out, stream);
}

}  // namespace attnres
