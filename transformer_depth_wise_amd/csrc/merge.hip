// Phase 2 of Block AttnRes on gfx950 and the block-completion sum.
//
// Phase 2 runs once per sublayer ("Attention Residuals" notes, section 10,
// second phase): the first sublayer of a block takes the phase-1 result as
// is; every later one scores the block's running partial sum and merges it
// with the phase-1 partition exactly.  With the phase-1 output o already
// normalised and lse its log-sum-exp, the two-partition merge of the reading
// notes' two-phase section reduces to
//     h = o + beta (p - o),   beta = 1 / (1 + e^{lse - z(p)}).
// The merge is element-wise, so it is fused with the consuming sublayer's
// PreNorm RMSNorm (CSDN summary, section 4.2; "ML 研究者的三层基本功",
// system layer) and with the partial-sum update p = partial + v_prev2 +
// v_prev (either of the first two terms optional).  Taking the two previous
// sublayer outputs lets a caller store the running partial only at every
// second sublayer: the sublayer in between reads the stored partial and one
// output and writes nothing.
//
// Each token row is processed by one team of threads (a wave for d <= 2048,
// the whole 256-thread workgroup above that).  A thread owns CPL chunks of 8
// channels; the row's two reductions (|p|^2 with w.p, then |h|^2) use wave
// shuffles and, for 256-thread teams, one LDS exchange each.  The per-channel
// parameters (w (.) g and gamma) stay in registers while a persistent grid of
// two workgroups per CU walks over the tokens; the raw rows of the team's next
// token are loaded before the current token is reduced, merged and stored, so
// HBM traffic continues through the reductions and barriers (the loop is
// unrolled twice over two register stages).
#include "attnres_device.h"
#include "attnres_launch.h"

namespace attnres {


template <typename St, typename Pt, int CPL>
struct Stage {
  Chunk<St> o[CPL], v[CPL], v2[CPL];
  Chunk<Pt> q[CPL];
  bool ok[CPL];
};

// Loads of one token for the team.  Every load is unconditional (an
// out-of-range token or chunk reads a clamped valid address and is zeroed
// when used), so the loads of a stage issue back to back.
template <typename St, typename Pt, int TEAM, int CPL, bool HAS_V, bool HAS_PIN, bool HAS_V2>
__device__ __forceinline__ void issue(Stage<St, Pt, CPL>& s, int64_t tok, int64_t T, int d, int C, int tl,
                                      const St* o1, const Pt* pin, const St* vprev2, const St* vprev,
                                      int64_t plane) {
  const bool live = tok < T;
  const int64_t tc = live ? tok : T - 1;
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int c0 = tl + TEAM * k;
    s.ok[k] = live && c0 < C;
    const int c = c0 < C ? c0 : C - 1;
    const int64_t off = tc * d + c * 8;
    s.o[k].load(o1 + off);
    if (HAS_V) s.v[k].load(vprev + off);
    if (HAS_V2) s.v2[k].load(vprev2 + off);
    if (HAS_PIN) s.q[k].load_at(pin, off, plane);
  }
}

template <typename St, typename Pt, int TEAM, int CPL, bool HAS_V, bool HAS_PIN, bool HAS_V2>
__device__ __forceinline__ void process(const Stage<St, Pt, CPL>& s, int64_t tok, int64_t T, int d, int C, int tl,
                                        const float* lse1, void* pout, bool pout24, int64_t plane,
                                        const float (&wq)[CPL][8], const float4* gm_lds, float eps, float inv_d,
                                        St* h_out, St* x_out, float (*red)[8], int& parity) {
  const bool live = tok < T;
  float h[CPL][8], p[CPL][8];
  float ss = 0.f, dot = 0.f;
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    s.o[k].unpack(h[k]);
    if (HAS_V) {
      // p = ((partial or 0) + (v_prev2 or 0)) + v_prev, in that order
      float v[8];
      s.v[k].unpack(v);
      if (HAS_PIN) {
        s.q[k].unpack(p[k]);
        if (HAS_V2) {
          float v2[8];
          s.v2[k].unpack(v2);
#pragma unroll
          for (int e = 0; e < 8; ++e) p[k][e] = p[k][e] + v2[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) p[k][e] = p[k][e] + v[e];
      } else if (HAS_V2) {
        s.v2[k].unpack(p[k]);
#pragma unroll
        for (int e = 0; e < 8; ++e) p[k][e] = p[k][e] + v[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) p[k][e] = v[e];
      }
    } else {
      zero8(p[k]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h[k][e] = s.ok[k] ? h[k][e] : 0.f;
      p[k][e] = s.ok[k] ? p[k][e] : 0.f;
    }
    if (HAS_V) {
      const int c = tl + TEAM * k;
      if (pout && s.ok[k]) {
        const int64_t off = tok * d + c * 8;
        if (pout24) {
          out24(static_cast<p24_t*>(pout), off, plane, p[k]);
        } else {
          out8(static_cast<float*>(pout) + off, p[k]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ss = fmaf(p[k][e], p[k][e], ss);
        dot = fmaf(wq[k][e], p[k][e], dot);
      }
    }
  }
  if (HAS_V) {
    float2 r;
    if (TEAM == 256) {
      r = block_sum2_256(ss, dot, red[parity]);
      parity ^= 1;
    } else {
      r.x = wave_sum(ss);
      r.y = wave_sum(dot);
    }
    const float zc = r.y / sqrtf(r.x * inv_d + eps);
    const float lse = lse1[live ? tok : T - 1];
    const float beta = 1.0f / (1.0f + expf(lse - zc));
#pragma unroll
    for (int k = 0; k < CPL; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) h[k][e] = fmaf(beta, p[k][e] - h[k][e], h[k][e]);
  }
  float sh = 0.f;
#pragma unroll
  for (int k = 0; k < CPL; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) sh = fmaf(h[k][e], h[k][e], sh);
  float r2 = 0.f;
  if (x_out) {
    if (TEAM == 256) {
      r2 = block_sum2_256(sh, 0.f, red[parity]).x;
      parity ^= 1;
    } else {
      r2 = wave_sum(sh);
    }
  }
  const float rinv = x_out ? 1.0f / sqrtf(r2 * inv_d + eps) : 1.f;
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    if (s.ok[k]) {
      const int64_t off = tok * d + (tl + TEAM * k) * 8;
      if (h_out) out8(h_out + off, h[k]);
      if (x_out) {
        const float4 g0 = gm_lds[2 * (tl + TEAM * k)], g1 = gm_lds[2 * (tl + TEAM * k) + 1];
        const float gk[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = gk[e] * (h[k][e] * rinv);
        out8(x_out + off, x);
      }
    }
  }
}

template <typename St, typename Pt, int TEAM, int CPL, bool HAS_V, bool HAS_PIN, bool HAS_V2>
__global__ __launch_bounds__(256) void k_merge(int64_t T, int d, const St* __restrict__ o1,
                                               const float* __restrict__ lse1, const Pt* __restrict__ pin,
                                               const St* __restrict__ vprev2, const St* __restrict__ vprev,
                                               void* __restrict__ pout, int pout24,
                                               const float* __restrict__ w, const float* __restrict__ kg,
                                               const float* __restrict__ gamma, float eps,
                                               St* __restrict__ h_out, St* __restrict__ x_out) {
  constexpr int TPW = 256 / TEAM;
  const int64_t plane = T * (int64_t)d;
  __shared__ float red[2][8];
  // the PreNorm gain, used once per token at the very end, waits in LDS; the
  // folded query w (.) g stays in registers
  extern __shared__ float4 gm_lds[];  // [d / 4]
  const int team = threadIdx.x / TEAM;
  const int tl = threadIdx.x % TEAM;
  const int C = d >> 3;
  const float inv_d = 1.0f / (float)d;
  // Prologue, ordered so that nothing waits before the first token's rows
  // are in flight: the parameter loads (clamped, unconditional), then the
  // first token's loads, then the LDS stores of gamma (which wait for gamma
  // only) and one barrier.
  constexpr int KG = (TEAM * CPL + 255) / 256;  // gamma chunks per thread
  float wq[CPL][8], gk[CPL][8], gv[KG][8];
  if (HAS_V) {
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int c0 = tl + TEAM * k;
      load8(w + (c0 < C ? c0 : C - 1) * 8, wq[k]);
    }
    if (kg) {
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const int c0 = tl + TEAM * k;
        load8(kg + (c0 < C ? c0 : C - 1) * 8, gk[k]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < CPL; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) gk[k][e] = 1.f;
    }
  } else {
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      zero8(wq[k]);
      zero8(gk[k]);
    }
  }
  if (x_out) {
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      const int c0 = (int)threadIdx.x + 256 * k;
      if (gamma) {
        load8(gamma + (c0 < C ? c0 : C - 1) * 8, gv[k]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) gv[k][e] = 1.f;
      }
    }
  }
  int parity = 0;
  const int64_t step = (int64_t)gridDim.x * TPW;
  int64_t tok = (int64_t)blockIdx.x * TPW + team;
  Stage<St, Pt, CPL> A, B;
  issue<St, Pt, TEAM, CPL, HAS_V, HAS_PIN, HAS_V2>(A, tok, T, d, C, tl, o1, pin, vprev2, vprev, plane);
  // w (.) g, with chunks past the end of d zeroed (x 1.0 exactly without g)
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const bool live = tl + TEAM * k < C;
#pragma unroll
    for (int e = 0; e < 8; ++e) wq[k][e] = live ? wq[k][e] * gk[k][e] : 0.f;
  }
  if (x_out) {
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      const int c = (int)threadIdx.x + 256 * k;
      if (c < C) {
        gm_lds[2 * c] = make_float4(gv[k][0], gv[k][1], gv[k][2], gv[k][3]);
        gm_lds[2 * c + 1] = make_float4(gv[k][4], gv[k][5], gv[k][6], gv[k][7]);
      }
    }
  }
  lds_barrier();
  while (tok - team < T) {
    issue<St, Pt, TEAM, CPL, HAS_V, HAS_PIN, HAS_V2>(B, tok + step, T, d, C, tl, o1, pin, vprev2, vprev, plane);
    process<St, Pt, TEAM, CPL, HAS_V, HAS_PIN, HAS_V2>(A, tok, T, d, C, tl, lse1, pout, pout24 != 0, plane, wq, gm_lds, eps,
                                              inv_d, h_out, x_out,
                                              red, parity);
    tok += step;
    if (tok - team >= T) break;
    issue<St, Pt, TEAM, CPL, HAS_V, HAS_PIN, HAS_V2>(A, tok + step, T, d, C, tl, o1, pin, vprev2, vprev, plane);
    process<St, Pt, TEAM, CPL, HAS_V, HAS_PIN, HAS_V2>(B, tok, T, d, C, tl, lse1, pout, pout24 != 0, plane, wq, gm_lds, eps,
                                              inv_d, h_out, x_out,
                                              red, parity);
    tok += step;
  }
}

// out = ((partial or 0) + (v2 or 0)) + v, in that order.
template <typename St, typename Pt>
__global__ __launch_bounds__(256) void k_accumulate(int64_t nchunks, const Pt* __restrict__ pin,
                                                    const St* __restrict__ v2, const St* __restrict__ v,
                                                    St* __restrict__ out) {
  const int64_t step = (int64_t)gridDim.x * 256;
  const int64_t plane = nchunks * 8;
  for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < nchunks; c += step) {
    float a[8], b[8];
    load8(v + c * 8, b);
    if (pin) {
      Chunk<Pt> q;
      q.load_at(pin, c * 8, plane);
      q.unpack(a);
      if (v2) {
        float t[8];
        load8(v2 + c * 8, t);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = a[e] + t[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = a[e] + b[e];
    } else if (v2) {
      load8(v2 + c * 8, a);
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = a[e] + b[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = b[e];
    }
    store8(out + c * 8, a);
  }
}

// ---------------------------------------------------------------------------

template <typename St, typename Pt, int TEAM, int CPL>
static hipError_t run_merge(int64_t T, int d, const void* o1, const float* lse1, const void* pin,
                            const void* vprev2, const void* vprev, void* pout, int pout24, const float* w,
                            const float* kg, const float* gamma, float eps, void* h_out, void* x_out,
                            hipStream_t stream) {
  constexpr int TPW = 256 / TEAM;
  const int64_t tiles = (T + TPW - 1) / TPW;
  // persistent: 2 workgroups per CU; 1 for the launches that read two
  // previous outputs and store the partial, over long token ranges (two
  // write streams besides four read streams: fewer concurrent streams kept
  // HBM at 5.4 instead of 5.1 TB/s at 16K tokens, while the lighter launches,
  // and every launch at 2K tokens, were faster with 2)
  const int64_t cus = device_cu_count();
  const int64_t cap = cus * ((vprev2 && T >= 32 * cus) ? 1 : 2);
  const dim3 grid((unsigned)(tiles < cap ? tiles : cap));
  const size_t lds = x_out ? sizeof(float) * (size_t)d : 0;  // PreNorm gain (at most 64 KiB)
  const St* o = static_cast<const St*>(o1);
  const Pt* pi = static_cast<const Pt*>(pin);
  const St* v2 = static_cast<const St*>(vprev2);
  const St* v = static_cast<const St*>(vprev);
  St* h = static_cast<St*>(h_out);
  St* x = static_cast<St*>(x_out);
  // above 60 KiB of dynamic LDS (d > 15360) the static reduction slots take
  // the total past 64 KiB: allow it explicitly
#define ATTNRES_MERGE(V_, PIN_, V2_)                                                                            \
  do {                                                                                                          \
    auto kern = k_merge<St, Pt, TEAM, CPL, V_, PIN_, V2_>;                                                      \
    if (lds > 60 * 1024) {                                                                                      \
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),                            \
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);          \
      if (e != hipSuccess) return e;                                                                            \
    }                                                                                                           \
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, stream, T, d, o, lse1, pi, v2, v, pout, pout24, w, kg, gamma, \
                       eps, h, x);                                                                              \
  } while (0)
  if (!vprev) {
    ATTNRES_MERGE(false, false, false);
  } else if (!pin) {
    if (vprev2) {
      ATTNRES_MERGE(true, false, true);
    } else {
      ATTNRES_MERGE(true, false, false);
    }
  } else if (vprev2) {
    ATTNRES_MERGE(true, true, true);
  } else {
    ATTNRES_MERGE(true, true, false);
  }
#undef ATTNRES_MERGE
  return hipGetLastError();
}

template <typename St, typename Pt>
static hipError_t pick_team(int64_t T, int d, const void* o1, const float* lse1, const void* pin,
                            const void* vprev2, const void* vprev, void* pout, int pout24, const float* w,
                            const float* kg, const float* gamma, float eps, void* h_out, void* x_out,
                            hipStream_t stream) {
  const int C = d >> 3;
#define ATTNRES_RUN_MERGE(TEAM_, CPL_)                                                                             \
  return run_merge<St, Pt, TEAM_, CPL_>(T, d, o1, lse1, pin, vprev2, vprev, pout, pout24, w, kg, gamma, eps, h_out, \
                                        x_out, stream)
  if (C <= 64) ATTNRES_RUN_MERGE(64, 1);
  if (C <= 128) ATTNRES_RUN_MERGE(64, 2);
  if (C <= 256) ATTNRES_RUN_MERGE(64, 4);
  if (C <= 512) ATTNRES_RUN_MERGE(256, 2);
  if (C <= 1024) ATTNRES_RUN_MERGE(256, 4);
  ATTNRES_RUN_MERGE(256, 8);
#undef ATTNRES_RUN_MERGE
}

template <typename St>
static hipError_t pick_pin(Dtype pdt, int64_t T, int d, const void* o1, const float* lse1, const void* pin,
                           const void* vprev2, const void* vprev, void* pout, int pout24, const float* w,
                           const float* kg, const float* gamma, float eps, void* h_out, void* x_out,
                           hipStream_t stream) {
  // without a partial input the partial type is irrelevant: one instance
  if (!pin || pdt == kF32)
    return pick_team<St, float>(T, d, o1, lse1, pin, vprev2, vprev, pout, pout24, w, kg, gamma, eps, h_out, x_out,
                                stream);
  if (pdt == kP24)
    return pick_team<St, p24_t>(T, d, o1, lse1, pin, vprev2, vprev, pout, pout24, w, kg, gamma, eps, h_out, x_out,
                                stream);
  return pick_team<St, St>(T, d, o1, lse1, pin, vprev2, vprev, pout, pout24, w, kg, gamma, eps, h_out, x_out,
                           stream);
}

hipError_t launch_merge(Dtype dt, int64_t T, int d, const void* o1, const float* lse1, Dtype pdt,
                        const void* pin, const void* vprev2, const void* vprev, Dtype podt, void* pout,
                        const float* w, const float* kg, const float* gamma, float eps, void* h_out, void* x_out,
                        hipStream_t stream) {
  const int pout24 = podt == kP24 ? 1 : 0;
  if (dt == kBF16)
    return pick_pin<bf16_t>(pdt, T, d, o1, lse1, pin, vprev2, vprev, pout, pout24, w, kg, gamma, eps, h_out, x_out,
                            stream);
  return pick_pin<float>(pdt, T, d, o1, lse1, pin, vprev2, vprev, pout, pout24, w, kg, gamma, eps, h_out, x_out,
                         stream);
}

template <typename St, typename Pt>
static hipError_t run_acc(int64_t T, int d, const void* pin, const void* v2, const void* v, void* out,
                          hipStream_t stream) {
  const int64_t nchunks = T * (int64_t)(d >> 3);
  const int64_t blocks = (nchunks + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 16;
  const dim3 grid((unsigned)(blocks < cap ? blocks : cap));
  hipLaunchKernelGGL((k_accumulate<St, Pt>), grid, dim3(256), 0, stream, nchunks, static_cast<const Pt*>(pin),
                     static_cast<const St*>(v2), static_cast<const St*>(v), static_cast<St*>(out));
  return hipGetLastError();
}

template <typename St>
static hipError_t acc_pin(Dtype pdt, int64_t T, int d, const void* pin, const void* v2, const void* v, void* out,
                          hipStream_t stream) {
  if (!pin || pdt == kF32) return run_acc<St, float>(T, d, pin, v2, v, out, stream);
  if (pdt == kP24) return run_acc<St, p24_t>(T, d, pin, v2, v, out, stream);
  return run_acc<St, St>(T, d, pin, v2, v, out, stream);
}

hipError_t launch_accumulate(Dtype dt, int64_t T, int d, Dtype pdt, const void* pin, const void* v2,
                             const void* v, void* out, hipStream_t stream) {
  if (dt == kBF16) return acc_pin<bf16_t>(pdt, T, d, pin, v2, v, out, stream);
  return acc_pin<float>(pdt, T, d, pin, v2, v, out, stream);
}

}  // namespace attnres
