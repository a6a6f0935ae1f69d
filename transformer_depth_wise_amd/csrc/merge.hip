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
// channels; the row's two reductions (|p|^2 with w.p, then |h|^2) use DPP
// row steps with scalar lane reads inside a wave (a few tens of cycles, where
// a shuffle butterfly waits on six LDS round trips) and, for 256-thread
// teams, one LDS exchange each.  The per-channel parameters stay on chip (w
// (.) g in registers, gamma in LDS) while a persistent grid of two
// workgroups per CU walks over the tokens; the raw rows of the team's next
// token are loaded before the current token is reduced, merged and stored,
// so HBM traffic continues through the reductions and barriers (the loop is
// unrolled twice over two register stages).  When every workgroup has a
// single token (short token ranges) nothing is prefetched.  Every row load
// and store is non-temporal: each row is used once per launch, and what a
// later launch reads again is far larger than the caches (with non-temporal
// loads and stores phase 2 of the 16K-token chunk took 37.4 ms instead of
// 40.0 on one MI355X, measured in one run).
#include "attnres_device.h"
#include "attnres_launch.h"

namespace attnres {


template <typename St, typename Pt, int CPL>
struct Stage {
  Chunk<St> o[CPL], v[CPL], v2[CPL];
  Chunk<Pt> q[CPL];
  RowExp<Pt> qe;
  float lse;  // the phase-1 log-sum-exp of the token (with a partial-sum source)
  bool ok[CPL];
};

// Formats of the stored partial sum (pfmt).
constexpr int kPoutF32 = 0, kPoutP24 = 1, kPoutQ16 = 2;

// Loads of one token for the team.  Every load is unconditional (an
// out-of-range token or chunk reads a clamped valid address and is zeroed
// when used), so the loads of a stage issue back to back.  ONE (the team's
// only token): the token's phase-1 log-sum-exp comes with them; otherwise it
// is loaded where it is used.
template <typename St, typename Pt, int TEAM, int CPL, bool HAS_V, bool HAS_PIN, bool HAS_V2, bool ONE>
__device__ __forceinline__ void issue(Stage<St, Pt, CPL>& s, int64_t tok, int64_t T, int d, int C, int tl,
                                      const St* o1, const float* lse1, const Pt* pin, const St* vprev2,
                                      const St* vprev, int64_t plane) {
  const bool live = tok < T;
  const int64_t tc = live ? tok : T - 1;
  if (HAS_PIN) s.qe.load(pin, tc, plane);
  if (HAS_V && ONE) s.lse = lse1[tc];
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int c0 = tl + TEAM * k;
    s.ok[k] = live && c0 < C;
    const int c = c0 < C ? c0 : C - 1;
    const int64_t off = tc * d + c * 8;
    s.o[k].load_nt(o1 + off);
    if (HAS_V) s.v[k].load_nt(vprev + off);
    if (HAS_V2) s.v2[k].load_nt(vprev2 + off);
    if (HAS_PIN) s.q[k].load_at_nt(pin, off, plane);
  }
}

// ONE: the log-sum-exp is in the stage and the PreNorm gain of the thread's
// chunks in gg (else the gain is read from LDS).
template <typename St, typename Pt, int TEAM, int CPL, bool HAS_V, bool HAS_PIN, bool HAS_V2, bool ONE>
__device__ __forceinline__ void process(const Stage<St, Pt, CPL>& s, int64_t tok, int64_t T, int d, int C, int tl,
                                        const float* lse1, void* pout, int pfmt, int64_t plane,
                                        const float (&wq)[CPL][8], const float4* gm_lds,
                                        const float (&gg)[CPL][8], float eps, float inv_d, St* h_out, St* x_out,
                                        float (*red)[12], int& parity) {
  const bool live = tok < T;
  // a Q16 partial is stored after the row's largest magnitude is known
  const bool q16 = pout && pfmt == kPoutQ16;
  float h[CPL][8], p[CPL][8];
  float ss = 0.f, dot = 0.f, amax = 0.f;
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    s.o[k].unpack(h[k]);
    if (HAS_V) {
      // p = ((partial or 0) + (v_prev2 or 0)) + v_prev, in that order
      float v[8];
      s.v[k].unpack(v);
      if (HAS_PIN) {
        unpack_partial(s.q[k], s.qe, p[k]);
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
      if (pout && !q16 && s.ok[k]) {
        const int64_t off = tok * d + c * 8;
        if (pfmt == kPoutP24) {
          out24_nt(static_cast<p24_t*>(pout), off, plane, p[k]);
        } else {
          out8_nt(static_cast<float*>(pout) + off, p[k]);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ss = fmaf(p[k][e], p[k][e], ss);
        dot = fmaf(wq[k][e], p[k][e], dot);
        amax = fmaxf(amax, fabsf(p[k][e]));
      }
    }
  }
  if (HAS_V) {
    float2 r;
    if (q16) {
      // one exchange for both sums and the row's largest magnitude
      float pmax;
      if (TEAM == 256) {
        const float3 r3 = block_sum2_max_256<true>(ss, dot, amax, red[parity]);
        parity ^= 1;
        r = make_float2(r3.x, r3.y);
        pmax = r3.z;
      } else {
        r.x = wave_sum_dpp(ss);
        r.y = wave_sum_dpp(dot);
        pmax = wave_max_dpp(amax);
      }
      const int e = q16_exponent(pmax);
      unsigned char* pb = static_cast<unsigned char*>(pout);
#pragma unroll
      for (int k = 0; k < CPL; ++k)
        if (s.ok[k]) st16_nt(pb + (tok * d + (tl + TEAM * k) * 8) * 2, q16_pack(p[k], e));
      if (live && tl == 0) *reinterpret_cast<int*>(pb + plane * 2 + tok * 4) = e;
    } else if (TEAM == 256) {
      r = block_sum2_256<true>(ss, dot, red[parity]);
      parity ^= 1;
    } else {
      r.x = wave_sum_dpp(ss);
      r.y = wave_sum_dpp(dot);
    }
    const float zc = r.y / sqrtf(r.x * inv_d + eps);
    const float lse = ONE ? s.lse : lse1[live ? tok : T - 1];
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
      r2 = block_sum2_256<true>(sh, 0.f, red[parity]).x;
      parity ^= 1;
    } else {
      r2 = wave_sum_dpp(sh);
    }
  }
  const float rinv = x_out ? 1.0f / sqrtf(r2 * inv_d + eps) : 1.f;
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    if (s.ok[k]) {
      const int64_t off = tok * d + (tl + TEAM * k) * 8;
      if (h_out) out8_nt(h_out + off, h[k]);
      if (x_out) {
        float gk[8];
        if (ONE) {
#pragma unroll
          for (int e = 0; e < 8; ++e) gk[e] = gg[k][e];
        } else {
          const float4 g0 = gm_lds[2 * (tl + TEAM * k)], g1 = gm_lds[2 * (tl + TEAM * k) + 1];
          gk[0] = g0.x, gk[1] = g0.y, gk[2] = g0.z, gk[3] = g0.w;
          gk[4] = g1.x, gk[5] = g1.y, gk[6] = g1.z, gk[7] = g1.w;
        }
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = gk[e] * (h[k][e] * rinv);
        out8_nt(x_out + off, x);
      }
    }
  }
}

template <typename St, typename Pt, int TEAM, int CPL, bool HAS_V, bool HAS_PIN, bool HAS_V2>
__global__ __launch_bounds__(256) void k_merge(int64_t T, int d, const St* __restrict__ o1,
                                               const float* __restrict__ lse1, const Pt* __restrict__ pin,
                                               const St* __restrict__ vprev2, const St* __restrict__ vprev,
                                               void* __restrict__ pout, int pfmt,
                                               const float* __restrict__ w, const float* __restrict__ kg,
                                               const float* __restrict__ gamma, float eps,
                                               St* __restrict__ h_out, St* __restrict__ x_out) {
  constexpr int TPW = 256 / TEAM;
  const int64_t plane = T * (int64_t)d;
  __shared__ float red[2][12];
  // the PreNorm gain, used once per token at the very end, waits in LDS; the
  // folded query w (.) g stays in registers
  extern __shared__ float4 gm_lds[];  // [d / 4]
  const int team = threadIdx.x / TEAM;
  const int tl = threadIdx.x % TEAM;
  const int C = d >> 3;
  const float inv_d = 1.0f / (float)d;
  int parity = 0;
  const int64_t step = (int64_t)gridDim.x * TPW;
  int64_t tok = (int64_t)blockIdx.x * TPW + team;
  if (step >= T) {
    // Every team has one token (short token ranges): its rows and phase-1
    // log-sum-exp are loaded first, then the parameters of the thread's own
    // chunks (the PreNorm gain too, kept in registers), with no prefetch
    // (which would share the compute unit's load path with the live rows)
    // and no barrier before the first reduction.  The arithmetic is that of
    // the persistent path below, so results do not depend on the path.
    Stage<St, Pt, CPL> A;
    issue<St, Pt, TEAM, CPL, HAS_V, HAS_PIN, HAS_V2, true>(A, tok, T, d, C, tl, o1, lse1, pin, vprev2, vprev, plane);
    float wq[CPL][8], gg[CPL][8];
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int c0 = tl + TEAM * k;
      const int c = c0 < C ? c0 : C - 1;
      if (HAS_V) {
        load8(w + c * 8, wq[k]);
        float gq[8];
        if (kg) {
          load8(kg + c * 8, gq);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) gq[e] = 1.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) wq[k][e] = c0 < C ? wq[k][e] * gq[e] : 0.f;
      } else {
        zero8(wq[k]);
      }
      if (x_out && gamma) {
        load8(gamma + c * 8, gg[k]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) gg[k][e] = 1.f;
      }
    }
    process<St, Pt, TEAM, CPL, HAS_V, HAS_PIN, HAS_V2, true>(A, tok, T, d, C, tl, lse1, pout, pfmt, plane, wq, gm_lds,
                                                              gg, eps, inv_d, h_out, x_out, red, parity);
    return;
  }
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
  Stage<St, Pt, CPL> A, B;
  issue<St, Pt, TEAM, CPL, HAS_V, HAS_PIN, HAS_V2, false>(A, tok, T, d, C, tl, o1, lse1, pin, vprev2, vprev, plane);
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
  // The loads of a workgroup's next token are unconditional (a token past
  // the end reads a clamped row), so the waits for the current token's rows
  // leave them in flight.  The log-sum-exp is loaded where it is used: the
  // wait for it then also drains the next token's rows before this token's
  // stores, which measured 2% faster at 16K tokens than loading it with the
  // rows.
  while (tok - team < T) {
    // the next token's loads are issued at a raised wave priority, so that
    // they leave the SIMD ahead of the arithmetic of the other workgroup's
    // waves (3.5-6.5% faster merges at the 16K chunk than at equal priority)
    __builtin_amdgcn_s_setprio(2);
    issue<St, Pt, TEAM, CPL, HAS_V, HAS_PIN, HAS_V2, false>(B, tok + step, T, d, C, tl, o1, lse1, pin, vprev2, vprev,
                                                            plane);
    __builtin_amdgcn_s_setprio(0);
    process<St, Pt, TEAM, CPL, HAS_V, HAS_PIN, HAS_V2, false>(A, tok, T, d, C, tl, lse1, pout, pfmt, plane, wq,
                                                               gm_lds, wq, eps, inv_d, h_out, x_out, red, parity);
    tok += step;
    if (tok - team >= T) break;
    __builtin_amdgcn_s_setprio(2);
    issue<St, Pt, TEAM, CPL, HAS_V, HAS_PIN, HAS_V2, false>(A, tok + step, T, d, C, tl, o1, lse1, pin, vprev2, vprev,
                                                            plane);
    __builtin_amdgcn_s_setprio(0);
    process<St, Pt, TEAM, CPL, HAS_V, HAS_PIN, HAS_V2, false>(B, tok, T, d, C, tl, lse1, pout, pfmt, plane, wq,
                                                               gm_lds, wq, eps, inv_d, h_out, x_out, red, parity);
    tok += step;
  }
}

// out = ((partial or 0) + (v2 or 0)) + v, in that order; the sum is stored
// as Ot (the rows' type, or fp32).  A workgroup item is a segment of 256
// chunks of one row (a partial sum's row exponent is read once per item), a
// thread one chunk, so at short token ranges every load of the launch is in
// flight at once.
template <typename St, typename Pt, typename Ot>
__global__ __launch_bounds__(256) void k_accumulate(int64_t T, int d, const Pt* __restrict__ pin,
                                                    const St* __restrict__ v2, const St* __restrict__ v,
                                                    Ot* __restrict__ out) {
  const int C = d >> 3;
  const int nseg = (C + 255) >> 8;
  const int64_t plane = T * (int64_t)d;
  const int64_t items = T * nseg;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int64_t t = it / nseg;
    const int c = (int)(it - t * nseg) * 256 + (int)threadIdx.x;
    RowExp<Pt> qe;
    if (pin) qe.load(pin, t, plane);
    if (c < C) {
      const int64_t off = t * d + c * 8;
      float a[8], b[8];
      load8(v + off, b);
      if (pin) {
        Chunk<Pt> q;
        q.load_at(pin, off, plane);
        unpack_partial(q, qe, a);
        if (v2) {
          float x[8];
          load8(v2 + off, x);
#pragma unroll
          for (int e = 0; e < 8; ++e) a[e] = a[e] + x[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = a[e] + b[e];
      } else if (v2) {
        load8(v2 + off, a);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = a[e] + b[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = b[e];
      }
      store8(out + off, a);
    }
  }
}

// ---------------------------------------------------------------------------

template <typename St, typename Pt, int TEAM, int CPL>
static hipError_t run_merge(int64_t T, int d, const void* o1, const float* lse1, const void* pin,
                            const void* vprev2, const void* vprev, void* pout, int pfmt, const float* w,
                            const float* kg, const float* gamma, float eps, void* h_out, void* x_out,
                            hipStream_t stream) {
  constexpr int TPW = 256 / TEAM;
  const int64_t tiles = (T + TPW - 1) / TPW;
  // Up to 8 tiles per CU, a workgroup per tile (the kernel's one-token path,
  // which keeps the PreNorm gain in registers: no dynamic LDS).  Beyond,
  // persistent: 2 workgroups per CU (with non-temporal accesses every
  // instance was fastest so; 1 per CU cost 7%).
  const int64_t cu = device_cu_count();
  const bool one = tiles <= 8 * cu;
  const int64_t cap = one ? tiles : cu * 2;
  const dim3 grid((unsigned)(tiles < cap ? tiles : cap));
  const size_t lds = (x_out && !one) ? sizeof(float) * (size_t)d : 0;  // PreNorm gain (at most 64 KiB)
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
    hipLaunchKernelGGL(kern, grid, dim3(256), lds, stream, T, d, o, lse1, pi, v2, v, pout, pfmt, w, kg, gamma, \
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
                            const void* vprev2, const void* vprev, void* pout, int pfmt, const float* w,
                            const float* kg, const float* gamma, float eps, void* h_out, void* x_out,
                            hipStream_t stream) {
  const int C = d >> 3;
#define ATTNRES_RUN_MERGE(TEAM_, CPL_)                                                                             \
  return run_merge<St, Pt, TEAM_, CPL_>(T, d, o1, lse1, pin, vprev2, vprev, pout, pfmt, w, kg, gamma, eps, h_out, \
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
                           const void* vprev2, const void* vprev, void* pout, int pfmt, const float* w,
                           const float* kg, const float* gamma, float eps, void* h_out, void* x_out,
                           hipStream_t stream) {
  // without a partial input the partial type is irrelevant: one instance
  if (!pin || pdt == kF32)
    return pick_team<St, float>(T, d, o1, lse1, pin, vprev2, vprev, pout, pfmt, w, kg, gamma, eps, h_out, x_out,
                                stream);
  if (pdt == kQ16)
    return pick_team<St, q16_t>(T, d, o1, lse1, pin, vprev2, vprev, pout, pfmt, w, kg, gamma, eps, h_out, x_out,
                                stream);
  if (pdt == kP24)
    return pick_team<St, p24_t>(T, d, o1, lse1, pin, vprev2, vprev, pout, pfmt, w, kg, gamma, eps, h_out, x_out,
                                stream);
  return pick_team<St, St>(T, d, o1, lse1, pin, vprev2, vprev, pout, pfmt, w, kg, gamma, eps, h_out, x_out,
                           stream);
}

hipError_t launch_merge(Dtype dt, int64_t T, int d, const void* o1, const float* lse1, Dtype pdt,
                        const void* pin, const void* vprev2, const void* vprev, Dtype podt, void* pout,
                        const float* w, const float* kg, const float* gamma, float eps, void* h_out, void* x_out,
                        hipStream_t stream) {
  const int pfmt = podt == kP24 ? kPoutP24 : podt == kQ16 ? kPoutQ16 : kPoutF32;
  if (dt == kBF16)
    return pick_pin<bf16_t>(pdt, T, d, o1, lse1, pin, vprev2, vprev, pout, pfmt, w, kg, gamma, eps, h_out, x_out,
                            stream);
  return pick_pin<float>(pdt, T, d, o1, lse1, pin, vprev2, vprev, pout, pfmt, w, kg, gamma, eps, h_out, x_out,
                         stream);
}

template <typename St, typename Pt, typename Ot>
static hipError_t run_acc(int64_t T, int d, const void* pin, const void* v2, const void* v, void* out,
                          hipStream_t stream) {
  const int64_t cap = (int64_t)device_cu_count() * 8;
  const int64_t items = T * (((d >> 3) + 255) >> 8);
  const dim3 grid((unsigned)(items < cap ? items : cap));
  hipLaunchKernelGGL((k_accumulate<St, Pt, Ot>), grid, dim3(256), 0, stream, T, d, static_cast<const Pt*>(pin),
                     static_cast<const St*>(v2), static_cast<const St*>(v), static_cast<Ot*>(out));
  return hipGetLastError();
}

template <typename St, typename Ot>
static hipError_t acc_pin(Dtype pdt, int64_t T, int d, const void* pin, const void* v2, const void* v, void* out,
                          hipStream_t stream) {
  if (!pin || pdt == kF32) return run_acc<St, float, Ot>(T, d, pin, v2, v, out, stream);
  if (pdt == kQ16) return run_acc<St, q16_t, Ot>(T, d, pin, v2, v, out, stream);
  if (pdt == kP24) return run_acc<St, p24_t, Ot>(T, d, pin, v2, v, out, stream);
  return run_acc<St, St, Ot>(T, d, pin, v2, v, out, stream);
}

hipError_t launch_accumulate(Dtype dt, Dtype odt, int64_t T, int d, Dtype pdt, const void* pin, const void* v2,
                             const void* v, void* out, hipStream_t stream) {
  if (dt == kBF16 && odt == kF32) return acc_pin<bf16_t, float>(pdt, T, d, pin, v2, v, out, stream);
  if (dt == kBF16) return acc_pin<bf16_t, bf16_t>(pdt, T, d, pin, v2, v, out, stream);
  return acc_pin<float, float>(pdt, T, d, pin, v2, v, out, stream);
}

}  // namespace attnres
