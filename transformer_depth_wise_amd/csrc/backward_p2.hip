#include "backward_common.h"

namespace attnres {

// ===========================================================================
// Backward through the block structure, split like the forward's two phases.
//
// Site j of a block reads the block sources u_1..u_n (b_0..b_{n-1}) and,
// after the block's first sublayer, the partial sum p_j.  With the phase-1
// partition (o_j normalised, lse_j) and beta_j = alpha of p_j, the forward
// is h_j = o_j + beta_j (p_j - o_j), and every block source has weight
// alpha_ji = (1 - beta_j) alpha1_ji, alpha1 the phase-1 softmax.  Backward,
// in reverse sublayer order (each sublayer's output gradient is complete
// only once every later site has run):
//
//  phase-2 backward, one launch per site (k_p2_bwd): recompute p_j, beta_j
//    and h_j, apply the PreNorm backward to get G_j = dL/dh_j, store G_j and
//    the per-token scalars c_j = 1 - beta_j and G_j.p_j, and add the partial
//    source's gradient
//        dp_j = beta_j G_j + dz_jp (w (.) g - y_p z_jp / d) / r(p_j),
//        dz_jp = beta_j G_j.(p_j - h_j)
//    into the running fp32 gradient of the block's outputs (the notes'
//    logit gradient, "Attention Residuals" notes, section 7; the RMSNorm
//    backward of "Attention Residuals 阅读补充", gradients along the tangent).
//
//  phase-1 backward, one launch per block (k_p1_bwd): for every token, the
//    S x n dot products G_j.u_i and (w_j (.) g_j).u_i and the sums of squares
//    of the sources give z_ji, alpha1_ji, dz_ji = c_j alpha1_ji (G_j.u_i -
//    G_j.h_j), and then, for all S sites at once,
//        du_i = sum_j c_j alpha1_ji G_j + r_i^-1 (sum_j dz_ji (w_j (.) g_j)
//               - y_i sum_j dz_ji z_ji / d),
//    added into the fp32 gradients of the sources.  G_j.h_j is formed there
//    from the same dot products, c_j sum_k alpha1_jk G_j.u_k + (1 - c_j)
//    G_j.p_j, not from the stored phase-1 output: when one source dominates,
//    u_i - h_j is small and the storage rounding of o_j would be a large part
//    of it.  The weight gradients of
//    the block sources, sum over tokens and i of dz_ji y_i, are a contraction
//    over rows: a separate channel-group-major pass (k_p1_bwd_wgrad) keeps
//    per-lane sums for its channels over a range of tokens, and a fixed-order
//    reduction adds them up (no atomics).

template <typename St, typename Pt, int CPL>
struct BStage {
  Chunk<St> o[CPL], v[CPL], v2[CPL], dx[CPL];
  Chunk<Pt> q[CPL];
  RowExp<Pt> qe;
  Chunk<float> r[CPL];
  bool ok[CPL];
};

template <typename St, typename Pt, int TEAM, int CPL, bool HAS_V, bool HAS_PIN, bool HAS_V2>
__device__ __forceinline__ void bissue(BStage<St, Pt, CPL>& s, int64_t tok, int64_t T, int d, int C, int tl,
                                       const St* o1, const Pt* pin, const St* vprev2, const St* vprev,
                                       const St* dx, const float* dpart, int64_t plane) {
  const bool live = tok < T;
  const int64_t tc = live ? tok : T - 1;
  if (HAS_PIN) s.qe.load(pin, tc, plane);
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int c0 = tl + TEAM * k;
    s.ok[k] = live && c0 < C;
    const int c = c0 < C ? c0 : C - 1;
    const int64_t off = tc * d + c * 8;
    s.o[k].load(o1 + off);
    s.dx[k].load(dx + off);
    if (HAS_V) {
      s.v[k].load(vprev + off);
      s.r[k].load(dpart + off);
    }
    if (HAS_V2) s.v2[k].load(vprev2 + off);
    if (HAS_PIN) s.q[k].load_at(pin, off, plane);
  }
}

__device__ __forceinline__ void lds8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w, v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
}

// Per-thread sums over the team's tokens: in LDS ([element][thread], so a
// wave's accesses are consecutive) or, for the widest teams, in registers.
template <int CPL, bool ACC_LDS>
struct BAcc {
  float r[ACC_LDS ? 1 : 2][ACC_LDS ? 1 : CPL * 8];
  float* lds;
  int stride, th;
  __device__ __forceinline__ void init(float* base, int wg, int thread) {
    lds = base, stride = wg, th = thread;
#pragma unroll
    for (int e = 0; e < CPL * 8; ++e) {
      if (ACC_LDS) {
        lds[e * stride + th] = 0.f;
        lds[(CPL * 8 + e) * stride + th] = 0.f;
      } else {
        r[0][e] = 0.f;
        r[1][e] = 0.f;
      }
    }
  }
  __device__ __forceinline__ void add(int which, int e, float x) {
    if (ACC_LDS) {
      lds[(which * CPL * 8 + e) * stride + th] += x;
    } else {
      r[which][e] += x;
    }
  }
  __device__ __forceinline__ float get(int which, int e) const {
    return ACC_LDS ? lds[(which * CPL * 8 + e) * stride + th] : r[which][e];
  }
};

template <typename St, int TEAM, int CPL, bool HAS_V, bool HAS_PIN, bool HAS_V2, bool ACC_LDS, typename Pt>
__device__ __forceinline__ void bprocess(const BStage<St, Pt, CPL>& s, int64_t tok, int64_t T, int d, int C,
                                         int tl, int wv, int lane, const float* lse1, const float* wql,
                                         const float* gml, int prenorm, float eps, float inv_d, float* dpart,
                                         St* g_out, float* c_out, float* gp_out, BAcc<CPL, ACC_LDS>& acc,
                                         float* red, int& parity) {
  constexpr int NW = TEAM / kWave;
  const bool live = tok < T;
  float h[CPL][8], p[CPL][8], G[CPL][8];
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    s.o[k].unpack(h[k]);
    s.dx[k].unpack(G[k]);
    if (HAS_V) {
      // p = ((partial or 0) + (v_prev2 or 0)) + v_prev, as the forward merge
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
      G[k][e] = s.ok[k] ? G[k][e] : 0.f;  // dx for now
    }
  }
  float beta = 0.f, zc = 0.f, rp = 1.f;
  if (HAS_V) {
    float r1[2] = {0.f, 0.f};
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      float wq[8];
      lds8(wql + (tl + TEAM * k) * 8, wq);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        r1[0] = fmaf(p[k][e], p[k][e], r1[0]);
        r1[1] = fmaf(wq[e], p[k][e], r1[1]);
      }
    }
    team_reduce<NW, 2>(r1, red + parity * NW * 4, wv, lane);
    parity ^= 1;
    rp = sqrtf(r1[0] * inv_d + eps);
    zc = r1[1] / rp;
    const float lse = lse1[live ? tok : T - 1];
    beta = 1.0f / (1.0f + expf(lse - zc));
#pragma unroll
    for (int k = 0; k < CPL; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) h[k][e] = fmaf(beta, p[k][e] - h[k][e], h[k][e]);
  }
  if (prenorm) {
    // G = (gamma dx - h (h . gamma dx) / (d r(h)^2)) / r(h); dgamma += dx (.) h / r(h)
    float r2[2] = {0.f, 0.f};
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      float gm[8];
      lds8(gml + (tl + TEAM * k) * 8, gm);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        r2[0] = fmaf(h[k][e], h[k][e], r2[0]);
        r2[1] = fmaf(h[k][e], gm[e] * G[k][e], r2[1]);
      }
    }
    team_reduce<NW, 2>(r2, red + parity * NW * 4, wv, lane);
    parity ^= 1;
    const float rhi = 1.0f / sqrtf(r2[0] * inv_d + eps);
    const float k2 = r2[1] * rhi * rhi * inv_d;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      float gm[8];
      lds8(gml + (tl + TEAM * k) * 8, gm);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float dxe = G[k][e];
        acc.add(1, k * 8 + e, dxe * (h[k][e] * rhi));
        G[k][e] = (gm[e] * dxe - h[k][e] * k2) * rhi;
      }
    }
  }
  // G as stored (the phase-1 backward reads it back): G.p of the stored
  // values keeps G.(u_i - h) consistent there
  float r3[2] = {0.f, 0.f};
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    float gr[8];
    if (sizeof(St) == 2) {
      Chunk<bf16_t> c;
      c.r = u32x4_t{pack_bf16x2(G[k][0], G[k][1]), pack_bf16x2(G[k][2], G[k][3]), pack_bf16x2(G[k][4], G[k][5]),
                    pack_bf16x2(G[k][6], G[k][7])};
      c.unpack(gr);
      if (s.ok[k]) st16(g_out + tok * d + (tl + TEAM * k) * 8, c.r);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) gr[e] = G[k][e];
      if (s.ok[k]) out8(g_out + tok * d + (tl + TEAM * k) * 8, G[k]);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      r3[0] = fmaf(gr[e], p[k][e], r3[0]);
      r3[1] = fmaf(G[k][e], p[k][e] - h[k][e], r3[1]);
    }
  }
  if (HAS_V) {
    team_reduce<NW, 2>(r3, red + parity * NW * 4, wv, lane);
    parity ^= 1;
  }
  if (tl == 0 && live) {
    c_out[tok] = 1.0f - beta;
    gp_out[tok] = HAS_V ? r3[0] : 0.f;
  }
  if (HAS_V) {
    const float dz = beta * r3[1];
    const float rpi = 1.0f / rp;
    const float zd = zc * inv_d;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      float r[8], wq[8];
      s.r[k].unpack(r);
      lds8(wql + (tl + TEAM * k) * 8, wq);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float yp = p[k][e] * rpi;
        acc.add(0, k * 8 + e, dz * yp);
        r[e] = r[e] + fmaf(beta, G[k][e], dz * (wq[e] - yp * zd) * rpi);
      }
      if (s.ok[k]) out8(dpart + tok * d + (tl + TEAM * k) * 8, r);
    }
  }
}

// Dynamic LDS of the phase-2 backward: w (.) g and gamma ([d] each, padded to
// whole team sweeps), then the per-thread sums when they live in LDS.
static size_t p2b_lds_bytes(int team, int cpl, bool acc_lds) {
  const int wg = team < 256 ? 256 : team;
  const size_t padded = (size_t)team * cpl * 8;
  return sizeof(float) * (2 * padded + (acc_lds ? (size_t)2 * cpl * 8 * wg : 0));
}

template <typename St, typename Pt, int TEAM, int CPL, bool HAS_V, bool HAS_PIN, bool HAS_V2, bool DB>
__global__ __launch_bounds__(TEAM < 256 ? 256 : TEAM) void k_p2_bwd(
    int64_t T, int d, const St* __restrict__ o1, const float* __restrict__ lse1, const Pt* __restrict__ pin,
    const St* __restrict__ vprev2, const St* __restrict__ vprev, const float* __restrict__ w,
    const float* __restrict__ kg, const float* __restrict__ gamma, int prenorm, float eps,
    const St* __restrict__ dx, float* __restrict__ dpart, St* __restrict__ g_out, float* __restrict__ c_out,
    float* __restrict__ gp_out, float* __restrict__ part) {
  constexpr int WG = TEAM < 256 ? 256 : TEAM;
  constexpr int TPW = WG / TEAM;
  constexpr int NW = TEAM / kWave;
  constexpr bool ACC_LDS = TEAM <= 512;
  constexpr int PAD = TEAM * CPL * 8;
  __shared__ float red[TPW][2 * NW * 4];
  extern __shared__ float p2lds[];
  float* wql = p2lds;
  float* gml = p2lds + PAD;
  const int team = threadIdx.x / TEAM;
  const int tl = threadIdx.x % TEAM;
  const int wv = tl / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int C = d >> 3;
  const float inv_d = 1.0f / (float)d;
  const int64_t plane = T * (int64_t)d;
  int parity = 0;
  const int64_t step = (int64_t)gridDim.x * TPW;
  int64_t tok = (int64_t)blockIdx.x * TPW + team;
  BStage<St, Pt, CPL> A, B;
  bissue<St, Pt, TEAM, CPL, HAS_V, HAS_PIN, HAS_V2>(A, tok, T, d, C, tl, o1, pin, vprev2, vprev, dx, dpart, plane);
  // parameters to LDS (w (.) g zero past d) while the first token loads
  for (int k = threadIdx.x; k < PAD; k += WG) {
    const bool in = k < d;
    wql[k] = in ? w[k] * (kg ? kg[k] : 1.f) : 0.f;
    gml[k] = in ? (gamma ? gamma[k] : 1.f) : 0.f;
  }
  BAcc<CPL, ACC_LDS> acc;
  acc.init(p2lds + 2 * PAD, WG, threadIdx.x);
  lds_barrier();
  if (DB) {
    while (tok - team < T) {
      bissue<St, Pt, TEAM, CPL, HAS_V, HAS_PIN, HAS_V2>(B, tok + step, T, d, C, tl, o1, pin, vprev2, vprev, dx, dpart,
                                                        plane);
      bprocess<St, TEAM, CPL, HAS_V, HAS_PIN, HAS_V2, ACC_LDS>(A, tok, T, d, C, tl, wv, lane, lse1, wql, gml, prenorm,
                                                               eps, inv_d, dpart, g_out, c_out, gp_out, acc,
                                                               red[team], parity);
      tok += step;
      if (tok - team >= T) break;
      bissue<St, Pt, TEAM, CPL, HAS_V, HAS_PIN, HAS_V2>(A, tok + step, T, d, C, tl, o1, pin, vprev2, vprev, dx, dpart,
                                                        plane);
      bprocess<St, TEAM, CPL, HAS_V, HAS_PIN, HAS_V2, ACC_LDS>(B, tok, T, d, C, tl, wv, lane, lse1, wql, gml, prenorm,
                                                               eps, inv_d, dpart, g_out, c_out, gp_out, acc,
                                                               red[team], parity);
      tok += step;
    }
  } else {
    while (tok - team < T) {
      bprocess<St, TEAM, CPL, HAS_V, HAS_PIN, HAS_V2, ACC_LDS>(A, tok, T, d, C, tl, wv, lane, lse1, wql, gml, prenorm,
                                                               eps, inv_d, dpart, g_out, c_out, gp_out, acc,
                                                               red[team], parity);
      tok += step;
      if (tok - team >= T) break;
      bissue<St, Pt, TEAM, CPL, HAS_V, HAS_PIN, HAS_V2>(A, tok, T, d, C, tl, o1, pin, vprev2, vprev, dx, dpart,
                                                        plane);
    }
  }
  // this team's sums over its tokens: [slot][A, dgamma][d]
  const int64_t slot = (int64_t)blockIdx.x * TPW + team;
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int c = tl + TEAM * k;
    if (c < C) {
      float a[8], g[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[e] = acc.get(0, k * 8 + e);
        g[e] = acc.get(1, k * 8 + e);
      }
      out8(part + slot * 2 * (int64_t)d + c * 8, a);
      out8(part + slot * 2 * (int64_t)d + d + c * 8, g);
    }
  }
}

// Teams of the phase-2 backward by row width (each thread one or two chunks).
static void p2b_team(int d, int& team, int& cpl) {
  const int C = d >> 3;
  if (C <= 64) { team = 64; cpl = 1; }
  else if (C <= 128) { team = 64; cpl = 2; }
  else if (C <= 256) { team = 256; cpl = 1; }
  else if (C <= 512) { team = 256; cpl = 2; }
  else if (C <= 1024) { team = 512; cpl = 2; }
  else { team = 1024; cpl = 2; }
}

int64_t p2_backward_slots(int64_t T, int d) {
  int team, cpl;
  p2b_team(d, team, cpl);
  const int tpw = team < 256 ? 256 / team : 1;
  const int64_t wgs = (T + tpw - 1) / tpw;
  return (wgs < 1024 ? wgs : 1024) * tpw;
}

template <typename St, typename Pt, int TEAM, int CPL>
static hipError_t run_p2b(int64_t T, int d, const void* o1, const float* lse1, const void* pin, const void* vprev2,
                          const void* vprev, const float* w, const float* kg, const float* gamma, int prenorm,
                          float eps, const void* dx, float* dpart, void* g_out, float* c_out, float* gp_out,
                          float* dw, float* dkg, float* dgamma, float* part, hipStream_t stream) {
  constexpr int WG = TEAM < 256 ? 256 : TEAM;
  constexpr int TPW = WG / TEAM;
  int64_t wgs = (T + TPW - 1) / TPW;
  int64_t cap = (int64_t)device_cu_count() * (WG >= 512 ? 1 : 2);
  if (cap > 1024) cap = 1024;
  if (wgs > cap) wgs = cap;
  const St* o = static_cast<const St*>(o1);
  const Pt* pi = static_cast<const Pt*>(pin);
  const St* v2 = static_cast<const St*>(vprev2);
  const St* v = static_cast<const St*>(vprev);
  const St* g = static_cast<const St*>(dx);
  St* go = static_cast<St*>(g_out);
  // one token's rows at a time for the widest teams and fp32 rows (registers)
  constexpr bool DB = TEAM < 1024 && (sizeof(St) == 2 || TEAM < 512);
  const size_t lds = p2b_lds_bytes(TEAM, CPL, TEAM <= 512);
#define ATTNRES_P2B(V_, PIN_, V2_)                                                                                \
  do {                                                                                                            \
    auto kern = k_p2_bwd<St, Pt, TEAM, CPL, V_, PIN_, V2_, DB>;                                                   \
    if (lds > 48 * 1024) {                                                                                        \
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),                              \
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);            \
      if (e != hipSuccess) return e;                                                                              \
    }                                                                                                             \
    hipLaunchKernelGGL(kern, dim3((unsigned)wgs), dim3(WG), lds, stream, T, d, o, lse1, pi, v2, v, w, kg, gamma,  \
                       prenorm, eps, g, dpart, go, c_out, gp_out, part);                                          \
  } while (0)
  if (!vprev) {
    ATTNRES_P2B(false, false, false);
  } else if (!pin) {
    if (vprev2) {
      ATTNRES_P2B(true, false, true);
    } else {
      ATTNRES_P2B(true, false, false);
    }
  } else if (vprev2) {
    ATTNRES_P2B(true, true, true);
  } else {
    ATTNRES_P2B(true, true, false);
  }
#undef ATTNRES_P2B
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_wgrad_reduce(wgs * TPW, d, part, w, kg, vprev ? dw : nullptr, vprev ? dkg : nullptr,
                             prenorm ? dgamma : nullptr, 1, stream);
}

template <typename St, typename Pt>
static hipError_t pick_p2b(int64_t T, int d, const void* o1, const float* lse1, const void* pin, const void* vprev2,
                           const void* vprev, const float* w, const float* kg, const float* gamma, int prenorm,
                           float eps, const void* dx, float* dpart, void* g_out, float* c_out, float* gp_out,
                           float* dw, float* dkg, float* dgamma, float* part, hipStream_t stream) {
  int team, cpl;
  p2b_team(d, team, cpl);
#define ATTNRES_P2B_RUN(TEAM_, CPL_)                                                                              \
  if (team == TEAM_ && cpl == CPL_)                                                                               \
  return run_p2b<St, Pt, TEAM_, CPL_>(T, d, o1, lse1, pin, vprev2, vprev, w, kg, gamma, prenorm, eps, dx, dpart, \
                                      g_out, c_out, gp_out, dw, dkg, dgamma, part, stream)
  ATTNRES_P2B_RUN(64, 1);
  ATTNRES_P2B_RUN(64, 2);
  ATTNRES_P2B_RUN(256, 1);
  ATTNRES_P2B_RUN(256, 2);
  ATTNRES_P2B_RUN(512, 2);
  ATTNRES_P2B_RUN(1024, 2);
#undef ATTNRES_P2B_RUN
  return hipErrorInvalidValue;
}

hipError_t launch_p2_backward(Dtype dt, int64_t T, int d, const void* o1, const float* lse1, Dtype pdt,
                              const void* pin, const void* vprev2, const void* vprev, const float* w, const float* kg,
                              const float* gamma, int prenorm, float eps, const void* dx, float* dpart, void* g_out,
                              float* c_out, float* gp_out, float* dw, float* dkg, float* dgamma, float* part,
                              hipStream_t stream) {
#define ATTNRES_P2B_PIN(St_)                                                                                       \
  do {                                                                                                             \
    if (!pin || pdt == kF32)                                                                                       \
      return pick_p2b<St_, float>(T, d, o1, lse1, pin, vprev2, vprev, w, kg, gamma, prenorm, eps, dx, dpart, g_out, \
                                  c_out, gp_out, dw, dkg, dgamma, part, stream);                                   \
    if (pdt == kQ16)                                                                                               \
      return pick_p2b<St_, q16_t>(T, d, o1, lse1, pin, vprev2, vprev, w, kg, gamma, prenorm, eps, dx, dpart, g_out, \
                                  c_out, gp_out, dw, dkg, dgamma, part, stream);                                   \
    if (pdt == kP24)                                                                                               \
      return pick_p2b<St_, p24_t>(T, d, o1, lse1, pin, vprev2, vprev, w, kg, gamma, prenorm, eps, dx, dpart, g_out, \
                                  c_out, gp_out, dw, dkg, dgamma, part, stream);                                   \
    return pick_p2b<St_, St_>(T, d, o1, lse1, pin, vprev2, vprev, w, kg, gamma, prenorm, eps, dx, dpart, g_out,     \
                              c_out, gp_out, dw, dkg, dgamma, part, stream);                                       \
  } while (0)
  if (dt == kBF16) ATTNRES_P2B_PIN(bf16_t);
  ATTNRES_P2B_PIN(float);
#undef ATTNRES_P2B_PIN
}


}  // namespace attnres
