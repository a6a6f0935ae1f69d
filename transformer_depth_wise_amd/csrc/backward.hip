// Backward of one depth-aggregation site on gfx950 (training).
//
// Forward of the site (one query over n sources, "Attention Residuals"
// notes, section 7):  y_i = u_i / r(u_i),  z_i = (w (.) g)^T y_i,
// alpha = softmax(z),  h = sum_i alpha_i u_i,  x = gamma (.) h / r(h)  (or
// x = h without PreNorm).  Given dx = dL/dx per token:
//   G_h  = (gamma (.) dx - y_h (y_h^T (gamma (.) dx)) / d) / r(h),  y_h = h/r(h)
//          (the RMSNorm backward of "Attention Residuals 阅读补充", gradients
//          along the tangent; G_h = dx without PreNorm),
//   dz_i = alpha_i G_h^T (u_i - h)        (the notes' logit gradient),
//   du_i = alpha_i G_h + (dz_i (w (.) g) - y_i z_i dz_i / d) / r(u_i)
//          (value path + score path through the key RMSNorm; the radial term
//          uses y_i^T (w (.) g) = z_i),
//   dw = g (.) A,  dg = w (.) A,  A = sum_tokens sum_i dz_i y_i,
//   dgamma = sum_tokens dx (.) y_h.
//
// One team of threads per token row, each thread owning one or two chunks of
// 8 channels (teams of 64 to 1024 threads by d); the per-source values of
// the current token sit in a small LDS table written by one thread.  For
// d <= 8192 all n rows of a token are loaded once, together, into registers
// (at most 16 rows x 2 chunks); wider rows are re-read by each pass (L2).
// Per token: pass 1 reduces the rows' sums of squares and scores in one
// batch; pass 2 forms h, reads dx and reduces |h|^2 and (gamma dx) . h;
// pass 3 reduces G_h . u_i and G_h . h; pass 4 writes du_i.  Every reduction is a fixed-order
// team reduction (wave shuffles, then waves in index order through LDS).  A
// and the dgamma sums are accumulated per thread over the team's tokens,
// written per team to the workspace, and summed over teams in a fixed order
// by a second kernel: no atomics, bitwise reproducible.
#include "backward_common.h"

namespace attnres {

template <typename St, int TEAM, int CPL, bool HOLD, int NR, int OUT>
__global__ __launch_bounds__(TEAM < 256 ? 256 : TEAM) void k_site_backward(
    int64_t T, int d, const St* __restrict__ src, int n, int64_t stride, const float* __restrict__ w,
    const float* __restrict__ kg, const float* __restrict__ gamma, int prenorm, float eps,
    const St* __restrict__ dx, void* __restrict__ dsrc_v, int64_t dstride, float* __restrict__ part) {
  constexpr bool ACC = OUT == kOutAdd;
  using Dt = typename std::conditional<OUT == kOutStore, St, float>::type;
  Dt* const dsrc = static_cast<Dt*>(dsrc_v);
  constexpr int WG = TEAM < 256 ? 256 : TEAM;
  constexpr int TPW = WG / TEAM;
  constexpr int NW = TEAM / kWave;
  constexpr int NV = 2 * NR + 2;  // NR: rows this instance handles (n <= NR)
  constexpr int kB = TEAM >= 1024 ? 2 : kBwdBatch;  // rows per load batch (registers of the widest teams)
  // HOLD: all n rows of the token are loaded once, together, and kept in
  // registers for the four passes (the per-thread sums and w (.) g then live
  // in LDS); otherwise every pass re-reads the rows (L2) and the sums and
  // w (.) g stay in registers
  Chunk<St> held[HOLD ? NR : 1][CPL];
  __shared__ float red[2][TPW][NW * NV];
  // per-source values of the team's current token: 1/r(u_i), z_i, alpha_i, dz_i
  __shared__ float sv[TPW][4][kBwdMax];
  // HOLD: [2][CPL * 8][WG] per-thread sums (A, dgamma), then w (.) g [d]
  extern __shared__ float dyn[];
  const int team = threadIdx.x / TEAM;
  const int tl = threadIdx.x % TEAM;
  const int wv = tl / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int C = d >> 3;
  const float inv_d = 1.0f / (float)d;
  float* const s_ri = sv[team][0];
  float* const s_z = sv[team][1];
  float* const s_al = sv[team][2];
  float* const s_dz = sv[team][3];
  float* const wq_lds = dyn + 2 * CPL * 8 * WG;
  auto acc = [&](int which, int c8, int e) -> float& {
    return dyn[((which * CPL + c8) * 8 + e) * WG + threadIdx.x];
  };
  bool ok[CPL];
  int cc[CPL];
#pragma unroll
  for (int c8 = 0; c8 < CPL; ++c8) {
    const int c0 = tl + TEAM * c8;
    ok[c8] = c0 < C;
    cc[c8] = ok[c8] ? c0 : C - 1;
  }
  float wr[HOLD ? 1 : CPL][8], accA[HOLD ? 1 : CPL][8], accG[HOLD ? 1 : CPL][8];
#pragma unroll
  for (int c8 = 0; c8 < CPL; ++c8) {
    float wv8[8], g8[8];
    load8(w + cc[c8] * 8, wv8);
    if (kg) {
      load8(kg + cc[c8] * 8, g8);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) g8[e] = 1.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float q = ok[c8] ? wv8[e] * g8[e] : 0.f;
      if (HOLD) {
        acc(0, c8, e) = 0.f;
        acc(1, c8, e) = 0.f;
      } else {
        wr[c8][e] = q;
        accA[c8][e] = 0.f;
        accG[c8][e] = 0.f;
      }
    }
    if (HOLD && ok[c8] && team == 0) {
      float4* q4 = reinterpret_cast<float4*>(wq_lds + cc[c8] * 8);
      q4[0] = make_float4(wv8[0] * g8[0], wv8[1] * g8[1], wv8[2] * g8[2], wv8[3] * g8[3]);
      q4[1] = make_float4(wv8[4] * g8[4], wv8[5] * g8[5], wv8[6] * g8[6], wv8[7] * g8[7]);
    }
  }
  if (HOLD) lds_barrier();
  // w (.) g for chunk c8 of this thread
  auto wq = [&](int c8, float (&q)[8]) {
    if (HOLD) {
      const float4* q4 = reinterpret_cast<const float4*>(wq_lds + cc[c8] * 8);
      const float4 a = q4[0], b = q4[1];
      q[0] = a.x; q[1] = a.y; q[2] = a.z; q[3] = a.w; q[4] = b.x; q[5] = b.y; q[6] = b.z; q[7] = b.w;
      if (!ok[c8]) zero8(q);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = wr[HOLD ? 0 : c8][e];
    }
  };
  int parity = 0;
  const int64_t step = (int64_t)gridDim.x * TPW;
  // every team of a workgroup runs the same number of iterations (the
  // reductions synchronise the workgroup); tokens past T are clamped and
  // neither stored nor accumulated
  for (int64_t tok = (int64_t)blockIdx.x * TPW + team; tok - team < T; tok += step) {
    const bool live = tok < T;
    const int64_t tc = live ? tok : T - 1;
    const St* base = src + tc * d;
    Chunk<St> dxc[CPL];
#pragma unroll
    for (int c8 = 0; c8 < CPL; ++c8) dxc[c8].load(dx + tc * d + cc[c8] * 8);
    if (HOLD) {
#pragma unroll
      for (int i = 0; i < NR; ++i) {
        const int ic = i < n ? i : n - 1;  // clamped: always a valid row
#pragma unroll
        for (int c8 = 0; c8 < CPL; ++c8) held[HOLD ? i : 0][c8].load(base + (int64_t)ic * stride + cc[c8] * 8);
      }
    }
    // row i of the token, chunk c8 (held, or loaded now)
    auto row = [&](int i, int c8) -> Chunk<St> {
      Chunk<St> ch;
      if (HOLD) {
        ch = held[HOLD ? i : 0][c8];
      } else {
        ch.load(base + (int64_t)(i < n ? i : n - 1) * stride + cc[c8] * 8);
      }
      return ch;
    };
    // ---- pass 1: |u_i|^2 and (w (.) g) . u_i
    {
      float v[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) v[i] = 0.f;
#pragma unroll
      for (int c8 = 0; c8 < CPL; ++c8) {
        float q[8];
        wq(c8, q);
#pragma unroll
        for (int b0 = 0; b0 < NR; b0 += kB) {
          if (b0 < n) {
            Chunk<St> u[kB];
#pragma unroll
            for (int r = 0; r < kB; ++r) u[r] = row(b0 + r, c8);
#pragma unroll
            for (int r = 0; r < kB; ++r) {
              if (b0 + r < n) {  // uniform: padding rows of the batch are skipped
                float f[8];
                u[r].unpack(f);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                  const float x = ok[c8] ? f[e] : 0.f;
                  v[2 * (b0 + r)] = fmaf(x, x, v[2 * (b0 + r)]);
                  v[2 * (b0 + r) + 1] = fmaf(q[e], x, v[2 * (b0 + r) + 1]);
                }
              }
            }
          }
        }
      }
      team_reduce<NW, NV>(v, &red[parity][team][0], wv, lane);
      parity ^= 1;
      // lane i of the team's first wave handles source i; max and sum over
      // the n sources with DPP (lanes >= n contribute -inf / 0)
      if (wv == 0) {
        float ss = 0.f, dt = 0.f;
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          ss = lane == i ? v[2 * i] : ss;
          dt = lane == i ? v[2 * i + 1] : dt;
        }
        const bool src_lane = lane < n;
        const float ri = 1.0f / sqrtf(ss * inv_d + eps);
        const float zi = src_lane ? dt * ri : -INFINITY;
        float M = zi;
        M = fmaxf(M, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(M), 0xB1, 0xF, 0xF, false)));
        M = fmaxf(M, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(M), 0x4E, 0xF, 0xF, false)));
        M = fmaxf(M, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(M), 0x141, 0xF, 0xF, false)));
        M = fmaxf(M, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(M), 0x140, 0xF, 0xF, false)));
        if (NR > 16) M = fmaxf(M, __shfl_xor(M, 16));  // rows of 16 lanes: 0-15 with 16-31
        const float e = src_lane ? expf(zi - M) : 0.f;
        const float den = wave_sum_dpp(e);  // lanes >= n hold zeros
        if (src_lane) {
          s_ri[lane] = ri;
          s_z[lane] = zi;
          s_al[lane] = e / den;
        }
      }
      lds_barrier();
    }
    // ---- pass 2: h, dx, then G_h (PreNorm backward)
    float h[CPL][8], gdx[CPL][8];
#pragma unroll
    for (int c8 = 0; c8 < CPL; ++c8) {
      zero8(h[c8]);
#pragma unroll
      for (int b0 = 0; b0 < NR; b0 += kB) {
        if (b0 < n) {
          Chunk<St> u[kB];
#pragma unroll
          for (int r = 0; r < kB; ++r) u[r] = row(b0 + r, c8);
#pragma unroll
          for (int r = 0; r < kB; ++r)
            if (b0 + r < n) {
              const float a = s_al[b0 + r];
              float f[8];
              u[r].unpack(f);
#pragma unroll
              for (int e = 0; e < 8; ++e) h[c8][e] = fmaf(a, f[e], h[c8][e]);
            }
        }
      }
      dxc[c8].unpack(gdx[c8]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (!ok[c8]) h[c8][e] = 0.f;
        gdx[c8][e] = ok[c8] ? gdx[c8][e] : 0.f;
      }
    }
    if (prenorm) {
      float gm[CPL][8];
#pragma unroll
      for (int c8 = 0; c8 < CPL; ++c8) {
        if (gamma) {
          load8(gamma + cc[c8] * 8, gm[c8]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) gm[c8][e] = 1.f;
        }
      }
      float p2[2] = {0.f, 0.f};
#pragma unroll
      for (int c8 = 0; c8 < CPL; ++c8)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p2[0] = fmaf(h[c8][e], h[c8][e], p2[0]);
          p2[1] = fmaf(gm[c8][e] * gdx[c8][e], h[c8][e], p2[1]);
        }
      team_reduce<NW, 2>(p2, &red[parity][team][0], wv, lane);
      parity ^= 1;
      const float rh = 1.0f / sqrtf(p2[0] * inv_d + eps);
      const float cr = p2[1] * rh * rh * rh * inv_d;
#pragma unroll
      for (int c8 = 0; c8 < CPL; ++c8)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (live) {
            if (HOLD) {
              acc(1, c8, e) = fmaf(gdx[c8][e], h[c8][e] * rh, acc(1, c8, e));
            } else {
              accG[HOLD ? 0 : c8][e] = fmaf(gdx[c8][e], h[c8][e] * rh, accG[HOLD ? 0 : c8][e]);
            }
          }
          gdx[c8][e] = gm[c8][e] * gdx[c8][e] * rh - h[c8][e] * cr;  // G_h
        }
    }
    // ---- pass 3: G_h . u_i and G_h . h -> dz_i
    {
      float v[NR + 1];
#pragma unroll
      for (int i = 0; i <= NR; ++i) v[i] = 0.f;
#pragma unroll
      for (int c8 = 0; c8 < CPL; ++c8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[NR] = fmaf(gdx[c8][e], h[c8][e], v[NR]);
#pragma unroll
        for (int b0 = 0; b0 < NR; b0 += kB) {
          if (b0 < n) {
            Chunk<St> u[kB];
#pragma unroll
            for (int r = 0; r < kB; ++r) u[r] = row(b0 + r, c8);
#pragma unroll
            for (int r = 0; r < kB; ++r) {
              if (b0 + r < n) {
                float f[8];
                u[r].unpack(f);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[b0 + r] = fmaf(gdx[c8][e], ok[c8] ? f[e] : 0.f, v[b0 + r]);
              }
            }
          }
        }
      }
      // the NR source sums and G_h . h (entry NR) in one reduction
      team_reduce<NW, NR + 1>(v, &red[parity][team][0], wv, lane);
      parity ^= 1;
      if (wv == 0) {
        float di = 0.f;
#pragma unroll
        for (int i = 0; i < NR; ++i) di = lane == i ? v[i] : di;
        if (lane < n) s_dz[lane] = s_al[lane] * (di - v[NR]);
      }
      lds_barrier();
    }
    // ---- pass 4: du_i and the A sums
#pragma unroll
    for (int c8 = 0; c8 < CPL; ++c8) {
      float q[8], tA[8];
      wq(c8, q);
      zero8(tA);
#pragma unroll
      for (int b0 = 0; b0 < NR; b0 += kB) {
        if (b0 < n) {
          Chunk<St> u[kB];
#pragma unroll
          for (int r = 0; r < kB; ++r) u[r] = row(b0 + r, c8);
          // ACC: the batch's earlier contributions, loaded together before
          // its stores (a load after a store of the same array would wait)
          float old[ACC ? kB : 1][8];
          if constexpr (ACC) {
#pragma unroll
            for (int r = 0; r < kB; ++r)
              if (b0 + r < n && live && ok[c8])
                load8(dsrc + (int64_t)(b0 + r) * dstride + tok * d + cc[c8] * 8, old[r]);
          }
#pragma unroll
          for (int r = 0; r < kB; ++r) {
            const int i = b0 + r;
            if (i < n) {
              const float a = s_al[i], g = s_dz[i], ri = s_ri[i], zi = s_z[i];
              float f[8], o[8];
              u[r].unpack(f);
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const float y = f[e] * ri;
                o[e] = fmaf(a, gdx[c8][e], g * ri * (q[e] - y * zi * inv_d));
                tA[e] = fmaf(g, y, tA[e]);
              }
              if (live && ok[c8]) {
                if constexpr (ACC) {
#pragma unroll
                  for (int e = 0; e < 8; ++e) o[e] += old[r][e];
                }
                store8(dsrc + (int64_t)i * dstride + tok * d + cc[c8] * 8, o);
              }
            }
          }
        }
      }
      if (live && ok[c8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (HOLD) {
            acc(0, c8, e) += tA[e];
          } else {
            accA[HOLD ? 0 : c8][e] += tA[e];
          }
        }
      }
    }
    // the next token's pass 1 rewrites the per-source values only after its
    // own reduction barrier, which every lane reaches after finishing here
  }
  // per-team partial sums: part[slot][0][d] = A, part[slot][1][d] = dgamma
  const int64_t slot = (int64_t)blockIdx.x * TPW + team;
  float* pa = part + slot * 2 * (int64_t)d;
#pragma unroll
  for (int c8 = 0; c8 < CPL; ++c8)
    if (ok[c8]) {
      float A8[8], G8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        A8[e] = HOLD ? acc(0, c8, e) : accA[HOLD ? 0 : c8][e];
        G8[e] = HOLD ? acc(1, c8, e) : accG[HOLD ? 0 : c8][e];
      }
      out8(pa + cc[c8] * 8, A8);
      out8(pa + d + cc[c8] * 8, G8);
    }
}

// Sum the per-team partials part[slot][0..1][d] in a fixed order: wave q of
// a workgroup adds a contiguous sixteenth of the slots for 64 channels, then
// the first wave adds the sixteen partial sums in wave order.  dw = g (.) A,
// dg = w (.) A, dgamma = G; with `add` they are added to the outputs instead
// of written.

__global__ __launch_bounds__(64 * kRedWaves) void k_wgrad_reduce(int64_t slots, int d,
                                                                 const float* __restrict__ part,
                                                                 const float* __restrict__ w,
                                                                 const float* __restrict__ kg,
                                                                 float* __restrict__ dw, float* __restrict__ dkg,
                                                                 float* __restrict__ dgamma, int add) {
  __shared__ float sums[kRedWaves][2][64];
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int k = blockIdx.x * 64 + lane;
  const int kc = k < d ? k : d - 1;
  const int64_t s0 = (slots * q) / kRedWaves, s1 = (slots * (q + 1)) / kRedWaves;
  float A = 0.f, G = 0.f;
  // unrolled so that eight slots' loads are in flight at once; the adds
  // keep slot order
#pragma unroll 8
  for (int64_t s = s0; s < s1; ++s) {
    A += part[s * 2 * (int64_t)d + kc];
    G += part[s * 2 * (int64_t)d + d + kc];
  }
  sums[q][0][lane] = A;
  sums[q][1][lane] = G;
  lds_barrier();
  if (q == 0 && k < d) {
    A = 0.f, G = 0.f;
    for (int r = 0; r < kRedWaves; ++r) {
      A += sums[r][0][lane];
      G += sums[r][1][lane];
    }
    const float a = kg ? kg[k] * A : A;
    if (dw) dw[k] = add ? dw[k] + a : a;
    if (dkg) dkg[k] = add ? dkg[k] + w[k] * A : w[k] * A;
    if (dgamma) dgamma[k] = add ? dgamma[k] + G : G;
  }
}

int backward_team(int d) {
  const int C = d >> 3;
  if (C <= 128) return 64;
  if (C <= 256) return 256;
  if (C <= 1024) return 512;
  return 1024;
}

int64_t backward_slots(int64_t T, int d) {
  const int team = backward_team(d);
  const int tpw = team < 256 ? 256 / team : 1;
  const int64_t wgs = (T + tpw - 1) / tpw;
  return (wgs < 1024 ? wgs : 1024) * tpw;
}

template <typename St, int TEAM, int CPL, bool HOLD, int NR, int OUT>
static hipError_t run_bwd(int64_t T, int d, const void* src, int n, int64_t stride, const float* w,
                          const float* kg, const float* gamma, int prenorm, float eps, const void* dx, void* dsrc,
                          int64_t dstride, int wadd, float* dw, float* dkg, float* dgamma, float* part,
                          hipStream_t stream) {
  constexpr int WG = TEAM < 256 ? 256 : TEAM;
  constexpr int TPW = WG / TEAM;
  int64_t wgs = (T + TPW - 1) / TPW;
  const int64_t cap = (int64_t)device_cu_count() * (TEAM >= 512 ? 1 : 2);  // one or two resident per CU
  if (wgs > cap) wgs = cap;
  if (wgs > 1024) wgs = 1024;
  const size_t lds = HOLD ? sizeof(float) * ((size_t)2 * CPL * 8 * WG + (size_t)d) : 0;
  if (lds > 48 * 1024) {
    const hipError_t e =
        hipFuncSetAttribute(reinterpret_cast<const void*>(k_site_backward<St, TEAM, CPL, HOLD, NR, OUT>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_site_backward<St, TEAM, CPL, HOLD, NR, OUT>), dim3((unsigned)wgs), dim3(WG), lds, stream, T,
                     d, static_cast<const St*>(src), n, stride, w, kg, gamma, prenorm, eps, static_cast<const St*>(dx),
                     dsrc, dstride, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_wgrad_reduce, dim3((unsigned)((d + 63) / 64)), dim3(64 * kRedWaves), 0, stream, wgs * TPW, d,
                     part, w, kg, dw, dkg, prenorm ? dgamma : nullptr, wadd);
  return hipGetLastError();
}

// More than 16 sources: the rows are re-read from L2 in every pass instead
// of held in registers.
template <typename St, int OUT>
static hipError_t pick_bwd(int64_t T, int d, const void* src, int n, int64_t stride, const float* w, const float* kg,
                           const float* gamma, int prenorm, float eps, const void* dx, void* dsrc, int64_t dstride,
                           int wadd, float* dw, float* dkg, float* dgamma, float* part, hipStream_t stream) {
  const int C = d >> 3;
#define ATTNRES_BWD(TEAM_, CPL_, HOLD_, NR_)                                                                  \
  return run_bwd<St, TEAM_, CPL_, HOLD_, NR_, OUT>(T, d, src, n, stride, w, kg, gamma, prenorm, eps, dx, dsrc, \
                                                   dstride, wadd, dw, dkg, dgamma, part, stream)
#define ATTNRES_BWD_HOLD(TEAM_, CPL_)                  \
  do {                                                 \
    if (n > 16) ATTNRES_BWD(TEAM_, CPL_, false, 32);   \
    if (n <= 8) ATTNRES_BWD(TEAM_, CPL_, true, 8);     \
    if (n <= 12) ATTNRES_BWD(TEAM_, CPL_, true, 12);   \
    ATTNRES_BWD(TEAM_, CPL_, true, 16);               \
  } while (0)
  if (C <= 64) ATTNRES_BWD_HOLD(64, 1);
  if (C <= 128) ATTNRES_BWD_HOLD(64, 2);
  if (C <= 256) ATTNRES_BWD_HOLD(256, 1);
  if (C <= 512) ATTNRES_BWD_HOLD(512, 1);
  if (C <= 1024) ATTNRES_BWD_HOLD(512, 2);
  if (n > 16) ATTNRES_BWD(1024, 2, false, 32);
  ATTNRES_BWD(1024, 2, false, 16);
#undef ATTNRES_BWD_HOLD
#undef ATTNRES_BWD
}

hipError_t launch_site_backward(Dtype dt, int64_t T, int d, const void* src, int n, int64_t stride, const float* w,
                                const float* kg, const float* gamma, int prenorm, float eps, const void* dx,
                                void* dsrc, int64_t dstride, int out_mode, int wadd, float* dw, float* dkg,
                                float* dgamma, float* part, hipStream_t stream) {
#define ATTNRES_SB(ST_, OUT_)                                                                                    \
  return pick_bwd<ST_, OUT_>(T, d, src, n, stride, w, kg, gamma, prenorm, eps, dx, dsrc, dstride, wadd, dw, dkg, \
                             dgamma, part, stream)
  if (dt == kBF16) {
    if (out_mode == kOutAdd) ATTNRES_SB(bf16_t, kOutAdd);
    if (out_mode == kOutF32) ATTNRES_SB(bf16_t, kOutF32);
    ATTNRES_SB(bf16_t, kOutStore);
  }
  // fp32 rows: storing in the storage type is storing fp32
  if (out_mode == kOutAdd) ATTNRES_SB(float, kOutAdd);
  ATTNRES_SB(float, kOutStore);
#undef ATTNRES_SB
}



hipError_t launch_wgrad_reduce(int64_t slots, int d, const float* part, const float* w, const float* kg, float* dw,
                               float* dkg, float* dgamma, int add, hipStream_t stream) {
  hipLaunchKernelGGL(k_wgrad_reduce, dim3((unsigned)((d + 63) / 64)), dim3(64 * kRedWaves), 0, stream, slots, d, part,
                     w, kg, dw, dkg, dgamma, add);
  return hipGetLastError();
}

// Token ranges of the weight-gradient pass (a fixed count, so the
// workspace size and the summation order do not depend on the device).
int64_t p1_backward_ranges(int d) {
  const int ngroups = ((d >> 2) + 63) >> 6;
  return (kWgradWaves + ngroups - 1) / ngroups;
}

hipError_t launch_p1_backward(Dtype dt, Dtype sdt, int64_t T, int d, const void* src, int n, int64_t stride, int S,
                              const float* w, const float* kg, float eps, const void* gin, int64_t gstride,
                              const float* c_in, const float* gp_in, float* dsrc, int64_t dstride, int accumulate,
                              float* dw, float* dkg, float* ws, hipStream_t stream) {
  // one site without a partial source (the final aggregation), rows of one
  // type: the site backward without PreNorm computes the same gradients, with
  // a team per token instead of one busy wave, into fp32 rows; its weight
  // sums are added
  if (S == 1 && !c_in && !gp_in && sdt == dt)
    return launch_site_backward(dt, T, d, src, n, stride, w, kg, nullptr, 0, eps, gin, dsrc, dstride,
                                accumulate ? kOutAdd : kOutF32, 1, dw, dkg, nullptr, ws, stream);
  if (sdt == kF32 && dt == kBF16)
    return launch_p1b_f32src(n, T, d, src, stride, S, w, kg, eps, gin, gstride, c_in, gp_in, dsrc, dstride,
                             accumulate, dw, dkg, ws, stream);
  if (dt == kBF16)
    return launch_p1b_bf16(n, T, d, src, stride, S, w, kg, eps, gin, gstride, c_in, gp_in, dsrc, dstride, accumulate,
                           dw, dkg, ws, stream);
  return launch_p1b_f32(n, T, d, src, stride, S, w, kg, eps, gin, gstride, c_in, gp_in, dsrc, dstride, accumulate, dw,
                        dkg, ws, stream);
}

}  // namespace attnres
