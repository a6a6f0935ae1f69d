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
constexpr int kRedWaves = 16;

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
  Chunk<float> r[CPL];
  bool ok[CPL];
};

template <typename St, typename Pt, int TEAM, int CPL, bool HAS_V, bool HAS_PIN, bool HAS_V2>
__device__ __forceinline__ void bissue(BStage<St, Pt, CPL>& s, int64_t tok, int64_t T, int d, int C, int tl,
                                       const St* o1, const Pt* pin, const St* vprev2, const St* vprev,
                                       const St* dx, const float* dpart, int64_t plane) {
  const bool live = tok < T;
  const int64_t tc = live ? tok : T - 1;
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
  hipLaunchKernelGGL(k_wgrad_reduce, dim3((unsigned)((d + 63) / 64)), dim3(64 * kRedWaves), 0, stream, wgs * TPW, d,
                     part, w, kg, vprev ? dw : nullptr, vprev ? dkg : nullptr, prenorm ? dgamma : nullptr, 1);
  return hipGetLastError();
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

// ---------------------------------------------------------------------------
// Phase-1 backward: one 512-thread workgroup per token at a time.  Part I:
// wave w takes the sites j = w, w + 8, ... (QW of them) and walks the row in
// groups of 64 chunks, accumulating G_j.u_i, (w_j (.) g_j).u_i and |u_i|^2 in
// registers (every wave reads all n source chunks; the eight waves of the
// workgroup walk the same groups, so seven of them hit in the caches), then
// DPP wave sums into LDS.  Part II (one thread per site, then one per source)
// forms the coefficients.  Part III: each thread owns chunks of 8 channels
// and writes du_i for all i, re-reading G_j, w_j, g_j and u_i.
constexpr int kP1bThreads = 512;
constexpr int kP1bSites = 32;  // S of one launch

// q = w (.) g for the S sites of a launch (gain NULL: ones).
__global__ __launch_bounds__(256) void k_fold_queries(int64_t n, const float* __restrict__ w,
                                                      const float* __restrict__ kg, float* __restrict__ q) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k < n) q[k] = kg ? w[k] * kg[k] : w[k];
}

// Sites per pass of part I: all QW of the wave's sites for up to 8 bf16
// sources; fewer for more sources or fp32 rows (registers).
template <typename St, int N, int QW>
struct P1bPass {
  static constexpr int kQB = N <= 8 ? (QW == 4 ? 2 : QW) : ((sizeof(St) == 4 || QW == 3) ? 1 : (QW < 2 ? QW : 2));
  static constexpr int kJ3 = N <= 8 ? 4 : 2;  // sites per step of part III
};

template <typename St, int N, int QW>
__global__ __launch_bounds__(kP1bThreads) void k_p1_bwd(int64_t T, int d, const St* __restrict__ src, int64_t stride,
                                                        int S, const float* __restrict__ q, float eps,
                                                        const St* __restrict__ gin, int64_t gstride,
                                                        const float* __restrict__ c_in,
                                                        const float* __restrict__ gp_in, float* __restrict__ dsrc,
                                                        int64_t dstride, int accumulate, float* __restrict__ coef) {
  constexpr int QB = P1bPass<St, N, QW>::kQB;
  constexpr int J3 = P1bPass<St, N, QW>::kJ3;
  const int SP = (S + 7) & ~7;  // sites of the coefficient table, padded
  __shared__ float tD[kP1bSites][N], tZ[kP1bSites][N], tss[N];
  __shared__ float ta[kP1bSites][N], tb[kP1bSites][N], tq[kP1bSites][N], te[N];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int C = d >> 3;
  const int ngroups = (C + 63) >> 6;
  const float inv_d = 1.0f / (float)d;
  for (int64_t tok = blockIdx.x; tok < T; tok += gridDim.x) {
    // ---- part I: dot products over the row, QB of the wave's sites per pass;
    // the next group's chunks load while the current group is used
#pragma unroll
    for (int qb = 0; qb < QW; qb += QB) {
      float D[QB][N], Z[QB][N], ss[N];
#pragma unroll
      for (int i = 0; i < N; ++i) {
        ss[i] = 0.f;
#pragma unroll
        for (int k = 0; k < QB; ++k) D[k][i] = Z[k][i] = 0.f;
      }
      Chunk<St> ua[N], ub[N], ga[QB], gb[QB];
      Chunk<float> qa[QB], qbf[QB];
      auto fetch = [&](Chunk<St>(&u)[N], Chunk<St>(&gq)[QB], Chunk<float>(&qq)[QB], int g) {
        const int c0 = g * 64 + lane;
        const int c = c0 < C ? c0 : C - 1;
#pragma unroll
        for (int i = 0; i < N; ++i) u[i].load(src + i * stride + tok * d + c * 8);
#pragma unroll
        for (int k = 0; k < QB; ++k) {
          const int j0 = wv + 8 * (qb + k);
          const int j = j0 < S ? j0 : S - 1;
          gq[k].load(gin + j * gstride + tok * d + c * 8);
          qq[k].load(q + (int64_t)j * d + c * 8);
        }
      };
      auto consume = [&](const Chunk<St>(&u)[N], const Chunk<St>(&gq)[QB], const Chunk<float>(&qq)[QB], int g) {
        const bool ok = g * 64 + lane < C;
        float gf[QB][8], qf[QB][8];
#pragma unroll
        for (int k = 0; k < QB; ++k) {
          gq[k].unpack(gf[k]);
          qq[k].unpack(qf[k]);
        }
#pragma unroll
        for (int i = 0; i < N; ++i) {
          float ue[8];
          u[i].unpack(ue);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            ue[e] = ok ? ue[e] : 0.f;
            if (qb == 0) ss[i] = fmaf(ue[e], ue[e], ss[i]);
          }
#pragma unroll
          for (int k = 0; k < QB; ++k)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              D[k][i] = fmaf(gf[k][e], ue[e], D[k][i]);
              Z[k][i] = fmaf(qf[k][e], ue[e], Z[k][i]);
            }
        }
      };
      // two-stage ring, ua holding group g at the top of every round.  The
      // rounds have no exit between a load and its use (an exit there lets
      // the compiler sink the loads to their use, which then waits for every
      // load before the dot products), and scheduling barriers keep the next
      // group's loads ahead of the current group's arithmetic.
      fetch(ua, ga, qa, 0);
      int g = 0;
      for (; g + 2 <= ngroups; g += 2) {
        fetch(ub, gb, qbf, g + 1);
        __builtin_amdgcn_sched_barrier(0);
        consume(ua, ga, qa, g);
        __builtin_amdgcn_sched_barrier(0);
        fetch(ua, ga, qa, g + 2 < ngroups ? g + 2 : ngroups - 1);
        __builtin_amdgcn_sched_barrier(0);
        consume(ub, gb, qbf, g + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (g < ngroups) consume(ua, ga, qa, g);
#pragma unroll
      for (int k = 0; k < QB; ++k) {
        const int j = wv + 8 * (qb + k);
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const float dv = wave_sum_dpp(D[k][i]);
          const float zv = wave_sum_dpp(Z[k][i]);
          if (lane == 0 && j < S) {
            tD[j][i] = dv;
            tZ[j][i] = zv;
          }
        }
      }
      if (qb == 0 && wv == 0) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const float sv = wave_sum_dpp(ss[i]);
          if (lane == 0) tss[i] = sv;
        }
      }
    }
    lds_barrier();
    // ---- part II: coefficients, one thread per site
    if ((int)threadIdx.x < S) {
      const int j = threadIdx.x;
      float z[N], a[N];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        z[i] = tZ[j][i] / sqrtf(tss[i] * inv_d + eps);
        mx = fmaxf(mx, z[i]);
      }
      float l = 0.f;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        a[i] = expf(z[i] - mx);
        l += a[i];
      }
      const float c = c_in ? c_in[(int64_t)j * T + tok] : 1.f;
      float go = 0.f;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        a[i] = a[i] / l;
        go = fmaf(a[i], tD[j][i], go);  // G.o, o the phase-1 partition's output
      }
      // G.h = c G.o + (1 - c) G.p, from the same dot products
      const float gh = gp_in ? fmaf(c, go, (1.0f - c) * gp_in[(int64_t)j * T + tok]) : go;
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const float ai = c * a[i];
        const float dz = ai * (tD[j][i] - gh);
        const float ri = 1.0f / sqrtf(tss[i] * inv_d + eps);
        ta[j][i] = ai;
        tb[j][i] = dz * ri;            // dz / r_i: weight of w_j (.) g_j, and of y_i in dw
        tq[j][i] = dz * z[i];
        coef[(tok * SP + j) * N + i] = dz * ri;
      }
    } else if ((int)threadIdx.x < SP) {
      // the table is padded to whole groups of 8 sites with zeros
#pragma unroll
      for (int i = 0; i < N; ++i) coef[(tok * SP + threadIdx.x) * N + i] = 0.f;
    }
    lds_barrier();
    if ((int)threadIdx.x < N) {
      const int i = threadIdx.x;
      float e = 0.f;
      for (int j = 0; j < S; ++j) e += tq[j][i];
      const float ri = 1.0f / sqrtf(tss[i] * inv_d + eps);
      te[i] = e * inv_d * ri * ri;     // coefficient of u_i in the radial term
    }
    lds_barrier();
    // ---- part III: du_i = sum_j a_ji G_j + sum_j b_ji (w_j (.) g_j) - e_i u_i;
    // the next batch of J3 sites loads while the current batch is used
    for (int c = threadIdx.x; c < C; c += kP1bThreads) {
      float du[N][8];
#pragma unroll
      for (int i = 0; i < N; ++i) zero8(du[i]);
      Chunk<St> ga[J3], gb[J3];
      Chunk<float> qa[J3], qbf[J3];
      auto fetch = [&](Chunk<St>(&gq)[J3], Chunk<float>(&qq)[J3], int j0) {
#pragma unroll
        for (int u = 0; u < J3; ++u) {
          const int j = j0 + u < S ? j0 + u : S - 1;
          gq[u].load(gin + j * gstride + tok * d + c * 8);
          qq[u].load(q + (int64_t)j * d + c * 8);
        }
      };
      auto consume = [&](const Chunk<St>(&gq)[J3], const Chunk<float>(&qq)[J3], int j0) {
#pragma unroll
        for (int u = 0; u < J3; ++u) {
          const int j = j0 + u;
          if (j < S) {
            float gf[8], qf[8];
            gq[u].unpack(gf);
            qq[u].unpack(qf);
#pragma unroll
            for (int i = 0; i < N; ++i) {
              const float ai = ta[j][i], bi = tb[j][i];
#pragma unroll
              for (int e = 0; e < 8; ++e) du[i][e] = fmaf(ai, gf[e], fmaf(bi, qf[e], du[i][e]));
            }
          }
        }
      };
      fetch(ga, qa, 0);
      for (int j0 = 0; j0 < S; j0 += 2 * J3) {
        fetch(gb, qbf, j0 + J3);
        consume(ga, qa, j0);
        if (j0 + J3 >= S) break;
        fetch(ga, qa, j0 + 2 * J3);
        consume(gb, qbf, j0 + J3);
      }
#pragma unroll
      for (int i = 0; i < N; ++i) {
        float u[8];
        load8(src + i * stride + tok * d + c * 8, u);
        const float ei = te[i];
        float* dst = dsrc + i * dstride + tok * d + c * 8;
        if (accumulate) {
          float old[8];
          load8(dst, old);
#pragma unroll
          for (int e = 0; e < 8; ++e) du[i][e] = old[e] + (du[i][e] - ei * u[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) du[i][e] = du[i][e] - ei * u[e];
        }
        out8(dst, du[i]);
      }
    }
    lds_barrier();  // the next token rewrites the tables
  }
}

// Weight gradients of the block sources: A_j = sum over tokens and sources
// of (dz_ji / r_i) u_i.  A wave owns one group of 256 channels (4 per lane,
// so all JT <= 32 sites keep their sums in registers and the sources are
// read once) and a range of tokens, with the next token's chunks in flight;
// the range's sums go to part[range][j][d].
constexpr int kWgradWaves = 2048;

template <typename St>
struct Quad;  // 4 consecutive channels
template <>
struct Quad<bf16_t> {
  u32x2_t r;
  __device__ __forceinline__ void load(const bf16_t* p) { r = ld8(p); }
  __device__ __forceinline__ void unpack(float (&v)[4]) const {
    v[0] = __uint_as_float(r.x << 16), v[1] = __uint_as_float(r.x & 0xffff0000u);
    v[2] = __uint_as_float(r.y << 16), v[3] = __uint_as_float(r.y & 0xffff0000u);
  }
};
template <>
struct Quad<float> {
  u32x4_t r;
  __device__ __forceinline__ void load(const float* p) { r = ld16(p); }
  __device__ __forceinline__ void unpack(float (&v)[4]) const {
    v[0] = __uint_as_float(r.x), v[1] = __uint_as_float(r.y), v[2] = __uint_as_float(r.z), v[3] = __uint_as_float(r.w);
  }
};

template <typename St, int N, int JT>
__global__ __launch_bounds__(256) void k_p1_bwd_wgrad(int64_t T, int d, const St* __restrict__ src, int64_t stride,
                                                      int S, const float* __restrict__ coef, int64_t tpr,
                                                      int64_t ranges, float* __restrict__ part) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Q = d >> 2;                 // quads of channels
  const int ngroups = (Q + 63) >> 6;
  const int grp = wid % ngroups;
  const int64_t range = wid / ngroups;
  const int64_t t0 = range * tpr;
  const int64_t t1 = t0 + tpr < T ? t0 + tpr : T;
  const int c0 = grp * 64 + lane;
  const int c = c0 < Q ? c0 : Q - 1;
  float acc[JT][4];
#pragma unroll
  for (int q = 0; q < JT; ++q) acc[q][0] = acc[q][1] = acc[q][2] = acc[q][3] = 0.f;
  Quad<St> ua[N], ub[N];
  auto fetch = [&](Quad<St>(&u)[N], int64_t t) {
    const int64_t tc = t < T ? t : T - 1;
#pragma unroll
    for (int i = 0; i < N; ++i) u[i].load(src + i * stride + tc * d + c * 4);
  };
  // the table holds JT (S rounded up to 8) sites per token, zeros past S
  auto use = [&](const Quad<St>(&u)[N], int64_t t) {
    const float* cf = coef + t * JT * N;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      float ue[4];
      u[i].unpack(ue);
#pragma unroll
      for (int q = 0; q < JT; ++q) {
        const float b = cf[q * N + i];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[q][e] = fmaf(b, ue[e], acc[q][e]);
      }
    }
  };
  if (t0 < t1) fetch(ua, t0);
  for (int64_t t = t0; t < t1; t += 2) {
    fetch(ub, t + 1);
    use(ua, t);
    if (t + 1 >= t1) break;
    fetch(ua, t + 2);
    use(ub, t + 1);
  }
  // every range stores its sums, zeros when it holds no token (the
  // reduction reads all ranges)
  if (c0 < Q && range < ranges) {
#pragma unroll
    for (int q = 0; q < JT; ++q) {
      if (q < S) {
        float* o = part + (range * S + q) * (int64_t)d + c * 4;
        *reinterpret_cast<float4*>(o) = make_float4(acc[q][0], acc[q][1], acc[q][2], acc[q][3]);
      }
    }
  }
}

// dw_j += g_j (.) A_j, dg_j += w_j (.) A_j, A_j summed over the ranges in
// order.  One thread per (site, channel).
__global__ __launch_bounds__(256) void k_p1_bwd_wgrad_reduce(int64_t ranges, int S, int d,
                                                             const float* __restrict__ part,
                                                             const float* __restrict__ w,
                                                             const float* __restrict__ kg, float* __restrict__ dw,
                                                             float* __restrict__ dkg) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k >= (int64_t)S * d) return;
  float A = 0.f;
  for (int64_t r = 0; r < ranges; ++r) A += part[r * S * (int64_t)d + k];
  dw[k] += kg ? kg[k] * A : A;
  if (dkg) dkg[k] += w[k] * A;
}

// Token ranges of the weight-gradient pass (a fixed count, so the
// workspace size and the summation order do not depend on the device).
int64_t p1_backward_ranges(int d) {
  const int ngroups = ((d >> 2) + 63) >> 6;
  return (kWgradWaves + ngroups - 1) / ngroups;
}

template <typename St, int N, int QW>
static hipError_t run_p1b_main(int64_t T, int d, const void* src, int64_t stride, int S, const float* q, float eps,
                               const void* gin, int64_t gstride, const float* c_in, const float* gp_in, float* dsrc,
                               int64_t dstride, int accumulate, float* coef, hipStream_t stream) {
  int64_t wgs = T;
  const int64_t cap = (int64_t)device_cu_count() * 2;
  if (wgs > cap) wgs = cap;
  hipLaunchKernelGGL((k_p1_bwd<St, N, QW>), dim3((unsigned)wgs), dim3(kP1bThreads), 0, stream, T, d,
                     static_cast<const St*>(src), stride, S, q, eps, static_cast<const St*>(gin), gstride, c_in,
                     gp_in, dsrc, dstride, accumulate, coef);
  return hipGetLastError();
}

template <typename St, int N, int JT>
static hipError_t run_p1b_wgrad(int64_t T, int d, const void* src, int64_t stride, int S, const float* coef,
                                float* part, hipStream_t stream) {
  const int64_t ranges = p1_backward_ranges(d);
  const int ngroups = ((d >> 2) + 63) >> 6;
  const int64_t tpr = (T + ranges - 1) / ranges;
  const int64_t waves = ranges * ngroups;
  hipLaunchKernelGGL((k_p1_bwd_wgrad<St, N, JT>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, T, d,
                     static_cast<const St*>(src), stride, S, coef, tpr, ranges, part);
  return hipGetLastError();
}

template <typename St, int N>
static hipError_t run_p1b(int64_t T, int d, const void* src, int64_t stride, int S, const float* w, const float* kg,
                          float eps, const void* gin, int64_t gstride, const float* c_in, const float* gp_in,
                          float* dsrc, int64_t dstride, int accumulate, float* dw, float* dkg, float* ws,
                          hipStream_t stream) {
  // workspace: coefficients [T][S][N], folded queries [S][d], range sums
  float* coef = ws;
  float* q = coef + T * (int64_t)((S + 7) & ~7) * N;
  float* part = q + (int64_t)S * d;
  const int64_t nq = (int64_t)S * d;
  hipLaunchKernelGGL(k_fold_queries, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0, stream, nq, w, kg, q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (S <= 8) {
    e = run_p1b_main<St, N, 1>(T, d, src, stride, S, q, eps, gin, gstride, c_in, gp_in, dsrc, dstride, accumulate,
                               coef, stream);
  } else if (S <= 16) {
    e = run_p1b_main<St, N, 2>(T, d, src, stride, S, q, eps, gin, gstride, c_in, gp_in, dsrc, dstride, accumulate,
                               coef, stream);
  } else if (S <= 24) {
    e = run_p1b_main<St, N, 3>(T, d, src, stride, S, q, eps, gin, gstride, c_in, gp_in, dsrc, dstride, accumulate,
                               coef, stream);
  } else {
    e = run_p1b_main<St, N, 4>(T, d, src, stride, S, q, eps, gin, gstride, c_in, gp_in, dsrc, dstride, accumulate,
                               coef, stream);
  }
  if (e != hipSuccess) return e;
  // (the coefficient table has (S rounded up to 8) sites per token)
  if (S <= 8) {
    e = run_p1b_wgrad<St, N, 8>(T, d, src, stride, S, coef, part, stream);
  } else if (S <= 16) {
    e = run_p1b_wgrad<St, N, 16>(T, d, src, stride, S, coef, part, stream);
  } else if (S <= 24) {
    e = run_p1b_wgrad<St, N, 24>(T, d, src, stride, S, coef, part, stream);
  } else {
    e = run_p1b_wgrad<St, N, 32>(T, d, src, stride, S, coef, part, stream);
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_p1_bwd_wgrad_reduce, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0, stream,
                     p1_backward_ranges(d), S, d, part, w, kg, dw, dkg);
  return hipGetLastError();
}

template <typename St>
static hipError_t pick_p1b(int n, int64_t T, int d, const void* src, int64_t stride, int S, const float* w,
                           const float* kg, float eps, const void* gin, int64_t gstride, const float* c_in,
                           const float* gp_in, float* dsrc, int64_t dstride, int accumulate, float* dw, float* dkg,
                           float* ws, hipStream_t stream) {
  switch (n) {
#define ATTNRES_CASE(N_)                                                                                           \
  case N_:                                                                                                         \
    return run_p1b<St, N_>(T, d, src, stride, S, w, kg, eps, gin, gstride, c_in, gp_in, dsrc, dstride, accumulate, \
                           dw, dkg, ws, stream);
    ATTNRES_CASE(1) ATTNRES_CASE(2) ATTNRES_CASE(3) ATTNRES_CASE(4) ATTNRES_CASE(5) ATTNRES_CASE(6)
    ATTNRES_CASE(7) ATTNRES_CASE(8) ATTNRES_CASE(9) ATTNRES_CASE(10) ATTNRES_CASE(11) ATTNRES_CASE(12)
    ATTNRES_CASE(13) ATTNRES_CASE(14) ATTNRES_CASE(15) ATTNRES_CASE(16)
#undef ATTNRES_CASE
  }
  return hipErrorInvalidValue;
}

hipError_t launch_p1_backward(Dtype dt, int64_t T, int d, const void* src, int n, int64_t stride, int S,
                              const float* w, const float* kg, float eps, const void* gin, int64_t gstride,
                              const float* c_in, const float* gp_in, float* dsrc, int64_t dstride, int accumulate,
                              float* dw, float* dkg, float* ws, hipStream_t stream) {
  // one site without a partial source (the final aggregation): the site
  // backward without PreNorm computes the same gradients, with a team per
  // token instead of one busy wave, into fp32 rows; its weight sums are added
  if (S == 1 && !c_in && !gp_in)
    return launch_site_backward(dt, T, d, src, n, stride, w, kg, nullptr, 0, eps, gin, dsrc, dstride,
                                accumulate ? kOutAdd : kOutF32, 1, dw, dkg, nullptr, ws, stream);
  if (dt == kBF16)
    return pick_p1b<bf16_t>(n, T, d, src, stride, S, w, kg, eps, gin, gstride, c_in, gp_in, dsrc, dstride, accumulate,
                            dw, dkg, ws, stream);
  return pick_p1b<float>(n, T, d, src, stride, S, w, kg, eps, gin, gstride, c_in, gp_in, dsrc, dstride, accumulate, dw,
                         dkg, ws, stream);
}

}  // namespace attnres
