#pragma once
// Private to libattnres: the phase-1 backward kernels as templates over the
// source rows' type Ut and the type St of the sites' G rows (equal, or fp32
// sources with bf16 G), instantiated by one translation unit per pair.
#include "backward_common.h"

namespace attnres {

// ---------------------------------------------------------------------------
// Phase-1 backward: one 512-thread workgroup per token at a time.  Part I
// with bf16 G rows runs on the matrix cores (p1b_part1_mfma below).  With
// fp32 G rows it runs on the vector ALUs: wave w takes the sites j = w, w + 8,
// ... (QW of them) and walks the row in groups of 64 chunks, accumulating
// G_j.u_i, (w_j (.) g_j).u_i and |u_i|^2 in registers (every wave reads all n
// source chunks; the eight waves of the workgroup walk the same groups, so
// seven of them hit in the caches), then DPP wave sums into LDS.  Part II
// (one thread per site, then one per source) forms the coefficients.  Part
// III: each thread owns chunks of 8 channels and writes du_i for all i,
// re-reading G_j, w_j, g_j and u_i.
constexpr int kP1bThreads = 512;
constexpr int kP1bSites = 32;  // S of one launch

// q = w (.) g for the S sites of a launch (gain NULL: ones).
static __global__ __launch_bounds__(256) void k_fold_queries(int64_t n, const float* __restrict__ w,
                                                      const float* __restrict__ kg, float* __restrict__ q) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k < n) q[k] = kg ? w[k] * kg[k] : w[k];
}

// Part I on the matrix cores (G rows in bf16).  Per token, D = G U^T and
// Z = Q U^T (32 sites x 16 sources, padded) over d in k-steps of 32
// channels: v_mfma_f32_16x16x32_bf16 with the sources split into bf16 high
// and low parts when they are fp32 (D = G U_hi + G U_lo; Z = Q_hi U_hi +
// Q_lo U_hi + Q_hi U_lo), so products keep ~16 mantissa bits.  The token's G
// and source rows come through LDS in groups of kP1bGE channels, loaded by
// whole-row pieces (each wave instruction covers contiguous bytes of one or
// two rows); the 8 waves take one k-step of a group each, and their partial
// sums are added in wave order at the end of the token.  The folded queries
// are packed once per launch as A operands: word ((ks * 2 + m) * 2 + h) * 64
// + lane holds, for site m * 16 + (lane & 15), channels ks * 32 + (lane >>
// 4) * 8 .. + 7, high (h = 0) or low (h = 1) bf16 parts.
constexpr int kP1bGE = 256;                // channels per staged group (8 k-steps)
constexpr int kP1bRow = kP1bGE + 8;        // staged row length in bf16 (16-byte pad)
constexpr int kP1bStage = 64 * kP1bRow;    // bf16 per LDS buffer: G [32], U_hi [16], U_lo [16]
constexpr int kP1bPieces = 4;              // 16-byte loads per thread per group
// register stages of groups (kP1bRing - 1 in flight; 3, 4 or 6 stages made
// the 16K chunk's phase-1 backward 1-2.5 ms slower on an MI355X)
constexpr int kP1bRing = 2;

static __global__ __launch_bounds__(256) void k_pack_bwd_queries(int S, int d, const float* __restrict__ q,
                                                               u32x4_t* __restrict__ pk) {
  const int ks_n = (d + 31) >> 5;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= ks_n * 2 * 64) return;
  const int lane = idx & 63, m = (idx >> 6) & 1, ks = idx >> 7;
  const int j = m * 16 + (lane & 15);
  const int e0 = ks * 32 + (lane >> 4) * 8;
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (j < S && e0 + e < d) ? q[(int64_t)j * d + e0 + e] : 0.f;
  u32x4_t hi, lo;
  hi.x = pack_bf16x2(v[0], v[1]); hi.y = pack_bf16x2(v[2], v[3]);
  hi.z = pack_bf16x2(v[4], v[5]); hi.w = pack_bf16x2(v[6], v[7]);
  float h[8];
  unpack_bf16x8(make_uint4(hi.x, hi.y, hi.z, hi.w), h);
  lo.x = pack_bf16x2(v[0] - h[0], v[1] - h[1]); lo.y = pack_bf16x2(v[2] - h[2], v[3] - h[3]);
  lo.z = pack_bf16x2(v[4] - h[4], v[5] - h[5]); lo.w = pack_bf16x2(v[6] - h[6], v[7] - h[7]);
  pk[((ks * 2 + m) * 2 + 0) * 64 + lane] = hi;
  pk[((ks * 2 + m) * 2 + 1) * 64 + lane] = lo;
}

// Bytes of the packed queries for rows of d channels.
constexpr int64_t p1b_packed_bytes(int64_t d) { return ((d + 31) >> 5) * 2 * 2 * 64 * 16; }

// Sites per pass of part I: all QW of the wave's sites for up to 8 bf16
// sources; fewer for more sources or fp32 rows (registers).
template <typename Ut, int N, int QW>
struct P1bPass {
  static constexpr int kQB = N <= 8 ? (QW == 4 ? 2 : QW) : ((sizeof(Ut) == 4 || QW == 3) ? 1 : (QW < 2 ? QW : 2));
  static constexpr int kJ3 = N <= 8 ? 4 : 2;  // sites per step of part III
};

// Part I of one token on the matrix cores (see above): tD[j][i] = G_j.u_i,
// tZ[j][i] = q_j.u_i, tss[i] = |u_i|^2 for j < S, i < N.  `lds` holds two
// staging buffers of kP1bStage bf16 (reused for the wave partials at the
// end).  Every wave of the workgroup calls it; it ends with the tables
// written but not yet visible to other waves (the caller's barrier).
template <typename Ut, typename St, int N>
__device__ __forceinline__ void p1b_part1_mfma(int64_t tok, int64_t T, int d, const Ut* __restrict__ src,
                                               int64_t stride, int S, const St* __restrict__ gin, int64_t gstride,
                                               const u32x4_t* __restrict__ pk, int wv, int lane,
                                               float (*tD)[N], float (*tZ)[N], float* tss, bf16_t* lds) {
  static_assert(std::is_same<St, bf16_t>::value, "G rows in bf16");
  constexpr bool F32U = sizeof(Ut) == 4;
  constexpr int CPP = 16 / sizeof(Ut);          // channels per 16-byte piece of a source row
  constexpr int PPR = kP1bGE / CPP;             // pieces per source row and group
  constexpr int PU = N * PPR;
  const int PG = S * (kP1bGE / 8);
  const int P = PU + PG;
  const int ngr = (d + kP1bGE - 1) / kP1bGE;
  const int t = threadIdx.x;
  const int col = lane & 15, grp = lane >> 4;
  // the thread's pieces: p = t + kP1bThreads * k
  u32x4_t rs[kP1bRing][kP1bPieces];
  float ssa[kP1bPieces];
#pragma unroll
  for (int k = 0; k < kP1bPieces; ++k) ssa[k] = 0.f;
  auto piece = [&](int p, int g, int& row, int& ch, bool& is_u) {
    is_u = p < PU;
    const int q = is_u ? p : p - PU;
    const int ppr = is_u ? PPR : kP1bGE / 8;
    row = q / ppr;
    ch = g * kP1bGE + (q - row * ppr) * (is_u ? CPP : 8);
  };
  auto issue = [&](u32x4_t(&r)[kP1bPieces], int g) {
    g = g < ngr ? g : ngr - 1;
#pragma unroll
    for (int k = 0; k < kP1bPieces; ++k) {
      const int p0 = t + kP1bThreads * k;
      const int p = p0 < P ? p0 : P - 1;  // clamped: always a valid row
      int row, ch;
      bool is_u;
      piece(p, g, row, ch, is_u);
      const int c = ch < d ? ch : 0;
      r[k] = is_u ? ld16(src + row * stride + tok * d + c) : ld16(gin + row * gstride + tok * d + c);
    }
  };
  // raw pieces of group g -> LDS buffer g & 1 (zeros past d), sums of squares
  auto stage = [&](const u32x4_t(&r)[kP1bPieces], int g) {
    bf16_t* buf = lds + (g & 1) * kP1bStage;
#pragma unroll
    for (int k = 0; k < kP1bPieces; ++k) {
      const int p = t + kP1bThreads * k;
      if (p < P) {
        int row, ch;
        bool is_u;
        piece(p, g, row, ch, is_u);
        const bool ok = ch < d;
        const int o = ch - g * kP1bGE;
        if (!is_u) {
          st16(buf + row * kP1bRow + o, ok ? r[k] : u32x4_t{0u, 0u, 0u, 0u});
        } else if (F32U) {
          float v[4] = {__uint_as_float(r[k].x), __uint_as_float(r[k].y), __uint_as_float(r[k].z),
                        __uint_as_float(r[k].w)};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = ok ? v[e] : 0.f;
            ssa[k] = fmaf(v[e], v[e], ssa[k]);
          }
          const unsigned h01 = pack_bf16x2(v[0], v[1]), h23 = pack_bf16x2(v[2], v[3]);
          float h[8];
          unpack_bf16x8(make_uint4(h01, h23, 0u, 0u), h);
          st8(buf + (32 + row) * kP1bRow + o, u32x2_t{h01, h23});
          st8(buf + (48 + row) * kP1bRow + o,
              u32x2_t{pack_bf16x2(v[0] - h[0], v[1] - h[1]), pack_bf16x2(v[2] - h[2], v[3] - h[3])});
        } else {
          const u32x4_t u = ok ? r[k] : u32x4_t{0u, 0u, 0u, 0u};
          float v[8];
          unpack_bf16x8(make_uint4(u.x, u.y, u.z, u.w), v);
#pragma unroll
          for (int e = 0; e < 8; ++e) ssa[k] = fmaf(v[e], v[e], ssa[k]);
          st16(buf + (32 + row) * kP1bRow + o, u);
        }
      }
    }
  };
  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4_t Dm[2] = {zero4, zero4}, Zm[2] = {zero4, zero4};
  // the wave's k-step of group g: channels g * kP1bGE + wv * 32 + grp * 8 .. + 7
  auto mfma = [&](int g) {
    const bf16_t* buf = lds + (g & 1) * kP1bStage;
    const int o = wv * 32 + grp * 8;
    const int ks = g * (kP1bGE / 32) + wv;
    const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, ld16(buf + (32 + col) * kP1bRow + o));
    bf16x8_t bl = bh;
    if (F32U) bl = __builtin_bit_cast(bf16x8_t, ld16(buf + (48 + col) * kP1bRow + o));
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const bf16x8_t ag = __builtin_bit_cast(bf16x8_t, ld16(buf + (m * 16 + col) * kP1bRow + o));
      const bf16x8_t qh = __builtin_bit_cast(bf16x8_t, pk[((ks * 2 + m) * 2 + 0) * 64 + lane]);
      const bf16x8_t ql = __builtin_bit_cast(bf16x8_t, pk[((ks * 2 + m) * 2 + 1) * 64 + lane]);
      Dm[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ag, bh, Dm[m], 0, 0, 0);
      Zm[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, bh, Zm[m], 0, 0, 0);
      Zm[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ql, bh, Zm[m], 0, 0, 0);
      if (F32U) {
        Dm[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ag, bl, Dm[m], 0, 0, 0);
        Zm[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qh, bl, Zm[m], 0, 0, 0);
      }
    }
  };
  // a ring of kP1bRing register stages: kP1bRing - 1 groups in flight while
  // the oldest is staged and used
#pragma unroll
  for (int s = 0; s < kP1bRing - 1; ++s) issue(rs[s], s);
  for (int g0 = 0; g0 < ngr; g0 += kP1bRing) {
#pragma unroll
    for (int s = 0; s < kP1bRing; ++s) {
      const int g = g0 + s;
      issue(rs[(s + kP1bRing - 1) % kP1bRing], g + kP1bRing - 1);
      __builtin_amdgcn_sched_barrier(0);
      if (g < ngr) {  // uniform
        stage(rs[s], g);
        lds_barrier();
        mfma(g);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  lds_barrier();  // every wave is done with the staging buffers
  // wave partials [wave][lane][16], then the sums of squares per piece
  float* pr = reinterpret_cast<float*>(lds);
  float* ssl = pr + 8 * 64 * 16;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[(wv * 64 + lane) * 16 + m * 4 + r] = Dm[m][r];
      pr[(wv * 64 + lane) * 16 + 8 + m * 4 + r] = Zm[m][r];
    }
#pragma unroll
  for (int k = 0; k < kP1bPieces; ++k) {
    const int p = t + kP1bThreads * k;
    if (p < PU) ssl[p] = ssa[k];
  }
  lds_barrier();
  if (t < S * N) {
    const int j = t / N, i = t - (t / N) * N;
    const int src_lane = ((j & 15) >> 2) * 16 + i, idx = (j >> 4) * 4 + (j & 3);
    float dsum = 0.f, zsum = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      dsum += pr[(w * 64 + src_lane) * 16 + idx];
      zsum += pr[(w * 64 + src_lane) * 16 + 8 + idx];
    }
    tD[j][i] = dsum;
    tZ[j][i] = zsum;
  }
  if (t < N) {
    float sv = 0.f;
    for (int o = 0; o < PPR; ++o) sv += ssl[t * PPR + o];
    tss[t] = sv;
  }
}

template <typename Ut, typename St, int N, int QW, bool MF>
__global__ __launch_bounds__(kP1bThreads) void k_p1_bwd(int64_t T, int d, const Ut* __restrict__ src, int64_t stride,
                                                        int S, const float* __restrict__ q, float eps,
                                                        const St* __restrict__ gin, int64_t gstride,
                                                        const float* __restrict__ c_in,
                                                        const float* __restrict__ gp_in, float* __restrict__ dsrc,
                                                        int64_t dstride, int accumulate, float* __restrict__ coef,
                                                        const u32x4_t* __restrict__ pk) {
  constexpr int QB = P1bPass<Ut, N, QW>::kQB;
  constexpr int J3 = P1bPass<Ut, N, QW>::kJ3;
  const int SP = (S + 7) & ~7;  // sites of the coefficient table, padded
  __shared__ float tD[kP1bSites][N], tZ[kP1bSites][N], tss[N];
  extern __shared__ bf16_t p1b_lds[];  // part I on the matrix cores: two staging buffers
  __shared__ float ta[kP1bSites][N], tb[kP1bSites][N], tq[kP1bSites][N], te[N];
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x >> 6;
  const int C = d >> 3;
  const int ngroups = (C + 63) >> 6;
  const float inv_d = 1.0f / (float)d;
  for (int64_t tok = blockIdx.x; tok < T; tok += gridDim.x) {
    if constexpr (MF) {
      p1b_part1_mfma<Ut, St, N>(tok, T, d, src, stride, S, gin, gstride, pk, wv, lane, tD, tZ, tss, p1b_lds);
    } else {
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
      Chunk<Ut> ua[N], ub[N];
      Chunk<St> ga[QB], gb[QB];
      Chunk<float> qa[QB], qbf[QB];
      auto fetch = [&](Chunk<Ut>(&u)[N], Chunk<St>(&gq)[QB], Chunk<float>(&qq)[QB], int g) {
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
      auto consume = [&](const Chunk<Ut>(&u)[N], const Chunk<St>(&gq)[QB], const Chunk<float>(&qq)[QB], int g) {
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
    }  // part I
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
static __global__ __launch_bounds__(256) void k_p1_bwd_wgrad_reduce(int64_t ranges, int S, int d,
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

template <typename Ut, typename St, int N, int QW>
static hipError_t run_p1b_main(int64_t T, int d, const void* src, int64_t stride, int S, const float* q, float eps,
                               const void* gin, int64_t gstride, const float* c_in, const float* gp_in, float* dsrc,
                               int64_t dstride, int accumulate, float* coef, u32x4_t* pk, hipStream_t stream) {
  int64_t wgs = T;
  const int64_t cap = (int64_t)device_cu_count() * 2;
  if (wgs > cap) wgs = cap;
  // part I on the matrix cores when G is bf16 (fp32 G keeps the fp32 vector path)
  constexpr bool MF = std::is_same<St, bf16_t>::value;
  size_t lds = 0;
  if (MF) {
    const int ks_n = (d + 31) >> 5;
    hipLaunchKernelGGL(k_pack_bwd_queries, dim3((unsigned)((ks_n * 128 + 255) / 256)), dim3(256), 0, stream, S, d, q,
                       pk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    lds = sizeof(bf16_t) * 2 * kP1bStage;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_p1_bwd<Ut, St, N, QW, MF>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_p1_bwd<Ut, St, N, QW, MF>), dim3((unsigned)wgs), dim3(kP1bThreads), lds, stream, T, d,
                     static_cast<const Ut*>(src), stride, S, q, eps, static_cast<const St*>(gin), gstride, c_in,
                     gp_in, dsrc, dstride, accumulate, coef, pk);
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

template <typename Ut, typename St, int N>
static hipError_t run_p1b(int64_t T, int d, const void* src, int64_t stride, int S, const float* w, const float* kg,
                          float eps, const void* gin, int64_t gstride, const float* c_in, const float* gp_in,
                          float* dsrc, int64_t dstride, int accumulate, float* dw, float* dkg, float* ws,
                          hipStream_t stream) {
  // workspace: coefficients [T][S][N], folded queries [S][d], range sums,
  // packed queries
  float* coef = ws;
  float* q = coef + T * (int64_t)((S + 7) & ~7) * N;
  float* part = q + (int64_t)S * d;
  u32x4_t* pk = reinterpret_cast<u32x4_t*>(part + p1_backward_ranges(d) * S * (int64_t)d);
  const int64_t nq = (int64_t)S * d;
  hipLaunchKernelGGL(k_fold_queries, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0, stream, nq, w, kg, q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (S <= 8) {
    e = run_p1b_main<Ut, St, N, 1>(T, d, src, stride, S, q, eps, gin, gstride, c_in, gp_in, dsrc, dstride, accumulate,
                               coef, pk, stream);
  } else if (S <= 16) {
    e = run_p1b_main<Ut, St, N, 2>(T, d, src, stride, S, q, eps, gin, gstride, c_in, gp_in, dsrc, dstride, accumulate,
                               coef, pk, stream);
  } else if (S <= 24) {
    e = run_p1b_main<Ut, St, N, 3>(T, d, src, stride, S, q, eps, gin, gstride, c_in, gp_in, dsrc, dstride, accumulate,
                               coef, pk, stream);
  } else {
    e = run_p1b_main<Ut, St, N, 4>(T, d, src, stride, S, q, eps, gin, gstride, c_in, gp_in, dsrc, dstride, accumulate,
                               coef, pk, stream);
  }
  if (e != hipSuccess) return e;
  // (the coefficient table has (S rounded up to 8) sites per token)
  if (S <= 8) {
    e = run_p1b_wgrad<Ut, N, 8>(T, d, src, stride, S, coef, part, stream);
  } else if (S <= 16) {
    e = run_p1b_wgrad<Ut, N, 16>(T, d, src, stride, S, coef, part, stream);
  } else if (S <= 24) {
    e = run_p1b_wgrad<Ut, N, 24>(T, d, src, stride, S, coef, part, stream);
  } else {
    e = run_p1b_wgrad<Ut, N, 32>(T, d, src, stride, S, coef, part, stream);
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_p1_bwd_wgrad_reduce, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0, stream,
                     p1_backward_ranges(d), S, d, part, w, kg, dw, dkg);
  return hipGetLastError();
}

template <typename Ut, typename St>
static hipError_t pick_p1b(int n, int64_t T, int d, const void* src, int64_t stride, int S, const float* w,
                           const float* kg, float eps, const void* gin, int64_t gstride, const float* c_in,
                           const float* gp_in, float* dsrc, int64_t dstride, int accumulate, float* dw, float* dkg,
                           float* ws, hipStream_t stream) {
  switch (n) {
#define ATTNRES_CASE(N_)                                                                                           \
  case N_:                                                                                                         \
    return run_p1b<Ut, St, N_>(T, d, src, stride, S, w, kg, eps, gin, gstride, c_in, gp_in, dsrc, dstride, accumulate, \
                           dw, dkg, ws, stream);
    ATTNRES_CASE(1) ATTNRES_CASE(2) ATTNRES_CASE(3) ATTNRES_CASE(4) ATTNRES_CASE(5) ATTNRES_CASE(6)
    ATTNRES_CASE(7) ATTNRES_CASE(8) ATTNRES_CASE(9) ATTNRES_CASE(10) ATTNRES_CASE(11) ATTNRES_CASE(12)
    ATTNRES_CASE(13) ATTNRES_CASE(14) ATTNRES_CASE(15) ATTNRES_CASE(16)
#undef ATTNRES_CASE
  }
  return hipErrorInvalidValue;
}

}  // namespace attnres
