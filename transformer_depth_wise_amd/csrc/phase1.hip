// Phase 1 of Block AttnRes on gfx950: one batched pass per block that scores
// every completed-block source against all S pseudo-queries of the block and
// returns normalised partial outputs with their softmax statistics
// ("Attention Residuals" notes, section 10, first phase; the reading notes'
// section on static queries: stacking the S queries turns S matrix-vector
// products into one Q K^T product, and each source row is read once per
// block instead of once per sublayer).
//
// Work decomposition.  S >= 2 uses two kernels; S == 1 (Full AttnRes sites and
// the final aggregation) uses one kernel that does both parts per tile.
//  part A  scores (one workgroup = 4 waves = a tile of 16 tokens).  Z[q][t][i] = sum_k (w_q g_q)[k] * u_i[t][k] is a dense
//          contraction over d, computed on the matrix cores with
//          v_mfma_f32_16x16x32_bf16 (bf16 rows; the fp32 query is split into
//          bf16 hi + lo parts, so the product keeps ~16 mantissa bits of the
//          query and accumulates in fp32) or v_mfma_f32_16x16x4_f32 (fp32
//          rows).  A lane supplies query (lane&15) of the A operand and token
//          (lane&15) of the B operand; the 4 lane groups and the 4 waves split
//          the channels.  Sum of squares of every source row (for its RMS) is
//          accumulated on the vector ALUs from the same registers.  The four
//          waves' partial sums are added in a fixed order through LDS, then
//          z = Z / r(u) and the softmax over sources is taken in LDS.
//          For S >= 2 the softmax weights go to a caller-provided workspace.
//  part B  outputs.  out[s][t] = sum_i alpha[t][s][i] u_i[t]: the source rows
//          are streamed again (16-byte loads, a wave reads 1 KiB of one row)
//          and each row chunk serves all S queries.
#include "attnres_device.h"
#include "attnres_launch.h"

namespace attnres {

template <typename St>
struct Mfma;

template <>
struct Mfma<bf16_t> {
  struct A {
    bf16x8_t hi, lo;
  };
  typedef bf16x8_t B;

  static __device__ __forceinline__ A make_a(const float (&q)[8]) {
    uint4 h;
    h.x = pack_bf16x2(q[0], q[1]);
    h.y = pack_bf16x2(q[2], q[3]);
    h.z = pack_bf16x2(q[4], q[5]);
    h.w = pack_bf16x2(q[6], q[7]);
    float hf[8];
    unpack_bf16x8(h, hf);
    uint4 l;
    l.x = pack_bf16x2(q[0] - hf[0], q[1] - hf[1]);
    l.y = pack_bf16x2(q[2] - hf[2], q[3] - hf[3]);
    l.z = pack_bf16x2(q[4] - hf[4], q[5] - hf[5]);
    l.w = pack_bf16x2(q[6] - hf[6], q[7] - hf[7]);
    A a;
    a.hi = __builtin_bit_cast(bf16x8_t, h);
    a.lo = __builtin_bit_cast(bf16x8_t, l);
    return a;
  }

  static __device__ __forceinline__ B load_b(const bf16_t* p, bool ok, float& ss) {
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (ok) u = *reinterpret_cast<const uint4*>(p);
    float f[8];
    unpack_bf16x8(u, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
    return __builtin_bit_cast(bf16x8_t, u);
  }

  static __device__ __forceinline__ void mma(f32x4_t& acc, const A& a, const B& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hi, b, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.lo, b, acc, 0, 0, 0);
  }
};

template <>
struct Mfma<float> {
  struct A {
    float v[8];
  };
  struct B {
    float v[8];
  };

  static __device__ __forceinline__ A make_a(const float (&q)[8]) {
    A a;
#pragma unroll
    for (int e = 0; e < 8; ++e) a.v[e] = q[e];
    return a;
  }

  static __device__ __forceinline__ B load_b(const float* p, bool ok, float& ss) {
    B b;
    if (ok) {
      load8(p, b.v);
    } else {
      zero8(b.v);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(b.v[e], b.v[e], ss);
    return b;
  }

  // One channel per lane group per instruction: channel e of the lane's chunk.
  static __device__ __forceinline__ void mma(f32x4_t& acc, const A& a, const B& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
  }
};

// Per-wave partial scores of the 16-token tile starting at tok0 against
// queries [0, 16*MT) for sources [g0, g0+G).  Channel chunks (8 channels)
// are visited in K-blocks of 16 chunks; wave w takes K-blocks w, w+4, ...;
// within a K-block, step s4 reads chunk 4*s4 + grp, so the 4 lane groups read
// 64 contiguous bytes of each token row per instruction.
template <typename St, int MT, int G>
__device__ __forceinline__ void score_pass(const St* __restrict__ src, int n, int64_t stride,
                                           int64_t T, int d, const float* __restrict__ w,
                                           const float* __restrict__ kg, int S, int64_t tok0,
                                           int g0, f32x4_t (&acc)[MT][G], float (&ss)[G]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int64_t tok = tok0 + col;
  const bool tok_ok = tok < T;
  const int C = d >> 3;
  const int nkb = (C + 15) >> 4;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < G; ++i) acc[m][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < G; ++i) ss[i] = 0.f;

  for (int kb = wave; kb < nkb; kb += 4) {
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int c = kb * 16 + s4 * 4 + grp;
      const bool cok = c < C;
      typename Mfma<St>::A a[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int q = m * 16 + col;
        float qv[8];
        if (cok && q < S) {
          load8(w + (int64_t)q * d + c * 8, qv);
          if (kg) {
            float gv[8];
            load8(kg + (int64_t)q * d + c * 8, gv);
#pragma unroll
            for (int e = 0; e < 8; ++e) qv[e] *= gv[e];
          }
        } else {
          zero8(qv);
        }
        a[m] = Mfma<St>::make_a(qv);
      }
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const int si = g0 + i;
        const bool ok = cok && tok_ok && si < n;
        const St* p = src + (int64_t)si * stride + tok * d + c * 8;
        typename Mfma<St>::B b = Mfma<St>::load_b(p, ok, ss[i]);
#pragma unroll
        for (int m = 0; m < MT; ++m) Mfma<St>::mma(acc[m][i], a[m], b);
      }
    }
  }
  // every lane group saw different channels of the same (token, source)
#pragma unroll
  for (int i = 0; i < G; ++i) {
    ss[i] += __shfl_xor(ss[i], 16, 64);
    ss[i] += __shfl_xor(ss[i], 32, 64);
  }
}

template <int MT, int G>
struct Red {
  static constexpr int kSlot = MT * G * 4 * 64 + G * 64;  // floats per slot

  static __device__ __forceinline__ void put(float* slot, const f32x4_t (&acc)[MT][G],
                                             const float (&ss)[G], int lane) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < G; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) slot[((m * G + i) * 4 + r) * 64 + lane] = acc[m][i][r];
#pragma unroll
    for (int i = 0; i < G; ++i) slot[MT * G * 256 + i * 64 + lane] = ss[i];
  }

  static __device__ __forceinline__ void add(const float* slot, f32x4_t (&acc)[MT][G],
                                             float (&ss)[G], int lane) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < G; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[m][i][r] += slot[((m * G + i) * 4 + r) * 64 + lane];
#pragma unroll
    for (int i = 0; i < G; ++i) ss[i] += slot[MT * G * 256 + i * 64 + lane];
  }

  // Sum the four waves' partials into wave 0 in the fixed order
  // (w0 + w2) + (w1 + w3).  `red` holds two slots.
  static __device__ __forceinline__ void reduce(float* red, f32x4_t (&acc)[MT][G], float (&ss)[G]) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    __syncthreads();  // previous readers of the slots are done
    if (wave >= 2) put(red + (wave - 2) * kSlot, acc, ss, lane);
    __syncthreads();
    if (wave < 2) add(red + wave * kSlot, acc, ss, lane);
    __syncthreads();
    if (wave == 1) put(red, acc, ss, lane);
    __syncthreads();
    if (wave == 0) add(red, acc, ss, lane);
  }
};

// ---------------------------------------------------------------------------
// S >= 2, first kernel: scores and softmax weights of a 16-token tile for up
// to 32 queries.  The weights go to the workspace as alpha[t][q][i]
// (i fastest), the statistics to m_out / lse_out.
template <typename St, int MT, int NB>
__global__ __launch_bounds__(256) void k_p1_scores(const St* __restrict__ src, int n, int64_t stride,
                                                   int64_t T, int d, const float* __restrict__ w,
                                                   const float* __restrict__ kg, int S, float eps,
                                                   float* __restrict__ alpha, float* __restrict__ m_out,
                                                   float* __restrict__ lse_out) {
  constexpr int G = NB < 8 ? NB : 8;
  constexpr int QP = 16 * MT;
  constexpr int NP = NB < 4 ? 4 : NB;
  typedef Red<MT, G> R;
  extern __shared__ float lds[];
  float* red = lds;
  float* zb = lds + 2 * R::kSlot;  // [16 tokens][QP queries][NP sources]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int64_t tok0 = (int64_t)blockIdx.x * 16;

  for (int g0 = 0; g0 < n; g0 += G) {
    f32x4_t acc[MT][G];
    float ss[G];
    score_pass<St, MT, G>(src, n, stride, T, d, w, kg, S, tok0, g0, acc, ss);
    R::reduce(red, acc, ss);
    if (wave == 0) {
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const int si = g0 + i;
        if (si < n) {
          const float r = sqrtf(ss[i] / (float)d + eps);
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              const int q = m * 16 + grp * 4 + rr;
              zb[(col * QP + q) * NP + si] = acc[m][i][rr] / r;
            }
        }
      }
    }
  }
  __syncthreads();

  // softmax over the n sources of every (token, query) pair
  for (int pidx = threadIdx.x; pidx < 16 * QP; pidx += 256) {
    const int t = pidx / QP, q = pidx - t * QP;
    const int64_t tok = tok0 + t;
    if (q >= S || tok >= T) continue;
    const float* row = zb + pidx * NP;
    float mx = row[0];
    for (int i = 1; i < n; ++i) mx = fmaxf(mx, row[i]);
    float l = 0.f;
    for (int i = 0; i < n; ++i) l += expf(row[i] - mx);
    float* a = alpha + (tok * S + q) * n;
    for (int i = 0; i < n; ++i) a[i] = expf(row[i] - mx) / l;
    if (m_out) m_out[(int64_t)q * T + tok] = mx;
    lse_out[(int64_t)q * T + tok] = mx + logf(l);
  }
}

// S >= 2, second kernel: out[q][t] = sum_i alpha[t][q][i] u_i[t].  A wave owns
// one (token, group of 64 chunks) item at a time, so the weights are
// wave-uniform and come in through scalar loads; every source chunk is used
// by all S queries; the next item's source chunks are loaded before the
// current item is computed.
template <typename St, int NB>
__device__ __forceinline__ void p1_issue(Chunk<St> (&s)[NB], int64_t item, int64_t items, int ngroups,
                                         const St* __restrict__ src, int n, int64_t stride, int d, int C,
                                         int lane) {
  const int64_t t = item / ngroups;
  const int c = (int)(item - t * ngroups) * 64 + lane;
  const bool ok = item < items && c < C;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    if (ok && i < n) {
      s[i].load(src + (int64_t)i * stride + t * d + c * 8);
    } else {
      s[i].zero();
    }
  }
}

template <typename St, int NB>
__device__ __forceinline__ void p1_emit(const Chunk<St> (&s)[NB], int64_t item, int ngroups, int n, int64_t T,
                                        int d, int C, int lane, const float* __restrict__ alpha, int S,
                                        St* __restrict__ out) {
  const int64_t t = item / ngroups;
  const int c = (int)(item - t * ngroups) * 64 + lane;
  float b[NB][8];
#pragma unroll
  for (int i = 0; i < NB; ++i) s[i].unpack(b[i]);
  const float* al = alpha + t * S * n;
  for (int q = 0; q < S; ++q) {
    float o[8];
    zero8(o);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (i < n) {
        const float a = al[q * n + i];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(a, b[i][e], o[e]);
      }
    }
    if (c < C) out8(out + ((int64_t)q * T + t) * d + c * 8, o);
  }
}

template <typename St, int NB>
__global__ __launch_bounds__(256) void k_p1_out(const St* __restrict__ src, int n, int64_t stride, int64_t T,
                                                int d, const float* __restrict__ alpha, int S,
                                                St* __restrict__ out) {
  const int C = d >> 3;
  const int ngroups = (C + 63) >> 6;
  const int64_t items = T * ngroups;
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  int64_t item = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Chunk<St> A[NB], B[NB];
  p1_issue<St, NB>(A, item, items, ngroups, src, n, stride, d, C, lane);
  while (item < items) {
    p1_issue<St, NB>(B, item + nw, items, ngroups, src, n, stride, d, C, lane);
    p1_emit<St, NB>(A, item, ngroups, n, T, d, C, lane, alpha, S, out);
    item += nw;
    if (item >= items) break;
    p1_issue<St, NB>(A, item + nw, items, ngroups, src, n, stride, d, C, lane);
    p1_emit<St, NB>(B, item, ngroups, n, T, d, C, lane, alpha, S, out);
    item += nw;
  }
}

// ---------------------------------------------------------------------------
// S == 1: one query, up to 32 sources in groups of G, optional PreNorm of
// the output (Full AttnRes sites and the final aggregation).
constexpr int kSingleNP = 32;

template <typename St, int G>
__global__ __launch_bounds__(256) void k_phase1_single(const St* __restrict__ src, int n, int64_t stride,
                                                       int64_t T, int d, const float* __restrict__ w,
                                                       const float* __restrict__ kg,
                                                       const float* __restrict__ gamma, float eps,
                                                       St* __restrict__ h_out, St* __restrict__ x_out,
                                                       float* __restrict__ m_out,
                                                       float* __restrict__ lse_out) {
  typedef Red<1, G> R;
  extern __shared__ float lds[];
  float* red = lds;
  float* zb = lds + 2 * R::kSlot;         // [16 tokens][kSingleNP sources]
  float* red2 = zb + 16 * kSingleNP;      // 2 x 8 floats for the PreNorm reduction

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int64_t tok0 = (int64_t)blockIdx.x * 16;

  for (int g0 = 0; g0 < n; g0 += G) {
    f32x4_t acc[1][G];
    float ss[G];
    score_pass<St, 1, G>(src, n, stride, T, d, w, kg, 1, tok0, g0, acc, ss);
    R::reduce(red, acc, ss);
    if (wave == 0 && grp == 0) {  // row 0 of the MFMA output = query 0
#pragma unroll
      for (int i = 0; i < G; ++i) {
        const int si = g0 + i;
        if (si < n) zb[col * kSingleNP + si] = acc[0][i][0] / sqrtf(ss[i] / (float)d + eps);
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    float* row = zb + threadIdx.x * kSingleNP;
    float mx = row[0];
    for (int i = 1; i < n; ++i) mx = fmaxf(mx, row[i]);
    float l = 0.f;
    for (int i = 0; i < n; ++i) {
      const float e = expf(row[i] - mx);
      row[i] = e;
      l += e;
    }
    for (int i = 0; i < n; ++i) row[i] = row[i] / l;
    const int64_t tok = tok0 + threadIdx.x;
    if (tok < T) {
      if (m_out) m_out[tok] = mx;
      if (lse_out) lse_out[tok] = mx + logf(l);
    }
  }
  __syncthreads();

  const int C = d >> 3;
  const int ntile = (int)((T - tok0) < 16 ? (T - tok0) : 16);
  int parity = 0;
  for (int t = 0; t < ntile; ++t) {
    const int64_t tok = tok0 + t;
    const float* al = zb + t * kSingleNP;
    float h[8][8];
    float ssq = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int c = threadIdx.x + 256 * k;
      zero8(h[k]);
      if (c < C) {
        const St* base = src + tok * d + c * 8;
        int i = 0;
        for (; i + 4 <= n; i += 4) {
          float u0[8], u1[8], u2[8], u3[8];
          load8(base + (int64_t)(i + 0) * stride, u0);
          load8(base + (int64_t)(i + 1) * stride, u1);
          load8(base + (int64_t)(i + 2) * stride, u2);
          load8(base + (int64_t)(i + 3) * stride, u3);
          const float a0 = al[i], a1 = al[i + 1], a2 = al[i + 2], a3 = al[i + 3];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            h[k][e] = fmaf(a0, u0[e], h[k][e]);
            h[k][e] = fmaf(a1, u1[e], h[k][e]);
            h[k][e] = fmaf(a2, u2[e], h[k][e]);
            h[k][e] = fmaf(a3, u3[e], h[k][e]);
          }
        }
        for (; i < n; ++i) {
          float u[8];
          load8(base + (int64_t)i * stride, u);
          const float a = al[i];
#pragma unroll
          for (int e = 0; e < 8; ++e) h[k][e] = fmaf(a, u[e], h[k][e]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) ssq = fmaf(h[k][e], h[k][e], ssq);
        if (h_out) store8(h_out + tok * d + c * 8, h[k]);
      }
    }
    if (x_out) {
      const float2 tot = block_sum2_256(ssq, 0.f, red2 + 8 * parity);
      parity ^= 1;
      const float rinv = 1.0f / sqrtf(tot.x / (float)d + eps);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int c = threadIdx.x + 256 * k;
        if (c < C) {
          float gm[8];
          if (gamma) {
            load8(gamma + c * 8, gm);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) gm[e] = 1.f;
          }
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = gm[e] * (h[k][e] * rinv);
          store8(x_out + tok * d + c * 8, x);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// launchers

template <typename Kern>
static hipError_t set_lds(Kern k, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

template <typename St, int MT, int NB>
static hipError_t run_multi(const void* src, int n, int64_t stride, int64_t T, int d, const float* w,
                            const float* kg, int S, float eps, void* out, float* m_out, float* lse_out,
                            float* alpha, hipStream_t stream) {
  constexpr int G = NB < 8 ? NB : 8;
  constexpr int NP = NB < 4 ? 4 : NB;
  const size_t lds = sizeof(float) * (2 * Red<MT, G>::kSlot + 16 * 16 * MT * NP);
  auto ks = k_p1_scores<St, MT, NB>;
  hipError_t e = set_lds(ks, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ks, dim3((unsigned)((T + 15) / 16)), dim3(256), lds, stream, static_cast<const St*>(src),
                     n, stride, T, d, w, kg, S, eps, alpha, m_out, lse_out);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t items = T * (int64_t)(((d >> 3) + 63) >> 6);
  const int64_t wgs = (items + 3) / 4;
  const int64_t cap = (int64_t)device_cu_count() * 4;
  hipLaunchKernelGGL((k_p1_out<St, NB>), dim3((unsigned)(wgs < cap ? wgs : cap)), dim3(256), 0, stream,
                     static_cast<const St*>(src), n, stride, T, d, alpha, S, static_cast<St*>(out));
  return hipGetLastError();
}

template <typename St, int MT>
static hipError_t pick_nb(const void* src, int n, int64_t stride, int64_t T, int d, const float* w,
                          const float* kg, int S, float eps, void* out, float* m_out, float* lse_out,
                          float* alpha, hipStream_t stream) {
  if (n <= 1) return run_multi<St, MT, 1>(src, n, stride, T, d, w, kg, S, eps, out, m_out, lse_out, alpha, stream);
  if (n <= 2) return run_multi<St, MT, 2>(src, n, stride, T, d, w, kg, S, eps, out, m_out, lse_out, alpha, stream);
  if (n <= 4) return run_multi<St, MT, 4>(src, n, stride, T, d, w, kg, S, eps, out, m_out, lse_out, alpha, stream);
  if (n <= 8) return run_multi<St, MT, 8>(src, n, stride, T, d, w, kg, S, eps, out, m_out, lse_out, alpha, stream);
  return run_multi<St, MT, 16>(src, n, stride, T, d, w, kg, S, eps, out, m_out, lse_out, alpha, stream);
}

hipError_t launch_phase1_multi(Dtype dt, const void* src, int n, int64_t stride, int64_t T, int d,
                               const float* w, const float* kg, int S, float eps, void* out,
                               float* m_out, float* lse_out, float* alpha, hipStream_t stream) {
  if (dt == kBF16) {
    if (S <= 16)
      return pick_nb<bf16_t, 1>(src, n, stride, T, d, w, kg, S, eps, out, m_out, lse_out, alpha, stream);
    return pick_nb<bf16_t, 2>(src, n, stride, T, d, w, kg, S, eps, out, m_out, lse_out, alpha, stream);
  }
  if (S <= 16) return pick_nb<float, 1>(src, n, stride, T, d, w, kg, S, eps, out, m_out, lse_out, alpha, stream);
  return pick_nb<float, 2>(src, n, stride, T, d, w, kg, S, eps, out, m_out, lse_out, alpha, stream);
}

template <typename St, int G>
static hipError_t run_single(const void* src, int n, int64_t stride, int64_t T, int d, const float* w,
                             const float* kg, const float* gamma, float eps, void* h_out, void* x_out,
                             float* m_out, float* lse_out, hipStream_t stream) {
  const size_t lds = sizeof(float) * (2 * Red<1, G>::kSlot + 16 * kSingleNP + 16);
  auto kern = k_phase1_single<St, G>;
  hipError_t e = set_lds(kern, lds);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((T + 15) / 16));
  hipLaunchKernelGGL(kern, grid, dim3(256), lds, stream, static_cast<const St*>(src), n, stride, T, d, w,
                     kg, gamma, eps, static_cast<St*>(h_out), static_cast<St*>(x_out), m_out, lse_out);
  return hipGetLastError();
}

template <typename St>
static hipError_t pick_g(const void* src, int n, int64_t stride, int64_t T, int d, const float* w,
                         const float* kg, const float* gamma, float eps, void* h_out, void* x_out,
                         float* m_out, float* lse_out, hipStream_t stream) {
  if (n <= 1) return run_single<St, 1>(src, n, stride, T, d, w, kg, gamma, eps, h_out, x_out, m_out, lse_out, stream);
  if (n <= 2) return run_single<St, 2>(src, n, stride, T, d, w, kg, gamma, eps, h_out, x_out, m_out, lse_out, stream);
  if (n <= 4) return run_single<St, 4>(src, n, stride, T, d, w, kg, gamma, eps, h_out, x_out, m_out, lse_out, stream);
  return run_single<St, 8>(src, n, stride, T, d, w, kg, gamma, eps, h_out, x_out, m_out, lse_out, stream);
}

hipError_t launch_phase1_single(Dtype dt, const void* src, int n, int64_t stride, int64_t T, int d,
                                const float* w, const float* kg, const float* gamma, float eps,
                                void* h_out, void* x_out, float* m_out, float* lse_out,
                                hipStream_t stream) {
  if (dt == kBF16)
    return pick_g<bf16_t>(src, n, stride, T, d, w, kg, gamma, eps, h_out, x_out, m_out, lse_out, stream);
  return pick_g<float>(src, n, stride, T, d, w, kg, gamma, eps, h_out, x_out, m_out, lse_out, stream);
}

}  // namespace attnres
