// Phase 1 of Block AttnRes on gfx950: one batched pass per block that scores
// every completed-block source against all S pseudo-queries of the block and
// returns normalised partial outputs with their softmax statistics
// ("Attention Residuals" notes, section 10, first phase; the reading notes'
// section on static queries: stacking the S queries turns S matrix-vector
// products into one Q K^T product, and each source row is read once per
// block instead of once per sublayer).
//
// Work decomposition.  For S >= 2 phase 1 is a streaming pair: pack the
// queries, score, then stream the outputs (the softmax over the sources in
// the scoring kernel for long token ranges, in its own launch or inside the
// output kernel for short ones).  S == 1 (Full AttnRes one-shot sites, the
// final aggregation) is one pass per token with an online softmax
// (k_site_online, k_site_team).
//  part A  scores.  Z[q][t][i] = sum_k (w_q g_q)[k] * u_i[t][k] is a dense
//          contraction over d, computed on the matrix cores with
//          v_mfma_f32_16x16x32_bf16 (bf16 rows; the fp32 query is split into
//          bf16 hi + lo parts, so the product keeps ~16 mantissa bits of the
//          query and accumulates in fp32) or v_mfma_f32_16x16x4_f32 (fp32
//          rows).  A lane supplies query (lane&15) of the A operand and token
//          (lane&15) of the B operand; the 4 lane groups split each K-block's
//          channels.  The sum of squares of every source row (for its RMS) is
//          accumulated on the vector ALUs from the same registers.  Two
//          kernels with the same summation order (bitwise equal results):
//          k_p1_scores gives each (16-token tile, source group, query tile)
//          a workgroup whose 4 waves take contiguous quarters of d (short
//          token ranges);
//          k_p1_scores_wide gives each 16-token tile over all of d one wave
//          (fp32 rows) or two that share its sources (bf16 rows) and shares
//          the queries of a workgroup's 4 tiles through LDS (long token
//          ranges).  The
//          queries are packed once per call into MFMA operand blocks; scores,
//          then softmax weights, go to the caller's workspace.
//  part B  outputs.  out[s][t] = sum_i alpha[t][s][i] u_i[t]: the source rows
//          are streamed again (16-byte loads, a wave reads 1 KiB of one row)
//          and each row chunk serves all S queries; with the first
//          sublayer's PreNorm, x_0 replaces out[0] (k_p1_out_tokens for long
//          ranges, k_p1_out_wg for short ones with rows over 256 chunks).
//
// Every global load is unconditional: an out-of-range token or chunk loads a
// clamped, valid address and the value is replaced by zero afterwards.  This
// keeps loads free of exec-mask branches, so the compiler issues a whole
// K-block (or the next item) of loads before the first wait.
#include <type_traits>

#include "attnres_device.h"
#include "attnres_launch.h"

namespace attnres {

__device__ __forceinline__ u32x4_t sel16(bool ok, u32x4_t v) {
  const u32x4_t z = {0u, 0u, 0u, 0u};
  return ok ? v : z;
}

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

  // Packed query chunk: 8 bf16 hi parts in the first half, the 8 lo parts
  // in the second.
  static __device__ __forceinline__ A from_halves(u32x4_t h, u32x4_t l) {
    A a;
    a.hi = __builtin_bit_cast(bf16x8_t, h);
    a.lo = __builtin_bit_cast(bf16x8_t, l);
    return a;
  }

  static __device__ __forceinline__ void pack(const float (&q)[8], u32x4_t* h, u32x4_t* l) {
    const A a = make_a(q);
    st16(h, __builtin_bit_cast(u32x4_t, a.hi));
    st16(l, __builtin_bit_cast(u32x4_t, a.lo));
  }

  static __device__ __forceinline__ B load_b(const bf16_t* p, bool ok) {
    return __builtin_bit_cast(bf16x8_t, sel16(ok, ld16(p)));
  }

  static __device__ __forceinline__ B zero_b() { return __builtin_bit_cast(bf16x8_t, u32x4_t{0u, 0u, 0u, 0u}); }

  static __device__ __forceinline__ void sumsq(const B& b, float& ss) {
    const u32x4_t u = __builtin_bit_cast(u32x4_t, b);
    float f[8];
    unpack_bf16x8(make_uint4(u.x, u.y, u.z, u.w), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
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

  // Packed query chunk: the 8 folded fp32 values, 4 in each half.
  static __device__ __forceinline__ A from_halves(u32x4_t x, u32x4_t y) {
    A a;
    a.v[0] = __uint_as_float(x.x); a.v[1] = __uint_as_float(x.y); a.v[2] = __uint_as_float(x.z);
    a.v[3] = __uint_as_float(x.w); a.v[4] = __uint_as_float(y.x); a.v[5] = __uint_as_float(y.y);
    a.v[6] = __uint_as_float(y.z); a.v[7] = __uint_as_float(y.w);
    return a;
  }

  static __device__ __forceinline__ void pack(const float (&q)[8], u32x4_t* h, u32x4_t* l) {
    st16(h, u32x4_t{__float_as_uint(q[0]), __float_as_uint(q[1]), __float_as_uint(q[2]), __float_as_uint(q[3])});
    st16(l, u32x4_t{__float_as_uint(q[4]), __float_as_uint(q[5]), __float_as_uint(q[6]), __float_as_uint(q[7])});
  }

  static __device__ __forceinline__ B load_b(const float* p, bool ok) {
    const u32x4_t x = sel16(ok, ld16(p)), y = sel16(ok, ld16(p + 4));
    B b;
    b.v[0] = __uint_as_float(x.x); b.v[1] = __uint_as_float(x.y); b.v[2] = __uint_as_float(x.z);
    b.v[3] = __uint_as_float(x.w); b.v[4] = __uint_as_float(y.x); b.v[5] = __uint_as_float(y.y);
    b.v[6] = __uint_as_float(y.z); b.v[7] = __uint_as_float(y.w);
    return b;
  }

  static __device__ __forceinline__ B zero_b() {
    B b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b.v[e] = 0.f;
    return b;
  }

  static __device__ __forceinline__ void sumsq(const B& b, float& ss) {
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(b.v[e], b.v[e], ss);
  }

  // One channel per lane group per instruction: channel e of the lane's chunk.
  static __device__ __forceinline__ void mma(f32x4_t& acc, const A& a, const B& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
  }
};

// The newest source of a phase-1 call formed from the pieces of the previous
// block's sum ("Attention Residuals" notes, section 8: b_n is the sum of the
// block's outputs): u = (partial + (v2 or 0)) + v in fp32, in that order,
// rounded to the sources' type exactly as the block-sum kernel stores it.
// `round_store` rounds 8 such values, stores them (when `st`) and returns the
// matrix-core operand of the rounded chunk.
template <typename St>
struct RoundB;
template <>
struct RoundB<bf16_t> {
  static __device__ __forceinline__ Mfma<bf16_t>::B round_store(const float (&x)[8], bf16_t* p, bool st) {
    const u32x4_t u{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                    pack_bf16x2(x[6], x[7])};
    if (st) st16(p, u);
    return __builtin_bit_cast(bf16x8_t, u);
  }
};
template <>
struct RoundB<float> {
  static __device__ __forceinline__ Mfma<float>::B round_store(const float (&x)[8], float* p, bool st) {
    if (st) {
      st16(p, u32x4_t{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])});
      st16(p + 4, u32x4_t{__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]), __float_as_uint(x[7])});
    }
    Mfma<float>::B b;
#pragma unroll
    for (int e = 0; e < 8; ++e) b.v[e] = x[e];
    return b;
  }
};

// One K-block of the newest source's pieces for one lane (4 chunks).
template <typename Vt, typename Pt>
struct PieceStage {
  Chunk<Pt> p[4];
  Chunk<Vt> a[4], b[4];
};

// Packed query operands.  Channels are grouped into K-blocks of 128 (16
// chunks of 8); K-block kb of a tile of 16*MT queries is a contiguous run of
// MT*4*2*64 16-byte words ordered [m][step][half][lane], where lane
// (grp*16 + col) holds query m*16+col, chunk kb*16 + step*4 + grp, half 0 =
// bf16 hi parts (fp32: values 0..3), half 1 = lo parts (values 4..7).  Rows
// >= S and chunks past the end of d are zero, so no load needs a guard and
// one wave reads 1 KiB of consecutive bytes per instruction.
constexpr int kKBlock = 16;          // chunks per K-block
constexpr int kPackedKBlockWords = 2 * 512;  // 16-byte words per K-block, room for 32 queries
template <int MT>
__device__ __forceinline__ int64_t packed_index(int kb, int m, int s4, int lane) {
  return (int64_t)kb * (MT * 512) + ((m * 4 + s4) * 2) * 64 + lane;
}

// Per-wave partial scores of the 16-token tile starting at tok0 against
// queries [0, 16*MT) for sources [g0, g0+G) (all valid).  Channel chunks (8
// channels) are visited in K-blocks of 16 chunks; wave w takes the w-th
// contiguous quarter [w*nkb/4, (w+1)*nkb/4) of the K-blocks, in order, so each
// wave streams through its part of every row; within a K-block, step s4 reads
// chunk 4*s4 + grp, so the 4 lane groups read 64 contiguous bytes of each
// token row per instruction.
// The queries come from `pk` (packed layout above, for MP tiles of 16, of
// which this pass takes tiles [m0, m0 + MT)) written by k_pack_queries.
template <typename St, int MT, int G, int KB, int MP>
__device__ __forceinline__ void score_pass(const St* __restrict__ src, int64_t stride, int64_t T, int d,
                                           const u32x4_t* __restrict__ pk, int64_t tok0, int g0,
                                           f32x4_t (&acc)[MT][G], float (&ss)[G], int m0) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const bool tok_ok = tok0 + col < T;
  const int64_t tok = tok_ok ? tok0 + col : T - 1;  // clamped: always a valid row
  const int C = d >> 3;
  const int nkb = (C + kKBlock - 1) / kKBlock;
  const St* base[G];
#pragma unroll
  for (int i = 0; i < G; ++i) base[i] = src + (int64_t)(g0 + i) * stride + tok * d;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < G; ++i) acc[m][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < G; ++i) ss[i] = 0.f;

  const int kb_end = ((wave + 1) * nkb) >> 2;
  for (int kb0 = (wave * nkb) >> 2; kb0 < kb_end; kb0 += KB) {
    // All loads of KB K-blocks first (queries and sources of their 4 steps
    // each), then the matrix-core work in K-block order: the scheduling
    // barrier keeps the compiler from sinking loads next to their first use,
    // so a wave keeps KB * 4 * (2*MT + G) 16-byte loads in flight.  A K-block
    // past the wave's range loads a valid one again and is skipped.
    typename Mfma<St>::A a[KB][4][MT];
    typename Mfma<St>::B b[KB][4][G];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int kb = kb0 + u < kb_end ? kb0 + u : kb0;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int c0 = kb * kKBlock + s4 * 4 + grp;
        const bool cok = c0 < C;
        const int c = cok ? c0 : C - 1;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const u32x4_t* qp = pk + packed_index<MP>(kb, m0 + m, s4, lane);
          a[u][s4][m] = Mfma<St>::from_halves(ld16(qp), ld16(qp + 64));
        }
#pragma unroll
        for (int i = 0; i < G; ++i) b[u][s4][i] = Mfma<St>::load_b(base[i] + c * 8, cok && tok_ok);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (kb0 + u < kb_end) {  // uniform
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
          for (int i = 0; i < G; ++i) {
            Mfma<St>::sumsq(b[u][s4][i], ss[i]);
#pragma unroll
            for (int m = 0; m < MT; ++m) Mfma<St>::mma(acc[m][i], a[u][s4][m], b[u][s4][i]);
          }
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
    lds_barrier();  // previous readers of the slots are done
    if (wave >= 2) put(red + (wave - 2) * kSlot, acc, ss, lane);
    lds_barrier();
    if (wave < 2) add(red + wave * kSlot, acc, ss, lane);
    lds_barrier();
    if (wave == 1) put(red, acc, ss, lane);
    lds_barrier();
    if (wave == 0) add(red, acc, ss, lane);
  }
};

// ---------------------------------------------------------------------------
// Prologue of the streaming pair: pack the tile's queries w (.) g once per
// call into matrix-core operands (layout above).  One thread per (K-block,
// m, step, lane).
template <typename St, int MT>
__global__ __launch_bounds__(256) void k_pack_queries(const float* __restrict__ w, const float* __restrict__ kg,
                                                      int S, int d, u32x4_t* __restrict__ pk) {
  const int C = d >> 3;
  const int nkb = (C + kKBlock - 1) / kKBlock;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= nkb * MT * 4 * 64) return;
  const int lane = idx & 63;
  const int s4 = (idx >> 6) & 3;
  const int m = (idx >> 8) % MT;
  const int kb = (idx >> 8) / MT;
  const int q = m * 16 + (lane & 15);
  const int c = kb * kKBlock + s4 * 4 + (lane >> 4);
  float qv[8];
  if (q < S && c < C) {
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
  u32x4_t* dst = pk + packed_index<MT>(kb, m, s4, lane);
  Mfma<St>::pack(qv, dst, dst + 64);
}

// First kernel of the streaming pair for short and mid-sized token ranges:
// the scores of sources [G*blockIdx.y, +G) (fewer in the last group) for a
// 16-token tile (blockIdx.x) and the query tiles [MT*blockIdx.z, +MT) of the
// MP packed ones (splitting the query tiles over workgroups doubles the
// workgroups of a short range and halves the packed-query bytes each one
// streams; every score is summed exactly as without the split).  The 4 waves take
// contiguous quarters of d (several K-blocks of loads in flight per wave),
// their partials are added in the fixed order (w0 + w2) + (w1 + w3) through
// LDS, and z = Z / r(u) goes to the weight slots alpha[t][q][i] of the
// workspace; k_p1_softmax turns them into weights.  G trades parallelism
// (workgroups) against re-reading the packed queries once per group.
template <typename St, int MT, int G, int MP>
__device__ __forceinline__ void score_sources(const St* src, int n, int64_t stride, int64_t T, int d,
                                              const u32x4_t* pk, int S, float eps, int64_t tok0, int g0,
                                              int m0, float* red, float* alpha) {
  constexpr int KB = G == 1 ? (MT == 1 ? 4 : 3) : (G == 2 ? 2 : 1);
  f32x4_t acc[MT][G];
  float ss[G];
  score_pass<St, MT, G, KB, MP>(src, stride, T, d, pk, tok0, g0, acc, ss, m0);
  Red<MT, G>::reduce(red, acc, ss);
  if ((threadIdx.x >> 6) == 0) {
    const int lane = threadIdx.x & 63;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int64_t tok = tok0 + col;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const float r = sqrtf(ss[i] / (float)d + eps);
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int q = (m0 + m) * 16 + grp * 4 + rr;
          if (q < S && tok < T) alpha[(tok * S + q) * n + g0 + i] = acc[m][i][rr] / r;
        }
    }
  }
}

template <typename St, int MT, int G, int MP = MT>
__global__ __launch_bounds__(256) void k_p1_scores(const St* __restrict__ src, int n, int64_t stride,
                                                   int64_t T, int d, const u32x4_t* __restrict__ pk, int S,
                                                   float eps, float* __restrict__ alpha) {
  __shared__ float red[2 * Red<MT, G>::kSlot];
  const int64_t tok0 = (int64_t)blockIdx.x * 16;
  const int g0 = blockIdx.y * G;
  const int m0 = blockIdx.z * MT;
  const int r = n - g0 < G ? n - g0 : G;  // uniform
  if (r == G) {
    score_sources<St, MT, G, MP>(src, n, stride, T, d, pk, S, eps, tok0, g0, m0, red, alpha);
  } else if (G > 1 && r == 1) {
    score_sources<St, MT, 1, MP>(src, n, stride, T, d, pk, S, eps, tok0, g0, m0, red, alpha);
  } else if (G > 2 && r == 2) {
    score_sources<St, MT, (G > 2 ? 2 : 1), MP>(src, n, stride, T, d, pk, S, eps, tok0, g0, m0, red, alpha);
  } else if (G > 3 && r == 3) {
    score_sources<St, MT, (G > 3 ? 3 : 1), MP>(src, n, stride, T, d, pk, S, eps, tok0, g0, m0, red, alpha);
  }
}

// Softmax over the n sources of every (token, query) pair, in place in the
// weight slots; the statistics go to m_out / lse_out.
__global__ __launch_bounds__(256) void k_p1_softmax(int64_t pairs, int n, int S, int64_t T,
                                                    float* __restrict__ alpha, float* __restrict__ m_out,
                                                    float* __restrict__ lse_out) {
  const int64_t pidx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (pidx >= pairs) return;
  const int64_t tok = pidx / S;
  const int q = (int)(pidx - tok * S);
  float* a = alpha + pidx * n;
  float mx = a[0];
  for (int i = 1; i < n; ++i) mx = fmaxf(mx, a[i]);
  float l = 0.f;
  for (int i = 0; i < n; ++i) l += expf(a[i] - mx);
  for (int i = 0; i < n; ++i) a[i] = expf(a[i] - mx) / l;
  if (m_out) m_out[(int64_t)q * T + tok] = mx;
  lse_out[(int64_t)q * T + tok] = mx + logf(l);
}

// Wide-tile variant of the scoring kernel for long token ranges, with the
// same results bit for bit.  A workgroup holds kWideWaves 16-token tiles over
// all of d, H compute waves per tile (bf16 sources: two, each scoring half of
// the sources, so that a compute unit has eight source streams in flight;
// fp32 sources: one), plus one loader wave.  A compute wave streams its source
// rows through a ring of D register stages (one K-block of one source per
// stage), so D-1 K-blocks are in flight while the matrix cores work on the
// oldest.  The loader wave copies the packed queries of each K-block straight
// from global memory into one of two or three LDS slots, one or two K-blocks
// ahead; the workgroup meets at one barrier per K-block.  The loader waits only
// on its own copies, so the source stream never waits behind a query load, and
// every packed query byte leaves L2 once per 64 tokens instead of once per 16.
// (Two waves per tile took phase 1 of an 8-source, 18-query block at 16384
// tokens, d = 7168, from 1.64-1.67 to 1.59-1.60 ms on an MI355X.  A
// vector-ALU-only scoring kernel for the same work, fp32 queries staged in LDS
// and 4-8 tokens x 12 queries per thread, took 673 us per launch at 16384
// tokens, d = 7168, 8 sources, 24 queries, against 254 us for the one-wave
// version of this one.)
//
// Summation order.  Per source, the K-blocks are visited in order; they form
// four contiguous classes [w*nkb/4, (w+1)*nkb/4), each summed from zero, the
// sum of squares of each class is reduced over the lane groups, and the
// classes are combined as (c0 + c2) + (c1 + c3): exactly what k_p1_scores
// gets from its four waves (one class each) and its fixed-order reduction.
struct KOrder {
  int nkb;
  __device__ __forceinline__ explicit KOrder(int n) : nkb(n) {}
  // K-block kb -> its class w; `last` marks the final K-block of the class
  __device__ __forceinline__ void at(int kb, int& w, bool& last) const {
    w = 0;
    while (w < 3 && (((w + 1) * nkb) >> 2) <= kb) ++w;
    last = kb + 1 == (((w + 1) * nkb) >> 2);
  }
};

constexpr int kWideWaves = 4;  // 16-token tiles per workgroup
// Bytes per token row of a compute wave's 16-row staging buffer: a 256-byte
// K-block plus 16, so that the operand-layout reads (16 tokens x 16 bytes
// per group of four lanes) fall on distinct banks.
constexpr int kRowPitch = 272;

// Wait until at most N vector-memory operations of this wave are in flight
// (they complete in issue order), e.g. copies straight into LDS.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Ring depth (stages of one K-block): 16 VGPRs per bf16 stage, 32 per fp32
// stage, within the 256 VGPRs a wave may hold (two waves share one SIMD).
// H: compute waves per tile.  bf16 sources take two (each scoring a share of
// the sources), at most 168 VGPRs per wave (three waves on one SIMD with the
// loader) and two stages each; fp32 sources one, with the whole register
// budget of a single wave per SIMD.
template <typename St>
struct WideHalves {
  static constexpr int value = sizeof(St) == 2 ? 2 : 1;
};
template <typename St, int MT>
struct WideDepth {
  static constexpr int value = WideHalves<St>::value == 2 ? 2 : (MT == 1 ? 6 : 4);
};
template <int MT>
struct WideDepth<float, MT> {
  static constexpr int value = 2;
};

// The wide scoring kernel.  FUSED: source n-1 is not read from src but
// formed from the pieces of the previous block's sum (npin: the stored partial, nv2: the one-before-last
// output or null, nv: the last output) and stored to ndst, the slab that
// later kernels read as source n-1; it is scored from the rounded values, so
// the results equal those of summing first and scoring afterwards, bit for
// bit.  Its K-blocks come last, through a ring of two stages of pieces.
template <typename St, int MT, typename Vt = St, typename Pt = float, bool FUSED = false,
          int kWideHalves = WideHalves<St>::value, bool ROWS = false>
__global__ __launch_bounds__(64 * (kWideWaves * kWideHalves + 1)) void k_p1_scores_wide(
    const St* __restrict__ src, int n, int64_t stride, int64_t T, int d, const u32x4_t* __restrict__ pk, int S,
    float eps, float* __restrict__ alpha, float* __restrict__ m_out, float* __restrict__ lse_out,
    const Pt* __restrict__ npin, const Vt* __restrict__ nv2, const Vt* __restrict__ nv, St* __restrict__ ndst,
    int nslot) {
  constexpr int D = WideDepth<St, MT>::value;
  constexpr int QW = MT * 512;  // 16-byte words per packed K-block
  // nslot (2 or 3) LDS slots of packed queries, then per tile z[16 tokens][S][n],
  // then (ROWS) a 16-row staging buffer per compute wave
  extern __shared__ u32x4_t wide_lds[];
  u32x4_t* const qs = wide_lds;
  float* const zs = reinterpret_cast<float*>(wide_lds + nslot * QW);
  unsigned char* const rowbuf = reinterpret_cast<unsigned char*>(zs + kWideWaves * 16 * S * n);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int C = d >> 3;
  const int nkb = (C + kKBlock - 1) / kKBlock;
  // With two waves per tile they score the sources [0, n0) and [n0, n); the
  // newest source (formed from its pieces when FUSED) is the last of its
  // half.  Both take one K-block step per barrier, the shorter half idling
  // through the longer one's extra steps.
  const int n0 = kWideHalves == 2 ? (n + 1) >> 1 : n;
  const int nsteps = n0 * nkb;  // K-block steps of the longer half
  const KOrder ko(nkb);
  // Global memory is touched only by loads until the last loop ends, and
  // every load below is unconditional (indices clamped), so the compiler
  // counts the loads in flight exactly and never waits for a younger stage.

  if (wave == kWideWaves * kWideHalves) {
    // loader: the queries of step `it` are copied from global memory
    // straight into LDS slot it % nslot (no registers), nslot - 1 steps
    // ahead; at the barrier of step it only the copies of later steps may
    // be in flight
    const int nit = nsteps;
    const int ahead = nslot - 1;
    auto fetch = [&](int it) {
      const u32x4_t* p = pk + (int64_t)(it % nkb) * QW + lane;
      u32x4_t* q = qs + (it % nslot) * QW;
#pragma unroll
      for (int j = 0; j < MT * 8; ++j) __builtin_amdgcn_global_load_lds(p + j * 64, q + j * 64, 16, 0, 0);
    };
    for (int k = 0; k < ahead && k < nit; ++k) fetch(k);
    for (int it = 0; it < nit; ++it) {
      if (ahead == 2 && it + 1 < nit) {
        wait_vmcnt<MT * 8>();
      } else {
        wait_vmcnt<0>();
      }
      // a bare barrier: the wait above already covers the copies that the
      // compute waves read after it (a fence would drain every copy)
      __builtin_amdgcn_s_barrier();
      if (it + ahead < nit) fetch(it + ahead);
    }
    return;
  }

  typedef typename Mfma<St>::B B;
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int tile = wave % kWideWaves;
  const int half = wave / kWideWaves;
  const int sb = half ? n0 : 0, se = half ? n : n0;  // this wave's sources (all of them for one wave per tile)
  const bool own_fused = FUSED && se == n && se > sb;  // the newest source is this wave's
  const int nitr = (se - sb - (own_fused ? 1 : 0)) * nkb;  // steps that read src
  const int64_t tok0 = (int64_t)blockIdx.x * (16 * kWideWaves) + tile * 16;
  const int64_t tokc = tok0 + col < T ? tok0 + col : T - 1;  // clamped row; results of such lanes are dropped
  const St* row = src + tokc * d;
  float* zw = zs + tile * (16 * S * n);
  unsigned char* const wb = rowbuf + wave * (16 * kRowPitch);  // ROWS: this wave's staging rows
  B b[D][4];
  auto issue = [&](B(&bs)[4], int it) {
    it = it < nitr ? it : nitr - 1;
    const int i = it / nkb;
    const int kb = it - i * nkb;
    if constexpr (ROWS) {
      // whole-row pieces: load s4 covers tokens 4 s4 .. 4 s4 + 3 of the
      // tile, 16 lanes (the K-block's 256 contiguous bytes) per token
      const St* sbase = src + (int64_t)(sb + i) * stride;
      const int c0 = kb * kKBlock + (lane & 15);
      const int cc = c0 < C ? c0 : C - 1;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int64_t tk = tok0 + s4 * 4 + (lane >> 4);
        bs[s4] = Mfma<St>::load_b(sbase + (tk < T ? tk : T - 1) * d + cc * 8, true);
      }
    } else {
      const St* base = row + (int64_t)(sb + i) * stride;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        // raw load: chunks past the end of d are zeroed when the stage is used,
        // so that nothing here waits for the data
        const int c0 = kb * kKBlock + s4 * 4 + grp;
        bs[s4] = Mfma<St>::load_b(base + (c0 < C ? c0 : C - 1) * 8, true);
      }
    }
  };

  const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
  f32x4_t acc[MT], P[MT], Q[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = P[m] = Q[m] = zero4;
  float ss = 0.f, PS = 0.f, QS = 0.f;

  // one iteration: wait for the queries, then the matrix-core work on the
  // oldest ring stage, then the per-class / per-source bookkeeping
  auto step = [&](B(&bs)[4], const u32x4_t* slot, int it, auto rows) {
    const int kb = it % nkb;
    const int i = sb + it / nkb;  // the source
    if constexpr (decltype(rows)::value) {
      // whole-row pieces to the operand layout through the wave's own LDS
      // rows (a wave's LDS accesses complete in order: no wait or barrier)
      static_assert(!decltype(rows)::value || sizeof(B) == 16, "whole-row staging is for bf16 rows");
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        *reinterpret_cast<u32x4_t*>(wb + (s4 * 4 + (lane >> 4)) * kRowPitch + (lane & 15) * 16) =
            *reinterpret_cast<const u32x4_t*>(&bs[s4]);
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        *reinterpret_cast<u32x4_t*>(&bs[s4]) =
            *reinterpret_cast<const u32x4_t*>(wb + col * kRowPitch + (s4 * 4 + grp) * 16);
    }
    int w;
    bool last;
    ko.at(kb, w, last);
    if ((kb + 1) * kKBlock > C) {  // the K-block runs past the end of d
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
        if (kb * kKBlock + s4 * 4 + grp >= C) bs[s4] = Mfma<St>::zero_b();
    }
    // the query fragments of the next matrix-core step are read from LDS
    // while the current one runs (two waves share a SIMD, so the register
    // file holds two fragment sets per wave, not a whole K-block's)
    typename Mfma<St>::A a[2][MT];
    const u32x4_t* q = slot + lane;
    auto frag = [&](typename Mfma<St>::A(&fa)[MT], int s4) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const u32x4_t* qp = q + ((m * 4 + s4) * 2) * 64;
        fa[m] = Mfma<St>::from_halves(qp[0], qp[64]);
      }
    };
    frag(a[0], 0);
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      if (s4 < 3) frag(a[(s4 + 1) & 1], s4 + 1);
      Mfma<St>::sumsq(bs[s4], ss);
#pragma unroll
      for (int m = 0; m < MT; ++m) Mfma<St>::mma(acc[m], a[s4 & 1][m], bs[s4]);
    }
    if (last) {
      float sw = ss;
      sw += __shfl_xor(sw, 16, 64);
      sw += __shfl_xor(sw, 32, 64);
      if (w == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m) P[m] = acc[m];
        PS = sw;
      } else if (w == 1) {
#pragma unroll
        for (int m = 0; m < MT; ++m) Q[m] = acc[m];
        QS = sw;
      } else if (w == 2) {
#pragma unroll
        for (int m = 0; m < MT; ++m) P[m] += acc[m];
        PS += sw;
      } else {
#pragma unroll
        for (int m = 0; m < MT; ++m) Q[m] += acc[m];
        QS += sw;
      }
#pragma unroll
      for (int m = 0; m < MT; ++m) acc[m] = zero4;
      ss = 0.f;
    }
    if (kb == nkb - 1) {
      // source i done: z = Z / r(u_i), kept in LDS until the softmax
      const float r = sqrtf((PS + QS) / (float)d + eps);
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int qi = m * 16 + grp * 4 + rr;
          if (qi < S) zw[(col * S + qi) * n + i] = (P[m][rr] + Q[m][rr]) / r;
        }
#pragma unroll
      for (int m = 0; m < MT; ++m) P[m] = Q[m] = zero4;
      PS = QS = 0.f;
    }
  };

  if (nitr > 0) {  // uniform
#pragma unroll
    for (int s = 0; s < D - 1; ++s) issue(b[s], s);
    int it0 = 0;
    for (; it0 + D <= nitr; it0 += D) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        issue(b[(s + D - 1) % D], it0 + s + D - 1);
        lds_barrier();  // the queries of this K-block are in slot (it0 + s) % nslot
        step(b[s], qs + ((it0 + s) % nslot) * QW, it0 + s, std::integral_constant<bool, ROWS>{});
      }
    }
#pragma unroll
    for (int s = 0; s < D - 1; ++s)  // tail: every stage is already loaded
      if (it0 + s < nitr) {
        lds_barrier();
        step(b[s], qs + ((it0 + s) % nslot) * QW, it0 + s, std::integral_constant<bool, ROWS>{});
      }
  }
  if (FUSED && own_fused) {
    // source n-1 from its pieces (loads unconditional: a missing v2 is
    // replaced by v and not added)
    const int64_t plane = T * (int64_t)d;
    const bool live = tok0 + col < T;
    RowExp<Pt> qe;
    qe.load(npin, tokc, plane);
    const Vt* v2p = nv2 ? nv2 : nv;
    PieceStage<Vt, Pt> ps[2];
    auto pissue = [&](PieceStage<Vt, Pt>& st, int kb) {
      kb = kb < nkb ? kb : nkb - 1;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int c0 = kb * kKBlock + s4 * 4 + grp;
        const int64_t off = tokc * d + (c0 < C ? c0 : C - 1) * 8;
        st.p[s4].load_at(npin, off, plane);
        st.a[s4].load(v2p + off);
        st.b[s4].load(nv + off);
      }
    };
    auto pstep = [&](const PieceStage<Vt, Pt>& st, int kb) {
      B bs[4];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const int c0 = kb * kKBlock + s4 * 4 + grp;
        float x[8], y[8];
        unpack_partial(st.p[s4], qe, x);
        if (nv2) {
          st.a[s4].unpack(y);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = x[e] + y[e];
        }
        st.b[s4].unpack(y);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = x[e] + y[e];
        bs[s4] = RoundB<St>::round_store(x, ndst + tokc * d + (c0 < C ? c0 : C - 1) * 8, live && c0 < C);
      }
      const int it = nitr + kb;
      step(bs, qs + (it % nslot) * QW, it, std::false_type{});
    };
    pissue(ps[0], 0);
    for (int kb = 0; kb < nkb; kb += 2) {
      pissue(ps[1], kb + 1);
      __builtin_amdgcn_sched_barrier(0);
      lds_barrier();
      pstep(ps[0], kb);
      __builtin_amdgcn_sched_barrier(0);
      pissue(ps[0], kb + 2);
      __builtin_amdgcn_sched_barrier(0);
      if (kb + 1 < nkb) {  // uniform
        lds_barrier();
        pstep(ps[1], kb + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // the shorter half's idle steps, then every score of the tile is in LDS
  for (int k = (se - sb) * nkb; k < nsteps; ++k) lds_barrier();
  lds_barrier();
  // softmax over the n sources of every (token, query) pair of the tile, the
  // pairs shared by the tile's two waves
  for (int pidx = half * 64 + lane; pidx < 16 * S; pidx += 64 * kWideHalves) {
    const int t = pidx / S, qi = pidx - t * S;
    const int64_t tok = tok0 + t;
    if (tok >= T) continue;
    const float* z = zw + pidx * n;
    float mx = z[0];
    for (int i = 1; i < n; ++i) mx = fmaxf(mx, z[i]);
    float l = 0.f;
    for (int i = 0; i < n; ++i) l += expf(z[i] - mx);
    float* a = alpha + (tok * S + qi) * n;
    for (int i = 0; i < n; ++i) a[i] = expf(z[i] - mx) / l;
    if (m_out) m_out[(int64_t)qi * T + tok] = mx;
    lse_out[(int64_t)qi * T + tok] = mx + logf(l);
  }
}

// S >= 2, second kernel: out[q][t] = sum_i alpha[t][q][i] u_i[t] (query 0 to
// out0, which is out itself unless the first query is redirected).  A wave owns
// one (token, group of 64 chunks) item at a time, so the weights are
// wave-uniform; every source chunk is used by all S queries; the next item's
// source chunks are loaded before the current item is computed (when the
// wave has a next item).  N is the exact number of sources.  The S output
// rows are written with non-temporal stores: they are read back only by the
// phase-2 launches, long after this kernel.
//
// SM: alpha holds the scores z rather than the weights, and the softmax over
// the n sources runs here: lane q loads and normalises query q's n scores
// with the operations of k_p1_softmax in the same order (the same weights bit
// for bit), the loop over the queries takes each weight from that lane, and
// the items of chunk group 0 store the statistics.  It saves the softmax
// launch of a short token range.  Without SM the weights come in through
// scalar loads.
template <typename Ut, int N, bool SM>
__device__ __forceinline__ void p1_issue(Chunk<Ut> (&s)[N], float (&z)[N], bool& ok, int64_t item, int64_t items,
                                         int ngroups, const Ut* __restrict__ src, int64_t stride, int d, int C,
                                         int lane, const float* __restrict__ alpha, int S) {
  const int64_t it = item < items ? item : items - 1;
  const int64_t t = it / ngroups;
  const int c0 = (int)(it - t * ngroups) * 64 + lane;
  ok = c0 < C;
  const int c = ok ? c0 : C - 1;
#pragma unroll
  for (int i = 0; i < N; ++i) s[i].load(src + (int64_t)i * stride + t * d + c * 8);
  if (SM) {
    const float* zr = alpha + (t * S + (lane < S ? lane : 0)) * N;
#pragma unroll
    for (int i = 0; i < N; ++i) z[i] = zr[i];
  }
}

template <typename Ut, typename St, int N, bool SM>
__device__ __forceinline__ void p1_emit(const Chunk<Ut> (&s)[N], const float (&z)[N], bool ok, int64_t item,
                                        int ngroups, int64_t T, int d, int lane, const float* __restrict__ alpha,
                                        int S, St* __restrict__ out, St* __restrict__ out0,
                                        float* __restrict__ m_out, float* __restrict__ lse_out) {
  const int64_t t = item / ngroups;
  const int g = (int)(item - t * ngroups);
  const int c = g * 64 + lane;
  float wt[N];
  if (SM) {
    float mx = z[0];
#pragma unroll
    for (int i = 1; i < N; ++i) mx = fmaxf(mx, z[i]);
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < N; ++i) l += expf(z[i] - mx);
#pragma unroll
    for (int i = 0; i < N; ++i) wt[i] = expf(z[i] - mx) / l;
    if (g == 0 && lane < S) {
      if (m_out) m_out[(int64_t)lane * T + t] = mx;
      lse_out[(int64_t)lane * T + t] = mx + logf(l);
    }
  }
  float b[N][8];
#pragma unroll
  for (int i = 0; i < N; ++i) s[i].unpack(b[i]);
  const float* al = alpha + t * S * N;
  for (int q = 0; q < S; ++q) {
    float o[8];
    zero8(o);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float a = SM ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt[i]), q)) : al[q * N + i];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = fmaf(a, b[i][e], o[e]);
    }
    if (ok) out8_nt((q == 0 ? out0 : out + (int64_t)q * T * d) + t * d + c * 8, o);
  }
}

template <typename Ut, typename St, int N, bool SM>
__global__ __launch_bounds__(256) void k_p1_out(const Ut* __restrict__ src, int64_t stride, int64_t T, int d,
                                                const float* __restrict__ alpha, int S, St* __restrict__ out,
                                                St* __restrict__ out0, float* __restrict__ m_out,
                                                float* __restrict__ lse_out) {
  const int C = d >> 3;
  const int ngroups = (C + 63) >> 6;
  const int64_t items = T * ngroups;
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  int64_t item = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Chunk<Ut> A[N], B[N];
  float zA[N], zB[N];
  bool okA, okB;
  if (item >= items) return;  // uniform over the wave
  p1_issue<Ut, N, SM>(A, zA, okA, item, items, ngroups, src, stride, d, C, lane, alpha, S);
  // the wave's last item has a branch of its own, so that the next item's
  // loads are unconditional in every other step (and stay in flight across
  // the wait for the current item's)
  while (true) {
    if (item + nw >= items) {
      p1_emit<Ut, St, N, SM>(A, zA, okA, item, ngroups, T, d, lane, alpha, S, out, out0, m_out, lse_out);
      break;
    }
    p1_issue<Ut, N, SM>(B, zB, okB, item + nw, items, ngroups, src, stride, d, C, lane, alpha, S);
    p1_emit<Ut, St, N, SM>(A, zA, okA, item, ngroups, T, d, lane, alpha, S, out, out0, m_out, lse_out);
    item += nw;
    if (item + nw >= items) {
      p1_emit<Ut, St, N, SM>(B, zB, okB, item, ngroups, T, d, lane, alpha, S, out, out0, m_out, lse_out);
      break;
    }
    p1_issue<Ut, N, SM>(A, zA, okA, item + nw, items, ngroups, src, stride, d, C, lane, alpha, S);
    p1_emit<Ut, St, N, SM>(B, zB, okB, item, ngroups, T, d, lane, alpha, S, out, out0, m_out, lse_out);
    item += nw;
  }
}

// The same outputs in token order, for long token ranges: each wave owns whole
// tokens (w, w + W, w + 2W, ... for the W waves of the grid) and walks the
// chunk groups of one token before the next, with the following group's
// source chunks in flight.  Launched with one workgroup per compute unit:
// fewer concurrent write streams keep HBM writes closer to their ceiling
// than the interleaved item order does.
//
// FIRST: the first query's output is the whole input of the block's first
// sublayer (it has no partial-sum source, "Attention Residuals" notes,
// section 10), so its PreNorm is applied here and o_0 itself is not stored:
// o_0 is rounded to the storage type (the value a store and a later load
// would give), kept in the wave's slice of LDS and its squares summed; after
// the token's last group the wave writes x_0 = gamma0 (.) o_0 / r(o_0)
// (and o_0 to h0 when asked).  `out` may then be null (one source: every
// query's output is the source row itself).
template <typename St>
struct FirstSlot;
template <>
struct FirstSlot<bf16_t> {
  static constexpr int kWords = 1;  // u32x4 words per 8-channel chunk
  __device__ static void put(u32x4_t* p, const float (&o)[8], float (&r)[8]) {
    const u32x4_t u{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                    pack_bf16x2(o[6], o[7])};
    p[0] = u;
    Chunk<bf16_t> c;
    c.r = u;
    c.unpack(r);
  }
  __device__ static void get(const u32x4_t* p, float (&r)[8]) {
    Chunk<bf16_t> c;
    c.r = p[0];
    c.unpack(r);
  }
};
template <>
struct FirstSlot<float> {
  static constexpr int kWords = 2;
  __device__ static void put(u32x4_t* p, const float (&o)[8], float (&r)[8]) {
    p[0] = u32x4_t{__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]), __float_as_uint(o[3])};
    p[1] = u32x4_t{__float_as_uint(o[4]), __float_as_uint(o[5]), __float_as_uint(o[6]), __float_as_uint(o[7])};
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = o[e];
  }
  __device__ static void get(const u32x4_t* p, float (&r)[8]) {
    const u32x4_t a = p[0], b = p[1];
    r[0] = __uint_as_float(a.x), r[1] = __uint_as_float(a.y), r[2] = __uint_as_float(a.z), r[3] = __uint_as_float(a.w);
    r[4] = __uint_as_float(b.x), r[5] = __uint_as_float(b.y), r[6] = __uint_as_float(b.z), r[7] = __uint_as_float(b.w);
  }
};

// LDS bytes of the FIRST variant: four per-wave copies of o_0 plus gamma0.
static inline size_t first_lds_bytes(int d, bool f32) {
  const size_t padded = (size_t)((((d >> 3) + 63) >> 6) * 64) * 8;  // channels, whole groups
  return 4 * padded * (f32 ? 4 : 2) + padded * 4;
}

template <typename Ut, int N>
__device__ __forceinline__ void p1_issue_tok(Chunk<Ut> (&s)[N], int64_t t, int g, int64_t T,
                                             const Ut* __restrict__ src, int64_t stride, int d, int C, int lane) {
  const int64_t tc = t < T ? t : T - 1;
  const int c0 = g * 64 + lane;
  const int c = c0 < C ? c0 : C - 1;
#pragma unroll
  for (int i = 0; i < N; ++i) s[i].load(src + (int64_t)i * stride + tc * d + c * 8);
}

template <typename Ut, typename St, int N, bool FIRST>
__global__ __launch_bounds__(256) void k_p1_out_tokens(const Ut* __restrict__ src, int64_t stride, int64_t T,
                                                       int d, const float* __restrict__ alpha, int S,
                                                       St* __restrict__ out, const float* __restrict__ gamma0,
                                                       float eps, St* __restrict__ x0, St* __restrict__ h0) {
  extern __shared__ u32x4_t first_lds[];
  const int C = d >> 3;
  const int ngroups = (C + 63) >> 6;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * 4;
  constexpr int kW = FirstSlot<St>::kWords;
  u32x4_t* mine = first_lds + (size_t)wave * ngroups * 64 * kW;  // this wave's o_0
  const float* gl = reinterpret_cast<const float*>(first_lds + (size_t)4 * ngroups * 64 * kW);
  if (FIRST) {
    float* g = reinterpret_cast<float*>(first_lds + (size_t)4 * ngroups * 64 * kW);
    for (int k = threadIdx.x; k < ngroups * 512; k += 256) g[k] = k < d ? (gamma0 ? gamma0[k] : 1.f) : 0.f;
    lds_barrier();
  }
  int64_t t = (int64_t)blockIdx.x * 4 + wave;  // current item (t, g)
  int g = 0;
  int64_t tn = t;  // next item
  int gn = g;
  auto advance = [&](int64_t& tt, int& gg) {
    if (++gg == ngroups) {
      gg = 0;
      tt += nw;
    }
  };
  advance(tn, gn);
  // |o_0|^2 in the order of the merge kernel's PreNorm, so that x_0 is the
  // same bits whichever path forms it: rows of at most 256 chunks (a wave per
  // token there) in one lane sum over the lane's chunks; wider rows (a
  // 256-thread team there, thread t holding chunks t, t + 256, ...) in four
  // sums by chunk group modulo 4, added as (s0 + s1) + (s2 + s3) after the
  // lane reductions
  const bool wide_row = C > 256;  // uniform
  float ss0 = 0.f, ss1 = 0.f, ss2 = 0.f, ss3 = 0.f;

  auto emit = [&](const Chunk<Ut>(&s)[N], int64_t tok, int grp) {
    const int c = grp * 64 + lane;
    const bool ok = c < C;
    float b[N][8];
#pragma unroll
    for (int i = 0; i < N; ++i) s[i].unpack(b[i]);
    const float* al = alpha + tok * S * N;
    int q = 0;
    if (FIRST) {
      float o[8];
      zero8(o);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const float a = al[i];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(a, b[i][e], o[e]);
      }
      float r[8];
      FirstSlot<St>::put(mine + (size_t)c * kW, o, r);
      if (ok) {
        // the chunk group's sum: all four read and written back as values
        // (selecting among the captured variables themselves selects their
        // addresses, which keeps them in scratch memory)
        const int sel = wide_row ? (grp & 3) : 0;
        const float a0 = ss0, a1 = ss1, a2 = ss2, a3 = ss3;
        float acc = sel == 0 ? a0 : sel == 1 ? a1 : sel == 2 ? a2 : a3;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(r[e], r[e], acc);
        ss0 = sel == 0 ? acc : a0;
        ss1 = sel == 1 ? acc : a1;
        ss2 = sel == 2 ? acc : a2;
        ss3 = sel == 3 ? acc : a3;
        if (h0) out8(h0 + tok * d + c * 8, o);
      }
      q = 1;
      if (!out) q = S;  // one source: nothing else to write
    }
    for (; q < S; ++q) {
      float o[8];
      zero8(o);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const float a = al[q * N + i];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(a, b[i][e], o[e]);
      }
      if (ok) out8_nt(out + ((int64_t)q * T + tok) * d + c * 8, o);
    }
    if (FIRST && grp == ngroups - 1) {
      // the token's last group: PreNorm of o_0 from the wave's LDS copy
      const float tot = wide_row ? (wave_sum_dpp(ss0) + wave_sum_dpp(ss1)) + (wave_sum_dpp(ss2) + wave_sum_dpp(ss3))
                                 : wave_sum_dpp(ss0);
      ss0 = ss1 = ss2 = ss3 = 0.f;
      const float rinv = 1.0f / sqrtf(tot * (1.0f / (float)d) + eps);
#pragma unroll 2
      for (int gg = 0; gg < ngroups; ++gg) {
        const int cc = gg * 64 + lane;
        if (cc < C) {
          float o[8], x[8];
          FirstSlot<St>::get(mine + (size_t)cc * kW, o);
          const float4 g0 = *reinterpret_cast<const float4*>(gl + cc * 8);
          const float4 g1 = *reinterpret_cast<const float4*>(gl + cc * 8 + 4);
          const float gm[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = gm[e] * (o[e] * rinv);
          out8(x0 + tok * d + cc * 8, x);
        }
      }
    }
  };

  Chunk<Ut> A[N], B[N];
  p1_issue_tok<Ut, N>(A, t, g, T, src, stride, d, C, lane);
  while (t < T) {
    p1_issue_tok<Ut, N>(B, tn, gn, T, src, stride, d, C, lane);
    emit(A, t, g);
    t = tn, g = gn;
    advance(tn, gn);
    if (t >= T) break;
    p1_issue_tok<Ut, N>(A, tn, gn, T, src, stride, d, C, lane);
    emit(B, t, g);
    t = tn, g = gn;
    advance(tn, gn);
  }
}

// Short token ranges with the first sublayer's PreNorm, rows of more than
// 256 chunks: a workgroup per token (persistent over tokens), wave w taking
// the chunk groups w, w + 4, w + 8, ...  Those are exactly the chunks of the
// merge kernel's wave w for such rows (its 256-thread team gives thread t
// the chunks t, t + 256, ...), so |o_0|^2 is summed in the merge's order (a
// lane sum in chunk order, the DPP wave sum, then (w0 + w1) + (w2 + w3)) and
// x_0 has the bits of phase 1 followed by the merge launch that this kernel
// replaces.  alpha holds the scores; the softmax runs here as in k_p1_out's
// SM variant (the same weights bit for bit) and wave 0 stores the
// statistics.  o_0 is rounded to the storage type and kept in LDS until the
// row's sum is known; slab 0 of out is not written.
template <typename Ut, typename St, int N>
__global__ __launch_bounds__(256) void k_p1_out_wg(const Ut* __restrict__ src, int64_t stride, int64_t T, int d,
                                                   const float* __restrict__ alpha, int S, St* __restrict__ out,
                                                   const float* __restrict__ gamma0, float eps, St* __restrict__ x0,
                                                   St* __restrict__ h0, float* __restrict__ m_out,
                                                   float* __restrict__ lse_out) {
  extern __shared__ u32x4_t wg_lds[];  // o_0 of the token, kW words per chunk
  __shared__ float red[4];
  constexpr int kW = FirstSlot<St>::kWords;
  const int C = d >> 3;
  const int ngroups = (C + 63) >> 6;  // at least 5 here
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const float inv_d = 1.0f / (float)d;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    // the token's weights: lane q normalises query q's scores
    float z[N], wt[N];
    {
      const float* zr = alpha + (t * S + (lane < S ? lane : 0)) * N;
#pragma unroll
      for (int i = 0; i < N; ++i) z[i] = zr[i];
    }
    Chunk<Ut> A[N], B[N];
    int g = wave;
    p1_issue_tok<Ut, N>(A, t, g, T, src, stride, d, C, lane);
    {
      float mx = z[0];
#pragma unroll
      for (int i = 1; i < N; ++i) mx = fmaxf(mx, z[i]);
      float l = 0.f;
#pragma unroll
      for (int i = 0; i < N; ++i) l += expf(z[i] - mx);
#pragma unroll
      for (int i = 0; i < N; ++i) wt[i] = expf(z[i] - mx) / l;
      if (wave == 0 && lane < S) {
        if (m_out) m_out[(int64_t)lane * T + t] = mx;
        lse_out[(int64_t)lane * T + t] = mx + logf(l);
      }
    }
    float ss = 0.f;
    auto emit = [&](const Chunk<Ut>(&s)[N], int grp) {
      const int c = grp * 64 + lane;
      const bool ok = c < C;
      float b[N][8];
#pragma unroll
      for (int i = 0; i < N; ++i) s[i].unpack(b[i]);
      {
        float o[8], r[8];
        zero8(o);
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt[i]), 0));
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = fmaf(a, b[i][e], o[e]);
        }
        if (ok) {
          FirstSlot<St>::put(wg_lds + (size_t)c * kW, o, r);
#pragma unroll
          for (int e = 0; e < 8; ++e) ss = fmaf(r[e], r[e], ss);
          if (h0) out8(h0 + t * d + c * 8, o);
        }
      }
      for (int q = 1; q < S; ++q) {
        float o[8];
        zero8(o);
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt[i]), q));
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = fmaf(a, b[i][e], o[e]);
        }
        if (ok) out8_nt(out + ((int64_t)q * T + t) * d + c * 8, o);
      }
    };
    // the wave's last group has a branch of its own, so that the next
    // group's loads are unconditional in every other step
    while (true) {
      if (g + 4 >= ngroups) {
        emit(A, g);
        break;
      }
      p1_issue_tok<Ut, N>(B, t, g + 4, T, src, stride, d, C, lane);
      emit(A, g);
      g += 4;
      if (g + 4 >= ngroups) {
        emit(B, g);
        break;
      }
      p1_issue_tok<Ut, N>(A, t, g + 4, T, src, stride, d, C, lane);
      emit(B, g);
      g += 4;
    }
    const float ws = wave_sum_dpp(ss);
    if (lane == 0) red[wave] = ws;
    lds_barrier();
    const float tot = (red[0] + red[1]) + (red[2] + red[3]);
    const float rinv = 1.0f / sqrtf(tot * inv_d + eps);
    for (int gg = wave; gg < ngroups; gg += 4) {
      const int cc = gg * 64 + lane;
      if (cc < C) {
        float o[8], gm[8], x[8];
        FirstSlot<St>::get(wg_lds + (size_t)cc * kW, o);
        if (gamma0) {
          load8(gamma0 + cc * 8, gm);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) gm[e] = 1.f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = gm[e] * (o[e] * rinv);
        out8(x0 + t * d + cc * 8, x);
      }
    }
    lds_barrier();  // the next token rewrites red and the copy of o_0
  }
}

// ---------------------------------------------------------------------------
// S == 1 with rows of at most 256 chunks (Full AttnRes one-shot sites, the
// final aggregation without a workspace): one pass over the sources with an
// online softmax, so every source row is read once.  A wave owns one token at
// a time; per batch of BS sources it forms each score (w (.) g).u / r(u) from
// the row held in registers (DPP wave sums for the dot product and the sum
// of squares), then rescales the running maximum, normaliser and output by
// the batch's new maximum -- the log-sum-exp merge of the notes' two-phase
// scheme, applied batch by batch -- and adds the batch's weighted rows.  The
// next (token, batch) item's loads are in flight while the current one is
// used (an exit-free two-stage ring; the last batch's missing sources load
// the last source again and get weight zero).
template <typename St, int K1>
__global__ __launch_bounds__(256) void k_site_online(const St* __restrict__ src, int n, int64_t stride, int64_t T,
                                                     int d, const float* __restrict__ w,
                                                     const float* __restrict__ kg,
                                                     const float* __restrict__ gamma, float eps,
                                                     St* __restrict__ h_out, St* __restrict__ x_out,
                                                     float* __restrict__ m_out, float* __restrict__ lse_out) {
  constexpr int BS = (sizeof(St) == 2 ? 8 : 4) / K1 > 0 ? (sizeof(St) == 2 ? 8 : 4) / K1 : 1;
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nw = (int64_t)gridDim.x * 4;
  const int C = d >> 3;
  const float inv_d = 1.0f / (float)d;
  // this lane's chunks of the folded query and of the PreNorm gain (zero /
  // one past the end of the row)
  float q[K1][8], gm[K1][8];
#pragma unroll
  for (int k = 0; k < K1; ++k) {
    const int c = lane + 64 * k;
    if (c < C) {
      load8(w + c * 8, q[k]);
      if (kg) {
        float g8[8];
        load8(kg + c * 8, g8);
#pragma unroll
        for (int e = 0; e < 8; ++e) q[k][e] *= g8[e];
      }
    } else {
      zero8(q[k]);
    }
    if (gamma && x_out && c < C) {
      load8(gamma + c * 8, gm[k]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) gm[k][e] = 1.f;
    }
  }
  const int64_t ntok = gw < T ? (T - gw + nw - 1) / nw : 0;  // this wave's tokens
  const int nb = (n + BS - 1) / BS;
  const int64_t items = ntok * nb;
  if (items == 0) return;
  auto issue = [&](Chunk<St>(&u)[BS][K1], int64_t it) {
    const int64_t itc = it < items ? it : items - 1;
    const int64_t tq = itc / nb;
    const int b = (int)(itc - tq * nb);
    const int64_t tok = gw + tq * nw;
#pragma unroll
    for (int j = 0; j < BS; ++j) {
      const int i = b * BS + j < n ? b * BS + j : n - 1;
#pragma unroll
      for (int k = 0; k < K1; ++k) {
        const int c0 = lane + 64 * k;
        u[j][k].load(src + (int64_t)i * stride + tok * d + (c0 < C ? c0 : C - 1) * 8);
      }
    }
  };
  float m = -INFINITY, l = 0.f;
  float o[K1][8];
#pragma unroll
  for (int k = 0; k < K1; ++k) zero8(o[k]);
  auto consume = [&](const Chunk<St>(&u)[BS][K1], int64_t it) {
    const int64_t tq = it / nb;
    const int b = (int)(it - tq * nb);
    float v[BS][K1][8], z[BS];
    float zmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < BS; ++j) {
      float zp = 0.f, sp = 0.f;
#pragma unroll
      for (int k = 0; k < K1; ++k) {
        u[j][k].unpack(v[j][k]);
        const bool cok = lane + 64 * k < C;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v[j][k][e] = cok ? v[j][k][e] : 0.f;
          zp = fmaf(q[k][e], v[j][k][e], zp);
          sp = fmaf(v[j][k][e], v[j][k][e], sp);
        }
      }
      const float zs = wave_sum_dpp(zp) / sqrtf(wave_sum_dpp(sp) * inv_d + eps);
      z[j] = b * BS + j < n ? zs : -INFINITY;
      zmax = fmaxf(zmax, z[j]);
    }
    if (b == 0) {
      m = -INFINITY;
      l = 0.f;
#pragma unroll
      for (int k = 0; k < K1; ++k) zero8(o[k]);
    }
    const float mn = fmaxf(m, zmax);            // finite: every batch has a source
    const float sc = m == -INFINITY ? 0.f : expf(m - mn);
    l *= sc;
#pragma unroll
    for (int k = 0; k < K1; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[k][e] *= sc;
#pragma unroll
    for (int j = 0; j < BS; ++j) {
      const float p = expf(z[j] - mn);          // 0 for a missing source
      l += p;
#pragma unroll
      for (int k = 0; k < K1; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[k][e] = fmaf(p, v[j][k][e], o[k][e]);
    }
    m = mn;
    if (b == nb - 1) {
      const int64_t tok = gw + tq * nw;
      const float il = 1.0f / l;
      float ssq = 0.f;
#pragma unroll
      for (int k = 0; k < K1; ++k) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o[k][e] *= il;
          ssq = fmaf(o[k][e], o[k][e], ssq);
        }
        const int c = lane + 64 * k;
        if (h_out && c < C) store8(h_out + tok * d + c * 8, o[k]);
      }
      if (x_out) {
        const float rinv = 1.0f / sqrtf(wave_sum_dpp(ssq) * inv_d + eps);
#pragma unroll
        for (int k = 0; k < K1; ++k) {
          const int c = lane + 64 * k;
          if (c < C) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = gm[k][e] * (o[k][e] * rinv);
            store8(x_out + tok * d + c * 8, x);
          }
        }
      }
      if (lane == 0) {
        if (m_out) m_out[tok] = m;
        if (lse_out) lse_out[tok] = m + logf(l);
      }
    }
  };
  Chunk<St> A[BS][K1], B[BS][K1];
  issue(A, 0);
  int64_t it = 0;
  for (; it + 2 <= items; it += 2) {
    issue(B, it + 1);
    __builtin_amdgcn_sched_barrier(0);
    consume(A, it);
    __builtin_amdgcn_sched_barrier(0);
    issue(A, it + 2);
    __builtin_amdgcn_sched_barrier(0);
    consume(B, it + 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (it < items) consume(A, it);
}

// ---------------------------------------------------------------------------
// S == 1 with wider rows (the final aggregation, Full AttnRes sites of more
// than 256 chunks): the same one-pass online softmax with a 512-thread
// workgroup per token, each thread owning CPT chunks of the row.  A batch's
// 2 x BS partial sums (w (.) g).u and |u|^2 are added over the workgroup in
// one fixed-order reduction (DPP wave sums, then the 8 waves in index order
// through LDS; two buffers alternate, so one barrier per reduction).  The
// next DEPTH - 1 (token, batch) items' loads are in flight meanwhile; the
// rows are read once, with non-temporal loads.  One source per batch, two
// stages and four workgroups per CU took the 16K chunk's final site (9
// sources, d = 7168) from 0.63 to 0.49 ms on an MI355X; batches of 3 or 4
// sources, or 3 to 6 stages, were slower in the same run.  Rows of at most
// 512 chunks take one chunk per thread (with two, every second load was a
// clamped duplicate) and three stages: 16384 tokens at d = 4096 with 17
// sources in 0.70-0.72 ms instead of 0.88-0.90 (9 sources 0.44 instead of
// 0.53); batches of two sources were 5% faster at 17 sources but 40% slower
// at one.
constexpr int kTeam = 512;

template <typename St, int CPT, int BS, int DEPTH>
__global__ __launch_bounds__(kTeam) void k_site_team(const St* __restrict__ src, int n, int64_t stride, int64_t T,
                                                     int d, const float* __restrict__ w,
                                                     const float* __restrict__ kg,
                                                     const float* __restrict__ gamma, float eps,
                                                     St* __restrict__ h_out, St* __restrict__ x_out,
                                                     float* __restrict__ m_out, float* __restrict__ lse_out) {
  constexpr int NW = kTeam / 64;
  __shared__ float red[2][NW][2 * BS];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int C = d >> 3;
  const float inv_d = 1.0f / (float)d;
  float q[CPT][8], gm[CPT][8];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    const int c = threadIdx.x + kTeam * k;
    if (c < C) {
      load8(w + c * 8, q[k]);
      if (kg) {
        float g8[8];
        load8(kg + c * 8, g8);
#pragma unroll
        for (int e = 0; e < 8; ++e) q[k][e] *= g8[e];
      }
    } else {
      zero8(q[k]);
    }
    if (gamma && x_out && c < C) {
      load8(gamma + c * 8, gm[k]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) gm[k][e] = 1.f;
    }
  }
  const int64_t ntok = (int64_t)blockIdx.x < T ? (T - blockIdx.x + gridDim.x - 1) / gridDim.x : 0;
  const int nb = (n + BS - 1) / BS;
  const int64_t items = ntok * nb;
  if (items == 0) return;  // uniform over the workgroup
  int parity = 0;
  // fixed-order workgroup sum of v[0..NV); every thread gets the sums
  auto team_sum = [&](auto& v) {
    constexpr int NV = sizeof(v) / sizeof(float);
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = wave_sum_dpp(v[i]);
    if (lane == 0) {
#pragma unroll
      for (int i = 0; i < NV; ++i) red[parity][wv][i] = v[i];
    }
    lds_barrier();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float t = red[parity][0][i];
#pragma unroll
      for (int r = 1; r < NW; ++r) t += red[parity][r][i];
      v[i] = t;
    }
    parity ^= 1;
  };
  auto issue = [&](Chunk<St>(&u)[BS][CPT], int64_t it) {
    const int64_t itc = it < items ? it : items - 1;
    const int64_t tq = itc / nb;
    const int b = (int)(itc - tq * nb);
    const int64_t tok = blockIdx.x + tq * gridDim.x;
#pragma unroll
    for (int j = 0; j < BS; ++j) {
      const int i = b * BS + j < n ? b * BS + j : n - 1;
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int c0 = threadIdx.x + kTeam * k;
        u[j][k].load_nt(src + (int64_t)i * stride + tok * d + (c0 < C ? c0 : C - 1) * 8);
      }
    }
  };
  float m = -INFINITY, l = 0.f;
  float o[CPT][8];
#pragma unroll
  for (int k = 0; k < CPT; ++k) zero8(o[k]);
  auto consume = [&](const Chunk<St>(&u)[BS][CPT], int64_t it) {
    const int64_t tq = it / nb;
    const int b = (int)(it - tq * nb);
    float part[2 * BS];
#pragma unroll
    for (int j = 0; j < BS; ++j) {
      float zp = 0.f, sp = 0.f;
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        float v[8];
        u[j][k].unpack(v);
        const bool cok = (int)threadIdx.x + kTeam * k < C;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = cok ? v[e] : 0.f;
          zp = fmaf(q[k][e], x, zp);
          sp = fmaf(x, x, sp);
        }
      }
      part[2 * j] = zp;
      part[2 * j + 1] = sp;
    }
    team_sum(part);
    float z[BS];
    float zmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < BS; ++j) {
      z[j] = b * BS + j < n ? part[2 * j] / sqrtf(part[2 * j + 1] * inv_d + eps) : -INFINITY;
      zmax = fmaxf(zmax, z[j]);
    }
    if (b == 0) {
      m = -INFINITY;
      l = 0.f;
#pragma unroll
      for (int k = 0; k < CPT; ++k) zero8(o[k]);
    }
    const float mn = fmaxf(m, zmax);  // finite: every batch has a source
    const float sc = m == -INFINITY ? 0.f : expf(m - mn);
    l *= sc;
#pragma unroll
    for (int k = 0; k < CPT; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[k][e] *= sc;
#pragma unroll
    for (int j = 0; j < BS; ++j) {
      const float p = expf(z[j] - mn);  // 0 for a missing source
      l += p;
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        float v[8];
        u[j][k].unpack(v);
        const bool cok = (int)threadIdx.x + kTeam * k < C;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[k][e] = fmaf(p, cok ? v[e] : 0.f, o[k][e]);
      }
    }
    m = mn;
    if (b == nb - 1) {
      const int64_t tok = blockIdx.x + tq * gridDim.x;
      const float il = 1.0f / l;
      float ssq = 0.f;
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o[k][e] *= il;
          ssq = fmaf(o[k][e], o[k][e], ssq);
        }
        const int c = threadIdx.x + kTeam * k;
        if (h_out && c < C) store8(h_out + tok * d + c * 8, o[k]);
      }
      if (x_out) {
        float sq[1] = {ssq};
        team_sum(sq);
        const float rinv = 1.0f / sqrtf(sq[0] * inv_d + eps);
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
          const int c = threadIdx.x + kTeam * k;
          if (c < C) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = gm[k][e] * (o[k][e] * rinv);
            store8(x_out + tok * d + c * 8, x);
          }
        }
      }
      if (threadIdx.x == 0) {
        if (m_out) m_out[tok] = m;
        if (lse_out) lse_out[tok] = m + logf(l);
      }
    }
  };
  // a ring of DEPTH stages: DEPTH - 1 (token, batch) items in flight while
  // the oldest is used
  Chunk<St> ring[DEPTH][BS][CPT];
#pragma unroll
  for (int s = 0; s < DEPTH - 1; ++s) issue(ring[s], s);
  int64_t it = 0;
  for (; it + DEPTH <= items; it += DEPTH) {
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) {
      issue(ring[(s + DEPTH - 1) % DEPTH], it + s + DEPTH - 1);
      __builtin_amdgcn_sched_barrier(0);
      consume(ring[s], it + s);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int s = 0; s < DEPTH - 1; ++s)  // tail: every stage is already loaded
    if (it + s < items) consume(ring[s], it + s);
}

// ---------------------------------------------------------------------------
// launchers

// Allow `dynamic` bytes of dynamic LDS when a launch needs more than 64 KiB
// in total (static + dynamic).
template <typename Kern>
static hipError_t set_lds(Kern k, size_t dynamic, size_t total) {
  if (total <= 65536) return hipSuccess;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)dynamic);
}
template <typename Kern>
static hipError_t set_lds(Kern k, size_t bytes) {
  return set_lds(k, bytes, bytes);
}

// Token order pays off when every wave of a one-workgroup-per-CU grid gets
// at least four whole tokens (at two per wave the interleaved order was
// faster, 7.6 vs 8.0 ms for a 2048-token chunk) and the last round of tokens
// leaves at most an eighth idle.
static bool token_order(int64_t T) {
  const int64_t W = 4 * (int64_t)device_cu_count();
  if (T < 4 * W) return false;
  return ((T + W - 1) / W) * W * 8 <= T * 9;
}

constexpr size_t kMaxLds = 160 * 1024;

// Whether k_p1_out has the variant with the softmax inside: its two register
// stages of source chunks and scores must fit (not for 9-16 fp32 sources).
template <typename Ut, int N>
constexpr bool kFuseSoftmax = sizeof(Ut) == 2 || N <= 8;

// Ut: source rows, St: outputs (the same type, or fp32 sources with bf16
// outputs; the first query's PreNorm is only fused for equal types).
template <typename Ut, typename St, int N>
static hipError_t run_out(const void* src, int64_t stride, int64_t T, int d, const float* al, int S, void* out,
                          const float* gamma0, float eps, void* x0, void* h0, float* m_out, float* lse_out,
                          bool sm, hipStream_t stream) {
  constexpr bool kSame = std::is_same<Ut, St>::value;
  const Ut* sp = static_cast<const Ut*>(src);
  St* op = static_cast<St*>(out);
  const bool tok = token_order(T);
  const dim3 tgrid((unsigned)device_cu_count());
  if (!kSame && x0) return hipErrorInvalidValue;
  // (one source and no outputs: only x_0 = PreNorm(u_0) is wanted, which the
  // merge kernel's PreNorm-only launch below forms with the same bits at its
  // streaming rate; the token-order kernel's four waves per CU took 158 us
  // for it at 16384 tokens, d = 7168)
  if (kSame && x0 && tok && (N > 1 || op) && first_lds_bytes(d, sizeof(St) == 4) <= kMaxLds) {
    const size_t lds = first_lds_bytes(d, sizeof(St) == 4);
    auto k = k_p1_out_tokens<Ut, St, N, kSame>;
    hipError_t e = set_lds(k, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, tgrid, dim3(256), lds, stream, sp, stride, T, d, al, S, op, gamma0, eps,
                       static_cast<St*>(x0), static_cast<St*>(h0));
    return hipGetLastError();
  }
  if constexpr (kSame && kFuseSoftmax<Ut, N>) {
    if (x0 && sm && op && (d >> 3) > 256) {
      // short range, wide rows: a workgroup per token with the softmax and
      // the first sublayer's PreNorm inside
      const size_t lds = (size_t)(d >> 3) * FirstSlot<St>::kWords * sizeof(u32x4_t);
      auto k = k_p1_out_wg<Ut, St, N>;
      hipError_t e = set_lds(k, lds, lds + 64);  // + the static reduction slots
      if (e != hipSuccess) return e;
      const int64_t cap = (int64_t)device_cu_count() * 4;
      hipLaunchKernelGGL(k, dim3((unsigned)(T < cap ? T : cap)), dim3(256), lds, stream, sp, stride, T, d, al, S, op,
                         gamma0, eps, static_cast<St*>(x0), static_cast<St*>(h0), m_out, lse_out);
      return hipGetLastError();
    }
  }
  // query 0 goes to h0 when the first sublayer's PreNorm follows in a second
  // launch and h0 is wanted (else to slab 0 of out, used as scratch)
  St* op0 = (x0 && h0) ? static_cast<St*>(h0) : op;
  if (op) {
    if (tok && !x0) {
      hipLaunchKernelGGL((k_p1_out_tokens<Ut, St, N, false>), tgrid, dim3(256), 0, stream, sp, stride, T, d, al, S,
                         op, nullptr, eps, nullptr, nullptr);
    } else {
      const int64_t items = T * (int64_t)(((d >> 3) + 63) >> 6);
      const int64_t wgs = (items + 3) / 4;
      const int64_t cap = (int64_t)device_cu_count() * 8;
      const dim3 grid((unsigned)(wgs < cap ? wgs : cap));
      if constexpr (kFuseSoftmax<Ut, N>) {
        if (sm) {
          hipLaunchKernelGGL((k_p1_out<Ut, St, N, true>), grid, dim3(256), 0, stream, sp, stride, T, d, al, S, op, op0,
                             m_out, lse_out);
        } else {
          hipLaunchKernelGGL((k_p1_out<Ut, St, N, false>), grid, dim3(256), 0, stream, sp, stride, T, d, al, S, op,
                             op0, nullptr, nullptr);
        }
      } else {
        if (sm) return hipErrorInvalidValue;
        hipLaunchKernelGGL((k_p1_out<Ut, St, N, false>), grid, dim3(256), 0, stream, sp, stride, T, d, al, S, op, op0,
                           nullptr, nullptr);
      }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !x0) return e;
  }
  // the first sublayer's input: h = o_0 (one source: the source row itself)
  const void* o0 = op ? static_cast<const void*>(op0) : src;
  void* hh = (h0 && o0 != h0) ? h0 : nullptr;
  return launch_merge(sizeof(St) == 4 ? kF32 : kBF16, T, d, o0, nullptr, kF32, nullptr, nullptr, nullptr, kF32,
                      nullptr, nullptr, nullptr, gamma0, eps, hh, x0, stream);
}

template <typename Ut, typename St>
static hipError_t pick_out(int n, const void* src, int64_t stride, int64_t T, int d, const float* al, int S,
                           void* out, const float* gamma0, float eps, void* x0, void* h0, float* m_out,
                           float* lse_out, bool sm, hipStream_t stream) {
  switch (n) {
#define ATTNRES_CASE(N_) \
  case N_:               \
    return run_out<Ut, St, N_>(src, stride, T, d, al, S, out, gamma0, eps, x0, h0, m_out, lse_out, sm, stream);
    ATTNRES_CASE(1) ATTNRES_CASE(2) ATTNRES_CASE(3) ATTNRES_CASE(4) ATTNRES_CASE(5) ATTNRES_CASE(6)
    ATTNRES_CASE(7) ATTNRES_CASE(8) ATTNRES_CASE(9) ATTNRES_CASE(10) ATTNRES_CASE(11) ATTNRES_CASE(12)
    ATTNRES_CASE(13) ATTNRES_CASE(14) ATTNRES_CASE(15) ATTNRES_CASE(16)
#undef ATTNRES_CASE
  }
  return hipErrorInvalidValue;
}

// The wide scoring kernel on sources of type Ut; Vt and Pt are the types of
// the newest source's pieces when FUSED.
template <typename Ut, int MT, typename Vt, typename Pt, bool FUSED, bool ROWS>
static hipError_t launch_wide_r(const void* src, int n, int64_t stride, int64_t T, int d, const u32x4_t* pk, int S,
                                float eps, float* al, float* m_out, float* lse_out, const Newest* nw,
                                hipStream_t stream) {
  const int64_t wide_groups = (T + 16 * kWideWaves - 1) / (16 * kWideWaves);
  // three query slots (copies two steps ahead) where the LDS has room, else two
  const size_t zl = sizeof(float) * kWideWaves * 16 * S * n;
  const size_t slot = sizeof(u32x4_t) * MT * 512;
  const size_t rb = ROWS ? (size_t)kWideWaves * WideHalves<Ut>::value * 16 * kRowPitch : 0;
  const int nslot = zl + 3 * slot + rb <= kMaxLds ? 3 : 2;
  const size_t lds = zl + nslot * slot + rb;
  auto kw = k_p1_scores_wide<Ut, MT, Vt, Pt, FUSED, WideHalves<Ut>::value, ROWS>;
  hipError_t e = set_lds(kw, lds);
  if (e != hipSuccess) return e;
  Ut* dst = FUSED ? static_cast<Ut*>(const_cast<void*>(src)) + (int64_t)(n - 1) * stride : nullptr;
  hipLaunchKernelGGL(kw, dim3((unsigned)wide_groups), dim3(64 * (kWideWaves * WideHalves<Ut>::value + 1)), lds, stream,
                     static_cast<const Ut*>(src), n, stride, T, d, pk, S, eps, al, m_out, lse_out,
                     static_cast<const Pt*>(FUSED ? nw->pin : nullptr), static_cast<const Vt*>(FUSED ? nw->v2 : nullptr),
                     static_cast<const Vt*>(FUSED ? nw->v : nullptr), dst, nslot);
  return hipGetLastError();
}

// bf16 rows are loaded as whole-row pieces and staged through LDS into the
// matrix-core operand layout where the LDS has room for the staging rows
// (16 tokens x 64 bytes per load instruction, the operand layout itself,
// streamed at 5.5 TB/s on an MI355X in a load-only probe of this kernel's
// pattern; 4 tokens x 256 bytes at 7.0-7.1)
template <typename Ut, int MT, typename Vt, typename Pt, bool FUSED>
static hipError_t launch_wide(const void* src, int n, int64_t stride, int64_t T, int d, const u32x4_t* pk, int S,
                              float eps, float* al, float* m_out, float* lse_out, const Newest* nw,
                              hipStream_t stream) {
  if constexpr (sizeof(Ut) == 2) {
    const size_t need = sizeof(float) * kWideWaves * 16 * S * n + 2 * sizeof(u32x4_t) * MT * 512 +
                        (size_t)kWideWaves * WideHalves<Ut>::value * 16 * kRowPitch;
    if (need <= kMaxLds)
      return launch_wide_r<Ut, MT, Vt, Pt, FUSED, true>(src, n, stride, T, d, pk, S, eps, al, m_out, lse_out, nw,
                                                        stream);
  }
  return launch_wide_r<Ut, MT, Vt, Pt, FUSED, false>(src, n, stride, T, d, pk, S, eps, al, m_out, lse_out, nw,
                                                     stream);
}

static constexpr Dtype kind_of_type(bool f32) { return f32 ? kF32 : kBF16; }

// The scores (and the query packing for their matrix-core type) follow the
// source rows' type Ut; the outputs are stored as St.
template <typename Ut, typename St, int MT>
static hipError_t run_multi(const void* src, int n, int64_t stride, int64_t T, int d, const float* w,
                            const float* kg, int S, float eps, void* out, float* m_out, float* lse_out,
                            const float* gamma0, void* x0, void* h0, float* ws, const Newest* nw,
                            hipStream_t stream) {
  // workspace: packed queries first (room for 32 queries), then the softmax
  // weights
  const int nkb = ((d >> 3) + kKBlock - 1) / kKBlock;
  u32x4_t* pk = reinterpret_cast<u32x4_t*>(ws);
  float* al = ws + (int64_t)nkb * kPackedKBlockWords * 4;
  const int npk = nkb * MT * 4 * 64;
  const int64_t wide_groups = (T + 16 * kWideWaves - 1) / (16 * kWideWaves);
  const bool wide = wide_groups >= device_cu_count();
  // the newest source from the pieces of a block sum: summed inside the wide
  // scoring kernel (a stored partial in Q16 or fp32), else by the block-sum
  // kernel first
  const bool fused = nw && wide && nw->pin && (nw->pdt == kQ16 || nw->pdt == kF32);
  bool sm = false;  // softmax inside the output kernel
  hipError_t e;
  if (nw && !fused) {
    e = launch_accumulate(nw->vdt, kind_of_type(sizeof(Ut) == 4), T, d, nw->pdt, nw->pin, nw->v2, nw->v,
                          static_cast<Ut*>(const_cast<void*>(src)) + (int64_t)(n - 1) * stride, stream);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_pack_queries<Ut, MT>), dim3((unsigned)((npk + 255) / 256)), dim3(256), 0, stream, w, kg,
                     S, d, pk);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (wide) {
    // enough 64-token tiles for one workgroup per compute unit
    if (!fused) {
      e = launch_wide<Ut, MT, St, float, false>(src, n, stride, T, d, pk, S, eps, al, m_out, lse_out, nw, stream);
    } else {
      // the pieces' type: bf16 (the only one bf16 sources take) or fp32
      bool bf16_pieces = true;
      if constexpr (sizeof(Ut) == 4) {
        bf16_pieces = nw->vdt == kBF16;
        if (!bf16_pieces)
          e = nw->pdt == kQ16 ? launch_wide<Ut, MT, float, q16_t, true>(src, n, stride, T, d, pk, S, eps, al, m_out,
                                                                       lse_out, nw, stream)
                              : launch_wide<Ut, MT, float, float, true>(src, n, stride, T, d, pk, S, eps, al, m_out,
                                                                       lse_out, nw, stream);
      }
      if (bf16_pieces)
        e = nw->pdt == kQ16 ? launch_wide<Ut, MT, bf16_t, q16_t, true>(src, n, stride, T, d, pk, S, eps, al, m_out,
                                                                      lse_out, nw, stream)
                            : launch_wide<Ut, MT, bf16_t, float, true>(src, n, stride, T, d, pk, S, eps, al, m_out,
                                                                      lse_out, nw, stream);
    }
    if (e != hipSuccess) return e;
  } else {
    // one workgroup per (16-token tile, group of G sources), then the
    // softmax per pair; G is the largest of 4, 2, 1 that still gives two
    // workgroups per compute unit
    const int64_t tiles = (T + 15) / 16;
    const int64_t want = 2 * (int64_t)device_cu_count();
    const int G = tiles * ((n + 3) / 4) >= want ? 4 : (tiles * ((n + 1) / 2) >= want ? 2 : 1);
    const dim3 grid((unsigned)tiles, (unsigned)((n + G - 1) / G));
    const Ut* sp = static_cast<const Ut*>(src);
    if (MT == 2 && tiles * n < want) {
      // still short of two workgroups per compute unit: one query tile each
      hipLaunchKernelGGL((k_p1_scores<Ut, 1, 1, MT>), dim3((unsigned)tiles, (unsigned)n, 2u), dim3(256), 0, stream,
                         sp, n, stride, T, d, pk, S, eps, al);
    } else if (G == 4) {
      hipLaunchKernelGGL((k_p1_scores<Ut, MT, 4>), grid, dim3(256), 0, stream, sp, n, stride, T, d, pk, S, eps, al);
    } else if (G == 2) {
      hipLaunchKernelGGL((k_p1_scores<Ut, MT, 2>), grid, dim3(256), 0, stream, sp, n, stride, T, d, pk, S, eps, al);
    } else {
      hipLaunchKernelGGL((k_p1_scores<Ut, MT, 1>), grid, dim3(256), 0, stream, sp, n, stride, T, d, pk, S, eps, al);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the softmax runs inside the output kernel when that is k_p1_out (short
    // ranges with outputs), else as a launch of its own
    sm = out != nullptr && !token_order(T) && (sizeof(Ut) == 2 || n <= 8);
    if (!sm) {
      const int64_t pairs = T * S;
      hipLaunchKernelGGL(k_p1_softmax, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0, stream, pairs, n, S, T,
                         al, m_out, lse_out);
    }
  }
  e = hipGetLastError();
  if (e != hipSuccess || (out == nullptr && x0 == nullptr)) return e;  // statistics only
  return pick_out<Ut, St>(n, src, stride, T, d, al, S, out, gamma0, eps, x0, h0, m_out, lse_out, sm, stream);
}

hipError_t launch_phase1_multi(Dtype dt, Dtype sdt, const void* src, int n, int64_t stride, int64_t T, int d,
                               const float* w, const float* kg, int S, float eps, void* out,
                               float* m_out, float* lse_out, const float* gamma0, void* x0, void* h0, float* ws,
                               const Newest* nw, hipStream_t stream) {
#define ATTNRES_MULTI(UT_, ST_)                                                                                   \
  return S <= 16 ? run_multi<UT_, ST_, 1>(src, n, stride, T, d, w, kg, S, eps, out, m_out, lse_out, gamma0, x0, h0, \
                                          ws, nw, stream)                                                        \
                 : run_multi<UT_, ST_, 2>(src, n, stride, T, d, w, kg, S, eps, out, m_out, lse_out, gamma0, x0, h0, \
                                          ws, nw, stream)
  if (dt == kBF16 && sdt == kBF16) ATTNRES_MULTI(bf16_t, bf16_t);
  if (dt == kBF16 && sdt == kF32) ATTNRES_MULTI(float, bf16_t);
  if (dt == kF32 && sdt == kF32) ATTNRES_MULTI(float, float);
#undef ATTNRES_MULTI
  return hipErrorInvalidValue;
}

template <typename St>
static hipError_t run_single(const void* src, int n, int64_t stride, int64_t T, int d, const float* w,
                             const float* kg, const float* gamma, float eps, void* h_out, void* x_out,
                             float* m_out, float* lse_out, hipStream_t stream) {
  const int C = d >> 3;
  if (C <= 256) {
    // one pass with an online softmax, a wave per token
    auto k = C <= 64 ? k_site_online<St, 1> : C <= 128 ? k_site_online<St, 2> : k_site_online<St, 4>;
    int64_t waves = T;
    const int64_t cap = (int64_t)device_cu_count() * 16;
    if (waves > cap) waves = cap;
    hipLaunchKernelGGL(k, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, static_cast<const St*>(src), n,
                       stride, T, d, w, kg, gamma, eps, static_cast<St*>(h_out), static_cast<St*>(x_out), m_out,
                       lse_out);
    return hipGetLastError();
  }
  if (C <= 4 * kTeam) {
    // the same one pass, a 512-thread workgroup per token
    auto k = C <= kTeam       ? k_site_team<St, 1, 1, 3>
             : C <= 2 * kTeam ? k_site_team<St, 2, 1, 2>
                              : k_site_team<St, 4, 1, 2>;
    int64_t wgs = T;
    const int64_t cap = (int64_t)device_cu_count() * 4;
    if (wgs > cap) wgs = cap;
    hipLaunchKernelGGL(k, dim3((unsigned)wgs), dim3(kTeam), 0, stream, static_cast<const St*>(src), n, stride, T, d,
                       w, kg, gamma, eps, static_cast<St*>(h_out), static_cast<St*>(x_out), m_out, lse_out);
    return hipGetLastError();
  }
  // d <= ATTNRES_MAX_D = 16384 (validated by the C ABI): at most 2048 chunks
  return hipErrorInvalidValue;
}

hipError_t launch_phase1_single(Dtype dt, const void* src, int n, int64_t stride, int64_t T, int d,
                                const float* w, const float* kg, const float* gamma, float eps,
                                void* h_out, void* x_out, float* m_out, float* lse_out,
                                hipStream_t stream) {
  if (dt == kBF16)
    return run_single<bf16_t>(src, n, stride, T, d, w, kg, gamma, eps, h_out, x_out, m_out, lse_out, stream);
  return run_single<float>(src, n, stride, T, d, w, kg, gamma, eps, h_out, x_out, m_out, lse_out, stream);
}

}  // namespace attnres
