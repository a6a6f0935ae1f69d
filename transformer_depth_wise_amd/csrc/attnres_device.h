// Device-side building blocks shared by the gfx950 AttnRes kernels.
// Private to libattnres: storage-type traits, 16-byte row-chunk loads and
// stores, and wave / workgroup reductions.  Compiled for gfx950 only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnres {

// Storage tag for bf16 rows (raw bits).  All arithmetic is fp32.
struct bf16_t {
  unsigned short bits;
};

// Storage tag for the 24-bit split format of a block's running partial sum:
// a plane of T*d 16-bit upper halves, then a plane of T*d bytes with bits
// 8..15 of the fp32 encoding rounded to nearest even at bit 8.
struct p24_t {
  unsigned char byte;
};

// Storage tag for the 16-bit fixed-point format of a block's running partial
// sum: a plane of T*d int16 values q, then T int32 row exponents e; element
// k of row t is q[t][k] * 2^(e[t] - 15), with 2^e[t] above the row's largest
// magnitude (so every element is kept to within 2^-15 of the row's largest).
struct q16_t {
  short q;
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---- 8-element row chunks ----------------------------------------------
// A "chunk" is 8 consecutive channels of one row: 16 bytes of bf16 or 32
// bytes of fp32.  d is a multiple of 8, rows are 16-byte aligned.

__device__ __forceinline__ void unpack_bf16x8(const uint4 u, float (&v)[8]) {
  v[0] = __uint_as_float(u.x << 16);
  v[1] = __uint_as_float(u.x & 0xffff0000u);
  v[2] = __uint_as_float(u.y << 16);
  v[3] = __uint_as_float(u.y & 0xffff0000u);
  v[4] = __uint_as_float(u.z << 16);
  v[5] = __uint_as_float(u.z & 0xffff0000u);
  v[6] = __uint_as_float(u.w << 16);
  v[7] = __uint_as_float(u.w & 0xffff0000u);
}

// Round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  bf16x2_t p;
  p.x = (__bf16)a;
  p.y = (__bf16)b;
  return __builtin_bit_cast(unsigned, p);
}

__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void load8(const bf16_t* p, float (&v)[8]) {
  unpack_bf16x8(*reinterpret_cast<const uint4*>(p), v);
}

__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

__device__ __forceinline__ void store8(bf16_t* p, const float (&v)[8]) {
  uint4 u;
  u.x = pack_bf16x2(v[0], v[1]);
  u.y = pack_bf16x2(v[2], v[3]);
  u.z = pack_bf16x2(v[4], v[5]);
  u.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = u;
}

__device__ __forceinline__ void zero8(float (&v)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = 0.f;
}

// ---- raw 16-byte chunks held in registers between load and use ------------
// Chunk<T> keeps 8 elements in their storage format so that loads for the
// next token or row chunk can be in flight while the current one is used.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }
__device__ __forceinline__ u32x2_t ld8(const void* p) { return *reinterpret_cast<const u32x2_t*>(p); }
__device__ __forceinline__ void st8(void* p, u32x2_t v) { *reinterpret_cast<u32x2_t*>(p) = v; }

// load_at(base, off, plane): the 8 elements at element offset `off` of a
// [T][d] buffer; `plane` = T*d is used by split formats only.
template <typename T> struct Chunk;
// Non-temporal 16- and 8-byte loads: for streams read once (or read again
// only by a later kernel), so that they do not displace reusable lines.
__device__ __forceinline__ u32x4_t ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ u32x2_t ld8_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
}

template <> struct Chunk<bf16_t> {
  u32x4_t r;
  __device__ __forceinline__ void load(const bf16_t* p) { r = ld16(p); }
  __device__ __forceinline__ void load_nt(const bf16_t* p) { r = ld16_nt(p); }
  __device__ __forceinline__ void load_at(const bf16_t* b, int64_t off, int64_t) { r = ld16(b + off); }
  __device__ __forceinline__ void load_at_nt(const bf16_t* b, int64_t off, int64_t) { r = ld16_nt(b + off); }
  __device__ __forceinline__ void zero() { r = u32x4_t{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ void unpack(float (&v)[8]) const {
    unpack_bf16x8(make_uint4(r.x, r.y, r.z, r.w), v);
  }
};
template <> struct Chunk<float> {
  u32x4_t a, b;
  __device__ __forceinline__ void load(const float* p) { a = ld16(p); b = ld16(p + 4); }
  __device__ __forceinline__ void load_nt(const float* p) { a = ld16_nt(p); b = ld16_nt(p + 4); }
  __device__ __forceinline__ void load_at(const float* p, int64_t off, int64_t) { load(p + off); }
  __device__ __forceinline__ void load_at_nt(const float* p, int64_t off, int64_t) { load_nt(p + off); }
  __device__ __forceinline__ void zero() { a = u32x4_t{0u, 0u, 0u, 0u}; b = a; }
  __device__ __forceinline__ void unpack(float (&v)[8]) const {
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  }
};
template <> struct Chunk<p24_t> {
  u32x4_t hi;  // 8 x 16-bit upper halves
  u32x2_t lo;  // 8 x 8-bit next bits
  __device__ __forceinline__ void load_at(const p24_t* b, int64_t off, int64_t plane) {
    const unsigned char* base = reinterpret_cast<const unsigned char*>(b);
    hi = ld16(base + off * 2);
    lo = ld8(base + plane * 2 + off);
  }
  __device__ __forceinline__ void load_at_nt(const p24_t* b, int64_t off, int64_t plane) {
    const unsigned char* base = reinterpret_cast<const unsigned char*>(b);
    hi = ld16_nt(base + off * 2);
    lo = ld8_nt(base + plane * 2 + off);
  }
  __device__ __forceinline__ void zero() {
    hi = u32x4_t{0u, 0u, 0u, 0u};
    lo = u32x2_t{0u, 0u};
  }
  __device__ __forceinline__ void unpack(float (&v)[8]) const {
    const unsigned h[4] = {hi.x, hi.y, hi.z, hi.w};
    const unsigned l[2] = {lo.x, lo.y};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const unsigned h16 = (h[e >> 1] >> (16 * (e & 1))) & 0xffffu;
      const unsigned l8 = (l[e >> 2] >> (8 * (e & 3))) & 0xffu;
      v[e] = __uint_as_float((h16 << 16) | (l8 << 8));
    }
  }
};

template <> struct Chunk<q16_t> {
  u32x4_t r;  // 8 int16 values
  __device__ __forceinline__ void load_at(const q16_t* b, int64_t off, int64_t) { r = ld16(b + off); }
  __device__ __forceinline__ void load_at_nt(const q16_t* b, int64_t off, int64_t) { r = ld16_nt(b + off); }
  __device__ __forceinline__ void zero() { r = u32x4_t{0u, 0u, 0u, 0u}; }
  // the values times 2^(e - 15)
  __device__ __forceinline__ void unpack(float (&v)[8], int e) const {
    const unsigned w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = (int)(short)(unsigned short)(w[i >> 1] >> (16 * (i & 1)));
      v[i] = ldexpf((float)q, e - 15);
    }
  }
};

// The per-row part of a partial-sum format: the row exponent of Q16, nothing
// for the others.  load(base, tok, plane) reads row tok's exponent from
// behind the plane of T*d values.
template <typename Pt> struct RowExp {
  __device__ __forceinline__ void load(const Pt*, int64_t, int64_t) {}
};
template <> struct RowExp<q16_t> {
  int e;
  __device__ __forceinline__ void load(const q16_t* b, int64_t tok, int64_t plane) {
    e = *reinterpret_cast<const int*>(reinterpret_cast<const unsigned char*>(b) + plane * 2 + tok * 4);
  }
};

// A partial-sum chunk as fp32 values, whatever its format.
template <typename Pt>
__device__ __forceinline__ void unpack_partial(const Chunk<Pt>& c, const RowExp<Pt>&, float (&v)[8]) {
  c.unpack(v);
}
template <>
__device__ __forceinline__ void unpack_partial(const Chunk<q16_t>& c, const RowExp<q16_t>& x, float (&v)[8]) {
  c.unpack(v, x.e);
}

// Q16 row exponent for a row whose largest magnitude is amax: the e with
// amax < 2^e (frexp's exponent; 0 for a zero row).
__device__ __forceinline__ int q16_exponent(float amax) {
  int e = 0;
  (void)frexpf(amax, &e);
  return e;
}

// 8 values of a row with exponent e as Q16 (nearest, ties to even; |q| <= 32767).
__device__ __forceinline__ u32x4_t q16_pack(const float (&v)[8], int e) {
  unsigned h[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float q = rintf(ldexpf(v[i], 15 - e));
    q = fminf(fmaxf(q, -32767.f), 32767.f);
    h[i] = (unsigned)(unsigned short)(short)(int)q;
  }
  return u32x4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

// fp32 -> upper 24 bits, round to nearest even at bit 8 (finite values).
__device__ __forceinline__ unsigned round24(float x) {
  const unsigned u = __float_as_uint(x);
  return u + 0x7fu + ((u >> 8) & 1u);
}

__device__ __forceinline__ void out24(p24_t* b, int64_t off, int64_t plane, const float (&v)[8]) {
  unsigned r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = round24(v[e]);
  unsigned char* base = reinterpret_cast<unsigned char*>(b);
  st16(base + off * 2, u32x4_t{(r[0] >> 16) | (r[1] & 0xffff0000u), (r[2] >> 16) | (r[3] & 0xffff0000u),
                               (r[4] >> 16) | (r[5] & 0xffff0000u), (r[6] >> 16) | (r[7] & 0xffff0000u)});
  st8(base + plane * 2 + off,
      u32x2_t{((r[0] >> 8) & 0xffu) | (((r[1] >> 8) & 0xffu) << 8) | (((r[2] >> 8) & 0xffu) << 16) |
                  (((r[3] >> 8) & 0xffu) << 24),
              ((r[4] >> 8) & 0xffu) | (((r[5] >> 8) & 0xffu) << 8) | (((r[6] >> 8) & 0xffu) << 16) |
                  (((r[7] >> 8) & 0xffu) << 24)});
}

// Non-temporal 16-byte store: for outputs that are not read again soon, so
// they do not displace reusable lines from the caches.
__device__ __forceinline__ void st16_nt(void* p, u32x4_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void st8_nt(void* p, u32x2_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(p));
}
// out24 with non-temporal stores
__device__ __forceinline__ void out24_nt(p24_t* b, int64_t off, int64_t plane, const float (&v)[8]) {
  unsigned r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = round24(v[e]);
  unsigned char* base = reinterpret_cast<unsigned char*>(b);
  st16_nt(base + off * 2, u32x4_t{(r[0] >> 16) | (r[1] & 0xffff0000u), (r[2] >> 16) | (r[3] & 0xffff0000u),
                                  (r[4] >> 16) | (r[5] & 0xffff0000u), (r[6] >> 16) | (r[7] & 0xffff0000u)});
  st8_nt(base + plane * 2 + off,
         u32x2_t{((r[0] >> 8) & 0xffu) | (((r[1] >> 8) & 0xffu) << 8) | (((r[2] >> 8) & 0xffu) << 16) |
                     (((r[3] >> 8) & 0xffu) << 24),
                 ((r[4] >> 8) & 0xffu) | (((r[5] >> 8) & 0xffu) << 8) | (((r[6] >> 8) & 0xffu) << 16) |
                     (((r[7] >> 8) & 0xffu) << 24)});
}
__device__ __forceinline__ void out8_nt(bf16_t* p, const float (&v)[8]) {
  st16_nt(p, u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])});
}
__device__ __forceinline__ void out8_nt(float* p, const float (&v)[8]) {
  st16_nt(p, u32x4_t{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
  st16_nt(p + 4, u32x4_t{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])});
}

__device__ __forceinline__ void out8(float* p, const float (&v)[8]) {
  st16(p, u32x4_t{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
  st16(p + 4, u32x4_t{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])});
}
__device__ __forceinline__ void out8(bf16_t* p, const float (&v)[8]) {
  st16(p, u32x4_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])});
}

// ---- reductions ------------------------------------------------------------

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// Sum over the 64 lanes of a wave without LDS: DPP butterflies inside each
// 16-lane row (swap neighbours, swap pairs, mirror halves, mirror the row;
// every step adds two equal-sized partial sums, so all lanes of a row hold
// the same bits), then the four row sums read into scalars and added as
// (r0 + r1) + (r2 + r3).  The result is the same in every lane.
template <int CTRL>
__device__ __forceinline__ float dpp_step(float x) {
  return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum_dpp(float x) {
  x = dpp_step<0xB1>(x);   // quad_perm [1,0,3,2]
  x = dpp_step<0x4E>(x);   // quad_perm [2,3,0,1]
  x = dpp_step<0x141>(x);  // row_half_mirror
  x = dpp_step<0x140>(x);  // row_mirror
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (r0 + r1) + (r2 + r3);
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// orders global memory, which makes every wave wait for all of its global
// loads and stores in flight (the prefetched next item included); here those
// stay in flight across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
  return x;
}

// The largest value over the 64 lanes with the same DPP steps as
// wave_sum_dpp (a maximum does not depend on the order).
template <int CTRL>
__device__ __forceinline__ float dpp_max_step(float x) {
  return fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false)));
}
__device__ __forceinline__ float wave_max_dpp(float x) {
  x = dpp_max_step<0xB1>(x);
  x = dpp_max_step<0x4E>(x);
  x = dpp_max_step<0x141>(x);
  x = dpp_max_step<0x140>(x);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Wave-level sum and maximum: the shuffle butterfly, or (DPP) the DPP row
// steps and scalar reads, which take a fraction of the shuffles' latency.
template <bool DPP>
__device__ __forceinline__ float wsum(float x) {
  return DPP ? wave_sum_dpp(x) : wave_sum(x);
}
template <bool DPP>
__device__ __forceinline__ float wmax(float x) {
  return DPP ? wave_max_dpp(x) : wave_max(x);
}

// Sums of a and b and the maximum of c over the 256 threads of a workgroup,
// in a fixed order (identical in every thread); `lds` holds 12 floats,
// alternated by the caller like block_sum2_256's.  DPP: the wave-level steps
// of wave_sum_dpp.
template <bool DPP = false>
__device__ __forceinline__ float3 block_sum2_max_256(float a, float b, float c, float* lds) {
  a = wsum<DPP>(a);
  b = wsum<DPP>(b);
  c = wmax<DPP>(c);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  if (lane == 0) {
    lds[3 * wave + 0] = a;
    lds[3 * wave + 1] = b;
    lds[3 * wave + 2] = c;
  }
  lds_barrier();
  float3 r;
  // the same order as block_sum2_256: (w0 + w1) + (w2 + w3)
  r.x = (lds[0] + lds[3]) + (lds[6] + lds[9]);
  r.y = (lds[1] + lds[4]) + (lds[7] + lds[10]);
  r.z = fmaxf(fmaxf(lds[2], lds[5]), fmaxf(lds[8], lds[11]));
  return r;
}

// Sum of (a, b) over the 256 threads of a workgroup, in a fixed order (the
// result is identical in every thread and from run to run).  `lds` holds 8
// floats; callers alternate between two such buffers so that one barrier per
// reduction suffices.  DPP: the wave-level steps of wave_sum_dpp.
template <bool DPP = false>
__device__ __forceinline__ float2 block_sum2_256(float a, float b, float* lds) {
  a = wsum<DPP>(a);
  b = wsum<DPP>(b);
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x >> 6;
  if (lane == 0) {
    lds[2 * wave + 0] = a;
    lds[2 * wave + 1] = b;
  }
  lds_barrier();
  float2 r;
  r.x = (lds[0] + lds[2]) + (lds[4] + lds[6]);
  r.y = (lds[1] + lds[3]) + (lds[5] + lds[7]);
  return r;
}

}  // namespace attnres
