// Streaming-bandwidth probe on gfx950: the achievable HBM rate of a kernel
// that reads NR and writes NW equally long byte streams, the way the
// aggregation kernels move rows (16-byte accesses, a wave touching 1 KiB of
// consecutive bytes per stream and instruction, a persistent grid-stride
// loop with several chunks in flight per thread).  It computes nothing of the
// method; it bounds what a kernel with that read/write mix can reach.
#include "attnres_device.h"
#include "attnres_launch.h"

namespace attnres {

template <bool NT>
__device__ __forceinline__ u32x4_t probe_ld(const unsigned char* p) {
  if (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return ld16(p);
}
template <bool NT>
__device__ __forceinline__ void probe_st(unsigned char* p, u32x4_t v) {
  if (NT) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
  } else {
    st16(p, v);
  }
}

// U chunks per stream in flight per thread; NT: non-temporal loads and stores.
template <int NR, int NW, int U, bool NT>
__global__ __launch_bounds__(256) void k_stream_probe(const unsigned char* __restrict__ src,
                                                      unsigned char* __restrict__ dst, int64_t chunks,
                                                      int64_t stream_bytes) {
  const int64_t step = (int64_t)gridDim.x * 256;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (int64_t c0 = (int64_t)blockIdx.x * 256 + threadIdx.x; c0 < chunks; c0 += step * U) {
    u32x4_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * step;
      const int64_t cc = c < chunks ? c : chunks - 1;  // clamped: loads stay unconditional
      v[u] = u32x4_t{(unsigned)cc, 0u, 0u, 0u};
#pragma unroll
      for (int r = 0; r < NR; ++r) v[u] ^= probe_ld<NT>(src + r * stream_bytes + cc * 16);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t c = c0 + u * step;
      if (NW == 0) {
        acc ^= v[u];
      } else if (c < chunks) {
#pragma unroll
        for (int k = 0; k < NW; ++k) probe_st<NT>(dst + k * stream_bytes + c * 16, v[u]);
      }
    }
  }
  // read-only: keep the loads alive with a store the data never triggers
  if (NW == 0 && acc.x == 0x9e3779b9u && acc.y == 0x7f4a7c15u && acc.z == acc.w) st16(dst, acc);
}

template <int NR, int NW, int U, bool NT>
static hipError_t run_probe(const void* src, void* dst, int64_t stream_bytes, int per_cu, hipStream_t stream) {
  const int64_t chunks = stream_bytes / 16;
  const int64_t blocks = (chunks + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * per_cu;
  const dim3 grid((unsigned)(blocks < cap ? blocks : cap));
  hipLaunchKernelGGL((k_stream_probe<NR, NW, U, NT>), grid, dim3(256), 0, stream,
                     static_cast<const unsigned char*>(src), static_cast<unsigned char*>(dst), chunks, stream_bytes);
  return hipGetLastError();
}

template <int NR, int NW>
static hipError_t probe_shape(const void* src, void* dst, int64_t stream_bytes, int per_cu, int unroll, bool nt,
                              hipStream_t stream) {
#define ATTNRES_PROBE_U(U_)                                                                        \
  if (unroll == U_)                                                                                \
    return nt ? run_probe<NR, NW, U_, true>(src, dst, stream_bytes, per_cu, stream)                \
              : run_probe<NR, NW, U_, false>(src, dst, stream_bytes, per_cu, stream)
  ATTNRES_PROBE_U(1);
  ATTNRES_PROBE_U(2);
  ATTNRES_PROBE_U(4);
  ATTNRES_PROBE_U(8);
#undef ATTNRES_PROBE_U
  return hipErrorInvalidValue;
}

hipError_t launch_stream_probe(int n_read, int n_write, const void* src, void* dst, int64_t stream_bytes,
                               int per_cu, int unroll, bool nontemporal, hipStream_t stream) {
#define ATTNRES_PROBE(R_, W_)         \
  if (n_read == R_ && n_write == W_) \
  return probe_shape<R_, W_>(src, dst, stream_bytes, per_cu, unroll, nontemporal, stream)
  ATTNRES_PROBE(1, 0);
  ATTNRES_PROBE(2, 0);
  ATTNRES_PROBE(3, 0);
  ATTNRES_PROBE(4, 0);
  ATTNRES_PROBE(0, 1);
  ATTNRES_PROBE(0, 2);
  ATTNRES_PROBE(1, 1);
  ATTNRES_PROBE(2, 1);
  ATTNRES_PROBE(3, 1);
  ATTNRES_PROBE(4, 1);
  ATTNRES_PROBE(1, 2);
  ATTNRES_PROBE(2, 2);
  ATTNRES_PROBE(3, 2);
  ATTNRES_PROBE(4, 2);
  ATTNRES_PROBE(8, 0);
  ATTNRES_PROBE(9, 1);
  ATTNRES_PROBE(7, 24);
#undef ATTNRES_PROBE
  return hipErrorInvalidValue;
}

}  // namespace attnres
