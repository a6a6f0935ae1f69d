// Host-side launchers of the gfx950 AttnRes kernels (private to libattnres).
// Arguments are validated by the C ABI layer before these are called.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attnres {

enum Dtype { kF32 = 0, kBF16 = 1, kP24 = 2, kQ16 = 3 };

int device_cu_count();

// Phase 1 of a block, one tile of at most 32 queries (n <= 16), sources of
// type sdt (dt, or fp32 sources with bf16 outputs and no x0); `alpha` is
// workspace for the packed queries and T * S * n fp32 softmax weights.  With
// x0 != null, query 0's output goes through the PreNorm with gain gamma0
// into x0 (and as is into h0 when not null) instead of slab 0 of out, which
// may be used as scratch; out may then be null when n == 1.  Or S == 1 with
// optional PreNorm (n <= 32).  With nw != null, source n-1 is first formed
// from the pieces nw describes (fused into the scoring kernel for long
// token ranges).  Return a hipError_t.
// The newest source of a phase-1 call as the pieces of a block sum:
// ((pin or 0) + (v2 or 0)) + v, the outputs v2, v of type vdt, the partial in
// format pdt; the sum is written to source slab n-1 (of the sources' type).
struct Newest {
  const void* pin;
  Dtype pdt;
  Dtype vdt;
  const void* v2;
  const void* v;
};

hipError_t launch_phase1_multi(Dtype dt, Dtype sdt, const void* src, int n, int64_t stride, int64_t T, int d,
                               const float* w, const float* kg, int S, float eps, void* out,
                               float* m_out, float* lse_out, const float* gamma0, void* x0, void* h0,
                               float* alpha, const Newest* nw, hipStream_t stream);

hipError_t launch_phase1_single(Dtype dt, const void* src, int n, int64_t stride, int64_t T, int d,
                                const float* w, const float* kg, const float* gamma, float eps,
                                void* h_out, void* x_out, float* m_out, float* lse_out,
                                hipStream_t stream);

hipError_t launch_merge(Dtype dt, int64_t T, int d, const void* o1, const float* lse1,
                        Dtype pdt, const void* pin, const void* vprev2, const void* vprev, Dtype podt, void* pout,
                        const float* w, const float* kg, const float* gamma, float eps,
                        void* h_out, void* x_out, hipStream_t stream);

hipError_t launch_merge_multi(Dtype dt, int64_t T, int d, const void* o1, const float* lse1, const void* src,
                              int k, int64_t stride, const float* w, const float* kg, const float* gamma, float eps,
                              void* h_out, void* x_out, hipStream_t stream);

hipError_t launch_site_backward(Dtype dt, int64_t T, int d, const void* src, int n, int64_t stride, const float* w,
                                const float* kg, const float* gamma, int prenorm, float eps, const void* dx,
                                void* dsrc, int64_t dstride, int out_mode, int wadd, float* dw, float* dkg,
                                float* dgamma, float* part, hipStream_t stream);
int64_t backward_slots(int64_t T, int d);

// Backward through the block structure (training).  Phase-2 backward of one
// site: G = dL/dh to g_out, c = 1 - beta and G.h per token, the partial
// source's gradient added into dpart (fp32), and the site's partial-source
// and PreNorm parameter gradients added into dw, dkg, dgamma (part: per-team
// sums, p2_backward_slots(T, d) x 2 x d floats).
hipError_t launch_p2_backward(Dtype dt, int64_t T, int d, const void* o1, const float* lse1, Dtype pdt,
                              const void* pin, const void* vprev2, const void* vprev, const float* w, const float* kg,
                              const float* gamma, int prenorm, float eps, const void* dx, float* dpart, void* g_out,
                              float* c_out, float* gp_out, float* dw, float* dkg, float* dgamma, float* part,
                              hipStream_t stream);
int64_t p2_backward_slots(int64_t T, int d);

// Phase-1 backward of a block: the block sources' gradients written or added
// (accumulate) into dsrc (fp32), the block-source part of dw, dkg added.
// Sources of type sdt (dt, or fp32 with bf16 G rows).
// ws: T * S * n coefficients + p1_backward_ranges(d) * S * d partial sums.
hipError_t launch_p1_backward(Dtype dt, Dtype sdt, int64_t T, int d, const void* src, int n, int64_t stride, int S,
                              const float* w, const float* kg, float eps, const void* gin, int64_t gstride,
                              const float* c_in, const float* gp_in, float* dsrc, int64_t dstride, int accumulate,
                              float* dw, float* dkg, float* ws, hipStream_t stream);
int64_t p1_backward_ranges(int d);

// Streaming-bandwidth probe: n_read byte streams of stream_bytes each read
// from src (consecutive), n_write written to dst (n_write == 0: dst holds 16
// bytes that are never written in practice); per_cu workgroups per compute
// unit, `unroll` chunks per stream in flight per thread (1, 2, 4 or 8),
// non-temporal loads and stores when `nontemporal`.
hipError_t launch_stream_probe(int n_read, int n_write, const void* src, void* dst, int64_t stream_bytes,
                               int per_cu, int unroll, bool nontemporal, hipStream_t stream);

// out (of type odt: dt, or fp32 for bf16 rows) = (pin + v2) + v.
hipError_t launch_accumulate(Dtype dt, Dtype odt, int64_t T, int d, Dtype pdt, const void* pin, const void* v2,
                             const void* v, void* out, hipStream_t stream);

}  // namespace attnres
