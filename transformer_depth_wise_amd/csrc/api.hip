// C ABI of libattnres: argument validation and dispatch to the gfx950
// kernels.  Every check runs on the host before anything is launched; see
// include/attnres.h for the contract of each entry point.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "../../include/attnres.h"
#include "attnres_launch.h"

namespace attnres {

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace attnres

namespace {

using attnres::Dtype;

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + static_cast<uintptr_t>(bytes)};
}

bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int64_t esize(attnres_dtype_t dt) { return dt == ATTNRES_F32 ? 4 : dt == ATTNRES_P24 ? 3 : 2; }

// Bytes of a [T][d] partial sum in format pdt (Q16: the values, then T row
// exponents).
int64_t partial_bytes(attnres_dtype_t pdt, int64_t T, int64_t d) {
  return T * d * esize(pdt) + (pdt == ATTNRES_Q16 ? T * 4 : 0);
}

// row storage: F32 or BF16; a partial sum may also be P24 or Q16
bool dtype_ok(attnres_dtype_t dt) { return dt == ATTNRES_F32 || dt == ATTNRES_BF16; }
bool partial_ok(attnres_dtype_t pdt, attnres_dtype_t dt) {
  return pdt == ATTNRES_F32 || pdt == ATTNRES_P24 || pdt == ATTNRES_Q16 || pdt == dt;
}

Dtype kind_of(attnres_dtype_t dt) {
  return dt == ATTNRES_F32   ? attnres::kF32
         : dt == ATTNRES_P24 ? attnres::kP24
         : dt == ATTNRES_Q16 ? attnres::kQ16
                             : attnres::kBF16;
}

attnres_status_t check_d(int64_t d) {
  if (d <= 0 || d > ATTNRES_MAX_D) return ATTNRES_EINVAL;
  if (d % 8 != 0) return ATTNRES_EALIGN;
  return ATTNRES_OK;
}

// token count and slab strides in range, so that every byte extent below
// fits in int64 (T * d * 4 < 2^47, S * T * d * 4 < 2^59, strides < 2^45 bytes)
bool extent_ok(int64_t T, std::initializer_list<int64_t> strides = {}) {
  if (T < 0 || T > ATTNRES_MAX_T) return false;
  for (int64_t s : strides)
    if (s < 0 || s > ATTNRES_MAX_STRIDE) return false;
  return true;
}

attnres_status_t hip_status(hipError_t e) { return e == hipSuccess ? ATTNRES_OK : ATTNRES_EHIP; }

// all non-null row pointers 16-byte aligned, statistics pointers 4-byte aligned
attnres_status_t check_align(std::initializer_list<const void*> rows,
                             std::initializer_list<const void*> stats = {}) {
  for (const void* p : rows)
    if (p && !aligned16(p)) return ATTNRES_EALIGN;
  for (const void* p : stats)
    if (p && !aligned4(p)) return ATTNRES_EALIGN;
  return ATTNRES_OK;
}

}  // namespace

extern "C" {

const char* attnres_status_string(attnres_status_t status) {
  switch (status) {
    case ATTNRES_OK: return "ATTNRES_OK";
    case ATTNRES_EINVAL: return "ATTNRES_EINVAL: null pointer, bad size or unsupported size combination";
    case ATTNRES_EDTYPE: return "ATTNRES_EDTYPE: unknown dtype";
    case ATTNRES_EALIGN: return "ATTNRES_EALIGN: d or a stride not a multiple of 8, or pointer not 16-byte aligned";
    case ATTNRES_EALIAS: return "ATTNRES_EALIAS: an output overlaps an input";
    case ATTNRES_EHIP: return "ATTNRES_EHIP: the HIP runtime reported an error";
    case ATTNRES_ESCRATCH:
      return "ATTNRES_ESCRATCH: the call needs more workspace than the allocation-free entry point's "
             "ATTNRES_NOALLOC_SCRATCH_BYTES";
  }
  return "ATTNRES_UNKNOWN_STATUS";
}

int64_t attnres_phase1_workspace_bytes(int64_t T, int64_t d, int64_t n_src, int64_t S) {
  if (!extent_ok(T) || n_src < 1 || S < 1 || S > ATTNRES_MAX_QUERIES || d <= 0 || d > ATTNRES_MAX_D || d % 8 != 0)
    return -1;
  if (n_src > ATTNRES_MAX_SOURCES_MULTI) return S == 1 ? 0 : -1;
  // packed queries (32 rows x 4 bytes x d rounded up to 128) + softmax
  // weights (T x n x min(S, 32) x 4 bytes)
  const int64_t sq = S < 32 ? S : 32;
  const int64_t kblocks = (d + 127) / 128;
  return 32 * 4 * 128 * kblocks + T * n_src * sq * (int64_t)sizeof(float);
}

// Shared by attnres_phase1 and attnres_phase1_first_prenorm (x0 != null).
// With nw != null (attnres_phase1_accumulate, validated there), source
// n_src-1 is first formed from the pieces of a block sum.
static attnres_status_t phase1_impl(attnres_dtype_t dt, attnres_dtype_t src_dt, const void* src, int64_t n_src,
                                    int64_t src_stride, int64_t T, int64_t d, const float* w,
                                    const float* key_gain, int64_t S, float eps, void* out, float* m_out,
                                    float* lse_out, const float* gamma0, void* x0, void* h0, void* workspace,
                                    int64_t workspace_bytes, void* stream, const attnres::Newest* nw = nullptr) {
  if (!dtype_ok(dt) || !dtype_ok(src_dt)) return ATTNRES_EDTYPE;
  // sources of the outputs' type, or fp32 sources with bf16 outputs
  const bool mixed = src_dt != dt;
  if (mixed && !(src_dt == ATTNRES_F32 && dt == ATTNRES_BF16)) return ATTNRES_EDTYPE;
  attnres_status_t st = check_d(d);
  if (st != ATTNRES_OK) return st;
  if (!extent_ok(T, {src_stride}) || S < 1 || S > ATTNRES_MAX_QUERIES || n_src < 1) return ATTNRES_EINVAL;
  if (n_src > (S == 1 && !x0 && !mixed ? ATTNRES_MAX_SOURCES : ATTNRES_MAX_SOURCES_MULTI)) return ATTNRES_EINVAL;
  if (mixed && x0) return ATTNRES_EINVAL;  // the first query's PreNorm is fused for equal types only
  if (!(eps >= 0.f)) return ATTNRES_EINVAL;
  if (T == 0) return ATTNRES_OK;  // empty token set: nothing is read or written
  if (!src || !w || !lse_out) return ATTNRES_EINVAL;
  if (x0 && !out && n_src > 1) return ATTNRES_EINVAL;
  if (n_src > 1 && (src_stride < T * d)) return ATTNRES_EINVAL;
  if (src_stride % 8 != 0) return ATTNRES_EALIGN;
  int64_t ws_need = attnres_phase1_workspace_bytes(T, d, n_src, S);
  // S == 1 without the first-query PreNorm (and sources of the outputs'
  // type): one pass over the sources with an online softmax; the workspace
  // is not used
  if (S == 1 && !x0 && !mixed) ws_need = 0;
  if (ws_need > 0 && (!workspace || workspace_bytes < ws_need)) return ATTNRES_EINVAL;
  st = check_align({src, w, key_gain, out, ws_need > 0 ? workspace : nullptr, gamma0, x0, h0}, {m_out, lse_out});
  if (st != ATTNRES_OK) return st;
  const int64_t es = esize(dt);
  const Range rs = range_of(src, ((n_src - 1) * src_stride + T * d) * esize(src_dt));
  const Range ro = out ? range_of(out, S * T * d * es) : Range{0, 0};
  const Range rl = range_of(lse_out, S * T * 4);
  const Range rm = m_out ? range_of(m_out, S * T * 4) : Range{0, 0};
  const Range rw = range_of(w, S * d * 4);
  const Range rg = key_gain ? range_of(key_gain, S * d * 4) : Range{0, 0};
  const Range rws = ws_need > 0 ? range_of(workspace, ws_need) : Range{0, 0};
  const Range rx = x0 ? range_of(x0, T * d * es) : Range{0, 0};
  const Range rh = h0 ? range_of(h0, T * d * es) : Range{0, 0};
  const Range rgm = gamma0 ? range_of(gamma0, d * 4) : Range{0, 0};
  for (Range o : {ro, rl, rm, rws, rx, rh})
    for (Range i : {rs, rw, rg, rgm})
      if (overlaps(o, i)) return ATTNRES_EALIAS;
  {
    const Range outs[] = {ro, rl, rm, rws, rx, rh};
    for (int a = 0; a < 6; ++a)
      for (int b = a + 1; b < 6; ++b)
        if (overlaps(outs[a], outs[b])) return ATTNRES_EALIAS;
  }

  const Dtype kdt = kind_of(dt);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (S == 1 && ws_need == 0) {
    if (nw) {
      void* newest = static_cast<char*>(const_cast<void*>(src)) + (n_src - 1) * src_stride * esize(src_dt);
      if (attnres::launch_accumulate(nw->vdt, kind_of(src_dt), T, (int)d, nw->pdt, nw->pin, nw->v2, nw->v, newest, s) !=
          hipSuccess)
        return ATTNRES_EHIP;
    }
    return hip_status(attnres::launch_phase1_single(kdt, src, (int)n_src, src_stride, T, (int)d, w, key_gain,
                                                    nullptr, eps, out, nullptr, m_out, lse_out, s));
  }
  for (int64_t s0 = 0; s0 < S; s0 += 32) {
    const int64_t sn = (S - s0) < 32 ? (S - s0) : 32;
    char* o = out ? static_cast<char*>(out) + s0 * T * d * es : nullptr;
    hipError_t e = attnres::launch_phase1_multi(kdt, kind_of(src_dt), src, (int)n_src, src_stride, T, (int)d,
                                                w + s0 * d,
                                                key_gain ? key_gain + s0 * d : nullptr, (int)sn, eps, o,
                                                m_out ? m_out + s0 * T : nullptr, lse_out + s0 * T, gamma0,
                                                s0 == 0 ? x0 : nullptr, s0 == 0 ? h0 : nullptr,
                                                static_cast<float*>(workspace), s0 == 0 ? nw : nullptr, s);
    if (e != hipSuccess) return ATTNRES_EHIP;
  }
  return ATTNRES_OK;
}

attnres_status_t attnres_phase1(attnres_dtype_t dt, attnres_dtype_t src_dt, const void* src, int64_t n_src,
                                int64_t src_stride, int64_t T, int64_t d, const float* w, const float* key_gain,
                                int64_t S, float eps, void* out, float* m_out, float* lse_out, void* workspace,
                                int64_t workspace_bytes, void* stream) {
  return phase1_impl(dt, src_dt, src, n_src, src_stride, T, d, w, key_gain, S, eps, out, m_out, lse_out, nullptr, nullptr,
                     nullptr, workspace, workspace_bytes, stream);
}

// ---------------------------------------------------------------------------
// Allocation-free phase 1: the workspace is this file's device array instead
// of caller memory.  Each GPU holds its own copy for the life of the process;
// its address on the current device is looked up once per device (with that
// device current) and kept, and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[ATTNRES_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mutex;
void* g_scratch_ptr[64] = {nullptr};

// The current device's copy of `scratch`, or nullptr if it cannot be found.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

attnres_status_t attnres_phase1_noalloc(attnres_dtype_t dt, const void* src, int64_t n_src, int64_t src_stride,
                                        int64_t T, int64_t d, const float* w, const float* key_gain, int64_t S,
                                        float eps, void* out, float* m_out, float* lse_out, void* stream) {
  // the sizes are checked (and T == 0 returns) before anything touches the device
  if (!dtype_ok(dt)) return ATTNRES_EDTYPE;
  const int64_t need = attnres_phase1_workspace_bytes(T, d, n_src, S);
  if (need < 0) return phase1_impl(dt, dt, src, n_src, src_stride, T, d, w, key_gain, S, eps, out, m_out, lse_out,
                                   nullptr, nullptr, nullptr, nullptr, 0, stream);
  if (need > ATTNRES_NOALLOC_SCRATCH_BYTES) return ATTNRES_ESCRATCH;
  if (T == 0)
    return phase1_impl(dt, dt, src, n_src, src_stride, T, d, w, key_gain, S, eps, out, m_out, lse_out, nullptr,
                       nullptr, nullptr, nullptr, 0, stream);
  void* ws = scratch_on_current_device();
  if (!ws) return ATTNRES_EHIP;
  return phase1_impl(dt, dt, src, n_src, src_stride, T, d, w, key_gain, S, eps, out, m_out, lse_out, nullptr, nullptr,
                     nullptr, ws, ATTNRES_NOALLOC_SCRATCH_BYTES, stream);
}

attnres_status_t attnres_phase1_first_prenorm(attnres_dtype_t dt, const void* src, int64_t n_src,
                                              int64_t src_stride, int64_t T, int64_t d, const float* w,
                                              const float* key_gain, int64_t S, float eps, void* out,
                                              float* m_out, float* lse_out, const float* prenorm_gain,
                                              void* x_out, void* h_out, void* workspace, int64_t workspace_bytes,
                                              void* stream) {
  if (!x_out) return ATTNRES_EINVAL;
  return phase1_impl(dt, dt, src, n_src, src_stride, T, d, w, key_gain, S, eps, out, m_out, lse_out, prenorm_gain,
                     x_out, h_out, workspace, workspace_bytes, stream);
}

attnres_status_t attnres_phase1_accumulate(attnres_dtype_t dt, attnres_dtype_t src_dt, void* src, int64_t n_src,
                                           int64_t src_stride, int64_t T, int64_t d, const float* w,
                                           const float* key_gain, int64_t S, float eps, attnres_dtype_t partial_dt,
                                           const void* partial_in, attnres_dtype_t sublayer_dt,
                                           const void* sublayer_prev2, const void* sublayer_prev, void* out,
                                           float* m_out, float* lse_out, const float* prenorm_gain, void* x_out,
                                           void* h_out, void* workspace, int64_t workspace_bytes, void* stream) {
  if (!dtype_ok(dt) || !dtype_ok(src_dt) || !dtype_ok(sublayer_dt) || !partial_ok(partial_dt, sublayer_dt))
    return ATTNRES_EDTYPE;
  // the phase-1 pair, and the block sum's (pieces of sublayer_dt stored as src_dt)
  if (src_dt != dt && !(src_dt == ATTNRES_F32 && dt == ATTNRES_BF16)) return ATTNRES_EDTYPE;
  if (src_dt != sublayer_dt && !(src_dt == ATTNRES_F32 && sublayer_dt == ATTNRES_BF16)) return ATTNRES_EDTYPE;
  if (x_out && src_dt != dt) return ATTNRES_EINVAL;  // as attnres_phase1_first_prenorm
  if (!x_out && (prenorm_gain || h_out)) return ATTNRES_EINVAL;
  attnres_status_t st = check_d(d);
  if (st != ATTNRES_OK) return st;
  if (!extent_ok(T, {src_stride}) || S < 1 || S > ATTNRES_MAX_QUERIES) return ATTNRES_EINVAL;
  const int64_t max_src = (S == 1 && !x_out && src_dt == dt) ? ATTNRES_MAX_SOURCES : ATTNRES_MAX_SOURCES_MULTI;
  if (n_src < 2 || n_src > max_src) return ATTNRES_EINVAL;
  if (T > 0) {
    if (!src || !sublayer_prev || !lse_out) return ATTNRES_EINVAL;
    st = check_align({partial_in, sublayer_prev2, sublayer_prev});
    if (st != ATTNRES_OK) return st;
    // the newest slab is written: no piece may overlap it, and no output
    // may overlap a piece (the outputs are checked against src below)
    const int64_t rows = T * d;
    const Range rn = range_of(static_cast<char*>(src) + (n_src - 1) * src_stride * esize(src_dt), rows * esize(src_dt));
    const Range pieces[] = {range_of(sublayer_prev, rows * esize(sublayer_dt)),
                            sublayer_prev2 ? range_of(sublayer_prev2, rows * esize(sublayer_dt)) : Range{0, 0},
                            partial_in ? range_of(partial_in, partial_bytes(partial_dt, T, d)) : Range{0, 0}};
    const int64_t es = esize(dt);
    const Range outs[] = {out ? range_of(out, S * rows * es) : Range{0, 0}, range_of(lse_out, S * T * 4),
                          m_out ? range_of(m_out, S * T * 4) : Range{0, 0},
                          x_out ? range_of(x_out, rows * es) : Range{0, 0},
                          h_out ? range_of(h_out, rows * es) : Range{0, 0},
                          workspace ? range_of(workspace, std::max<int64_t>(0, attnres_phase1_workspace_bytes(
                                                                     T, d, n_src, S)))
                                    : Range{0, 0}};
    for (Range pr : pieces) {
      if (overlaps(pr, rn)) return ATTNRES_EALIAS;
      for (Range o : outs)
        if (overlaps(pr, o)) return ATTNRES_EALIAS;
    }
  }
  const attnres::Newest nw{partial_in, kind_of(partial_dt), kind_of(sublayer_dt), sublayer_prev2, sublayer_prev};
  return phase1_impl(dt, src_dt, src, n_src, src_stride, T, d, w, key_gain, S, eps, out, m_out, lse_out,
                     x_out ? prenorm_gain : nullptr, x_out, h_out, workspace, workspace_bytes, stream, &nw);
}

attnres_status_t attnres_phase2_merge(attnres_dtype_t dt, int64_t T, int64_t d, const void* p1_out,
                                      const float* p1_lse, attnres_dtype_t partial_dt, const void* partial_in,
                                      const void* sublayer_prev2, const void* sublayer_prev,
                                      attnres_dtype_t partial_out_dt, void* partial_out,
                                      const float* w, const float* key_gain, const float* prenorm_gain, float eps,
                                      void* h_out, void* x_out, void* stream) {
  if (!dtype_ok(dt) || !partial_ok(partial_dt, dt)) return ATTNRES_EDTYPE;
  if (partial_out_dt != ATTNRES_F32 && partial_out_dt != ATTNRES_P24 && partial_out_dt != ATTNRES_Q16)
    return ATTNRES_EDTYPE;
  attnres_status_t st = check_d(d);
  if (st != ATTNRES_OK) return st;
  if (!extent_ok(T) || !(eps >= 0.f)) return ATTNRES_EINVAL;
  if (!sublayer_prev && (partial_in || partial_out || sublayer_prev2)) return ATTNRES_EINVAL;
  if (T == 0) return ATTNRES_OK;  // empty token set: nothing is read or written
  if (!p1_out || !p1_lse || (!h_out && !x_out)) return ATTNRES_EINVAL;
  if (sublayer_prev && !w) return ATTNRES_EINVAL;
  st = check_align({p1_out, partial_in, sublayer_prev2, sublayer_prev, partial_out, w, key_gain, prenorm_gain, h_out,
                    x_out},
                   {p1_lse});
  if (st != ATTNRES_OK) return st;
  const int64_t es = esize(dt);
  const int64_t rows = T * d;
  const Range r_o = range_of(p1_out, rows * es), r_l = range_of(p1_lse, T * 4);
  const Range r_pi = partial_in ? range_of(partial_in, partial_bytes(partial_dt, T, d)) : Range{0, 0};
  const Range r_v = sublayer_prev ? range_of(sublayer_prev, rows * es) : Range{0, 0};
  const Range r_v2 = sublayer_prev2 ? range_of(sublayer_prev2, rows * es) : Range{0, 0};
  const Range r_po = partial_out ? range_of(partial_out, partial_bytes(partial_out_dt, T, d)) : Range{0, 0};
  const Range r_w = w ? range_of(w, d * 4) : Range{0, 0};
  const Range r_g = key_gain ? range_of(key_gain, d * 4) : Range{0, 0};
  const Range r_gm = prenorm_gain ? range_of(prenorm_gain, d * 4) : Range{0, 0};
  const Range r_h = h_out ? range_of(h_out, rows * es) : Range{0, 0};
  const Range r_x = x_out ? range_of(x_out, rows * es) : Range{0, 0};
  // partial_out may be exactly partial_in (same format, element-wise in place); no other overlap
  const bool in_place = partial_out && partial_in == static_cast<const void*>(partial_out) &&
                        partial_dt == partial_out_dt;
  for (Range o : {r_h, r_x, r_po})
    for (Range i : {r_o, r_l, r_pi, r_v, r_v2, r_w, r_g, r_gm}) {
      if (in_place && o.lo == r_po.lo && o.hi == r_po.hi && i.lo == r_pi.lo && i.hi == r_pi.hi) continue;
      if (overlaps(o, i)) return ATTNRES_EALIAS;
    }
  if (overlaps(r_h, r_x) || overlaps(r_h, r_po) || overlaps(r_x, r_po)) return ATTNRES_EALIAS;
  return hip_status(attnres::launch_merge(kind_of(dt), T, (int)d, p1_out, p1_lse, kind_of(partial_dt), partial_in,
                                          sublayer_prev2, sublayer_prev, kind_of(partial_out_dt), partial_out, w,
                                          key_gain,
                                          x_out ? prenorm_gain : nullptr, eps, h_out, x_out,
                                          static_cast<hipStream_t>(stream)));
}

attnres_status_t attnres_phase2_merge_multi(attnres_dtype_t dt, int64_t T, int64_t d, const void* p1_out,
                                            const float* p1_lse, const void* src, int64_t n_src,
                                            int64_t src_stride, const float* w, const float* key_gain,
                                            const float* prenorm_gain, float eps, void* h_out, void* x_out,
                                            void* stream) {
  if (!dtype_ok(dt)) return ATTNRES_EDTYPE;
  attnres_status_t st = check_d(d);
  if (st != ATTNRES_OK) return st;
  if (!extent_ok(T, {src_stride}) || n_src < 0 || n_src > ATTNRES_MAX_GROUP_SOURCES || !(eps >= 0.f))
    return ATTNRES_EINVAL;
  if (T == 0) return ATTNRES_OK;  // empty token set: nothing is read or written
  if (!p1_out || !p1_lse || (!h_out && !x_out)) return ATTNRES_EINVAL;
  if (n_src > 0 && (!src || !w)) return ATTNRES_EINVAL;
  if (n_src > 1 && src_stride < T * d) return ATTNRES_EINVAL;
  if (n_src > 0 && src_stride % 8 != 0) return ATTNRES_EALIGN;
  st = check_align({p1_out, n_src > 0 ? src : nullptr, w, key_gain, prenorm_gain, h_out, x_out}, {p1_lse});
  if (st != ATTNRES_OK) return st;
  const int64_t es = esize(dt);
  const Range r_o = range_of(p1_out, T * d * es), r_l = range_of(p1_lse, T * 4);
  const Range r_s = n_src > 0 ? range_of(src, ((n_src - 1) * src_stride + T * d) * es) : Range{0, 0};
  const Range r_w = w ? range_of(w, d * 4) : Range{0, 0};
  const Range r_g = key_gain ? range_of(key_gain, d * 4) : Range{0, 0};
  const Range r_gm = prenorm_gain ? range_of(prenorm_gain, d * 4) : Range{0, 0};
  const Range r_h = h_out ? range_of(h_out, T * d * es) : Range{0, 0};
  const Range r_x = x_out ? range_of(x_out, T * d * es) : Range{0, 0};
  for (Range o : {r_h, r_x})
    for (Range i : {r_o, r_l, r_s, r_w, r_g, r_gm})
      if (overlaps(o, i)) return ATTNRES_EALIAS;
  if (overlaps(r_h, r_x)) return ATTNRES_EALIAS;
  return hip_status(attnres::launch_merge_multi(kind_of(dt), T, (int)d, p1_out, p1_lse, n_src > 0 ? src : nullptr,
                                                (int)n_src, src_stride, w, key_gain, x_out ? prenorm_gain : nullptr,
                                                eps, h_out, x_out, static_cast<hipStream_t>(stream)));
}

int64_t attnres_site_backward_workspace_bytes(int64_t T, int64_t d) {
  if (!extent_ok(T) || d <= 0 || d > ATTNRES_MAX_D || d % 8 != 0) return -1;
  if (T == 0) return 0;
  return attnres::backward_slots(T, (int)d) * 2 * d * (int64_t)sizeof(float);
}

// Shared by the storing and the accumulating entry points: dsrc holds rows
// of the storage type, or fp32 rows to add to (acc).
static attnres_status_t site_backward_impl(attnres_dtype_t dt, const void* src, int64_t n_src, int64_t src_stride,
                                           int64_t T, int64_t d, const float* w, const float* key_gain,
                                           const float* prenorm_gain, int prenorm, float eps, const void* dx,
                                           void* dsrc, int64_t dsrc_stride, bool acc, float* dw, float* dkey_gain,
                                           float* dprenorm_gain, void* workspace, int64_t workspace_bytes,
                                           void* stream) {
  if (!dtype_ok(dt)) return ATTNRES_EDTYPE;
  attnres_status_t st = check_d(d);
  if (st != ATTNRES_OK) return st;
  if (!extent_ok(T, {src_stride, dsrc_stride}) || n_src < 1 || n_src > ATTNRES_MAX_SOURCES || !(eps >= 0.f))
    return ATTNRES_EINVAL;
  if (T == 0) return ATTNRES_OK;  // empty token set: nothing is read or written
  if (!src || !w || !dx || !dsrc || !dw) return ATTNRES_EINVAL;
  if (n_src > 1 && (src_stride < T * d || dsrc_stride < T * d)) return ATTNRES_EINVAL;
  if (src_stride % 8 != 0 || dsrc_stride % 8 != 0) return ATTNRES_EALIGN;
  const int64_t ws_need = attnres_site_backward_workspace_bytes(T, d);
  if (!workspace || workspace_bytes < ws_need) return ATTNRES_EINVAL;
  st = check_align({src, w, key_gain, prenorm_gain, dx, dsrc, workspace}, {dw, dkey_gain, dprenorm_gain});
  if (st != ATTNRES_OK) return st;
  const int64_t es = esize(dt);
  const Range rs = range_of(src, ((n_src - 1) * src_stride + T * d) * es);
  const Range rds = range_of(dsrc, ((n_src - 1) * dsrc_stride + T * d) * (acc ? 4 : es));
  const Range rdx = range_of(dx, T * d * es);
  const Range rw = range_of(w, d * 4);
  const Range rg = key_gain ? range_of(key_gain, d * 4) : Range{0, 0};
  const Range rgm = prenorm_gain ? range_of(prenorm_gain, d * 4) : Range{0, 0};
  const Range rws = range_of(workspace, ws_need);
  const Range odw = range_of(dw, d * 4);
  const Range odg = dkey_gain ? range_of(dkey_gain, d * 4) : Range{0, 0};
  const Range odm = (prenorm && dprenorm_gain) ? range_of(dprenorm_gain, d * 4) : Range{0, 0};
  const Range outs[] = {rds, odw, odg, odm, rws};
  for (Range o : outs)
    for (Range i : {rs, rdx, rw, rg, rgm})
      if (overlaps(o, i)) return ATTNRES_EALIAS;
  for (int a = 0; a < 5; ++a)
    for (int b = a + 1; b < 5; ++b)
      if (overlaps(outs[a], outs[b])) return ATTNRES_EALIAS;
  return hip_status(attnres::launch_site_backward(kind_of(dt), T, (int)d, src, (int)n_src, src_stride, w, key_gain,
                                                  prenorm ? prenorm_gain : nullptr, prenorm ? 1 : 0, eps, dx, dsrc,
                                                  dsrc_stride, acc ? 1 : 0, 0, dw, dkey_gain,
                                                  prenorm ? dprenorm_gain : nullptr, static_cast<float*>(workspace),
                                                  static_cast<hipStream_t>(stream)));
}

attnres_status_t attnres_site_backward(attnres_dtype_t dt, const void* src, int64_t n_src, int64_t src_stride,
                                       int64_t T, int64_t d, const float* w, const float* key_gain,
                                       const float* prenorm_gain, int prenorm, float eps, const void* dx,
                                       void* dsrc, int64_t dsrc_stride, float* dw, float* dkey_gain,
                                       float* dprenorm_gain, void* workspace, int64_t workspace_bytes,
                                       void* stream) {
  return site_backward_impl(dt, src, n_src, src_stride, T, d, w, key_gain, prenorm_gain, prenorm, eps, dx, dsrc,
                            dsrc_stride, false, dw, dkey_gain, dprenorm_gain, workspace, workspace_bytes, stream);
}

attnres_status_t attnres_site_backward_accumulate(attnres_dtype_t dt, const void* src, int64_t n_src,
                                                  int64_t src_stride, int64_t T, int64_t d, const float* w,
                                                  const float* key_gain, const float* prenorm_gain, int prenorm,
                                                  float eps, const void* dx, float* dsrc, int64_t dsrc_stride,
                                                  float* dw, float* dkey_gain, float* dprenorm_gain, void* workspace,
                                                  int64_t workspace_bytes, void* stream) {
  return site_backward_impl(dt, src, n_src, src_stride, T, d, w, key_gain, prenorm_gain, prenorm, eps, dx, dsrc,
                            dsrc_stride, true, dw, dkey_gain, dprenorm_gain, workspace, workspace_bytes, stream);
}

int64_t attnres_phase2_backward_workspace_bytes(int64_t T, int64_t d) {
  if (!extent_ok(T) || d <= 0 || d > ATTNRES_MAX_D || d % 8 != 0) return -1;
  if (T == 0) return 0;
  return attnres::p2_backward_slots(T, (int)d) * 2 * d * (int64_t)sizeof(float);
}

attnres_status_t attnres_phase2_backward(attnres_dtype_t dt, int64_t T, int64_t d, const void* p1_out,
                                         const float* p1_lse, attnres_dtype_t partial_dt, const void* partial_in,
                                         const void* sublayer_prev2, const void* sublayer_prev, const float* w,
                                         const float* key_gain, const float* prenorm_gain, int prenorm, float eps,
                                         const void* dx, float* dpartial, void* g_out, float* c_out, float* gp_out,
                                         float* dw, float* dkey_gain, float* dprenorm_gain, void* workspace,
                                         int64_t workspace_bytes, void* stream) {
  if (!dtype_ok(dt) || !partial_ok(partial_dt, dt)) return ATTNRES_EDTYPE;
  attnres_status_t st = check_d(d);
  if (st != ATTNRES_OK) return st;
  if (!extent_ok(T) || !(eps >= 0.f)) return ATTNRES_EINVAL;
  if (!sublayer_prev && (partial_in || sublayer_prev2)) return ATTNRES_EINVAL;
  if (T == 0) return ATTNRES_OK;  // empty token set: nothing is read or written
  if (!p1_out || !dx || !g_out || !c_out || !gp_out || !w) return ATTNRES_EINVAL;
  if (sublayer_prev && (!p1_lse || !dpartial)) return ATTNRES_EINVAL;
  const int64_t ws_need = attnres_phase2_backward_workspace_bytes(T, d);
  if (!workspace || workspace_bytes < ws_need) return ATTNRES_EINVAL;
  st = check_align({p1_out, partial_in, sublayer_prev2, sublayer_prev, w, key_gain, prenorm_gain, dx, dpartial, g_out,
                    workspace},
                   {p1_lse, c_out, gp_out, dw, dkey_gain, dprenorm_gain});
  if (st != ATTNRES_OK) return st;
  const int64_t es = esize(dt), rows = T * d;
  const Range i_o = range_of(p1_out, rows * es), i_l = p1_lse ? range_of(p1_lse, T * 4) : Range{0, 0};
  const Range i_p = partial_in ? range_of(partial_in, partial_bytes(partial_dt, T, d)) : Range{0, 0};
  const Range i_v2 = sublayer_prev2 ? range_of(sublayer_prev2, rows * es) : Range{0, 0};
  const Range i_v = sublayer_prev ? range_of(sublayer_prev, rows * es) : Range{0, 0};
  const Range i_w = range_of(w, d * 4), i_g = key_gain ? range_of(key_gain, d * 4) : Range{0, 0};
  const Range i_gm = prenorm_gain ? range_of(prenorm_gain, d * 4) : Range{0, 0};
  const Range i_dx = range_of(dx, rows * es);
  const Range o_dp = sublayer_prev ? range_of(dpartial, rows * 4) : Range{0, 0};
  const Range o_g = range_of(g_out, rows * es), o_c = range_of(c_out, T * 4), o_gp = range_of(gp_out, T * 4);
  const Range o_dw = (sublayer_prev && dw) ? range_of(dw, d * 4) : Range{0, 0};
  const Range o_dk = (sublayer_prev && dkey_gain) ? range_of(dkey_gain, d * 4) : Range{0, 0};
  const Range o_dm = (prenorm && dprenorm_gain) ? range_of(dprenorm_gain, d * 4) : Range{0, 0};
  const Range o_ws = range_of(workspace, ws_need);
  const Range outs[] = {o_dp, o_g, o_c, o_gp, o_dw, o_dk, o_dm, o_ws};
  for (Range o : outs)
    for (Range i : {i_o, i_l, i_p, i_v2, i_v, i_w, i_g, i_gm, i_dx})
      if (overlaps(o, i)) return ATTNRES_EALIAS;
  for (int a = 0; a < 8; ++a)
    for (int b = a + 1; b < 8; ++b)
      if (overlaps(outs[a], outs[b])) return ATTNRES_EALIAS;
  return hip_status(attnres::launch_p2_backward(
      kind_of(dt), T, (int)d, p1_out, p1_lse, kind_of(partial_dt), partial_in, sublayer_prev2, sublayer_prev, w,
      key_gain, prenorm ? prenorm_gain : nullptr, prenorm ? 1 : 0, eps, dx, dpartial, g_out, c_out, gp_out, dw,
      dkey_gain, prenorm ? dprenorm_gain : nullptr, static_cast<float*>(workspace),
      static_cast<hipStream_t>(stream)));
}

int64_t attnres_phase1_backward_workspace_bytes(int64_t T, int64_t d, int64_t n_src, int64_t S) {
  if (!extent_ok(T) || d <= 0 || d > ATTNRES_MAX_D || d % 8 != 0) return -1;
  // one site (S == 1) without c_in / gp_in runs on the site backward, which
  // takes up to ATTNRES_MAX_SOURCES sources and needs only its per-team sums
  if (S == 1 && n_src > ATTNRES_MAX_SOURCES_MULTI && n_src <= ATTNRES_MAX_SOURCES)
    return T == 0 ? 0 : attnres_site_backward_workspace_bytes(T, d);
  if (n_src < 1 || n_src > ATTNRES_MAX_SOURCES_MULTI || S < 1 || S > 32) return -1;
  if (T == 0) return 0;
  // coefficients [T][S rounded up to 8][n], folded queries [S][d],
  // per-range weight sums, the queries packed as matrix-core operands
  // (4096 bytes per 32 channels); one site (S == 1) may run on the site
  // backward, whose per-team sums need attnres_site_backward_workspace_bytes
  const int64_t sp = (S + 7) & ~(int64_t)7;
  const int64_t need = (T * sp * n_src + S * d + attnres::p1_backward_ranges((int)d) * S * d) * (int64_t)sizeof(float) +
                       ((d + 31) / 32) * 4096;
  const int64_t site = S == 1 ? attnres_site_backward_workspace_bytes(T, d) : 0;
  return need > site ? need : site;
}

attnres_status_t attnres_phase1_backward(attnres_dtype_t dt, attnres_dtype_t src_dt, const void* src,
                                         int64_t n_src, int64_t src_stride, int64_t T, int64_t d, const float* w,
                                         const float* key_gain, int64_t S, float eps, const void* g_in,
                                         int64_t g_stride, const float* c_in, const float* gp_in, float* dsrc,
                                         int64_t dsrc_stride, int accumulate, float* dw, float* dkey_gain,
                                         void* workspace, int64_t workspace_bytes, void* stream) {
  if (!dtype_ok(dt) || !dtype_ok(src_dt)) return ATTNRES_EDTYPE;
  // sources of G's type, or fp32 sources with bf16 G
  const bool mixed = src_dt != dt;
  if (mixed && !(src_dt == ATTNRES_F32 && dt == ATTNRES_BF16)) return ATTNRES_EDTYPE;
  attnres_status_t st = check_d(d);
  if (st != ATTNRES_OK) return st;
  // one site without c_in / gp_in (the final aggregation) with rows of one
  // type takes as many sources as the site backward it runs on
  const bool one_site = S == 1 && !c_in && !gp_in && !mixed;
  const int64_t max_src = one_site ? ATTNRES_MAX_SOURCES : ATTNRES_MAX_SOURCES_MULTI;
  if (!extent_ok(T, {src_stride, g_stride, dsrc_stride}) || n_src < 1 || n_src > max_src || S < 1 || S > 32 ||
      !(eps >= 0.f))
    return ATTNRES_EINVAL;
  if (gp_in == nullptr && c_in != nullptr) return ATTNRES_EINVAL;  // a partial weight needs its G.p
  if (T == 0) return ATTNRES_OK;  // empty token set: nothing is read or written
  if (!src || !w || !g_in || !dsrc || !dw) return ATTNRES_EINVAL;
  if ((n_src > 1 && (src_stride < T * d || dsrc_stride < T * d)) || (S > 1 && g_stride < T * d))
    return ATTNRES_EINVAL;
  if (src_stride % 8 != 0 || dsrc_stride % 8 != 0 || g_stride % 8 != 0) return ATTNRES_EALIGN;
  const int64_t ws_need = attnres_phase1_backward_workspace_bytes(T, d, n_src, S);
  if (!workspace || workspace_bytes < ws_need) return ATTNRES_EINVAL;
  st = check_align({src, w, key_gain, g_in, dsrc, workspace}, {c_in, gp_in, dw, dkey_gain});
  if (st != ATTNRES_OK) return st;
  const int64_t es = esize(dt);
  const Range i_s = range_of(src, ((n_src - 1) * src_stride + T * d) * esize(src_dt));
  const Range i_w = range_of(w, S * d * 4), i_k = key_gain ? range_of(key_gain, S * d * 4) : Range{0, 0};
  const Range i_g = range_of(g_in, ((S - 1) * g_stride + T * d) * es);
  const Range i_c = c_in ? range_of(c_in, S * T * 4) : Range{0, 0};
  const Range i_h = gp_in ? range_of(gp_in, S * T * 4) : Range{0, 0};
  const Range o_ds = range_of(dsrc, ((n_src - 1) * dsrc_stride + T * d) * 4);
  const Range o_dw = range_of(dw, S * d * 4), o_dk = dkey_gain ? range_of(dkey_gain, S * d * 4) : Range{0, 0};
  const Range o_ws = range_of(workspace, ws_need);
  const Range outs[] = {o_ds, o_dw, o_dk, o_ws};
  for (Range o : outs)
    for (Range i : {i_s, i_w, i_k, i_g, i_c, i_h})
      if (overlaps(o, i)) return ATTNRES_EALIAS;
  for (int a = 0; a < 4; ++a)
    for (int b = a + 1; b < 4; ++b)
      if (overlaps(outs[a], outs[b])) return ATTNRES_EALIAS;
  return hip_status(attnres::launch_p1_backward(kind_of(dt), kind_of(src_dt), T, (int)d, src, (int)n_src, src_stride,
                                                (int)S, w,
                                                key_gain, eps, g_in, g_stride, c_in, gp_in, dsrc, dsrc_stride,
                                                accumulate ? 1 : 0, dw, dkey_gain, static_cast<float*>(workspace),
                                                static_cast<hipStream_t>(stream)));
}

attnres_status_t attnres_full(attnres_dtype_t dt, const void* src, int64_t n_src, int64_t src_stride, int64_t T,
                              int64_t d, const float* w, const float* key_gain, const float* prenorm_gain,
                              float eps, void* h_out, void* x_out, float* lse_out, void* stream) {
  if (!dtype_ok(dt)) return ATTNRES_EDTYPE;
  attnres_status_t st = check_d(d);
  if (st != ATTNRES_OK) return st;
  if (!extent_ok(T, {src_stride}) || n_src < 1 || n_src > ATTNRES_MAX_SOURCES || !(eps >= 0.f))
    return ATTNRES_EINVAL;
  if (T == 0) return ATTNRES_OK;  // empty token set: nothing is read or written
  if (!src || !w || (!h_out && !x_out)) return ATTNRES_EINVAL;
  if (n_src > 1 && src_stride < T * d) return ATTNRES_EINVAL;
  if (src_stride % 8 != 0) return ATTNRES_EALIGN;
  st = check_align({src, w, key_gain, prenorm_gain, h_out, x_out}, {lse_out});
  if (st != ATTNRES_OK) return st;
  const int64_t es = esize(dt);
  const Range rs = range_of(src, ((n_src - 1) * src_stride + T * d) * es);
  const Range rh = h_out ? range_of(h_out, T * d * es) : Range{0, 0};
  const Range rx = x_out ? range_of(x_out, T * d * es) : Range{0, 0};
  const Range rl = lse_out ? range_of(lse_out, T * 4) : Range{0, 0};
  const Range rw = range_of(w, d * 4);
  const Range rg = key_gain ? range_of(key_gain, d * 4) : Range{0, 0};
  const Range rgm = prenorm_gain ? range_of(prenorm_gain, d * 4) : Range{0, 0};
  for (Range o : {rh, rx, rl})
    for (Range i : {rs, rw, rg, rgm})
      if (overlaps(o, i)) return ATTNRES_EALIAS;
  if (overlaps(rh, rx) || overlaps(rh, rl) || overlaps(rx, rl)) return ATTNRES_EALIAS;
  const Dtype kdt = kind_of(dt);
  return hip_status(attnres::launch_phase1_single(kdt, src, (int)n_src, src_stride, T, (int)d, w, key_gain,
                                                  prenorm_gain, eps, h_out, x_out, nullptr, lse_out,
                                                  static_cast<hipStream_t>(stream)));
}

attnres_status_t attnres_block_accumulate(attnres_dtype_t dt, int64_t T, int64_t d, attnres_dtype_t partial_dt,
                                          const void* partial_in, const void* v2, const void* v, void* out,
                                          attnres_dtype_t out_dt, void* stream) {
  if (!dtype_ok(dt) || !partial_ok(partial_dt, dt)) return ATTNRES_EDTYPE;
  if (out_dt != dt && !(out_dt == ATTNRES_F32 && dt == ATTNRES_BF16)) return ATTNRES_EDTYPE;
  attnres_status_t st = check_d(d);
  if (st != ATTNRES_OK) return st;
  if (!extent_ok(T)) return ATTNRES_EINVAL;
  if (T == 0) return ATTNRES_OK;  // empty token set: nothing is read or written
  if (!v || !out) return ATTNRES_EINVAL;
  st = check_align({partial_in, v2, v, out});
  if (st != ATTNRES_OK) return st;
  const int64_t rows = T * d;
  const Range ro = range_of(out, rows * esize(out_dt));
  const Range rv = range_of(v, rows * esize(dt));
  const Range rp = partial_in ? range_of(partial_in, partial_bytes(partial_dt, T, d)) : Range{0, 0};
  const Range rv2 = v2 ? range_of(v2, rows * esize(dt)) : Range{0, 0};
  if (overlaps(ro, rv) || overlaps(ro, rv2)) return ATTNRES_EALIAS;
  const bool in_place = partial_in == out && partial_dt == out_dt;
  if (!in_place && overlaps(ro, rp)) return ATTNRES_EALIAS;
  return hip_status(attnres::launch_accumulate(kind_of(dt), kind_of(out_dt), T, (int)d, kind_of(partial_dt),
                                               partial_in, v2, v, out, static_cast<hipStream_t>(stream)));
}

attnres_status_t attnres_stream_probe(int64_t n_read, int64_t n_write, const void* src, void* dst,
                                      int64_t stream_bytes, int64_t workgroups_per_cu, int64_t unroll,
                                      int64_t nontemporal, void* stream) {
  const bool many = (n_read == 8 && n_write == 0) || (n_read == 9 && n_write == 1) || (n_read == 7 && n_write == 24);
  if (!many && (n_read < 0 || n_read > 4 || n_write < 0 || n_write > 2 || n_read + n_write == 0))
    return ATTNRES_EINVAL;
  if (workgroups_per_cu < 1 || workgroups_per_cu > 16) return ATTNRES_EINVAL;
  if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) return ATTNRES_EINVAL;
  if (stream_bytes <= 0 || stream_bytes > (int64_t)1 << 40) return ATTNRES_EINVAL;
  if (stream_bytes % 16 != 0) return ATTNRES_EALIGN;
  if ((n_read > 0 && !src) || !dst) return ATTNRES_EINVAL;
  attnres_status_t st = check_align({src, dst});
  if (st != ATTNRES_OK) return st;
  const Range r = range_of(src, n_read * stream_bytes);
  const Range w = range_of(dst, (n_write > 0 ? n_write * stream_bytes : 16));
  if (n_read > 0 && overlaps(r, w)) return ATTNRES_EALIAS;
  return hip_status(attnres::launch_stream_probe((int)n_read, (int)n_write, src, dst, stream_bytes,
                                                 (int)workgroups_per_cu, (int)unroll, nontemporal != 0,
                                                 static_cast<hipStream_t>(stream)));
}

}  // extern "C"
