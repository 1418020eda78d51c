// C ABI of the token-level dynamic local-global attention forward: argument
// validation, target count, workspace sizing, dispatch to the HIP kernels,
// kernel timing. Every entry point is declared and documented in
// include/logo.h. No C++ exception leaves this file.
#include "../../include/logo.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <utility>
#include <vector>

#include "logo_internal.h"

namespace {

thread_local char g_last_error[512] = "";

logo_status fail(logo_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
logo_status fail(logo_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

logo_status hip_fail(hipError_t e, const char* what) {
  return fail(LOGO_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define LOGO_TRY(expr)                 \
  do {                                 \
    logo_status _s = (expr);           \
    if (_s != LOGO_OK) return _s;      \
  } while (0)

int64_t target_count(double rho, int64_t n) {
  if (std::isnan(rho) || n < 0) return -1;
  double k = std::ceil(rho * (double)n);
  if (k < 0) k = 0;
  if (k > (double)n) k = (double)n;
  return (int64_t)k;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Resolves and checks one tensor's (batch, head, token) strides.
logo_status check_view(const char* name, const int64_t st[3], int64_t B, int64_t H, int64_t n,
                       int64_t d, int64_t esize, bool output, logo::View* out) {
  int64_t sb = st[0], sh = st[1], stok = st[2];
  if (sb == 0 && sh == 0 && stok == 0) {
    stok = d;
    sh = n * d;
    sb = H * n * d;
  } else {
    if (sb < 0 || sh < 0 || stok < 0)
      return fail(LOGO_ERR_INVALID_ARG, "%s strides must be >= 0", name);
    if (stok < d)
      return fail(LOGO_ERR_INVALID_ARG, "%s token stride %lld is below d = %lld", name,
                  (long long)stok, (long long)d);
    if ((sb * esize) % 16 || (sh * esize) % 16 || (stok * esize) % 16)
      return fail(LOGO_ERR_INVALID_ARG, "%s strides must be multiples of 16 bytes", name);
    if (sb >= (int64_t(1) << 60) || sh >= (int64_t(1) << 60))
      return fail(LOGO_ERR_UNSUPPORTED, "%s strides beyond the supported range", name);
    if (output) {
      // Sufficient for distinct elements: sorted by stride, each dimension
      // steps over everything the smaller ones cover.
      std::pair<int64_t, int64_t> dims[4] = {{1, d}, {stok, n}, {sh, H}, {sb, B}};
      std::sort(dims, dims + 4);
      int64_t need = 1;
      for (const auto& dm : dims) {
        if (dm.second <= 1) continue;
        if (dm.first < need)
          return fail(LOGO_ERR_INVALID_ARG, "%s strides make output rows overlap", name);
        need = dm.first * dm.second;
      }
    }
  }
  if (n > 0 && ((n - 1) * stok + d) * esize >= (int64_t(1) << 31))
    return fail(LOGO_ERR_UNSUPPORTED, "%s: one sequence spans 2^31 bytes or more", name);
  out->sb = sb;
  out->sh = sh;
  out->st = (int)stok;
  return LOGO_OK;
}

// Validates the problem and fills the kernels' view of it.
logo_status check_problem(const logo_problem* p, logo::Dims* out) {
  if (!p) return fail(LOGO_ERR_INVALID_ARG, "problem is NULL");
  if (p->B < 0 || p->n < 0) return fail(LOGO_ERR_INVALID_ARG, "B and n must be >= 0");
  if (p->Hq < 1 || p->Hkv < 1) return fail(LOGO_ERR_INVALID_ARG, "Hq and Hkv must be >= 1");
  if (p->Hq % p->Hkv != 0)
    return fail(LOGO_ERR_INVALID_ARG, "Hq (%lld) must be a multiple of Hkv (%lld)",
                (long long)p->Hq, (long long)p->Hkv);
  if (p->window < 1) return fail(LOGO_ERR_INVALID_ARG, "window must be >= 1");
  if (std::isnan(p->rho) || p->rho < 0.0 || p->rho > 1.0)
    return fail(LOGO_ERR_INVALID_ARG, "rho must be in [0, 1]");
  if (!std::isfinite(p->scale) || p->scale < 0.0f)
    return fail(LOGO_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if (p->dtype != LOGO_F32 && p->dtype != LOGO_BF16)
    return fail(LOGO_ERR_INVALID_ARG, "dtype must be LOGO_F32 or LOGO_BF16");
  if (p->d != 64 && p->d != 128)
    return fail(LOGO_ERR_UNSUPPORTED, "head dimension %lld not supported (64 or 128)",
                (long long)p->d);
  if (p->n >= (int64_t(1) << 30) || p->Hq >= (int64_t(1) << 20) || p->B >= (int64_t(1) << 20))
    return fail(LOGO_ERR_UNSUPPORTED, "sizes beyond the supported range");
  const double elems = (double)p->B * (double)p->Hq * (double)p->n * (double)p->d;
  if (elems >= 4.0e18) return fail(LOGO_ERR_UNSUPPORTED, "problem too large");
  out->B = (int)p->B;
  out->Hq = (int)p->Hq;
  out->Hkv = (int)p->Hkv;
  out->n = (int)p->n;
  out->d = (int)p->d;
  out->window = (int)std::min<int64_t>(p->window, int64_t(1) << 30);
  out->k = (int)target_count(p->rho, p->n);
  out->scale = p->scale == 0.0f ? (float)(1.0 / std::sqrt((double)p->d)) : p->scale;
  out->dtype = p->dtype;
  const int64_t es = p->dtype == LOGO_BF16 ? 2 : 4;
  LOGO_TRY(check_view("q", p->q_strides, p->B, p->Hq, p->n, p->d, es, false, &out->vq));
  LOGO_TRY(check_view("k", p->k_strides, p->B, p->Hkv, p->n, p->d, es, false, &out->vk));
  LOGO_TRY(check_view("v", p->v_strides, p->B, p->Hkv, p->n, p->d, es, false, &out->vv));
  LOGO_TRY(check_view("o", p->o_strides, p->B, p->Hq, p->n, p->d, es, true, &out->vo));
  return LOGO_OK;
}

bool empty(const logo::Dims& d) { return d.B == 0 || d.n == 0; }

logo_status need_ptr(const void* ptr, const char* name) {
  if (!ptr) return fail(LOGO_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(ptr)) return fail(LOGO_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return LOGO_OK;
}


// The global branch's workgroup queues (one int per (b, kv head)).
size_t queue_bytes(const logo::Dims& d) {  // none when nothing is selected
  return d.k == 0 ? 0 : (logo::attn_bf16_sched_ints(d, false) * sizeof(int32_t) + 255) / 256 * 256;
}
// logo_forward's workspace: the float32 local outputs of the selected rows,
// then the queues.
size_t scratch_only_bytes(const logo::Dims& d) {
  const size_t b = (size_t)d.B * d.Hq * d.k * d.d * sizeof(float);
  return (b + 255) / 256 * 256;
}
// and, for a bf16 problem small enough that the global branch splits its
// key ranges, the partials of the split
size_t split_bytes(const logo::Dims& d) {
  if (d.dtype != LOGO_BF16) return 0;
  return (logo::attn_bf16_split_floats(d) * sizeof(float) + 255) / 256 * 256;
}
// and, where the single-launch fused forward applies, the unselected
// positions of each sequence (the rows its local-only work gathers)
size_t nidx_bytes(const logo::Dims& d) {
  if (!logo::attn_bf16_fused_ok(d)) return 0;
  return ((size_t)d.B * (d.n - d.k) * sizeof(int32_t) + 255) / 256 * 256;
}
size_t scratch_bytes(const logo::Dims& d) {
  return scratch_only_bytes(d) + queue_bytes(d) + split_bytes(d) + nidx_bytes(d);
}

// ---- kernel timing --------------------------------------------------------
struct Profiler {
  std::mutex mu;
  bool on = false;
  struct Rec {
    hipEvent_t a, b;
    int stage;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
};
Profiler g_prof;
constexpr size_t kMaxRecords = 4096;

// Records the start event of a stage; returns the record slot or -1.
long prof_start(int stage, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (!g_prof.on || g_prof.recs.size() >= kMaxRecords) return -1;
  while (g_prof.pool.size() < 2 * (g_prof.recs.size() + 1)) {
    // Timing only: no system-scope fence when the event completes, so
    // recording one writes back and invalidates no cache (the kernel after
    // it would otherwise start on a cold L2). Nothing reads results through
    // these events; callers synchronise the stream themselves.
    hipEvent_t e;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return -1;
    g_prof.pool.push_back(e);
  }
  Profiler::Rec r{g_prof.pool[2 * g_prof.recs.size()], g_prof.pool[2 * g_prof.recs.size() + 1],
                  stage};
  if (hipEventRecord(r.a, s) != hipSuccess) return -1;
  g_prof.recs.push_back(r);
  return (long)g_prof.recs.size() - 1;
}

void prof_stop(long slot, hipStream_t s) {
  if (slot < 0) return;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (slot < (long)g_prof.recs.size()) (void)hipEventRecord(g_prof.recs[slot].b, s);
}

struct StageTimer {
  long slot;
  hipStream_t s;
  StageTimer(int stage, hipStream_t st) : slot(prof_start(stage, st)), s(st) {}
  ~StageTimer() { prof_stop(slot, s); }
};

hipError_t run_attn(const logo::Dims& d, logo::Epi epi, const logo::AttnArgs& a,
                    hipStream_t s) {
  return d.dtype == LOGO_BF16 ? logo::launch_attn_bf16(d, epi, a, s)
                              : logo::launch_attn_f32(d, epi, a, s);
}

}  // namespace

extern "C" {

int64_t logo_target_count(double rho, int64_t n) { return target_count(rho, n); }

const char* logo_status_string(logo_status s) {
  switch (s) {
    case LOGO_OK: return "ok";
    case LOGO_ERR_INVALID_ARG: return "invalid argument";
    case LOGO_ERR_UNSUPPORTED: return "unsupported problem";
    case LOGO_ERR_WORKSPACE: return "workspace missing or too small";
    case LOGO_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* logo_last_error(void) { return g_last_error; }

logo_status logo_workspace_size(const logo_problem* p, size_t* bytes) {
  logo::Dims d;
  LOGO_TRY(check_problem(p, &d));
  if (!bytes) return fail(LOGO_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = empty(d) ? 0 : scratch_bytes(d);
  return LOGO_OK;
}

logo_status logo_select_queries(const logo_problem* p, const float* gate, uint8_t* mask,
                                int32_t* idx, int32_t* rank, void* stream) {
  logo::Dims d;
  LOGO_TRY(check_problem(p, &d));
  if (empty(d)) return LOGO_OK;
  LOGO_TRY(need_ptr(gate, "gate"));
  LOGO_TRY(need_ptr(mask, "mask"));
  LOGO_TRY(need_ptr(rank, "rank"));
  if (d.k > 0) LOGO_TRY(need_ptr(idx, "idx"));
  hipStream_t s = static_cast<hipStream_t>(stream);
  StageTimer tm(0, s);
  hipError_t e = logo::launch_select(d, gate, mask, d.k > 0 ? idx : nullptr, rank, s);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  return LOGO_OK;
}

logo_status logo_local_attn(const logo_problem* p, const void* q, const void* k,
                            const void* v, float* o_local, void* stream) {
  logo::Dims d;
  LOGO_TRY(check_problem(p, &d));
  if (empty(d)) return LOGO_OK;
  LOGO_TRY(need_ptr(q, "q"));
  LOGO_TRY(need_ptr(k, "k"));
  LOGO_TRY(need_ptr(v, "v"));
  LOGO_TRY(need_ptr(o_local, "o_local"));
  logo::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out_f32 = o_local;
  hipStream_t s = static_cast<hipStream_t>(stream);
  StageTimer tm(1, s);
  hipError_t e = run_attn(d, logo::Epi::LocalAll, a, s);
  if (e != hipSuccess) return hip_fail(e, "local attention launch");
  return LOGO_OK;
}

logo_status logo_global_attn_sparse(const logo_problem* p, const void* q, const void* k,
                                    const void* v, const int32_t* idx, float* o_global,
                                    void* stream) {
  logo::Dims d;
  LOGO_TRY(check_problem(p, &d));
  if (empty(d) || d.k == 0) return LOGO_OK;
  LOGO_TRY(need_ptr(q, "q"));
  LOGO_TRY(need_ptr(k, "k"));
  LOGO_TRY(need_ptr(v, "v"));
  LOGO_TRY(need_ptr(idx, "idx"));
  LOGO_TRY(need_ptr(o_global, "o_global"));
  logo::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.idx = idx;
  a.out_f32 = o_global;
  hipStream_t s = static_cast<hipStream_t>(stream);
  StageTimer tm(2, s);
  hipError_t e = run_attn(d, logo::Epi::GlobalAll, a, s);
  if (e != hipSuccess) return hip_fail(e, "global attention launch");
  return LOGO_OK;
}

logo_status logo_combine(const logo_problem* p, const float* o_local, const float* o_global,
                         const int32_t* rank, const float* gate, void* o, void* stream) {
  logo::Dims d;
  LOGO_TRY(check_problem(p, &d));
  if (empty(d)) return LOGO_OK;
  LOGO_TRY(need_ptr(o_local, "o_local"));
  LOGO_TRY(need_ptr(rank, "rank"));
  LOGO_TRY(need_ptr(gate, "gate"));
  LOGO_TRY(need_ptr(o, "o"));
  if (d.k > 0) LOGO_TRY(need_ptr(o_global, "o_global"));
  hipStream_t s = static_cast<hipStream_t>(stream);
  StageTimer tm(3, s);
  hipError_t e = logo::launch_combine(d, o_local, o_global, rank, gate, o, s);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return LOGO_OK;
}

logo_status logo_forward(const logo_problem* p, const void* q, const void* k, const void* v,
                         const float* gate, void* o, uint8_t* mask, int32_t* idx,
                         int32_t* rank, void* workspace, size_t workspace_bytes,
                         void* stream) {
  logo::Dims d;
  LOGO_TRY(check_problem(p, &d));
  if (empty(d)) return LOGO_OK;
  LOGO_TRY(need_ptr(q, "q"));
  LOGO_TRY(need_ptr(k, "k"));
  LOGO_TRY(need_ptr(v, "v"));
  LOGO_TRY(need_ptr(gate, "gate"));
  LOGO_TRY(need_ptr(o, "o"));
  LOGO_TRY(need_ptr(mask, "mask"));
  LOGO_TRY(need_ptr(rank, "rank"));
  const size_t ws_need = scratch_bytes(d);
  if (d.k > 0) {
    LOGO_TRY(need_ptr(idx, "idx"));
    if (!workspace || workspace_bytes < ws_need)
      return fail(LOGO_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", ws_need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(LOGO_ERR_INVALID_ARG, "workspace misaligned");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  // bf16 problems with enough work and a (b, kv head) count that maps onto
  // the XCDs: selection (also listing the unselected positions), then one
  // launch for every row (selected rows compute both branches)
  const bool fused = logo::attn_bf16_fused_ok(d);
  int32_t* nidx = fused ? reinterpret_cast<int32_t*>(
                              static_cast<char*>(workspace) + scratch_only_bytes(d) +
                              queue_bytes(d) + split_bytes(d))
                        : nullptr;
  {
    StageTimer tm(0, s);
    e = logo::launch_select(d, gate, mask, d.k > 0 ? idx : nullptr, rank, s, nidx);
  }
  if (e != hipSuccess) return hip_fail(e, "select launch");
  logo::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.idx = idx;
  a.rank = rank;
  a.gate = gate;
  a.out_f32 = static_cast<float*>(workspace);
  a.scratch = static_cast<const float*>(workspace);
  a.out_io = o;
  if (fused) {
    StageTimer tm(9, s);
    e = logo::launch_attn_bf16_fused(d, a, nidx, s);
    if (e != hipSuccess) return hip_fail(e, "fused attention launch");
    return LOGO_OK;
  }
  if (d.k > 0 && d.dtype == LOGO_BF16) {
    a.sched = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + scratch_only_bytes(d));
    if (split_bytes(d) > 0)
      a.split_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                              scratch_only_bytes(d) + queue_bytes(d));
  }
  if (a.split_part && logo::attn_bf16_pair_ok(d)) {
    // split global branch and local band in one launch, then the merge
    StageTimer tm(10, s);
    e = logo::launch_attn_bf16_pair(d, a, s);
    if (e != hipSuccess) return hip_fail(e, "paired attention launch");
    return LOGO_OK;
  }
  {
    StageTimer tm(1, s);
    e = run_attn(d, logo::Epi::LocalFused, a, s);
  }
  if (e != hipSuccess) return hip_fail(e, "local attention launch");
  if (d.k > 0) {
    StageTimer tm(2, s);
    e = run_attn(d, logo::Epi::GlobalFused, a, s);
    if (e != hipSuccess) return hip_fail(e, "global attention launch");
  }
  return LOGO_OK;
}

}  // extern "C"

// ---- the forward without allocation ------------------------------------
// logo_forward_noalloc runs logo_forward on a file-scope device array
// instead of a caller's workspace. In host code `scratch` names a host-side
// stand-in, not device memory: its device address on the current device
// comes from hipGetSymbolAddress, looked up once per device and kept in
// g_scratch_ptr; only that address is ever passed to kernels.
namespace {

__device__ __align__(256) unsigned char scratch[LOGO_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

logo_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(LOGO_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(LOGO_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LOGO_OK;
}

}  // namespace

extern "C" {

logo_status logo_forward_noalloc(const logo_problem* p, const void* q, const void* k,
                                 const void* v, const float* gate, void* o, uint8_t* mask,
                                 int32_t* idx, int32_t* rank, void* stream) {
  logo::Dims d;
  LOGO_TRY(check_problem(p, &d));
  if (empty(d)) return LOGO_OK;
  const size_t need = scratch_bytes(d);
  if (need > (size_t)LOGO_NOALLOC_SCRATCH_BYTES)
    return fail(LOGO_ERR_WORKSPACE,
                "this problem needs %zu bytes of scratch; logo_forward_noalloc holds %zu "
                "(use logo_forward with a workspace)",
                need, (size_t)LOGO_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0) LOGO_TRY(scratch_address(&ws));
  return logo_forward(p, q, k, v, gate, o, mask, idx, rank, ws, need, stream);
}

logo_status logo_forward_train(const logo_problem* p, const void* q, const void* k,
                               const void* v, const float* gate, void* o, uint8_t* mask,
                               int32_t* idx, int32_t* rank, float* lse_local, float* lse_global,
                               float* o_local_sel, float* o_global, void* stream) {
  logo::Dims d;
  LOGO_TRY(check_problem(p, &d));
  if (empty(d)) return LOGO_OK;
  LOGO_TRY(need_ptr(q, "q"));
  LOGO_TRY(need_ptr(k, "k"));
  LOGO_TRY(need_ptr(v, "v"));
  LOGO_TRY(need_ptr(gate, "gate"));
  LOGO_TRY(need_ptr(o, "o"));
  LOGO_TRY(need_ptr(mask, "mask"));
  LOGO_TRY(need_ptr(rank, "rank"));
  LOGO_TRY(need_ptr(lse_local, "lse_local"));
  if (d.k > 0) {
    LOGO_TRY(need_ptr(idx, "idx"));
    LOGO_TRY(need_ptr(lse_global, "lse_global"));
    LOGO_TRY(need_ptr(o_local_sel, "o_local_sel"));
    LOGO_TRY(need_ptr(o_global, "o_global"));
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  {
    StageTimer tm(0, s);
    e = logo::launch_select(d, gate, mask, d.k > 0 ? idx : nullptr, rank, s);
  }
  if (e != hipSuccess) return hip_fail(e, "select launch");
  logo::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.idx = idx;
  a.rank = rank;
  a.gate = gate;
  a.out_f32 = o_local_sel;
  a.scratch = o_local_sel;
  a.out_io = o;
  a.lse_out = lse_local;
  {
    StageTimer tm(1, s);
    e = run_attn(d, logo::Epi::LocalFused, a, s);
  }
  if (e != hipSuccess) return hip_fail(e, "local attention launch");
  if (d.k > 0) {
    a.lse_out = lse_global;
    a.og_out = o_global;
    StageTimer tm(2, s);
    e = run_attn(d, logo::Epi::GlobalFused, a, s);
    if (e != hipSuccess) return hip_fail(e, "global attention launch");
  }
  return LOGO_OK;
}

logo_status logo_backward_workspace_size(const logo_problem* p, size_t* bytes) {
  logo::Dims d;
  LOGO_TRY(check_problem(p, &d));
  if (!bytes) return fail(LOGO_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = empty(d) ? 0 : logo::bwd_workspace(d).total;
  return LOGO_OK;
}

logo_status logo_backward(const logo_problem* p, const void* q, const void* k, const void* v,
                          const float* gate, const void* o, const void* dout,
                          const int32_t* idx, const int32_t* rank, const float* lse_local,
                          const float* lse_global, const float* o_local_sel,
                          const float* o_global, float* dq, float* dk, float* dv, float* dgate,
                          void* workspace, size_t workspace_bytes, void* stream) {
  logo::Dims d;
  LOGO_TRY(check_problem(p, &d));
  if (empty(d)) return LOGO_OK;
  LOGO_TRY(need_ptr(q, "q"));
  LOGO_TRY(need_ptr(k, "k"));
  LOGO_TRY(need_ptr(v, "v"));
  LOGO_TRY(need_ptr(gate, "gate"));
  LOGO_TRY(need_ptr(o, "o"));
  LOGO_TRY(need_ptr(dout, "dout"));
  LOGO_TRY(need_ptr(rank, "rank"));
  LOGO_TRY(need_ptr(lse_local, "lse_local"));
  LOGO_TRY(need_ptr(dq, "dq"));
  LOGO_TRY(need_ptr(dk, "dk"));
  LOGO_TRY(need_ptr(dv, "dv"));
  LOGO_TRY(need_ptr(dgate, "dgate"));
  if (d.k > 0) {
    LOGO_TRY(need_ptr(idx, "idx"));
    LOGO_TRY(need_ptr(lse_global, "lse_global"));
    LOGO_TRY(need_ptr(o_local_sel, "o_local_sel"));
    LOGO_TRY(need_ptr(o_global, "o_global"));
  }
  const logo::BwdWorkspace ws = logo::bwd_workspace(d);
  if (!workspace || workspace_bytes < ws.total)
    return fail(LOGO_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", ws.total,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(LOGO_ERR_INVALID_ARG, "workspace misaligned");
  char* w = static_cast<char*>(workspace);
  logo::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.gate = gate;
  a.o = o;
  a.dout = dout;
  a.idx = idx;
  a.rank = rank;
  a.lse_l = lse_local;
  a.lse_g = lse_global;
  a.o_ls = o_local_sel;
  a.o_g = o_global;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dgate = dgate;
  a.D_l = reinterpret_cast<float*>(w + ws.D_l);
  a.D_g = reinterpret_cast<float*>(w + ws.D_g);
  a.L2_l = reinterpret_cast<float*>(w + ws.L2_l);
  a.L2_g = reinterpret_cast<float*>(w + ws.L2_g);
  a.qs = w + ws.qs;
  a.dog = w + ws.dog;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = d.dtype == LOGO_BF16;
  hipError_t e;
  {
    StageTimer tm(4, s);
    e = logo::launch_bwd_prep(d, a, s);
  }
  if (e != hipSuccess) return hip_fail(e, "backward prep launch");
  {
    StageTimer tm(5, s);
    e = bf ? logo::launch_bwd_dkdv_bf16(d, a, s) : logo::launch_bwd_dkdv_f32(d, a, s);
  }
  if (e != hipSuccess) return hip_fail(e, "backward dk/dv launch");
  {
    StageTimer tm(6, s);
    e = bf ? logo::launch_bwd_dq_bf16(d, false, a, s) : logo::launch_bwd_dq_f32(d, false, a, s);
    if (e == hipSuccess && d.k > 0)
      e = bf ? logo::launch_bwd_dq_bf16(d, true, a, s) : logo::launch_bwd_dq_f32(d, true, a, s);
  }
  if (e != hipSuccess) return hip_fail(e, "backward dq launch");
  return LOGO_OK;
}

// Routed forward workspace: float32 local outputs of every row, then the
// per-head router partials.
size_t routed_local_bytes(const logo::Dims& d) {
  return ((size_t)d.B * d.Hq * d.n * d.d * sizeof(float) + 255) / 256 * 256;
}
size_t routed_part_bytes(const logo::Dims& d) {
  return ((size_t)d.B * d.Hq * d.n * sizeof(float) + 255) / 256 * 256;
}
size_t routed_bytes(const logo::Dims& d) {
  return routed_local_bytes(d) + routed_part_bytes(d) + queue_bytes(d);
}

logo_status logo_routed_workspace_size(const logo_problem* p, size_t* bytes) {
  logo::Dims d;
  LOGO_TRY(check_problem(p, &d));
  if (!bytes) return fail(LOGO_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = empty(d) ? 0 : routed_bytes(d);
  return LOGO_OK;
}

logo_status logo_forward_routed(const logo_problem* p, const void* q, const void* k,
                                const void* v, const float* router_w, float router_bias,
                                float* gate, void* o, uint8_t* mask, int32_t* idx,
                                int32_t* rank, void* workspace, size_t workspace_bytes,
                                void* stream) {
  logo::Dims d;
  LOGO_TRY(check_problem(p, &d));
  if (empty(d)) return LOGO_OK;
  if (!std::isfinite(router_bias))
    return fail(LOGO_ERR_INVALID_ARG, "router_bias must be finite");
  LOGO_TRY(need_ptr(q, "q"));
  LOGO_TRY(need_ptr(k, "k"));
  LOGO_TRY(need_ptr(v, "v"));
  LOGO_TRY(need_ptr(router_w, "router_w"));
  LOGO_TRY(need_ptr(gate, "gate"));
  LOGO_TRY(need_ptr(o, "o"));
  LOGO_TRY(need_ptr(mask, "mask"));
  LOGO_TRY(need_ptr(rank, "rank"));
  if (d.k > 0) LOGO_TRY(need_ptr(idx, "idx"));
  const size_t need = routed_bytes(d);
  if (!workspace || workspace_bytes < need)
    return fail(LOGO_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(LOGO_ERR_INVALID_ARG, "workspace misaligned");
  float* o_local = static_cast<float*>(workspace);
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + routed_local_bytes(d));
  hipStream_t s = static_cast<hipStream_t>(stream);
  logo::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.idx = idx;
  a.rank = rank;
  a.gate = gate;
  a.out_f32 = o_local;
  a.scratch = o_local;
  a.out_io = o;
  a.router_w = router_w;
  a.router_part = part;
  if (d.dtype == LOGO_BF16)
    a.sched = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + routed_local_bytes(d) +
                                         routed_part_bytes(d));
  hipError_t e;
  {
    StageTimer tm(1, s);
    e = run_attn(d, logo::Epi::LocalRouted, a, s);
  }
  if (e != hipSuccess) return hip_fail(e, "local attention launch");
  {
    StageTimer tm(7, s);
    e = logo::launch_router_sum(d, part, router_bias, gate, s);
  }
  if (e != hipSuccess) return hip_fail(e, "router launch");
  {
    StageTimer tm(0, s);
    e = logo::launch_select(d, gate, mask, d.k > 0 ? idx : nullptr, rank, s);
  }
  if (e != hipSuccess) return hip_fail(e, "select launch");
  if (d.k > 0) {
    StageTimer tm(2, s);
    e = run_attn(d, logo::Epi::GlobalRouted, a, s);
    if (e != hipSuccess) return hip_fail(e, "global attention launch");
  }
  return LOGO_OK;
}

logo_status check_decode(const logo_decode_problem* p, logo::DecodeDims* out) {
  if (!p) return fail(LOGO_ERR_INVALID_ARG, "problem is NULL");
  if (p->B < 0) return fail(LOGO_ERR_INVALID_ARG, "B must be >= 0");
  if (p->Hq < 1 || p->Hkv < 1 || p->Hq % p->Hkv != 0)
    return fail(LOGO_ERR_INVALID_ARG, "Hq must be a positive multiple of Hkv");
  if (p->cap < 1) return fail(LOGO_ERR_INVALID_ARG, "cache capacity must be >= 1");
  if (p->window < 1) return fail(LOGO_ERR_INVALID_ARG, "window must be >= 1");
  if (std::isnan(p->rho) || p->rho < 0.0 || p->rho > 1.0)
    return fail(LOGO_ERR_INVALID_ARG, "rho must be in [0, 1]");
  if (!std::isfinite(p->eta) || p->eta < 0.0f)
    return fail(LOGO_ERR_INVALID_ARG, "eta must be finite and >= 0");
  if (!std::isfinite(p->scale) || p->scale < 0.0f)
    return fail(LOGO_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if (p->dtype != LOGO_F32 && p->dtype != LOGO_BF16)
    return fail(LOGO_ERR_INVALID_ARG, "dtype must be LOGO_F32 or LOGO_BF16");
  if (p->d != 64 && p->d != 128)
    return fail(LOGO_ERR_UNSUPPORTED, "head dimension %lld not supported (64 or 128)",
                (long long)p->d);
  if (p->cap >= (int64_t(1) << 30) || p->B >= (int64_t(1) << 20) || p->Hq >= (int64_t(1) << 16))
    return fail(LOGO_ERR_UNSUPPORTED, "sizes beyond the supported range");
  // work items (b, branch, kv head, chunk) are counted in 32-bit integers
  if (2 * p->B * p->Hkv * logo::decode_chunks(p->cap) >= (int64_t(1) << 30))
    return fail(LOGO_ERR_UNSUPPORTED, "B * Hkv * cache chunks beyond the supported range");
  out->B = (int)p->B;
  out->Hq = (int)p->Hq;
  out->Hkv = (int)p->Hkv;
  out->cap = (int)p->cap;
  out->d = (int)p->d;
  out->window = (int)std::min<int64_t>(p->window, int64_t(1) << 30);
  out->rho = p->rho;
  out->eta = p->eta;
  out->scale = p->scale == 0.0f ? (float)(1.0 / std::sqrt((double)p->d)) : p->scale;
  out->dtype = p->dtype;
  if (!logo::decode_group_supported(*out))
    return fail(LOGO_ERR_UNSUPPORTED,
                "query heads per kv head %lld not supported (up to 16 for bf16 caches of at most "
                "1023 sequences; otherwise 1, 2, 4, 7 or 8)",
                (long long)(p->Hq / p->Hkv));
  return LOGO_OK;
}

logo_status logo_decode_workspace_size(const logo_decode_problem* p, size_t* bytes) {
  logo::DecodeDims d;
  LOGO_TRY(check_decode(p, &d));
  if (!bytes) return fail(LOGO_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = d.B == 0 ? 0 : logo::decode_partial_bytes(d);
  return LOGO_OK;
}

logo_status logo_decode_step(const logo_decode_problem* p, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* lens, const float* gate,
                             float* tau, void* o, uint8_t* selected, void* workspace,
                             size_t workspace_bytes, void* stream) {
  logo::DecodeDims d;
  LOGO_TRY(check_decode(p, &d));
  if (d.B == 0) return LOGO_OK;
  LOGO_TRY(need_ptr(q, "q"));
  LOGO_TRY(need_ptr(k_cache, "k_cache"));
  LOGO_TRY(need_ptr(v_cache, "v_cache"));
  LOGO_TRY(need_ptr(lens, "lens"));
  LOGO_TRY(need_ptr(gate, "gate"));
  LOGO_TRY(need_ptr(tau, "tau"));
  LOGO_TRY(need_ptr(o, "o"));
  LOGO_TRY(need_ptr(selected, "selected"));
  const size_t need = logo::decode_partial_bytes(d);
  if (!workspace || workspace_bytes < need)
    return fail(LOGO_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(LOGO_ERR_INVALID_ARG, "workspace misaligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = logo::launch_decode_ctrl(d, gate, tau, selected, s);
  if (e != hipSuccess) return hip_fail(e, "controller launch");
  logo::DecodeArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.lens = lens;
  a.gate = gate;
  a.selected = selected;
  a.part = static_cast<float*>(workspace);
  a.o = o;
  {
    StageTimer tm(8, s);
    e = logo::launch_decode(d, a, s);
  }
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return LOGO_OK;
}

logo_status logo_calibrate_threshold(const logo_problem* p, const float* gate,
                                     const uint8_t* mask, float* tau, void* stream) {
  logo::Dims d;
  LOGO_TRY(check_problem(p, &d));
  if (d.B == 0) return LOGO_OK;
  LOGO_TRY(need_ptr(gate, "gate"));
  LOGO_TRY(need_ptr(mask, "mask"));
  LOGO_TRY(need_ptr(tau, "tau"));
  if (d.n == 0) return fail(LOGO_ERR_INVALID_ARG, "n must be >= 1 to calibrate");
  hipError_t e = logo::launch_calibrate(d, gate, mask, tau, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "calibrate launch");
  return LOGO_OK;
}

logo_status logo_select_threshold(const logo_problem* p, const float* gate, const float* tau,
                                  uint8_t* mask, int32_t* idx, int32_t* count, void* stream) {
  logo::Dims d;
  LOGO_TRY(check_problem(p, &d));
  if (empty(d)) return LOGO_OK;
  LOGO_TRY(need_ptr(gate, "gate"));
  LOGO_TRY(need_ptr(tau, "tau"));
  LOGO_TRY(need_ptr(mask, "mask"));
  LOGO_TRY(need_ptr(idx, "idx"));
  LOGO_TRY(need_ptr(count, "count"));
  hipError_t e = logo::launch_select_threshold(d, gate, tau, mask, idx, count,
                                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "threshold select launch");
  return LOGO_OK;
}

// Packed examples: the per-example table, per-token example starts, the
// float32 local outputs of the selected rows and the global branch's
// workgroup order.
struct VarlenWs {
  size_t seg, seg_start, scratch, sched, nidx, total;
  bool fused;   // the single launch runs the stream (nidx: its unselected positions)
};
VarlenWs varlen_ws(const logo::Dims& d, int64_t E, int64_t K) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  VarlenWs w;
  w.seg = 0;
  w.seg_start = up((size_t)E * 16);
  w.scratch = w.seg_start + up((size_t)d.n * 4);
  w.sched = w.scratch + up((size_t)d.Hq * (size_t)K * d.d * sizeof(float));
  logo::Dims dk = d;
  dk.k = (int)K;
  w.nidx = w.sched + up(logo::attn_bf16_sched_ints(dk, true) * sizeof(int32_t));
  w.fused = logo::attn_bf16_fused_ok(dk);
  w.total = w.nidx + (w.fused ? up((size_t)(d.n - K) * sizeof(int32_t)) : 0);
  return w;
}

logo_status check_varlen(const logo_problem* p, int64_t E, int64_t K, logo::Dims* d) {
  LOGO_TRY(check_problem(p, d));
  if (p->B != 1)
    return fail(LOGO_ERR_INVALID_ARG, "packed batches are one token stream: B must be 1");
  if (E < 1 || E > (int64_t(1) << 30))
    return fail(LOGO_ERR_INVALID_ARG, "n_examples must be >= 1");
  if (K < 0 || K > p->n)
    return fail(LOGO_ERR_INVALID_ARG, "total_selected must be in [0, n]");
  d->k = (int)K;
  return LOGO_OK;
}

int64_t logo_varlen_selected_count(double rho, const int32_t* cu, int64_t E) {
  if (std::isnan(rho) || rho < 0.0 || rho > 1.0 || !cu || E < 1) return -1;
  if (cu[0] != 0) return -1;
  int64_t K = 0;
  for (int64_t e = 0; e < E; ++e) {
    if (cu[e + 1] < cu[e]) return -1;
    K += target_count(rho, (int64_t)cu[e + 1] - cu[e]);
  }
  return K;
}

logo_status logo_varlen_workspace_size(const logo_problem* p, int64_t n_examples,
                                       int64_t total_selected, size_t* bytes) {
  logo::Dims d;
  LOGO_TRY(check_varlen(p, n_examples, total_selected, &d));
  if (!bytes) return fail(LOGO_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = d.n == 0 ? 0 : varlen_ws(d, n_examples, total_selected).total;
  return LOGO_OK;
}

logo_status logo_forward_varlen(const logo_problem* p, const int32_t* cu_seqlens,
                                int64_t n_examples, int64_t total_selected, const void* q,
                                const void* k, const void* v, const float* gate, void* o,
                                uint8_t* mask, int32_t* idx, int32_t* rank, void* workspace,
                                size_t workspace_bytes, void* stream) {
  logo::Dims d;
  LOGO_TRY(check_varlen(p, n_examples, total_selected, &d));
  if (d.n == 0) return LOGO_OK;
  LOGO_TRY(need_ptr(cu_seqlens, "cu_seqlens"));
  LOGO_TRY(need_ptr(q, "q"));
  LOGO_TRY(need_ptr(k, "k"));
  LOGO_TRY(need_ptr(v, "v"));
  LOGO_TRY(need_ptr(gate, "gate"));
  LOGO_TRY(need_ptr(o, "o"));
  LOGO_TRY(need_ptr(mask, "mask"));
  LOGO_TRY(need_ptr(rank, "rank"));
  if (d.k > 0) LOGO_TRY(need_ptr(idx, "idx"));
  const VarlenWs ws = varlen_ws(d, n_examples, total_selected);
  if (!workspace || workspace_bytes < ws.total)
    return fail(LOGO_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", ws.total,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(LOGO_ERR_INVALID_ARG, "workspace misaligned");
  char* w = static_cast<char*>(workspace);
  int4* seg = reinterpret_cast<int4*>(w + ws.seg);
  int32_t* seg_start = reinterpret_cast<int32_t*>(w + ws.seg_start);
  float* scratch = reinterpret_cast<float*>(w + ws.scratch);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  // bf16 streams with enough selected rows: the selection also lists the
  // unselected positions, then one launch computes every row (as logo_forward)
  int32_t* nidx = ws.fused ? reinterpret_cast<int32_t*>(w + ws.nidx) : nullptr;
  {
    StageTimer tm(0, s);
    e = logo::launch_varlen_prep(cu_seqlens, (int)n_examples, d.n, p->rho, seg, seg_start, s);
    if (e == hipSuccess)
      e = logo::launch_select_segments((int)n_examples, seg, gate, mask, d.k > 0 ? idx : nullptr,
                                       rank, d.k, s, nidx, d.n - d.k);
  }
  if (e != hipSuccess) return hip_fail(e, "select launch");
  logo::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.idx = idx;
  a.rank = rank;
  a.gate = gate;
  a.out_f32 = scratch;
  a.scratch = scratch;
  a.out_io = o;
  a.seg_start = seg_start;
  a.sched = d.dtype == LOGO_BF16 ? reinterpret_cast<int32_t*>(w + ws.sched) : nullptr;
  if (ws.fused) {
    StageTimer tm(9, s);
    e = logo::launch_attn_bf16_fused(d, a, nidx, s);
    if (e != hipSuccess) return hip_fail(e, "fused attention launch");
    return LOGO_OK;
  }
  {
    StageTimer tm(1, s);
    e = run_attn(d, logo::Epi::LocalFused, a, s);
  }
  if (e != hipSuccess) return hip_fail(e, "local attention launch");
  if (d.k > 0) {
    StageTimer tm(2, s);
    e = run_attn(d, logo::Epi::GlobalFused, a, s);
    if (e != hipSuccess) return hip_fail(e, "global attention launch");
  }
  return LOGO_OK;
}

logo_status logo_profile_begin(void) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on = true;
  g_prof.recs.clear();
  return LOGO_OK;
}

logo_status logo_profile_end(double* stage_ms, int64_t* stage_launches, int32_t n_stages) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.on = false;
  if (n_stages < 0 || (n_stages > 0 && (!stage_ms || !stage_launches)))
    return fail(LOGO_ERR_INVALID_ARG, "stage arrays missing");
  for (int i = 0; i < n_stages; ++i) {
    stage_ms[i] = 0.0;
    stage_launches[i] = 0;
  }
  for (auto& r : g_prof.recs) {
    hipError_t e = hipEventSynchronize(r.b);
    if (e != hipSuccess) return hip_fail(e, "profile event wait");
    float ms = 0.0f;
    e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e, "profile event time");
    if (r.stage >= 0 && r.stage < n_stages) {
      stage_ms[r.stage] += ms;
      stage_launches[r.stage] += 1;
    }
  }
  g_prof.recs.clear();
  return LOGO_OK;
}

}  // extern "C"
