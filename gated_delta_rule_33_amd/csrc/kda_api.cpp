// C ABI of the KDA forward library: argument validation, workspace layout and
// kernel launches.  Declarations and the contract of every entry point are in
// include/kda.h.
//
// Error conventions follow the chunk_kda integration described on the page
// "feat(kda): integrate KDA attention with tokamax backend and CP support"
// (Runtime guards; the review commits of its second copy): unsupported shapes
// are NOT_IMPLEMENTED, invalid configurations (a safe-gate lower bound outside
// [-5, 0), packed input without a positive segment bound) are
// INVALID_ARGUMENT, and there is never a silent fallback to another path.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>

#include "kda.h"
#include "kda_launch.h"

namespace {

thread_local std::string g_last_error;
kda_launch_observer_t g_observer = nullptr;
void* g_observer_user = nullptr;
bool g_fused_forward = false;

// Enqueue one kernel, with the observer (if any) called around it.
template <class F>
hipError_t observed(const char* name, hipStream_t s, F&& launch) {
  if (g_observer) g_observer(name, s, 0, g_observer_user);
  const hipError_t e = launch();
  if (g_observer) g_observer(name, s, 1, g_observer_user);
  return e;
}

kda_status_t fail(kda_status_t st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Plan {
  int64_t nc_fixed = 0, cmax = 0, smax = 0, record_bytes = 0;
  size_t off_hdr = 0, off_segs = 0, off_chunks = 0, off_rows = 0, off_records = 0, off_fused = 0, total = 0;
};

bool is_pow_ok(int64_t d) { return d == 64 || d == 128; }

// The integer a caller stored in an enum field or argument.  C callers (and
// ctypes) can pass any int there; reading it as the enum type would be
// undefined for values outside the enumerators, so its bytes are copied.
int32_t enum_int(const kda_dtype_t& e) {
  int32_t x;
  static_assert(sizeof(x) == sizeof(e), "enum is int-sized");
  std::memcpy(&x, &e, sizeof(x));
  return x;
}
bool dtype_ok(const kda_dtype_t& e) { return enum_int(e) == KDA_F32 || enum_int(e) == KDA_BF16; }
bool is_bf16(const kda_dtype_t& e) { return enum_int(e) == KDA_BF16; }

// a * b into *out unless it overflows int64 (both >= 0).
bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

kda_status_t validate(const kda_fwd_desc_t* d, bool has_seg, Plan* plan) {
  if (d == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->B < 0 || d->T < 0 || d->H < 0)
    return fail(KDA_ERR_INVALID_ARGUMENT, "B, T and H must be >= 0");
  int64_t tokens = 0;
  if (d->T > (int64_t)1 << 30 || !mul_ok(d->B, d->T, &tokens) || tokens > (int64_t)1 << 31)
    return fail(KDA_ERR_NOT_IMPLEMENTED, "B*T above 2^31 tokens is not supported");
  if (d->H > (int64_t)1 << 16) return fail(KDA_ERR_NOT_IMPLEMENTED, "more than 65536 heads is not supported");
  if (!is_pow_ok(d->K) || !is_pow_ok(d->V))
    return fail(KDA_ERR_NOT_IMPLEMENTED, "K and V must each be 64 or 128");
  if (!dtype_ok(d->dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "dtype must be KDA_F32 or KDA_BF16");
  if (!dtype_ok(d->o_dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "o_dtype must be KDA_F32 or KDA_BF16");
  if (d->chunk_size != 64) return fail(KDA_ERR_NOT_IMPLEMENTED, "chunk_size must be 64");
  if (d->use_qk_l2norm != 0 && d->use_qk_l2norm != 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "use_qk_l2norm must be 0 or 1");
  if (d->safe_gate != 0 && d->safe_gate != 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "safe_gate must be 0 or 1");
  if (d->safe_gate && !(d->lower_bound >= -5.f && d->lower_bound < 0.f))
    return fail(KDA_ERR_INVALID_ARGUMENT, "with safe_gate, lower_bound must lie in [-5, 0)");
  if (!std::isnan(d->scale) && !std::isfinite(d->scale))
    return fail(KDA_ERR_INVALID_ARGUMENT, "scale must be finite (or NaN for 1/sqrt(K))");
  if (has_seg && d->max_segments < 1)
    return fail(KDA_ERR_INVALID_ARGUMENT, "packed input (segment_ids) needs max_segments >= 1");
  // Every size below fits int64 (and size_t) once these hold.
  int64_t slots = 0, chunk_slots = 0, rec_total = 0;
  const int64_t n_seg = has_seg ? d->max_segments : 1;
  if (!mul_ok(d->B, n_seg, &slots) || slots > (int64_t)1 << 31 ||
      !mul_ok(d->B, (d->T + 63) / 64 + (has_seg ? d->max_segments : 0), &chunk_slots) ||
      !mul_ok(chunk_slots, d->H, &rec_total) || !mul_ok(rec_total, (int64_t)1 << 22, &rec_total))
    return fail(KDA_ERR_NOT_IMPLEMENTED, "the workspace for this request would not fit a 64-bit size");

  const kda::InType in = is_bf16(d->dtype) ? kda::InType::BF16 : kda::InType::F32;
  Plan p;
  p.nc_fixed = (d->T + 63) / 64;
  p.record_bytes = kda::record_bytes(in, d->K, d->V);
  if (has_seg) {
    p.smax = d->B * (int64_t)d->max_segments;
    p.cmax = d->B * (p.nc_fixed + d->max_segments);
  } else {
    p.smax = d->B;
    p.cmax = d->B * p.nc_fixed;
  }
  size_t off = 0;
  p.off_hdr = off;
  off = align_up(off + sizeof(kda::TableHeader));
  p.off_segs = off;
  off = align_up(off + (has_seg ? (size_t)p.smax * sizeof(kda::SegEntry) : 0));
  p.off_chunks = off;
  off = align_up(off + (has_seg ? (size_t)p.cmax * sizeof(kda::ChunkEntry) : 0));
  p.off_rows = off;
  off = align_up(off + (has_seg ? (size_t)d->B * sizeof(kda::RowInfo) : 0));
  p.off_records = off;
  off = align_up(off + (size_t)p.cmax * (size_t)d->H * (size_t)p.record_bytes);
  p.off_fused = off;   // scheduling words, ready words and lane states of the fused forward
  off = align_up(off + sizeof(kda::FusedCtl) + (size_t)p.cmax * (size_t)d->H * sizeof(uint32_t));
  off = align_up(off + (has_seg ? 0 : (size_t)d->B * (size_t)d->H * (size_t)d->K * (size_t)d->V * sizeof(float)));
  p.total = off;
  *plan = p;
  return KDA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// What the forward entry points add to the plain call.
struct FwdExtra {
  int gate_mode = 0;          // 0: g is the log decay; 1, 2: activated in the kernel (without / with safe gate)
  const float* a_log = nullptr;
  const float* dt_bias = nullptr;
  float* transition = nullptr;   // also compute each row's transition
  bool rerun = false;            // only the recurrence, from the records already in the workspace
};

kda_status_t forward(const kda_fwd_desc_t* desc, const void* q, const void* k, const void* v, const void* g,
                     const void* beta, const FwdExtra& x, const float* initial_state, const int32_t* segment_ids,
                     void* o, float* final_state, void* workspace, size_t workspace_bytes, void* stream);

}  // namespace

extern "C" {

kda_status_t kda_chunk_fwd_workspace_size(const kda_fwd_desc_t* desc, int has_segment_ids, size_t* bytes) {
  if (bytes == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  Plan plan;
  const kda_status_t st = validate(desc, has_segment_ids != 0, &plan);
  if (st != KDA_OK) return st;
  *bytes = plan.total;
  return KDA_OK;
}

kda_status_t kda_chunk_fwd(const kda_fwd_desc_t* desc, const void* q, const void* k, const void* v,
                           const void* g, const void* beta, const float* initial_state,
                           const int32_t* segment_ids, void* o, float* final_state, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return forward(desc, q, k, v, g, beta, FwdExtra{}, initial_state, segment_ids, o, final_state, workspace,
                 workspace_bytes, stream);
}

kda_status_t kda_chunk_fwd_gated(const kda_fwd_desc_t* desc, const void* q, const void* k, const void* v,
                                 const void* g, const void* beta, const float* A_log, const float* dt_bias,
                                 const float* initial_state, const int32_t* segment_ids, void* o,
                                 float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
  FwdExtra x;
  x.gate_mode = (desc != nullptr && desc->safe_gate) ? 2 : 1;
  x.a_log = A_log;
  x.dt_bias = dt_bias;
  return forward(desc, q, k, v, g, beta, x, initial_state, segment_ids, o, final_state, workspace, workspace_bytes,
                 stream);
}

kda_status_t kda_chunk_fwd_transition(const kda_fwd_desc_t* desc, const void* q, const void* k, const void* v,
                                      const void* g, const void* beta, const float* initial_state,
                                      const int32_t* segment_ids, void* o, float* final_state, float* transition,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (transition == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "transition is NULL");
  FwdExtra x;
  x.transition = transition;
  return forward(desc, q, k, v, g, beta, x, initial_state, segment_ids, o, final_state, workspace, workspace_bytes,
                 stream);
}

kda_status_t kda_chunk_fwd_rerun(const kda_fwd_desc_t* desc, const float* initial_state, const int32_t* segment_ids,
                                 void* o, float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
  FwdExtra x;
  x.rerun = true;
  return forward(desc, nullptr, nullptr, nullptr, nullptr, nullptr, x, initial_state, segment_ids, o, final_state,
                 workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// The forward's workspace for callers that cannot allocate: a fixed region
// in device memory, one copy per GPU, held until the process ends.  In host
// code `scratch` only names the symbol; its device address (different on
// every GPU) is looked up once per device with hipGetSymbolAddress and used
// from then on.
__device__ __attribute__((aligned(256))) char scratch[KDA_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

kda_status_t static_workspace(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(KDA_ERR_NOT_IMPLEMENTED, "device index above 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(KDA_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status_t kda_chunk_fwd_noalloc(const kda_fwd_desc_t* desc, const void* q, const void* k, const void* v,
                                   const void* g, const void* beta, const float* initial_state,
                                   const int32_t* segment_ids, void* o, float* final_state, void* stream) {
  Plan plan;
  kda_status_t st = validate(desc, segment_ids != nullptr, &plan);
  if (st != KDA_OK) return st;
  if (plan.total > (size_t)KDA_STATIC_WORKSPACE_BYTES)
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "this forward needs " + std::to_string(plan.total) +
                                                 " bytes of workspace; the fixed region holds " +
                                                 std::to_string((size_t)KDA_STATIC_WORKSPACE_BYTES));
  void* ws = nullptr;
  st = static_workspace(&ws);
  if (st != KDA_OK) return st;
  return forward(desc, q, k, v, g, beta, FwdExtra{}, initial_state, segment_ids, o, final_state, ws,
                 (size_t)KDA_STATIC_WORKSPACE_BYTES, stream);
}

}  // extern "C"

namespace {

kda_status_t forward(const kda_fwd_desc_t* desc, const void* q, const void* k, const void* v, const void* g,
                     const void* beta, const FwdExtra& x, const float* initial_state, const int32_t* segment_ids,
                     void* o, float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
  const bool has_seg = segment_ids != nullptr;
  Plan plan;
  kda_status_t st = validate(desc, has_seg, &plan);
  if (st != KDA_OK) return st;
  const kda_fwd_desc_t& d = *desc;
  const int64_t tokens = d.B * d.T;
  if (tokens > 0 && d.H > 0) {
    if (!x.rerun && (!q || !k || !v || !g || !beta))
      return fail(KDA_ERR_INVALID_ARGUMENT, "q, k, v, g, beta and o must be non-NULL");
    if (!o) return fail(KDA_ERR_INVALID_ARGUMENT, "q, k, v, g, beta and o must be non-NULL");
    const void* ptrs[] = {q, k, v, g, beta, o, initial_state, segment_ids, final_state, workspace, x.transition};
    for (const void* ptr : ptrs)
      if (ptr && !aligned16(ptr)) return fail(KDA_ERR_INVALID_ARGUMENT, "every pointer must be 16-byte aligned");
    const void* gate_ptrs[] = {x.a_log, x.dt_bias};
    for (const void* ptr : gate_ptrs)
      if (ptr && (reinterpret_cast<uintptr_t>(ptr) & 3) != 0)
        return fail(KDA_ERR_INVALID_ARGUMENT, "A_log and dt_bias must be float-aligned");
  }
  if (workspace_bytes < plan.total || (plan.total > 0 && workspace == nullptr))
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL,
                "workspace needs " + std::to_string(plan.total) + " bytes, got " + std::to_string(workspace_bytes));

  kda::CallArgs a{};
  a.B = d.B; a.T = d.T; a.H = d.H; a.K = d.K; a.V = d.V;
  a.in = is_bf16(d.dtype) ? kda::InType::BF16 : kda::InType::F32;
  a.out = is_bf16(d.o_dtype) ? kda::OutType::BF16 : kda::OutType::F32;
  a.scale = std::isnan(d.scale) ? (float)(1.0 / std::sqrt((double)d.K)) : d.scale;
  a.l2norm = d.use_qk_l2norm;
  a.n_max = has_seg ? d.max_segments : 0;
  a.nc_fixed = plan.nc_fixed;
  a.cmax = plan.cmax;
  a.smax = plan.smax;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.gate_mode = x.gate_mode;
  a.lower_bound = d.lower_bound;
  a.a_log = x.a_log;
  a.dt_bias = x.dt_bias;
  a.trans = x.transition;
  a.init = initial_state;
  a.seg_ids = segment_ids;
  a.o = o;
  a.fin = final_state;
  char* ws = static_cast<char*>(workspace);
  a.hdr = reinterpret_cast<kda::TableHeader*>(ws + plan.off_hdr);
  a.segs = reinterpret_cast<kda::SegEntry*>(ws + plan.off_segs);
  a.chunks = reinterpret_cast<kda::ChunkEntry*>(ws + plan.off_chunks);
  a.rows = reinterpret_cast<kda::RowInfo*>(ws + plan.off_rows);
  a.records = ws + plan.off_records;
  a.fused_ctl = reinterpret_cast<kda::FusedCtl*>(ws + plan.off_fused);
  a.fused_ready = reinterpret_cast<uint32_t*>(ws + plan.off_fused + sizeof(kda::FusedCtl));
  a.fused_lane_state = has_seg ? nullptr
                               : reinterpret_cast<float*>(ws + align_up(plan.off_fused + sizeof(kda::FusedCtl) +
                                                                        (size_t)plan.cmax * (size_t)d.H * 4));
  a.n_xcd = kda::xcd_count();
  a.record_bytes = plan.record_bytes;
  a.stream = static_cast<hipStream_t>(stream);

  if (d.B == 0 || d.H == 0) return KDA_OK;
  hipError_t e = hipSuccess;
  const hipStream_t s = a.stream;
  if (d.T == 0) {
    // No token, so no segment: every requested state slot (and transition) is zero.
    if (!x.rerun) e = observed("kda_zero_states", s, [&] { return kda::launch_zero_states(a); });
    if (e != hipSuccess) return fail(KDA_ERR_HIP, std::string("launch: ") + hipGetErrorString(e));
    return KDA_OK;
  }
  if (!x.rerun && g_fused_forward && kda::fused_supported(a)) {
    e = observed("kda_fused", s, [&] { return kda::launch_fused(a); });
  } else {
    if (!x.rerun) {
      if (has_seg) e = observed("kda_prep", s, [&] { return kda::launch_prep(a); });
      else if (KDA_DEBUG_CHECKS)
        e = observed("kda_clear_flags", s, [&] { return kda::launch_fill_zero(reinterpret_cast<float*>(&a.hdr->flags), 1, s); });
      if (e == hipSuccess) e = observed("kda_intra", s, [&] { return kda::launch_intra(a); });
    }
    if (e == hipSuccess) e = observed("kda_recur", s, [&] { return kda::launch_recur(a); });
  }
  if (e == hipSuccess && a.trans != nullptr) {
    kda::CallArgs t = a;
    t.trans_only = true;
    e = observed("kda_transition", s, [&] { return kda::launch_recur(t); });
  }
  if (e != hipSuccess) return fail(KDA_ERR_HIP, std::string("launch: ") + hipGetErrorString(e));
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status_t kda_short_conv_fwd(int64_t B, int64_t T, int64_t D, int32_t W, kda_dtype_t dtype, const void* x,
                                const float* weight, const int32_t* segment_ids, void* y, void* stream) {
  if (B < 0 || T < 0 || D < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "B, T and D must be >= 0");
  if (W < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "W must be >= 1 (W = 0 disables the convolution: skip the call)");
  if (W > 8) return fail(KDA_ERR_NOT_IMPLEMENTED, "kernel sizes above 8 are not supported");
  if (D % 8 != 0) return fail(KDA_ERR_NOT_IMPLEMENTED, "D must be a multiple of 8");
  if (!dtype_ok(dtype)) return fail(KDA_ERR_INVALID_ARGUMENT, "dtype must be KDA_F32 or KDA_BF16");
  if (B * T * D == 0) return KDA_OK;
  if (!x || !weight || !y) return fail(KDA_ERR_INVALID_ARGUMENT, "x, weight and y must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(y) & 15) ||
      (reinterpret_cast<uintptr_t>(weight) & 3) || (reinterpret_cast<uintptr_t>(segment_ids) & 3))
    return fail(KDA_ERR_INVALID_ARGUMENT, "x and y must be 16-byte aligned, weight and segment_ids 4-byte aligned");
  kda::ConvArgs a{B, T, D, W, is_bf16(dtype), x, weight, segment_ids, y, static_cast<hipStream_t>(stream)};
  const hipError_t e = observed("kda_short_conv", a.stream, [&] { return kda::launch_short_conv(a); });
  if (e != hipSuccess) return fail(KDA_ERR_HIP, std::string("launch: ") + hipGetErrorString(e));
  return KDA_OK;
}

kda_status_t kda_gated_rmsnorm_fwd(int64_t rows, int64_t V, kda_dtype_t o_dtype, kda_dtype_t gate_dtype,
                                   kda_dtype_t y_dtype, const void* o, const void* gate, const float* weight,
                                   float eps, void* y, void* stream) {
  if (rows < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "rows must be >= 0");
  if (V != 64 && V != 128 && V != 256) return fail(KDA_ERR_NOT_IMPLEMENTED, "V must be 64, 128 or 256");
  if (!dtype_ok(o_dtype) || !dtype_ok(gate_dtype) || !dtype_ok(y_dtype))
    return fail(KDA_ERR_INVALID_ARGUMENT, "dtypes must be KDA_F32 or KDA_BF16");
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(KDA_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if (rows == 0) return KDA_OK;
  if (!o || !gate || !weight || !y) return fail(KDA_ERR_INVALID_ARGUMENT, "o, gate, weight and y must be non-NULL");
  const void* ptrs[] = {o, gate, weight, y};
  for (const void* p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) & 3) return fail(KDA_ERR_INVALID_ARGUMENT, "pointers must be 4-byte aligned");
  kda::NormArgs a{rows, V, is_bf16(o_dtype), is_bf16(gate_dtype), is_bf16(y_dtype), o, gate, weight, eps, y,
                  static_cast<hipStream_t>(stream)};
  const hipError_t e = observed("kda_gated_rmsnorm", a.stream, [&] { return kda::launch_gated_rmsnorm(a); });
  if (e != hipSuccess) return fail(KDA_ERR_HIP, std::string("launch: ") + hipGetErrorString(e));
  return KDA_OK;
}

kda_status_t kda_chunk_fwd_flags(const void* workspace, size_t workspace_bytes, void* stream, uint32_t* flags) {
  if (flags == nullptr || workspace == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "NULL argument");
  if (workspace_bytes < sizeof(kda::TableHeader))
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL, "workspace smaller than its header");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(s);
  kda::TableHeader hdr;
  if (e == hipSuccess) e = hipMemcpy(&hdr, workspace, sizeof(hdr), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(KDA_ERR_HIP, std::string("flags: ") + hipGetErrorString(e));
  *flags = hdr.flags;
  return KDA_OK;
}

void kda_set_fused_forward(int enable) { g_fused_forward = enable != 0; }

void kda_set_launch_observer(kda_launch_observer_t fn, void* user) {
  g_observer = fn;
  g_observer_user = user;
}

const char* kda_last_error(void) { return g_last_error.c_str(); }

const char* kda_version(void) { return KDA_DEBUG_CHECKS ? "kda-mi355x 0.2.0 debug-checks" : "kda-mi355x 0.2.0"; }

}  // extern "C"

namespace {

kda_status_t cp_validate(const kda_cp_desc_t* d) {
  if (d == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "desc is NULL");
  if (d->B < 0 || d->T < 0 || d->H < 0) return fail(KDA_ERR_INVALID_ARGUMENT, "B, T and H must be >= 0");
  if (d->P < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "P must be >= 1");
  if (d->T % d->P != 0) return fail(KDA_ERR_INVALID_ARGUMENT, "T must be a multiple of P");
  if (d->n_states < 1) return fail(KDA_ERR_INVALID_ARGUMENT, "n_states must be >= 1");
  if (!is_pow_ok(d->K) || !is_pow_ok(d->V)) return fail(KDA_ERR_NOT_IMPLEMENTED, "K and V must each be 64 or 128");
  int64_t n = 0;
  if (!mul_ok(d->B, d->P, &n) || !mul_ok(n, d->n_states, &n) || !mul_ok(n, d->H, &n) || n > (int64_t)INT32_MAX ||
      d->T > (int64_t)1 << 30)
    return fail(KDA_ERR_NOT_IMPLEMENTED, "B * P * n_states * H above 2^31 (or T above 2^30) is not supported");
  return KDA_OK;
}

kda::CpArgs cp_args(const kda_cp_desc_t* d, void* stream) {
  kda::CpArgs a{};
  a.B = d->B; a.T = d->T; a.H = d->H; a.K = d->K; a.V = d->V;
  a.P = d->P;
  a.nm = d->n_states;
  a.stream = static_cast<hipStream_t>(stream);
  return a;
}

kda_status_t cp_launch(const char* name, hipStream_t s, hipError_t (*fn)(const kda::CpArgs&), const kda::CpArgs& a) {
  const hipError_t e = observed(name, s, [&] { return fn(a); });
  if (e != hipSuccess) return fail(KDA_ERR_HIP, std::string("launch: ") + hipGetErrorString(e));
  return KDA_OK;
}

bool all_aligned16(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return false;
  return true;
}

}  // namespace

extern "C" {

kda_status_t kda_cp_plan(const kda_cp_desc_t* desc, const int32_t* segment_ids, int32_t* plan, void* stream) {
  kda_status_t st = cp_validate(desc);
  if (st != KDA_OK) return st;
  if (desc->B == 0) return KDA_OK;
  if (plan == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (desc->T == 0) return fail(KDA_ERR_INVALID_ARGUMENT, "T must be >= 1 to be cut into slices");
  if (!all_aligned16({segment_ids, plan})) return fail(KDA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  kda::CpArgs a = cp_args(desc, stream);
  a.seg = segment_ids;
  a.plan = plan;
  return cp_launch("kda_cp_plan", a.stream, kda::launch_cp_plan, a);
}

kda_status_t kda_cp_gather_states(const kda_cp_desc_t* desc, const int32_t* plan, const float* initial_state,
                                  const float* carry, float* local_states, void* stream) {
  kda_status_t st = cp_validate(desc);
  if (st != KDA_OK) return st;
  if (desc->B == 0 || desc->H == 0) return KDA_OK;
  if (!plan || !local_states) return fail(KDA_ERR_INVALID_ARGUMENT, "plan and local_states must be non-NULL");
  if (!all_aligned16({plan, initial_state, carry, local_states}))
    return fail(KDA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  kda::CpArgs a = cp_args(desc, stream);
  a.plan = const_cast<int32_t*>(plan);
  a.init = initial_state;
  a.carry = const_cast<float*>(carry);
  a.local = local_states;
  return cp_launch("kda_cp_gather", a.stream, kda::launch_cp_gather, a);
}

kda_status_t kda_cp_chain(const kda_cp_desc_t* desc, const int32_t* plan, const float* local_final,
                          const float* transition, float* carry, void* stream) {
  kda_status_t st = cp_validate(desc);
  if (st != KDA_OK) return st;
  if (desc->B == 0 || desc->H == 0) return KDA_OK;
  if (!plan || !local_final || !transition || !carry)
    return fail(KDA_ERR_INVALID_ARGUMENT, "plan, local_final, transition and carry must be non-NULL");
  if (!all_aligned16({plan, local_final, transition, carry}))
    return fail(KDA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  kda::CpArgs a = cp_args(desc, stream);
  a.plan = const_cast<int32_t*>(plan);
  a.local = const_cast<float*>(local_final);
  a.trans = transition;
  a.carry = carry;
  return cp_launch("kda_cp_chain", a.stream, kda::launch_cp_chain, a);
}

kda_status_t kda_cp_scatter_states(const kda_cp_desc_t* desc, const int32_t* plan, const float* local_final,
                                   float* final_state, void* stream) {
  kda_status_t st = cp_validate(desc);
  if (st != KDA_OK) return st;
  if (desc->B == 0 || desc->H == 0) return KDA_OK;
  if (!plan || !local_final || !final_state)
    return fail(KDA_ERR_INVALID_ARGUMENT, "plan, local_final and final_state must be non-NULL");
  if (!all_aligned16({plan, local_final, final_state}))
    return fail(KDA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  kda::CpArgs a = cp_args(desc, stream);
  a.plan = const_cast<int32_t*>(plan);
  a.local = const_cast<float*>(local_final);
  a.fin = final_state;
  return cp_launch("kda_cp_scatter", a.stream, kda::launch_cp_scatter, a);
}

}  // extern "C"

namespace {

struct BwdPlan {
  Plan t;                      // tables (the forward's layout up to its records)
  size_t off_rec = 0, off_hs = 0, off_dhs = 0, off_ds = 0, off_dds = 0, total = 0;
};

kda_status_t bwd_validate(const kda_fwd_desc_t* d, bool has_seg, BwdPlan* bp) {
  BwdPlan b;
  const kda_status_t st = validate(d, has_seg, &b.t);
  if (st != KDA_OK) return st;
  const size_t slots = 4 * (size_t)b.t.cmax, H = (size_t)d->H;
  b.off_rec = b.t.off_records;
  size_t off = align_up(b.off_rec + slots * H * (size_t)kda::bwd_record_floats(d->K, d->V) * sizeof(float));
  b.off_hs = off;   // the state entering every 64-token chunk
  off = align_up(off + (size_t)b.t.cmax * H * (size_t)(d->K * d->V) * sizeof(float));
  b.off_dhs = off;
  off = align_up(off + slots * H * (size_t)(d->K * d->V) * sizeof(float));
  b.off_ds = off;
  off = align_up(off + slots * H * (size_t)(16 * d->V) * sizeof(float));
  b.off_dds = off;
  b.total = align_up(off + slots * H * (size_t)(16 * d->V) * sizeof(float));
  *bp = b;
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status_t kda_chunk_bwd_workspace_size(const kda_fwd_desc_t* desc, int has_segment_ids, size_t* bytes) {
  if (bytes == nullptr) return fail(KDA_ERR_INVALID_ARGUMENT, "bytes is NULL");
  BwdPlan bp;
  const kda_status_t st = bwd_validate(desc, has_segment_ids != 0, &bp);
  if (st != KDA_OK) return st;
  *bytes = bp.total;
  return KDA_OK;
}

}  // extern "C"

namespace {

// The backward; `rerun` keeps the chunk records and states a previous call
// left in the workspace and runs only the reverse recurrence and the
// per-chunk gradients again.
kda_status_t backward(const kda_fwd_desc_t* desc, const void* q, const void* k, const void* v, const void* g,
                      const void* beta, const float* initial_state, const int32_t* segment_ids, const void* d_o,
                      const float* d_final_state, float* dq, float* dk, float* dv, float* dg, float* dbeta,
                      float* d_initial_state, void* workspace, size_t workspace_bytes, void* stream, bool rerun) {
  const bool has_seg = segment_ids != nullptr;
  BwdPlan bp;
  kda_status_t st = bwd_validate(desc, has_seg, &bp);
  if (st != KDA_OK) return st;
  const kda_fwd_desc_t& d = *desc;
  if (d.B * d.T > 0 && d.H > 0) {
    const void* need[] = {q, k, v, g, beta, d_o, dq, dk, dv, dg, dbeta};
    for (const void* ptr : need)
      if (!ptr) return fail(KDA_ERR_INVALID_ARGUMENT, "q, k, v, g, beta, d_o and every gradient must be non-NULL");
    const void* ptrs[] = {q, k, v, g, beta, d_o, dq, dk, dv, dg, dbeta, initial_state, segment_ids, d_final_state,
                          d_initial_state, workspace};
    for (const void* ptr : ptrs)
      if (ptr && !aligned16(ptr)) return fail(KDA_ERR_INVALID_ARGUMENT, "every pointer must be 16-byte aligned");
  }
  if (workspace_bytes < bp.total || (bp.total > 0 && workspace == nullptr))
    return fail(KDA_ERR_WORKSPACE_TOO_SMALL,
                "workspace needs " + std::to_string(bp.total) + " bytes, got " + std::to_string(workspace_bytes));
  if (d.B == 0 || d.H == 0) return KDA_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  kda::CallArgs t{};   // the segment tables, built as for the forward
  t.B = d.B; t.T = d.T; t.H = d.H; t.K = d.K; t.V = d.V;
  t.in = is_bf16(d.dtype) ? kda::InType::BF16 : kda::InType::F32;
  t.out = kda::OutType::F32;
  t.n_max = has_seg ? d.max_segments : 0;
  t.nc_fixed = bp.t.nc_fixed;
  t.cmax = bp.t.cmax;
  t.smax = bp.t.smax;
  t.seg_ids = segment_ids;
  t.hdr = reinterpret_cast<kda::TableHeader*>(ws + bp.t.off_hdr);
  t.segs = reinterpret_cast<kda::SegEntry*>(ws + bp.t.off_segs);
  t.chunks = reinterpret_cast<kda::ChunkEntry*>(ws + bp.t.off_chunks);
  t.rows = reinterpret_cast<kda::RowInfo*>(ws + bp.t.off_rows);
  t.stream = s;
  const int64_t slot_elems = d.H * d.K * d.V;
  hipError_t e = hipSuccess;
  auto zero = [&](float* x, int64_t n) {
    if (e == hipSuccess) e = observed("kda_bwd_zero", s, [&] { return kda::launch_fill_zero(x, n, s); });
  };
  if (d.T == 0) {
    zero(d_initial_state, bp.t.smax * slot_elems);
  } else {
    if (has_seg && !rerun) {
      // padding tokens, unrecorded segments and absent state slots keep zero gradients
      e = observed("kda_prep", s, [&] { return kda::launch_prep(t); });
      const int64_t tok = d.B * d.T * d.H;
      zero(dq, tok * d.K);
      zero(dk, tok * d.K);
      zero(dg, tok * d.K);
      zero(dv, tok * d.V);
      zero(dbeta, tok);
      zero(d_initial_state, bp.t.smax * slot_elems);
    }
    kda::BwdArgs a{};
    a.B = d.B; a.T = d.T; a.H = d.H; a.K = d.K; a.V = d.V;
    a.in = t.in;
    a.do_bf16 = is_bf16(d.o_dtype);
    a.scale = std::isnan(d.scale) ? (float)(1.0 / std::sqrt((double)d.K)) : d.scale;
    a.l2norm = d.use_qk_l2norm;
    a.n_max = t.n_max;
    a.nc_fixed = t.nc_fixed;
    a.cmax = t.cmax;
    a.smax = t.smax;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.d_o = d_o;
    a.init = initial_state;
    a.d_final = d_final_state;
    a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta; a.d_init = d_initial_state;
    a.hdr = t.hdr; a.segs = t.segs; a.chunks = t.chunks;
    a.rec = reinterpret_cast<float*>(ws + bp.off_rec);
    a.hs = reinterpret_cast<float*>(ws + bp.off_hs);
    a.dhs = reinterpret_cast<float*>(ws + bp.off_dhs);
    a.ds = reinterpret_cast<float*>(ws + bp.off_ds);
    a.dds = reinterpret_cast<float*>(ws + bp.off_dds);
    a.stream = s;
    static const char* const names[4] = {"kda_bwd_chunk", "kda_bwd_states", "kda_bwd_dstates", "kda_bwd_local"};
    for (int stage = rerun ? 2 : 0; stage < 4 && e == hipSuccess; ++stage)
      e = observed(names[stage], s, [&] { return kda::launch_bwd(a, stage); });
  }
  if (e != hipSuccess) return fail(KDA_ERR_HIP, std::string("launch: ") + hipGetErrorString(e));
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status_t kda_chunk_bwd(const kda_fwd_desc_t* desc, const void* q, const void* k, const void* v, const void* g,
                           const void* beta, const float* initial_state, const int32_t* segment_ids,
                           const void* d_o, const float* d_final_state, float* dq, float* dk, float* dv, float* dg,
                           float* dbeta, float* d_initial_state, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return backward(desc, q, k, v, g, beta, initial_state, segment_ids, d_o, d_final_state, dq, dk, dv, dg, dbeta,
                  d_initial_state, workspace, workspace_bytes, stream, false);
}

kda_status_t kda_chunk_bwd_rerun(const kda_fwd_desc_t* desc, const void* q, const void* k, const void* v,
                                 const void* g, const void* beta, const float* initial_state,
                                 const int32_t* segment_ids, const void* d_o, const float* d_final_state, float* dq,
                                 float* dk, float* dv, float* dg, float* dbeta, float* d_initial_state,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  return backward(desc, q, k, v, g, beta, initial_state, segment_ids, d_o, d_final_state, dq, dk, dv, dg, dbeta,
                  d_initial_state, workspace, workspace_bytes, stream, true);
}

}  // extern "C"

extern "C" {

kda_status_t kda_cp_gather_final_grads(const kda_cp_desc_t* desc, const int32_t* plan, const float* d_final_state,
                                       const float* carry_grad, float* local_d_final, void* stream) {
  kda_status_t st = cp_validate(desc);
  if (st != KDA_OK) return st;
  if (desc->B == 0 || desc->H == 0) return KDA_OK;
  if (!plan || !local_d_final) return fail(KDA_ERR_INVALID_ARGUMENT, "plan and local_d_final must be non-NULL");
  if (!all_aligned16({plan, d_final_state, carry_grad, local_d_final}))
    return fail(KDA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  kda::CpArgs a = cp_args(desc, stream);
  a.plan = const_cast<int32_t*>(plan);
  a.init = d_final_state;
  a.carry = const_cast<float*>(carry_grad);
  a.local = local_d_final;
  a.grads = true;
  return cp_launch("kda_cp_gather", a.stream, kda::launch_cp_gather, a);
}

kda_status_t kda_cp_chain_bwd(const kda_cp_desc_t* desc, const int32_t* plan, const float* local_d_initial,
                              const float* transition, float* carry_grad, void* stream) {
  kda_status_t st = cp_validate(desc);
  if (st != KDA_OK) return st;
  if (desc->B == 0 || desc->H == 0) return KDA_OK;
  if (!plan || !local_d_initial || !transition || !carry_grad)
    return fail(KDA_ERR_INVALID_ARGUMENT, "plan, local_d_initial, transition and carry_grad must be non-NULL");
  if (!all_aligned16({plan, local_d_initial, transition, carry_grad}))
    return fail(KDA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  kda::CpArgs a = cp_args(desc, stream);
  a.plan = const_cast<int32_t*>(plan);
  a.local = const_cast<float*>(local_d_initial);
  a.trans = transition;
  a.carry = carry_grad;
  return cp_launch("kda_cp_chain_bwd", a.stream, kda::launch_cp_chain_bwd, a);
}

kda_status_t kda_cp_scatter_initial_grads(const kda_cp_desc_t* desc, const int32_t* plan,
                                          const float* local_d_initial, float* d_initial_state, void* stream) {
  kda_status_t st = cp_validate(desc);
  if (st != KDA_OK) return st;
  if (desc->B == 0 || desc->H == 0) return KDA_OK;
  if (!plan || !local_d_initial || !d_initial_state)
    return fail(KDA_ERR_INVALID_ARGUMENT, "plan, local_d_initial and d_initial_state must be non-NULL");
  if (!all_aligned16({plan, local_d_initial, d_initial_state}))
    return fail(KDA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  kda::CpArgs a = cp_args(desc, stream);
  a.plan = const_cast<int32_t*>(plan);
  a.local = const_cast<float*>(local_d_initial);
  a.fin = d_initial_state;
  a.grads = true;
  return cp_launch("kda_cp_scatter", a.stream, kda::launch_cp_scatter, a);
}

}  // extern "C"
