// k3moe_api.cpp — the C ABI of include/k3moe.h: host-side argument validation,
// workspace carving and kernel dispatch. No device memory is allocated here; every
// launch goes onto the caller's stream.
#include "k3moe.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "k3moe_cache.h"
#include "k3moe_launch.h"

namespace k3moe {
thread_local LaunchTiming* t_launch_timing = nullptr;
}  // namespace k3moe

namespace {

thread_local std::string g_err;

// One-shot timing probe (k3moe_time_next_kernel).
thread_local int g_probe_which = 0;
thread_local hipEvent_t g_probe_start = nullptr, g_probe_stop = nullptr;

// Times one launch when armed for `which`: the launcher stamps the kernel's own begin and end
// (launch_timed); a launcher that does not time its kernel leaves events recorded around
// its launches.
struct Probe {
  int which;
  hipStream_t s;
  bool armed;
  k3moe::LaunchTiming lt;
  Probe(int w, hipStream_t st) : which(w), s(st), armed(g_probe_which == w) {
    if (armed) {
      (void)hipEventRecord(g_probe_start, s);
      lt = {g_probe_start, g_probe_stop, false};
      k3moe::t_launch_timing = &lt;
    }
  }
  ~Probe() {
    if (armed) {
      k3moe::t_launch_timing = nullptr;
      if (!lt.used) (void)hipEventRecord(g_probe_stop, s);
      g_probe_which = 0;
    }
  }
};

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

constexpr int kMaxE = 4096;
constexpr int kMaxK = 32;
constexpr int kMaxT = 1 << 20;
constexpr int kMaxWidth = 16384;
// From this many tokens on (bf16 activations) the expert matmuls run as grouped MFMA GEMMs;
// below, as per-expert GEMVs. At 32 tokens the MFMA path's down projection already streams
// twice as fast as the GEMV one.
constexpr int kMfmaMinTokens = 16;

enum Region {
  R_PART, R_IDS, R_GATES, R_OFFS, R_ROWS, R_ACT, R_NACT, R_PPOS, R_PEXP, R_HIST, R_BASE,
  R_MASK, R_H, R_Z, R_XHAT, R_HSH, R_SSH, R_MTILE, R_X8, R_XS, R_SIDS, R_COUNT
};

struct Layout {
  size_t off[R_COUNT];
  size_t total;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

Layout layout_for(const k3moe_dims& dm, int64_t T) {
  const int64_t d = dm.d_model, f = dm.d_ff, E = dm.n_experts, k = dm.top_k;
  const int64_t P = T * k;
  const int64_t NB = (T + k3moe::kBucketTokens - 1) / k3moe::kBucketTokens;
  const int64_t NC = k3moe::router_num_chunks((int)d);
  const int64_t tg = T < k3moe::kRouterGemvMaxT ? T : k3moe::kRouterGemvMaxT;
  // many-token router: up to 8 K-chunk partials, T * chunks bounded (monotone in T)
  const int64_t budget = k3moe::router_split_budget((int)E);
  const int64_t tk = T * 8 < budget ? T * 8 : budget;
  const size_t part_small = (size_t)(NC * tg * E * 8),
               part_big = (size_t)((tk > T ? tk : T) * E * 8);
  size_t sz[R_COUNT];
  sz[R_PART] = part_small > part_big ? part_small : part_big;
  sz[R_IDS] = (size_t)P * 4;
  sz[R_GATES] = (size_t)P * 4;
  sz[R_OFFS] = (size_t)(E + 1) * 4;
  sz[R_ROWS] = (size_t)P * 4;
  sz[R_ACT] = (size_t)E * 4;
  sz[R_NACT] = 16;
  sz[R_PPOS] = (size_t)P * 4;
  sz[R_PEXP] = (size_t)P * 4;
  sz[R_HIST] = (size_t)(NB * E * 4);
  sz[R_BASE] = (size_t)(NB * E * 4);
  sz[R_MASK] = (size_t)(NB * E * 8);
  sz[R_H] = (size_t)(P * f * 4);  // fp32 h, or three FP8 terms + their block scales
  sz[R_Z] = (size_t)(P * d * 4);
  sz[R_XHAT] = (size_t)(T * d * 4);
  sz[R_HSH] = (size_t)(T * f * 4);
  sz[R_SSH] = (size_t)(T * d * 4);
  sz[R_MTILE] = (size_t)(E + 1) * 4;
  sz[R_X8] = (size_t)(T * 2 * d);  // token rows as two FP8 terms
  sz[R_XS] = (size_t)(T * 2);      // their E8M0 scales
  sz[R_SIDS] = (size_t)P * 4;      // slot ids of the cached layer
  Layout L;
  size_t o = 0;
  for (int r = 0; r < R_COUNT; ++r) {
    L.off[r] = o;
    o = align_up(o + sz[r], 256);
  }
  L.total = o + 256;  // slack to align the caller's base pointer
  return L;
}

struct Ws {
  char* base;
  Layout L;
  template <class P>
  P* at(Region r) const { return reinterpret_cast<P*>(base + L.off[r]); }
};

int check_dims(const k3moe_dims* dims) {
  if (!dims) return fail(K3MOE_EINVAL, "dims is NULL");
  const k3moe_dims& d = *dims;
  if (d.d_model <= 0 || d.d_model % 32)
    return fail(K3MOE_EINVAL, "d_model=%d must be a positive multiple of 32", d.d_model);
  if (d.d_ff <= 0 || d.d_ff % 32)
    return fail(K3MOE_EINVAL, "d_ff=%d must be a positive multiple of 32", d.d_ff);
  if (d.n_experts < 1) return fail(K3MOE_EINVAL, "n_experts=%d must be >= 1", d.n_experts);
  const int kmax = d.n_experts < kMaxK ? d.n_experts : kMaxK;
  if (d.top_k < 1 || d.top_k > kmax)
    return fail(K3MOE_EINVAL, "top_k=%d outside [1, %d]", d.top_k, kmax);
  if (d.n_experts > kMaxE) return fail(K3MOE_EUNSUPPORTED, "n_experts=%d > %d", d.n_experts, kMaxE);
  if (d.d_model > kMaxWidth || d.d_ff > kMaxWidth)
    return fail(K3MOE_EUNSUPPORTED, "d_model/d_ff above %d", kMaxWidth);
  return K3MOE_OK;
}

int check_T(int32_t T) {
  if (T < 0) return fail(K3MOE_EINVAL, "T=%d is negative", T);
  if (T > kMaxT) return fail(K3MOE_EUNSUPPORTED, "T=%d > %d", T, kMaxT);
  return K3MOE_OK;
}

int check_dtype(int x_dtype) {
  if (x_dtype != K3MOE_BF16 && x_dtype != K3MOE_F32)
    return fail(K3MOE_EINVAL, "unknown x_dtype %d", x_dtype);
  return K3MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int need_ptr(const void* p, const char* name, bool align16 = false) {
  if (!p) return fail(K3MOE_EINVAL, "%s is NULL", name);
  if (align16 && !aligned16(p)) return fail(K3MOE_EINVAL, "%s is not 16-byte aligned", name);
  return K3MOE_OK;
}

int check_experts(const k3moe_mx_experts* ex) {
  if (!ex) return fail(K3MOE_EINVAL, "experts is NULL");
  int rc;
  if ((rc = need_ptr(ex->gate_q, "experts->gate_q", true))) return rc;
  if ((rc = need_ptr(ex->gate_s, "experts->gate_s"))) return rc;
  if ((rc = need_ptr(ex->up_q, "experts->up_q", true))) return rc;
  if ((rc = need_ptr(ex->up_s, "experts->up_s"))) return rc;
  if ((rc = need_ptr(ex->down_q, "experts->down_q", true))) return rc;
  if ((rc = need_ptr(ex->down_s, "experts->down_s"))) return rc;
  return K3MOE_OK;
}

int check_expert_shape(const k3moe_dims& dm) {
  if (!k3moe::gemv_shape_supported(dm.d_model, dm.d_ff))
    return fail(K3MOE_EUNSUPPORTED, "expert shape d_model=%d d_ff=%d not supported", dm.d_model,
                dm.d_ff);
  return K3MOE_OK;
}

int get_ws(const k3moe_dims& dm, int32_t T, void* ws, size_t ws_bytes, Ws* out) {
  out->L = layout_for(dm, T);
  if (ws_bytes < out->L.total)
    return fail(K3MOE_EWORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, out->L.total);
  if (!ws) return fail(K3MOE_EINVAL, "ws is NULL");
  out->base = reinterpret_cast<char*>(align_up(reinterpret_cast<uintptr_t>(ws), 256));
  return K3MOE_OK;
}

// Compute units of the current device (cached per device ordinal).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

int hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(K3MOE_EHIP, "%s: %s", what, hipGetErrorString(e));
  return K3MOE_OK;
}

k3moe::BucketOut bucket_out(const Ws& ws, int32_t* offsets, int32_t* rows) {
  k3moe::BucketOut o;
  o.offsets = offsets;
  o.rows = rows;
  o.act = ws.at<int32_t>(R_ACT);
  o.n_act = ws.at<int32_t>(R_NACT);
  o.pair_pos = ws.at<int32_t>(R_PPOS);
  o.pair_exp = ws.at<int32_t>(R_PEXP);
  o.mtile_off = ws.at<int32_t>(R_MTILE);
  return o;
}

// HIP objects the library keeps between calls: per device, one side stream (block mode)
// and kCopyStreams copy streams (slot cache), created on first use; per host thread and
// device, the fork/join events of block mode and of the copy streams. They live until
// k3moe_release() or the process ends. g_created tells k3moe_release whether anything was
// ever made (so it touches no HIP state in a process that never ran a kernel).
constexpr int kMaxDev = 64;
constexpr int kCopyStreams = 4;
std::mutex g_obj_mu;
hipStream_t g_side[kMaxDev] = {};
hipStream_t g_copy[kMaxDev][kCopyStreams] = {};
std::atomic<bool> g_created{false};
thread_local hipEvent_t t_fj[kMaxDev][2] = {};
thread_local hipEvent_t t_cp[kMaxDev][kCopyStreams + 1] = {};

bool make_event(hipEvent_t& ev) {
  if (ev) return true;
  if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) {
    ev = nullptr;
    return false;
  }
  g_created.store(true);
  return true;
}

bool make_stream(hipStream_t& st) {  // caller holds g_obj_mu
  if (st) return true;
  if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) {
    st = nullptr;
    return false;
  }
  g_created.store(true);
  return true;
}

// Fork and join events of block mode: one pair per host thread and device, created on
// first use and kept. Each call records them again; a stream wait takes the event's record
// at the time of the wait, calls from one thread are ordered on the host, and other
// threads have their own pair. (Creating and destroying them per call cost more host
// time than a decoder block's kernels take on the GPU.)
bool fork_join_events(hipEvent_t& fork, hipEvent_t& joined) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return false;
  if (!make_event(t_fj[dev][0]) || !make_event(t_fj[dev][1])) return false;
  fork = t_fj[dev][0];
  joined = t_fj[dev][1];
  return true;
}

// One non-blocking side stream per device (default priority) for work that can overlap
// the routed path.
hipStream_t side_stream() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
  std::lock_guard<std::mutex> lock(g_obj_mu);
  return make_stream(g_side[dev]) ? g_side[dev] : nullptr;
}

// Copy streams of the expert slot cache: kCopyStreams non-blocking streams per device
// (default priority), so the host -> HBM copies of several missing experts run on several
// DMA engines at once; plus, per host thread and device, one fork event and one join event
// per copy stream.
bool copy_streams(hipStream_t (&cs)[kCopyStreams], hipEvent_t& fork,
                  hipEvent_t (&join)[kCopyStreams]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return false;
  {
    std::lock_guard<std::mutex> lock(g_obj_mu);
    for (int i = 0; i < kCopyStreams; ++i)
      if (!make_stream(g_copy[dev][i])) return false;
    for (int i = 0; i < kCopyStreams; ++i) cs[i] = g_copy[dev][i];
  }
  for (int i = 0; i <= kCopyStreams; ++i)
    if (!make_event(t_cp[dev][i])) return false;
  for (int i = 0; i < kCopyStreams; ++i) join[i] = t_cp[dev][i + 1];
  fork = t_cp[dev][0];
  return true;
}

int run_router(const k3moe_dims& dm, int32_t T, const void* x, int xf32, const uint16_t* w,
               const float* bias, int32_t* ids, float* gates, const Ws& ws, hipStream_t s,
               const k3moe::BucketOut* bucket1 = nullptr) {
  double* part = ws.at<double>(R_PART);
  int nsum = 1;
  hipError_t e;
  Probe probe(K3MOE_KERNEL_ROUTER, s);
  if (T <= k3moe::kRouterGemvMaxT) {
    e = k3moe::launch_router_gemv(T, dm.d_model, dm.n_experts, x, xf32, w, part, s);
    nsum = k3moe::router_num_chunks(dm.d_model);
  } else {
    e = k3moe::launch_router_gemm(T, dm.d_model, dm.n_experts, x, xf32, w, part, &nsum, s);
  }
  int rc = hip_check(e, "router logits");
  if (rc) return rc;
  return hip_check(k3moe::launch_route_topk(T, dm.n_experts, dm.top_k, part, nsum, bias, ids,
                                            gates, bucket1, s),
                   "softmax/top-k");
}


// shared_ready (nullable): an event the stream waits on before the launch that reads
// `shared` (the shared expert runs on a side stream).
int run_ffn(const k3moe_dims& dm, int32_t T, const void* x, int xf32,
            const k3moe_mx_experts* ex, const int32_t* offsets, const int32_t* rows,
            const float* gates, const float* resid, const float* shared, float* y,
            uint16_t* y_bf16, const Ws& ws, hipStream_t s, hipEvent_t shared_ready = nullptr,
            bool packed = false, const k3moe::SharedDown* shared_down = nullptr) {
  auto join = [&]() -> int {
    return shared_ready ? hip_check(hipStreamWaitEvent(s, shared_ready, 0), "join shared expert")
                        : 0;
  };
  const int d = dm.d_model, f = dm.d_ff, E = dm.n_experts, k = dm.top_k;
  k3moe::MxPtrs w{ex->gate_q, ex->gate_s, ex->up_q, ex->up_s, ex->down_q, ex->down_s};
  const int64_t P = (int64_t)T * k;
  const int max_act = (int)(P < E ? P : E);
  float* h = ws.at<float>(R_H);
  int rc;
  const bool scales4 = ((reinterpret_cast<uintptr_t>(ex->gate_s) |
                         reinterpret_cast<uintptr_t>(ex->up_s) |
                         reinterpret_cast<uintptr_t>(ex->down_s)) & 3u) == 0;
  if (packed && T == 1 && k3moe::down_decode_mfma_supported(d, f, k)) {
    // packed tile layout, one token: h per (slot, 16-row tile) (and, in block mode, the shared
    // expert's down GEMV in the same launch), then the decode down kernel adds the slots in
    // order
    {
      Probe probe(K3MOE_KERNEL_GATE_UP, s);
      rc = hip_check(k3moe::launch_gateup_decode_packed(d, f, k, x, xf32, w,
                                                        ws.at<int32_t>(R_PPOS),
                                                        ws.at<int32_t>(R_PEXP), h, s,
                                                        shared_down),
                     "gate/up (decode, packed)");
    }
    if (rc || (rc = join())) return rc;
    Probe probe(K3MOE_KERNEL_DOWN, s);
    return hip_check(k3moe::launch_down_decode_mfma(d, f, k, w, h, ws.at<int32_t>(R_PPOS),
                                                    ws.at<int32_t>(R_PEXP), gates, resid, shared,
                                                    y, y_bf16, cu_count(), s, true),
                     "down+combine (decode, packed)");
  }
  if (shared_down)  // only the one-token packed launch runs it; callers check the shape first
    return fail(K3MOE_EUNSUPPORTED, "the shared expert's down GEMV rides only in the one-token "
                                    "packed gate/up launch");
  if (packed) {
    // packed tile layout: grouped GEMMs on the block-scaled MFMA for every token count (the
    // shapes and the bf16 activations were checked by the entry point)
    uint8_t* h8 = ws.at<uint8_t>(R_H);
    uint8_t* hs8 = h8 + (size_t)P * 3 * f;
    float* z = ws.at<float>(R_Z);
    {
      Probe probe(K3MOE_KERNEL_GATE_UP, s);
      rc = hip_check(k3moe::launch_gateup_mfma(T, d, f, E, k, static_cast<const uint16_t*>(x), w,
                                               offsets, rows, ws.at<int32_t>(R_ACT),
                                               ws.at<int32_t>(R_NACT), ws.at<int32_t>(R_MTILE),
                                               h8, hs8, ws.at<uint8_t>(R_X8),
                                               ws.at<uint8_t>(R_XS), s, true),
                     "gate/up (MFMA, packed)");
    }
    if (rc) return rc;
    {
      Probe probe(K3MOE_KERNEL_DOWN, s);
      rc = hip_check(k3moe::launch_down_mfma(T, d, f, E, k, w, h8, hs8, offsets, rows,
                                             ws.at<int32_t>(R_ACT), ws.at<int32_t>(R_NACT),
                                             ws.at<int32_t>(R_MTILE), z, s, true),
                     "down (MFMA, packed)");
    }
    if (rc || (rc = join())) return rc;
    return hip_check(k3moe::launch_combine(T, d, k, z, gates, ws.at<int32_t>(R_PPOS), resid,
                                           shared, y, y_bf16, s),
                     "combine");
  }
  if (T >= kMfmaMinTokens && !xf32 && scales4 && k3moe::mfma_shape_supported(d, f)) {
    // many tokens per expert: grouped GEMMs on the block-scaled FP4 x FP8 MFMA, h kept as
    // three E4M3 terms [P][3][f] with per-32-block scales [P][3][f/32] (in the h region)
    uint8_t* h8 = ws.at<uint8_t>(R_H);
    uint8_t* hs8 = h8 + (size_t)P * 3 * f;
    float* z = ws.at<float>(R_Z);
    const int32_t* mt = ws.at<int32_t>(R_MTILE);
    {
      Probe probe(K3MOE_KERNEL_GATE_UP, s);
      rc = hip_check(k3moe::launch_gateup_mfma(T, d, f, E, k, static_cast<const uint16_t*>(x), w,
                                               offsets, rows, ws.at<int32_t>(R_ACT),
                                               ws.at<int32_t>(R_NACT), mt, h8, hs8,
                                               ws.at<uint8_t>(R_X8), ws.at<uint8_t>(R_XS), s),
                     "gate/up (MFMA)");
    }
    if (rc) return rc;
    {
      Probe probe(K3MOE_KERNEL_DOWN, s);
      rc = hip_check(k3moe::launch_down_mfma(T, d, f, E, k, w, h8, hs8, offsets, rows,
                                             ws.at<int32_t>(R_ACT), ws.at<int32_t>(R_NACT), mt, z,
                                             s),
                     "down (MFMA)");
    }
    if (rc || (rc = join())) return rc;
    return hip_check(k3moe::launch_combine(T, d, k, z, gates, ws.at<int32_t>(R_PPOS), resid,
                                           shared, y, y_bf16, s),
                     "combine");
  }
  if (T == 1 && k3moe::down_fused_supported(f, k) && k3moe::gateup_decode_supported(d)) {
    // single token: persistent decode kernels
    {
      Probe probe(K3MOE_KERNEL_GATE_UP, s);
      rc = hip_check(k3moe::launch_gateup_decode(d, f, k, x, xf32, w, offsets,
                                                 ws.at<int32_t>(R_ACT), ws.at<int32_t>(R_NACT),
                                                 h, cu_count(), s),
                     "gate/up (decode)");
    }
    if (rc || (rc = join())) return rc;
    Probe probe(K3MOE_KERNEL_DOWN, s);
    return hip_check(k3moe::launch_down_decode(d, f, k, w, h, ws.at<int32_t>(R_PPOS),
                                               ws.at<int32_t>(R_PEXP), gates, resid, shared, y,
                                               y_bf16, cu_count(), s),
                     "down+combine (decode)");
  }
  {
    Probe probe(K3MOE_KERNEL_GATE_UP, s);
    rc = hip_check(k3moe::launch_gateup_gemv(T, d, f, E, k, x, xf32, w, offsets, rows,
                                             ws.at<int32_t>(R_ACT), ws.at<int32_t>(R_NACT),
                                             max_act, h, s),
                   "gate/up");
  }
  if (rc) return rc;
  float* z = ws.at<float>(R_Z);
  {
    Probe probe(K3MOE_KERNEL_DOWN, s);
    rc = hip_check(k3moe::launch_down_gemv(T, d, f, E, k, w, h, offsets, rows,
                                           ws.at<int32_t>(R_ACT), ws.at<int32_t>(R_NACT),
                                           max_act, z, s),
                   "down");
  }
  if (rc || (rc = join())) return rc;
  return hip_check(k3moe::launch_combine(T, d, k, z, gates, ws.at<int32_t>(R_PPOS), resid,
                                         shared, y, y_bf16, s),
                   "combine");
}

}  // namespace

extern "C" {

int k3moe_version(void) { return K3MOE_VERSION; }

int k3moe_time_next_kernel(int which, void* ev_start, void* ev_stop) {
  if (which != K3MOE_KERNEL_ROUTER && which != K3MOE_KERNEL_GATE_UP && which != K3MOE_KERNEL_DOWN)
    return fail(K3MOE_EINVAL, "unknown kernel id %d", which);
  if (!ev_start || !ev_stop) {
    g_probe_which = 0;
    return K3MOE_OK;
  }
  g_probe_which = which;
  g_probe_start = (hipEvent_t)ev_start;
  g_probe_stop = (hipEvent_t)ev_stop;
  return K3MOE_OK;
}

const char* k3moe_last_error(void) { return g_err.c_str(); }

int k3moe_set_hot_tokens(int32_t hot_tokens) {
  if (!k3moe::set_hot_tokens(hot_tokens))
    return fail(K3MOE_EINVAL, "hot_tokens must be in [0, 16] (got %d)", (int)hot_tokens);
  return K3MOE_OK;
}

int32_t k3moe_hot_tokens(void) { return k3moe::hot_tokens(); }

int k3moe_release(void) {
  if (!g_created.load()) return K3MOE_OK;
  int cur = 0;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  int rc = K3MOE_OK;
  auto note = [&](hipError_t e, const char* what) {
    if (e != hipSuccess && rc == K3MOE_OK) rc = hip_check(e, what);
  };
  {
    std::lock_guard<std::mutex> lock(g_obj_mu);
    for (int dev = 0; dev < kMaxDev; ++dev) {
      hipStream_t* own[1 + kCopyStreams] = {&g_side[dev]};
      for (int i = 0; i < kCopyStreams; ++i) own[1 + i] = &g_copy[dev][i];
      bool any = false;
      for (hipStream_t* p : own) any = any || *p;
      for (hipEvent_t ev : t_fj[dev]) any = any || ev;
      for (hipEvent_t ev : t_cp[dev]) any = any || ev;
      if (!any) continue;
      note(hipSetDevice(dev), "release: set device");
      for (hipStream_t* p : own)
        if (*p) {
          note(hipStreamSynchronize(*p), "release: synchronize stream");
          note(hipStreamDestroy(*p), "release: destroy stream");
          *p = nullptr;
        }
      for (hipEvent_t& ev : t_fj[dev])
        if (ev) {
          note(hipEventDestroy(ev), "release: destroy event");
          ev = nullptr;
        }
      for (hipEvent_t& ev : t_cp[dev])
        if (ev) {
          note(hipEventDestroy(ev), "release: destroy event");
          ev = nullptr;
        }
    }
  }
  if (have_cur) note(hipSetDevice(cur), "release: restore device");
  return rc;
}

size_t k3moe_workspace_bytes(const k3moe_dims* dims, int32_t max_tokens) {
  if (check_dims(dims) || max_tokens < 0 || max_tokens > kMaxT) return 0;
  return layout_for(*dims, max_tokens < 1 ? 1 : max_tokens).total;
}

int k3moe_router(const k3moe_dims* dims, int32_t T, const void* x, int x_dtype,
                 const uint16_t* w_router, const float* logit_bias, int32_t* topk_ids,
                 float* topk_gates, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_T(T)) || (rc = check_dtype(x_dtype))) return rc;
  if (T == 0) return K3MOE_OK;
  if ((rc = need_ptr(x, "x", true)) || (rc = need_ptr(w_router, "w_router")) ||
      (rc = need_ptr(topk_ids, "topk_ids")) || (rc = need_ptr(topk_gates, "topk_gates")))
    return rc;
  Ws w;
  if ((rc = get_ws(*dims, T, ws, ws_bytes, &w))) return rc;
  return run_router(*dims, T, x, x_dtype == K3MOE_F32, w_router, logit_bias, topk_ids,
                    topk_gates, w, (hipStream_t)stream);
}

int k3moe_route_bucket(const k3moe_dims* dims, int32_t T, const int32_t* topk_ids,
                       int32_t* expert_offsets, int32_t* bucket_rows, void* ws, size_t ws_bytes,
                       void* stream) {
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_T(T))) return rc;
  if (T == 0) return K3MOE_OK;
  if ((rc = need_ptr(topk_ids, "topk_ids")) || (rc = need_ptr(expert_offsets, "expert_offsets")) ||
      (rc = need_ptr(bucket_rows, "bucket_rows")))
    return rc;
  Ws w;
  if ((rc = get_ws(*dims, T, ws, ws_bytes, &w))) return rc;
  return hip_check(k3moe::launch_bucket(T, dims->n_experts, dims->top_k, topk_ids,
                                        bucket_out(w, expert_offsets, bucket_rows),
                                        w.at<uint32_t>(R_HIST), w.at<uint32_t>(R_BASE),
                                        w.at<uint64_t>(R_MASK), (hipStream_t)stream),
                   "bucket");
}

int k3moe_expert_ffn(const k3moe_dims* dims, int32_t T, const void* x, int x_dtype,
                     const k3moe_mx_experts* experts, const int32_t* expert_offsets,
                     const int32_t* bucket_rows, const float* topk_gates, float* y, void* ws,
                     size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_T(T)) || (rc = check_dtype(x_dtype))) return rc;
  if (T == 0) return K3MOE_OK;
  if ((rc = check_expert_shape(*dims))) return rc;
  if ((rc = need_ptr(x, "x", true)) || (rc = check_experts(experts)) ||
      (rc = need_ptr(expert_offsets, "expert_offsets")) ||
      (rc = need_ptr(bucket_rows, "bucket_rows")) || (rc = need_ptr(topk_gates, "topk_gates")) ||
      (rc = need_ptr(y, "y", true)))
    return rc;
  Ws w;
  if ((rc = get_ws(*dims, T, ws, ws_bytes, &w))) return rc;
  hipStream_t s = (hipStream_t)stream;
  const k3moe::BucketOut o = bucket_out(w, const_cast<int32_t*>(expert_offsets),
                                        const_cast<int32_t*>(bucket_rows));
  rc = hip_check(k3moe::launch_pairs_from_bucket(T, dims->n_experts, dims->top_k,
                                                 expert_offsets, bucket_rows, o, s),
                 "bucket index");
  if (rc) return rc;
  return run_ffn(*dims, T, x, x_dtype == K3MOE_F32, experts, expert_offsets, bucket_rows,
                 topk_gates, nullptr, nullptr, y, nullptr, w, s);
}

size_t k3moe_cache_state_bytes(int32_t n_experts, int32_t n_slots, int32_t max_ids) {
  return k3moe::cache_state_bytes(n_experts, n_slots, max_ids);
}

int k3moe_cache_init(void* state, size_t state_bytes, int32_t n_experts, int32_t n_slots,
                     int32_t max_ids) {
  const int r = k3moe::cache_init(state, state_bytes, n_experts, n_slots, max_ids);
  if (r == -3)
    return fail(K3MOE_EWORKSPACE, "cache state of %zu bytes < %zu needed", state_bytes,
                k3moe::cache_state_bytes(n_experts, n_slots, max_ids));
  if (r)
    return fail(K3MOE_EINVAL,
                "cache init: need 1 <= n_slots=%d <= n_experts=%d, max_ids=%d >= 1 and an "
                "8-byte aligned state",
                n_slots, n_experts, max_ids);
  return K3MOE_OK;
}

int k3moe_cache_plan(void* state, int32_t n_ids, const int32_t* ids, int32_t* slot_ids,
                     int32_t* fetch, int32_t* n_fetch) {
  k3moe::CacheView v = k3moe::cache_view(state);
  if (!v.h) return fail(K3MOE_EINVAL, "state is not an initialised cache state");
  if (n_ids < 0) return fail(K3MOE_EINVAL, "n_ids=%d is negative", n_ids);
  if (n_ids > 0 && (!ids || !slot_ids || !fetch)) return fail(K3MOE_EINVAL, "NULL array");
  if (!n_fetch) return fail(K3MOE_EINVAL, "n_fetch is NULL");
  int32_t nd = 0;
  const int r = k3moe::cache_plan(v, n_ids, ids, slot_ids, fetch, n_fetch, &nd);
  if (r == -1) return fail(K3MOE_EINVAL, "an id is outside [0, %d)", v.h->n_experts);
  if (r == -2)
    return fail(K3MOE_EUNSUPPORTED, "%d distinct experts in one call, more than the %d slots", nd,
                v.h->n_slots);
  return K3MOE_OK;
}

int k3moe_cache_stats_get(const void* state, k3moe_cache_stats* out) {
  k3moe::CacheView v = k3moe::cache_view(const_cast<void*>(state));
  if (!v.h) return fail(K3MOE_EINVAL, "state is not an initialised cache state");
  if (!out) return fail(K3MOE_EINVAL, "out is NULL");
  out->hits = v.h->hits;
  out->misses = v.h->misses;
  out->bytes_copied = v.h->bytes;
  out->distinct = 0;
  return K3MOE_OK;
}

int k3moe_layer_forward_cached(const k3moe_dims* dims, int32_t T, const void* x, int x_dtype,
                               const uint16_t* w_router, const float* logit_bias,
                               const k3moe_mx_experts* host_experts,
                               const k3moe_mx_experts* slot_experts, void* state, float* y,
                               uint16_t* y_bf16, int32_t* topk_ids, float* topk_gates,
                               k3moe_cache_stats* call_stats, void* ws, size_t ws_bytes,
                               void* stream) {
  int rc;
  if (call_stats) *call_stats = k3moe_cache_stats{0, 0, 0, 0};
  if ((rc = check_dims(dims)) || (rc = check_T(T)) || (rc = check_dtype(x_dtype))) return rc;
  if (T == 0) return K3MOE_OK;
  if ((rc = check_expert_shape(*dims))) return rc;
  if ((rc = need_ptr(x, "x", true)) || (rc = need_ptr(w_router, "w_router")) ||
      (rc = check_experts(host_experts)) || (rc = check_experts(slot_experts)) ||
      (rc = need_ptr(y, "y", true)))
    return rc;
  k3moe::CacheView cv = k3moe::cache_view(state);
  if (!cv.h) return fail(K3MOE_EINVAL, "state is not an initialised cache state");
  if (cv.h->n_experts != dims->n_experts)
    return fail(K3MOE_EINVAL, "cache state has %d experts, dims %d", cv.h->n_experts,
                dims->n_experts);
  const int k = dims->top_k, C = cv.h->n_slots;
  const int64_t P = (int64_t)T * k;
  if (P > cv.h->max_ids)
    return fail(K3MOE_EUNSUPPORTED, "T*top_k=%lld above the state's max_ids=%d", (long long)P,
                cv.h->max_ids);
  if (k > C) return fail(K3MOE_EUNSUPPORTED, "top_k=%d above n_slots=%d", k, C);
  Ws w;
  if ((rc = get_ws(*dims, T, ws, ws_bytes, &w))) return rc;
  hipStream_t s = (hipStream_t)stream;
  int32_t* ids = topk_ids ? topk_ids : w.at<int32_t>(R_IDS);
  float* gates = topk_gates ? topk_gates : w.at<float>(R_GATES);
  const int xf32 = x_dtype == K3MOE_F32;
  if ((rc = run_router(*dims, T, x, xf32, w_router, logit_bias, ids, gates, w, s))) return rc;
  // the plan needs the routed ids on the host
  if ((rc = hip_check(hipMemcpyAsync(cv.ids, ids, (size_t)P * 4, hipMemcpyDeviceToHost, s),
                      "routed ids to host")) ||
      (rc = hip_check(hipStreamSynchronize(s), "routed ids to host")))
    return rc;
  int32_t nf = 0, nd = 0;
  const int pr = k3moe::cache_plan(cv, (int32_t)P, cv.ids, cv.slots, cv.fetch, &nf, &nd);
  if (pr == -1) return fail(K3MOE_EINVAL, "a routed id is outside [0, %d)", dims->n_experts);
  if (pr == -2)
    return fail(K3MOE_EUNSUPPORTED, "%d distinct experts in one call, more than the %d slots", nd,
                C);
  const size_t d = (size_t)dims->d_model, f = (size_t)dims->d_ff;
  const size_t nq_gu = f * d / 2, ns_gu = f * d / 32, nq_d = d * f / 2, ns_d = d * f / 32;
  const size_t sizes[6] = {nq_gu, ns_gu, nq_gu, ns_gu, nq_d, ns_d};
  const uint8_t* src[6] = {host_experts->gate_q, host_experts->gate_s, host_experts->up_q,
                           host_experts->up_s, host_experts->down_q, host_experts->down_s};
  const uint8_t* dst[6] = {slot_experts->gate_q, slot_experts->gate_s, slot_experts->up_q,
                           slot_experts->up_s, slot_experts->down_q, slot_experts->down_s};
  // missing experts round-robin over the copy streams (forked from and joined back into
  // `s` by events; in order on `s` if they cannot be set up)
  hipStream_t cs[kCopyStreams];
  hipEvent_t fork = nullptr, join[kCopyStreams];
  const int ncs = nf > 1 && copy_streams(cs, fork, join) ? (nf < kCopyStreams ? nf : kCopyStreams)
                                                          : 0;
  if (ncs) {
    if ((rc = hip_check(hipEventRecord(fork, s), "fork expert copies"))) return rc;
    for (int j = 0; j < ncs; ++j)
      if ((rc = hip_check(hipStreamWaitEvent(cs[j], fork, 0), "fork expert copies"))) return rc;
  }
  size_t bytes = 0;
  for (int32_t i = 0; i < nf; ++i) {
    const size_t e = (size_t)cv.fetch[2 * i], sl = (size_t)cv.fetch[2 * i + 1];
    hipStream_t cps = ncs ? cs[i % ncs] : s;
    for (int a = 0; a < 6; ++a) {
      rc = hip_check(hipMemcpyAsync(const_cast<uint8_t*>(dst[a]) + sl * sizes[a],
                                    src[a] + e * sizes[a], sizes[a], hipMemcpyHostToDevice, cps),
                     "expert to its slot");
      if (rc) return rc;
      bytes += sizes[a];
    }
  }
  for (int j = 0; j < ncs; ++j)
    if ((rc = hip_check(hipEventRecord(join[j], cs[j]), "join expert copies")) ||
        (rc = hip_check(hipStreamWaitEvent(s, join[j], 0), "join expert copies")))
      return rc;
  cv.h->bytes += (int64_t)bytes;
  int32_t* sids = w.at<int32_t>(R_SIDS);
  if ((rc = hip_check(hipMemcpyAsync(sids, cv.slots, (size_t)P * 4, hipMemcpyHostToDevice, s),
                      "slot ids to device")))
    return rc;
  k3moe_dims dc = *dims;
  dc.n_experts = C;
  int32_t* offs = w.at<int32_t>(R_OFFS);
  int32_t* rows = w.at<int32_t>(R_ROWS);
  const k3moe::BucketOut bo = bucket_out(w, offs, rows);
  rc = hip_check(k3moe::launch_bucket(T, C, k, sids, bo, w.at<uint32_t>(R_HIST),
                                      w.at<uint32_t>(R_BASE), w.at<uint64_t>(R_MASK), s),
                 "bucket by slot");
  if (rc) return rc;
  if (call_stats) *call_stats = k3moe_cache_stats{nd - nf, nf, (int64_t)bytes, nd};
  return run_ffn(dc, T, x, xf32, slot_experts, offs, rows, gates, nullptr, nullptr, y, y_bf16, w,
                 s);
}

}  // extern "C"

namespace {

// Host-side checks of a whole-layer call (everything but the workspace).
int check_layer(const k3moe_dims* dims, int32_t T, const void* x, int x_dtype,
                const uint16_t* w_router, const k3moe_mx_experts* experts, const k3moe_block* blk,
                const float* y) {
  int rc;
  if ((rc = check_dims(dims)) || (rc = check_T(T)) || (rc = check_dtype(x_dtype))) return rc;
  if (T == 0) return K3MOE_OK;
  if ((rc = check_expert_shape(*dims))) return rc;
  if ((rc = need_ptr(x, "x", true)) || (rc = need_ptr(w_router, "w_router")) ||
      (rc = check_experts(experts)) || (rc = need_ptr(y, "y", true)))
    return rc;
  if (blk) {
    if (x_dtype != K3MOE_F32) return fail(K3MOE_EINVAL, "block mode needs an fp32 residual x");
    if ((rc = need_ptr(blk->rms_gamma, "blk->rms_gamma")) ||
        (rc = need_ptr(blk->sh_gate, "blk->sh_gate", true)) ||
        (rc = need_ptr(blk->sh_up, "blk->sh_up", true)) ||
        (rc = need_ptr(blk->sh_down, "blk->sh_down", true)))
      return rc;
    if (!(blk->rms_eps >= 0.0f)) return fail(K3MOE_EINVAL, "rms_eps must be >= 0");
  }
  return K3MOE_OK;
}

// One token on the packed layout runs the one-token kernels, which also take fp32 tokens
// (and so block mode, whose RMSNorm output is fp32).
bool packed_one_token(const k3moe_dims& dm, int32_t T) {
  return T == 1 && k3moe::down_decode_mfma_supported(dm.d_model, dm.d_ff, dm.top_k);
}

// The layer on a carved workspace. side_ok: block mode's shared expert may run on the
// library's side stream (created on first use); otherwise it runs in order on `s` (same
// kernels, same buffers, so the same results bit for bit).
int run_layer(const k3moe_dims* dims, int32_t T, const void* x, int x_dtype,
              const uint16_t* w_router, const float* logit_bias, const k3moe_mx_experts* experts,
              const k3moe_block* blk, float* y, uint16_t* y_bf16, int32_t* topk_ids,
              float* topk_gates, const Ws& w, hipStream_t s, bool side_ok,
              bool packed = false) {
  int rc;
  const int d = dims->d_model;
  int32_t* ids = topk_ids ? topk_ids : w.at<int32_t>(R_IDS);
  float* gates = topk_gates ? topk_gates : w.at<float>(R_GATES);
  const void* xin = x;
  int xf32 = x_dtype == K3MOE_F32;
  int32_t* offs = w.at<int32_t>(R_OFFS);
  int32_t* rows = w.at<int32_t>(R_ROWS);
  const k3moe::BucketOut bo = bucket_out(w, offs, rows);
  // One token: the RMSNorm and the shared expert's two GEMVs ride in the router and top-k
  // launches (which also write the token's bucket), all on `s`.
  if (blk && T == 1 &&
      k3moe::route_shared_supported(d, dims->n_experts, dims->top_k, w_router)) {
    float* xhat = w.at<float>(R_XHAT);
    float* ssh = w.at<float>(R_SSH);
    if (packed && packed_one_token(*dims, T)) {
      // packed experts: the shared gate/up rides with the top-k, the shared down with the
      // expert gate/up
      {
        Probe probe(K3MOE_KERNEL_ROUTER, s);
        rc = hip_check(k3moe::launch_route_norm_shared_gateup(
                           d, dims->d_ff, dims->n_experts, dims->top_k,
                           static_cast<const float*>(x), blk->rms_gamma, blk->rms_eps, xhat,
                           w_router, logit_bias, w.at<double>(R_PART), blk->sh_gate,
                           blk->sh_up, w.at<float>(R_HSH), ids, gates, bo, s),
                       "rmsnorm + router, top-k + shared gate/up");
      }
      if (rc) return rc;
      const k3moe::SharedDown sdn{w.at<float>(R_HSH), blk->sh_down, ssh};
      return run_ffn(*dims, T, xhat, 1, experts, offs, rows, gates,
                     static_cast<const float*>(x), ssh, y, y_bf16, w, s, nullptr, packed, &sdn);
    }
    {
      Probe probe(K3MOE_KERNEL_ROUTER, s);
      rc = hip_check(k3moe::launch_route_shared(
                         d, dims->d_ff, dims->n_experts, dims->top_k,
                         static_cast<const float*>(x), blk->rms_gamma, blk->rms_eps, xhat,
                         w_router, logit_bias, w.at<double>(R_PART), blk->sh_gate, blk->sh_up,
                         blk->sh_down, w.at<float>(R_HSH), ssh, ids, gates, bo, 0, s),
                     "rmsnorm + router + shared expert");
    }
    if (rc) return rc;
    return run_ffn(*dims, T, xhat, 1, experts, offs, rows, gates, static_cast<const float*>(x),
                   ssh, y, y_bf16, w, s, nullptr, packed);
  }
  if (blk) {
    float* xhat = w.at<float>(R_XHAT);
    rc = hip_check(k3moe::launch_rmsnorm(T, d, static_cast<const float*>(x), blk->rms_gamma,
                                         blk->rms_eps, xhat, s),
                   "rmsnorm");
    if (rc) return rc;
    xin = xhat;
    xf32 = 1;
  }
  // The shared expert needs only xhat: it runs on a side stream, overlapping the router,
  // top-k and gate/up, and the launch that adds it into y waits for it (per-call events).
  const float* resid = nullptr;
  const float* shared = nullptr;
  hipEvent_t fork = nullptr, joined = nullptr;
  if (blk) {
    float* ssh = w.at<float>(R_SSH);
    hipStream_t s2 = side_ok ? side_stream() : nullptr;
    if (s2 && !fork_join_events(fork, joined))
      s2 = nullptr;  // no side stream: the shared expert runs in order on `s`
    if (s2) {
      if ((rc = hip_check(hipEventRecord(fork, s), "fork shared expert")) ||
          (rc = hip_check(hipStreamWaitEvent(s2, fork, 0), "fork shared expert")))
        return rc;
    }
    // beside the routed path each shared-expert GEMV runs one block per CU (it has until the
    // down launch to finish), so the latency-bound router and top-k find room on every CU:
    // at d = 7168 the 8-block stack took 0.749 ms per token so, 0.76-0.80 ms with one block
    // per row group (384 and 448 blocks), 0.80 ms with 128 blocks and 0.96 ms with 64
    rc = hip_check(k3moe::launch_dense_swiglu(T, d, dims->d_ff, static_cast<const float*>(xin),
                                              blk->sh_gate, blk->sh_up, blk->sh_down,
                                              w.at<float>(R_HSH), ssh, s2 ? s2 : s,
                                              s2 ? cu_count() : 0),
                   "shared expert");
    if (rc) return rc;
    if (s2 && (rc = hip_check(hipEventRecord(joined, s2), "join shared expert"))) return rc;
    if (!s2) joined = nullptr;
    resid = static_cast<const float*>(x);
    shared = ssh;
  }
  // a single token's bucket is written by the top-k kernel itself
  if ((rc = run_router(*dims, T, xin, xf32, w_router, logit_bias, ids, gates, w, s,
                       T == 1 ? &bo : nullptr)))
    return rc;
  if (T > 1) {
    rc = hip_check(k3moe::launch_bucket(T, dims->n_experts, dims->top_k, ids, bo,
                                        w.at<uint32_t>(R_HIST), w.at<uint32_t>(R_BASE),
                                        w.at<uint64_t>(R_MASK), s),
                   "bucket");
    if (rc) return rc;
  }
  return run_ffn(*dims, T, xin, xf32, experts, offs, rows, gates, resid, shared, y, y_bf16, w, s,
                 joined, packed);
}

// Shapes and activations the packed-layout kernels take (packed_one_token above).

int check_packed(const k3moe_dims& dm, int32_t T, int x_dtype) {
  if (!k3moe::packed_shape_supported(dm.d_model, dm.d_ff))
    return fail(K3MOE_EUNSUPPORTED,
                "packed layout needs d_model %% 1024 == 0 and d_ff %% 512 == 0 (d_model=%d, "
                "d_ff=%d)",
                dm.d_model, dm.d_ff);
  if (x_dtype != K3MOE_BF16 && !packed_one_token(dm, T))
    return fail(K3MOE_EUNSUPPORTED,
                "the packed-layout kernels take bf16 activations (fp32 only for one token)");
  return K3MOE_OK;
}


}  // namespace

// Scratch of the allocation-free entry point, one copy per device (each GPU the library runs
// on holds it until the process ends). In host code this name is not a device address: the
// address comes from hipGetSymbolAddress, once per device (scratch_on_device).
static __device__ __align__(256) uint8_t scratch[K3MOE_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` on the current device, looked up by the first call made with
// that device current and kept; nullptr (message set) if the lookup fails.
void* scratch_on_device() {
  static std::mutex mu;
  static void* addr[kMaxDev] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    fail(K3MOE_EHIP, "no current HIP device");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      fail(K3MOE_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      return nullptr;
    }
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace

extern "C" {

int k3moe_layer_forward(const k3moe_dims* dims, int32_t T, const void* x, int x_dtype,
                        const uint16_t* w_router, const float* logit_bias,
                        const k3moe_mx_experts* experts, const k3moe_block* blk, float* y,
                        uint16_t* y_bf16, int32_t* topk_ids, float* topk_gates, void* ws,
                        size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_layer(dims, T, x, x_dtype, w_router, experts, blk, y))) return rc;
  if (T == 0) return K3MOE_OK;
  Ws w;
  if ((rc = get_ws(*dims, T, ws, ws_bytes, &w))) return rc;
  return run_layer(dims, T, x, x_dtype, w_router, logit_bias, experts, blk, y, y_bf16, topk_ids,
                   topk_gates, w, (hipStream_t)stream, true);
}

int k3moe_packed_expert_bytes(const k3moe_dims* dims, k3moe_packed_bytes* per_expert) {
  int rc;
  if ((rc = check_dims(dims))) return rc;
  if (!per_expert) return fail(K3MOE_EINVAL, "per_expert is NULL");
  if ((rc = check_packed(*dims, 1, K3MOE_BF16))) return rc;
  const size_t d = (size_t)dims->d_model, f = (size_t)dims->d_ff;
  per_expert->gate_q = per_expert->up_q = f * d / 2;
  per_expert->down_q = d * f / 2;
  per_expert->gate_s = per_expert->up_s = k3moe::packed_scale_bytes((int)f, (int)d);
  per_expert->down_s = k3moe::packed_scale_bytes((int)d, (int)f);
  return K3MOE_OK;
}

int k3moe_pack_experts(const k3moe_dims* dims, const k3moe_mx_experts* src,
                       const k3moe_mx_experts* dst, void* stream) {
  int rc;
  k3moe_packed_bytes pb;
  if ((rc = k3moe_packed_expert_bytes(dims, &pb))) return rc;
  if ((rc = check_experts(src)) || (rc = check_experts(dst))) return rc;
  if ((reinterpret_cast<uintptr_t>(dst->gate_s) | reinterpret_cast<uintptr_t>(dst->up_s) |
       reinterpret_cast<uintptr_t>(dst->down_s)) & 7u)
    return fail(K3MOE_EINVAL, "packed scale arrays must be 8-byte aligned");
  const int d = dims->d_model, f = dims->d_ff, E = dims->n_experts;
  hipStream_t s = (hipStream_t)stream;
  if ((rc = hip_check(k3moe::launch_pack_matrix(f, d, E, src->gate_q, src->gate_s,
                                                const_cast<uint8_t*>(dst->gate_q),
                                                const_cast<uint8_t*>(dst->gate_s), s),
                      "pack gate")) ||
      (rc = hip_check(k3moe::launch_pack_matrix(f, d, E, src->up_q, src->up_s,
                                                const_cast<uint8_t*>(dst->up_q),
                                                const_cast<uint8_t*>(dst->up_s), s),
                      "pack up")))
    return rc;
  return hip_check(k3moe::launch_pack_matrix(d, f, E, src->down_q, src->down_s,
                                             const_cast<uint8_t*>(dst->down_q),
                                             const_cast<uint8_t*>(dst->down_s), s),
                   "pack down");
}

int k3moe_layer_forward_packed(const k3moe_dims* dims, int32_t T, const void* x, int x_dtype,
                               const uint16_t* w_router, const float* logit_bias,
                               const k3moe_mx_experts* experts, const k3moe_block* blk, float* y,
                               uint16_t* y_bf16, int32_t* topk_ids, float* topk_gates, void* ws,
                               size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_layer(dims, T, x, x_dtype, w_router, experts, blk, y))) return rc;
  if (T == 0) return K3MOE_OK;
  // block mode feeds the experts the fp32 RMSNorm output
  if ((rc = check_packed(*dims, T, blk ? K3MOE_F32 : x_dtype))) return rc;
  if (((reinterpret_cast<uintptr_t>(experts->gate_s) | reinterpret_cast<uintptr_t>(experts->up_s) |
        reinterpret_cast<uintptr_t>(experts->down_s)) & 7u))
    return fail(K3MOE_EINVAL, "packed scale arrays must be 8-byte aligned");
  Ws w;
  if ((rc = get_ws(*dims, T, ws, ws_bytes, &w))) return rc;
  return run_layer(dims, T, x, x_dtype, w_router, logit_bias, experts, blk, y, y_bf16, topk_ids,
                   topk_gates, w, (hipStream_t)stream, true, true);
}

int k3moe_layer_forward_noalloc(const k3moe_dims* dims, int32_t T, const void* x, int x_dtype,
                                const uint16_t* w_router, const float* logit_bias,
                                const k3moe_mx_experts* experts, const k3moe_block* blk,
                                float* y, uint16_t* y_bf16, int32_t* topk_ids,
                                float* topk_gates, void* stream) {
  int rc;
  if ((rc = check_layer(dims, T, x, x_dtype, w_router, experts, blk, y))) return rc;
  if (T == 0) return K3MOE_OK;
  Ws w;
  w.L = layout_for(*dims, T);
  if (w.L.total > (size_t)K3MOE_NOALLOC_SCRATCH_BYTES)
    return fail(K3MOE_EUNSUPPORTED,
                "T=%d needs %zu bytes of scratch, above the %zu bytes of the allocation-free "
                "entry point's static scratch (k3moe_layer_forward takes a workspace instead)",
                T, w.L.total, (size_t)K3MOE_NOALLOC_SCRATCH_BYTES);
  void* base = scratch_on_device();
  if (!base) return K3MOE_EHIP;
  w.base = static_cast<char*>(base);  // 256-byte aligned
  return run_layer(dims, T, x, x_dtype, w_router, logit_bias, experts, blk, y, y_bf16, topk_ids,
                   topk_gates, w, (hipStream_t)stream, false);
}

}  // extern "C"
