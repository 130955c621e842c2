// C ABI of the prefill attention library: argument validation, launch planning,
// status codes and optional kernel timing. Every entry point validates on the
// host before touching the GPU; on an error nothing is enqueued. There is no
// fallback path: a request the kernels cannot serve is refused with a status.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/prefill_attn.h"
#include "common.h"

namespace {

// Longest key range of the dense entry points: the workgroup keeps two flag bits
// per 64-key step in LDS after its K/V rings (128 KB), within the 160 KB of a CU.
constexpr int PA_MAX_T = (1 << 22) - 4096;

thread_local std::string g_last_hip_error;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return PA_OK;
  g_last_hip_error = hipGetErrorString(e);
  return PA_EHIP;
}

bool aligned16(const void* p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool pow2_block(int b) { return b >= 16 && b <= 256 && (b & (b - 1)) == 0; }
bool good_scale(float s) { return std::isfinite(s) && s > 0.f; }

// ---------------------------------------------------------------- timing
struct TimedKernel {
  const char* name;
  double total_ms = 0.0;
  int64_t launches = 0;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending;
};

std::mutex g_timing_mu;
bool g_timing_on = false;
TimedKernel g_timed[] = {{"attn_dense"}, {"attn_blocksparse"}, {"mask_classify"}, {"stage_values"},
                         {"attn_combine"}, {"pool"}, {"select"}, {"fold"}, {"attn_gather"}};
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

TimedKernel* find_timed(const char* name) {
  for (auto& t : g_timed)
    if (std::strcmp(t.name, name) == 0) return &t;
  return nullptr;
}

// Runs `launch` on `stream`, bracketed by events when timing is on (and the
// caller allows it: the allocation-free entry point never creates events).
template <class F>
hipError_t timed(const char* name, hipStream_t stream, F&& launch, bool allow = true) {
  hipEvent_t a = nullptr, b = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_timing_mu);
    if (g_timing_on && allow) {
      a = take_event();
      b = take_event();
    }
  }
  if ((a != nullptr) != (b != nullptr)) {   // only one event could be had: time nothing
    std::lock_guard<std::mutex> lk(g_timing_mu);
    if (a) g_event_pool.push_back(a);
    if (b) g_event_pool.push_back(b);
    a = b = nullptr;
  }
  if (a && b) {
    hipError_t e = hipEventRecord(a, stream);
    if (e != hipSuccess) {
      std::lock_guard<std::mutex> lk(g_timing_mu);
      g_event_pool.push_back(a);
      g_event_pool.push_back(b);
      return e;
    }
  }
  hipError_t err = launch();
  if (a && b) {
    if (err == hipSuccess) err = hipEventRecord(b, stream);
    std::lock_guard<std::mutex> lk(g_timing_mu);
    if (err == hipSuccess) find_timed(name)->pending.emplace_back(a, b);
    else { g_event_pool.push_back(a); g_event_pool.push_back(b); }
  }
  return err;
}

// The dense entry points after their own argument checks: size limits, the
// workspace, then mask-tile flags (if any), value staging, attention and (when
// the key range is split) the combine, all on `s`.
enum DenseKind { DENSE_F16_MASK, DENSE_BITS, DENSE_CAUSAL };

int enqueue_dense(DenseKind kind, const uint16_t* Q, int C, int n_q, const uint16_t* K, const uint16_t* V,
                  int T, int n_kv, int d, const void* mask, int64_t mask_ld, int q_start, float scale, float* O,
                  void* workspace, size_t workspace_bytes, hipStream_t s, bool allow_timing = true) {
  auto timed = [&](const char* name, hipStream_t st, auto&& launch) {
    return ::timed(name, st, launch, allow_timing);
  };
  if (d != 64 && d != 128) return PA_EUNSUPPORTED;
  if (T > PA_MAX_T) return PA_EUNSUPPORTED;   // the per-tile flag row must fit in LDS
  const pa::DensePlan plan = pa::plan_dense(C, T, n_q, n_kv, d);
  if ((long long)plan.n_qt * n_q * plan.splits >= (1LL << 31)) return PA_EUNSUPPORTED;
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
      workspace_bytes < plan.total_bytes)
    return PA_EWORKSPACE;
  uint8_t* flags = static_cast<uint8_t*>(workspace);
  float* part_o = plan.splits > 1 ? reinterpret_cast<float*>(flags + plan.flags_bytes) : nullptr;
  float* part_ml =
      plan.splits > 1 ? reinterpret_cast<float*>(flags + plan.flags_bytes + plan.part_o_bytes) : nullptr;
  uint8_t* stage = flags + plan.stage_off;
  const uint16_t* V16 = reinterpret_cast<const uint16_t*>(stage + plan.stage.v16_off);
  const float* vscales = reinterpret_cast<const float*>(stage + plan.stage.scales_off);
  const uint16_t* m16 = static_cast<const uint16_t*>(mask);
  hipError_t e = hipSuccess;
  if (kind == DENSE_F16_MASK) {
    e = timed("mask_classify", s, [&] { return pa::launch_mask_classify(m16, mask_ld, C, T, flags, s); });
  } else if (kind == DENSE_BITS) {
    e = timed("mask_classify", s, [&] {
      return pa::launch_mask_classify_bits(static_cast<const uint32_t*>(mask), mask_ld, C, T, flags, s);
    });
  } else if (mask != nullptr) {   // one-row classification of the per-key mask's 64-key tiles
    e = timed("mask_classify", s, [&] {
      return pa::launch_mask_classify(m16, ((int64_t)T + 7) / 8 * 8, 1, T, flags, s);
    });
  }
  if (e != hipSuccess) return hip_status(e);
  e = timed("stage_values", s, [&] { return pa::launch_stage_values(V, T, n_kv, d, stage, s); });
  if (e != hipSuccess) return hip_status(e);
  e = timed("attn_dense", s, [&] {
    if (kind == DENSE_CAUSAL)
      return pa::launch_attn_dense(Q, C, n_q, K, V16, vscales, T, n_kv, d, m16, T, scale, O, plan,
                                   mask != nullptr ? flags : nullptr, part_o, part_ml, q_start, s);
    return pa::launch_attn_dense(Q, C, n_q, K, V16, vscales, T, n_kv, d, m16, mask_ld, scale, O, plan, flags,
                                 part_o, part_ml, -1, s, kind == DENSE_BITS);
  });
  if (e != hipSuccess) return hip_status(e);
  if (plan.splits > 1) {
    e = timed("attn_combine", s, [&] {
      return pa::launch_attn_combine(C, n_q, d, plan.splits, part_o, part_ml, O, s);
    });
    if (e != hipSuccess) return hip_status(e);
  }
  return PA_OK;
}

// ---------------------------------------------------------------- allocation-free scratch
// Device memory for prefill_attn_dense_noalloc: what prefill_attn_dense takes as
// its workspace (tile flags, split partials, staged fp16 values). Each GPU the
// library runs on holds its own copy for the life of the process. In host code
// `scratch` names a host-side stand-in, not device memory: only the address
// hipGetSymbolAddress returns for the current device is ever used.
static __device__ __align__(256) uint8_t scratch[PA_NOALLOC_SCRATCH_BYTES];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;   // per device id; null until looked up

// The current device's copy of `scratch`, looked up once per device with that
// device current (nullptr and the HIP error on failure).
void* device_scratch(hipError_t* err) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) { *err = e; return nullptr; }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize(dev + 1, nullptr);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) { *err = e != hipSuccess ? e : hipErrorInvalidSymbol; return nullptr; }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_EINVAL: return "invalid argument";
    case PA_EUNSUPPORTED: return "unsupported size or parameter";
    case PA_EWORKSPACE: return "workspace missing or too small";
    case PA_ESCRATCH: return "sizes need more scratch than the allocation-free entry point's static array holds";
    case PA_EHIP: {
      thread_local std::string msg;
      msg = "HIP runtime error: " + g_last_hip_error;
      return msg.c_str();
    }
    default: return "unknown status";
  }
}

size_t prefill_attn_dense_workspace(int C, int T, int n_q, int n_kv, int d) {
  if (C < 1 || T < 1 || n_q < 1 || n_kv < 1 || n_q % n_kv || (d != 64 && d != 128)) return 0;
  return pa::plan_dense(C, T, n_q, n_kv, d).total_bytes;
}

int prefill_attn_dense(const uint16_t* Q, int C, int n_q, const uint16_t* K, const uint16_t* V,
                       int T, int n_kv, int d, const uint16_t* mask, int64_t mask_ld, float scale,
                       float* O, void* workspace, size_t workspace_bytes, void* stream) {
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(mask) || !aligned16(O))
    return PA_EINVAL;
  if (C < 1 || T < 1 || n_q < 1 || n_kv < 1 || n_q % n_kv != 0) return PA_EINVAL;
  if (mask_ld < T || !good_scale(scale)) return PA_EINVAL;
  return enqueue_dense(DENSE_F16_MASK, Q, C, n_q, K, V, T, n_kv, d, mask, mask_ld, -1, scale, O, workspace,
                       workspace_bytes, static_cast<hipStream_t>(stream));
}

int prefill_attn_dense_noalloc(const uint16_t* Q, int C, int n_q, const uint16_t* K, const uint16_t* V,
                               int T, int n_kv, int d, const uint16_t* mask, int64_t mask_ld, float scale,
                               float* O, void* stream) {
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(mask) || !aligned16(O))
    return PA_EINVAL;
  if (C < 1 || T < 1 || n_q < 1 || n_kv < 1 || n_q % n_kv != 0) return PA_EINVAL;
  if (mask_ld < T || !good_scale(scale)) return PA_EINVAL;
  if (d != 64 && d != 128) return PA_EUNSUPPORTED;
  if (T > PA_MAX_T) return PA_EUNSUPPORTED;
  if (pa::plan_dense(C, T, n_q, n_kv, d).total_bytes > PA_NOALLOC_SCRATCH_BYTES) return PA_ESCRATCH;
  hipError_t e = hipSuccess;
  void* ws = device_scratch(&e);
  if (ws == nullptr) return hip_status(e);
  return enqueue_dense(DENSE_F16_MASK, Q, C, n_q, K, V, T, n_kv, d, mask, mask_ld, -1, scale, O, ws,
                       PA_NOALLOC_SCRATCH_BYTES, static_cast<hipStream_t>(stream), false);
}

size_t prefill_attn_dense_noalloc_limit(void) { return PA_NOALLOC_SCRATCH_BYTES; }

int prefill_attn_dense_bits(const uint16_t* Q, int C, int n_q, const uint16_t* K, const uint16_t* V,
                            int T, int n_kv, int d, const uint32_t* mask_bits, int64_t bits_ld,
                            float scale, float* O, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(mask_bits) || !aligned16(O))
    return PA_EINVAL;
  if (C < 1 || T < 1 || n_q < 1 || n_kv < 1 || n_q % n_kv != 0) return PA_EINVAL;
  if (bits_ld < ((int64_t)T + 31) / 32 || !good_scale(scale)) return PA_EINVAL;
  return enqueue_dense(DENSE_BITS, Q, C, n_q, K, V, T, n_kv, d, mask_bits, bits_ld, -1, scale, O, workspace,
                       workspace_bytes, static_cast<hipStream_t>(stream));
}

int prefill_attn_dense_causal(const uint16_t* Q, int C, int q_start, int n_q, const uint16_t* K,
                              const uint16_t* V, int T, int n_kv, int d, const uint16_t* kmask,
                              float scale, float* O, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return PA_EINVAL;
  if (kmask != nullptr && !aligned16(kmask)) return PA_EINVAL;
  if (C < 1 || q_start < 0 || n_q < 1 || n_kv < 1 || n_q % n_kv != 0) return PA_EINVAL;
  if ((long long)q_start + C > T || !good_scale(scale)) return PA_EINVAL;
  return enqueue_dense(DENSE_CAUSAL, Q, C, n_q, K, V, T, n_kv, d, kmask, T, q_start, scale, O, workspace,
                       workspace_bytes, static_cast<hipStream_t>(stream));
}

int fold_keep_mask(const int32_t* keep_idx, int64_t keep_ld, const int32_t* keep_cnt, int C,
                   int q_start, int T, int width, int recent, uint16_t* mask, int64_t mask_ld,
                   void* stream) {
  if (!aligned16(keep_cnt) || !aligned16(mask) || (keep_ld > 0 && !aligned16(keep_idx)))
    return PA_EINVAL;
  if (C < 1 || q_start < 0 || (long long)q_start + C > T || width < 1 || recent < 0 || keep_ld < 0)
    return PA_EINVAL;
  if (mask_ld < T) return PA_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(timed("fold", s, [&] {
    return pa::launch_fold_keep(keep_idx, keep_ld, keep_cnt, C, q_start, T, width, recent, mask,
                                mask_ld, s);
  }));
}

int fold_keep_bits(const int32_t* keep_idx, int64_t keep_ld, const int32_t* keep_cnt, int C, int q_start,
                   int T, int width, int recent, uint32_t* bits, int64_t bits_ld, void* stream) {
  if (!aligned16(keep_cnt) || !aligned16(bits) || (keep_ld > 0 && !aligned16(keep_idx))) return PA_EINVAL;
  if (C < 1 || q_start < 0 || (long long)q_start + C > T || width < 1 || recent < 0 || keep_ld < 0)
    return PA_EINVAL;
  if (bits_ld < ((long long)T + 31) / 32) return PA_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(timed("fold", s, [&] {
    return pa::launch_fold_keep_bits(keep_idx, keep_ld, keep_cnt, C, q_start, T, width, recent, bits, bits_ld,
                                     s);
  }));
}

int prefill_attn_gather(const uint16_t* Q, int C, int q_start, int n_q, const uint16_t* K,
                        const uint16_t* V, int T, int n_kv, int d, const int32_t* keep_idx,
                        int64_t keep_ld, const int32_t* keep_cnt, int width, int recent, float scale,
                        float* O, void* stream) {
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(keep_cnt) ||
      (keep_ld > 0 && !aligned16(keep_idx)))
    return PA_EINVAL;
  if (C < 1 || q_start < 0 || (long long)q_start + C > T || n_q < 1 || n_kv < 1 || n_q % n_kv != 0 ||
      width < 1 || recent < 0 || keep_ld < 0 || !good_scale(scale))
    return PA_EINVAL;
  if ((d != 64 && d != 128) || width > 64) return PA_EUNSUPPORTED;
  if ((long long)C * n_kv > (1LL << 30)) return PA_EUNSUPPORTED;
  const pa::GatherPlan pl = pa::plan_gather(T, keep_ld, width);
  if (pl.waves < 1) return PA_EUNSUPPORTED;   // one row's bitmap and list exceed the LDS
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(timed("attn_gather", s, [&] {
    return pa::launch_gather_attn(Q, C, q_start, n_q, K, V, T, n_kv, d, keep_idx, keep_ld, keep_cnt, width,
                                  recent, scale, O, pl, s);
  }));
}

int build_pooled_index_ld(const uint16_t* K, const uint16_t* V, int T, int n_kv, int d, int block,
                          int b_first, float* K_pool, float* V_pool, int pool_ld, void* stream) {
  if (!aligned16(K) || !aligned16(V) || !aligned16(K_pool) || !aligned16(V_pool)) return PA_EINVAL;
  if (T < 1 || n_kv < 1) return PA_EINVAL;
  if ((d != 64 && d != 128) || !pow2_block(block)) return PA_EUNSUPPORTED;
  const int nb = (T + block - 1) / block;
  if (b_first < 0 || b_first > nb || pool_ld < nb) return PA_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(timed("pool", s, [&] {
    return pa::launch_pool(K, V, T, n_kv, d, block, b_first, K_pool, V_pool, pool_ld, s);
  }));
}

int build_pooled_index(const uint16_t* K, const uint16_t* V, int T, int n_kv, int d, int block,
                       float* K_pool, float* V_pool, void* stream) {
  if (T < 1 || !pow2_block(block)) return T < 1 ? PA_EINVAL : PA_EUNSUPPORTED;
  return build_pooled_index_ld(K, V, T, n_kv, d, block, 0, K_pool, V_pool, (T + block - 1) / block,
                               stream);
}

int select_blocks_ld(const uint16_t* Q, int C, int q_start, int n_q, int n_kv, int d,
                     const float* K_pool, int pool_ld, int T, int block, float alpha, float scale,
                     int sink_tokens, int window_blocks, int dense_tail_blocks,
                     int32_t* sel_idx, int32_t* sel_cnt, void* stream) {
  if (!aligned16(Q) || !aligned16(K_pool) || !aligned16(sel_idx) || !aligned16(sel_cnt))
    return PA_EINVAL;
  if (C < 1 || q_start < 0 || n_q < 1 || n_kv < 1 || n_q % n_kv != 0) return PA_EINVAL;
  if ((long long)q_start + C != T) return PA_EINVAL;
  if (!std::isfinite(alpha) || alpha < 0.f || !good_scale(scale)) return PA_EINVAL;
  if ((d != 64 && d != 128) || !pow2_block(block)) return PA_EUNSUPPORTED;
  const int nb = (T + block - 1) / block;
  if (nb > 8192) return PA_EUNSUPPORTED;
  if (pool_ld < nb) return PA_EINVAL;
  if (sink_tokens < 0 || window_blocks < 0 || dense_tail_blocks < 0) return PA_EINVAL;
  const int sink_blocks = (int)std::min<long long>(((long long)sink_tokens + block - 1) / block, nb);
  // theta = ln(alpha)/scale in fp64; alpha = 0 keeps every block
  const double theta = alpha == 0.f ? -HUGE_VAL : std::log((double)alpha) / (double)scale;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return hip_status(timed("select", s, [&] {
    return pa::launch_select(Q, C, q_start, n_q, n_kv, d, K_pool, pool_ld, T, block, theta,
                             sink_blocks, std::min(window_blocks, nb), std::min(dense_tail_blocks, nb),
                             sel_idx, sel_cnt, s);
  }));
}

int select_blocks(const uint16_t* Q, int C, int q_start, int n_q, int n_kv, int d,
                  const float* K_pool, int T, int block, float alpha, float scale,
                  int32_t* sel_idx, int32_t* sel_cnt, void* stream) {
  if (T < 1 || !pow2_block(block)) return T < 1 ? PA_EINVAL : PA_EUNSUPPORTED;
  return select_blocks_ld(Q, C, q_start, n_q, n_kv, d, K_pool, (T + block - 1) / block, T, block,
                          alpha, scale, 0, 0, 0, sel_idx, sel_cnt, stream);
}

// room for the pooled operands of the smallest block size (16)
static int pool_rows_max(int T) { return (T + 15) / 16; }

size_t prefill_attn_blocksparse_workspace(int T, int n_kv, int d) {
  if (T < 1 || n_kv < 1 || (d != 64 && d != 128)) return 0;
  return pa::plan_stage(T, n_kv, d, pool_rows_max(T)).bytes;
}

int prefill_attn_blocksparse_ld(const uint16_t* Q, int C, int q_start, int n_q, const uint16_t* K,
                                const uint16_t* V, int T, int n_kv, int d, const float* K_pool,
                                const float* V_pool, int pool_ld, int block, const int32_t* sel_idx,
                                const int32_t* sel_cnt, float scale, float* O, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(K_pool) || !aligned16(V_pool) ||
      !aligned16(sel_idx) || !aligned16(sel_cnt) || !aligned16(O))
    return PA_EINVAL;
  if (C < 1 || q_start < 0 || n_q < 1 || n_kv < 1 || n_q % n_kv != 0) return PA_EINVAL;
  if ((long long)q_start + C != T || !good_scale(scale)) return PA_EINVAL;
  if ((d != 64 && d != 128) || !pow2_block(block)) return PA_EUNSUPPORTED;
  const int nb = (T + block - 1) / block;
  if (nb > 8192) return PA_EUNSUPPORTED;
  if (pool_ld < nb) return PA_EINVAL;
  const pa::StagePlan sp = pa::plan_stage(T, n_kv, d, pool_rows_max(T));
  if (workspace == nullptr || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 ||
      workspace_bytes < sp.bytes)
    return PA_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* stage = static_cast<uint8_t*>(workspace);
  // the staged values, then the pooled operands (scaled by the values' factor)
  hipError_t e = timed("stage_values", s, [&] {
    const hipError_t e1 = pa::launch_stage_values(V, T, n_kv, d, stage, s);
    if (e1 != hipSuccess) return e1;
    return pa::launch_stage_pooled(K_pool, V_pool, pool_ld, nb, n_kv, d, stage, sp, s);
  });
  if (e != hipSuccess) return hip_status(e);
  const uint16_t* V16 = reinterpret_cast<const uint16_t*>(stage + sp.v16_off);
  const float* vscales = reinterpret_cast<const float*>(stage + sp.scales_off);
  const uint16_t* Kp16 = reinterpret_cast<const uint16_t*>(stage + sp.kp16_off);
  const uint16_t* Vp16 = reinterpret_cast<const uint16_t*>(stage + sp.vp16_off);
  return hip_status(timed("attn_blocksparse", s, [&] {
    return pa::launch_attn_blocksparse(Q, C, q_start, n_q, K, V16, vscales, T, n_kv, d, Kp16, Vp16, block,
                                       sel_idx, sel_cnt, scale, O, s);
  }));
}

int prefill_attn_blocksparse(const uint16_t* Q, int C, int q_start, int n_q, const uint16_t* K,
                             const uint16_t* V, int T, int n_kv, int d, const float* K_pool,
                             const float* V_pool, int block, const int32_t* sel_idx,
                             const int32_t* sel_cnt, float scale, float* O, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (T < 1 || block < 1) return PA_EINVAL;
  return prefill_attn_blocksparse_ld(Q, C, q_start, n_q, K, V, T, n_kv, d, K_pool, V_pool,
                                     (T + block - 1) / block, block, sel_idx, sel_cnt, scale, O,
                                     workspace, workspace_bytes, stream);
}

int pa_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_timing_on = on != 0;
  return PA_OK;
}

int pa_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  for (auto& t : g_timed) {
    for (auto& pr : t.pending) {
      hipEventSynchronize(pr.second);
      g_event_pool.push_back(pr.first);
      g_event_pool.push_back(pr.second);
    }
    t.pending.clear();
    t.total_ms = 0.0;
    t.launches = 0;
  }
  return PA_OK;
}

int pa_select_path_counts(int64_t* counts, int reset) {
  if (counts == nullptr) return PA_EINVAL;
  return hip_status(pa::select_path_counts(counts, reset != 0));
}

int pa_timing_read(const char* kernel, double* total_ms, int64_t* launches) {
  if (kernel == nullptr || total_ms == nullptr || launches == nullptr) return PA_EINVAL;
  std::lock_guard<std::mutex> lk(g_timing_mu);
  TimedKernel* t = find_timed(kernel);
  if (t == nullptr) return PA_EINVAL;
  // pairs are taken off the pending list as they are read, so an error leaves
  // only the unread ones pending and no event is both pooled and pending
  size_t done = 0;
  hipError_t err = hipSuccess;
  for (; done < t->pending.size(); ++done) {
    const auto& pr = t->pending[done];
    hipError_t e = hipEventSynchronize(pr.second);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pr.first, pr.second);
    if (e != hipSuccess) { err = e; break; }
    t->total_ms += ms;
    t->launches += 1;
    g_event_pool.push_back(pr.first);
    g_event_pool.push_back(pr.second);
  }
  t->pending.erase(t->pending.begin(), t->pending.begin() + done);
  if (err != hipSuccess) return hip_status(err);
  *total_ms = t->total_ms;
  *launches = t->launches;
  return PA_OK;
}

}  // extern "C"
