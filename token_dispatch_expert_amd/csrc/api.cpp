// C ABI of the MoE layer library (declared in include/moe.h).
//
// Every entry point validates all of its arguments on the host before it makes any HIP call,
// so an invalid call returns a status without touching the device or enqueuing anything.
// Valid calls only enqueue kernels on the caller's stream: no allocation, no synchronisation.
// The only library state is a per-device cache of the compute-unit count.
#include <climits>
#include <mutex>
#include <vector>

#include "moe_internal.h"

namespace moe {

hipError_t device_info(DeviceInfo* out) {
  static std::mutex mu;
  static DeviceInfo cache[64];
  int dev = 0;
  hipError_t st = hipGetDevice(&dev);
  if (st != hipSuccess) return st;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev].device != dev) {
    int cus = 0;
    st = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (st != hipSuccess) return st;
    cache[dev].num_cus = cus > 0 ? cus : 1;
    cache[dev].device = dev;
  }
  *out = cache[dev];
  return hipSuccess;
}

constexpr size_t kMaxSideStreams = 64;  // (device, caller stream) pairs with a second stream

bool side_stream_for(hipStream_t caller, SideStream* out) {
  static std::mutex mu;
  struct Entry { int dev; hipStream_t caller; SideStream side; };
  static std::vector<Entry> table;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry& en : table)
    if (en.dev == dev && en.caller == caller) {
      *out = en.side;
      return true;
    }
  // The table is never pruned (a caller stream may be destroyed and its handle reused), so it
  // is bounded: past kMaxSideStreams pairs a call takes the one-stream schedule instead.
  if (table.size() >= kMaxSideStreams) return false;
  // Creating a stream and events is allowed while a graph is being captured once this thread's
  // capture mode is relaxed (the documented way to make such calls during a capture); the
  // previous mode is restored afterwards.
  hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
  if (hipThreadExchangeStreamCaptureMode(&mode) != hipSuccess) return false;
  SideStream side;
  bool ok = hipStreamCreateWithFlags(&side.stream, hipStreamNonBlocking) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&side.fork, hipEventDisableTiming) == hipSuccess;
  ok = ok && hipEventCreateWithFlags(&side.join, hipEventDisableTiming) == hipSuccess;
  if (!ok) {
    if (side.fork) (void)hipEventDestroy(side.fork);
    if (side.stream) (void)hipStreamDestroy(side.stream);
  }
  (void)hipThreadExchangeStreamCaptureMode(&mode);
  if (!ok) return false;
  table.push_back(Entry{dev, caller, side});
  *out = side;
  return true;
}

}  // namespace moe

namespace {

using moe::align_up;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// A pointer to `count` elements: NULL is allowed only for an empty array.
bool ok_ptr(const void* p, long long count, size_t align) {
  if (count == 0) return p == nullptr || aligned(p, align);
  return p != nullptr && aligned(p, align);
}

moe_status_t check_sizes(int T, int E, int k) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if ((long long)T * k > INT_MAX) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

constexpr int kMaxDim = 1 << 20;

int act_bytes(moe_dtype_t dt) { return dt == MOE_F32 ? 4 : 2; }

moe_status_t check_route(const float* logits, int T, int E, int k, const int32_t* ids,
                         const float* gates, const int32_t* counts) {
  moe_status_t s = check_sizes(T, E, k);
  if (s != MOE_OK) return s;
  const long long R = (long long)T * k;
  if (!ok_ptr(logits, (long long)T * E, 4) || !ok_ptr(ids, R, 4) || !ok_ptr(gates, R, 4))
    return MOE_ERR_INVALID_ARG;
  if (counts && !aligned(counts, 4)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status_t check_permute_io(const void* x, moe_dtype_t x_dt, const int32_t* ids, int T, int E,
                              int k, int d, const int32_t* counts, const int32_t* offsets,
                              const int32_t* s2f, const int32_t* f2s, const void* x_sorted) {
  moe_status_t s = check_sizes(T, E, k);
  if (s != MOE_OK) return s;
  if (d < 1 || d > kMaxDim) return MOE_ERR_INVALID_ARG;
  if (x_dt != MOE_F32 && x_dt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if ((d * act_bytes(x_dt)) % 16 != 0) return MOE_ERR_UNSUPPORTED;
  const long long R = (long long)T * k;
  if (!ok_ptr(x, (long long)T * d, 16) || !ok_ptr(ids, R, 4) || !ok_ptr(counts, E, 4) ||
      !ok_ptr(offsets, E + 1, 4) || !ok_ptr(s2f, R, 4) || !ok_ptr(f2s, R, 4) ||
      !ok_ptr(x_sorted, R * d, 16))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status_t check_permute(const void* x, moe_dtype_t x_dt, const int32_t* ids, int T, int E,
                           int k, int d, const int32_t* counts, const int32_t* offsets,
                           const int32_t* s2f, const int32_t* f2s, const void* x_sorted,
                           const void* ws, size_t ws_bytes) {
  moe_status_t s = check_permute_io(x, x_dt, ids, T, E, k, d, counts, offsets, s2f, f2s, x_sorted);
  if (s != MOE_OK) return s;
  const size_t need = moe_permute_workspace_size(T, E, k);
  if (need > 0 && (ws == nullptr || !aligned(ws, 16) || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

moe_status_t check_ffn(const void* x_sorted, moe_dtype_t act, const int32_t* offsets, int rows,
                       int E, int d, int d_ff, const void* wg, const void* wu, const void* wd,
                       moe_dtype_t wdt, const float* sg, const float* su, const float* sd,
                       const float* y_sorted, const void* ws, size_t ws_bytes) {
  if (rows < 0 || E < 1 || d < 1 || d_ff < 1 || d > kMaxDim || d_ff > kMaxDim)
    return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
  if (act == MOE_F32) {
    if (wdt != MOE_F32) return MOE_ERR_UNSUPPORTED;
  } else if (act == MOE_BF16) {
    if (wdt != MOE_BF16 && wdt != MOE_FP8_E4M3FN && wdt != MOE_BF16_BLOCKED &&
        wdt != MOE_FP8_E4M3FN_BLOCKED)
      return MOE_ERR_UNSUPPORTED;
  } else {
    return MOE_ERR_UNSUPPORTED;
  }
  const bool fp8 = wdt == MOE_FP8_E4M3FN || wdt == MOE_FP8_E4M3FN_BLOCKED;
  const int mult = fp8 ? 128 : (wdt == MOE_BF16_BLOCKED ? 64 : 8);
  // blocked fp8 runs on the direct-to-LDS tiles only, which stage scales for contractions up to this
  if (wdt == MOE_FP8_E4M3FN_BLOCKED && (d > 65536 || d_ff > 65536)) return MOE_ERR_UNSUPPORTED;
  if (d % mult != 0 || d_ff % mult != 0) return MOE_ERR_UNSUPPORTED;
  const long long wel = (long long)E * d * d_ff;
  if (!ok_ptr(x_sorted, (long long)rows * d, 16) || !ok_ptr(offsets, E + 1, 4) ||
      !ok_ptr(wg, wel, 16) || !ok_ptr(wu, wel, 16) || !ok_ptr(wd, wel, 16) ||
      !ok_ptr(y_sorted, (long long)rows * d, 16))
    return MOE_ERR_INVALID_ARG;
  if (fp8) {
    const long long ns = (long long)E * (d / 128) * (d_ff / 128);
    if (!ok_ptr(sg, ns, 4) || !ok_ptr(su, ns, 4) || !ok_ptr(sd, ns, 4)) return MOE_ERR_INVALID_ARG;
  } else if (sg || su || sd) {
    return MOE_ERR_INVALID_ARG;
  }
  const size_t need = moe_ffn_workspace_size(rows, E, d, d_ff, act, wdt);
  if (need > 0 && (ws == nullptr || !aligned(ws, 16) || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

moe_status_t check_combine(const float* y_sorted, const int32_t* f2s, const float* gates, int T,
                           int k, int d, const void* y, moe_dtype_t y_dtype) {
  if (T < 0 || k < 1 || k > MOE_MAX_TOPK || d < 1 || d > kMaxDim) return MOE_ERR_INVALID_ARG;
  if ((long long)T * k > INT_MAX) return MOE_ERR_INVALID_ARG;
  if (y_dtype != MOE_F32 && y_dtype != MOE_BF16 && y_dtype != MOE_FP8_E4M3FN) return MOE_ERR_INVALID_ARG;
  if (y_dtype == MOE_FP8_E4M3FN) return MOE_ERR_UNSUPPORTED;
  if (d % 4 != 0) return MOE_ERR_UNSUPPORTED;
  const long long R = (long long)T * k;
  if (!ok_ptr(y_sorted, R * d, 16) || !ok_ptr(f2s, R, 4) || !ok_ptr(gates, R, 4) ||
      !ok_ptr(y, (long long)T * d, 16))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape, dtype or limit";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

moe_status_t moe_route(const float* logits, int T, int E, int k, int32_t* topk_ids,
                       float* topk_gates, int32_t* counts, void* stream) {
  moe_status_t s = check_route(logits, T, E, k, topk_ids, topk_gates, counts);
  if (s != MOE_OK) return s;
  return hip_status(moe::launch_route(logits, T, E, k, topk_ids, topk_gates, counts,
                                      static_cast<hipStream_t>(stream)));
}

size_t moe_route_gemm_workspace_size(int T, int E, int k) {
  if (check_sizes(T, E, k) != MOE_OK || E > moe::kRouterMaxExperts) return 0;
  return moe::route_gemm_workspace_bytes(T, E);
}

moe_status_t moe_route_gemm(const void* x, moe_dtype_t x_dtype, const void* w_router,
                            moe_dtype_t w_dtype, int T, int E, int k, int d, float* logits,
                            int32_t* topk_ids, float* topk_gates, int32_t* counts,
                            void* workspace, size_t workspace_bytes, void* stream) {
  moe_status_t s = check_sizes(T, E, k);
  if (s != MOE_OK) return s;
  if (d < 1 || d > kMaxDim) return MOE_ERR_INVALID_ARG;
  if (x_dtype != MOE_BF16 || w_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (E > moe::kRouterMaxExperts || d % 32 != 0) return MOE_ERR_UNSUPPORTED;
  const long long R = (long long)T * k;
  if (!ok_ptr(x, (long long)T * d, 16) || !ok_ptr(w_router, (long long)E * d, 16) ||
      !ok_ptr(topk_ids, R, 4) || !ok_ptr(topk_gates, R, 4))
    return MOE_ERR_INVALID_ARG;
  if ((logits && !aligned(logits, 4)) || (counts && !aligned(counts, 4))) return MOE_ERR_INVALID_ARG;
  const size_t need = moe::route_gemm_workspace_bytes(T, E);
  if (need > 0 && (workspace == nullptr || !aligned(workspace, 16) || workspace_bytes < need))
    return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_route_gemm(x, w_router, T, E, k, d, logits, topk_ids, topk_gates,
                                           counts, workspace, static_cast<hipStream_t>(stream)));
}

size_t moe_permute_workspace_size(int T, int E, int k) {
  if (check_sizes(T, E, k) != MOE_OK) return 0;
  return align_up(moe::permute_workspace_ints(T, E, k) * sizeof(int32_t), 256);
}

moe_status_t moe_permute(const void* x, moe_dtype_t x_dtype, const int32_t* topk_ids, int T,
                         int E, int k, int d, int32_t* counts, int32_t* offsets,
                         int32_t* sorted_to_flat, int32_t* flat_to_sorted, void* x_sorted,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return moe_permute_capped(x, x_dtype, topk_ids, T, E, k, d, INT_MAX, counts, offsets,
                            sorted_to_flat, flat_to_sorted, x_sorted, workspace, workspace_bytes,
                            stream);
}

static_assert(moe::kStaticPermuteInts * sizeof(int32_t) == MOE_PERMUTE_NOALLOC_SCRATCH_BYTES,
              "the static scratch is the size the header states");

moe_status_t moe_permute_noalloc(const void* x, moe_dtype_t x_dtype, const int32_t* topk_ids,
                                 int T, int E, int k, int d, int32_t* counts, int32_t* offsets,
                                 int32_t* sorted_to_flat, int32_t* flat_to_sorted, void* x_sorted,
                                 void* stream) {
  moe_status_t s = check_permute_io(x, x_dtype, topk_ids, T, E, k, d, counts, offsets,
                                    sorted_to_flat, flat_to_sorted, x_sorted);
  if (s != MOE_OK) return s;
  // the per-tile counts must fit the static scratch (checked before any HIP call)
  if (moe_permute_workspace_size(T, E, k) > MOE_PERMUTE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  int32_t* scratch = nullptr;
  if (moe::permute_static_scratch(&scratch) != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_permute(x, act_bytes(x_dtype), topk_ids, T, E, k, d, INT_MAX,
                                        counts, offsets, sorted_to_flat, flat_to_sorted, x_sorted,
                                        scratch, static_cast<hipStream_t>(stream)));
}

int moe_expert_capacity(int T, int E, int k, int factor_percent) {
  if (T < 0 || E < 1 || k < 1 || factor_percent < 0) return -1;
  const long long num = (long long)factor_percent * T * k, den = 100LL * E;
  const long long cap = (num + den - 1) / den;
  return cap > INT_MAX ? INT_MAX : (int)cap;
}

moe_status_t moe_permute_capped(const void* x, moe_dtype_t x_dtype, const int32_t* topk_ids,
                                int T, int E, int k, int d, int capacity, int32_t* counts,
                                int32_t* offsets, int32_t* sorted_to_flat,
                                int32_t* flat_to_sorted, void* x_sorted, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (capacity < 0) return MOE_ERR_INVALID_ARG;
  moe_status_t s = check_permute(x, x_dtype, topk_ids, T, E, k, d, counts, offsets,
                                 sorted_to_flat, flat_to_sorted, x_sorted, workspace,
                                 workspace_bytes);
  if (s != MOE_OK) return s;
  return hip_status(moe::launch_permute(x, act_bytes(x_dtype), topk_ids, T, E, k, d, capacity,
                                        counts, offsets, sorted_to_flat, flat_to_sorted, x_sorted,
                                        static_cast<int32_t*>(workspace),
                                        static_cast<hipStream_t>(stream)));
}

size_t moe_ffn_workspace_size(int rows, int E, int d, int d_ff, moe_dtype_t act_dtype,
                              moe_dtype_t w_dtype) {
  if (rows < 0 || E < 1 || d < 1 || d_ff < 1 || d > kMaxDim || d_ff > kMaxDim) return 0;
  if (act_dtype != MOE_F32 && act_dtype != MOE_BF16) return 0;
  return moe::ffn_workspace_bytes(rows, E, d, d_ff, act_dtype, w_dtype);
}

moe_status_t moe_grouped_ffn(const void* x_sorted, moe_dtype_t act_dtype, const int32_t* offsets,
                             int rows, int E, int d, int d_ff, const void* w_gate,
                             const void* w_up, const void* w_down, moe_dtype_t w_dtype,
                             const float* s_gate, const float* s_up, const float* s_down,
                             float* y_sorted, void* workspace, size_t workspace_bytes,
                             void* stream) {
  moe_status_t s = check_ffn(x_sorted, act_dtype, offsets, rows, E, d, d_ff, w_gate, w_up, w_down,
                             w_dtype, s_gate, s_up, s_down, y_sorted, workspace, workspace_bytes);
  if (s != MOE_OK) return s;
  if (rows == 0) return MOE_OK;
  moe::DeviceInfo dev;
  hipError_t e = moe::device_info(&dev);
  if (e != hipSuccess) return MOE_ERR_HIP;
  moe::FfnArgs a{x_sorted, act_dtype, offsets, rows, E, d, d_ff, w_gate, w_up, w_down,
                 w_dtype, s_gate, s_up, s_down, y_sorted, workspace};
  return hip_status(moe::launch_grouped_ffn(a, dev, static_cast<hipStream_t>(stream)));
}

moe_status_t moe_block_weights(const void* src, void* dst, moe_dtype_t w_dtype, int E, int N, int K,
                               void* stream) {
  if (w_dtype != MOE_BF16 && w_dtype != MOE_FP8_E4M3FN) return MOE_ERR_UNSUPPORTED;
  const int esize = w_dtype == MOE_BF16 ? 2 : 1;
  const int B = 128 / esize;  // contraction elements per block row (128 bytes)
  if (E < 1 || N < 8 || K < B || N % 8 != 0 || K % B != 0) return MOE_ERR_INVALID_ARG;
  if ((long long)N * K * esize >= (1LL << 31)) return MOE_ERR_INVALID_ARG;  // one matrix under 2 GiB
  const long long n = (long long)E * N * K;
  if (n >= (1LL << 40)) return MOE_ERR_INVALID_ARG;
  if (!ok_ptr(src, n, 16) || !ok_ptr(dst, n, 16)) return MOE_ERR_INVALID_ARG;
  const char* s0 = static_cast<const char*>(src);
  const char* d0 = static_cast<const char*>(dst);
  if (s0 < d0 + esize * n && d0 < s0 + esize * n) return MOE_ERR_INVALID_ARG;  // overlap
  return hip_status(moe::launch_block_weights(src, dst, E, N, (long long)K * esize,
                                              static_cast<hipStream_t>(stream)));
}

moe_status_t moe_combine(const float* y_sorted, const int32_t* flat_to_sorted,
                         const float* topk_gates, int T, int k, int d, void* y,
                         moe_dtype_t y_dtype, void* stream) {
  moe_status_t s = check_combine(y_sorted, flat_to_sorted, topk_gates, T, k, d, y, y_dtype);
  if (s != MOE_OK) return s;
  return hip_status(moe::launch_combine(y_sorted, flat_to_sorted, topk_gates, T, k, d, y,
                                        y_dtype == MOE_BF16, static_cast<hipStream_t>(stream)));
}

size_t moe_layer_workspace_size(int T, int E, int k, int d, int d_ff, moe_dtype_t act_dtype,
                                moe_dtype_t w_dtype) {
  if (check_sizes(T, E, k) != MOE_OK) return 0;
  return moe_permute_workspace_size(T, E, k) +
         moe_ffn_workspace_size(T * k, E, d, d_ff, act_dtype, w_dtype);
}

moe_status_t moe_layer_capped(const float* logits, const void* x, moe_dtype_t act_dtype, int T,
                              int E, int k, int d, int d_ff, int capacity, const void* w_gate, const void* w_up,
                       const void* w_down, moe_dtype_t w_dtype, const float* s_gate,
                       const float* s_up, const float* s_down, int32_t* topk_ids,
                       float* topk_gates, int32_t* counts, int32_t* offsets,
                       int32_t* sorted_to_flat, int32_t* flat_to_sorted, void* x_sorted,
                       float* y_sorted, void* y, moe_dtype_t y_dtype, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (capacity < 0) return MOE_ERR_INVALID_ARG;
  moe_status_t s = check_route(logits, T, E, k, topk_ids, topk_gates, nullptr);
  if (s != MOE_OK) return s;
  const size_t ws_perm = moe_permute_workspace_size(T, E, k);
  const size_t ws_ffn = moe_ffn_workspace_size(T * k, E, d, d_ff, act_dtype, w_dtype);
  if (ws_perm + ws_ffn > 0 &&
      (workspace == nullptr || !aligned(workspace, 16) || workspace_bytes < ws_perm + ws_ffn))
    return MOE_ERR_WORKSPACE;
  char* wsb = static_cast<char*>(workspace);
  s = check_permute(x, act_dtype, topk_ids, T, E, k, d, counts, offsets, sorted_to_flat,
                    flat_to_sorted, x_sorted, wsb, ws_perm);
  if (s != MOE_OK) return s;
  s = check_ffn(x_sorted, act_dtype, offsets, T * k, E, d, d_ff, w_gate, w_up, w_down, w_dtype,
                s_gate, s_up, s_down, y_sorted, ws_ffn ? wsb + ws_perm : nullptr, ws_ffn);
  if (s != MOE_OK) return s;
  s = check_combine(y_sorted, flat_to_sorted, topk_gates, T, k, d, y, y_dtype);
  if (s != MOE_OK) return s;

  hipStream_t st = static_cast<hipStream_t>(stream);
  moe::DeviceInfo dev;
  if (moe::device_info(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (moe::launch_route(logits, T, E, k, topk_ids, topk_gates, nullptr, st) != hipSuccess)
    return MOE_ERR_HIP;
  if (moe::launch_permute(x, act_bytes(act_dtype), topk_ids, T, E, k, d, capacity, counts, offsets,
                          sorted_to_flat, flat_to_sorted, x_sorted,
                          reinterpret_cast<int32_t*>(wsb), st) != hipSuccess)
    return MOE_ERR_HIP;
  moe::FfnArgs a{x_sorted, act_dtype, offsets, T * k, E, d, d_ff, w_gate, w_up, w_down,
                 w_dtype, s_gate, s_up, s_down, y_sorted, wsb + ws_perm};
  if (moe::launch_grouped_ffn(a, dev, st) != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_combine(y_sorted, flat_to_sorted, topk_gates, T, k, d, y,
                                        y_dtype == MOE_BF16, st));
}

moe_status_t moe_layer(const float* logits, const void* x, moe_dtype_t act_dtype, int T, int E,
                       int k, int d, int d_ff, const void* w_gate, const void* w_up,
                       const void* w_down, moe_dtype_t w_dtype, const float* s_gate,
                       const float* s_up, const float* s_down, int32_t* topk_ids,
                       float* topk_gates, int32_t* counts, int32_t* offsets,
                       int32_t* sorted_to_flat, int32_t* flat_to_sorted, void* x_sorted,
                       float* y_sorted, void* y, moe_dtype_t y_dtype, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return moe_layer_capped(logits, x, act_dtype, T, E, k, d, d_ff, INT_MAX, w_gate, w_up, w_down,
                          w_dtype, s_gate, s_up, s_down, topk_ids, topk_gates, counts, offsets,
                          sorted_to_flat, flat_to_sorted, x_sorted, y_sorted, y, y_dtype,
                          workspace, workspace_bytes, stream);
}

}  // extern "C"
