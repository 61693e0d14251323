// Internal declarations shared by the HIP kernels and the C ABI host code (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---------------------------------------------------------------------------------------
// vector types used for MFMA operands and 16-byte memory moves
// ---------------------------------------------------------------------------------------
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));  // plain 16-byte load/store

constexpr int kWave = 64;

// Permutation tiles: flat assignments are processed in tiles of this many entries.
constexpr int kPermuteTile = 256;

// Grouped-FFN streaming kernel geometry (see ffn.hip).
constexpr int kStreamWaves = 4;     // waves per workgroup; they split the contraction axis
constexpr int kStreamMFrags = 4;    // 16-row MFMA fragments per item -> up to 64 rows
constexpr int kStreamRows = 16 * kStreamMFrags;

struct DeviceInfo {
  int device = -1;
  int num_cus = 0;
};

// Queried once per device, cached (mutex-guarded) in api.cpp.
hipError_t device_info(DeviceInfo* out);

// A second stream that runs work beside the caller's stream inside one call, with the events
// that fork it from and join it back to the caller's stream. One per (device, caller stream),
// created on first use (default priority, non-blocking; also during a graph capture, with this
// thread's capture mode relaxed for the creation) and kept until the process ends. Returns
// false when it cannot be created (the caller then runs everything on its own stream).
struct SideStream {
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
bool side_stream_for(hipStream_t caller, SideStream* out);

// ---------------------------------------------------------------------------------------
// launchers (each enqueues on `stream` and returns the launch status)
// ---------------------------------------------------------------------------------------
hipError_t launch_fill_i32(int32_t* p, int n, int32_t value, hipStream_t stream);

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* gates,
                        int32_t* counts, hipStream_t stream);

// fused router GEMM + top-k: bf16 x [T, d] and w_router [E, d], E <= kRouterMaxExperts,
// d a multiple of 32; logits (nullable) receives the fp32 logits [T, E]
// Batches of at most kRouterSplitMaxT tokens split the contraction over several workgroups and
// need route_gemm_workspace_bytes of workspace (fp32 partial logits); larger ones need none.
constexpr int kRouterMaxExperts = 256;
constexpr int kRouterSplitMaxT = 1024;
size_t route_gemm_workspace_bytes(int T, int E);
hipError_t launch_route_gemm(const void* x, const void* w_router, int T, int E, int k, int d,
                             float* logits, int32_t* ids, float* gates, int32_t* counts,
                             void* workspace, hipStream_t stream);

// workspace: n_tiles * E int32 (per-tile histograms, then per-tile bases)
size_t permute_workspace_ints(int T, int E, int k);
// cap: most kept assignments per expert (INT_MAX: no capacity limit)
hipError_t launch_permute(const void* x, int elem_bytes, const int32_t* ids, int T, int E, int k,
                          int d, int cap, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_to_flat, int32_t* flat_to_sorted, void* x_sorted,
                          int32_t* ws, hipStream_t stream);

// No-allocation permutation: the device address of this GPU's static scratch array of
// kStaticPermuteInts int32 (looked up once per device, with that device current, and cached).
constexpr size_t kStaticPermuteInts = size_t(1) << 20;  // 4 MiB
hipError_t permute_static_scratch(int32_t** out);

struct FfnArgs {
  const void* x_sorted;
  moe_dtype_t act;
  const int32_t* offsets;
  int rows, E, d, d_ff;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  moe_dtype_t wdt;
  const float* s_gate;
  const float* s_up;
  const float* s_down;
  float* y_sorted;
  void* h;  // [rows, d_ff] in act dtype (workspace)
};
size_t ffn_workspace_bytes(int rows, int E, int d, int d_ff, moe_dtype_t act, moe_dtype_t wdt);
// [E, N, row_bytes] row-major -> [E][N/8][row_bytes/128][8][128 bytes] (N % 8 == 0,
// row_bytes % 128 == 0): the blocked weight layouts
hipError_t launch_block_weights(const void* src, void* dst, int E, int N, long long row_bytes,
                                hipStream_t stream);
hipError_t launch_grouped_ffn(const FfnArgs& a, const DeviceInfo& dev, hipStream_t stream);

hipError_t launch_combine(const float* y_sorted, const int32_t* flat_to_sorted,
                          const float* gates, int T, int k, int d, void* y, bool bf16_out,
                          hipStream_t stream);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace moe
