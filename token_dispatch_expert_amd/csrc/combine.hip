// Un-permute and gate-weighted combine, one workgroup per token.
//
// Operation: "Expert Parallelism" tutorial page, section 4, combine: results go back to the
// original token order and each token's k expert outputs are summed with their gate
// weights. Reading taken: fp32 sum in slot order j = 0..k-1 (no atomics, deterministic).
//
// HBM-bound: each token reads its k fp32 rows of y_sorted (16-byte vectors, coalesced across
// the workgroup) and writes one fp32 row. The row indices and gates are uniform per
// workgroup, so they come through scalar loads.
#include "moe_internal.h"

namespace moe {

__global__ __launch_bounds__(256) void combine_kernel(const float4* __restrict__ ys,
                                                      const int32_t* __restrict__ f2s,
                                                      const float* __restrict__ gates, int k,
                                                      int vec_per_row, int R,
                                                      float4* __restrict__ y) {
  const int t = blockIdx.x;
  const int32_t* pos = f2s + (size_t)t * k;
  const float* g = gates + (size_t)t * k;
  for (int v = threadIdx.x; v < vec_per_row; v += blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const int p = pos[j];
      if ((unsigned)p >= (unsigned)R) continue;  // corrupt map: never read out of bounds
      const float w = g[j];
      const float4 r = ys[(size_t)p * vec_per_row + v];
      acc.x = fmaf(w, r.x, acc.x);
      acc.y = fmaf(w, r.y, acc.y);
      acc.z = fmaf(w, r.z, acc.z);
      acc.w = fmaf(w, r.w, acc.w);
    }
    y[(size_t)t * vec_per_row + v] = acc;
  }
}

hipError_t launch_combine(const float* y_sorted, const int32_t* flat_to_sorted,
                          const float* gates, int T, int k, int d, float* y, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const int vpr = d / 4;
  const int threads = vpr >= 256 ? 256 : ((vpr + kWave - 1) / kWave) * kWave;
  combine_kernel<<<T, threads, 0, stream>>>(reinterpret_cast<const float4*>(y_sorted),
                                            flat_to_sorted, gates, k, vpr, T * k,
                                            reinterpret_cast<float4*>(y));
  return hipGetLastError();
}

}  // namespace moe
