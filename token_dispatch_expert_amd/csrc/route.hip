// Top-k expert selection and gate weights, one wavefront per token.
//
// Operation: "Expert Parallelism" tutorial page, section 4 (router output: each token's
// experts) and section 1 (each token goes to k of E experts). Readings taken where the page
// is silent: selection on the fp32 logits; descending order; equal logits go to the lower
// expert index (+0.0 == -0.0 under float comparison); gates are the softmax over the k
// chosen logits, computed relative to the largest one.
//
// Layout: lane L of the wave holds experts L, L+64, L+128, ... (coalesced row load); the
// selection is the wave-level top-k of topk_wave.h.
#include <math.h>

#include "topk_wave.h"

namespace moe {

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int n, int32_t value) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = value;
}

hipError_t launch_fill_i32(int32_t* p, int n, int32_t value, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  fill_i32_kernel<<<(n + 255) / 256, 256, 0, stream>>>(p, n, value);
  return hipGetLastError();
}

// EPL = experts per lane (ceil(E / 64)).
template <int EPL>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int T,
                                                    int E, int k, int32_t* __restrict__ ids,
                                                    float* __restrict__ gates,
                                                    int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (t >= T) return;  // uniform per wave

  const float* row = logits + (size_t)t * E;
  float v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    v[i] = e < E ? row[e] : 0.0f;
  }
  float slot_val;
  int slot_id;
  wave_topk<EPL>(v, E, k, slot_val, slot_id);
  write_topk(slot_val, slot_id, k, (size_t)t, ids, gates, counts);
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* gates,
                        int32_t* counts, hipStream_t stream) {
  if (counts) {
    hipError_t st = launch_fill_i32(counts, E, 0, stream);
    if (st != hipSuccess) return st;
  }
  if (T == 0) return hipSuccess;
  const int tokens_per_block = 256 / kWave;
  dim3 grid((T + tokens_per_block - 1) / tokens_per_block), block(256);
  if (E <= 64)
    route_kernel<1><<<grid, block, 0, stream>>>(logits, T, E, k, ids, gates, counts);
  else if (E <= 128)
    route_kernel<2><<<grid, block, 0, stream>>>(logits, T, E, k, ids, gates, counts);
  else if (E <= 256)
    route_kernel<4><<<grid, block, 0, stream>>>(logits, T, E, k, ids, gates, counts);
  else if (E <= 512)
    route_kernel<8><<<grid, block, 0, stream>>>(logits, T, E, k, ids, gates, counts);
  else
    route_kernel<16><<<grid, block, 0, stream>>>(logits, T, E, k, ids, gates, counts);
  return hipGetLastError();
}

}  // namespace moe
