// Top-k expert selection and gate weights, one wavefront per token.
//
// Operation: "Expert Parallelism" tutorial page, section 4 (router output: each token's
// experts) and section 1 (each token goes to k of E experts). Readings taken where the page
// is silent: selection on the fp32 logits; descending order; equal logits go to the lower
// expert index (+0.0 == -0.0 under float comparison); gates are the softmax over the k
// chosen logits, computed relative to the largest one.
//
// Layout: lane L of the wave holds experts L, L+64, L+128, ... (coalesced row load). Each of
// the k rounds takes every lane's best unchosen candidate and reduces it across the wave
// under the total order (value desc, index asc): DPP moves combine lanes inside each 16-lane
// row (xor 1, xor 2, half-row mirror, row mirror), then the four row winners are read with
// readlane and compared in scalar registers, so every lane agrees on the winner without LDS
// traffic or a barrier. Slot j's result stays in lane j.
#include <math.h>

#include "moe_internal.h"

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

constexpr int kNone = 0x7fffffff;

// (value, index) candidate order: a valid candidate beats none; larger value wins; equal values
// go to the lower index.
__device__ __forceinline__ bool better(float ov, int oi, float bv, int bi) {
  return oi != kNone && (bi == kNone || ov > bv || (ov == bv && oi < bi));
}

template <int CTRL>
__device__ __forceinline__ void dpp_step(float& bv, int& bi) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bv), CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(0, bi, CTRL, 0xF, 0xF, false);
  if (better(ov, oi, bv, bi)) {
    bv = ov;
    bi = oi;
  }
}

// DPP controls: quad_perm [1,0,3,2] (xor 1), quad_perm [2,3,0,1] (xor 2), row_half_mirror,
// row_mirror.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

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

  unsigned taken = 0;  // bit i set: expert lane + 64*i already chosen
  float slot_val = 0.0f;
  int slot_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = 0.0f;
    int bi = kNone;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + kWave * i;
      const bool free_ = e < E && !((taken >> i) & 1u);
      // strict '>' keeps the lowest index among this lane's equal candidates
      if (free_ && (bi == kNone || v[i] > bv)) {
        bv = v[i];
        bi = e;
      }
    }
    dpp_step<kDppXor1>(bv, bi);
    dpp_step<kDppXor2>(bv, bi);
    dpp_step<kDppHalfMirror>(bv, bi);
    dpp_step<kDppMirror>(bv, bi);
    // row winners sit in every lane of their row; combine rows 0..3 in scalar registers
    float wv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
    int wi = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
    for (int r = 1; r < 4; ++r) {
      const float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 16 * r));
      const int ri = __builtin_amdgcn_readlane(bi, 16 * r);
      if (better(rv, ri, wv, wi)) {
        wv = rv;
        wi = ri;
      }
    }
    bv = wv;
    bi = wi;
    if (lane == (bi & (kWave - 1))) taken |= 1u << (bi / kWave);
    if (lane == j) {
      slot_val = bv;
      slot_id = bi;
    }
  }

  const float top = __shfl(slot_val, 0);
  const float ex = lane < k ? expf(slot_val - top) : 0.0f;
  float sum = ex;
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    ids[(size_t)t * k + lane] = slot_id;
    gates[(size_t)t * k + lane] = ex / sum;
    if (counts) atomicAdd(&counts[slot_id], 1);
  }
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
