// Wave-level top-k over a row of E values (one wavefront per row), shared by the router
// kernels. Lane L holds values L, L+64, L+128, ...; each of the k rounds takes every lane's
// best unchosen candidate and reduces it across the wave under the total order (value desc,
// index asc): DPP moves combine lanes inside each 16-lane row (xor 1, xor 2, half-row mirror,
// row mirror), then the four row winners are read with readlane and compared in scalar
// registers, so every lane agrees on the winner without LDS traffic or a barrier. Slot j's
// result ends up in lane j.
#pragma once

#include <math.h>

#include "moe_internal.h"

namespace moe {

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

// v[i] holds the value of index lane + 64*i (valid when < E). On return lane j < k holds
// slot j: its value and index.
template <int EPL>
__device__ __forceinline__ void wave_topk(const float (&v)[EPL], int E, int k, float& slot_val,
                                          int& slot_id) {
  const int lane = threadIdx.x & (kWave - 1);
  unsigned taken = 0;  // bit i set: index lane + 64*i already chosen
  slot_val = 0.0f;
  slot_id = 0;
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
    if (lane == (wi & (kWave - 1))) taken |= 1u << (wi / kWave);
    if (lane == j) {
      slot_val = wv;
      slot_id = wi;
    }
  }
}

// Gates of the k chosen values (softmax over them relative to the largest, slot 0) and the
// stores of row t's ids, gates and (optionally) per-index counts.
__device__ __forceinline__ void write_topk(float slot_val, int slot_id, int k, size_t t,
                                           int32_t* __restrict__ ids, float* __restrict__ gates,
                                           int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & (kWave - 1);
  const float top = __shfl(slot_val, 0);
  const float ex = lane < k ? expf(slot_val - top) : 0.0f;
  float sum = ex;
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
  if (lane < k) {
    ids[t * k + lane] = slot_id;
    gates[t * k + lane] = ex / sum;
    if (counts) atomicAdd(&counts[slot_id], 1);
  }
}

}  // namespace moe
