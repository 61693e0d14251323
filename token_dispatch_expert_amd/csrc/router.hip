// Router GEMM fused with top-k gating: logits[t, e] = sum_i x[t, i] * w_router[e, i] in fp32,
// then each token's top-k experts and gate weights, without a round trip of the logits through
// memory (they can still be written out for inspection).
//
// Operation: "Expert Parallelism" tutorial page, section 4: the router decides each token's
// destination experts, and section 1: each token goes to k of the E experts. The router's
// scores are the product of the token's hidden state with one weight row per expert (the
// linear gate the tutorial's router stands for). Readings: bf16 x and router weights, exact
// products accumulated in fp32; the selection and gates are those of moe_route on these fp32
// logits (ties to the lower expert index, softmax over the k chosen).
//
// One workgroup of 8 waves takes 16 tokens (32 for large batches) and every expert (E <= 256).
// The waves split the contraction axis (wave w takes the 32-wide steps w, w+8, ...); every lane
// loads its MFMA fragments straight from memory (16 bytes each: x rows and weight rows are
// contiguous along the contraction axis), so x is read once and the weights stream through L2.
// The eight partial tiles are added in LDS in a fixed order (waves w and w+4 into slot w, then
// the four slots in order: deterministic), then each wave runs the wave-level top-k on its
// tokens' rows.
#include "topk_wave.h"

namespace moe {

constexpr int kRouterWaves = 8;   // they split the contraction axis
constexpr int kRouterSplit = 16;  // contraction chunks per token tile for small batches
constexpr int kRouterSlots = 4;   // LDS partial tiles: waves w and w + 4 share slot w

// NF = ceil(E / 16) expert fragments, TMF 16-token fragments. DB: double-buffered loads (used
// where the registers allow it without spills). SPLIT > 0: the grid's y dimension splits the contraction into SPLIT
// chunks and the workgroup stores its partial TM x E tile to partials[chunk] instead of
// selecting (route_partials_topk_kernel finishes).
template <int NF, int TMF, bool DB, int SPLIT>
__global__ __launch_bounds__(kRouterWaves * kWave) void route_gemm_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ wr, int T, int E, int k, int d,
    float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ gates,
    int32_t* __restrict__ counts, float* __restrict__ partials) {
  constexpr int TM = 16 * TMF;       // tokens per workgroup
  constexpr int EPAD = NF * 16 + 4;  // LDS row stride (floats): rows 16 bytes apart in banks
  extern __shared__ float part[];    // [kRouterSlots][TM][EPAD]
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int t0 = blockIdx.x * TM;
  // contraction steps of this workgroup: all of them, or chunk blockIdx.y of SPLIT
  const int nall = d / 32;
  const int sbeg = SPLIT ? (int)((long long)nall * blockIdx.y / SPLIT) : 0;
  const int send = SPLIT ? (int)((long long)nall * (blockIdx.y + 1) / SPLIT) : nall;

  // fragment sources: lane -> row lane % 16 (token / expert), contraction offset (lane / 16) * 8
  const int r = lane & 15, kq = (lane >> 4) * 8;
  const __bf16* xa[TMF];
#pragma unroll
  for (int mf = 0; mf < TMF; ++mf) xa[mf] = x + (size_t)min(t0 + mf * 16 + r, T - 1) * d + kq;
  const __bf16* wb[NF];
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) wb[nf] = wr + (size_t)min(nf * 16 + r, E - 1) * d + kq;

  f32x4 acc[TMF][NF];
#pragma unroll
  for (int mf = 0; mf < TMF; ++mf)
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) acc[mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto load = [&](u32x4 (&av)[TMF], u32x4 (&bv)[NF], int s) __attribute__((always_inline)) {
    const size_t ko = (size_t)min(s, send - 1) * 32;  // clamped: loads stay in bounds
#pragma unroll
    for (int mf = 0; mf < TMF; ++mf) av[mf] = *reinterpret_cast<const u32x4*>(xa[mf] + ko);
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) bv[nf] = *reinterpret_cast<const u32x4*>(wb[nf] + ko);
  };
  auto compute = [&](const u32x4 (&av)[TMF], const u32x4 (&bv)[NF]) __attribute__((always_inline)) {
#pragma unroll
    for (int mf = 0; mf < TMF; ++mf) {
      bf16x8 a;
      __builtin_memcpy(&a, &av[mf], 16);
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) {
        bf16x8 b;
        __builtin_memcpy(&b, &bv[nf], 16);
        acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[mf][nf], 0, 0, 0);
      }
    }
  };
  if constexpr (DB) {
    // double buffer: the loads of this wave's next step go out before the MFMAs of the current
    // one; the scheduling barriers keep the compiler from sinking each load to its first use
    u32x4 a0[TMF], b0[NF], a1[TMF], b1[NF];
    if (sbeg + wave < send) load(a0, b0, sbeg + wave);
    for (int s = sbeg + wave; s < send; s += 2 * kRouterWaves) {
      load(a1, b1, s + kRouterWaves);
      __builtin_amdgcn_sched_barrier(0);
      compute(a0, b0);
      if (s + kRouterWaves >= send) break;  // uniform per wave
      load(a0, b0, s + 2 * kRouterWaves);
      __builtin_amdgcn_sched_barrier(0);
      compute(a1, b1);
    }
  } else {
#pragma unroll 2
    for (int s = sbeg + wave; s < send; s += kRouterWaves) {
      u32x4 av[TMF], bv[NF];
      load(av, bv, s);
      compute(av, bv);
    }
  }
  // partial tiles: waves 0..3 store into slots 0..3, then waves 4..7 add theirs (slot w - 4);
  // C fragment: lane holds rows (lane / 16) * 4 + j, column lane % 16
  float* slot = part + (size_t)(wave % kRouterSlots) * TM * EPAD;
  for (int round = 0; round < 2; ++round) {
    if (wave / kRouterSlots == round) {
#pragma unroll
      for (int mf = 0; mf < TMF; ++mf)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float* q = slot + (mf * 16 + (lane >> 4) * 4 + j) * EPAD + nf * 16 + r;
            *q = round == 0 ? acc[mf][nf][j] : *q + acc[mf][nf][j];
          }
    }
    __syncthreads();
  }
  // logits (or this chunk's partial) = ((s0 + s1) + s2) + s3, into slot 0
  for (int i = tid; i < TM * NF * 16; i += kRouterWaves * kWave) {
    const int row = i / (NF * 16), col = i % (NF * 16);
    float v = part[row * EPAD + col];
#pragma unroll
    for (int w = 1; w < kRouterSlots; ++w) v += part[((size_t)w * TM + row) * EPAD + col];
    part[row * EPAD + col] = v;
    if (col < E && t0 + row < T) {
      if (SPLIT) partials[((size_t)blockIdx.y * T + t0 + row) * E + col] = v;
      else if (logits) logits[(size_t)(t0 + row) * E + col] = v;
    }
  }
  if (SPLIT) return;  // uniform
  __syncthreads();
  constexpr int EPL = (NF * 16 + kWave - 1) / kWave;
  for (int row = wave; row < TM; row += kRouterWaves) {
    if (t0 + row >= T) break;  // uniform per wave
    float v[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane + kWave * i;
      v[i] = e < E ? part[row * EPAD + e] : 0.0f;
    }
    float slot_val;
    int slot_id;
    wave_topk<EPL>(v, E, k, slot_val, slot_id);
    write_topk(slot_val, slot_id, k, (size_t)(t0 + row), ids, gates, counts);
  }
}

// Small batches: the contraction chunks' partial logits [SPLIT][T][E] summed in chunk order
// (deterministic), then the wave-level top-k; one wave per token.
template <int EPL>
__global__ __launch_bounds__(256) void route_partials_topk_kernel(
    const float* __restrict__ partials, int split, int T, int E, int k, float* __restrict__ logits,
    int32_t* __restrict__ ids, float* __restrict__ gates, int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (t >= T) return;  // uniform per wave
  float v[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + kWave * i;
    float sum = 0.0f;
    if (e < E)
      for (int c = 0; c < split; ++c) sum += partials[((size_t)c * T + t) * E + e];
    v[i] = sum;
    if (logits && e < E) logits[(size_t)t * E + e] = sum;
  }
  float slot_val;
  int slot_id;
  wave_topk<EPL>(v, E, k, slot_val, slot_id);
  write_topk(slot_val, slot_id, k, (size_t)t, ids, gates, counts);
}

template <int NF, int TMF, bool DB, int SPLIT>
static hipError_t launch_route_gemm_nf(const void* x, const void* wr, int T, int E, int k, int d,
                                       float* logits, int32_t* ids, float* gates, int32_t* counts,
                                       float* partials, hipStream_t stream) {
  constexpr int TM = 16 * TMF;
  const size_t lds = (size_t)kRouterSlots * TM * (NF * 16 + 4) * sizeof(float);
  auto kern = &route_gemm_kernel<NF, TMF, DB, SPLIT>;
  if (lds > 64 * 1024) {
    hipError_t st = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (st != hipSuccess) return st;
  }
  dim3 grid((T + TM - 1) / TM, SPLIT ? SPLIT : 1);
  kern<<<grid, kRouterWaves * kWave, lds, stream>>>(static_cast<const __bf16*>(x),
                                                     static_cast<const __bf16*>(wr), T, E, k, d,
                                                     logits, ids, gates, counts, partials);
  if (!SPLIT) return hipGetLastError();
  hipError_t st = hipGetLastError();
  if (st != hipSuccess) return st;
  constexpr int EPL = (NF * 16 + kWave - 1) / kWave;
  route_partials_topk_kernel<EPL><<<(T + 3) / 4, 256, 0, stream>>>(partials, SPLIT, T, E, k,
                                                                    logits, ids, gates, counts);
  return hipGetLastError();
}

size_t route_gemm_workspace_bytes(int T, int E) {
  return T <= kRouterSplitMaxT ? align_up((size_t)kRouterSplit * T * E * sizeof(float), 256) : 0;
}

hipError_t launch_route_gemm(const void* x, const void* w_router, int T, int E, int k, int d,
                             float* logits, int32_t* ids, float* gates, int32_t* counts,
                             void* workspace, hipStream_t stream) {
  if (counts) {
    hipError_t st = launch_fill_i32(counts, E, 0, stream);
    if (st != hipSuccess) return st;
  }
  if (T == 0) return hipSuccess;
  float* ws = static_cast<float*>(workspace);
  // small batches: too few token tiles to fill the GPU, so the contraction is split over
  // kRouterSplit workgroups per tile; large ones: one fused pass, 32-token tiles once there are
  // enough of them (half the router-weight traffic through L2 per token)
  if (T <= kRouterSplitMaxT) {
    if (E <= 64) return launch_route_gemm_nf<4, 1, true, kRouterSplit>(x, w_router, T, E, k, d, logits, ids, gates, counts, ws, stream);
    if (E <= 128) return launch_route_gemm_nf<8, 1, true, kRouterSplit>(x, w_router, T, E, k, d, logits, ids, gates, counts, ws, stream);
    return launch_route_gemm_nf<16, 1, false, kRouterSplit>(x, w_router, T, E, k, d, logits, ids, gates, counts, ws, stream);
  }
  const bool wide = T >= 8192;
  if (E <= 64)
    return wide ? launch_route_gemm_nf<4, 2, true, 0>(x, w_router, T, E, k, d, logits, ids, gates, counts, ws, stream)
                : launch_route_gemm_nf<4, 1, true, 0>(x, w_router, T, E, k, d, logits, ids, gates, counts, ws, stream);
  if (E <= 128)
    return wide ? launch_route_gemm_nf<8, 2, true, 0>(x, w_router, T, E, k, d, logits, ids, gates, counts, ws, stream)
                : launch_route_gemm_nf<8, 1, true, 0>(x, w_router, T, E, k, d, logits, ids, gates, counts, ws, stream);
  return wide ? launch_route_gemm_nf<16, 2, false, 0>(x, w_router, T, E, k, d, logits, ids, gates, counts, ws, stream)
              : launch_route_gemm_nf<16, 1, false, 0>(x, w_router, T, E, k, d, logits, ids, gates, counts, ws, stream);
}

}  // namespace moe
