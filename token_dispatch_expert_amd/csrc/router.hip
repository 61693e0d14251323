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
// One workgroup of 4 waves takes 16 tokens and every expert (E <= 256). The waves split the
// contraction axis (wave w takes the 32-wide steps w, w+4, ...); every lane loads its MFMA
// fragments straight from memory (16 bytes each: x rows and weight rows are contiguous along the
// contraction axis), so x is read once and the weights stream through L2. The four partial
// 16 x E tiles are added in LDS in wave order (deterministic), then each wave runs the
// wave-level top-k on 4 tokens' rows.
#include "topk_wave.h"

namespace moe {

constexpr int kRouterTM = 16;   // tokens per workgroup
constexpr int kRouterWaves = 4;

template <int NF>  // NF = ceil(E / 16) expert fragments
__global__ __launch_bounds__(kRouterWaves * kWave) void route_gemm_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ wr, int T, int E, int k, int d,
    float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ gates,
    int32_t* __restrict__ counts) {
  constexpr int EPAD = NF * 16 + 4;  // LDS row stride (floats): rows 16 bytes apart in banks
  extern __shared__ float part[];    // [kRouterWaves][kRouterTM][EPAD]
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int t0 = blockIdx.x * kRouterTM;
  const int nsteps = d / 32;

  // fragment sources: lane -> row lane % 16 (token / expert), contraction offset (lane / 16) * 8
  const int r = lane & 15, kq = (lane >> 4) * 8;
  const __bf16* xa = x + (size_t)min(t0 + r, T - 1) * d + kq;
  const __bf16* wb[NF];
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) wb[nf] = wr + (size_t)min(nf * 16 + r, E - 1) * d + kq;

  f32x4 acc[NF];
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) acc[nf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int s = wave; s < nsteps; s += kRouterWaves) {
    const size_t ko = (size_t)s * 32;
    const u32x4 av = *reinterpret_cast<const u32x4*>(xa + ko);
    u32x4 bv[NF];
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) bv[nf] = *reinterpret_cast<const u32x4*>(wb[nf] + ko);
    bf16x8 a;
    __builtin_memcpy(&a, &av, 16);
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) {
      bf16x8 b;
      __builtin_memcpy(&b, &bv[nf], 16);
      acc[nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[nf], 0, 0, 0);
    }
  }
  // C fragment: lane holds rows (lane / 16) * 4 + j, column lane % 16
  float* mine = part + (size_t)wave * kRouterTM * EPAD;
#pragma unroll
  for (int nf = 0; nf < NF; ++nf)
#pragma unroll
    for (int j = 0; j < 4; ++j) mine[((lane >> 4) * 4 + j) * EPAD + nf * 16 + r] = acc[nf][j];
  __syncthreads();
  // logits = ((p0 + p1) + p2) + p3, into p0
  for (int i = tid; i < kRouterTM * NF * 16; i += kRouterWaves * kWave) {
    const int row = i / (NF * 16), col = i % (NF * 16);
    float v = part[row * EPAD + col];
#pragma unroll
    for (int w = 1; w < kRouterWaves; ++w) v += part[((size_t)w * kRouterTM + row) * EPAD + col];
    part[row * EPAD + col] = v;
    if (logits && col < E && t0 + row < T) logits[(size_t)(t0 + row) * E + col] = v;
  }
  __syncthreads();
  constexpr int EPL = (NF * 16 + kWave - 1) / kWave;
  for (int row = wave; row < kRouterTM; row += kRouterWaves) {
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

template <int NF>
static hipError_t launch_route_gemm_nf(const void* x, const void* wr, int T, int E, int k, int d,
                                       float* logits, int32_t* ids, float* gates, int32_t* counts,
                                       hipStream_t stream) {
  const size_t lds = (size_t)kRouterWaves * kRouterTM * (NF * 16 + 4) * sizeof(float);
  auto kern = &route_gemm_kernel<NF>;
  if (lds > 64 * 1024) {
    hipError_t st = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (st != hipSuccess) return st;
  }
  kern<<<(T + kRouterTM - 1) / kRouterTM, kRouterWaves * kWave, lds, stream>>>(
      static_cast<const __bf16*>(x), static_cast<const __bf16*>(wr), T, E, k, d, logits, ids,
      gates, counts);
  return hipGetLastError();
}

hipError_t launch_route_gemm(const void* x, const void* w_router, int T, int E, int k, int d,
                             float* logits, int32_t* ids, float* gates, int32_t* counts,
                             hipStream_t stream) {
  if (counts) {
    hipError_t st = launch_fill_i32(counts, E, 0, stream);
    if (st != hipSuccess) return st;
  }
  if (T == 0) return hipSuccess;
  if (E <= 64) return launch_route_gemm_nf<4>(x, w_router, T, E, k, d, logits, ids, gates, counts, stream);
  if (E <= 128) return launch_route_gemm_nf<8>(x, w_router, T, E, k, d, logits, ids, gates, counts, stream);
  return launch_route_gemm_nf<16>(x, w_router, T, E, k, d, logits, ids, gates, counts, stream);
}

}  // namespace moe
