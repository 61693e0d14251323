// Grouped SwiGLU FFN over expert-contiguous rows.
//
// Operation: "Expert Parallelism" tutorial page, section 4, compute (each expert processes
// its own contiguous rows; all experts in one grouped launch) with the SwiGLU expert
// h = silu(x Wg) * (x Wu), y = h Wd. The makespan-dispatcher abstract (on the page titled
// UltraEP) measures two regimes: with few rows per expert the time is spent streaming the
// expert's weights from HBM; with many rows it is GEMM tiles. This file holds the streaming
// kernel: every weight byte of an expert with rows is read once per 32-row group, straight
// from HBM into MFMA operand registers, with no padding of rows to a large M tile.
//
// Data layout: weights are stored contraction-contiguous ([E, N, K] row-major: gate/up
// N = d_ff, K = d; down N = d, K = d_ff), activations are [rows, K] row-major. The gfx950
// MFMA operand layout v_mfma_f32_16x16x32_bf16 gives lane L the 8 consecutive contraction
// elements (L/16)*8..+7 of row/column L%16, so each lane's fragment is one 16-byte load
// (8-byte for fp8, 2x16-byte for fp32 with 16x16x4 f32 MFMA).
//
// Work decomposition: an item is (expert e, 32-row group mg, column block nb of NF*16
// columns [x2 for gate and up]). A workgroup of 4 waves processes one item at a time from a
// device-side item list (persistent grid); the waves split the contraction axis in 128-wide
// blocks, keep one block of loads in flight while the previous block feeds the MFMAs, and
// reduce their partial tiles through LDS in a fixed order (deterministic). The epilogue
// applies SwiGLU and rounds h to the activation format (gate/up pass) or writes fp32
// y_sorted (down pass).
//
// fp8 weights (OCP e4m3fn, fp32 scale per 128x128 block): codes are converted exactly to bf16
// in registers, each 128-long contraction block is accumulated from zero in fp32 and then
// added to the running sum times the block's scale.
#include <math.h>

#include "moe_internal.h"

namespace moe {

enum : int { kF32 = 0, kBF16 = 1, kFP8 = 2 };

// Raw 8-element contraction fragment of one lane, per storage format.
template <int F> struct Raw;
template <> struct Raw<kBF16> { uint4 v; };
template <> struct Raw<kF32> { float4 lo, hi; };
template <> struct Raw<kFP8> { uint2 v; };

template <int F> __device__ __forceinline__ int elem_bytes() { return F == kF32 ? 4 : (F == kBF16 ? 2 : 1); }

template <int F>
__device__ __forceinline__ void load_frag(Raw<F>& r, const void* base, size_t elem, bool ok) {
  if constexpr (F == kBF16) {
    r.v = ok ? *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem)
             : make_uint4(0, 0, 0, 0);
  } else if constexpr (F == kF32) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    r.lo = ok ? p[0] : make_float4(0, 0, 0, 0);
    r.hi = ok ? p[1] : make_float4(0, 0, 0, 0);
  } else {
    r.v = ok ? *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(base) + elem)
             : make_uint2(0, 0);
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& v) {
  bf16x8 o;
  __builtin_memcpy(&o, &v, 16);
  return o;
}

// e4m3fn codes -> bf16, exact (every e4m3fn value is a bf16 value).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(const uint2& v) {
  bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, false);
  bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.x, 1.0f, true);
  bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, false);
  bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v.y, 1.0f, true);
  bf16x8 o;
  o[0] = p0[0]; o[1] = p0[1]; o[2] = p1[0]; o[3] = p1[1];
  o[4] = p2[0]; o[5] = p2[1]; o[6] = p3[0]; o[7] = p3[1];
  return o;
}

// acc += A(16 x 32) * B(32 x 16) for one lane's fragments.
template <int AF, int WF>
__device__ __forceinline__ void mma(f32x4& acc, const Raw<AF>& a, const Raw<WF>& b) {
  if constexpr (AF == kF32) {
    static_assert(WF == kF32, "fp32 activations need fp32 weights");
    const float av[8] = {a.lo.x, a.lo.y, a.lo.z, a.lo.w, a.hi.x, a.hi.y, a.hi.z, a.hi.w};
    const float bv[8] = {b.lo.x, b.lo.y, b.lo.z, b.lo.w, b.hi.x, b.hi.y, b.hi.z, b.hi.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], bv[i], acc, 0, 0, 0);
  } else if constexpr (WF == kBF16) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a.v), as_bf16x8(b.v), acc, 0, 0, 0);
  } else {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a.v), fp8x8_to_bf16(b.v), acc, 0, 0, 0);
  }
}

struct StreamArgs {
  const void* X;        // [rows, K] activations
  const void* W1;       // [E, N, K] (gate, or down)
  const void* W2;       // [E, N, K] (up; gated pass only)
  const float* S1;      // fp8 block scales [E, ceil(N/128), ceil(K/128)]
  const float* S2;
  void* out;            // gated: h [rows, N] in act format; else y_sorted fp32 [rows, N]
  const int32_t* offsets;
  int E, K, N, rows;
  int max_rows;         // experts with more rows are left to another kernel
};

constexpr int kMF = 2;                 // 16-row fragments per item
constexpr int kItemRows = 16 * kMF;    // rows per item

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Rows [a, b) of expert e, with the offsets clamped into [0, rows] and made non-decreasing so
// that corrupt offsets can never address memory out of bounds.
__device__ __forceinline__ void expert_rows(const int32_t* offsets, int e, int rows, int& a, int& b) {
  a = offsets[e];
  b = offsets[e + 1];
  a = a < 0 ? 0 : (a > rows ? rows : a);
  b = b < a ? a : (b > rows ? rows : b);
}

// Build the item prefix over experts in LDS: pre[e] = first item of expert e; pre[E] = total.
__device__ void build_item_prefix(int32_t* pre, int32_t* scratch, const int32_t* offsets, int E,
                                  int rows, int max_rows, int items_per_group) {
  const int tid = threadIdx.x;
  const int per = (E + blockDim.x - 1) / blockDim.x;  // experts per thread (<= 4)
  int local[4];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * per + i;
    int n = 0;
    if (i < per && e < E) {
      int a, b;
      expert_rows(offsets, e, rows, a, b);
      n = b - a;
    }
    local[i] = (n > 0 && n <= max_rows) ? ((n + kItemRows - 1) / kItemRows) * items_per_group : 0;
    sum += local[i];
  }
  scratch[tid] = sum;
  __syncthreads();
  for (int off = 1; off < (int)blockDim.x; off <<= 1) {
    const int v = tid >= off ? scratch[tid - off] : 0;
    __syncthreads();
    scratch[tid] += v;
    __syncthreads();
  }
  int run = scratch[tid] - sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid * per + i;
    if (i < per && e < E) {
      pre[e] = run;
      run += local[i];
    }
  }
  if (tid == blockDim.x - 1) pre[E] = scratch[tid];
  __syncthreads();
}

// MATS = 2 for the gate/up pass (gate and up share an item), 1 for the down pass.
// SPB = 32-long MFMA steps per contraction block (a wave's unit of work and of prefetch).
template <int AF, int WF, int MATS, int NF, int SPB>
__global__ __launch_bounds__(256) void ffn_stream_kernel(StreamArgs p) {
  constexpr int kCols = MATS * NF * 16;  // columns of the partial tile
  constexpr int kLdsStride = kCols + 4;
  constexpr int KB = SPB * 32;           // contraction block
  extern __shared__ __align__(16) unsigned char smem[];
  int32_t* pre = reinterpret_cast<int32_t*>(smem);                               // E+1
  int32_t* scan_tmp = pre + ((p.E + 1 + 3) & ~3);                                // 256
  float* red = reinterpret_cast<float*>(scan_tmp + 256);                         // 4*32*stride

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int NB = (p.N + NF * 16 - 1) / (NF * 16);
  build_item_prefix(pre, scan_tmp, p.offsets, p.E, p.rows, p.max_rows, NB);
  const int total = pre[p.E];
  const int nkb = (p.K + KB - 1) / KB;
  const int kb_begin = (nkb * wave) / kStreamWaves;
  const int kb_end = (nkb * (wave + 1)) / kStreamWaves;
  const int nNB128 = (p.N + 127) / 128, nKB128 = (p.K + 127) / 128;
  const size_t wstride = (size_t)p.N * p.K;  // elements per expert matrix

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    // expert owning this item: largest e with pre[e] <= item
    int lo = 0, hi = p.E;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int local = item - pre[e];
    const int mg = local / NB, nb = local % NB;
    int e_begin, e_end;
    expert_rows(p.offsets, e, p.rows, e_begin, e_end);
    const int r_begin = e_begin + mg * kItemRows;
    const int r_end = min(r_begin + kItemRows, e_end);
    const int nmf = (r_end - r_begin + 15) / 16;
    const int n0 = nb * NF * 16;

    // per-lane operand addresses (clamped in-bounds; masked on store)
    size_t a_row[kMF];
#pragma unroll
    for (int mf = 0; mf < kMF; ++mf) a_row[mf] = (size_t)min(r_begin + mf * 16 + (lane & 15), r_end - 1) * p.K;
    size_t b_row[NF];
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) b_row[nf] = (size_t)e * wstride + (size_t)min(n0 + nf * 16 + (lane & 15), p.N - 1) * p.K;
    const void* Wm[2] = {p.W1, p.W2};
    const float* Sm[2] = {p.S1, p.S2};
    const int kl = (lane >> 4) * 8;

    f32x4 acc[kMF][MATS][NF];
#pragma unroll
    for (int mf = 0; mf < kMF; ++mf)
#pragma unroll
      for (int m = 0; m < MATS; ++m)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) acc[mf][m][nf] = f32x4{0.f, 0.f, 0.f, 0.f};

    Raw<AF> a_cur[kMF][SPB], a_nxt[kMF][SPB];
    Raw<WF> b_cur[MATS][NF][SPB], b_nxt[MATS][NF][SPB];

    auto load_block = [&](int kb, Raw<AF> (&a)[kMF][SPB], Raw<WF> (&b)[MATS][NF][SPB]) {
#pragma unroll
      for (int s = 0; s < SPB; ++s) {
        const int k = kb * KB + s * 32 + kl;
        const bool kok = k < p.K;
#pragma unroll
        for (int m = 0; m < MATS; ++m)
#pragma unroll
          for (int nf = 0; nf < NF; ++nf) load_frag<WF>(b[m][nf][s], Wm[m], b_row[nf] + k, kok);
#pragma unroll
        for (int mf = 0; mf < kMF; ++mf) load_frag<AF>(a[mf][s], p.X, a_row[mf] + k, kok && mf < nmf);
      }
    };

    if (kb_begin < kb_end) load_block(kb_begin, a_cur, b_cur);
    for (int kb = kb_begin; kb < kb_end; ++kb) {
      if (kb + 1 < kb_end) load_block(kb + 1, a_nxt, b_nxt);
      if constexpr (WF == kFP8) {
        f32x4 part[kMF][MATS][NF];
#pragma unroll
        for (int mf = 0; mf < kMF; ++mf)
#pragma unroll
          for (int m = 0; m < MATS; ++m)
#pragma unroll
            for (int nf = 0; nf < NF; ++nf) part[mf][m][nf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < SPB; ++s)
#pragma unroll
          for (int mf = 0; mf < kMF; ++mf)
            if (mf < nmf)
#pragma unroll
              for (int m = 0; m < MATS; ++m)
#pragma unroll
                for (int nf = 0; nf < NF; ++nf) mma<AF, WF>(part[mf][m][nf], a_cur[mf][s], b_cur[m][nf][s]);
#pragma unroll
        for (int m = 0; m < MATS; ++m)
#pragma unroll
          for (int nf = 0; nf < NF; ++nf) {
            const int nbs = (n0 + nf * 16) / 128;
            const float sc = Sm[m][((size_t)e * nNB128 + min(nbs, nNB128 - 1)) * nKB128 + (kb * KB) / 128];
#pragma unroll
            for (int mf = 0; mf < kMF; ++mf)
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[mf][m][nf][j] = fmaf(sc, part[mf][m][nf][j], acc[mf][m][nf][j]);
          }
      } else {
#pragma unroll
        for (int s = 0; s < SPB; ++s)
#pragma unroll
          for (int mf = 0; mf < kMF; ++mf)
            if (mf < nmf)
#pragma unroll
              for (int m = 0; m < MATS; ++m)
#pragma unroll
                for (int nf = 0; nf < NF; ++nf) mma<AF, WF>(acc[mf][m][nf], a_cur[mf][s], b_cur[m][nf][s]);
      }
      if (kb + 1 < kb_end) {
#pragma unroll
        for (int s = 0; s < SPB; ++s) {
#pragma unroll
          for (int mf = 0; mf < kMF; ++mf) a_cur[mf][s] = a_nxt[mf][s];
#pragma unroll
          for (int m = 0; m < MATS; ++m)
#pragma unroll
            for (int nf = 0; nf < NF; ++nf) b_cur[m][nf][s] = b_nxt[m][nf][s];
        }
      }
    }

    // partial tiles -> LDS: lane holds rows (lane/16)*4 + j, column lane%16 of each fragment
    float* mine = red + (size_t)wave * kItemRows * kLdsStride;
#pragma unroll
    for (int mf = 0; mf < kMF; ++mf)
#pragma unroll
      for (int m = 0; m < MATS; ++m)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            mine[(mf * 16 + (lane >> 4) * 4 + j) * kLdsStride + m * NF * 16 + nf * 16 + (lane & 15)] = acc[mf][m][nf][j];
    __syncthreads();

    const int nrows = r_end - r_begin;
    if constexpr (MATS == 2) {
      // gate/up epilogue: h = silu(gate) * up, 8 (bf16) or 4 (fp32) columns per task
      constexpr int G = (AF == kF32) ? 4 : 8;
      constexpr int groups = NF * 16 / G;
      for (int task = threadIdx.x; task < kItemRows * groups; task += blockDim.x) {
        const int r = task / groups, c0 = (task % groups) * G;
        if (r >= nrows || n0 + c0 >= p.N) continue;
        float hv[G];
#pragma unroll
        for (int c = 0; c < G; ++c) {
          float g = 0.f, u = 0.f;
#pragma unroll
          for (int w = 0; w < kStreamWaves; ++w) {
            g += red[((size_t)w * kItemRows + r) * kLdsStride + c0 + c];
            u += red[((size_t)w * kItemRows + r) * kLdsStride + NF * 16 + c0 + c];
          }
          hv[c] = silu(g) * u;
        }
        const size_t o = (size_t)(r_begin + r) * p.N + n0 + c0;
        if constexpr (AF == kF32) {
          *reinterpret_cast<float4*>(static_cast<float*>(p.out) + o) = make_float4(hv[0], hv[1], hv[2], hv[3]);
        } else {
          bf16x8 hb;
#pragma unroll
          for (int c = 0; c < 8; ++c) hb[c] = (__bf16)hv[c];
          uint4 u4;
          __builtin_memcpy(&u4, &hb, 16);
          *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + o) = u4;
        }
      }
    } else {
      constexpr int groups = NF * 16 / 4;
      for (int task = threadIdx.x; task < kItemRows * groups; task += blockDim.x) {
        const int r = task / groups, c0 = (task % groups) * 4;
        if (r >= nrows || n0 + c0 >= p.N) continue;
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float s = 0.f;
#pragma unroll
          for (int w = 0; w < kStreamWaves; ++w) s += red[((size_t)w * kItemRows + r) * kLdsStride + c0 + c];
          v[c] = s;
        }
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + (size_t)(r_begin + r) * p.N + n0 + c0) =
            make_float4(v[0], v[1], v[2], v[3]);
      }
    }
    __syncthreads();
  }
}

template <int AF, int WF, int MATS, int NF, int SPB>
static hipError_t launch_stream(const StreamArgs& p, const DeviceInfo& dev, hipStream_t stream) {
  constexpr int kCols = MATS * NF * 16;
  const size_t lds = ((size_t)(p.E + 1 + 3) / 4 * 4 + 256) * sizeof(int32_t) +
                     (size_t)kStreamWaves * kItemRows * (kCols + 4) * sizeof(float);
  const int grid = dev.num_cus * 2;
  ffn_stream_kernel<AF, WF, MATS, NF, SPB><<<grid, 256, lds, stream>>>(p);
  return hipGetLastError();
}

size_t ffn_workspace_bytes(int rows, int E, int d, int d_ff, moe_dtype_t act, moe_dtype_t wdt) {
  (void)E; (void)d; (void)wdt;
  const size_t hb = act == MOE_F32 ? 4 : 2;
  return align_up((size_t)rows * d_ff * hb, 256);
}

hipError_t launch_grouped_ffn(const FfnArgs& a, const DeviceInfo& dev, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  StreamArgs gu{a.x_sorted, a.w_gate, a.w_up, a.s_gate, a.s_up, a.h, a.offsets,
                a.E, a.d, a.d_ff, a.rows, 0x7fffffff};
  StreamArgs dn{a.h, a.w_down, nullptr, a.s_down, nullptr, a.y_sorted, a.offsets,
                a.E, a.d_ff, a.d, a.rows, 0x7fffffff};
  hipError_t st;
  if (a.act == MOE_F32) {
    st = launch_stream<kF32, kF32, 2, 1, 2>(gu, dev, stream);
    if (st != hipSuccess) return st;
    return launch_stream<kF32, kF32, 1, 2, 2>(dn, dev, stream);
  }
  if (a.wdt == MOE_BF16) {
    st = launch_stream<kBF16, kBF16, 2, 2, 4>(gu, dev, stream);
    if (st != hipSuccess) return st;
    return launch_stream<kBF16, kBF16, 1, 4, 4>(dn, dev, stream);
  }
  st = launch_stream<kBF16, kFP8, 2, 2, 4>(gu, dev, stream);
  if (st != hipSuccess) return st;
  return launch_stream<kBF16, kFP8, 1, 4, 4>(dn, dev, stream);
}

}  // namespace moe
