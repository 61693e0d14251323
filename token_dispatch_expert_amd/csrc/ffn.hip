// Grouped SwiGLU FFN over expert-contiguous rows.
//
// Operation: "Expert Parallelism" tutorial page, section 4, compute (each expert processes
// its own contiguous rows; all experts in one grouped launch) with the SwiGLU expert
// h = silu(x Wg) * (x Wu), y = h Wd. The makespan-dispatcher abstract (on the page titled
// UltraEP) measures two regimes: with few rows per expert the time is spent streaming the
// expert's weights from HBM; with many rows it is GEMM tiles.
//
// Data layout: weights are stored contraction-contiguous ([E, N, K] row-major: gate/up
// N = d_ff, K = d; down N = d, K = d_ff), activations are [rows, K] row-major. The gfx950
// MFMA operand layout v_mfma_f32_16x16x32_bf16 gives lane L 8 contraction elements of
// row/column L%16 (the same 8 for both operands; which 8 of the 32 is the kernel's choice), so
// each lane's fragment is one 16-byte load (fp8 weights: 8 bytes, or 16 bytes serving two
// MFMAs; fp32: 2x16 bytes with the 16x16x4 f32 MFMA).
//
// Kernels (launch_grouped_ffn at the end picks them from the sizes; each expert's rows go to
// one of them from its row count, decided on the device):
//  - ffn_stream_kernel: weights straight from HBM into MFMA operand registers, 16-row items,
//    the contraction split over the 4 waves and reduced through LDS in a fixed order; fp32,
//    widths not multiples of 64, and, beside the register-staged tiles, experts with <= 16
//    rows in fp8 launches longer than the direct-to-LDS kernel takes.
//  - dl_tiles (in ffn_tiled_dl_kernel and ffn_prefill_kernel): tiles loaded straight into a
//    ring of LDS slots by buffer loads, XOR-swizzled for conflict-free fragment reads, on a
//    persistent grid whose rounds of tiles are dealt to the XCDs in runs; decode-sized
//    launches (bf16: 64 x 128 tiles, with a contraction split when there are few tiles; fp8:
//    32 x 128) and, in
//    ffn_prefill_kernel, both roles of prefill-sized launches: workgroups streaming the experts
//    with <= 16 rows beside workgroups running 256-row tiles of the others.
//  - ffn_tiled_kernel: the older register-staged tiles, kept for fp8 weights whose contraction
//    (d or d_ff) is longer than 65536, beyond what the direct-to-LDS kernel stages scales for.
//
// fp8 weights (OCP e4m3fn, fp32 scale per 128x128 block): codes are converted exactly to bf16
// in registers, each 128-long contraction block is accumulated from zero in fp32 and then
// added to the running sum times the block's scale.
#include <math.h>

#include <type_traits>
#include <utility>

#include <algorithm>

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

constexpr int kMF = 1;                 // 16-row fragments per item
constexpr int kStreamMaxRows = 16;     // larger experts use the tiled kernel (bf16 path)
constexpr int kItemRows = 16 * kMF;    // rows per item

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Workgroup barrier that orders LDS only: unlike __syncthreads() it does not wait for the
// wave's outstanding global loads, so prefetches stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Rows [a, b) of expert e, with the offsets clamped into [0, rows] and made non-decreasing so
// that corrupt offsets can never address memory out of bounds.
__device__ __forceinline__ void expert_rows(const int32_t* offsets, int e, int rows, int& a, int& b) {
  a = offsets[e];
  b = offsets[e + 1];
  a = a < 0 ? 0 : (a > rows ? rows : a);
  b = b < a ? a : (b > rows ? rows : b);
}

// Build the item prefix over experts in LDS: pre[e] = first item of expert e; pre[E] = total.
// offs (optional) receives the clamped row offsets of every expert, offs[0..E].
// Item of workgroup b (of G) in the round of a persistent grid that starts at item `base`, or
// -1.
// The hardware deals workgroups to the 8 XCDs round-robin (workgroup b runs on XCD b % 8), and
// each XCD has its own L2. To let the workgroups of one XCD share operands, a round's n items
// are cut into 8 runs of ceil(n / 8) consecutive items and run x goes to the workgroups of XCD
// x; a short last round is thus spread over all XCDs. Grids that are not a multiple of 8 take
// items in plain order.
__device__ __forceinline__ int xcd_round_item(int base, int total, int b, int G) {
  constexpr int kXcd = 8;
  if (G % kXcd != 0) return base + b < total ? base + b : -1;
  const int n = min(G, total - base);
  const int run = (n + kXcd - 1) / kXcd;
  const int i = b / kXcd;
  const int local = (b % kXcd) * run + i;
  return (i < run && local < n) ? base + local : -1;
}

__device__ void build_item_prefix(int32_t* pre, int32_t* scratch, const int32_t* offsets, int E,
                                  int rows, int max_rows, int items_per_group,
                                  int32_t* offs = nullptr, int min_rows = 0,
                                  int rows_per_group = kItemRows) {
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
      if (offs) {
        offs[e] = a;
        if (e == E - 1) offs[E] = b;
      }
    }
    local[i] = (n > min_rows && n <= max_rows)
                   ? ((n + rows_per_group - 1) / rows_per_group) * items_per_group : 0;
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

// A workgroup of 4 waves streams one item at a time: (expert e, 32-row group, NF*16 columns
// of each of the MATS matrices). The waves split the item's contraction axis into 4 ranges;
// each wave's blocks (KB = SPB*32 elements) form one continuous stream across the items of
// its workgroup: a ring of NBUF register slots keeps NBUF-1 blocks of loads in flight ahead
// of the block feeding the MFMAs, across item boundaries. Every slot load is issued
// unconditionally (addresses clamped in-bounds, out-of-range data discarded), which keeps the
// compiler's memory-counter waits exact. At the end of an item the waves reduce their partial
// tiles through LDS in a fixed order (deterministic) and all 256 threads run the epilogue.
template <int AF, int WF, int MATS, int NF, int SPB>
struct Slot {
  Raw<AF> a[kMF][SPB];
  Raw<WF> b[MATS][NF][SPB];
  int e, r_begin, nrows, n0, kb;
  bool valid, last, dummy;
};

template <int AF, int WF, int MATS, int NF, int SPB, int NBUF>
__global__ __launch_bounds__(256) void ffn_stream_kernel(StreamArgs p) {
  constexpr int KB = SPB * 32;
  constexpr int kCols = MATS * NF * 16;
  constexpr int kStride = kCols + 4;
  extern __shared__ __align__(16) unsigned char smem[];
  const int Epad = (p.E + 1 + 3) & ~3;
  int32_t* pre = reinterpret_cast<int32_t*>(smem);         // E+1
  int32_t* offs = pre + Epad;                               // E+1 clamped row offsets
  int32_t* scan_tmp = offs + Epad;                          // 256
  float* red = reinterpret_cast<float*>(scan_tmp + 256);    // [4][kItemRows][kStride]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NB = (p.N + NF * 16 - 1) / (NF * 16);
  build_item_prefix(pre, scan_tmp, p.offsets, p.E, p.rows, p.max_rows, NB, offs);
  const int total = __builtin_amdgcn_readfirstlane(pre[p.E]);
  if ((int)blockIdx.x >= total) return;  // uniform per workgroup
  const int nkb = (p.K + KB - 1) / KB;
  // this wave's contraction blocks [kb0, kb0 + nblk); a wave with no blocks (tiny K) runs one
  // masked dummy block per item so that it still meets every item's barrier
  const int per = (nkb + kStreamWaves - 1) / kStreamWaves;
  const int kb0 = min(wave * per, nkb);
  const int kb1 = min(kb0 + per, nkb);
  const bool dummy = kb0 >= kb1;
  const int nblk = dummy ? 1 : kb1 - kb0;
  const int nNB128 = (p.N + 127) / 128, nKB128 = (p.K + 127) / 128;
  const size_t wstride = (size_t)p.N * p.K;
  const int kl = (lane >> 4) * 8;
  const void* Wm[2] = {p.W1, p.W2};
  const float* Sm[2] = {p.S1, p.S2};

  // load cursor (wave-uniform; readfirstlane keeps it in scalar registers)
  int l_item = blockIdx.x, l_j = 0;
  int l_e = 0, l_rb = 0, l_nr = 0, l_n0 = 0;
  auto decode = [&](int item) {
    int lo = 0, hi = p.E;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (__builtin_amdgcn_readfirstlane(pre[mid]) <= item) lo = mid; else hi = mid - 1;
    }
    const int eb = __builtin_amdgcn_readfirstlane(offs[lo]);
    const int ee = __builtin_amdgcn_readfirstlane(offs[lo + 1]);
    const int local = item - __builtin_amdgcn_readfirstlane(pre[lo]);
    const int mg = local / NB;
    l_e = lo;
    l_rb = eb + mg * kItemRows;
    l_nr = min(kItemRows, ee - l_rb);
    l_n0 = (local % NB) * NF * 16;
  };
  decode(l_item);

  Slot<AF, WF, MATS, NF, SPB> slot[NBUF];

  auto issue = [&](Slot<AF, WF, MATS, NF, SPB>& s) {
    const bool valid = l_item < total;
    const int kb = dummy ? nkb - 1 : kb0 + l_j;
    s.valid = valid;
    s.e = l_e; s.r_begin = l_rb; s.nrows = l_nr; s.n0 = l_n0; s.kb = kb;
    s.last = l_j == nblk - 1;
    s.dummy = dummy;
    size_t b_row[NF];
#pragma unroll
    for (int nf = 0; nf < NF; ++nf)
      b_row[nf] = (size_t)l_e * wstride + (size_t)min(l_n0 + nf * 16 + (lane & 15), p.N - 1) * p.K;
    size_t a_row[kMF];
#pragma unroll
    for (int mf = 0; mf < kMF; ++mf)
      a_row[mf] = (size_t)(l_rb + min(mf * 16 + (lane & 15), l_nr - 1)) * p.K;
#pragma unroll
    for (int st = 0; st < SPB; ++st) {
      const int k = kb * KB + st * 32 + kl;
      const int kc = k < p.K ? k : p.K - 8;
#pragma unroll
      for (int m = 0; m < MATS; ++m)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) load_frag<WF>(s.b[m][nf][st], Wm[m], b_row[nf] + kc, true);
#pragma unroll
      for (int mf = 0; mf < kMF; ++mf) load_frag<AF>(s.a[mf][st], p.X, a_row[mf] + kc, true);
    }
    if (valid && ++l_j == nblk) {
      l_j = 0;
      l_item += gridDim.x;
      if (l_item < total) decode(l_item);
    }
  };

  f32x4 acc[kMF][MATS][NF];
#pragma unroll
  for (int mf = 0; mf < kMF; ++mf)
#pragma unroll
    for (int m = 0; m < MATS; ++m)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) acc[mf][m][nf] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](Slot<AF, WF, MATS, NF, SPB>& s) {
    if (s.dummy) return;
    const int nmf = (s.nrows + 15) / 16;
    // contraction tail (K not a multiple of the block): lanes past K loaded a clamped
    // in-bounds address; zero their activation operand now that the data has arrived
    if ((s.kb + 1) * KB > p.K) {
#pragma unroll
      for (int st = 0; st < SPB; ++st)
        if (s.kb * KB + st * 32 + kl >= p.K)
#pragma unroll
          for (int mf = 0; mf < kMF; ++mf) s.a[mf][st] = Raw<AF>{};
    }
    if constexpr (WF == kFP8) {
      f32x4 part[kMF][MATS][NF];
#pragma unroll
      for (int mf = 0; mf < kMF; ++mf)
#pragma unroll
        for (int m = 0; m < MATS; ++m)
#pragma unroll
          for (int nf = 0; nf < NF; ++nf) part[mf][m][nf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < SPB; ++st)
#pragma unroll
        for (int mf = 0; mf < kMF; ++mf)
          if (mf < nmf)
#pragma unroll
            for (int m = 0; m < MATS; ++m)
#pragma unroll
              for (int nf = 0; nf < NF; ++nf) mma<AF, WF>(part[mf][m][nf], s.a[mf][st], s.b[m][nf][st]);
#pragma unroll
      for (int m = 0; m < MATS; ++m)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) {
          const int nbs = min((s.n0 + nf * 16) / 128, nNB128 - 1);
          const float sc = Sm[m][((size_t)s.e * nNB128 + nbs) * nKB128 + (s.kb * KB) / 128];
#pragma unroll
          for (int mf = 0; mf < kMF; ++mf)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[mf][m][nf][j] = fmaf(sc, part[mf][m][nf][j], acc[mf][m][nf][j]);
        }
    } else {
#pragma unroll
      for (int st = 0; st < SPB; ++st)
#pragma unroll
        for (int mf = 0; mf < kMF; ++mf)
          if (mf < nmf)
#pragma unroll
            for (int m = 0; m < MATS; ++m)
#pragma unroll
              for (int nf = 0; nf < NF; ++nf) mma<AF, WF>(acc[mf][m][nf], s.a[mf][st], s.b[m][nf][st]);
    }
  };

  // end of an item: partial tiles -> LDS (lane holds rows (lane/16)*4 + j, column lane%16 of
  // each fragment), barrier, fixed-order reduction + epilogue by all threads, barrier
  auto finish = [&](const Slot<AF, WF, MATS, NF, SPB>& s) {
    float* mine = red + (size_t)wave * kItemRows * kStride;
#pragma unroll
    for (int mf = 0; mf < kMF; ++mf)
#pragma unroll
      for (int m = 0; m < MATS; ++m)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            mine[(mf * 16 + (lane >> 4) * 4 + j) * kStride + m * NF * 16 + nf * 16 + (lane & 15)] = acc[mf][m][nf][j];
          acc[mf][m][nf] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    lds_barrier();
    if constexpr (MATS == 2) {
      constexpr int G = (AF == kF32) ? 4 : 8;
      constexpr int groups = NF * 16 / G;
      for (int task = threadIdx.x; task < kItemRows * groups; task += blockDim.x) {
        const int r = task / groups, c0 = (task % groups) * G;
        if (r >= s.nrows || s.n0 + c0 >= p.N) continue;
        float hv[G];
#pragma unroll
        for (int c = 0; c < G; ++c) {
          float g = 0.f, u = 0.f;
#pragma unroll
          for (int w = 0; w < kStreamWaves; ++w) {
            g += red[((size_t)w * kItemRows + r) * kStride + c0 + c];
            u += red[((size_t)w * kItemRows + r) * kStride + NF * 16 + c0 + c];
          }
          hv[c] = silu(g) * u;
        }
        const size_t o = (size_t)(s.r_begin + r) * p.N + s.n0 + c0;
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
        if (r >= s.nrows || s.n0 + c0 >= p.N) continue;
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float sum = 0.f;
#pragma unroll
          for (int w = 0; w < kStreamWaves; ++w) sum += red[((size_t)w * kItemRows + r) * kStride + c0 + c];
          v[c] = sum;
        }
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + (size_t)(s.r_begin + r) * p.N + s.n0 + c0) =
            make_float4(v[0], v[1], v[2], v[3]);
      }
    }
    lds_barrier();
  };

#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i) issue(slot[i]);
  for (;;) {
#pragma unroll
    for (int i = 0; i < NBUF; ++i) {
      issue(slot[(i + NBUF - 1) % NBUF]);
      if (!slot[i].valid) return;  // the same for every wave of the workgroup
      compute(slot[i]);
      if (slot[i].last) finish(slot[i]);
    }
  }
}

template <int AF, int WF, int MATS, int NF, int SPB, int NBUF>
static hipError_t launch_stream(const StreamArgs& p, const DeviceInfo& dev, hipStream_t stream) {
  constexpr int kCols = MATS * NF * 16;
  const size_t lds = ((size_t)(p.E + 1 + 3) / 4 * 4 * 2 + 256) * sizeof(int32_t) +
                     (size_t)kStreamWaves * kItemRows * (kCols + 4) * sizeof(float);
  const int grid = dev.num_cus * 2;
  ffn_stream_kernel<AF, WF, MATS, NF, SPB, NBUF><<<grid, 256, lds, stream>>>(p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Tiled kernel for experts with many rows (the GEMM-tile regime): a workgroup of 4 waves
// computes a (2*WM)-row x (2*WN)-column output tile over the whole contraction axis in
// 64-wide steps. For the gate/up pass the tile's columns are WN gate and the same WN up
// columns of h. Operand tiles are staged in LDS (double-buffered: the next step's global
// loads are in flight while the MFMAs consume the current one), so each weight tile is read
// from memory once per 2*WM rows of its expert and each activation tile once per tile of
// columns. The waves split the tile 2 x 2; wave (wm, wn) owns rows wm*WM..+WM-1 and, in the
// gate/up pass, gate and up columns c0 + wn*WN/2.. (so SwiGLU is applied in registers).
// Two shapes are instantiated: 64 x 64 per wave for decode-sized batches and 128 x 128 per
// wave (256 fp32 accumulators per lane, in AGPRs) for prefill, where a larger tile halves
// the LDS and L2 traffic per MFMA. (Only fp8 weights with a contraction longer than 65536
// reach this kernel now; the direct-to-LDS tiles below take every other tiled launch.)
// LDS tiles hold 64-wide rows of bf16 (128 bytes = 8 chunks of 16 bytes) with an XOR
// swizzle: chunk c of row r is stored at chunk c ^ ((r >> 1) & 7). A 16-byte fragment load
// reads one chunk from each of 16 consecutive rows, and the staging store writes the 8 chunks
// of two consecutive rows per 16 lanes; with the swizzle both touch all 64 banks exactly once.
constexpr int kTK = 64;
constexpr int kLdsRow = kTK;
__device__ __forceinline__ int swz(int row, int chunk) { return row * kLdsRow + ((chunk ^ ((row >> 1) & 7)) << 3); }

struct TiledArgs {
  const void* X;
  const void* W1;
  const void* W2;
  const float* S1;
  const float* S2;
  void* out;
  const int32_t* offsets;
  int E, K, N, rows;
  int min_rows;  // experts with at most this many rows are left to the streaming kernel
  // contraction split of launches with few tiles: fp32 partial tiles, and the grid of the launch
  // that computes them (both launches derive the chunk count from it)
  float* partial = nullptr;
  int split_ranks = 0;
  // tail split of prefill launches: {S, first split item, end of the split items}, written by
  // the launch that computes the chunks and read by the one that adds them
  int32_t* split_info = nullptr;
  // prefill: 1 when ffn_lean_kernel runs beside this launch on a second stream and may take the
  // experts with at most kStreamMaxRows rows (both kernels decide from the counts alike)
  int lean = 0;
  // weights in a blocked layout (8 rows x 128 bytes per 1 KB block); only read by the
  // direct-to-LDS tiles whose steps take 128 bytes of a weight row, and the lean kernel
  int wblk = 0;
};

template <int WF, bool GATED, int WM, int WN, int WGM, int WGN>
__global__ __launch_bounds__(64 * WGM * WGN) void ffn_tiled_kernel(TiledArgs p) {
  constexpr int NTH = 64 * WGM * WGN;                        // threads per workgroup
  constexpr int TM = WGM * WM, TN = WGN * WN;
  constexpr int MF = WM / 16, NF = WN / 16;
  constexpr int ACH = TM * 8 / NTH;                         // 16-byte A chunks per thread
  constexpr int BCH = (WF == kFP8) ? TN * 4 / NTH : TN * 8 / NTH;
  extern __shared__ __align__(16) unsigned char smem[];
  const int Epad = (p.E + 1 + 3) & ~3;
  int32_t* pre = reinterpret_cast<int32_t*>(smem);
  int32_t* offs = pre + Epad;
  int32_t* scan_tmp = offs + Epad;
  __bf16* lds_a = reinterpret_cast<__bf16*>(scan_tmp + NTH);   // [2][TM][kLdsRow]
  __bf16* lds_b = lds_a + 2 * TM * kLdsRow;                     // [2][TN][kLdsRow]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WGM, wn = wave / WGM;
  constexpr int cols_per_tile = GATED ? TN / 2 : TN;
  const int NT = (p.N + cols_per_tile - 1) / cols_per_tile;
  build_item_prefix(pre, scan_tmp, p.offsets, p.E, p.rows, 0x7fffffff, NT, offs, p.min_rows, TM);
  const int total = __builtin_amdgcn_readfirstlane(pre[p.E]);
  const int nkb = p.K / kTK;  // K is a multiple of kTK on this path
  const int nNB128 = (p.N + 127) / 128, nKB128 = (p.K + 127) / 128;
  const size_t wstride = (size_t)p.N * p.K;
  const int kl = (lane >> 4) * 8;

  for (int base = 0; base < total; base += gridDim.x) {
    const int item = xcd_round_item(base, total, blockIdx.x, gridDim.x);
    if (item < 0) continue;  // uniform per workgroup
    int lo = 0, hi = p.E;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (__builtin_amdgcn_readfirstlane(pre[mid]) <= item) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int local = item - __builtin_amdgcn_readfirstlane(pre[e]);
    // Tile order within an expert: groups of kGroupM row tiles, column tiles outer and row
    // tiles inner within a group. Consecutive items run on one XCD, so its concurrent
    // workgroups cover kGroupM row tiles x several column tiles of the same expert and share
    // both operands in that XCD's L2.
    constexpr int kGroupM = 4;
    const int ebeg = __builtin_amdgcn_readfirstlane(offs[e]);
    const int MT = (__builtin_amdgcn_readfirstlane(offs[e + 1]) - ebeg + TM - 1) / TM;
    const int g = local / (kGroupM * NT);
    const int gm = min(kGroupM, MT - g * kGroupM);
    const int j = local - g * kGroupM * NT;
    const int nt = j / gm;
    const int mt = g * kGroupM + j % gm;
    const int r0 = ebeg + mt * TM;
    const int nrows = min(TM, __builtin_amdgcn_readfirstlane(offs[e + 1]) - r0);
    const int c0 = nt * cols_per_tile;

    // weight row held by LDS tile row t
    auto wrow = [&](int t) __attribute__((always_inline)) -> int {
      int n;
      if constexpr (GATED) {
        const int half = t / WN, q = t % WN;
        n = c0 + half * (WN / 2) + (q % (WN / 2));
      } else {
        n = c0 + t;
      }
      return min(n, p.N - 1);
    };
    auto is_up = [&](int t) __attribute__((always_inline)) -> bool { return GATED && (t % WN) >= WN / 2; };

    // global -> LDS mapping in 16-byte chunks: chunk i of thread tid covers tile row
    // (tid / CPR) + i * (256 / CPR) and column chunk tid % CPR (CPR = chunks per 64-wide row).
    // Addresses are recomputed per load from a few base values instead of being held in
    // registers. Activation rows past the expert's end are not loaded: their LDS rows (stale
    // but finite data) only feed output rows that are never stored, and MFMA rows are
    // independent.
    constexpr int ACPR = 8, ARPI = NTH / ACPR;                       // A: chunks per row, rows per i
    constexpr int BCPR = (WF == kFP8) ? 4 : 8, BRPI = NTH / BCPR;    // B
    constexpr int BELEM = (WF == kFP8) ? 16 : 8;                     // elements per B chunk
    const int a_r = tid / ACPR, a_c = tid % ACPR;
    const int b_r = tid / BCPR, b_c = tid % BCPR;
    const uint16_t* xa = static_cast<const uint16_t*>(p.X) + (size_t)r0 * p.K + a_c * 8;
    const char* w1 = static_cast<const char*>(p.W1) + ((size_t)e * wstride + b_c * BELEM) * (WF == kFP8 ? 1 : 2);
    const char* w2 = GATED ? static_cast<const char*>(p.W2) + ((size_t)e * wstride + b_c * BELEM) * (WF == kFP8 ? 1 : 2) : w1;

    struct Stage {
      u32x4 a[ACH];
      u32x4 b[BCH];
    };
    auto gload = [&](int kb, Stage st) __attribute__((always_inline)) -> Stage {
      const size_t ko = (size_t)kb * kTK;
#pragma unroll
      for (int i = 0; i < ACH; ++i) {
        const int row = a_r + i * ARPI;
        if (row < nrows) st.a[i] = *reinterpret_cast<const u32x4*>(xa + (size_t)row * p.K + ko);
      }
#pragma unroll
      for (int i = 0; i < BCH; ++i) {
        const int t = b_r + i * BRPI;
        const char* base = is_up(t) ? w2 : w1;
        st.b[i] = *reinterpret_cast<const u32x4*>(base + ((size_t)wrow(t) * p.K + ko) * (WF == kFP8 ? 1 : 2));
      }
      return st;
    };
    // (ARPI and BRPI are multiples of 16, so the swizzle term of row + i * RPI equals row's)
    auto lstore = [&](int buf, const Stage& st) __attribute__((always_inline)) {
      __bf16* A = lds_a + buf * TM * kLdsRow + swz(a_r, a_c);
#pragma unroll
      for (int i = 0; i < ACH; ++i) *reinterpret_cast<u32x4*>(A + i * ARPI * kLdsRow) = st.a[i];
#pragma unroll
      for (int i = 0; i < BCH; ++i) {
        if constexpr (WF == kFP8) {
          __bf16* B = lds_b + buf * TN * kLdsRow + (b_r + i * BRPI) * kLdsRow;
          *reinterpret_cast<bf16x8*>(B + ((((2 * b_c) ^ ((b_r >> 1) & 7))) << 3)) =
              fp8x8_to_bf16(make_uint2(st.b[i][0], st.b[i][1]));
          *reinterpret_cast<bf16x8*>(B + ((((2 * b_c + 1) ^ ((b_r >> 1) & 7))) << 3)) =
              fp8x8_to_bf16(make_uint2(st.b[i][2], st.b[i][3]));
        } else {
          __bf16* B = lds_b + buf * TN * kLdsRow + swz(b_r, b_c);
          *reinterpret_cast<u32x4*>(B + i * BRPI * kLdsRow) = st.b[i];
        }
      }
    };

    constexpr int PF = (WF == kFP8) ? MF : 1;   // fp8: per-block partial sums
    f32x4 acc[MF][NF], part[PF][(WF == kFP8) ? NF : 1];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int j = 0; j < NF; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < PF; ++i)
#pragma unroll
      for (int j = 0; j < ((WF == kFP8) ? NF : 1); ++j) part[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    Stage stage{};
    stage = gload(0, stage);
    lstore(0, stage);
    __syncthreads();
    for (int kb = 0; kb < nkb; ++kb) {
      const int buf = kb & 1;
      if (kb + 1 < nkb) stage = gload(kb + 1, stage);
      const __bf16* A = lds_a + buf * TM * kLdsRow;
      const __bf16* B = lds_b + buf * TN * kLdsRow;
#pragma unroll
      for (int ks = 0; ks < kTK / 32; ++ks) {
        // all fragment reads of this 32-long step first, then the MFMAs, so that the LDS
        // latency of later fragments overlaps the MFMAs of earlier ones
        const int chunk = ks * 4 + (lane >> 4);
        bf16x8 bfr[NF], afr[MF];
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
          bfr[nf] = *reinterpret_cast<const bf16x8*>(B + swz(wn * WN + nf * 16 + (lane & 15), chunk));
#pragma unroll
        for (int mf = 0; mf < MF; ++mf)
          afr[mf] = *reinterpret_cast<const bf16x8*>(A + swz(wm * WM + mf * 16 + (lane & 15), chunk));
#pragma unroll
        for (int mf = 0; mf < MF; ++mf)
#pragma unroll
          for (int nf = 0; nf < NF; ++nf) {
            if constexpr (WF == kFP8)
              part[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[mf], bfr[nf], part[mf][nf], 0, 0, 0);
            else
              acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[mf], bfr[nf], acc[mf][nf], 0, 0, 0);
          }
      }
      if constexpr (WF == kFP8) {
        // end of a 128-long contraction block (two steps): scale the partial sums
        if ((kb & 1) == 1 || kb + 1 == nkb) {
          const int kb128 = (kb * kTK) / 128;
#pragma unroll
          for (int nf = 0; nf < NF; ++nf) {
            const int t = wn * WN + nf * 16;       // LDS tile row of this fragment
            const float* S = is_up(t) ? p.S2 : p.S1;
            const float sc = S[((size_t)e * nNB128 + wrow(t) / 128) * nKB128 + kb128];
#pragma unroll
            for (int mf = 0; mf < MF; ++mf) {
#pragma unroll
              for (int j = 0; j < 4; ++j) acc[mf][nf][j] = fmaf(sc, part[mf][nf][j], acc[mf][nf][j]);
              part[mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
          }
        }
      }
      if (kb + 1 < nkb) lstore(buf ^ 1, stage);
      __syncthreads();
    }

    // epilogue from registers: lane holds rows (lane/16)*4 + j, column lane%16 of each fragment
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wm * WM + mf * 16 + (lane >> 4) * 4 + j;
        if (r >= nrows) continue;
        const size_t orow = (size_t)(r0 + r) * p.N;
        if constexpr (GATED) {
#pragma unroll
          for (int nf = 0; nf < NF / 2; ++nf) {
            const int col = c0 + wn * (WN / 2) + nf * 16 + (lane & 15);
            if (col < p.N)
              static_cast<__bf16*>(p.out)[orow + col] = (__bf16)(silu(acc[mf][nf][j]) * acc[mf][nf + NF / 2][j]);
          }
        } else {
#pragma unroll
          for (int nf = 0; nf < NF; ++nf) {
            const int col = c0 + wn * WN + nf * 16 + (lane & 15);
            if (col < p.N) static_cast<float*>(p.out)[orow + col] = acc[mf][nf][j];
          }
        }
      }
  }
}

template <int WF, bool GATED, int WM, int WN, int WGM, int WGN>
static hipError_t launch_tiled(const TiledArgs& p, const DeviceInfo& dev, hipStream_t stream) {
  constexpr int NTH = 64 * WGM * WGN;
  const size_t lds = ((size_t)(p.E + 1 + 3) / 4 * 4 * 2 + NTH) * sizeof(int32_t) +
                     (size_t)2 * (WGM * WM + WGN * WN) * kLdsRow * sizeof(__bf16);
  auto kern = &ffn_tiled_kernel<WF, GATED, WM, WN, WGM, WGN>;
  if (lds > 64 * 1024) {
    hipError_t st = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (st != hipSuccess) return st;
  }
  const int per_cu = lds > 80 * 1024 ? 1 : 2;
  kern<<<dev.num_cus * per_cu, NTH, lds, stream>>>(p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Tiled kernel with direct-to-LDS operand loads (bf16 or fp8 weights). Same tile decomposition
// as ffn_tiled_kernel, but operands go from memory straight into LDS (buffer loads into LDS, 16
// bytes per lane, no register staging) through a ring of RING contraction steps of DK
// elements. A step's slot is refilled as soon as every wave holds the fragments of the step's
// last 32-wide slice in registers, and the fragment reads of each slice overlap the MFMAs of
// the one before, so the MFMA pipe waits neither on LDS reads nor on the barrier's refill.
// Shapes:
//  - prefill, 256 x 256 tiles, DK = 64, 2 slots (128 KB): the operands mostly hit in L2, one
//    barrier per 64-wide step (32-wide steps in 4 slots, twice the barriers with 1.5x the bytes
//    in flight, measured 9% slower), the next step's loads in flight while the MFMAs consume
//    the current one;
//  - decode, 64 x 128 tiles, DK = 64, 3 slots, two workgroups per CU: weight streaming, where
//    each weight row is read a full 128-byte line per step (64-byte pieces of many rows
//    measured ~15% below line-sized ones in HBM throughput);
//  - prefill fp8: 128 x 256 tiles, DK = 128 (one step per scale block), 2 slots of 64 KB
//    (8.5% faster than 64-wide steps in 4 slots).
// The loading lanes pick their source addresses so that the linear LDS image is the swizzled
// tile (see dswz).
constexpr int kDK = 64;     // contraction step
constexpr int kFp8DlMaxK = 65536;  // longest contraction of the fp8 direct-to-LDS kernel
// Word 3 of a raw buffer descriptor (32-bit data format, bounds-checked offsets): loads at or
// past num_records bytes return zeros.
constexpr int kBufferWord3 = 0x00020000;

// 16 bytes per lane from a buffer into LDS at lds + 16 * lane (the loads are wrapped in a device
// function: called directly from a kernel template, the host compilation pass drops the
// kernel's launch stub)
// AUX is the load's cache policy; kNonTemporal marks data read once (streamed weights), so its
// lines are the first to leave the L2 and do not push out the operands other tiles reuse.
constexpr int kNonTemporal = 2;  // the nt bit of the gfx950 cache-policy field
template <int AUX = 0>
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t rsrc, void* lds, int voffset,
                                                  int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16,
                                           voffset, soffset, 0, AUX);
}
constexpr int kRing = 4;    // LDS ring depth
// contraction split (decode-sized launches with few tiles): at most kSplitMaxUnits chunks, each
// with a partial tile of kSplitTileElems fp32 values
constexpr int kSplitMaxUnits = 512;
constexpr int kSplitTileElems = 64 * 128;
constexpr int kSplitMaxChunks = 16;  // the sum keeps one fragment's chunks in registers
constexpr int kTailMaxUnits = 256;   // chunks of a prefill launch's last round

// LDS image of a tile row of CPR chunks of 16 bytes: chunk c of row r sits at chunk c ^ x(r),
// x(r) = (r >> 2) & 3 for 4 chunks, (r >> 1) & 7 for 8 and r & 15 for 16, so that the 16 rows
// read by one fragment load (same chunk) fall on distinct banks.
template <int CPR>
__device__ __forceinline__ int dswz(int row, int chunk) {
  static_assert(CPR == 4 || CPR == 8 || CPR == 16, "row width");
  if constexpr (CPR == 4) return row * 4 + (chunk ^ ((row >> 2) & 3));
  else if constexpr (CPR == 8) return row * 8 + (chunk ^ ((row >> 1) & 7));
  else return row * 16 + (chunk ^ (row & 15));
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8; the others are left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>), in order
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}
// s_waitcnt lgkmcnt(0) alone (vmcnt and expcnt at their maxima)
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}
// the same with a wave-uniform runtime count in [0, MAX] (a scalar branch per candidate)
template <int... Ns>
__device__ __forceinline__ void wait_vmcnt_dyn_impl(int n, std::integer_sequence<int, Ns...>) {
  ((n == Ns ? (wait_vmcnt<Ns>(), 0) : 0), ...);
}
template <int MAX>
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  wait_vmcnt_dyn_impl(n, std::make_integer_sequence<int, MAX + 1>{});
}

// Epilogue of one tile: rows below nrows and columns below N of the accumulator tile go out;
// the gated GEMM writes h = silu(gate) * up in bf16, the other one fp32.
template <bool GATED, int WM, int WN, int MF, int NF>
__device__ __forceinline__ void tile_epilogue_impl(const TiledArgs& p, const f32x4 (&acc)[MF][NF],
                                                   int wm, int wn, int lane, int r0, int nrows,
                                                   int c0, int mf_only, int nf_only) {
#pragma unroll
  for (int mf = 0; mf < MF; ++mf)
#pragma unroll
    for (int jr = 0; jr < 4; ++jr) {
      if (mf_only >= 0 && mf != mf_only) continue;  // another unit's fragment rows
      const int r = wm * WM + mf * 16 + (lane >> 4) * 4 + jr;
      if (r >= nrows) continue;
      const size_t orow = (size_t)(r0 + r) * p.N;
      if constexpr (GATED) {
#pragma unroll
        for (int nf = 0; nf < NF / 2; ++nf) {
          if (nf_only >= 0 && nf != nf_only) continue;
          const int col = c0 + wn * (WN / 2) + nf * 16 + (lane & 15);
          if (col < p.N)
            static_cast<__bf16*>(p.out)[orow + col] = (__bf16)(silu(acc[mf][nf][jr]) * acc[mf][nf + NF / 2][jr]);
        }
      } else {
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) {
          if (nf_only >= 0 && nf != nf_only) continue;
          const int col = c0 + wn * WN + nf * 16 + (lane & 15);
          if (col < p.N) static_cast<float*>(p.out)[orow + col] = acc[mf][nf][jr];
        }
      }
    }
}

// WF: weight format, kBF16 or kFP8 (e4m3fn with fp32 scales per 128 x 128 block). fp8 weights
// go to LDS as bytes and are widened to bf16 exactly after the fragment load; the MFMAs of one
// 128-long contraction block accumulate into a partial tile that is then added to the
// accumulator times the block's scale (identical dequantisation: the scale multiplies the
// exact fp8 products' fp32 sum, never a rounded weight). fp8 needs DK >= 64 (a scale block is
// one or two steps).
// The tile loop of one workgroup, which is rank `rank` of `nranks` workgroups sharing the
// tiles of the experts with more than min_rows and at most max_rows rows.
// MODE 0 runs whole tiles. With few tiles, MODE 1 cuts each tile's contraction into S chunks
// of consecutive steps, one per workgroup, and stores each chunk's fp32 partial tile; MODE 3
// runs the rounds in which every workgroup has a tile whole and cuts only the last, partial
// round's tiles that way. MODE 2 (a second launch) adds a tile's S partials in chunk order and
// applies the epilogue, so the result does not depend on timing and needs no synchronisation
// inside a launch.
// HYB (the large prefill tiles): an expert's rows are dealt to its row tiles in whole 16-row
// fragments as evenly as the tile count allows (300 rows: two tiles of 10 and 9 fragments, not
// 256 + 44), so that the row tiles of one column block, which run side by side on one XCD and
// read the same weights, take about the same time; and each wave runs a body compiled for the
// number of its 16-row fragments that hold rows (absent ones take no LDS reads and no MFMAs),
// so a partial tile costs what its fragments need while every body keeps a branch-free inner
// loop.
template <int WF, bool GATED, int WM, int WN, int WGM, int WGN, int RING = kRing, int DK = kDK,
          bool ASKIP = false, int MODE = 0, bool HYB = false>
__device__ __forceinline__ void dl_tiles(const TiledArgs& p, unsigned char* smem, int rank,
                                         int nranks, int min_rows, int max_rows) {
  static_assert(DK == 64 || DK == 128, "contraction step: an even number of 32-wide slices");
  static_assert(WF == kBF16 || (WF == kFP8 && DK >= 64), "weight format");
  static_assert(MODE == 0 || !ASKIP, "contraction split: every row loaded");
  static_assert(!HYB || !ASKIP, "row skipping is chosen per tile");
  static_assert(MODE != 1 || (WF == kBF16 && WGM * WM * WGN * WN <= kSplitTileElems),
                "decode contraction split: bf16 weights, tiles of at most 64 x 128");
  constexpr bool F8 = WF == kFP8;
  constexpr int WB = F8 ? 1 : 2;                        // weight bytes per element
  constexpr bool BLKOK = DK * WB == 128;                 // a step reads 128 bytes of a B row:
                                                        // the shapes that read blocked weights
  constexpr int NW = WGM * WGN, NTH = 64 * NW;
  constexpr int TM = WGM * WM, TN = WGN * WN;
  constexpr int MF = WM / 16, NF = WN / 16;
  constexpr int CPRA = DK * 2 / 16, CPRB = DK * WB / 16;  // 16-byte chunks per tile row
  constexpr int AI = TM * CPRA / 64, BI = TN * CPRB / 64;  // 1 KB load instructions per step
  static_assert(BI % NW == 0 && (AI % NW == 0 || AI < NW), "loads must split evenly over waves");
  // A loads per wave: AI / NW each, or (short tiles) one each for the first AI waves
  constexpr int AIW = AI >= NW ? AI / NW : 1, BIW = BI / NW;
  constexpr int LPW = AIW + BIW;                        // most loads per wave per step
  constexpr int ACH = TM * CPRA;                        // A chunks per ring slot
  constexpr int STAGE = ACH + TN * CPRB;                // 16-byte chunks per ring slot
  constexpr int KBS = 128 / DK;                         // steps per fp8 scale block
  const int Epad = (p.E + 1 + 3) & ~3;
  int32_t* pre = reinterpret_cast<int32_t*>(smem);
  int32_t* offs = pre + Epad;
  int32_t* scan_tmp = offs + Epad;
  u32x4* ring = reinterpret_cast<u32x4*>(scan_tmp + ((NTH + 3) & ~3));   // [RING][STAGE]
  // fp8: the current item's scales, [WGN column blocks][gate, up][K / 128], read from LDS in
  // the loop (a global load there would make the compiler drain the prefetched steps)
  float* sc_lds = reinterpret_cast<float*>(ring + RING * STAGE);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool loads_a = AI >= NW || wave < AI;  // wave-uniform
  // HYB: waves w and w + 4 share a SIMD (the hardware deals a workgroup's waves to the four
  // SIMDs in turn), so wave w takes the row block w / WGN: with two row blocks the two waves of a
  // SIMD own different halves of the tile, and a tile whose rows fill only the upper half still
  // keeps every SIMD busy with half the work.
  const int wm = HYB ? wave / WGN : wave % WGM, wn = HYB ? wave % WGN : wave / WGM;
  constexpr int cols_per_tile = GATED ? TN / 2 : TN;
  const int NT = (p.N + cols_per_tile - 1) / cols_per_tile;
  build_item_prefix(pre, scan_tmp, p.offsets, p.E, p.rows, max_rows, NT, offs, min_rows, TM);
  int total = __builtin_amdgcn_readfirstlane(pre[p.E]);
  const int nst = p.K / DK;  // K is a multiple of 64 (of 128 for fp8) on this path
  const size_t wstride = (size_t)p.N * p.K * WB;  // bytes per expert matrix
  const int NB = p.N / 128, KBn = p.K / 128;     // fp8 scale blocks

  auto tile_epilogue = [&](const TiledArgs& pp, const f32x4 (&a)[MF][NF], int wm_, int wn_, int lane_,
                           int r0_, int nrows_, int c0_, int mf_only = -1, int nf_only = -1) __attribute__((always_inline)) {
    tile_epilogue_impl<GATED, WM, WN, MF, NF>(pp, a, wm_, wn_, lane_, r0_, nrows_, c0_, mf_only, nf_only);
  };
  // tile of item `item`: expert, first row, rows, first column
  auto tile_of = [&](int item, int& e, int& r0, int& nrows, int& c0) __attribute__((always_inline)) {
    int lo = 0, hi = p.E;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (__builtin_amdgcn_readfirstlane(pre[mid]) <= item) lo = mid; else hi = mid - 1;
    }
    e = lo;
    const int local = item - __builtin_amdgcn_readfirstlane(pre[e]);
    constexpr int kGroupM = 4;
    const int ebeg = __builtin_amdgcn_readfirstlane(offs[e]);
    const int MT = (__builtin_amdgcn_readfirstlane(offs[e + 1]) - ebeg + TM - 1) / TM;
    const int g = local / (kGroupM * NT);
    const int gm = min(kGroupM, MT - g * kGroupM);
    const int j = local - g * kGroupM * NT;
    const int nt = j / gm;
    const int mt = g * kGroupM + j % gm;
    if constexpr (HYB) {
      // fragments dealt evenly: the first fr % MT tiles take one more (at most TM / 16 each,
      // at least one, since MT = ceil(n / TM)); the ragged last fragment ends the last tile
      const int fr = (__builtin_amdgcn_readfirstlane(offs[e + 1]) - ebeg + 15) / 16;
      const int q = fr / MT, rem = fr - q * MT;
      r0 = ebeg + 16 * (mt * q + min(mt, rem));
      nrows = min(16 * (q + (mt < rem ? 1 : 0)), __builtin_amdgcn_readfirstlane(offs[e + 1]) - r0);
    } else {
      r0 = ebeg + mt * TM;
      nrows = min(TM, __builtin_amdgcn_readfirstlane(offs[e + 1]) - r0);
    }
    c0 = nt * cols_per_tile;
  };

  // contraction split: S chunks per tile (at least 2 steps each), so that the tile count times S
  // fits the split launch's grid and the partial buffer; the same in both split launches
  // Tail split (MODE 3, prefill): the rounds in which every workgroup has a tile run whole
  // tiles; the tiles of the last, partial round (first_split .. total) are cut into S chunks
  // so that the round keeps every workgroup busy, and a second launch (MODE 2) adds them.
  int S = 1, first_split = 0;
  if constexpr (MODE == 1) {
    const int units_max = min(kSplitMaxUnits, p.split_ranks);
    S = max(1, min(min(kSplitMaxChunks, max(1, nst / 2)), units_max / max(total, 1)));
  } else if constexpr (MODE == 2) {
    if (p.split_info) {
      // the header of the launch before: accepted only if its chunks fit the partial buffer
      // (anything else is treated as no split)
      S = p.split_info[0];
      first_split = p.split_info[1];
      const int end = p.split_info[2];
      const bool ok = S >= 1 && S <= kSplitMaxChunks && first_split >= 0 && end >= first_split &&
                      end <= total && (long long)(end - first_split) * S <= kTailMaxUnits;
      if (!ok) { S = 1; first_split = total; }
      else total = end;  // items past the split range were finished whole
    } else {
      const int units_max = min(kSplitMaxUnits, p.split_ranks);
      S = max(1, min(min(kSplitMaxChunks, max(1, nst / 2)), units_max / max(total, 1)));
    }
  } else if constexpr (MODE == 3) {
    first_split = total / nranks * nranks;
    const int R = total - first_split;
    if (R > 0) S = max(1, min(min(kSplitMaxChunks, max(1, nst / 2)), min(nranks, kTailMaxUnits) / R));
    if (S == 1) first_split = total;  // nothing to split
    if (rank == 0 && tid == 0 && p.split_info) {
      p.split_info[0] = S;
      p.split_info[1] = first_split;
      p.split_info[2] = S > 1 ? total : first_split;
    }
  }
  constexpr int kSlot = MF * NF * 4 * NTH;  // floats of one partial tile, in register order
  // partial tile fragment (mf, nf) of thread tid sits at ((mf * NF + nf) * NTH + tid) * 4
  if constexpr (MODE == 2) {
    // one unit per (tile, 16-row fragment index, 16-column fragment index; gated tiles keep
    // a gate column fragment and its up partner together): MF * NFU workgroups per tile
    constexpr int NFU = GATED ? NF / 2 : NF;
    for (int u = rank; u < (total - first_split) * MF * NFU; u += nranks) {
      const int item = first_split + u / (MF * NFU), mfu = (u / NFU) % MF, nfu = u % NFU;
      int e, r0, nrows, c0;
      tile_of(item, e, r0, nrows, c0);
      f32x4 acc[MF][NF];
      const float* first = p.partial + (size_t)(item - first_split) * S * kSlot;
#pragma unroll
      for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) {
          f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
          // fragments of absent rows hold nothing; other fragments belong to other units
          if (mf == mfu && (nf == nfu || (GATED && nf == nfu + NF / 2)) && wm * WM + mf * 16 < nrows) {
            // every chunk's load is in flight before the sum, which then goes in chunk order
            f32x4 v[kSplitMaxChunks];
#pragma unroll
            for (int c = 0; c < kSplitMaxChunks; ++c)
              if (c < S)
                v[c] = *reinterpret_cast<const f32x4*>(first + (size_t)c * kSlot + ((mf * NF + nf) * NTH + tid) * 4);
#pragma unroll
            for (int c = 0; c < kSplitMaxChunks; ++c)
              if (c < S) sum += v[c];
          }
          acc[mf][nf] = sum;
        }
      tile_epilogue(p, acc, wm, wn, lane, r0, nrows, c0, mfu, nfu);
    }
    return;
  }

  // units: whole tiles first (MODE 0 and 3), then S chunks per split tile
  const int units = first_split + (total - first_split) * S;
  for (int base = 0; base < units; base += nranks) {
    const int unit = xcd_round_item(base, units, rank, nranks);
    if (unit < 0) continue;  // uniform per workgroup
    const bool split = unit >= first_split && S > 1;
    const int item = split ? first_split + (unit - first_split) / S : unit;
    const int chunk = split ? (unit - first_split) % S : 0;
    const int st_lo = split ? chunk * nst / S : 0, st_hi = split ? (chunk + 1) * nst / S : nst;
    int e, r0, nrows, c0;
    tile_of(item, e, r0, nrows, c0);
    // MFP: this wave's 16-row fragments that hold rows of the tile, fixed at compile time (HYB:
    // one body per count, so the fragment loop has no branches), or -1: checked at run time
    // (ASKIP)
    auto run_tile = [&](auto mfp_tag) __attribute__((always_inline)) {
      constexpr int MFP = decltype(mfp_tag)::value;
      auto present = [&](int mf) __attribute__((always_inline)) {
        return MFP >= 0 ? mf < MFP : !(ASKIP && wm * WM + mf * 16 >= nrows);
      };
      // Weight tiles of an expert whose rows fit one row tile are read exactly once: in the decode
      // tiles and the streaming role they load with the non-temporal policy, so they leave the
      // L2 first and the weights of experts with several row tiles stay there for their re-reads
      // (c2 FFN -7%, c3 -6.5%). The large prefill tiles keep the default policy (+3.8% at c4 with
      // the same rule).
      const bool b_once = (ASKIP || MODE == 0 || MODE == 1) &&
                          __builtin_amdgcn_readfirstlane(offs[e + 1]) -
                                  __builtin_amdgcn_readfirstlane(offs[e]) <= TM;
      // With ASKIP, A load instructions whose rows all lie past the expert's last row are not
      // issued (HYB: they are issued out of the descriptor's range, which reads nothing and
      // keeps the load count fixed), and the 16-row fragments past it take no LDS reads and no
      // MFMAs: those LDS rows keep stale data or zeros, which could only reach accumulator rows
      // that are never stored (row r of the product depends on row r of A alone).
      constexpr int RPI = 64 / CPRA;  // tile rows per A load instruction
      int aiw = 0;
  #pragma unroll
      for (int i = 0; i < AIW; ++i)
        aiw += (loads_a && (!ASKIP || (wave + i * NW) * RPI < nrows)) ? 1 : 0;
      const int lpw = aiw + BIW;  // this wave's loads per step

      // Loads are buffer loads into LDS: a descriptor per operand holds the tile's base and its
      // byte extent (rows past the expert's last row, or past the last column, read as zeros, so
      // nothing is clamped), one 32-bit lane offset serves all of a wave's load instructions, and
      // the per-instruction and per-step parts are wave-uniform scalar offsets. That keeps the
      // address registers at two, whatever the number of load instructions.
      // Instruction i of this wave covers tile rows shifted by i * NW * rows-per-instruction; the
      // XOR swizzle of a row repeats with that period, so the lane's chunk is the same for all i.
      const uint8_t* Xt = static_cast<const uint8_t*>(p.X) + (size_t)r0 * p.K * 2;
      const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
          (void*)Xt, (short)0, (int)((unsigned)nrows * (unsigned)p.K * 2u), kBufferWord3);
      const size_t wcol = (size_t)c0 * p.K * WB;  // the tile's first B row (weight row c0)
      const size_t bbytes = (size_t)(p.N - c0) * p.K * WB;
      const unsigned bext = bbytes > 0xffffffffu ? 0xffffffffu : (unsigned)bbytes;
      const __amdgpu_buffer_rsrc_t rB1 = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(static_cast<const uint8_t*>(p.W1) + (size_t)e * wstride + wcol), (short)0, (int)bext, kBufferWord3);
      const __amdgpu_buffer_rsrc_t rB2 = GATED ? __builtin_amdgcn_make_buffer_rsrc(
          (void*)(static_cast<const uint8_t*>(p.W2) + (size_t)e * wstride + wcol), (short)0, (int)bext, kBufferWord3) : rB1;
      constexpr int RPA = 64 / CPRA, RPB = 64 / CPRB;  // tile rows per load instruction
      int a_lane, b_lane;  // byte offsets of instruction 0 (this lane)
      {
        const int q = wave * 64 + lane;
        const int r = q / CPRA, c = dswz<CPRA>(r, q % CPRA) - r * CPRA;  // source chunk (XOR involution)
        a_lane = (r * p.K * 2) + c * 16;
      }
      // B row t of the tile -> weight row offset from c0 (gated tiles interleave gate and up
      // halves of WN rows per wave block)
      auto b_row = [&](int t) __attribute__((always_inline)) {
        return GATED ? (t / WN) * (WN / 2) + (t % WN) % (WN / 2) : t;
      };
      {
        const int q = wave * 64 + lane;
        const int t = q / CPRB, c = dswz<CPRB>(t, q % CPRB) - t * CPRB;
        b_lane = b_row(t) * p.K * WB + c * 16;
        // blocked weights: a load instruction's 8 rows (b_row(t) & 7 is this lane's row among
        // them, the first is a multiple of 8) are one 1 KB block per step, row r at r * 128
        if constexpr (BLKOK)
          if (p.wblk) b_lane = (b_row(t) & ~7) * p.K * WB + (b_row(t) & 7) * 128 + c * 16;
      }
      const int t0w = wave * RPB;  // first B row of this wave's instruction 0 (wave-uniform)
      // bytes between steps in a B row: DK elements, or one 1 KB block (blocked weights)
      const int kbstep = (BLKOK && p.wblk) ? 1024 : DK * WB;

      auto issue = [&](int st) __attribute__((always_inline)) {
        u32x4* slot = ring + (st % RING) * STAGE;
        const int ka = st * DK * 2, kb = st * kbstep;
  #pragma unroll
        for (int i = 0; i < AIW; ++i)
          if (loads_a && (!ASKIP || (wave + i * NW) * RPA < nrows))
            buffer_load_lds16(rA, slot + (wave + i * NW) * 64, a_lane,
                              (HYB && (wave + i * NW) * RPA >= nrows) ? 0x40000000
                                                                      : i * NW * RPA * p.K * 2 + ka);
  #pragma unroll
        for (int i = 0; i < BIW; ++i) {
          const int ti = t0w + i * NW * RPB;  // first row of instruction i (wave-uniform)
          const bool up = GATED && (ti % WN) >= WN / 2;
          if (b_once)
            buffer_load_lds16<kNonTemporal>(up ? rB2 : rB1, slot + ACH + (wave + i * NW) * 64, b_lane,
                                            (b_row(ti) - b_row(t0w)) * p.K * WB + kb);
          else
            buffer_load_lds16<0>(up ? rB2 : rB1, slot + ACH + (wave + i * NW) * 64, b_lane,
                                 (b_row(ti) - b_row(t0w)) * p.K * WB + kb);
        }
      };

      f32x4 acc[MF][NF];
      f32x4 part[F8 ? MF : 1][F8 ? NF : 1];  // fp8: this scale block's sums
  #pragma unroll
      for (int i = 0; i < MF; ++i)
  #pragma unroll
        for (int jj = 0; jj < NF; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (F8) {
  #pragma unroll
        for (int i = 0; i < MF; ++i)
  #pragma unroll
          for (int jj = 0; jj < NF; ++jj) part[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // fp8: stage the scale rows of every wave column block (gate and up halves for the gated
      // GEMM) in LDS; nothing is in flight here, the previous item ended with a full drain
      if constexpr (F8) {
        for (int idx = tid; idx < WGN * 2 * KBn; idx += NTH) {
          const int blk = idx / (2 * KBn), half = (idx / KBn) & 1, kb = idx % KBn;
          const int n0 = GATED ? c0 + blk * (WN / 2) : c0 + blk * WN;
          const size_t srow = ((size_t)e * NB + min(n0 / 128, NB - 1)) * KBn + kb;
          sc_lds[idx] = (GATED && half) ? p.S2[srow] : (half ? 0.f : p.S1[srow]);
        }
        __syncthreads();
      }

      // Software pipeline over 32-wide contraction slices: the fragments of the next slice are read
      // from LDS while the MFMAs of the current one run (B fragments into the other of two
      // register sets, A fragment mf right after its last MFMA of the current slice), so the MFMA
      // pipe never waits for a fresh read. The barrier that hands a step's slot back sits before
      // the MFMAs of the step's last slice, whose fragments are already in registers.
      constexpr int NS = DK / 32;  // slices per step (even)
      // k order inside a step. bf16: slice h, lane L holds k = 32h + 8(L/16) .. +7 (16-byte chunk
      // 4h + L/16 of the A and B rows). fp8: a B chunk of 16 bytes holds 16 k, so a lane reads
      // chunk 4j + L/16 of its B row once for the slice pair (2j, 2j+1), its bytes 0-7 in slice 2j
      // and 8-15 in slice 2j+1, and A follows the same k (bf16 chunks 8j + 2(L/16) + {0, 1}). Any
      // k order is the same contraction as long as A and B agree.
      auto read_a = [&](const u32x4* slot, int h, int mf, bf16x8& dst) __attribute__((always_inline)) {
        const int c = F8 ? (h >> 1) * 8 + (lane >> 4) * 2 + (h & 1) : h * 4 + (lane >> 4);
        const u32x4 v = slot[dswz<CPRA>(wm * WM + mf * 16 + (lane & 15), c)];
        __builtin_memcpy(&dst, &v, 16);
      };
      // B chunk of 16-row fragment nf: bf16, the chunk of slice h; fp8, the chunk of slice pair h/2
      auto read_b = [&](const u32x4* slot, int h, int nf, u32x4& dst) __attribute__((always_inline)) {
        const int c = F8 ? (h >> 1) * 4 + (lane >> 4) : h * 4 + (lane >> 4);
        dst = slot[ACH + dswz<CPRB>(wn * WN + nf * 16 + (lane & 15), c)];
      };
      auto bar = [&]() __attribute__((always_inline)) {
        // A bare s_barrier: a fence here would make the compiler drain all outstanding
        // direct-to-LDS loads. The signal fences only stop the compiler from moving LDS accesses
        // across the barrier.
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
      };
      bf16x8 afr[MF];
      // B chunks: bf16, those of the current slice and of the next; fp8, one set (a slice pair's)
      u32x4 bq[F8 ? 1 : 2][NF];
      // the whole ring is free (the previous item ended with a barrier after its last reads)
  #pragma unroll
      for (int r = 0; r < RING; ++r)
        if (st_lo + r < st_hi) issue(st_lo + r);
      // this wave's loads of the first step are done once at most the later steps' are pending
      wait_vmcnt_dyn<(RING - 1) * LPW>(min(RING - 1, st_hi - 1 - st_lo) * lpw);
      bar();
      {
        const u32x4* slot = ring + (st_lo % RING) * STAGE;
  #pragma unroll
        for (int nf = 0; nf < NF; ++nf) read_b(slot, 0, nf, bq[0][nf]);
  #pragma unroll
        for (int mf = 0; mf < MF; ++mf)
          if (present(mf)) read_a(slot, 0, mf, afr[mf]);
      }
      for (int st = st_lo; st < st_hi; ++st) {
        const u32x4* slot = ring + (st % RING) * STAGE;
        const u32x4* nslot = ring + ((st + 1) % RING) * STAGE;
        static_for<NS>([&](auto hc) __attribute__((always_inline)) {
          constexpr int h = decltype(hc)::value;
          constexpr int P = h & 1;  // B register set of this slice (bf16)
          // The next slice is read whether or not it exists: past the item's last step the reads
          // land in registers that are never used (in-bounds LDS, no loads in flight), which keeps
          // the code free of branches and the compiler's read counts exact.
          if (h == NS - 1) {
            wait_lgkmcnt0();  // this wave's reads of step st are back
            if (st + 1 < st_hi) {
              // the next slice opens step st+1: this wave's loads of it have landed (at most the
              // later steps' are pending), and after the barrier both hold for every wave, so
              // step st's slot takes step st+RING
              wait_vmcnt_dyn<(RING - 2) * LPW>(min(RING - 2, st_hi - 2 - st) * lpw);
              bar();
              if (st + RING < st_hi) issue(st + RING);
            }
          }
          // fp8: the wave issuing a slice's conversions, MFMAs and reads runs at raised priority, so
          // the SIMD's other wave, in its barrier or load issue, does not hold it back (c5 FFN -2%;
          // bf16 tiles measured 0.5% slower with it)
          if constexpr (F8) __builtin_amdgcn_s_setprio(1);
          const u32x4* rs = h + 1 < NS ? slot : nslot;
          const int rh = (h + 1) % NS;
          bf16x8 bfr[NF];
  #pragma unroll
          for (int nf = 0; nf < NF; ++nf) {
            if constexpr (F8) {
              const u32x4 v = bq[0][nf];
              bfr[nf] = fp8x8_to_bf16((h & 1) ? make_uint2(v[2], v[3]) : make_uint2(v[0], v[1]));
            } else {
              __builtin_memcpy(&bfr[nf], &bq[P][nf], 16);
            }
          }
          // next B chunks: bf16 every slice (into the other set); fp8 after the second slice of a
          // pair has been widened (into the same set)
          constexpr int NBR = F8 ? ((h & 1) ? NF : 0) : NF;
          if constexpr (NBR > 0 && MFP != 0) {
  #pragma unroll
            for (int nf = 0; nf < NF; ++nf) read_b(rs, rh, nf, bq[F8 ? 0 : P ^ 1][nf]);
          }
  #pragma unroll
          for (int mf = 0; mf < MF; ++mf) {
            if (!present(mf)) continue;  // wave-uniform: absent rows
  #pragma unroll
            for (int nf = 0; nf < NF; ++nf) {
              if constexpr (F8)
                part[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[mf], bfr[nf], part[mf][nf], 0, 0, 0);
              else
                acc[mf][nf] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr[mf], bfr[nf], acc[mf][nf], 0, 0, 0);
            }
            read_a(rs, rh, mf, afr[mf]);
          }
          // instruction order of the slice: the B reads, then per 16-row fragment its MFMAs and
          // the read of its next A fragment
          if constexpr (NBR > 0 && MFP != 0) __builtin_amdgcn_sched_group_barrier(0x100, NBR, 0);
  #pragma unroll
          for (int mf = 0; mf < (MFP >= 0 ? MFP : MF); ++mf) {
            __builtin_amdgcn_sched_group_barrier(0x008, NF, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          // the reads stay in this slice (not sunk to their first use)
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          if constexpr (F8) __builtin_amdgcn_s_setprio(0);
          if constexpr (F8) {
            if (h == NS - 1 && (st + 1) % KBS == 0) {  // end of a 128-long scale block
              const int kb = st / KBS;
              const float s0 = sc_lds[(wn * 2) * KBn + kb];
              const float s1 = GATED ? sc_lds[(wn * 2 + 1) * KBn + kb] : s0;
  #pragma unroll
              for (int mf = 0; mf < MF; ++mf)
  #pragma unroll
                for (int nf = 0; nf < NF; ++nf) {
                  const float sc = (GATED && nf >= NF / 2) ? s1 : s0;
                  acc[mf][nf] += sc * part[mf][nf];
                  part[mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            }
          }
        });
      }
      __syncthreads();  // all waves done reading the ring before the next item refills it
      if (MODE == 1 || (MODE == 3 && split)) {
        float* mine = p.partial + ((size_t)(item - first_split) * S + chunk) * kSlot;
  #pragma unroll
        for (int mf = 0; mf < MF; ++mf) {
          if (wm * WM + mf * 16 >= nrows) continue;  // absent rows: nothing to keep
  #pragma unroll
          for (int nf = 0; nf < NF; ++nf)
            *reinterpret_cast<f32x4*>(mine + ((mf * NF + nf) * NTH + tid) * 4) = acc[mf][nf];
        }
      } else {
        tile_epilogue(p, acc, wm, wn, lane, r0, nrows, c0);
      }
    };
    if constexpr (HYB) {
      // this wave's present fragments (wave-uniform), one body per count
      const int nfw = __builtin_amdgcn_readfirstlane(min(MF, max(0, (nrows - wm * WM + 15) / 16)));
      static_for<MF + 1>([&](auto c) __attribute__((always_inline)) {
        if (nfw == decltype(c)::value) run_tile(std::integral_constant<int, decltype(c)::value>{});
      });
    } else {
      run_tile(std::integral_constant<int, ASKIP ? -1 : MF>{});
    }
  }
}

template <int WF, bool GATED, int WM, int WN, int WGM, int WGN, int RING = kRing, int DK = kDK,
          bool ASKIP = false, int MODE = 0, bool HYB = false>
__global__ __launch_bounds__(64 * WGM * WGN) void ffn_tiled_dl_kernel(TiledArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  dl_tiles<WF, GATED, WM, WN, WGM, WGN, RING, DK, ASKIP, MODE, HYB>(p, smem, blockIdx.x, gridDim.x,
                                                                    p.min_rows, 0x7fffffff);
}

// LDS bytes of dl_tiles for a tile shape (prefix arrays, ring, fp8 scale rows)
template <int WF, int WM, int WN, int WGM, int WGN, int RING, int DK>
static size_t dl_lds_bytes(const TiledArgs& p) {
  constexpr int NTH = 64 * WGM * WGN;
  constexpr int WB = WF == kFP8 ? 1 : 2;
  return ((size_t)(p.E + 1 + 3) / 4 * 4 * 2 + ((NTH + 3) & ~3)) * sizeof(int32_t) +
         (size_t)RING * (WGM * WM * DK * 2 + WGN * WN * DK * WB) +
         (WF == kFP8 ? (size_t)WGN * 2 * (p.K / 128) * sizeof(float) : 0);
}

// Prefill grouped GEMM in one launch with two kinds of workgroups. Experts with at most
// kStreamMaxRows rows only stream their weights (HBM-bound); the others are MFMA-bound tiles
// that mostly hit in L2. The first X workgroups take the small experts in 16-row tiles (COLD
// shape) while the other G - X take the large ones (HOT shape), so the weight streaming runs
// on a few CUs beside the matrix work instead of after it (c4: -8.5%, c5: -11% FFN time against
// separate streaming and tiled launches). X balances the two: bytes of the small experts'
// weights at kColdCuGBps per CU against the large experts' tile flops at kHotCuTflops per CU,
// computed identically by every workgroup from the routed counts. The constants are effective
// rates picked by sweeping them on MI355X (25/30/35/50 GB/s): 30 was best for both prefill
// workloads; the split is coarse (multiples of 8 CUs), and too few streaming CUs costs far more
// than too many.
constexpr float kColdCuGBps = 30.0f;    // weight streaming per CU, GB/s (effective)
constexpr float kHotCuTflops = 4.0f;    // tile MFMA rate per CU, TFLOP/s
// Work of the two kinds of experts of a prefill launch, from the counts, summed by one wave
// (every lane gets the totals; the same code in every kernel that decides from them, so the
// decisions agree): weight bytes of the experts with 1..kStreamMaxRows rows, and tile-padded
// MFMA flops (row tiles of HTM) of the larger ones.
template <bool GATED, int WB, int HTM>
__device__ __forceinline__ void small_large_work(const TiledArgs& p, int lane, float& small_bytes,
                                                 float& large_flops) {
  small_bytes = 0.f;
  large_flops = 0.f;
  for (int e = lane; e < p.E; e += kWave) {
    int a, b;
    expert_rows(p.offsets, e, p.rows, a, b);
    const int n = b - a;
    const float wbytes = (GATED ? 2.f : 1.f) * (float)p.N * (float)p.K * WB;
    const float padded = (float)((n + HTM - 1) / HTM * HTM);
    const float flops = 2.f * padded * (float)p.K * (float)(GATED ? 2 * p.N : p.N);
    small_bytes += (n > 0 && n <= kStreamMaxRows) ? wbytes : 0.f;
    large_flops += n > kStreamMaxRows ? flops : 0.f;
  }
  for (int off = kWave / 2; off >= 1; off >>= 1) {
    small_bytes += __shfl_xor(small_bytes, off);
    large_flops += __shfl_xor(large_flops, off);
  }
}
// The lean kernel (below) takes the small experts when streaming their weights at its rate
// beside the tiles ends no later than the large tiles on all G CUs would; otherwise the
// prefill kernel keeps them in its streaming role and the lean kernel does nothing. Its rate
// beside the large tiles is low, one wave per CU sharing the CU's memory pipeline with them:
// ~0.9 TB/s on 256 CUs (c4 routing: 5.3 GB of gate/up weights in 5.8 ms), so the c4 routing's
// 90 small experts stay in the streaming role while routings with fewer small experts beside
// large ones (Zipf s = 0.6, 1.5, 2.5 at the c4 shape) move to the lean kernel.
constexpr float kLeanCuGBps = 3.5f;  // the lean kernel's streaming rate per CU beside the tiles, GB/s
__device__ __forceinline__ bool lean_takes_small(float small_bytes, float large_flops, int G) {
  return small_bytes > 0.f && large_flops > 0.f &&
         small_bytes / ((float)G * kLeanCuGBps * 1e9f) <= large_flops / ((float)G * kHotCuTflops * 1e12f);
}

template <int WF, bool GATED, int HWM, int HWN, int HRING, int HDK, int CWN, int CRING, int CDK>
__global__ __launch_bounds__(512) void ffn_prefill_kernel(TiledArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int HTM = 2 * HWM, HTN = 4 * HWN;   // hot tiles: 2 x 4 waves
  constexpr int WB = WF == kFP8 ? 1 : 2;
  // work of each kind from the counts (one wave; the others wait at the barrier)
  __shared__ float work[3];
  if (threadIdx.x < kWave) {
    float cold_bytes, hot_flops;
    small_large_work<GATED, WB, HTM>(p, threadIdx.x, cold_bytes, hot_flops);
    if (threadIdx.x == 0) {
      work[0] = cold_bytes / (kColdCuGBps * 1e9f);
      work[1] = hot_flops / (kHotCuTflops * 1e12f);
      work[2] = (p.lean && lean_takes_small(cold_bytes, hot_flops, gridDim.x)) ? 1.f : 0.f;
    }
  }
  __syncthreads();
  const int G = gridDim.x;
  const float tc = work[0], th = work[1];
  // X is a multiple of 8 so that both roles keep the rank -> XCD pairing their tile order
  // relies on (block b runs on XCD b % 8); with the lean kernel taking the small experts every
  // workgroup runs large tiles
  int X = 0;
  if (tc > 0.f) X = th > 0.f ? (int)(G * tc / (tc + th) / 8.f + 0.5f) * 8 : G;
  if (tc > 0.f && X < 8) X = 8 < G ? 8 : G;
  if (th > 0.f && X > G - 8) X = G - 8;
  if (work[2] != 0.f) X = 0;
  X = __builtin_amdgcn_readfirstlane(X);
  __syncthreads();  // `work` is read by every thread before smem is reused
  // no hot role: an empty tail-split header for the launch that adds the chunks
  if (X >= G && blockIdx.x == 0 && threadIdx.x == 0 && p.split_info) {
    p.split_info[0] = 1;
    p.split_info[1] = 0;
    p.split_info[2] = 0;
  }
  // consecutive block indices go to different XCDs, so the first X are spread over all of them
  if ((int)blockIdx.x < X)
    dl_tiles<WF, GATED, 16, CWN, 1, 8, CRING, CDK, true>(p, smem, blockIdx.x, X, 0, kStreamMaxRows);
  else
    dl_tiles<WF, GATED, HWM, HWN, 2, 4, HRING, HDK, false, 3, true>(p, smem, blockIdx.x - X, G - X,
                                                                    kStreamMaxRows, 0x7fffffff);
}

// Lean streaming kernel for the experts with 1..kStreamMaxRows rows of a prefill-sized bf16
// launch, run on a second stream beside ffn_prefill_kernel so that every CU keeps its large
// tiles: a large-tile workgroup leaves 32 VGPRs per SIMD and ~19.5 KB of LDS unused, and this
// kernel's single-wave workgroups fit there (a 32-VGPR budget, which the compiler meets with one
// slice's fragments live at a time; kLeanRing * 6 KB of LDS; the host checks both against the
// code objects before using it). Each
// wave streams its items through a private ring of direct-to-LDS loads (no barriers; the waits
// are its own load counts) that runs on across item boundaries. An item is (expert, 16 gate and
// the same 16 up columns of h) or (expert, 32 columns of y); a 64-wide step loads the item's
// 16 activation rows (rows past the expert's last read as zeros) and its 32 weight rows,
// 128 bytes each, into an XOR-swizzled slot, and runs 2 x 2 MFMAs. The weights are read once
// and load with the non-temporal policy.
// Whether workgroups of a and b bytes of LDS fit on one CU together (160 KB), with each
// allocation rounded up to the allocation unit (512 bytes here; 1280 and 2048 are checked too,
// so that a coarser unit could not leave the pair unable to share a CU).
static inline bool lds_pair_fits(size_t a, size_t b) {
  for (size_t unit : {size_t(512), size_t(1280), size_t(2048)})
    if (align_up(a, unit) + align_up(b, unit) > size_t(160) * 1024) return false;
  return true;
}
constexpr int kLeanRing = 3;         // (4 slots, with a 3-slot streaming role in the prefill kernel to
                                     // make room, measured no faster)
constexpr int kPrefillColdRing = 4;  // the prefill kernel's streaming-role ring (bf16)
constexpr int kLeanSlotBytes = 6 * 1024;
constexpr int kLeanLdsBytes = kLeanRing * kLeanSlotBytes;
template <bool GATED, int HTM>
__global__ __launch_bounds__(64) __attribute__((amdgpu_num_vgpr(32)))
void ffn_lean_kernel(TiledArgs p, int G, const int32_t* __restrict__ offs) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int lane = threadIdx.x;
  {
    float sb, lf;
    small_large_work<GATED, 2, HTM>(p, lane, sb, lf);
    if (!p.lean || !lean_takes_small(sb, lf, G)) return;  // wave-uniform
  }
  constexpr int NC = GATED ? 16 : 32;  // output columns per item
  const int NT = p.N / NC;             // N is a multiple of 64 on this path
  const int nst = p.K / kDK;           // K is a multiple of 64
  const size_t wstride = (size_t)p.N * p.K * 2;
  // items in expert order (NT per small expert); this wave takes items blockIdx.x + j * gridDim.x
  int total = 0;
  for (int e = lane; e < p.E; e += kWave) {
    int a, b;
    expert_rows(p.offsets, e, p.rows, a, b);
    total += (b - a > 0 && b - a <= kStreamMaxRows) ? NT : 0;
  }
  for (int off = kWave / 2; off >= 1; off >>= 1) total += __shfl_xor(total, off);
  total = __builtin_amdgcn_readfirstlane(total);
  const int first = blockIdx.x, stride = gridDim.x;
  const int mine = first < total ? (total - first + stride - 1) / stride : 0;
  const int nsteps = mine * nst;  // < 2^31: at most E * N / 16 items of K / 64 steps
  if (nsteps == 0) return;

  // A walker over the small experts, moved forward item by item (items only increase): the
  // expert holding item `it`, its rows and its first item
  struct Walker { int e, base, r0, n; };
  auto advance = [&](Walker& w, int it) __attribute__((always_inline)) {
    while (w.e < p.E) {  // (the items counted above end before the last expert)
      // a wave-uniform index, so these are scalar loads: a vector load here would make the
      // compiler wait for every direct-to-LDS load in flight
      const int e = __builtin_amdgcn_readfirstlane(w.e);
      const int a = min(max(offs[e], 0), p.rows);
      const int b = min(max(offs[e + 1], a), p.rows);
      const int cnt = (b - a > 0 && b - a <= kStreamMaxRows) ? NT : 0;
      if (it < w.base + cnt) { w.r0 = a; w.n = b - a; return; }
      w.base += cnt;
      ++w.e;
    }
    w.r0 = 0;
    w.n = 0;
  };
  // lane offsets of the two load shapes (even and odd 8-row groups differ in their swizzle)
  const int lr = lane >> 3;                              // row within an 8-row load
  const int c0s = (lane & 7) ^ ((lr >> 1) & 7);          // source chunk, rows 0..7 of a group
  const int c1s = (lane & 7) ^ (((8 + lr) >> 1) & 7);    // rows 8..15
  const int off0 = lr * p.K * 2 + c0s * 16, off1 = lr * p.K * 2 + c1s * 16;
  const int row8 = 8 * p.K * 2;                          // bytes of 8 operand rows
  // weight loads: the same, or in blocked weights row lr of the 8-row block at lr * 128, 1 KB
  // per step
  const int boff0 = p.wblk ? lr * 128 + c0s * 16 : off0, boff1 = p.wblk ? lr * 128 + c1s * 16 : off1;
  const int bstep = p.wblk ? 1024 : kDK * 2;

  // issue side: the next step to load, as (item index j of this wave, step); compute side alike
  Walker wi{0, 0, 0, 0}, wc{0, 0, 0, 0};
  int ij = 0, ist = 0;
  auto issue = [&](int g) __attribute__((always_inline)) {
    const int it = first + ij * stride;
    advance(wi, it);
    const int c0 = (it - wi.base) * NC;
    const uint8_t* Xt = static_cast<const uint8_t*>(p.X) + (size_t)wi.r0 * p.K * 2;
    const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc(
        (void*)Xt, (short)0, (int)((unsigned)wi.n * (unsigned)p.K * 2u), kBufferWord3);
    const size_t wcol = (size_t)c0 * p.K * 2;
    const unsigned bext = (unsigned)min((size_t)0xffffffffu, (size_t)(p.N - c0) * p.K * 2);
    const __amdgpu_buffer_rsrc_t rB1 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const uint8_t*>(p.W1) + (size_t)wi.e * wstride + wcol), (short)0, (int)bext, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rB2 = GATED ? __builtin_amdgcn_make_buffer_rsrc(
        (void*)(static_cast<const uint8_t*>(p.W2) + (size_t)wi.e * wstride + wcol), (short)0, (int)bext, kBufferWord3) : rB1;
    u32x4* slot = reinterpret_cast<u32x4*>(smem + (g % kLeanRing) * kLeanSlotBytes);
    const int ks = ist * kDK * 2, kw = ist * bstep;
    // slot rows: 0..15 activations, 16..31 gate (or weight rows 0..15), 32..47 up (or 16..31)
    buffer_load_lds16(rA, slot + 0 * 64, off0, ks);
    buffer_load_lds16(rA, slot + 1 * 64, off1, row8 + ks);
    buffer_load_lds16<kNonTemporal>(rB1, slot + 2 * 64, boff0, kw);
    buffer_load_lds16<kNonTemporal>(rB1, slot + 3 * 64, boff1, row8 + kw);
    buffer_load_lds16<kNonTemporal>(rB2, slot + 4 * 64, boff0, (GATED ? 0 : 2 * row8) + kw);
    buffer_load_lds16<kNonTemporal>(rB2, slot + 5 * 64, boff1, (GATED ? 0 : 2 * row8) + row8 + kw);
    if (++ist == nst) { ist = 0; ++ij; }
  };
  constexpr int kLoads = 6;  // load instructions per step

  f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  for (int g = 0; g < kLeanRing && g < nsteps; ++g) issue(g);
  int cj = 0, cst = 0;
  for (int g = 0; g < nsteps; ++g) {
    // this step's loads have landed once at most the later steps' are pending
    wait_vmcnt_dyn<(kLeanRing - 1) * kLoads>(min(kLeanRing - 1, nsteps - 1 - g) * kLoads);
    const u32x4* slot = reinterpret_cast<const u32x4*>(smem + (g % kLeanRing) * kLeanSlotBytes);
#pragma unroll
    for (int h = 0; h < kDK / 32; ++h) {
      const int c = h * 4 + (lane >> 4);
      bf16x8 a, b0, b1;
      const u32x4 va = slot[dswz<8>(lane & 15, c)];
      const u32x4 v0 = slot[dswz<8>(16 + (lane & 15), c)];
      const u32x4 v1 = slot[dswz<8>(32 + (lane & 15), c)];
      __builtin_memcpy(&a, &va, 16);
      __builtin_memcpy(&b0, &v0, 16);
      __builtin_memcpy(&b1, &v1, 16);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b1, acc1, 0, 0, 0);
      // one slice's fragments live at a time (the register budget of a wave beside the tiles)
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_lgkmcnt0();  // the slot's reads are in registers before its refill
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (g + kLeanRing < nsteps) issue(g + kLeanRing);
    if (++cst == nst) {  // the item's last step: epilogue
      cst = 0;
      const int it = first + cj * stride;
      ++cj;
      advance(wc, it);
      const int c0 = (it - wc.base) * NC;
#pragma unroll
      for (int jr = 0; jr < 4; ++jr) {
        const int r = (lane >> 4) * 4 + jr;
        if (r >= wc.n) continue;
        const size_t orow = (size_t)(wc.r0 + r) * p.N;
        const int col = c0 + (lane & 15);
        if constexpr (GATED) {
          static_cast<__bf16*>(p.out)[orow + col] = (__bf16)(silu(acc0[jr]) * acc1[jr]);
        } else {
          static_cast<float*>(p.out)[orow + col] = acc0[jr];
          static_cast<float*>(p.out)[orow + col + 16] = acc1[jr];
        }
      }
      acc0 = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1 = acc0;
    }
  }
}

template <int WF, bool GATED, int HWM, int HWN, int HRING, int HDK, int CWN, int CRING, int CDK>
static hipError_t launch_prefill(const TiledArgs& p, const DeviceInfo& dev, hipStream_t stream) {
  const size_t lh = dl_lds_bytes<WF, HWM, HWN, 2, 4, HRING, HDK>(p);
  const size_t lc = dl_lds_bytes<WF, 16, CWN, 1, 8, CRING, CDK>(p);
  const size_t lds = lh > lc ? lh : lc;
  auto kern = &ffn_prefill_kernel<WF, GATED, HWM, HWN, HRING, HDK, CWN, CRING, CDK>;
  hipError_t st = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (st != hipSuccess) return st;
  kern<<<dev.num_cus, 512, lds, stream>>>(p);
  st = hipGetLastError();
  if (st != hipSuccess) return st;
  // the tail split's chunks, added in chunk order (a launch of its own: the kernel boundary
  // orders the partial tiles' stores before these loads); only the item prefix in LDS
  TiledArgs q = p;
  q.min_rows = kStreamMaxRows;
  const size_t lds2 = ((size_t)(p.E + 1 + 3) / 4 * 4 * 2 + 512) * sizeof(int32_t);
  ffn_tiled_dl_kernel<WF, GATED, HWM, HWN, 2, 4, HRING, HDK, false, 2, true><<<dev.num_cus, 512, lds2, stream>>>(q);
  return hipGetLastError();
}

// Whether a lean-kernel wave fits in the registers that two prefill-kernel waves leave on a SIMD
// (512 per lane, allocated in units of 8), from the kernels' code objects; read once.
static bool lean_regs_fit() {
  static const bool fit = [] {
    auto regs = [](const void* f) {
      hipFuncAttributes a{};
      return hipFuncGetAttributes(&a, f) == hipSuccess ? (int)align_up((size_t)a.numRegs, 8) : 1 << 20;
    };
    const int lean = std::max(regs(reinterpret_cast<const void*>(&ffn_lean_kernel<true, 256>)),
                              regs(reinterpret_cast<const void*>(&ffn_lean_kernel<false, 256>)));
    const int pre = std::max(
        regs(reinterpret_cast<const void*>(&ffn_prefill_kernel<kBF16, true, 128, 64, 2, 64, 32, kPrefillColdRing, 64>)),
        regs(reinterpret_cast<const void*>(&ffn_prefill_kernel<kBF16, false, 128, 64, 2, 64, 32, kPrefillColdRing, 64>)));
    return 2 * pre + lean <= 512;
  }();
  return fit;
}

template <int WF, bool GATED, int WM, int WN, int WGM, int WGN, int RING = kRing, int DK = kDK,
          bool ASKIP = false>
static hipError_t launch_tiled_dl(const TiledArgs& p, const DeviceInfo& dev, hipStream_t stream) {
  constexpr int NTH = 64 * WGM * WGN;
  constexpr int WB = WF == kFP8 ? 1 : 2;
  const size_t lds = ((size_t)(p.E + 1 + 3) / 4 * 4 * 2 + ((NTH + 3) & ~3)) * sizeof(int32_t) +
                     (size_t)RING * (WGM * WM * DK * 2 + WGN * WN * DK * WB) +
                     (WF == kFP8 ? (size_t)WGN * 2 * (p.K / 128) * sizeof(float) : 0);
  auto kern = &ffn_tiled_dl_kernel<WF, GATED, WM, WN, WGM, WGN, RING, DK, ASKIP>;
  if (lds > 64 * 1024) {
    hipError_t st = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (st != hipSuccess) return st;
  }
  const int fit = (int)((160 * 1024) / lds);  // workgroups per CU that the LDS allows
  const int per_cu = fit < 1 ? 1 : (fit > 4 ? 4 : fit);
  kern<<<dev.num_cus * per_cu, NTH, lds, stream>>>(p);
  return hipGetLastError();
}

// Decode-sized bf16 launches whose tile count is small whatever the routing (at most
// kSplitMaxUnits / 2 tiles of 64 rows x cols_per_tile columns, bounded with every expert that
// can hold a row active) split the contraction across workgroups; the host decides from the
// sizes alone, and the workspace holds the partial tiles after h.
static bool split_gemm(int rows, int E, int N, int cols_per_tile) {
  const long long nt = (N + cols_per_tile - 1) / cols_per_tile;
  const long long tiles = nt * ((rows + 63) / 64 + (long long)(E < rows ? E : rows));
  return tiles <= kSplitMaxUnits / 2;
}
// Prefill-sized launches (the host knows the sizes, not the routing): bf16 weights from 32 rows
// per configured expert; fp8 weights from more than 8. With fp8 weights the prefill kernel beat
// the decode-sized tiles by 11-32% on every routing measured between 8 and 32 rows per expert
// (Zipf 0 and 1.2, both model shapes) and tied at 8; with bf16 weights the better of the two
// there depends on the routing's skew (near-uniform routings, every expert with ~30 rows, run
// 5-38% faster on the decode-sized tiles, skewed ones 8-17% faster on the prefill kernel), so
// the bf16 switch stays where the prefill kernel wins whatever the routing.
static bool prefill_sized(int rows, int E, moe_dtype_t wdt) {
  return wdt == MOE_FP8_E4M3FN ? (long long)rows > 8LL * E : (long long)rows >= 32LL * E;
}
static bool decode_tiled_bf16(int rows, int E, int d, int d_ff, moe_dtype_t act, moe_dtype_t wdt) {
  return act == MOE_BF16 && wdt == MOE_BF16 && d % kTK == 0 && d_ff % kTK == 0 &&
         !prefill_sized(rows, E, wdt);
}
static bool uses_split(int rows, int E, int d, int d_ff, moe_dtype_t act, moe_dtype_t wdt) {
  return decode_tiled_bf16(rows, E, d, d_ff, act, wdt) &&
         (split_gemm(rows, E, d_ff, 64) || split_gemm(rows, E, d, 128));
}
constexpr size_t kPartialBytes = (size_t)kSplitMaxUnits * kSplitTileElems * sizeof(float);

// Prefill-sized launches run ffn_prefill_kernel, whose last round's tiles may be split: a
// 256-byte header and kTailMaxUnits partial tiles of the hot tile size follow h.
static bool prefill_tiled(int rows, int E, int d, int d_ff, moe_dtype_t act, moe_dtype_t wdt) {
  return act == MOE_BF16 && d % kTK == 0 && d_ff % kTK == 0 && prefill_sized(rows, E, wdt) &&
         (wdt == MOE_BF16 || (wdt == MOE_FP8_E4M3FN && d <= kFp8DlMaxK && d_ff <= kFp8DlMaxK));
}
constexpr size_t kHotTileElemsBF16 = 256 * 256, kHotTileElemsFP8 = 128 * 256;
static size_t tail_partial_bytes(moe_dtype_t wdt) {
  return 256 + (size_t)kTailMaxUnits * (wdt == MOE_BF16 ? kHotTileElemsBF16 : kHotTileElemsFP8) * sizeof(float);
}

size_t ffn_workspace_bytes(int rows, int E, int d, int d_ff, moe_dtype_t act, moe_dtype_t wdt) {
  // the blocked layouts: the same kernels and workspace as their row-major formats
  if (wdt == MOE_BF16_BLOCKED) wdt = MOE_BF16;
  if (wdt == MOE_FP8_E4M3FN_BLOCKED) wdt = MOE_FP8_E4M3FN;
  const size_t hb = act == MOE_F32 ? 4 : 2;
  const size_t h = align_up((size_t)rows * d_ff * hb, 256);
  if (uses_split(rows, E, d, d_ff, act, wdt)) return h + kPartialBytes;
  if (prefill_tiled(rows, E, d, d_ff, act, wdt)) return h + tail_partial_bytes(wdt);
  return h;
}

// The split pair of one GEMM: chunk partials, then the in-order sum and epilogue.
template <bool GATED>
static hipError_t launch_split(TiledArgs p, const DeviceInfo& dev, hipStream_t stream) {
  constexpr int WM = 32, WN = 64, WGM = 2, WGN = 2, RING = 3, DK = 64, NTH = 64 * WGM * WGN;
  const size_t lds = dl_lds_bytes<kBF16, WM, WN, WGM, WGN, RING, DK>(p);
  const int fit = (int)((160 * 1024) / lds);
  const int grid = dev.num_cus * (fit < 1 ? 1 : (fit > 4 ? 4 : fit));
  p.split_ranks = grid;
  auto k1 = &ffn_tiled_dl_kernel<kBF16, GATED, WM, WN, WGM, WGN, RING, DK, false, 1>;
  if (lds > 64 * 1024) {
    hipError_t st = hipFuncSetAttribute(reinterpret_cast<const void*>(k1),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (st != hipSuccess) return st;
  }
  k1<<<grid, NTH, lds, stream>>>(p);
  hipError_t st = hipGetLastError();
  if (st != hipSuccess) return st;
  // the sum needs only the item prefix in LDS
  const size_t lds2 = ((size_t)(p.E + 1 + 3) / 4 * 4 * 2 + ((NTH + 3) & ~3)) * sizeof(int32_t);
  ffn_tiled_dl_kernel<kBF16, GATED, WM, WN, WGM, WGN, RING, DK, false, 2><<<grid, NTH, lds2, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_grouped_ffn(const FfnArgs& a_in, const DeviceInfo& dev, hipStream_t stream) {
  if (a_in.rows == 0) return hipSuccess;
  // blocked weights run their format's kernels with the blocked addressing. Validated: bf16 d
  // and d_ff multiples of 64, so every bf16 tiled path below reads them, none of the streaming
  // kernel's; fp8 d and d_ff at most 65536, so the direct-to-LDS tiles take every fp8 expert
  // (also in the smallest launches, which otherwise stream their <= 16-row experts)
  FfnArgs a = a_in;
  const int wblk = (a.wdt == MOE_BF16_BLOCKED || a.wdt == MOE_FP8_E4M3FN_BLOCKED) ? 1 : 0;
  if (a.wdt == MOE_BF16_BLOCKED) a.wdt = MOE_BF16;
  if (a.wdt == MOE_FP8_E4M3FN_BLOCKED) a.wdt = MOE_FP8_E4M3FN;
  // Which kernel takes which expert (decided per expert on the device from its row count):
  //  - fp32, or widths that are not multiples of 64: the streaming kernel takes every expert;
  //  - decode-sized batches (T*k < 32*E with bf16 weights, T*k <= 8*E with fp8 weights): the
  //    direct-to-LDS tiles take every expert;
  //  - prefill-sized batches: one launch per GEMM whose workgroups split into a streaming role
  //    (experts with <= 16 rows, 16 x 256 tiles) and a large-tile role (the rest).
  const bool tiled = a.act == MOE_BF16 && a.d % kTK == 0 && a.d_ff % kTK == 0;
  const bool big = prefill_sized(a.rows, a.E, a.wdt);
  int small = tiled ? kStreamMaxRows : 0x7fffffff;
  // fp8 at decode sizes: every expert on the direct-to-LDS tiles, except in launches so small
  // that bf16 would split the contraction (at most a few rows in all), where streaming the
  // small experts, whose kernel splits each item's contraction over its waves, is faster
  const bool fp8_dl_small = a.wdt == MOE_FP8_E4M3FN && tiled && !big && a.d <= kFp8DlMaxK &&
                            a.d_ff <= kFp8DlMaxK && (wblk || !split_gemm(a.rows, a.E, a.d_ff, 64));
  if (tiled && !big && (a.wdt == MOE_BF16 || fp8_dl_small)) small = 0;
  StreamArgs gu{a.x_sorted, a.w_gate, a.w_up, a.s_gate, a.s_up, a.h, a.offsets,
                a.E, a.d, a.d_ff, a.rows, small};
  StreamArgs dn{a.h, a.w_down, nullptr, a.s_down, nullptr, a.y_sorted, a.offsets,
                a.E, a.d_ff, a.d, a.rows, small};
  TiledArgs tgu{a.x_sorted, a.w_gate, a.w_up, a.s_gate, a.s_up, a.h, a.offsets,
                a.E, a.d, a.d_ff, a.rows, small};
  TiledArgs tdn{a.h, a.w_down, nullptr, a.s_down, nullptr, a.y_sorted, a.offsets,
                a.E, a.d_ff, a.d, a.rows, small};
  tgu.wblk = tdn.wblk = wblk;
  // the fp8 direct-to-LDS kernel keeps an item's scale rows in LDS: 4 x 2 x K/128 floats
  const bool fp8_dl = big && a.d <= kFp8DlMaxK && a.d_ff <= kFp8DlMaxK;
  hipError_t st = hipSuccess;
  if (a.act == MOE_F32) {
    st = launch_stream<kF32, kF32, 2, 1, 1, 4>(gu, dev, stream);
    if (st == hipSuccess) st = launch_stream<kF32, kF32, 1, 2, 1, 4>(dn, dev, stream);
    return st;
  }
  // prefill-sized batches: small and large experts in one launch per GEMM (ffn_prefill_kernel)
  if (tiled && big && (a.wdt == MOE_BF16 || fp8_dl)) {
    TiledArgs pgu = tgu, pdn = tdn;
    pgu.min_rows = pdn.min_rows = 0;
    // tail-split header and partial tiles after h (shared by the two GEMMs, which run in order)
    char* tail = static_cast<char*>(a.h) + align_up((size_t)a.rows * a.d_ff * 2, 256);
    pgu.split_info = pdn.split_info = reinterpret_cast<int32_t*>(tail);
    pgu.partial = pdn.partial = reinterpret_cast<float*>(tail + 256);
    if (a.wdt == MOE_BF16) {
      // The experts with <= kStreamMaxRows rows may go to ffn_lean_kernel on a second stream
      // beside the large tiles (both kernels decide from the counts), if its workgroups fit in
      // the LDS a prefill workgroup leaves.
      const size_t lds_pre = std::max(dl_lds_bytes<kBF16, 128, 64, 2, 4, 2, 64>(pgu),
                                      dl_lds_bytes<kBF16, 16, 32, 1, 8, kPrefillColdRing, 64>(pgu));
      SideStream side;
      const bool lean = lds_pair_fits(lds_pre, kLeanLdsBytes) && lean_regs_fit() &&
                        side_stream_for(stream, &side);
      pgu.lean = pdn.lean = lean ? 1 : 0;
      if (lean) {
        // the side stream waits for what the caller's stream holds before this call
        st = hipEventRecord(side.fork, stream);
        if (st == hipSuccess) st = hipStreamWaitEvent(side.stream, side.fork, 0);
        if (st != hipSuccess) return st;
      }
      st = launch_prefill<kBF16, true, 128, 64, 2, 64, 32, kPrefillColdRing, 64>(pgu, dev, stream);
      if (st == hipSuccess && lean) {
        ffn_lean_kernel<true, 256><<<dev.num_cus, kWave, kLeanLdsBytes, side.stream>>>(pgu, dev.num_cus, pgu.offsets);
        st = hipGetLastError();
      }
      if (st == hipSuccess) st = launch_prefill<kBF16, false, 128, 64, 2, 64, 32, kPrefillColdRing, 64>(pdn, dev, stream);
      if (st == hipSuccess && lean) {
        // after the lean gate/up on its stream: it reads the h rows that launch wrote
        ffn_lean_kernel<false, 256><<<dev.num_cus, kWave, kLeanLdsBytes, side.stream>>>(pdn, dev.num_cus, pdn.offsets);
        st = hipGetLastError();
      }
      if (lean) {
        // the caller's stream waits for the side stream's work (even after a failed launch)
        const hipError_t j1 = hipEventRecord(side.join, side.stream);
        const hipError_t j2 = j1 == hipSuccess ? hipStreamWaitEvent(stream, side.join, 0) : j1;
        if (st == hipSuccess) st = j2;
      }
    } else {
      st = launch_prefill<kFP8, true, 64, 64, 2, 128, 32, 3, 128>(pgu, dev, stream);
      if (st == hipSuccess) st = launch_prefill<kFP8, false, 64, 64, 2, 128, 32, 3, 128>(pdn, dev, stream);
    }
    return st;
  }
  if (a.wdt == MOE_BF16) {
    if (!tiled) {
      st = launch_stream<kBF16, kBF16, 2, 2, 2, 4>(gu, dev, stream);
      if (st == hipSuccess) st = launch_stream<kBF16, kBF16, 1, 4, 2, 4>(dn, dev, stream);
      return st;
    }
    // launches with few tiles whatever the routing split the contraction (partials in the
    // workspace after h)
    float* partial = reinterpret_cast<float*>(static_cast<char*>(a.h) +
                                              align_up((size_t)a.rows * a.d_ff * 2, 256));
    tgu.partial = tdn.partial = partial;
    st = split_gemm(a.rows, a.E, a.d_ff, 64) ? launch_split<true>(tgu, dev, stream)
                                             : launch_tiled_dl<kBF16, true, 32, 64, 2, 2, 3, 64>(tgu, dev, stream);
    if (st == hipSuccess)
      st = split_gemm(a.rows, a.E, a.d, 128) ? launch_split<false>(tdn, dev, stream)
                                             : launch_tiled_dl<kBF16, false, 32, 64, 2, 2, 3, 64>(tdn, dev, stream);
    return st;
  }
  // fp8 weights outside the prefill kernel: decode-sized launches (at most 8 rows per expert)
  // run their tiled experts on the direct-to-LDS tiles, 32 rows tall with 128-wide steps in a
  // 3-slot ring (24 KB slots, two workgroups per CU: 16 KB of weights per step, as the bf16
  // tiles load), every expert as for bf16 unless the launch is tiny; contractions longer than
  // the direct-to-LDS kernel stages scales for stream the experts with <= 16 rows and run the
  // rest on the register-staged tiles (128 rows tall from 32 rows per expert, else 64)
  const bool fp8_dl_dec = !big && a.d <= kFp8DlMaxK && a.d_ff <= kFp8DlMaxK;
  const bool tall = (long long)a.rows >= 32LL * a.E;
  if (!fp8_dl_small) st = launch_stream<kBF16, kFP8, 2, 2, 2, 4>(gu, dev, stream);
  if (st == hipSuccess && tiled)
    st = fp8_dl_dec ? launch_tiled_dl<kFP8, true, 16, 64, 2, 2, 3, 128>(tgu, dev, stream)
         : tall       ? launch_tiled<kFP8, true, 128, 64, 2, 2>(tgu, dev, stream)
                      : launch_tiled<kFP8, true, 64, 64, 2, 2>(tgu, dev, stream);
  if (st == hipSuccess && !fp8_dl_small) st = launch_stream<kBF16, kFP8, 1, 4, 2, 4>(dn, dev, stream);
  if (st == hipSuccess && tiled)
    st = fp8_dl_dec ? launch_tiled_dl<kFP8, false, 16, 64, 2, 2, 3, 128>(tdn, dev, stream)
         : tall       ? launch_tiled<kFP8, false, 128, 64, 2, 2>(tdn, dev, stream)
                      : launch_tiled<kFP8, false, 64, 64, 2, 2>(tdn, dev, stream);
  return st;
}

}  // namespace moe
