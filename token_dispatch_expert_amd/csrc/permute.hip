// Expert sort of the T*k assignments: histogram, exclusive scan, stable scatter, row copy.
//
// Operation: "Expert Parallelism" tutorial page, section 4, dispatch (sort by destination
// expert, count, every expert ends up with a contiguous block of rows) and section 9 (an
// unsorted batch means divergent, uncoalesced work). Reading taken: the sort is stable in
// the flat index i = t*k + j, so within an expert rows appear in token order and the
// permutation is unique (the k experts of one token are distinct).
//
// Capacity factor ("Expert Parallelism" tutorial page, section 5, mitigation 1): with a
// capacity c, an expert keeps its first c assignments in flat order; the counts and offsets
// are those of the kept rows, a dropped assignment gets flat_to_sorted = -1 and no row.
// Every position is still ranked among all of the expert's assignments, and a position at or
// past the expert's capped end is dropped, so capping costs nothing extra.
//
// Batches of more than kSmallR assignments take four launches, none using float atomics, all
// deterministic (smaller batches use one workgroup for the first three, see
// permute_small_kernel):
//   hist : one workgroup per tile of kPermuteTile flat entries; LDS histogram -> ws[tile][e]
//   scan : one workgroup per kScanExperts experts; per expert an exclusive prefix over the
//          tiles (groups of threads take ranges of tiles) -> ws[tile][e], relative to the
//          expert's first row, and the kept count -> counts[e]
//   rank : one wavefront per tile; it first scans the kept counts over the experts (offsets;
//          the first tile's wavefront also stores them), then walks its entries in flat order,
//          64 at a time; lanes with the same expert find each other with ballots over the
//          expert id's bits, so a lane's rank among equal keys is a popcount of lower lanes;
//          the group's last lane advances the running base in LDS. Writes both index maps.
//   copy : one workgroup per token reads x[t] once in 16-byte vectors and stores it to its
//          k sorted rows.
#include <mutex>

#include "moe_internal.h"

namespace moe {

size_t permute_workspace_ints(int T, int E, int k) {
  const size_t R = (size_t)T * (size_t)k;
  const size_t tiles = (R + kPermuteTile - 1) / kPermuteTile;
  return tiles * (size_t)E;
}

__device__ __forceinline__ int clamp_expert(int e, int E) { return e < 0 ? 0 : (e >= E ? E - 1 : e); }

// word 3 of a raw buffer descriptor on gfx950 (32-bit elements, no swizzle, bounds-checked);
// entry j of the tile through `rsrc`, 0 past its extent
constexpr int kRawBufferWord3 = 0x00020000;
__device__ __forceinline__ int load_tile_id(__amdgpu_buffer_rsrc_t rsrc, int j) {
  return __builtin_amdgcn_raw_buffer_load_b32(rsrc, j * 4, 0, 0);
}

__global__ __launch_bounds__(256) void permute_hist_kernel(const int32_t* __restrict__ ids, int R,
                                                           int E, int32_t* __restrict__ ws) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int base = blockIdx.x * kPermuteTile;
  const int end = min(base + kPermuteTile, R);
  for (int i = base + threadIdx.x; i < end; i += blockDim.x)
    atomicAdd(&hist[clamp_expert(ids[i], E)], 1);
  __syncthreads();
  int32_t* out = ws + (size_t)blockIdx.x * E;
  for (int e = threadIdx.x; e < E; e += blockDim.x) out[e] = hist[e];
}

constexpr int kScanThreads = 1024;  // >= MOE_MAX_EXPERTS
constexpr int kScanRegTiles = 64;   // tile counts one scan thread keeps in registers

// Inclusive prefix sum of v over the 1024 threads of the workgroup: shuffles within each wave,
// then the 16 wave totals by one wave.
__device__ __forceinline__ int block_inclusive_scan_1024(int v, int32_t* wave_sum) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  constexpr int kWaves = kScanThreads / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int t = __shfl_up(v, off);
    if (lane >= off) v += t;
  }
  if (lane == kWave - 1) wave_sum[wave] = v;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kWaves ? wave_sum[lane] : 0;
#pragma unroll
    for (int off = 1; off < kWaves; off <<= 1) {
      const int t = __shfl_up(w, off);
      if (lane >= off) w += t;
    }
    if (lane < kWaves) wave_sum[lane] = w;
  }
  __syncthreads();
  return v + (wave > 0 ? wave_sum[wave - 1] : 0);
}

// Workgroup b takes experts b*kScanExperts .. +kScanExperts-1; its threads are kScanGroups
// groups of kScanExperts, and group g takes a contiguous range of tiles, so thread (g, e) scans
// at most kScanRegTiles tile counts of expert e in registers (all loaded at once). Group totals
// give each group's base; the expert's total, capped, is its kept count. The scan over the
// experts (offsets) is left to the rank kernel, so no single workgroup reads every tile.
constexpr int kScanExperts = 16;
constexpr int kScanGroups = 16;
constexpr int kScanWgThreads = kScanExperts * kScanGroups;
__global__ __launch_bounds__(kScanWgThreads) void permute_scan_kernel(int32_t* __restrict__ ws,
                                                                      int n_tiles, int E, int cap,
                                                                      int32_t* __restrict__ counts,
                                                                      int32_t* __restrict__ offsets) {
  __shared__ int32_t gsum[kScanWgThreads];  // [group][expert] group totals
  const int tid = threadIdx.x;
  const int g = tid / kScanExperts, el = tid - g * kScanExperts;
  const int e = blockIdx.x * kScanExperts + el;
  const bool active = e < E;
  const int tpg = (n_tiles + kScanGroups - 1) / kScanGroups;
  const int t0 = min(g * tpg, n_tiles), t1 = min(t0 + tpg, n_tiles);
  const bool in_regs = tpg <= kScanRegTiles;
  int pre[kScanRegTiles];
  int run = 0;  // exclusive prefix within the group, then the group total
  if (active) {
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < kScanRegTiles; ++u) pre[u] = t0 + u < t1 ? ws[(size_t)(t0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < kScanRegTiles; ++u) {
        const int h = pre[u];
        pre[u] = run;
        run += h;
      }
    } else {
      constexpr int B = 16;  // batches of independent loads
      for (int tb = t0; tb < t1; tb += B) {
        int h[B];
#pragma unroll
        for (int u = 0; u < B; ++u) h[u] = (tb + u < t1) ? ws[(size_t)(tb + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < B; ++u) {
          if (tb + u < t1) {
            ws[(size_t)(tb + u) * E + e] = run;
            run += h[u];
          }
        }
      }
    }
  }
  gsum[tid] = run;
  __syncthreads();
  int gbase = 0, total = 0;
#pragma unroll
  for (int gg = 0; gg < kScanGroups; ++gg) {
    const int v = gsum[gg * kScanExperts + el];
    gbase += gg < g ? v : 0;
    total += v;
  }
  if (active && g == 0) {
    counts[e] = min(total, cap);  // kept assignments (capacity factor)
    if (n_tiles == 0) {           // no rank launch follows: the offsets of an empty batch
      offsets[e] = 0;
      if (e == 0) offsets[E] = 0;
    }
  }
  if (active) {
    if (in_regs) {
#pragma unroll
      for (int u = 0; u < kScanRegTiles; ++u)
        if (t0 + u < t1) ws[(size_t)(t0 + u) * E + e] = pre[u] + gbase;
    } else {
      for (int t = t0; t < t1; ++t) ws[(size_t)t * E + e] += gbase;
    }
  }
}

__global__ __launch_bounds__(kWave) void permute_rank_kernel(const int32_t* __restrict__ ids,
                                                             int R, int E, int nbits,
                                                             const int32_t* __restrict__ ws,
                                                             const int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ s2f,
                                                             int32_t* __restrict__ f2s) {
  extern __shared__ int32_t run[];  // [E] running positions, then [E] end of each expert
  int32_t* lim = run + E;
  const int lane = threadIdx.x;
  const int32_t* bases = ws + (size_t)blockIdx.x * E;
  for (int e = lane; e < E; e += kWave) {
    run[e] = bases[e];  // relative to the expert's first row
    lim[e] = counts[e];
  }
  // One wavefront per workgroup: its LDS accesses take effect in program order, so no barrier
  // is needed between LDS writes and later reads, nor between a chunk's reads of the running
  // positions and their update (a workgroup barrier would also wait for this wave's global
  // stores of the index maps, once per chunk). The wave barriers only keep the compiler from
  // moving LDS accesses across them.
  __builtin_amdgcn_wave_barrier();
  // offsets: exclusive scan of the kept counts, lane l taking experts l*epl .. +epl-1
  {
    const int epl = (E + kWave - 1) / kWave;
    const int e0 = min(lane * epl, E), e1 = min(e0 + epl, E);
    int sum = 0;
    for (int e = e0; e < e1; ++e) sum += lim[e];
    int incl = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int t = __shfl_up(incl, off);
      if (lane >= off) incl += t;
    }
    int o = incl - sum;
    for (int e = e0; e < e1; ++e) {
      const int c = lim[e];
      if (blockIdx.x == 0) offsets[e] = o;
      run[e] += o;
      lim[e] = o + c;  // positions at or past it are beyond the capacity
      o += c;
    }
    if (blockIdx.x == 0 && lane == kWave - 1) offsets[E] = incl;
  }
  __builtin_amdgcn_wave_barrier();
  const int base = blockIdx.x * kPermuteTile;
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  // the tile's expert ids, all loaded before the walk (one memory latency, not one per chunk):
  // buffer loads through a descriptor that ends at the batch's last entry read zeros past it,
  // so the loads carry no condition that the compiler could turn into a branch around each
  const __amdgpu_buffer_rsrc_t tile_ids = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(ids + base), (short)0, (int)(min(R - base, kPermuteTile) * 4), kRawBufferWord3);
  constexpr int kChunks = kPermuteTile / kWave;
  int key[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) key[c] = clamp_expert(load_tile_id(tile_ids, c * kWave + lane), E);
#pragma unroll
  for (int cc = 0; cc < kChunks; ++cc) {
    const int c = cc * kWave;
    const int i = base + c + lane;
    const bool valid = i < R;
    const int e = key[cc];
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t ones = __ballot(bit);
      same &= bit ? ones : ~ones;
    }
    if (valid) {
      // positions at or past the expert's end are beyond its capacity: dropped
      const int pos = run[e] + __popcll(same & lower);
      if (pos < lim[e]) s2f[pos] = i;
      f2s[i] = pos < lim[e] ? pos : -1;
    }
    __builtin_amdgcn_wave_barrier();
    // the highest lane of each group of equal experts advances that expert's base
    if (valid && (63 - __clzll(same)) == lane) run[e] += __popcll(same);
    __builtin_amdgcn_wave_barrier();
  }
}

__global__ __launch_bounds__(256) void permute_copy_kernel(const uint4* __restrict__ x, int k,
                                                           int vec_per_row,
                                                           const int32_t* __restrict__ f2s,
                                                           uint4* __restrict__ xs) {
  const int t = blockIdx.x;
  const int32_t* pos = f2s + (size_t)t * k;
  const uint4* src = x + (size_t)t * vec_per_row;
  constexpr int U = 4;  // a thread's loads in flight before its stores
  for (int v0 = threadIdx.x; v0 < vec_per_row; v0 += U * blockDim.x) {
    uint4 val[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + u * blockDim.x;
      val[u] = v < vec_per_row ? src[v] : make_uint4(0, 0, 0, 0);
    }
    for (int j = 0; j < k; ++j) {
      const int p = pos[j];
      if (p < 0) continue;  // dropped slot
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int v = v0 + u * blockDim.x;
        if (v < vec_per_row) xs[(size_t)p * vec_per_row + v] = val[u];
      }
    }
  }
}

// Small batches (R <= kSmallR): one workgroup of 16 waves does histogram, scan and stable
// rank. The R entries are split into 16 contiguous slices, one per wave (slice order = flat
// order). Each wave ranks its slice 64 entries at a time with the ballot match (ids staged in
// LDS first) and keeps a per-expert running count in its own LDS row; a prefix over the 16
// rows plus the exclusive scan over experts then gives every slice's base per expert.
constexpr int kSmallWaves = 16;
constexpr int kSmallChunks = 8;  // 64-entry chunks per wave -> R <= 16 * 8 * 64
constexpr int kSmallR = kSmallWaves * kSmallChunks * kWave;
static_assert(kSmallWaves * kWave == kScanThreads, "the small kernel's scan is the 1024-thread one");

__global__ __launch_bounds__(kSmallWaves * kWave) void permute_small_kernel(
    const int32_t* __restrict__ ids, int R, int E, int nbits, int cap, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ s2f, int32_t* __restrict__ f2s) {
  extern __shared__ int32_t sm[];
  int32_t* wc = sm;                                  // [16][E] per-wave counts, then bases
  int32_t* sc = wc + kSmallWaves * E;                // [1024] scan
  int32_t* key = sc + kSmallWaves * kWave;           // [R] staged (clamped) expert ids
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  for (int i = tid; i < kSmallWaves * E; i += blockDim.x) wc[i] = 0;
  for (int i = tid; i < R; i += blockDim.x) key[i] = clamp_expert(ids[i], E);
  __syncthreads();

  const int slice = ((R + kSmallWaves - 1) / kSmallWaves + kWave - 1) / kWave * kWave;
  const int lo = min(wave * slice, R), hi = min(lo + slice, R);
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  int32_t* mine = wc + wave * E;
  int rank[kSmallChunks], exp_[kSmallChunks];
#pragma unroll
  for (int c = 0; c < kSmallChunks; ++c) {
    const int i = lo + c * kWave + lane;
    const bool valid = i < hi;
    const int e = valid ? key[i] : 0;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t ones = __ballot(bit);
      same &= bit ? ones : ~ones;
    }
    exp_[c] = e;
    rank[c] = valid ? mine[e] + __popcll(same & lower) : 0;
    // LDS ops of one wave complete in order: every lane's read above precedes this update
    if (valid && (63 - __clzll(same)) == lane) mine[e] += __popcll(same);
  }
  __syncthreads();

  int total = 0;
  if (tid < E) {
    for (int w = 0; w < kSmallWaves; ++w) {
      const int t = wc[w * E + tid];
      wc[w * E + tid] = total;
      total += t;
    }
    total = min(total, cap);  // kept assignments (capacity factor)
    counts[tid] = total;
  }
  // inclusive scan of the capped counts over the 1024 threads (three barriers)
  __shared__ int32_t wave_sum[kSmallWaves];
  sc[tid] = block_inclusive_scan_1024(total, wave_sum);
  __syncthreads();
  if (tid < E) {
    const int base = sc[tid] - total;
    offsets[tid] = base;
    for (int w = 0; w < kSmallWaves; ++w) wc[w * E + tid] += base;
  }
  if (tid == 0) offsets[E] = sc[kSmallWaves * kWave - 1];
  __syncthreads();
  // sc[e] (inclusive scan) is the end of expert e's rows: positions at or past it are beyond
  // the capacity and dropped
#pragma unroll
  for (int c = 0; c < kSmallChunks; ++c) {
    const int i = lo + c * kWave + lane;
    if (i < hi) {
      const int pos = mine[exp_[c]] + rank[c];
      const bool keep = pos < sc[exp_[c]];
      if (keep) s2f[pos] = i;
      f2s[i] = keep ? pos : -1;
    }
  }
}

// Scratch of the no-allocation entry point: the per-tile histograms and bases (the same
// n_tiles * E int32 as the caller's workspace of moe_permute) in a file-scope device array,
// kStaticPermuteInts entries. Every GPU the library runs on holds its own copy until the
// process ends. The histogram launch writes every entry the later launches read, so nothing
// needs clearing between calls; calls that overlap on one GPU share the array and race.
static __device__ __align__(256) int32_t scratch[kStaticPermuteInts];

hipError_t permute_static_scratch(int32_t** out) {
  static std::mutex mu;
  static int32_t* ptrs[64] = {};
  int dev = 0;
  hipError_t st = hipGetDevice(&dev);
  if (st != hipSuccess) return st;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    // the device address of this GPU's copy (the array's name in host code is only a handle)
    void* p = nullptr;
    st = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (st != hipSuccess) return st;
    if (p == nullptr) return hipErrorInvalidSymbol;
    ptrs[dev] = static_cast<int32_t*>(p);
  }
  *out = ptrs[dev];
  return hipSuccess;
}

hipError_t launch_permute(const void* x, int elem_bytes, const int32_t* ids, int T, int E, int k,
                          int d, int cap, int32_t* counts, int32_t* offsets,
                          int32_t* sorted_to_flat, int32_t* flat_to_sorted, void* x_sorted,
                          int32_t* ws, hipStream_t stream) {
  const int R = T * k;
  const int n_tiles = (R + kPermuteTile - 1) / kPermuteTile;
  const size_t lds = (size_t)E * sizeof(int32_t);
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const int vpr = d * elem_bytes / 16;
  const int threads = vpr >= 256 ? 256 : ((vpr + kWave - 1) / kWave) * kWave;
  if (R > 0 && R <= kSmallR) {
    const size_t slds = ((size_t)kSmallWaves * E + kSmallWaves * kWave + R) * sizeof(int32_t);
    if (slds > 64 * 1024) {
      hipError_t st = hipFuncSetAttribute(reinterpret_cast<const void*>(&permute_small_kernel),
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)slds);
      if (st != hipSuccess) return st;
    }
    permute_small_kernel<<<1, kSmallWaves * kWave, slds, stream>>>(ids, R, E, nbits, cap, counts,
                                                                   offsets, sorted_to_flat,
                                                                   flat_to_sorted);
    hipError_t st = hipGetLastError();
    if (st != hipSuccess) return st;
    permute_copy_kernel<<<T, threads, 0, stream>>>(static_cast<const uint4*>(x), k, vpr,
                                                   flat_to_sorted, static_cast<uint4*>(x_sorted));
    return hipGetLastError();
  }
  if (n_tiles > 0) {
    permute_hist_kernel<<<n_tiles, 256, lds, stream>>>(ids, R, E, ws);
    hipError_t st = hipGetLastError();
    if (st != hipSuccess) return st;
  }
  permute_scan_kernel<<<(E + kScanExperts - 1) / kScanExperts, kScanWgThreads, 0, stream>>>(
      ws, n_tiles, E, cap, counts, offsets);
  hipError_t st = hipGetLastError();
  if (st != hipSuccess || n_tiles == 0) return st;
  permute_rank_kernel<<<n_tiles, kWave, 2 * lds, stream>>>(ids, R, E, nbits, ws, counts, offsets,
                                                            sorted_to_flat, flat_to_sorted);
  st = hipGetLastError();
  if (st != hipSuccess) return st;
  permute_copy_kernel<<<T, threads, 0, stream>>>(static_cast<const uint4*>(x), k, vpr,
                                                 flat_to_sorted, static_cast<uint4*>(x_sorted));
  return hipGetLastError();
}

}  // namespace moe
