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
// Batches of more than kSmallR assignments take two or three launches, none using float
// atomics, all deterministic (smaller batches use one workgroup for the index work, see
// permute_small_kernel):
//   hist : one workgroup per tile of kPermuteTile flat entries; LDS histogram -> ws[tile][e]
//   rank : one 1024-thread workgroup per tile. It sums, per expert, the histograms of the tiles
//          before its own (its base inside the expert) and of all tiles (the expert's count,
//          capped), threads splitting the tiles into slices and adding the slices in LDS; a
//          block scan of the kept counts gives the expert offsets (the first tile's workgroup
//          stores counts and offsets). Its first wavefront then walks the tile's entries in
//          flat order, 64 at a time; lanes with the same expert find each other with ballots
//          over the expert id's bits, so a lane's rank among equal keys is a popcount of lower
//          lanes; the group's last lane advances the running position in LDS. Writes both
//          index maps.
//   copy : one workgroup per token reads x[t] once in 16-byte vectors and stores it to its
//          k sorted rows.
// Mid-size batches (at most kCountMaxR assignments, at most kCountMaxE experts) replace hist
// and rank by one launch whose workgroups count the ids themselves (permute_count_rank_kernel).
// (A separate scan launch between hist and rank, with the expert offsets scanned again by
// every rank wavefront, took one more dependent launch: ~6 us of the 8192-token index phase.)
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

constexpr int kRankThreads = 1024;  // = kScanThreads: the block scan below is the 1024-thread one
static_assert(kRankThreads >= MOE_MAX_EXPERTS, "one thread per expert in the offsets scan");

// The rank step of tile t, once thread e < E holds `base` (expert e's assignments in the tiles
// before t) and `tot` (all of expert e's assignments); other threads hold zeros. A block scan
// of the kept counts gives the expert offsets (tile 0's workgroup stores counts and offsets).
// The first wavefront then walks the tile's entries in flat order, 64 at a time: lanes with the
// same expert find each other with ballots over the expert id's bits, so a lane's rank among
// equal keys is a popcount of lower lanes, and the group's last lane advances the running
// position in LDS. Writes both index maps.
__device__ __forceinline__ void rank_tile(const int32_t* __restrict__ ids, int R, int E, int nbits,
                                          int cap, int t, int base, int tot,
                                          int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                          int32_t* __restrict__ s2f, int32_t* __restrict__ f2s) {
  __shared__ int32_t run[MOE_MAX_EXPERTS], lim[MOE_MAX_EXPERTS];
  __shared__ int32_t wave_sum[kRankThreads / kWave];
  const int tid = threadIdx.x;
  const int kept = tid < E ? min(tot, cap) : 0;  // kept assignments (capacity factor)
  const int incl = block_inclusive_scan_1024(kept, wave_sum);
  if (tid < E) {
    const int o = incl - kept;  // the expert's first row
    run[tid] = o + base;        // this tile's first position inside the expert
    lim[tid] = o + kept;        // positions at or past it are beyond the capacity
    if (t == 0) {
      counts[tid] = kept;
      offsets[tid] = o;
      if (tid == E - 1) offsets[E] = incl;
    }
  }
  __syncthreads();
  if (tid >= kWave) return;
  // One wavefront walks the tile: its LDS accesses take effect in program order, so no barrier is
  // needed between a chunk's reads of the running positions and their update; the wave barriers
  // only keep the compiler from moving LDS accesses across them.
  const int lane = tid;
  const int base_i = t * kPermuteTile;
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  // the tile's expert ids, all loaded before the walk (one memory latency, not one per chunk):
  // buffer loads through a descriptor that ends at the batch's last entry read zeros past it,
  // so the loads carry no condition that the compiler could turn into a branch around each
  const __amdgpu_buffer_rsrc_t tile_ids = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(ids + base_i), (short)0, (int)(min(R - base_i, kPermuteTile) * 4), kRawBufferWord3);
  constexpr int kChunks = kPermuteTile / kWave;
  int key[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) key[c] = clamp_expert(load_tile_id(tile_ids, c * kWave + lane), E);
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int cc = 0; cc < kChunks; ++cc) {
    const int i = base_i + cc * kWave + lane;
    const bool valid = i < R;
    const int ek = key[cc];
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (ek >> b) & 1;
      const uint64_t ones = __ballot(bit);
      same &= bit ? ones : ~ones;
    }
    if (valid) {
      // positions at or past the expert's end are beyond its capacity: dropped
      const int pos = run[ek] + __popcll(same & lower);
      if (pos < lim[ek]) s2f[pos] = i;
      f2s[i] = pos < lim[ek] ? pos : -1;
    }
    __builtin_amdgcn_wave_barrier();
    // the highest lane of each group of equal experts advances that expert's position
    if (valid && (63 - __clzll(same)) == lane) run[ek] += __popcll(same);
    __builtin_amdgcn_wave_barrier();
  }
}

// One workgroup per tile t. Thread (q, e) sums expert e's histogram entries over slice q of the
// tiles (all of them, and those before t), loads issued 16 at a time; the slices are added in
// LDS in a fixed order; then rank_tile.
__global__ __launch_bounds__(kRankThreads) void permute_rank_kernel(const int32_t* __restrict__ ids,
                                                                    int R, int E, int nbits, int cap,
                                                                    const int32_t* __restrict__ hist,
                                                                    int n_tiles,
                                                                    int32_t* __restrict__ counts,
                                                                    int32_t* __restrict__ offsets,
                                                                    int32_t* __restrict__ s2f,
                                                                    int32_t* __restrict__ f2s) {
  __shared__ int32_t pre_s[kRankThreads], tot_s[kRankThreads];
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  int Ep = 1;
  while (Ep < E) Ep <<= 1;  // <= 1024
  const int Q = kRankThreads / Ep;
  const int e = tid % Ep, q = tid / Ep;
  const int tpq = (n_tiles + Q - 1) / Q;
  const int t0 = min(q * tpq, n_tiles), t1 = min(t0 + tpq, n_tiles);
  int pre = 0, tot = 0;
  if (e < E) {
    constexpr int B = 16;
    for (int tb = t0; tb < t1; tb += B) {
      int h[B];
#pragma unroll
      for (int u = 0; u < B; ++u) h[u] = tb + u < t1 ? hist[(size_t)(tb + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < B; ++u) {
        tot += h[u];
        pre += tb + u < t ? h[u] : 0;
      }
    }
  }
  pre_s[tid] = pre;
  tot_s[tid] = tot;
  __syncthreads();
  int base = 0, tt = 0;
  if (tid < E) {
    for (int qq = 0; qq < Q; ++qq) {
      tt += tot_s[qq * Ep + tid];
      base += pre_s[qq * Ep + tid];
    }
  }
  rank_tile(ids, R, E, nbits, cap, t, base, tt, counts, offsets, s2f, f2s);
}

// Mid-size batches (R <= kCountMaxR, E <= kCountMaxE): one launch does the counting and the
// ranking. Every tile's workgroup counts the whole batch itself (the ids are R * 4 bytes, as
// many as the tile histograms the rank kernel above reads when E = kPermuteTile) into per-wave
// LDS histograms, split at its own tile's start, which saves the histogram launch; then
// rank_tile. Wave w counts the 64-entry chunks w, w + 16, w + 32, ..., kCountBatch loads in
// flight; its histograms are its own, so only lanes of one instruction share an address (LDS
// atomic adds). (64 loads in flight instead of 32 measured the same at 65,536 assignments.)
constexpr int kCountMaxR = 65536;
constexpr int kCountMaxE = 256;
constexpr int kCountBatch = 32;
__global__ __launch_bounds__(kRankThreads) void permute_count_rank_kernel(
    const int32_t* __restrict__ ids, int R, int E, int nbits, int cap, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ s2f, int32_t* __restrict__ f2s) {
  constexpr int NWV = kRankThreads / kWave;
  __shared__ int32_t before[NWV * kCountMaxE], from[NWV * kCountMaxE];
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int t = blockIdx.x;
  const int base_i = t * kPermuteTile;  // a multiple of 64: no chunk straddles it
  for (int i = tid; i < NWV * kCountMaxE; i += kRankThreads) {
    before[i] = 0;
    from[i] = 0;
  }
  __syncthreads();
  const __amdgpu_buffer_rsrc_t all_ids =
      __builtin_amdgcn_make_buffer_rsrc((void*)ids, (short)0, R * 4, kRawBufferWord3);
  const int nchunks = (R + kWave - 1) / kWave;
  int32_t* mine_before = before + wave * kCountMaxE;
  int32_t* mine_from = from + wave * kCountMaxE;
  for (int c0 = wave; c0 < nchunks; c0 += NWV * kCountBatch) {
    int key[kCountBatch];
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u) key[u] = load_tile_id(all_ids, (c0 + u * NWV) * kWave + lane);
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u) {
      const int c = c0 + u * NWV;
      if (c * kWave + lane < R)
        atomicAdd((c * kWave < base_i ? mine_before : mine_from) + clamp_expert(key[u], E), 1);
    }
  }
  __syncthreads();
  int base = 0, tot = 0;
  if (tid < E) {
    for (int w = 0; w < NWV; ++w) {
      base += before[w * kCountMaxE + tid];
      tot += from[w * kCountMaxE + tid];
    }
    tot += base;
  }
  rank_tile(ids, R, E, nbits, cap, t, base, tot, counts, offsets, s2f, f2s);
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
  if (n_tiles == 0) {  // an empty batch: no rows, every expert's count and offset is zero
    hipError_t st = launch_fill_i32(counts, E, 0, stream);
    return st == hipSuccess ? launch_fill_i32(offsets, E + 1, 0, stream) : st;
  }
  hipError_t st;
  if (R <= kCountMaxR && E <= kCountMaxE) {
    permute_count_rank_kernel<<<n_tiles, kRankThreads, 0, stream>>>(ids, R, E, nbits, cap, counts, offsets,
                                                                     sorted_to_flat, flat_to_sorted);
  } else {
    permute_hist_kernel<<<n_tiles, 256, lds, stream>>>(ids, R, E, ws);
    st = hipGetLastError();
    if (st != hipSuccess) return st;
    permute_rank_kernel<<<n_tiles, kRankThreads, 0, stream>>>(ids, R, E, nbits, cap, ws, n_tiles, counts,
                                                               offsets, sorted_to_flat, flat_to_sorted);
  }
  st = hipGetLastError();
  if (st != hipSuccess) return st;
  permute_copy_kernel<<<T, threads, 0, stream>>>(static_cast<const uint4*>(x), k, vpr,
                                                 flat_to_sorted, static_cast<uint4*>(x_sorted));
  return hipGetLastError();
}

}  // namespace moe
