// Conversion of expert weights into the blocked layouts that the GEMM tiles read (8 rows x 128
// bytes per block: 64 bf16 or 128 fp8 e4m3fn contraction elements of 8 consecutive output rows).
// A layout change only, done once before the weights are used: the order of every expert's
// arithmetic in the tiles is unchanged, only the address of each 16-byte piece they load.
//
// HBM-bound copy: each 16-byte piece is read once and written once.
#include "moe_internal.h"

namespace moe {

// Blocked weights from row-major ones (8 rows x 128 bytes per block): threads walk the 16-byte
// pieces of the destination in destination order (a grid-stride loop: a tensor may hold more
// pieces than one dispatch has threads), so the stores are contiguous and each source piece is
// read by one thread.
__global__ __launch_bounds__(256) void block_weights_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                            long long row_bytes, long long pieces) {
  const long long per_row = row_bytes / 128;
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < pieces; i += stride) {
    // destination piece i: block (e, n/8, 128-byte column c8), row n%8 of it, 16-byte piece c
    const int c = (int)(i & 7), r = (int)((i >> 3) & 7);
    const long long blk = i >> 6;                  // (e * (N/8) + n/8) * (row_bytes/128) + c8
    const long long c8 = blk % per_row;
    const long long row = blk / per_row * 8 + r;   // e * N + n
    dst[i] = src[(row * row_bytes + c8 * 128 + c * 16) / 16];
  }
}

hipError_t launch_block_weights(const void* src, void* dst, int E, int N, long long row_bytes,
                                hipStream_t stream) {
  const long long pieces = (long long)E * N * row_bytes / 16;
  // at most 2^20 workgroups (2^28 threads): far below the dispatch's 32-bit thread count, and
  // enough to fill every compute unit many times over
  const long long want = (pieces + 255) / 256;
  const unsigned grid = (unsigned)(want < (1LL << 20) ? want : (1LL << 20));
  block_weights_kernel<<<grid, 256, 0, stream>>>(static_cast<const u32x4*>(src), static_cast<u32x4*>(dst),
                                                 row_bytes, pieces);
  return hipGetLastError();
}

}  // namespace moe
