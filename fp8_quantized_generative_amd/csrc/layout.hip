// Offline weight packing into the slab layout the GEMM streams fastest from HBM.
//
// The GEMM reads a tile's weights as slabs of (tile columns) rows x 64 K bytes.  In the
// [N][K] row layout each slab row is a separate 64-byte piece K bytes from the next, and HBM
// streams such pieces markedly slower than contiguous runs.  The slab layout [B][K/64][N][64]
// stores the 64-byte K slab of every row of a matrix together, rows in order, so a tile's slab
// is one contiguous run and the tiles working on one slab read neighbouring runs.  Packing is
// a byte permutation: the values, scales and results are those of the row layout.

#include "common.h"

namespace rq {
namespace {

// One thread per 16-byte granule of the output, in output order: writes are contiguous and
// every 64-byte piece of a source row is read by four neighbouring lanes.
__global__ __launch_bounds__(256) void pack_slabs_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                         int64_t total, int64_t N, int64_t K) {
  const int64_t per_matrix = N * K / 16;  // granules of one matrix
  const int64_t per_slab = N * 4;         // granules of one K slab (N rows x 64 bytes)
  for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < total;
       d += (int64_t)gridDim.x * blockDim.x) {
    const int64_t b = d / per_matrix;
    const int64_t rem = d - b * per_matrix;
    const int64_t slab = rem / per_slab;
    const int64_t within = rem - slab * per_slab;
    const int64_t row = b * N + (within >> 2);
    dst[d] = src[(row * K + slab * 64) / 16 + (within & 3)];
  }
}

}  // namespace

hipError_t launch_pack_slabs(const uint8_t* w_q, int64_t B, int64_t N, int64_t K, uint8_t* w_packed,
                             hipStream_t stream) {
  const int64_t total = B * N * K / 16;
  if (total == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 8192);
  hipLaunchKernelGGL(pack_slabs_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(w_q), reinterpret_cast<uint4*>(w_packed), total, N, K);
  return hipGetLastError();
}

}  // namespace rq
