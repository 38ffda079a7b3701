// FP8 (OCP E4M3) x FP8 GEMM with FP32 accumulation and a fused per-token x per-channel
// dequantization to FP16, for gfx950 (MI355X).
//
// Computes y[m][n] = fl16(fl32(acc * s_a[m]) * s_b[n]), acc = sum_k a[m][k] * b[n][k]:
// the FP8 product with FP32 accumulation and the cast back to FP16 of page "Quantized
// Inference for OneRec-V2：生成式推荐开始直接吃 LLM 量化栈", section 关键证据, with the
// quantize -> FP8 GEMM -> dequantize flow of page "FP8量化在生成式推荐系统OneRec-V2中的
// 优化实践", §2.3 / Fig. 2.  Both operands are K-contiguous ("TN"): activations [M][K],
// weights [N][K] in the nn.Linear layout.
//
// Design (CDNA4):
// * Matrix core: v_mfma_f32_16x16x128_f8f6f4 (FP8 x FP8, K = 128 per instruction, the
//   full-rate FP8 MFMA of gfx950).  Each lane feeds 32 bytes of one A row and 32 bytes of
//   one B column; the four 16-lane groups take the four 32-byte quarters of the 128-byte
//   K block.  A and B use the same K assignment, so the dot product is the plain one.
// * Tiles: 128 x 128 outputs per 256-thread workgroup, 4 wavefronts in a 2 x 2 grid, each
//   owning 64 x 64 outputs = 4 x 4 MFMA tiles (64 FP32 accumulators per lane).
// * LDS: A and B K-slabs of 128 x 128 bytes, double-buffered (64 KB).  Rows are 128 bytes;
//   the 16-byte granule g of row r is stored at granule g ^ (r & 7) ^ ((r >> 3) & 1), so the
//   16-byte fragment reads of 16 consecutive rows and the 16-byte stores of 8 lanes along a
//   row both spread over all banks.
// * Global loads are 16-byte vectors, 8 lanes per 128-byte row segment; the next K-slab is
//   fetched into registers while the MFMAs consume the current one; one barrier per slab.
// * Tile order: the hardware hands consecutive workgroup ids to the 8 XCDs in turn; ids are
//   remapped so each XCD receives a contiguous range of the logical order, and the logical
//   order walks groups of 8 M-tiles across all N-tiles, so tiles that share A rows or B
//   columns run on the same XCD and hit its L2.
// * Epilogue: per-row and per-column FP32 scales, round to nearest even to FP16.
//
// Grouped (MoE) mode: the M-tiles are the concatenation over experts of
// ceil(count_e / 128) tiles each (tile_start = exclusive scan, built on the device by the
// routing plan).  A workgroup finds its expert by binary search, reads A rows through the
// permutation (token perm[r] / top_k) when the input is per token, uses expert e's
// weights and scales, and writes permuted output rows.  Tiles past the device-side total
// exit at once, so the host never needs the per-expert counts.
// Ragged edges (M, N not multiples of 128, K not a multiple of 128) are zero-filled in LDS
// and masked in the epilogue.

#include "common.h"

namespace rq {
namespace {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 128;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;
constexpr int kLoadsPerThread = BM * BK / 16 / kThreads;  // 16-byte granules per operand

__device__ __forceinline__ int swz(int row, int g) { return g ^ (row & 7) ^ ((row >> 3) & 1); }

struct TileInfo {
  int64_t row_begin;
  int64_t row_end;
  int nt;
  int expert;
};

template <bool GROUPED>
__device__ __forceinline__ bool map_tile(const GemmArgs& p, int m_tiles, int n_tiles, TileInfo& t) {
  const int total = (int)gridDim.x;
  int bid = (int)blockIdx.x;
  if ((total & 7) == 0) bid = (bid & 7) * (total >> 3) + (bid >> 3);
  const int per_group = kGroupM * n_tiles;
  const int group = bid / per_group;
  const int first_m = group * kGroupM;
  const int gm = min(m_tiles - first_m, kGroupM);
  const int in_group = bid - group * per_group;
  const int mt = first_m + in_group % gm;
  t.nt = in_group / gm;
  if (GROUPED) {
    const int real_tiles = p.tile_start[p.E];
    if (mt >= real_tiles) return false;
    int lo = 0, hi = p.E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.tile_start[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    t.expert = lo;
    t.row_begin = (int64_t)p.offsets[lo] + (int64_t)(mt - p.tile_start[lo]) * BM;
    const int64_t end = p.offsets[lo + 1];
    t.row_end = t.row_begin + BM < end ? t.row_begin + BM : end;
  } else {
    t.expert = 0;
    t.row_begin = (int64_t)mt * BM;
    t.row_end = t.row_begin + BM < p.M ? t.row_begin + BM : p.M;
  }
  return true;
}

template <bool GROUPED>
__device__ __forceinline__ int64_t a_source_row(const GemmArgs& p, int64_t r) {
  if (GROUPED && p.gather_tokens) return (int64_t)(p.perm[r] / p.top_k);
  return r;
}

template <bool GROUPED>
__global__ __launch_bounds__(kThreads) void gemm_fp8_kernel(GemmArgs p, int m_tiles, int n_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (BM + BN) * BK];
  TileInfo t;
  if (!map_tile<GROUPED>(p, m_tiles, n_tiles, t)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t K = p.K;
  const int64_t N = p.N;
  const uint8_t* __restrict__ B = p.b + (int64_t)t.expert * N * K;
  const float* __restrict__ sb = p.b_scale + (int64_t)t.expert * N;
  const int n0 = t.nt * BN;

  // ---- global -> LDS assignment: granule (row, g) with g = tid & 7
  const int g = tid & 7;
  const uint8_t* a_src[kLoadsPerThread];
  const uint8_t* b_src[kLoadsPerThread];
  int lds_off[kLoadsPerThread];
#pragma unroll
  for (int i = 0; i < kLoadsPerThread; ++i) {
    const int row = (tid >> 3) + 32 * i;
    const int64_t r = t.row_begin + row;
    a_src[i] = (r < t.row_end) ? p.a + a_source_row<GROUPED>(p, r) * K + 16 * g : nullptr;
    const int64_t n = n0 + row;
    b_src[i] = (n < N) ? B + n * K + 16 * g : nullptr;
    lds_off[i] = row * BK + 16 * swz(row, g);
  }

  uint4 ra[kLoadsPerThread], rb[kLoadsPerThread];
  auto load_slab = [&](int64_t k0) {
    const bool kin = (k0 + 16 * g) < K;
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
      ra[i] = (kin && a_src[i]) ? ld_global_16(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
      rb[i] = (kin && b_src[i]) ? ld_global_16(b_src[i] + k0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_slab = [&](int buf) {
    uint8_t* As = smem + buf * (BM + BN) * BK;
    uint8_t* Bs = As + BM * BK;
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
      *reinterpret_cast<uint4*>(As + lds_off[i]) = ra[i];
      *reinterpret_cast<uint4*>(Bs + lds_off[i]) = rb[i];
    }
  };

  // ---- MFMA fragment addressing: lane -> (row within 16, K quarter)
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int frow = lane & 15;
  const int quarter = lane >> 4;
  const int f_off0 = frow * BK + 16 * swz(frow, 2 * quarter);
  const int f_off1 = frow * BK + 16 * swz(frow, 2 * quarter + 1);

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (v4f){0.f, 0.f, 0.f, 0.f};

  const int ktiles = (int)((K + BK - 1) / BK);
  load_slab(0);
  store_slab(0);
  __syncthreads();

  for (int kt = 0; kt < ktiles; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < ktiles) load_slab((int64_t)(kt + 1) * BK);

    const uint8_t* As = smem + cur * (BM + BN) * BK + (wm * 64) * BK;
    const uint8_t* Bs = smem + cur * (BM + BN) * BK + BM * BK + (wn * 64) * BK;
    v8i af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 lo = *reinterpret_cast<const uint4*>(As + i * 16 * BK + f_off0);
      const uint4 hi = *reinterpret_cast<const uint4*>(As + i * 16 * BK + f_off1);
      af[i] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 lo = *reinterpret_cast<const uint4*>(Bs + j * 16 * BK + f_off0);
      const uint4 hi = *reinterpret_cast<const uint4*>(Bs + j * 16 * BK + f_off1);
      bf[j] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bf[j], acc[i][j],
                                                                      0, 0, 0, 0, 0, 0);

    if (kt + 1 < ktiles) store_slab(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds rows 4*quarter + r, column frow of each 16x16 tile
  float sbv[4];
  int64_t ncol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ncol[j] = n0 + wn * 64 + 16 * j + frow;
    sbv[j] = ncol[j] < N ? sb[ncol[j]] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = t.row_begin + wm * 64 + 16 * i + 4 * quarter + r;
      if (row >= t.row_end) continue;
      const float sa = p.a_scale[a_source_row<GROUPED>(p, row)];
      uint16_t* yr = p.y + row * N;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (ncol[j] < N) {
          const float v = (acc[i][j][r] * sa) * sbv[j];
          yr[ncol[j]] = (uint16_t)float_to_half_bits(v);
        }
      }
    }
  }
}

}  // namespace

int grouped_tile_m() { return BM; }

int64_t grouped_max_mtiles(int64_t R, int64_t E) { return (R + BM - 1) / BM + E; }

hipError_t launch_gemm_dense(const GemmArgs& g, hipStream_t stream) {
  if (g.M <= 0) return hipSuccess;
  const int m_tiles = (int)((g.M + BM - 1) / BM);
  const int n_tiles = (int)((g.N + BN - 1) / BN);
  gemm_fp8_kernel<false><<<dim3(m_tiles * n_tiles), dim3(kThreads), 0, stream>>>(g, m_tiles, n_tiles);
  return hipGetLastError();
}

hipError_t launch_gemm_grouped(const GemmArgs& g, hipStream_t stream) {
  if (g.M <= 0) return hipSuccess;
  const int m_tiles = (int)grouped_max_mtiles(g.M, g.E);
  const int n_tiles = (int)((g.N + BN - 1) / BN);
  gemm_fp8_kernel<true><<<dim3(m_tiles * n_tiles), dim3(kThreads), 0, stream>>>(g, m_tiles, n_tiles);
  return hipGetLastError();
}

}  // namespace rq
