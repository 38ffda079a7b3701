// Per-row FP8 E4M3 quantizer for gfx950: one 64-lane wavefront per row.
//
// Serves the per-output-channel weight quantization (offline) and the per-token
// activation quantization (run time) that page "Quantized Inference for OneRec-V2：
// 生成式推荐开始直接吃 LLM 量化栈", section 关键证据, describes; the recipe (scale from the
// row's absolute maximum with an epsilon floor, round, saturate) is the per-token
// quantizer of page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.2, read for E4M3
// with the +/-448 range of its §1.2.
//
// Per row of K values:
//   amax = max|x_i|                      (FP16 magnitudes compared as integers)
//   s    = fl32(max(amax, 2^-24) / 448)  (correctly rounded FP32 division)
//   q_i  = sign(x_i) | E4M3_RNE(min(fl32(|x_i| / s), 448))
//
// The per-element quotient uses Markstein's correction: with y = fl32(1/s) correctly
// rounded, q0 = fl32(|x| * y), r = fma(-q0, s, |x|) (exact) and q = fma(r, y, q0) is the
// correctly rounded |x| / s.  For this kernel's domain (|x| an FP16 value no larger than
// the row's FP16 amax, s derived from that amax) the identity was checked exhaustively,
// all 5.0e8 (x, amax) pairs, so the quotient is bit-identical to an IEEE division at a
// third of its cost.  Working on |x| and OR-ing the FP16 sign bit into the byte keeps
// -0 and negative underflow as 0x80 (RNE is symmetric in the sign).
//
// The FP32 -> E4M3 cast is the hardware v_cvt_pk_fp8_f32 (OCP E4M3 on gfx950, round to
// nearest even) on inputs already clamped to [0, 448], so it never sees an out-of-range
// value.
//
// RQ_ACT_SILU_MUL rows are [g (K) | u (K)] FP16; the quantized row is
// h = fl16(silu(g) * u) computed in FP32, so the SiLU, the FP16 rounding of h and the
// quantization happen in one pass over HBM.
//
// MoE rows quantized once per token go straight to each of the token's permuted slots
// (one copy per routed expert), so the grouped GEMM reads contiguous rows.
//
// Memory: each lane owns 16-byte chunks of the row (8 FP16 values), held in registers
// between the amax reduction and the cast, so the input is read from HBM once; loads and
// stores are 16- and 8-byte vectors, contiguous across the wave (each load instruction covers
// 1 KB of a row; pairing adjacent chunks per lane for 16-byte stores measured 20-55% slower).
// A row is one wavefront's, or is split over 2 or 4 wavefronts.
// Rows wider than 8192 values fall back to a two-pass loop that re-reads the row.

#include <atomic>

#include "common.h"

namespace rq {
namespace {

constexpr int kRowsPerBlock = 4;  // 4 wavefronts of 64 lanes, one row each

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// A 16-byte load marked non-temporal: each input row is read exactly once, so it should
// not displace the cached data that the next kernel reads (this kernel's own output, the
// GEMM's weights).  Measured on MI355X: 30% faster when the input is not cache-resident,
// 1% when it is.
__device__ __forceinline__ uint4 ld_stream_16(const void* p) {
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint32_t absmax_packed(uint4 v, uint32_t m) {
  // max over the 8 FP16 magnitudes; for non-NaN FP16, magnitude order = integer order
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo = w[i] & 0x7FFFu, hi = (w[i] >> 16) & 0x7FFFu;
    m = m > lo ? m : lo;
    m = m > hi ? m : hi;
  }
  return m;
}

__device__ __forceinline__ uint4 silu_mul8(uint4 g, uint4 u) {
  return make_uint4(silu_mul_pair(g.x, u.x), silu_mul_pair(g.y, u.y),
                    silu_mul_pair(g.z, u.z), silu_mul_pair(g.w, u.w));
}

// Largest finite magnitude of the target format: E4M3 448, or E5M2 57344 (the E5M2
// activations of page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.2).  57344 = 448 * 128,
// so an E5M2 row's scale and rcp(scale) are the E4M3 ones times 2^-7 and 2^7 exactly and every
// step of the quotient below scales by 2^7 exactly: the exhaustive check of the E4M3 quotient
// covers the E5M2 one as well.
template <bool E5>
constexpr float kQMax = E5 ? 57344.0f : kFp8Max;

template <bool E5>
__device__ __forceinline__ float quotient(uint32_t hbits, float s, float rcp) {
  float ax = half_bits_to_float(hbits & 0x7FFFu);
  float q0 = ax * rcp;
  float r = __builtin_fmaf(-q0, s, ax);
  float q = __builtin_fmaf(r, rcp, q0);
  return __builtin_fminf(q, kQMax<E5>);
}

// Four FP16 values (two packed words) -> four E4M3 (or E5M2) bytes (one word).  The cast is
// the hardware v_cvt_pk_fp8_f32 (v_cvt_pk_bf8_f32 for E5M2: OCP formats on gfx950, round to
// nearest even) on magnitudes already clamped to the format's largest finite value.
template <bool E5 = false>
__device__ __forceinline__ uint32_t cast4(uint32_t d0, uint32_t d1, float s, float rcp) {
  int w;
  if constexpr (E5) {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(quotient<E5>(d0, s, rcp), quotient<E5>(d0 >> 16, s, rcp), 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(quotient<E5>(d1, s, rcp), quotient<E5>(d1 >> 16, s, rcp), w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(quotient<E5>(d0, s, rcp), quotient<E5>(d0 >> 16, s, rcp), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(quotient<E5>(d1, s, rcp), quotient<E5>(d1 >> 16, s, rcp), w, true);
  }
  uint32_t signs = ((d0 >> 8) & 0x80u) | ((d0 >> 16) & 0x8000u) | ((d1 << 8) & 0x800000u) |
                   (d1 & 0x80000000u);
  return (uint32_t)w | signs;
}

template <bool E5 = false>
__device__ __forceinline__ void row_scale(uint32_t amax_bits, float& s, float& rcp) {
  float amax = half_bits_to_float(amax_bits);
  s = __fdiv_rn(__builtin_fmaxf(amax, kScaleFloor), kQMax<E5>);
  rcp = __fdiv_rn(1.0f, s);
}

// One row per SPLIT wavefronts (SPLIT = 1, 2 or 4; 4 wavefronts per workgroup): lane l of
// wavefront part p owns chunks c = 64 p + l + 64 SPLIT j, j < CPL.  Splitting a long row over
// several wavefronts keeps enough of them in flight when there are few rows; their partial
// maxima meet in LDS.
// The workgroups walk groups of 4 / SPLIT rows (group g, g + gridDim.x, ...).  With PREFETCH a
// wavefront issues the loads of its next group before it reduces, casts and stores the
// current one, so its loads stay in flight through the latency of the row's reduction: the
// launch holds only as many workgroups as stay resident, and each streams several groups.
template <int CPL, bool SILU, int SPLIT, bool E5, bool PREFETCH>
__global__ __launch_bounds__(256) void quant_rows_regs(const uint16_t* __restrict__ x, int64_t rows,
                                                       int K, uint8_t* __restrict__ q,
                                                       float* __restrict__ scale,
                                                       uint16_t* __restrict__ h_out,
                                                       const int32_t* __restrict__ pos, int fanout) {
  static_assert(SPLIT == 1 || SPLIT == 2 || SPLIT == 4, "wavefronts per row");
  constexpr int kGroupRows = kRowsPerBlock / SPLIT;
  constexpr int NL = SILU ? 2 : 1;  // 16-byte loads per chunk: x, or g then u
  __shared__ uint32_t part_max[2][kRowsPerBlock];  // alternate groups use alternate halves
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int part = wave % SPLIT;
  const int64_t groups = (rows + kGroupRows - 1) / kGroupRows;
  const int nchunk = K >> 3;
  const int64_t in_stride = SILU ? 2 * (int64_t)K : (int64_t)K;
  const int c0 = 64 * part + lane;

  // this wavefront's input chunks of group grp (zero past the row's end or the last row)
  uint4 raw[CPL][NL];
  auto load = [&](int64_t grp) {
    const int64_t row = grp * kGroupRows + wave / SPLIT;
    const bool ok = row < rows;
    const uint16_t* xr = x + (ok ? row : 0) * in_stride;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = c0 + 64 * SPLIT * j;
#pragma unroll
      for (int t = 0; t < NL; ++t)
        raw[j][t] = ok && c < nchunk ? ld_stream_16(xr + (int64_t)t * K + 8 * c) : make_uint4(0, 0, 0, 0);
    }
  };
  int64_t grp = blockIdx.x;
  if (PREFETCH) load(grp);
  for (int it = 0; grp < groups; grp += gridDim.x, ++it) {
    if (!PREFETCH) load(grp);
    uint4 cur[CPL][NL];
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
      for (int t = 0; t < NL; ++t) cur[j][t] = raw[j][t];
    if (PREFETCH && grp + gridDim.x < groups) load(grp + gridDim.x);  // workgroup-uniform

    const int64_t row = grp * kGroupRows + wave / SPLIT;
    const bool valid = row < rows;
    uint4 v[CPL];
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = c0 + 64 * SPLIT * j;
      v[j] = make_uint4(0, 0, 0, 0);
      if (valid && c < nchunk) {
        v[j] = SILU ? silu_mul8(cur[j][0], cur[j][NL - 1]) : cur[j][0];
        amax = absmax_packed(v[j], amax);
      }
    }
    amax = wave_max_u32(amax);
    if (SPLIT > 1) {
      if (lane == 0) part_max[it & 1][wave] = amax;
      __syncthreads();
      const int first = wave - part;
#pragma unroll
      for (int p2 = 0; p2 < SPLIT; ++p2)
        amax = amax > part_max[it & 1][first + p2] ? amax : part_max[it & 1][first + p2];
    }
    if (!valid) continue;
    float s, rcp;
    row_scale<E5>(amax, s, rcp);

    uint2 out[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = c0 + 64 * SPLIT * j;
      if (c < nchunk) {
        out[j].x = cast4<E5>(v[j].x, v[j].y, s, rcp);
        out[j].y = cast4<E5>(v[j].z, v[j].w, s, rcp);
        if (SILU && h_out != nullptr) st_global_16(h_out + row * (int64_t)K + 8 * c, v[j]);
      }
    }
    const int copies = pos != nullptr ? fanout : 1;
    for (int d = 0; d < copies; ++d) {
      const int64_t orow = pos != nullptr ? (int64_t)pos[row * fanout + d] : row;
      uint8_t* qr = q + orow * (int64_t)K;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = c0 + 64 * SPLIT * j;
        if (c < nchunk) *reinterpret_cast<uint2*>(qr + 8 * c) = out[j];
      }
      if (part == 0 && lane == 0) scale[orow] = s;
    }
  }
}

// Rows wider than 64 * 8 * 16 values: two passes, the second re-reading the row.
template <bool SILU, bool E5>
__global__ __launch_bounds__(256) void quant_rows_loop(const uint16_t* __restrict__ x, int64_t rows,
                                                       int64_t K, uint8_t* __restrict__ q,
                                                       float* __restrict__ scale,
                                                       uint16_t* __restrict__ h_out,
                                                       const int32_t* __restrict__ pos, int fanout) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t nchunk = K >> 3;
  const int64_t in_stride = SILU ? 2 * K : K;
  const uint16_t* xr = x + row * in_stride;
  // the first pass loads normally so that the second, the row's last read, finds it cached
  auto chunk = [&](int64_t c, bool last) -> uint4 {
    auto ld = [&](const uint16_t* q) { return last ? ld_stream_16(q) : ld_global_16(q); };
    if (SILU) return silu_mul8(ld(xr + 8 * c), ld(xr + K + 8 * c));
    return ld(xr + 8 * c);
  };
  uint32_t amax = 0;
  for (int64_t c = lane; c < nchunk; c += 64) amax = absmax_packed(chunk(c, false), amax);
  amax = wave_max_u32(amax);
  float s, rcp;
  row_scale<E5>(amax, s, rcp);
  const int copies = pos != nullptr ? fanout : 1;
  for (int64_t c = lane; c < nchunk; c += 64) {
    uint4 v = chunk(c, true);
    uint2 out;
    out.x = cast4<E5>(v.x, v.y, s, rcp);
    out.y = cast4<E5>(v.z, v.w, s, rcp);
    for (int d = 0; d < copies; ++d) {
      const int64_t orow = pos != nullptr ? (int64_t)pos[row * fanout + d] : row;
      *reinterpret_cast<uint2*>(q + orow * K + 8 * c) = out;
    }
    if (SILU && h_out != nullptr) st_global_16(h_out + row * K + 8 * c, v);
  }
  for (int d = 0; d < copies && lane == 0; ++d)
    scale[pos != nullptr ? (int64_t)pos[row * fanout + d] : row] = s;
}

// Workgroups of the prefetching row quantizer the device keeps resident at once (all CUs),
// cached per device and wavefronts-per-row count with atomic operations (concurrent host
// threads may both compute it and store the same value).  0 if the runtime cannot tell.
template <int CPL, bool SILU, bool E5>
int64_t resident_quant_blocks(int split) {
  constexpr int kDevices = 64;
  static std::atomic<int> cache[kDevices][3];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevices) return 0;
  const int si = split == 4 ? 2 : split == 2 ? 1 : 0;
  const int known = cache[dev][si].load(std::memory_order_relaxed);
  if (known > 0) return known;
  int cus = 0, per_cu = 0;
  hipError_t e;
  if (split == 4) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quant_rows_regs<CPL, SILU, 4, E5, true>, 256, 0);
  else if (split == 2) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quant_rows_regs<CPL, SILU, 2, E5, true>, 256, 0);
  else e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, quant_rows_regs<CPL, SILU, 1, E5, true>, 256, 0);
  if (e != hipSuccess || per_cu <= 0 ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 0;
  cache[dev][si].store(cus * per_cu, std::memory_order_relaxed);
  return (int64_t)cus * per_cu;
}

template <int CPL, bool SILU, bool E5>
hipError_t launch_split(int split, const uint16_t* x, int64_t rows, int k, uint8_t* q, float* scale, uint16_t* h,
                        const int32_t* pos, int fanout, hipStream_t stream) {
  const dim3 block(64 * kRowsPerBlock);
  const int per_block = kRowsPerBlock / split;
  const int64_t groups = (rows + per_block - 1) / per_block;
  // Prefetching launch: as many workgroups as stay resident, each walking several groups with
  // two sets of CPL chunks in registers (the current group's and the next one's).  Used while
  // the sets stay small and each workgroup walks at most 4 groups; longer launches run one
  // group per workgroup at the occupancy of a single set.  Measured on MI355X with caches
  // flushed: 4096 x 8192 rows 23.7 -> 23.1 us, 16384 x 2048 rows with two output copies
  // 29.0 -> 28.4 us, 4096 x 2048 rows 11.1 -> 10.4 us; 32768 x 4096 rows (16 groups per
  // resident workgroup) 67.3 -> 69.7 us, hence the limit.
  constexpr bool kCanPrefetch = CPL * (SILU ? 2 : 1) <= 8;
  bool prefetch = false;
  int64_t blocks = groups;
  if constexpr (kCanPrefetch) {
    const int64_t cap = resident_quant_blocks<CPL, SILU, E5>(split);
    if (cap > 0 && groups <= 4 * cap) {
      prefetch = true;
      blocks = groups < cap ? groups : cap;
    }
  }
  const dim3 grid((unsigned)blocks);
  if (prefetch) {
    if (split == 4)
      quant_rows_regs<CPL, SILU, 4, E5, kCanPrefetch><<<grid, block, 0, stream>>>(x, rows, k, q, scale, h, pos, fanout);
    else if (split == 2)
      quant_rows_regs<CPL, SILU, 2, E5, kCanPrefetch><<<grid, block, 0, stream>>>(x, rows, k, q, scale, h, pos, fanout);
    else
      quant_rows_regs<CPL, SILU, 1, E5, kCanPrefetch><<<grid, block, 0, stream>>>(x, rows, k, q, scale, h, pos, fanout);
  } else {
    if (split == 4)
      quant_rows_regs<CPL, SILU, 4, E5, false><<<grid, block, 0, stream>>>(x, rows, k, q, scale, h, pos, fanout);
    else if (split == 2)
      quant_rows_regs<CPL, SILU, 2, E5, false><<<grid, block, 0, stream>>>(x, rows, k, q, scale, h, pos, fanout);
    else
      quant_rows_regs<CPL, SILU, 1, E5, false><<<grid, block, 0, stream>>>(x, rows, k, q, scale, h, pos, fanout);
  }
  return hipGetLastError();
}

template <bool SILU, bool E5>
hipError_t launch_impl(const uint16_t* x, int64_t rows, int64_t K, uint8_t* q, float* scale,
                       uint16_t* h, const int32_t* pos, int fanout, hipStream_t stream) {
  const int64_t nchunk = K / 8;
  const int k = (int)K;
  if (nchunk > 64 * 16) {
    const dim3 grid((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
    quant_rows_loop<SILU, E5><<<grid, dim3(64 * kRowsPerBlock), 0, stream>>>(x, rows, K, q, scale, h, pos, fanout);
    return hipGetLastError();
  }
  // Wavefronts per row: split long rows while the launch would hold fewer than 65536
  // wavefronts, keeping at least 2 chunks per lane.  Measured on MI355X with L2 and the
  // last-level cache flushed: 4096 x 8192 rows 25.1 -> 22.9 us (4 wavefronts per row),
  // 16384 x 2048 rows with two output copies 30.2 -> 28.1 us and 32768 x 4096 rows
  // 68.4 -> 65.7 us (2 per row), against one or two per row under an 8192-wavefront rule.
  int split = 1;
  while (split < 4 && rows * split < 65536 && nchunk >= 64 * 2 * 2 * split) split *= 2;
  const int64_t per_lane = (nchunk + 64 * split - 1) / (64 * split);
  if (per_lane <= 1) return launch_split<1, SILU, E5>(split, x, rows, k, q, scale, h, pos, fanout, stream);
  if (per_lane <= 2) return launch_split<2, SILU, E5>(split, x, rows, k, q, scale, h, pos, fanout, stream);
  if (per_lane <= 4) return launch_split<4, SILU, E5>(split, x, rows, k, q, scale, h, pos, fanout, stream);
  if (per_lane <= 8) return launch_split<8, SILU, E5>(split, x, rows, k, q, scale, h, pos, fanout, stream);
  return launch_split<16, SILU, E5>(split, x, rows, k, q, scale, h, pos, fanout, stream);
}

// ---- weight scales per 128 x 128 block and per tensor (page "FP8量化在生成式推荐系统
// OneRec-V2中的优化实践", §2.1 / §2.2: MoE expert weights block-wise, dense FFN weights per
// tensor).  The row formula above applies to the set of values that shares a scale; the
// quotient is the same Markstein one, valid because every |x| in the set is at most the
// set's FP16 amax.

// One 128 x 128 block per workgroup of 256 lanes: lane t reads 64 consecutive values (eight
// 16-byte chunks) of block row t / 2, holds them in registers across the block's amax
// reduction, then casts and stores them.  Scales are written in [B][N/128][K/128] order,
// which is the workgroup order.
__global__ __launch_bounds__(256) void quant_blocks_kernel(const uint16_t* __restrict__ w, int64_t N, int64_t K,
                                                           uint8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ uint32_t part_max[4];
  const int64_t nb = N / kScaleBlock, kb = K / kScaleBlock;
  const int64_t blk = blockIdx.x;
  const int64_t mat = blk / (nb * kb), in_mat = blk % (nb * kb);
  const int64_t bi = in_mat / kb, bj = in_mat % kb;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t row = mat * N + bi * kScaleBlock + (t >> 1);
  const int64_t col = bj * kScaleBlock + (t & 1) * 64;
  const uint16_t* src = w + row * K + col;
  uint4 v[8];
  uint32_t amax = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    v[j] = ld_global_16(src + 8 * j);
    amax = absmax_packed(v[j], amax);
  }
  amax = wave_max_u32(amax);
  if (lane == 0) part_max[wave] = amax;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) amax = amax > part_max[i] ? amax : part_max[i];
  float s, rcp;
  row_scale(amax, s, rcp);
  uint8_t* dst = q + row * K + col;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    *reinterpret_cast<uint2*>(dst + 8 * j) = make_uint2(cast4(v[j].x, v[j].y, s, rcp), cast4(v[j].z, v[j].w, s, rcp));
  if (t == 0) scale[blk] = s;
}

// Per-tensor scales in three steps on the stream: clear each matrix's amax word, fold every
// row's FP16 magnitude maximum into it (an integer maximum, so the order of the atomic
// updates does not matter), then quantize every row with its matrix's scale and finally
// replace each amax word by the FP32 scale.  The amax words live in the scale array itself.
__global__ __launch_bounds__(256) void clear_words(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ __launch_bounds__(256) void tensor_amax_kernel(const uint16_t* __restrict__ w, int64_t rows, int64_t N,
                                                          int64_t K, uint32_t* __restrict__ amax_word) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  const uint16_t* xr = w + row * K;
  uint32_t amax = 0;
  for (int64_t c = lane; c < K / 8; c += 64) amax = absmax_packed(ld_stream_16(xr + 8 * c), amax);
  amax = wave_max_u32(amax);
  if (lane == 0) atomicMax(amax_word + row / N, amax);
}

__global__ __launch_bounds__(256) void tensor_cast_kernel(const uint16_t* __restrict__ w, int64_t rows, int64_t N,
                                                          int64_t K, const uint32_t* __restrict__ amax_word,
                                                          uint8_t* __restrict__ q) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  float s, rcp;
  row_scale(amax_word[row / N], s, rcp);
  const uint16_t* xr = w + row * K;
  uint8_t* qr = q + row * K;
  for (int64_t c = lane; c < K / 8; c += 64) {
    const uint4 v = ld_stream_16(xr + 8 * c);
    *reinterpret_cast<uint2*>(qr + 8 * c) = make_uint2(cast4(v.x, v.y, s, rcp), cast4(v.z, v.w, s, rcp));
  }
}

__global__ __launch_bounds__(256) void tensor_scale_kernel(float* __restrict__ scale, int64_t B) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= B) return;
  float s, rcp;
  row_scale(__builtin_bit_cast(uint32_t, scale[b]), s, rcp);
  scale[b] = s;
}

}  // namespace

hipError_t launch_quant_blocks(const uint16_t* w, int64_t B, int64_t N, int64_t K, uint8_t* q, float* scale,
                               hipStream_t stream) {
  const int64_t blocks = B * (N / kScaleBlock) * (K / kScaleBlock);
  if (blocks <= 0) return hipSuccess;
  quant_blocks_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(w, N, K, q, scale);
  return hipGetLastError();
}

hipError_t launch_quant_tensor(const uint16_t* w, int64_t B, int64_t N, int64_t K, uint8_t* q, float* scale,
                               hipStream_t stream) {
  const int64_t rows = B * N;
  if (rows <= 0) return hipSuccess;
  uint32_t* word = reinterpret_cast<uint32_t*>(scale);
  const unsigned row_blocks = (unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock);
  const unsigned b_blocks = (unsigned)((B + 255) / 256);
  clear_words<<<dim3(b_blocks), dim3(256), 0, stream>>>(word, B);
  tensor_amax_kernel<<<dim3(row_blocks), dim3(64 * kRowsPerBlock), 0, stream>>>(w, rows, N, K, word);
  tensor_cast_kernel<<<dim3(row_blocks), dim3(64 * kRowsPerBlock), 0, stream>>>(w, rows, N, K, word, q);
  tensor_scale_kernel<<<dim3(b_blocks), dim3(256), 0, stream>>>(scale, B);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t K, int act, uint8_t* q,
                             float* scale, uint16_t* h, const int32_t* pos, int fanout,
                             hipStream_t stream, int fmt) {
  if (rows <= 0) return hipSuccess;
  if (fmt == kFmtE5M2) {
    if (act == 1) return launch_impl<true, true>(x, rows, K, q, scale, h, pos, fanout, stream);
    return launch_impl<false, true>(x, rows, K, q, scale, nullptr, pos, fanout, stream);
  }
  if (act == 1) return launch_impl<true, false>(x, rows, K, q, scale, h, pos, fanout, stream);
  return launch_impl<false, false>(x, rows, K, q, scale, nullptr, pos, fanout, stream);
}

}  // namespace rq
