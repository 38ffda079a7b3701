// MoE routing plan and weighted combine for the expert grouped GEMM (gfx950).
//
// Page "Quantized Inference for OneRec-V2：生成式推荐开始直接吃 LLM 量化栈", section
// 关键证据, runs the sparse-MoE experts as one grouped GEMM on the quantized path; page
// "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.1, keeps the routing gate in FP16, so
// its top-k expert ids and weights are inputs here.
//
// Plan: slot j = t * top_k + k goes to expert ids[j].  The canonical permuted order sorts
// slots by (expert, j) - a stable counting sort - computed without any host round trip.  Up to
// 8192 slots (and 256 experts) one workgroup does it all in a single launch (plan_single);
// beyond, three kernels:
//   1. plan_hist:    per block of 1024 slots, a histogram over experts (LDS atomics on
//                    integer counts, so the result is deterministic);
//   2. plan_scan:    one workgroup turns the block histograms into per-expert offsets,
//                    per-(block, expert) base rows, the per-expert M-tile prefix sum and
//                    the M-tile table {expert, first row, end row} the grouped GEMM reads,
//                    with every thread busy (segment sums, LDS scans, one table entry each);
//   3. plan_scatter: each slot's rank among equal experts inside its wavefront comes from
//                    ballots over the bits of the expert id; ranks across the block's 16
//                    wavefronts come from an LDS prefix; perm[row] = j and pos[j] = row.
// Combine: out[t] = fl16(sum_k fl32(w[t][k] * y_perm[pos[t*top_k + k]])), summed in FP32 in
// slot order (each FP16 x FP16 product is exact in FP32), 16-byte loads and stores.

#include "common.h"

namespace rq {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;

// Device error word of this GPU (each device holds its own copy): the routing-plan kernels
// set kErrExpertId when an expert id lies outside [0, E).  Host code reads and clears it with
// read_error_flags (rq_debug_flag in the C ABI).
__device__ unsigned int g_error_flags;

// The expert of slot j.  An id outside [0, E) breaks the caller's contract: it is reported
// in the error word (report = true in the one kernel that reads every slot first) and mapped
// into [0, E) so that every index the plan produces stays inside the workspace; the rows of
// such slots are then meaningless, but no kernel reads or writes out of bounds.
__device__ __forceinline__ int checked_expert(int e, int E, bool report) {
  if (e < 0 || e >= E) {
    if (report) atomicOr(&g_error_flags, (unsigned)kErrExpertId);
    e = e < 0 ? 0 : E - 1;
  }
  return e;
}

__device__ __forceinline__ int expert_of(const int32_t* ids, int64_t j, int E, bool report) {
  return checked_expert(ids[j], E, report);
}

__global__ __launch_bounds__(kPlanThreads) void plan_hist(const int32_t* __restrict__ ids, int64_t R, int E,
                                                          int32_t* __restrict__ block_hist) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += kPlanThreads) hist[e] = 0;
  __syncthreads();
  const int64_t j = (int64_t)blockIdx.x * kPlanThreads + threadIdx.x;
  if (j < R) atomicAdd(&hist[expert_of(ids, j, E, true)], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kPlanThreads) block_hist[(int64_t)blockIdx.x * E + e] = hist[e];
}

// Exclusive scan of one value per thread across the 1024-thread block.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_sums, int& total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_sums[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = lane < kPlanWaves ? wave_sums[lane] : 0;
    int wi = w;
#pragma unroll
    for (int off = 1; off < kPlanWaves; off <<= 1) {
      const int o = __shfl_up(wi, off, 64);
      if (lane >= off) wi += o;
    }
    if (lane < kPlanWaves) wave_sums[lane] = wi - w;  // exclusive wave prefix
    if (lane == kPlanWaves - 1) wave_sums[kPlanWaves] = wi;
  }
  __syncthreads();
  total = wave_sums[kPlanWaves];
  return wave_sums[wave] + incl - v;
}

// M-tile prefix (tile_start [E + 1]) and table (tile_table, one {expert, first row, end row,
// 0} entry per M-tile) for tiles of tile_m rows.  All lanes call it; lane e < E passes its
// expert's row count; s_off holds every expert's first row, s_tstart is LDS scratch [E + 1].
__device__ void tile_tables(int count, int E, int total_rows, int tile_m, int32_t* __restrict__ tile_start,
                            int32_t* __restrict__ tile_table, int* s_tstart, const int* s_off, int* wave_sums) {
  const int tid = threadIdx.x;
  int total_tiles;
  const int tstart = block_exclusive_scan(tid < E ? (count + tile_m - 1) / tile_m : 0, wave_sums, total_tiles);
  if (tid < E) {
    tile_start[tid] = tstart;
    s_tstart[tid] = tstart;
  }
  if (tid == 0) {
    tile_start[E] = total_tiles;
    s_tstart[E] = total_tiles;
  }
  __syncthreads();
  // the expert of tile t is found by binary search over the tile prefix
  for (int t = tid; t < total_tiles; t += kPlanThreads) {
    int lo = 0, hi = E - 1;  // largest x with s_tstart[x] <= t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tstart[mid] <= t) lo = mid; else hi = mid - 1;
    }
    const int first = s_off[lo] + (t - s_tstart[lo]) * tile_m;
    const int end_e = lo + 1 < E ? s_off[lo + 1] : total_rows;
    int32_t* ent = tile_table + 4 * (int64_t)t;
    ent[0] = lo;
    ent[1] = first;
    ent[2] = first + tile_m < end_e ? first + tile_m : end_e;
    ent[3] = 0;
  }
  __syncthreads();  // s_tstart is reused by the next call
}

// One workgroup turns the [nb][E] block histograms into per-expert offsets and M-tile
// prefixes, the M-tile table, and per-(block, expert) base rows.  The blocks are split into
// G contiguous segments (G groups of E threads, consecutive threads on consecutive experts
// so every load is coalesced): each group sums its segment, the segment sums are scanned
// per expert in LDS, and each group then rewrites its segment with running base rows.
__global__ __launch_bounds__(kPlanThreads) void plan_scan(int32_t* __restrict__ block_hist, int nblocks, int E,
                                                          int32_t* __restrict__ offsets, TileTables tt) {
  __shared__ int wave_sums[kPlanWaves + 1];
  __shared__ int seg[kPlanThreads];        // [G][E] segment sums, then their exclusive scans
  __shared__ int s_tstart[kPlanThreads + 1];
  __shared__ int s_off[kPlanThreads];
  const int tid = threadIdx.x;
  const int groups = kPlanThreads / E;     // E <= 1024
  const int g = tid / E, e = tid % E;
  const bool active = g < groups;
  const int per = (nblocks + groups - 1) / groups;
  const int b0 = active ? g * per : 0;
  const int b1 = active ? min(nblocks, b0 + per) : 0;
  int sum = 0;
  for (int b = b0; b < b1; ++b) sum += block_hist[(int64_t)b * E + e];
  if (active) seg[tid] = sum;
  __syncthreads();
  // per-expert totals and exclusive scan over the segments (thread e walks its column)
  int count = 0;
  if (tid < E) {
    for (int gg = 0; gg < groups; ++gg) {
      const int c = seg[gg * E + tid];
      seg[gg * E + tid] = count;
      count += c;
    }
  }
  __syncthreads();
  int total_rows;
  const int off = block_exclusive_scan(tid < E ? count : 0, wave_sums, total_rows);
  if (tid < E) {
    offsets[tid] = off;
    s_off[tid] = off;
  }
  if (tid == 0) offsets[E] = total_rows;
  __syncthreads();
  // M-tile tables for both tile heights, so a later call may reuse the plan with either
  tile_tables(count, E, total_rows, tt.rows[0], tt.start[0], tt.table[0], s_tstart, s_off, wave_sums);
  tile_tables(count, E, total_rows, tt.rows[1], tt.start[1], tt.table[1], s_tstart, s_off, wave_sums);
  // base row of (block b, expert e) = offset of e + rows of e in earlier blocks
  if (active) {
    int run = s_off[e] + seg[tid];
    for (int b = b0; b < b1; ++b) {
      const int c = block_hist[(int64_t)b * E + e];
      block_hist[(int64_t)b * E + e] = run;
      run += c;
    }
  }
}

__global__ __launch_bounds__(kPlanThreads) void plan_scatter(const int32_t* __restrict__ ids, int64_t R, int E,
                                                             int nbits, const int32_t* __restrict__ block_base,
                                                             int32_t* __restrict__ perm, int32_t* __restrict__ pos) {
  extern __shared__ int32_t wcount[];  // [kPlanWaves][E]
  for (int i = threadIdx.x; i < kPlanWaves * E; i += kPlanThreads) wcount[i] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t j = (int64_t)blockIdx.x * kPlanThreads + threadIdx.x;
  const bool valid = j < R;
  const int e = valid ? expert_of(ids, j, E, false) : 0;
  uint64_t peers = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const uint64_t m = __ballot(((e >> b) & 1) != 0);
    peers &= ((e >> b) & 1) ? m : ~m;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(peers & below);
  if (valid && rank == 0) wcount[wave * E + e] = __popcll(peers);
  __syncthreads();
  for (int x = threadIdx.x; x < E; x += kPlanThreads) {
    int run = 0;
    for (int w = 0; w < kPlanWaves; ++w) {
      const int c = wcount[w * E + x];
      wcount[w * E + x] = run;
      run += c;
    }
  }
  __syncthreads();
  if (valid) {
    const int row = block_base[(int64_t)blockIdx.x * E + e] + wcount[wave * E + e] + rank;
    perm[row] = (int32_t)j;
    pos[j] = row;
  }
}

// The whole plan in one workgroup (one launch instead of three) for up to
// kSinglePlanMaxRows slots and kSinglePlanMaxExperts experts: each thread loads its IPT slot
// ids (slots tid, tid + 1024, ...) into registers at once, so the kernel waits for global
// memory a single time; then the expert histogram (LDS integer atomics), the scans and the
// M-tile table as in plan_scan, and the stable scatter over chunks of 1024 slots taken in slot
// order, each ranked like plan_scatter and placed after the rows of earlier chunks.  The chunks
// are serial and one compute unit issues every scattered store, so the single launch only
// pays for small plans: on MI355X 32768 slots over 32 Zipf-loaded experts take 55 us in one
// workgroup against 17 us in the three kernels, while 1024 slots save two launches.
constexpr int64_t kSinglePlanMaxRows = 8192;
constexpr int64_t kSinglePlanMaxExperts = 256;  // keeps its LDS (19 E + 1 words) under 20 KB

template <int IPT>
__global__ __launch_bounds__(kPlanThreads) void plan_single(const int32_t* __restrict__ ids, int R, int E,
                                                            int nbits, int32_t* __restrict__ offsets, TileTables tt,
                                                            int32_t* __restrict__ perm, int32_t* __restrict__ pos) {
  extern __shared__ int32_t sh[];
  int32_t* base = sh;                  // [E] rows per expert, then the next free row of each expert
  int32_t* s_off = sh + E;             // [E] first row of each expert
  int32_t* s_tstart = sh + 2 * E;      // [E + 1] first M-tile of each expert
  int32_t* wcount = sh + 3 * E + 1;    // [kPlanWaves][E] per-wave counts of a chunk, then their prefix
  __shared__ int wave_sums[kPlanWaves + 1];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int ex[IPT];  // experts of slots tid + 1024 c (0 past R: never used)
#pragma unroll
  for (int c = 0; c < IPT; ++c) {
    const int j = c * kPlanThreads + tid;
    ex[c] = j < R ? ids[j] : 0;
  }
  for (int e = tid; e < E; e += kPlanThreads) base[e] = 0;
  __syncthreads();
#pragma unroll
  for (int c = 0; c < IPT; ++c) {
    const int j = c * kPlanThreads + tid;
    if (j < R) {
      ex[c] = checked_expert(ex[c], E, true);
      atomicAdd(&base[ex[c]], 1);
    }
  }
  __syncthreads();
  // offsets (E <= kPlanThreads: one expert per thread), then the M-tile tables of both heights
  const int count = tid < E ? base[tid] : 0;
  int total_rows;
  const int off = block_exclusive_scan(count, wave_sums, total_rows);
  if (tid < E) {
    offsets[tid] = off;
    s_off[tid] = off;
    base[tid] = off;
  }
  if (tid == 0) offsets[E] = total_rows;
  __syncthreads();
  tile_tables(count, E, total_rows, tt.rows[0], tt.start[0], tt.table[0], s_tstart, s_off, wave_sums);
  tile_tables(count, E, total_rows, tt.rows[1], tt.start[1], tt.table[1], s_tstart, s_off, wave_sums);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int c = 0; c < IPT; ++c) {
    if (c * kPlanThreads >= R) break;  // uniform
    const int j = c * kPlanThreads + tid;
    const bool valid = j < R;
    const int e = ex[c];
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t m = __ballot(((e >> b) & 1) != 0);
      peers &= ((e >> b) & 1) ? m : ~m;
    }
    const int rank = __popcll(peers & below);
    for (int i = tid; i < kPlanWaves * E; i += kPlanThreads) wcount[i] = 0;
    __syncthreads();
    if (valid && rank == 0) wcount[wave * E + e] = __popcll(peers);
    __syncthreads();
    int chunk_rows = 0;
    if (tid < E) {
      for (int w = 0; w < kPlanWaves; ++w) {
        const int n = wcount[w * E + tid];
        wcount[w * E + tid] = chunk_rows;
        chunk_rows += n;
      }
    }
    __syncthreads();
    if (valid) {
      const int row = base[e] + wcount[wave * E + e] + rank;
      perm[row] = j;
      pos[j] = row;
    }
    __syncthreads();
    if (tid < E) base[tid] += chunk_rows;
  }
}

__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y_perm,
                                                      const int32_t* __restrict__ pos,
                                                      const uint16_t* __restrict__ topk_w, int top_k,
                                                      int64_t N, int64_t R, uint16_t* __restrict__ out) {
  const int64_t t = blockIdx.x;
  const int64_t nchunk = N / 8;
  for (int64_t c = threadIdx.x; c < nchunk; c += blockDim.x) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < top_k; ++k) {
      const int64_t slot = t * top_k + k;
      const float w = half_bits_to_float(topk_w[slot]);
      const int64_t row = min(max((int64_t)pos[slot], (int64_t)0), R - 1);  // a reused plan is clamped
      const uint4 v = ld_global_16(y_perm + row * N + 8 * c);
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = acc[2 * i] + w * half_bits_to_float(d[i] & 0xFFFFu);
        acc[2 * i + 1] = acc[2 * i + 1] + w * half_bits_to_float(d[i] >> 16);
      }
    }
    uint4 o;
    o.x = float_to_half_bits(acc[0]) | (float_to_half_bits(acc[1]) << 16);
    o.y = float_to_half_bits(acc[2]) | (float_to_half_bits(acc[3]) << 16);
    o.z = float_to_half_bits(acc[4]) | (float_to_half_bits(acc[5]) << 16);
    o.w = float_to_half_bits(acc[6]) | (float_to_half_bits(acc[7]) << 16);
    st_global_16(out + t * N + 8 * c, o);
  }
}

}  // namespace

int64_t moe_plan_blocks(int64_t R) { return (R + kPlanThreads - 1) / kPlanThreads; }

hipError_t launch_moe_plan(const int32_t* ids, int64_t T, int top_k, int64_t E, int32_t* offsets,
                           const TileTables& tt, int32_t* perm, int32_t* pos, int32_t* block_hist,
                           hipStream_t stream) {
  const int64_t R = T * top_k;
  const int nb = (int)moe_plan_blocks(R);
  const int e = (int)E;
  int nbits = 0;
  while ((1 << nbits) < e) ++nbits;
  if (R <= kSinglePlanMaxRows && E <= kSinglePlanMaxExperts) {
    const size_t lds = (size_t)(3 * e + 1 + kPlanWaves * e) * sizeof(int32_t);
    const dim3 g1(1), blk(kPlanThreads);
    const int r = (int)R, per = (int)((R + kPlanThreads - 1) / kPlanThreads);  // ids per thread
    if (per <= 1) plan_single<1><<<g1, blk, lds, stream>>>(ids, r, e, nbits, offsets, tt, perm, pos);
    else if (per <= 4) plan_single<4><<<g1, blk, lds, stream>>>(ids, r, e, nbits, offsets, tt, perm, pos);
    else plan_single<8><<<g1, blk, lds, stream>>>(ids, r, e, nbits, offsets, tt, perm, pos);
    return hipGetLastError();
  }
  if (nb > 0) {
    plan_hist<<<dim3(nb), dim3(kPlanThreads), e * sizeof(int32_t), stream>>>(ids, R, e, block_hist);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  plan_scan<<<dim3(1), dim3(kPlanThreads), 0, stream>>>(block_hist, nb, e, offsets, tt);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nb == 0) return err;
  plan_scatter<<<dim3(nb), dim3(kPlanThreads), kPlanWaves * e * sizeof(int32_t), stream>>>(
      ids, R, e, nbits, block_hist, perm, pos);
  return hipGetLastError();
}

hipError_t read_error_flags(unsigned int* flags, bool clear) {
  hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) return e;
  e = hipMemcpyFromSymbol(flags, HIP_SYMBOL(g_error_flags), sizeof(unsigned int), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess || !clear) return e;
  const unsigned int zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(g_error_flags), &zero, sizeof(unsigned int), 0, hipMemcpyHostToDevice);
}

hipError_t launch_moe_combine(const uint16_t* y_perm, const int32_t* pos, const uint16_t* topk_w,
                              int64_t T, int top_k, int64_t N, uint16_t* out, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  combine_kernel<<<dim3((unsigned)T), dim3(256), 0, stream>>>(y_perm, pos, topk_w, top_k, N, T * top_k, out);
  return hipGetLastError();
}

}  // namespace rq
