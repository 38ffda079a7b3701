// Batched top-k over FP16 candidate rows (beam search) for gfx950: a radix select.
//
// Page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §3.2, replaces the default TopK with a
// RadixSelect kernel run batched with zero copies; its §5.3 keeps TopK results in FP16.  Here:
// for each row of n FP16 scores, the k candidates ranked first by score (larger first, in
// the IEEE total order: -0 below +0), equal scores ranking the lower index first; their
// int32 indices and FP16 scores in rank order.
//
// Keys: an FP16 bit pattern b maps to the 16-bit key (b & 0x8000) ? ~b : b | 0x8000, whose
// unsigned order is the score order, so selecting by score is selecting by key.
//
// One workgroup (1024 lanes) selects the k best of one segment held in LDS:
//   1. histogram of the key's high byte (per-wavefront LDS histograms, then summed), and the
//      bin holding the k-th best key;
//   2. histogram of the low byte among keys with that high byte: the k-th best key T and the
//      number of keys above it, so the k - above keys equal to T with the lowest positions
//      complete the selection;
//   3. compaction in segment order: each lane holds a contiguous run of the segment in
//      registers, so one workgroup scan of the lanes' counts places keys above T, then the
//      first k - above keys equal to T;
//   4. each pick's rank among the picks by (key descending, index ascending) - a count over
//      the picks in LDS, no barrier per step - and the output written in rank order.
// Rows longer than one segment run in stages (a segment's top k holds every member of the
// row's top k that lies in it): stage 0 reads FP16 scores in segments of 16384 and writes
// each segment's k best as (key, index) pairs in rank order; later stages take segments of
// 8192 pairs of that list until one segment covers the row.  Equal keys keep their index
// order through the list (segments in index order, each in rank order), so "lowest position
// first" in a later stage is "lowest index first".  Segments shorter than k (the row's tail)
// pad their output with a key below every real one, which is never selected since a row
// holds at least k real candidates.

#include <climits>

#include "common.h"

namespace rq {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kSegScores = 16384;  // FP16 scores per stage-0 segment (32 KB of keys)
constexpr int kSegPairs = 8192;    // (key, index) pairs per later-stage segment
constexpr int kMaxTopK = 1024;
constexpr uint32_t kPadKey = 0;    // below every key of a non-NaN FP16 value (those are >= 0x3FF)

__device__ __forceinline__ uint32_t key_of(uint32_t b) { return (b & 0x8000u) ? (~b & 0xFFFFu) : (b | 0x8000u); }
__device__ __forceinline__ uint32_t bits_of(uint32_t key) { return (key & 0x8000u) ? (key & 0x7FFFu) : (~key & 0xFFFFu); }

// Among 256 bins of per-wavefront counts (hist[w][b], bins 255..0 = best first), the bin
// holding the need-th best key and the count of keys in better bins, written to res[0],
// res[1].  Lane t < 256 sums bin 255 - t over the wavefronts itself.  All lanes call it.
__device__ void find_bin(const int (*hist)[256], int need, int* res, int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int c = 0, incl = 0;
  if (tid < 256) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) c += hist[w][255 - tid];
    incl = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) wsum[wave] = incl;
  }
  __syncthreads();
  if (tid < 256) {
    for (int w = 0; w < wave; ++w) incl += wsum[w];
    const int excl = incl - c;
    if (excl < need && need <= incl) {
      res[0] = 255 - tid;
      res[1] = excl;
    }
  }
  __syncthreads();
}

// Exclusive prefix of v over the workgroup in lane order, and the total (wsum: kWaves ints).
__device__ __forceinline__ int block_scan(int v, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int t = wsum[w];
    before += w < wave ? t : 0;
    total += t;
  }
  __syncthreads();
  return before + incl - v;
}

// One segment of one row.  PAIRS = false: in = FP16 scores [rows][n], segments of kSegScores
// and an index is the position in the row; PAIRS = true: in = pairs [rows][n] (int2 {key,
// index}), segments of kSegPairs.  Lane t holds the segment's elements [E t, E t + E) in
// registers, so lane order is segment order.  FINAL: write idx / vals (one segment per row),
// else k pairs per segment, in rank order, to out_pairs [rows][segments][k].
template <bool PAIRS, bool FINAL>
__global__ __launch_bounds__(kThreads) void topk_segment(const void* __restrict__ in, int64_t n, int k,
                                                         int2* __restrict__ out_pairs, int32_t* __restrict__ out_idx,
                                                         uint16_t* __restrict__ out_vals) {
  constexpr int SEG = PAIRS ? kSegPairs : kSegScores;
  constexpr int E = SEG / kThreads;  // elements per lane: 8 pairs or 16 scores
  __shared__ int hist[kWaves][256];   // high-byte counts per wavefront
  __shared__ int hist2[kWaves][256];  // low-byte counts per wavefront
  __shared__ unsigned long long sel[kMaxTopK];
  __shared__ int wsum[kWaves];
  __shared__ int res[2];
  const int tid = threadIdx.x, wave = tid >> 6;
  const int64_t row = blockIdx.y;
  const int64_t seg0 = (int64_t)blockIdx.x * SEG;
  const int len = (int)(n - seg0 < SEG ? n - seg0 : SEG);  // > 0
  const int need = len < k ? len : k;
  const int first = E * tid;  // this lane's first element in the segment

  // ---- the lane's keys (kPadKey past the segment's end: below every real key, never counted)
  uint32_t key[E];
  int32_t id[E];
  if constexpr (PAIRS) {
    const int2* src = reinterpret_cast<const int2*>(in) + row * n + seg0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int2 p = first + j < len ? src[first + j] : make_int2((int)kPadKey, INT_MAX);
      key[j] = (uint32_t)p.x;
      id[j] = p.y;
    }
  } else {
    const uint16_t* src = reinterpret_cast<const uint16_t*>(in) + row * n + seg0;
    if ((n & 7) == 0 && first + E <= len) {  // 16-byte aligned rows: two 16-byte loads
      const uint4 a = *reinterpret_cast<const uint4*>(src + first);
      const uint4 b = *reinterpret_cast<const uint4*>(src + first + 8);
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        key[2 * q] = key_of(w[q] & 0xFFFFu);
        key[2 * q + 1] = key_of(w[q] >> 16);
      }
    } else {
#pragma unroll
      for (int j = 0; j < E; ++j) key[j] = first + j < len ? key_of(src[first + j]) : kPadKey;
    }
#pragma unroll
    for (int j = 0; j < E; ++j) id[j] = (int32_t)(seg0 + first + j);
  }
  for (int i = tid; i < kWaves * 256; i += kThreads) {
    (&hist[0][0])[i] = 0;
    (&hist2[0][0])[i] = 0;
  }
  __syncthreads();

  // ---- pass 1: histogram of the high byte (pad keys excluded)
#pragma unroll
  for (int j = 0; j < E; ++j)
    if (first + j < len) atomicAdd(&hist[wave][key[j] >> 8], 1);
  __syncthreads();
  find_bin(hist, need, res, wsum);
  const uint32_t hi = (uint32_t)res[0];
  const int above_hi = res[1];
  // ---- pass 2: histogram of the low byte among keys with that high byte
#pragma unroll
  for (int j = 0; j < E; ++j)
    if (first + j < len && (key[j] >> 8) == hi) atomicAdd(&hist2[wave][key[j] & 0xFF], 1);
  __syncthreads();
  find_bin(hist2, need - above_hi, res, wsum);
  const uint32_t T = (hi << 8) | (uint32_t)res[0];
  const int n_gt = above_hi + res[1];  // keys above T
  const int take_eq = need - n_gt;     // keys equal to T taken, lowest positions first

  // ---- pass 3: compaction in segment order: one scan of the lane's counts (above T in the
  // high 16 bits, equal to T in the low; a segment has at most 16384 of each)
  int c_gt = 0, c_eq = 0;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const bool ok = first + j < len;
    c_gt += ok && key[j] > T;
    c_eq += ok && key[j] == T;
  }
  int total;
  const int pre = block_scan((c_gt << 16) | c_eq, wsum, total);
  int g = pre >> 16, e = pre & 0xFFFF;
#pragma unroll
  for (int j = 0; j < E; ++j) {
    if (first + j >= len) continue;
    const unsigned long long comp = ((unsigned long long)key[j] << 32) | (0xFFFFFFFFu - (uint32_t)id[j]);
    if (key[j] > T) {
      if (g < need) sel[g] = comp;  // always: g < n_gt
      ++g;
    } else if (key[j] == T) {
      if (e < take_eq) sel[n_gt + e] = comp;
      ++e;
    }
  }
  __syncthreads();

  // ---- pass 4: rank of each pick among the need picks (key descending, index ascending;
  // equal entries - only pads can repeat - by position), then the output in rank order
  if (tid < need) {
    const unsigned long long c = sel[tid];
    int rank = 0;
    int u = 0;
    for (; u + 8 <= need; u += 8) {  // eight LDS reads in flight per step
      unsigned long long o[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) o[q] = sel[u + q];
#pragma unroll
      for (int q = 0; q < 8; ++q) rank += (o[q] > c) || (o[q] == c && u + q < tid);
    }
    for (; u < need; ++u) {
      const unsigned long long o = sel[u];
      rank += (o > c) || (o == c && u < tid);
    }
    const uint32_t kk = (uint32_t)(c >> 32);
    const int32_t idx = (int32_t)(0xFFFFFFFFu - (uint32_t)c);
    if constexpr (FINAL) {
      out_idx[row * k + rank] = idx;
      out_vals[row * k + rank] = (uint16_t)bits_of(kk);
    } else {
      out_pairs[(row * gridDim.x + blockIdx.x) * k + rank] = make_int2((int)kk, idx);
    }
  }
  if constexpr (!FINAL) {  // a segment shorter than k pads its list
    for (int i = need + tid; i < k; i += kThreads)
      out_pairs[(row * gridDim.x + blockIdx.x) * k + i] = make_int2((int)kPadKey, INT_MAX);
  }
}

int64_t segments(int64_t len, int seg) { return (len + seg - 1) / seg; }

}  // namespace

int topk_max_k() { return kMaxTopK; }

// Pairs of the largest intermediate list, per buffer (two buffers alternate between stages).
int64_t topk_pairs_per_buffer(int64_t rows, int64_t n, int k) {
  if (segments(n, kSegScores) <= 1) return 0;
  return rows * segments(n, kSegScores) * k;
}

hipError_t launch_topk(const uint16_t* scores, int64_t rows, int64_t n, int k, int32_t* idx, uint16_t* vals,
                       int2* buf0, int2* buf1, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const dim3 block(kThreads);
  int64_t nseg = segments(n, kSegScores);
  if (nseg == 1) {
    topk_segment<false, true><<<dim3(1, (unsigned)rows), block, 0, stream>>>(scores, n, k, nullptr, idx, vals);
    return hipGetLastError();
  }
  topk_segment<false, false><<<dim3((unsigned)nseg, (unsigned)rows), block, 0, stream>>>(scores, n, k, buf0, nullptr,
                                                                                          nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t len = nseg * k;  // pairs per row
  int2* cur = buf0;
  int2* nxt = buf1;
  while (true) {
    nseg = segments(len, kSegPairs);
    if (nseg == 1) {
      topk_segment<true, true><<<dim3(1, (unsigned)rows), block, 0, stream>>>(cur, len, k, nullptr, idx, vals);
      return hipGetLastError();
    }
    topk_segment<true, false><<<dim3((unsigned)nseg, (unsigned)rows), block, 0, stream>>>(cur, len, k, nxt, nullptr,
                                                                                           nullptr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    len = nseg * k;
    int2* t = cur;
    cur = nxt;
    nxt = t;
  }
}

}  // namespace rq
