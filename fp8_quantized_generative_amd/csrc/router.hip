// MoE router for gfx950: FP16 gate logits and top-k expert selection.
//
// Page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §2.1, keeps the routing gate in FP16
// (outside the FP8 path); its top-k result feeds the MoE grouped GEMM.  Per token row x [K]
// and gate weights W [E][K] (both FP16):
//   logit[e] = sum_k x[k] * W[e][k]     FP16 products (exact in FP32), FP32 accumulation
//   ids      = the top_k experts by logit, larger first, equal logits to the lower index
//   weights  = fl16(softmax of the selected logits), computed in FP32
//
// Design: the logits are a [T x K] x [K x E] product with E <= 32, so one wavefront owns 32
// tokens x 32 experts and accumulates them with v_mfma_f32_32x32x16_f16 (K = 16 per
// instruction).  The gate weights are the instruction's first operand and the tokens its
// second, so lane l ends with token l & 31 and 16 of the 32 experts (register r: expert
// 8 (r / 4) + 4 (l / 32) + r % 4); lanes l and l ^ 32 hold the two halves.  K advances in
// groups of 64: lane l reads 64 contiguous bytes (32 values) of token row l & 31 and of gate
// row l & 31 at K offset 64 g + 32 (l / 32), and the group's four MFMAs take 8 values each
// from them - the same K assignment for both operands, so the sums are the plain ones, and
// every load is a full 16-byte vector.  The K groups of a 32-token tile are split over the
// four wavefronts of a workgroup (so a 16384-token batch keeps 2048 wavefronts streaming);
// each runs its loads three groups ahead of its MFMAs, and the four partial tiles meet in LDS,
// summed in wavefront order (deterministic).  Wavefront 0 then selects: an insertion into a
// per-lane sorted list of top_k, then a merge with the partner lane's list across the 32-lane
// halves.

#include <type_traits>

#include "common.h"

namespace rq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
constexpr int kMaxTopK = 4;
constexpr int kGroupAhead = 3;
constexpr int kSplit = 4;  // wavefronts per 32-token tile, each a quarter of the K groups

__device__ __forceinline__ h8 as_h8(uint4 v) { return __builtin_bit_cast(h8, v); }

// (logit, expert) order: larger logit first, equal logits to the lower expert.
__device__ __forceinline__ bool before(float a, int ia, float b, int ib) { return a > b || (a == b && ia < ib); }

template <int TOPK>
__device__ __forceinline__ void insert(float (&v)[TOPK], int (&id)[TOPK], float x, int ix) {
#pragma unroll
  for (int i = 0; i < TOPK; ++i) {
    if (before(x, ix, v[i], id[i])) {
      const float tv = v[i];
      const int ti = id[i];
      v[i] = x;
      id[i] = ix;
      x = tv;
      ix = ti;
    }
  }
}

template <int TOPK>
__global__ __launch_bounds__(64 * kSplit) void router_topk_kernel(const uint16_t* __restrict__ x, int64_t T, int K,
                                                                  const uint16_t* __restrict__ w, int E,
                                                                  int32_t* __restrict__ ids,
                                                                  uint16_t* __restrict__ topk_w,
                                                                  float* __restrict__ logits) {
  __shared__ float part[kSplit - 1][16][64];  // partial tiles of waves 1..3, register-major
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r32 = lane & 31, half = lane >> 5;
  const int64_t t0 = (int64_t)blockIdx.x * 32;
  const int64_t tok = t0 + r32;
  // rows past T or E read row 0 (valid memory); their results are never used
  const uint16_t* xr = x + (tok < T ? tok : 0) * (int64_t)K + 32 * half;
  const uint16_t* wr = w + (int64_t)(r32 < E ? r32 : 0) * K + 32 * half;
  const int groups = K / 64;
  const int g_begin = groups * wave / kSplit, g_end = groups * (wave + 1) / kSplit;

  v16f acc = {};
  // a ring of kGroupAhead + 1 register slots; every slot index is a compile-time constant
  // (a run-time index would put the ring in scratch memory)
  uint4 xa[kGroupAhead + 1][4], wa[kGroupAhead + 1][4];
  auto load = [&](auto slot_c, int g) {
    constexpr int kSlot = decltype(slot_c)::value;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      xa[kSlot][j] = ld_global_16(xr + 64 * g + 8 * j);
      wa[kSlot][j] = ld_global_16(wr + 64 * g + 8 * j);
    }
  };
  auto stage = [&](auto slot_c, int g) {  // group g in slot kSlot; fetch group g + kGroupAhead
    constexpr int kSlot = decltype(slot_c)::value;
    if (g + kGroupAhead < g_end) load(std::integral_constant<int, (kSlot + kGroupAhead) % (kGroupAhead + 1)>{},
                                      g + kGroupAhead);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(wa[kSlot][j]), as_h8(xa[kSlot][j]), acc, 0, 0, 0);
  };
  static_assert(kGroupAhead == 3, "the loop below is unrolled for a ring of four slots");
  if (g_begin < g_end) load(std::integral_constant<int, 0>{}, g_begin);
  if (g_begin + 1 < g_end) load(std::integral_constant<int, 1>{}, g_begin + 1);
  if (g_begin + 2 < g_end) load(std::integral_constant<int, 2>{}, g_begin + 2);
  for (int g = g_begin; g < g_end; g += 4) {
    stage(std::integral_constant<int, 0>{}, g);
    if (g + 1 < g_end) stage(std::integral_constant<int, 1>{}, g + 1);
    if (g + 2 < g_end) stage(std::integral_constant<int, 2>{}, g + 2);
    if (g + 3 < g_end) stage(std::integral_constant<int, 3>{}, g + 3);
  }
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) part[wave - 1][r][lane] = acc[r];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int q = 0; q < kSplit - 1; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] += part[q][r][lane];

  // register r holds expert 8 (r / 4) + 4 half + r % 4 of token tok
  if (logits != nullptr && tok < T) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e0 = 8 * q + 4 * half;
      if ((E & 3) == 0 && e0 + 3 < E) {  // 16-byte aligned when E is a multiple of 4
        *reinterpret_cast<float4*>(logits + tok * E + e0) = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2],
                                                                        acc[4 * q + 3]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (e0 + i < E) logits[tok * E + e0 + i] = acc[4 * q + i];
      }
    }
  }
  float v[TOPK];
  int id[TOPK];
#pragma unroll
  for (int i = 0; i < TOPK; ++i) {
    v[i] = -__builtin_inff();
    id[i] = 1 << 30;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int e = 8 * (r / 4) + 4 * half + r % 4;
    if (e < E) insert(v, id, acc[r], e);
  }
  // merge with the partner lane's list (the other 16 experts of the same token)
  float pv[TOPK];
  int pid[TOPK];
#pragma unroll
  for (int i = 0; i < TOPK; ++i) {
    pv[i] = __builtin_bit_cast(float, __shfl_xor(__builtin_bit_cast(int, v[i]), 32, 64));
    pid[i] = __shfl_xor(id[i], 32, 64);
  }
#pragma unroll
  for (int i = 0; i < TOPK; ++i) insert(v, id, pv[i], pid[i]);
  if (half != 0 || tok >= T) return;
  float z[TOPK], sum = 0.0f;
#pragma unroll
  for (int i = 0; i < TOPK; ++i) {
    z[i] = __expf(v[i] - v[0]);
    sum += z[i];
  }
#pragma unroll
  for (int i = 0; i < TOPK; ++i) {
    ids[tok * TOPK + i] = id[i];
    topk_w[tok * TOPK + i] = (uint16_t)float_to_half_bits(__fdiv_rn(z[i], sum));
  }
}

template <int TOPK>
hipError_t launch(const uint16_t* x, int64_t T, int64_t K, const uint16_t* w, int E, int32_t* ids, uint16_t* tw,
                  float* logits, hipStream_t stream) {
  const unsigned blocks = (unsigned)((T + 31) / 32);
  router_topk_kernel<TOPK><<<dim3(blocks), dim3(64 * kSplit), 0, stream>>>(x, T, (int)K, w, E, ids, tw, logits);
  return hipGetLastError();
}

}  // namespace

int router_max_topk() { return kMaxTopK; }

hipError_t launch_router_topk(const uint16_t* x, int64_t T, int64_t K, const uint16_t* w, int64_t E, int top_k,
                              int32_t* ids, uint16_t* topk_w, float* logits, hipStream_t stream) {
  if (T <= 0) return hipSuccess;
  switch (top_k) {
    case 1: return launch<1>(x, T, K, w, (int)E, ids, topk_w, logits, stream);
    case 2: return launch<2>(x, T, K, w, (int)E, ids, topk_w, logits, stream);
    case 3: return launch<3>(x, T, K, w, (int)E, ids, topk_w, logits, stream);
    default: return launch<4>(x, T, K, w, (int)E, ids, topk_w, logits, stream);
  }
}

}  // namespace rq
