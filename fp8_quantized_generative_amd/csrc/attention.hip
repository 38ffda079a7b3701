// Short-context attention core for gfx950 (FP16 in, FP16 out), between the QKV and O linears.
//
// Page "FP8量化在生成式推荐系统OneRec-V2中的优化实践", §3.2: serving contexts are short (tens
// of positions per request); the attention core is not quantized (page "Quantized Inference
// for OneRec-V2：生成式推荐开始直接吃 LLM 量化栈", section 关键证据, quantizes only the linears).
// Per request of L <= 32 consecutive token rows and per head of D = 128 columns of the QKV
// output row [q | k | v]:
//   s[i][j] = q_i . k_j / sqrt(D)  for j <= i (causal), -inf otherwise
//   p[i][j] = softmax_j(s[i][j])     in FP32
//   o_i     = sum_j fl16(p[i][j]) v_j  with FP32 accumulation, rounded to FP16
//
// One wavefront per (request, head), four per workgroup.  Scores: v_mfma_f32_32x32x16_f16
// with the keys as first operand and the queries as second, so lane l ends with query l & 31
// and 16 keys (register r: key 8 (r / 4) + 4 (l / 32) + r % 4; the partner lane l ^ 32 holds
// the other 16) - the row softmax needs one cross-half exchange.  Operands are read straight
// from the QKV rows: lane l reads 64 contiguous bytes of row l & 31 per 64-wide slice of the
// head, the same K assignment for both.  The probabilities, rounded to FP16, are already laid
// out as the second operand of the output product o^T = v^T p^T: MFMA m (keys 16 m ..) takes
// registers 8 m .. 8 m + 7.  v is staged through LDS transposed ([dim][key]) so each lane
// reads its 8 keys of one dimension as two 8-byte reads; the output tile comes out with a
// lane per query and 4 consecutive dimensions per register group, stored as 8-byte writes.

#include "common.h"

namespace rq {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kHeadDim = 128;
constexpr int kMaxLen = 32;
constexpr int kWaves = 4;

__device__ __forceinline__ h8 as_h8(uint4 v) { return __builtin_bit_cast(h8, v); }

__global__ __launch_bounds__(64 * kWaves) void attention_core_kernel(const uint16_t* __restrict__ qkv,
                                                                     int64_t requests, int L, int heads,
                                                                     uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) _Float16 vt_all[kWaves][kHeadDim][kMaxLen];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t pair = (int64_t)blockIdx.x * kWaves + wave;  // (request, head)
  const bool active = pair < requests * heads;
  const int64_t req = active ? pair / heads : 0;
  const int head = active ? (int)(pair % heads) : 0;
  const int hidden = heads * kHeadDim;
  const int64_t stride = 3 * (int64_t)hidden;
  const int pos = lane & 31, half = lane >> 5;
  // rows past the request's L read its first row (valid memory); those keys are masked and
  // those queries never stored
  const uint16_t* row = qkv + (req * L + (pos < L ? pos : 0)) * stride + (int64_t)head * kHeadDim;
  _Float16 (*vt)[kMaxLen] = vt_all[wave];

  // ---- scores: D = 128 in two 64-wide slices, four MFMAs each
  v16f s = {};
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    uint4 qa[4], ka[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qa[j] = ld_global_16(row + 64 * g + 32 * half + 8 * j);
      ka[j] = ld_global_16(row + hidden + 64 * g + 32 * half + 8 * j);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) s = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(ka[j]), as_h8(qa[j]), s, 0, 0, 0);
  }
  // ---- v into LDS, transposed: lane (key pos, half) holds dims 64 half .. 64 half + 63
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const h8 v = as_h8(ld_global_16(row + 2 * hidden + 64 * half + 8 * j));
#pragma unroll
    for (int e = 0; e < 8; ++e) vt[64 * half + 8 * j + e][pos] = v[e];
  }

  // ---- causal softmax of query pos over keys 8 (r / 4) + 4 half + r % 4
  const float scale = 0.08838834764831845f;  // fl32(1 / sqrt(128))
  float m = -__builtin_inff();
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = 8 * (r / 4) + 4 * half + r % 4;
    s[r] = (key <= pos && key < L) ? s[r] * scale : -__builtin_inff();
    m = __builtin_fmaxf(m, s[r]);
  }
  m = __builtin_fmaxf(m, __builtin_bit_cast(float, __shfl_xor(__builtin_bit_cast(int, m), 32, 64)));
  float sum = 0.0f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s[r] = __expf(s[r] - m);  // exp(-inf) = 0 for masked keys
    sum += s[r];
  }
  sum += __builtin_bit_cast(float, __shfl_xor(__builtin_bit_cast(int, sum), 32, 64));
  h8 p[2];
#pragma unroll
  for (int r = 0; r < 16; ++r) p[r / 8][r % 8] = (_Float16)__fdiv_rn(s[r], sum);

  __syncthreads();  // every wave's v^T is in LDS

  // ---- o^T = v^T p^T: dims 32 c .. 32 c + 31, keys in two chunks of 16.  Every lane takes
  // part (lane l supplies dimension row l & 31 of v^T and query column l & 31 of p^T to the
  // whole wavefront's product); only the stores are limited to the request's L queries.
  if (!active) return;  // the whole wavefront
  const bool store = pos < L;
  uint16_t* orow = out + (req * L + (store ? pos : 0)) * (int64_t)hidden + (int64_t)head * kHeadDim;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    v16f o = {};
#pragma unroll
    for (int mk = 0; mk < 2; ++mk) {
      const _Float16* vr = &vt[32 * c + pos][16 * mk + 4 * half];
      const h4 lo = *reinterpret_cast<const h4*>(vr);
      const h4 hi = *reinterpret_cast<const h4*>(vr + 8);
      const h8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      o = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, p[mk], o, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const h4 v = {(_Float16)o[4 * q], (_Float16)o[4 * q + 1], (_Float16)o[4 * q + 2], (_Float16)o[4 * q + 3]};
      if (store) *reinterpret_cast<h4*>(orow + 32 * c + 8 * q + 4 * half) = v;
    }
  }
}

}  // namespace

int attention_head_dim() { return kHeadDim; }
int attention_max_len() { return kMaxLen; }

hipError_t launch_attention_core(const uint16_t* qkv, int64_t requests, int length, int heads, uint16_t* out,
                                 hipStream_t stream) {
  const int64_t pairs = requests * heads;
  if (pairs <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((pairs + kWaves - 1) / kWaves);
  attention_core_kernel<<<dim3(blocks), dim3(64 * kWaves), 0, stream>>>(qkv, requests, length, heads, out);
  return hipGetLastError();
}

}  // namespace rq
