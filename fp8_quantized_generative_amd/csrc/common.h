// Internal helpers of the gfx950 W8A8 FP8 library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace rq {

// Packed vector types.
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr float kFp8Max = 448.0f;        // largest finite OCP E4M3 magnitude
constexpr float kScaleFloor = 0x1p-24f;  // smallest positive FP16: floor of a row's amax

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
}

__device__ __forceinline__ uint32_t float_to_half_bits(float f) {
  return (uint32_t)__builtin_bit_cast(unsigned short, (_Float16)f);  // round to nearest even
}

// Two FP32 values rounded to FP16 (nearest even), packed low then high: one
// v_cvt_pk_f16_f32.  The empty asm makes the inputs plain FP32 values, so the compiler cannot
// fuse the multiply that produced them into a single-rounding multiply-to-FP16.
typedef float f2v __attribute__((ext_vector_type(2)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
  f2v v = {lo, hi};
  asm("" : "+v"(v));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2v));
}

// p = fl32(fl32(silu(g)) * u) for the FP16 halves (low: HI = 0, high: HI = 1) of g2 and u2,
// with silu(g) = fl32(g * rcp(1 + exp2(fl32(g * -log2 e)))) through the hardware exp2 and
// reciprocal (about one FP32 ulp each; the correctly rounded division would cost ten
// instructions per value).  Each multiply that takes an FP16 operand is a v_fma_mix_f32 with
// an addend of -0: the FP16 value widens exactly, a * b + (-0) is a * b under every rounding
// (also for a zero product of either sign), so the result equals the FP32 multiply of the
// widened value, without the separate widening instruction.  One asm block, so the wait
// state that each transcendental result needs before its next use is explicit.
template <int HI>
__device__ __forceinline__ float silu_mul_half(uint32_t g2, uint32_t u2) {
  constexpr float kNegLog2e = -1.44269502162933349609375f;  // fl32(-log2 e)
  float p, t;
  if constexpr (HI) {
    asm("v_fma_mix_f32 %1, %2, %4, neg(0) op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
        "v_exp_f32 %1, %1\n\t"
        "s_nop 0\n\t"
        "v_add_f32 %1, 1.0, %1\n\t"
        "v_rcp_f32 %1, %1\n\t"
        "s_nop 0\n\t"
        "v_fma_mix_f32 %1, %2, %1, neg(0) op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
        "v_fma_mix_f32 %0, %3, %1, neg(0) op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=v"(p), "=&v"(t)
        : "v"(g2), "v"(u2), "s"(kNegLog2e));
  } else {
    asm("v_fma_mix_f32 %1, %2, %4, neg(0) op_sel_hi:[1,0,0]\n\t"
        "v_exp_f32 %1, %1\n\t"
        "s_nop 0\n\t"
        "v_add_f32 %1, 1.0, %1\n\t"
        "v_rcp_f32 %1, %1\n\t"
        "s_nop 0\n\t"
        "v_fma_mix_f32 %1, %2, %1, neg(0) op_sel_hi:[1,0,0]\n\t"
        "v_fma_mix_f32 %0, %3, %1, neg(0) op_sel_hi:[1,0,0]"
        : "=v"(p), "=&v"(t)
        : "v"(g2), "v"(u2), "s"(kNegLog2e));
  }
  return p;
}

// h = fl16(fl32(silu(g) * u)) for two packed FP16 pairs (the product above, rounded once to
// FP16).  The quantizer's SiLU*up input transform and the GEMM's gated output both use this
// one definition, so the two FFN formulations give identical h.
__device__ __forceinline__ uint32_t silu_mul_pair(uint32_t g2, uint32_t u2) {
  return pack_half2(silu_mul_half<0>(g2, u2), silu_mul_half<1>(g2, u2));
}

__device__ __forceinline__ uint4 ld_global_16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ void st_global_16(void* p, uint4 v) {
  *reinterpret_cast<uint4*>(p) = v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    uint32_t o = (uint32_t)__shfl_xor((int)v, off, 64);
    v = v > o ? v : o;
  }
  return v;
}

// Launch helpers ---------------------------------------------------------------------

// Quantize `rows` FP16 rows (act: 0 none, 1 SiLU*up).  With pos == nullptr row t goes to
// output row t; otherwise to output rows pos[t * fanout + k], k < fanout (a token's copies
// in the permuted MoE order).  h (SiLU only, may be null) receives the FP16 SiLU*up rows.
// Activation formats (the values of the C ABI's RQ_FP8_*): OCP E4M3, or OCP E5M2.
enum { kFmtE4M3 = 0, kFmtE5M2 = 1 };

hipError_t launch_quant_rows(const uint16_t* x, int64_t rows, int64_t K, int act,
                             uint8_t* q, float* scale, uint16_t* h, const int32_t* pos, int fanout,
                             hipStream_t stream, int fmt = kFmtE4M3);

// Weight-scale granularities (the values of the C ABI's RQ_WSCALE_*): one FP32 scale per
// output channel ([E][N]), per tensor ([E]) or per 128 x 128 block ([E][N/128][K/128]).
enum { kScaleChannel = 0, kScaleTensor = 1, kScaleBlock128 = 2 };
constexpr int kScaleBlock = 128;

// Offline weight quantization at tensor or block granularity: B matrices [N][K] -> E4M3
// bytes and B scales (tensor) or B * N/128 * K/128 scales (block; N, K multiples of 128).
hipError_t launch_quant_tensor(const uint16_t* w, int64_t B, int64_t N, int64_t K, uint8_t* q, float* scale,
                               hipStream_t stream);
hipError_t launch_quant_blocks(const uint16_t* w, int64_t B, int64_t N, int64_t K, uint8_t* q, float* scale,
                               hipStream_t stream);
// w_q [B][N][K] bytes -> the slab layout [B][K/64][N][64] (K a multiple of 64).
hipError_t launch_pack_slabs(const uint8_t* w_q, int64_t B, int64_t N, int64_t K, uint8_t* w_packed,
                             hipStream_t stream);

struct GemmArgs {
  const uint8_t* a;       // [a_rows][K] E4M3 (token rows, or permuted rows in grouped mode)
  const float* a_scale;   // [a_rows]
  const uint8_t* b;       // [E][N][K] E4M3 (E = 1 for a dense linear)
  const float* b_scale;   // [E][N]
  uint16_t* y;            // [a_rows][N] FP16
  int32_t M;              // dense: rows of A and y.  grouped: R (routed rows)
  int32_t a_rows;         // rows of the A array (M, or R)
  int32_t N;
  int32_t K;
  // grouped only
  const int32_t* tile_start;  // [E+1] first m-tile of each expert (exclusive scan); [E] = total
  const int32_t* tile_table;  // [m-tiles][4] {expert, first row, end row, 0}
  int32_t E;
  int32_t gate;               // 1: gated SiLU output (see rq_fp8.h, RQ_ACT_GATE_SILU), y is [rows][N/2]
  int32_t b_gran;             // kScaleChannel, kScaleTensor or kScaleBlock128 (layout of b_scale)
  int32_t a_fmt;              // kFmtE4M3 or kFmtE5M2 (the bytes of a)
  // split-K (dense only): the K range is cut into `splits` equal parts; part s of every tile
  // writes its FP32 sum to partial [splits][M][N] and a reduce kernel adds the parts in order
  // and applies the epilogue
  int32_t splits;             // 1: no split
  float* partial;
  // weight byte layout: 0 rows ([E][N][K]); 1 slabs ([E][K/64][N][64], see
  // rq_fp8_pack_weights; K a multiple of 64): the 64-byte K slab of every weight row stored
  // together, so that a GEMM tile's slab is one contiguous run of BN * 64 bytes
  int32_t b_slabs;
};

// GEMM tile shapes (rows x columns of output per workgroup).
enum { kTileBig = 0, kTileWide, kTileSmall, kTileThin, kTileThinWide, kTileMid, kTileKinds };
constexpr int kMinTileRows = 64;  // fewest rows of any tile shape (sizes the MoE tile table)

hipError_t launch_gemm_dense(const GemmArgs& g, hipStream_t stream);
// K parts of a dense M x N x K GEMM (1 = no split) and the FP32 partial-sum bytes they need.
int dense_splits(int64_t M, int64_t N, int64_t K, int act, int w_gran);
size_t dense_partial_bytes(int64_t M, int64_t N, int64_t K, int act, int w_gran);
hipError_t launch_gemm_grouped(const GemmArgs& g, int kind, hipStream_t stream);
int pick_grouped(int64_t R, int64_t E, int64_t N, bool gate);  // tile shape for R routed rows over E experts
int tile_rows(int kind);                       // M rows of a tile shape
int64_t grouped_max_mtiles(int64_t R, int64_t E, int tile_m);

// The M-tile prefix and table of a routing plan for two tile heights (the 64- and the
// 256-row tiles of the grouped GEMM), so a later call may reuse the plan with either.
struct TileTables {
  int rows[2];
  int32_t* start[2];  // [E + 1]
  int32_t* table[2];  // [grouped_max_mtiles(R, E, rows)][4]
};

hipError_t launch_moe_plan(const int32_t* ids, int64_t T, int top_k, int64_t E, int32_t* offsets,
                           const TileTables& tt, int32_t* perm, int32_t* pos, int32_t* block_hist,
                           hipStream_t stream);
int64_t moe_plan_blocks(int64_t R);

// MoE router: FP16 logits of T rows x [K] against E <= 32 gate rows, top_k <= router_max_topk()
// ids and FP16 weights per row, optional FP32 logits [T][E].  K a multiple of 64.
hipError_t launch_router_topk(const uint16_t* x, int64_t T, int64_t K, const uint16_t* w, int64_t E, int top_k,
                              int32_t* ids, uint16_t* topk_w, float* logits, hipStream_t stream);
int router_max_topk();

// Short-context attention core: requests of `length` <= attention_max_len() rows, `heads` heads
// of attention_head_dim() columns; qkv [requests * length][3 * hidden], out [.][hidden].
hipError_t launch_attention_core(const uint16_t* qkv, int64_t requests, int length, int heads, uint16_t* out,
                                 hipStream_t stream);
int attention_head_dim();
int attention_max_len();

// Batched top-k of FP16 rows (k <= topk_max_k()): idx [rows][k] int32 and vals [rows][k] FP16
// in rank order; buf0 / buf1 hold topk_pairs_per_buffer() (key, index) pairs each (unused
// when a row fits one segment).
hipError_t launch_topk(const uint16_t* scores, int64_t rows, int64_t n, int k, int32_t* idx, uint16_t* vals,
                       int2* buf0, int2* buf1, hipStream_t stream);
int topk_max_k();
int64_t topk_pairs_per_buffer(int64_t rows, int64_t n, int k);

// Bits of the device error word (the values of the C ABI's RQ_FLAG_*).
enum : unsigned { kErrExpertId = 1u };

// Wait for all work on the current device, then read (and optionally clear) its error word.
hipError_t read_error_flags(unsigned int* flags, bool clear);

hipError_t launch_moe_combine(const uint16_t* y_perm, const int32_t* pos, const uint16_t* topk_w,
                              int64_t T, int top_k, int64_t N, uint16_t* out, hipStream_t stream);

}  // namespace rq
