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
// * Matrix core: v_mfma_f32_32x32x64_f8f6f4 (FP8 x FP8, 32 x 32 outputs, K = 64 per
//   instruction, full FP8 rate on gfx950).  Lane l feeds 32 bytes of A row (l & 31) and of
//   B column (l & 31); the two 32-lane halves take the two 32-byte halves of the 64-byte K
//   slab.  A and B use the same K assignment, so the dot product is the plain one.
// * Tiles: BM x BN outputs per workgroup (256x256, 256x128 or 128x128) split over a grid of
//   wavefronts (2 x 4, 4 x 2 or 2 x 2), each owning a block of 32x32 MFMA tiles.
// * Pipeline: K advances in 64-byte slabs (BM A rows + BN B rows, 32 KB at 256x256) held
//   in a ring of S LDS buffers (5 at 256x256, filling the 160 KB LDS).  Slabs are fetched
//   S - 1 ahead of the one being multiplied with buffer loads that write LDS directly (no
//   registers held for data in flight); one vmcnt wait and one barrier per slab.  Measured on MI355X, a single slab of lookahead
//   left the matrix cores idle about 70% of the time waiting for global loads.
// * LDS layout: 64-byte rows; the 16-byte granule g of row r sits at granule
//   g ^ ((r>>1)&1) ^ ((r>>1)&2) ^ ((r>>3)&1), so a fragment read (32 consecutive rows, one
//   granule) touches every bank once per 8- or 16-lane phase.  Each direct-to-LDS load
//   fills 16 consecutive rows; lanes fetch the granule that the swizzle puts at their slot.
//   Rows outside the tile and K past the end read as zero through the buffer range check.
// * Tile order: the hardware hands consecutive workgroup ids to the 8 XCDs in turn; ids are
//   remapped so each XCD receives a contiguous range of the logical order, and the logical
//   order walks groups of 8 M-tiles across all N-tiles, so tiles that share A rows or B
//   columns run on the same XCD and hit its L2.
// * Epilogue: accumulators are scaled (FP32 per-row and per-column scales), rounded to
//   FP16, staged through LDS one 32-row strip per wave, and written with 16-byte stores so
//   each output row segment is one contiguous burst.
//
// Grouped (MoE) mode: the M-tiles are the concatenation over experts of
// ceil(count_e / BM) tiles each, listed by the routing plan on the device in a table of
// {expert, first row, end row}.  A workgroup reads its entry with one load, reads A rows through the
// permutation (token perm[r] / top_k) when the input is per token, uses expert e's weights
// and scales, and writes permuted output rows.  Tiles past the device-side total exit at
// once, so the host never needs the per-expert counts.

#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "common.h"

namespace rq {
namespace {

constexpr int kGroupM = 8;
constexpr int BK = 64;          // K bytes per slab
constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset that always reads zero

template <int BM_, int BN_, int S_, int WGM_, int WGN_>
struct Cfg {
  static constexpr int BM = BM_;
  static constexpr int BN = BN_;
  static constexpr int S = S_;                   // LDS ring depth (slabs); S - 1 in flight
  static constexpr int WGM = WGM_;               // wavefronts along M
  static constexpr int WGN = WGN_;               // wavefronts along N
  static constexpr int WAVES = WGM * WGN;
  static constexpr int NT = 64 * WAVES;          // threads per workgroup
  static constexpr int WM = BM / WGM;            // wave tile rows
  static constexpr int WN = BN / WGN;            // wave tile columns
  static constexpr int TI = WM / 32;             // 32x32 MFMA tiles per wave, M direction
  static constexpr int TJ = WN / 32;             // ... N direction
  static constexpr int ROWS = BM + BN;           // A rows then B rows in one LDS slab
  static constexpr int STAGE = ROWS * BK;        // bytes per slab
  static constexpr int ROWS_PER_WAVE = ROWS / WAVES;
  static constexpr int LOADS = ROWS_PER_WAVE / 16;  // direct-to-LDS loads per lane per slab
  static constexpr int EPI_STRIDE = WN * 2 + 16;    // padded FP16 strip row (bytes)
  static constexpr int EPI_BYTES = 32 * EPI_STRIDE;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile");
  static_assert(ROWS_PER_WAVE % 16 == 0, "whole 16-row load groups per wave");
  static_assert(WAVES * EPI_BYTES + 4 * (BM + BN) <= S * STAGE, "epilogue staging fits in the ring");
  static_assert(NT >= BM && NT >= BN, "one thread per row / column scale");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile of whole 32x32 MFMA tiles");
  static_assert(S * STAGE <= 160 * 1024, "ring fits in the 160 KB LDS of a CU");
  static_assert((S - 1) * LOADS < 64, "outstanding loads fit the 6-bit vmcnt");
};

__device__ __forceinline__ int swz(int row, int g) {
  return g ^ ((row >> 1) & 1) ^ ((row >> 1) & 2) ^ ((row >> 3) & 1);
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] | vmcnt[5:4] << 14,
// expcnt and lgkmcnt at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The same, also waiting for all LDS reads (lgkmcnt = 0).
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// Scheduling pattern: MFMA q followed by its share of the next slab's fragment reads, the
// R reads spread over the first RM of the M MFMAs.
template <int Q, int M, int R, int RM>
__device__ __forceinline__ void interleave_mfma_reads() {
  if constexpr (Q < M) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    constexpr int hi = (Q + 1) * R / RM < R ? (Q + 1) * R / RM : R;
    constexpr int lo = Q * R / RM < R ? Q * R / RM : R;
    if constexpr (hi - lo > 0) __builtin_amdgcn_sched_group_barrier(0x100, hi - lo, 0);  // DS reads
    interleave_mfma_reads<Q + 1, M, R, RM>();
  }
}

// Wait until at most n slabs of L loads each remain outstanding (n clamped to [0, MAXN]).
template <int L, int MAXN, bool LGKM0>
__device__ __forceinline__ void wait_slabs(int n) {
  if constexpr (MAXN > 0) {
    if (n >= MAXN) {
      if constexpr (LGKM0) wait_vmcnt_lgkm0<MAXN * L>(); else wait_vmcnt<MAXN * L>();
      return;
    }
    wait_slabs<L, MAXN - 1, LGKM0>(n);
  } else {
    if constexpr (LGKM0) wait_vmcnt_lgkm0<0>(); else wait_vmcnt<0>();
  }
}

struct TileInfo {
  int64_t row_begin;
  int64_t row_end;
  int nt;
  int expert;
};

template <int BM, bool GROUPED>
__device__ __forceinline__ bool map_tile(const GemmArgs& p, int m_tiles, int n_tiles, TileInfo& t) {
  // Workgroup ids go round-robin over the 8 XCDs.  Give each XCD a contiguous slice of the
  // logical tile order (neighbouring tiles share operands in that XCD's L2).  In grouped
  // mode the grid is sized for the worst case, so the slices cover only the real tiles
  // (known on the device) and the surplus workgroups of every XCD exit.
  int total = (int)gridDim.x;
  if (GROUPED) {
    m_tiles = p.tile_start[p.E];  // real M-tiles; the grid covers the worst case
    total = m_tiles * n_tiles;
  }
  int bid = (int)blockIdx.x;
  if ((gridDim.x & 7) == 0) {
    const int per_xcd = (total + 7) >> 3;
    bid = (bid & 7) * per_xcd + (bid >> 3);
    if (bid >= total || (int)(blockIdx.x >> 3) >= per_xcd) return false;
  } else if (bid >= total) {
    return false;
  }
  const int per_group = kGroupM * n_tiles;
  const int group = bid / per_group;
  const int first_m = group * kGroupM;
  const int gm = min(m_tiles - first_m, kGroupM);
  const int in_group = bid - group * per_group;
  const int mt = first_m + in_group % gm;
  t.nt = in_group / gm;
  if (GROUPED) {
    const int4 ent = *reinterpret_cast<const int4*>(p.tile_table + 4 * (int64_t)mt);
    t.expert = ent.x;
    t.row_begin = ent.y;
    t.row_end = ent.z;
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

typedef int v4i __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: base, stride 0, num_records = bytes (reads at or past it return
// zero), gfx9 data format word.
__device__ __forceinline__ v4i make_desc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return (v4i){__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
               __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFFu)),
               __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
}

// One 16-byte-per-lane buffer load that writes LDS directly: lane l's 16 bytes land at
// LDS byte address lds_base + lds_imm + 16 l; the global address is base + voffset + soffset.
// Written as inline asm so that the compiler does not treat the outstanding LDS writes as
// aliasing every later LDS read (it would otherwise wait for all loads in flight before
// each fragment read); completion is tracked with explicit vmcnt waits instead.  The asm
// has no output registers.  One wait state separates the m0 write from the load.
// m0 is a reserved register, so clang warns about it in a clobber list: the clobber is only
// safe while no compiler-generated code in this file relies on m0, which a host-side ISA test
// (tests/test_kernel_isa.py) checks on every build.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds_16(const v4i& desc, uint32_t voffset, uint32_t soffset,
                                            uint32_t lds_base, int lds_imm) {
  asm volatile(
      "s_add_u32 m0, %0, %4\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(lds_base), "v"(voffset), "s"(desc), "s"(soffset), "i"(lds_imm)
      : "memory", "m0", "scc");
}
#pragma clang diagnostic pop

typedef float v16f __attribute__((ext_vector_type(16)));

template <class C, bool GROUPED>
__global__ __launch_bounds__(C::NT) void gemm_fp8_kernel(GemmArgs p, int m_tiles, int n_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::S * C::STAGE];
  TileInfo t;
  if (!map_tile<C::BM, GROUPED>(p, m_tiles, n_tiles, t)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps addressing scalar
  const int64_t K = p.K;
  const int64_t N = p.N;
  const int n0 = t.nt * C::BN;
  const v4i a_desc = make_desc(p.a, (uint32_t)(p.a_rows * K));
  const v4i b_desc = make_desc(p.b + (int64_t)t.expert * N * K, (uint32_t)(N * K));
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  const float* __restrict__ sb = p.b_scale + (int64_t)t.expert * N;

  // Row / column scales for the epilogue: issued before the first direct-to-LDS load, so
  // they complete before it (vector memory loads return in order) and cost no wait later.
  float my_sa = 0.f, my_sb = 0.f;
  if (tid < C::BM) {
    const int64_t r = t.row_begin + tid;
    if (r < t.row_end) my_sa = p.a_scale[a_source_row<GROUPED>(p, r)];
  }
  if (tid < C::BN && n0 + tid < N) my_sb = sb[n0 + tid];

  // ---- direct-to-LDS loads.  Load t of wave w fills slab rows [row0, row0 + 16) with
  // row0 = w * ROWS_PER_WAVE + 16 t; lane l writes 16 bytes at row row0 + l / 4, physical
  // granule l % 4, so it fetches logical granule (l % 4) ^ f(row) of that row.
  // The swizzle depends only on row bits 1..3, which (lane >> 2) fixes for every load, so
  // each lane fetches the same granule in all of its loads.
  const int gran = swz(lane >> 2, lane & 3);  // XOR swizzle is its own inverse
  uint32_t src_off[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int row0 = wave * C::ROWS_PER_WAVE + 16 * i;
    const int row = row0 + (lane >> 2);
    const int g = gran;
    if (row0 < C::BM) {
      const int64_t r = t.row_begin + row;
      const bool ok = GROUPED ? r < t.row_end : true;  // dense rows past M read zero
      src_off[i] = ok ? (uint32_t)(a_source_row<GROUPED>(p, r) * K + 16 * g) : kOutOfRange;
    } else {
      src_off[i] = (uint32_t)((n0 + (row - C::BM)) * K + 16 * g);  // rows past N read zero
    }
  }
  // Wave-uniform LDS byte address of this wave's first 16-row group in ring buffer `buf`.
  auto wave_lds = [&](int buf) -> uint32_t {
    return (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(smem_lds + buf * C::STAGE + wave * C::ROWS_PER_WAVE * BK));
  };
  // Full slab (all 64 K bytes in range): the K offset travels in the scalar soffset.
  auto issue_full = [&](int slab, uint32_t lds, int i) {
    const int row0 = wave * C::ROWS_PER_WAVE + 16 * i;
    load_lds_16(row0 < C::BM ? a_desc : b_desc, src_off[i], (uint32_t)__builtin_amdgcn_readfirstlane(slab * BK),
                lds, 16 * BK * i);
  };
  // Any slab, including the ragged last one: granules past K read zero.
  auto issue_one = [&](int slab, int buf, int i) {
    const uint32_t k0 = (uint32_t)slab * BK;
    const int row0 = wave * C::ROWS_PER_WAVE + 16 * i;
    const bool kin = (int64_t)k0 + 16 * gran < K;
    const uint32_t off = kin ? src_off[i] + k0 : kOutOfRange;
    load_lds_16(row0 < C::BM ? a_desc : b_desc, off, 0u, wave_lds(buf), 16 * BK * i);
  };
  auto issue_slab = [&](int slab, int buf) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) issue_one(slab, buf, i);
  };

  // ---- MFMA fragment addressing: lane -> (row within 32, K half).  A fragment is two
  // 16-byte LDS reads (granules 2 half and 2 half + 1 of its row).
  const int wm = wave / C::WGN;
  const int wn = wave % C::WGN;
  const int frow = lane & 31;
  const int half = lane >> 5;
  const int f_off[2] = {frow * BK + 16 * swz(frow, 2 * half), frow * BK + 16 * swz(frow, 2 * half + 1)};
  constexpr int kReads = 2 * (C::TI + C::TJ);   // 16-byte fragment reads per slab
  constexpr int kMfma = C::TI * C::TJ;
  // The next slab's fragment reads go out during the first half of the MFMAs, so they have
  // landed by the lgkmcnt wait that precedes the next barrier.
  constexpr int kReadMfmas = kMfma / 2 > 0 ? kMfma / 2 : 1;
  // read r of a slab: A fragments first, then B; r / 2 selects the fragment, r % 2 the half
  auto read_one = [&](const uint8_t* S, int r) -> uint4 {
    const int f = r >> 1;
    const int row = f < C::TI ? wm * C::WM + 32 * f : C::BM + wn * C::WN + 32 * (f - C::TI);
    return *reinterpret_cast<const uint4*>(S + row * BK + f_off[r & 1]);
  };

  v16f acc[C::TI][C::TJ];
#pragma unroll
  for (int i = 0; i < C::TI; ++i)
#pragma unroll
    for (int j = 0; j < C::TJ; ++j) acc[i][j] = (v16f){};

  // Two fragment register sets: the MFMAs of slab kt use one while the reads of slab kt+1
  // fill the other.
  uint4 fr0[kReads], fr1[kReads];
  auto as_v8 = [](const uint4& lo, const uint4& hi) -> v8i {
    return (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };

  const int ktiles = (int)((K + BK - 1) / BK);
  // prologue: slabs 0..S-1 in flight, then slab 0's fragments
#pragma unroll
  for (int s = 0; s < C::S; ++s)
    if (s < ktiles) issue_slab(s, s);
  wait_slabs<C::LOADS, C::S - 1, false>((ktiles < C::S ? ktiles : C::S) - 1);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kReads; ++r) fr0[r] = read_one(smem, r);

  // One slab: wait for slab kt+1 and the reads of slab kt, barrier (slab kt's buffer is then
  // free for slab kt+4), then the MFMAs of slab kt interleaved with the fragment reads of
  // slab kt+1 and the direct-to-LDS loads of slab kt+4.  A single wave can issue only about
  // a dozen other instructions in the shadow of one 32x32x64 MFMA, so the steady-state step
  // (every slab involved complete and in range) carries no run-time conditions and no
  // vector address arithmetic; the generic step handles the last slabs and a ragged K.
  auto step = [&](auto steady, int kt, uint4 (&cur)[kReads], uint4 (&nxt)[kReads]) {
    constexpr bool kSteady = decltype(steady)::value;
    bool has_next = true, has_load = true;
    if constexpr (kSteady) {
      wait_vmcnt_lgkm0<(C::S - 2) * C::LOADS>();
    } else {
      wait_slabs<C::LOADS, C::S - 2, true>(ktiles - 2 - kt);  // slabs issued after kt+1
      has_next = kt + 1 < ktiles;
      has_load = kt + C::S < ktiles;
    }
    __syncthreads();
    const uint8_t* Sn = smem + ((kt + 1) % C::S) * C::STAGE;
    const uint32_t lds_dst = wave_lds(kt % C::S);
    int r = 0, l = 0;
#pragma unroll
    for (int q = 0; q < kMfma; ++q) {
      const int i = q / C::TJ, j = q % C::TJ;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          as_v8(cur[2 * i], cur[2 * i + 1]), as_v8(cur[2 * (C::TI + j)], cur[2 * (C::TI + j) + 1]),
          acc[i][j], 0, 0, 0, 0, 0, 0);
      const int r_end = (q + 1) * kReads / kReadMfmas < kReads ? (q + 1) * kReads / kReadMfmas : kReads;
      for (; r < r_end; ++r)
        if (kSteady || has_next) nxt[r] = read_one(Sn, r);
      const int l_end = (q + 1) * C::LOADS / kMfma;
      for (; l < l_end; ++l) {
        if constexpr (kSteady) issue_full(kt + C::S, lds_dst, l);
        else if (has_load) issue_one(kt + C::S, kt % C::S, l);
      }
    }
    interleave_mfma_reads<0, kMfma, kReads, kReadMfmas>();
  };

  using Steady = std::integral_constant<bool, true>;
  using Generic = std::integral_constant<bool, false>;
  const int full_slabs = (int)(K / BK);
  int kt = 0;
  for (; kt + 1 + C::S < full_slabs; kt += 2) {  // kt and kt+1 steady: kt+1+S < full_slabs
    step(Steady{}, kt, fr0, fr1);
    step(Steady{}, kt + 1, fr1, fr0);
  }
  for (; kt + 1 < ktiles; kt += 2) {
    step(Generic{}, kt, fr0, fr1);
    step(Generic{}, kt + 1, fr1, fr0);
  }
  if (kt < ktiles) step(Generic{}, kt, fr0, fr1);
  __syncthreads();

  // ---- epilogue: one 32-row strip of the wave tile at a time, staged through LDS.
  // 32x32 MFMA output layout: lane holds column (lane & 31) and, for register r, row
  // 8 (r / 4) + 4 (lane / 32) + r % 4.  Strip rows are EPI_STRIDE bytes apart (padded so
  // the two lane halves hit different banks); read back as 16-byte chunks of 8 columns.
  // The row and column scales, loaded into registers at kernel start, go to LDS first.
  uint8_t* strip = smem + wave * C::EPI_BYTES;
  float* s_sa = reinterpret_cast<float*>(smem + C::WAVES * C::EPI_BYTES);
  float* s_sb = s_sa + C::BM;
  if (tid < C::BM) s_sa[tid] = my_sa;
  if (tid < C::BN) s_sb[tid] = my_sb;
  __syncthreads();
  float sbv[C::TJ];
#pragma unroll
  for (int j = 0; j < C::TJ; ++j) sbv[j] = s_sb[wn * C::WN + 32 * j + frow];
  constexpr int kChunksPerRow = C::WN / 8;
  constexpr int kChunks = 32 * kChunksPerRow;
#pragma unroll
  for (int i = 0; i < C::TI; ++i) {
    const int64_t strip_row0 = t.row_begin + wm * C::WM + 32 * i;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int srow = 8 * (r >> 2) + 4 * half + (r & 3);
      const float sa = s_sa[wm * C::WM + 32 * i + srow];
      uint16_t* dst = reinterpret_cast<uint16_t*>(strip + srow * C::EPI_STRIDE) + frow;
#pragma unroll
      for (int j = 0; j < C::TJ; ++j) dst[32 * j] = (uint16_t)float_to_half_bits((acc[i][j][r] * sa) * sbv[j]);
    }
    __syncthreads();
#pragma unroll
    for (int c = lane; c < kChunks; c += 64) {
      const int srow = c / kChunksPerRow;
      const int scol = (c % kChunksPerRow) * 8;
      const int64_t row = strip_row0 + srow;
      const int64_t col = n0 + wn * C::WN + scol;
      const uint4 v = *reinterpret_cast<const uint4*>(strip + srow * C::EPI_STRIDE + 2 * scol);
      if (row < t.row_end && col < N) st_global_16(p.y + row * N + col, v);
    }
    __syncthreads();
  }
}

template <class C, bool GROUPED>
hipError_t launch(const GemmArgs& g, int m_tiles, hipStream_t stream) {
  const int n_tiles = (int)((g.N + C::BN - 1) / C::BN);
  gemm_fp8_kernel<C, GROUPED><<<dim3(m_tiles * n_tiles), dim3(C::NT), 0, stream>>>(g, m_tiles, n_tiles);
  return hipGetLastError();
}

// Eight wavefronts (two per SIMD) for the large tiles: while one wavefront of a SIMD waits
// on a load issue, an LDS read or the barrier, the other keeps the matrix core busy.
// Measured on MI355X: +8% (256x256) and +5% (256x128) over four wavefronts of twice the
// tile each.  The 64-row tiles serve small M (the weight-streaming regime) and MoE experts
// with few rows, where 256-row tiles would spend most MFMA work on padding.
using Big = Cfg<256, 256, 4, 2, 4>;      // 128 KB ring, 128x64 per wavefront
using Wide = Cfg<256, 128, 4, 4, 2>;     // 96 KB ring, 64x64 per wavefront
using Small = Cfg<128, 128, 4, 2, 2>;    // 64 KB ring, two workgroups per CU
using Thin = Cfg<64, 128, 4, 1, 4>;      // 48 KB ring, three workgroups per CU
using ThinWide = Cfg<64, 256, 4, 1, 4>;  // 80 KB ring, two workgroups per CU

struct TileDesc {
  const char* name;
  int bm, bn;
};
const TileDesc kTiles[kTileKinds] = {
    {"256x256", 256, 256}, {"256x128", 256, 128}, {"128x128", 128, 128}, {"64x128", 64, 128}, {"64x256", 64, 256},
};

int tile_override() {
  const char* e = std::getenv("RQ_GEMM_TILE");
  if (e == nullptr) return -1;
  for (int k = 0; k < kTileKinds; ++k)
    if (std::strcmp(e, kTiles[k].name) == 0) return k;
  return -1;
}

// Pick the tile for a dense M x N problem: the largest tile (most operand reuse per byte
// loaded) that still yields enough workgroups to occupy the 256 CUs, else the thinnest.
// On MI355X this rule picks the fastest shape for every linear of the workloads (measured
// over all five shapes at M = 512 and M = 4096).
int pick_dense(int64_t M, int64_t N) {
  const int forced = tile_override();
  if (forced >= 0) return forced;
  const int order[] = {kTileBig, kTileWide, kTileSmall, kTileThin};
  for (int o : order) {
    const TileDesc& d = kTiles[o];
    const int64_t tiles = ((M + d.bm - 1) / d.bm) * ((N + d.bn - 1) / d.bn);
    if (tiles >= 192) return o;
  }
  return kTileThin;
}

template <class C>
hipError_t launch_dense(const GemmArgs& g, hipStream_t stream) {
  return launch<C, false>(g, (int)((g.M + C::BM - 1) / C::BM), stream);
}

}  // namespace

int pick_grouped(int64_t R, int64_t E) {
  const int forced = tile_override();
  if (forced == kTileBig || forced == kTileThinWide) return forced;
  // experts average R / E rows: 64-row tiles once 256-row tiles would be mostly padding
  return R >= 192 * E ? kTileBig : kTileThinWide;
}

int tile_rows(int kind) { return kTiles[kind].bm; }

int64_t grouped_max_mtiles(int64_t R, int64_t E, int tile_m) { return (R + tile_m - 1) / tile_m + E; }

hipError_t launch_gemm_dense(const GemmArgs& g, hipStream_t stream) {
  if (g.M <= 0) return hipSuccess;
  switch (pick_dense(g.M, g.N)) {
    case kTileBig: return launch_dense<Big>(g, stream);
    case kTileWide: return launch_dense<Wide>(g, stream);
    case kTileSmall: return launch_dense<Small>(g, stream);
    case kTileThin: return launch_dense<Thin>(g, stream);
    default: return launch_dense<ThinWide>(g, stream);
  }
}

hipError_t launch_gemm_grouped(const GemmArgs& g, int kind, hipStream_t stream) {
  if (g.M <= 0) return hipSuccess;
  if (kind == kTileThinWide)
    return launch<ThinWide, true>(g, (int)grouped_max_mtiles(g.M, g.E, ThinWide::BM), stream);
  return launch<Big, true>(g, (int)grouped_max_mtiles(g.M, g.E, Big::BM), stream);
}

}  // namespace rq
