// FP8 (OCP E4M3) x FP8 GEMM with FP32 accumulation and a fused per-token x per-channel
// dequantization to FP16, for gfx950 (MI355X).
//
// Computes y[m][n] = fl16(fl32(fl32(acc * s_a[m]) * s_b[n])), acc = sum_k a[m][k] * b[n][k]:
// the FP8 product with FP32 accumulation and the cast back to FP16 of page "Quantized
// Inference for OneRec-V2：生成式推荐开始直接吃 LLM 量化栈", section 关键证据, with the
// quantize -> FP8 GEMM -> dequantize flow of page "FP8量化在生成式推荐系统OneRec-V2中的
// 优化实践", §2.3 / Fig. 2.  Both operands are K-contiguous ("TN"): activations [M][K],
// weights [N][K] in the nn.Linear layout.
//
// Design (CDNA4):
// * Matrix core: v_mfma_f32_32x32x64_f8f6f4 (FP8 x FP8, 32 x 32 outputs, K = 64 per
//   instruction, full FP8 rate on gfx950).  Lane l feeds 32 bytes of row (l & 31) of each
//   operand; the two 32-lane halves take the two 32-byte halves of the 64-byte K slab.  Both
//   operands use the same K assignment, so the dot product is the plain one.  The weight
//   fragment is the instruction's first operand and the activation fragment its second, so
//   the 32 x 32 result comes out transposed: lane l holds token row (l & 31) and, in
//   register r, output column 8 (r / 4) + 4 (l / 32) + r % 4 - four consecutive columns
//   per group of four registers, which the epilogue writes straight to memory.
// * Tiles: BM x BN outputs per workgroup (256x256, 256x192, 256x128, 128x128, 64x128 or 64x256)
//   split over a grid of wavefronts, each owning a block of 32x32 MFMA tiles.
// * Persistent workgroups: the grid holds as many workgroups as the CUs keep resident and
//   each walks a list of tiles, so one tile's epilogue overlaps the loads of the next.
// * Pipeline: K advances in 64-byte slabs (BM A rows + BN B rows, 32 KB at 256x256) held
//   in a ring of S LDS buffers.  Slabs are fetched S - 1 ahead of the one being multiplied
//   with buffer loads that write LDS directly (no registers held for data in flight); one
//   vmcnt wait and one barrier per slab.  The ring runs on across tiles: the last S steps
//   of a tile fetch the first S slabs of the workgroup's next tile, and the row and column
//   scales of each tile arrive the same way in a small double-buffered LDS area.  Measured
//   on MI355X, a single slab of lookahead left the matrix cores idle about 70% of the time
//   waiting for global loads.
// * LDS layout: 64-byte rows; the 16-byte granule g of row r sits at granule
//   g ^ ((r>>1)&1) ^ ((r>>1)&2) ^ ((r>>3)&1), so a fragment read (32 consecutive rows, one
//   granule) touches every bank once per 8- or 16-lane phase.  Each direct-to-LDS load
//   fills 16 consecutive rows; lanes fetch the granule that the swizzle puts at their slot.
//   Rows outside the tile and K past the end read as zero through the buffer range check.
// * Tile order: the hardware hands consecutive workgroup ids to the 8 XCDs in turn; each
//   XCD's workgroups share a contiguous slice of the logical order, and the logical order
//   walks groups of 4 M-tiles across all N-tiles, so tiles that share A rows or B columns
//   run on the same XCD at the same time and hit its L2.  In grouped mode the groups never
//   straddle two experts (an expert's M-tiles are cut into groups of at most 4), so the
//   tiles running together read one expert's weights rather than two.
// * Epilogue: each lane scales its four-column groups (FP32 row and column scales read from
//   LDS) and rounds them to FP16; column groups are paired across the two 32-lane halves
//   so each lane stores 16 bytes.
// * Wavefront roles (the 256-row tiles): half the wavefronts issue every global load and
//   never store, the other half issue every output store (the loaders' outputs reach them
//   through LDS strips) and never wait for loads to land (see the kernel).
//
// Grouped (MoE) mode: the M-tiles are the concatenation over experts of
// ceil(count_e / BM) tiles each, listed by the routing plan on the device in a table of
// {expert, first row, end row}.  A tile reads its entry with one scalar load, multiplies
// permuted rows [first, end) of A with expert e's weights and scales, and writes the same
// permuted output rows.  The device-side tile total bounds the walk, so the host never
// needs the per-expert counts.

#include <atomic>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "common.h"

namespace rq {
namespace {

// M-tiles per group of the tile walk.  A group's A rows stay in the XCD's L2 while its tiles
// walk the N-tiles; measured on MI355X (GEMM kernel time, caches flushed, interleaved runs):
// groups of 4 beat 8 by 1-2% on the MoE and FFN GEMMs, 2 and 16 are slower.
constexpr int kGroupM = 4;
constexpr int BK = 64;          // K bytes per slab
constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset that always reads zero

template <int BM_, int BN_, int S_, int WGM_, int WGN_, bool SPLIT_>
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
  // Wavefront roles (SPLIT): waves 0..LOADERS-1 issue every load, waves LOADERS.. every
  // output store (see the kernel), so no wave ever waits for its stores to retire.
  // Otherwise every wave loads and stores its own outputs.
  static constexpr bool SPLIT = SPLIT_;
  static constexpr int LOADERS = SPLIT ? WAVES / 2 : WAVES;
  static constexpr int LOADS = ROWS / 16 / LOADERS;  // direct-to-LDS loads per loader lane per slab
  static constexpr int A_LOADS = BM / 16 / LOADERS;  // the first A_LOADS of them fetch A rows
  static constexpr int SCALE_BYTES = 4 * ROWS;       // BM row scales, then BN column scales
  static constexpr int SCALE_LOADS = ROWS / 64;      // 4-byte-per-lane loads per tile
  static constexpr int EPI_STRIDE = 2 * WN + 16;     // padded FP16 row of an output strip
  static constexpr int GATE_STRIDE = WN + 16;        // padded FP16 row of a gated (half-width) strip
  // a loader's strip: one 32-row output block, or two of the gated output
  static constexpr int STRIP = 32 * EPI_STRIDE > 64 * GATE_STRIDE ? 32 * EPI_STRIDE : 64 * GATE_STRIDE;
  static constexpr int SCALE_OFF = S * STAGE;
  static constexpr int EPI_OFF = SCALE_OFF + 2 * SCALE_BYTES;
  static constexpr int LDS = EPI_OFF + (SPLIT ? LOADERS * STRIP : 0);
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile");
  static_assert((!SPLIT || WAVES % 2 == 0) && (ROWS / 16) % LOADERS == 0, "whole 16-row load groups per loader");
  static_assert((BM / 16) % LOADERS == 0, "each load fetches only A rows or only B rows");
  static_assert((16 * WN / 8) % 64 == 0, "whole strip reads per lane");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile of whole 32x32 MFMA tiles");
  static_assert(LDS <= 160 * 1024, "ring, scales and strips fit in the 160 KB LDS of a CU");
  static_assert(S >= 2 && S * LOADS + (SCALE_LOADS + LOADERS - 1) / LOADERS < 64,
                "outstanding loads fit the 6-bit vmcnt");
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

// Only the LDS reads (lgkmcnt = 0; vmcnt and expcnt at their maxima).
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// Scheduling pattern of one slab (M MFMAs over TI x TJ tiles, i-major): each MFMA followed
// by the fragment reads it frees or that are due - two B reads after each of the first TJ
// MFMAs, and A fragment i's two reads after the last MFMA that uses it.
// RESC (block scales, see the kernel): 1 in the last slab of a K block, where the 16
// multiplies rescaling MFMA tile q - 1's accumulator follow MFMA q (that tile's MFMA has
// finished by then, and the multiplies run in the shadow of MFMA q); 2 in the first slab of
// the next block, where the last tile's rescale follows MFMA 0.
template <int Q, int M, int TJ, int RESC = 0>
__device__ __forceinline__ void interleave_mfma_reads() {
  if constexpr (Q < M) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    if constexpr ((RESC == 1 && Q >= 1) || (RESC == 2 && Q == 0))
      __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);  // a tile's 16 rescale multiplies
    constexpr int reads = (Q < TJ ? 2 : 0) + (Q % TJ == TJ - 1 ? 2 : 0);
    if constexpr (reads > 0) __builtin_amdgcn_sched_group_barrier(0x100, reads, 0);  // DS reads
    interleave_mfma_reads<Q + 1, M, TJ, RESC>();
  }
}

// Wait until at most n slabs of L loads each remain outstanding (n clamped to [0, MAXN]).
// Loads return in issue order, so every slab issued before the last n is then in LDS.
// Any other vector memory operation issued later (scale loads, output stores) only makes
// the wait stricter.
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

// A wave-uniform load through the scalar cache, from memory that no kernel writes while
// this one runs (the routing plan's tables).
__device__ __forceinline__ int load_uniform(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)(p);
}
__device__ __forceinline__ float load_uniform_f(const float* p) {
  return *(const __attribute__((address_space(4))) float*)(p);
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

// Buffer loads that write LDS directly: lane l's 16 bytes land at LDS byte address
// lds_base + lds_imm + 16 l (4 bytes at lds_addr + 4 l for the dword form); the global
// address is base + voffset + soffset.
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

__device__ __forceinline__ void load_lds_4(const v4i& desc, uint32_t voffset, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(lds_addr), "v"(voffset), "s"(desc)
      : "memory", "m0");
}
#pragma clang diagnostic pop

typedef float v16f __attribute__((ext_vector_type(16)));

struct TileInfo {
  int row_begin;  // first output row (permuted row in grouped mode)
  int row_end;    // one past the last valid row
  int n0;         // first output column
  int expert;
  int part;       // split-K: the K part this work item sums (0 without split)
};

// Logical tile L -> rows and columns: groups of kGroupM M-tiles walked column by column.  In
// grouped mode expert e owns logical tiles [tile_start[e], tile_start[e + 1]) * n_tiles and
// its M-tiles are grouped on their own.
template <int BM, int BN, bool GROUPED>
__device__ __forceinline__ TileInfo tile_info(const GemmArgs& p, int L, int m_tiles, int n_tiles,
                                              int tiles_per_part = 0, int mt_cap = 0) {
  int part = 0;
  if (tiles_per_part > 0) {  // split-K: work item L is part L / tiles of tile L % tiles
    part = L / tiles_per_part;
    L -= part * tiles_per_part;
  }
  int base = 0;
  if (GROUPED) {  // the expert whose M-tiles hold L: largest e with tile_start[e] * n_tiles <= L
    int lo = 0, hi = p.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (load_uniform(p.tile_start + mid) * n_tiles <= L) lo = mid; else hi = mid;
    }
    base = load_uniform(p.tile_start + lo);
    m_tiles = load_uniform(p.tile_start + lo + 1) - base;
    L -= base * n_tiles;
  }
  const int per_group = kGroupM * n_tiles;
  const int group = L / per_group;
  const int first_m = group * kGroupM;
  const int gm = GROUPED ? max(min(m_tiles - first_m, kGroupM), 1) : min(m_tiles - first_m, kGroupM);
  const int in_group = L - group * per_group;
  const int mt = base + first_m + in_group % gm;
  TileInfo t;
  t.part = part;
  t.n0 = (in_group / gm) * BN;
  if (GROUPED) {
    t.n0 = min(max(t.n0, 0), (n_tiles - 1) * BN);
    // the plan may come from an earlier call (RQ_MOE_PLAN_READY): every value is clamped into
    // range, so even a plan that does not belong to these ids cannot move an access outside the
    // operands (it only gives wrong rows); for the plan the call builds itself these are no-ops
    const int32_t* ent = p.tile_table + 4 * (int64_t)min(max(mt, 0), mt_cap - 1);
    t.expert = min(max(load_uniform(ent), 0), p.E - 1);
    t.row_begin = min(max(load_uniform(ent + 1), 0), p.a_rows);
    t.row_end = min(max(load_uniform(ent + 2), t.row_begin), min(t.row_begin + BM, p.a_rows));
  } else {
    t.expert = 0;
    t.row_begin = mt * BM;
    t.row_end = min(t.row_begin + BM, p.M);
  }
  return t;
}

// Buffer descriptors of one tile: A covers its valid rows, B its valid weight rows, so
// everything past them reads zero.
struct TileDesc2 {
  v4i a, b;
};

// Selects between descriptor values (a conditional on references would force them into
// memory).
__device__ __forceinline__ v4i pick(bool c, v4i x, v4i y) { return c ? x : y; }

// Split-K: the descriptors start at the part's first K byte (kl bytes per part), so the K
// loop runs over the part as over a whole row; the row stride stays K.
// Slab-layout weights ([E][K/64][N][64]): the tile's rows start at byte (k0 / 64) * 64 N +
// 64 n0 of the expert's matrix and the range runs to the matrix's end.  Rows past N then read
// the first rows of the next slab (or zero past the matrix): they only feed output columns
// past N, which are never stored.
template <int BN>
__device__ __forceinline__ TileDesc2 tile_descs(const GemmArgs& p, const TileInfo& t, int kl = 0) {
  TileDesc2 d;
  const int k0 = t.part * kl;
  d.a = make_desc(p.a + (int64_t)t.row_begin * p.K + k0, (uint32_t)((t.row_end - t.row_begin) * p.K - k0));
  if (p.b_slabs) {
    const int rel = k0 * p.N + 64 * t.n0;  // k0 is a multiple of 64
    d.b = make_desc(p.b + (int64_t)t.expert * p.N * p.K + rel, (uint32_t)(p.N * p.K - rel));
  } else {
    d.b = make_desc(p.b + ((int64_t)t.expert * p.N + t.n0) * p.K + k0, (uint32_t)(min(BN, p.N - t.n0) * p.K - k0));
  }
  return d;
}

template <class C, bool GROUPED, bool GATE, bool BLK, bool A5, bool SPLITK>
__global__ __launch_bounds__(C::NT) void gemm_fp8_kernel(GemmArgs p, int m_tiles, int n_tiles) {
  // operand formats of the MFMA: the weight fragment (first operand) is E4M3, the activation
  // fragment (second) E4M3 or, with A5, E5M2 (format code 1 of the f8f6f4 instruction)
  constexpr int kFmtB = A5 ? 1 : 0;
  static_assert(!SPLITK || (!GROUPED && !GATE && !BLK && !C::SPLIT),
                "split-K: dense, plain output, per-channel or per-tensor scales, every wave stores");
  static_assert(!BLK || (C::WN <= kScaleBlock && kScaleBlock % C::WN == 0),
                "a wave's columns lie in one 128-column scale block");
  static_assert(!GATE || C::TJ % 2 == 0, "gated output pairs 32-column gate and up blocks in a wave");
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];

  // ---- this workgroup's tiles: logical tiles first, first + stride, ... below last.
  // Workgroup ids go round-robin over the 8 XCDs; each XCD's workgroups share a contiguous
  // slice of the logical order.  In grouped mode the real M-tile count is on the device.
  // grouped: the real M-tile count is on the device, at most the host's bound m_tiles
  const int mt_cap = m_tiles;
  if (GROUPED) m_tiles = min(max(load_uniform(p.tile_start + p.E), 0), mt_cap);
  const int tiles_pp = SPLITK ? m_tiles * n_tiles : 0;  // split-K: tiles per K part
  const int total = m_tiles * n_tiles * (SPLITK ? p.splits : 1);
  int first, stride, last;
  {
    const int bid = (int)blockIdx.x;
    if ((gridDim.x & 7) == 0) {
      const int per_xcd = (total + 7) >> 3;
      const int xcd = bid & 7;
      first = xcd * per_xcd + (bid >> 3);
      stride = (int)(gridDim.x >> 3);
      last = min(total, (xcd + 1) * per_xcd);
    } else {
      first = bid;
      stride = (int)gridDim.x;
      last = total;
    }
  }
  if (first >= last) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps addressing scalar
  // gfx9 counts loads and stores in one vmcnt per wave, so a wave that stored its outputs
  // would wait for those stores to retire at its next slab wait - with every CU writing its
  // tile at once, several microseconds.  With SPLIT, loader waves therefore issue all loads
  // and never store; storer waves issue all output stores (their own rows and their partner
  // loader's, handed over in LDS) and never wait on vmcnt - the barrier after the loaders'
  // waits tells them a slab has landed.  Tiles with few MFMAs per slab keep every wave a
  // loader: there a single wave could not issue a whole slab's loads in the time of its
  // MFMAs.
  const bool loader = wave < C::LOADERS;                  // every wave unless SPLIT
  const bool storer = !C::SPLIT || wave >= C::LOADERS;    // every wave unless SPLIT
  const int K = p.K;    // row stride of both operands
  const int N = p.N;
  const uint32_t smem_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  const int KL = SPLITK ? K / p.splits : K;  // K bytes one work item sums (a multiple of BK when split)
  const int ktiles = (KL + BK - 1) / BK;
  const int full_slabs = KL / BK;

  // ---- direct-to-LDS loads.  Load i of loader w fills slab rows [row0, row0 + 16) with
  // row0 = 16 (i * LOADERS + w); lane l writes 16 bytes at row row0 + l / 4, physical
  // granule l % 4, so it fetches logical granule (l % 4) ^ f(row) of that row.  Loads
  // i < A_LOADS cover the BM A rows, the rest the BN B rows.
  // The swizzle depends only on row bits 1..3, which (lane >> 2) fixes for every load, so
  // each lane fetches the same granule in all of its loads.  Offsets are relative to the
  // tile's descriptors, so they are the same for every tile.
  // Slab-layout weights: B row r of the tile sits at 64 r and K slab s at 64 N s past the
  // tile's start (bstep: the B byte offset of one K byte, N instead of 1).
  const int gran = swz(lane >> 2, lane & 3);  // XOR swizzle is its own inverse
  const uint32_t bstep = p.b_slabs ? (uint32_t)N : 1u;
  uint32_t voff[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int row = 16 * (i * C::LOADERS + wave) + (lane >> 2);
    const int brow = p.b_slabs ? (row - C::BM) * BK : (row - C::BM) * K;
    voff[i] = (uint32_t)((i < C::A_LOADS ? row * K : brow) + 16 * gran);
  }
  // Wave-uniform LDS byte address of this wave's first 16-row group in ring buffer `buf`.
  auto wave_lds = [&](int buf) -> uint32_t {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)(smem_lds + buf * C::STAGE + wave * 16 * BK));
  };
  // Full slab (all 64 K bytes in range): the K offset (soff = slab * 64) travels in the
  // scalar soffset.
  auto issue_full = [&](const TileDesc2& d, uint32_t soff, uint32_t lds, int i) {
    load_lds_16(i < C::A_LOADS ? d.a : d.b, voff[i], i < C::A_LOADS ? soff : soff * bstep, lds,
                16 * BK * C::LOADERS * i);
  };
  // Any slab, including the ragged last one: granules past K read zero.
  auto issue_one = [&](const TileDesc2& d, int slab, uint32_t lds, int i) {
    const uint32_t k0 = (uint32_t)slab * BK;
    const bool kin = (int)k0 + 16 * gran < KL;
    load_lds_16(i < C::A_LOADS ? d.a : d.b, kin ? voff[i] + (i < C::A_LOADS ? k0 : k0 * bstep) : kOutOfRange, 0u,
                lds, 16 * BK * C::LOADERS * i);
  };
  // The tile's BM row scales and BN column scales into scale area `region` (0 or 1);
  // entries past the tile's rows or columns read zero and are never used.
  auto issue_scales = [&](const TileInfo& t, int region) {
    if (!loader || SPLITK) return;  // split-K parts are scaled by the reduce kernel
    const uint32_t base = smem_lds + C::SCALE_OFF + region * C::SCALE_BYTES;
    for (int q = wave; q < C::SCALE_LOADS; q += C::LOADERS) {
      const uint32_t dst = (uint32_t)__builtin_amdgcn_readfirstlane((int)(base + 256 * q));
      if (q < C::BM / 64) {
        const v4i d = make_desc(p.a_scale + t.row_begin, (uint32_t)(4 * (t.row_end - t.row_begin)));
        load_lds_4(d, (uint32_t)(4 * (64 * q + lane)), dst);
      } else {
        // column scales: the channel's own, the tensor's one scale, or (block scales) the
        // scale of the channel's last K block, the one the accumulator is kept relative to
        const int col = 64 * (q - C::BM / 64) + lane;
        if (p.b_gran == kScaleTensor) {
          load_lds_4(make_desc(p.b_scale + t.expert, 4u), 0u, dst);
        } else if (BLK) {
          const int kb = K / kScaleBlock, per_expert = (N / kScaleBlock) * kb;
          const v4i d = make_desc(p.b_scale + (int64_t)t.expert * per_expert, (uint32_t)(4 * per_expert));
          const int n = t.n0 + col;
          load_lds_4(d, n < N ? (uint32_t)(4 * ((n / kScaleBlock) * kb + kb - 1)) : kOutOfRange, dst);
        } else {
          const v4i d = make_desc(p.b_scale + (int64_t)t.expert * N + t.n0, (uint32_t)(4 * min(C::BN, N - t.n0)));
          load_lds_4(d, (uint32_t)(4 * col), dst);
        }
      }
    }
  };

  // ---- MFMA fragment addressing: lane -> (row within 32, K half).  A fragment is two
  // 16-byte LDS reads (granules 2 half and 2 half + 1 of its row).
  const int wm = wave / C::WGN;
  const int wn = wave % C::WGN;
  const int frow = lane & 31;
  const int half = lane >> 5;
  const int f_off[2] = {frow * BK + 16 * swz(frow, 2 * half), frow * BK + 16 * swz(frow, 2 * half + 1)};
  constexpr int kMfma = C::TI * C::TJ;
  constexpr int kDmaGroups = kMfma < 2 ? kMfma : 2;
  // Fragment r (= 2 f + h) of the A (or B) rows of a slab: half h of 32-row fragment f.
  auto read_a = [&](const uint8_t* S, int r) -> uint4 {
    return *reinterpret_cast<const uint4*>(S + (wm * C::WM + 32 * (r >> 1)) * BK + f_off[r & 1]);
  };
  auto read_b = [&](const uint8_t* S, int r) -> uint4 {
    return *reinterpret_cast<const uint4*>(S + (C::BM + wn * C::WN + 32 * (r >> 1)) * BK + f_off[r & 1]);
  };
  auto as_v8 = [](const uint4& lo, const uint4& hi) -> v8i {
    return (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };

  v16f acc[C::TI][C::TJ];
  // Fragments: the A fragments of a slab live in one register set, each reloaded with the
  // next slab's data as soon as the MFMAs that use it have issued; the B fragments, used by
  // every MFMA of the slab, alternate between two sets.
  uint4 fa[2 * C::TI], fb0[2 * C::TJ], fb1[2 * C::TJ];

  // ---- current and next tile
  TileInfo cur = tile_info<C::BM, C::BN, GROUPED>(p, first, m_tiles, n_tiles, tiles_pp, mt_cap);
  TileDesc2 dc = tile_descs<C::BN>(p, cur, SPLITK ? KL : 0);
  int rb = 0;  // ring buffer that holds slab 0 of the current tile

  // A tile's scales and slabs 0..min(S, ktiles)-1 into ring buffers 0.., then (after the
  // wait) slab 0's fragments.
  auto prologue = [&](const TileInfo& t, TileDesc2 d, int region) {
    if (!loader) return;
    issue_scales(t, region);
    // An opaque zero keeps the compiler from computing these offsets once for all tiles
    // and holding them (or spilling them) across the whole tile loop.
    int s0 = 0;
    asm volatile("" : "+s"(s0));
#pragma unroll
    for (int s = 0; s < C::S; ++s)
      if (s < ktiles)
#pragma unroll
        for (int i = 0; i < C::LOADS; ++i) issue_one(d, s + s0, wave_lds(s), i);
  };
  // Wait for slab 0 of a tile (in ring buffer `buf`), then read its fragments.
  auto wait_read_first = [&](int buf) {
    if (loader) wait_slabs<C::LOADS, C::S - 1, false>((ktiles < C::S ? ktiles : C::S) - 1);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 2 * C::TI; ++r) fa[r] = read_a(smem + buf * C::STAGE, r);
#pragma unroll
    for (int r = 0; r < 2 * C::TJ; ++r) fb0[r] = read_b(smem + buf * C::STAGE, r);
  };
  prologue(cur, dc, 0);
  wait_read_first(0);

  using True = std::integral_constant<bool, true>;
  using False = std::integral_constant<bool, false>;

  for (int L = first, j = 0; L < last; L += stride, ++j) {
    const bool has_next = L + stride < last;
    TileInfo nxt = cur;
    TileDesc2 dn = dc;
    if (has_next) {
      nxt = tile_info<C::BM, C::BN, GROUPED>(p, L + stride, m_tiles, n_tiles, tiles_pp, mt_cap);
      dn = tile_descs<C::BN>(p, nxt, SPLITK ? KL : 0);
    }
    // With K of at least S slabs the last S steps fetch slabs 0..S-1 of the next tile.
    const bool pre = has_next && ktiles >= C::S;
    const int lim = pre ? ktiles + C::S : ktiles;  // slabs (from this tile's first) fetched here

    // Block scales (BLK): the wave's columns share one 128-column block, so its K-block scales
    // S[0..] form one row.  The accumulator is kept relative to the scale of the K block
    // being summed: between K blocks b - 1 and b (b >= 1) each MFMA tile's accumulator is
    // multiplied by S[b-1] / S[b], so after the last block it holds sum_b S[b] P_b / S[last]
    // and the epilogue's column scale is S[last].  A K block is two slabs: tile q's multiply
    // follows MFMA q + 1 of the block's last slab (the last tile's, MFMA 0 of the next
    // block's first slab), always after the tile's last MFMA of block b - 1 and before its
    // first of block b.  S[b + 1] is loaded in the first slab of block b, a slab before the
    // ratio needs it.
    const float* srow = nullptr;
    float s_prev = 1.0f, s_next = 1.0f, ratio = 1.0f;
    if constexpr (BLK) {
      const int kb = K / kScaleBlock, nbk = N / kScaleBlock;
      const int nb = min((cur.n0 + wn * C::WN) / kScaleBlock, nbk - 1);  // waves past N: any row
      srow = p.b_scale + ((int64_t)cur.expert * nbk + nb) * kb;
      s_prev = load_uniform_f(srow);
      if (kb > 1) s_next = load_uniform_f(srow + 1);
    }

    // One slab: wait for slab kt+1 and the reads of slab kt, barrier (slab kt's buffer is
    // then free for slab kt+S), then the MFMAs of slab kt interleaved with the fragment reads
    // of slab kt+1 and the direct-to-LDS loads of slab kt+S.  A single wave can issue only
    // about a dozen other instructions in the shadow of one 32x32x64 MFMA, so the
    // steady-state step (every slab involved complete, in range and in this tile) carries
    // no run-time conditions and no vector address arithmetic; the generic step handles the
    // last slabs, a ragged K and the fetches for the next tile.  The first step of a tile
    // starts its accumulators from zero.
    // `role`: 0 decided at run time, 1 a loader, 2 not a loader.
    // `resc` (block scales): 0 no rescale, 1 the last slab of a K block that another follows,
    // 2 the first slab of a K block after the first, 3 decided at run time.
    auto step = [&](auto steady, auto first_step, auto role, auto resc, int kt, uint4 (&bc)[2 * C::TJ],
                    uint4 (&bn)[2 * C::TJ]) {
      constexpr bool kSteady = decltype(steady)::value;
      constexpr bool kFirst = decltype(first_step)::value;
      constexpr int kRole = decltype(role)::value;
      constexpr int kResc = BLK ? decltype(resc)::value : 0;
      const bool resc_last = kResc == 1 || (kResc == 3 && (kt & 1) == 1 && kt + 1 < ktiles);
      const bool resc_first = kResc == 2 || (kResc == 3 && (kt & 1) == 0 && kt >= 2);
      if (BLK && resc_last) {
        ratio = __fdiv_rn(s_prev, s_next);
        s_prev = s_next;
      }
      if (BLK && resc_first && kt + 2 < ktiles) s_next = load_uniform_f(srow + (kt >> 1) + 1);
      const bool loads = kRole == 1 || (kRole == 0 && loader);
      bool has_read = true;
      int fetch = 1;  // 0: nothing, 1: slab kt+S of this tile, 2: slab kt+S-ktiles of the next
      if constexpr (kSteady) {
        if (loads) wait_vmcnt_lgkm0<(C::S - 2) * C::LOADS>();
        else wait_lgkm0();
      } else {
        if (loader) wait_slabs<C::LOADS, C::S - 2, true>(lim - kt - 2);  // slabs issued after kt+1
        else wait_lgkm0();
        has_read = kt + 1 < ktiles;
        fetch = !loader ? 0 : kt + C::S < ktiles ? 1 : (pre ? 2 : 0);
      }
      __syncthreads();
      const unsigned slot = (unsigned)(rb + kt);  // ring buffer of slab kt
      const uint8_t* Sn = smem + ((slot + 1) % C::S) * C::STAGE;
      const uint32_t lds_dst = wave_lds(slot % C::S);
      const uint32_t soff = (uint32_t)__builtin_amdgcn_readfirstlane((kt + C::S) * BK);
      if (!kSteady && fetch == 2 && kt + C::S == ktiles) issue_scales(nxt, (j + 1) & 1);
      int l = 0;
#pragma unroll
      for (int q = 0; q < kMfma; ++q) {
        const int i = q / C::TJ, jj = q % C::TJ;
        const v8i bf = as_v8(bc[2 * jj], bc[2 * jj + 1]);
        const v8i af = as_v8(fa[2 * i], fa[2 * i + 1]);
        if constexpr (kFirst)
          acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf, af, (v16f){}, 0, kFmtB, 0, 0, 0, 0);
        else
          acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf, af, acc[i][jj], 0, kFmtB, 0, 0, 0, 0);
        if constexpr (BLK) {
          if (resc_last && q >= 1) acc[(q - 1) / C::TJ][(q - 1) % C::TJ] *= ratio;
          if (resc_first && q == 0) acc[C::TI - 1][C::TJ - 1] *= ratio;
        }
        if (kSteady || has_read) {
          if (q < C::TJ) {
            bn[2 * q] = read_b(Sn, 2 * q);
            bn[2 * q + 1] = read_b(Sn, 2 * q + 1);
          }
          if (jj == C::TJ - 1) {
            fa[2 * i] = read_a(Sn, 2 * i);
            fa[2 * i + 1] = read_a(Sn, 2 * i + 1);
          }
        }
        // the slab's loads go out in kDmaGroups bursts after the first MFMAs (one role test
        // per burst)
        const int l_end = q < kDmaGroups ? (q + 1) * C::LOADS / kDmaGroups : C::LOADS;
        if constexpr (kSteady) {
          if (l < l_end && loads)
            for (; l < l_end; ++l) issue_full(dc, soff, lds_dst, l);
        }
        for (; l < l_end; ++l) {
          if constexpr (kSteady) {
          } else if (fetch != 0) {
            const bool nx = fetch == 2;
            issue_one(TileDesc2{pick(nx, dn.a, dc.a), pick(nx, dn.b, dc.b)}, nx ? kt + C::S - ktiles : kt + C::S,
                      lds_dst, l);
          }
        }
      }
      interleave_mfma_reads<0, kMfma, C::TJ, (kResc == 1 || kResc == 2) ? kResc : 0>();
    };

    using Any = std::integral_constant<int, 0>;
    using NoK = std::integral_constant<int, 0>;    // no rescale
    using LastK = std::integral_constant<int, 1>;  // last slab of a K block (kt odd)
    using NewK = std::integral_constant<int, 2>;   // first slab of a K block (kt even, kt >= 2)
    using RtK = std::integral_constant<int, 3>;    // decided at run time
    // A slab for a wave none of whose rows lies in the tile (whole waves past the valid rows
    // of an expert's or the matrix's last M-tile): the waits, the barrier and its share of
    // the loads, without the MFMAs and fragment reads that would only feed rows never stored.
    auto idle = [&](int kt) {
      if (loader) wait_slabs<C::LOADS, C::S - 2, true>(lim - kt - 2);
      else wait_lgkm0();
      const int fetch = !loader ? 0 : kt + C::S < ktiles ? 1 : (pre ? 2 : 0);
      __syncthreads();
      const uint32_t lds_dst = wave_lds((unsigned)(rb + kt) % C::S);
      if (fetch == 2 && kt + C::S == ktiles) issue_scales(nxt, (j + 1) & 1);
      if (fetch != 0) {
        const bool nx = fetch == 2;
        for (int l = 0; l < C::LOADS; ++l)
          issue_one(TileDesc2{pick(nx, dn.a, dc.a), pick(nx, dn.b, dc.b)}, nx ? kt + C::S - ktiles : kt + C::S,
                    lds_dst, l);
      }
    };
    const bool busy = cur.row_end - cur.row_begin > wm * C::WM;  // wave-uniform
    if (!busy) {
      for (int kt = 0; kt < ktiles; ++kt) idle(kt);
    } else {
      if (C::S < full_slabs) step(True{}, True{}, Any{}, NoK{}, 0, fb0, fb1);
      else step(False{}, True{}, Any{}, NoK{}, 0, fb0, fb1);
      int kt = 1;
      for (; kt + 1 + C::S < full_slabs; kt += 2) {  // kt and kt+1 steady: kt+1+S < full_slabs
        step(True{}, False{}, Any{}, LastK{}, kt, fb1, fb0);
        step(True{}, False{}, Any{}, NewK{}, kt + 1, fb0, fb1);
      }
      for (; kt + 1 < ktiles; kt += 2) {
        step(False{}, False{}, Any{}, RtK{}, kt, fb1, fb0);
        step(False{}, False{}, Any{}, RtK{}, kt + 1, fb0, fb1);
      }
      if (kt < ktiles) step(False{}, False{}, Any{}, RtK{}, kt, fb1, fb0);
    }
    // Every wave is past this tile's last barrier and no fragment read is pending, so the
    // ring is free unless `pre` already refilled it.
    if (has_next && !pre) prologue(nxt, dn, (j + 1) & 1);

    // ---- epilogue.  Lane: token row wm*WM + 32 i + (lane & 31); register group g of tile
    // (i, jj): columns wn*WN + 32 jj + 8 g + 4 half + 0..3, scaled and rounded to FP16.
    // GATE: MFMA tiles jj = 2 o and 2 o + 1 are the gate and up columns of the same 32
    // features, so output block o holds h = fl16(silu(g) * u) of those features (half the
    // columns; the row stride of y is N / 2).
    // Storers store their own blocks straight from registers: a 32-lane swap between column
    // groups g and g+1 gives each lane 8 consecutive columns (16 bytes) of its row.  With
    // SPLIT, loaders stage each 32-row block in an LDS strip shared with their storer; after
    // a barrier the storer reads it back as 16-byte chunks along the rows (whole 128-byte
    // row segments per store) and stores it; a second barrier frees the strip.
    if constexpr (SPLITK) {
      // FP32 part sums straight from registers: register group g of tile (i, jj) holds 4
      // consecutive columns of one row, one 16-byte store
      float* pt = p.partial + ((int64_t)cur.part * p.M + cur.row_begin) * N + cur.n0;
      const int rows = cur.row_end - cur.row_begin;
      const int erow = lane & 31, ehalf = lane >> 5;
#pragma unroll
      for (int i = 0; i < C::TI; ++i) {
        const int lrow = wm * C::WM + 32 * i + erow;
#pragma unroll
        for (int jj = 0; jj < C::TJ; ++jj)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = wn * C::WN + 32 * jj + 8 * g + 4 * ehalf;
            if (lrow < rows && cur.n0 + col < N) {
              const v16f& a = acc[i][jj];
              *reinterpret_cast<v4f*>(pt + (int64_t)lrow * N + col) =
                  (v4f){a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
            }
          }
      }
    } else {
      constexpr int kOutTJ = GATE ? C::TJ / 2 : C::TJ;  // 32-column output blocks per wave
      constexpr int kOutWN = 32 * kOutTJ;               // output columns per wave
      const int NO = GATE ? N / 2 : N;                   // output row length
      const int n0o = GATE ? cur.n0 / 2 : cur.n0;
      const float* sc = reinterpret_cast<const float*>(smem + C::SCALE_OFF + (j & 1) * C::SCALE_BYTES);
      const int partner = loader ? wave : wave - C::LOADERS;
      uint8_t* strip = smem + C::EPI_OFF + partner * C::STRIP;
      constexpr int kCpr = kOutWN / 8;  // 16-byte chunks per strip row
      int el = lane;                    // opaque copy: addressing is redone per tile, not hoisted
      asm volatile("" : "+v"(el));
      const int erow = el & 31, ehalf = el >> 5;  // MFMA output row and column half
      const int rows = cur.row_end - cur.row_begin;
      const int cols = NO - n0o;
      const int pwm = partner / C::WGN, pwn = partner % C::WGN;
      uint16_t* ytile = p.y + (int64_t)cur.row_begin * NO + n0o;
      // FP16 of register group g of tile (i, jj): 4 columns
      // the column scales of the wave's register groups, the same for every row block i: read
      // from LDS once per tile, ahead of the first multiply
      v4f sbv[C::TJ][4];
#pragma unroll
      for (int jj = 0; jj < C::TJ; ++jj)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          sbv[jj][g] = *reinterpret_cast<const v4f*>(sc + C::BM + wn * C::WN + 32 * jj + 8 * g + 4 * ehalf);
      auto group = [&](int i, int jj, int g, float sa) -> uint2 {
        const v4f& sb = sbv[jj][g];
        const v16f& a = acc[i][jj];
        uint2 v;
        v.x = pack_half2((a[4 * g] * sa) * sb[0], (a[4 * g + 1] * sa) * sb[1]);
        v.y = pack_half2((a[4 * g + 2] * sa) * sb[2], (a[4 * g + 3] * sa) * sb[3]);
        return v;
      };
      // the 4 output columns of register group g of output block o
      auto out_group = [&](int i, int o, int g, float sa) -> uint2 {
        if constexpr (GATE) {
          const uint2 gt = group(i, 2 * o, g, sa), up = group(i, 2 * o + 1, g, sa);
          return make_uint2(silu_mul_pair(gt.x, up.x), silu_mul_pair(gt.y, up.y));
        } else {
          return group(i, o, g, sa);
        }
      };
      // SPLIT: the gated output (half the columns) passes through the strips two row blocks at a
      // time, so one pair of barriers serves two blocks
      constexpr int kBlk = (GATE && C::SPLIT && C::TI % 2 == 0) ? 2 : 1;
      constexpr int kStride = kBlk == 2 ? C::GATE_STRIDE : C::EPI_STRIDE;
      static_assert(kBlk * 32 * kStride <= C::STRIP, "strip holds the blocks of one round");
#pragma unroll
      for (int i0 = 0; i0 < C::TI; i0 += kBlk) {
#pragma unroll
        for (int i = i0; i < i0 + kBlk; ++i) {
          const float sa = sc[wm * C::WM + 32 * i + erow];
          if (!storer) {
#pragma unroll
            for (int o = 0; o < kOutTJ; ++o)
#pragma unroll
              for (int g = 0; g < 4; ++g)
                *reinterpret_cast<uint2*>(strip + (32 * (i - i0) + erow) * kStride + 2 * (32 * o + 8 * g + 4 * ehalf)) =
                    out_group(i, o, g, sa);
          } else {
            const int lrow = wm * C::WM + 32 * i + erow;
            uint16_t* yrow = ytile + (int64_t)lrow * NO + wn * kOutWN + 8 * ehalf;
#pragma unroll
            for (int o = 0; o < kOutTJ; ++o) {
#pragma unroll
              for (int gp = 0; gp < 2; ++gp) {
                const uint2 x = out_group(i, o, 2 * gp, sa), y = out_group(i, o, 2 * gp + 1, sa);
                const auto s0 = __builtin_amdgcn_permlane32_swap(x.x, y.x, false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(x.y, y.y, false, false);
                const int col = wn * kOutWN + 32 * o + 16 * gp + 8 * ehalf;
                if (lrow < rows && col < cols)
                  st_global_16(yrow + 32 * o + 16 * gp, make_uint4(s0[0], s1[0], s0[1], s1[1]));
              }
            }
          }
        }
        if constexpr (C::SPLIT) {
          __syncthreads();
          if (!loader) {
#pragma unroll
            // chunk c of the round's strip rows: row c / kCpr (block r / 32 of the round, its
            // row r % 32), columns 8 (c % kCpr) ..
            for (int t = 0; t < 32 * kBlk * kCpr / 64; ++t) {
              const int c = el + 64 * t;
              const int r = c / kCpr, lc = 8 * (c % kCpr);
              const uint4 v = *reinterpret_cast<const uint4*>(strip + r * kStride + 2 * lc);
              const int orow = pwm * C::WM + 32 * i0 + r;
              if (orow < rows && lc < cols - pwn * kOutWN)
                st_global_16(ytile + (int64_t)orow * NO + pwn * kOutWN + lc, v);
            }
          }
          __syncthreads();
        }
      }
    }
    if (!has_next) break;
    cur = nxt;
    dc = dn;
    rb = pre ? (rb + ktiles) % C::S : 0;
    wait_read_first(rb);
  }
}

// Workgroups of this kernel the device keeps resident at once (all CUs), cached per device.
// The cache is read and filled with atomic operations, so concurrent calls from several
// host threads are safe: two threads may both compute the value, and both store the same one.
template <class C, bool GROUPED, bool GATE, bool BLK, bool A5, bool SPLITK>
int resident_workgroups() {
  constexpr int kDevices = 64;
  static std::atomic<int> cache[kDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  const int slot = dev < kDevices ? dev : kDevices - 1;
  const int known = cache[slot].load(std::memory_order_relaxed);
  if (known > 0) return known;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gemm_fp8_kernel<C, GROUPED, GATE, BLK, A5, SPLITK>,
                                                    C::NT, 0) != hipSuccess ||
      per_cu <= 0)
    per_cu = 1;
  const int value = cus * per_cu;
  if (dev < kDevices) cache[slot].store(value, std::memory_order_relaxed);  // devices past the table: no cache
  return value;
}

// RQ_GEMM_GRID=n caps the number of persistent workgroups (tests use it to give small
// problems many tiles per workgroup); unset or invalid: no cap.
int64_t grid_cap_override() {
  const char* e = std::getenv("RQ_GEMM_GRID");
  if (e == nullptr) return 0;
  const long v = std::strtol(e, nullptr, 10);
  return v > 0 ? (int64_t)v : 0;
}

template <class C, bool GROUPED, bool GATE, bool BLK, bool A5, bool SPLITK = false>
hipError_t launch_one(const GemmArgs& g, int m_tiles, hipStream_t stream) {
  const int n_tiles = (int)((g.N + C::BN - 1) / C::BN);
  // work items: tiles (grouped: the worst case), times the K parts with split-K
  const int64_t tiles = (int64_t)m_tiles * n_tiles * (SPLITK ? g.splits : 1);
  int64_t cap = resident_workgroups<C, GROUPED, GATE, BLK, A5, SPLITK>();
  const int64_t forced = grid_cap_override();
  if (forced > 0 && forced < cap) cap = forced;
  const int64_t want = (tiles + 7) / 8 * 8;
  const int64_t grid = want < cap ? want : cap;
  gemm_fp8_kernel<C, GROUPED, GATE, BLK, A5, SPLITK>
      <<<dim3((unsigned)grid), dim3(C::NT), 0, stream>>>(g, m_tiles, n_tiles);
  return hipGetLastError();
}

// Split-K reduce: adds the K parts of each output in part order (FP32) and applies the GEMM
// kernel's epilogue, y = fl16(fl32(fl32(acc * s_a[m]) * s_b[n])) with the same roundings, or
// with GATE h = silu_mul of the FP16 gate and up values (output block o of 32 features takes
// gate columns [64 o, 64 o + 32) and up columns [64 o + 32, 64 o + 64)).  One thread per 8
// output values: 16-byte loads of each part, one 16-byte store.
template <bool GATE>
__global__ __launch_bounds__(256) void splitk_reduce(const float* __restrict__ partial, int splits, int M, int N,
                                                     const float* __restrict__ a_scale,
                                                     const float* __restrict__ b_scale, int b_gran,
                                                     uint16_t* __restrict__ y) {
  const int NO = GATE ? N / 2 : N;
  const int per_row = NO / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)M * per_row) return;
  const int m = (int)(idx / per_row);
  const int c = 8 * (int)(idx % per_row);  // first output column
  const int64_t part_stride = (int64_t)M * N;
  const float sa = a_scale[m];
  // FP16 of the 8 columns starting at column n0 of the GEMM output
  auto columns = [&](int n0, uint32_t (&out)[4]) {
    const float* src = partial + (int64_t)m * N + n0;
    v4f lo = *reinterpret_cast<const v4f*>(src), hi = *reinterpret_cast<const v4f*>(src + 4);
    for (int s = 1; s < splits; ++s) {
      lo += *reinterpret_cast<const v4f*>(src + s * part_stride);
      hi += *reinterpret_cast<const v4f*>(src + s * part_stride + 4);
    }
    float sb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sb[i] = b_gran == kScaleTensor ? b_scale[0] : b_scale[n0 + i];
    out[0] = pack_half2((lo[0] * sa) * sb[0], (lo[1] * sa) * sb[1]);
    out[1] = pack_half2((lo[2] * sa) * sb[2], (lo[3] * sa) * sb[3]);
    out[2] = pack_half2((hi[0] * sa) * sb[4], (hi[1] * sa) * sb[5]);
    out[3] = pack_half2((hi[2] * sa) * sb[6], (hi[3] * sa) * sb[7]);
  };
  uint32_t v[4];
  if constexpr (GATE) {
    const int gcol = 64 * (c / 32) + c % 32;
    uint32_t g[4], u[4];
    columns(gcol, g);
    columns(gcol + 32, u);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = silu_mul_pair(g[i], u[i]);
  } else {
    columns(c, v);
  }
  *reinterpret_cast<uint4*>(y + (int64_t)m * NO + c) = make_uint4(v[0], v[1], v[2], v[3]);
}

hipError_t launch_splitk_reduce(const GemmArgs& g, hipStream_t stream) {
  const int64_t threads = (int64_t)g.M * ((g.gate ? g.N / 2 : g.N) / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (g.gate)
    splitk_reduce<true><<<grid, dim3(256), 0, stream>>>(g.partial, g.splits, g.M, g.N, g.a_scale, g.b_scale,
                                                        g.b_gran, g.y);
  else
    splitk_reduce<false><<<grid, dim3(256), 0, stream>>>(g.partial, g.splits, g.M, g.N, g.a_scale, g.b_scale,
                                                         g.b_gran, g.y);
  return hipGetLastError();
}

template <class C, bool GROUPED, bool BLK, bool A5>
hipError_t launch_gate(const GemmArgs& g, int m_tiles, hipStream_t stream) {
  if constexpr (C::TJ % 2 == 0) {
    if (g.gate) return launch_one<C, GROUPED, true, BLK, A5>(g, m_tiles, stream);
  } else {
    if (g.gate) return hipErrorInvalidValue;  // tile shapes with one 32-column block per wave
  }
  return launch_one<C, GROUPED, false, BLK, A5>(g, m_tiles, stream);
}

template <class C, bool GROUPED, bool A5>
hipError_t launch_fmt(const GemmArgs& g, int m_tiles, hipStream_t stream) {
  if (g.b_gran == kScaleBlock128) {
    if constexpr (kScaleBlock % C::WN == 0) return launch_gate<C, GROUPED, true, A5>(g, m_tiles, stream);
    else return hipErrorInvalidValue;  // a wave's columns would straddle two scale blocks
  }
  return launch_gate<C, GROUPED, false, A5>(g, m_tiles, stream);
}

template <class C, bool GROUPED>
hipError_t launch(const GemmArgs& g, int m_tiles, hipStream_t stream) {
  if (g.a_fmt == kFmtE5M2) return launch_fmt<C, GROUPED, true>(g, m_tiles, stream);
  return launch_fmt<C, GROUPED, false>(g, m_tiles, stream);
}

// Eight wavefronts (two per SIMD) for the large tiles: while one wavefront of a SIMD waits
// on a load issue, an LDS read or the barrier, the other keeps the matrix core busy.
// Measured on MI355X: +8% (256x256) and +5% (256x128) over four wavefronts of twice the
// tile each.  The 64-row tiles serve small M (the weight-streaming regime) and MoE experts
// with few rows, where 256-row tiles would spend most MFMA work on padding.
using Big = Cfg<256, 256, 4, 2, 4, true>;       // 128 KB ring, 128x64 per wavefront
using Wide = Cfg<256, 128, 4, 4, 2, true>;      // 96 KB ring, 64x64 per wavefront
using Small = Cfg<128, 128, 4, 2, 2, false>;    // 64 KB ring, two workgroups per CU
using Thin = Cfg<64, 128, 4, 1, 4, false>;      // 48 KB ring, three workgroups per CU
// 60 KB ring, two workgroups per CU.  A four-slab ring (80 KB plus the scale areas) leaves
// room for only one; measured on MI355X (top-2 of 32 experts), the three-slab ring with two
// resident workgroups is as fast on the 512-token MoE (gate/up 103.0 us, down 72 us) and, at
// 1024 tokens, 4% faster on the gate/up and 4% slower on the down projection.
using ThinWide = Cfg<64, 256, 3, 1, 4, false>;
// 112 KB ring, 64x96 per wavefront: three quarters of a 256x256 tile, for linears whose
// 256x256 tile count ends in a partly filled round (per-channel or per-tensor scales, plain
// output: a wavefront's 96 columns hold no gate/up pair and straddle 128-column scale blocks).
using Mid = Cfg<256, 192, 4, 4, 2, true>;
// 160 KB of LDS per CU: the resident workgroup counts above (and the grouped tile rule)
// depend on these sizes.
constexpr int kLdsPerCu = 160 * 1024;
static_assert(2 * Small::LDS <= kLdsPerCu && 3 * Thin::LDS <= kLdsPerCu && 2 * ThinWide::LDS <= kLdsPerCu,
              "workgroups per CU");

struct TileDesc {
  const char* name;
  int bm, bn;
};
const TileDesc kTiles[kTileKinds] = {
    {"256x256", 256, 256}, {"256x128", 256, 128}, {"128x128", 128, 128}, {"64x128", 64, 128}, {"64x256", 64, 256},
    {"256x192", 256, 192},
};

int tile_override() {
  const char* e = std::getenv("RQ_GEMM_TILE");
  if (e == nullptr) return -1;
  for (int k = 0; k < kTileKinds; ++k)
    if (std::strcmp(e, kTiles[k].name) == 0) return k;
  return -1;
}

// Pick the tile for a dense M x N problem cut into `splits` K parts: the largest tile (most
// operand reuse per byte loaded) whose work items (tiles x parts) still occupy the 256 CUs,
// else the thinnest.  Split-K runs only on the tiles whose every wave stores (128x128 and
// smaller), and there a taller tile is skipped when it pads the rows by more than an eighth
// beyond 64-row tiles; a 256x256 pick may then become 256x192 (below).  On MI355X the rule
// picked the fastest of the other five shapes for every linear of the workloads (measured at
// M = 512 and M = 4096).  Split cases, measured
// (slab weights, caches flushed): 512 x 2048 x 8192 in 4 parts 29.4 -> 26.3 us and
// 256 x 4096 x 8192 31.0 -> 27.2 us on 128x128 tiles; 300 x 6144 x 4096 stays on 64x128
// (31.7 us; 34.7 us on 128x128, whose third M-tile is a third full).
int pick_dense(int64_t M, int64_t N, bool gate, bool blocks, int splits) {
  const int forced = tile_override();
  const bool mid_ok = !gate && !blocks && splits == 1;  // what the 256x192 tile serves
  if (forced >= 0 && !(gate && forced == kTileThin) && !(forced == kTileMid && !mid_ok)) return forced;
  const int order[] = {kTileBig, kTileWide, kTileSmall, kTileThin};
  auto padded = [&](int o) { return (M + kTiles[o].bm - 1) / kTiles[o].bm * kTiles[o].bm; };
  for (int o : order) {
    if (splits > 1 && (o == kTileBig || o == kTileWide)) continue;
    if (splits > 1 && o != kTileThin && padded(o) * 8 > padded(kTileThin) * 9) continue;
    const TileDesc& d = kTiles[o];
    const int64_t tiles = ((M + d.bm - 1) / d.bm) * ((N + d.bn - 1) / d.bn) * splits;
    if (tiles < 192) continue;
    // 256x256 tiles that end in a partly filled round of the 256 CUs: 256x192 tiles whose
    // rounds, at 7/8 of the time each (three quarters of the MFMA work, 7/8 of the operand
    // bytes), take less time.  4096 x 6144: 384 tiles (2 rounds) -> 512 tiles (2 rounds).
    if (o == kTileBig && mid_ok && N % 192 == 0) {
      const int64_t mid = ((M + 255) / 256) * (N / 192);
      if ((mid + 255) / 256 * 7 < (tiles + 255) / 256 * 8) return kTileMid;
    }
    return gate && o == kTileThin ? kTileThinWide : o;
  }
  // a gated output needs both 32-column blocks of a feature group in one wavefront
  return gate ? kTileThinWide : kTileThin;
}

template <class C>
hipError_t launch_dense(const GemmArgs& g, hipStream_t stream) {
  const int m_tiles = (int)((g.M + C::BM - 1) / C::BM);
  if constexpr (!C::SPLIT) {
    // split-K: the GEMM writes FP32 part sums (plain output, the operand format picks the
    // instantiation), then the reduce kernel applies the epilogue
    if (g.splits > 1 && g.partial != nullptr && g.b_gran != kScaleBlock128) {
      const hipError_t e = g.a_fmt == kFmtE5M2 ? launch_one<C, false, false, false, true, true>(g, m_tiles, stream)
                                               : launch_one<C, false, false, false, false, true>(g, m_tiles, stream);
      if (e != hipSuccess) return e;
      return launch_splitk_reduce(g, stream);
    }
  }
  GemmArgs one = g;
  one.splits = 1;
  return launch<C, false>(one, m_tiles, stream);
}

}  // namespace

int pick_grouped(int64_t R, int64_t E, int64_t N, bool gate) {
  const int forced = tile_override();
  if (forced == kTileBig || forced == kTileThinWide || (forced == kTileThin && !gate)) return forced;
  // Rounds of resident workgroups (256 CUs; one 256x256 or two 64x256 workgroups per CU)
  // each shape needs, counting a whole extra M-tile for each expert (its last, partial one:
  // under skewed loads most experts fit in one partial tile).  A tile's K loop costs about
  // the same in both shapes (measured), so fewer rounds win; ties go to the 256-row tiles,
  // which read each expert's weights fewer times.  Measured on MI355X over 384-3072 tokens,
  // top-2 of 32 Zipf-loaded experts: counting half an extra tile per expert kept 256-row
  // tiles at 1024 tokens, where they spill into a second round (down projection 99 us
  // against 70 us with 64-row tiles); counting a whole one picks the faster or an equal
  // shape at every measured point but 1536 tokens, which it leaves as before.
  const int64_t nonempty = E < R ? E : R;
  auto rounds = [&](int bm, int bn, int per_cu) {
    const int64_t tiles = ((R + bm - 1) / bm + nonempty) * ((N + bn - 1) / bn);
    const int64_t cap = 256 * per_cu;
    return (tiles + cap - 1) / cap;
  };
  if (rounds(256, 256, 1) <= rounds(64, 256, 2)) return kTileBig;
  // Few routed rows (the weight-streaming regime): while the 64x256 tiles leave resident slots
  // idle and the 64x128 tiles, three per CU, still fit one round, the plain (ungated) output
  // takes 64x128 tiles - twice the workgroups streaming weights.  Measured on MI355X, 512
  // tokens, top-2 of 32 Zipf-loaded experts, down projection: 71.4 -> 64.7 us; at 1024 tokens
  // the 64x256 tiles fill a round and stay.
  auto tiles = [&](int bm, int bn) { return ((R + bm - 1) / bm + nonempty) * ((N + bn - 1) / bn); };
  if (!gate && tiles(64, 256) < 256 * 2 && tiles(64, 128) <= 256 * 3) return kTileThin;
  return kTileThinWide;
}

int tile_rows(int kind) { return kTiles[kind].bm; }

// Split-K for small M (the weight-streaming regime): a GEMM with few tiles keeps only part of
// the 256 CUs streaming weights, each over a long K loop.  Cutting K into s equal parts (s a
// power of two up to 8) multiplies the work items while the 64 x 128 tile count stays within
// three per CU and every part keeps at least 32 slabs of 64 bytes: the FP32 part sums cost
// 8 s M N bytes of traffic (written, then read by the reduce), which only a long K loop
// repays (measured on the 512-row layer: K = 8192 gains 34%, K = 2048 loses 20-60%).  It
// depends on M, N and K only - not on the output form - so the gated and the plain gate/up
// linear sum K the same way.
int dense_splits(int64_t M, int64_t N, int64_t K, int act, int w_gran) {
  (void)act;
  if (w_gran == kScaleBlock128 || M > 1024 || K % BK != 0) return 1;
  const int64_t base = ((M + 63) / 64) * ((N + 127) / 128);
  const int64_t slabs = K / BK;
  int s = 1;
  while (s < 8 && base * s * 2 <= 3 * 256 && slabs % (2 * s) == 0 && slabs / (2 * s) >= 32) s *= 2;
  return s;
}

size_t dense_partial_bytes(int64_t M, int64_t N, int64_t K, int act, int w_gran) {
  const int s = dense_splits(M, N, K, act, w_gran);
  return s > 1 ? (size_t)s * (size_t)M * (size_t)N * sizeof(float) : 0;
}

int64_t grouped_max_mtiles(int64_t R, int64_t E, int tile_m) { return (R + tile_m - 1) / tile_m + E; }

hipError_t launch_gemm_dense(const GemmArgs& g, hipStream_t stream) {
  if (g.M <= 0) return hipSuccess;
  // the K parts the launch will run (launch_dense splits only with a partial-sum buffer and
  // per-channel or per-tensor scales)
  const int splits = g.splits > 1 && g.partial != nullptr && g.b_gran != kScaleBlock128 ? g.splits : 1;
  switch (pick_dense(g.M, g.N, g.gate != 0, g.b_gran == kScaleBlock128, splits)) {
    case kTileBig: return launch_dense<Big>(g, stream);
    case kTileWide: return launch_dense<Wide>(g, stream);
    case kTileMid: return launch_dense<Mid>(g, stream);
    case kTileSmall: return launch_dense<Small>(g, stream);
    case kTileThin: return launch_dense<Thin>(g, stream);
    default: return launch_dense<ThinWide>(g, stream);
  }
}

hipError_t launch_gemm_grouped(const GemmArgs& g, int kind, hipStream_t stream) {
  if (g.M <= 0) return hipSuccess;
  if (kind == kTileThinWide)
    return launch<ThinWide, true>(g, (int)grouped_max_mtiles(g.M, g.E, ThinWide::BM), stream);
  if (kind == kTileThin) return launch<Thin, true>(g, (int)grouped_max_mtiles(g.M, g.E, Thin::BM), stream);
  return launch<Big, true>(g, (int)grouped_max_mtiles(g.M, g.E, Big::BM), stream);
}

}  // namespace rq
