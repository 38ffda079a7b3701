// C ABI of the gfx950 W8A8 FP8 library: argument validation, workspace layout and the
// launch sequence of each entry point.  The operations are specified in rq_fp8.h.

#include <atomic>
#include <climits>
#include <cstring>
#include <mutex>

#include "rq_fp8.h"
#include "common.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kMaxExperts = 1024;
constexpr int kMaxDevices = 64;
constexpr int64_t kMaxOperandBytes = ((int64_t)1 << 31) - 1;  // 32-bit buffer offsets
constexpr int64_t kMaxK = (int64_t)1 << 22;  // rows just past a tile edge stay out of range

// One-shot per-thread timing hooks (rq_time_next_kernel).
thread_local hipEvent_t t_hook_start[RQ_KERNEL_KINDS] = {};
thread_local hipEvent_t t_hook_stop[RQ_KERNEL_KINDS] = {};

struct Hook {
  int kind;
  hipStream_t stream;
  bool armed;
  Hook(int k, hipStream_t s) : kind(k), stream(s), armed(t_hook_start[k] != nullptr) {
    if (armed) (void)hipEventRecord(t_hook_start[kind], stream);
  }
  ~Hook() {
    if (armed) {
      (void)hipEventRecord(t_hook_stop[kind], stream);
      t_hook_start[kind] = nullptr;
      t_hook_stop[kind] = nullptr;
    }
  }
};

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Per-device arch cache: 0 unknown, 1 gfx950, 2 other.
std::atomic<int> g_arch[kMaxDevices];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return RQ_ERR_HIP;
  const int r = rq_device_supported(dev);
  if (r < 0) return RQ_ERR_HIP;
  return r == 1 ? RQ_OK : RQ_ERR_UNSUPPORTED;
}

struct Carve {
  uint8_t* base;
  size_t used = 0;
  template <typename T>
  T* take(size_t bytes) {
    T* p = reinterpret_cast<T*>(base + used);
    used += align_up(bytes);
    return p;
  }
};

// MoE workspace: the routing plan first, at offsets that depend only on (T, top_k, E), so a
// later call with the same routing can reuse it from the same workspace (RQ_MOE_PLAN_READY);
// then the quantized GEMM operand and, for the combined output, the permuted GEMM output.
struct MoeLayout {
  size_t offsets, tile_start[2], tile_table[2], perm, pos, block_hist;  // the plan
  size_t a_q, a_scale, y_perm;
};

constexpr int kPlanTileRows[2] = {rq::kMinTileRows, 256};  // the grouped GEMM's tile heights

MoeLayout moe_layout(int64_t T, int top_k, int64_t E, int64_t N, int64_t K, int act, int out_layout) {
  const int64_t R = T * top_k;
  MoeLayout l;
  l.offsets = (size_t)(E + 1) * sizeof(int32_t);
  for (int i = 0; i < 2; ++i) {
    l.tile_start[i] = (size_t)(E + 1) * sizeof(int32_t);
    l.tile_table[i] = (size_t)rq::grouped_max_mtiles(R, E, kPlanTileRows[i]) * 4 * sizeof(int32_t);
  }
  l.perm = (size_t)R * sizeof(int32_t);
  l.pos = (size_t)R * sizeof(int32_t);
  l.block_hist = (size_t)(rq::moe_plan_blocks(R) * E) * sizeof(int32_t);
  l.a_q = (size_t)(R * K);  // the GEMM operand: one quantized row per routed slot
  l.a_scale = (size_t)R * sizeof(float);
  const int64_t NO = act == RQ_ACT_GATE_SILU ? N / 2 : N;  // output row length
  l.y_perm = out_layout == RQ_MOE_OUT_COMBINED ? (size_t)(R * NO) * sizeof(uint16_t) : 0;
  return l;
}

size_t plan_bytes(const MoeLayout& l) {
  return align_up(l.offsets) + align_up(l.tile_start[0]) + align_up(l.tile_start[1]) + align_up(l.tile_table[0]) +
         align_up(l.tile_table[1]) + align_up(l.perm) + align_up(l.pos) + align_up(l.block_hist);
}

// Device scratch of the allocation-free linear (rq_fp8_linear_noalloc): the quantized
// activation rows and their scales.  Each GPU the library runs on holds its own copy, for the
// life of the process.  In host code `scratch` is only a host-side stand-in for the symbol:
// its device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) uint8_t scratch[RQ_STATIC_SCRATCH_BYTES];

// Per-device address of `scratch` (resolved on a call's first use of a device, with that
// device current).  g_scratch_state: 0 not resolved, 1 resolved, 2 failed.
std::mutex g_scratch_mutex;
std::atomic<int> g_scratch_state[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

int static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return RQ_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return RQ_ERR_UNSUPPORTED;
  int state = g_scratch_state[dev].load(std::memory_order_acquire);
  if (state == 0) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    state = g_scratch_state[dev].load(std::memory_order_relaxed);
    if (state == 0) {
      void* ptr = nullptr;
      const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      g_scratch_ptr[dev] = ptr;
      state = (e == hipSuccess && ptr != nullptr) ? 1 : 2;
      g_scratch_state[dev].store(state, std::memory_order_release);
    }
  }
  if (state != 1) return RQ_ERR_HIP;
  *out = g_scratch_ptr[dev];
  return RQ_OK;
}

}  // namespace

extern "C" {

const char* rq_status_string(int status) {
  switch (status) {
    case RQ_OK: return "ok";
    case RQ_ERR_NULL: return "null pointer";
    case RQ_ERR_SHAPE: return "unsupported shape";
    case RQ_ERR_ALIGN: return "misaligned size or pointer";
    case RQ_ERR_WORKSPACE: return "workspace too small";
    case RQ_ERR_UNSUPPORTED: return "device is not gfx950";
    case RQ_ERR_HIP: return "HIP runtime error";
    case RQ_ERR_ARG: return "invalid argument";
    case RQ_ERR_SCRATCH: return "request exceeds the static scratch buffer";
    default: return "unknown status";
  }
}

int rq_time_next_kernel(int kernel, void* start_event, void* stop_event) {
  if (kernel < 0 || kernel >= RQ_KERNEL_KINDS) return RQ_ERR_ARG;
  if ((start_event == nullptr) != (stop_event == nullptr)) return RQ_ERR_NULL;
  t_hook_start[kernel] = (hipEvent_t)start_event;
  t_hook_stop[kernel] = (hipEvent_t)stop_event;
  return RQ_OK;
}

int rq_debug_flag(int clear) {
  unsigned int flags = 0;
  if (rq::read_error_flags(&flags, clear != 0) != hipSuccess) return -1;
  return (int)(flags & 0x7FFFFFFFu);
}

int rq_device_supported(int device) {
  if (device < 0) return -1;
  if (device < kMaxDevices) {
    const int c = g_arch[device].load(std::memory_order_relaxed);
    if (c != 0) return c == 1 ? 1 : 0;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return -1;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (device < kMaxDevices) g_arch[device].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? 1 : 0;
}

int rq_fp8_quant_weights_ex(const uint16_t* w, int64_t B, int64_t N, int64_t K, int w_gran, uint8_t* w_q,
                            float* w_scale, void* stream) {
  if (w_gran != RQ_WSCALE_CHANNEL && w_gran != RQ_WSCALE_TENSOR && w_gran != RQ_WSCALE_BLOCK128) return RQ_ERR_ARG;
  if (B < 0 || N < 0 || K <= 0) return RQ_ERR_SHAPE;
  if (K % 16 != 0) return RQ_ERR_ALIGN;
  if (w_gran == RQ_WSCALE_BLOCK128 && (N % rq::kScaleBlock != 0 || K % rq::kScaleBlock != 0)) return RQ_ERR_ALIGN;
  if (B > 0 && N > 0 && B > INT64_MAX / N) return RQ_ERR_SHAPE;
  const int64_t rows = B * N;
  if (rows == 0) return RQ_OK;
  if (!w || !w_q || !w_scale) return RQ_ERR_NULL;
  if (!aligned(w, 16) || !aligned(w_q, 16) || !aligned(w_scale, 4)) return RQ_ERR_ALIGN;
  const int dev = check_device();
  if (dev != RQ_OK) return dev;
  Hook hook(RQ_KERNEL_QUANT, (hipStream_t)stream);
  hipError_t e;
  if (w_gran == RQ_WSCALE_TENSOR)
    e = rq::launch_quant_tensor(w, B, N, K, w_q, w_scale, (hipStream_t)stream);
  else if (w_gran == RQ_WSCALE_BLOCK128)
    e = rq::launch_quant_blocks(w, B, N, K, w_q, w_scale, (hipStream_t)stream);
  else
    e = rq::launch_quant_rows(w, rows, K, RQ_ACT_NONE, w_q, w_scale, nullptr, nullptr, 0, (hipStream_t)stream);
  return e == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}

int rq_fp8_quant_weights(const uint16_t* w, int64_t B, int64_t N, int64_t K, uint8_t* w_q,
                         float* w_scale, void* stream) {
  return rq_fp8_quant_weights_ex(w, B, N, K, RQ_WSCALE_CHANNEL, w_q, w_scale, stream);
}

int rq_fp8_pack_weights(const uint8_t* w_q, int64_t B, int64_t N, int64_t K, uint8_t* w_packed, void* stream) {
  if (B < 0 || N < 0 || K <= 0) return RQ_ERR_SHAPE;
  if (K % 64 != 0) return RQ_ERR_ALIGN;
  if (N > 0 && B > INT64_MAX / N / K) return RQ_ERR_SHAPE;
  if (B * N == 0) return RQ_OK;
  if (!w_q || !w_packed) return RQ_ERR_NULL;
  if (w_q == w_packed) return RQ_ERR_ARG;
  if (!aligned(w_q, 16) || !aligned(w_packed, 16)) return RQ_ERR_ALIGN;
  const int dev = check_device();
  if (dev != RQ_OK) return dev;
  return rq::launch_pack_slabs(w_q, B, N, K, w_packed, (hipStream_t)stream) == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}

size_t rq_fp8_linear_workspace_size(int64_t M, int64_t K, int act) {
  (void)act;
  if (M < 0 || K <= 0) return 0;
  return align_up((size_t)(M * K)) + align_up((size_t)M * sizeof(float));
}

size_t rq_fp8_linear_workspace_size_ex(int64_t M, int64_t N, int64_t K, int act) {
  if (M < 0 || K <= 0 || N <= 0) return 0;
  return rq_fp8_linear_workspace_size(M, K, act) + align_up(rq::dense_partial_bytes(M, N, K, act, RQ_WSCALE_CHANNEL));
}

int rq_fp8_linear_ex(const uint16_t* x, int64_t M, int64_t K, int act, int a_fmt, const uint8_t* w_q,
                     const float* w_scale, int w_gran, int64_t N, uint16_t* y, void* workspace,
                     size_t workspace_bytes, const rq_debug_out* dbg, void* stream) {
  if (act != RQ_ACT_NONE && act != RQ_ACT_SILU_MUL && act != RQ_ACT_GATE_SILU) return RQ_ERR_ARG;
  if (a_fmt != RQ_FP8_E4M3 && a_fmt != RQ_FP8_E5M2) return RQ_ERR_ARG;
  const bool slabs = (w_gran & RQ_WLAYOUT_SLABS) != 0;
  w_gran &= ~RQ_WLAYOUT_SLABS;
  if (w_gran != RQ_WSCALE_CHANNEL && w_gran != RQ_WSCALE_TENSOR && w_gran != RQ_WSCALE_BLOCK128) return RQ_ERR_ARG;
  if (M < 0 || K <= 0 || N <= 0) return RQ_ERR_SHAPE;
  if (K % 16 != 0 || N % 16 != 0 || (act == RQ_ACT_GATE_SILU && N % 64 != 0)) return RQ_ERR_ALIGN;
  if (slabs && K % 64 != 0) return RQ_ERR_ALIGN;
  if (w_gran == RQ_WSCALE_BLOCK128 && (N % rq::kScaleBlock != 0 || K % rq::kScaleBlock != 0)) return RQ_ERR_ALIGN;
  if (K > kMaxK || N > (int64_t)1 << 30 || M > (int64_t)1 << 31) return RQ_ERR_SHAPE;
  if (M * K > kMaxOperandBytes || N * K > kMaxOperandBytes) return RQ_ERR_SHAPE;
  if (!w_q || !w_scale) return RQ_ERR_NULL;
  if (M > 0 && (!x || !y)) return RQ_ERR_NULL;
  uint8_t* dq = dbg ? dbg->a_q : nullptr;
  float* ds = dbg ? dbg->a_scale : nullptr;
  uint16_t* dh = dbg ? dbg->h : nullptr;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(w_q, 16) || !aligned(w_scale, 4) ||
      !aligned(workspace, 16) || !aligned(dq, 16) || !aligned(ds, 4) || !aligned(dh, 16))
    return RQ_ERR_ALIGN;
  const size_t need_q = dq ? 0 : align_up((size_t)(M * K));
  const size_t need_s = ds ? 0 : align_up((size_t)M * sizeof(float));
  if (need_q + need_s > 0 && (!workspace || workspace_bytes < need_q + need_s))
    return M == 0 ? RQ_OK : RQ_ERR_WORKSPACE;
  if (M == 0) return RQ_OK;
  const int dev = check_device();
  if (dev != RQ_OK) return dev;

  Carve c{reinterpret_cast<uint8_t*>(workspace)};
  uint8_t* xq = dq ? dq : c.take<uint8_t>((size_t)(M * K));
  float* sx = ds ? ds : c.take<float>((size_t)M * sizeof(float));
  // split-K partial sums when the workspace holds them (see rq_fp8_linear_workspace_size_ex)
  const size_t part_bytes = rq::dense_partial_bytes(M, N, K, act, w_gran);
  float* partial = nullptr;
  if (part_bytes > 0 && workspace != nullptr && workspace_bytes >= c.used + part_bytes)
    partial = c.take<float>(part_bytes);
  hipStream_t s = (hipStream_t)stream;
  {
    Hook hook(RQ_KERNEL_QUANT, s);
    const int in_act = act == RQ_ACT_SILU_MUL ? RQ_ACT_SILU_MUL : RQ_ACT_NONE;
    if (rq::launch_quant_rows(x, M, K, in_act, xq, sx, act == RQ_ACT_SILU_MUL ? dh : nullptr, nullptr, 0, s,
                              a_fmt) != hipSuccess)
      return RQ_ERR_HIP;
  }
  rq::GemmArgs g{};
  g.a = xq;
  g.a_scale = sx;
  g.b = w_q;
  g.b_scale = w_scale;
  g.y = y;
  g.M = (int32_t)M;  // sizes validated above: every product fits 31 bits
  g.a_rows = (int32_t)M;
  g.N = (int32_t)N;
  g.K = (int32_t)K;
  g.E = 1;
  g.gate = act == RQ_ACT_GATE_SILU ? 1 : 0;
  g.b_gran = w_gran;
  g.a_fmt = a_fmt;
  g.splits = partial != nullptr ? rq::dense_splits(M, N, K, act, w_gran) : 1;
  g.partial = partial;
  g.b_slabs = slabs ? 1 : 0;
  Hook hook(RQ_KERNEL_GEMM, s);
  return rq::launch_gemm_dense(g, s) == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}

int rq_fp8_linear(const uint16_t* x, int64_t M, int64_t K, int act, const uint8_t* w_q,
                  const float* w_scale, int64_t N, uint16_t* y, void* workspace,
                  size_t workspace_bytes, const rq_debug_out* dbg, void* stream) {
  return rq_fp8_linear_ex(x, M, K, act, RQ_FP8_E4M3, w_q, w_scale, RQ_WSCALE_CHANNEL, N, y, workspace,
                          workspace_bytes, dbg, stream);
}

int rq_fp8_linear_noalloc(const uint16_t* x, int64_t M, int64_t K, int act, const uint8_t* w_q,
                          const float* w_scale, int64_t N, uint16_t* y, void* stream) {
  if (M < 0 || K <= 0 || N <= 0) return RQ_ERR_SHAPE;
  if (M == 0)  // validates the remaining arguments and enqueues nothing
    return rq_fp8_linear_ex(x, M, K, act, RQ_FP8_E4M3, w_q, w_scale, RQ_WSCALE_CHANNEL, N, y, nullptr, 0,
                            nullptr, stream);
  if (K > kMaxK || M > (int64_t)1 << 31) return RQ_ERR_SHAPE;
  if (rq_fp8_linear_workspace_size(M, K, act) > (size_t)RQ_STATIC_SCRATCH_BYTES) return RQ_ERR_SCRATCH;
  void* ptr = nullptr;
  const int st = static_scratch(&ptr);
  if (st != RQ_OK) return st;
  return rq_fp8_linear_ex(x, M, K, act, RQ_FP8_E4M3, w_q, w_scale, RQ_WSCALE_CHANNEL, N, y, ptr,
                          (size_t)RQ_STATIC_SCRATCH_BYTES, nullptr, stream);
}

size_t rq_fp8_moe_workspace_size(int64_t T, int top_k, int64_t E, int64_t N, int64_t K,
                                 int in_layout, int act, int out_layout) {
  (void)in_layout;
  if (T < 0 || top_k < 1 || E < 1 || N <= 0 || K <= 0) return 0;
  const MoeLayout l = moe_layout(T, top_k, E, N, K, act, out_layout);
  return plan_bytes(l) + align_up(l.a_q) + align_up(l.a_scale) + align_up(l.y_perm);
}

int rq_fp8_moe_grouped_linear_ex(const uint16_t* x, int in_layout, int act, int a_fmt, const int32_t* topk_ids,
                                 const uint16_t* topk_w, int64_t T, int top_k, const uint8_t* w_q,
                                 const float* w_scale, int w_gran, int64_t E, int64_t N, int64_t K, uint16_t* y,
                                 int out_layout, void* workspace, size_t workspace_bytes,
                                 const rq_debug_out* dbg, void* stream) {
  if (act != RQ_ACT_NONE && act != RQ_ACT_SILU_MUL && act != RQ_ACT_GATE_SILU) return RQ_ERR_ARG;
  const bool slabs = (w_gran & RQ_WLAYOUT_SLABS) != 0;
  w_gran &= ~RQ_WLAYOUT_SLABS;
  if (w_gran != RQ_WSCALE_CHANNEL && w_gran != RQ_WSCALE_TENSOR && w_gran != RQ_WSCALE_BLOCK128) return RQ_ERR_ARG;
  if (a_fmt != RQ_FP8_E4M3 && a_fmt != RQ_FP8_E5M2) return RQ_ERR_ARG;
  // RQ_MOE_PLAN_READY: reuse the plan in the workspace (permuted input only: a token input
  // would scatter rows through the plan's slot positions)
  const bool plan_ready = (in_layout & RQ_MOE_PLAN_READY) != 0;
  in_layout &= ~RQ_MOE_PLAN_READY;
  if (in_layout != RQ_MOE_IN_TOKENS && in_layout != RQ_MOE_IN_PERMUTED) return RQ_ERR_ARG;
  if (plan_ready && in_layout != RQ_MOE_IN_PERMUTED) return RQ_ERR_ARG;
  if (out_layout != RQ_MOE_OUT_PERMUTED && out_layout != RQ_MOE_OUT_COMBINED) return RQ_ERR_ARG;
  if (T < 0 || K <= 0 || N <= 0 || E < 1 || E > kMaxExperts || top_k < 1 || top_k > E)
    return RQ_ERR_SHAPE;
  if (K % 16 != 0 || N % 16 != 0 || (act == RQ_ACT_GATE_SILU && N % 64 != 0)) return RQ_ERR_ALIGN;
  if (w_gran == RQ_WSCALE_BLOCK128 && (N % rq::kScaleBlock != 0 || K % rq::kScaleBlock != 0)) return RQ_ERR_ALIGN;
  if (slabs && K % 64 != 0) return RQ_ERR_ALIGN;
  if (K > kMaxK || N > (int64_t)1 << 30 || T * top_k > ((int64_t)1 << 31) - 1)
    return RQ_ERR_SHAPE;
  if (T * top_k * K > kMaxOperandBytes || N * K > kMaxOperandBytes) return RQ_ERR_SHAPE;
  if (!w_q || !w_scale) return RQ_ERR_NULL;
  if (T > 0 && (!x || !y || !topk_ids)) return RQ_ERR_NULL;
  if (T > 0 && out_layout == RQ_MOE_OUT_COMBINED && !topk_w) return RQ_ERR_ARG;
  uint8_t* dq = dbg ? dbg->a_q : nullptr;
  float* ds = dbg ? dbg->a_scale : nullptr;
  uint16_t* dh = dbg ? dbg->h : nullptr;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(w_q, 16) || !aligned(w_scale, 4) ||
      !aligned(topk_ids, 4) || !aligned(topk_w, 2) || !aligned(workspace, 16) || !aligned(dq, 16) ||
      !aligned(ds, 4) || !aligned(dh, 16))
    return RQ_ERR_ALIGN;
  if (T == 0) return RQ_OK;
  const size_t need = rq_fp8_moe_workspace_size(T, top_k, E, N, K, in_layout, act, out_layout);
  if (!workspace || workspace_bytes < need) return RQ_ERR_WORKSPACE;
  const int dev = check_device();
  if (dev != RQ_OK) return dev;

  const int64_t R = T * top_k;
  const int64_t rows = in_layout == RQ_MOE_IN_TOKENS ? T : R;
  const MoeLayout l = moe_layout(T, top_k, E, N, K, act, out_layout);
  Carve c{reinterpret_cast<uint8_t*>(workspace)};
  int32_t* offsets = c.take<int32_t>(l.offsets);
  rq::TileTables tt;
  for (int i = 0; i < 2; ++i) {
    tt.rows[i] = kPlanTileRows[i];
    tt.start[i] = c.take<int32_t>(l.tile_start[i]);
  }
  for (int i = 0; i < 2; ++i) tt.table[i] = c.take<int32_t>(l.tile_table[i]);
  int32_t* perm = c.take<int32_t>(l.perm);
  int32_t* pos = c.take<int32_t>(l.pos);
  int32_t* block_hist = c.take<int32_t>(l.block_hist);
  uint8_t* aq = c.take<uint8_t>(l.a_q);
  float* as = c.take<float>(l.a_scale);
  uint16_t* y_perm = out_layout == RQ_MOE_OUT_COMBINED ? c.take<uint16_t>(l.y_perm) : y;
  if (dq) aq = dq;
  if (ds) as = ds;

  hipStream_t s = (hipStream_t)stream;
  const int kind = rq::pick_grouped(R, E, N, act == RQ_ACT_GATE_SILU);
  const int which = rq::tile_rows(kind) == kPlanTileRows[0] ? 0 : 1;
  if (!plan_ready && rq::launch_moe_plan(topk_ids, T, top_k, E, offsets, tt, perm, pos, block_hist, s) != hipSuccess)
    return RQ_ERR_HIP;
  int32_t* tile_start = tt.start[which];
  int32_t* tile_table = tt.table[which];
  {
    Hook hook(RQ_KERNEL_QUANT, s);
    // per-token rows are written to each of the token's permuted slots
    const bool tokens = in_layout == RQ_MOE_IN_TOKENS;
    const int in_act = act == RQ_ACT_SILU_MUL ? RQ_ACT_SILU_MUL : RQ_ACT_NONE;
    if (rq::launch_quant_rows(x, rows, K, in_act, aq, as, act == RQ_ACT_SILU_MUL ? dh : nullptr,
                              tokens ? pos : nullptr, tokens ? top_k : 0, s, a_fmt) != hipSuccess)
      return RQ_ERR_HIP;
  }
  rq::GemmArgs g{};
  g.a = aq;
  g.a_scale = as;
  g.b = w_q;
  g.b_scale = w_scale;
  g.y = y_perm;
  g.M = (int32_t)R;  // sizes validated above: every product fits 31 bits
  g.a_rows = (int32_t)R;
  g.N = (int32_t)N;
  g.K = (int32_t)K;
  g.splits = 1;
  g.tile_start = tile_start;
  g.tile_table = tile_table;
  g.E = (int32_t)E;
  g.gate = act == RQ_ACT_GATE_SILU ? 1 : 0;
  g.b_gran = w_gran;
  g.a_fmt = a_fmt;
  g.b_slabs = slabs ? 1 : 0;
  {
    Hook hook(RQ_KERNEL_GEMM, s);
    if (rq::launch_gemm_grouped(g, kind, s) != hipSuccess) return RQ_ERR_HIP;
  }
  if (out_layout == RQ_MOE_OUT_COMBINED) {
    Hook hook(RQ_KERNEL_COMBINE, s);
    const int64_t NO = act == RQ_ACT_GATE_SILU ? N / 2 : N;  // output row length
    if (rq::launch_moe_combine(y_perm, pos, topk_w, T, top_k, NO, y, s) != hipSuccess) return RQ_ERR_HIP;
  }
  return RQ_OK;
}

int rq_moe_router_topk(const uint16_t* x, int64_t T, int64_t K, const uint16_t* w_gate, int64_t E, int top_k,
                       int32_t* topk_ids, uint16_t* topk_w, float* logits, void* stream) {
  if (T < 0 || K <= 0 || E < 1 || E > 32 || top_k < 1 || top_k > E || top_k > rq::router_max_topk())
    return RQ_ERR_SHAPE;
  if (K % 64 != 0) return RQ_ERR_ALIGN;
  if (K > kMaxK || T * K > ((int64_t)1 << 40)) return RQ_ERR_SHAPE;
  if (!w_gate) return RQ_ERR_NULL;
  if (T > 0 && (!x || !topk_ids || !topk_w)) return RQ_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_gate, 16) || !aligned(topk_ids, 4) || !aligned(topk_w, 2) ||
      !aligned(logits, 16))
    return RQ_ERR_ALIGN;
  if (T == 0) return RQ_OK;
  const int dev = check_device();
  if (dev != RQ_OK) return dev;
  Hook hook(RQ_KERNEL_ROUTER, (hipStream_t)stream);
  return rq::launch_router_topk(x, T, K, w_gate, E, top_k, topk_ids, topk_w, logits, (hipStream_t)stream) ==
                 hipSuccess
             ? RQ_OK
             : RQ_ERR_HIP;
}

int rq_attention_core(const uint16_t* qkv, int64_t requests, int length, int heads, int head_dim, uint16_t* out,
                      void* stream) {
  if (requests < 0 || length < 1 || length > rq::attention_max_len() || heads < 1 ||
      head_dim != rq::attention_head_dim())
    return RQ_ERR_SHAPE;
  if ((int64_t)heads * head_dim * 3 > kMaxOperandBytes / 2 ||
      requests * length * (int64_t)heads * head_dim * 3 > ((int64_t)1 << 40))
    return RQ_ERR_SHAPE;
  if (requests > 0 && (!qkv || !out)) return RQ_ERR_NULL;
  if (!aligned(qkv, 16) || !aligned(out, 16)) return RQ_ERR_ALIGN;
  if (requests == 0) return RQ_OK;
  const int dev = check_device();
  if (dev != RQ_OK) return dev;
  Hook hook(RQ_KERNEL_ATTENTION, (hipStream_t)stream);
  return rq::launch_attention_core(qkv, requests, length, heads, out, (hipStream_t)stream) == hipSuccess
             ? RQ_OK
             : RQ_ERR_HIP;
}

size_t rq_topk_workspace_size(int64_t rows, int64_t n, int k) {
  if (rows < 0 || n < 1 || k < 1 || k > rq::topk_max_k() || k > n) return 0;
  const int64_t pairs = rq::topk_pairs_per_buffer(rows, n, k);
  return pairs > 0 ? 2 * align_up((size_t)pairs * sizeof(int2)) : 0;
}

int rq_topk(const uint16_t* scores, int64_t rows, int64_t n, int k, int32_t* idx, uint16_t* vals, void* workspace,
            size_t workspace_bytes, void* stream) {
  if (rows < 0 || n < 1 || n > INT32_MAX || rows > 65535 || k < 1 || k > rq::topk_max_k() || k > n)
    return RQ_ERR_SHAPE;
  if (rows > 0 && (!scores || !idx || !vals)) return RQ_ERR_NULL;
  if (!aligned(scores, 16) || !aligned(idx, 4) || !aligned(vals, 2) || !aligned(workspace, 16)) return RQ_ERR_ALIGN;
  if (rows == 0) return RQ_OK;
  const size_t need = rq_topk_workspace_size(rows, n, k);
  if (need > 0 && (!workspace || workspace_bytes < need)) return RQ_ERR_WORKSPACE;
  const int dev = check_device();
  if (dev != RQ_OK) return dev;
  int2* b0 = need > 0 ? reinterpret_cast<int2*>(workspace) : nullptr;
  int2* b1 = need > 0 ? reinterpret_cast<int2*>(reinterpret_cast<uint8_t*>(workspace) + need / 2) : nullptr;
  Hook hook(RQ_KERNEL_TOPK, (hipStream_t)stream);
  return rq::launch_topk(scores, rows, n, k, idx, vals, b0, b1, (hipStream_t)stream) == hipSuccess ? RQ_OK
                                                                                                   : RQ_ERR_HIP;
}

int rq_fp8_moe_grouped_linear(const uint16_t* x, int in_layout, int act, const int32_t* topk_ids,
                              const uint16_t* topk_w, int64_t T, int top_k, const uint8_t* w_q,
                              const float* w_scale, int64_t E, int64_t N, int64_t K, uint16_t* y,
                              int out_layout, void* workspace, size_t workspace_bytes,
                              const rq_debug_out* dbg, void* stream) {
  return rq_fp8_moe_grouped_linear_ex(x, in_layout, act, RQ_FP8_E4M3, topk_ids, topk_w, T, top_k, w_q, w_scale,
                                      RQ_WSCALE_CHANNEL, E, N, K, y, out_layout, workspace, workspace_bytes, dbg,
                                      stream);
}

}  // extern "C"
