// Host side of the C ABI declared in include/lce.h: argument validation (before any HIP
// call), workspace sizing and carving, and the launch sequence on the caller's stream.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "lce.h"
#include "lce_launch.h"

namespace lce {

// The forward's pieces (also what the pipelined and column-chunked backward kernels use):
// the small per-token pieces first, then the per-tile LSE partials, which the merge consumes
// before any backward kernel runs (the two-pass backward reuses their memory).
size_t fused_small_bytes(int64_t BT, int64_t V) {
  const int64_t bt = BT > 0 ? BT : 1;
  const int64_t nblk = merge_blocks(bt);
  size_t n = ws_align(16);                         // n_valid, n_bad
  n += ws_align((size_t)bt * 4);                   // lse
  n += ws_align((size_t)bt * 4);                   // zy
  n += ws_align((size_t)nblk * 2 * 8);             // block sums
  n += ws_align((size_t)bt * 8);                   // per-token (LSE, target) for the backward
  n += ws_align((size_t)V * 4);                    // fp32 bias for the backward
  return n;
}
size_t fused_base_bytes(int64_t BT, int64_t V) {
  const int64_t bt = BT > 0 ? BT : 1;
  const int64_t nt = (V + kFwdTileV - 1) / kFwdTileV;
  return fused_small_bytes(BT, V) + ws_align((size_t)nt * (size_t)bt * 4);  // + lse_part
}

size_t logits_chunk_budget(int64_t BT, int64_t H, int64_t V) {
  const int64_t inc = (V + H - 1) / H;
  const int64_t need = (BT + inc - 1) / inc;
  int64_t cs = 1;
  while (cs < need) cs <<= 1;
  return (size_t)cs * (size_t)V * 4;
}

size_t fused_workspace_bytes(int64_t BT, int64_t H, int64_t V, bool bf16) {
  size_t n = fused_base_bytes(BT, V);
  if (bf16) {
    // the two-pass region starts where the LSE partials do
    TwoPass tp{};
    if (H > 1024) tp = twopass_plan(BT, H, V);
    const SgPlan sp = sg_plan(BT, H, V), sf = sg_plan(BT, H, V, kSgFiltered);  // (exact, filtered or sorted)
    n = std::max(n, fused_small_bytes(BT, V) + std::max({tp.on ? tp.bytes : (size_t)0, sp.on ? sp.bytes : (size_t)0,
                                                         sf.on ? sf.bytes : (size_t)0}));
  }
  return n;
}

FusedWs fused_carve(void* ws, int64_t BT, int64_t H, int64_t V, bool bf16) {
  const int64_t bt = BT > 0 ? BT : 1;
  FusedWs w;
  w.nt = (V + kFwdTileV - 1) / kFwdTileV;
  w.nblk = BT > 0 ? merge_blocks(BT) : 0;
  const int64_t nblk_alloc = merge_blocks(bt);
  char* p = static_cast<char*>(ws);
  w.n_valid = reinterpret_cast<int64_t*>(p);
  w.n_bad = reinterpret_cast<int32_t*>(p + 8);
  p += ws_align(16);
  w.lse = reinterpret_cast<float*>(p);
  p += ws_align((size_t)bt * 4);
  w.zy = reinterpret_cast<float*>(p);
  p += ws_align((size_t)bt * 4);
  w.blk = reinterpret_cast<double*>(p);
  p += ws_align((size_t)nblk_alloc * 2 * 8);
  w.tok = reinterpret_cast<float2*>(p);
  p += ws_align((size_t)bt * 8);
  w.biasf = reinterpret_cast<float*>(p);
  p += ws_align((size_t)V * 4);
  w.lse_part = reinterpret_cast<float*>(p);  // (at fused_small_bytes)
  w.big = nullptr;
  if (bf16 && ((H > 1024 && twopass_plan(BT, H, V).on) || sg_plan(BT, H, V).on || sg_plan(BT, H, V, kSgFiltered).on))
    w.big = p;
  return w;
}

static bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

static const char* kStageNames[kNumStages] = {"targets", "fwd_lse", "target_logit", "merge",
                                               "loss",    "bwd_dinput", "bwd_dweight"};

static lce_status fused_call(const void* hidden, const void* W, const void* bias, const int64_t* targets,
                             int64_t BT, int64_t H, int64_t V, lce_dtype dtype, int64_t ignore_index,
                             float z_loss_mult, lce_reduction reduction, uint32_t flags, float* loss_out,
                             void* grad_input, void* grad_W, void* grad_b, int64_t* n_valid_out,
                             float* lse_out, void* workspace, size_t workspace_bytes, void* stream,
                             void* const* ev_start, void* const* ev_stop, float filter_eps,
                             int64_t* filter_counts, bool allow_sort = false) {
  // ---- validation: no HIP calls before this block has passed
  if (BT < 0 || V < 1 || H < 8 || (H % 8) != 0) return LCE_ERR_SHAPE;
  if (BT > ((int64_t)1 << 40) || V > ((int64_t)1 << 31) - 2 || H > ((int64_t)1 << 20)) return LCE_ERR_SHAPE;
  if (dtype != LCE_DTYPE_BF16 && dtype != LCE_DTYPE_F32) return LCE_ERR_DTYPE;
  if (W == nullptr || loss_out == nullptr || workspace == nullptr) return LCE_ERR_NULL;
  if (BT > 0 && (hidden == nullptr || targets == nullptr)) return LCE_ERR_NULL;
  if (reduction != LCE_REDUCTION_MEAN && reduction != LCE_REDUCTION_SUM) return LCE_ERR_ARG;
  if (!(z_loss_mult >= 0.f) || !std::isfinite(z_loss_mult)) return LCE_ERR_ARG;
  if (grad_b != nullptr && bias == nullptr) return LCE_ERR_ARG;
  const uint32_t allowed = LCE_FLAG_CHECK_TARGETS | LCE_FLAG_GRAD_W_FP32 | (allow_sort ? LCE_FLAG_SORT_VOCAB : 0u);
  if ((flags & ~allowed) != 0) return LCE_ERR_ARG;
  const bool sort = (flags & LCE_FLAG_SORT_VOCAB) != 0;
  // (the sort's grids hold one block per 256 hidden rows and one wave per entry)
  if (sort && (BT > ((int64_t)1 << 24) || V > ((int64_t)1 << 24))) return LCE_ERR_SHAPE;
  if (!(filter_eps >= 0.f) || !std::isfinite(filter_eps)) return LCE_ERR_ARG;
  const size_t es = dtype == LCE_DTYPE_BF16 ? 2 : 4;
  if (!aligned(hidden, 16) || !aligned(W, 16) || !aligned(grad_input, 16) || !aligned(grad_W, 16) ||
      !aligned(workspace, 16) || !aligned(bias, es) || !aligned(grad_b, es) || !aligned(targets, 8) ||
      !aligned(loss_out, 4) || !aligned(n_valid_out, 8) || !aligned(lse_out, 4) || !aligned(filter_counts, 8))
    return LCE_ERR_ALIGNMENT;
  const size_t ws_fused = fused_workspace_bytes(BT, H, V, dtype == LCE_DTYPE_BF16);
  if (workspace_bytes < ws_fused + (sort ? sort_workspace_bytes(BT, H, V, es) : 0)) return LCE_ERR_WORKSPACE;

  FusedArgs a;
  a.hidden = hidden;
  a.W = W;
  a.bias = bias;
  a.targets = targets;
  a.BT = BT;
  a.H = H;
  a.V = V;
  a.bf16 = dtype == LCE_DTYPE_BF16;
  a.ignore_index = ignore_index;
  a.mu = z_loss_mult;
  a.mean = reduction == LCE_REDUCTION_MEAN;
  a.loss_out = loss_out;
  a.grad_input = grad_input;
  a.grad_W = grad_W;
  a.grad_b = grad_b;
  a.n_valid_out = n_valid_out;
  a.lse_out = lse_out;
  a.grad_w_f32 = (flags & LCE_FLAG_GRAD_W_FP32) != 0 && dtype == LCE_DTYPE_BF16;
  a.out_row_map = nullptr;
  a.filter_eps = filter_eps;
  a.filter_counts = filter_eps > 0.f ? filter_counts : nullptr;
  const FusedWs w = fused_carve(workspace, BT, H, V, dtype == LCE_DTYPE_BF16);
  hipStream_t st = static_cast<hipStream_t>(stream);

  typedef hipError_t (*Launch)(const FusedArgs&, const FusedWs&, hipStream_t);
  static const Launch kLaunch[kNumStages] = {launch_targets,    launch_fwd_lse,    launch_target_logit,
                                             launch_merge,      launch_loss,       launch_bwd_dinput,
                                             launch_bwd_dweight};
  if (sort) {
    // Vocabulary sorting: count the targets and check them as given, order the vocabulary,
    // then run every stage on the sorted copies (the first stage again, for the sorted
    // bias), with grad_W / grad_b rows written back through the order.
    if (launch_targets(a, w, st) != hipSuccess) return LCE_ERR_HIP;
    if (flags & LCE_FLAG_CHECK_TARGETS) {
      int32_t bad = 0;
      if (hipMemcpyAsync(&bad, w.n_bad, sizeof(bad), hipMemcpyDeviceToHost, st) != hipSuccess) return LCE_ERR_HIP;
      if (hipStreamSynchronize(st) != hipSuccess) return LCE_ERR_HIP;
      if (bad != 0) return LCE_ERR_TARGET_RANGE;
      flags &= ~LCE_FLAG_CHECK_TARGETS;
    }
    const SortWs sw = sort_carve(static_cast<char*>(workspace) + ws_fused, BT, H, V, es);
    if (launch_sort_vocab(a, sw, w.n_valid, st) != hipSuccess) return LCE_ERR_HIP;
    a.W = sw.Ws;
    if (a.bias != nullptr) a.bias = sw.bs;
    if (BT > 0) a.targets = sw.ys;
    a.out_row_map = sw.perm;
  }
  for (int k = 0; k < kNumStages; ++k) {
    if (ev_start && ev_start[k] && hipEventRecord(static_cast<hipEvent_t>(ev_start[k]), st) != hipSuccess)
      return LCE_ERR_HIP;
    if (kLaunch[k](a, w, st) != hipSuccess) return LCE_ERR_HIP;
    if (ev_stop && ev_stop[k] && hipEventRecord(static_cast<hipEvent_t>(ev_stop[k]), st) != hipSuccess)
      return LCE_ERR_HIP;
    if (k == kStTargets && (flags & LCE_FLAG_CHECK_TARGETS)) {
      int32_t bad = 0;
      if (hipMemcpyAsync(&bad, w.n_bad, sizeof(bad), hipMemcpyDeviceToHost, st) != hipSuccess) return LCE_ERR_HIP;
      if (hipStreamSynchronize(st) != hipSuccess) return LCE_ERR_HIP;
      if (bad != 0) return LCE_ERR_TARGET_RANGE;
    }
  }
  return LCE_OK;
}

}  // namespace lce

extern "C" {

size_t lce_fwd_bwd_workspace_bytes(int64_t BT, int64_t H, int64_t V, lce_dtype dtype, uint32_t flags) {
  if (BT < 0 || V < 1 || H < 8 || (H % 8) != 0) return 0;
  if (dtype != LCE_DTYPE_BF16 && dtype != LCE_DTYPE_F32) return 0;
  const size_t es = dtype == LCE_DTYPE_BF16 ? 2 : 4;
  return lce::fused_workspace_bytes(BT, H, V, dtype == LCE_DTYPE_BF16) +
         ((flags & LCE_FLAG_SORT_VOCAB) ? lce::sort_workspace_bytes(BT, H, V, es) : 0);
}

lce_status lce_fwd_bwd(const void* hidden, const void* W, const void* bias, const int64_t* targets, int64_t BT,
                       int64_t H, int64_t V, lce_dtype dtype, int64_t ignore_index, float z_loss_mult,
                       lce_reduction reduction, uint32_t flags, float* loss_out, void* grad_input,
                       void* grad_W, void* grad_b, int64_t* n_valid_out, float* lse_out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return lce::fused_call(hidden, W, bias, targets, BT, H, V, dtype, ignore_index, z_loss_mult, reduction,
                         flags, loss_out, grad_input, grad_W, grad_b, n_valid_out, lse_out, workspace,
                         workspace_bytes, stream, nullptr, nullptr, 0.f, nullptr);
}

lce_status lce_fwd_bwd_profiled(const void* hidden, const void* W, const void* bias, const int64_t* targets,
                                int64_t BT, int64_t H, int64_t V, lce_dtype dtype, int64_t ignore_index,
                                float z_loss_mult, lce_reduction reduction, uint32_t flags, float* loss_out,
                                void* grad_input, void* grad_W, void* grad_b, int64_t* n_valid_out,
                                float* lse_out, void* workspace, size_t workspace_bytes, void* stream,
                                void* const* ev_start, void* const* ev_stop) {
  return lce::fused_call(hidden, W, bias, targets, BT, H, V, dtype, ignore_index, z_loss_mult, reduction,
                         flags, loss_out, grad_input, grad_W, grad_b, n_valid_out, lse_out, workspace,
                         workspace_bytes, stream, ev_start, ev_stop, 0.f, nullptr);
}

lce_status lce_fwd_bwd_filtered(const void* hidden, const void* W, const void* bias, const int64_t* targets,
                                int64_t BT, int64_t H, int64_t V, lce_dtype dtype, int64_t ignore_index,
                                float z_loss_mult, lce_reduction reduction, uint32_t flags, float* loss_out,
                                void* grad_input, void* grad_W, void* grad_b, int64_t* n_valid_out,
                                float* lse_out, void* workspace, size_t workspace_bytes, void* stream,
                                float filter_eps, int64_t* filter_counts) {
  return lce::fused_call(hidden, W, bias, targets, BT, H, V, dtype, ignore_index, z_loss_mult, reduction,
                         flags, loss_out, grad_input, grad_W, grad_b, n_valid_out, lse_out, workspace,
                         workspace_bytes, stream, nullptr, nullptr, filter_eps, filter_counts, true);
}

lce_status lce_filter_tile_shape(int64_t BT, int64_t H, int64_t V, lce_dtype dtype, int64_t* rows, int64_t* cols) {
  if (rows == nullptr || cols == nullptr || BT < 0 || V < 1 || H < 8 || (H % 8) != 0) return LCE_ERR_ARG;
  if (dtype != LCE_DTYPE_BF16 && dtype != LCE_DTYPE_F32) return LCE_ERR_ARG;
  const bool one = dtype == LCE_DTYPE_BF16 && lce::sg_plan(BT, H, V, lce::kSgFiltered).on;
  *rows = one ? 256 : 64;
  *cols = one ? 64 : 16;
  return LCE_OK;
}

size_t lce_fwd_bwd_chunked_workspace_bytes(int64_t BT, int64_t H, int64_t V, lce_dtype dtype, uint32_t flags) {
  if (BT < 0 || V < 1 || H < 8 || (H % 8) != 0) return 0;
  if (dtype != LCE_DTYPE_BF16) return 0;
  return lce::chunked_workspace_bytes(BT, H, V, (flags & LCE_FLAG_GRAD_W_FP32) != 0);
}

}  // extern "C"

namespace lce {

// Argument checks shared by the chunked entry points (before any HIP call) and the argument
// block they build.
static lce_status chunk_args(const void* hidden, const void* W, const void* bias, const int64_t* targets,
                             int64_t BT, int64_t H, int64_t V, lce_dtype dtype, int64_t ignore_index,
                             float z_loss_mult, uint32_t flags, uint32_t allowed_flags, void* grad_input,
                             void* grad_W, void* grad_b, int64_t* n_valid_out, void* workspace,
                             size_t workspace_bytes, size_t need, FusedArgs* a) {
  if (BT < 0 || V < 1 || H < 8 || (H % 8) != 0) return LCE_ERR_SHAPE;
  // (V <= 2^22: the byte offsets inside a 256-row logits tile of the chunk stay 32-bit)
  if (BT > ((int64_t)1 << 40) || V > ((int64_t)1 << 22) || H > ((int64_t)1 << 20)) return LCE_ERR_SHAPE;
  if (dtype != LCE_DTYPE_BF16) return LCE_ERR_DTYPE;
  if (W == nullptr || workspace == nullptr) return LCE_ERR_NULL;
  if (BT > 0 && (hidden == nullptr || targets == nullptr)) return LCE_ERR_NULL;
  if (!(z_loss_mult >= 0.f) || !std::isfinite(z_loss_mult)) return LCE_ERR_ARG;
  if (grad_b != nullptr && bias == nullptr) return LCE_ERR_ARG;
  if ((flags & ~allowed_flags) != 0) return LCE_ERR_ARG;
  if (!aligned(hidden, 16) || !aligned(W, 16) || !aligned(grad_input, 16) || !aligned(grad_W, 16) ||
      !aligned(workspace, 16) || !aligned(bias, 2) || !aligned(grad_b, 2) || !aligned(targets, 8) ||
      !aligned(n_valid_out, 8))
    return LCE_ERR_ALIGNMENT;
  if (workspace_bytes < need) return LCE_ERR_WORKSPACE;
  *a = FusedArgs{};
  a->hidden = hidden;
  a->W = W;
  a->bias = bias;
  a->targets = targets;
  a->BT = BT;
  a->H = H;
  a->V = V;
  a->bf16 = true;
  a->ignore_index = ignore_index;
  a->mu = z_loss_mult;
  a->grad_input = grad_input;
  a->grad_W = grad_W;
  a->grad_b = grad_b;
  a->n_valid_out = n_valid_out;
  return LCE_OK;
}

// the token-chunked composition's workspace (0 for sizes it does not take: chunk_args then
// reports the shape error)
static size_t chunk_need(int64_t BT, int64_t H, int64_t V, lce_dtype dtype, uint32_t flags) {
  if (BT < 0 || V < 1 || H < 8 || (H % 8) != 0 || dtype != LCE_DTYPE_BF16) return 0;
  return chunked_workspace_bytes(BT, H, V, (flags & LCE_FLAG_GRAD_W_FP32) != 0);
}

// Per-row outputs and their backward on the one-pass plan (kSgRows), when it fits: workspace
// [fused small pieces | per-token coefficients and entropy | region], the region holding either
// the forward's LSE and mean-logit partials for fsub tokens at a time or the one-pass plan's
// buffers.  Everything stays within the one-chunk budget.  one = false: the token-chunked
// composition instead.
struct RowsLayout {
  bool one;
  SgPlan plan;
  size_t extra;     // coefficients (rows_coef_bytes) + entropy [BT]
  int64_t fsub;     // tokens per forward launch (a multiple of 256, or all)
  size_t part;      // bytes of one partial array (nt x fsub floats)
  size_t bytes;
};
static RowsLayout rows_layout(int64_t BT, int64_t H, int64_t V) {
  RowsLayout r{};
  const int64_t bt = BT > 0 ? BT : 1;
  r.extra = rows_coef_bytes(BT) + ws_align((size_t)bt * 4);
  r.plan = sg_plan(bt, H, V, kSgRows, r.extra);
  const int64_t nt = (V + kFwdTileV - 1) / kFwdTileV;
  const size_t budget = logits_chunk_budget(bt, H, V);
  const size_t fixed = fused_small_bytes(BT, V) + r.extra + 4096 + alloc_slack(budget);
  if (!r.plan.on || !r.plan.one || budget <= fixed) return r;
  // the forward's two partial arrays in the region: as many tokens per launch as fit (all, or
  // a multiple of 256)
  const size_t room = std::max(budget - fixed, r.plan.bytes);
  const size_t half = room / 2 > kWsAlign ? room / 2 - kWsAlign : 0;
  const int64_t fit = (int64_t)(half / ((size_t)nt * 4));
  r.fsub = fit >= bt ? bt : fit / 256 * 256;
  if (r.fsub < 1) return r;
  r.part = ws_align((size_t)nt * (size_t)r.fsub * 4);
  r.bytes = fused_small_bytes(BT, V) + r.extra + std::max(r.plan.bytes, 2 * r.part);
  r.one = true;
  return r;
}

// The per-row forward (lse .. row_loss, each may be NULL) in launches of fsub tokens whose
// partials go to lse_part / ez_part; zy from w.
static hipError_t rows_forward_sub(const FusedArgs& a, const FusedWs& w, float* lse_part, float* ez_part, int64_t fsub,
                                   float* lse, float* lp, float* ent, float* rl, hipStream_t st) {
  const uint16_t* h = static_cast<const uint16_t*>(a.hidden);  // (bf16 rows)
  auto off = [](float* q, int64_t r0) { return q ? q + r0 : nullptr; };
  for (int64_t r0 = 0; r0 < a.BT; r0 += fsub) {
    const int64_t rows = std::min(fsub, a.BT - r0);
    FusedArgs s = a;
    s.hidden = h + r0 * a.H;
    s.targets = a.targets + r0;
    s.BT = rows;
    FusedWs ws = w;
    ws.lse_part = lse_part;
    ws.zy = w.zy + r0;
    const hipError_t e = launch_rows_fused_forward(s, ws, ez_part, off(lse, r0), off(lp, r0), off(ent, r0),
                                                   off(rl, r0), st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

static lce_status chunk_call(const FusedArgs& a, ChunkMode mode, const RowsHost& io, uint32_t flags, void* ws,
                             void* stream) {
  bool bad = false;
  if (chunk_loop(a, mode, io, (flags & LCE_FLAG_GRAD_W_FP32) != 0, (flags & LCE_FLAG_CHECK_TARGETS) != 0, ws,
                 static_cast<hipStream_t>(stream), &bad) != hipSuccess)
    return LCE_ERR_HIP;
  return bad ? LCE_ERR_TARGET_RANGE : LCE_OK;
}

}  // namespace lce

extern "C" {

lce_status lce_fwd_bwd_chunked(const void* hidden, const void* W, const void* bias, const int64_t* targets,
                               int64_t BT, int64_t H, int64_t V, lce_dtype dtype, int64_t ignore_index,
                               float z_loss_mult, lce_reduction reduction, uint32_t flags, float* loss_out,
                               void* grad_input, void* grad_W, void* grad_b, int64_t* n_valid_out,
                               float* lse_out, void* workspace, size_t workspace_bytes, void* stream) {
  lce::FusedArgs a;
  const lce_status s = lce::chunk_args(hidden, W, bias, targets, BT, H, V, dtype, ignore_index, z_loss_mult, flags,
                                       LCE_FLAG_CHECK_TARGETS | LCE_FLAG_GRAD_W_FP32, grad_input, grad_W, grad_b,
                                       n_valid_out, workspace, workspace_bytes,
                                       lce::chunk_need(BT, H, V, dtype, flags), &a);
  if (s != LCE_OK) return s;
  if (loss_out == nullptr) return LCE_ERR_NULL;
  if (reduction != LCE_REDUCTION_MEAN && reduction != LCE_REDUCTION_SUM) return LCE_ERR_ARG;
  if (!lce::aligned(loss_out, 4) || !lce::aligned(lse_out, 4)) return LCE_ERR_ALIGNMENT;
  a.mean = reduction == LCE_REDUCTION_MEAN;
  a.loss_out = loss_out;
  a.lse_out = lse_out;
  return lce::chunk_call(a, lce::kLoss, lce::RowsHost{}, flags, workspace, stream);
}

// The per-row forward's own pieces (without the one-pass layout): the fused forward's workspace
// and the per-tile mean logits.
static size_t rows_forward_bytes(int64_t BT, int64_t V) {
  const int64_t nt = (V + lce::kFwdTileV - 1) / lce::kFwdTileV;
  return lce::fused_base_bytes(BT, V) + lce::ws_align((size_t)nt * (size_t)(BT > 0 ? BT : 1) * 4);
}

size_t lce_rows_workspace_bytes(int64_t BT, int64_t H, int64_t V, lce_dtype dtype, uint32_t flags) {
  size_t c = lce_fwd_bwd_chunked_workspace_bytes(BT, H, V, dtype, flags);
  if (c == 0) return 0;
  const lce::RowsLayout r = lce::rows_layout(BT, H, V);
  if (r.one) return r.bytes;
  c += lce::rows_coef_bytes(BT);  // (the backward from saved forward outputs)
  const size_t f = rows_forward_bytes(BT, V);
  return c > f ? c : f;
}

lce_status lce_rows_forward(const void* hidden, const void* W, const void* bias, const int64_t* targets,
                            int64_t BT, int64_t H, int64_t V, lce_dtype dtype, int64_t ignore_index,
                            float z_loss_mult, uint32_t flags, float* lse_out, float* logprobs_out,
                            float* entropy_out, float* row_loss_out, int64_t* n_valid_out, void* workspace,
                            size_t workspace_bytes, void* stream) {
  lce::FusedArgs a;
  const lce_status s = lce::chunk_args(hidden, W, bias, targets, BT, H, V, dtype, ignore_index, z_loss_mult, flags,
                                       LCE_FLAG_CHECK_TARGETS, nullptr, nullptr, nullptr, n_valid_out, workspace,
                                       workspace_bytes, lce_rows_workspace_bytes(BT, H, V, dtype, flags), &a);
  if (s != LCE_OK) return s;
  if (!lce::aligned(lse_out, 4) || !lce::aligned(logprobs_out, 4) || !lce::aligned(entropy_out, 4) ||
      !lce::aligned(row_loss_out, 4))
    return LCE_ERR_ALIGNMENT;
  // one pass over the vocabulary: the fused forward with an (LSE, mean logit) epilogue
  const lce::FusedWs w = lce::fused_carve(workspace, BT, H, V, false);
  const lce::RowsLayout r = lce::rows_layout(BT, H, V);
  hipStream_t st = static_cast<hipStream_t>(stream);
  lce::FusedArgs t = a;
  t.bias = nullptr;  // (the pre-pass only counts; the forward adds the bias itself)
  if (lce::launch_targets(t, w, st) != hipSuccess) return LCE_ERR_HIP;
  if (flags & LCE_FLAG_CHECK_TARGETS) {
    int32_t bad = 0;
    if (hipMemcpyAsync(&bad, w.n_bad, sizeof(bad), hipMemcpyDeviceToHost, st) != hipSuccess) return LCE_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return LCE_ERR_HIP;
    if (bad != 0) return LCE_ERR_TARGET_RANGE;
  }
  if (r.one) {  // (partials of r.fsub tokens at a time, in the region after the per-row pieces)
    char* region = static_cast<char*>(workspace) + lce::fused_small_bytes(BT, V) + r.extra;
    if (lce::rows_forward_sub(a, w, reinterpret_cast<float*>(region), reinterpret_cast<float*>(region + r.part),
                              r.fsub, lse_out, logprobs_out, entropy_out, row_loss_out, st) != hipSuccess)
      return LCE_ERR_HIP;
  } else {
    float* ez_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + lce::fused_base_bytes(BT, V));
    if (lce::launch_rows_fused_forward(a, w, ez_part, lse_out, logprobs_out, entropy_out, row_loss_out, st) !=
        hipSuccess)
      return LCE_ERR_HIP;
  }
  if (n_valid_out != nullptr &&
      hipMemcpyAsync(n_valid_out, w.n_valid, sizeof(int64_t), hipMemcpyDeviceToDevice, st) != hipSuccess)
    return LCE_ERR_HIP;
  return LCE_OK;
}

lce_status lce_rows_backward(const void* hidden, const void* W, const void* bias, const int64_t* targets,
                             int64_t BT, int64_t H, int64_t V, lce_dtype dtype, int64_t ignore_index,
                             float z_loss_mult, uint32_t flags, const float* grad_row_loss,
                             const float* grad_logprobs, const float* grad_entropy, const float* lse_saved,
                             const float* entropy_saved, void* grad_input, void* grad_W, void* grad_b,
                             void* workspace, size_t workspace_bytes, void* stream) {
  lce::FusedArgs a;
  const lce_status s = lce::chunk_args(hidden, W, bias, targets, BT, H, V, dtype, ignore_index, z_loss_mult, flags,
                                       LCE_FLAG_CHECK_TARGETS | LCE_FLAG_GRAD_W_FP32, grad_input, grad_W, grad_b,
                                       nullptr, workspace, workspace_bytes,
                                       lce_rows_workspace_bytes(BT, H, V, dtype, flags), &a);
  if (s != LCE_OK) return s;
  if (!lce::aligned(grad_row_loss, 4) || !lce::aligned(grad_logprobs, 4) || !lce::aligned(grad_entropy, 4) ||
      !lce::aligned(lse_saved, 4) || !lce::aligned(entropy_saved, 4))
    return LCE_ERR_ALIGNMENT;
  if ((lse_saved == nullptr) != (entropy_saved == nullptr)) return LCE_ERR_ARG;
  const lce::RowsLayout r = lce::rows_layout(BT, H, V);
  if (!r.one) {
    const lce::RowsHost io{nullptr,       nullptr,       nullptr,      nullptr,  grad_row_loss,
                           grad_logprobs, grad_entropy,  lse_saved,    entropy_saved};
    return lce::chunk_call(a, lce::kRowGrads, io, flags, workspace, stream);
  }
  // One pass: the per-token coefficients (from the saved LSE and entropy, or from a per-row
  // forward into the workspace), then the one-pass sweep with the per-row dlogits.
  hipStream_t st = static_cast<hipStream_t>(stream);
  lce::FusedWs w = lce::fused_carve(workspace, BT, H, V, false);
  const size_t bt = (size_t)(BT > 0 ? BT : 1);
  char* ex = static_cast<char*>(workspace) + lce::fused_small_bytes(BT, V);
  float4* rtok = reinterpret_cast<float4*>(ex);
  int32_t* rcy = reinterpret_cast<int32_t*>(ex + lce::ws_align(bt * 16));
  float* ent = reinterpret_cast<float*>(ex + lce::rows_coef_bytes(BT));
  char* region = ex + r.extra;
  lce::FusedArgs t = a;
  t.bias = nullptr;
  if (lce::launch_targets(t, w, st) != hipSuccess) return LCE_ERR_HIP;
  if (flags & LCE_FLAG_CHECK_TARGETS) {
    int32_t bad = 0;
    if (hipMemcpyAsync(&bad, w.n_bad, sizeof(bad), hipMemcpyDeviceToHost, st) != hipSuccess) return LCE_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return LCE_ERR_HIP;
    if (bad != 0) return LCE_ERR_TARGET_RANGE;
  }
  const float* lse = lse_saved;
  const float* entropy = entropy_saved;
  if (lse == nullptr) {
    if (lce::rows_forward_sub(a, w, reinterpret_cast<float*>(region), reinterpret_cast<float*>(region + r.part),
                              r.fsub, w.lse, nullptr, ent, nullptr, st) != hipSuccess)
      return LCE_ERR_HIP;
    lse = w.lse;
    entropy = ent;
  }
  if (lce::launch_rows_coef(lse, entropy, a.targets, a.BT, a.V, a.ignore_index, a.mu, grad_row_loss, grad_logprobs,
                            grad_entropy, rtok, rcy, st) != hipSuccess)
    return LCE_ERR_HIP;
  w.big = region;
  a.mean = false;  // (the per-row weights carry their own scale)
  a.grad_w_f32 = (flags & LCE_FLAG_GRAD_W_FP32) != 0;
  if (lce::launch_rows_onepass(a, w, r.plan, rtok, rcy, st) != hipSuccess) return LCE_ERR_HIP;
  return LCE_OK;
}

const char* lce_stage_name(int k) {
  if (k < 0 || k >= lce::kNumStages) return nullptr;
  return lce::kStageNames[k];
}

size_t lce_ce_workspace_bytes(int64_t B, int64_t V, lce_dtype dtype) {
  if (B < 0 || V < 1) return 0;
  if (dtype != LCE_DTYPE_BF16 && dtype != LCE_DTYPE_F32 && dtype != LCE_DTYPE_F16) return 0;
  return lce::ce_workspace_bytes(B);
}

lce_status lce_ce_with_grad_inplace(void* logits, const int64_t* targets, int64_t B, int64_t V, lce_dtype dtype,
                                    int64_t ignore_index, float z_loss_mult, float* ce_sum_out,
                                    float* z_sum_out, int64_t* n_valid_out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (B < 0 || V < 1 || V > ((int64_t)1 << 31) - 2 || B > ((int64_t)1 << 31) - 1) return LCE_ERR_SHAPE;
  if (dtype != LCE_DTYPE_BF16 && dtype != LCE_DTYPE_F32 && dtype != LCE_DTYPE_F16) return LCE_ERR_DTYPE;
  if (ce_sum_out == nullptr || z_sum_out == nullptr || workspace == nullptr) return LCE_ERR_NULL;
  if (B > 0 && (logits == nullptr || targets == nullptr)) return LCE_ERR_NULL;
  if (!(z_loss_mult >= 0.f) || !std::isfinite(z_loss_mult)) return LCE_ERR_ARG;
  const size_t es = dtype == LCE_DTYPE_F32 ? 4 : 2;
  if (!lce::aligned(logits, 16) || !lce::aligned(workspace, 16) || !lce::aligned(targets, 8) ||
      !lce::aligned(ce_sum_out, 4) || !lce::aligned(z_sum_out, 4) || !lce::aligned(n_valid_out, 8))
    return LCE_ERR_ALIGNMENT;
  (void)es;
  if (workspace_bytes < lce::ce_workspace_bytes(B)) return LCE_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int ct = dtype == LCE_DTYPE_BF16 ? lce::kCeBf16 : (dtype == LCE_DTYPE_F16 ? lce::kCeF16 : lce::kCeF32);
  if (lce::launch_ce_inplace(logits, ct, targets, B, V, V, ignore_index, z_loss_mult,
                             ce_sum_out, z_sum_out, n_valid_out, nullptr, workspace, false, st) != hipSuccess)
    return LCE_ERR_HIP;
  return LCE_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Scratch memory of lce_ce_with_grad_inplace_noalloc: the standalone cross-entropy's
// workspace (per-row ce, z and valid flag) for up to LCE_NOALLOC_MAX_ROWS rows, in a
// file-scope device array that each GPU holds from the library's load to the end of the
// process.  In host code `scratch` only names the variable; its device address, different on
// every GPU, comes from hipGetSymbolAddress once per device and is what the kernels receive.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kNoAllocScratchBytes = 3 * (size_t)LCE_NOALLOC_MAX_ROWS * 4;
static_assert(kNoAllocScratchBytes >= 3 * 256, "scratch holds the three per-row arrays");
}  // namespace
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {nullptr};

// The current device's address of `scratch` (looked up on the first call on that device).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

extern "C" {

lce_status lce_ce_with_grad_inplace_noalloc(void* logits, const int64_t* targets, int64_t B, int64_t V,
                                            lce_dtype dtype, int64_t ignore_index, float z_loss_mult,
                                            float* ce_sum_out, float* z_sum_out, int64_t* n_valid_out,
                                            void* stream) {
  if (B < 0 || V < 1 || V > ((int64_t)1 << 31) - 2) return LCE_ERR_SHAPE;
  if (B > LCE_NOALLOC_MAX_ROWS) return LCE_ERR_SCRATCH_LIMIT;
  if (dtype != LCE_DTYPE_BF16 && dtype != LCE_DTYPE_F32 && dtype != LCE_DTYPE_F16) return LCE_ERR_DTYPE;
  if (ce_sum_out == nullptr || z_sum_out == nullptr) return LCE_ERR_NULL;
  if (B > 0 && (logits == nullptr || targets == nullptr)) return LCE_ERR_NULL;
  if (!(z_loss_mult >= 0.f) || !std::isfinite(z_loss_mult)) return LCE_ERR_ARG;
  if (!lce::aligned(logits, 16) || !lce::aligned(targets, 8) || !lce::aligned(ce_sum_out, 4) ||
      !lce::aligned(z_sum_out, 4) || !lce::aligned(n_valid_out, 8))
    return LCE_ERR_ALIGNMENT;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return LCE_ERR_HIP;
  // (the per-row arrays are written for every row before the reduction reads them: nothing
  // in the scratch needs clearing)
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int ct = dtype == LCE_DTYPE_BF16 ? lce::kCeBf16 : (dtype == LCE_DTYPE_F16 ? lce::kCeF16 : lce::kCeF32);
  if (lce::launch_ce_inplace(logits, ct, targets, B, V, V, ignore_index, z_loss_mult, ce_sum_out, z_sum_out,
                             n_valid_out, nullptr, ws, false, st) != hipSuccess)
    return LCE_ERR_HIP;
  return LCE_OK;
}

const char* lce_status_string(lce_status s) {
  switch (s) {
    case LCE_OK: return "ok";
    case LCE_ERR_NULL: return "a required pointer is NULL";
    case LCE_ERR_SHAPE: return "invalid shape (need BT >= 0, V >= 1, H >= 8 and a multiple of 8)";
    case LCE_ERR_DTYPE: return "unsupported dtype";
    case LCE_ERR_ALIGNMENT: return "misaligned pointer (tensors and workspace must be 16-byte aligned)";
    case LCE_ERR_WORKSPACE: return "workspace too small";
    case LCE_ERR_ARG: return "invalid argument";
    case LCE_ERR_TARGET_RANGE: return "a target is neither ignore_index nor in [0, V)";
    case LCE_ERR_HIP: return "HIP runtime error";
    case LCE_ERR_SCRATCH_LIMIT: return "size beyond the no-allocation entry point's scratch (B > LCE_NOALLOC_MAX_ROWS)";
  }
  return "unknown status";
}

const char* lce_version(void) { return "0.1.0 gfx950"; }

}  // extern "C"
