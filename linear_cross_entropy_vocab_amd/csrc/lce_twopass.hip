// Backward of the fused path for bf16 inputs with H > 1024.
//
// The pipelined backward keeps a workgroup's 64 stationary rows and their 64 x H fp32
// accumulators on chip, which stops at H = 1024.  Above that, the recompute of "Fused Linear
// Cross-Entropy: The Math, the Memory Wall, and Two Ways Around It" ("Why two passes") is
// done with stored dlogits instead, in blocks that fit the memory the forward leaves of the
// one-logits-chunk budget ("The chunk-size trick"):
//   pass 2 (grad_input), for each block of tb tokens:
//     G = dlogits(hidden[block] . W^T + b, LSE, y)   forward kernel, dlogits epilogue -> bf16
//     grad_input[block] = c * G . W                    stored-dlogits GEMM (vocabulary ranges
//                                                      summed by mat_reduce)
//   pass 1 (grad_W, grad_b), for each block of vb vocabulary rows:
//     G = dlogits(hidden . W[block]^T + b[block], LSE, y)
//     grad_W[block] = c * G^T . hidden, grad_b[block] = c * column sums of G
// Each gradient element is still produced by one workgroup (no atomics) and z is recomputed
// once per pass, as in the pipelined path (10 BT V H flops in all).  The dlogits are those of
// the summed loss, formed in fp32 from the GEMM accumulator and the forward's LSE and rounded
// once to bf16 (the pipelined kernels use the same operand precision).
#include <algorithm>

#include "lce_common.h"
#include "lce_launch.h"

#include <vector>

namespace lce {

static int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Compute units of the MI355X, for sizing blocks to whole rounds of workgroups (on another
// device count only the efficiency of the choice changes).
constexpr int64_t kPlanCUs = 256;

TwoPass twopass_plan(int64_t BT, int64_t H, int64_t V) {
  TwoPass t{};
  t.on = false;
  mat_plan(H, &t.nb, &t.hchunks);
  const size_t budget = logits_chunk_budget(BT, H, V);
  // the region overlaps the forward's LSE partials (consumed by the merge); part of the budget
  // is left to the caller's allocator (alloc_slack), so that the workspace block it holds
  // still fits
  const size_t base = fused_small_bytes(BT, V);
  const size_t slack = alloc_slack(budget);
  if (budget <= base + 4096 + slack) return t;
  const size_t avail = budget - base - 4096 - slack;  // (4096: a grad_b placeholder, aligned)
  const int64_t vpad = round_up(V, 64);
  // pass 1: vocabulary blocks with all tokens, at most as many rows as fit.  Each block's
  // grad_W GEMM is vb/64 row tiles x hchunks workgroups of equal length, about one per compute
  // unit at a time, so a grid just over a multiple of the device costs a whole extra round:
  // of the sizes from half the fit to the fit (multiples of 64), the one whose blocks take the
  // fewest rounds in all, the largest on a tie (fewest dlogits launches)
  if (BT > 0) {
    // (each stored block under 2^31 bytes: one buffer descriptor with 32-bit offsets)
    const int64_t v_fit =
        std::min<int64_t>({(int64_t)(avail / ((size_t)BT * 2)) / 64 * 64, vpad, (0x7fffffffll / (BT * 2)) / 64 * 64});
    if (v_fit < 64) return t;
    auto rounds = [&](int64_t rows) { return ((rows + 63) / 64 * t.hchunks + kPlanCUs - 1) / kPlanCUs; };
    const int64_t step = std::max<int64_t>(64, round_up(v_fit / 2 / 4096, 64));
    int64_t best_vb = v_fit, best_cost = -1;
    for (int64_t vb = v_fit; vb >= 64 && 2 * vb >= v_fit; vb -= step) {
      const int64_t cost = (V / vb) * rounds(vb) + (V % vb != 0 ? rounds(V % vb) : 0);
      if (best_cost < 0 || cost < best_cost) {
        best_vb = vb;
        best_cost = cost;
      }
    }
    t.vb = best_vb;
  } else {
    t.vb = vpad;
  }
  t.ldv = t.vb;
  const size_t pass1 = ws_align((size_t)(BT > 0 ? BT : 1) * (size_t)t.ldv * 2);
  // pass 2, candidate A: token blocks of 256 rows (the forward kernel's token tile, so its
  // dlogits GEMM wastes no MFMA work) over vocabulary blocks of vr rows, each block's grad_input
  // GEMM adding into the same fp32 partial sums (its vocabulary split into ranges: about two
  // workgroups per compute unit as far as the partial sums fit, with blocks of >= 64Ki rows or
  // the whole vocabulary, so that each dlogits launch still fills the device)
  const int64_t bt_pad = round_up(std::max<int64_t>(BT, 1), 64);
  int64_t a_tb = 0, a_grid = 0, a_vr = 0;
  int a_ns = 0;
  {
    const int64_t tbb = std::min<int64_t>(256, bt_pad);
    const int64_t base_wg = (tbb + 63) / 64 * t.hchunks;
    const int64_t vr_min = std::min<int64_t>(vpad, 65536);
    for (int64_t ns = std::min<int64_t>((512 + base_wg - 1) / base_wg, 64); ns >= 1; ns /= 2) {
      const size_t pb = ws_align((size_t)ns * (size_t)tbb * (size_t)H * 4) + kWsAlign;
      if (pb >= avail) continue;
      const int64_t vr = std::min(vpad, (int64_t)((avail - pb) / ((size_t)tbb * 2)) / 64 * 64);
      if (vr < vr_min) continue;
      // (each block's ranges are multiples of 16 rows; the first block holds the most)
      const int64_t vr0 = std::min(vr, V);
      const int64_t xs = round_up((vr0 + ns - 1) / ns, 16);
      a_tb = tbb;
      a_grid = base_wg * ((vr0 + xs - 1) / xs);
      a_ns = (int)ns;
      a_vr = vr;
      break;
    }
  }
  // candidate B: token blocks of 64 .. 1024 rows against the whole vocabulary, split into
  // ranges as above; the largest block whose grid fills the device, else the largest grid
  int64_t b_tb = 0, b_grid = 0;
  int b_ns = 0;
  for (int64_t tb = 1024; tb >= 64; tb /= 2) {
    const int64_t tbb = std::min(tb, bt_pad);
    const size_t gb = ws_align((size_t)tbb * (size_t)vpad * 2);
    if (gb >= avail) continue;
    const int64_t base_wg = (tbb + 63) / 64 * t.hchunks;
    int64_t ns = (512 + base_wg - 1) / base_wg;
    const int64_t max_ns = std::max<int64_t>(1, (V + 1023) / 1024);
    ns = std::max<int64_t>(1, std::min<int64_t>(ns, std::min<int64_t>(max_ns, 64)));
    const int64_t ns_mem = (int64_t)((avail - gb) / ((size_t)tbb * (size_t)H * 4 + kWsAlign));
    ns = std::min(ns, ns_mem);
    if (ns < 1) continue;
    const int64_t grid = base_wg * ns;
    if (b_tb == 0 || (b_grid < 256 && grid > b_grid)) {
      b_tb = tbb;
      b_grid = grid;
      b_ns = (int)ns;
    }
    if (b_grid >= 256) break;
  }
  // A unless its grid-stride GEMMs would leave more of the device idle than B's
  int64_t best_tb = 0;
  int best_ns = 0;
  if (a_tb > 0 && (b_tb == 0 || a_grid >= std::min<int64_t>(256, b_grid))) {
    best_tb = a_tb;
    best_ns = a_ns;
    t.vr = a_vr;
    t.ldt = a_vr;
  } else {
    best_tb = b_tb;
    best_ns = b_ns;
    t.vr = V;
    t.ldt = vpad;
  }
  if (best_tb == 0) return t;
  t.tb = best_tb;
  const int64_t vr0 = std::min(t.vr, V);
  t.x_split = round_up((vr0 + best_ns - 1) / best_ns, 16);
  t.nsplit = (int)((vr0 + t.x_split - 1) / t.x_split);
  // (pass 1's buffer and pass 2's buffer + partial sums overlap: the passes run one after
  // the other on the stream)
  t.g_bytes = ws_align((size_t)t.tb * (size_t)t.ldt * 2);
  t.part_bytes = ws_align((size_t)t.nsplit * (size_t)t.tb * (size_t)H * 4);
  t.bytes = 256 + std::max(pass1, t.g_bytes + t.part_bytes);
  if (t.bytes > avail + 4096) return t;
  t.on = true;
  return t;
}

hipError_t launch_sg_dinput(const FusedArgs& a, const FusedWs& w, hipStream_t st);
hipError_t launch_sg_dweight(const FusedArgs& a, const FusedWs& w, hipStream_t st);
hipError_t launch_sg_onepass(const FusedArgs& a, const FusedWs& w, hipStream_t st);

// Exact calls take the stored-operand GEMM plan; filtered and sorted calls its one-pass plan
// for filtering (flags of 256 x 64 tiles, rows through the sort's order) where that fits,
// else the plan above (the stored-dlogits GEMMs of lce_bwd.hip, 64 x 16 tiles).
static bool exact_call(const FusedArgs& a) { return !(a.filter_eps > 0.f) && a.out_row_map == nullptr; }
bool use_twopass(const FusedArgs& a) {
  if (!a.bf16) return false;
  if (exact_call(a) && sg_plan(a.BT, a.H, a.V).on) return true;
  if (!exact_call(a) && sg_plan(a.BT, a.H, a.V, kSgFiltered).on) return true;
  return a.H > 1024 && twopass_plan(a.BT, a.H, a.V).on;
}

// Gradient filtering ("Cut Cross Entropy visualized", "Gradient Filtering") in the stored-
// dlogits GEMMs: their tiles are the fused kernels' (64 tokens x 16 vocabulary entries for
// grad_input, 64 entries x 16 tokens for grad_W, aligned at 0: the blocks are multiples of
// 64 rows and the vocabulary ranges multiples of 16), tested on the stored bf16 dlogits.
static void set_filter(MatArgs& m, const FusedArgs& a, int which) {
  m.filter_eps = a.filter_eps;
  m.filter_counts = a.filter_counts != nullptr && a.filter_eps > 0.f
                        ? reinterpret_cast<unsigned long long*>(a.filter_counts + 2 * which)
                        : nullptr;
}

// Region layout: [256 B: grad_b placeholder] then pass 1: [G (vb columns)], pass 2:
// [G (all columns) | partial sums]
// With the one-pass plan the grad_input stage runs the whole backward and the grad_W stage has
// nothing left to do (unless grad_input is not asked for: then the grad_W stage runs pass 1).
hipError_t launch_twopass_dinput(const FusedArgs& a, const FusedWs& w, hipStream_t st) {
  if (exact_call(a)) {
    const SgPlan t = sg_plan(a.BT, a.H, a.V);
    if (t.on) return t.one ? launch_sg_onepass(a, w, st) : launch_sg_dinput(a, w, st);
  } else if (sg_plan(a.BT, a.H, a.V, kSgFiltered).on) {
    return launch_sg_onepass(a, w, st);
  }
  const TwoPass t = twopass_plan(a.BT, a.H, a.V);
  if (!t.on || w.big == nullptr) return hipErrorInvalidValue;
  bf16_t* g = reinterpret_cast<bf16_t*>(w.big + 256);
  float* part = reinterpret_cast<float*>(w.big + 256 + t.g_bytes);
  const bf16_t* h = static_cast<const bf16_t*>(a.hidden);
  const bf16_t* W = static_cast<const bf16_t*>(a.W);
  const bf16_t* b = static_cast<const bf16_t*>(a.bias);
  hipError_t e;
  for (int64_t t0 = 0; t0 < a.BT; t0 += t.tb) {
    const int64_t rows = std::min(t.tb, a.BT - t0);
    // vocabulary blocks of vr rows: dlogits, then their grad_input GEMM adding into the
    // partial sums of the earlier blocks (ranges of x_split rows, the first block's the most)
    for (int64_t v0 = 0; v0 < a.V; v0 += t.vr) {
      const int64_t cols = std::min(t.vr, a.V - v0);
      if ((e = launch_dlogits_block(W + v0 * a.H, h + t0 * a.H, b != nullptr ? b + v0 : nullptr, w.tok + t0, a.mu,
                                    rows, a.H, cols, v0, g, t.ldt, st)) != hipSuccess)
        return e;
      MatArgs m{};
      m.G = g;
      m.ld = t.ldt;
      m.g_rows = rows;
      m.H = a.H;
      m.hchunks = t.hchunks;
      m.n_valid = w.n_valid;
      m.mean = a.mean ? 1 : 0;
      m.X = W + v0 * a.H;
      m.nS = rows;
      m.nX = cols;
      m.x_split = t.x_split;
      m.nsplit = (int)((cols + t.x_split - 1) / t.x_split);
      m.part = part;
      m.part_add = v0 > 0 ? 1 : 0;
      set_filter(m, a, 0);
      if ((e = launch_mat_gemm(false, m, st)) != hipSuccess) return e;
    }
    if ((e = launch_mat_reduce(part, t.nsplit, rows, a.H, static_cast<bf16_t*>(a.grad_input) + t0 * a.H, w.n_valid,
                               a.mean, st)) != hipSuccess)
      return e;
  }
  return hipSuccess;
}

hipError_t launch_twopass_dweight(const FusedArgs& a, const FusedWs& w, hipStream_t st) {
  const SgPlan sp = sg_plan(a.BT, a.H, a.V, exact_call(a) ? kSgExact : kSgFiltered);
  if (sp.on) {
    if (sp.one && a.grad_input != nullptr && a.BT > 0) return hipSuccess;  // (done with grad_input)
    return launch_sg_dweight(a, w, st);
  }
  const TwoPass t = twopass_plan(a.BT, a.H, a.V);
  if (!t.on || w.big == nullptr) return hipErrorInvalidValue;
  float* gb_flag = reinterpret_cast<float*>(w.big);  // never read or written (one pass per row)
  bf16_t* g = reinterpret_cast<bf16_t*>(w.big + 256);
  const bf16_t* h = static_cast<const bf16_t*>(a.hidden);
  const bf16_t* W = static_cast<const bf16_t*>(a.W);
  const bf16_t* b = static_cast<const bf16_t*>(a.bias);
  hipError_t e;
  for (int64_t v0 = 0; v0 < a.V; v0 += t.vb) {
    const int64_t cols = std::min(t.vb, a.V - v0);
    if ((e = launch_dlogits_block(W + v0 * a.H, h, b != nullptr ? b + v0 : nullptr, w.tok, a.mu, a.BT, a.H, cols, v0,
                                  g, t.ldv, st)) != hipSuccess)
      return e;
    MatArgs m{};
    m.G = g;
    m.ld = t.ldv;
    m.g_rows = a.BT;
    m.H = a.H;
    m.hchunks = t.hchunks;
    m.n_valid = w.n_valid;
    m.mean = a.mean ? 1 : 0;
    m.X = h;
    m.nS = cols;
    m.nX = a.BT;
    m.x_split = round_up(std::max<int64_t>(a.BT, 1), 16);
    m.nsplit = 1;
    m.part = nullptr;
    m.acc = nullptr;
    m.first = 1;
    m.last = 1;
    // output rows: the block's rows in place, or (vocabulary sorting) through the order
    const int64_t o0 = a.out_row_map != nullptr ? 0 : v0;
    m.out_row_map = a.out_row_map != nullptr ? a.out_row_map + v0 : nullptr;
    if (a.grad_W != nullptr) {
      m.out_f32 = a.grad_w_f32 ? 1 : 0;
      m.out = a.grad_w_f32 ? static_cast<void*>(static_cast<float*>(a.grad_W) + o0 * a.H)
                           : static_cast<void*>(static_cast<bf16_t*>(a.grad_W) + o0 * a.H);
    }
    m.gb_acc = a.grad_b != nullptr ? gb_flag : nullptr;
    m.gb_out = a.grad_b != nullptr ? static_cast<bf16_t*>(a.grad_b) + o0 : nullptr;
    set_filter(m, a, 1);
    if ((e = launch_mat_gemm(true, m, st)) != hipSuccess) return e;
  }
  return hipSuccess;
}


// ---------------------------------------------------------------------------
// The exact (unfiltered) call runs both passes on the stored-operand GEMM (lce_sgemm.hip):
//   pass 1, per block of vb vocabulary rows: G^T = transposed dlogits of the block against all
//     tokens (forward kernel, kEpiDlogitsT), grad_W[block] = c G^T . hidden straight into the
//     output, grad_b[block] = c row sums of the dlogits (summed in fp32 by the dlogits kernel
//     per token tile of 256, then over the tiles);
//   pass 2, per block of tb tokens and vocabulary block of vr rows: G = dlogits (kEpiDlogits),
//     partial sums over K-ranges of ksplit vocabulary rows += G . W[vocabulary block]; then
//     grad_input[token block] = c * the sum of the partial sums.
// Block sizes come from a cost model in units of one 256 x 256 x 64 MFMA stage per compute
// unit: a launch costs its rounds of workgroups over the device times the stages of one of its
// tiles, plus a fixed launch cost; the dlogits kernel's tiles are 256 x 256 x H.
// ---------------------------------------------------------------------------
namespace {
// Against the pipelined kernels (H <= 1024): at H = 1024 the one-pass plan measured faster
// (backward 84.9 against 90.5 ms at the headline) and the two-pass plan slower (grad_W 56.9
// against 46.2 ms); narrower rows keep the pipelined kernels (not measured).
constexpr int64_t kSgMinH = 1024;       // the stored-operand plans from here
constexpr int64_t kSgTwoPassMinH = 1025;  // the two-pass plan from here (one pass only at 1024)
constexpr double kLaunchStages = 4.0;   // launch and drain of one kernel
constexpr double kDlFactor = 1.25;      // a dlogits tile stage against a GEMM stage (exp and stores)
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
double cost_dl(int64_t rows, int64_t cols, int64_t H) {
  const int64_t tiles = cdiv(rows, 256) * cdiv(cols, 256);
  return (double)cdiv(tiles, kPlanCUs) * (double)cdiv(H, 64) * kDlFactor + kLaunchStages;
}
double cost_gemm(int64_t M, int64_t N, int64_t K, int64_t ksplit) {
  const int64_t ns = cdiv(K, ksplit);
  const int64_t tiles = cdiv(M, 256) * cdiv(N, 256) * ns;
  return (double)cdiv(tiles, kPlanCUs) * (double)cdiv(std::min(K, ksplit), 64) + kLaunchStages;
}
// two products in one grouped launch: the longer of one tile of the first and the whole work
// spread over the device (workgroups are dispatched as compute units free up)
double cost_pair(int64_t M0, int64_t N0, int64_t K0, int64_t ks0, int64_t M1, int64_t N1, int64_t K1) {
  const double s0 = (double)cdiv(std::min(K0, ks0), 64), s1 = (double)cdiv(K1, 64);
  const double work = (double)(cdiv(M0, 256) * cdiv(N0, 256) * cdiv(K0, ks0)) * s0 +
                      (double)(cdiv(M1, 256) * cdiv(N1, 256)) * s1;
  return std::max(s0, work / (double)kPlanCUs) + kLaunchStages;
}
// streaming bytes at about 4 TB/s against a stage of about 1.4 us
double cost_bytes(double bytes) { return bytes / 4e12 / 1.4e-6; }
// tile flags of gradient filtering for blocks of vb vocabulary rows (SgPlan)
int64_t flag_ldfi(int64_t vb) { return round_up(4 * cdiv(vb, 256), 16); }
int64_t flag_ldfw(int64_t BT) { return round_up(4 * cdiv(BT, 256), 16); }
size_t flag_bytes(int64_t BT, int64_t vb) {
  return ws_align((size_t)cdiv(BT, 256) * (size_t)flag_ldfi(vb)) + ws_align((size_t)cdiv(vb, 256) * (size_t)flag_ldfw(BT));
}
}  // namespace

SgPlan sg_plan(int64_t BT, int64_t H, int64_t V, int kind, size_t reserve) {
  SgPlan t{};
  t.on = false;
  const bool filt = kind == kSgFiltered, one_only = kind != kSgExact;
  if (BT <= 0 || V <= 0 || (kind != kSgRows && H < kSgMinH)) return t;
  const size_t budget = logits_chunk_budget(BT, H, V);
  const size_t base = fused_small_bytes(BT, V);  // (as in twopass_plan)
  const size_t slack = alloc_slack(budget);
  if (budget <= base + 4096 + slack + reserve) return t;
  const size_t avail = budget - base - 4096 - slack - reserve;
  // hidden is the B operand of pass 1 (32-bit offsets)
  if ((int64_t)BT * H * 2 >= 0x7fffffffll) return t;
  // pass 1: evenly sized vocabulary blocks (multiples of 64 rows) whose G^T fits
  t.ldv = round_up(BT, 64);
  // Every stored dlogits block spans less than 2^31 bytes: its kernels address it through one
  // buffer descriptor with 32-bit offsets and park masked lanes at offset 2^31, which must lie
  // past the descriptor's range (and the grouped GEMM declines larger transposed operands).
  const int64_t g_rows_max = (0x7fffffffll / (t.ldv * 2)) / 64 * 64;
  // (grad_b: fp32 partial sums of each vocabulary row per token tile of 256)
  const size_t gb_row = (size_t)cdiv(BT, 256) * 4;
  const int64_t v_fit =
      std::min<int64_t>({(int64_t)(avail / ((size_t)t.ldv * 2)) / 64 * 64, round_up(V, 64), g_rows_max});
  if (v_fit < 64) return t;
  double best1 = -1.0, best2 = -1.0;
  if (!one_only) {  // (filtered, sorted and per-row calls take the one-pass plan below or none)
  // (with ns1 > 1 the tokens are split into K-ranges whose fp32 partial sums are reduced into
  // the grad_W rows of the block: more workgroups per block when H gives few column tiles)
  for (int64_t ns1 = 1; ns1 <= 16; ++ns1) {
    const int64_t ks1 = round_up(cdiv(BT, ns1), 64);
    if (ns1 > 1 && cdiv(BT, ks1) != ns1) continue;
    const size_t per_row = (size_t)t.ldv * 2 + (ns1 > 1 ? (size_t)ns1 * (size_t)H * 4 : 0) + gb_row;
    const int64_t fit = std::min<int64_t>({(int64_t)(avail / per_row) / 64 * 64, round_up(V, 64), g_rows_max});
    if (fit < 64) continue;
    for (int64_t nb = cdiv(V, fit); nb <= cdiv(V, fit) + 8 && nb <= cdiv(V, 64); ++nb) {
      const int64_t vb = std::min(round_up(cdiv(V, nb), 64), fit);
      const int64_t n = cdiv(V, vb), last = V - (n - 1) * vb;
      const double red = ns1 > 1 ? cost_bytes((double)V * H * (4.0 * ns1 + 4.0)) + (double)n * kLaunchStages : 0.0;
      const double c1 = (double)(n - 1) * (cost_dl(BT, vb, H) + cost_gemm(vb, H, BT, ks1)) + cost_dl(BT, last, H) +
                        cost_gemm(last, H, BT, ks1) + cost_bytes((double)V * t.ldv * 2) + red;
      if (best1 < 0 || c1 < best1) {
        best1 = c1;
        t.vb = vb;
        t.nsplit1 = (int)ns1;
        t.ksplit1 = ks1;
      }
    }
  }
  if (best1 < 0) return t;
  t.g1_bytes = ws_align((size_t)t.vb * (size_t)t.ldv * 2);
  t.part1_bytes = t.nsplit1 > 1 ? ws_align((size_t)t.nsplit1 * (size_t)t.vb * (size_t)H * 4) : 0;
  t.gb_bytes = ws_align(gb_row * (size_t)t.vb);
  const size_t pass1 = t.g1_bytes + t.part1_bytes + t.gb_bytes;
  // pass 2: token blocks tb, K-ranges of the partial sums, vocabulary blocks vr
  const int64_t bt_top = std::min<int64_t>(round_up(BT, 256), 8192);
  for (int64_t tb0 = 256; tb0 <= bt_top; tb0 *= 2) {
    const int64_t tb = std::min(tb0, BT);
    const int64_t ntb = cdiv(BT, tb), tb_last = BT - (ntb - 1) * tb;
    for (int64_t ns = 1; ns <= 64; ++ns) {
      const size_t part = ws_align((size_t)ns * (size_t)tb * (size_t)H * 4);
      if (part + 4096 >= avail) break;
      const int64_t vr_fit = std::min<int64_t>({(int64_t)((avail - part) / ((size_t)tb * 2)) / 256 * 256,
                                                round_up(V, 256), (0x7fffffffll / (tb * 2)) / 256 * 256});
      if (vr_fit < 256 || vr_fit * H * 2 >= 0x7fffffffll) continue;
      for (int64_t nvb = cdiv(V, vr_fit); nvb <= cdiv(V, vr_fit) + 3; ++nvb) {
        const int64_t vr = std::min(round_up(cdiv(V, nvb), 256), vr_fit);
        const int64_t ksplit = round_up(cdiv(vr, ns), 64);
        const int64_t n = cdiv(V, vr), last = V - (n - 1) * vr;
        // (each vocabulary block after the first reads and writes the partial sums again)
        auto block_cost = [&](int64_t rows) {
          const double pbytes = (double)cdiv(vr, ksplit) * rows * H * 4;
          return (double)(n - 1) * (cost_dl(rows, vr, H) + cost_gemm(rows, H, vr, ksplit)) +
                 cost_dl(rows, last, H) + cost_gemm(rows, H, last, ksplit) +
                 cost_bytes(pbytes * (2.0 * (double)n - 1.0) + pbytes + (double)rows * H * 2) + kLaunchStages;
        };
        const double c2 = (double)(ntb - 1) * block_cost(tb) + block_cost(tb_last);
        if (best2 < 0 || c2 < best2) {
          best2 = c2;
          t.tb = tb;
          t.vr = vr;
          t.ksplit = ksplit;
          t.nsplit = (int)cdiv(std::min(vr, V), ksplit);  // ranges of the first (largest) block
        }
      }
    }
  }
  if (best2 >= 0) {  // (else only the one-pass plan below)
    t.ldt = round_up(t.vr, 64);
    t.g_bytes = ws_align((size_t)t.tb * (size_t)t.ldt * 2);
    t.part_bytes = ws_align((size_t)t.nsplit * (size_t)t.tb * (size_t)H * 4);
    t.bytes = 256 + std::max(pass1, t.g_bytes + t.part_bytes);
    t.on = t.bytes <= avail + 4096 && H >= kSgTwoPassMinH;
  }
  }
  // One pass instead: pass 1's blocks also give grad_input, summed over the blocks as hi + lo
  // (hi in the output, lo here), so the dlogits are formed once: 8 instead of 10 BT V H flops.
  // Taken when the cost model prefers it with the smaller blocks the lo buffer leaves.
  // A filtered call also keeps the tile flags (room for them at the largest block) and takes
  // blocks of whole 256-row tiles (or one block), so that the tiles of grad_W start at multiples
  // of 256 vocabulary entries.
  const size_t lo = ws_align((size_t)BT * (size_t)H);  // (one byte of remainder per element)
  const size_t fl_res = filt ? flag_bytes(BT, round_up(V, 256)) : 0;
  if (lo + fl_res + 4096 < avail && (int64_t)BT * H * 2 < 0x7fffffffll) {
    const size_t avail1 = avail - lo - fl_res;
    double best = -1.0;
    int64_t vb1 = 0, ks1b = 0;
    int ns1b = 0;
    for (int64_t ns1 = 1; ns1 <= 16; ++ns1) {
      const int64_t ks1 = round_up(cdiv(BT, ns1), 64);
      if (ns1 > 1 && cdiv(BT, ks1) != ns1) continue;
      const size_t per_row = (size_t)t.ldv * 2 + (ns1 > 1 ? (size_t)ns1 * (size_t)H * 4 : 0) + gb_row;
      const int64_t fit = std::min<int64_t>({(int64_t)(avail1 / per_row) / 64 * 64, round_up(V, 64), g_rows_max});
      if (fit < 64) continue;
      // candidates: evenly sized blocks near the fit, and multiples of 256 rows down to half of
      // it (whole 256-row tiles: a grad_W launch of whole rounds of workgroups)
      std::vector<int64_t> cand;
      for (int64_t nb = cdiv(V, fit); nb <= cdiv(V, fit) + 8 && nb <= cdiv(V, 64); ++nb)
        cand.push_back(std::min(round_up(cdiv(V, nb), 64), fit));
      for (int64_t vb = fit / 256 * 256; vb >= 256 && 2 * vb >= fit; vb -= 256) cand.push_back(vb);
      for (const int64_t vb : cand) {
        if (filt && vb % 256 != 0 && vb < V) continue;
        const int64_t n = cdiv(V, vb), last = V - (n - 1) * vb;
        const double red = ns1 > 1 ? cost_bytes((double)V * H * (4.0 * ns1 + 4.0)) + (double)n * kLaunchStages : 0.0;
        // the running sum's traffic (3 bytes per element read and written between blocks)
        const double sum_bytes = (double)BT * H * (6.0 * (double)n - 5.0);
        // (grad_W and grad_input of a block in one grouped launch)
        const double c = (double)(n - 1) * (cost_dl(BT, vb, H) + cost_pair(vb, H, BT, ks1, BT, H, vb)) +
                         cost_dl(BT, last, H) + cost_pair(last, H, BT, ks1, BT, H, last) +
                         cost_bytes((double)V * t.ldv * 2) + red + cost_bytes(sum_bytes);
        if (best < 0 || c < best) {
          best = c;
          vb1 = vb;
          ns1b = (int)ns1;
          ks1b = ks1;
        }
      }
    }
    if (best >= 0 && (one_only || !t.on || best < best1 + best2)) {
      t.one = true;
      t.lo_bytes = lo;
      t.vb = vb1;
      t.nsplit1 = ns1b;
      t.ksplit1 = ks1b;
      t.g1_bytes = ws_align((size_t)t.vb * (size_t)t.ldv * 2);
      t.part1_bytes = t.nsplit1 > 1 ? ws_align((size_t)t.nsplit1 * (size_t)t.vb * (size_t)H * 4) : 0;
      if (filt) {
        t.ldfi = flag_ldfi(t.vb);
        t.ldfw = flag_ldfw(BT);
        t.fl_bytes = flag_bytes(BT, t.vb);
      }
      t.gb_bytes = ws_align(gb_row * (size_t)t.vb);
      t.bytes = 256 + t.g1_bytes + t.part1_bytes + t.lo_bytes + t.fl_bytes + t.gb_bytes;
      t.on = t.bytes <= avail + 4096;
    }
  }
  if (!t.on) t.one = false;
  return t;
}

hipError_t launch_sg_dinput(const FusedArgs& a, const FusedWs& w, hipStream_t st) {
  const SgPlan t = sg_plan(a.BT, a.H, a.V);
  if (!t.on || w.big == nullptr) return hipErrorInvalidValue;
  bf16_t* g = reinterpret_cast<bf16_t*>(w.big + 256);
  float* part = reinterpret_cast<float*>(w.big + 256 + t.g_bytes);
  const bf16_t* h = static_cast<const bf16_t*>(a.hidden);
  const bf16_t* W = static_cast<const bf16_t*>(a.W);
  const bf16_t* b = static_cast<const bf16_t*>(a.bias);
  hipError_t e;
  for (int64_t t0 = 0; t0 < a.BT; t0 += t.tb) {
    const int64_t rows = std::min(t.tb, a.BT - t0);
    for (int64_t v0 = 0; v0 < a.V; v0 += t.vr) {
      const int64_t cols = std::min(t.vr, a.V - v0);
      if ((e = launch_dlogits_block(W + v0 * a.H, h + t0 * a.H, b != nullptr ? b + v0 : nullptr, w.tok + t0, a.mu,
                                    rows, a.H, cols, v0, g, t.ldt, st)) != hipSuccess)
        return e;
      SgArgs m{};
      m.A = g;
      m.lda = t.ldt;
      m.B = W + v0 * a.H;
      m.ldb = a.H;
      m.M = rows;
      m.N = a.H;
      m.K = cols;
      m.ksplit = t.ksplit;
      m.nsplit = (int)((cols + t.ksplit - 1) / t.ksplit);
      m.C = part;
      m.ldc = a.H;
      m.split_stride = rows * a.H;  // (the layout mat_reduce reads: [nsplit][rows][H])
      m.accumulate = v0 > 0 ? 1 : 0;  // (a later block has at most the first block's ranges)
      if ((e = launch_sgemm(m, st)) != hipSuccess) return e;
    }
    if ((e = launch_mat_reduce(part, t.nsplit, rows, a.H, static_cast<bf16_t*>(a.grad_input) + t0 * a.H, w.n_valid,
                               a.mean, st)) != hipSuccess)
      return e;
  }
  return hipSuccess;
}

// Pass 1 (grad_W, grad_b) and, with `dinput`, grad_input in the same sweep (one-pass plan).
// Per block of vb vocabulary rows: G^T of the block against all tokens (forward kernel,
// kEpiDlogitsT); grad_W[block] = c G^T . hidden (directly, or over K-ranges of tokens into fp32
// partial sums reduced into the rows); grad_b[block] = c row sums of the fp32 dlogits (the
// dlogits kernel's sums per token tile, then a fixed-order sum over the tiles: rounding each
// dlogit to bf16 first would bias the sum when many tokens have nearly the same probability);
// with `dinput`, grad_input += G . W[block] from the same G^T read transposed, kept as hi (bf16)
// + an 8-bit remainder code between blocks and written as c * the sum by the last block.  The
// two products of a block share one launch.
// Filtered and sorted calls (their plan): with filter_eps > 0 the transposed dlogits kernel also
// flags the tiles of both products that hold a dlogit of magnitude >= filter_eps, and the GEMMs
// run the flagged K stages only (grad_b likewise sums the flagged token groups only); with the
// sort's order, the rows of grad_W and grad_b go to out_row_map[row].
// With rtok / rcy (the per-row backward), the dlogits are those of the per-row weighted sum
// (kEpiRowsDlogitsT, coefficients of rows_coef_kernel) and a.mean is false.
static hipError_t sg_sweep(const FusedArgs& a, const FusedWs& w, const SgPlan& t, bool dinput, hipStream_t st,
                           const float4* rtok = nullptr, const int32_t* rcy = nullptr) {
  bf16_t* g = reinterpret_cast<bf16_t*>(w.big + 256);
  float* part1 = reinterpret_cast<float*>(w.big + 256 + t.g1_bytes);
  uint8_t* lo = reinterpret_cast<uint8_t*>(w.big + 256 + t.g1_bytes + t.part1_bytes);
  DltExtra flt{};
  if (a.filter_eps > 0.f) {
    if (t.fl_bytes == 0) return hipErrorInvalidValue;
    flt.eps = a.filter_eps;
    flt.fin = lo + t.lo_bytes;
    flt.ldfi = t.ldfi;
    flt.fw = flt.fin + ws_align((size_t)((a.BT + 255) / 256) * (size_t)t.ldfi);
    flt.ldfw = t.ldfw;
    flt.cnt = reinterpret_cast<unsigned long long*>(a.filter_counts);
  }
  const int32_t* map = a.out_row_map;
  if (a.grad_b != nullptr) {  // (after the flags: [256 | G^T | partial sums | lo | flags | grad_b partials])
    flt.gbp = reinterpret_cast<float*>(lo + t.lo_bytes + t.fl_bytes);
    flt.ldgb = t.vb;
  }
  const bf16_t* h = static_cast<const bf16_t*>(a.hidden);
  const bf16_t* W = static_cast<const bf16_t*>(a.W);
  const bf16_t* b = static_cast<const bf16_t*>(a.bias);
  const int64_t nblk = (a.V + t.vb - 1) / t.vb;
  hipError_t e;
  for (int64_t k = 0; k < nblk; ++k) {
    const int64_t v0 = k * t.vb, rows = std::min(t.vb, a.V - v0);
    e = rtok != nullptr ? launch_rows_dlogits_block_t(W + v0 * a.H, h, b != nullptr ? b + v0 : nullptr, rtok, rcy,
                                                      a.BT, a.H, rows, v0, g, t.ldv, st, flt)
                        : launch_dlogits_block_t(W + v0 * a.H, h, b != nullptr ? b + v0 : nullptr, w.tok, a.mu, a.BT,
                                                 a.H, rows, v0, g, t.ldv, st, flt);
    if (e != hipSuccess) return e;
    void* wout = nullptr;
    const int64_t o0 = map != nullptr ? 0 : v0;  // (sorted: rows through the order)
    SgArgs mw{};  // grad_W[block] = c G^T . hidden
    if (a.grad_W != nullptr) {
      wout = a.grad_w_f32 ? static_cast<void*>(static_cast<float*>(a.grad_W) + o0 * a.H)
                          : static_cast<void*>(static_cast<bf16_t*>(a.grad_W) + o0 * a.H);
      mw.kflags = flt.fw;
      mw.ldkf = flt.ldfw;
      mw.A = g;
      mw.lda = t.ldv;
      mw.B = h;
      mw.ldb = a.H;
      mw.M = rows;
      mw.N = a.H;
      mw.K = a.BT;
      mw.ksplit = t.ksplit1;
      mw.nsplit = t.nsplit1;
      mw.n_valid = w.n_valid;
      mw.mean = a.mean ? 1 : 0;
      if (t.nsplit1 > 1) {  // K-ranges into partial sums, reduced into the rows below
        mw.C = part1;
        mw.ldc = a.H;
        mw.split_stride = rows * a.H;
      } else {
        mw.out = wout;
        mw.out_f32 = a.grad_w_f32 ? 1 : 0;
        mw.ldo = a.H;
        mw.row_map = map != nullptr ? map + v0 : nullptr;
      }
    }
    SgArgs mi{};  // grad_input += G . W[block]
    if (dinput) {
      mi.A = g;  // G^T [rows][ldv]: A = G read transposed, K = the block's vocabulary rows
      mi.lda = t.ldv;
      mi.B = W + v0 * a.H;
      mi.ldb = a.H;
      mi.M = a.BT;
      mi.N = a.H;
      mi.K = rows;
      mi.ksplit = (rows + 63) / 64 * 64;
      mi.nsplit = 1;
      mi.out = a.grad_input;
      mi.ldo = a.H;
      mi.n_valid = w.n_valid;
      mi.mean = a.mean ? 1 : 0;
      mi.hilo = nblk == 1 ? 0 : (k == 0 ? 1 : (k == nblk - 1 ? 3 : 2));
      mi.lo = lo;
      mi.ldlo = a.H;
      mi.kflags = flt.fin;
      mi.ldkf = flt.ldfi;
    }
    if (a.grad_W != nullptr && dinput) e = launch_sgemm_pair(mw, mi, st);
    else if (a.grad_W != nullptr) e = launch_sgemm(mw, st);
    else if (dinput) e = launch_sgemm_at(mi, st);
    if (e != hipSuccess) return e;
    if (a.grad_W != nullptr && t.nsplit1 > 1 &&
        (e = launch_sg_reduce(part1, t.nsplit1, rows * a.H, rows * a.H, wout, a.grad_w_f32, w.n_valid, a.mean, st,
                              map != nullptr ? map + v0 : nullptr, a.H)) != hipSuccess)
      return e;
    if (a.grad_b != nullptr &&
        (e = launch_part_sum(flt.gbp, t.vb, (a.BT + 255) / 256, rows, static_cast<bf16_t*>(a.grad_b) + o0, w.n_valid,
                             a.mean, st, map != nullptr ? map + v0 : nullptr)) != hipSuccess)
      return e;
  }
  return hipSuccess;
}

hipError_t launch_sg_dweight(const FusedArgs& a, const FusedWs& w, hipStream_t st) {
  const SgPlan t = sg_plan(a.BT, a.H, a.V, exact_call(a) ? kSgExact : kSgFiltered);
  if (!t.on || w.big == nullptr) return hipErrorInvalidValue;
  return sg_sweep(a, w, t, false, st);
}

// One-pass plan: the whole backward (grad_input and, as requested, grad_W and grad_b).
hipError_t launch_sg_onepass(const FusedArgs& a, const FusedWs& w, hipStream_t st) {
  const SgPlan t = sg_plan(a.BT, a.H, a.V, exact_call(a) ? kSgExact : kSgFiltered);
  if (!t.on || !t.one || w.big == nullptr) return hipErrorInvalidValue;
  return sg_sweep(a, w, t, a.grad_input != nullptr && a.BT > 0, st);
}

// The per-row backward on the one-pass plan (kSgRows): grad_input, grad_W and grad_b of
// sum_t gl row_loss_t + gp logprobs_t + ge entropy_t from the per-token coefficients rtok / rcy,
// with the same grouped GEMMs and running sum as the exact call.  a.mean must be false.
hipError_t launch_rows_onepass(const FusedArgs& a, const FusedWs& w, const SgPlan& t, const float4* rtok,
                               const int32_t* rcy, hipStream_t st) {
  if (!t.on || !t.one || w.big == nullptr || a.mean || rtok == nullptr || rcy == nullptr) return hipErrorInvalidValue;
  return sg_sweep(a, w, t, a.grad_input != nullptr && a.BT > 0, st, rtok, rcy);
}

}  // namespace lce
