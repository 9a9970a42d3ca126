// Token-chunked composition of linear cross-entropy ("Fused Linear Cross-Entropy: The Math,
// the Memory Wall, and Two Ways Around It", Strategy 1 and "The chunk-size trick"; "Greyhound
// -- Cross-Entropy", "Relationship to Chunked Linear Loss"):
//
//   for each chunk of cs tokens:
//     logits chunk  z = h_chunk W^T + b           (MFMA GEMM, bf16 into one reused buffer)
//     in place      z <- valid * (softmax(z)(1 + 2 mu LSE) - onehot(y))   (standalone CE)
//     grad_input[chunk] = c * z . W                (stored-operand GEMM, lce_sgemm.hip)
//     grad_W += z^T . h_chunk,  grad_b += column sums of z   (fp32 sums over the chunks; z read
//                                                  transposed by the same GEMM)
//   loss = c * sum over chunks of (ce_sum + mu z_sum)
//
// No logits are recomputed (6 BT V H flops in all), at the price of one bf16 logits chunk and
// an fp32 grad_W accumulator in device memory.  c = 1 / max(n_valid, 1) (mean) or 1 (sum) is
// known before the first chunk from the target pre-pass, so grad_input rows are final as soon
// as their chunk is done.
#include <algorithm>

#include "lce_common.h"
#include "lce_launch.h"

namespace lce {

// Rows per chunk: the pages' rule sizes an fp32 chunk as next_pow2(ceil(BT / ceil(V / H)))
// rows; the bf16 buffer of the same byte size holds twice as many.  Rows are padded to a
// multiple of 64 elements (16-byte aligned rows for the vector loads).
ChunkPlan chunk_plan(int64_t BT, int64_t H, int64_t V) {
  ChunkPlan c;
  const int64_t inc = (V + H - 1) / H;
  const int64_t want = (BT + inc - 1) / inc;
  int64_t p2 = 1;
  while (p2 < want) p2 <<= 1;
  c.cs = std::max<int64_t>(1, std::min<int64_t>(2 * p2, BT));
  c.ld = (V + 63) / 64 * 64;
  c.nchunks = BT > 0 ? (BT + c.cs - 1) / c.cs : 0;
  mat_plan(H, &c.nb, &c.hchunks);
  // grad_input: enough vocabulary ranges for about two workgroups per compute unit
  const int64_t base = ((c.cs + 63) / 64) * c.hchunks;
  int64_t ns = (512 + base - 1) / base;
  const int64_t max_ns = std::max<int64_t>(1, (V + 1023) / 1024);  // at least 64 tiles per range
  ns = std::max<int64_t>(1, std::min<int64_t>(ns, std::min<int64_t>(max_ns, 64)));
  c.x_split = ((V + ns - 1) / ns + 15) / 16 * 16;
  c.nsplit = (int)((V + c.x_split - 1) / c.x_split);
  return c;
}

size_t chunked_workspace_bytes(int64_t BT, int64_t H, int64_t V, bool grad_w_fp32) {
  const ChunkPlan c = chunk_plan(BT, H, V);
  const int64_t nch = std::max<int64_t>(1, c.nchunks);
  size_t n = ws_align(16);                                   // n_valid, n_bad
  n += ws_align((size_t)c.cs * (size_t)c.ld * 2);            // logits / dlogits chunk
  n += ws_align(ce_workspace_bytes(c.cs));                   // per-row CE results
  n += 2 * ws_align((size_t)nch * 4) + ws_align((size_t)nch * 8);  // per-chunk sums
  n += ws_align((size_t)c.nsplit * (size_t)c.cs * (size_t)H * 4);  // grad_input partials
  if (!grad_w_fp32) n += ws_align((size_t)V * (size_t)H * 4);       // grad_W fp32 sum
  n += ws_align((size_t)V * 4);                              // grad_b fp32 sum
  return n;
}

size_t rows_coef_bytes(int64_t BT) {
  const size_t bt = (size_t)std::max<int64_t>(BT, 1);
  return ws_align(bt * 16) + ws_align(bt * 4);
}

// loss = c * sum_k (ce_k + mu z_k) over the chunks in order, in fp64.
__global__ void chunk_loss_kernel(const float* __restrict__ ce, const float* __restrict__ z, int64_t nch,
                                  const int64_t* __restrict__ n_valid, float mu, int mean, float* loss_out,
                                  int64_t* n_valid_out) {
  if (threadIdx.x != 0) return;
  double a = 0.0, b = 0.0;
  for (int64_t k = 0; k < nch; ++k) {
    a += (double)ce[k];
    b += (double)z[k];
  }
  const long long n = *n_valid;
  const double c = mean ? 1.0 / (double)(n > 1 ? n : 1) : 1.0;
  *loss_out = (float)(c * (a + (double)mu * b));
  if (n_valid_out) *n_valid_out = n;
}

// Launch sequence of the chunked calls (arguments validated by the caller; bf16 only).
//   kLoss:      loss and gradients of the mean/sum loss (the standalone CE kernel in place)
//   kRowStats:  per-row outputs only (no gradients)
//   kRowGrads:  gradients of the per-row weighted sum sum_t gl row_loss + gp logprobs + ge entropy
// *bad_targets is set when check_targets found an out-of-range target (nothing after the
// pre-pass is launched then).
hipError_t chunk_loop(const FusedArgs& a, ChunkMode mode, const RowsHost& io, bool grad_w_fp32,
                      bool check_targets, void* workspace, hipStream_t st, bool* bad_targets) {
  *bad_targets = false;
  const ChunkPlan c = chunk_plan(a.BT, a.H, a.V);
  const int64_t nch = std::max<int64_t>(1, c.nchunks);
  char* p = static_cast<char*>(workspace);
  FusedWs w{};
  w.n_valid = reinterpret_cast<int64_t*>(p);
  w.n_bad = reinterpret_cast<int32_t*>(p + 8);
  p += ws_align(16);
  bf16_t* zbuf = reinterpret_cast<bf16_t*>(p);
  p += ws_align((size_t)c.cs * (size_t)c.ld * 2);
  void* ce_ws = p;
  p += ws_align(ce_workspace_bytes(c.cs));
  float* ce_k = reinterpret_cast<float*>(p);
  p += ws_align((size_t)nch * 4);
  float* z_k = reinterpret_cast<float*>(p);
  p += ws_align((size_t)nch * 4);
  int64_t* nv_k = reinterpret_cast<int64_t*>(p);
  p += ws_align((size_t)nch * 8);
  float* part = reinterpret_cast<float*>(p);
  p += ws_align((size_t)c.nsplit * (size_t)c.cs * (size_t)a.H * 4);
  float* gw_acc = nullptr;
  if (!grad_w_fp32) {
    gw_acc = reinterpret_cast<float*>(p);
    p += ws_align((size_t)a.V * (size_t)a.H * 4);
  } else {
    gw_acc = static_cast<float*>(a.grad_W);
  }
  float* gb_acc = reinterpret_cast<float*>(p);
  p += ws_align((size_t)a.V * 4);
  // (per-row backward from saved forward outputs) per-token coefficients and target columns
  const bool saved = mode == kRowGrads && io.lse_in != nullptr && io.ent_in != nullptr;
  float4* rtok = reinterpret_cast<float4*>(p);
  int32_t* rcy = reinterpret_cast<int32_t*>(p + ws_align((size_t)std::max<int64_t>(a.BT, 1) * 16));

  // target pre-pass: n_valid (so c is known to every chunk) and the range check
  FusedArgs t = a;
  t.bias = nullptr;
  t.filter_counts = nullptr;
  hipError_t e = launch_targets(t, w, st);
  if (e != hipSuccess) return e;
  if (check_targets) {
    int32_t bad = 0;
    if ((e = hipMemcpyAsync(&bad, w.n_bad, sizeof(bad), hipMemcpyDeviceToHost, st)) != hipSuccess) return e;
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
    if (bad != 0) {
      *bad_targets = true;
      return hipSuccess;
    }
  }
  const bf16_t* h = static_cast<const bf16_t*>(a.hidden);
  const bf16_t* W = static_cast<const bf16_t*>(a.W);
  const bool grads = mode != kRowStats;
  if (saved && (e = launch_rows_coef(io.lse_in, io.ent_in, a.targets, a.BT, a.V, a.ignore_index, a.mu, io.gl, io.gp,
                                     io.ge, rtok, rcy, st)) != hipSuccess)
    return e;
  const bool want_dw = grads && (a.grad_W != nullptr || a.grad_b != nullptr);
  auto off = [](const float* q, int64_t r0) { return q ? q + r0 : nullptr; };
  auto offw = [](float* q, int64_t r0) { return q ? q + r0 : nullptr; };
  // (an empty batch still runs one chunk of 0 rows, which writes zero gradients)
  for (int64_t k = 0; k < nch; ++k) {
    const int64_t r0 = k * c.cs;
    const int64_t rows = std::max<int64_t>(0, std::min<int64_t>(c.cs, a.BT - r0));
    const bf16_t* hk = h + r0 * a.H;
    if (saved) {
      // the chunk's dlogits straight from the GEMM accumulator
      e = launch_rows_dlogits_chunk(W, hk, static_cast<const bf16_t*>(a.bias), rtok + r0, rcy + r0, rows, a.H, a.V,
                                    zbuf, c.ld, st);
    } else if ((e = launch_logits_chunk(W, hk, static_cast<const bf16_t*>(a.bias), rows, a.H, a.V, zbuf, c.ld, st)) !=
               hipSuccess) {
      return e;
    } else if (mode == kLoss) {
      e = launch_ce_inplace(zbuf, kCeBf16, a.targets + r0, rows, a.V, c.ld, a.ignore_index, a.mu, ce_k + k, z_k + k,
                            nv_k + k, offw(a.lse_out, r0), ce_ws, true, st);
    } else {
      e = launch_rows_stats(zbuf, a.targets + r0, rows, a.V, c.ld, a.ignore_index, a.mu, offw(io.lse, r0),
                            offw(io.logprobs, r0), offw(io.entropy, r0), offw(io.row_loss, r0), off(io.gl, r0),
                            off(io.gp, r0), off(io.ge, r0), mode == kRowGrads, st);
    }
    if (e != hipSuccess) return e;
    if (!grads) continue;
    const bool mean = mode == kLoss && a.mean;  // (per-row weights carry their own scale)
    if (a.grad_input != nullptr && rows > 0) {
      // grad_input[chunk] = c * G . W on the stored-operand GEMM: the vocabulary split into
      // K-ranges (about one workgroup per compute unit, within the partial buffers), summed by
      // mat_reduce
      SgArgs m{};
      m.A = zbuf;
      m.lda = c.ld;
      m.B = W;
      m.ldb = a.H;
      m.M = rows;
      m.N = a.H;
      m.K = a.V;
      const int64_t tiles = ((rows + 255) / 256) * ((a.H + 255) / 256);
      const int64_t ns = std::max<int64_t>(1, std::min<int64_t>(c.nsplit, (256 + tiles - 1) / tiles));
      m.ksplit = ((a.V + ns - 1) / ns + 63) / 64 * 64;
      m.nsplit = (int)((a.V + m.ksplit - 1) / m.ksplit);
      m.C = part;
      m.ldc = a.H;
      m.split_stride = rows * a.H;
      if ((e = launch_sgemm(m, st)) != hipSuccess) return e;
      if ((e = launch_mat_reduce(part, m.nsplit, rows, a.H, static_cast<bf16_t*>(a.grad_input) + r0 * a.H, w.n_valid,
                                 mean, st)) != hipSuccess)
        return e;
    }
    if (want_dw && a.grad_W != nullptr) {
      // grad_W sum over chunks += G^T . h_chunk (G read transposed), in fp32
      SgArgs m{};
      m.A = zbuf;
      m.lda = c.ld;
      m.B = hk;
      m.ldb = a.H;
      m.M = a.V;
      m.N = a.H;
      m.K = rows;
      m.ksplit = std::max<int64_t>(64, (rows + 63) / 64 * 64);
      m.nsplit = 1;
      m.C = gw_acc;
      m.ldc = a.H;
      m.split_stride = 0;
      m.accumulate = k > 0 ? 1 : 0;
      if ((e = launch_sgemm_at(m, st)) != hipSuccess) return e;
      if (k == nch - 1 && (e = launch_sg_reduce(gw_acc, 1, a.V * a.H, a.V * a.H, a.grad_W, grad_w_fp32, w.n_valid,
                                                mean, st)) != hipSuccess)
        return e;
    }
    if (want_dw && a.grad_b != nullptr &&
        (e = launch_colsum(zbuf, c.ld, rows, a.V, gb_acc, k == 0, k == nch - 1, static_cast<bf16_t*>(a.grad_b),
                           w.n_valid, mean, st)) != hipSuccess)
      return e;
  }
  if (mode == kLoss) {
    hipLaunchKernelGGL(chunk_loss_kernel, dim3(1), dim3(64), 0, st, ce_k, z_k, nch, w.n_valid, a.mu,
                       a.mean ? 1 : 0, a.loss_out, a.n_valid_out);
    return hipGetLastError();
  }
  if (a.n_valid_out != nullptr)
    return hipMemcpyAsync(a.n_valid_out, w.n_valid, sizeof(int64_t), hipMemcpyDeviceToDevice, st);
  return hipSuccess;
}

}  // namespace lce
