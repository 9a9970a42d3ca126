// Internal interface between the C-ABI host layer and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lce {

constexpr size_t kWsAlign = 256;
inline size_t ws_align(size_t n) { return (n + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Forward logits tile of the fused path: vocabulary rows per tile (one partial LSE per
// token per tile is kept in the workspace) and tokens per tile.
constexpr int kFwdTileV = 256;
constexpr int kFwdTileT = 128;

// Workspace carve-up of the fused path (all offsets 256-byte aligned).
struct FusedWs {
  int64_t* n_valid;   // [1] rows with y != ignore_index and y in range
  int32_t* n_bad;     // [1] targets neither ignore_index nor in [0, V)
  float* lse_part;    // [NT][BT] per-vocab-tile log-sum-exp partials
  float* lse;         // [BT]
  float* zy;          // [BT] target logits
  double* blk;        // [2][nblk] per-block sums of ce and LSE^2 terms
  float2* tok;        // [BT] (LSE, bits of int: target + 1, or 0 for rows that contribute nothing)
  float* biasf;       // [V] the bias in fp32 (written only when there is a bias)
  int64_t nt;         // number of vocab tiles
  int64_t nblk;       // number of merge blocks
  char* big;          // the two-pass backward's buffers (bf16, H > 1024; over lse_part), or NULL
};
constexpr int kMergeThreads = 256;
// sliced merge of the per-tile partials: tokens per workgroup (one wave) and ranges of
// vocabulary tiles per token (one wave each); the fused call takes it up to kMergeSlicedMaxBT
// tokens (one pass per token, kMergeThreads tokens per workgroup, above)
constexpr int kMergeTok = 64, kMergeSlices = 16;
constexpr int64_t kMergeSlicedMaxBT = 32768;
// workgroups of the fused call's merge (one block sum pair each)
inline int64_t merge_blocks(int64_t BT) {
  return BT <= kMergeSlicedMaxBT ? (BT + kMergeTok - 1) / kMergeTok : (BT + kMergeThreads - 1) / kMergeThreads;
}

size_t fused_workspace_bytes(int64_t BT, int64_t H, int64_t V, bool bf16);
size_t fused_base_bytes(int64_t BT, int64_t V);   // small pieces + LSE partials
size_t fused_small_bytes(int64_t BT, int64_t V);  // the pieces the backward reads
// Of the one-chunk budget, what a caching allocator that rounds large blocks up to 2 MiB
// (PyTorch's does) may add to a workspace block: 2 MiB for large budgets.
inline size_t alloc_slack(size_t budget) { return budget / 64 < ((size_t)2 << 20) ? budget / 64 : ((size_t)2 << 20); }
FusedWs fused_carve(void* ws, int64_t BT, int64_t H, int64_t V, bool bf16);

// Bytes of one fp32 logits chunk of the pages' chunk-size rule ("Fused Linear Cross-Entropy:
// ...", "The chunk-size trick"): the extra-memory budget of the fused path.
size_t logits_chunk_budget(int64_t BT, int64_t H, int64_t V);

// Backward of the fused path for bf16 with H > 1024, in two passes over stored dlogits that
// fit the budget left by the forward's workspace: pass 1 (grad_W, grad_b) takes blocks of vb
// vocabulary rows with all tokens, pass 2 (grad_input) blocks of tb tokens with the whole
// vocabulary; each block's dlogits are recomputed from hidden, W and the forward's LSE by the
// forward kernel and consumed by the stored-dlogits GEMMs.  on = false: the sizes leave too
// little room, and the column-chunked kernel is used instead.
struct TwoPass {
  bool on;
  int64_t vb, ldv;          // pass 1: vocabulary rows per block, row length of its buffer
  int64_t tb, ldt;          // pass 2: tokens per block, row length of its buffer
  int64_t vr;               // pass 2: vocabulary rows per dlogits block (ldt = vr rounded up to 64)
  int64_t x_split;          // pass 2: vocabulary rows per partial-sum range within a block
  int nsplit, nb, hchunks;  // pass 2 partial sums (ranges of the first block); column plan
  size_t g_bytes, part_bytes, bytes;
};
TwoPass twopass_plan(int64_t BT, int64_t H, int64_t V);
// The same two passes on the stored-operand GEMM (exact calls): pass 1 stores each vocabulary
// block's dlogits transposed (vb rows of ldv tokens) and writes grad_W rows directly; pass 2
// takes tb tokens x vr vocabulary rows per dlogits block and sums the GEMM's K-ranges of
// ksplit rows in nsplit fp32 partial buffers.
struct SgPlan {
  bool on;
  int64_t vb, ldv, ksplit1;  // pass 1 (ksplit1 < tokens: K-ranges summed in fp32 partial buffers)
  int nsplit1;
  size_t g1_bytes, part1_bytes;
  int64_t tb, vr, ldt, ksplit;
  int nsplit;
  size_t g_bytes, part_bytes, bytes;
  // one pass: grad_input is summed over pass 1's vocabulary blocks from the same stored
  // transposed dlogits (hi in the output, lo_bytes of 8-bit remainder codes), and pass 2 is dropped
  bool one;
  size_t lo_bytes;
  // gradient filtering on the one-pass plan: per block, one byte per (256 tokens x 64
  // vocabulary entries) of grad_input (rows ldfi apart, one per token tile) and per (256
  // vocabulary entries x 64 tokens) of grad_W (rows ldfw apart, one per vocabulary tile), 1
  // where the tile holds a dlogit of magnitude >= eps
  int64_t ldfi, ldfw;
  size_t fl_bytes;
  // grad_b: per block, partial sums of the fp32 dlogits per token tile of 256 (DltExtra.gbp),
  // rows of vb floats
  size_t gb_bytes;
};
// kSgExact: the exact call's plan (H >= 1024; one pass, or two above H = 1024).
// kSgFiltered: a filtered or sorted call's (one pass only, blocks of whole 256-row tiles, room
// for the tile flags).  kSgRows: the per-row backward's (one pass only, any H).  `reserve`
// bytes of the one-chunk budget are left to the caller.  on = false if the plan does not fit.
enum SgPlanKind { kSgExact = 0, kSgFiltered = 1, kSgRows = 2 };
SgPlan sg_plan(int64_t BT, int64_t H, int64_t V, int kind = kSgExact, size_t reserve = 0);


struct FusedArgs {
  const void* hidden;
  const void* W;
  const void* bias;
  const int64_t* targets;
  int64_t BT, H, V;
  bool bf16;
  int64_t ignore_index;
  float mu;
  bool mean;
  float* loss_out;
  void* grad_input;
  void* grad_W;
  void* grad_b;
  int64_t* n_valid_out;
  float* lse_out;
  bool grad_w_f32;           // (bf16 inputs) grad_W is written in fp32
  const int32_t* out_row_map;  // grad_W / grad_b row i goes to row out_row_map[i] (or NULL)
  float filter_eps;          // > 0: gradient filtering (tiles of |dlogits| < eps are skipped)
  int64_t* filter_counts;    // [4] skipped / examined tiles of the grad_input and grad_W passes, or NULL
};

// Vocabulary sorting for the filtered call: the sorted copies and the sort's scratch.
struct SortWs {
  void* Ws;                 // [V][H] W rows in sorted order
  void* bs;                 // [V] bias in sorted order
  int64_t* ys;              // [BT] targets as sorted positions
  int32_t* perm;            // [V] id at each sorted position
  int32_t* pos;             // [V] sorted position of each id
  unsigned long long* keys; // [N] sort keys (N = power of two >= V)
  float* part;              // [nblk][H] block sums of the counted hidden rows
  float* hbar;              // [H]
  int64_t N, nblk;
};
size_t sort_workspace_bytes(int64_t BT, int64_t H, int64_t V, size_t es);
SortWs sort_carve(void* ws, int64_t BT, int64_t H, int64_t V, size_t es);
hipError_t launch_sort_vocab(const FusedArgs& a, const SortWs& s, const int64_t* n_valid, hipStream_t st);

// Stages of the fused call, in launch order.
enum Stage { kStTargets = 0, kStFwd, kStTargetLogit, kStMerge, kStLoss, kStBwdDX, kStBwdDW, kNumStages };

hipError_t launch_targets(const FusedArgs& a, const FusedWs& w, hipStream_t st);
hipError_t launch_fwd_lse(const FusedArgs& a, const FusedWs& w, hipStream_t st);
hipError_t launch_target_logit(const FusedArgs& a, const FusedWs& w, hipStream_t st);
hipError_t launch_merge(const FusedArgs& a, const FusedWs& w, hipStream_t st);
hipError_t launch_loss(const FusedArgs& a, const FusedWs& w, hipStream_t st);
hipError_t launch_bwd_dinput(const FusedArgs& a, const FusedWs& w, hipStream_t st);
hipError_t launch_bwd_dweight(const FusedArgs& a, const FusedWs& w, hipStream_t st);
hipError_t launch_twopass_dinput(const FusedArgs& a, const FusedWs& w, hipStream_t st);
hipError_t launch_twopass_dweight(const FusedArgs& a, const FusedWs& w, hipStream_t st);
// The per-row backward on the one-pass plan t (kSgRows), from per-token coefficients.
hipError_t launch_rows_onepass(const FusedArgs& a, const FusedWs& w, const SgPlan& t, const float4* rtok,
                               const int32_t* rcy, hipStream_t st);
bool use_twopass(const FusedArgs& a);

// Gradient GEMMs on stored (unscaled) dlogits G [g_rows][ld] of one token chunk.
struct MatArgs {
  const uint16_t* X;  // streamed rows [nX][H] (bf16): W (grad_input) or the chunk's hidden (grad_W)
  const uint16_t* G;  // dlogits of the chunk, row-major [g_rows][ld] (bf16)
  int64_t ld, g_rows, H;
  int64_t nS, nX;     // stationary rows (chunk tokens, resp. V) and streamed rows (V, resp. chunk tokens)
  int64_t x_split;    // streamed rows per split (multiple of 16)
  int nsplit, hchunks;
  float* part;        // grad_input: [nsplit][nS][H] fp32 partial sums
  int part_add;       // grad_input: add into the partial sums instead of overwriting them
  float* acc;         // grad_W: [V][H] fp32 sum over the chunks so far (may equal out when out_f32)
  void* out;          // grad_W output (written by the last chunk, scaled by c), or NULL
  int out_f32, first, last;
  float* gb_acc;      // grad_b: [V] fp32 sum over chunks, or NULL (no grad_b)
  uint16_t* gb_out;   // grad_b output (bf16)
  const int64_t* n_valid;
  int mean;
  const int32_t* out_row_map;  // grad_W / grad_b: output row of stationary row i (or NULL: i)
  float filter_eps;            // > 0: gradient filtering of the g tiles (as the fused kernels)
  unsigned long long* filter_counts;  // [2] skipped, examined tiles (with filter_eps > 0), or NULL
};
void mat_plan(int64_t H, int* nb, int* hchunks);
hipError_t launch_mat_gemm(bool dw, const MatArgs& a, hipStream_t st);
hipError_t launch_mat_reduce(const float* part, int nsplit, int64_t rows, int64_t H, uint16_t* out,
                             const int64_t* n_valid, bool mean, hipStream_t st);
hipError_t launch_logits_chunk(const uint16_t* W, const uint16_t* h_chunk, const uint16_t* bias, int64_t rows,
                               int64_t H, int64_t V, uint16_t* zout, int64_t ld, hipStream_t st);
hipError_t launch_rows_fused_forward(const FusedArgs& a, const FusedWs& w, float* ez_part, float* lse_out,
                                     float* logprobs, float* entropy, float* row_loss, hipStream_t st);
hipError_t launch_rows_coef(const float* lse, const float* entropy, const int64_t* y, int64_t BT, int64_t V,
                            int64_t ignore_index, float mu, const float* gl, const float* gp, const float* ge,
                            float4* rtok, int32_t* rcy, hipStream_t st);
hipError_t launch_rows_dlogits_chunk(const uint16_t* W, const uint16_t* h_chunk, const uint16_t* bias, const float4* rtok,
                                     const int32_t* rcy, int64_t rows, int64_t H, int64_t V, uint16_t* gout, int64_t ld,
                                     hipStream_t st);
hipError_t launch_dlogits_block(const uint16_t* W_block, const uint16_t* h_block, const uint16_t* bias_block,
                                const float2* tok_block, float mu, int64_t rows, int64_t H, int64_t V,
                                int64_t vbase, uint16_t* gout, int64_t ld, hipStream_t st);

// Extra outputs of the transposed dlogits kernel.
//  * Gradient filtering, with fin != NULL: tile flags as SgPlan describes them (fin[token tile *
//    ldfi + entry / 64], fw[entry / 256 * ldfw + token / 64], entries of the block), and in cnt[4]
//    the skipped and examined tiles of grad_input, then of grad_W, added to by every launch.
//  * grad_b, with gbp != NULL: per token tile of 256, the sum of each entry's fp32 dlogits over
//    the tile's tokens (with filtering, over its 64-token groups whose grad_W flag is set):
//    gbp[token tile * ldgb + entry] for the block's entries.
struct DltExtra {
  float eps;
  uint8_t* fin;
  int64_t ldfi;
  uint8_t* fw;
  int64_t ldfw;
  unsigned long long* cnt;
  float* gbp;
  int64_t ldgb;
};
hipError_t launch_dlogits_block_t(const uint16_t* W_block, const uint16_t* h, const uint16_t* bias_block,
                                  const float2* tok, float mu, int64_t rows, int64_t H, int64_t V, int64_t vbase,
                                  uint16_t* gout, int64_t ld, hipStream_t st, const DltExtra& flt = DltExtra{});
// Transposed per-row dlogits (the per-row backward's G^T), coefficients rtok / rcy per token.
hipError_t launch_rows_dlogits_block_t(const uint16_t* W_block, const uint16_t* h, const uint16_t* bias_block,
                                       const float4* rtok, const int32_t* rcy, int64_t rows, int64_t H, int64_t V,
                                       int64_t vbase, uint16_t* gout, int64_t ld, hipStream_t st,
                                       const DltExtra& ext = DltExtra{});

// Stored-operand GEMM (bf16, fp32 accumulation): C = A . B over K split into ranges of ksplit
// (a multiple of 64), one workgroup per (256 x 256 tile, range).  A [M][lda] is K-contiguous,
// B [K][ldb] N-contiguous; N a multiple of 8, rows 16-byte aligned, elements of A past K up to
// the next multiple of 8 zero.  With C: range s writes its fp32 partial sums to
// C + s * split_stride ([M][ldc]), adding to what is there if accumulate; else (one range)
// out = c * C in bf16 or fp32 (rows ldo apart), c = 1 / max(n_valid, 1) if mean, else 1.
struct SgArgs {
  const uint16_t* A;
  int64_t lda;
  const uint16_t* B;
  int64_t ldb;
  int64_t M, N, K, ksplit;
  int nsplit;
  float* C;
  int64_t ldc, split_stride;
  int accumulate;
  void* out;
  int64_t ldo;
  int out_f32;
  const int64_t* n_valid;
  int mean;
  // Running sum over several launches (bf16 out only, one K-range, N a multiple of 8): the
  // sum is kept as hi (bf16, in `out`) and an 8-bit code of the remainder s - hi in `lo` (in
  // steps of 2^-8 of hi's last place: about 16 significant bits).  hilo = 1: the first launch
  // writes both; 2: later launches add; 3: the last one adds and writes c * sum to `out`;
  // 0: plain output (c * C).
  int hilo;
  uint8_t* lo;
  int64_t ldlo;
  // Gradient filtering: K-stage s of row tile mt runs only if kflags[mt * ldkf + kb / 64 + s]
  // is 1 (kb the first K of the tile's range; flags 0 or 1; rows of ldkf bytes, a multiple of
  // 16, from a 16-byte aligned base).  NULL: every stage runs.
  const uint8_t* kflags;
  int64_t ldkf;
  // (plain output, hilo 0, one K-range) output row of each row of A: row_map[m] for m < M, or
  // NULL for row m of `out`
  const int32_t* row_map;
};
hipError_t launch_sgemm(const SgArgs& a, hipStream_t st);
// The same with A given transposed: At [K][lda] (M contiguous, a multiple of 8 elements per row
// read, elements past M zero or never stored beyond lda).
hipError_t launch_sgemm_at(const SgArgs& a, hipStream_t st);
// Both in one grid (the tiles of p0, as launch_sgemm takes it, then those of p1, A given
// transposed): the rounds of workgroups over the device are filled with both products.
hipError_t launch_sgemm_pair(const SgArgs& p0, const SgArgs& p1, hipStream_t st);
// acc[v] = (first ? 0 : acc[v]) + sum over rows of g[t][v] (bf16 rows ld apart), and with last
// out[v] = c * acc[v] in bf16.
hipError_t launch_colsum(const uint16_t* g, int64_t ld, int64_t rows, int64_t cols, float* acc, bool first, bool last,
                         uint16_t* out, const int64_t* n_valid, bool mean, hipStream_t st);
// out[i] = c * sum_s part[s * stride + i] for i < n (n a multiple of 4), in bf16 or fp32; with
// row_map, element i of row r = i / width goes to row row_map[r] of out (width a multiple of 4).
hipError_t launch_sg_reduce(const float* part, int nsplit, int64_t n, int64_t stride, void* out, bool out_f32,
                            const int64_t* n_valid, bool mean, hipStream_t st, const int32_t* row_map = nullptr,
                            int64_t width = 0);
// out[i] = c * sum_s part[s * ld + i] over nparts partial sums (fp32, in order of s), in bf16,
// for i < n; with row_map, into out[row_map[i]].
hipError_t launch_part_sum(const float* part, int64_t ld, int64_t nparts, int64_t n, uint16_t* out,
                           const int64_t* n_valid, bool mean, hipStream_t st, const int32_t* row_map = nullptr);

// Token-chunked composition (bf16): chunk rows, padded row length of the logits chunk, and
// the plan of the gradient GEMMs on it.
struct ChunkPlan {
  int64_t cs, ld, nchunks, x_split;
  int nsplit, nb, hchunks;
};
ChunkPlan chunk_plan(int64_t BT, int64_t H, int64_t V);
size_t chunked_workspace_bytes(int64_t BT, int64_t H, int64_t V, bool grad_w_fp32);
enum ChunkMode { kLoss = 0, kRowStats, kRowGrads };
struct RowsHost {  // per-row outputs ([BT], each may be NULL) and upstream gradients ([BT] or NULL)
  float* lse;
  float* logprobs;
  float* entropy;
  float* row_loss;
  const float* gl;
  const float* gp;
  const float* ge;
  const float* lse_in;  // (kRowGrads) the forward's LSE and entropy, or NULL: then the logits
  const float* ent_in;  // chunk and its per-row statistics are recomputed
};
// Bytes the per-row backward with saved forward outputs adds to the chunked workspace.
size_t rows_coef_bytes(int64_t BT);
hipError_t chunk_loop(const FusedArgs& a, ChunkMode mode, const RowsHost& io, bool grad_w_fp32,
                      bool check_targets, void* workspace, hipStream_t st, bool* bad_targets);

// Per-row outputs (LSE, target log-probability, entropy, row loss; each may be NULL) of a
// bf16 logits chunk with rows ld apart; with grad, the rows are overwritten with the dlogits
// of sum_t gl_t row_loss_t + gp_t logprobs_t + ge_t entropy_t (gl/gp/ge may be NULL = 0).
hipError_t launch_rows_stats(void* logits, const int64_t* targets, int64_t B, int64_t V, int64_t ld,
                             int64_t ignore_index, float mu, float* lse, float* logprobs, float* entropy,
                             float* row_loss, const float* gl, const float* gp, const float* ge, bool grad,
                             hipStream_t st);

// Standalone cross-entropy.
size_t ce_workspace_bytes(int64_t B);
// Rows are ld >= V elements apart; with ld > V the rows must be 16-byte aligned and the
// columns V..ld-1 are overwritten with 0.  `resident` says the logits were just written and are
// still held in the device's caches: rows longer than the register cache then take the
// two-pass streaming kernel (its second read hits cache, at full occupancy) rather than the
// single-read register+LDS kernel, which runs one 512-thread workgroup per compute unit.
enum { kCeF32 = 0, kCeBf16 = 1, kCeF16 = 2 };  // element type of the logits
hipError_t launch_ce_inplace(void* logits, int dtype, const int64_t* targets, int64_t B, int64_t V,
                             int64_t ld, int64_t ignore_index, float mu, float* ce_sum, float* z_sum,
                             int64_t* n_valid, float* lse_rows, void* workspace, bool resident,
                             hipStream_t st);

}  // namespace lce
