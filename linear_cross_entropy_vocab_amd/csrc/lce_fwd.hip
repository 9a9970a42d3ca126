// Forward half of fused linear cross-entropy on gfx950.
//
//   targets  : valid-row count (integer) and range check.
//   fwd_lse  : vocabulary-tiled logits GEMM on MFMA with a fused fp32 (max, sum-exp)
//              epilogue; one partial log-sum-exp per (vocab tile, token).  The logits
//              tile lives only in accumulator registers ("Fused Linear Cross-Entropy: The
//              Math, the Memory Wall, and Two Ways Around It", Strategy 2, forward and the
//              online-softmax update; "Cut Cross Entropy visualized", "Forward Kernel").
//   target_logit : indexed dot z_y = W[y] . h + b[y] ("Cut Cross Entropy visualized",
//              "Breakdown: Forward Pass", first kernel).
//   merge    : log-add-exp of the partials per token (the global LSE, starting from -inf),
//              per-row loss terms and fixed-order block sums.
//   loss     : final fixed-order sum and the 1/max(n_valid, 1) scale.
#include "lce_common.h"
#include "lce_launch.h"

namespace lce {

// ------------------------------------------------------------------ targets
constexpr int kTgtThreads = 1024;

// Also copies the bias to fp32 (the backward stages it per tile, 4 bytes per entry).
template <typename T>
__global__ void __launch_bounds__(kTgtThreads) targets_kernel(const int64_t* __restrict__ y, int64_t BT,
                                                               int64_t V, int64_t ignore_index,
                                                               int64_t* n_valid, int32_t* n_bad,
                                                               const T* __restrict__ bias,
                                                               float* __restrict__ biasf,
                                                               int64_t* __restrict__ filter_counts) {
  if (filter_counts != nullptr && threadIdx.x < 4) filter_counts[threadIdx.x] = 0;
  if (bias != nullptr)
    for (int64_t i = threadIdx.x; i < V; i += kTgtThreads) biasf[i] = Elem<T>::to_f(bias[i]);
  __shared__ long long s_v[kTgtThreads / kWave], s_b[kTgtThreads / kWave];
  long long nv = 0, nb = 0;
  for (int64_t i = threadIdx.x; i < BT; i += kTgtThreads) {
    const int64_t t = y[i];
    if (t != ignore_index) {
      if (t >= 0 && t < V) ++nv;
      else ++nb;
    }
  }
  nv = wave_sum_ll(nv);
  nb = wave_sum_ll(nb);
  if (threadIdx.x % kWave == 0) { s_v[threadIdx.x / kWave] = nv; s_b[threadIdx.x / kWave] = nb; }
  __syncthreads();
  if (threadIdx.x == 0) {
    long long a = 0, b = 0;
    for (int i = 0; i < kTgtThreads / kWave; ++i) { a += s_v[i]; b += s_b[i]; }
    *n_valid = a;
    *n_bad = (int32_t)(b > 0x7fffffff ? 0x7fffffff : b);
  }
}

hipError_t launch_targets(const FusedArgs& a, const FusedWs& w, hipStream_t st) {
  if (a.bf16)
    hipLaunchKernelGGL(targets_kernel<bf16_t>, dim3(1), dim3(kTgtThreads), 0, st, a.targets, a.BT, a.V,
                       a.ignore_index, w.n_valid, w.n_bad, static_cast<const bf16_t*>(a.bias), w.biasf,
                       a.filter_counts);
  else
    hipLaunchKernelGGL(targets_kernel<float>, dim3(1), dim3(kTgtThreads), 0, st, a.targets, a.BT, a.V,
                       a.ignore_index, w.n_valid, w.n_bad, static_cast<const float*>(a.bias), w.biasf,
                       a.filter_counts);
  return hipGetLastError();
}

// ------------------------------------------------------------------ fwd_lse
// Workgroup tile: kFwdTileV (256) vocabulary rows x kFwdTileT (128) tokens, computed as
// z^T = W_tile . h_tile^T so that the accumulator's register index runs over vocabulary
// rows and the per-token reduction over the vocabulary stays mostly inside each lane.
// Four waves in a 2 x 2 grid; each wave owns 128 vocab rows x 64 tokens = 4 x 2 MFMA tiles.
// K is staged through LDS 128 bytes per row at a time, double buffered.
constexpr int kFwdThreads = 256;
constexpr int kStageBytes = 128;          // K bytes per row per stage
constexpr int kLdsRow = kStageBytes + 16; // padded LDS row stride (bank-conflict free 16 B reads)


template <typename T>
__global__ void __launch_bounds__(kFwdThreads) fwd_lse_kernel(const T* __restrict__ W,
                                                               const T* __restrict__ h,
                                                               const T* __restrict__ bias,
                                                               int64_t BT, int64_t H, int64_t V,
                                                               int64_t nt_v, int64_t nt_t,
                                                               float* __restrict__ lse_part) {
  constexpr int ES = sizeof(T);
  constexpr int EPC = 16 / ES;                 // elements per 16 B chunk
  constexpr int KSTEPS = kStageBytes / (16 * ES);  // MFMA k-steps (16 elements) per stage
  constexpr int A_CH = kFwdTileV * 8 / kFwdThreads;  // 16 B chunks per thread per stage
  constexpr int B_CH = kFwdTileT * 8 / kFwdThreads;
  __shared__ __attribute__((aligned(16))) char sA[2][kFwdTileV * kLdsRow];
  __shared__ __attribute__((aligned(16))) char sB[2][kFwdTileT * kLdsRow];
  __shared__ float s_bias[kFwdTileV];
  __shared__ float red_m[2][kFwdTileT], red_s[2][kFwdTileT];

  const int64_t nwg = nt_v * nt_t;
  const int64_t id = xcd_remap(blockIdx.x, nwg);
  // grouped raster: groups of 8 token tiles, vocab tiles inside a group
  constexpr int GT = 8;
  const int64_t group = id / (GT * nt_v);
  const int64_t first_t = group * GT;
  const int64_t gsize = (nt_t - first_t) < GT ? (nt_t - first_t) : GT;
  const int64_t in_g = id % (GT * nt_v);
  const int64_t ttile = first_t + in_g % gsize;
  const int64_t vtile = in_g / gsize;
  const int64_t v0 = vtile * kFwdTileV;
  const int64_t t0 = ttile * kFwdTileT;

  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int wv = wave >> 1, wt = wave & 1;

  if (tid < kFwdTileV) {
    const int64_t v = v0 + tid;
    s_bias[tid] = (bias != nullptr && v < V) ? Elem<T>::to_f(bias[v]) : 0.f;
  }

  uint4 ra[A_CH], rb[B_CH];
  const int64_t nk = (H * ES + kStageBytes - 1) / kStageBytes;

  auto gload = [&](int64_t ks) {
    const int64_t kel0 = ks * (kStageBytes / ES);
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + kFwdThreads * i, row = c >> 3, cc = c & 7;
      const int64_t v = v0 + row, k = kel0 + cc * EPC;
      ra[i] = (v < V && k < H) ? *reinterpret_cast<const uint4*>(W + v * H + k) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + kFwdThreads * i, row = c >> 3, cc = c & 7;
      const int64_t t = t0 + row, k = kel0 + cc * EPC;
      rb[i] = (t < BT && k < H) ? *reinterpret_cast<const uint4*>(h + t * H + k) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + kFwdThreads * i, row = c >> 3, cc = c & 7;
      *reinterpret_cast<uint4*>(&sA[buf][row * kLdsRow + cc * 16]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + kFwdThreads * i, row = c >> 3, cc = c & 7;
      *reinterpret_cast<uint4*>(&sB[buf][row * kLdsRow + cc * 16]) = rb[i];
    }
  };

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int64_t ks = 0; ks < nk; ++ks) {
    const int buf = (int)(ks & 1);
    if (ks + 1 < nk) gload(ks + 1);
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
      const int boff = kk * 16 * ES + (lane >> 5) * 8 * ES;
      Frag<T> fa[4], fb[2];
#pragma unroll
      for (int vb = 0; vb < 4; ++vb)
        load8(fa[vb], reinterpret_cast<const T*>(&sA[buf][(wv * 128 + vb * 32 + (lane & 31)) * kLdsRow + boff]));
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
        load8(fb[tb], reinterpret_cast<const T*>(&sB[buf][(wt * 64 + tb * 32 + (lane & 31)) * kLdsRow + boff]));
#pragma unroll
      for (int vb = 0; vb < 4; ++vb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) mfma_32x32x16(fa[vb], fb[tb], acc[vb][tb]);
    }
    if (ks + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: per token column, (max, sum exp) over this wave's 128 vocab rows, then over
  // the two vocab halves of the tile; columns past V count as -inf (they are skipped).
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    float m = -INFINITY;
#pragma unroll
    for (int vb = 0; vb < 4; ++vb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int vr = wv * 128 + vb * 32 + acc_row(lane, r);
        if (v0 + vr < V) m = fmaxf(m, acc[vb][tb][r] + s_bias[vr]);
      }
    float s = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int vb = 0; vb < 4; ++vb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int vr = wv * 128 + vb * 32 + acc_row(lane, r);
          if (v0 + vr < V) s += __expf(acc[vb][tb][r] + s_bias[vr] - m);
        }
    }
    ms_merge(m, s, __shfl_xor(m, 32, kWave), __shfl_xor(s, 32, kWave));
    if (lane < 32) {
      red_m[wv][wt * 64 + tb * 32 + lane] = m;
      red_s[wv][wt * 64 + tb * 32 + lane] = s;
    }
  }
  __syncthreads();
  if (tid < kFwdTileT) {
    float m = red_m[0][tid], s = red_s[0][tid];
    ms_merge(m, s, red_m[1][tid], red_s[1][tid]);
    const int64_t t = t0 + tid;
    if (t < BT) lse_part[vtile * BT + t] = m + __logf(s);
  }
}

// bf16 forward: 256 vocabulary rows x 256 tokens per workgroup, 8 waves (two per SIMD, so
// one wave's epilogue and LDS traffic overlap the other's MFMAs), each wave 128 x 64.
// K is staged 64 elements (128 bytes per row) at a time by buffer->LDS DMA into a double
// buffer: every wave moves 8 KiB of the stage, rows past V or BT and K past H read as zero
// (out-of-range buffer offsets).  LDS rows are unpadded: the 16-byte fragment reads of
// this pattern are conflict free on gfx950.
constexpr int kFwdThreads2 = 512;
constexpr int kFwdTileT2 = 256;

// XOR for the 16-byte chunk index of an LDS row of 128 bytes: distinct for any 8 and any
// 16 consecutive rows.
__device__ __forceinline__ int fsw(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// MODE kEpiLse: the (max, sum-exp) epilogue, one partial LSE per (vocabulary tile, token).
// MODE kEpiLogits: the logits tile z + b is written in bf16 to zout[t][v] (rows ld elements
// apart, ld a multiple of 64 and >= V; columns V..ld-1 are written as 0): the logits chunk of
// the token-chunked composition ("Fused Linear Cross-Entropy: ...", Strategy 1).
// MODE kEpiLseEz: kEpiLse, and beside each partial LSE the tile's softmax-weighted mean logit
// sum_v e^(z_v - m) z_v / sum_v e^(z_v - m) in ez_part (for the per-row entropy).
// MODE kEpiDlogits: as kEpiLogits, but what is written is the dlogit of the summed loss,
// valid * (e^(z - LSE) (1 + 2 mu LSE) - onehot(y)), from the fp32 accumulator and the
// per-token (LSE, target + 1) of tok[] (the forward's result); vbase is the vocabulary id of
// row 0 of W (for the one-hot term when W is a block of the vocabulary).
// MODE kEpiRowsDlogits: as kEpiLogits, but what is written is the dlogit of a per-row weighted
// sum of row losses, target log-probabilities and entropies, p (alpha + beta z) - gamma [v = y],
// from the fp32 accumulator and the per-token (-LSE log2 e, alpha, beta, gamma) of rtok[] and
// target column (or -1) of rcy[].
// MODE kEpiDlogitsT: the kEpiDlogits values written transposed, G^T[v][t] (vocabulary rows of
// ld tokens; token columns BT..ld-1 are written as 0): the K-contiguous operand of the grad_W
// product G^T . hidden.
// MODE kEpiDlogitsTF: kEpiDlogitsT, and the tile flags of gradient filtering ("Cut Cross Entropy
// visualized", "Gradient Filtering") in flt: whether each 64-entry quarter of the tile (all 256
// of its tokens) and each 64-token quarter (all 256 of its entries) holds a dlogit (the fp32
// value, before rounding) of magnitude >= flt.eps; with the counts of quarters without one.
// MODE kEpiRowsDlogitsT: the kEpiRowsDlogits values written transposed, as kEpiDlogitsT writes
// its own (the grad_W operand of the per-row backward).
// GB (transposed modes): also the grad_b partial sums into flt.gbp (which is then not null).
constexpr int kEpiLse = 0, kEpiLogits = 1, kEpiDlogits = 2, kEpiLseEz = 3, kEpiRowsDlogits = 4, kEpiDlogitsT = 5,
              kEpiDlogitsTF = 6, kEpiRowsDlogitsT = 7;

// (m, s, t) with s = sum e^(z - m), t = sum e^(z - m) z, merged with a second such triple
__device__ __forceinline__ void mst_combine(float& m, float& s, float& t, float m2, float s2, float t2) {
  if (m2 > m) {
    const float f = __expf(m - m2);
    s = s * f + s2;
    t = t * f + t2;
    m = m2;
  } else if (m2 != -INFINITY) {
    const float f = __expf(m2 - m);
    s += s2 * f;
    t += t2 * f;
  }
}
template <int MODE, bool GB = false>
__global__ void __launch_bounds__(kFwdThreads2, 1) fwd_lse_dma_kernel(const bf16_t* __restrict__ W,
                                                                    const bf16_t* __restrict__ h,
                                                                    const bf16_t* __restrict__ bias,
                                                                    int64_t BT, int64_t H, int64_t V,
                                                                    int64_t nt_v, int64_t nt_t,
                                                                    float* __restrict__ lse_part,
                                                                    bf16_t* __restrict__ zout, int64_t ld,
                                                                    const float2* __restrict__ tok, float mu,
                                                                    int64_t vbase, float* __restrict__ ez_part,
                                                                    const float4* __restrict__ rtok,
                                                                    const int32_t* __restrict__ rcy, DltExtra flt) {
  constexpr bool RD = MODE == kEpiRowsDlogits || MODE == kEpiRowsDlogitsT;
  constexpr bool FLT = MODE == kEpiDlogitsTF;
  constexpr bool DLT = MODE == kEpiDlogitsT || FLT || MODE == kEpiRowsDlogitsT;
  constexpr bool DL = MODE == kEpiDlogits || MODE == kEpiDlogitsT || FLT;  // (per-token LSE and target)
  constexpr bool STORE = MODE == kEpiLogits || DL || RD;
  constexpr bool EZ = MODE == kEpiLseEz;
  constexpr int ROWB = 128;                       // bytes of one row per stage
  constexpr int TILE_A = kFwdTileV * ROWB;        // 32 KiB
  constexpr int TILE_B = kFwdTileT2 * ROWB;       // 32 KiB
  __shared__ __attribute__((aligned(1024))) char sA[2][TILE_A];
  __shared__ __attribute__((aligned(1024))) char sB[2][TILE_B];
  // Per-tile side data, loaded into LDS one tile ahead (double buffer): bf16 bias entries
  // (1 KiB region), then (DL) the tokens' (LSE, target + 1) or (RD) their coefficients and
  // target columns.
  constexpr int kSideTok = 1024, kSideRcy = kSideTok + (RD ? 16 : 8) * kFwdTileT2;
  constexpr int kSide = kSideTok + (DL ? 8 * kFwdTileT2 : 0) + (RD ? 20 * kFwdTileT2 : 0);
  __shared__ __attribute__((aligned(16))) char s_side[2][kSide];
  __shared__ float red_m[2][kFwdTileT2], red_s[2][kFwdTileT2];
  __shared__ float red_t[EZ ? 2 : 1][EZ ? kFwdTileT2 : 1];
  __shared__ int s_flw[FLT ? 8 : 1];  // (FLT) per wave: bit 0 / 1 its first / second 64 rows hold a large dlogit
  __shared__ float s_gb[DLT ? 8 : 1][DLT ? 128 : 1];  // (DLT, grad_b) per wave: its rows' sums over its 64 tokens
  // (FLT) threads 0-3: grad_input quarters (entries 64 tid ..) examined and skipped over this
  // workgroup's tiles; threads 4-7: grad_W quarters (tokens 64 (tid - 4) ..)
  unsigned long long n_exam = 0, n_skip = 0;

  const int64_t nwg = nt_v * nt_t;
  const int tid = threadIdx.x, w = wave_id(), lane = tid % kWave;
  const int wv = w >> 2, wt = w & 3;
  const int64_t row_bytes = H * 2;
  const int64_t nk = (H + 63) / 64;

  // Tiles of this workgroup: blockIdx.x, + gridDim.x, ...  Consecutive logical indices go to
  // one XCD's L2 in contiguous ranges (xcd_remap), then in groups of GT token tiles over
  // the vocabulary tiles, so that concurrently running workgroups share operand tiles.
  struct Tile {
    int64_t v0, t0, vtile;
  };
  // (32-bit scalar arithmetic: the tile counts fit, and the results stay in SGPRs)
  auto tile_of = [&](int64_t blk64) {
    const uint32_t n = (uint32_t)nwg, ntv = (uint32_t)nt_v, ntt = (uint32_t)nt_t;
    const uint32_t blk = (uint32_t)blk64;
    const uint32_t x = blk % 8, q = blk / 8, Q = n / 8, r = n % 8;
    const uint32_t id = (x < r) ? x * (Q + 1) + q : r * (Q + 1) + (x - r) * Q + q;
    constexpr uint32_t GT = 4;  // token tiles per raster group
    const uint32_t group = id / (GT * ntv);
    const uint32_t first_t = group * GT;
    const uint32_t gsize = (ntt - first_t) < GT ? (ntt - first_t) : GT;
    const uint32_t in_g = id % (GT * ntv);
    Tile t;
    t.vtile = (int64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(in_g / gsize));
    t.v0 = t.vtile * kFwdTileV;
    t.t0 = (int64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(first_t + in_g % gsize)) * kFwdTileT2;
    return t;
  };

  auto lds_addr = [](const char* p) {
    return (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
  };
  const uint32_t la = lds_addr(sA[0]), lb = lds_addr(sB[0]);
  // DMA lane mapping: instruction j of this wave covers rows 8 (4 w + j) .. + 7 of the
  // stage; lane l lands on row + l / 8, physical 16-byte chunk l % 8, which holds logical
  // chunk (l % 8) ^ fsw(row).  The swizzle makes the 16-byte fragment reads of 8 and of 16
  // consecutive rows hit distinct banks.
  const int drow = lane >> 3, dch = lane & 7;
  auto dma = [&](const Tile& tl, int64_t ks, int buf) {
    const u32x4_t ra = make_rsrc_words(W + tl.v0 * H, (V - tl.v0) * row_bytes);
    const u32x4_t rb = make_rsrc_words(h + tl.t0 * H, (BT - tl.t0) * row_bytes);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 8 * (4 * w + j) + drow;
      const int64_t k = ks * 64 + (dch ^ fsw(row)) * 8;  // first element of this lane's chunk
      const uint32_t off = k < H ? (uint32_t)(row * row_bytes + k * 2) : 0xfffffff0u;
      dma16(ra, la + (uint32_t)(buf * TILE_A + 1024 * (4 * w + j)), off);
      dma16(rb, lb + (uint32_t)(buf * TILE_B + 1024 * (4 * w + j)), off);
    }
  };

  // A tile's side data, one 16-byte load into LDS per lane from one wave each: wave 0 the
  // bias entries (from the 16-byte boundary at or below the tile's first entry: bsh entries
  // earlier), waves 1-2 the token pairs, or waves 3-6 the coefficients and wave 7 the target
  // columns.  A 16-byte load is whole or zero, so each range is taken up to the end of its last
  // 16-byte block (the token arrays' workspace regions are padded to 256 bytes; a block never
  // crosses a page); entries past V and tokens past BT are masked where they are read.
  const uint32_t lside = lds_addr(s_side[0]);
  const int bsh = (int)((reinterpret_cast<uintptr_t>(bias) & 15) >> 1);
  auto side = [&](const Tile& t1, int sb) {
    const uint32_t ls = lside + (uint32_t)(sb * kSide);
    if (w == 0 && bias != nullptr) {
      const bf16_t* b0 = bias + t1.v0 - bsh;  // 16-byte aligned
      const u32x4_t r = make_rsrc_words(b0, ((V - t1.v0 + bsh) * 2 + 15) & ~(int64_t)15);
      dma16(r, ls, lane < 33 ? (uint32_t)(16 * lane) : 0x80000000u);
    }
    if constexpr (DL) {
      if (w == 1 || w == 2) {
        const u32x4_t r = make_rsrc_words(tok + t1.t0, ((BT - t1.t0) * 8 + 15) & ~(int64_t)15);
        dma16(r, ls + kSideTok + 1024u * (w - 1), (uint32_t)(1024 * (w - 1) + 16 * lane));
      }
    }
    if constexpr (RD) {
      if (w >= 3 && w <= 6) {
        const u32x4_t r = make_rsrc_words(rtok + t1.t0, (BT - t1.t0) * 16);
        dma16(r, ls + kSideTok + 1024u * (w - 3), (uint32_t)(1024 * (w - 3) + 16 * lane));
      } else if (w == 7) {
        const u32x4_t r = make_rsrc_words(rcy + t1.t0, ((BT - t1.t0) * 4 + 15) & ~(int64_t)15);
        dma16(r, ls + kSideRcy, (uint32_t)(16 * lane));
      }
    }
  };

  // fragment rows: (wv*128 + vb*32 + lane%32) and (wt*64 + tb*32 + lane%32); the swizzle
  // depends only on row % 16 = lane % 16, so one XOR value serves every block
  const int fs = fsw(lane & 31);
  int64_t blk = blockIdx.x;
  if (blk >= nwg) return;
  Tile tl = tile_of(blk);
  int buf = 0, sb = 0;
  bool first = true;
  dma(tl, 0, 0);
  side(tl, 0);
  for (;;) {
    const bf16_t* const s_bias = reinterpret_cast<const bf16_t*>(s_side[sb]) + bsh;
    const float2* const s_tok = reinterpret_cast<const float2*>(s_side[sb] + kSideTok);
    const float4* const s_rt = reinterpret_cast<const float4*>(s_side[sb] + kSideTok);
    const int32_t* const s_rcy = reinterpret_cast<const int32_t*>(s_side[sb] + kSideRcy);
    (void)s_tok; (void)s_rt; (void)s_rcy;
    const int64_t nblk = blk + gridDim.x;
    const bool has_next = nblk < nwg;
    const Tile tn = has_next ? tile_of(nblk) : tl;
    f32x16_t acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    for (int64_t ks = 0; ks < nk; ++ks) {
      // this wave's part of stage ks (and, at ks = 0, of the tile's side data) has landed;
      // after a transposed-dlogits tile its 16 stores per lane followed these loads, and the
      // counter retires loads and stores in issue order, so they need not have completed
      if (DLT && ks == 0 && !first) vm_wait<16>();
      else vm_wait<0>();
      __syncthreads();  // stage ks is in LDS for every wave; the other buffer is no longer read
      const char* a_base = sA[buf] + (wv * 128 + (lane & 31)) * ROWB;
      const char* b_base = sB[buf] + (wt * 64 + (lane & 31)) * ROWB;
      Frag<bf16_t> fa[2][4], fb[2][2];
      auto rd = [&](int kk, int slot) {
        const int off = ((2 * kk + (lane >> 5)) ^ fs) << 4;
#pragma unroll
        for (int vb = 0; vb < 4; ++vb) lds_frag_ptr(fa[slot][vb], a_base + vb * 32 * ROWB + off);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) lds_frag_ptr(fb[slot][tb], b_base + tb * 32 * ROWB + off);
      };
      rd(0, 0);
      // the next stage, which after the last one is the first stage of the next tile (so its
      // load overlaps this tile's epilogue), issued after the first step's fragment reads so
      // that their latency overlaps the load issue
      if (ks + 1 < nk) {
        dma(tl, ks + 1, buf ^ 1);
      } else if (has_next) {
        dma(tn, 0, buf ^ 1);
        side(tn, sb ^ 1);  // (the previous tile, the last reader of that buffer, is done)
      }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk + 1 < 4) rd(kk + 1, (kk + 1) & 1);
#pragma unroll
        for (int vb = 0; vb < 4; ++vb)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) mfma_32x32x16(fa[kk & 1][vb], fb[kk & 1][tb], acc[vb][tb]);
      }
      // Pin the order: the first step's six fragment reads, then each step's eight MFMAs
      // interleaved with the next step's reads (left to itself the compiler issues each read
      // just before the MFMA that needs it, which exposes the LDS latency).
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int kk = 0; kk < 3; ++kk) {
#pragma unroll
        for (int i = 0; i < 6; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      buf ^= 1;
    }

    first = false;
    // z += b as one more MFMA step per accumulator: A holds b[row] at k = 0 (lanes 0..31,
    // the rows of the 32-row block), B holds 1 at k = 0; both bf16, so the product is exact
    // and the bias costs no per-element work in the epilogue.
    if (bias != nullptr) {
      Frag<bf16_t> fbias[4], fone;
      zero8(fone);
      if (lane < 32) fone.v[0] = (short)0x3f80;  // bf16 bits of 1.0
#pragma unroll
      for (int vb = 0; vb < 4; ++vb) {
        zero8(fbias[vb]);
        const int bi = wv * 128 + vb * 32 + lane;
        if (lane < 32 && tl.v0 + bi < V) fbias[vb].v[0] = (short)s_bias[bi];
      }
#pragma unroll
      for (int vb = 0; vb < 4; ++vb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) mfma_32x32x16(fbias[vb], fone, acc[vb][tb]);
    }
    constexpr float kLog2e = 1.4426950408889634f;
    const int vlim = (int)((V - tl.v0) < kFwdTileV ? (V - tl.v0) : kFwdTileV);
    int ln = lane;
    asm volatile("" : "+v"(ln));  // keeps the row indices below from being hoisted out of the loop
    const int vrow = wv * 128 + 4 * (ln >> 5);
    // Row vrow + c exists iff c < lim; the checks are needed in the last vocabulary tile only
    // (a wave-uniform branch) and compare with small constants.
    const int lim = vlim - vrow;
    if constexpr (DLT) {
      // Lane (t, half) holds token t's dlogits for vocabulary rows vrow + vb 32 + 8 rr + e.
      // Lanes t and t ^ 1 swap one value per pair of rows (e, e + 1), so that the even lane
      // holds row e and the odd lane row e + 1, each for both tokens; these 4-byte pairs go to
      // an LDS block of the wave's 32 rows x 64 tokens (the stage buffer the last K step read:
      // waves 0-3 in A's, 4-7 in B's), and each lane then stores 8 tokens of one row with one
      // 16-byte store.  Rows past V fall outside the store descriptor; token groups at or past
      // ld are not stored.
      constexpr int kPitch = 144;  // bytes per staged row (64 tokens and 16 bytes of padding)
      const bool odd = (ln & 1) != 0;
      const __amdgpu_buffer_rsrc_t rz = make_rsrc(zout + tl.v0 * ld, (V - tl.v0) * ld * 2);
      __syncthreads();  // every wave has read the last K step's buffers
      char* const stg = (w < 4 ? sA[buf ^ 1] : sB[buf ^ 1]) + (w & 3) * 32 * kPitch;
      // per token: the base-2 exponent offset, the factor of p (the z-loss factor, or with RD
      // alpha + beta z: fac2 = alpha, be2 = beta), the value added at the target column (-1, or
      // -gamma) and that column in this lane's rows (none if < 0)
      float ra2[2], fac2[2], be2[2], tg2[2];
      int cy2[2];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        if constexpr (RD) {
          const int tr = wt * 64 + tb * 32 + (ln & 31);
          const bool tv = tl.t0 + tr < BT;
          const float4 rt = tv ? s_rt[tr] : make_float4(-INFINITY, 0.f, 0.f, 0.f);
          const int yv = tv ? s_rcy[tr] : -1;
          ra2[tb] = rt.x;
          fac2[tb] = rt.y;
          be2[tb] = rt.z;
          tg2[tb] = -rt.w;
          cy2[tb] = yv >= 0 ? yv - (int)(vbase + tl.v0) - vrow : -1;
        } else {
          const int tr = wt * 64 + tb * 32 + (ln & 31);
          const float2 tk = tl.t0 + tr < BT ? s_tok[tr] : make_float2(0.f, 0.f);
          const int yv = __float_as_int(tk.y) - 1;
          ra2[tb] = yv >= 0 ? -tk.x * kLog2e : -INFINITY;
          fac2[tb] = 1.f + 2.f * mu * tk.x;
          be2[tb] = 0.f;
          tg2[tb] = -1.f;
          cy2[tb] = yv >= 0 ? yv - (int)(vbase + tl.v0) - vrow : -1;
        }
      }
      const int rl = ln >> 3, cl = 8 * (ln & 7);  // read-back: rows 8 i + rl, tokens cl .. cl + 7
      const int64_t tcol = tl.t0 + wt * 64 + cl;
      const bool col_ok = tcol + 8 <= ld;
      bool big[2] = {false, false};  // (FLT) a large dlogit in the wave's rows 0-63 / 64-127
      constexpr bool gbs = GB;  // (grad_b: row sums of the fp32 values)
      // byte selector of the pair exchange below: the even lane takes its own row-e value and
      // its partner's, the odd lane its partner's row-(e + 1) value and its own
      const uint32_t psel = odd ? 0x03020706u : 0x05040100u;
#pragma unroll
      for (int vb = 0; vb < 4; ++vb) {
        float rs[16];  // (grad_b) rows 8 (r / 4) + r % 4 of this vb: the sum over the lane's two tokens
#pragma unroll
        for (int r = 0; r < 16; ++r) rs[r] = 0.f;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int c0 = vb * 32 + 8 * rr;  // this lane's rows c0 .. c0 + 3 (+ vrow) of the 4-row group
            float pe[4], fe[4], z[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float a = acc[vb][tb][4 * rr + e];
              pe[e] = __builtin_amdgcn_exp2f(fmaf(a, kLog2e, ra2[tb]));
              // (RD: an entry with p = 0, e.g. a -inf logit of an entry masked by a -inf bias,
              // has dlogit 0: p (alpha + beta z) -> 0, while 0 * (beta * -inf) would be NaN)
              fe[e] = RD ? (pe[e] != 0.f ? fmaf(be2[tb], a, fac2[tb]) : 0.f) : fac2[tb];
              z[e] = fmaf(pe[e], fe[e], 0.f);
            }
            // the token's target column is at most one of the four rows, and rarely any of
            // them (a wave-divergent branch): there the target term enters the same fmaf
            const int dt = cy2[tb] - c0;
            if ((unsigned)dt < 4u) {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (e == dt) z[e] = fmaf(pe[e], fe[e], tg2[tb]);
            }
            if constexpr (FLT) {  // (rows past the block do not count; tokens past BT hold 0)
#pragma unroll
              for (int e = 0; e < 4; ++e) big[vb >> 1] = big[vb >> 1] || (c0 + e < lim && !(fabsf(z[e]) < flt.eps));
            }
            if constexpr (GB) {
#pragma unroll
              for (int e = 0; e < 4; ++e) rs[4 * rr + e] += z[e];
            }
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
              // lanes t and t ^ 1 (quad_perm (1, 0, 3, 2)) swap their packed rows e, e + 1, and
              // each keeps one row of both tokens: the even lane row e, the odd lane row e + 1
              const uint32_t pk = pack_bf2(z[e], z[e + 1]);
              const uint32_t other = (uint32_t)__builtin_amdgcn_mov_dpp((int)pk, 0xB1, 0xF, 0xF, false);
              const uint32_t v = __builtin_amdgcn_perm(other, pk, psel);
              // staged row 4 half + 8 rr + e (+1 odd), tokens tb 32 + t (even lane's t)
              const int srow = 4 * (ln >> 5) + 8 * rr + e + (odd ? 1 : 0);
              const int scol = tb * 32 + (ln & 31) - (odd ? 1 : 0);
              *reinterpret_cast<uint32_t*>(stg + srow * kPitch + 2 * scol) = v;
            }
          }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4_t q = *reinterpret_cast<const u32x4_t*>(stg + (8 * i + rl) * kPitch + 2 * cl);
          const int row = wv * 128 + vb * 32 + 8 * i + rl;  // of the tile
          const uint32_t off = col_ok ? (uint32_t)(((int64_t)row * ld + tcol) * 2) : 0x80000000u;
          __builtin_amdgcn_raw_buffer_store_b128(q, rz, (int)off, 0, 2);  // (nt: streaming)
        }
        asm volatile("" ::: "memory");  // (the block is rewritten for the next vb)
        if (gbs) {
          // Sums over the 32 lanes (tokens) of each half: four halving exchanges leave lane t
          // with row index r(t) = bits 1-4 of t (the lower half of its values kept where the
          // partner's bit is set, and the upper half where it is clear), then a last one adds
          // the partner t ^ 1's sum of the same row.
          const int t = ln & 31;
          float v8[8], v4[4], v2[2];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const bool up = (t & 16) != 0;
            v8[i] = (up ? rs[i + 8] : rs[i]) + __shfl_xor(up ? rs[i] : rs[i + 8], 16, kWave);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool up = (t & 8) != 0;
            v4[i] = (up ? v8[i + 4] : v8[i]) + __shfl_xor(up ? v8[i] : v8[i + 4], 8, kWave);
          }
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const bool up = (t & 4) != 0;
            v2[i] = (up ? v4[i + 2] : v4[i]) + __shfl_xor(up ? v4[i] : v4[i + 2], 4, kWave);
          }
          const bool up = (t & 2) != 0;
          float v1 = (up ? v2[1] : v2[0]) + __shfl_xor(up ? v2[0] : v2[1], 2, kWave);
          v1 += __shfl_xor(v1, 1, kWave);
          const int r = ((t >> 1) & 1) | (((t >> 2) & 1) << 1) | (((t >> 3) & 1) << 2) | (((t >> 4) & 1) << 3);
          if ((t & 1) == 0) s_gb[w][vb * 32 + 8 * (r >> 2) + (r & 3) + 4 * (ln >> 5)] = v1;
        }
      }
      (void)lse_part;
      if constexpr (FLT) {
        const bool b0 = __builtin_amdgcn_ballot_w64(big[0]) != 0, b1 = __builtin_amdgcn_ballot_w64(big[1]) != 0;
        if (ln == 0) s_flw[w] = (b0 ? 1 : 0) | (b1 ? 2 : 0);
      }
      // (the staging regions and the side data need no barrier here: the next tile rewrites the
      // former only after the barrier of its first K stage, the latter a tile later)
      if constexpr (FLT || GB) __syncthreads();  // every wave's flags and row sums are in LDS
      if (gbs && tid < kFwdTileV && tid < vlim) {
        // the tile's rows: the sum of the four waves' 64-token sums (with filtering, of the
        // 64-token groups whose grad_W flag is set), in order
        const int wv0 = tid >> 7, rw = tid & 127;
        float acc1 = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bool inc = true;
          if constexpr (FLT) inc = (s_flw[q] | s_flw[4 + q]) != 0;
          if (inc) acc1 += s_gb[4 * wv0 + q][rw];
        }
        flt.gbp[(tl.t0 / kFwdTileT2) * flt.ldgb + tl.v0 + tid] = acc1;
      }
      if constexpr (FLT) {
        // (s_flw and s_gb are rewritten only after the next tile's K loop and its barriers)
        if (tid < 4) {  // entries 64 tid .. of the tile against its 256 tokens: waves 4 (tid / 2) + 0..3
          const int q = tid, f = s_flw[4 * (q >> 1)] | s_flw[4 * (q >> 1) + 1] | s_flw[4 * (q >> 1) + 2] |
                                     s_flw[4 * (q >> 1) + 3];
          if (64 * q < vlim) {
            const uint8_t on = (uint8_t)((f >> (q & 1)) & 1);
            flt.fin[(tl.t0 / kFwdTileT2) * flt.ldfi + tl.vtile * 4 + q] = on;
            ++n_exam;
            n_skip += on ? 0 : 1;
          }
        } else if (tid < 8) {  // tokens 64 q .. of the tile against its 256 entries: waves q, 4 + q
          const int q = tid - 4;
          if (tl.t0 + 64 * q < BT) {
            const uint8_t on = (uint8_t)((s_flw[q] | s_flw[4 + q]) != 0 ? 1 : 0);
            flt.fw[tl.vtile * flt.ldfw + tl.t0 / 64 + q] = on;
            ++n_exam;
            n_skip += on ? 0 : 1;
          }
        }
      }
      if (!has_next) break;
      blk = nblk;
      tl = tn;
      sb ^= 1;
      continue;
    }
    if constexpr (STORE) {
      const bool full = vlim == kFwdTileV;
      // Lane (t, half) holds, per 32-row block vb, vocabulary rows 8 rr + 4 half + 0..3 for
      // rr = 0..3.  Lanes t and t + 32 swap halves so that each owns whole 8-row runs
      // (rr = 2 p + half, p = 0, 1) and writes them as 16-byte stores along the token's row.
      const int half = ln >> 5;
      const int64_t tcol0 = tl.t0 + wt * 64;
      const __amdgpu_buffer_rsrc_t rz = make_rsrc(zout + tl.t0 * ld, (BT - tl.t0) * ld * 2);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        const int trow = (int)(tcol0 - tl.t0) + tb * 32 + (ln & 31);
        // (dlogits) the token's base-2 exponent offset (-inf if it does not count), its
        // z-loss factor, and the column c of its target in this lane's rows (none if < 0)
        float ra = 0.f, fac = 0.f;
        int cy = -1;
        if constexpr (MODE == kEpiDlogits) {
          const float2 tk = tl.t0 + trow < BT ? s_tok[trow] : make_float2(0.f, 0.f);
          const int yv = __float_as_int(tk.y) - 1;
          ra = yv >= 0 ? -tk.x * kLog2e : -INFINITY;
          fac = 1.f + 2.f * mu * tk.x;
          cy = yv >= 0 ? yv - (int)(vbase + tl.v0) - vrow : -1;
        }
        float al = 0.f, be = 0.f, ga = 0.f;
        if constexpr (RD) {
          const bool tv = tl.t0 + trow < BT;
          const float4 rt = tv ? s_rt[trow] : make_float4(-INFINITY, 0.f, 0.f, 0.f);
          ra = rt.x;
          al = rt.y;
          be = rt.z;
          ga = -rt.w;
          const int yv = tv ? s_rcy[trow] : -1;
          cy = yv >= 0 ? yv - (int)(vbase + tl.v0) - vrow : -1;
        }
#pragma unroll
        for (int vb = 0; vb < 4; ++vb) {
          uint32_t pk[4][2];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            float f[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int c = vb * 32 + 8 * rr + e;
              float zv = acc[vb][tb][4 * rr + e];
              if constexpr (MODE == kEpiDlogits)
                zv = fmaf(__builtin_amdgcn_exp2f(fmaf(zv, kLog2e, ra)), fac, c == cy ? -1.f : 0.f);
              if constexpr (RD) {  // (p = 0: dlogit 0, as in the transposed form)
                const float pv = __builtin_amdgcn_exp2f(fmaf(zv, kLog2e, ra));
                zv = fmaf(pv, pv != 0.f ? fmaf(be, zv, al) : 0.f, c == cy ? ga : 0.f);
              }
              f[e] = (full || c < lim) ? zv : 0.f;
            }
            pk[rr][0] = pack_bf2(f[0], f[1]);
            pk[rr][1] = pack_bf2(f[2], f[3]);
          }
#pragma unroll
          for (int pp = 0; pp < 2; ++pp) {
            // keep run 2 pp + half, send run 2 pp + (1 - half)
            const uint32_t k0 = half ? pk[2 * pp + 1][0] : pk[2 * pp][0];
            const uint32_t k1 = half ? pk[2 * pp + 1][1] : pk[2 * pp][1];
            const uint32_t s0 = half ? pk[2 * pp][0] : pk[2 * pp + 1][0];
            const uint32_t s1 = half ? pk[2 * pp][1] : pk[2 * pp + 1][1];
            const uint32_t r0 = (uint32_t)__shfl_xor((int)s0, 32, kWave);
            const uint32_t r1 = (uint32_t)__shfl_xor((int)s1, 32, kWave);
            // the run's first four rows come from the lane with half = 0
            const uint4 v = half ? make_uint4(r0, r1, k0, k1) : make_uint4(k0, k1, r0, r1);
            const int64_t vcol = tl.v0 + wv * 128 + vb * 32 + 8 * (2 * pp + half);
            if (vcol < ld) store16(rz, (uint32_t)(trow * ld * 2 + vcol * 2), v);
          }
        }
      }
      (void)lse_part;
      if (!has_next) break;
      blk = nblk;
      tl = tn;
      sb ^= 1;
      continue;
    }
    // Epilogue: per token column, (max, sum exp) over this wave's 128 vocabulary rows, the
    // two lane halves, then the two vocabulary halves of the tile.  Rows past V (only in the
    // last vocabulary tile) are set to -inf first, so the two passes need no checks.
    if (vlim < kFwdTileV) {
#pragma unroll
      for (int vb = 0; vb < 4; ++vb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (vb * 32 + 8 * (r >> 2) + (r & 3) >= lim) acc[vb][tb][r] = -INFINITY;
    }
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      float m = -INFINITY;
#pragma unroll
      for (int vb = 0; vb < 4; ++vb)
#pragma unroll
        for (int r = 0; r < 16; ++r) m = fmaxf(m, acc[vb][tb][r]);
      float sm = 0.f, st = 0.f;
      if (m != -INFINITY) {
        // e^(z - m) = 2^(z log2 e - m log2 e): one FMA and the hardware base-2 exponential
        const float mb = m * kLog2e;
#pragma unroll
        for (int vb = 0; vb < 4; ++vb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = __builtin_amdgcn_exp2f(fmaf(acc[vb][tb][r], kLog2e, -mb));
            sm += e;
            // (rows past V hold -inf and e = 0: the product uses the largest finite value)
            if constexpr (EZ) st = fmaf(e, fmaxf(acc[vb][tb][r], -3.0e38f), st);
          }
      }
      if constexpr (EZ) {
        const float m2 = __shfl_xor(m, 32, kWave), s2 = __shfl_xor(sm, 32, kWave), t2 = __shfl_xor(st, 32, kWave);
        mst_combine(m, sm, st, m2, s2, t2);
      } else {
        ms_merge(m, sm, __shfl_xor(m, 32, kWave), __shfl_xor(sm, 32, kWave));
      }
      if (lane < 32) {
        red_m[wv][wt * 64 + tb * 32 + lane] = m;
        red_s[wv][wt * 64 + tb * 32 + lane] = sm;
        if constexpr (EZ) red_t[wv][wt * 64 + tb * 32 + lane] = st;
      }
    }
    __syncthreads();
    if (tid < kFwdTileT2) {
      float m = red_m[0][tid], sm = red_s[0][tid];
      const int64_t t = tl.t0 + tid;
      if constexpr (EZ) {
        float st = red_t[0][tid];
        mst_combine(m, sm, st, red_m[1][tid], red_s[1][tid], red_t[1][tid]);
        if (t < BT) {
          lse_part[tl.vtile * BT + t] = m + __logf(sm);
          ez_part[tl.vtile * BT + t] = sm > 0.f ? st / sm : 0.f;
        }
      } else {
        ms_merge(m, sm, red_m[1][tid], red_s[1][tid]);
        if (t < BT) lse_part[tl.vtile * BT + t] = m + __logf(sm);
      }
    }
    if (!has_next) break;
    blk = nblk;
    tl = tn;
    sb ^= 1;
  }
  if constexpr (FLT) {
    if (tid < 8 && flt.cnt != nullptr && n_exam > 0) {
      atomicAdd(&flt.cnt[tid < 4 ? 0 : 2], n_skip);
      atomicAdd(&flt.cnt[tid < 4 ? 1 : 3], n_exam);
    }
  }
  vm_wait<0>();
}

// Workgroups of the persistent forward: one per compute unit of the current device.
static int64_t fwd_grid(int64_t nwg) {
  static int cu[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cu[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cu[dev] = n;
  }
  const int64_t g = cu[dev];
  return nwg < g ? nwg : g;
}

hipError_t launch_fwd_lse(const FusedArgs& a, const FusedWs& w, hipStream_t st) {
  if (a.BT == 0) return hipSuccess;
  if (a.bf16) {
    const int64_t nt_t2 = (a.BT + kFwdTileT2 - 1) / kFwdTileT2;
    hipLaunchKernelGGL(fwd_lse_dma_kernel<kEpiLse>, dim3((unsigned)fwd_grid(w.nt * nt_t2)), dim3(kFwdThreads2), 0,
                       st, (const bf16_t*)a.W, (const bf16_t*)a.hidden, (const bf16_t*)a.bias, a.BT, a.H, a.V, w.nt,
                       nt_t2, w.lse_part, (bf16_t*)nullptr, (int64_t)0, (const float2*)nullptr, 0.f, (int64_t)0,
                       (float*)nullptr, (const float4*)nullptr, (const int32_t*)nullptr, DltExtra{});
    return hipGetLastError();
  }
  const int64_t nt_t = (a.BT + kFwdTileT - 1) / kFwdTileT;
  const int64_t n = w.nt * nt_t;
  hipLaunchKernelGGL(fwd_lse_kernel<float>, dim3((unsigned)n), dim3(kFwdThreads), 0, st,
                     (const float*)a.W, (const float*)a.hidden, (const float*)a.bias, a.BT, a.H, a.V,
                     w.nt, nt_t, w.lse_part);
  return hipGetLastError();
}

// ------------------------------------------------------------------ target_logit
constexpr int kTlWaves = 4;

template <typename T>
__global__ void __launch_bounds__(kTlWaves * kWave) target_logit_kernel(
    const T* __restrict__ h, const T* __restrict__ W, const T* __restrict__ bias,
    const int64_t* __restrict__ y, int64_t BT, int64_t H, int64_t V, int64_t ignore_index,
    float* __restrict__ zy) {
  constexpr int EPC = 16 / sizeof(T);
  const int lane = threadIdx.x % kWave;
  const int64_t t = (int64_t)blockIdx.x * kTlWaves + threadIdx.x / kWave;
  if (t >= BT) return;
  const int64_t yt = y[t];
  if (yt == ignore_index || yt < 0 || yt >= V) {
    if (lane == 0) zy[t] = 0.f;
    return;
  }
  const T* hr = h + t * H;
  const T* wr = W + yt * H;
  float acc = 0.f;
  for (int64_t c = lane; c < H / EPC; c += kWave) {
    Frag<T> fh, fw;  // 8 elements; for fp32 only the first 4 are used per chunk
    if constexpr (sizeof(T) == 2) {
      load8(fh, hr + c * EPC);
      load8(fw, wr + c * EPC);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += bf2f((bf16_t)fh.v[e]) * bf2f((bf16_t)fw.v[e]);
    } else {
      const float4 a4 = reinterpret_cast<const float4*>(hr)[c];
      const float4 b4 = reinterpret_cast<const float4*>(wr)[c];
      acc += a4.x * b4.x + a4.y * b4.y + a4.z * b4.z + a4.w * b4.w;
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) zy[t] = acc + (bias != nullptr ? Elem<T>::to_f(bias[yt]) : 0.f);
}

hipError_t launch_target_logit(const FusedArgs& a, const FusedWs& w, hipStream_t st) {
  if (a.BT == 0) return hipSuccess;
  const unsigned g = (unsigned)((a.BT + kTlWaves - 1) / kTlWaves);
  if (a.bf16)
    hipLaunchKernelGGL(target_logit_kernel<bf16_t>, dim3(g), dim3(kTlWaves * kWave), 0, st,
                       (const bf16_t*)a.hidden, (const bf16_t*)a.W, (const bf16_t*)a.bias, a.targets, a.BT,
                       a.H, a.V, a.ignore_index, w.zy);
  else
    hipLaunchKernelGGL(target_logit_kernel<float>, dim3(g), dim3(kTlWaves * kWave), 0, st,
                       (const float*)a.hidden, (const float*)a.W, (const float*)a.bias, a.targets, a.BT,
                       a.H, a.V, a.ignore_index, w.zy);
  return hipGetLastError();
}

// ------------------------------------------------------------------ merge
// Sliced merge (the per-row merge, and the fused call's for up to kMergeSlicedMaxBT tokens):
// the partials of a token are split into kMergeSlices contiguous ranges of vocabulary tiles,
// one wave per range and 64 tokens per workgroup (so that a launch of a few thousand tokens
// fills the device: one pass per token, as in merge_kernel, is bound by the latency of its
// sequential loads there), merged online within a range, four loads in flight, then across the
// ranges in order.  Tiles holding -inf are skipped as in merge_kernel.
static_assert(kMergeTok == kWave, "one wave of tokens per merge workgroup");
__device__ __forceinline__ void merge_range(const float* __restrict__ part, const float* __restrict__ ez, int64_t BT,
                                            int64_t t, int64_t k0, int64_t k1, float& m, float& s, float& te) {
  m = -INFINITY;
  s = 0.f;
  te = 0.f;
  for (int64_t k = k0; k < k1; k += 4) {
    float p[4], e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = k + i < k1 ? part[(k + i) * BT + t] : -INFINITY;
      e[i] = ez != nullptr && k + i < k1 ? ez[(k + i) * BT + t] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (p[i] == -INFINITY) continue;
      if (p[i] > m) {
        const float f = __expf(m - p[i]);
        s = s * f + 1.f;
        te = te * f + e[i];
        m = p[i];
      } else {
        const float f = __expf(p[i] - m);
        s += f;
        te = fmaf(f, e[i], te);
      }
    }
  }
}

__global__ void __launch_bounds__(kMergeThreads) merge_kernel(
    const float* __restrict__ part, int64_t nt, int64_t BT, const float* __restrict__ zy,
    const int64_t* __restrict__ y, int64_t V, int64_t ignore_index, float* __restrict__ lse,
    float* __restrict__ lse_out, double* __restrict__ blk_ce, double* __restrict__ blk_z,
    int64_t nblk, float2* __restrict__ tok) {
  __shared__ double s_a[kMergeThreads / kWave], s_b[kMergeThreads / kWave];
  const int64_t t = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  double ce = 0.0, zz = 0.0;
  if (t < BT) {
    float m = -INFINITY, s = 0.f;
    for (int64_t k = 0; k < nt; ++k) {
      const float p = part[k * BT + t];
      // a vocabulary tile with no finite logit (every entry masked by a -inf bias) holds
      // -inf and adds e^-inf = 0: skipped, so that -inf - -inf never occurs
      if (p == -INFINITY) continue;
      if (p > m) {
        s = s * __expf(m - p) + 1.f;
        m = p;
      } else {
        s += __expf(p - m);
      }
    }
    const float L = m + __logf(s);
    lse[t] = L;
    if (lse_out) lse_out[t] = L;
    const int64_t yt = y[t];
    const bool valid = yt != ignore_index && yt >= 0 && yt < V;
    if (valid) {
      ce = (double)L - (double)zy[t];
      zz = (double)L * (double)L;
    }
    tok[t] = make_float2(L, __int_as_float(valid ? (int32_t)yt + 1 : 0));
  }
  ce = wave_sum_d(ce);
  zz = wave_sum_d(zz);
  if (threadIdx.x % kWave == 0) { s_a[threadIdx.x / kWave] = ce; s_b[threadIdx.x / kWave] = zz; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double a = 0.0, b = 0.0;
    for (int i = 0; i < kMergeThreads / kWave; ++i) { a += s_a[i]; b += s_b[i]; }
    blk_ce[blockIdx.x] = a;
    blk_z[blockIdx.x] = b;
  }
}

__global__ void __launch_bounds__(kMergeTok * kMergeSlices) merge_sliced_kernel(
    const float* __restrict__ part, int64_t nt, int64_t BT, const float* __restrict__ zy,
    const int64_t* __restrict__ y, int64_t V, int64_t ignore_index, float* __restrict__ lse,
    float* __restrict__ lse_out, double* __restrict__ blk_ce, double* __restrict__ blk_z,
    float2* __restrict__ tok) {
  __shared__ float s_m[kMergeSlices][kMergeTok], s_s[kMergeSlices][kMergeTok];
  const int lane = threadIdx.x % kMergeTok, sl = threadIdx.x / kMergeTok;
  const int64_t t = (int64_t)blockIdx.x * kMergeTok + lane;
  float m = -INFINITY, s = 0.f, te;
  if (t < BT) merge_range(part, nullptr, BT, t, nt * sl / kMergeSlices, nt * (sl + 1) / kMergeSlices, m, s, te);
  s_m[sl][lane] = m;
  s_s[sl][lane] = s;
  __syncthreads();
  if (sl != 0) return;
  double ce = 0.0, zz = 0.0;
  if (t < BT) {
    m = -INFINITY;
    s = 0.f;
#pragma unroll
    for (int j = 0; j < kMergeSlices; ++j) ms_merge(m, s, s_m[j][lane], s_s[j][lane]);
    const float L = m + __logf(s);
    lse[t] = L;
    if (lse_out) lse_out[t] = L;
    const int64_t yt = y[t];
    const bool valid = yt != ignore_index && yt >= 0 && yt < V;
    if (valid) {
      ce = (double)L - (double)zy[t];
      zz = (double)L * (double)L;
    }
    tok[t] = make_float2(L, __int_as_float(valid ? (int32_t)yt + 1 : 0));
  }
  ce = wave_sum_d(ce);
  zz = wave_sum_d(zz);
  if (lane == 0) {
    blk_ce[blockIdx.x] = ce;
    blk_z[blockIdx.x] = zz;
  }
}

// One pass per token where the tokens fill the device (at the largest sizes the step measured
// no faster with the sliced merge, which alone is faster); w.nblk (merge_blocks) follows the
// choice.
hipError_t launch_merge(const FusedArgs& a, const FusedWs& w, hipStream_t st) {
  if (a.BT == 0) return hipSuccess;
  if (a.BT <= kMergeSlicedMaxBT)
    hipLaunchKernelGGL(merge_sliced_kernel, dim3((unsigned)w.nblk), dim3(kMergeTok * kMergeSlices), 0, st,
                       w.lse_part, w.nt, a.BT, w.zy, a.targets, a.V, a.ignore_index, w.lse, a.lse_out, w.blk,
                       w.blk + w.nblk, w.tok);
  else
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)w.nblk), dim3(kMergeThreads), 0, st, w.lse_part, w.nt,
                       a.BT, w.zy, a.targets, a.V, a.ignore_index, w.lse, a.lse_out, w.blk,
                       w.blk + w.nblk, w.nblk, w.tok);
  return hipGetLastError();
}

// ------------------------------------------------------------------ per-row outputs
// Per token, from the per-tile partials of the kEpiLseEz forward: LSE and the softmax-weighted
// mean logit E_p[z], then the per-row outputs of "Fused Linear Cross-Entropy: ...", Strategy 2:
// target log-probability z_y - LSE and row loss LSE - z_y + mu LSE^2 for counted rows (0
// otherwise), entropy LSE - E_p[z] for every row.
__global__ void __launch_bounds__(kMergeTok * kMergeSlices) rows_merge_kernel(
    const float* __restrict__ lse_part, const float* __restrict__ ez_part, int64_t nt, int64_t BT,
    const float* __restrict__ zy, const int64_t* __restrict__ y, int64_t V, int64_t ignore_index, float mu,
    float* __restrict__ lse_out, float* __restrict__ logprobs, float* __restrict__ entropy,
    float* __restrict__ row_loss) {
  __shared__ float s_m[kMergeSlices][kMergeTok], s_s[kMergeSlices][kMergeTok], s_t[kMergeSlices][kMergeTok];
  const int lane = threadIdx.x % kMergeTok, sl = threadIdx.x / kMergeTok;
  const int64_t t = (int64_t)blockIdx.x * kMergeTok + lane;
  float m = -INFINITY, s = 0.f, te = 0.f;
  if (t < BT) merge_range(lse_part, ez_part, BT, t, nt * sl / kMergeSlices, nt * (sl + 1) / kMergeSlices, m, s, te);
  s_m[sl][lane] = m;
  s_s[sl][lane] = s;
  s_t[sl][lane] = te;
  __syncthreads();
  if (sl != 0 || t >= BT) return;
  m = -INFINITY;
  s = 0.f;
  te = 0.f;
#pragma unroll
  for (int j = 0; j < kMergeSlices; ++j) mst_combine(m, s, te, s_m[j][lane], s_s[j][lane], s_t[j][lane]);
  const float L = m + __logf(s);
  const int64_t yt = y[t];
  const bool valid = yt != ignore_index && yt >= 0 && yt < V;
  if (lse_out) lse_out[t] = L;
  if (entropy) entropy[t] = L - te / s;
  if (logprobs) logprobs[t] = valid ? zy[t] - L : 0.f;
  if (row_loss) row_loss[t] = valid ? L - zy[t] + mu * L * L : 0.f;
}

// The per-row outputs in one pass over the vocabulary (bf16): the forward GEMM with the
// (LSE, E_p[z]) epilogue, the target-logit dot and the merge above.  The targets pre-pass
// (n_valid, range check) has run.  ez_part: [number of vocabulary tiles][BT] floats.
hipError_t launch_rows_fused_forward(const FusedArgs& a, const FusedWs& w, float* ez_part, float* lse_out,
                                     float* logprobs, float* entropy, float* row_loss, hipStream_t st) {
  if (a.BT == 0) return hipSuccess;
  const int64_t nt_t2 = (a.BT + kFwdTileT2 - 1) / kFwdTileT2;
  hipLaunchKernelGGL(fwd_lse_dma_kernel<kEpiLseEz>, dim3((unsigned)fwd_grid(w.nt * nt_t2)), dim3(kFwdThreads2), 0,
                     st, (const bf16_t*)a.W, (const bf16_t*)a.hidden, (const bf16_t*)a.bias, a.BT, a.H, a.V, w.nt,
                     nt_t2, w.lse_part, (bf16_t*)nullptr, (int64_t)0, (const float2*)nullptr, 0.f, (int64_t)0,
                     ez_part, (const float4*)nullptr, (const int32_t*)nullptr, DltExtra{});
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = launch_target_logit(a, w, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(rows_merge_kernel, dim3((unsigned)((a.BT + kMergeTok - 1) / kMergeTok)),
                     dim3(kMergeTok * kMergeSlices), 0, st, w.lse_part, ez_part, w.nt, a.BT, w.zy, a.targets, a.V,
                     a.ignore_index, a.mu, lse_out, logprobs, entropy, row_loss);
  return hipGetLastError();
}

// ------------------------------------------------------------------ loss
constexpr int kLossThreads = 256;

__global__ void __launch_bounds__(kLossThreads) loss_kernel(const double* __restrict__ blk_ce,
                                                             const double* __restrict__ blk_z,
                                                             int64_t nblk, const int64_t* __restrict__ n_valid,
                                                             float mu, int mean, float* loss_out,
                                                             int64_t* n_valid_out) {
  __shared__ double s_a[kLossThreads / kWave], s_b[kLossThreads / kWave];
  double ce = 0.0, zz = 0.0;
  for (int64_t i = threadIdx.x; i < nblk; i += kLossThreads) { ce += blk_ce[i]; zz += blk_z[i]; }
  ce = wave_sum_d(ce);
  zz = wave_sum_d(zz);
  if (threadIdx.x % kWave == 0) { s_a[threadIdx.x / kWave] = ce; s_b[threadIdx.x / kWave] = zz; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double a = 0.0, b = 0.0;
    for (int i = 0; i < kLossThreads / kWave; ++i) { a += s_a[i]; b += s_b[i]; }
    const long long n = *n_valid;
    const double c = mean ? 1.0 / (double)(n > 1 ? n : 1) : 1.0;
    *loss_out = (float)(c * (a + (double)mu * b));
    if (n_valid_out) *n_valid_out = n;
  }
}

hipError_t launch_loss(const FusedArgs& a, const FusedWs& w, hipStream_t st) {
  hipLaunchKernelGGL(loss_kernel, dim3(1), dim3(kLossThreads), 0, st, w.blk, w.blk + w.nblk, w.nblk,
                     w.n_valid, a.mu, a.mean ? 1 : 0, a.loss_out, a.n_valid_out);
  return hipGetLastError();
}

}  // namespace lce

namespace lce {

// Logits of a token chunk: zout[t][v] = (h_chunk W^T + b)[t][v] in bf16, rows ld apart.
hipError_t launch_logits_chunk(const bf16_t* W, const bf16_t* h_chunk, const bf16_t* bias, int64_t rows,
                               int64_t H, int64_t V, bf16_t* zout, int64_t ld, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const int64_t nt_v = (V + kFwdTileV - 1) / kFwdTileV;
  const int64_t nt_t2 = (rows + kFwdTileT2 - 1) / kFwdTileT2;
  hipLaunchKernelGGL(fwd_lse_dma_kernel<kEpiLogits>, dim3((unsigned)fwd_grid(nt_v * nt_t2)), dim3(kFwdThreads2), 0,
                     st, W, h_chunk, bias, rows, H, V, nt_v, nt_t2, (float*)nullptr, zout, ld, (const float2*)nullptr,
                     0.f, (int64_t)0, (float*)nullptr, (const float4*)nullptr, (const int32_t*)nullptr, DltExtra{});
  return hipGetLastError();
}

// Dlogits of the summed loss for `rows` tokens (hidden rows h_block, per-token tok_block) against
// the vocabulary rows vbase .. vbase + V - 1 (W_block = W + vbase * H, bias_block likewise or
// NULL), as bf16 rows of ld elements (columns V..ld-1 written as 0).
hipError_t launch_dlogits_block(const bf16_t* W_block, const bf16_t* h_block, const bf16_t* bias_block,
                                const float2* tok_block, float mu, int64_t rows, int64_t H, int64_t V,
                                int64_t vbase, bf16_t* gout, int64_t ld, hipStream_t st) {
  if (rows <= 0 || V <= 0) return hipSuccess;
  const int64_t nt_v = (V + kFwdTileV - 1) / kFwdTileV;
  const int64_t nt_t2 = (rows + kFwdTileT2 - 1) / kFwdTileT2;
  hipLaunchKernelGGL(fwd_lse_dma_kernel<kEpiDlogits>, dim3((unsigned)fwd_grid(nt_v * nt_t2)), dim3(kFwdThreads2), 0,
                     st, W_block, h_block, bias_block, rows, H, V, nt_v, nt_t2, (float*)nullptr, gout, ld, tok_block,
                     mu, vbase, (float*)nullptr, (const float4*)nullptr, (const int32_t*)nullptr, DltExtra{});
  return hipGetLastError();
}

// Transposed dlogits of the summed loss for the vocabulary rows vbase .. vbase + V - 1 (W_block,
// bias_block) against all `rows` tokens: gout[v][t] in bf16, rows of ld >= rows tokens (columns
// rows..ld-1 written as 0).
// With flt.fin, also the tile flags of gradient filtering; with flt.gbp, the grad_b partial
// sums (DltExtra).
hipError_t launch_dlogits_block_t(const bf16_t* W_block, const bf16_t* h, const bf16_t* bias_block,
                                  const float2* tok, float mu, int64_t rows, int64_t H, int64_t V, int64_t vbase,
                                  bf16_t* gout, int64_t ld, hipStream_t st, const DltExtra& flt) {
  if (rows <= 0 || V <= 0) return hipSuccess;
  if (V * ld * 2 > 0x7fffffffll) return hipErrorInvalidValue;
  const int64_t nt_v = (V + kFwdTileV - 1) / kFwdTileV;
  const int64_t nt_t2 = (ld + kFwdTileT2 - 1) / kFwdTileT2;
  // every grad_b partial lands inside its row
  if (flt.gbp != nullptr && flt.ldgb < V) return hipErrorInvalidValue;
  if (flt.fin != nullptr) {
    // every flag lands inside its row
    if (flt.fw == nullptr || flt.ldfi < 4 * nt_v || flt.ldfw < 4 * nt_t2) return hipErrorInvalidValue;
    auto k = flt.gbp != nullptr ? fwd_lse_dma_kernel<kEpiDlogitsTF, true> : fwd_lse_dma_kernel<kEpiDlogitsTF, false>;
    hipLaunchKernelGGL(k, dim3((unsigned)fwd_grid(nt_v * nt_t2)), dim3(kFwdThreads2), 0, st, W_block, h, bias_block,
                       rows, H, V, nt_v, nt_t2, (float*)nullptr, gout, ld, tok, mu, vbase, (float*)nullptr,
                       (const float4*)nullptr, (const int32_t*)nullptr, flt);
    return hipGetLastError();
  }
  auto k = flt.gbp != nullptr ? fwd_lse_dma_kernel<kEpiDlogitsT, true> : fwd_lse_dma_kernel<kEpiDlogitsT, false>;
  hipLaunchKernelGGL(k, dim3((unsigned)fwd_grid(nt_v * nt_t2)), dim3(kFwdThreads2), 0, st, W_block, h, bias_block,
                     rows, H, V, nt_v, nt_t2, (float*)nullptr, gout, ld, tok, mu, vbase, (float*)nullptr,
                     (const float4*)nullptr, (const int32_t*)nullptr, flt);
  return hipGetLastError();
}

// Transposed per-row dlogits (kEpiRowsDlogitsT) of the vocabulary rows vbase .. vbase + V - 1
// (W_block, bias_block) against all `rows` tokens, from the per-token coefficients rtok / rcy
// (rows_coef_kernel): gout[v][t] in bf16, rows of ld >= rows tokens (columns rows..ld-1 written
// as 0); with ext.gbp, grad_b partial sums as DltExtra describes them.
hipError_t launch_rows_dlogits_block_t(const bf16_t* W_block, const bf16_t* h, const bf16_t* bias_block,
                                       const float4* rtok, const int32_t* rcy, int64_t rows, int64_t H, int64_t V,
                                       int64_t vbase, bf16_t* gout, int64_t ld, hipStream_t st,
                                       const DltExtra& ext) {
  if (rows <= 0 || V <= 0) return hipSuccess;
  if (V * ld * 2 > 0x7fffffffll || ld < rows) return hipErrorInvalidValue;
  if (ext.fin != nullptr || (ext.gbp != nullptr && ext.ldgb < V)) return hipErrorInvalidValue;
  const int64_t nt_v = (V + kFwdTileV - 1) / kFwdTileV;
  const int64_t nt_t2 = (ld + kFwdTileT2 - 1) / kFwdTileT2;
  auto k = ext.gbp != nullptr ? fwd_lse_dma_kernel<kEpiRowsDlogitsT, true> : fwd_lse_dma_kernel<kEpiRowsDlogitsT, false>;
  hipLaunchKernelGGL(k, dim3((unsigned)fwd_grid(nt_v * nt_t2)), dim3(kFwdThreads2), 0, st, W_block, h, bias_block,
                     rows, H, V, nt_v, nt_t2, (float*)nullptr, gout, ld, (const float2*)nullptr, 0.f, vbase,
                     (float*)nullptr, rtok, rcy, ext);
  return hipGetLastError();
}

// Per-token coefficients of the per-row backward from the saved forward outputs (LSE and
// entropy, so E_p[z] = LSE - entropy): for F = sum_t gl_t row_loss_t + gp_t logprobs_t +
// ge_t entropy_t ("Fused Linear Cross-Entropy: ...", Strategy 2, per-row outputs), dF/dz_tv =
// p_tv (alpha_t + beta_t z_tv) - gamma_t [v = y_t] with
//   alpha = valid (gl (1 + 2 mu LSE) - gp) + ge E_p[z],  beta = -ge,  gamma = valid (gl - gp).
__global__ void __launch_bounds__(kMergeThreads) rows_coef_kernel(
    const float* __restrict__ lse, const float* __restrict__ entropy, const int64_t* __restrict__ y, int64_t BT,
    int64_t V, int64_t ignore_index, float mu, const float* __restrict__ gl, const float* __restrict__ gp,
    const float* __restrict__ ge, float4* __restrict__ rtok, int32_t* __restrict__ rcy) {
  const int64_t t = (int64_t)blockIdx.x * kMergeThreads + threadIdx.x;
  if (t >= BT) return;
  const int64_t yt = y[t];
  const bool valid = yt != ignore_index && yt >= 0 && yt < V;
  const float L = lse[t];
  const float ez = L - entropy[t];
  const float a = gl ? gl[t] : 0.f, b = gp ? gp[t] : 0.f, c = ge ? ge[t] : 0.f;
  const float alpha = (valid ? a * (1.f + 2.f * mu * L) - b : 0.f) + c * ez;
  const float gamma = valid ? a - b : 0.f;
  constexpr float kLog2e = 1.4426950408889634f;
  rtok[t] = make_float4(-L * kLog2e, alpha, -c, gamma);
  rcy[t] = valid ? (int32_t)yt : -1;
}

hipError_t launch_rows_coef(const float* lse, const float* entropy, const int64_t* y, int64_t BT, int64_t V,
                            int64_t ignore_index, float mu, const float* gl, const float* gp, const float* ge,
                            float4* rtok, int32_t* rcy, hipStream_t st) {
  if (BT <= 0) return hipSuccess;
  hipLaunchKernelGGL(rows_coef_kernel, dim3((unsigned)((BT + kMergeThreads - 1) / kMergeThreads)),
                     dim3(kMergeThreads), 0, st, lse, entropy, y, BT, V, ignore_index, mu, gl, gp, ge, rtok, rcy);
  return hipGetLastError();
}

// Per-row dlogits of `rows` tokens (hidden rows h_chunk, coefficients rtok/rcy of those tokens)
// against the whole vocabulary, as bf16 rows of ld elements (columns V..ld-1 written as 0).
hipError_t launch_rows_dlogits_chunk(const bf16_t* W, const bf16_t* h_chunk, const bf16_t* bias, const float4* rtok,
                                     const int32_t* rcy, int64_t rows, int64_t H, int64_t V, bf16_t* gout, int64_t ld,
                                     hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const int64_t nt_v = (V + kFwdTileV - 1) / kFwdTileV;
  const int64_t nt_t2 = (rows + kFwdTileT2 - 1) / kFwdTileT2;
  hipLaunchKernelGGL(fwd_lse_dma_kernel<kEpiRowsDlogits>, dim3((unsigned)fwd_grid(nt_v * nt_t2)), dim3(kFwdThreads2),
                     0, st, W, h_chunk, bias, rows, H, V, nt_v, nt_t2, (float*)nullptr, gout, ld, (const float2*)nullptr,
                     0.f, (int64_t)0, (float*)nullptr, rtok, rcy, DltExtra{});
  return hipGetLastError();
}

}  // namespace lce
