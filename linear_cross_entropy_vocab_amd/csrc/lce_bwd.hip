// Backward half of fused linear cross-entropy on gfx950: grad_input and grad_W (+ grad_b)
// with the dlogits tiles recomputed on chip and consumed by MFMA without ever reaching HBM.
//
// Math ("Fused Linear Cross-Entropy: The Math, the Memory Wall, and Two Ways Around It",
// "From dlogits to grad_input and grad_W" and "Why two passes"; "Cut Cross Entropy
// visualized", "Breakdown: Backward Pass"):
//   z = S . X^T (+ b),   g = valid * (exp(z - LSE) * (1 + 2 mu LSE) - onehot(y)),
//   acc += g . X,        output = c * acc,  c = 1/max(n_valid, 1) (mean) or 1 (sum).
// grad_input: S = hidden rows (stationary), X = W rows (streamed over the vocabulary).
// grad_W:     S = W rows (stationary),      X = hidden rows (streamed over tokens);
//             grad_b is the row sum of g in the same pass.
// Each workgroup owns 64 stationary rows and an output column range, and reduces over the
// whole streamed dimension itself, so no partial results or atomics are needed.  The
// price is recomputing z once per output (the "recompute" option of "Why two passes").
//
// Workgroup layout (4 waves, one per SIMD):
//   GEMM1 z[64 x 32] = S[64 x H] . X[32 x H]^T, K split across the waves (wave w owns a
//          quarter of H); each wave's partial z goes through LDS and is summed per row.
//   dlogits: each wave forms g for 16 rows x 32 columns and writes it to LDS as the A
//          operand of GEMM3 (bf16 rounded to nearest even for bf16 inputs, fp32 otherwise).
//   GEMM3 acc[64 x NCOL] += g[64 x 32] . X[32 x NCOL] for the wave's own NCOL output
//          columns; the X operand is read from LDS with ds_read_b64_tr_b16 (bf16).
// When the whole of H fits one workgroup (H <= 1024), wave w's K quarter and its output
// columns coincide, so the X rows loaded for GEMM1 are the ones GEMM3 needs, and the
// stationary S fragments stay in registers for the whole sweep.
#include <type_traits>

#include "lce_common.h"
#include "lce_launch.h"

namespace lce {

constexpr int kBwdThreads = 256;
constexpr int kBS = 64;  // stationary rows per workgroup
constexpr int kBX = 32;  // streamed rows per tile

template <typename T>
struct BwdArgs {
  const T* S;
  const T* X;
  const T* bias;
  const int64_t* y;
  const float* lse;
  const float2* tok;  // per token: (LSE, target + 1, or 0 for rows that contribute nothing)
  const float* biasf;  // bias in fp32, or NULL
  float filter_eps;     // > 0: skip the GEMM3 work of tiles whose |g| are all below it
  unsigned long long* filter_counts;  // [2] skipped / examined tiles (atomics), or NULL
  int64_t nS, nX, H, BT, V;
  int64_t ignore_index;
  float mu;
  const int64_t* n_valid;
  int mean;
  T* out;
  float* out_f32;  // (bf16 inputs) fp32 output instead of out, or NULL
  const int32_t* out_row_map;  // (grad_W) output row of each stationary row, or NULL (same row)
  T* grad_b;
  int64_t nchunks;
};

__device__ __forceinline__ void store8(char* p, const float* v, bf16_t) {
  *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]),
                                            pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7]));
}
__device__ __forceinline__ void store8(char* p, const float* v, float) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void store4(char* p, const float* v, bf16_t) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
}
__device__ __forceinline__ void store4(char* p, const float* v, float) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void lds_frag(Frag<bf16_t>& f, const char* p) {
  f.v = *reinterpret_cast<const bf16x8_t*>(p);
}
__device__ __forceinline__ void lds_frag(Frag<float>& f, const char* p) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// LDS tiles read by GEMM3 are row-major with a row stride of 64 (mod 256) bytes and the low
// two bits of the 16-byte chunk index XORed with bits 2..3 of the row.  Sixteen consecutive
// rows then cover all 64 banks for 16-byte stores, while the four consecutive rows of a
// transposed read (same bits 2..3) keep the conflict-free layout of the padded stride, and
// column offsets that are multiples of 64 bytes stay immediate offsets.
template <int ROW, int NCH>
__device__ __forceinline__ int swz(int row, int byte_col) {
  static_assert(NCH % 4 == 0, "rows must hold a multiple of four 16-byte chunks");
  return row * ROW + ((((byte_col >> 4) ^ ((row >> 2) & 3)) << 4) | (byte_col & 15));
}

// Store an 8-element fragment (one 16-byte chunk for bf16, two for fp32) into a swizzled tile.
template <int ROW, int NCH>
__device__ __forceinline__ void store_frag(char* t, int row, int byte_col, const Frag<bf16_t>& f) {
  *reinterpret_cast<bf16x8_t*>(t + swz<ROW, NCH>(row, byte_col)) = f.v;
}
template <int ROW, int NCH>
__device__ __forceinline__ void store_frag(char* t, int row, int byte_col, const Frag<float>& f) {
  *reinterpret_cast<float4*>(t + swz<ROW, NCH>(row, byte_col)) = make_float4(f.v[0], f.v[1], f.v[2], f.v[3]);
  *reinterpret_cast<float4*>(t + swz<ROW, NCH>(row, byte_col + 16)) = make_float4(f.v[4], f.v[5], f.v[6], f.v[7]);
}

// MFMA operand from a swizzled row-major LDS tile whose rows run along K: lane l needs
// column (l % 32) of a 32-column block starting at col0 and K rows kbase + 8*(l/32) .. +7.
template <int ROW, int NCH>
__device__ __forceinline__ void tile_frag(Frag<bf16_t>& f, const char* t, int kbase, int col0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int col = col0 + (g & 1) * 16 + 4 * (i & 3);
  const int row = kbase + (g >> 1) * 8 + (i >> 2);
  const i16x4_t a = lds_read_tr16(reinterpret_cast<const bf16_t*>(t + swz<ROW, NCH>(row, col * 2)));
  const i16x4_t b = lds_read_tr16(reinterpret_cast<const bf16_t*>(t + swz<ROW, NCH>(row + 4, col * 2)));
  f.v = bf16x8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
template <int ROW, int NCH>
__device__ __forceinline__ void tile_frag(Frag<float>& f, const char* t, int kbase, int col0, int lane) {
  const int col = col0 + (lane & 31);
  const int row = kbase + 8 * (lane >> 5);
#pragma unroll
  for (int s = 0; s < 8; ++s) f.v[s] = *reinterpret_cast<const float*>(t + swz<ROW, NCH>(row + s, col * 4));
}

__device__ __forceinline__ void zero_unless(Frag<bf16_t>& f, bool keep) {
  const bf16x8_t z = {0, 0, 0, 0, 0, 0, 0, 0};
  f.v = keep ? f.v : z;
}
__device__ __forceinline__ void zero_unless(Frag<float>& f, bool keep) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = keep ? f.v[i] : 0.f;
}

// Padding that makes a row stride equal 64 (mod 256) bytes: four consecutive rows then fall
// on disjoint LDS banks for the 16-lane groups of the transposed reads.
constexpr int pad_64mod256(int bytes) { return ((64 - bytes % 256) % 256 + 256) % 256; }

// SINGLE: whole H handled by one workgroup, NB = H-columns per wave / 32 (= K quarter / 32).
// CHUNKED: output columns split into nchunks chunks of 4*NB*32; S streamed from L2.
template <typename T, bool DW, bool SINGLE, int NB>
__global__ void __launch_bounds__(kBwdThreads, 1) bwd_kernel(BwdArgs<T> p) {
  constexpr int ES = sizeof(T);
  constexpr int NCOL = NB * 32;
  constexpr int XT_ROW = NCOL * ES + pad_64mod256(NCOL * ES);  // bytes per row of a wave's X tile
  constexpr int G_ROW = kBS * ES + pad_64mod256(kBS * ES);      // bytes per row of the dlogits tile
  constexpr int XT_NCH = NCOL * ES / 16;
  constexpr int G_NCH = kBS * ES / 16;
  constexpr int ZCOL = kBS + 4;                                   // floats per column of a partial z
  constexpr int KS1S = 2 * NB;                                    // GEMM1 k-steps per wave (SINGLE)
  constexpr int XCH = NCOL * ES / 16;                             // 16 B chunks per row (CHUNKED)
  constexpr int XCH_LANE = kBX * XCH / kWave;
  // Layouts: partial z is column-major [x][s]; the dlogits tile is [x][s] (the K index of
  // GEMM3 runs along x, read back with transposed LDS reads); each wave's X tile is
  // row-major [x][its NCOL columns].
  __shared__ __attribute__((aligned(16))) float zpart[4][kBX * ZCOL];
  __shared__ __attribute__((aligned(16))) char gtile[kBX * G_ROW];
  __shared__ __attribute__((aligned(16))) char xtile[4][kBX * XT_ROW];
  __shared__ __attribute__((aligned(16))) float s_a[kBS];
  __shared__ __attribute__((aligned(16))) float s_b[kBS];
  __shared__ __attribute__((aligned(16))) int32_t s_y[kBS];
  // gradient filtering (p.filter_eps > 0): wave w's share of each 16-column half of the
  // dlogits tile is negligible
  __shared__ int s_small[4][2];

  const int tid = threadIdx.x, w = wave_id(), lane = tid % kWave;
  const int64_t s_tile = blockIdx.x / p.nchunks;
  const int64_t chunk = blockIdx.x % p.nchunks;
  const int64_t s0 = s_tile * kBS;
  const int64_t h0 = chunk * (4 * NCOL);  // first output column of this workgroup
  const int64_t hw0 = h0 + w * NCOL;      // first output column of this wave
  const int64_t H = p.H;
  const int64_t KW = SINGLE ? (int64_t)NCOL : ((H + 63) / 64) * 16;  // GEMM1 K range per wave
  const int64_t kw0 = w * KW;
  const int ks1 = (int)(KW / 16);
  const int khalf = 8 * (lane >> 5);

  const long long nvalid = *p.n_valid;
  const float cscale = p.mean ? 1.f / (float)(nvalid > 1 ? nvalid : 1) : 1.f;

  // Per stationary-row tables.
  //   grad_input: s_a = LSE, s_b = 1 + 2 mu LSE, s_y = target (or -1 if the token row does not count)
  //   grad_W:     s_a = bias of the vocab row, s_y = 1 if the vocab row exists
  if (tid < kBS) {
    const int64_t r = s0 + tid;
    if (!DW) {
      float L = 0.f;
      int32_t yv = -1;
      if (r < p.BT) {
        const int64_t yt = p.y[r];
        if (yt != p.ignore_index && yt >= 0 && yt < p.V) {
          yv = (int32_t)yt;
          L = p.lse[r];
        }
      }
      s_a[tid] = L;
      s_b[tid] = 1.f + 2.f * p.mu * L;
      s_y[tid] = yv;
    } else {
      s_a[tid] = (p.bias != nullptr && r < p.V) ? Elem<T>::to_f(p.bias[r]) : 0.f;
      s_b[tid] = 0.f;
      s_y[tid] = r < p.V ? 1 : 0;
    }
  }

  // Stationary fragments (SINGLE): S rows s0 + sb*32 + lane%32, this wave's K quarter.
  // Buffer descriptors: S rebased at the workgroup's first row, X rebased per tile, so rows
  // past the end read as zero.  K past H (the last wave's quarter when H is not a multiple of
  // 4 x 32 x NB) reads the next row's data, which meets a zeroed S fragment.
  const int64_t row_bytes = H * ES;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.S + s0 * H, (p.nS - s0) * row_bytes);
  const uint32_t off_lane = (uint32_t)((lane & 31) * row_bytes + (kw0 + khalf) * ES);
  Frag<T> sf[SINGLE ? KS1S : 1][2];
  if constexpr (SINGLE) {
#pragma unroll
    for (int ks = 0; ks < KS1S; ++ks)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        load8(sf[ks][sb], rs, off_lane + (uint32_t)(sb * 32 * row_bytes + ks * 16 * ES));
        zero_unless(sf[ks][sb], kw0 + ks * 16 + khalf < H);
      }
  }

  f32x16_t acc[2][NB];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[sb][cb][r] = 0.f;
  float gb[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) gb[e] = 0.f;

  // Per streamed-column quantities of the next tile (prefetched with its X rows):
  //   grad_input: bias of the vocab column;  grad_W: LSE and target (or -1) of the token column.
  float pc_a = 0.f;
  int32_t pc_y = -1;
  auto load_col = [&](int64_t x0n) {
    const int64_t xc = x0n + (lane & 31);
    if (!DW) {
      pc_a = p.bias != nullptr ? Elem<T>::to_f(p.bias[xc < p.V ? xc : p.V - 1]) : 0.f;
      pc_y = 0;
    } else {
      const int64_t t = xc < p.BT ? xc : p.BT - 1;
      const int64_t yt = p.y[t];
      pc_a = p.lse[t];
      pc_y = (xc < p.BT && yt != p.ignore_index && yt >= 0 && yt < p.V) ? (int32_t)yt : -1;
    }
  };

  // X fragments of GEMM1: the first PF k-steps of the next tile are prefetched during the
  // current tile; the remaining ones are issued when the tile starts (register budget).
  constexpr int PF = (SINGLE && KS1S > 8) ? KS1S - 4 : KS1S;
  Frag<T> xf[SINGLE ? KS1S : 1];
  auto x_rsrc = [&](int64_t x0n) { return make_rsrc(p.X + x0n * H, (p.nX - x0n) * row_bytes); };
  auto load_x = [&](int64_t x0n, int from, int to) {
    const __amdgpu_buffer_rsrc_t rx = x_rsrc(x0n);
#pragma unroll
    for (int ks = 0; ks < (SINGLE ? KS1S : 1); ++ks)
      if (ks >= from && ks < to) load8(xf[ks], rx, off_lane + (uint32_t)(ks * 16 * ES));
  };

  char* xt = xtile[w];
  const int c = lane & 31;                // reduce step: streamed column of this lane
  const int r0 = 16 * w + 8 * (lane >> 5);  // reduce step: first of this lane's 8 stationary rows
  const int64_t ntiles = (p.nX + kBX - 1) / kBX;
  const bool filt = p.filter_eps > 0.f;
  float gpend[8];  // (filtering) grad_b terms of this tile, added once the tile is kept
  unsigned long long n_skipped = 0;
  if (ntiles > 0) {
    if constexpr (SINGLE) load_x(0, 0, PF);
    load_col(0);
  }
  for (int64_t xtl = 0; xtl < ntiles; ++xtl) {
    const int64_t x0 = xtl * kBX;
    const float col_a = pc_a;
    const int32_t col_y = pc_y;
    // ---------------- GEMM1: partial z[64 x 32] over this wave's K quarter
    f32x16_t zp[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) zp[sb][r] = 0.f;
    if constexpr (SINGLE) {
      if constexpr (PF < KS1S) load_x(x0, PF, KS1S);
#pragma unroll
      for (int ks = 0; ks < KS1S; ++ks) {
        // the same X values are GEMM3's operand for this wave's output columns
        store_frag<XT_ROW, XT_NCH>(xt, lane & 31, (ks * 16 + khalf) * ES, xf[ks]);
        mfma_32x32x16(sf[ks][0], xf[ks], zp[0]);
        mfma_32x32x16(sf[ks][1], xf[ks], zp[1]);
      }
      if (xtl + 1 < ntiles) {  // prefetch the next tile into the registers just consumed
        load_x(x0 + kBX, 0, PF);
        load_col(x0 + kBX);
      }
    } else {
      // X rows for this wave's output columns: issued first, stored to LDS after GEMM1
      const __amdgpu_buffer_rsrc_t rx = x_rsrc(x0);
      uint4 xg[XCH_LANE];
#pragma unroll
      for (int i = 0; i < XCH_LANE; ++i) {
        const int cidx = lane + kWave * i, r = cidx / XCH, cc = cidx % XCH;
        const int64_t col = hw0 + cc * (16 / ES);
        // columns past H read the next row (or zero past the end): they only feed
        // output columns >= H, which are never stored
        xg[i] = load16(rx, (uint32_t)(r * row_bytes + col * ES));
      }
      // GEMM1 with a 4-deep register pipeline over the K steps
      constexpr int P = 4;
      Frag<T> rxf[P], ra[P], rb[P];
      auto ld = [&](int j, int ks) {
        const uint32_t o = off_lane + (uint32_t)(ks * 16 * ES);
        load8(rxf[j], rx, o);
        load8(ra[j], rs, o);
        load8(rb[j], rs, o + (uint32_t)(32 * row_bytes));
        const bool kin = kw0 + ks * 16 + khalf < H;
        zero_unless(ra[j], kin);
        zero_unless(rb[j], kin);
      };
#pragma unroll
      for (int j = 0; j < P; ++j) ld(j, j);
      for (int ks = 0; ks < ks1; ks += P) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
          if (ks + j < ks1) {
            mfma_32x32x16(ra[j], rxf[j], zp[0]);
            mfma_32x32x16(rb[j], rxf[j], zp[1]);
          }
          ld(j, ks + j + P);
        }
      }
#pragma unroll
      for (int i = 0; i < XCH_LANE; ++i) {
        const int cidx = lane + kWave * i, r = cidx / XCH, cc = cidx % XCH;
        *reinterpret_cast<uint4*>(xt + swz<XT_ROW, XT_NCH>(r, cc * 16)) = xg[i];
      }
      if (xtl + 1 < ntiles) load_col(x0 + kBX);
    }
    // ---------------- partial z to LDS, column-major, 16-byte stores
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = sb * 32 + 8 * j + 4 * (lane >> 5);
        *reinterpret_cast<float4*>(&zpart[w][(lane & 31) * ZCOL + row]) =
            make_float4(zp[sb][4 * j], zp[sb][4 * j + 1], zp[sb][4 * j + 2], zp[sb][4 * j + 3]);
      }
    __syncthreads();
    // ---------------- z and dlogits for column c, rows r0 .. r0+7, in two halves of 4 rows
    // (bounds the live registers of this step)
    const int64_t xc = x0 + c;
    bool small_lane = true;
#pragma unroll 1
    for (int hf = 0; hf < 2; ++hf) {
      const int rh = r0 + 4 * hf;
      float z[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 a = *reinterpret_cast<const float4*>(&zpart[q][c * ZCOL + rh]);
        z[0] += a.x; z[1] += a.y; z[2] += a.z; z[3] += a.w;
      }
      const float4 ta = *reinterpret_cast<const float4*>(&s_a[rh]);
      const int4 ty = *reinterpret_cast<const int4*>(&s_y[rh]);
      const float va[4] = {ta.x, ta.y, ta.z, ta.w};
      const int32_t vy[4] = {ty.x, ty.y, ty.z, ty.w};
      float g[4];
      if (!DW) {
        const float4 tb = *reinterpret_cast<const float4*>(&s_b[rh]);
        const float vf[4] = {tb.x, tb.y, tb.z, tb.w};
        const bool colok = xc < p.V;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float ex = __expf(z[e] + col_a - va[e]) * vf[e] - ((int64_t)vy[e] == xc ? 1.f : 0.f);
          g[e] = (vy[e] >= 0 && colok) ? ex : 0.f;
        }
      } else {
        const float ft = 1.f + 2.f * p.mu * col_a;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t srow = s0 + rh + e;
          const float ex = __expf(z[e] + va[e] - col_a) * ft - ((int64_t)col_y == srow ? 1.f : 0.f);
          g[e] = (vy[e] != 0 && col_y >= 0) ? ex : 0.f;
        }
        if (hf == 0) {
#pragma unroll
          for (int e = 0; e < 4; ++e) gpend[e] = g[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) gpend[4 + e] = g[e];
        }
      }
      if (filt) {
        bool sm = true;
#pragma unroll
        for (int e = 0; e < 4; ++e) sm = sm && fabsf(g[e]) < p.filter_eps;
        small_lane = hf == 0 ? sm : (small_lane && sm);
      }
      store4(gtile + swz<G_ROW, G_NCH>(c, rh * ES), g, T());
    }
    if (filt) {
      // columns 0..15 of the tile are lanes 0-15 and 32-47, columns 16..31 the others
      const unsigned long long big = __builtin_amdgcn_ballot_w64(!small_lane);
      if (lane == 0) {
        s_small[w][0] = (big & 0x0000ffff0000ffffull) == 0 ? 1 : 0;
        s_small[w][1] = (big & 0xffff0000ffff0000ull) == 0 ? 1 : 0;
      }
    }
    __syncthreads();
    // (filtering) a 64 x 16 half of the tile whose dlogits are all negligible adds nothing
    bool skip_half[2] = {false, false};
    if (filt) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        skip_half[hh] = (s_small[0][hh] & s_small[1][hh] & s_small[2][hh] & s_small[3][hh]) != 0;
        if (skip_half[hh] && x0 + 16 * hh < p.nX) ++n_skipped;  // (halves past nX are not tiles)
      }
    }
    if (DW) {
      const bool keep = !skip_half[c >> 4];
#pragma unroll
      for (int e = 0; e < 8; ++e) gb[e] += keep ? gpend[e] : 0.f;
    }
    // ---------------- GEMM3: acc += g . X[:, wave columns]
#pragma unroll
    for (int kk = 0; kk < kBX / 16; ++kk) {
      if (skip_half[kk]) continue;
      Frag<T> ga[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) tile_frag<G_ROW, G_NCH>(ga[sb], gtile, kk * 16, sb * 32, lane);
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        Frag<T> xb;
        tile_frag<XT_ROW, XT_NCH>(xb, xt, kk * 16, cb * 32, lane);
        mfma_32x32x16(ga[0], xb, acc[0][cb]);
        mfma_32x32x16(ga[1], xb, acc[1][cb]);
      }
    }
  }

  // ---------------- write c * acc
  if (p.out != nullptr) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int64_t col = hw0 + cb * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = s0 + sb * 32 + acc_row(lane, r);
          if (row < p.nS && col < H) {
            const int64_t orow = p.out_row_map != nullptr ? p.out_row_map[row] : row;
            p.out[orow * H + col] = Elem<T>::from_f(cscale * acc[sb][cb][r]);
          }
        }
      }
  } else if (p.out_f32 != nullptr) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int64_t col = hw0 + cb * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = s0 + sb * 32 + acc_row(lane, r);
          if (row < p.nS && col < H) {
            const int64_t orow = p.out_row_map != nullptr ? p.out_row_map[row] : row;
            p.out_f32[orow * H + col] = cscale * acc[sb][cb][r];
          }
        }
      }
  }
  if (filt && p.filter_counts != nullptr && chunk == 0 && threadIdx.x == 0) {
    atomicAdd(&p.filter_counts[0], n_skipped);
    atomicAdd(&p.filter_counts[1], (unsigned long long)((p.nX + 15) / 16));
  }
  if (DW && p.grad_b != nullptr && chunk == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = gb[e];
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) v += __shfl_xor(v, off, kWave);
      const int64_t srow = s0 + r0 + e;
      if (c == 0 && srow < p.V)
        p.grad_b[p.out_row_map != nullptr ? p.out_row_map[srow] : srow] = Elem<T>::from_f(cscale * v);
    }
  }
}

// ---------------------------------------------------------------------------
// bf16, H <= 1024: software-pipelined variant.
//
// Streamed tiles are 16 rows.  Each wave owns NCOL = 32*NB columns of H (its GEMM1 K range
// and its GEMM3 output columns), so it only ever touches its own share of a streamed tile:
// it loads that share into LDS itself (buffer-to-LDS loads, four buffers per wave) and no
// barrier guards the tile buffers.  One loop iteration i overlaps two tiles:
//   phase A: first half of GEMM1 for tile i+1 (16x16x32 MFMA, partial z over the wave's K
//            range) beside the dlogits of tile i from the partial z sums of every wave;
//            barrier
//   phase B: second half of GEMM1 for tile i+1, GEMM3 for tile i (32x32x16 MFMA,
//            acc += g . X), the partial z of tile i+1 written out for the other waves;
//            barrier
// and tile i+4 is requested into the buffer tile i used (half in phase B, half in the next
// phase A), together with the tile's column values (per token (LSE, target), or the bias).
//
// Shared-memory layouts (all reads conflict-free; every address is a per-lane constant plus
// an immediate, so the loop does almost no address arithmetic):
//  * a wave's tile share is NB planes of 1 KB; plane j holds the 16-byte chunks 4j..4j+3 of
//    the 16 rows (columns 32j..32j+31 of the wave's range): chunk (n, 4j+u) sits at
//    1024 j + 64 n + 16 (u ^ tsw(n)).
//  * GEMM3 reads 16 of its K rows as four quads; quad k holds tile rows tq(k, 0..3).
//  * the dlogits tile g[n][m] (n = streamed row, m = stationary row) keeps row n in 128 B
//    with its four 32-byte groups (16 m values each) permuted by gsw2(n).
// ---------------------------------------------------------------------------
constexpr int kPS = 64;   // stationary rows per workgroup (16 per wave after the exchange)
constexpr int kPX = 16;   // streamed rows per tile
constexpr int kPBuf = 4;  // tile buffers per wave

typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int tsw(int n) { return ((n >> 1) + (n >> 3)) & 3; }
__device__ __forceinline__ int tq(int k, int r) { return ((k & 1) << 1) + ((k >> 1) << 3) + (r & 1) + ((r >> 1) << 2); }
__device__ __forceinline__ int gsw2(int n) { return (n & 1) | ((n >> 1) & 2); }

// 16x16x32 bf16 MFMA with a VGPR accumulator (see mfma_32x32x16_v).  Its operands here come
// from memory loads only (no VALU writes), so no wait states are needed in front of it.
__device__ __forceinline__ void mfma16_v0(const bf16x8_t& a, const bf16x8_t& b, f32x4v& c) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16_v(const bf16x8_t& a, const bf16x8_t& b, f32x4v& c) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ bf16x8_t lds_b128(const char* p) { return *reinterpret_cast<const bf16x8_t*>(p); }
__device__ __forceinline__ bf16x8_t tr_pair(const char* p0, const char* p1) {
  const i16x4_t a = lds_read_tr16(reinterpret_cast<const bf16_t*>(p0));
  const i16x4_t b = lds_read_tr16(reinterpret_cast<const bf16_t*>(p1));
  return bf16x8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Workgroup barrier that leaves this wave's newest N LDS reads in flight (__syncthreads
// waits for every outstanding LDS access).  A wave's LDS accesses complete in order, so with
// at most N accesses outstanding, everything issued before the compiler order point
// `lds_order()` that precedes those N reads has completed, and writes made before it are
// visible to the other waves after the barrier.  (Scalar loads share the counter; they can
// only make the wait longer.)  The reads are waited for where their registers are used.
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }
template <int N>
__device__ __forceinline__ void barrier_reads_in_flight() {
  asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// f(integral_constant<int, I>) for I = B .. E-1, in order.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Plane j of a tile share: 1 KB of LDS from this lane's 16 bytes at off + 64 j.
template <int J, int N>
struct DmaPlanes {
  static __device__ __forceinline__ void run(const u32x4_t& rx, uint32_t lds, uint32_t off) {
    dma16(rx, lds + 1024 * J, off + 64 * J);
    DmaPlanes<J + 1, N>::run(rx, lds, off);
  }
};
template <int N>
struct DmaPlanes<N, N> {
  static __device__ __forceinline__ void run(const u32x4_t&, uint32_t, uint32_t) {}
};

// FILT: gradient filtering ("Cut Cross Entropy visualized", "Gradient Filtering"): a tile
// (64 stationary rows x 16 streamed rows) whose dlogits of the summed loss are all below
// p.filter_eps in magnitude adds nothing to the gradient (its GEMM3 work and its grad_b
// share are skipped).
template <bool DW, int NB, bool FILT>
__global__ void __launch_bounds__(kBwdThreads, 1) bwd_pipe_kernel(BwdArgs<bf16_t> p) {
  constexpr int NCOL = 32 * NB;       // columns of H owned by a wave
  constexpr int XW = kPX * NCOL * 2;  // bytes of a wave's share of one tile (NB planes)
  constexpr int NQ = NB + 1;          // loads queued per tile: its planes and its column values
  __shared__ __attribute__((aligned(1024))) char xs[4][kPBuf][XW];
  __shared__ __attribute__((aligned(1024))) char zx[4][4][1024];  // [writer][row block]
  __shared__ __attribute__((aligned(256))) char gl[kPX * 128];
  // column values of each buffered tile, loaded with it: per token (LSE, target + 1) (DW)
  // or the fp32 bias of each vocabulary row
  __shared__ __attribute__((aligned(256))) char cs[4][kPBuf][256];
  __shared__ int s_small[4];  // (FILT) wave w's share of the current dlogits tile is negligible

  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63;
  const int l16 = lane & 15, q = lane >> 4;       // 16x16 operand coordinates
  const int tc = lane & 3, tr = (lane >> 2) & 3;  // transposed-read coordinates
  const int64_t s0 = (int64_t)blockIdx.x * kPS;
  const int64_t H = p.H, row_bytes = H * 2;
  const int kw0 = w * NCOL;
  const long long nvalid = *p.n_valid;
  const float cscale = p.mean ? 1.f / (float)(nvalid > 1 ? nvalid : 1) : 1.f;
  const int64_t ntiles = (p.nX + kPX - 1) / kPX;

  // ---- per-lane constants of the stationary rows m = 16 w + 4 q + i (after the exchange).
  // The dlogit of (row, column) is g = 2^(z log2 e + ra + ca) * f - onehot, where ra and ca
  // are the row's and the column's additive terms in base 2: -LSE log2 e for a token, the
  // bias times log2 e for a vocabulary entry, and -inf for a row or column that contributes
  // nothing (an ignored token, an entry past V), which makes the exponential exactly 0; f is
  // the token's z-loss factor 1 + 2 mu LSE.  The one-hot term can only match a counted pair.
  constexpr float kLog2e = 1.4426950408889634f;
  float ra[4], rf[4];
  int32_t ry[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = s0 + 16 * w + 4 * q + i;
    if (!DW) {  // token rows: target (-1: the row contributes nothing)
      int32_t yv = -1;
      float L = 0.f;
      if (r < p.BT) {
        const float2 tk = p.tok[r];
        yv = __float_as_int(tk.y) - 1;
        L = yv >= 0 ? tk.x : 0.f;
      }
      ra[i] = yv >= 0 ? -L * kLog2e : -INFINITY;
      rf[i] = 1.f + 2.f * p.mu * L;
      ry[i] = yv;
    } else {  // vocabulary rows (the index is rebuilt from vrow0 where it is needed)
      ra[i] = r < p.V ? (p.bias != nullptr ? bf2f(p.bias[r]) * kLog2e : 0.f) : -INFINITY;
      rf[i] = 0.f;
      ry[i] = 0;
    }
  }

  // vocabulary rows (DW): row 16 w + 4 q + i is vocabulary entry vrow0 + i
  const int32_t vrow0 = (int32_t)(s0 + 16 * w + 4 * q);

  // ---- stationary GEMM1 A fragments: rows 16 rb + l16, k = kw0 + 32 ks + 8 q .. + 7
  bf16x8_t sf[NB][4];
  {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.S + s0 * H, (p.nS - s0) * row_bytes);
#pragma unroll
    for (int ks = 0; ks < NB; ++ks)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        const int col = kw0 + 32 * ks + 8 * q;
        const uint32_t off = col < H ? (uint32_t)((16 * rb + l16) * row_bytes + col * 2) : 0x80000000u;
        sf[ks][rb] = __builtin_bit_cast(bf16x8_t, load16(rs, off));
      }
  }

  f32x16_t acc[2][NB];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[sb][cb][r] = 0.f;
  float gb[4] = {0.f, 0.f, 0.f, 0.f};
  float gpend[4] = {0.f, 0.f, 0.f, 0.f};
  unsigned long long n_skipped = 0;

  // ---- per-lane LDS offsets
  // DMA: instruction j of a tile fills plane j; lane l lands at slot l = (row n, chunk u).
  const int dn = lane >> 2, du = (lane & 3) ^ tsw(lane >> 2);
  const uint32_t dma_off =
      (kw0 + 8 * du < H) ? (uint32_t)(dn * row_bytes + (kw0 + 8 * du) * 2) : 0x80000000u;
  // GEMM1 B operand: tile row l16, chunk 4 ks + q  ->  plane ks, slot (l16, q)
  const int o_g1 = 64 * l16 + 16 * (q ^ tsw(l16));
  // GEMM3 B operand (transposed reads): quad 2 (q >> 1) + rd, row tq(.., tr), columns
  // 16 (q & 1) + 4 tc .. + 3 of the plane's 32
  int o_g3[2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int n = tq(2 * (q >> 1) + rd, tr);
    const int u = 2 * (q & 1) + (tc >> 1);
    o_g3[rd] = 64 * n + 16 * (u ^ tsw(n)) + 8 * (tc & 1);
  }
  // GEMM3 A operand (dlogits, transposed reads): m group 2 sb + (q & 1)
  int o_ga[2][2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int n = tq(2 * (q >> 1) + rd, tr);
      o_ga[sb][rd] = 128 * n + 32 * ((2 * sb + (q & 1)) ^ gsw2(n)) + 8 * tc;
    }
  // dlogits writes: column n = l16, rows m = 16 w + 4 q .. + 3
  const int o_gw = 128 * l16 + 32 * (w ^ gsw2(l16)) + 8 * q;

  char* const xw = xs[w][0];
  const uint32_t xw_lds = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)xw));
  const uint32_t cs_lds = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)cs[w][0]));
  // column values of a tile: 4 bytes per lane (DW: 16 tokens x 8 B; otherwise 16 x 4 B)
  const uint32_t col_off = lane < (DW ? 32 : 16) ? 4u * lane : 0x80000000u;
  auto col_rsrc = [&](int64_t tile) {
    const int64_t x0 = tile * kPX;
    return DW ? make_rsrc_words(p.tok + x0, (p.BT - x0) * 8)
              : make_rsrc_words(p.biasf + x0, p.biasf != nullptr ? (p.V - x0) * 4 : 0);
  };
  auto dma = [&](int64_t tile, int buf) {
    const int64_t x0 = tile * kPX;
    dma4(col_rsrc(tile), cs_lds + (uint32_t)(buf * 256), col_off);
    const u32x4_t rx = make_rsrc_words(p.X + x0 * H, (p.nX - x0) * row_bytes);
    DmaPlanes<0, NB>::run(rx, xw_lds + (uint32_t)(buf * XW), dma_off);
  };
  // column values of tile `tile` for column l16 (see the row constants above): DW: the
  // token x0 + l16's additive term, z-loss factor and target (-1: not counted); otherwise the
  // vocabulary row x0 + l16's term and index (-2 past V, so it matches no row's target)
  float nc_a = 0.f, nc_f = 0.f;
  int32_t nc_y = -1;
  auto take_col = [&](int64_t tile, int buf) {  // after the loads of `tile` have landed
    if (DW) {
      const float2 t = *reinterpret_cast<const float2*>(cs[w][buf] + 8 * l16);
      const float L = t.x;
      nc_y = __float_as_int(t.y) - 1;
      nc_a = nc_y >= 0 ? -L * kLog2e : -INFINITY;
      nc_f = nc_y >= 0 ? 1.f + 2.f * p.mu * L : 0.f;
    } else {
      const int64_t xc = tile * kPX + l16;
      const float b = *reinterpret_cast<const float*>(cs[w][buf] + 4 * l16);
      nc_a = xc < p.V ? b * kLog2e : -INFINITY;
      nc_y = xc < p.V ? (int32_t)xc : -2;
    }
  };

  // ---- GEMM1 of one tile: partial z[64 x 16] over this wave's K range, four 16-row blocks,
  // in two halves (the dlogits of the previous tile are computed between them)
  f32x4v zp[4];
  bf16x8_t xf1[NB];
  auto gemm1_reads = [&](int buf, auto k0c, auto k1c) {
    constexpr int K0 = decltype(k0c)::value, K1 = decltype(k1c)::value;
    const char* xb = xw + buf * XW + o_g1;
#pragma unroll
    for (int ks = K0; ks < K1; ++ks) xf1[ks] = lds_b128(xb + 1024 * ks);
  };
  auto gemm1_part = [&](auto k0c, auto k1c) {
    constexpr int K0 = decltype(k0c)::value, K1 = decltype(k1c)::value;
#pragma unroll
    for (int ks = K0; ks < K1; ++ks)
#pragma unroll
      for (int rb = 0; rb < 4; ++rb) {
        if (ks == 0) mfma16_v0(sf[ks][rb], xf1[ks], zp[rb]);
        else mfma16_v(sf[ks][rb], xf1[ks], zp[rb]);
      }
  };
  // partial z of the other waves' row blocks to LDS; the own block stays in registers
  f32x4v zown;
  auto put_partials = [&]() {
    // wait states after the last MFMA writing zp, before anything else reads it
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(zp[0]), "+v"(zp[1]), "+v"(zp[2]), "+v"(zp[3]));
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) {
      if (rb == w) {
        zown = zp[rb];
      } else {
        *reinterpret_cast<f32x4v*>(zx[w][rb] + 16 * lane) = zp[rb];
      }
    }
  };
  // the other waves' partial sums of this wave's row block (written before the last barrier)
  f32x4v zpr[3];
  auto partial_reads = [&]() {
#pragma unroll
    for (int x = 1; x < 4; ++x) zpr[x - 1] = *reinterpret_cast<const f32x4v*>(zx[w ^ x][w] + 16 * lane);
  };
  // dlogits of one tile for rows 16 w + 4 q + i, column l16 -> LDS (bf16), in eight steps
  // that the first half of the next tile's GEMM1 interleaves with its MFMAs (one step after
  // each of eight MFMAs).  Each step starts by passing the values it reads through an empty
  // asm statement: the compiler cannot move the step's arithmetic above the MFMA before it,
  // and its results are consumed after the next MFMA, so it executes while the MFMAs run.
  float dz[4], dt[4], de[4];
  auto dl_step = [&](auto kc) {
    constexpr int K = decltype(kc)::value;
    if constexpr (K == 0) {  // the partial sums have landed by now
      asm volatile("" : "+v"(zpr[0]), "+v"(zpr[1]), "+v"(zpr[2]), "+v"(zown));
#pragma unroll
      for (int i = 0; i < 4; ++i) dz[i] = zown[i] + zpr[0][i];
    } else if constexpr (K == 1 || K == 2) {
      asm volatile("" : "+v"(dz[0]), "+v"(dz[1]), "+v"(dz[2]), "+v"(dz[3]));
#pragma unroll
      for (int i = 0; i < 4; ++i) dz[i] += zpr[K][i];
    } else if constexpr (K == 3) {
      asm volatile("" : "+v"(dz[0]), "+v"(dz[1]), "+v"(dz[2]), "+v"(dz[3]));
#pragma unroll
      for (int i = 0; i < 4; ++i) dt[i] = fmaf(dz[i], kLog2e, ra[i] + nc_a);
    } else if constexpr (K == 4) {
      asm volatile("" : "+v"(dt[0]), "+v"(dt[1]), "+v"(dt[2]), "+v"(dt[3]));
      de[0] = __builtin_amdgcn_exp2f(dt[0]);
      de[1] = __builtin_amdgcn_exp2f(dt[1]);
    } else if constexpr (K == 5) {
      asm volatile("" : "+v"(dt[2]), "+v"(dt[3]), "+v"(de[0]), "+v"(de[1]));
      de[2] = __builtin_amdgcn_exp2f(dt[2]);
      de[3] = __builtin_amdgcn_exp2f(dt[3]);
    } else if constexpr (K == 6) {
      asm volatile("" : "+v"(de[0]), "+v"(de[1]), "+v"(de[2]), "+v"(de[3]));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!DW) dz[i] = fmaf(de[i], rf[i], ry[i] == nc_y ? -1.f : 0.f);
        else dz[i] = fmaf(de[i], nc_f, nc_y == vrow0 + i ? -1.f : 0.f);
      }
    } else {
      asm volatile("" : "+v"(dz[0]), "+v"(dz[1]), "+v"(dz[2]), "+v"(dz[3]));
      const float* g = dz;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (DW) {
          if (FILT) gpend[i] = g[i];  // added to grad_b once the tile is known to be kept
          else gb[i] += g[i];
        }
      }
      *reinterpret_cast<uint2*>(gl + o_gw) = make_uint2(pack_bf2(g[0], g[1]), pack_bf2(g[2], g[3]));
      if (FILT) {
        const float e = p.filter_eps;
        const bool small = fabsf(g[0]) < e && fabsf(g[1]) < e && fabsf(g[2]) < e && fabsf(g[3]) < e;
        const bool all_small = __builtin_amdgcn_ballot_w64(!small) == 0;
        if (lane == 0) s_small[w] = all_small ? 1 : 0;
      }
    }
  };
  // first half of GEMM1 (the MFMAs of gemm1_part(C0, CH)) with the eight dlogits steps after
  // MFMAs NM-10 .. NM-3 (the earlier ones cover the latency of the partial-sum reads); with
  // fewer MFMAs the remaining steps follow them
  auto gemm1a_dlogits = [&]() {
    constexpr int NM = 4 * (NB / 2);
    constexpr int P0 = NM > 10 ? NM - 10 : 0;
    static_for<0, NM>([&](auto nc) {
      constexpr int n = decltype(nc)::value;
      constexpr int ks = n / 4, rb = n % 4;
      if constexpr (ks == 0) mfma16_v0(sf[ks][rb], xf1[ks], zp[rb]);
      else mfma16_v(sf[ks][rb], xf1[ks], zp[rb]);
      if constexpr (n >= P0 && n - P0 < 8) dl_step(std::integral_constant<int, n - P0>{});
    });
    static_for<(NM - P0 < 8 ? NM - P0 : 8), 8>([&](auto kc) { dl_step(kc); });
  };  // (FILT) after the barrier that follows dlogits: is the whole tile negligible?
  auto tile_skipped = [&]() { return FILT && (s_small[0] & s_small[1] & s_small[2] & s_small[3]) != 0; };
  // GEMM3 of one tile: acc[64 x NCOL] += g[64 x 16] . X[16 x NCOL]; with `refill`, planes
  // 0 .. NB/2-1 of the buffer are reloaded (tile `next`) as soon as their last read has
  // completed; the other half is queued during the next phase A (refill_rest), so that the
  // loads of the four waves spread over both phases.
  u32x4_t rx_next;
  uint32_t lds_next = 0;
  // `mid` runs after GEMM3's operand reads are issued and before its MFMAs.
  auto gemm3 = [&](int buf, bool refill, int64_t next, auto&& mid) {
    const char* xb = xw + buf * XW;
    const int64_t x0 = next * kPX;
    rx_next = make_rsrc_words(p.X + x0 * H, (p.nX - x0) * row_bytes);
    lds_next = xw_lds + (uint32_t)(buf * XW);
    if (refill) dma4(col_rsrc(next), cs_lds + (uint32_t)(buf * 256), col_off);
    if (FILT) {
      if (tile_skipped()) {  // no MFMA work; the buffer refill still happens (nothing reads it)
        ++n_skipped;
        mid();
        if (refill) {
#pragma unroll
          for (int cb = 0; cb < NB / 2; ++cb) dma16(rx_next, lds_next + 1024 * cb, dma_off + 64 * cb);
        }
        return;
      }
      if (DW) {
#pragma unroll
        for (int i = 0; i < 4; ++i) gb[i] += gpend[i];
      }
    }
    // Every operand read is issued before the first refill: a refill is an asm statement with
    // a memory clobber, so no LDS read can be moved across it, and reads issued after it would
    // leave the MFMAs waiting for each read's latency.
    Frag<bf16_t> ga[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) ga[sb].v = tr_pair(gl + o_ga[sb][0], gl + o_ga[sb][1]);
    Frag<bf16_t> xf[NB];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) xf[cb].v = tr_pair(xb + 1024 * cb + o_g3[0], xb + 1024 * cb + o_g3[1]);
    mid();
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      mfma_32x32x16(ga[0], xf[cb], acc[0][cb]);
      mfma_32x32x16(ga[1], xf[cb], acc[1][cb]);
      if (refill && cb < NB / 2) dma16_after(rx_next, lds_next + 1024 * cb, dma_off + 64 * cb, xf[cb].v);
    }
  };
  // (the reads of these planes completed in the previous phase: GEMM3 waited for them)
  auto refill_rest = [&]() {
#pragma unroll
    for (int cb = NB / 2; cb < NB; ++cb) dma16(rx_next, lds_next + 1024 * cb, dma_off + 64 * cb);
  };
  typedef std::integral_constant<int, 0> C0;
  typedef std::integral_constant<int, NB / 2> CH;
  typedef std::integral_constant<int, NB> CN;

  if (ntiles > 0) {
    // prologue: tiles 0 and 1, the column values of tile 0, tile 2 (short sweeps repeat the
    // last tile into buffers that are never read, so the queue always has the same shape)
    const int64_t last = ntiles - 1;
#pragma unroll
    for (int b = 0; b < kPBuf; ++b) dma(b < last ? b : last, b);
    vm_wait<(kPBuf - 1) * NQ>();  // tile 0 has landed
    gemm1_reads(0, C0{}, CN{});
    gemm1_part(C0{}, CN{});
    put_partials();
    vm_wait<(kPBuf - 2) * NQ>();  // tile 1 has landed
    lds_order();
    gemm1_reads(1 % kPBuf, C0{}, CH{});  // first half of GEMM1(1), in flight across the barrier
    barrier_reads_in_flight<NB / 2>();
  }
  // Loads of a wave, in issue order: phase B of iteration i queues the column values and
  // the first half of tile i+4, phase A of iteration i+1 its second half.  At the top of
  // iteration i, the newest loads are those of B(i-1), A(i-1) and B(i-2) (tiles i+3 and
  // i+2): everything older, so all of tile i+1, must have landed.
  for (int64_t i = 0; i < ntiles; ++i) {
    const int bi = (int)(i % kPBuf), bn = (int)((i + 1) % kPBuf);
    const bool more = i + 1 < ntiles;
    // GEMM1 of tile i+1 is split over both phases, so that each phase has MFMA work that does
    // not wait for its barrier: the first half covers the latency of the partial-sum reads
    // and runs beside the dlogits of tile i, the second half covers the dlogits reads of
    // GEMM3.  (In the last iteration it works on a stale buffer and its result is unused.)
    // ---- phase A (the first half of GEMM1(i+1)'s operands was read before the barrier)
    partial_reads();
    take_col(i, bi);
    gemm1a_dlogits();
    lds_order();
    gemm1_reads(bn, CH{}, CN{});  // in flight across the barrier
    if (i > 0) refill_rest();     // second half of tile i+3 (the buffer of tile i-1)
    barrier_reads_in_flight<NB - NB / 2>();
    // ---- phase B: GEMM3 of tile i (refilling its buffer with tile i+4 plane by plane; past
    // the end the last tile is repeated, never read), partial z of tile i+1
    // (the partial z of tile i+1 are written out between GEMM3's reads and its MFMAs, so the
    // writes complete while the MFMAs run)
    gemm1_part(CH{}, CN{});
    gemm3(bi, more, i + kPBuf < ntiles ? i + kPBuf : ntiles - 1, [&]() {
      if (more) put_partials();
    });
    // The next phase A starts on GEMM1(i+2) at once: its first operand half is read here,
    // in flight across the barrier, once tile i+2 has landed.  The newest loads are then
    // those of B(i), A(i) and B(i-1) (tiles i+4 and i+3); everything older, so all of tile
    // i+2, must have landed.  (In the last two iterations the reads hit a buffer whose
    // contents are never used.)
    vm_wait<NQ + NB / 2 + 1>();
    lds_order();
    gemm1_reads((int)((i + 2) % kPBuf), C0{}, CH{});
    barrier_reads_in_flight<NB / 2>();
  }
  vm_wait<0>();  // no load into LDS may still be in flight when the workgroup ends
  if (FILT && p.filter_counts != nullptr && tid == 0) {
    atomicAdd(&p.filter_counts[0], n_skipped);
    atomicAdd(&p.filter_counts[1], (unsigned long long)ntiles);
  }

  // ---- write c * acc
  if (p.out != nullptr) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int64_t col = kw0 + cb * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = s0 + sb * 32 + acc_row(lane, r);
          if (row < p.nS && col < H) {
            const int64_t orow = p.out_row_map != nullptr ? p.out_row_map[row] : row;
            p.out[orow * H + col] = f2bf(cscale * acc[sb][cb][r]);
          }
        }
      }
  } else if (p.out_f32 != nullptr) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const int64_t col = kw0 + cb * 32 + (lane & 31);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = s0 + sb * 32 + acc_row(lane, r);
          if (row < p.nS && col < H) {
            const int64_t orow = p.out_row_map != nullptr ? p.out_row_map[row] : row;
            p.out_f32[orow * H + col] = cscale * acc[sb][cb][r];
          }
        }
      }
  }
  if (DW && p.grad_b != nullptr) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = gb[i];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) v += __shfl_xor(v, off, kWave);
      const int64_t r = s0 + 16 * w + 4 * q + i;
      if (l16 == 0 && r < p.V) p.grad_b[p.out_row_map != nullptr ? p.out_row_map[r] : r] = f2bf(cscale * v);
    }
  }
}

template <bool DW, bool FILT>
static hipError_t launch_bwd_pipe_f(int nb, const BwdArgs<bf16_t>& a, dim3 grid, hipStream_t st) {
  switch (nb) {
    case 1: hipLaunchKernelGGL((bwd_pipe_kernel<DW, 1, FILT>), grid, dim3(kBwdThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL((bwd_pipe_kernel<DW, 2, FILT>), grid, dim3(kBwdThreads), 0, st, a); break;
    case 4: hipLaunchKernelGGL((bwd_pipe_kernel<DW, 4, FILT>), grid, dim3(kBwdThreads), 0, st, a); break;
    case 8: hipLaunchKernelGGL((bwd_pipe_kernel<DW, 8, FILT>), grid, dim3(kBwdThreads), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
template <bool DW>
static hipError_t launch_bwd_pipe(int nb, const BwdArgs<bf16_t>& a, dim3 grid, hipStream_t st) {
  return a.filter_eps > 0.f ? launch_bwd_pipe_f<DW, true>(nb, a, grid, st)
                            : launch_bwd_pipe_f<DW, false>(nb, a, grid, st);
}

template <typename T, bool DW, bool SINGLE, int N>
static hipError_t launch_bwd_one(const BwdArgs<T>& a, dim3 grid, hipStream_t st) {
  if constexpr (sizeof(T) == 4 && N > 4) {
    return hipErrorInvalidValue;  // fp32 column blocks are capped at 4 (LDS size)
  } else {
    hipLaunchKernelGGL((bwd_kernel<T, DW, SINGLE, N>), grid, dim3(kBwdThreads), 0, st, a);
    return hipGetLastError();
  }
}

template <typename T, bool DW, bool SINGLE>
static hipError_t launch_bwd_nb(int nb, const BwdArgs<T>& a, dim3 grid, hipStream_t st) {
  switch (nb) {
    case 1: return launch_bwd_one<T, DW, SINGLE, 1>(a, grid, st);
    case 2: return launch_bwd_one<T, DW, SINGLE, 2>(a, grid, st);
    case 3: return launch_bwd_one<T, DW, SINGLE, 3>(a, grid, st);
    case 4: return launch_bwd_one<T, DW, SINGLE, 4>(a, grid, st);
    case 5: return launch_bwd_one<T, DW, SINGLE, 5>(a, grid, st);
    case 6: return launch_bwd_one<T, DW, SINGLE, 6>(a, grid, st);
    case 7: return launch_bwd_one<T, DW, SINGLE, 7>(a, grid, st);
    case 8: return launch_bwd_one<T, DW, SINGLE, 8>(a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

// Column split: H <= 1024 (bf16) or H <= 512 (fp32) is one chunk with the stationary
// fragments in registers; otherwise ceil(H / 1024) (bf16) or ceil(H / 512) (fp32, LDS
// bound) chunks of 4 * NB * 32 columns.
struct BwdPlan {
  bool single;
  int nb;
  int64_t nchunks;
};
static BwdPlan bwd_plan(int64_t H, bool bf16) {
  BwdPlan pl;
  const int64_t single_max = bf16 ? 1024 : 512;
  if (H <= single_max) {
    pl.single = true;
    pl.nb = (int)((H + 127) / 128);
    pl.nchunks = 1;
  } else {
    pl.single = false;
    const int64_t cmax = bf16 ? 1024 : 512;
    pl.nchunks = (H + cmax - 1) / cmax;
    const int64_t per = (H + pl.nchunks - 1) / pl.nchunks;
    pl.nb = (int)((per + 127) / 128);
  }
  return pl;
}

template <typename T>
static hipError_t launch_bwd(const FusedArgs& fa, const FusedWs& w, bool dw, hipStream_t st) {
  BwdArgs<T> a;
  a.bias = static_cast<const T*>(fa.bias);
  a.y = fa.targets;
  a.lse = w.lse;
  a.tok = w.tok;
  a.filter_eps = fa.filter_eps;
  a.filter_counts = fa.filter_counts == nullptr
                        ? nullptr
                        : reinterpret_cast<unsigned long long*>(fa.filter_counts + (dw ? 2 : 0));
  a.biasf = fa.bias != nullptr ? w.biasf : nullptr;
  a.H = fa.H;
  a.BT = fa.BT;
  a.V = fa.V;
  a.ignore_index = fa.ignore_index;
  a.mu = fa.mu;
  a.n_valid = w.n_valid;
  a.mean = fa.mean ? 1 : 0;
  if (!dw) {
    a.S = static_cast<const T*>(fa.hidden);
    a.X = static_cast<const T*>(fa.W);
    a.nS = fa.BT;
    a.nX = fa.V;
    a.out = static_cast<T*>(fa.grad_input);
    a.out_f32 = nullptr;
    a.out_row_map = nullptr;
    a.grad_b = nullptr;
  } else {
    a.S = static_cast<const T*>(fa.W);
    a.X = static_cast<const T*>(fa.hidden);
    a.nS = fa.V;
    a.nX = fa.BT;
    a.out = fa.grad_w_f32 ? nullptr : static_cast<T*>(fa.grad_W);
    a.out_f32 = fa.grad_w_f32 ? static_cast<float*>(fa.grad_W) : nullptr;
    a.out_row_map = fa.out_row_map;
    a.grad_b = static_cast<T*>(fa.grad_b);
  }
  const BwdPlan pl = bwd_plan(fa.H, sizeof(T) == 2);
  a.nchunks = pl.nchunks;
  const int64_t ntile = (a.nS + kBS - 1) / kBS;
  if (ntile == 0) return hipSuccess;
  dim3 grid((unsigned)(ntile * pl.nchunks));
  if constexpr (sizeof(T) == 2) {
    if (pl.single) {
      // whole H per workgroup: the DMA kernel, with the column blocks rounded up to a power of two
      const int nb2 = pl.nb <= 1 ? 1 : (pl.nb <= 2 ? 2 : (pl.nb <= 4 ? 4 : 8));
      return dw ? launch_bwd_pipe<true>(nb2, a, grid, st) : launch_bwd_pipe<false>(nb2, a, grid, st);
    }
  }
  if (!dw) {
    return pl.single ? launch_bwd_nb<T, false, true>(pl.nb, a, grid, st)
                     : launch_bwd_nb<T, false, false>(pl.nb, a, grid, st);
  }
  return pl.single ? launch_bwd_nb<T, true, true>(pl.nb, a, grid, st)
                   : launch_bwd_nb<T, true, false>(pl.nb, a, grid, st);
}

// ---------------------------------------------------------------------------
// Gradient GEMMs on stored dlogits (the token-chunked composition of "Fused Linear
// Cross-Entropy: The Math, the Memory Wall, and Two Ways Around It", Strategy 1: a chunk of
// tokens has its logits written to HBM, turned into dlogits in place by the standalone
// cross-entropy kernel, and then consumed by the two gradient products).
//
// This is the GEMM3 half of the pipelined kernel above with the g tile read from HBM instead
// of recomputed: a workgroup owns 64 stationary rows and an output column range of 4 * NCOL
// columns (any H, in column chunks), streams 16-row tiles of X, and accumulates
// acc[64 x NCOL] += g[64 x 16] . X[16 x NCOL] per wave.  Loads go to LDS by buffer-to-LDS
// DMA: each wave loads its own NB planes of the X tile (as in the pipelined kernel) and a
// quarter of the 2 KiB g tile; one barrier per tile makes the g quarters visible to all.
//   grad_input (DW = false): stationary = the chunk's tokens, X = W rows (the vocabulary,
//     optionally split into ranges whose fp32 partial sums are added by mat_reduce_kernel);
//     the g tile is G[64 tokens][16 vocab], kept as rows of 32 bytes per token.
//   grad_W (DW = true): stationary = vocabulary rows, X = the chunk's hidden rows; the g tile
//     is G[16 tokens][64 vocab], kept in the pipelined kernel's layout; the fp32 sum over
//     chunks lives in `acc` (or in an fp32 output) and the last chunk writes c * sum; grad_b
//     is the column sum of G, accumulated the same way.
// ---------------------------------------------------------------------------
// FILT: gradient filtering of the g tiles (a separate instantiation: the skip branch around
// the MFMAs makes the compiler copy the accumulators, which the unfiltered kernel must not pay).
template <bool DW, int NB, bool FILT>
__global__ void __launch_bounds__(kBwdThreads, 1) mat_gemm_kernel(MatArgs p) {
  constexpr int NCOL = 32 * NB;
  constexpr int XW = kPX * NCOL * 2;
  constexpr int NQ = NB + 1;            // loads per tile and wave: NB planes + a g quarter
  constexpr int kGBuf = kPBuf + 1;      // a g slot is refilled one iteration after its last read
  constexpr int GT = kPX * 128;         // bytes of a g tile
  __shared__ __attribute__((aligned(1024))) char xs[4][kPBuf][XW];
  __shared__ __attribute__((aligned(1024))) char gs[kGBuf][GT];

  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63;
  const int q = lane >> 4, l16 = lane & 15;
  const int tc = lane & 3, tr = (lane >> 2) & 3;
  const int64_t nrt = (p.nS + kPS - 1) / kPS;
  const int64_t total = nrt * p.hchunks * p.nsplit;
  const int64_t id = xcd_remap(blockIdx.x, total);
  const int64_t rt = id % nrt, rest = id / nrt;
  const int hc = (int)(rest % p.hchunks), split = (int)(rest / p.hchunks);
  const int64_t s0 = rt * kPS;
  const int64_t H = p.H, row_bytes = H * 2, ldb = p.ld * 2;
  const int kw0 = hc * 4 * NCOL + w * NCOL;
  const int64_t xb0 = (int64_t)split * p.x_split;
  const int64_t xe = (xb0 + p.x_split) < p.nX ? (xb0 + p.x_split) : p.nX;
  const int64_t ntiles = xe > xb0 ? (xe - xb0 + kPX - 1) / kPX : 0;

  f32x16_t acc[2][NB];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[sb][cb][r] = 0.f;

  // X planes: as in the pipelined kernel (lane l lands on slot (row l/4, chunk l%4))
  const int dn = lane >> 2, du = (lane & 3) ^ tsw(lane >> 2);
  const uint32_t dma_off =
      (kw0 + 8 * du < H) ? (uint32_t)(dn * row_bytes + (kw0 + 8 * du) * 2) : 0x80000000u;
  // g quarter of this wave: lanes 0..31, 16 bytes each, landing at 512 w + 16 lane
  uint32_t g_off;
  if (DW) {  // row n = 4 w + lane/8 of G[16 tokens][64 vocab]; physical 32-byte group permuted
    const int n = 4 * w + (lane >> 3), c = lane & 7;
    const int lg = (c >> 1) ^ gsw2(n);
    g_off = (uint32_t)(n * ldb + (16 * lg + 8 * (c & 1)) * 2);
  } else {   // token row m = 16 w + lane/2 of G[64 tokens][16 vocab]
    g_off = (uint32_t)((16 * w + (lane >> 1)) * ldb + 16 * (lane & 1));
  }
  char* const xw = xs[w][0];
  auto lds_u32 = [](const char* ptr) {
    return (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)(uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)ptr));
  };
  const uint32_t xw_lds = lds_u32(xw);
  const uint32_t gs_lds = lds_u32(gs[0]) + 512u * (uint32_t)w;
  auto x_rsrc = [&](int64_t tile) {
    const int64_t x0 = xb0 + tile * kPX;
    return make_rsrc_words(p.X + x0 * H, (xe - x0) * row_bytes);
  };
  auto g_rsrc = [&](int64_t tile) {
    const int64_t x0 = xb0 + tile * kPX;
    return DW ? make_rsrc_words(p.G + x0 * p.ld + s0, (p.g_rows - x0) * ldb - s0 * 2)
              : make_rsrc_words(p.G + s0 * p.ld + x0, (p.g_rows - s0) * ldb - x0 * 2);
  };
  auto g_dma = [&](int64_t tile, int slot) {
    const u32x4_t rg = g_rsrc(tile);
    if (lane < 32) dma16(rg, gs_lds + (uint32_t)(slot * GT), g_off);
  };
  auto x_dma = [&](int64_t tile, int buf) {
    DmaPlanes<0, NB>::run(x_rsrc(tile), xw_lds + (uint32_t)(buf * XW), dma_off);
  };

  // GEMM3 operand offsets (as in the pipelined kernel)
  int o_g3[2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int n = tq(2 * (q >> 1) + rd, tr);
    const int u = 2 * (q & 1) + (tc >> 1);
    o_g3[rd] = 64 * n + 16 * (u ^ tsw(n)) + 8 * (tc & 1);
  }
  int o_ga[2][2];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int n = tq(2 * (q >> 1) + rd, tr);
      o_ga[sb][rd] = DW ? 128 * n + 32 * ((2 * sb + (q & 1)) ^ gsw2(n)) + 8 * tc
                        : 32 * (32 * sb + (lane & 31)) + 16 * (lane >> 5);
    }
  // (DW) grad_b: lane (q, l16) of wave w sums g[n = 4q..4q+3][m = 16 w + l16]
  const bool do_gb = DW && p.gb_acc != nullptr && hc == 0;
  float gbs = 0.f;
  constexpr bool filt = FILT;
  unsigned long long n_skipped = 0;

  if (ntiles > 0) {
    const int64_t last = ntiles - 1;
#pragma unroll
    for (int b = 0; b < kPBuf; ++b) {
      const int64_t t = b < last ? b : last;
      g_dma(t, b);
      x_dma(t, b);
    }
  }
  for (int64_t i = 0; i < ntiles; ++i) {
    const int bi = (int)(i % kPBuf), gi = (int)(i % kGBuf);
    const int64_t nxt = i + kPBuf < ntiles ? i + kPBuf : ntiles - 1;
    vm_wait<(kPBuf - 1) * NQ>();  // tile i has landed (tiles i+1 .. i+3 may be in flight)
    __syncthreads();               // every quarter of g(i) is in LDS; slot (i-1) % 5 is free
    g_dma(nxt, (int)((i + kPBuf) % kGBuf));
    const char* gb = gs[gi];
    const char* xb = xw + bi * XW;
    const u32x4_t rx = x_rsrc(nxt);
    const uint32_t lds_next = xw_lds + (uint32_t)(bi * XW);
    bool skip = false;
    if constexpr (filt) {
      // gradient filtering: every wave reads the whole g tile (2 KiB) and, when all of it is
      // below filter_eps in magnitude, takes zero operands instead of reading the tile's X and
      // g fragments (the LDS traffic is what bounds this kernel; the MFMAs still run, adding
      // zero, so the accumulators never sit across a branch) and drops its grad_b share
      const uint4 a0 = *reinterpret_cast<const uint4*>(gb + 16 * lane);
      const uint4 a1 = *reinterpret_cast<const uint4*>(gb + 1024 + 16 * lane);
      const uint32_t wv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      float mx = 0.f;  // largest magnitude (no short-circuit: no branches per element)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        mx = fmaxf(mx, fmaxf(fabsf(__uint_as_float(wv[k] << 16)), fabsf(__uint_as_float(wv[k] & 0xffff0000u))));
      skip = __builtin_amdgcn_ballot_w64(!(mx < p.filter_eps)) == 0;
      if (skip) ++n_skipped;
    }
    Frag<bf16_t> ga[2];
    // every operand read is issued before the first refill (a refill is an asm statement with
    // a memory clobber: no LDS read can move across it, and reads issued after it would
    // leave each pair of MFMAs waiting for its read's latency)
    Frag<bf16_t> xf[NB];
    if (!skip) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        if (DW) {
          ga[sb].v = tr_pair(gb + o_ga[sb][0], gb + o_ga[sb][1]);
        } else {
          // tokens' rows hold vocabulary columns n = 0..15 in order; the B operand pairs its
          // k index with the columns 0,1,4,5,2,3,6,7 (+8): swap the middle dwords
          const uint4 r = *reinterpret_cast<const uint4*>(gb + o_ga[sb][0]);
          ga[sb].v = __builtin_bit_cast(bf16x8_t, make_uint4(r.x, r.z, r.y, r.w));
        }
      }
      if (do_gb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = 4 * q + j;
          gbs += bf2f(*reinterpret_cast<const bf16_t*>(gb + 128 * n + 32 * (w ^ gsw2(n)) + 2 * l16));
        }
      }
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) xf[cb].v = tr_pair(xb + 1024 * cb + o_g3[0], xb + 1024 * cb + o_g3[1]);
    } else {
      zero8(ga[0]);
      zero8(ga[1]);
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) zero8(xf[cb]);
    }
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      mfma_32x32x16(ga[0], xf[cb], acc[0][cb]);
      mfma_32x32x16(ga[1], xf[cb], acc[1][cb]);
      dma16_after(rx, lds_next + 1024 * cb, dma_off + 64 * cb, xf[cb].v);
    }
  }
  vm_wait<0>();  // no load into LDS may still be in flight when the workgroup ends
  if (FILT && p.filter_counts != nullptr && hc == 0 && tid == 0) {  // (each tile counted once)
    atomicAdd(&p.filter_counts[0], n_skipped);
    atomicAdd(&p.filter_counts[1], (unsigned long long)ntiles);
  }

  const long long nvalid = *p.n_valid;
  const float cscale = p.mean ? 1.f / (float)(nvalid > 1 ? nvalid : 1) : 1.f;
  if (!DW) {
    float* part = p.part + (int64_t)split * p.nS * H;
    auto put = [&](auto add) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
          const int64_t col = kw0 + cb * 32 + (lane & 31);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t row = s0 + sb * 32 + acc_row(lane, r);
            if (row < p.nS && col < H) {
              float* q = part + row * H + col;
              *q = decltype(add)::value ? acc[sb][cb][r] + *q : acc[sb][cb][r];
            }
          }
        }
    };
    if (p.part_add) put(std::true_type{});
    else put(std::false_type{});
  } else {
    if (p.acc != nullptr || p.out != nullptr) {
      // Read-modify-write of the running fp32 sums in 16-byte pieces: each half (32 rows) of
      // the wave's accumulator block goes through the wave's own tile buffers (no load is in
      // flight any more; no other wave uses them) and comes back one row per instruction,
      // 4 consecutive columns per lane, with every load of a half issued before its stores.
      static_assert(kPBuf * XW == 32 * NCOL * 4, "a half accumulator block fills the wave's tile buffers");
      float* const tb = reinterpret_cast<float*>(xw);
      constexpr int NQL = NCOL / 4;  // lanes per row
      const bool lane_on = lane < NQL;
      const int64_t col = kw0 + 4 * lane;
      const bool col_ok = lane_on && col < H;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
#pragma unroll
        for (int cb = 0; cb < NB; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) tb[acc_row(lane, r) * NCOL + cb * 32 + (lane & 31)] = acc[sb][cb][r];
        float4 old[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int64_t row = s0 + sb * 32 + i;
          old[i] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (!p.first && col_ok && row < p.nS) old[i] = *reinterpret_cast<const float4*>(p.acc + row * H + col);
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          const int64_t row = s0 + sb * 32 + i;
          if (!(col_ok && row < p.nS)) continue;
          const float4 t = lane_on ? *reinterpret_cast<const float4*>(tb + i * NCOL + 4 * lane) : old[i];
          const float4 v = make_float4(t.x + old[i].x, t.y + old[i].y, t.z + old[i].z, t.w + old[i].w);
          const int64_t k = row * H + col;
          const int64_t ko = (p.out_row_map != nullptr ? (int64_t)p.out_row_map[row] : row) * H + col;
          if (!p.last) {
            *reinterpret_cast<float4*>(p.acc + k) = v;
          } else if (p.out_f32) {
            *reinterpret_cast<float4*>(static_cast<float*>(p.out) + ko) =
                make_float4(cscale * v.x, cscale * v.y, cscale * v.z, cscale * v.w);
          } else {
            *reinterpret_cast<uint2*>(static_cast<bf16_t*>(p.out) + ko) =
                make_uint2(pack_bf2(cscale * v.x, cscale * v.y), pack_bf2(cscale * v.z, cscale * v.w));
          }
        }
        // (the next half overwrites the buffers only after this wave's reads above)
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      }
    }
    if (do_gb) {
      gbs += __shfl_xor(gbs, 16, kWave);
      gbs += __shfl_xor(gbs, 32, kWave);
      const int64_t r = s0 + 16 * w + l16;
      if (q == 0 && r < p.nS) {
        const float v = gbs + (p.first ? 0.f : p.gb_acc[r]);
        if (!p.last) p.gb_acc[r] = v;
        else p.gb_out[p.out_row_map != nullptr ? p.out_row_map[r] : r] = f2bf(cscale * v);
      }
    }
  }
}

// grad_input rows of a chunk: c * (sum of the per-range partials), in bf16.
__global__ void __launch_bounds__(256) mat_reduce_kernel(const float* __restrict__ part, int nsplit,
                                                         int64_t n, int64_t stride, bf16_t* __restrict__ out,
                                                         const int64_t* __restrict__ n_valid, int mean) {
  const long long nvalid = *n_valid;
  const float cscale = mean ? 1.f / (float)(nvalid > 1 ? nvalid : 1) : 1.f;
  for (int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 4; i < n;
       i += (int64_t)gridDim.x * blockDim.x * 4) {
    float4 a = *reinterpret_cast<const float4*>(part + i);
    for (int s = 1; s < nsplit; ++s) {
      const float4 b = *reinterpret_cast<const float4*>(part + s * stride + i);
      a.x += b.x;
      a.y += b.y;
      a.z += b.z;
      a.w += b.w;
    }
    *reinterpret_cast<uint2*>(out + i) =
        make_uint2(pack_bf2(cscale * a.x, cscale * a.y), pack_bf2(cscale * a.z, cscale * a.w));
  }
}

// Column blocks per wave for the stored-dlogits GEMMs: H <= 1024 in one chunk of 4 * 32 * NB
// columns; larger H in chunks of 4 * 32 * NB with NB from {8, 6, 4}, the least padding first.
void mat_plan(int64_t H, int* nb, int* hchunks) {
  if (H <= 1024) {
    const int64_t per = (H + 127) / 128;
    *nb = per <= 1 ? 1 : (per <= 2 ? 2 : (per <= 4 ? 4 : (per <= 6 ? 6 : 8)));
    *hchunks = 1;
    return;
  }
  int best_nb = 8;
  int64_t best_waste = -1;
  for (int cand : {8, 6, 4}) {
    const int64_t w = 128 * cand;
    const int64_t waste = (H + w - 1) / w * w - H;
    if (best_waste < 0 || waste < best_waste) {
      best_waste = waste;
      best_nb = cand;
    }
  }
  *nb = best_nb;
  *hchunks = (int)((H + 128 * best_nb - 1) / (128 * best_nb));
}

template <bool DW>
static hipError_t launch_mat_dw(int nb, const MatArgs& a, dim3 grid, hipStream_t st) {
  if (a.filter_eps > 0.f) {  // (filtering is used by the two-pass backward, H > 1024: NB 4, 6, 8)
    switch (nb) {
      case 4: hipLaunchKernelGGL((mat_gemm_kernel<DW, 4, true>), grid, dim3(kBwdThreads), 0, st, a); break;
      case 6: hipLaunchKernelGGL((mat_gemm_kernel<DW, 6, true>), grid, dim3(kBwdThreads), 0, st, a); break;
      case 8: hipLaunchKernelGGL((mat_gemm_kernel<DW, 8, true>), grid, dim3(kBwdThreads), 0, st, a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (nb) {
    case 1: hipLaunchKernelGGL((mat_gemm_kernel<DW, 1, false>), grid, dim3(kBwdThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL((mat_gemm_kernel<DW, 2, false>), grid, dim3(kBwdThreads), 0, st, a); break;
    case 4: hipLaunchKernelGGL((mat_gemm_kernel<DW, 4, false>), grid, dim3(kBwdThreads), 0, st, a); break;
    case 6: hipLaunchKernelGGL((mat_gemm_kernel<DW, 6, false>), grid, dim3(kBwdThreads), 0, st, a); break;
    case 8: hipLaunchKernelGGL((mat_gemm_kernel<DW, 8, false>), grid, dim3(kBwdThreads), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mat_gemm(bool dw, const MatArgs& a, hipStream_t st) {
  int nb = 0, hc = 0;
  mat_plan(a.H, &nb, &hc);
  if (hc != a.hchunks || a.nsplit < 1 || (a.x_split % kPX) != 0) return hipErrorInvalidValue;
  const int64_t nrt = (a.nS + kPS - 1) / kPS;
  const int64_t total = nrt * a.hchunks * a.nsplit;
  if (total == 0) return hipSuccess;
  if (total > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)total);
  return dw ? launch_mat_dw<true>(nb, a, grid, st) : launch_mat_dw<false>(nb, a, grid, st);
}

hipError_t launch_mat_reduce(const float* part, int nsplit, int64_t rows, int64_t H, bf16_t* out,
                             const int64_t* n_valid, bool mean, hipStream_t st) {
  const int64_t n = rows * H;
  if (n == 0) return hipSuccess;
  int64_t blocks = (n / 4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(mat_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, st, part, nsplit, n, n, out,
                     n_valid, mean ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_bwd_dinput(const FusedArgs& a, const FusedWs& w, hipStream_t st) {
  if (a.grad_input == nullptr || a.BT == 0) return hipSuccess;
  if (use_twopass(a)) return launch_twopass_dinput(a, w, st);
  return a.bf16 ? launch_bwd<bf16_t>(a, w, false, st) : launch_bwd<float>(a, w, false, st);
}

hipError_t launch_bwd_dweight(const FusedArgs& a, const FusedWs& w, hipStream_t st) {
  if (a.grad_W == nullptr && a.grad_b == nullptr) return hipSuccess;
  if (use_twopass(a)) return launch_twopass_dweight(a, w, st);
  return a.bf16 ? launch_bwd<bf16_t>(a, w, true, st) : launch_bwd<float>(a, w, true, st);
}

}  // namespace lce
