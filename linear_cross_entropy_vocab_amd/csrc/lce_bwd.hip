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
#include "lce_common.h"
#include "lce_launch.h"

namespace lce {

constexpr int kBwdThreads = 256;
constexpr int kBS = 64;  // stationary rows per workgroup
constexpr int kBX = 32;  // streamed rows per tile
constexpr int kZStride = 36;  // floats per row of a partial-z buffer (padded)

template <typename T>
struct BwdArgs {
  const T* S;
  const T* X;
  const T* bias;
  const int64_t* y;
  const float* lse;
  int64_t nS, nX, H, BT, V;
  int64_t ignore_index;
  float mu;
  const int64_t* n_valid;
  int mean;
  T* out;
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
__device__ __forceinline__ void store_frag(char* p, const Frag<bf16_t>& f) {
  *reinterpret_cast<bf16x8_t*>(p) = f.v;
}
__device__ __forceinline__ void store_frag(char* p, const Frag<float>& f) {
  reinterpret_cast<float4*>(p)[0] = make_float4(f.v[0], f.v[1], f.v[2], f.v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(f.v[4], f.v[5], f.v[6], f.v[7]);
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

// B operand of GEMM3 from the row-major X tile in LDS: lane l needs column (l % 32) of a
// 32-column block and K rows kbase + 8*(l/32) .. +7.
__device__ __forceinline__ void xt_frag(Frag<bf16_t>& f, const char* xt, int row_bytes, int kbase,
                                        int col0, int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int col = col0 + (g & 1) * 16 + 4 * (i & 3);
  const int row = kbase + (g >> 1) * 8 + (i >> 2);
  const bf16_t* p0 = reinterpret_cast<const bf16_t*>(xt + row * row_bytes + col * 2);
  const bf16_t* p1 = reinterpret_cast<const bf16_t*>(xt + (row + 4) * row_bytes + col * 2);
  const i16x4_t a = lds_read_tr16(p0);
  const i16x4_t b = lds_read_tr16(p1);
  f.v = bf16x8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ void xt_frag(Frag<float>& f, const char* xt, int row_bytes, int kbase,
                                        int col0, int lane) {
  const int col = col0 + (lane & 31);
  const int row = kbase + 8 * (lane >> 5);
#pragma unroll
  for (int s = 0; s < 8; ++s) f.v[s] = *reinterpret_cast<const float*>(xt + (row + s) * row_bytes + col * 4);
}

template <typename T>
__device__ __forceinline__ bool load_frag_masked(Frag<T>& f, const T* base, int64_t row, int64_t nrows,
                                                 int64_t k, int64_t H) {
  if (row < nrows && k < H) {
    load8(f, base + row * H + k);
    return true;
  }
  zero8(f);
  return false;
}

// SINGLE: whole H handled by one workgroup, NB = H-columns per wave / 32 (= K quarter / 32).
// CHUNKED: output columns split into nchunks chunks of 4*NB*32; S streamed from L2.
template <typename T, bool DW, bool SINGLE, int NB>
__global__ void __launch_bounds__(kBwdThreads, 1) bwd_kernel(BwdArgs<T> p) {
  constexpr int ES = sizeof(T);
  constexpr int NCOL = NB * 32;
  constexpr int XT_ROW = NCOL * ES + 64;            // bytes per row of a wave's X tile
  constexpr int G_ROW = kBX * ES + 16;              // bytes per row of the dlogits tile
  constexpr int KS1S = 2 * NB;                      // GEMM1 k-steps per wave (SINGLE)
  __shared__ __attribute__((aligned(16))) float zpart[4][kBS * kZStride];
  __shared__ __attribute__((aligned(16))) char gtile[kBS * G_ROW];
  __shared__ __attribute__((aligned(16))) char xtile[4][kBX * XT_ROW];

  const int tid = threadIdx.x, w = tid / kWave, lane = tid % kWave;
  const int64_t s_tile = blockIdx.x / p.nchunks;
  const int64_t chunk = blockIdx.x % p.nchunks;
  const int64_t s0 = s_tile * kBS;
  const int64_t h0 = chunk * (4 * NCOL);            // first output column of this workgroup
  const int64_t hw0 = h0 + w * NCOL;                // first output column of this wave
  const int64_t H = p.H;
  // GEMM1 K range of this wave
  const int64_t KW = SINGLE ? (int64_t)NCOL : ((H + 63) / 64) * 16;
  const int64_t kw0 = w * KW;
  const int ks1 = SINGLE ? KS1S : (int)(KW / 16);

  const long long nvalid = *p.n_valid;
  const float cscale = p.mean ? 1.f / (float)(nvalid > 1 ? nvalid : 1) : 1.f;

  // Reduce-step assignment: row rr of the 64, columns c0 .. c0+7 of the 32.
  const int rr = 16 * w + (lane >> 2);
  const int c0 = (lane & 3) * 8;
  const int64_t srow = s0 + rr;
  // Per stationary-row quantities.
  float row_lse = 0.f, row_f = 0.f, row_bias = 0.f;
  int64_t row_y = -1;
  bool row_ok = false;
  if (!DW) {
    if (srow < p.BT) {
      const int64_t yt = p.y[srow];
      row_ok = (yt != p.ignore_index) && yt >= 0 && yt < p.V;
      row_y = yt;
      row_lse = p.lse[srow];
      row_f = 1.f + 2.f * p.mu * row_lse;
    }
  } else {
    row_ok = srow < p.V;
    row_bias = (p.bias != nullptr && row_ok) ? Elem<T>::to_f(p.bias[srow]) : 0.f;
  }
  float gb_acc = 0.f;

  // Stationary fragments (SINGLE only): S rows s0 + sb*32 + lane%32, K quarter of wave w.
  Frag<T> sf[SINGLE ? KS1S : 1][2];
  if (SINGLE) {
#pragma unroll
    for (int ks = 0; ks < KS1S; ++ks)
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
        load_frag_masked(sf[ks][sb], p.S, s0 + sb * 32 + (lane & 31), p.nS, kw0 + ks * 16 + 8 * (lane >> 5), H);
  }

  f32x16_t acc[2][NB];
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[sb][cb][r] = 0.f;

  char* xt = xtile[w];
  const int64_t ntiles = (p.nX + kBX - 1) / kBX;
  for (int64_t xtl = 0; xtl < ntiles; ++xtl) {
    const int64_t x0 = xtl * kBX;
    const int64_t xrow = x0 + (lane & 31);
    // ---------------- GEMM1: partial z over this wave's K quarter
    f32x16_t zp[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) zp[sb][r] = 0.f;
    if (SINGLE) {
#pragma unroll
      for (int ks = 0; ks < KS1S; ++ks) {
        Frag<T> xf;
        load_frag_masked(xf, p.X, xrow, p.nX, kw0 + ks * 16 + 8 * (lane >> 5), H);
        // the same X values are GEMM3's operand for this wave's columns
        store_frag(xt + (lane & 31) * XT_ROW + (ks * 16 + 8 * (lane >> 5)) * ES, xf);
        mfma_32x32x16(sf[ks][0], xf, zp[0]);
        mfma_32x32x16(sf[ks][1], xf, zp[1]);
      }
    } else {
      for (int ks = 0; ks < ks1; ++ks) {
        const int64_t k = kw0 + ks * 16 + 8 * (lane >> 5);
        Frag<T> xf, a0, a1;
        load_frag_masked(xf, p.X, xrow, p.nX, k, H);
        load_frag_masked(a0, p.S, s0 + (lane & 31), p.nS, k, H);
        load_frag_masked(a1, p.S, s0 + 32 + (lane & 31), p.nS, k, H);
        mfma_32x32x16(a0, xf, zp[0]);
        mfma_32x32x16(a1, xf, zp[1]);
      }
      // X rows for this wave's output columns
      constexpr int CH = NCOL * ES / 16;  // 16 B chunks per row
#pragma unroll
      for (int i = 0; i < (kBX * CH + kWave - 1) / kWave; ++i) {
        const int c = lane + kWave * i;
        if (c < kBX * CH) {
          const int r = c / CH, cc = c % CH;
          const int64_t col = hw0 + cc * (16 / ES);
          uint4 v = make_uint4(0, 0, 0, 0);
          if (x0 + r < p.nX && col < H) v = *reinterpret_cast<const uint4*>(p.X + (x0 + r) * H + col);
          *reinterpret_cast<uint4*>(xt + r * XT_ROW + cc * 16) = v;
        }
      }
    }
    // ---------------- partial z to LDS
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) zpart[w][(sb * 32 + acc_row(lane, r)) * kZStride + (lane & 31)] = zp[sb][r];
    __syncthreads();
    // ---------------- z for row rr, columns c0..c0+7; dlogits
    float z[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) z[e] = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 a = *reinterpret_cast<const float4*>(&zpart[q][rr * kZStride + c0]);
      const float4 b = *reinterpret_cast<const float4*>(&zpart[q][rr * kZStride + c0 + 4]);
      z[0] += a.x; z[1] += a.y; z[2] += a.z; z[3] += a.w;
      z[4] += b.x; z[5] += b.y; z[6] += b.z; z[7] += b.w;
    }
    float g[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t xc = x0 + c0 + e;  // streamed row index of this column
      float gv = 0.f;
      if (!DW) {
        // token = srow, vocab = xc
        if (row_ok && xc < p.V) {
          const float b = p.bias != nullptr ? Elem<T>::to_f(p.bias[xc]) : 0.f;
          gv = __expf(z[e] + b - row_lse) * row_f - (xc == row_y ? 1.f : 0.f);
        }
      } else {
        // vocab = srow, token = xc
        if (row_ok && xc < p.BT) {
          const int64_t yt = p.y[xc];
          if (yt != p.ignore_index && yt >= 0 && yt < p.V) {
            const float L = p.lse[xc];
            gv = __expf(z[e] + row_bias - L) * (1.f + 2.f * p.mu * L) - (yt == srow ? 1.f : 0.f);
          }
        }
      }
      g[e] = gv;
    }
    if (DW) {
#pragma unroll
      for (int e = 0; e < 8; ++e) gb_acc += g[e];
    }
    store8(gtile + rr * G_ROW + c0 * ES, g, T());
    __syncthreads();
    // ---------------- GEMM3: acc += g . X[:, wave columns]
#pragma unroll
    for (int kk = 0; kk < kBX / 16; ++kk) {
      Frag<T> ga[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
        lds_frag(ga[sb], gtile + (sb * 32 + (lane & 31)) * G_ROW + (kk * 16 + 8 * (lane >> 5)) * ES);
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        Frag<T> xb;
        xt_frag(xb, xt, XT_ROW, kk * 16, cb * 32, lane);
        mfma_32x32x16(ga[0], xb, acc[0][cb]);
        mfma_32x32x16(ga[1], xb, acc[1][cb]);
      }
    }
  }

  // ---------------- write c * acc
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      const int64_t col = hw0 + cb * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = s0 + sb * 32 + acc_row(lane, r);
        if (p.out != nullptr && row < p.nS && col < H) p.out[row * H + col] = Elem<T>::from_f(cscale * acc[sb][cb][r]);
      }
    }
  if (DW && p.grad_b != nullptr && chunk == 0) {
    gb_acc += __shfl_xor(gb_acc, 1, kWave);
    gb_acc += __shfl_xor(gb_acc, 2, kWave);
    if ((lane & 3) == 0 && srow < p.V) p.grad_b[srow] = Elem<T>::from_f(cscale * gb_acc);
  }
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
    a.grad_b = nullptr;
  } else {
    a.S = static_cast<const T*>(fa.W);
    a.X = static_cast<const T*>(fa.hidden);
    a.nS = fa.V;
    a.nX = fa.BT;
    a.out = static_cast<T*>(fa.grad_W);
    a.grad_b = static_cast<T*>(fa.grad_b);
  }
  const BwdPlan pl = bwd_plan(fa.H, sizeof(T) == 2);
  a.nchunks = pl.nchunks;
  const int64_t ntile = (a.nS + kBS - 1) / kBS;
  if (ntile == 0) return hipSuccess;
  dim3 grid((unsigned)(ntile * pl.nchunks));
  if (!dw) {
    return pl.single ? launch_bwd_nb<T, false, true>(pl.nb, a, grid, st)
                     : launch_bwd_nb<T, false, false>(pl.nb, a, grid, st);
  }
  return pl.single ? launch_bwd_nb<T, true, true>(pl.nb, a, grid, st)
                   : launch_bwd_nb<T, true, false>(pl.nb, a, grid, st);
}

hipError_t launch_bwd_dinput(const FusedArgs& a, const FusedWs& w, hipStream_t st) {
  if (a.grad_input == nullptr || a.BT == 0) return hipSuccess;
  return a.bf16 ? launch_bwd<bf16_t>(a, w, false, st) : launch_bwd<float>(a, w, false, st);
}

hipError_t launch_bwd_dweight(const FusedArgs& a, const FusedWs& w, hipStream_t st) {
  if (a.grad_W == nullptr && a.grad_b == nullptr) return hipSuccess;
  return a.bf16 ? launch_bwd<bf16_t>(a, w, true, st) : launch_bwd<float>(a, w, true, st);
}

}  // namespace lce
