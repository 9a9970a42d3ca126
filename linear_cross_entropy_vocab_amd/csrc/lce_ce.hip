// Standalone cross-entropy + dlogits on existing logits, written in place.
//
// Follows "Greyhound -- Cross-Entropy", section "Kernel design": one workgroup per row
// computes the row's log-sum-exp with fp32 online (max, sum) accumulation, reduces it
// across the workgroup, then overwrites the row with
//   valid * (softmax * (1 + 2 mu LSE) - onehot(y)).
// Differences from that design, for gfx950: the row is cached in VGPRs between the two
// passes when it fits (1024 threads x up to 16 x 16 B = 256 KiB), so HBM sees one read
// and one write per element; reductions are wave64 shuffles plus an LDS step; per-row
// results go to a buffer and a second kernel sums them in a fixed order (no atomics),
// with the valid count kept as an integer.
#include "lce_common.h"
#include "lce_launch.h"

namespace lce {

constexpr int kCEThreads = 1024;
constexpr int kCEWaves = kCEThreads / kWave;

struct CERowOut {
  float* ce;     // [B] LSE - x_y (0 for ignored rows)
  float* zsq;    // [B] LSE^2     (0 for ignored rows)
  int32_t* valid;  // [B] 1 if the row counts
};

template <typename T>
struct Vec16;  // 16 bytes of T
template <> struct Vec16<bf16_t> {
  static constexpr int N = 8;
  uint4 raw;
  __device__ __forceinline__ float get(int i) const {
    const uint32_t w = (&raw.x)[i >> 1];
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  uint4 raw;
  __device__ __forceinline__ float get(int i) const { return __uint_as_float((&raw.x)[i]); }
};

__device__ __forceinline__ uint4 pack_out(const float* v, bf16_t) {
  return make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]),
                    pack_bf2(v[6], v[7]));
}
__device__ __forceinline__ uint4 pack_out(const float* v, float) {
  return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                    __float_as_uint(v[3]));
}

// Block-wide (max, sum) merge: every thread returns the row's (m, s).
__device__ __forceinline__ void block_ms(float& m, float& s, float* sm, float* ss) {
  wave_ms(m, s);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  if (l == 0) { sm[w] = m; ss[w] = s; }
  __syncthreads();
  m = -INFINITY;
  s = 0.f;
  for (int i = 0; i < kCEWaves; ++i) ms_merge(m, s, sm[i], ss[i]);  // same order in every thread
}

// Row cached in registers: NV vectors of 16 B per thread.
template <typename T, int NV>
__global__ void __launch_bounds__(kCEThreads) ce_rows_cached(T* __restrict__ logits,
                                                              const int64_t* __restrict__ targets,
                                                              int64_t V, int64_t ignore_index,
                                                              float mu, CERowOut out) {
  constexpr int EPV = Vec16<T>::N;
  __shared__ float sm[kCEWaves], ss[kCEWaves];
  __shared__ float s_xy;
  const int64_t row = blockIdx.x;
  T* x = logits + row * V;
  const int64_t nvec = V / EPV;  // V * sizeof(T) is a multiple of 16 on this path
  const int tid = threadIdx.x;
  const int64_t y = targets[row];
  const bool valid = (y != ignore_index) && (y >= 0) && (y < V);

  Vec16<T> buf[NV];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int64_t vi = (int64_t)j * kCEThreads + tid;
    if (vi < nvec) buf[j].raw = reinterpret_cast<const uint4*>(x)[vi];
    else buf[j].raw = make_uint4(0, 0, 0, 0);
  }
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int64_t vi = (int64_t)j * kCEThreads + tid;
    if (vi < nvec) {
#pragma unroll
      for (int e = 0; e < EPV; ++e) m = fmaxf(m, buf[j].get(e));
    }
  }
  float s = 0.f;
  if (m != -INFINITY) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int64_t vi = (int64_t)j * kCEThreads + tid;
      if (vi < nvec) {
#pragma unroll
        for (int e = 0; e < EPV; ++e) s += __expf(buf[j].get(e) - m);
      }
    }
  }
  if (valid) {
    const int64_t vi = y / EPV;
    if ((vi % kCEThreads) == tid) {
      const int j = (int)(vi / kCEThreads);
#pragma unroll
      for (int jj = 0; jj < NV; ++jj)
        if (jj == j) s_xy = buf[jj].get((int)(y % EPV));
    }
  }
  block_ms(m, s, sm, ss);
  const float lse = m + __logf(s);
  const float scale = valid ? (1.f + 2.f * mu * lse) : 0.f;
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const int64_t vi = (int64_t)j * kCEThreads + tid;
    if (vi < nvec) {
      float d[EPV];
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const int64_t col = vi * EPV + e;
        float g = __expf(buf[j].get(e) - lse) * scale;
        if (valid && col == y) g -= 1.f;
        d[e] = g;
      }
      reinterpret_cast<uint4*>(x)[vi] = pack_out(d, T());
    }
  }
  if (tid == 0) {
    out.ce[row] = valid ? (lse - s_xy) : 0.f;
    out.zsq[row] = valid ? lse * lse : 0.f;
    out.valid[row] = valid ? 1 : 0;
  }
}

// Any V: two passes over global memory (the second read usually hits the last-level cache).
template <typename T>
__global__ void __launch_bounds__(kCEThreads) ce_rows_stream(T* __restrict__ logits,
                                                              const int64_t* __restrict__ targets,
                                                              int64_t V, int64_t ignore_index,
                                                              float mu, CERowOut out) {
  __shared__ float sm[kCEWaves], ss[kCEWaves];
  const int64_t row = blockIdx.x;
  T* x = logits + row * V;
  const int tid = threadIdx.x;
  const int64_t y = targets[row];
  const bool valid = (y != ignore_index) && (y >= 0) && (y < V);
  float m = -INFINITY, s = 0.f;
  for (int64_t c = tid; c < V; c += kCEThreads) {
    const float v = Elem<T>::to_f(x[c]);
    if (v > m) {
      s = s * __expf(m - v) + 1.f;
      m = v;
    } else {
      s += __expf(v - m);
    }
  }
  const float xy = valid ? Elem<T>::to_f(x[y]) : 0.f;
  block_ms(m, s, sm, ss);
  const float lse = m + __logf(s);
  const float scale = valid ? (1.f + 2.f * mu * lse) : 0.f;
  for (int64_t c = tid; c < V; c += kCEThreads) {
    float g = __expf(Elem<T>::to_f(x[c]) - lse) * scale;
    if (valid && c == y) g -= 1.f;
    x[c] = Elem<T>::from_f(g);
  }
  if (tid == 0) {
    out.ce[row] = valid ? (lse - xy) : 0.f;
    out.zsq[row] = valid ? lse * lse : 0.f;
    out.valid[row] = valid ? 1 : 0;
  }
}

// Fixed-order sums of the per-row results (one workgroup).
__global__ void __launch_bounds__(kCEThreads) ce_reduce(const float* __restrict__ ce,
                                                         const float* __restrict__ zsq,
                                                         const int32_t* __restrict__ valid,
                                                         int64_t B, int use_z, float* ce_sum,
                                                         float* z_sum, int64_t* n_valid) {
  __shared__ double s_ce[kCEWaves], s_z[kCEWaves];
  __shared__ long long s_n[kCEWaves];
  double a = 0.0, b = 0.0;
  long long n = 0;
  for (int64_t i = threadIdx.x; i < B; i += kCEThreads) {
    a += (double)ce[i];
    b += (double)zsq[i];
    n += valid[i];
  }
  a = wave_sum_d(a);
  b = wave_sum_d(b);
  n = wave_sum_ll(n);
  const int w = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) { s_ce[w] = a; s_z[w] = b; s_n[w] = n; }
  __syncthreads();
  if (threadIdx.x == 0) {
    double ta = 0.0, tb = 0.0;
    long long tn = 0;
    for (int i = 0; i < kCEWaves; ++i) { ta += s_ce[i]; tb += s_z[i]; tn += s_n[i]; }
    *ce_sum = (float)ta;
    *z_sum = use_z ? (float)tb : 0.f;
    if (n_valid) *n_valid = tn;
  }
}

template <typename T>
static hipError_t launch_rows(T* logits, const int64_t* targets, int64_t B, int64_t V,
                              int64_t ignore_index, float mu, CERowOut out, hipStream_t st) {
  constexpr int EPV = 16 / (int)sizeof(T);
  const bool vec_ok = ((V * (int64_t)sizeof(T)) % 16) == 0;
  const int64_t nvec = V / EPV;
  const int64_t per = (nvec + kCEThreads - 1) / kCEThreads;
  dim3 grid((unsigned)B), block(kCEThreads);
  if (vec_ok && per <= 16) {
    if (per <= 1) hipLaunchKernelGGL((ce_rows_cached<T, 1>), grid, block, 0, st, logits, targets, V, ignore_index, mu, out);
    else if (per <= 2) hipLaunchKernelGGL((ce_rows_cached<T, 2>), grid, block, 0, st, logits, targets, V, ignore_index, mu, out);
    else if (per <= 4) hipLaunchKernelGGL((ce_rows_cached<T, 4>), grid, block, 0, st, logits, targets, V, ignore_index, mu, out);
    else if (per <= 8) hipLaunchKernelGGL((ce_rows_cached<T, 8>), grid, block, 0, st, logits, targets, V, ignore_index, mu, out);
    else hipLaunchKernelGGL((ce_rows_cached<T, 16>), grid, block, 0, st, logits, targets, V, ignore_index, mu, out);
  } else {
    hipLaunchKernelGGL((ce_rows_stream<T>), grid, block, 0, st, logits, targets, V, ignore_index, mu, out);
  }
  return hipGetLastError();
}

hipError_t launch_ce_inplace(void* logits, bool bf16, const int64_t* targets, int64_t B, int64_t V,
                             int64_t ignore_index, float mu, float* ce_sum, float* z_sum,
                             int64_t* n_valid, void* workspace, hipStream_t st) {
  CERowOut out;
  char* ws = static_cast<char*>(workspace);
  const size_t a = ws_align((size_t)B * 4);
  out.ce = reinterpret_cast<float*>(ws);
  out.zsq = reinterpret_cast<float*>(ws + a);
  out.valid = reinterpret_cast<int32_t*>(ws + 2 * a);
  hipError_t e = hipSuccess;
  if (B > 0) {
    e = bf16 ? launch_rows<bf16_t>(static_cast<bf16_t*>(logits), targets, B, V, ignore_index, mu, out, st)
             : launch_rows<float>(static_cast<float*>(logits), targets, B, V, ignore_index, mu, out, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(ce_reduce, dim3(1), dim3(kCEThreads), 0, st, out.ce, out.zsq, out.valid, B,
                     mu != 0.f ? 1 : 0, ce_sum, z_sum, n_valid);
  return hipGetLastError();
}

size_t ce_workspace_bytes(int64_t B) { return 3 * ws_align((size_t)(B > 0 ? B : 1) * 4); }

}  // namespace lce
