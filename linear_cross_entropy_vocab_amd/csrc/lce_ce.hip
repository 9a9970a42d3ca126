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
  __device__ static uint4 neg_inf() { return make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u); }
  __device__ __forceinline__ float get(int i) const {
    const uint32_t w = (&raw.x)[i >> 1];
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
  // Same value, through an asm statement the optimiser cannot merge with an earlier one,
  // so a pass over the row does not keep the previous pass's unpacked floats alive.
  __device__ __forceinline__ float fresh(int i) const {
    const uint32_t w = (&raw.x)[i >> 1];
    uint32_t r;
    if (i & 1)
      asm volatile("v_and_b32 %0, 0xffff0000, %1" : "=v"(r) : "v"(w));
    else
      asm volatile("v_lshlrev_b32 %0, 16, %1" : "=v"(r) : "v"(w));
    return __uint_as_float(r);
  }
  __device__ static float elem(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0) << 16);
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  uint4 raw;
  __device__ static uint4 neg_inf() { return make_uint4(0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u); }
  __device__ __forceinline__ float get(int i) const { return __uint_as_float((&raw.x)[i]); }
  __device__ __forceinline__ float fresh(int i) const { return get(i); }
  __device__ static float elem(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
  }
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

// Row cached in registers: NV vectors of 16 B per thread, all loaded before any is used
// (buffer loads: bytes past the row read as zero and stores there are dropped).  Only the
// last vector index can run past the row; those lanes replace it with -inf so neither pass
// needs a per-element mask.  exp(x - c) is evaluated as exp2(x * log2(e) - c * log2(e)).
template <typename T, int NV>
__global__ void __launch_bounds__(kCEThreads) ce_rows_cached(T* __restrict__ logits,
                                                              const int64_t* __restrict__ targets,
                                                              int64_t V, int64_t ignore_index,
                                                              float mu, CERowOut out) {
  constexpr int EPV = Vec16<T>::N;
  constexpr float kLog2e = 1.4426950408889634f;
  // one descriptor per vector index j, based at the j-th 16 KiB slice of the row, so every
  // access uses the same lane offset tid*16 and the bounds check still ends at the row's end
  constexpr int64_t kSlice = (int64_t)kCEThreads * 16;
  __shared__ float sm[kCEWaves], ss[kCEWaves];
  const int64_t row = blockIdx.x;
  T* x = logits + row * V;
  const int tid = threadIdx.x;
  const int64_t y = targets[row];
  const bool valid = (y != ignore_index) && (y >= 0) && (y < V);
  const int64_t row_bytes = V * (int64_t)sizeof(T);
  const uint32_t lane_off = (uint32_t)tid * 16u;

  // x_y for the row result (thread 0 only; other lanes read past the end and get 0)
  const float xy = Vec16<T>::elem(make_rsrc(x, row_bytes),
                                  (tid == 0 && valid) ? (uint32_t)(y * (int64_t)sizeof(T)) : 0xfffffff0u);
  Vec16<T> buf[NV];
  // the possibly partial last vector first, so its fix-up waits for one load only
  buf[NV - 1].raw = load16(make_rsrc((const char*)x + (NV - 1) * kSlice, row_bytes - (NV - 1) * kSlice), lane_off);
#pragma unroll
  for (int j = 0; j < NV - 1; ++j)
    buf[j].raw = load16(make_rsrc((const char*)x + j * kSlice, row_bytes - j * kSlice), lane_off);
  {
    const int nvec = (int)(V / EPV);  // V * sizeof(T) is a multiple of 16 on this path
    const uint32_t keep = ((NV - 1) * kCEThreads + tid < nvec) ? 0xffffffffu : 0u;
    const uint4 ni = Vec16<T>::neg_inf();
    uint4& r = buf[NV - 1].raw;
    r.x = (r.x & keep) | (ni.x & ~keep);
    r.y = (r.y & keep) | (ni.y & ~keep);
    r.z = (r.z & keep) | (ni.z & ~keep);
    r.w = (r.w & keep) | (ni.w & ~keep);
  }

  float m = -INFINITY;
#pragma unroll
  for (int j = NV - 1; j >= 0; --j)
#pragma unroll
    for (int e = 0; e < EPV; ++e) m = fmaxf(m, buf[j].get(e));
  float s = 0.f;
  const float ml = m * kLog2e;
#pragma unroll
  for (int j = NV - 1; j >= 0; --j)
#pragma unroll
    for (int e = 0; e < EPV; ++e) s += __builtin_amdgcn_exp2f(fmaf(buf[j].fresh(e), kLog2e, -ml));
  if (m == -INFINITY) s = 0.f;
  block_ms(m, s, sm, ss);
  const float lse = m + __logf(s);
  const float scale = valid ? (1.f + 2.f * mu * lse) : 0.f;
  const float ll = lse * kLog2e;
  // the lane holding column y subtracts the one-hot term; the test on the wave and the
  // vector index is wave-uniform, so the other waves branch around it
  const int yv = valid ? (int)(y / EPV) : 0;
  const bool owner_wave = valid && ((yv % kCEThreads) / kWave) == wave_id();
  const bool owner_lane = (yv % kCEThreads) == tid;
  const int jy = yv / kCEThreads, ey = (int)(y % EPV);
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    float d[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) d[e] = __builtin_amdgcn_exp2f(fmaf(buf[j].fresh(e), kLog2e, -ll)) * scale;
    if (owner_wave && j == jy) {
#pragma unroll
      for (int e = 0; e < EPV; ++e) d[e] -= (owner_lane && e == ey) ? 1.f : 0.f;
    }
    store16(make_rsrc((char*)x + j * kSlice, row_bytes - j * kSlice), lane_off, pack_out(d, T()));
  }
  if (tid == 0) {
    out.ce[row] = valid ? (lse - xy) : 0.f;
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
