// Vocabulary sorting for gradient filtering ("Cut Cross Entropy visualized", "Vocabulary
// Sorting"): before the backward, the vocabulary is ordered by each entry's average logit
// over the batch, so that the entries likely to carry gradient share a few tiles and the
// rest fall into tiles the filter skips.
//
//   hbar     = mean of the hidden rows whose target counts (fixed-order block sums)
//   avg[v]   = W[v] . hbar + b[v]      (the batch mean of z_t[v], by linearity)
//   perm     = entries by decreasing avg, ties by increasing id (bitonic sort of 64-bit keys
//              (~order(avg) << 32 | v), padded to a power of two)
//   W_s = W[perm], b_s = b[perm], y_s = position of y in perm (ignored / out-of-range
//   targets unchanged)
// The filtered call then runs on (hidden, W_s, b_s, y_s) and the grad_W / grad_b rows are
// written back through perm.
#include "lce_common.h"
#include "lce_launch.h"

namespace lce {

constexpr int kHbarRows = 256;  // hidden rows per block sum

// part[blk][k] = sum of hidden[t][k] over the rows t of block blk whose target counts
template <typename T>
__global__ void __launch_bounds__(256) hbar_partial_kernel(const T* __restrict__ h, const int64_t* __restrict__ y,
                                                           int64_t BT, int64_t H, int64_t V, int64_t ignore_index,
                                                           float* __restrict__ part) {
  // blockIdx.x: block of rows (the long grid axis), blockIdx.y: slice of the hidden columns
  const int64_t r0 = (int64_t)blockIdx.x * kHbarRows;
  const int64_t r1 = (r0 + kHbarRows) < BT ? (r0 + kHbarRows) : BT;
  for (int64_t k = (int64_t)blockIdx.y * blockDim.x + threadIdx.x; k < H; k += (int64_t)gridDim.y * blockDim.x) {
    float acc = 0.f;
    for (int64_t t = r0; t < r1; ++t) {
      const int64_t yt = y[t];
      if (yt != ignore_index && yt >= 0 && yt < V) acc += Elem<T>::to_f(h[t * H + k]);
    }
    part[(int64_t)blockIdx.x * H + k] = acc;
  }
}

// hbar[k] = sum over blocks (in order) / max(n_valid, 1)
__global__ void __launch_bounds__(256) hbar_final_kernel(const float* __restrict__ part, int64_t nblk, int64_t H,
                                                         const int64_t* __restrict__ n_valid, float* __restrict__ hbar) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= H) return;
  double acc = 0.0;
  for (int64_t b = 0; b < nblk; ++b) acc += (double)part[b * H + k];
  const long long n = *n_valid;
  hbar[k] = (float)(acc / (double)(n > 1 ? n : 1));
}

// One wave per vocabulary entry: avg = W[v] . hbar + b[v], then the sort key.
__device__ __forceinline__ uint32_t float_order(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // unsigned order = float order
}
template <typename T>
__global__ void __launch_bounds__(256) avg_keys_kernel(const T* __restrict__ W, const T* __restrict__ bias,
                                                       const float* __restrict__ hbar, int64_t V, int64_t H,
                                                       int64_t N, unsigned long long* __restrict__ keys) {
  const int64_t v = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
  const int lane = threadIdx.x % kWave;
  if (v >= N) return;
  if (v >= V) {
    if (lane == 0) keys[v] = ~0ull;  // padding sorts last
    return;
  }
  float acc = 0.f;
  for (int64_t k = lane; k < H; k += kWave) acc += Elem<T>::to_f(W[v * H + k]) * hbar[k];
  acc = wave_sum(acc);
  if (lane == 0) {
    const float avg = acc + (bias != nullptr ? Elem<T>::to_f(bias[v]) : 0.f);
    keys[v] = ((unsigned long long)(~float_order(avg)) << 32) | (unsigned long long)(uint32_t)v;
  }
}

// Bitonic sort (ascending) of N = 2^m keys: merge steps with stride j >= 2048 go over global
// memory, the remaining steps of a stage run inside one 2048-key block in LDS.
constexpr int kSortBlock = 2048;
__device__ __forceinline__ void cmp_swap(unsigned long long& a, unsigned long long& b, bool up) {
  if ((a > b) == up) {
    const unsigned long long t = a;
    a = b;
    b = t;
  }
}
__global__ void __launch_bounds__(256) bitonic_global_kernel(unsigned long long* __restrict__ keys, int64_t N,
                                                             int64_t j, int64_t k) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one per pair
  if (i >= N / 2) return;
  const int64_t lo = (i / j) * 2 * j + (i % j), hi = lo + j;
  const bool up = (lo & k) == 0;
  unsigned long long a = keys[lo], b = keys[hi];
  cmp_swap(a, b, up);
  keys[lo] = a;
  keys[hi] = b;
}
// steps j = j0, j0/2, ..., 1 of stage k inside each block of kSortBlock keys
__global__ void __launch_bounds__(1024) bitonic_local_kernel(unsigned long long* __restrict__ keys, int64_t k_lo,
                                                             int64_t k_hi, int64_t j0_cap) {
  __shared__ unsigned long long s[kSortBlock];
  const int64_t base = (int64_t)blockIdx.x * kSortBlock;
  const int tid = threadIdx.x;
  s[tid] = keys[base + tid];
  s[tid + 1024] = keys[base + tid + 1024];
  __syncthreads();
  for (int64_t k = k_lo; k <= k_hi; k <<= 1) {
    for (int64_t j = (k >> 1) < j0_cap ? (k >> 1) : j0_cap; j >= 1; j >>= 1) {
      const int lo = (int)((tid / j) * 2 * j + (tid % j)), hi = lo + (int)j;
      const bool up = ((base + lo) & k) == 0;
      cmp_swap(s[lo], s[hi], up);
      __syncthreads();
    }
  }
  keys[base + tid] = s[tid];
  keys[base + tid + 1024] = s[tid + 1024];
}

__global__ void __launch_bounds__(256) perm_kernel(const unsigned long long* __restrict__ keys, int64_t V,
                                                   int32_t* __restrict__ perm, int32_t* __restrict__ pos) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= V) return;
  const int32_t v = (int32_t)(keys[i] & 0xffffffffull);
  perm[i] = v;
  pos[v] = (int32_t)i;
}

// dst row i = src row perm[i] (rows of `row_bytes`, a multiple of 16)
__global__ void __launch_bounds__(256) gather_rows_kernel(const char* __restrict__ src, const int32_t* __restrict__ perm,
                                                          int64_t rows, int64_t row_bytes, char* __restrict__ dst) {
  const int64_t per = row_bytes / 16;
  const int64_t n = rows * per;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = i / per, c = i % per;
    reinterpret_cast<uint4*>(dst + r * row_bytes)[c] =
        reinterpret_cast<const uint4*>(src + (int64_t)perm[r] * row_bytes)[c];
  }
}

template <typename T>
__global__ void __launch_bounds__(256) gather_bias_kernel(const T* __restrict__ b, const int32_t* __restrict__ perm,
                                                          int64_t V, T* __restrict__ bs) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < V) bs[i] = b[perm[i]];
}

__global__ void __launch_bounds__(256) remap_targets_kernel(const int64_t* __restrict__ y, const int32_t* __restrict__ pos,
                                                            int64_t BT, int64_t V, int64_t ignore_index,
                                                            int64_t* __restrict__ ys) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= BT) return;
  const int64_t v = y[t];
  ys[t] = (v != ignore_index && v >= 0 && v < V) ? (int64_t)pos[v] : v;
}

static int64_t pow2_at_least(int64_t n) {
  int64_t p = kSortBlock;
  while (p < n) p <<= 1;
  return p;
}

size_t sort_workspace_bytes(int64_t BT, int64_t H, int64_t V, size_t es) {
  const int64_t N = pow2_at_least(V);
  const int64_t nblk = (BT + kHbarRows - 1) / kHbarRows;
  size_t n = 0;
  n += ws_align((size_t)V * (size_t)H * es);   // W in sorted order
  n += ws_align((size_t)V * es);               // bias in sorted order
  n += ws_align((size_t)(BT > 0 ? BT : 1) * 8);  // targets as sorted positions
  n += 2 * ws_align((size_t)V * 4);            // perm, pos
  n += ws_align((size_t)N * 8);                // sort keys
  n += ws_align((size_t)(nblk > 0 ? nblk : 1) * (size_t)H * 4);  // block sums of hidden
  n += ws_align((size_t)H * 4);                // hbar
  return n;
}

SortWs sort_carve(void* ws, int64_t BT, int64_t H, int64_t V, size_t es) {
  SortWs s;
  s.N = pow2_at_least(V);
  s.nblk = (BT + kHbarRows - 1) / kHbarRows;
  char* p = static_cast<char*>(ws);
  s.Ws = p;
  p += ws_align((size_t)V * (size_t)H * es);
  s.bs = p;
  p += ws_align((size_t)V * es);
  s.ys = reinterpret_cast<int64_t*>(p);
  p += ws_align((size_t)(BT > 0 ? BT : 1) * 8);
  s.perm = reinterpret_cast<int32_t*>(p);
  p += ws_align((size_t)V * 4);
  s.pos = reinterpret_cast<int32_t*>(p);
  p += ws_align((size_t)V * 4);
  s.keys = reinterpret_cast<unsigned long long*>(p);
  p += ws_align((size_t)s.N * 8);
  s.part = reinterpret_cast<float*>(p);
  p += ws_align((size_t)(s.nblk > 0 ? s.nblk : 1) * (size_t)H * 4);
  s.hbar = reinterpret_cast<float*>(p);
  return s;
}

template <typename T>
static hipError_t sort_vocab_t(const FusedArgs& a, const SortWs& s, const int64_t* n_valid, hipStream_t st) {
  const T* h = static_cast<const T*>(a.hidden);
  const T* W = static_cast<const T*>(a.W);
  const T* b = static_cast<const T*>(a.bias);
  if (a.BT > 0) {
    const dim3 g1((unsigned)s.nblk, (unsigned)((a.H + 255) / 256 < 64 ? (a.H + 255) / 256 : 64));
    hipLaunchKernelGGL(hbar_partial_kernel<T>, g1, dim3(256), 0, st, h, a.targets, a.BT, a.H, a.V, a.ignore_index,
                       s.part);
  }
  hipLaunchKernelGGL(hbar_final_kernel, dim3((unsigned)((a.H + 255) / 256)), dim3(256), 0, st, s.part, s.nblk, a.H,
                     n_valid, s.hbar);
  hipLaunchKernelGGL(avg_keys_kernel<T>, dim3((unsigned)((s.N * kWave + 255) / 256)), dim3(256), 0, st, W, b, s.hbar,
                     a.V, a.H, s.N, s.keys);
  // bitonic sort: the stages k <= kSortBlock entirely in LDS; each larger stage takes its
  // steps j >= kSortBlock over global memory and the rest in LDS
  hipLaunchKernelGGL(bitonic_local_kernel, dim3((unsigned)(s.N / kSortBlock)), dim3(1024), 0, st, s.keys,
                     (int64_t)2, (int64_t)kSortBlock, (int64_t)kSortBlock / 2);
  for (int64_t k = 2 * kSortBlock; k <= s.N; k <<= 1) {
    for (int64_t j = k >> 1; j >= kSortBlock; j >>= 1)
      hipLaunchKernelGGL(bitonic_global_kernel, dim3((unsigned)((s.N / 2 + 255) / 256)), dim3(256), 0, st, s.keys,
                         s.N, j, k);
    hipLaunchKernelGGL(bitonic_local_kernel, dim3((unsigned)(s.N / kSortBlock)), dim3(1024), 0, st, s.keys, k, k,
                       (int64_t)kSortBlock / 2);
  }
  hipLaunchKernelGGL(perm_kernel, dim3((unsigned)((a.V + 255) / 256)), dim3(256), 0, st, s.keys, a.V, s.perm, s.pos);
  const int64_t row_bytes = a.H * (int64_t)sizeof(T);
  const int64_t n16 = a.V * (row_bytes / 16);
  const int64_t gb = (n16 + 255) / 256 < 8192 ? (n16 + 255) / 256 : 8192;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)gb), dim3(256), 0, st, static_cast<const char*>(a.W), s.perm,
                     a.V, row_bytes, static_cast<char*>(s.Ws));
  if (b != nullptr)
    hipLaunchKernelGGL(gather_bias_kernel<T>, dim3((unsigned)((a.V + 255) / 256)), dim3(256), 0, st, b, s.perm, a.V,
                       static_cast<T*>(s.bs));
  if (a.BT > 0)
    hipLaunchKernelGGL(remap_targets_kernel, dim3((unsigned)((a.BT + 255) / 256)), dim3(256), 0, st, a.targets, s.pos,
                       a.BT, a.V, a.ignore_index, s.ys);
  return hipGetLastError();
}

hipError_t launch_sort_vocab(const FusedArgs& a, const SortWs& s, const int64_t* n_valid, hipStream_t st) {
  return a.bf16 ? sort_vocab_t<bf16_t>(a, s, n_valid, st) : sort_vocab_t<float>(a, s, n_valid, st);
}

}  // namespace lce
