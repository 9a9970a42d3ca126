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
  float* lse;    // [B] LSE of every row, or NULL
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
template <> struct Vec16<f16_t> {
  static constexpr int N = 8;
  uint4 raw;
  __device__ static uint4 neg_inf() { return make_uint4(0xfc00fc00u, 0xfc00fc00u, 0xfc00fc00u, 0xfc00fc00u); }
  __device__ __forceinline__ float get(int i) const {
    const uint32_t w = (&raw.x)[i >> 1];
    return (float)__builtin_bit_cast(f16_t, (uint16_t)((i & 1) ? (w >> 16) : (w & 0xffffu)));
  }
  // (as for bf16: an asm conversion the optimiser cannot merge with the first pass's)
  __device__ __forceinline__ float fresh(int i) const {
    const uint32_t w = (&raw.x)[i >> 1];
    float r;
    if (i & 1)
      asm volatile("v_lshrrev_b32 %0, 16, %1\n\tv_cvt_f32_f16 %0, %0" : "=&v"(r) : "v"(w));
    else
      asm volatile("v_cvt_f32_f16 %0, %1" : "=v"(r) : "v"(w));
    return r;
  }
  __device__ static float elem(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return (float)__builtin_bit_cast(f16_t, (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0));
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
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (f16_t)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (f16_t)b) << 16);
}
__device__ __forceinline__ uint4 pack_out(const float* v, f16_t) {
  return make_uint4(pack_h2(v[0], v[1]), pack_h2(v[2], v[3]), pack_h2(v[4], v[5]), pack_h2(v[6], v[7]));
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

// Lanes of vector index j whose elements lie at or past V get -inf there (rows are read
// with the padded row length ld as the bound, so those elements are zero or padding).
template <typename T>
__device__ __forceinline__ void mask_tail(Vec16<T>& v, int64_t c0, int64_t V);
template <>
__device__ __forceinline__ void mask_tail(Vec16<bf16_t>& v, int64_t c0, int64_t V) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t& x = (&v.raw.x)[d];
    const uint32_t lo = (c0 + 2 * d < V) ? (x & 0x0000ffffu) : 0x0000ff80u;
    const uint32_t hi = (c0 + 2 * d + 1 < V) ? (x & 0xffff0000u) : 0xff800000u;
    x = lo | hi;
  }
}
template <>
__device__ __forceinline__ void mask_tail(Vec16<f16_t>& v, int64_t c0, int64_t V) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t& x = (&v.raw.x)[d];
    const uint32_t lo = (c0 + 2 * d < V) ? (x & 0x0000ffffu) : 0x0000fc00u;
    const uint32_t hi = (c0 + 2 * d + 1 < V) ? (x & 0xffff0000u) : 0xfc000000u;
    x = lo | hi;
  }
}
template <>
__device__ __forceinline__ void mask_tail(Vec16<float>& v, int64_t c0, int64_t V) {
#pragma unroll
  for (int d = 0; d < 4; ++d) (&v.raw.x)[d] = (c0 + d < V) ? (&v.raw.x)[d] : 0xff800000u;
}

// The same for a vector whose first element is element `first` of a run with `rem` elements
// before V (32-bit arithmetic): elements at or past rem become -inf.
template <typename T>
__device__ __forceinline__ void mask_run(Vec16<T>& v, int first, int rem) {
  constexpr int EPV = Vec16<T>::N;
  if constexpr (EPV == 4) {
#pragma unroll
    for (int d = 0; d < 4; ++d) (&v.raw.x)[d] = (first + d < rem) ? (&v.raw.x)[d] : 0xff800000u;
  } else {
    const uint32_t ninf = Vec16<T>::neg_inf().x;  // two -inf halves
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t& x = (&v.raw.x)[d];
      const uint32_t lo = (first + 2 * d < rem) ? (x & 0x0000ffffu) : (ninf & 0x0000ffffu);
      const uint32_t hi = (first + 2 * d + 1 < rem) ? (x & 0xffff0000u) : (ninf & 0xffff0000u);
      x = lo | hi;
    }
  }
}

// Row cached in registers: NV vectors of 16 B per thread, all loaded before any is used
// (buffer loads: bytes past the row read as zero and stores there are dropped; the stores
// use the non-temporal cache policy, measured 4% faster, the loads the default one, which
// measured faster than non-temporal loads).  NV is the
// per-thread vector count rounded up to a power of two, so every vector index below NV/2 is
// inside the row; the upper half is masked per element (-inf past V), so neither pass needs
// a mask.  Rows are ld elements apart (ld >= V; ld * sizeof(T) a multiple of 16); the
// columns V..ld-1 are written as 0.  exp(x - c) is evaluated as exp2(x * log2(e) - c * log2(e)).
template <typename T, int NV>
__global__ void __launch_bounds__(kCEThreads) ce_rows_cached(T* __restrict__ logits,
                                                              const int64_t* __restrict__ targets,
                                                              int64_t V, int64_t ld, int64_t ignore_index,
                                                              float mu, CERowOut out) {
  constexpr int EPV = Vec16<T>::N;
  constexpr float kLog2e = 1.4426950408889634f;
  // one descriptor per vector index j, based at the j-th 16 KiB slice of the row, so every
  // access uses the same lane offset tid*16 and the bounds check still ends at the row's end
  constexpr int64_t kSlice = (int64_t)kCEThreads * 16;
  __shared__ float sm[kCEWaves], ss[kCEWaves];
  const int64_t row = blockIdx.x;
  T* x = logits + row * ld;
  const int tid = threadIdx.x;
  const int64_t y = targets[row];
  const bool valid = (y != ignore_index) && (y >= 0) && (y < V);
  const int64_t row_bytes = ld * (int64_t)sizeof(T);
  const uint32_t lane_off = (uint32_t)tid * 16u;

  // x_y for the row result (thread 0 only; other lanes read past the end and get 0)
  const float xy = Vec16<T>::elem(make_rsrc(x, row_bytes),
                                  (tid == 0 && valid) ? (uint32_t)(y * (int64_t)sizeof(T)) : 0xfffffff0u);
  Vec16<T> buf[NV];
  // the possibly partial upper vectors first (last one first), so their fix-up waits for as
  // few loads as possible
  constexpr int JM = NV / 2;  // vectors JM .. NV-1 may run past V
#pragma unroll
  for (int j = NV - 1; j >= 0; --j)
    buf[j].raw = load16(make_rsrc((const char*)x + j * kSlice, row_bytes - j * kSlice), lane_off);
#pragma unroll
  for (int j = NV - 1; j >= JM; --j) mask_tail(buf[j], ((int64_t)j * kCEThreads + tid) * EPV, V);

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
    store16_nt(make_rsrc((char*)x + j * kSlice, row_bytes - j * kSlice), lane_off, pack_out(d, T()));
  }
  if (tid == 0) {
    out.ce[row] = valid ? (lse - xy) : 0.f;
    out.zsq[row] = valid ? lse * lse : 0.f;
    out.valid[row] = valid ? 1 : 0;
    if (out.lse != nullptr) out.lse[row] = lse;
  }
}

// Rows longer than the register cache of a 1024-thread workgroup and at most 512 KiB (the fp32
// rows of a 128Ki-entry vocabulary, 513 KB): a 512-thread workgroup (256 registers per lane)
// keeps NVR 16-byte vectors per thread in VGPRs and NVL more in LDS (NVL x 8 KiB), the latter
// loaded straight into LDS by buffer->LDS loads, so that HBM still sees one read and one write
// per element.  The row is cut into 64 runs of NV = NVR + NVL lines of 128 bytes; lanes
// 8 g .. 8 g + 7 of the workgroup own run g, lane c of them the 16-byte column c of each line,
// so a thread's vectors sit at immediate offsets 128 j from one base and every load instruction
// still reads whole lines.  Each thread reads back only the LDS vectors its own wave loaded
// (no barrier needed).
constexpr int kCELThreads = 512;
constexpr int kCELWaves = kCELThreads / kWave;
template <typename T, int NVR, int NVL>
__global__ void __launch_bounds__(kCELThreads) ce_rows_cached_lds(T* __restrict__ logits,
                                                                   const int64_t* __restrict__ targets,
                                                                   int64_t V, int64_t ld, int64_t ignore_index,
                                                                   float mu, CERowOut out) {
  constexpr int EPV = Vec16<T>::N;
  constexpr int NV = NVR + NVL;
  constexpr float kLog2e = 1.4426950408889634f;
  __shared__ float sm[kCELWaves], ss[kCELWaves];
  __shared__ __attribute__((aligned(1024))) char lv[NVL][kCELThreads * 16];
  const int64_t row = blockIdx.x;
  T* x = logits + row * ld;
  const int tid = threadIdx.x;
  const int64_t y = targets[row];
  const bool valid = (y != ignore_index) && (y >= 0) && (y < V);
  const int64_t row_bytes = ld * (int64_t)sizeof(T);
  const int g = tid >> 3, c = tid & 7;
  const uint32_t base = (uint32_t)(g * NV * 128 + c * 16);  // byte offset of vector 0
  const int64_t e0 = (int64_t)base / (int64_t)sizeof(T);       // its first element
  constexpr int64_t kStepE = 128 / (int64_t)sizeof(T);         // elements between vectors j, j + 1
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(x, row_bytes);
  const u32x4_t rw = make_rsrc_words(x, row_bytes);
  const float xy = Vec16<T>::elem(rs, (tid == 0 && valid) ? (uint32_t)(y * (int64_t)sizeof(T)) : 0xfffffff0u);
  // LDS part first (its loads are the oldest, so they land first), then the register part
  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lv[0]));
  const uint32_t wave_lds = lds0 + (uint32_t)(wave_id() * kWave * 16);
#pragma unroll
  for (int j = NVR; j < NV; ++j)
    dma16(rw, wave_lds + (uint32_t)((j - NVR) * kCELThreads * 16), base + (uint32_t)j * 128u);
  Vec16<T> buf[NVR];
#pragma unroll
  for (int j = NVR - 1; j >= 0; --j) buf[j].raw = load16(rs, base + (uint32_t)j * 128u);
  // elements of this thread's run that lie before V (32-bit; clamped): element e of vector j is
  // read as -inf at or past it (a select on each value read, so the cached vectors themselves
  // are never rewritten)
  const int64_t rem64 = V - e0;
  const int rem = (int)(rem64 < 0 ? 0 : (rem64 > NV * kStepE ? NV * kStepE : rem64));
  // (each pass takes its own opaque copy of rem, so the compiler cannot hoist one predicate per
  // element out of the passes and keep them all alive)
  int rem_p = rem;
  auto fresh_rem = [&]() {
    rem_p = rem;
    asm volatile("" : "+v"(rem_p));
  };
  auto val = [&](float f, int j, int e) { return (j * (int)kStepE + e < rem_p) ? f : -INFINITY; };
  auto lds_vec = [&](int j) {
    Vec16<T> v;
    v.raw = *reinterpret_cast<const uint4*>(&lv[j - NVR][tid * 16]);
    return v;
  };
  vm_wait<0>();

  float m = -INFINITY;
  fresh_rem();
#pragma unroll
  for (int j = NV - 1; j >= NVR; --j) {
    const Vec16<T> v = lds_vec(j);
#pragma unroll
    for (int e = 0; e < EPV; ++e) m = fmaxf(m, val(v.get(e), j, e));
  }
#pragma unroll
  for (int j = NVR - 1; j >= 0; --j)
#pragma unroll
    for (int e = 0; e < EPV; ++e) m = fmaxf(m, val(buf[j].get(e), j, e));
  float s = 0.f;
  const float ml = m * kLog2e;
  fresh_rem();
#pragma unroll
  for (int j = NV - 1; j >= NVR; --j) {
    const Vec16<T> v = lds_vec(j);
#pragma unroll
    for (int e = 0; e < EPV; ++e) s += __builtin_amdgcn_exp2f(fmaf(val(v.fresh(e), j, e), kLog2e, -ml));
  }
#pragma unroll
  for (int j = NVR - 1; j >= 0; --j)
#pragma unroll
    for (int e = 0; e < EPV; ++e) s += __builtin_amdgcn_exp2f(fmaf(val(buf[j].fresh(e), j, e), kLog2e, -ml));
  if (m == -INFINITY) s = 0.f;
  // workgroup (max, sum): waves, then the kCELWaves partials in a fixed order
  wave_ms(m, s);
  {
    const int w = tid / kWave, l = tid % kWave;
    if (l == 0) { sm[w] = m; ss[w] = s; }
    __syncthreads();
    m = -INFINITY;
    s = 0.f;
    for (int i = 0; i < kCELWaves; ++i) ms_merge(m, s, sm[i], ss[i]);
  }
  const float lse = m + __logf(s);
  const float scale = valid ? (1.f + 2.f * mu * lse) : 0.f;
  const float ll = lse * kLog2e;
  // the thread and vector holding column y: line L = byte / 128 is vector L % NV of run L / NV
  const int64_t yb = valid ? y * (int64_t)sizeof(T) : 0;
  const int64_t yl = yb / 128;
  const int ty = (int)(8 * (yl / NV) + (yb % 128) / 16), jy = (int)(yl % NV), ey = (int)((yb % 16) / sizeof(T));
  const bool owner = valid && ty == tid;
  auto emit = [&](int j, const Vec16<T>& v) {
    float d[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) d[e] = __builtin_amdgcn_exp2f(fmaf(val(v.fresh(e), j, e), kLog2e, -ll)) * scale;
#pragma unroll
    for (int e = 0; e < EPV; ++e) d[e] -= (owner && j == jy && e == ey) ? 1.f : 0.f;
    store16_nt(rs, base + (uint32_t)j * 128u, pack_out(d, T()));
  };
  fresh_rem();
#pragma unroll
  for (int j = 0; j < NVR; ++j) emit(j, buf[j]);
#pragma unroll
  for (int j = NVR; j < NV; ++j) emit(j, lds_vec(j));
  if (tid == 0) {
    out.ce[row] = valid ? (lse - xy) : 0.f;
    out.zsq[row] = valid ? lse * lse : 0.f;
    out.valid[row] = valid ? 1 : 0;
    if (out.lse != nullptr) out.lse[row] = lse;
  }
}

// Rows too long for the register cache, 16-byte aligned: two passes over global memory in
// 16-byte vectors (the second read usually hits the last-level cache); elements past V are
// masked to -inf and the padding columns are written as 0.
template <typename T>
__global__ void __launch_bounds__(kCEThreads) ce_rows_stream_vec(T* __restrict__ logits,
                                                                  const int64_t* __restrict__ targets,
                                                                  int64_t V, int64_t ld, int64_t ignore_index,
                                                                  float mu, CERowOut out) {
  constexpr int EPV = Vec16<T>::N;
  constexpr float kLog2e = 1.4426950408889634f;
  __shared__ float sm[kCEWaves], ss[kCEWaves];
  const int64_t row = blockIdx.x;
  T* x = logits + row * ld;
  const int tid = threadIdx.x;
  const int64_t y = targets[row];
  const bool valid = (y != ignore_index) && (y >= 0) && (y < V);
  const int64_t row_bytes = ld * (int64_t)sizeof(T);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(x, row_bytes);
  const int64_t nvec = (V + EPV - 1) / EPV;
  const float xy = Vec16<T>::elem(rs, (tid == 0 && valid) ? (uint32_t)(y * (int64_t)sizeof(T)) : 0xfffffff0u);
  float m = -INFINITY, s = 0.f;
  for (int64_t j = tid; j < nvec; j += kCEThreads) {
    Vec16<T> v;
    v.raw = load16(rs, (uint32_t)(j * 16));
    mask_tail(v, j * EPV, V);
    float vm = -INFINITY;
#pragma unroll
    for (int e = 0; e < EPV; ++e) vm = fmaxf(vm, v.get(e));
    if (vm > m) {
      s *= __builtin_amdgcn_exp2f((m - vm) * kLog2e);
      m = vm;
    }
    if (m != -INFINITY) {
      const float ml = m * kLog2e;
#pragma unroll
      for (int e = 0; e < EPV; ++e) s += __builtin_amdgcn_exp2f(fmaf(v.get(e), kLog2e, -ml));
    }
  }
  if (m == -INFINITY) s = 0.f;
  block_ms(m, s, sm, ss);
  const float lse = m + __logf(s);
  const float scale = valid ? (1.f + 2.f * mu * lse) : 0.f;
  const float ll = lse * kLog2e;
  const int64_t nvec_ld = ld / EPV;
  for (int64_t j = tid; j < nvec_ld; j += kCEThreads) {
    Vec16<T> v;
    v.raw = load16(rs, (uint32_t)(j * 16));
    mask_tail(v, j * EPV, V);
    float d[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      d[e] = __builtin_amdgcn_exp2f(fmaf(v.get(e), kLog2e, -ll)) * scale;
      if (valid && j * EPV + e == y) d[e] -= 1.f;
    }
    store16_nt(rs, (uint32_t)(j * 16), pack_out(d, T()));
  }
  if (tid == 0) {
    out.ce[row] = valid ? (lse - xy) : 0.f;
    out.zsq[row] = valid ? lse * lse : 0.f;
    out.valid[row] = valid ? 1 : 0;
    if (out.lse != nullptr) out.lse[row] = lse;
  }
}

// Any V: two passes over global memory, element by element (rows not 16-byte aligned).
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
    } else if (m != -INFINITY) {  // (-inf entries so far: e^-inf = 0, never -inf - -inf)
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
    if (out.lse != nullptr) out.lse[row] = lse;
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

// ---------------------------------------------------------------------------
// Per-row outputs and their gradients on a logits chunk (bf16, rows ld apart), for
// RL-style use ("Fused Linear Cross-Entropy: ...", Strategy 2 keeps each row's target
// log-probability and softmax entropy beside the LSE):
//   logprobs[t] = valid (z_y - LSE),  entropy[t] = LSE - E_p[z],
//   row_loss[t] = valid (LSE - z_y + mu LSE^2).
// With GRAD the row is overwritten with the dlogits of
//   sum_t gl_t row_loss_t + gp_t logprobs_t + ge_t entropy_t,
// which is p (alpha + beta z) - gamma onehot(y) with
//   alpha = valid (gl (1 + 2 mu LSE) - gp) + ge E_p[z],  beta = -ge,  gamma = valid (gl - gp)
// (d LSE / dz_v = p_v and d E_p[z] / dz_v = p_v (1 + z_v - E_p[z])).
// Two passes over the row in 16-byte vectors: (max, sum exp, sum exp * z) online, then the
// outputs (the second read usually hits the last-level cache).
// ---------------------------------------------------------------------------
struct RowsIO {
  float* lse;
  float* logprobs;
  float* entropy;
  float* row_loss;
  const float* gl;  // upstream gradient of row_loss, or NULL (0)
  const float* gp;  // of logprobs
  const float* ge;  // of entropy
};

// (max, sum exp(x - max), sum exp(x - max) x) merge; m = -inf is the identity.
__device__ __forceinline__ void mst_merge(float& m, float& s, float& t, float m2, float s2, float t2) {
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

template <bool GRAD>
__global__ void __launch_bounds__(kCEThreads) rows_stats_kernel(bf16_t* __restrict__ logits,
                                                                 const int64_t* __restrict__ targets,
                                                                 int64_t V, int64_t ld, int64_t ignore_index,
                                                                 float mu, RowsIO io) {
  typedef Vec16<bf16_t> VT;
  constexpr int EPV = VT::N;
  constexpr float kLog2e = 1.4426950408889634f;
  __shared__ float sm[kCEWaves], ss[kCEWaves], st[kCEWaves];
  const int64_t row = blockIdx.x;
  bf16_t* x = logits + row * ld;
  const int tid = threadIdx.x;
  const int64_t y = targets[row];
  const bool valid = (y != ignore_index) && (y >= 0) && (y < V);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(x, ld * 2);
  const int64_t nvec = (V + EPV - 1) / EPV;
  float m = -INFINITY, s = 0.f, t = 0.f;
  for (int64_t j = tid; j < nvec; j += kCEThreads) {
    VT v;
    v.raw = load16(rs, (uint32_t)(j * 16));
    mask_tail(v, j * EPV, V);
    float vm = -INFINITY;
#pragma unroll
    for (int e = 0; e < EPV; ++e) vm = fmaxf(vm, v.get(e));
    if (vm > m) {
      const float f = __builtin_amdgcn_exp2f((m - vm) * kLog2e);
      s *= f;
      t *= f;
      m = vm;
    }
    if (m != -INFINITY) {
      const float ml = m * kLog2e;
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float xe = v.get(e);
        const float pe = __builtin_amdgcn_exp2f(fmaf(xe, kLog2e, -ml));
        s += pe;
        t += pe != 0.f ? pe * xe : 0.f;
      }
    }
  }
  // block-wide merge (every thread ends with the row's values)
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off, kWave), s2 = __shfl_xor(s, off, kWave), t2 = __shfl_xor(t, off, kWave);
    mst_merge(m, s, t, m2, s2, t2);
  }
  const int w = tid / kWave;
  if (tid % kWave == 0) {
    sm[w] = m;
    ss[w] = s;
    st[w] = t;
  }
  __syncthreads();
  m = -INFINITY;
  s = 0.f;
  t = 0.f;
  for (int i = 0; i < kCEWaves; ++i) mst_merge(m, s, t, sm[i], ss[i], st[i]);
  const float lse = m + __logf(s);
  const float ez = t / s;
  const float zy = valid ? VT::elem(rs, (uint32_t)(y * 2)) : 0.f;
  if (tid == 0) {
    if (io.lse) io.lse[row] = lse;
    if (io.logprobs) io.logprobs[row] = valid ? zy - lse : 0.f;
    if (io.entropy) io.entropy[row] = lse - ez;
    if (io.row_loss) io.row_loss[row] = valid ? lse - zy + mu * lse * lse : 0.f;
  }
  if constexpr (GRAD) {
    const float gl = io.gl ? io.gl[row] : 0.f;
    const float gp = io.gp ? io.gp[row] : 0.f;
    const float ge = io.ge ? io.ge[row] : 0.f;
    const float alpha = (valid ? gl * (1.f + 2.f * mu * lse) - gp : 0.f) + ge * ez;
    const float beta = -ge;
    const float gamma = valid ? gl - gp : 0.f;
    const float ll = lse * kLog2e;
    const int64_t nvec_ld = ld / EPV;
    for (int64_t j = tid; j < nvec_ld; j += kCEThreads) {
      VT v;
      v.raw = load16(rs, (uint32_t)(j * 16));
      mask_tail(v, j * EPV, V);
      float d[EPV];
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float xe = v.get(e);
        const float pe = __builtin_amdgcn_exp2f(fmaf(xe, kLog2e, -ll));
        d[e] = pe != 0.f ? pe * fmaf(beta, xe, alpha) : 0.f;
        if (valid && j * EPV + e == y) d[e] -= gamma;
      }
      store16(rs, (uint32_t)(j * 16), pack_out(d, bf16_t()));
    }
  }
}

hipError_t launch_rows_stats(void* logits, const int64_t* targets, int64_t B, int64_t V, int64_t ld,
                             int64_t ignore_index, float mu, float* lse, float* logprobs, float* entropy,
                             float* row_loss, const float* gl, const float* gp, const float* ge, bool grad,
                             hipStream_t st) {
  if (B <= 0) return hipSuccess;
  if ((ld % 8) != 0 || (reinterpret_cast<uintptr_t>(logits) % 16) != 0) return hipErrorInvalidValue;
  RowsIO io{lse, logprobs, entropy, row_loss, gl, gp, ge};
  if (grad)
    hipLaunchKernelGGL(rows_stats_kernel<true>, dim3((unsigned)B), dim3(kCEThreads), 0, st,
                       static_cast<bf16_t*>(logits), targets, V, ld, ignore_index, mu, io);
  else
    hipLaunchKernelGGL(rows_stats_kernel<false>, dim3((unsigned)B), dim3(kCEThreads), 0, st,
                       static_cast<bf16_t*>(logits), targets, V, ld, ignore_index, mu, io);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_rows(T* logits, const int64_t* targets, int64_t B, int64_t V, int64_t ld,
                              int64_t ignore_index, float mu, CERowOut out, bool resident, hipStream_t st) {
  constexpr int EPV = 16 / (int)sizeof(T);
  const bool vec_ok = ((ld * (int64_t)sizeof(T)) % 16) == 0 &&
                      (reinterpret_cast<uintptr_t>(logits) % 16) == 0;
  const int64_t nvec = (V + EPV - 1) / EPV;
  const int64_t per = (nvec + kCEThreads - 1) / kCEThreads;
  dim3 grid((unsigned)B), block(kCEThreads);
  if (vec_ok && per <= 16) {
    if (per <= 1) hipLaunchKernelGGL((ce_rows_cached<T, 1>), grid, block, 0, st, logits, targets, V, ld, ignore_index, mu, out);
    else if (per <= 2) hipLaunchKernelGGL((ce_rows_cached<T, 2>), grid, block, 0, st, logits, targets, V, ld, ignore_index, mu, out);
    else if (per <= 4) hipLaunchKernelGGL((ce_rows_cached<T, 4>), grid, block, 0, st, logits, targets, V, ld, ignore_index, mu, out);
    else if (per <= 8) hipLaunchKernelGGL((ce_rows_cached<T, 8>), grid, block, 0, st, logits, targets, V, ld, ignore_index, mu, out);
    else hipLaunchKernelGGL((ce_rows_cached<T, 16>), grid, block, 0, st, logits, targets, V, ld, ignore_index, mu, out);
  } else if (vec_ok && !resident && ld * (int64_t)sizeof(T) <= 64 * 64 * 128) {
    // rows up to 512 KiB: 64 runs of 64 lines, 45 of them per thread in registers, 19 in LDS
    hipLaunchKernelGGL((ce_rows_cached_lds<T, 45, 19>), grid, dim3(kCELThreads), 0, st, logits, targets, V, ld,
                       ignore_index, mu, out);
  } else if (vec_ok) {
    hipLaunchKernelGGL((ce_rows_stream_vec<T>), grid, block, 0, st, logits, targets, V, ld, ignore_index, mu, out);
  } else {
    if (ld != V) return hipErrorInvalidValue;  // padded rows are always 16-byte aligned
    hipLaunchKernelGGL((ce_rows_stream<T>), grid, block, 0, st, logits, targets, V, ignore_index, mu, out);
  }
  return hipGetLastError();
}

hipError_t launch_ce_inplace(void* logits, int dtype, const int64_t* targets, int64_t B, int64_t V,
                             int64_t ld, int64_t ignore_index, float mu, float* ce_sum, float* z_sum,
                             int64_t* n_valid, float* lse_rows, void* workspace, bool resident, hipStream_t st) {
  CERowOut out;
  out.lse = lse_rows;
  char* ws = static_cast<char*>(workspace);
  const size_t a = ws_align((size_t)B * 4);
  out.ce = reinterpret_cast<float*>(ws);
  out.zsq = reinterpret_cast<float*>(ws + a);
  out.valid = reinterpret_cast<int32_t*>(ws + 2 * a);
  hipError_t e = hipSuccess;
  if (B > 0) {
    if (dtype == kCeBf16)
      e = launch_rows<bf16_t>(static_cast<bf16_t*>(logits), targets, B, V, ld, ignore_index, mu, out, resident, st);
    else if (dtype == kCeF16)
      e = launch_rows<f16_t>(static_cast<f16_t*>(logits), targets, B, V, ld, ignore_index, mu, out, resident, st);
    else
      e = launch_rows<float>(static_cast<float*>(logits), targets, B, V, ld, ignore_index, mu, out, resident, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(ce_reduce, dim3(1), dim3(kCEThreads), 0, st, out.ce, out.zsq, out.valid, B,
                     mu != 0.f ? 1 : 0, ce_sum, z_sum, n_valid);
  return hipGetLastError();
}

size_t ce_workspace_bytes(int64_t B) { return 3 * ws_align((size_t)(B > 0 ? B : 1) * 4); }

}  // namespace lce
