// Device-side building blocks shared by the gfx950 kernels: storage types, bf16
// rounding, MFMA fragment types and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {

typedef uint16_t bf16_t;  // raw bfloat16 bits

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Round to nearest bfloat16, ties to even (finite inputs; NaN stays NaN).
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (bf16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// Two floats to packed bfloat16 (round to nearest even) with gfx950's v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_hw));
}

// Element type traits: storage type and conversions.
template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float to_f(bf16_t v) { return bf2f(v); }
  __device__ __forceinline__ static bf16_t from_f(float v) { return f2bf(v); }
};
typedef _Float16 f16_t;  // IEEE half (standalone cross-entropy only)
template <> struct Elem<f16_t> {
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float to_f(f16_t v) { return (float)v; }
  __device__ __forceinline__ static f16_t from_f(float v) { return (f16_t)v; }  // nearest even
};
template <> struct Elem<float> {
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static float to_f(float v) { return v; }
  __device__ __forceinline__ static float from_f(float v) { return v; }
};

// ---------------------------------------------------------------------------
// MFMA 32x32 tiles with K = 16 per step.
//
// Operand fragment: each lane holds 8 consecutive K values of one row (A) or one
// column (B): lane l covers row/col (l % 32) and K values 8*(l/32) .. 8*(l/32)+7.
// For bf16 that is one v_mfma_f32_32x32x16_bf16; for fp32 it is eight
// v_mfma_f32_32x32x2_f32 where sub-step s pairs K values s and 8+s (the same
// K permutation on both operands, so the sum over K is unchanged).
// Accumulator layout (both): lane l holds column l % 32 and rows
//   8*(r/4) + 4*(l/32) + (r%4) for r = 0..15.
// ---------------------------------------------------------------------------
template <typename T> struct Frag;
template <> struct Frag<bf16_t> {
  bf16x8_t v;
};
template <> struct Frag<float> {
  float v[8];
};

__device__ __forceinline__ void mfma_32x32x16(const Frag<bf16_t>& a, const Frag<bf16_t>& b, f32x16_t& c) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, c, 0, 0, 0);
}
// The same bf16 MFMA with its accumulator in VGPRs.  The builtin puts every MFMA
// accumulator in AGPRs once a kernel uses them; a kernel whose long-lived accumulator fills
// the AGPR file uses these for a short-lived second one so the two never compete.
// Hazards the compiler cannot see through the asm are covered here: two wait states
// before each MFMA (a VALU write of an operand just before it), and mfma_v_drain() after
// the last one of a chain, before anything but another MFMA reads the accumulator.
__device__ __forceinline__ void mfma_32x32x16_v0(const Frag<bf16_t>& a, const Frag<bf16_t>& b, f32x16_t& c) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a.v), "v"(b.v));
}
__device__ __forceinline__ void mfma_32x32x16_v(const Frag<bf16_t>& a, const Frag<bf16_t>& b, f32x16_t& c) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a.v), "v"(b.v));
}
__device__ __forceinline__ void mfma_v_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

__device__ __forceinline__ void mfma_32x32x16(const Frag<float>& a, const Frag<float>& b, f32x16_t& c) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.v[s], b.v[s], c, 0, 0, 0);
}

// Row index (within a 32x32 accumulator tile) of accumulator register r in lane l.
__device__ __forceinline__ int acc_row(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Load 8 consecutive elements (16 B for bf16, 32 B for fp32); ptr must be 16-byte aligned.
__device__ __forceinline__ void load8(Frag<bf16_t>& f, const bf16_t* p) {
  f.v = *reinterpret_cast<const bf16x8_t*>(p);
}
__device__ __forceinline__ void load8(Frag<float>& f, const float* p) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
__device__ __forceinline__ void lds_frag_ptr(Frag<bf16_t>& f, const char* p) {
  f.v = *reinterpret_cast<const bf16x8_t*>(p);
}
__device__ __forceinline__ void zero8(Frag<bf16_t>& f) { f.v = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0}; }
__device__ __forceinline__ void zero8(Frag<float>& f) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = 0.f;
}

// ---------------------------------------------------------------------------
// Raw buffer loads: a scalar descriptor (base, size in bytes) plus a 32-bit per-lane byte
// offset.  Reads at or past `bytes` return zero, which is how tile edges are masked.
// Descriptor word 3 = 0x00020000 (gfx9 family: 32-bit data format, no swizzle).
// ---------------------------------------------------------------------------
// The arguments must be wave-uniform; readfirstlane keeps the descriptor in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xffffffffll ? 0xffffffffu : (uint32_t)bytes);
  n = (uint32_t)__builtin_amdgcn_readfirstlane((int)n);
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  void* b = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(b, (short)0, (int)n, 0x00020000);
}

// Loads into LDS issued from inline assembly.  The compiler models a buffer-to-LDS load as a
// store to LDS of unknown extent and would then wait for every one still in flight before
// any later LDS read, which would undo the prefetch; here the kernel itself tracks which
// loads must have landed (vm_wait) before it reads a buffer.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
// Buffer descriptor words (base, size in bytes; same format as make_rsrc), wave-uniform.
__device__ __forceinline__ u32x4_t make_rsrc_words(const void* base, int64_t bytes) {
  uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xffffffffll ? 0xffffffffu : (uint32_t)bytes);
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4_t r;
  r.x = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)) & 0xffffu;
  r.z = (uint32_t)__builtin_amdgcn_readfirstlane((int)n);
  r.w = 0x00020000u;
  return r;
}
// 16 bytes per lane from rsrc + voff to LDS address lds + 16 * lane.
__device__ __forceinline__ void dma16(const u32x4_t& rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voff),
               "s"(rsrc)
               : "memory", "m0");
}
// Same, ordered after the LDS read that produced `dep` has completed (the compiler waits for
// the registers an asm statement reads): used to refill a buffer region right after its
// last read.
// 4 bytes per lane from rsrc + voff to LDS address lds + 4 * lane.
__device__ __forceinline__ void dma4(const u32x4_t& rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
__device__ __forceinline__ void dma16_after(const u32x4_t& rsrc, uint32_t lds, uint32_t voff, const bf16x8_t& dep) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voff),
               "s"(rsrc), "v"(dep)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void lgkm_wait0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Workgroups are dealt round-robin to the 8 XCDs; this gives each XCD a contiguous range of
// the logical tile order (0 .. n-1), so workgroups that share operand tiles share an L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t id, int64_t n) {
  const int64_t x = id % 8, q = id / 8, Q = n / 8, r = n % 8;
  return (x < r) ? x * (Q + 1) + q : r * (Q + 1) + (x - r) * Q + q;
}

// Index of the calling wave within its workgroup, as a scalar (wave-uniform) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / 64)); }
__device__ __forceinline__ void load8(Frag<bf16_t>& f, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  f.v = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ void load8(Frag<float>& f, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  const float4 a = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
  const float4 b = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + 16), 0, 0));
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// Stores at or past the descriptor's size are dropped.
__device__ __forceinline__ void store16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, 0);
}
// The same with the non-temporal cache policy, for data a streaming kernel writes once and
// no later kernel of the same call reads soon.
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ void store16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, kCachePolicyNT);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane (4*r + c) supplies the address of
// row r, columns 4c..4c+3 of a 4 x 16 block of 16-bit values; lane i of the group receives
// column i, rows 0..3.
__device__ __forceinline__ i16x4_t lds_read_tr16(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
}

// ---------------------------------------------------------------------------
// Wave-level reductions (64 lanes).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
__device__ __forceinline__ long long wave_sum_ll(long long v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Combine two (max, sum-of-exp(x - max)) pairs.  A pair with m = -inf and s = 0 is the
// identity; no -inf - -inf is ever formed.
__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2) {
  if (m2 > m) {
    s = s * __expf(m - m2) + s2;
    m = m2;
  } else if (m2 != -INFINITY) {
    s = s + s2 * __expf(m2 - m);
  }
}

__device__ __forceinline__ void wave_ms(float& m, float& s) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    float m2 = __shfl_xor(m, off, kWave);
    float s2 = __shfl_xor(s, off, kWave);
    ms_merge(m, s, m2, s2);
  }
}

}  // namespace lce
