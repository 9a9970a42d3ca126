// Stored-operand GEMM on gfx950 for the gradient products of stored dlogits blocks
// ("Fused Linear Cross-Entropy: The Math, the Memory Wall, and Two Ways Around It", "From
// dlogits to grad_input and grad_W": grad_input = dlogits . W, grad_W = dlogits^T . hidden).
//
//   C[m][n] = sum_k A[m][k] B[k][n]      A: [M][lda] bf16, K contiguous (a dlogits block, or
//                                         its transpose)
//                                         B: [K][ldb] bf16, N contiguous (W or hidden rows)
// with fp32 accumulation, over K split into ranges of ksplit: every (256 x 256 tile, range)
// is one workgroup, which either writes its fp32 partial sums (optionally adding to the
// values already there) or, with a single range, the scaled result c * C in the output dtype.
//
// Workgroup: 8 waves (two per SIMD) in a 2 x 4 grid, each 128 x 64 of the tile on
// v_mfma_f32_32x32x16_bf16.  K is staged 64 at a time into a double buffer by buffer->LDS
// loads (8 per wave and stage):
//  * A stage: 256 rows x 128 bytes, each row's 16-byte chunks XOR-swizzled by the row, read
//    as 16-byte fragments (conflict free).
//  * B stage: eight planes of 32 columns; plane p holds the 64 K-rows as rows of 64 bytes
//    (sub-block j = K-rows 16 j .. 16 j + 15 in 1 KiB).  The B operand of a 32 x 32 x 16 step
//    (K-rows 8 h .. 8 h + 7 of column c in lane 32 h + c) is two ds_read_b64_tr_b16 of that
//    layout: a 16-lane group reads a 4-row x 32-byte block and receives it transposed.
// The next stage's loads are issued right after the barrier that frees their buffer (after the
// first step's fragment reads), so they overlap the current stage's MFMAs.
// Gradient filtering ("Cut Cross Entropy visualized", "Gradient Filtering"): with per-tile
// stage flags (SgArgs::kflags), a tile runs only its flagged K stages, in order, through the
// same load pipeline; a running-sum tile with none leaves the sum as it is.  With a row map
// (SgArgs::row_map) the plain output's rows go where the map says (vocabulary sorting).
#include "lce_common.h"
#include "lce_launch.h"

namespace lce {

constexpr int kSgThreads = 512;
constexpr int kSgTile = 256;

__device__ __forceinline__ int sg_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ bf16x8_t sg_tr_pair(const char* p0, const char* p1) {
  const i16x4_t a = lds_read_tr16(reinterpret_cast<const bf16_t*>(p0));
  const i16x4_t b = lds_read_tr16(reinterpret_cast<const bf16_t*>(p1));
  return bf16x8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// ATRANS: A is given transposed, At [K][lda] with M contiguous (the dlogits chunk of the
// token-chunked composition, [tokens][vocabulary], as the grad_W operand G^T): its stage is
// loaded and read like B's (planes of 32 M-columns, transposed reads).
constexpr int kSgStage = kSgTile * 128;  // 32 KiB: A (256 rows x 64 K) or B (64 K x 256 columns)

// Running sum over launches: s = hi + q 2^(e - 142), hi the bf16 nearest to s (exponent field
// e) and q an int8, the remainder s - hi (at most half of hi's unit in the last place, 2^(e -
// 134)) in steps of 2^-8 of that unit, so s keeps about 16 significant bits.  Sums below 2^-111
// keep hi only.
__device__ __forceinline__ float rem_step(uint32_t hi) {  // 2^(e - 142)
  const uint32_t e = (hi >> 7) & 0xffu;
  return e >= 16 ? __uint_as_float((e - 15u) << 23) : 0.f;
}
__device__ __forceinline__ float rem_inv(uint32_t hi) {  // 2^(142 - e)
  const uint32_t e = (hi >> 7) & 0xffu;
  return e >= 16 ? __uint_as_float((269u - e) << 23) : 0.f;
}
__device__ __forceinline__ uint32_t rem_code(float s, uint32_t hi) {  // q as a byte
  const float q = fminf(fmaxf(rintf((s - bf2f((bf16_t)hi)) * rem_inv(hi)), -128.f), 127.f);
  return (uint32_t)(int32_t)q & 0xffu;
}

__device__ __forceinline__ uint32_t sg_tiles(const SgArgs& p) {
  return (uint32_t)((p.M + kSgTile - 1) / kSgTile) * (uint32_t)((p.N + kSgTile - 1) / kSgTile) * (uint32_t)p.nsplit;
}

// One workgroup's tile `id` of problem p (ids: columns fastest, then rows, then K ranges, so
// that concurrent workgroups share A rows and B ranges), staged through sA / sB.
template <bool ATRANS>
__device__ __forceinline__ void sgemm_tile(const SgArgs& p, uint32_t id, char (*sA)[kSgStage], char (*sB)[kSgStage]) {
  constexpr int STAGE = kSgStage;
  const int tid = threadIdx.x, w = wave_id(), lane = tid & 63;
  const int wm = w >> 2, wn = w & 3;
  const uint32_t ntm = (uint32_t)((p.M + kSgTile - 1) / kSgTile), ntn = (uint32_t)((p.N + kSgTile - 1) / kSgTile);
  const uint32_t nt = id % ntn, rest = id / ntn;
  const uint32_t mt = rest % ntm, split = rest / ntm;
  const int64_t m0 = (int64_t)mt * kSgTile, n0 = (int64_t)nt * kSgTile;
  const int64_t kb = (int64_t)split * p.ksplit;
  const int64_t ke = (kb + p.ksplit) < p.K ? (kb + p.ksplit) : p.K;
  const int nk = ke > kb ? (int)((ke - kb + 63) / 64) : 0;

  // ---- the K stages to run, in increasing order (wave-uniform: every wave walks the same
  // flags).  Gradient filtering: the row tile's flags of global stages [s0, s1) are read a page
  // of 1024 at a time (16 per lane, one 16-byte load; bytes outside the range masked), then
  // taken a 16-stage group at a time from the lane that holds it.
  const bool filt = p.kflags != nullptr;
  const int s0 = (int)(kb / 64), s1 = s0 + nk;
  const uint8_t* krow = filt ? p.kflags + (int64_t)mt * p.ldkf : nullptr;
  int seq = 0;                       // (no filtering) the next stage
  int pg = s0 & ~15;                 // first stage of the loaded page
  u32x4_t fl = {0u, 0u, 0u, 0u};     // lane l: flags of stages pg + 16 l .. + 15
  uint64_t groups = 0;               // groups of the page with a flag left to take
  uint32_t steps = 0;                // stages of the current group left to run
  int gbase = 0;
  auto load_page = [&]() {
    const int first = pg + 16 * lane;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (first < s1 && first + 16 > s0) v = *reinterpret_cast<const u32x4_t*>(krow + first);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = first + 4 * i;  // bytes b .. b + 3 of dword i: keep those in [s0, s1)
      uint32_t m = 0xffffffffu;
      const int lo = s0 - b, hi = s1 - b;
      if (lo > 0) m = lo >= 4 ? 0u : m << (8 * lo);
      if (hi < 4) m = hi <= 0 ? 0u : m & (0xffffffffu >> (8 * (4 - hi)));
      v[i] &= m;
    }
    fl = v;
    groups = __builtin_amdgcn_ballot_w64((v[0] | v[1] | v[2] | v[3]) != 0u);
  };
  auto next_stage = [&]() -> int {  // stage index relative to s0, or -1 when done
    if (!filt) return seq < nk ? seq++ : -1;
    for (;;) {
      if (steps != 0) {
        const int b = __builtin_ctz(steps);
        steps &= steps - 1;
        return gbase + b - s0;
      }
      if (groups == 0) {
        pg += 1024;
        if (pg >= s1) return -1;
        load_page();
        continue;
      }
      const int g = __builtin_ctzll(groups);
      groups &= groups - 1;
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // flag bytes (0 or 1) of lane g -> 4 bits per dword
        const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)fl[i], g);
        m |= ((d & 1u) | ((d >> 7) & 2u) | ((d >> 14) & 4u) | ((d >> 21) & 8u)) << (4 * i);
      }
      steps = m;
      gbase = pg + 16 * g;
    }
  };
  if (filt && nk > 0) load_page();

  // ---- loads of one stage: A rows 8 (4 w + j) + l / 8, physical chunk l % 8 holding logical
  // chunk (l % 8) ^ swz(row); B plane w, sub-block j: K-row 16 j + l / 4, columns
  // 32 w + 8 (l % 4) .. + 7.  Elements past M, N or the K range read as zero.
  const int64_t mrows = (p.M - m0) < kSgTile ? (p.M - m0) : kSgTile;
  const u32x4_t ra = ATRANS ? make_rsrc_words(p.A + kb * p.lda, (p.K - kb) * p.lda * 2)
                            : make_rsrc_words(p.A + m0 * p.lda, mrows * p.lda * 2);
  const u32x4_t rb = make_rsrc_words(p.B + kb * p.ldb, (p.K - kb) * p.ldb * 2);
  int a_k[4];
  uint32_t a_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 8 * (4 * w + j) + (lane >> 3);
    a_k[j] = 8 * ((lane & 7) ^ sg_swz(row));
    a_off[j] = (uint32_t)(row * p.lda * 2 + (kb + a_k[j]) * 2);
  }
  const int64_t bcol = n0 + 32 * w + 8 * (lane & 3);
  const bool bcol_ok = bcol < p.N;
  const uint32_t b_off0 = (uint32_t)((lane >> 2) * p.ldb * 2 + bcol * 2);
  // (ATRANS) A plane w: M-columns m0 + 32 w + 8 (l % 4) .. + 7 of K-rows 16 j + l / 4
  const int64_t acol = m0 + 32 * w + 8 * (lane & 3);
  const bool acol_ok = acol < p.M;
  const uint32_t at_off0 = (uint32_t)((lane >> 2) * p.lda * 2 + acol * 2);
  const uint32_t la = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)sA[0]));
  const uint32_t lb = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)sB[0]));
  const int64_t klen = ke - kb;
  auto dma = [&](int ks, int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (ATRANS) {
        const int kr = 64 * ks + 16 * j + (lane >> 2);
        const bool ok = acol_ok && kr < klen;
        dma16(ra, la + (uint32_t)(buf * STAGE + 1024 * (4 * w + j)),
              ok ? at_off0 + (uint32_t)((64 * ks + 16 * j) * p.lda * 2) : 0x80000000u);
      } else {
        const bool ok = 64 * ks + a_k[j] < klen;
        dma16(ra, la + (uint32_t)(buf * STAGE + 1024 * (4 * w + j)), ok ? a_off[j] + 128u * ks : 0x80000000u);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int kr = 64 * ks + 16 * j + (lane >> 2);
      const bool ok = bcol_ok && kr < klen;
      dma16(rb, lb + (uint32_t)(buf * STAGE + 1024 * (4 * w + j)),
            ok ? b_off0 + (uint32_t)((64 * ks + 16 * j) * p.ldb * 2) : 0x80000000u);
    }
  };

  // ---- fragment addresses
  const int fs = sg_swz(lane & 31);
  const int g = lane >> 4, r4 = (lane >> 2) & 3, cc = lane & 3;
  int o_b[2];
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) o_b[rd] = 64 * (8 * (g >> 1) + 4 * rd + r4) + 32 * (g & 1) + 8 * cc;

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  int buf = 0;
  int cur = next_stage();
  const bool any = cur >= 0;
  // A running sum to which this tile adds nothing stays as it is.
  if (!any && p.hilo == 2) return;
  if (any) dma(cur, 0);
  while (cur >= 0) {
    vm_wait<0>();     // this wave's loads of stage cur have landed
    const int nxt = next_stage();
    __syncthreads();  // every wave's have; nobody reads the other buffer any more
    const char* a_base = ATRANS ? sA[buf] + (4 * wm) * 4096 : sA[buf] + (wm * 128 + (lane & 31)) * 128;
    const char* b_base = sB[buf] + (2 * wn) * 4096;
    Frag<bf16_t> fa[2][4], fb[2][2];
    auto rd = [&](int kk, int slot) {
      const int off = ((2 * kk + (lane >> 5)) ^ fs) << 4;
#pragma unroll
      for (int vb = 0; vb < 4; ++vb) {
        if constexpr (ATRANS) {
          const char* pa = a_base + vb * 4096 + kk * 1024;
          fa[slot][vb].v = sg_tr_pair(pa + o_b[0], pa + o_b[1]);
        } else {
          lds_frag_ptr(fa[slot][vb], a_base + vb * 32 * 128 + off);
        }
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const char* pb = b_base + nb * 4096 + kk * 1024;
        fb[slot][nb].v = sg_tr_pair(pb + o_b[0], pb + o_b[1]);
      }
    };
    rd(0, 0);
    // the next stage's loads after the first step's fragment reads, so that their latency
    // overlaps the load issue
    if (nxt >= 0) dma(nxt, buf ^ 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk + 1 < 4) rd(kk + 1, (kk + 1) & 1);
#pragma unroll
      for (int vb = 0; vb < 4; ++vb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) mfma_32x32x16(fa[kk & 1][vb], fb[kk & 1][nb], acc[vb][nb]);
    }
    // the first step's fragment reads (8, or 12 with A read transposed), then each step's eight
    // MFMAs interleaved with the next step's reads (two after each of the first four MFMAs when
    // there are 12)
    __builtin_amdgcn_sched_group_barrier(0x100, ATRANS ? 12 : 8, 0);
#pragma unroll
    for (int kk = 0; kk < 3; ++kk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, ATRANS ? 2 : 1, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    buf ^= 1;
    cur = nxt;
  }

  // ---- epilogue: lane l holds column n0 + 64 wn + 32 nb + l % 32 of rows
  // m0 + 128 wm + 32 vb + 8 (r / 4) + 4 (l / 32) + r % 4
  const int64_t ncol = n0 + 64 * wn + (lane & 31);
  const int mrow0 = 128 * wm + 4 * (lane >> 5);
  // Rows of whole 8-element groups: each 32-row block of the wave's results goes through its
  // own LDS region (waves 0-3 in the A buffers, 4-7 in the B buffers; rows 72 floats apart, so
  // the two row groups of a write fall on disjoint banks), and each lane then handles 8
  // consecutive columns of a row with 16-byte global accesses (8x fewer than one per element).
  const bool vec = p.N % 8 == 0 && (p.C != nullptr ? p.ldc % 8 == 0
                                                     : p.ldo % 8 == 0 && (p.hilo == 0 || p.ldlo % 8 == 0));
  if (vec) {
    constexpr int kPitch = 72;
    __syncthreads();  // every wave has read its last stage: the buffers are free
    float* reg = reinterpret_cast<float*>(w < 4 ? &sA[0][0] : &sB[0][0]) + (w & 3) * 32 * kPitch;
    const long long nvalid = *p.n_valid;
    const float cs = p.C != nullptr ? 1.f : (p.mean ? 1.f / (float)(nvalid > 1 ? nvalid : 1) : 1.f);
    const int rl = lane >> 3, cl = 8 * (lane & 7);  // this lane: rows 8 i + rl, columns cl .. cl + 7
    const int64_t n8 = n0 + 64 * wn + cl;
    const bool cok = n8 < p.N;
    const int es = p.C != nullptr ? 4 : (p.out_f32 ? 4 : 2);
    const int64_t ld = p.C != nullptr ? p.ldc : p.ldo;
    char* const base = p.C != nullptr ? reinterpret_cast<char*>(p.C + (int64_t)split * p.split_stride + m0 * p.ldc)
                                      : static_cast<char*>(p.out) + m0 * p.ldo * es;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(base, mrows * ld * es);
    const __amdgpu_buffer_rsrc_t rl8 =
        make_rsrc(p.hilo != 0 ? reinterpret_cast<char*>(p.lo + m0 * p.ldlo) : base, p.hilo != 0 ? mrows * p.ldlo : 0);
    if (p.hilo >= 2) {
      // the running sum's middle and last blocks (read, add, write): each 32-row block's hi and
      // remainder loads are issued two blocks ahead, so that their round trips overlap (all four
      // ahead would not fit the registers)
      typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
      u32x4_t hv[2][4];
      u32x2_t lv[2][4];
      auto issue = [&](int vb, int slot) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = 128 * wm + 32 * vb + 8 * i + rl;
          const uint32_t o = cok ? (uint32_t)((m * ld + n8) * es) : 0x80000000u;
          const uint32_t ol = cok ? (uint32_t)(m * p.ldlo + n8) : 0x80000000u;
          hv[slot][i] = __builtin_amdgcn_raw_buffer_load_b128(ro, (int)o, 0, 0);
          lv[slot][i] = __builtin_amdgcn_raw_buffer_load_b64(rl8, (int)ol, 0, 0);
        }
      };
      issue(0, 0);
      issue(1, 1);
#pragma unroll
      for (int vb = 0; vb < 4; ++vb) {
        const int slot = vb & 1;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            reg[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * kPitch + 32 * nb + (lane & 31)] = acc[vb][nb][r];
        float v[4][8];
        uint32_t off[4], offl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 a = *reinterpret_cast<const float4*>(reg + (8 * i + rl) * kPitch + cl);
          const float4 b = *reinterpret_cast<const float4*>(reg + (8 * i + rl) * kPitch + cl + 4);
          v[i][0] = a.x; v[i][1] = a.y; v[i][2] = a.z; v[i][3] = a.w;
          v[i][4] = b.x; v[i][5] = b.y; v[i][6] = b.z; v[i][7] = b.w;
          const int m = 128 * wm + 32 * vb + 8 * i + rl;
          off[i] = cok ? (uint32_t)((m * ld + n8) * es) : 0x80000000u;
          offl[i] = cok ? (uint32_t)(m * p.ldlo + n8) : 0x80000000u;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t h16 = (e & 1) ? (hv[slot][i][e >> 1] >> 16) : (hv[slot][i][e >> 1] & 0xffffu);
            const int32_t q = (int32_t)(int8_t)((lv[slot][i][e >> 2] >> (8 * (e & 3))) & 0xffu);
            v[i][e] += bf2f((bf16_t)h16) + (float)q * rem_step(h16);
          }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x4_t ho;
          uint32_t lo[2] = {0u, 0u};
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            if (p.hilo == 3) {
              ho[e >> 1] = (uint32_t)f2bf(cs * v[i][e]) | ((uint32_t)f2bf(cs * v[i][e + 1]) << 16);
            } else {
              const uint32_t h0 = f2bf(v[i][e]), h1 = f2bf(v[i][e + 1]);
              ho[e >> 1] = h0 | (h1 << 16);
              lo[e >> 2] |= (rem_code(v[i][e], h0) | (rem_code(v[i][e + 1], h1) << 8)) << (8 * (e & 2));
            }
          }
          __builtin_amdgcn_raw_buffer_store_b128(ho, ro, (int)off[i], 0, 0);
          if (p.hilo != 3) __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{lo[0], lo[1]}, rl8, (int)offl[i], 0, 0);
        }
        if (vb + 2 < 4) issue(vb + 2, slot);
        asm volatile("" ::: "memory");  // (the region is rewritten for the next block)
      }
    } else {
#pragma unroll
      for (int vb = 0; vb < 4; ++vb) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            reg[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * kPitch + 32 * nb + (lane & 31)] = acc[vb][nb][r];
        float v[4][8];
        uint32_t off[4], offl[4];
        int64_t orow[4];  // (row_map) output row, or -1 past the tile's rows or columns
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 a = *reinterpret_cast<const float4*>(reg + (8 * i + rl) * kPitch + cl);
          const float4 b = *reinterpret_cast<const float4*>(reg + (8 * i + rl) * kPitch + cl + 4);
          v[i][0] = a.x; v[i][1] = a.y; v[i][2] = a.z; v[i][3] = a.w;
          v[i][4] = b.x; v[i][5] = b.y; v[i][6] = b.z; v[i][7] = b.w;
          const int m = 128 * wm + 32 * vb + 8 * i + rl;
          off[i] = cok ? (uint32_t)((m * ld + n8) * es) : 0x80000000u;
          offl[i] = cok ? (uint32_t)(m * p.ldlo + n8) : 0x80000000u;
          orow[i] = p.row_map != nullptr && cok && m < mrows ? (int64_t)p.row_map[m0 + m] : -1;
        }
        if (p.C != nullptr) {  // fp32 partial sums, written or added
          if (p.accumulate) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float4 a = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(ro, (int)off[i], 0, 0));
              const float4 b =
                  __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(ro, (int)(off[i] + 16), 0, 0));
              v[i][0] += a.x; v[i][1] += a.y; v[i][2] += a.z; v[i][3] += a.w;
              v[i][4] += b.x; v[i][5] += b.y; v[i][6] += b.z; v[i][7] += b.w;
            }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, make_float4(v[i][0], v[i][1], v[i][2], v[i][3])),
                                                   ro, (int)off[i], 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, make_float4(v[i][4], v[i][5], v[i][6], v[i][7])),
                                                   ro, (int)(off[i] + 16), 0, 0);
          }
        } else if (p.hilo != 0) {  // the running sum's first block: hi + q (rem_step above), written
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            u32x4_t ho;
            uint32_t lo[2] = {0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
              const uint32_t h0 = f2bf(v[i][e]), h1 = f2bf(v[i][e + 1]);
              ho[e >> 1] = h0 | (h1 << 16);
              lo[e >> 2] |= (rem_code(v[i][e], h0) | (rem_code(v[i][e + 1], h1) << 8)) << (8 * (e & 2));
            }
            __builtin_amdgcn_raw_buffer_store_b128(ho, ro, (int)off[i], 0, 0);
            typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
            __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{lo[0], lo[1]}, rl8, (int)offl[i], 0, 0);
          }
        } else if (p.row_map != nullptr) {  // rows through the map (64-bit addresses)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (orow[i] < 0) continue;
            if (p.out_f32) {
              float4* d = reinterpret_cast<float4*>(static_cast<float*>(p.out) + orow[i] * p.ldo + n8);
              d[0] = make_float4(cs * v[i][0], cs * v[i][1], cs * v[i][2], cs * v[i][3]);
              d[1] = make_float4(cs * v[i][4], cs * v[i][5], cs * v[i][6], cs * v[i][7]);
            } else {
              u32x4_t ho;
#pragma unroll
              for (int e = 0; e < 8; e += 2)
                ho[e >> 1] = (uint32_t)f2bf(cs * v[i][e]) | ((uint32_t)f2bf(cs * v[i][e + 1]) << 16);
              *reinterpret_cast<u32x4_t*>(static_cast<bf16_t*>(p.out) + orow[i] * p.ldo + n8) = ho;
            }
          }
        } else if (p.out_f32) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4_t, make_float4(cs * v[i][0], cs * v[i][1], cs * v[i][2], cs * v[i][3])), ro,
                (int)off[i], 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(
                __builtin_bit_cast(u32x4_t, make_float4(cs * v[i][4], cs * v[i][5], cs * v[i][6], cs * v[i][7])), ro,
                (int)(off[i] + 16), 0, 0);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            u32x4_t ho;
#pragma unroll
            for (int e = 0; e < 8; e += 2)
              ho[e >> 1] = (uint32_t)f2bf(cs * v[i][e]) | ((uint32_t)f2bf(cs * v[i][e + 1]) << 16);
            __builtin_amdgcn_raw_buffer_store_b128(ho, ro, (int)off[i], 0, 0);
          }
        }
        asm volatile("" ::: "memory");  // (the region is rewritten for the next block)
      }
    }
  } else if (p.C != nullptr) {
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(p.C + (int64_t)split * p.split_stride + m0 * p.ldc, mrows * p.ldc * 4);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const bool cok = ncol + 32 * nb < p.N;
#pragma unroll
      for (int vb = 0; vb < 4; ++vb) {
        uint32_t off[16];
        float old[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = mrow0 + 32 * vb + 8 * (r >> 2) + (r & 3);
          off[r] = cok ? (uint32_t)((m * p.ldc + ncol + 32 * nb) * 4) : 0x80000000u;
          old[r] = 0.f;
        }
        if (p.accumulate) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            old[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rc, (int)off[r], 0, 0));
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, acc[vb][nb][r] + old[r]), rc,
                                                (int)off[r], 0, 0);
      }
    }
  } else {
    const long long nvalid = *p.n_valid;
    const float cs = p.mean ? 1.f / (float)(nvalid > 1 ? nvalid : 1) : 1.f;
    const int es = p.out_f32 ? 4 : 2;
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(static_cast<char*>(p.out) + m0 * p.ldo * es, mrows * p.ldo * es);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const bool cok = ncol + 32 * nb < p.N;
#pragma unroll
      for (int vb = 0; vb < 4; ++vb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = mrow0 + 32 * vb + 8 * (r >> 2) + (r & 3);
          const uint32_t off = cok ? (uint32_t)((m * p.ldo + ncol + 32 * nb) * es) : 0x80000000u;
          const float v = cs * acc[vb][nb][r];
          if (p.out_f32)
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), ro, (int)off, 0, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f2bf(v), ro, (int)off, 0, 0);
        }
    }
  }
  vm_wait<0>();
}

// Consecutive logical tile ids stay on one XCD (xcd_remap).
template <bool ATRANS>
__global__ void __launch_bounds__(kSgThreads, 1) sgemm_kernel(SgArgs p) {
  __shared__ __attribute__((aligned(1024))) char sA[2][kSgStage];
  __shared__ __attribute__((aligned(1024))) char sB[2][kSgStage];
  const uint32_t total = sg_tiles(p);
  const uint32_t id = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)xcd_remap(blockIdx.x, total));
  sgemm_tile<ATRANS>(p, id, sA, sB);
}

// Two products in one grid, the tiles of p0 (A K-contiguous) first, then those of p1 (A given
// transposed): a launch whose products are each short of a whole number of workgroup rounds
// over the device fills the rounds with both.  Each product's tiles are spread over all XCDs
// (XCD-contiguous within the product); p0's part of the grid is padded to a multiple of 8 with
// workgroups that do nothing, so that both parts start on XCD 0.
__global__ void __launch_bounds__(kSgThreads, 1) sgemm_pair_kernel(SgArgs p0, SgArgs p1) {
  __shared__ __attribute__((aligned(1024))) char sA[2][kSgStage];
  __shared__ __attribute__((aligned(1024))) char sB[2][kSgStage];
  const uint32_t t0 = sg_tiles(p0), t0p = (t0 + 7) / 8 * 8;
  const uint32_t b = blockIdx.x;
  if (b < t0p) {
    const uint32_t id = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)xcd_remap(b, t0p));
    if (id < t0) sgemm_tile<false>(p0, id, sA, sB);
  } else {
    const uint32_t id = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)xcd_remap(b - t0p, sg_tiles(p1)));
    sgemm_tile<true>(p1, id, sA, sB);
  }
}

// the running-sum output: bf16 out, one K-range, rows of whole 8-element groups (the staged
// epilogue), a remainder buffer (32-bit offsets per tile)
static bool hilo_ok(const SgArgs& a) {
  if (a.hilo == 0) return true;
  return a.hilo >= 1 && a.hilo <= 3 && a.C == nullptr && !a.out_f32 && a.nsplit == 1 && a.lo != nullptr &&
         a.N % 8 == 0 && a.ldo % 8 == 0 && a.ldlo % 8 == 0 && kSgTile * a.ldlo < 0x80000000ll;
}

static int64_t sg_total(const SgArgs& a) {
  const int64_t ntm = (a.M + kSgTile - 1) / kSgTile, ntn = (a.N + kSgTile - 1) / kSgTile;
  return ntm * ntn * a.nsplit;
}

// Shapes the kernel takes: K-ranges of whole 64-element stages, and every descriptor the kernel
// forms spanning less than 2^31 bytes (the offset 2^31 it uses for masked elements is then out
// of range).  ATRANS: At [K][lda] with rows of whole 8-element vectors.
static bool sg_args_ok(const SgArgs& a, bool atrans) {
  if (a.nsplit < 1 || sg_total(a) > 0x7fffffff || a.ksplit % 64 != 0 || a.ksplit <= 0) return false;
  // the mapped rows take the staged epilogue's plain output; flag rows of whole 16-byte loads
  if (a.row_map != nullptr && (a.C != nullptr || a.hilo != 0 || a.nsplit != 1 || a.N % 8 != 0 || a.ldo % 8 != 0))
    return false;
  if (a.kflags != nullptr &&
      (a.ldkf % 16 != 0 || reinterpret_cast<uintptr_t>(a.kflags) % 16 != 0 || a.ldkf < (a.K + 63) / 64))
    return false;
  if (atrans) {
    if (a.K * a.lda * 2 >= 0x80000000ll) return false;
    if (a.M % 8 != 0 && a.lda < (a.M + 7) / 8 * 8) return false;
  } else if (kSgTile * a.lda * 2 >= 0x80000000ll) {
    return false;
  }
  if (a.K * a.ldb * 2 >= 0x80000000ll) return false;
  if (a.C != nullptr && kSgTile * a.ldc * 4 >= 0x80000000ll) return false;
  if (a.C == nullptr && (a.out == nullptr || kSgTile * a.ldo * 4 >= 0x80000000ll)) return false;
  return hilo_ok(a);
}

hipError_t launch_sgemm(const SgArgs& a, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (!sg_args_ok(a, false)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sgemm_kernel<false>, dim3((unsigned)sg_total(a)), dim3(kSgThreads), 0, st, a);
  return hipGetLastError();
}

// The same with A given transposed: At [K][lda], M contiguous.
hipError_t launch_sgemm_at(const SgArgs& a, hipStream_t st) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  if (!sg_args_ok(a, true)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sgemm_kernel<true>, dim3((unsigned)sg_total(a)), dim3(kSgThreads), 0, st, a);
  return hipGetLastError();
}

// Column sums of a dlogits chunk G [rows][ld] (bf16) into an fp32 running sum over chunks:
// acc[v] = (first ? 0 : acc[v]) + sum_t G[t][v]; on the last chunk out[v] = c * acc[v] (bf16).
__global__ void __launch_bounds__(256) colsum_kernel(const bf16_t* __restrict__ g, int64_t ld, int64_t rows,
                                                     int64_t cols, float* __restrict__ acc, int first, int last,
                                                     bf16_t* __restrict__ out, const int64_t* __restrict__ n_valid,
                                                     int mean) {
  const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (v >= cols) return;
  float s = first ? 0.f : acc[v];
  for (int64_t t = 0; t < rows; ++t) s += bf2f(g[t * ld + v]);
  acc[v] = s;
  if (last) {
    const long long nv = *n_valid;
    const float cs = mean ? 1.f / (float)(nv > 1 ? nv : 1) : 1.f;
    out[v] = f2bf(cs * s);
  }
}

hipError_t launch_colsum(const bf16_t* g, int64_t ld, int64_t rows, int64_t cols, float* acc, bool first, bool last,
                         bf16_t* out, const int64_t* n_valid, bool mean, hipStream_t st) {
  if (cols <= 0) return hipSuccess;
  hipLaunchKernelGGL(colsum_kernel, dim3((unsigned)((cols + 255) / 256)), dim3(256), 0, st, g, ld, rows, cols, acc,
                     first ? 1 : 0, last ? 1 : 0, out, n_valid, mean ? 1 : 0);
  return hipGetLastError();
}

// out = c * sum over nsplit partial buffers ([nsplit][n] fp32, `stride` floats apart), in bf16
// or fp32; c = 1 / max(n_valid, 1) if mean, else 1.  n a multiple of 4.  With row_map, element
// i (row i / width) goes to row row_map[i / width] of out.
__global__ void __launch_bounds__(256) sg_reduce_kernel(const float* __restrict__ part, int nsplit, int64_t n,
                                                        int64_t stride, void* __restrict__ out, int out_f32,
                                                        const int64_t* __restrict__ n_valid, int mean,
                                                        const int32_t* __restrict__ row_map, int64_t width) {
  const long long nvalid = *n_valid;
  const float cs = mean ? 1.f / (float)(nvalid > 1 ? nvalid : 1) : 1.f;
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
    int64_t o = i;
    if (row_map != nullptr) {
      const int64_t r = i / width;
      o = (int64_t)row_map[r] * width + (i - r * width);
    }
    if (out_f32)
      *reinterpret_cast<float4*>(static_cast<float*>(out) + o) = make_float4(cs * a.x, cs * a.y, cs * a.z, cs * a.w);
    else
      *reinterpret_cast<uint2*>(static_cast<bf16_t*>(out) + o) =
          make_uint2(pack_bf2(cs * a.x, cs * a.y), pack_bf2(cs * a.z, cs * a.w));
  }
}

hipError_t launch_sg_reduce(const float* part, int nsplit, int64_t n, int64_t stride, void* out, bool out_f32,
                            const int64_t* n_valid, bool mean, hipStream_t st, const int32_t* row_map,
                            int64_t width) {
  if (n <= 0) return hipSuccess;
  if (n % 4 != 0) return hipErrorInvalidValue;
  if (row_map != nullptr && (width <= 0 || width % 4 != 0 || n % width != 0)) return hipErrorInvalidValue;
  int64_t blocks = (n / 4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(sg_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, st, part, nsplit, n, stride, out,
                     out_f32 ? 1 : 0, n_valid, mean ? 1 : 0, row_map, width);
  return hipGetLastError();
}

// grad_b of a block of vocabulary rows from the transposed dlogits kernel's partial sums (one
// row of fp32 sums per token tile): out[i] = c * sum_s part[s * ld + i], in order of s.
__global__ void __launch_bounds__(256) part_sum_kernel(const float* __restrict__ part, int64_t ld, int64_t nparts,
                                                       int64_t n, bf16_t* __restrict__ out,
                                                       const int64_t* __restrict__ n_valid, int mean,
                                                       const int32_t* __restrict__ row_map) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int64_t k = 0; k < nparts; ++k) s += part[k * ld + i];
  const long long nv = *n_valid;
  const float cs = mean ? 1.f / (float)(nv > 1 ? nv : 1) : 1.f;
  out[row_map != nullptr ? (int64_t)row_map[i] : i] = f2bf(cs * s);
}

hipError_t launch_part_sum(const float* part, int64_t ld, int64_t nparts, int64_t n, bf16_t* out,
                           const int64_t* n_valid, bool mean, hipStream_t st, const int32_t* row_map) {
  if (n <= 0) return hipSuccess;
  if (ld < n || nparts < 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(part_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, ld, nparts, n, out,
                     n_valid, mean ? 1 : 0, row_map);
  return hipGetLastError();
}

// Two products in one launch: p0 as launch_sgemm takes it, p1 as launch_sgemm_at.
hipError_t launch_sgemm_pair(const SgArgs& p0, const SgArgs& p1, hipStream_t st) {
  if (p0.M <= 0 || p0.N <= 0) return launch_sgemm_at(p1, st);
  if (p1.M <= 0 || p1.N <= 0) return launch_sgemm(p0, st);
  if (!sg_args_ok(p0, false) || !sg_args_ok(p1, true)) return hipErrorInvalidValue;
  const int64_t total = (sg_total(p0) + 7) / 8 * 8 + sg_total(p1);
  if (total > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(sgemm_pair_kernel, dim3((unsigned)total), dim3(kSgThreads), 0, st, p0, p1);
  return hipGetLastError();
}

}  // namespace lce
