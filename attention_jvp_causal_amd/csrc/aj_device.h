// Device-side building blocks shared by the gfx950 kernels of this library:
// vector types, the direct buffer -> LDS DMA of 16-byte chunks into swizzled
// tiles, explicit vmcnt waits, and the cross-lane reductions over the lanes
// that share one row of an MFMA accumulator.  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "aj_tiles.h"

namespace aj {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int BM = kTileM;   // query rows per workgroup
constexpr int BN = kTileN;   // keys per streamed tile
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t x) { return __builtin_bit_cast(bf16x8_t, x); }

// 16-byte chunk c of tile row r is stored at position c ^ swz(r).  For the
// q16 shape at D = 128 (16 chunks per 256-byte row) one swizzle serves both
// read patterns of a tile:
//  * ds_read_b128 of chunk c0 + g from rows j = 0..15 (lane 16g + j), served
//    in four groups of lanes l with equal l % 4: conflict-free when
//    swz(r) >> 2 takes four different values over r = k, k+4, k+8, k+12;
//  * ds_read_b64_tr_b16 of chunk pairs from rows 4g + j/4 (8 rows per half
//    wave): conflict-free when swz(r) >> 1 differs over each 8 rows.
// swz(r) = 4 ((r >> 2) ^ 2 ((r >> 1) & 1)) + 2 (r & 1) meets both.  These lane
// groupings were inferred from the LDS bank-conflict counter: it reads 0 for
// this swizzle in the kernels, and about 4 stalled cycles per b128 read for
// 2 (r % 8) + (r / 8) % 2, which meets only the second condition.  Built for
// D = 128 (the JVP and the 16-key dK / dV kernel).  At D = 64, where a row is
// 128 bytes and two rows share a bank line, the rows k, k+4, k+8, k+12 of one
// read group always fall in one half line (a 2-way conflict on every b128
// read); the d = 64 kernels use the 32-row shape and swz_q32 instead.
template <int D>
__device__ __forceinline__ int swz_q16(int r) {
  static_assert(D == 128, "the 16-row tile layout is built for head_dim 128");
  return ((((r >> 2) ^ (((r >> 1) & 1) << 1)) & 3) << 2) | ((r & 1) << 1);
}
template <int D>
__device__ __forceinline__ int swz_q32(int r) {
  static_assert(D == 64 || D == 128, "head_dim");
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kRsrcWord3 = 0x00020000;  // gfx9 raw buffer resource: 32-bit data, no swizzle

// One direct buffer -> LDS load of 16 bytes per lane: lane l's chunk lands at
// LDS byte address lds_base + 16 l.  Written as inline asm so that the
// compiler does not track it: the kernel waits for these loads itself
// (wait_vmcnt) right before the barrier that publishes a buffer.  The
// compiler cannot tell the two buffers apart and would wait for the next
// tile's loads before the first read of the current one.
// The instruction has no register results; it only writes LDS.  m0 is set
// here and used by nothing else in these kernels (checked by a build test).
__device__ __forceinline__ void lds_dma_16(uint32_t lds_base, uint32_t voffset, i32x4_t rsrc) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_base), "v"(voffset), "s"(rsrc)
      : "memory", "m0");
}

__device__ __forceinline__ i32x4_t make_rsrc(const void* base, int nbytes) {
  const uint64_t b = (uint64_t)base;
  i32x4_t rs;
  rs.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  rs.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32) & 0xffff);  // stride 0
  rs.z = __builtin_amdgcn_readfirstlane(nbytes);
  rs.w = kRsrcWord3;
  return rs;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}

// Per-lane byte offsets (inside one key tile of one tensor) of the 16-byte
// chunks this lane moves.  Wave instruction i fills 1 KB block blk = wave +
// NW*i of the tile: lane l writes LDS chunk blk*64 + l, i.e. row r = chunk /
// CH at swizzled position p, so it fetches logical chunk p ^ swz(r) of row r.
template <int NW, int D>
struct TileLoadPlan {
  static constexpr int CH = D / 8;                   // 16-byte chunks per row
  static constexpr int NI = (BN * CH) / (64 * NW);   // wave instructions per tensor
  uint32_t voff[NI];
  __device__ __forceinline__ TileLoadPlan(int64_t sl, int wave, int lane, int (*swz)(int)) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int ci = (wave + NW * i) * 64 + lane;
      const int r = ci / CH, p = ci % CH;
      voff[i] = uint32_t(r * sl * 2 + ((p ^ swz(r)) << 4));
    }
  }
};

// A value every lane of the wave holds alike, moved to a scalar register.  The
// tile-map walk (task, entry offsets, entries) is wave-uniform; held in scalar
// registers it lets the compiler do the key-tile DMA's address arithmetic on
// the scalar unit, instead of in vector registers followed by readfirstlane
// and the wait states that a scalar read of a vector-written value needs.
__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ Entry load_entry(const Entry* p) {
  const Entry e = *p;
  return Entry{wave_uniform(e.kt0), wave_uniform(e.kt1), wave_uniform(e.pidx), wave_uniform(e.flags)};
}

// Workgroup index -> (task rank, flattened head b * H + h).  The B * H heads
// are taken in groups of G: all workgroups of one group come before those of
// the next, so only G heads' keys are being streamed at any time, and inside a
// group consecutive workgroups cycle through its heads, task rank outer.  The
// dispatcher deals workgroups to the eight XCDs in turn, so with G dividing 8
// each XCD, and its L2, serves one head of the group.  G = B * H is the plain
// rank-major order.
struct TaskCoord {
  int rank, bh;
};
__device__ __forceinline__ TaskCoord task_coord(int idx, int n_tasks, int BH, int G) {
  const int per = G * n_tasks;
  const int grp = idx / per;
  const int rem = idx - grp * per;
  const int gsz = min(G, BH - grp * G);
  const int rank = rem / gsz;
  return {rank, grp * G + (rem - rank * gsz)};
}

// LDS addresses below are byte addresses in the workgroup's LDS: the
// kernels take the address of their LDS struct once (lds_addr) and add the
// struct's constant member offsets, so that with the wave index and the tile
// index in scalar registers the DMA addresses are scalar arithmetic.

// DMA of rows [row0, row0 + BN) of two [L, D] tensors into the two tiles
// starting at LDS byte address lds_buf (rows past L read as zero).
template <int NW, int D>
__device__ __forceinline__ void issue_pair_loads(uint32_t lds_buf, const TileLoadPlan<NW, D>& plan,
                                                 const uint16_t* s0, const uint16_t* s1, int64_t sl, int row0, int L,
                                                 int wave) {
  const int nrec = int((int64_t)min(L - row0, BN) * sl * 2);
  const i32x4_t r0 = make_rsrc(s0 + (int64_t)row0 * sl, nrec);
  const i32x4_t r1 = make_rsrc(s1 + (int64_t)row0 * sl, nrec);
#pragma unroll
  for (int i = 0; i < TileLoadPlan<NW, D>::NI; ++i)
    lds_dma_16(lds_buf + (wave + NW * i) * 1024, plan.voff[i], r0);
#pragma unroll
  for (int i = 0; i < TileLoadPlan<NW, D>::NI; ++i)
    lds_dma_16(lds_buf + BN * D * 2 + (wave + NW * i) * 1024, plan.voff[i], r1);
}

// Wave 0 loads the 128 per-row key bitmasks (1 KB) of partial tile pidx to
// LDS byte address lds_bits.
__device__ __forceinline__ void issue_bits_load(uint32_t lds_bits, const uint64_t* bits, int pidx, int lane) {
  lds_dma_16(lds_bits, uint32_t(lane) * 16u, make_rsrc(bits + (int64_t)pidx * BM, BM * 8));
}
// The same for a partial tile of a 256-row task: wave w < 2 loads rows
// 128 w .. 128 w + 127 (1 KB) to LDS byte address lds_bits + 1024 w.
__device__ __forceinline__ void issue_bits_load_wide(uint32_t lds_bits, const uint64_t* bits, int pidx, int wave,
                                                     int lane) {
  lds_dma_16(lds_bits + wave * 1024, uint32_t(lane) * 16u,
             make_rsrc(bits + (int64_t)pidx * kTileMWide + wave * BM, BM * 8));
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  // no load of DMA'd data may be scheduled above the wait
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// max over lanes l and l^32 (the two halves of one q32 query row) without
// the LDS pipe: v_permlane32_swap exchanges the upper half of one operand with
// the lower half of the other.
__device__ __forceinline__ float row_max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// max / sum over the four lanes l, l^16, l^32, l^48 of one q16 query row
__device__ __forceinline__ float row4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Lazy rescale of the online softmax: a row's reference max moves only when
// its max grows by more than 2^8 (log2 units).
constexpr float kLazyRescaleLog2 = 8.0f;

// Rewrites, in place, the 16-byte chunks of NTEN key tiles (V, then tV) that this
// wave's lanes brought in by DMA (issue_tile_loads: wave instruction i of lane
// l fills chunk (wave + NW i) * 64 + l of each tensor tile) from bf16 to fp16.
// Every bf16 value of magnitude in [2^-14, 65504] is an fp16 value, so the
// conversion is exact there; smaller magnitudes keep fp16's subnormal
// resolution (2^-24) and larger ones saturate to 65504 (round toward zero).
// Called after the wave's own DMA has landed (vmcnt 0) and before the barrier
// that publishes the buffer, so no other wave reads these chunks meanwhile.
// One 32-bit pair of bf16 values (low half first) as a pair of fp16 values.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t x) {
  const float lo = __uint_as_float(x << 16), hi = __uint_as_float(x & 0xffff0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

template <int NW, int D, int NTEN>
__device__ __forceinline__ void bf16_chunks_to_f16(uint16_t* t0, uint16_t* t1, int wave, int lane) {
  constexpr int NI = TileLoadPlan<NW, D>::NI;
#pragma unroll
  for (int i = 0; i < NTEN * NI; ++i) {
    uint16_t* p = (i < NI ? t0 : t1) + (wave + NW * (i % NI)) * 512 + 8 * lane;
    const u32x4_t x = *(const u32x4_t*)p;
    u32x4_t y;
#pragma unroll
    for (int w = 0; w < 4; ++w) y[w] = bf16x2_to_f16x2(x[w]);
    *(u32x4_t*)p = y;
  }
}

// Key-tile buffers of the bf16 kernels: NT = 4 tensors (K, tK, V, tV) for the
// JVP, NT = 2 (K, V) for the primal forward, whose smaller footprint lets two
// workgroups share a CU.
template <int D, int NT, int ROWS = BM>
struct Bf16Lds {
  static constexpr int TILE = BN * D;  // elements per tensor tile
  uint16_t t[2][NT][TILE];             // [buffer][tensor]
  uint64_t bits[2][ROWS];              // per-row key bitmask of a partial tile (ROWS query rows)
  // LDS slot of tensor t in {0: K, 1: tK, 2: V, 3: tV}
  static constexpr __device__ int slot(int t) { return NT == 4 ? t : t / 2; }
  // byte offsets of t[b][0] and bits[b] from the start of the struct
  static constexpr __device__ uint32_t t_off(int b) { return uint32_t(b) * NT * TILE * 2; }
  static constexpr __device__ uint32_t bits_off(int b) { return 2u * NT * TILE * 2 + uint32_t(b) * ROWS * 8; }
};
// Issues the DMA of key tile [key0, key0 + BN) of K and V, and of tK and tV
// when TANG, into one LDS buffer.  Returns immediately; completion is tracked
// by vmcnt.  The buffer resource ends at row L, so rows past the end read as
// zero.
// lds_buf: LDS byte address of the buffer's first tensor tile; tensor slot s
// starts BN * D * 2 * s bytes further on.
template <int NW, int D, bool TANG, int NT>
__device__ __forceinline__ void issue_tile_loads(uint32_t lds_buf, const TileLoadPlan<NW, D>& plan,
                                                 const uint16_t* const src[4], int64_t sl, int key0, int L,
                                                 int wave) {
  const int nrec = int((int64_t)min(L - key0, BN) * sl * 2);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (!TANG && (t & 1)) continue;  // tK, tV
    const i32x4_t rs = make_rsrc(src[t] + (int64_t)key0 * sl, nrec);
    const uint32_t tile = lds_buf + uint32_t(NT == 4 ? t : t / 2) * BN * D * 2;
#pragma unroll
    for (int i = 0; i < TileLoadPlan<NW, D>::NI; ++i) lds_dma_16(tile + (wave + NW * i) * 1024, plan.voff[i], rs);
  }
}

}  // namespace aj
