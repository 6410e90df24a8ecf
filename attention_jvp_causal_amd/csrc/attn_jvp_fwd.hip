// Custom-mask attention JVP forward for gfx950 (MI355X).
//
// "Causal-rCM", App. B: one online-softmax pass computes the primal output of
// masked attention (Eq. 42) and its tangent (Eq. 44, evaluated as Eq. 45),
// streaming only the admissible key tiles of the mask; the same tile schedule
// serves the scores and their tangents.
//
// Work decomposition.  A workgroup (4 waves, 256 lanes) owns one 128-row query
// tile of one (batch, head); wave w owns query rows 32w..32w+31 of that tile.
// Keys stream in tiles of 64 through LDS.  Per key tile and wave:
//   S^T  = K Q^T             (keys x queries, MFMA 32x32x16 bf16, fp32 acc)
//   tS^T = tK Q^T + K tQ^T   (one accumulator chain)
// Computing the transposed scores puts one query row in each lane (lanes l and
// l+32 share a row and split its keys), so the softmax statistics are per lane
// and the accumulator registers feed the next MFMA as its B operand without any
// data movement:
//   O~^T += V^T P~^T        (A + B)^T += V^T (P~ . tS)^T + tV^T P~^T
// V and tV are read from LDS with transpose reads.
//
// Online softmax (fp32, per row): running max m, denominator l, and the JVP
// accumulators A = sum p~ ts v, B = sum p~ tv, mu = sum p~ ts share one rescale
// factor with O~.  Only A + B enters the result, so A and B are accumulated
// in one register set.  Finally O = O~/l and tO = (A + B - mu O)/l (Eq. 45).
// Rescaling is lazy: the reference max only moves when a row's max grows by
// more than 2^8, which is exact in real arithmetic (all terms of a row share
// the reference) and bounds p~ by 256.
// The bf16 MFMA operands p~ and p~.ts are rounded once; l and mu are summed
// from the same rounded values, so the cancellation in A - mu O is exact for
// the rounded operands.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "aj_internal.h"
#include "aj_launch.h"

namespace aj {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int BM = kTileM;   // query rows per workgroup
constexpr int BN = kTileN;   // keys per streamed tile
constexpr int NWAVES = 4;
constexpr int NTHREADS = 64 * NWAVES;
constexpr float kLazyRescaleLog2 = 8.0f;  // rescale when a row max grows by > 2^8
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t x) { return __builtin_bit_cast(bf16x8_t, x); }

// ---------------------------------------------------------------------------
// bf16 inputs
// ---------------------------------------------------------------------------

// LDS holds two buffers of {K, tK, V, tV} key tiles, each [BN][D] bf16 with
// unpadded rows.  The 16-byte chunks of row r are stored XOR-swizzled:
// logical chunk c sits at position c ^ swz(r), swz(r) = 2*(r%4) + (r/4)%2.
// This makes both read patterns bank-conflict free: ds_read_b128 of one chunk
// from 8 consecutive rows (K operands), and the transpose reads of V, which
// take two adjacent chunks from 4 consecutive rows.
template <int D>
struct Bf16Lds {
  static constexpr int TILE = BN * D;  // elements per tensor tile
  uint16_t t[2][4][TILE];              // [buffer][K, tK, V, tV]
  uint64_t bits[2][BM];                // per-row key bitmask of a partial tile
};

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kRsrcWord3 = 0x00020000;  // gfx9 raw buffer resource: 32-bit data, no swizzle

// Per-lane byte offsets (inside one key tile of one tensor) of the 16-byte
// chunks this lane moves with direct buffer -> LDS loads.  Wave instruction
// i fills 1 KB block blk = wave + 4i of the tile: lane l writes LDS chunk
// blk*64 + l, i.e. row r = chunk / CH at swizzled position p, so it fetches
// logical chunk p ^ swz(r) of row r.
template <int D>
struct TileLoadPlan {
  static constexpr int CH = D / 8;                       // 16-byte chunks per row
  static constexpr int NI = (BN * CH) / (64 * NWAVES);   // wave instructions per tensor
  uint32_t voff[NI];
  __device__ __forceinline__ TileLoadPlan(int64_t sl, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int ci = (wave + NWAVES * i) * 64 + lane;
      const int r = ci / CH, p = ci % CH;
      voff[i] = uint32_t(r * sl * 2 + ((p ^ swz(r)) << 4));
    }
  }
};

// One direct buffer -> LDS load of 16 bytes per lane: lane l's chunk lands at
// LDS byte address lds_base + 16 l.  Written as inline asm so that the compiler
// does not track it: the kernel waits for these loads itself (wait_vmcnt)
// right before the barrier that publishes the buffer, instead of the
// compiler's conservative wait for every load in flight into any buffer.
// The instruction has no register results; it only writes LDS.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void lds_dma_16(uint32_t lds_base, uint32_t voffset, i32x4_t rsrc) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_base), "v"(voffset), "s"(rsrc)
      : "memory", "m0");
}

// Issues the loads of key tile [key0, key0 + BN) of the four tensors into one
// LDS buffer (dst = its K, tK, V, tV tiles).  Returns immediately; completion
// is tracked by vmcnt.  The buffer resource starts at row key0 and ends at row
// L, so rows past the end read as zero.
template <int D>
__device__ __forceinline__ void issue_tile_loads(uint16_t (*dst)[BN * D], const TileLoadPlan<D>& plan,
                                                 const uint16_t* const src[4], int64_t sl, int key0, int L,
                                                 int wave) {
  const int nrec = int((int64_t)(L - key0) * sl * 2);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const uint64_t base = (uint64_t)(src[t] + (int64_t)key0 * sl);
    i32x4_t rs;
    rs.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)base);
    rs.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32) & 0xffff);  // stride 0
    rs.z = __builtin_amdgcn_readfirstlane(nrec);
    rs.w = kRsrcWord3;
#pragma unroll
    for (int i = 0; i < TileLoadPlan<D>::NI; ++i) {
      const uint32_t lds = __builtin_amdgcn_readfirstlane(
          (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(dst[t] + (wave + NWAVES * i) * 512));
      lds_dma_16(lds, plan.voff[i], rs);
    }
  }
}

// Wave 0 loads the 128 per-row key bitmasks (1 KB) of partial tile pidx into
// LDS: one 16-byte chunk (two rows) per lane.
__device__ __forceinline__ void issue_bits_load(uint64_t* dst, const uint64_t* bits, int pidx, int lane) {
  const uint64_t base = (uint64_t)(bits + (int64_t)pidx * BM);
  i32x4_t rs;
  rs.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)base);
  rs.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32) & 0xffff);
  rs.z = BM * 8;
  rs.w = kRsrcWord3;
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)dst);
  lds_dma_16(lds, uint32_t(lane) * 16u, rs);
}

template <int D>
constexpr int loads_per_tile() {
  return 4 * (BN * (D / 8)) / (64 * NWAVES);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

template <int D, bool OUT_F32>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS), amdgpu_waves_per_eu(1, 1)))
void attn_jvp_fwd_bf16_kernel(FwdArgs a) {
  constexpr int NKK = D / 16;  // MFMA k-steps over d for the score products
  constexpr int NDB = D / 32;  // 32-row blocks of d for the value products
  constexpr int CH = D / 8;
  constexpr int NLOADS = loads_per_tile<D>();
  __shared__ __attribute__((aligned(1024))) Bf16Lds<D> s;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int BH = a.B * a.H;
  const int rank = blockIdx.x / BH, bh = blockIdx.x - rank * BH;
  const int bb = bh / a.H, hh = bh - bb * a.H;
  const int qt = a.tasks[rank];
  const int L = a.L;
  const int64_t in_off = bb * a.isb + hh * a.ish;
  const uint16_t* __restrict__ Qg = (const uint16_t*)a.q + in_off;
  const uint16_t* __restrict__ tQg = (const uint16_t*)a.tq + in_off;
  const uint16_t* const src[4] = {(const uint16_t*)a.k + in_off, (const uint16_t*)a.tk + in_off,
                                  (const uint16_t*)a.v + in_off, (const uint16_t*)a.tv + in_off};
  const int q_row = qt * BM + wave * 32 + l32;

  // first key tile in flight before the prologue
  const TileLoadPlan<D> plan(a.isl, wave, lane);
  const int e0 = a.qt_off[qt], e1 = a.qt_off[qt + 1];
  int e = e0, kt = 0;
  Entry en = {0, 0, -1, 0};
  if (e < e1) {
    en = a.entries[e];
    kt = en.kt0;
    issue_tile_loads<D>(s.t[0], plan, src, a.isl, kt * BN, L, wave);
    if (en.pidx >= 0 && wave == 0) issue_bits_load(s.bits[0], a.bits, en.pidx, lane);
  }

  // Q and tQ of this lane's query row, as B operands: k-step kk holds
  // d = 16kk + 8hi .. 16kk + 8hi + 7.
  bf16x8_t Qr[NKK], tQr[NKK];
  {
    const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int64_t off = q_row * a.isl + kk * 16 + 8 * hi;
      Qr[kk] = as_bf16x8(q_row < L ? *(const u32x4_t*)(Qg + off) : zero);
      tQr[kk] = as_bf16x8(q_row < L ? *(const u32x4_t*)(tQg + off) : zero);
    }
  }
  // Q, tQ and the first key tile have landed; nothing the compiler tracks is
  // in flight inside the loop below.
  wait_vmcnt<0>();

  f32x16_t Oacc[NDB], ABacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) Oacc[db][r] = ABacc[db][r] = 0.f;
  float m_run = -INFINITY;            // reference max (log2 units, scale folded in)
  float l_part = 0.f, mu_part = 0.f;  // this lane's half of the row sums
  const float sl2 = a.scale_log2, c = a.scale;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  // Per-lane LDS offsets (elements) that do not depend on the tile; the rest
  // of every read offset is a compile-time constant.
  // K operand of 32-key block kb, k-step kk: row kb*32 + l32, logical chunk
  // 2kk + hi.  swz(kb*32 + l32) == swz(l32), and chunk 2kk + hi differs from
  // 2(kk%4) + hi only in bit 3, which the swizzle never touches.
  int koff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) koff[q] = l32 * D + (((2 * q + hi) ^ swz(l32)) << 3);
  // V^T operand (transpose read): within each 16-lane group g, lane j names
  // key 4hi + j/4 (+8 for the second read) and d = 32db + 16(g%2) + 4(j%4);
  // logical chunk 4db + c0 with c0 = d/8 % 4, swizzle of the row is swz(vrow0).
  const int g = lane >> 4, j = lane & 15;
  const int vrow0 = 4 * hi + (j >> 2);
  const int vd0 = 16 * (g & 1) + 4 * (j & 3);
  int voff2[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) voff2[q] = vrow0 * D + (((4 * q + (vd0 >> 3)) ^ swz(vrow0)) << 3) + (vd0 & 7);

  int buf = 0;
  while (e < e1) {
    // prefetch the next key tile into the other buffer
    int e_n = e, kt_n = kt + 1;
    Entry en_n = en;
    if (kt_n >= en.kt1) {
      e_n = e + 1;
      if (e_n < e1) {
        en_n = a.entries[e_n];
        kt_n = en_n.kt0;
      }
    }
    const bool has_next = e_n < e1;
    if (has_next) {
      issue_tile_loads<D>(s.t[buf ^ 1], plan, src, a.isl, kt_n * BN, L, wave);
      // wait for all but the next tile's loads (issued last)
      if (en_n.pidx >= 0 && wave == 0) {
        issue_bits_load(s.bits[buf ^ 1], a.bits, en_n.pidx, lane);
        wait_vmcnt<NLOADS + 1>();
      } else {
        wait_vmcnt<NLOADS>();
      }
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    const uint64_t bits = en.pidx >= 0 ? s.bits[buf][wave * 32 + l32] : ~0ull;
    const uint16_t* Kt = s.t[buf][0];
    const uint16_t* tKt = s.t[buf][1];
    const uint16_t* Vt = s.t[buf][2];
    const uint16_t* tVt = s.t[buf][3];

#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      // ---- scores and score tangents of 32 keys (transposed: lane = query) ----
      f32x16_t S, TS;
#pragma unroll
      for (int r = 0; r < 16; ++r) S[r] = TS[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int off = kb * 32 * D + (kk >> 2) * 64 + koff[kk & 3];
        const bf16x8_t kop = as_bf16x8(*(const u32x4_t*)(Kt + off));
        const bf16x8_t tkop = as_bf16x8(*(const u32x4_t*)(tKt + off));
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, Qr[kk], S, 0, 0, 0);
        TS = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tkop, Qr[kk], TS, 0, 0, 0);
        TS = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, tQr[kk], TS, 0, 0, 0);
      }
      // lane holds keys kb*32 + 8*(r/4) + 4*hi + r%4 of its query row

      // ---- partial tile: masked-out pairs take no part (select; no tangent) ----
      if (en.pidx >= 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          const bool ok = (bits >> key) & 1ull;
          S[r] = ok ? S[r] : -INFINITY;
          TS[r] = ok ? TS[r] : 0.f;
        }
      }

      // ---- online softmax with lazy rescale ----
      float mx = S[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
      mx = fmaxf(mx, wave_xor32(mx));
      const float m_new = fmaxf(m_run, mx * sl2);
      const bool need = m_new > m_run + kLazyRescaleLog2;
      if (__any(need)) {
        const float alpha = need ? fast_exp2(m_run - m_new) : 1.f;
        m_run = need ? m_new : m_run;
        l_part *= alpha;
        mu_part *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            Oacc[db][r] *= alpha;
            ABacc[db][r] *= alpha;
          }
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;

      // p~ = exp2(c log2e s - m); u = p~ * (c ts).  Both rounded to bf16 once;
      // l and mu are summed from the rounded values.
      bf16x8_t P[2], U[2];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int t = 0; t < 8; t += 2) {
          const int r = 8 * st + t;
          f32x2_t p, u;
          p.x = fast_exp2(__builtin_fmaf(S[r], sl2, -m_use));
          p.y = fast_exp2(__builtin_fmaf(S[r + 1], sl2, -m_use));
          u.x = p.x * (TS[r] * c);
          u.y = p.y * (TS[r + 1] * c);
          const bf16x2_t pb = __builtin_convertvector(p, bf16x2_t);
          const bf16x2_t ub = __builtin_convertvector(u, bf16x2_t);
          l_part = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, l_part, false);
          mu_part = __builtin_amdgcn_fdot2_f32_bf16(ub, ones, mu_part, false);
          P[st][t] = pb.x;
          P[st][t + 1] = pb.y;
          U[st][t] = ub.x;
          U[st][t + 1] = ub.y;
        }

      // ---- value products (transposed: rows = d, cols = queries) ----
      //   O~ += V^T P~^T ;  (A + B) += V^T U^T + tV^T P~^T
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          // keys kb*32 + 16st + vrow0 (slots 0..3) and 8 further (slots 4..7)
          const int off_a = (kb * 32 + 16 * st) * D + (db >> 1) * 64 + voff2[db & 1];
          const int off_b = off_a + 8 * D;
          const s16x4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(Vt + off_a));
          const s16x4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(Vt + off_b));
          const s16x4_t ta = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tVt + off_a));
          const s16x4_t tb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tVt + off_b));
          const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
          const bf16x8_t tvop = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(ta, tb, 0, 1, 2, 3, 4, 5, 6, 7));
          Oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, P[st], Oacc[db], 0, 0, 0);
          ABacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, U[st], ABacc[db], 0, 0, 0);
          ABacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tvop, P[st], ABacc[db], 0, 0, 0);
        }
      }
    }
    __syncthreads();  // every wave is done with this buffer before it is refilled
    e = e_n;
    kt = kt_n;
    en = en_n;
    buf ^= 1;
  }

  // ---- epilogue (Eq. 45): O = O~/l, tO = (A + B - mu O)/l ----
  const float l_tot = l_part + wave_xor32(l_part);
  const float mu_tot = mu_part + wave_xor32(mu_part);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_row < L) {
    const int64_t out_off = bb * a.osb + hh * a.osh + q_row * a.osl;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = db * 32 + 8 * gq + 4 * hi;
        f32x4_t ov, tv;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = 4 * gq + jj;
          const float o = Oacc[db][r] * inv;
          ov[jj] = o;
          tv[jj] = (ABacc[db][r] - mu_tot * o) * inv;
        }
        if constexpr (OUT_F32) {
          *(f32x4_t*)((float*)a.o + out_off + d0) = ov;
          *(f32x4_t*)((float*)a.to + out_off + d0) = tv;
        } else {
          *(bf16x4_t*)((__bf16*)a.o + out_off + d0) = __builtin_convertvector(ov, bf16x4_t);
          *(bf16x4_t*)((__bf16*)a.to + out_off + d0) = __builtin_convertvector(tv, bf16x4_t);
        }
      }
    if (hi == 0)
      a.lse[(int64_t)bh * L + q_row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs: same decomposition with MFMA 32x32x2 fp32 and no rounding of
// p~ or p~.ts.  V needs no transpose: with two keys per MFMA step each lane
// reads one value of a key row.
// ---------------------------------------------------------------------------

template <int D>
struct F32Lds {
  static constexpr int P = D + 4;
  float k[BN * P];
  float tk[BN * P];
  float v[BN * P];
  float tv[BN * P];
};

template <int D>
__device__ __forceinline__ void stage_one_f32(float* __restrict__ dst, const float* __restrict__ src,
                                              int64_t sl, int key0, int L, int tid) {
  constexpr int CH = D / 4;  // 16-byte chunks per row
  constexpr int N = BN * CH / NTHREADS;
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  f32x4_t r[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int c = tid + i * NTHREADS;
    const int key = c / CH, col = (c % CH) * 4;
    const int gk = key0 + key;
    r[i] = gk < L ? *(const f32x4_t*)(src + gk * sl + col) : zero;
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int c = tid + i * NTHREADS;
    const int key = c / CH, col = (c % CH) * 4;
    *(f32x4_t*)(dst + key * F32Lds<D>::P + col) = r[i];
  }
}

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS), amdgpu_waves_per_eu(1, 1)))
void attn_jvp_fwd_f32_kernel(FwdArgs a) {
  constexpr int NKK = D / 2;
  constexpr int NDB = D / 32;
  using Lds = F32Lds<D>;
  __shared__ __attribute__((aligned(16))) Lds s;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int BH = a.B * a.H;
  const int rank = blockIdx.x / BH, bh = blockIdx.x - rank * BH;
  const int bb = bh / a.H, hh = bh - bb * a.H;
  const int qt = a.tasks[rank];
  const int L = a.L;
  const int64_t in_off = bb * a.isb + hh * a.ish;
  const float* __restrict__ Qg = (const float*)a.q + in_off;
  const float* __restrict__ Kg = (const float*)a.k + in_off;
  const float* __restrict__ Vg = (const float*)a.v + in_off;
  const float* __restrict__ tQg = (const float*)a.tq + in_off;
  const float* __restrict__ tKg = (const float*)a.tk + in_off;
  const float* __restrict__ tVg = (const float*)a.tv + in_off;
  const int q_row = qt * BM + wave * 32 + l32;

  float Qr[NKK], tQr[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    const int64_t off = q_row * a.isl + 2 * kk + hi;
    Qr[kk] = q_row < L ? Qg[off] : 0.f;
    tQr[kk] = q_row < L ? tQg[off] : 0.f;
  }

  f32x16_t Oacc[NDB], ABacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) Oacc[db][r] = ABacc[db][r] = 0.f;
  float m_run = -INFINITY, l_part = 0.f, mu_part = 0.f;
  const float sl2 = a.scale_log2, c = a.scale;

  const int e0 = a.qt_off[qt], e1 = a.qt_off[qt + 1];
  for (int e = e0; e < e1; ++e) {
    const Entry en = a.entries[e];
    const uint64_t bits = en.pidx >= 0 ? a.bits[(int64_t)en.pidx * BM + wave * 32 + l32] : ~0ull;
    for (int kt = en.kt0; kt < en.kt1; ++kt) {
      __syncthreads();
      stage_one_f32<D>(s.k, Kg, a.isl, kt * BN, L, tid);
      stage_one_f32<D>(s.tk, tKg, a.isl, kt * BN, L, tid);
      stage_one_f32<D>(s.v, Vg, a.isl, kt * BN, L, tid);
      stage_one_f32<D>(s.tv, tVg, a.isl, kt * BN, L, tid);
      __syncthreads();

#pragma unroll 1
      for (int kb = 0; kb < BN / 32; ++kb) {
        f32x16_t S, TS;
#pragma unroll
        for (int r = 0; r < 16; ++r) S[r] = TS[r] = 0.f;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const int off = (kb * 32 + l32) * Lds::P + 2 * kk + hi;
          const float kop = s.k[off], tkop = s.tk[off];
          S = __builtin_amdgcn_mfma_f32_32x32x2f32(kop, Qr[kk], S, 0, 0, 0);
          TS = __builtin_amdgcn_mfma_f32_32x32x2f32(tkop, Qr[kk], TS, 0, 0, 0);
          TS = __builtin_amdgcn_mfma_f32_32x32x2f32(kop, tQr[kk], TS, 0, 0, 0);
        }
        if (en.pidx >= 0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            const bool ok = (bits >> key) & 1ull;
            S[r] = ok ? S[r] : -INFINITY;
            TS[r] = ok ? TS[r] : 0.f;
          }
        }
        float mx = S[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
        mx = fmaxf(mx, wave_xor32(mx));
        const float m_new = fmaxf(m_run, mx * sl2);
        const bool need = m_new > m_run + kLazyRescaleLog2;
        if (__any(need)) {
          const float alpha = need ? fast_exp2(m_run - m_new) : 1.f;
          m_run = need ? m_new : m_run;
          l_part *= alpha;
          mu_part *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              Oacc[db][r] *= alpha;
              ABacc[db][r] *= alpha;
            }
        }
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
        float P[16], U[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          P[r] = fast_exp2(__builtin_fmaf(S[r], sl2, -m_use));
          U[r] = P[r] * (TS[r] * c);
          l_part += P[r];
          mu_part += U[r];
        }
        // two keys per MFMA step: lanes hi = 0 / 1 supply key 8*(r/4) + 4*hi + r%4
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const int off = key * Lds::P + db * 32 + l32;
            const float vop = s.v[off], tvop = s.tv[off];
            Oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vop, P[r], Oacc[db], 0, 0, 0);
            ABacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vop, U[r], ABacc[db], 0, 0, 0);
            ABacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(tvop, P[r], ABacc[db], 0, 0, 0);
          }
        }
      }
    }
  }

  const float l_tot = l_part + wave_xor32(l_part);
  const float mu_tot = mu_part + wave_xor32(mu_part);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_row < L) {
    const int64_t out_off = bb * a.osb + hh * a.osh + q_row * a.osl;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = db * 32 + 8 * g + 4 * hi;
        f32x4_t ov, tv;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * g + j;
          const float o = Oacc[db][r] * inv;
          ov[j] = o;
          tv[j] = (ABacc[db][r] - mu_tot * o) * inv;
        }
        *(f32x4_t*)((float*)a.o + out_off + d0) = ov;
        *(f32x4_t*)((float*)a.to + out_off + d0) = tv;
      }
    if (hi == 0)
      a.lse[(int64_t)bh * L + q_row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------

int launch_fwd(const FwdArgs& a, int in_dtype, int out_dtype, int head_dim, hipStream_t stream) {
  const int64_t grid64 = int64_t(a.n_tasks) * a.B * a.H;
  if (grid64 <= 0 || grid64 > 0x7fffffff) return AJ_EINVAL;
  const dim3 grid((unsigned)grid64), block(NTHREADS);
  if (in_dtype == AJ_BF16) {
    if (out_dtype == AJ_BF16) {
      if (head_dim == 128) hipLaunchKernelGGL((attn_jvp_fwd_bf16_kernel<128, false>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((attn_jvp_fwd_bf16_kernel<64, false>), grid, block, 0, stream, a);
    } else {
      if (head_dim == 128) hipLaunchKernelGGL((attn_jvp_fwd_bf16_kernel<128, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((attn_jvp_fwd_bf16_kernel<64, true>), grid, block, 0, stream, a);
    }
  } else {
    if (head_dim == 128) hipLaunchKernelGGL((attn_jvp_fwd_f32_kernel<128>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_jvp_fwd_f32_kernel<64>), grid, block, 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? AJ_OK : AJ_EHIP;
}

}  // namespace aj
