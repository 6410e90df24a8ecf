// Custom-mask attention JVP forward for gfx950 (MI355X).
//
// "Causal-rCM", App. B: one online-softmax pass computes the primal output of
// masked attention (Eq. 42) and its tangent (Eq. 44, evaluated as Eq. 45),
// streaming only the admissible key tiles of the mask; the same tile schedule
// serves the scores and their tangents.
//
// Work decomposition.  A workgroup owns one 128-row query tile of one (batch,
// head), split into 16-row waves (8 per workgroup) or 32-row waves (4 per
// workgroup); the shapes are described below.  Keys stream in tiles of 64
// through LDS.  Per key tile and wave:
//   S^T  = K Q^T             (keys x queries, bf16 MFMA, fp32 accumulation)
//   tS^T = tK Q^T + K tQ^T   (one accumulator chain)
// Computing the transposed scores puts each query row in one lane column (the
// lanes of a column split its keys), so the softmax statistics are per lane up
// to a cross-lane exchange, and the accumulator registers feed the next MFMA
// as its B operand without any data movement:
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

#include <type_traits>

#include "aj_device.h"
#include "aj_launch.h"

namespace aj {

// ---------------------------------------------------------------------------
// bf16 inputs, 16-row waves (the JVP at head_dim 128)
// ---------------------------------------------------------------------------
//
// A workgroup is 8 waves (two per SIMD); wave w owns query rows 16w .. 16w+15
// of the 128-row tile.  With 16 rows per wave the row state (Q, tQ, O~, A+B,
// scores) fits in 256 registers, so each SIMD runs two waves and the hardware
// overlaps one wave's softmax and LDS latency with the other wave's MFMAs.
// MFMA v_mfma_f32_16x16x32_bf16 on transposed scores S^T = K Q^T: lane
// l = 16g + j holds keys 4g + r (r = 0..3) of each 16-key block for query row
// j, i.e. one query per 16-lane column with its keys split over the four
// groups g.  Two 16-key blocks form the 8 k-slots of a value MFMA's B
// operand, so the score accumulators feed O~^T += V^T P~^T directly.
//
// Key tiles of 64 keys (K, tK, V, tV rows and, for partial tiles, the 128
// per-row key bitmasks) stream by direct buffer -> LDS DMA into a double
// buffer: tile t+1 loads while tile t computes.  V and tV are read with
// gfx950's LDS transpose read.  Rows are unpadded; 16-byte chunk c of row r is
// stored at position c ^ swz_q16(r) (aj_device.h), one layout that keeps both
// the row reads of K and the transpose reads of V free of bank conflicts.
// The 32-row kernels of attn_fwd_q32.hip use the same streaming scheme.

constexpr int kWavesQ16 = 8;

// ---- q16 shape --------------------------------------------------------------

template <int D, bool OUT_F32, bool VARIANTS>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kWavesQ16, 64 * kWavesQ16), amdgpu_waves_per_eu(2, 2)))
void attn_jvp_fwd_bf16_q16_kernel(FwdArgs a) {
  constexpr int NKS = D / 32;  // MFMA k-steps over d for the score products
  constexpr int NDB = D / 16;  // 16-row blocks of d for the value products
  using Lds = Bf16Lds<D, 4>;
  __shared__ __attribute__((aligned(1024))) Lds s;
  static_assert(offsetof(Lds, bits) == Lds::bits_off(0), "LDS layout");
  const uint32_t lds0 = lds_addr(&s);

  const int tid = threadIdx.x, wave = wave_uniform(tid >> 6), lane = tid & 63, j16 = lane & 15, g = lane >> 4;
  const int BH = a.B * a.H;
  const TaskCoord tc = task_coord(blockIdx.x, a.n_tasks, BH, a.head_group);
  const int rank = tc.rank, bh = tc.bh;
  const int bb = bh / a.H, hh = bh - bb * a.H;
  const int qt = wave_uniform(a.tasks[rank]);
  const int L = a.L;
  const int64_t in_off = bb * a.isb + hh * a.ish;
  const int64_t kv_off = bb * a.ksb + hh * a.ksh;
  const uint16_t* __restrict__ Qg = (const uint16_t*)a.q + in_off;
  const uint16_t* __restrict__ tQg = (const uint16_t*)a.tq + in_off;
  const uint16_t* const src[4] = {(const uint16_t*)a.k + kv_off, (const uint16_t*)a.tk + kv_off,
                                  (const uint16_t*)a.v + kv_off, (const uint16_t*)a.tv + kv_off};
  const int q_row = qt * BM + wave * 16 + j16;

  // Q and tQ of this lane's query row, as B operands: k-step ks holds
  // d = 32ks + 8g .. 32ks + 8g + 7.
  bf16x8_t Qr[NKS], tQr[NKS];
  {
    const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int64_t off = q_row * a.isl + ks * 32 + 8 * g;
      Qr[ks] = as_bf16x8(q_row < L ? *(const u32x4_t*)(Qg + off) : zero);
      tQr[ks] = as_bf16x8(q_row < L ? *(const u32x4_t*)(tQg + off) : zero);
    }
  }
  // Q and tQ have landed before any DMA is in flight: the compiler tracks no
  // load inside the tile loop.
  wait_vmcnt<0>();

  const TileLoadPlan<kWavesQ16, D> plan(a.ksl, wave, lane, swz_q16<D>);
  // DMA of key tile kti of entry x (tangent tiles only where x carries them)
  auto prefetch = [&](int b, const Entry& x, int kti) {
    if (!VARIANTS || x.flags == kTileJvp)
      issue_tile_loads<kWavesQ16, D, true, 4>(lds0 + Lds::t_off(b), plan, src, a.ksl, kti * BN, a.Lk, wave);
    else
      issue_tile_loads<kWavesQ16, D, false, 4>(lds0 + Lds::t_off(b), plan, src, a.ksl, kti * BN, a.Lk, wave);
    if (x.pidx >= 0 && wave == 0) issue_bits_load(lds0 + Lds::bits_off(b), a.bits, x.pidx, lane);
  };

  const int e0 = wave_uniform(a.qt_off[qt]), e1 = wave_uniform(a.qt_off[qt + 1]);
  int e = e0, kt = 0;
  Entry en = {0, 0, -1, 0};
  if (e < e1) {
    en = load_entry(a.entries + e);
    kt = en.kt0;
    prefetch(0, en, kt);
  }

  f32x4_t Oacc[NDB], ABacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) Oacc[db][r] = ABacc[db][r] = 0.f;
  float m_run = -INFINITY;            // reference max (log2 units, scale folded in)
  float l_part = 0.f, mu_part = 0.f;  // this lane's share of the row sums
  const float sl2 = a.scale_log2, c = a.scale;
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};

  // Per-lane LDS offsets (elements) that do not depend on the tile.
  // K operand of 16-key block kb, k-step ks: row 16kb + j16 (swz(16kb + j16)
  // == swz(j16)), logical chunk 4ks + g.
  int koff[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) koff[ks] = j16 * D + (((4 * ks + g) ^ swz_q16<D>(j16)) << 3);
  // V^T operand (transpose read) of value k-step p (keys 32p .. 32p+31), d
  // block db: lane j16 of group g names key 32p + 4g + j16/4 (+16 for the
  // second read) and d = 16db + 4(j16%4), i.e. logical chunk 2db + (j16%4)/2,
  // half j16 % 2.  swz depends on the row mod 16, which 32p and 16 keep.
  const int vrow = 4 * g + (j16 >> 2);
  // The second read of a pair is 16 rows further on, at the same swizzle
  // (swz_q16 depends on the row mod 16): a constant offset of 16 D.
  int voff[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int chunk = 2 * db + ((j16 & 3) >> 1);
    voff[db] = vrow * D + ((chunk ^ swz_q16<D>(vrow)) << 3) + 4 * (j16 & 1);
  }

  int buf = 0;

  // One 64-key tile of the variant VAR (which tangents the tile carries).
  auto tile = [&](auto var_tag) __attribute__((always_inline)) {
    constexpr int VAR = decltype(var_tag)::value;
    constexpr bool HAS_TS = VAR != kTileAllFree;  // score tangent nonzero
    constexpr bool HAS_TKV = VAR == kTileJvp;     // tK and tV tiles present
    const uint16_t* Kt = s.t[buf][0];
    const uint16_t* tKt = s.t[buf][1];
    const uint16_t* Vt = s.t[buf][2];
    const uint16_t* tVt = s.t[buf][3];

    // ---- scores and score tangents (transposed) ----
    // k-step outer, key block inner: four independent accumulator chains per
    // operand, so consecutive MFMAs never depend on each other.
    f32x4_t S[4], TS[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) S[kb][r] = TS[kb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8_t kop[4], tkop[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int off = kb * 16 * D + koff[ks];
        kop[kb] = as_bf16x8(*(const u32x4_t*)(Kt + off));
        if constexpr (HAS_TKV) tkop[kb] = as_bf16x8(*(const u32x4_t*)(tKt + off));
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) S[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kb], Qr[ks], S[kb], 0, 0, 0);
      if constexpr (HAS_TKV) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          TS[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tkop[kb], Qr[ks], TS[kb], 0, 0, 0);
      }
      if constexpr (HAS_TS) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          TS[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[kb], tQr[ks], TS[kb], 0, 0, 0);
      }
    }
    // lane holds keys 16kb + 4g + r of query row j16

    // ---- partial tile: masked-out pairs take no part (select; no tangent) ----
    if (en.pidx >= 0) {
      const uint64_t bits = s.bits[buf][wave * 16 + j16] >> (4 * g);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool ok = (bits >> (16 * kb + r)) & 1ull;
          S[kb][r] = ok ? S[kb][r] : -INFINITY;
          if constexpr (HAS_TS) TS[kb][r] = ok ? TS[kb][r] : 0.f;
        }
    }

    // ---- online softmax with lazy rescale ----
    float mx = S[0][0];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, S[kb][r]);
    mx = row4_max(mx);
    const float m_new = fmaxf(m_run, mx * sl2);
    const bool need = m_new > m_run + kLazyRescaleLog2;
    if (__any(need)) {
      const float alpha = need ? fast_exp2(m_run - m_new) : 1.f;
      m_run = need ? m_new : m_run;
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) Oacc[db][r] *= alpha;
      mu_part *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) ABacc[db][r] *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;

    // p~ = exp2(c log2e s - m); u = p~ * (c ts).  Both rounded to bf16 once;
    // l and mu are summed from the rounded values.  Value k-step p takes
    // blocks 2p (slots 0..3) and 2p+1 (slots 4..7).
    bf16x8_t P[2], U[2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        f32x2_t p, u;
        p.x = fast_exp2(__builtin_fmaf(S[kb][r], sl2, -m_use));
        p.y = fast_exp2(__builtin_fmaf(S[kb][r + 1], sl2, -m_use));
        if constexpr (HAS_TS) {
          u.x = p.x * (TS[kb][r] * c);
          u.y = p.y * (TS[kb][r + 1] * c);
        }
        const bf16x2_t pb = __builtin_convertvector(p, bf16x2_t);
        bf16x2_t ub;
        if constexpr (HAS_TS) ub = __builtin_convertvector(u, bf16x2_t);
        l_part = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, l_part, false);
        if constexpr (HAS_TS) mu_part = __builtin_amdgcn_fdot2_f32_bf16(ub, ones, mu_part, false);
        const int slot = 4 * (kb & 1) + r;
        P[kb >> 1][slot] = pb.x;
        P[kb >> 1][slot + 1] = pb.y;
        if constexpr (HAS_TS) {
          U[kb >> 1][slot] = ub.x;
          U[kb >> 1][slot + 1] = ub.y;
        }
      }

    // ---- value products (transposed: rows = d, cols = queries) ----
    //   O~ += V^T P~^T ;  (A + B) += V^T U^T + tV^T P~^T
    // four d blocks at a time: independent accumulator chains between the
    // dependent (A + B) updates
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
      for (int d4 = 0; d4 < NDB; d4 += 4) {
        bf16x8_t vop[4], tvop[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int off_a = 32 * p * D + voff[d4 + i];
          const int off_b = off_a + 16 * D;
          const s16x4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(Vt + off_a));
          const s16x4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(Vt + off_b));
          s16x4_t ta, tb;
          if constexpr (HAS_TKV) {
            ta = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tVt + off_a));
            tb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tVt + off_b));
          }
          vop[i] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
          if constexpr (HAS_TKV)
            tvop[i] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(ta, tb, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) Oacc[d4 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[i], P[p], Oacc[d4 + i], 0, 0, 0);
        if constexpr (HAS_TS) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            ABacc[d4 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[i], U[p], ABacc[d4 + i], 0, 0, 0);
        }
        if constexpr (HAS_TKV) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            ABacc[d4 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tvop[i], P[p], ABacc[d4 + i], 0, 0, 0);
        }
      }
    }
  };

  while (e < e1) {
    // next key tile, loaded into the other buffer while this one is computed
    int e_n = e, kt_n = kt + 1;
    Entry en_n = en;
    if (kt_n >= en.kt1) {
      e_n = e + 1;
      if (e_n < e1) {
        en_n = load_entry(a.entries + e_n);
        kt_n = en_n.kt0;
      }
    }
    // One barrier per tile: after it, every wave's loads of this tile have
    // landed and every wave is done with the other buffer, which the next
    // tile's DMA then refills.
    wait_vmcnt<0>();
    __syncthreads();
    if (e_n < e1) prefetch(buf ^ 1, en_n, kt_n);
    if constexpr (!VARIANTS) {
      tile(std::integral_constant<int, kTileJvp>{});
    } else {
      const int var = __builtin_amdgcn_readfirstlane(en.flags);
      if (var == kTileJvp) tile(std::integral_constant<int, kTileJvp>{});
      else if (var == kTileKeysFree) tile(std::integral_constant<int, kTileKeysFree>{});
      else tile(std::integral_constant<int, kTileAllFree>{});
    }
    e = e_n;
    kt = kt_n;
    en = en_n;
    buf ^= 1;
  }

  // ---- epilogue (Eq. 45): O = O~/l, tO = (A + B - mu O)/l ----
  const float l_tot = row4_sum(l_part);
  const float mu_tot = row4_sum(mu_part);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // the lane's group, recomputed here rather than kept live across the loop
  const int ge = int(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u))) >> 4;
  if (q_row < L) {
    const int64_t out_off = bb * a.osb + hh * a.osh + q_row * a.osl;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d0 = db * 16 + 4 * ge;
      f32x4_t ov, tv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float o = Oacc[db][r] * inv;
        ov[r] = o;
        tv[r] = (ABacc[db][r] - mu_tot * o) * inv;
      }
      if constexpr (OUT_F32) {
        *(f32x4_t*)((float*)a.o + out_off + d0) = ov;
        *(f32x4_t*)((float*)a.to + out_off + d0) = tv;
      } else {
        *(bf16x4_t*)((__bf16*)a.o + out_off + d0) = __builtin_convertvector(ov, bf16x4_t);
        *(bf16x4_t*)((__bf16*)a.to + out_off + d0) = __builtin_convertvector(tv, bf16x4_t);
      }
    }
    if (ge == 0)
      a.lse[(int64_t)bh * L + q_row] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// Enqueues the 16-row JVP kernel (head_dim 128) over `grid` workgroups.
void launch_q16(const FwdArgs& a, bool out_f32, bool variants, dim3 grid, hipStream_t stream) {
  const dim3 block(64 * kWavesQ16);
  if (variants) {
    if (out_f32) hipLaunchKernelGGL((attn_jvp_fwd_bf16_q16_kernel<128, true, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_jvp_fwd_bf16_q16_kernel<128, false, true>), grid, block, 0, stream, a);
  } else {
    if (out_f32) hipLaunchKernelGGL((attn_jvp_fwd_bf16_q16_kernel<128, true, false>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_jvp_fwd_bf16_q16_kernel<128, false, false>), grid, block, 0, stream, a);
  }
}

}  // namespace aj
