// Masked attention forward kernels for gfx950 (MI355X) besides the 16-row JVP
// kernel of attn_jvp_fwd.hip, and the launcher that picks among them:
// * the 32-row bf16 kernel: the JVP at head_dim 64, and without its tangent
//   products the primal forward (attn_fwd, "Causal-rCM" Sec. 3.1.1, Eq. 8;
//   App. B, Eq. 42) and the KV-cache forward (Sec. 3.2.1) at both head dims;
// * the fp32-input JVP kernel.
// The arithmetic, the online softmax and the streaming scheme are those
// described in attn_jvp_fwd.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <type_traits>

#include "../../include/attn_jvp.h"
#include "aj_device.h"
#include "aj_launch.h"

namespace aj {

constexpr int NWAVES = 4;
constexpr int NTHREADS = 64 * NWAVES;

// ---------------------------------------------------------------------------
// bf16 inputs, 32-row waves
// ---------------------------------------------------------------------------
//
// A workgroup is 4 waves of 32 rows each, two workgroups per CU (three for the
// d = 64 primal kernel; the d = 128 primal kernel runs one workgroup of 8
// waves, see NWV below); MFMA
// v_mfma_f32_32x32x16_bf16 on S^T, lanes l and l+32 share one query row.  At
// d = 64 the softmax's vector work matches the matrix work per element, and
// the larger waves amortise the per-tile fixed costs better; without the
// tangents the register state fits two 32-row waves per SIMD at d = 128 too,
// and K, V tiles alone (66 KB of LDS) let two workgroups share a CU.  Tiles
// are stored at chunk position c ^ swz_q32(r) (aj_device.h).

constexpr int kWavesQ32 = 4;

// v_mfma_f32_32x32x16 with bf16 or fp16 operands
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma32(f16x8_t a, f16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// ---- q32 shape --------------------------------------------------------------

// SCALE_IN_Q: the scale is a power of two in (0, 1] and is folded into the Q
// and tQ registers (exact: a power-of-two multiple of a bf16 value is a bf16
// value, and every fp32 partial sum of the score products scales with it), so
// the MFMAs deliver c s and c ts and u = p~ (c ts) takes one multiply less.
// The results are bit for bit those of the unfolded kernel.
//
// Occupancy: two workgroups per CU (two waves per SIMD, up to 256 VGPRs),
// except the d = 64 primal kernel, which fits 168 VGPRs and 34 KB of LDS and
// runs three.
template <int D, bool JVP>
constexpr int q32_waves_per_simd() { return D == 64 && !JVP ? 3 : 2; }

// NWV: waves per workgroup, 4 (128-row tasks of the descriptor's row map) or,
// for the primal forward at d = 128, 8 (256-row tasks of its wide map): the
// eight waves fill the CU's two waves per SIMD as one workgroup, so every
// streamed key tile serves 256 rows, half the DMA and LDS writes per FLOP of
// two 128-row workgroups (5 % on the KV-cache step).
//
// VARIANTS (JVP only): the descriptor declares tangent-free tokens; tiles whose
// keys carry no tangent skip the tK and tV DMA, reads and products, the others
// run them.  Tiles where neither queries nor keys carry tangents take the same
// keys-tangent-free path: their tQ is zero, so their score tangents and u are
// exact zeros.
//
// V16 (JVP at d = 64 only): V and tV come as fp16 copies made by
// bf16_to_f16_kv_kernel before the launch (a.v16, a.tv16, with the key
// strides), so the per-tile conversion in LDS is skipped; the values are the
// same, so are the results, bit for bit.
template <int D, bool OUT_F32, bool JVP, bool SCALE_IN_Q = false, bool VARIANTS = false, int NWV = kWavesQ32,
          bool V16 = false>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NWV, 64 * NWV),
                          amdgpu_waves_per_eu(q32_waves_per_simd<D, JVP>(), q32_waves_per_simd<D, JVP>())))
void attn_jvp_fwd_bf16_q32_kernel(FwdArgs a) {
  static_assert(NWV == kWavesQ32 || (NWV == 8 && D == 128 && !JVP), "8-wave workgroups: d = 128 primal only");
  static_assert(!V16 || (JVP && D == 64), "fp16 copies of V and tV: the JVP at d = 64 only");
  constexpr int NKK = D / 16;  // MFMA k-steps over d for the score products
  constexpr int NDB = D / 32;  // 32-row blocks of d for the value products
  constexpr int NT = JVP ? 4 : 2;
  constexpr int BMW = 32 * NWV;  // query rows per task
  using Lds = Bf16Lds<D, NT, BMW>;
  // The JVP runs its value products in fp16: V and tV are converted in LDS
  // (exact for bf16 values of magnitude in [2^-14, 65504]), and p~ 2^-8 and
  // u = p~ 2^-8 (c ts) are rounded to fp16 (11 significant bits against
  // bf16's 8).  The tangent's A - mu O cancellation is sensitive to the
  // rounding of both p~ (through O) and u; in fp16 their error is eight times
  // smaller.  The 2^-8 keeps p~ 2^-8 <= 1 under the lazy rescale (p~ <= 2^8),
  // so u stays finite for |c ts| < 65504.  The primal kernel stays in bf16.
  constexpr bool F16 = JVP;
  typedef std::conditional_t<F16, f16x8_t, bf16x8_t> op8_t;
  typedef std::conditional_t<F16, f16x2_t, bf16x2_t> op2_t;
  constexpr float kPScaleLog2 = F16 ? 8.0f : 0.0f;  // p~ is stored as p~ 2^-kPScaleLog2
  __shared__ __attribute__((aligned(1024))) Lds s;
  static_assert(offsetof(Lds, bits) == Lds::bits_off(0), "LDS layout");
  const uint32_t lds0 = lds_addr(&s);

  const int tid = threadIdx.x, wave = wave_uniform(tid >> 6), lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int BH = a.B * a.H;
  const TaskCoord tc = task_coord(blockIdx.x, a.n_tasks, BH, a.head_group);
  const int rank = tc.rank, bh = tc.bh;
  const int bb = bh / a.H, hh = bh - bb * a.H;
  const int qt = wave_uniform(a.tasks[rank]);
  const int L = a.L;
  const int64_t in_off = bb * a.isb + hh * a.ish;
  const int64_t kv_off = bb * a.ksb + hh * a.ksh;
  const uint16_t* __restrict__ Qg = (const uint16_t*)a.q + in_off;
  const uint16_t* __restrict__ tQg = JVP ? (const uint16_t*)a.tq + in_off : nullptr;
  const void* const vsrc = V16 ? a.v16 : a.v;
  const void* const tvsrc = V16 ? a.tv16 : a.tv;
  const uint16_t* const src[4] = {(const uint16_t*)a.k + kv_off, JVP ? (const uint16_t*)a.tk + kv_off : nullptr,
                                  (const uint16_t*)vsrc + kv_off, JVP ? (const uint16_t*)tvsrc + kv_off : nullptr};
  const int q_row = qt * BMW + wave * 32 + l32;

  const TileLoadPlan<NWV, D> plan(a.ksl, wave, lane, swz_q32<D>);
  // DMA of key tile kti of entry x (tK and tV only where x carries them)
  auto prefetch = [&](int b, const Entry& x, int kti) {
    if (JVP && (!VARIANTS || x.flags == kTileJvp))
      issue_tile_loads<NWV, D, true, NT>(lds0 + Lds::t_off(b), plan, src, a.ksl, kti * BN, a.Lk, wave);
    else
      issue_tile_loads<NWV, D, false, NT>(lds0 + Lds::t_off(b), plan, src, a.ksl, kti * BN, a.Lk, wave);
    if constexpr (NWV == 8) {
      if (x.pidx >= 0 && wave < 2) issue_bits_load_wide(lds0 + Lds::bits_off(b), a.bits, x.pidx, wave, lane);
    } else {
      if (x.pidx >= 0 && wave == 0) issue_bits_load(lds0 + Lds::bits_off(b), a.bits, x.pidx, lane);
    }
  };

  // first key tile in flight before the prologue
  const int e0 = wave_uniform(a.qt_off[qt]), e1 = wave_uniform(a.qt_off[qt + 1]);
  int e = e0, kt = 0;
  Entry en = {0, 0, -1, 0};
  if (e < e1) {
    en = load_entry(a.entries + e);
    kt = en.kt0;
    prefetch(0, en, kt);
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
      tQr[kk] = as_bf16x8(JVP && q_row < L ? *(const u32x4_t*)(tQg + off) : zero);
    }
  }
  // Q, tQ and the first key tile have landed; nothing the compiler tracks is
  // in flight inside the loop below.
  wait_vmcnt<0>();
  if constexpr (SCALE_IN_Q) {
    typedef float f32x8_t __attribute__((ext_vector_type(8)));
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      Qr[kk] = __builtin_convertvector(__builtin_convertvector(Qr[kk], f32x8_t) * a.scale, bf16x8_t);
      tQr[kk] = __builtin_convertvector(__builtin_convertvector(tQr[kk], f32x8_t) * a.scale, bf16x8_t);
    }
  }

  f32x16_t Oacc[NDB], ABacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) Oacc[db][r] = ABacc[db][r] = 0.f;
  float m_run = -INFINITY;            // reference max (log2 units, scale folded in)
  float l_part = 0.f, mu_part = 0.f;  // this lane's half of the row sums
  // log2(e) and 1 when the scale is already in the scores
  const float sl2 = SCALE_IN_Q ? 1.44269504088896340736f : a.scale_log2, c = SCALE_IN_Q ? 1.0f : a.scale;
  const op2_t ones = {1.0f, 1.0f};

  int koff[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) koff[kk] = l32 * D + (((2 * kk + hi) ^ swz_q32<D>(l32)) << 3);
  const int g = lane >> 4, j = lane & 15;
  const int vrow0 = 4 * hi + (j >> 2);
  const int vd0 = 16 * (g & 1) + 4 * (j & 3);
  int voff[2][NDB];
#pragma unroll
  for (int h8 = 0; h8 < 2; ++h8)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int row = vrow0 + 8 * h8;
      voff[h8][db] = row * D + (((4 * db + (vd0 >> 3)) ^ swz_q32<D>(row)) << 3) + (vd0 & 7);
    }

  int buf = 0;

  // One 64-key tile of the variant VAR (which tangents the tile carries).
  // tkv_rt: the tile carries tK and tV (wave-uniform; false only for the
  // keys-tangent-free tiles of a VARIANTS instance).  One code with branches
  // around the tK and tV work rather than a second copy of the tile code: two
  // copies need more than the 256 registers of two workgroups per CU.
  auto tile = [&](auto var_tag, bool tkv_rt) __attribute__((always_inline)) {
    constexpr int VAR = decltype(var_tag)::value;
    constexpr bool HAS_TS = JVP && VAR != kTileAllFree;  // score tangent nonzero
    constexpr bool HAS_TKV = JVP && VAR == kTileJvp;     // tK and tV products built
    const bool tkv = HAS_TKV && tkv_rt;
    const uint64_t bits = en.pidx >= 0 ? s.bits[buf][wave * 32 + l32] : ~0ull;
    const uint16_t* Kt = s.t[buf][Lds::slot(0)];
    const uint16_t* tKt = s.t[buf][Lds::slot(1)];
    const uint16_t* Vt = s.t[buf][Lds::slot(2)];
    const uint16_t* tVt = s.t[buf][Lds::slot(3)];

#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
      // ---- scores and score tangents of 32 keys (transposed: lane = query) ----
      f32x16_t S, TS;
#pragma unroll
      for (int r = 0; r < 16; ++r) S[r] = TS[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int off = kb * 32 * D + koff[kk];
        const bf16x8_t kop = as_bf16x8(*(const u32x4_t*)(Kt + off));
        bf16x8_t tkop;
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, Qr[kk], S, 0, 0, 0);
        if constexpr (HAS_TKV) {
          if (tkv) {
            tkop = as_bf16x8(*(const u32x4_t*)(tKt + off));
            TS = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tkop, Qr[kk], TS, 0, 0, 0);
          }
        }
        if constexpr (HAS_TS) TS = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, tQr[kk], TS, 0, 0, 0);
      }
      // lane holds keys kb*32 + 8*(r/4) + 4*hi + r%4 of its query row
      // JVP at d = 64: the block that holds the first half's softmax, its value
      // products and these score products of the second half is scheduled as
      // 24 x (one MFMA, three vector instructions), so that the softmax issues
      // between the MFMAs instead of ahead of them (1.2-1.6 % on the stress
      // workload; other ratios measured 0-0.6 %).
      if constexpr (F16) {
        if (kb == 1) {
#pragma unroll
          for (int i = 0; i < 24; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
          }
        }
      }

      // ---- partial tile: masked-out pairs take no part (select; no tangent) ----
      if (en.pidx >= 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          const bool ok = (bits >> key) & 1ull;
          S[r] = ok ? S[r] : -INFINITY;
          if constexpr (HAS_TS) TS[r] = ok ? TS[r] : 0.f;
        }
      }

      // ---- online softmax with lazy rescale ----
      float mx = S[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
      mx = row_max_halves(mx);
      const float m_new = fmaxf(m_run, mx * sl2);
      const bool need = m_new > m_run + kLazyRescaleLog2;
      if (__any(need)) {
        const float alpha = need ? fast_exp2(m_run - m_new) : 1.f;
        m_run = need ? m_new : m_run;
        l_part *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) Oacc[db][r] *= alpha;
        if constexpr (JVP) {
          mu_part *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) ABacc[db][r] *= alpha;
        }
      }
      const float m_use = (m_run == -INFINITY ? 0.f : m_run) + kPScaleLog2;

      // p~ = exp2(c log2e s - m) (times 2^-8 in fp16); u = p~ * (c ts).  Both
      // rounded once to the value-product type; l and mu are summed from the
      // rounded values.
      op8_t P[2], U[2];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int t = 0; t < 8; t += 2) {
          const int r = 8 * st + t;
          f32x2_t p, u;
          p.x = fast_exp2(__builtin_fmaf(S[r], sl2, -m_use));
          p.y = fast_exp2(__builtin_fmaf(S[r + 1], sl2, -m_use));
          if constexpr (HAS_TS) {
            u.x = p.x * (TS[r] * c);
            u.y = p.y * (TS[r + 1] * c);
          }
          const op2_t pb = __builtin_convertvector(p, op2_t);
          op2_t ub;
          if constexpr (HAS_TS) ub = __builtin_convertvector(u, op2_t);
          if constexpr (F16) {
            l_part = __builtin_amdgcn_fdot2(pb, ones, l_part, false);
            if constexpr (HAS_TS) mu_part = __builtin_amdgcn_fdot2(ub, ones, mu_part, false);
          } else {
            l_part = __builtin_amdgcn_fdot2_f32_bf16(pb, ones, l_part, false);
            if constexpr (HAS_TS) mu_part = __builtin_amdgcn_fdot2_f32_bf16(ub, ones, mu_part, false);
          }
          P[st][t] = pb.x;
          P[st][t + 1] = pb.y;
          if constexpr (HAS_TS) {
            U[st][t] = ub.x;
            U[st][t + 1] = ub.y;
          }
        }

      // ---- value products (transposed: rows = d, cols = queries) ----
      //   O~ += V^T P~^T ;  (A + B) += V^T U^T + tV^T P~^T
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          // keys kb*32 + 16st + vrow0 (slots 0..3) and 8 further (slots 4..7)
          const int off_a = (kb * 32 + 16 * st) * D + voff[0][db];
          const int off_b = (kb * 32 + 16 * st) * D + voff[1][db];
          const s16x4_t va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(Vt + off_a));
          const s16x4_t vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(Vt + off_b));
          const op8_t vop = __builtin_bit_cast(op8_t, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
          Oacc[db] = mfma32(vop, P[st], Oacc[db]);
          if constexpr (HAS_TS) ABacc[db] = mfma32(vop, U[st], ABacc[db]);
          if constexpr (HAS_TKV) {
            if (tkv) {
              const s16x4_t ta = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tVt + off_a));
              const s16x4_t tb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tVt + off_b));
              const op8_t tvop = __builtin_bit_cast(op8_t, __builtin_shufflevector(ta, tb, 0, 1, 2, 3, 4, 5, 6, 7));
              ABacc[db] = mfma32(tvop, P[st], ABacc[db]);
            }
          }
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
    // fp16 value products: this wave's share of the V and tV tiles, converted
    // before the barrier publishes them
    if constexpr (F16 && !V16) {
      if (!VARIANTS || en.flags == kTileJvp)
        bf16_chunks_to_f16<NWV, D, 2>(s.t[buf][Lds::slot(2)], s.t[buf][Lds::slot(3)], wave, lane);
      else
        bf16_chunks_to_f16<NWV, D, 1>(s.t[buf][Lds::slot(2)], s.t[buf][Lds::slot(3)], wave, lane);
    }
    __syncthreads();
    if (e_n < e1) prefetch(buf ^ 1, en_n, kt_n);
    if constexpr (!JVP) tile(std::integral_constant<int, kTileAllFree>{}, false);
    else tile(std::integral_constant<int, kTileJvp>{}, !VARIANTS || en.flags == kTileJvp);
    e = e_n;
    kt = kt_n;
    en = en_n;
    buf ^= 1;
  }

  // ---- epilogue (Eq. 45): O = O~/l, tO = (A + B - mu O)/l ----
  const float l_tot = l_part + wave_xor32(l_part);
  const float mu_tot = JVP ? mu_part + wave_xor32(mu_part) : 0.f;
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
          if constexpr (JVP) *(f32x4_t*)((float*)a.to + out_off + d0) = tv;
        } else {
          *(bf16x4_t*)((__bf16*)a.o + out_off + d0) = __builtin_convertvector(ov, bf16x4_t);
          if constexpr (JVP) *(bf16x4_t*)((__bf16*)a.to + out_off + d0) = __builtin_convertvector(tv, bf16x4_t);
        }
        // primal rows of a JVP call (all their tangents declared zero): tO = 0
        if constexpr (!JVP) {
          if (a.to) {
            if constexpr (OUT_F32) *(f32x4_t*)((float*)a.to + out_off + d0) = f32x4_t{0.f, 0.f, 0.f, 0.f};
            else *(u32x2_t*)((__bf16*)a.to + out_off + d0) = u32x2_t{0u, 0u};
          }
        }
      }
    if (hi == 0)
      a.lse[(int64_t)bh * L + q_row] = l_tot > 0.f ? (m_run + kPScaleLog2 + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

// fp16 copies of V and tV for the V16 instances: every row of every (b, h)
// up to the key length, at the key strides, each 32-bit pair of bf16 values
// rewritten by bf16x2_to_f16x2 (the conversion bf16_chunks_to_f16 applies in
// LDS).  One thread per 16-byte chunk: threads [0, n) take V, [n, 2n) tV,
// n = B * H * Lk * D / 8.
template <int D>
__global__ __launch_bounds__(256) void bf16_to_f16_kv_kernel(FwdArgs a) {
  constexpr int CH = D / 8;  // 16-byte chunks per row
  const int64_t n = int64_t(a.B) * a.H * a.Lk * CH;
  int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= 2 * n) return;
  const bool t = i >= n;
  if (t) i -= n;
  const int c = int(i % CH);
  const int64_t row = i / CH;  // (b * H + h) * Lk + l
  const int64_t l = row % a.Lk, bh = row / a.Lk;
  const int64_t b = bh / a.H, h = bh - b * a.H;
  const int64_t off = b * a.ksb + h * a.ksh + l * a.ksl + 8 * c;
  const u32x4_t x = *(const u32x4_t*)((const uint16_t*)(t ? a.tv : a.v) + off);
  u32x4_t y;
#pragma unroll
  for (int w = 0; w < 4; ++w) y[w] = bf16x2_to_f16x2(x[w]);
  *(u32x4_t*)((uint16_t*)(t ? a.tv16 : a.v16) + off) = y;
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
  const TaskCoord tc = task_coord(blockIdx.x, a.n_tasks, BH, a.head_group);
  const int rank = tc.rank, bh = tc.bh;
  const int bb = bh / a.H, hh = bh - bb * a.H;
  const int qt = wave_uniform(a.tasks[rank]);
  const int L = a.L;
  const int64_t in_off = bb * a.isb + hh * a.ish;
  const float* __restrict__ Qg = (const float*)a.q + in_off;
  const int64_t kv_off = bb * a.ksb + hh * a.ksh;
  const float* __restrict__ Kg = (const float*)a.k + kv_off;
  const float* __restrict__ Vg = (const float*)a.v + kv_off;
  const float* __restrict__ tQg = (const float*)a.tq + in_off;
  const float* __restrict__ tKg = (const float*)a.tk + kv_off;
  const float* __restrict__ tVg = (const float*)a.tv + kv_off;
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

  const int e0 = wave_uniform(a.qt_off[qt]), e1 = wave_uniform(a.qt_off[qt + 1]);
  for (int e = e0; e < e1; ++e) {
    const Entry en = a.entries[e];
    const uint64_t bits = en.pidx >= 0 ? a.bits[(int64_t)en.pidx * BM + wave * 32 + l32] : ~0ull;
    for (int kt = en.kt0; kt < en.kt1; ++kt) {
      __syncthreads();
      stage_one_f32<D>(s.k, Kg, a.ksl, kt * BN, a.Lk, tid);
      stage_one_f32<D>(s.tk, tKg, a.ksl, kt * BN, a.Lk, tid);
      stage_one_f32<D>(s.v, Vg, a.ksl, kt * BN, a.Lk, tid);
      stage_one_f32<D>(s.tv, tVg, a.ksl, kt * BN, a.Lk, tid);
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

template <bool JVP, bool VARIANTS>
static void launch_bf16(const FwdArgs& a, bool out_f32, int head_dim, dim3 grid, hipStream_t stream) {
  const dim3 b32(64 * kWavesQ32);
  if (!JVP && head_dim == 128 && a.tile_m == kTileMWide) {
    // primal forward on the wide map: 8 x 32-row waves, one workgroup per CU
    const dim3 b256(64 * 8);
    if (out_f32) hipLaunchKernelGGL((attn_jvp_fwd_bf16_q32_kernel<128, true, false, false, false, 8>), grid, b256, 0, stream, a);
    else hipLaunchKernelGGL((attn_jvp_fwd_bf16_q32_kernel<128, false, false, false, false, 8>), grid, b256, 0, stream, a);
  } else if (!JVP && head_dim == 128) {
    // primal forward on the row map (the primal-only query tiles of a
    // tangent-free JVP): 4 x 32-row waves, two workgroups per CU
    if (out_f32) hipLaunchKernelGGL((attn_jvp_fwd_bf16_q32_kernel<128, true, false>), grid, b32, 0, stream, a);
    else hipLaunchKernelGGL((attn_jvp_fwd_bf16_q32_kernel<128, false, false>), grid, b32, 0, stream, a);
  } else if (head_dim == 128) {
    launch_q16(a, out_f32, VARIANTS, grid, stream);
  } else {
    // the JVP with a power-of-two scale (1/8 is the usual one at d = 64):
    // the scale folded into Q and tQ
    int e2 = 0;
    const bool pow2 = a.scale > 0.f && a.scale <= 1.f && std::frexp(a.scale, &e2) == 0.5f;
    if constexpr (JVP) {
      if (a.v16) {  // V and tV converted by bf16_to_f16_kv_kernel, launched just before
        if (pow2) {
          if (out_f32)
            hipLaunchKernelGGL((attn_jvp_fwd_bf16_q32_kernel<64, true, true, true, VARIANTS, kWavesQ32, true>), grid, b32,
                               0, stream, a);
          else
            hipLaunchKernelGGL((attn_jvp_fwd_bf16_q32_kernel<64, false, true, true, VARIANTS, kWavesQ32, true>), grid, b32,
                               0, stream, a);
        } else {
          if (out_f32)
            hipLaunchKernelGGL((attn_jvp_fwd_bf16_q32_kernel<64, true, true, false, VARIANTS, kWavesQ32, true>), grid, b32,
                               0, stream, a);
          else
            hipLaunchKernelGGL((attn_jvp_fwd_bf16_q32_kernel<64, false, true, false, VARIANTS, kWavesQ32, true>), grid,
                               b32, 0, stream, a);
        }
        return;
      }
      if (pow2) {
        if (out_f32)
          hipLaunchKernelGGL((attn_jvp_fwd_bf16_q32_kernel<64, true, true, true, VARIANTS>), grid, b32, 0, stream, a);
        else
          hipLaunchKernelGGL((attn_jvp_fwd_bf16_q32_kernel<64, false, true, true, VARIANTS>), grid, b32, 0, stream, a);
        return;
      }
    }
    if (out_f32) hipLaunchKernelGGL((attn_jvp_fwd_bf16_q32_kernel<64, true, JVP, false, VARIANTS>), grid, b32, 0, stream, a);
    else hipLaunchKernelGGL((attn_jvp_fwd_bf16_q32_kernel<64, false, JVP, false, VARIANTS>), grid, b32, 0, stream, a);
  }
}

int launch_fwd(FwdArgs a, int in_dtype, int out_dtype, int head_dim, bool jvp, bool variants,
               hipStream_t stream) {
  const int64_t grid64 = int64_t(a.n_tasks) * a.B * a.H;
  if (grid64 <= 0 || grid64 > 0x7fffffff) return AJ_EINVAL;
  a.head_group = head_group_for(a.B * a.H);
  const dim3 grid((unsigned)grid64);
  if (a.v16 && !(jvp && in_dtype == AJ_BF16 && head_dim == 64)) return AJ_ENOTSUP;
  if (a.v16) {
    // fp16 copies of V and tV for the d = 64 JVP, in stream order before it
    const int64_t threads = 2 * int64_t(a.B) * a.H * a.Lk * (64 / 8);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffff) return AJ_EINVAL;
    hipLaunchKernelGGL(bf16_to_f16_kv_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  }
  if (in_dtype == AJ_BF16) {
    if (!jvp) launch_bf16<false, false>(a, out_dtype == AJ_F32, head_dim, grid, stream);
    else if (variants) launch_bf16<true, true>(a, out_dtype == AJ_F32, head_dim, grid, stream);
    else launch_bf16<true, false>(a, out_dtype == AJ_F32, head_dim, grid, stream);
  } else {
    // fp32 inputs: the JVP only; tangent-free tiles run the general code
    // (their tangents are zero, so every extra product adds zero)
    if (!jvp) return AJ_ENOTSUP;
    const dim3 b_f32(NTHREADS);
    if (head_dim == 128) hipLaunchKernelGGL((attn_jvp_fwd_f32_kernel<128>), grid, b_f32, 0, stream, a);
    else hipLaunchKernelGGL((attn_jvp_fwd_f32_kernel<64>), grid, b_f32, 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? AJ_OK : AJ_EHIP;
}

}  // namespace aj
