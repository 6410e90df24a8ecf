// Gradients of masked attention for gfx950 (MI355X): dQ, dK and dV for a
// cotangent dO, on the mask descriptor of the forward pass.
//
// Training through the packed teacher-forcing forward ("Causal-rCM",
// Sec. 3.1.1, Eq. 8) differentiates one masked attention (Eq. 42).  With the
// forward's lse, P_ij = exp(c <q_i, k_j> - lse_i) on allowed pairs, and
//   D_i = <dO_i, O_i>,  dS_ij = P_ij (<dO_i, v_j> - D_i),
//   dQ_i = c sum_j dS_ij k_j,  dK_j = c sum_i dS_ij q_i,  dV_j = sum_i P_ij dO_i.
//
// Two kernels, no atomics (results are deterministic):
// * dQ (query-parallel, the forward's tile map): a workgroup owns a 128-row
//   query tile and streams its admissible 64-key tiles of K and V.  As in the
//   forward, the scores are computed transposed (S^T = K Q^T, dP^T = V dO^T
//   with Q and dO of the lane's row held as MFMA B operands), so the row
//   statistics lse and D are one value per lane and the dS accumulator feeds
//   dQ^T += K^T dS^T directly, K^T coming from LDS transpose reads.  It also
//   computes and stores D.
// * dK / dV (key-parallel, the transposed tile map): a workgroup owns a tile
//   of 128 keys and streams the admissible 64-query tiles of Q and dO (plus
//   their lse and D).  Here the scores are computed untransposed (S = Q K^T,
//   dP = dO V^T with K and V of the lane's key as B operands): one key per
//   lane column, so P and dS feed dV^T += dO^T P and dK^T += Q^T dS directly,
//   dO^T and Q^T coming from transpose reads.
// dQ runs 4 waves of 32 rows (v_mfma_f32_32x32x16_bf16, two workgroups per
// CU at d = 128, three at d = 64).  dK / dV runs 8 waves of 16 keys at
// d = 128 (v_mfma_f32_16x16x32_bf16, two waves per SIMD) and 4 waves of 32
// keys at d = 64 (v_mfma_f32_32x32x16_bf16, two workgroups per CU).  All use
// the direct buffer -> LDS DMA into a double buffer and the swizzled tile
// layouts of the forward kernels.  The dP chains start from -D, so the MFMAs
// deliver dP - D.  Masked pairs are removed by select (P = dS = 0), never by
// arithmetic on -inf.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "../../include/attn_jvp.h"
#include "aj_device.h"
#include "aj_internal.h"
#include "aj_launch.h"

namespace aj {

constexpr int kDqWaves32 = 4;   // 32-row waves of the dQ kernel
constexpr float kLog2e = 1.44269504088896340736f;

template <int D>
struct BwdLds {
  static constexpr int TILE = BN * D;  // elements per tensor tile
  uint16_t t[2][2][TILE];              // [buffer][(K, V) for dQ | (Q, dO) for dK, dV]
  uint64_t bits[2][BM];                // per-row bitmask of a partial tile
  float rowv[2][2][BN];                // [buffer][lse, D] of the 64 streamed queries
  // byte offsets of t[b][0], bits[b] and rowv[b][i] from the start of the struct
  static constexpr __device__ uint32_t t_off(int b) { return uint32_t(b) * 2 * TILE * 2; }
  static constexpr __device__ uint32_t bits_off(int b) { return 4u * TILE * 2 + uint32_t(b) * BM * 8; }
  static constexpr __device__ uint32_t rowv_off(int b, int i) {
    return 4u * TILE * 2 + 2u * BM * 8 + uint32_t(2 * b + i) * BN * 4;
  }
};

// K and V tiles only (the 32-row dQ kernel): 66 KB at d = 128 (two workgroups
// per CU), 34 KB at d = 64 (three).
template <int D>
struct KvLds {
  static constexpr int TILE = BN * D;
  uint16_t t[2][2][TILE];  // [buffer][K, V]
  uint64_t bits[2][BM];
  static constexpr __device__ uint32_t t_off(int b) { return uint32_t(b) * 2 * TILE * 2; }
  static constexpr __device__ uint32_t bits_off(int b) { return 4u * TILE * 2 + uint32_t(b) * BM * 8; }
};

// One direct buffer -> LDS load of 4 bytes per lane (lane l's dword lands at
// lds_base + 4 l); out-of-range dwords read as zero.  Same rules as lds_dma_16.
__device__ __forceinline__ void lds_dma_4(uint32_t lds_base, uint32_t voffset, i32x4_t rsrc) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(lds_base), "v"(voffset), "s"(rsrc)
      : "memory", "m0");
}

__device__ __forceinline__ float bf16_dot8(bf16x8_t x, bf16x8_t y, float acc) {
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const bf16x2_t a = {x[e], x[e + 1]}, b = {y[e], y[e + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(a, b, acc, false);
  }
  return acc;
}

// ---- dQ (and D) ---------------------------------------------------------------

// dQ with 32-row waves (v_mfma_f32_32x32x16_bf16): 4 waves own the 128-row
// query tile and two workgroups share a CU.  Lanes l and l + 32 hold the same
// query row; S^T, dP^T and dS^T keep the forward q32 kernel's layout, so the
// K^T transpose reads and the slot order of the B operand are the same.
// Two workgroups per CU at d = 128; three at d = 64 (at most 168 VGPRs, 34 KB
// of LDS each).
template <int D, bool OUT_F32>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kDqWaves32, 64 * kDqWaves32),
                          amdgpu_waves_per_eu(D == 64 ? 3 : 2, D == 64 ? 3 : 2)))
void attn_bwd_dq32_kernel(BwdArgs a) {
  constexpr int NKK = D / 16;  // MFMA k-steps over d for S^T and dP^T
  constexpr int NDB = D / 32;  // 32-row blocks of d for dQ^T
  using Lds = KvLds<D>;
  __shared__ __attribute__((aligned(1024))) Lds s;
  static_assert(offsetof(Lds, bits) == Lds::bits_off(0), "LDS layout");
  const uint32_t lds0 = lds_addr(&s);

  const int tid = threadIdx.x, wave = wave_uniform(tid >> 6), lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int BH = a.B * a.H;
  const TaskCoord tc = task_coord(blockIdx.x, a.n_row_tasks, BH, a.head_group);
  const int rank = tc.rank, bh = tc.bh;
  const int bb = bh / a.H, hh = bh - bb * a.H;
  const int qt = wave_uniform(a.rows.tasks[rank]);
  const int L = a.L;
  const int64_t in_off = bb * a.isb + hh * a.ish;
  const int64_t bhL = (int64_t)bh * L;
  const uint16_t* Kg = (const uint16_t*)a.k + in_off;
  const uint16_t* Vg = (const uint16_t*)a.v + in_off;
  const int q_row = qt * BM + wave * 32 + l32;

  // Q, dO of this lane's row as B operands (k-step kk: d = 16kk + 8hi ..),
  // D = <dO, O> and the row's lse
  bf16x8_t Qr[NKK], dOr[NKK];
  float dpart = 0.f;
  {
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    const uint16_t* Qg = (const uint16_t*)a.q + in_off;
    const uint16_t* dOg = (const uint16_t*)a.dout + in_off;
    const uint16_t* Og = (const uint16_t*)a.o + in_off;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int64_t off = q_row * a.isl + kk * 16 + 8 * hi;
      Qr[kk] = as_bf16x8(q_row < L ? *(const u32x4_t*)(Qg + off) : zero);
      dOr[kk] = as_bf16x8(q_row < L ? *(const u32x4_t*)(dOg + off) : zero);
      const bf16x8_t Or = as_bf16x8(q_row < L ? *(const u32x4_t*)(Og + off) : zero);
      dpart = bf16_dot8(dOr[kk], Or, dpart);
    }
  }
  const float lse_l2 = q_row < L ? a.lse[bhL + q_row] * kLog2e : 0.f;
  wait_vmcnt<0>();
  const float delta = dpart + wave_xor32(dpart);
  // dP^T chains start from -D (the lane's row value in all 16 registers), so
  // they deliver dP - D and dS = P (dP - D) takes one multiply per element
  f32x16_t negD;
#pragma unroll
  for (int r = 0; r < 16; ++r) negD[r] = -delta;

  const TileLoadPlan<kDqWaves32, D> plan(a.isl, wave, lane, swz_q32<D>);
  auto prefetch = [&](int b, const Entry& x, int kti) {
    issue_pair_loads<kDqWaves32, D>(lds0 + Lds::t_off(b), plan, Kg, Vg, a.isl, kti * BN, L, wave);
    if (x.pidx >= 0 && wave == 0) issue_bits_load(lds0 + Lds::bits_off(b), a.rows.bits, x.pidx, lane);
  };
  const int e0 = wave_uniform(a.rows.qt_off[qt]), e1 = wave_uniform(a.rows.qt_off[qt + 1]);
  int e = e0, kt = 0;
  Entry en = {0, 0, -1, 0};
  if (e < e1) {
    en = load_entry(a.rows.entries + e);
    kt = en.kt0;
    prefetch(0, en, kt);
  }

  f32x16_t dQacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dQacc[db][r] = 0.f;
  const float sl2 = a.scale_log2;

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
  while (e < e1) {
    int e_n = e, kt_n = kt + 1;
    Entry en_n = en;
    if (kt_n >= en.kt1) {
      e_n = e + 1;
      if (e_n < e1) {
        en_n = load_entry(a.rows.entries + e_n);
        kt_n = en_n.kt0;
      }
    }
    // one barrier per tile (loads landed; other buffer free for the next DMA)
    wait_vmcnt<0>();
    __syncthreads();
    if (e_n < e1) prefetch(buf ^ 1, en_n, kt_n);
    const bool part = en.pidx >= 0;  // uniform: only partial tiles test the row mask
    const uint64_t bits = part ? s.bits[buf][wave * 32 + l32] : ~0ull;
    const uint16_t* Kt = s.t[buf][0];
    const uint16_t* Vt = s.t[buf][1];

#pragma unroll 1
    for (int kb = 0; kb < BN / 32; ++kb) {
      // S^T = K Q^T and dP^T = V dO^T for 32 keys (lane = query)
      f32x16_t S, dP = negD;
#pragma unroll
      for (int r = 0; r < 16; ++r) S[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int off = kb * 32 * D + koff[kk];
        const bf16x8_t kop = as_bf16x8(*(const u32x4_t*)(Kt + off));
        const bf16x8_t vop = as_bf16x8(*(const u32x4_t*)(Vt + off));
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, Qr[kk], S, 0, 0, 0);
        dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, dOr[kk], dP, 0, 0, 0);
      }
      // lane holds keys kb*32 + 8*(r/4) + 4*hi + r%4 of its query row
      bf16x8_t DS[2];
      auto make_ds = [&](auto masked_tag) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int t = 0; t < 8; t += 2) {
            const int r = 8 * st + t;
            const float p0 = fast_exp2(__builtin_fmaf(S[r], sl2, -lse_l2));
            const float p1 = fast_exp2(__builtin_fmaf(S[r + 1], sl2, -lse_l2));
            f32x2_t ds;
            ds.x = p0 * dP[r];
            ds.y = p1 * dP[r + 1];
            if constexpr (MASKED) {
              const int key0 = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
              ds.x = (bits >> key0) & 1ull ? ds.x : 0.f;
              ds.y = (bits >> (key0 + 1)) & 1ull ? ds.y : 0.f;
            }
            const bf16x2_t d2 = __builtin_convertvector(ds, bf16x2_t);
            DS[st][t] = d2.x;
            DS[st][t + 1] = d2.y;
          }
      };
      if (part) make_ds(std::true_type{});
      else make_ds(std::false_type{});
      // dQ^T += K^T dS^T (rows = d, columns = queries)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int off_a = (kb * 32 + 16 * st) * D + voff[0][db];
          const int off_b = (kb * 32 + 16 * st) * D + voff[1][db];
          const s16x4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(Kt + off_a));
          const s16x4_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(Kt + off_b));
          const bf16x8_t top = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
          dQacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(top, DS[st], dQacc[db], 0, 0, 0);
        }
      }
    }
    e = e_n;
    kt = kt_n;
    en = en_n;
    buf ^= 1;
  }

  if (q_row < L) {
    const float c = a.scale;
    const int64_t out_off = bb * a.osb + hh * a.osh + q_row * a.osl;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = db * 32 + 8 * gq + 4 * hi;
        f32x4_t v;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) v[jj] = dQacc[db][4 * gq + jj] * c;
        if constexpr (OUT_F32) *(f32x4_t*)((float*)a.dq + out_off + d0) = v;
        else *(bf16x4_t*)((__bf16*)a.dq + out_off + d0) = __builtin_convertvector(v, bf16x4_t);
      }
    if (hi == 0) a.delta[bhL + q_row] = delta;
  }
}

// ---- dK, dV -------------------------------------------------------------------

// Waves of 16 keys, 8 per workgroup (one 128-key tile of the column map, two
// waves per SIMD); head_dim 128.  Head_dim 64 runs the 32-key kernel below.
template <int D>
constexpr int dkdv_waves() { return 8; }

template <int D, bool OUT_F32>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * dkdv_waves<D>(), 64 * dkdv_waves<D>()),
                          amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv_kernel(BwdArgs a) {
  static_assert(D == 128, "16-key dK / dV waves are built for head_dim 128");
  constexpr int NKS = D / 32;
  constexpr int NDB = D / 16;
  constexpr int NW = dkdv_waves<D>();
  constexpr int PARTS = BM / (16 * NW);  // workgroups per column-map tile
  using Lds = BwdLds<D>;
  __shared__ __attribute__((aligned(1024))) Lds s;
  static_assert(offsetof(Lds, bits) == Lds::bits_off(0) && offsetof(Lds, rowv) == Lds::rowv_off(0, 0), "LDS layout");
  const uint32_t lds0 = lds_addr(&s);

  const int tid = threadIdx.x, wave = wave_uniform(tid >> 6), lane = tid & 63, j16 = lane & 15, g = lane >> 4;
  const int BH = a.B * a.H;
  const TaskCoord tc = task_coord(blockIdx.x, a.n_col_tasks * PARTS, BH, a.head_group);
  const int rank = tc.rank / PARTS, kpart = tc.rank - rank * PARTS, bh = tc.bh;
  const int bb = bh / a.H, hh = bh - bb * a.H;
  const int ktile = wave_uniform(a.cols.tasks[rank]);
  const int key_in_tile = kpart * 16 * NW + wave * 16 + j16;  // row of the tile's bitmask
  const int L = a.L;
  const int64_t in_off = bb * a.isb + hh * a.ish;
  const int64_t bhL = (int64_t)bh * L;
  const uint16_t* Qg = (const uint16_t*)a.q + in_off;
  const uint16_t* dOg = (const uint16_t*)a.dout + in_off;
  const int k_row = ktile * BM + key_in_tile;

  // K, V of this lane's key as B operands (k-step ks: d = 32ks + 8g ..)
  bf16x8_t Kr[NKS], Vr[NKS];
  {
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    const uint16_t* Kg = (const uint16_t*)a.k + in_off;
    const uint16_t* Vg = (const uint16_t*)a.v + in_off;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int64_t off = k_row * a.isl + ks * 32 + 8 * g;
      Kr[ks] = as_bf16x8(k_row < L ? *(const u32x4_t*)(Kg + off) : zero);
      Vr[ks] = as_bf16x8(k_row < L ? *(const u32x4_t*)(Vg + off) : zero);
    }
  }
  wait_vmcnt<0>();

  const TileLoadPlan<NW, D> plan(a.isl, wave, lane, swz_q16<D>);
  // Q, dO rows of query tile qti; wave 1 brings their lse and D, wave 0 the
  // key bitmasks of a partial tile
  auto prefetch = [&](int b, const Entry& x, int qti) {
    const int row0 = qti * BN;
    issue_pair_loads<NW, D>(lds0 + Lds::t_off(b), plan, Qg, dOg, a.isl, row0, L, wave);
    if (wave == 1) {
      const int nrec = min(L - row0, BN) * 4;
      lds_dma_4(lds0 + Lds::rowv_off(b, 0), uint32_t(lane) * 4u, make_rsrc(a.lse + bhL + row0, nrec));
      lds_dma_4(lds0 + Lds::rowv_off(b, 1), uint32_t(lane) * 4u, make_rsrc(a.delta + bhL + row0, nrec));
    }
    if (x.pidx >= 0 && wave == 0) issue_bits_load(lds0 + Lds::bits_off(b), a.cols.bits, x.pidx, lane);
  };
  const int e0 = wave_uniform(a.cols.qt_off[ktile]), e1 = wave_uniform(a.cols.qt_off[ktile + 1]);
  int e = e0, qtl = 0;
  Entry en = {0, 0, -1, 0};
  if (e < e1) {
    en = load_entry(a.cols.entries + e);
    qtl = en.kt0;
    prefetch(0, en, qtl);
  }

  f32x4_t dKacc[NDB], dVacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) dKacc[db][r] = dVacc[db][r] = 0.f;
  const float sl2 = a.scale_log2;

  int koff[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) koff[ks] = j16 * D + (((4 * ks + g) ^ swz_q16<D>(j16)) << 3);
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
  while (e < e1) {
    int e_n = e, qt_n = qtl + 1;
    Entry en_n = en;
    if (qt_n >= en.kt1) {
      e_n = e + 1;
      if (e_n < e1) {
        en_n = load_entry(a.cols.entries + e_n);
        qt_n = en_n.kt0;
      }
    }
    // one barrier per tile (loads landed; other buffer free for the next DMA).
    // Wave 1 brought the tile's 64 lse and D values, one of each per lane: it
    // takes lse to log2 units and negates D in place before the barrier
    // publishes them, once per query instead of once per (query, key) element
    // below; the dP chains start from -D and deliver dP - D.
    wait_vmcnt<0>();
    if (wave == 1) {
      s.rowv[buf][0][lane] *= kLog2e;
      s.rowv[buf][1][lane] = -s.rowv[buf][1][lane];
    }
    __syncthreads();
    if (e_n < e1) prefetch(buf ^ 1, en_n, qt_n);
    const uint16_t* Qt = s.t[buf][0];
    const uint16_t* dOt = s.t[buf][1];

    // S = Q K^T and dP = dO V^T for the 64 queries of the tile (16-query
    // blocks qb; lane holds queries 16qb + 4g + r of key j16)
    f32x4_t S[4], dP[4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      dP[qb] = *(const f32x4_t*)(&s.rowv[buf][1][16 * qb + 4 * g]);  // -D of the lane's queries
#pragma unroll
      for (int r = 0; r < 4; ++r) S[qb][r] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8_t qop[4], dop[4];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const int off = qb * 16 * D + koff[ks];
        qop[qb] = as_bf16x8(*(const u32x4_t*)(Qt + off));
        dop[qb] = as_bf16x8(*(const u32x4_t*)(dOt + off));
      }
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) S[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qop[qb], Kr[ks], S[qb], 0, 0, 0);
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
        dP[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(dop[qb], Vr[ks], dP[qb], 0, 0, 0);
    }

    const bool part = en.pidx >= 0;  // uniform: only partial tiles test the row mask
    const uint64_t bits = part ? s.bits[buf][key_in_tile] >> (4 * g) : ~0ull;
    bf16x8_t P[2], DS[2];
    auto make_p_ds = [&](auto masked_tag) __attribute__((always_inline)) {
      constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const f32x4_t lse4 = *(const f32x4_t*)(&s.rowv[buf][0][16 * qb + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          f32x2_t pv, ds;
          pv.x = fast_exp2(__builtin_fmaf(S[qb][r], sl2, -lse4[r]));
          pv.y = fast_exp2(__builtin_fmaf(S[qb][r + 1], sl2, -lse4[r + 1]));
          if constexpr (MASKED) {
            pv.x = (bits >> (16 * qb + r)) & 1ull ? pv.x : 0.f;
            pv.y = (bits >> (16 * qb + r + 1)) & 1ull ? pv.y : 0.f;
          }
          ds.x = pv.x * dP[qb][r];
          ds.y = pv.y * dP[qb][r + 1];
          const bf16x2_t pb = __builtin_convertvector(pv, bf16x2_t);
          const bf16x2_t db2 = __builtin_convertvector(ds, bf16x2_t);
          const int slot = 4 * (qb & 1) + r;
          P[qb >> 1][slot] = pb.x;
          P[qb >> 1][slot + 1] = pb.y;
          DS[qb >> 1][slot] = db2.x;
          DS[qb >> 1][slot + 1] = db2.y;
        }
      }
    };
    if (part) make_p_ds(std::true_type{});
    else make_p_ds(std::false_type{});

    // dV^T += dO^T P and dK^T += Q^T dS (rows = d, columns = keys)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
#pragma unroll
      for (int d4 = 0; d4 < NDB; d4 += 4) {
        bf16x8_t oop[4], qtop[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int off_a = 32 * p * D + voff[d4 + i];
          const int off_b = off_a + 16 * D;
          const s16x4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(dOt + off_a));
          const s16x4_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(dOt + off_b));
          const s16x4_t y0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(Qt + off_a));
          const s16x4_t y1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(Qt + off_b));
          oop[i] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
          qtop[i] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(y0, y1, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dVacc[d4 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oop[i], P[p], dVacc[d4 + i], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dKacc[d4 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qtop[i], DS[p], dKacc[d4 + i], 0, 0, 0);
      }
    }
    e = e_n;
    qtl = qt_n;
    en = en_n;
    buf ^= 1;
  }

  const int ge = int(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u))) >> 4;
  if (k_row < L) {
    const float c = a.scale;
    const int64_t out_off = bb * a.osb + hh * a.osh + k_row * a.osl;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d0 = db * 16 + 4 * ge;
      f32x4_t kv, vv;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        kv[r] = dKacc[db][r] * c;
        vv[r] = dVacc[db][r];
      }
      if constexpr (OUT_F32) {
        *(f32x4_t*)((float*)a.dk + out_off + d0) = kv;
        *(f32x4_t*)((float*)a.dv + out_off + d0) = vv;
      } else {
        *(bf16x4_t*)((__bf16*)a.dk + out_off + d0) = __builtin_convertvector(kv, bf16x4_t);
        *(bf16x4_t*)((__bf16*)a.dv + out_off + d0) = __builtin_convertvector(vv, bf16x4_t);
      }
    }
  }
}

// ---- dK, dV with 32-key waves (head_dim 64) ------------------------------------
//
// The dQ kernel's shape with the roles of queries and keys exchanged: a
// workgroup of 4 waves owns one 128-key tile of the column map, each wave 32
// keys, lanes l and l + 32 sharing a key.  K and V of the lane's key are held
// as MFMA B operands; the 64-query tiles of Q and dO (plus their lse and D)
// stream through LDS.  With v_mfma_f32_32x32x16_bf16
//   S = Q K^T,  dP = dO V^T      (rows = queries, columns = keys)
// put one key per lane column; the accumulator registers are the B operand of
//   dV^T += dO^T P,  dK^T += Q^T dS
// with dO^T and Q^T from LDS transpose reads, the same k-slot order as the dQ
// kernel's K^T.  Against the 16-key waves every Q / dO operand read from LDS
// serves twice the keys: half the LDS bytes per FLOP, which bound the 16-key
// kernel at d = 64 (LDS busy 60 %); the register state (about 200 VGPRs) fits
// two waves per SIMD.  At d = 128 it would need about 300 registers.
template <int D, bool OUT_F32>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * kDqWaves32, 64 * kDqWaves32), amdgpu_waves_per_eu(2, 2)))
void attn_bwd_dkdv32_kernel(BwdArgs a) {
  static_assert(D == 64, "32-key dK / dV waves are built for head_dim 64");
  constexpr int NKK = D / 16;  // MFMA k-steps over d for S and dP
  constexpr int NDB = D / 32;  // 32-row blocks of d for dK^T and dV^T
  using Lds = BwdLds<D>;
  __shared__ __attribute__((aligned(1024))) Lds s;
  static_assert(offsetof(Lds, bits) == Lds::bits_off(0) && offsetof(Lds, rowv) == Lds::rowv_off(0, 0), "LDS layout");
  const uint32_t lds0 = lds_addr(&s);

  const int tid = threadIdx.x, wave = wave_uniform(tid >> 6), lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int BH = a.B * a.H;
  const TaskCoord tc = task_coord(blockIdx.x, a.n_col_tasks, BH, a.head_group);
  const int rank = tc.rank, bh = tc.bh;
  const int bb = bh / a.H, hh = bh - bb * a.H;
  const int ktile = wave_uniform(a.cols.tasks[rank]);
  const int key_in_tile = wave * 32 + l32;  // row of the tile's bitmask
  const int L = a.L;
  const int64_t in_off = bb * a.isb + hh * a.ish;
  const int64_t bhL = (int64_t)bh * L;
  const uint16_t* Qg = (const uint16_t*)a.q + in_off;
  const uint16_t* dOg = (const uint16_t*)a.dout + in_off;
  const int k_row = ktile * BM + key_in_tile;

  // K, V of this lane's key as B operands (k-step kk: d = 16kk + 8hi ..)
  bf16x8_t Kr[NKK], Vr[NKK];
  {
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    const uint16_t* Kg = (const uint16_t*)a.k + in_off;
    const uint16_t* Vg = (const uint16_t*)a.v + in_off;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int64_t off = k_row * a.isl + kk * 16 + 8 * hi;
      Kr[kk] = as_bf16x8(k_row < L ? *(const u32x4_t*)(Kg + off) : zero);
      Vr[kk] = as_bf16x8(k_row < L ? *(const u32x4_t*)(Vg + off) : zero);
    }
  }
  wait_vmcnt<0>();

  const TileLoadPlan<kDqWaves32, D> plan(a.isl, wave, lane, swz_q32<D>);
  // Q, dO rows of query tile qti; wave 1 brings their lse and D, wave 0 the
  // key bitmasks of a partial tile
  auto prefetch = [&](int b, const Entry& x, int qti) {
    const int row0 = qti * BN;
    issue_pair_loads<kDqWaves32, D>(lds0 + Lds::t_off(b), plan, Qg, dOg, a.isl, row0, L, wave);
    if (wave == 1) {
      const int nrec = min(L - row0, BN) * 4;
      lds_dma_4(lds0 + Lds::rowv_off(b, 0), uint32_t(lane) * 4u, make_rsrc(a.lse + bhL + row0, nrec));
      lds_dma_4(lds0 + Lds::rowv_off(b, 1), uint32_t(lane) * 4u, make_rsrc(a.delta + bhL + row0, nrec));
    }
    if (x.pidx >= 0 && wave == 0) issue_bits_load(lds0 + Lds::bits_off(b), a.cols.bits, x.pidx, lane);
  };
  const int e0 = wave_uniform(a.cols.qt_off[ktile]), e1 = wave_uniform(a.cols.qt_off[ktile + 1]);
  int e = e0, qtl = 0;
  Entry en = {0, 0, -1, 0};
  if (e < e1) {
    en = load_entry(a.cols.entries + e);
    qtl = en.kt0;
    prefetch(0, en, qtl);
  }

  f32x16_t dKacc[NDB], dVacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dKacc[db][r] = dVacc[db][r] = 0.f;
  const float sl2 = a.scale_log2;

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
  while (e < e1) {
    int e_n = e, qt_n = qtl + 1;
    Entry en_n = en;
    if (qt_n >= en.kt1) {
      e_n = e + 1;
      if (e_n < e1) {
        en_n = load_entry(a.cols.entries + e_n);
        qt_n = en_n.kt0;
      }
    }
    // one barrier per tile (loads landed; other buffer free for the next DMA).
    // Wave 1 brought the tile's 64 lse and D values, one of each per lane: it
    // takes lse to log2 units and negates D in place before the barrier
    // publishes them, once per query instead of once per (query, key) element
    // below; the dP chains start from -D and deliver dP - D.
    wait_vmcnt<0>();
    if (wave == 1) {
      s.rowv[buf][0][lane] *= kLog2e;
      s.rowv[buf][1][lane] = -s.rowv[buf][1][lane];
    }
    __syncthreads();
    if (e_n < e1) prefetch(buf ^ 1, en_n, qt_n);
    const bool part = en.pidx >= 0;  // uniform: only partial tiles test the row mask
    const uint64_t bits = part ? s.bits[buf][key_in_tile] : ~0ull;
    const uint16_t* Qt = s.t[buf][0];
    const uint16_t* dOt = s.t[buf][1];

#pragma unroll 1
    for (int qb = 0; qb < BN / 32; ++qb) {
      // S = Q K^T and dP = dO V^T for 32 queries (lane = key)
      // dP starts from -D of the lane's queries qb*32 + 8*(r/4) + 4*hi + r%4
      f32x16_t S, dP;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x4_t nd4 = *(const f32x4_t*)(&s.rowv[buf][1][qb * 32 + 8 * i + 4 * hi]);
#pragma unroll
        for (int t = 0; t < 4; ++t) dP[4 * i + t] = nd4[t];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) S[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int off = qb * 32 * D + koff[kk];
        const bf16x8_t qop = as_bf16x8(*(const u32x4_t*)(Qt + off));
        const bf16x8_t dop = as_bf16x8(*(const u32x4_t*)(dOt + off));
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qop, Kr[kk], S, 0, 0, 0);
        dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dop, Vr[kk], dP, 0, 0, 0);
      }
      // lane holds queries qb*32 + 8*(r/4) + 4*hi + r%4 of its key; their
      // lse come from LDS, four consecutive queries per read
      bf16x8_t P[2], DS[2];
      auto make_p_ds = [&](auto masked_tag) __attribute__((always_inline)) {
        constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int q0 = qb * 32 + 8 * i + 4 * hi;
          const f32x4_t lse4 = *(const f32x4_t*)(&s.rowv[buf][0][q0]);
#pragma unroll
          for (int t = 0; t < 4; t += 2) {
            const int r = 4 * i + t;
            f32x2_t pv, ds;
            pv.x = fast_exp2(__builtin_fmaf(S[r], sl2, -lse4[t]));
            pv.y = fast_exp2(__builtin_fmaf(S[r + 1], sl2, -lse4[t + 1]));
            if constexpr (MASKED) {
              pv.x = (bits >> (q0 + t)) & 1ull ? pv.x : 0.f;
              pv.y = (bits >> (q0 + t + 1)) & 1ull ? pv.y : 0.f;
            }
            ds.x = pv.x * dP[r];
            ds.y = pv.y * dP[r + 1];
            const bf16x2_t pb = __builtin_convertvector(pv, bf16x2_t);
            const bf16x2_t d2 = __builtin_convertvector(ds, bf16x2_t);
            // value step st = i / 2 takes rows 16 st .. 16 st + 15, slots 4 (i % 2) + t
            const int st = i >> 1, slot = 4 * (i & 1) + t;
            P[st][slot] = pb.x;
            P[st][slot + 1] = pb.y;
            DS[st][slot] = d2.x;
            DS[st][slot + 1] = d2.y;
          }
        }
      };
      if (part) make_p_ds(std::true_type{});
      else make_p_ds(std::false_type{});
      // dV^T += dO^T P and dK^T += Q^T dS (rows = d, columns = keys)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int off_a = (qb * 32 + 16 * st) * D + voff[0][db];
          const int off_b = (qb * 32 + 16 * st) * D + voff[1][db];
          const s16x4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(dOt + off_a));
          const s16x4_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(dOt + off_b));
          const s16x4_t y0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(Qt + off_a));
          const s16x4_t y1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(Qt + off_b));
          const bf16x8_t oop = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
          const bf16x8_t qtop = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(y0, y1, 0, 1, 2, 3, 4, 5, 6, 7));
          dVacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oop, P[st], dVacc[db], 0, 0, 0);
          dKacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qtop, DS[st], dKacc[db], 0, 0, 0);
        }
      }
    }
    e = e_n;
    qtl = qt_n;
    en = en_n;
    buf ^= 1;
  }

  if (k_row < L) {
    const float c = a.scale;
    const int64_t out_off = bb * a.osb + hh * a.osh + k_row * a.osl;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = db * 32 + 8 * gq + 4 * hi;
        f32x4_t kv, vv;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          kv[jj] = dKacc[db][4 * gq + jj] * c;
          vv[jj] = dVacc[db][4 * gq + jj];
        }
        if constexpr (OUT_F32) {
          *(f32x4_t*)((float*)a.dk + out_off + d0) = kv;
          *(f32x4_t*)((float*)a.dv + out_off + d0) = vv;
        } else {
          *(bf16x4_t*)((__bf16*)a.dk + out_off + d0) = __builtin_convertvector(kv, bf16x4_t);
          *(bf16x4_t*)((__bf16*)a.dv + out_off + d0) = __builtin_convertvector(vv, bf16x4_t);
        }
      }
  }
}

// ---------------------------------------------------------------------------

template <int D, bool OUT_F32>
static void launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
  constexpr int NW = dkdv_waves<D>();
  hipLaunchKernelGGL((attn_bwd_dq32_kernel<D, OUT_F32>), dim3(unsigned(int64_t(a.n_row_tasks) * a.B * a.H)),
                     dim3(64 * kDqWaves32), 0, stream, a);
  if constexpr (D == 64) {
    hipLaunchKernelGGL((attn_bwd_dkdv32_kernel<D, OUT_F32>), dim3(unsigned(int64_t(a.n_col_tasks) * a.B * a.H)),
                       dim3(64 * kDqWaves32), 0, stream, a);
  } else {
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, OUT_F32>),
                       dim3(unsigned(int64_t(a.n_col_tasks) * (BM / (16 * NW)) * a.B * a.H)), dim3(64 * NW), 0,
                       stream, a);
  }
}

int launch_bwd(BwdArgs a, int out_dtype, int head_dim, hipStream_t stream) {
  // key-parallel workgroups per column-map tile: one 4 x 32-key workgroup at
  // d = 64, one 8 x 16-key workgroup at 128
  const int64_t parts = head_dim == 64 ? 1 : BM / (16 * dkdv_waves<128>());
  const int64_t g1 = int64_t(a.n_row_tasks) * a.B * a.H, g2 = int64_t(a.n_col_tasks) * parts * a.B * a.H;
  if (g1 <= 0 || g2 <= 0 || g1 > 0x7fffffff || g2 > 0x7fffffff) return AJ_EINVAL;
  a.head_group = head_group_for(a.B * a.H);
  const bool f32 = out_dtype == AJ_F32;
  if (head_dim == 128) {
    if (f32) launch_bwd_d<128, true>(a, stream);
    else launch_bwd_d<128, false>(a, stream);
  } else {
    if (f32) launch_bwd_d<64, true>(a, stream);
    else launch_bwd_d<64, false>(a, stream);
  }
  return hipGetLastError() == hipSuccess ? AJ_OK : AJ_EHIP;
}

// Row statistic D of the gradient kernels for attn_bwd_noalloc, which takes
// no workspace argument: written by the dQ kernel, read by the dK / dV kernel
// of the same call.  One array per GPU for the life of the process; every
// attn_bwd_noalloc call on a GPU uses it, so calls that overlap on one GPU
// race.  Nothing in it needs clearing: each call writes every entry it reads
// before reading it.  Host code never names the array itself (its host-side
// name is not a device address): it uses the address bwd_scratch returns.
static __device__ __align__(256) float scratch[kBwdScratchFloats];

int bwd_scratch(float** out) {
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return AJ_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return AJ_ENOTSUP;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return AJ_EHIP;
    addr[dev] = static_cast<float*>(p);
  }
  *out = addr[dev];
  return AJ_OK;
}

}  // namespace aj
