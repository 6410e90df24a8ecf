// Kernel launch arguments and the launcher shared by the C ABI and the HIP
// kernels.  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "aj_tiles.h"

namespace aj {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* tq;
  const void* tk;
  const void* tv;
  void* o;
  void* to;
  float* lse;
  int64_t isb, ish, isl;  // query (and tangent) strides (elements)
  int64_t ksb, ksh, ksl;  // key / value strides (elements)
  int64_t osb, osh, osl;  // output strides (elements)
  int32_t B, H, L, n_tasks;
  int32_t Lk;             // key length (= L except for the KV-cache forward)
  int32_t head_group;     // heads whose workgroups are interleaved (set by launch_fwd)
  float scale;       // softmax scale c
  float scale_log2;  // c * log2(e)
  const int32_t* qt_off;
  const Entry* entries;
  const int32_t* tasks;
  const uint64_t* bits;
  int32_t tile_m;  // query rows per task: kTileM, or kTileMWide (the primal forward's wide map)
  // the JVP at d = 64 only: caller-owned buffers with the key strides that
  // receive fp16 copies of v and tv before the kernel reads them; null: the
  // kernel converts each key tile in LDS
  void* v16;
  void* tv16;
};

// Arguments of the gradient kernels (bf16 inputs [B, H, L, D] sharing the
// input strides; dq, dk, dv sharing the output strides; lse and delta
// contiguous [B, H, L] float32).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* delta;  // written by the dQ kernel, read by the dK / dV kernel
  void* dq;
  void* dk;
  void* dv;
  int64_t isb, ish, isl;
  int64_t osb, osh, osl;
  int32_t B, H, L, n_row_tasks, n_col_tasks;
  int32_t head_group;  // set by launch_bwd
  float scale;
  float scale_log2;
  DeviceMap rows;  // query tiles -> key-tile runs
  DeviceMap cols;  // key tiles -> query-tile runs
};

// Number of heads whose workgroups are interleaved (the grouping of
// task_coord): one head per XCD.  Each XCD then runs 32 (q16) or 64 (q32)
// query tiles of one head at a time, taken longest-first, so tiles of equal
// key range start together and stream the same key tiles through that XCD's
// L2 at about the same time.  Smaller groups leave a tail: the last group's
// longest tiles start late.
constexpr int32_t kHeadGroup = 8;
inline int32_t head_group_for(int32_t BH) { return BH < kHeadGroup ? BH : kHeadGroup; }

// Enqueues the dQ kernel and then the dK / dV kernel on `stream`.
int launch_bwd(BwdArgs a, int out_dtype, int head_dim, hipStream_t stream);

// Enqueues the 16-row JVP kernel at head_dim 128 (attn_jvp_fwd.hip); the
// variants instance when the descriptor declares tangent-free tiles.
void launch_q16(const FwdArgs& a, bool out_f32, bool variants, dim3 grid, hipStream_t stream);

// Enqueues the forward kernel; returns an aj_status.  jvp = false computes
// only O and lse (tq, tk, tv and to are not used).  variants = true when the
// descriptor declares tangent-free tiles: the kernel instance that skips
// their zero products runs instead of the plain one.  a.v16 non-null (the
// bf16 JVP at head_dim 64 only, else AJ_ENOTSUP): a conversion kernel first
// writes fp16 copies of v and tv to a.v16 and a.tv16, which the JVP kernel
// then reads instead of converting every key tile in LDS.
int launch_fwd(FwdArgs a, int in_dtype, int out_dtype, int head_dim, bool jvp, bool variants,
               hipStream_t stream);

}  // namespace aj
