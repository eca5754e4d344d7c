// fa_launch.hpp -- host-side launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Block-level flags of a key-padding mask, per batch element b and 64-key
// tile t (built by launch_mask_tiles): words[b*T + t] has bit j set iff key
// 64t + j exists and is visible; prefix[b*(T+1) + t] counts the non-empty
// tiles before t; list[b*T + i] is the i-th non-empty tile.
struct MaskTiles {
  const uint64_t* words;
  const int* prefix;
  const int* list;
  int n_tiles;  // T = ceil(N / 64)
};

// Grouped heads: query head bh = b*H + h reads K/V head b*Hkv + h/G, with
// G = H / Hkv, i.e. K/V head bh / G.  Kernels number the query heads of a
// launch so that the G heads sharing K/V are NG = B*Hkv apart: slot s is
// query head (s % NG) * G + s / NG (the identity when G = 1).  With NG a
// multiple of 8 every group then lands on one XCD and shares its L2.
__host__ __device__ inline int head_of_slot(int s, int BH, int G) {
  const int NG = BH / G;
  return (s % NG) * G + s / NG;
}

// Dropout (dropout mode only): Philox4x64-10 key (seed, 0), counter offset,
// threshold floor(p * 65536) and keep scale 65536 / (65536 - thr).
struct DropoutArgs {
  uint64_t seed;
  uint64_t offset;
  uint32_t thr;
  float keep_scale;
};

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int64_t N;
  int BH;          // B * H (query heads)
  int H, Hkv;      // query heads and K/V heads per batch element; Hkv divides H
  int n_qtiles;    // ceil(N / queries per workgroup), filled in by the launcher
  float scale_log2;  // scale * log2(e)
  // Split-K/V mode only: number of key ranges and the FP32 partial states,
  // part_lse [n_splits][B*H*N] and part_o [n_splits][B*H*N][D].
  int n_splits;
  float* part_lse;
  float* part_o;
  MaskTiles mask;  // key-padding mask mode only
  DropoutArgs drop;
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const float* lse;
  const uint16_t* dout;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;      // workspace: [B*H*N] FP32
  int64_t N;
  int BH;            // B * H (query heads)
  int H, Hkv;        // query heads and K/V heads per batch element; Hkv divides H
  float scale;       // the caller's scale (for dQ, dK)
  float scale_log2;  // scale * log2(e)
  MaskTiles mask;    // key-padding mask mode only
  DropoutArgs drop;  // dropout mode only
  // Parts of the dK/dV pass: the (query head, query tile) positions a
  // workgroup walks -- all query tiles of the G query heads that read its K/V
  // head -- are split into head_parts contiguous ranges; with more than one,
  // each part writes FP32 partial dK, dV [head_parts][B*Hkv][N][D] (dK not yet
  // scaled) and a reduce kernel sums them in part order.
  int head_parts;
  float* part_dk;
  float* part_dv;
  // Parts of the dQ pass: the key tiles a workgroup walks are split into
  // dq_parts contiguous ranges; with more than one, each part writes FP32
  // partial dQ [dq_parts][B*H][N][D] (not yet scaled), summed in part order.
  int dq_parts;
  float* part_dq;
};

// Number of parts of the dK/dV pass: 1 when one workgroup per (K/V head,
// 128 keys) already gives kWantWorkgroups, else enough parts to get there --
// few K/V heads (MQA, or few heads of a long sequence) would otherwise leave
// most of the 256 CUs idle -- but no more than one query head per part or
// 8 query tiles (512 queries) per part on average, whichever allows more.
constexpr int64_t kWantWorkgroups = 1024;
inline int bwd_head_parts(int64_t B, int64_t H, int64_t Hkv, int64_t N) {
  const int64_t G = H / Hkv;
  const int64_t wgs = B * Hkv * ((N + 127) / 128);
  if (wgs >= kWantWorkgroups) return 1;
  const int64_t parts = (kWantWorkgroups + wgs - 1) / wgs;
  const int64_t by_tiles = G * ((N + 63) / 64) / 8;
  const int64_t cap = by_tiles > G ? by_tiles : G;
  return (int)(parts < cap ? parts : cap);
}

// Number of key-range parts for the dQ pass (one workgroup per 128 queries):
// the same target, at most one part per 8 key tiles (512 keys).
inline int bwd_dq_parts(int64_t B, int64_t H, int64_t N) {
  const int64_t wgs = B * H * ((N + 127) / 128);
  if (wgs >= kWantWorkgroups) return 1;
  const int64_t parts = (kWantWorkgroups + wgs - 1) / wgs;
  const int64_t cap = ((N + 63) / 64) / 8;
  return (int)(parts < cap ? parts : (cap > 1 ? cap : 1));
}

// Argument checks of the backward entry points other than the workspace:
// FA_OK or an fa_status code (defined with the C ABI).
int check_bwd_args(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t D,
                   int causal, float scale, int dtype);

// The kernel launch_fwd runs for B*H heads of N queries at head size D:
// the key-split kernel (fa_fwd_short.hip), the 64-queries-per-wave kernel
// (fa_fwd_d128.hip) or the 128-query kernel (fa_fwd.hip).
enum class FwdPath { kShort, kD128, kTiled };
FwdPath fwd_path(int64_t BH, int64_t N, int64_t D, bool causal);
// Within the key-split path: D = 128 from N = 1024 on runs the software-
// pipelined variant (fwd_short_pipe_kernel), shorter or D = 64 the plain one.
inline bool short_pipelined(int64_t N, int64_t D) { return D == 128 && N >= 1024; }
hipError_t launch_fwd(const FwdArgs& a, int D, bool causal, int dtype, hipStream_t stream);
// The forward at D = 128 with 64 queries per wave (fa_fwd_d128.hip).
hipError_t launch_fwd_d128(const FwdArgs& a, bool causal, int dtype, hipStream_t stream);
// The forward for small launches: 32 queries per workgroup, keys split over
// its four waves (fa_fwd_short.hip).
hipError_t launch_fwd_short(const FwdArgs& a, int D, bool causal, int dtype, hipStream_t stream);
hipError_t launch_fwd_splitkv(const FwdArgs& a, int D, bool causal, int dtype, hipStream_t stream);
hipError_t launch_bwd(const BwdArgs& a, int D, bool causal, int dtype, hipStream_t stream);
hipError_t launch_fwd_masked(const FwdArgs& a, int D, bool causal, int dtype, hipStream_t stream);
hipError_t launch_bwd_masked(const BwdArgs& a, int D, bool causal, int dtype, hipStream_t stream);
hipError_t launch_fwd_dropout(const FwdArgs& a, int D, bool causal, int dtype, hipStream_t stream);
hipError_t launch_bwd_dropout(const BwdArgs& a, int D, bool causal, int dtype, hipStream_t stream);
hipError_t launch_fwd_masked_dropout(const FwdArgs& a, int D, bool causal, int dtype, hipStream_t stream);
hipError_t launch_fwd_splitkv_dropout(const FwdArgs& a, int D, bool causal, int dtype, hipStream_t stream);
hipError_t launch_fwd_splitkv_masked(const FwdArgs& a, int D, bool causal, int dtype, hipStream_t stream);
hipError_t launch_fwd_splitkv_masked_dropout(const FwdArgs& a, int D, bool causal, int dtype, hipStream_t stream);
hipError_t launch_bwd_masked_dropout(const BwdArgs& a, int D, bool causal, int dtype, hipStream_t stream);
// keep[b][h][i][j] (bytes, 1 = kept) of the dropout mask, for tests.
hipError_t launch_dropout_mask(uint8_t* keep, int64_t BH, int64_t N, const DropoutArgs& d, hipStream_t stream);
// Builds the MaskTiles sections (words, prefix, list) from a [B, N] byte mask.
hipError_t launch_mask_tiles(const uint8_t* key_mask, int64_t B, int64_t N, uint64_t* words, int* prefix, int* list,
                             hipStream_t stream);

}  // namespace fa
