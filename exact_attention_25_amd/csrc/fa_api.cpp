// fa_api.cpp -- the C ABI declared in include/fa.h: argument checks, then
// dispatch to the template instance for (D, causal, dtype) on the caller's
// stream.  Every check runs before anything is enqueued, so a rejected call
// leaves the stream untouched.
#include "fa.h"

#include <hip/hip_runtime.h>
#include <math.h>

#include "fa_launch.hpp"

namespace {

constexpr int64_t kMaxWorkgroups = (int64_t(1) << 31) - 1;
constexpr int64_t kMaxN = int64_t(1) << 30;  // row indices inside a head are 32-bit in the kernels
constexpr int kMaxSplits = 64;
// Smallest scale: the backward keeps -LSE/scale in FP32, which must stay
// finite for |LSE| up to ~2^40.
constexpr float kMinScale = 0x1p-64f;
constexpr float kLog2e = 1.4426950408889634f;

size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_common(int64_t B, int64_t H, int64_t N, int64_t D, int causal, float scale, int dtype) {
  if (B <= 0 || H <= 0 || N <= 0 || N > kMaxN) return FA_ERR_SHAPE;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  if (dtype != FA_FP16 && dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return FA_ERR_UNSUPPORTED;
  if (!(scale >= kMinScale) || !isfinite(scale)) return FA_ERR_UNSUPPORTED;
  // Grid sizes: B*H*ceil(N/64) workgroups at most; B*H must fit an int.
  if (B > kMaxWorkgroups / H) return FA_ERR_SHAPE;
  const int64_t bh = B * H;
  if (bh > kMaxWorkgroups / ((N + 63) / 64)) return FA_ERR_SHAPE;
  return FA_OK;
}

// Grouped heads: H_kv K/V heads, each shared by H / H_kv query heads.
int check_heads(int64_t H, int64_t H_kv) {
  if (H_kv <= 0 || H_kv > H || H % H_kv != 0) return FA_ERR_SHAPE;
  return FA_OK;
}

// Sections of a key-mask tile table for B batch elements and T tiles.
struct TileTableLayout {
  size_t prefix_off, list_off, bytes;
};
TileTableLayout tile_table_layout(int64_t B, int64_t T) {
  TileTableLayout l;
  l.prefix_off = align256(static_cast<size_t>(B * T) * sizeof(uint64_t));
  l.list_off = l.prefix_off + align256(static_cast<size_t>(B * (T + 1)) * sizeof(int));
  l.bytes = l.list_off + align256(static_cast<size_t>(B * T) * sizeof(int));
  return l;
}

fa::MaskTiles mask_tiles_view(const void* tiles, int64_t B, int64_t N) {
  const int64_t T = (N + 63) / 64;
  const TileTableLayout l = tile_table_layout(B, T);
  const char* base = static_cast<const char*>(tiles);
  fa::MaskTiles m;
  m.words = reinterpret_cast<const uint64_t*>(base);
  m.prefix = reinterpret_cast<const int*>(base + l.prefix_off);
  m.list = reinterpret_cast<const int*>(base + l.list_off);
  m.n_tiles = static_cast<int>(T);
  return m;
}

// Dropout parameters: thr = floor(p * 65536) (p in [0, 1)), keep scale
// 65536 / (65536 - thr).  Returns false for p outside [0, 1).
bool dropout_args(float p, uint64_t seed, uint64_t offset, fa::DropoutArgs* d) {
  if (!(p >= 0.f && p < 1.f)) return false;
  const double thr = floor(static_cast<double>(p) * 65536.0);
  d->seed = seed;
  d->offset = offset;
  d->thr = static_cast<uint32_t>(thr);
  d->keep_scale = static_cast<float>(65536.0 / (65536.0 - thr));
  return true;
}

fa::MaskTiles no_mask() {
  fa::MaskTiles m;
  m.words = nullptr;
  m.prefix = nullptr;
  m.list = nullptr;
  m.n_tiles = 0;
  return m;
}

fa::FwdArgs fwd_args(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                     int64_t H_kv, int64_t N, float scale) {
  fa::FwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.N = N;
  a.BH = static_cast<int>(B * H);
  a.H = static_cast<int>(H);
  a.Hkv = static_cast<int>(H_kv);
  a.n_qtiles = 0;  // set by the launcher from its tile shape
  a.scale_log2 = scale * kLog2e;
  a.n_splits = 1;
  a.part_lse = nullptr;
  a.part_o = nullptr;
  a.mask = no_mask();
  dropout_args(0.f, 0, 0, &a.drop);
  return a;
}

// Backward workspace: Delta (FP32 [B*H*N]); then, when the dK/dV pass splits
// its query positions into P > 1 parts, FP32 partial dK and dV
// [P][B*H_kv*N][D] each; then, when the dQ pass splits its key tiles into
// Q > 1 parts, FP32 partial dQ [Q][B*H*N][D]; every section 256-byte aligned.
struct BwdLayout {
  size_t delta, part_kv, part_q;  // section sizes (0 when absent)
  size_t total() const { return delta + 2 * part_kv + part_q; }
};
BwdLayout bwd_layout(int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t D) {
  BwdLayout l;
  l.delta = align256(static_cast<size_t>(B * H * N) * sizeof(float));
  const int kv_parts = fa::bwd_head_parts(B, H, H_kv, N);
  l.part_kv = kv_parts > 1 ? align256(static_cast<size_t>(kv_parts) * static_cast<size_t>(B * H_kv * N) *
                                      static_cast<size_t>(D) * sizeof(float))
                           : 0;
  const int q_parts = fa::bwd_dq_parts(B, H, N);
  l.part_q = q_parts > 1 ? align256(static_cast<size_t>(q_parts) * static_cast<size_t>(B * H * N) *
                                    static_cast<size_t>(D) * sizeof(float))
                         : 0;
  return l;
}
size_t bwd_workspace_layout(int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t D) {
  return bwd_layout(B, H, H_kv, N, D).total();
}

fa::BwdArgs bwd_args(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                     void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t D,
                     float scale, void* workspace) {
  fa::BwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.lse = lse;
  a.dout = static_cast<const uint16_t*>(dout);
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.delta = static_cast<float*>(workspace);
  a.N = N;
  a.BH = static_cast<int>(B * H);
  a.H = static_cast<int>(H);
  a.Hkv = static_cast<int>(H_kv);
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  a.mask = no_mask();
  dropout_args(0.f, 0, 0, &a.drop);
  // Parts of the dK/dV and dQ passes and their FP32 partial sums, placed
  // after Delta in the workspace (see bwd_layout).
  const BwdLayout l = bwd_layout(B, H, H_kv, N, D);
  char* ws = static_cast<char*>(workspace);
  a.head_parts = fa::bwd_head_parts(B, H, H_kv, N);
  a.part_dk = a.head_parts > 1 ? reinterpret_cast<float*>(ws + l.delta) : nullptr;
  a.part_dv = a.head_parts > 1 ? reinterpret_cast<float*>(ws + l.delta + l.part_kv) : nullptr;
  a.dq_parts = fa::bwd_dq_parts(B, H, N);
  a.part_dq = a.dq_parts > 1 ? reinterpret_cast<float*>(ws + l.delta + 2 * l.part_kv) : nullptr;
  return a;
}

int check_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t H_kv,
              int64_t N, int64_t D, int causal, float scale, int dtype) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_common(B, H, N, D, causal, scale, dtype);
  if (st != FA_OK) return st;
  st = check_heads(H, H_kv);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse)) return FA_ERR_ALIGN;
  return FA_OK;
}

int check_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
              void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t D, int causal,
              float scale, int dtype, void* workspace, size_t workspace_bytes) {
  const int st = fa::check_bwd_args(q, k, v, o, lse, dout, dq, dk, dv, B, H, H_kv, N, D, causal, scale, dtype);
  if (st != FA_OK) return st;
  const size_t need = bwd_workspace_layout(B, H, H_kv, N, D);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  return FA_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

}  // namespace

namespace fa {

int check_bwd_args(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t H_kv, int64_t N, int64_t D,
                   int causal, float scale, int dtype) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL;
  int st = check_common(B, H, N, D, causal, scale, dtype);
  if (st != FA_OK) return st;
  st = check_heads(H, H_kv);
  if (st != FA_OK) return st;
  const void* ptrs[] = {q, k, v, o, lse, dout, dq, dk, dv};
  for (const void* p : ptrs)
    if (!aligned16(p)) return FA_ERR_ALIGN;
  return FA_OK;
}

}  // namespace fa

namespace {

size_t splitkv_workspace(int64_t B, int64_t H, int64_t N, int64_t D, int splits);

// The split-K/V forward for H_kv K/V heads, with dropout when drop_p >= 0 and
// a key-padding mask when tiles is not NULL.
int splitkv_common(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                   int64_t H_kv, int64_t N, int64_t D, int causal, float scale, int dtype, int num_splits,
                   float drop_p, uint64_t seed, uint64_t offset, const void* tiles, void* workspace,
                   size_t workspace_bytes, void* stream) {
  const int st = check_fwd(q, k, v, o, lse, B, H, H_kv, N, D, causal, scale, dtype);
  if (st != FA_OK) return st;
  if (tiles && !aligned16(tiles)) return FA_ERR_ALIGN;
  if (num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_UNSUPPORTED;
  if (B * H * ((N + 63) / 64) > kMaxWorkgroups / num_splits) return FA_ERR_SHAPE;
  const size_t need = splitkv_workspace(B, H, N, D, num_splits);
  if (!workspace || workspace_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  fa::FwdArgs a = fwd_args(q, k, v, o, lse, B, H, H_kv, N, scale);
  const bool drop = drop_p >= 0.f;
  if (drop && !dropout_args(drop_p, seed, offset, &a.drop)) return FA_ERR_UNSUPPORTED;
  a.n_splits = num_splits;
  const size_t rows = static_cast<size_t>(B * H * N) * static_cast<size_t>(num_splits);
  a.part_lse = static_cast<float*>(workspace);
  a.part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(rows * sizeof(float)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int d = static_cast<int>(D);
  const bool c = causal != 0;
  if (tiles) {
    a.mask = mask_tiles_view(tiles, B, N);
    return status_of(drop ? fa::launch_fwd_splitkv_masked_dropout(a, d, c, dtype, s)
                          : fa::launch_fwd_splitkv_masked(a, d, c, dtype, s));
  }
  return status_of(drop ? fa::launch_fwd_splitkv_dropout(a, d, c, dtype, s) : fa::launch_fwd_splitkv(a, d, c, dtype, s));
}

// The options of an _ex call, checked (opt == NULL: the defaults).  The
// backward ignores num_splits.
struct Options {
  int64_t h_kv;
  const void* tiles;
  bool drop;
  float p;
  uint64_t seed, offset;
  int splits;
};
int64_t option_h_kv(const fa_options* opt, int64_t H) { return (opt && opt->h_kv != 0) ? opt->h_kv : H; }
int read_options(const fa_options* opt, int64_t H, bool forward, Options* o) {
  *o = Options{H, nullptr, false, 0.f, 0, 0, 0};
  if (!opt) return FA_OK;
  o->h_kv = option_h_kv(opt, H);
  if (check_heads(H, o->h_kv) != FA_OK) return FA_ERR_SHAPE;
  if (opt->dropout != 0 && opt->dropout != 1) return FA_ERR_UNSUPPORTED;
  o->drop = opt->dropout == 1;
  o->p = opt->dropout_p;
  o->seed = opt->dropout_seed;
  o->offset = opt->dropout_offset;
  if (o->drop && !(o->p >= 0.f && o->p < 1.f)) return FA_ERR_UNSUPPORTED;
  if (forward) {
    if (opt->num_splits < 0 || opt->num_splits > kMaxSplits) return FA_ERR_UNSUPPORTED;
    o->splits = opt->num_splits;
  }
  o->tiles = opt->mask_tiles;
  if (o->tiles && !aligned16(o->tiles)) return FA_ERR_ALIGN;
  return FA_OK;
}

size_t splitkv_workspace(int64_t B, int64_t H, int64_t N, int64_t D, int splits) {
  const size_t rows = static_cast<size_t>(B * H * N) * static_cast<size_t>(splits);
  return align256(rows * sizeof(float)) + align256(rows * static_cast<size_t>(D) * sizeof(float));
}

}  // namespace

extern "C" {

const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE:
      return "FA_ERR_SHAPE: B, H or N is not positive, H_kv does not divide H, or the problem is too large";
    case FA_ERR_UNSUPPORTED:
      return "FA_ERR_UNSUPPORTED: need D in {64,128}, dtype fp16/bf16, causal 0/1, finite scale >= 2^-64";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: a pointer is not 16-byte aligned";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime rejected a launch";
    case FA_ERR_SCRATCH_LIMIT:
      return "FA_ERR_SCRATCH_LIMIT: the shape needs more backward workspace than the static scratch of "
             "fa_bwd_noalloc (FA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown fa_status";
  }
}

// ---- forward ---------------------------------------------------------------

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t N,
           int64_t D, int causal, float scale, int dtype, void* stream) {
  return fa_fwd_ex(q, k, v, o, lse, B, H, N, D, causal, scale, dtype, nullptr, nullptr, 0, stream);
}

size_t fa_fwd_ex_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int causal, int dtype,
                                 const fa_options* opt) {
  if (check_common(B, H, N, D, causal, 1.0f, dtype) != FA_OK) return 0;
  Options op;
  if (read_options(opt, H, true, &op) != FA_OK) return 0;
  return op.splits > 0 ? splitkv_workspace(B, H, N, D, op.splits) : 0;
}

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t N,
              int64_t D, int causal, float scale, int dtype, const fa_options* opt, void* workspace,
              size_t workspace_bytes, void* stream) {
  int st = check_fwd(q, k, v, o, lse, B, H, option_h_kv(opt, H), N, D, causal, scale, dtype);
  if (st != FA_OK) return st;
  Options op;
  st = read_options(opt, H, true, &op);
  if (st != FA_OK) return st;
  if (op.splits > 0)
    return splitkv_common(q, k, v, o, lse, B, H, op.h_kv, N, D, causal, scale, dtype, op.splits,
                          op.drop ? op.p : -1.f, op.seed, op.offset, op.tiles, workspace, workspace_bytes, stream);
  fa::FwdArgs a = fwd_args(q, k, v, o, lse, B, H, op.h_kv, N, scale);
  if (op.drop && !dropout_args(op.p, op.seed, op.offset, &a.drop)) return FA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int d = static_cast<int>(D);
  const bool c = causal != 0;
  if (op.tiles) {
    a.mask = mask_tiles_view(op.tiles, B, N);
    return status_of(op.drop ? fa::launch_fwd_masked_dropout(a, d, c, dtype, s) : fa::launch_fwd_masked(a, d, c, dtype, s));
  }
  return status_of(op.drop ? fa::launch_fwd_dropout(a, d, c, dtype, s) : fa::launch_fwd(a, d, c, dtype, s));
}

const char* fa_fwd_kernel_name(int64_t B, int64_t H, int64_t N, int64_t D, int causal) {
  if (check_common(B, H, N, D, causal, 1.0f, FA_FP16) != FA_OK) return "";
  switch (fa::fwd_path(B * H, N, D, causal != 0)) {
    case fa::FwdPath::kShort:
      return fa::short_pipelined(N, D) ? "fwd_short_pipe_kernel" : "fwd_short_kernel";
    case fa::FwdPath::kD128:
      return "fwd_d128_kernel";
    default:
      return "fwd_kernel";
  }
}

int fa_fwd_splitkv_num_splits(int64_t B, int64_t H, int64_t N, int64_t D, int causal) {
  if (check_common(B, H, N, D, causal, 1.0f, FA_FP16) != FA_OK) return 0;
  // Measured on MI355X (fp16, D = 128): B1 H1 N16384 runs at 481 TFLOP/s in
  // one pass and 939 with 4 splits; B2 H8 N2048 (256 workgroups, 1024-key
  // ranges at S = 2) is fastest unsplit.
  const int64_t wg = B * H * ((N + 127) / 128);
  int s = 1;
  while (s < 16 && wg * s < 512 && N / (2 * s) >= 2048) s *= 2;
  return s;
}

size_t fa_mask_tiles_bytes(int64_t B, int64_t N) {
  if (B <= 0 || N <= 0 || N > kMaxN) return 0;
  const int64_t T = (N + 63) / 64;
  if (B > kMaxWorkgroups / T) return 0;
  return tile_table_layout(B, T).bytes;
}

int fa_mask_tiles(const uint8_t* key_mask, int64_t B, int64_t N, void* tiles, size_t tiles_bytes, void* stream) {
  if (!key_mask) return FA_ERR_NULL;
  if (B <= 0 || N <= 0 || N > kMaxN) return FA_ERR_SHAPE;
  const size_t need = fa_mask_tiles_bytes(B, N);
  if (need == 0) return FA_ERR_SHAPE;
  if (!tiles || tiles_bytes < need) return FA_ERR_WORKSPACE;
  if (!aligned16(tiles)) return FA_ERR_ALIGN;
  const fa::MaskTiles m = mask_tiles_view(tiles, B, N);
  return status_of(fa::launch_mask_tiles(key_mask, B, N, const_cast<uint64_t*>(m.words), const_cast<int*>(m.prefix),
                                         const_cast<int*>(m.list), static_cast<hipStream_t>(stream)));
}

// ---- backward --------------------------------------------------------------

size_t fa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int causal, int dtype) {
  if (check_common(B, H, N, D, causal, 1.0f, dtype) != FA_OK) return 0;
  return bwd_workspace_layout(B, H, H, N, D);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
           void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t D, int causal, float scale,
           int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return fa_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, causal, scale, dtype, nullptr, workspace,
                   workspace_bytes, stream);
}

size_t fa_bwd_ex_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int causal, int dtype,
                                 const fa_options* opt) {
  if (check_common(B, H, N, D, causal, 1.0f, dtype) != FA_OK) return 0;
  Options op;
  if (read_options(opt, H, false, &op) != FA_OK) return 0;
  return bwd_workspace_layout(B, H, op.h_kv, N, D);
}

int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
              void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t D, int causal, float scale,
              int dtype, const fa_options* opt, void* workspace, size_t workspace_bytes, void* stream) {
  const int64_t h_kv = option_h_kv(opt, H);
  int st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, h_kv, N, D, causal, scale, dtype, workspace,
                     workspace_bytes);
  if (st != FA_OK) return st;
  Options op;
  st = read_options(opt, H, false, &op);
  if (st != FA_OK) return st;
  fa::BwdArgs a = bwd_args(q, k, v, o, lse, dout, dq, dk, dv, B, H, op.h_kv, N, D, scale, workspace);
  if (op.drop && !dropout_args(op.p, op.seed, op.offset, &a.drop)) return FA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int d = static_cast<int>(D);
  const bool c = causal != 0;
  if (op.tiles) {
    a.mask = mask_tiles_view(op.tiles, B, N);
    return status_of(op.drop ? fa::launch_bwd_masked_dropout(a, d, c, dtype, s) : fa::launch_bwd_masked(a, d, c, dtype, s));
  }
  return status_of(op.drop ? fa::launch_bwd_dropout(a, d, c, dtype, s) : fa::launch_bwd(a, d, c, dtype, s));
}

int fa_dropout_mask(uint8_t* keep, int64_t B, int64_t H, int64_t N, float dropout_p, uint64_t seed, uint64_t offset,
                    void* stream) {
  if (!keep) return FA_ERR_NULL;
  if (B <= 0 || H <= 0 || N <= 0 || N > kMaxN) return FA_ERR_SHAPE;
  if (B > kMaxWorkgroups / H || N > (int64_t(1) << 24)) return FA_ERR_SHAPE;
  const int64_t per_head = N * ((N + 15) / 16);  // threads per head, <= 2^44
  if (B * H > (kMaxWorkgroups * 256) / per_head) return FA_ERR_SHAPE;
  fa::DropoutArgs d;
  if (!dropout_args(dropout_p, seed, offset, &d)) return FA_ERR_UNSUPPORTED;
  return status_of(fa::launch_dropout_mask(keep, B * H, N, d, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
