// fa_bwd.hip -- FlashAttention backward by recomputation, for gfx950.
//
// With P = exp(scale * Q K^T + M - LSE) rebuilt tile by tile from the saved
// natural-log LSE ("Why FlashAttention does not need to store the attention
// matrix", §3.3; "FlashAttention algorithm details", §4.3.2 step 2):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - Delta),
//   dQ = scale * dS K,  dK = scale * dS^T Q,
// with Delta_i = rowsum(dO_i * O_i), which equals rowsum(P_i * dP_i) because
// O = P V ("FlashAttention dataflow and engineering validation on MI50", §3.3:
// a light first pass computes this correction term).
//
// Three kernels, in order on one stream:
//  1. delta_kernel: Delta for every query row (HBM-bound, one pass over O, dO).
//  2. dkdv_kernel: one workgroup per 128 keys (32 per wave), K and V resident
//     in VGPRs, looping over query tiles of 64 -- the outer-K/V, inner-Q order
//     of "FlashAttention algorithm details", §4.3.2.  dK and dV accumulate in
//     registers and are written once.
//  3. dq_kernel: one workgroup per 128 queries, Q and dO resident, looping
//     over key tiles of 64; dQ accumulates in registers and is written once.
// Splitting dQ into its own pass (instead of atomically adding partial dQ
// from every key tile) costs a second recomputation of S and dP but makes the
// result bitwise reproducible.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr int kThreads = 256;

template <class T>
__device__ __forceinline__ float lo16_to_f32(uint32_t w);
template <class T>
__device__ __forceinline__ float hi16_to_f32(uint32_t w);
template <>
__device__ __forceinline__ float lo16_to_f32<Fp16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
template <>
__device__ __forceinline__ float hi16_to_f32<Fp16>(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}
template <>
__device__ __forceinline__ float lo16_to_f32<Bf16>(uint32_t w) {
  return __uint_as_float(w << 16);
}
template <>
__device__ __forceinline__ float hi16_to_f32<Bf16>(uint32_t w) {
  return __uint_as_float(w & 0xffff0000u);
}

// ---------------------------------------------------------------------------
// Delta_i = sum_d dO_id * O_id in FP32 (D/8 lanes per row, 8 elements each).
// ---------------------------------------------------------------------------
template <int D, class T>
__global__ __launch_bounds__(kThreads) void delta_kernel(const uint16_t* __restrict__ o,
                                                         const uint16_t* __restrict__ dout,
                                                         float* __restrict__ delta, int64_t rows) {
  constexpr int TPR = D / 8;
  constexpr int RPB = kThreads / TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 x = *(const u32x4*)(o + row * D + c * 8);
    const u32x4 y = *(const u32x4*)(dout + row * D + c * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = __builtin_fmaf(lo16_to_f32<T>(x[i]), lo16_to_f32<T>(y[i]), acc);
      acc = __builtin_fmaf(hi16_to_f32<T>(x[i]), hi16_to_f32<T>(y[i]), acc);
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (c == 0 && row < rows) delta[row] = acc;
}

// ---------------------------------------------------------------------------
// Tile staging helpers.  A 64-row x D-column tile of a [.., D] row-major
// tensor is kept in LDS as swizzled 16-byte chunks, either row-major
// ("rows", D/8 chunks per row) or transposed ("cols": D rows of 64 entries,
// 8 chunks per row).
// ---------------------------------------------------------------------------
constexpr int kTileRows = 64;

// 128 threads stage one tile into BOTH layouts: thread t owns rows
// 8*(t/16) .. +7 and columns (D/16)*(t%16) .. +D/16-1.
template <int D>
struct DualStager {
  static constexpr int CW = D / 16;  // columns per thread: 4 or 8
  uint32_t buf[8][CW / 2];
  int cg, rg;
  __device__ void init(int t) {
    cg = t % 16;
    rg = t / 16;
  }
  __device__ void load(const uint16_t* __restrict__ src) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint16_t* p = src + (int64_t)(rg * 8 + r) * D + cg * CW;
      if constexpr (CW == 8) {
        const u32x4 x = *(const u32x4*)p;
        buf[r][0] = x[0];
        buf[r][1] = x[1];
        buf[r][2] = x[2];
        buf[r][3] = x[3];
      } else {
        const u32x2 x = *(const u32x2*)p;
        buf[r][0] = x[0];
        buf[r][1] = x[1];
      }
    }
  }
  __device__ void store(u32x4* lds_rows, u32x4* lds_cols) const {
    constexpr int RCH = D / 8;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = rg * 8 + r;
      if constexpr (CW == 8) {
        lds_rows[swz(row * RCH + cg)] = u32x4{buf[r][0], buf[r][1], buf[r][2], buf[r][3]};
      } else {
        u32x2* dst = (u32x2*)&lds_rows[swz(row * RCH + (cg >> 1))];
        dst[cg & 1] = u32x2{buf[r][0], buf[r][1]};
      }
    }
#pragma unroll
    for (int j = 0; j < CW; ++j) {
      u32x4 w;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t lo = buf[2 * p][j >> 1], hi = buf[2 * p + 1][j >> 1];
        w[p] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      lds_cols[swz((cg * CW + j) * (kTileRows / 8) + rg)] = w;
    }
  }
};

// 128 threads stage one tile row-major only, in 16-byte chunks.
template <int D>
struct RowStager {
  static constexpr int PER = kTileRows * (D / 8) / 128;
  u32x4 buf[PER];
  int t;
  __device__ void init(int t_) { t = t_; }
  __device__ void load(const uint16_t* __restrict__ src) {
#pragma unroll
    for (int i = 0; i < PER; ++i) buf[i] = *(const u32x4*)(src + (t + i * 128) * 8);
  }
  __device__ void store(u32x4* lds_rows) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) lds_rows[swz(t + i * 128)] = buf[i];
  }
};

// ---------------------------------------------------------------------------
// dK, dV: workgroup = 128 keys of one head; wave w owns keys k0w .. k0w+31.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, class T>
__global__ __launch_bounds__(kThreads, 1) void dkdv_kernel(BwdArgs a) {
  constexpr int BK = 128, BQ = kTileRows;
  constexpr int RCH = D / 8, TCH = BQ / 8;
  __shared__ u32x4 lds_q[BQ * RCH];
  __shared__ u32x4 lds_qt[D * TCH];
  __shared__ u32x4 lds_do[BQ * RCH];
  __shared__ u32x4 lds_dot[D * TCH];
  __shared__ __attribute__((aligned(16))) float lds_lse[BQ];
  __shared__ __attribute__((aligned(16))) float lds_dl[BQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int64_t N = a.N;
  const int bh = blockIdx.x % a.BH;
  const int kt = blockIdx.x / a.BH;  // key tiles heaviest (lowest) first
  const int64_t head = (int64_t)bh * N * D;
  const int64_t rowbase = (int64_t)bh * N;

  const int k0w = kt * BK + wave * 32;
  const bool active = k0w < N;
  const int my_k = k0w + l32;

  // Resident B operands: lane (key, g) holds K[my_k][16c+8g..+8] and V likewise.
  u32x4 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const int64_t off = head + (int64_t)my_k * D + c * 16 + g * 8;
    kf[c] = active ? *(const u32x4*)(a.k + off) : u32x4{0, 0, 0, 0};
    vf[c] = active ? *(const u32x4*)(a.v + off) : u32x4{0, 0, 0, 0};
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  const bool is_q_stager = tid < 128;  // waves 0-1 stage Q, waves 2-3 stage dO
  DualStager<D> st;
  st.init(tid & 127);
  const uint16_t* stage_src = (is_q_stager ? a.q : a.dout) + head;
  u32x4* lds_rows = is_q_stager ? lds_q : lds_do;
  u32x4* lds_cols = is_q_stager ? lds_qt : lds_dot;
  float lse_next = 0.f, dl_next = 0.f;

  const int n_qt = (int)(N / BQ);
  const int qt_begin = CAUSAL ? (kt * BK) / BQ : 0;
  const float c2 = a.scale_log2;

  auto load = [&](int qt) {
    st.load(stage_src + (int64_t)qt * BQ * D);
    if (tid < BQ) {
      lse_next = a.lse[rowbase + qt * BQ + tid] * kLog2e;
      dl_next = a.delta[rowbase + qt * BQ + tid];
    }
  };

  if (qt_begin < n_qt) load(qt_begin);
  for (int qt = qt_begin; qt < n_qt; ++qt) {
    __syncthreads();
    st.store(lds_rows, lds_cols);
    if (tid < BQ) {
      lds_lse[tid] = lse_next;
      lds_dl[tid] = dl_next;
    }
    __syncthreads();
    if (qt + 1 < n_qt) load(qt + 1);
    if (!active) continue;

    const int q0 = qt * BQ;
#pragma unroll
    for (int qb = 0; qb < BQ / 32; ++qb) {
      const int qb0 = q0 + qb * 32;
      if (CAUSAL && qb0 + 31 < k0w) continue;  // every query precedes every key
      // S (queries x keys) and dP = dO V^T, query rows read in perm23 order.
      f32x16 s = f32x16{}, dp = f32x16{};
      const int arow = qb * 32 + perm23(l32);
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        s = mfma32<T>(lds_q[swz(arow * RCH + 2 * c + g)], kf[c], s);
        dp = mfma32<T>(lds_do[swz(arow * RCH + 2 * c + g)], vf[c], dp);
      }
      // P = exp2(S*scale*log2e - LSE*log2e); dS = P (dP - Delta).
      // Register r holds query qb*32 + acc_row(r, g): two runs of 8.
      const f32x4* lse4 = (const f32x4*)lds_lse;
      const f32x4* dl4 = (const f32x4*)lds_dl;
      float lse_r[16], dl_r[16];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v4 = 0; v4 < 2; ++v4) {
          const int idx = (qb * 32 + h * 16 + g * 8) / 4 + v4;
          const f32x4 x = lse4[idx], y = dl4[idx];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lse_r[h * 8 + v4 * 4 + e] = x[e];
            dl_r[h * 8 + v4 * 4 + e] = y[e];
          }
        }
      const bool diag = CAUSAL && qb0 < k0w + 31;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(__builtin_fmaf(s[r], c2, -lse_r[r]));
        if (diag && my_k > qb0 + acc_row(r, g)) p = 0.f;
        s[r] = p;
        dp[r] = p * (dp[r] - dl_r[r]);
      }
      // dV^T += dO^T P and dK^T += Q^T dS over the 32 queries, 16 per step.
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const u32x4 pf = pack8<T>(s, t2 * 8);
        const u32x4 sf = pack8<T>(dp, t2 * 8);
        const int ch = qb * 4 + t2 * 2 + g;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          dv[db] = mfma32<T>(lds_dot[swz((db * 32 + l32) * TCH + ch)], pf, dv[db]);
          dk[db] = mfma32<T>(lds_qt[swz((db * 32 + l32) * TCH + ch)], sf, dk[db]);
        }
      }
    }
  }

  if (!active) return;
  uint16_t* dk_row = a.dk + head + (int64_t)my_k * D;
  uint16_t* dv_row = a.dv + head + (int64_t)my_k * D;
  const float sc = a.scale;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int d = db * 32 + rq * 8 + g * 4;
      *(u32x2*)(dk_row + d) = u32x2{pack2<T>(dk[db][rq * 4 + 0] * sc, dk[db][rq * 4 + 1] * sc),
                                    pack2<T>(dk[db][rq * 4 + 2] * sc, dk[db][rq * 4 + 3] * sc)};
      *(u32x2*)(dv_row + d) = u32x2{pack2<T>(dv[db][rq * 4 + 0], dv[db][rq * 4 + 1]),
                                    pack2<T>(dv[db][rq * 4 + 2], dv[db][rq * 4 + 3])};
    }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = 128 queries of one head; wave w owns queries q0w .. q0w+31.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, class T>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1) void dq_kernel(BwdArgs a) {
  constexpr int BM = 128, BN = kTileRows;
  constexpr int RCH = D / 8, TCH = BN / 8;
  __shared__ u32x4 lds_k[BN * RCH];
  __shared__ u32x4 lds_kt[D * TCH];
  __shared__ u32x4 lds_v[BN * RCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 31, g = lane >> 5;
  const int64_t N = a.N;
  const int n_qtiles = (int)((N + BM - 1) / BM);
  const int bh = blockIdx.x % a.BH;
  const int rank = blockIdx.x / a.BH;
  const int qt = CAUSAL ? (n_qtiles - 1 - rank) : rank;
  const int64_t head = (int64_t)bh * N * D;

  const int q0w = qt * BM + wave * 32;
  const bool active = q0w < N;
  const int my_q = q0w + ql;

  u32x4 qf[D / 16], gf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const int64_t off = head + (int64_t)my_q * D + c * 16 + g * 8;
    qf[c] = active ? *(const u32x4*)(a.q + off) : u32x4{0, 0, 0, 0};
    gf[c] = active ? *(const u32x4*)(a.dout + off) : u32x4{0, 0, 0, 0};
  }
  const float lse2 = active ? a.lse[(int64_t)bh * N + my_q] * kLog2e : 0.f;
  const float dl = active ? a.delta[(int64_t)bh * N + my_q] : 0.f;
  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dq[i] = f32x16{};

  const bool is_k_stager = tid < 128;  // waves 0-1 stage K (both layouts), 2-3 stage V
  DualStager<D> kst;
  RowStager<D> vst;
  kst.init(tid & 127);
  vst.init(tid & 127);
  auto load = [&](int kt) {
    const int64_t off = head + (int64_t)kt * BN * D;
    if (is_k_stager)
      kst.load(a.k + off);
    else
      vst.load(a.v + off);
  };

  const int n_kt_all = (int)(N / BN);
  const int n_kt = CAUSAL ? min(n_kt_all, ((qt + 1) * BM) / BN) : n_kt_all;
  const float c2 = a.scale_log2;

  load(0);
  for (int kt = 0; kt < n_kt; ++kt) {
    __syncthreads();
    if (is_k_stager)
      kst.store(lds_k, lds_kt);
    else
      vst.store(lds_v);
    __syncthreads();
    if (kt + 1 < n_kt) load(kt + 1);

    const int k0 = kt * BN;
    if (!active || (CAUSAL && k0 > q0w + 31)) continue;

    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
      const int krow = kb * 32 + perm23(ql);
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        s[kb] = mfma32<T>(lds_k[swz(krow * RCH + 2 * c + g)], qf[c], s[kb]);
        dp[kb] = mfma32<T>(lds_v[swz(krow * RCH + 2 * c + g)], gf[c], dp[kb]);
      }
    }
    const bool diag = CAUSAL && k0 + BN - 1 > q0w;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(__builtin_fmaf(s[kb][r], c2, -lse2));
        if (diag && k0 + kb * 32 + acc_row(r, g) > my_q) p = 0.f;
        dp[kb][r] = p * (dp[kb][r] - dl);
      }
    // dQ^T += K^T dS^T, 16 keys per step (registers 8*(t%2).. of block t/2).
#pragma unroll
    for (int t = 0; t < BN / 16; ++t) {
      const u32x4 sf = pack8<T>(dp[t >> 1], (t & 1) * 8);
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        dq[db] = mfma32<T>(lds_kt[swz((db * 32 + ql) * TCH + 2 * t + g)], sf, dq[db]);
    }
  }

  if (!active) return;
  uint16_t* row = a.dq + head + (int64_t)my_q * D;
  const float sc = a.scale;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq)
      *(u32x2*)(row + db * 32 + rq * 8 + g * 4) =
          u32x2{pack2<T>(dq[db][rq * 4 + 0] * sc, dq[db][rq * 4 + 1] * sc),
                pack2<T>(dq[db][rq * 4 + 2] * sc, dq[db][rq * 4 + 3] * sc)};
}

template <int D, bool CAUSAL, class T>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.BH * a.N;
  constexpr int rpb = kThreads / (D / 8);
  hipLaunchKernelGGL((delta_kernel<D, T>), dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(kThreads), 0, stream,
                     a.o, a.dout, a.delta, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n_ktiles = (a.N + 127) / 128;
  hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL, T>), dim3((unsigned)(a.BH * n_ktiles)), dim3(kThreads), 0, stream,
                     a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n_qtiles = (a.N + 127) / 128;
  hipLaunchKernelGGL((dq_kernel<D, CAUSAL, T>), dim3((unsigned)(a.BH * n_qtiles)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int D, bool causal, int dtype, hipStream_t stream) {
#define FA_BWD_CASE(DD, CC, TT) \
  if (D == DD && causal == CC && dtype == TT::id) return launch_bwd_t<DD, CC, TT>(a, stream);
  FA_BWD_CASE(64, false, Fp16)
  FA_BWD_CASE(64, true, Fp16)
  FA_BWD_CASE(128, false, Fp16)
  FA_BWD_CASE(128, true, Fp16)
  FA_BWD_CASE(64, false, Bf16)
  FA_BWD_CASE(64, true, Bf16)
  FA_BWD_CASE(128, false, Bf16)
  FA_BWD_CASE(128, true, Bf16)
#undef FA_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace fa
