// fa_fwd.hip -- FlashAttention forward for gfx950.
//
// Computes O = softmax(scale * Q K^T + M) V and the natural-log row LSE with
// the online-softmax recurrence ("CUDA FlashAttention: from online softmax to
// the long-sequence IO limit", §4; "FlashAttention algorithm details",
// §4.2.1-4.2.2): per key tile, m' = max(m, rowmax S), alpha = exp(m - m'),
// l = alpha l + rowsum exp(S - m'), O = alpha O + exp(S - m') V.  The mask is
// applied before the tile max, the old output is rescaled before the new
// P V is added, and alpha is 0 while m is still -inf ("CUDA FlashAttention
// ...", §6).  Tiles wholly above the causal diagonal are never visited
// ("Why FlashAttention does not need to store the attention matrix", §4.5).
//
// Work decomposition (one workgroup = 4 waves = 128 queries of one head):
//  * Each wave owns 32 queries.  Their Q rows stay in VGPRs for the whole
//    pass as the B operand of S^T = K Q^T (32 keys x 32 queries per MFMA).
//  * Keys and values stream in tiles of 64 through LDS.  K is stored row
//    major (swizzled); V is stored transposed (V^T, keys contiguous) so that
//    O^T = V^T P^T reads 16-byte operand fragments.  While a tile is being
//    used, the next one is already in flight from HBM into registers.
//  * Computing S^T puts one query per lane (two lanes per query, 32 keys
//    each), so the row max is an in-lane reduction plus one cross-half swap,
//    and the row sum needs no cross-lane step until the epilogue.
//  * Softmax runs in base 2 with scale*log2(e) folded into one FMA.
//  * Workgroups are numbered heaviest-first for causal masks, and all query
//    tiles of one head get workgroup ids congruent modulo 8, so they run on
//    the same XCD and share its L2 for the re-streamed K/V.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr int kFwdBM = 128;  // queries per workgroup
constexpr int kFwdBN = 64;   // keys per tile
constexpr int kFwdThreads = 256;
constexpr float kLazy = 8.0f;         // max probability 2^8 between rescales
constexpr float kFastLimit = 4096.0f; // |scale*log2e*S| below this: one-FMA exponent

template <int D, bool CAUSAL, class T>
__global__ __launch_bounds__(kFwdThreads, 2) void fwd_kernel(FwdArgs a) {
  constexpr int BM = kFwdBM, BN = kFwdBN, NT = kFwdThreads;
  constexpr int KCH = D / 8;             // 16-byte chunks per K row
  constexpr int K_CHUNKS = BN * KCH;     // chunks per K tile
  constexpr int VCH = BN / 8;            // 16-byte chunks per V^T row
  constexpr int KPT = K_CHUNKS / NT;     // K chunks loaded per thread
  constexpr int DV = (BN * D) / (8 * NT);  // V columns per thread (8 keys each)
  constexpr int DGROUPS = D / DV;        // threads per group of 8 keys
  static_assert(KPT * NT == K_CHUNKS, "K tile split");
  static_assert(DGROUPS * (BN / 8) == NT, "V tile split");
  static_assert(DV == 2 || DV == 4, "V column split");

  __shared__ u32x4 lds_k[K_CHUNKS];
  __shared__ u32x4 lds_vt[D * VCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ql = lane & 31, g = lane >> 5;

  const int64_t N = a.N;
  const int bh = blockIdx.x % a.BH;
  const int rank = blockIdx.x / a.BH;
  const int qt = CAUSAL ? (a.n_qtiles - 1 - rank) : rank;
  const int64_t head = (int64_t)bh * N * D;
  const uint16_t* __restrict__ Qh = a.q + head;
  const uint16_t* __restrict__ Kh = a.k + head;
  const uint16_t* __restrict__ Vh = a.v + head;

  const int q0w = qt * BM + wave * 32;  // first query of this wave
  const bool active = q0w < N;          // N % 64 == 0: whole wave in or out
  const int my_q = q0w + ql;

  // Q^T operand fragments: lane (ql, g) holds Q[my_q][16c + 8g .. +8].
  u32x4 qf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    qf[c] = active ? *(const u32x4*)(Qh + (int64_t)my_q * D + c * 16 + g * 8) : u32x4{0, 0, 0, 0};
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = f32x16{};
  float r_raw = -INFINITY;  // reference max, in raw (unscaled) score units
  float l_run = 0.f;        // this lane's part of the running sum

  const int n_kt_all = (int)(N / BN);
  const int n_kt = CAUSAL ? min(n_kt_all, ((qt + 1) * BM) / BN) : n_kt_all;

  // Next tile in flight: K chunks and 8 keys x DV columns of V.
  const int dg = tid % DGROUPS, kg = tid / DGROUPS;
  u32x4 kreg[KPT];
  uint32_t vreg[8][DV / 2];

  auto load_tile = [&](int kt) {
    const uint16_t* Kt = Kh + (int64_t)kt * BN * D;
#pragma unroll
    for (int i = 0; i < KPT; ++i) kreg[i] = *(const u32x4*)(Kt + (tid + i * NT) * 8);
    const uint16_t* Vt = Vh + (int64_t)kt * BN * D + (int64_t)(kg * 8) * D + dg * DV;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      if constexpr (DV == 4) {
        u32x2 x = *(const u32x2*)(Vt + r * D);
        vreg[r][0] = x[0];
        vreg[r][1] = x[1];
      } else {
        vreg[r][0] = *(const uint32_t*)(Vt + r * D);
      }
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KPT; ++i) lds_k[swz(tid + i * NT)] = kreg[i];
    // transpose 8 keys x DV columns into DV rows of V^T (8 keys each)
#pragma unroll
    for (int j = 0; j < DV; ++j) {
      u32x4 w;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint32_t lo = vreg[2 * p][j >> 1], hi = vreg[2 * p + 1][j >> 1];
        w[p] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      const int d = dg * DV + j;
      lds_vt[swz(d * VCH + kg)] = w;
    }
  };

  const float c2 = a.scale_log2;
  load_tile(0);
  for (int kt = 0; kt < n_kt; ++kt) {
    __syncthreads();  // every wave is done reading the previous tile
    store_tile();
    __syncthreads();
    if (kt + 1 < n_kt) load_tile(kt + 1);

    const int k0 = kt * BN;
    if (!active || (CAUSAL && k0 > q0w + 31)) continue;  // nothing visible

    // S^T = K Q^T for 64 keys (two 32-key blocks) x 32 queries.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const int krow = kb * 32 + perm23(ql);
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const u32x4 kf = lds_k[swz(krow * KCH + c * 2 + g)];
        s[kb] = mfma32<T>(kf, qf[c], s[kb]);
      }
    }

    if (CAUSAL && k0 + BN - 1 > q0w) {  // diagonal tile: mask before the max
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (k0 + kb * 32 + acc_row(r, g) > my_q) s[kb][r] = -INFINITY;
    }

    float mx = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
    mx = xhalf_max(mx);  // raw max of this row over the tile

    // The reference max r_raw is always one of the raw scores (exact).  In
    // the usual case the exponent is one FMA, s*c2 - RN(r_raw*c2), and the
    // reference is only raised when the tile max exceeds it by more than
    // kLazy in log2 units, so probabilities stay below 2^kLazy and the O/l
    // rescale is skipped on most tiles; the result is unchanged because O and
    // l always share the same reference.  When scaled scores are so large
    // that RN(r_raw*c2) is off by a meaningful amount (|.| >= kFastLimit), the
    // scores are first shifted by r_raw in raw units, where the difference is
    // exact for scores near the max, and the same FMA then scales them.
    const float mc_tile = mx * c2;
    float mref = r_raw * c2;
    const bool fast_ok = (fabsf(mc_tile) < kFastLimit || mc_tile == -INFINITY) &&
                         (fabsf(mref) < kFastLimit || mref == -INFINITY);
    const bool exact = !wave_all(fast_ok);
    if (exact || wave_any(mc_tile > mref + kLazy)) {
      const float r_new = fmaxf(r_raw, mx);
      const float lg = exact ? (r_raw - r_new) * c2 : mref - r_new * c2;
      const float alpha = (r_raw == -INFINITY) ? 0.f : fast_exp2(lg);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < D / 32; ++i) oacc[i] *= alpha;
      r_raw = r_new;
      mref = r_raw * c2;
    }
    float m_use = (mref == -INFINITY) ? 0.f : mref;
    if (exact) {
      const float ru = (r_raw == -INFINITY) ? 0.f : r_raw;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] -= ru;
      m_use = 0.f;
    }
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[kb][r], c2, -m_use));
        s[kb][r] = p;
        lsum += p;
      }
    l_run += lsum;

    // O^T += V^T P^T, 16 keys per step: step t uses keys 16t .. 16t+15, which
    // are accumulator registers 8*(t%2) .. +7 of block t/2 (see acc_row).
#pragma unroll
    for (int t = 0; t < BN / 16; ++t) {
      const u32x4 pf = pack8<T>(s[t >> 1], (t & 1) * 8);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const u32x4 vf = lds_vt[swz((db * 32 + ql) * VCH + 2 * t + g)];
        oacc[db] = mfma32<T>(vf, pf, oacc[db]);
      }
    }
  }

  if (!active) return;
  const float l_tot = xhalf_sum(l_run);
  const float inv = 1.f / l_tot;
  uint16_t* Orow = a.o + head + (int64_t)my_q * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      u32x2 w;
      w[0] = pack2<T>(oacc[db][rq * 4 + 0] * inv, oacc[db][rq * 4 + 1] * inv);
      w[1] = pack2<T>(oacc[db][rq * 4 + 2] * inv, oacc[db][rq * 4 + 3] * inv);
      *(u32x2*)(Orow + db * 32 + rq * 8 + g * 4) = w;
    }
  if (g == 0) a.lse[(int64_t)bh * N + my_q] = (r_raw * c2 + __log2f(l_tot)) * kLn2;
}

template <int D, bool CAUSAL, class T>
hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
  const int64_t n_wg = (int64_t)a.BH * a.n_qtiles;
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL, T>), dim3((unsigned)n_wg), dim3(kFwdThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int fwd_block_m() { return kFwdBM; }

hipError_t launch_fwd(const FwdArgs& a, int D, bool causal, int dtype, hipStream_t stream) {
#define FA_FWD_CASE(DD, CC, TT) \
  if (D == DD && causal == CC && dtype == TT::id) return launch_fwd_t<DD, CC, TT>(a, stream);
  FA_FWD_CASE(64, false, Fp16)
  FA_FWD_CASE(64, true, Fp16)
  FA_FWD_CASE(128, false, Fp16)
  FA_FWD_CASE(128, true, Fp16)
  FA_FWD_CASE(64, false, Bf16)
  FA_FWD_CASE(64, true, Bf16)
  FA_FWD_CASE(128, false, Bf16)
  FA_FWD_CASE(128, true, Bf16)
#undef FA_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace fa
