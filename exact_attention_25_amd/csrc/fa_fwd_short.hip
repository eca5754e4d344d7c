// fa_fwd_short.hip -- the forward for launches too small to fill the chip
// with whole query tiles: short sequences and few heads.
//
// Same result as the tiled forward (online softmax over 64-key tiles, "CUDA
// FlashAttention: from online softmax to the long-sequence IO limit", §4;
// "FlashAttention algorithm details", §4.2.1-4.2.2), with the work cut
// differently.  When B*H*N is small, a grid of 128-query workgroups leaves
// most of the 256 compute units idle, and the time is that of the workgroup
// with the longest key walk (the last query tile of a causal head), one tile
// after another, each waiting on copies issued one tile earlier.  Here the
// four waves of a workgroup share its queries and split the keys: wave w
// takes key tiles w, w+4, w+8, ... of the tiles those queries see, with its
// own running max, sum and output.  The four partial states are then merged
// as split-K/V partial results are ("CUDA FlashAttention ...", §7: rescale
// each part by exp of its max minus the common max, add, divide by the
// combined sum), through LDS inside the workgroup, so no FP32 partials go to
// HBM.  The critical path is a quarter of the key walk.
//
// A wave owns QB blocks of 32 queries: every K fragment and every V^T
// fragment it fetches feeds QB MFMAs, which keeps the bytes moved from L2
// per MFMA at those of a 32*QB-query tile.  Per tile: S^T = K Q^T (Q^T
// fragments stay in VGPRs; K fragments are loaded straight from memory into
// VGPRs, 16 bytes per lane in MFMA operand order, one tile ahead), the mask
// on diagonal and partial tiles, the row max, the exponentials and the row
// sum, then O^T += V^T P^T with V staged through a ring of VS wave-private
// LDS buffers (direct buffer_load ... lds copies issued VS tiles ahead, XOR
// swizzle, transposing ds_read_b64_tr_b16 reads).  Waves never wait for one
// another until the merge.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr int kShortBN = 64;      // keys per tile
constexpr int kShortWaves = 4;    // waves per workgroup = key splits
constexpr int kShortThreads = 64 * kShortWaves;
constexpr float kShortLazy = 8.0f;          // max probability 2^8 between rescales
constexpr float kShortFastLimit = 4096.0f;  // |scale*log2e*S| below this: one-FMA exponent

// One 64-row tile of a row-major [rows, D] tensor into a wave's LDS buffer:
// copy i of a lane lands at chunk 64i + lane and reads byte src[i % NX] of
// the tile plus 16 rows per NX copies.  Rows from `valid` on read as zero.
template <int D, int LPW, int NX>
__device__ __forceinline__ void copy_tile_wave(const uint16_t* tile, int valid, const int* src, u32x4* dst) {
  const __amdgpu_buffer_rsrc_t r = buffer_rsrc(tile, valid * D * 2);
#pragma unroll
  for (int i = 0; i < LPW; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + i * 64), 16,
                                             src[i % NX], (i / NX) * 16 * D * 2, 0, 0);
}

// QB: query blocks of 32 per wave (1 or 2); the V ring has QB buffers per
// wave, which also hold the wave's partial output for the merge.  QB = 2
// needs about 400 registers (one wave per SIMD); QB = 1 fits two
// workgroups per compute unit.  Every MFMA is preceded by the two wait
// states a vector write of one of its operands requires: with few registers
// the allocator parks operands in the other register class and copies them
// back right before their MFMA, a hazard it does not see through inline
// assembly (without the wait, such an MFMA read stale operands whenever two
// workgroups shared a CU).
template <int D, int QB, bool CAUSAL, class T>
__global__ __launch_bounds__(kShortThreads, QB == 1 ? 2 : 1) void fwd_short_kernel(FwdArgs a) {
  constexpr int VS = QB;
  constexpr int BN = kShortBN;
  constexpr int RC = D / 8;        // 16-byte chunks per row
  constexpr int TC = BN * RC;      // chunks per V tile
  constexpr int LPW = TC / 64;     // copies per lane per V tile
  constexpr int NX = RC / 4;       // copies with distinct swizzle patterns (rows repeat every 16)
  constexpr int NC = D / 16;       // K (and Q) fragments per 32 rows
  constexpr int NV = (BN / 16) * (D / 32);  // P V MFMAs per tile and query block
  constexpr int WQ = 32 * QB;      // queries per wave = per workgroup
  static_assert(LPW % NX == 0 && NX * 64 / RC == 16, "copy pattern");
  static_assert(VS >= QB, "a wave's ring must hold its FP32 partial output for the merge");

  // A ring of VS V tiles per wave; after the key walk the same bytes hold
  // the wave's FP32 partial output for the merge (32*QB x D floats).
  __shared__ u32x4 lds_v[kShortWaves][VS * TC];
  __shared__ float lds_ml[kShortWaves][QB][3][64];  // per lane: reference, its rounding residual, row sum

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, g = lane >> 5;

  const int64_t N = a.N;
  const int G = a.H / a.Hkv;
  const int bh = head_of_slot(blockIdx.x % a.BH, a.BH, G);
  const int rank = blockIdx.x / a.BH;
  const int qt = CAUSAL ? (a.n_qtiles - 1 - rank) : rank;  // heaviest tiles first when causal
  const int q0 = qt * WQ;
  const int64_t head = (int64_t)bh * N * D;
  const int64_t kv_head = (int64_t)(bh / G) * N * D;
  const uint16_t* __restrict__ Qh = a.q + head;
  const uint16_t* __restrict__ Kh = a.k + kv_head;
  const uint16_t* __restrict__ Vh = a.v + kv_head;

  const int n_kt_all = (int)((N + BN - 1) / BN);
  const int n_kt = CAUSAL ? min(n_kt_all, (q0 + WQ - 1) / BN + 1) : n_kt_all;

  // V copies: copy i of this lane fills chunk 64i + lane of a ring buffer,
  // which holds logical chunk (pos ^ dual_xor(row)) of tile row
  // (64i + lane) / RC.  Every 16 rows the swizzle repeats, so copies NX
  // apart differ only by 16 rows.
  int vsrc[NX];
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    const int p = x * 64 + lane, r = p / RC;
    vsrc[x] = (r * D + ((p % RC) ^ dual_xor<RC>(r)) * 8) * 2;
  }
  u32x4* const vring = lds_v[wave];

  // K fragments of a tile in S^T operand order: fragment kb*NC + c of lane
  // (ql, g) is K[64kt + 32kb + perm23(ql)][16c + 8g .. +8], so accumulator
  // register r of lane-half g holds key 32kb + acc_row(r, g).  Rows past N
  // re-read row N-1; their scores are masked.
  const int krow = perm23(ql);
  u32x4 kf[2 * NC];
  auto load_k = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint16_t* row = Kh + (int64_t)min(kt * BN + kb * 32 + krow, (int)N - 1) * D + g * 8;
#pragma unroll
      for (int c = 0; c < NC; ++c) kf[kb * NC + c] = *(const u32x4*)(row + c * 16);
    }
  };

  // Q^T fragments, resident in AGPRs for the whole walk (rows past N
  // re-read row N-1 and are not stored).  All loads are issued before the
  // first move, so they overlap.
  u32x4 qa[QB][NC], qv[QB][NC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const uint16_t* row = Qh + (int64_t)min(q0 + 32 * qb + ql, (int)N - 1) * D + g * 8;
#pragma unroll
    for (int c = 0; c < NC; ++c) qv[qb][c] = *(const u32x4*)(row + c * 16);
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int c = 0; c < NC; ++c) asm volatile("s_nop 1" : "=a"(qa[qb][c]) : "0"(qv[qb][c]));

  // V^T reads: lane j of 16-lane group vq reads row 8g + j/4 (+4 for the
  // second half) at columns 32db + 16(vq%2) + 4(j%4).
  const int vj = lane & 15, vq = lane >> 4;
  const int v_row0 = 8 * g + (vj >> 2);
  const int v_col = 16 * (vq & 1) + 4 * (vj & 3);
  const uint32_t v_off0 = dual_chunk<RC>(v_row0, v_col >> 3) * 16 + (v_col & 7) * 2;
  const uint32_t v_off1 = dual_chunk<RC>(v_row0 + 4, v_col >> 3) * 16 + (v_col & 7) * 2;

  f32x16 oacc[QB][D / 32];
  // Reference state of each query block (as in the tiled forward): r_raw is
  // one of the raw scores; in the usual case exponents are one FMA against
  // mref = RN(r_raw*c2); raw_mode shifts scores by r_raw first when some
  // reference of the wave is too large for that FMA to be accurate.
  float r_raw[QB], mref[QB], mlazy[QB], m_use[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[qb][i] = f32x16{};
    r_raw[qb] = mref[qb] = mlazy[qb] = -INFINITY;
    m_use[qb] = l_run[qb] = 0.f;
  }
  bool raw_mode = false;
  const float c2 = a.scale_log2;

  // Issue order, which the waits below rely on (loads complete in order):
  // per step t, K(t+1) before the P V products and V(t+VS) after them;
  // first V(0) K(0) V(1) .. V(VS-1) when VS > 1, so that V(t) precedes K(t)
  // and the wait for K(t) also covers V(t); K(0) V(0) when VS = 1.
  int kt = wave;
  if (kt < n_kt) {
    if (VS == 1) load_k(kt);
#pragma unroll
    for (int st = 0; st < VS; ++st) {
      const int kv = kt + st * kShortWaves;
      if (kv < n_kt)
        copy_tile_wave<D, LPW, NX>(Vh + (int64_t)kv * BN * D, min(BN, (int)N - kv * BN), vsrc, vring + st * TC);
      if (VS > 1 && st == 0) load_k(kt);
    }
  }
  for (int step = 0; kt < n_kt; kt += kShortWaves, ++step) {
    const int k0 = kt * BN;
    const bool more = kt + kShortWaves < n_kt;
    // K of this tile (and with VS > 1 its V) has landed.
    if (VS > 1 && more)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPW) : "memory");
    else if (VS > 1)
      wait_vmem();
    else
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPW) : "memory");
    f32x16 s[QB][2];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          if (c == 0)
            mfma_s_first<T, true>(s[qb][kb], kf[kb * NC + c], qa[qb][c]);
          else
            mfma_s_acc<T, true>(s[qb][kb], kf[kb * NC + c], qa[qb][c]);
        }
    scores_ready(s);

    // Mask: keys above the diagonal and keys past N (uniform test per
    // tile).  Key k0 + 32kb + acc_row(r, g) is hidden from query q iff it
    // exceeds lim = min(q, N-1); acc_row(r, g) = 8g + (a constant of r), so
    // each element is one compare of a constant against lim - k0 - 32kb - 8g.
    // (The compare and select are written out so that each costs one
    // instruction with VCC, not a mask pair per element.)
    if ((CAUSAL && k0 + BN - 1 > q0) || k0 + BN > N) {
      const float ninf = -INFINITY;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int lim = CAUSAL ? min(q0 + 32 * qb + ql, (int)N - 1) : (int)N - 1;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int t = lim - k0 - 32 * kb - 8 * g;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            asm("v_cmp_gt_i32_e32 vcc, %1, %2\n\tv_cndmask_b32_e32 %0, %0, %3, vcc"
                : "+v"(s[qb][kb][r])
                : "i"(acc_row(r, 0)), "v"(t), "v"(ninf)
                : "vcc");
        }
      }
    }
    float mx[QB];
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // Four independent chains: one wave per SIMD hides no dependent latency.
      float m4[4] = {s[qb][0][0], s[qb][0][1], s[qb][1][0], s[qb][1][1]};
#pragma unroll
      for (int r = 2; r < 16; r += 2) {
        m4[0] = fmaxf(m4[0], s[qb][0][r]);
        m4[1] = fmaxf(m4[1], s[qb][0][r + 1]);
        m4[2] = fmaxf(m4[2], s[qb][1][r]);
        m4[3] = fmaxf(m4[3], s[qb][1][r + 1]);
      }
      // This lane's half of the keys: enough for the vote (scale > 0, so the
      // full max crosses the threshold exactly when one half does).
      mx[qb] = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
      need = need || (mx[qb] * c2 > mlazy[qb]);
    }
    if (wave_any(need)) {
      // Raise the references (rare after the first tile).
      float r_new[QB];
      bool big = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        r_new[qb] = fmaxf(r_raw[qb], xhalf_max(mx[qb]));
        const float nm = r_new[qb] * c2;
        big = big || (fabsf(nm) >= kShortFastLimit && nm != -INFINITY);
      }
      const bool raw_new = wave_any(big);
      if (step > 0) {  // before the wave's first tile O and l are still zero
        o_ready(oacc);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float lg = (raw_mode || raw_new) ? (r_raw[qb] - r_new[qb]) * c2 : mref[qb] - r_new[qb] * c2;
          const float alpha = (r_raw[qb] == -INFINITY) ? 0.f : fast_exp2(lg);
          l_run[qb] *= alpha;
#pragma unroll
          for (int i = 0; i < D / 32; ++i) oacc[qb][i] *= alpha;
        }
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float nm = r_new[qb] * c2;
        r_raw[qb] = r_new[qb];
        mref[qb] = nm;
        mlazy[qb] = nm + kShortLazy;
        m_use[qb] = (nm == -INFINITY) ? 0.f : nm;
      }
      raw_mode = raw_new;
    }
    // Probabilities, the P^T operands (16 keys each) and the row sums: fp16
    // sums the rounded probabilities that weight V, bf16 the FP32 ones.
    u32x4 pf[QB][BN / 16];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mu = m_use[qb];
      if (raw_mode) {
        const float ru = (r_raw[qb] == -INFINITY) ? 0.f : r_raw[qb];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[qb][kb] -= ru;
        mu = 0.f;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[qb][kb][r] = fast_exp2(__builtin_fmaf(s[qb][kb][r], c2, -mu));
      float ls[BN / 16];  // one partial sum per operand: independent chains
#pragma unroll
      for (int t = 0; t < BN / 16; ++t) {
        pf[qb][t] = pack8<T>(s[qb][t >> 1], (t & 1) * 8);
        ls[t] = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          if constexpr (T::id == Fp16::id) {
            ls[t] = add_pair<T>(pf[qb][t][w], ls[t]);
          } else {
            ls[t] += s[qb][t >> 1][(t & 1) * 8 + 2 * w];
            ls[t] += s[qb][t >> 1][(t & 1) * 8 + 2 * w + 1];
          }
        }
      }
      l_run[qb] += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    }

    // K of this wave's next tile, into the registers the score MFMAs read;
    // issued here rather than right after them so that it is not live
    // beside the scores.
    if (more) load_k(kt + kShortWaves);

    // O^T += V^T P^T; each V^T fragment feeds the QB query blocks.
    if constexpr (VS == 1) {
      if (more)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NC) : "memory");
      else
        wait_vmem();
    }
    const int st = VS == 1 ? 0 : (step % VS);
    const char* __restrict__ Vl = (const char*)(vring + st * TC);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int t = i / (D / 32), db = i % (D / 32);
      const u32x2 lo = lds_read_tr16(Vl + (v_off0 ^ (64 * db)) + t * 16 * RC * 16);
      const u32x2 hi = lds_read_tr16(Vl + (v_off1 ^ (64 * db)) + t * 16 * RC * 16);
      const u32x4 vf = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) mfma_o<T, true>(oacc[qb][db], vf, pf[qb][t]);
    }
    // V of the tile VS steps ahead goes into this buffer once every read
    // above has returned.
    const int kn = kt + VS * kShortWaves;
    if (kn < n_kt) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      copy_tile_wave<D, LPW, NX>(Vh + (int64_t)kn * BN * D, min(BN, (int)N - kn * BN), vsrc, vring + st * TC);
    }
  }
  wait_vmem();
  o_ready(oacc);

  // Merge.  Each wave's state is relative to its own references: 2^mref in
  // the fast mode, 2^(r_raw*c2) in raw mode.  Every wave publishes its
  // outputs and, per row, its sum, reference and the residual r_raw*c2 -
  // mref of the fast mode; then wave w finishes query block w/2, half of
  // the head dimension, weighting each part by 2^((r_raw - R)*c2 - residual)
  // with R the largest reference of the row, a part with no visible key by 0.
  {
    float* const ob = (float*)vring;  // [QB][D/32][4][64 lanes][4]
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          *(f32x4*)(ob + (((qb * (D / 32) + db) * 4 + rq) * 64 + lane) * 4) =
              f32x4{oacc[qb][db][rq * 4], oacc[qb][db][rq * 4 + 1], oacc[qb][db][rq * 4 + 2],
                    oacc[qb][db][rq * 4 + 3]};
      lds_ml[wave][qb][0][lane] = r_raw[qb];
      lds_ml[wave][qb][1][lane] = (raw_mode || r_raw[qb] == -INFINITY) ? 0.f : __builtin_fmaf(r_raw[qb], c2, -mref[qb]);
      lds_ml[wave][qb][2][lane] = xhalf_sum(l_run[qb]);
    }
  }
  __syncthreads();

  // A lane's output is U units of four floats, unit (qb*(D/32) + db)*4 + rq
  // holding O^T accumulator registers 4rq .. 4rq+3 of block (qb, db); wave w
  // finishes units w*UW .. w*UW + UW-1, all of one query block mq.
  constexpr int NDB = D / 32;
  constexpr int UW = QB * NDB * 4 / kShortWaves;
  const int u0 = wave * UW;
  const int mq = u0 / (NDB * 4);
  float R = -INFINITY;
#pragma unroll
  for (int w = 0; w < kShortWaves; ++w) R = fmaxf(R, lds_ml[w][mq][0][lane]);
  // R is finite: key 0 is visible to every query.
  float wt[kShortWaves], L = 0.f;
#pragma unroll
  for (int w = 0; w < kShortWaves; ++w) {
    const float rw = lds_ml[w][mq][0][lane];
    wt[w] = (rw == -INFINITY) ? 0.f : fast_exp2((rw - R) * c2 - lds_ml[w][mq][1][lane]);
    L += wt[w] * lds_ml[w][mq][2][lane];
  }
  // All parts are read before any is used, so the LDS reads overlap.
  f32x4 part[kShortWaves][UW];
#pragma unroll
  for (int w = 0; w < kShortWaves; ++w) {
    const float* obw = (const float*)lds_v[w];
#pragma unroll
    for (int j = 0; j < UW; ++j) part[w][j] = *(const f32x4*)(obw + ((u0 + j) * 64 + lane) * 4);
  }
  __builtin_amdgcn_sched_barrier(0);
  f32x4 acc[UW];
#pragma unroll
  for (int j = 0; j < UW; ++j) {
    acc[j] = wt[0] * part[0][j];
#pragma unroll
    for (int w = 1; w < kShortWaves; ++w) acc[j] += wt[w] * part[w][j];
  }
  const int my_q = q0 + 32 * mq + ql;
  if (my_q < N) {
    const float inv = 1.f / L;
    uint16_t* Orow = a.o + head + (int64_t)my_q * D;
#pragma unroll
    for (int j = 0; j < UW; ++j) {
      const int u = u0 + j, db = (u >> 2) % NDB, rq = u & 3;
      u32x2 o2;
      o2[0] = pack2<T>(acc[j][0] * inv, acc[j][1] * inv);
      o2[1] = pack2<T>(acc[j][2] * inv, acc[j][3] * inv);
      *(u32x2*)(Orow + db * 32 + rq * 8 + g * 4) = o2;
    }
    if (u0 % (NDB * 4) == 0 && g == 0) a.lse[(int64_t)bh * N + my_q] = (R * c2 + __log2f(L)) * kLn2;
  }
}

// Head size 128: the same cut (64 queries per workgroup, keys split over
// the four waves, merge in LDS), with a wave's two 32-query blocks software-
// pipelined against each other so that every MFMA has the other block's
// vector work beside it.  A tile is four phases of 16 MFMA slots:
//   C: scores of block 1 (tile t)       | exponentials, packs of block 0 (t)
//   D: P V of block 0 (t)               | row max of block 1 (t), row sums
//                                         of block 0, K fragments of t+1
//   A: scores of block 0 (tile t+1)     | exponentials, packs of block 1 (t)
//   B: P V of block 1 (t)               | row max of block 0 (t+1), row sums
//                                         of block 1
// each slot closed by a scheduling barrier.  Block 0's rescale decision for
// tile t+1 is taken after B, block 1's for tile t after D, so each block's
// reference is settled before its exponentials.  The V ring has two stages,
// held in two LDS objects so that the compiler can tell the reads of one
// stage from the copies in flight into the other; V of tile t is read in D
// and B of its step and V of t+2 is copied into its stage after B.  On a
// wave's last tile phase A computes scores from its own tile's K fragments
// again and discards them (skipping them in a branch measured slower on long
// walks); the pipeline pays off from about four tiles per wave, so shorter
// sequences take fwd_short_kernel.

// 16 wait states after the MFMAs that wrote one query block's two score
// accumulators (or its four output accumulators), before vector access.
__device__ __forceinline__ void block_scores_ready(f32x16 (&s)[2]) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1]));
}
__device__ __forceinline__ void block_o_ready(f32x16 (&o)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]));
}

template <bool CAUSAL, class T>
__global__ __launch_bounds__(kShortThreads, 1) void fwd_short_pipe_kernel(FwdArgs a) {
  constexpr int D = 128, BN = kShortBN, WQ = 64;
  constexpr int RC = D / 8, TC = BN * RC, LPW = TC / 64, NX = RC / 4, NC = D / 16, NDB = D / 32;
  constexpr int NSL = 16;  // slots per phase: 2*NC score MFMAs = 4*NDB P V MFMAs per block
  constexpr int PV = 2;    // V^T fragments read ahead of their MFMAs
  static_assert(2 * NC == NSL && 4 * NDB == NSL, "phase length");

  __shared__ u32x4 lds_vs0[kShortWaves][TC], lds_vs1[kShortWaves][TC];
  __shared__ float lds_ml[kShortWaves][2][3][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, g = lane >> 5;

  const int64_t N = a.N;
  const int G = a.H / a.Hkv;
  const int bh = head_of_slot(blockIdx.x % a.BH, a.BH, G);
  const int rank = blockIdx.x / a.BH;
  const int qt = CAUSAL ? (a.n_qtiles - 1 - rank) : rank;
  const int q0 = qt * WQ;
  const int64_t head = (int64_t)bh * N * D;
  const int64_t kv_head = (int64_t)(bh / G) * N * D;
  const uint16_t* __restrict__ Qh = a.q + head;
  const uint16_t* __restrict__ Kh = a.k + kv_head;
  const uint16_t* __restrict__ Vh = a.v + kv_head;

  const int n_kt_all = (int)((N + BN - 1) / BN);
  const int n_kt = CAUSAL ? min(n_kt_all, (q0 + WQ - 1) / BN + 1) : n_kt_all;

  int vsrc[NX];
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    const int p = x * 64 + lane, r = p / RC;
    vsrc[x] = (r * D + ((p % RC) ^ dual_xor<RC>(r)) * 8) * 2;
  }
  u32x4* const vst0 = lds_vs0[wave];
  u32x4* const vst1 = lds_vs1[wave];

  // K fragment f = kb*NC + c of lane (ql, g): K[64kt + 32kb + perm23(ql)][16c + 8g .. +8].
  const int krow = perm23(ql);
  u32x4 kf[2 * NC];
  auto k_ptr = [&](int kt, int kb) __attribute__((always_inline)) {
    return Kh + (int64_t)min(kt * BN + kb * 32 + krow, (int)N - 1) * D + g * 8;
  };

  u32x4 qa[2][NC], qv[2][NC];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const uint16_t* row = Qh + (int64_t)min(q0 + 32 * qb + ql, (int)N - 1) * D + g * 8;
#pragma unroll
    for (int c = 0; c < NC; ++c) qv[qb][c] = *(const u32x4*)(row + c * 16);
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int c = 0; c < NC; ++c) asm volatile("s_nop 1" : "=a"(qa[qb][c]) : "0"(qv[qb][c]));

  const int vj = lane & 15, vq = lane >> 4;
  const int v_row0 = 8 * g + (vj >> 2);
  const int v_col = 16 * (vq & 1) + 4 * (vj & 3);
  const uint32_t v_off0 = dual_chunk<RC>(v_row0, v_col >> 3) * 16 + (v_col & 7) * 2;
  const uint32_t v_off1 = dual_chunk<RC>(v_row0 + 4, v_col >> 3) * 16 + (v_col & 7) * 2;

  f32x16 oacc[2][NDB];
  float r_raw[2], mref[2], mlazy[2], m_use[2], mu[2], l_run[2], mx[2];
  bool raw_mode[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[qb][i] = f32x16{};
    r_raw[qb] = mref[qb] = mlazy[qb] = -INFINITY;
    m_use[qb] = mu[qb] = l_run[qb] = 0.f;
    raw_mode[qb] = false;
  }
  const float c2 = a.scale_log2;
  f32x16 s[2][2];
  u32x4 pf[2][4];
  float mp[4], ls[4];

  // Score MFMA i of block qb: accumulator kb = i % 2, chunk c = i / 2.
  auto s_mfma = [&](int qb, int i) __attribute__((always_inline)) {
    const int c = i >> 1, kb = i & 1;
    if (c == 0)
      mfma_s_first<T, true>(s[qb][kb], kf[kb * NC + c], qa[qb][c]);
    else
      mfma_s_acc<T, true>(s[qb][kb], kf[kb * NC + c], qa[qb][c]);
  };
  // K fragment of score slot i (issued one phase before that slot).
  auto k_load = [&](int kt, int i) __attribute__((always_inline)) {
    const int c = i >> 1, kb = i & 1;
    kf[kb * NC + c] = *(const u32x4*)(k_ptr(kt, kb) + c * 16);
  };
  // V^T fragment of P V slot i: keys 16*(i/4) .., columns 32*(i%4) ..
  auto v_read = [&](const u32x4* vb, int i) __attribute__((always_inline)) {
    const char* base = (const char*)vb + (i >> 2) * 16 * RC * 16;
    const int db = i & 3;
    const u32x2 lo = lds_read_tr16(base + (v_off0 ^ (64 * db)));
    const u32x2 hi = lds_read_tr16(base + (v_off1 ^ (64 * db)));
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  // Element pair p (0..15) of block qb in operand order: operand p/4,
  // accumulator (p/4)/2, registers ((p/4)%2)*8 + 2*(p%4), +1.
  auto exp_pair = [&](int qb, int p) __attribute__((always_inline)) {
    const int o = p >> 2, kb = o >> 1, r = (o & 1) * 8 + 2 * (p & 3);
    float e0 = fast_exp2(__builtin_fmaf(s[qb][kb][r], c2, -mu[qb]));
    float e1 = fast_exp2(__builtin_fmaf(s[qb][kb][r + 1], c2, -mu[qb]));
    // Computed in this slot: an empty volatile asm keeps IR-level passes
    // from sinking the work past the slot's MFMA (volatile asm stays in order).
    asm volatile("" : "+v"(e0), "+v"(e1));
    s[qb][kb][r] = e0;
    s[qb][kb][r + 1] = e1;
  };
  auto max_pair = [&](int qb, int p) __attribute__((always_inline)) {
    const int o = p >> 2, kb = o >> 1, r = (o & 1) * 8 + 2 * (p & 3);
    mp[p & 3] = fmaxf(mp[p & 3], fmaxf(s[qb][kb][r], s[qb][kb][r + 1]));
    asm volatile("" : "+v"(mp[p & 3]));
  };
  // Row-sum share of slot i: dword i%4 of operand i/4 (fp16: the rounded
  // probabilities that weight V; bf16: the FP32 ones).
  auto sum_dw = [&](int qb, int i) __attribute__((always_inline)) {
    const int o = i >> 2, w = i & 3;
    if constexpr (T::id == Fp16::id) {
      ls[o] = add_pair<T>(pf[qb][o][w], ls[o]);
    } else {
      const int kb = o >> 1, r = (o & 1) * 8 + 2 * w;
      ls[o] += s[qb][kb][r];
      ls[o] += s[qb][kb][r + 1];
    }
    asm volatile("" : "+v"(ls[o]));
  };
  auto mask_block = [&](int qb, int k0) __attribute__((always_inline)) {
    if ((CAUSAL && k0 + BN - 1 > q0 + 32 * qb) || k0 + BN > N) {
      const float ninf = -INFINITY;
      const int lim = CAUSAL ? min(q0 + 32 * qb + ql, (int)N - 1) : (int)N - 1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int t = lim - k0 - 32 * kb - 8 * g;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          asm("v_cmp_gt_i32_e32 vcc, %1, %2\n\tv_cndmask_b32_e32 %0, %0, %3, vcc"
              : "+v"(s[qb][kb][r])
              : "i"(acc_row(r, 0)), "v"(t), "v"(ninf)
              : "vcc");
      }
    }
  };
  // Reference of block qb for its current tile (see the tiled forward:
  // lazy by kLazy in log2 units; raw mode for huge references); first: no
  // tile of this block has been accumulated yet, so O and l are still zero.
  auto decide = [&](int qb, bool first) __attribute__((always_inline)) {
    if (wave_any(mx[qb] * c2 > mlazy[qb])) {
      const float r_new = fmaxf(r_raw[qb], xhalf_max(mx[qb]));
      const float nm = r_new * c2;
      const bool raw_new = wave_any(fabsf(nm) >= kShortFastLimit && nm != -INFINITY);
      if (!first) {
        const float lg = (raw_mode[qb] || raw_new) ? (r_raw[qb] - r_new) * c2 : mref[qb] - nm;
        const float alpha = (r_raw[qb] == -INFINITY) ? 0.f : fast_exp2(lg);
        block_o_ready(oacc[qb]);
        l_run[qb] *= alpha;
#pragma unroll
        for (int i = 0; i < NDB; ++i) oacc[qb][i] *= alpha;
      }
      r_raw[qb] = r_new;
      mref[qb] = nm;
      mlazy[qb] = nm + kShortLazy;
      m_use[qb] = (nm == -INFINITY) ? 0.f : nm;
      raw_mode[qb] = raw_new;
    }
    mu[qb] = m_use[qb];
    if (raw_mode[qb]) {
      const float ru = (r_raw[qb] == -INFINITY) ? 0.f : r_raw[qb];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[qb][kb] -= ru;
      mu[qb] = 0.f;
    }
  };
  auto reset_max = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 4; ++c) mp[c] = -INFINITY;
  };
  auto reset_sum = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < 4; ++c) ls[c] = 0.f;
  };
  auto fold_max = [&]() __attribute__((always_inline)) {
    // This lane's half of the keys: enough for the rescale vote, which
    // exchanges lane halves only when it raises the reference.
    return fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
  };
  auto fold_sum = [&]() __attribute__((always_inline)) { return (ls[0] + ls[1]) + (ls[2] + ls[3]); };

  // Prologue: V of the first two tiles, K of the first; scores of block 0
  // for the first tile, its max and reference.
  int kt = wave;
  if (kt < n_kt) {
    copy_tile_wave<D, LPW, NX>(Vh + (int64_t)kt * BN * D, min(BN, (int)N - kt * BN), vsrc, vst0);
#pragma unroll
    for (int i = 0; i < NSL; ++i) k_load(kt, i);
    const int k1 = kt + kShortWaves;
    if (k1 < n_kt) copy_tile_wave<D, LPW, NX>(Vh + (int64_t)k1 * BN * D, min(BN, (int)N - k1 * BN), vsrc, vst1);
#pragma unroll
    for (int i = 0; i < NSL; ++i) s_mfma(0, i);
    block_scores_ready(s[0]);
    mask_block(0, kt * BN);
    reset_max();
#pragma unroll
    for (int p = 0; p < NSL; ++p) max_pair(0, p);
    mx[0] = fold_max();
    decide(0, true);
  }

  for (int step = 0; kt < n_kt;) {
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      if (kt < n_kt) {
        const bool more = kt + kShortWaves < n_kt;
        const int kn = more ? kt + kShortWaves : kt;  // the last step re-reads K of its own tile
        const u32x4* vb = par ? vst1 : vst0;
        // C: scores of block 1 | exponentials and packs of block 0.
#pragma unroll
        for (int i = 0; i < NSL; ++i) {
          s_mfma(1, i);
          exp_pair(0, i);
          if ((i & 3) == 3) {
            pf[0][i >> 2] = pack8<T>(s[0][i >> 3], ((i >> 2) & 1) * 8);
            asm volatile("" : "+v"(pf[0][i >> 2]));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        block_scores_ready(s[1]);
        mask_block(1, kt * BN);
        reset_max();
        reset_sum();
        // D: P V of block 0 | max of block 1, row sums of block 0, K of the next tile.
        u32x4 vqr[PV + 1];
#pragma unroll
        for (int i = 0; i < PV; ++i) vqr[i] = v_read(vb, i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NSL; ++i) {
          if (i + PV < NSL) vqr[(i + PV) % (PV + 1)] = v_read(vb, i + PV);
          mfma_o<T, true>(oacc[0][i & 3], vqr[i % (PV + 1)], pf[0][i >> 2]);
          max_pair(1, i);
          sum_dw(0, i);
          k_load(kn, i);
          __builtin_amdgcn_sched_barrier(0);
        }
        l_run[0] += fold_sum();
        mx[1] = fold_max();
        decide(1, step == 0);
        // A: scores of block 0 for the next tile | exponentials and packs of block 1.
#pragma unroll
        for (int i = 0; i < NSL; ++i) {
          s_mfma(0, i);
          exp_pair(1, i);
          if ((i & 3) == 3) {
            pf[1][i >> 2] = pack8<T>(s[1][i >> 3], ((i >> 2) & 1) * 8);
            asm volatile("" : "+v"(pf[1][i >> 2]));
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        block_scores_ready(s[0]);
        if (more) mask_block(0, kn * BN);
        reset_max();
        reset_sum();
        // B: P V of block 1 | max of block 0 (next tile), row sums of block 1.
#pragma unroll
        for (int i = 0; i < PV; ++i) vqr[i] = v_read(vb, i);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NSL; ++i) {
          if (i + PV < NSL) vqr[(i + PV) % (PV + 1)] = v_read(vb, i + PV);
          mfma_o<T, true>(oacc[1][i & 3], vqr[i % (PV + 1)], pf[1][i >> 2]);
          max_pair(0, i);
          sum_dw(1, i);
          __builtin_amdgcn_sched_barrier(0);
        }
        l_run[1] += fold_sum();
        if (more) {
          mx[0] = fold_max();
          decide(0, false);
        }
        // V of the tile two steps ahead into this step's stage, once its reads have returned.
        const int k2 = kt + 2 * kShortWaves;
        if (k2 < n_kt) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          copy_tile_wave<D, LPW, NX>(Vh + (int64_t)k2 * BN * D, min(BN, (int)N - k2 * BN), vsrc,
                                     par ? vst1 : vst0);
        }
        kt += kShortWaves;
        ++step;
      }
    }
  }
  wait_vmem();
  o_ready(oacc);

  // Merge, as in fwd_short_kernel: every wave publishes its partial O (both
  // stages of its ring hold the 32 KB) and per-row state; wave w finishes
  // units w*8 .. w*8+7 (query block w/2, half of the head dimension).
  {
    float* const ob0 = (float*)vst0;
    float* const ob1 = (float*)vst1;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float* const ob = qb ? ob1 : ob0;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          *(f32x4*)(ob + ((db * 4 + rq) * 64 + lane) * 4) =
              f32x4{oacc[qb][db][rq * 4], oacc[qb][db][rq * 4 + 1], oacc[qb][db][rq * 4 + 2],
                    oacc[qb][db][rq * 4 + 3]};
      lds_ml[wave][qb][0][lane] = r_raw[qb];
      lds_ml[wave][qb][1][lane] =
          (raw_mode[qb] || r_raw[qb] == -INFINITY) ? 0.f : __builtin_fmaf(r_raw[qb], c2, -mref[qb]);
      lds_ml[wave][qb][2][lane] = xhalf_sum(l_run[qb]);
    }
  }
  __syncthreads();

  constexpr int UW = 2 * NDB * 4 / kShortWaves;  // 8 units per wave
  const int mq = wave >> 1, u0 = (wave & 1) * UW;  // units of block mq: (db*4 + rq)
  float R = -INFINITY;
#pragma unroll
  for (int w = 0; w < kShortWaves; ++w) R = fmaxf(R, lds_ml[w][mq][0][lane]);
  float wt[kShortWaves], L = 0.f;
#pragma unroll
  for (int w = 0; w < kShortWaves; ++w) {
    const float rw = lds_ml[w][mq][0][lane];
    wt[w] = (rw == -INFINITY) ? 0.f : fast_exp2((rw - R) * c2 - lds_ml[w][mq][1][lane]);
    L += wt[w] * lds_ml[w][mq][2][lane];
  }
  f32x4 part[kShortWaves][UW];
#pragma unroll
  for (int w = 0; w < kShortWaves; ++w) {
    const float* obw = (const float*)(mq ? lds_vs1[w] : lds_vs0[w]);
#pragma unroll
    for (int j = 0; j < UW; ++j) part[w][j] = *(const f32x4*)(obw + ((u0 + j) * 64 + lane) * 4);
  }
  __builtin_amdgcn_sched_barrier(0);
  const int my_q = q0 + 32 * mq + ql;
  if (my_q < N) {
    const float inv = 1.f / L;
    uint16_t* Orow = a.o + head + (int64_t)my_q * D;
#pragma unroll
    for (int j = 0; j < UW; ++j) {
      f32x4 acc = wt[0] * part[0][j];
#pragma unroll
      for (int w = 1; w < kShortWaves; ++w) acc += wt[w] * part[w][j];
      const int u = u0 + j, db = u >> 2, rq = u & 3;
      u32x2 o2;
      o2[0] = pack2<T>(acc[0] * inv, acc[1] * inv);
      o2[1] = pack2<T>(acc[2] * inv, acc[3] * inv);
      *(u32x2*)(Orow + db * 32 + rq * 8 + g * 4) = o2;
    }
    if (u0 == 0 && g == 0) a.lse[(int64_t)bh * N + my_q] = (R * c2 + __log2f(L)) * kLn2;
  }
}

// D = 64 takes one query block per wave (measured faster for the smallest
// grids, where two workgroups share a CU); D = 128 two.
template <int D, bool CAUSAL, class T>
hipError_t launch_short_t(FwdArgs a, hipStream_t stream) {
  constexpr int QB = D == 64 ? 1 : 2;
  a.n_qtiles = (int)((a.N + 32 * QB - 1) / (32 * QB));
  const int64_t n_wg = (int64_t)a.BH * a.n_qtiles;
  // D = 128 from N = 1024 (a wave walks at least four tiles when causal):
  // the pipelined kernel; measured slower than the plain one below that.
  if (short_pipelined(a.N, D))
    hipLaunchKernelGGL((fwd_short_pipe_kernel<CAUSAL, T>), dim3((unsigned)n_wg), dim3(kShortThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_short_kernel<D, QB, CAUSAL, T>), dim3((unsigned)n_wg), dim3(kShortThreads), 0, stream,
                       a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_short(const FwdArgs& a, int D, bool causal, int dtype, hipStream_t stream) {
#define FA_SHORT_CASE(DD, CC, TT) \
  if (D == DD && causal == CC && dtype == TT::id) return launch_short_t<DD, CC, TT>(a, stream);
  FA_SHORT_CASE(64, false, Fp16)
  FA_SHORT_CASE(64, true, Fp16)
  FA_SHORT_CASE(128, false, Fp16)
  FA_SHORT_CASE(128, true, Fp16)
  FA_SHORT_CASE(64, false, Bf16)
  FA_SHORT_CASE(64, true, Bf16)
  FA_SHORT_CASE(128, false, Bf16)
  FA_SHORT_CASE(128, true, Bf16)
#undef FA_SHORT_CASE
  return hipErrorInvalidValue;
}

}  // namespace fa
