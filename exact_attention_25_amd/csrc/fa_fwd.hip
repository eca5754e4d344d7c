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
// Grouped heads (GQA/MQA): a query head reads the K/V head of its group in
// place, never a copy ("CUDA FlashAttention ...", §7), and the workgroups of
// one group are numbered so that they share an XCD (head_of_slot).
//
// Work decomposition (one workgroup = 4 waves of one head):
//  * Each wave owns QB blocks of 32 queries (QB = 1 or 2).  Their Q rows stay
//    in VGPRs for the whole pass as the B operand of S^T = K Q^T (32 keys x
//    32 queries per MFMA).  With QB = 2 every K or V^T fragment read from
//    LDS feeds two independent MFMAs, halving LDS traffic per FLOP.
//  * Keys and values stream in tiles of 64 keys straight from HBM into a
//    double-buffered LDS ring (buffer_load_dwordx4 ... lds: no VGPR staging), one
//    workgroup barrier per tile.  Both tiles stay row-major with an XOR
//    swizzle of 16-byte chunks (K: swz, V: dual_chunk, each conflict-free
//    for its read); K fragments are read with ds_read_b128 and the V^T
//    fragments of O^T = V^T P^T with the transposing ds_read_b64_tr_b16, so
//    V is never transposed in memory.
//  * Computing S^T puts one query per lane (two lanes per query, 32 keys
//    each), so the row max is an in-lane reduction plus one cross-half swap,
//    and the row sum needs no cross-lane step until the epilogue.
//  * Softmax runs in base 2 with scale*log2(e) folded into one FMA.  Every
//    matrix instruction has vector work beside it: the exponentials of tile
//    j run between the score MFMAs of tile j+1 (K streams one tile ahead of
//    V), and the packing of tile j's probabilities and the row max of tile
//    j+1 run between the P V MFMAs of tile j.  On gfx950 an MFMA holds the
//    vector issue port only for part of its duration, so vector work placed
//    this way is largely hidden, and what is left is bounded by the count of
//    vector instructions per tile; the loop keeps that count low (read
//    offsets held in registers, a one-compare rescale decision).
//  * Workgroups are numbered heaviest-first for causal masks, and all query
//    tiles of one head get workgroup ids congruent modulo 8, so they run on
//    the same XCD and share its L2 for the re-streamed K/V.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr int kFwdBN = 64;   // keys per tile
// Query blocks per wave.  Two blocks halve LDS reads per MFMA but need about
// 420 live registers, i.e. one wave per SIMD; measured on MI355X that loses
// far more latency hiding than it saves (causal D=128: 210 vs 850 TFLOP/s),
// so the shipped tiling is one block per wave, two waves per SIMD.
constexpr int kFwdQB = 1;
constexpr int kFwdThreads = 256;
constexpr float kLazy = 8.0f;          // max probability 2^8 between rescales
constexpr float kFastLimit = 4096.0f;  // |scale*log2e*S| below this: one-FMA exponent

template <int QB>
struct FwdShape {
  static constexpr int BM = 32 * QB * (kFwdThreads / 64);  // queries per workgroup
};

// SPLIT: the workgroup covers only key tiles [kt_begin, kt_end) of its split
// (with MASK: its share of the list of non-empty tiles)
// and writes FP32 partial states (O normalised within the range, and the
// range's LSE) for merge_kernel instead of the final O and LSE.
// MASK: a key-padding mask given by its block-level flags (a.mask): the
// workgroup visits only the listed non-empty tiles, tests elements only in
// tiles whose visibility word is not all ones, and a row left with no
// visible key gets O = 0 and LSE = -inf.
// DROP: attention dropout ([FA-WHY]-style regeneration from a Philox seed
// and offset, see dropout_bits_st): dropped probabilities are zeroed before
// P weights V, the row sum l keeps the undropped ones (LSE is that of the
// undropped softmax), and O is multiplied by the keep scale at the end (with
// SPLIT, each split's O; the merge weights are those of the undropped LSEs).
template <int D, int QB, bool CAUSAL, class T, bool SPLIT, bool MASK, bool DROP>
__global__ __launch_bounds__(kFwdThreads, QB == 1 ? 2 : 1) void fwd_kernel(FwdArgs a) {
  constexpr int BM = FwdShape<QB>::BM, BN = kFwdBN, NT = kFwdThreads;
  constexpr int RC = D / 8;              // 16-byte chunks per row
  constexpr int TC = BN * RC;            // chunks per K or V tile
  constexpr int LPT = TC / NT;           // direct copies per thread per tile
  constexpr int WQ = 32 * QB;            // queries per wave
  static_assert(LPT * NT == TC, "tile split");

  // Two K and two V tile buffers as separate LDS objects, so the compiler
  // can tell reads of one buffer from the copies in flight into the other.
  __shared__ u32x4 lds_k0[TC], lds_k1[TC], lds_v0[TC], lds_v1[TC];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, g = lane >> 5;

  const int64_t N = a.N;
  const int G = a.H / a.Hkv;  // query heads per K/V head
  const int bh = head_of_slot(blockIdx.x % a.BH, a.BH, G);
  const int split = SPLIT ? (blockIdx.x / a.BH) % a.n_splits : 0;
  const int rank = SPLIT ? blockIdx.x / (a.BH * a.n_splits) : blockIdx.x / a.BH;
  const int qt = CAUSAL ? (a.n_qtiles - 1 - rank) : rank;
  const int64_t head = (int64_t)bh * N * D;
  const int64_t kv_head = (int64_t)(bh / G) * N * D;  // the K/V head this query head reads
  const uint16_t* __restrict__ Qh = a.q + head;
  const uint16_t* __restrict__ Kh = a.k + kv_head;
  const uint16_t* __restrict__ Vh = a.v + kv_head;

  const int q0w = qt * BM + wave * WQ;  // first query of this wave
  const bool active = q0w < N;          // the wave has at least one real query

  // Q^T operand fragments: lane (ql, g) of block qb holds
  // Q[q0w + 32qb + ql][16c + 8g .. +8].  Lanes past the last query re-read
  // row N-1; their results are never stored.
  u32x4 qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
      qf[qb][c] = active ? *(const u32x4*)(Qh + (int64_t)min(q0w + 32 * qb + ql, (int)N - 1) * D + c * 16 + g * 8)
                         : u32x4{0, 0, 0, 0};

  f32x16 oacc[QB][D / 32];
  float r_raw[QB], l_run[QB];  // reference max (raw score units); this lane's part of l
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[qb][i] = f32x16{};
    r_raw[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }

  const int n_kt_all = (int)((N + BN - 1) / BN);  // the last tile may be partial
  const int n_kt = CAUSAL ? min(n_kt_all, ((qt + 1) * BM) / BN) : n_kt_all;
  // The workgroup walks positions i_begin .. i_end-1 of a tile sequence:
  // without a mask position i is key tile i (all visible tiles, or this
  // split's share); with a mask it is the i-th non-empty tile of the list,
  // and the tiles before the causal limit n_kt are the first prefix[n_kt].
  int i_begin = 0, i_end;
  const int64_t b = MASK ? bh / a.H : 0;  // batch element (mask mode only)
  if constexpr (MASK) {
    const int i_all = a.mask.prefix[b * (a.mask.n_tiles + 1) + n_kt];
    i_begin = SPLIT ? (int)(((int64_t)split * i_all) / a.n_splits) : 0;
    i_end = SPLIT ? (int)(((int64_t)(split + 1) * i_all) / a.n_splits) : i_all;
  } else {
    i_begin = SPLIT ? (int)(((int64_t)split * n_kt_all) / a.n_splits) : 0;
    i_end = SPLIT ? min(n_kt, (int)(((int64_t)(split + 1) * n_kt_all) / a.n_splits)) : n_kt;
  }

  // Direct copies: copy i of wave w fills LDS chunks i*NT + 64w + lane.  The
  // per-lane source offsets (elements within a tile) differ between copies
  // only by a constant, because the swizzles depend on low row bits only.
  const int p0 = wave * 64 + lane;
  const int ksrc0 = swz(p0) * 8;
  const int vr0 = p0 / RC;
  const int vsrc0 = vr0 * D + ((p0 % RC) ^ dual_xor<RC>(vr0)) * 8;
  auto load_k = [&](int kt, u32x4* dst) {
    copy_tile_rows<D, LPT, NT>(Kh + (int64_t)kt * BN * D, ksrc0, dst + wave * 64, min(BN, (int)N - kt * BN));
  };
  auto load_v = [&](int kt, u32x4* dst) {
    copy_tile_rows<D, LPT, NT>(Vh + (int64_t)kt * BN * D, vsrc0, dst + wave * 64, min(BN, (int)N - kt * BN));
  };

  // S^T = K Q^T for one 64-key tile: two 32-key blocks, K rows read in
  // perm23 order so that register r of lane-half g holds key acc_row(r, g).
  // Each K fragment feeds the QB query blocks.
  const int krow = perm23(ql);
  // The swizzles XOR only chunk bits below the row, so the byte offset of K
  // row kb*32 + krow, chunk 2c + g is k_off ^ (32c), plus kb*32 rows as an
  // immediate.  The XORs are redone on every call (the empty asm makes the
  // base look new each time) so that only one base register stays live
  // instead of one address register per fragment and buffer.
  const uint32_t k_off = swz(krow * RC + g) * 16;
  auto scores = [&](const u32x4* __restrict__ Kl, f32x16 (&s)[QB][2]) {
    uint32_t kbase = k_off;
    asm volatile("" : "+v"(kbase));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb][kb] = f32x16{};
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const u32x4 kf = *(const u32x4*)((const char*)Kl + (kbase ^ (32 * c)) + kb * 32 * RC * 16);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32<T>(kf, qf[qb][c], s[qb][kb]);
      }
    }
  };

  // Lane-constant parts of the transposed V reads: lane j of 16-lane group q
  // reads row 8g + j/4 (+4 for the second half), columns d0 + 4*(j%4), with
  // d0 = 32*db + 16*(q%2).
  const int vj = lane & 15, vq = lane >> 4;
  const int v_row0 = 8 * g + (vj >> 2);
  const int v_col = 16 * (vq & 1) + 4 * (vj & 3);
  // V^T fragment (rows 16t + v_row0 + 4h, columns 32db + v_col): byte offset
  // v_off[h] ^ (64 db), plus 16t rows as an immediate.
  const uint32_t v_off0 = dual_chunk<RC>(v_row0, v_col >> 3) * 16 + (v_col & 7) * 2;
  const uint32_t v_off1 = dual_chunk<RC>(v_row0 + 4, v_col >> 3) * 16 + (v_col & 7) * 2;
  // All chunk-XORed read offsets stay in registers for the whole pass (they
  // differ only by XORs with constants, so they are formed once here).
  uint32_t k_addr[RC / 2], v_addr[2][D / 32];
#pragma unroll
  for (int c = 0; c < RC / 2; ++c) k_addr[c] = k_off ^ (32 * c);
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    v_addr[0][db] = v_off0 ^ (64 * db);
    v_addr[1][db] = v_off1 ^ (64 * db);
  }
  const float c2 = a.scale_log2;

  // Raw max over the tile of the pending scores, per query row; carried from
  // the step that computed those scores to the step that exponentiates them.
  // mx: a tile's row max over this lane's half of the keys (the two lanes
  // of a query each hold one half).  The rescale vote needs no more: with
  // scale > 0, max(h0, h1) * c2 > t exactly when h0 * c2 > t or h1 * c2 > t,
  // and the vote covers both lanes; only a rescale takes the full max.
  float mx[QB];

  // Mask of a tile's raw scores before its max: diagonal, partial last or
  // partially visible tiles only (a block wholly above its queries is masked
  // entirely and contributes zero probabilities; keys >= N do not exist).
  // The tests are uniform, so other tiles take no per-element branch.
  auto mask_tile = [&](f32x16 (&s)[QB][2], int k0, uint32_t wlo, uint32_t whi) __attribute__((always_inline)) {
    const bool partial = MASK ? (wlo & whi) != 0xffffffffu : k0 + BN > N;
    if ((CAUSAL && k0 + BN - 1 > q0w) || partial) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + acc_row(r, g);
            const bool hidden = MASK ? key_hidden(wlo, whi, kb, r, g) : key >= N;
            if ((CAUSAL && key > q0w + 32 * qb + ql) || hidden) s[qb][kb][r] = -INFINITY;
          }
    }
  };
  auto tile_max = [&](const f32x16 (&s)[QB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float m = s[qb][0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) m = fmaxf(m, s[qb][0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, s[qb][1][r]);
      mx[qb] = m;
    }
  };

  // Reference state.  The reference max r_raw is always one of the raw
  // scores (exact); mref = RN(r_raw*c2), m_use the same with -inf read as 0,
  // mlazy = mref + kLazy.  In the usual case the exponent is one FMA,
  // s*c2 - mref, and the reference is only raised (d_rescale) when a tile's
  // max exceeds it by more than kLazy in log2 units, so probabilities stay
  // below 2^kLazy and the O/l rescale is skipped on most tiles; the result is
  // unchanged because O and l always share the same reference.  When the
  // reference of some row of the wave is so large that RN(r_raw*c2) is off
  // by a meaningful amount (|mref| >= kFastLimit: raw_mode), the scores are
  // first shifted by r_raw in raw units, where the difference is exact for
  // scores near the max, and the same FMA then scales them.  A row's
  // exponents can only be large when its reference is, so the mode changes
  // only when a reference does.
  float mref[QB], m_use[QB], mlazy[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) mref[qb] = mlazy[qb] = -INFINITY, m_use[qb] = 0.f;
  bool raw_mode = false, d_rescale = false;
  // Decision for the pending tile, taken as soon as its max is known.
  auto decide = [&]() __attribute__((always_inline)) {
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) need = need || (mx[qb] * c2 > mlazy[qb]);
    d_rescale = wave_any(need);
  };

  // One position i of the tile sequence (key tile kt, its successors kt1
  // and kt2 at positions i+1 and i+2), software-pipelined so that every
  // matrix instruction has vector work beside it: on entry s holds the
  // masked raw scores of tile kt and mx their row max (both produced by the
  // previous step).  While the exponentials of tile kt run, the score MFMAs
  // of tile kt1 (its K is already in LDS) are issued into s_nxt; while the
  // P V MFMAs of tile kt run, the probabilities are packed just ahead of the
  // MFMA that consumes them and the row max of tile kt1 is taken.  K
  // therefore streams one tile ahead of V: the copies started here are K of
  // tile kt2 (into the buffer that held K of tile kt) and V of tile kt1.
  // wlo1/whi1: visibility word of tile kt1 (mask mode).
  auto step = [&](int i, int kt, int kt1, int kt2, uint32_t wlo1, uint32_t whi1, const u32x4* __restrict__ Knext,
                  const u32x4* __restrict__ Vcur, u32x4* kdst, u32x4* vdst, f32x16 (&s)[QB][2],
                  f32x16 (&s_nxt)[QB][2]) {
    wait_vmem();      // K of tile kt1 and V of tile kt have landed (this wave's part)
    __syncthreads();  // ... everyone's part; everyone is done with the previous tile
    if (i + 2 < i_end) load_k(kt2, kdst);
    if (i + 1 < i_end) load_v(kt1, vdst);

    const int k0 = kt * BN;
    if (!active || (CAUSAL && k0 > q0w + WQ - 1)) return;  // nothing visible

    // Raise the reference when decide asked for it (rare).
    if (d_rescale) {
      float r_new[QB];
      bool big = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        r_new[qb] = fmaxf(r_raw[qb], xhalf_max(mx[qb]));
        const float nm = r_new[qb] * c2;
        big = big || (fabsf(nm) >= kFastLimit && nm != -INFINITY);
      }
      const bool raw_new = wave_any(big);
      const bool raw_diff = raw_mode || raw_new;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float lg = raw_diff ? (r_raw[qb] - r_new[qb]) * c2 : mref[qb] - r_new[qb] * c2;
        const float alpha = (r_raw[qb] == -INFINITY) ? 0.f : fast_exp2(lg);
        l_run[qb] *= alpha;
#pragma unroll
        for (int i = 0; i < D / 32; ++i) oacc[qb][i] *= alpha;
        r_raw[qb] = r_new[qb];
        mref[qb] = r_new[qb] * c2;
        mlazy[qb] = mref[qb] + kLazy;
        m_use[qb] = (mref[qb] == -INFINITY) ? 0.f : mref[qb];
      }
      raw_mode = raw_new;
    }
    float mu[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) mu[qb] = m_use[qb];
    if (raw_mode) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float ru = (r_raw[qb] == -INFINITY) ? 0.f : r_raw[qb];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[qb][kb] -= ru;
        mu[qb] = 0.f;
      }
    }

    // Wave priority: the two waves sharing a SIMD are usually in different
    // phases; the one in its P V phase (one MFMA and few vector
    // instructions per slice) issues first, so its MFMAs keep the matrix
    // core fed while the other wave's exponentials fill the vector port
    // (measured +1 %).
    __builtin_amdgcn_s_setprio(0);
    // Scores of the next tile (its K is resident), software-pipelined with
    // the exponentials of this tile: slice i issues the K read for score
    // MFMA i + PK, score MFMA i, and 32/NS of the exponentials; a scheduling
    // barrier closes each slice so the reads stay PK MFMAs ahead.  On a
    // wave's last tile the score MFMAs read a stale buffer and the result is
    // discarded.
    {
      constexpr int NS = 2 * (D / 16);  // score MFMAs per tile
      constexpr int PK = 3;             // K fragments in flight
      constexpr int EPI = 32 / NS;      // exponentials per slice and query block
      const char* __restrict__ Kb = (const char*)Knext;
      u32x4 kq[PK + 1];
#pragma unroll
      for (int i = 0; i < PK; ++i)
        kq[i] = *(const u32x4*)(Kb + k_addr[i >> 1] + (i & 1) * 32 * RC * 16);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s_nxt[qb][0] = s_nxt[qb][1] = f32x16{};
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if (i + PK < NS) {
          const int j = i + PK;
          kq[j % (PK + 1)] = *(const u32x4*)(Kb + k_addr[j >> 1] + (j & 1) * 32 * RC * 16);
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s_nxt[qb][i & 1] = mfma32<T>(kq[i % (PK + 1)], qf[qb][i >> 1], s_nxt[qb][i & 1]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int e = 0; e < EPI; ++e) {
            const int idx = i * EPI + e;
            s[qb][idx >> 4][idx & 15] = fast_exp2(__builtin_fmaf(s[qb][idx >> 4][idx & 15], c2, -mu[qb]));
          }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // O^T += V^T P^T, 16 keys per MFMA: MFMA i uses keys 16t .. 16t+15 with
    // t = i / (D/32), which are accumulator registers 8*(t%2) .. +7 of block
    // t/2 (see acc_row).  V^T fragments run PV reads ahead of their MFMAs.
    // P = exp2(s*c2 - m) is packed to fp16/bf16 (round to nearest even) one
    // dword per slice, ahead of the MFMA that reads it; for fp16 the row sum
    // l adds the same rounded probabilities that weight V, pairwise in FP32
    // (v_dot2 with ones); bf16 keeps only 8 bits, so there l sums the FP32
    // values.  The slices also fold the next tile's raw scores into its row
    // max.
    constexpr int NV = (BN / 16) * (D / 32);  // P V MFMAs per tile
    constexpr int PV = 2;
    constexpr int NPK = NV - D / 32;          // slices that pack operands 1 .. BN/16-1
    constexpr int WPK = (4 * (BN / 16 - 1)) / NPK;  // dwords packed per such slice
    constexpr int MPS = 32 / NV;              // next-tile scores folded per slice
    static_assert(WPK * NPK == 4 * (BN / 16 - 1) && MPS * NV == 32, "slice split");
    const char* __restrict__ Vl = (const char*)Vcur;
    auto pv_phase = [&]() __attribute__((always_inline)) {
      auto vread = [&](int i) {
        const int t = i / (D / 32), db = i % (D / 32);
        const u32x2 lo = lds_read_tr16(Vl + v_addr[0][db] + t * 16 * RC * 16);
        const u32x2 hi = lds_read_tr16(Vl + v_addr[1][db] + t * 16 * RC * 16);
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
      u32x4 vq[PV + 1];
#pragma unroll
      for (int i = 0; i < PV; ++i) vq[i] = vread(i);

      u32x4 pf[QB][BN / 16];
      float lsum[QB], mn[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        lsum[qb] = 0.f;
        mn[qb] = -INFINITY;
      }
      // dword idx (0 .. 4*BN/16-1) of the packed operands: operand idx/4,
      // elements 2*(idx%4), +1 of its eight.
      auto pack_dw = [&](int idx) __attribute__((always_inline)) {
        const int t = idx >> 2, lo = (t & 1) * 8 + 2 * (idx & 3);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float x0 = s[qb][t >> 1][lo], x1 = s[qb][t >> 1][lo + 1];
          pf[qb][t][idx & 3] = pack2<T>(x0, x1);
          if constexpr (T::id == Fp16::id) {
            lsum[qb] = add_pair<T>(pf[qb][t][idx & 3], lsum[qb]);
          } else {
            lsum[qb] += x0;
            lsum[qb] += x1;
          }
          asm volatile("" : "+v"(lsum[qb]));  // the sum stays in this slice
        }
      };
      if constexpr (DROP) {
        // l sums the undropped FP32 probabilities; then the dropped ones are
        // zeroed before packing (the keep scale is applied to O at the end).
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) lsum[qb] += s[qb][kb][r];
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const uint32_t keep = dropout_bits_st(k0 + kb * 32, q0w + 32 * qb + ql, (uint64_t)bh, a.drop.seed,
                                                  a.drop.offset, a.drop.thr, g);
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (!((keep >> r) & 1u)) s[qb][kb][r] = 0.f;
          }
#pragma unroll
          for (int t = 0; t < BN / 16; ++t) pf[qb][t] = pack8<T>(s[qb][t >> 1], (t & 1) * 8);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) pack_dw(e);
      }
      __builtin_amdgcn_sched_barrier(0);

#pragma unroll
      for (int i = 0; i < NV; ++i) {
        if (i + PV < NV) vq[(i + PV) % (PV + 1)] = vread(i + PV);
        const int t = i / (D / 32), db = i % (D / 32);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = mfma32<T>(vq[i % (PV + 1)], pf[qb][t], oacc[qb][db]);
        if constexpr (!DROP) {
          if (i < NPK) {
#pragma unroll
            for (int w = 0; w < WPK; ++w) pack_dw(4 + i * WPK + w);
          }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int e = 0; e < MPS; ++e) {
            const int idx = i * MPS + e;
            mn[qb] = fmaxf(mn[qb], s_nxt[qb][idx >> 4][idx & 15]);
          }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) asm volatile("" : "+v"(mn[qb]));  // the max stays in this slice
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        l_run[qb] += lsum[qb];
        mx[qb] = mn[qb];
      }
      decide();
    };

    // The row max of tile kt1 is taken during the loop (on a last position
    // it is that of stale scores and never used); when tile kt1 needs a mask
    // it is masked afterwards and its max taken again.  Tile kt1 is pending
    // for the next step unless this is the last position or the whole tile
    // lies above this wave's queries.
    __builtin_amdgcn_s_setprio(1);
    pv_phase();
    const int k1 = kt1 * BN;
    const bool pending = i + 1 < i_end && !(CAUSAL && k1 > q0w + WQ - 1);
    const bool mask1 = (CAUSAL && k1 + BN - 1 > q0w) || (MASK ? (wlo1 & whi1) != 0xffffffffu : k1 + BN > N);
    if (pending && mask1) {
      asm volatile("");  // keeps this a branch: the masking is not speculated
      mask_tile(s_nxt, k1, wlo1, whi1);
      tile_max(s_nxt);
      decide();
    }
  };

  // Prologue: K and V of the first tile, K of the second, scores of the
  // first; then the steps, two per iteration so the LDS buffers alternate.
  f32x16 sA[QB][2], sB[QB][2];
  if constexpr (!MASK) {
    if (i_begin < i_end) {  // workgroup-uniform
      load_k(i_begin, lds_k0);
      load_v(i_begin, lds_v0);
      if (i_begin + 1 < i_end) load_k(i_begin + 1, lds_k1);
      wait_vmem();
      __syncthreads();
      constexpr uint32_t kAll = 0xffffffffu;
      if (active) {
        scores(lds_k0, sA);
        mask_tile(sA, i_begin * BN, kAll, kAll);
        tile_max(sA);
        decide();
      }
      for (int kt = i_begin; kt < i_end; kt += 2) {
        step(kt, kt, kt + 1, kt + 2, kAll, kAll, lds_k1, lds_v0, lds_k0, lds_v1, sA, sB);
        if (kt + 1 < i_end) step(kt + 1, kt + 1, kt + 2, kt + 3, kAll, kAll, lds_k0, lds_v1, lds_k1, lds_v0, sB, sA);
      }
    }
  } else if (i_begin < i_end) {  // workgroup-uniform
    TileWindow win;
    win.init(a.mask.list + b * a.mask.n_tiles, a.mask.words + b * a.mask.n_tiles, i_end, lane, i_begin);
    // Tiles at positions i and i+1 (carried from step to step), their words.
    int kt_c = win.tile(i_begin, lane);
    int kt_n = i_begin + 1 < i_end ? win.tile(i_begin + 1, lane) : 0;
    uint32_t w_lo, w_hi, wn_lo = 0, wn_hi = 0;
    win.word(i_begin, w_lo, w_hi);
    if (i_begin + 1 < i_end) win.word(i_begin + 1, wn_lo, wn_hi);
    load_k(kt_c, lds_k0);
    load_v(kt_c, lds_v0);
    if (i_begin + 1 < i_end) load_k(kt_n, lds_k1);
    wait_vmem();
    __syncthreads();
    if (active) {
      scores(lds_k0, sA);
      mask_tile(sA, kt_c * BN, w_lo, w_hi);
      tile_max(sA);
      decide();
    }
    // One position: the carried tiles advance by one and position i+2 is
    // looked up first (before the step's wait, which any window refill shares).
    auto run = [&](int i, const u32x4* Kn, const u32x4* Vc, u32x4* kd, u32x4* vd, f32x16 (&s)[QB][2],
                   f32x16 (&sn)[QB][2]) {
      int kt2 = 0;
      uint32_t lo2 = 0, hi2 = 0;
      if (i + 2 < i_end) {
        kt2 = win.tile(i + 2, lane);
        win.word(i + 2, lo2, hi2);
      }
      step(i, kt_c, kt_n, kt2, wn_lo, wn_hi, Kn, Vc, kd, vd, s, sn);
      kt_c = kt_n;
      kt_n = kt2;
      w_lo = wn_lo;
      w_hi = wn_hi;
      wn_lo = lo2;
      wn_hi = hi2;
    };
    for (int i = i_begin; i < i_end; i += 2) {
      run(i, lds_k1, lds_v0, lds_k0, lds_v1, sA, sB);
      if (i + 1 < i_end) run(i + 1, lds_k0, lds_v1, lds_k1, lds_v0, sB, sA);
    }
  }

  if (!active) return;
  if constexpr (SPLIT) {
    // Partial state of this split: O normalised within the split, FP32, and
    // the split's natural-log LSE; a row that saw no key in the split gets
    // O = 0 and LSE = -inf, which the merge weights by zero.
    const int64_t rows = (int64_t)a.BH * N;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int my_q = q0w + 32 * qb + ql;
      const float l_tot = xhalf_sum(l_run[qb]);
      const float inv = (l_tot > 0.f ? 1.f / l_tot : 0.f) * (DROP ? a.drop.keep_scale : 1.f);
      if (my_q >= N) continue;
      const int64_t row = (int64_t)bh * N + my_q;
      float* Orow = a.part_o + ((int64_t)split * rows + row) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq)
          *(f32x4*)(Orow + db * 32 + rq * 8 + g * 4) =
              f32x4{oacc[qb][db][rq * 4 + 0] * inv, oacc[qb][db][rq * 4 + 1] * inv,
                    oacc[qb][db][rq * 4 + 2] * inv, oacc[qb][db][rq * 4 + 3] * inv};
      if (g == 0)
        a.part_lse[(int64_t)split * rows + row] =
            l_tot > 0.f ? (r_raw[qb] * c2 + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
    return;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int my_q = q0w + 32 * qb + ql;
    const float l_tot = xhalf_sum(l_run[qb]);
    // l_tot = 0 only for a row with no visible key (mask mode): O = 0, and
    // the LSE below evaluates to -inf + -inf = -inf.
    const float inv = (l_tot > 0.f ? 1.f / l_tot : 0.f) * (DROP ? a.drop.keep_scale : 1.f);
    if (my_q >= N) continue;  // lanes past the last query
    uint16_t* Orow = a.o + head + (int64_t)my_q * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        u32x2 w;
        w[0] = pack2<T>(oacc[qb][db][rq * 4 + 0] * inv, oacc[qb][db][rq * 4 + 1] * inv);
        w[1] = pack2<T>(oacc[qb][db][rq * 4 + 2] * inv, oacc[qb][db][rq * 4 + 3] * inv);
        *(u32x2*)(Orow + db * 32 + rq * 8 + g * 4) = w;
      }
    if (g == 0) a.lse[(int64_t)bh * N + my_q] = (r_raw[qb] * c2 + __log2f(l_tot)) * kLn2;
  }
}

// Merge of split-K/V partial states, one row per D/4 lanes ("CUDA
// FlashAttention ...", §7: split along K, each part yields local (m, l, o),
// combined with the same merge formula).  With LSE_s the natural-log
// log-sum-exp of split s and O_s its normalised output,
//   LSE = m + ln sum_s exp(LSE_s - m),  O = sum_s exp(LSE_s - LSE) O_s,
// where m = max_s LSE_s; splits with LSE_s = -inf carry weight 0.
template <int D, class T>
__global__ __launch_bounds__(256) void merge_kernel(const float* __restrict__ part_lse,
                                                    const float* __restrict__ part_o, uint16_t* __restrict__ o,
                                                    float* __restrict__ lse, int64_t rows, int n_splits) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  if (row >= rows) return;
  float m = -INFINITY;
  for (int sp = 0; sp < n_splits; ++sp) m = fmaxf(m, part_lse[(int64_t)sp * rows + row]);
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int sp = 0; sp < n_splits; ++sp) {
      const float ls = part_lse[(int64_t)sp * rows + row];
      const float w = ls == -INFINITY ? 0.f : fast_exp2((ls - m) * kLog2e);
      const f32x4 x = *(const f32x4*)(part_o + ((int64_t)sp * rows + row) * D + c * 4);
      acc += w * x;
      wsum += w;
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  *(u32x2*)(o + row * D + c * 4) = u32x2{pack2<T>(acc[0] * inv, acc[1] * inv), pack2<T>(acc[2] * inv, acc[3] * inv)};
  if (c == 0) lse[row] = wsum > 0.f ? m + __logf(wsum) : -INFINITY;
}

template <int D, int QB, bool CAUSAL, class T>
hipError_t launch_fwd_t(FwdArgs a, hipStream_t stream) {
  constexpr int BM = FwdShape<QB>::BM;
  a.n_qtiles = (int)((a.N + BM - 1) / BM);
  const int64_t n_wg = (int64_t)a.BH * a.n_qtiles;
  hipLaunchKernelGGL((fwd_kernel<D, QB, CAUSAL, T, false, false, false>), dim3((unsigned)n_wg), dim3(kFwdThreads), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, int QB, bool CAUSAL, class T>
hipError_t launch_fwd_masked_t(FwdArgs a, hipStream_t stream) {
  constexpr int BM = FwdShape<QB>::BM;
  a.n_qtiles = (int)((a.N + BM - 1) / BM);
  const int64_t n_wg = (int64_t)a.BH * a.n_qtiles;
  hipLaunchKernelGGL((fwd_kernel<D, QB, CAUSAL, T, false, true, false>), dim3((unsigned)n_wg), dim3(kFwdThreads), 0,
                     stream, a);
  return hipGetLastError();
}

template <int D, int QB, bool CAUSAL, class T, bool MASK>
hipError_t launch_fwd_dropout_t(FwdArgs a, hipStream_t stream) {
  constexpr int BM = FwdShape<QB>::BM;
  a.n_qtiles = (int)((a.N + BM - 1) / BM);
  const int64_t n_wg = (int64_t)a.BH * a.n_qtiles;
  hipLaunchKernelGGL((fwd_kernel<D, QB, CAUSAL, T, false, MASK, true>), dim3((unsigned)n_wg), dim3(kFwdThreads), 0,
                     stream, a);
  return hipGetLastError();
}

// keep[bh][i][j] of the dropout mask: one thread per (bh, query, 16 keys).
__global__ __launch_bounds__(256) void dropout_mask_kernel(uint8_t* __restrict__ keep, int64_t BH, int64_t N,
                                                           DropoutArgs d) {
  const int64_t T = (N + 15) / 16;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= BH * N * T) return;
  const int64_t t = idx % T, i = (idx / T) % N, bh = idx / (T * N);
  const uint32_t bits = dropout_bits16((int)t, (int)i, (uint64_t)bh, d.seed, d.offset, d.thr);
  uint8_t* row = keep + (bh * N + i) * N;
  for (int e = 0; e < 16; ++e) {
    const int64_t j = t * 16 + e;
    if (j < N) row[j] = (uint8_t)((bits >> e) & 1u);
  }
}

template <int D, int QB, bool CAUSAL, class T, bool MASK, bool DROP>
hipError_t launch_fwd_split_t(FwdArgs a, hipStream_t stream) {
  constexpr int BM = FwdShape<QB>::BM;
  a.n_qtiles = (int)((a.N + BM - 1) / BM);
  const int64_t n_wg = (int64_t)a.BH * a.n_qtiles * a.n_splits;
  hipLaunchKernelGGL((fwd_kernel<D, QB, CAUSAL, T, true, MASK, DROP>), dim3((unsigned)n_wg), dim3(kFwdThreads), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)a.BH * a.N;
  constexpr int rpb = 256 / (D / 4);
  hipLaunchKernelGGL((merge_kernel<D, T>), dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0, stream,
                     a.part_lse, a.part_o, a.o, a.lse, rows, a.n_splits);
  return hipGetLastError();
}

}  // namespace

// Which forward runs is set by how many workgroups it would launch (256
// compute units): with fewer 128-query tiles than compute units, the
// key-split forward of fa_fwd_short.hip; at D = 128 with at least
// kD128From 256-query tiles, the 64-queries-per-wave kernel; otherwise this
// file's 128-query kernel (thresholds from measured sweeps over N and H).
// A causal launch of exactly one tile per compute unit with long keys
// (N >= kShortCausalFrom) also takes the key-split forward: there the
// 128-query kernel's heaviest workgroup walks all N/64 key tiles alone at
// the end (measured: one head N = 32768 0.36 vs 0.49 ms, two heads N = 16384
// 0.19 vs 0.25 ms).
constexpr int64_t kShortBelow = 256;
constexpr int64_t kShortCausalFrom = 8192;
constexpr int64_t kD128From = 1024;

FwdPath fwd_path(int64_t BH, int64_t N, int64_t D, bool causal) {
  const int64_t tiles = BH * ((N + 127) / 128);
  if (tiles < kShortBelow || (causal && tiles == kShortBelow && N >= kShortCausalFrom)) return FwdPath::kShort;
  if (D == 128 && BH * ((N + 255) / 256) >= kD128From) return FwdPath::kD128;
  return FwdPath::kTiled;
}

hipError_t launch_fwd(const FwdArgs& a, int D, bool causal, int dtype, hipStream_t stream) {
  const FwdPath path = fwd_path(a.BH, a.N, D, causal);
  if (path == FwdPath::kShort) return launch_fwd_short(a, D, causal, dtype, stream);
  if (path == FwdPath::kD128) return launch_fwd_d128(a, causal, dtype, stream);
#define FA_FWD_CASE(DD, CC, TT) \
  if (D == DD && causal == CC && dtype == TT::id) return launch_fwd_t<DD, kFwdQB, CC, TT>(a, stream);
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

hipError_t launch_fwd_masked(const FwdArgs& a, int D, bool causal, int dtype, hipStream_t stream) {
#define FA_FWD_CASE(DD, CC, TT) \
  if (D == DD && causal == CC && dtype == TT::id) return launch_fwd_masked_t<DD, kFwdQB, CC, TT>(a, stream);
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

hipError_t launch_fwd_dropout(const FwdArgs& a, int D, bool causal, int dtype, hipStream_t stream) {
#define FA_FWD_CASE(DD, CC, TT) \
  if (D == DD && causal == CC && dtype == TT::id) return launch_fwd_dropout_t<DD, kFwdQB, CC, TT, false>(a, stream);
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

hipError_t launch_fwd_masked_dropout(const FwdArgs& a, int D, bool causal, int dtype, hipStream_t stream) {
#define FA_FWD_CASE(DD, CC, TT) \
  if (D == DD && causal == CC && dtype == TT::id) return launch_fwd_dropout_t<DD, kFwdQB, CC, TT, true>(a, stream);
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

hipError_t launch_dropout_mask(uint8_t* keep, int64_t BH, int64_t N, const DropoutArgs& d, hipStream_t stream) {
  const int64_t threads = BH * N * ((N + 15) / 16);
  hipLaunchKernelGGL(dropout_mask_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, keep, BH, N,
                     d);
  return hipGetLastError();
}

hipError_t launch_fwd_splitkv(const FwdArgs& a, int D, bool causal, int dtype, hipStream_t stream) {
#define FA_FWD_CASE(DD, CC, TT) \
  if (D == DD && causal == CC && dtype == TT::id) return launch_fwd_split_t<DD, kFwdQB, CC, TT, false, false>(a, stream);
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

hipError_t launch_fwd_splitkv_masked(const FwdArgs& a, int D, bool causal, int dtype, hipStream_t stream) {
#define FA_FWD_CASE(DD, CC, TT) \
  if (D == DD && causal == CC && dtype == TT::id) return launch_fwd_split_t<DD, kFwdQB, CC, TT, true, false>(a, stream);
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

hipError_t launch_fwd_splitkv_masked_dropout(const FwdArgs& a, int D, bool causal, int dtype, hipStream_t stream) {
#define FA_FWD_CASE(DD, CC, TT) \
  if (D == DD && causal == CC && dtype == TT::id) return launch_fwd_split_t<DD, kFwdQB, CC, TT, true, true>(a, stream);
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

hipError_t launch_fwd_splitkv_dropout(const FwdArgs& a, int D, bool causal, int dtype, hipStream_t stream) {
#define FA_FWD_CASE(DD, CC, TT) \
  if (D == DD && causal == CC && dtype == TT::id) return launch_fwd_split_t<DD, kFwdQB, CC, TT, false, true>(a, stream);
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
