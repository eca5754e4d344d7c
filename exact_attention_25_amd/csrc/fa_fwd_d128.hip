// fa_fwd_d128.hip -- FlashAttention forward for head size 128 with 64 queries
// per wave, for gfx950.
//
// Same computation as fwd_kernel in fa_fwd.hip (online softmax: per key tile
// m' = max(m, rowmax S), l = alpha l + rowsum exp(S - m'), O = alpha O +
// exp(S - m') V, "CUDA FlashAttention: from online softmax to the
// long-sequence IO limit", §4; "FlashAttention algorithm details",
// §4.2.1-4.2.2; tiles wholly above the causal diagonal are never visited,
// "Why FlashAttention does not need to store the attention matrix", §4.5),
// with a different work split:
//  * A wave owns 64 queries (two 32-query blocks), one wave per SIMD, so each
//    K or V^T fragment read from LDS feeds two MFMAs: half the LDS operand
//    bytes per FLOP of a 32-query wave.  A key/value tile read once serves
//    more query rows ("CUDA FlashAttention ...", §5.1): the workgroup's 256
//    queries also halve the HBM/L2 -> LDS tile traffic per query.  Measured,
//    the chip then holds a higher clock under this kernel (about 1.7 vs 1.5
//    GHz) at fewer busy matrix-core cycles.
//  * That needs about 450 live registers: the O accumulators (128) and the Q
//    fragments (64) are held in AGPRs and the scores (2 x 64) in VGPRs.  The
//    compiler assigns accumulators to one register class per kernel, so the
//    MFMAs are written as inline assembly with explicit operand classes.
//    Inline assembly is opaque to the compiler's hazard checks, so the wait
//    states gfx950 requires are placed by hand: 12 between an MFMA that
//    writes a register and a vector instruction that reads it (16 are used:
//    after each batch of score MFMAs, and before O is read).  A vector write
//    needs 2 before an MFMA reads that register; every probability operand
//    is packed at least eight slots before its first P V MFMA, so none are
//    placed there (the test suite scans the generated code for both).
//  * With one wave per SIMD nothing hides a stall, so a step of the tile loop
//    is written as 64 MFMA slots with the other work placed beside them (see
//    the step below): no LDS read, barrier or copy waits on data issued just
//    before it.  K and V tiles of 64 keys stream HBM -> LDS directly into
//    four-buffer rings (buffer_load ... lds), two tiles ahead of their use,
//    with one workgroup barrier per tile placed in the middle of the P V
//    MFMAs.
#include "fa_common.hpp"
#include "fa_launch.hpp"

#include <type_traits>

namespace fa {

namespace {

constexpr int kD = 128;
constexpr int kBN = 64;                  // keys per tile
constexpr int kNT = 256;                 // threads per workgroup (4 waves)
constexpr int kWQ = 64;                  // queries per wave
constexpr int kBM = kWQ * (kNT / 64);    // queries per workgroup
constexpr int kRC = kD / 8;              // 16-byte chunks per row
constexpr int kTC = kBN * kRC;           // chunks per K or V tile
constexpr int kLPT = kTC / kNT;          // direct copies per thread per tile
constexpr float kLazy = 8.0f;
constexpr float kFastLimit = 4096.0f;
constexpr int kPK = 3;                   // K fragments read ahead of their MFMAs
constexpr int kPV = 3;                   // V^T fragments read ahead of their MFMAs

template <class T, bool CAUSAL>
__global__ __launch_bounds__(kNT, 1) void fwd_d128_kernel(FwdArgs a) {
  // LDS: four K and four V tile buffers of 16 KB.  Tile t of K lives in K
  // buffer t % 4, tile t of V in V buffer t % 4.  Separate objects, so that
  // the compiler can tell the reads of one buffer from the copies in flight
  // into another (otherwise it waits for every copy before the next read).
  __shared__ u32x4 lds_k0[kTC], lds_k1[kTC], lds_k2[kTC], lds_k3[kTC];
  __shared__ u32x4 lds_v0[kTC], lds_v1[kTC], lds_v2[kTC], lds_v3[kTC];
  auto kbuf = [&](int b) __attribute__((always_inline)) {
    return b == 0 ? lds_k0 : b == 1 ? lds_k1 : b == 2 ? lds_k2 : lds_k3;
  };
  auto vbuf = [&](int b) __attribute__((always_inline)) {
    return b == 0 ? lds_v0 : b == 1 ? lds_v1 : b == 2 ? lds_v2 : lds_v3;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, g = lane >> 5;

  const int64_t N = a.N;
  const int G = a.H / a.Hkv;
  const int bh = head_of_slot(blockIdx.x % a.BH, a.BH, G);
  const int rank = blockIdx.x / a.BH;
  const int qt = CAUSAL ? (a.n_qtiles - 1 - rank) : rank;
  const int64_t head = (int64_t)bh * N * kD;
  const int64_t kv_head = (int64_t)(bh / G) * N * kD;
  const uint16_t* __restrict__ Qh = a.q + head;
  const uint16_t* __restrict__ Kh = a.k + kv_head;
  const uint16_t* __restrict__ Vh = a.v + kv_head;

  const int q0w = qt * kBM + wave * kWQ;  // first query of this wave
  const bool active = q0w < N;

  // Q^T operand fragments in AGPRs: lane (ql, g) of block qb holds
  // Q[q0w + 32qb + ql][16c + 8g .. +8]; rows past N re-read row N-1.
  // All sixteen loads are issued here; they are bound to the AGPRs only
  // after the first tile copies have been issued (see the prologue).
  u32x4 qa[2][kD / 16], qv[2][kD / 16];
  if (active) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const uint16_t* Qrow = Qh + (int64_t)min(q0w + 32 * qb + ql, (int)N - 1) * kD + g * 8;
#pragma unroll
      for (int c = 0; c < kD / 16; ++c) qv[qb][c] = *(const u32x4*)(Qrow + c * 16);
    }
  } else {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int c = 0; c < kD / 16; ++c) qv[qb][c] = u32x4{0, 0, 0, 0};
  }

  f32x16 oacc[2][kD / 32];
  float r_raw[2], l_run[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
    for (int i = 0; i < kD / 32; ++i) oacc[qb][i] = f32x16{};
    r_raw[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }

  const int n_kt_all = (int)((N + kBN - 1) / kBN);
  const int n_kt = CAUSAL ? min(n_kt_all, ((qt + 1) * kBM) / kBN) : n_kt_all;  // tiles of the workgroup
  // Tiles this wave computes: a causal wave's last one holds its last query.
  const int n_act = !active ? 0 : (CAUSAL ? min(n_kt, (q0w + kWQ - 1) / kBN + 1) : n_kt);

  // Direct copies: part p of a tile is one 16-byte chunk per lane.  A tile
  // past the workgroup's last one is given a buffer of zero bytes: its
  // copies read nothing and fill a free LDS buffer with zeros, so they need
  // no branch.
  const int p0 = wave * 64 + lane;
  const int ksrc0 = swz(p0) * 8;
  const int vr0 = p0 / kRC;
  const int vsrc0 = vr0 * kD + ((p0 % kRC) ^ dual_xor<kRC>(vr0)) * 8;
  // The wave's offset in a buffer is made opaque at each copy, so that the
  // compiler forms each destination beside its copy instead of keeping one
  // scalar register per buffer and part live across the loop.
  auto copy_part = [&](const uint16_t* base, int tile, int src0, u32x4* dst, int p) __attribute__((always_inline)) {
    const int valid = tile < n_kt ? min(kBN, (int)N - tile * kBN) : 0;
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(base + (int64_t)tile * kBN * kD, valid * kD * 2);
    int wofs = wave * 64 * 16;  // bytes: the destination is then one scalar add
    asm volatile("" : "+s"(wofs));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)((char*)dst + wofs + p * kNT * 16), 16,
                                             src0 * 2, p * kNT * 16, 0, 0);
  };
  auto copy_k = [&](int tile, int buf, int p) __attribute__((always_inline)) {
    copy_part(Kh, tile, ksrc0, kbuf(buf), p);
  };
  auto copy_v = [&](int tile, int buf, int p) __attribute__((always_inline)) {
    copy_part(Vh, tile, vsrc0, vbuf(buf), p);
  };

  // LDS read offsets (bytes within a buffer), formed once.  K fragment
  // f = (c = f/2, key block kb = f%2): k_addr[c] + kb*8 KB.  V^T fragment
  // v = (t = v/4, db = v%4): lo half at v_addr[0][db] + t*4 KB, hi half at
  // v_addr[1][db] + t*4 KB.
  const int krow = perm23(ql);
  const uint32_t k_off = swz(krow * kRC + g) * 16;
  const int vj = lane & 15, vq4 = lane >> 4;
  const int v_row0 = 8 * g + (vj >> 2);
  const int v_col = 16 * (vq4 & 1) + 4 * (vj & 3);
  const uint32_t v_off0 = dual_chunk<kRC>(v_row0, v_col >> 3) * 16 + (v_col & 7) * 2;
  const uint32_t v_off1 = dual_chunk<kRC>(v_row0 + 4, v_col >> 3) * 16 + (v_col & 7) * 2;
  uint32_t k_addr[kRC / 2], v_addr[2][kD / 32];
#pragma unroll
  for (int c = 0; c < kRC / 2; ++c) k_addr[c] = k_off ^ (32 * c);
#pragma unroll
  for (int db = 0; db < kD / 32; ++db) {
    v_addr[0][db] = v_off0 ^ (64 * db);
    v_addr[1][db] = v_off1 ^ (64 * db);
  }
  auto kread = [&](int b, int f) __attribute__((always_inline)) {
    return *(const u32x4*)((const char*)kbuf(b) + k_addr[f >> 1] + (f & 1) * 32 * kRC * 16);
  };
  auto vread = [&](int b, int v) __attribute__((always_inline)) {
    const int t = v / (kD / 32), db = v % (kD / 32);
    const char* Vl = (const char*)vbuf(b);
    const u32x2 lo = lds_read_tr16(Vl + v_addr[0][db] + t * 16 * kRC * 16);
    const u32x2 hi = lds_read_tr16(Vl + v_addr[1][db] + t * 16 * kRC * 16);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  const float c2 = a.scale_log2;

  // Mask a tile's raw scores before its max (diagonal and partial last
  // tiles only; the test is uniform).  Register r of lane-half g holds key
  // k0 + 32kb + acc_row(r, g) = k0 + 32kb + 16(r/8) + (r%8) + 8g for query
  // q0w + 32qb + ql, so key > query and key >= N compare one per-lane value
  // with a constant per register; the lane values are formed here, inside
  // the branch, so that nothing stays live across the loop.
  // Each element is one compare into VCC and one select (inline assembly,
  // so the compiler cannot hoist all 64 compare results into scalar pairs).
  auto mask_tile = [&](f32x16 (&s)[2][2], int k0) __attribute__((always_inline)) {
    const int dn = min((int)N - k0, kBN) - 8 * g - 1;  // key < N      <=>  c <= dn
    const int dq = ql - 8 * g + (q0w - k0);          // key <= query  <=>  c <= dq + 32qb
    const float ninf = -INFINITY;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int lim = CAUSAL ? min(dq + 32 * qb, dn) : dn;  // visible iff c <= lim
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 32 * kb + 16 * (r >> 3) + (r & 7);
          asm("v_cmp_gt_i32_e32 vcc, %1, %2\n\tv_cndmask_b32_e32 %0, %0, %3, vcc"
              : "+v"(s[qb][kb][r])
              : "i"(c), "v"(lim), "v"(ninf)
              : "vcc");
        }
    }
  };
  // Row maxima of both query blocks across the two lane halves: one swap
  // exchanges the halves of the two values (lanes 0-31 then see block 0 in
  // both registers, lanes 32-63 block 1), a second spreads each block's
  // result to every lane.  med3(x, y, +inf) is max(x, y) without the
  // canonicalising moves fmaxf adds.
  auto xhalf_max2 = [&](float a0, float a1, float& m0, float& m1) __attribute__((always_inline)) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a0), __float_as_uint(a1), false, false);
    const float t = __builtin_amdgcn_fmed3f(__uint_as_float(r[0]), __uint_as_float(r[1]), INFINITY);
    auto u = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
    m0 = __uint_as_float(u[0]);
    m1 = __uint_as_float(u[1]);
  };
  auto needs_mask = [&](int k0) { return (CAUSAL && k0 + kBN - 1 > q0w) || k0 + kBN > N; };
  // mx: a tile's row max over this lane's half of the keys (the two lanes
  // of a query each hold one half).  The rescale decision needs no more:
  // max(h0, h1) * c2 > t exactly when h0 * c2 > t or h1 * c2 > t (c2 > 0,
  // rounding is monotone), and the vote covers both lanes.  Only a rescale
  // takes the full max, so the common path has no lane-half exchange.
  float mx[2];
  auto tile_max = [&](const f32x16 (&s)[2][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float m = s[qb][0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) m = fmaxf(m, s[qb][0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) m = fmaxf(m, s[qb][1][r]);
      mx[qb] = m;
    }
  };

  // Reference state, as in fwd_kernel: the reference max r_raw is one of
  // the raw scores; mref = RN(r_raw*c2); the exponent is one FMA s*c2 - mref
  // until a row's reference reaches |mref| >= kFastLimit (raw_mode: scores
  // are first shifted by r_raw).  A tile raises the reference only when its
  // max exceeds it by more than kLazy (log2 units).  The decision for tile
  // j+1 is taken at the end of step j; O and l are rescaled at the start of
  // step j+1, after the P V MFMAs of tile j and before those of tile j+1.
  float mref[2], m_use[2], mlazy[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) mref[qb] = mlazy[qb] = -INFINITY, m_use[qb] = 0.f;
  bool raw_mode = false, d_rescale = false;
  auto decide = [&]() __attribute__((always_inline)) {
    const bool need = (mx[0] * c2 > mlazy[0]) || (mx[1] * c2 > mlazy[1]);
    d_rescale = wave_any(need);
  };
  auto rescale = [&]() __attribute__((always_inline)) {
    float r_new[2], m_full[2];
    xhalf_max2(mx[0], mx[1], m_full[0], m_full[1]);
    bool big = false;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      r_new[qb] = fmaxf(r_raw[qb], m_full[qb]);
      const float nm = r_new[qb] * c2;
      big = big || (fabsf(nm) >= kFastLimit && nm != -INFINITY);
    }
    const bool raw_new = wave_any(big);
    const bool raw_diff = raw_mode || raw_new;
    o_ready(oacc);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float lg = raw_diff ? (r_raw[qb] - r_new[qb]) * c2 : mref[qb] - r_new[qb] * c2;
      const float alpha = (r_raw[qb] == -INFINITY) ? 0.f : fast_exp2(lg);
      l_run[qb] *= alpha;
#pragma unroll
      for (int i = 0; i < kD / 32; ++i) oacc[qb][i] *= alpha;
      r_raw[qb] = r_new[qb];
      mref[qb] = r_new[qb] * c2;
      mlazy[qb] = mref[qb] + kLazy;
      m_use[qb] = (mref[qb] == -INFINITY) ? 0.f : mref[qb];
    }
    raw_mode = raw_new;
  };

  constexpr int NS = 2 * (kD / 16);           // K fragments per tile (16), two MFMAs each
  constexpr int NV = (kBN / 16) * (kD / 32);  // V^T fragments per tile (16), two MFMAs each
  constexpr int PK = kPK, PV = kPV;
  u32x4 kq[PK + 1];  // K fragment ring; fragments 0 .. PK-1 of the next tile are read one step ahead

  // One step j (PH = j % 4 fixes the LDS buffers): 64 MFMA slots.
  //  Slots 0-31 (phase A): score MFMAs of tile j+1 (two per K fragment),
  //    the exponentials of tile j beside them (two per MFMA); from slot 24 the
  //    first probability operand (keys 0-15) of tile j is packed and the first
  //    V^T fragments of tile j are read.
  //  Slots 32-63 (phase B): P V MFMAs of tile j (two per V^T fragment), the
  //    packing of operands 1-3 eight slots ahead of their first MFMA, the row
  //    sums (two v_fma_mix per slot) and the row max of tile j+1 (one max3 per
  //    slot).  At slot 48 the workgroup barrier, after this wave's copies of
  //    the previous step (K of tile j+2, V of tile j+1) have landed; after it
  //    the first K fragments of tile j+2 are read for the next step.  MFMAs
  //    whose operands are already in registers run on both sides of it.
  //  The copies of K of tile j+3 and V of tile j+2 (eight per lane) follow
  //    the barrier, one every two slots (slots 49, 51, ..., 63), so that
  //    each has most of a step to land before the next barrier waits for
  //    all of them; issued together they would hold every SIMD until the
  //    CU's address unit took them.  Their buffers were last read before the
  //    previous step's barrier.  (Measured 0.8-1.2 % faster, in interleaved
  //    A/B runs on two boxes, than one copy every four slots of phase A.)
  auto step = [&](auto phc, int j, f32x16 (&s)[2][2], f32x16 (&s_nxt)[2][2]) __attribute__((always_inline)) {
    constexpr int PH = decltype(phc)::value;
    constexpr int kbA = (PH + 1) % 4;  // K buffer of tile j+1
    constexpr int kbN = (PH + 2) % 4;  // K buffer of tile j+2
    constexpr int vbB = PH % 4;        // V buffer of tile j
    // Both rare blocks are marked unlikely, so the compiler places them out
    // of line and the common path falls through (measured ~0.5 % faster).
    if (__builtin_expect(d_rescale, 0)) rescale();
    float mu[2] = {m_use[0], m_use[1]};
    if (__builtin_expect(raw_mode, 0)) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float ru = (r_raw[qb] == -INFINITY) ? 0.f : r_raw[qb];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) s[qb][kb] -= ru;
        mu[qb] = 0.f;
      }
    }
    u32x4 pf[2][kBN / 16];
    u32x4 vq[PV + 1];
    // ---- phase A ----
#pragma unroll
    for (int i = 0; i < 2 * NS; ++i) {
      const int qb = i & 1, f = i >> 1;
      if (qb == 0 && f + PK < NS) kq[(f + PK) % (PK + 1)] = kread(kbA, f + PK);
      // One LDS wait per two fragments: before fragment f's first MFMA (f
      // even) wait for fragment f+1 as well.
      if (qb == 0 && (f & 1) == 0) asm volatile("" ::"v"(kq[(f + 1) % (PK + 1)]));
      if (f < 2)
        mfma_s_first<T>(s_nxt[qb][f & 1], kq[f % (PK + 1)], qa[qb][f >> 1]);
      else
        mfma_s_acc<T>(s_nxt[qb][f & 1], kq[f % (PK + 1)], qa[qb][f >> 1]);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int idx = 2 * f + e;
        s[qb][idx >> 4][idx & 15] = fast_exp2(__builtin_fmaf(s[qb][idx >> 4][idx & 15], c2, -mu[qb]));
      }
      if (i >= 2 * NS - 8) {  // operand 0 (keys 0-15 = registers 0-7 of key block 0)
        const int w = (i - (2 * NS - 8)) >> 1;
        pf[qb][0][w] = pack2<T>(s[qb][0][2 * w], s[qb][0][2 * w + 1]);
      }

      if (qb == 1 && i >= 2 * NS - 2 * PV) {  // the first PV V^T fragments of tile j
        const int v = (i - (2 * NS - 2 * PV)) >> 1;
        vq[v] = vread(vbB, v);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    scores_ready(s_nxt);

    // ---- phase B ----
    float lsum[2], lsum2[2], mn[2] = {-INFINITY, -INFINITY};
    if constexpr (T::id != Fp16::id) lsum[0] = lsum[1] = 0.f;
#pragma unroll
    for (int i = 0; i < 2 * NV; ++i) {
      const int qb = i & 1, v = i >> 1, t = v / (kD / 32), db = v % (kD / 32);
      if (i == 2 * NV / 2) {  // slot 48: the copies of the previous step have landed everywhere
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        barrier_only();
      }
      if (i > 2 * NV / 2 && (i & 1) == 1) {  // slots 49, 51, ..., 63: the eight copies
        const int cp = (i - 17) >> 1;
        if (cp < kLPT)
          copy_k(j + 3, (PH + 3) % 4, cp);
        else
          copy_v(j + 2, (PH + 2) % 4, cp - kLPT);
      }
      if (qb == 0 && v + PV < NV) vq[(v + PV) % (PV + 1)] = vread(vbB, v + PV);
      if (qb == 0 && (v & 1) == 0) asm volatile("" ::"v"(vq[(v + 1) % (PV + 1)]));
      mfma_o<T, false>(oacc[qb][db], vq[v % (PV + 1)], pf[qb][t]);
      if (i < 24) {  // operand 1 + i/8, dword (i/2) % 4 of block qb
        const int tp = 1 + (i >> 3), w = (i >> 1) & 3;
        const int lo = (tp & 1) * 8 + 2 * w;
        pf[qb][tp][w] = pack2<T>(s[qb][tp >> 1][lo], s[qb][tp >> 1][lo + 1]);
      }
      {  // row sum of dword i/2 of block qb (packed at least eight slots ago)
        const int d = i >> 1;
        if constexpr (T::id == Fp16::id) {
          // The two halves of the dword go to two FP32 sums, so that the two
          // v_fma_mix of a slot do not wait for each other.  (Adding dword
          // pairs as fp16 first saves instructions but its extra rounding
          // was measured to cost accuracy.)
          if (d == 0)  // the first dword starts both sums
            asm("v_fma_mix_f32 %0, %2, 1.0, 0 op_sel_hi:[1,0,0]\n\t"
                "v_fma_mix_f32 %1, %2, 1.0, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
                : "=&v"(lsum[qb]), "=&v"(lsum2[qb])
                : "v"(pf[qb][0][0]));
          else
            asm("v_fma_mix_f32 %0, %2, 1.0, %0 op_sel_hi:[1,0,0]\n\t"
                "v_fma_mix_f32 %1, %2, 1.0, %1 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
                : "+v"(lsum[qb]), "+v"(lsum2[qb])
                : "v"(pf[qb][d >> 2][d & 3]));
          asm volatile("" : "+v"(lsum2[qb]));
        } else {
          const int lo = ((d >> 2) & 1) * 8 + 2 * (d & 3);
          lsum[qb] += s[qb][d >> 3][lo];
          lsum[qb] += s[qb][d >> 3][lo + 1];
        }
        asm volatile("" : "+v"(lsum[qb]));
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int idx = 2 * v + e;
        mn[qb] = fmaxf(mn[qb], s_nxt[qb][idx >> 4][idx & 15]);
      }
      asm volatile("" : "+v"(mn[qb]));
      if (qb == 1 && i >= 2 * NV - 2 * PK) {  // slots 58-63: fragments 0 .. PK-1 of tile j+2
        const int f = (i - (2 * NV - 2 * PK)) >> 1;
        kq[f] = kread(kbN, f);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) l_run[qb] += T::id == Fp16::id ? lsum[qb] + lsum2[qb] : lsum[qb];
    mx[0] = mn[0];
    mx[1] = mn[1];
    // The row max of tile j+1 was taken beside the MFMAs (with no branch
    // between the phases, so that nothing is moved out of its slot); a tile
    // that needs a mask is masked now and its max taken again.
    const bool pending = j + 1 < n_act;
    const int k1 = (j + 1) * kBN;
    if (pending && needs_mask(k1)) {
      asm volatile("");
      mask_tile(s_nxt, k1);
      tile_max(s_nxt);
    }
    if (pending) decide();
    else d_rescale = false;
  };

  // Prologue: K of tiles 0-2 and V of tiles 0-1; the scores of tile 0 and
  // the first K fragments of tile 1.
  f32x16 sA[2][2], sB[2][2];
#pragma unroll
  for (int p = 0; p < kLPT; ++p) {
    copy_k(0, 0, p);
    copy_v(0, 0, p);
    copy_k(1, 1, p);
    copy_v(1, 1, p);
    copy_k(2, 2, p);
  }
  // Q reaches its AGPRs only now, so that its loads and the first tile
  // copies are in flight together.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int c = 0; c < kD / 16; ++c) asm volatile("s_nop 1" : "=a"(qa[qb][c]) : "0"(qv[qb][c]));
  wait_vmem();
  __syncthreads();
  if (active) {
#pragma unroll
    for (int i = 0; i < PK; ++i) kq[i] = kread(0, i);
#pragma unroll
    for (int i = 0; i < 2 * NS; ++i) {
      const int qb = i & 1, f = i >> 1;
      if (qb == 0 && f + PK < NS) kq[(f + PK) % (PK + 1)] = kread(0, f + PK);
      if (f < 2)
        mfma_s_first<T>(sA[qb][f & 1], kq[f % (PK + 1)], qa[qb][f >> 1]);
      else
        mfma_s_acc<T>(sA[qb][f & 1], kq[f % (PK + 1)], qa[qb][f >> 1]);
    }
    scores_ready(sA);
    if (needs_mask(0)) mask_tile(sA, 0);
    tile_max(sA);
    decide();
  }
  if (active) {
#pragma unroll
    for (int i = 0; i < PK; ++i) kq[i] = kread(1, i);
  }

  // The tiles this wave computes, four per iteration so that the LDS buffers
  // and the two score sets rotate with compile-time offsets; then, for the
  // workgroup's remaining tiles, only the copies and the barriers.
  int j = 0;
  for (; j + 3 < n_act; j += 4) {
    step(std::integral_constant<int, 0>{}, j, sA, sB);
    step(std::integral_constant<int, 1>{}, j + 1, sB, sA);
    step(std::integral_constant<int, 2>{}, j + 2, sA, sB);
    step(std::integral_constant<int, 3>{}, j + 3, sB, sA);
  }
  if (j < n_act) step(std::integral_constant<int, 0>{}, j, sA, sB);
  if (j + 1 < n_act) step(std::integral_constant<int, 1>{}, j + 1, sB, sA);
  if (j + 2 < n_act) step(std::integral_constant<int, 2>{}, j + 2, sA, sB);
  for (j = n_act; j < n_kt; ++j) {
#pragma unroll
    for (int p = 0; p < kLPT; ++p) {
      copy_k(j + 3, (j + 3) % 4, p);
      copy_v(j + 2, (j + 2) % 4, p);
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kLPT) : "memory");
    barrier_only();
  }

  // Copies past the last tile still write (zeros) into LDS: they must land
  // before the workgroup ends and its LDS is handed to the next one.
  wait_vmem();
  if (!active) return;
  o_ready(oacc);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int my_q = q0w + 32 * qb + ql;
    const float l_tot = xhalf_sum(l_run[qb]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (my_q >= N) continue;
    uint16_t* Orow = a.o + head + (int64_t)my_q * kD;
#pragma unroll
    for (int db = 0; db < kD / 32; ++db)
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

template <class T, bool CAUSAL>
hipError_t launch_t(FwdArgs a, hipStream_t stream) {
  a.n_qtiles = (int)((a.N + kBM - 1) / kBM);
  const int64_t n_wg = (int64_t)a.BH * a.n_qtiles;
  hipLaunchKernelGGL((fwd_d128_kernel<T, CAUSAL>), dim3((unsigned)n_wg), dim3(kNT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_d128(const FwdArgs& a, bool causal, int dtype, hipStream_t stream) {
  if (dtype == Fp16::id) return causal ? launch_t<Fp16, true>(a, stream) : launch_t<Fp16, false>(a, stream);
  if (dtype == Bf16::id) return causal ? launch_t<Bf16, true>(a, stream) : launch_t<Bf16, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
