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
//     registers and are written once (or, when the pass runs in parts, as
//     FP32 partial sums that dkdv_reduce_kernel adds in part order).
//  3. dq_kernel: one workgroup per 128 queries, Q and dO resident, looping
//     over key tiles of 64; dQ accumulates in registers and is written once
//     (in parts: FP32 partial sums, added by dq_reduce_kernel).
// The streamed tiles go HBM -> LDS directly into a double-buffered ring (one
// barrier per tile) and stay row-major; the transposed operands (Q^T, dO^T,
// K^T) come from ds_read_b64_tr_b16, so nothing is transposed in memory.
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
// Tiles of 64 rows x D columns of a row-major [.., D] tensor are copied from
// HBM straight into LDS (buffer_load_dwordx4 ... lds, 256 threads, D/32 copies
// each) as 16-byte chunks in row-major order.  A tile that is read both by
// rows and transposed uses the dual_chunk swizzle; a tile read only by rows
// uses swz.  Copy i of wave w fills LDS chunks i*256 + 64w + lane; because
// both swizzles depend only on the low four bits of the row index, the
// per-lane source offset of copy i is copy 0's plus i*256 chunks.
// ---------------------------------------------------------------------------
constexpr int kTileRows = 64;

template <int D, bool DUAL>
__device__ __forceinline__ int tile_src_offset(int p) {
  constexpr int RC = D / 8;
  if constexpr (DUAL) {
    const int r = p / RC;
    return r * D + ((p % RC) ^ dual_xor<RC>(r)) * 8;
  } else {
    return swz(p) * 8;  // swz is its own inverse
  }
}

// `valid` = rows of the tile inside the tensor (the last tile may be partial).
template <int D>
__device__ __forceinline__ void copy_tile(const uint16_t* __restrict__ src, int src0, u32x4* dst, int wave,
                                          int valid) {
  constexpr int LPT = kTileRows * (D / 8) / kThreads;
  copy_tile_rows<D, LPT, kThreads>(src, src0, dst + wave * 64, valid);
}

// LSE * log2(e) of a query row as the backward uses it: a row that saw no
// key (LSE = -inf) must get P = 0, which an exponent offset of +inf gives.
__device__ __forceinline__ float lse_offset(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// Transposed operand read from a dual-swizzled tile: rows r..r+3 (r = the
// lane's row for this 16-lane group), column col (see lds_read_tr16).
template <int RC>
__device__ __forceinline__ int tr_offset(int r, int col) {
  return dual_chunk<RC>(r, col >> 3) * 16 + (col & 7) * 2;
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = 128 keys of one K/V head; wave w owns keys k0w ..
// k0w+31.  K and V rows stay in VGPRs as B operands; tiles of 64 queries of
// Q and dO (plus their LSE and Delta) stream through a double-buffered LDS
// ring -- for grouped heads, the tiles of every query head that shares this
// K/V head, one head after the other, so dK and dV sum over the group in
// registers.
//   S    = Q K^T        (A = Q rows,  B = K^T)        queries x keys
//   dP   = dO V^T       (A = dO rows, B = V^T)
//   P    = exp2(S*scale*log2e - LSE*log2e), dS = P (dP - Delta)
//   dV^T += dO^T P      (A = dO^T via transposed reads, B = P)
//   dK^T += Q^T dS      (A = Q^T  via transposed reads, B = dS)
// Query rows are read in perm23 order, so register r of lane-half g holds
// query acc_row(r, g) of its 32-query block, and P / dS feed the next two
// products straight from their accumulators.
// MASK (key-padding mask): a hidden key has P = 0 in its whole column, so its
// dK and dV rows are exactly zero and the visible keys' columns do not
// depend on it (P uses the saved LSE).  Hidden keys are therefore computed
// like the others and zeroed at the end; a wave whose 32 keys are all hidden
// skips the products, and a workgroup with no visible key skips the loop.
// ---------------------------------------------------------------------------
// DROP (attention dropout): with Z the keep mask regenerated from the Philox
// seed and offset and s the keep scale, dV = (P*Z*s)^T dO and
// dS = P * ((dO V^T)*Z*s - Delta).  A lane holds one key and 16 queries, but
// a Philox block yields 16 keys of one query, so each lane computes the
// block of (query qb0 + lane % 32, keys k0w + 16*(lane / 32) ..) and the keep
// bits are transposed through 128 bytes of LDS per wave.
template <int D, bool CAUSAL, class T, bool MASK, bool DROP>
__global__ __launch_bounds__(kThreads, (D == 64 || !DROP) ? 2 : 1) void dkdv_kernel(BwdArgs a) {
  constexpr int BK = 128, BQ = kTileRows;
  constexpr int RC = D / 8, TC = BQ * RC;
  __shared__ u32x4 lq0[TC], lq1[TC], lg0[TC], lg1[TC];
  __shared__ __attribute__((aligned(16))) float ll0[BQ], ll1[BQ], ld0[BQ], ld1[BQ];
  // Dropout: per wave and 32-query block, 32 words (one per query); bits
  // 0-15 keys k0w..k0w+15, bits 16-31 keys k0w+16..k0w+31.
  __shared__ __attribute__((aligned(16))) uint32_t drop_w[DROP ? kThreads / 64 : 1][2][32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int64_t N = a.N;
  const int G = a.H / a.Hkv;              // query heads per K/V head
  const int BHkv = a.BH / G;
  const int n_parts = a.head_parts;
  const int bhk = blockIdx.x % BHkv;       // K/V head; its query heads are bhk*G .. bhk*G+G-1
  const int part = (blockIdx.x / BHkv) % n_parts;
  const int kt = blockIdx.x / (BHkv * n_parts);  // key tiles heaviest (lowest) first
  const int64_t head = (int64_t)bhk * N * D;

  const int k0w = kt * BK + wave * 32;
  const bool in_range = k0w < N;
  const int my_k = k0w + l32;
  // Mask mode: visibility words of the workgroup's two 64-key tiles; this
  // wave's keys are half (wave % 2) of tile 2kt + wave / 2.
  bool key_vis = true, wg_any = true;
  uint32_t wave_bits = 0xffffffffu;
  if constexpr (MASK) {
    const int64_t b = bhk / a.Hkv;
    const uint64_t* wb = a.mask.words + b * a.mask.n_tiles;
    const uint64_t w0 = wb[2 * kt];
    const uint64_t w1 = 2 * kt + 1 < a.mask.n_tiles ? wb[2 * kt + 1] : 0;
    wave_bits = (uint32_t)(((wave < 2) ? w0 : w1) >> ((wave & 1) * 32));
    key_vis = ((wave_bits >> l32) & 1u) != 0;
    wg_any = (w0 | w1) != 0;
  }
  const bool active = in_range && wave_bits != 0;

  // Resident B operands: lane (key, g) holds K[my_k][16c+8g..+8] and V
  // likewise; lanes past the last key re-read row N-1 and store nothing.
  u32x4 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const int64_t off = head + (int64_t)min(my_k, (int)N - 1) * D + c * 16 + g * 8;
    kf[c] = active ? *(const u32x4*)(a.k + off) : u32x4{0, 0, 0, 0};
    vf[c] = active ? *(const u32x4*)(a.v + off) : u32x4{0, 0, 0, 0};
  }
  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  // LDS byte offsets (see fwd): row reads of query row qb*32 + perm23(l32),
  // chunk 2c + g; transposed reads of rows qb*32 + 16*t2 + 8g + j/4 (+4),
  // columns 32db + 16(q%2) + 4(j%4).  Whole 16-row steps are immediates.
  // The dual swizzle XORs only chunk bits below the row, so the row read of
  // chunk 2c + g is roff0 ^ (32c) and the transposed read of columns 32db +
  // ... is toff[h] ^ (64db); whole 16-row steps are immediates.
  const uint32_t roff0 = dual_chunk<RC>(perm23(l32), g) * 16;
  const int vj = lane & 15, vq = lane >> 4;
  const int t_row0 = 8 * g + (vj >> 2);
  const int t_col = 16 * (vq & 1) + 4 * (vj & 3);
  const uint32_t toff0 = tr_offset<RC>(t_row0, t_col), toff1 = tr_offset<RC>(t_row0 + 4, t_col);
  constexpr int ROW16 = 16 * RC * 16;  // bytes of 16 rows

  const int src0 = tile_src_offset<D, true>(wave * 64 + lane);
  const int n_qt = (int)((N + BQ - 1) / BQ);
  const int qt_begin = CAUSAL ? (kt * BK) / BQ : 0;
  const float c2 = a.scale_log2;

  // The row terms of the next tile travel through registers of threads 0..63
  // and are written to LDS at the end of a step: LSE * log2 e and Delta, or
  // with PRE (D = 128 without dropout) the accumulator starts -LSE / scale
  // and -Delta.  Rows past the last query (and rows that saw no key) get
  // P = 0, hence dS = 0: an offset of +inf, or a start of -inf.
  constexpr bool PRE = D == 128 && !DROP;
  float lse_n = 0.f, dl_n = 0.f;
  auto fetch_rows = [&](int j, int qt) {  // query head bhk*G + j, tile qt
    if (tid < BQ) {
      const int64_t rowbase = (int64_t)(bhk * G + j) * N;
      const int row = qt * BQ + tid;
      if constexpr (PRE) {
        const float l = row < N ? a.lse[rowbase + row] : -INFINITY;
        lse_n = l == -INFINITY ? -INFINITY : -l / a.scale;
        dl_n = row < N ? -a.delta[rowbase + row] : 0.f;
      } else {
        lse_n = row < N ? lse_offset(a.lse[rowbase + row]) : INFINITY;
        dl_n = row < N ? a.delta[rowbase + row] : 0.f;
      }
    }
  };
  auto put_rows = [&](float* ll, float* ld) {
    if (tid < BQ) {
      // The byte offset is made opaque so that it is formed here rather than
      // kept per buffer in live registers across the loop.
      int t4 = tid * 4;
      asm volatile("" : "+v"(t4));
      *(float*)((char*)ll + t4) = lse_n;
      *(float*)((char*)ld + t4) = dl_n;
    }
  };

  // D = 128 with dropout (one wave per SIMD): one 64-query tile = two
  // 32-query blocks, as a software pipeline of four
  // stages whose slices pair one MFMA with one LDS read (kept PR reads
  // ahead) and a share of the vector work, closed by scheduling barriers:
  //   1. S, dP of block 0              (row reads of Q and dO)
  //   2. S, dP of block 1  | P, dS of block 0
  //   3. dV, dK of block 0 | P, dS of block 1   (transposed reads of dO, Q)
  //   4. dV, dK of block 1
  // A block wholly before this wave's keys (causal) is computed and masked
  // to zero rather than skipped, which keeps the pipeline uniform; it only
  // occurs on diagonal tiles.
  constexpr int DB = D / 32;
  constexpr int N1 = 2 * (D / 16);  // S + dP MFMAs per block
  constexpr int N3 = 4 * DB;        // dV + dK MFMAs per block
  constexpr int E1 = 16 / N1 > 0 ? (16 + N1 - 1) / N1 : 1;  // softmax elements per slice
  constexpr int PR = 3;             // row reads in flight
  constexpr int PT = 2;             // transposed read pairs in flight
  auto compute_pipe = [&](int j, int qt, const u32x4* Ql, const u32x4* Gl, const float* ll, const float* ld) {
    const char* Qb = (const char*)Ql;
    const char* Gb = (const char*)Gl;
    const int q0 = qt * BQ;
    uint32_t rb = roff0, tb0 = toff0, tb1 = toff1;
    asm volatile("" : "+v"(rb), "+v"(tb0), "+v"(tb1));
    // row fragment m of the tile: block m / N1; within it, n even -> Q chunk
    // n/2 (S), n odd -> dO chunk n/2 (dP)
    auto row_frag = [&](int m) {
      const int qb = m / N1, n = m % N1;
      return *(const u32x4*)(((n & 1) ? Gb : Qb) + qb * 2 * ROW16 + (rb ^ (32 * (n >> 1))));
    };
    // transposed fragment m: block m / N3; n = (t2*DB + db)*2 + w, w = 0 -> dO^T (dV), 1 -> Q^T (dK)
    auto tr_frag = [&](int m) {
      const int qb = m / N3, n = m % N3;
      const int w = n & 1, db = (n >> 1) % DB, t2 = (n >> 1) / DB;
      const char* base = (w ? Qb : Gb) + (qb * 2 + t2) * ROW16;
      const u32x2 lo = lds_read_tr16(base + (tb0 ^ (64 * db)));
      const u32x2 hi = lds_read_tr16(base + (tb1 ^ (64 * db)));
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    f32x16 s[2], dp[2];
    float lse_r[2][16], dl_r[2][16];
    uint32_t kbits[2] = {0xffffffffu, 0xffffffffu};  // dropout keep bit r: query qb0 + acc_row(r, g)
    if constexpr (DROP) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const uint32_t row_bits = dropout_bits16(k0w / 16 + g, q0 + qb * 32 + l32, (uint64_t)(bhk * G + j),
                                                 a.drop.seed, a.drop.offset, a.drop.thr);
        ((uint16_t*)&drop_w[wave][qb][l32])[g] = (uint16_t)row_bits;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's LDS ops run in order
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const u32x4* wv = (const u32x4*)&drop_w[wave][qb][0];
        const u32x4 w0 = wv[2 * g], w1 = wv[2 * g + 1], w2 = wv[4 + 2 * g], w3 = wv[5 + 2 * g];
        const uint32_t wq[16] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3],
                                 w2[0], w2[1], w2[2], w2[3], w3[0], w3[1], w3[2], w3[3]};
        uint32_t b = 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) b |= ((wq[r] >> l32) & 1u) << r;
        kbits[qb] = b;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the next tile rewrites it
    }
    // LSE (x log2 e) and Delta of the rows a lane's registers hold: register
    // r of block qb is query qb*32 + acc_row(r, g), two runs of 8.
    auto load_rows = [&](int qb) {
      const f32x4* lse4 = (const f32x4*)ll;
      const f32x4* dl4 = (const f32x4*)ld;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v4 = 0; v4 < 2; ++v4) {
          const int idx = (qb * 32 + h * 16 + g * 8) / 4 + v4;
          const f32x4 x = lse4[idx], y = dl4[idx];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lse_r[qb][h * 8 + v4 * 4 + e] = x[e];
            dl_r[qb][h * 8 + v4 * 4 + e] = y[e];
          }
        }
    };
    // Causal mask of block qb on its raw scores (-inf), only where the block
    // meets the diagonal (a uniform test), before its exponentials.
    auto mask_block = [&](int qb) {
      const int qb0 = q0 + qb * 32;
      if (CAUSAL && qb0 < k0w + 31) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (my_k > qb0 + acc_row(r, g)) s[qb][r] = -INFINITY;
      }
    };
    // P and dS of element r of block qb (in place in s, dp)
    const float ks = DROP ? a.drop.keep_scale : 1.f;
    auto softmax_elem = [&](int qb, int r) {
      const float p = fast_exp2(__builtin_fmaf(s[qb][r], c2, -lse_r[qb][r]));
      float pv, ds;
      if constexpr (DROP) {
        const bool keep = (kbits[qb] >> r) & 1u;
        pv = keep ? p * ks : 0.f;                                // dropped, scaled P for dV
        ds = p * ((keep ? dp[qb][r] * ks : 0.f) - dl_r[qb][r]);  // dS
      } else {
        pv = p;
        ds = p * (dp[qb][r] - dl_r[qb][r]);
      }
      // The results stay in this slice (IR-level sinking would otherwise
      // move them past the slice's MFMA, out of its shadow).
      asm volatile("" : "+v"(pv), "+v"(ds));
      s[qb][r] = pv;
      dp[qb][r] = ds;
    };
    u32x4 pf[2][2], sf[2][2];
    // One dword of block qb's packed operands: idx 0-3 P and 4-7 dS of
    // queries 0-7 of each run (t2 = 0), 8-15 the same for t2 = 1.  The dV/dK
    // MFMAs of a block use t2 = 0 first, so the t2 = 1 half is packed in the
    // shadow of those MFMAs.
    auto pack_dw = [&](int qb, int idx) __attribute__((always_inline)) {
      const int t2 = idx >> 3, e = idx & 3, lo = t2 * 8 + 2 * e;
      uint32_t w = (idx & 4) ? pack2<T>(dp[qb][lo], dp[qb][lo + 1]) : pack2<T>(s[qb][lo], s[qb][lo + 1]);
      asm volatile("" : "+v"(w));  // packed in this slice
      if (idx & 4) sf[qb][t2][e] = w;
      else pf[qb][t2][e] = w;
    };
    auto mfma1 = [&](int m, u32x4 f) {  // S or dP MFMA m of the tile
      const int qb = m / N1, n = m % N1;
      if (n & 1) dp[qb] = mfma32<T>(f, vf[n >> 1], dp[qb]);
      else s[qb] = mfma32<T>(f, kf[n >> 1], s[qb]);
    };
    auto mfma3 = [&](int m, u32x4 f) {  // dV or dK MFMA m of the tile
      const int qb = m / N3, n = m % N3;
      const int w = n & 1, db = (n >> 1) % DB, t2 = (n >> 1) / DB;
      if (w) dk[db] = mfma32<T>(f, sf[qb][t2], dk[db]);
      else dv[db] = mfma32<T>(f, pf[qb][t2], dv[db]);
    };

    s[0] = s[1] = dp[0] = dp[1] = f32x16{};
    u32x4 rq[PR + 1];
#pragma unroll
    for (int m = 0; m < PR; ++m) rq[m] = row_frag(m);
    // stage 1: S, dP of block 0
#pragma unroll
    for (int m = 0; m < N1; ++m) {
      rq[(m + PR) % (PR + 1)] = row_frag(m + PR);
      if (m == 1) load_rows(0);
      mfma1(m, rq[m % (PR + 1)]);
      __builtin_amdgcn_sched_barrier(0);
    }
    mask_block(0);
    __builtin_amdgcn_sched_barrier(0);
    // stage 2: S, dP of block 1 | P, dS of block 0
#pragma unroll
    for (int m = N1; m < 2 * N1; ++m) {
      if (m + PR < 2 * N1) rq[(m + PR) % (PR + 1)] = row_frag(m + PR);
      if (m == N1 + 1) load_rows(1);
      mfma1(m, rq[m % (PR + 1)]);
#pragma unroll
      for (int e = 0; e < E1; ++e)
        if ((m - N1) * E1 + e < 16) softmax_elem(0, (m - N1) * E1 + e);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int idx = 0; idx < 8; ++idx) pack_dw(0, idx);
    mask_block(1);
    u32x4 tq[PT + 1];
#pragma unroll
    for (int m = 0; m < PT; ++m) tq[m] = tr_frag(m);
    __builtin_amdgcn_sched_barrier(0);
    // stage 3: dV, dK of block 0 | P, dS of block 1
    constexpr int E3 = (16 + N3 - 1) / N3;
#pragma unroll
    for (int m = 0; m < N3; ++m) {
      tq[(m + PT) % (PT + 1)] = tr_frag(m + PT);
      mfma3(m, tq[m % (PT + 1)]);
      if (m < 8) pack_dw(0, 8 + m);
#pragma unroll
      for (int e = 0; e < E3; ++e)
        if (m * E3 + e < 16) softmax_elem(1, m * E3 + e);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int idx = 0; idx < 8; ++idx) pack_dw(1, idx);
    __builtin_amdgcn_sched_barrier(0);
    // stage 4: dV, dK of block 1
#pragma unroll
    for (int m = N3; m < 2 * N3; ++m) {
      if (m + PT < 2 * N3) tq[(m + PT) % (PT + 1)] = tr_frag(m + PT);
      mfma3(m, tq[m % (PT + 1)]);
      if (m - N3 < 8) pack_dw(1, 8 + m - N3);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // D = 64: the same work one 32-query block at a time, leaving the
  // schedule to the compiler -- the pipelined form needs more registers
  // there and costs one wave per SIMD of occupancy, which measures slower;
  // so does starting the accumulators at -LSE/scale and -Delta (as PRE does
  // below), whose LDS reads then head the critical path of a block of only
  // eight S and dP MFMAs.
  auto compute_blocks = [&](int j, int qt, const u32x4* Ql, const u32x4* Gl, const float* ll, const float* ld) {
    const char* Qb = (const char*)Ql;
    const char* Gb = (const char*)Gl;
    const int q0 = qt * BQ;
#pragma unroll
    for (int qb = 0; qb < BQ / 32; ++qb) {
      const int qb0 = q0 + qb * 32;
      if (CAUSAL && qb0 + 31 < k0w) continue;  // every query precedes every key
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        s = mfma32<T>(*(const u32x4*)(Qb + qb * 2 * ROW16 + (roff0 ^ (32 * c))), kf[c], s);
        dp = mfma32<T>(*(const u32x4*)(Gb + qb * 2 * ROW16 + (roff0 ^ (32 * c))), vf[c], dp);
      }
      // Register r holds query qb*32 + acc_row(r, g): two runs of 8.
      const f32x4* lse4 = (const f32x4*)ll;
      const f32x4* dl4 = (const f32x4*)ld;
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
      uint32_t kbits = 0xffffffffu;
      if constexpr (DROP) {
        const uint32_t row_bits = dropout_bits16(k0w / 16 + g, qb0 + l32, (uint64_t)(bhk * G + j), a.drop.seed,
                                                 a.drop.offset, a.drop.thr);
        asm volatile("" ::: "memory");
        ((uint16_t*)&drop_w[wave][0][l32])[g] = (uint16_t)row_bits;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's LDS ops run in order
        const u32x4* wv = (const u32x4*)&drop_w[wave][0][0];
        const u32x4 w0 = wv[2 * g], w1 = wv[2 * g + 1], w2 = wv[4 + 2 * g], w3 = wv[5 + 2 * g];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // read before the next block rewrites it
        const uint32_t wq[16] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3],
                                 w2[0], w2[1], w2[2], w2[3], w3[0], w3[1], w3[2], w3[3]};
        kbits = 0;
#pragma unroll
        for (int r = 0; r < 16; ++r) kbits |= ((wq[r] >> l32) & 1u) << r;
      }
      const float ks = DROP ? a.drop.keep_scale : 1.f;
      // Causal mask on the raw scores, only on blocks that meet the diagonal
      // (a uniform branch; as a select on every block it cost a quarter of
      // the loop's instructions at D = 64).
      if (__builtin_expect(diag, 0)) {
        asm volatile("");  // keeps the branch
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (my_k > qb0 + acc_row(r, g)) s[r] = -INFINITY;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(__builtin_fmaf(s[r], c2, -lse_r[r]));
        if constexpr (DROP) {
          const bool keep = (kbits >> r) & 1u;
          s[r] = keep ? p * ks : 0.f;                         // dropped, scaled P for dV
          dp[r] = p * ((keep ? dp[r] * ks : 0.f) - dl_r[r]);  // dS
        } else {
          s[r] = p;
          dp[r] = p * (dp[r] - dl_r[r]);
        }
      }
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        const u32x4 pf = pack8<T>(s, t2 * 8);
        const u32x4 sf = pack8<T>(dp, t2 * 8);
        const int rows = (qb * 2 + t2) * ROW16;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const u32x2 glo = lds_read_tr16(Gb + rows + (toff0 ^ (64 * db)));
          const u32x2 ghi = lds_read_tr16(Gb + rows + (toff1 ^ (64 * db)));
          dv[db] = mfma32<T>(u32x4{glo[0], glo[1], ghi[0], ghi[1]}, pf, dv[db]);
          const u32x2 qlo = lds_read_tr16(Qb + rows + (toff0 ^ (64 * db)));
          const u32x2 qhi = lds_read_tr16(Qb + rows + (toff1 ^ (64 * db)));
          dk[db] = mfma32<T>(u32x4{qlo[0], qlo[1], qhi[0], qhi[1]}, sf, dk[db]);
        }
      }
    }
  };
  // D = 128 without dropout (PRE): one 32-query block at a time, at two
  // waves per SIMD.  The S and dP accumulators start at -LSE/scale and
  // -Delta of their rows, read from LDS straight into them, so that
  // P = exp2(S * scale * log2 e) and dS = P dP take no per-row operands and
  // the rows' LSE and Delta hold no registers (with them the kernel needs
  // more than 256 and runs one wave per SIMD).  LDS reads run PFR MFMAs
  // ahead, and the second half of P and dS is packed beside the first dV/dK
  // MFMAs.
  constexpr int PFR = MASK ? 1 : 2, PFT = PFR;  // reads ahead (the mask's state leaves no room for 2)
  auto compute_pre = [&](int qt, const u32x4* Ql, const u32x4* Gl, const float* ll, const float* ld) {
    const char* Qb = (const char*)Ql;
    const char* Gb = (const char*)Gl;
    const int q0 = qt * BQ;
#pragma unroll
    for (int qb = 0; qb < BQ / 32; ++qb) {
      const int qb0 = q0 + qb * 32;
      if (CAUSAL && qb0 + 31 < k0w) continue;  // every query precedes every key
      // Offsets opaque per block: the XORed offsets are formed beside their
      // reads instead of being hoisted out of the loop into live registers.
      uint32_t rb = roff0, tb0 = toff0, tb1 = toff1, g32 = g * 32;
      asm volatile("" : "+v"(rb), "+v"(tb0), "+v"(tb1), "+v"(g32));
      // Register r holds query qb*32 + acc_row(r, g): two runs of 8.
      f32x16 s, dp;
      const f32x4* lse4 = (const f32x4*)((const char*)ll + g32);
      const f32x4* dl4 = (const f32x4*)((const char*)ld + g32);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int v4 = 0; v4 < 2; ++v4) {
          const int idx = (qb * 32 + h * 16) / 4 + v4;
          const f32x4 x = lse4[idx], y = dl4[idx];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            s[h * 8 + v4 * 4 + e] = x[e];
            dp[h * 8 + v4 * 4 + e] = y[e];
          }
        }
      // S and dP: row fragment m is Q chunk m/2 (m even) or dO chunk m/2.
      auto rowf = [&](int m) {
        return *(const u32x4*)(((m & 1) ? Gb : Qb) + qb * 2 * ROW16 + (rb ^ (32 * (m >> 1))));
      };
      constexpr int NR = 2 * (D / 16);
      u32x4 rq[PFR + 1];
#pragma unroll
      for (int m = 0; m < PFR; ++m) rq[m] = rowf(m);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < NR; ++m) {
        if (m + PFR < NR) rq[(m + PFR) % (PFR + 1)] = rowf(m + PFR);
        if (m & 1) dp = mfma32<T>(rq[m % (PFR + 1)], vf[m >> 1], dp);
        else s = mfma32<T>(rq[m % (PFR + 1)], kf[m >> 1], s);
        __builtin_amdgcn_sched_barrier(0);
      }
      // P and dS in place.  Causal: both block starts are multiples of 32,
      // so a block meets the diagonal only when qb0 == k0w, and there query
      // acc_row(r, g) precedes key l32 exactly when l32 > acc_row(r, g): a
      // lane mask per register, applied on that block only, behind a uniform
      // branch (as a select on every block it cost one instruction per score;
      // measured 0.7-1.8 % of the backward).
      const bool diag = CAUSAL && qb0 == k0w;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = fast_exp2(s[r] * c2);
      if (__builtin_expect(diag, 0)) {  // uniform: one block per wave meets the diagonal
        asm volatile("");  // keeps the branch (no select on every block)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (l32 > acc_row(r, g)) s[r] = 0.f;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] = s[r] * dp[r];
      // dV, dK: transposed fragment n = (t2*DB + db)*2 + w (w = 0: dO^T for
      // dV, 1: Q^T for dK); queries 16*t2 .. 16*t2+15 of the block.
      constexpr int DB = D / 32, NT = 4 * DB;
      auto trf = [&](int n) {
        const int w = n & 1, db = (n >> 1) % DB, t2 = (n >> 1) / DB;
        const char* base = (w ? Qb : Gb) + (qb * 2 + t2) * ROW16;
        const u32x2 lo = lds_read_tr16(base + (tb0 ^ (64 * db)));
        const u32x2 hi = lds_read_tr16(base + (tb1 ^ (64 * db)));
        return u32x4{lo[0], lo[1], hi[0], hi[1]};
      };
      u32x4 pf[2], sf[2];
      pf[0] = pack8<T>(s, 0);
      sf[0] = pack8<T>(dp, 0);
      u32x4 tq[PFT + 1];
#pragma unroll
      for (int n = 0; n < PFT; ++n) tq[n] = trf(n);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        if (n + PFT < NT) tq[(n + PFT) % (PFT + 1)] = trf(n + PFT);
        const int w = n & 1, db = (n >> 1) % DB, t2 = (n >> 1) / DB;
        if (w) dk[db] = mfma32<T>(tq[n % (PFT + 1)], sf[t2], dk[db]);
        else dv[db] = mfma32<T>(tq[n % (PFT + 1)], pf[t2], dv[db]);
        if (n == 0) pf[1] = pack8<T>(s, 8);  // queries 16..31, packed beside the t2 = 0 MFMAs
        if (n == 1) sf[1] = pack8<T>(dp, 8);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto compute = [&](int j, int qt, const u32x4* Ql, const u32x4* Gl, const float* ll, const float* ld) {
    if constexpr (PRE) compute_pre(qt, Ql, Gl, ll, ld);
    else if constexpr (D == 128) compute_pipe(j, qt, Ql, Gl, ll, ld);
    else compute_blocks(j, qt, Ql, Gl, ll, ld);
  };

  // The positions of this K/V head and key tile are the query tiles qt of
  // query heads bhk*G + j, j-major (all tiles of a head, then the next head);
  // this part walks its contiguous range of them, as p = 0 .. n_pos-1.  A
  // step computes its tile and starts the copies of the next position's tile
  // (jn, qtn) into the other buffers.
  const int qt_end = wg_any ? n_qt : qt_begin;  // workgroup-uniform
  const int nq = qt_end - qt_begin;
  const int64_t n_all = (int64_t)G * nq;
  const int64_t pos0 = part * n_all / n_parts;
  const int n_pos = (int)((part + 1) * n_all / n_parts - pos0);
  const int j_begin = nq > 0 ? (int)(pos0 / nq) : 0;
  const int qt_first = nq > 0 ? qt_begin + (int)(pos0 % nq) : qt_begin;
  auto load = [&](int j, int qt, u32x4* Qn, u32x4* Gn) {
    const int64_t off = (int64_t)(bhk * G + j) * N * D + (int64_t)qt * BQ * D;
    const int valid = min(BQ, (int)N - qt * BQ);
    copy_tile<D>(a.q + off, src0, Qn, wave, valid);
    copy_tile<D>(a.dout + off, src0, Gn, wave, valid);
  };
  auto step = [&](int p, int j, int qt, int jn, int qtn, const u32x4* Ql, const u32x4* Gl, const float* ll,
                  const float* ld, u32x4* Qn, u32x4* Gn, float* lln, float* ldn) {
    wait_vmem();      // this wave's copies of position p have landed
    __syncthreads();  // everyone's have (and the LSE/Delta rows); position p-1 is done
    if (p + 1 < n_pos) {
      fetch_rows(jn, qtn);  // first, so that storing them later need not wait for the tile copies
      load(jn, qtn, Qn, Gn);
    }
    if (active) compute(j, qt, Ql, Gl, ll, ld);
    if (p + 1 < n_pos) put_rows(lln, ldn);
  };
  // (j, qt) -> the next position
  auto advance = [&](int& j, int& qt) {
    if (++qt == qt_end) {
      qt = qt_begin;
      ++j;
    }
  };

  if (n_pos > 0) {
    load(j_begin, qt_first, lq0, lg0);
    fetch_rows(j_begin, qt_first);
    put_rows(ll0, ld0);
  }
  int j_c = j_begin, qt_c = qt_first;
  for (int p = 0; p < n_pos; p += 2) {
    int j1 = j_c, qt1 = qt_c;
    advance(j1, qt1);
    step(p, j_c, qt_c, j1, qt1, lq0, lg0, ll0, ld0, lq1, lg1, ll1, ld1);
    if (p + 1 < n_pos) {
      int j2 = j1, qt2 = qt1;
      advance(j2, qt2);
      step(p + 1, j1, qt1, j2, qt2, lq1, lg1, ll1, ld1, lq0, lg0, ll0, ld0);
      j_c = j2;
      qt_c = qt2;
    }
  }

  if (!in_range || my_k >= N) return;
  if (MASK && !key_vis) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      dk[i] = f32x16{};
      dv[i] = f32x16{};
    }
  }
  if (n_parts > 1) {  // FP32 partial sums of this part's positions
    const int64_t prow = ((int64_t)part * BHkv + bhk) * N + my_k;
    float* pk = a.part_dk + prow * D;
    float* pv = a.part_dv + prow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d = db * 32 + rq * 8 + g * 4;
        *(f32x4*)(pk + d) = f32x4{dk[db][rq * 4 + 0], dk[db][rq * 4 + 1], dk[db][rq * 4 + 2], dk[db][rq * 4 + 3]};
        *(f32x4*)(pv + d) = f32x4{dv[db][rq * 4 + 0], dv[db][rq * 4 + 1], dv[db][rq * 4 + 2], dv[db][rq * 4 + 3]};
      }
    return;
  }
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
// dQ: workgroup = 128 queries of one query head (its K/V from the head it
// shares); wave w owns queries q0w .. q0w+31.
// Q and dO rows stay in VGPRs as B operands; tiles of 64 keys of K and V
// stream through a double-buffered LDS ring.
//   S^T  = K Q^T        (A = K rows, B = Q^T)         keys x queries
//   dP^T = V dO^T       (A = V rows, B = dO^T)
//   P^T  = exp2(S^T*scale*log2e - LSE*log2e), dS^T = P^T (dP^T - Delta)
//   dQ^T += K^T dS^T    (A = K^T via transposed reads, B = dS^T)
// MASK (key-padding mask): only the non-empty key tiles of the batch
// element's list are visited, and hidden keys of partial tiles get P = 0.
// ---------------------------------------------------------------------------
// DROP: dS^T = P^T * ((V dO^T)*Z*s - Delta), with the keep bits of the
// S^T layout (one query per lane) as in the forward pass.
template <int D, bool CAUSAL, class T, bool MASK, bool DROP>
__global__ __launch_bounds__(kThreads, 2) void dq_kernel(BwdArgs a) {
  constexpr int BM = 128, BN = kTileRows;
  constexpr int RC = D / 8, TC = BN * RC;
  __shared__ u32x4 lk0[TC], lk1[TC], lv0[TC], lv1[TC];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 31, g = lane >> 5;
  const int64_t N = a.N;
  const int n_qtiles = (int)((N + BM - 1) / BM);
  const int G = a.H / a.Hkv;  // query heads per K/V head
  const int n_dqp = a.dq_parts;
  const int bh = head_of_slot(blockIdx.x % a.BH, a.BH, G);
  const int dpart = (blockIdx.x / a.BH) % n_dqp;  // this workgroup's part of the key tiles
  const int rank = blockIdx.x / (a.BH * n_dqp);
  const int qt = CAUSAL ? (n_qtiles - 1 - rank) : rank;
  const int64_t head = (int64_t)bh * N * D;
  const int64_t kv_head = (int64_t)(bh / G) * N * D;
  const uint16_t* __restrict__ Kh = a.k + kv_head;
  const uint16_t* __restrict__ Vh = a.v + kv_head;

  const int q0w = qt * BM + wave * 32;
  const bool active = q0w < N;
  const int my_q = q0w + ql;

  // Lanes past the last query re-read row N-1 and store nothing.
  const bool real_q = my_q < N;
  u32x4 qf[D / 16], gf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    const int64_t off = head + (int64_t)min(my_q, (int)N - 1) * D + c * 16 + g * 8;
    qf[c] = active ? *(const u32x4*)(a.q + off) : u32x4{0, 0, 0, 0};
    gf[c] = active ? *(const u32x4*)(a.dout + off) : u32x4{0, 0, 0, 0};
  }
  const float lse2 = real_q ? lse_offset(a.lse[(int64_t)bh * N + my_q]) : 0.f;
  const float dl = real_q ? a.delta[(int64_t)bh * N + my_q] : 0.f;
  f32x16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dq[i] = f32x16{};

  // LDS byte offsets: K rows (dual swizzle) and V rows (swz) of key
  // kb*32 + perm23(ql), chunk 2c + g are koff0 / voff0 ^ (32c); transposed
  // K reads of rows 16t + 8g + j/4 (+4), columns 32db + 16(q%2) + 4(j%4) are
  // toff0 / toff1 ^ (64db) (the swizzles XOR only chunk bits below the row).
  const int krow = perm23(ql);
  const int vj = lane & 15, vq = lane >> 4;
  const int t_row0 = 8 * g + (vj >> 2);
  const int t_col = 16 * (vq & 1) + 4 * (vj & 3);
  constexpr int ROW16 = 16 * RC * 16;

  const int ksrc0 = tile_src_offset<D, true>(wave * 64 + lane);
  const int vsrc0 = tile_src_offset<D, false>(wave * 64 + lane);
  const int n_kt_all = (int)((N + BN - 1) / BN);
  const int n_kt = CAUSAL ? min(n_kt_all, ((qt + 1) * BM) / BN) : n_kt_all;
  const float c2 = a.scale_log2;

  // One 64-key tile as a software pipeline of four stages whose slices pair
  // one MFMA with one LDS read (kept PR ahead) and a share of the vector
  // work, closed by scheduling barriers:
  //   1. S^T, dP^T of keys 0-31                     (row reads of K and V)
  //   2. S^T, dP^T of keys 32-63 | P, dS of keys 0-31
  //   3. dQ^T += K^T dS^T, keys 0-31 | P, dS of keys 32-63  (transposed K reads)
  //   4. dQ^T += K^T dS^T, keys 32-63
  // Masks (causal diagonal, partial last tile, partly visible tile) set the
  // raw scores of a 32-key block to -inf between stages, in a uniform branch.
  constexpr int DB = D / 32;
  constexpr int N1 = 2 * (D / 16);  // S + dP MFMAs per 32-key block
  constexpr int N3 = 2 * DB;        // dQ MFMAs per 32-key block
  constexpr int PR = 3, PT = 2;
  const uint32_t koff0 = dual_chunk<RC>(krow, g) * 16, voff0 = swz(krow * RC + g) * 16;
  const uint32_t toff0 = tr_offset<RC>(t_row0, t_col), toff1 = tr_offset<RC>(t_row0 + 4, t_col);
  auto compute = [&](int kt, uint32_t wlo, uint32_t whi, const u32x4* Kl, const u32x4* Vl) {
    const char* Kb = (const char*)Kl;
    const char* Vb = (const char*)Vl;
    const int k0 = kt * BN;
    uint32_t kb_ = koff0, vb_ = voff0, tb0 = toff0, tb1 = toff1;
    asm volatile("" : "+v"(kb_), "+v"(vb_), "+v"(tb0), "+v"(tb1));
    // row fragment m: block m / N1; n even -> K chunk n/2 (S^T), odd -> V chunk n/2 (dP^T)
    auto row_frag = [&](int m) {
      const int kb = m / N1, n = m % N1;
      return (n & 1) ? *(const u32x4*)(Vb + kb * 2 * ROW16 + (vb_ ^ (32 * (n >> 1))))
                     : *(const u32x4*)(Kb + kb * 2 * ROW16 + (kb_ ^ (32 * (n >> 1))));
    };
    // transposed K fragment m: 16-key step t = m / DB, column block db = m % DB
    auto tr_frag = [&](int m) {
      const int t = m / DB, db = m % DB;
      const u32x2 lo = lds_read_tr16(Kb + t * ROW16 + (tb0 ^ (64 * db)));
      const u32x2 hi = lds_read_tr16(Kb + t * ROW16 + (tb1 ^ (64 * db)));
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    f32x16 s[2], dp[2];
    const bool need_mask = (CAUSAL && k0 + BN - 1 > q0w) || (MASK ? (wlo & whi) != 0xffffffffu : k0 + BN > N);
    auto mask_block = [&](int kb) {
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + acc_row(r, g);
          const bool hidden = MASK ? key_hidden(wlo, whi, kb, r, g) : key >= N;
          if ((CAUSAL && key > my_q) || hidden) s[kb][r] = -INFINITY;
        }
      }
    };
    uint32_t keep[2] = {0xffffffffu, 0xffffffffu};
    if constexpr (DROP) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        keep[kb] = dropout_bits_st(k0 + kb * 32, my_q, (uint64_t)bh, a.drop.seed, a.drop.offset, a.drop.thr, g);
    }
    const float ks = DROP ? a.drop.keep_scale : 1.f;
    auto softmax_elem = [&](int kb, int r) {
      const float p = fast_exp2(__builtin_fmaf(s[kb][r], c2, -lse2));
      float ds;
      if constexpr (DROP) ds = p * ((((keep[kb] >> r) & 1u) ? dp[kb][r] * ks : 0.f) - dl);
      else ds = p * (dp[kb][r] - dl);
      asm volatile("" : "+v"(ds));  // the result stays in this slice
      dp[kb][r] = ds;
    };
    u32x4 sf[BN / 16];
    auto pack_block = [&](int kb) {
      sf[2 * kb] = pack8<T>(dp[kb], 0);
      sf[2 * kb + 1] = pack8<T>(dp[kb], 8);
    };
    auto mfma1 = [&](int m, u32x4 f) {
      const int kb = m / N1, n = m % N1;
      if (n & 1) dp[kb] = mfma32<T>(f, gf[n >> 1], dp[kb]);
      else s[kb] = mfma32<T>(f, qf[n >> 1], s[kb]);
    };
    auto mfma3 = [&](int m, u32x4 f) { dq[m % DB] = mfma32<T>(f, sf[m / DB], dq[m % DB]); };

    s[0] = s[1] = dp[0] = dp[1] = f32x16{};
    u32x4 rq[PR + 1];
#pragma unroll
    for (int m = 0; m < PR; ++m) rq[m] = row_frag(m);
#pragma unroll
    for (int m = 0; m < N1; ++m) {  // stage 1
      rq[(m + PR) % (PR + 1)] = row_frag(m + PR);
      mfma1(m, rq[m % (PR + 1)]);
      __builtin_amdgcn_sched_barrier(0);
    }
    mask_block(0);
    __builtin_amdgcn_sched_barrier(0);
    constexpr int E1 = (16 + N1 - 1) / N1;
#pragma unroll
    for (int m = N1; m < 2 * N1; ++m) {  // stage 2
      if (m + PR < 2 * N1) rq[(m + PR) % (PR + 1)] = row_frag(m + PR);
      mfma1(m, rq[m % (PR + 1)]);
#pragma unroll
      for (int e = 0; e < E1; ++e)
        if ((m - N1) * E1 + e < 16) softmax_elem(0, (m - N1) * E1 + e);
      __builtin_amdgcn_sched_barrier(0);
    }
    pack_block(0);
    mask_block(1);
    u32x4 tq[PT + 1];
#pragma unroll
    for (int m = 0; m < PT; ++m) tq[m] = tr_frag(m);
    __builtin_amdgcn_sched_barrier(0);
    constexpr int E3 = (16 + N3 - 1) / N3;
#pragma unroll
    for (int m = 0; m < N3; ++m) {  // stage 3
      tq[(m + PT) % (PT + 1)] = tr_frag(m + PT);
      mfma3(m, tq[m % (PT + 1)]);
#pragma unroll
      for (int e = 0; e < E3; ++e)
        if (m * E3 + e < 16) softmax_elem(1, m * E3 + e);
      __builtin_amdgcn_sched_barrier(0);
    }
    pack_block(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = N3; m < 2 * N3; ++m) {  // stage 4
      if (m + PT < 2 * N3) tq[(m + PT) % (PT + 1)] = tr_frag(m + PT);
      mfma3(m, tq[m % (PT + 1)]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  constexpr uint32_t kAll = 0xffffffffu;
  if constexpr (!MASK) {
    // this part's key tiles: kt_lo .. kt_hi-1
    const int kt_lo = (int)((int64_t)dpart * n_kt / n_dqp), kt_hi = (int)((int64_t)(dpart + 1) * n_kt / n_dqp);
    auto step = [&](int kt, const u32x4* Kl, const u32x4* Vl, u32x4* Kn, u32x4* Vn) {
      wait_vmem();
      __syncthreads();
      if (kt + 1 < kt_hi) {
        const int valid = min(BN, (int)N - (kt + 1) * BN);
        copy_tile<D>(Kh + (int64_t)(kt + 1) * BN * D, ksrc0, Kn, wave, valid);
        copy_tile<D>(Vh + (int64_t)(kt + 1) * BN * D, vsrc0, Vn, wave, valid);
      }
      if (!active || (CAUSAL && kt * BN > q0w + 31)) return;
      compute(kt, kAll, kAll, Kl, Vl);
    };
    if (kt_lo < kt_hi) {
      const int valid = min(BN, (int)N - kt_lo * BN);
      copy_tile<D>(Kh + (int64_t)kt_lo * BN * D, ksrc0, lk0, wave, valid);
      copy_tile<D>(Vh + (int64_t)kt_lo * BN * D, vsrc0, lv0, wave, valid);
    }
    for (int kt = kt_lo; kt < kt_hi; kt += 2) {
      step(kt, lk0, lv0, lk1, lv1);
      if (kt + 1 < kt_hi) step(kt + 1, lk1, lv1, lk0, lv0);
    }
  } else {
    // The batch element's non-empty key tiles below the causal limit, at
    // positions 0 .. i_all-1, of which this part walks i_lo .. i_end-1;
    // position i is tile kt_c with word (w_lo, w_hi), and the copies started
    // in its step are of the tile at position i+1.
    const int64_t b = bh / a.H;
    const int i_all = a.mask.prefix[b * (a.mask.n_tiles + 1) + n_kt];
    const int i_lo = (int)((int64_t)dpart * i_all / n_dqp), i_end = (int)((int64_t)(dpart + 1) * i_all / n_dqp);
    auto load = [&](int kt, u32x4* Kn, u32x4* Vn) {
      const int valid = min(BN, (int)N - kt * BN);
      copy_tile<D>(Kh + (int64_t)kt * BN * D, ksrc0, Kn, wave, valid);
      copy_tile<D>(Vh + (int64_t)kt * BN * D, vsrc0, Vn, wave, valid);
    };
    if (i_end > i_lo) {  // workgroup-uniform
      TileWindow win;
      win.init(a.mask.list + b * a.mask.n_tiles, a.mask.words + b * a.mask.n_tiles, i_end, lane, i_lo);
      int kt_c = win.tile(i_lo, lane);
      uint32_t w_lo, w_hi;
      win.word(i_lo, w_lo, w_hi);
      load(kt_c, lk0, lv0);
      auto step = [&](int i, const u32x4* Kl, const u32x4* Vl, u32x4* Kn, u32x4* Vn) {
        int kt1 = 0;
        uint32_t lo1 = 0, hi1 = 0;
        if (i + 1 < i_end) {
          kt1 = win.tile(i + 1, lane);
          win.word(i + 1, lo1, hi1);
        }
        wait_vmem();
        __syncthreads();
        if (i + 1 < i_end) load(kt1, Kn, Vn);
        if (active && !(CAUSAL && kt_c * BN > q0w + 31)) compute(kt_c, w_lo, w_hi, Kl, Vl);
        kt_c = kt1;
        w_lo = lo1;
        w_hi = hi1;
      };
      for (int i = i_lo; i < i_end; i += 2) {
        step(i, lk0, lv0, lk1, lv1);
        if (i + 1 < i_end) step(i + 1, lk1, lv1, lk0, lv0);
      }
    }
  }

  if (!active || !real_q) return;
  if (n_dqp > 1) {  // FP32 partial sum of this part's key tiles, not yet scaled
    float* prow = a.part_dq + (((int64_t)dpart * a.BH + bh) * N + my_q) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq)
        *(f32x4*)(prow + db * 32 + rq * 8 + g * 4) =
            f32x4{dq[db][rq * 4 + 0], dq[db][rq * 4 + 1], dq[db][rq * 4 + 2], dq[db][rq * 4 + 3]};
    return;
  }
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

// Sum of the key-range parts' FP32 dQ (in part order, so the result is
// reproducible), scaled and rounded to T: D/4 threads per query row.
template <int D, class T>
__global__ __launch_bounds__(kThreads) void dq_reduce_kernel(const float* __restrict__ part_dq,
                                                             uint16_t* __restrict__ dq, int64_t rows, int n_parts,
                                                             float scale) {
  constexpr int TPR = D / 4;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / TPR) + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  if (row >= rows) return;
  f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < n_parts; ++p) s += *(const f32x4*)(part_dq + ((int64_t)p * rows + row) * D + c * 4);
  s *= scale;
  *(u32x2*)(dq + row * D + c * 4) = u32x2{pack2<T>(s[0], s[1]), pack2<T>(s[2], s[3])};
}

// Sum of the parts' FP32 dK, dV (in part order, so the result is
// reproducible), dK scaled, both rounded to T: D/4 threads per key row.
template <int D, class T>
__global__ __launch_bounds__(kThreads) void dkdv_reduce_kernel(const float* __restrict__ part_dk,
                                                               const float* __restrict__ part_dv,
                                                               uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                                                               int64_t rows, int n_parts, float scale) {
  constexpr int TPR = D / 4;
  constexpr int RPB = kThreads / TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  if (row >= rows) return;
  f32x4 sk = f32x4{0.f, 0.f, 0.f, 0.f}, sv = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < n_parts; ++p) {
    const int64_t off = ((int64_t)p * rows + row) * D + c * 4;
    sk += *(const f32x4*)(part_dk + off);
    sv += *(const f32x4*)(part_dv + off);
  }
  sk *= scale;
  *(u32x2*)(dk + row * D + c * 4) = u32x2{pack2<T>(sk[0], sk[1]), pack2<T>(sk[2], sk[3])};
  *(u32x2*)(dv + row * D + c * 4) = u32x2{pack2<T>(sv[0], sv[1]), pack2<T>(sv[2], sv[3])};
}

template <int D, bool CAUSAL, class T, bool MASK, bool DROP>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.BH * a.N;
  constexpr int rpb = kThreads / (D / 8);
  hipLaunchKernelGGL((delta_kernel<D, T>), dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(kThreads), 0, stream,
                     a.o, a.dout, a.delta, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n_ktiles = (a.N + 127) / 128;
  const int64_t n_kv_heads = a.BH / (a.H / a.Hkv);
  hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL, T, MASK, DROP>), dim3((unsigned)(n_kv_heads * n_ktiles * a.head_parts)),
                     dim3(kThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.head_parts > 1) {
    const int64_t kv_rows = n_kv_heads * a.N;
    constexpr int rpb = kThreads / (D / 4);
    hipLaunchKernelGGL((dkdv_reduce_kernel<D, T>), dim3((unsigned)((kv_rows + rpb - 1) / rpb)), dim3(kThreads), 0,
                       stream, a.part_dk, a.part_dv, a.dk, a.dv, kv_rows, a.head_parts, a.scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t n_qtiles = (a.N + 127) / 128;
  hipLaunchKernelGGL((dq_kernel<D, CAUSAL, T, MASK, DROP>), dim3((unsigned)(a.BH * n_qtiles * a.dq_parts)),
                     dim3(kThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.dq_parts <= 1) return e;
  constexpr int rpq = kThreads / (D / 4);
  hipLaunchKernelGGL((dq_reduce_kernel<D, T>), dim3((unsigned)((rows + rpq - 1) / rpq)), dim3(kThreads), 0, stream,
                     a.part_dq, a.dq, rows, a.dq_parts, a.scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a, int D, bool causal, int dtype, hipStream_t stream) {
#define FA_BWD_CASE(DD, CC, TT) \
  if (D == DD && causal == CC && dtype == TT::id) return launch_bwd_t<DD, CC, TT, false, false>(a, stream);
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

hipError_t launch_bwd_dropout(const BwdArgs& a, int D, bool causal, int dtype, hipStream_t stream) {
#define FA_BWD_CASE(DD, CC, TT) \
  if (D == DD && causal == CC && dtype == TT::id) return launch_bwd_t<DD, CC, TT, false, true>(a, stream);
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

hipError_t launch_bwd_masked_dropout(const BwdArgs& a, int D, bool causal, int dtype, hipStream_t stream) {
#define FA_BWD_CASE(DD, CC, TT) \
  if (D == DD && causal == CC && dtype == TT::id) return launch_bwd_t<DD, CC, TT, true, true>(a, stream);
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

hipError_t launch_bwd_masked(const BwdArgs& a, int D, bool causal, int dtype, hipStream_t stream) {
#define FA_BWD_CASE(DD, CC, TT) \
  if (D == DD && causal == CC && dtype == TT::id) return launch_bwd_t<DD, CC, TT, true, false>(a, stream);
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
