// fa_mask.hip -- block-level flags of a key-padding mask.
//
// "FlashAttention dataflow and engineering validation on MI50" (§4.3) warns
// that on 64-wide waves an element-level padding test diverges inside the
// wave, and asks that the mask of variable-length sequences be compressed
// beforehand into per-block marks, so that the block loop branches once per
// block.  Here the marks are one 64-bit visibility word per 64-key tile (a
// ballot of the tile's 64 mask bytes), plus a compacted, ascending list of
// the tiles whose word is non-zero and its prefix counts.  Attention kernels
// then visit only listed tiles, test elements only where the word is not all
// ones, and never touch the byte mask.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

namespace {

constexpr int kMaskThreads = 256;

// One wave per (b, tile): lane j reads the byte of key 64t + j.
__global__ __launch_bounds__(kMaskThreads) void mask_words_kernel(const uint8_t* __restrict__ mask,
                                                                 uint64_t* __restrict__ words, int64_t B, int64_t N,
                                                                 int T) {
  const int lane = threadIdx.x & 63;
  const int64_t wt = (int64_t)blockIdx.x * (kMaskThreads / 64) + (threadIdx.x >> 6);
  if (wt >= B * T) return;
  const int64_t b = wt / T;
  const int64_t key = (wt % T) * 64 + lane;
  const bool vis = key < N && mask[b * N + key] != 0;
  const uint64_t w = __builtin_amdgcn_ballot_w64(vis);
  if (lane == 0) words[wt] = w;
}

// One workgroup per batch element: exclusive scan of "word != 0" over the
// element's tiles, 256 tiles per round, writing prefix counts and the list.
__global__ __launch_bounds__(kMaskThreads) void mask_scan_kernel(const uint64_t* __restrict__ words,
                                                                int* __restrict__ prefix, int* __restrict__ list,
                                                                int T) {
  __shared__ int wave_count[kMaskThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t b = blockIdx.x;
  const uint64_t* wb = words + b * T;
  int* pb = prefix + b * (T + 1);
  int* lb = list + b * T;
  int running = 0;
  for (int t0 = 0; t0 < T; t0 += kMaskThreads) {
    const int t = t0 + threadIdx.x;
    const bool nz = t < T && wb[t] != 0;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(nz);
    const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
    if (lane == 0) wave_count[wave] = __builtin_popcountll(bal);
    __syncthreads();
    int before = running, total = 0;
#pragma unroll
    for (int w = 0; w < kMaskThreads / 64; ++w) {
      before += w < wave ? wave_count[w] : 0;
      total += wave_count[w];
    }
    if (t < T) {
      pb[t] = before + below;
      if (nz) lb[before + below] = t;
    }
    running += total;
    __syncthreads();  // wave_count is rewritten next round
  }
  if (threadIdx.x == 0) pb[T] = running;
}

}  // namespace

hipError_t launch_mask_tiles(const uint8_t* key_mask, int64_t B, int64_t N, uint64_t* words, int* prefix, int* list,
                             hipStream_t stream) {
  const int T = (int)((N + 63) / 64);
  const int64_t waves = B * T;
  const int64_t wpb = kMaskThreads / 64;
  hipLaunchKernelGGL(mask_words_kernel, dim3((unsigned)((waves + wpb - 1) / wpb)), dim3(kMaskThreads), 0, stream,
                     key_mask, words, B, N, T);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mask_scan_kernel, dim3((unsigned)B), dim3(kMaskThreads), 0, stream, words, prefix, list, T);
  return hipGetLastError();
}

}  // namespace fa
