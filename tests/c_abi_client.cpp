// c_abi_client.cpp -- a client of libfa written against include/fa.h alone:
// no PyTorch, only the HIP runtime for device memory and a stream.
//
//   c_abi_client IN OUT B H N D causal dtype scale
//
// IN holds q, k, v, dout ([B,H,N,D] each, 16-bit elements of `dtype`, in
// that order); OUT receives o, dq, dk, dv (same shape and type) and then the
// FP32 LSE [B,H,N].  The program calls fa_fwd, fa_bwd_workspace_bytes and
// fa_bwd on one stream, checks every status with fa_status_str, and exits
// non-zero on any error.  The test that runs it compares OUT with the oracle.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "fa.h"

namespace {

bool hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return false;
}

bool fa_ok(int st, const char* what) {
  if (st == FA_OK) return true;
  std::fprintf(stderr, "%s: %s\n", what, fa_status_str(st));
  return false;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 10) {
    std::fprintf(stderr, "usage: %s IN OUT B H N D causal dtype scale\n", argv[0]);
    return 2;
  }
  const int64_t B = std::atoll(argv[3]), H = std::atoll(argv[4]), N = std::atoll(argv[5]), D = std::atoll(argv[6]);
  const int causal = std::atoi(argv[7]), dtype = std::atoi(argv[8]);
  const float scale = static_cast<float>(std::atof(argv[9]));
  if (B <= 0 || H <= 0 || N <= 0 || D <= 0) return 2;
  const size_t elems = static_cast<size_t>(B * H * N * D), rows = static_cast<size_t>(B * H * N);
  const size_t tbytes = elems * 2;

  std::vector<uint16_t> host(4 * elems);
  FILE* f = std::fopen(argv[1], "rb");
  if (!f || std::fread(host.data(), 2, host.size(), f) != host.size()) {
    std::fprintf(stderr, "cannot read %s\n", argv[1]);
    return 2;
  }
  std::fclose(f);

  hipStream_t stream;
  if (!hip_ok(hipStreamCreate(&stream), "hipStreamCreate")) return 1;
  void *q, *k, *v, *dout, *o, *dq, *dk, *dv, *ws = nullptr;
  float* lse;
  void** bufs[] = {&q, &k, &v, &dout, &o, &dq, &dk, &dv};
  for (void** p : bufs)
    if (!hip_ok(hipMalloc(p, tbytes), "hipMalloc")) return 1;
  if (!hip_ok(hipMalloc(reinterpret_cast<void**>(&lse), rows * sizeof(float)), "hipMalloc")) return 1;
  const size_t ws_bytes = fa_bwd_workspace_bytes(B, H, N, D, causal, dtype);
  if (ws_bytes == 0) {
    std::fprintf(stderr, "fa_bwd_workspace_bytes rejected the shape\n");
    return 1;
  }
  if (!hip_ok(hipMalloc(&ws, ws_bytes), "hipMalloc")) return 1;
  void* ins[] = {q, k, v, dout};
  for (int i = 0; i < 4; ++i)
    if (!hip_ok(hipMemcpy(ins[i], host.data() + i * elems, tbytes, hipMemcpyHostToDevice), "hipMemcpy")) return 1;

  if (!fa_ok(fa_fwd(q, k, v, o, lse, B, H, N, D, causal, scale, dtype, stream), "fa_fwd")) return 1;
  if (!fa_ok(fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, N, D, causal, scale, dtype, ws, ws_bytes, stream),
             "fa_bwd"))
    return 1;
  if (!hip_ok(hipStreamSynchronize(stream), "hipStreamSynchronize")) return 1;

  std::vector<uint16_t> out(4 * elems);
  void* outs[] = {o, dq, dk, dv};
  for (int i = 0; i < 4; ++i)
    if (!hip_ok(hipMemcpy(out.data() + i * elems, outs[i], tbytes, hipMemcpyDeviceToHost), "hipMemcpy")) return 1;
  std::vector<float> lse_h(rows);
  if (!hip_ok(hipMemcpy(lse_h.data(), lse, rows * sizeof(float), hipMemcpyDeviceToHost), "hipMemcpy")) return 1;
  FILE* g = std::fopen(argv[2], "wb");
  if (!g || std::fwrite(out.data(), 2, out.size(), g) != out.size() ||
      std::fwrite(lse_h.data(), sizeof(float), rows, g) != rows) {
    std::fprintf(stderr, "cannot write %s\n", argv[2]);
    return 1;
  }
  std::fclose(g);
  for (void** p : bufs) (void)hipFree(*p);
  (void)hipFree(lse);
  (void)hipFree(ws);
  (void)hipStreamDestroy(stream);
  std::printf("c_abi_client: ok\n");
  return 0;
}
