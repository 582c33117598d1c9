// Standalone user of the C ABI (no Python, no torch): reads bf16 Q, K, V, dO from a binary file,
// runs flash_attn_fwd and flash_attn_bwd (plus the masked forward with lengths and dropout) on a
// stream of its own, and writes O, LSE, dQ, dK, dV and the masked O, LSE to another file.
//
//   abi_roundtrip IN OUT B H N d causal
// IN:  q, k, v, do as bf16 [B,H,N,d] one after the other; then int32 seqlens [B].
// OUT: o (bf16), lse (f32), dq, dk, dv (bf16), o_masked (bf16), lse_masked (f32).
// Exit status 0 on success; any library or runtime error prints its status string and exits 1.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../include/flash_attn.h"

#define CHECK_HIP(x)                                                        \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      std::fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));          \
      std::exit(1);                                                         \
    }                                                                       \
  } while (0)
#define CHECK_FA(x)                                                         \
  do {                                                                      \
    fa_status_t s_ = (x);                                                   \
    if (s_ != FA_OK) {                                                      \
      std::fprintf(stderr, "%s: %s\n", #x, flash_attn_status_string(s_));   \
      std::exit(1);                                                         \
    }                                                                       \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 8) {
    std::fprintf(stderr, "usage: %s IN OUT B H N d causal\n", argv[0]);
    return 2;
  }
  const int B = std::atoi(argv[3]), H = std::atoi(argv[4]), N = std::atoi(argv[5]), d = std::atoi(argv[6]);
  const int causal = std::atoi(argv[7]);
  const size_t elems = (size_t)B * H * N * d, rows = (size_t)B * H * N;
  std::vector<uint16_t> host(4 * elems);
  std::vector<int32_t> seqlens(B);
  FILE* f = std::fopen(argv[1], "rb");
  if (!f || std::fread(host.data(), 2, host.size(), f) != host.size() ||
      std::fread(seqlens.data(), 4, B, f) != (size_t)B) {
    std::fprintf(stderr, "cannot read %s\n", argv[1]);
    return 1;
  }
  std::fclose(f);

  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  void *q, *k, *v, *dout, *o, *dq, *dk, *dv, *om, *ws;
  float *lse, *lsem;
  int32_t* sl;
  const size_t bytes = elems * 2;
  for (void** p : {&q, &k, &v, &dout, &o, &dq, &dk, &dv, &om}) CHECK_HIP(hipMalloc(p, bytes));
  CHECK_HIP(hipMalloc((void**)&lse, rows * 4));
  CHECK_HIP(hipMalloc((void**)&lsem, rows * 4));
  CHECK_HIP(hipMalloc((void**)&sl, B * 4));
  const size_t ws_bytes = flash_attn_bwd_workspace_size(B, H, N, d, FA_DTYPE_BF16);
  CHECK_HIP(hipMalloc(&ws, ws_bytes));
  void* ins[4] = {q, k, v, dout};
  for (int i = 0; i < 4; ++i) CHECK_HIP(hipMemcpy(ins[i], host.data() + i * elems, bytes, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(sl, seqlens.data(), B * 4, hipMemcpyHostToDevice));

  const float scale = 1.0f / std::sqrt((float)d);
  CHECK_FA(flash_attn_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, FA_DTYPE_BF16, stream));
  CHECK_FA(flash_attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, ws_bytes, B, H, N, d, scale, causal, FA_DTYPE_BF16,
                          stream));
  CHECK_FA(flash_attn_fwd_masked(q, k, v, om, lsem, B, H, N, d, scale, causal, sl, nullptr, 0.25f,
                                 0x5eedULL, FA_DTYPE_BF16, stream));
  CHECK_HIP(hipStreamSynchronize(stream));

  std::vector<uint16_t> ob(elems);
  std::vector<float> lb(rows);
  FILE* g = std::fopen(argv[2], "wb");
  if (!g) return 1;
  auto put16 = [&](void* src) {
    CHECK_HIP(hipMemcpy(ob.data(), src, bytes, hipMemcpyDeviceToHost));
    std::fwrite(ob.data(), 2, elems, g);
  };
  auto put32 = [&](float* src) {
    CHECK_HIP(hipMemcpy(lb.data(), src, rows * 4, hipMemcpyDeviceToHost));
    std::fwrite(lb.data(), 4, rows, g);
  };
  put16(o);
  put32(lse);
  put16(dq);
  put16(dk);
  put16(dv);
  put16(om);
  put32(lsem);
  std::fclose(g);
  for (void* p : {q, k, v, dout, o, dq, dk, dv, om, ws}) CHECK_HIP(hipFree(p));
  CHECK_HIP(hipFree(lse));
  CHECK_HIP(hipFree(lsem));
  CHECK_HIP(hipFree(sl));
  CHECK_HIP(hipStreamDestroy(stream));
  return 0;
}
