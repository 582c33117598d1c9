// The attention-dropout keep mask as bytes, from the same generator and element map the attention
// kernels use (dropout_words in fa_device.h). Not on the attention path itself: it lets a caller
// (or a test) see exactly which probabilities a given seed drops.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

// One thread per Philox call: (flattened head, row, 32-key block, half) -> the 16 keys of that
// half-block, keep[bh][row][key] = 1 if kept else 0 (keys >= Nk are not written).
__global__ __launch_bounds__(256) void dropout_mask_kernel(uint8_t* keep, int Nq, int Nk, long calls, uint32_t seed_lo,
                                                           uint32_t seed_hi, int thr) {
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  if (t >= calls) return;
  const int n_blk = (Nk + 31) / 32;
  const int half = (int)(t & 1);
  const long rest = t >> 1;
  const int blk = (int)(rest % n_blk);
  const long rowi = rest / n_blk;  // bh * Nq + row
  const int row = (int)(rowi % Nq);
  const int bh = (int)(rowi / Nq);
  uint32_t w[4];
  dropout_words(row, blk, bh, half, seed_lo, seed_hi, w);
  uint8_t* dst = keep + rowi * (long)Nk;
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = 32 * blk + 8 * g + 4 * half + e;
      if (key < Nk) dst[key] = dropout_keep(w[g], e, thr) ? 1 : 0;
    }
}

hipError_t launch_dropout_mask(uint8_t* keep, int BH, int Nq, int Nk, const Dropout& drop, hipStream_t stream) {
  const long calls = (long)BH * Nq * ((Nk + 31) / 32) * 2;
  const long blocks = (calls + 255) / 256;
  if (blocks > 0x7fffffffL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dropout_mask_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, keep, Nq, Nk, calls,
                     (uint32_t)drop.seed, (uint32_t)(drop.seed >> 32), drop.threshold);
  return hipGetLastError();
}

}  // namespace fa
