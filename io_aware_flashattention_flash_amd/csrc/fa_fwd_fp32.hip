// Fused fp32 attention forward for gfx950.
//
// The same tiled online-softmax algorithm as the bf16 kernel (52jiny.com
// FlashAttention explainer, "key ideas" parts 1-3; codechina.net
// CUDA/FlashAttention article, sections 4.1-4.2), with fp32 storage and the
// fp32 matrix instruction v_mfma_f32_32x32x2_f32, so no operand is rounded:
// P stays fp32 in the P V product. A wave owns 32 query rows and computes
// S^T = K Q^T; K/V tiles of 32 keys pass through LDS (rows padded by one float
// to spread banks). This path serves small or precision-sensitive problems;
// the bf16 kernel is the throughput path.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

struct FwdF32Params {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int N;
  int nh;
  int n_qt;
  float c;  // scale * log2(e)
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_fp32_kernel(FwdF32Params p) {
  constexpr int NW = 4, BR = 32 * NW, BC = 32, LD = D + 1, NT = 256;
  constexpr int NDB = D / 32;
  constexpr int PER = BC * D / NT;  // K (and V) elements each thread moves per tile
  __shared__ float ks_buf[2][BC * LD];
  __shared__ float vs_buf[2][BC * LD];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lq = l & 31, hf = l >> 5;
  const int N = p.N;
  int head, qt;
  map_workgroup(blockIdx.x, p.n_qt, p.nh, CAUSAL ? Order::kLongestFirst : Order::kHeadMajor, true, head, qt);
  const size_t base = (size_t)head * N * D;
  const int q_w0 = qt * BR + 32 * w;
  const int q = q_w0 + lq;

  // Q^T operand of the K=2 instruction: lane (q, hf) holds Q[q][2*kk + hf].
  float qreg[D / 2];
#pragma unroll
  for (int kk = 0; kk < D / 2; ++kk) qreg[kk] = (q < N) ? p.q[base + (size_t)q * D + 2 * kk + hf] : 0.f;

  int n_kv = (N + BC - 1) / BC;
  if (CAUSAL) n_kv = min(n_kv, (min(N, (qt + 1) * BR) - 1) / BC + 1);

  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // K/V tiles are double-buffered: tile j+1's global loads are issued into registers before tile
  // j is computed and stored to the other buffer after it, so their latency hides behind the
  // compute. The barrier at the top of an iteration makes the stores visible and guarantees that
  // every wave is done with the buffer the next stores overwrite.
  float kx[PER], vx[PER];
  auto fetch = [&](int j) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int x = tid + NT * i, r = x / D, c = x % D, key = j * BC + r;
      kx[i] = key < N ? p.k[base + (size_t)key * D + c] : 0.f;
      vx[i] = key < N ? p.v[base + (size_t)key * D + c] : 0.f;
    }
  };
  auto deposit = [&](int b) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int x = tid + NT * i, r = x / D, c = x % D;
      ks_buf[b][r * LD + c] = kx[i];
      vs_buf[b][r * LD + c] = vx[i];
    }
  };
  if (n_kv > 0) {
    fetch(0);
    deposit(0);
  }
  for (int j = 0; j < n_kv; ++j) {
    const int key0 = j * BC;
    __syncthreads();  // tile j is in buffer j % 2; every wave is done with buffer (j + 1) % 2
    if (j + 1 < n_kv) fetch(j + 1);
    const float* ks = ks_buf[j & 1];
    const float* vs = vs_buf[j & 1];
    if (!(CAUSAL && key0 > q_w0 + 31)) {  // wave-uniform: skip tiles whose keys all follow this wave's rows
      f32x16 s = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 2; ++kk) s = mfma_f32_32x32x2(ks[lq * LD + 2 * kk + hf], qreg[kk], s);

      const bool need_mask = (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > q_w0);
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[r] * p.c;
        if (need_mask) {
          const int key = key0 + (r >> 2) * 8 + 4 * hf + (r & 3);
          if (key >= N || (CAUSAL && key > q)) x = -INFINITY;
        }
        s[r] = x;
        mx = fmaxf(mx, x);
      }
      mx = half_swap_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      float rs = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = fast_exp2(s[r] - m_use);
        rs += s[r];
      }
      l_run = l_run * alpha + rs;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        acc_o[db] *= alpha;
        // k-step t pairs register t of both halves: keys (t/4)*8 + 4*hf + t%4.
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int key = (t >> 2) * 8 + 4 * hf + (t & 3);
          acc_o[db] = mfma_f32_32x32x2(vs[key * LD + 32 * db + lq], s[t], acc_o[db]);
        }
      }
    }
    if (j + 1 < n_kv) deposit((j + 1) & 1);
  }

  const float l_tot = half_swap_sum(l_run);
  const float inv = 1.0f / l_tot;
  if (q < N) {
    float* Oq = p.o + base + (size_t)q * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = acc_o[db][4 * g + e] * inv;
        *reinterpret_cast<f32x4*>(Oq + 32 * db + 8 * g + 4 * hf) = t;
      }
    }
    if (hf == 0 && p.lse) p.lse[(size_t)head * N + q] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_cfg(const FwdF32Params& prm, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_fp32_kernel<D, CAUSAL>), dim3(prm.n_qt * prm.nh), dim3(256), 0, stream, prm);
  return hipGetLastError();
}

hipError_t launch_fwd_fp32(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N,
                           int d, float scale, bool causal, hipStream_t stream) {
  FwdF32Params prm;
  prm.q = static_cast<const float*>(q);
  prm.k = static_cast<const float*>(k);
  prm.v = static_cast<const float*>(v);
  prm.o = static_cast<float*>(o);
  prm.lse = lse;
  prm.N = N;
  prm.nh = BH;
  prm.n_qt = (N + 127) / 128;
  prm.c = scale * kLog2e;
  if (d == 64) return causal ? launch_cfg<64, true>(prm, stream) : launch_cfg<64, false>(prm, stream);
  if (d == 128) return causal ? launch_cfg<128, true>(prm, stream) : launch_cfg<128, false>(prm, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
