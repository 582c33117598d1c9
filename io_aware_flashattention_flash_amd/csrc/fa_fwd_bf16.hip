// Fused bf16 attention forward for gfx950.
//
// What it computes (52jiny.com FlashAttention explainer, "key ideas" parts 1-3;
// codechina.net CUDA/FlashAttention article, sections 4.1-4.2 and 5.1): one
// workgroup owns a tile of BR query rows of one (batch, head). It keeps that Q
// tile in registers and streams the K/V tiles of the same head through LDS.
// Per K/V tile it forms the scores on the matrix cores, applies the scale and
// the causal / ragged-tail mask, updates every row's running maximum m and
// running sum l of exponentials (rescaling the earlier output accumulation
// when m grows), and accumulates P V on the matrix cores. Only O and the
// per-row log-sum-exp LSE = m + ln l leave the chip; the N x N score matrix
// never exists in HBM.
//
// gfx950 mapping:
//  * a wave owns 32 query rows and computes the transposed score block
//    S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so each lane holds the scores
//    of ONE query (its column) for 16 of every 32 keys; the other 16 sit in
//    the lane 32 apart. Row max is an in-register max plus one permlane32 swap;
//    the row sum is kept per half and combined once at the end.
//  * the same accumulator registers, rounded to bf16, are the B operand of
//    O^T += V^T P^T; V^T comes from the row-major V tile in LDS through the
//    gfx950 LDS transpose read (ds_read_b64_tr_b16), with the key order chosen
//    to match the accumulator's row order.
//  * the row sum l is accumulated from the fp32 probabilities before they are
//    rounded to bf16 for the matrix cores: summing the rounded values would
//    put up to ~1.6e-3 of error into LSE on rows dominated by a few keys.
//  * exp2 with scale*log2(e) folded in; LSE is converted back to natural log.
//  * K/V tiles are double-buffered in LDS: the global loads of tile j+1 are in
//    flight while tile j is computed; one barrier per tile.
//  * causal: tiles entirely above the diagonal are never loaded; a wave whose
//    32 rows are all above a tile skips its compute; only diagonal and ragged
//    tiles evaluate the mask.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

struct FwdBf16Params {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  int N;
  int nh;
  int n_qt;
  float c;  // scale * log2(e)
};

template <int D, int BC, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void fwd_bf16_kernel(FwdBf16Params p) {
  constexpr int BR = 32 * NW;
  constexpr int NCH = D / 8;
  constexpr int NT = NW * 64;
  constexpr int TILE_BYTES = BC * D * 2;
  constexpr int KCH = BC * NCH / NT;  // 16-byte chunks per thread per K (or V) tile
  static_assert(KCH * NT == BC * NCH, "tile must split evenly over the workgroup");
  constexpr int NKB = BC / 32;  // 32-key blocks per tile
  constexpr int NDB = D / 32;   // 32-row blocks of O^T
  constexpr int NKK = D / 16;   // k-steps of K Q^T
  constexpr int NKS = BC / 16;  // k-steps of V^T P^T
  using T = SwizzledTile<D>;

  __shared__ __attribute__((aligned(16))) char smem[4 * TILE_BYTES];  // [buffer][K, V]

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lq = l & 31, hf = l >> 5;
  const int N = p.N;

  int head, qt;
  map_workgroup(blockIdx.x, p.n_qt, p.nh, CAUSAL, head, qt);
  const size_t base = (size_t)head * N * D;
  const bf16* Qh = p.q + base;
  const bf16* Kh = p.k + base;
  const bf16* Vh = p.v + base;

  const int q_w0 = qt * BR + 32 * w;  // first query row of this wave
  const int q = q_w0 + lq;            // this lane's query row

  // Q^T operand: lane (q, hf) holds Q[q][16*kk + 8*hf .. +7].
  bf16x8 qreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    u32x4 t = {0, 0, 0, 0};
    if (q < N) t = ld_global16(Qh + (size_t)q * D + 16 * kk + 8 * hf);
    qreg[kk] = __builtin_bit_cast(bf16x8, t);
  }

  int n_kv = (N + BC - 1) / BC;
  if (CAUSAL) n_kv = min(n_kv, (min(N, (qt + 1) * BR) - 1) / BC + 1);

  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // Staging registers for the next K/V tile (global -> registers -> LDS).
  u32x4 stK[KCH], stV[KCH];
  auto gload = [&](int j) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int x = tid + i * NT, r = x / NCH, c = x % NCH, key = j * BC + r;
      stK[i] = u32x4{0, 0, 0, 0};
      stV[i] = u32x4{0, 0, 0, 0};
      if (key < N) {
        stK[i] = ld_global16(Kh + (size_t)key * D + 8 * c);
        stV[i] = ld_global16(Vh + (size_t)key * D + 8 * c);
      }
    }
  };
  auto swrite = [&](int buf) {
    char* kb = smem + buf * 2 * TILE_BYTES;
    char* vb = kb + TILE_BYTES;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int x = tid + i * NT, r = x / NCH, c = x % NCH;
      const int off = T::chunk_off(r, c);
      lds_write16(kb, off, stK[i]);
      lds_write16(vb, off, stV[i]);
    }
  };

  // Lane-constant parts of the V^T transpose-read addresses.
  const int g16 = l >> 4, j16 = l & 15;
  const int v_row_lane = 4 * hf + (j16 >> 2);
  const int v_col_lane = 16 * (g16 & 1) + 4 * (j16 & 3);

  gload(0);
  swrite(0);
  __syncthreads();

  for (int j = 0; j < n_kv; ++j) {
    if (j + 1 < n_kv) gload(j + 1);
    const char* kbuf = smem + (j & 1) * 2 * TILE_BYTES;
    const char* vbuf = kbuf + TILE_BYTES;
    const int key0 = j * BC;
    const bool active = !CAUSAL || key0 <= q_w0 + 31;  // wave-uniform
    if (active) {
      // S^T = K Q^T for the NKB 32-key blocks of this tile.
      f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
          s[kb] = mfma_bf16_32x32x16(lds_read16(kbuf, T::chunk_off(32 * kb + lq, 2 * kk + hf)), qreg[kk], s[kb]);
      }
      // Scale into the log2 domain, mask, running max.
      const bool need_mask = (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > q_w0);
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[kb][r] * p.c;
          if (need_mask) {
            const int key = key0 + 32 * kb + (r >> 2) * 8 + 4 * hf + (r & 3);
            if (key >= N || (CAUSAL && key > q)) x = -INFINITY;
          }
          s[kb][r] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = half_swap_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      // P^T = exp2(S - m), rounded to bf16, packed as the B operand of V^T P^T.
      bf16x8 pk[NKS];
      float rs = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pe = fast_exp2(s[ks >> 1][(ks & 1) * 8 + e] - m_use);
          rs += pe;
          pk[ks][e] = (bf16)pe;
        }
      }
      l_run = l_run * alpha + rs;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;
      // O^T += V^T P^T. k-step ks covers keys 16ks + {4hf..4hf+3, 8+4hf..8+4hf+3}, matching
      // accumulator registers (ks&1)*8 + 0..7 of block ks>>1.
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const int col = 32 * db + v_col_lane;
          const bf16x4 a0 = lds_read_tr16(vbuf, T::elem_off(16 * ks + v_row_lane, col));
          const bf16x4 a1 = lds_read_tr16(vbuf, T::elem_off(16 * ks + 8 + v_row_lane, col));
          acc_o[db] = mfma_bf16_32x32x16(cat4(a0, a1), pk[ks], acc_o[db]);
        }
      }
    }
    if (j + 1 < n_kv) swrite((j + 1) & 1);
    __syncthreads();
  }

  // Epilogue: O = O_acc / l, LSE = ln2 * (m + log2 l).
  const float l_tot = half_swap_sum(l_run);
  const float inv = 1.0f / l_tot;
  if (q < N) {
    bf16* Oq = p.o + base + (size_t)q * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = (bf16)(acc_o[db][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(Oq + 32 * db + 8 * g + 4 * hf) = t;
      }
    }
    if (hf == 0 && p.lse) p.lse[(size_t)head * N + q] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

template <int D, int BC, int NW, bool CAUSAL>
static hipError_t launch_cfg(const FwdBf16Params& prm, hipStream_t stream) {
  const int grid = prm.n_qt * prm.nh;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, BC, NW, CAUSAL>), dim3(grid), dim3(NW * 64), 0, stream, prm);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N,
                           int d, float scale, bool causal, hipStream_t stream) {
  constexpr int NW = 4, BR = 32 * NW;
  FwdBf16Params prm;
  prm.q = static_cast<const bf16*>(q);
  prm.k = static_cast<const bf16*>(k);
  prm.v = static_cast<const bf16*>(v);
  prm.o = static_cast<bf16*>(o);
  prm.lse = lse;
  prm.N = N;
  prm.nh = BH;
  prm.n_qt = (N + BR - 1) / BR;
  prm.c = scale * kLog2e;
  if (d == 64) return causal ? launch_cfg<64, 64, NW, true>(prm, stream) : launch_cfg<64, 64, NW, false>(prm, stream);
  if (d == 128) return causal ? launch_cfg<128, 64, NW, true>(prm, stream) : launch_cfg<128, 64, NW, false>(prm, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
