// Recompute-based attention backward for gfx950 (bf16 storage, fp32 math).
//
// The forward saves only O and the per-row LSE; the backward recomputes the
// probabilities tile by tile from them instead of reading a stored N x N
// matrix (52jiny.com FlashAttention explainer, "key ideas" part 4). For the
// loss sum(O * dO) the gradients are, with P = exp(scale * Q K^T - LSE):
//   delta = rowsum(dO * O)      dV = P^T dO      dP = dO V^T
//   dS = P * (dP - delta)       dQ = scale * dS K      dK = scale * dS^T Q
// (the chain rule through the row softmax; the pages give the recompute idea,
// not the formulas).
//
// Three kernels, launched in order on one stream, no atomics (deterministic):
//  1. delta kernel: one fp32 value per query row into the workspace.
//  2. dK/dV kernel (key-outer): a workgroup owns 32*NW keys, a wave owns 32 of
//     them and keeps K^T / V^T operands and the dK^T / dV^T accumulators in
//     registers while Q, dO, LSE and delta tiles stream through LDS. It uses
//     the untransposed score block S = Q K^T, so a lane holds one key and the
//     registers run over queries: P and dS, rounded to bf16, are directly the
//     B operands of dV^T += dO^T P and dK^T += Q^T dS, whose A operands
//     (dO^T, Q^T) come from the LDS transpose read.
//  3. dQ kernel (query-outer): the forward's layout (S^T = K Q^T, a lane holds
//     one query); recomputes P and dP, forms dS^T and accumulates
//     dQ^T += K^T dS^T with K^T from the LDS transpose read.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

struct BwdParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const bf16* dout;
  const float* lse;
  float* delta;
  bf16* dq;
  bf16* dk;
  bf16* dv;
  int N;
  int nh;
  int n_tiles;
  float c;      // scale * log2(e)
  float scale;
};

// ---------------------------------------------------------------------------------------------
// 1. delta = rowsum(dO * O)
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdParams p) {
  constexpr int TPR = D / 8;        // threads per row, one 16-byte chunk each
  constexpr int RPB = 256 / TPR;    // rows per block
  const int tid = threadIdx.x;
  const size_t rows = (size_t)p.nh * p.N;
  const size_t row = (size_t)blockIdx.x * RPB + tid / TPR;
  const int c = tid % TPR;
  float acc = 0.f;
  if (row < rows) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, ld_global16(p.o + row * D + 8 * c));
    const bf16x8 b = __builtin_bit_cast(bf16x8, ld_global16(p.dout + row * D + 8 * c));
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && c == 0) p.delta[row] = acc;
}

// ---------------------------------------------------------------------------------------------
// 2. dK, dV (key-outer)
// ---------------------------------------------------------------------------------------------
template <int D, int NW, int BQ, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, (D > 64 ? 1 : 2)) void bwd_dkdv_kernel(BwdParams p) {
  constexpr int BKV = 32 * NW;
  constexpr int NCH = D / 8;
  constexpr int NT = NW * 64;
  constexpr int TILE_BYTES = BQ * D * 2;
  constexpr int KCH = BQ * NCH / NT;
  static_assert(KCH * NT == BQ * NCH, "tile must split evenly over the workgroup");
  static_assert(BQ <= NT, "one thread per row of LSE/delta");
  constexpr int NKK = D / 16, NDB = D / 32, NQB = BQ / 32;
  constexpr int BUF_BYTES = 2 * TILE_BYTES + 2 * BQ * 4;  // Q, dO, lse2, delta
  using T = SwizzledTile<D>;

  __shared__ __attribute__((aligned(16))) char smem[2 * BUF_BYTES];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lq = l & 31, hf = l >> 5;
  const int N = p.N;
  int head, kt;
  map_workgroup(blockIdx.x, p.n_tiles, p.nh, false, head, kt);  // causal: tile 0 has the most work
  const size_t base = (size_t)head * N * D;
  const size_t rbase = (size_t)head * N;
  const int key_w0 = kt * BKV + 32 * w;
  const int key = key_w0 + lq;

  // K^T and V^T operands (B side of S = Q K^T and dP = dO V^T): lane (key, hf).
  bf16x8 kreg[NKK], vreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
    if (key < N) {
      a = ld_global16(p.k + base + (size_t)key * D + 16 * kk + 8 * hf);
      b = ld_global16(p.v + base + (size_t)key * D + 16 * kk + 8 * hf);
    }
    kreg[kk] = __builtin_bit_cast(bf16x8, a);
    vreg[kk] = __builtin_bit_cast(bf16x8, b);
  }

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  const int n_qt = (N + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? (kt * BKV) / BQ : 0;

  u32x4 stQ[KCH], stO[KCH];
  float stL = 0.f, stD = 0.f;
  auto gload = [&](int i) {
#pragma unroll
    for (int t = 0; t < KCH; ++t) {
      const int x = tid + t * NT, r = x / NCH, c = x % NCH, row = i * BQ + r;
      stQ[t] = u32x4{0, 0, 0, 0};
      stO[t] = u32x4{0, 0, 0, 0};
      if (row < N) {
        stQ[t] = ld_global16(p.q + base + (size_t)row * D + 8 * c);
        stO[t] = ld_global16(p.dout + base + (size_t)row * D + 8 * c);
      }
    }
    if (tid < BQ) {
      const int row = i * BQ + tid;
      stL = row < N ? p.lse[rbase + row] * kLog2e : 0.f;
      stD = row < N ? p.delta[rbase + row] : 0.f;
    }
  };
  auto swrite = [&](int buf) {
    char* qb = smem + buf * BUF_BYTES;
    char* ob = qb + TILE_BYTES;
    float* lb = reinterpret_cast<float*>(ob + TILE_BYTES);
#pragma unroll
    for (int t = 0; t < KCH; ++t) {
      const int x = tid + t * NT, r = x / NCH, c = x % NCH;
      const int off = T::chunk_off(r, c);
      lds_write16(qb, off, stQ[t]);
      lds_write16(ob, off, stO[t]);
    }
    if (tid < BQ) {
      lb[tid] = stL;
      lb[BQ + tid] = stD;
    }
  };

  const int g16 = l >> 4, j16 = l & 15;
  const int tr_row_lane = 4 * hf + (j16 >> 2);
  const int tr_col_lane = 16 * (g16 & 1) + 4 * (j16 & 3);

  if (qt0 < n_qt) {
    gload(qt0);
    swrite(qt0 & 1);
  }
  __syncthreads();

  for (int i = qt0; i < n_qt; ++i) {
    if (i + 1 < n_qt) gload(i + 1);
    const char* qbuf = smem + (i & 1) * BUF_BYTES;
    const char* obuf = qbuf + TILE_BYTES;
    const float* lbuf = reinterpret_cast<const float*>(obuf + TILE_BYTES);
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int q0 = i * BQ + 32 * qb;
      if (q0 >= N) continue;                          // ragged last tile
      if (CAUSAL && q0 + 31 < key_w0) continue;       // every query precedes every key of this wave
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int off = T::chunk_off(32 * qb + lq, 2 * kk + hf);
        s = mfma_bf16_32x32x16(lds_read16(qbuf, off), kreg[kk], s);
        dp = mfma_bf16_32x32x16(lds_read16(obuf, off), vreg[kk], dp);
      }
      const bool need_mask = (q0 + 32 > N) || (CAUSAL && q0 < key_w0 + 31);
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 lse4 = *reinterpret_cast<const f32x4*>(lbuf + 32 * qb + 8 * g + 4 * hf);
        const f32x4 dl4 = *reinterpret_cast<const f32x4*>(lbuf + BQ + 32 * qb + 8 * g + 4 * hf);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float pr = fast_exp2(s[r] * p.c - lse4[e]);
          if (need_mask) {
            const int qr = q0 + 8 * g + 4 * hf + e;
            if (qr >= N || (CAUSAL && key > qr)) pr = 0.f;
          }
          const float ds = pr * (dp[r] - dl4[e]);
          pb[r >> 3][r & 7] = (bf16)pr;
          dsb[r >> 3][r & 7] = (bf16)ds;
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS; k-step ks covers queries
      // 32qb + 16ks + {4hf..4hf+3, 8+4hf..8+4hf+3}.
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int col = 32 * db + tr_col_lane;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int r0 = 32 * qb + 16 * ks + tr_row_lane;
          const int o0 = T::elem_off(r0, col), o1 = T::elem_off(r0 + 8, col);
          dv[db] = mfma_bf16_32x32x16(cat4(lds_read_tr16(obuf, o0), lds_read_tr16(obuf, o1)), pb[ks], dv[db]);
          dk[db] = mfma_bf16_32x32x16(cat4(lds_read_tr16(qbuf, o0), lds_read_tr16(qbuf, o1)), dsb[ks], dk[db]);
        }
      }
    }
    if (i + 1 < n_qt) swrite((i + 1) & 1);
    __syncthreads();
  }

  if (key < N) {
    bf16* dKr = p.dk + base + (size_t)key * D;
    bf16* dVr = p.dv + base + (size_t)key * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = (bf16)(dk[db][4 * g + e] * p.scale);
          b[e] = (bf16)dv[db][4 * g + e];
        }
        *reinterpret_cast<bf16x4*>(dKr + 32 * db + 8 * g + 4 * hf) = a;
        *reinterpret_cast<bf16x4*>(dVr + 32 * db + 8 * g + 4 * hf) = b;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// 3. dQ (query-outer)
// ---------------------------------------------------------------------------------------------
template <int D, int BC, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dq_kernel(BwdParams p) {
  constexpr int BR = 32 * NW;
  constexpr int NCH = D / 8;
  constexpr int NT = NW * 64;
  constexpr int TILE_BYTES = BC * D * 2;
  constexpr int KCH = BC * NCH / NT;
  static_assert(KCH * NT == BC * NCH, "tile must split evenly over the workgroup");
  constexpr int NKB = BC / 32, NDB = D / 32, NKK = D / 16, NKS = BC / 16;
  using T = SwizzledTile<D>;

  __shared__ __attribute__((aligned(16))) char smem[4 * TILE_BYTES];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lq = l & 31, hf = l >> 5;
  const int N = p.N;
  int head, qt;
  map_workgroup(blockIdx.x, p.n_tiles, p.nh, CAUSAL, head, qt);
  const size_t base = (size_t)head * N * D;
  const int q_w0 = qt * BR + 32 * w;
  const int q = q_w0 + lq;

  bf16x8 qreg[NKK], oreg[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    u32x4 a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
    if (q < N) {
      a = ld_global16(p.q + base + (size_t)q * D + 16 * kk + 8 * hf);
      b = ld_global16(p.dout + base + (size_t)q * D + 16 * kk + 8 * hf);
    }
    qreg[kk] = __builtin_bit_cast(bf16x8, a);
    oreg[kk] = __builtin_bit_cast(bf16x8, b);
  }
  const float lse2 = q < N ? p.lse[(size_t)head * N + q] * kLog2e : 0.f;
  const float dlt = q < N ? p.delta[(size_t)head * N + q] : 0.f;

  int n_kv = (N + BC - 1) / BC;
  if (CAUSAL) n_kv = min(n_kv, (min(N, (qt + 1) * BR) - 1) / BC + 1);

  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq[db] = f32x16{};

  u32x4 stK[KCH], stV[KCH];
  auto gload = [&](int j) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int x = tid + i * NT, r = x / NCH, c = x % NCH, key = j * BC + r;
      stK[i] = u32x4{0, 0, 0, 0};
      stV[i] = u32x4{0, 0, 0, 0};
      if (key < N) {
        stK[i] = ld_global16(p.k + base + (size_t)key * D + 8 * c);
        stV[i] = ld_global16(p.v + base + (size_t)key * D + 8 * c);
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

  const int g16 = l >> 4, j16 = l & 15;
  const int tr_row_lane = 4 * hf + (j16 >> 2);
  const int tr_col_lane = 16 * (g16 & 1) + 4 * (j16 & 3);

  gload(0);
  swrite(0);
  __syncthreads();

  for (int j = 0; j < n_kv; ++j) {
    if (j + 1 < n_kv) gload(j + 1);
    const char* kbuf = smem + (j & 1) * 2 * TILE_BYTES;
    const char* vbuf = kbuf + TILE_BYTES;
    const int key0 = j * BC;
    const bool active = !CAUSAL || key0 <= q_w0 + 31;
    if (active) {
      f32x16 s[NKB], dp[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16{};
        dp[kb] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const int off = T::chunk_off(32 * kb + lq, 2 * kk + hf);
          s[kb] = mfma_bf16_32x32x16(lds_read16(kbuf, off), qreg[kk], s[kb]);
          dp[kb] = mfma_bf16_32x32x16(lds_read16(vbuf, off), oreg[kk], dp[kb]);
        }
      }
      const bool need_mask = (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > q_w0);
      bf16x8 dsb[NKS];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pr = fast_exp2(s[kb][r] * p.c - lse2);
          if (need_mask) {
            const int kr = key0 + 32 * kb + (r >> 2) * 8 + 4 * hf + (r & 3);
            if (kr >= N || (CAUSAL && kr > q)) pr = 0.f;
          }
          dsb[2 * kb + (r >> 3)][r & 7] = (bf16)(pr * (dp[kb][r] - dlt));
        }
      }
      // dQ^T += K^T dS^T; k-step ks covers keys 16ks + {4hf..4hf+3, 8+4hf..8+4hf+3}.
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int col = 32 * db + tr_col_lane;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const bf16x4 a0 = lds_read_tr16(kbuf, T::elem_off(16 * ks + tr_row_lane, col));
          const bf16x4 a1 = lds_read_tr16(kbuf, T::elem_off(16 * ks + 8 + tr_row_lane, col));
          dq[db] = mfma_bf16_32x32x16(cat4(a0, a1), dsb[ks], dq[db]);
        }
      }
    }
    if (j + 1 < n_kv) swrite((j + 1) & 1);
    __syncthreads();
  }

  if (q < N) {
    bf16* dQr = p.dq + base + (size_t)q * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = (bf16)(dq[db][4 * g + e] * p.scale);
        *reinterpret_cast<bf16x4*>(dQr + 32 * db + 8 * g + 4 * hf) = t;
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------------
namespace {
constexpr int kDqNW = 4, kDqBC = 64, kKvNW = 4, kKvBQ = 64;

BwdParams make_params(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, const float* delta, void* dq, void* dk, void* dv, int BH, int N,
                      float scale) {
  BwdParams prm;
  prm.q = static_cast<const bf16*>(q);
  prm.k = static_cast<const bf16*>(k);
  prm.v = static_cast<const bf16*>(v);
  prm.o = static_cast<const bf16*>(o);
  prm.dout = static_cast<const bf16*>(dout);
  prm.lse = lse;
  prm.delta = const_cast<float*>(delta);
  prm.dq = static_cast<bf16*>(dq);
  prm.dk = static_cast<bf16*>(dk);
  prm.dv = static_cast<bf16*>(dv);
  prm.N = N;
  prm.nh = BH;
  prm.n_tiles = 0;
  prm.c = scale * kLog2e;
  prm.scale = scale;
  return prm;
}

template <int D>
hipError_t delta_d(BwdParams prm, hipStream_t stream) {
  constexpr int RPB = 256 / (D / 8);
  const long rows = (long)prm.nh * prm.N;
  hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, stream, prm);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t dkdv_d(BwdParams prm, hipStream_t stream) {
  prm.n_tiles = (prm.N + 32 * kKvNW - 1) / (32 * kKvNW);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, kKvNW, kKvBQ, CAUSAL>), dim3(prm.n_tiles * prm.nh), dim3(kKvNW * 64), 0,
                     stream, prm);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t dq_d(BwdParams prm, hipStream_t stream) {
  prm.n_tiles = (prm.N + 32 * kDqNW - 1) / (32 * kDqNW);
  hipLaunchKernelGGL((bwd_dq_kernel<D, kDqBC, kDqNW, CAUSAL>), dim3(prm.n_tiles * prm.nh), dim3(kDqNW * 64), 0,
                     stream, prm);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_bwd_delta(const void* o, const void* dout, float* delta, int BH, int N, int d,
                            hipStream_t stream) {
  BwdParams prm = make_params(nullptr, nullptr, nullptr, o, nullptr, dout, delta, nullptr, nullptr, nullptr, BH, N,
                              1.f);
  if (d == 64) return delta_d<64>(prm, stream);
  if (d == 128) return delta_d<128>(prm, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                           const float* delta, void* dk, void* dv, int BH, int N, int d, float scale, bool causal,
                           hipStream_t stream) {
  BwdParams prm = make_params(q, k, v, nullptr, lse, dout, delta, nullptr, dk, dv, BH, N, scale);
  if (d == 64) return causal ? dkdv_d<64, true>(prm, stream) : dkdv_d<64, false>(prm, stream);
  if (d == 128) return causal ? dkdv_d<128, true>(prm, stream) : dkdv_d<128, false>(prm, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                         const float* delta, void* dq, int BH, int N, int d, float scale, bool causal,
                         hipStream_t stream) {
  BwdParams prm = make_params(q, k, v, nullptr, lse, dout, delta, dq, nullptr, nullptr, BH, N, scale);
  if (d == 64) return causal ? dq_d<64, true>(prm, stream) : dq_d<64, false>(prm, stream);
  if (d == 128) return causal ? dq_d<128, true>(prm, stream) : dq_d<128, false>(prm, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
