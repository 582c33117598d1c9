// Fused fp32 attention forward for gfx950.
//
// The same tiled online-softmax algorithm as the bf16 kernel (52jiny.com
// FlashAttention explainer, "key ideas" parts 1-3; codechina.net
// CUDA/FlashAttention article, sections 4.1-4.2), with fp32 storage and the
// fp32 matrix instruction v_mfma_f32_32x32x2_f32, so no operand is rounded:
// P stays fp32 in the P V product. A wave owns 32 query rows and computes
// S^T = K Q^T; K/V tiles of 32 keys pass through LDS (rows padded by one float
// to spread banks). On longer rows two waves share each 32-row group, one on
// the even and one on the odd key tiles, and their partial (m, l, O) are merged
// by the online softmax's block merge (same pages, same sections). This path
// serves small or precision-sensitive problems; the bf16 kernel is the
// throughput path.
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

// KH = 1: 4 waves, one per 32-row query group, each over all key tiles. KH = 2: 8 waves, two per
// query group taking the even and the odd key tiles, merged at the end (two waves per SIMD hide
// each other's load and exp latencies on long rows; on a few tiles the merge costs more).
template <int D, bool CAUSAL, int KH>
__global__ __launch_bounds__(256 * KH) void fwd_fp32_kernel(FwdF32Params p) {
  constexpr int NQG = 4, BR = 32 * NQG, BC = 32, LD = D + 1, NT = 256 * KH;
  constexpr int NDB = D / 32;
  constexpr int TILE = BC * LD;                  // floats of one K (or V) tile in LDS
  constexpr int PER = KH * BC * D / NT;          // K (and V) elements each thread moves per stage
  constexpr int REC = 2 + 16 * NDB;              // merge record per lane: m, l, O accumulator
  static_assert(KH == 1 || NQG * 64 * REC <= 4 * KH * TILE, "merge records fit in the tile buffers");
  // [buffer][key half] K tiles, then the same for V; reused for the merge at the end
  __shared__ float lds[4 * KH * TILE];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lq = l & 31, hf = l >> 5;
  const int qg = w & 3, kh = KH == 1 ? 0 : w >> 2;  // query group (32 rows) and key half
  const int N = p.N;
  int head, qt;
  map_workgroup(blockIdx.x, p.n_qt, p.nh, CAUSAL ? Order::kLongestFirst : Order::kHeadMajor, true, head, qt);
  const size_t base = (size_t)head * N * D;
  const int q_w0 = qt * BR + 32 * qg;
  const int q = q_w0 + lq;

  // Q^T operand of the K=2 instruction: lane (q, hf) holds Q[q][2*kk + hf].
  float qreg[D / 2];
#pragma unroll
  for (int kk = 0; kk < D / 2; ++kk) qreg[kk] = (q < N) ? p.q[base + (size_t)q * D + 2 * kk + hf] : 0.f;

  int n_kv = (N + BC - 1) / BC;
  if (CAUSAL) n_kv = min(n_kv, (min(N, (qt + 1) * BR) - 1) / BC + 1);
  const int n_st = (n_kv + KH - 1) / KH;  // stage i holds tiles KH i .. KH i + KH - 1 (one per key half)

  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // The two tiles of a stage are double-buffered: stage i+1's global loads are issued into
  // registers before stage i is computed and stored to the other buffer after it, so their latency
  // hides behind the compute. The barrier at the top of an iteration makes the stores visible and
  // guarantees that every wave is done with the buffer the next stores overwrite.
  float kx[PER], vx[PER];
  auto fetch = [&](int i) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int x = tid + NT * e, h = x / (BC * D), y = x % (BC * D), r = y / D, c = y % D;
      const int key = (KH * i + h) * BC + r;
      kx[e] = key < N ? p.k[base + (size_t)key * D + c] : 0.f;
      vx[e] = key < N ? p.v[base + (size_t)key * D + c] : 0.f;
    }
  };
  auto deposit = [&](int b) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int x = tid + NT * e, h = x / (BC * D), y = x % (BC * D), r = y / D, c = y % D;
      lds[(KH * b + h) * TILE + r * LD + c] = kx[e];
      lds[(2 * KH + KH * b + h) * TILE + r * LD + c] = vx[e];
    }
  };
  if (n_st > 0) {
    fetch(0);
    deposit(0);
  }
  for (int i = 0; i < n_st; ++i) {
    __syncthreads();  // stage i is in buffer i % 2; every wave is done with buffer (i + 1) % 2
    if (i + 1 < n_st) fetch(i + 1);
    const int j = KH * i + kh, key0 = j * BC;
    const float* ks = lds + (KH * (i & 1) + kh) * TILE;
    const float* vs = lds + (2 * KH + KH * (i & 1) + kh) * TILE;
    // wave-uniform: this wave's tile exists and some of its keys precede this wave's last row
    if (j < n_kv && !(CAUSAL && key0 > q_w0 + 31)) {
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
    debug_stage_sync();
    if (i + 1 < n_st) deposit((i + 1) & 1);
    debug_stage_sync();
  }

  // KH = 2: merge the two key halves of each query group. The odd-tile wave publishes its running
  // max, sum and output accumulator; the even-tile wave rescales both to the common max (the
  // online softmax's block merge) and writes the result.
  if constexpr (KH == 2) {
    __syncthreads();  // every wave is done with the tile buffers
    float* rec = lds + (qg * 64 + l) * REC;
    if (kh == 1) {
      rec[0] = m_run;
      rec[1] = l_run;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) rec[2 + 16 * db + e] = acc_o[db][e];
    }
    __syncthreads();
    if (kh == 1) return;
    {
      const float m1 = rec[0], l1 = rec[1];
      const float m_new = fmaxf(m_run, m1);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float a0 = fast_exp2(m_run - m_use), a1 = fast_exp2(m1 - m_use);
      l_run = l_run * a0 + l1 * a1;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc_o[db][e] = acc_o[db][e] * a0 + rec[2 + 16 * db + e] * a1;
      m_run = m_new;
    }
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

// Small problems (few 128-row tiles in all): one workgroup per 32-row query group, so the work
// spreads over more compute units. Its KH waves take the key tiles j = kh, kh + KH, ... and merge
// their partial (m, l, O) at the end with the online softmax's block merge. Each tile is read by
// one wave only, so operands come straight from global memory into registers (no LDS staging);
// the next tile's loads are issued before the current tile is computed. The dot product runs over
// the columns in a permuted order that both Q and K use: k-step kk of lane half hf takes column
// (D / 2) hf + kk, so each lane reads whole 16-byte chunks of its row.
template <int D, bool CAUSAL, int KH>
__global__ __launch_bounds__(64 * KH) void fwd_fp32_split_kernel(FwdF32Params p) {
  constexpr int BC = 32, NDB = D / 32, NK = D / 2;
  constexpr int REC = 2 + 16 * NDB;  // merge record per lane: m, l, O accumulator
  __shared__ float rec[(KH > 1 ? KH - 1 : 1) * 64 * REC];
  const int l = threadIdx.x & 63, lq = l & 31, hf = l >> 5;
  const int kh = threadIdx.x >> 6;
  const int N = p.N;
  int head, qt;
  map_workgroup(blockIdx.x, p.n_qt, p.nh, CAUSAL ? Order::kLongestFirst : Order::kHeadMajor, true, head, qt);
  const size_t base = (size_t)head * N * D;
  const int q0 = qt * 32, q = q0 + lq;

  // Q^T operand: lane (q, hf) holds Q[q][NK hf + kk]; rows >= N read as zero.
  float qreg[NK];
#pragma unroll
  for (int c = 0; c < NK; c += 4) {
    const f32x4 t = q < N ? *reinterpret_cast<const f32x4*>(p.q + base + (size_t)q * D + NK * hf + c) : f32x4{};
#pragma unroll
    for (int e = 0; e < 4; ++e) qreg[c + e] = t[e];
  }
  int n_kv = (N + BC - 1) / BC;
  if (CAUSAL) n_kv = min(n_kv, (min(N, q0 + 32) - 1) / BC + 1);

  // Tile j's operands: K^T rows (lane (key lq, hf): K[key][NK hf + kk]) and V columns (lane (col lq, hf):
  // V[key(t, hf)][32 db + lq] for the 16 keys t of its half), keys >= N as zero.
  float kreg[NK], vreg[NDB][16];
  auto fetch = [&](int j) __attribute__((always_inline)) {
    const int key = j * BC + lq;
#pragma unroll
    for (int c = 0; c < NK; c += 4) {
      const f32x4 t = key < N ? *reinterpret_cast<const f32x4*>(p.k + base + (size_t)key * D + NK * hf + c) : f32x4{};
#pragma unroll
      for (int e = 0; e < 4; ++e) kreg[c + e] = t[e];
    }
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const int kv = j * BC + (t >> 2) * 8 + 4 * hf + (t & 3);
#pragma unroll
      for (int db = 0; db < NDB; ++db) vreg[db][t] = kv < N ? p.v[base + (size_t)kv * D + 32 * db + lq] : 0.f;
    }
  };

  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  if (kh < n_kv) fetch(kh);
  for (int j = kh; j < n_kv; j += KH) {
    f32x16 s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) s = mfma_f32_32x32x2(kreg[kk], qreg[kk], s);
    float vt[NDB][16];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int t = 0; t < 16; ++t) vt[db][t] = vreg[db][t];
    if (j + KH < n_kv) fetch(j + KH);  // next tile's loads overlap this tile's softmax and P V
    const int key0 = j * BC;
    const bool need_mask = (key0 + BC > N) || (CAUSAL && key0 + BC - 1 > q0);
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
#pragma unroll
      for (int t = 0; t < 16; ++t) acc_o[db] = mfma_f32_32x32x2(vt[db][t], s[t], acc_o[db]);
    }
  }

  // Block merge of the KH partials of each row: waves 1 .. KH-1 publish (m, l, O accumulator);
  // wave 0 rescales all of them to the common maximum and writes the result.
  if constexpr (KH > 1) {
    if (kh > 0) {
      float* r = rec + ((kh - 1) * 64 + l) * REC;
      r[0] = m_run;
      r[1] = l_run;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) r[2 + 16 * db + e] = acc_o[db][e];
    }
    __syncthreads();
    if (kh > 0) return;
    for (int w = 1; w < KH; ++w) {
      const float* r = rec + ((w - 1) * 64 + l) * REC;
      const float m1 = r[0], l1 = r[1];
      const float m_new = fmaxf(m_run, m1);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float a0 = fast_exp2(m_run - m_use), a1 = fast_exp2(m1 - m_use);
      l_run = l_run * a0 + l1 * a1;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc_o[db][e] = acc_o[db][e] * a0 + r[2 + 16 * db + e] * a1;
      m_run = m_new;
    }
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

// Problems with fewer 128-row tiles in all than this run as 32-row workgroups (the split kernel).
constexpr int kSmallTiles = 64;

template <int D, bool CAUSAL>
static hipError_t launch_cfg(const FwdF32Params& prm, hipStream_t stream) {
  const int n_tiles128 = prm.n_qt * prm.nh;
  if (prm.N <= 512 && n_tiles128 < kSmallTiles) {
    FwdF32Params sp = prm;
    sp.n_qt = (prm.N + 31) / 32;
    const int n_kv = (prm.N + 31) / 32;
    const dim3 grid(sp.n_qt * sp.nh);
    if (n_kv >= 4)
      hipLaunchKernelGGL((fwd_fp32_split_kernel<D, CAUSAL, 4>), grid, dim3(256), 0, stream, sp);
    else if (n_kv >= 2)
      hipLaunchKernelGGL((fwd_fp32_split_kernel<D, CAUSAL, 2>), grid, dim3(128), 0, stream, sp);
    else
      hipLaunchKernelGGL((fwd_fp32_split_kernel<D, CAUSAL, 1>), grid, dim3(64), 0, stream, sp);
    return hipGetLastError();
  }
  // two key halves pay from about eight key tiles per row (measured: N = 128 is 10% faster with
  // one, N = 1000 16% faster with two)
  if (prm.N > 256)
    hipLaunchKernelGGL((fwd_fp32_kernel<D, CAUSAL, 2>), dim3(prm.n_qt * prm.nh), dim3(512), 0, stream, prm);
  else
    hipLaunchKernelGGL((fwd_fp32_kernel<D, CAUSAL, 1>), dim3(prm.n_qt * prm.nh), dim3(256), 0, stream, prm);
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
