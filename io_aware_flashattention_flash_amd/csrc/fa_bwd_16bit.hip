// Recompute-based attention backward for gfx950 (16-bit storage: bf16 or fp16; fp32 math).
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
// Kernels (no atomics, deterministic). The full backward launches 3 then 2 on one stream; 1 is a
// standalone stage computing only delta.
//  1. delta kernel: one fp32 value per query row.
//  2. dK/dV kernel (key-outer): a workgroup owns 32*NW keys, a wave owns 32 of
//     them and keeps K^T / V^T operands and the dK^T / dV^T accumulators in
//     registers while Q, dO, LSE and delta tiles stream through LDS. It uses
//     the untransposed score block S = Q K^T, so a lane holds one key and the
//     registers run over queries: P and dS, rounded to the 16-bit type, are directly the
//     B operands of dV^T += dO^T P and dK^T += Q^T dS, whose A operands
//     (dO^T, Q^T) come from the LDS transpose read. In small causal launches the longest key
//     tiles run as two workgroups of 64 keys each (split_rank).
//  3. dQ kernel (query-outer): the forward's layout (S^T = K Q^T, a lane holds
//     one query); computes its rows' delta from O and dO (and publishes it for
//     kernel 2), recomputes P and dP, forms dS^T and accumulates
//     dQ^T += K^T dS^T with K^T from the LDS transpose read. In small causal launches a
//     workgroup takes 64 rows and its two wave pairs take the even and the odd key tiles.
#include <algorithm>
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <typename E>
struct BwdParams {
  const E* q;
  const E* k;
  const E* v;
  const E* o;
  const E* dout;
  const float* lse;
  float* delta;
  E* dq;
  E* dk;
  E* dv;
  int N;
  int nh;
  int n_tiles;
  int n_units;  // workgroups per head (dQ: n_tiles, or (n_tiles + 1) / 2 when causal tiles are paired)
  // Split dK/dV launches (small dense causal ones): the first n_split key tiles of each head run as
  // two half-size workgroups; n_long orders a head's workgroups (see split_rank).
  int n_split;
  int n_long;
  float c;      // scale * log2(e)
  float scale;
  // Masked launches only: per-sequence valid rows (sequence = head / heads; clamped to [0, N]) and
  // the block-sparse map [head][n_mb][n_mb] (one byte per 128 x 128 block; zero = skipped), or null.
  const int* seqlens;
  const uint8_t* block_mask;
  int heads;
  int n_mb;
  // Dropout launches only: Philox key, keep threshold T and 256 / T.
  uint32_t seed_lo;
  uint32_t seed_hi;
  int drop_thr;
  float drop_scale;
};

// Valid rows of this head's sequence.
template <bool MASKED, typename P>
__device__ __forceinline__ int valid_rows(const P& p, int head) {
  return (MASKED && p.seqlens) ? min(max(p.seqlens[head / p.heads], 0), p.N) : p.N;
}

// Compacts the enabled entries among map[0], map[stride], ..., map[(n - 1) * stride] (n <= the list
// size) into `list` in increasing order and returns their count (wave-uniform). Every wave counts;
// wave 0 writes. The caller synchronises the workgroup before reading the list.
__device__ __forceinline__ int build_block_list(const uint8_t* map, size_t stride, int n, short* list, int wave,
                                                int lane) {
  int cnt = 0;
  for (int b0 = 0; b0 < n; b0 += 64) {
    const int b = b0 + lane;
    const bool on = b < n && map[(size_t)b * stride] != 0;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(on);
    if (wave == 0 && on)
      list[cnt + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0))] = b;
    cnt += __builtin_popcountll(bal);
  }
  return cnt;
}

// ---------------------------------------------------------------------------------------------
// 1. delta = rowsum(dO * O)
// ---------------------------------------------------------------------------------------------
template <int X>
constexpr int pow2_at_least() { int t = 1; while (t < X) t *= 2; return t; }

template <typename E, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdParams<E> p) {
  using e16x8 = typename Half16<E>::x8;
  constexpr int TPR = pow2_at_least<D / 8>();  // threads per row, one 16-byte chunk each (idle beyond D)
  constexpr int RPI = 256 / TPR;               // rows per block per step
  constexpr int STEPS = 4;                     // rows per thread (independent loads in flight)
  const int tid = threadIdx.x;
  const long rows = (long)p.nh * p.N;
  const long row0 = (long)blockIdx.x * RPI * STEPS + tid / TPR;
  const int c = tid % TPR;
  u32x4 a[STEPS], b[STEPS];
#pragma unroll
  for (int i = 0; i < STEPS; ++i) {
    const long row = row0 + (long)i * RPI;
    a[i] = u32x4{0, 0, 0, 0};
    b[i] = u32x4{0, 0, 0, 0};
    if (row < rows && 8 * c < D) {
      a[i] = ld_global16(p.o + row * D + 8 * c);
      b[i] = ld_global16(p.dout + row * D + 8 * c);
    }
  }
#pragma unroll
  for (int i = 0; i < STEPS; ++i) {
    const e16x8 av = __builtin_bit_cast(e16x8, a[i]), bv = __builtin_bit_cast(e16x8, b[i]);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)av[e] * (float)bv[e];
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    const long row = row0 + (long)i * RPI;
    if (row < rows && c == 0) p.delta[row] = acc;
  }
}

// ---------------------------------------------------------------------------------------------
// 2. dK, dV (key-outer)
// ---------------------------------------------------------------------------------------------
// MASKED: padding rows (>= the sequence's length) and, with a block-sparse map, only the query
// blocks enabled in this key tile's map column; keys no query sees get dK = dV = 0.
// DROPOUT (with MASKED): the forward's keep mask is regenerated; the weights of dV are the kept
// probabilities scaled by 256 / T, and the gradient reaching P is dP scaled by the same kept factor.
// This kernel's lanes hold keys, not queries, so each wave draws the Philox words of its 32 x 32
// block in the forward's layout (one call per lane) and transposes the bytes through LDS.
//
// PART: 0 computes dK and dV; 1 only dV (needs K, not V); 2 only dK. d = 256 runs parts 1 and 2 as
// two launches: K and V operands (128 registers per lane) plus both accumulators (256) do not fit
// one wave's 512 registers beside the temporaries, and recomputing S once more is cheaper than
// spilling. Non-causal d = 128 also runs the two parts, each at two waves per SIMD (measured
// faster than one wave per SIMD for the whole; causal d = 128 is faster whole).
// Waves per SIMD: 2 where the registers fit 256 per lane (d <= 64, d = 96, the parts at d = 128),
// else 1. The dense causal d = 64 kernel fits 168 registers and runs 3 (measured 2.4% faster; the
// non-causal one was 2.4% slower at 3, and the masked ones spill there).
// Split launches. Key tile kt of a causal head sees n_qt - 2 kt query tiles of 64 rows, so when a
// launch's workgroups all fit on the chip at once, the launch lasts as long as key tile 0. Its
// first n_split key tiles then run as two workgroups each, one per 64-key half (hs = 0, 1): wave w
// takes the 32 keys of group w & 1 against query block w >> 1 of every query tile, and the two waves
// of a key group add their partial sums through LDS at the end. A head's workgroups run longest
// first: key tiles n_split .. n_long - 1 (longer than any half), the halves, then the rest.
__device__ __forceinline__ void split_rank(int r, int n_split, int n_long, int& kt, int& hs) {
  if (r < n_long - n_split) {
    kt = n_split + r;
    hs = -1;
  } else if (r < n_long + n_split) {
    const int j = r - (n_long - n_split);
    kt = j >> 1;
    hs = j & 1;
  } else {
    kt = r - n_split;
    hs = -1;
  }
}

template <int D, int PART, bool CAUSAL, bool MASKED>
constexpr int dkdv_waves_per_simd() {
  return (D > 128 || (D == 128 && PART == 0)) ? 1 : ((D == 64 && CAUSAL && !MASKED) ? 3 : 2);
}

//
// QSTREAM (small causal launches whose 64-key workgroups all fit at once): a workgroup takes 64
// keys, and its two wave pairs take the even and the odd query tiles: wave w runs the 32 keys of
// group w & 1 over query tiles w >> 1, (w >> 1) + 2, ..., each pair with its own double buffer,
// and the two waves of a key group exchange their dK and dV partial sums at the end. (Its tile
// buffers take 64 KB at d = 64, 96-128 KB at d = 96, 128: two or one workgroups per CU.)
template <typename E, int D, int NW, int BQ, bool CAUSAL, bool MASKED, bool DROPOUT, int PART, bool QSPLIT = false,
          bool QSTREAM = false>
__global__ __launch_bounds__(NW * 64, (QSTREAM ? (D <= 64 ? 2 : 1) : dkdv_waves_per_simd<D, PART, CAUSAL, MASKED>())) void bwd_dkdv_kernel(BwdParams<E> p) {
  constexpr bool WANT_DV = PART != 2, WANT_DK = PART != 1;
  using H = Half16<E>;
  using e16x8 = typename H::x8;
  constexpr int BKV = 32 * NW;
  constexpr int NCH = D / 8;
  constexpr int TILE_BYTES = BQ * D * 2;
  constexpr int NLD = BQ * NCH / (64 * NW);  // LDS-DMA instructions per wave per tensor per tile
  static_assert(NLD * 64 * NW == BQ * NCH, "tile must split evenly over the workgroup's waves");
  static_assert(BQ == 64, "wave 0 stages one LSE / delta row per lane");
  static_assert(BKV % BQ == 0, "key tiles start on query-tile boundaries");
  static_assert(!MASKED || BKV == kMaskBlock, "a key tile is one column of the block map");
  constexpr int NKK = D / 16, NDB = D / 32, NQB = BQ / 32;
  using T = SwizzledTile<D>;
  // dS = P * (dP - delta): without dropout, delta is folded into the dP product's initial
  // accumulator, one VALU operation less per score (not in the one-wave d = 128 kernel, whose
  // registers are full: measured slower there).
  constexpr bool FOLD_DELTA = !DROPOUT && !(D == 128 && PART == 0);
  static_assert(!QSPLIT || (CAUSAL && !MASKED && PART == 0 && NW == 4 && BQ == 64),
                "split launches: dense causal dK and dV, 2 key groups x 2 query blocks of 32");
  static_assert(!QSTREAM || (!QSPLIT && CAUSAL && !MASKED && PART == 0 && NW == 4 && BQ == 64),
                "stream launches: dense causal dK and dV");
  constexpr int KW = QSTREAM ? 64 : BKV;      // keys per workgroup
  constexpr int DW = QSTREAM ? 2 : NW;        // waves that load one tile
  constexpr int NLDW = BQ * NCH / (64 * DW);  // their DMA instructions per tensor and tile
  static_assert(NLDW * 64 * DW == BQ * NCH, "a tile splits evenly over its loading waves");

  __shared__ __attribute__((aligned(16))) char sq0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char so0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char sq1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char so1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) float sr0[2 * BQ];  // [lse * log2(e) | delta] of the tile's rows
  __shared__ __attribute__((aligned(16))) float sr1[2 * BQ];
  // the odd-tile pair's buffers (stream launches)
  __shared__ __attribute__((aligned(16))) char sqb0[QSTREAM ? TILE_BYTES : 16];
  __shared__ __attribute__((aligned(16))) char sob0[QSTREAM ? TILE_BYTES : 16];
  __shared__ __attribute__((aligned(16))) char sqb1[QSTREAM ? TILE_BYTES : 16];
  __shared__ __attribute__((aligned(16))) char sob1[QSTREAM ? TILE_BYTES : 16];
  __shared__ __attribute__((aligned(16))) float srb0[QSTREAM ? 2 * BQ : 4];
  __shared__ __attribute__((aligned(16))) float srb1[QSTREAM ? 2 * BQ : 4];
  __shared__ short blist[MASKED ? kMaxMaskBlocks : 1];  // enabled query blocks of this key tile
  __shared__ __attribute__((aligned(16))) uint8_t sdrop[DROPOUT ? NW * 1024 : 4];  // per wave: bytes [key][query]

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, lq = l & 31, hf = l >> 5;
  const int N = p.N;
  int head, kt, hs = -1;
  // causal: key tile 0 has the most work; with sequence lengths, padding key tiles run last
  if constexpr (QSTREAM) {
    map_workgroup(blockIdx.x, p.n_units, p.nh, Order::kLongestFirst, false, head, kt);  // 64-key tiles
  } else if constexpr (QSPLIT) {
    int r;
    map_workgroup(blockIdx.x, p.n_tiles + p.n_split, p.nh, Order::kLongestFirst, false, head, r);
    split_rank(r, p.n_split, p.n_long, kt, hs);
  } else if (!(MASKED && p.seqlens &&
               map_workgroup_varlen(blockIdx.x, p.n_tiles, p.nh, p.heads, p.seqlens, p.N, BKV, CAUSAL, false, head, kt))) {
    map_workgroup(blockIdx.x, p.n_tiles, p.nh, CAUSAL ? Order::kLongestFirst : Order::kHeadMajor, false, head, kt);
  }
  const bool split = QSPLIT && hs >= 0;                  // a 64-key half (wave-uniform)
  const int kspan0 = kt * KW + (split ? 64 * hs : 0);   // the workgroup's first key
  const int stream = QSTREAM ? (w >> 1) : 0;  // stream launches: even (0) or odd (1) query tiles
  const int wl = QSTREAM ? (w & 1) : w;       // the wave's index among the waves loading its tiles
  const size_t base = (size_t)head * N * D;
  const size_t rbase = (size_t)head * N;
  const int head_bytes = N * D * 2;
  const int key_w0 = kspan0 + 32 * (split ? (w & 1) : wl);
  const int key = key_w0 + lq;
  const int Lb = valid_rows<MASKED>(p, head);  // rows >= Lb of every input read as zero

  // K^T and V^T operands (B side of S = Q K^T and dP = dO V^T): lane (key, hf); keys >= Lb read 0.
  e16x8 kreg[NKK], vreg[NKK];
  {
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + base, Lb * (D * 2));
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + base, Lb * (D * 2));
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int off = key * (D * 2) + (16 * kk + 8 * hf) * 2;
      kreg[kk] = __builtin_bit_cast(e16x8, buf_load16(rk, off));
      if (WANT_DK) vreg[kk] = __builtin_bit_cast(e16x8, buf_load16(rv, off));
    }
  }

  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  const int n_qt = (Lb + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? kspan0 / BQ : 0;
  // Loop positions u = 0 .. n_t - 1 map to query tiles tile(u): qt0 + u, or with a block map the
  // tile pairs of the enabled 128-row blocks (causal: from the diagonal block on).
  constexpr int TPB = kMaskBlock / BQ;
  int n_t = n_qt - qt0;
  if (MASKED && kt * BKV >= Lb) n_t = 0;  // padding keys only
  const bool sparse = MASKED && p.block_mask != nullptr;
  int n_diag = CAUSAL ? BKV / BQ : 0;     // leading positions that meet the diagonal
  if (sparse && n_t > 0) {
    const int cnt = build_block_list(p.block_mask + (size_t)head * p.n_mb * p.n_mb + (size_t)(CAUSAL ? kt : 0) * p.n_mb + kt,
                                     p.n_mb, (n_qt + TPB - 1) / TPB - (CAUSAL ? kt : 0), blist, w, l);
    __syncthreads();
    n_t = TPB * cnt;
    // list entries are relative to the first block scanned (the diagonal one when causal)
    if (CAUSAL && (cnt == 0 || __builtin_amdgcn_readfirstlane(blist[0]) != 0)) n_diag = 0;
  }
  if (QSTREAM) {
    // this wave pair's query tiles qt0 + stream, qt0 + stream + 2, ...; both pairs run as many
    // positions as the even tiles need (the odd pair's last may be past the head: zero rows).
    // Only the first query tile meets the 64-key diagonal, the even pair's first position.
    n_t = (n_t + 1) / 2;
    n_diag = stream == 0 ? 2 : 0;
  }
  auto tile = [&](int u) __attribute__((always_inline)) -> int {
    if (QSTREAM) return qt0 + 2 * u + stream;
    if (!sparse) return qt0 + u;
    return qt0 + TPB * __builtin_amdgcn_readfirstlane(blist[u / TPB]) + u % TPB;
  };

  int goff[NLDW];
#pragma unroll
  for (int i = 0; i < NLDW; ++i) {
    const int pos = (wl + DW * i) * 64 + l;
    const int row = pos / NCH, pc = pos % NCH;
    goff[i] = row * (D * 2) + ((pc ^ T::swz(row)) * 16);
  }
  const __amdgpu_buffer_rsrc_t rlse = make_rsrc(p.lse + rbase, Lb * 4);
  const __amdgpu_buffer_rsrc_t rdel = make_rsrc(p.delta + rbase, Lb * 4);
  float st_l = 0.f, st_d = 0.f;  // wave 0: this tile's row statistics, staged in registers
  auto dma = [&](int i, char* qb, char* ob) __attribute__((always_inline)) {
    // (wave-uniform by construction; readfirstlane keeps the descriptors in scalar registers)
    const int row0 = i * BQ;
    const int bytes = __builtin_amdgcn_readfirstlane(max(0, min(BQ, Lb - row0)) * (D * 2));
    const int first = __builtin_amdgcn_readfirstlane(min(row0, Lb));
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + base + (size_t)first * D, bytes);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.dout + base + (size_t)first * D, bytes);
#pragma unroll
    for (int t = 0; t < NLDW; ++t) {
      buf_load16_to_lds(rq, qb + (wl + DW * t) * 1024, goff[t]);
      buf_load16_to_lds(ro, ob + (wl + DW * t) * 1024, goff[t]);
    }
    if (wl == 0) {
      st_l = buf_load4f(rlse, (row0 + l) * 4) * kLog2e;
      st_d = buf_load4f(rdel, (row0 + l) * 4);
    }
  };
  auto stage_rows = [&](float* sr) __attribute__((always_inline)) {
    if (wl == 0) {
      sr[l] = st_l;
      sr[BQ + l] = FOLD_DELTA ? -st_d : st_d;
    }
  };

  const int g16 = l >> 4, j16 = l & 15;
  const int tr_row_lane = 4 * hf + (j16 >> 2);
  const int tr_col_lane = 16 * (g16 & 1) + 4 * (j16 & 3);
  const float c = p.c;

  // One query tile. DIAG (causal only): the tile meets this key tile's diagonal, so blocks
  // entirely before a wave's keys are skipped and the rest are masked. Query rows >= N need no
  // mask here: their Q and dO rows arrive as zeros, so they add nothing to dK or dV.
  auto compute = [&](auto diag_tag, int i, const char* qbuf, const char* obuf, const float* sr) __attribute__((always_inline)) {
    constexpr bool DIAG = decltype(diag_tag)::value;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      if (split && qb != (w >> 1)) continue;  // the other wave of this key group takes the block
      const int q0 = i * BQ + 32 * qb;
      if (DIAG && q0 + 31 < key_w0) continue;  // wave-uniform: every query precedes every key
      // FOLD_DELTA: the dP product starts from -delta of each register's query, so it yields
      // dP - delta directly (the staged row statistics hold -delta then).
      f32x16 s = f32x16{}, dp = f32x16{};
      if constexpr (FOLD_DELTA) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 nd4 = *reinterpret_cast<const f32x4*>(sr + BQ + 32 * qb + 8 * g + 4 * hf);
#pragma unroll
          for (int e = 0; e < 4; ++e) dp[4 * g + e] = nd4[e];
        }
      }
      if constexpr (D >= 128) {
        // one wave per SIMD (or the d = 128 parts): the next k-step's Q / dO fragments are read one
        // step ahead, as no other wave hides the LDS latency in front of each product
        e16x8 qn = lds_read16<E>(qbuf, T::chunk_off(32 * qb + lq, hf)), on{};  // on: unused in the dV-only part
        if (WANT_DK) on = lds_read16<E>(obuf, T::chunk_off(32 * qb + lq, hf));
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const e16x8 qc = qn, oc = on;
          if (kk + 1 < NKK) {
            const int off = T::chunk_off(32 * qb + lq, 2 * (kk + 1) + hf);
            qn = lds_read16<E>(qbuf, off);
            if (WANT_DK) on = lds_read16<E>(obuf, off);
          }
          __builtin_amdgcn_sched_barrier(0);
          s = H::mfma(qc, kreg[kk], s);
          if (WANT_DK) dp = H::mfma(oc, vreg[kk], dp);
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const int off = T::chunk_off(32 * qb + lq, 2 * kk + hf);
          s = H::mfma(lds_read16<E>(qbuf, off), kreg[kk], s);
          if (WANT_DK) dp = H::mfma(lds_read16<E>(obuf, off), vreg[kk], dp);
        }
      }
      // Register r holds query q0 + 8*(r/4) + 4*hf + r%4 against this lane's key.
      const int kmin = key - q0 - 4 * hf;  // (DIAG) query offsets below this are masked
      uint32_t kwt[4];  // dropout: byte e of kwt[g] belongs to register 4g + e
      if constexpr (DROPOUT) {
        // Lane (q, h) draws the words of query q0 + q, half h of the wave's 32-key block, and
        // stores byte (g, e) at [key 8g + 4h + e][query q]; lane (key, hf) then reads its key's row.
        uint8_t* mt = sdrop + w * 1024;
        uint32_t wd[4];
        dropout_words(q0 + lq, key_w0 >> 5, head, hf, p.seed_lo, p.seed_hi, wd);
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int e = 0; e < 4; ++e) mt[(8 * g + 4 * hf + e) * 32 + lq] = (uint8_t)(wd[g] >> (8 * e));
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes have landed
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int g = 0; g < 4; ++g) kwt[g] = *reinterpret_cast<const uint32_t*>(mt + lq * 32 + 8 * g + 4 * hf);
        __builtin_amdgcn_s_waitcnt(0xc07f);  // reads done before the next block's writes
        __builtin_amdgcn_wave_barrier();
      }
      e16x8 pb[2], dsb[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 lse4 = *reinterpret_cast<const f32x4*>(sr + 32 * qb + 8 * g + 4 * hf);
        const f32x4 dl4 = FOLD_DELTA ? f32x4{} : *reinterpret_cast<const f32x4*>(sr + BQ + 32 * qb + 8 * g + 4 * hf);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float pr = fast_exp2(fmaf(s[r], c, -lse4[e]));
          if constexpr (DIAG) pr = (8 * g + e < kmin) ? 0.f : pr;
          float dpr = dp[r];
          if constexpr (DROPOUT) {
            const bool kept = dropout_keep(kwt[g], e, p.drop_thr);
            pb[r >> 3][r & 7] = (E)(kept ? pr * p.drop_scale : 0.f);
            dpr = kept ? dpr * p.drop_scale : 0.f;
          } else {
            pb[r >> 3][r & 7] = (E)pr;
          }
          dsb[r >> 3][r & 7] = (E)(FOLD_DELTA ? pr * dpr : pr * (dpr - dl4[e]));
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS; k-step ks covers queries
      // 32qb + 16ks + {4hf..4hf+3, 8+4hf..8+4hf+3} (registers 8ks..8ks+7).
      if constexpr (D >= 128) {
        // the transposed dO / Q fragments of step (db, ks) + 1 read before step (db, ks)'s products
        auto tr_off = [&](int st, int& o0, int& o1) __attribute__((always_inline)) {
          const int db = st >> 1, ks = st & 1;
          const int r0 = 32 * qb + 16 * ks + tr_row_lane, col = 32 * db + tr_col_lane;
          o0 = T::elem_off(r0, col);
          o1 = T::elem_off(r0 + 8, col);
        };
        e16x8 vn{}, kn{};  // each unused in the part that does not compute it
        {
          int o0, o1;
          tr_off(0, o0, o1);
          if (WANT_DV) vn = cat4<E>(lds_read_tr16<E>(obuf, o0), lds_read_tr16<E>(obuf, o1));
          if (WANT_DK) kn = cat4<E>(lds_read_tr16<E>(qbuf, o0), lds_read_tr16<E>(qbuf, o1));
        }
#pragma unroll
        for (int st = 0; st < 2 * NDB; ++st) {
          const e16x8 vc = vn, kc = kn;
          if (st + 1 < 2 * NDB) {
            int o0, o1;
            tr_off(st + 1, o0, o1);
            if (WANT_DV) vn = cat4<E>(lds_read_tr16<E>(obuf, o0), lds_read_tr16<E>(obuf, o1));
            if (WANT_DK) kn = cat4<E>(lds_read_tr16<E>(qbuf, o0), lds_read_tr16<E>(qbuf, o1));
          }
          __builtin_amdgcn_sched_barrier(0);
          const int db = st >> 1, ks = st & 1;
          if (WANT_DV) dv[db] = H::mfma(vc, pb[ks], dv[db]);
          if (WANT_DK) dk[db] = H::mfma(kc, dsb[ks], dk[db]);
        }
      } else {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int col = 32 * db + tr_col_lane;
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const int r0 = 32 * qb + 16 * ks + tr_row_lane;
            const int o0 = T::elem_off(r0, col), o1 = T::elem_off(r0 + 8, col);
            if (WANT_DV)
              dv[db] = H::mfma(cat4<E>(lds_read_tr16<E>(obuf, o0), lds_read_tr16<E>(obuf, o1)), pb[ks], dv[db]);
            if (WANT_DK)
              dk[db] = H::mfma(cat4<E>(lds_read_tr16<E>(qbuf, o0), lds_read_tr16<E>(qbuf, o1)), dsb[ks], dk[db]);
          }
        }
      }
    }
  };
  // Ping-pong over two LDS buffers: query tile i+1 streams in while tile i is computed. A causal
  // key tile's first BKV / BQ query tiles meet its diagonal; they run first, in their own loop, so
  // the steady-state loop body holds only the unmasked path.
  static_assert((BKV / BQ) % 2 == 0, "the diagonal section must keep the buffer parity");
  auto pair = [&](auto diag_tag, int u) __attribute__((always_inline)) {
    if (u + 1 < n_t) dma(tile(u + 1), sq1, so1);
    debug_stage_sync();
    compute(diag_tag, tile(u), sq0, so0, sr0);
    debug_stage_sync();
    wait_vmem();
    stage_rows(sr1);
    __syncthreads();
    if (u + 1 < n_t) {
      if (u + 2 < n_t) dma(tile(u + 2), sq0, so0);
      debug_stage_sync();
      compute(diag_tag, tile(u + 1), sq1, so1, sr1);
      debug_stage_sync();
      wait_vmem();
      stage_rows(sr0);
      __syncthreads();
    }
  };
  if constexpr (QSTREAM) {
    // Each wave pair runs the tile loop on its own buffers; every loop position ends with one
    // workgroup barrier and both pairs run n_t positions, so the barriers match. (The plain
    // launches keep the loop below written out on their buffers.)
    auto tiles = [&](char* Q0, char* O0, char* Q1, char* O1, float* R0, float* R1) __attribute__((always_inline)) {
      auto pair_b = [&](auto diag_tag, int u) __attribute__((always_inline)) {
        if (u + 1 < n_t) dma(tile(u + 1), Q1, O1);
        debug_stage_sync();
        compute(diag_tag, tile(u), Q0, O0, R0);
        debug_stage_sync();
        wait_vmem();
        stage_rows(R1);
        __syncthreads();
        if (u + 1 < n_t) {
          if (u + 2 < n_t) dma(tile(u + 2), Q0, O0);
          debug_stage_sync();
          compute(diag_tag, tile(u + 1), Q1, O1, R1);
          debug_stage_sync();
          wait_vmem();
          stage_rows(R0);
          __syncthreads();
        }
      };
      dma(tile(0), Q0, O0);
      stage_rows(R0);
      wait_vmem();
      __syncthreads();
      int u = 0;
#pragma unroll 1
      for (; u < n_diag && u < n_t; u += 2) pair_b(std::true_type{}, u);
#pragma unroll 1
      for (; u < n_t; u += 2) pair_b(std::false_type{}, u);
    };
    if (stream == 1) tiles(sqb0, sob0, sqb1, sob1, srb0, srb1);
    else tiles(sq0, so0, sq1, so1, sr0, sr1);
  } else if (n_t > 0) {
    dma(tile(0), sq0, so0);
    stage_rows(sr0);
    wait_vmem();
    __syncthreads();
    int u = 0;
#pragma unroll 1
    for (; u < n_diag && u < n_t; u += 2) pair(std::true_type{}, u);
#pragma unroll 1
    for (; u < n_t; u += 2) pair(std::false_type{}, u);
  }
  if (MASKED && key >= Lb) {  // padding keys (their K, V read as zero but queries still saw them)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      dk[db] = f32x16{};
      dv[db] = f32x16{};
    }
  }

  // dK = scale * dK^T^T and dV, written as whole rows through this wave's idle tile buffer.
  __syncthreads();  // every wave is done reading the last Q / dO tile
  char* stage = w == 0 ? sq0 : (w == 1 ? so0 : (w == 2 ? sq1 : so1));
  if constexpr (QSTREAM) {
    // Waves g and g + 2 hold key group g's partial sums over the even and the odd query tiles.
    // Wave g + 2 hands its dK partial to wave g, wave g hands its dV partial to wave g + 2 (fp32,
    // one of the odd pair's idle tile buffers each: 128 * D bytes); then wave g writes dK and wave
    // g + 2 writes dV, staging in buffers the exchange does not use.
    static_assert(NDB * 4 * 64 * 16 == TILE_BYTES, "a partial fills one tile buffer");
    f32x4* xk = reinterpret_cast<f32x4*>(wl ? sqb1 : sqb0);
    f32x4* xv = reinterpret_cast<f32x4*>(wl ? sob1 : sob0);
    auto give = [&](const f32x16(&acc)[NDB], f32x4* out4) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          out4[(4 * db + q4) * 64 + l] = f32x4{acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2], acc[db][4 * q4 + 3]};
    };
    auto take = [&](f32x16(&acc)[NDB], const f32x4* in4) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 t = in4[(4 * db + q4) * 64 + l];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[db][4 * q4 + e] += t[e];
        }
    };
    if (stream == 1) give(dk, xk);
    else give(dv, xv);
    __syncthreads();
    if (stream == 0) {
      take(dk, xk);
      store_rows_via_lds<E, D, TILE_BYTES>(stage, dk, p.scale, make_rsrc(p.dk + base, head_bytes), key_w0, l);
    } else {
      take(dv, xv);
      store_rows_via_lds<E, D, TILE_BYTES>(stage, dv, 1.0f, make_rsrc(p.dv + base, head_bytes), key_w0, l);
    }
    return;
  }
  if (split) {
    // Waves g and g + 2 hold key group g's partial sums over query blocks 0 and 1. Wave g + 2 hands
    // its dK partial to wave g, wave g hands its dV partial to wave g + 2 (fp32, through the tile
    // buffers: each partial is 128 * D bytes, one tile buffer); then wave g writes dK and wave
    // g + 2 writes dV.
    const int g = w & 1;
    const bool fin_dk = w < 2;
    char* xbuf_dk = g ? sq1 : sq0;
    char* xbuf_dv = g ? so1 : so0;
    static_assert(NDB * 4 * 64 * 16 == TILE_BYTES, "a partial fills one tile buffer");
    auto give = [&](const f32x16(&acc)[NDB], char* buf) __attribute__((always_inline)) {
      f32x4* out4 = reinterpret_cast<f32x4*>(buf);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          out4[(4 * db + q4) * 64 + l] = f32x4{acc[db][4 * q4], acc[db][4 * q4 + 1], acc[db][4 * q4 + 2], acc[db][4 * q4 + 3]};
    };
    auto take = [&](f32x16(&acc)[NDB], const char* buf) __attribute__((always_inline)) {
      const f32x4* in4 = reinterpret_cast<const f32x4*>(buf);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 t = in4[(4 * db + q4) * 64 + l];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[db][4 * q4 + e] += t[e];
        }
    };
    if (fin_dk) give(dv, xbuf_dv);
    else give(dk, xbuf_dk);
    __syncthreads();
    if (fin_dk) take(dk, xbuf_dk);
    else take(dv, xbuf_dv);
    __syncthreads();  // every handed-over partial is read before the staging areas are reused
    if (fin_dk) store_rows_via_lds<E, D, TILE_BYTES>(stage, dk, p.scale, make_rsrc(p.dk + base, head_bytes), key_w0, l);
    else store_rows_via_lds<E, D, TILE_BYTES>(stage, dv, 1.0f, make_rsrc(p.dv + base, head_bytes), key_w0, l);
    return;
  }
  if (WANT_DK) store_rows_via_lds<E, D, TILE_BYTES>(stage, dk, p.scale, make_rsrc(p.dk + base, head_bytes), key_w0, l);
  if (WANT_DV) store_rows_via_lds<E, D, TILE_BYTES>(stage, dv, 1.0f, make_rsrc(p.dv + base, head_bytes), key_w0, l);
}

// ---------------------------------------------------------------------------------------------
// 3. dQ (query-outer)
// ---------------------------------------------------------------------------------------------
// MASKED: padding rows and, with a block-sparse map, only the key blocks enabled in this query
// tile's map row; every tile takes the masked path.
// DROPOUT (with MASKED): dS = P * (dP * keep * 256 / T - delta), the keep mask regenerated in
// the forward's layout.
// (Split launches at d = 96 hold 96 KB of tile buffers: one workgroup, one wave per SIMD.)
template <typename E, int D, int BC, int NW, bool CAUSAL, bool MASKED, bool DROPOUT, bool QSPLIT = false>
__global__ __launch_bounds__(NW * 64, (D > 128 || (QSPLIT && D == 96)) ? 1 : 2) void bwd_dq_kernel(BwdParams<E> p) {
  using H = Half16<E>;
  using e16x8 = typename H::x8;
  using e16x4 = typename H::x4;
  constexpr int BR = 32 * NW;
  constexpr int NCH = D / 8;
  constexpr int TILE_BYTES = BC * D * 2;
  constexpr int NLD = BC * NCH / (64 * NW);
  static_assert(NLD * 64 * NW == BC * NCH, "tile must split evenly over the workgroup's waves");
  constexpr int NKB = BC / 32, NDB = D / 32, NKK = D / 16, NKS = BC / 16;
  using T = SwizzledTile<D>;
  // dS = P * (dP - delta): without dropout, -delta (constant per lane: one query) is the dP
  // product's initial accumulator, one VALU operation less per score. Not at d = 96, where the 16
  // extra registers spill (measured slower).
  constexpr bool FOLD_DELTA = !DROPOUT && D != 96;
  static_assert(!MASKED || BR == kMaskBlock, "a query tile is one row of the block map");
  // Split launches (small dense causal ones, see the host side): a workgroup takes 64 query rows,
  // and its two wave pairs take the even and the odd K/V tiles: wave w runs the 32 rows of group
  // w & 1 over tiles w >> 1, (w >> 1) + 2, ..., each pair with its own double buffer, and the pair
  // of odd tiles hands its dQ partial sums to the other at the end. A wave's per-tile work is the
  // same as in the plain launch; each row's key loop is half as long.
  static_assert(!QSPLIT || (CAUSAL && !MASKED && !DROPOUT && NW == 4 && D <= 128), "split launches: dense causal");
  constexpr int RW = QSPLIT ? 64 : BR;        // query rows per workgroup
  constexpr int DW = QSPLIT ? 2 : NW;         // waves that load one tile
  constexpr int NLDW = BC * NCH / (64 * DW);  // their DMA instructions per tile
  static_assert(NLDW * 64 * DW == BC * NCH, "a tile splits evenly over its loading waves");

  __shared__ __attribute__((aligned(16))) char sk0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char sv0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char sk1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char sv1[TILE_BYTES];
  // the odd-tile pair's buffers (split launches)
  __shared__ __attribute__((aligned(16))) char skb0[QSPLIT ? TILE_BYTES : 16];
  __shared__ __attribute__((aligned(16))) char svb0[QSPLIT ? TILE_BYTES : 16];
  __shared__ __attribute__((aligned(16))) char skb1[QSPLIT ? TILE_BYTES : 16];
  __shared__ __attribute__((aligned(16))) char svb1[QSPLIT ? TILE_BYTES : 16];
  __shared__ short blist[MASKED ? kMaxMaskBlocks : 1];  // enabled key blocks of this query tile

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, lq = l & 31, hf = l >> 5;
  const int N = p.N;
  // Large causal launches pair query tiles: workgroup (head, u) takes tiles n_tiles-1-u and u one
  // after the other, so every workgroup does the same work and the launch has no tail of short
  // workgroups. (With few workgroups per CU the pairing would only serialise work, so it is off;
  // then tiles are dispatched longest-first.)
  const bool paired = !QSPLIT && CAUSAL && p.n_units != p.n_tiles;
  int head, unit;
  if constexpr (QSPLIT) {
    map_workgroup(blockIdx.x, p.n_units, p.nh, Order::kLongestFirst, true, head, unit);  // 64-row tiles
  } else if (!(MASKED && p.seqlens && !paired &&
               map_workgroup_varlen(blockIdx.x, p.n_units, p.nh, p.heads, p.seqlens, p.N, BR, CAUSAL, true, head,
                                    unit))) {
    // (with sequence lengths the host leaves pairing off, and padding tiles run last)
    map_workgroup(blockIdx.x, p.n_units, p.nh, paired ? Order::kHeadMajor : (CAUSAL ? Order::kLongestFirst : Order::kHeadMajor),
                  !paired, head, unit);
  }
  const int stream = QSPLIT ? (w >> 1) : 0;  // split launches: even (0) or odd (1) K/V tiles
  const int wl = QSPLIT ? (w & 1) : w;       // the wave's index among the waves loading its tiles
  const int n_items = (paired && p.n_tiles - 1 - unit != unit) ? 2 : 1;
  const int Lb = valid_rows<MASKED>(p, head);  // rows >= Lb of every input read as zero
#pragma unroll 1
  for (int item = 0; item < n_items; ++item) {
  const int qt = (paired && item == 0) ? p.n_tiles - 1 - unit : unit;
  if (item > 0) __syncthreads();  // the previous item's staging reads are done before tiles land
  const size_t base = (size_t)head * N * D;
  const size_t rbase = (size_t)head * N;
  const int head_bytes = N * D * 2;
  const int row0 = qt * RW;  // the workgroup's first row
  const int q_w0 = row0 + 32 * wl;
  const int q = q_w0 + lq;

  // Q^T and dO^T operands: lane (q, hf) holds columns 16*kk + 8*hf .. +7 of its row. The same
  // lanes load the matching half of O's row, so delta = rowsum(dO * O) for this row is a dot
  // product over the lane's 8*NKK columns plus one exchange with the lane 32 apart; it is
  // written to the delta buffer for the dK/dV kernel, which runs after this one.
  e16x8 qreg[NKK], oreg[NKK];
  float lse2, dlt;
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + base, Lb * (D * 2));
    const __amdgpu_buffer_rsrc_t rdo = make_rsrc(p.dout + base, Lb * (D * 2));
    const __amdgpu_buffer_rsrc_t rof = make_rsrc(p.o + base, Lb * (D * 2));
    float part = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int off = q * (D * 2) + (16 * kk + 8 * hf) * 2;
      qreg[kk] = __builtin_bit_cast(e16x8, buf_load16(rq, off));
      oreg[kk] = __builtin_bit_cast(e16x8, buf_load16(rdo, off));
      const e16x8 ov = __builtin_bit_cast(e16x8, buf_load16(rof, off));
#pragma unroll
      for (int e = 0; e < 8; ++e) part = fmaf((float)oreg[kk][e], (float)ov[e], part);
    }
    dlt = half_swap_sum(part);
    lse2 = buf_load4f(make_rsrc(p.lse + rbase, Lb * 4), q * 4) * kLog2e;
    if (hf == 0 && stream == 0) buf_store4(make_rsrc(p.delta + rbase, N * 4), q * 4, dlt);
  }

  int n_kv = (Lb + BC - 1) / BC;
  if (CAUSAL) n_kv = min(n_kv, (min(Lb, row0 + RW) - 1) / BC + 1);
  if (MASKED && qt * BR >= Lb) n_kv = 0;  // padding rows only: dQ = 0
  // Loop positions u = 0 .. n_t - 1 map to key tiles tile(u): u, or with a block map the tiles of
  // the enabled 128-key blocks.
  constexpr int TPB = kMaskBlock / BC;
  int n_t = n_kv;
  const bool sparse = MASKED && p.block_mask != nullptr;
  if (sparse && n_t > 0) {
    const int cnt = build_block_list(p.block_mask + ((size_t)head * p.n_mb + qt) * p.n_mb, 1, (n_kv + TPB - 1) / TPB,
                                     blist, w, l);
    __syncthreads();
    n_t = TPB * cnt;
  }
  auto tile = [&](int u) __attribute__((always_inline)) -> int {
    if (QSPLIT) return 2 * u + stream;
    if (!sparse) return u;
    return TPB * __builtin_amdgcn_readfirstlane(blist[u / TPB]) + u % TPB;
  };

  f32x16 dq[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq[db] = f32x16{};

  int goff[NLDW];
#pragma unroll
  for (int i = 0; i < NLDW; ++i) {
    const int pos = (wl + DW * i) * 64 + l;
    const int row = pos / NCH, pc = pos % NCH;
    goff[i] = row * (D * 2) + ((pc ^ T::swz(row)) * 16);
  }
  auto dma = [&](int j, char* kb, char* vb) __attribute__((always_inline)) {
    // (wave-uniform by construction; readfirstlane keeps the descriptors in scalar registers)
    const int key0 = j * BC;
    const int bytes = __builtin_amdgcn_readfirstlane(max(0, min(BC, Lb - key0)) * (D * 2));
    const int first = __builtin_amdgcn_readfirstlane(min(key0, Lb));
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k + base + (size_t)first * D, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v + base + (size_t)first * D, bytes);
#pragma unroll
    for (int i = 0; i < NLDW; ++i) {
      buf_load16_to_lds(rk, kb + (wl + DW * i) * 1024, goff[i]);
      buf_load16_to_lds(rv, vb + (wl + DW * i) * 1024, goff[i]);
    }
  };

  const int g16 = l >> 4, j16 = l & 15;
  const int tr_row_lane = 4 * hf + (j16 >> 2);
  const int tr_col_lane = 16 * (g16 & 1) + 4 * (j16 & 3);
  const int key_lim = CAUSAL ? min(q, Lb - 1) : Lb - 1;
  const float c = p.c;
  f32x16 ndlt;
#pragma unroll
  for (int r = 0; r < 16; ++r) ndlt[r] = -dlt;

  // One key tile; MASK for diagonal and ragged tiles (compiled separately from the clean path).
  // Two 32-key blocks per tile (d <= 96) are software-pipelined inside the tile:
  //   A: S and dP of block 0 on the matrix cores;
  //   B: S and dP of block 1, interleaved with block 0's elementwise work (P, dS);
  //   C: dQ += K^T dS^T for block 0, interleaved with block 1's elementwise work;
  //   D: dQ for block 1.
  // Every matrix instruction is followed by a slice of the elementwise work (stages: exponent
  // argument, exp2 and mask, dS and 16-bit packing; each a step after the previous), fenced by
  // scheduling barriers, so a wave keeps the matrix cores and the VALU busy together. The
  // arithmetic and its order per element are those of the plain sequence.
  auto compute = [&](auto mask_tag, int j, const char* kbuf, const char* vbuf) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    const int key0 = j * BC;
    const int lim = key_lim - key0 - 4 * hf;
    uint32_t kw[NKB][4];  // dropout: Philox words of each 32-key half of the tile
    // K^T fragment of dQ k-step ks, output columns 32*db ..: keys 16ks + {4hf..4hf+3, 8+4hf..}.
    auto frag_dq = [&](int ks, int db) __attribute__((always_inline)) -> e16x8 {
      const int col = 32 * db + tr_col_lane;
      const e16x4 a0 = lds_read_tr16<E>(kbuf, T::elem_off(16 * ks + tr_row_lane, col));
      const e16x4 a1 = lds_read_tr16<E>(kbuf, T::elem_off(16 * ks + 8 + tr_row_lane, col));
      return cat4<E>(a0, a1);
    };
    if constexpr (NKB == 2) {
      // fragment i of block kb's S / dP products: even i = K (S), odd i = V (dP), k-step i / 2
      auto frag_sdp = [&](int kb, int i) __attribute__((always_inline)) -> e16x8 {
        return lds_read16<E>((i & 1) ? vbuf : kbuf, T::chunk_off(32 * kb + lq, 2 * (i >> 1) + hf));
      };
      f32x16 s0, dp0, s1, dp1;
      s0 = f32x16{};
      dp0 = FOLD_DELTA ? ndlt : f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        s0 = H::mfma(frag_sdp(0, 2 * kk), qreg[kk], s0);
        dp0 = H::mfma(frag_sdp(0, 2 * kk + 1), oreg[kk], dp0);
      }
      if constexpr (DROPOUT) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) dropout_words(q, (key0 >> 5) + kb, head, hf, p.seed_lo, p.seed_hi, kw[kb]);
      }
      float xv[16], pv[16], dv[16];
      // stage st of score r of block kb (scores sb, dP - delta or dP in db), packed into dsb
      auto elem = [&](int kb, const f32x16& sb, const f32x16& db, e16x8 (&dsb)[2], int r, int st)
                      __attribute__((always_inline)) {
        if (st == 0) {
          xv[r] = fmaf(sb[r], c, -lse2);
          asm volatile("" ::"v"(xv[r]));
        } else if (st == 1) {
          float pr = fast_exp2(xv[r]);
          if constexpr (MASK) {
            const int krel = 32 * kb + (r >> 2) * 8 + (r & 3);
            pr = krel <= lim ? pr : 0.f;
          }
          pv[r] = pr;
          asm volatile("" ::"v"(pv[r]));
        } else {
          float dpr = db[r];
          if constexpr (DROPOUT) dpr = dropout_keep(kw[kb][r >> 2], r & 3, p.drop_thr) ? dpr * p.drop_scale : 0.f;
          dv[r] = FOLD_DELTA ? pv[r] * dpr : pv[r] * (dpr - dlt);
          if (r & 1) {
            dsb[r >> 3][(r & 7) - 1] = (E)dv[r - 1];
            dsb[r >> 3][r & 7] = (E)dv[r];
            asm volatile("" ::"v"(dsb[r >> 3]));
          }
        }
      };
      // NM matrix instructions (fragment i from frag(i), issued by issue(i, fragment)) with the
      // 16 scores' elementwise stages spread over them; fragments fetched PF instructions ahead.
      auto stage = [&](auto nm_c, auto&& frag, auto&& issue, auto&& work) __attribute__((always_inline)) {
        constexpr int NM = decltype(nm_c)::value;
        constexpr int PF = NM < 3 ? NM : 3;
        e16x8 fr[NM];
#pragma unroll
        for (int i = 0; i < PF; ++i) fr[i] = frag(i);
#pragma unroll
        for (int i = 0; i < NM + 2; ++i) {
          if (i + PF < NM) fr[i + PF] = frag(i + PF);
          if (i < NM) issue(i, fr[i]);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int s0_ = r * NM / 16;
            if (s0_ + 2 == i) work(r, 2);
            if (s0_ + 1 == i) work(r, 1);
            if (s0_ == i) work(r, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      e16x8 dsb0[2], dsb1[2];
      // B
      stage(std::integral_constant<int, 2 * NKK>{}, [&](int i) __attribute__((always_inline)) { return frag_sdp(1, i); },
            [&](int i, const e16x8& f) __attribute__((always_inline)) {
              if (i & 1)
                dp1 = H::mfma(f, oreg[i >> 1], i == 1 ? (FOLD_DELTA ? ndlt : f32x16{}) : dp1);
              else
                s1 = H::mfma(f, qreg[i >> 1], i == 0 ? f32x16{} : s1);
            },
            [&](int r, int st) __attribute__((always_inline)) { elem(0, s0, dp0, dsb0, r, st); });
      // C
      stage(std::integral_constant<int, 2 * NDB>{},
            [&](int i) __attribute__((always_inline)) { return frag_dq(i / NDB, i % NDB); },
            [&](int i, const e16x8& f) __attribute__((always_inline)) { dq[i % NDB] = H::mfma(f, dsb0[i / NDB], dq[i % NDB]); },
            [&](int r, int st) __attribute__((always_inline)) { elem(1, s1, dp1, dsb1, r, st); });
      // D
#pragma unroll
      for (int i = 0; i < 2 * NDB; ++i) dq[i % NDB] = H::mfma(frag_dq(2 + i / NDB, i % NDB), dsb1[i / NDB], dq[i % NDB]);
    } else {
      f32x16 s[NKB], dp[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16{};
        // FOLD_DELTA: dP starts from -delta (the lane's query), giving dP - delta directly
        dp[kb] = FOLD_DELTA ? ndlt : f32x16{};
        // (d >= 128, one 32-key block per tile) the next k-step's K / V fragments read one step ahead
        e16x8 kn = lds_read16<E>(kbuf, T::chunk_off(32 * kb + lq, hf));
        e16x8 vn = lds_read16<E>(vbuf, T::chunk_off(32 * kb + lq, hf));
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const e16x8 kc = kn, vc = vn;
          if (kk + 1 < NKK) {
            const int off = T::chunk_off(32 * kb + lq, 2 * (kk + 1) + hf);
            kn = lds_read16<E>(kbuf, off);
            vn = lds_read16<E>(vbuf, off);
          }
          __builtin_amdgcn_sched_barrier(0);
          s[kb] = H::mfma(kc, qreg[kk], s[kb]);
          dp[kb] = H::mfma(vc, oreg[kk], dp[kb]);
        }
      }
      if constexpr (DROPOUT) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) dropout_words(q, (key0 >> 5) + kb, head, hf, p.seed_lo, p.seed_hi, kw[kb]);
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        e16x8 dsb;
        e16x8 fn = frag_dq(ks, 0);  // read before the elementwise work, which covers its latency
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = (ks & 1) * 8 + e;
          float pr = fast_exp2(fmaf(s[ks >> 1][r], c, -lse2));
          if constexpr (MASK) {
            const int krel = 32 * (ks >> 1) + (r >> 2) * 8 + (r & 3);
            pr = krel <= lim ? pr : 0.f;
          }
          float dpr = dp[ks >> 1][r];
          if constexpr (DROPOUT) dpr = dropout_keep(kw[ks >> 1][r >> 2], r & 3, p.drop_thr) ? dpr * p.drop_scale : 0.f;
          dsb[e] = (E)(FOLD_DELTA ? pr * dpr : pr * (dpr - dlt));
        }
        // dQ^T += K^T dS^T; k-step ks covers keys 16ks + {4hf..4hf+3, 8+4hf..8+4hf+3}. The next
        // output block's fragment is read one product ahead.
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const e16x8 fc = fn;
          if (db + 1 < NDB) fn = frag_dq(ks, db + 1);
          __builtin_amdgcn_sched_barrier(0);
          dq[db] = H::mfma(fc, dsb, dq[db]);
        }
      }
    }
  };
  // Key tiles below the workgroup's diagonal (and not the ragged last tile) run unmasked in the
  // first loop; the remaining ones run the masked path. Both keep the two-buffer ping-pong.
  int j_mask = CAUSAL ? row0 / BC : n_kv;
  if (N % BC != 0) j_mask = min(j_mask, n_kv - 1);
  j_mask = min(j_mask, n_kv);
  if (MASKED) j_mask = 0;
  if (QSPLIT) {
    // loop positions of this wave pair: its clean tiles, then as many positions as the even
    // tiles need for both pairs (the odd pair's last one may lie past its rows: masked, skipped)
    j_mask = max(0, (j_mask - stream + 1) / 2);
    n_t = (n_kv + 1) / 2;
  }
  // Causal: a masked-path tile whose first key follows every row of this wave contributes nothing
  // to the wave's rows (all its scores are masked); the wave skips it but still issues its share of
  // the tile loads and meets the barriers.
  auto run = [&](auto mask_tag, int j, const char* kbuf, const char* vbuf) __attribute__((always_inline)) {
    if (!(CAUSAL && decltype(mask_tag)::value) || j * BC <= q_w0 + 31) compute(mask_tag, j, kbuf, vbuf);
  };
  auto pair = [&](auto mask_tag, int u, int u_end) __attribute__((always_inline)) {
    if (u + 1 < n_t) dma(tile(u + 1), sk1, sv1);
    debug_stage_sync();
    run(mask_tag, tile(u), sk0, sv0);
    debug_stage_sync();
    wait_vmem();
    __syncthreads();
    if (u + 1 < u_end) {
      if (u + 2 < n_t) dma(tile(u + 2), sk0, sv0);
      debug_stage_sync();
      run(mask_tag, tile(u + 1), sk1, sv1);
      debug_stage_sync();
      wait_vmem();
      __syncthreads();
    }
  };
  if constexpr (QSPLIT) {
    // Each wave pair runs the tile loop on its own buffers; every loop position ends with one
    // workgroup barrier in either loop, and both pairs run n_t positions, so the barriers match.
    // (The plain launches keep the loop below written out on their four buffers.)
    auto tiles = [&](char* K0, char* V0, char* K1, char* V1) __attribute__((always_inline)) {
      auto pair_b = [&](auto mask_tag, int u, int u_end) __attribute__((always_inline)) {
        if (u + 1 < n_t) dma(tile(u + 1), K1, V1);
        debug_stage_sync();
        run(mask_tag, tile(u), K0, V0);
        debug_stage_sync();
        wait_vmem();
        __syncthreads();
        if (u + 1 < u_end) {
          if (u + 2 < n_t) dma(tile(u + 2), K0, V0);
          debug_stage_sync();
          run(mask_tag, tile(u + 1), K1, V1);
          debug_stage_sync();
          wait_vmem();
          __syncthreads();
        }
      };
      dma(tile(0), K0, V0);
      wait_vmem();
      __syncthreads();
      int u = 0;
#pragma unroll 1
      for (; u + 1 < j_mask; u += 2) pair_b(std::false_type{}, u, j_mask);
#pragma unroll 1
      for (; u < n_t; u += 2) pair_b(std::true_type{}, u, n_t);
    };
    if (stream == 1) tiles(skb0, svb0, skb1, svb1);
    else tiles(sk0, sv0, sk1, sv1);
  } else if (!MASKED || n_t > 0) {
    dma(tile(0), sk0, sv0);
    wait_vmem();
    __syncthreads();
    int u = 0;
#pragma unroll 1
    for (; u + 1 < j_mask; u += 2) pair(std::false_type{}, u, j_mask);
    // u is even here. A single clean tile may remain before the masked ones; it is run through the
    // masked path (its mask is all-pass), which keeps the buffer parity simple.
#pragma unroll 1
    for (; u < n_t; u += 2) pair(std::true_type{}, u, n_t);
  }

  __syncthreads();  // every wave is done reading the last K / V tile
  char* stage = w == 0 ? sk0 : (w == 1 ? sv0 : (w == 2 ? sk1 : sv1));
  bool stored = false;
  if constexpr (QSPLIT) {
    // the odd-tile pair hands its dQ partial sums (fp32, 128 * D bytes per wave: one or two of its
    // idle tile buffers) to the even-tile wave of the same rows, which adds them and writes the rows
    constexpr int XCH = TILE_BYTES / 1024;  // 1 KB chunks (64 lanes x 16 bytes) per tile buffer
    static_assert(NDB * 4 <= 2 * XCH, "a partial fits two tile buffers");
    f32x4* xa = reinterpret_cast<f32x4*>(wl ? skb1 : skb0);
    f32x4* xb = reinterpret_cast<f32x4*>(wl ? svb1 : svb0);
    if (stream == 1) {
#pragma unroll
      for (int c = 0; c < 4 * NDB; ++c)
        (c < XCH ? xa + c * 64 : xb + (c - XCH) * 64)[l] =
            f32x4{dq[c >> 2][4 * (c & 3)], dq[c >> 2][4 * (c & 3) + 1], dq[c >> 2][4 * (c & 3) + 2], dq[c >> 2][4 * (c & 3) + 3]};
    }
    __syncthreads();
    if (stream == 0) {
#pragma unroll
      for (int c = 0; c < 4 * NDB; ++c) {
        const f32x4 t = (c < XCH ? xa + c * 64 : xb + (c - XCH) * 64)[l];
#pragma unroll
        for (int e = 0; e < 4; ++e) dq[c >> 2][4 * (c & 3) + e] += t[e];
      }
      store_rows_via_lds<E, D, TILE_BYTES>(stage, dq, p.scale, make_rsrc(p.dq + base, head_bytes), q_w0, l);
    }
    stored = true;
  }
  if (!stored) store_rows_via_lds<E, D, TILE_BYTES>(stage, dq, p.scale, make_rsrc(p.dq + base, head_bytes), q_w0, l);
  }  // item
}

// ---------------------------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------------------------
namespace {
// dQ kernel: 4 waves x 32 query rows; key tiles of 64 (32 at d >= 128, where the score and
// dP blocks of a 64-key tile would not fit beside the operands).
// dK/dV kernel: 4 waves x 32 keys; query tiles of 64.
constexpr int kDqNW = 4, kKvNW = 4, kKvBQ = 64;
template <int D>
constexpr int dq_bc() { return D >= 128 ? 32 : 64; }

template <typename E>
BwdParams<E> make_params(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, const float* delta, void* dq, void* dk, void* dv, int BH, int N,
                         float scale) {
  BwdParams<E> prm;
  prm.q = static_cast<const E*>(q);
  prm.k = static_cast<const E*>(k);
  prm.v = static_cast<const E*>(v);
  prm.o = static_cast<const E*>(o);
  prm.dout = static_cast<const E*>(dout);
  prm.lse = lse;
  prm.delta = const_cast<float*>(delta);
  prm.dq = static_cast<E*>(dq);
  prm.dk = static_cast<E*>(dk);
  prm.dv = static_cast<E*>(dv);
  prm.N = N;
  prm.nh = BH;
  prm.n_tiles = 0;
  prm.n_units = 0;
  prm.n_split = 0;
  prm.n_long = 0;
  prm.c = scale * kLog2e;
  prm.scale = scale;
  prm.seqlens = nullptr;
  prm.block_mask = nullptr;
  prm.heads = 1;
  prm.n_mb = (N + kMaskBlock - 1) / kMaskBlock;
  prm.seed_lo = prm.seed_hi = 0;
  prm.drop_thr = 256;
  prm.drop_scale = 1.f;
  return prm;
}

template <typename E, int D>
hipError_t delta_d(BwdParams<E> prm, hipStream_t stream) {
  constexpr int RPB = 256 / pow2_at_least<D / 8>() * 4;  // rows per block (4 per thread group)
  const long rows = (long)prm.nh * prm.N;
  hipLaunchKernelGGL((bwd_delta_kernel<E, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, stream, prm);
  return hipGetLastError();
}

template <typename E, int D, bool CAUSAL, bool MASKED = false, bool DROPOUT = false>
hipError_t dkdv_d(BwdParams<E> prm, hipStream_t stream) {
  prm.n_tiles = (prm.N + 32 * kKvNW - 1) / (32 * kKvNW);
  const dim3 grid(prm.n_tiles * prm.nh), block(kKvNW * 64);
  if constexpr (D > 128 || (D == 128 && !CAUSAL)) {  // dV, then dK (see bwd_dkdv_kernel)
    hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, kKvNW, kKvBQ, CAUSAL, MASKED, DROPOUT, 1>), grid, block, 0, stream, prm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, kKvNW, kKvBQ, CAUSAL, MASKED, DROPOUT, 2>), grid, block, 0, stream, prm);
  } else {
    if constexpr (CAUSAL && !MASKED) {
      // Small launch whose 64-key workgroups all fit on the chip at once (two per CU at d <= 64;
      // one at d = 96, 128, whose doubled tile buffers take 96-128 KB): the stream kernel halves
      // each key's query loop.
      const long per_cu = D <= 64 ? 2 : 1;
      if (prm.N >= 512 && 2L * prm.n_tiles * prm.nh <= per_cu * device_cu_count()) {
        prm.n_units = (prm.N + 63) / 64;
        hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, kKvNW, kKvBQ, CAUSAL, MASKED, DROPOUT, 0, false, true>),
                           dim3(prm.n_units * prm.nh), block, 0, stream, prm);
        return hipGetLastError();
      }
      // Otherwise, when its 128-key workgroups fit at once: split about 3/8 of the key tiles, as
      // long as the extra workgroups still fit. Halving a tile costs ~25% more time per query tile
      // (half the work per barrier and tile load), so key tile 0's halves then last about as long
      // as the first unsplit tile.
      const long slots = (long)device_cu_count() * dkdv_waves_per_simd<D, 0, CAUSAL, MASKED>();
      const long wgs = (long)prm.n_tiles * prm.nh;
      if (prm.n_tiles >= 8 && wgs < slots) {
        const long fit = slots / prm.nh - prm.n_tiles;
        const int n_split = (int)std::min<long>((3 * prm.n_tiles + 4) / 8, fit);
        if (n_split >= 3) {
          const int n_qt = (prm.N + kKvBQ - 1) / kKvBQ;
          prm.n_split = n_split;
          prm.n_long = std::max(n_split, std::min(prm.n_tiles, (n_qt + 3) / 4));
          hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, kKvNW, kKvBQ, CAUSAL, MASKED, DROPOUT, 0, true>),
                             dim3((prm.n_tiles + n_split) * prm.nh), block, 0, stream, prm);
          return hipGetLastError();
        }
      }
    }
    hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, kKvNW, kKvBQ, CAUSAL, MASKED, DROPOUT, 0>), grid, block, 0, stream, prm);
  }
  return hipGetLastError();
}

template <typename E, int D, bool CAUSAL, bool MASKED = false, bool DROPOUT = false>
hipError_t dq_d(BwdParams<E> prm, hipStream_t stream) {
  prm.n_tiles = (prm.N + 32 * kDqNW - 1) / (32 * kDqNW);
  // Pair causal tiles when there are at least four workgroups per CU to begin with, except where
  // the kernel orders tiles by sequence length instead (map_workgroup_varlen's conditions).
  const bool by_length = MASKED && prm.seqlens && prm.heads % 8 == 0 && prm.nh / prm.heads <= 64;
  prm.n_units = (CAUSAL && !by_length && (long)prm.n_tiles * prm.nh >= 4L * device_cu_count()) ? (prm.n_tiles + 1) / 2
                                                                                              : prm.n_tiles;
  if constexpr (CAUSAL && !MASKED && D <= 128) {
    // Small launch: when its 64-row workgroups all fit on the chip at once (two per CU; one at
    // d = 96, whose doubled tile buffers take 96 KB), the split kernel halves each row's key loop.
    const long slots = (D == 96 ? 1L : 2L) * device_cu_count();
    if (prm.N >= 512 && 2L * prm.n_tiles * prm.nh <= slots) {
      prm.n_units = (prm.N + 63) / 64;
      hipLaunchKernelGGL((bwd_dq_kernel<E, D, dq_bc<D>(), kDqNW, CAUSAL, MASKED, DROPOUT, true>),
                         dim3(prm.n_units * prm.nh), dim3(kDqNW * 64), 0, stream, prm);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((bwd_dq_kernel<E, D, dq_bc<D>(), kDqNW, CAUSAL, MASKED, DROPOUT>), dim3(prm.n_units * prm.nh),
                     dim3(kDqNW * 64), 0, stream, prm);
  return hipGetLastError();
}
}  // namespace

namespace {
template <typename E>
hipError_t delta_typed(const void* o, const void* dout, float* delta, int BH, int N, int d, hipStream_t stream) {
  BwdParams<E> prm = make_params<E>(nullptr, nullptr, nullptr, o, nullptr, dout, delta, nullptr, nullptr, nullptr, BH,
                                    N, 1.f);
  return with_head_dim(d, [&](auto dd) { return delta_d<E, decltype(dd)::value>(prm, stream); });
}

template <typename E>
hipError_t dkdv_typed(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                      const float* delta, void* dk, void* dv, int BH, int N, int d, float scale, bool causal,
                      hipStream_t stream) {
  BwdParams<E> prm = make_params<E>(q, k, v, nullptr, lse, dout, delta, nullptr, dk, dv, BH, N, scale);
  return with_head_dim(d, [&](auto dd) {
    constexpr int D = decltype(dd)::value;
    return causal ? dkdv_d<E, D, true>(prm, stream) : dkdv_d<E, D, false>(prm, stream);
  });
}

template <typename E>
hipError_t dq_typed(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                    float* delta, void* dq, int BH, int N, int d, float scale, bool causal, hipStream_t stream) {
  BwdParams<E> prm = make_params<E>(q, k, v, o, lse, dout, delta, dq, nullptr, nullptr, BH, N, scale);
  return with_head_dim(d, [&](auto dd) {
    constexpr int D = decltype(dd)::value;
    return causal ? dq_d<E, D, true>(prm, stream) : dq_d<E, D, false>(prm, stream);
  });
}
template <typename E, int D, bool DROPOUT>
hipError_t masked_d(const BwdParams<E>& prm, bool causal, hipStream_t stream) {
  hipError_t e = causal ? dq_d<E, D, true, true, DROPOUT>(prm, stream) : dq_d<E, D, false, true, DROPOUT>(prm, stream);
  if (e != hipSuccess) return e;
  return causal ? dkdv_d<E, D, true, true, DROPOUT>(prm, stream) : dkdv_d<E, D, false, true, DROPOUT>(prm, stream);
}

template <typename E>
hipError_t masked_typed(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                        float* delta, void* dq, void* dk, void* dv, int BH, int N, int d, float scale, bool causal,
                        const Masks& m, const Dropout& drop, hipStream_t stream) {
  BwdParams<E> prm = make_params<E>(q, k, v, o, lse, dout, delta, dq, dk, dv, BH, N, scale);
  prm.seqlens = m.seqlens;
  prm.block_mask = m.block_mask;
  prm.heads = m.heads;
  prm.seed_lo = (uint32_t)drop.seed;
  prm.seed_hi = (uint32_t)(drop.seed >> 32);
  prm.drop_thr = drop.threshold;
  prm.drop_scale = drop.threshold > 0 ? 256.0f / (float)drop.threshold : 0.f;
  const bool dr = drop.active();
  return with_head_dim(d, [&](auto dd) {
    constexpr int D = decltype(dd)::value;
    return dr ? masked_d<E, D, true>(prm, causal, stream) : masked_d<E, D, false>(prm, causal, stream);
  });
}
}  // namespace

hipError_t launch_bwd_masked(bool fp16, const void* q, const void* k, const void* v, const void* o, const float* lse,
                             const void* dout, float* delta, void* dq, void* dk, void* dv, int BH, int N, int d,
                             float scale, bool causal, const Masks& masks, const Dropout& drop, hipStream_t stream) {
  return fp16 ? masked_typed<f16>(q, k, v, o, lse, dout, delta, dq, dk, dv, BH, N, d, scale, causal, masks, drop, stream)
              : masked_typed<bf16>(q, k, v, o, lse, dout, delta, dq, dk, dv, BH, N, d, scale, causal, masks, drop,
                                   stream);
}

hipError_t launch_bwd_delta(bool fp16, const void* o, const void* dout, float* delta, int BH, int N, int d,
                            hipStream_t stream) {
  return fp16 ? delta_typed<f16>(o, dout, delta, BH, N, d, stream) : delta_typed<bf16>(o, dout, delta, BH, N, d, stream);
}

hipError_t launch_bwd_dkdv(bool fp16, const void* q, const void* k, const void* v, const float* lse, const void* dout,
                           const float* delta, void* dk, void* dv, int BH, int N, int d, float scale, bool causal,
                           hipStream_t stream) {
  return fp16 ? dkdv_typed<f16>(q, k, v, lse, dout, delta, dk, dv, BH, N, d, scale, causal, stream)
              : dkdv_typed<bf16>(q, k, v, lse, dout, delta, dk, dv, BH, N, d, scale, causal, stream);
}

hipError_t launch_bwd_dq(bool fp16, const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, float* delta, void* dq, int BH, int N, int d, float scale, bool causal,
                         hipStream_t stream) {
  return fp16 ? dq_typed<f16>(q, k, v, o, lse, dout, delta, dq, BH, N, d, scale, causal, stream)
              : dq_typed<bf16>(q, k, v, o, lse, dout, delta, dq, BH, N, d, scale, causal, stream);
}

}  // namespace fa
