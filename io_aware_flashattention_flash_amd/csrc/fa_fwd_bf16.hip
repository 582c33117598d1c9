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
//  * K/V tiles go from HBM straight into the swizzled LDS layout with
//    buffer_load ... lds (no staging registers, no LDS write instructions); a
//    per-tile buffer descriptor bounds the ragged last tile, whose missing rows
//    arrive as zeros. Two LDS buffers alternate: tile j+1 is in flight while
//    tile j is computed, with one barrier per tile.
//  * softmax in the log2 domain: one FMA per score, p = exp2(s*c - m*c) with
//    c = |scale| * log2(e) (a negative scale is applied by negating Q, which is
//    exact in bf16). The running max is raised only when a tile's max exceeds
//    it by more than 2^8, so the O / l rescale runs on a handful of tiles
//    instead of every tile; p then stays below 2^8, far inside fp32/bf16 range,
//    and O / l uses the same reference max in numerator and denominator, so the
//    result is unchanged.
//  * two row sums are kept: l over the fp32 probabilities (for LSE: summing the
//    rounded values would put up to ~1.6e-3 of error into LSE on rows dominated
//    by a few keys), and l~ over the bf16-rounded probabilities that actually
//    multiply V (v_dot2_f32_bf16, half an instruction per score). O is divided
//    by l~, so the weights applied to V sum to one exactly; with a stale
//    reference max the dominant probability is no longer exactly 1, and
//    dividing by l would leave its rounding error (up to 2^-9 |V|) in O.
//  * causal: tiles entirely above the diagonal are never loaded; only diagonal
//    and ragged tiles evaluate the mask, with a branch-free compare per score.
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
  float c;        // |scale| * log2(e) (a tiny positive value when scale == 0)
  uint32_t qsign;  // 0x80008000 to negate Q (negative scale), else 0
};

// Threshold (log2 units) by which a tile's max must exceed the running max before the
// running max is raised and the accumulators rescaled.
constexpr float kRescaleThreshold = 8.0f;

template <int D, int BC, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void fwd_bf16_kernel(FwdBf16Params p) {
  constexpr int BR = 32 * NW;
  constexpr int NCH = D / 8;
  constexpr int TILE_BYTES = BC * D * 2;
  constexpr int NLD = BC * NCH / (64 * NW);  // LDS-DMA instructions per wave per tensor per tile
  static_assert(NLD * 64 * NW == BC * NCH, "tile must split evenly over the workgroup's waves");
  constexpr int NKB = BC / 32;  // 32-key blocks per tile
  constexpr int NDB = D / 32;   // 32-row blocks of O^T
  constexpr int NKK = D / 16;   // k-steps of K Q^T
  constexpr int NKS = BC / 16;  // k-steps of V^T P^T
  using T = SwizzledTile<D>;

  __shared__ __attribute__((aligned(16))) char sk0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char sv0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char sk1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char sv1[TILE_BYTES];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, lq = l & 31, hf = l >> 5;
  const int N = p.N;

  int head, qt;
  map_workgroup(blockIdx.x, p.n_qt, p.nh, CAUSAL ? Order::kLongestFirst : Order::kHeadMajor, true, head, qt);
  const size_t base = (size_t)head * N * D;
  const bf16* Kh = p.k + base;
  const bf16* Vh = p.v + base;
  const int head_bytes = N * D * 2;

  const int q_w0 = qt * BR + 32 * w;  // first query row of this wave
  const int q = q_w0 + lq;            // this lane's query row

  // Q^T operand: lane (q, hf) holds Q[q][16*kk + 8*hf .. +7]; rows >= N read as zero.
  bf16x8 qreg[NKK];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + base, head_bytes);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 t = buf_load16(rq, q * (D * 2) + (16 * kk + 8 * hf) * 2);
      t ^= p.qsign;
      qreg[kk] = __builtin_bit_cast(bf16x8, t);
    }
  }

  int n_kv = (N + BC - 1) / BC;
  if (CAUSAL) n_kv = min(n_kv, (min(N, (qt + 1) * BR) - 1) / BC + 1);

  // Byte offsets (within a tile) of the 16-byte chunks this lane deposits: DMA instruction i of
  // wave w fills LDS chunk positions (w + NW*i)*64 + lane, i.e. swizzled (row, chunk) slots.
  int goff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    const int pos = (w + NW * i) * 64 + l;
    const int row = pos / NCH, pc = pos % NCH;
    goff[i] = row * (D * 2) + ((pc ^ T::swz(row)) * 16);
  }
  auto dma = [&](int j, char* kb, char* vb) __attribute__((always_inline)) {
    const int key0 = j * BC;
    const int bytes = min(BC, N - key0) * (D * 2);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + (size_t)key0 * D, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vh + (size_t)key0 * D, bytes);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      buf_load16_to_lds(rk, kb + (w + NW * i) * 1024, goff[i]);
      buf_load16_to_lds(rv, vb + (w + NW * i) * 1024, goff[i]);
    }
  };

  // Lane-constant parts of the LDS read addresses.
  const int g16 = l >> 4, j16 = l & 15;
  const int v_row_lane = 4 * hf + (j16 >> 2);
  const int v_col_lane = 16 * (g16 & 1) + 4 * (j16 & 3);
  // Largest key index this lane's query may see (causal and ragged tail).
  const int key_lim = CAUSAL ? min(q, N - 1) : N - 1;

  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f, lr_run = 0.f;
  const float c = p.c;

  auto compute = [&](int j, const char* kbuf, const char* vbuf) __attribute__((always_inline)) {
    const int key0 = j * BC;
    // (A wave whose rows all precede this tile's keys still runs it: the mask zeroes every
    // probability. Branching around it would cost more in register copies than the ~1.5% of
    // matrix work it saves.)
    // S^T = K Q^T for the NKB 32-key blocks of this tile.
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        s[kb] = mfma_bf16_32x32x16(lds_read16(kbuf, T::chunk_off(32 * kb + lq, 2 * kk + hf)), qreg[kk], s[kb]);
    }
    // Mask (diagonal / ragged tiles only): key index relative to the tile vs this lane's limit.
    if ((key0 + BC > N) || (CAUSAL && key0 + BC - 1 > q_w0)) {
      const int lim = key_lim - key0 - 4 * hf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int krel = 32 * kb + (r >> 2) * 8 + (r & 3);
          s[kb][r] = krel <= lim ? s[kb][r] : -INFINITY;
        }
    }
    // Row max of the raw scores (c > 0), across both halves of the 32-key blocks. The
    // NaN-propagating maximum maps to v_maximum3_f32 and needs no quieting of the MFMA outputs.
    float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        mx0 = vmax3(mx0, s[kb][r], s[kb][r + 1]);
        mx1 = vmax3(mx1, s[kb][r + 2], s[kb][r + 3]);
      }
    const float mx = half_swap_max(vmax(mx0, mx1)) * c;
    // Raise the running max only when this tile exceeds it by more than the threshold.
    const bool raise = mx > m_run + kRescaleThreshold;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float alpha = raise ? fast_exp2(m_run - mx) : 1.0f;
      m_run = raise ? mx : m_run;
      l_run *= alpha;
      lr_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;
    }
    const float neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
    // P^T = exp2(s*c - m), summed in fp32, rounded to bf16 as the B operand of O^T += V^T P^T.
    // k-step ks covers keys 16ks + {4hf..4hf+3, 8+4hf..8+4hf+3}, i.e. accumulator registers
    // (ks&1)*8 + 0..7 of block ks>>1. Each k-step's products are issued as soon as its eight
    // probabilities exist, so the matrix cores work on step ks while the VALU forms step ks+1.
    float rs0 = 0.f, rs1 = 0.f, rr = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 pkk;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float pa = fast_exp2(fmaf(s[ks >> 1][(ks & 1) * 8 + e], c, neg_m));
        const float pb = fast_exp2(fmaf(s[ks >> 1][(ks & 1) * 8 + e + 1], c, neg_m));
        rs0 += pa;
        rs1 += pb;
        const bf16x2 pr = {(bf16)pa, (bf16)pb};
        rr = dot2_ones(pr, rr);
        pkk[e] = pr[0];
        pkk[e + 1] = pr[1];
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int col = 32 * db + v_col_lane;
        const bf16x4 a0 = lds_read_tr16(vbuf, T::elem_off(16 * ks + v_row_lane, col));
        const bf16x4 a1 = lds_read_tr16(vbuf, T::elem_off(16 * ks + 8 + v_row_lane, col));
        acc_o[db] = mfma_bf16_32x32x16(cat4(a0, a1), pkk, acc_o[db]);
      }
    }
    l_run += rs0 + rs1;
    lr_run += rr;
  };

  // Ping-pong over the two LDS buffers: tile j+1 streams in while tile j is computed.
  dma(0, sk0, sv0);
  wait_vmem();
  __syncthreads();
  int j = 0;
  for (; j + 1 < n_kv; j += 2) {
    dma(j + 1, sk1, sv1);
    compute(j, sk0, sv0);
    wait_vmem();
    __syncthreads();
    if (j + 2 < n_kv) dma(j + 2, sk0, sv0);
    compute(j + 1, sk1, sv1);
    wait_vmem();
    __syncthreads();
  }
  if (j < n_kv) compute(j, sk0, sv0);

  // Epilogue: O = O_acc / l~, LSE = ln2 * (m + log2 l). The accumulator holds one query row per
  // lane, so O is staged through LDS (each wave in one of the now idle tile buffers, rows padded
  // by 16 bytes) and written back as whole rows of 16-byte chunks. Rows >= N fall outside the
  // buffer descriptors and are dropped.
  const float l_tot = half_swap_sum(l_run);
  const float inv = 1.0f / half_swap_sum(lr_run);
  __syncthreads();  // every wave is done reading the last K/V tile
  char* ostage = w == 0 ? sk0 : (w == 1 ? sv0 : (w == 2 ? sk1 : sv1));
  store_rows_via_lds<D, TILE_BYTES>(ostage, acc_o, inv, make_rsrc(p.o + base, head_bytes), q_w0, l);
  if (p.lse && hf == 0) {
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(p.lse + (size_t)head * N, N * 4);
    buf_store4(rl, q * 4, (m_run + __log2f(l_tot)) * kLn2);
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
  // Scores are scale * q.k = |scale| * (sign(scale) q).k: the sign goes into Q (exact), the
  // magnitude into c. A zero scale uses a tiny c: every exp2 argument then rounds to 0, which is
  // exactly the uniform softmax a zero scale means, and masked scores still map to -inf.
  prm.c = scale == 0.f ? 1e-30f : fabsf(scale) * kLog2e;
  prm.qsign = scale < 0.f ? 0x80008000u : 0u;
  if (d == 64) return causal ? launch_cfg<64, 64, NW, true>(prm, stream) : launch_cfg<64, 64, NW, false>(prm, stream);
  if (d == 128) return causal ? launch_cfg<128, 64, NW, true>(prm, stream) : launch_cfg<128, 64, NW, false>(prm, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
