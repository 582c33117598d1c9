// Fused attention forward for gfx950, 16-bit storage (bf16 or fp16).
//
// What it computes (52jiny.com FlashAttention explainer, "key ideas" parts 1-3;
// codechina.net CUDA/FlashAttention article, sections 4.1-4.2 and 5.1): one
// workgroup owns a tile of BR query rows of one (batch, head). It keeps that Q
// tile in registers and streams the K/V tiles of the same head through LDS.
// Per K/V tile it forms the scores on the matrix cores, applies the scale and
// the causal / ragged-tail mask, keeps every row's running reference maximum m
// and running sum l of exponentials (rescaling the earlier output accumulation
// when m moves), and accumulates P V on the matrix cores. Only O and the
// per-row log-sum-exp LSE = m + ln l leave the chip; the N x N score matrix
// never exists in HBM.
//
// gfx950 mapping:
//  * a wave owns 32 query rows and computes the transposed score block
//    S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (or _f16), so each lane holds the scores
//    of ONE query (its column) for 16 of every 32 keys; the other 16 sit in
//    the lane 32 apart.
//  * the same accumulator registers, rounded to the 16-bit type, are the B operand of
//    O^T += V^T P^T; V^T comes from the row-major V tile in LDS through the
//    gfx950 LDS transpose read (ds_read_b64_tr_b16), with the key order chosen
//    to match the accumulator's row order.
//  * K/V tiles of 64 keys go from HBM straight into the swizzled LDS layout with
//    buffer_load ... lds (no staging registers, no LDS write instructions); a
//    per-tile buffer descriptor bounds the ragged last tile, whose missing rows
//    arrive as zeros.
//  * software pipeline over 32-key halves. A matrix instruction takes 32 cycles,
//    and the VALU work of the softmax (about five issue slots per score) only
//    hides behind it if the two are interleaved in the instruction stream. Each
//    tile j is therefore split into halves and processed in two phases:
//      A(j): S(j, keys 32-63) and O += P(j-1, keys 32-63) V on the matrix cores,
//            probabilities of S(j, keys 0-31) on the VALU;
//      B(j): S(j+1, keys 0-31) and O += P(j, keys 0-31) V on the matrix cores,
//            probabilities of S(j, keys 32-63) on the VALU.
//    Inside a phase every matrix instruction is followed by a slice of the
//    element work (exponent argument, exp2, sums, 16-bit packing) of different
//    scores, each stage a step after the previous one, and LDS fragments are
//    fetched four instructions ahead; scheduling barriers keep this order.
//    One barrier per tile: K(j+2) and V(j+1) are issued right after the barrier
//    that follows A(j), the last reader of the buffers they overwrite. The last two
//    tiles run without the look-ahead: no scores of a tile past the end, and a final
//    O += P V for the last half on its own.
//  * softmax in the log2 domain: p = exp2(s*c - m) with c = |scale| * log2(e)
//    (a negative scale is applied by negating Q, which is exact in 16 bits). There
//    is no per-tile row maximum: any reference m gives the same O = sum p V /
//    sum p and LSE = m + log l, so m is only moved when it has to be. The
//    per-lane sum of a half's 16 probabilities (needed anyway for l) bounds each
//    of them; when it exceeds 2^16 (always on a row's first half, where m is
//    still a placeholder, and later only if the scores climb by more than ~16
//    log2 units) the half takes a slow path that raises m to the half's max,
//    rescales O and the sums, and recomputes. Probabilities therefore stay
//    below 2^16 (2^15 for fp16, whose largest value is 65504), and the maximum reduction leaves
//    the common path.
//  * two row sums are kept: l over the fp32 probabilities (for LSE: summing the
//    rounded values would put up to ~2e-3 of error into LSE on rows dominated
//    by a few keys), and l~ over the 16-bit-rounded probabilities that actually
//    multiply V (v_dot2_f32_bf16 / _f16, half an instruction per score). O is divided
//    by l~, so the weights applied to V sum to one exactly; with a reference
//    max that is not the row max the dominant probability is not exactly 1, and
//    dividing by l would leave its rounding error (up to 2^-9 |V|) in O.
//  * causal: tiles entirely above the workgroup's last row are never loaded;
//    only diagonal and ragged halves evaluate the mask, with a branch-free
//    compare per score. The tile count is padded to even so the two-tile loop
//    body needs no exit in its middle; the padded tile is fully masked.
#include <type_traits>

#include "fa_device.h"
#include "fa_launch.h"

namespace fa {

template <typename E>
struct Fwd16Params {
  const E* q;
  const E* k;
  const E* v;
  E* o;
  float* lse;
  int N;           // query rows (Q, O, LSE)
  int nh;
  int n_qt;
  float c;        // |scale| * log2(e) (a tiny positive value when scale == 0)
  uint32_t qsign;  // 0x80008000 to negate Q (negative scale; the sign bit of both 16-bit types), else 0
  // Key-split launches only (KV_SPLIT): key rows, the causal offset of query row 0 (query i sees
  // keys j <= i + key_offset), K/V tiles per split, and the fp32 partials
  // opart [split][head][row][D] and lsepart [split][head][row].
  int Nk;
  int key_offset;
  int tiles_per_split;
  float* opart;
  float* lsepart;
  // Key-split launches only: nonzero when each head has a single query tile, so every K/V tile is
  // read by exactly one workgroup; its loads then carry the non-temporal cache hint.
  int kv_once;
  // Key-split launches only: nonzero when there is a single split (and split_direct_ok(D)). Its
  // workgroups then write the final O and LSE themselves (what the merge would produce with one
  // split: weight exactly 1), and no partials are written or merged.
  int kv_direct;
  // Per-sequence lengths (sequence = head / heads), or null: kMasked, the valid rows of Q and K/V;
  // kSplit, the valid keys of the cache. Values are clamped to [0, N] (kSplit: [0, Nk]).
  const int* seqlens;
  // kMasked only: block-sparse map [head][n_qt][n_kb], one byte per 128 x 128 block of scores
  // (zero: skipped), or null.
  const uint8_t* block_mask;
  int heads;
  int n_kb;
  // kMaskedDropout only: Philox key, keep threshold T (twice, one per 16-bit half) and 256 / T.
  uint32_t seed_lo;
  uint32_t seed_hi;
  uint32_t drop_thr2;
  float drop_scale;
};

// A block's per-lane probability sum above this bound means some probability may have left the
// safe range (or the running max is still the initial placeholder): the block then takes the
// slow path, which raises the running max to the block's max and recomputes.
// (fp16 tops out at 65504, so its probabilities are held below 2^15.)
template <typename E>
constexpr float kOverflowSum = std::is_same<E, f16>::value ? 32768.0f : 65536.0f;
constexpr float kInitMax = -1e30f;

// Head dims whose key-split kernel writes O and LSE itself when there is one split. At d = 256 the
// second epilogue costs registers the kernel does not have (it would spill), so it keeps the merge.
__host__ __device__ constexpr bool split_direct_ok(int d) { return d <= 128; }

// buf_load16_to_lds with the non-temporal cache policy (bit 1 of the cache-policy operand, "nt"):
// for data that no other workgroup reads again.
__device__ __forceinline__ void buf_load16_to_lds_once(__amdgpu_buffer_rsrc_t r, char* lds_dst, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, off, 0, 0, 2);
}

// Launch modes.
//  kDense:  Q and K/V have the same length N; O, LSE are final.
//  kSplit:  this workgroup covers only the K/V tiles of split blockIdx.y and writes its rows'
//           partial (O, LSE) in fp32 (rows with no visible key in the split: O = 0, LSE = -inf); a
//           merge kernel combines the splits. Optional per-sequence cache lengths.
//  kMasked: square, with optional per-sequence lengths (rows >= L of Q and K/V are padding) and
//           an optional block-sparse map; the workgroup walks only the key blocks its map row
//           enables. Rows that see no key get O = 0, LSE = -inf.
//  kMaskedDropout: kMasked plus attention dropout: each probability that multiplies V is kept
//           or zeroed by its Philox byte (dropout_words), kept ones scaled by 256 / T at the end;
//           the row sums (hence LSE and the normaliser) are those of the undropped softmax.
enum FwdMode : int { kDense = 0, kSplit = 1, kMasked = 2, kMaskedDropout = 3 };

// d = 256 needs more than half the register file per lane (O accumulator 128, Q operand 64): one
// workgroup per CU, one wave per SIMD. Smaller head dims run two workgroups per CU.
//
// QSPLIT (dense launches at d <= 128 whose 128-row tiles are no more than the CUs, or half of
// them at d > 64, where the doubled tile buffers leave room for one workgroup per CU; causal ones
// with long rows up to twice that): a workgroup
// takes 64 query rows, and its two wave pairs take the even and the odd K/V tiles: wave w runs the
// 32 rows of group w & 1 over tiles w >> 1, (w >> 1) + 2, ..., each pair with its own double
// buffer, and the pair of odd tiles hands its (m, l, l~, O) to the other at the end, which merges
// them by the online-softmax rule. A wave's loop is the same as in the plain launch; the
// workgroups are twice as many and each row's key loop half as long.
template <typename E, int D, int BC, int NW, bool CAUSAL, int MODE, bool QSPLIT = false>
__global__ __launch_bounds__(NW * 64, D > 128 ? 1 : 2) void fwd16_kernel(Fwd16Params<E> p) {
  constexpr bool KV_SPLIT = MODE == kSplit, DROPOUT = MODE == kMaskedDropout;
  constexpr bool MASKED = MODE == kMasked || DROPOUT;
  using H = Half16<E>;
  using e16x8 = typename H::x8;
  using e16x4 = typename H::x4;
  using e16x2 = typename H::x2;
  static_assert(BC == 64, "two 32-key halves per tile");
  constexpr int BR = 32 * NW;
  constexpr int NCH = D / 8;
  constexpr int TILE_BYTES = BC * D * 2;
  constexpr int NLD = BC * NCH / (64 * NW);
  static_assert(NLD * 64 * NW == BC * NCH, "tile must split evenly over the workgroup's waves");
  constexpr int NDB = D / 32;
  constexpr int NKK = D / 16;
  using T = SwizzledTile<D>;
  static_assert(!MASKED || BR == kMaskBlock, "a query tile is one row of the block map");
  static_assert(!QSPLIT || (MODE == kDense && D <= 128 && NW == 4), "split launches: dense forward, d <= 128");
  constexpr int RW = QSPLIT ? 64 : BR;    // query rows per workgroup
  constexpr int DW = QSPLIT ? 2 : NW;     // waves that load one tile
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
  const int N = p.N;                         // query rows
  const int Nk = KV_SPLIT ? p.Nk : p.N;      // key rows

  int head, qt;
  // Masked launches with lengths: tiles with work first, padding tiles last (map_workgroup_varlen);
  // the padding tiles' zero rows are then written by the head's tiles with work, spread over the
  // launch, and the padding workgroups themselves exit at once.
  const bool vmapped = MASKED && p.seqlens &&
                       map_workgroup_varlen(blockIdx.x, p.n_qt, p.nh, p.heads, p.seqlens, p.N, BR, CAUSAL, true, head, qt);
  if (!vmapped)
    map_workgroup(blockIdx.x, p.n_qt, p.nh, CAUSAL ? Order::kLongestFirst : Order::kHeadMajor, true, head, qt);
  // Valid query rows Lq and keys Lk of this head's sequence.
  int Lq = N, Lk = Nk;
  if ((KV_SPLIT || MASKED) && p.seqlens) {
    Lk = min(max(p.seqlens[head / p.heads], 0), Nk);
    if (MASKED) Lq = Lk;
  }
  const int koff = KV_SPLIT ? Lk - N : 0;  // causal: query i sees keys j <= i + koff
  const size_t base = (size_t)head * N * D;
  const size_t kbase = (size_t)head * Nk * D;
  const E* Kh = p.k + kbase;
  const E* Vh = p.v + kbase;
  const int head_bytes = N * D * 2;
  const int stream = QSPLIT ? (w >> 1) : 0;  // split launches: even (0) or odd (1) K/V tiles
  const int wl = QSPLIT ? (w & 1) : w;       // the wave's index among the waves loading its tiles
  const int q_w0 = qt * RW + 32 * wl;
  const int q = q_w0 + lq;

  // Rows that see no key at all (padding rows, empty map rows): O = 0, LSE = -inf. This lane's
  // row of tile t.
  auto write_empty_row = [&](int t) __attribute__((always_inline)) {
    const int row = t * BR + 32 * w + lq;
    if (row < N) {
      const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.o + base, head_bytes);
#pragma unroll
      for (int i = 0; i < D / 16; ++i) buf_store16(ro, (row * D + 8 * (2 * i + hf)) * 2, u32x4{0, 0, 0, 0});
      if (p.lse && hf == 0) p.lse[(size_t)head * N + row] = -INFINITY;
    }
  };
  auto write_empty_rows = [&]() __attribute__((always_inline)) { write_empty_row(qt); };
  // A tile with work also writes the padding tiles T + qt, 2T + qt, ... of its head (T = the tiles
  // with work), when the padding workgroups leave them to it (vmapped).
  auto write_carried_rows = [&]() __attribute__((always_inline)) {
    const int T = (Lq + BR - 1) / BR;
    if (MASKED && vmapped && T > 0)
      for (int pt = T + qt; pt < p.n_qt; pt += T) write_empty_row(pt);
  };
  if (MASKED && qt * BR >= Lq) {  // a tile of padding rows only (uniform over the workgroup)
    if (!vmapped || Lq == 0) write_empty_rows();  // else a tile with work of this head writes them
    return;
  }

  // Q^T operand: lane (q, hf) holds Q[q][16*kk + 8*hf .. +7]; rows >= Lq read as zero.
  e16x8 qreg[NKK];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.q + base, Lq * (D * 2));
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 t = buf_load16(rq, q * (D * 2) + (16 * kk + 8 * hf) * 2);
      t ^= p.qsign;
      qreg[kk] = __builtin_bit_cast(e16x8, t);
    }
  }
  int n_kv = (Lk + BC - 1) / BC;
  if (CAUSAL) {
    const int last_key = min(Lq, (qt + 1) * RW) - 1 + koff;  // the last key any row here sees
    n_kv = min(n_kv, last_key < 0 ? 0 : last_key / BC + 1);
  }
  // K/V tiles [jb, je) of this workgroup; keys at or beyond key_end are masked.
  int jb = 0, je = n_kv;
  if (KV_SPLIT) {
    jb = blockIdx.y * p.tiles_per_split;
    je = min(n_kv, jb + p.tiles_per_split);
    if (jb >= je) {  // no visible key in this split: empty partials (uniform over the workgroup)
      if (split_direct_ok(D) && p.kv_direct) {
        write_empty_rows();
        return;
      }
      if (q < N) {
        const size_t row = ((size_t)blockIdx.y * p.nh + head) * N + q;
        if (hf == 0) p.lsepart[row] = -INFINITY;
        for (int c4 = 4 * hf; c4 < D; c4 += 8) *reinterpret_cast<f32x4*>(p.opart + row * D + c4) = f32x4{};
      }
      return;
    }
  }
  const int key_end = KV_SPLIT ? min(Lk, je * BC) : Lk;

  // Block-sparse: compact the enabled 128-key blocks of this tile's map row into blist (the
  // tile pair of block b is 2b, 2b + 1). Every wave counts; wave 0 writes the list.
  int n_t = je - jb;
  const bool sparse = MASKED && p.block_mask != nullptr;
  if (sparse) {
    const int nblk = (n_kv + 1) / 2;
    const uint8_t* mrow = p.block_mask + ((size_t)head * p.n_qt + qt) * p.n_kb;
    int cnt = 0;
    for (int b0 = 0; b0 < nblk; b0 += 64) {
      const int b = b0 + l;
      const bool on = b < nblk && mrow[b] != 0;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(on);
      if (w == 0 && on)
        blist[cnt + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0))] = b;
      cnt += __builtin_popcountll(bal);
    }
    __syncthreads();
    if (cnt == 0) {
      write_empty_rows();
      write_carried_rows();
      return;
    }
    n_t = 2 * cnt;
  }
  // Split launches: this wave pair's tiles stream, stream + 2, ...; both pairs run as many loop
  // positions as the even tiles need (the odd pair's last one may be padding).
  int n_loop = n_t;
  if (QSPLIT) {
    n_t = (n_kv - stream + 1) / 2;
    n_loop = (n_kv + 1) / 2;
  }
  // Tile index of loop position u. Positions past the end (the pipeline's look-ahead) map to a
  // tile beyond every key this workgroup can see: fully masked and never loaded.
  auto tile = [&](int u) __attribute__((always_inline)) -> int {
    if (QSPLIT) return 2 * u + stream;
    if (!sparse) return jb + u;
    if (u >= n_t) return n_kv + 2;
    return 2 * __builtin_amdgcn_readfirstlane(blist[u >> 1]) + (u & 1);
  };

  // Byte offsets (within a tile) of the 16-byte chunks this lane deposits: DMA instruction i of
  // loading wave wl (one of the NW waves, or of a split launch's pair) fills LDS chunk positions
  // (wl + DW*i)*64 + lane, i.e. swizzled (row, chunk) slots. Tiles past the end of the head load
  // zeros.
  int goff[NLDW];
#pragma unroll
  for (int i = 0; i < NLDW; ++i) {
    const int pos = (wl + DW * i) * 64 + l;
    const int row = pos / NCH, pc = pos % NCH;
    goff[i] = row * (D * 2) + ((pc ^ T::swz(row)) * 16);
  }
  // A key-split launch with one query tile per head reads each K/V tile exactly once (decoding):
  // those loads are marked non-temporal so the streamed cache does not crowd the caches. Where
  // several query tiles share a head's K/V (dense, masked, or longer key-split launches), the
  // tiles are re-read through L2 and keep the default policy.
  auto dma = [&](const E* src, int j, char* dst) __attribute__((always_inline)) {
    const int key0 = j * BC;
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(BC, Lk - key0)));
    const __amdgpu_buffer_rsrc_t r = make_rsrc(src + (size_t)min(key0, Lk) * D, rows * (D * 2));
    if (KV_SPLIT && p.kv_once) {
#pragma unroll
      for (int i = 0; i < NLDW; ++i) buf_load16_to_lds_once(r, dst + (wl + DW * i) * 1024, goff[i]);
    } else {
#pragma unroll
      for (int i = 0; i < NLDW; ++i) buf_load16_to_lds(r, dst + (wl + DW * i) * 1024, goff[i]);
    }
  };

  // Lane-constant parts of the LDS read addresses.
  const int g16 = l >> 4, j16 = l & 15;
  const int v_row_lane = 4 * hf + (j16 >> 2);
  const int v_col_lane = 16 * (g16 & 1) + 4 * (j16 & 3);
  const int key_lim = CAUSAL ? min(q + koff, key_end - 1) : key_end - 1;

  f32x16 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x16{};
  float m_run = kInitMax, l_run = 0.f, lr_run = 0.f;
  const float c = p.c;

  // S^T for the 32-key half `h` of a K tile.
  auto s_half = [&](f32x16& s, const char* kbuf, int h) __attribute__((always_inline)) {
    s = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      s = H::mfma(lds_read16<E>(kbuf, T::chunk_off(32 * h + lq, 2 * kk + hf)), qreg[kk], s);
  };
  // Causal / ragged mask of the 32-key half `h` of tile j (only where it can bite).
  auto mask_half = [&](f32x16& s, int j, int h) __attribute__((always_inline)) {
    const int key0 = j * BC + 32 * h;
    if ((key0 + 32 > key_end) || (CAUSAL && key0 + 31 > q_w0 + koff)) {
      const int lim = key_lim - key0 - 4 * hf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int krel = (r >> 2) * 8 + (r & 3);
        s[r] = krel <= lim ? s[r] : -INFINITY;
      }
    }
  };
  f32x16 s0, s1;
  e16x8 p0[2], p1[2];
  float rs, rr;
  // One pipeline phase: NS = NKK MFMAs of S^T for K half `hs` (into s_out; none without with_s),
  // NPV = 2 * NDB MFMAs of O^T += V^T P^T for V half `hv` (from p_in), and the probabilities of s_in
  // (into p_out), with their fp32 sum in rs and the sum of their 16-bit roundings in rr. The work is
  // issued in a fixed interleave, fenced by scheduling barriers.
  uint32_t kw[4];  // dropout: the Philox words of the half whose probabilities are being formed
  auto phase = [&](auto with_pv, auto with_s, f32x16& s_out, const char* kbuf, int hs, const e16x8 (&p_in)[2],
                   const char* vbuf, int hv, const f32x16& s_in, e16x8 (&p_out)[2], int jh) __attribute__((always_inline)) {
    constexpr bool PV = decltype(with_pv)::value;
    if constexpr (DROPOUT) dropout_words(q, jh, head, hf, p.seed_lo, p.seed_hi, kw);
    constexpr int NS = decltype(with_s)::value ? NKK : 0, NPV = PV ? 2 * NDB : 0, NM = NS + NPV;
    auto frag = [&](int i) __attribute__((always_inline)) -> e16x8 {
      if (i < NS) return lds_read16<E>(kbuf, T::chunk_off(32 * hs + lq, 2 * i + hf));
      const int t = (i - NS) / NDB, db = (i - NS) % NDB, ks = 2 * hv + t;
      const int col = 32 * db + v_col_lane;
      const e16x4 a0 = lds_read_tr16<E>(vbuf, T::elem_off(16 * ks + v_row_lane, col));
      const e16x4 a1 = lds_read_tr16<E>(vbuf, T::elem_off(16 * ks + 8 + v_row_lane, col));
      return cat4<E>(a0, a1);
    };
    const float neg_m = -m_run;
    float a0 = 0.f, a1 = 0.f, r0 = 0.f;
    // Element k of the 16 probabilities goes through three stages, each in a later matrix step
    // than the previous so no stage waits on the latency of the one before: x = s*c - m,
    // p = exp2(x), then the sums and (odd k) the 16-bit pair.
    float xv[16], pv[16];
    auto st_fma = [&](int k) __attribute__((always_inline)) {
      xv[k] = fmaf(s_in[k], c, neg_m);
      asm volatile("" ::"v"(xv[k]));
    };
    auto st_exp = [&](int k) __attribute__((always_inline)) {
      pv[k] = fast_exp2(xv[k]);
      asm volatile("" ::"v"(pv[k]));
    };
    auto st_acc = [&](int k) __attribute__((always_inline)) {
      const int t = k >> 3, e = k & 7;
      if ((k & 1) == 0) {
        a0 = k == 0 ? pv[k] : a0 + pv[k];
        asm volatile("" ::"v"(a0));
      } else {
        a1 = k == 1 ? pv[k] : a1 + pv[k];
        e16x2 pr = {(E)pv[k - 1], (E)pv[k]};
        r0 = H::dot2_ones(pr, r0);  // l~ sums the undropped probabilities
        if constexpr (DROPOUT)
          pr = __builtin_bit_cast(e16x2, __builtin_bit_cast(uint32_t, pr) & dropout_pair_mask(kw[k >> 2], (k >> 1) & 1, p.drop_thr2));
        p_out[t][e - 1] = pr[0];
        p_out[t][e] = pr[1];
        asm volatile("" ::"v"(a1), "v"(r0), "v"(pr));
      }
    };
    constexpr int PF = 4;          // LDS fragment prefetch distance (matrix steps)
    constexpr int NSTEP = NM + 2;  // two extra steps drain the element pipeline
    // Matrix step i issues slot(i) (slots 0 .. NS-1 are S, NS .. NM-1 are P V). At d <= 64 the S
    // and P V instructions alternate, so none waits on the accumulator the one before it wrote
    // (measured 3-5% faster there; at larger d the plain order is as fast or faster).
    constexpr int NMIN = NS < NPV ? NS : NPV;
    auto slot = [](int i) constexpr -> int {
      if (D > 64) return i;
      return i < 2 * NMIN ? ((i & 1) ? NS + (i >> 1) : (i >> 1)) : (NS > NPV ? i - NMIN : NS + (i - NMIN));
    };
    e16x8 fr[NM];
#pragma unroll
    for (int i = 0; i < PF && i < NM; ++i) fr[i] = frag(slot(i));
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
      if (i + PF < NM) fr[i + PF] = frag(slot(i + PF));
      if (i < NM) {
        const int u = slot(i);
        if (u < NS) {
          s_out = H::mfma(fr[i], qreg[u], u == 0 ? f32x16{} : s_out);
        } else {
          const int t = (u - NS) / NDB, db = (u - NS) % NDB;
          acc_o[db] = H::mfma(fr[i], p_in[t], acc_o[db]);
        }
      }
      // element work per step: stage f of element k runs at step (k * NM / 16) + f
      // (stages: 0 fma, 1 exp, 2 sums)
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int s0_ = k * NM / 16;
        if (s0_ + 2 == i) st_acc(k);
        if (s0_ + 1 == i) st_exp(k);
        if (s0_ == i) st_fma(k);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    rs = a0 + a1;
    rr = r0;
    // keep the fast-path results in this block (not sunk past the overflow check)
    asm volatile("" : "+v"(p_out[0]), "+v"(p_out[1]), "+v"(rs), "+v"(rr));
  };
  // Slow-path recomputation of one half's probabilities against the current m.
  auto probs = [&](const f32x16& s, e16x8 (&pk)[2], float& rs_, float& rr_) __attribute__((always_inline)) {
    const float neg_m = -m_run;
    float a0 = 0.f, a1 = 0.f, r0 = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float pa = fast_exp2(fmaf(s[8 * t + e], c, neg_m));
        const float pb = fast_exp2(fmaf(s[8 * t + e + 1], c, neg_m));
        a0 += pa;
        a1 += pb;
        e16x2 pr = {(E)pa, (E)pb};
        r0 = H::dot2_ones(pr, r0);
        if constexpr (DROPOUT)
          pr = __builtin_bit_cast(e16x2, __builtin_bit_cast(uint32_t, pr) & dropout_pair_mask(kw[t * 2 + (e >> 2)], (e >> 1) & 1, p.drop_thr2));
        pk[t][e] = pr[0];
        pk[t][e + 1] = pr[1];
      }
    rs_ = a0 + a1;
    rr_ = r0;
  };
  // Accept a half's probabilities, or (some lane's sum above kOverflowSum<E>) raise m to the half's
  // max for the affected rows (both lanes of a row decide together), rescale O, l and l~, and
  // recompute the half.
  auto settle = [&](const f32x16& s, e16x8 (&pk)[2]) __attribute__((always_inline)) {
    if (__builtin_amdgcn_ballot_w64(rs > kOverflowSum<E>)) {
      const float trig = half_swap_max(rs > kOverflowSum<E> ? 1.f : 0.f);
      float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; r += 4) {
        mx0 = vmax3(mx0, s[r], s[r + 1]);
        mx1 = vmax3(mx1, s[r + 2], s[r + 3]);
      }
      const float mx = half_swap_max(vmax(mx0, mx1)) * c;
      const float m_new = trig > 0.5f ? vmax(m_run, mx) : m_run;
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
      lr_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc_o[db] *= alpha;
      probs(s, pk, rs, rr);
    }
    l_run += rs;
    lr_run += rr;
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  auto phase_a = [&](int j, const char* kbuf, const char* vprev, auto with_pv) __attribute__((always_inline)) {
    mask_half(s0, j, 0);
    phase(with_pv, yes{}, s1, kbuf, 1, p1, vprev, 1, s0, p0, 2 * j);
    settle(s0, p0);
  };
  // with_s = no: the last tile's B phase, with no scores of a following tile to start.
  auto phase_b = [&](int j, const char* knext, const char* vcur, auto with_s) __attribute__((always_inline)) {
    mask_half(s1, j, 1);
    phase(yes{}, with_s, s0, knext, 0, p0, vcur, 0, s1, p1, 2 * j + 1);
    settle(s1, p1);
  };
  // O^T += V^T P^T for V half `hv` alone (the pipeline's drain after the last tile).
  auto pv_only = [&](const char* vbuf, int hv, const e16x8 (&p_in)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2 * NDB; ++i) {
      const int t = i / NDB, db = i % NDB, ks = 2 * hv + t;
      const int col = 32 * db + v_col_lane;
      const e16x4 a0 = lds_read_tr16<E>(vbuf, T::elem_off(16 * ks + v_row_lane, col));
      const e16x4 a1 = lds_read_tr16<E>(vbuf, T::elem_off(16 * ks + 8 + v_row_lane, col));
      acc_o[db] = H::mfma(cat4<E>(a0, a1), p_in[t], acc_o[db]);
    }
  };
  // K(j) and V(j) live in buffer j % 2. K(j+2) / V(j+1) are issued right after the barrier that
  // follows phase A(j), the last reader of K(j) and V(j-1), and are awaited one tile later. The
  // tile count is padded to even; a padded tile is fully masked (its probabilities are zero) and
  // its V rows are real data or zeros, so it leaves O and l unchanged.
  if constexpr (QSPLIT) {
    // Each wave pair runs the tile loop below on its own buffers. (The plain launches keep the loop
    // written out on their four buffers: bound through this lambda, the compiler allocates their
    // registers worse, one wave per SIMD fewer at d = 64.)
    auto main_loop = [&](char* K0, char* V0, char* K1, char* V1) __attribute__((always_inline)) {
      const int n_eff = (n_loop + 1) & ~1;
      const int j_first = tile(0);
      dma(Kh, j_first, K0);
      dma(Vh, j_first, V0);
      if (n_t > 1) dma(Kh, tile(1), K1);
      wait_vmem();
      __syncthreads();
      s_half(s0, K0, 0);
      debug_stage_sync();
      phase_a(j_first, K0, V1, no{});
      debug_stage_sync();
#pragma unroll 1
      for (int t = 0; t < n_eff - 2; t += 2) {
        const int j0 = tile(t), j1 = tile(t + 1), j2 = tile(t + 2);
        wait_vmem();
        __syncthreads();
        if (t + 2 < n_t) dma(Kh, j2, K0);
        dma(Vh, j1, V1);
        debug_stage_sync();
        phase_b(j0, K1, V0, yes{});
        debug_stage_sync();
        phase_a(j1, K1, V0, yes{});
        debug_stage_sync();
        wait_vmem();
        __syncthreads();
        if (t + 3 < n_t) dma(Kh, tile(t + 3), K1);
        dma(Vh, j2, V0);
        debug_stage_sync();
        phase_b(j1, K0, V1, yes{});
        debug_stage_sync();
        phase_a(j2, K0, V1, yes{});
        debug_stage_sync();
      }
      {  // the last two tiles: the same steps without scoring a tile past the end
        const int t = n_eff - 2;
        const int j0 = tile(t), j1 = tile(t + 1);
        wait_vmem();
        __syncthreads();
        dma(Vh, j1, V1);
        debug_stage_sync();
        phase_b(j0, K1, V0, yes{});
        debug_stage_sync();
        phase_a(j1, K1, V0, yes{});
        debug_stage_sync();
        wait_vmem();
        __syncthreads();
        phase_b(j1, K0, V1, no{});
        debug_stage_sync();
        pv_only(V1, 1, p1);
      }
    };
    if (stream == 1) main_loop(skb0, svb0, skb1, svb1);
    else main_loop(sk0, sv0, sk1, sv1);
  } else {
    const int n_eff = (n_loop + 1) & ~1;
    const int j_first = tile(0);
    dma(Kh, j_first, sk0);
    dma(Vh, j_first, sv0);
    if (n_t > 1) dma(Kh, tile(1), sk1);
    wait_vmem();
    __syncthreads();
    s_half(s0, sk0, 0);
    debug_stage_sync();
    phase_a(j_first, sk0, sv1, no{});
    debug_stage_sync();
#pragma unroll 1
    for (int t = 0; t < n_eff - 2; t += 2) {
      const int j0 = tile(t), j1 = tile(t + 1), j2 = tile(t + 2);
      wait_vmem();
      __syncthreads();
      if (t + 2 < n_t) dma(Kh, j2, sk0);
      dma(Vh, j1, sv1);
      debug_stage_sync();
      phase_b(j0, sk1, sv0, yes{});
      debug_stage_sync();
      phase_a(j1, sk1, sv0, yes{});
      debug_stage_sync();
      wait_vmem();
      __syncthreads();
      if (t + 3 < n_t) dma(Kh, tile(t + 3), sk1);
      dma(Vh, j2, sv0);
      debug_stage_sync();
      phase_b(j1, sk0, sv1, yes{});
      debug_stage_sync();
      phase_a(j2, sk0, sv1, yes{});
      debug_stage_sync();
    }
    {  // the last two tiles: the same steps without scoring a tile past the end
      const int t = n_eff - 2;
      const int j0 = tile(t), j1 = tile(t + 1);
      wait_vmem();
      __syncthreads();
      dma(Vh, j1, sv1);
      debug_stage_sync();
      phase_b(j0, sk1, sv0, yes{});
      debug_stage_sync();
      phase_a(j1, sk1, sv0, yes{});
      debug_stage_sync();
      wait_vmem();
      __syncthreads();
      phase_b(j1, sk0, sv1, no{});
      debug_stage_sync();
      pv_only(sv1, 1, p1);
    }
  }
  if constexpr (QSPLIT) {
    // The odd-tile pair hands (m, l, l~, O) to the even-tile pair, which merges them:
    // m = max(m_a, m_b), each part scaled by exp2(m_x - m) (the online-softmax block merge).
    static_assert(NDB * 4 * 64 * 16 <= TILE_BYTES && 3 * 64 * 4 <= TILE_BYTES, "exchange fits a tile buffer");
    __syncthreads();  // every wave is done reading its last K/V tiles
    f32x4* xo = reinterpret_cast<f32x4*>(wl ? skb1 : skb0);
    float* xs = reinterpret_cast<float*>(wl ? svb1 : svb0);
    if (stream == 1) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          xo[(4 * db + q4) * 64 + l] = f32x4{acc_o[db][4 * q4], acc_o[db][4 * q4 + 1], acc_o[db][4 * q4 + 2], acc_o[db][4 * q4 + 3]};
      xs[l] = m_run;
      xs[64 + l] = l_run;
      xs[128 + l] = lr_run;
    }
    __syncthreads();
    if (stream == 1) return;  // (no workgroup barrier follows)
    const float mb = xs[l], m_new = vmax(m_run, mb);
    const float aa = fast_exp2(m_run - m_new), ab = fast_exp2(mb - m_new);
    m_run = m_new;
    l_run = l_run * aa + xs[64 + l] * ab;
    lr_run = lr_run * aa + xs[128 + l] * ab;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 t = xo[(4 * db + q4) * 64 + l];
#pragma unroll
        for (int e = 0; e < 4; ++e) acc_o[db][4 * q4 + e] = acc_o[db][4 * q4 + e] * aa + t[e] * ab;
      }
  }

  // Epilogue: O = O_acc / l~, LSE = ln2 * (m + log2 l). The accumulator holds one query row per
  // lane, so O is staged through LDS (each wave in one of the now idle tile buffers, rows padded
  // by 16 bytes) and written back as whole rows of 16-byte chunks. Rows >= N fall outside the
  // buffer descriptors and are dropped.
  const float l_tot = half_swap_sum(l_run);
  if (KV_SPLIT && !(split_direct_ok(D) && p.kv_direct)) {
    // fp32 partial: O_s = O_acc / l~ and LSE_s; a row with no visible key in this split (l~ = 0)
    // gets O_s = 0, LSE_s = -inf, so the merge gives it no weight. Lane (q, hf) holds columns
    // 32*db + 8*g + 4*hf .. +3 of row q.
    const float lr = half_swap_sum(lr_run);
    const bool empty = lr == 0.f;
    const float inv = empty ? 0.f : 1.0f / lr;
    const size_t row0 = ((size_t)blockIdx.y * p.nh + head) * N;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(p.opart + row0 * D, N * D * 4);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = acc_o[db][4 * g + e] * inv;
        buf_store16(ro, (q * D + 32 * db + 8 * g + 4 * hf) * 4, __builtin_bit_cast(u32x4, t));
      }
    if (hf == 0) {
      const __amdgpu_buffer_rsrc_t rl = make_rsrc(p.lsepart + row0, N * 4);
      buf_store4(rl, q * 4, empty ? -INFINITY : (m_run + __log2f(l_tot)) * kLn2);
    }
    return;
  }
  float inv = 1.0f / half_swap_sum(lr_run);
  float lse_row = (m_run + __log2f(l_tot)) * kLn2;
  if (MASKED || KV_SPLIT) {
    // padding rows, and rows whose visible keys all fell in disabled blocks or the causal mask
    // (key-split: a cache shorter than the row's position)
    const bool empty = q >= Lq || half_swap_sum(lr_run) == 0.f;
    if (DROPOUT) inv *= p.drop_scale;
    inv = empty ? 0.f : inv;
    lse_row = empty ? -INFINITY : lse_row;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc_o[db][r] = empty ? 0.f : acc_o[db][r];
  }
  if (!QSPLIT) __syncthreads();  // every wave is done reading the last K/V tiles (split: merged above)
  char* ostage = w == 0 ? sk0 : (w == 1 ? sv0 : (w == 2 ? sk1 : sv1));
  store_rows_via_lds<E, D, TILE_BYTES>(ostage, acc_o, inv, make_rsrc(p.o + base, head_bytes), q_w0, l);
  if (p.lse && hf == 0) {
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(p.lse + (size_t)head * N, N * 4);
    buf_store4(rl, q * 4, lse_row);
  }
  write_carried_rows();
}

template <typename E, int D, int BC, int NW, bool CAUSAL, int MODE, bool QSPLIT = false>
static hipError_t launch_cfg(const Fwd16Params<E>& prm, int n_splits, hipStream_t stream) {
  hipLaunchKernelGGL((fwd16_kernel<E, D, BC, NW, CAUSAL, MODE, QSPLIT>), dim3(prm.n_qt * prm.nh, n_splits), dim3(NW * 64),
                     0, stream, prm);
  return hipGetLastError();
}

// Launch arguments beyond the dense forward's (key-split partials, masks).
struct FwdExtra {
  int Nk;
  int n_splits = 1;
  int tiles_per_split = 0;
  float* opart = nullptr;
  float* lsepart = nullptr;
  Masks masks;
  Dropout drop;
};

template <typename E, int MODE>
static hipError_t launch_typed(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N, int d,
                               float scale, bool causal, const FwdExtra& x, hipStream_t stream) {
  constexpr int NW = 4, BR = 32 * NW;
  Fwd16Params<E> prm;
  prm.q = static_cast<const E*>(q);
  prm.k = static_cast<const E*>(k);
  prm.v = static_cast<const E*>(v);
  prm.o = static_cast<E*>(o);
  prm.lse = lse;
  prm.N = N;
  prm.nh = BH;
  prm.n_qt = (N + BR - 1) / BR;
  // Scores are scale * q.k = |scale| * (sign(scale) q).k: the sign goes into Q (exact), the
  // magnitude into c. A zero scale uses a tiny c: every exp2 argument then rounds to 0, which is
  // exactly the uniform softmax a zero scale means, and masked scores still map to -inf.
  prm.c = scale == 0.f ? 1e-30f : fabsf(scale) * kLog2e;
  prm.qsign = scale < 0.f ? 0x80008000u : 0u;
  prm.Nk = x.Nk;
  prm.key_offset = x.Nk - N;
  prm.tiles_per_split = x.tiles_per_split;
  prm.opart = x.opart;
  prm.lsepart = x.lsepart;
  // Measured on decoding and chunked-prefill shapes (d = 128, 8192 keys): one query tile per head
  // gains 11-15% from non-temporal K/V loads, two to four are neutral, eight or more lose 3-15%.
  prm.kv_once = MODE == kSplit && prm.n_qt == 1;
  prm.kv_direct = MODE == kSplit && x.n_splits == 1 && split_direct_ok(d);
  prm.seqlens = x.masks.seqlens;
  prm.block_mask = x.masks.block_mask;
  prm.heads = x.masks.heads;
  prm.n_kb = (N + kMaskBlock - 1) / kMaskBlock;
  prm.seed_lo = (uint32_t)x.drop.seed;
  prm.seed_hi = (uint32_t)(x.drop.seed >> 32);
  prm.drop_thr2 = (uint32_t)x.drop.threshold | ((uint32_t)x.drop.threshold << 16);
  prm.drop_scale = x.drop.threshold > 0 ? 256.0f / (float)x.drop.threshold : 0.f;
  return with_head_dim(d, [&](auto dd) {
    constexpr int D = decltype(dd)::value;
    if constexpr (MODE == kDense && D <= 128) {
      // Small launch (no more 128-row tiles than CUs, half as many at d > 64, whose split
      // workgroups need 96-128 KB of LDS: one per CU; N >= 256): 64-row workgroups whose wave pairs
      // take the even and the odd K/V tiles (fwd16_kernel, QSPLIT), twice the workgroups, each
      // with half the key loop. Causal launches with up to twice as many tiles also take it when
      // their rows are long (N >= 4096 at d <= 64, N >= 2048 above): their longest rows then set
      // the launch's length (measured +7 to +26%; shorter rows lose up to 8%).
      const long tiles = (long)prm.n_qt * BH * (D > 64 ? 2 : 1), cus = device_cu_count();
      const bool long_causal = causal && tiles <= 2 * cus && N >= (D > 64 ? 2048 : 4096);
      if (N >= 256 && (tiles <= cus || long_causal)) {
        Fwd16Params<E> sp = prm;
        sp.n_qt = (N + 63) / 64;
        return causal ? launch_cfg<E, D, 64, NW, true, MODE, true>(sp, 1, stream)
                      : launch_cfg<E, D, 64, NW, false, MODE, true>(sp, 1, stream);
      }
    }
    return causal ? launch_cfg<E, D, 64, NW, true, MODE>(prm, x.n_splits, stream)
                  : launch_cfg<E, D, 64, NW, false, MODE>(prm, x.n_splits, stream);
  });
}

hipError_t launch_fwd_16(bool fp16, const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N,
                         int d, float scale, bool causal, hipStream_t stream) {
  FwdExtra x;
  x.Nk = N;
  return fp16 ? launch_typed<f16, kDense>(q, k, v, o, lse, BH, N, d, scale, causal, x, stream)
              : launch_typed<bf16, kDense>(q, k, v, o, lse, BH, N, d, scale, causal, x, stream);
}

hipError_t launch_fwd_16_masked(bool fp16, const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                                int N, int d, float scale, bool causal, const Masks& masks, const Dropout& drop,
                                hipStream_t stream) {
  FwdExtra x;
  x.Nk = N;
  x.masks = masks;
  x.drop = drop;
  if (drop.active())
    return fp16 ? launch_typed<f16, kMaskedDropout>(q, k, v, o, lse, BH, N, d, scale, causal, x, stream)
                : launch_typed<bf16, kMaskedDropout>(q, k, v, o, lse, BH, N, d, scale, causal, x, stream);
  return fp16 ? launch_typed<f16, kMasked>(q, k, v, o, lse, BH, N, d, scale, causal, x, stream)
              : launch_typed<bf16, kMasked>(q, k, v, o, lse, BH, N, d, scale, causal, x, stream);
}

// ---------------------------------------------------------------------------------------------
// Key-split forward: partials per split, then a merge.
// ---------------------------------------------------------------------------------------------
// One wave per query row: LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s (the same
// combination rule the online softmax applies to consecutive blocks, here across splits).
template <typename E, int D>
__global__ __launch_bounds__(256) void kvsplit_merge_kernel(const float* opart, const float* lsepart, E* o,
                                                            float* lse, int rows, int n_splits) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  if (row >= rows) return;
  const float ls = l < n_splits ? lsepart[(size_t)l * rows + row] : -INFINITY;
  float mx = ls;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if (mx == -INFINITY) {  // the row sees no key in any split (cache shorter than its position)
    for (int c = l; c < D; c += 64) o[(size_t)row * D + c] = (E)0.f;
    if (l == 0 && lse) lse[row] = -INFINITY;
    return;
  }
  // mx is finite here, or NaN from NaN inputs, which propagates
  float wgt = l < n_splits ? __expf(ls - mx) : 0.f;
  float sum = wgt;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
  wgt /= sum;
  constexpr int CPL = (D + 63) / 64;  // columns per lane: l, l + 64, ... below D
  float acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
  for (int sp = 0; sp < n_splits; ++sp) {
    const float ws = __shfl(wgt, sp);
    const float* src = opart + ((size_t)sp * rows + row) * D;
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      if (l + 64 * c < D) acc[c] += ws * src[l + 64 * c];
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c)
    if (l + 64 * c < D) o[(size_t)row * D + l + 64 * c] = (E)acc[c];
  if (l == 0 && lse) lse[row] = mx + __logf(sum);
}

template <typename E>
static hipError_t launch_split_typed(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N,
                                     int d, float scale, bool causal, const FwdExtra& x, hipStream_t stream) {
  hipError_t e = launch_typed<E, kSplit>(q, k, v, o, lse, BH, N, d, scale, causal, x, stream);
  if (e != hipSuccess || (x.n_splits == 1 && split_direct_ok(d))) return e;  // one split writes O and LSE itself
  const int n_splits = x.n_splits;
  float* opart = x.opart;
  float* lsepart = x.lsepart;
  const int rows = BH * N;
  const dim3 grid((rows + 3) / 4);
  return with_head_dim(d, [&](auto dd) {
    constexpr int D = decltype(dd)::value;
    hipLaunchKernelGGL((kvsplit_merge_kernel<E, D>), grid, dim3(256), 0, stream, opart, lsepart, static_cast<E*>(o),
                       lse, rows, n_splits);
    return hipGetLastError();
  });
}

hipError_t launch_fwd_16_kvsplit(bool fp16, const void* q, const void* k, const void* v, void* o, float* lse, int BH,
                                 int N, int Nk, int d, float scale, bool causal, int n_splits, int tiles_per_split,
                                 float* opart, float* lsepart, const int* seqlens_k, int heads, hipStream_t stream) {
  FwdExtra x;
  x.Nk = Nk;
  x.n_splits = n_splits;
  x.tiles_per_split = tiles_per_split;
  x.opart = opart;
  x.lsepart = lsepart;
  x.masks.seqlens = seqlens_k;
  x.masks.heads = heads;
  return fp16 ? launch_split_typed<f16>(q, k, v, o, lse, BH, N, d, scale, causal, x, stream)
              : launch_split_typed<bf16>(q, k, v, o, lse, BH, N, d, scale, causal, x, stream);
}

}  // namespace fa
