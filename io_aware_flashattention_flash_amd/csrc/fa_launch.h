// Internal host-side launch functions shared by the C-ABI entry points (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

// Block-sparse maps hold one byte per kMaskBlock x kMaskBlock block of scores; a workgroup keeps the
// list of its enabled blocks in LDS, which bounds the blocks per map row.
constexpr int kMaskBlock = 128;
constexpr int kMaxMaskBlocks = 1024;

// Optional masks (device pointers, or null). seqlens: [B] valid length of each sequence
// (sequence = head / heads). block_mask: [B*H][ceil(N/128)][ceil(N/128)] bytes, zero = skipped.
struct Masks {
  const int* seqlens = nullptr;
  const uint8_t* block_mask = nullptr;
  int heads = 1;
};

// Attention dropout: keep iff the element's Philox byte < threshold (256 keeps everything; the
// kernels then take their dropout-free path).
struct Dropout {
  uint64_t seed = 0;
  int threshold = 256;
  bool active() const { return threshold < 256; }
};

// Forward, 16-bit storage: bf16 (fp16 = false) or IEEE fp16 (fp16 = true). BH = B*H.
// d in {32, 64, 96, 128, 256} for every 16-bit launcher below.
hipError_t launch_fwd_16(bool fp16, const void* q, const void* k, const void* v, void* o, float* lse,
                         int BH, int N, int d, float scale, bool causal, hipStream_t stream);

// Forward with padding / block-sparse masks (16-bit storage; rows that see no key: O = 0,
// LSE = -inf).
hipError_t launch_fwd_16_masked(bool fp16, const void* q, const void* k, const void* v, void* o, float* lse,
                                int BH, int N, int d, float scale, bool causal, const Masks& masks,
                                const Dropout& drop, hipStream_t stream);

// Writes the dropout keep mask (1 kept, 0 dropped) of every score element, uint8 [BH][Nq][Nk].
hipError_t launch_dropout_mask(uint8_t* keep, int BH, int Nq, int Nk, const Dropout& drop, hipStream_t stream);

// Key-split forward (Nq = N query rows against Nk >= N key rows; causal: query i sees keys
// j <= i + L - N, L = the sequence's cache length, Nk without seqlens_k). The K/V tiles are dealt to
// n_splits groups of tiles_per_split tiles; each group's fp32 partial (O, LSE) goes to
// opart [n_splits][BH][N][d] / lsepart [n_splits][BH][N], then a merge kernel writes O and LSE.
hipError_t launch_fwd_16_kvsplit(bool fp16, const void* q, const void* k, const void* v, void* o, float* lse,
                                 int BH, int N, int Nk, int d, float scale, bool causal, int n_splits,
                                 int tiles_per_split, float* opart, float* lsepart, const int* seqlens_k,
                                 int heads, hipStream_t stream);

// Compute units of the current device (cached per device).
int device_cu_count();

// Forward, fp32 storage. d in {64, 128}.
hipError_t launch_fwd_fp32(const void* q, const void* k, const void* v, void* o, float* lse,
                           int BH, int N, int d, float scale, bool causal, hipStream_t stream);

// Backward stages, 16-bit storage (bf16 or fp16). delta: float32 [BH, N].
hipError_t launch_bwd_delta(bool fp16, const void* o, const void* dout, float* delta, int BH, int N, int d,
                            hipStream_t stream);
hipError_t launch_bwd_dkdv(bool fp16, const void* q, const void* k, const void* v, const float* lse,
                           const void* dout, const float* delta, void* dk, void* dv, int BH, int N,
                           int d, float scale, bool causal, hipStream_t stream);
hipError_t launch_bwd_dq(bool fp16, const void* q, const void* k, const void* v, const void* o,
                         const float* lse, const void* dout, float* delta, void* dq, int BH, int N,
                         int d, float scale, bool causal, hipStream_t stream);

// Full backward (dQ with delta, then dK/dV) under padding / block-sparse masks.
hipError_t launch_bwd_masked(bool fp16, const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, float* delta, void* dq, void* dk, void* dv,
                             int BH, int N, int d, float scale, bool causal, const Masks& masks,
                             const Dropout& drop, hipStream_t stream);

// Head dims of the 16-bit kernels: calls f(std::integral_constant<int, D>) for d in
// {32, 64, 96, 128, 256}; any other d is an invalid value.
template <typename F>
hipError_t with_head_dim(int d, F&& f) {
  switch (d) {
    case 32: return f(std::integral_constant<int, 32>{});
    case 64: return f(std::integral_constant<int, 64>{});
    case 96: return f(std::integral_constant<int, 96>{});
    case 128: return f(std::integral_constant<int, 128>{});
    case 256: return f(std::integral_constant<int, 256>{});
    default: return hipErrorInvalidValue;
  }
}

// Work decomposition shared by the kernels: workgroup id -> (head, tile).
// The hardware hands consecutive workgroup ids to the 8 XCDs round-robin, each with its own L2.
// When the head count is a multiple of 8, heads are dealt to XCDs so that all tiles of one head
// run on one XCD (its K/V stay in that XCD's L2).
//   kHeadMajor: within an XCD, one head's tiles after another (equal-cost tiles: keeps the
//               fewest heads in flight, best L2 reuse).
//   kLongestFirst: within an XCD, tile-major over its heads, tiles ordered from the most work to
//               the least (causal tiles: longest-processing-time-first dispatch, so the last
//               workgroups to start are the short ones and the kernel ends without a long tail).
//               `last_is_longest` says whether tile n_tiles-1 (forward, dQ) or tile 0 (dK/dV)
//               carries the most work.
enum class Order { kHeadMajor, kLongestFirst };
__device__ __forceinline__ void map_workgroup(int wg, int n_tiles, int nh, Order order, bool last_is_longest,
                                              int& head, int& tile) {
  int rank;
  if ((nh & 7) == 0) {
    const int xcd = wg & 7, pos = wg >> 3, hpx = nh >> 3;
    int t;
    if (order == Order::kLongestFirst) {
      t = pos % hpx;
      rank = pos / hpx;
    } else {
      t = pos / n_tiles;
      rank = pos - t * n_tiles;
    }
    head = xcd + 8 * t;
  } else if (order == Order::kLongestFirst) {
    head = wg % nh;
    rank = wg / nh;
  } else {
    head = wg / n_tiles;
    rank = wg - head * n_tiles;
  }
  tile = last_is_longest ? n_tiles - 1 - rank : rank;
}

// Work decomposition with per-sequence lengths (sequence b = head / heads, valid rows L_b; a tile
// of BR rows is padding when it starts at or past L_b). map_workgroup would interleave padding
// tiles, which finish at once, with long ones; the hardware dispatches a launch's workgroups in
// order and lets CUs idle behind such a mix (measured: a quarter of the slots on a length mix of
// [N/4, N]). Here every XCD takes the same heads as in map_workgroup (head = xcd + 8 t), runs all
// its tiles with work first, in the same order (longest-first: by tile index over its heads,
// descending when tile n_tiles-1 carries the most work, ascending when tile 0 does; head-major:
// tiles of one head after another), and then all its padding tiles.
// Applies when heads % 8 == 0 and there are at most 64 sequences (lane b of the wave holds
// sequence b's tile count); returns false otherwise, and the caller uses map_workgroup.
// Wave-uniform; every wave of the workgroup computes the same result.
__device__ __forceinline__ bool map_workgroup_varlen(int wg, int n_tiles, int nh, int heads, const int* seqlens,
                                                     int N, int BR, bool longest_first, bool last_is_longest,
                                                     int& head, int& tile) {
  const int nseq = nh / heads;
  if ((heads & 7) != 0 || nseq > 64) return false;
  const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0));
  int t_lane = 0;  // tiles with work of sequence `lane`
  if (lane < nseq) t_lane = (min(max(seqlens[lane], 0), N) + BR - 1) / BR;
  auto tiles_of = [&](int b) __attribute__((always_inline)) { return __builtin_amdgcn_readlane(t_lane, b); };
  const int x = wg & 7, hp8 = heads >> 3;  // heads of each sequence on this XCD: b*heads + x + 8j, j < hp8
  int pos = wg >> 3;
  if (longest_first) {
    for (int i = 0; i < n_tiles; ++i) {
      const int q = last_is_longest ? n_tiles - 1 - i : i;
      const uint64_t m = __builtin_amdgcn_ballot_w64(lane < nseq && t_lane > q);
      const int c = hp8 * __builtin_popcountll(m);
      if (pos < c) {
        int k = pos / hp8;
        uint64_t mm = m;
        for (; k > 0; --k) mm &= mm - 1;  // drop the k lowest sequences that have tile q
        head = __builtin_ctzll(mm) * heads + x + 8 * (pos % hp8);
        tile = q;
        return true;
      }
      pos -= c;
    }
  } else {
    for (int b = 0; b < nseq; ++b) {
      const int tb = tiles_of(b), c = hp8 * tb;
      if (pos < c) {
        head = b * heads + x + 8 * (pos / tb);
        tile = pos % tb;
        return true;
      }
      pos -= c;
    }
  }
  for (int b = 0; b < nseq; ++b) {  // padding tiles
    const int pb = n_tiles - tiles_of(b), c = hp8 * pb;
    if (pos < c) {
      head = b * heads + x + 8 * (pos / pb);
      tile = n_tiles - pb + pos % pb;
      return true;
    }
    pos -= c;
  }
  head = tile = 0;  // not reached: the grid holds n_tiles * nh workgroups
  return true;
}

}  // namespace fa
