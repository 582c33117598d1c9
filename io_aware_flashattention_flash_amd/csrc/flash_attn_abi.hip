// C-ABI entry points: argument validation, then dispatch to the kernels' launchers.
// Every check runs before anything is launched, so a call that returns an error status
// has launched nothing and written nothing. The library allocates nothing.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/flash_attn.h"
#include "fa_launch.h"

// Scratch of flash_attn_fwd_kvsplit_noalloc: a fixed device array, one copy per GPU the library
// runs on, held until the process ends. Host code never uses the array's name as an address: each
// device's address is looked up once (hipGetSymbolAddress, with that device current) and kept.
static __device__ __align__(256) char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices];  // guarded by g_scratch_mutex

// Address of the current device's scratch array (looked up on the first call on that device).
fa_status_t scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FA_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return FA_OK;
}
}  // namespace

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

fa_status_t check_shape(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_BAD_SHAPE;
  const int64_t elems = (int64_t)B * H * N * d;
  if (elems >= ((int64_t)1 << 31)) return FA_ERR_BAD_SHAPE;
  // One head is addressed with 32-bit byte offsets (buffer descriptors).
  if ((int64_t)N * d >= ((int64_t)1 << 29)) return FA_ERR_BAD_SHAPE;
  return FA_OK;
}

bool supported_d(int d) { return d == 32 || d == 64 || d == 96 || d == 128 || d == 256; }  // 16-bit paths
bool supported_d_fp32(int d) { return d == 64 || d == 128; }
bool is_16bit(int dtype) { return dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_FP16; }

}  // namespace

namespace fa {
// Compute units of the current device, cached per device. Concurrent first calls may each query
// the runtime, but every store and load of the cache is atomic.
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}
}  // namespace fa

namespace {
constexpr int kMaxSplits = 64;
constexpr int kQueryTile = 128;  // query rows per workgroup of the forward kernels
constexpr int kKeyTile = 64;     // keys per K/V tile

// Split plan of the key-split forward: `requested` splits (0 = enough to give every CU two
// workgroups), each covering a whole number of K/V tiles. Returns the number of splits used.
int kvsplit_plan(int BH, int Nq, int Nk, int requested, int* tiles_per_split) {
  const int n_qt = (Nq + kQueryTile - 1) / kQueryTile;
  const int n_tiles = (Nk + kKeyTile - 1) / kKeyTile;
  int s = requested;
  if (s == 0) {
    const long want = 2L * fa::device_cu_count();
    const long have = (long)n_qt * BH;
    s = (int)((want + have - 1) / have);
  }
  s = s < 1 ? 1 : (s > kMaxSplits ? kMaxSplits : s);
  if (s > n_tiles) s = n_tiles;
  const int tps = (n_tiles + s - 1) / s;
  *tiles_per_split = tps;
  return (n_tiles + tps - 1) / tps;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Block-sparse maps: the map row of a query tile must fit the kernels' LDS block list.
fa_status_t check_masks(int N, const int32_t* seqlens, const uint8_t* block_mask) {
  if (seqlens && !aligned4(seqlens)) return FA_ERR_MISALIGNED;
  if (block_mask && (N + fa::kMaskBlock - 1) / fa::kMaskBlock > fa::kMaxMaskBlocks) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Dropout probability -> keep threshold T = round(256 (1 - p)); T must be >= 1 (p below 511/512).
fa_status_t dropout_plan(float p, uint64_t seed, fa::Dropout* out) {
  if (!isfinite(p) || p < 0.f || p > 1.f) return FA_ERR_BAD_DROPOUT;
  const int t = (int)floor(256.0 * (1.0 - (double)p) + 0.5);
  if (t < 1) return FA_ERR_BAD_DROPOUT;
  out->seed = seed;
  out->threshold = t;
  return FA_OK;
}

fa_status_t check_kvsplit_shape(int B, int H, int Nq, int Nk, int d, int num_splits) {
  fa_status_t st = check_shape(B, H, Nq, d);
  if (st != FA_OK) return st;
  st = check_shape(B, H, Nk, d);
  if (st != FA_OK) return st;
  if (Nq > Nk || num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_BAD_SHAPE;
  return FA_OK;
}

// Argument checks of the key-split forward (everything but the workspace).
fa_status_t check_kvsplit_args(const void* q, const void* k, const void* v, const void* o, const float* lse, int B,
                               int H, int Nq, int Nk, int d, float scale, const int32_t* seqlens_k, int num_splits,
                               int dtype) {
  if (!q || !k || !v || !o) return FA_ERR_NULL_POINTER;
  fa_status_t st = check_kvsplit_shape(B, H, Nq, Nk, d, num_splits);
  if (st != FA_OK) return st;
  if (!is_16bit(dtype) || !supported_d(d)) return FA_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return FA_ERR_BAD_SCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned4(lse)) ||
      (seqlens_k && !aligned4(seqlens_k)))
    return FA_ERR_MISALIGNED;
  return FA_OK;
}

// Key-split forward with its fp32 partials in `workspace` (checked by the caller: large enough,
// 16-byte aligned). Every partial the merge reads is written by the split kernel first.
fa_status_t launch_kvsplit(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq,
                           int Nk, int d, float scale, int causal, const int32_t* seqlens_k, int num_splits,
                           void* workspace, int dtype, void* stream) {
  int tps = 0;
  const int s = kvsplit_plan(B * H, Nq, Nk, num_splits, &tps);
  const size_t rows = (size_t)s * B * H * Nq;
  float* opart = static_cast<float*>(workspace);
  float* lsepart = reinterpret_cast<float*>(static_cast<char*>(workspace) + round256(rows * d * sizeof(float)));
  hipError_t e = fa::launch_fwd_16_kvsplit(dtype == FA_DTYPE_FP16, q, k, v, o, lse, B * H, Nq, Nk, d, scale,
                                           causal != 0, s, tps, opart, lsepart, seqlens_k, H,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}
}  // namespace

extern "C" {

fa_status_t flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                           int d, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o) return FA_ERR_NULL_POINTER;
  fa_status_t st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (is_16bit(dtype) ? !supported_d(d) : (dtype != FA_DTYPE_FP32 || !supported_d_fp32(d))) return FA_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return FA_ERR_BAD_SCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned4(lse)))
    return FA_ERR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = is_16bit(dtype)
                     ? fa::launch_fwd_16(dtype == FA_DTYPE_FP16, q, k, v, o, lse, B * H, N, d, scale, causal != 0, s)
                     : fa::launch_fwd_fp32(q, k, v, o, lse, B * H, N, d, scale, causal != 0, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t flash_attn_fwd_kvsplit_workspace_size(int B, int H, int Nq, int Nk, int d, int num_splits, int dtype) {
  (void)dtype;
  if (check_kvsplit_shape(B, H, Nq, Nk, d, num_splits) != FA_OK) return 0;
  int tps = 0;
  const int s = num_splits == 0 ? kvsplit_plan(B * H, Nq, Nk, 0, &tps) : num_splits;
  const size_t rows = (size_t)s * B * H * Nq;
  return round256(rows * d * sizeof(float)) + round256(rows * sizeof(float));
}

fa_status_t flash_attn_fwd_masked(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                  int N, int d, float scale, int causal, const int32_t* seqlens,
                                  const uint8_t* block_mask, float dropout_p, uint64_t seed, int dtype,
                                  void* stream) {
  if (!q || !k || !v || !o) return FA_ERR_NULL_POINTER;
  fa_status_t st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (!is_16bit(dtype) || !supported_d(d)) return FA_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return FA_ERR_BAD_SCALE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned4(lse)))
    return FA_ERR_MISALIGNED;
  st = check_masks(N, seqlens, block_mask);
  if (st != FA_OK) return st;
  fa::Dropout drop;
  st = dropout_plan(dropout_p, seed, &drop);
  if (st != FA_OK) return st;
  fa::Masks m;
  m.seqlens = seqlens;
  m.block_mask = block_mask;
  m.heads = H;
  hipError_t e = fa::launch_fwd_16_masked(dtype == FA_DTYPE_FP16, q, k, v, o, lse, B * H, N, d, scale, causal != 0, m,
                                          drop, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t flash_attn_fwd_kvsplit(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                   int Nq, int Nk, int d, float scale, int causal, const int32_t* seqlens_k,
                                   int num_splits, void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  fa_status_t st = check_kvsplit_args(q, k, v, o, lse, B, H, Nq, Nk, d, scale, seqlens_k, num_splits, dtype);
  if (st != FA_OK) return st;
  if (!workspace || workspace_bytes < flash_attn_fwd_kvsplit_workspace_size(B, H, Nq, Nk, d, num_splits, dtype))
    return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_MISALIGNED;
  return launch_kvsplit(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, seqlens_k, num_splits, workspace, dtype,
                        stream);
}

fa_status_t flash_attn_fwd_kvsplit_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                           int H, int Nq, int Nk, int d, float scale, int causal,
                                           const int32_t* seqlens_k, int num_splits, int dtype, void* stream) {
  fa_status_t st = check_kvsplit_args(q, k, v, o, lse, B, H, Nq, Nk, d, scale, seqlens_k, num_splits, dtype);
  if (st != FA_OK) return st;
  if (flash_attn_fwd_kvsplit_workspace_size(B, H, Nq, Nk, d, num_splits, dtype) > FA_NOALLOC_SCRATCH_BYTES)
    return FA_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != FA_OK) return st;
  return launch_kvsplit(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, seqlens_k, num_splits, ws, dtype, stream);
}

size_t flash_attn_bwd_workspace_size(int B, int H, int N, int d, int dtype) {
  (void)dtype;
  if (check_shape(B, H, N, d) != FA_OK) return 0;
  const size_t bytes = (size_t)B * H * N * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

namespace {
// Checks shared by the backward entry points (16-bit types only).
fa_status_t check_bwd_common(int B, int H, int N, int d, float scale, int dtype) {
  fa_status_t st = check_shape(B, H, N, d);
  if (st != FA_OK) return st;
  if (!is_16bit(dtype) || !supported_d(d)) return FA_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return FA_ERR_BAD_SCALE;
  return FA_OK;
}
}  // namespace

fa_status_t flash_attn_bwd_delta(const void* o, const void* dout, float* delta, int B, int H, int N, int d,
                                 int dtype, void* stream) {
  if (!o || !dout || !delta) return FA_ERR_NULL_POINTER;
  fa_status_t st = check_bwd_common(B, H, N, d, 1.0f, dtype);
  if (st != FA_OK) return st;
  if (!aligned16(o) || !aligned16(dout) || !aligned4(delta)) return FA_ERR_MISALIGNED;
  hipError_t e = fa::launch_bwd_delta(dtype == FA_DTYPE_FP16, o, dout, delta, B * H, N, d, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t flash_attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                                const float* delta, void* dk, void* dv, int B, int H, int N, int d, float scale,
                                int causal, int dtype, void* stream) {
  if (!q || !k || !v || !lse || !dout || !delta || !dk || !dv) return FA_ERR_NULL_POINTER;
  fa_status_t st = check_bwd_common(B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dk) || !aligned16(dv) ||
      !aligned4(lse) || !aligned4(delta))
    return FA_ERR_MISALIGNED;
  hipError_t e = fa::launch_bwd_dkdv(dtype == FA_DTYPE_FP16, q, k, v, lse, dout, delta, dk, dv, B * H, N, d, scale,
                                     causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t flash_attn_bwd_dq(const void* q, const void* k, const void* v, const void* o, const float* lse,
                              const void* dout, float* delta, void* dq, int B, int H, int N, int d, float scale,
                              int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !delta || !dq) return FA_ERR_NULL_POINTER;
  fa_status_t st = check_bwd_common(B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned4(lse) || !aligned4(delta))
    return FA_ERR_MISALIGNED;
  hipError_t e = fa::launch_bwd_dq(dtype == FA_DTYPE_FP16, q, k, v, o, lse, dout, delta, dq, B * H, N, d, scale,
                                   causal != 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t flash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                           int B, int H, int N, int d, float scale, int causal, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL_POINTER;
  fa_status_t st = check_bwd_common(B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned4(lse))
    return FA_ERR_MISALIGNED;
  if (!workspace || workspace_bytes < flash_attn_bwd_workspace_size(B, H, N, d, dtype)) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* delta = static_cast<float*>(workspace);
  const bool fp16 = dtype == FA_DTYPE_FP16;
  hipError_t e = fa::launch_bwd_dq(fp16, q, k, v, o, lse, dout, delta, dq, B * H, N, d, scale, causal != 0, s);
  if (e == hipSuccess)
    e = fa::launch_bwd_dkdv(fp16, q, k, v, lse, dout, delta, dk, dv, B * H, N, d, scale, causal != 0, s);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t flash_attn_bwd_masked(const void* q, const void* k, const void* v, const void* o, const float* lse,
                                  const void* dout, void* dq, void* dk, void* dv, void* workspace,
                                  size_t workspace_bytes, int B, int H, int N, int d, float scale, int causal,
                                  const int32_t* seqlens, const uint8_t* block_mask, float dropout_p,
                                  uint64_t seed, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_NULL_POINTER;
  fa_status_t st = check_bwd_common(B, H, N, d, scale, dtype);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned4(lse))
    return FA_ERR_MISALIGNED;
  st = check_masks(N, seqlens, block_mask);
  if (st != FA_OK) return st;
  fa::Dropout drop;
  st = dropout_plan(dropout_p, seed, &drop);
  if (st != FA_OK) return st;
  if (!workspace || workspace_bytes < flash_attn_bwd_workspace_size(B, H, N, d, dtype)) return FA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return FA_ERR_MISALIGNED;
  fa::Masks m;
  m.seqlens = seqlens;
  m.block_mask = block_mask;
  m.heads = H;
  hipError_t e = fa::launch_bwd_masked(dtype == FA_DTYPE_FP16, q, k, v, o, lse, dout, static_cast<float*>(workspace),
                                       dq, dk, dv, B * H, N, d, scale, causal != 0, m, drop,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status_t flash_attn_dropout_mask(uint8_t* keep, int B, int H, int Nq, int Nk, float dropout_p, uint64_t seed,
                                    void* stream) {
  if (!keep) return FA_ERR_NULL_POINTER;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || (int64_t)B * H * Nq * Nk >= ((int64_t)1 << 40)) return FA_ERR_BAD_SHAPE;
  fa::Dropout drop;
  fa_status_t st = dropout_plan(dropout_p, seed, &drop);
  if (st != FA_OK) return st;
  hipError_t e = fa::launch_dropout_mask(keep, B * H, Nq, Nk, drop, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

const char* flash_attn_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL_POINTER: return "FA_ERR_NULL_POINTER: a required pointer is NULL";
    case FA_ERR_BAD_SHAPE: return "FA_ERR_BAD_SHAPE: B, H, N, d must be >= 1 and each tensor < 2^31 elements";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: (dtype, head dim, pass) not supported";
    case FA_ERR_BAD_SCALE: return "FA_ERR_BAD_SCALE: scale must be finite";
    case FA_ERR_MISALIGNED: return "FA_ERR_MISALIGNED: pointers must be 16-byte aligned (lse 4-byte)";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or smaller than flash_attn_bwd_workspace_size()";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported a launch error";
    case FA_ERR_BAD_DROPOUT: return "FA_ERR_BAD_DROPOUT: dropout_p must be finite and in [0, 511/512]";
    case FA_ERR_SCRATCH_LIMIT:
      return "FA_ERR_SCRATCH_LIMIT: the call needs more scratch than FA_NOALLOC_SCRATCH_BYTES; use the entry point "
             "that takes a workspace";
    default: return "unknown flash_attn status";
  }
}

}  // extern "C"
