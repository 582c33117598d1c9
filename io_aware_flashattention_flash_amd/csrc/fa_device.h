// Device-side building blocks for the gfx950 (CDNA4, wave64) attention kernels.
//
// Lane layouts below were measured on gfx950 with a probe kernel and are the
// contract every kernel in this library relies on:
//
//   v_mfma_f32_32x32x16_bf16 / _f16   C[32x32] += A[32x16] * B[16x32]
//     A: lane l holds row  (l % 32), 8 consecutive k of group (l / 32)
//     B: lane l holds col  (l % 32), 8 consecutive k of group (l / 32)
//     C: lane l holds col  (l % 32); accumulator register r holds
//        row (r / 4) * 8 + (l / 32) * 4 + (r % 4)
//   v_mfma_f32_32x32x2_f32     same A/B/C roles with one k per lane (k = l / 32)
//
//   ds_read_b64_tr_b16: within every group of 16 lanes, treat the 16 lanes'
//     8-byte reads as a 16 x 4 matrix M (row j = the 4 halfwords lane j
//     addressed); lane i of the group receives M[4e + i/4][i % 4], e = 0..3.
//
//   v_permlane32_swap(x, x) returns {x[l % 32], x[l % 32 + 32]} in every lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x4_lds __attribute__((ext_vector_type(4)));  // the transpose-read builtin's type
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) fp16x4_lds lds_f16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// The 16-bit storage element of the matrix path: bf16 or IEEE fp16. Both are two bytes, so tiles,
// swizzles and transpose reads are shared; they differ in the matrix instruction, the LDS
// transpose-read builtin, the float -> 16-bit conversion (a plain cast, round to nearest even) and
// the two-element dot product.
template <typename E>
struct Half16;
template <>
struct Half16<bf16> {
  using x8 = bf16x8;
  using x4 = bf16x4;
  using x2 = bf16x2;
  static __device__ __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ x4 read_tr(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p);
  }
  // p[0] + p[1] accumulated in fp32
  static __device__ __forceinline__ float dot2_ones(x2 p, float acc) {
    const x2 ones = {(bf16)1.0f, (bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(p, ones, acc, false);
  }
};
template <>
struct Half16<f16> {
  using x8 = f16x8;
  using x4 = f16x4;
  using x2 = f16x2;
  static __device__ __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ x4 read_tr(const char* p) {
    return __builtin_bit_cast(x4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_f16x4*)p));
  }
  static __device__ __forceinline__ float dot2_ones(x2 p, float acc) {
    const x2 ones = {(f16)1.0f, (f16)1.0f};
    return __builtin_amdgcn_fdot2(p, ones, acc, false);
  }
};

__device__ __forceinline__ f32x16 mfma_f32_32x32x2(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// NaN-propagating maximum (IEEE 754-2019 maximum): v_maximum3_f32 on gfx950, with no quieting
// of the inputs, unlike fmaxf.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(a, vmax(b, c)); }

// Max / sum of a lane value with the lane 32 apart (the other half of a 32-row block).
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_min(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and Shaw ("Parallel Random
// Numbers: As Easy as 1, 2, 3", SC 2011): ten rounds, each two 32 x 32 -> 64-bit products of
// counter words with fixed multipliers, the high halves xored with the other counter words and the
// key, the key advanced by two Weyl increments between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                              uint32_t k1, uint32_t (&out)[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    // Three-way xor. In the first two rounds parts of the counter may still be wave-uniform, and
    // the compiler folds those into scalar instructions; later rounds use one v_bitop3 (truth
    // table 0x96 = a ^ b ^ c) in place of two vector xors.
    const uint32_t n0 = r < 2 ? (uint32_t)(p1 >> 32) ^ c1 ^ k0 : __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = r < 2 ? (uint32_t)(p0 >> 32) ^ c3 ^ k1 : __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

// Attention dropout's random bytes. Score element (row i, key j) of flattened head bh uses byte
// j % 4 of word (j % 32) / 8 of Philox4x32-10 at counter (i, j / 32, bh, (j / 4) % 2) and key
// (seed low, seed high); it is kept iff that byte is below the threshold T = round(256 (1 - p)).
// In the transposed score layout (a lane holds query i and, for its half hf of a 32-key block,
// register r = 4 g + e holds key 8 g + 4 hf + e) one call gives the lane's 16 bytes: register r
// takes byte e of word g.
__device__ __forceinline__ void dropout_words(int row, int block32, int head, int half, uint32_t seed_lo,
                                              uint32_t seed_hi, uint32_t (&w)[4]) {
  philox4x32_10((uint32_t)row, (uint32_t)block32, (uint32_t)head, (uint32_t)half, seed_lo, seed_hi, w);
}
__device__ __forceinline__ bool dropout_keep(uint32_t word, int byte, int thr) {
  return (int)((word >> (8 * byte)) & 0xffu) < thr;
}
// 0xffff in each 16-bit half of a packed pair whose element is kept: the pair is bytes 2c, 2c + 1
// of `word`; thr2 = T | T << 16. (Byte minus T is negative iff kept; an arithmetic shift spreads
// the sign over the half.)
typedef short i16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t dropout_pair_mask(uint32_t word, int c, uint32_t thr2) {
  const uint32_t y = word >> (16 * c);
  const uint32_t x = (y & 0xffu) | ((y & 0xff00u) << 8);
  i16x2 d = __builtin_bit_cast(i16x2, x) - __builtin_bit_cast(i16x2, thr2);
  d = d >> (i16x2){15, 15};
  return __builtin_bit_cast(uint32_t, d);
}

// 16-byte global load / store helpers (addresses are 16-byte aligned by contract).
__device__ __forceinline__ u32x4 ld_global16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st_global16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Row-major 16-bit tile of ROWS x D in LDS, stored as 16-byte chunks with an XOR swizzle so that
// (a) 16 consecutive rows read at the same logical chunk, and (b) 4 consecutive rows times 4
// consecutive chunks (the transpose-read pattern), both land on distinct 16-byte bank groups.
//
// The XOR value depends on the head dim (chunks per row):
//   4, 8, 16 chunks: rows are grouped by 256-byte bank line; the value combines the row's line and
//                    quarter so both patterns above spread over all 16 bank groups;
//   12 chunks:       (row / 4) % 4 flips only the low two chunk bits (the row stays inside its 12
//                    chunks); the 192-byte row stride already puts 4 consecutive rows in distinct
//                    quarters of a bank line, and the XOR separates the 4 rows within a quarter;
//   32 chunks:       4 (row % 4) + (row / 4) % 4, a different low-4-bit value for each of 16 rows.
template <int D>
struct SwizzledTile {
  static constexpr int kChunks = D / 8;                       // 16-byte chunks per row
  static constexpr int kRowsPerLine = kChunks >= 16 ? 1 : 16 / kChunks;  // rows per 256-byte bank line
  static constexpr int kQuarter = kChunks / 4;
  static_assert(kChunks == 4 || kChunks == 8 || kChunks == 12 || kChunks == 16 || kChunks == 32,
                "D must be 32, 64, 96, 128 or 256");
  __device__ __forceinline__ static int swz(int row) {
    if constexpr (kChunks == 12) return (row >> 2) & 3;
    if constexpr (kChunks == 32) return 4 * (row & 3) + ((row >> 2) & 3);
    int m = row / kRowsPerLine;
    return 4 * (m % kQuarter) + (m / kQuarter) % 4;
  }
  // Byte offset of logical (row, chunk).
  __device__ __forceinline__ static int chunk_off(int row, int chunk) {
    return (row * kChunks + (chunk ^ swz(row))) * 16;
  }
  // Byte offset of element (row, col); col % 4 == 0 keeps an 8-byte read aligned.
  __device__ __forceinline__ static int elem_off(int row, int col) {
    return chunk_off(row, col >> 3) + (col & 7) * 2;
  }
};

// Buffer resources (V#) for bounds-checked loads/stores: an access at byte offset >= num_bytes
// reads zero / is dropped. Word 3 selects the raw 32-bit data format used for untyped access.
constexpr int kBufferWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, num_bytes, kBufferWord3);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ float buf_load4f(__amdgpu_buffer_rsrc_t r, int off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, int off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, int off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, int off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
// Global -> LDS without registers: lane l's 16 bytes at byte offset `off` land at lds_dst + 16*l
// (lds_dst must be wave-uniform; it is placed in M0). Out-of-range lanes deposit zeros.
__device__ __forceinline__ void buf_load16_to_lds(__amdgpu_buffer_rsrc_t r, char* lds_dst, int off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst, 16, off, 0, 0, 0);
}
// Wait until this wave's outstanding vector-memory operations (including LDS DMA) have completed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Race-guard build (compiled with -DFA_DEBUG_SYNC=1): every pipeline stage of the tiled kernels
// ends with all of the wave's memory operations complete (global, LDS and LDS DMA) and a workgroup
// barrier, so no stage overlaps another and every tile load is complete before any wave reads it.
// The stages compute exactly what they compute in the normal build, so both builds must give
// bitwise-equal results; a difference would expose a missing wait or barrier (a read racing the
// write that fills or overwrites a buffer). In the normal build this is nothing.
#ifndef FA_DEBUG_SYNC
#define FA_DEBUG_SYNC 0
#endif
__device__ __forceinline__ void debug_stage_sync() {
  if constexpr (FA_DEBUG_SYNC != 0) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
}

template <typename E>
__device__ __forceinline__ typename Half16<E>::x8 lds_read16(const char* base, int off) {
  return *reinterpret_cast<const typename Half16<E>::x8*>(base + off);
}
__device__ __forceinline__ void lds_write16(char* base, int off, u32x4 v) {
  *reinterpret_cast<u32x4*>(base + off) = v;
}
template <typename E>
__device__ __forceinline__ typename Half16<E>::x4 lds_read_tr16(const char* base, int off) {
  return Half16<E>::read_tr(base + off);
}

template <typename E>
__device__ __forceinline__ typename Half16<E>::x8 cat4(typename Half16<E>::x4 a, typename Half16<E>::x4 b) {
  return typename Half16<E>::x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Write a wave's 32 x D block from the MFMA accumulator layout (lane l holds row l % 32, and
// register r of block db holds column 32*db + 8*(r/4) + 4*(l/32) + r%4) to rows row0..row0+31 of a
// row-major 16-bit [rows, D] tensor (element E, rounded to nearest even), scaled by `mul`. The block is staged through `stage` (LDS
// owned by this wave, STAGE_BYTES long; rows padded by 16 bytes against bank conflicts; two
// passes of 16 rows when 32 rows do not fit) so global stores are whole rows of 16-byte chunks.
// Rows beyond the descriptor's range are dropped.
template <typename E, int D, int STAGE_BYTES>
__device__ __forceinline__ void store_rows_via_lds(char* stage, const f32x16 (&acc)[D / 32], float mul,
                                                   __amdgpu_buffer_rsrc_t r, int row0, int lane) {
  constexpr int PITCH = D * 2 + 16, NCH = D / 8;
  constexpr int ROWS = 32 * PITCH <= STAGE_BYTES ? 32 : 16;  // rows staged per pass
  static_assert(ROWS * PITCH <= STAGE_BYTES, "staging area too small");
  const int lq = lane & 31, hf = lane >> 5;
#pragma unroll
  for (int pass = 0; pass < 32 / ROWS; ++pass) {
    if ((lq / ROWS) == pass) {
      const int srow = lq % ROWS;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          typename Half16<E>::x4 t;
#pragma unroll
          for (int e = 0; e < 4; ++e) t[e] = (E)(acc[db][4 * g + e] * mul);
          *reinterpret_cast<typename Half16<E>::x4*>(stage + srow * PITCH + (32 * db + 8 * g + 4 * hf) * 2) = t;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes have landed
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < ROWS * NCH / 64; ++i) {
      const int x = lane + 64 * i, row = x / NCH, ch = x % NCH;
      buf_store16(r, (row0 + pass * ROWS + row) * (D * 2) + ch * 16,
                  *reinterpret_cast<const u32x4*>(stage + row * PITCH + ch * 16));
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // the staging area may be reused once the reads are done
    __builtin_amdgcn_wave_barrier();
  }
}


}  // namespace fa
