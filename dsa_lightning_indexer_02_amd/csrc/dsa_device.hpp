// Device-side building blocks shared by the DSA kernels (gfx950 / CDNA4, wave64).
//
// MFMA operand layouts used throughout (16x16 tiles; lane l, group g = l / 16):
//  - A (M x K) and B (K x N) operands: lane l supplies row (A) / column (B) l % 16 and
//    a contiguous run of the contraction index starting at (run length) * g.  Only the
//    agreement between the A and B runs matters for a full-K dot product.
//  - C / D (16 x 16 fp32): lane l holds rows 4 g + r (r = 0..3) of column l % 16.
// 32x32x16 tiles (lane l, half h = l / 32): A / B lane l supplies row / column l % 32 and
// contraction indices 8 h + j (j = 0..7); C / D lane l holds element r (r = 0..15) at row
// 8 (r / 4) + 4 h + r % 4 of column l % 32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// FP8 (OCP E4M3) 16x16x128 MFMA, fp32 accumulate, no block scales.
__device__ __forceinline__ v4f mfma_fp8_16x16x128(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// The same product with E8M0 operand scales: lane l's byte sa (sb) multiplies the 32 A (B)
// elements it supplies, i.e. row (column) l % 16 of its k-block, by 2^(byte - 127).
__device__ __forceinline__ v4f mfma_fp8_16x16x128_scaled(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ v4f mfma_bf16_16x16x32(const s16x8& a, const s16x8& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_f16_16x16x32(const s16x8& a, const s16x8& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ v16f mfma_bf16_32x32x16(const s16x8& a, const s16x8& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ v16f mfma_f16_32x32x16(const s16x8& a, const s16x8& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);  // v_cvt_pk_bf16_f32: round to nearest even
}
// Two fp32 -> packed bf16 (a in the low half), one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, bf16x2_t));
}

// Order-preserving map of an fp32 score to uint32 (larger score -> larger key); -0.0 maps
// like +0.0 so that the two compare equal.
__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Physical block of a block-table entry: ids outside [0, num_blocks) (a caller error: the
// readers' precondition is that every entry covering a visible position lies in the pool) are
// redirected to block 0, so a bad table gives unspecified scores instead of an out-of-bounds read.
__device__ __forceinline__ int64_t safe_block(int32_t id, int64_t num_blocks) {
  return (uint32_t)id < (uint64_t)num_blocks ? (int64_t)id : 0;
}

// Physical row of logical position s in one sequence's paged storage.  A null table is
// the identity (contiguous storage).
struct RowMap {
  const int32_t* table;
  int32_t block_shift;  // log2(block size)
  int64_t num_blocks;   // pool size in blocks (table entries are clamped into it)
  __device__ __forceinline__ int64_t operator()(int64_t s) const {
    if (!table) return s;
    const int64_t blk = safe_block(table[s >> block_shift], num_blocks);
    return (blk << block_shift) | (s & ((1 << block_shift) - 1));
  }
};

// ---- LDS helpers
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One wave-wide global -> LDS transfer (gfx950 LDS DMA): lane l's 16 bytes at gaddr land at
// lds_base + 16 l.  Completion is tracked by the vector-memory counter.
__device__ __forceinline__ void lds_dma_16B(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(gaddr) : "memory");
}

// The same transfer from a scalar base address: lane l's 16 bytes at base + voff (32-bit per lane).
__device__ __forceinline__ void lds_dma_16B_sbase(const void* base, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff), "s"(base) : "memory");
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding): at most N operations pending.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most n (wave-uniform, 0 <= n) vector-memory operations of this wave are pending;
// n above 15 waits for 15.
__device__ __forceinline__ void vm_wait_pending(int n) {
  switch (n) {
    case 0: vm_wait<0>(); break;
    case 1: vm_wait<1>(); break;
    case 2: vm_wait<2>(); break;
    case 3: vm_wait<3>(); break;
    case 4: vm_wait<4>(); break;
    case 5: vm_wait<5>(); break;
    case 6: vm_wait<6>(); break;
    case 7: vm_wait<7>(); break;
    case 8: vm_wait<8>(); break;
    case 9: vm_wait<9>(); break;
    case 10: vm_wait<10>(); break;
    case 11: vm_wait<11>(); break;
    case 12: vm_wait<12>(); break;
    case 13: vm_wait<13>(); break;
    case 14: vm_wait<14>(); break;
    default: vm_wait<15>(); break;
  }
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16): within each group of 16 lanes, lane i
// receives element i % 4 of the four 16-bit words addressed by lanes 4 j + i / 4 of its group,
// j = 0..3.  With lane a of group g addressing row r0 + a / 4, columns c0 + 4 (a % 4) .. + 3 of a
// row-major 16-bit matrix, lane i receives column c0 + i at rows r0 .. r0 + 3.
__device__ __forceinline__ s16x4 lds_transpose_read16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

// Eight FP8 E4M3 codes (two dwords) -> eight bf16 values (exact: E4M3 values are bf16 values).
__device__ __forceinline__ s16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  s16x8 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t w = h ? hi : lo;
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);  // bytes 0, 1
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);   // bytes 2, 3
    r[4 * h + 0] = (short)(__float_as_uint(a[0]) >> 16);
    r[4 * h + 1] = (short)(__float_as_uint(a[1]) >> 16);
    r[4 * h + 2] = (short)(__float_as_uint(b[0]) >> 16);
    r[4 * h + 3] = (short)(__float_as_uint(b[1]) >> 16);
  }
  return r;
}

__device__ __forceinline__ float wave_sum_xor16_32(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

}  // namespace dsa
