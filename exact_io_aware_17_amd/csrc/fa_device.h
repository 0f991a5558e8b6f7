// Device-side types and helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace fa {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float NEG_INF = -__builtin_huge_valf();
constexpr float POS_INF = __builtin_huge_valf();
constexpr float LN2 = 0.69314718055994530942f;
constexpr float LOG2E = 1.44269504088896340736f;

// Forward K/V tiles (rows of D 16-bit elements, D * 2 / 16 chunks of 16
// bytes). Chunk c of row `row` is stored at slot kslot(row, c) (K) or
// vslot(row, c) (V) of that row, a per-row permutation chosen so that the
// operand reads spread over all 64 LDS banks (4-byte banks; 16 lanes of a
// 16-byte read, or 32 lanes of an 8-byte read, per pass):
//  * K rows are read whole: 16 consecutive rows at one chunk;
//  * V rows are read transposed: 4 consecutive rows x 4 chunks per half-wave.
// Rows of 256 or 512 bytes (D = 128, 256) all start at bank 0 and share one
// pattern; 64-byte rows (D = 32) cycle through the banks every 4 rows, so
// K slots are XORed with row / 4; 192-byte rows (D = 96) have 12 chunks, so
// K slots are rotated by (row / 4) mod 4 instead (an XOR would leave the
// row). The V reads of D = 32 and 96 are conflict-free unpermuted.
template <int D>
__device__ __forceinline__ int kslot(int row, int c) {
  static_assert(D == 32 || D == 64 || D == 96 || D == 128 || D == 256, "head dimension");
  if constexpr (D >= 128) {
    return c ^ (row & 15);
  } else if constexpr (D == 64) {
    return c ^ ((row >> 1) & 7);
  } else if constexpr (D == 32) {
    return c ^ ((row >> 2) & 3);
  } else {
    return (c + ((row >> 2) & 3)) % 12;
  }
}
// The chunk stored at slot s of K row `row` (the inverse permutation).
template <int D>
__device__ __forceinline__ int kchunk(int row, int s) {
  if constexpr (D == 96) {
    return (s + 12 - ((row >> 2) & 3)) % 12;
  } else {
    return kslot<D>(row, s);  // an XOR is its own inverse
  }
}
template <int D>
__device__ __forceinline__ int vslot(int row, int c) {
  if constexpr (D >= 128) {
    return c ^ (4 * (row & 3));
  } else if constexpr (D == 64) {
    return c ^ (4 * ((row >> 1) & 1));
  } else {
    return c;
  }
}
template <int D>
__device__ __forceinline__ int vchunk(int row, int s) {
  return vslot<D>(row, s);  // an XOR or the identity: its own inverse
}

// Position of index x inside its 16-group of a transposed tile: bits 2 and 3
// swapped. This is the order in which a 32x32 MFMA accumulator holds the
// rows of its C tile when they are fed back as the 8-wide contraction slots
// of the next MFMA.
__device__ __forceinline__ int swap23(int x) {
  return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Round two floats to bf16 (round-to-nearest-even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(unsigned, r);
}

// Lanes l and l^32 share a row; permlane32_swap hands each lane the pair
// {x[l & 31], x[(l & 31) + 32]} in its two results, so the combinations below
// are bitwise identical on both lanes.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Low / high bf16 of a packed word, as raw 16-bit values.
__device__ __forceinline__ unsigned lo16(unsigned w) { return w & 0xffffu; }
__device__ __forceinline__ unsigned hi16(unsigned w) { return w >> 16; }

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// s_waitcnt vmcnt(0): this wave's outstanding global loads (and LDS DMAs) are done.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
// (i % 4) of the 8-byte rows loaded by lanes 4j + i/4 (j = 0..3), i.e. four
// lanes reading four consecutive rows hand every lane one column of them.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* lds) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)lds);
}

// Sum of a packed pair of bf16 values added to an fp32 accumulator (v_dot2c_f32_bf16).
__device__ __forceinline__ float add_bf16_pair(unsigned w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w),
                                         __builtin_bit_cast(bf16x2, 0x3F803F80u), acc, false);
}

// Sum of a packed pair of fp16 values added to an fp32 accumulator (v_dot2_f32_f16).
__device__ __forceinline__ float add_f16_pair(unsigned w, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), __builtin_bit_cast(f16x2, 0x3C003C00u),
                                acc, false);
}

// The 16-bit input element types: bf16 and fp16 share every kernel; only the
// matrix instruction, the rounding of fp32 values to the element type
// (round-to-nearest-even) and the pair sum differ.
template <typename T>
struct Elem;
template <>
struct Elem<__bf16> {
  typedef bf16x8 x8;
  static __device__ __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack(float a, float b) { return pack_bf16x2(a, b); }
  static __device__ __forceinline__ float add_pair(unsigned w, float acc) {
    return add_bf16_pair(w, acc);
  }
  static __device__ __forceinline__ float lo(unsigned w) { return __uint_as_float(w << 16); }
  static __device__ __forceinline__ float hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
};
template <>
struct Elem<_Float16> {
  typedef f16x8 x8;
  static __device__ __forceinline__ f32x16 mfma(x8 a, x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack(float a, float b) {
    f32x2 v = {a, b};
    f16x2 r = __builtin_convertvector(v, f16x2);
    return __builtin_bit_cast(unsigned, r);
  }
  static __device__ __forceinline__ float add_pair(unsigned w, float acc) {
    return add_f16_pair(w, acc);
  }
  static __device__ __forceinline__ float lo(unsigned w) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xffffu));
  }
  static __device__ __forceinline__ float hi(unsigned w) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
  }
};

// Raw buffer resource over `base` (byte offsets up to 2^31 - 1, no bounds
// checking beyond that; the caller keeps offsets inside its allocation).
typedef __amdgpu_buffer_rsrc_t buffer_rsrc;
__device__ __forceinline__ buffer_rsrc make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}

// Device-coherent 16-byte store / load (cache policy sc1, the encoding of
// agent-scope atomic accesses): visible to every XCD without a cache-wide
// write-back or invalidation.
constexpr int CPOL_SC1 = 16;
__device__ __forceinline__ void store_coherent16(f32x4 v, buffer_rsrc r, int byte_off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, CPOL_SC1);
}
__device__ __forceinline__ f32x4 load_coherent16(buffer_rsrc r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, CPOL_SC1);
}

// 16-byte buffer load into LDS (buffer_load_dwordx4 ... lds): lane l's 16
// bytes at byte offset voff of the resource land at lds + 16 * l. `lds`
// must be the same for the whole wave; completion is tracked by vmcnt.
__device__ __forceinline__ void dma16_buf(buffer_rsrc r, int voff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ void zero(f32x16& x) {
#pragma unroll
  for (int r = 0; r < 16; ++r) x[r] = 0.f;
}

}  // namespace dev
}  // namespace fa
