// Device helpers shared by the HIP kernels of libbsfa (prefill and decode): vector
// types, wave reductions, scalar loads through the constant address space, and the
// register staging of 64-row K/V tiles. Internal; included inside namespace
// bsfa::{anonymous} by each kernel source.
#pragma once

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int BLK = 64;

// Order-preserving map of a float onto a signed int (for non-NaN values, -inf included),
// so maxima can be reduced with integer max, which needs no NaN canonicalisation.
__device__ __forceinline__ int f2ord(float x) {
  const int b = __float_as_int(x);
  return b ^ ((b >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float ord2f(int k) {
  return __int_as_float(k ^ ((k >> 31) & 0x7fffffff));
}

// Maximum over the 64 lanes of a wave, returned as a wave-uniform value: halves swapped
// across lane 32, then a DPP all-reduce inside each 16-lane row, then rows 0 and 1.
__device__ __forceinline__ float wave_max(float x) {
  int k = f2ord(x);
  const auto sw = __builtin_amdgcn_permlane32_swap(k, k, false, false);
  k = max((int)sw[0], (int)sw[1]);
  k = max(k, __builtin_amdgcn_update_dpp(0, k, 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  k = max(k, __builtin_amdgcn_update_dpp(0, k, 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  k = max(k, __builtin_amdgcn_update_dpp(0, k, 0x124, 0xF, 0xF, false));  // row_ror:4
  k = max(k, __builtin_amdgcn_update_dpp(0, k, 0x128, 0xF, 0xF, false));  // row_ror:8
  return ord2f(max(__builtin_amdgcn_readlane(k, 0), __builtin_amdgcn_readlane(k, 16)));
}

// {x[l], x[l ^ 32]} in some order, for every lane l.
__device__ __forceinline__ void pair32(float x, float& a, float& b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Read-only kernel inputs (block lists, thresholds) are read through the constant
// address space: with a wave-uniform index they become scalar loads, which wait on
// their own counter instead of the vector-memory counter the K/V prefetch uses.
template <typename T>
__device__ __forceinline__ T ldc(const T* p, int64_t i) {
  return ((const __attribute__((address_space(4))) T*)(p))[i];
}

// Byte i of a 4-byte aligned byte array, read as its aligned dword (a scalar load).
__device__ __forceinline__ int ldc_byte(const uint8_t* p, int64_t i) {
  const uint32_t w = ldc(reinterpret_cast<const uint32_t*>(p), i >> 2);
  return (int)((w >> (8 * (i & 3))) & 0xFFu);
}

// Bits [0, n) of a 64-bit word, n clamped to [0, 64].
__device__ __forceinline__ uint64_t bits_below(int64_t n) {
  n = n < 0 ? 0 : (n > 64 ? 64 : n);
  return n >= 64 ? ~0ull : ((1ull << n) - 1ull);
}

// LDS tiles are 64 rows x D bf16 with padded rows. K rows are D + 8 elements apart, so
// 16 consecutive rows at one column hit 16 distinct 4-bank groups. V rows are D + 32
// elements apart, so the four rows x 64 bytes that 32 lanes of a transpose read touch
// cover all 64 banks once. Every LDS read is one per-lane base address plus immediate
// offsets.
//
// K/V tiles are staged through registers with bounds-checked buffer loads: one 16-byte
// chunk per lane and instruction, with the tile's offset as the scalar offset, so the
// address math is a single scalar multiply per tile. A row at or past N reads as zeros
// (its scores are masked and its weights are zero).
template <int D, int NT>
struct Stage {
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int CPT = BLK * CPR / NT;  // chunks per thread
  static_assert(BLK * CPR % NT == 0, "tile chunks must divide evenly");
  uint32_t goff[CPT];  // byte offset of this thread's chunks inside a tile (global)

  __device__ __forceinline__ void init(int tid, int64_t sn) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = tid + i * NT;
      goff[i] = (uint32_t)((ch / CPR) * sn * 2 + (ch % CPR) * 16);
    }
  }
  __device__ __forceinline__ void load(u32x4_t (&r)[CPT], __amdgpu_buffer_rsrc_t rsrc,
                                       uint32_t tile_off) const {
#pragma unroll
    for (int i = 0; i < CPT; ++i)
      r[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                             rsrc, goff[i], tile_off, 0));
  }
  // Write the chunks into an LDS tile whose rows are ROW elements apart.
  template <int ROW>
  __device__ __forceinline__ static void store(uint16_t* tile, const u32x4_t (&r)[CPT],
                                               int tid) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = tid + i * NT;
      *reinterpret_cast<u32x4_t*>(tile + (ch / CPR) * ROW + (ch % CPR) * 8) = r[i];
    }
  }
};
