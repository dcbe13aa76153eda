// Device-side helpers shared by the bdstep kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bd {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// ---------------------------------------------------------------- cross-lane moves
// DPP moves inside a 16-lane row.  After the xor-1, xor-2, xor-4 (half-row mirror)
// and xor-8 (row mirror) steps every lane of a row holds the row's reduction; the
// four rows are then combined through readlane in a fixed order (0, 16, 32, 48), so
// every reduction here has one fixed association order: results are reproducible.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}

constexpr int kDppXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

__device__ __forceinline__ float readlane_f32(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// Wave-wide max of a float; the result is uniform (NaN inputs are ignored by fmaxf
// unless every input is NaN).
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  float r = fmaxf(readlane_f32(v, 0), readlane_f32(v, 16));
  r = fmaxf(r, readlane_f32(v, 32));
  return fmaxf(r, readlane_f32(v, 48));
}

// Wave-wide sum of a float in a fixed association order; the result is uniform.
__device__ __forceinline__ float wave_sum(float v) {
  v = v + dpp_f32<kDppXor1>(v);
  v = v + dpp_f32<kDppXor2>(v);
  v = v + dpp_f32<kDppHalfMirror>(v);
  v = v + dpp_f32<kDppMirror>(v);
  float r = readlane_f32(v, 0) + readlane_f32(v, 16);
  r = r + readlane_f32(v, 32);
  return r + readlane_f32(v, 48);
}

__device__ __forceinline__ int wave_min_i32(int v) {
  v = min(v, dpp_i32<kDppXor1>(v));
  v = min(v, dpp_i32<kDppXor2>(v));
  v = min(v, dpp_i32<kDppHalfMirror>(v));
  v = min(v, dpp_i32<kDppMirror>(v));
  int r = min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16));
  r = min(r, __builtin_amdgcn_readlane(v, 32));
  return min(r, __builtin_amdgcn_readlane(v, 48));
}

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0; }

// ---------------------------------------------------------------- Philox4x32-10
// Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11):
// ten rounds of the 4x32 S-P network; the key advances by the Weyl increments
// between rounds, the first round using the key as given.
struct Philox4 {
  uint32_t w[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    const uint32_t n3 = (uint32_t)p0;
    c0 = n0;
    c1 = n1;
    c2 = n2;
    c3 = n3;
  }
  Philox4 out;
  out.w[0] = c0;
  out.w[1] = c1;
  out.w[2] = c2;
  out.w[3] = c3;
  return out;
}

// Standard Gumbel draw from one Philox word: u = ((r >> 8) + 0.5) 2^-24 (exact in
// fp64, strictly inside (0, 1)), g = -ln(-ln u), all in fp64.
__device__ __forceinline__ double gumbel_from_word(uint32_t r) {
  const double u = ((double)(r >> 8) + 0.5) * 0x1p-24;
  return -log(-log(u));
}

}  // namespace bd
