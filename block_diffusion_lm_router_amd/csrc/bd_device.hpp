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

// The fp32 value v as such, for a conversion to fp16 that must round this fp32 value: without
// the barrier the compiler may fuse the multiply or multiply-add that produced v into one
// mixed-precision instruction (v_fma_mixlo_f16) that rounds the exact result to fp16 once,
// which differs from fp32-then-fp16 rounding near ties.
__device__ __forceinline__ float keep_f32(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// The done gate of a denoising loop: a kernel given a driver state (int32 [4]; word 2 is the
// done flag the loop update sets) returns at once when the block is done, before touching
// anything.  The flag was written by an earlier launch on the stream, so a plain load sees it.
__device__ __forceinline__ bool gated_off(const int32_t* __restrict__ gate) {
  return gate != nullptr && gate[2] != 0;
}

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

// Inclusive prefix sum over the 64 lanes of a wave (every lane active).  Within each row of
// 16 lanes the value of the lane 1, 2, 4 and 8 places below is added (DPP row shifts); then
// the last lane of row 0 and of row 2 is added to rows 1 and 3 (row broadcast of lane 15),
// and the last lane of row 1 to rows 2 and 3 (row broadcast of lane 31).
__device__ __forceinline__ int wave_incl_scan_i32(int v) {
  const int lane = lane_id();
  const int rl = lane & 15;
  int t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  if (rl >= 1) v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  if (rl >= 2) v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  if (rl >= 4) v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  if (rl >= 8) v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x142, 0xf, 0xf, false);   // row_bcast:15
  if ((lane & 31) >= 16) v += t;
  t = __builtin_amdgcn_update_dpp(0, v, 0x143, 0xf, 0xf, false);   // row_bcast:31
  if (lane >= 32) v += t;
  return v;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Reorder 8 halves (h0..h7) to (h0,h4,h1,h5,h2,h6,h3,h7): the k-order in which the GEMMs'
// nibble dequantisation yields weights.
__device__ __forceinline__ u32x4_t permute8(u32x4_t v) {
  u32x4_t r;
  r[0] = __builtin_amdgcn_perm(v[2], v[0], 0x05040100u);
  r[1] = __builtin_amdgcn_perm(v[2], v[0], 0x07060302u);
  r[2] = __builtin_amdgcn_perm(v[3], v[1], 0x05040100u);
  r[3] = __builtin_amdgcn_perm(v[3], v[1], 0x07060302u);
  return r;
}

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
