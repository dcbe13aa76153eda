// Grouped W4A16 expert GEMMs on MFMA (gfx950): gate/up with the GeGLU epilogue, and down.
//
// Source: axe-diffusion-ksl-xe model card, "the kernels we built": the GEMM reads packed
// nibbles and dequantises them inline, one launch covers all experts, and the activation
// is folded into the first GEMM's epilogue; "requirements": asymmetric uint4, fp16 scale
// and zero-point per group along the contraction dim, two nibbles per byte.
//
// Work decomposition.  A block owns one work item (an expert and up to 32 of its routed
// tokens) and one tile of 128 weight rows: gate/up takes 64 gate rows and the 64 up rows
// that pair with them, so the GeGLU product is formed in registers; down takes 128
// consecutive output rows.  Each wave owns two 16-row sets.  The block streams every
// packed byte of its rows exactly once (8 bytes per lane per 64-group: one group of one
// row for four lanes), so the expert's weights cross HBM once per 32 tokens.
//
// MFMA layout (v_mfma_f32_16x16x32_f16).  A = activations (16 tokens x 32 k), B =
// dequantised weights (32 k x 16 rows), D = 16 tokens x 16 rows in fp32.  Lane (n, kb) =
// (lane % 16, lane / 16) supplies weight row n at k-slots 8kb..8kb+7 and receives D for
// tokens 4kb..4kb+3 of row n, so each lane needs one scale and one zero-point per group.
//
// Dequantisation.  One 32-bit word holds 8 nibbles k0..k7 (k0 lowest).  OR-ing 0x6400
// into a half whose low mantissa bits hold a nibble q gives the fp16 value 1024 + q; the
// masks 0x000F000F and 0x00F000F0 (and the same after >> 8) yield the pairs (k0,k4),
// (16k1,16k5), (k2,k6), (16k3,16k7).  One packed add of -(1024 + z) or one packed fma
// by 1/16 then -(64 + z) turns each pair into the exact fp16 values q - z.  The k-order
// of a lane's 8 weights is therefore (0,4,1,5,2,6,3,7); the activation tile in LDS is
// stored in the same order, so the contraction is unchanged.  The 64-group partial sums
// come out of MFMA in fp32 and are scaled by that group's fp16 scale in fp32.
//
// Pipeline.  The contraction dim is walked in stages of 4 groups (256 k).  While stage
// c is contracted, the packed bytes of stage c+1 are in flight in registers and the
// activations and scales/zero-points of stage c+1 are fetched into registers, then
// written to the other LDS buffer.  One barrier per stage.

#include "bd_device.hpp"
#include "bd_internal.hpp"

namespace bd {

namespace {

constexpr int kThreads = 256;
constexpr int kStageK = 256;                 // contraction entries per stage
constexpr int kStageGroups = kStageK / 64;   // 64-groups per stage
constexpr int kXStride = kStageK + 8;        // halves; 16-byte pad against bank aliasing
constexpr int kRowsPerBlock = 128;

struct GemmArgs {
  const uint8_t* q;        // [E][R][K/2]
  const uint16_t* scale;   // [E][R][K/64]
  const uint16_t* zero;    // [E][R][K/64]
  int K;                   // contraction dim
  int R;                   // rows per expert
  int d_ff;                // gate/up: first up row
  int top_k;
  const uint16_t* act;     // gate/up: x [T][K]; down: h [T*k][K] (bucket order, permuted k)
  const int32_t* perm;     // bucket position -> assignment t*k + j
  const int32_t* items;    // [0] = count, then (expert, first position, tokens)
  uint16_t* h_out;         // gate/up output [T*k][d_ff]
  float* o_out;            // down output [T*k][d_model]
  int out_ld;
};

__device__ __forceinline__ half8_t dequant8(uint32_t w, _Float16 zc1, _Float16 zc2) {
  const uint32_t kLo = 0x000F000Fu, kHi = 0x00F000F0u, kMagic = 0x64006400u;
  const uint32_t a = (w & kLo) | kMagic;
  const uint32_t b = (w & kHi) | kMagic;
  const uint32_t w8 = w >> 8;
  const uint32_t c = (w8 & kLo) | kMagic;
  const uint32_t d = (w8 & kHi) | kMagic;
  const half2_t z1 = {zc1, zc1};
  const half2_t z2 = {zc2, zc2};
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t ha = __builtin_bit_cast(half2_t, a) + z1;
  const half2_t hb = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, b), sixteenth, z2);
  const half2_t hc = __builtin_bit_cast(half2_t, c) + z1;
  const half2_t hd = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, d), sixteenth, z2);
  half8_t r;
  r[0] = ha[0];
  r[1] = ha[1];
  r[2] = hb[0];
  r[3] = hb[1];
  r[4] = hc[0];
  r[5] = hc[1];
  r[6] = hd[0];
  r[7] = hd[1];
  return r;
}

// Reorder 8 halves (h0..h7) to (h0,h4,h1,h5,h2,h6,h3,h7).
__device__ __forceinline__ uint4 permute8(uint4 v) {
  uint4 r;
  r.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);
  r.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);
  r.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);
  r.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);
  return r;
}

__device__ __forceinline__ float gelu_tanh(float a) {
  const float u = 0.7978845608028654f * fmaf(0.044715f * a, a * a, a);
  const float th = 1.f - 2.f / (1.f + __expf(2.f * u));
  return 0.5f * a * (1.f + th);
}

template <bool GATED>
__global__ __launch_bounds__(kThreads) void w4a16_gemm_kernel(GemmArgs a) {
  const int item = blockIdx.y;
  if (item >= a.items[0]) return;
  const int e = a.items[1 + 3 * item];
  const int pos0 = a.items[2 + 3 * item];
  const int mcount = a.items[3 + 3 * item];
  const int tile = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int kb = lane >> 4;
  const int G = a.K >> 6;
  const int NS = (G + kStageGroups - 1) / kStageGroups;
  const int nMT = (mcount + 15) >> 4;

  const int rA = GATED ? tile * 64 + wave * 16 + n : tile * kRowsPerBlock + wave * 32 + n;
  const int rB = GATED ? a.d_ff + rA : rA + 16;
  const size_t rowbytes = (size_t)(a.K >> 1);
  const uint8_t* __restrict__ qA = a.q + ((size_t)e * a.R + rA) * rowbytes + kb * 8;
  const uint8_t* __restrict__ qB = a.q + ((size_t)e * a.R + rB) * rowbytes + kb * 8;

  __shared__ __attribute__((aligned(16))) _Float16 xs[2][kItemTokens][kXStride];
  __shared__ __attribute__((aligned(16))) _Float16 szs[2][2][kRowsPerBlock][kStageGroups];

  // Staging roles: activations (row m, 32-half segment) and scale/zero (row slot, group pair).
  const int st_m = tid >> 3;
  const int st_seg = tid & 7;
  const uint16_t* xsrc = nullptr;
  if (st_m < mcount) {
    if (GATED) {
      const int tok = a.perm[pos0 + st_m] / a.top_k;
      xsrc = a.act + (size_t)tok * a.K + st_seg * 32;
    } else {
      xsrc = a.act + (size_t)(pos0 + st_m) * a.K + st_seg * 32;
    }
  }
  const int sz_r = tid >> 1;
  const int sz_gp = (tid & 1) * 2;
  int sz_row;
  {
    const int w = sz_r >> 5, b = (sz_r >> 4) & 1, nn = sz_r & 15;
    sz_row = GATED ? (b ? a.d_ff : 0) + tile * 64 + w * 16 + nn : tile * kRowsPerBlock + w * 32 + b * 16 + nn;
  }
  const uint16_t* __restrict__ ssrc = a.scale + ((size_t)e * a.R + sz_row) * G;
  const uint16_t* __restrict__ zsrc = a.zero + ((size_t)e * a.R + sz_row) * G;

  uint4 xr[4];
  uint32_t sr = 0, zr = 0;
  auto stage_load = [&](int c) {
    const int k0 = c * kStageK + st_seg * 32;
    if (xsrc != nullptr && k0 < a.K) {
#pragma unroll
      for (int i = 0; i < 4; ++i) xr[i] = *reinterpret_cast<const uint4*>(xsrc + c * kStageK + 8 * i);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) xr[i] = make_uint4(0, 0, 0, 0);
    }
    const int g0 = c * kStageGroups + sz_gp;
    const uint32_t s0 = g0 < G ? ssrc[g0] : 0u, s1 = g0 + 1 < G ? ssrc[g0 + 1] : 0u;
    const uint32_t z0 = g0 < G ? zsrc[g0] : 0u, z1 = g0 + 1 < G ? zsrc[g0 + 1] : 0u;
    sr = s0 | (s1 << 16);
    zr = z0 | (z1 << 16);
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 v = GATED ? permute8(xr[i]) : xr[i];
      *reinterpret_cast<uint4*>(&xs[buf][st_m][st_seg * 32 + 8 * i]) = v;
    }
    *reinterpret_cast<uint32_t*>(&szs[buf][0][sz_r][sz_gp]) = sr;
    *reinterpret_cast<uint32_t*>(&szs[buf][1][sz_r][sz_gp]) = zr;
  };

  uint2 nA0[kStageGroups], nB0[kStageGroups], nA1[kStageGroups], nB1[kStageGroups];
  auto nib_load = [&](int c, uint2 (&na)[kStageGroups], uint2 (&nb)[kStageGroups]) {
#pragma unroll
    for (int gl = 0; gl < kStageGroups; ++gl) {
      const int g = c * kStageGroups + gl;
      if (g < G) {
        na[gl] = *reinterpret_cast<const uint2*>(qA + g * 32);
        nb[gl] = *reinterpret_cast<const uint2*>(qB + g * 32);
      } else {
        na[gl] = make_uint2(0, 0);
        nb[gl] = make_uint2(0, 0);
      }
    }
  };

  float4_t totA[2], totB[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    totA[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
    totB[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
  const float4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int c, int buf, const uint2 (&na)[kStageGroups], const uint2 (&nb)[kStageGroups]) {
    typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
    const half4_t sA = *reinterpret_cast<const half4_t*>(&szs[buf][0][wave * 32 + n][0]);
    const half4_t zA = *reinterpret_cast<const half4_t*>(&szs[buf][1][wave * 32 + n][0]);
    const half4_t sB = *reinterpret_cast<const half4_t*>(&szs[buf][0][wave * 32 + 16 + n][0]);
    const half4_t zB = *reinterpret_cast<const half4_t*>(&szs[buf][1][wave * 32 + 16 + n][0]);
#pragma unroll
    for (int gl = 0; gl < kStageGroups; ++gl) {
      if (c * kStageGroups + gl >= G) break;
      const _Float16 za = zA[gl], zb = zB[gl];
      const half8_t bA0 = dequant8(na[gl].x, -((_Float16)1024.f + za), -((_Float16)64.f + za));
      const half8_t bA1 = dequant8(na[gl].y, -((_Float16)1024.f + za), -((_Float16)64.f + za));
      const half8_t bB0 = dequant8(nb[gl].x, -((_Float16)1024.f + zb), -((_Float16)64.f + zb));
      const half8_t bB1 = dequant8(nb[gl].y, -((_Float16)1024.f + zb), -((_Float16)64.f + zb));
      const float fsA = (float)sA[gl], fsB = (float)sB[gl];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        if (mt < nMT) {
          const _Float16* xrow = &xs[buf][mt * 16 + n][gl * 64 + kb * 16];
          const half8_t a0 = *reinterpret_cast<const half8_t*>(xrow);
          const half8_t a1 = *reinterpret_cast<const half8_t*>(xrow + 8);
          float4_t accA = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bA0, zero4, 0, 0, 0);
          accA = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bA1, accA, 0, 0, 0);
          float4_t accB = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bB0, zero4, 0, 0, 0);
          accB = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bB1, accB, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            totA[mt][r] = fmaf(fsA, accA[r], totA[mt][r]);
            totB[mt][r] = fmaf(fsB, accB[r], totB[mt][r]);
          }
        }
      }
    }
  };

  // Prologue: stage 0 into LDS buffer 0, its packed bytes into registers set 0.
  stage_load(0);
  nib_load(0, nA0, nB0);
  stage_store(0);
  __syncthreads();
  for (int c = 0; c < NS; c += 2) {
    // even stage: registers set 0, LDS buffer 0
    if (c + 1 < NS) {
      stage_load(c + 1);
      nib_load(c + 1, nA1, nB1);
    }
    compute(c, 0, nA0, nB0);
    if (c + 1 < NS) stage_store(1);
    __syncthreads();
    if (c + 1 >= NS) break;
    // odd stage: registers set 1, LDS buffer 1
    if (c + 2 < NS) {
      stage_load(c + 2);
      nib_load(c + 2, nA0, nB0);
    }
    compute(c + 1, 1, nA1, nB1);
    if (c + 2 < NS) stage_store(0);
    __syncthreads();
  }

  // Epilogue: D lane layout = tokens 4kb..4kb+3 of weight row n.
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    if (mt >= nMT) break;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mt * 16 + kb * 4 + r;
      if (m >= mcount) continue;
      if (GATED) {
        const float hv = gelu_tanh(totA[mt][r]) * totB[mt][r];
        const int col = tile * 64 + wave * 16 + n;
        const int pcol = (col & ~7) | ((col & 3) << 1) | ((col >> 2) & 1);
        const _Float16 h16 = (_Float16)hv;
        a.h_out[(size_t)(pos0 + m) * a.d_ff + pcol] = __builtin_bit_cast(uint16_t, h16);
      } else {
        const int slot = a.perm[pos0 + m];
        const int row = tile * kRowsPerBlock + wave * 32 + n;
        a.o_out[(size_t)slot * a.out_ld + row] = totA[mt][r];
        a.o_out[(size_t)slot * a.out_ld + row + 16] = totB[mt][r];
      }
    }
  }
}

}  // namespace

hipError_t launch_gate_up(const W4A16Matrix& gu, int E, int d_model, int d_ff, int top_k, int T,
                          const uint16_t* x, const MoeWorkspace& ws, hipStream_t stream) {
  GemmArgs a;
  a.q = gu.q;
  a.scale = gu.scale;
  a.zero = gu.zero;
  a.K = d_model;
  a.R = 2 * d_ff;
  a.d_ff = d_ff;
  a.top_k = top_k;
  a.act = x;
  a.perm = ws.perm;
  a.items = ws.items;
  a.h_out = ws.h;
  a.o_out = nullptr;
  a.out_ld = d_ff;
  (void)E;
  (void)T;
  hipLaunchKernelGGL(w4a16_gemm_kernel<true>, dim3(d_ff / 64, ws.max_items), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_down(const W4A16Matrix& dn, int E, int d_model, int d_ff, int top_k, int T,
                       float* expert_out, const MoeWorkspace& ws, hipStream_t stream) {
  GemmArgs a;
  a.q = dn.q;
  a.scale = dn.scale;
  a.zero = dn.zero;
  a.K = d_ff;
  a.R = d_model;
  a.d_ff = d_ff;
  a.top_k = top_k;
  a.act = ws.h;
  a.perm = ws.perm;
  a.items = ws.items;
  a.h_out = nullptr;
  a.o_out = expert_out;
  a.out_ld = d_model;
  (void)E;
  (void)T;
  hipLaunchKernelGGL(w4a16_gemm_kernel<false>, dim3(d_model / kRowsPerBlock, ws.max_items),
                     dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bd
