// The two steps either side of the expert FFN's routing: the fused RMS norm that produces the
// FFN input, and the router projection whose fp32 logits feed the top-k.
//
// Sources: axe-diffusion-ksl-xe model card, "the kernels we built" (one fused launch for the
// RMS norm in place of about six element-wise ones; the norm runs 180 times in a forward
// pass); "what the model is" (128 experts scored per token, top-8 kept).
//
// RMS norm.  One wave per row, four rows per 256-thread block.  A row of d <= 4096 halves is
// at most eight 16-byte vectors per lane: the wave loads the row once into registers, sums
// the squares in fp32 (each square of an fp16 value is exact in fp32; lanes sum in element
// order, then one fixed-order wave reduction), loading its share of w alongside, and writes
//     y = fp16_rne(x * (1 / sqrt(sum / d + eps)) * w)
// from the same registers.  HBM traffic is the row in and the row out, plus w from L2.  The
// row moves through buffer loads and stores whose range check zero-fills (and drops) the
// lanes past a short row, so no vector of the row needs a branch of its own.
//
// Router projection.  logits[t][e] = sum_k x[t][k] W_r[e][k] on v_mfma_f32_16x16x32_f16:
// fp16 products are exact and accumulate in fp32.  A block owns one 16-token x 16-expert tile
// and its eight waves (four when d % 256 != 0) split the contraction dim into equal parts; the
// parts' 16 x 16 sums meet in LDS and are added in wave order, so the result is reproducible.  Each lane streams its
// 16-byte fragments of x and W_r straight from memory (both stay in L2: 1.4 MB and 0.7 MB at
// the layer's shape).  Fragment layout as in the expert GEMMs: lane (m, kb) = (lane % 16,
// lane / 16) supplies row m at k-slots 8kb..8kb+7 of A (tokens) and of B (experts), and
// receives D for tokens 4kb..4kb+3 of expert m.

#include "bd_device.hpp"
#include "bd_internal.hpp"

namespace bd {

namespace {

constexpr int kNormThreads = 256;
constexpr int kNormRows = kNormThreads / kWave;
constexpr int kNormMaxVec = 8;  // 8 vectors x 8 halves x 64 lanes = 4096 features

__device__ __forceinline__ half8_t as_half8(u32x4_t v) { return __builtin_bit_cast(half8_t, v); }
__device__ __forceinline__ u32x4_t as_u32x4(half8_t v) { return __builtin_bit_cast(u32x4_t, v); }

// Buffer loads and stores over one row: a read past the row's byte range returns zeros and a
// write past it is dropped, so the lanes past the end of a row need no branch (a zero adds
// nothing to the sum of squares).  Word 3 of a gfx9 descriptor: raw 32-bit data.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ w, int T, int d, float eps,
    uint16_t* __restrict__ y, const int32_t* __restrict__ gate) {
  if (gated_off(gate)) return;
  const int row = blockIdx.x * kNormRows + (int)(threadIdx.x / kWave);
  if (row >= T) return;  // wave-uniform
  const int lane = lane_id();
  const uint32_t bytes = (uint32_t)d * 2u;
  const __amdgpu_buffer_rsrc_t src = row_rsrc(h + (size_t)row * d, bytes);
  const __amdgpu_buffer_rsrc_t wsrc = row_rsrc(w, bytes);
  const __amdgpu_buffer_rsrc_t dst = row_rsrc(y + (size_t)row * d, bytes);
  u32x4_t v[kNormMaxVec], g[kNormMaxVec];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < kNormMaxVec; ++i) {
    const int off = (lane + i * kWave) * 16;
    v[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(src, off, 0, 2));
    g[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wsrc, off, 0, 0));
  }
#pragma unroll
  for (int i = 0; i < kNormMaxVec; ++i) {
    const half8_t x = as_half8(v[i]);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float f = (float)x[q];
      ss = fmaf(f, f, ss);
    }
  }
  const float total = wave_sum(ss);
  const float r = 1.f / sqrtf(total / (float)d + eps);
#pragma unroll
  for (int i = 0; i < kNormMaxVec; ++i) {
    const half8_t x = as_half8(v[i]);
    const half8_t gw = as_half8(g[i]);
    half8_t o;
#pragma unroll
    for (int q = 0; q < 8; ++q) o[q] = (_Float16)keep_f32(((float)x[q] * r) * (float)gw[q]);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, as_u32x4(o)), dst,
                                           (lane + i * kWave) * 16, 0, 0);
  }
}

// One 16 x 16 (token x expert) tile per block; WAVES waves split the contraction dim into
// equal parts (8 when d % 256 == 0, else 4), each a chain of MFMA steps with its loads eight
// steps ahead, and the parts are summed in a fixed order through LDS.
template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void router_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int E, int d,
    float* __restrict__ logits, const int32_t* __restrict__ gate) {
  if (gated_off(gate)) return;
  __shared__ float4_t part[WAVES][kWave];
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int m = lane & 15;
  const int kb = lane >> 4;
  const int t0 = blockIdx.x * 16;
  const int e0 = blockIdx.y * 16;
  // Rows past the ends are clamped onto the last row: their sums are computed and dropped.
  const int t = min(t0 + m, T - 1);
  const int e = min(e0 + m, E - 1);
  const int kq = d / WAVES;
  const int steps = kq / 32;
  const half8_t* __restrict__ xa =
      reinterpret_cast<const half8_t*>(x + (size_t)t * d + wave * kq + kb * 8);
  const half8_t* __restrict__ wb =
      reinterpret_cast<const half8_t*>(wr + (size_t)e * d + wave * kq + kb * 8);
  float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int s = 0; s < steps; ++s)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[s * 4], wb[s * 4], acc, 0, 0, 0);
  part[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  float4_t sum = part[0][lane];
#pragma unroll
  for (int q = 1; q < WAVES; ++q) {
    const float4_t p = part[q][lane];
    sum[0] += p[0];
    sum[1] += p[1];
    sum[2] += p[2];
    sum[3] += p[3];
  }
  const int ee = e0 + m;
  if (ee >= E) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tt = t0 + 4 * kb + i;
    if (tt < T) logits[(size_t)tt * E + ee] = sum[i];
  }
}

}  // namespace

hipError_t launch_rmsnorm(const uint16_t* h, const uint16_t* weight, int T, int d, float eps,
                          uint16_t* y, hipStream_t stream, const int32_t* gate) {
  const int blocks = (T + kNormRows - 1) / kNormRows;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(blocks), dim3(kNormThreads), 0, stream, h, weight, T,
                     d, eps, y, gate);
  return hipGetLastError();
}

hipError_t launch_router(const uint16_t* x, const uint16_t* w_router, int T, int d, int E,
                         float* logits, hipStream_t stream, const int32_t* gate) {
  const dim3 grid((T + 15) / 16, (E + 15) / 16);
  if (d % 256 == 0)
    hipLaunchKernelGGL(router_kernel<8>, grid, dim3(8 * kWave), 0, stream, x, w_router, T, E, d,
                       logits, gate);
  else
    hipLaunchKernelGGL(router_kernel<4>, grid, dim3(4 * kWave), 0, stream, x, w_router, T, E, d,
                       logits, gate);
  return hipGetLastError();
}

}  // namespace bd
