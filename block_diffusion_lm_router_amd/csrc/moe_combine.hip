// Fixed-order weighted combine of the per-assignment expert outputs, the same combine
// followed by the next layer's RMS norm in one launch, and the plain streaming copy and read
// used to calibrate HBM traffic counters and to measure the achievable read rate.
//
// Source: axe-diffusion-ksl-xe model card, "the kernels we built": the weighted combine
// is a fixed-order reduction instead of index_add_ with atomics, because a 1-ulp
// difference can flip an acceptance threshold; the RMS norm is one fused launch.  Here every
// output element has exactly one writer, which sums its k slots in ascending j with fp32 fma
// and rounds the fp32 sum to fp16 once.

#include "bd_device.hpp"
#include "bd_internal.hpp"

namespace bd {

namespace {

constexpr int kCombineThreads = 256;
constexpr int kUnrolledK = 8;                 // top-k with the slots' loads issued together
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float* __restrict__ o,
                                                                  const float* __restrict__ w,
                                                                  int T, int k, int d,
                                                                  uint16_t* __restrict__ y,
                                                                  const int32_t* __restrict__ gate) {
  if (gated_off(gate)) return;
  const int d4 = d >> 2;
  const int64_t i = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x;
  if (i >= (int64_t)T * d4) return;
  const int t = (int)(i / d4);
  const int c = (int)(i % d4) * 4;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  auto term = [&](float wj, const float4& v) {
    a0 = fmaf(wj, v.x, a0);
    a1 = fmaf(wj, v.y, a1);
    a2 = fmaf(wj, v.z, a2);
    a3 = fmaf(wj, v.w, a3);
  };
  const float* wt = w + (size_t)t * k;
  const float* ot = o + (size_t)t * k * d + c;
  if (k == kUnrolledK) {
    // Every slot's row read before the first product (one memory round trip, not k), then
    // the sum in ascending j as below.
    // The expert outputs are read once: nontemporal loads.
    float wj[kUnrolledK];
    float4 v[kUnrolledK];
#pragma unroll
    for (int j = 0; j < kUnrolledK; ++j) {
      wj[j] = wt[j];
      const f32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(ot + (size_t)j * d));
      v[j] = make_float4(q[0], q[1], q[2], q[3]);
    }
#pragma unroll
    for (int j = 0; j < kUnrolledK; ++j) term(wj[j], v[j]);
  } else {
    for (int j = 0; j < k; ++j) term(wt[j], *reinterpret_cast<const float4*>(ot + (size_t)j * d));
  }
  // The fp32 sums rounded to fp16 (keep_f32: no multiply-add fused into the conversion).
  const _Float16 h0 = (_Float16)keep_f32(a0), h1 = (_Float16)keep_f32(a1);
  const _Float16 h2 = (_Float16)keep_f32(a2), h3 = (_Float16)keep_f32(a3);
  uint2 out;
  out.x = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
  out.y = (uint32_t)__builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
  *reinterpret_cast<uint2*>(y + (size_t)t * d + c) = out;
}

// The combine followed by the next layer's RMS norm, one block per token row.  Phase 1 is the
// combine above (each output element: its k slots summed in ascending j with fp32 fma, rounded
// once to fp16), with every slot load of the thread issued before the first product; the fp16
// row goes to y and to LDS.  Phase 2: wave 0 takes the row from LDS in the RMS norm kernel's
// layout (lane l: 8-half vectors l, l + 64, ... in element order, squares accumulated with
// fp32 fma, then the same wave reduction), so the factor 1 / sqrt(mean + eps) is the one that
// kernel computes from y.  Phase 3: every thread writes fp16(y * r * weight) for its elements
// from its registers, the norm kernel's expression.  With the same fp32-then-fp16 roundings
// (keep_f32 in all three kernels) both outputs are bit-identical to the combine launch followed
// by the RMS norm launch, without the second read of y.
constexpr int kCNThreads = 256;
constexpr int kCNMaxGroups = 4;             // 4-element groups per thread: d <= 4096
constexpr int kCNMaxFeatures = kCNThreads * kCNMaxGroups * 4;
constexpr int kCNMaxVec = kCNMaxFeatures / 8 / kWave;    // 8-half vectors per lane in phase 2

__global__ __launch_bounds__(kCNThreads) void combine_norm_kernel(
    const float* __restrict__ o, const float* __restrict__ w, int k, int d,
    const uint16_t* __restrict__ gw, float eps, uint16_t* __restrict__ y,
    uint16_t* __restrict__ xn, const int32_t* __restrict__ gate) {
  if (gated_off(gate)) return;
  __shared__ __attribute__((aligned(16))) uint16_t row[kCNMaxFeatures];
  __shared__ float r_sh;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int d4 = d >> 2;
  const float* wt = w + (size_t)t * k;
  const float* ot = o + (size_t)t * k * d;
  uint2 yv[kCNMaxGroups];
  auto finish = [&](int i, int g, float a0, float a1, float a2, float a3) {
    const _Float16 h0 = (_Float16)keep_f32(a0), h1 = (_Float16)keep_f32(a1);
    const _Float16 h2 = (_Float16)keep_f32(a2), h3 = (_Float16)keep_f32(a3);
    uint2 out;
    out.x = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    out.y = (uint32_t)__builtin_bit_cast(uint16_t, h2) | ((uint32_t)__builtin_bit_cast(uint16_t, h3) << 16);
    yv[i] = out;
    *reinterpret_cast<uint2*>(y + (size_t)t * d + g * 4) = out;
    *reinterpret_cast<uint2*>(row + g * 4) = out;
  };
  if (k == kUnrolledK) {
    float wj[kUnrolledK];
    f32x4_t v[kCNMaxGroups][kUnrolledK];
#pragma unroll
    for (int j = 0; j < kUnrolledK; ++j) wj[j] = wt[j];
#pragma unroll
    for (int i = 0; i < kCNMaxGroups; ++i) {
      const int g = tid + i * kCNThreads;
      if (g < d4) {
#pragma unroll
        for (int j = 0; j < kUnrolledK; ++j)
          v[i][j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(ot + (size_t)j * d + g * 4));
      }
    }
#pragma unroll
    for (int i = 0; i < kCNMaxGroups; ++i) {
      const int g = tid + i * kCNThreads;
      if (g < d4) {
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
        for (int j = 0; j < kUnrolledK; ++j) {
          a0 = fmaf(wj[j], v[i][j][0], a0);
          a1 = fmaf(wj[j], v[i][j][1], a1);
          a2 = fmaf(wj[j], v[i][j][2], a2);
          a3 = fmaf(wj[j], v[i][j][3], a3);
        }
        finish(i, g, a0, a1, a2, a3);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < kCNMaxGroups; ++i) {
      const int g = tid + i * kCNThreads;
      if (g < d4) {
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
        for (int j = 0; j < k; ++j) {
          const float wjj = wt[j];
          const float4 q = *reinterpret_cast<const float4*>(ot + (size_t)j * d + g * 4);
          a0 = fmaf(wjj, q.x, a0);
          a1 = fmaf(wjj, q.y, a1);
          a2 = fmaf(wjj, q.z, a2);
          a3 = fmaf(wjj, q.w, a3);
        }
        finish(i, g, a0, a1, a2, a3);
      }
    }
  }
  __syncthreads();
  if (tid < kWave) {
    const int nv = d >> 3;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < kCNMaxVec; ++i) {
      const int j = tid + i * kWave;
      if (j < nv) {
        const half8_t x = __builtin_bit_cast(half8_t, *reinterpret_cast<const u32x4_t*>(row + j * 8));
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float f = (float)x[q];
          ss = fmaf(f, f, ss);
        }
      }
    }
    const float total = wave_sum(ss);
    if (tid == 0) r_sh = 1.f / sqrtf(total / (float)d + eps);
  }
  __syncthreads();
  const float r = r_sh;
#pragma unroll
  for (int i = 0; i < kCNMaxGroups; ++i) {
    const int g = tid + i * kCNThreads;
    if (g < d4) {
      const uint2 gv = *reinterpret_cast<const uint2*>(gw + g * 4);
      const uint32_t xs[2] = {yv[i].x, yv[i].y}, ws2[2] = {gv.x, gv.y};
      uint32_t outw[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const half2_t xv = __builtin_bit_cast(half2_t, xs[h]);
        const half2_t wv = __builtin_bit_cast(half2_t, ws2[h]);
        const _Float16 lo = (_Float16)keep_f32(((float)xv[0] * r) * (float)wv[0]);
        const _Float16 hi = (_Float16)keep_f32(((float)xv[1] * r) * (float)wv[1]);
        outw[h] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      *reinterpret_cast<uint2*>(xn + (size_t)t * d + g * 4) = make_uint2(outw[0], outw[1]);
    }
  }
}

constexpr int kCopyThreads = 256;

__global__ __launch_bounds__(kCopyThreads) void copy_kernel(const u32x4_t* __restrict__ src,
                                                            u32x4_t* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * kCopyThreads;
  for (size_t i = (size_t)blockIdx.x * kCopyThreads + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Streaming read: XOR of every 32-bit word, one nontemporal 16-byte load per thread per
// iteration over a grid-stride sweep by 1024 blocks of 512 threads (the fastest of the
// thread/block/unroll shapes tried for plain and nontemporal loads).  Each block folds its
// threads (wave shuffles, then LDS) and writes one partial to part[blockIdx.x]; a one-block
// pass folds the partials into part[-1].  No two blocks write the same word, so the read is
// not serialised behind same-address atomics.
constexpr int kReadBlocks = 1024;
constexpr int kReadThreads = 512;

template <int THREADS>
__device__ __forceinline__ uint32_t block_xor(uint32_t v) {
  __shared__ uint32_t w[THREADS / 64];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v ^= (uint32_t)__shfl_xor((int)v, off, 64);
  if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = v;
  __syncthreads();
  v = 0;
#pragma unroll
  for (int i = 0; i < THREADS / 64; ++i) v ^= w[i];
  return v;
}

__global__ __launch_bounds__(kReadThreads) void read_kernel(const u32x4_t* __restrict__ src, size_t n,
                                                            uint32_t* __restrict__ part) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x; i < n; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  acc = block_xor<kReadThreads>(acc);
  if (threadIdx.x == 0) part[blockIdx.x] = acc;
}

__global__ __launch_bounds__(kCopyThreads) void read_finish_kernel(uint32_t* __restrict__ out,
                                                                   int nparts) {
  uint32_t acc = 0;
  for (int i = threadIdx.x; i < nparts; i += kCopyThreads) acc ^= out[1 + i];
  acc = block_xor<kCopyThreads>(acc);
  if (threadIdx.x == 0) out[0] = acc;
}

}  // namespace

hipError_t launch_combine(const float* expert_out, const float* topk_weights, int T, int k, int d,
                          uint16_t* y, hipStream_t stream, const int32_t* gate) {
  const int64_t n = (int64_t)T * (d / 4);
  const int blocks = (int)((n + kCombineThreads - 1) / kCombineThreads);
  hipLaunchKernelGGL(combine_kernel, dim3(blocks), dim3(kCombineThreads), 0, stream, expert_out,
                     topk_weights, T, k, d, y, gate);
  return hipGetLastError();
}

hipError_t launch_combine_norm(const float* expert_out, const float* topk_weights, int T, int k,
                               int d, const uint16_t* weight, float eps, uint16_t* y, uint16_t* xn,
                               hipStream_t stream, const int32_t* gate) {
  if (d > kCNMaxFeatures || d % 8 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_norm_kernel, dim3(T), dim3(kCNThreads), 0, stream, expert_out,
                     topk_weights, k, d, weight, eps, y, xn, gate);
  return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  const size_t n = bytes / 16;
  size_t blocks = (n + kCopyThreads - 1) / kCopyThreads;
  if (blocks > 256 * 32) blocks = 256 * 32;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, stream,
                     reinterpret_cast<const u32x4_t*>(src), reinterpret_cast<u32x4_t*>(dst), n);
  return hipGetLastError();
}

hipError_t launch_read(const void* src, size_t bytes, uint32_t* checksum, hipStream_t stream) {
  const size_t n = bytes / 16;
  size_t blocks = (n + kReadThreads - 1) / kReadThreads;
  if (blocks > kReadBlocks) blocks = kReadBlocks;
  if (blocks > 0)
    hipLaunchKernelGGL(read_kernel, dim3((unsigned)blocks), dim3(kReadThreads), 0, stream,
                       reinterpret_cast<const u32x4_t*>(src), n, checksum + 1);
  hipLaunchKernelGGL(read_finish_kernel, dim3(1), dim3(kCopyThreads), 0, stream, checksum,
                     (int)blocks);
  return hipGetLastError();
}

}  // namespace bd
