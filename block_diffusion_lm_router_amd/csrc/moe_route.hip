// Routing kernels of the MoE layer: per-token top-k with softmax weights, then a stable
// bucketing of the T*k assignments by expert and the work list of touched experts.
//
// Source: axe-diffusion-ksl-xe model card, "what the model is" (128 experts, top-8 per
// token) and "the kernels we built" (one launch covers all experts instead of a
// per-expert loop, which needs the assignments grouped by expert on the device).

#include "bd_device.hpp"
#include "bd_internal.hpp"

namespace bd {

namespace {

constexpr int kTopkThreads = 256;
constexpr int kBucketThreads = 1024;
constexpr int kMaxE = 256;
constexpr int kPassTokens = 1024;         // tokens per bitmask pass of the bucketing
constexpr int kPassWords = kPassTokens / 64;

// Order-preserving map of a float to uint32 (-0 folded onto +0).
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_order_key(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __builtin_bit_cast(float, u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

// One wave per token.  Key = (order(logit) << 32) | (0xffffffff - expert): the maximum
// key is the largest logit, the lower expert id first among equal logits.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ logits,
                                                            int T, int E, int k,
                                                            int32_t* __restrict__ ids,
                                                            float* __restrict__ weights) {
  const int t = blockIdx.x * (kTopkThreads / kWave) + threadIdx.x / kWave;
  if (t >= T) return;  // uniform per wave
  const int lane = lane_id();
  uint64_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + kWave * i;
    key[i] = e < E ? ((uint64_t)order_key(logits[(size_t)t * E + e]) << 32) | (0xffffffffu - (uint32_t)e)
                   : 0ull;
  }
  int my_id = 0;
  float my_val = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t b = key[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) b = key[i] > b ? key[i] : b;
    b = wave_max_u64(b);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (key[i] == b) key[i] = 0ull;
    if (lane == j) {
      my_id = (int)(0xffffffffu - (uint32_t)b);
      my_val = from_order_key((uint32_t)(b >> 32));
    }
  }
  const float l0 = readlane_f32(my_val, 0);
  const float ex = lane < k ? expf(my_val - l0) : 0.f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    weights[(size_t)t * k + lane] = ex / sum;
  }
}

// Inclusive scan of 256 ints in LDS by the first 256 threads (Hillis-Steele).
__device__ void scan256(int* buf, int tid) {
  for (int off = 1; off < kMaxE; off <<= 1) {
    int v = 0;
    if (tid < kMaxE && tid >= off) v = buf[tid - off];
    __syncthreads();
    if (tid < kMaxE) buf[tid] += v;
    __syncthreads();
  }
}

// One block.  Bucket positions are stable in assignment order a = t*k + j: the rank of
// (t, j) inside expert e's bucket is the number of earlier tokens routed to e, counted
// with per-expert token bitmasks (a token picks an expert at most once).
__global__ __launch_bounds__(kBucketThreads) void bucket_kernel(const int32_t* __restrict__ ids,
                                                                int T, int k, int E,
                                                                int32_t* __restrict__ offsets,
                                                                int32_t* __restrict__ items,
                                                                int32_t* __restrict__ perm) {
  __shared__ int cnt[kMaxE];
  __shared__ int off[kMaxE];
  __shared__ int itoff[kMaxE];
  __shared__ int running[kMaxE];
  __shared__ unsigned long long bits[kMaxE * kPassWords];
  __shared__ int pre[kMaxE * kPassWords];
  const int tid = threadIdx.x;
  const int A = T * k;
  if (tid < kMaxE) {
    cnt[tid] = 0;
    running[tid] = 0;
  }
  __syncthreads();
  for (int a = tid; a < A; a += kBucketThreads) atomicAdd(&cnt[ids[a]], 1);
  __syncthreads();
  if (tid < kMaxE) {
    off[tid] = cnt[tid];
    itoff[tid] = (cnt[tid] + kItemTokens - 1) / kItemTokens;
  }
  __syncthreads();
  scan256(off, tid);
  scan256(itoff, tid);
  // inclusive -> exclusive, write offsets and the work list
  if (tid < E) {
    const int c = cnt[tid];
    const int o = off[tid] - c;
    const int ni = (c + kItemTokens - 1) / kItemTokens;
    const int io = itoff[tid] - ni;
    offsets[tid] = o;
    for (int i = 0; i < ni; ++i) {
      int32_t* it = items + 1 + 3 * (io + i);
      it[0] = tid;
      it[1] = o + i * kItemTokens;
      it[2] = min(kItemTokens, c - i * kItemTokens);
    }
  }
  if (tid == 0) {
    offsets[E] = A;
    items[0] = itoff[E - 1];
  }
  __syncthreads();
  if (tid < kMaxE) off[tid] -= cnt[tid];
  __syncthreads();
  for (int t0 = 0; t0 < T; t0 += kPassTokens) {
    for (int i = tid; i < kMaxE * kPassWords; i += kBucketThreads) bits[i] = 0ull;
    __syncthreads();
    const int a0 = t0 * k, a1 = min(T, t0 + kPassTokens) * k;
    for (int a = a0 + tid; a < a1; a += kBucketThreads) {
      const int lt = a / k - t0;
      atomicOr(&bits[ids[a] * kPassWords + (lt >> 6)], 1ull << (lt & 63));
    }
    __syncthreads();
    if (tid < E) {
      int r = running[tid];
      for (int w = 0; w < kPassWords; ++w) {
        pre[tid * kPassWords + w] = r;
        r += __popcll(bits[tid * kPassWords + w]);
      }
      running[tid] = r;
    }
    __syncthreads();
    for (int a = a0 + tid; a < a1; a += kBucketThreads) {
      const int lt = a / k - t0;
      const int e = ids[a];
      const int w = lt >> 6;
      const unsigned long long below = (1ull << (lt & 63)) - 1ull;
      const int rank = pre[e * kPassWords + w] + __popcll(bits[e * kPassWords + w] & below);
      perm[off[e] + rank] = a;
    }
    __syncthreads();
  }
}

}  // namespace

int moe_max_items(int T, int E, int k) {
  const int A = T * k;
  return A / kItemTokens + (E < A ? E : A);
}

size_t moe_workspace_bytes(int T, int E, int k, int d_model, int d_ff) {
  const size_t A = (size_t)T * k;
  return align_up((size_t)(E + 1) * 4) + align_up((size_t)(1 + 3 * moe_max_items(T, E, k)) * 4) +
         align_up(A * 4) + align_up(A * (size_t)d_ff * 2) + align_up((size_t)T * d_model * 2);
}

MoeWorkspace moe_workspace_carve(void* base, int T, int E, int k, int d_model, int d_ff) {
  const size_t A = (size_t)T * k;
  char* p = reinterpret_cast<char*>(base);
  MoeWorkspace ws;
  ws.max_items = moe_max_items(T, E, k);
  ws.offsets = reinterpret_cast<int32_t*>(p);
  p += align_up((size_t)(E + 1) * 4);
  ws.items = reinterpret_cast<int32_t*>(p);
  p += align_up((size_t)(1 + 3 * ws.max_items) * 4);
  ws.perm = reinterpret_cast<int32_t*>(p);
  p += align_up(A * 4);
  ws.h = reinterpret_cast<uint16_t*>(p);
  p += align_up(A * (size_t)d_ff * 2);
  ws.xp = reinterpret_cast<uint16_t*>(p);
  (void)d_model;
  return ws;
}

hipError_t launch_route(const float* router_logits, int T, int E, int k, int32_t* topk_ids,
                        float* topk_weights, const MoeWorkspace& ws, hipStream_t stream) {
  const int per_block = kTopkThreads / kWave;
  hipLaunchKernelGGL(topk_kernel, dim3((T + per_block - 1) / per_block), dim3(kTopkThreads), 0,
                     stream, router_logits, T, E, k, topk_ids, topk_weights);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(kBucketThreads), 0, stream, topk_ids, T, k, E,
                     ws.offsets, ws.items, ws.perm);
  return hipGetLastError();
}

}  // namespace bd
