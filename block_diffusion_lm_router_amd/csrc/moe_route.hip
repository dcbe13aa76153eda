// Routing kernels of the MoE layer: per-token top-k with softmax weights, then a stable
// bucketing of the T*k assignments by expert and the work list of touched experts (one
// block, in a second launch).
//
// Source: axe-diffusion-ksl-xe model card, "what the model is" (128 experts, top-8 per
// token) and "the kernels we built" (one launch covers all experts instead of a
// per-expert loop, which needs the assignments grouped by expert on the device).

#include "bd_device.hpp"
#include "bd_internal.hpp"

namespace bd {

namespace {

constexpr int kTopkThreads = 256;
constexpr int kMaxTopk = 16;
constexpr int kMaxE = 256;
constexpr int kBucketThreads = 1024;
constexpr int kPassTokens = 1024;         // tokens per bitmask pass of the bucketing
constexpr int kPassWords = kPassTokens / 64;

// Order-preserving map of a float to uint32 (-0 folded onto +0).
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

typedef unsigned long long u64x2_t __attribute__((ext_vector_type(2)));

// Top-k of one token per block.  Key of expert e = (order(logit) << 32) | (0xffffffff - e):
// keys are distinct, a larger logit gives a larger key and the lower expert id wins a tie.
// The rank of a key is the number of the token's keys above it; thread (i, part) counts
// the keys above key i in one of 256/Ep contiguous parts of the key list (read back from
// LDS as broadcasts), the parts are summed, and rank r < k puts expert i in slot r.
// Weights = softmax over the k selected logits, summed in a fixed order.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ logits,
                                                            int T, int E, int k,
                                                            int32_t* __restrict__ ids,
                                                            int32_t* __restrict__ ids_copy,
                                                            float* __restrict__ weights,
                                                            const int32_t* __restrict__ gate) {
  if (gated_off(gate)) return;
  __shared__ __attribute__((aligned(16))) unsigned long long keys[kMaxE];
  __shared__ int part_rank[kTopkThreads];
  __shared__ int sel_id[kMaxTopk];
  __shared__ float sel_val[kMaxTopk];
  const int tid = threadIdx.x;
  const int t = blockIdx.x;
  const int Ep = E <= 64 ? 64 : (E <= 128 ? 128 : 256);
  const int parts = kTopkThreads / Ep;
  const int span = Ep / parts;                 // keys per part: 16, 64 or 256
  const int i = tid % Ep, part = tid / Ep;
  float val = 0.f;
  uint64_t key = 0ull;
  if (i < E) {
    val = logits[(size_t)t * E + i];
    key = ((uint64_t)order_key(val) << 32) | (0xffffffffu - (uint32_t)i);
  }
  if (part == 0) keys[i] = key;                // zeros past E never outrank a key
  __syncthreads();
  int r = 0;
  const unsigned long long* kp = keys + part * span;
#pragma unroll 8
  for (int j = 0; j < span; j += 2) {
    const u64x2_t o = *reinterpret_cast<const u64x2_t*>(kp + j);
    r += (o[0] > key) + (o[1] > key);
  }
  part_rank[tid] = r;
  __syncthreads();
  if (part == 0 && i < E) {
    int rank = 0;
    for (int p = 0; p < parts; ++p) rank += part_rank[p * Ep + i];
    if (rank < k) {
      sel_id[rank] = i;
      sel_val[rank] = val;
    }
  }
  __syncthreads();
  if (tid < kWave) {
    const int lane = tid;
    const int my_id = lane < k ? sel_id[lane] : 0;
    const float my_val = lane < k ? sel_val[lane] : 0.f;
    const float l0 = readlane_f32(my_val, 0);
    const float ex = lane < k ? expf(my_val - l0) : 0.f;
    const float sum = wave_sum(ex);
    if (lane < k) {
      ids[(size_t)t * k + lane] = my_id;
      ids_copy[(size_t)t * k + lane] = my_id;
      weights[(size_t)t * k + lane] = ex / sum;
    }
  }
}

struct BucketArgs {
  const int32_t* ids;      // [T * k]
  int T, k, E;
  int32_t* offsets;        // [E + 1]
  int32_t* items;          // [0] = count, then (expert, first position, tokens)
  int32_t* perm;           // [T * k]
  const int32_t* gate;     // loop driver state or NULL (see gated_off)
};

// Expert id of an assignment, clamped into [0, E) so that no value read can index past the
// bucket tables (the routing only writes ids in range).
__device__ __forceinline__ int expert_of(const int32_t* ids, int a, int E) {
  return (int)min((uint32_t)ids[a], (uint32_t)(E - 1));
}

struct BucketShared {
  unsigned long long bits[kMaxE * kPassWords];   // token bitmask of each expert, one pass
  int wpre[kMaxE * kPassWords];                  // bucket rank at the start of each word
  int cnt[kMaxE];
  int eoff[kMaxE];
  int ecnt[kMaxE];
  int ioff[kMaxE + 1];
  int wsum[8];
};

// Called by every thread of the block.  Thread e < Ep holds tot = the assignment count of
// expert e (0 past E).  Exclusive prefixes over experts of the counts and of the item
// counts ceil(tot / kItemTokens), by wave scans and the wave totals; then the offsets and
// the work list (item it belongs to the last expert whose first item is <= it).
__device__ void expert_scan(int tot, int E, int Ep, int A, BucketShared& sh,
                            int32_t* __restrict__ offsets, int32_t* __restrict__ items) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int ni = (tot + kItemTokens - 1) / kItemTokens;
  int it = 0, ii = 0;
  if (tid < Ep) {                               // whole waves: Ep is a multiple of 64
    it = wave_incl_scan_i32(tot);
    ii = wave_incl_scan_i32(ni);
    if (lane == kWave - 1) {
      sh.wsum[wave] = it;
      sh.wsum[4 + wave] = ii;
    }
  }
  __syncthreads();
  if (tid < Ep) {
    int bt = 0, bi = 0;
    for (int w = 0; w < wave; ++w) {
      bt += sh.wsum[w];
      bi += sh.wsum[4 + w];
    }
    const int ex_t = bt + it - tot, ex_i = bi + ii - ni;
    if (tid < E) {
      sh.eoff[tid] = ex_t;
      sh.ecnt[tid] = tot;
      sh.ioff[tid] = ex_i;
      offsets[tid] = ex_t;
    }
    if (tid == Ep - 1) {                        // inclusive totals (experts past E hold 0)
      sh.ioff[E] = bi + ii;
      items[0] = bi + ii;
      offsets[E] = A;
    }
  }
  __syncthreads();
  const int nitems = sh.ioff[E];
  for (int m = tid; m < nitems; m += kBucketThreads) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sh.ioff[mid] <= m) lo = mid; else hi = mid - 1;
    }
    const int q = m - sh.ioff[lo];
    int32_t* out = items + 1 + 3 * m;
    out[0] = lo;
    out[1] = sh.eoff[lo] + q * kItemTokens;
    out[2] = min(kItemTokens, sh.ecnt[lo] - q * kItemTokens);
  }
}

constexpr int kIdCache = 4;                    // assignments per thread held in registers

// The bucketing when all tokens fit one pass (T <= kPassTokens): each thread loads its
// assignments' expert ids once, into registers, and the block takes four barriers (bitmasks
// cleared / marked / counted and scanned / offsets published).
__device__ void bucket_one_pass(const BucketArgs& g, BucketShared& sh) {
  const int tid = threadIdx.x;
  const int T = g.T, k = g.k, E = g.E, A = T * k;
  const int Ep = E <= 64 ? 64 : (E <= 128 ? 128 : 256);
  const int W = (T + 63) / 64;
  int eid[kIdCache];
#pragma unroll
  for (int i = 0; i < kIdCache; ++i) {
    const int a = tid + i * kBucketThreads;
    eid[i] = a < A ? expert_of(g.ids, a, E) : 0;
  }
  for (int i = tid; i < E * kPassWords; i += kBucketThreads) sh.bits[i] = 0ull;
  __syncthreads();
  auto mark = [&](int e, int a) {
    const int t = a / k;
    atomicOr(&sh.bits[e * kPassWords + (t >> 6)], 1ull << (t & 63));
  };
#pragma unroll
  for (int i = 0; i < kIdCache; ++i) {
    const int a = tid + i * kBucketThreads;
    if (a < A) mark(eid[i], a);
  }
  for (int a = tid + kIdCache * kBucketThreads; a < A; a += kBucketThreads)
    mark(expert_of(g.ids, a, E), a);
  __syncthreads();
  int tot = 0;                                  // thread e < E: rank at each word's start
  if (tid < E) {
    for (int w = 0; w < W; ++w) {
      sh.wpre[tid * kPassWords + w] = tot;
      tot += __popcll(sh.bits[tid * kPassWords + w]);
    }
  }
  expert_scan(tot, E, Ep, A, sh, g.offsets, g.items);   // publishes eoff behind a barrier
  auto place = [&](int e, int a) {
    const int t = a / k;
    const int w = e * kPassWords + (t >> 6);
    const int rank = sh.wpre[w] + __popcll(sh.bits[w] & ((1ull << (t & 63)) - 1ull));
    g.perm[sh.eoff[e] + rank] = a;
  };
#pragma unroll
  for (int i = 0; i < kIdCache; ++i) {
    const int a = tid + i * kBucketThreads;
    if (a < A) place(eid[i], a);
  }
  for (int a = tid + kIdCache * kBucketThreads; a < A; a += kBucketThreads)
    place(expert_of(g.ids, a, E), a);
}

// The bucketing, by one block of kBucketThreads.  Bucket position of assignment a = (t, j)
// routed to e is offsets[e] + (tokens t' < t routed to e), so each bucket lists its
// assignments by ascending token.  Tokens are taken in passes of kPassTokens: a bitmask per
// expert marks the pass's tokens routed to it, popcounts of the words give the rank at each
// word's start, and the rank of (t, j) adds the popcount of the bits below t in its word.
// With one pass the counts come from the bitmasks; with several, from a histogram first.
__device__ void bucket_all(const BucketArgs& g, BucketShared& sh) {
  if (g.T <= kPassTokens) {
    bucket_one_pass(g, sh);
    return;
  }
  const int tid = threadIdx.x;
  const int T = g.T, k = g.k, E = g.E, A = T * k;
  const int Ep = E <= 64 ? 64 : (E <= 128 ? 128 : 256);
  const int npass = (T + kPassTokens - 1) / kPassTokens;
  int run = 0;                                  // thread e < E: rank reached by earlier passes
  if (npass > 1) {
    if (tid < kMaxE) sh.cnt[tid] = 0;
    __syncthreads();
    for (int a = tid; a < A; a += kBucketThreads) atomicAdd(&sh.cnt[expert_of(g.ids, a, E)], 1);
    __syncthreads();
    expert_scan(tid < E ? sh.cnt[tid] : 0, E, Ep, A, sh, g.offsets, g.items);
  }
  for (int p = 0; p < npass; ++p) {
    const int t0 = p * kPassTokens;
    const int nt = min(kPassTokens, T - t0);
    const int W = (nt + 63) / 64;
    for (int i = tid; i < E * kPassWords; i += kBucketThreads) sh.bits[i] = 0ull;
    __syncthreads();
    const int a0 = t0 * k, a1 = (t0 + nt) * k;
    for (int a = a0 + tid; a < a1; a += kBucketThreads) {
      const int lt = a / k - t0;
      atomicOr(&sh.bits[expert_of(g.ids, a, E) * kPassWords + (lt >> 6)], 1ull << (lt & 63));
    }
    __syncthreads();
    if (tid < E) {
      for (int w = 0; w < W; ++w) {
        sh.wpre[tid * kPassWords + w] = run;
        run += __popcll(sh.bits[tid * kPassWords + w]);
      }
    }
    if (npass == 1) expert_scan(tid < E ? run : 0, E, Ep, A, sh, g.offsets, g.items);
    __syncthreads();
    for (int a = a0 + tid; a < a1; a += kBucketThreads) {
      const int e = expert_of(g.ids, a, E);
      const int lt = a / k - t0;
      const int w = e * kPassWords + (lt >> 6);
      const int rank = sh.wpre[w] + __popcll(sh.bits[w] & ((1ull << (lt & 63)) - 1ull));
      g.perm[sh.eoff[e] + rank] = a;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kBucketThreads) void bucket_kernel(BucketArgs g) {
  if (gated_off(g.gate)) return;
  __shared__ BucketShared sh;
  bucket_all(g, sh);
}

// x -> xp with every 8 consecutive halves in the GEMMs' k-order (for the tile kernel, which
// moves activations HBM -> LDS without passing through registers).
__global__ __launch_bounds__(kBucketThreads) void permute_kernel(const u32x4_t* __restrict__ x,
                                                                 u32x4_t* __restrict__ xp, int n8,
                                                                 const int32_t* __restrict__ gate) {
  if (gated_off(gate)) return;
  const int i = blockIdx.x * kBucketThreads + threadIdx.x;
  if (i < n8) xp[i] = permute8(x[i]);
}

}  // namespace

int moe_max_items(int T, int E, int k) {
  const int A = T * k;
  return A / kItemTokens + (E < A ? E : A);
}

size_t moe_workspace_bytes(int T, int E, int k, int d_model, int d_ff) {
  const size_t A = (size_t)T * k;
  return align_up((size_t)(E + 1) * 4) + align_up((size_t)(1 + 3 * moe_max_items(T, E, k)) * 4) +
         align_up(A * 4) + align_up(A * (size_t)d_ff * 2) + align_up((size_t)T * d_model * 2) +
         align_up(A * 4);
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
  p += align_up((size_t)T * d_model * 2);
  ws.ids = reinterpret_cast<int32_t*>(p);
  return ws;
}

hipError_t launch_route(const float* router_logits, int T, int E, int k, int32_t* topk_ids,
                        float* topk_weights, const MoeWorkspace& ws, hipStream_t stream,
                        const int32_t* gate) {
  hipLaunchKernelGGL(topk_kernel, dim3(T), dim3(kTopkThreads), 0, stream, router_logits, T, E, k,
                     topk_ids, ws.ids, topk_weights, gate);
  BucketArgs g;
  g.ids = ws.ids;
  g.T = T;
  g.k = k;
  g.E = E;
  g.offsets = ws.offsets;
  g.items = ws.items;
  g.perm = ws.perm;
  g.gate = gate;
  hipLaunchKernelGGL(bucket_kernel, dim3(1), dim3(kBucketThreads), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_permute(int T, const uint16_t* x, int d_model, const MoeWorkspace& ws,
                          hipStream_t stream, const int32_t* gate) {
  const int n8 = T * d_model / 8;
  hipLaunchKernelGGL(permute_kernel, dim3((n8 + kBucketThreads - 1) / kBucketThreads),
                     dim3(kBucketThreads), 0, stream, reinterpret_cast<const u32x4_t*>(x),
                     reinterpret_cast<u32x4_t*>(ws.xp), n8, gate);
  return hipGetLastError();
}

}  // namespace bd
