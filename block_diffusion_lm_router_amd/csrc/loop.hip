// Denoising-loop driver kernels around the per-step sampler: the random initial canvas of a
// block and the per-step stability update that ends a block early.
//
// Source: DiffusionGemma block-diffusion page, "How it works" (the canvas starts from seeded
// random ids; a block ends early once its canvas has stayed the same for stability_threshold
// steps in a row), "CLI flags" (step budget).
//
// Both kernels keep the driver's state on the device (int32 [4]: steps run, consecutive
// unchanged steps, done, frozen count) so a host loop needs no synchronisation to advance
// it.  The init kernel also clears that state, so a block's start needs no memset.

#include "bd_device.hpp"
#include "bd_internal.hpp"

namespace bd {

namespace {

constexpr int kInitThreads = 256;
constexpr int kLoopThreads = 1024;
enum { kStep = 0, kStable = 1, kDone = 2, kNFrozen = 3 };

// Position p of block b draws Philox counter (p, b, 0, 2) word 0 and maps it to [0, vocab)
// by multiply-shift: floor(word * vocab / 2^32).
__global__ __launch_bounds__(kInitThreads) void canvas_init_kernel(
    int32_t* __restrict__ canvas, int32_t* __restrict__ prev, uint8_t* __restrict__ frozen,
    int32_t* __restrict__ state, int P, uint32_t vocab, uint32_t k0, uint32_t k1, uint32_t block) {
  const int p = blockIdx.x * kInitThreads + threadIdx.x;
  if (p == 0) {
    state[kStep] = 0;
    state[kStable] = 0;
    state[kDone] = 0;
    state[kNFrozen] = 0;
  }
  if (p >= P) return;
  const Philox4 r = philox4x32_10((uint32_t)p, block, 0u, 2u, k0, k1);
  const int32_t id = (int32_t)(((uint64_t)r.w[0] * vocab) >> 32);
  canvas[p] = id;
  prev[p] = id;
  frozen[p] = 0;
}

// One block of up to 1024 threads, one position per thread.  A finished block is left as is.
__global__ __launch_bounds__(kLoopThreads) void loop_update_kernel(
    const int32_t* __restrict__ tokens, int32_t* __restrict__ canvas, int32_t* __restrict__ prev,
    const uint8_t* __restrict__ frozen, int32_t* __restrict__ state, int P, int threshold,
    int max_steps, int write_drafts) {
  const int p = threadIdx.x;
  const int done = state[kDone];
  __syncthreads();  // every thread has read the flag before thread 0 may rewrite it
  if (done) return;
  bool changed = false, fz = false;
  if (p < P) {
    int32_t c = canvas[p];
    if (write_drafts) {
      const int32_t t = tokens[p];
      if (t >= 0) {
        c = t;
        canvas[p] = t;
      }
    }
    changed = c != prev[p];
    prev[p] = c;
    fz = frozen[p] != 0;
  }
  const int any_changed = __syncthreads_or(changed);
  const int n_frozen = __syncthreads_count(fz);
  if (p == 0) {
    const int step = state[kStep] + 1;
    const int stable = any_changed ? 0 : state[kStable] + 1;
    state[kStep] = step;
    state[kStable] = stable;
    state[kNFrozen] = n_frozen;
    state[kDone] = (stable >= threshold || n_frozen == P || step >= max_steps) ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_canvas_init(int32_t* canvas, int32_t* prev, uint8_t* frozen, int32_t* state,
                              int P, int vocab, uint64_t seed, uint32_t block,
                              hipStream_t stream) {
  const int blocks = (P + kInitThreads - 1) / kInitThreads;
  hipLaunchKernelGGL(canvas_init_kernel, dim3(blocks), dim3(kInitThreads), 0, stream, canvas, prev,
                     frozen, state, P, (uint32_t)vocab, (uint32_t)(seed & 0xffffffffu),
                     (uint32_t)(seed >> 32), block);
  return hipGetLastError();
}

hipError_t launch_loop_update(const int32_t* tokens, int32_t* canvas, int32_t* prev,
                              const uint8_t* frozen, int32_t* state, int P, int threshold,
                              int max_steps, int write_drafts, hipStream_t stream) {
  int threads = kWave;
  while (threads < P) threads <<= 1;
  hipLaunchKernelGGL(loop_update_kernel, dim3(1), dim3(threads), 0, stream, tokens, canvas, prev,
                     frozen, state, P, threshold, max_steps, write_drafts);
  return hipGetLastError();
}

}  // namespace bd
