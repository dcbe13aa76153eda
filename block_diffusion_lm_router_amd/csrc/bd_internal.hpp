// Host/device declarations shared between the kernels' translation units and the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bd {

inline size_t align_up(size_t n, size_t a = 256) { return (n + a - 1) / a * a; }

// Partial state of one V-split of one row (56 bytes): the entropy sums, the temperature-0
// argmax and the split's best two level-1 draws.
struct PartState {
  float m;            // reference maximum (-inf: empty)
  float n;            // entries equal to m
  float s;            // sum of exp(x - m) over the other entries
  float t;            // sum of exp(x - m) (x - m)
  float best_v;       // temperature-0 argmax value
  int best_i;         // and its lowest index
  int nan;            // a NaN was seen where no finite entry could carry it
  int best_c;         // chunk of the largest level-1 key (lowest chunk on ties)
  int second_c;       // chunk of the second largest
  double best_key;    // the largest key, L_c + G_c (-inf: none)
  double second_key;  // the second largest (-inf: none)
};

// ---------------------------------------------------------------- MoE
#ifndef BD_ITEM_TOKENS
#define BD_ITEM_TOKENS 32
#endif
constexpr int kItemTokens = BD_ITEM_TOKENS;  // tokens per work item of the grouped GEMMs (16 or 32)

struct MoeWorkspace {
  int32_t* offsets;  // [E + 1] bucket starts
  int32_t* items;    // [0] = count, then (expert, first bucket position, tokens) triples
  int32_t* perm;     // [T * k] assignment index t*k + j at each bucket position
  uint16_t* h;       // [T * k][d_ff] fp16 GeGLU activations, bucket order, k-permuted
  uint16_t* xp;      // [T][d_model] fp16 activations with k permuted within blocks of 8
  int32_t* ids;      // [T * k] copy of the top-k expert ids
  int max_items;
};

int moe_max_items(int T, int E, int k);
size_t moe_workspace_bytes(int T, int E, int k, int d_model, int d_ff);
MoeWorkspace moe_workspace_carve(void* base, int T, int E, int k, int d_model, int d_ff);

// Top-k ids and weights (the ids also into ws.ids), then the stable grouping of the
// assignments by expert and the work list into ws (a second, one-block launch).
// Every launcher below that takes `gate` (NULL: always run) launches kernels that return at
// once when gate[2] (a loop driver's done flag) is set.
hipError_t launch_route(const float* router_logits, int T, int E, int k, int32_t* topk_ids,
                        float* topk_weights, const MoeWorkspace& ws, hipStream_t stream,
                        const int32_t* gate = nullptr);
// x permuted into ws.xp (the k-order of the dequantised nibbles), for the tile kernel.
hipError_t launch_permute(int T, const uint16_t* x, int d_model, const MoeWorkspace& ws,
                          hipStream_t stream, const int32_t* gate = nullptr);

struct W4A16Matrix {
  const uint8_t* q;
  const uint16_t* scale;
  const uint16_t* zero;
  const uint8_t* pk;    // packed stream for the 256-row tiles, or nullptr
  int group;            // group size of scale/zero (64, or 128 for repacking only)
  int affine;           // zero holds the bias b of w = q s + b (packed stream only)
};

int pk_tiles(bool gated, int d_model, int d_ff);
// The gate/up stream of a matrix grouped at 128 holds one (scale, zero) pair per row and stage.
bool pk_compact(bool gated, int group);
size_t pk_bytes(bool gated, int E, int d_model, int d_ff, bool compact);
hipError_t launch_pack(const W4A16Matrix& m, bool gated, int E, int d_model, int d_ff,
                       uint8_t* out, hipStream_t stream);

hipError_t launch_gate_up(const W4A16Matrix& gu, int E, int d_model, int d_ff, int top_k, int T,
                          const uint16_t* x, const MoeWorkspace& ws, hipStream_t stream,
                          const int32_t* gate = nullptr);
hipError_t launch_down(const W4A16Matrix& dn, int E, int d_model, int d_ff, int top_k, int T,
                       float* expert_out, const MoeWorkspace& ws, hipStream_t stream,
                       const int32_t* gate = nullptr);
hipError_t launch_combine(const float* expert_out, const float* topk_weights, int T, int k, int d,
                          uint16_t* y, hipStream_t stream, const int32_t* gate = nullptr);
// The combine, then the RMS norm of its output rows with `weight` into xn (one block per row,
// d % 8 == 0, d <= 4096); both outputs equal launch_combine followed by launch_rmsnorm.
hipError_t launch_combine_norm(const float* expert_out, const float* topk_weights, int T, int k,
                               int d, const uint16_t* weight, float eps, uint16_t* y, uint16_t* xn,
                               hipStream_t stream, const int32_t* gate);

// RMS norm of fp16 rows (one wave per row) and the router projection (MFMA, split-K).
hipError_t launch_rmsnorm(const uint16_t* h, const uint16_t* weight, int T, int d, float eps,
                          uint16_t* y, hipStream_t stream, const int32_t* gate = nullptr);
hipError_t launch_router(const uint16_t* x, const uint16_t* w_router, int T, int d, int E,
                         float* logits, hipStream_t stream, const int32_t* gate = nullptr);

// ---------------------------------------------------------------- sampler
int sample_split_count(int P, int V);
size_t sample_workspace_bytes(int P, int V);
hipError_t launch_sample_entropy(const float* logits, int P, int V, float temperature,
                                 uint64_t seed, uint32_t step, const uint8_t* frozen,
                                 int32_t* tokens_out, float* entropy_out, float* conf_out,
                                 void* workspace, hipStream_t stream,
                                 const int32_t* gate = nullptr);
// The per-device address of the static split-state array (for the allocation-free entry
// point); hipErrorInvalidValue if `need` bytes do not fit it.
hipError_t static_sample_scratch(size_t need, void** out);
hipError_t launch_accept(const float* entropy, const int32_t* tokens, int P, float bound,
                         uint8_t* frozen, int32_t* canvas, uint8_t* accept_out,
                         int32_t* num_accepted, hipStream_t stream,
                         const int32_t* gate = nullptr);
hipError_t launch_accept_confidence(const float* conf, const int32_t* tokens, int P,
                                    float threshold, uint8_t* frozen, int32_t* canvas,
                                    uint8_t* accept_out, int32_t* num_accepted,
                                    hipStream_t stream, const int32_t* gate = nullptr);

// ---------------------------------------------------------------- denoising-loop driver
hipError_t launch_canvas_init(int32_t* canvas, int32_t* prev, uint8_t* frozen, int32_t* state,
                              int P, int vocab, uint64_t seed, uint32_t block,
                              hipStream_t stream);
hipError_t launch_loop_update(const int32_t* tokens, int32_t* canvas, int32_t* prev,
                              const uint8_t* frozen, int32_t* state, int P, int threshold,
                              int max_steps, int write_drafts, hipStream_t stream);

// ---------------------------------------------------------------- measurement
hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);
hipError_t launch_read(const void* src, size_t bytes, uint32_t* checksum, hipStream_t stream);

}  // namespace bd
