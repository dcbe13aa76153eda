// C ABI of libbdstep: host-side validation, workspace carving and kernel launches.
// Every check runs before the first launch, so a failing call enqueues nothing.

#include <math.h>

#include "../../include/bdstep.h"
#include "bd_internal.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int to_status(hipError_t err) { return err == hipSuccess ? BD_OK : BD_ERR_HIP; }


int check_moe_shape(const bd_moe_weights* w, int T) {
  if (w == nullptr) return BD_ERR_NULL;
  if (T < 1 || T > BD_MAX_TOKENS) return BD_ERR_SHAPE;
  if (w->num_experts < 1 || w->num_experts > BD_MAX_EXPERTS) return BD_ERR_SHAPE;
  if (w->top_k < 1 || w->top_k > BD_MAX_TOPK || w->top_k > w->num_experts) return BD_ERR_SHAPE;
  if (w->d_model < 1 || w->d_ff < 1) return BD_ERR_SHAPE;
  const int gd = w->down_group_size ? w->down_group_size : w->group_size;
  if ((w->group_size != 64 && w->group_size != 128) || (gd != 64 && gd != 128))
    return BD_ERR_UNSUPPORTED;
  if (w->d_model % 128 != 0 || w->d_ff % 64 != 0) return BD_ERR_UNSUPPORTED;
  if (w->d_model % w->group_size != 0 || w->d_ff % gd != 0) return BD_ERR_SHAPE;
  if (w->format != BD_FORMAT_ASYMMETRIC && w->format != BD_FORMAT_AFFINE) return BD_ERR_UNSUPPORTED;
  if (w->d_model > 4096 || w->d_ff > 4096) return BD_ERR_UNSUPPORTED;  // per-block scale table
  if ((int64_t)T * w->top_k > (int64_t)BD_MAX_TOKENS * BD_MAX_TOPK) return BD_ERR_SHAPE;
  return BD_OK;
}

int check_workspace(const void* ws, size_t have, size_t need) {
  if (ws == nullptr) return BD_ERR_NULL;
  if (!aligned16(ws)) return BD_ERR_ALIGN;
  if (have < need) return BD_ERR_WORKSPACE;
  return BD_OK;
}

// A matrix is usable by the GEMMs through its packed stream (then the raw arrays may be NULL)
// or through its raw nibble, scale and zero-point arrays.
int check_matrix(const uint8_t* q, const uint16_t* scale, const uint16_t* zero,
                 const uint8_t* packed, int group, int format) {
  if (packed) return aligned16(packed) ? BD_OK : BD_ERR_ALIGN;
  // 128-groups and the affine form go through the packed stream only
  if (group != 64 || format != BD_FORMAT_ASYMMETRIC) return BD_ERR_UNSUPPORTED;
  if (!q || !scale || !zero) return BD_ERR_NULL;
  if (!aligned16(q) || !aligned16(scale) || !aligned16(zero)) return BD_ERR_ALIGN;
  return BD_OK;
}

int down_group(const bd_moe_weights* w) {
  return w->down_group_size ? w->down_group_size : w->group_size;
}

int check_gate_up_weights(const bd_moe_weights* w) {
  return check_matrix(w->gate_up_q, w->gate_up_scale, w->gate_up_zero, w->gate_up_packed,
                      w->group_size, w->format);
}

int check_down_weights(const bd_moe_weights* w) {
  return check_matrix(w->down_q, w->down_scale, w->down_zero, w->down_packed, down_group(w),
                      w->format);
}

bd::W4A16Matrix gate_up_of(const bd_moe_weights* w) {
  return bd::W4A16Matrix{w->gate_up_q, w->gate_up_scale, w->gate_up_zero, w->gate_up_packed,
                         w->group_size, w->format == BD_FORMAT_AFFINE ? 1 : 0};
}
bd::W4A16Matrix down_of(const bd_moe_weights* w) {
  return bd::W4A16Matrix{w->down_q, w->down_scale, w->down_zero, w->down_packed, down_group(w),
                         w->format == BD_FORMAT_AFFINE ? 1 : 0};
}

int check_sample_shape(int P, int V, float temperature) {
  if (P < 1 || P > BD_MAX_POSITIONS) return BD_ERR_SHAPE;
  if (V < 1 || V > BD_MAX_VOCAB) return BD_ERR_SHAPE;
  if (!(temperature >= 0.f) || !isfinite(temperature)) return BD_ERR_SHAPE;
  if (temperature > 0.f && !isfinite(1.f / temperature)) return BD_ERR_SHAPE;  // 1/T overflows
  return BD_OK;
}

}  // namespace

extern "C" {

int bd_abi_version(void) { return BD_ABI_VERSION; }

const char* bd_status_string(int status) {
  switch (status) {
    case BD_OK: return "ok";
    case BD_ERR_NULL: return "a required pointer is NULL";
    case BD_ERR_SHAPE: return "a size is out of range or inconsistent";
    case BD_ERR_ALIGN: return "a pointer is not aligned as the ABI requires";
    case BD_ERR_WORKSPACE: return "workspace missing or smaller than required";
    case BD_ERR_UNSUPPORTED: return "shape or format not supported by this build";
    case BD_ERR_HIP: return "a HIP launch or runtime call failed";
    default: return "unknown status";
  }
}

size_t bd_moe_packed_size(const bd_moe_weights* w, int matrix) {
  if (check_moe_shape(w, 1) != BD_OK || (matrix != 0 && matrix != 1)) return 0;
  const bool gated = matrix == 0;
  return bd::pk_bytes(gated, w->num_experts, w->d_model, w->d_ff,
                      bd::pk_compact(gated, gated ? w->group_size : down_group(w)));
}

int moe_w4a16_prepare(const bd_moe_weights* w, uint8_t* gate_up_packed, uint8_t* down_packed,
                      hipStream_t stream) {
  int st = check_moe_shape(w, 1);
  if (st != BD_OK) return st;
  if (!gate_up_packed || !down_packed || !w->gate_up_q || !w->gate_up_scale ||
      !w->gate_up_zero || !w->down_q || !w->down_scale || !w->down_zero)
    return BD_ERR_NULL;
  if (!aligned16(gate_up_packed) || !aligned16(down_packed) || !aligned16(w->gate_up_q) ||
      !aligned16(w->down_q))
    return BD_ERR_ALIGN;
  bd::W4A16Matrix gu = gate_up_of(w), dn = down_of(w);
  gu.pk = nullptr;
  dn.pk = nullptr;
  st = to_status(bd::launch_pack(gu, true, w->num_experts, w->d_model, w->d_ff, gate_up_packed,
                                 stream));
  if (st != BD_OK) return st;
  return to_status(bd::launch_pack(dn, false, w->num_experts, w->d_model, w->d_ff, down_packed,
                                   stream));
}

size_t bd_moe_workspace_size(int T, const bd_moe_weights* w) {
  if (check_moe_shape(w, T) != BD_OK) return 0;
  return bd::moe_workspace_bytes(T, w->num_experts, w->top_k, w->d_model, w->d_ff);
}

size_t bd_moe_w4a16_ffn_workspace_size(int T, const bd_moe_weights* w) {
  return bd_moe_workspace_size(T, w);
}

int moe_route_topk(const bd_moe_weights* w, int T, const float* router_logits, int32_t* topk_ids,
                   float* topk_weights, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_moe_shape(w, T);
  if (st != BD_OK) return st;
  if (!router_logits || !topk_ids || !topk_weights) return BD_ERR_NULL;
  if (!aligned4(router_logits) || !aligned4(topk_ids) || !aligned4(topk_weights))
    return BD_ERR_ALIGN;
  st = check_workspace(workspace, workspace_bytes, bd_moe_workspace_size(T, w));
  if (st != BD_OK) return st;
  const bd::MoeWorkspace ws =
      bd::moe_workspace_carve(workspace, T, w->num_experts, w->top_k, w->d_model, w->d_ff);
  return to_status(bd::launch_route(router_logits, T, w->num_experts, w->top_k, topk_ids,
                                    topk_weights, ws, stream));
}

int moe_w4a16_gate_up(const bd_moe_weights* w, int T, const uint16_t* x, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  int st = check_moe_shape(w, T);
  if (st != BD_OK) return st;
  if ((st = check_gate_up_weights(w)) != BD_OK) return st;
  if (!x) return BD_ERR_NULL;
  if (!aligned16(x)) return BD_ERR_ALIGN;
  st = check_workspace(workspace, workspace_bytes, bd_moe_workspace_size(T, w));
  if (st != BD_OK) return st;
  const bd::MoeWorkspace ws =
      bd::moe_workspace_carve(workspace, T, w->num_experts, w->top_k, w->d_model, w->d_ff);
  return to_status(bd::launch_gate_up(gate_up_of(w), w->num_experts, w->d_model, w->d_ff,
                                      w->top_k, T, x, ws, stream));
}

int moe_w4a16_down(const bd_moe_weights* w, int T, float* expert_out, void* workspace,
                   size_t workspace_bytes, hipStream_t stream) {
  int st = check_moe_shape(w, T);
  if (st != BD_OK) return st;
  if ((st = check_down_weights(w)) != BD_OK) return st;
  if (!expert_out) return BD_ERR_NULL;
  if (!aligned16(expert_out)) return BD_ERR_ALIGN;
  st = check_workspace(workspace, workspace_bytes, bd_moe_workspace_size(T, w));
  if (st != BD_OK) return st;
  const bd::MoeWorkspace ws =
      bd::moe_workspace_carve(workspace, T, w->num_experts, w->top_k, w->d_model, w->d_ff);
  return to_status(bd::launch_down(down_of(w), w->num_experts, w->d_model, w->d_ff, w->top_k, T,
                                   expert_out, ws, stream));
}

static int ffn_call(const bd_moe_weights* w, int T, const uint16_t* x, const float* router_logits,
                    int32_t* topk_ids, float* topk_weights, float* expert_out, void* workspace,
                    size_t workspace_bytes, const int32_t* gate, hipStream_t stream) {
  int st = check_moe_shape(w, T);
  if (st != BD_OK) return st;
  if ((st = check_gate_up_weights(w)) != BD_OK) return st;
  if ((st = check_down_weights(w)) != BD_OK) return st;
  if (!x || !router_logits || !topk_ids || !topk_weights || !expert_out) return BD_ERR_NULL;
  if (!aligned16(x) || !aligned4(router_logits) || !aligned4(topk_ids) ||
      !aligned4(topk_weights) || !aligned16(expert_out))
    return BD_ERR_ALIGN;
  st = check_workspace(workspace, workspace_bytes, bd_moe_workspace_size(T, w));
  if (st != BD_OK) return st;
  const bd::MoeWorkspace ws =
      bd::moe_workspace_carve(workspace, T, w->num_experts, w->top_k, w->d_model, w->d_ff);
  hipStream_t s = stream;
  hipError_t err = bd::launch_route(router_logits, T, w->num_experts, w->top_k, topk_ids,
                                    topk_weights, ws, s, gate);
  if (err == hipSuccess)
    err = bd::launch_gate_up(gate_up_of(w), w->num_experts, w->d_model, w->d_ff, w->top_k, T, x,
                             ws, s, gate);
  if (err == hipSuccess)
    err = bd::launch_down(down_of(w), w->num_experts, w->d_model, w->d_ff, w->top_k, T,
                          expert_out, ws, s, gate);
  return to_status(err);
}

int moe_w4a16_ffn(const bd_moe_weights* w, int T, const uint16_t* x, const float* router_logits,
                  int32_t* topk_ids, float* topk_weights, float* expert_out, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  return ffn_call(w, T, x, router_logits, topk_ids, topk_weights, expert_out, workspace,
                  workspace_bytes, nullptr, stream);
}

int moe_w4a16_ffn_gated(const bd_moe_weights* w, int T, const uint16_t* x,
                        const float* router_logits, int32_t* topk_ids, float* topk_weights,
                        float* expert_out, void* workspace, size_t workspace_bytes,
                        const int32_t* loop_state, hipStream_t stream) {
  if (!loop_state) return BD_ERR_NULL;
  if (!aligned4(loop_state)) return BD_ERR_ALIGN;
  return ffn_call(w, T, x, router_logits, topk_ids, topk_weights, expert_out, workspace,
                  workspace_bytes, loop_state, stream);
}

static int combine_call(const float* expert_out, const float* topk_weights, int T, int k, int d,
                        uint16_t* y, const int32_t* gate, hipStream_t stream) {
  if (!expert_out || !topk_weights || !y) return BD_ERR_NULL;
  if (T < 1 || T > BD_MAX_TOKENS || k < 1 || k > BD_MAX_TOPK || d < 4 || d % 4 != 0)
    return BD_ERR_SHAPE;
  if (!aligned16(expert_out) || !aligned4(topk_weights) || !aligned16(y)) return BD_ERR_ALIGN;
  return to_status(bd::launch_combine(expert_out, topk_weights, T, k, d, y, stream, gate));
}

int moe_combine_fixed_order(const float* expert_out, const float* topk_weights, int T, int k,
                            int d, uint16_t* y, hipStream_t stream) {
  return combine_call(expert_out, topk_weights, T, k, d, y, nullptr, stream);
}

int moe_combine_fixed_order_gated(const float* expert_out, const float* topk_weights, int T,
                                  int k, int d, uint16_t* y, const int32_t* loop_state,
                                  hipStream_t stream) {
  if (!loop_state) return BD_ERR_NULL;
  if (!aligned4(loop_state)) return BD_ERR_ALIGN;
  return combine_call(expert_out, topk_weights, T, k, d, y, loop_state, stream);
}

static int rmsnorm_call(const uint16_t* h, const uint16_t* weight, int T, int d, float eps,
                        uint16_t* y, const int32_t* gate, hipStream_t stream) {
  if (T < 1 || T > BD_MAX_TOKENS || d < 8 || d > BD_MAX_FEATURES || d % 8 != 0 ||
      !isfinite(eps) || eps < 0.f)
    return BD_ERR_SHAPE;
  if (!h || !weight || !y) return BD_ERR_NULL;
  if (!aligned16(h) || !aligned16(weight) || !aligned16(y)) return BD_ERR_ALIGN;
  return to_status(bd::launch_rmsnorm(h, weight, T, d, eps, y, stream, gate));
}

int moe_rmsnorm(const uint16_t* h, const uint16_t* weight, int T, int d, float eps, uint16_t* y,
                hipStream_t stream) {
  return rmsnorm_call(h, weight, T, d, eps, y, nullptr, stream);
}

int moe_rmsnorm_gated(const uint16_t* h, const uint16_t* weight, int T, int d, float eps,
                      uint16_t* y, const int32_t* loop_state, hipStream_t stream) {
  if (!loop_state) return BD_ERR_NULL;
  if (!aligned4(loop_state)) return BD_ERR_ALIGN;
  return rmsnorm_call(h, weight, T, d, eps, y, loop_state, stream);
}

static int combine_norm_call(const float* expert_out, const float* topk_weights, int T, int k,
                             int d, const uint16_t* weight, float eps, uint16_t* y, uint16_t* xn,
                             const int32_t* gate, hipStream_t stream) {
  if (!expert_out || !topk_weights || !weight || !y || !xn) return BD_ERR_NULL;
  if (T < 1 || T > BD_MAX_TOKENS || k < 1 || k > BD_MAX_TOPK || d < 8 || d > BD_MAX_FEATURES ||
      d % 8 != 0 || !isfinite(eps) || eps < 0.f)
    return BD_ERR_SHAPE;
  if (!aligned16(expert_out) || !aligned4(topk_weights) || !aligned16(weight) || !aligned16(y) ||
      !aligned16(xn))
    return BD_ERR_ALIGN;
  return to_status(
      bd::launch_combine_norm(expert_out, topk_weights, T, k, d, weight, eps, y, xn, stream, gate));
}

int moe_combine_rmsnorm(const float* expert_out, const float* topk_weights, int T, int k, int d,
                        const uint16_t* weight, float eps, uint16_t* y, uint16_t* xn,
                        hipStream_t stream) {
  return combine_norm_call(expert_out, topk_weights, T, k, d, weight, eps, y, xn, nullptr, stream);
}

int moe_combine_rmsnorm_gated(const float* expert_out, const float* topk_weights, int T, int k,
                              int d, const uint16_t* weight, float eps, uint16_t* y, uint16_t* xn,
                              const int32_t* loop_state, hipStream_t stream) {
  if (!loop_state) return BD_ERR_NULL;
  if (!aligned4(loop_state)) return BD_ERR_ALIGN;
  return combine_norm_call(expert_out, topk_weights, T, k, d, weight, eps, y, xn, loop_state,
                           stream);
}

static int router_call(const uint16_t* x, const uint16_t* w_router, int T, int d, int E,
                       float* logits, const int32_t* gate, hipStream_t stream) {
  if (T < 1 || T > BD_MAX_TOKENS || E < 1 || E > BD_MAX_EXPERTS || d < 128 ||
      d > BD_MAX_FEATURES || d % 128 != 0)
    return BD_ERR_SHAPE;
  if (!x || !w_router || !logits) return BD_ERR_NULL;
  if (!aligned16(x) || !aligned16(w_router) || !aligned4(logits)) return BD_ERR_ALIGN;
  return to_status(bd::launch_router(x, w_router, T, d, E, logits, stream, gate));
}

int moe_router_logits(const uint16_t* x, const uint16_t* w_router, int T, int d, int E,
                      float* logits, hipStream_t stream) {
  return router_call(x, w_router, T, d, E, logits, nullptr, stream);
}

int moe_router_logits_gated(const uint16_t* x, const uint16_t* w_router, int T, int d, int E,
                            float* logits, const int32_t* loop_state, hipStream_t stream) {
  if (!loop_state) return BD_ERR_NULL;
  if (!aligned4(loop_state)) return BD_ERR_ALIGN;
  return router_call(x, w_router, T, d, E, logits, loop_state, stream);
}

size_t bd_sample_workspace_size(int P, int V) {
  if (check_sample_shape(P, V, 0.f) != BD_OK) return 0;
  return bd::sample_workspace_bytes(P, V);
}

int diffusion_sample_entropy(const float* logits, int P, int V, float temperature, uint64_t seed,
                             uint32_t step, const uint8_t* frozen, int32_t* tokens_out,
                             float* entropy_out, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  int st = check_sample_shape(P, V, temperature);
  if (st != BD_OK) return st;
  if (!logits || !tokens_out || !entropy_out) return BD_ERR_NULL;
  if (!aligned16(logits) || !aligned4(tokens_out) || !aligned4(entropy_out)) return BD_ERR_ALIGN;
  st = check_workspace(workspace, workspace_bytes, bd::sample_workspace_bytes(P, V));
  if (st != BD_OK) return st;
  return to_status(bd::launch_sample_entropy(logits, P, V, temperature, seed, step, frozen,
                                             tokens_out, entropy_out, nullptr, workspace,
                                             stream));
}

int diffusion_accept_entropy_bound(const float* entropy, const int32_t* tokens, int P, float bound,
                                   uint8_t* frozen, int32_t* canvas, uint8_t* accept_out,
                                   int32_t* num_accepted, hipStream_t stream) {
  if (P < 1 || P > BD_MAX_POSITIONS || !isfinite(bound)) return BD_ERR_SHAPE;
  if (!entropy || !tokens || !accept_out || !num_accepted) return BD_ERR_NULL;
  if (!aligned4(entropy) || !aligned4(tokens) || !aligned4(num_accepted) ||
      (canvas && !aligned4(canvas)))
    return BD_ERR_ALIGN;
  return to_status(bd::launch_accept(entropy, tokens, P, bound, frozen, canvas, accept_out,
                                     num_accepted, stream));
}

static int step_call(const float* logits, int P, int V, float temperature, float entropy_bound,
                     uint64_t seed, uint32_t step, uint8_t* frozen, int32_t* canvas,
                     int32_t* tokens_out, float* entropy_out, uint8_t* accept_out,
                     int32_t* num_accepted, void* workspace, size_t workspace_bytes,
                     const int32_t* gate, hipStream_t stream) {
  int st = check_sample_shape(P, V, temperature);
  if (st != BD_OK) return st;
  if (!isfinite(entropy_bound)) return BD_ERR_SHAPE;
  if (!logits || !tokens_out || !entropy_out || !accept_out || !num_accepted) return BD_ERR_NULL;
  if (!aligned16(logits) || !aligned4(tokens_out) || !aligned4(entropy_out) ||
      !aligned4(num_accepted) || (canvas && !aligned4(canvas)))
    return BD_ERR_ALIGN;
  st = check_workspace(workspace, workspace_bytes, bd::sample_workspace_bytes(P, V));
  if (st != BD_OK) return st;
  hipStream_t s = stream;
  hipError_t err = bd::launch_sample_entropy(logits, P, V, temperature, seed, step, frozen,
                                             tokens_out, entropy_out, nullptr, workspace, s,
                                             gate);
  if (err == hipSuccess)
    err = bd::launch_accept(entropy_out, tokens_out, P, entropy_bound, frozen, canvas, accept_out,
                            num_accepted, s, gate);
  return to_status(err);
}

int diffusion_sample_step(const float* logits, int P, int V, float temperature,
                          float entropy_bound, uint64_t seed, uint32_t step, uint8_t* frozen,
                          int32_t* canvas, int32_t* tokens_out, float* entropy_out,
                          uint8_t* accept_out, int32_t* num_accepted, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  return step_call(logits, P, V, temperature, entropy_bound, seed, step, frozen, canvas,
                   tokens_out, entropy_out, accept_out, num_accepted, workspace, workspace_bytes,
                   nullptr, stream);
}

int diffusion_sample_step_gated(const float* logits, int P, int V, float temperature,
                                float entropy_bound, uint64_t seed, uint32_t step,
                                uint8_t* frozen, int32_t* canvas, int32_t* tokens_out,
                                float* entropy_out, uint8_t* accept_out, int32_t* num_accepted,
                                void* workspace, size_t workspace_bytes,
                                const int32_t* loop_state, hipStream_t stream) {
  if (!loop_state) return BD_ERR_NULL;
  if (!aligned4(loop_state)) return BD_ERR_ALIGN;
  return step_call(logits, P, V, temperature, entropy_bound, seed, step, frozen, canvas,
                   tokens_out, entropy_out, accept_out, num_accepted, workspace, workspace_bytes,
                   loop_state, stream);
}

int diffusion_sample_step_noalloc(const float* logits, int P, int V, float temperature,
                                  float entropy_bound, uint64_t seed, uint32_t step,
                                  uint8_t* frozen, int32_t* canvas, int32_t* tokens_out,
                                  float* entropy_out, uint8_t* accept_out, int32_t* num_accepted,
                                  hipStream_t stream) {
  int st = check_sample_shape(P, V, temperature);
  if (st != BD_OK) return st;
  if (!isfinite(entropy_bound)) return BD_ERR_SHAPE;
  if (!logits || !tokens_out || !entropy_out || !accept_out || !num_accepted) return BD_ERR_NULL;
  if (!aligned16(logits) || !aligned4(tokens_out) || !aligned4(entropy_out) ||
      !aligned4(num_accepted) || (canvas && !aligned4(canvas)))
    return BD_ERR_ALIGN;
  void* workspace = nullptr;
  const hipError_t got = bd::static_sample_scratch(bd::sample_workspace_bytes(P, V), &workspace);
  if (got == hipErrorInvalidValue) return BD_ERR_WORKSPACE;
  if (got != hipSuccess) return BD_ERR_HIP;
  hipError_t err = bd::launch_sample_entropy(logits, P, V, temperature, seed, step, frozen,
                                             tokens_out, entropy_out, nullptr, workspace, stream);
  if (err == hipSuccess)
    err = bd::launch_accept(entropy_out, tokens_out, P, entropy_bound, frozen, canvas, accept_out,
                            num_accepted, stream);
  return to_status(err);
}

static bool threshold_ok(float threshold) { return threshold >= 0.f && threshold <= 1.f; }

int diffusion_sample_confidence(const float* logits, int P, int V, float temperature,
                                uint64_t seed, uint32_t step, const uint8_t* frozen,
                                int32_t* tokens_out, float* entropy_out, float* confidence_out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_sample_shape(P, V, temperature);
  if (st != BD_OK) return st;
  if (!logits || !tokens_out || !confidence_out) return BD_ERR_NULL;
  if (!aligned16(logits) || !aligned4(tokens_out) || !aligned4(confidence_out) ||
      (entropy_out && !aligned4(entropy_out)))
    return BD_ERR_ALIGN;
  st = check_workspace(workspace, workspace_bytes, bd::sample_workspace_bytes(P, V));
  if (st != BD_OK) return st;
  return to_status(bd::launch_sample_entropy(logits, P, V, temperature, seed, step, frozen,
                                             tokens_out, entropy_out, confidence_out, workspace,
                                             stream));
}

int diffusion_accept_confidence(const float* confidence, const int32_t* tokens, int P,
                                float threshold, uint8_t* frozen, int32_t* canvas,
                                uint8_t* accept_out, int32_t* num_accepted, hipStream_t stream) {
  if (P < 1 || P > BD_MAX_POSITIONS || !threshold_ok(threshold)) return BD_ERR_SHAPE;
  if (!confidence || !tokens || !accept_out || !num_accepted) return BD_ERR_NULL;
  if (!aligned4(confidence) || !aligned4(tokens) || !aligned4(num_accepted) ||
      (canvas && !aligned4(canvas)))
    return BD_ERR_ALIGN;
  return to_status(bd::launch_accept_confidence(confidence, tokens, P, threshold, frozen, canvas,
                                                accept_out, num_accepted, stream));
}

static int step_confidence_call(const float* logits, int P, int V, float temperature,
                                float threshold, uint64_t seed, uint32_t step, uint8_t* frozen,
                                int32_t* canvas, int32_t* tokens_out, float* confidence_out,
                                uint8_t* accept_out, int32_t* num_accepted, void* workspace,
                                size_t workspace_bytes, const int32_t* gate,
                                hipStream_t stream) {
  int st = check_sample_shape(P, V, temperature);
  if (st != BD_OK) return st;
  if (!threshold_ok(threshold)) return BD_ERR_SHAPE;
  if (!logits || !tokens_out || !confidence_out || !accept_out || !num_accepted)
    return BD_ERR_NULL;
  if (!aligned16(logits) || !aligned4(tokens_out) || !aligned4(confidence_out) ||
      !aligned4(num_accepted) || (canvas && !aligned4(canvas)))
    return BD_ERR_ALIGN;
  st = check_workspace(workspace, workspace_bytes, bd::sample_workspace_bytes(P, V));
  if (st != BD_OK) return st;
  hipStream_t s = stream;
  hipError_t err = bd::launch_sample_entropy(logits, P, V, temperature, seed, step, frozen,
                                             tokens_out, nullptr, confidence_out, workspace, s,
                                             gate);
  if (err == hipSuccess)
    err = bd::launch_accept_confidence(confidence_out, tokens_out, P, threshold, frozen, canvas,
                                       accept_out, num_accepted, s, gate);
  return to_status(err);
}

int diffusion_sample_step_confidence(const float* logits, int P, int V, float temperature,
                                     float threshold, uint64_t seed, uint32_t step,
                                     uint8_t* frozen, int32_t* canvas, int32_t* tokens_out,
                                     float* confidence_out, uint8_t* accept_out,
                                     int32_t* num_accepted, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  return step_confidence_call(logits, P, V, temperature, threshold, seed, step, frozen, canvas,
                              tokens_out, confidence_out, accept_out, num_accepted, workspace,
                              workspace_bytes, nullptr, stream);
}

int diffusion_sample_step_confidence_gated(const float* logits, int P, int V, float temperature,
                                           float threshold, uint64_t seed, uint32_t step,
                                           uint8_t* frozen, int32_t* canvas, int32_t* tokens_out,
                                           float* confidence_out, uint8_t* accept_out,
                                           int32_t* num_accepted, void* workspace,
                                           size_t workspace_bytes, const int32_t* loop_state,
                                           hipStream_t stream) {
  if (!loop_state) return BD_ERR_NULL;
  if (!aligned4(loop_state)) return BD_ERR_ALIGN;
  return step_confidence_call(logits, P, V, temperature, threshold, seed, step, frozen, canvas,
                              tokens_out, confidence_out, accept_out, num_accepted, workspace,
                              workspace_bytes, loop_state, stream);
}

int bd_canvas_length(int max_canvas, int min_canvas, int remaining, int full_canvas) {
  if (max_canvas < 1 || min_canvas < 1 || remaining < 0) return 0;
  if (full_canvas) return max_canvas;
  const int want = remaining > min_canvas ? remaining : min_canvas;
  return want < max_canvas ? want : max_canvas;
}

int diffusion_canvas_init(int32_t* canvas, int32_t* prev_canvas, uint8_t* frozen,
                          int32_t* loop_state, int P, int vocab, uint64_t seed, uint32_t block,
                          hipStream_t stream) {
  if (P < 1 || P > BD_MAX_POSITIONS || vocab < 1 || vocab > BD_MAX_VOCAB) return BD_ERR_SHAPE;
  if (!canvas || !prev_canvas || !frozen || !loop_state) return BD_ERR_NULL;
  if (!aligned4(canvas) || !aligned4(prev_canvas) || !aligned4(loop_state)) return BD_ERR_ALIGN;
  return to_status(bd::launch_canvas_init(canvas, prev_canvas, frozen, loop_state, P, vocab, seed,
                                          block, stream));
}

int diffusion_loop_update(const int32_t* tokens, int32_t* canvas, int32_t* prev_canvas,
                          const uint8_t* frozen, int32_t* loop_state, int P,
                          int stability_threshold, int max_steps, int write_drafts,
                          hipStream_t stream) {
  if (P < 1 || P > BD_MAX_POSITIONS || stability_threshold < 1 || max_steps < 1)
    return BD_ERR_SHAPE;
  if (!canvas || !prev_canvas || !frozen || !loop_state || (write_drafts && !tokens))
    return BD_ERR_NULL;
  if ((tokens && !aligned4(tokens)) || !aligned4(canvas) || !aligned4(prev_canvas) ||
      !aligned4(loop_state))
    return BD_ERR_ALIGN;
  return to_status(bd::launch_loop_update(tokens, canvas, prev_canvas, frozen, loop_state, P,
                                          stability_threshold, max_steps, write_drafts ? 1 : 0,
                                          stream));
}

int bd_hbm_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  if (!src || !dst) return BD_ERR_NULL;
  if (bytes % 16 != 0) return BD_ERR_SHAPE;
  if (!aligned16(src) || !aligned16(dst)) return BD_ERR_ALIGN;
  return to_status(bd::launch_copy(src, dst, bytes, stream));
}

int bd_hbm_read(const void* src, size_t bytes, uint32_t* checksum, hipStream_t stream) {
  if (!checksum || (!src && bytes)) return BD_ERR_NULL;
  if (bytes % 16 != 0) return BD_ERR_SHAPE;
  if (!aligned16(src) || !aligned16(checksum)) return BD_ERR_ALIGN;
  return to_status(bd::launch_read(src, bytes, checksum, stream));
}

}  // extern "C"
