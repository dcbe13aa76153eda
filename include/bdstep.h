/*
 * bdstep.h -- C ABI of the block-diffusion denoising-step hot path on MI355X (gfx950).
 *
 * Two parts, as on the pages this library implements:
 *
 *  1. The mixture-of-experts FFN of one layer over a canvas of T tokens: top-k routing
 *     over E experts, the W4A16 expert GEMMs (asymmetric uint4 weights with an fp16
 *     scale and fp16 zero-point per 64-element group along the contraction dim,
 *     dequantised inline), the gated GELU folded into the gate/up epilogue, and a
 *     fixed-order weighted combine.  Source: axe-diffusion-ksl-xe model card,
 *     sections "what the model is", "the kernels we built" and "requirements".
 *
 *  2. The per-step sampler: per-position entropy and a gumbel-max (or argmax) token in
 *     one streaming pass over fp32 logits, then the entropy-bound acceptance rule
 *     (sort by ascending entropy, accept while (cumsum - cummax) <= bound, at least
 *     one).  Sources: axe-diffusion-ksl-xe model card, "the kernels we built";
 *     DiffusionGemma block-diffusion page, "Samplers".
 *
 * Conventions shared by every entry point
 *  - Every pointer argument except `workspace` sizes and host structs is a DEVICE
 *    pointer into memory the caller owns.  The library allocates nothing, frees
 *    nothing and keeps no pointer after the call's work completes on the stream.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  All work is
 *    enqueued on it asynchronously; no call synchronises the host.
 *  - fp16 values travel as uint16_t bit patterns.  Arrays are dense and row-major.
 *    The arrays read or written with vector accesses -- logits, x, expert_out, y, the
 *    packed weights with their scales and zero-points, and workspaces -- must be
 *    16-byte aligned (BD_ERR_ALIGN otherwise); every other array needs only the
 *    alignment of its element type.
 *  - Every argument is validated on the host BEFORE anything is enqueued; on any
 *    error the call returns a nonzero bd_status and enqueues nothing.  A launch
 *    failure returns BD_ERR_HIP.  Device faults surface at the caller's next sync.
 *  - Calls are reentrant and the library holds no mutable global state.  Calls that
 *    share a workspace must be ordered on one stream.
 */
#ifndef BDSTEP_H
#define BDSTEP_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BD_ABI_VERSION 13
/* Entries per chunk of the two-level gumbel-max draw (see diffusion_sample_entropy). */
#define BD_SAMPLE_CHUNK 1024
/* Limits checked on the host. */
#define BD_MAX_EXPERTS 256
#define BD_MAX_TOPK 16
#define BD_MAX_TOKENS 65536
#define BD_MAX_POSITIONS 1024
#define BD_MAX_VOCAB (1 << 24)
#define BD_MAX_FEATURES 4096
/* Routed tokens per work item of the grouped GEMMs (see the routing state below). */
#define BD_MOE_ITEM_TOKENS 32

typedef enum {
  BD_OK = 0,
  BD_ERR_NULL = 1,        /* a required pointer is NULL                         */
  BD_ERR_SHAPE = 2,       /* a size is out of range or inconsistent             */
  BD_ERR_ALIGN = 3,       /* a pointer lacks the alignment the ABI requires     */
  BD_ERR_WORKSPACE = 4,   /* workspace missing or smaller than the queried size */
  BD_ERR_UNSUPPORTED = 5, /* valid in principle, not implemented (e.g. g != 64) */
  BD_ERR_HIP = 6          /* a HIP launch or runtime call failed                */
} bd_status;

/*
 * Packed W4A16 expert weights of one layer (all device pointers).
 * Source: axe-diffusion-ksl-xe model card, "the kernels we built" and "requirements":
 * asymmetric uint4, fp16 scale and zero-point per group, two nibbles per byte,
 * groups along the contraction dimension.
 *
 *   gate_up_q      uint8 [E][2*d_ff][d_model/2]   rows 0..d_ff-1 = gate, d_ff..2*d_ff-1 = up
 *   gate_up_scale  fp16  [E][2*d_ff][d_model/g]      g  = group_size
 *   gate_up_zero   fp16  [E][2*d_ff][d_model/g]
 *   down_q         uint8 [E][d_model][d_ff/2]
 *   down_scale     fp16  [E][d_model][d_ff/gd]      gd = down_group_size (0: gd = g)
 *   down_zero      fp16  [E][d_model][d_ff/gd]
 *
 * Byte i of a packed row holds element 2i in its low nibble and element 2i+1 in its
 * high nibble.  The dequantised weight is w[n][k] = (q[n][k] - zero[n][k/g]) *
 * scale[n][k/g].  Zero-points are the uint4 code of the zero (an integer 0..15 held
 * in fp16); the GEMM subtracts them exactly in fp16, a non-integer zero-point is
 * rounded to the nearest integer first.
 * Supported: d_model % 128 == 0, d_ff % 64 == 0, d_model and d_ff <= 4096; g and gd each 64
 * or 128 and dividing that matrix's contraction dim (d_model for gate/up, d_ff for down).
 * A group of 128 is used through the packed stream only (moe_w4a16_prepare keeps one scale
 * and zero-point per 128-group in the gate/up stream and spreads them over the two 64-group
 * slots of the down stream); a GEMM over raw arrays with a group of 128 returns
 * BD_ERR_UNSUPPORTED.  The model card's checkpoint format ("requirements") is g = 128,
 * gd = 64.
 *
 * format BD_FORMAT_AFFINE: the *_zero arrays hold a free fp16 bias b per group and the weight
 * is w = q * scale + b (the MLX-style affine 4-bit form, named on the TensorFold XPU page).
 * The GEMMs then form fp16(q * scale + b) for the MFMA (one rounding per weight) and need the
 * packed stream; over raw arrays they return BD_ERR_UNSUPPORTED.
 *
 * gate_up_packed / down_packed (optional, NULL when absent): the matrix repacked once by
 * moe_w4a16_prepare into the stream the 256-row GEMM tiles consume.  A GEMM whose packed
 * stream is present reads only that stream (its q, scale and zero pointers may then be NULL);
 * without it the GEMM runs on 128-row tiles over q, scale and zero.  Both contract exact fp16
 * (q - z) per 64-group and scale each group's sum in fp32; they differ only in the order of
 * the fp32 sums.
 */
#define BD_FORMAT_ASYMMETRIC 0  /* w = (q - zero) * scale, zero an integer 0..15 in fp16 */
#define BD_FORMAT_AFFINE 1      /* w = q * scale + bias, bias a free fp16 in the zero slot */

typedef struct bd_moe_weights {
  int32_t num_experts; /* E, 1..256          */
  int32_t top_k;       /* k, 1..min(E, 16)   */
  int32_t d_model;     /* d                  */
  int32_t d_ff;        /* f                  */
  int32_t group_size;  /* g of gate/up: 64 or 128 (128 via the packed stream only) */
  const uint8_t* gate_up_q;
  const uint16_t* gate_up_scale;
  const uint16_t* gate_up_zero;
  const uint8_t* down_q;
  const uint16_t* down_scale;
  const uint16_t* down_zero;
  const uint8_t* gate_up_packed;  /* optional, bd_moe_packed_size(w, 0) bytes, 16-byte aligned */
  const uint8_t* down_packed;     /* optional, bd_moe_packed_size(w, 1) bytes, 16-byte aligned */
  int32_t down_group_size;        /* gd of down: 0 (= g), 64 or 128 (128 via the packed stream) */
  int32_t format;                 /* BD_FORMAT_ASYMMETRIC or BD_FORMAT_AFFINE (see above) */
} bd_moe_weights;

/* Library ABI version (BD_ABI_VERSION of the build). */
int bd_abi_version(void);

/* Static, never-NULL text for a bd_status value. */
const char* bd_status_string(int status);

/* ------------------------------------------------------------------ MoE FFN */

/*
 * Bytes of the packed stream of the gate/up matrix (matrix 0) or the down matrix (matrix 1);
 * 0 if the shape is invalid.
 */
size_t bd_moe_packed_size(const bd_moe_weights* w, int matrix);

/*
 * One-time repacking of a layer's weights for the 256-row GEMM tiles, into the caller's
 * buffers (sizes from bd_moe_packed_size; 16-byte aligned).  Reads w's q, scale and zero
 * arrays of both matrices (all required here).
 *
 * A tile covers 256 tile rows: for gate/up, tile row r < 128 is the gate row of column
 * 128t + r and tile row r >= 128 the up row of column 128t + r - 128; for down, tile row r
 * is row 256t + r.  Rows past the matrix and the group past an odd number of groups are
 * written as zeros.  The stream is [E][tiles][stages][18432 bytes]; a stage covers 128
 * contraction elements (groups 2s and 2s+1) and holds
 *   bytes 0..16383: for w = 0..7, set S = 0, 1, lane l = 0..63 (n = l % 16, b = l / 16), at
 *     ((2w + S) * 64 + l) * 16: packed bytes 8b..8b+7 of group 2s, then of group 2s+1, of
 *     tile row R(w, S, n), where R = 128S + 16w + n for gate/up and 32w + 16S + n for down;
 *   bytes 16384..18431: for w = 0..7, n = 0..15, at 16384 + (16w + n) * 16: the fp16 values
 *     scale[2s], scale[2s+1], zero[2s], zero[2s+1] of tile row R(w, 0, n), then the same four
 *     of tile row R(w, 1, n).
 * The gate/up stream of a matrix grouped at 128 (g = 128) has stages of 17408 bytes instead:
 * the same 16384 bytes of nibbles, then for w = 0..7, n = 0..15, at 16384 + (16w + n) * 8,
 * scale and zero of the stage's 128-group (group s) of tile row R(w, 0, n), then of tile row
 * R(w, 1, n).  bd_moe_packed_size accounts for it.
 * Store the results in gate_up_packed and down_packed of the weights struct for the GEMM
 * entry points to use them.
 */
int moe_w4a16_prepare(const bd_moe_weights* w, uint8_t* gate_up_packed, uint8_t* down_packed,
                      hipStream_t stream);

/*
 * Device workspace bytes needed by the MoE entry points for T tokens.  The same
 * workspace carries the routing state from moe_route_topk to moe_w4a16_gate_up and
 * moe_w4a16_down (a copy of the top-k ids, the expert buckets, the work list, the
 * permuted activations for raw weights and the fp16 GeGLU activations h [T*k][d_ff]).
 * Its contents need no initialisation.  Returns 0 if the shape is invalid.
 *
 * Routing state (written by moe_route_topk, read by the GEMMs; with A = T*k, up(n) = n
 * rounded up to a multiple of 256 and M = A / BD_MOE_ITEM_TOKENS + min(E, A)):
 *   byte 0:                    int32 offsets[E + 1]; offsets[e] = assignments routed to
 *                              experts below e (offsets[E] = A)
 *   byte up(4(E + 1)):         int32 items[1 + 3M]; items[0] = number of work items, then per
 *                              item (expert, first bucket position, tokens): every touched
 *                              expert in ascending order, its bucket cut into consecutive
 *                              items of BD_MOE_ITEM_TOKENS positions (the last may be shorter)
 *   byte up(4(E + 1)) + up(4(1 + 3M)):  int32 perm[A]; bucket position -> t*k + j, each
 *                              expert's bucket in ascending t (a stable counting sort)
 * The GEMMs clamp every index they read from the workspace into the ranges of the current
 * call, so a workspace routed for another shape gives wrong outputs but no access outside the
 * caller's buffers.
 */
size_t bd_moe_workspace_size(int T, const bd_moe_weights* w);

/* The same value under the name the hot-path contract gives it (moe_w4a16_ffn's workspace). */
size_t bd_moe_w4a16_ffn_workspace_size(int T, const bd_moe_weights* w);

/*
 * Routing: per token, the top_k experts by descending router logit (the lower expert
 * id first on equal logits) and their weights = softmax over the k selected logits.
 * A second launch (one block) writes the stable bucketing of the T*k assignments by
 * expert (ordered by token, then slot) and the work list of touched experts to the
 * workspace, for moe_w4a16_gate_up and moe_w4a16_down.
 * Source: axe-diffusion-ksl-xe model card, "what the model is" (128 experts, top-8)
 * and "the kernels we built" (one launch over all experts, not a per-expert loop).
 *
 *   router_logits  fp32  [T][E]   finite values
 *   topk_ids       int32 [T][k]   out
 *   topk_weights   fp32  [T][k]   out
 *   workspace      device, >= bd_moe_workspace_size(T, w) bytes (routing state written)
 */
int moe_route_topk(const bd_moe_weights* w, int T, const float* router_logits,
                   int32_t* topk_ids, float* topk_weights,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Gate/up grouped W4A16 GEMM with the GeGLU epilogue, over every touched expert in
 * one launch: for each assignment (t, j) routed to expert e,
 *   h = gelu_tanh(W_gate[e] x_t) * (W_up[e] x_t),
 * gelu_tanh(a) = a/2 (1 + tanh(sqrt(2/pi) (a + 0.044715 a^3))).  Packed nibbles are
 * streamed once per expert tile, dequantised in registers, contracted on MFMA with
 * fp32 accumulation per 64-group, scaled per group; h is kept in the workspace as fp16.
 * The expert buckets and the work list come from the routing in the workspace.  With
 * packed weights x is reordered in registers on its way to LDS; with raw weights a
 * small launch first writes a reordered copy of x into the workspace.
 * Source: axe-diffusion-ksl-xe model card, "the kernels we built" (inline dequant of
 * packed nibbles, activation folded into the first GEMM's epilogue).
 * Requires a preceding moe_route_topk on the same workspace and stream.
 *
 *   x   fp16 [T][d_model]
 */
int moe_w4a16_gate_up(const bd_moe_weights* w, int T, const uint16_t* x,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Down grouped W4A16 GEMM: o[t][j] = W_down[e] h_(t,j) for every assignment, written
 * in slot order with exactly one writer per row (no atomics).
 * Requires a preceding moe_w4a16_gate_up on the same workspace and stream.
 *
 *   expert_out  fp32 [T][k][d_model]   out
 */
int moe_w4a16_down(const bd_moe_weights* w, int T, float* expert_out,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* moe_route_topk, moe_w4a16_gate_up and moe_w4a16_down in one call. */
int moe_w4a16_ffn(const bd_moe_weights* w, int T, const uint16_t* x,
                  const float* router_logits, int32_t* topk_ids, float* topk_weights,
                  float* expert_out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The same, gated by a denoising loop's driver state (see diffusion_loop_update): when
 * loop_state[2] (done) is nonzero as the launches run, every kernel returns at once and no
 * output or workspace byte is written.  So a fixed sequence of steps captured in one graph
 * does no work after its block has ended.  loop_state: int32 [4], device, required.
 * Source: DiffusionGemma block-diffusion page, "How it works" (the block ends early).
 */
int moe_w4a16_ffn_gated(const bd_moe_weights* w, int T, const uint16_t* x,
                        const float* router_logits, int32_t* topk_ids, float* topk_weights,
                        float* expert_out, void* workspace, size_t workspace_bytes,
                        const int32_t* loop_state, hipStream_t stream);

/*
 * Fixed-order weighted combine: y[t] = fp16( sum_{j=0}^{k-1} w[t][j] * o[t][j] ), the
 * sum taken in fp32 as acc = fma(w[t][j], o[t][j], acc) for j = 0, 1, ..., k-1 from
 * acc = 0, then rounded once to fp16 (round to nearest even).  No atomics: results are
 * bit-identical from run to run.
 * Source: axe-diffusion-ksl-xe model card, "the kernels we built" (fixed-order
 * reduction instead of index_add_, since a 1-ulp change can flip an acceptance).
 *
 *   expert_out    fp32 [T][k][d]
 *   topk_weights  fp32 [T][k]
 *   y             fp16 [T][d]   out;  d % 4 == 0
 */
int moe_combine_fixed_order(const float* expert_out, const float* topk_weights,
                            int T, int k, int d, uint16_t* y, hipStream_t stream);

/* moe_combine_fixed_order gated like moe_w4a16_ffn_gated (nothing written once done). */
int moe_combine_fixed_order_gated(const float* expert_out, const float* topk_weights, int T,
                                  int k, int d, uint16_t* y, const int32_t* loop_state,
                                  hipStream_t stream);

/* ------------------------------------------------------------------ layer neighbours */

/*
 * Fused RMS norm of fp16 rows, one launch:
 *   y[t][i] = fp16_rne( h[t][i] / sqrt(mean_i(h[t][i]^2) + eps) * weight[i] )
 * evaluated in fp32 (squares exact, fixed summation order).  The FFN input of a layer.
 * Source: axe-diffusion-ksl-xe model card, "the kernels we built" (RMS norm as one launch
 * instead of about six elementwise ones).  No bias, no mean subtraction, weight as stored.
 *
 *   h       fp16 [T][d], 16-byte aligned        weight  fp16 [d], 16-byte aligned
 *   y       fp16 [T][d] out, 16-byte aligned (may not overlap h)
 *   T in 1..BD_MAX_TOKENS; d in 8..BD_MAX_FEATURES with d % 8 == 0; eps finite, >= 0.
 */
int moe_rmsnorm(const uint16_t* h, const uint16_t* weight, int T, int d, float eps, uint16_t* y,
                hipStream_t stream);

/*
 * Router projection: logits[t][e] = sum_i x[t][i] * w_router[e][i], fp16 operands (exact
 * products), fp32 accumulation (MFMA), fp32 out; the input of moe_route_topk.
 * Source: axe-diffusion-ksl-xe model card, "what the model is" (every token scores the 128
 * experts and keeps the top 8).
 *
 *   x         fp16 [T][d], 16-byte aligned (e.g. the output of moe_rmsnorm)
 *   w_router  fp16 [E][d], expert-major, 16-byte aligned
 *   logits    fp32 [T][E] out
 *   T in 1..BD_MAX_TOKENS; E in 1..BD_MAX_EXPERTS; d in 128..BD_MAX_FEATURES, d % 128 == 0.
 */
int moe_router_logits(const uint16_t* x, const uint16_t* w_router, int T, int d, int E,
                      float* logits, hipStream_t stream);

/*
 * moe_rmsnorm and moe_router_logits gated like moe_w4a16_ffn_gated: the kernel reads
 * loop_state[2] (done) when it starts and writes nothing once it is set, so that a captured
 * graph of a whole block can chain the layers (norm -> router -> FFN -> combine -> next
 * layer) and do no work after the block has ended.  loop_state: int32 [4], device, 4-byte
 * aligned, the state diffusion_loop_update keeps (NULL -> BD_ERR_NULL).  Otherwise the
 * arguments, checks and results are those of the plain entry points.
 */
int moe_rmsnorm_gated(const uint16_t* h, const uint16_t* weight, int T, int d, float eps,
                      uint16_t* y, const int32_t* loop_state, hipStream_t stream);
int moe_router_logits_gated(const uint16_t* x, const uint16_t* w_router, int T, int d, int E,
                            float* logits, const int32_t* loop_state, hipStream_t stream);

/*
 * The combine of layer l and the RMS norm that starts layer l + 1, one launch: y is exactly
 * moe_combine_fixed_order(expert_out, topk_weights) and xn exactly moe_rmsnorm(y, weight,
 * eps), bit for bit, but y is not read back from memory for the norm (each row's sum of
 * squares is taken in the norm's own order from the row the same block has just combined).
 * Sources: axe-diffusion-ksl-xe model card, "the kernels we built" (the fixed-order combine;
 * the RMS norm as one launch) and "what the model is" (a layer's output is the next layer's
 * input).
 *
 *   expert_out, topk_weights, T, k: as moe_combine_fixed_order (k in 1..BD_MAX_TOPK)
 *   weight  fp16 [d], the next layer's norm weight, 16-byte aligned
 *   y       fp16 [T][d] out, the layer output, 16-byte aligned
 *   xn      fp16 [T][d] out, the next layer's FFN and router input, 16-byte aligned
 *   d in 8..BD_MAX_FEATURES with d % 8 == 0; eps finite, >= 0.  No output may overlap an
 *   input or the other output.
 */
int moe_combine_rmsnorm(const float* expert_out, const float* topk_weights, int T, int k, int d,
                        const uint16_t* weight, float eps, uint16_t* y, uint16_t* xn,
                        hipStream_t stream);

/* moe_combine_rmsnorm gated like moe_rmsnorm_gated (nothing written once the block is done). */
int moe_combine_rmsnorm_gated(const float* expert_out, const float* topk_weights, int T, int k,
                              int d, const uint16_t* weight, float eps, uint16_t* y, uint16_t* xn,
                              const int32_t* loop_state, hipStream_t stream);

/* ------------------------------------------------------------------ sampler */

/* Device workspace bytes needed by diffusion_sample_entropy for P rows of V logits. */
size_t bd_sample_workspace_size(int P, int V);

/*
 * One streaming pass over fp32 logits [P][V] (row-major): for every position p that
 * is not frozen,
 *   entropy_out[p] = H_p = -sum_v softmax(x_p)_v * ln softmax(x_p)_v   (temperature 1)
 *   tokens_out[p]  = argmax_v x_pv (lowest v on ties)                  if temperature == 0
 *                  = a draw from softmax(x_p / temperature)             otherwise.
 * The draw is gumbel-max on two levels: the row is cut into chunks of BD_SAMPLE_CHUNK
 * entries; level 1 takes the chunk c maximising L_c + G_c with L_c = ln sum_{v in c}
 * exp(x_v / temperature); level 2 takes, inside that chunk, the v maximising
 * x_v / temperature + g_v (exact in distribution; identical to flat gumbel-max when
 * V <= BD_SAMPLE_CHUNK).  Noise is Philox4x32-10 (Salmon et al., SC'11) keyed by
 * (seed & 0xffffffff, seed >> 32): g_v from counter (v >> 2, p, step, 0) word v & 3,
 * G_c from counter (c, p, step, 1) word 0; u = ((r >> 8) + 0.5) * 2^-24 and
 * g = -ln(-ln u), both evaluated in fp64, as is the level-2 score.
 * Sources: axe-diffusion-ksl-xe model card, "the kernels we built" (entropy once per
 * step in a single streaming pass; one gumbel-max kernel instead of softmax +
 * multinomial); configuration text "Philox, seed per step".
 *
 *   frozen       uint8 [P] or NULL (none frozen).  Frozen rows are not read; they get
 *                tokens_out = -1 and entropy_out = +inf.
 *   A row containing NaN or +inf, or only -inf, gets entropy NaN and token -1.
 *   temperature  0, or positive with 1/temperature finite in fp32 (>= about 2.9e-39)
 *   P in 1..BD_MAX_POSITIONS, V in 1..BD_MAX_VOCAB.  V % 4 == 0 takes the vector path;
 *   other V are handled, more slowly.
 */
int diffusion_sample_entropy(const float* logits, int P, int V, float temperature,
                             uint64_t seed, uint32_t step, const uint8_t* frozen,
                             int32_t* tokens_out, float* entropy_out,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Entropy-bound acceptance on one workgroup.  Candidates are the positions that are
 * not frozen and whose entropy is not NaN; they are sorted by (entropy ascending,
 * position ascending) and scanned in that order in fp32: S = S + H_i; c = S - H_i
 * (cumsum - cummax, cummax being H_i in ascending order); position i is accepted
 * while c <= bound, and the scan stops at the first failure.  If candidates exist and
 * none passed, the first one is accepted.  Each accepted p gets accept_out[p] = 1,
 * canvas[p] = tokens[p] and frozen[p] = 1; every other accept_out entry is 0.
 * Source: DiffusionGemma block-diffusion page, "Samplers" (entropy-bound).
 *
 *   entropy       fp32  [P]      (the device's own entropies, e.g. from above)
 *   tokens        int32 [P]
 *   frozen        uint8 [P] in/out, or NULL (none frozen, nothing recorded)
 *   canvas        int32 [P] in/out, or NULL (not updated)
 *   accept_out    uint8 [P] out
 *   num_accepted  int32 [1] out
 *   bound         finite
 */
int diffusion_accept_entropy_bound(const float* entropy, const int32_t* tokens, int P,
                                   float bound, uint8_t* frozen, int32_t* canvas,
                                   uint8_t* accept_out, int32_t* num_accepted, hipStream_t stream);

/* diffusion_sample_entropy then diffusion_accept_entropy_bound on the same stream. */
int diffusion_sample_step(const float* logits, int P, int V, float temperature,
                          float entropy_bound, uint64_t seed, uint32_t step,
                          uint8_t* frozen, int32_t* canvas, int32_t* tokens_out,
                          float* entropy_out, uint8_t* accept_out, int32_t* num_accepted,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* diffusion_sample_step gated like moe_w4a16_ffn_gated: once loop_state[2] (done) is set,
 * nothing is read or written (tokens, entropies, mask, count, canvas and frozen set stay). */
int diffusion_sample_step_gated(const float* logits, int P, int V, float temperature,
                                float entropy_bound, uint64_t seed, uint32_t step,
                                uint8_t* frozen, int32_t* canvas, int32_t* tokens_out,
                                float* entropy_out, uint8_t* accept_out, int32_t* num_accepted,
                                void* workspace, size_t workspace_bytes,
                                const int32_t* loop_state, hipStream_t stream);

/*
 * diffusion_sample_step without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments (less the workspace), same results bit for bit.  The streaming pass's split
 * states live in a static device array of the library (512 KiB per GPU, held until the
 * process ends; every valid P, V fits, else BD_ERR_WORKSPACE); the call allocates nothing.
 * All calls on one GPU share that array: calls that overlap on a GPU (other streams, other
 * threads) race and must not be issued; calls ordered on one stream are safe.  The first call
 * on a device looks the array's address up (hipGetSymbolAddress, no allocation); make it
 * outside graph capture if the capture forbids that.
 */
int diffusion_sample_step_noalloc(const float* logits, int P, int V, float temperature,
                                  float entropy_bound, uint64_t seed, uint32_t step,
                                  uint8_t* frozen, int32_t* canvas, int32_t* tokens_out,
                                  float* entropy_out, uint8_t* accept_out, int32_t* num_accepted,
                                  hipStream_t stream);

/*
 * Confidence-threshold variant of the sampler.  The same single streaming pass as
 * diffusion_sample_entropy (same tokens, same entropies), which also writes the top-1
 * probability of every position that is not frozen:
 *   confidence_out[p] = max_v softmax(x_p)_v = 1 / sum_v exp(x_pv - max_v x_pv)
 * (temperature 1, whatever the sampling temperature), evaluated in fp32 from the pass's
 * running sums.  Frozen rows get -1 (and token -1, entropy +inf); invalid rows (NaN, +inf,
 * or only -inf) get NaN.  entropy_out may be NULL.
 * Source: DiffusionGemma block-diffusion page, "Samplers" (confidence-threshold: the top-1
 * token probability of each unrevealed position).
 */
int diffusion_sample_confidence(const float* logits, int P, int V, float temperature,
                                uint64_t seed, uint32_t step, const uint8_t* frozen,
                                int32_t* tokens_out, float* entropy_out, float* confidence_out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Confidence-threshold acceptance on one workgroup.  Candidates are the positions that
 * are not frozen and whose confidence is neither NaN nor negative.  Every candidate with
 * confidence > threshold (strict, fp32) is accepted; if candidates exist and none
 * qualifies, the candidate with the largest confidence (lowest position on ties) is
 * accepted alone, so each call makes progress.  Each accepted p gets accept_out[p] = 1,
 * canvas[p] = tokens[p] and frozen[p] = 1; every other accept_out entry is 0.
 * Source: DiffusionGemma block-diffusion page, "Samplers" (confidence-threshold) and its
 * options table (threshold default 0.9, validated to [0, 1]).
 *
 *   confidence    fp32  [P]      (the device's own confidences, e.g. from above)
 *   tokens        int32 [P]
 *   frozen        uint8 [P] in/out, or NULL (none frozen, nothing recorded)
 *   canvas        int32 [P] in/out, or NULL (not updated)
 *   accept_out    uint8 [P] out
 *   num_accepted  int32 [1] out
 *   threshold     in [0, 1], else BD_ERR_SHAPE
 */
int diffusion_accept_confidence(const float* confidence, const int32_t* tokens, int P,
                                float threshold, uint8_t* frozen, int32_t* canvas,
                                uint8_t* accept_out, int32_t* num_accepted, hipStream_t stream);

/* diffusion_sample_confidence (no entropy output) then diffusion_accept_confidence on the
 * same stream. */
int diffusion_sample_step_confidence(const float* logits, int P, int V, float temperature,
                                     float threshold, uint64_t seed, uint32_t step,
                                     uint8_t* frozen, int32_t* canvas, int32_t* tokens_out,
                                     float* confidence_out, uint8_t* accept_out,
                                     int32_t* num_accepted, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* diffusion_sample_step_confidence gated like diffusion_sample_step_gated. */
int diffusion_sample_step_confidence_gated(const float* logits, int P, int V, float temperature,
                                           float threshold, uint64_t seed, uint32_t step,
                                           uint8_t* frozen, int32_t* canvas, int32_t* tokens_out,
                                           float* confidence_out, uint8_t* accept_out,
                                           int32_t* num_accepted, void* workspace,
                                           size_t workspace_bytes, const int32_t* loop_state,
                                           hipStream_t stream);

/* ------------------------------------------------------------------ denoising-loop driver */

/*
 * Canvas length of the next block (host only, no device work):
 *   full_canvas ? max_canvas : min(max_canvas, max(remaining, min_canvas)).
 * Returns 0 if max_canvas < 1, min_canvas < 1 or remaining < 0.
 * Source: DiffusionGemma block-diffusion page, "How it works" (length rule) and "CLI flags"
 * (minimum 64, maximum the model's canvas length, the full-canvas option).
 */
int bd_canvas_length(int max_canvas, int min_canvas, int remaining, int full_canvas);

/*
 * Start of a block: canvas[p] = prev_canvas[p] = floor(w_p * vocab / 2^32) with w_p word 0 of
 * Philox4x32-10 (key = seed low word, high word) at counter (p, block, 0, 2); frozen[p] = 0;
 * loop_state[0..3] = 0.  loop_state is int32 [4]: steps run, consecutive unchanged steps,
 * done flag, frozen count.
 * Source: DiffusionGemma block-diffusion page, "How it works" (canvas of uniformly random
 * token ids) and "Reproducibility" (the seed fixes the initial canvas).
 *   P in 1..BD_MAX_POSITIONS; vocab in 1..BD_MAX_VOCAB; all pointers device memory.
 */
int diffusion_canvas_init(int32_t* canvas, int32_t* prev_canvas, uint8_t* frozen,
                          int32_t* loop_state, int P, int vocab, uint64_t seed, uint32_t block,
                          hipStream_t stream);

/*
 * The driver's update after one step's sampler call (one workgroup).  Unless loop_state
 * says the block is done (then nothing changes): if write_drafts, every position the step
 * sampled (tokens[p] >= 0) takes its draft, canvas[p] = tokens[p] (frozen positions keep
 * their token, tokens = -1 there); the canvas is compared with prev_canvas, which then
 * takes the canvas; steps += 1; the unchanged count is reset on any change, else
 * incremented; done = unchanged >= stability_threshold, or every position frozen, or
 * steps >= max_steps.
 * Source: DiffusionGemma block-diffusion page, "How it works" (the whole canvas is updated
 * at every step; the early stop once the canvas has not changed for stability_threshold
 * steps; the step budget).
 *   tokens  int32 [P] (may be NULL if write_drafts == 0); canvas, prev_canvas int32 [P];
 *   frozen  uint8 [P] (after the step's acceptance); loop_state int32 [4] in/out.
 *   P in 1..BD_MAX_POSITIONS; stability_threshold >= 1; max_steps >= 1.
 */
int diffusion_loop_update(const int32_t* tokens, int32_t* canvas, int32_t* prev_canvas,
                          const uint8_t* frozen, int32_t* loop_state, int P,
                          int stability_threshold, int max_steps, int write_drafts,
                          hipStream_t stream);

/* ------------------------------------------------------------------ measurement */

/*
 * Plain device-to-device copy of `bytes` bytes (bytes % 16 == 0, both pointers 16-byte
 * aligned) with a streaming kernel: the calibration for HBM traffic counters and the
 * achievable-bandwidth figure beside the 8 TB/s specification.
 */
int bd_hbm_copy(const void* src, void* dst, size_t bytes, hipStream_t stream);

/*
 * Streaming read of `bytes` bytes at src (bytes % 16 == 0; src and checksum 16-byte aligned,
 * both device memory): checksum points to BD_HBM_READ_WORDS uint32 words; word 0 receives
 * the XOR of all 32-bit words of src (0 for bytes == 0) and the others are scratch.  The read
 * cannot be optimised away and can be checked on the host.  The achievable read-only
 * bandwidth beside the copy figure: nontemporal 16-byte loads, the form the weight and logits
 * streams use.  Two launches on `stream` (read, then a one-block fold of the per-block
 * partials); the caller owns both buffers.  src may be NULL when bytes == 0.
 */
#define BD_HBM_READ_WORDS 2049
int bd_hbm_read(const void* src, size_t bytes, uint32_t* checksum, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* BDSTEP_H */
