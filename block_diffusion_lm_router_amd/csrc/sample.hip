// Per-step sampler kernels: streaming entropy + token pass, per-row finish (entropy, top-1
// probability, token), and the two acceptance rules (entropy-bound: selection, then sort and
// scan; confidence-threshold: one block-wide count and max).
//
// Sources: axe-diffusion-ksl-xe model card, "the kernels we built" (entropy once per
// step in one streaming pass over the fp32 logits; gumbel-max instead of softmax +
// multinomial); DiffusionGemma block-diffusion page, "Samplers" (entropy-bound and
// confidence-threshold rules).
//
// Streaming pass.  The logits are read exactly once.  A wave takes one chunk of 1024
// consecutive entries at a time (16 per lane, four coalesced 16-byte loads), finds the
// chunk maximum m_c with DPP, and folds exp(x - m_c) into per-lane running sums kept
// against a wave-uniform running maximum:
//     n  = count of entries equal to the running maximum,
//     s  = sum of exp(x - m) over the other entries,
//     t  = sum of exp(x - m) (x - m).
// With Z = n + s the entropy is H = ln Z - t / Z = log1p((n - 1) + s) - t / Z; keeping
// the maximal entries out of s keeps H accurate when it is near zero.  The temperature-0
// argmax needs only the chunk maxima.  For T > 0 the pass also forms each chunk's log-mass
// L_c = ln sum exp(x / T) and draws the level-1 key L_c + G_c (Philox, fp64): lane b of a wave
// keeps the b-th chunk's L_c, and every 64 chunks (and at the end) the lanes draw their keys
// at once and the wave keeps its best two.  Partial states of the V-splits of a row are merged
// in split order by the finish kernel.  Its level-1 decision is the fp64 one: the chunks whose
// fp32 keys lie too close to the best to be told apart are rescored in fp64.  It then re-reads
// the one winning chunk (1024 entries) for the level-2 draw.

#include <mutex>

#include "bd_device.hpp"
#include "bd_internal.hpp"

namespace bd {

namespace {

constexpr int kChunk = 1024;
#ifndef BD_SAMPLE_THREADS
#define BD_SAMPLE_THREADS 256
#endif
#ifndef BD_SAMPLE_RING
#define BD_SAMPLE_RING 2
#endif
#ifndef BD_SAMPLE_BLOCKS
#define BD_SAMPLE_BLOCKS 1024  // target blocks of the streaming pass (splits per row = this / P)
#endif
constexpr int kStreamThreads = BD_SAMPLE_THREADS;
constexpr int kStreamWaves = kStreamThreads / kWave;
constexpr int kRing = BD_SAMPLE_RING;  // chunks in flight per wave

// Loads chunk c of a row: entry e(j, q) = c*1024 + (j*64 + lane)*4 + q lands in x[4j + q].
// Entries past V read as -inf (they carry no probability mass).
__device__ __forceinline__ void load_chunk(const float* __restrict__ row, int V, int c, bool vec,
                                           float (&x)[16]) {
  const int lane = lane_id();
  const int base = c * kChunk;
  if (vec) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = base + (j * kWave + lane) * 4;
      if (idx < V) {
        // Nontemporal: each logit is used once (plain loads measured 10 % slower here).
        const float4_t v = __builtin_nontemporal_load(reinterpret_cast<const float4_t*>(row + idx));
        x[4 * j + 0] = v[0];
        x[4 * j + 1] = v[1];
        x[4 * j + 2] = v[2];
        x[4 * j + 3] = v[3];
      } else {
        x[4 * j + 0] = x[4 * j + 1] = x[4 * j + 2] = x[4 * j + 3] = -INFINITY;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int idx = base + ((i >> 2) * kWave + lane) * 4 + (i & 3);
      x[i] = idx < V ? row[idx] : -INFINITY;
    }
  }
}

struct LaneState {
  float m;  // wave-uniform running maximum
  float n;  // wave-uniform count of entries equal to m (the whole wave's)
  float s, t;  // per-lane sums
  float best_v;  // temperature-0 argmax (wave-uniform)
  int best_i;
  bool nan;      // NaN seen in a chunk with no finite entry (wave-uniform)
};

// Larger key first, then the lower index: a total order, so every reduction by it gives the
// same result whatever its order.
__device__ __forceinline__ bool better_key(double ka, int ia, double kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// Wave-wide best (key, index) by better_key; the result is uniform.
__device__ __forceinline__ void wave_argmax(double& key, int& idx) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const double ok = __shfl_xor(key, off);
    const int oi = __shfl_xor(idx, off);
    if (better_key(ok, oi, key, idx)) {
      key = ok;
      idx = oi;
    }
  }
}

// MODE 0: temperature 0 (argmax); 1: temperature 1; 2: any other temperature.  Returns the
// chunk's log-mass L_c for MODE > 0 (-inf for a chunk without a finite entry).
template <int MODE>
__device__ __forceinline__ float process_chunk(const float (&x)[16], int c, float invT,
                                               LaneState& st) {
  const int lane = lane_id();
  float lm = x[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) lm = fmaxf(lm, x[i]);
  const float mc = wave_max(lm);
  if (mc == -INFINITY) {  // no finite entry: only NaN can hide here
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 16; ++i) bad |= (x[i] != x[i]);
    if (wave_any(bad)) st.nan = true;
    return -INFINITY;
  }
  float sc = 0.f, tc = 0.f, zt = 0.f;
  int at_max = 0;  // wave-wide count of the chunk's entries equal to mc (scalar popcounts)
  const float scaleT = kLog2e * invT;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float d = x[i] - mc;
    const float e = __builtin_amdgcn_exp2f(d * kLog2e);
    const bool off_max = d != 0.f;  // true for NaN as well, which then poisons s
    sc += off_max ? e : 0.f;
    at_max += __popcll(__ballot(!off_max));
    tc = fmaf(e, fmaxf(d, -200.f), tc);
    if (MODE == 2) zt += __builtin_amdgcn_exp2f(d * scaleT);
  }
  const float nc = (float)at_max;
  // The maximal entries count once for the wave: lane 0 carries them in the per-lane sums.
  const float nl = lane == 0 ? st.n : 0.f;
  // Fold the chunk into the running per-lane state (branches are wave-uniform).
  if (mc > st.m) {
    if (st.m == -INFINITY) {
      st.n = nc;
      st.s = sc;
      st.t = tc;
    } else {
      const float delta = st.m - mc;
      const float r = __builtin_amdgcn_exp2f(delta * kLog2e);
      st.t = fmaf(r, fmaf(delta, st.s + nl, st.t), tc);
      st.s = fmaf(r, st.s + nl, sc);
      st.n = nc;
    }
    st.m = mc;
  } else if (mc == st.m) {
    st.n += nc;
    st.s += sc;
    st.t += tc;
  } else {
    const float delta = mc - st.m;
    const float r = __builtin_amdgcn_exp2f(delta * kLog2e);
    const float zc = (lane == 0 ? nc : 0.f) + sc;
    st.t = fmaf(r, fmaf(delta, zc, tc), st.t);
    st.s = fmaf(r, zc, st.s);
  }
  if (MODE == 0) {
    if (mc > st.best_v) {
      const int base = c * kChunk;
      int idx = 0x7fffffff;
#pragma unroll
      for (int i = 15; i >= 0; --i)
        if (x[i] == mc) idx = base + ((i >> 2) * kWave + lane) * 4 + (i & 3);
      st.best_i = wave_min_i32(idx);
      st.best_v = mc;
    }
    return 0.f;
  }
  const float z = MODE == 1 ? nc + wave_sum(sc) : wave_sum(zt);
  return (MODE == 1 ? mc : mc * invT) + __builtin_amdgcn_logf(z) * kLn2;
}

// Best two level-1 (key, chunk) pairs by better_key.  Chunk ids are distinct, so the pair is
// the same whatever order the candidates arrive in.
struct Top2 {
  double k1, k2;
  int c1, c2;
};
__device__ __forceinline__ Top2 top2_empty() {
  return Top2{-INFINITY, -INFINITY, 0x7fffffff, 0x7fffffff};
}
__device__ __forceinline__ void top2_insert(Top2& t, double k, int c) {
  if (better_key(k, c, t.k1, t.c1)) {
    t.k2 = t.k1;
    t.c2 = t.c1;
    t.k1 = k;
    t.c1 = c;
  } else if (better_key(k, c, t.k2, t.c2)) {
    t.k2 = k;
    t.c2 = c;
  }
}

// Merge state b into a (a's maximum is the reference when larger); the level-1 pairs of both
// are merged into a's best two.
__device__ __forceinline__ void merge_state(PartState& a, const PartState& b) {
  a.nan |= b.nan;
  Top2 t{a.best_key, a.second_key, a.best_c, a.second_c};
  top2_insert(t, b.best_key, b.best_c);
  top2_insert(t, b.second_key, b.second_c);
  a.best_key = t.k1;
  a.best_c = t.c1;
  a.second_key = t.k2;
  a.second_c = t.c2;
  if (b.best_v > a.best_v || (b.best_v == a.best_v && b.best_i < a.best_i)) {
    a.best_v = b.best_v;
    a.best_i = b.best_i;
  }
  if (b.m == -INFINITY) return;
  if (a.m == -INFINITY) {
    a.m = b.m;
    a.n = b.n;
    a.s = b.s;
    a.t = b.t;
    return;
  }
  if (b.m > a.m) {
    const float delta = a.m - b.m;
    const float r = __builtin_amdgcn_exp2f(delta * kLog2e);
    a.t = fmaf(r, fmaf(delta, a.n + a.s, a.t), b.t);
    a.s = fmaf(r, a.s + a.n, b.s);
    a.n = b.n;
    a.m = b.m;
  } else if (b.m == a.m) {
    a.n += b.n;
    a.s += b.s;
    a.t += b.t;
  } else {
    const float delta = b.m - a.m;
    const float r = __builtin_amdgcn_exp2f(delta * kLog2e);
    const float zb = b.n + b.s;
    a.t = fmaf(r, fmaf(delta, zb, b.t), a.t);
    a.s = fmaf(r, zb, a.s);
  }
}

// One wave's streaming pass over chunks c_begin + wave, c_begin + wave + WAVES, ... < c_end of
// row p: its entropy sums, its temperature-0 argmax and its best two level-1 keys.
template <int MODE, int WAVES>
__device__ __forceinline__ PartState stream_chunks(const float* __restrict__ row, int V, int p,
                                                   int c_begin, int c_end, float invT,
                                                   uint32_t k0, uint32_t k1, uint32_t step) {
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const bool vec = (V & 3) == 0;

  // Level-1 batch: lane b holds the log-mass of the b-th chunk since the last draw.  A draw
  // gives each held chunk its key L_c + G_c, G_c from counter (c, p, step, 1) word 0, and
  // folds the batch's best two keys into the wave's.
  float bL = -INFINITY;
  int bC = 0;
  int nb = 0;
  Top2 top = top2_empty();
  // Noise of the chunk lane b will hold in the current batch, drawn ahead of the chunk
  // (its counter depends only on the chunk id), so the draw at a batch's end is one add.
  double bG = 0.0;
  int batch0 = c_begin + wave;                  // first chunk of the current batch
  auto noise = [&]() {
    const int c = batch0 + lane * WAVES;
    if (MODE != 0 && c < c_end) {
      const Philox4 r = philox4x32_10((uint32_t)c, (uint32_t)p, step, 1u, k0, k1);
      bG = gumbel_from_word(r.w[0]);
    }
  };
  auto draw = [&]() {
    double key = -INFINITY;
    int kc = 0x7fffffff;
    if (lane < nb && bL != -INFINITY) {
      key = (double)bL + bG;
      kc = bC;
    }
    double ka = key;
    int ca = kc;
    wave_argmax(ka, ca);
    double kb = kc == ca ? -INFINITY : key;
    int cb = kc == ca ? 0x7fffffff : kc;
    wave_argmax(kb, cb);
    top2_insert(top, ka, ca);
    top2_insert(top, kb, cb);
    nb = 0;
    batch0 += kWave * WAVES;
    noise();
  };
  auto fold = [&](float L, int c) {
    if (MODE == 0) return;
    if (lane == nb) {
      bL = L;
      bC = c;
    }
    if (++nb == kWave) draw();
  };

  LaneState st;
  st.m = -INFINITY;
  st.n = st.s = st.t = 0.f;
  st.best_v = -INFINITY;
  st.best_i = 0x7fffffff;
  st.nan = false;

  // Ring of kRing chunks in registers per wave: chunk i of the wave's sequence sits in slot
  // i % kRing and is refilled with chunk i + kRing right after it has been folded in.
  float x[kRing][16];
  const int c0 = c_begin + wave;
#pragma unroll
  for (int r = 0; r < kRing; ++r)
    if (c0 + r * WAVES < c_end) load_chunk(row, V, c0 + r * WAVES, vec, x[r]);
  if (MODE != 0) noise();
  for (int base = c0; base < c_end; base += kRing * WAVES) {
#pragma unroll
    for (int r = 0; r < kRing; ++r) {
      const int c = base + r * WAVES;
      if (c < c_end) {
        fold(process_chunk<MODE>(x[r], c, invT, st), c);
        const int cn = c + kRing * WAVES;
        if (cn < c_end) load_chunk(row, V, cn, vec, x[r]);
      }
    }
  }
  if (MODE != 0 && nb > 0) draw();

  // Lanes share the reference maximum: the wave state is a plain sum.
  PartState ws;
  ws.best_key = top.k1;
  ws.best_c = top.c1;
  ws.second_key = top.k2;
  ws.second_c = top.c2;
  ws.m = st.m;
  ws.n = st.n;
  ws.s = wave_sum(st.s);
  ws.t = wave_sum(st.t);
  ws.best_v = st.best_v;
  ws.best_i = st.best_i;
  ws.nan = st.nan ? 1 : 0;
  return ws;
}

// Block (s, p) streams split s of row p with kStreamWaves waves; wave w writes its state to
// part[p][s][w] (no barrier at the end of the pass: the finish merges the states in order).
template <int MODE>
__global__ __launch_bounds__(kStreamThreads) void sample_stream_kernel(
    const float* __restrict__ logits, int V, int nC, int S, float invT, uint32_t k0,
    uint32_t k1, uint32_t step, const uint8_t* __restrict__ frozen,
    PartState* __restrict__ part, const int32_t* __restrict__ gate) {
  if (gated_off(gate)) return;
  const int p = blockIdx.y;
  const int s = blockIdx.x;
  if (frozen != nullptr && frozen[p]) return;
  const int c_begin = (int)((int64_t)s * nC / S);
  const int c_end = (int)((int64_t)(s + 1) * nC / S);
  const PartState ws = stream_chunks<MODE, kStreamWaves>(logits + (size_t)p * V, V, p, c_begin,
                                                         c_end, invT, k0, k1, step);
  if (lane_id() == 0) part[((size_t)p * S + s) * kStreamWaves + threadIdx.x / kWave] = ws;
}

// ---------------------------------------------------------------- finishing a row

// The identity of merge_state: no entries, no keys.
__device__ __forceinline__ PartState empty_state() {
  PartState e;
  e.m = -INFINITY;
  e.n = e.s = e.t = 0.f;
  e.best_v = -INFINITY;
  e.best_i = 0x7fffffff;
  e.nan = 0;
  e.best_c = e.second_c = 0x7fffffff;
  e.best_key = e.second_key = -INFINITY;
  return e;
}

// The state held by the lane `d` above (every field).
__device__ __forceinline__ PartState shfl_down_state(const PartState& a, int d) {
  PartState b;
  b.m = __shfl_down(a.m, d);
  b.n = __shfl_down(a.n, d);
  b.s = __shfl_down(a.s, d);
  b.t = __shfl_down(a.t, d);
  b.best_v = __shfl_down(a.best_v, d);
  b.best_i = __shfl_down(a.best_i, d);
  b.nan = __shfl_down(a.nan, d);
  b.best_c = __shfl_down(a.best_c, d);
  b.second_c = __shfl_down(a.second_c, d);
  b.best_key = __shfl_down(a.best_key, d);
  b.second_key = __shfl_down(a.second_key, d);
  return b;
}

constexpr int kMaxCand = 64;                   // level-1 candidates rescored one by one

// Block-wide argmax of (key, index) by better_key; uniform result, one barrier.
template <int NW>
__device__ __forceinline__ void block_argmax(double& key, int& idx, double* wkey, int* widx) {
  wave_argmax(key, idx);
  const int wave = threadIdx.x / kWave;
  if (lane_id() == 0) {
    wkey[wave] = key;
    widx[wave] = idx;
  }
  __syncthreads();
  key = wkey[0];
  idx = widx[0];
#pragma unroll
  for (int w = 1; w < NW; ++w)
    if (better_key(wkey[w], widx[w], key, idx)) {
      key = wkey[w];
      idx = widx[w];
    }
}

// Standard Gumbel draw from one Philox word in fp32, for the level-2 pre-selection only.
// u = ((r >> 8) + 0.5) 2^-24; w = -ln u is formed without cancellation: from u itself when
// u < 1/2 (exact in fp32), else as -log1p(-v) with v = 1 - u = (2^24 - 1 - (r >> 8) + 0.5)
// 2^-24 (exact in fp32), by Goldberg's correction log1p(x) = ln(1 + x) x / ((1 + x) - 1)
// (y = 1 + x rounded, y - 1 exact; x itself when y rounds to 1).  g = -ln w.  The logarithms
// are the hardware log2 (v_log_f32, within a few ulp for these normal inputs) times ln 2,
// so |g - g_exact| stays below 1e-5 (|log2| <= 25, w >= 2^-25); the pre-selection margin
// (2e-4 + 2e-6 |max|) is twenty times that, and the published decision is the fp64 one.
__device__ __forceinline__ float gumbel32_from_word(uint32_t r) {
  const uint32_t k = r >> 8;
  float w;
  if (k < (1u << 23)) {
    w = -__builtin_amdgcn_logf(((float)k + 0.5f) * 0x1p-24f) * kLn2;
  } else {
    const float v = ((float)((1u << 24) - 1u - k) + 0.5f) * 0x1p-24f;
    const float y = 1.f - v;
    w = y == 1.f ? v : __builtin_amdgcn_logf(y) * kLn2 * v * __builtin_amdgcn_rcpf(y - 1.f);
  }
  return -__builtin_amdgcn_logf(w) * kLn2;
}

// How far a level-1 key formed from fp32 chunk sums can sit from the fp64 key of the same
// chunk, doubled (both the winner's key and a rival's may be off).  The fp32 log-mass
// L = m / T + ln(sum_c exp2((x - m) log2(e) / T)) carries: per term a relative error below
// 1.2e-7 (exp2) plus 1.5e-7 per unit of the exponent's magnitude (the rounding of x - m,
// 1/T and the product), which the sum weights by exp(x - m) so that it stays below ~1.3e-6
// in relative terms; the fp32 summation over at most 16 per lane and six wave levels below
// 1.3e-6; the log2 within 1 ulp (under 1e-6 absolute for sums of at most 1024 terms), and
// the rounding of m / T and of the final sums, below 2e-7 |L|.  That is below 5e-6 +
// 2e-7 |L|; the margin takes twice 1e-5 + 1e-6 |L| with |L| <= |key| + 20 (the Gumbel draw
// of a 24-bit uniform lies in [-2.9, 17]).
__device__ __forceinline__ double level1_margin(double key) {
  return 2.0 * (1e-5 + 1e-6 * (fabs(key) + 20.0));
}

// The level-1 key of chunk c of row p in fp64, the definition: L_c = m + ln sum exp(x_v / T -
// m) over the chunk's finite entries (m their largest x_v / T), plus G_c.  Run by one wave
// (every lane gets the same value; the sums are taken in a fixed order).
__device__ double chunk_key64(const float* __restrict__ row, int V, int c, double T, int p,
                              uint32_t step, uint32_t k0, uint32_t k1) {
  const int lane = lane_id();
  double y[16];
  double m = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int v = c * kChunk + ((i >> 2) * kWave + lane) * 4 + (i & 3);
    const float xv = v < V ? row[v] : -INFINITY;
    y[i] = (double)xv / T;
    if (y[i] > m) m = y[i];
  }
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) m = fmax(m, __shfl_xor(m, off));
  if (m == -INFINITY) return -INFINITY;
  double z = 0.0;
#pragma unroll
  for (int i = 0; i < 16; ++i) z += y[i] == -INFINITY ? 0.0 : exp(y[i] - m);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) z += __shfl_xor(z, off);
  const Philox4 r = philox4x32_10((uint32_t)c, (uint32_t)p, step, 1u, k0, k1);
  return m + log(z) + gumbel_from_word(r.w[0]);
}

// Finish row p with the block's kFinishThreads threads from the nst partial states in st (LDS, in stream order):
// entropy, top-1 probability and token.  The states are merged in order by one lane.  At
// T > 0 the level-1 winner is the chunk with the best fp32 key unless another chunk's key lies
// within level1_margin of it: then the candidates (each state's best key within the margin)
// are rescored in fp64 by chunk_key64 and the fp64 best wins; if some state's second key is
// also within the margin, that state may hold further candidates, and every chunk of the row
// is rescored.  Level 2 re-reads the winning chunk: its scores x_v / T + g_v are first formed
// in fp32 (error below 2e-5 + 2.4e-7 |score|); when a single entry is within the margin of
// the fp32 maximum it is the fp64 argmax, otherwise the entries within the margin are scored
// again in fp64 (the definition) and the fp64 argmax decides.
constexpr int kFinishThreads = 256;

// Entries v0 .. v0 + 3 of a row (v0 % 4 == 0), -inf past V.
__device__ __forceinline__ void load4(const float* __restrict__ row, int V, int v0,
                                      float (&x)[4]) {
  if ((V & 3) == 0 && v0 + 3 < V) {
    const float4_t v = *reinterpret_cast<const float4_t*>(row + v0);
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = v[q];
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = v0 + q < V ? row[v0 + q] : -INFINITY;
  }
}

__device__ __forceinline__ void finish_row(const float* __restrict__ logits, int V, int p,
                                           const PartState* __restrict__ st, int nst,
                                           bool is_frozen, float temperature, uint32_t k0,
                                           uint32_t k1, uint32_t step,
                                           int32_t* __restrict__ tokens_out,
                                           float* __restrict__ entropy_out,
                                           float* __restrict__ conf_out) {
  constexpr int NT = kFinishThreads;
  constexpr int NW = NT / kWave;
  constexpr int EPT = kChunk / NT;  // level-2 entries per thread: one Philox call's four words
  static_assert(EPT == 4, "a chunk covers four entries per thread");
  __shared__ double wkey[NW];
  __shared__ int widx[NW];
  __shared__ float wmax[NW];
  __shared__ int sValid, sChunk, sRescore, sFallback, sCand;
  __shared__ double sLim;
  __shared__ int cand[kMaxCand];
  __shared__ PartState wst[NW];
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = lane_id();
  const bool sampled = temperature != 0.f;
  const float* row = logits + (size_t)p * V;
  const int nC = (V + kChunk - 1) / kChunk;
  // The row's states merged in a fixed order: thread t left-folds states [t q, (t + 1) q),
  // then pairs of neighbouring threads (lower first) within each wave, level by level, then
  // the waves in order.  Empty states are identities, so lanes past the end need no care.
  const int q = (nst + NT - 1) / NT;
  const int sb = tid * q, se = min(sb + q, nst);
  PartState acc = sb < nst ? st[sb] : empty_state();
  if (is_frozen) {
    if (tid == 0) {
      tokens_out[p] = -1;
      if (entropy_out != nullptr) entropy_out[p] = INFINITY;
      if (conf_out != nullptr) conf_out[p] = -1.f;
    }
    return;
  }
  for (int s = sb + 1; s < se; ++s) merge_state(acc, st[s]);
  const int active = (nst + q - 1) / q;   // threads holding states
  for (int d = 1; d < kWave && d < active; d <<= 1) {
    const PartState o = shfl_down_state(acc, d);
    if ((lane & (2 * d - 1)) == 0) merge_state(acc, o);
  }
  if (active > kWave) {
    if (lane == 0) wst[wave] = acc;
    __syncthreads();
  }
  if (tid == 0) {
    if (active > kWave)
      for (int w = 1; w < NW; ++w) merge_state(acc, wst[w]);
    float H = NAN, conf = NAN;
    bool valid = !acc.nan && acc.m != -INFINITY;
    if (valid) {
      // Z = sum exp(x - m); the top-1 probability is exp(0) / Z.
      const float Z = acc.n + acc.s;
      H = log1pf((acc.n - 1.f) + acc.s) - acc.t / Z;
      conf = 1.f / Z;
      valid = !(H != H);
    }
    sValid = valid && (!sampled || acc.best_key > -INFINITY) ? 1 : 0;
    sChunk = acc.best_c;
    sLim = acc.best_key - level1_margin(acc.best_key);
    // The merged pair is the best two keys over every state, so when the second lies outside
    // the margin the best chunk is the only candidate and nothing needs rescoring.
    sRescore = acc.second_key >= sLim ? 1 : 0;
    sFallback = 0;
    sCand = 0;
    if (entropy_out != nullptr) entropy_out[p] = valid ? H : NAN;
    if (conf_out != nullptr) conf_out[p] = valid ? conf : NAN;
    if (!valid) tokens_out[p] = -1;
    else if (!sampled) tokens_out[p] = acc.best_i;
  }
  if (!sampled) return;
  __syncthreads();
  if (!sValid) {
    if (tid == 0) tokens_out[p] = -1;   // valid row without a comparable chunk key
    return;
  }
  int bestc = sChunk;
  if (sRescore) {
    // Level 1: the chunks whose fp32 key may still be the fp64 best.
    const double lim = sLim;
    for (int s = tid; s < nst; s += NT) {
      if (st[s].second_key >= lim) sFallback = 1;
      if (st[s].best_key >= lim) {
        const int i = atomicAdd(&sCand, 1);
        if (i < kMaxCand) cand[i] = st[s].best_c;
      }
    }
    __syncthreads();
    // The second key within the margin is another state's best (a second candidate) or a
    // state's second (a state that may hold more): rescore the candidates, or every chunk.
    const bool all = sFallback || sCand > kMaxCand;
    const int n = all ? nC : sCand;
    double best = -INFINITY;
    int bc = 0x7fffffff;
    for (int i = wave; i < n; i += NW) {
      const int c = all ? i : cand[i];
      const double key = chunk_key64(row, V, c, (double)temperature, p, step, k0, k1);
      if (better_key(key, c, best, bc)) {
        best = key;
        bc = c;
      }
    }
    block_argmax<NW>(best, bc, wkey, widx);
    bestc = bc;
  }
  if (bestc < 0 || bestc >= nC) {  // no chunk had a comparable key
    if (tid == 0) tokens_out[p] = -1;
    return;
  }
  // Level 2: inside chunk bestc, maximise x_v / T + g_v, g_v from (v >> 2, p, step, 0).
  const int v0 = bestc * kChunk + EPT * tid;
  const int vend = min(V, (bestc + 1) * kChunk);
  float xv[EPT], s32[EPT];
#pragma unroll
  for (int q = 0; q < EPT; ++q) xv[q] = s32[q] = -INFINITY;
  Philox4 r = {};
  float lmax = -INFINITY;
  if (v0 < vend) {
    load4(row, V, v0, xv);
    r = philox4x32_10((uint32_t)(v0 >> 2), (uint32_t)p, step, 0u, k0, k1);
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
      if (v0 + q < vend) {
        s32[q] = xv[q] / temperature + gumbel32_from_word(r.w[(v0 + q) & 3]);
        lmax = fmaxf(lmax, s32[q]);
      }
    }
  }
  float m = wave_max(lmax);
  if (lane_id() == 0) wmax[wave] = m;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) m = fmaxf(m, wmax[w]);
  // Entries that may still be the fp64 argmax: within twice the fp32 error bound of the
  // maximum (all entries when the fp32 maximum is not finite).
  const bool everything = !(fabsf(m) < 1e30f);
  const float margin = 2e-4f + 2e-6f * fabsf(m);
  int mask = 0;
#pragma unroll
  for (int q = 0; q < EPT; ++q)
    if (v0 + q < vend && (everything || s32[q] >= m - margin)) mask |= 1 << q;
  // Candidates in the block, one barrier: per-wave counts from ballots of each entry slot.
  __shared__ int wcand[NW];
  int wc = 0;
#pragma unroll
  for (int q = 0; q < EPT; ++q) wc += __popcll(__ballot((mask >> q) & 1));
  if (lane_id() == 0) wcand[wave] = wc;
  __syncthreads();
  int cands = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) cands += wcand[w];
  if (cands == 1) {
    if (mask != 0) tokens_out[p] = v0 + __builtin_ctz(mask);
    return;
  }
  double sbest = -INFINITY;
  int sv = 0x7fffffff;
  const double T = (double)temperature;
#pragma unroll
  for (int q = 0; q < EPT; ++q) {
    if (mask & (1 << q)) {
      const double sc = (double)xv[q] / T + gumbel_from_word(r.w[(v0 + q) & 3]);
      if (better_key(sc, v0 + q, sbest, sv)) {
        sbest = sc;
        sv = v0 + q;
      }
    }
  }
  block_argmax<NW>(sbest, sv, wkey, widx);
  if (tid == 0) tokens_out[p] = sv;
}

// Second launch: one block per row merges the row's split states in split order
// and finishes the row.
__global__ __launch_bounds__(kFinishThreads) void sample_finish_kernel(
    const float* __restrict__ logits, int V, int S, float temperature, uint32_t k0, uint32_t k1,
    uint32_t step, const uint8_t* __restrict__ frozen, const PartState* __restrict__ part,
    int32_t* __restrict__ tokens_out, float* __restrict__ entropy_out,
    float* __restrict__ conf_out, const int32_t* __restrict__ gate) {
  if (gated_off(gate)) return;
  const int p = blockIdx.x;
  // The frozen flag and the first split states are read together (one memory round trip); a
  // frozen row's states were not written by the streaming pass and are not used.
  const bool is_frozen = frozen != nullptr && frozen[p] != 0;
  const int nst = S * kStreamWaves;
  finish_row(logits, V, p, part + (size_t)p * nst, nst, is_frozen, temperature, k0, k1, step,
             tokens_out, entropy_out, conf_out);
}

// ---------------------------------------------------------------- acceptance (one block)

constexpr int kAcceptThreads = 1024;

// Order-preserving map of a float to uint32 (-0 is folded onto +0).
__device__ __forceinline__ uint32_t float_order_key(float h) {
  uint32_t u = __builtin_bit_cast(uint32_t, h);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float float_from_order_key(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __builtin_bit_cast(float, u);
}

// Block-wide minimum of one 64-bit key per thread (uniform result, one barrier; wmin is an
// LDS slot of blockDim.x / 64 entries that no other thread reads before the next barrier).
__device__ __forceinline__ unsigned long long block_min_u64(unsigned long long k,
                                                            unsigned long long* wmin) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const unsigned long long o = __shfl_xor(k, off);
    k = o < k ? o : k;
  }
  if (lane_id() == 0) wmin[threadIdx.x / kWave] = k;
  __syncthreads();
  unsigned long long m = wmin[0];
  for (int w = 1; w < (int)(blockDim.x / kWave); ++w) m = wmin[w] < m ? wmin[w] : m;
  return m;
}

constexpr int kSelectSteps = 8;  // positions taken by selection before the full sort

__global__ __launch_bounds__(kAcceptThreads) void accept_kernel(
    const float* __restrict__ entropy, const int32_t* __restrict__ tokens, int P, float bound,
    uint8_t* __restrict__ frozen, int32_t* __restrict__ canvas, uint8_t* __restrict__ accept_out,
    int32_t* __restrict__ num_accepted, const int32_t* __restrict__ gate) {
  if (gated_off(gate)) return;
  __shared__ uint64_t keys[kAcceptThreads];
  __shared__ unsigned long long wmin[2][kAcceptThreads / kWave];
  __shared__ int sCount;
  // The block has n threads, n the smallest power of two >= max(P, 64); thread i holds key i.
  const int tid = threadIdx.x;
  const int n = blockDim.x;
  unsigned long long key = ~0ull;  // non-candidates sort last
  int32_t my_token = 0;            // read with the entropy: the selection takes its own position
  if (tid < P) {
    const float h = entropy[tid];
    const bool is_frozen = frozen != nullptr && frozen[tid];
    if (canvas != nullptr) my_token = tokens[tid];
    if (!is_frozen && !(h != h)) key = ((uint64_t)float_order_key(h) << 32) | (uint32_t)tid;
    accept_out[tid] = 0;
  }
  auto take = [&](int pos) {  // run by the thread that holds position pos
    accept_out[pos] = 1;
    if (canvas != nullptr) canvas[pos] = pos == tid ? my_token : tokens[pos];
    if (frozen != nullptr) frozen[pos] = 1;
  };
  // Selection: the smallest remaining key, block-wide, one at a time; every thread runs the
  // same fp32 scan on the same uniform values.  Most steps end here, after a few positions.
  float S = 0.f;
  int cnt = 0;
  bool stop = false;
  for (int it = 0; it < kSelectSteps && !stop; ++it) {
    const unsigned long long m = block_min_u64(key, wmin[it & 1]);
    if (m == ~0ull) {
      stop = true;  // no candidate left
      break;
    }
    const float h = float_from_order_key((uint32_t)(m >> 32));
    const float S2 = __fadd_rn(S, h);
    const float c = __fsub_rn(S2, h);
    const bool pass = c <= bound;
    if (pass || cnt == 0) {  // the first candidate is accepted whatever the bound
      if (key == m) {
        take(tid);
        key = ~0ull;
      }
      ++cnt;
      S = S2;
    }
    if (!pass) stop = true;
  }
  if (!stop) {
    // Still accepting: sort the remaining keys (the taken ones sort last) and continue the scan.
    // Bitonic sort, ascending, of the n keys held one per thread.  Exchanges with a partner
    // in the same wave (j < 64) go through cross-lane shuffles; wider ones through LDS.
    for (int k = 2; k <= n; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        unsigned long long other;
        if (j < kWave) {
          other = __shfl_xor(key, j);
        } else {
          keys[tid] = key;
          __syncthreads();
          other = keys[tid ^ j];
          __syncthreads();
        }
        const bool up = (tid & k) == 0;
        const bool lower = (tid & j) == 0;  // this thread holds the lower index of the pair
        key = (lower == up) ? (key < other ? key : other) : (key < other ? other : key);
      }
    }
    keys[tid] = key;
    __syncthreads();
    // One lane: the sequential fp32 scan over the sorted remainder.
    if (tid == 0) {
      int more = 0;
      bool done = false;
      for (int base = 0; base < n && !done; base += 8) {
        uint64_t kk[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) kk[q] = (base + q < n) ? keys[base + q] : ~0ull;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if (done) break;
          if (kk[q] == ~0ull) {
            done = true;
            break;
          }
          const float h = float_from_order_key((uint32_t)(kk[q] >> 32));
          S = __fadd_rn(S, h);
          const float c = __fsub_rn(S, h);
          if (!(c <= bound)) {
            done = true;
            break;
          }
          ++more;
        }
      }
      sCount = more;
    }
    __syncthreads();
    if (tid < sCount) take((int)(uint32_t)keys[tid]);
    cnt += sCount;
  }
  if (tid == 0) *num_accepted = cnt;
}

// Confidence-threshold acceptance on one workgroup.  Candidates: not frozen, confidence
// not NaN and >= 0 (frozen rows carry -1).  Every candidate with confidence > threshold is
// accepted; if none is, the candidate with the largest confidence (lowest position on ties)
// is.  The fallback key orders by confidence, then by inverted position, so one max
// reduction picks it.
__global__ __launch_bounds__(kAcceptThreads) void accept_conf_kernel(
    const float* __restrict__ conf, const int32_t* __restrict__ tokens, int P, float threshold,
    uint8_t* __restrict__ frozen, int32_t* __restrict__ canvas, uint8_t* __restrict__ accept_out,
    int32_t* __restrict__ num_accepted, const int32_t* __restrict__ gate) {
  if (gated_off(gate)) return;
  __shared__ uint64_t wbest[kAcceptThreads / kWave];
  __shared__ int sPick;
  const int tid = threadIdx.x;
  const int nw = (int)(blockDim.x / kWave);
  bool cand = false, pass = false;
  uint64_t key = 0;
  int32_t my_token = 0;
  if (tid < P) {
    const float c = conf[tid];
    const bool is_frozen = frozen != nullptr && frozen[tid];
    if (canvas != nullptr) my_token = tokens[tid];
    cand = !is_frozen && c >= 0.f;  // false for NaN
    pass = cand && c > threshold;
    if (cand) key = ((uint64_t)float_order_key(c) << 32) | (uint32_t)(0xffffffffu - (uint32_t)tid);
  }
  const int n_pass = __syncthreads_count(pass);
  bool take = pass;
  int count = n_pass;
  if (n_pass == 0) {
    for (int off = 1; off < kWave; off <<= 1) {
      const uint64_t o = __shfl_xor(key, off);
      key = o > key ? o : key;
    }
    if (lane_id() == 0) wbest[tid / kWave] = key;
    __syncthreads();
    if (tid == 0) {
      uint64_t b = 0;
      for (int w = 0; w < nw; ++w) b = wbest[w] > b ? wbest[w] : b;
      sPick = b == 0 ? -1 : (int)(0xffffffffu - (uint32_t)b);
    }
    __syncthreads();
    take = tid == sPick;
    count = sPick >= 0 ? 1 : 0;
  }
  if (tid < P) {
    accept_out[tid] = take ? 1 : 0;
    if (take) {
      if (canvas != nullptr) canvas[tid] = my_token;
      if (frozen != nullptr) frozen[tid] = 1;
    }
  }
  if (tid == 0) *num_accepted = count;
}

}  // namespace

// ---------------------------------------------------------------- host-side launchers

int sample_split_count(int P, int V) {
  const int nC = (V + kChunk - 1) / kChunk;
  int S = (BD_SAMPLE_BLOCKS + P - 1) / P;
  S = min(S, nC / 8);
  return S < 1 ? 1 : S;
}

hipError_t launch_sample_entropy(const float* logits, int P, int V, float temperature,
                                 uint64_t seed, uint32_t step, const uint8_t* frozen,
                                 int32_t* tokens_out, float* entropy_out, float* conf_out,
                                 void* workspace, hipStream_t stream, const int32_t* gate) {
  const int nC = (V + kChunk - 1) / kChunk;
  const float invT = temperature > 0.f ? 1.f / temperature : 0.f;
  const uint32_t k0 = (uint32_t)(seed & 0xffffffffu), k1 = (uint32_t)(seed >> 32);
  const int mode = temperature == 0.f ? 0 : (temperature == 1.f ? 1 : 2);
  const int S = sample_split_count(P, V);
  PartState* part = reinterpret_cast<PartState*>(workspace);
  const dim3 grid(S, P);
#define BD_STREAM(M)                                                                        \
  hipLaunchKernelGGL(sample_stream_kernel<M>, grid, dim3(kStreamThreads), 0, stream, logits, V, \
                     nC, S, invT, k0, k1, step, frozen, part, gate)
  if (mode == 0) BD_STREAM(0);
  else if (mode == 1) BD_STREAM(1);
  else BD_STREAM(2);
#undef BD_STREAM
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(sample_finish_kernel, dim3(P), dim3(kFinishThreads), 0, stream, logits, V, S,
                     temperature, k0, k1, step, frozen, part, tokens_out, entropy_out, conf_out,
                     gate);
  return hipGetLastError();
}

size_t sample_workspace_bytes(int P, int V) {
  const int S = sample_split_count(P, V);
  return align_up((size_t)P * S * kStreamWaves * sizeof(PartState));
}

hipError_t launch_accept(const float* entropy, const int32_t* tokens, int P, float bound,
                         uint8_t* frozen, int32_t* canvas, uint8_t* accept_out,
                         int32_t* num_accepted, hipStream_t stream, const int32_t* gate) {
  int n = kWave;
  while (n < P) n <<= 1;
  hipLaunchKernelGGL(accept_kernel, dim3(1), dim3(n), 0, stream, entropy, tokens, P, bound, frozen,
                     canvas, accept_out, num_accepted, gate);
  return hipGetLastError();
}

hipError_t launch_accept_confidence(const float* conf, const int32_t* tokens, int P,
                                    float threshold, uint8_t* frozen, int32_t* canvas,
                                    uint8_t* accept_out, int32_t* num_accepted,
                                    hipStream_t stream, const int32_t* gate) {
  int n = kWave;
  while (n < P) n <<= 1;
  hipLaunchKernelGGL(accept_conf_kernel, dim3(1), dim3(n), 0, stream, conf, tokens,
                     P, threshold, frozen, canvas, accept_out, num_accepted, gate);
  return hipGetLastError();
}


// ---------------------------------------------------------------- allocation-free workspace
//
// For callers that cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc): the split states of the streaming pass live in one
// static device array per GPU instead of a caller's workspace.  Its device address is looked
// up once per device with that device current and kept per device; host code uses only that
// address, never the array's name (which on the host is a stand-in, not a device pointer).
// Every call on a GPU shares its array, and the array keeps the last call's contents: the
// streaming pass writes every state the finish reads, so nothing needs clearing, and calls
// that overlap on one GPU race.

namespace {
constexpr size_t kStaticScratchBytes = 512 * 1024;
constexpr int kMaxScratchDevices = 64;
// The largest workspace: P * S * kStreamWaves states with S = min(ceil(1024 / P), ...) gives
// at most (1024 + P - 1) * kStreamWaves <= 2047 * 4 states, 256-byte aligned.
static_assert(2047 * kStreamWaves * sizeof(PartState) + 256 <= kStaticScratchBytes,
              "static sampler scratch");
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
std::mutex scratch_mu;
void* scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t static_sample_scratch(size_t need, void** out) {
  if (need > kStaticScratchBytes) return hipErrorInvalidValue;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace bd
