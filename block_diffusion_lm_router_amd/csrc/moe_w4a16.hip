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
// consecutive output rows.  The 8 waves form 4 row groups of 32 rows (two 16-row sets) times
// 2 parities: wave (g, p) contracts the 64-groups of parity p of every stage for row group g,
// and the two parities' fp32 sums are added in a fixed order at the end.  Every packed byte of
// the block's rows crosses HBM once per item.
//
// Block order.  Consecutive block ids are dispatched round-robin over the 8 XCDs.  Block b
// maps to XCD b % 8.  In the 128-row tile kernel the blocks an XCD receives walk through all
// row tiles of one item before the next, so the item's activation rows are fetched into that
// XCD's L2 once; the packed kernel orders its blocks for weight reuse instead (see there).
//
// Data movement.  The contraction dim is walked in stages of kSG 64-groups.  Packed weight
// rows and activation rows go from HBM straight into a ring of LDS stage buffers with
// global_load_lds_dwordx4 (no VGPRs held while in flight); each wave fetches its own
// weight rows (whole 16-byte chunks of kSG*32 contiguous bytes per row) and a share of
// the block's activation rows, kDepth stages ahead.  The compiler does not order LDS reads
// after these loads, so each stage starts with an explicit s_waitcnt vmcnt for the wave's
// own loads followed by a block barrier.  Scales and zero-points (two halves per row and
// group) are fetched through registers and written to the stage buffer before the barrier.
// Both LDS layouts are XOR-swizzled by row so that MFMA fragment reads are conflict-free.
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
// of a lane's 8 weights is therefore (0,4,1,5,2,6,3,7); the activations are stored in the same
// order (x by a small permutation pass before gate/up, h by the gate/up epilogue), so the
// contraction is unchanged.  The 64-group partial sums come
// out of MFMA in fp32 and are scaled by that group's fp16 scale in fp32.

#include "bd_device.hpp"
#include "bd_internal.hpp"

namespace bd {

namespace {

#ifndef BD_STAGE_GROUPS
#define BD_STAGE_GROUPS 2
#endif
#ifndef BD_DEPTH
#define BD_DEPTH 2
#endif

constexpr int kThreads = 512;                        // 8 waves: 4 row groups x 2 group parities
constexpr int kRowGroups = 4;                        // 32 weight rows each
constexpr int kRowsPerBlock = 128;
constexpr int kXcds = 8;
constexpr int kSG = BD_STAGE_GROUPS;                 // 64-groups per stage (2 or 4)
constexpr int kRing = BD_DEPTH + 1;                 // stage buffers at the largest item size
constexpr int kStageK = kSG * 64;
constexpr int kWRowBytes = kSG * 32;                 // packed bytes of one row per stage
constexpr int kWChunks = kWRowBytes / 16;            // 16-byte chunks per row per stage
constexpr int kWRowsPerLoad = 1024 / kWRowBytes;     // rows covered by one wave-wide load
constexpr int kWLoads = 32 / kWRowsPerLoad;          // loads per wave per stage (32 rows)
constexpr int kWWaveBytes = 32 * kWRowBytes;
constexpr int kWBytes = kRowGroups * kWWaveBytes;
constexpr int kXRowBytes = kStageK * 2;
constexpr int kXChunks = kXRowBytes / 16;
constexpr int kXRowsPerLoad = 1024 / kXRowBytes;
// The ring holds kRingBytes.  A stage is the weight tile plus NMT*16 activation rows, so items
// of at most 16 tokens fit one more stage in flight than items of up to 32.
constexpr int kRingBytes = kRing * (kWBytes + kItemTokens * kXRowBytes);
template <int NMT>
struct Ring {
  static constexpr int kXBytes = NMT * 16 * kXRowBytes;
  static constexpr int kStageBytes = kWBytes + kXBytes;
  static constexpr int kSlots = kRingBytes / kStageBytes;
  static constexpr int kDepth = kSlots - 1;          // stages in flight ahead of compute
};
// Scale and zero-point tables of the block's 128 rows for the whole contraction dim, loaded
// once per block: [2 arrays][128 rows][G] halves.  G is at most kMaxGroups.
constexpr int kMaxGroups = 64;
constexpr int kSZTableBytes = 2 * kRowsPerBlock * kMaxGroups * 2;
constexpr int kLdsBytes = kRingBytes + kSZTableBytes;
static_assert(kItemTokens == 16 || kItemTokens == 32, "work items hold at most 32 tokens");
static_assert(kWChunks * 16 == kWRowBytes && kXChunks >= 16, "stage geometry");
static_assert(kWLoads == 2 && kSG % 2 == 0, "one weight load per wave per stage");

// Row swizzles: rows that alias in the 64 LDS banks get different chunk rotations.
__device__ __forceinline__ int wswz(int r) { return (r / (64 / (kWRowBytes / 4))) & (kWChunks - 1); }
__device__ __forceinline__ int xswz(int m) { return m & 15; }

struct GemmArgs {
  const uint8_t* q;        // [E][R][K/2]
  const uint16_t* scale;   // [E][R][K/64]
  const uint16_t* zero;    // [E][R][K/64]
  int K;                   // contraction dim
  int R;                   // rows per expert
  int d_ff;                // gate/up: first up row
  int top_k;
  int tiles;               // row tiles per item
  const uint16_t* act;     // gate/up: x [T][K]; down: h [T*k][K] (bucket order); both k-permuted
  const int32_t* perm;     // bucket position -> assignment t*k + j
  const int32_t* items;    // [0] = count, then (expert, first position, tokens)
  const uint8_t* pk;       // packed stream (packed kernel), see pack_kernel
  uint16_t* h_out;         // gate/up output [T*k][d_ff]
  float* o_out;            // down output [T*k][d_model]
  int out_ld;
  int affine;              // packed stream holds (scale, bias) of w = q s + b, not (scale, zero)
  int E;                   // experts
  int A;                   // assignments T * top_k of this call
  int max_items;           // capacity of the work list
  const int32_t* gate;     // loop driver state or NULL (see gated_off)
  int sz_compact;          // packed stream with one (scale, zero) pair per row and stage
};

// Work item `item` of the list: (expert, first bucket position, tokens), every value clamped
// into the ranges of this call, so that no workspace content can index past the caller's
// buffers (a workspace routed for another shape gives wrong outputs, never a wild access).
struct Item {
  int e, pos0, mcount;
};
__device__ __forceinline__ int item_count(const GemmArgs& a) {
  return min(max(a.items[0], 0), a.max_items);
}
__device__ __forceinline__ Item load_item(const GemmArgs& a, int item) {
  Item it;
  it.e = min(max(a.items[1 + 3 * item], 0), a.E - 1);
  it.pos0 = min(max(a.items[2 + 3 * item], 0), a.A - 1);
  it.mcount = min(max(a.items[3 + 3 * item], 1), min(kItemTokens, a.A - it.pos0));
  return it;
}
// Assignment t*k + j at a bucket position, clamped into [0, A).
__device__ __forceinline__ int perm_at(const GemmArgs& a, int pos) {
  return min(max(a.perm[pos], 0), a.A - 1);
}

// The masks and the magic exponent are passed in registers (see DequantConsts) so that each
// (w & mask) | magic is one v_and_or_b32.
struct DequantConsts {
  uint32_t lo, hi, magic;
};
__device__ __forceinline__ DequantConsts dequant_consts() {
  DequantConsts k;
  asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(k.lo));
  asm volatile("v_mov_b32 %0, 0x00f000f0" : "=v"(k.hi));
  asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(k.magic));
  return k;
}

__device__ __forceinline__ half8_t dequant8(uint32_t w, _Float16 zc1, _Float16 zc2,
                                            const DequantConsts& k) {
  const uint32_t kLo = k.lo, kHi = k.hi, kMagic = k.magic;
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

// Affine form (w = q s + b with a free fp16 bias): the same nibble extraction, the exact fp16
// q (one packed add or fma), then one packed fma q s + b, rounded once to fp16.  The weights
// come out in the same k-order as dequant8's.
__device__ __forceinline__ half8_t dequant8_affine(uint32_t w, half2_t s2, half2_t b2,
                                                   const DequantConsts& k) {
  const uint32_t kLo = k.lo, kHi = k.hi, kMagic = k.magic;
  const uint32_t a = (w & kLo) | kMagic;
  const uint32_t b = (w & kHi) | kMagic;
  const uint32_t w8 = w >> 8;
  const uint32_t c = (w8 & kLo) | kMagic;
  const uint32_t d = (w8 & kHi) | kMagic;
  const half2_t m1024 = {(_Float16)-1024.f, (_Float16)-1024.f};
  const half2_t m64 = {(_Float16)-64.f, (_Float16)-64.f};
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t qa = __builtin_bit_cast(half2_t, a) + m1024;
  const half2_t qb = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, b), sixteenth, m64);
  const half2_t qc = __builtin_bit_cast(half2_t, c) + m1024;
  const half2_t qd = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, d), sixteenth, m64);
  const half2_t ha = __builtin_elementwise_fma(qa, s2, b2);
  const half2_t hb = __builtin_elementwise_fma(qb, s2, b2);
  const half2_t hc = __builtin_elementwise_fma(qc, s2, b2);
  const half2_t hd = __builtin_elementwise_fma(qd, s2, b2);
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

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float gelu_tanh(float a) {
  const float u = 0.7978845608028654f * fmaf(0.044715f * a, a * a, a);
  const float th = 1.f - 2.f / (1.f + __expf(2.f * u));
  return 0.5f * a * (1.f + th);
}

// Wait until at most N of this wave's vector-memory operations are outstanding.  Written as
// asm with a memory clobber so that no LDS read is scheduled above it.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Block barrier for LDS data only: this wave's LDS writes complete, then s_barrier.  Unlike
// __syncthreads() it does not drain outstanding global loads (the stage prefetches).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <bool GATED, int NMT>
__device__ __forceinline__ void gemm_item(const GemmArgs& a, char* lds, int e, int pos0,
                                          int mcount, int tile) {
  // Per stage the block issues 2 weight loads per row group and 4*NMT activation loads (4 rows
  // each).  Wave (rg, par) issues the weight load of set par of row group rg and activation
  // load rg + 4*par if that one exists.
  constexpr int kXLoadsBlock = (NMT * 16) / kXRowsPerLoad;
  static_assert(kXLoadsBlock == 4 || kXLoadsBlock == 8, "activation loads per stage");
  constexpr int kStageBytes = Ring<NMT>::kStageBytes;
  constexpr int kSlots = Ring<NMT>::kSlots;
  constexpr int kDepth = Ring<NMT>::kDepth;
  static_assert(kDepth >= 1 && 2 * kDepth < 64, "ring depth");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const int rg = wave & 3;                 // row group: 32 weight rows
  const int par = wave >> 2;               // which 64-groups of each stage this wave contracts
  const bool xload = rg + 4 * par < kXLoadsBlock;
  const int n = lane & 15;
  const int kb = lane >> 4;
  const int G = a.K >> 6;
  const int NS = (G + kSG - 1) / kSG;
  const size_t rowbytes = (size_t)(a.K >> 1);
  const DequantConsts dq = dequant_consts();

  // Weight rows of this row group: set A = rows rA0.., set B = rows rB0.. (16 each).
  const int rA0 = GATED ? tile * 64 + rg * 16 : tile * kRowsPerBlock + rg * 32;
  const int rB0 = GATED ? a.d_ff + rA0 : rA0 + 16;
  const int slotA = GATED ? rg * 16 + n : rg * 32 + n;         // rows in the scale table
  const int slotB = GATED ? 64 + rg * 16 + n : rg * 32 + 16 + n;
  // Weight load: rows of set `par`; lane -> (row, chunk slot), the slot holding global chunk
  // slot ^ wswz(row).
  const int wr = lane / kWChunks;                               // 0..15
  const uint8_t* wsrc = a.q + ((size_t)e * a.R + (par ? rB0 : rA0) + wr) * rowbytes;
  const int wchunk = (lane % kWChunks) ^ wswz(wr);
  // Activation load rg + 4*par: rows (rg + 4*par)*4 + lane/16.
  const int xm = (rg + 4 * par) * kXRowsPerLoad + lane / kXChunks;
  const uint16_t* xsrc;
  {
    const int mm = min(xm, mcount - 1);                         // padding rows re-read a valid row
    const int row = GATED ? perm_at(a, pos0 + mm) / a.top_k : pos0 + mm;
    xsrc = a.act + (size_t)row * a.K;   // both activations are stored k-permuted
  }
  const int xchunk = (lane % kXChunks) ^ xswz(xm);

  // Scale / zero-point table, copied once: the block's rows form contiguous 16-byte aligned
  // ranges of each array (gate/up: 64 gate rows and 64 up rows; down: 128 rows), laid out in
  // LDS back to back as [array][row slot][group].  Chunk q (16 bytes) of the concatenated
  // ranges goes to table byte 16q; a wave-wide copy covers 64 consecutive chunks, and lanes
  // past the end re-read the last chunk into the table's padding.
  char* sztab = lds + kRingBytes;
  {
    const int rows = GATED ? 64 : kRowsPerBlock;
    const int rchunks = rows * G * 2 / 16;
    const int ranges = GATED ? 4 : 2;
    const int total = ranges * rchunks;
    for (int q0 = wave * 64; q0 < total; q0 += kThreads) {
      const int q = min(q0 + lane, total - 1);
      const int rng = q / rchunks;
      const int arr = GATED ? (rng >> 1) : rng;
      const int row0 = GATED ? ((rng & 1) ? a.d_ff : 0) + tile * 64 : tile * kRowsPerBlock;
      const char* src = reinterpret_cast<const char*>((arr ? a.zero : a.scale) +
                                                      ((size_t)e * a.R + row0) * G) +
                        (q % rchunks) * 16;
      __builtin_amdgcn_global_load_lds(src, sztab + q0 * 16, 16, 0, 0);
    }
  }
  const _Float16* stab = reinterpret_cast<const _Float16*>(sztab);
  const _Float16* ztab = stab + kRowsPerBlock * G;

  // Issue this wave's loads of stage c into ring slot `slot`.  Chunks past the last group
  // (odd G) re-read group 0 of their row; compute never uses them.
  auto dma = [&](int c, int slot) {
    char* st = lds + slot * kStageBytes;
    int byte = c * kWRowBytes + wchunk * 16;
    if ((byte >> 5) >= G) byte &= 31;
    __builtin_amdgcn_global_load_lds(wsrc + byte, st + rg * kWWaveBytes + par * 1024, 16, 0, 0);
    if (xload) {
      int col = c * kStageK + xchunk * 8;
      if (col >= a.K) col &= 63;
      __builtin_amdgcn_global_load_lds(xsrc + col, st + kWBytes + (rg + 4 * par) * 1024, 16, 0, 0);
    }
  };

  float4_t totA[NMT], totB[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    totA[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
    totB[mt] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
  const float4_t zero4 = {0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int c, int slot) {
    const char* st = lds + slot * kStageBytes;
    const char* wbase = st + rg * kWWaveBytes;
    const char* xbase = st + kWBytes;
#pragma unroll
    for (int gq = 0; gq < kSG / 2; ++gq) {
      const int gl = 2 * gq + par;
      const int g = c * kSG + gl;
      if (g >= G) break;
      const int chunk = 2 * gl + (kb >> 1);
      const int sw = wswz(n);
      const u32x2_t wa = *reinterpret_cast<const u32x2_t*>(
          wbase + n * kWRowBytes + ((chunk ^ sw) << 4) + ((kb & 1) << 3));
      const u32x2_t wb = *reinterpret_cast<const u32x2_t*>(
          wbase + (16 + n) * kWRowBytes + ((chunk ^ sw) << 4) + ((kb & 1) << 3));
      const _Float16 za = ztab[slotA * G + g], zb = ztab[slotB * G + g];
      const float fsA = (float)stab[slotA * G + g], fsB = (float)stab[slotB * G + g];
      const _Float16 za1 = -((_Float16)1024.f + za), za2 = -((_Float16)64.f + za);
      const _Float16 zb1 = -((_Float16)1024.f + zb), zb2 = -((_Float16)64.f + zb);
      const half8_t bA0 = dequant8(wa[0], za1, za2, dq);
      const half8_t bA1 = dequant8(wa[1], za1, za2, dq);
      const half8_t bB0 = dequant8(wb[0], zb1, zb2, dq);
      const half8_t bB1 = dequant8(wb[1], zb1, zb2, dq);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const int m = mt * 16 + n;
        const char* xrow = xbase + m * kXRowBytes;
        const int c8 = gl * 8 + kb * 2;                      // 8-half chunk of step 0
        const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(xrow + (((c8 + 0) ^ xswz(m)) << 4));
        const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(xrow + (((c8 + 1) ^ xswz(m)) << 4));
        const half8_t a0 = __builtin_bit_cast(half8_t, v0);
        const half8_t a1 = __builtin_bit_cast(half8_t, v1);
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
  };

  // Prologue: the first kDepth stages in flight (stages past the end re-read the last one).
#pragma unroll
  for (int s = 0; s < kDepth; ++s) dma(min(s, NS - 1), s);
  // Every stage issues the loads of stage cc + kDepth, also past the end (re-reading the last
  // stage, an L2 hit, into a ring slot nobody reads), so the number of loads this wave issued
  // after a stage's own is always its per-stage count times kDepth - 1.  Loads complete in
  // order, so waiting down to that many outstanding completes the stage's loads (and the table
  // copy issued before them); the barrier then publishes every wave's loads to the block.
  for (int c = 0; c < NS; c += kSlots) {
#pragma unroll
    for (int u = 0; u < kSlots; ++u) {  // unrolled so every ring slot is a constant
      const int cc = c + u;
      if (cc >= NS) break;
      if (xload)
        wait_vmcnt<2 * (kDepth - 1)>();
      else
        wait_vmcnt<1 * (kDepth - 1)>();
      lds_barrier();
      dma(min(cc + kDepth, NS - 1), (u + kDepth) % kSlots);
      compute(cc, u);
    }
  }
  wait_vmcnt<0>();   // no LDS write may still be in flight when the block ends

  // Reduce the two group parities of each row group in a fixed order (par 0 + par 1), in the
  // ring's LDS, which no load targets any more.
  lds_barrier();
  float* red = reinterpret_cast<float*>(lds) + (rg * 64 + lane) * (NMT * 8);
  if (par == 1) {
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        red[mt * 8 + r] = totA[mt][r];
        red[mt * 8 + 4 + r] = totB[mt][r];
      }
  }
  lds_barrier();
  if (par == 1) return;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      totA[mt][r] += red[mt * 8 + r];
      totB[mt][r] += red[mt * 8 + 4 + r];
    }

  // Epilogue: D lane layout = tokens 4kb..4kb+3 of weight row n.
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mt * 16 + kb * 4 + r;
      if (m >= mcount) continue;
      if (GATED) {
        const float hv = gelu_tanh(totA[mt][r]) * totB[mt][r];
        const int col = tile * 64 + rg * 16 + n;
        const int pcol = (col & ~7) | ((col & 3) << 1) | ((col >> 2) & 1);
        const _Float16 h16 = (_Float16)hv;
        a.h_out[(size_t)(pos0 + m) * a.d_ff + pcol] = __builtin_bit_cast(uint16_t, h16);
      } else {
        const int slot = perm_at(a, pos0 + m);
        const int row = tile * kRowsPerBlock + rg * 32 + n;
        a.o_out[(size_t)slot * a.out_ld + row] = totA[mt][r];
        a.o_out[(size_t)slot * a.out_ld + row + 16] = totB[mt][r];
      }
    }
  }
}

template <bool GATED>
__global__ __launch_bounds__(kThreads) void w4a16_gemm_kernel(GemmArgs a) {
  if (gated_off(a.gate)) return;
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int b = blockIdx.x;
  const int local = b / kXcds;
  const int item = (local / a.tiles) * kXcds + (b % kXcds);
  const int tile = local % a.tiles;
  if (item >= item_count(a)) return;
  const Item it = load_item(a, item);
  const int e = it.e, pos0 = it.pos0, mcount = it.mcount;
  if (kItemTokens > 16 && mcount > 16)
    gemm_item<GATED, (kItemTokens > 16 ? 2 : 1)>(a, lds, e, pos0, mcount, tile);
  else
    gemm_item<GATED, 1>(a, lds, e, pos0, mcount, tile);
}


int grid_blocks(int max_items, int tiles) {
  return ((max_items + kXcds - 1) / kXcds) * kXcds * tiles;
}

// ------------------------------------------------------------------ packed kernel
//
// The same GEMM on 256-row tiles over weights repacked once by pack_kernel.  The packed
// stream of an (expert, tile) is its stages in order, each 18 KB: for waves w = 0..7 and row
// sets S = A, B the 1 KB that wave w's lanes consume (lane (n, kb): row n of the set, bytes
// 8kb..8kb+7 of group 2s and of group 2s+1), then 2 KB of scales and zero-points (for wave w,
// row n: scale and zero-point of groups 2s and 2s+1 of row n of set A, then of set B).  Every
// wave therefore streams its own weights, scales and zero-points straight into registers with
// 16-byte loads over contiguous 1 KB runs, kDepth stages ahead, with no LDS and no barrier on
// that path; the loads are unconditional, so the compiler counts them exactly.  Only the
// activation tile of a stage is shared by the 8 waves: each wave loads its share into registers
// with the stage's other loads and writes it to an LDS double buffer one stage ahead of use.
//
// Rows: gate/up wave w holds gate columns 16w..16w+15 of the tile (set A) and the matching up
// rows (set B); down wave w holds rows 32w..32w+31 (A: first 16, B: next 16).  A tile past the
// end of the matrix (d_ff % 128 == 64, d_model % 256 == 128) leaves waves 4..7 without rows:
// they re-load wave w-4's stream (L2 hits), keep their activation duties and skip compute.
constexpr int kPkRows = 256;
constexpr int kPkWBytes = kPkRows * kWRowBytes;                 // 16 KB of nibbles per stage
constexpr int kPkSZBytes = kPkRows * 8;                         // 2 KB of scales/zero-points
constexpr int kPkStage = kPkWBytes + kPkSZBytes;                // 18 KB
constexpr int kPkChunks = kPkStage / 16;
// A gate/up matrix grouped at 128 has one group per stage, so its stage holds one (scale,
// zero) pair per row: 1 KB instead of 2 KB (see pack_kernel).
constexpr int kPkSZBytesC = kPkRows * 4;
constexpr int kPkStageC = kPkWBytes + kPkSZBytesC;              // 17 KB
constexpr int kPkChunksC = kPkStageC / 16;
constexpr int kPkDepth = 3;                                     // stages in registers ahead
constexpr int kPkXSlot = kItemTokens * kXRowBytes;              // 8 KB
static_assert(kSG == 2 && kItemTokens == 32 && kXRowBytes == 256, "packed stage geometry");

// One 64-group of a stage for a wave's two 16-row sets (A, B) and NMT 16-token tiles: the
// weights dequantised into MFMA operands, the activation fragments from the LDS tile, and the
// products added to the running fp32 sums.  Asymmetric form: exact fp16 (q - z), the group's
// MFMA sum scaled by its fp32 scale.  Affine form: fp16 q s + b, accumulated directly.
// sz holds, per set, (scale g0, scale g1, zero or bias g0, zero or bias g1).
// The zero-point constants of both groups of a stage for one row set, formed with two packed
// ops: -(1024 + z) for the low nibbles and -(64 + z) for the high ones (see dequant8).
struct ZeroPairs {
  half2_t z1, z2;
};
__device__ __forceinline__ ZeroPairs zero_pairs(half4_t sz) {
  const half2_t z = {sz[2], sz[3]};
  const half2_t k1024 = {(_Float16)1024.f, (_Float16)1024.f};
  const half2_t k64 = {(_Float16)64.f, (_Float16)64.f};
  return ZeroPairs{-(k1024 + z), -(k64 + z)};
}

template <int NMT, bool AFF>
__device__ __forceinline__ void group_mfma(const u32x4_t& wa, const u32x4_t& wb, half4_t szA,
                                           half4_t szB, const ZeroPairs& zpA,
                                           const ZeroPairs& zpB, int j, const char* xt, int n,
                                           int kb, float4_t (&totA)[NMT], float4_t (&totB)[NMT],
                                           const DequantConsts& dq) {
  half8_t bA0, bA1, bB0, bB1;
  float fsA = 0.f, fsB = 0.f;
  if constexpr (AFF) {
    const half2_t sA = {szA[j], szA[j]}, oA = {szA[2 + j], szA[2 + j]};
    const half2_t sB = {szB[j], szB[j]}, oB = {szB[2 + j], szB[2 + j]};
    bA0 = dequant8_affine(wa[2 * j], sA, oA, dq);
    bA1 = dequant8_affine(wa[2 * j + 1], sA, oA, dq);
    bB0 = dequant8_affine(wb[2 * j], sB, oB, dq);
    bB1 = dequant8_affine(wb[2 * j + 1], sB, oB, dq);
  } else {
    const _Float16 za1 = zpA.z1[j], za2 = zpA.z2[j];
    const _Float16 zb1 = zpB.z1[j], zb2 = zpB.z2[j];
    fsA = (float)szA[j];
    fsB = (float)szB[j];
    bA0 = dequant8(wa[2 * j], za1, za2, dq);
    bA1 = dequant8(wa[2 * j + 1], za1, za2, dq);
    bB0 = dequant8(wb[2 * j], zb1, zb2, dq);
    bB1 = dequant8(wb[2 * j + 1], zb1, zb2, dq);
  }
  const float4_t zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
    const int m = mt * 16 + n;
    const char* xrow = xt + m * kXRowBytes;
    const int c8 = j * 8 + kb * 2;
    const half8_t a0 = __builtin_bit_cast(half8_t, *reinterpret_cast<const u32x4_t*>(xrow + (((c8 + 0) ^ xswz(m)) << 4)));
    const half8_t a1 = __builtin_bit_cast(half8_t, *reinterpret_cast<const u32x4_t*>(xrow + (((c8 + 1) ^ xswz(m)) << 4)));
    if constexpr (AFF) {
      totA[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bA0, totA[mt], 0, 0, 0);
      totA[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bA1, totA[mt], 0, 0, 0);
      totB[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bB0, totB[mt], 0, 0, 0);
      totB[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bB1, totB[mt], 0, 0, 0);
    } else {
      float4_t accA = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bA0, zero4, 0, 0, 0);
      accA = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bA1, accA, 0, 0, 0);
      float4_t accB = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, bB0, zero4, 0, 0, 0);
      accB = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, bB1, accB, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        totA[mt][q] = fmaf(fsA, accA[q], totA[mt][q]);
        totB[mt][q] = fmaf(fsB, accB[q], totB[mt][q]);
      }
    }
  }
}

// Buffer loads: a block-uniform descriptor (base, byte range) in scalar registers, a lane
// offset in one VGPR and the stage offset in a scalar register, so that a stage's loads cost
// no vector address arithmetic; a read past the range returns zeros.  Word 3 of a gfx9
// descriptor: raw 32-bit data, no swizzle.  AUX 2 marks the load nontemporal (the line is not
// kept for reuse), used for weight streams that no other block reads.
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRsrcWord3);
}
template <int AUX>
__device__ __forceinline__ u32x4_t bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t,
                            __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, AUX));
}
template <int AUX>
__device__ __forceinline__ u32x2_t bload64(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                           uint32_t soff) {
  return __builtin_bit_cast(u32x2_t,
                            __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, AUX));
}
// Both halves of a word set to its low (high) half: (s, z) of a 128-group becomes the
// (s, s) and (z, z) pairs of its two 64-groups.
__device__ __forceinline__ uint32_t dup_lo(uint32_t v) { return __builtin_amdgcn_perm(v, v, 0x01000100u); }
__device__ __forceinline__ uint32_t dup_hi(uint32_t v) { return __builtin_amdgcn_perm(v, v, 0x03020302u); }

struct PkStage {
  u32x4_t wa, wb, sz, x;
};

template <bool GATED, int NMT, int NSC, bool AFF, bool NT, bool CSZ>
__device__ __forceinline__ void packed_item(const GemmArgs& a, char* lds, int e, int pos0,
                                            int mcount, int tile) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int kb = lane >> 4;
  const int G = a.K >> 6;
  const int NS = NSC > 0 ? NSC : (G + 1) >> 1;
  const DequantConsts dq = dequant_consts();

  const int rows_here = GATED ? min(128, a.d_ff - tile * 128) : min(kPkRows, a.R - tile * kPkRows);
  const bool valid = GATED ? wave * 16 < rows_here : wave * 32 < rows_here;
  const int lw = valid ? wave : wave - 4;              // whose stream this wave loads
  // The (expert, tile) stream: one descriptor, the lane's offsets within a stage.
  constexpr int kStage = CSZ ? kPkStageC : kPkStage;
  const uint32_t stream_bytes = (uint32_t)NS * kStage;
  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(a.pk + ((size_t)e * a.tiles + tile) * stream_bytes, stream_bytes);
  const uint32_t wa_off = ((lw * 2 + 0) * 64 + lane) * 16;
  const uint32_t sz_off = kPkWBytes + (lw * 16 + n) * (CSZ ? 8 : 16);

  // Activation share: thread tid loads the 16-byte chunk tid % 16 of row (tid / 16) mod
  // 16*NMT of the stage; with NMT = 1 the upper 256 threads repeat the lower ones' loads and
  // do not write.  Gate/up reads x as given and puts each chunk into the dequantised
  // weights' k-order (permute8) on its way to LDS; down reads h, already in that order.
  const int xm = (tid >> 4) & (NMT * 16 - 1);
  const int xc = tid & 15;
  const bool x_writer = tid < NMT * 256;
  // Activation rows: gate/up gathers token rows of x [T][K] (T * K * 2 < 2^32 bytes); down
  // reads the item's consecutive rows of h [T * k][K] from the item's first row on.  The
  // chunks past K in the half stage of an odd group count read whatever follows (or zeros past
  // the range) and are never used.
  const __amdgpu_buffer_rsrc_t xrs =
      GATED ? make_rsrc(a.act, (uint32_t)(a.A / a.top_k) * (uint32_t)a.K * 2u)
            : make_rsrc(a.act + (size_t)pos0 * a.K, (uint32_t)mcount * (uint32_t)a.K * 2u);
  uint32_t x_off;
  {
    const int mm = min(xm, mcount - 1);
    const int row = GATED ? perm_at(a, pos0 + mm) / a.top_k : mm;
    x_off = ((uint32_t)row * (uint32_t)a.K + xc * 8) * 2;
  }
  const int xdst = xm * kXRowBytes + ((xc ^ xswz(xm)) << 4);
  constexpr int kAux = NT ? 2 : 0;

  auto load = [&](int c) {
    const uint32_t st = (uint32_t)min(c, NS - 1) * kStage;
    PkStage r;
    r.x = bload<0>(xrs, x_off, (uint32_t)min(c, NS - 1) * kStageK * 2);
    r.wa = bload<kAux>(wrs, wa_off, st);
    r.wb = bload<kAux>(wrs, wa_off + 1024, st);
    if constexpr (CSZ) {
      const u32x2_t v = bload64<kAux>(wrs, sz_off, st);
      r.sz = u32x4_t{v[0], v[1], 0u, 0u};
    } else {
      r.sz = bload<kAux>(wrs, sz_off, st);
    }
    return r;
  };
  auto put_x = [&](const PkStage& r, int slot) {
    if (x_writer)
      *reinterpret_cast<u32x4_t*>(lds + slot * kPkXSlot + xdst) = GATED ? permute8(r.x) : r.x;
  };

  float4_t totA[NMT], totB[NMT];
  const float4_t zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) totA[mt] = totB[mt] = zero4;

  auto compute = [&](const PkStage& r, int c, int slot) {
    const char* xt = lds + slot * kPkXSlot;
    // [scale g0, scale g1, zero g0, zero g1] of the lane's row in set A, then set B
    const half4_t szA = CSZ ? __builtin_bit_cast(half4_t, u32x2_t{dup_lo(r.sz[0]), dup_hi(r.sz[0])})
                            : __builtin_bit_cast(half4_t, u32x2_t{r.sz[0], r.sz[1]});
    const half4_t szB = CSZ ? __builtin_bit_cast(half4_t, u32x2_t{dup_lo(r.sz[1]), dup_hi(r.sz[1])})
                            : __builtin_bit_cast(half4_t, u32x2_t{r.sz[2], r.sz[3]});
    const ZeroPairs zpA = zero_pairs(szA), zpB = zero_pairs(szB);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int g = 2 * c + j;
      if (g >= G) break;
      group_mfma<NMT, AFF>(r.wa, r.wb, szA, szB, zpA, zpB, j, xt, n, kb, totA, totB, dq);
    }
  };

  // Stage c sits in buf[c % kPkDepth] from iteration c - kPkDepth on; its activation share is
  // written to LDS slot c % 2 during iteration c - 1, and the barrier that ends iteration c - 1
  // publishes it.  The barrier ending iteration c also frees slot c % 2 for stage c + 2.
  PkStage buf[kPkDepth];
#pragma unroll
  for (int s2 = 0; s2 < kPkDepth; ++s2) buf[s2] = load(s2);
  put_x(buf[0], 0);
  lds_barrier();
  if constexpr (NSC > 0) {
    // Contraction dims with a specialisation: the stage loop is unrolled completely, so
    // every stage's registers are distinct values in straight-line code and each wait the
    // compiler places covers exactly the loads that stage needs.
#pragma unroll
    for (int cc = 0; cc < NSC; ++cc) {
      if (cc + 1 < NSC) put_x(buf[(cc + 1) % kPkDepth], (cc + 1) & 1);
      if (valid) compute(buf[cc % kPkDepth], cc, cc & 1);
      if (cc + kPkDepth < NSC) buf[cc % kPkDepth] = load(cc + kPkDepth);
      if (cc + 1 < NSC) lds_barrier();
    }
  } else {
    // Other dims: whole rounds of kPkDepth stages (stages past the end load the last stage
    // again and skip compute), the same loads in the same order on every path.
    for (int c = 0; c < NS; c += kPkDepth) {
#pragma unroll
      for (int u = 0; u < kPkDepth; ++u) {
        const int cc = c + u;
        put_x(buf[(u + 1) % kPkDepth], (u + 1 + c) & 1);
        if (valid && cc < NS) compute(buf[u], cc, (u + c) & 1);
        buf[u] = load(cc + kPkDepth);
        lds_barrier();
      }
    }
  }
  if (!valid) return;

  // Epilogue: D lane layout = tokens 4kb..4kb+3 of row n.
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mt * 16 + kb * 4 + r;
      if (m >= mcount) continue;
      if (GATED) {
        const float hv = gelu_tanh(totA[mt][r]) * totB[mt][r];
        const int col = tile * 128 + wave * 16 + n;
        const int pcol = (col & ~7) | ((col & 3) << 1) | ((col >> 2) & 1);
        const _Float16 h16 = (_Float16)hv;
        a.h_out[(size_t)(pos0 + m) * a.d_ff + pcol] = __builtin_bit_cast(uint16_t, h16);
      } else {
        const int slot = perm_at(a, pos0 + m);
        const int row = tile * kPkRows + wave * 32 + n;
        a.o_out[(size_t)slot * a.out_ld + row] = totA[mt][r];
        a.o_out[(size_t)slot * a.out_ld + row + 16] = totB[mt][r];
      }
    }
  }
}

// The item's path: two 16-token tiles above 16 tokens, nontemporal weight loads when this
// block reads the expert's stream alone, the compact scale/zero layout of 128-groups.
template <bool GATED, int NSC, bool AFF, bool CSZ>
__device__ __forceinline__ void packed_dispatch(const GemmArgs& a, char* lds, int e, int pos0,
                                                int mcount, int tile, bool alone) {
  if (mcount > 16) {
    if (alone)
      packed_item<GATED, 2, NSC, AFF, true, CSZ>(a, lds, e, pos0, mcount, tile);
    else
      packed_item<GATED, 2, NSC, AFF, false, CSZ>(a, lds, e, pos0, mcount, tile);
  } else {
    if (alone)
      packed_item<GATED, 1, NSC, AFF, true, CSZ>(a, lds, e, pos0, mcount, tile);
    else
      packed_item<GATED, 1, NSC, AFF, false, CSZ>(a, lds, e, pos0, mcount, tile);
  }
}

// NSC > 0: compiled for exactly NSC stages (the caller checks); 0: any number of stages.
template <bool GATED, int NSC, bool AFF>
__global__ __launch_bounds__(kThreads, 2) void w4a16_packed_kernel(GemmArgs a) {
  if (gated_off(a.gate)) return;
  __shared__ __attribute__((aligned(16))) char lds[2 * kPkXSlot];
  // XCD b % 8 owns a contiguous range of work items (the items of one expert are consecutive,
  // so a hot expert's items mostly share an XCD) and walks it tile-major: the blocks of one
  // tile of neighbouring items start together, and all but the first read the tile's stream
  // from that XCD's L2.
  const int b = blockIdx.x;
  const int n_items = item_count(a);
  const int per = (n_items + kXcds - 1) / kXcds;
  const int local = b / kXcds;
  const int tile = local / per;
  const int item = (b % kXcds) * per + local % per;
  if (tile >= a.tiles || item >= n_items) return;
  const Item it = load_item(a, item);
  const int e = it.e, pos0 = it.pos0, mcount = it.mcount;
  // An expert whose tokens fit one work item has its stream read by this block alone: those
  // loads are nontemporal.  An expert split over several items keeps them cached, so that its
  // other items' blocks on the same XCD read the stream from L2.
  const bool alone = (item == 0 || a.items[1 + 3 * (item - 1)] != a.items[1 + 3 * item]) &&
                     (item + 1 >= n_items || a.items[1 + 3 * (item + 1)] != a.items[1 + 3 * item]);
  if (GATED && a.sz_compact) {
    if constexpr (GATED) packed_dispatch<GATED, NSC, AFF, true>(a, lds, e, pos0, mcount, tile, alone);
  } else {
    packed_dispatch<GATED, NSC, AFF, false>(a, lds, e, pos0, mcount, tile, alone);
  }
}

// ------------------------------------------------------------------ down, resident rows
//
// The down GEMM over the packed stream when an item's activation rows fit LDS (K <= 1024:
// 32 rows x K halves <= 64 KB).  The block loads its item's h rows into LDS once, one 8 KB
// slot per stage in the same swizzled layout as the staged kernel, and then walks
// kDownTilesPerBlock consecutive 256-row tiles of the expert.  Those tiles are one contiguous
// run of the packed stream, so each wave streams its 1 KB runs and scale/zero pairs through
// a register ring kPkDepth stages deep across tile boundaries, with no barrier after the
// prologue.  A tile past the matrix end holds zero rows in the packed stream; they are
// computed and not stored.
#ifndef BD_DOWN_TILES_PER_BLOCK
#define BD_DOWN_TILES_PER_BLOCK 2
#endif
constexpr int kDownTilesPerBlock = BD_DOWN_TILES_PER_BLOCK;
constexpr int kResidentMaxStages = 8;

struct PkW {
  u32x4_t wa, wb, sz;
};

template <int NMT, bool AFF>
__device__ __forceinline__ void down_resident_item(const GemmArgs& a, char* lds, int e, int pos0,
                                                   int mcount, int tile0, int ntiles) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;
  const int kb = lane >> 4;
  const int G = a.K >> 6;
  const int NS = (G + 1) >> 1;
  const int F = ntiles * NS;                           // stages the block streams
  const DequantConsts dq = dequant_consts();
  const uint32_t run_bytes = (uint32_t)F * kPkStage;
  const __amdgpu_buffer_rsrc_t wrs =
      make_rsrc(a.pk + ((size_t)e * a.tiles + tile0) * (size_t)NS * kPkStage, run_bytes);
  const uint32_t wa_off = ((wave * 2 + 0) * 64 + lane) * 16;
  const uint32_t sz_off = kPkWBytes + (wave * 16 + n) * 16;
  auto load = [&](int f) {
    const uint32_t st = (uint32_t)min(f, F - 1) * kPkStage;
    PkW r;
    r.wa = bload<0>(wrs, wa_off, st);
    r.wb = bload<0>(wrs, wa_off + 1024, st);
    r.sz = bload<0>(wrs, sz_off, st);
    return r;
  };

  // Output slots of the lane's tokens (D rows 4kb..4kb+3 of each 16-token tile), loaded first
  // so that no later wait is for them.
  int slot[NMT][4];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = mt * 16 + kb * 4 + r;
      slot[mt][r] = perm_at(a, pos0 + min(m, mcount - 1));
      if (m >= mcount) slot[mt][r] = -1;
    }

  // Prologue: rows 0..16*NMT-1 of the item (rows past mcount repeat the last one), stage s
  // at slot s, 16-byte chunk ch of row m at (ch ^ xswz(m)).  Every thread issues the same
  // loads (chunks past K or stages past NS read clamped, in-bounds addresses and are not
  // written), then the first weight stages, then writes its rows to LDS.
  constexpr int kRows = NMT * 16;
  constexpr int kPer = kResidentMaxStages * kRows * 16 / kThreads;
  constexpr int kStep = kThreads / (kRows * 16);        // stages between a thread's chunks
  const int xm = (tid >> 4) % kRows;
  const int xch = tid & 15;
  const int xs0 = tid / (kRows * 16);
  const char* xsrc = reinterpret_cast<const char*>(a.act) +
                     (size_t)(pos0 + min(xm, mcount - 1)) * a.K * 2;
  u32x4_t xv[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int k0 = min((xs0 + i * kStep) * kStageK + xch * 8, a.K - 8);
    xv[i] = *reinterpret_cast<const u32x4_t*>(xsrc + (size_t)k0 * 2);
  }
  // The issue order is kept (rows, then stage 0, 1, ...) so that each wait below and in the
  // loop covers only the loads it needs.
  __builtin_amdgcn_sched_barrier(0);
  PkW buf[kPkDepth];
#pragma unroll
  for (int u = 0; u < kPkDepth; ++u) {
    buf[u] = load(u);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int st = xs0 + i * kStep;
    if (st < NS && st * kStageK + xch * 8 < a.K)
      *reinterpret_cast<u32x4_t*>(lds + st * kPkXSlot + xm * kXRowBytes + ((xch ^ xswz(xm)) << 4)) = xv[i];
  }
  lds_barrier();

  float4_t totA[NMT], totB[NMT];
  const float4_t zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) totA[mt] = totB[mt] = zero4;

  auto compute = [&](const PkW& r, int c) {
    const char* xt = lds + c * kPkXSlot;
    const half4_t szA = __builtin_bit_cast(half4_t, u32x2_t{r.sz[0], r.sz[1]});
    const half4_t szB = __builtin_bit_cast(half4_t, u32x2_t{r.sz[2], r.sz[3]});
    const ZeroPairs zpA = zero_pairs(szA), zpB = zero_pairs(szB);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (2 * c + j >= G) break;
      group_mfma<NMT, AFF>(r.wa, r.wb, szA, szB, zpA, zpB, j, xt, n, kb, totA, totB, dq);
    }
  };
  auto store = [&](int tile) {
    const int row = tile * kPkRows + wave * 32 + n;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (slot[mt][r] < 0) continue;
        float* o = a.o_out + (size_t)slot[mt][r] * a.out_ld;
        if (row < a.R) o[row] = totA[mt][r];
        if (row + 16 < a.R) o[row + 16] = totB[mt][r];
      }
      totA[mt] = totB[mt] = zero4;
    }
  };

  // Rounds of kPkDepth stages; stage f of the run sits in buf[f % kPkDepth] and the load
  // that refills it (stage f + kPkDepth, clamped to the run) is issued right after its use.
  // A finished tile is stored before that load, so the waits for later stages never cover
  // the stores.
  int c = 0, tile = tile0;
  for (int f0 = 0; f0 < F; f0 += kPkDepth) {
#pragma unroll
    for (int u = 0; u < kPkDepth; ++u) {
      const bool live = f0 + u < F;
      if (live) compute(buf[u], c);
      if (live && ++c == NS) {
        store(tile);
        c = 0;
        ++tile;
      }
      buf[u] = load(f0 + u + kPkDepth);
    }
  }
}

template <bool AFF>
__global__ __launch_bounds__(kThreads, 2) void w4a16_down_resident_kernel(GemmArgs a) {
  if (gated_off(a.gate)) return;
  extern __shared__ __attribute__((aligned(16))) char lds_dyn[];
  // Same XCD-aware order as the staged kernel, over (item, group of tiles).
  const int b = blockIdx.x;
  const int groups = (a.tiles + kDownTilesPerBlock - 1) / kDownTilesPerBlock;
  const int n_items = item_count(a);
  const int per = (n_items + kXcds - 1) / kXcds;
  const int local = b / kXcds;
  const int grp = local / per;
  const int item = (b % kXcds) * per + local % per;
  if (grp >= groups || item >= n_items) return;
  const Item it = load_item(a, item);
  const int e = it.e, pos0 = it.pos0, mcount = it.mcount;
  const int tile0 = grp * kDownTilesPerBlock;
  const int ntiles = min(kDownTilesPerBlock, a.tiles - tile0);
  if (mcount > 16)
    down_resident_item<2, AFF>(a, lds_dyn, e, pos0, mcount, tile0, ntiles);
  else
    down_resident_item<1, AFF>(a, lds_dyn, e, pos0, mcount, tile0, ntiles);
}

// Stage counts with a fully unrolled kernel: the contraction dims 2816 (gate/up) and 704
// (down) of the 26B-A4B expert shape.
template <bool GATED, bool AFF>
void launch_packed_as(const GemmArgs& a, int max_items, hipStream_t stream) {
  const int NS = (a.K / 64 + 1) / 2;
  if (!GATED && NS <= kResidentMaxStages) {
    const int groups = (a.tiles + kDownTilesPerBlock - 1) / kDownTilesPerBlock;
    hipLaunchKernelGGL(w4a16_down_resident_kernel<AFF>, dim3(grid_blocks(max_items, groups)),
                       dim3(kThreads), NS * kPkXSlot, stream, a);
    return;
  }
  const dim3 grid(grid_blocks(max_items, a.tiles)), block(kThreads);
  if (NS == 22)
    hipLaunchKernelGGL((w4a16_packed_kernel<GATED, 22, AFF>), grid, block, 0, stream, a);
  else if (NS == 6)
    hipLaunchKernelGGL((w4a16_packed_kernel<GATED, 6, AFF>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((w4a16_packed_kernel<GATED, 0, AFF>), grid, block, 0, stream, a);
}

// The weight form of the packed stream picks the kernels' dequantisation.
template <bool GATED>
void launch_packed(const GemmArgs& a, int max_items, hipStream_t stream) {
  if (a.affine)
    launch_packed_as<GATED, true>(a, max_items, stream);
  else
    launch_packed_as<GATED, false>(a, max_items, stream);
}

// Repacking into the packed stream (layout above).  One thread per 16-byte chunk of the output;
// rows past the matrix and the group past an odd G are written as zeros.  With source groups of
// 128 (gshift 1) each 64-group slot takes the scale and zero-point of the 128-group holding it.
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ q,
                                                   const uint16_t* __restrict__ scale,
                                                   const uint16_t* __restrict__ zero, int R, int K,
                                                   int tiles, int gated, int d_ff, int gshift,
                                                   int compact, size_t chunks,
                                                   u32x4_t* __restrict__ out) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= chunks) return;
  const int G = K / 64, NS = (G + 1) / 2;
  const int stage_chunks = compact ? kPkChunksC : kPkChunks;
  const int ch = (int)(i % stage_chunks);
  const size_t qs = i / stage_chunks;
  const int s = (int)(qs % NS);
  const int tile = (int)((qs / NS) % tiles);
  const size_t e = qs / ((size_t)NS * tiles);
  // matrix row of tile row tr, or -1 past the matrix
  auto mrow = [&](int tr) -> int {
    if (gated) {
      const int col = tile * 128 + (tr & 127);
      return col < d_ff ? (tr < 128 ? 0 : d_ff) + col : -1;
    }
    const int row = tile * kPkRows + tr;
    return row < R ? row : -1;
  };
  auto tile_row = [&](int w, int set, int nn) {
    return gated ? (set ? 128 : 0) + w * 16 + nn : w * 32 + set * 16 + nn;
  };
  const int g0 = 2 * s, g1 = 2 * s + 1;
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (ch < kPkWBytes / 16) {
    const int w = ch / 128, set = (ch / 64) & 1, l = ch & 63;
    const int row = mrow(tile_row(w, set, l & 15));
    const int kbl = l >> 4;
    if (row >= 0) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(q + ((size_t)e * R + row) * (K / 2));
      v[0] = src[(g0 * 32 + kbl * 8) / 4];
      v[1] = src[(g0 * 32 + kbl * 8) / 4 + 1];
      if (g1 < G) {
        v[2] = src[(g1 * 32 + kbl * 8) / 4];
        v[3] = src[(g1 * 32 + kbl * 8) / 4 + 1];
      }
    }
  } else if (compact) {
    // One group of 128 per stage (group s): chunk idx holds, for (w, n) = 2 idx and
    // 2 idx + 1 in turn, scale | zero << 16 of tile row R(w, 0, n), then of R(w, 1, n).
    const int idx = ch - kPkWBytes / 16;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int wn = 2 * idx + h;
      const int w = wn / 16, nn = wn & 15;
#pragma unroll
      for (int set = 0; set < 2; ++set) {
        const int row = mrow(tile_row(w, set, nn));
        if (row < 0) continue;
        const size_t at = ((size_t)e * R + row) * (G >> 1) + s;
        v[2 * h + set] = (uint32_t)scale[at] | ((uint32_t)zero[at] << 16);
      }
    }
  } else {
    const int idx = ch - kPkWBytes / 16;
    const int w = idx / 16, nn = idx & 15;
#pragma unroll
    for (int set = 0; set < 2; ++set) {
      const int row = mrow(tile_row(w, set, nn));
      if (row < 0) continue;
      const size_t base = ((size_t)e * R + row) * (G >> gshift);
      const uint32_t s0 = scale[base + (g0 >> gshift)], z0 = zero[base + (g0 >> gshift)];
      const uint32_t s1 = g1 < G ? scale[base + (g1 >> gshift)] : 0u;
      const uint32_t z1 = g1 < G ? zero[base + (g1 >> gshift)] : 0u;
      v[2 * set] = s0 | (s1 << 16);
      v[2 * set + 1] = z0 | (z1 << 16);
    }
  }
  out[i] = v;
}


}  // namespace

bool pk_compact(bool gated, int group) { return gated && group == 128; }

int pk_tiles(bool gated, int d_model, int d_ff) {
  return gated ? (d_ff + 127) / 128 : (d_model + kPkRows - 1) / kPkRows;
}

size_t pk_bytes(bool gated, int E, int d_model, int d_ff, bool compact) {
  const int K = gated ? d_model : d_ff;
  const int NS = (K / 64 + 1) / 2;
  return (size_t)E * pk_tiles(gated, d_model, d_ff) * NS * (compact ? kPkStageC : kPkStage);
}

hipError_t launch_pack(const W4A16Matrix& m, bool gated, int E, int d_model, int d_ff,
                       uint8_t* out, hipStream_t stream) {
  const int K = gated ? d_model : d_ff;
  const int R = gated ? 2 * d_ff : d_model;
  const bool compact = pk_compact(gated, m.group);
  const size_t chunks = pk_bytes(gated, E, d_model, d_ff, compact) / 16;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream,
                     m.q, m.scale, m.zero, R, K, pk_tiles(gated, d_model, d_ff), gated ? 1 : 0,
                     d_ff, m.group == 128 ? 1 : 0, compact ? 1 : 0, chunks,
                     reinterpret_cast<u32x4_t*>(out));
  return hipGetLastError();
}

hipError_t launch_gate_up(const W4A16Matrix& gu, int E, int d_model, int d_ff, int top_k, int T,
                          const uint16_t* x, const MoeWorkspace& ws, hipStream_t stream,
                          const int32_t* gate) {
  GemmArgs a;
  a.q = gu.q;
  a.scale = gu.scale;
  a.zero = gu.zero;
  a.K = d_model;
  a.R = 2 * d_ff;
  a.d_ff = d_ff;
  a.top_k = top_k;
  a.tiles = d_ff / 64;
  a.act = x;
  a.perm = ws.perm;
  a.items = ws.items;
  a.pk = gu.pk;
  a.affine = gu.affine;
  a.sz_compact = gu.pk != nullptr && pk_compact(true, gu.group) ? 1 : 0;
  a.h_out = ws.h;
  a.o_out = nullptr;
  a.out_ld = d_ff;
  a.E = E;
  a.A = T * top_k;
  a.max_items = ws.max_items;
  a.gate = gate;
  // The expert buckets and the work list are in ws from the routing launch.  The packed
  // kernel reorders x in registers; the tile kernel needs a reordered copy first.
  if (gu.pk) {
    a.tiles = pk_tiles(true, d_model, d_ff);
    launch_packed<true>(a, ws.max_items, stream);
  } else {
    hipError_t err = launch_permute(T, x, d_model, ws, stream, gate);
    if (err != hipSuccess) return err;
    a.act = ws.xp;
    hipLaunchKernelGGL(w4a16_gemm_kernel<true>, dim3(grid_blocks(ws.max_items, a.tiles)),
                       dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_down(const W4A16Matrix& dn, int E, int d_model, int d_ff, int top_k, int T,
                       float* expert_out, const MoeWorkspace& ws, hipStream_t stream,
                       const int32_t* gate) {
  GemmArgs a;
  a.q = dn.q;
  a.scale = dn.scale;
  a.zero = dn.zero;
  a.K = d_ff;
  a.R = d_model;
  a.d_ff = d_ff;
  a.top_k = top_k;
  a.tiles = d_model / kRowsPerBlock;
  a.act = ws.h;
  a.perm = ws.perm;
  a.items = ws.items;
  a.pk = dn.pk;
  a.affine = dn.affine;
  a.sz_compact = 0;
  a.h_out = nullptr;
  a.o_out = expert_out;
  a.out_ld = d_model;
  a.E = E;
  a.A = T * top_k;
  a.max_items = ws.max_items;
  a.gate = gate;
  if (dn.pk) {
    a.tiles = pk_tiles(false, d_model, d_ff);
    launch_packed<false>(a, ws.max_items, stream);
  } else {
    hipLaunchKernelGGL(w4a16_gemm_kernel<false>, dim3(grid_blocks(ws.max_items, a.tiles)),
                       dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace bd
