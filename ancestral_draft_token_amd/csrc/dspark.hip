// dspark.hip -- DSpark ancestral draft-block sampler for MI355X (gfx950).
//
// The method ("brb-nv/TensorRT-LLM pull 21", section "2. Golden sampling
// semantics"; "brb-nv/TensorRT-LLM pull 27", section "2. One fused kernel per
// draft position"): each position k of a draft block samples d_k, by
// Gumbel-max, from the softmax of (base_k + E[d_{k-1}] . W) * (1/T), with
// E[d] . W a rank-r Markov head evaluated at the previous position's sample;
// after the block the proposal q_k = softmax(logits_k / T) is written from the
// same float32 logits the samples were taken from.
//
// Kernels, all on one stream (capturable into one hipGraph):
//   markov_bias_gumbel_argmax (once per position): streams W and the base
//     logits for one vocabulary chunk, forms the float32 biased logits, scales
//     by 1/T, adds Philox Gumbel noise, and leaves per-chunk softmax statistics
//     and a per-chunk (score, index) argmax partial.
//   pick_and_gather (once per position, B > 1): reduces each row's partials
//     in a fixed order, writes d_k and the row's (max, sum-exp), and gathers
//     E[d_k] for the next position.
//   proposal_softmax (once per block): q = exp(s - M) / S over all rows and
//     positions.
// At B = 1 there is no pick launch: every workgroup of position k reduces the
// (few, L2-resident) partials of position k-1 itself while its W loads are in
// flight, and the proposal kernel reduces the last position's partials.
//
// Exact arithmetic conventions are stated in include/dspark.h. This file is
// compiled with FMA contraction off; the bias products use an explicit fmaf.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "dspark.h"

namespace dspark {

constexpr int kThreads = 256;        // every kernel runs 256-thread workgroups (4 wave64)
constexpr int kWaves = kThreads / 64;
constexpr int kTile = 128;           // vocabulary columns per tile of the fused kernel
constexpr int kSlices = 16;          // rank slices of the VALU bias GEMV
constexpr int kRowsPerSlice = 16;    // contiguous rank rows per slice and pass (16 x 16 = 256)
constexpr int kMaxRank = 1024;
constexpr int kMaxK = 255;
constexpr int kDefaultChunk = kTile; // one tile per workgroup: 1563 workgroups at V = 200064
constexpr int kPickPerThread = 8;    // in-kernel pick: at most 8 x 256 = 2048 partials per row

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
// as 1, 2, 3", SC'11, section 3): ten rounds of the 4x32 bijection; the key is
// bumped by the Weyl increments between rounds.
// ---------------------------------------------------------------------------
// One Philox4x32 round: the two products as full 64-bit results (one
// v_mad_u64_u32 each instead of a mul_lo/mul_hi pair) and the three-input
// exclusive or as one v_bitop3_b32 (truth table 0x96).
__device__ __forceinline__ uint4 philox_round(uint4 c, uint32_t k0, uint32_t k1) {
  const uint64_t pa = (uint64_t)0xD2511F53u * (uint64_t)c.x;
  const uint64_t pb = (uint64_t)0xCD9E8D57u * (uint64_t)c.z;
  return make_uint4(__builtin_amdgcn_bitop3_b32((uint32_t)(pb >> 32), c.y, k0, 0x96), (uint32_t)pb,
                    __builtin_amdgcn_bitop3_b32((uint32_t)(pa >> 32), c.w, k1, 0x96), (uint32_t)pa);
}

// A hook with nothing to do (see philox4x32_10_hooked).
struct NoHook {
  template <int J>
  __device__ __forceinline__ void step() {}
};

// Philox4x32-10 with hook.step<J>() after rounds 2J + 1 (J = 0..4): a place to
// issue unrelated work between the rounds (the large-batch kernel issues its
// next matrix chain there). The step index is a template argument so that
// whatever it indexes stays in registers.
template <class Hook>
__device__ __forceinline__ uint4 philox4x32_10_hooked(uint4 c, uint32_t k0, uint32_t k1, Hook& hook) {
  constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  c = philox_round(c, k0, k1);
  c = philox_round(c, k0 + W0, k1 + W1);
  hook.template step<0>();
  c = philox_round(c, k0 + 2 * W0, k1 + 2 * W1);
  c = philox_round(c, k0 + 3 * W0, k1 + 3 * W1);
  hook.template step<1>();
  c = philox_round(c, k0 + 4 * W0, k1 + 4 * W1);
  c = philox_round(c, k0 + 5 * W0, k1 + 5 * W1);
  hook.template step<2>();
  c = philox_round(c, k0 + 6 * W0, k1 + 6 * W1);
  c = philox_round(c, k0 + 7 * W0, k1 + 7 * W1);
  hook.template step<3>();
  c = philox_round(c, k0 + 8 * W0, k1 + 8 * W1);
  c = philox_round(c, k0 + 9 * W0, k1 + 9 * W1);
  hook.template step<4>();
  return c;
}

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
  NoHook none;
  return philox4x32_10_hooked(c, k0, k1, none);
}

// Standard Gumbel variate from the top 23 bits of a Philox word:
// u = ((x >> 9) + 1/2) 2^-23 is exact in float32; g = -ln(-ln u), evaluated
// with the hardware base-2 logarithm as -ln2 * (log2(-log2 u) + log2(ln 2)).
// Over all 2^23 values of u this is within 2.0e-6 of -ln(-ln u) in double.
__device__ __forceinline__ float gumbel_from_bits(uint32_t x) {
  const float u = __fmul_rn(__fadd_rn((float)(x >> 9), 0.5f), 0x1p-23f);
  const float e2 = -__builtin_amdgcn_logf(u);                 // -log2(u) > 0
  return -0.693147182f * (__builtin_amdgcn_logf(e2) + -0.528766364f);
}

// Total-order key of a score: larger key = better; NaN is the smallest key;
// equal scores prefer the lower vocabulary index (the low word holds ~v).
__device__ __forceinline__ uint64_t score_key(float z, uint32_t v) {
  if (z == 0.0f) z = 0.0f;  // -0 and +0 compare equal, so they key equal
  const uint32_t bits = __float_as_uint(z);
  uint32_t ord = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
  if (z != z) ord = 0u;
  return ((uint64_t)ord << 32) | (uint64_t)(~v);
}

__device__ __forceinline__ uint32_t key_token(uint64_t key) { return ~(uint32_t)key; }

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Running softmax statistics (m, l): l = sum exp(s - m).
struct Stat {
  float m;
  float l;
};

// Branch-free: an empty side (m = -inf) contributes exp(-inf) = 0.
__device__ __forceinline__ Stat stat_merge(Stat a, Stat b) {
  const float m = fmaxf(a.m, b.m);
  const float da = (a.m == -INFINITY) ? -INFINITY : __fsub_rn(a.m, m);
  const float db = (b.m == -INFINITY) ? -INFINITY : __fsub_rn(b.m, m);
  const float la = __fmul_rn(a.l, __expf(da));
  const float lb = __fmul_rn(b.l, __expf(db));
  return Stat{m, __fadd_rn(la, lb)};
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int mask, int width) {
  const uint32_t lo = __shfl_xor((uint32_t)x, mask, width);
  const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), mask, width);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Reduce (key, stat) over `width` consecutive lanes (a power of two <= 64).
__device__ __forceinline__ void reduce_lanes(uint64_t& key, Stat& st, int width) {
  for (int mask = 1; mask < width; mask <<= 1) {
    key = umax64(key, shfl_xor_u64(key, mask, width));
    Stat o;
    o.m = __shfl_xor(st.m, mask, width);
    o.l = __shfl_xor(st.l, mask, width);
    st = stat_merge(st, o);
  }
}

// Merge of (key, statistics) partials over the four 16-lane rows of a wave
// (lane l with l ^ 16, then with l ^ 32), with the gfx950 lane-swap
// instructions instead of LDS-routed shuffles. Swapping a register with itself
// hands every lane the pair {lower row's value, upper row's value} in that
// order, so all lanes of a pair compute the same merge (max and stat_merge are
// symmetric in any case).
__device__ __forceinline__ void row_merge4(uint64_t& key, Stat& st) {
#define DSPARK_SWAP_MERGE(swap)                                                                   \
  {                                                                                              \
    const auto lo = swap((uint32_t)key, (uint32_t)key, false, false);                            \
    const auto hi = swap((uint32_t)(key >> 32), (uint32_t)(key >> 32), false, false);            \
    const auto mm = swap(__float_as_uint(st.m), __float_as_uint(st.m), false, false);            \
    const auto ll = swap(__float_as_uint(st.l), __float_as_uint(st.l), false, false);            \
    key = umax64(((uint64_t)hi[0] << 32) | lo[0], ((uint64_t)hi[1] << 32) | lo[1]);               \
    st = stat_merge(Stat{__uint_as_float(mm[0]), __uint_as_float(ll[0])},                         \
                    Stat{__uint_as_float(mm[1]), __uint_as_float(ll[1])});                        \
  }
  DSPARK_SWAP_MERGE(__builtin_amdgcn_permlane16_swap)
  DSPARK_SWAP_MERGE(__builtin_amdgcn_permlane32_swap)
#undef DSPARK_SWAP_MERGE
}

// Maximum of a 64-bit value over the 64 lanes of a wave, every lane getting
// it, without LDS: DPP within quads (xor 1, xor 2), then the half-row and row
// mirrors (which pair quad 0 with quad 1 and half 0 with half 1), then the
// lane swaps across 16-lane rows.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#define DSPARK_DPP_MAX(ctrl)                                                                           \
  {                                                                                                    \
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, ctrl, 0xF, 0xF, false); \
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), ctrl, 0xF, 0xF, false); \
    x = umax64(x, ((uint64_t)hi << 32) | lo);                                                          \
  }
  DSPARK_DPP_MAX(0xB1)    // quad_perm(1,0,3,2): lane ^ 1
  DSPARK_DPP_MAX(0x4E)    // quad_perm(2,3,0,1): lane ^ 2
  DSPARK_DPP_MAX(0x141)   // row_half_mirror
  DSPARK_DPP_MAX(0x140)   // row_mirror
#undef DSPARK_DPP_MAX
#define DSPARK_SWAP_MAX(swap)                                                                  \
  {                                                                                            \
    const auto lo = swap((uint32_t)x, (uint32_t)x, false, false);                              \
    const auto hi = swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);              \
    x = umax64(((uint64_t)hi[0] << 32) | lo[0], ((uint64_t)hi[1] << 32) | lo[1]);               \
  }
  DSPARK_SWAP_MAX(__builtin_amdgcn_permlane16_swap)
  DSPARK_SWAP_MAX(__builtin_amdgcn_permlane32_swap)
#undef DSPARK_SWAP_MAX
  return x;
}

// Merge of (key, statistics) over the 64 lanes of a wave, every lane getting
// the result: DPP within 16-lane rows (lane ^ 1, lane ^ 2, then the half-row
// and row mirrors, which pair the quads and the halves of a row), then the
// lane swaps across rows. Each step merges two partials of the same shape, and
// max and stat_merge are symmetric, so every lane computes the same merge.
__device__ __forceinline__ void wave_merge_key_stat(uint64_t& key, Stat& st) {
#define DSPARK_DPP_MERGE(ctrl)                                                                            \
  {                                                                                                       \
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)key, ctrl, 0xF, 0xF, false); \
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(key >> 32), ctrl, 0xF, 0xF, false); \
    const int om = __builtin_amdgcn_update_dpp(0, __float_as_int(st.m), ctrl, 0xF, 0xF, false);          \
    const int ol = __builtin_amdgcn_update_dpp(0, __float_as_int(st.l), ctrl, 0xF, 0xF, false);          \
    key = umax64(key, ((uint64_t)hi << 32) | lo);                                                         \
    st = stat_merge(st, Stat{__int_as_float(om), __int_as_float(ol)});                                    \
  }
  DSPARK_DPP_MERGE(0xB1)    // quad_perm(1,0,3,2): lane ^ 1
  DSPARK_DPP_MERGE(0x4E)    // quad_perm(2,3,0,1): lane ^ 2
  DSPARK_DPP_MERGE(0x141)   // row_half_mirror
  DSPARK_DPP_MERGE(0x140)   // row_mirror
#undef DSPARK_DPP_MERGE
  row_merge4(key, st);
}

// The statistics half of wave_merge_key_stat: the same steps in the same
// order, so the merged (m, l) are bit for bit those it gives.
__device__ __forceinline__ void wave_merge_stat(Stat& st) {
#define DSPARK_DPP_MERGE_STAT(ctrl)                                                              \
  {                                                                                              \
    const int om = __builtin_amdgcn_update_dpp(0, __float_as_int(st.m), ctrl, 0xF, 0xF, false); \
    const int ol = __builtin_amdgcn_update_dpp(0, __float_as_int(st.l), ctrl, 0xF, 0xF, false); \
    st = stat_merge(st, Stat{__int_as_float(om), __int_as_float(ol)});                           \
  }
  DSPARK_DPP_MERGE_STAT(0xB1)    // quad_perm(1,0,3,2): lane ^ 1
  DSPARK_DPP_MERGE_STAT(0x4E)    // quad_perm(2,3,0,1): lane ^ 2
  DSPARK_DPP_MERGE_STAT(0x141)   // row_half_mirror
  DSPARK_DPP_MERGE_STAT(0x140)   // row_mirror
#undef DSPARK_DPP_MERGE_STAT
#define DSPARK_SWAP_MERGE_STAT(swap)                                                      \
  {                                                                                      \
    const auto mm = swap(__float_as_uint(st.m), __float_as_uint(st.m), false, false);    \
    const auto ll = swap(__float_as_uint(st.l), __float_as_uint(st.l), false, false);    \
    st = stat_merge(Stat{__uint_as_float(mm[0]), __uint_as_float(ll[0])},                 \
                    Stat{__uint_as_float(mm[1]), __uint_as_float(ll[1])});                \
  }
  DSPARK_SWAP_MERGE_STAT(__builtin_amdgcn_permlane16_swap)
  DSPARK_SWAP_MERGE_STAT(__builtin_amdgcn_permlane32_swap)
#undef DSPARK_SWAP_MERGE_STAT
}

// Maximum of a 64-bit value over the lanes of a wave with equal lane % RB
// (RB = 1, 2 or 4), every lane getting its class's maximum: rotations within
// 16-lane rows by RB, 2 RB, ... (which keep the class), then the lane swaps
// across rows.
template <int RB>
__device__ __forceinline__ uint64_t wave_max_u64_class(uint64_t x) {
  if constexpr (RB == 1) {
    return wave_max_u64(x);
  } else {
#define DSPARK_ROR_MAX(n)                                                                                    \
  {                                                                                                          \
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, 0x120 + (n), 0xF, 0xF, false); \
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), 0x120 + (n), 0xF, 0xF, false); \
    x = umax64(x, ((uint64_t)hi << 32) | lo);                                                                \
  }
    if constexpr (RB <= 2) DSPARK_ROR_MAX(2)   // row_ror:2
    DSPARK_ROR_MAX(4)                           // row_ror:4
    DSPARK_ROR_MAX(8)                           // row_ror:8
#undef DSPARK_ROR_MAX
    const auto l16 = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
    const auto h16 = __builtin_amdgcn_permlane16_swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);
    x = umax64(((uint64_t)h16[0] << 32) | l16[0], ((uint64_t)h16[1] << 32) | l16[1]);
    const auto l32 = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
    const auto h32 = __builtin_amdgcn_permlane32_swap((uint32_t)(x >> 32), (uint32_t)(x >> 32), false, false);
    x = umax64(((uint64_t)h32[0] << 32) | l32[0], ((uint64_t)h32[1] << 32) | l32[1]);
    return x;
  }
}

__device__ __forceinline__ int clamp_token(int d, int V) { return d < 0 ? 0 : (d > V - 1 ? V - 1 : d); }

struct StepArgs {
  const void* base;          // [B,K,V]
  const uint16_t* E;         // [V,r]
  const uint16_t* W;         // [r,V]
  const int32_t* prev_token; // [B], d_{-1}
  const uint16_t* e_buf;     // [B,r] bf16: E[d_{k-1}] gathered by pick_and_gather (k > 0, B > 1)
  const uint64_t* prev_key;  // [B,C] partials of position k-1 (in-kernel pick, B == 1)
  const Stat* prev_stat;     // [B,C]
  const int64_t* seed;
  const int64_t* offset;
  const float* temperature;
  const int32_t* n_real;     // may be null
  float* logits;             // [B,K,V]
  int32_t* tokens;           // [B,K]
  Stat* row_stat;            // [B,K]
  uint64_t* part_key;        // [B,C] partials of position k
  Stat* part_stat;           // [B,C]
  int B, K, V, r, k;
  int chunk_cols, n_chunks;
};

// Per-row sampling state of the epilogue.
struct RowState {
  float invT;
  bool greedy;
  bool pad;
  uint32_t key0, key1, ctr2, ctr3;
};

// A row's sampling state from its temperature, Philox key (seed) and slot
// offset; row b is padding when b >= n_real.
__device__ __forceinline__ RowState row_state_of(float T, int64_t seed, int64_t offset, int b, int n_real) {
  RowState rs;
  rs.greedy = !(T > 0.0f);
  rs.invT = rs.greedy ? 0.0f : __fdiv_rn(1.0f, T);
  rs.pad = b >= n_real;
  const uint64_t sd = (uint64_t)seed;
  const uint64_t of = (uint64_t)offset;
  rs.key0 = (uint32_t)sd;
  rs.key1 = (uint32_t)(sd >> 32);
  rs.ctr2 = (uint32_t)of;
  rs.ctr3 = (uint32_t)(of >> 32);
  return rs;
}

__device__ __forceinline__ RowState row_state(const float* temperature, const int64_t* seed,
                                              const int64_t* offset, int b, int n_real) {
  return row_state_of(temperature[b], seed[b], offset[b], b, n_real);
}

__device__ __forceinline__ RowState row_state(const StepArgs& a, int b, int n_real) {
  return row_state(a.temperature, a.seed, a.offset, b, n_real);
}

// Base logits of 4 consecutive columns, loaded early and widened late.
template <bool kBf16Base>
struct Base4 {
  uint2 h;
  float4 f;
};

// Nontemporal (kNt): base logits are read once, and not letting them displace
// the just-written logits in the Infinity Cache lets the proposal pass re-read
// more of those from the cache instead of HBM. Only where one load instruction
// covers whole cache lines: a nontemporal read of part of a line does not keep
// the line for its other parts, which are then fetched again (the large-batch
// kernel reads 64 or 32 bytes of a 128-byte line per tile, so it loads
// without the hint: B=88 fetch 734 -> 634 MB, B=44 333 -> 252 MB).
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4v_t __attribute__((ext_vector_type(4)));

template <bool kBf16Base, bool kNt = true>
__device__ __forceinline__ void load_base4(Base4<kBf16Base>& bv, const void* base, size_t off) {
  if (kBf16Base) {
    const u32x2_t* p = reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(base) + off);
    const u32x2_t x = kNt ? __builtin_nontemporal_load(p) : *p;
    bv.h = make_uint2(x.x, x.y);
  } else {
    const f32x4v_t* p = reinterpret_cast<const f32x4v_t*>(static_cast<const float*>(base) + off);
    const f32x4v_t x = kNt ? __builtin_nontemporal_load(p) : *p;
    bv.f = make_float4(x.x, x.y, x.z, x.w);
  }
}

// The base logits of N = 1 or 2 consecutive columns (N = 2: off even): their
// bf16 in h.x, or their floats in f.x, f.y.
template <bool kBf16Base, int N>
__device__ __forceinline__ void load_base_n(Base4<kBf16Base>& bv, const void* base, size_t off) {
  static_assert(N == 1 || N == 2, "columns");
  if (kBf16Base) {
    if constexpr (N == 1) bv.h.x = (uint32_t)__builtin_nontemporal_load(static_cast<const uint16_t*>(base) + off);
    else bv.h.x = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(base) + off));
  } else {
    if constexpr (N == 1) {
      bv.f.x = __builtin_nontemporal_load(static_cast<const float*>(base) + off);
    } else {
      const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(static_cast<const float*>(base) + off));
      bv.f.x = __uint_as_float(x.x);
      bv.f.y = __uint_as_float(x.y);
    }
  }
}

template <bool kBf16Base, int N>
__device__ __forceinline__ void widen_base_n(const Base4<kBf16Base>& bv, float out[N]) {
  if (kBf16Base) {
    out[0] = bf16_lo(bv.h.x);
    if constexpr (N == 2) out[1] = bf16_hi(bv.h.x);
  } else {
    out[0] = bv.f.x;
    if constexpr (N == 2) out[1] = bv.f.y;
  }
}

template <bool kBf16Base>
__device__ __forceinline__ void widen_base4(const Base4<kBf16Base>& bv, float out[4]) {
  if (kBf16Base) {
    out[0] = bf16_lo(bv.h.x); out[1] = bf16_hi(bv.h.x);
    out[2] = bf16_lo(bv.h.y); out[3] = bf16_hi(bv.h.y);
  } else {
    out[0] = bv.f.x; out[1] = bv.f.y; out[2] = bv.f.z; out[3] = bv.f.w;
  }
}

// The epilogue of 4 consecutive columns v0..v0+3 of one row: float32 logits,
// 1/T, Gumbel noise, and the running argmax key and softmax statistics.
__device__ __forceinline__ void epilogue4(const RowState& rs, int k, uint32_t v0, const float base[4],
                                          const float bias[4], float* logits_out, uint64_t& best,
                                          Stat& st) {
  float lg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lg[i] = __fadd_rn(base[i], bias[i]);
  *reinterpret_cast<float4*>(logits_out) = make_float4(lg[0], lg[1], lg[2], lg[3]);
  if (rs.greedy) {
#pragma unroll
    for (int i = 0; i < 4; ++i) best = umax64(best, score_key(lg[i], v0 + i));
    return;
  }
  const uint4 x = philox4x32_10(make_uint4(v0 >> 2, (uint32_t)k, rs.ctr2, rs.ctr3), rs.key0, rs.key1);
  const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
  float s[4];
  float m4 = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s[i] = __fmul_rn(lg[i], rs.invT);
    const float z = __fadd_rn(s[i], gumbel_from_bits(xs[i]));
    best = umax64(best, score_key(z, v0 + i));
    m4 = fmaxf(m4, s[i]);
  }
  float l4 = 0.0f;
  if (m4 != -INFINITY) {
#pragma unroll
    for (int i = 0; i < 4; ++i) l4 = __fadd_rn(l4, __expf(__fsub_rn(s[i], m4)));
  }
  st = stat_merge(st, Stat{m4, l4});
}

// Finish a workgroup-wide reduction of (key, stat) in a fixed order: lanes,
// then waves in index order. Every thread returns the result.
__device__ __forceinline__ void wg_reduce(uint64_t& key, Stat& st, uint64_t* s_key, Stat* s_stat) {
  reduce_lanes(key, st, 64);
  const int t = threadIdx.x;
  if ((t & 63) == 0) {
    s_key[t >> 6] = key;
    s_stat[t >> 6] = st;
  }
  __syncthreads();
  key = s_key[0];
  st = s_stat[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) {
    key = umax64(key, s_key[w]);
    st = stat_merge(st, s_stat[w]);
  }
}

// One pass of the VALU GEMV: acc[rr][c] += sum over this thread's 16 rank
// rows of e_rr[j] * W[j, col + c].
template <int RB>
__device__ __forceinline__ void gemv_pass(const uint4 (&wv)[kRowsPerSlice], const uint4 (&ev)[RB][2],
                                          float (&acc)[RB][8]) {
#pragma unroll
  for (int i = 0; i < kRowsPerSlice; ++i) {
    const uint4 w = wv[i];
    const float wf[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                         bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const uint4 eh = ev[rr][i / 8];
      const uint32_t pair = (i % 8) < 2 ? eh.x : (i % 8) < 4 ? eh.y : (i % 8) < 6 ? eh.z : eh.w;
      const float e = (i % 2) ? bf16_hi(pair) : bf16_lo(pair);
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[rr][c] = fmaf(e, wf[c], acc[rr][c]);
    }
  }
}

// Sum the 16 rank slices of column ec..ec+3 of row er in a fixed order.
template <int RB>
__device__ __forceinline__ void slice_sum(const float (&red)[kSlices][RB][kTile], int er, int ec,
                                          float bias[4]) {
  bias[0] = bias[1] = bias[2] = bias[3] = 0.0f;
#pragma unroll
  for (int q = 0; q < kSlices; ++q) {
    const float4 pq = *reinterpret_cast<const float4*>(&red[q][er][ec]);
    bias[0] = __fadd_rn(bias[0], pq.x);
    bias[1] = __fadd_rn(bias[1], pq.y);
    bias[2] = __fadd_rn(bias[2], pq.z);
    bias[3] = __fadd_rn(bias[3], pq.w);
  }
}

template <int RB>
__device__ __forceinline__ void store_slices(float (&red)[kSlices][RB][kTile], int js, int cg,
                                             const float (&acc)[RB][8]) {
#pragma unroll
  for (int rr = 0; rr < RB; ++rr) {
    *reinterpret_cast<float4*>(&red[js][rr][cg * 8]) =
        make_float4(acc[rr][0], acc[rr][1], acc[rr][2], acc[rr][3]);
    *reinterpret_cast<float4*>(&red[js][rr][cg * 8 + 4]) =
        make_float4(acc[rr][4], acc[rr][5], acc[rr][6], acc[rr][7]);
  }
}

template <int RB>
__device__ __forceinline__ void load_e(const uint16_t* const (&erow)[RB], const uint16_t* any_row,
                                       int j0, bool j_ok, uint4 (&ev)[RB][2]) {
#pragma unroll
  for (int rr = 0; rr < RB; ++rr) {
    // unconditional loads from a valid address; rows that do not exist read zeros
    const bool ok = j_ok && erow[rr] != nullptr;
    const uint16_t* src = ok ? erow[rr] + j0 : any_row;
    const uint4 lo = *reinterpret_cast<const uint4*>(src);
    const uint4 hi = *reinterpret_cast<const uint4*>(src + 8);
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    ev[rr][0] = ok ? lo : z;
    ev[rr][1] = ok ? hi : z;
  }
}

// The 16 W loads (16 bytes each) of one thread for one (tile, pass): rank rows
// j0..j0+15 at columns col..col+7. An out-of-range slice loads a valid
// address instead (straight-line code, no wait to overwrite a pending load);
// its values are never used: absent rank slices skip their FMAs and absent
// columns are never stored.
__device__ __forceinline__ void issue_w(const uint16_t* W, int V, bool ok, int j0, int col,
                                        uint4 (&wv)[kRowsPerSlice]) {
  const uint16_t* src = W + (ok ? (size_t)j0 * V + col : 0);
  const size_t stride = ok ? (size_t)V : 0;
#pragma unroll
  for (int i = 0; i < kRowsPerSlice; ++i) wv[i] = *reinterpret_cast<const uint4*>(src + i * stride);
}

// ---------------------------------------------------------------------------
// Kernel 1, small B (RB = 1, 2 or 4 rows: all rows of the block):
// markov_bias_gumbel_argmax with a VALU GEMV for the bias.
// Workgroup = one vocabulary chunk of 128-column tiles. GEMV mapping: thread t
// owns 8 columns (t % 16) and 16 contiguous rank rows (t / 16) per pass of 256
// rank rows; a wave's load instruction reads 4 rank rows x 256 contiguous
// bytes. The 16 W loads of the first tile are issued before anything waits
// on them; the token of the previous position is resolved and E[d] is
// gathered while they are in flight. The 16 rank slices are summed through
// LDS in a fixed order; the epilogue gives each row 32 threads x 4 columns,
// so one Philox block serves the 4 columns a thread owns.
// ---------------------------------------------------------------------------
template <int RB, bool kBf16Base, bool kInKernelPick>
__global__ __launch_bounds__(kThreads) void markov_bias_gumbel_argmax_gemv(StepArgs a) {
  __shared__ float red[kSlices][RB][kTile];
  __shared__ uint64_t s_key[kWaves];
  __shared__ Stat s_stat[kWaves];

  const int t = threadIdx.x;
  const int chunk = blockIdx.x;
  const int V = a.V, r = a.r, K = a.K, k = a.k, C = a.n_chunks;
  const int chunk_lo = chunk * a.chunk_cols;
  const int chunk_hi = min(V, chunk_lo + a.chunk_cols);
  const int n_tiles = (chunk_hi - chunk_lo + kTile - 1) / kTile;
  const int n_pass = (r + kSlices * kRowsPerSlice - 1) / (kSlices * kRowsPerSlice);
  const int n_real = a.n_real ? *a.n_real : a.B;

  const int cg = t % 16;          // 8-column group of the GEMV
  const int js = t / 16;          // rank slice of the GEMV
  const int er = t / 32;          // epilogue row
  const int ec = (t % 32) * 4;    // epilogue column offset within the tile
  const bool e_row = er < RB && er < a.B;
  const bool pick_here = kInKernelPick && k > 0;

  // (0) per-row state and the rows' embedding sources: uniform addresses, so
  // scalar loads, issued before the W stream (a vector load issued after the
  // W loads could only be waited on together with them)
  RowState rows[RB];
  const uint16_t* erow[RB];   // embedding row of each row of the block (null = zero row)
#pragma unroll
  for (int rr = 0; rr < RB; ++rr) {
    rows[rr] = RowState{};
    erow[rr] = nullptr;
    if (rr < a.B) {
      rows[rr] = row_state(a, rr, n_real);
      if (k == 0)
        erow[rr] = a.E + (size_t)clamp_token(a.prev_token[rr], V) * r;
      else if (!kInKernelPick)
        erow[rr] = a.e_buf + (size_t)rr * r;
    }
  }
  RowState rs = rows[0];
#pragma unroll
  for (int rr = 1; rr < RB; ++rr)
    if (er == rr) rs = rows[rr];

  // (1) partials of position k-1 (masks are applied when they are reduced,
  // not here: a select right after a load would wait for it)
  uint64_t pk[kPickPerThread];
  Stat ps[kPickPerThread];
  if (pick_here) {
#pragma unroll
    for (int i = 0; i < kPickPerThread; ++i) {
      const int c = t + i * kThreads;
      const int ci = c < C ? c : 0;
      pk[i] = a.prev_key[ci];
      if (chunk == 0) ps[i] = a.prev_stat[ci];
    }
  }

  // (2) W loads of tile 0, pass 0
  uint4 wv[kRowsPerSlice];
  {
    const int col = chunk_lo + cg * 8;
    const int j0 = js * kRowsPerSlice;
    issue_w(a.W, V, col < chunk_hi && j0 < r, j0, col, wv);
  }

  // (3) base logits of tile 0 (epilogue threads)
  Base4<kBf16Base> bv;
  auto prefetch_base = [&](int tile) {
    const int v0 = chunk_lo + tile * kTile + ec;
    const bool ok = e_row && v0 < chunk_hi && !rs.pad;
    const size_t off = ok ? ((size_t)er * K + k) * (size_t)V + v0 : 0;
    load_base4<kBf16Base>(bv, a.base, off);
  };
  prefetch_base(0);

  // (4) d_{k-1} at B == 1: the previous position's argmax over all chunks
  if (pick_here) {
    uint64_t key = 0;
    Stat sst{-INFINITY, 0.0f};
#pragma unroll
    for (int i = 0; i < kPickPerThread; ++i) {
      const bool in = t + i * kThreads < C;
      key = umax64(key, in ? pk[i] : 0ull);
      if (chunk == 0) sst = stat_merge(sst, in ? ps[i] : Stat{-INFINITY, 0.0f});
    }
    wg_reduce(key, sst, s_key, s_stat);
    const int d = clamp_token((int)key_token(key), V);
    if (chunk == 0 && t == 0) {
      a.tokens[(size_t)(k - 1)] = d;
      a.row_stat[(size_t)(k - 1)] = sst;
    }
    erow[0] = a.E + (size_t)d * r;
  }

  uint64_t best = 0;
  Stat st{-INFINITY, 0.0f};

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int tile0 = chunk_lo + tile * kTile;
    const int col = tile0 + cg * 8;
    float acc[RB][8];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[rr][i] = 0.0f;
    if (tile > 0) prefetch_base(tile);

    for (int p = 0; p < n_pass; ++p) {
      const int j0 = p * (kSlices * kRowsPerSlice) + js * kRowsPerSlice;
      const bool j_ok = j0 < r;
      if (tile > 0 || p > 0) issue_w(a.W, V, col < chunk_hi && j_ok, j0, col, wv);
      uint4 ev[RB][2];
      load_e<RB>(erow, a.E, j0, j_ok, ev);
      if (j_ok) gemv_pass<RB>(wv, ev, acc);
    }

    store_slices<RB>(red, js, cg, acc);
    __syncthreads();
    const int v0 = tile0 + ec;
    if (e_row && v0 < chunk_hi) {
      float bias[4];
      slice_sum<RB>(red, er, ec, bias);
      float base[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (!rs.pad) widen_base4<kBf16Base>(bv, base);
      epilogue4(rs, k, (uint32_t)v0, base, bias, a.logits + ((size_t)er * K + k) * (size_t)V + v0, best, st);
    }
    __syncthreads();  // red is rewritten by the next tile
  }

  reduce_lanes(best, st, 32);
  if (e_row && (t % 32) == 0) {
    a.part_key[(size_t)er * C + chunk] = best;
    a.part_stat[(size_t)er * C + chunk] = st;
  }
}

// ---------------------------------------------------------------------------
// Kernel 1, any B (rows processed 4 at a time): the same fused kernel with the
// GEMV re-run per row tile. Used above 4 rows.
// ---------------------------------------------------------------------------
template <bool kBf16Base>
__global__ __launch_bounds__(kThreads) void markov_bias_gumbel_argmax_rows(StepArgs a) {
  constexpr int RB = 4;
  __shared__ float red[kSlices][RB][kTile];

  const int t = threadIdx.x;
  const int chunk = blockIdx.x;
  const int V = a.V, r = a.r, K = a.K, k = a.k, C = a.n_chunks;
  const int chunk_lo = chunk * a.chunk_cols;
  const int chunk_hi = min(V, chunk_lo + a.chunk_cols);
  const int n_tiles = (chunk_hi - chunk_lo + kTile - 1) / kTile;
  const int n_pass = (r + kSlices * kRowsPerSlice - 1) / (kSlices * kRowsPerSlice);
  const int n_real = a.n_real ? *a.n_real : a.B;
  const int cg = t % 16, js = t / 16, er = t / 32, ec = (t % 32) * 4;

  for (int rb0 = 0; rb0 < a.B; rb0 += RB) {
    const uint16_t* erow[RB];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const int b = rb0 + rr;
      erow[rr] = nullptr;
      if (b < a.B)
        erow[rr] = (k == 0) ? a.E + (size_t)clamp_token(a.prev_token[b], V) * r : a.e_buf + (size_t)b * r;
    }
    const int eb = rb0 + er;
    const bool e_row = er < RB && eb < a.B;
    RowState rs{};
    if (e_row) rs = row_state(a, eb, n_real);
    uint64_t best = 0;
    Stat st{-INFINITY, 0.0f};

    for (int tile = 0; tile < n_tiles; ++tile) {
      const int tile0 = chunk_lo + tile * kTile;
      const int col = tile0 + cg * 8;
      const bool col_ok = col < chunk_hi;
      float acc[RB][8];
#pragma unroll
      for (int rr = 0; rr < RB; ++rr)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[rr][i] = 0.0f;
      Base4<kBf16Base> bv;
      const int v0 = tile0 + ec;
      const bool e_col = e_row && v0 < chunk_hi;
      const size_t eoff = ((size_t)eb * K + k) * (size_t)V + v0;
      for (int p = 0; p < n_pass; ++p) {
        const int j0 = p * (kSlices * kRowsPerSlice) + js * kRowsPerSlice;
        const bool j_ok = j0 < r;
        uint4 wv[kRowsPerSlice];
        issue_w(a.W, V, j_ok && col_ok, j0, col, wv);
        if (p == 0 && e_col && !rs.pad) load_base4<kBf16Base>(bv, a.base, eoff);
        uint4 ev[RB][2];
        load_e<RB>(erow, a.E, j0, j_ok, ev);
        if (j_ok) gemv_pass<RB>(wv, ev, acc);
      }
      store_slices<RB>(red, js, cg, acc);
      __syncthreads();
      if (e_col) {
        float bias[4];
        slice_sum<RB>(red, er, ec, bias);
        float base[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (!rs.pad) widen_base4<kBf16Base>(bv, base);
        epilogue4(rs, k, (uint32_t)v0, base, bias, a.logits + eoff, best, st);
      }
      __syncthreads();
    }
    reduce_lanes(best, st, 32);
    if (e_row && (t % 32) == 0) {
      a.part_key[(size_t)eb * C + chunk] = best;
      a.part_stat[(size_t)eb * C + chunk] = st;
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel 2: pick_and_gather. One workgroup per row: the row's chunk partials
// are reduced in a fixed order, d_k and the merged (M, S) are written, and
// E[d_k] is gathered into e_buf for position k+1.
// ---------------------------------------------------------------------------
struct PickArgs {
  const uint64_t* part_key;
  const Stat* part_stat;
  const uint16_t* E;
  int32_t* tokens;       // [B,K]
  Stat* row_stat;        // [B,K]
  uint16_t* e_buf;       // [B,r]
  int B, K, V, r, k, n_chunks;
};

__global__ __launch_bounds__(kThreads) void pick_and_gather(PickArgs a) {
  __shared__ uint64_t s_key[kWaves];
  __shared__ Stat s_stat[kWaves];
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  uint64_t best = 0;
  Stat st{-INFINITY, 0.0f};
  for (int c = t; c < a.n_chunks; c += kThreads) {
    best = umax64(best, a.part_key[(size_t)b * a.n_chunks + c]);
    st = stat_merge(st, a.part_stat[(size_t)b * a.n_chunks + c]);
  }
  wg_reduce(best, st, s_key, s_stat);
  const int d = clamp_token((int)key_token(best), a.V);
  if (t == 0) {
    a.tokens[(size_t)b * a.K + a.k] = d;
    a.row_stat[(size_t)b * a.K + a.k] = st;
  }
  if (a.k + 1 < a.K) {
    const uint16_t* src = a.E + (size_t)d * a.r;
    for (int j = t * 8; j < a.r; j += kThreads * 8)
      *reinterpret_cast<uint4*>(a.e_buf + (size_t)b * a.r + j) = *reinterpret_cast<const uint4*>(src + j);
  }
}

// ---------------------------------------------------------------------------
// Kernel 3: proposal_softmax. Grid = (row, position) x column blocks of
// 1024 kVec columns; thread t handles float4 j at column 4 (j * 256 + t) of
// its block, so every load and store instruction of a wave is one contiguous
// 1 KiB. All of a thread's logits loads are issued before the row's (M, S) is
// merged, so the merge runs while they are in flight. Positions are visited
// from last to first: the most recently written logits are read first, while
// they may still be in the Infinity Cache. Logits are read with the
// nontemporal hint (not touched again by this call); q is written with
// ordinary stores (B=88: 174 us against 189 with nontemporal stores). Sampling rows
// recompute s = logit * invT exactly as the draw did; greedy rows get one-hot
// at d_k; positions a resident block left without a token (token -1 after an
// expired wait) get NaN. With last_from_partials (B == 1), the last position's token and
// (M, S) are reduced here from its chunk partials; block 0 of that row stores
// them.
// ---------------------------------------------------------------------------
// float4 per thread: 16 (16384 columns per block) from 8 rows up, 8 below,
// where 16384-column blocks would leave too few blocks (B=1: 91)
constexpr int kPropVecSmall = 8;
constexpr int kPropVecLarge = 16;
constexpr int kPropLargeRows = 8;
template <int kVec>
constexpr int prop_cols() { return kThreads * 4 * kVec; }

typedef float fx4_t __attribute__((ext_vector_type(4)));

struct PropArgs {
  const float* logits;
  const float* temperature;
  int32_t* tokens;
  Stat* row_stat;
  const uint64_t* last_key;   // [B,C] partials of position K-1 (last_from_partials)
  const Stat* last_stat;
  const Stat* part_stat;      // [K,B,n_part] per-workgroup statistics (n_part > 0)
  float* q;
  const int32_t* slot;        // [B] row b's proposals go to q row slot[b] (NULL: row b)
  int n_slots;                // rows of q (slots outside [0, n_slots) write none)
  int B, K, V, n_chunks;
  int blocks_per_row;
  int last_from_partials;
  int n_part;
};

// One block of proposal_softmax; kChecked: the row's last block, whose
// accesses are bounds-checked (all others are unconditional, so the
// compiler's waits for the loads stay exact).
template <int kVec, bool kChecked>
__device__ __forceinline__ void proposal_block(const PropArgs& a, int b, int k, int cb, uint64_t* s_key,
                                               Stat* s_stat) {
  const int t = threadIdx.x;
  const int bk = b * a.K + k;
  const float T = a.temperature[b];
  const bool greedy = !(T > 0.0f);
  const size_t row = (size_t)bk * a.V;
  const int c0 = cb * prop_cols<kVec>() + 4 * t;
  auto in_row = [&](int v) { return !kChecked || v < a.V; };
  // where the row's proposals go: its own row, or its slot (a slot out of
  // range writes none; the token and statistics below are still kept)
  const int sb = a.slot ? a.slot[b] : b;
  const bool q_ok = sb >= 0 && sb < a.n_slots;
  float* const qrow = a.q + ((size_t)(q_ok ? sb : 0) * a.K + k) * a.V;

  // the first statistics partial of this thread is loaded before the logits,
  // so the merge waits for it alone (loads complete in order)
  const bool parts = a.n_part > 0 && !(a.last_from_partials && k == a.K - 1);
  const Stat* ps = a.part_stat + ((size_t)k * a.B + b) * a.n_part;
  Stat p0{-INFINITY, 0.0f};
  fx4_t lg[kVec];
  if (!greedy) {
    if (parts) {
      if (t < a.n_part) p0 = ps[t];
      for (int i = t + kThreads; i < a.n_part; i += kThreads) p0 = stat_merge(p0, ps[i]);   // > 256 CUs
    }
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const int v = c0 + j * kThreads * 4;
      lg[j] = in_row(v) ? __builtin_nontemporal_load(reinterpret_cast<const fx4_t*>(a.logits + row + v))
                        : fx4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
  }

  Stat st;
  int tok;
  if (a.last_from_partials && k == a.K - 1) {
    uint64_t best = 0;
    Stat sst{-INFINITY, 0.0f};
    for (int c = t; c < a.n_chunks; c += kThreads) {
      best = umax64(best, a.last_key[(size_t)b * a.n_chunks + c]);
      sst = stat_merge(sst, a.last_stat[(size_t)b * a.n_chunks + c]);
    }
    wg_reduce(best, sst, s_key, s_stat);
    st = sst;
    tok = clamp_token((int)key_token(best), a.V);
    if (cb == 0 && t == 0) {
      a.tokens[bk] = tok;
      a.row_stat[bk] = st;
    }
  } else if (parts) {
    // the resident kernels leave one statistics partial per workgroup
    Stat sst = p0;
    uint64_t unused = 0;
    wg_reduce(unused, sst, s_key, s_stat);
    st = sst;
    tok = a.tokens[bk];
  } else {
    st = a.row_stat[bk];
    tok = a.tokens[bk];
  }

  if (tok < 0) {
    // a resident block whose bounded wait expired left this position without
    // a token (and without complete statistics): its proposal is NaN
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const int v = c0 + j * kThreads * 4;
      if (q_ok && in_row(v)) *reinterpret_cast<fx4_t*>(qrow + v) = fx4_t{nan, nan, nan, nan};
    }
    return;
  }
  if (greedy) {
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const int v = c0 + j * kThreads * 4;
      if (q_ok && in_row(v)) {
        const fx4_t out{v == tok ? 1.0f : 0.0f, v + 1 == tok ? 1.0f : 0.0f, v + 2 == tok ? 1.0f : 0.0f,
                        v + 3 == tok ? 1.0f : 0.0f};
        *reinterpret_cast<fx4_t*>(qrow + v) = out;
      }
    }
    return;
  }
  const float invT = __fdiv_rn(1.0f, T);
  const float invS = __fdiv_rn(1.0f, st.l);
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const int v = c0 + j * kThreads * 4;
    if (q_ok && in_row(v)) {
      fx4_t out;
      out.x = __fmul_rn(__expf(__fsub_rn(__fmul_rn(lg[j].x, invT), st.m)), invS);
      out.y = __fmul_rn(__expf(__fsub_rn(__fmul_rn(lg[j].y, invT), st.m)), invS);
      out.z = __fmul_rn(__expf(__fsub_rn(__fmul_rn(lg[j].z, invT), st.m)), invS);
      out.w = __fmul_rn(__expf(__fsub_rn(__fmul_rn(lg[j].w, invT), st.m)), invS);
      *reinterpret_cast<fx4_t*>(qrow + v) = out;
    }
  }
}

template <int kVec>
__global__ __launch_bounds__(kThreads) void proposal_softmax(PropArgs a) {
  __shared__ uint64_t s_key[kWaves];
  __shared__ Stat s_stat[kWaves];
  const int rk = blockIdx.x / a.blocks_per_row;
  const int cb = blockIdx.x % a.blocks_per_row;
  const int k = a.K - 1 - rk / a.B;
  const int b = rk % a.B;
  if ((cb + 1) * prop_cols<kVec>() <= a.V)
    proposal_block<kVec, false>(a, b, k, cb, s_key, s_stat);
  else
    proposal_block<kVec, true>(a, b, k, cb, s_key, s_stat);
}

// ---------------------------------------------------------------------------
// Resident path (B <= 2): one persistent launch runs all K positions, and each
// workgroup keeps its slice of W on chip for the whole block, so W is read
// from HBM once per block instead of once per position.
//
// One 512-thread workgroup per compute unit owns up to 784 vocabulary columns
// (98 groups of 8). A (group, rank slice of 32 rows) unit holds 8 columns x 16
// bf16 pairs (rows 2p, 2p+1 packed in one dword); groups 0..63 live in VGPRs
// (thread = one unit), groups 64..97 in LDS. The bias GEMV is v_dot2 of those
// pairs with the embedding pairs, then a reduce-scatter over the 8 rank
// slices leaves every lane of the epilogue one column (one row) or 2
// consecutive columns of one row (two rows; two lanes share a Philox block).
// Positions are separated by an exchange: each workgroup publishes its
// per-row argmax key as one 64-bit word tagged with the position as soon as
// it is merged, and every workgroup polls all words (a bounded wait) and
// reduces them in the same order, so all agree on d_k. The softmax
// statistics (read only by the proposal) and the Gumbel noise of position k+1
// do not depend on d_k and are computed while the first reads are in flight;
// the base logits of k+1 are loaded with the E rows of d_k.
// ---------------------------------------------------------------------------
constexpr int kResThreads = 512;
constexpr int kResWaves = kResThreads / 64;
constexpr int kResSlice = 784;                             // max columns per workgroup
constexpr int kResGroups = kResSlice / 8;                  // 98 groups of 8 columns
constexpr int kResRegGroups = kResWaves * 8;               // 64 groups in VGPRs
constexpr int kResLdsUnits = (kResGroups - kResRegGroups) * 8;  // 272 units in LDS
constexpr int kResRank = 256;                              // 8 rank slices of 32 rows
constexpr int kResPairs = 16;                              // bf16 pairs per unit column
// rows of this kernel: from three rows the MFMA form below is faster (B=3:
// 100 us a block against 144, B=4: 102 against 146; B=2: 89.7 against ~99)
constexpr int kResRowsMax = 2;
constexpr size_t kResLdsW = (size_t)kResPairs * kResLdsUnits * 32;   // 139,264 bytes
constexpr size_t kResLdsE = (size_t)kResRowsMax * kResRank * 2;      // 1,024 bytes
constexpr size_t kResLdsBytes = kResLdsW + kResLdsE;
// packed W (dspark_pack_w): 16-byte units per workgroup and kernel, and those
// of the register part (the rest is the kernel's LDS image)
constexpr size_t kPackWgU4 = (size_t)kResSlice * kResRank * 2 / 16;   // 25,088
constexpr int kPackRegU4 = 16384;
static_assert(kResPairs * 2 * kResThreads == kPackRegU4, "small-batch register units");
static_assert((size_t)kPackRegU4 * 16 + kResLdsW == kPackWgU4 * 16, "small-batch block size");
constexpr int kResTagShift = 50;                           // word: tag | ord(z) | index
constexpr uint64_t kResIdxMask = (1ull << 18) - 1;         // V <= 2^18
constexpr int kResMaxCUs = 512;
constexpr unsigned kDefaultWaitLimit = 1u << 20;           // about a second of polling
constexpr int kExRows = 128;                               // exchange rows per workgroup (both resident kernels)
constexpr int kExZeroWords = 512;                          // 4 KB that are never written

// Exchange state of the resident kernels: one copy per device, in the
// library's own device memory (zero when the code object is loaded), so it
// never needs clearing before a call. Every resident launch has G = the
// device's compute-unit count; workgroup i of the launches on a device takes
// arrival number i in launch order, so call c = arrival / G is the same for
// all workgroups of one launch (launches never overlap: each needs every CU).
// A word published at position k of call c carries the tag (c & 1, k + 1).
// At exit every workgroup rewrites each of its slots this call did not use
// with a tag of this call (res_retire), so when call c + 1 starts every slot
// holds a tag of parity c & 1, which no tag call c + 1 waits for can equal.
struct ResExchange {
  unsigned long long arrivals;   // resident workgroups started on this device
  unsigned long long failed;     // 1 + the index of the last call in which a bounded wait expired
  unsigned long long pad[30];    // the words below start on their own cache line
  uint64_t xrow[2][kResMaxCUs][kExRows];   // per-workgroup tagged words, by position parity
  uint64_t xwin[2][kExRows];               // tagged row winners (MFMA kernel), by position parity
  uint64_t zeros[kExZeroWords];            // never written: base logits of rows that have none
};
__device__ __align__(256) ResExchange g_exchange;

__device__ __forceinline__ uint64_t res_tag(uint32_t cpar, int k) {
  return (((uint64_t)cpar << 8) | (uint64_t)(k + 1)) << kResTagShift;
}

__device__ __forceinline__ uint64_t ld_agent_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The call index of this launch (thread 0 only; it is the first device
// access of the workgroup, and its result is needed only at the first
// publish).
__device__ __forceinline__ unsigned long long res_arrive(ResExchange* ex, int G) {
  return __hip_atomic_fetch_add(&ex->arrivals, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) /
         (unsigned long long)G;
}

__device__ __forceinline__ void res_fail(ResExchange* ex, unsigned long long call) {
  __hip_atomic_fetch_max(&ex->failed, call + 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Rewrite, with a tag of this call, each slot of workgroup g that this call
// did not publish into: rows >= B, and the parity buffers of positions it
// never reached (n_pub = positions it published; buffer h is used from
// position h on). Winner slots of rows b = g, g + G, ... are owned by g
// (n_win = positions it published winners for; 0 where the kernel has none).
// Called by every thread of the workgroup once it is done with the exchange.
__device__ __forceinline__ void res_retire(ResExchange* ex, int g, int G, int B, int n_pub, int n_win,
                                           uint32_t cpar, int t_in, int nthreads) {
  // the thread index through an opaque copy, so the slot addresses are formed
  // here and not hoisted into registers held across the caller's loops
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"(t_in));
  const uint64_t old = res_tag(cpar, -1);   // tag (c & 1, 0): never waited for
  for (int i = t; i < 2 * kExRows; i += nthreads) {
    const int h = i / kExRows, b = i % kExRows;
    if (!(b < B && n_pub > h)) st_agent_u64(&ex->xrow[h][g][b], old);
  }
  for (int i = t; i < 2 * kExRows; i += nthreads) {
    const int h = i / kExRows, b = i % kExRows;
    if (b % G == g && !(b < B && n_win > h)) st_agent_u64(&ex->xwin[h][b], old);
  }
}

// Status of the last resident call on this device: 1 if one of its bounded
// waits expired, else 0 (also when no resident call has run).
__global__ void res_status(ResExchange* ex, unsigned G, int32_t* out) {
  const unsigned long long a = __hip_atomic_load(&ex->arrivals, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned long long f = __hip_atomic_load(&ex->failed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  out[0] = (a >= G && f == a / G) ? 1 : 0;
}

typedef __attribute__((address_space(1))) void* lds_gptr_t;   // global source of an LDS-direct load
typedef __attribute__((address_space(3))) void* lds_lptr_t;   // its LDS destination

struct ResArgs {
  const void* base;
  const uint16_t* E;
  const uint16_t* W;
  const int32_t* prev_token;
  const int64_t* seed;
  const int64_t* offset;
  const float* temperature;
  const int32_t* n_real;
  float* logits;
  int32_t* tokens;
  ResExchange* ex;     // the device's exchange state
  Stat* stat_part;     // [K][B][G] per-workgroup softmax statistics
  const uint4* Wp;     // packed W, this kernel's layout (kPacked), else unused
  int B, K, V, r, slice;
  unsigned spin_limit; // reads of a word before its wait expires (0: expires at once)
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t w, uint32_t e, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, e),
                                        acc, false);
}

// (a.lo16, b.lo16) and (a.hi16, b.hi16): bf16 pairs of two rank rows
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// rows 2p (x) and 2p+1 (y), 8 columns each -> 8 column pairs
__device__ __forceinline__ void pack_pairs(uint4 x, uint4 y, uint32_t out[8]) {
  out[0] = pair_lo(x.x, y.x); out[1] = pair_hi(x.x, y.x);
  out[2] = pair_lo(x.y, y.y); out[3] = pair_hi(x.y, y.y);
  out[4] = pair_lo(x.z, y.z); out[5] = pair_hi(x.z, y.z);
  out[6] = pair_lo(x.w, y.w); out[7] = pair_hi(x.w, y.w);
}

// Value of lane partner(l) within its group of 8 lanes, by DPP: the half-row
// mirror (l <-> 7 - l, pairing the lanes that differ in bit 2), lane ^ 2 and
// lane ^ 1. No LDS round trip, unlike a lane shuffle.
__device__ __forceinline__ float dpp_mirror8(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}

// Reduce-scatter of acc[RB][8] over the 8 rank-slice lanes of a column group
// (lanes differing in bits 0..2): every step halves what a lane keeps, so
// lane js (bits b2 b1 b0) ends with RB sums: one row, column js (RB = 1); two
// rows, row b2, columns 2 (js & 3) and 2 (js & 3) + 1 (RB = 2). The three
// exchange steps pair lanes of opposite bit 2 (by the half-row mirror, which
// pairs 0-7, 1-6, 2-5, 3-4), then of opposite bit 1, then of opposite bit 0,
// and still add every slice exactly once.
template <int RB>
__device__ __forceinline__ void reduce_scatter(const float (&acc)[RB][8], int js, float bias[RB]) {
  static_assert(RB == 1 || RB == 2, "rows of the small-batch resident kernel");
  const int b0 = js & 1, b1 = (js >> 1) & 1, b2 = (js >> 2) & 1;
  if constexpr (RB == 1) {
    float h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float keep = b2 ? acc[0][4 + i] : acc[0][i];
      const float send = b2 ? acc[0][i] : acc[0][4 + i];
      h[i] = __fadd_rn(keep, dpp_mirror8(send));
    }
    float q[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float keep = b1 ? h[2 + i] : h[i];
      const float send = b1 ? h[i] : h[2 + i];
      q[i] = __fadd_rn(keep, dpp_xor2(send));
    }
    bias[0] = __fadd_rn(b0 ? q[1] : q[0], dpp_xor1(b0 ? q[0] : q[1]));
  } else {
    // the mirror keeps a row (b2), xor 2 half its columns (b1), xor 1 a pair (b0)
    float h[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float keep = b2 ? acc[1 % RB][c] : acc[0][c];
      const float send = b2 ? acc[0][c] : acc[1 % RB][c];
      h[c] = __fadd_rn(keep, dpp_mirror8(send));
    }
    float q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float keep = b1 ? h[4 + i] : h[i];
      const float send = b1 ? h[i] : h[4 + i];
      q[i] = __fadd_rn(keep, dpp_xor2(send));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float keep = b0 ? q[2 + i] : q[i];
      const float send = b0 ? q[i] : q[2 + i];
      bias[i % RB] = __fadd_rn(keep, dpp_xor1(send));
    }
  }
}

// Gumbel noise of N = 1 or 2 consecutive columns v .. v + N - 1 at position k
// (two columns start at an even v): components v % 4 .. of the Philox block
// of columns v - v % 4 .., the values every column gets from its block.
template <int N>
__device__ __forceinline__ void noise_n(const RowState& rs, int k, uint32_t v, float g[N]) {
  uint32_t k0 = rs.key0, k1 = rs.key1;
  if constexpr (N == 2) {
    // two rows: the keys differ by lane; taken through an opaque copy, the
    // round keys are formed here instead of being precomputed and held in
    // vector registers across the position loop (which spilled them)
    asm volatile("v_mov_b32 %0, %1" : "=v"(k0) : "v"(rs.key0));
    asm volatile("v_mov_b32 %0, %1" : "=v"(k1) : "v"(rs.key1));
  }
  const uint4 x = philox4x32_10(make_uint4(v >> 2, (uint32_t)k, rs.ctr2, rs.ctr3), k0, k1);
  const uint32_t c = v & 3u;
  g[0] = gumbel_from_bits(c == 0 ? x.x : c == 1 ? x.y : c == 2 ? x.z : x.w);
  if constexpr (N == 2) g[1] = gumbel_from_bits(c == 0 ? x.y : x.w);
}

// The epilogue of N consecutive columns with the noise already drawn, in two
// parts (the arithmetic of epilogue4 per column): the logits and the argmax
// key first, keeping the scaled logits s, and the softmax statistics of s
// later (only the proposal reads them).
template <int N>
__device__ __forceinline__ void epilogue_n_key(const RowState& rs, uint32_t v, const float base[N],
                                               const float bias[N], const float g[N], float* logits_out,
                                               uint64_t& best, float s[N]) {
  float lg[N];
#pragma unroll
  for (int i = 0; i < N; ++i) lg[i] = __fadd_rn(base[i], bias[i]);
  if constexpr (N == 1) *logits_out = lg[0];
  else *reinterpret_cast<float2*>(logits_out) = make_float2(lg[0], lg[1]);
  if (rs.greedy) {
#pragma unroll
    for (int i = 0; i < N; ++i) best = umax64(best, score_key(lg[i], v + i));
    return;
  }
#pragma unroll
  for (int i = 0; i < N; ++i) {
    s[i] = __fmul_rn(lg[i], rs.invT);
    best = umax64(best, score_key(__fadd_rn(s[i], g[i]), v + i));
  }
}

template <int N>
__device__ __forceinline__ void epilogue_n_stat(const float s[N], Stat& st) {
  float m = -INFINITY;   // a NaN score counts as -inf
#pragma unroll
  for (int i = 0; i < N; ++i) m = fmaxf(m, s[i]);
  float l = 0.0f;
  if (m != -INFINITY) {
#pragma unroll
    for (int i = 0; i < N; ++i) l = __fadd_rn(l, __expf(__fsub_rn(s[i], m)));
  }
  st = stat_merge(st, Stat{m, l});
}

template <int RB, bool kBf16Base, bool kPacked>
__global__ __launch_bounds__(kResThreads, 1) void markov_bias_gumbel_argmax_resident(ResArgs a) {
  extern __shared__ __align__(16) unsigned char res_lds[];
  uint32_t* lds_w = reinterpret_cast<uint32_t*>(res_lds);               // [16][272][8]
  uint32_t* lds_e = reinterpret_cast<uint32_t*>(res_lds + kResLdsW);    // [RB][128] bf16 pairs
  __shared__ uint64_t s_key[kResWaves][RB];
  __shared__ Stat s_stat[kResWaves][RB];
  __shared__ uint64_t s_x[kResWaves][RB];
  __shared__ int s_fail;
  __shared__ unsigned long long s_call;

  const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
  const int g = blockIdx.x, G = gridDim.x;
  const int V = a.V, r = a.r, K = a.K, B = a.B;
  const int js = lane & 7;                    // rank slice: rows 32 js .. 32 js + 31
  const bool j_ok = 32 * js < r;
  const int col0 = g * a.slice;
  const int ncols = max(0, min(a.slice, V - col0));
  const int ngroups = ncols / 8;
  const int cg_r = 8 * wv + (lane >> 3);      // this thread's VGPR unit: column group
  const bool reg_ok = cg_r < ngroups;
  const int n_lds_units = max(0, ngroups - kResRegGroups) * 8;
  const bool lds_ok = t < n_lds_units;        // this thread's LDS unit (if any) is unit t
  const int cg_l = kResRegGroups + (t >> 3);

  // epilogue lane mapping after the reduce-scatter: every lane has RB columns
  // (RB = 1: column js of its group; RB = 2: columns 2 (js & 3) .. + 1 of row er)
  static_assert(RB == 1 || RB == 2, "rows of the small-batch resident kernel");
  const int er = RB == 2 ? (js >> 2) : 0;
  const bool e_act = er < B;
  const int ecol = RB == 1 ? js : 2 * (js & 3);
  const uint32_t v_r = (uint32_t)(col0 + 8 * cg_r + ecol);   // epilogue column(s), VGPR unit
  const uint32_t v_l = (uint32_t)(col0 + 8 * cg_l + ecol);   // epilogue column(s), LDS unit
  const bool ep_r = e_act && reg_ok;
  const bool ep_l = e_act && lds_ok;

  // the rows' inputs: position 0's tokens d_{-1}, temperatures, Philox keys
  // and offsets, the padding count; then this lane's row state
  int tok_in[RB];
  float t_in[RB];
  int64_t sd_in[RB], of_in[RB];
  int n_real = B;
  auto load_inputs = [&]() {
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const bool in = rr < B;
      tok_in[rr] = in ? a.prev_token[rr] : 0;
      t_in[rr] = in ? a.temperature[rr] : 0.0f;
      sd_in[rr] = in ? a.seed[rr] : 0;
      of_in[rr] = in ? a.offset[rr] : 0;
    }
    n_real = a.n_real ? *a.n_real : B;
  };
  RowState rs;
  int d0[RB];
  auto set_rows = [&]() {
    RowState rows[RB];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      rows[rr] = rr < B ? row_state_of(t_in[rr], sd_in[rr], of_in[rr], rr, n_real) : RowState{};
      d0[rr] = rr < B ? clamp_token(tok_in[rr], V) : 0;
    }
    rs = rows[0];
#pragma unroll
    for (int rr = 1; rr < RB; ++rr)
      if (er == rr) rs = rows[rr];
  };

  // ---- noise and base logits of a position for this lane's epilogue columns
  float gq[2][RB];
  Base4<kBf16Base> bq[2];
  auto make_noise = [&](int k) {
    if (e_act && !rs.greedy) {
      noise_n<RB>(rs, k, v_r, gq[0]);
      if (lds_ok) noise_n<RB>(rs, k, v_l, gq[1]);
    }
  };
  auto load_base = [&](int k) {
    const size_t row_off = ((size_t)er * K + k) * (size_t)V;
    const bool br = ep_r && !rs.pad, bl = ep_l && !rs.pad;
    load_base_n<kBf16Base, RB>(bq[0], a.base, br ? row_off + v_r : 0);
    load_base_n<kBf16Base, RB>(bq[1], a.base, bl ? row_off + v_l : 0);
  };
  auto prepare = [&](int k) {
    make_noise(k);
    load_base(k);
  };

  // ---- the embedding rows E[d] of a position's tokens, into LDS
  auto gather_e = [&](const int* d) {
    const uint32_t* E32 = reinterpret_cast<const uint32_t*>(a.E);
    for (int i = t; i < RB * (kResRank / 2); i += kResThreads) {
      const int rr = i / (kResRank / 2), jj = i % (kResRank / 2);
      uint32_t v = 0u;
      if (rr < B && jj < r / 2) v = E32[(size_t)d[rr] * (r / 2) + jj];
      lds_e[rr * (kResRank / 2) + jj] = v;
    }
  };

  // ---- setup: W on chip for the block (this thread's VGPR unit of 32 rank
  // rows x 8 columns as bf16 pairs, and the LDS units), the rows' inputs, this
  // workgroup's arrival (its count names the call), and position 0's E rows,
  // noise and base logits. The order is each W form's fastest as measured.
  uint32_t wr[8][kResPairs];
  unsigned long long arrival = 0;
  if constexpr (kPacked) {
    // The rows' inputs first, as scalar loads (uniform, read before any other
    // memory access), whose waits are not tied to the W stream's; then the W
    // stream before anything else, since every vector load behind it waits
    // for all of it (loads complete in order for their counter)
    load_inputs();
    // packed W: unit (i, t) of this workgroup's block holds columns 4h .. 4h + 3
    // (h = i % 2) of pair i / 2, already paired (512 x 16 B per instruction);
    // the LDS image follows, copied by LDS-direct loads (each wave instruction
    // 1 KB, lane i's 16 bytes at 16 i), waited for before the first barrier
    const uint4* src = a.Wp + (size_t)g * kPackWgU4 + t;
#pragma unroll
    for (int i = 0; i < 2 * kResPairs; ++i) {
      const uint4 v = src[(size_t)i * kResThreads];
      wr[4 * (i & 1) + 0][i >> 1] = v.x;
      wr[4 * (i & 1) + 1][i >> 1] = v.y;
      wr[4 * (i & 1) + 2][i >> 1] = v.z;
      wr[4 * (i & 1) + 3][i >> 1] = v.w;
    }
    unsigned char* dst = reinterpret_cast<unsigned char*>(lds_w) + (size_t)64 * wv * 16;
#pragma unroll
    for (int j = 0; j < (int)(kResLdsW / 16 / kResThreads); ++j)
      __builtin_amdgcn_global_load_lds((lds_gptr_t)(src + kPackRegU4 + (size_t)j * kResThreads),
                                       (lds_lptr_t)(dst + (size_t)j * kResThreads * 16), 16, 0, 0);
    set_rows();
    // position 0's E rows, noise and base logits, and the arrival, all issued
    // before any is waited for (only the first barrier needs them)
    uint32_t e0 = 0u;
    if (t < RB * (kResRank / 2)) {
      const int rr = t / (kResRank / 2), jj = t % (kResRank / 2);
      int tok = d0[0];
#pragma unroll
      for (int q = 1; q < RB; ++q)
        if (rr == q) tok = d0[q];
      if (rr < B && jj < r / 2) e0 = reinterpret_cast<const uint32_t*>(a.E)[(size_t)tok * (r / 2) + jj];
    }
    prepare(0);
    if (t == 0) arrival = __hip_atomic_fetch_add(&a.ex->arrivals, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (t < RB * (kResRank / 2)) lds_e[t] = e0;
  } else {
    // W [r, V] itself: the arrival and the rows' inputs first, then W (8 rank
    // rows of the VGPR unit per batch, 512 threads x 8 x 16 B = 64 KB in flight
    // per workgroup, paired in registers; then the LDS units the same way)
    if (t == 0) arrival = __hip_atomic_fetch_add(&a.ex->arrivals, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    load_inputs();
    set_rows();
    {
      const bool ok = reg_ok && j_ok;
      const uint16_t* src = a.W + (ok ? (size_t)(32 * js) * V + col0 + 8 * cg_r : 0);
      const size_t stride = ok ? (size_t)V : 0;
#pragma unroll
      for (int b8 = 0; b8 < 4; ++b8) {
        uint4 raw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) raw[i] = *reinterpret_cast<const uint4*>(src + (8 * b8 + i) * stride);
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          uint32_t pr[8];
          pack_pairs(raw[2 * pp], raw[2 * pp + 1], pr);
#pragma unroll
          for (int c = 0; c < 8; ++c) wr[c][4 * b8 + pp] = pr[c];
        }
      }
    }
    if (lds_ok) {
      const uint16_t* src = a.W + (j_ok ? (size_t)(32 * js) * V + col0 + 8 * cg_l : 0);
      const size_t stride = j_ok ? (size_t)V : 0;
#pragma unroll
      for (int b8 = 0; b8 < 4; ++b8) {
        uint4 raw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) raw[i] = *reinterpret_cast<const uint4*>(src + (8 * b8 + i) * stride);
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          uint32_t pr[8];
          pack_pairs(raw[2 * pp], raw[2 * pp + 1], pr);
          uint4* dst = reinterpret_cast<uint4*>(lds_w + ((size_t)(4 * b8 + pp) * kResLdsUnits + t) * 8);
          dst[0] = make_uint4(pr[0], pr[1], pr[2], pr[3]);
          dst[1] = make_uint4(pr[4], pr[5], pr[6], pr[7]);
        }
      }
    }
    gather_e(d0);
    prepare(0);
  }
  if (t == 0) {
    s_fail = 0;
    s_call = arrival / (unsigned long long)G;   // as res_arrive
  }
  if constexpr (kPacked) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's LDS-direct loads have landed
  __syncthreads();
  // the call's parity, wave-uniform (a scalar register); the full index is
  // read from LDS only where a wait expires
  const uint32_t cpar = __builtin_amdgcn_readfirstlane((uint32_t)s_call & 1u);

  for (int k = 0; k < K; ++k) {
    // ---- bias GEMV: VGPR unit, then LDS unit; reduce-scatter over the rank slices
    float bias_r[RB], bias_l[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) bias_l[i] = 0.0f;
    {
      float acc[RB][8];
#pragma unroll
      for (int rr = 0; rr < RB; ++rr)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[rr][c] = 0.0f;
      if (j_ok) {
#pragma unroll
        for (int pq = 0; pq < kResPairs / 4; ++pq) {
          uint4 e4[RB];
#pragma unroll
          for (int rr = 0; rr < RB; ++rr)
            e4[rr] = *reinterpret_cast<const uint4*>(lds_e + rr * (kResRank / 2) + 16 * js + 4 * pq);
#pragma unroll
          for (int p4 = 0; p4 < 4; ++p4) {
#pragma unroll
            for (int rr = 0; rr < RB; ++rr) {
              const uint32_t e = p4 == 0 ? e4[rr].x : p4 == 1 ? e4[rr].y : p4 == 2 ? e4[rr].z : e4[rr].w;
#pragma unroll
              for (int c = 0; c < 8; ++c) acc[rr][c] = dot2_bf16(wr[c][4 * pq + p4], e, acc[rr][c]);
            }
          }
        }
      }
      reduce_scatter<RB>(acc, js, bias_r);
    }
    if (lds_ok) {   // whole groups of 8 lanes take this branch together
      float acc[RB][8];
#pragma unroll
      for (int rr = 0; rr < RB; ++rr)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[rr][c] = 0.0f;
      if (j_ok) {
#pragma unroll
        for (int pq = 0; pq < kResPairs / 4; ++pq) {
          uint4 e4[RB];
#pragma unroll
          for (int rr = 0; rr < RB; ++rr)
            e4[rr] = *reinterpret_cast<const uint4*>(lds_e + rr * (kResRank / 2) + 16 * js + 4 * pq);
#pragma unroll
          for (int p4 = 0; p4 < 4; ++p4) {
            const int p = 4 * pq + p4;
            const uint4* src = reinterpret_cast<const uint4*>(lds_w + ((size_t)p * kResLdsUnits + t) * 8);
            const uint4 w0 = src[0], w1 = src[1];
            const uint32_t wl[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int rr = 0; rr < RB; ++rr) {
              const uint32_t e = p4 == 0 ? e4[rr].x : p4 == 1 ? e4[rr].y : p4 == 2 ? e4[rr].z : e4[rr].w;
#pragma unroll
              for (int c = 0; c < 8; ++c) acc[rr][c] = dot2_bf16(wl[c], e, acc[rr][c]);
            }
          }
        }
      }
      reduce_scatter<RB>(acc, js, bias_l);
    }

    // ---- epilogue of the lane's column(s): logits and argmax keys now; the
    // scaled logits are kept for the softmax statistics, which only the
    // proposal reads
    uint64_t best = 0;
    float sr[RB], sl[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) sr[i] = sl[i] = 0.0f;
    {
      float* out = a.logits + ((size_t)er * K + k) * (size_t)V;
      if (ep_r) {
        float base[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i) base[i] = 0.0f;
        if (!rs.pad) widen_base_n<kBf16Base, RB>(bq[0], base);
        epilogue_n_key<RB>(rs, v_r, base, bias_r, gq[0], out + v_r, best, sr);
      }
      if (ep_l) {
        float base[RB];
#pragma unroll
        for (int i = 0; i < RB; ++i) base[i] = 0.0f;
        if (!rs.pad) widen_base_n<kBf16Base, RB>(bq[1], base);
        epilogue_n_key<RB>(rs, v_l, base, bias_l, gq[1], out + v_l, best, sl);
      }
    }

    // ---- this workgroup's key per row (lanes, then waves), published at once
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const uint64_t kk = wave_max_u64((er == rr) ? best : 0ull);
      if (lane == 0) s_key[wv][rr] = kk;
    }
    __syncthreads();
    if (t < B) {
      uint64_t kk = s_key[0][t];
#pragma unroll
      for (int w = 1; w < kResWaves; ++w) kk = umax64(kk, s_key[w][t]);
      // a workgroup without columns has no candidate (kk == 0): it publishes the
      // tag alone, which every real candidate beats
      const uint64_t ord = kk >> 32;
      const uint64_t idx = kk ? kResIdxMask - (uint64_t)key_token(kk) : 0ull;
      st_agent_u64(&a.ex->xrow[k & 1][g][t], res_tag(cpar, k) | (ord << 18) | idx);
    }

    // ---- exchange: every workgroup's word for every row. Thread t polls row
    // t % RB (RB is a power of two dividing the thread count) of workgroups
    // t / RB, t / RB + 512 / RB, ...; rows >= B are padding and not polled.
    // The first read of the first word goes out now: the statistics and
    // position k+1's noise are computed while it is in flight, and the second
    // read follows it by that time.
    const int xr = t % RB;
    const bool polls = xr < B && t / RB < G && a.spin_limit != 0;
    const uint64_t* pw_first = &a.ex->xrow[k & 1][t / RB][xr];
    uint64_t w_first = 0;
    if (polls) w_first = ld_agent_u64(pw_first);

    // ---- softmax statistics per row: lanes, then waves through LDS (merged
    // by the workgroup once the exchange is done)
    {
      Stat st{-INFINITY, 0.0f};
      if (!rs.greedy) {
        if (ep_r) epilogue_n_stat<RB>(sr, st);
        if (ep_l) epilogue_n_stat<RB>(sl, st);
      }
#pragma unroll
      for (int rr = 0; rr < RB; ++rr) {
        Stat ss = (er == rr) ? st : Stat{-INFINITY, 0.0f};
        wave_merge_stat(ss);
        if (lane == 0) s_stat[wv][rr] = ss;
      }
    }
    auto store_stat = [&]() {
      if (t < B) {
        Stat ss = s_stat[0][t];
#pragma unroll
        for (int w = 1; w < kResWaves; ++w) ss = stat_merge(ss, s_stat[w][t]);
        a.stat_part[((size_t)k * B + t) * G + g] = ss;
      }
    };

    // ---- position k+1's noise does not depend on d_k: drawn now (its base
    // logits are loaded with the E rows, after the exchange, so that no load
    // is issued between the two reads of the first word)
    if (k + 1 < K) make_noise(k + 1);

    uint64_t xb = 0;
    bool failed = false;
    const uint64_t tag = res_tag(cpar, k) >> kResTagShift;
    // two reads of a word in flight, checked in turn: the first two are
    // staggered (the first word's by the work above, the others' by ~1500
    // cycles), so a word that lands between them is seen half a round trip
    // sooner; later rounds read it twice again (three in flight were no
    // better: more traffic)
    auto poll_word = [&](const uint64_t* pw, uint64_t w0, uint64_t w1) -> bool {
      for (unsigned reads = 2;; reads += 2) {
        if ((w0 >> kResTagShift) == tag) { xb = umax64(xb, w0); return true; }
        if ((w1 >> kResTagShift) == tag) { xb = umax64(xb, w1); return true; }
        if (reads >= a.spin_limit) return false;
        w0 = ld_agent_u64(pw);
        w1 = ld_agent_u64(pw);
      }
    };
    if (xr < B && t / RB < G) {
      if (!polls) {
        failed = true;   // a limit of 0: every wait expires at once, without reading
      } else {
        failed = !poll_word(pw_first, w_first, ld_agent_u64(pw_first));
        for (int gg = t / RB + kResThreads / RB; !failed && gg < G; gg += kResThreads / RB) {
          const uint64_t* pw = &a.ex->xrow[k & 1][gg][xr];
          const uint64_t w0 = ld_agent_u64(pw);
          __builtin_amdgcn_s_sleep(24);
          failed = !poll_word(pw, w0, ld_agent_u64(pw));
        }
      }
    }
    if (failed) {
      s_fail = 1;
      res_fail(a.ex, s_call);
    }
    // lanes of the same row (equal t % RB) combine
    xb = wave_max_u64_class<RB>(xb);
    if (lane < RB) s_x[wv][lane] = xb;
    __syncthreads();
    if (s_fail) {
      // an expired wait: this position and the later ones get no token (this
      // position's statistics are still stored: other workgroups may have
      // drawn its token)
      store_stat();
      if (g == 0 && t < B)
        for (int kk = k; kk < K; ++kk) a.tokens[(size_t)t * K + kk] = -1;
      res_retire(a.ex, g, G, B, k + 1, 0, cpar, t, kResThreads);
      return;
    }
    int d[RB];
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      uint64_t x = s_x[0][rr];
#pragma unroll
      for (int w = 1; w < kResWaves; ++w) x = umax64(x, s_x[w][rr]);
      d[rr] = clamp_token((int)(kResIdxMask - (x & kResIdxMask)), V);
    }
    if (g == 0 && t < B) a.tokens[(size_t)t * K + k] = d[t % RB];
    // the E rows of the tokens just drawn and position k+1's base logits:
    // loaded now; the E rows are stored to LDS after the statistics are
    // merged (which run while the loads are in flight), and the base logits
    // are first needed by the next epilogue
    const bool e_thr = t < RB * (kResRank / 2);
    uint32_t ev = 0u;
    if (k + 1 < K) {
      if (e_thr) {
        const int rr = t / (kResRank / 2), jj = t % (kResRank / 2);
        int tok = d[0];
#pragma unroll
        for (int q = 1; q < RB; ++q)
          if (rr == q) tok = d[q];
        if (rr < B && jj < r / 2) ev = reinterpret_cast<const uint32_t*>(a.E)[(size_t)tok * (r / 2) + jj];
      }
      load_base(k + 1);
    }
    store_stat();
    if (k + 1 < K) {
      if (e_thr) lds_e[t] = ev;   // row t / 128, pair t % 128
      __syncthreads();
    }
  }
  res_retire(a.ex, g, G, B, K, 0, cpar, t, kResThreads);
}

// ---------------------------------------------------------------------------
// Resident path, MFMA form (2 < B <= 128). Same block structure as the VALU
// resident kernel: one persistent launch, one workgroup per CU owning up to
// 784 columns, W on chip for the whole block; here 256 threads, one wave per
// SIMD with all 512 registers of a lane. The slice is held as bf16 A-operand
// fragments of v_mfma_f32_16x16x32_bf16 (A = W^T: 16 columns x 32 rank rows;
// lane l holds column l % 16, rank rows 8 (l / 16) .. + 7): M-tiles 0..31 in
// registers (eight per wave, their fragments in AGPRs), 32..48 in LDS. The B
// operand is the embedding rows of one N-tile of 16 rows, staged in LDS
// (double-buffered) and held in registers while every M-tile of the wave
// uses it. The accumulator leaves each lane 4 consecutive columns of one row
// (rows 4 (l / 16) .. + 3 of D = columns, column l % 16 of D = row), the
// epilogue's shape: one Philox block per lane.
// Positions are separated by a two-level exchange: every workgroup publishes
// one tagged word per row; the workgroup owning a row reduces its G words and
// publishes the row's tagged winner; every workgroup reads the B winners.
// ---------------------------------------------------------------------------
constexpr int kMfThreads = 256;                            // one wave per SIMD: 512 registers a lane
constexpr int kMfWaves = kMfThreads / 64;
constexpr int kMfTilesPerWave = 8;                         // VGPR M-tiles per wave (256 registers)
constexpr int kMfRegTiles = kMfWaves * kMfTilesPerWave;    // 32
constexpr int kMfLdsTiles = kResSlice / 16 - kMfRegTiles;  // 17
constexpr int kMfLdsPerWave = (kMfLdsTiles + kMfWaves - 1) / kMfWaves;   // 5
constexpr int kMfTilesMax = kMfTilesPerWave + kMfLdsPerWave;            // 13
constexpr int kMfKSteps = kResRank / 32;                   // 8
constexpr int kMfAhead = 5;                                // base logits loaded this many tiles ahead (B=88: -4 us against 4)
constexpr int kMfNextAt = kMfTilesMax - kMfAhead;          // the last kMfAhead tiles load the next N-tile's first bases
constexpr int kMfRowsMax = 128;                            // 8 N-tiles of 16 rows
constexpr int kMfERow = 528;                               // bytes per staged E row: 512 + 16 (16-byte aligned rows; 16 lanes of one 128-bit read cover all banks)
constexpr int kMfSinkFloats = 1024;                        // sink: stores of lanes without a row or column
constexpr size_t kMfLdsW = (size_t)kMfLdsTiles * kMfKSteps * 64 * 16;   // 139,264 bytes
constexpr size_t kMfLdsE = (size_t)2 * 16 * kMfERow;                    // 16,896 bytes
constexpr size_t kMfLdsBytes = kMfLdsW + kMfLdsE;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Register-resident W fragments are defined in AGPRs by an empty asm whose
// output is tied to its input with the AGPR constraint. The instruction reads
// its A operand from either register file, so the builtin then takes them
// straight from AGPRs; without this the register allocator parks them in
// AGPRs on its own and copies each one back to VGPRs before every use (four
// VALU moves per instruction).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4_t in_agpr(u32x4_t v) {
  u32x4_t r;
  asm volatile("; W fragment kept in AGPRs %0" : "=a"(r) : "0"(v));
  return r;
}
// The same for a fragment loaded from memory: not volatile, so the scheduler
// may issue every load before the first of these (a volatile one would keep
// each load's wait in program order: one memory round trip per fragment).
__device__ __forceinline__ u32x4_t in_agpr_loaded(u32x4_t v) {
  u32x4_t r;
  asm("; W fragment kept in AGPRs %0" : "=a"(r) : "0"(v));
  return r;
}
__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// The bias chain of one LDS M-tile, issued from the epilogue's hooks: step J
// runs the matrix instruction of K-step J and reads the A fragment of K-step
// J + 2 into the registers that instruction has just taken as its A operand
// (A and B are consumed at issue: the compiler's hazard model, which sees
// these builtins, requires no wait states for that rewrite, only for the
// accumulator). Two fragments are in flight, so each read has two stretches of VALU
// work to arrive in (with one in flight a tile carrying an LDS chain took
// ~1150 cycles against ~780 for a tile whose chain reads registers; with two,
// ~940). Fences keep the scheduler from gathering the
// reads and multiplies back into one read-wait-multiply run ahead of the
// epilogue (the register pressure here leaves it no room to overlap them).
struct LdsChain {
  const unsigned char* fb;   // this lane's fragment of K-step 0; K-steps are 1 KB apart
  uint4 e[kMfKSteps];        // B fragments
  u32x4_t fr0, fr1;          // A fragments in flight: even and odd K-steps
  f32x4_t an;
  __device__ __forceinline__ u32x4_t frag(int ks) const { return *reinterpret_cast<const u32x4_t*>(fb + ks * 1024); }
  __device__ __forceinline__ void start() {
    fr0 = frag(0);
    fr1 = frag(1);
    an = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  template <int J>
  __device__ __forceinline__ void step() {
    __builtin_amdgcn_sched_barrier(0);
    if constexpr ((J & 1) == 0) {
      an = mfma_bf16(fr0, e[J], an);
      if constexpr (J + 2 < kMfKSteps) fr0 = frag(J + 2);
    } else {
      an = mfma_bf16(fr1, e[J], an);
      if constexpr (J + 2 < kMfKSteps) fr1 = frag(J + 2);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
};

// ---------------------------------------------------------------------------
// Packed W. W is a weight: the same for every block. dspark_pack_w writes it
// once in the order in which the two resident kernels hold it on chip, one
// contiguous block of 401,408 bytes per workgroup and kernel, so that each
// kernel's setup is one coalesced stream (and its LDS part a linear copy by
// LDS-direct loads) instead of 16-byte pieces from 256 rank rows 400 KB apart.
// Region 0, the small-batch kernel (slice a multiple of 8 columns): 32 x 512
// units, unit (i, t) = thread t's 16 bytes of its W pairs, i = 2 p + h (pair
// p, columns 4h .. 4h + 3 of the thread's 8), then the LDS image [16][272][8]
// dwords. Region 1, the MFMA kernel (slice a multiple of 16): 64 x 256 units,
// unit (f, t) = thread t's A fragment f = 8 mt + ks, then the LDS-tile image
// [17][8][64] fragments. A fragment of M-tile T, K-step ks, lane L holds the 8
// bf16 of column 16 T + L % 16, rank rows 32 ks + 8 (L / 16) .. + 7; a pair
// dword rows 2p (low half) and 2p + 1. Past the rank or the slice: zeros.
static_assert(kMfTilesPerWave * kMfKSteps * kMfThreads == kPackRegU4, "MFMA register units");
static_assert((size_t)kPackRegU4 * 16 + kMfLdsW == kPackWgU4 * 16, "MFMA block size");

struct PackArgs {
  const uint16_t* W;   // [r, V]
  uint4* out;          // [2][G][kPackWgU4]
  int V, r, G, slice8, slice16;
};

__device__ __forceinline__ uint32_t packed_w_at(const PackArgs& a, int row, int col0, int ncols, int c) {
  return (row < a.r && c < ncols) ? (uint32_t)a.W[(size_t)row * a.V + col0 + c] : 0u;
}

__global__ __launch_bounds__(256) void pack_w(PackArgs a) {
  const size_t per = (size_t)a.G * kPackWgU4;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= 2 * per) return;
  const bool mf = idx >= per;
  const size_t j = mf ? idx - per : idx;
  const int g = (int)(j / kPackWgU4), x = (int)(j % kPackWgU4);
  uint32_t d[4];
  if (!mf) {
    const int col0 = g * a.slice8, ncols = max(0, min(a.slice8, a.V - col0));
    int js, cg, pr, h;
    if (x < kPackRegU4) {            // thread t's VGPR unit: rank slice t % 8, column group 8 (t / 64) + t % 64 / 8
      const int i = x / kResThreads, t = x % kResThreads;
      js = t & 7; cg = 8 * (t >> 6) + ((t & 63) >> 3); pr = i >> 1; h = i & 1;
    } else {                         // LDS unit u: rank slice u % 8, column group 64 + u / 8
      const int y = x - kPackRegU4, u = (y % (2 * kResLdsUnits)) >> 1;
      pr = y / (2 * kResLdsUnits); h = y & 1; js = u & 7; cg = kResRegGroups + (u >> 3);
    }
    const int row = 32 * js + 2 * pr;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int c = 8 * cg + 4 * h + jj;
      d[jj] = packed_w_at(a, row, col0, ncols, c) | (packed_w_at(a, row + 1, col0, ncols, c) << 16);
    }
  } else {
    const int col0 = g * a.slice16, ncols = max(0, min(a.slice16, a.V - col0));
    int T, ks, L;
    if (x < kPackRegU4) {            // thread t's fragment f: M-tile 8 (t / 64) + f / 8, K-step f % 8
      const int f = x / kMfThreads, t = x % kMfThreads;
      T = kMfTilesPerWave * (t >> 6) + f / kMfKSteps; ks = f % kMfKSteps; L = t & 63;
    } else {                         // LDS-tile fragment: M-tile 32 + fr / 8, K-step fr % 8
      const int y = x - kPackRegU4, fr = y >> 6;
      L = y & 63; T = kMfRegTiles + fr / kMfKSteps; ks = fr % kMfKSteps;
    }
    const int c = 16 * T + (L & 15), row = 32 * ks + 8 * (L >> 4);
#pragma unroll
    for (int e2 = 0; e2 < 4; ++e2)
      d[e2] = packed_w_at(a, row + 2 * e2, col0, ncols, c) | (packed_w_at(a, row + 2 * e2 + 1, col0, ncols, c) << 16);
  }
  a.out[idx] = make_uint4(d[0], d[1], d[2], d[3]);
}

struct MfArgs {
  const void* base;
  const uint16_t* E;
  const uint16_t* W;
  const int32_t* prev_token;
  const int64_t* seed;
  const int64_t* offset;
  const float* temperature;
  const int32_t* n_real;
  float* logits;
  int32_t* tokens;
  ResExchange* ex;     // the device's exchange state (arrivals, failure record, retire)
  uint64_t* xrow;      // ex->xrow, ex->xwin and ex->zeros, passed as their own arguments
  uint64_t* xwin;      // (derived from ex inside the N-tile loop they cost scalar registers
  const void* zeros;   // that were spilled to vector lanes and reloaded every tile)
  Stat* stat_part;     // [K][B][G]
  float* sink;         // [kMfSinkFloats] stores of lanes without a real row or column
  const u32x4_t* Wp;   // packed W, this kernel's layout (kPacked), else unused
  int B, K, V, r, slice;
  unsigned spin_limit; // reads of a word before its wait expires (0: expires at once)
};

// Row state kept in LDS for the whole launch (temperature, slot, padding).
struct MfRow {
  float invT;            // 1/T; 1 for greedy rows
  uint32_t flags;        // bit 0: greedy, bit 1: padding
  uint32_t key0, key1, ctr2, ctr3;
};

// Stage the embedding rows of N-tile nt (16 rows x 512 bytes) into an LDS
// buffer: thread t copies 32 bytes (row t / 16, bytes 32 (t % 16) ..) of E[d[row]].
// Rows beyond the batch and rank rows beyond r load a valid address and are
// zeroed when stored (not when loaded: overwriting a register with a load in
// flight would make the wave wait for it).
struct ERow2 {
  uint4 lo, hi;
  bool ok;
};

// Running argmax of one lane's perturbed scores, visited in increasing column
// order: only a strictly larger score replaces the best, so ties keep the
// lowest column, and NaN (never larger) never wins. kNoCol marks "empty"; the
// first ordered score (even -inf) fills it.
constexpr uint32_t kNoCol = 0xFFFFFFFFu;
struct Best {
  float z;
  uint32_t v;
};

// c ? a : b as a bit select (v_bfi), which the compiler keeps as straight-line
// code instead of turning it into a branch around the costlier operand
__device__ __forceinline__ uint32_t usel(bool c, uint32_t a, uint32_t b) {
  const uint32_t m = 0u - (uint32_t)c;
  return (a & m) | (b & ~m);
}
__device__ __forceinline__ float fsel(bool c, float a, float b) {
  return __uint_as_float(usel(c, __float_as_uint(a), __float_as_uint(b)));
}

__device__ __forceinline__ void best_update4(Best& b, const float z[4], uint32_t v0) {
  const float m = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));   // NaN only if all four are
  uint32_t j = usel(z[2] == m, 2u, 3u);
  j = usel(z[1] == m, 1u, j);
  j = usel(z[0] == m, 0u, j);
  const bool take = (m > b.z) | ((b.v == kNoCol) & (m == m));
  b.z = fsel(take, m, b.z);
  b.v = usel(take, v0 + j, b.v);
}

__device__ __forceinline__ uint64_t best_key(const Best& b) { return b.v == kNoCol ? 0ull : score_key(b.z, b.v); }

// Online softmax statistics of one lane, accumulated in base 2: after each
// group of 4 scores, l = sum over the lane's scores of 2^(s L - M) with m
// their running maximum, L = log2(e) rounded to float and M = fl(m L); each
// term is one fma and one v_exp. stat_to_natural turns (m, l) into the usual
// form sum exp(s - m) = l 2^(M - m L), exactly up to a few ulp.
constexpr float kLog2e = 1.44269504f;
__device__ __forceinline__ void run_update4(Stat& st, const float s[4]) {
  const float m4 = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  const float mn = fmaxf(st.m, m4);
  const float mr = mn == -INFINITY ? 0.0f : mn;   // nothing finite yet: every term is 0
  const float Mr = __fmul_rn(mr, kLog2e);
  float l = __fmul_rn(st.l, __builtin_amdgcn_exp2f(__fsub_rn(__fmul_rn(st.m, kLog2e), Mr)));
#pragma unroll
  for (int i = 0; i < 4; ++i) l = __fadd_rn(l, __builtin_amdgcn_exp2f(__fmaf_rn(s[i], kLog2e, -Mr)));
  st = Stat{mn, l};
}

// d = m L - M is the rounding error of M (found exactly by the fma); 2^-d is
// 1 - d ln2 to far below float precision (|d| <= ulp(M) / 2).
__device__ __forceinline__ Stat stat_to_natural(Stat st) {
  if (!(st.l > 0.0f)) return st;
  const float M = __fmul_rn(st.m, kLog2e);
  const float d = __fmaf_rn(st.m, kLog2e, -M);
  return Stat{st.m, __fmaf_rn(st.l, __fmul_rn(-d, 0.693147182f), st.l)};
}

// log2(-log2 u) for u = ((x >> 9) + 1/2) 2^-23 of a Philox word x, with the
// hardware base-2 logarithm; the Gumbel variate is g = -ln(-ln u) =
// -ln2 * log2(-log2 u) - ln(ln 2). u is formed from bits: the float with
// exponent 0 and mantissa x >> 9 (one alignbit) is 1 + (x >> 9) 2^-23, and
// subtracting 1 - 2^-24 from it is exact, giving the same u as the integer
// conversion.
__device__ __forceinline__ float gumbel_log2(uint32_t x) {
  const float f = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, x, 9));
  const float u = __fsub_rn(f, 0x1.fffffep-1f);
  return __builtin_amdgcn_logf(-__builtin_amdgcn_logf(u));
}

// This lane's row of one (position, N-tile): its Philox slot, the scale 1/T and
// the Gumbel coefficient (greedy rows: 1 and 0, which makes the perturbed
// score the logit itself), where its base logits are read (a zeroed region
// for padding rows and for rows past the batch) and where its logits go (the
// sink for rows past the batch).
struct MfLane {
  float invT, gco;
  uint32_t key0, key1, ctr2, ctr3;
  const unsigned char* bp;   // base logits of (row, position, first column of the slice)
  float* op;                 // logits of the same
};

// Epilogue of one MFMA output fragment: columns v0..v0+3 of one row; returns
// the float32 logits (the caller stores them). Straight-line code (no branch
// on the row kind), so the whole tile is one basic block that the scheduler
// can interleave with the matrix instructions of the next tile. The ranked
// score is z = s + gco * log2(-log2 u): with gco = -ln 2 that is s + g + ln(ln 2)
// for the Gumbel variate g, a shift by one constant for the whole row, so the
// argmax is that of s + g. kRagged (a vocabulary that is not a multiple of 16):
// fragments without real columns (ok false) take part as scores that never win
// (NaN) and softmax terms that are 0. The statistics of greedy rows are not used.
// hook.step<J>(), J = 0..7, runs at eight points spread over the epilogue's work.
template <bool kBf16Base, bool kRagged, class Hook>
__device__ __forceinline__ float4 mf_epilogue(const MfLane& L, int k, uint32_t v0, const Base4<kBf16Base>& bv,
                                              f32x4_t acc, bool ok, Best& best, Stat& st, Hook& hook) {
  float base[4];
  widen_base4<kBf16Base>(bv, base);
  const uint4 x = philox4x32_10_hooked(make_uint4(v0 >> 2, (uint32_t)k, L.ctr2, L.ctr3), L.key0, L.key1, hook);
  const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
  float lg[4], s[4], z[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lg[i] = __fadd_rn(base[i], acc[i]);
    s[i] = __fmul_rn(lg[i], L.invT);
    z[i] = __fmaf_rn(gumbel_log2(xs[i]), L.gco, s[i]);
    if (kRagged) {
      z[i] = fsel(ok, z[i], __builtin_nanf(""));
      s[i] = fsel(ok, s[i], -INFINITY);
    }
    if (i == 1) hook.template step<5>();
  }
  hook.template step<6>();
  best_update4(best, z, v0);
  hook.template step<7>();
  run_update4(st, s);
  return make_float4(lg[0], lg[1], lg[2], lg[3]);
}

struct ERowSrc {
  const uint16_t* src;
  bool ok;
};

__device__ __forceinline__ ERowSrc mf_erow_src(const MfArgs& a, const int* s_d, int nt, int t_in) {
  // Row and LDS addresses are recomputed from an opaque copy of the thread
  // index at every use. Kept live across the position loop they were spilled
  // to scratch, and the reload's wait (vmcnt 0) at the start of every
  // position also waited for all logit stores still in flight.
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"(t_in));
  const int row = 16 * nt + t / 16, j16 = 16 * (t % 16);
  const bool ok = row < a.B && j16 < a.r;
  return ERowSrc{a.E + (ok ? (size_t)s_d[row] * a.r + j16 : 0), ok};
}

// The same with the row's token given (d of this thread's row of N-tile nt,
// valid wherever the row exists).
__device__ __forceinline__ ERowSrc mf_erow_src_tok(const MfArgs& a, int tok, int nt, int t_in) {
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"(t_in));
  const int row = 16 * nt + t / 16, j16 = 16 * (t % 16);
  const bool ok = row < a.B && j16 < a.r;
  return ERowSrc{a.E + (ok ? (size_t)tok * a.r + j16 : 0), ok};
}

__device__ __forceinline__ ERow2 mf_load_erow(const ERowSrc& es) {
  return ERow2{*reinterpret_cast<const uint4*>(es.src), *reinterpret_cast<const uint4*>(es.src + 8), es.ok};
}

__device__ __forceinline__ ERow2 mf_load_erow(const MfArgs& a, const int* s_d, int nt, int t) {
  return mf_load_erow(mf_erow_src(a, s_d, nt, t));
}

__device__ __forceinline__ void mf_store_erow(unsigned char* ebuf, int t, const ERow2& v) {
  const uint32_t m = v.ok ? ~0u : 0u;
  uint4* dst = reinterpret_cast<uint4*>(ebuf + (t / 16) * kMfERow + 32 * (t % 16));
  dst[0] = make_uint4(v.lo.x & m, v.lo.y & m, v.lo.z & m, v.lo.w & m);
  dst[1] = make_uint4(v.hi.x & m, v.hi.y & m, v.hi.z & m, v.hi.w & m);
}

template <bool kBf16Base, bool kRagged, bool kPacked>
__global__ __launch_bounds__(kMfThreads, 1) void markov_bias_gumbel_argmax_resident_mfma(MfArgs a) {
  extern __shared__ __align__(16) unsigned char mf_lds[];
  unsigned char* lds_w = mf_lds;                         // [17][8][64][16 B] fragments
  unsigned char* lds_e = mf_lds + kMfLdsW;               // [2][16][kMfERow]
  __shared__ uint64_t s_rk[2][kMfWaves][16];             // per-wave row partials, by N-tile parity
  __shared__ Stat s_rs[2][kMfWaves][16];
  __shared__ MfRow s_row[kMfRowsMax];
  __shared__ int s_d[kMfRowsMax];                        // previous token per row
  __shared__ int s_fail;
  __shared__ unsigned long long s_call;

  const int t = threadIdx.x, lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);   // wave-uniform
  const int g = blockIdx.x, G = gridDim.x;
  unsigned long long call0 = 0;
  if (t == 0) call0 = res_arrive(a.ex, G);
  const int V = a.V, r = a.r, K = a.K, B = a.B;
  const int NT = (B + 15) / 16;
  const int col0 = g * a.slice;
  const int ncols = max(0, min(a.slice, V - col0));
  const int n_real = a.n_real ? *a.n_real : B;
  const int lr = lane & 15;           // row of an N-tile / column of an M-tile
  const int lq = lane >> 4;           // quad: rank rows 8 lq .. of a K-step; columns 4 lq .. of D

  if (t == 0) s_fail = 0;
  for (int b = t; b < B; b += kMfThreads) {
    const RowState rs = row_state(a.temperature, a.seed, a.offset, b, n_real);
    s_row[b] = MfRow{rs.greedy ? 1.0f : rs.invT, (rs.greedy ? 1u : 0u) | (rs.pad ? 2u : 0u), rs.key0, rs.key1,
                     rs.ctr2, rs.ctr3};
    s_d[b] = clamp_token(a.prev_token[b], V);
  }


  // ---- (1) VGPR M-tiles 8w..8w+7, in two rounds of four K-steps. In each,
  // rank rows 128 h .. 128 h + 127 of the slice's first 512 columns are copied
  // into the (not yet used) LDS-tile region by LDS-direct loads (one 1 KB row
  // per wave instruction, lane i's 16 bytes at 16 i; no registers hold the
  // data), rows past the rank and columns past the slice from the zeroed
  // region; then every wave gathers its A fragments from there (lane l:
  // column l % 16 of the tile, rank rows 8 (l / 16) .. + 7).
  u32x4_t wf[kMfTilesPerWave][kMfKSteps];   // A fragments, kept in AGPRs
  if constexpr (kPacked) {
    // packed W: thread t's fragment f = 8 mt + ks is unit (f, t) of this
    // workgroup's block (256 x 16 B per instruction); the LDS-tile image
    // follows it, copied by LDS-direct loads (each wave instruction 1 KB, lane
    // i's 16 bytes at 16 i), issued first (they need no registers) and waited
    // for before the barrier below
    const u32x4_t* src = a.Wp + (size_t)g * kPackWgU4 + t;
    unsigned char* dst = lds_w + (size_t)64 * wv * 16;
#pragma unroll
    for (int j = 0; j < (int)(kMfLdsW / 16 / kMfThreads); ++j)
      __builtin_amdgcn_global_load_lds((lds_gptr_t)(src + kPackRegU4 + (size_t)j * kMfThreads),
                                       (lds_lptr_t)(dst + (size_t)j * kMfThreads * 16), 16, 0, 0);
    // the two fragments that stay in VGPRs first, then the 62 kept in AGPRs
    constexpr int kLastMt = kMfTilesPerWave - 1;
#pragma unroll
    for (int ks = kMfKSteps - 2; ks < kMfKSteps; ++ks)
      wf[kLastMt][ks] = src[(size_t)(kLastMt * kMfKSteps + ks) * kMfThreads];
#pragma unroll
    for (int mt = 0; mt < kMfTilesPerWave; ++mt)
#pragma unroll
      for (int ks = 0; ks < kMfKSteps; ++ks)
        if (!(mt == kLastMt && ks >= kMfKSteps - 2))
          wf[mt][ks] = in_agpr_loaded(src[(size_t)(mt * kMfKSteps + ks) * kMfThreads]);
  } else {
    constexpr int kStageRow = 2 * 16 * kMfRegTiles + 16;       // bytes per staged row (1 KB + pad)
    constexpr int kRoundRows = kResRank / 2;                   // 128
    constexpr int kRowsPerWave = kRoundRows / kMfWaves;        // 32
    static_assert((size_t)kRoundRows * kStageRow <= kMfLdsW, "staging fits the LDS-tile region");
    const uint16_t* st16 = reinterpret_cast<const uint16_t*>(lds_w);
    const int c8 = 8 * lane;                                   // this lane's 8 columns of a staged row
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll 8
      for (int i = 0; i < kRowsPerWave; ++i) {
        const int rl = kRowsPerWave * wv + i, row = kRoundRows * h + rl;
        const bool ok = row < r && c8 < ncols;
        const uint16_t* src = ok ? a.W + (size_t)row * V + col0 + c8
                                 : static_cast<const uint16_t*>(a.zeros) + c8;
        __builtin_amdgcn_global_load_lds((lds_gptr_t)src, (lds_lptr_t)(lds_w + (size_t)rl * kStageRow), 16, 0, 0);
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0) (expcnt, lgkmcnt not waited): every row of this wave has landed
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kMfKSteps / 2; ++kk) {
        const int ks = (kMfKSteps / 2) * h + kk;
#pragma unroll
        for (int mt = 0; mt < kMfTilesPerWave; ++mt) {
          const int col = 16 * (kMfTilesPerWave * wv + mt) + lr;
          uint32_t d[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int rr = 32 * kk + 8 * lq + 2 * e;   // staged row of rank row 32 ks + 8 lq + 2 e
            const uint32_t lo = st16[(rr * kStageRow) / 2 + col];
            const uint32_t hi = st16[((rr + 1) * kStageRow) / 2 + col];
            d[e] = lo | (hi << 16);
          }
          // 62 fragments and the two 4-register accumulators fill the 256
          // AGPRs exactly; the last two fragments stay ordinary VGPR values
          // (left to the allocator, it moves two of its own choosing and has
          // at times spilled one to scratch instead)
          const u32x4_t f = u32x4_t{d[0], d[1], d[2], d[3]};
          wf[mt][ks] = (mt == kMfTilesPerWave - 1 && ks >= kMfKSteps - 2) ? f : in_agpr(f);
        }
      }
      __syncthreads();   // the staging area is overwritten next
    }

    // ---- (2) LDS M-tiles 32..48: each 16-byte load (8 columns of one rank row)
    // is scattered into the fragment layout (element e of lane l at byte l*16 + 2e).
    // Consecutive threads take consecutive rank rows (so the 2-byte stores of a
    // wave spread over the LDS banks); each thread issues its loads in batches
    // of 17 before storing any (one memory latency per batch, not per item).
    // Beyond the rank or the slice a valid address is read and the value zeroed
    // when stored.
    {
      constexpr int kItems = kMfLdsTiles * kResRank * 2;         // 8704
      constexpr int kPerThread = kItems / kMfThreads;            // 34
      constexpr int kBatch = 17;
      static_assert(kItems % kMfThreads == 0 && kPerThread % kBatch == 0, "item split");
#pragma unroll
      for (int b0 = 0; b0 < kPerThread; b0 += kBatch) {
        uint4 v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int q = t + (b0 + u) * kMfThreads;
          const int ti = q / (kResRank * 2), rem = q % (kResRank * 2);
          const int j = rem / 2, h = rem % 2;
          const int c8 = 16 * (kMfRegTiles + ti) + 8 * h;
          const bool ok = j < r && c8 < ncols;
          v[u] = *reinterpret_cast<const uint4*>(a.W + (ok ? (size_t)j * V + col0 + c8 : 0));
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int q = t + (b0 + u) * kMfThreads;
          const int ti = q / (kResRank * 2), rem = q % (kResRank * 2);
          const int j = rem / 2, h = rem % 2;
          const int c8 = 16 * (kMfRegTiles + ti) + 8 * h;
          const uint32_t m = (j < r && c8 < ncols) ? ~0u : 0u;
          const uint32_t w4[4] = {v[u].x & m, v[u].y & m, v[u].z & m, v[u].w & m};
          unsigned char* frag = lds_w + ((size_t)ti * kMfKSteps + j / 32) * 1024;
          const int lbase = 8 * h + 16 * ((j % 32) / 8);
#pragma unroll
          for (int c = 0; c < 8; ++c) {
            const uint16_t val = (uint16_t)(w4[c / 2] >> (16 * (c % 2)));
            *reinterpret_cast<uint16_t*>(frag + (lbase + c) * 16 + 2 * (j % 8)) = val;
          }
        }
      }
    }
  }

  if constexpr (kPacked) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's LDS-direct loads have landed
  __syncthreads();

  // ---- (3) the E rows of N-tiles 0 and 1 of position 0. Every N-tile nt
  // stores the rows of nt + 1 (held in epre) into the other buffer and
  // prefetches nt + 2; rows past the batch are zeros, so the schedule has no
  // branches. At a position start epre is stored at once as well, so no load
  // is in flight in it when the first N-tile stores it again.
  ERow2 epre;
  {
    const ERow2 e0 = mf_load_erow(a, s_d, 0, t);   // both loads in flight before either store
    epre = mf_load_erow(a, s_d, 1, t);
    mf_store_erow(lds_e, t, e0);
    mf_store_erow(lds_e + 16 * kMfERow, t, epre);
  }
  if (t == 0) s_call = call0;

  // the wave's tiles: i < 8 are VGPR tiles 8 wv + i; i >= 8 are LDS tiles 32 + wv + 4 (i - 8)
  auto tile_m = [&](int i) {
    return i < kMfTilesPerWave ? kMfTilesPerWave * wv + i : kMfRegTiles + wv + kMfWaves * (i - kMfTilesPerWave);
  };
  int n_mine = 0;   // tiles with columns in this slice
  for (int i = 0; i < kMfTilesMax; ++i) {
    const int m = tile_m(i);
    if ((i < kMfTilesPerWave || m < kMfRegTiles + kMfLdsTiles) && 16 * m < ncols) n_mine = i + 1;
  }

  // this lane's row of (position k, N-tile nt)
  constexpr int kEsz = kBf16Base ? 2 : 4;   // bytes per base logit
  auto lane_base = [&](int k, int nt) -> const unsigned char* {
    const int b = 16 * nt + lr;
    const bool read = k < K && b < B && !(s_row[b].flags & 2u);
    return read ? static_cast<const unsigned char*>(a.base) + (((size_t)b * K + k) * (size_t)V + col0) * kEsz
                : static_cast<const unsigned char*>(a.zeros);
  };
  auto lane_row = [&](int k, int nt, const unsigned char* bp) {
    MfLane L;
    const int b = 16 * nt + lr;
    const bool real = b < B;
    const MfRow mr = s_row[real ? b : 0];
    L.invT = mr.invT;
    L.gco = (mr.flags & 1u) ? 0.0f : -0.693147182f;
    L.key0 = mr.key0; L.key1 = mr.key1; L.ctr2 = mr.ctr2; L.ctr3 = mr.ctr3;
    L.bp = bp;
    L.op = real ? a.logits + ((size_t)b * K + k) * (size_t)V + col0 : a.sink;
    return L;
  };
  // base logits of tile i of a lane row (its first column when the tile has
  // none here: a valid address, the value unused)
  auto base_at = [&](const unsigned char* bp, int i) -> const void* {
    const int c4 = 16 * tile_m(i) + 4 * lq;
    const bool has = i < n_mine && (!kRagged || c4 < ncols);
    return bp + (has ? c4 : 0) * kEsz;
  };
  // the bias fragment of VGPR tile i < 8 (rank rows >= r are zero in both operands, so all
  // 8 K-steps run); the chains of LDS tiles are issued from the epilogue's hooks
  auto tile_bias = [&](int i, const uint4 (&ef)[kMfKSteps]) {
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < kMfKSteps; ++ks) acc = mfma_bf16(wf[i][ks], ef[ks], acc);
    return acc;
  };

  __syncthreads();
  // the call's parity, wave-uniform (a scalar register); the full index is
  // read from LDS only where a wait expires
  const uint32_t cpar = __builtin_amdgcn_readfirstlane((uint32_t)s_call & 1u);

  // Combine the waves' partials of N-tile nt and publish each row's tagged
  // word. Wave 1 does it (wave 0 may own one more tile than the others):
  // lane = row (lane % 16) x wave (lane / 16), merged over the 4 rows of lanes.
  auto publish = [&](int k, int nt) {
    // after a failed wait nothing more is published (the workgroup's rows may
    // be computed from an unknown token): every wait for its words expires
    if (wv == 1 && !s_fail) {
      // the lane's row is taken through an opaque instruction, so the address
      // arithmetic below is done here rather than hoisted out of the loops
      // (held across them it was spilled, and the reloads waited for every
      // logit store still in flight)
      int row;
      asm volatile("v_and_b32 %0, 15, %1" : "=v"(row) : "v"(lane));
      const int w = lane >> 4;
      uint64_t kk = s_rk[nt & 1][w][row];
      Stat ss = s_rs[nt & 1][w][row];
      row_merge4(kk, ss);
      const int b = 16 * nt + row;
      if (lane < 16 && b < B) {
        a.stat_part[((size_t)k * B + b) * G + g] = ss;
        const uint64_t idx = kk ? kResIdxMask - (uint64_t)key_token(kk) : 0ull;
        st_agent_u64(a.xrow + ((size_t)(k & 1) * kResMaxCUs + g) * kExRows + b, res_tag(cpar, k) | ((kk >> 32) << 18) | idx);
      }
    }
  };

  // ---- the exchange. Level 2, after a position's last N-tile: the owner of
  // row b (workgroup b, b + G, ...) reduces the G words of its row in wave 0
  // alone (each lane polls G / 64 of them, the first loads of a group of four
  // in flight together; no LDS, no barrier) and publishes the row's tagged
  // winner. A winner is published only when all G words were seen: a wait
  // that expires publishes nothing, so no workgroup can take a winner made of
  // part of the words.
  auto level2 = [&](int k) {
    if (wv != 0) return;
    const uint64_t tagw = res_tag(cpar, k);
    const uint64_t tag = tagw >> kResTagShift;
    const uint64_t* xr = a.xrow + (size_t)(k & 1) * kResMaxCUs * kExRows;
    uint64_t* xw = a.xwin + (size_t)(k & 1) * kExRows;
    bool failed = false;
    for (int b = g; b < B; b += G) {
      uint64_t x = 0;
      bool lfail = a.spin_limit == 0;
      for (int i0 = lane; i0 < G && !lfail; i0 += 4 * 64) {
        // the words still missing are reloaded together: one round trip per pass
        uint64_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[q] = i0 + 64 * q < G ? ld_agent_u64(xr + (size_t)(i0 + 64 * q) * kExRows + b) : tagw;
        for (unsigned reads = 1;; ++reads) {
          bool all = true;
#pragma unroll
          for (int q = 0; q < 4; ++q) all = all && (w[q] >> kResTagShift) == tag;
          if (all) break;
          if (reads >= a.spin_limit) { lfail = true; break; }
          __builtin_amdgcn_s_sleep(1);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if ((w[q] >> kResTagShift) != tag) w[q] = ld_agent_u64(xr + (size_t)(i0 + 64 * q) * kExRows + b);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) x = umax64(x, w[q]);
      }
      x = wave_max_u64(x);
      const bool wave_failed = __ballot(lfail) != 0ull;
      failed = failed || wave_failed;
      if (lane == 0 && !wave_failed) st_agent_u64(xw + b, tagw | (x & ((1ull << kResTagShift) - 1)));
    }
    if (failed && lane == 0) s_fail = 1;
  };

  // Level 3: d_{k-1} of this thread's row of N-tile nt (16 threads a row, each
  // reading the row's winner word; one request per row), taken when the E
  // rows of that N-tile are prefetched: the previous tokens at k = 0, else the
  // row's winner of position k - 1. Workgroup 0 also writes it to tokens. A
  // wait that expires marks the workgroup failed and gives token 0 (a valid
  // address; the workgroup leaves at its next barrier).
  auto row_tok = [&](int k, int nt) -> int {
    int tt;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tt) : "v"(t));
    const int row = 16 * nt + tt / 16;
    if (row >= B) return 0;
    if (k == 0) return s_d[row];
    if (s_fail) return 0;   // failed already: no more waits
    const uint64_t tag = res_tag(cpar, k - 1) >> kResTagShift;
    const uint64_t* pw = a.xwin + (size_t)((k - 1) & 1) * kExRows + row;
    bool lfail = a.spin_limit == 0;
    uint64_t w = lfail ? 0 : ld_agent_u64(pw);
    for (unsigned reads = 1; !lfail && (w >> kResTagShift) != tag; ++reads) {
      if (reads >= a.spin_limit) { lfail = true; break; }
      __builtin_amdgcn_s_sleep(1);
      w = ld_agent_u64(pw);
    }
    if (lfail) {
      s_fail = 1;
      return 0;
    }
    const uint64_t low = w & ((1ull << kResTagShift) - 1);
    const int tok = low ? clamp_token((int)(kResIdxMask - (low & kResIdxMask)), V) : 0;
    if (g == 0 && tt % 16 == 0) a.tokens[(size_t)row * K + (k - 1)] = tok;
    return tok;
  };

  // A wait that expired (seen by every thread after a barrier): workgroup 0
  // marks positions k - 1 on (those whose tokens may be incomplete) with -1,
  // and every slot of this workgroup is rewritten with an unused tag of this
  // call.
  auto fail_exit = [&](int k) {
    if (t == 0) res_fail(a.ex, s_call);
    if (g == 0)
      for (int b = t; b < B; b += kMfThreads)
        for (int kk = k > 0 ? k - 1 : 0; kk < K; ++kk) a.tokens[(size_t)b * K + kk] = -1;
    res_retire(a.ex, g, G, B, 0, 0, cpar, t, kMfThreads);
  };

  // Base logits of each tile, one register set per tile (compile-time indices
  // after unrolling, so nothing is copied while a load is in flight): tile
  // i + kMfAhead is loaded during tile i, and the first kMfAhead tiles of the
  // next N-tile (or of the next position's first N-tile, which does not depend
  // on the token) during the last kMfAhead tiles.
  Base4<kBf16Base> bq[kMfTilesMax];
  const unsigned char* bp = lane_base(0, 0);   // base logits of this N-tile's row of the lane
#pragma unroll
  for (int i = 0; i < kMfAhead; ++i) load_base4<kBf16Base, false>(bq[i], base_at(bp, i), 0);

  for (int k = 0; k < K; ++k) {
    for (int nt = 0; nt < NT; ++nt) {
      // source of the E rows of N-tile nt + 2 (its rows' tokens of position
      // k - 1), read before the barrier so its latency overlaps the wait
      const ERowSrc es = mf_erow_src_tok(a, row_tok(k, nt + 2), nt + 2, t);
      __syncthreads();   // E buffer nt & 1 is complete; s_rk[(nt - 1) & 1] is complete
      if (nt > 0) publish(k, nt - 1);

      // B operand of this N-tile: lane = row lr, rank rows 32 ks + 8 lq ..
      uint4 ef[kMfKSteps];
      const unsigned char* eb = lds_e + (nt & 1) * 16 * kMfERow + lr * kMfERow + 16 * lq;
#pragma unroll
      for (int ks = 0; ks < kMfKSteps; ++ks) ef[ks] = *reinterpret_cast<const uint4*>(eb + 64 * ks);
      // the other buffer was last read in N-tile nt - 1, before the barrier above
      mf_store_erow(lds_e + ((nt + 1) & 1) * 16 * kMfERow, t, epre);
      epre = mf_load_erow(es);

      // the lane's row here; only the base pointer of the next one is kept (for its prefetch)
      const MfLane L = lane_row(k, nt, bp);
      const unsigned char* bpn = nt + 1 < NT ? lane_base(k, nt + 1) : lane_base(k + 1, 0);
      Best best{-INFINITY, kNoCol};
      Stat st{-INFINITY, 0.0f};

      // the bias of tile i + 1 is issued to the matrix cores before the epilogue of tile i
      f32x4_t acc[2];
      acc[0] = tile_bias(0, ef);
#pragma unroll
      for (int i = 0; i < kMfTilesMax; ++i) {
        if (i + kMfAhead < kMfTilesMax) load_base4<kBf16Base, false>(bq[i + kMfAhead], base_at(bp, i + kMfAhead), 0);
        if (i >= kMfNextAt && i < kMfNextAt + kMfAhead)
          load_base4<kBf16Base, false>(bq[i - kMfNextAt], base_at(bpn, i - kMfNextAt), 0);
        // One store per tile, after the branch (to the sink when there is no
        // tile, row or column), keeps the compiler's count of memory
        // operations issued after each prefetch exact; the base registers are
        // consumed on both paths for the same reason. Inside the branch the
        // matrix instructions of tile i + 1 and the epilogue of tile i form
        // one basic block (the epilogue has no branches), so the scheduler
        // can interleave them.
        float* out = a.sink + 4 * lane;
        float4 lgv;
        if (i < n_mine) {
          const int c4 = 16 * tile_m(i) + 4 * lq;   // column offset in the slice
          const bool ok = !kRagged || c4 < ncols;
          out = ok ? L.op + c4 : a.sink + c4;
          const uint32_t v0 = (uint32_t)(col0 + c4);
          if (i + 1 < kMfTilesPerWave) {
            // the chain of tile i + 1 (W in AGPRs) runs on the matrix cores
            // while the epilogue of tile i issues: 8 x (one matrix
            // instruction, 18 VALU)
            acc[(i + 1) & 1] = tile_bias(i + 1, ef);
            NoHook none;
            lgv = mf_epilogue<kBf16Base, kRagged>(L, k, v0, bq[i], acc[i & 1], ok, best, st, none);
#pragma unroll
            for (int n = 0; n < kMfKSteps; ++n) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 18, 0);
            }
          } else if (i + 1 < kMfTilesMax) {
            // the chain of LDS tile i + 1 (a tile this wave does not have reads
            // a valid one; its results are not used), placed by hand: the
            // epilogue issues one matrix instruction at each of its eight
            // hooks and the next fragment read after it (the scheduler would
            // otherwise run read, wait, multiply eight times in a row before
            // the epilogue)
            const int ml = tile_m(i + 1) < kMfRegTiles + kMfLdsTiles ? tile_m(i + 1) - kMfRegTiles : 0;
            LdsChain ch;
            ch.fb = lds_w + (size_t)ml * kMfKSteps * 1024 + lane * 16;
#pragma unroll
            for (int ks = 0; ks < kMfKSteps; ++ks) ch.e[ks] = ef[ks];
            ch.start();
            lgv = mf_epilogue<kBf16Base, kRagged>(L, k, v0, bq[i], acc[i & 1], ok, best, st, ch);
            acc[(i + 1) & 1] = ch.an;
          } else {
            NoHook none;
            lgv = mf_epilogue<kBf16Base, kRagged>(L, k, v0, bq[i], acc[i & 1], ok, best, st, none);
          }
        } else {
          float bw[4];
          widen_base4<kBf16Base>(bq[i], bw);
          lgv = make_float4(bw[0], bw[1], bw[2], bw[3]);
        }
        *reinterpret_cast<float4*>(out) = lgv;
        __builtin_amdgcn_sched_barrier(0);
      }
      // lanes of one row (equal lane % 16) combine; lanes 0..15 hold the wave's partials
      uint64_t key = best_key(best);
      st = stat_to_natural(st);
      row_merge4(key, st);
      if (lane < 16) {
        s_rk[nt & 1][wv][lane] = key;
        s_rs[nt & 1][wv][lane] = st;
      }
      bp = bpn;
    }
    __syncthreads();
    if (s_fail) {
      fail_exit(k);
      return;
    }
    publish(k, NT - 1);
    // the owners' reductions: rows of the earlier N-tiles were published long
    // ago (no wait); only the owners of the last N-tile's rows wait for the
    // slowest workgroup, and nobody waits for them before N-tile NT - 3 of
    // the next position
    level2(k);
    if (k + 1 < K) {
      // E rows of the next position's N-tiles 0 and 1 (both loads in flight
      // before either store); the buffers were last read before the barrier above
      const ERow2 e0 = mf_load_erow(mf_erow_src_tok(a, row_tok(k + 1, 0), 0, t));
      epre = mf_load_erow(mf_erow_src_tok(a, row_tok(k + 1, 1), 1, t));
      mf_store_erow(lds_e, t, e0);
      mf_store_erow(lds_e + 16 * kMfERow, t, epre);
    }
  }
  // the last position's tokens (workgroup 0)
  if (g == 0)
    for (int nt = 0; nt < NT; ++nt) (void)row_tok(K, nt);
  __syncthreads();
  if (s_fail) {
    fail_exit(K);
    return;
  }
  res_retire(a.ex, g, G, B, K, K, cpar, t, kMfThreads);
}

// ---------------------------------------------------------------------------
// Standard token-level verification of a draft block ("brb-nv/TensorRT-LLM
// pull 21", section "2. Golden sampling semantics": rejection_sample_method
// standard, the default). The rule is the textbook one (Leviathan, Kalman and
// Matias, ICML 2023, section 2.3): accept d_k with probability
// min(1, p_k(d_k) / q_k(d_k)); at the first rejection emit a draw from
// max(0, p_k - q_k) normalised; if all K are accepted emit a bonus draw from
// p_K. Conventions (ratio in float32, the Philox counters of the uniforms and
// of the Gumbel noise, the fallback for an empty residual) are stated in
// include/dspark.h.
//
// Two launches, no counters (the workspace needs no initialisation):
// verify_partials, one block per (1024..8192-column chunk, row), streams the row
// the emitted token is drawn from (p_j and q_j, or p_K) once and leaves the
// chunk's best Gumbel-max key; verify_finish, one wave per row, merges them.
// Every wave finds the first rejected position itself: lane i tests position
// i (64 at a time) and a ballot picks the first failure.
// ---------------------------------------------------------------------------
constexpr int kVerColsMin = 4 * kThreads;   // columns per verify_partials block: 1024 x 1, 2, 4 or 8

struct VerArgs {
  const int32_t* draft;    // [B,K]
  const float* q;          // [B,K,V]
  const float* p;          // [B,K+1,V]
  const int64_t* seed;
  const int64_t* offset;
  uint64_t* part;          // [B][n_chunks]: best key of the draw's distribution
  int32_t* n_accepted;     // [B]
  int32_t* out_tokens;     // [B,K+1]
  int B, K, V, n_chunks;   // n_chunks = ceil(V / columns per block)
};

__device__ __forceinline__ uint4 verify_philox(uint64_t seed, uint64_t off, uint32_t x, uint32_t y) {
  return philox4x32_10(make_uint4(x, y, (uint32_t)off, (uint32_t)(off >> 32)), (uint32_t)seed,
                       (uint32_t)(seed >> 32));
}

// The first rejected position of row b (K if every draft is accepted); every
// lane of the wave gets it.
__device__ __forceinline__ int verify_first_reject(const VerArgs& a, int b) {
  const int lane = threadIdx.x & 63;
  const uint64_t seed = (uint64_t)a.seed[b], off = (uint64_t)a.offset[b];
  for (int k0 = 0; k0 < a.K; k0 += 64) {
    const int k = k0 + lane;
    bool reject = false;
    if (k < a.K) {
      const int d = clamp_token(a.draft[(size_t)b * a.K + k], a.V);
      const float pv = a.p[((size_t)b * (a.K + 1) + k) * a.V + d];
      const float qv = a.q[((size_t)b * a.K + k) * a.V + d];
      const float ratio = __fdiv_rn(pv, qv);
      const uint32_t x = verify_philox(seed, off, 0xFFFFFFFFu, 256u + (uint32_t)k).x;
      const float u = __fmul_rn(__fadd_rn((float)(x >> 9), 0.5f), 0x1p-23f);   // exact
      reject = !(u < ratio);
    }
    const uint64_t m = __ballot(reject);
    if (m) return k0 + __builtin_ctzll(m);
  }
  return a.K;
}

// kIt x 1024 columns per block: every thread issues all its loads (kIt
// float4 of p_j, and of q_j after a rejection) as soon as the position is
// known, then scores them. Only the draw's own distribution is scored; the
// fallback for an empty residual is left to verify_finish.
template <int kIt>
__global__ __launch_bounds__(kThreads) void verify_partials(VerArgs a) {
  __shared__ uint64_t s_k[kWaves];
  const int c = blockIdx.x, b = blockIdx.y, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int j = verify_first_reject(a, b);
  const bool residual = j < a.K;
  const float* pj = a.p + ((size_t)b * (a.K + 1) + j) * a.V;
  const float* qj = a.q + ((size_t)b * a.K + (residual ? j : 0)) * a.V;
  const uint64_t seed = (uint64_t)a.seed[b], off = (uint64_t)a.offset[b];
  const int c0 = c * (kIt * kVerColsMin) + 4 * t;
  // read once: nontemporal loads (B=88: 34.4 us against 36.7)
  fx4_t pv[kIt], qv[kIt];
#pragma unroll
  for (int i = 0; i < kIt; ++i) {
    const int v = c0 + i * kVerColsMin;
    pv[i] = v < a.V ? __builtin_nontemporal_load(reinterpret_cast<const fx4_t*>(pj + v)) : fx4_t{0.0f, 0.0f, 0.0f, 0.0f};
    qv[i] = (residual && v < a.V) ? __builtin_nontemporal_load(reinterpret_cast<const fx4_t*>(qj + v))
                                  : fx4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  uint64_t kw = 0;   // best key over w = max(0, p - q) (or p)
#pragma unroll
  for (int i = 0; i < kIt; ++i) {
    const int v = c0 + i * kVerColsMin;
    if (v >= a.V) break;
    const uint4 x = verify_philox(seed, off, (uint32_t)v >> 2, 512u);
    const float pe[4] = {pv[i].x, pv[i].y, pv[i].z, pv[i].w};
    const float qe[4] = {qv[i].x, qv[i].y, qv[i].z, qv[i].w};
    const uint32_t xe[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // base-2 form of ln w + g: log2 w - log2(-log2 u) (the same order)
      const float gl = gumbel_log2(xe[e]);
      const float w = residual ? __fsub_rn(pe[e], qe[e]) : pe[e];
      if (w > 0.0f) kw = umax64(kw, score_key(__fsub_rn(__builtin_amdgcn_logf(w), gl), (uint32_t)(v + e)));
    }
  }
  kw = wave_max_u64(kw);
  if (lane == 0) s_k[wv] = kw;
  __syncthreads();
  if (t == 0) {
    uint64_t m = s_k[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = umax64(m, s_k[w]);
    a.part[(size_t)b * a.n_chunks + c] = m;
  }
}

__global__ __launch_bounds__(64) void verify_finish(VerArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int n = verify_first_reject(a, b);
  uint64_t key = 0;
  for (int c = lane; c < a.n_chunks; c += 64) key = umax64(key, a.part[(size_t)b * a.n_chunks + c]);
  key = wave_max_u64(key);
  if (key == 0 && n < a.K) {
    // an empty residual (only through rounding, as p = q then): the draw
    // falls back to p_n, scored here by this one wave (slow, never on the
    // common path)
    const float* pn = a.p + ((size_t)b * (a.K + 1) + n) * a.V;
    const uint64_t seed = (uint64_t)a.seed[b], off = (uint64_t)a.offset[b];
    for (int v = 4 * lane; v < a.V; v += 4 * 64) {
      const float4 pv = *reinterpret_cast<const float4*>(pn + v);
      const uint4 x = verify_philox(seed, off, (uint32_t)v >> 2, 512u);
      const float pe[4] = {pv.x, pv.y, pv.z, pv.w};
      const uint32_t xe[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (pe[e] > 0.0f)
          key = umax64(key, score_key(__fsub_rn(__builtin_amdgcn_logf(pe[e]), gumbel_log2(xe[e])), (uint32_t)(v + e)));
    }
    key = wave_max_u64(key);
  }
  // no positive entry at all gives token 0
  const int tok = key ? clamp_token((int)key_token(key), a.V) : 0;
  int32_t* out = a.out_tokens + (size_t)b * (a.K + 1);
  for (int i = lane; i <= a.K; i += 64)
    out[i] = i < n ? clamp_token(a.draft[(size_t)b * a.K + i], a.V) : (i == n ? tok : -1);
  if (lane == 0) a.n_accepted[b] = n;
}

// ---------------------------------------------------------------------------
// Block verification of a draft block ("brb-nv/TensorRT-LLM pull 21",
// section "2. Golden sampling semantics": rejection_sample_method block;
// Sun, Mendlovic, Leviathan, Aharoni, Beirami, Ro and Suresh, "Block
// Verification Accelerates Speculative Decoding", 2024). With prefix weights
// w_0 = 1, w_{j+1} = min(1, w_j p_j(d_j) / q_j(d_j)), residual masses
// S_j = sum_v max(w_j p_j(v) - q_j(v), 0) and thresholds
// h_j = S_j / (S_j + 1 - w_j) (j < K), h_K = w_K, the row keeps the longest
// prefix d_0 .. d_{n-1} whose test eta_n < h_n passes (n = 0 if none) and
// emits a draw from max(w_n p_n - q_n, 0), or from p_K when n = K. The
// precision of each step (weights, masses and thresholds in double, the
// draw's weights rounded to float32) and the Philox counters are stated in
// include/dspark.h. The emission noise is the same at every position, so its
// Philox block and Gumbel logarithms are computed once per column, not once
// per position.
//
// Every S_j is needed before n is known, so the whole of p_0..p_K and
// q_0..q_{K-1} is read once: vblock_partials, one block per (chunk, row),
// streams each position of its chunk and leaves the chunk's partial S_j and
// the best Gumbel-max key of each position's emission distribution (so the
// draw needs no second pass). vblock_finish, one wave per row, sums the
// partials in a fixed order, finds n and merges the keys of position n.
// ---------------------------------------------------------------------------
struct VbArgs {
  const int32_t* draft;    // [B,K]
  const float* q;          // [B,K,V]
  const float* p;          // [B,K+1,V]
  const int64_t* seed;
  const int64_t* offset;
  double* part_s;          // [B][n_chunks][K]: partial residual masses (index 0 unused)
  uint64_t* part_k;        // [B][n_chunks][K+1]: best key of each position's emission
  int32_t* n_accepted;     // [B]
  int32_t* out_tokens;     // [B,K+1]
  int B, K, V, n_chunks;
  int pos_per_block;       // positions a vblock_partials block covers (all K+1 at large B)
};

// Prefix weights w_0 .. w_K of row b into s_w (all threads of the block
// take part; s_w is ready after the call).
__device__ __forceinline__ void vblock_weights(const VbArgs& a, int b, double* s_w, double* s_r) {
  for (int j = threadIdx.x; j < a.K; j += blockDim.x) {
    const int d = clamp_token(a.draft[(size_t)b * a.K + j], a.V);
    const double pv = (double)a.p[((size_t)b * (a.K + 1) + j) * a.V + d];
    const double qv = (double)a.q[((size_t)b * a.K + j) * a.V + d];
    s_r[j] = pv / qv;   // IEEE double division
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double w = 1.0;
    s_w[0] = w;
    for (int j = 0; j < a.K; ++j) {
      const double t = __dmul_rn(w, s_r[j]);
      w = t >= 1.0 ? 1.0 : (t > 0.0 ? t : 0.0);
      s_w[j + 1] = w;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = __dadd_rn(x, __shfl_xor(x, m));
  return x;
}

// One block per (chunk of kIt x 1024 columns, group of positions, row): at
// large B one group holds all K+1 positions, so the Gumbel terms serve them
// all; small batches split the positions over blocks to fill the GPU. No
// barrier inside the position loop: each wave leaves its per-position
// partials in LDS and the block merges them once at the end. Per lane the best draw of a position is
// kept as (score, column) and compared strictly in ascending column order,
// so equal scores keep the lowest column, as the 64-bit key order does.
template <int kIt>
__global__ __launch_bounds__(kThreads) void vblock_partials(VbArgs a) {
  __shared__ double s_w[kMaxK + 1], s_r[kMaxK];
  __shared__ uint64_t s_k[kMaxK + 1][kWaves];
  __shared__ double s_s[kMaxK][kWaves];
  const int c = blockIdx.x, b = blockIdx.z, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int j0 = blockIdx.y * a.pos_per_block;
  const int j1 = min(j0 + a.pos_per_block, a.K + 1);
  const int c0 = c * (kIt * kVerColsMin) + 4 * t;
  const size_t slot = (size_t)b * a.n_chunks + c;
  fx4_t pv[kIt], qv[kIt];
  auto load = [&](int j) {
    const bool bonus = j == a.K;
    const float* pj = a.p + ((size_t)b * (a.K + 1) + j) * a.V;
    const float* qj = a.q + ((size_t)b * a.K + (bonus ? 0 : j)) * a.V;
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int v = c0 + i * kVerColsMin;
      pv[i] = v < a.V ? __builtin_nontemporal_load(reinterpret_cast<const fx4_t*>(pj + v))
                      : fx4_t{0.0f, 0.0f, 0.0f, 0.0f};
      qv[i] = (!bonus && v < a.V) ? __builtin_nontemporal_load(reinterpret_cast<const fx4_t*>(qj + v))
                                  : fx4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  load(j0);   // in flight while the prefix weights and the Gumbel terms are made
  vblock_weights(a, b, s_w, s_r);
  const uint64_t seed = (uint64_t)a.seed[b], off = (uint64_t)a.offset[b];
  // the emission noise does not depend on the position: its Gumbel terms are
  // computed once and serve every position of the block
  float gl[kIt][4];
#pragma unroll
  for (int i = 0; i < kIt; ++i) {
    const uint4 x = verify_philox(seed, off, (uint32_t)(c0 + i * kVerColsMin) >> 2, 512u);
    gl[i][0] = gumbel_log2(x.x);
    gl[i][1] = gumbel_log2(x.y);
    gl[i][2] = gumbel_log2(x.z);
    gl[i][3] = gumbel_log2(x.w);
  }
  for (int j = j0; j < j1; ++j) {
    const bool bonus = j == a.K;
    if (j > j0) load(j);
    const double wj = s_w[j];
    double sj = 0.0;
    float zb = 0.0f;
    int ib = -1;
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
      const int v = c0 + i * kVerColsMin;
      const float pe[4] = {pv[i].x, pv[i].y, pv[i].z, pv[i].w};
      const float qe[4] = {qv[i].x, qv[i].y, qv[i].z, qv[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float wt = pe[e];
        if (!bonus) {
          const double r = __builtin_fmax(__dsub_rn(__dmul_rn(wj, (double)pe[e]), (double)qe[e]), 0.0);
          sj = __dadd_rn(sj, r);
          wt = __double2float_rn(r);
        }
        const float z = __fsub_rn(__builtin_amdgcn_logf(wt), gl[i][e]);
        const bool take = wt > 0.0f && (ib < 0 || z > zb);
        zb = take ? z : zb;
        ib = take ? v + e : ib;
      }
    }
    const uint64_t kw = wave_max_u64(ib < 0 ? 0ull : score_key(zb, (uint32_t)ib));
    sj = wave_sum_f64(sj);
    if (lane == 0) {
      s_k[j][wv] = kw;
      if (!bonus) s_s[j][wv] = sj;
    }
  }
  __syncthreads();
  for (int j = j0 + t; j < j1; j += kThreads) {
    uint64_t m = s_k[j][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = umax64(m, s_k[j][w]);
    a.part_k[slot * (a.K + 1) + j] = m;
    if (j < a.K) {
      double sum = s_s[j][0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) sum = __dadd_rn(sum, s_s[j][w]);
      a.part_s[slot * a.K + j] = sum;
    }
  }
}

__global__ __launch_bounds__(64) void vblock_finish(VbArgs a) {
  __shared__ double s_w[kMaxK + 1], s_r[kMaxK];
  const int b = blockIdx.x, lane = threadIdx.x;
  vblock_weights(a, b, s_w, s_r);
  const uint64_t seed = (uint64_t)a.seed[b], off = (uint64_t)a.offset[b];
  const size_t row = (size_t)b * a.n_chunks;
  int n = 0;
  for (int j = 1; j <= a.K; ++j) {
    double h;
    if (j < a.K) {
      double s = 0.0;
      for (int c = lane; c < a.n_chunks; c += 64) s = __dadd_rn(s, a.part_s[(row + c) * a.K + j]);
      s = wave_sum_f64(s);
      h = s > 0.0 ? s / __dadd_rn(s, __dsub_rn(1.0, s_w[j])) : 0.0;
    } else {
      h = s_w[a.K];
    }
    const uint32_t x = verify_philox(seed, off, 0xFFFFFFFFu, 256u + (uint32_t)(j - 1)).x;
    const float eta = __fmul_rn(__fadd_rn((float)(x >> 9), 0.5f), 0x1p-23f);   // exact
    if ((double)eta < h) n = j;
  }
  uint64_t key = 0;
  for (int c = lane; c < a.n_chunks; c += 64) key = umax64(key, a.part_k[(row + c) * (a.K + 1) + n]);
  key = wave_max_u64(key);
  if (key == 0 && n < a.K) {
    // an empty residual: the draw falls back to p_n, scored here by this one
    // wave (slow, never on the common path)
    const float* pn = a.p + ((size_t)b * (a.K + 1) + n) * a.V;
    for (int v = 4 * lane; v < a.V; v += 4 * 64) {
      const float4 pv = *reinterpret_cast<const float4*>(pn + v);
      const uint4 x = verify_philox(seed, off, (uint32_t)v >> 2, 512u);
      const float pe[4] = {pv.x, pv.y, pv.z, pv.w};
      const uint32_t xe[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (pe[e] > 0.0f)
          key = umax64(key, score_key(__fsub_rn(__builtin_amdgcn_logf(pe[e]), gumbel_log2(xe[e])), (uint32_t)(v + e)));
    }
    key = wave_max_u64(key);
  }
  const int tok = key ? clamp_token((int)key_token(key), a.V) : 0;
  int32_t* out = a.out_tokens + (size_t)b * (a.K + 1);
  for (int i = lane; i <= a.K; i += 64)
    out[i] = i < n ? clamp_token(a.draft[(size_t)b * a.K + i], a.V) : (i == n ? tok : -1);
  if (lane == 0) a.n_accepted[b] = n;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct Workspace {
  uint64_t* part_key[2];   // double-buffered by position parity
  Stat* part_stat[2];
  Stat* row_stat;
  uint16_t* e_buf;
  Stat* stat_part;         // resident paths: [K][B][kResMaxCUs]
  float* sink;             // resident MFMA path: [kMfSinkFloats] discarded stores
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Layout for the largest chunk count (chunk = 128 columns), plus the resident
// paths' per-workgroup statistics and sink when B <= 128. (Their exchange
// words live in the library's own device memory, g_exchange.)
inline size_t workspace_layout(int B, int K, int V, int r, Workspace* ws, char* base) {
  const size_t max_chunks = (size_t)(V + kTile - 1) / kTile;
  size_t off = 0;
  size_t o_key[2], o_pst[2];
  for (int i = 0; i < 2; ++i) {
    o_key[i] = off; off = align_up(off + (size_t)B * max_chunks * sizeof(uint64_t), 256);
    o_pst[i] = off; off = align_up(off + (size_t)B * max_chunks * sizeof(Stat), 256);
  }
  const size_t o_rst = off; off = align_up(off + (size_t)B * K * sizeof(Stat), 256);
  const size_t o_e = off;   off = align_up(off + (size_t)B * r * sizeof(uint16_t), 256);
  size_t o_sp = 0, o_s = 0;
  const bool resident_ws = B <= kMfRowsMax;
  if (resident_ws) {
    o_sp = off; off = align_up(off + (size_t)K * B * kResMaxCUs * sizeof(Stat), 256);
    o_s = off;  off = align_up(off + kMfSinkFloats * sizeof(float), 256);
  }
  if (ws) {
    for (int i = 0; i < 2; ++i) {
      ws->part_key[i] = reinterpret_cast<uint64_t*>(base + o_key[i]);
      ws->part_stat[i] = reinterpret_cast<Stat*>(base + o_pst[i]);
    }
    ws->row_stat = reinterpret_cast<Stat*>(base + o_rst);
    ws->e_buf = reinterpret_cast<uint16_t*>(base + o_e);
    ws->stat_part = resident_ws ? reinterpret_cast<Stat*>(base + o_sp) : nullptr;
    ws->sink = resident_ws ? reinterpret_cast<float*>(base + o_s) : nullptr;
  }
  return off;
}

// Scratch of dspark_draft_block_noalloc, for callers that cannot allocate
// device memory: one copy per device, held until the process ends. Host code
// uses only the device address hipGetSymbolAddress gives for it (set-up, once
// per device); the name itself is a host-side stand-in, not a device address.
constexpr size_t kScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Per-device facts the resident path needs (filled by dspark_init).
struct DeviceInfo {
  bool ready;
  bool resident_ok;   // one 512-thread workgroup with kResLdsBytes of LDS fits on every CU
  bool mfma_ok;       // the same for the MFMA resident kernel
  int cus;
  ResExchange* exchange;   // device address of this device's g_exchange
  unsigned char* scratch;  // device address of this device's scratch
};
constexpr int kMaxDevices = 64;
DeviceInfo g_devices[kMaxDevices];

// Reads of an exchange word before a resident kernel's wait expires (set by
// dspark_set_wait_limit; taken at each call, so a captured graph keeps the
// value of its capture).
unsigned g_wait_limit = kDefaultWaitLimit;

template <int RB, bool kBf16, bool kPacked>
bool prepare_resident_kernel() {
  const void* fn = reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_resident<RB, kBf16, kPacked>);
  int occ = 0;
  const bool ok =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kResLdsBytes) == hipSuccess &&
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, markov_bias_gumbel_argmax_resident<RB, kBf16, kPacked>,
                                                   kResThreads, kResLdsBytes) == hipSuccess;
  // a probe that fails only rules the plan out: clear the error it leaves
  // behind, or the caller's next HIP call would report it
  if (!ok) (void)hipGetLastError();
  return ok && occ >= 1;
}

template <bool kBf16, bool kRagged, bool kPacked>
bool prepare_mfma_kernel() {
  const void* fn = reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_resident_mfma<kBf16, kRagged, kPacked>);
  int occ = 0;
  const bool ok =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMfLdsBytes) == hipSuccess &&
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, markov_bias_gumbel_argmax_resident_mfma<kBf16, kRagged, kPacked>,
                                                   kMfThreads, kMfLdsBytes) == hipSuccess;
  if (!ok) (void)hipGetLastError();
  return ok && occ >= 1;
}

int init_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSPARK_ERR_HIP;
  DeviceInfo& info = g_devices[dev];
  if (info.ready) return DSPARK_OK;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return DSPARK_ERR_HIP;
  bool ok = cus > 0 && cus <= kResMaxCUs;
  ok = ok && prepare_resident_kernel<1, false, false>() && prepare_resident_kernel<1, true, false>();
  ok = ok && prepare_resident_kernel<2, false, false>() && prepare_resident_kernel<2, true, false>();
  ok = ok && prepare_resident_kernel<1, false, true>() && prepare_resident_kernel<1, true, true>();
  ok = ok && prepare_resident_kernel<2, false, true>() && prepare_resident_kernel<2, true, true>();
  bool mok = cus > 0 && cus <= kResMaxCUs;
  mok = mok && prepare_mfma_kernel<false, false, false>() && prepare_mfma_kernel<true, false, false>();
  mok = mok && prepare_mfma_kernel<false, true, false>() && prepare_mfma_kernel<true, true, false>();
  mok = mok && prepare_mfma_kernel<false, false, true>() && prepare_mfma_kernel<true, false, true>();
  mok = mok && prepare_mfma_kernel<false, true, true>() && prepare_mfma_kernel<true, true, true>();
  // the device's own copy of the exchange state: its address from the symbol
  // (the name itself is no device address in host code)
  void* ex = nullptr;
  if (hipGetSymbolAddress(&ex, HIP_SYMBOL(g_exchange)) != hipSuccess || ex == nullptr) return DSPARK_ERR_HIP;
  info.exchange = static_cast<ResExchange*>(ex);
  void* sc = nullptr;
  if (hipGetSymbolAddress(&sc, HIP_SYMBOL(scratch)) != hipSuccess || sc == nullptr) return DSPARK_ERR_HIP;
  info.scratch = static_cast<unsigned char*>(sc);
  info.cus = cus;
  info.resident_ok = ok;
  info.mfma_ok = mok;
  info.ready = true;
  return DSPARK_OK;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_sizes(int B, int K, int V, int r) {
  if (B < 0 || K < 0 || V <= 0 || r <= 0) return DSPARK_ERR_ARG;
  if (V % 8 != 0 || r % 32 != 0 || r > kMaxRank || K > kMaxK) return DSPARK_ERR_UNSUPPORTED;
  if ((long long)V >= (1LL << 31) - kTile) return DSPARK_ERR_UNSUPPORTED;
  return DSPARK_OK;
}

template <bool kBf16>
hipError_t launch_fused(const StepArgs& sa, bool in_kernel_pick, hipStream_t stream) {
  const dim3 grid(sa.n_chunks), block(kThreads);
  if (sa.B == 1) {
    if (in_kernel_pick)
      hipLaunchKernelGGL((markov_bias_gumbel_argmax_gemv<1, kBf16, true>), grid, block, 0, stream, sa);
    else
      hipLaunchKernelGGL((markov_bias_gumbel_argmax_gemv<1, kBf16, false>), grid, block, 0, stream, sa);
  } else if (sa.B == 2) {
    hipLaunchKernelGGL((markov_bias_gumbel_argmax_gemv<2, kBf16, false>), grid, block, 0, stream, sa);
  } else if (sa.B <= 4) {
    hipLaunchKernelGGL((markov_bias_gumbel_argmax_gemv<4, kBf16, false>), grid, block, 0, stream, sa);
  } else {
    hipLaunchKernelGGL((markov_bias_gumbel_argmax_rows<kBf16>), grid, block, 0, stream, sa);
  }
  return hipGetLastError();
}

// Which kernels one call enqueues, in order.
struct Plan {
  bool resident;
  bool resident_mfma;
  bool in_kernel_pick;
  int n_chunks;
  int chunk_cols;
  int G;
  int slice;
  ResExchange* exchange;
  unsigned char* scratch;
};

int make_plan(int B, int K, int V, int r, int chunk_cols, Plan* plan) {
  (void)K;
  const bool explicit_chunk = chunk_cols != 0;
  if (chunk_cols == 0) chunk_cols = kDefaultChunk;
  int rc = init_device();
  if (rc != DSPARK_OK) return rc;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DSPARK_ERR_HIP;
  const DeviceInfo& info = g_devices[dev];
  plan->G = info.cus;
  plan->exchange = info.exchange;
  plan->scratch = info.scratch;
  plan->slice = info.cus > 0 ? ((V + info.cus - 1) / info.cus + 7) / 8 * 8 : 0;
  // resident path: all positions in one persistent launch with W kept on chip
  plan->resident = !explicit_chunk && info.resident_ok && B <= kResRowsMax && r <= kResRank &&
                   V <= (int)kResIdxMask + 1 && plan->slice <= kResSlice;
  const int mf_slice = info.cus > 0 ? ((V + info.cus - 1) / info.cus + 15) / 16 * 16 : 0;
  plan->resident_mfma = !plan->resident && !explicit_chunk && info.mfma_ok && B > kResRowsMax &&
                        B <= kMfRowsMax && r <= kResRank && V <= (int)kResIdxMask + 1 &&
                        mf_slice <= kResSlice;
  if (plan->resident_mfma) plan->slice = mf_slice;   // whole 16-column M-tiles
  plan->chunk_cols = chunk_cols;
  plan->n_chunks = (V + chunk_cols - 1) / chunk_cols;
  // one row: every workgroup picks the previous token itself (no pick launch)
  plan->in_kernel_pick = (B == 1) && plan->n_chunks <= kPickPerThread * kThreads;
  return DSPARK_OK;
}

// The workspace one call needs for its own plan only (the no-allocation entry
// point lays it out in the scratch array): a resident plan needs the
// per-workgroup statistics [K][B][G] and the sink, a per-position plan its
// chunk partials (double-buffered), row statistics and embedding rows.
inline size_t plan_layout(const Plan& plan, int B, int K, int r, Workspace* ws, char* base) {
  size_t off = 0;
  size_t o_key[2] = {0, 0}, o_pst[2] = {0, 0}, o_rst = 0, o_e = 0, o_sp = 0, o_s = 0;
  if (plan.resident || plan.resident_mfma) {
    o_sp = off; off = align_up(off + (size_t)K * B * plan.G * sizeof(Stat), 256);
    o_s = off;  off = align_up(off + kMfSinkFloats * sizeof(float), 256);
  } else {
    for (int i = 0; i < 2; ++i) {
      o_key[i] = off; off = align_up(off + (size_t)B * plan.n_chunks * sizeof(uint64_t), 256);
      o_pst[i] = off; off = align_up(off + (size_t)B * plan.n_chunks * sizeof(Stat), 256);
    }
    o_rst = off; off = align_up(off + (size_t)B * K * sizeof(Stat), 256);
    o_e = off;   off = align_up(off + (size_t)B * r * sizeof(uint16_t), 256);
  }
  if (ws) {
    const bool res = plan.resident || plan.resident_mfma;
    for (int i = 0; i < 2; ++i) {
      ws->part_key[i] = res ? nullptr : reinterpret_cast<uint64_t*>(base + o_key[i]);
      ws->part_stat[i] = res ? nullptr : reinterpret_cast<Stat*>(base + o_pst[i]);
    }
    ws->row_stat = res ? nullptr : reinterpret_cast<Stat*>(base + o_rst);
    ws->e_buf = res ? nullptr : reinterpret_cast<uint16_t*>(base + o_e);
    ws->stat_part = res ? reinterpret_cast<Stat*>(base + o_sp) : nullptr;
    ws->sink = res ? reinterpret_cast<float*>(base + o_s) : nullptr;
  }
  return off;
}

// workspace == nullptr with use_scratch: the call lays its workspace out in the
// device's scratch array (dspark_draft_block_noalloc).
// Packed-W geometry on the current device: the two kernels' slices (multiples
// of 8 and of 16 columns) and the bytes of both regions; 0 bytes when no
// resident plan can run these sizes (then there is nothing to pack).
struct PackGeom {
  int G, slice8, slice16;
  size_t bytes;
};
inline PackGeom packed_w_geom(int V, int r) {
  PackGeom pg{0, 0, 0, 0};
  if (V <= 0 || r <= 0 || V % 8 != 0 || r % 32 != 0 || r > kResRank || V > (int)kResIdxMask + 1) return pg;
  if (init_device() != DSPARK_OK) return pg;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return pg;
  const int G = g_devices[dev].cus;
  if (G <= 0 || G > kResMaxCUs) return pg;
  pg.G = G;
  pg.slice8 = ((V + G - 1) / G + 7) / 8 * 8;
  pg.slice16 = ((V + G - 1) / G + 15) / 16 * 16;
  if (pg.slice16 > kResSlice) return pg;
  pg.bytes = 2 * (size_t)G * kPackWgU4 * 16;
  return pg;
}
inline size_t packed_w_bytes(int V, int r) { return packed_w_geom(V, r).bytes; }

int draft_block_impl(const void* base, int base_dtype, const uint16_t* E, const uint16_t* W,
                     const int32_t* prev_token, const int64_t* seed, const int64_t* offset,
                     const float* temperature, const int32_t* n_real, int B, int K, int V, int r,
                     int chunk_cols, int32_t* tokens, float* logits, float* q, void* workspace,
                     size_t workspace_bytes, void* stream_ptr, void* const* events = nullptr,
                     int n_events = 0, bool use_scratch = false, const void* W_packed = nullptr,
                     size_t packed_bytes = 0, const int32_t* slot_index = nullptr, int n_slots = 0) {
  int rc = check_sizes(B, K, V, r);
  if (rc != DSPARK_OK) return rc;
  const bool packed = W_packed != nullptr;
  if (base_dtype != DSPARK_F32 && base_dtype != DSPARK_BF16) return DSPARK_ERR_ARG;
  if (chunk_cols < 0 || chunk_cols % kTile != 0) return DSPARK_ERR_UNSUPPORTED;
  const bool explicit_chunk = chunk_cols != 0;
  if (chunk_cols == 0) chunk_cols = kDefaultChunk;
  if (B == 0 || K == 0) return DSPARK_OK;
  if (!base || !E || !W || !prev_token || !seed || !offset || !temperature || !tokens || !logits ||
      !q)
    return DSPARK_ERR_ARG;
  if (!aligned16(base) || !aligned16(E) || !aligned16(W) || !aligned16(logits) || !aligned16(q))
    return DSPARK_ERR_ARG;
  if (packed && !aligned16(W_packed)) return DSPARK_ERR_ARG;
  if (!use_scratch) {
    const size_t need = workspace_layout(B, K, V, r, nullptr, nullptr);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return DSPARK_ERR_WORKSPACE;
  }
  // the packed copy must be this device's, for these sizes (its size says so)
  if (packed && packed_bytes != packed_w_bytes(V, r)) return DSPARK_ERR_ARG;
  if (slot_index && n_slots <= 0) return DSPARK_ERR_ARG;

  Plan plan;
  rc = make_plan(B, K, V, r, explicit_chunk ? chunk_cols : 0, &plan);
  if (rc != DSPARK_OK) return rc;
  if (use_scratch && plan_layout(plan, B, K, r, nullptr, nullptr) > kScratchBytes) return DSPARK_ERR_SCRATCH;
  const bool resident = plan.resident || plan.resident_mfma;
  const bool in_kernel_pick = plan.in_kernel_pick;
  const int n_chunks = plan.n_chunks;
  const int G = plan.G;
  const int slice = plan.slice;
  const int n_launches = resident ? 2 : in_kernel_pick ? K + 1 : 2 * K + 1;
  if (events && n_events < n_launches + 1) return DSPARK_ERR_ARG;

  Workspace ws;
  if (use_scratch)
    plan_layout(plan, B, K, r, &ws, reinterpret_cast<char*>(plan.scratch));
  else
    workspace_layout(B, K, V, r, &ws, static_cast<char*>(workspace));
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  int n_marks = 0;
  auto mark = [&]() -> bool {
    if (!events) return true;
    return hipEventRecord(static_cast<hipEvent_t>(events[n_marks++]), stream) == hipSuccess;
  };
  if (!mark()) return DSPARK_ERR_HIP;
  const bool bf16 = base_dtype == DSPARK_BF16;

  if (resident) {
    const dim3 grid(G);
    if (plan.resident_mfma) {
      MfArgs ma;
      ma.base = base; ma.E = E; ma.W = W; ma.prev_token = prev_token; ma.seed = seed; ma.offset = offset;
      ma.temperature = temperature; ma.n_real = n_real; ma.logits = logits; ma.tokens = tokens;
      ma.ex = plan.exchange; ma.stat_part = ws.stat_part; ma.sink = ws.sink;
      ma.xrow = &plan.exchange->xrow[0][0][0];   // host arithmetic on the device address
      ma.xwin = &plan.exchange->xwin[0][0];
      ma.zeros = plan.exchange->zeros;
      ma.B = B; ma.K = K; ma.V = V; ma.r = r; ma.slice = slice;
      ma.spin_limit = g_wait_limit;
      const dim3 mblock(kMfThreads);
      // columns come in whole tiles of 16 unless the vocabulary is ragged
      const bool ragged = V % 16 != 0;
      ma.Wp = packed ? reinterpret_cast<const u32x4_t*>(W_packed) + (size_t)G * kPackWgU4 : nullptr;
#define DSPARK_LAUNCH_MF(BF, RG, PK) \
  hipLaunchKernelGGL((markov_bias_gumbel_argmax_resident_mfma<BF, RG, PK>), grid, mblock, kMfLdsBytes, stream, ma)
      if (packed) {
        if (bf16 && !ragged) DSPARK_LAUNCH_MF(true, false, true);
        else if (!ragged) DSPARK_LAUNCH_MF(false, false, true);
        else if (bf16) DSPARK_LAUNCH_MF(true, true, true);
        else DSPARK_LAUNCH_MF(false, true, true);
      } else {
        if (bf16 && !ragged) DSPARK_LAUNCH_MF(true, false, false);
        else if (!ragged) DSPARK_LAUNCH_MF(false, false, false);
        else if (bf16) DSPARK_LAUNCH_MF(true, true, false);
        else DSPARK_LAUNCH_MF(false, true, false);
      }
#undef DSPARK_LAUNCH_MF
    } else {
      ResArgs ra;
      ra.base = base; ra.E = E; ra.W = W; ra.prev_token = prev_token; ra.seed = seed; ra.offset = offset;
      ra.temperature = temperature; ra.n_real = n_real; ra.logits = logits; ra.tokens = tokens;
      ra.ex = plan.exchange; ra.stat_part = ws.stat_part;
      ra.B = B; ra.K = K; ra.V = V; ra.r = r; ra.slice = slice;
      ra.spin_limit = g_wait_limit;
      const dim3 block(kResThreads);
      ra.Wp = packed ? reinterpret_cast<const uint4*>(W_packed) : nullptr;
#define DSPARK_LAUNCH_RES(RBV, BF, PK) \
  hipLaunchKernelGGL((markov_bias_gumbel_argmax_resident<RBV, BF, PK>), grid, block, kResLdsBytes, stream, ra)
#define DSPARK_LAUNCH_RES_B(PK)                                                       \
  do {                                                                                \
    if (B == 1) { if (bf16) DSPARK_LAUNCH_RES(1, true, PK); else DSPARK_LAUNCH_RES(1, false, PK); } \
    else { if (bf16) DSPARK_LAUNCH_RES(2, true, PK); else DSPARK_LAUNCH_RES(2, false, PK); } \
  } while (0)
      if (packed) DSPARK_LAUNCH_RES_B(true);
      else DSPARK_LAUNCH_RES_B(false);
#undef DSPARK_LAUNCH_RES_B
#undef DSPARK_LAUNCH_RES
    }
    if (hipGetLastError() != hipSuccess || !mark()) return DSPARK_ERR_HIP;
  }

  for (int k = 0; k < K && !resident; ++k) {
    StepArgs sa;
    sa.base = base; sa.E = E; sa.W = W; sa.prev_token = prev_token; sa.e_buf = ws.e_buf;
    sa.prev_key = ws.part_key[(k + 1) & 1]; sa.prev_stat = ws.part_stat[(k + 1) & 1];
    sa.seed = seed; sa.offset = offset; sa.temperature = temperature; sa.n_real = n_real;
    sa.logits = logits; sa.tokens = tokens; sa.row_stat = ws.row_stat;
    sa.part_key = ws.part_key[k & 1]; sa.part_stat = ws.part_stat[k & 1];
    sa.B = B; sa.K = K; sa.V = V; sa.r = r; sa.k = k;
    sa.chunk_cols = chunk_cols; sa.n_chunks = n_chunks;
    const hipError_t err = bf16 ? launch_fused<true>(sa, in_kernel_pick, stream)
                                : launch_fused<false>(sa, in_kernel_pick, stream);
    if (err != hipSuccess || !mark()) return DSPARK_ERR_HIP;

    if (!in_kernel_pick) {
      PickArgs pa;
      pa.part_key = ws.part_key[k & 1]; pa.part_stat = ws.part_stat[k & 1]; pa.E = E;
      pa.tokens = tokens; pa.row_stat = ws.row_stat; pa.e_buf = ws.e_buf;
      pa.B = B; pa.K = K; pa.V = V; pa.r = r; pa.k = k; pa.n_chunks = n_chunks;
      hipLaunchKernelGGL(pick_and_gather, dim3(B), dim3(kThreads), 0, stream, pa);
      if (hipGetLastError() != hipSuccess || !mark()) return DSPARK_ERR_HIP;
    }
  }

  PropArgs pr;
  pr.logits = logits; pr.temperature = temperature; pr.tokens = tokens; pr.row_stat = ws.row_stat;
  pr.last_key = ws.part_key[(K - 1) & 1]; pr.last_stat = ws.part_stat[(K - 1) & 1];
  pr.q = q; pr.B = B; pr.K = K; pr.V = V; pr.n_chunks = n_chunks;
  pr.slot = slot_index; pr.n_slots = slot_index ? n_slots : B;
  pr.last_from_partials = (in_kernel_pick && !resident) ? 1 : 0;
  pr.part_stat = resident ? ws.stat_part : nullptr;
  pr.n_part = resident ? G : 0;
  const bool large = B >= kPropLargeRows;
  const int cols = large ? prop_cols<kPropVecLarge>() : prop_cols<kPropVecSmall>();
  pr.blocks_per_row = (V + cols - 1) / cols;
  const long long n_blocks = (long long)pr.blocks_per_row * B * K;
  if (n_blocks >= (1LL << 31)) return DSPARK_ERR_UNSUPPORTED;
  if (large)
    hipLaunchKernelGGL(proposal_softmax<kPropVecLarge>, dim3((unsigned)n_blocks), dim3(kThreads), 0, stream, pr);
  else
    hipLaunchKernelGGL(proposal_softmax<kPropVecSmall>, dim3((unsigned)n_blocks), dim3(kThreads), 0, stream, pr);
  if (hipGetLastError() != hipSuccess || !mark()) return DSPARK_ERR_HIP;
  return DSPARK_OK;
}

// 1024-column units per verify_partials block: the fewest that still give
// ~4096 blocks (small batches get more, smaller blocks). At B=88, V=200064
// that is 4 units (4312 blocks: 36.5 us against 38.6 us with 8 units and
// 38.1 us with 2).
inline int verify_iters(int B, int V) {
  const long long units = (long long)B * ((V + kVerColsMin - 1) / kVerColsMin);
  return units >= 8 * 4096 ? 8 : units >= 4 * 4096 ? 4 : units >= 2 * 4096 ? 2 : 1;
}
inline int verify_chunks(int B, int V) {
  const int cols = verify_iters(B, V) * kVerColsMin;
  return (V + cols - 1) / cols;
}

inline int verify_check(int B, int K, int V) {
  if (B < 0 || K < 0 || V <= 0) return DSPARK_ERR_ARG;
  if (K > kMaxK || V % 4 != 0 || B > 65535) return DSPARK_ERR_UNSUPPORTED;
  return DSPARK_OK;
}

inline size_t verify_workspace(int B, int V) {
  return align_up((size_t)B * verify_chunks(B, V) * sizeof(uint64_t), 256);
}

int verify_standard_impl(const int32_t* draft, const float* q, const float* p, const int64_t* seed,
                         const int64_t* offset, int B, int K, int V, int32_t* n_accepted,
                         int32_t* out_tokens, void* workspace, size_t workspace_bytes, void* stream_ptr) {
  int rc = verify_check(B, K, V);
  if (rc != DSPARK_OK) return rc;
  if (B == 0) return DSPARK_OK;
  if ((K > 0 && (!draft || !q)) || !p || !seed || !offset || !n_accepted || !out_tokens) return DSPARK_ERR_ARG;
  if ((K > 0 && !aligned16(q)) || !aligned16(p)) return DSPARK_ERR_ARG;
  if (!workspace || workspace_bytes < verify_workspace(B, V) || (reinterpret_cast<uintptr_t>(workspace) & 7u))
    return DSPARK_ERR_WORKSPACE;
  VerArgs a;
  a.draft = draft; a.q = q; a.p = p; a.seed = seed; a.offset = offset;
  a.part = static_cast<uint64_t*>(workspace);
  a.n_accepted = n_accepted; a.out_tokens = out_tokens;
  a.B = B; a.K = K; a.V = V; a.n_chunks = verify_chunks(B, V);
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const dim3 grid(a.n_chunks, B);
  switch (verify_iters(B, V)) {
    case 8: hipLaunchKernelGGL(verify_partials<8>, grid, dim3(kThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL(verify_partials<4>, grid, dim3(kThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL(verify_partials<2>, grid, dim3(kThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL(verify_partials<1>, grid, dim3(kThreads), 0, stream, a); break;
  }
  if (hipGetLastError() != hipSuccess) return DSPARK_ERR_HIP;
  hipLaunchKernelGGL(verify_finish, dim3(B), dim3(64), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return DSPARK_ERR_HIP;
  return DSPARK_OK;
}

// 1024-column units per vblock_partials block: 2 once that still gives
// ~4096 blocks, else 1 (a block streams up to K+1 positions; at B=88,
// V=200064: 185 us with 2 units against 193 with 1 and 189 with 4).
inline int vblock_iters(int B, int V) {
  const long long units = (long long)B * ((V + kVerColsMin - 1) / kVerColsMin);
  return units >= 2 * 4096 ? 2 : 1;
}
inline int vblock_chunks(int B, int V) {
  const int cols = vblock_iters(B, V) * kVerColsMin;
  return (V + cols - 1) / cols;
}
inline size_t vblock_part_s_bytes(int B, int K, int V) {
  return align_up((size_t)B * vblock_chunks(B, V) * K * sizeof(double), 256);
}
inline size_t vblock_workspace(int B, int K, int V) {
  return vblock_part_s_bytes(B, K, V) + align_up((size_t)B * vblock_chunks(B, V) * (K + 1) * sizeof(uint64_t), 256);
}

int verify_block_impl(const int32_t* draft, const float* q, const float* p, const int64_t* seed,
                      const int64_t* offset, int B, int K, int V, int32_t* n_accepted, int32_t* out_tokens,
                      void* workspace, size_t workspace_bytes, void* stream_ptr) {
  int rc = verify_check(B, K, V);
  if (rc != DSPARK_OK) return rc;
  if (B == 0) return DSPARK_OK;
  if ((K > 0 && (!draft || !q)) || !p || !seed || !offset || !n_accepted || !out_tokens) return DSPARK_ERR_ARG;
  if ((K > 0 && !aligned16(q)) || !aligned16(p)) return DSPARK_ERR_ARG;
  if (!workspace || workspace_bytes < vblock_workspace(B, K, V) || (reinterpret_cast<uintptr_t>(workspace) & 7u))
    return DSPARK_ERR_WORKSPACE;
  VbArgs a;
  a.draft = draft; a.q = q; a.p = p; a.seed = seed; a.offset = offset;
  a.part_s = static_cast<double*>(workspace);
  a.part_k = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + vblock_part_s_bytes(B, K, V));
  a.n_accepted = n_accepted; a.out_tokens = out_tokens;
  a.B = B; a.K = K; a.V = V; a.n_chunks = vblock_chunks(B, V);
  // small batches split the positions over ~4096 blocks (B=1, V=200064: 196
  // blocks of 8 positions would leave most of the GPU idle)
  const long long cb = (long long)B * a.n_chunks;
  const int groups = cb >= 2048 ? 1 : (int)std::min<long long>(K + 1, (4096 + cb - 1) / cb);
  a.pos_per_block = (K + 1 + groups - 1) / groups;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const dim3 grid(a.n_chunks, (K + 1 + a.pos_per_block - 1) / a.pos_per_block, B);
  if (vblock_iters(B, V) == 2)
    hipLaunchKernelGGL(vblock_partials<2>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(vblock_partials<1>, grid, dim3(kThreads), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return DSPARK_ERR_HIP;
  hipLaunchKernelGGL(vblock_finish, dim3(B), dim3(64), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return DSPARK_ERR_HIP;
  return DSPARK_OK;
}

}  // namespace dspark

extern "C" {

int dspark_init(void) {
  using namespace dspark;
  if (init_device() != DSPARK_OK) return DSPARK_ERR_HIP;
  hipFuncAttributes attr;
  const void* kernels[] = {
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_gemv<1, false, true>),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_gemv<1, true, true>),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_gemv<1, false, false>),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_gemv<1, true, false>),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_gemv<2, false, false>),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_gemv<2, true, false>),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_gemv<4, false, false>),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_gemv<4, true, false>),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_rows<false>),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_rows<true>),
      reinterpret_cast<const void*>(&pick_and_gather),
      reinterpret_cast<const void*>(&proposal_softmax<kPropVecSmall>),
      reinterpret_cast<const void*>(&proposal_softmax<kPropVecLarge>),
      reinterpret_cast<const void*>(&res_status),
      reinterpret_cast<const void*>(&verify_partials<1>),
      reinterpret_cast<const void*>(&verify_partials<2>),
      reinterpret_cast<const void*>(&verify_partials<4>),
      reinterpret_cast<const void*>(&verify_partials<8>),
      reinterpret_cast<const void*>(&verify_finish),
      reinterpret_cast<const void*>(&vblock_partials<1>),
      reinterpret_cast<const void*>(&vblock_partials<2>),
      reinterpret_cast<const void*>(&vblock_finish),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_resident_mfma<false, false, false>),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_resident_mfma<true, false, false>),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_resident_mfma<false, true, false>),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_resident_mfma<true, true, false>),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_resident_mfma<false, false, true>),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_resident_mfma<true, false, true>),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_resident_mfma<false, true, true>),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_resident_mfma<true, true, true>),
      reinterpret_cast<const void*>(&pack_w),
  };
  for (const void* kfn : kernels)
    if (hipFuncGetAttributes(&attr, kfn) != hipSuccess) return DSPARK_ERR_HIP;
  return DSPARK_OK;
}

size_t dspark_workspace_bytes(int B, int K, int V, int r) {
  if (dspark::check_sizes(B, K, V, r) != DSPARK_OK) return 0;
  return dspark::workspace_layout(B, K, V, r, nullptr, nullptr);
}

size_t dspark_verify_workspace_bytes(int B, int K, int V) {
  if (dspark::verify_check(B, K, V) != DSPARK_OK) return 0;
  return dspark::verify_workspace(B, V);
}

int dspark_verify_standard(const int32_t* draft_tokens, const float* draft_probs, const float* target_probs,
                           const int64_t* seed, const int64_t* offset, int B, int K, int V,
                           int32_t* n_accepted, int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return dspark::verify_standard_impl(draft_tokens, draft_probs, target_probs, seed, offset, B, K, V, n_accepted,
                                      out_tokens, workspace, workspace_bytes, stream);
}

size_t dspark_verify_block_workspace_bytes(int B, int K, int V) {
  if (dspark::verify_check(B, K, V) != DSPARK_OK) return 0;
  return dspark::vblock_workspace(B, K, V);
}

int dspark_verify_block(const int32_t* draft_tokens, const float* draft_probs, const float* target_probs,
                        const int64_t* seed, const int64_t* offset, int B, int K, int V, int32_t* n_accepted,
                        int32_t* out_tokens, void* workspace, size_t workspace_bytes, void* stream) {
  return dspark::verify_block_impl(draft_tokens, draft_probs, target_probs, seed, offset, B, K, V, n_accepted,
                                   out_tokens, workspace, workspace_bytes, stream);
}

int dspark_draft_block(const void* base_logits, int base_dtype, const uint16_t* E, const uint16_t* W,
                       const int32_t* prev_token, const int64_t* seed, const int64_t* offset,
                       const float* temperature, const int32_t* n_real, int B, int K, int V, int r,
                       int32_t* tokens, float* logits_f32, float* draft_probs, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return dspark::draft_block_impl(base_logits, base_dtype, E, W, prev_token, seed, offset, temperature,
                                  n_real, B, K, V, r, 0, tokens, logits_f32, draft_probs, workspace,
                                  workspace_bytes, stream);
}

int dspark_draft_block_noalloc(const void* base_logits, int base_dtype, const uint16_t* E, const uint16_t* W,
                               const int32_t* prev_token, const int64_t* seed, const int64_t* offset,
                               const float* temperature, const int32_t* n_real, int B, int K, int V, int r,
                               int32_t* tokens, float* logits_f32, float* draft_probs, void* stream) {
  return dspark::draft_block_impl(base_logits, base_dtype, E, W, prev_token, seed, offset, temperature,
                                  n_real, B, K, V, r, 0, tokens, logits_f32, draft_probs, nullptr, 0, stream,
                                  nullptr, 0, /*use_scratch=*/true);
}

size_t dspark_noalloc_scratch_bytes(void) { return dspark::kScratchBytes; }

int dspark_draft_block_chunked(const void* base_logits, int base_dtype, const uint16_t* E,
                               const uint16_t* W, const int32_t* prev_token, const int64_t* seed,
                               const int64_t* offset, const float* temperature, const int32_t* n_real,
                               int B, int K, int V, int r, int chunk_cols, int32_t* tokens,
                               float* logits_f32, float* draft_probs, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return dspark::draft_block_impl(base_logits, base_dtype, E, W, prev_token, seed, offset, temperature,
                                  n_real, B, K, V, r, chunk_cols, tokens, logits_f32, draft_probs,
                                  workspace, workspace_bytes, stream);
}

int dspark_draft_block_events(const void* base_logits, int base_dtype, const uint16_t* E,
                              const uint16_t* W, const int32_t* prev_token, const int64_t* seed,
                              const int64_t* offset, const float* temperature, const int32_t* n_real,
                              int B, int K, int V, int r, int32_t* tokens, float* logits_f32,
                              float* draft_probs, void* workspace, size_t workspace_bytes, void* stream,
                              void* const* events, int n_events) {
  if (!events) return DSPARK_ERR_ARG;
  return dspark::draft_block_impl(base_logits, base_dtype, E, W, prev_token, seed, offset, temperature,
                                  n_real, B, K, V, r, 0, tokens, logits_f32, draft_probs, workspace,
                                  workspace_bytes, stream, events, n_events);
}

size_t dspark_packed_w_bytes(int V, int r) { return dspark::packed_w_bytes(V, r); }

int dspark_pack_w(const uint16_t* W, int V, int r, void* W_packed, size_t packed_bytes, void* stream) {
  using namespace dspark;
  if (V <= 0 || r <= 0) return DSPARK_ERR_ARG;
  const PackGeom pg = packed_w_geom(V, r);
  if (pg.bytes == 0) return DSPARK_ERR_UNSUPPORTED;
  if (!W || !W_packed || packed_bytes < pg.bytes || !aligned16(W_packed)) return DSPARK_ERR_ARG;
  PackArgs pa;
  pa.W = W; pa.out = static_cast<uint4*>(W_packed);
  pa.V = V; pa.r = r; pa.G = pg.G; pa.slice8 = pg.slice8; pa.slice16 = pg.slice16;
  const size_t units = pg.bytes / 16;
  hipLaunchKernelGGL(pack_w, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, static_cast<hipStream_t>(stream), pa);
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP;
}

int dspark_draft_block_packed(const void* base_logits, int base_dtype, const uint16_t* E, const uint16_t* W,
                              const void* W_packed, size_t packed_bytes, const int32_t* prev_token,
                              const int64_t* seed, const int64_t* offset, const float* temperature,
                              const int32_t* n_real, int B, int K, int V, int r, int32_t* tokens,
                              float* logits_f32, float* draft_probs, void* workspace, size_t workspace_bytes,
                              void* stream, void* const* events, int n_events) {
  if (!W_packed) return DSPARK_ERR_ARG;
  return dspark::draft_block_impl(base_logits, base_dtype, E, W, prev_token, seed, offset, temperature,
                                  n_real, B, K, V, r, 0, tokens, logits_f32, draft_probs, workspace,
                                  workspace_bytes, stream, events, events ? n_events : 0, false, W_packed,
                                  packed_bytes);
}

int dspark_draft_block_slots(const void* base_logits, int base_dtype, const uint16_t* E, const uint16_t* W,
                             const void* W_packed, size_t packed_bytes, const int32_t* prev_token,
                             const int64_t* seed, const int64_t* offset, const float* temperature,
                             const int32_t* n_real, const int32_t* slot_index, int n_slots, int B, int K,
                             int V, int r, int32_t* tokens, float* logits_f32, float* draft_probs,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (!slot_index) return DSPARK_ERR_ARG;
  return dspark::draft_block_impl(base_logits, base_dtype, E, W, prev_token, seed, offset, temperature,
                                  n_real, B, K, V, r, 0, tokens, logits_f32, draft_probs, workspace,
                                  workspace_bytes, stream, nullptr, 0, false, W_packed,
                                  W_packed ? packed_bytes : 0, slot_index, n_slots);
}

int dspark_launch_plan(int B, int K, int V, int r, int* kinds, int max_kinds) {
  using namespace dspark;
  if (check_sizes(B, K, V, r) != DSPARK_OK) return DSPARK_ERR_UNSUPPORTED;
  if (B == 0 || K == 0) return 0;
  Plan plan;
  const int rc = make_plan(B, K, V, r, 0, &plan);
  if (rc != DSPARK_OK) return rc;
  int n = 0;
  auto put = [&](int kind) {
    if (kinds && n < max_kinds) kinds[n] = kind;
    ++n;
  };
  if (plan.resident || plan.resident_mfma) {
    put(DSPARK_LAUNCH_RESIDENT_BLOCK);
  } else {
    for (int k = 0; k < K; ++k) {
      put(DSPARK_LAUNCH_FUSED_POSITION);
      if (!plan.in_kernel_pick) put(DSPARK_LAUNCH_PICK);
    }
  }
  put(DSPARK_LAUNCH_PROPOSAL);
  return n;
}

unsigned dspark_set_wait_limit(unsigned reads) {
  const unsigned prev = dspark::g_wait_limit;
  dspark::g_wait_limit = reads;
  return prev;
}

int dspark_block_status(int32_t* status, void* stream) {
  using namespace dspark;
  if (!status) return DSPARK_ERR_ARG;
  const int rc = init_device();
  if (rc != DSPARK_OK) return rc;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DSPARK_ERR_HIP;
  const DeviceInfo& info = g_devices[dev];
  hipLaunchKernelGGL(res_status, dim3(1), dim3(1), 0, static_cast<hipStream_t>(stream), info.exchange,
                     (unsigned)info.cus, status);
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP;
}

const char* dspark_status_string(int status) {
  switch (status) {
    case DSPARK_OK: return "ok";
    case DSPARK_ERR_ARG: return "invalid argument (null or misaligned pointer, bad size or dtype)";
    case DSPARK_ERR_UNSUPPORTED: return "unsupported size (V % 8, r % 32, r > 1024, K > 255, chunk)";
    case DSPARK_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case DSPARK_ERR_HIP: return "HIP runtime error";
    case DSPARK_ERR_SCRATCH: return "sizes need more scratch than dspark_draft_block_noalloc's static buffer holds";
    default: return "unknown status";
  }
}

}  // extern "C"
