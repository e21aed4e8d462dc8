// dspark.hip -- DSpark ancestral draft-block sampler for MI355X (gfx950).
//
// The method ("brb-nv/TensorRT-LLM pull 21", section "2. Golden sampling
// semantics"; "brb-nv/TensorRT-LLM pull 27", section "2. One fused kernel per
// draft position"): position k of a draft block is drawn from
// softmax((base_k + bias(d_{k-1})) / T) by Gumbel-max, where bias(d) = E[d] . W
// is a rank-r Markov head and d_{k-1} the token drawn just before; after the
// block the proposal q_k = softmax(logits_k / T) is written from the same
// float32 logits the draw used.
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
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    if (round) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo_a = 0xD2511F53u * c.x;
    const uint32_t hi_a = __umulhi(0xD2511F53u, c.x);
    const uint32_t lo_b = 0xCD9E8D57u * c.z;
    const uint32_t hi_b = __umulhi(0xCD9E8D57u, c.z);
    c = make_uint4(hi_b ^ c.y ^ k0, lo_b, hi_a ^ c.w ^ k1, lo_a);
  }
  return c;
}

// Standard Gumbel variate from the top 23 bits of a Philox word:
// u = ((x >> 9) + 1/2) 2^-23 is exact in float32; g = -ln(-ln u).
__device__ __forceinline__ float gumbel_from_bits(uint32_t x) {
  const float u = __fmul_rn(__fadd_rn((float)(x >> 9), 0.5f), 0x1p-23f);
  return -logf(-logf(u));
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

__device__ __forceinline__ RowState row_state(const StepArgs& a, int b, int n_real) {
  RowState rs;
  const float T = a.temperature[b];
  rs.greedy = !(T > 0.0f);
  rs.invT = rs.greedy ? 0.0f : __fdiv_rn(1.0f, T);
  rs.pad = b >= n_real;
  const uint64_t sd = (uint64_t)a.seed[b];
  const uint64_t of = (uint64_t)a.offset[b];
  rs.key0 = (uint32_t)sd;
  rs.key1 = (uint32_t)(sd >> 32);
  rs.ctr2 = (uint32_t)of;
  rs.ctr3 = (uint32_t)(of >> 32);
  return rs;
}

// Base logits of 4 consecutive columns, loaded early and widened late.
template <bool kBf16Base>
struct Base4 {
  uint2 h;
  float4 f;
};

template <bool kBf16Base>
__device__ __forceinline__ void load_base4(Base4<kBf16Base>& bv, const void* base, size_t off) {
  if (kBf16Base)
    bv.h = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + off);
  else
    bv.f = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
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
// Kernel 3: proposal_softmax. Grid = (row, position) x column blocks; each
// thread writes 4 consecutive entries of q. Sampling rows recompute
// s = logit * invT exactly as the draw did; greedy rows get one-hot at d_k.
// With last_from_partials (B == 1), the last position's token and (M, S) are
// reduced here from its chunk partials; block 0 of that row stores them.
// ---------------------------------------------------------------------------
struct PropArgs {
  const float* logits;
  const float* temperature;
  int32_t* tokens;
  Stat* row_stat;
  const uint64_t* last_key;   // [B,C] partials of position K-1 (last_from_partials)
  const Stat* last_stat;
  float* q;
  int B, K, V, n_chunks;
  int blocks_per_row;
  int last_from_partials;
};

__global__ __launch_bounds__(kThreads) void proposal_softmax(PropArgs a) {
  __shared__ uint64_t s_key[kWaves];
  __shared__ Stat s_stat[kWaves];
  const int bk = blockIdx.x / a.blocks_per_row;
  const int cb = blockIdx.x % a.blocks_per_row;
  const int b = bk / a.K;
  const int k = bk % a.K;
  const int v0 = (cb * kThreads + threadIdx.x) * 4;
  const float T = a.temperature[b];
  const bool greedy = !(T > 0.0f);

  Stat st;
  int tok;
  if (a.last_from_partials && k == a.K - 1) {
    uint64_t best = 0;
    Stat sst{-INFINITY, 0.0f};
    for (int c = threadIdx.x; c < a.n_chunks; c += kThreads) {
      best = umax64(best, a.last_key[(size_t)b * a.n_chunks + c]);
      sst = stat_merge(sst, a.last_stat[(size_t)b * a.n_chunks + c]);
    }
    wg_reduce(best, sst, s_key, s_stat);
    st = sst;
    tok = clamp_token((int)key_token(best), a.V);
    if (cb == 0 && threadIdx.x == 0) {
      a.tokens[bk] = tok;
      a.row_stat[bk] = st;
    }
  } else {
    st = a.row_stat[bk];
    tok = a.tokens[bk];
  }
  if (v0 >= a.V) return;
  const size_t off = (size_t)bk * a.V + v0;
  float4 out;
  if (greedy) {
    out = make_float4(v0 == tok ? 1.0f : 0.0f, v0 + 1 == tok ? 1.0f : 0.0f,
                      v0 + 2 == tok ? 1.0f : 0.0f, v0 + 3 == tok ? 1.0f : 0.0f);
  } else {
    const float invT = __fdiv_rn(1.0f, T);
    const float invS = __fdiv_rn(1.0f, st.l);
    const float4 lg = *reinterpret_cast<const float4*>(a.logits + off);
    out.x = __fmul_rn(__expf(__fsub_rn(__fmul_rn(lg.x, invT), st.m)), invS);
    out.y = __fmul_rn(__expf(__fsub_rn(__fmul_rn(lg.y, invT), st.m)), invS);
    out.z = __fmul_rn(__expf(__fsub_rn(__fmul_rn(lg.z, invT), st.m)), invS);
    out.w = __fmul_rn(__expf(__fsub_rn(__fmul_rn(lg.w, invT), st.m)), invS);
  }
  *reinterpret_cast<float4*>(a.q + off) = out;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
struct Workspace {
  uint64_t* part_key[2];   // double-buffered by position parity
  Stat* part_stat[2];
  Stat* row_stat;
  uint16_t* e_buf;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Layout for the largest chunk count (chunk = 128 columns).
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
  if (ws) {
    for (int i = 0; i < 2; ++i) {
      ws->part_key[i] = reinterpret_cast<uint64_t*>(base + o_key[i]);
      ws->part_stat[i] = reinterpret_cast<Stat*>(base + o_pst[i]);
    }
    ws->row_stat = reinterpret_cast<Stat*>(base + o_rst);
    ws->e_buf = reinterpret_cast<uint16_t*>(base + o_e);
  }
  return off;
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

int draft_block_impl(const void* base, int base_dtype, const uint16_t* E, const uint16_t* W,
                     const int32_t* prev_token, const int64_t* seed, const int64_t* offset,
                     const float* temperature, const int32_t* n_real, int B, int K, int V, int r,
                     int chunk_cols, int32_t* tokens, float* logits, float* q, void* workspace,
                     size_t workspace_bytes, void* stream_ptr, void* const* events = nullptr,
                     int n_events = 0) {
  int rc = check_sizes(B, K, V, r);
  if (rc != DSPARK_OK) return rc;
  if (base_dtype != DSPARK_F32 && base_dtype != DSPARK_BF16) return DSPARK_ERR_ARG;
  if (chunk_cols < 0 || chunk_cols % kTile != 0) return DSPARK_ERR_UNSUPPORTED;
  if (chunk_cols == 0) chunk_cols = kDefaultChunk;
  if (B == 0 || K == 0) return DSPARK_OK;
  if (!base || !E || !W || !prev_token || !seed || !offset || !temperature || !tokens || !logits ||
      !q)
    return DSPARK_ERR_ARG;
  if (!aligned16(base) || !aligned16(E) || !aligned16(W) || !aligned16(logits) || !aligned16(q))
    return DSPARK_ERR_ARG;
  const size_t need = workspace_layout(B, K, V, r, nullptr, nullptr);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return DSPARK_ERR_WORKSPACE;

  const int n_chunks = (V + chunk_cols - 1) / chunk_cols;
  // one row: every workgroup picks the previous token itself (no pick launch)
  const bool in_kernel_pick = (B == 1) && n_chunks <= kPickPerThread * kThreads;
  const int n_launches = in_kernel_pick ? K + 1 : 2 * K + 1;
  if (events && n_events < n_launches + 1) return DSPARK_ERR_ARG;

  Workspace ws;
  workspace_layout(B, K, V, r, &ws, static_cast<char*>(workspace));
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  int n_marks = 0;
  auto mark = [&]() -> bool {
    if (!events) return true;
    return hipEventRecord(static_cast<hipEvent_t>(events[n_marks++]), stream) == hipSuccess;
  };
  if (!mark()) return DSPARK_ERR_HIP;
  const bool bf16 = base_dtype == DSPARK_BF16;

  for (int k = 0; k < K; ++k) {
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
  pr.last_from_partials = in_kernel_pick ? 1 : 0;
  pr.blocks_per_row = (V + kThreads * 4 - 1) / (kThreads * 4);
  const long long n_blocks = (long long)pr.blocks_per_row * B * K;
  if (n_blocks >= (1LL << 31)) return DSPARK_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(proposal_softmax, dim3((unsigned)n_blocks), dim3(kThreads), 0, stream, pr);
  if (hipGetLastError() != hipSuccess || !mark()) return DSPARK_ERR_HIP;
  return DSPARK_OK;
}

}  // namespace dspark

extern "C" {

int dspark_init(void) {
  using namespace dspark;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DSPARK_ERR_HIP;
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
      reinterpret_cast<const void*>(&proposal_softmax),
  };
  for (const void* kfn : kernels)
    if (hipFuncGetAttributes(&attr, kfn) != hipSuccess) return DSPARK_ERR_HIP;
  return DSPARK_OK;
}

size_t dspark_workspace_bytes(int B, int K, int V, int r) {
  if (dspark::check_sizes(B, K, V, r) != DSPARK_OK) return 0;
  return dspark::workspace_layout(B, K, V, r, nullptr, nullptr);
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

const char* dspark_status_string(int status) {
  switch (status) {
    case DSPARK_OK: return "ok";
    case DSPARK_ERR_ARG: return "invalid argument (null or misaligned pointer, bad size or dtype)";
    case DSPARK_ERR_UNSUPPORTED: return "unsupported size (V % 8, r % 32, r > 1024, K > 255, chunk)";
    case DSPARK_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case DSPARK_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
