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
// Three kernels per block, all on one stream (2K + 1 launches, capturable):
//   markov_bias_gumbel_argmax (once per position): streams W and the base
//     logits for one vocabulary chunk, forms the float32 biased logits, scales
//     by 1/T, adds Philox Gumbel noise, and leaves per-chunk softmax statistics
//     and a per-chunk (score, index) argmax partial.
//   pick_and_gather (once per position): reduces the partials of each row in
//     a fixed order, writes d_k and the row's (max, sum-exp), and gathers
//     E[d_k] for the next position.
//   proposal_softmax (once per block): q = exp(s - M) / S over all rows and
//     positions.
//
// Exact arithmetic conventions are stated in include/dspark.h. This file is
// compiled with FMA contraction off; the few products that may fuse use an
// explicit fmaf.

#include <hip/hip_runtime.h>

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "dspark.h"

namespace dspark {

constexpr int kThreads = 256;        // every kernel runs 256-thread workgroups (4 wave64)
constexpr int kTile = 128;           // vocabulary columns per tile of the fused kernel
constexpr int kSlices = 16;          // rank slices of the VALU bias GEMV (one per 16 threads)
constexpr int kMaxRank = 1024;
constexpr int kMaxK = 255;
constexpr int kDefaultChunk = kTile; // one tile per workgroup: ~1563 workgroups at V = 200064

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

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Running softmax statistics (m, l): l = sum exp(s - m).
struct Stat {
  float m;
  float l;
};

__device__ __forceinline__ Stat stat_merge(Stat a, Stat b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return Stat{-INFINITY, 0.0f};
  const float la = (a.m == -INFINITY) ? 0.0f : __fmul_rn(a.l, __expf(__fsub_rn(a.m, m)));
  const float lb = (b.m == -INFINITY) ? 0.0f : __fmul_rn(b.l, __expf(__fsub_rn(b.m, m)));
  return Stat{m, __fadd_rn(la, lb)};
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int mask, int width) {
  const uint32_t lo = __shfl_xor((uint32_t)x, mask, width);
  const uint32_t hi = __shfl_xor((uint32_t)(x >> 32), mask, width);
  return ((uint64_t)hi << 32) | lo;
}

struct StepArgs {
  const void* base;          // [B,K,V]
  const uint16_t* E;         // [V,r]
  const uint16_t* W;         // [r,V]
  const int32_t* prev_token; // [B], used at k == 0
  const uint16_t* e_buf;     // [B,r] bf16, E[d_{k-1}] gathered by pick_and_gather (k > 0)
  const int64_t* seed;
  const int64_t* offset;
  const float* temperature;
  const int32_t* n_real;     // may be null
  float* logits;             // [B,K,V]
  uint64_t* part_key;        // [B, n_chunks]
  Stat* part_stat;           // [B, n_chunks]
  int B, K, V, r, k;
  int chunk_cols, n_chunks;
};

// ---------------------------------------------------------------------------
// Kernel 1: markov_bias_gumbel_argmax, VALU GEMV form.
// Workgroup = one vocabulary chunk; rows are processed RB at a time. The bias
// tile [RB x 128] is a GEMV over r: thread t owns 8 columns (t % 16) and one
// rank slice (t / 16), loads W with 16-byte loads (a wave reads 4 rank rows x
// 256 contiguous bytes), and the 16 slices are summed through LDS in a fixed
// order. The epilogue gives each row 32 threads x 4 columns, so one Philox
// block serves the 4 columns a thread owns.
// ---------------------------------------------------------------------------
template <int RB, bool kBf16Base>
__global__ __launch_bounds__(kThreads) void markov_bias_gumbel_argmax_gemv(StepArgs a) {
  __shared__ float e_lds[RB][kMaxRank];
  __shared__ float red[kSlices][RB][kTile];
  __shared__ float bias_lds[RB][kTile];

  const int t = threadIdx.x;
  const int chunk = blockIdx.x;
  const int V = a.V, r = a.r, K = a.K, k = a.k;
  const int chunk_lo = chunk * a.chunk_cols;
  const int chunk_hi = min(V, chunk_lo + a.chunk_cols);
  const int n_real = a.n_real ? *a.n_real : a.B;

  const int cg = t % 16;          // 8-column group of the GEMV
  const int js = t / 16;          // rank slice of the GEMV
  const int er = t / 32;          // epilogue row within the row tile
  const int ec = (t % 32) * 4;    // epilogue column offset within the tile

  for (int rb0 = 0; rb0 < a.B; rb0 += RB) {
    // gather the Markov embedding rows of this row tile
    for (int i = t; i < RB * r; i += kThreads) {
      const int rr = i / r, j = i % r;
      const int b = rb0 + rr;
      float e = 0.0f;
      if (b < a.B) {
        uint16_t h;
        if (k == 0) {
          int d = a.prev_token[b];
          d = d < 0 ? 0 : (d > V - 1 ? V - 1 : d);
          h = a.E[(size_t)d * r + j];
        } else {
          h = a.e_buf[(size_t)b * r + j];
        }
        e = __uint_as_float((uint32_t)h << 16);
      }
      e_lds[rr][j] = e;
    }
    __syncthreads();

    // per-thread running state of its epilogue row over the chunk's tiles
    const int eb = rb0 + er;
    const bool e_row = (er < RB) && (eb < a.B);
    float T = 1.0f, invT = 1.0f;
    bool greedy = false, pad = false;
    uint32_t key0 = 0, key1 = 0, ctr2 = 0, ctr3 = 0;
    if (e_row) {
      T = a.temperature[eb];
      greedy = !(T > 0.0f);
      invT = greedy ? 0.0f : __fdiv_rn(1.0f, T);
      pad = eb >= n_real;
      const uint64_t sd = (uint64_t)a.seed[eb];
      const uint64_t of = (uint64_t)a.offset[eb];
      key0 = (uint32_t)sd;
      key1 = (uint32_t)(sd >> 32);
      ctr2 = (uint32_t)of;
      ctr3 = (uint32_t)(of >> 32);
    }
    uint64_t best = 0;
    Stat st{-INFINITY, 0.0f};

    for (int tile0 = chunk_lo; tile0 < chunk_hi; tile0 += kTile) {
      // ---- bias GEMV over the rank dimension
      float acc[RB][8];
#pragma unroll
      for (int rr = 0; rr < RB; ++rr)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[rr][i] = 0.0f;
      const int col = tile0 + cg * 8;
      if (col < chunk_hi) {
        const uint16_t* wp = a.W + col;
#pragma unroll 4
        for (int j = js; j < r; j += kSlices) {
          const uint4 w = *reinterpret_cast<const uint4*>(wp + (size_t)j * V);
          const float wf[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                               bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
#pragma unroll
          for (int rr = 0; rr < RB; ++rr) {
            const float e = e_lds[rr][j];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[rr][i] = fmaf(e, wf[i], acc[rr][i]);
          }
        }
      }
#pragma unroll
      for (int rr = 0; rr < RB; ++rr)
#pragma unroll
        for (int i = 0; i < 8; ++i) red[js][rr][cg * 8 + i] = acc[rr][i];
      __syncthreads();
      for (int o = t; o < RB * kTile; o += kThreads) {
        const int rr = o / kTile, c = o % kTile;
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < kSlices; ++q) s = __fadd_rn(s, red[q][rr][c]);
        bias_lds[rr][c] = s;
      }
      __syncthreads();

      // ---- epilogue: logits, 1/T, Gumbel noise, argmax and softmax statistics
      const int v0 = tile0 + ec;
      if (e_row && v0 < chunk_hi) {
        const size_t off = ((size_t)eb * K + k) * (size_t)V + v0;
        float base[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (!pad) {
          if (kBf16Base) {
            const uint2 h = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.base) + off);
            base[0] = bf16_lo(h.x); base[1] = bf16_hi(h.x);
            base[2] = bf16_lo(h.y); base[3] = bf16_hi(h.y);
          } else {
            const float4 f = *reinterpret_cast<const float4*>(static_cast<const float*>(a.base) + off);
            base[0] = f.x; base[1] = f.y; base[2] = f.z; base[3] = f.w;
          }
        }
        float lg[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) lg[i] = __fadd_rn(base[i], bias_lds[er][ec + i]);
        *reinterpret_cast<float4*>(a.logits + off) = make_float4(lg[0], lg[1], lg[2], lg[3]);
        if (greedy) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint64_t kk = score_key(lg[i], (uint32_t)(v0 + i));
            best = kk > best ? kk : best;
          }
        } else {
          const uint4 x = philox4x32_10(make_uint4((uint32_t)v0 >> 2, (uint32_t)k, ctr2, ctr3), key0, key1);
          const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
          float s[4];
          float m4 = -INFINITY;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            s[i] = __fmul_rn(lg[i], invT);
            const float z = __fadd_rn(s[i], gumbel_from_bits(xs[i]));
            const uint64_t kk = score_key(z, (uint32_t)(v0 + i));
            best = kk > best ? kk : best;
            m4 = fmaxf(m4, s[i]);
          }
          float l4 = 0.0f;
          if (m4 != -INFINITY) {
#pragma unroll
            for (int i = 0; i < 4; ++i) l4 = __fadd_rn(l4, __expf(__fsub_rn(s[i], m4)));
          }
          st = stat_merge(st, Stat{m4, l4});
        }
      }
      __syncthreads();  // red / bias_lds are rewritten by the next tile
    }

    // ---- reduce each row's 32 threads (one half-wave) and store the partials
    {
#pragma unroll
      for (int mask = 1; mask < 32; mask <<= 1) {
        const uint64_t ob = shfl_xor_u64(best, mask, 32);
        best = ob > best ? ob : best;
        Stat o;
        o.m = __shfl_xor(st.m, mask, 32);
        o.l = __shfl_xor(st.l, mask, 32);
        st = stat_merge(st, o);
      }
      if (e_row && (t % 32) == 0) {
        a.part_key[(size_t)eb * a.n_chunks + chunk] = best;
        a.part_stat[(size_t)eb * a.n_chunks + chunk] = st;
      }
    }
    __syncthreads();  // e_lds is rewritten by the next row tile
  }
}

// ---------------------------------------------------------------------------
// Kernel 2: pick_and_gather. One workgroup per row: the row's chunk partials
// are reduced in a fixed order (strided per thread, then a fixed tree), d_k
// and the merged (M, S) are written, and E[d_k] is gathered for position k+1.
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
  __shared__ uint64_t s_key[kThreads / 64];
  __shared__ Stat s_stat[kThreads / 64];
  __shared__ int32_t s_tok;
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  uint64_t best = 0;
  Stat st{-INFINITY, 0.0f};
  for (int c = t; c < a.n_chunks; c += kThreads) {
    const uint64_t kk = a.part_key[(size_t)b * a.n_chunks + c];
    best = kk > best ? kk : best;
    st = stat_merge(st, a.part_stat[(size_t)b * a.n_chunks + c]);
  }
#pragma unroll
  for (int mask = 1; mask < 64; mask <<= 1) {
    const uint64_t ob = shfl_xor_u64(best, mask, 64);
    best = ob > best ? ob : best;
    Stat o;
    o.m = __shfl_xor(st.m, mask, 64);
    o.l = __shfl_xor(st.l, mask, 64);
    st = stat_merge(st, o);
  }
  if ((t % 64) == 0) {
    s_key[t / 64] = best;
    s_stat[t / 64] = st;
  }
  __syncthreads();
  if (t == 0) {
    uint64_t bb = s_key[0];
    Stat ss = s_stat[0];
    for (int w = 1; w < kThreads / 64; ++w) {
      bb = s_key[w] > bb ? s_key[w] : bb;
      ss = stat_merge(ss, s_stat[w]);
    }
    int32_t d = (int32_t)(~(uint32_t)bb);
    d = d < 0 ? 0 : (d > a.V - 1 ? a.V - 1 : d);
    a.tokens[(size_t)b * a.K + a.k] = d;
    a.row_stat[(size_t)b * a.K + a.k] = ss;
    s_tok = d;
  }
  __syncthreads();
  if (a.k + 1 < a.K) {
    const uint16_t* src = a.E + (size_t)s_tok * a.r;
    for (int j = t; j < a.r; j += kThreads) a.e_buf[(size_t)b * a.r + j] = src[j];
  }
}

// ---------------------------------------------------------------------------
// Kernel 3: proposal_softmax. Every (row, position) is one grid row; each
// thread writes 4 consecutive entries of q. Sampling rows recompute
// s = logit * invT exactly as the draw did; greedy rows get one-hot at d_k.
// ---------------------------------------------------------------------------
struct PropArgs {
  const float* logits;
  const float* temperature;
  const int32_t* tokens;
  const Stat* row_stat;
  float* q;
  int B, K, V;
  int blocks_per_row;
};

__global__ __launch_bounds__(kThreads) void proposal_softmax(PropArgs a) {
  const int bk = blockIdx.x / a.blocks_per_row;
  const int b = bk / a.K;
  const int v0 = ((blockIdx.x % a.blocks_per_row) * kThreads + threadIdx.x) * 4;
  if (v0 >= a.V) return;
  const size_t off = (size_t)bk * a.V + v0;
  const float T = a.temperature[b];
  float4 out;
  if (!(T > 0.0f)) {
    const int tok = a.tokens[bk];
    out = make_float4(v0 == tok ? 1.0f : 0.0f, v0 + 1 == tok ? 1.0f : 0.0f,
                      v0 + 2 == tok ? 1.0f : 0.0f, v0 + 3 == tok ? 1.0f : 0.0f);
  } else {
    const float invT = __fdiv_rn(1.0f, T);
    const Stat st = a.row_stat[bk];
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
  uint64_t* part_key;
  Stat* part_stat;
  Stat* row_stat;
  uint16_t* e_buf;
};

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Layout for the largest chunk count (chunk = 128 columns).
inline size_t workspace_layout(int B, int K, int V, int r, Workspace* ws, char* base) {
  const size_t max_chunks = (size_t)(V + kTile - 1) / kTile;
  size_t off = 0;
  const size_t o_key = off; off = align_up(off + (size_t)B * max_chunks * sizeof(uint64_t), 256);
  const size_t o_pst = off; off = align_up(off + (size_t)B * max_chunks * sizeof(Stat), 256);
  const size_t o_rst = off; off = align_up(off + (size_t)B * K * sizeof(Stat), 256);
  const size_t o_e = off;   off = align_up(off + (size_t)B * r * sizeof(uint16_t), 256);
  if (ws) {
    ws->part_key = reinterpret_cast<uint64_t*>(base + o_key);
    ws->part_stat = reinterpret_cast<Stat*>(base + o_pst);
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

template <int RB>
hipError_t launch_step(const StepArgs& sa, bool bf16, hipStream_t stream) {
  const dim3 grid(sa.n_chunks), block(kThreads);
  if (bf16)
    hipLaunchKernelGGL((markov_bias_gumbel_argmax_gemv<RB, true>), grid, block, 0, stream, sa);
  else
    hipLaunchKernelGGL((markov_bias_gumbel_argmax_gemv<RB, false>), grid, block, 0, stream, sa);
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

  if (events && n_events < 2 * K + 2) return DSPARK_ERR_ARG;

  Workspace ws;
  workspace_layout(B, K, V, r, &ws, static_cast<char*>(workspace));
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  int n_marks = 0;
  auto mark = [&]() -> bool {
    if (!events) return true;
    return hipEventRecord(static_cast<hipEvent_t>(events[n_marks++]), stream) == hipSuccess;
  };
  if (!mark()) return DSPARK_ERR_HIP;
  const int n_chunks = (V + chunk_cols - 1) / chunk_cols;
  const bool bf16 = base_dtype == DSPARK_BF16;

  for (int k = 0; k < K; ++k) {
    StepArgs sa;
    sa.base = base; sa.E = E; sa.W = W; sa.prev_token = prev_token; sa.e_buf = ws.e_buf;
    sa.seed = seed; sa.offset = offset; sa.temperature = temperature; sa.n_real = n_real;
    sa.logits = logits; sa.part_key = ws.part_key; sa.part_stat = ws.part_stat;
    sa.B = B; sa.K = K; sa.V = V; sa.r = r; sa.k = k;
    sa.chunk_cols = chunk_cols; sa.n_chunks = n_chunks;
    const hipError_t err = (B == 1) ? launch_step<1>(sa, bf16, stream) : launch_step<4>(sa, bf16, stream);
    if (err != hipSuccess || !mark()) return DSPARK_ERR_HIP;

    PickArgs pa;
    pa.part_key = ws.part_key; pa.part_stat = ws.part_stat; pa.E = E; pa.tokens = tokens;
    pa.row_stat = ws.row_stat; pa.e_buf = ws.e_buf;
    pa.B = B; pa.K = K; pa.V = V; pa.r = r; pa.k = k; pa.n_chunks = n_chunks;
    hipLaunchKernelGGL(pick_and_gather, dim3(B), dim3(kThreads), 0, stream, pa);
    if (hipGetLastError() != hipSuccess || !mark()) return DSPARK_ERR_HIP;
  }

  PropArgs pr;
  pr.logits = logits; pr.temperature = temperature; pr.tokens = tokens; pr.row_stat = ws.row_stat;
  pr.q = q; pr.B = B; pr.K = K; pr.V = V;
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
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_gemv<1, false>),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_gemv<1, true>),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_gemv<4, false>),
      reinterpret_cast<const void*>(&markov_bias_gumbel_argmax_gemv<4, true>),
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
