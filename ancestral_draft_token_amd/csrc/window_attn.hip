// window_attn.hip -- non-causal windowed block attention of a DSpark drafter
// layer on gfx950 (MI355X).
//
// What it computes ("brb-nv/TensorRT-LLM pull 21", section "1. Non-causal
// DSpark draft blocks on TRTLLM (default path)"; the modeling_dspark.py /
// modeling_dflash.py note of the MiniMax-M3.1-Flash page): K draft-block
// queries at positions P .. P+K-1 after a context of P tokens; query i
// attends every existing key t (t < P + K) with |i - t| <= W - 1: the
// whole draft block and the context keys at most W - 1 positions back. GQA: 16 query
// heads share one key/value head. Outputs o (float32) and the log-sum-exp
// (natural log) of every (position, query head).
//
// On the pages' hardware this runs as a causal sliding-window decode whose
// log-sum-exp is then merged with the keys of the rest of the block, since
// their attention kernel has only a causal window.
// Here the two-sided window is computed directly: one pass over the key
// range [max(0, P - W + 1), P + K), split over workgroups, each query
// masking its own lower bound; the splits are then combined by the same
// log-sum-exp merge.
//
// wa_partials: one 512-thread workgroup per (split, key/value head, row).
// The key range is streamed in tiles of 64 keys through LDS (K as rows with
// swizzled 16-byte chunks, V transposed as dim rows with swizzled key pairs),
// the next tile's global loads in flight while the current one is used.
// Wave w owns draft position w (eight waves, ~124 registers: four waves per
// SIMD); a position's 16 heads are one MFMA tile. Scores are computed transposed,
// S^T = K Q^T (v_mfma_f32_16x16x32_bf16: M = 16 keys, N = 16 heads, 4 steps
// over D = 128), with the keys of each 32-key step assigned to the two score
// tiles so that the accumulators land exactly in the B-operand layout of the
// second product, O^T += V^T P^T (M = 16 dims x 8 tiles, N = 16 heads, 32 keys
// per step): each lane holds keys 8 (lane / 16) .. + 7 of one head, with no
// data movement between the two products. Online softmax in base 2 per head;
// probabilities rounded to bf16 for the second product.
// wa_combine: one 256-thread block per (position, key/value head, row)
// merges the splits of its 16 heads (wa_combine_splits, for many splits,
// spreads one head's splits over its threads): M = max m_s, L = sum l_s 2^(m_s - M), o = sum 2^(m_s - M) o_s / L,
// lse = (M + log2 L) ln 2.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "dspark.h"

namespace dspark_wa {

constexpr int kD = 128;                      // head dimension
constexpr int kG = 16;                       // query heads per key/value head
constexpr int kKMax = 8;                     // draft positions: one per wave of wa_partials
constexpr int kThreads = 256;                // wa_combine
constexpr int kQ = 1;                        // draft positions per wave of wa_partials
constexpr int kPW = kKMax / kQ;              // waves of a wa_partials workgroup
constexpr int kPartThreads = 64 * kPW;

constexpr int kTileKeys = 64;
constexpr int kKUnits = kTileKeys * 16 / kPartThreads;       // 16-byte K pieces a thread stages per tile
constexpr int kVUnits = kTileKeys / 2 * 16 / kPartThreads;   // (key pair, 8 dims) V pieces
constexpr int kKRow = kD * 2;                // LDS bytes per key row (16-byte chunks swizzled by row)
constexpr int kVRow = kTileKeys * 2 + 16;    // LDS bytes per transposed V row (one dim, 64 keys)
constexpr int kLdsK = kTileKeys * kKRow;     // 17,408
constexpr int kLdsV = kD * kVRow;            // 18,432
constexpr int kSlots = 512;                  // resident workgroups: two per CU on 256 CUs
constexpr int kMaxSplits = 128;              // splits of one key range at most (wa_combine_splits' table)
constexpr int kFewSplits = 16;               // up to this many, each merge thread walks the splits itself
constexpr double kMergeBatchCost = 0.2;      // one batch of eight splits' reads in the merge, in tiles

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  c, 0, 0, 0);
}

// two float32 -> a packed bf16 pair (low half first), round to nearest even:
// one v_cvt_pk_bf16_f32 on gfx950
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// K rows in LDS: 16-byte chunk j of row r sits at chunk j ^ kswz(r). The 16
// rows one score-tile read touches (r = 32 st + 8 (c / 4) + 4 tt + c % 4 for
// c = 0..15) get 16 different offsets, so a read is free of bank conflicts
// with 32 or 64 banks; the stores (16 lanes per row) stay conflict-free.
__device__ __forceinline__ int kswz(int r) { return (r & 3) | (((r >> 3) & 3) << 2); }

struct WaArgs {
  const uint16_t* q;        // [B,K,Hq,D] bf16
  const uint16_t* kc;       // [B,L,Hkv,D] bf16
  const uint16_t* vc;       // [B,L,Hkv,D] bf16
  const int32_t* ctx_len;   // [B]
  float* part_o;            // [B][Hkv][S][K][16][D] unnormalised partial outputs
  float* part_ml;           // [B][Hkv][S][K][16][2]: running max (base-2 units) and sum
  float* out;               // [B,K,Hq,D]
  float* lse;               // [B,K,Hq]
  int B, K, Hkv, L, W, S, keys_per_split;
  float scale_log2;         // scale * log2(e)
  size_t key_stride;        // cache elements between consecutive keys of one head
  size_t head_stride;       // cache elements between the heads of one key
};

// The first element of row b, head kvh in a cache of either layout (a row
// holds L * Hkv * D elements in both).
__device__ __forceinline__ const uint16_t* cache_head(const uint16_t* cache, const WaArgs& a, int b, int kvh) {
  return cache + (size_t)b * a.L * a.Hkv * kD + (size_t)kvh * a.head_stride;
}

__device__ __forceinline__ int clamp_ctx(const WaArgs& a, int b) {
  const int P = a.ctx_len[b];
  return P < 0 ? 0 : (P > a.L - a.K ? a.L - a.K : P);
}

// Transposed V rows are swizzled: key pair j of dim row d is stored at pair
// j ^ (4 ((d / 16) % 8)), which keeps the transposing stores and the
// fragment reads free of bank conflicts (rows of 144 bytes).
__global__ __launch_bounds__(kPartThreads, 4) void wa_partials(WaArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsK + kLdsV];
  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int Hq = a.Hkv * kG;
  const int P = clamp_ctx(a, b);
  const int lo0 = P - (a.W - 1) > 0 ? P - (a.W - 1) : 0;
  const int hi = P + a.K;
  const int k_begin = lo0 + s * a.keys_per_split;
  const int k_end = k_begin + a.keys_per_split < hi ? k_begin + a.keys_per_split : hi;
  const size_t rs = a.key_stride;                                       // elements between keys
  const uint16_t* kb = cache_head(a.kc, a, b, kvh);
  const uint16_t* vb = cache_head(a.vc, a, b, kvh);
  const size_t pslot = (((size_t)b * a.Hkv + kvh) * a.S + s) * a.K;    // (b, kvh, s, position 0)

  // the two draft positions of this wave and their query fragments:
  // lane (c, g) holds head kvh*16 + c, dims 32 ds + 8 g .. + 7
  int kq[kQ];
  bool has[kQ];
  u32x4_t qf[kQ][4];
#pragma unroll
  for (int qi = 0; qi < kQ; ++qi) {
    kq[qi] = wv + kPW * qi;
    has[qi] = kq[qi] < a.K;
    const uint16_t* qrow = a.q + (((size_t)b * a.K + (has[qi] ? kq[qi] : 0)) * Hq + kvh * kG + c) * kD;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
      qf[qi][ds] = has[qi] ? *reinterpret_cast<const u32x4_t*>(qrow + 32 * ds + 8 * g) : u32x4_t{0u, 0u, 0u, 0u};
  }
  f32x4_t acc[kQ][8];
  float m[kQ], l[kQ];
#pragma unroll
  for (int qi = 0; qi < kQ; ++qi) {
    m[qi] = -INFINITY;
    l[qi] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[qi][dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // staging: K rows as 16-byte pieces (16 lanes per 256-byte row), V as
  // pairs of keys x 8 dims (written transposed, a dword per dim)
  static_assert(kKUnits == 2 && kVUnits == 1, "staging below is written for 512 threads");
  uint4 ks0, ks1, vs0, vs1;
#define WA_LOAD_TILE(tb)                                                                              \
  do {                                                                                                \
    const int tb_ = (tb);                                                                             \
    const int r0_ = tb_ + (t >> 4), r1_ = r0_ + 32, cw_ = (t & 15) * 8;                               \
    ks0 = *reinterpret_cast<const uint4*>(kb + (size_t)(r0_ < hi ? r0_ : hi - 1) * rs + cw_);         \
    ks1 = *reinterpret_cast<const uint4*>(kb + (size_t)(r1_ < hi ? r1_ : hi - 1) * rs + cw_);         \
    const int p_ = tb_ + 2 * (t >> 4);                                                                \
    vs0 = *reinterpret_cast<const uint4*>(vb + (size_t)(p_ < hi ? p_ : hi - 1) * rs + cw_);           \
    vs1 = *reinterpret_cast<const uint4*>(vb + (size_t)(p_ + 1 < hi ? p_ + 1 : hi - 1) * rs + cw_);   \
  } while (0)

  const int n_tiles = k_begin < k_end ? (k_end - k_begin + kTileKeys - 1) / kTileKeys : 0;
  if (n_tiles > 0) WA_LOAD_TILE(k_begin);
  const int lo_max = P + a.K - 1 - (a.W - 1);   // the largest lower bound of a position
  for (int n = 0; n < n_tiles; ++n) {
    const int tb = k_begin + n * kTileKeys;
    __syncthreads();   // the previous tile is no longer read
    {
      // K pieces: rows t / 16 and t / 16 + 32, chunk t % 16 (swizzled); V: key
      // pair t / 16, dims 8 (t % 16) .. + 7, transposed and swizzled
      const int kr = t >> 4, kc = t & 15;
      *reinterpret_cast<uint4*>(lds + kr * kKRow + 16 * (kc ^ kswz(kr))) = ks0;
      *reinterpret_cast<uint4*>(lds + (kr + 32) * kKRow + 16 * (kc ^ kswz(kr + 32))) = ks1;
      const int sl = 4 * (kr ^ (4 * ((kc >> 1) & 7)));
      unsigned char* vd = lds + kLdsK + kc * 8 * kVRow + sl;
      const uint32_t a0[4] = {vs0.x, vs0.y, vs0.z, vs0.w};
      const uint32_t a1[4] = {vs1.x, vs1.y, vs1.z, vs1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = 16 * (e & 1);
        *reinterpret_cast<uint32_t*>(vd + e * kVRow) =
            ((a0[e >> 1] >> sh) & 0xFFFFu) | (((a1[e >> 1] >> sh) & 0xFFFFu) << 16);
      }
    }
    __syncthreads();
    if (n + 1 < n_tiles) WA_LOAD_TILE(tb + kTileKeys);   // in flight while this tile is used

    // scores of the whole tile: sc[qi][2 st + tt]; score tile (st, tt) has A
    // row r = key 32 st + 8 (r / 4) + 4 tt + r % 4, so lane (c, g) ends up with
    // keys 32 st + 8 g + 4 tt + i of head c
    f32x4_t sc[kQ][4];
#pragma unroll
    for (int qi = 0; qi < kQ; ++qi)
#pragma unroll
      for (int u = 0; u < 4; ++u) sc[qi][u] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int krow = 32 * (u >> 1) + 8 * (c >> 2) + 4 * (u & 1) + (c & 3);
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
        const u32x4_t af = *reinterpret_cast<const u32x4_t*>(lds + krow * kKRow + 16 * ((4 * ds + g) ^ kswz(krow)));
#pragma unroll
        for (int qi = 0; qi < kQ; ++qi)
          if (has[qi]) sc[qi][u] = mfma_bf16(af, qf[qi][ds], sc[qi][u]);
      }
    }
    // only the tiles at a split's ends or below a position's window start mask
    const bool edge = tb < lo_max || tb + kTileKeys > k_end;
    // both positions' probabilities first, so each V^T fragment is read once
    // per wave: pb[qi][st] is the bf16 B operand of keys 32 st + 8 g .. + 7
    u32x4_t pb[kQ][2];
    bool live[kQ];
#pragma unroll
    for (int qi = 0; qi < kQ; ++qi) {
      pb[qi][0] = pb[qi][1] = u32x4_t{0u, 0u, 0u, 0u};
      live[qi] = false;
      if (!has[qi]) continue;
      // x[8 st + j]: key tb + 32 st + 8 g + j
      float x[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) x[j] = sc[qi][2 * (j >> 3) + ((j >> 2) & 1)][j & 3];   // raw <q, k>
      if (edge) {
        const int lo_k = P + kq[qi] - (a.W - 1);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int kt = tb + 32 * (j >> 3) + 8 * g + (j & 7);
          if (!(kt >= lo_k && kt < k_end)) x[j] = -INFINITY;
        }
      }
      // the maximum of the raw scores, then scaled (the scale is positive);
      // the exponent below is one fma per score
      float mt = x[0];
#pragma unroll
      for (int j = 1; j < 16; ++j) mt = fmaxf(mt, x[j]);
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      mt *= a.scale_log2;
      if (mt == -INFINITY && m[qi] == -INFINITY) continue;   // no key of this position yet (uniform)
      live[qi] = true;
      if (mt > m[qi]) {
        // the running maximum grows: rescale (skipped once it has settled)
        const float alpha = __builtin_amdgcn_exp2f(m[qi] - mt);
        l[qi] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[qi][dt] *= alpha;
        m[qi] = mt;
      }
      float ps = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        x[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[j], a.scale_log2, -m[qi]));
        ps += x[j];
      }
      l[qi] += ps;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const float* pp = x + 8 * st;
        pb[qi][st] = u32x4_t{pack_bf16(pp[0], pp[1]), pack_bf16(pp[2], pp[3]), pack_bf16(pp[4], pp[5]),
                             pack_bf16(pp[6], pp[7])};
      }
    }
    // O^T += V^T P^T; V^T fragment of dim 16 dt + c: logical key pairs
    // 16 st + 4 g .. + 3, stored at pair (16 st + 4 g) ^ 4 dt
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const u32x4_t vf = *reinterpret_cast<const u32x4_t*>(lds + kLdsK + (16 * dt + c) * kVRow +
                                                             4 * ((16 * st + 4 * g) ^ (4 * dt)));
#pragma unroll
        for (int qi = 0; qi < kQ; ++qi)
          if (live[qi]) acc[qi][dt] = mfma_bf16(vf, pb[qi][st], acc[qi][dt]);
      }
    }
  }
#undef WA_LOAD_TILE

  // partials: lane (c, g) holds O^T dims 16 dt + 4 g .. + 3 of head c
#pragma unroll
  for (int qi = 0; qi < kQ; ++qi) {
    if (!has[qi]) continue;
    float lt = l[qi];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const size_t row = (pslot + kq[qi]) * kG + c;
    float* po = a.part_o + row * kD;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4_t*>(po + 16 * dt + 4 * g) = acc[qi][dt];
    if (g == 0) {
      a.part_ml[2 * row] = m[qi];
      a.part_ml[2 * row + 1] = lt;
    }
  }
}

// One 256-thread block per (position, key/value head, row): thread t merges
// dims 8 (t % 16) .. + 7 of head t / 16 over the splits. The 16 threads of a
// head read the same (max, sum) words (cached) and each computes the
// weights itself; the partial outputs are read as float4.
__global__ __launch_bounds__(kThreads) void wa_combine(WaArgs a) {
  const int k = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int c = t >> 4, d0 = 8 * (t & 15);
  const int Hq = a.Hkv * kG;
  // row of split s: base + s * stride
  const size_t base = ((((size_t)b * a.Hkv + kvh) * a.S) * a.K + k) * kG + c;
  const size_t stride = (size_t)a.K * kG;
  float M = -INFINITY;
#pragma unroll 4
  for (int s = 0; s < a.S; ++s) M = fmaxf(M, a.part_ml[2 * (base + s * stride)]);
  float Ls = 0.0f;
  f32x4_t o0{0.0f, 0.0f, 0.0f, 0.0f}, o1{0.0f, 0.0f, 0.0f, 0.0f};
  // unrolled so several splits' loads are in flight; a split without a key
  // of this head (max -inf) gets weight 0 and its (finite) partial adds 0
#pragma unroll 4
  for (int s = 0; s < a.S; ++s) {
    const size_t row = base + s * stride;
    const float ms = a.part_ml[2 * row];
    const float ls = a.part_ml[2 * row + 1];
    const f32x4_t* po = reinterpret_cast<const f32x4_t*>(a.part_o + row * kD + d0);
    const f32x4_t p0 = po[0], p1 = po[1];
    const float w = ms == -INFINITY ? 0.0f : exp2f(ms - M);
    Ls += ls * w;
    o0 += p0 * w;
    o1 += p1 * w;
  }
  const size_t orow = ((size_t)b * a.K + k) * Hq + kvh * kG + c;
  f32x4_t* out = reinterpret_cast<f32x4_t*>(a.out + orow * kD + d0);
  out[0] = o0 / Ls;
  out[1] = o1 / Ls;
  if ((t & 15) == 0) a.lse[orow] = (M + log2f(Ls)) * 0.69314718055994531f;
}

// The merge for many splits (small batches: B=1 has 65): one 128-thread
// block per (head, position, row), the splits' maxima and weights read in
// parallel (one split per thread), eight splits' partial outputs in flight.
__global__ __launch_bounds__(kD) void wa_combine_splits(WaArgs a) {
  __shared__ float s_w[kMaxSplits];
  __shared__ float s_red[2][kD / 64];
  const int h = blockIdx.x, k = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  const int kvh = h / kG, c = h % kG;
  const int Hq = a.Hkv * kG;
  // row of split s: base + s * stride
  const size_t base = ((((size_t)b * a.Hkv + kvh) * a.S) * a.K + k) * kG + c;
  const size_t stride = (size_t)a.K * kG;
  // the splits' maxima and sums, one split per thread (every split is read once)
  float mx = -INFINITY;
  for (int s = d; s < a.S; s += kD) mx = fmaxf(mx, a.part_ml[2 * (base + s * stride)]);
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if ((d & 63) == 0) s_red[0][d >> 6] = mx;
  __syncthreads();
  float M = s_red[0][0];
  for (int w = 1; w < kD / 64; ++w) M = fmaxf(M, s_red[0][w]);
  float ls = 0.0f;
  for (int s = d; s < a.S; s += kD) {
    const float ms = a.part_ml[2 * (base + s * stride)];
    const float wgt = ms == -INFINITY ? 0.0f : exp2f(ms - M);   // a split without a key of this head: 0
    s_w[s] = wgt;
    ls += a.part_ml[2 * (base + s * stride) + 1] * wgt;
  }
  for (int o = 32; o >= 1; o >>= 1) ls += __shfl_xor(ls, o);
  if ((d & 63) == 0) s_red[1][d >> 6] = ls;
  __syncthreads();
  float Ls = s_red[1][0];
  for (int w = 1; w < kD / 64; ++w) Ls += s_red[1][w];
  // the weighted sum of the partial outputs, 8 splits' loads in flight
  float o = 0.0f;
  int s = 0;
  for (; s + 8 <= a.S; s += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = s_w[s + i] == 0.0f ? 0.0f : a.part_o[(base + (s + i) * stride) * kD + d];
#pragma unroll
    for (int i = 0; i < 8; ++i) o += v[i] * s_w[s + i];
  }
  for (; s < a.S; ++s)
    if (s_w[s] != 0.0f) o += a.part_o[(base + s * stride) * kD + d] * s_w[s];
  const size_t orow = ((size_t)b * a.K + k) * Hq + h;
  a.out[orow * kD + d] = o / Ls;
  if (d == 0) a.lse[orow] = (M + log2f(Ls)) * 0.69314718055994531f;
}

// ---------------------------------------------------------------------------
// wa_block: the large-batch form. One 256-thread workgroup (four waves) per
// (key/value head, row), two per CU (up to 256 registers a lane: two waves
// per SIMD, so one hides the other's latencies). The key range streams
// through an LDS ring of kNB tiles of 32 keys, loaded straight from HBM into
// LDS by LDS-direct loads (no registers), kNB - 1 tiles ahead; each wave
// loads 8 keys of every tile. The waves split the draft positions (wave w:
// positions kPos w .. + kPos - 1) and each reads the whole tile from LDS, so
// a position's softmax and output stay in one wave and no merge is needed:
//   scores S^T = K Q^T (v_mfma_f32_16x16x32_bf16: 16 keys x 16 heads, 4 steps
//     over D) for each half of the tile, K rows with their 16-byte chunks
//     XOR-swizzled by key (the swizzle is applied by choosing each lane's
//     source chunk);
//   O^T += V^T P^T over all 32 keys at once (v_mfma_f32_16x16x32_bf16: 16 dims
//     x 16 heads). The reduction index pairs k = 8 g + 4 h + i with key
//     16 h + 4 g + i, which is where the score accumulators already hold
//     P^T (lane (c, g) of half h: keys 16 h + 4 g + i of head c), so they are
//     the B operand once packed. The A operand (dim 16 dt + c of those 8
//     keys) comes from two transposing LDS reads ds_read_b64_tr_b16 of the
//     row-major V tile: lane r of a 16-lane group reads 4 dims of key r / 4
//     and lane j receives dim j of the group's 4 keys.
// Online softmax in base 2 per position and head, with a reference that moves
// only when a score passes it by a margin (below); outputs are normalised and
// written by the wave that owns them.
// ---------------------------------------------------------------------------
constexpr int kBT = 32;                        // keys per tile (each wave loads 8)
constexpr int kBWaves = 4;
constexpr int kBThreads = 64 * kBWaves;
constexpr int kNB = 4;                         // tiles in the LDS ring
constexpr int kBTile = kBT * kD * 2;           // bytes of one tensor's tile (8 KB)
constexpr int kBLds = kNB * 2 * kBTile;        // 64 KB
constexpr long long kBlockMinPairs = 256;      // (row, key/value head) pairs from which wa_block is used
constexpr float kTau = 8.0f;                   // lazy softmax reference: e stays below 2^kTau
static_assert(kKMax <= 2 * kBWaves, "positions per wave");
constexpr int kBRows = kBT / kBWaves;          // key rows each wave loads per tile
constexpr int kBLoads = 2 * kBRows / 4;        // its LDS-direct loads per tile (K and V, 4 rows each)

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// Chunk swizzles of the ring rows (256 bytes, 16 chunks of 16 bytes): logical
// chunk j of key row r sits at physical chunk j ^ swz(r). K: r % 16, so the
// 16 rows of a fragment read (one chunk each) hit 16 different chunks. V:
// 2 (r % 8), so the 4 rows of a transposing read's 16-lane group (a chunk
// pair each) hit 4 different pairs.
__device__ __forceinline__ int kswz_b(int r) { return r & 15; }
__device__ __forceinline__ int vswz_b(int r) { return 2 * (r & 7); }

// s_waitcnt vmcnt(n) with the other counters left alone (n < 64)
#define WA_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

// One LDS-direct load, 16 bytes a lane: lane i's bytes at gsrc land at LDS
// byte lds + 16 i (lds wave-uniform, in M0). Written out so that the compiler
// does not tie later LDS reads to these loads (it would make every read wait
// for all of them, emptying the ring); the tile loop waits for them itself
// with vmcnt, which counts them in issue order like any vector memory load.
// The instruction writes no register; one wait state separates the M0 write
// from the load that reads it. M0 is declared clobbered, though the compiler
// reserves it (hence the silenced warning): the kernels of this file make no
// other use of M0, which tests/test_isa_window_attn.py checks in the
// generated code.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* gsrc, const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) unsigned char*)lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "s"(m0)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// max over the 4 lanes l, l ^ 16, l ^ 32, l ^ 48 (the lanes of one head in an
// MFMA accumulator layout) by two lane-row swaps, no LDS round trip:
// permlane32_swap(x, x) leaves x[l] in one result and x[l ^ 32] in the other,
// permlane16_swap(y, y) likewise y[l] and y[l ^ 16]. The results are taken
// out of the returned pair as scalars before the float reinterpretation
// (a bit cast of a subscripted element of that vector type reads element 0).
__device__ __forceinline__ float max_over_heads_lanes(float x) {
  const unsigned u = __float_as_uint(x);
  const auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned a0 = s32[0], a1 = s32[1];
  const float y = fmaxf(__uint_as_float(a0), __uint_as_float(a1));
  const unsigned v = __float_as_uint(y);
  const auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  const unsigned b0 = s16[0], b1 = s16[1];
  return fmaxf(__uint_as_float(b0), __uint_as_float(b1));
}

// s_waitcnt for the LDS-direct loads of all but the newest `behind` tiles
// (kBLoads loads a tile per wave; behind is at most kNB - 2)
__device__ __forceinline__ void wait_tiles_behind(int behind) {
  static_assert(kNB <= 6, "wait counts below");
  switch (behind) {
    case 4: WA_WAIT_VMCNT(4 * kBLoads); break;
    case 3: WA_WAIT_VMCNT(3 * kBLoads); break;
    case 2: WA_WAIT_VMCNT(2 * kBLoads); break;
    case 1: WA_WAIT_VMCNT(kBLoads); break;
    default: WA_WAIT_VMCNT(0); break;
  }
}

// One pass over the ring's slots: tiles n, n + 1, .. in slots kSlot, kSlot + 1,
// .. (compile-time slots, so every LDS offset is an immediate), up to the
// last tile.
template <int kSlot, int kN, class F>
__device__ __forceinline__ void ring_round(F& step, int n, int n_tiles) {
  step(n, std::integral_constant<int, kSlot>{});
  if constexpr (kSlot + 1 < kN) {
    if (n + 1 < n_tiles) ring_round<kSlot + 1, kN>(step, n + 1, n_tiles);
  }
}

template <int kPos>
__global__ __launch_bounds__(kBThreads, 2) void wa_block(WaArgs a) {
  extern __shared__ __align__(16) unsigned char wlds[];          // the ring (kBLds bytes)
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int t = threadIdx.x, lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int Hq = a.Hkv * kG;
  const int P = clamp_ctx(a, b);
  const int lo0 = P - (a.W - 1) > 0 ? P - (a.W - 1) : 0;
  const int hi = P + a.K;
  const size_t rs = a.key_stride;                                       // elements between keys
  const uint16_t* kb = cache_head(a.kc, a, b, kvh);
  const uint16_t* vb = cache_head(a.vc, a, b, kvh);
  const int n_tiles = (hi - lo0 + kBT - 1) / kBT;
  const int p0 = wv * kPos;                                           // this wave's first position
  const int np = a.K - p0 < kPos ? a.K - p0 : kPos;                   // its positions (may be <= 0)
  // slots p >= np repeat position K - 1 (computed, not written): the loop
  // below runs the same code for every slot
  int pos[kPos];
#pragma unroll
  for (int p = 0; p < kPos; ++p) pos[p] = p0 + p < a.K ? p0 + p : a.K - 1;

  // Query fragments (B operand of the scores): lane (c, g) holds head kvh*16 + c,
  // dims 32 ds + 8 g .. + 7 of every position of this wave
  u32x4_t qf[kPos][4];
#pragma unroll
  for (int p = 0; p < kPos; ++p) {
    const uint16_t* qrow = a.q + (((size_t)b * a.K + pos[p]) * Hq + kvh * kG + c) * kD;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) qf[p][ds] = *reinterpret_cast<const u32x4_t*>(qrow + 32 * ds + 8 * g);
  }
  // the fragments are in before the ring starts (a wait for them inside the
  // tile loop would also wait for every tile in flight): an empty use here
  // makes the compiler wait for them at this point
#pragma unroll
  for (int p = 0; p < kPos; ++p)
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) asm volatile("" ::"v"(qf[p][ds]));

  // Tile n into ring slot n % kNB: this wave's kBRows keys of K and of V,
  // 1 KB LDS-direct loads (4 key rows of 256 bytes a load). Lane i of a load
  // fills physical chunk i % 16 of key row i / 16. A tile's rows sit at the
  // same offsets in every tile (32 keys: the row swizzles repeat), so each
  // lane's source addresses step by one tile of keys; the last tile clamps
  // keys past the range to the last key (masked).
  const int ph = lane & 15;
  const uint16_t* gsrc[2][kBRows / 4];                 // [K, V][load] at tile 0
#pragma unroll
  for (int i = 0; i < kBRows / 4; ++i) {
    const int kr = kBRows * wv + 4 * i + (lane >> 4);
    gsrc[0][i] = kb + (size_t)(lo0 + kr) * rs + 8 * (ph ^ kswz_b(kr));
    gsrc[1][i] = vb + (size_t)(lo0 + kr) * rs + 8 * (ph ^ vswz_b(kr));
  }
  const size_t tile_step = (size_t)kBT * rs;            // elements between tiles
  auto issue = [&](int n, int slot) {
    const int tb = lo0 + n * kBT;
    unsigned char* kbuf = wlds + slot * 2 * kBTile;
    unsigned char* vbuf = kbuf + kBTile;
    if (tb + kBT <= hi) {                              // wave-uniform: every key in range
#pragma unroll
      for (int i = 0; i < kBRows / 4; ++i) {
        const int r0 = kBRows * wv + 4 * i;            // first key row of this load
        lds_dma16(gsrc[0][i] + n * tile_step, kbuf + r0 * 256);
        lds_dma16(gsrc[1][i] + n * tile_step, vbuf + r0 * 256);
      }
    } else {
#pragma unroll
      for (int i = 0; i < kBRows / 4; ++i) {
        const int r0 = kBRows * wv + 4 * i;
        const int kr = r0 + (lane >> 4);
        const int key = tb + kr < hi ? tb + kr : hi - 1;
        lds_dma16(kb + (size_t)key * rs + 8 * (ph ^ kswz_b(kr)), kbuf + r0 * 256);
        lds_dma16(vb + (size_t)key * rs + 8 * (ph ^ vswz_b(kr)), vbuf + r0 * 256);
      }
    }
  };

  // Online softmax with a lazy reference: m is the running maximum (base-2
  // units) as of its last update, and e = 2^(s log2(e) - m) may exceed 1 by
  // up to 2^kTau before m moves again. A tile updates m (and rescales) only
  // if one of its raw scores exceeds thr = (m + kTau) / (scale log2(e)): the
  // common tile costs one compare per score instead of a reduction across
  // lanes. Before the first key m = thr = -inf.
  f32x4_t acc[kPos][8];
  float m[kPos], l[kPos], thr[kPos];
#pragma unroll
  for (int p = 0; p < kPos; ++p) {
    m[p] = -INFINITY;
    thr[p] = -INFINITY;
    l[p] = 0.0f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[p][dt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  const float inv_scale_log2 = 1.0f / a.scale_log2;

  // the largest window start of a position: tiles below it, and the last
  // tile, need masks
  const int lo_max = P + a.K - 1 - (a.W - 1);
  // lane-constant LDS offsets within a tile (the half h adds 16 rows, 4 KB):
  // K fragment ds of key row c (logical chunk 4 ds + g), and the transposing
  // V read of dims 16 dt + 4 (c % 4) .. + 3 of key 4 g + c / 4 (logical chunk
  // 2 dt + (c % 4) / 2, half (c % 2) of it)
  int kofs[4], vofs[8];
#pragma unroll
  for (int ds = 0; ds < 4; ++ds) kofs[ds] = c * 256 + 16 * ((4 * ds + g) ^ kswz_b(c));
  const int vkr = 4 * g + (c >> 2), vq = c & 3;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) vofs[dt] = vkr * 256 + 16 * ((2 * dt + (vq >> 1)) ^ vswz_b(vkr)) + 8 * (vq & 1);

  // scores of one tile whose K sits at kbuf: S^T per half and position
  // (lane (c, g): keys 16 h + 4 g .. + 3, head c)
  auto scores = [&](const unsigned char* kbuf, f32x4_t (&out)[2][kPos]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4_t kf[4];
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) kf[ds] = *reinterpret_cast<const u32x4_t*>(kbuf + 4096 * h + kofs[ds]);
#pragma unroll
      for (int p = 0; p < kPos; ++p) {
        out[h][p] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) out[h][p] = mfma_bf16(kf[ds], qf[p][ds], out[h][p]);
      }
    }
  };

  // The tiles are pipelined by one: step n finishes tile n (softmax and P V,
  // from the scores the previous step left in sc) and computes the scores of
  // tile n + 1, which do not depend on tile n's softmax, so the scheduler can
  // interleave those matrix instructions with the softmax's vector work.
  // Tile n + 1 must therefore be in LDS at step n: the step waits for it
  // (tile n + 2 stays in flight), and then refills the slot tile n - 1 used.
  f32x4_t sc[2][kPos];
  auto step = [&](int n, auto slot_tag) {
    constexpr int slot = decltype(slot_tag)::value;
    if (n + 1 < n_tiles) {
      // this wave's loads of tile n + 1 have landed (the younger tiles, up to
      // n + kNB - 2, may still be in flight), then every wave's; every wave is
      // past step n - 1, the last to read slot (n - 1) % kNB
      if (n + kNB - 2 < n_tiles) WA_WAIT_VMCNT((kNB - 3) * kBLoads);
      else wait_tiles_behind(n_tiles - 1 - (n + 1));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (n + kNB - 1 < n_tiles) issue(n + kNB - 1, (slot + kNB - 1) % kNB);
    }
    const int tb = lo0 + n * kBT;
    const unsigned char* vbuf = wlds + slot * 2 * kBTile + kBTile;
    // the next tile's K (after the last tile: a stale slot, scores unused)
    const unsigned char* knext = wlds + ((slot + 1) % kNB) * 2 * kBTile;

    // keys outside a position's range score -inf; a tile wholly below the
    // range leaves P = 0 and the running state unchanged
    float x[kPos][8];                                    // raw <q, k>: half h at 4 h + i
#pragma unroll
    for (int p = 0; p < kPos; ++p)
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[p][4 * h + i] = sc[h][p][i];
    if (tb < lo_max || tb + kBT > hi) {
#pragma unroll
      for (int p = 0; p < kPos; ++p) {
        const int lo_p = P + pos[p] - (a.W - 1);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = tb + 16 * h + 4 * g + i;
            if (!(key >= lo_p && key < hi)) x[p][4 * h + i] = -INFINITY;
          }
      }
    }
    bool over = false;
#pragma unroll
    for (int p = 0; p < kPos; ++p)
#pragma unroll
      for (int i = 0; i < 8; ++i) over |= x[p][i] > thr[p];
    if (__any(over)) {
      // a score past its threshold: the exact maximum of this tile per
      // position and head, and the new references (alpha = 1 where the
      // maximum did not grow, 0 from the empty start)
#pragma unroll
      for (int p = 0; p < kPos; ++p) {
        float mt = fmaxf(fmaxf(fmaxf(x[p][0], x[p][1]), fmaxf(x[p][2], x[p][3])),
                         fmaxf(fmaxf(x[p][4], x[p][5]), fmaxf(x[p][6], x[p][7])));
        mt = max_over_heads_lanes(mt) * a.scale_log2;
        const float mn = fmaxf(mt, m[p]);
        const float alpha = __builtin_amdgcn_exp2f(m[p] - mn);
        l[p] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[p][dt] *= alpha;
        m[p] = mn;
        thr[p] = (mn + kTau) * inv_scale_log2;
      }
    }
    u32x4_t pb[kPos];
#pragma unroll
    for (int p = 0; p < kPos; ++p) {
      const float mref = m[p] == -INFINITY ? 0.0f : m[p];   // no key seen yet: every e is 0
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[p][i], a.scale_log2, -mref));
        l[p] += e[i];
      }
      pb[p] = u32x4_t{pack_bf16(e[0], e[1]), pack_bf16(e[2], e[3]), pack_bf16(e[4], e[5]), pack_bf16(e[6], e[7])};
    }

    // the next tile's scores
    scores(knext, sc);

    // O^T += V^T P^T: the A operand of dims 16 dt .. + 15 (lane: dim 16 dt + c,
    // keys 4 g .. + 3 of each half) by one transposing read per half
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      v4i16_t vh[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
        vh[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(vbuf + 4096 * h + vofs[dt]));
      const u32x4_t va = __builtin_bit_cast(u32x4_t, __builtin_shufflevector(vh[0], vh[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int p = 0; p < kPos; ++p) acc[p][dt] = mfma_bf16(va, pb[p], acc[p][dt]);
    }
  };

  // prologue: kNB - 1 tiles in flight, the first one waited for and scored
#pragma unroll 1
  for (int n = 0; n < kNB - 1 && n < n_tiles; ++n) issue(n, n);
  wait_tiles_behind((n_tiles < kNB - 1 ? n_tiles : kNB - 1) - 1);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  scores(wlds, sc);
#pragma unroll 1
  for (int n = 0; n < n_tiles; n += kNB) ring_round<0, kNB>(step, n, n_tiles);

  // the outputs of this wave's positions: lane (c, g) holds O^T dims
  // 16 dt + 4 g .. + 3 of head c; the sum over keys gathers the 4 lanes of head c
#pragma unroll
  for (int p = 0; p < kPos; ++p) {
    if (p >= np) break;
    float lt = l[p];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const size_t row = ((size_t)b * a.K + p0 + p) * Hq + kvh * kG + c;
    const float inv = 1.0f / lt;
    float* o = a.out + row * kD;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4_t*>(o + 16 * dt + 4 * g) = acc[p][dt] * inv;
    if (g == 0) a.lse[row] = (m[p] + log2f(lt)) * 0.69314718055994531f;
  }
}

struct Plan {
  int S, keys_per_split;
  bool block;   // the large-batch kernel (wa_block)
};

inline int check(int B, int K, int Hq, int Hkv, int D, int L, int W) {
  if (B < 0 || K <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || L <= 0 || W <= 0) return DSPARK_ERR_ARG;
  if (D != kD || Hq != kG * Hkv || K > kKMax || K > W || L < K || B > 65535 || Hkv > 65535)
    return DSPARK_ERR_UNSUPPORTED;
  return DSPARK_OK;
}

// Splits of the key range, from a cost in units of one 64-key tile of K and
// V (32 KB): a round of resident workgroups (two per CU) takes as long as
// its largest split plus the partial output it writes (16 heads x K
// positions x 128 floats, ~1.8 tiles at K = 7), and the merge reads every
// partial once more, spread over the GPU, with its reads of one output's
// splits in dependent batches of eight (kMergeBatchCost tiles each: about
// a memory round trip against a latency-bound tile of a split). B=88, 4
// heads: 4 splits (1408 workgroups in 3 rounds) against 3 (1056 in 3 rounds
// of larger splits) or 13 (fuller rounds, 4x the partials). B=1, window
// 4096: 33 splits of two tiles (18.7 us a call against 23.0 with 65 of one,
// 20.0 with 17 of four, 26.9 with 9 of eight).
inline Plan plan(int B, int K, int Hkv, int W) {
  const long long span = (long long)W - 1 + K;                 // keys of the widest range
  const long long tiles = (span + kTileKeys - 1) / kTileKeys;
  const long long pairs = (long long)B * Hkv > 0 ? (long long)B * Hkv : 1;
  const long long smax = tiles < kMaxSplits ? tiles : kMaxSplits;
  const double part = (double)K * kG * kD * 4 / (kTileKeys * kD * 2 * 2);   // partial output, in tiles
  long long best = 1;
  double best_cost = 0.0;
  for (long long S = 1; S <= smax; ++S) {
    const long long per = (tiles + S - 1) / S;                 // tiles per split
    const long long ns = (tiles + per - 1) / per;              // splits actually used
    const long long rounds = (pairs * ns + kSlots - 1) / kSlots;
    const double cost = (double)rounds * ((double)per + part) + (double)(pairs * ns) * part / kSlots +
                        (ns > 1 ? kMergeBatchCost * (double)((ns + 7) / 8) : 0.0);
    if (S == 1 || cost < best_cost - 1e-9) {
      best_cost = cost;
      best = S;
    }
  }
  const long long per = ((tiles + best - 1) / best) * kTileKeys;
  Plan p;
  p.keys_per_split = (int)per;
  p.S = (int)((span + per - 1) / per);
  p.block = false;
  // enough (row, key/value head) pairs to fill the GPU with one workgroup
  // each: the large-batch kernel, one split (no partials, no merge launch)
  if (pairs >= kBlockMinPairs) {
    p.block = true;
    p.S = 1;
    p.keys_per_split = (int)span;
  }
  return p;
}

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline size_t workspace(int B, int K, int Hkv, int W, size_t* o_bytes) {
  const Plan p = plan(B, K, Hkv, W);
  // the single-launch kernel keeps nothing between launches: a token size,
  // so that 0 still means "unsupported"
  if (p.block) {
    if (o_bytes) *o_bytes = 0;
    return 256;
  }
  const size_t rows = (size_t)B * Hkv * p.S * K * kG;
  const size_t ob = align_up(rows * kD * sizeof(float), 256);
  if (o_bytes) *o_bytes = ob;
  return ob + align_up(rows * 2 * sizeof(float), 256);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace dspark_wa

extern "C" {

size_t dspark_window_attention_workspace_bytes(int B, int K, int Hq, int Hkv, int D, int L, int W) {
  using namespace dspark_wa;
  if (check(B, K, Hq, Hkv, D, L, W) != DSPARK_OK) return 0;
  return workspace(B, K, Hkv, W, nullptr);
}

int dspark_window_block_attention_layout(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                         const int32_t* ctx_len, int B, int K, int Hq, int Hkv, int D, int L,
                                         int W, float scale, int layout, float* out, float* lse,
                                         void* workspace_ptr, size_t workspace_bytes, void* stream_ptr) {
  using namespace dspark_wa;
  int rc = check(B, K, Hq, Hkv, D, L, W);
  if (rc != DSPARK_OK) return rc;
  if (layout != DSPARK_KV_LAYOUT_BLHD && layout != DSPARK_KV_LAYOUT_BHLD) return DSPARK_ERR_ARG;
  if (B == 0) return DSPARK_OK;
  if (!q || !k_cache || !v_cache || !ctx_len || !out || !lse) return DSPARK_ERR_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return DSPARK_ERR_ARG;
  if (!(scale > 0.0f) || scale == INFINITY) return DSPARK_ERR_ARG;
  size_t ob = 0;
  const size_t need = workspace(B, K, Hkv, W, &ob);
  if (!workspace_ptr || workspace_bytes < need || !aligned16(workspace_ptr)) return DSPARK_ERR_WORKSPACE;
  const Plan p = plan(B, K, Hkv, W);
  WaArgs a;
  a.q = q; a.kc = k_cache; a.vc = v_cache; a.ctx_len = ctx_len;
  a.part_o = static_cast<float*>(workspace_ptr);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace_ptr) + ob);
  a.out = out; a.lse = lse;
  a.B = B; a.K = K; a.Hkv = Hkv; a.L = L; a.W = W; a.S = p.S; a.keys_per_split = p.keys_per_split;
  a.scale_log2 = scale * 1.44269504088896341f;
  a.key_stride = layout == DSPARK_KV_LAYOUT_BLHD ? (size_t)Hkv * kD : (size_t)kD;
  a.head_stride = layout == DSPARK_KV_LAYOUT_BLHD ? (size_t)kD : (size_t)L * kD;
  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  if (p.block) {
    // one split: the workgroups write o and lse themselves
    const dim3 grid(1, Hkv, B), block(kBThreads);
    switch ((K + kBWaves - 1) / kBWaves) {
      case 1: hipLaunchKernelGGL(wa_block<1>, grid, block, kBLds, stream, a); break;
      default: hipLaunchKernelGGL(wa_block<2>, grid, block, kBLds, stream, a); break;
    }
    return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_ERR_HIP;
  }
  hipLaunchKernelGGL(wa_partials, dim3(p.S, Hkv, B), dim3(kPartThreads), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return DSPARK_ERR_HIP;
  if (p.S <= kFewSplits)
    hipLaunchKernelGGL(wa_combine, dim3(K, Hkv, B), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(wa_combine_splits, dim3(Hq, K, B), dim3(kD), 0, stream, a);
  if (hipGetLastError() != hipSuccess) return DSPARK_ERR_HIP;
  return DSPARK_OK;
}

int dspark_window_block_attention(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                  const int32_t* ctx_len, int B, int K, int Hq, int Hkv, int D, int L, int W,
                                  float scale, float* out, float* lse, void* workspace_ptr,
                                  size_t workspace_bytes, void* stream_ptr) {
  return dspark_window_block_attention_layout(q, k_cache, v_cache, ctx_len, B, K, Hq, Hkv, D, L, W, scale,
                                              DSPARK_KV_LAYOUT_BLHD, out, lse, workspace_ptr, workspace_bytes,
                                              stream_ptr);
}

}  // extern "C"
