/*
 * dspark.h -- C ABI of the DSpark ancestral draft-block sampler for MI355X (gfx950).
 *
 * What one call computes ("brb-nv/TensorRT-LLM pull 21", section "2. Golden
 * sampling semantics"; "brb-nv/TensorRT-LLM pull 27", section "2. One fused
 * kernel per draft position"): for each row b and each draft position
 * k = 0..K-1,
 *
 *     logits[b,k,:] = float32(base[b,k,:]) + bias(d_{k-1}),   bias(d) = E[d,:] . W
 *     d_k           = argmax_v ( logits[b,k,v] * (1/T_b) + Gumbel noise ),
 *
 * where d_{-1} = prev_token[b] and the Gumbel noise comes from a counter-based
 * Philox4x32-10 stream keyed by the row's (seed, offset) slot and k. After the
 * block, draft_probs[b,k,:] = softmax(logits[b,k,:] * (1/T_b)), recomputed
 * bit for bit from the stored float32 logits exactly as the draw used them.
 * Greedy rows (!(T_b > 0)) take the argmax chain of the logits and get a
 * one-hot proposal. Graph-padding rows (b >= *n_real) draw from the bias
 * alone: their base row is never read.
 *
 * Exact conventions (the pages leave these open; this library fixes them):
 *   - bias accumulates exact bf16 x bf16 products in float32 and is added to
 *     the float32 base in one float32 addition; it is never rounded to bf16.
 *   - invT = float32(1 / T); s = float32(logit * invT).
 *   - Philox key = (lo32(seed), hi32(seed)); counter = (v >> 2, k,
 *     lo32(offset), hi32(offset)); noise word = output word (v & 3).
 *   - u = ((x >> 9) + 0.5) * 2^-23 (exact, in [2^-24, 1 - 2^-24]);
 *     g = -ln(-ln u); z = float32(s + g). Greedy rows use z = logit.
 *   - d_k is the lowest index among the largest z. NaN scores never win; a
 *     row whose every score is NaN draws token 0.
 *   - q = exp(s - M) / S with M the row maximum of s and S = sum exp(s - M).
 *
 * Memory: every array argument is a DEVICE pointer owned by the caller,
 * row-major and contiguous, 16-byte aligned. The library never allocates,
 * frees, synchronises, or reads device data on the host, so a call can be
 * captured into a hipGraph and replayed; seeds, offsets, temperatures and
 * n_real are read on the device, so replays see new values without a new
 * capture. The caller advances `offset` between blocks (a new offset draws
 * anew).
 *
 * Errors: argument checks run on the host before anything is enqueued; a
 * failed check returns a negative status and enqueues nothing. A failed
 * kernel launch returns DSPARK_ERR_HIP. No C++ exception crosses the ABI.
 * Device data never causes an error: an out-of-range prev_token is clamped
 * into [0, V), and a drawn token is always in [0, V). The one exception is
 * a resident-plan block whose bounded device wait expired (below): its
 * positions from the failure on hold token -1 and NaN proposals.
 *
 * Device waits (resident plans, see dspark_launch_plan): one persistent
 * launch runs the whole block, one workgroup per compute unit, and the
 * workgroups exchange each position's argmax partials through the library's
 * own device memory. This needs every compute unit of the device free for
 * the launch: no other kernel may hold a compute unit while it runs, and two
 * such calls must never run at the same time on one device (calls ordered on
 * one stream are fine). The waits are bounded: if one expires (a compute unit
 * was held elsewhere), the block's positions from one at or before the first
 * it could not complete get token -1 and NaN proposals, and
 * dspark_block_status reports it. Nothing hangs.
 *
 * Concurrency: calls on different streams must use different workspaces
 * and outputs, and resident calls must not overlap (above).
 */
#ifndef DSPARK_H_
#define DSPARK_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DSPARK_F32 = 0,   /* base logits are float32 */
    DSPARK_BF16 = 1   /* base logits are bfloat16 (uint16 bit patterns) */
} dspark_dtype_t;

typedef enum {
    DSPARK_OK = 0,
    DSPARK_ERR_ARG = -1,          /* null pointer, bad size, misaligned pointer, bad dtype */
    DSPARK_ERR_UNSUPPORTED = -2,  /* V % 8 != 0, r % 32 != 0, r > 1024, K > 255, ... */
    DSPARK_ERR_WORKSPACE = -3,    /* workspace missing or smaller than dspark_workspace_bytes */
    DSPARK_ERR_HIP = -4,          /* a HIP runtime call or kernel launch failed */
    DSPARK_ERR_SCRATCH = -5       /* dspark_draft_block_noalloc: the call needs more than its static scratch */
} dspark_status_t;

/* Loads the kernels on the current device. Call once per device before any
 * stream capture. Returns DSPARK_OK or DSPARK_ERR_HIP. */
int dspark_init(void);

/* Device workspace bytes a call with these sizes needs (for any chunking).
 * Returns 0 for sizes the library does not support. */
size_t dspark_workspace_bytes(int B, int K, int V, int r);

/* One K-position draft block ("brb-nv/TensorRT-LLM pull 27", section
 * "2. One fused kernel per draft position").
 *
 *   base_logits  [B,K,V] float32 or bf16 (per base_dtype); read only, never written
 *   E            [V,r]   bf16 Markov embedding
 *   W            [r,V]   bf16 Markov head
 *   prev_token   [B]     int32, d_{-1}: the row's last committed token (clamped)
 *   seed         [B]     int64, Philox key bits
 *   offset       [B]     int64, Philox slot offset
 *   temperature  [B]     float32; !(T > 0) marks a greedy row
 *   n_real       device int32 scalar, or NULL (all rows real); rows b >= *n_real
 *                are graph padding
 *   B, K, V, r   sizes: B >= 0, 0 <= K <= 255, V > 0 and V % 8 == 0,
 *                0 < r <= 1024 and r % 32 == 0. B == 0 or K == 0 enqueues nothing.
 *   tokens       [B,K]   int32 out: the drawn tokens
 *   logits_f32   [B,K,V] float32 out: base + bias, before the 1/T scaling
 *   draft_probs  [B,K,V] float32 out: the proposal q_k
 *   workspace    device scratch of at least dspark_workspace_bytes(B,K,V,r) bytes;
 *                its contents need no initialisation and are not meaningful after
 *   stream       hipStream_t to enqueue on (NULL = the null stream)
 */
int dspark_draft_block(
    const void* base_logits, int base_dtype,
    const uint16_t* E, const uint16_t* W,
    const int32_t* prev_token, const int64_t* seed, const int64_t* offset,
    const float* temperature, const int32_t* n_real,
    int B, int K, int V, int r,
    int32_t* tokens, float* logits_f32, float* draft_probs,
    void* workspace, size_t workspace_bytes, void* stream);

/* The same block for callers that cannot allocate device memory (code under
 * stream capture that may not allocate, tight serving loops, harnesses that
 * forbid it): no workspace argument; the call lays out the scratch its plan
 * needs in a static device array the library holds, one per device, of
 * dspark_noalloc_scratch_bytes() bytes (8 MiB), taken when the device is first
 * used and kept until the process ends. Arguments, outputs, launches and
 * results are those of dspark_draft_block (the same kernels). A call whose plan
 * needs more scratch than that returns DSPARK_ERR_SCRATCH and enqueues
 * nothing: the resident plans need 8 K B x (compute units) + 4 KB (on 256 CUs,
 * B K <= 4094), the per-position plans 32 B ceil(V/128) + 8 B K + 2 B r. Nothing
 * in the scratch needs to start at zero. Every call on a device shares that
 * device's array, so calls that overlap on one device (other streams, other
 * threads) race and give wrong results: enqueue them in order. Allocates
 * nothing (no hipMalloc, hipFree or allocating library call). */
int dspark_draft_block_noalloc(
    const void* base_logits, int base_dtype,
    const uint16_t* E, const uint16_t* W,
    const int32_t* prev_token, const int64_t* seed, const int64_t* offset,
    const float* temperature, const int32_t* n_real,
    int B, int K, int V, int r,
    int32_t* tokens, float* logits_f32, float* draft_probs, void* stream);

/* Size in bytes of dspark_draft_block_noalloc's static scratch (per device). */
size_t dspark_noalloc_scratch_bytes(void);

/* The same block with an explicit vocabulary chunking: each workgroup of the
 * fused per-position kernel owns `chunk_cols` consecutive vocabulary columns
 * (a positive multiple of 128; 0 = the library's choice) and writes one
 * softmax-statistics and argmax partial per row. The pages test one and three
 * vocabulary chunks ("brb-nv/TensorRT-LLM pull 27", section "Test Coverage");
 * tokens and logits do not depend on the chunking, q only through the order
 * of a float32 sum. */
int dspark_draft_block_chunked(
    const void* base_logits, int base_dtype,
    const uint16_t* E, const uint16_t* W,
    const int32_t* prev_token, const int64_t* seed, const int64_t* offset,
    const float* temperature, const int32_t* n_real,
    int B, int K, int V, int r, int chunk_cols,
    int32_t* tokens, float* logits_f32, float* draft_probs,
    void* workspace, size_t workspace_bytes, void* stream);

/* The default-chunked block with timing marks, for measurement: events[0]
 * is recorded on `stream` before the first launch and events[i + 1] after
 * the i-th launch, in the order dspark_launch_plan reports. n_events must be
 * at least the launch count plus one; the events are caller-created
 * hipEvent_t handles passed as void*. Returns DSPARK_ERR_ARG if events is
 * NULL or too short; otherwise as dspark_draft_block. */
int dspark_draft_block_events(
    const void* base_logits, int base_dtype,
    const uint16_t* E, const uint16_t* W,
    const int32_t* prev_token, const int64_t* seed, const int64_t* offset,
    const float* temperature, const int32_t* n_real,
    int B, int K, int V, int r,
    int32_t* tokens, float* logits_f32, float* draft_probs,
    void* workspace, size_t workspace_bytes, void* stream,
    void* const* events, int n_events);

/* W packed for the resident kernels. W is a weight, the same for every
 * block, so it can be laid out once in the order in which the two resident
 * kernels (see dspark_launch_plan) hold it on chip: for each kernel, one
 * contiguous block per compute unit of this device with that unit's slice of
 * W (784 columns x 256 rank rows, bf16, zero past r and past V), then each
 * kernel's setup is one coalesced stream instead of 16-byte pieces of 256
 * rank rows. The bias it computes is the pages' E[d] . W ("brb-nv/TensorRT-LLM
 * pull 27", section "2. One fused kernel per draft position"), bit for bit the
 * same as from W itself.
 *
 * dspark_packed_w_bytes: bytes of the packed copy for V, r on the current
 * device (2 x 401,408 x its compute units: 205.5 MB on 256), or 0 when no
 * resident plan can run these sizes (r > 256, V > 2^18, V > 784 x units, or
 * V % 8 or r % 32 not 0): nothing to pack then.
 *
 * dspark_pack_w: enqueues on `stream` the writing of W [r, V] (device bf16)
 * into W_packed (device, 16-byte aligned, at least dspark_packed_w_bytes).
 * The copy belongs to this V, this r and this device's compute-unit count:
 * pack on the device that will use it, with the sizes the blocks will use,
 * and again after W changes. Its size depends on the compute-unit count
 * only, so a copy packed for another V or r is not detected (its blocks are
 * wrong); one packed on a device with another count is (DSPARK_ERR_ARG).
 * DSPARK_ERR_UNSUPPORTED when the size is 0, DSPARK_ERR_ARG for null or
 * misaligned pointers or a short buffer, DSPARK_ERR_HIP if the launch fails. */
size_t dspark_packed_w_bytes(int V, int r);
int dspark_pack_w(const uint16_t* W, int V, int r, void* W_packed, size_t packed_bytes, void* stream);

/* dspark_draft_block with W also given packed (dspark_pack_w on this device,
 * packed_bytes exactly dspark_packed_w_bytes(V, r), else DSPARK_ERR_ARG): the
 * resident plans read W_packed, the per-position plans W. Same launches and
 * results as dspark_draft_block, bit for bit. `events` may be NULL; if not, it
 * and n_events are as for dspark_draft_block_events. */
int dspark_draft_block_packed(
    const void* base_logits, int base_dtype,
    const uint16_t* E, const uint16_t* W, const void* W_packed, size_t packed_bytes,
    const int32_t* prev_token, const int64_t* seed, const int64_t* offset,
    const float* temperature, const int32_t* n_real,
    int B, int K, int V, int r,
    int32_t* tokens, float* logits_f32, float* draft_probs,
    void* workspace, size_t workspace_bytes, void* stream,
    void* const* events, int n_events);

/* dspark_draft_block with the proposals written by slot: the proposal pass
 * stores row b's q_k into row slot_index[b] of draft_probs [n_slots, K, V]
 * instead of row b ("brb-nv/TensorRT-LLM pull 27", section "2. One fused
 * kernel per draft position": the proposals go into draft_probs indexed by
 * the request's slot). tokens [B, K] and logits_f32 [B, K, V] stay indexed by
 * row. W_packed may be NULL (W alone is used); if not, it and packed_bytes are
 * as for dspark_draft_block_packed.
 *   slot_index   [B]     int32, device; a slot outside [0, n_slots) stores no
 *                        proposal for that row (its tokens and logits are
 *                        still written); two rows with one slot race, so slots
 *                        should be distinct
 *   n_slots               rows of draft_probs (host int, > 0)
 *   draft_probs  [n_slots, K, V] float32, device, 16-byte aligned; rows no
 *                        row is sent to are left as they were
 * Same launches, tokens and logits as dspark_draft_block, and the same q bit
 * for bit in each written slot. DSPARK_ERR_ARG for a NULL slot_index or
 * n_slots <= 0, otherwise the errors of dspark_draft_block(_packed). */
int dspark_draft_block_slots(
    const void* base_logits, int base_dtype,
    const uint16_t* E, const uint16_t* W, const void* W_packed, size_t packed_bytes,
    const int32_t* prev_token, const int64_t* seed, const int64_t* offset,
    const float* temperature, const int32_t* n_real,
    const int32_t* slot_index, int n_slots,
    int B, int K, int V, int r,
    int32_t* tokens, float* logits_f32, float* draft_probs,
    void* workspace, size_t workspace_bytes, void* stream);

/* Kinds of kernel launch a block is made of. */
typedef enum {
    DSPARK_LAUNCH_FUSED_POSITION = 0,  /* markov_bias_gumbel_argmax for one position */
    DSPARK_LAUNCH_PICK = 1,            /* pick_and_gather for one position */
    DSPARK_LAUNCH_PROPOSAL = 2,        /* proposal_softmax for the whole block */
    DSPARK_LAUNCH_CLEAR = 3,           /* reserved (no plan uses it) */
    DSPARK_LAUNCH_RESIDENT_BLOCK = 4   /* markov_bias_gumbel_argmax for all K positions at once */
} dspark_launch_kind_t;

/* The launches dspark_draft_block enqueues on the current device for these
 * sizes, in order: writes up to max_kinds dspark_launch_kind_t values to
 * `kinds` (host memory, may be NULL) and returns the launch count, or a
 * negative status. Three plans exist:
 *   - resident (r <= 256, V <= 2^18, V <= 784 x the device's CU count, at
 *     most 512 CUs, and B <= 128): RESIDENT_BLOCK, PROPOSAL. One persistent
 *     launch runs all K positions; each workgroup keeps its slice of W on chip
 *     for the block (B <= 2: a VALU GEMV with 512 threads; 2 < B <= 128: bf16
 *     MFMA tiles with 256 threads). It needs every workgroup resident at once
 *     (one per compute unit); its device-side waits are bounded, and if one
 *     expires the affected tokens are -1 instead of hanging (see "Device
 *     waits" above and dspark_block_status).
 *   - B == 1 otherwise: K x FUSED_POSITION, PROPOSAL (each fused kernel picks
 *     the previous position's token itself).
 *   - otherwise: K x (FUSED_POSITION, PICK), PROPOSAL.
 * dspark_draft_block_chunked always uses the last two plans. */
int dspark_launch_plan(int B, int K, int V, int r, int* kinds, int max_kinds);

/* Whether a bounded device wait of the most recent resident-plan block on the
 * current device expired. Enqueues one tiny kernel on `stream` that writes
 * 1 (a wait expired: that block's tokens from a position at or before the
 * first incomplete one on are -1 and their proposals NaN) or 0 (it did not,
 * or no resident block has run on the device) into *status, a DEVICE int32.
 * Enqueue it on the stream of the block it reports on, after the block;
 * graph-capturable. Plans without device waits (per-position plans) cannot
 * fail this way and do not change it. Returns DSPARK_ERR_ARG for a null
 * pointer, DSPARK_ERR_HIP if the launch fails, else DSPARK_OK. */
int dspark_block_status(int32_t* status, void* stream);

/* Sets how many times a resident kernel reads an exchange word before its wait
 * expires, for the calls made after it (a captured graph keeps the value in
 * force at its capture); returns the previous value. The default, 2^20 reads,
 * is about a second. 0 makes every wait expire at once without reading, which
 * is how the failure path is tested. Process-wide, not thread-safe against
 * concurrent calls. */
unsigned dspark_set_wait_limit(unsigned reads);

/* Standard token-level verification of a draft block ("brb-nv/TensorRT-LLM
 * pull 21", section "2. Golden sampling semantics": rejection_sample_method
 * standard, token-level verification). The pages name the rule; this is the
 * textbook one (Leviathan, Kalman and Matias, "Fast Inference from
 * Transformers via Speculative Decoding", ICML 2023, section 2.3): for
 * k = 0 .. K-1 accept d_k with probability min(1, p_k(d_k) / q_k(d_k)); at the
 * first rejection emit a token drawn from max(0, p_k - q_k) normalised and
 * stop; if all K drafts are accepted, emit a bonus token drawn from p_K.
 *
 *   draft_tokens  [B,K]    int32 d_k (as dspark_draft_block writes them; clamped into [0,V))
 *   draft_probs   [B,K,V]  float32 q_k (dspark_draft_block's draft_probs); may be NULL if K == 0
 *   target_probs  [B,K+1,V] float32 p_k, the target's distributions
 *   seed, offset  [B]      int64, the request's Philox slot (as for the draft)
 *   B, K, V       B >= 0, 0 <= K <= 255, V > 0 and V % 4 == 0, B <= 65535
 *   n_accepted    [B]      int32 out: the number n of drafts accepted (0..K)
 *   out_tokens    [B,K+1]  int32 out: d_0 .. d_{n-1}, the emitted token, then -1
 *   workspace     device scratch of at least dspark_verify_workspace_bytes(B,K,V)
 *                 bytes, 8-byte aligned; contents need no initialisation
 *
 * Conventions (the pages leave them open):
 *   - ratio = float32(p_k(d_k) / q_k(d_k)), one IEEE division; accept iff
 *     u_k < ratio. q = 0 < p accepts; 0/0 (NaN) rejects.
 *   - u_k = ((x >> 9) + 1/2) 2^-23 (exact in float32), x = output word 0 of
 *     Philox4x32-10 at counter (0xFFFFFFFF, 256 + k, lo32(offset),
 *     hi32(offset)) under key (lo32(seed), hi32(seed)). The draft block uses
 *     counter word 1 = k < 256, so the two streams never meet.
 *   - The emitted token at position j (j < K after a rejection, j = K for the
 *     bonus) is the Gumbel-max draw over w_v = float32(p_j(v) - q_j(v)) (or
 *     p_K(v)) among v with w_v > 0: the lowest index of the largest
 *     ln w_v + g_v, g_v = -ln(-ln u) of output word (v & 3) of counter
 *     (v >> 2, 512, lo32(offset), hi32(offset)), the same at every position
 *     (a row emits one drawn token; where is decided by the uniforms, another
 *     stream). A residual with no
 *     positive entry (only through rounding) is replaced by p_j; a row with
 *     no positive entry at all emits token 0.
 *
 * Two launches on `stream` (a partial pass per chunk of 1024 to 8192
 * columns and row, then a merge per row); graph-capturable; nothing is
 * allocated. Errors as
 * for dspark_draft_block: DSPARK_ERR_ARG for null or misaligned pointers
 * (q and p need 16-byte alignment), DSPARK_ERR_UNSUPPORTED for sizes outside
 * the limits above, DSPARK_ERR_WORKSPACE, DSPARK_ERR_HIP. B == 0 enqueues
 * nothing. */
size_t dspark_verify_workspace_bytes(int B, int K, int V);
int dspark_verify_standard(
    const int32_t* draft_tokens, const float* draft_probs, const float* target_probs,
    const int64_t* seed, const int64_t* offset, int B, int K, int V,
    int32_t* n_accepted, int32_t* out_tokens,
    void* workspace, size_t workspace_bytes, void* stream);

/* Block verification of a draft block ("brb-nv/TensorRT-LLM pull 21",
 * section "2. Golden sampling semantics": rejection_sample_method block).
 * The pages name the rule; this is the algorithm of Sun, Mendlovic,
 * Leviathan, Aharoni, Beirami, Ro and Suresh, "Block Verification
 * Accelerates Speculative Decoding" (2024), in the draft block's indices:
 *   w_0 = 1, w_{j+1} = min(1, w_j p_j(d_j) / q_j(d_j));
 *   S_j = sum_v max(w_j p_j(v) - q_j(v), 0);
 *   h_j = S_j / (S_j + 1 - w_j) for 1 <= j < K, h_K = w_K;
 *   n = the largest j in 1..K with eta_j < h_j, else 0;
 *   out: d_0 .. d_{n-1}, then a token drawn from max(w_n p_n - q_n, 0)
 *   normalised (n < K) or from p_K (n = K).
 * Arguments, layouts and errors as for dspark_verify_standard; the
 * workspace is at least dspark_verify_block_workspace_bytes(B,K,V) bytes,
 * 8-byte aligned, and needs no initialisation.
 *
 * Conventions (the pages leave them open):
 *   - w, S and h in double: the ratio is one IEEE double division of the
 *     float32 inputs, w_{j+1} = w_j * ratio clamped to [0, 1] (q = 0 < p
 *     gives 1, 0/0 gives 0); residual entries are the double product w_j p
 *     minus q (no fused multiply-add), clamped at 0; h_j = 0 when S_j = 0.
 *     Only the summation order of S_j is the implementation's own.
 *   - eta_j is the token-level rule's u_{j-1} (same Philox word); the test
 *     is eta_j < h_j in double.
 *   - The emitted token is drawn as in the token-level rule (the same
 *     Gumbel words), from the weights float32(max(w_n p_n(v) - q_n(v), 0))
 *     or p_K(v); an empty residual is replaced by p_n; a row with no
 *     positive entry at all emits token 0.
 *
 * Two launches on `stream` (a pass over all K+1 target and K draft
 * distributions per chunk and row, then a merge per row); graph-capturable;
 * nothing is allocated. */
size_t dspark_verify_block_workspace_bytes(int B, int K, int V);
int dspark_verify_block(
    const int32_t* draft_tokens, const float* draft_probs, const float* target_probs,
    const int64_t* seed, const int64_t* offset, int B, int K, int V,
    int32_t* n_accepted, int32_t* out_tokens,
    void* workspace, size_t workspace_bytes, void* stream);

/* Non-causal windowed block attention of a DSpark drafter layer
 * ("brb-nv/TensorRT-LLM pull 21", section "1. Non-causal DSpark draft blocks
 * on TRTLLM (default path)"): K draft-block queries at positions
 * P .. P+K-1 after a context of P tokens; query i attends every key t < P+K
 * with |i - t| <= W - 1 (the whole draft block and the context keys at most
 * W - 1 back). GQA with 16 query heads per key/value head.
 *
 *   q          [B,K,Hq,D]   bf16 queries, 16-byte aligned
 *   k_cache    [B,L,Hkv,D]  bf16 keys of positions 0 .. L-1 (the block's own
 *   v_cache    [B,L,Hkv,D]  keys and values already at P .. P+K-1), 16-byte aligned
 *   ctx_len    [B]          int32 P per row, device; clamped into [0, L-K]
 *   D == 128, Hq == 16 Hkv, 1 <= K <= 8, K <= W, K <= L, B <= 65535
 *   scale      the score scale (s = scale <q, k>), finite and > 0
 *   out        [B,K,Hq,D]   float32 out: softmax-weighted values
 *   lse        [B,K,Hq]     float32 out: ln sum_t exp(s_t)
 *   workspace  at least dspark_window_attention_workspace_bytes(...) bytes,
 *              16-byte aligned; contents need no initialisation
 *
 * Scores are bf16 products accumulated in float32, the softmax is float32
 * in base 2, and the probabilities are rounded to bf16 for the product with
 * V. With B * Hkv >= 256 one launch on `stream` (one workgroup per row and
 * key/value head over the whole key range); below that, two (the key range
 * split over workgroups, then a log-sum-exp merge of the splits).
 * Graph-capturable; nothing is allocated.
 * Errors: DSPARK_ERR_ARG (null or misaligned pointers, bad scale or sizes),
 * DSPARK_ERR_UNSUPPORTED (sizes outside the limits), DSPARK_ERR_WORKSPACE,
 * DSPARK_ERR_HIP. B == 0 enqueues nothing. */
size_t dspark_window_attention_workspace_bytes(int B, int K, int Hq, int Hkv, int D, int L, int W);
int dspark_window_block_attention(
    const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* ctx_len,
    int B, int K, int Hq, int Hkv, int D, int L, int W, float scale,
    float* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Key/value cache layouts of dspark_window_block_attention_layout. */
#define DSPARK_KV_LAYOUT_BLHD 0   /* [B, L, Hkv, D]: the heads of one position adjacent */
#define DSPARK_KV_LAYOUT_BHLD 1   /* [B, Hkv, L, D]: each head's positions contiguous */

/* dspark_window_block_attention with the cache layout given: k_cache and
 * v_cache are [B, L, Hkv, D] (DSPARK_KV_LAYOUT_BLHD, what
 * dspark_window_block_attention takes) or [B, Hkv, L, D]
 * (DSPARK_KV_LAYOUT_BHLD). The attention computed, the other arguments, the
 * workspace size and the errors are the same; another layout value is
 * DSPARK_ERR_ARG. In the head-major layout each (row, head) key range is one
 * contiguous span, which the kernels stream faster (256-byte rows at a
 * 1 KB stride become one run). */
int dspark_window_block_attention_layout(
    const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache, const int32_t* ctx_len,
    int B, int K, int Hq, int Hkv, int D, int L, int W, float scale, int layout,
    float* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* A static, human-readable name for a status code. */
const char* dspark_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DSPARK_H_ */
