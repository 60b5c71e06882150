/*
 * qmoe.h -- C ABI of the quantized routed-MoE layer for AMD Instinct MI355X
 * (gfx950).
 *
 * What the layer computes comes from the ds4 pages:
 *   [digest]  "antirez/ds4 - Metal向け DeepSeek V4 Flash ローカル推論エンジン"
 *             (ja.news.hada.io/topic?id=29299), sections "Model weights"
 *             (only the routed MoE experts are quantized: up/gate in a 2-bit
 *             codebook format, down in a 2-bit K-quant format; shared expert
 *             and routing stay unquantized) and the overview (few active
 *             parameters -- sparse top-k experts -- is what makes it fast).
 *   [upppp]   "ds4 ..." article (upppp.jp/open-source/20260512-142644),
 *             section "asymmetric 2-bit quantization" (experts take most of
 *             the bytes; shared expert / projections kept at higher precision).
 *   [osrepos] "ds4: A Fast Local Inference Engine ..." (osrepos.com), the
 *             "Q4KExperts" model file name (a 4-bit K-quant expert variant).
 *   [blog]    Korean user blog (modu-print.com), server log excerpts
 *             (prompts are prefilled in chunks of 2048 tokens, cap 8192).
 *
 * The pages name the formats but do not define their bytes.  This header is
 * the format definition; the CB2/K2/K4/BF16 paragraphs below are normative.
 *
 * ---------------------------------------------------------------------------
 * Conventions for every call
 *   Ownership: the caller owns every buffer.  The library never allocates or
 *     frees device memory and keeps no pointer after a call returns, except
 *     a moe_expert_cache: it keeps the layer's pointers and the slot memory
 *     given at creation until moe_expert_cache_destroy, and page-locked host
 *     staging of its own (freed there).
 *   Pointers: "device" pointers are HIP device memory on the current device;
 *     "host" pointers are ordinary process memory.  Device base pointers must
 *     be 16-byte aligned.
 *   Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *     stream).  Device calls enqueue kernels and return without waiting.
 *   Errors: arguments are checked on the host before anything is enqueued.
 *     On failure a call returns a nonzero MOE_ERR_* code, leaves its outputs
 *     untouched (one exception: moe_layer_decode_streamed, below) and sets
 *     a thread-local message readable with
 *     moe_last_error().  A failed kernel launch returns MOE_ERR_HIP.  No call
 *     aborts, exits or lets a C++ exception escape.
 *   Determinism: every result is a fixed-order computation (no atomics in
 *     any floating-point sum), so repeated calls give identical bits.
 *   Range: the expert FFN calls give each token t an exponent
 *     e_t = floor(log2 max_i |x_ti|) - 1, clamped to [-60, 60] (a token of
 *     zeros gets -60).  Routed-expert GEMMs take x_t * 2^-e_t as fp16
 *     operands (largest magnitude in [2, 4)), and h is stored as
 *     fp16(h_t * 2^-2e_t); the power of two is removed again in fp32, which
 *     is exact.  So tokens with max |x_t| from 2^-59 to 2^62 keep fp16's full
 *     precision whatever their scale (sums must stay inside fp32's range);
 *     values of x below
 *     2^(e_t - 13) (about 2^-15 of the token's largest, or less) and of the
 *     scaled h below 2^-14 lose precision on fp16's subnormal grid, and the
 *     scaled h must stay below 65504 (it does for any weights with
 *     |W_gate x_t 2^-e_t| |W_up x_t 2^-e_t| < 65504).
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG 1
#define MOE_ERR_UNSUPPORTED 2
#define MOE_ERR_WORKSPACE 3
#define MOE_ERR_HIP 4

/* Weight formats.
 *
 * Every weight matrix W [rows, k] (rows = output features, k = reduction
 * dimension, row-major) is stored as tiles of 16 rows x 256 columns.  k is
 * zero-padded up to kp = 256 * ceil(k / 256); rows must be a multiple of 16.
 * Tiles are stored row-tile major: tile (rt, kc) starts at byte
 * (rt * kp/256 + kc) * TILE, rt = row / 16, kc = col / 256.
 * Inside a tile, row n = row % 16 and column kk = col % 256 split as
 *   kb = kk / 32, qq = (kk % 32) / 8, j = kk % 8, and lane c = 16*qq + n.
 * Lane c owns weights (n, kb, qq, j = 0..7) for kb = 0..7: exactly the 8
 * values one lane of a 64-wide wavefront feeds to a 16x16x32 MFMA as its B
 * operand for k-block kb.  All multi-byte fields are little-endian.
 *
 * MOE_FMT_CB2 (2-bit codebook, 2.5 bits/weight; [digest] "Model weights",
 *   up/gate).  A group is 8 consecutive weights (n, kb, qq, j=0..7).  It holds
 *   an 8-bit index into a 256 x 8 table T of values in {-3,-1,1,3} (units of
 *   1/4, see moe_codebook_generate) and 8 flip bits; every 32 weights (n, kb)
 *   share one fp16 scale s.  Weight j = s * T[idx][j] / 4, negated when flip
 *   bit j is set.  Tile (1280 bytes):
 *     [0, 1024)    lane c at 16*c: 8 uint16 codes, code for kb at byte 2*kb,
 *                  code = idx | flip << 8 (flip bit j = bit 8+j).
 *     [1024, 1280) row n at 1024 + 16*n: 8 fp16 scales, kb at byte 2*kb.
 *
 * MOE_FMT_K2 (2-bit K-quant, 2.625 bits/weight; [digest] "Model weights",
 *   down).  Each row's 256 columns of a tile form one super-block of 16
 *   sub-blocks of 16 (sub-block sb = kk / 16 = 2*kb + qq/2), with 2-bit codes
 *   q, 4-bit sc and m per sub-block and fp16 d, dmin per super-block:
 *   weight = d*sc*q - dmin*m.  Tile (1344 bytes):
 *     [0, 1024)    lane c at 16*c: 4 uint32 words; word i holds kb = 2i and
 *                  2i+1: the code of (kb, j) sits at bit 2*(4*(kb%2) + j/2)
 *                  + 16*(j%2).
 *     [1024, 1280) row n at 1024 + 16*n: byte sb = sc | m << 4.
 *     [1280, 1344) row n at 1280 + 4*n: fp16 d, fp16 dmin.
 *
 * MOE_FMT_K4 (4-bit K-quant, 4.5 bits/weight; [osrepos] "Q4KExperts").  One
 *   super-block per row per tile of 8 sub-blocks of 32 (sub-block = kb), 4-bit
 *   q, 6-bit sc and m, fp16 d, dmin: weight = d*sc*q - dmin*m.  Tile (2304):
 *     [0, 2048)    for half h = kb / 4: lane c at 1024*h + 16*c: 4 uint32
 *                  words, word kb%4 holds the 8 codes of kb: code of j at bit
 *                  4*(j/2) + 16*(j%2).
 *     [2048, 2240) row n at 2048 + 12*n: 96-bit little-endian bit stream of
 *                  16 six-bit values sc0..sc7, m0..m7 (value i at bit 6*i).
 *     [2240, 2304) row n at 2240 + 4*n: fp16 d, fp16 dmin.
 *
 * MOE_FMT_BF16 (unquantized shared expert).  Tile (8192 bytes): element
 *   (n, kb, qq, j) at byte 1024*kb + 16*c + 2*j (c = 16*qq + n), bf16.
 *
 * MOE_FMT_Q8 (8-bit shared expert, 8.5 bits/weight; [upppp] "asymmetric
 *   2-bit quantization": shared experts stay at Q8_0 or F16; [osrepos] the
 *   "Q8Shared" model file name).  Every 32 weights (n, kb) share one fp16
 *   scale d; weight = d * q with q a signed 8-bit code in -127..127.
 *   Tile (4352 bytes):
 *     [0, 4096)    piece i = 0..3 at 1024*i: lane c at 1024*i + 16*c holds
 *                  the 8 codes (j = 0..7) of k-block a = 4*(i%2) + i/2, then
 *                  the 8 codes of k-block a + 2 (int8 each); so k-block kb
 *                  sits in piece 2*(kb%2) + kb/4, second half when
 *                  (kb/2) % 2 == 1.
 *     [4096, 4352) row n at 4096 + 16*n: 8 fp16 scales, kb at byte 2*kb.
 */
#define MOE_FMT_BF16 0
#define MOE_FMT_CB2 1
#define MOE_FMT_K2 2
#define MOE_FMT_K4 3
#define MOE_FMT_Q8 4

/* ---------------------------------------------------------------------------
 * Host-only calls (no GPU needed).
 */

/* Fills table_out[256*8] (entry-major) with the CB2 codebook: SplitMix64
 * (Steele, Lea, Flood, OOPSLA 2014) started from `seed`; draw i sets entry
 * i/8, value i%8 to {-3,-1,1,3}[draw >> 62].  Returns MOE_OK, or
 * MOE_ERR_INVALID_ARG if table_out is NULL. */
int moe_codebook_generate(uint64_t seed, int8_t* table_out);

/* Bytes of a packed matrix [rows, k] in format fmt (k padded to 256).
 * Returns 0 when rows is not a positive multiple of 16, k < 1 or fmt is
 * unknown. */
size_t moe_packed_bytes(int fmt, int64_t rows, int64_t k);

/* Quantizes and packs a host fp32 matrix w [rows, k] (row-major) into
 * out (host, out_bytes >= moe_packed_bytes(fmt, rows, k)): the quantized
 * expert matrices of [digest] "Model weights" (CB2 for up/gate, K2 for down)
 * and [osrepos] "Q4KExperts" (K4), and the shared expert (BF16 or Q8,
 * [upppp] "asymmetric 2-bit quantization"; [osrepos] "Q8Shared").  Columns beyond k up to the next
 * multiple of 256 are taken as zero.
 *   CB2: per 32 weights s = fp16(max|w| / 0.75) (fp64 quotient, one rounding
 *        to fp16); per group the lowest index e minimizing
 *        sum_{j=0..7} (|w_j| - s*|T[e][j]|/4)^2 (fp64, j ascending); flip bit j
 *        = (w_j < 0) != (T[e][j] < 0).  `codebook` = the 256x8 table (host).
 *   K2/K4: per sub-block lo = min(0, min w), hi = max w, a = (hi-lo)/Q,
 *        b = 0-lo; d = fp16(max a / S), dmin = fp16(max b / S);
 *        sc = min(S, floor(a/d + 1/2)), m = min(S, floor(b/dmin + 1/2))
 *        (0 when d or dmin is 0); q = clamp(floor((w + dmin*m)/(d*sc) + 1/2),
 *        0, Q) (0 when d*sc is 0).  K2: Q=3, S=15; K4: Q=15, S=63.
 *   Q8:  per 32 weights d = fp16(max|w| / 127) (fp64 quotient, one
 *        rounding); q = sign(w) * min(127, floor(|w|/d + 1/2)) (fp64; 0
 *        when d is 0).
 *   BF16: each value rounded to bf16 (nearest, ties to even).
 * n_threads <= 0 uses all hardware threads.  Errors: MOE_ERR_INVALID_ARG for
 * NULL pointers, bad shapes, non-finite weights, |w| too large for an fp16
 * scale (CB2 s, Q8 d, K-quant d or dmin would round to infinity), a missing or
 * malformed codebook (CB2) or out_bytes too small; every check runs before
 * the first byte of out is written. */
int moe_quantize_pack(int fmt, const float* w, int64_t rows, int64_t k,
                      const int8_t* codebook, void* out, size_t out_bytes,
                      int n_threads);

/* ---------------------------------------------------------------------------
 * Device calls.
 */

/* One MoE layer's weights (all pointers device, 16-byte aligned).
 *   up, gate: n_experts packed matrices [inter, hidden] back to back, each
 *             moe_packed_bytes(fmt_up, inter, hidden) bytes.
 *   down:     n_experts packed matrices [hidden, inter].
 *   shared_*: packed [shared_inter, hidden] (up, gate) and
 *             [hidden, shared_inter] (down) in format fmt_shared; NULL when
 *             shared_inter == 0.
 *   fmt_shared: MOE_FMT_BF16 (0, so a zero-initialized field keeps the
 *             unquantized shared expert) or MOE_FMT_Q8.
 *   codebook: device copy of the 256x8 CB2 table (int8), or NULL if no CB2.
 * Supported: hidden a multiple of 256; inter and shared_inter multiples of
 * 16; (fmt_up, fmt_gate, fmt_down) = (CB2, CB2, K2) or (K4, K4, K4). */
typedef struct moe_weights {
  int32_t n_experts;
  int32_t hidden;
  int32_t inter;
  int32_t shared_inter;
  int32_t fmt_up, fmt_gate, fmt_down;
  int32_t fmt_shared;
  const void* up;
  const void* gate;
  const void* down;
  const int8_t* codebook;
  const void* shared_up;
  const void* shared_gate;
  const void* shared_down;
} moe_weights;

/* Workspace bytes moe_route needs for T tokens over E experts. */
size_t moe_route_workspace_bytes(int32_t T, int32_t E);

/* Router ([digest] "Model weights": routing stays unquantized; the function
 * is softmax over experts, keep the top k, renormalize over the kept k).
 *   x_bf16   device bf16 [T, H];  w_router device fp32 [E, H];
 *   logit_bias device fp32 [E] added to the logits, or NULL.
 *   topk_idx device int32 [T, k]: experts by descending logit, ties to the
 *            lower index;  topk_w device fp32 [T, k]: exp(l_j - l_0) /
 *            sum_i exp(l_i - l_0) over the kept logits.
 * Logits are fp32 sums.  ws: device scratch, >= moe_route_workspace_bytes(T,
 * E); its contents need no initialization.
 * Limits: 1 <= k <= min(E, 16), E <= 1024, H a multiple of 8. */
int moe_route(const void* x_bf16, const float* w_router, const float* logit_bias,
              int32_t T, int32_t H, int32_t E, int32_t k, int32_t* topk_idx,
              float* topk_w, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes moe_group_tokens needs. */
size_t moe_group_workspace_bytes(int32_t T, int32_t k, int32_t E);

/* Stable grouping of the T*k (token, choice) slots by expert (slot = t*k + j)
 * -- the per-expert token lists that sparse activation works on ([digest]
 * overview).  Outputs (device int32): expert_offsets [E+1] (exclusive scan of
 * per-expert counts), sorted_slots [T*k] (slots ordered by expert, slot order
 * kept within an expert), slot_pos [T*k] (inverse of sorted_slots).  A slot
 * whose expert id lies outside [0, E) is dropped (its slot_pos is -1) and
 * counted: the int32 at byte 0 of ws accumulates the number of such slots
 * (atomically, over calls); zero it before the call to read one call's
 * count.  The rest of ws needs no initialization. */
int moe_group_tokens(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                     int32_t* expert_offsets, int32_t* sorted_slots, int32_t* slot_pos,
                     void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of the expert FFN for T tokens with k choices each
 * (prefill != 0: the grouped prefill path; else decode, T <= 16). */
size_t moe_ffn_workspace_bytes(const moe_weights* w, int32_t T, int32_t k, int prefill);

/* Expert FFN for 1..16 tokens (decode / draft verification): the routed
 * experts with quantized weights plus the unquantized shared expert
 * ([digest] "Model weights"; [upppp] "asymmetric 2-bit quantization"), run
 * only for the k experts each token chose (sparse activation, [digest]
 * overview):
 *   y[t] = sum_j topk_w[t,j] * FFN_{topk_idx[t,j]}(x[t]) + FFN_shared(x[t]),
 *   FFN(x) = W_down (SiLU(W_gate x) * (W_up x)), summed j = 0..k-1 then the
 *   shared expert.  x_bf16 device bf16 [T, H]; y device fp32 [T, H]
 *   (overwritten).  The intermediate h is fp16 (scaled per token, see
 *   "Range" above); sums are fp32.  Up to 3
 *   tokens run the single-token kernels once per token, which decode the
 *   weights exactly (scales applied to fp32 block sums); for T >= 4 a layer
 *   with CB2 up/gate, hidden <= 4096 and inter, shared_inter <= 2048 takes
 *   batched kernels that read each distinct expert once and fold the CB2
 *   scales into fp16 weights (one rounding per weight, as
 *   moe_expert_ffn_prefill does); their K2 down weights stay exact.  A choice whose
 *   expert id lies outside [0, E) contributes nothing (and is not counted);
 *   a token may name one expert in several choices (each contributes).  ws
 *   needs no initialization; its first bytes hold h * 2^-2e_t as fp16
 *   [T*k, inter] (slot order) after the call.  Limits: 1 <= T <= 16,
 *   1 <= k <= 16. */
int moe_expert_ffn_decode(const moe_weights* w, const void* x_bf16, int32_t T, int32_t k,
                          const int32_t* topk_idx, const float* topk_w, float* y,
                          void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes of moe_layer_decode (0 for invalid arguments). */
size_t moe_layer_decode_workspace_bytes(const moe_weights* w, int32_t T, int32_t k);

/* One decode step of the whole layer ([digest] "Model weights": unquantized
 * router, quantized routed experts, unquantized shared expert; batch-1
 * generation as the pages benchmark it): moe_route then
 * moe_expert_ffn_decode in one call, with the same results (topk_idx, topk_w
 * and y as those two calls give; topk_* are outputs here).  One token on a CB2 layer with
 * hidden <= 4096 and E <= 64*max(4, hidden/256) has its experts ranked
 * inside the up/gate kernel, from the router's logits, while the shared
 * expert's weights already stream; other shapes run the router's top-k
 * kernel first.  Arguments as for those two calls; ws: device scratch
 * of at least moe_layer_decode_workspace_bytes(w, T, k), 16-byte aligned,
 * no initialization needed; its first bytes hold h as moe_expert_ffn_decode
 * leaves it.  Limits: 1 <= T <= 16, 1 <= k <= min(E, 16), E <= 1024. */
int moe_layer_decode(const moe_weights* w, const float* w_router, const float* logit_bias,
                     const void* x_bf16, int32_t T, int32_t k, int32_t* topk_idx, float* topk_w,
                     float* y, void* ws, size_t ws_bytes, void* stream);

/* moe_layer_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same step, the same results, with its workspace in an
 * array the library holds in device memory, MOE_NOALLOC_SCRATCH_BYTES
 * (8 MiB) per GPU, kept until the process ends.  The call allocates nothing.
 * Arguments as for moe_layer_decode without ws / ws_bytes.  Every call on one
 * GPU uses that GPU's one array: calls that overlap in time on one GPU (on
 * different streams, or from different threads without ordering) race and
 * give undefined results; calls ordered on one stream are safe.  Errors:
 * as moe_layer_decode; MOE_ERR_WORKSPACE when
 * moe_layer_decode_workspace_bytes(w, T, k) exceeds the array (nothing is
 * enqueued).  The array's contents are not preserved between calls. */
#define MOE_NOALLOC_SCRATCH_BYTES (8u << 20)
int moe_layer_decode_noalloc(const moe_weights* w, const float* w_router, const float* logit_bias,
                             const void* x_bf16, int32_t T, int32_t k, int32_t* topk_idx, float* topk_w,
                             float* y, void* stream);

/* Expert FFN for a prefill chunk (any T >= 1; the pages prefill prompts in
 * chunks of 2048 tokens, [blog] server logs), same result as the decode
 * call, computed as grouped GEMMs over moe_group_tokens' output (device
 * int32 arrays as that call writes them).  Dequantized weights and h are
 * fp16 MFMA operands; sums are fp32.  ws needs no initialization; its first
 * bytes hold h * 2^-2e_t as fp16 [T*k, inter] in grouped (sorted_slots)
 * order after the call. */
int moe_expert_ffn_prefill(const moe_weights* w, const void* x_bf16, int32_t T, int32_t k,
                           const int32_t* topk_idx, const float* topk_w,
                           const int32_t* expert_offsets, const int32_t* sorted_slots,
                           const int32_t* slot_pos, float* y, void* ws, size_t ws_bytes,
                           void* stream);

/* Decodes a packed matrix on the device into fp32 out [rows, kp] with the
 * same decode routines the FFN kernels use (kp = k padded to 256).  For
 * tests: every value is the exact format value rounded once to fp32. */
int moe_debug_dequant(int fmt, const void* packed, int64_t rows, int64_t k,
                      const int8_t* codebook, float* out, void* stream);

/* Measurement hook.  Kernel ids for moe_profile_next_launch: */
#define MOE_KERNEL_ROUTE_LOGITS 0
#define MOE_KERNEL_ROUTE_TOPK 1
#define MOE_KERNEL_DECODE_UPGATE 2
#define MOE_KERNEL_DECODE_DOWN 3
#define MOE_KERNEL_DECODE_COMBINE 4
#define MOE_KERNEL_GROUP 5
#define MOE_KERNEL_PREFILL_UPGATE 6
#define MOE_KERNEL_PREFILL_DOWN 7
#define MOE_KERNEL_PREFILL_COMBINE 8
#define MOE_KERNEL_READ 9

/* Makes the next launch of kernel `kernel_id` by this thread record the HIP
 * events start_event / stop_event (hipEvent_t as void*, owned by the caller)
 * at the start and the end of that kernel's execution (hipExtLaunchKernel's
 * dispatch events), so that hipEventElapsedTime gives that one kernel's
 * duration.  Up to 8 requests
 * (for different or repeated ids) can be pending; each is consumed by the
 * next launch of its kernel.  kernel_id -1 drops all pending requests.
 * Returns MOE_ERR_INVALID_ARG for an unknown id, NULL events or more than 8
 * pending requests. */
int moe_profile_next_launch(int kernel_id, void* start_event, void* stop_event);

/* Measurement: reads `bytes` of device memory at src once (16-byte vectors,
 * coalesced, streaming) with `blocks` workgroups of 256 threads (0: four per
 * compute unit) and XORs every 32-bit word into *out (device uint32, not
 * reset: zero it first to read the XOR of the buffer).  Its rate is the
 * measured ceiling that the bandwidth-bound decode kernels are compared with
 * at the same byte count (kernel id MOE_KERNEL_READ for
 * moe_profile_next_launch).  src 16-byte aligned, bytes a positive multiple
 * of 16; MOE_ERR_INVALID_ARG otherwise. */
int moe_measure_read(const void* src, size_t bytes, uint32_t* out, int blocks, void* stream);

/* ---------------------------------------------------------------------------
 * Expert streaming ([osrepos] "SSD Streaming for Large Models": for models
 * larger than GPU memory the routed MoE experts are loaded from storage as
 * they are needed, into an expert cache whose size the user sets).  Here the
 * routed experts stay in host memory and an HBM cache of n_slots experts
 * holds the ones in use.  A step maps its top-k expert ids to cache slots
 * (moe_expert_cache_plan), copies the experts it misses into their slots
 * (moe_expert_cache_fetch), and runs the expert FFN over the cache, which is
 * a weight set of n_slots experts (moe_expert_cache_weights), with the slot
 * ids in place of the expert ids.  Routing weights, the shared expert and
 * the order of every sum are those of the resident layer, so the output is
 * the same to the bit.
 *
 * Replacement (the pages name none; least recently used over steps): a step
 * needs the distinct ids of its [T, k] choices in order of first appearance
 * (ids outside [0, n_experts) are skipped); resident ones are hits; each miss
 * takes the lowest free slot, else evicts the least recently used resident
 * expert that this step does not need and that was not used in the last
 * `keep` steps; after the step its experts count as used now, later-appearing
 * ones more recently.  A cache is used by one thread at a time. */
typedef struct moe_expert_cache moe_expert_cache;

/* Device bytes of the slot storage for n_slots experts of layer w (three
 * slot arrays: up, gate, down; each 256-byte aligned); 0 on bad arguments. */
size_t moe_expert_cache_slot_bytes(const moe_weights* w, int32_t n_slots);

/* A cache holds host state that its calls read and change: calls on one
 * cache must not overlap (one thread at a time).
 *
 * Creates a cache.  host_layer: the layer as in moe_weights, except that up,
 * gate and down point to HOST memory holding all n_experts packed experts
 * (page-locked memory makes the copies asynchronous; the caller keeps it
 * alive and unchanged while the cache exists); shared_* and codebook are
 * device pointers, used as they are.  slot_mem: device memory of at least
 * moe_expert_cache_slot_bytes(host_layer, n_slots) bytes, 256-byte aligned,
 * owned by the caller.  1 <= n_slots <= n_experts; keep >= 0 (1 when a step
 * may be planned while the previous one still runs on the GPU).  Runs on the
 * host only.  Returns MOE_OK and *out, or MOE_ERR_INVALID_ARG /
 * MOE_ERR_UNSUPPORTED (as moe_expert_ffn_decode's weight checks). */
int moe_expert_cache_create(const moe_weights* host_layer, int32_t n_slots, int32_t keep, void* slot_mem,
                            size_t slot_mem_bytes, moe_expert_cache** out);

/* Frees the cache's host state (and its page-locked staging buffers). */
int moe_expert_cache_destroy(moe_expert_cache* cache);

/* The cache as a weight set: n_experts = n_slots, up/gate/down = the slot
 * arrays, the other fields as host_layer. */
int moe_expert_cache_weights(const moe_expert_cache* cache, moe_weights* out);

/* Host only.  Maps one step's n expert ids (host, e.g. [T, k] top-k choices)
 * to slots: slots_out[i] (host, n entries) is the slot of ids[i] (-1 for an
 * id outside [0, n_experts)).  The misses (experts now assigned a slot whose
 * bytes must be copied) go to miss_experts[0 .. *n_miss) and miss_slots
 * (host, at least n entries each), in order of first appearance.  If the
 * step needs more experts than the slots that are free or evictable it
 * returns MOE_ERR_INVALID_ARG and changes nothing. */
int moe_expert_cache_plan(moe_expert_cache* cache, const int32_t* ids, int32_t n, int32_t* slots_out,
                          int32_t* miss_experts, int32_t* miss_slots, int32_t* n_miss);

/* Enqueues on `stream` the host-to-device copies of n_miss experts (up,
 * gate and down of miss_experts[i] into slot miss_slots[i]; host arrays as
 * moe_expert_cache_plan wrote them).  The FFN that reads those slots must
 * run after them (the same stream, or an event). */
int moe_expert_cache_fetch(moe_expert_cache* cache, const int32_t* miss_experts, const int32_t* miss_slots,
                           int32_t n_miss, void* stream);

/* Host only: the expert held by each slot (expert_of_slot[n_slots], -1 when
 * free) and the hit and miss counts since creation. */
int moe_expert_cache_state(const moe_expert_cache* cache, int32_t* expert_of_slot, int64_t* hits,
                           int64_t* misses);

/* Workspace bytes of moe_layer_decode_streamed for T tokens, k choices. */
size_t moe_layer_decode_streamed_workspace_bytes(const moe_expert_cache* cache, int32_t T, int32_t k);

/* One decode step with the routed experts streamed through the cache:
 * moe_route of x, a copy of the choices to the host (the host waits for
 * `stream` here, so the call cannot be captured in a graph), plan, the
 * misses' copies on copy_stream (NULL: on stream; `stream` waits for them),
 * then moe_expert_ffn_decode over the cache with the slot ids.  topk_idx,
 * topk_w and y as in moe_layer_decode (expert ids, not slots).  T <= 16.
 * Errors as the calls it makes, plus MOE_ERR_INVALID_ARG when the step needs
 * more experts than the cache can hold: that is known only after routing,
 * so on this error topk_idx and topk_w hold the step's choices; y, the cache
 * and its slots are untouched. */
int moe_layer_decode_streamed(moe_expert_cache* cache, const float* w_router, const float* logit_bias,
                              const void* x_bf16, int32_t T, int32_t k, int32_t* topk_idx, float* topk_w,
                              float* y, void* ws, size_t ws_bytes, void* stream, void* copy_stream);

/* Message of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QMOE_H */
