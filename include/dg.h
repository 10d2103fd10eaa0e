/*
 * dg.h -- C ABI of the MI355X (gfx950) canvas-denoising library.
 *
 * The library runs the hot path of DiffusionGemma-style text diffusion: a
 * canvas of placeholder tokens is refined over a fixed number of parallel
 * denoise passes; each pass runs a decoder stack over every canvas position
 * at once and locks the most confident predictions, which stay fixed as
 * context for the following passes.  Sources (page title, section):
 *
 *   [4xFaster]     "DiffusionGemma: The Diffusion Era Begins with 4x Faster
 *                  Text Generation" -- "What is Diffusion and Why is it
 *                  Coming to Text Generation Now?" (canvas of random
 *                  placeholder tokens; locked tokens serve as context) and
 *                  "DiffusionGemma's Technical Architecture" (canvas 256,
 *                  128 experts with 8 active + 1 shared, sliding window 1024,
 *                  encoder KV cache read by the decoder through
 *                  cross-attention, bidirectional attention over the canvas).
 *   [HandsOn]      "Hands-On with Diffusion Gemma: Another Gemma with a
 *                  Diffusion Mechanism" -- "Detailed Specs" (local/global
 *                  layer pattern, GELU-tanh gated MLP, norm layers, tied
 *                  embedding and LM head, RoPE and p-RoPE, KV cache bridge).
 *   [ParadigmShift] "DiffusionGemma: Exploring the Paradigm Shift in
 *                  Non-Autoregressive Language Modeling" -- "Analysis of
 *                  Implications" (uncertain tokens are re-noised).
 *   [Experimental] "DiffusionGemma: Google's Experimental Diffusion LLM" --
 *                  "How Text Diffusion Actually Works" (a small fixed number
 *                  of passes per block).
 *
 * Conventions for every call:
 *   - All device pointers are plain HIP device addresses on the context's
 *     device; host pointers are marked "host".  No call takes ownership of a
 *     caller buffer.
 *   - Work is enqueued asynchronously on the stream given to dg_create (0 =
 *     the null stream); the caller synchronises before reading outputs.
 *   - Arguments are validated before anything is enqueued; on an error
 *     nothing is enqueued, output buffers are untouched and the status is
 *     returned.  A HIP error reported by the runtime (including an
 *     asynchronous fault of an earlier call) is returned as DG_EHIP.
 *   - dg_last_error() gives a message for the context's last error.
 *   - Token ids must lie in [0, V) (V = 262144 in the pages' model, [4xFaster]
 *     "DiffusionGemma's Technical Architecture").  Ids live in device memory,
 *     so they are checked on the device: the embedding reads an id outside
 *     that range as a zero row and records it, and the first call on the
 *     context after that work has run returns DG_EINVAL (naming the id, its
 *     canvas and position) with nothing enqueued; the record is then cleared.
 *     Synchronise the stream before that call to see the report there.
 *   - A context is not thread-safe: one host thread at a time.
 *   - bf16 values are raw 16-bit patterns (upper half of an IEEE float32);
 *     "T" below is float for DG_F32 contexts and bf16 for DG_BF16 contexts.
 *   - Weight matrices use the math layout y = x @ W with W row-major
 *     [in, out].
 */
#ifndef DG_H
#define DG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dg_status {
  DG_OK = 0,
  DG_EINVAL = -1,       /* bad argument (null pointer, size out of range) */
  DG_ENOMEM = -2,       /* device allocation failed */
  DG_EHIP = -3,         /* HIP runtime error */
  DG_ESTATE = -4,       /* call not valid in the context's state */
  DG_EUNSUPPORTED = -5  /* shape or dtype the library does not handle */
} dg_status;

typedef enum dg_dtype { DG_F32 = 0, DG_BF16 = 1 } dg_dtype;

/* Architecture and capacity of a context. */
typedef struct dg_config {
  int32_t n_layers;       /* decoder layers (<= 64) */
  int32_t hidden;         /* H, multiple of 32 */
  int32_t n_heads;        /* query heads Hq */
  int32_t n_kv_heads;     /* KV heads Hkv; Hq % Hkv == 0 (grouped-query attention) */
  int32_t head_dim;       /* D, multiple of 32, <= 256 */
  int32_t n_experts;      /* routed experts E, multiple of 16, <= 256 */
  int32_t top_k;          /* active routed experts per token, 1..8 */
  int32_t n_shared;       /* always-on shared experts; must be 1 */
  int32_t expert_ffn;     /* F, multiple of 32 */
  int32_t vocab;          /* V, multiple of 16 (0 allowed when has_lm_head == 0) */
  int32_t canvas_len;     /* N, canvas slots per canvas, multiple of 16 */
  int32_t window;         /* sliding window of local layers (prompt positions) */
  int32_t max_batch;      /* canvases per call, 1..64, max_batch*canvas_len <= 4096 */
  int32_t max_prompt_len; /* largest prompt KV length of any slot */
  uint64_t global_layer_mask; /* bit l set: layer l is global (GQA over the whole
                                 prompt, p-RoPE); clear: sliding window, RoPE */
  float rope_theta;       /* RoPE base */
  float prope_frac;       /* fraction of rotary pairs p-RoPE rotates on global layers */
  float rms_eps;          /* RMSNorm epsilon */
  int32_t dtype;          /* dg_dtype of weights, KV and stored activations */
  int32_t has_lm_head;    /* 0: decoder layers only (dg_forward_hidden) */
  int32_t post_ffn_norm;  /* 1: normalise the MoE output before the residual add */
  int32_t expert_format;  /* dg_expert_format of the routed and shared experts' matrices */
} dg_config;

/* Storage of the expert matrices (w_gate, w_up, w_down, sh_*).  MXFP4 (OCP
 * Microscaling Formats v1.0: 4-bit E2M1 elements, one E8M0 scale per 32
 * consecutive input-dimension entries of a column) is the gfx950-native
 * analogue of the 4-bit builds the pages list ([Experimental] "DiffusionGemma:
 * Google's Experimental Diffusion LLM"; [ParadigmShift] "Serving in
 * Production": GGUF Q4_K_M, NVFP4).  Weights are still given as T; the
 * library quantises them when they are set (scale s = floor(log2 max|x|) - 2
 * clamped to [-126, 127]; each element the nearest E2M1 value of x / 2^s, ties
 * to the even mantissa, saturating at 6) and the expert GEMMs multiply bf16
 * activations by the exact dequantised values.  DG_BF16 contexts only. */
typedef enum dg_expert_format { DG_EXPERT_NATIVE = 0, DG_EXPERT_MXFP4 = 1 } dg_expert_format;

/* One decoder layer's weights (caller-owned device pointers, dtype T).
 * Shapes: wq [H, Hq*D]; wk, wv [H, Hkv*D]; wo [Hq*D, H]; router [H, E];
 * w_gate, w_up [E, H, F]; w_down [E, F, H]; sh_gate, sh_up [H, F];
 * sh_down [F, H]; norm_in, norm_pa, norm_pf, norm_pf2 [H] (used as 1 + w). */
typedef struct dg_layer_weights {
  const void *wq, *wk, *wv, *wo, *router;
  const void *w_gate, *w_up, *w_down;
  const void *sh_gate, *sh_up, *sh_down;
  const void *norm_in, *norm_pa, *norm_pf, *norm_pf2;
} dg_layer_weights;

typedef struct dg_ctx dg_ctx;

/* Create a context on `device` (its current HIP device is set on every call)
 * enqueuing on `hip_stream` (a hipStream_t, may be NULL).  Allocates the
 * workspaces for max_batch canvases.  *out is NULL on failure. */
dg_status dg_create(const dg_config* cfg, int32_t device, void* hip_stream, dg_ctx** out);

/* Synchronise the context's stream and free everything the context owns.
 * NULL is accepted. */
dg_status dg_destroy(dg_ctx* ctx);

/* Message of the last error of `ctx` (NULL: the last dg_create failure).
 * The string stays valid until the next call on the context. */
const char* dg_last_error(const dg_ctx* ctx);

/* Copy one layer's weights into library-owned storage, repacked into the
 * layout of the matrix-core kernels.  The caller may free its buffers once
 * the stream has passed this call. */
dg_status dg_set_layer_weights(dg_ctx* ctx, int32_t layer, const dg_layer_weights* w);

/* Copy the embedding [V, H] (also the tied LM head, [HandsOn] "Detailed
 * Specs", weight sharing) and the final norm weight [H]. */
dg_status dg_set_embedding(dg_ctx* ctx, const void* embed, const void* norm_final);

/* All weights at once: `layers` is a host array of n_layers entries; embed
 * and norm_final may be NULL when has_lm_head == 0. */
dg_status dg_init_weights(dg_ctx* ctx, const void* embed, const void* norm_final,
                          const dg_layer_weights* layers);

/* Load the cached prompt KV of canvas slot `slot` (0 <= slot < max_batch),
 * the encoder's KV cache read by the decoder ([4xFaster] "DiffusionGemma's
 * Technical Architecture").  k[l], v[l] (host arrays of n_layers device
 * pointers) are [len_l, Hkv, D] of dtype T with len_l = prompt_len on global
 * layers and min(prompt_len, window) -- the last positions -- on local
 * layers.  K is already position-encoded.  The canvas of this slot sits at
 * positions prompt_len + i.  0 <= prompt_len <= max_prompt_len. */
dg_status dg_load_prompt_kv(dg_ctx* ctx, int32_t slot, int32_t prompt_len,
                            const void* const* k, const void* const* v);

/* One denoise pass over canvases 0..batch-1: embed, decoder stack, final
 * norm, tied LM head, per-position argmax and confidence (softmax
 * probability of the argmax), then per canvas lock the
 * ceil(remaining / steps_left[b]) unlocked positions of highest confidence
 * (ties to the lower position): they take their predicted token and become
 * locked; the others keep their placeholder ([4xFaster] "What is
 * Diffusion...", [ParadigmShift] "Analysis of Implications").
 *   tokens  int32 [batch, N] device, in/out
 *   locked  uint8 [batch, N] device, in/out (1 = locked)
 *   steps_left_host  int32 [batch] host, each >= 1
 *   conf_out float [batch, N] device or NULL; pred_out int32 [batch, N] or NULL
 * Requires all weights and the prompt KV of slots 0..batch-1. */
dg_status dg_denoise_step(dg_ctx* ctx, int32_t batch, int32_t* tokens, uint8_t* locked,
                          const int32_t* steps_left_host, float* conf_out, int32_t* pred_out);

/* n_steps passes, pass t with steps_left = n_steps - t for every canvas, so
 * every position is locked at the end ([Experimental] "How Text Diffusion
 * Actually Works").  No host synchronisation inside. */
dg_status dg_generate_block(dg_ctx* ctx, int32_t batch, int32_t n_steps, int32_t* tokens,
                            uint8_t* locked);

/* ---- entropy-bounded (EB) denoising ---------------------------------------
 * The sampler the pages recommend ([4xFaster] "Recommended Inference
 * Settings": EB sampler, at most 48 steps, temperature decaying linearly from
 * 0.8 to 0.4, entropy bound 0.1, adaptive stop once the mean canvas entropy is
 * below 0.005 and the high-probability tokens hold for 2 consecutive steps;
 * [ParadigmShift] "Serving in Production: The Role of vLLM": two consecutive
 * passes in agreement halt the block).  Pass t of at most t_max runs at
 * tau = 0.8 + (0.4 - 0.8) t / (t_max - 1) (0.8 when t_max == 1).  Per
 * position: entropy H of softmax(l / tau) in nats; a sample, the id of the
 * largest l * (float)(1/tau) + g (product and sum rounded apart, ties to the
 * lower id) with Gumbel noise g = -log(-log u), u = (2n + 1) 2^-24 from the top
 * 23 bits n of a Philox4x32-10 word (Salmon et al., SC 2011) with key
 * (seeds[b], block), counter ((v >> 6) * 16 + (v & 15), position, t, 0) and
 * word (v >> 4) & 3 for vocabulary id v; the greedy id (lowest among the
 * largest logits).  Per canvas not yet done: the unlocked positions in order
 * of increasing H (ties to the lower position) are locked with their sample
 * while the float32 running sum of their H stays <= 0.1f, at least one (every
 * unlocked one when t == t_max - 1); the canvas stops when a previous pass's
 * greedy ids are recorded, equal this pass's at every position, and the
 * float32 mean of H over the canvas (sum in position order, then / N) is
 * < 0.005f: its remaining unlocked positions then take their greedy ids.  A
 * canvas is done once it stops or has no unlocked position; done canvases are
 * left untouched.
 *
 * Per-canvas state (device, caller-owned): prev_pred int32 [batch, N], the
 * greedy ids of the previous pass; status int32 [batch], bit 0 done, bit 1
 * prev_pred holds a previous pass, bit 2 this pass stopped the canvas.  Set
 * status to 0 before a block's first pass. */

/* One EB pass t of at most t_max over canvases 0..batch-1.
 *   tokens int32 [batch, N], locked uint8 [batch, N] device, in/out
 *   seeds_host uint32 [batch] host; block: the noise key's second word
 *   prev_pred, status: the state above, in/out
 *   entropy_out float, sample_out int32, pred_out int32 [batch, N] device or NULL
 * Requires all weights and the prompt KV of slots 0..batch-1; 0 <= t < t_max. */
dg_status dg_eb_step(dg_ctx* ctx, int32_t batch, int32_t* tokens, uint8_t* locked, int32_t t, int32_t t_max,
                     const uint32_t* seeds_host, uint32_t block, int32_t* prev_pred, int32_t* status,
                     float* entropy_out, int32_t* sample_out, int32_t* pred_out);

/* EB passes 0, 1, ... until every canvas is done, at most t_max (the pages'
 * setting is 48), with the state held by the context.  After each pass the
 * host reads the canvases' status (one stream synchronisation per pass), so
 * the call returns when the block is resolved.  passes_out int32 [batch]
 * host or NULL: the number of passes after which each canvas was done. */
dg_status dg_generate_block_eb(dg_ctx* ctx, int32_t batch, int32_t* tokens, uint8_t* locked,
                               const uint32_t* seeds_host, uint32_t block, int32_t t_max,
                               int32_t* passes_out);

/* Block continuation: commits the resolved canvases (or N prompt tokens) to
 * the prompt KV cache.  The decoder stack runs once over tokens at positions
 * prompt_len + i with causal attention inside the block (position i sees the
 * cached context and block positions <= i), the causal context building of a
 * finished block before the next one ([HandsOn] "How Is This Different from
 * Previous Models?", Figure 3).  After each layer's attention the block's
 * K (after RoPE) and V are appended to that layer's cache (sliding-window
 * layers keep the last `window` positions), and every slot's prompt_len grows
 * by N, so the next canvas sits at positions prompt_len + N + i.  Starting
 * from an empty cache (dg_load_prompt_kv with prompt_len 0), successive
 * commits of N prompt tokens build the prompt KV from token ids.
 *   tokens  int32 [batch, N] device, ids in [0, V)
 * Requires the embedding, all weights, the prompt KV of slots 0..batch-1 and
 * prompt_len + N <= max_prompt_len for each (DG_EINVAL otherwise, nothing
 * enqueued).  The first commit of a slot allocates the buffers its grown
 * caches move between (synchronising the stream); later commits only enqueue
 * work. */
dg_status dg_commit_block(dg_ctx* ctx, int32_t batch, const int32_t* tokens);

/* dg_commit_block for the first n (1 <= n <= N) tokens of each canvas row:
 * positions prompt_len + i, i < n, join the caches and prompt_len grows by n.
 * tokens int32 [batch, N] device; entries past n are ignored (any value).  By
 * the causal mask the block's positions past n influence none before them,
 * so this equals a causal pass over the n tokens alone: successive calls
 * build the prompt KV of a prompt of any length from its token ids (the
 * encoder prefill), N tokens at a time and a shorter last chunk. */
dg_status dg_commit_tokens(dg_ctx* ctx, int32_t batch, const int32_t* tokens, int32_t n);

/* Test export: one expert matrix as the expert GEMMs multiply by it, in math
 * layout.  expert in [0, E] (E = the shared expert); which 0 = gate [H, F],
 * 1 = up [H, F], 2 = down [F, H].  values T [K, N] device (the dequantised
 * weights for MXFP4); for MXFP4 contexts codes uint8 [K, N] (one E2M1 code per
 * byte, sign in bit 3) and scales uint8 [K / 32, N] (s + 127) device, or NULL.
 * Any output may be NULL. */
dg_status dg_get_expert_weight(dg_ctx* ctx, int32_t layer, int32_t expert, int32_t which, void* values,
                               uint8_t* codes, uint8_t* scales);

/* Test export: the prompt KV cache of one slot and layer as
 * [len, Hkv, D] (k after RoPE, v) into caller buffers k, v (device, the
 * context's element type, either may be NULL); *len_out (host, may be NULL)
 * receives len, the positions visible to that layer. */
dg_status dg_get_prompt_kv(dg_ctx* ctx, int32_t slot, int32_t layer, void* k, void* v, int32_t* len_out);

/* Decoder layers only on a given residual stream: x_in, x_out float
 * [batch*N, H] device (may alias).  Prompt KV of slots 0..batch-1 required. */
dg_status dg_forward_hidden(dg_ctx* ctx, int32_t batch, const float* x_in, float* x_out);

/* Decoder layers [first, first + count) only, as dg_forward_hidden: x_in,
 * x_out float [batch*N, H] device (may alias).  A trace set by dg_set_trace
 * receives the routing of these layers at their own layer index. */
dg_status dg_forward_layers(dg_ctx* ctx, int32_t batch, int32_t first, int32_t count, const float* x_in,
                            float* x_out);

/* Record every pass's expert choice: route_idx int32 [n_layers, batch*N,
 * top_k] device (slot order: logit descending, index ascending), written by
 * each following dg_denoise_step / dg_forward_hidden (a block overwrites it
 * per pass).  NULL switches recording off. */
dg_status dg_set_trace(dg_ctx* ctx, int32_t* route_idx);

/* ---- single-kernel entry points (same kernels as the pass) ---------------- */

/* Per-row argmax (lowest index among equal maxima) and confidence
 * 1 / sum_v exp(l_v - l_max) of float logits [rows, vocab] ([HandsOn]
 * "Detailed Specs": the probability distribution judges which tokens are
 * final).  pred int32 [rows], conf float [rows] (rows == 0: nothing is done
 * and the pointers may be NULL).  vocab % 4 == 0.  `stream` may be NULL. */
dg_status dg_k_argmax_conf(const float* logits, int32_t rows, int32_t vocab, int32_t* pred,
                           float* conf, void* stream);

/* Lock-and-remask step alone (see dg_denoise_step) on given conf/pred
 * [batch, n] (conf finite, as a probability is); steps_left_host host [batch]
 * (>= 1); batch <= 64, n <= 4096. */
dg_status dg_k_lock_select(int32_t batch, int32_t n, const float* conf, const int32_t* pred,
                           int32_t* tokens, uint8_t* locked, const int32_t* steps_left_host,
                           void* stream);

/* EB statistics of float logits [rows, vocab], rows a multiple of canvas_len
 * (row r is position r % canvas_len of canvas r / canvas_len, at most 64
 * canvases): pred int32, entropy float, sample int32 [rows] for pass t of at
 * most t_max, noise key (seeds_host[canvas], block) (see the EB section). */
dg_status dg_k_eb_rows(const float* logits, int32_t rows, int32_t vocab, int32_t canvas_len, int32_t t,
                       int32_t t_max, const uint32_t* seeds_host, uint32_t block, int32_t* pred,
                       float* entropy, int32_t* sample, void* stream);

/* The EB sampler's Gumbel noise: noise float [rows, vocab] for pass t, row
 * r being position r % canvas_len of canvas r / canvas_len (at most 64
 * canvases), key (seeds_host[canvas], block) (see the EB section). */
dg_status dg_k_eb_noise(int32_t rows, int32_t vocab, int32_t canvas_len, int32_t t, const uint32_t* seeds_host,
                        uint32_t block, float* noise, void* stream);

/* The EB lock step alone on given entropy float (finite, >= 0), sample int32,
 * pred int32 [batch, n]: updates tokens, locked, prev_pred [batch, n] and
 * status [batch] as an EB pass t of at most t_max does; batch <= 64,
 * n <= 4096. */
dg_status dg_k_eb_select(int32_t batch, int32_t n, const float* entropy, const int32_t* sample,
                         const int32_t* pred, int32_t* tokens, uint8_t* locked, int32_t* prev_pred,
                         int32_t* status, int32_t t, int32_t t_max, void* stream);

/* Top-k routing on float router logits [rows, E] ([4xFaster] "DiffusionGemma's
 * Technical Architecture": 8 of 128 experts active): idx int32 [rows, k]
 * ordered (logit desc, expert asc); gates float [rows, k] = softmax over the
 * k kept logits; counts int32 [E]; offsets int32 [E + 2] (expert e's rows
 * are [offsets[e], offsets[e+1]), offsets[E] = rows*k, offsets[E+1] =
 * rows*k + rows for the shared expert); perm int32 [rows*k] = t*k + s of
 * each routed row, tokens ascending within an expert.  Any of counts,
 * offsets, perm may be NULL.  rows <= 4096, E <= 256, k <= 8,
 * E * ceil(rows / 32) <= 16384. */
dg_status dg_k_moe_route(const float* logits, int32_t rows, int32_t n_experts, int32_t top_k,
                         int32_t* idx, float* gates, int32_t* counts, int32_t* offsets,
                         int32_t* perm, void* stream);

/* q/k/v projections with RoPE (p-RoPE on global layers) of layer `layer`:
 * a T [batch*N, H] -> q T [batch, N, Hq, D], k, v T [batch, N, Hkv, D],
 * positions prompt_len(slot b) + i. */
dg_status dg_k_qkv(dg_ctx* ctx, int32_t layer, int32_t batch, const void* a, void* q, void* k,
                   void* v);

/* Attention of layer `layer` for canvases 0..batch-1: one softmax over the
 * keys [prompt KV visible to the layer ; canvas keys] (canvas keys left out
 * when canvas_keys == 0), grouped-query heads, no causal mask.  q T [batch,
 * N, Hq, D], k, v T [batch, N, Hkv, D] -> o T [batch, N, Hq*D]. */
dg_status dg_k_canvas_attn(dg_ctx* ctx, int32_t layer, int32_t batch, const void* q,
                           const void* k, const void* v, void* o, int32_t canvas_keys);

/* Routed MoE of layer `layer` with given routing: f T [batch*N, H], idx
 * int32 [batch*N, k], gates float [batch*N, k] -> m float [batch*N, H] =
 * sum_s gates[t,s] * FFN_idx[t,s](f_t) + FFN_shared(f_t), with
 * FFN(z) = (gelu_tanh(z Wg) * (z Wu)) Wd and the gated activation stored as
 * T ([HandsOn] "Detailed Specs": GELU-tanh gated MLP).  The k ids of a row
 * must be distinct and in [0, E): ids out of range are clamped, and a
 * repeated id yields an unspecified (finite, in-bounds) result. */
dg_status dg_k_moe_ffn(dg_ctx* ctx, int32_t layer, int32_t batch, const void* f,
                       const int32_t* idx, const float* gates, float* m);

/* Tied LM head: h T [batch*N, H] -> logits float [batch*N, V] = h @ embed^T. */
dg_status dg_k_lm_head(dg_ctx* ctx, int32_t batch, const void* h, float* logits);

/* Tied LM head reduced to per-row prediction and confidence, as a pass runs
 * it (bf16 contexts: fused, the logits never reach memory): h T [batch*N, H]
 * -> pred int32 [batch*N] = the lowest id among the largest logits, conf
 * float [batch*N] = 1 / sum_v exp(l_v - l_max) ([HandsOn] "Detailed Specs":
 * tied embedding and LM head; the output distribution judges which tokens
 * are final). */
dg_status dg_k_lm_argmax(dg_ctx* ctx, int32_t batch, const void* h, int32_t* pred, float* conf);

/* dg_k_lm_argmax without any allocation, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid it): the same kernels, with their per-(vocabulary tile, row)
 * partials in a static array of the library that each device holds until the
 * process ends (12 MiB: at most 2^20 (tile of 256 ids, row) pairs, i.e.
 * batch * N <= 2^20 / ceil(V / 256), 1024 rows at V = 262144; larger batches
 * return DG_EINVAL with nothing enqueued).  bf16 contexts only
 * (DG_EUNSUPPORTED otherwise).  Every call on a device shares that array:
 * calls that overlap in time on one device (other streams or contexts) race
 * and give undefined results; calls on one stream are ordered and safe.
 * Nothing needs clearing between calls (every partial is written before it is
 * read). */
dg_status dg_k_lm_argmax_noalloc(dg_ctx* ctx, int32_t batch, const void* h, int32_t* pred, float* conf);

/* EB statistics of the tied LM head as an EB pass runs it (bf16 contexts:
 * fused, the logits never reach memory): h T [batch*N, H] -> pred int32,
 * entropy float, sample int32 [batch*N] for pass t of at most t_max with the
 * noise key (seeds_host[b], block) (see the EB section above). */
dg_status dg_k_lm_sample(dg_ctx* ctx, int32_t batch, const void* h, int32_t t, int32_t t_max,
                         const uint32_t* seeds_host, uint32_t block, int32_t* pred, float* entropy,
                         int32_t* sample);

/* ---- kernel timing ----------------------------------------------------------
 * Per-launch device durations of selected kernel classes.  dg_profile(ctx,
 * mask) with mask != 0 synchronises the stream, clears the record and times
 * every later launch of the classes whose bit (1 << DG_PROF_x) is set; mask = 0
 * switches timing off (the record stays).  With DG_PROF_KEEP or'd in, the mask
 * changes without synchronising or clearing (timing resumes into the same
 * record), so timing can be switched on for some passes of a timed loop.  Kernel classes are timed by HIP events bound to their own
 * dispatches (start of the first kernel, end of the last); DG_PROF_PASS by an
 * event pair recorded on the stream around the pass.  Each timed launch adds a
 * few microseconds of dispatch latency around itself, so time only what is
 * needed.  dg_profile_read synchronises the stream and returns the number of
 * recorded launches of `kernel` and their summed duration in milliseconds. */
typedef enum dg_prof_kernel {
  DG_PROF_GATE_UP = 0,  /* grouped expert GEMM gate|up with the gated GELU-tanh */
  DG_PROF_DOWN = 1,     /* grouped expert GEMM down with the gate scale */
  DG_PROF_ATTN = 2,     /* canvas attention (splits and merge) */
  DG_PROF_LM_HEAD = 3,  /* tied LM head GEMM */
  DG_PROF_PASS = 4,     /* one whole denoise pass */
  DG_PROF_COUNT = 5,
  DG_PROF_ALL = (1 << 5) - 1,
  DG_PROF_KEEP = 1 << 30
} dg_prof_kernel;
dg_status dg_profile(dg_ctx* ctx, int32_t mask);
dg_status dg_profile_read(dg_ctx* ctx, int32_t kernel, int32_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* DG_H */
