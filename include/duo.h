/*
 * duo.h - C ABI of libduo: attention over a head-partitioned KV cache on AMD Instinct
 * MI355X (gfx950).
 *
 * The method (arXiv 2410.10819, "DuoAttention: Efficient Long-Context LLM Inference with
 * Retrieval and Streaming Heads") splits the KV heads of every layer into retrieval heads,
 * which keep and attend over every token, and streaming heads, which keep and attend over a
 * constant-size cache of attention-sink tokens plus a window of recent tokens. Citations
 * below name the web pages about the paper and the section on them:
 *   explainer        = paper-graph-ui.vercel.app walkthrough of the paper;
 *   OpenReview thread = paperhub.cn page with the authors' rebuttal.
 *
 * Conventions shared by every call
 * --------------------------------
 * - All calls are C, never throw and return a duo_status. DUO_OK is 0.
 * - Argument and capacity checks happen on the host before anything is launched; when a
 *   call returns an error other than DUO_ERR_HIP nothing was launched and no state changed.
 *   DUO_ERR_HIP means a HIP runtime call or launch failed (the device state is then
 *   unspecified). Faults inside kernels surface asynchronously, as in any stream API.
 * - Device work is enqueued on `stream` (a hipStream_t; NULL is the default stream) and is
 *   asynchronous; only duo_slot_positions synchronizes. Calls on one cache must be ordered
 *   on one stream: decode calls share the cache's split-K workspace.
 * - The library never allocates or frees device memory. The caller owns the arena and every
 *   input/output buffer; all device pointers must stay valid until the work completes.
 * - Layouts are row-major and contiguous in the native head order of the model:
 *     decode  q, out      [B][Hq][d]        lse [B][Hq]
 *     prefill q, out      [B][m][Hq][d]     lse [B][m][Hq]   (seq = -1: every sequence)
 *                         [m][Hq][d]        lse [m][Hq]      (seq >= 0: one sequence)
 *     append/prefill k, v [B][m][Hkv][d]   or [m][Hkv][d] (seq >= 0)
 *   Query head h reads KV head h / G with G = Hq / Hkv (contiguous groups). KV heads are
 *   never repeated into query heads (OpenReview thread, "GQA Compatibility").
 * - Element types: q, k, v and both caches use cfg.dtype; out uses cfg.out_dtype (DUO_F32,
 *   or equal to cfg.dtype); lse is always float, natural log of the softmax denominator.
 */
#ifndef DUO_H
#define DUO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DUO_OK = 0,
  DUO_ERR_INVALID = 1,     /* bad argument, null pointer, bad layer/sequence, bad config */
  DUO_ERR_CAPACITY = 2,    /* an append would exceed cfg.capacity tokens */
  DUO_ERR_UNSUPPORTED = 3, /* valid but not built: head_dim, group size or dtype */
  DUO_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} duo_status;

typedef enum { DUO_F32 = 0, DUO_BF16 = 1 } duo_dtype;

/* Streaming-head visibility during chunked pre-filling (explainer, "Chunked Pre-filling").
 * WINDOW: query p sees the t <= p with t < S or t >= p - R + 1, the same Lambda mask as
 * decoding. CHUNK: query p of a chunk starting at c sees every token the streaming cache
 * holds at c (the sinks and the R tokens before c) and the chunk's tokens t <= p, the cache
 * being pruned only between chunks. Both agree while c + (position in chunk) < S + R. */
typedef enum { DUO_PREFILL_WINDOW = 0, DUO_PREFILL_CHUNK = 1 } duo_prefill_mode;

/* Cache configuration. head_dim is 64 or 128; G = num_q_heads / num_kv_heads is 1, 2, 4 or
 * 8; sink >= 0 and recent >= 1 (explainer, "The Full and Streaming Attention Masks": the
 * streaming mask keeps the first `sink` tokens and the `recent` most recent ones, the query's
 * own token included). capacity bounds the tokens of each sequence in a retrieval cache. */
typedef struct {
  int32_t num_layers;
  int32_t batch;           /* sequences, 1..512 */
  int32_t num_q_heads;
  int32_t num_kv_heads;    /* 1..64 */
  int32_t head_dim;
  int32_t sink;            /* S */
  int32_t recent;          /* R */
  int32_t capacity;        /* max tokens per sequence, >= 1 */
  int32_t dtype;           /* duo_dtype of q, k, v and the caches */
  int32_t out_dtype;       /* duo_dtype of out */
  float softmax_scale;     /* <= 0 selects 1/sqrt(head_dim) */
  int32_t max_splits;      /* split-K workspace per (sequence, query head), <= 1024;
                              0 selects 256; with kv_bits = 4 not 1 (a retrieval head then
                              uses up to max_splits - 1 context splits plus one partial for
                              its residual rows) */
  int32_t prefill_tiles;   /* prefill split-K workspace in tiles of 128 query rows,
                              <= 65536; 0 selects 2048 */
  const uint8_t* retrieval_mask; /* host [num_layers][num_kv_heads], nonzero = retrieval;
                                    copied by duo_cache_create */
  int32_t streaming_prefill; /* duo_prefill_mode of streaming heads in duo_attn_prefill */
  int32_t kv_bits;         /* 0 or 16: full caches in dtype. 4 or 8: full (retrieval) caches
                              in 4 or 8 bits, see below (bf16 only); streaming caches keep
                              dtype */
  float rope_theta;        /* > 0 (kv_bits = 4 or 8 only): keys are appended before RoPE
                              with this base, see below; <= 0: keys are appended as
                              attended */
} duo_config;

/* 4-bit and 8-bit full caches (cfg.kv_bits = 4 or 8; explainer, "Combination with
 * Quantization": the full caches pair with 4-bit per-channel KV quantization; "Category 3: KV
 * Cache Quantization": 4-bit or 8-bit storage). With L = 15 (4 bits) or 255 (8 bits), codes c
 * in 0..L read back as c * scale + zero with scale = bf16((max - min) / L) and zero =
 * bf16(min) as stored (bf16 round to nearest even), the code being rint((x - zero) / scale) in
 * float32 against the stored values, clamped to 0..L (0 when scale = 0). Keys: per channel
 * over aligned groups of 128 tokens (positions 128 g .. 128 g + 127). Values: per token over
 * the channels. The tokens of the last, incomplete group stay in dtype in a residual block
 * until the group completes. Per retrieval head, with G = ceil(capacity / 128), b the bits
 * and P = max(4 d, 512) G:
 *   K region: codes [128 G][d b / 32] 32-bit words, then P bytes holding bf16 [G][2][d]
 *             (scale row, zero row), then the residual [128][d] in dtype (row t % 128);
 *   V region: codes [G][d * 128 b / 32] words, then P bytes holding one word per token
 *             [128 G] (bf16 scale in the low half, bf16 zero in the high half), then the
 *             residual.
 * 4 bits: a code word holds 8 codes, element e in bits 4e .. 4e + 3. Key row t: the word in
 * slot (d / 32) j + k holds channels 32 k + 8 j .. + 7 of token t. Value group g: word
 * ((s (d / 64) + h) 64 + 16 j + c % 16) 4 + w, with c / 16 = 4 h + w, holds channel c; its
 * element e is token 128 g + 32 s + 16 (e / 4) + 4 j + e % 4.
 * 8 bits: a code word holds 4 codes, element e in byte e. Key row t: the word in slot
 * 2 (d / 32) j + 2 k + h holds channels 32 k + 8 j + 4 h .. + 3. Value group g: word
 * ((s (d / 32) + h) 64 + 16 j + c % 16) 4 + u, with c / 16 = 2 h + u / 2, holds channel c;
 * its element e is token 128 g + 32 s + 16 (u % 2) + 4 j + e.
 * duo_kv_append, duo_attn_decode and duo_decode_step handle them (a step whose token completes
 * a group of some sequence runs as append + decode); duo_attn_prefill_staged pre-fills over
 * them; duo_attn_prefill and duo_attn_gate_mixed return DUO_ERR_UNSUPPORTED on a layer with
 * 4- or 8-bit retrieval caches. */
#define DUO_KV4_GROUP 128

/* Pre-RoPE keys (cfg.rope_theta > 0 with kv_bits = 4 or 8; OpenReview thread, the authors'
 * reply on combining DuoAttention with KV quantization: their 4-bit keys are
 * quantized before the rotary position embedding). The caller passes every key of the layer before RoPE, to
 * duo_kv_append and duo_decode_step alike, and every query after its own rotation; attention
 * scores each key at its own position t. RoPE here is the rotate-half form: channel i < d/2
 * pairs with channel i + d/2 and the pair turns by the angle t * theta^(-2i/d). Every cache
 * keeps the keys as given: a retrieval head's codes, scales and zeros are taken of them, and
 * decoding rotates each dequantized key, each residual row and each streaming slot at the
 * position it holds. Values are never rotated. The cos/sin tables live in the arena (layout.rope_off) and are
 * written by duo_cache_reset. Pre-filling goes through duo_attn_prefill_staged, which stages
 * every key the chunk reads turned (duo_attn_prefill returns DUO_ERR_UNSUPPORTED). */

/* Byte offsets inside the caller's arena (all 256-byte aligned). Inside each cache region
 * the layers follow one another in order, each starting on a 256-byte boundary. */
typedef struct {
  uint64_t arena_bytes;
  uint64_t full_k_off;     /* retrieval caches: per layer [B][H_r][capacity][d] */
  uint64_t full_v_off;
  uint64_t str_k_off;      /* streaming caches: per layer [B][H_s][S+R][d] */
  uint64_t str_v_off;
  uint64_t slot_pos_off;   /* int32 [L][B][S+R]: position held by each slot, -1 = empty */
  uint64_t seq_len_off;    /* int32 [L][B]: tokens appended so far */
  uint64_t workspace_off;  /* split-K partials of decode and prefill (shared) */
  uint64_t workspace_bytes;
  uint64_t rope_off;       /* cfg.rope_theta > 0: the cos/sin tables (library-private
                              contents), rope_bytes long; 0 bytes otherwise */
  uint64_t rope_bytes;
} duo_layout;

typedef struct duo_cache duo_cache; /* opaque host object; owns no device memory */

/* Sizes and offsets of the device arena for `cfg`. Host only. DUO_ERR_INVALID or
 * DUO_ERR_UNSUPPORTED for a bad or unbuilt configuration. The layout is the split KV layout
 * of the explainer's "Deployment Architecture": one full cache per retrieval head and one
 * constant-size cache per streaming head, each head's rows contiguous. */
duo_status duo_layout_query(const duo_config* cfg, duo_layout* out);

/* Build the host object for a cache living in `arena` (device memory of at least
 * layout.arena_bytes, 256-byte aligned). Host only: nothing is launched; call
 * duo_cache_reset before first use. The cache keeps a host mirror of every sequence length
 * so that capacity checks and launch shapes need no device-to-host copy. */
duo_status duo_cache_create(const duo_config* cfg, void* arena, uint64_t arena_bytes,
                            duo_cache** out);

/* duo_cache_create followed by duo_cache_reset on `stream`: a ready, empty cache. */
duo_status duo_cache_init(const duo_config* cfg, void* arena, uint64_t arena_bytes,
                          void* stream, duo_cache** out);

/* Set the length of every sequence of every layer, int32 [L][B] (0 <= len <= capacity;
 * otherwise DUO_ERR_INVALID and nothing changes), for caches whose rows were filled outside
 * the library. Each layer's slot table is rebuilt to match the lengths: slot s holds the
 * latest token t < n with slot(t) = s, or -1 (explainer, "Decoding Procedure", step 4). The
 * K/V rows are not touched. Enqueues one small kernel per layer on `stream`. */
duo_status duo_cache_set_lengths(duo_cache* cache, const int32_t* lens, void* stream);

/* Empty every sequence of every layer: lengths 0, slot table -1; with cfg.rope_theta > 0
 * also (re)write the cos/sin tables at layout.rope_off. Enqueues one fill kernel on `stream`
 * (two with the tables; no memset node, so it can be graph-captured). */
duo_status duo_cache_reset(duo_cache* cache, void* stream);

/* Free the host object (not the arena). NULL is accepted. */
duo_status duo_cache_destroy(duo_cache* cache);

/* Append n_new tokens to one layer (explainer, "Decoding Procedure" step 4 and "Chunked
 * Pre-filling"): for each new position t and KV head, a retrieval head stores K_t, V_t at row
 * t of its full cache; a streaming head stores them at slot t if t < S, else at slot
 * S + (t - S) mod R, but only when the token is still held after the append (t < S or
 * t >= n + n_new - R), which evicts the oldest non-sink tokens. The slot table and lengths
 * are updated. seq = -1 appends n_new tokens to every sequence (k, v [B][n_new][Hkv][d]);
 * seq >= 0 appends to that sequence only (k, v [n_new][Hkv][d]). n_new = 0 is a no-op.
 * DUO_ERR_CAPACITY if a sequence would exceed cfg.capacity. */
duo_status duo_kv_append(duo_cache* cache, int32_t layer, int32_t seq, const void* k,
                         const void* v, int32_t n_new, void* stream);

/* One decoding step of one layer for every sequence (explainer, "Decoding Procedure" steps
 * 1-5). The step's token must already be appended, so the query at position n-1 attends to
 * itself. Retrieval heads attend over all n tokens of their full cache; streaming heads over
 * the sinks and the last R tokens held by their cache (the Lambda mask). Outputs are written
 * in the native head order. q [B][Hq][d]; out [B][Hq][d]; lse [B][Hq] or NULL.
 * DUO_ERR_INVALID if some sequence is empty. */
duo_status duo_attn_decode(duo_cache* cache, int32_t layer, const void* q, void* out,
                           float* lse, void* stream);

/* duo_attn_decode for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments, layouts and
 * result (within floating-point rounding of the split count), but the split-K partials live in
 * a static device array of the library (8 MiB per GPU it runs on, kept until the process
 * ends) instead of the cache's workspace; the call itself allocates and frees nothing. The
 * split count is capped so that batch * num_q_heads * parts * (head_dim + 2) * 4 bytes fit in
 * the array (parts = splits, plus one for a 4- or 8-bit cache's residual rows); DUO_ERR_CAPACITY
 * when not even the least such a cache needs (two parts) fits, nothing launched. Every call on one
 * GPU shares that GPU's array and nothing in it needs to start at zero, but calls that overlap
 * on one GPU (other streams, other caches) race on it. The first call on each device looks the
 * array's device address up (DUO_ERR_HIP if that fails). */
duo_status duo_attn_decode_noalloc(duo_cache* cache, int32_t layer, const void* q, void* out,
                                   float* lse, void* stream);

/* One decoding step with its append fused in (explainer, "Decoding Procedure" steps 1-5):
 * the same result and cache state as duo_kv_append(cache, layer, -1, k, v, 1, stream)
 * followed by duo_attn_decode(cache, layer, q, out, lse, stream), in one pass over the
 * caches. k, v [B][Hkv][d] hold the step's token of every sequence; q, out, lse as in
 * duo_attn_decode. DUO_ERR_CAPACITY if a sequence is full. */
duo_status duo_decode_step(duo_cache* cache, int32_t layer, const void* q, const void* k,
                           const void* v, void* out, float* lse, void* stream);

/* Attention of one pre-filling chunk (explainer, "Chunked Pre-filling"). The chunk holds
 * positions c .. c+m-1 where c is the sequence's current length. Query p attends to every
 * t <= p on retrieval heads (full cache rows 0..c-1 plus the chunk, causally) and, on
 * streaming heads, to the t <= p with t < S or t >= p - R + 1 (sinks and ring before the
 * chunk, plus the chunk) under DUO_PREFILL_WINDOW, or to every token the streaming cache
 * holds plus the chunk's t <= p under DUO_PREFILL_CHUNK (cfg.streaming_prefill). The cache is
 * not modified: the caller then appends the same k, v with duo_kv_append. Layouts as in the
 * header comment; n_chunk = 0 is a no-op. Precision (bf16 caches): the PV product takes the
 * softmax weights and the values in fp16, so value magnitudes must stay below 65504 (the
 * values read, cache rows and chunk alike); the fp32 dtype has no such limit. */
duo_status duo_attn_prefill(duo_cache* cache, int32_t layer, int32_t seq, const void* q,
                            const void* k, const void* v, int32_t n_chunk, void* out,
                            float* lse, void* stream);

/* duo_attn_prefill over a layer whose retrieval caches are in 4 or 8 bits (explainer,
 * "Combination with Quantization": quantized caches serve the whole context). The retrieval
 * heads' earlier tokens are first read back into `staging` as bf16 values, complete groups as
 * bf16(float32(c * scale + zero)) and residual rows as stored, [nb][Hr][c_max][d] for K then
 * the same for V (nb = 1, or B when seq = -1; Hr the layer's retrieval heads; c_max the
 * longest current length among the sequences); the chunk then attends as in duo_attn_prefill,
 * its own keys and values exact. The values (the read-back, the chunk's and the streaming
 * caches') enter staging as fp16 copies of those bf16 values, as the kernel's PV product takes
 * them (below).
 * With cfg.rope_theta > 0 (pre-RoPE keys; OpenReview thread, the authors' reply on KV
 * quantization) q holds the chunk's queries after RoPE and k its keys before RoPE, as
 * appended. Every key the chunk attends to is then staged turned at its own position t
 * (rotate-half pairs (i, i + d/2) by t theta^(-2i/d), in float32) and rounded to bf16: the
 * retrieval prefix after its read-back, the chunk's keys into [nb][m][Hkv][d], and the held
 * streaming slots into [B][Hs][S+R][d]. Values are staged as without RoPE.
 * On a bf16 cache (kv_bits 0) with non-null staging, the values the chunk attends to are
 * first converted to fp16 copies in staging, each element as duo_attn_prefill converts it on
 * the way into its PV product: the retrieval prefix [nb][Hr][c_max][d], the chunk's values
 * [nb][m][Hkv][d] and the streaming caches [B][Hs][S+R][d] (the rows of the call's sequences).
 * The prefill kernel then reads V tiles without converting them, and the outputs and
 * log-sum-exps are bit-identical to duo_attn_prefill's. With null staging, and on an fp32
 * cache, this is duo_attn_prefill.
 * staging: caller-owned device memory, 16-byte aligned, at least
 * duo_prefill_staging_bytes(.., n_chunk, ..) bytes (else DUO_ERR_INVALID); its contents are
 * scratch. On a 4- or 8-bit cache duo_attn_prefill itself returns DUO_ERR_UNSUPPORTED for
 * layers with retrieval heads, and for every layer with cfg.rope_theta > 0. */
duo_status duo_attn_prefill_staged(duo_cache* cache, int32_t layer, int32_t seq, const void* q,
                                   const void* k, const void* v, int32_t n_chunk, void* out,
                                   float* lse, void* staging, uint64_t staging_bytes,
                                   void* stream);

/* Bytes of staging duo_attn_prefill_staged needs for this layer, seq (-1 = all sequences) and
 * a chunk of n_chunk tokens at the cache's current lengths, with P = nb * Hr * c_max * d * 2,
 * C = nb * n_chunk * Hkv * d * 2, T = B * Hs * (S + R) * d * 2 and up() rounding up to 256
 * bytes: up(E) + up(C) + T, the chunk's and the streaming values in fp16 after E bytes of
 * read-backs, where E = 2 P on a 4- or 8-bit cache (E = up(2 P) + up(C) + T with
 * cfg.rope_theta > 0: the turned chunk and streaming keys) and E = P on a bf16 cache (the
 * prefix values in fp16); 0 on an fp32 cache.
 * DUO_ERR_INVALID for a bad layer or seq, n_chunk < 0 or a null `bytes`. Host only. */
duo_status duo_prefill_staging_bytes(const duo_cache* cache, int32_t layer, int32_t seq,
                                     int32_t n_chunk, uint64_t* bytes);

/* Gate-mixed attention of one chunk, the attention of the retrieval-head identification phase
 * (explainer, "Gate Parameterization"): every query head h of KV head j = h / G returns
 * alpha[j] * full_attn + (1 - alpha[j]) * streaming_attn, where full_attn is softmax attention
 * over the t <= p (full cache rows 0..c-1, then the chunk) and streaming_attn the same over the
 * t <= p with t < S or t >= p - R + 1 (explainer, "The Full and Streaming Attention Masks").
 * The two outputs are normalized separately, then blended. Every KV head of `layer` must be a
 * retrieval head (each keeps its full history); alpha: host float [num_kv_heads] in [0, 1].
 * q, k, v, out and the chunk positions as in duo_attn_prefill (no lse); the cache is not
 * modified. Runs as two launches on `stream`: full attention into out, then the windowed
 * attention blended into it (with a bf16 out the full result is rounded once before the blend).
 * DUO_ERR_INVALID for a layer with streaming heads, a gate outside [0, 1] or the argument
 * errors of duo_attn_prefill; DUO_ERR_CAPACITY as there. */
duo_status duo_attn_gate_mixed(duo_cache* cache, int32_t layer, int32_t seq, const void* q,
                               const void* k, const void* v, int32_t n_chunk,
                               const float* alpha, void* out, void* stream);

/* Copy the slot table of one layer, int32 [B][S+R], to host memory. Synchronizes `stream`. */
duo_status duo_slot_positions(duo_cache* cache, int32_t layer, int32_t* host_out,
                              void* stream);

/* Host mirror of the lengths, int32 [L][B]. Host only. */
duo_status duo_cache_lengths(const duo_cache* cache, int32_t* host_out);

/* KV bytes one layer holds for sequences of the given lengths (int32 [B]): under full
 * attention (every KV head keeps every token) and under the split layout
 * (H_r * n + H_s * min(n, S + R)) * d * 2 * element size, summed over sequences (explainer,
 * "Decoding Procedure", memory formula). With 4- or 8-bit full caches the retrieval term is,
 * per head, the codes of the 128 floor(n / 128) grouped tokens (d bits / 4 bytes per token
 * for K and V),
 * their parameters (4 d bytes per key group, 4 bytes per value token) and the residual tokens
 * in dtype. The second figure is also the K/V bytes one decode step of that layer reads.
 * Host only. */
duo_status duo_kv_bytes(const duo_config* cfg, const int32_t* seq_lens, int32_t layer,
                        uint64_t* full_attn_bytes, uint64_t* duo_bytes);

/* Override the number of context splits per retrieval head used by duo_attn_decode
 * (0 = automatic from the lengths; otherwise 1..cfg.max_splits, capped at max_splits - 1 on
 * a 4- or 8-bit cache). The result does not depend on it beyond floating-point rounding. Host only. */
duo_status duo_set_decode_splits(duo_cache* cache, int32_t splits);

/* Kernel timers (a measurement aid, off by default). duo_timing_enable(cache, n) creates n
 * HIP event pairs per kind on the current device (n <= 65536; n = 0 switches timing off and
 * frees the events) and resets the counts; DUO_ERR_HIP if an event cannot be created. While
 * on, each duo_attn_decode / duo_decode_step records one pair on its stream immediately
 * before and after its split attention kernel (the split merge kernel is outside the pair),
 * and each duo_attn_prefill one pair around its attention kernel (the merge outside), until
 * n pairs of that kind are used; later calls run unrecorded. duo_timing_read waits for the
 * last recorded event of `kind`, writes the summed elapsed time of its pairs in
 * milliseconds and their count, and resets that count so the pairs are reused. Calls that
 * overlap on several streams still record, but then a pair spans whatever else the device
 * ran between its two events. */
typedef enum { DUO_TIMING_DECODE = 0, DUO_TIMING_PREFILL = 1 } duo_timing_kind;
duo_status duo_timing_enable(duo_cache* cache, int32_t max_records);
duo_status duo_timing_read(duo_cache* cache, int32_t kind, double* total_ms, int32_t* records);

/* Streaming-read probe (a measurement aid; no passage of the pages defines it). Reads `bytes`
 * bytes at `src` once with the non-temporal 16-byte loads the decode kernels use, in a grid
 * of `blocks` blocks of 256 threads (0: two per compute unit), and stores at most one word at
 * `flag` (device memory, 4 bytes; written only for an improbable XOR of the data, so that the
 * loads stay live). Timed with events around it, it gives the rate a plain read-only kernel
 * reaches on the device, reported beside the decode kernels' bandwidth and the spec peak.
 * src: device memory, 16-byte aligned; bytes: a multiple of 16. DUO_ERR_INVALID otherwise
 * (nothing is launched), DUO_ERR_HIP if the launch fails. */
duo_status duo_read_probe(const void* src, uint64_t bytes, uint32_t* flag, int32_t blocks,
                          void* stream);

/* ---- From trained gates to the deployed head split (one-time preprocessing) ---- */

/* Retrieval/streaming assignment of every KV head of a model from its trained gates
 * (explainer, "Binarization: From Continuous Gates to Hard Assignments", Equation 4: full
 * attention iff the gate exceeds a threshold tau placed at the quantile that keeps a target
 * fraction of the heads). alpha: host float [n_layers][n_kv_heads], finite. The quantile runs
 * over all heads together: the n = floor(ratio * n_layers * n_kv_heads + 0.5) heads (product
 * in double precision) ranked first by decreasing gate, equal gates ranked by (layer, head)
 * ascending, get mask_out = 1 (retrieval), the others 0 (streaming). mask_out: host uint8
 * [n_layers][n_kv_heads], the layout of duo_config.retrieval_mask. tau_out (may be NULL): the
 * gate of the first head left out, -inf when every head is kept; with distinct gates the mask
 * is exactly alpha > tau. n_retrieval_out (may be NULL): n. Host only. DUO_ERR_INVALID for a
 * null alpha or mask_out, sizes below 1, a non-finite gate or ratio outside [0, 1]. */
duo_status duo_binarize_gates(const float* alpha, int32_t n_layers, int32_t n_kv_heads,
                              double ratio, uint8_t* mask_out, float* tau_out,
                              int32_t* n_retrieval_out);

/* Head order of one layer after reordering (explainer, "Head Reordering Preprocessing": the
 * retrieval heads take the first H_r head slots of the Q, K and V projections, the streaming
 * heads the rest). mask: host uint8 [n_kv_heads], nonzero = retrieval. kv_order_out[i]: the
 * native KV head placed at slot i, retrieval heads first, each class in native order.
 * q_order_out (may be NULL) [n_kv_heads * group]: the native query head at each query slot,
 * the group's query heads moving with their KV head (head h belongs to KV head h / group).
 * Host only. DUO_ERR_INVALID for null pointers, n_kv_heads outside 1..1024 or group < 1. */
duo_status duo_head_order(const uint8_t* mask, int32_t n_kv_heads, int32_t group,
                          int32_t* kv_order_out, int32_t* q_order_out);

/* Reorder equal blocks of a device tensor on `stream` (the weight permutation of the same
 * section): dst[o][i] = src[o][order[i]] for o < outer and i < n_blocks, every block
 * block_bytes long. The rows of a Q, K or V projection [heads * head_dim][hidden] are outer
 * = 1, one block of head_dim * hidden elements per head; the columns of the output projection
 * [hidden][heads * head_dim] are outer = hidden, one block of head_dim elements per head.
 * order: host int32 [n_blocks], a permutation of 0..n_blocks-1 (copied into the launch).
 * src and dst: device memory, 16-byte aligned, not overlapping; block_bytes a positive
 * multiple of 16; n_blocks 1..1024; outer * n_blocks * block_bytes / 16 below 2^31. outer = 0
 * is a no-op. DUO_ERR_INVALID otherwise (nothing is launched), DUO_ERR_HIP if the launch
 * fails. */
duo_status duo_permute_blocks(const void* src, void* dst, int64_t outer, int32_t n_blocks,
                              int64_t block_bytes, const int32_t* order, void* stream);

/* Static text for a status code. */
const char* duo_status_string(duo_status status);

#ifdef __cplusplus
}
#endif

#endif /* DUO_H */
