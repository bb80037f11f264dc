/*
 * mk.h — C ABI of the MI355X batch-1 decode megakernel library (libmk.so).
 *
 * One decode step of a Llama-style decoder runs as ONE persistent kernel launch, as
 * in the Hazy Research "Megakernel" article on Llama-3.2-1B (section "Megakernel: a
 * fusion design from scratch"): the whole forward pass — RMSNorm+QKV+RoPE, grouped-
 * query attention over the cache, O-projection+residual, RMSNorm+SiLU(gate)*up,
 * down-projection+residual, final RMSNorm+LM head — is executed by an on-GPU
 * instruction interpreter following per-CU instruction lists that a host-side
 * scheduler lays out once, before the first token, and reuses for every token.
 *
 * Conventions for every entry point:
 *   - Return 0 (MK_OK) on success or a negative MK_E* code; no call throws.
 *   - "device pointer" = memory on the context's HIP device (e.g. torch-allocated);
 *     the library borrows it and never frees it.  The caller keeps it alive and
 *     unmodified for as long as the context may use it.
 *   - bf16 matrices are row-major [out][in] (a row is one output feature), dense.
 *   - One context serves one stream at a time; calls on one context are not
 *     thread-safe.  Work is asynchronous on the given stream unless stated.
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MK_OK 0
#define MK_EINVAL -1   /* null pointer, bad shape, unsupported configuration          */
#define MK_ERANGE -2   /* pos >= max_ctx, or token outside [0, vocab)                  */
#define MK_ESTATE -3   /* weights not loaded, or context in an unusable state         */
#define MK_EHIP -4     /* a HIP runtime call failed; mk_strerror() names it            */
#define MK_ETIMEOUT -5 /* a device-side bounded wait expired (the step was abandoned) */
#define MK_ENOMEM -6   /* device allocation failed                                    */

/* Model shape and numerics.  The article's model is Llama-3.2-1B: 16 layers, hidden
 * 2048, 32 query / 8 KV heads of 64, SwiGLU 8192, vocab 128256.  The kernel is compiled
 * for a fixed list of widths (hidden, query heads, KV heads, head_dim, ffn): the
 * Llama-3.2-1B and Llama-3.1-8B shapes (4096, 32, 8, 128, 14336) and three small test
 * decoders; n_layers, vocab and max_ctx are free.  mk_create rejects other widths with
 * MK_EINVAL and lists the compiled ones (mk_strerror). */
typedef struct mk_config {
  int32_t n_layers;
  int32_t hidden;      /* d                                   */
  int32_t n_q_heads;   /* Hq                                  */
  int32_t n_kv_heads;  /* Hkv                                 */
  int32_t head_dim;    /* hd                                  */
  int32_t ffn;         /* F (SwiGLU intermediate)             */
  int32_t vocab;       /* V                                   */
  int32_t max_ctx;     /* KV-cache slots per (layer, kv head) */
  float rms_eps;       /* RMSNorm epsilon, inside the root    */
  float rope_theta;    /* RoPE base (rotate-half pairing)     */
} mk_config;

/* Borrowed device pointers to bf16 weights.  The per-layer entries are HOST arrays of
 * n_layers device pointers each; the library copies the arrays, not the weights.
 *   embed      [vocab][hidden]      token embedding (row gathered, not scaled)
 *   lm_head    [vocab][hidden]      may equal embed (tied)
 *   final_norm [hidden]             RMSNorm gain before the LM head
 *   attn_norm  [hidden]             per layer, gain before QKV
 *   wq [Hq*hd][hidden], wk [Hkv*hd][hidden], wv [Hkv*hd][hidden]
 *   wo [hidden][Hq*hd]
 *   mlp_norm   [hidden]             per layer, gain before gate/up
 *   w_gate, w_up [ffn][hidden], w_down [hidden][ffn]                              */
typedef struct mk_weights {
  const void* embed;
  const void* lm_head;
  const void* final_norm;
  const void* const* attn_norm;
  const void* const* wq;
  const void* const* wk;
  const void* const* wv;
  const void* const* wo;
  const void* const* mlp_norm;
  const void* const* w_gate;
  const void* const* w_up;
  const void* const* w_down;
} mk_weights;

typedef struct mk_ctx mk_ctx;

/* Create a context for `cfg` on HIP device `hip_device`.  Validates the shape,
 * queries the device (compute units) and checks that one work-group of the step kernel
 * fits on a CU; allocates nothing yet.  Each step launches one work-group per CU, and
 * all of them must be resident at once (they wait on each other's results), so a step
 * only completes once no other kernel holds CUs.
 * Serves the article's interpreter, which gives every streaming multiprocessor its own
 * execution plan (Megakernel article, section "Megakernel: a fusion design from
 * scratch", interpreter paragraph); here one work-group per CU takes that role.
 * Errors: MK_EINVAL (null/unsupported shape, mk_strerror names the compiled shapes),
 * MK_EHIP (no such device, or the kernel does not fit on a CU). */
int mk_create(const mk_config* cfg, int hip_device, mk_ctx** out);

/* Record the weight pointers and build the static schedule: per-CU instruction lists
 * (article: plans laid out statically before runtime and reused for every token,
 * section "Megakernel: a fusion design from scratch", static-plan paragraph), the
 * device-side communication buffers, the RoPE cos/sin table [max_ctx][hd/2] (fp32,
 * computed in double on the host) and the control block.  Synchronous; allocates with
 * hipMalloc (about 11 MB for the Llama-3.2-1B shape).  May be called again to switch
 * weights.  Matrices must be 16-byte aligned, gains 4-byte aligned.
 * Errors: MK_EINVAL (null or misaligned pointer), MK_ENOMEM, MK_EHIP. */
int mk_load_weights(mk_ctx* ctx, const mk_weights* w);

/* One decode step (asynchronous on `stream`, a hipStream_t; NULL = default stream):
 * the article's six fused instructions for one token, RMSNorm+QKV+RoPE through the
 * final RMSNorm + LM head, in one kernel launch (section "Megakernel: a fusion design
 * from scratch", instruction list; the greedy choice is the plainest reading of
 * generating one token).
 *   token      input token id, in [0, vocab)
 *   pos        its position; keys 0..pos are attended; 0 <= pos < max_ctx
 *   kv_cache   device bf16 [n_layers][2 (K,V)][n_kv_heads][max_ctx][head_dim], 16-byte
 *              aligned; slots [0, pos) must hold the keys (already rotated) and values of
 *              the prefix; slot pos of every layer is overwritten with the new K, V
 *              (rounded to bf16, round-to-nearest-even); slots past pos are neither read nor
 *              written.
 *   logits_out device fp32 [vocab], 4-byte aligned: logits of the next token.
 *   next_token device int32 [1] or NULL: receives argmax(logits), lowest index on ties.
 * Differs from a bare (token, pos, kv_cache, logits_out) signature by the optional
 * next_token output and the stream argument (void*, so the header needs no HIP header).
 * Errors: MK_ESTATE (no weights), MK_ERANGE, MK_EINVAL (null or misaligned buffer),
 * MK_EHIP.  A device-side failure (MK_ETIMEOUT) is reported by the next mk_sync(); every
 * step launched after the failed one and before that mk_sync() does nothing (it writes
 * no cache slot, logits or token).  After such a failure the cache slot `pos` of the
 * failed step may hold the new K/V of some layers and not of others: run that step
 * again after mk_sync(). */
int mk_decode_step(mk_ctx* ctx, int32_t token, int32_t pos, void* kv_cache,
                   float* logits_out, int32_t* next_token, void* stream);

/* As mk_decode_step, but the token is read on the device from token_dev (device
 * int32 [1]) when the step starts — e.g. the previous step's next_token — so a
 * greedy loop needs no host synchronisation between steps (the article reuses one
 * schedule for many tokens: section "Megakernel: a fusion design from scratch",
 * static-plan paragraph).  token_dev and next_token may be the same buffer.
 * Out-of-range device tokens are clamped to [0, vocab) by the kernel and flagged as
 * MK_ERANGE at the next mk_sync().  Errors as mk_decode_step, plus MK_EINVAL for a
 * null or misaligned token_dev. */
int mk_decode_step_dev(mk_ctx* ctx, const int32_t* token_dev, int32_t pos, void* kv_cache,
                       float* logits_out, int32_t* next_token, void* stream);

/* As mk_decode_step, for callers that cannot allocate device memory while they run
 * steps: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  It calls no hipMalloc, hipFree or other allocating routine: the step's
 * scratch (communication words, argmax keys, control block, token sink) lives in a
 * 16 MiB array the library holds statically on every device it runs on (set up by
 * mk_create; held until the process ends), instead of the context's own buffers.  The
 * context must have weights loaded (mk_load_weights allocates once, at set-up).  Shapes
 * whose scratch exceeds 16 MiB (wider than the Llama-3.2-1B shape) are rejected with
 * MK_EINVAL and a message giving the size needed.  Every context on one GPU shares that
 * array and it keeps the last step's contents: calls that overlap on one GPU (from other
 * streams or threads, or interleaved with another context's calls on another stream)
 * race and must not be made.  A device-side failure is reported by mk_sync(ctx); the
 * array is then re-armed (on the device, no allocation) by the next call of this entry.
 * Errors as mk_decode_step, plus MK_ESTATE if the device's array was not set up. */
int mk_decode_step_noalloc(mk_ctx* ctx, int32_t token, int32_t pos, void* kv_cache,
                           float* logits_out, int32_t* next_token, void* stream);

/* Wait for the context's outstanding steps on `stream` and surface device-side
 * errors: MK_ETIMEOUT (a bounded wait expired; the article's counter waits are
 * unbounded, section "Megakernel: a fusion design from scratch", counter paragraph —
 * here every wait has a budget), MK_ERANGE for a clamped device token.  After an error
 * the context resets its device state (communication words, control block) on the
 * next step.  Errors: MK_EINVAL (null), MK_ESTATE (no weights), MK_EHIP. */
int mk_sync(mk_ctx* ctx, void* stream);

/* Device-side wait budget in microseconds (default 2,000,000).  Every bounded wait in
 * the kernel gives up after this long, records MK_ETIMEOUT and exits; 0 makes every
 * wait give up at its first round (a step then fails unless no wave ever waits).
 * Errors: MK_EINVAL (null context, negative budget). */
int mk_set_watchdog_us(mk_ctx* ctx, int64_t us);

/* Schedule introspection (host only; valid after mk_load_weights or mk_plan_only).
 * mk_plan_info fills: [0] number of CUs planned, [1] instruction record size in
 * int32 words, [2] total records, [3] page bytes, [4] pages in the LDS ring,
 * [5] compute waves per CU, [6] attention splits per KV head, [7] LDS bytes.
 * mk_plan_copy copies `n_cus`+1 list offsets then the records (int32 words). */
int mk_plan_info(const mk_ctx* ctx, int32_t info[8]);
int mk_plan_copy(const mk_ctx* ctx, int32_t* offsets, int32_t* records, int64_t records_capacity_words);

/* Build only the static schedule for a hypothetical device with `n_cus` compute units
 * (no HIP calls, no allocation on any device): for host-side tests of the scheduler. */
int mk_plan_only(const mk_config* cfg, int n_cus, mk_ctx** out);

/* Debug: copy the device communication words of the last step to host memory
 * (synchronous).  Each word is (fp32 value | epoch << 32).  offsets[0..5] receive the
 * word offsets of: x after each residual [2L+1][hidden] (entry 0 unused), raw q/k/v
 * [L][kv head][q heads of the group | k | v][head_dim], split partials, attention
 * output [L][Hq*hd], SiLU(gate)*up [L][ffn], and the total word count; `host` may be
 * NULL to query the offsets only.  Errors: MK_ESTATE before mk_load_weights. */
int mk_debug_dump(const mk_ctx* ctx, uint64_t* host, int64_t capacity_words, int64_t offsets[6]);

/* Per-instruction timestamp trace: the MI355X form of the article's time breakdown of
 * one forward (section "Megakernel: a fusion design from scratch", results paragraph).
 * dev_buf is a borrowed device buffer of uint64 [n_cus][L][12] with L the longest per-CU
 * instruction list, at most 272; *required_words receives n_cus * L * 12 (pass dev_buf
 * NULL to query, which also turns tracing off).  The buffer must be zeroed before every traced step;
 * the step writes, per CU and instruction i, s_memrealtime ticks (100 MHz): [0] leader
 * starts i, [1] it starts polling i's inputs, [2] the inputs are all present, [3] i's
 * activation slot is free, [4] activation staged, [5] compute wave 0 starts i, [6] the
 * last compute wave finished i (a running maximum), [7] leader finished i (incl.
 * attention merge / argmax), [8] leader saw every compute wave finish i (attention and
 * LM head only), [9] ticks the compute waves spent waiting for i's weight (or cached
 * key/value) pages to land, summed over the waves (a duration, not a time stamp), [10]
 * a loader wave issued the first of i's pages that go through the LDS ring, [11] ticks
 * the loader waves spent waiting for a ring slot with nothing of their own in flight
 * while holding one of i's pages, summed over the two loaders (a duration: the CU's HBM
 * stream idles then because its buffers are full).
 * Tracing changes no result.  Errors: MK_ESTATE before a schedule exists, MK_EINVAL if
 * the buffer is too small or not 8-byte aligned. */
int mk_set_trace(mk_ctx* ctx, uint64_t* dev_buf, int64_t capacity_words, int64_t* required_words);

/* Free everything the context allocated (not the borrowed weights or caches).  Waits
 * for nothing: the caller must have synchronised the context's streams.  NULL is a
 * no-op.  (Host-side teardown of the plan's owner, no citation needed.) */
void mk_destroy(mk_ctx* ctx);

/* Static text for an MK_* code.  For MK_EHIP and MK_EINVAL it gives the detail of the
 * failure of this thread's last ABI call, if that call recorded one. */
const char* mk_strerror(int code);

/* ---- Measurement (not part of the decode path) ---------------------------------
 * A plain streaming read of `bytes` bytes at device pointer `buf` (both 16-byte
 * multiples/aligned): `blocks` work-groups of 256 threads, each thread keeping `unroll`
 * (1, 4, 8 or 16) 16-byte non-temporal loads in flight, grid-stride over the buffer.  It
 * is the practical HBM read ceiling the decode step's bandwidth is reported against (the
 * pages model a forward as its bytes over the part's bandwidth: Megakernel article,
 * section "Why are traditional inference methods so inefficient?", bandwidth paragraph).
 * unroll -8: plain (cached) loads instead of non-temporal ones, 8 in flight.
 * `sink` is device uint32 [blocks], written only for an input no caller produces (it
 * keeps the loads live).  Asynchronous on `stream`; time it with events on that stream.
 * Errors: MK_EINVAL (bad size, alignment or launch shape), MK_EHIP (launch failed). */
int mk_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t blocks, int32_t unroll, void* stream);

/* Per-page cost of the matrix-vector work on the compute units (a measurement, not part
 * of the decode path): `blocks` work-groups of 4 waves, each wave computing `pages` times
 * one 16 KiB page (4 rows x 2048 bf16, the Llama-3.2-1B row) against an fp32 activation,
 * operands already in LDS.  variant 0: fp32 FMA on the widened bf16 (the decode kernel's
 * path); 1: v_dot2 on bf16 pairs against a two-term bf16 split of the activation; 2: the
 * 16x16x32 bf16 matrix instruction against a three-term split; 3: the LDS reads alone.
 * The article finds the best matrix-vector unit differs by GPU generation (section
 * "Megakernel: a fusion design from scratch", matrix-vector paragraph).  ticks: device
 * uint64 [blocks * 4], s_memrealtime ticks (100 MHz) per wave; out: device fp32
 * [blocks * 4 * 8]: per wave, 4 running sums then the first page's 4 row results.
 * Errors: MK_EINVAL (bad variant, sizes or null), MK_EHIP (launch failed). */
int mk_bench_gemv_page(int32_t variant, int32_t pages, int32_t blocks, unsigned long long* ticks, float* out,
                       void* stream);

/* Round trip of one dependency poll while the CU streams weights (a measurement, not
 * part of the decode path): `blocks` work-groups; in each, one wave times `probes` loads
 * of single 64-bit words (probe_words: device uint64 [blocks * probes * 16], read only;
 * vector agent-scope loads, or scalar loads past the scalar cache when `scalar` is 1),
 * about 1 us apart, while two waves stream the work-group's `region_bytes` slice of
 * stream_buf (device, blocks * region_bytes bytes, read only) into LDS with 1 KiB
 * LDS-direct loads, keeping `depth` (0-4) pages of 16 KiB in flight each — as the decode
 * step's loaders do.  The article's consistency waits are this poll, repeated (section
 * "Megakernel: a fusion design from scratch", counter paragraph).  out: device uint64
 * [blocks * (probes + 4)]: ticks (100 MHz) per probe, then per work-group the time the
 * probes ended, the pages each loader streamed (two words) and the loaders' start time,
 * for the streaming rate at that depth.  Errors: MK_EINVAL, MK_EHIP. */
int mk_bench_poll_latency(const void* stream_buf, int64_t region_bytes, const uint64_t* probe_words, int32_t depth,
                          int32_t scalar, int32_t probes, int32_t blocks, unsigned long long* out, void* stream);

/* Time for `blocks` single-wave work-groups to read 16 KiB of 64-bit words with
 * agent-scope loads, `reps` times ~0.5 us apart: all the same 16 KiB (shared = 1, the
 * decode step's activation broadcast) or each its own (shared = 0; buf then holds blocks
 * * 16 KiB).  out: device uint64 [blocks * reps], ticks per read.  A measurement.
 * Errors: MK_EINVAL, MK_EHIP. */
int mk_bench_bcast_read(const uint64_t* buf, int32_t shared, int32_t reps, int32_t blocks, unsigned long long* out,
                        void* stream);

/* Library version string. */
const char* mk_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
