/*
 * kivi.h -- C ABI of libkivi, a gfx950 (MI355X) library for single-token
 * decode attention over a KIVI-style asymmetrically quantized KV cache.
 *
 * Sources (web pages; cited by page and section, never by line):
 *   [P1] discosf.com KIVI tutorial (news/3594501): section 2.1 (KV-cache size
 *        formula; keys have per-channel outliers, values do not), section 3.1
 *        (group-wise quantization plus an fp16 remainder window), section 3.2
 *        (value cache management), section 5.2 (parameters nbits,
 *        q_group_size, residual_length).
 *   [P2] unite.ai "KV cache quantization axis selection guide": section on
 *        what quantization error is made of (uniform min/step quantizer,
 *        step = range / (2^B - 1), error <= step/2), section on keys (outliers
 *        sit in fixed channels, so keys are grouped per channel), section on
 *        values (values are grouped per token), section on rotary
 *        embeddings (quantize keys before the rotation), section on the
 *        systems tax (recent tokens stay full precision until enough
 *        accumulate), future-directions section (high-precision windows for
 *        the recent and the attention-sink tokens).
 *
 * Everything here is asynchronous on the caller's HIP stream.  The library
 * never allocates, frees or synchronises; every buffer is caller-owned device
 * memory (for example torch tensors) in the layouts documented below, dense
 * and contiguous.  Alignment: the 32-bit arrays (q_len, r_len, status,
 * tickets, prefill's len and res) and the fp32 output start on a 4-byte
 * boundary; every other buffer (codes, scales, zeros, fp16 rows, the query,
 * the new and the sink tokens, prefill's source, the workspace) on a 16-byte
 * boundary (torch allocations start on 256 bytes).  A null or misaligned
 * pointer gives KIVI_EINVAL before anything is launched.  No C++ exception crosses this boundary.  Calls on
 * different caches are independent and reentrant; a cache must not be
 * touched concurrently from two streams.
 */
#ifndef KIVI_H
#define KIVI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes (host side) ------------------------------------------ */
#define KIVI_OK            0
#define KIVI_EINVAL       -1  /* bad dims, null or misaligned pointer, bad scalar */
#define KIVI_ENOSPC       -2  /* workspace smaller than kivi_decode_workspace_bytes */
#define KIVI_EHIP         -3  /* a kernel launch failed (hipGetLastError)      */
#define KIVI_EUNSUPPORTED -4  /* valid dims that no compiled kernel covers     */

/* ---- sticky device status bits, OR-ed into *status by kernels ----------- */
#define KIVI_ST_RESIDUAL_FULL 0x1u /* append found r_len == R: token dropped  */
#define KIVI_ST_CAPACITY      0x2u /* flush/prefill would pass capacity       */
#define KIVI_ST_BAD_LENGTH    0x4u /* a length array held an impossible value */
#define KIVI_ST_TICKETS       0x8u /* a ticket counter (cache->tickets or the
                                      decode workspace) did not start at zero:
                                      it was never initialised; that call's
                                      length commit or split merge is lost */

/*
 * Problem dimensions.  The names follow the pages' parameters:
 *   bits      B, the code width ("nbits", [P1] section 5.2: 2, 4 or 8 bits).
 *   group     G, tokens per key group and channels per value group
 *             ("q_group_size", [P1] sections 3.1 and 5.2).  Must divide
 *             head_dim, residual and capacity.
 *   residual  R, the fp16 window length ("residual_length", [P1] 3.1/5.2);
 *             a multiple of G.
 *   capacity  quantized tokens each sequence can hold; a multiple of G.
 *   batch, heads, head_dim as in the cache-size formula of [P1] section 2.1.
 * Host validation (kivi_validate_dims): all > 0 except capacity >= 0,
 * bits in {2,4,8}, head_dim % group == 0, residual % group == 0,
 * capacity % group == 0, (head_dim * bits) % 32 == 0.
 * Compiled kernels cover head_dim == 128 and group in {32, 64, 128};
 * other valid dims return KIVI_EUNSUPPORTED.
 */
typedef struct {
  int32_t batch, heads, head_dim, bits, group, residual, capacity;
} kivi_dims;

/*
 * The cache.  W = head_dim * bits / 32 words per token; D = head_dim.
 *
 *   k_codes  uint32 [batch][heads][capacity/G][W][G]
 *   v_codes  uint32 [batch][heads][capacity/G][W][G]
 *       Codes are stored in tiles of G consecutive tokens.  Inside a tile,
 *       word (w, t) holds the codes of token t of the tile for channels
 *       w*(32/B) + i, i in [0, 32/B); channel w*(32/B)+i sits at bits
 *       [i*B, i*B + B) (least significant first).  Token n of a sequence is
 *       in tile n / G at position n % G.
 *   k_scale, k_zero  fp16 [batch][heads][capacity/G][D]
 *       Per key group (G consecutive tokens x 1 channel): the step and the
 *       group minimum ([P2] keys section; [P1] section 3.1).
 *   v_scale, v_zero  fp16 [batch][heads][capacity/G][D/G][G]
 *       Per value group (1 token x G consecutive channels): step and minimum
 *       ([P2] values section; [P1] section 2.1).  Stored in the same tiles
 *       of G tokens as the codes, group-major inside a tile: the value of
 *       token n, channel group j is at [n / G][j][n % G].
 *   k_res, v_res     fp16 [batch][heads][R][D]   the fp16 window.
 *   q_len  int32 [batch]  quantized tokens held (multiple of G, <= capacity)
 *   r_len  int32 [batch]  window tokens held, 0 <= r_len <= R
 *   status uint32 [1]     sticky KIVI_ST_* bits (caller clears it).
 *   tickets uint32 [batch][64]  per-sequence counters of kivi_flush_residual
 *                          and kivi_decode_step (element [b][0]; the rest
 *                          of each row keeps counters on separate cache
 *                          lines); zero before first use (kivi_cache_init
 *                          or a zero-filled allocation), left zero by every
 *                          call.  A counter found non-zero is reported as
 *                          KIVI_ST_TICKETS and that sequence's lengths are
 *                          then not committed.
 * Sequence b's context is its q_len[b] quantized tokens followed by its
 * r_len[b] window tokens, oldest first.
 *
 * Dequantized value of a code c with step s and minimum z: z + c * s.
 * Quantizer (fixed fp32 sequence, identical in every kernel that encodes):
 *   mn = min(x) + 0.0f; mx = max(x) + 0.0f; s = fp16_rne((mx - mn) / (2^B - 1));
 *   c = s == 0 ? 0 : clamp(rint_half_even((x - mn) / (float)s), 0, 2^B - 1);
 *   stored zero = fp16(mn) (exact), stored scale = s.
 * ([P2] quantization-error section: zero-point = minimum, step = range over
 *  the number of levels, round to the nearest step.)
 */
typedef struct {
  void *k_codes, *k_scale, *k_zero;
  void *v_codes, *v_scale, *v_zero;
  void *k_res, *v_res;
  int32_t *q_len, *r_len;
  uint32_t *status;
  uint32_t *tickets;
} kivi_cache;

/* Host-only check of dims; KIVI_OK, KIVI_EINVAL or KIVI_EUNSUPPORTED. */
int kivi_validate_dims(const kivi_dims *dims);

/*
 * Make a freshly allocated cache empty and ready: q_len[b] = r_len[b] = 0
 * for every sequence, every element of cache->tickets and *status zero.
 * Codes, scales, zeros and the window are left as they are (an empty
 * cache never reads them).  Enqueued as one kernel on `stream` (no memset,
 * so it may be captured in a HIP graph); allocates nothing.  Every other
 * call leaves cache->tickets zero again, so this is needed once per cache
 * (or after a KIVI_ST_TICKETS report).  KIVI_EINVAL for bad dims or a null
 * or misaligned pointer.
 */
int kivi_cache_init(const kivi_dims *dims, const kivi_cache *cache, void *stream);

/*
 * Make a decode workspace ready for use: zero-fills the counters that
 * kivi_decode_attn and its variants use to find the last workgroup of a
 * split (sequence, head).  workspace_bytes must be at least
 * kivi_decode_workspace_bytes(dims) (else KIVI_ENOSPC).  One kernel on
 * `stream` (no memset); allocates nothing.  Every decode leaves the counters
 * zero again, so this is needed once per workspace (or after a
 * KIVI_ST_TICKETS report); a workspace allocated zero-filled needs no call.
 */
int kivi_workspace_init(const kivi_dims *dims, void *workspace, size_t workspace_bytes,
                        void *stream);

/*
 * Append one new token per sequence to the fp16 window ([P1] section 3.2:
 * new tokens enter the window in fp16).
 *   k_new, v_new  fp16 [batch][heads][D], device.
 * For every b with r_len[b] < R: writes slot r_len[b] of k_res/v_res, then
 * r_len[b] += 1.  A sequence with r_len[b] >= R (or a negative r_len) is left
 * unchanged and KIVI_ST_RESIDUAL_FULL (or KIVI_ST_BAD_LENGTH) is set.
 */
int kivi_append_kv(const kivi_dims *dims, const kivi_cache *cache,
                   const void *k_new, const void *v_new, void *stream);

/*
 * Flush full windows ([P1] section 3.1: once R tokens have accumulated they
 * are quantized group-wise and the window is emptied; [P2] systems section).
 * For every b with r_len[b] == R: window tokens [0, R) are quantized (keys as
 * R/G per-channel groups, values as R per-token groups of G channels) into
 * quantized token slots [q_len[b], q_len[b] + R); then q_len[b] += R and
 * r_len[b] = 0.  Sequences with r_len[b] < R are untouched.  If
 * q_len[b] + R > capacity the sequence is untouched and KIVI_ST_CAPACITY is
 * set.  One kernel: the workgroup that finishes reading sequence b's
 * lengths last updates them (through cache->tickets).
 */
int kivi_flush_residual(const kivi_dims *dims, const kivi_cache *cache,
                        void *stream);

/*
 * Initialise every sequence from a prompt (the remainder split of [P1]
 * section 3.1).  k, v: fp16 [batch][heads][src_len][D], device.
 * len: device int32 [batch], tokens of sequence b, 0 <= len[b] <= src_len.
 * res: device int32 [batch] window tokens to keep, or NULL for len[b] % G.
 * Tokens [0, len-res) are quantized into slots [0, len-res) and tokens
 * [len-res, len) are copied to window slots [0, res); then q_len[b] =
 * len-res, r_len[b] = res.  Sequences whose len-res is not a multiple of G,
 * or with res outside [0, R] or len outside [0, src_len], are left with
 * q_len = r_len = 0 and KIVI_ST_BAD_LENGTH set; len-res > capacity sets
 * KIVI_ST_CAPACITY likewise.  Codes are bit-identical to those that appends
 * plus flushes of the same tokens produce.
 */
int kivi_prefill(const kivi_dims *dims, const kivi_cache *cache,
                 const void *k, const void *v, int32_t src_len,
                 const int32_t *len, const int32_t *res, void *stream);

/*
 * Bytes of workspace kivi_decode_attn needs for these dims (a function of
 * batch, heads, bits, group, residual and capacity only).
 */
size_t kivi_decode_workspace_bytes(const kivi_dims *dims);

/* Number of token splits per (sequence, head) kivi_decode_attn launches. */
int kivi_decode_splits(const kivi_dims *dims);

/*
 * Number of kernels kivi_decode_step launches for these dims: 1 (the
 * whole-step kernel) or 3 (append, decode, flush).  Negative error code for
 * invalid or unsupported dims.
 */
int kivi_decode_step_kernels(const kivi_dims *dims);

/*
 * Decode attention for one new query token per (sequence, head):
 *   out[b,h,:] = softmax(sm_scale * q[b,h,:] . Khat^T) . Vhat
 * over the q_len[b] dequantized tokens followed by the r_len[b] fp16 window
 * tokens ([P2] values section: the output is a softmax-weighted sum of the
 * value vectors; [P2] "why the KV cache matters": the whole cache is read for
 * every generated token).  An empty context gives out = 0.
 *   q        fp16 [batch][heads][D], device
 *   out      fp32 [batch][heads][D], device (written)
 *   workspace  device buffer of at least kivi_decode_workspace_bytes(dims)
 *            bytes.  Before its first use it must go through
 *            kivi_workspace_init (or be allocated zero-filled); every call
 *            leaves its counters zero again.  A workspace whose counters
 *            were not zero makes the split merge of that call lose its
 *            output for the (sequence, head) pairs split over several
 *            workgroups, and sets KIVI_ST_TICKETS.  One workspace must not
 *            be used by two calls that can run at the same time.
 * Read-only on the cache.  A sequence whose lengths are impossible (q_len not
 * a multiple of G or above capacity, r_len outside [0, R]) gets out = 0 and
 * KIVI_ST_BAD_LENGTH.  Returns KIVI_ENOSPC if workspace_bytes is too small.
 */
int kivi_decode_attn(const kivi_dims *dims, const kivi_cache *cache,
                     const void *q, float *out, float sm_scale,
                     void *workspace, size_t workspace_bytes, void *stream);

/*
 * kivi_decode_attn without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The split partials and their counters
 * live in one device array inside the library, 8 MiB per GPU, held until the
 * process ends; this call allocates nothing (no hipMalloc, no hipFree, no
 * allocating library routine).  The same result as kivi_decode_attn bit for
 * bit (the same kernels).  Limits: batch * heads <= 4096 and
 * batch * heads * kivi_decode_splits(dims) * (head_dim + 4) * 4 bytes <= 7 MiB
 * (the 131072-token, 32-head workload takes 135 KB), else KIVI_ENOSPC with
 * nothing launched.  Every call on one GPU shares that GPU's array: calls
 * that can overlap on one GPU (on two streams, or from two threads without
 * ordering) race and give wrong outputs.  The first call on a device takes
 * the array's device address and clears its counters with a kernel on
 * `stream`.  Other arguments and errors as kivi_decode_attn.
 */
int kivi_decode_attn_noalloc(const kivi_dims *dims, const kivi_cache *cache,
                             const void *q, float *out, float sm_scale, void *stream);

/*
 * kivi_decode_attn with an fp16 attention-sink segment ([P2]
 * future-directions section: besides the window of recent tokens, a
 * high-precision window is kept for the attention-sink tokens, the first
 * tokens of the sequence).  The attention runs over the n_sink sink tokens,
 * then the q_len[b] quantized tokens, then the r_len[b] window tokens:
 *   out = softmax(sm_scale * q . [K_sink; K^; K_res]^T) . [V_sink; V^; V_res]
 *   k_sink, v_sink  device fp16 [batch][heads][n_sink][head_dim], contiguous,
 *                   owned by the caller and only read (typically the
 *                   prompt's first n_sink rows, with the cache built from
 *                   the rest); the same n_sink for every sequence
 *   n_sink          0 .. 4096; with rope_base 0, n_sink 0 gives exactly
 *                   kivi_decode_attn (the pointers are then not read and
 *                   may be NULL)
 *   rope_base       0: no rotary embedding (positions play no part).
 *                   Otherwise > 1 and finite: keys stored before the
 *                   rotation, as in kivi_decode_attn_rope, with sink token
 *                   s at position s, quantized token t at n_sink + t and
 *                   window slot r at n_sink + q_len[b] + r; q already
 *                   rotated.  The sink keys are stored before the rotation
 *                   too.
 * Other arguments, layouts, workspace and errors as kivi_decode_attn;
 * KIVI_EINVAL for n_sink out of range, a NULL or misaligned sink pointer
 * with n_sink > 0, or a bad rope_base.  An empty cache with n_sink > 0
 * attends over the sink alone.
 */
int kivi_decode_attn_sink(const kivi_dims *dims, const kivi_cache *cache,
                          const void *k_sink, const void *v_sink, int32_t n_sink,
                          const void *q, float *out, float sm_scale, double rope_base,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * kivi_decode_attn for keys stored before the rotary embedding ([P2]
 * rotary-embedding section: quantize keys before the rotation and apply it
 * after dequantization, since rotating first mixes an outlier channel into
 * its partner; its list of things to do calls this a correctness matter).
 * Every key -- quantized or in the fp16 window, exactly as
 * kivi_append_kv / kivi_flush_residual / kivi_prefill stored it -- is
 * rotated after dequantization by its position in the sequence: quantized
 * tokens take positions 0 .. q_len[b] - 1, window slot r takes q_len[b] + r.
 * Channel pair f = (2f, 2f + 1), f < head_dim / 2, turns by the angle
 * position * rope_base^(-2f / head_dim) (the original rotary embedding; a
 * head stored in the "rotate half" pairing maps onto it by one fixed channel
 * permutation of queries and keys).  q must already be rotated to the new
 * token's position.  Values are not rotated.
 *   rope_base  > 1 and finite (10000 for Llama-2)
 * Other arguments, layouts, workspace and errors as kivi_decode_attn;
 * KIVI_EINVAL for a bad rope_base.  Angles are formed in fp64 and the
 * sine and cosine taken in fp32.
 */
int kivi_decode_attn_rope(const kivi_dims *dims, const kivi_cache *cache,
                          const void *q, float *out, float sm_scale,
                          double rope_base, void *workspace,
                          size_t workspace_bytes, void *stream);

/*
 * ---- value queue ([P1] section 3.2, value cache management) -----------
 * A cache kept with these four calls (and only these) holds its values in
 * an fp16 queue of the newest R: each appended value enters the queue and,
 * once R are queued, the oldest leaves it and is quantized on its own (per
 * token, D/G groups of G channels, the quantizer above).  Keys keep the
 * window of kivi_append_kv / kivi_flush_residual ([P1] section 3.1).  With
 * T = q_len[b] + r_len[b] tokens in all, the first vq = max(0, T - R) values
 * are quantized (value position t at [t / G][..][t % G] of the value tiles,
 * exactly the codes the bulk per-token quantizer gives token t), and v_res
 * is a ring: the value of token t >= vq is in slot t mod R.  The context is
 * tokens [0, vq) with quantized keys and values, [vq, q_len) with quantized
 * keys and fp16 values, [q_len, T) with fp16 keys and values.  The buffers,
 * lengths, status bits and errors are those of the calls without _vq.
 */

/* kivi_prefill for a value-queue cache: keys as kivi_prefill; of the values,
 * tokens [0, max(0, len - R)) quantized, the rest copied to ring slots
 * t mod R; value positions past the quantized ones left zero. */
int kivi_prefill_vq(const kivi_dims *dims, const kivi_cache *cache,
                    const void *k, const void *v, int32_t src_len,
                    const int32_t *len, const int32_t *res, void *stream);

/* Append one token per sequence: the key to key-window slot r_len[b] (as
 * kivi_append_kv); with T = q_len[b] + r_len[b] >= R, the value in ring slot
 * T mod R (token T - R) is first quantized into value position T - R; the
 * slot then takes the new value; r_len[b] += 1.  One kernel (a workgroup
 * per sequence); KIVI_ST_RESIDUAL_FULL / KIVI_ST_BAD_LENGTH as
 * kivi_append_kv. */
int kivi_append_kv_vq(const kivi_dims *dims, const kivi_cache *cache,
                      const void *k_new, const void *v_new, void *stream);

/* kivi_flush_residual for a value-queue cache: a full key window becomes R/G
 * key groups (q_len += R, r_len = 0); the values are not touched. */
int kivi_flush_residual_vq(const kivi_dims *dims, const kivi_cache *cache,
                           void *stream);

/* kivi_decode_attn over a value-queue cache's context (above), in token
 * order; arguments, workspace and errors as kivi_decode_attn. */
int kivi_decode_attn_vq(const kivi_dims *dims, const kivi_cache *cache,
                        const void *q, float *out, float sm_scale,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * One whole generation step: kivi_append_kv, then kivi_decode_attn, then
 * kivi_flush_residual ([P1] section 3.1: append to the fp16 window, attend
 * over quantized and window tokens, quantize the window once it holds R
 * tokens), arguments as there.  The cache contents, lengths and status bits
 * are exactly those of the three calls in that order; the output is theirs
 * up to rounding (the summation order may differ).  When one workgroup
 * covers a whole (sequence, head) (kivi_decode_splits: 1) and the grid is
 * at most one workgroup per compute unit (batch * heads <= 256) and B is 2
 * or 4, it is a single kernel: each workgroup appends its (sequence, head)'s
 * token, uses it from registers in the attention, and if the window is then full quantizes
 * it (from the registers that hold it for the attention when R <= 128, else
 * re-reading it), and the last workgroup of the sequence commits the lengths
 * through cache->tickets.  Otherwise it launches the three kernels.
 * Errors as for the three calls; KIVI_ENOSPC if workspace_bytes is too small.
 */
int kivi_decode_step(const kivi_dims *dims, const kivi_cache *cache,
                     const void *k_new, const void *v_new, const void *q,
                     float *out, float sm_scale, void *workspace,
                     size_t workspace_bytes, void *stream);

/*
 * kivi_decode_step with the decode over an fp16 attention-sink segment
 * first ([P2] future-directions section): the same cache state as
 * kivi_append_kv, kivi_decode_attn_sink (rope_base 0) and
 * kivi_flush_residual in that order, the output equal up to rounding; one
 * kernel under the same condition as kivi_decode_step.  k_sink, v_sink and
 * n_sink as in kivi_decode_attn_sink (n_sink 0 gives kivi_decode_step).
 * Errors as kivi_decode_step and kivi_decode_attn_sink.
 */
int kivi_decode_step_sink(const kivi_dims *dims, const kivi_cache *cache,
                          const void *k_new, const void *v_new,
                          const void *k_sink, const void *v_sink, int32_t n_sink,
                          const void *q, float *out, float sm_scale,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * Measurement aid, not a step of the method: reads `bytes` bytes of device
 * memory at `src` once with 16-byte loads and writes one XOR fold per wave
 * to `sink`, so that its duration gives the HBM read rate the device
 * sustains for that size, the ceiling against which the decode's achieved
 * bandwidth is also reported.  `workgroups` 512-thread workgroups each
 * stream one contiguous slice of about bytes / workgroups.
 *   src   device, 16-byte aligned; bytes a non-zero multiple of 16
 *   sink  device uint32 [workgroups * 8] (written; the values mean nothing)
 * Returns KIVI_EINVAL for a null pointer, a misaligned or empty buffer, or
 * workgroups outside [1, 2^20].  Asynchronous on `stream`; allocates nothing.
 */
int kivi_stream_read(const void *src, size_t bytes, int32_t workgroups,
                     uint32_t *sink, void *stream);

/* Static description of a return code. */
const char *kivi_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* KIVI_H */
