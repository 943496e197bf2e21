/*
 * kvq.h -- C ABI of libkvq: SRFT-rotated low-bit KV-cache quantization and fused
 * single-token decode attention for AMD Instinct MI355X (gfx950).
 *
 * Method (sources are web pages, cited by title and section):
 *   [QF] "When Quantization Is Free: An int4 KV Cache That Outruns fp16 on Apple Silicon",
 *        gist.science explainer, technical summary, Methodology 1 (SRFT(x) = pack(F diag(s) x),
 *        F the unitary DFT, s a fixed random sign vector), Methodology 2 (one fused write kernel:
 *        sign, FFT, Hermitian pack, per-channel lambda, per-group absmax, signed int4/int8
 *        rounding, nibble packing) and Methodology 3 (per-channel + per-group-of-16 scaling).
 *   [KS] xugj520 article on KVSplit, "核心技术创新": keys 8-bit, values 4-bit (K8V4).
 *   [GM] hotdry blog on Gemini KV caches on Apple Silicon, "Flash Attention 与 Metal 内核融合":
 *        tiled attention with an online softmax.
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless the comment says "host".  The caller owns and
 *     allocates every buffer; the library allocates nothing, frees nothing and keeps no
 *     pointer after the call returns.
 *   - Every compute call is asynchronous on `stream` (a hipStream_t passed as void*; NULL is the
 *     default stream).  Launch errors are reported as KVQ_ERR_HIP; faults during execution
 *     surface at the caller's next synchronization.
 *   - Arguments are validated on the host before any HIP call.  On any error the call returns
 *     without launching work and leaves every output untouched; kvq_last_error_message() then
 *     holds a thread-local description.
 *   - Plane, input and output pointers must be 16-byte aligned (KVQ_ERR_MISALIGNED otherwise);
 *     sign and lambda vectors must be 4-byte aligned.
 *   - The library is reentrant and thread-safe; calls on distinct streams may overlap.
 *   - Non-finite inputs give unspecified (but in-range) codes.
 *
 * Cache layout ("planes"; separate code and scale planes per tensor)
 *   For a tensor quantized with `bits` (4 or 8), head dimension d and group size g (16, or d):
 *     codes : uint8 [batch, kv_heads, capacity, d*bits/8]
 *             int4: byte j of a token holds channel 2j in its low nibble and channel 2j+1 in its
 *             high nibble, each a two's-complement 4-bit code in [-7, 7];
 *             int8: one two's-complement byte per channel, codes in [-127, 127].
 *     scales: fp16  [batch, kv_heads, capacity, d/g], one scale per group of g consecutive
 *             channels of the rotated vector.  g = 16 is the method's grouping ([QF]
 *             Methodology 3); g = d (one scale per vector, the per-token scaling that the
 *             per-group scheme replaces) is a comparison mode of kvq_quantize and
 *             kvq_dequantize only.
 *   Channel c of the rotated vector is the real, norm-preserving layout of the unitary DFT of
 *   s*x: c=0 -> Re X0, c=1 -> Re X_{d/2}, c=2k -> sqrt2 Re Xk, c=2k+1 -> sqrt2 Im Xk (0<k<d/2),
 *   with Xk = d^-1/2 sum_n s_n x_n exp(-2 pi i k n / d).
 *   `batch` may fold layers (batch = layers x sequences): sign and lambda take a batch stride.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, q_heads % kv_heads != 0, range */
  KVQ_ERR_UNSUPPORTED = 2,      /* head_dim not 128/256, group not 16 (or d: write path   */
                                /* only), bits not 4/8, G > 64                            */
  KVQ_ERR_MISALIGNED = 3,       /* a pointer violates the alignment rule above */
  KVQ_ERR_WORKSPACE_TOO_SMALL = 4,
  KVQ_ERR_HIP = 5               /* a HIP runtime call or kernel launch failed */
} kvq_status;

/* Host struct describing one quantized cache (passed by const pointer, read during the call). */
typedef struct {
  int32_t batch;      /* sequences (optionally x layers); >= 1                                */
  int32_t kv_heads;   /* >= 1                                                                   */
  int32_t q_heads;    /* multiple of kv_heads; GQA ratio G = q_heads / kv_heads; head h reads  */
                      /* kv head h / G                                                          */
  int32_t head_dim;   /* d: 128 or 256                                                          */
  int32_t group_size; /* 16; or head_dim: one scale per vector (kvq_quantize, kvq_dequantize and */
                      /* the sizing calls only; the decode calls return KVQ_ERR_UNSUPPORTED)   */
  int32_t k_bits;     /* 4 or 8 (K8V4 is [KS]'s pairing; K4V8 and K8V8 are the other widths)   */
  int32_t v_bits;     /* 4 or 8                                                                 */
  int32_t capacity;   /* tokens allocated per (sequence, kv head): the token stride of planes   */
  int32_t transform;  /* rotation of the write path and of the decode: KVQ_TRANSFORM_SRFT (0,    */
                      /* [QF] Methodology 1) or KVQ_TRANSFORM_SRHT (1, the pages' alternative:  */
                      /* d^-1/2 H diag(s) x with the Sylvester-ordered Walsh-Hadamard matrix)   */
} kvq_layout;

enum { KVQ_TRANSFORM_SRFT = 0, KVQ_TRANSFORM_SRHT = 1 };

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t kvq_version(void);

/* Name of a status code (static string). */
const char* kvq_status_string(kvq_status status);

/* Thread-local text describing the last failed call on this thread ("" if none). */
const char* kvq_last_error_message(void);

/* Bytes of one code plane: batch * kv_heads * capacity * head_dim * bits / 8.
 * Footprint formula of the hotdry blog ("INT8/INT4 量化策略") with b-bit codes.
 * Returns 0 if the layout or bits are invalid. Host-only, no HIP call. */
size_t kvq_codes_bytes(const kvq_layout* layout, int32_t bits);

/* Bytes of one scale plane: batch * kv_heads * capacity * (head_dim / group_size) * 2: one fp16
 * scale per group of 16 channels ([QF] Methodology 3, per-group scaling), the scale term of the
 * hotdry blog's footprint formula ("INT8/INT4 量化策略").  0 if the layout is invalid. */
size_t kvq_scales_bytes(const kvq_layout* layout);

/*
 * kvq_quantize -- the write path ([QF] Methodology 2 and 3).
 * For every vector x = x_f16[b, h, t, :] (t < n_tok) writes token pos + t of row (b, h):
 *   u      = SRFT_s(x) / lambda                  (s = sign row b, lambda = lambda row (b, h))
 *   scale  = fp16(max_{c in group} |u_c| / qmax) (round to nearest even, saturated at 65504)
 *   code_c = clamp(round_half_even(u_c / scale), -qmax, qmax), 0 where scale == 0
 * qmax = 7 (bits 4) or 127 (bits 8).  The code decision is taken in float32.
 *   bits      : 4 or 8 (the tensor's width; use layout->k_bits for K, layout->v_bits for V)
 *   x_f16     : fp16 [batch, kv_heads, n_tok, head_dim], contiguous
 *   pos,n_tok : 0 <= pos, 1 <= n_tok, pos + n_tok <= capacity
 *   sign      : float [*, head_dim] of +-1; row b starts at b * sign_batch_stride (0 = shared)
 *   lambda    : float [*, kv_heads, head_dim], > 0; row b at b * lambda_batch_stride (0 = shared);
 *               NULL means lambda = 1
 *   codes     : code plane (see layout above); scales: scale plane
 * Only the written tokens' bytes change.
 */
kvq_status kvq_quantize(const kvq_layout* layout, int32_t bits, const void* x_f16, int32_t pos,
                        int32_t n_tok, const float* sign, int64_t sign_batch_stride,
                        const float* lambda, int64_t lambda_batch_stride, void* codes,
                        void* scales, void* stream);

/*
 * kvq_quantize_fft -- the same write path as kvq_quantize, with the rotation computed as an
 * in-register radix-2 FFT of length head_dim/2 plus the Hermitian unpack ([QF] Methodology 1 and
 * 2: the FFT, the Hermitian pack and the rest of the fused write kernel's steps), one GPU lane per vector,
 * instead of as a matrix product on the matrix cores.  Same arguments, validation, outputs and
 * error codes as kvq_quantize; its codes and scales meet the write path's bar against the same
 * definition (they may differ from kvq_quantize's on float32 near-ties of the rounding).
 */
kvq_status kvq_quantize_fft(const kvq_layout* layout, int32_t bits, const void* x_f16, int32_t pos,
                            int32_t n_tok, const float* sign, int64_t sign_batch_stride,
                            const float* lambda, int64_t lambda_batch_stride, void* codes,
                            void* scales, void* stream);

/*
 * kvq_dequantize -- inverse of the write path ([QF] Methodology 2 run backwards: unpack, times
 * scale and lambda, inverse rotation, sign), for inspection and tests.
 *   out[b, h, t, :] = s * SRFT^-1(lambda * code * scale) for tokens pos .. pos+n_tok-1,
 *   out: float [batch, kv_heads, n_tok, head_dim], contiguous.  Other arguments as kvq_quantize.
 */
kvq_status kvq_dequantize(const kvq_layout* layout, int32_t bits, const void* codes,
                          const void* scales, int32_t pos, int32_t n_tok, const float* sign,
                          int64_t sign_batch_stride, const float* lambda,
                          int64_t lambda_batch_stride, float* out, void* stream);

/*
 * kvq_calibrate_lambda -- per-channel calibration of lambda (the pages call lambda "learned or
 * calibrated", [QF] Methodology 2): lambda[b, h, c] = max_{t < n_cal} |SRFT_s(x[b, h, t])_c|,
 * replaced by 1 where that maximum is 0.
 *   x_f16  : fp16 [batch, kv_heads, n_tok, head_dim] contiguous; 1 <= n_cal <= n_tok
 *   lambda : float [batch, kv_heads, head_dim] output
 */
kvq_status kvq_calibrate_lambda(const kvq_layout* layout, const void* x_f16, int32_t n_tok,
                                int32_t n_cal, const float* sign, int64_t sign_batch_stride,
                                float* lambda, void* stream);

/* Workspace bytes kvq_decode_attn / kvq_decode_attn_fp16 need for any seq_len <= max_seq_len.
 * 0 if the layout is invalid. */
size_t kvq_decode_attn_workspace_bytes(const kvq_layout* layout, int32_t max_seq_len);

/*
 * kvq_decode_attn -- fused dequant + single-token decode attention over the quantized cache
 * ([GM] tiled attention with online softmax; [QF] Methodology 1 rotation).  For every sequence
 * b and query head h (kv head j = h / G), with L = seq_lens ? seq_lens[b] : seq_len:
 *   out[b, h] = sum_{t<L} softmax_t(sm_scale * q[b,h] . x_hat_K[b,j,t]) x_hat_V[b,j,t]
 * where x_hat = s * SRFT^-1(lambda * code * scale).  Computed in the rotated domain: the query is
 * rotated once, scores and the value sum use the codes directly, and the output is
 * inverse-rotated once.
 *   q_f16        : fp16 [batch, q_heads, head_dim] contiguous
 *   k_codes, ... : the four planes (K with layout->k_bits, V with layout->v_bits)
 *   seq_len      : 1 <= seq_len <= capacity (the maximum length when seq_lens is given)
 *   seq_lens     : device int32 [batch] or NULL; entries are clamped to [0, seq_len]; a sequence
 *                  of length 0 gets a zero output
 *   sign_k/v     : float [*, head_dim] +-1, row stride sign_batch_stride (0 = shared)
 *   lambda_k/v   : float [*, kv_heads, head_dim] or NULL (= 1), row stride lambda_batch_stride
 *   sm_scale     : softmax scale; <= 0 selects 1/sqrt(head_dim)
 *   workspace    : >= kvq_decode_attn_workspace_bytes(layout, seq_len) bytes, 256-byte aligned.
 *                  Its first 65536 bytes are completion counters: zero them once after
 *                  allocating the workspace; every call that runs to completion leaves them
 *                  zero.  The rest is scratch.  After a call that did not complete (a launch
 *                  error reported by a later call, a device fault, a stream torn down while
 *                  it ran), zero the first 65536 bytes again before the next call: stale
 *                  counters make later calls merge at the wrong count.
 *                  One workspace serves one call at a time (calls in flight on different
 *                  streams need their own); in use until the work on `stream` completes.
 *                  batch * kv_heads * (G / head tile) must not exceed 16384, where the head
 *                  tile is the largest divisor of G = q_heads / kv_heads that is at most 16
 *                  (head_dim 128) or 8 (head_dim 256); KVQ_ERR_UNSUPPORTED otherwise.
 *   out          : float [batch, q_heads, head_dim]
 */
kvq_status kvq_decode_attn(const kvq_layout* layout, const void* q_f16, const void* k_codes,
                           const void* k_scales, const void* v_codes, const void* v_scales,
                           int32_t seq_len, const int32_t* seq_lens, const float* sign_k,
                           const float* sign_v, int64_t sign_batch_stride, const float* lambda_k,
                           const float* lambda_v, int64_t lambda_batch_stride, float sm_scale,
                           void* workspace, size_t workspace_bytes, float* out, void* stream);

/*
 * kvq_decode_attn_noalloc -- kvq_decode_attn without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the call makes no allocation of any kind.  Its completion counters and chunk
 * partials live in a device array built into the library, 32 MiB (33554432 bytes) per GPU, held
 * until the process ends; the first call on a device looks up that device's copy and clears its
 * counters (a fill kernel on `stream`), and every call that runs to completion leaves them zero.
 * All calls on one GPU share the array: calls whose execution overlaps on one GPU (different
 * streams, or host threads) race and give wrong results; serialize them.  After a call that did not
 * complete, the counters are stale and later calls of this entry point give wrong results.
 * Computation, precision, plan and result are those of kvq_decode_attn (the same kernels).
 * Arguments as kvq_decode_attn without workspace/workspace_bytes.
 * Errors: those of kvq_decode_attn; KVQ_ERR_WORKSPACE_TOO_SMALL when the call would need more than
 * the built-in 32 MiB (kvq_decode_attn_workspace_bytes(layout, seq_len) > 33554432, e.g. very many
 * chunks of many units); KVQ_ERR_HIP if the scratch cannot be set up.
 */
kvq_status kvq_decode_attn_noalloc(const kvq_layout* layout, const void* q_f16, const void* k_codes,
                                   const void* k_scales, const void* v_codes, const void* v_scales,
                                   int32_t seq_len, const int32_t* seq_lens, const float* sign_k,
                                   const float* sign_v, int64_t sign_batch_stride,
                                   const float* lambda_k, const float* lambda_v,
                                   int64_t lambda_batch_stride, float sm_scale, float* out,
                                   void* stream);

/*
 * kvq_decode_attn_append -- one decode step in one launch: the write path ([QF] Methodology 2,
 * the steps of the fused kernel) on the step's new K and V vectors, then kvq_decode_attn over
 * the cache that now holds them ([QF] Key results: one vector written per head and step, the
 * whole prefix read).  For every sequence b with L = seq_lens ? seq_lens[b] : seq_len
 * (clamped to [0, seq_len]) and L >= 1, and every kv head j, the vectors k_new[b, j] and
 * v_new[b, j] are quantized into position L - 1 of the planes as kvq_quantize(pos = L - 1,
 * n_tok = 1) does with the same signs and lambdas (K with layout->k_bits, V with
 * layout->v_bits); then out is what kvq_decode_attn returns for that cache.  A sequence with
 * L = 0 is not written and gets a zero output.
 *   k_new, v_new : fp16 [batch, kv_heads, head_dim] contiguous, 16-byte aligned
 *   k_codes, ... : the four planes, read and (at L - 1) written
 *   other arguments, the workspace rules and the error behaviour as kvq_decode_attn, except
 *   that the head tile is the largest divisor of G that is at most 14 (head_dim 128) or 8
 *   (head_dim 256).  Positions other than L - 1 are not written.  The codes agree with
 *   kvq_quantize's to the write path's parity bar (the two use the same arithmetic).
 */
kvq_status kvq_decode_attn_append(const kvq_layout* layout, const void* q_f16, const void* k_new_f16,
                                  const void* v_new_f16, void* k_codes, void* k_scales, void* v_codes,
                                  void* v_scales, int32_t seq_len, const int32_t* seq_lens,
                                  const float* sign_k, const float* sign_v, int64_t sign_batch_stride,
                                  const float* lambda_k, const float* lambda_v,
                                  int64_t lambda_batch_stride, float sm_scale, void* workspace,
                                  size_t workspace_bytes, float* out, void* stream);

/*
 * kvq_decode_attn_paged -- kvq_decode_attn (and, with k_new_f16/v_new_f16, the fused append of
 * kvq_decode_attn_append) over a paged cache: the planes hold num_pages pages of page_size
 * tokens, codes uint8 [num_pages, kv_heads, page_size, d*bits/8] and scales fp16
 * [num_pages, kv_heads, page_size, d/16], and token t of sequence b lives in page
 * page_table[b * pages_per_seq + t / page_size] at offset t % page_size.  This answers the
 * cache-management concerns of [GM] ("KV 缓存分片与内存管理": a full num_ctx reservation per
 * sequence, prefix reuse across requests, sliding-window eviction): a cache grows by pages,
 * sequences may point at the same pages for a shared prefix, and a window is a table whose
 * leading entries the caller retires.  The computation, its precision and its result are those
 * of kvq_decode_attn on the same tokens.  An appending call writes only the page holding
 * position L - 1 of each sequence, which must not be shared with another sequence of the call.
 *   page_table    : device int32 [batch, pages_per_seq]; entries are clamped to [0, num_pages)
 *                   on the device (an out-of-range entry reads a wrong page, never out of the
 *                   planes); entries of pages past a sequence's length are not read
 *   page_size     : a positive multiple of 64 (KVQ_ERR_UNSUPPORTED otherwise)
 *   pages_per_seq : >= 1, and layout->capacity must equal pages_per_seq * page_size
 *   num_pages     : >= 1, pages in the planes
 *   k_new_f16, v_new_f16 : both NULL (attend only) or both set (append token L - 1 of every
 *                   sequence into its page first, as kvq_decode_attn_append; the head tile
 *                   limit of that call applies)
 * Other arguments, the workspace rules and the errors are those of kvq_decode_attn; the
 * workspace size from kvq_decode_attn_workspace_bytes covers paged calls.
 */
kvq_status kvq_decode_attn_paged(const kvq_layout* layout, const void* q_f16, const void* k_new_f16,
                                 const void* v_new_f16, void* k_codes, void* k_scales, void* v_codes,
                                 void* v_scales, const int32_t* page_table, int32_t pages_per_seq,
                                 int32_t page_size, int32_t num_pages, int32_t seq_len,
                                 const int32_t* seq_lens, const float* sign_k, const float* sign_v,
                                 int64_t sign_batch_stride, const float* lambda_k,
                                 const float* lambda_v, int64_t lambda_batch_stride, float sm_scale,
                                 void* workspace, size_t workspace_bytes, float* out, void* stream);

/*
 * kvq_decode_attn_fp16 -- the same decode attention over an unquantized fp16 cache, the baseline
 * the quantized cache is measured against ([GM] "INT8/INT4 量化策略": the fp16 cache of 2 bytes
 * per element that int4 shrinks to 25%; [QF] Key results: int4 decode against fp16 KV).
 * k_f16, v_f16 are fp16 [batch, kv_heads, capacity, head_dim]; no rotation, no lambda.
 * layout->k_bits/v_bits are ignored.  Other arguments as kvq_decode_attn.
 */
kvq_status kvq_decode_attn_fp16(const kvq_layout* layout, const void* q_f16, const void* k_f16,
                                const void* v_f16, int32_t seq_len, const int32_t* seq_lens,
                                float sm_scale, void* workspace, size_t workspace_bytes,
                                float* out, void* stream);

/*
 * kvq_launch_plan -- how a call splits its work (host only, no HIP call): for capacity planning,
 * occupancy reasoning and tests that must reach a given loop depth.  The split is the one the
 * call itself launches with; it depends on the layout and n only.
 *   call : KVQ_CALL_QUANTIZE (n = n_tok of kvq_quantize) or one of the decode calls (n = seq_len)
 *   out  : host struct, written on success
 * Decode calls: one work-group per (sequence, kv head, head tile, chunk of `chunk` tokens); each
 * of its 4 waves walks superblocks of `wave_tokens` tokens, so a wave handles up to
 * superblocks_per_wave of them.  Quantize: 16-vector blocks, each work-group a contiguous range of
 * at most blocks_per_work_group of them.  Fields that do not apply to a call are 0.
 * Errors: KVQ_ERR_INVALID_ARGUMENT / KVQ_ERR_UNSUPPORTED as the call itself would return for the
 * layout and n.
 */
typedef enum {
  KVQ_CALL_QUANTIZE = 0,
  KVQ_CALL_DECODE = 1,              /* kvq_decode_attn */
  KVQ_CALL_DECODE_APPEND = 2,       /* kvq_decode_attn_append */
  KVQ_CALL_DECODE_PAGED = 3,        /* kvq_decode_attn_paged without new vectors */
  KVQ_CALL_DECODE_PAGED_APPEND = 4, /* kvq_decode_attn_paged with new vectors */
  KVQ_CALL_DECODE_FP16 = 5          /* kvq_decode_attn_fp16 */
} kvq_call;

typedef struct {
  int64_t work_groups;           /* grid size of the call's kernel                         */
  int32_t head_tile;             /* decode: query heads per work-group                     */
  int32_t head_tiles;            /* decode: G / head_tile                                  */
  int32_t chunk;                 /* decode: tokens per work-group                          */
  int32_t n_chunks;              /* decode: work-groups per (sequence, kv head, head tile) */
  int32_t wave_tokens;           /* decode: tokens of one wave superblock (64; fp16: 32)   */
  int32_t superblocks_per_wave;  /* decode: ceil(chunk / (4 * wave_tokens))                */
  int64_t blocks;                /* quantize: 16-vector blocks of the call                 */
  int64_t blocks_per_work_group; /* quantize: largest block range of one work-group        */
  int32_t query_tile;            /* kvq_attn: query tokens per work-group (decode calls: 1) */
  int32_t query_tiles;           /* kvq_attn: ceil(n_query / query_tile) (decode calls: 1)  */
} kvq_plan;

kvq_status kvq_launch_plan(const kvq_layout* layout, kvq_call call, int32_t n, kvq_plan* out);

/*
 * kvq_attn -- attention of several query tokens per sequence over the quantized cache, with an
 * optional sliding window, on contiguous rows, a ring buffer or a paged cache.
 *   Several query tokens: the step before single-token decode (chunked prefill, speculative
 *   verification: [GM] "Flash Attention 与 Metal 内核融合", tiled attention with an online
 *   softmax).  The n_query new tokens are the last n_query positions of every sequence's cache
 *   (already written with kvq_quantize); query i of a sequence of length L sits at position
 *   p = L - n_query + i and attends positions t <= p (causal).  A query with p < 0 gets a zero
 *   output.
 *   Sliding window ([GM] "KV 缓存分片与内存管理": keep the latest tokens): with window W >= 1 a
 *   query at p attends only t in [max(0, p - W + 1), p].
 *   Ring buffer: position t of a row is stored at slot t % capacity (contiguous rows) or at
 *   page_table[b * pages_per_seq + (t % capacity) / page_size], offset t % page_size (paged), so a
 *   row of `capacity` slots holds the latest `capacity` positions of an unbounded sequence.
 * For every sequence b, query token i and query head h (kv head h / G):
 *   out[b, i, h] = sum_t softmax_t(sm_scale * q[b, i, h] . x_hat_K[b, j, t]) x_hat_V[b, j, t]
 * over the positions above; computed in the rotated domain as kvq_decode_attn does (same kernel
 * family; n_query = 1 with no window gives kvq_decode_attn's result).
 *   opts         : host struct (n_query >= 1, window >= 0 with 0 = none, ring 0 or 1)
 *   q_f16        : fp16 [batch, n_query, q_heads, head_dim] contiguous
 *   page_table   : NULL for contiguous rows (planes [batch, kv_heads, capacity, .]); otherwise
 *                  device int32 [batch, pages_per_seq] with the page rules of
 *                  kvq_decode_attn_paged (page_size a multiple of 64, capacity = pages_per_seq x
 *                  page_size, entries clamped to [0, num_pages))
 *   seq_len      : the largest length; without a ring 1 <= seq_len <= capacity; with a ring any
 *                  seq_len >= 1, capacity a multiple of 64, window >= 1 and
 *                  window + n_query - 1 <= capacity (the attended positions of a unit are
 *                  still in the ring)
 *   seq_lens     : device int32 [batch] or NULL, clamped to [0, seq_len]
 *   workspace    : >= kvq_attn_workspace_bytes(layout, opts, seq_len) bytes, 256-byte aligned,
 *                  first 65536 bytes zeroed counters, as kvq_decode_attn's
 *   out          : float [batch, n_query, q_heads, head_dim]
 * Other arguments and errors as kvq_decode_attn / kvq_decode_attn_paged.
 */
typedef struct {
  int32_t n_query; /* query tokens per sequence, >= 1                              */
  int32_t window;  /* 0: no window; W >= 1: the W latest positions up to the query */
  int32_t ring;    /* 0: position t at slot t; 1: at slot t % capacity             */
} kvq_attn_opts;

kvq_status kvq_attn(const kvq_layout* layout, const kvq_attn_opts* opts, const void* q_f16,
                    const void* k_codes, const void* k_scales, const void* v_codes,
                    const void* v_scales, const int32_t* page_table, int32_t pages_per_seq,
                    int32_t page_size, int32_t num_pages, int32_t seq_len, const int32_t* seq_lens,
                    const float* sign_k, const float* sign_v, int64_t sign_batch_stride,
                    const float* lambda_k, const float* lambda_v, int64_t lambda_batch_stride,
                    float sm_scale, void* workspace, size_t workspace_bytes, float* out,
                    void* stream);

/* Workspace bytes kvq_attn needs for any seq_len <= max_seq_len with these options (contiguous or
 * paged).  0 if the layout or options are invalid. */
size_t kvq_attn_workspace_bytes(const kvq_layout* layout, const kvq_attn_opts* opts,
                                int32_t max_seq_len);

/* The launch shape of kvq_attn (host only), as kvq_launch_plan describes the other calls; paged:
 * nonzero for a paged cache.  query_tile / query_tiles give the split of the query tokens. */
kvq_status kvq_attn_launch_plan(const kvq_layout* layout, const kvq_attn_opts* opts, int32_t seq_len,
                                int32_t paged, kvq_plan* out);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
