/*
 * kvq.h - low-bit KV-cache quantize-on-append and packed-cache decode attention
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (sources cited by page and section):
 *   - "KVQuant reading notes": keys quantized per channel and before RoPE, values
 *     per token (sections 3.1, 3.2, 3.6); non-uniform codebooks looked up by
 *     argmin (sections 1.2, 3.3); about 1% of each vector kept exactly in fp16 as
 *     sparse outliers, CSR for keys and CSC for values (section 3.4); the
 *     attention kernel dequantizes, merges outliers and applies RoPE on the fly
 *     (section 3.7, Algorithm 1).
 *   - "KVarN" summary: a 128-point Hadamard rotation across channels and 8
 *     Sinkhorn-style variance-normalisation iterations per 128-token block before
 *     RTN, with a second stored scale s1 (core method, method steps).
 *   - "reproducing TurboQuant" blog: symmetric int4 over 128-element
 *     sequence-direction blocks with fp16 scales, dequantized inside attention
 *     (sections 2.1, 4.1, 4.2, 5.2).
 *
 * Conventions for every function:
 *   - Host-callable, never throws, returns kvq_status (KVQ_OK = 0).
 *   - "dev" pointers are device pointers (hipMalloc / torch CUDA tensors); "host"
 *     pointers are host memory. The caller owns every buffer it passes and keeps
 *     it alive until the stream has passed the call.
 *   - stream is a hipStream_t (NULL = the default stream). Work is enqueued on it
 *     and the call returns without synchronizing, except kvq_cache_init, which
 *     synchronizes its stream once after uploading its tables.
 *   - Arguments, shapes and state are validated on the host before anything is
 *     launched; a failed check launches nothing and changes no state.
 *     kvq_last_error() describes the last failure of the calling thread.
 *   - Device faults surface at the caller's next synchronization.
 *   - One handle is used from one stream at a time; calls on one handle that
 *     overlap on different streams race (they share the decode workspace).
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
  KVQ_ERR_ARG = -1,       /* invalid argument or configuration */
  KVQ_ERR_SIZE = -2,      /* a buffer is too small */
  KVQ_ERR_CAPACITY = -3,  /* append would exceed max_tokens */
  KVQ_ERR_STATE = -4,     /* operation not valid in the current state */
  KVQ_ERR_HIP = -5        /* a HIP runtime call failed */
} kvq_status;

typedef enum {
  KVQ_MODE_RTN = 0,       /* asymmetric uniform RTN, min/range (KVQuant notes 1.2, 3.1) */
  KVQ_MODE_NUQ = 1,       /* codebook argmin on [-1, 1] (KVQuant notes 1.2, 3.3) */
  KVQ_MODE_KVARN = 2,     /* Hadamard + VarN + RTN with s1 (KVarN core method) */
  KVQ_MODE_SYM_INT4 = 3,  /* symmetric int4 (int8 with bits = 8), fp16 scales (TurboQuant blog 4.2) */
  KVQ_MODE_ASYM_INT4 = 4  /* asymmetric int4 clamp(round((x - zero) / scale), -8, 7), fp16 scale and
                             zero (TurboQuant blog 2.1) */
} kvq_mode;

#define KVQ_HEAD_DIM 128
#define KVQ_BLOCK_TOKENS 128
#define KVQ_MAX_OUTLIERS 8
#define KVQ_MAX_GROUP 8
#define KVQ_MAX_SPLITS 64
#define KVQ_STATIC_SCRATCH_BYTES (8u << 20)
#define KVQ_MAX_SINK 128
#define KVQ_MAX_WINDOW 8192
#define KVQ_MAX_PAGED_BATCH 64
#define KVQ_MAX_POOL_BYTES (4294967296ull - 131072ull)

typedef struct {
  int32_t n_layers;         /* >= 1 */
  int32_t batch;            /* >= 1; every sequence holds the same number of tokens, except in
                               a paged cache (paged_pages > 0), where each has its own */
  int32_t n_kv_heads;       /* >= 1 */
  int32_t n_q_heads;        /* multiple of n_kv_heads, group n_q_heads/n_kv_heads in {1,2,4,8} */
  int32_t head_dim;         /* must be 128 */
  int32_t max_tokens;       /* capacity per sequence and layer, multiple of 128, >= 128 */
  int32_t mode;             /* kvq_mode */
  int32_t bits;             /* 2, 3 or 4; 8 with RTN, KVARN or SYM_INT4 (the blog's 8-bit KV for
                               sensitive layers, 2.2 / 5.1); KVQ_MODE_SYM_INT4 requires 4 or 8,
                               KVQ_MODE_ASYM_INT4 4 */
  int32_t outliers_per_vec; /* 0..8 fp16 outliers per quantization vector; 0 with KVARN */
  int32_t pre_rope;         /* 1: keys are stored before RoPE and rotated at decode; 0 with KVARN */
  float rope_theta;         /* RoPE base (10000 in the pages), > 0 when pre_rope */
  int32_t varn_iters;       /* KVARN: 0..64 Sinkhorn iterations (8 in the pages) */
  int32_t sink_tokens;      /* 0..KVQ_MAX_SINK: the first tokens of every sequence stay fp16
                               and form no block (KVQuant notes 3.5: attention sink) */
  int32_t fp16_window;      /* 0..KVQ_MAX_WINDOW, a multiple of 128: a block is quantized only
                               once this many newer tokens follow it (KVQuant notes 4.2:
                               KIVI's full-precision window of recent tokens) */
  int32_t paged_pages;      /* 0: each (layer, sequence, kv head) owns max_tokens / 128 block
                               records in place. > 0: a paged cache. Each layer keeps a pool of
                               this many pages, a page being one 128-token block of one sequence
                               (its n_kv_heads records), and a caller-owned block table maps the
                               blocks of every sequence to pages; sequences hold ragged lengths.
                               Requires batch <= KVQ_MAX_PAGED_BATCH, sink_tokens = fp16_window
                               = 0, and a pool of at most KVQ_MAX_POOL_BYTES per layer. */
} kvq_config;

typedef struct kvq_cache_s* kvq_cache;   /* opaque host handle; owns no device memory */

/* Bytes of device memory a cache with this configuration needs (pure host). */
kvq_status kvq_cache_bytes(const kvq_config* cfg, size_t* bytes);

/*
 * Create a handle over a caller-owned device buffer dev_buf of at least
 * kvq_cache_bytes(cfg) bytes, 256-byte aligned. Uploads the RoPE tables (when
 * pre_rope), sets every layer's length to 0 and synchronizes stream once.
 * The buffer holds, per layer and (sequence, kv head): 128-token block records
 * (layout below), a fp16 tail of up to 127 tokens, the codebooks, the RoPE
 * tables and a workspace for decode split partials.
 */
kvq_status kvq_cache_init(const kvq_config* cfg, void* dev_buf, size_t bytes, void* stream,
                          kvq_cache* out);

/* Free the host handle (not dev_buf). NULL is ignored. */
void kvq_cache_destroy(kvq_cache cache);

/*
 * Load the NUQ codebook of one (layer, kv head) for keys (which = 0) or values
 * (which = 1). host_codebook: n_entries = 2^bits fp32 values, finite, within
 * [-1, 1], ascending with consecutive entries at least 2^-21 apart (KVQuant notes
 * 3.3: one datatype per layer and head; the library keeps one per (layer, kv head,
 * K/V)). The gap guarantees that the fp32 argmin of |u - C_j| (ties to the smaller
 * j) is decided between the two entries around u; the library derives the decision
 * threshold between each pair of consecutive entries on the host and uploads it with
 * the entries. The handle keeps a host copy, so host_codebook may be freed on return.
 * Errors: KVQ_ERR_ARG for a codebook that breaks these rules; KVQ_ERR_STATE outside
 * KVQ_MODE_NUQ.
 */
kvq_status kvq_codebook_load(kvq_cache cache, int layer, int kv_head, int which,
                             const float* host_codebook, int n_entries, void* stream);

/*
 * Append n_new tokens to every sequence of one layer.
 * k_f16, v_f16: dev, fp16 [batch][n_kv_heads][n_new][128], contiguous; keys
 * before RoPE when pre_rope. Tokens take the next absolute positions.
 * Positions 0 .. sink_tokens-1 are sink tokens, kept in fp16. The later tokens
 * (body token u at position sink_tokens + u) form 128-token blocks; body block j
 * is quantized (KVQuant notes Algorithm 1; KVarN method steps; blog 4.2) as soon
 * as the body holds 128 (j + 1) + fp16_window tokens; until then its tokens stay
 * in fp16 (blog 5.2). With sink_tokens = fp16_window = 0 a block is quantized
 * when it is complete. n_new = 0 is a no-op.
 * Errors: KVQ_ERR_CAPACITY if length + n_new > max_tokens; KVQ_ERR_STATE in
 * NUQ mode unless both codebooks of every kv head of the layer are loaded.
 */
kvq_status kvq_quantize_append(kvq_cache cache, int layer, const void* k_f16, const void* v_f16,
                               int n_new, void* stream);

/*
 * Decode attention for one layer over every cached token (quantized blocks and
 * the fp16 tail), reading the packed cache directly: one split-K kernel and,
 * when the context is split, a small kernel that merges the split partials.
 * q_f16: dev, fp16 [batch][n_q_heads][128], already rotated for its own position.
 * out:   dev, fp32 [batch][n_q_heads][128].
 * Query head h reads kv head h / (n_q_heads / n_kv_heads). Scores are
 * softmax_scale * q . RoPE(k_n, n) (RoPE only when pre_rope; n is the 0-based
 * absolute position); softmax_scale <= 0 selects 1/sqrt(128)
 * (KVQuant notes Algorithm 1, attention part).
 * Errors: KVQ_ERR_STATE if the layer holds no tokens.
 *
 * Kernel selection (fixed by the configuration; results agree within the tolerance the
 * tests state, records are the same):
 *   - pre_rope = 1, one query head per kv head, 2 or 3 bits, RTN or NUQ: the table kernel
 *     (per-block LDS tables of the rotated query over the code pairs of each channel pair);
 *   - pre_rope = 0, no outliers, 2 or 4 bits, RTN, KVARN or SYM_INT4: the matrix-core
 *     kernel (products on v_mfma_f32_16x16x32_f16), unless kvq_set_matrix_cores(cache, 0);
 *   - every other configuration: the vector-unit kernel. It is correct for all of them but
 *     not tuned: with pre_rope = 1 and with 8 query heads per kv head its per-lane state
 *     exceeds the register file and part of it lives in scratch memory.
 * Caches with sink tokens or an fp16 window run one more kernel for the fp16 tokens.
 */
kvq_status kvq_decode_attn(kvq_cache cache, int layer, const void* q_f16, float* out,
                           float softmax_scale, void* stream);

/*
 * For callers that cannot allocate device memory or call allocating routines (code under
 * HIP graph capture, tight serving loops, harnesses that forbid it): kvq_decode_attn with
 * the split partials kept in a library-owned static device array of
 * KVQ_STATIC_SCRATCH_BYTES (8 MiB) instead of the cache buffer's workspace. Same
 * arguments, kernels and results as kvq_decode_attn (with sink tokens or an fp16 window, the
 * fp16 part may be cut into fewer chunks, one partial each, to fit the array: the results then
 * agree within the decode tolerance, not bit for bit); it calls no allocating routine.
 * Each GPU the library runs on holds its own copy of the array until the process ends
 * (looked up once per device, with that device current). Every call on one GPU shares
 * that copy, whatever the handle: calls that overlap on one GPU (different streams or
 * threads) race; serialize them. Every partial is written before it is read, so the
 * array's previous contents never matter.
 * Errors: those of kvq_decode_attn (KVQ_ERR_STATE for a paged cache, before any device
 * call), and KVQ_ERR_SIZE (nothing launched) when the call's
 * split partials, (splits + 1 if the cache keeps an fp16 part) x batch x n_q_heads x 520
 * bytes, exceed the array; lower the
 * split count with kvq_set_decode_splits. KVQ_ERR_HIP if the array's device address
 * cannot be obtained.
 */
kvq_status kvq_decode_attn_static(kvq_cache cache, int layer, const void* q_f16, float* out,
                                  float softmax_scale, void* stream);

/*
 * Quantization-error diagnostic (KVarN summary, core method: the error of a token vector
 * splits into a norm part and a direction part). For every token of quantized body blocks
 * block0 .. block0 + n_blocks - 1 of one layer (body block j holds positions
 * sink_tokens + 128 j ...), with x the original vector and x_hat its dequantized cache value
 * (original domain, keys before RoPE, outliers replaced by their fp16 values):
 *   E_M = (||x|| - ||x_hat||)^2,  E_D = 2 ||x|| ||x_hat|| (1 - cos angle(x, x_hat)),
 * so that E_M + E_D = ||x - x_hat||^2. Computed in fp64.
 * k_f16, v_f16: dev, fp16 [batch][n_kv_heads][n_blocks * 128][128], the original keys and
 *   values of those blocks, contiguous, 16-byte aligned.
 * out: dev, fp64 [batch][n_kv_heads][n_blocks * 128][4] = E_M(key), E_D(key), E_M(value),
 *   E_D(value).
 * Errors: KVQ_ERR_ARG unless every requested block is quantized.
 */
kvq_status kvq_error_decomposition(kvq_cache cache, int layer, int block0, int n_blocks, const void* k_f16,
                                   const void* v_f16, double* out, void* stream);

/*
 * NUQ codebook builder (KVQuant notes 3.3, Algorithm 2: sensitivity-weighted k-means on
 * activations normalised to [-1, 1]). 2^bits centres start evenly spaced over [-1, 1];
 * each iteration assigns every activation to its nearest centre (ties to the smaller
 * index) and moves each centre to the weighted mean of its members (a centre without
 * members stays); it stops when no assignment changes, after at most max_iters updates.
 * Sums and centres are fp64 with a fixed summation order (reproducible).
 * act:    dev, fp32 [n], the normalised activations (e.g. key channels or value tokens of
 *         calibration data mapped to [-1, 1] by (x - z) / h as the quantizer does).
 * weight: dev, fp32 [n], non-negative weights (Fisher information in the notes), or NULL
 *         for unit weights.
 * workspace: dev, 256-byte aligned, kvq_codebook_build_workspace(n, bits) bytes.
 * codebook: dev, fp32 [2^bits] out, ascending, ready for kvq_codebook_load (which checks
 *         its entry spacing). iters: dev int32 [1] out, the update steps taken, or NULL.
 * Asynchronous on stream (2 max_iters + 1 launches; after convergence they do nothing).
 * Errors: KVQ_ERR_ARG (n < 1, bits not 2..4, max_iters not 1..1000, NULL or misaligned
 * pointers), KVQ_ERR_SIZE (workspace too small).
 */
kvq_status kvq_codebook_build_workspace(int64_t n, int bits, size_t* bytes);
kvq_status kvq_codebook_build(const float* act, const float* weight, int64_t n, int bits, int max_iters,
                              void* workspace, size_t workspace_bytes, float* codebook, int32_t* iters,
                              void* stream);

/*
 * Paged caches (paged_pages > 0; KVQuant notes 7.2 (b-3) and 7.3 item 5: the packed cache
 * and its outliers in a paged memory pool for serving with requests of different lengths;
 * TurboQuant blog 4.1: the block allocator and index table of a paged KV cache).
 * Ragged batches: sequence b of the batch holds its own number of tokens n_b.
 * Records of a layer live in a pool of paged_pages pages; page p holds one block of
 * one sequence: the records of kv heads 0 .. n_kv_heads-1 back to back (kvq_page_span).
 * block_table: dev, int32 [batch][max_tokens / 128], caller-owned: entry [b][j] is the
 * page of block j of sequence b (positions 128 j .. 128 j + 127). The caller allocates
 * pages (distinct pages for distinct blocks) and writes the entries before the call
 * that first quantizes that block; entries of blocks not yet complete are not read.
 * An entry outside 0 .. paged_pages-1 is clamped into the pool: wrong results, never an
 * access outside the cache buffer. The at most 127 newest tokens of each sequence (its
 * incomplete last block) stay in fp16 in a fixed per-(sequence, kv head) tail, as in
 * unpaged caches (kvq_tail_span).
 */

/*
 * Append to the sequences of one layer of a paged cache, each its own number of tokens.
 * k_f16, v_f16: dev, fp16 [batch][n_kv_heads][max_new][128]; rows 0 .. n_new[b]-1 of
 *   sequence b are appended at its next positions (keys before RoPE when pre_rope).
 * n_new: host, int32 [batch], each in 0 .. max_new.
 * Every block that a sequence completes is quantized exactly as kvq_quantize_append does
 * and written to its page. One launch quantizes the blocks of all sequences.
 * Errors: KVQ_ERR_STATE for an unpaged cache (and in NUQ mode without loaded codebooks);
 * KVQ_ERR_CAPACITY if a sequence would exceed max_tokens (nothing appended);
 * KVQ_ERR_ARG for a bad n_new or NULL pointers.
 */
kvq_status kvq_quantize_append_paged(kvq_cache cache, int layer, const void* k_f16, const void* v_f16,
                                     const int32_t* n_new, int max_new, const int32_t* block_table,
                                     void* stream);

/*
 * Decode attention over one layer of a paged cache: sequence b attends to its own n_b
 * tokens (its blocks through block_table, then its fp16 tail). Arguments, scores and
 * output as for kvq_decode_attn; block_table as above.
 * Errors: KVQ_ERR_STATE for an unpaged cache or if a sequence of the layer holds no token.
 */
kvq_status kvq_decode_attn_paged(kvq_cache cache, int layer, const void* q_f16, float* out,
                                 float softmax_scale, const int32_t* block_table, void* stream);

/* Tokens held by sequence b of a layer (either kind of cache; host-side counter). */
kvq_status kvq_sequence_length(kvq_cache cache, int layer, int b, int32_t* n_tokens);

/* Forget the tokens of sequence b of a layer of a paged cache (its pages are the caller's to
 * reuse). KVQ_ERR_STATE for an unpaged cache, whose sequences keep equal lengths. */
kvq_status kvq_sequence_reset(kvq_cache cache, int layer, int b);

/* Byte range inside dev_buf of the record of kv_head in page `page` of a layer's pool
 * (layout as for kvq_block_span). KVQ_ERR_STATE for an unpaged cache. */
kvq_status kvq_page_span(kvq_cache cache, int layer, int page, int kv_head, size_t* offset, size_t* bytes);

/* Tokens currently held by a layer (host-side counter, no device access); in a paged
 * cache, the largest length over its sequences. */
kvq_status kvq_cache_length(kvq_cache cache, int layer, int32_t* n_tokens);

/* Forget the tokens of a layer, every sequence (length = 0; device memory is not touched). */
kvq_status kvq_cache_reset(kvq_cache cache, int layer);

/*
 * Number of decode splits per (sequence, kv head): 0 = automatic (default),
 * otherwise 1..KVQ_MAX_SPLITS (capped at decode time to the layer's number of
 * full 128-token blocks). Returns KVQ_ERR_ARG outside 0..KVQ_MAX_SPLITS.
 */
kvq_status kvq_set_decode_splits(kvq_cache cache, int splits);

/*
 * Whether decode may use the matrix cores: 1 (default) or 0. With 0 every product runs on the
 * vector unit: the table kernel's 2-bit RTN value product goes through its LDS table of code
 * pairs, and caches the matrix-core kernel would take go to the vector-unit kernel. Results
 * agree within the decode tolerance either way (summation orders differ); the switch exists
 * to measure what the matrix cores contribute ("KVQuant reading notes" 3.7 and 3.8 run both
 * products as vector kernels). Returns KVQ_ERR_ARG for another value.
 */
kvq_status kvq_set_matrix_cores(kvq_cache cache, int enable);

/*
 * Byte range of one block record inside dev_buf. The record of block j of
 * (layer, sequence b, kv head h) holds, each segment starting on a 16-byte
 * boundary, the record padded to 256 bytes (T = 128 tokens, D = 128 channels,
 * R = 16*bits bytes per 128 codes):
 *   kc  key codes, token-major: 128 rows of R bytes, row t = channels 0..127
 *   vc  value codes, channel-major in two token halves: [2][128][R/2],
 *       row (half, c) holds the 64 tokens 64*half + u of channel c with the 4x4
 *       grid of 4-token groups transposed: position p holds
 *       u = 16*((p>>2)&3) + 4*(p>>4) + (p&3) (storage order only)
 *   ks  key statistics per channel: RTN/KVARN f32 s[128] then f32 m[128];
 *       NUQ f32 z[128] then f32 h[128]; SYM_INT4 f16 s[128]; ASYM_INT4 f16 s[128]
 *       then f16 zero[128]
 *   vs  value statistics: per token (RTN/KVARN s then m, NUQ z then h, f32);
 *       SYM_INT4 / ASYM_INT4 per channel, as for the keys
 *   k1  KVARN only: f32 s1[128] per token;  v1: KVARN only: f32 s1[128] per channel
 *   outliers (outliers_per_vec = k > 0):
 *       key CSR by token:     f16 val[128k], u16 row_ptr[129], u8 channel[128k]
 *       value CSC by channel: f16 val[128k], u16 col_ptr[129], u8 token[128k]
 *       entries sorted by (row, column); val holds the original fp16 bits, and
 *       the dense code at an outlier position is 0.
 * Code packing of n codes: 4-bit byte j = code 2j | code 2j+1 << 4; 2-bit byte j
 * = codes 4j..4j+3 at bits 2i; 3-bit = the low 2 bits of all n codes packed as
 * 2-bit (n/4 bytes) then bit 2 of code 8j+i at bit i of byte j (n/8 bytes).
 * 8-bit: byte j = code j.
 * Codes: RTN/KVARN q in 0..2^b-1 with x = q*s + m (KVARN: times s1);
 * NUQ q indexes the codebook, x = C[q]*h + z; SYM_INT4 u = q + 2^(b-1), x = (u - 2^(b-1))*s
 * (4 bits: u = q + 8, s = fp16(absmax / 7); 8 bits: u = q + 128, s = fp16(absmax / 127));
 * ASYM_INT4 u = q + 8, x = (u - 8)*s + zero with s = fp16((max - min) / 15) and
 * zero = fp16(min + 8 s) over the vector (keys and values per channel over the block).
 */
kvq_status kvq_block_span(kvq_cache cache, int layer, int b, int kv_head, int block,
                          size_t* offset, size_t* bytes);

/*
 * Byte range of the fp16 rows of (layer, b, kv head): K [R][128] then V [R][128] with
 * R = sink_tokens + fp16_window + 128. Row p < sink_tokens holds sink token p; row
 * sink_tokens + (u mod (fp16_window + 128)) holds body token u while it is not quantized.
 */
kvq_status kvq_tail_span(kvq_cache cache, int layer, int b, int kv_head, size_t* offset,
                         size_t* bytes);

/*
 * Algorithmic bytes a decode call on this layer must move now: block records
 * without padding, the fp16 tail rows, q, out, codebooks and the RoPE base rows
 * of the blocks it reads.
 */
kvq_status kvq_decode_bytes(kvq_cache cache, int layer, size_t* bytes);

/* Static text for a status code. */
const char* kvq_strerror(kvq_status status);

/* Description of the calling thread's last failure ("" if none). */
const char* kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
