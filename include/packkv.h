/*
 * packkv.h - C ABI of the MI355X (gfx950) PackKV decode library.
 *
 * PackKV ("PackKV: Reducing KV Cache Memory Footprint through LLM-Aware Lossy
 * Compression", arXiv 2512.24449) keeps the attention KV cache quantised,
 * token-reordered and bit-packed, and fuses decompression into the two
 * decode-time matrix-vector products (abstract; TL;DR; Fig. 1 and Fig. 2
 * captions):
 *
 *   K side:  scores[t] = q . K_hat[t]
 *   V side:  out       = sum_t p[t] * V_hat[t]
 *
 * Packed format (one record per block of B tokens of one stream; integers
 * little-endian):
 *   K record: scale[D] fp16 | zero[D] fp16 | hdr[nr][D] | 0-pad to 16 B |
 *             payload | 0-pad to 16 B
 *   V record: scale[B] fp16 | zero[B] fp16 (slot order, 0 past n) |
 *             hdr[nr][D] | 0-pad to 16 B | payload | 0-pad to 16 B
 *   nr = ceil(n / R) runs of R = 32 slots; hdr = the byte (w << 4) | m for
 *   b <= 4, the little-endian u16 (w << 8) | m for b = 5..8, for the run's
 *   width w = bit_length(max - min) and minimum m; payload = for each run r,
 *   for each channel c (payload_order 0; in order 1 a K record takes the
 *   channels of each run by decreasing w, equal w by channel), w u32 words
 *   holding u = q - m of its 32 slots in the sliced order: with c-bit containers (c = 4 for b <= 4, 8 above), slot i
 *   is field j = i % (32/c) of container k = i / (32/c), and bit p of its u
 *   is bit c*j + Q of run word W, where W = k / g, Q = w*(k % g) + p if w
 *   divides c (g = c/w), else W = k, Q = p for k < w and W = p, Q = k for
 *   k >= w.  Quantisation: K per channel over the block's tokens, V
 *   per token over D channels; zero = group minimum, scale = the smallest
 *   fp16 h with h * (2^b - 1) >= max - min, q = round-half-even((x-min)/h).
 *   Slot i of block j holds token j*B + perm[j][i]; the permutation is the
 *   greedy L1 grouping of the block's quantised (K, V) rows (identity when it
 *   does not shrink the payload).
 *
 * Conventions for every entry point
 *   - Every pointer inside packkv_cache_t and every tensor argument is DEVICE
 *     memory owned by the caller (e.g. allocated with torch on ROCm).  The
 *     library never allocates or frees device memory, and all state of a
 *     cache lives in the caller's buffers; calls on different caches are
 *     independent.  The only process-wide state is a table of per-shape
 *     occupancy figures (resident workgroups per device), asked from the
 *     runtime once per kernel shape and read-only after that, and the
 *     scratch array of packkv_attention_decode_noalloc (one per GPU).
 *   - `stream` is a hipStream_t passed as void*.  Every call only enqueues
 *     work on that stream and returns without synchronising, except
 *     packkv_check, which synchronises the stream.
 *   - Host-detectable precondition failures (null pointer, unsupported
 *     configuration, size over capacity, bad stride) return a nonzero
 *     status BEFORE anything is launched; a failed launch returns
 *     PACKKV_EHIP.  Conditions only the device can see (arena overflow, a
 *     corrupt header) set *cache->status, skip the affected writes, and are
 *     reported by packkv_check.
 *   - Inputs are never modified.  Outputs are written over [0, n_tokens);
 *     entries of a leading dimension past that are left untouched.
 *   - scores, p and the decompressed ints are in SLOT order (attention does
 *     not depend on the order of bound (K, V) pairs, TL;DR); perm maps slots
 *     back to tokens.
 */
#ifndef PACKKV_H_
#define PACKKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  PACKKV_OK = 0,
  PACKKV_EINVAL = 1,       /* bad argument (null pointer, size, stride), or, as
                              a device latch, an input value outside the
                              method's domain (non-finite K/V, a V-GEMV weight
                              that is negative or non-finite)                 */
  PACKKV_EUNSUPPORTED = 2, /* configuration outside D 64/128/256, b 2..8, B 64/128, R 32,
                              or payload order 1 above 4 bits                 */
  PACKKV_ECAPACITY = 3,    /* tokens over max_tokens, or arena region overflow */
  PACKKV_ECORRUPT = 4,     /* a record header is inconsistent                  */
  PACKKV_EHIP = 5,         /* a HIP runtime call or kernel launch failed       */
  PACKKV_ESTATE = 6        /* call not valid in the cache's current state      */
};

/* Format parameters. */
typedef struct {
  int32_t head_dim;     /* D: 64, 128 or 256 (Fig. 5 caption: quantisation  */
                        /* groups along the channel axis; the paged cache  */
                        /* takes 128 only)                                  */
  int32_t bits;         /* b: 2 .. 8 (5..8: two-byte header entries)         */
  int32_t block_tokens; /* B: 64 or 128                                      */
  int32_t run_tokens;   /* R: must be 32                                     */
  int32_t permute;      /* token order inside blocks (Fig. 2 caption, step   */
                        /* (1)): 0 identity, 1 greedy L1 grouping, 2 sorted  */
                        /* by the total of the token's K and V ints; modes   */
                        /* 1 and 2 fall back to the identity unless the      */
                        /* block's payload shrinks.  Other values: EINVAL    */
  int32_t payload_order; /* order of a K record's payload entries (explainer */
                        /* page, "Block matrix before and after repacking": */
                        /* a layout that suits the consuming GPU): 0 run-   */
                        /* major then channel; 1 each run row by decreasing */
                        /* width, equal widths by channel, so that the      */
                        /* entries a wave decodes together share a width.   */
                        /* Headers and V records keep order 0; record sizes */
                        /* do not change.  1 needs b <= 4 (EUNSUPPORTED     */
                        /* otherwise); other values: EINVAL                 */
} packkv_config_t;

/*
 * A packed cache of S independent streams (stream = batch entry x KV head),
 * all holding the same number of tokens.  The caller fills every field and
 * allocates every array with the sizes packkv_cache_sizes() reports, zeroed
 * where noted.  n_tokens is maintained by the library's host code: the
 * compress and append calls update it when they return PACKKV_OK.
 */
typedef struct {
  packkv_config_t cfg;
  int32_t n_streams;      /* S >= 1                                           */
  int64_t max_tokens;     /* capacity per stream                              */
  int64_t n_tokens;       /* tokens currently held per stream (start at 0)    */
  uint64_t arena_stride;  /* bytes per stream region of each arena (multiple of
                             256, >= packkv_arena_stride_bytes, < 2^32)       */
  uint8_t* k_arena;       /* [S][arena_stride] K records, back to back        */
  uint8_t* v_arena;       /* [S][arena_stride] V records                      */
  uint32_t* k_off;        /* [S][max_blocks + 1] byte offset of each record
                             within its stream region; entry nb = used bytes  */
  uint32_t* v_off;        /* [S][max_blocks + 1]                              */
  uint8_t* perm;          /* [S][max_blocks][B] slot -> in-block token index,
                             0xFF for empty slots                             */
  uint16_t* tail_k;       /* [S][B][D] fp16 raw tokens of the open tail block */
  uint16_t* tail_v;       /* [S][B][D]                                        */
  int32_t* status;        /* [1] device error latch, zero-initialised         */
} packkv_cache_t;

/* Sizes (in bytes) of every array of a cache. */
typedef struct {
  uint64_t arena_stride;  /* per stream, worst case (every run at w = b)      */
  uint64_t arena_bytes;   /* S * arena_stride, for each of k_arena, v_arena   */
  uint64_t off_bytes;     /* S * (max_blocks + 1) * 4, for each of k_off, v_off */
  uint64_t perm_bytes;    /* S * max_blocks * B                               */
  uint64_t tail_bytes;    /* S * B * D * 2, for each of tail_k, tail_v        */
  int64_t max_blocks;     /* ceil(max_tokens / B)                             */
} packkv_sizes_t;

/* Validate cfg and report the sizes of a cache for S streams of up to
 * max_tokens tokens.  Host only.  Returns PACKKV_OK, EINVAL or EUNSUPPORTED. */
int packkv_cache_sizes(const packkv_config_t* cfg, int32_t n_streams,
                       int64_t max_tokens, packkv_sizes_t* out);

/* Worst-case bytes of one stream's arena region (every run at full width b,
 * plus slack for the kernels' vector over-reads), rounded up to 256 B.  0 on
 * an invalid cfg. */
uint64_t packkv_arena_stride_bytes(const packkv_config_t* cfg, int64_t max_tokens);

/* Bytes of workspace packkv_pv_gemv needs for `group` queries per stream:
 * fp32 split partial sums, then one 32-bit counter per stream. */
uint64_t packkv_pv_workspace_bytes(const packkv_cache_t* cache, int32_t group);

/*
 * packkv_compress_block - encode n_tokens tokens of every stream at once
 * (prefill).  Abstract: PackKV compresses the KV cache; Fig. 2 caption and
 * TL;DR: quantise, reorder, then bit-pack losslessly in channel direction.
 *   k_f16, v_f16: device fp16 [S][n_tokens][D], token order, contiguous,
 *                 16-byte aligned (else PACKKV_EINVAL).
 * The cache must be empty (n_tokens == 0, else PACKKV_ESTATE) and
 * 1 <= n_tokens <= max_tokens (else EINVAL / ECAPACITY).  Writes every
 * record, k_off/v_off[0 .. nb], perm, and the raw tail staging (the last,
 * partial block's tokens).  Sets cache->n_tokens on success.  An infinite
 * or NaN input value latches PACKKV_EINVAL in *status (the method quantises
 * finite values only); the records stay well-formed, with unspecified
 * contents for the blocks holding such values.
 */
int packkv_compress_block(packkv_cache_t* cache, const void* k_f16, const void* v_f16,
                          int64_t n_tokens, void* stream);

/*
 * packkv_append_tokens - append n_new tokens to every stream (decode).
 * Abstract: the method stays compatible with the dynamically growing cache.
 * The open tail block is kept as raw fp16 and re-encoded in full on every
 * call; closed blocks never change, so appending gives exactly the bytes a
 * one-shot compress of all tokens gives.
 *   k_f16, v_f16: device fp16 [S][n_new][D], contiguous, 16-byte aligned
 *                 (else PACKKV_EINVAL).
 * n_new >= 1 and n_tokens + n_new <= max_tokens (else EINVAL / ECAPACITY).
 * Updates cache->n_tokens on success.  Non-finite values latch EINVAL as in
 * packkv_compress_block.
 */
int packkv_append_tokens(packkv_cache_t* cache, const void* k_f16, const void* v_f16,
                         int32_t n_new, void* stream);

/*
 * packkv_qk_gemv - fused K decompress + GEMV (TL;DR: decompression integrated
 * into the matrix-vector product, no writeback of decompressed data).
 *   q_f16:  device fp16 [S][group][D].
 *   scores: device fp32 [S][group][ld]; scores[s][g][j*B + i] =
 *           q[s][g] . K_hat[s][block j, slot i] for every j*B + i < n_tokens.
 * group >= 1, ld >= n_tokens, n_tokens >= 1, else EINVAL / ESTATE.
 */
int packkv_qk_gemv(const packkv_cache_t* cache, const void* q_f16, int32_t group,
                   float* scores, int64_t ld, void* stream);

/*
 * packkv_pv_gemv - fused V decompress + GEMV with a split-T partial-sum
 * reduction in a fixed order (Fig. 1 caption: weighted V vectors summed).
 *   p:         device fp32 [S][group][ld], slot order (as scores); every
 *              weight >= 0 and finite (softmax weights: the V block code
 *              turns them into fixed point relative to each block's largest
 *              weight).  A block holding any other weight contributes
 *              nothing and latches PACKKV_EINVAL in *status.
 *   out:       device fp32 [S][group][D]; out[s][g][c] =
 *              sum_t p[s][g][t] * V_hat[s][t][c].
 *   workspace: device memory of at least packkv_pv_workspace_bytes(cache,
 *              group) bytes (ws_bytes), caller-owned.  It holds the split
 *              partial sums and, at its end, one counter per stream that
 *              the last-arriving workgroup of each stream uses to find that
 *              it should do the final sum.  The counters must be zero when
 *              a workspace is first used (allocate it zero-filled); every
 *              call leaves them zero again.  Calls that share a workspace
 *              must not run concurrently.
 * The partial sums are added in split order, so results are bitwise
 * reproducible run to run.  Single kernel launch.
 */
int packkv_pv_gemv(const packkv_cache_t* cache, const float* p, int64_t ld, int32_t group,
                   float* out, void* workspace, uint64_t ws_bytes, void* stream);

/*
 * packkv_attention_decode - decode attention in one pass over both packed
 * caches: out[s][g] = sum_t softmax_t(scale * q[s][g] . K_hat[s][t]) *
 * V_hat[s][t] over the stream's n_tokens slots (Fig. 1 caption: scores,
 * softmax, weighted sum of V; TL;DR: decompression fused into the products so
 * that nothing decompressed is written back).  It is the K GEMV, the softmax
 * and the V GEMV fused: no scores or weights reach memory.
 *   q_f16:     device fp16 [S][group][D].
 *   scale:     softmax scale (e.g. 1/sqrt(D)), finite and > 0.
 *   out:       device fp32 [S][group][D].
 *   workspace: device memory of at least
 *              packkv_attention_workspace_bytes(cache, group) bytes
 *              (ws_bytes), caller-owned: per split partial sums with their
 *              running max and weight sum, then one counter per stream,
 *              which must be zero when a workspace is first used (allocate
 *              it zero-filled); every call leaves them zero.  Calls that
 *              share a workspace must not run concurrently.
 * The splits are merged in a fixed order, so results are bitwise
 * reproducible.  Single kernel launch.  Errors as for the GEMVs.
 */
int packkv_attention_decode(const packkv_cache_t* cache, const void* q_f16, int32_t group, float scale,
                            float* out, void* workspace, uint64_t ws_bytes, void* stream);

/* Bytes of workspace packkv_attention_decode needs for `group` queries. */
uint64_t packkv_attention_workspace_bytes(const packkv_cache_t* cache, int32_t group);

/*
 * packkv_attention_decode_multi - packkv_attention_decode for n_caches
 * caches of one shape (typically the layers of a model at one decode step),
 * in one kernel launch per 32 caches instead of one per cache.  Same
 * arithmetic as n_caches separate calls, with the same results bit for bit.
 *   caches:    host array of n_caches >= 1 caches with equal cfg.bits,
 *              cfg.block_tokens, n_streams, max_tokens, n_tokens and
 *              arena_stride (else PACKKV_EINVAL).
 *   q_f16:     device fp16 [n_caches][S][group][D].
 *   out:       device fp32 [n_caches][S][group][D].
 *   workspace: at least packkv_attention_multi_workspace_bytes(caches[0],
 *              group, n_caches) bytes: one packkv_attention_decode
 *              workspace per cache, back to back, with the same rules
 *              (counters zero before first use, left zero, no concurrent
 *              calls on one workspace).
 */
int packkv_attention_decode_multi(const packkv_cache_t* const* caches, int32_t n_caches, const void* q_f16,
                                  int32_t group, float scale, float* out, void* workspace, uint64_t ws_bytes,
                                  void* stream);

/*
 * packkv_attention_decode_noalloc - packkv_attention_decode without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same kernels, same work division and the same results bit
 * for bit.  It allocates nothing: the split partials and the per-stream
 * arrival counters live in a file-scope device array of the library, 16 MiB
 * per GPU, held from the library's load until the process ends.  Limits:
 * at most 16384 streams and at most 16 MiB - 64 KiB of partials
 * (n_streams * group * splits * 528 bytes; a few MiB at the shapes measured
 * here), else PACKKV_ECAPACITY before any launch.  Each call first clears
 * the counters of its streams with a small kernel on `stream`.  Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (different
 * streams, or host threads) race and must not be issued.
 */
int packkv_attention_decode_noalloc(const packkv_cache_t* cache, const void* q_f16, int32_t group, float scale,
                                    float* out, void* stream);

/* Bytes of workspace packkv_attention_decode_multi needs (0 if n_caches < 1). */
uint64_t packkv_attention_multi_workspace_bytes(const packkv_cache_t* cache, int32_t group, int32_t n_caches);

/*
 * packkv_decompress - decode the cache.  Not a step of the method (the
 * pages fuse decompression into the products so that nothing decompressed
 * is written, TL;DR); a test and debug path that writes the quantised ints
 * or the dequantised values out so they can be compared bit for bit.
 *   which: 0 = K, 1 = V.
 *   mode 0: out is uint8 [S][n_tokens][D], the quantised ints q in SLOT order.
 *   mode 1: out is fp32 [S][n_tokens][D], x_hat = zero + scale * q rounded
 *           once to fp32, in TOKEN order (through perm).
 */
int packkv_decompress(const packkv_cache_t* cache, int32_t which, int32_t mode,
                      void* out, void* stream);

/*
 * packkv_softmax_rows - p = exp(s*scale - max) / sum over the first T entries
 * of each of `rows` rows (row stride ld); the step between the two GEMVs
 * (Fig. 1 caption).  scores and p may be the same buffer.
 */
int packkv_softmax_rows(const float* scores, float* p, int32_t rows, int64_t T,
                        int64_t ld, float scale, void* stream);

/* Synchronise `stream`, then return and clear the device error latch
 * (PACKKV_OK if no kernel reported a problem). */
int packkv_check(const packkv_cache_t* cache, void* stream);

/*
 * packkv_stream_read - a measurement helper, not a step of the method: reads
 * every 16-byte chunk of the device buffer buf[0 .. bytes) once (grid-stride
 * over up to 4096 workgroups of 1024 threads) and stores the XOR of the
 * 32-bit words workgroup w read to the device
 * word sink[w] (sink holds 4096 words; the words of workgroups the launch
 * does not use are left untouched, so the XOR of a zero-filled sink is the
 * XOR of the whole buffer).  Timed over as many bytes as a decode launch
 * reads, it is the streaming-read ceiling of the device that the kernels'
 * bandwidth is compared with.  EINVAL if buf or sink is null, buf is not
 * 16-byte aligned, or bytes is not a positive multiple of 16.
 */
int packkv_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, void* stream);

/*
 * packkv_stats - width histogram and byte counts of the cache, into device
 * memory out[32] (uint64): out[0..4] K runs with w = 0..4, out[5..9] the
 * same for V, out[10] K record bytes, out[11] V record bytes, out[12] K
 * payload words, out[13] V payload words, out[14] K runs, out[15] V runs,
 * out[16..19] K runs with w = 5..8, out[20..23] the same for V (zero for
 * b <= 4).  out must be zeroed by the caller.
 */
int packkv_stats(const packkv_cache_t* cache, uint64_t* out, void* stream);

/* Static text for a status code. */
const char* packkv_status_str(int status);

/* ------------------------------------------------------------------------
 * Paged cache.  The pages list PagedAttention among the prior work and name
 * paging as a running cost of custom packed formats; this is the form of it
 * for variable-size records.  The records of every stream share one pool of
 * fixed-size pages and are found through per-stream block tables, and each
 * stream holds its own number of tokens.
 *
 *   - A stream's closed blocks are placed in block order, the K records one
 *     after another in its current K page and the V records in its current V
 *     page.  A record that does not fit takes a new page from a free-page
 *     stack on the device, so no record straddles two pages and a page
 *     belongs to one stream and one of K, V.
 *   - The open (partial) block's K and V records live in two fixed tail
 *     slots of the stream, past the pages, and are re-encoded there by every
 *     append; the append that fills the block writes it into the pages.
 *   - Releasing a stream returns its pages to the stack.
 *   - Every record is byte-identical to the one packkv_cache_t holds for the
 *     same tokens; only where it lives differs.
 *
 * Same conventions as packkv_cache_t (caller-owned device memory, one HIP
 * stream per call, host checks before any launch, device-only failures
 * latched in *status).  Device-side failures: no free page left
 * (PACKKV_ECAPACITY; the pool is then in an undefined state and must be set
 * up again with packkv_paged_init) and inconsistent table entries
 * (PACKKV_ECORRUPT).
 */
typedef struct {
  packkv_config_t cfg;
  int32_t n_streams;      /* S >= 1                                           */
  int32_t n_pages;        /* pages in the pool, >= 1                          */
  int64_t max_tokens;     /* capacity of each stream (sizes the block tables) */
  uint64_t page_bytes;    /* multiple of 256 and >= min_page_bytes            */
  uint8_t* pool;          /* [pool_bytes]: n_pages pages, then the tail slots */
  uint64_t* k_table;      /* [S][max_blocks]: bits 0-31 the record's start in
                             16-byte units of the pool, bits 32-63 its size
                             in bytes; valid for blocks < ceil(length / B)    */
  uint64_t* v_table;      /* [S][max_blocks]                                  */
  int32_t* lengths;       /* [S] tokens held by each stream                   */
  uint32_t* alloc;        /* [alloc_bytes / 4] allocator state: [0] free pages,
                             [1] 0, [2 + 4s] stream s's current K page
                             (0xFFFFFFFF: none) and [3 + 4s] its fill in
                             16-byte units, [4 + 4s], [5 + 4s] the same for
                             V, then the stack of free pages                  */
  uint8_t* perm;          /* [S][max_blocks][B], as in packkv_cache_t         */
  uint16_t* tail_k;       /* [S][B][D] fp16 raw tokens of each open block     */
  uint16_t* tail_v;       /* [S][B][D]                                        */
  int32_t* status;        /* [1] device error latch                           */
  int32_t* host_lengths;  /* HOST memory [S]: the library keeps it equal to
                             `lengths` (it sizes launches from it)            */
} packkv_paged_t;

typedef struct {
  uint64_t pool_bytes;     /* n_pages * page_bytes + S * 2 * slot_bytes       */
  uint64_t table_bytes;    /* S * max_blocks * 8, for each of k_table, v_table */
  uint64_t alloc_bytes;    /* (2 + 4 * S + n_pages) * 4                       */
  uint64_t lengths_bytes;  /* S * 4                                           */
  uint64_t perm_bytes;     /* S * max_blocks * B                              */
  uint64_t tail_bytes;     /* S * B * D * 2, for each of tail_k, tail_v       */
  uint64_t slot_bytes;     /* one tail slot: the largest K or V record        */
  uint64_t min_page_bytes; /* slot_bytes rounded up to 256                    */
  int64_t max_blocks;      /* ceil(max_tokens / B)                            */
} packkv_paged_sizes_t;

/* Validate and report the sizes of a paged cache.  Host only.  EINVAL when
 * page_bytes is not a multiple of 256 or below min_page_bytes, n_pages < 1,
 * or the pool would not be addressable in 16-byte units by 32 bits. */
int packkv_paged_sizes(const packkv_config_t* cfg, int32_t n_streams, int64_t max_tokens, int32_t n_pages,
                       uint64_t page_bytes, packkv_paged_sizes_t* out);

/* Every page free, every stream empty, the status clear (device and host). */
int packkv_paged_init(packkv_paged_t* cache, void* stream);

/*
 * packkv_paged_prefill - packkv_compress_block for streams stream0 ..
 * stream0 + n - 1, which must be empty (else ESTATE).  k_f16, v_f16: device
 * fp16 [n][n_tokens][D], contiguous, 16-byte aligned; 1 <= n_tokens <=
 * max_tokens.  Pages are taken as the records are placed; without enough
 * free pages the streams stay empty and ECAPACITY is latched.
 */
int packkv_paged_prefill(packkv_paged_t* cache, int32_t stream0, int32_t n, const void* k_f16,
                         const void* v_f16, int64_t n_tokens, void* stream);

/*
 * packkv_paged_append - one decode step: token k_f16[s], v_f16[s] (device
 * fp16 [S][1][D]) is appended to every stream s at its own position, with
 * the open-block re-encode of packkv_append_tokens.  ECAPACITY (before any
 * launch) if a stream is full.
 */
int packkv_paged_append(packkv_paged_t* cache, const void* k_f16, const void* v_f16, void* stream);

/* Stream s back to empty; its pages return to the free stack. */
int packkv_paged_release(packkv_paged_t* cache, int32_t s, void* stream);

/* Workspace of packkv_paged_attention for `group` queries per stream. */
uint64_t packkv_paged_attention_workspace_bytes(const packkv_paged_t* cache, int32_t group);

/*
 * packkv_paged_attention - packkv_attention_decode over the paged cache,
 * each stream over its own length; an empty stream's output is zero.  ESTATE
 * if every stream is empty.
 */
int packkv_paged_attention(const packkv_paged_t* cache, const void* q_f16, int32_t group, float scale,
                           float* out, void* workspace, uint64_t ws_bytes, void* stream);

/* packkv_check for a paged cache. */
int packkv_paged_check(const packkv_paged_t* cache, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PACKKV_H_ */
