// Kernel argument blocks and launchers shared by the kernels and the C ABI.
#pragma once

#include "common.hpp"

namespace packkv {

enum EncMode : int { kPass1 = 0, kPass2 = 1, kTail = 2 };

// Page allocator state of a paged cache, in one device array of u32:
//   [0] free pages, [1] 0, [2 + 4s] stream s's current K page (kNoPage:
//   none), [3 + 4s] its fill in 16-byte units, [4 + 4s], [5 + 4s] the same
//   for V, then the stack of free page indices.
// A stream's K records of closed blocks are placed one after another, in
// block order, in its current K page (V records in its V page), so each
// wave of the attention kernel still reads one sequential run per page; a
// record that does not fit takes a new page from the stack, so no record
// straddles two pages.  The open block's K and V records live in two fixed
// tail slots per stream past the pages.
constexpr uint32_t kNoPage = 0xFFFFFFFFu;
struct PageAlloc {
  uint32_t* state;
  int32_t n_streams;
  uint32_t n_pages;
  uint32_t page16;          // page size in 16-byte units
  uint32_t tail16;          // start of the tail slots in 16-byte units
  uint32_t slot16;          // one tail slot in 16-byte units
};

struct EncArgs {
  const uint16_t* k;        // raw fp16 source of token 0 of stream 0
  const uint16_t* v;
  int64_t src_stream;       // elements between streams in the source
  int64_t src_block;        // elements between blocks in the source
  int64_t n_tokens;         // total tokens per stream after this call
  int32_t bits, B, D, permute, mode;
  int32_t korder;           // payload order of the K records (0 by channel, 1 width-sorted)
  int32_t block0;           // kTail: index of the block being (re)encoded
  // kTail: tokens appended by this call, [S][new_cnt][D] fp16 (new_stream
  // elements apart), at positions new_at.. of the open block; they are read
  // from here and copied into the raw tail staging (k, v) as they are read.
  // Null: every token comes from the staging.
  const uint16_t* new_k;
  const uint16_t* new_v;
  int64_t new_stream;
  int32_t new_at;
  uint8_t* k_arena;
  uint8_t* v_arena;
  uint64_t arena_limit;     // usable bytes per stream region
  uint64_t arena_stride;
  uint32_t* k_off;
  uint32_t* v_off;
  int64_t off_stride;       // max_blocks + 1
  uint8_t* perm;
  int64_t perm_stride;      // max_blocks * B
  int32_t* status;
  // Paged cache (k_arena = v_arena = the pool, paged != 0): record j of
  // stream s starts 16 * k_tab[s * off_stride + j].x bytes into the pool and
  // is .y bytes long; the stream's length is lengths[s] (kTail appends one
  // token per stream and reads its position from there).  Streams of the
  // launch are stream0 + blockIdx.y.
  int32_t paged;
  int32_t stream0;
  uint2* k_tab;
  uint2* v_tab;
  int32_t* lengths;
  PageAlloc pages;
};

struct GemvArgs {
  const uint8_t* arena;
  uint64_t arena_stride;
  const uint32_t* off;
  int64_t off_stride;
  int64_t n_tokens;
  int32_t nb;            // records per stream = ceil(T / B)
  int32_t bits;
  int32_t D;             // head_dim: 64, 128 or 256
  int32_t blocks_per_wg;
  int32_t splits;        // workgroups per stream
  int32_t G;
  int32_t korder;        // payload order of K records (0 by channel, 1 width-sorted); 0 for V
  const uint16_t* q;     // K: q [S][G][D] fp16
  const float* p;        // V: p [S][G][ld] fp32
  float* scores;         // K: [S][G][ld]
  int64_t ld;
  float* ws;             // V: partial sums [S][G][splits][D]
  uint32_t* tickets;     // V: per-stream arrival counters, zero between calls
  float* out;            // V: [S][G][D]
  int32_t* status;
};


// Fused decode attention over both packed caches of a cache object.
// Fused attention over up to kAttnMaxCaches caches of one shape (the layers
// of a model) in one launch: blockIdx.y picks the cache.
constexpr int kAttnMaxCaches = 32;
struct AttnCache {
  const uint8_t* k_arena;   // paged: the pool
  const uint8_t* v_arena;
  const uint32_t* k_off;
  const uint32_t* v_off;
  int32_t* status;
  const uint2* k_tab;       // paged: block tables [S][off_stride] and lengths [S]
  const uint2* v_tab;
  const int32_t* lengths;
};
struct AttnArgs {
  AttnCache cache[kAttnMaxCaches];
  uint64_t arena_stride;    // paged: the pool's size in bytes
  int64_t off_stride;       // paged: block-table entries per stream
  int64_t n_tokens;         // paged: unused (lengths[s] per stream)
  int32_t nb;
  int32_t bits;
  int32_t D;                // head_dim: 64, 128 or 256 (the paged cache: 128)
  int32_t blocks_per_wg;
  int32_t splits;
  int32_t G;
  int32_t korder;        // payload order of the K records (0 by channel, 1 width-sorted)
  float scale_log2e;     // softmax scale times log2(e)
  const uint16_t* q;     // [caches][S][G][D] fp16
  float* out;            // [caches][S][G][D]
  int64_t qo_stride;     // elements per cache in q and out: S * G * D
  uint8_t* ws;           // per cache ws_stride bytes of partials [S][G][splits][D + 4]
  uint64_t ws_stride;
  uint8_t* tk;           // per cache tk_stride bytes: per-stream arrival counters
  uint64_t tk_stride;    //   (u32 [S], zero between calls)
};

hipError_t launch_encode(const EncArgs& a, int n_streams, int n_blocks, hipStream_t st);
hipError_t launch_scan_offsets(uint32_t* k_off, uint32_t* v_off, int64_t off_stride,
                               int n_streams, int nb, hipStream_t st);
hipError_t launch_stage_tail(const uint16_t* k, const uint16_t* v, int64_t src_stream,
                             uint16_t* tk, uint16_t* tv, int B, int D, int at, int cnt,
                             int n_streams, hipStream_t st);
hipError_t launch_qk(const GemvArgs& a, int B, int n_streams, hipStream_t st);
hipError_t launch_pv(const GemvArgs& a, int B, int n_streams, hipStream_t st);
hipError_t launch_attention(const AttnArgs& a, int B, int n_streams, int n_caches, hipStream_t st,
                            bool paged = false);
int attention_resident_wgs(int B, int bits, int G, int D);
hipError_t launch_paged_alloc(const EncArgs& a, int n_streams, int64_t n_tokens, hipStream_t st);
hipError_t launch_paged_init(const PageAlloc& p, int32_t* lengths, int32_t* status, hipStream_t st);
hipError_t launch_paged_release(const PageAlloc& p, const uint2* k_tab, const uint2* v_tab,
                                int64_t tab_stride, int32_t* lengths, int B, int stream, hipStream_t st);
hipError_t launch_decompress(const GemvArgs& a, int B, bool is_v, int n_streams, const uint8_t* perm,
                             int64_t perm_stride, int mode, void* out, hipStream_t st);
hipError_t launch_stats(const GemvArgs& a, int B, bool is_v, int n_streams, unsigned long long* out,
                        hipStream_t st);
hipError_t launch_softmax(const float* scores, float* p, int rows, int64_t T, int64_t ld, float scale,
                          hipStream_t st);
hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t st);

}  // namespace packkv
