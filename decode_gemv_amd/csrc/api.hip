// C ABI of the packkv library: argument validation, work decomposition and
// kernel launches on the caller's stream.  No device memory is allocated
// here; every buffer belongs to the caller.
#include <string.h>

#include <cmath>
#include <mutex>

#include "kernels.hpp"

using namespace packkv;

namespace {

constexpr uint64_t kArenaSlack = 64;   // over-read room for 16-byte vector loads

int check_cfg(const packkv_config_t* c) {
  if (!c) return PACKKV_EINVAL;
  if (!head_dim_ok(c->head_dim) || c->run_tokens != kR) return PACKKV_EUNSUPPORTED;
  if (c->bits < 2 || c->bits > 8) return PACKKV_EUNSUPPORTED;
  if (c->block_tokens != 64 && c->block_tokens != 128) return PACKKV_EUNSUPPORTED;
  if (c->permute < 0 || c->permute > 2) return PACKKV_EINVAL;
  if (c->payload_order < 0 || c->payload_order > 1) return PACKKV_EINVAL;
  if (c->payload_order == 1 && c->bits > 4) return PACKKV_EUNSUPPORTED;
  return PACKKV_OK;
}

int64_t max_blocks_of(const packkv_config_t* c, int64_t max_tokens) {
  return (max_tokens + c->block_tokens - 1) / c->block_tokens;
}

uint64_t stride_bytes(const packkv_config_t* c, int64_t max_tokens) {
  const int B = c->block_tokens;
  const uint64_t rk = (uint64_t)max_record_bytes(false, B, c->bits, c->head_dim);
  const uint64_t rv = (uint64_t)max_record_bytes(true, B, c->bits, c->head_dim);
  const uint64_t per = rk > rv ? rk : rv;
  const uint64_t need = (uint64_t)max_blocks_of(c, max_tokens) * per + kArenaSlack;
  return (need + 255) & ~(uint64_t)255;
}

int check_cache(const packkv_cache_t* c) {
  if (!c) return PACKKV_EINVAL;
  int e = check_cfg(&c->cfg);
  if (e) return e;
  if (c->n_streams < 1 || c->max_tokens < 1 || c->n_tokens < 0 || c->n_tokens > c->max_tokens)
    return PACKKV_EINVAL;
  if (!c->k_arena || !c->v_arena || !c->k_off || !c->v_off || !c->perm || !c->tail_k || !c->tail_v ||
      !c->status)
    return PACKKV_EINVAL;
  if (c->arena_stride % 256 || c->arena_stride >= (1ull << 32) ||
      c->arena_stride < stride_bytes(&c->cfg, c->max_tokens))
    return PACKKV_EINVAL;
  if (max_blocks_of(&c->cfg, c->max_tokens) >= (1ll << 31)) return PACKKV_EINVAL;
  return PACKKV_OK;
}

// Blocks per workgroup.  The V GEMV and fused attention keep about two
// rounds of one-wave workgroups over the chip's resident slots (16 per CU):
// their workgroups end with a partial sum that the last one of the stream
// merges, so fewer, longer workgroups pay less for it.  The K GEMV has no
// merge and is fastest with many short workgroups (better balance at the
// kernel's end).  Always even, at most 64.  The division depends only on the
// cache's shape, so results are the same from run to run.
int gemv_blocks_per_wg(int64_t n_streams, int nb, bool split_merge, int group, int bits) {
  int64_t j;
  if (!split_merge) {
    // K GEMV (no merge): short workgroups keep many blocks in flight; at 2
    // and 3 bits, where the decode is the heaviest per byte, 4 blocks repay
    // the per-workgroup set-up.  Measured (K GEMV): 2 bits 127.7 -> 123.9 us
    // and 3 bits (append-64k) 258.9 -> 252.8 us (A/B in one process); at 4 and
    // 8 bits 4 blocks are 2-4 % slower, and with four queries 8 blocks are
    // no faster
    j = bits <= 3 && group == 1 ? 4 : 2;
  }
  else {
    // at 3 bits with one query, about four rounds instead of two (shorter
    // workgroups): measured in bench.py's step at append-64k, three
    // alternating processes each, V GEMV 230.3 -> 220.5 us and fused
    // attention 389.4 -> 387.1 us
    const int64_t per = bits == 3 && group == 1 ? 15360 : 7680;
    j = (n_streams * (int64_t)nb + per - 1) / per;
    j += j & 1;
    // several queries per block: twice the blocks, so the split partials
    // (one per query) stay few; measured with 4 queries and 128-token
    // blocks, fused attention 306 -> 300 us and the V GEMV 157 -> 149 us
    if (group > 1) j *= 2;
  }
  j += j & 1;
  const int lo = split_merge ? 4 : 2;   // the V workspace assumes at least 4
  if (j < lo) j = lo;
  if (j > 64) j = 64;
  return (int)j;
}

int hip_status(hipError_t e) { return e == hipSuccess ? PACKKV_OK : PACKKV_EHIP; }

// Split count of a fused attention launch over `units` (caches x streams)
// workgroup rows.  When the default count leaves the launch within two
// rounds of resident workgroups, the second round runs partly empty; the
// largest count that fits one round is then taken instead, if it keeps at
// most 64 blocks per workgroup.  Only ever lowers the count, so the
// workspace sized for the default still holds the partials.  Measured with
// 32 streams of 131072 tokens, four queries per stream: 86 -> 48 splits,
// fused attention 204 -> 178 us; with hundreds of streams (three or more
// rounds) one round measured slower and the default stays.
int attention_splits(int64_t units, int splits, int nb, int B, int bits, int G, int D) {
  const int64_t R = attention_resident_wgs(B, bits, G, D);
  if (R <= 0 || units <= 0 || units * splits > 2 * R) return splits;
  const int64_t sp = R / units;
  if (sp < 1 || sp >= splits || (nb + sp - 1) / sp > 64) return splits;
  return (int)sp;
}

GemvArgs gemv_args(const packkv_cache_t* c, bool is_v, int group = 1) {
  GemvArgs a;
  memset(&a, 0, sizeof(a));
  a.arena = is_v ? c->v_arena : c->k_arena;
  a.arena_stride = c->arena_stride;
  a.off = is_v ? c->v_off : c->k_off;
  a.off_stride = max_blocks_of(&c->cfg, c->max_tokens) + 1;
  a.n_tokens = c->n_tokens;
  a.nb = (int)((c->n_tokens + c->cfg.block_tokens - 1) / c->cfg.block_tokens);
  a.bits = c->cfg.bits;
  a.D = c->cfg.head_dim;
  a.blocks_per_wg = gemv_blocks_per_wg(c->n_streams, a.nb, is_v, group, c->cfg.bits);
  a.splits = (a.nb + a.blocks_per_wg - 1) / a.blocks_per_wg;
  a.korder = is_v ? 0 : c->cfg.payload_order;
  a.status = c->status;
  return a;
}

EncArgs enc_args(const packkv_cache_t* c) {
  EncArgs a;
  memset(&a, 0, sizeof(a));
  a.bits = c->cfg.bits;
  a.B = c->cfg.block_tokens;
  a.D = c->cfg.head_dim;
  a.permute = c->cfg.permute;
  a.korder = c->cfg.payload_order;
  a.k_arena = c->k_arena;
  a.v_arena = c->v_arena;
  a.arena_stride = c->arena_stride;
  a.arena_limit = c->arena_stride - kArenaSlack;
  a.k_off = c->k_off;
  a.v_off = c->v_off;
  a.off_stride = max_blocks_of(&c->cfg, c->max_tokens) + 1;
  a.perm = c->perm;
  a.perm_stride = max_blocks_of(&c->cfg, c->max_tokens) * c->cfg.block_tokens;
  a.status = c->status;
  return a;
}

}  // namespace

extern "C" {

int packkv_cache_sizes(const packkv_config_t* cfg, int32_t n_streams, int64_t max_tokens,
                       packkv_sizes_t* out) {
  int e = check_cfg(cfg);
  if (e) return e;
  if (!out || n_streams < 1 || max_tokens < 1) return PACKKV_EINVAL;
  const int64_t mb = max_blocks_of(cfg, max_tokens);
  out->max_blocks = mb;
  out->arena_stride = stride_bytes(cfg, max_tokens);
  if (out->arena_stride >= (1ull << 32)) return PACKKV_EINVAL;
  out->arena_bytes = (uint64_t)n_streams * out->arena_stride;
  out->off_bytes = (uint64_t)n_streams * (uint64_t)(mb + 1) * 4;
  out->perm_bytes = (uint64_t)n_streams * (uint64_t)mb * (uint64_t)cfg->block_tokens;
  out->tail_bytes = (uint64_t)n_streams * (uint64_t)cfg->block_tokens * (uint64_t)cfg->head_dim * 2;
  return PACKKV_OK;
}

uint64_t packkv_arena_stride_bytes(const packkv_config_t* cfg, int64_t max_tokens) {
  if (check_cfg(cfg) || max_tokens < 1) return 0;
  return stride_bytes(cfg, max_tokens);
}

// V workspace: fp32 partial sums [S][G][splits][D] for the largest split
// count the cache can need, then one u32 arrival counter per stream.
static uint64_t pv_partial_bytes(const packkv_cache_t* c, int32_t group) {
  const int64_t mb = max_blocks_of(&c->cfg, c->max_tokens);
  const int64_t splits = (mb + 3) / 4;     // blocks per workgroup is at least 4
  return (uint64_t)c->n_streams * (uint64_t)group * (uint64_t)splits * (uint64_t)c->cfg.head_dim * sizeof(float);
}

uint64_t packkv_pv_workspace_bytes(const packkv_cache_t* c, int32_t group) {
  if (check_cache(c) || group < 1) return 0;
  return pv_partial_bytes(c, group) + (((uint64_t)c->n_streams * 4u + 255u) & ~(uint64_t)255u);
}

int packkv_compress_block(packkv_cache_t* c, const void* k_f16, const void* v_f16, int64_t n_tokens,
                          void* stream) {
  int e = check_cache(c);
  if (e) return e;
  if (!k_f16 || !v_f16 || n_tokens < 1) return PACKKV_EINVAL;
  if (((uintptr_t)k_f16 | (uintptr_t)v_f16) & 15u) return PACKKV_EINVAL;   // read with 16-byte loads
  if (c->n_tokens != 0) return PACKKV_ESTATE;
  if (n_tokens > c->max_tokens) return PACKKV_ECAPACITY;
  hipStream_t st = (hipStream_t)stream;
  const int B = c->cfg.block_tokens, D = c->cfg.head_dim;
  const int nb = (int)((n_tokens + B - 1) / B);
  EncArgs a = enc_args(c);
  a.k = (const uint16_t*)k_f16;
  a.v = (const uint16_t*)v_f16;
  a.src_stream = n_tokens * D;
  a.src_block = (int64_t)B * D;
  a.n_tokens = n_tokens;
  a.mode = kPass1;
  if ((e = hip_status(launch_encode(a, c->n_streams, nb, st)))) return e;
  if ((e = hip_status(launch_scan_offsets(c->k_off, c->v_off, a.off_stride, c->n_streams, nb, st))))
    return e;
  a.mode = kPass2;
  if ((e = hip_status(launch_encode(a, c->n_streams, nb, st)))) return e;
  const int64_t nfull = n_tokens / B;
  const int rem = (int)(n_tokens - nfull * B);
  if (rem) {
    e = hip_status(launch_stage_tail((const uint16_t*)k_f16 + nfull * B * D,
                                     (const uint16_t*)v_f16 + nfull * B * D, n_tokens * D, c->tail_k,
                                     c->tail_v, B, D, 0, rem, c->n_streams, st));
    if (e) return e;
  }
  c->n_tokens = n_tokens;
  return PACKKV_OK;
}

int packkv_append_tokens(packkv_cache_t* c, const void* k_f16, const void* v_f16, int32_t n_new,
                         void* stream) {
  int e = check_cache(c);
  if (e) return e;
  if (!k_f16 || !v_f16 || n_new < 1) return PACKKV_EINVAL;
  if (((uintptr_t)k_f16 | (uintptr_t)v_f16) & 15u) return PACKKV_EINVAL;   // read with 16-byte loads
  if (c->n_tokens + n_new > c->max_tokens) return PACKKV_ECAPACITY;
  hipStream_t st = (hipStream_t)stream;
  const int B = c->cfg.block_tokens, D = c->cfg.head_dim;
  EncArgs a = enc_args(c);
  a.k = c->tail_k;
  a.v = c->tail_v;
  a.src_stream = (int64_t)B * D;
  a.src_block = 0;
  a.mode = kTail;
  int done = 0;
  while (done < n_new) {
    const int64_t T = c->n_tokens;
    const int n_tail = (int)(T % B);
    const int cnt = (n_new - done) < (B - n_tail) ? (n_new - done) : (B - n_tail);
    // the encoder reads the new tokens from the caller and stages them itself
    a.new_k = (const uint16_t*)k_f16 + (int64_t)done * D;
    a.new_v = (const uint16_t*)v_f16 + (int64_t)done * D;
    a.new_stream = (int64_t)n_new * D;
    a.new_at = n_tail;
    a.block0 = (int)(T / B);
    a.n_tokens = T + cnt;
    if ((e = hip_status(launch_encode(a, c->n_streams, 1, st)))) return e;
    c->n_tokens = T + cnt;
    done += cnt;
  }
  return PACKKV_OK;
}

int packkv_qk_gemv(const packkv_cache_t* c, const void* q_f16, int32_t group, float* scores, int64_t ld,
                   void* stream) {
  int e = check_cache(c);
  if (e) return e;
  if (!q_f16 || !scores || group < 1) return PACKKV_EINVAL;
  if (c->n_tokens < 1) return PACKKV_ESTATE;
  if (ld < c->n_tokens) return PACKKV_EINVAL;
  GemvArgs a = gemv_args(c, false);
  a.G = group;
  a.q = (const uint16_t*)q_f16;
  a.scores = scores;
  a.ld = ld;
  return hip_status(launch_qk(a, c->cfg.block_tokens, c->n_streams, (hipStream_t)stream));
}

int packkv_pv_gemv(const packkv_cache_t* c, const float* p, int64_t ld, int32_t group, float* out,
                   void* workspace, uint64_t ws_bytes, void* stream) {
  int e = check_cache(c);
  if (e) return e;
  if (!p || !out || !workspace || group < 1) return PACKKV_EINVAL;
  if (c->n_tokens < 1) return PACKKV_ESTATE;
  if (ld < c->n_tokens) return PACKKV_EINVAL;
  GemvArgs a = gemv_args(c, true, group);
  a.G = group;
  a.p = p;
  a.ld = ld;
  a.ws = (float*)workspace;
  a.tickets = (uint32_t*)((uint8_t*)workspace + pv_partial_bytes(c, group));
  a.out = out;
  if (ws_bytes < packkv_pv_workspace_bytes(c, group)) return PACKKV_EINVAL;
  return hip_status(launch_pv(a, c->cfg.block_tokens, c->n_streams, (hipStream_t)stream));
}

// Attention workspace: per (stream, query, split) D + 4 floats, then
// one u32 arrival counter per stream.
static uint64_t attn_partial_bytes(const packkv_cache_t* c, int32_t group) {
  const int64_t mb = max_blocks_of(&c->cfg, c->max_tokens);
  const int64_t splits = (mb + 3) / 4;     // blocks per workgroup is at least 4
  return (uint64_t)c->n_streams * (uint64_t)group * (uint64_t)splits * attn_partial_floats(c->cfg.head_dim) *
         sizeof(float);
}

uint64_t packkv_attention_workspace_bytes(const packkv_cache_t* c, int32_t group) {
  if (check_cache(c) || group < 1) return 0;
  return attn_partial_bytes(c, group) + (((uint64_t)c->n_streams * 4u + 255u) & ~(uint64_t)255u);
}

// Launch arguments of fused attention over caches of c's shape (n per
// launch at most kAttnMaxCaches): the split-merge work division, the scale,
// q/out strides.  Workspace pointers are left to the caller.
static AttnArgs attention_args(const packkv_cache_t* c, int32_t n, int32_t group, float scale) {
  const GemvArgs g = gemv_args(c, true, group);   // the split-merge work division
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.arena_stride = c->arena_stride;
  a.off_stride = g.off_stride;
  a.n_tokens = c->n_tokens;
  a.nb = g.nb;
  a.bits = c->cfg.bits;
  a.blocks_per_wg = g.blocks_per_wg;
  a.splits = attention_splits((int64_t)c->n_streams * (n < kAttnMaxCaches ? n : kAttnMaxCaches), g.splits, g.nb,
                              c->cfg.block_tokens, c->cfg.bits, group, c->cfg.head_dim);
  a.G = group;
  a.korder = c->cfg.payload_order;
  a.scale_log2e = scale * 1.4426950408889634f;
  a.qo_stride = (int64_t)c->n_streams * group * c->cfg.head_dim;
  a.D = c->cfg.head_dim;
  return a;
}

// Decode attention over n caches of one shape, in launches of up to
// kAttnMaxCaches caches.
static int attention_decode(const packkv_cache_t* const* cs, int32_t n, const void* q_f16, int32_t group,
                            float scale, float* out, void* workspace, uint64_t ws_bytes, void* stream) {
  if (!cs || n < 1) return PACKKV_EINVAL;
  const packkv_cache_t* c = cs[0];
  int e = check_cache(c);
  if (e) return e;
  for (int32_t i = 1; i < n; ++i) {
    const packkv_cache_t* d = cs[i];
    if ((e = check_cache(d))) return e;
    if (d->cfg.bits != c->cfg.bits || d->cfg.block_tokens != c->cfg.block_tokens || d->cfg.head_dim != c->cfg.head_dim ||
        d->cfg.payload_order != c->cfg.payload_order ||
        d->n_streams != c->n_streams || d->max_tokens != c->max_tokens || d->n_tokens != c->n_tokens ||
        d->arena_stride != c->arena_stride)
      return PACKKV_EINVAL;
  }
  if (!q_f16 || !out || !workspace || group < 1 || !(scale > 0.f) || !std::isfinite(scale)) return PACKKV_EINVAL;
  if (c->n_tokens < 1) return PACKKV_ESTATE;
  const uint64_t per_cache = packkv_attention_workspace_bytes(c, group);
  if (ws_bytes < per_cache * (uint64_t)n) return PACKKV_EINVAL;
  AttnArgs a = attention_args(c, n, group, scale);
  a.ws_stride = per_cache;
  a.tk_stride = per_cache;
  for (int32_t i0 = 0; i0 < n; i0 += kAttnMaxCaches) {
    const int32_t m = n - i0 < kAttnMaxCaches ? n - i0 : kAttnMaxCaches;
    for (int32_t i = 0; i < m; ++i) {
      const packkv_cache_t* d = cs[i0 + i];
      a.cache[i] = AttnCache{d->k_arena, d->v_arena, d->k_off, d->v_off, d->status};
    }
    a.q = (const uint16_t*)q_f16 + i0 * a.qo_stride;
    a.out = out + i0 * a.qo_stride;
    a.ws = (uint8_t*)workspace + (uint64_t)i0 * per_cache;
    a.tk = a.ws + attn_partial_bytes(c, group);
    if ((e = hip_status(launch_attention(a, c->cfg.block_tokens, c->n_streams, m, (hipStream_t)stream)))) return e;
  }
  return PACKKV_OK;
}

int packkv_attention_decode(const packkv_cache_t* c, const void* q_f16, int32_t group, float scale, float* out,
                            void* workspace, uint64_t ws_bytes, void* stream) {
  return attention_decode(&c, 1, q_f16, group, scale, out, workspace, ws_bytes, stream);
}

int packkv_attention_decode_multi(const packkv_cache_t* const* caches, int32_t n_caches, const void* q_f16,
                                  int32_t group, float scale, float* out, void* workspace, uint64_t ws_bytes,
                                  void* stream) {
  return attention_decode(caches, n_caches, q_f16, group, scale, out, workspace, ws_bytes, stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Fused attention with the library's own scratch memory, for callers that
// cannot allocate.  The split partials and the per-stream arrival counters
// live in one file-scope device array per GPU: counters first, at fixed
// places (so a call of any shape finds them where the previous call, of any
// shape, left them at zero), then the partials of the current call.
namespace {

constexpr uint64_t kScratchBytes = 16ull << 20;
constexpr int32_t kScratchStreams = 16384;
constexpr uint64_t kScratchCounterBytes = (uint64_t)kScratchStreams * 4;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

// The counters the kernel relies on start at zero: cleared with a kernel
// (not a memset, which graph capture would record as a memset node) on the
// call's stream before the attention launch.
__global__ __launch_bounds__(256) void k_clear_counters(uint32_t* counters, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) counters[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
uint8_t* scratch_dev[kMaxDevices];   // device address of `scratch` on each GPU, once asked

// The device address of the current device's scratch array (each GPU holds
// its own copy at its own address; the array's name is only a host-side
// handle, so host code passes this address to kernels, never the name).
int scratch_of_current_device(uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PACKKV_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return PACKKV_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PACKKV_EHIP;
    scratch_dev[dev] = static_cast<uint8_t*>(p);
  }
  *out = scratch_dev[dev];
  return PACKKV_OK;
}

}  // namespace

extern "C" {

int packkv_attention_decode_noalloc(const packkv_cache_t* c, const void* q_f16, int32_t group, float scale,
                                    float* out, void* stream) {
  int e = check_cache(c);
  if (e) return e;
  if (!q_f16 || !out || group < 1 || !(scale > 0.f) || !std::isfinite(scale)) return PACKKV_EINVAL;
  if (c->n_tokens < 1) return PACKKV_ESTATE;
  AttnArgs a = attention_args(c, 1, group, scale);
  const uint64_t partials =
      (uint64_t)c->n_streams * (uint64_t)group * (uint64_t)a.splits * attn_partial_floats(c->cfg.head_dim) * 4u;
  if (c->n_streams > kScratchStreams || partials > kScratchBytes - kScratchCounterBytes) return PACKKV_ECAPACITY;
  uint8_t* base = nullptr;
  if ((e = scratch_of_current_device(&base))) return e;
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(k_clear_counters, dim3((c->n_streams + 255) / 256), dim3(256), 0, st,
                     reinterpret_cast<uint32_t*>(base), c->n_streams);
  if ((e = hip_status(hipGetLastError()))) return e;
  a.cache[0] = AttnCache{c->k_arena, c->v_arena, c->k_off, c->v_off, c->status};
  a.q = (const uint16_t*)q_f16;
  a.out = out;
  a.tk = base;
  a.ws = base + kScratchCounterBytes;
  return hip_status(launch_attention(a, c->cfg.block_tokens, c->n_streams, 1, st));
}

uint64_t packkv_attention_multi_workspace_bytes(const packkv_cache_t* c, int32_t group, int32_t n_caches) {
  if (n_caches < 1) return 0;
  return packkv_attention_workspace_bytes(c, group) * (uint64_t)n_caches;
}

int packkv_decompress(const packkv_cache_t* c, int32_t which, int32_t mode, void* out, void* stream) {
  int e = check_cache(c);
  if (e) return e;
  if (!out || (which != 0 && which != 1) || (mode != 0 && mode != 1)) return PACKKV_EINVAL;
  if (c->n_tokens < 1) return PACKKV_ESTATE;
  GemvArgs a = gemv_args(c, which == 1);
  const int64_t perm_stride = max_blocks_of(&c->cfg, c->max_tokens) * c->cfg.block_tokens;
  return hip_status(launch_decompress(a, c->cfg.block_tokens, which == 1, c->n_streams, c->perm,
                                      perm_stride, mode, out, (hipStream_t)stream));
}

int packkv_softmax_rows(const float* scores, float* p, int32_t rows, int64_t T, int64_t ld, float scale,
                        void* stream) {
  if (!scores || !p || rows < 1 || T < 1 || ld < T) return PACKKV_EINVAL;
  return hip_status(launch_softmax(scores, p, rows, T, ld, scale, (hipStream_t)stream));
}

int packkv_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 || ((uintptr_t)buf & 15u)) return PACKKV_EINVAL;
  return hip_status(launch_stream_read(buf, bytes, sink, (hipStream_t)stream));
}

int packkv_check(const packkv_cache_t* c, void* stream) {
  if (!c || !c->status) return PACKKV_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  if (hipStreamSynchronize(st) != hipSuccess) return PACKKV_EHIP;
  int32_t v = 0;
  if (hipMemcpy(&v, c->status, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return PACKKV_EHIP;
  if (v) {
    const int32_t zero = 0;
    if (hipMemcpy(c->status, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return PACKKV_EHIP;
  }
  return v;
}

int packkv_stats(const packkv_cache_t* c, uint64_t* out, void* stream) {
  int e = check_cache(c);
  if (e) return e;
  if (!out) return PACKKV_EINVAL;
  if (c->n_tokens < 1) return PACKKV_ESTATE;
  hipStream_t st = (hipStream_t)stream;
  for (int which = 0; which < 2; ++which) {
    GemvArgs a = gemv_args(c, which == 1);
    e = hip_status(launch_stats(a, c->cfg.block_tokens, which == 1, c->n_streams,
                                (unsigned long long*)out, st));
    if (e) return e;
  }
  return PACKKV_OK;
}

const char* packkv_status_str(int s) {
  switch (s) {
    case PACKKV_OK: return "ok";
    case PACKKV_EINVAL: return "invalid argument";
    case PACKKV_EUNSUPPORTED: return "unsupported configuration";
    case PACKKV_ECAPACITY: return "capacity exceeded";
    case PACKKV_ECORRUPT: return "corrupt record";
    case PACKKV_EHIP: return "HIP runtime error";
    case PACKKV_ESTATE: return "invalid cache state";
    default: return "unknown status";
  }
}

// ---------------------------------------------------------------------------
// Paged cache.

namespace {

constexpr int kPagedD = 128;   // head_dim of the paged cache

uint64_t paged_slot_bytes(const packkv_config_t* c) {
  const int B = c->block_tokens;
  const uint64_t rk = (uint64_t)max_record_bytes(false, B, c->bits, kPagedD);
  const uint64_t rv = (uint64_t)max_record_bytes(true, B, c->bits, kPagedD);
  return ((rk > rv ? rk : rv) + 15) & ~(uint64_t)15;
}
uint64_t paged_min_page(const packkv_config_t* c) { return (paged_slot_bytes(c) + 255) & ~(uint64_t)255; }
uint64_t paged_pool_bytes(const packkv_config_t* c, int32_t n_streams, int32_t n_pages, uint64_t page_bytes) {
  return (uint64_t)n_pages * page_bytes + (uint64_t)n_streams * 2u * paged_slot_bytes(c) + 256u;
}

int check_paged(const packkv_paged_t* c) {
  if (!c) return PACKKV_EINVAL;
  int e = check_cfg(&c->cfg);
  if (e) return e;
  if (c->cfg.head_dim != kPagedD) return PACKKV_EUNSUPPORTED;
  if (c->n_streams < 1 || c->n_pages < 1 || c->max_tokens < 1) return PACKKV_EINVAL;
  if (c->page_bytes % 256 || c->page_bytes < paged_min_page(&c->cfg)) return PACKKV_EINVAL;
  if (paged_pool_bytes(&c->cfg, c->n_streams, c->n_pages, c->page_bytes) >= (1ull << 36)) return PACKKV_EINVAL;
  if (max_blocks_of(&c->cfg, c->max_tokens) >= (1ll << 31)) return PACKKV_EINVAL;
  if (!c->pool || !c->k_table || !c->v_table || !c->lengths || !c->alloc || !c->perm || !c->tail_k ||
      !c->tail_v || !c->status || !c->host_lengths)
    return PACKKV_EINVAL;
  return PACKKV_OK;
}

PageAlloc page_alloc_of(const packkv_paged_t* c) {
  PageAlloc p;
  p.state = c->alloc;
  p.n_streams = c->n_streams;
  p.n_pages = (uint32_t)c->n_pages;
  p.page16 = (uint32_t)(c->page_bytes / 16);
  p.tail16 = (uint32_t)((uint64_t)c->n_pages * c->page_bytes / 16);
  p.slot16 = (uint32_t)(paged_slot_bytes(&c->cfg) / 16);
  return p;
}

EncArgs paged_enc_args(const packkv_paged_t* c) {
  EncArgs a;
  memset(&a, 0, sizeof(a));
  const int64_t mb = max_blocks_of(&c->cfg, c->max_tokens);
  a.bits = c->cfg.bits;
  a.B = c->cfg.block_tokens;
  a.D = kPagedD;
  a.permute = c->cfg.permute;
  a.korder = c->cfg.payload_order;
  a.k_arena = c->pool;
  a.v_arena = c->pool;
  a.arena_limit = paged_pool_bytes(&c->cfg, c->n_streams, c->n_pages, c->page_bytes);
  a.off_stride = mb;
  a.perm = c->perm;
  a.perm_stride = mb * c->cfg.block_tokens;
  a.status = c->status;
  a.paged = 1;
  a.k_tab = reinterpret_cast<uint2*>(c->k_table);
  a.v_tab = reinterpret_cast<uint2*>(c->v_table);
  a.lengths = c->lengths;
  a.pages = page_alloc_of(c);
  return a;
}

uint64_t paged_partial_bytes(const packkv_paged_t* c, int32_t group) {
  const int64_t mb = max_blocks_of(&c->cfg, c->max_tokens);
  const int64_t splits = (mb + 3) / 4;     // blocks per workgroup is at least 4
  return (uint64_t)c->n_streams * (uint64_t)group * (uint64_t)splits * attn_partial_floats(kPagedD) * sizeof(float);
}

}  // namespace

int packkv_paged_sizes(const packkv_config_t* cfg, int32_t n_streams, int64_t max_tokens, int32_t n_pages,
                       uint64_t page_bytes, packkv_paged_sizes_t* out) {
  int e = check_cfg(cfg);
  if (e) return e;
  if (cfg->head_dim != kPagedD) return PACKKV_EUNSUPPORTED;
  if (!out || n_streams < 1 || max_tokens < 1 || n_pages < 1) return PACKKV_EINVAL;
  const int64_t mb = max_blocks_of(cfg, max_tokens);
  out->max_blocks = mb;
  out->slot_bytes = paged_slot_bytes(cfg);
  out->min_page_bytes = paged_min_page(cfg);
  if (page_bytes % 256 || page_bytes < out->min_page_bytes) return PACKKV_EINVAL;
  out->pool_bytes = paged_pool_bytes(cfg, n_streams, n_pages, page_bytes);
  if (out->pool_bytes >= (1ull << 36) || mb >= (1ll << 31)) return PACKKV_EINVAL;   // 32-bit 16-byte units
  out->table_bytes = (uint64_t)n_streams * (uint64_t)mb * 8;
  out->alloc_bytes = (2u + 4u * (uint64_t)n_streams + (uint64_t)n_pages) * 4;
  out->lengths_bytes = (uint64_t)n_streams * 4;
  out->perm_bytes = (uint64_t)n_streams * (uint64_t)mb * (uint64_t)cfg->block_tokens;
  out->tail_bytes = (uint64_t)n_streams * (uint64_t)cfg->block_tokens * kPagedD * 2;
  return PACKKV_OK;
}

int packkv_paged_init(packkv_paged_t* c, void* stream) {
  int e = check_paged(c);
  if (e) return e;
  if ((e = hip_status(launch_paged_init(page_alloc_of(c), c->lengths, c->status, (hipStream_t)stream)))) return e;
  memset(c->host_lengths, 0, sizeof(int32_t) * (size_t)c->n_streams);
  return PACKKV_OK;
}

int packkv_paged_prefill(packkv_paged_t* c, int32_t stream0, int32_t n, const void* k_f16, const void* v_f16,
                         int64_t n_tokens, void* stream) {
  int e = check_paged(c);
  if (e) return e;
  if (!k_f16 || !v_f16 || n < 1 || stream0 < 0 || (int64_t)stream0 + n > c->n_streams || n_tokens < 1)
    return PACKKV_EINVAL;
  if (((uintptr_t)k_f16 | (uintptr_t)v_f16) & 15u) return PACKKV_EINVAL;   // read with 16-byte loads
  if (n_tokens > c->max_tokens) return PACKKV_ECAPACITY;
  for (int32_t s = stream0; s < stream0 + n; ++s)
    if (c->host_lengths[s] != 0) return PACKKV_ESTATE;
  hipStream_t st = (hipStream_t)stream;
  const int B = c->cfg.block_tokens;
  const int nb = (int)((n_tokens + B - 1) / B);
  EncArgs a = paged_enc_args(c);
  a.stream0 = stream0;
  a.k = (const uint16_t*)k_f16;
  a.v = (const uint16_t*)v_f16;
  a.src_stream = n_tokens * kPagedD;
  a.src_block = (int64_t)B * kPagedD;
  a.n_tokens = n_tokens;
  a.mode = kPass1;
  if ((e = hip_status(launch_encode(a, n, nb, st)))) return e;
  if ((e = hip_status(launch_paged_alloc(a, n, n_tokens, st)))) return e;
  a.mode = kPass2;
  if ((e = hip_status(launch_encode(a, n, nb, st)))) return e;
  const int64_t nfull = n_tokens / B;
  const int rem = (int)(n_tokens - nfull * B);
  if (rem) {
    const int64_t t0 = (int64_t)stream0 * B * kPagedD;
    e = hip_status(launch_stage_tail((const uint16_t*)k_f16 + nfull * B * kPagedD,
                                     (const uint16_t*)v_f16 + nfull * B * kPagedD, n_tokens * kPagedD, c->tail_k + t0,
                                     c->tail_v + t0, B, kPagedD, 0, rem, n, st));
    if (e) return e;
  }
  for (int32_t s = stream0; s < stream0 + n; ++s) c->host_lengths[s] = (int32_t)n_tokens;
  return PACKKV_OK;
}

int packkv_paged_append(packkv_paged_t* c, const void* k_f16, const void* v_f16, void* stream) {
  int e = check_paged(c);
  if (e) return e;
  if (!k_f16 || !v_f16) return PACKKV_EINVAL;
  if (((uintptr_t)k_f16 | (uintptr_t)v_f16) & 15u) return PACKKV_EINVAL;
  for (int32_t s = 0; s < c->n_streams; ++s)
    if ((int64_t)c->host_lengths[s] + 1 > c->max_tokens) return PACKKV_ECAPACITY;
  const int B = c->cfg.block_tokens;
  EncArgs a = paged_enc_args(c);
  a.k = c->tail_k;                // the raw staging of each open block
  a.v = c->tail_v;
  a.src_stream = (int64_t)B * kPagedD;
  a.mode = kTail;
  a.new_k = (const uint16_t*)k_f16;
  a.new_v = (const uint16_t*)v_f16;
  a.new_stream = kPagedD;              // one token per stream
  if ((e = hip_status(launch_encode(a, c->n_streams, 1, (hipStream_t)stream)))) return e;
  for (int32_t s = 0; s < c->n_streams; ++s) c->host_lengths[s] += 1;
  return PACKKV_OK;
}

int packkv_paged_release(packkv_paged_t* c, int32_t s, void* stream) {
  int e = check_paged(c);
  if (e) return e;
  if (s < 0 || s >= c->n_streams) return PACKKV_EINVAL;
  e = hip_status(launch_paged_release(page_alloc_of(c), reinterpret_cast<const uint2*>(c->k_table),
                                      reinterpret_cast<const uint2*>(c->v_table),
                                      max_blocks_of(&c->cfg, c->max_tokens), c->lengths, c->cfg.block_tokens, s,
                                      (hipStream_t)stream));
  if (e) return e;
  c->host_lengths[s] = 0;
  return PACKKV_OK;
}

uint64_t packkv_paged_attention_workspace_bytes(const packkv_paged_t* c, int32_t group) {
  if (check_paged(c) || group < 1) return 0;
  return paged_partial_bytes(c, group) + (((uint64_t)c->n_streams * 4u + 255u) & ~(uint64_t)255u);
}

int packkv_paged_attention(const packkv_paged_t* c, const void* q_f16, int32_t group, float scale, float* out,
                           void* workspace, uint64_t ws_bytes, void* stream) {
  int e = check_paged(c);
  if (e) return e;
  if (!q_f16 || !out || !workspace || group < 1 || !(scale > 0.f) || !std::isfinite(scale))
    return PACKKV_EINVAL;
  const uint64_t need = packkv_paged_attention_workspace_bytes(c, group);
  if (ws_bytes < need) return PACKKV_EINVAL;
  int64_t longest = 0;
  for (int32_t s = 0; s < c->n_streams; ++s) longest = c->host_lengths[s] > longest ? c->host_lengths[s] : longest;
  if (longest < 1) return PACKKV_ESTATE;
  const int B = c->cfg.block_tokens;
  // the launch is sized for the longest stream; every stream spreads its
  // own blocks evenly over the same splits (at most J each)
  const int nb = (int)((longest + B - 1) / B);
  const int J = gemv_blocks_per_wg(c->n_streams, nb, true, group, c->cfg.bits);
  AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.cache[0] = AttnCache{c->pool, c->pool, nullptr, nullptr, c->status,
                         reinterpret_cast<const uint2*>(c->k_table), reinterpret_cast<const uint2*>(c->v_table),
                         c->lengths};
  a.arena_stride = paged_pool_bytes(&c->cfg, c->n_streams, c->n_pages, c->page_bytes);
  a.off_stride = max_blocks_of(&c->cfg, c->max_tokens);
  a.bits = c->cfg.bits;
  a.blocks_per_wg = J;
  // the same division as the contiguous cache for the same lengths
  a.splits = attention_splits(c->n_streams, (nb + J - 1) / J, nb, B, c->cfg.bits, group, kPagedD);
  a.D = kPagedD;
  a.G = group;
  a.korder = c->cfg.payload_order;
  a.scale_log2e = scale * 1.4426950408889634f;
  a.q = (const uint16_t*)q_f16;
  a.out = out;
  a.qo_stride = (int64_t)c->n_streams * group * kPagedD;
  a.ws = (uint8_t*)workspace;
  a.ws_stride = need;
  a.tk = a.ws + paged_partial_bytes(c, group);
  a.tk_stride = need;
  return hip_status(launch_attention(a, B, c->n_streams, 1, (hipStream_t)stream, true));
}

int packkv_paged_check(const packkv_paged_t* c, void* stream) {
  if (!c || !c->status) return PACKKV_EINVAL;
  hipStream_t st = (hipStream_t)stream;
  if (hipStreamSynchronize(st) != hipSuccess) return PACKKV_EHIP;
  int32_t v = 0;
  if (hipMemcpy(&v, c->status, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return PACKKV_EHIP;
  if (v) {
    const int32_t zero = 0;
    if (hipMemcpy(c->status, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) return PACKKV_EHIP;
  }
  return v;
}

}  // extern "C"
