// Shared device and host helpers of the packkv library (gfx950 / CDNA4).
//
// Record layout (one block of B tokens of one stream), from the PackKV
// pipeline of quantise -> reorder tokens -> lossless channel-direction
// bit-packing (Fig. 2 caption; TL;DR):
//   K: scale[D] f16 | zero[D] f16 | hdr[nr][D] | pad16 | payload | pad16
//   V: scale[B] f16 | zero[B] f16 | hdr[nr][D] | pad16 | payload | pad16
// hdr per (run, channel): the byte (w << 4) | m for b <= 4, the
// little-endian u16 (w << 8) | m for b = 5..8 (m needs the whole byte);
// payload = for run r, channel c: w little-endian u32 words in the sliced
// order described below (sliced_to_nibbles / sliced_to_bytes).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "packkv.h"

namespace packkv {

constexpr int kR = 32;         // run length (slots)
constexpr int kWave = 64;      // CDNA wavefront

// head_dim D is 64, 128 or 256 (a template parameter of every kernel)
__host__ __device__ constexpr bool head_dim_ok(int D) { return D == 64 || D == 128 || D == 256; }

__host__ __device__ constexpr int pad16(int x) { return (x + 15) & ~15; }
__host__ __device__ constexpr int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }

// Geometry of a record holding n tokens (nr runs) of a block of B tokens of
// D channels.
__host__ __device__ constexpr int n_params(bool is_v, int B, int D) { return is_v ? B : D; }
__host__ __device__ constexpr int hdr_offset(bool is_v, int B, int D) { return 4 * n_params(is_v, B, D); }
__host__ __device__ constexpr int hdr_entry_bytes(int bits) { return bits > 4 ? 2 : 1; }
__host__ __device__ constexpr int payload_offset(bool is_v, int B, int nr, int hb, int D) {
  return pad16(4 * n_params(is_v, B, D) + hb * nr * D);
}
__host__ __device__ constexpr int max_record_bytes(bool is_v, int B, int bits, int D) {
  return payload_offset(is_v, B, B / kR, hdr_entry_bytes(bits), D) + 4 * (B / kR) * D * bits;
}
// Fused attention's partial result per (stream, query, split): D partial
// sums, running max, weight sum, 2 pad
__host__ __device__ constexpr int attn_partial_floats(int D) { return D + 4; }

// ---------------------------------------------------------------------------
// fp16 bit helpers (exact).
__device__ __forceinline__ float f16_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);   // v_cvt_f32_f16, exact
}
__device__ __forceinline__ double f16_bits_to_double(uint32_t h) {
  return (double)f16_bits_to_float(h);                        // both conversions exact
}

// ---------------------------------------------------------------------------
// Run payload -> container words.  A run's u = q - m values (32 slots, w
// bits each) are stored in w words laid out for these decoders: with c-bit
// containers (c = 4 for b <= 4, 8 for b = 5..8), slot i belongs to
// container word k = i / (32/c), field j = i % (32/c), and bit p of its u
// sits in run word W at bit c*j + Q, where W = k / g, Q = w*(k % g) + p if
// w divides c (g = c/w), else W = k, Q = p for k < w and W = p, Q = k for
// k >= w.  Rebuilding the container words (every slot's u in its own field,
// upper bits zero) then takes only shifts and masks.

// Nibble containers: out[k] holds u of slots 8k .. 8k+7 (nibble j = slot
// 8k + j), from the run's first W words wd[0 .. W-1].
template <int W>
__device__ __forceinline__ void sliced_to_nibbles(const uint32_t wd[4], uint32_t out[4]) {
  if constexpr (W == 4) {
    out[0] = wd[0]; out[1] = wd[1]; out[2] = wd[2]; out[3] = wd[3];
  } else if constexpr (W == 3) {
    // containers 0..2 in the low 3 bits of words 0..2; bit p of container
    // 3 in bit 3 of every nibble of word p
    out[0] = wd[0] & 0x77777777u;
    out[1] = wd[1] & 0x77777777u;
    out[2] = wd[2] & 0x77777777u;
    out[3] = ((wd[0] >> 3) & 0x11111111u) | ((wd[1] >> 2) & 0x22222222u) | ((wd[2] >> 1) & 0x44444444u);
  } else if constexpr (W == 2) {
    out[0] = wd[0] & 0x33333333u;
    out[1] = (wd[0] >> 2) & 0x33333333u;
    out[2] = wd[1] & 0x33333333u;
    out[3] = (wd[1] >> 2) & 0x33333333u;
  } else if constexpr (W == 1) {
    out[0] = wd[0] & 0x11111111u;
    out[1] = (wd[0] >> 1) & 0x11111111u;
    out[2] = (wd[0] >> 2) & 0x11111111u;
    out[3] = (wd[0] >> 3) & 0x11111111u;
  } else {
    out[0] = out[1] = out[2] = out[3] = 0u;
  }
}

// Byte containers: out[k] holds u of slots 4k .. 4k+3 (byte j = slot 4k + j),
// from the run's first W words wd[0 .. W-1].
template <int W>
__device__ __forceinline__ void sliced_to_bytes(const uint32_t (&wd)[8], uint32_t (&out)[8]) {
  constexpr uint32_t rep = 0x01010101u;
  if constexpr (W == 0) {
#pragma unroll
    for (int k = 0; k < 8; ++k) out[k] = 0u;
  } else if constexpr (8 % W == 0) {
    constexpr int g = 8 / W;
    constexpr uint32_t low = W == 8 ? 0xFFFFFFFFu : ((1u << W) - 1u) * rep;
#pragma unroll
    for (int k = 0; k < 8; ++k) out[k] = (wd[k / g] >> (W * (k % g))) & low;
  } else {
    constexpr uint32_t low = ((1u << W) - 1u) * rep;
#pragma unroll
    for (int k = 0; k < W; ++k) out[k] = wd[k] & low;
#pragma unroll
    for (int k = W; k < 8; ++k) {
      uint32_t x = 0u;
#pragma unroll
      for (int p = 0; p < W; ++p) x |= (wd[p] >> (k - p)) & (rep << p);
      out[k] = x;
    }
  }
}

// m (0..15) in all eight nibbles of a word: one shift-or and a byte broadcast
// (written as v_perm_b32 so that it is not turned into a quarter-rate
// 32-bit multiply; register-only ALU instruction, no memory access).
__device__ __forceinline__ uint32_t nibble_splat(uint32_t m) {
  const uint32_t b = (m & 15u) | ((m & 15u) << 4);
  uint32_t r;
  asm("v_perm_b32 %0, %1, %1, %2" : "=v"(r) : "v"(b), "v"(0u));
  return r;
}

// Decode one run (R = 32 slots) stored at width w (0 .. WMAX) with minimum m
// into four nibble words: word k holds q = m + u of slots 8k .. 8k+7
// (nibble i = slot 8k+i).  Valid for m + 2^w - 1 <= 15.  `wd` holds the
// run's first four payload words (words past the run are ignored).
template <int WMAX = 4>
__device__ __forceinline__ void run_to_nibbles(int w, uint32_t m, const uint32_t wd[4], uint32_t out[4]) {
  // widths above WMAX do not occur at the call site; the widest one that
  // does is tested first
  if (WMAX >= 4 && w == 4) sliced_to_nibbles<4>(wd, out);
  else if (WMAX >= 3 && w == 3) sliced_to_nibbles<3>(wd, out);
  else if (WMAX >= 2 && w == 2) sliced_to_nibbles<2>(wd, out);
  else if (w == 1) sliced_to_nibbles<1>(wd, out);
  else sliced_to_nibbles<0>(wd, out);
  const uint32_t mm = nibble_splat(m);   // m in every nibble; no carries
  out[0] += mm; out[1] += mm; out[2] += mm; out[3] += mm;
}

// A run of width w = 0, 1 or 2 (below a full width of 2 or 3) from its first
// two payload words, without a branch on w: both widths divide the 4-bit
// container, so container k sits in word (k w) / 4 at bit (k w) % 4 of each
// nibble, under the mask of w low bits per nibble (0 for w = 0).
__device__ __forceinline__ void narrow_to_nibbles(int w, uint32_t m, uint32_t x0, uint32_t x1, uint32_t out[4]) {
  const uint32_t mask = (0x11111111u << w) - 0x11111111u;
  const bool two = w == 2;
  const uint32_t mm = nibble_splat(m);
  out[0] = (x0 & mask) + mm;
  out[1] = ((x0 >> w) & mask) + mm;
  out[2] = ((two ? x1 : x0 >> 2) & mask) + mm;
  out[3] = ((two ? x1 >> 2 : x0 >> 3) & mask) + mm;
}

// A run of width w = 0 .. 3 (below a full width of 4) from its first three
// payload words, without a branch on w: widths 0, 1 and 2 as in
// narrow_to_nibbles, width 3 as in sliced_to_nibbles<3>, one of the two
// chosen per lane.  Where a wave's narrow runs come in several widths this
// replaces one masked pass per width present.
__device__ __forceinline__ void narrow4_to_nibbles(int w, uint32_t m, const uint32_t wd[4], uint32_t out[4]) {
  uint32_t lo[4], w3[4];
  narrow_to_nibbles(w, m, wd[0], wd[1], lo);
  sliced_to_nibbles<3>(wd, w3);
  const uint32_t mm = nibble_splat(m);
  const bool three = w == 3;
#pragma unroll
  for (int k = 0; k < 4; ++k) out[k] = three ? w3[k] + mm : lo[k];
}

// A run stored at the full width BITS: its BITS words -> four container words.
template <int BITS>
__device__ __forceinline__ void full_to_nibbles(const uint32_t wd[4], uint32_t out[4]) {
  sliced_to_nibbles<BITS>(wd, out);
}

// Four header bytes (w << 4 | m) of runs that are all at the full width BITS
// with a consistent minimum (m + 2^(BITS-1) <= 2^BITS - 1): SWAR test.
template <int BITS>
__device__ __forceinline__ bool hdr4_full(uint32_t x) {
  constexpr uint32_t want = (uint32_t)BITS * 0x10101010u;
  constexpr uint32_t mbad = (0x0Fu & ~((1u << (BITS - 1)) - 1u)) * 0x01010101u;
  return ((x ^ want) & (0xF0F0F0F0u | mbad)) == 0u;
}

// Four header bytes (w << 4 | m): true if any of them is inconsistent, i.e.
// its width is above BITS or its minimum leaves no room for the width (a
// valid run has max - m in [2^(w-1), 2^w - 1] and max <= L = 2^BITS - 1).
// SWAR: a byte-wise table lookup (v_perm_b32 on w & 7) gives
// c(w) = 2^(w-1) (0 for w = 0, 16 for w > BITS) plus 127 - L, so that
// m + c(w) sets bit 7 exactly when m + 2^(w-1) > L; bit 7 of the header
// byte itself is set for w >= 8.  No byte carries into the next
// (m + c <= 15 + 16 + 124).
template <int BITS>
__device__ __forceinline__ bool hdr4_bad(uint32_t x) {
  constexpr uint32_t L = (1u << BITS) - 1u;
  constexpr uint32_t c0 = 127u - L, c1 = 1u + c0, c2 = (BITS >= 2 ? 2u : 16u) + c0,
                     c3 = (BITS >= 3 ? 4u : 16u) + c0, c4 = (BITS >= 4 ? 8u : 16u) + c0, cx = 16u + c0;
  constexpr uint32_t lo = c0 | c1 << 8 | c2 << 16 | c3 << 24;
  constexpr uint32_t hi = c4 | cx << 8 | cx << 16 | cx << 24;
  const uint32_t c = __builtin_amdgcn_perm(hi, lo, (x >> 4) & 0x07070707u);
  return (((x & 0x0F0F0F0Fu) + c) | x) & 0x80808080u;
}

// Latch the first device-side error code.
__device__ __forceinline__ void latch(int32_t* status, int code) {
  if (status) atomicCAS(status, 0, code);
}

// Cross-lane helpers on DPP (VALU only, no LDS round trips).
// dpp<CTRL>(v): row_shr:n = 0x110+n, row_bcast:15 = 0x142, row_bcast:31 = 0x143;
// lanes without a source read 0, lanes of disabled rows get 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, true);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, true));
}
// Inclusive prefix sum over the 64 lanes (Hillis-Steele inside 16-lane rows,
// then row broadcasts).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp_i<0x111>(v);
  v += dpp_i<0x112>(v);
  v += dpp_i<0x114>(v);
  v += dpp_i<0x118>(v);
  v += dpp_i<0x142, 0xA>(v);
  v += dpp_i<0x143, 0xC>(v);
  return v;
}
__device__ __forceinline__ float wave_incl_scan_f(float v) {
  v += dpp_f<0x111>(v);
  v += dpp_f<0x112>(v);
  v += dpp_f<0x114>(v);
  v += dpp_f<0x118>(v);
  v += dpp_f<0x142, 0xA>(v);
  v += dpp_f<0x143, 0xC>(v);
  return v;
}
// Wave-wide maximum of non-negative floats (returned wave-uniform).
__device__ __forceinline__ float wave_max_nonneg(float x) {
  // for x >= 0 the fp32 order is the order of the bit patterns as signed ints
  int v = __float_as_int(x);
  v = max(v, dpp_i<0x111>(v));
  v = max(v, dpp_i<0x112>(v));
  v = max(v, dpp_i<0x114>(v));
  v = max(v, dpp_i<0x118>(v));
  v = max(v, dpp_i<0x142, 0xA>(v));
  v = max(v, dpp_i<0x143, 0xC>(v));
  return __int_as_float(__builtin_amdgcn_readlane(v, 63));
}
// Bitwise OR over each group of 8 consecutive lanes (result in all 8 lanes):
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], then row_half_mirror.
__device__ __forceinline__ uint32_t or8(uint32_t v) {
  v |= (uint32_t)dpp_i<0xB1>((int)v);
  v |= (uint32_t)dpp_i<0x4E>((int)v);
  v |= (uint32_t)dpp_i<0x141>((int)v);
  return v;
}

// Wave-wide sums, returned as wave-uniform values.
__device__ __forceinline__ float wave_sum(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_incl_scan_f(v)), 63));
}
__device__ __forceinline__ int wave_sum_i(int v) {
  return __builtin_amdgcn_readlane(wave_incl_scan(v), 63);
}
__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

}  // namespace packkv
