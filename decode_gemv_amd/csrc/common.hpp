// Shared device and host helpers of the packkv library (gfx950 / CDNA4).
//
// Record layout (one block of B tokens of one stream), from the PackKV
// pipeline of quantise -> reorder tokens -> lossless channel-direction
// bit-packing (Fig. 2 caption; TL;DR):
//   K: scale[D] f16 | zero[D] f16 | hdr[nr][D] | pad16 | payload | pad16
//   V: scale[B] f16 | zero[B] f16 | hdr[nr][D] | pad16 | payload | pad16
// hdr per (run, channel): the byte (w << 4) | m for b <= 4, the
// little-endian u16 (w << 8) | m for b = 5..8 (m needs the whole byte);
// payload = for run r, channel c: w little-endian u32 words, slot i of the
// run in bits [i*w, i*w + w).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "packkv.h"

namespace packkv {

constexpr int kD = 128;        // head_dim
constexpr int kR = 32;         // run length (slots)
constexpr int kWave = 64;      // CDNA wavefront

__host__ __device__ constexpr int pad16(int x) { return (x + 15) & ~15; }
__host__ __device__ constexpr int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }

// Geometry of a record holding n tokens (nr runs) of a block of B tokens.
__host__ __device__ constexpr int n_params(bool is_v, int B) { return is_v ? B : kD; }
__host__ __device__ constexpr int hdr_offset(bool is_v, int B) { return 4 * n_params(is_v, B); }
__host__ __device__ constexpr int hdr_entry_bytes(int bits) { return bits > 4 ? 2 : 1; }
__host__ __device__ constexpr int payload_offset(bool is_v, int B, int nr, int hb = 1) {
  return pad16(4 * n_params(is_v, B) + hb * nr * kD);
}
__host__ __device__ constexpr int max_record_bytes(bool is_v, int B, int bits) {
  return payload_offset(is_v, B, B / kR, hdr_entry_bytes(bits)) + 4 * (B / kR) * kD * bits;
}

// ---------------------------------------------------------------------------
// fp16 bit helpers (exact).
__device__ __forceinline__ float f16_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);   // v_cvt_f32_f16, exact
}
__device__ __forceinline__ double f16_bits_to_double(uint32_t h) {
  return (double)f16_bits_to_float(h);                        // both conversions exact
}

// ---------------------------------------------------------------------------
// Spread the fields of one 8-slot group into eight 4-bit nibbles.
// Input: the group's 8*w bits at the bottom of x.  Output: nibble i = field i.
__device__ __forceinline__ uint32_t spread3to4(uint32_t x) {
  uint32_t a = (x & 0xFFFu) | ((x & 0xFFF000u) << 4);
  uint32_t b = (a & 0x003F003Fu) | ((a & 0x0FC00FC0u) << 2);
  return (b & 0x07070707u) | ((b & 0x38383838u) << 1);
}
// 2-bit fields: the 8 fields of bytes 2H and 2H+1 of x.  v_perm puts the
// two bytes in bytes 0 and 2, then two shift-or-mask steps split each byte
// into its nibbles and each nibble into its two fields.
template <int H>
__device__ __forceinline__ uint32_t spread2to4(uint32_t x) {
  const uint32_t a = __builtin_amdgcn_perm(0u, x, H ? 0x0c030c02u : 0x0c010c00u);
  const uint32_t b = (a | (a << 4)) & 0x0F0F0F0Fu;
  return (b | (b << 2)) & 0x33333333u;
}
__device__ __forceinline__ uint32_t spread1to4(uint32_t x) {
  uint32_t a = (x & 0xFu) | ((x & 0xF0u) << 12);
  uint32_t b = (a & 0x00030003u) | ((a & 0x000C000Cu) << 6);
  return (b & 0x01010101u) | ((b & 0x02020202u) << 3);
}

// 32 bits of the run's bit string starting at bit p (p a compile-time
// multiple of 8 inside a switch), from its words w0..w3.
template <int P>
__device__ __forceinline__ uint32_t bits_at(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  constexpr int wi = P >> 5, sh = P & 31;
  uint32_t lo = wi == 0 ? w0 : wi == 1 ? w1 : wi == 2 ? w2 : w3;
  uint32_t hi = wi == 0 ? w1 : wi == 1 ? w2 : wi == 2 ? w3 : 0u;
  if constexpr (sh == 0) return lo;
  else return __builtin_amdgcn_alignbit(hi, lo, sh);
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

// Decode one run (R = 32 slots) stored at width w with minimum m into four
// nibble words: word k holds q = m + u of slots 8k .. 8k+7 (nibble i = slot
// 8k+i).  Valid for m + 2^w - 1 <= 15.  `wd` holds the run's first four
// payload words (words past the run are ignored).
template <int WMAX = 4>
__device__ __forceinline__ void run_to_nibbles(int w, uint32_t m, const uint32_t wd[4], uint32_t out[4]) {
  const uint32_t a = wd[0], b = wd[1], c = wd[2], d = wd[3];
  // widths above WMAX do not occur at the call site; the widest one that
  // does is tested first
  if (WMAX >= 4 && w == 4) {
    out[0] = a; out[1] = b; out[2] = c; out[3] = d;
  } else if (WMAX >= 3 && w == 3) {
    out[0] = spread3to4(bits_at<0>(a, b, c, d));
    out[1] = spread3to4(bits_at<24>(a, b, c, d));
    out[2] = spread3to4(bits_at<48>(a, b, c, d));
    out[3] = spread3to4(bits_at<72>(a, b, c, d));
  } else if (WMAX >= 2 && w == 2) {
    out[0] = spread2to4<0>(a);
    out[1] = spread2to4<1>(a);
    out[2] = spread2to4<0>(b);
    out[3] = spread2to4<1>(b);
  } else if (w == 1) {
    out[0] = spread1to4(a);
    out[1] = spread1to4(a >> 8);
    out[2] = spread1to4(a >> 16);
    out[3] = spread1to4(a >> 24);
  } else {
    out[0] = out[1] = out[2] = out[3] = 0u;
  }
  const uint32_t mm = nibble_splat(m);   // m in every nibble; no carries
  out[0] += mm; out[1] += mm; out[2] += mm; out[3] += mm;
}

// A run stored at the full width BITS: its BITS words -> four container words.
template <int BITS>
__device__ __forceinline__ void full_to_nibbles(const uint32_t wd[4], uint32_t out[4]) {
  if constexpr (BITS == 4) {
    out[0] = wd[0]; out[1] = wd[1]; out[2] = wd[2]; out[3] = wd[3];
  } else if constexpr (BITS == 3) {
    out[0] = spread3to4(bits_at<0>(wd[0], wd[1], wd[2], 0u));
    out[1] = spread3to4(bits_at<24>(wd[0], wd[1], wd[2], 0u));
    out[2] = spread3to4(bits_at<48>(wd[0], wd[1], wd[2], 0u));
    out[3] = spread3to4(bits_at<72>(wd[0], wd[1], wd[2], 0u));
  } else {
    out[0] = spread2to4<0>(wd[0]);
    out[1] = spread2to4<1>(wd[0]);
    out[2] = spread2to4<0>(wd[1]);
    out[3] = spread2to4<1>(wd[1]);
  }
}

// Four header bytes (w << 4 | m) of runs that are all at the full width BITS
// with a consistent minimum (m + 2^(BITS-1) <= 2^BITS - 1): SWAR test.
template <int BITS>
__device__ __forceinline__ bool hdr4_full(uint32_t x) {
  constexpr uint32_t want = (uint32_t)BITS * 0x10101010u;
  constexpr uint32_t mbad = (0x0Fu & ~((1u << (BITS - 1)) - 1u)) * 0x01010101u;
  return ((x ^ want) & (0xF0F0F0F0u | mbad)) == 0u;
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
