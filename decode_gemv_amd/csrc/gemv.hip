// Fused decompress + GEMV kernels for the packed KV cache (gfx950).
//
// PackKV integrates decompression into the decode-time matrix-vector
// products so that no decompressed tensor is written back (TL;DR; Fig. 2
// caption: "computation-aware decompression + matrix-vector multiplication").
// Dequantisation x_hat = zero + scale * q is folded onto the dense operand:
//   K:  scores[t] = sum_c q[c] zero[c] + sum_c (q[c] scale[c]) * qint[t][c]
//   V:  out[c]    = sum_t p[t] zero[t] + sum_t (p[t] scale[t]) * qint[t][c]
// so the inner loop is: unpack ints -> convert -> one fp32 FMA per element.
//
// One wavefront per workgroup.  A workgroup owns a contiguous range of blocks
// of one stream.  Per block:
//   1. the record (<= 9.2 KB) is streamed into LDS with coalesced 16-byte
//      loads; the next block's record is already in flight in registers;
//   2. lane l owns runs l, l+64, ...: it reads their header bytes, and a wave
//      prefix sum of the widths gives every run's payload word offset;
//   3. each run is decoded (any width 0..4) into four words of 4-bit
//      containers q = m + u (slots 8k..8k+7 in word k);
//   4. K: the containers go to an LDS plane [slot group][channel] and every
//      lane reduces 16 channels for 8 slots; V: each lane accumulates its own
//      channels over the run's 32 slots directly from registers.
// Integers become floats through v_cvt_pk_f32_fp8 (two per instruction): a
// byte n <= 15 read as an fp8 e4m3 number is exactly n * c for a power of two
// c, and 1/c is folded into the dense operand.
#include "kernels.hpp"

namespace packkv {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float fp8_unit() {
  // value of the e4m3 byte 0x01; every byte n <= 15 converts to exactly n * unit
  f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8(1u, false);
  return v.x;
}

// 8 slot values of one container word: f[i] = nibble i * unit.
__device__ __forceinline__ void nibbles_to_f32(uint32_t w, float f[8]) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  f[0] = a.x; f[2] = a.y; f[4] = b.x; f[6] = b.y;
  f[1] = c.x; f[3] = c.y; f[5] = d.x; f[7] = d.y;
}

// A record is usable only if it lies inside its stream region and fits the
// staging buffer; corrupt offsets must never turn into wild loads.
__device__ __forceinline__ bool record_ok(uint32_t o, uint32_t size, uint64_t stride, int rec_max) {
  return size >= 16u && size <= (uint32_t)rec_max && (uint64_t)o + size <= stride;
}

// Record staging: chunks of 16 bytes, lane l takes chunks l, l+64, ...
template <int NCH>
__device__ __forceinline__ void load_record(const uint8_t* g, uint32_t bytes, int lane, u32x4 pre[NCH]) {
  const u32x4* src = reinterpret_cast<const u32x4*>(g);
  const int nch = (int)(bytes >> 4);
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int c = lane + 64 * k;
    if (c < nch) pre[k] = __builtin_nontemporal_load(src + c);
  }
}
template <int NCH>
__device__ __forceinline__ void store_record(uint8_t* lds, uint32_t bytes, int lane, const u32x4 pre[NCH]) {
  u32x4* dst = reinterpret_cast<u32x4*>(lds);
  const int nch = (int)(bytes >> 4);
#pragma unroll
  for (int k = 0; k < NCH; ++k) {
    const int c = lane + 64 * k;
    if (c < nch) dst[c] = pre[k];
  }
}

// Header decode + width scan for the lane's runs (NRL runs per lane, run
// index l + 64k).  Returns false if the record is inconsistent.
template <int NRL>
__device__ __forceinline__ bool scan_runs(const uint8_t* rec, int hdr_off, int pay_off, uint32_t size,
                                          int nruns, int bits, int lane,
                                          int w[NRL], uint32_t m[NRL], uint32_t off[NRL]) {
  const int L = (1 << bits) - 1;
  int bad = 0;
  uint32_t base = 0;
#pragma unroll
  for (int k = 0; k < NRL; ++k) {
    const int ri = lane + 64 * k;
    uint32_t h = ri < nruns ? rec[hdr_off + ri] : 0u;
    w[k] = (int)(h >> 4);
    m[k] = h & 15u;
    // a valid run has max - m in [2^(w-1), 2^w - 1] and max <= L
    bad |= (w[k] > bits) | ((int)m[k] > L) | (w[k] > 0 && (int)m[k] + (1 << (w[k] - 1)) > L);
    const int incl = wave_incl_scan(w[k], lane);
    off[k] = base + (uint32_t)(incl - w[k]);
    base += (uint32_t)__shfl(incl, 63, kWave);
  }
  bad = wave_sum_i(bad);
  return bad == 0 && (uint32_t)pad16(pay_off + 4 * (int)base) == size;
}

// Read the first four payload words of a run from LDS (may run past the run
// into padding; the staging buffer has 16 bytes of slack).
__device__ __forceinline__ void run_words(const uint8_t* rec, int pay_off, uint32_t off, uint32_t wd[4]) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(rec + pay_off) + off;
  wd[0] = p[0]; wd[1] = p[1]; wd[2] = p[2]; wd[3] = p[3];
}

// ---------------------------------------------------------------------------
// K side.
template <int B, int GT>
__global__ __launch_bounds__(64) void k_qk_gemv(GemvArgs a) {
  constexpr int NR = B / kR;                       // runs per block
  constexpr int NRL = NR * kD / 64;                // runs per lane
  constexpr int REC = max_record_bytes(false, B, 4);
  constexpr int NCH = (REC + 1023) / 1024;
  constexpr int ROWW = kD + 4;                     // plane row: 128 words + 16 B pad
  constexpr int HDR = hdr_offset(false, B);
  constexpr int REDB = GT * 64 * 9 * 4;            // channel-group reduction
  constexpr int BUF = (REC + 16) > REDB ? (REC + 16) : REDB;
  __shared__ __attribute__((aligned(16))) uint8_t rec[BUF];
  __shared__ __attribute__((aligned(16))) uint32_t plane[(B / 8) * ROWW];
  __shared__ __attribute__((aligned(16))) float qs[GT * kD];
  float* red = reinterpret_cast<float*>(rec);      // reuses the staging buffer

  const int lane = threadIdx.x;
  const int s = blockIdx.x / a.splits;
  const int split = blockIdx.x % a.splits;
  const int j0 = split * a.blocks_per_wg;
  const int j1 = min(a.nb, j0 + a.blocks_per_wg);
  if (j0 >= j1) return;
  const uint8_t* arena = a.arena + (uint64_t)s * a.arena_stride;
  const uint32_t* offs = a.off + (int64_t)s * a.off_stride;
  const float unit_inv = 1.0f / fp8_unit();

  // offsets of this workgroup's records: lane i holds off[j0 + i]
  const int nj = j1 - j0;
  uint32_t my_off = lane <= nj ? offs[j0 + lane] : 0u;
  uint32_t my_off2 = lane + 64 <= nj ? offs[j0 + 64 + lane] : 0u;
  auto off_of = [&](int i) -> uint32_t {
    return i < 64 ? (uint32_t)__shfl((int)my_off, i, kWave) : (uint32_t)__shfl((int)my_off2, i - 64, kWave);
  };

  const int g8 = lane & 7, cg = lane >> 3;

  for (int gq0 = 0; gq0 < a.G; gq0 += GT) {
    // queries for the channels this lane stages (c = lane, lane + 64)
    float qa[GT], qb[GT];
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const bool ok = gq0 + g < a.G;
      const uint16_t* qp = a.q + ((int64_t)s * a.G + gq0 + g) * kD;
      qa[g] = ok ? f16_bits_to_float(qp[lane]) : 0.f;
      qb[g] = ok ? f16_bits_to_float(qp[lane + 64]) : 0.f;
    }
    u32x4 pre[NCH];
    {
      const uint32_t o0 = off_of(0), s0 = off_of(1) - o0;
      if (record_ok(o0, s0, a.arena_stride, REC)) load_record<NCH>(arena + o0, s0, lane, pre);
    }
    for (int jj = 0; jj < nj; ++jj) {
      const int j = j0 + jj;
      const uint32_t o = off_of(jj), size = off_of(jj + 1) - o;
      const int n = (int)imin64(B, a.n_tokens - (int64_t)j * B);
      const int nr = (n + kR - 1) / kR;
      __syncthreads();
      if (!record_ok(o, size, a.arena_stride, REC)) {
        if (lane == 0) latch(a.status, PACKKV_ECORRUPT);
        break;
      }
      store_record<NCH>(rec, size, lane, pre);
      if (jj + 1 < nj) {
        const uint32_t o1 = off_of(jj + 1), s1 = off_of(jj + 2) - o1;
        if (record_ok(o1, s1, a.arena_stride, REC)) load_record<NCH>(arena + o1, s1, lane, pre);
      }
      __syncthreads();

      const int pay = payload_offset(false, B, nr);
      int w[NRL];
      uint32_t m[NRL], ro[NRL];
      if (!scan_runs<NRL>(rec, HDR, pay, size, nr * kD, a.bits, lane, w, m, ro)) {
        if (lane == 0) latch(a.status, PACKKV_ECORRUPT);
        continue;
      }
      // decode every run of the lane into the container plane
#pragma unroll
      for (int k = 0; k < NRL; ++k) {
        const int ri = lane + 64 * k;
        const int r = ri / kD, c = ri % kD;
        uint32_t wd[4], nib[4];
        if (r < nr) {
          run_words(rec, pay, ro[k], wd);
          run_to_nibbles(w[k], m[k], wd, nib);
        } else {
          nib[0] = nib[1] = nib[2] = nib[3] = 0u;
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) plane[(r * 4 + kk) * ROWW + c] = nib[kk];
      }
      // q' = q * scale (per channel), beta = q . zero
      float beta[GT];
      {
        const uint16_t* sc = reinterpret_cast<const uint16_t*>(rec);
        const float sa = f16_bits_to_float(sc[lane]), sb = f16_bits_to_float(sc[lane + 64]);
        const float za = f16_bits_to_float(sc[kD + lane]), zb = f16_bits_to_float(sc[kD + lane + 64]);
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          qs[g * kD + lane] = qa[g] * sa * unit_inv;
          qs[g * kD + lane + 64] = qb[g] * sb * unit_inv;
          beta[g] = wave_sum(qa[g] * za + qb[g] * zb);
        }
      }
      __syncthreads();

      // container plane x q': lane (g8, cg) covers slot group g8 of a 64-slot
      // half and channels cg*16 .. cg*16+15
#pragma unroll
      for (int h = 0; h < B / 64; ++h) {
        float acc[GT][8];
#pragma unroll
        for (int g = 0; g < GT; ++g)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[g][i] = 0.f;
        const int row = h * 8 + g8;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int c0 = cg * 16 + i4 * 4;
          const uint4 nw = *reinterpret_cast<const uint4*>(&plane[row * ROWW + c0]);
          const uint32_t words[4] = {nw.x, nw.y, nw.z, nw.w};
          float qq[GT][4];
#pragma unroll
          for (int g = 0; g < GT; ++g) {
            const float4 t = *reinterpret_cast<const float4*>(&qs[g * kD + c0]);
            qq[g][0] = t.x; qq[g][1] = t.y; qq[g][2] = t.z; qq[g][3] = t.w;
          }
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            float f[8];
            nibbles_to_f32(words[cc], f);
#pragma unroll
            for (int g = 0; g < GT; ++g)
#pragma unroll
              for (int i = 0; i < 8; ++i) acc[g][i] = fmaf(qq[g][cc], f[i], acc[g][i]);
          }
        }
        // reduce the 8 channel groups: red[g][slot][cg], slot = g8*8 + i
        __syncthreads();
#pragma unroll
        for (int g = 0; g < GT; ++g)
#pragma unroll
          for (int i = 0; i < 8; ++i) red[(g * 64 + g8 * 8 + i) * 9 + cg] = acc[g][i];
        __syncthreads();
        const int64_t t = (int64_t)j * B + h * 64 + lane;
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          float sum = beta[g];
#pragma unroll
          for (int u = 0; u < 8; ++u) sum += red[(g * 64 + lane) * 9 + u];
          if (gq0 + g < a.G && h * 64 + lane < n)
            a.scores[((int64_t)s * a.G + gq0 + g) * a.ld + t] = sum;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// V side: split-T partial sums into ws, then a fixed-order reduction.
template <int B, int GT>
__global__ __launch_bounds__(64) void k_pv_gemv(GemvArgs a) {
  constexpr int NR = B / kR;
  constexpr int NRL = NR * kD / 64;
  constexpr int REC = max_record_bytes(true, B, 4);
  constexpr int NCH = (REC + 1023) / 1024;
  constexpr int HDR = hdr_offset(true, B);
  __shared__ __attribute__((aligned(16))) uint8_t rec[REC + 16];
  __shared__ __attribute__((aligned(16))) float pp[GT * B];

  const int lane = threadIdx.x;
  const int s = blockIdx.x / a.splits;
  const int split = blockIdx.x % a.splits;
  const int j0 = split * a.blocks_per_wg;
  const int j1 = min(a.nb, j0 + a.blocks_per_wg);
  const uint8_t* arena = a.arena + (uint64_t)s * a.arena_stride;
  const uint32_t* offs = a.off + (int64_t)s * a.off_stride;
  const float unit_inv = 1.0f / fp8_unit();
  const int nj = max(0, j1 - j0);
  uint32_t my_off = lane <= nj ? offs[j0 + lane] : 0u;
  uint32_t my_off2 = lane + 64 <= nj ? offs[j0 + 64 + lane] : 0u;
  auto off_of = [&](int i) -> uint32_t {
    return i < 64 ? (uint32_t)__shfl((int)my_off, i, kWave) : (uint32_t)__shfl((int)my_off2, i - 64, kWave);
  };

  for (int gq0 = 0; gq0 < a.G; gq0 += GT) {
    float acc[GT][2];
    float pz[GT];
#pragma unroll
    for (int g = 0; g < GT; ++g) { acc[g][0] = acc[g][1] = 0.f; pz[g] = 0.f; }
    u32x4 pre[NCH];
    if (nj > 0) {
      const uint32_t o0 = off_of(0), s0 = off_of(1) - o0;
      if (record_ok(o0, s0, a.arena_stride, REC)) load_record<NCH>(arena + o0, s0, lane, pre);
    }
    for (int jj = 0; jj < nj; ++jj) {
      const int j = j0 + jj;
      const uint32_t o = off_of(jj), size = off_of(jj + 1) - o;
      const int n = (int)imin64(B, a.n_tokens - (int64_t)j * B);
      const int nr = (n + kR - 1) / kR;
      __syncthreads();
      if (!record_ok(o, size, a.arena_stride, REC)) {
        if (lane == 0) latch(a.status, PACKKV_ECORRUPT);
        break;
      }
      store_record<NCH>(rec, size, lane, pre);
      if (jj + 1 < nj) {
        const uint32_t o1 = off_of(jj + 1), s1 = off_of(jj + 2) - o1;
        if (record_ok(o1, s1, a.arena_stride, REC)) load_record<NCH>(arena + o1, s1, lane, pre);
      }
      __syncthreads();
      // p' = p * scale per slot; sum p * zero
      {
        const uint16_t* sc = reinterpret_cast<const uint16_t*>(rec);
#pragma unroll
        for (int h = 0; h < B / 64; ++h) {
          const int sl = h * 64 + lane;
#pragma unroll
          for (int g = 0; g < GT; ++g) {
            float pv = 0.f;
            if (sl < n && gq0 + g < a.G)
              pv = a.p[((int64_t)s * a.G + gq0 + g) * a.ld + (int64_t)j * B + sl];
            pp[g * B + sl] = pv * f16_bits_to_float(sc[sl]) * unit_inv;
            pz[g] = fmaf(pv, f16_bits_to_float(sc[B + sl]), pz[g]);
          }
        }
      }
      __syncthreads();
      const int pay = payload_offset(true, B, nr);
      int w[NRL];
      uint32_t m[NRL], ro[NRL];
      if (!scan_runs<NRL>(rec, HDR, pay, size, nr * kD, a.bits, lane, w, m, ro)) {
        if (lane == 0) latch(a.status, PACKKV_ECORRUPT);
        continue;
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if (r >= nr) break;
        float pr[GT][32];
#pragma unroll
        for (int g = 0; g < GT; ++g)
#pragma unroll
          for (int i = 0; i < 32; i += 4) {
            const float4 t = *reinterpret_cast<const float4*>(&pp[g * B + r * 32 + i]);
            pr[g][i] = t.x; pr[g][i + 1] = t.y; pr[g][i + 2] = t.z; pr[g][i + 3] = t.w;
          }
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
          const int k = r * 2 + ch;            // run index lane + 64k = r*128 + ch*64 + lane
          uint32_t wd[4], nib[4];
          run_words(rec, pay, ro[k], wd);
          run_to_nibbles(w[k], m[k], wd, nib);
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            float f[8];
            nibbles_to_f32(nib[kk], f);
#pragma unroll
            for (int g = 0; g < GT; ++g)
#pragma unroll
              for (int i = 0; i < 8; ++i) acc[g][ch] = fmaf(pr[g][kk * 8 + i], f[i], acc[g][ch]);
          }
        }
      }
    }
    // partial result of this split
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float z = wave_sum(pz[g]);
      if (gq0 + g < a.G) {
        float* dst = a.ws + (((int64_t)s * a.G + gq0 + g) * a.splits + split) * kD;
        dst[lane] = acc[g][0] + z;
        dst[lane + 64] = acc[g][1] + z;
      }
    }
  }
}

__global__ __launch_bounds__(128) void k_pv_reduce(const float* ws, int splits, float* out) {
  const int row = blockIdx.x;          // s * G + g
  const int c = threadIdx.x;
  const float* src = ws + (int64_t)row * splits * kD + c;
  float sum = 0.f;
  for (int i = 0; i < splits; ++i) sum += src[(int64_t)i * kD];
  out[(int64_t)row * kD + c] = sum;
}

// ---------------------------------------------------------------------------
// Decompress (test path): mode 0 -> u8 q in slot order, mode 1 -> fp32 x_hat
// in token order.
template <int B, bool IS_V>
__global__ __launch_bounds__(64) void k_decompress(GemvArgs a, const uint8_t* perm, int64_t perm_stride,
                                                   int mode, void* out) {
  constexpr int NR = B / kR;
  constexpr int NRL = NR * kD / 64;
  constexpr int REC = max_record_bytes(IS_V, B, 4);
  constexpr int NCH = (REC + 1023) / 1024;
  constexpr int HDR = hdr_offset(IS_V, B);
  __shared__ __attribute__((aligned(16))) uint8_t rec[REC + 16];
  const int lane = threadIdx.x;
  const int s = blockIdx.y, j = blockIdx.x;
  const uint8_t* arena = a.arena + (uint64_t)s * a.arena_stride;
  const uint32_t* offs = a.off + (int64_t)s * a.off_stride;
  const uint32_t o = offs[j], size = offs[j + 1] - o;
  const int n = (int)imin64(B, a.n_tokens - (int64_t)j * B);
  const int nr = (n + kR - 1) / kR;
  if (!record_ok(o, size, a.arena_stride, REC)) {
    if (lane == 0) latch(a.status, PACKKV_ECORRUPT);
    return;
  }
  u32x4 pre[NCH];
  load_record<NCH>(arena + o, size, lane, pre);
  store_record<NCH>(rec, size, lane, pre);
  __syncthreads();
  const int pay = payload_offset(IS_V, B, nr);
  int w[NRL];
  uint32_t m[NRL], ro[NRL];
  if (!scan_runs<NRL>(rec, HDR, pay, size, nr * kD, a.bits, lane, w, m, ro)) {
    if (lane == 0) latch(a.status, PACKKV_ECORRUPT);
    return;
  }
  const uint16_t* sc = reinterpret_cast<const uint16_t*>(rec);
  const uint8_t* pm = perm + (int64_t)s * perm_stride + (int64_t)j * B;
#pragma unroll
  for (int k = 0; k < NRL; ++k) {
    const int ri = lane + 64 * k;
    const int r = ri / kD, c = ri % kD;
    if (r >= nr) continue;
    uint32_t wd[4], nib[4];
    run_words(rec, pay, ro[k], wd);
    run_to_nibbles(w[k], m[k], wd, nib);
    for (int i = 0; i < kR; ++i) {
      const int sl = r * kR + i;
      if (sl >= n) break;
      const uint32_t qv = (nib[i >> 3] >> (4 * (i & 7))) & 15u;
      if (mode == 0) {
        uint8_t* o8 = reinterpret_cast<uint8_t*>(out);
        o8[(((int64_t)s * a.n_tokens) + (int64_t)j * B + sl) * kD + c] = (uint8_t)qv;
      } else {
        const float scale = f16_bits_to_float(IS_V ? sc[sl] : sc[c]);
        const float zero = f16_bits_to_float(IS_V ? sc[B + sl] : sc[kD + c]);
        float* of = reinterpret_cast<float*>(out);
        const int tok = pm[sl];
        if (tok >= n) {
          latch(a.status, PACKKV_ECORRUPT);
          continue;
        }
        const int64_t t = (int64_t)j * B + tok;
        of[((int64_t)s * a.n_tokens + t) * kD + c] = fmaf(scale, (float)qv, zero);
      }
    }
  }
}

// Width histogram and byte counts.
template <int B, bool IS_V>
__global__ __launch_bounds__(64) void k_stats(GemvArgs a, unsigned long long* out) {
  constexpr int NR = B / kR;
  const int lane = threadIdx.x;
  const int s = blockIdx.y, j = blockIdx.x;
  const uint8_t* arena = a.arena + (uint64_t)s * a.arena_stride;
  const uint32_t* offs = a.off + (int64_t)s * a.off_stride;
  const uint32_t o = offs[j], size = offs[j + 1] - o;
  const int n = (int)imin64(B, a.n_tokens - (int64_t)j * B);
  const int nr = (n + kR - 1) / kR;
  if (!record_ok(o, size, a.arena_stride, max_record_bytes(IS_V, B, 4))) {
    if (lane == 0) latch(a.status, PACKKV_ECORRUPT);
    return;
  }
  const uint8_t* hdr = arena + o + hdr_offset(IS_V, B);
  unsigned long long hist[5] = {0, 0, 0, 0, 0};
  unsigned long long words = 0;
  for (int ri = lane; ri < nr * kD; ri += 64) {
    const int w = hdr[ri] >> 4;
    if (w <= 4) hist[w]++;
    words += (unsigned long long)w;
  }
  const int base = IS_V ? 5 : 0;
  for (int i = 0; i < 5; ++i)
    if (hist[i]) atomicAdd(&out[base + i], hist[i]);
  if (words) atomicAdd(&out[IS_V ? 13 : 12], words);
  if (lane == 0) {
    atomicAdd(&out[IS_V ? 11 : 10], (unsigned long long)size);
    atomicAdd(&out[IS_V ? 15 : 14], (unsigned long long)(nr * kD));
  }
  (void)NR;
}

// Softmax over the first T entries of each row: p = exp(s*scale - max)/sum.
__global__ __launch_bounds__(256) void k_softmax(const float* scores, float* p, int64_t T, int64_t ld,
                                                 float scale) {
  __shared__ float red[8];
  const float* x = scores + (int64_t)blockIdx.x * ld;
  float* y = p + (int64_t)blockIdx.x * ld;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  float mx = -INFINITY;
  for (int64_t i = tid; i < T; i += 256) mx = fmaxf(mx, x[i] * scale);
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  if (lane == 0) red[wv] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float sum = 0.f;
  for (int64_t i = tid; i < T; i += 256) sum += expf(x[i] * scale - mx);
  sum = wave_sum(sum);
  if (lane == 0) red[4 + wv] = sum;
  __syncthreads();
  const float inv = 1.0f / ((red[4] + red[5]) + (red[6] + red[7]));
  for (int64_t i = tid; i < T; i += 256) y[i] = expf(x[i] * scale - mx) * inv;
}

// ---------------------------------------------------------------------------
// Launchers.
template <int B>
static hipError_t qk_dispatch(const GemvArgs& a, int n_streams, hipStream_t st) {
  dim3 grid(n_streams * a.splits), block(64);
  if (a.G == 1) hipLaunchKernelGGL((k_qk_gemv<B, 1>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((k_qk_gemv<B, 4>), grid, block, 0, st, a);
  return hipGetLastError();
}
hipError_t launch_qk(const GemvArgs& a, int B, int n_streams, hipStream_t st) {
  return B == 64 ? qk_dispatch<64>(a, n_streams, st) : qk_dispatch<128>(a, n_streams, st);
}

template <int B>
static hipError_t pv_dispatch(const GemvArgs& a, int n_streams, hipStream_t st) {
  dim3 grid(n_streams * a.splits), block(64);
  if (a.G == 1) hipLaunchKernelGGL((k_pv_gemv<B, 1>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((k_pv_gemv<B, 4>), grid, block, 0, st, a);
  return hipGetLastError();
}
hipError_t launch_pv(const GemvArgs& a, int B, int n_streams, float* out, hipStream_t st) {
  hipError_t e = B == 64 ? pv_dispatch<64>(a, n_streams, st) : pv_dispatch<128>(a, n_streams, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_pv_reduce, dim3(n_streams * a.G), dim3(128), 0, st, a.ws, a.splits, out);
  return hipGetLastError();
}

hipError_t launch_decompress(const GemvArgs& a, int B, bool is_v, int n_streams, const uint8_t* perm,
                             int64_t perm_stride, int mode, void* out, hipStream_t st) {
  dim3 grid(a.nb, n_streams), block(64);
  if (B == 64) {
    if (is_v) hipLaunchKernelGGL((k_decompress<64, true>), grid, block, 0, st, a, perm, perm_stride, mode, out);
    else hipLaunchKernelGGL((k_decompress<64, false>), grid, block, 0, st, a, perm, perm_stride, mode, out);
  } else {
    if (is_v) hipLaunchKernelGGL((k_decompress<128, true>), grid, block, 0, st, a, perm, perm_stride, mode, out);
    else hipLaunchKernelGGL((k_decompress<128, false>), grid, block, 0, st, a, perm, perm_stride, mode, out);
  }
  return hipGetLastError();
}

hipError_t launch_stats(const GemvArgs& a, int B, bool is_v, int n_streams, unsigned long long* out,
                        hipStream_t st) {
  dim3 grid(a.nb, n_streams), block(64);
  if (B == 64) {
    if (is_v) hipLaunchKernelGGL((k_stats<64, true>), grid, block, 0, st, a, out);
    else hipLaunchKernelGGL((k_stats<64, false>), grid, block, 0, st, a, out);
  } else {
    if (is_v) hipLaunchKernelGGL((k_stats<128, true>), grid, block, 0, st, a, out);
    else hipLaunchKernelGGL((k_stats<128, false>), grid, block, 0, st, a, out);
  }
  return hipGetLastError();
}

hipError_t launch_softmax(const float* scores, float* p, int rows, int64_t T, int64_t ld, float scale,
                          hipStream_t st) {
  hipLaunchKernelGGL(k_softmax, dim3(rows), dim3(256), 0, st, scores, p, T, ld, scale);
  return hipGetLastError();
}

}  // namespace packkv
