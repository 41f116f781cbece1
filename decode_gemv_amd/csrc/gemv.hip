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
// Integers become floats exactly, with the conversion's power of two folded
// into the dense operand: at 2 bits each byte of a container word goes
// through one fp4 pair conversion (the e2m1 codes 0..4 are exact multiples
// of their step); at 3 and 4 bits nibbles masked into 16-bit halves are fp16
// subnormals that the mixed-precision FMA reads as they stand; bytes of the
// wide (5..8-bit) containers convert one at a time.
#include <atomic>
#include <type_traits>

#include "kernels.hpp"

namespace packkv {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// LDS ordering inside one wave: wait for the wave's LDS accesses and keep
// the compiler from moving memory operations across.  Unlike __syncthreads
// it involves no other wave, so waves of one workgroup may run different
// code between their workgroup barriers.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Value of the e2m1 (fp4) code 1.  Up to 2 bits a container nibble holds
// at most 4 in any record whose header passes the checks (m + 2^(w-1) <= 3
// bounds m + 2^w - 1 by 4), and the fp4 codes 0..4 are exactly 0, 1, 2, 3, 4
// times it, so such a nibble converts as it stands.
__device__ __forceinline__ float fp4_unit() {
  f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(1u, 1.0f, 0);
  return v.x;
}

// 8 slot values of one container word (2-bit runs): f[i] = nibble i *
// fp4_unit, each byte (two nibbles) one fp4 pair conversion.
__device__ __forceinline__ void nibbles_to_f32_fp4(uint32_t w, float f[8]) {
  const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  f[0] = a.x; f[1] = a.y; f[2] = b.x; f[3] = b.y;
  f[4] = c.x; f[5] = c.y; f[6] = d.x; f[7] = d.y;
}

// A record is usable only if it lies inside its stream region and fits the
// staging buffer; corrupt offsets must never turn into wild loads.
__device__ __forceinline__ bool record_ok(uint64_t o, uint32_t size, uint64_t stride, int rec_max) {
  return size >= 16u && size <= (uint32_t)rec_max && o + size <= stride;
}

// Raw buffer resource over [base, base + bytes): the hardware range check
// turns every load at or past `bytes` into zero without a memory access, so
// loads can be issued unconditionally (bytes = 0 for "nothing to load") and
// the compiler can count outstanding loads exactly instead of draining them.
constexpr int kBufferFormat = 0x00020000;          // 32-bit data format
constexpr int kNonTemporal = 2;
constexpr int kCoherent = 16;     // sc1: agent-coherent, as relaxed agent-scope atomics
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferFormat);
}

// Record staging: chunks of 16 bytes, lane l takes chunks l, l+64, ...
// Chunks past `bytes` (a multiple of 16) read as zero.
template <int NCH>
__device__ __forceinline__ void load_record(const uint8_t* g, uint32_t bytes, int lane, u32x4 pre[NCH]) {
  const __amdgpu_buffer_rsrc_t r = buffer_rsrc(g, bytes);
#pragma unroll
  for (int k = 0; k < NCH; ++k)
    pre[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 16 * (lane + 64 * k), 0, kNonTemporal));
}
template <int NCH>
__device__ __forceinline__ void store_record(uint8_t* lds, const u32x4 pre[NCH], int lane) {
  u32x4* dst = reinterpret_cast<u32x4*>(lds);
#pragma unroll
  for (int k = 0; k < NCH; ++k) dst[lane + 64 * k] = pre[k];
}
// LDS staging for records of at most rec bytes: every chunk a load can bring
// (NCH x 1 KiB, stored without a bounds test) plus 16 bytes of slack that the
// decoder may read past the record's end.
__host__ __device__ constexpr int staging_bytes(int rec) {
  return ((rec + 1023) / 1024) * 1024 > rec + 16 ? ((rec + 1023) / 1024) * 1024 : rec + 16;
}

// Header decode + width scan for the lane's runs (NRL runs per lane, run
// index l + 64k, DL of them per run row of D channels).  Returns false if the
// record is inconsistent.  When every run is at full width the offsets are
// implicit and no scan is needed.  wsorted: payload order 1 (each run row by
// decreasing width, equal widths by channel).
template <int NRL, int HB = 1, int DL = 2>
__device__ __forceinline__ bool scan_runs(const uint8_t* rec, int hdr_off, int pay_off, uint32_t size,
                                          int nruns, int bits, int lane,
                                          int w[NRL], uint32_t m[NRL], uint32_t off[NRL], bool& full,
                                          bool wsorted = false) {
  const int L = (1 << bits) - 1;
  bool bad = false, narrow = false;
#pragma unroll
  for (int k = 0; k < NRL; ++k) {
    const int ri = lane + 64 * k;
    uint32_t h = 0u;
    if (ri < nruns) h = HB == 2 ? reinterpret_cast<const uint16_t*>(rec + hdr_off)[ri] : rec[hdr_off + ri];
    w[k] = (int)(HB == 2 ? h >> 8 : h >> 4);
    m[k] = HB == 2 ? h & 255u : h & 15u;
    // a valid run has max - m in [2^(w-1), 2^w - 1] and max <= L
    bad |= w[k] > bits || (int)m[k] > L || (w[k] > 0 && (int)m[k] + (1 << (w[k] - 1)) > L);
    narrow |= w[k] != bits;
  }
  if (__ballot(bad)) return false;
  uint32_t base;
  full = __ballot(narrow) == 0;
  if (full) {
#pragma unroll
    for (int k = 0; k < NRL; ++k) off[k] = (uint32_t)((lane + 64 * k) * bits);
    base = (uint32_t)(NRL * 64 * bits);
  } else if (wsorted) {
    base = 0;
    for (int r = 0; r < NRL / DL; ++r) {
      uint32_t above = 0;                               // words of the row's wider entries
      for (int j = 0; j < DL; ++j) off[r * DL + j] = base;
      for (int v = bits; v >= 1; --v) {
        uint32_t before = 0;                            // width-v entries of lower channel groups
        for (int j = 0; j < DL; ++j) {
          const int k = r * DL + j;
          const uint64_t mk = __ballot(w[k] == v);
          const uint32_t rank = before + __builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32),
                                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
          if (w[k] == v) off[k] = base + above + rank * (uint32_t)v;
          before += (uint32_t)__builtin_popcountll(mk);
        }
        above += before * (uint32_t)v;
      }
      base += above;
    }
  } else {
    base = 0;
#pragma unroll
    for (int k = 0; k < NRL; ++k) {
      const int incl = wave_incl_scan(w[k]);
      off[k] = base + (uint32_t)(incl - w[k]);
      base += (uint32_t)__builtin_amdgcn_readlane(incl, 63);
    }
  }
  return (uint32_t)pad16(pay_off + 4 * (int)base) == size;
}

// The first four payload words of a run (may run past the run into the next
// run or the padding; the staging buffer has 16 bytes of slack).  `al16`:
// the run starts on a 16-byte boundary.
__device__ __forceinline__ void run_words(const uint8_t* rec, int pay_off, uint32_t off, bool al16, uint32_t wd[4]) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(rec + pay_off) + off;
  if (al16) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
    wd[0] = v.x; wd[1] = v.y; wd[2] = v.z; wd[3] = v.w;
  } else {
    wd[0] = p[0]; wd[1] = p[1]; wd[2] = p[2]; wd[3] = p[3];
  }
}

// ---------------------------------------------------------------------------
// Shared per-block decode: header check, run offsets, container words.
//
// Fast path (uniform per wave): every run of a full block is at the full width
// BITS with a consistent minimum; offsets are then implicit and each run is
// BITS words at (run index) * BITS.  Otherwise the headers are validated one
// by one and a wave prefix sum gives the offsets.
template <int B, int BITS, bool IS_V, int D>
struct BlockDecoder {
  static constexpr int NR = B / kR;
  static constexpr int DL = D / 64;                 // runs of one block run per lane
  static constexpr int NRL = NR * DL;               // runs per lane: run l + 64k, r = k / DL
  static constexpr int HDR = hdr_offset(IS_V, B, D);
  static constexpr int HW = NR * D / 4;             // header dwords of a full block

  // Word offsets of the lane's runs in payload order 1: in run row r the
  // entries of width v follow every wider entry of the row, in channel
  // order (run k = r*DL + j holds channel lane + 64j).  Runs of width 0 get
  // the row's start (they hold no words; the reads there stay inside the
  // record).  Returns the payload's words.
  __device__ __forceinline__ static uint32_t sorted_offsets(const uint32_t h[NRL], uint32_t off[NRL]) {
    uint32_t row_base = 0;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      uint32_t above = 0;                               // words of the row's wider entries
#pragma unroll
      for (int j = 0; j < DL; ++j) off[r * DL + j] = row_base;
#pragma unroll
      for (int v = BITS; v >= 1; --v) {
        uint32_t before = 0;                            // width-v entries of lower channel groups
#pragma unroll
        for (int j = 0; j < DL; ++j) {
          const int k = r * DL + j;
          const bool mine = (int)(h[k] >> 4) == v;
          const uint64_t m = __ballot(mine);
          const uint32_t rank =
              before + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          if (mine) off[k] = row_base + above + rank * (uint32_t)v;
          before += (uint32_t)__builtin_popcountll(m);
        }
        above += before * (uint32_t)v;
      }
      row_base += above;
    }
    return row_base;
  }

  // Decode the lane's runs of the staged record into container words
  // nib[k][0..3] (run l + 64k).  Returns false if the record is inconsistent
  // (a width above BITS, a minimum that leaves no room for its width, or
  // widths that do not add up to the record size).
  // One code path for every block: offsets start from the full-width layout;
  // a block holding narrower runs (or a partial block) corrects them with
  // the width deficit of earlier runs, and its narrow runs are re-decoded at
  // the end.  Both corrections are uniform branches taken by few blocks.
  // wsorted: the K payload is in order 1 (each run row by decreasing width,
  // equal widths by channel); a row of equal widths is then laid out as in
  // order 0, so only the narrow-run branch differs.
  __device__ __forceinline__ static bool decode(const uint8_t* rec, uint32_t size, int nr, int lane,
                                                uint32_t nib[NRL][4], bool wsorted = false) {
    const int pay = payload_offset(IS_V, B, nr, 1, D);
    const int nruns = nr * D;
    uint32_t h[NRL];
    // read unconditionally (the staging always holds a full-size header) and
    // select, instead of a branch around each read; all reads are issued
    // before the first value is pinned, so they are in flight together
#pragma unroll
    for (int k = 0; k < NRL; ++k) h[k] = rec[HDR + lane + 64 * k];
#pragma unroll
    for (int k = 0; k < NRL; ++k) {
      asm volatile("" : "+v"(h[k]));
      h[k] = k / DL < nr ? h[k] : 0u;
    }
    // header dwords lane + 64i, four runs each; dwords past the record's
    // nr rows of runs read as width 0, minimum 0 (consistent, not full)
    constexpr int HWL = (HW + 63) / 64;
    uint32_t hx[HWL];
    bool full = nr == NR;
#pragma unroll
    for (int i = 0; i < HWL; ++i) {
      const int di = lane + 64 * i;
      hx[i] = 0u;
      if (HW % 64 == 0 || di < HW) {
        const uint32_t x = reinterpret_cast<const uint32_t*>(rec + HDR)[di];
        hx[i] = di < nruns / 4 ? x : 0u;
        full &= hdr4_full<BITS>(hx[i]);
      }
    }
    const bool all_full = __ballot(!full) == 0;
    uint32_t off[NRL];
#pragma unroll
    for (int k = 0; k < NRL; ++k) off[k] = (uint32_t)((lane + 64 * k) * BITS);
    uint32_t total = (uint32_t)(nruns * BITS);
    bool bad = false;
    if (!all_full) {
      // as scan_runs: a valid run has max - m in [2^(w-1), 2^w - 1] and
      // max <= L, so its containers m + u never carry into the next slot
#pragma unroll
      for (int i = 0; i < HWL; ++i) bad |= hdr4_bad<BITS>(hx[i]);
      if (!IS_V && wsorted) {
        total = sorted_offsets(h, off);
      } else {
      uint32_t running = 0;                            // deficit of earlier groups
#pragma unroll
      for (int k = 0; k < NRL; ++k) {
        const int w = (int)(h[k] >> 4);
        const int d = (lane + 64 * k) < nruns ? BITS - w : 0;
        off[k] -= running;
        const uint64_t short_runs = __ballot(d != 0);
        if (short_runs != 0) {
          if (BITS < 4 && __ballot(d > 1) == 0) {
            // deficits of 0 or 1 (the usual case below 4 bits): count the
            // lanes below (at 4 bits the extra path costs registers)
            off[k] -= __builtin_amdgcn_mbcnt_hi((uint32_t)(short_runs >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)short_runs, 0u));
            running += (uint32_t)__builtin_popcountll(short_runs);
          } else {
            const int incl = wave_incl_scan(d);
            off[k] -= (uint32_t)(incl - d);
            running += (uint32_t)__builtin_amdgcn_readlane(incl, 63);
          }
        }
      }
      total -= running;
      }
    }
    const bool ok = __ballot(bad) == 0 && (uint32_t)pad16(pay + 4 * (int)total) == size;
    // container words: all reads are issued first.  At 4 bits a run's words
    // are its container words; narrower full widths are converted after.
    auto read_run = [&](int k) __attribute__((always_inline)) -> u32x4 {
      if (all_full && BITS != 3) {
        // runs of 4 (2) words at a 16 (8) byte aligned lane stride: one wide
        // LDS read per run instead of 4 (2) dword reads that would hit the
        // same banks
        if (BITS == 4) return reinterpret_cast<const u32x4*>(rec + pay)[ok ? lane + 64 * k : 0];
        const uint2 t = reinterpret_cast<const uint2*>(rec + pay)[ok ? lane + 64 * k : 0];
        return u32x4{t.x, t.y, 0u, 0u};
      }
      const uint32_t* p = reinterpret_cast<const uint32_t*>(rec + pay) + (ok ? off[k] : 0u);
      return u32x4{p[0], BITS > 1 ? p[1] : 0u, BITS > 2 ? p[2] : 0u, BITS > 3 ? p[3] : 0u};
    };
    if constexpr (BITS == 4) {
#pragma unroll
      for (int k = 0; k < NRL; ++k) {
        const u32x4 t = read_run(k);
        nib[k][0] = t.x; nib[k][1] = t.y; nib[k][2] = t.z; nib[k][3] = t.w;
      }
#pragma unroll
      for (int k = 0; k < NRL; ++k) {
        const uint32_t mm = nibble_splat(h[k]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) nib[k][kk] += mm;
      }
    } else {
      u32x4 t[NRL];
#pragma unroll
      for (int k = 0; k < NRL; ++k) t[k] = read_run(k);
#pragma unroll
      for (int k = 0; k < NRL; ++k) {
        const uint32_t wd[4] = {t[k].x, t[k].y, t[k].z, t[k].w};
        full_to_nibbles<BITS>(wd, nib[k]);
        const uint32_t mm = nibble_splat(h[k]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) nib[k][kk] += mm;
      }
    }
    if (!all_full && ok) {
      // narrower runs: read their words again and decode at their width
#pragma unroll
      for (int k = 0; k < NRL; ++k) {
        const int w = (int)(h[k] >> 4);
        if (w != BITS) {
          if (k / DL < nr) {
            if constexpr (BITS == 4) {
              // the words read are nib - m in every nibble (mod 2^32)
              const uint32_t mm = nibble_splat(h[k]);
              uint32_t wd[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) wd[i] = nib[k][i] - mm;
              // K: one branch-free pass for every width (1-2 % faster on
              // clustered data); V keeps the pass per width present, whose
              // registers its block loop can afford
              if constexpr (!IS_V) narrow4_to_nibbles(w, h[k] & 15u, wd, nib[k]);
              else run_to_nibbles<3>(w, h[k] & 15u, wd, nib[k]);
            } else {
              const uint32_t* p = reinterpret_cast<const uint32_t*>(rec + pay) + off[k];
              narrow_to_nibbles(w, h[k] & 15u, p[0], BITS == 3 ? p[1] : 0u, nib[k]);
            }
          } else {
            nib[k][0] = nib[k][1] = nib[k][2] = nib[k][3] = 0u;
          }
        }
      }
    }
    return ok;
  }
};

// ---------------------------------------------------------------------------
// Offsets of a workgroup's records: lane i holds off[j0 + i] and
// off[j0 + 64 + i] (up to 128 blocks), read back with readlane.
// A window of at most 64 consecutive blocks (the work division never gives
// a workgroup more): lane l keeps block j0 + l's record offset in the
// stream region and its size, so a block's record costs one readlane each.
struct RecordOffsets {
  uint32_t st, sz;
  __device__ __forceinline__ void load(const uint32_t* offs, int j0, int nj, int lane) {
    const uint32_t a = lane < nj ? offs[j0 + lane] : 0u;
    const uint32_t b = lane < nj ? offs[j0 + lane + 1] : 0u;
    st = a;
    sz = b - a;
  }
  // block i (any i: lane i & 63 is read, the caller discards i >= nj): byte
  // offset o and size, and whether [o, o + size) lies in a region of
  // `limit` bytes (32-bit arithmetic, exact)
  __device__ __forceinline__ void at(int i, uint32_t limit, uint64_t& o, uint32_t& size, bool& fits) const {
    const uint32_t so = readlane_u32(st, i & 63);
    size = readlane_u32(sz, i & 63);
    o = so;
    fits = so <= limit && size <= limit - so;
  }
};

// The same window read from a paged cache's block table: entry j holds the
// record's start in 16-byte units of the pool and its size in bytes.  Lane l
// keeps entry j0 + l (windows of at most 64 blocks).
struct RecordTable {
  uint32_t st, sz;
  __device__ __forceinline__ void load(const uint2* tab, int j0, int nj, int lane) {
    const uint2 e = lane < nj ? tab[j0 + lane] : make_uint2(0u, 0u);
    st = e.x;
    sz = e.y;
  }
  // as RecordOffsets::at, with `limit` the pool's size in 16-byte units; a
  // size that is not a multiple of 16 may reach 15 bytes past that, into
  // the pool's slack
  __device__ __forceinline__ void at(int i, uint32_t limit, uint64_t& o, uint32_t& size, bool& fits) const {
    const uint32_t s16 = readlane_u32(st, i & 63);
    size = readlane_u32(sz, i & 63);
    o = (uint64_t)s16 << 4;
    fits = s16 <= limit && (size >> 4) <= limit - s16;
  }
};

// ---------------------------------------------------------------------------
// K side, one staged block.
//
//   scores[g][t] = beta_g + sum_c q'_g[c] (m + u)[t][c],   q' = q * scale
//
// The record's containers go to an LDS plane [slot group][channel] (row
// pitch D + 8 words; the quad order rotates per channel group).  Lane (g8,
// cg) then covers 8 slots x D/8 channels: each container word gives the 8
// slot values exactly (fp4 pair conversions at 2 bits, fp16-subnormal halves
// at 3 and 4 bits; see HALVES), one FMA per element, and an LDS transpose
// sums the 8 channel groups.  Lane l ends with the scores of slots h*64 + l.
// v[g] for a lane-dependent g, as a chain of selects.  Each candidate is made
// opaque first: the compiler otherwise recognises the chain as v[g] and
// indexes a copy of v in scratch memory.
template <class T, int N>
__device__ __forceinline__ T lane_pick(const T (&v)[N], int g) {
  T r = v[0];
#pragma unroll
  for (int k = 1; k < N; ++k) {
    T c = v[k];
    asm volatile("" : "+v"(c));
    r = g == k ? c : r;
  }
  return r;
}

// A split's partial sum goes to the workspace with a relaxed agent-scope
// store: it lands in the device-coherent level, so the workgroup that merges
// the splits can read it on any XCD.
__device__ __forceinline__ void store_partial(float* dst, float v) {
  __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// WS: the records are in payload order 1 (width-sorted rows).
template <int B, int BITS, int GT, int D, bool WS = false>
struct KBlock {
  using Dec = BlockDecoder<B, BITS, false, D>;
  static constexpr int NRL = Dec::NRL;
  static constexpr int DL = D / 64;                   // channels per lane: lane + 64j
  static constexpr int CW = D / 8;                    // channels per channel group
  static constexpr int NQ = CW / 4;                   // 16-byte quads per channel group
  static constexpr int NH = B / 64;
  static constexpr int ROWW = D + 8;
  static constexpr int PLANE_BYTES = (B / 8) * ROWW * 4;
  static constexpr int RED_BYTES = 64 * 9 * 4;        // channel-group reduction, one query
  // The plane and the reduction live in the record's staging buffer: once a
  // record is decoded into registers its bytes are dead.  Each half's
  // reduction reuses that half's plane rows, one query at a time.
  static constexpr int HALF_BYTES = 8 * ROWW * 4;
  static_assert(RED_BYTES <= HALF_BYTES, "reduction must fit a half's plane rows");
  static constexpr int SCRATCH_BYTES = PLANE_BYTES;
  // Slot values for the FMAs.  At 2 bits a container word goes through four
  // fp4 pair conversions (nibbles_to_f32_fp4).  From 3 bits on a nibble
  // reaches 7 (15), past the linear fp4 codes; there the nibbles are masked
  // into the low bits of 16-bit halves: nibble 2i of a half is an fp16
  // subnormal n * 2^-24, nibble 2i+1 one of 16 n * 2^-24, both exact, and the
  // mixed-precision FMA takes the half as it stands.  q' is then kept twice,
  // the second copy divided by 16.
  static_assert(BITS >= 2 && BITS <= 4, "one-byte headers and 4-bit containers");
  static constexpr bool HALVES = BITS >= 3;
  static constexpr int QS_BYTES = GT * D * 4 * (HALVES ? 2 : 1);

  float* qs;                                          // [GT][D] q' of the block (then [GT][D] q' / 16)
  int lane, g8, cg;
  float qu[GT][DL];                                   // queries / unit at channels lane + 64j

  __device__ __forceinline__ void init(uint8_t* qs_, int lane_) {
    qs = reinterpret_cast<float*>(qs_);
    lane = lane_;
    g8 = lane & 7;
    cg = lane >> 3;
  }
  __device__ __forceinline__ void set_queries(const uint16_t* q, int64_t s, int G, int gq0) {
    const float unit_inv = HALVES ? 0x1p24f : 1.0f / fp4_unit();
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const bool ok = gq0 + g < G;
      const uint16_t* qp = q + (s * G + gq0 + g) * D;
#pragma unroll
      for (int j = 0; j < DL; ++j)                    // exact: unit is a power of two
        qu[g][j] = (ok ? f16_bits_to_float(qp[lane + 64 * j]) : 0.f) * unit_inv;
    }
  }

  // rec: the staged record (size bytes, nr runs); it is overwritten by the
  // plane and the reduction.  sink(g, h, score, ok) takes query g's score of
  // slot h*64 + lane as soon as it is reduced; ok: the record decoded
  // consistently (the scores of one that did not are meaningless).  Returns
  // ok.
  template <class Sink>
  __device__ __forceinline__ bool run(uint8_t* rec, uint32_t size, int nr, Sink&& sink) {
    // q' = q * scale (per channel) and beta = q . zero, before the bytes go
    float beta[GT];
    {
      const uint16_t* sc = reinterpret_cast<const uint16_t*>(rec);
      float sv[DL], zv[DL];
#pragma unroll
      for (int j = 0; j < DL; ++j) {
        sv[j] = f16_bits_to_float(sc[lane + 64 * j]);
        zv[j] = f16_bits_to_float(sc[D + lane + 64 * j]);
      }
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float bz = 0.f;
#pragma unroll
        for (int j = 0; j < DL; ++j) {
          const float v = qu[g][j] * sv[j];
          qs[g * D + lane + 64 * j] = v;
          if constexpr (HALVES) qs[(GT + g) * D + lane + 64 * j] = v * 0.0625f;   // exact
          bz = fmaf(qu[g][j], zv[j], bz);
        }
        beta[g] = wave_sum(bz) * (HALVES ? 0x1p-24f : fp4_unit());
      }
    }
    uint32_t nib[NRL][4];
    const bool ok = Dec::decode(rec, size, nr, lane, nib, WS);
    wave_sync();                                  // every lane has read the record
    uint32_t* plane = reinterpret_cast<uint32_t*>(rec);
#pragma unroll
    for (int k = 0; k < NRL; ++k) {
      const int r = k / DL, c = lane + 64 * (k % DL);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) plane[(r * 4 + kk) * ROWW + c] = nib[k][kk];
    }
    wave_sync();
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      float acc[GT][8];
#pragma unroll
      for (int g = 0; g < GT; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[g][i] = 0.f;
      const int row = h * 8 + g8;
#pragma unroll
      for (int i4 = 0; i4 < NQ; ++i4) {
        // the quad order rotates per channel group, so the lanes of one
        // 16-byte read spread over more banks
        const int c0 = cg * CW + ((i4 + cg) % NQ) * 4;
        const u32x4 nw = *reinterpret_cast<const u32x4*>(&plane[row * ROWW + c0]);
        const uint32_t words[4] = {nw.x, nw.y, nw.z, nw.w};
        float qq[GT][4], qh[GT][4];
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          const float4 t = *reinterpret_cast<const float4*>(&qs[g * D + c0]);
          qq[g][0] = t.x; qq[g][1] = t.y; qq[g][2] = t.z; qq[g][3] = t.w;
          if constexpr (HALVES) {
            const float4 u = *reinterpret_cast<const float4*>(&qs[(GT + g) * D + c0]);
            qh[g][0] = u.x; qh[g][1] = u.y; qh[g][2] = u.z; qh[g][3] = u.w;
          }
        }
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          if constexpr (HALVES) {
            // halves k: slots k (low) and k + 4 (high), 16x for odd k
            const uint32_t x = words[cc], y = x >> 8;
            const uint32_t hw[4] = {x & 0x000F000Fu, x & 0x00F000F0u, y & 0x000F000Fu, y & 0x00F000F0u};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const f16x2 hh = __builtin_bit_cast(f16x2, hw[k]);
              const float lo = (float)hh.x, hi = (float)hh.y;
#pragma unroll
              for (int g = 0; g < GT; ++g) {
                const float qv = (k & 1) ? qh[g][cc] : qq[g][cc];
                acc[g][k] = fmaf(qv, lo, acc[g][k]);
                acc[g][k + 4] = fmaf(qv, hi, acc[g][k + 4]);
              }
            }
          } else {
            float f[8];
            nibbles_to_f32_fp4(words[cc], f);
#pragma unroll
            for (int g = 0; g < GT; ++g)
#pragma unroll
              for (int i = 0; i < 8; ++i) acc[g][i] = fmaf(qq[g][cc], f[i], acc[g][i]);
          }
        }
      }
      // reduce the 8 channel groups, one query at a time, in this half's
      // (now dead) plane rows: red[slot][cg], slot = g8*8 + i
      float* red = reinterpret_cast<float*>(rec + h * HALF_BYTES);
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        wave_sync();
#pragma unroll
        for (int i = 0; i < 8; ++i) red[(g8 * 8 + i) * 9 + cg] = acc[g][i];
        wave_sync();
        float sum = beta[g];
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += red[lane * 9 + u];
        sink(g, h, sum, ok);
      }
    }
    return ok;
  }
};

// ---------------------------------------------------------------------------
// K side on the matrix cores, one staged block.
//
//   scores[g][t] = beta_g + sum_c q'_g[c] u[t][c],   q' = q * scale (per channel)
//
// The channel sum is a (queries x channels) by (channels x tokens) product,
// and v_mfma_i32_16x16x64_i8 takes 16 tokens x 64 channels of it at a time,
// which moves the multiply-adds off the vector ALU.  Per block and query, q'
// is written in fixed point, Q = rint(q' 2^E) with |Q| < 2^24 (E from the
// block's largest |q'|), and split into four 7-bit digits, the last one
// signed, so every product and sum is an exact integer; row 4g + d of the
// operand is digit d of query g.  The ints come from the LDS plane [slot
// group][channel] of 4-bit containers: each lane transposes 8 x 8 nibble
// tiles (8 channels x 8 slots; a 16-bit, an 8-bit and a 4-bit exchange stage,
// with v_perm and v_bfi) into a token-major plane [slot][channel / 8], from
// which an MFMA lane reads 16 channels of one token and spreads the nibbles to
// bytes: even nibbles first, then odd.  The digit rows store the channels in
// that same order (opos), since A and B of the MFMA pair byte b of lane l with
// the same k.  Each lane (g, token) adds up its query's four digit sums,
// scales by 2^-E and adds beta.
template <int B, int BITS, int GT, bool WS = false>
struct KBlockM {
  static constexpr int kD = 128;                      // the matrix-core tiles are laid out for D = 128
  using Dec = BlockDecoder<B, BITS, false, kD>;
  static constexpr int NRL = Dec::NRL;
  static constexpr int NH = B / 64;
  static constexpr int NT = B / 16;                   // token tiles of the MFMA
  static constexpr int ROWW = kD + 8;                 // plane row pitch (words)
  static constexpr int PLANE_BYTES = (B / 8) * ROWW * 4;
  static constexpr int TP = 18;                       // token-major pitch: 16 octets + 2 (no bank conflicts)
  static constexpr int TPLANE_BYTES = B * TP * 4;
  static constexpr int SCRATCH_BYTES = PLANE_BYTES > TPLANE_BYTES ? PLANE_BYTES : TPLANE_BYTES;
  static constexpr int QS_BYTES = 16 * kD;            // digit rows [16][128]
  static constexpr int NTILE_LANE = (B / 8) * 16 / 64;   // 8x8 tiles per lane
  static_assert(GT * B * 4 <= SCRATCH_BYTES, "the scores reuse the scratch");
  static_assert(4 * GT <= 16, "one operand row per (query, digit)");

  uint8_t* dig;
  int lane;
  float qa[GT], qb[GT];                               // queries at channels lane, lane + 64

  __device__ __forceinline__ void init(uint8_t* qs_, int lane_) {
    dig = qs_;
    lane = lane_;
  }
  __device__ __forceinline__ void set_queries(const uint16_t* q, int64_t s, int G, int gq0) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const bool ok = gq0 + g < G;
      const uint16_t* qp = q + (s * G + gq0 + g) * kD;
      qa[g] = ok ? f16_bits_to_float(qp[lane]) : 0.f;
      qb[g] = ok ? f16_bits_to_float(qp[lane + 64]) : 0.f;
    }
    // the rows past the queries' digits stay zero
    constexpr int ZW = (16 - 4 * GT) * kD / 16;
    for (int i = lane; i < ZW; i += 64) reinterpret_cast<u32x4*>(dig + 4 * GT * kD)[i] = u32x4{0u, 0u, 0u, 0u};
  }
  // byte position of channel c inside a digit row (the operand order)
  __device__ __forceinline__ static int opos(int c) {
    const int o = c >> 3, n = c & 7;
    return 64 * (o >> 3) + 16 * ((o & 7) >> 1) + 8 * (o & 1) + 4 * (n & 1) + (n >> 1);
  }
  // in place: W[i] nibble j  ->  W[j] nibble i
  __device__ __forceinline__ static void transpose8(uint32_t (&W)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {                     // 16-bit halves of words i, i + 4
      const uint32_t a = W[i], b = W[i + 4];
      W[i] = __builtin_amdgcn_perm(b, a, 0x05040100u);
      W[i + 4] = __builtin_amdgcn_perm(b, a, 0x07060302u);
    }
#pragma unroll
    for (int i0 = 0; i0 < 8; i0 += 4)                 // bytes of words i, i + 2
#pragma unroll
      for (int i = i0; i < i0 + 2; ++i) {
        const uint32_t a = W[i], b = W[i + 2];
        W[i] = __builtin_amdgcn_perm(b, a, 0x06020400u);
        W[i + 2] = __builtin_amdgcn_perm(b, a, 0x07030501u);
      }
#pragma unroll
    for (int i = 0; i < 8; i += 2) {                  // nibbles of words i, i + 1
      const uint32_t a = W[i], b = W[i + 1];
      W[i] = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);
      W[i + 1] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
    }
  }

  // As KBlock::run: rec is overwritten; sink(g, h, score, ok) takes query g's
  // score of slot h*64 + lane.
  template <class Sink>
  __device__ __forceinline__ bool run(uint8_t* rec, uint32_t size, int nr, Sink&& sink) {
    float beta[GT];
    int E[GT];
    {
      const uint16_t* sc = reinterpret_cast<const uint16_t*>(rec);
      const float sa = f16_bits_to_float(sc[lane]), sb = f16_bits_to_float(sc[lane + 64]);
      const float za = f16_bits_to_float(sc[kD + lane]), zb = f16_bits_to_float(sc[kD + lane + 64]);
      const int pa = opos(lane), pb = opos(lane + 64);
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        beta[g] = wave_sum(fmaf(qa[g], za, qb[g] * zb));
        const float xa = qa[g] * sa, xb = qb[g] * sb;
        const float M = wave_max_nonneg(fmaxf(fabsf(xa), fabsf(xb)));
        E[g] = M > 0.f ? 24 - __builtin_amdgcn_frexp_expf(M) : 0;    // M 2^E in [2^23, 2^24)
        const int Qa = (int)rintf(ldexpf(xa, E[g])), Qb = (int)rintf(ldexpf(xb, E[g]));
        uint8_t* row = dig + 4 * g * kD;
        row[pa] = (uint8_t)(Qa & 127);
        row[kD + pa] = (uint8_t)((Qa >> 7) & 127);
        row[2 * kD + pa] = (uint8_t)((Qa >> 14) & 127);
        row[3 * kD + pa] = (uint8_t)(Qa >> 21);
        row[pb] = (uint8_t)(Qb & 127);
        row[kD + pb] = (uint8_t)((Qb >> 7) & 127);
        row[2 * kD + pb] = (uint8_t)((Qb >> 14) & 127);
        row[3 * kD + pb] = (uint8_t)(Qb >> 21);
      }
    }
    uint32_t nib[NRL][4];
    const bool ok = Dec::decode(rec, size, nr, lane, nib, WS);
    wave_sync();                                  // every lane has read the record
    uint32_t* plane = reinterpret_cast<uint32_t*>(rec);
#pragma unroll
    for (int k = 0; k < NRL; ++k) {
      const int r = k >> 1, c = lane + 64 * (k & 1);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) plane[(r * 4 + kk) * ROWW + c] = nib[k][kk];
    }
    wave_sync();
    // tiles (slot group, octet): the lane's 8 words of 8 channels, transposed
    // to 8 words of 8 slots
    uint32_t T[NTILE_LANE][8];
#pragma unroll
    for (int it = 0; it < NTILE_LANE; ++it) {
      const int tile = it * 64 + lane, sg = tile >> 4, o = tile & 15;
      const u32x4 w0 = *reinterpret_cast<const u32x4*>(&plane[sg * ROWW + 8 * o]);
      const u32x4 w1 = *reinterpret_cast<const u32x4*>(&plane[sg * ROWW + 8 * o + 4]);
      uint32_t W[8] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
      transpose8(W);
#pragma unroll
      for (int j = 0; j < 8; ++j) T[it][j] = W[j];
    }
    wave_sync();                                  // the plane is read: the token-major plane replaces it
    uint32_t* tpl = plane;
#pragma unroll
    for (int it = 0; it < NTILE_LANE; ++it) {
      const int tile = it * 64 + lane, sg = tile >> 4, o = tile & 15;
#pragma unroll
      for (int j = 0; j < 8; ++j) tpl[(8 * sg + j) * TP + o] = T[it][j];
    }
    wave_sync();
    i32x4 A[2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
      A[s] = *reinterpret_cast<const i32x4*>(dig + (lane & 15) * kD + 64 * s + 16 * (lane >> 4));
    i32x4 C[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      C[tt] = i32x4{0, 0, 0, 0};
      const int t = 16 * tt + (lane & 15);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const uint2 w = *reinterpret_cast<const uint2*>(&tpl[t * TP + 8 * s + 2 * (lane >> 4)]);
        const i32x4 Bv = {(int)(w.x & 0x0F0F0F0Fu), (int)((w.x >> 4) & 0x0F0F0F0Fu), (int)(w.y & 0x0F0F0F0Fu),
                          (int)((w.y >> 4) & 0x0F0F0F0Fu)};
        C[tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[s], Bv, C[tt], 0, 0, 0);
      }
    }
    // lane (g, token): the four digit sums of query g
    const int g = lane >> 4;
    const float bsel = lane_pick(beta, g);
    const int esel = lane_pick(E, g);
    wave_sync();                                  // the token-major plane is read
    float* scs = reinterpret_cast<float*>(rec);
    if (g < GT) {
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const float v = fmaf(2097152.f, (float)C[tt][3],
                             fmaf(16384.f, (float)C[tt][2], fmaf(128.f, (float)C[tt][1], (float)C[tt][0])));
        scs[g * B + 16 * tt + (lane & 15)] = ldexpf(v, -esel) + bsel;
      }
    }
    wave_sync();
#pragma unroll
    for (int gg = 0; gg < GT; ++gg)
#pragma unroll
      for (int h = 0; h < NH; ++h) sink(gg, h, scs[gg * B + h * 64 + lane], ok);
    return ok;
  }
};


// ---------------------------------------------------------------------------
// V side, one staged block.
//
//   out[c] = sum_t p_t zero_t + sum_t p'_t q[t][c],   p'_t = p_t scale_t >= 0
//
// The second sum runs over the slots of a run, which is the axis a container
// word packs (8 slots of one channel).  Per block and query, p' is written as
// a 20-bit fixed-point integer relative to the block's largest p'
// (P_t = round(p'_t 2^E), P_t < 2^20) and split into five 4-bit digits; the
// digit words of 8 slots are built once per block with DPP and shared through
// LDS.  One v_dot8_u32_u4 then multiplies a container word by a digit word:
// 5 instructions per 8 elements, with exact integer sums that are scaled by
// 2^-E once per block and channel.  Per element the weight error is at most
// 2^-21 of the block's largest weight.  Lane l accumulates channels l + 64j.
// STAGED: the weights' digit words are assembled from weights staged in
// LDS (one word per lane and pass) rather than by an OR across each group of
// 8 lanes per digit.  Measured: the V GEMV 2-9 % faster staged; fused
// attention unchanged with one query and 5 % slower with four, where the
// extra LDS round trip sits on the V wave's path between two barriers.
template <int B, int BITS, int GT, int D, bool STAGED = true>
struct VBlock {
  using Dec = BlockDecoder<B, BITS, true, D>;
  static constexpr int NR = Dec::NR;
  static constexpr int NRL = Dec::NRL;                // run l + 64k: r = k / DL, channel l + 64 (k % DL)
  static constexpr int DL = D / 64;
  static constexpr int NA = DL;                       // accumulators per query: channels lane + 64j
  static constexpr int NH = B / 64;                   // slots per lane
  static constexpr int NG = B / 8;                    // 8-slot groups per block
  static constexpr int ND = 5;                        // 4-bit digits of p'
  static constexpr int DIG_WORDS = GT * ND * NG;
  static constexpr int LDS_WORDS = DIG_WORDS + (STAGED ? GT * B : 0);   // digit words, then the weights
  static constexpr int SCRATCH_BYTES = 0;            // the staged record is only read

  uint32_t* dig;                                      // [GT][ND][NG]
  uint32_t* pst;                                      // [GT][B] fixed-point weights
  int lane, nib_shift;

  __device__ __forceinline__ void init(uint32_t* lds, int lane_) {
    dig = lds;
    pst = lds + DIG_WORDS;
    lane = lane_;
    nib_shift = 4 * (lane & 7);
  }

  // acc[g][j]: query g at channel lane + 64j
  __device__ __forceinline__ void rescale(float (&acc)[GT][NA], const float (&alpha)[GT]) const {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
#pragma unroll
      for (int j = 0; j < NA; ++j) acc[g][j] *= alpha[g];
    }
  }
  // dst(g): query g's partial sums (nullptr for an absent query)
  template <class Dst>
  __device__ __forceinline__ void store(const float (&acc)[GT][NA], const float (&z)[GT], Dst&& dst) const {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      float* d = dst(g);
      if (d) {
#pragma unroll
        for (int j = 0; j < NA; ++j) store_partial(d + lane + 64 * j, acc[g][j] + z[g]);
      }
    }
  }

  // pw[g][h]: weight of slot h*64 + lane (0 past the valid slots).  use:
  // whether the block may contribute (its record is in range).  Returns
  // whether the record decoded consistently; a block that does not adds
  // nothing.
  __device__ __forceinline__ bool run(const uint8_t* rec, uint32_t size, int nr, bool use,
                                      const float (&pw)[GT][NH], float (&acc)[GT][NA], float (&pz)[GT]) {
    int E[GT];
    bool live[GT];
    float pzb[GT];
    {
      const uint16_t* sc = reinterpret_cast<const uint16_t*>(rec);
      float pp[GT][NH];
#pragma unroll
      for (int g = 0; g < GT; ++g) pzb[g] = 0.f;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int sl = h * 64 + lane;
        const float scl = f16_bits_to_float(sc[sl]), zer = f16_bits_to_float(sc[B + sl]);
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          pp[g][h] = pw[g][h] * scl;
          pzb[g] = fmaf(pw[g][h], zer, pzb[g]);
        }
      }
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float mx = pp[g][0];
#pragma unroll
        for (int h = 1; h < NH; ++h) mx = fmaxf(mx, pp[g][h]);
        const float M = wave_max_nonneg(mx);
        live[g] = M > 0.f;
        // M * 2^E in [2^19, 2^20): M = f * 2^e with f in [0.5, 1), so
        // ilogb(M) = e - 1
        E[g] = live[g] ? 20 - __builtin_amdgcn_frexp_expf(M) : 0;
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const uint32_t P = min((uint32_t)(ldexpf(pp[g][h], E[g]) + 0.5f), 0xFFFFFu);
          if constexpr (STAGED) {
            pst[g * B + h * 64 + lane] = P;
          } else {
#pragma unroll
            for (int d = 0; d < ND; ++d) {
              const uint32_t wv = or8(((P >> (4 * d)) & 15u) << nib_shift);
              if ((lane & 7) == 0) dig[(g * ND + d) * NG + h * 8 + (lane >> 3)] = wv;
            }
          }
        }
      }
    }
    if constexpr (STAGED) {
      wave_sync();
      // digit word (g, d, q): digit d (bits 4d .. 4d+3) of the weights of
      // slots 8q .. 8q+7, slot 8q + k in nibble k; one word per lane and pass
#pragma unroll
      for (int i0 = 0; i0 < DIG_WORDS; i0 += 64) {
        const int i = i0 + lane;
        if (DIG_WORDS % 64 == 0 || i < DIG_WORDS) {
          const int g = i / (ND * NG), d = (i / NG) % ND, q = i % NG;
          const u32x4* src = reinterpret_cast<const u32x4*>(pst + g * B + 8 * q);
          const u32x4 a = src[0], b = src[1];
          const uint32_t sh = 4u * (uint32_t)d;
          uint32_t wv = __builtin_amdgcn_ubfe(a[0], sh, 4);
          wv |= __builtin_amdgcn_ubfe(a[1], sh, 4) << 4;
          wv |= __builtin_amdgcn_ubfe(a[2], sh, 4) << 8;
          wv |= __builtin_amdgcn_ubfe(a[3], sh, 4) << 12;
          wv |= __builtin_amdgcn_ubfe(b[0], sh, 4) << 16;
          wv |= __builtin_amdgcn_ubfe(b[1], sh, 4) << 20;
          wv |= __builtin_amdgcn_ubfe(b[2], sh, 4) << 24;
          wv |= __builtin_amdgcn_ubfe(b[3], sh, 4) << 28;
          dig[i] = wv;
        }
      }
    }
    uint32_t nib[NRL][4];
    const bool ok = Dec::decode(rec, size, nr, lane, nib) && use;
    wave_sync();
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      if (!ok || !live[g]) continue;
      uint32_t sd[DL][ND];
#pragma unroll
      for (int ch = 0; ch < DL; ++ch)
#pragma unroll
        for (int d = 0; d < ND; ++d) sd[ch][d] = 0u;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if (r >= nr) break;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          uint32_t W[ND];                             // digit words of slots 8(4r+kk) ...
#pragma unroll
          for (int d = 0; d < ND; ++d) W[d] = dig[(g * ND + d) * NG + 4 * r + kk];
#pragma unroll
          for (int ch = 0; ch < DL; ++ch)
#pragma unroll
            for (int d = 0; d < ND; ++d)
              sd[ch][d] = __builtin_amdgcn_udot8(nib[DL * r + ch][kk], W[d], sd[ch][d], false);
        }
      }
      const float unit = ldexpf(1.0f, -E[g]);
#pragma unroll
      for (int ch = 0; ch < DL; ++ch) {
        // each digit sum is <= NR*32*15*15 < 2^15, so the total stays below 2^32
        const uint32_t x = sd[ch][0] + (sd[ch][1] << 4) + (sd[ch][2] << 8) + (sd[ch][3] << 12) + (sd[ch][4] << 16);
        acc[g][ch] = fmaf((float)x, unit, acc[g][ch]);
      }
    }
#pragma unroll
    for (int g = 0; g < GT; ++g)
      if (ok) pz[g] += pzb[g];
    return ok;
  }
};

// ---------------------------------------------------------------------------
// V side on the matrix cores, one staged block, for a tile of four queries.
//
//   out[g][c] = sum_t p_t zero_t + sum_t p'_g[t] u[t][c]
//
// The second sum is a (queries x tokens) by (tokens x channels) product, and
// the payload already packs each channel's tokens together, so no transpose
// is needed: the decoded container words go to an LDS plane [channel][slot
// group], and each lane of v_mfma_i32_16x16x64_i8 reads 16 tokens of one
// channel and spreads the nibbles to bytes (even nibbles first).  The
// weights are the same 20-bit fixed point as VBlock's (P = round(p' 2^E) per
// block and query), split into three 7-bit digits; operand row 4g + d holds
// digit d of query g in the token order of the spread (tpos), row 4g + 3 is
// zero.  Eight MFMAs cover the 128 channels; lane l then holds query l / 16
// at channels 16j + l % 16 (acc[j / 2][j % 2]) and adds its three digit sums
// scaled by 2^-E.
template <int B, int BITS, int GT>
struct VBlockM {
  static constexpr int kD = 128;                      // the matrix-core tiles are laid out for D = 128
  using Dec = BlockDecoder<B, BITS, true, kD>;
  static constexpr int NRL = Dec::NRL;
  static constexpr int NA = 2;                        // accumulators: channels 16j + l % 16 as [j / 2][j % 2]
  static constexpr int NH = B / 64;
  static constexpr int KS = B / 64;                   // 64-token steps of the MFMA
  static constexpr int VP = B / 8 + 2;                // plane pitch per channel (words)
  static constexpr int LDS_WORDS = 16 * B / 4;        // digit rows [16][B] bytes
  static constexpr int SCRATCH_BYTES = kD * VP * 4;   // the plane overwrites the staged record
  static_assert(GT == 4, "operand rows are (query, digit) for four queries");

  uint8_t* dig;
  int lane;

  __device__ __forceinline__ void init(uint32_t* lds, int lane_) {
    dig = reinterpret_cast<uint8_t*>(lds);
    lane = lane_;
    // the rows 4g + 3 are never written: zero
#pragma unroll
    for (int g = 0; g < GT; ++g)
      for (int i = lane; i < B / 16; i += 64) reinterpret_cast<u32x4*>(dig + (4 * g + 3) * B)[i] = u32x4{0u, 0u, 0u, 0u};
  }
  // position of token t of the block inside a digit row (the operand order)
  __device__ __forceinline__ static int tpos(int t) {
    const int rs = t & 15, n = rs & 7;
    return 64 * (t >> 6) + 16 * ((t >> 4) & 3) + 8 * (rs >> 3) + 4 * (n & 1) + (n >> 1);
  }
  __device__ __forceinline__ void rescale(float (&acc)[GT][NA], const float (&alpha)[GT]) const {
    const float f = lane_pick(alpha, lane >> 4);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j >> 1][j & 1] *= f;
  }
  template <class Dst>
  __device__ __forceinline__ void store(const float (&acc)[GT][NA], const float (&z)[GT], Dst&& dst) const {
    const int g = lane >> 4;
    const float zg = lane_pick(z, g);
    float* d = dst(g);
    if (d) {
#pragma unroll
      for (int j = 0; j < 8; ++j) store_partial(d + 16 * j + (lane & 15), acc[j >> 1][j & 1] + zg);
    }
  }

  // As VBlock::run; rec is overwritten by the plane.
  __device__ __forceinline__ bool run(uint8_t* rec, uint32_t size, int nr, bool use,
                                      const float (&pw)[GT][NH], float (&acc)[GT][NA], float (&pz)[GT]) {
    int E[GT];
    float pzb[GT];
    {
      const uint16_t* sc = reinterpret_cast<const uint16_t*>(rec);
      float pp[GT][NH];
#pragma unroll
      for (int g = 0; g < GT; ++g) pzb[g] = 0.f;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int sl = h * 64 + lane;
        const float scl = f16_bits_to_float(sc[sl]), zer = f16_bits_to_float(sc[B + sl]);
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          pp[g][h] = pw[g][h] * scl;
          pzb[g] = fmaf(pw[g][h], zer, pzb[g]);
        }
      }
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float mx = pp[g][0];
#pragma unroll
        for (int h = 1; h < NH; ++h) mx = fmaxf(mx, pp[g][h]);
        const float M = wave_max_nonneg(mx);
        E[g] = M > 0.f ? 20 - __builtin_amdgcn_frexp_expf(M) : 0;    // M 2^E in [2^19, 2^20)
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const uint32_t P = min((uint32_t)(ldexpf(pp[g][h], E[g]) + 0.5f), 0xFFFFFu);
          const int p = tpos(h * 64 + lane);
          dig[(4 * g) * B + p] = (uint8_t)(P & 127u);
          dig[(4 * g + 1) * B + p] = (uint8_t)((P >> 7) & 127u);
          dig[(4 * g + 2) * B + p] = (uint8_t)(P >> 14);
        }
      }
    }
    uint32_t nib[NRL][4];
    const bool ok = Dec::decode(rec, size, nr, lane, nib) && use;
    wave_sync();                                  // every lane has read the record
    uint32_t* vpl = reinterpret_cast<uint32_t*>(rec);
#pragma unroll
    for (int k = 0; k < NRL; ++k) {
      const int r = k >> 1, c = lane + 64 * (k & 1);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) vpl[c * VP + 4 * r + kk] = nib[k][kk];
    }
    wave_sync();
    i32x4 A[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
      A[s] = *reinterpret_cast<const i32x4*>(dig + (lane & 15) * B + 64 * s + 16 * (lane >> 4));
    const float unit = ldexpf(1.0f, -lane_pick(E, lane >> 4));
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      i32x4 C = {0, 0, 0, 0};
      const int ch = 16 * j + (lane & 15);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const uint2 w = *reinterpret_cast<const uint2*>(&vpl[ch * VP + 8 * s + 2 * (lane >> 4)]);
        const i32x4 Bv = {(int)(w.x & 0x0F0F0F0Fu), (int)((w.x >> 4) & 0x0F0F0F0Fu), (int)(w.y & 0x0F0F0F0Fu),
                          (int)((w.y >> 4) & 0x0F0F0F0Fu)};
        C = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[s], Bv, C, 0, 0, 0);
      }
      if (ok) {
        const float x = fmaf(16384.f, (float)C[2], fmaf(128.f, (float)C[1], (float)C[0]));
        acc[j >> 1][j & 1] = fmaf(x, unit, acc[j >> 1][j & 1]);
      }
    }
#pragma unroll
    for (int gg = 0; gg < GT; ++gg)
      if (ok) pz[gg] += pzb[gg];
    return ok;
  }
};

// ---------------------------------------------------------------------------
// Wide widths, b = 5..8: two-byte header entries (w << 8 | m) and byte
// containers.  The block code is the plain form of the 4-bit path: every
// run is decoded with a prefix sum of its widths (no full-width shortcut),
// K converts bytes with v_cvt_f32_ubyte and V takes the 20-bit weights as
// three byte digits with v_dot4_u32_u8.

// Decode of one staged record: lane l holds runs l + 64k (k < NRL) as eight
// words of byte containers, word i = q of slots 4i .. 4i+3 (byte j = slot
// 4i + j), q = m + u.  Returns false if the record is inconsistent (a width
// above bits, a minimum that leaves no room for its width, or widths that do
// not add up to the record size); the containers are then zero.
template <int B, bool IS_V, int D>
struct DecW {
  static constexpr int NR = B / kR;
  static constexpr int NRL = NR * D / 64;
  static constexpr int HDR = hdr_offset(IS_V, B, D);

  // the R fields of width W of a run's W words, as byte containers
  template <int W>
  __device__ __forceinline__ static void spread(const uint32_t (&wd)[8], uint32_t (&out)[8]) {
    sliced_to_bytes<W>(wd, out);
  }

  __device__ __forceinline__ static bool decode(const uint8_t* rec, uint32_t size, int nr, int lane, int bits,
                                                uint32_t (&cont)[NRL][8]) {
    const int pay = payload_offset(IS_V, B, nr, 2, D);
    const int nruns = nr * D;
    const int L = (1 << bits) - 1;
    const uint16_t* hd = reinterpret_cast<const uint16_t*>(rec + HDR);
    int w[NRL];
    uint32_t m[NRL], off[NRL];
    bool bad = false, narrow = nr != NR;
#pragma unroll
    for (int k = 0; k < NRL; ++k) {
      const int ri = lane + 64 * k;
      const uint32_t h = ri < nruns ? hd[ri] : 0u;
      w[k] = (int)(h >> 8);
      m[k] = h & 255u;
      // a valid run has max - m in [2^(w-1), 2^w - 1] and max <= L
      bad |= w[k] > bits || (int)m[k] > L || (w[k] > 0 && (int)m[k] + (1 << (w[k] - 1)) > L);
      narrow |= w[k] != bits;
    }
    // a full block whose runs are all at the full width has implicit offsets
    // (run i at word i * bits); otherwise a wave prefix sum of the widths
    const bool all_full = __ballot(narrow) == 0;
    uint32_t base = 0;
    if (all_full) {
#pragma unroll
      for (int k = 0; k < NRL; ++k) off[k] = (uint32_t)((lane + 64 * k) * bits);
      base = (uint32_t)(NRL * 64 * bits);
    } else {
#pragma unroll
      for (int k = 0; k < NRL; ++k) {
        const int incl = wave_incl_scan(w[k]);
        off[k] = base + (uint32_t)(incl - w[k]);
        base += (uint32_t)__builtin_amdgcn_readlane(incl, 63);
      }
    }
    const bool ok = __ballot(bad) == 0 && (uint32_t)pad16(pay + 4 * (int)base) == size;
    const uint32_t* pw = reinterpret_cast<const uint32_t*>(rec + pay);
    // at the full width 8 every run is 32 bytes at a 32-byte boundary: two
    // 16-byte reads instead of eight dword reads 32 bytes apart across the
    // lanes (which fall in the same banks)
    const bool wide8 = all_full && bits == 8 && ok;
#pragma unroll
    for (int k = 0; k < NRL; ++k) {
      // a consistent record keeps every run's words inside it
      const int wr = ok ? w[k] : 0;
      uint32_t wd[8];
      if (wide8) {
        const u32x4 a = reinterpret_cast<const u32x4*>(pw + off[k])[0];
        const u32x4 b = reinterpret_cast<const u32x4*>(pw + off[k])[1];
        wd[0] = a.x; wd[1] = a.y; wd[2] = a.z; wd[3] = a.w;
        wd[4] = b.x; wd[5] = b.y; wd[6] = b.z; wd[7] = b.w;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) wd[i] = i < wr ? pw[off[k] + i] : 0u;
      }
      switch (wr) {
        case 0: spread<0>(wd, cont[k]); break;
        case 1: spread<1>(wd, cont[k]); break;
        case 2: spread<2>(wd, cont[k]); break;
        case 3: spread<3>(wd, cont[k]); break;
        case 4: spread<4>(wd, cont[k]); break;
        case 5: spread<5>(wd, cont[k]); break;
        case 6: spread<6>(wd, cont[k]); break;
        case 7: spread<7>(wd, cont[k]); break;
        default: spread<8>(wd, cont[k]); break;
      }
      const uint32_t mm = (ok ? m[k] : 0u) * 0x01010101u;   // m + u <= 255: no carries
#pragma unroll
      for (int i = 0; i < 8; ++i) cont[k][i] += mm;
    }
    return ok;
  }
};

// K side, wide widths, one staged block (the interface of KBlock).  The
// containers go to an LDS plane [slot quad][channel]; lane (g8, cg) then
// takes slots 8 g8 .. 8 g8 + 7 of 16 channels, converts the bytes exactly
// and multiply-adds q' = q * scale, and the 8 channel groups are reduced
// through LDS as in KBlock.
template <int B, int GT, int D>
struct KBlockW {
  using Dec = DecW<B, false, D>;
  static constexpr int NRL = Dec::NRL;
  static constexpr int DL = D / 64;                   // channels per lane: lane + 64j
  static constexpr int CW = D / 8;                    // channels per channel group
  static constexpr int NQ = CW / 4;                   // 16-byte quads per channel group
  static constexpr int NH = B / 64;
  static constexpr int ROWW = D + 8;
  static constexpr int PLANE_BYTES = (B / 4) * ROWW * 4;
  static constexpr int RED_BYTES = 64 * 9 * 4;
  static constexpr int HALF_BYTES = 16 * ROWW * 4;    // the quad rows of 64 slots
  static_assert(RED_BYTES <= HALF_BYTES, "reduction must fit a half's plane rows");
  static constexpr int SCRATCH_BYTES = PLANE_BYTES;
  static constexpr int QS_BYTES = GT * D * 4;

  float* qs;
  int lane, g8, cg, bits = 8;
  float qv[GT][DL];                                   // queries at channels lane + 64j

  __device__ __forceinline__ void init(uint8_t* qs_, int lane_) {
    qs = reinterpret_cast<float*>(qs_);
    lane = lane_;
    g8 = lane & 7;
    cg = lane >> 3;
  }
  __device__ __forceinline__ void set_queries(const uint16_t* q, int64_t s, int G, int gq0) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const bool ok = gq0 + g < G;
      const uint16_t* qp = q + (s * G + gq0 + g) * D;
#pragma unroll
      for (int j = 0; j < DL; ++j) qv[g][j] = ok ? f16_bits_to_float(qp[lane + 64 * j]) : 0.f;
    }
  }

  template <class Sink>
  __device__ __forceinline__ bool run(uint8_t* rec, uint32_t size, int nr, Sink&& sink) {
    float beta[GT];
    {
      const uint16_t* sc = reinterpret_cast<const uint16_t*>(rec);
      float sv[DL], zv[DL];
#pragma unroll
      for (int j = 0; j < DL; ++j) {
        sv[j] = f16_bits_to_float(sc[lane + 64 * j]);
        zv[j] = f16_bits_to_float(sc[D + lane + 64 * j]);
      }
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float bz = 0.f;
#pragma unroll
        for (int j = 0; j < DL; ++j) {
          qs[g * D + lane + 64 * j] = qv[g][j] * sv[j];
          bz = fmaf(qv[g][j], zv[j], bz);
        }
        beta[g] = wave_sum(bz);
      }
    }
    uint32_t cont[NRL][8];
    const bool ok = Dec::decode(rec, size, nr, lane, bits, cont);
    wave_sync();                                  // every lane has read the record
    uint32_t* plane = reinterpret_cast<uint32_t*>(rec);
#pragma unroll
    for (int k = 0; k < NRL; ++k) {
      const int r = k / DL, c = lane + 64 * (k % DL);
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) plane[(r * 8 + kk) * ROWW + c] = cont[k][kk];
    }
    wave_sync();
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      float acc[GT][8];
#pragma unroll
      for (int g = 0; g < GT; ++g)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[g][i] = 0.f;
      const int row = h * 16 + 2 * g8;
#pragma unroll
      for (int i4 = 0; i4 < NQ; ++i4) {
        const int c0 = cg * CW + ((i4 + cg) % NQ) * 4;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(&plane[row * ROWW + c0]);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(&plane[(row + 1) * ROWW + c0]);
        float qq[GT][4];
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          const float4 t = *reinterpret_cast<const float4*>(&qs[g * D + c0]);
          qq[g][0] = t.x; qq[g][1] = t.y; qq[g][2] = t.z; qq[g][3] = t.w;
        }
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          float f[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f[i] = (float)((lo[cc] >> (8 * i)) & 255u);
            f[4 + i] = (float)((hi[cc] >> (8 * i)) & 255u);
          }
#pragma unroll
          for (int g = 0; g < GT; ++g)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[g][i] = fmaf(qq[g][cc], f[i], acc[g][i]);
        }
      }
      float* red = reinterpret_cast<float*>(rec + h * HALF_BYTES);
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        wave_sync();
#pragma unroll
        for (int i = 0; i < 8; ++i) red[(g8 * 8 + i) * 9 + cg] = acc[g][i];
        wave_sync();
        float sum = beta[g];
#pragma unroll
        for (int u = 0; u < 8; ++u) sum += red[lane * 9 + u];
        sink(g, h, sum, ok);
      }
    }
    return ok;
  }
};

// V side, wide widths, one staged block (the interface of VBlock).  The
// weights are VBlock's 20-bit fixed point per block and query, split into
// three byte digits; v_dot4_u32_u8 takes 4 slots of one channel per
// instruction.  Each digit sum is at most B * 255 * 255 < 2^24, so the three
// are exact in fp32 and are combined there.
template <int B, int GT, int D>
struct VBlockW {
  using Dec = DecW<B, true, D>;
  static constexpr int NR = B / kR;
  static constexpr int NRL = Dec::NRL;
  static constexpr int DL = D / 64;
  static constexpr int NA = DL;                       // accumulators per query: channels lane + 64j
  static constexpr int NH = B / 64;
  static constexpr int NQ = B / 4;                    // 4-slot groups per block
  static constexpr int ND = 3;                        // byte digits of p'
  static constexpr int DIG_WORDS = GT * ND * NQ;
  static constexpr int LDS_WORDS = DIG_WORDS + GT * B;
  static constexpr int SCRATCH_BYTES = 0;            // the staged record is only read

  uint32_t* dig;                                      // [GT][ND][NQ]
  uint32_t* pst;                                      // [GT][B] fixed-point weights
  int lane, bits = 8;

  __device__ __forceinline__ void init(uint32_t* lds, int lane_) {
    dig = lds;
    pst = lds + DIG_WORDS;
    lane = lane_;
  }
  __device__ __forceinline__ void rescale(float (&acc)[GT][NA], const float (&alpha)[GT]) const {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
#pragma unroll
      for (int j = 0; j < NA; ++j) acc[g][j] *= alpha[g];
    }
  }
  template <class Dst>
  __device__ __forceinline__ void store(const float (&acc)[GT][NA], const float (&z)[GT], Dst&& dst) const {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      float* d = dst(g);
      if (d) {
#pragma unroll
        for (int j = 0; j < NA; ++j) store_partial(d + lane + 64 * j, acc[g][j] + z[g]);
      }
    }
  }

  __device__ __forceinline__ bool run(const uint8_t* rec, uint32_t size, int nr, bool use,
                                      const float (&pw)[GT][NH], float (&acc)[GT][NA], float (&pz)[GT]) {
    int E[GT];
    bool live[GT];
    float pzb[GT];
    {
      const uint16_t* sc = reinterpret_cast<const uint16_t*>(rec);
      float pp[GT][NH];
#pragma unroll
      for (int g = 0; g < GT; ++g) pzb[g] = 0.f;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int sl = h * 64 + lane;
        const float scl = f16_bits_to_float(sc[sl]), zer = f16_bits_to_float(sc[B + sl]);
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          pp[g][h] = pw[g][h] * scl;
          pzb[g] = fmaf(pw[g][h], zer, pzb[g]);
        }
      }
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float mx = pp[g][0];
#pragma unroll
        for (int h = 1; h < NH; ++h) mx = fmaxf(mx, pp[g][h]);
        const float M = wave_max_nonneg(mx);
        live[g] = M > 0.f;
        E[g] = live[g] ? 20 - __builtin_amdgcn_frexp_expf(M) : 0;   // M 2^E in [2^19, 2^20)
#pragma unroll
        for (int h = 0; h < NH; ++h)
          pst[g * B + h * 64 + lane] = min((uint32_t)(ldexpf(pp[g][h], E[g]) + 0.5f), 0xFFFFFu);
      }
    }
    wave_sync();
    // digit word (g, d, q): byte d of the weights of slots 4q .. 4q+3, slot
    // 4q + j in byte j; one word per lane and pass
#pragma unroll
    for (int i0 = 0; i0 < DIG_WORDS; i0 += 64) {
      const int i = i0 + lane;
      if (DIG_WORDS % 64 == 0 || i < DIG_WORDS) {
        const int g = i / (ND * NQ), d = (i / NQ) % ND, q = i % NQ;
        const u32x4 a = *reinterpret_cast<const u32x4*>(pst + g * B + 4 * q);
        const uint32_t sh = 8u * (uint32_t)d;
        dig[i] = __builtin_amdgcn_ubfe(a[0], sh, 8) | (__builtin_amdgcn_ubfe(a[1], sh, 8) << 8) |
                 (__builtin_amdgcn_ubfe(a[2], sh, 8) << 16) | (__builtin_amdgcn_ubfe(a[3], sh, 8) << 24);
      }
    }
    uint32_t cont[NRL][8];
    const bool ok = Dec::decode(rec, size, nr, lane, bits, cont) && use;
    wave_sync();
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      if (!ok || !live[g]) continue;
      uint32_t sd[DL][ND];
#pragma unroll
      for (int ch = 0; ch < DL; ++ch)
#pragma unroll
        for (int d = 0; d < ND; ++d) sd[ch][d] = 0u;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if (r >= nr) break;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          uint32_t W[ND];                             // digit words of slots 4(8r+kk) ...
#pragma unroll
          for (int d = 0; d < ND; ++d) W[d] = dig[(g * ND + d) * NQ + 8 * r + kk];
#pragma unroll
          for (int ch = 0; ch < DL; ++ch)
#pragma unroll
            for (int d = 0; d < ND; ++d)
              sd[ch][d] = __builtin_amdgcn_udot4(cont[DL * r + ch][kk], W[d], sd[ch][d], false);
        }
      }
      const float unit = ldexpf(1.0f, -E[g]);
#pragma unroll
      for (int ch = 0; ch < DL; ++ch) {
        const float x = fmaf(65536.f, (float)sd[ch][2], fmaf(256.f, (float)sd[ch][1], (float)sd[ch][0]));
        acc[g][ch] = fmaf(x, unit, acc[g][ch]);
      }
    }
#pragma unroll
    for (int g = 0; g < GT; ++g)
      if (ok) pz[g] += pzb[g];
    return ok;
  }
};

// The K block code the kernels use: wide widths (b > 4) take KBlockW; at
// b <= 4 the matrix cores (KBlockM) for a tile of four queries, vector FMAs
// (KBlock) for one.  Measured (A/B in one process): with four queries,
// 128-token blocks, fused attention 295 -> 264 us and the K GEMV 128 -> 117
// us; with one query the matrix version is slower (K GEMV +9-10 %, one wave
// less occupancy; fused attention +1-3 %), as its transposes and LDS round
// trips are not repaid by 32 FMAs per packed word.
// The matrix-core tiles are laid out for D = 128; other head_dims take the
// vector code for every tile.
// WS: payload order 1, taken only up to 4 bits.
template <int B, int BITS, int GT, int D, bool WS = false>
using KSel = std::conditional_t<(BITS > 4), KBlockW<B, GT, D>,
                                std::conditional_t<(GT > 1 && D == 128), KBlockM<B, BITS, GT, WS>,
                                                   KBlock<B, BITS, GT, D, WS>>>;

// The V block code the kernels use: wide widths take VBlockW; at b <= 4 the
// matrix cores (VBlockM) for a tile of four queries (D = 128), v_dot8
// (VBlock) otherwise.
template <int B, int BITS, int GT, int D, bool STAGED = true>
using VSel = std::conditional_t<(BITS > 4), VBlockW<B, GT, D>,
                                std::conditional_t<(GT > 1 && D == 128), VBlockM<B, BITS, GT>,
                                                   VBlock<B, BITS, GT, D, STAGED>>>;


// ---------------------------------------------------------------------------
// Streaming skeleton shared by the GEMVs and by each wave of fused
// attention: a wave walks J consecutive blocks of one stream.  Records are
// staged into LDS from registers with one record in flight: block jj + 1 is
// requested into the registers that block jj has just left for LDS, while
// block jj is processed.  A scheduling barrier keeps the request's loads
// together.  The loop body has no exits: a missing block (jj >= nj) is
// requested as zero bytes, and a missing or corrupt block contributes
// nothing (an exit inside the body would give the wait-count analysis a path
// with a different set of loads in flight, and it would then drain the load
// queue at every block).
template <int NCH, int REC, class Loc = RecordOffsets>
struct RecordStream {
  const uint8_t* arena;
  uint32_t limit;        // the region's bytes (RecordOffsets) or the pool's 16-byte units (RecordTable)
  Loc offs;
  int nj, lane;
  // block jj's record: present (jj < nj), in range and of a sane size
  __device__ __forceinline__ bool locate(int jj, uint64_t& o, uint32_t& size) const {
    bool fits;
    offs.at(jj, limit, o, size, fits);
    return jj < nj && fits && size >= 16u && size <= (uint32_t)REC;
  }
  __device__ __forceinline__ void request(int jj, u32x4 (&pre)[NCH]) const {
    uint64_t o;
    uint32_t size;
    const bool ok = locate(jj, o, size);
    load_record<NCH>(arena + o, ok ? size : 0u, lane, pre);
  }
  // size of block jj's record, 0 if jj is missing; rok: present, in range and sane
  __device__ __forceinline__ uint32_t size_of(int jj, bool& rok) const {
    uint64_t o;
    uint32_t size;
    rok = locate(jj, o, size);
    return rok ? size : 0u;
  }
};

// Occupancy asked of the register allocator for the K GEMV: at 2 and 3 bits
// with one query and 64-token blocks 6 waves per SIMD (80 VGPRs, a few
// values kept in scratch outside the block loop; measured 3-4 % faster than
// 5 waves), at 4 bits the allocator's own choice (6 waves there: 4.5 %
// slower); with four queries on the matrix cores and 128-token blocks 3
// waves (154 VGPRs instead of 188, no scratch; 17.5 % faster than 2 waves).
// (Tuned at D = 128.)
template <int B, int BITS, int GT, int D>
constexpr int qk_waves_per_eu() {
  return D != 128 ? 1 : B == 64 && BITS <= 3 && GT == 1 ? 6 : B == 128 && BITS <= 4 && GT > 1 ? 3 : 1;
}

// WS: the K records are in payload order 1 (a separate instantiation, so
// that the default one carries none of its code).
template <int B, int BITS, int GT, int D, bool WS = false>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(qk_waves_per_eu<B, BITS, GT, D>())))
void k_qk_gemv(GemvArgs a) {
  using KB = KSel<B, BITS, GT, D, WS>;
  constexpr int REC = max_record_bytes(false, B, BITS, D);
  constexpr int NCH = (REC + 1023) / 1024;
  constexpr int BUF = staging_bytes(REC) > KB::SCRATCH_BYTES ? staging_bytes(REC) : KB::SCRATCH_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t rec[BUF];
  __shared__ __attribute__((aligned(16))) uint8_t qs[KB::QS_BYTES];

  const int lane = threadIdx.x;
  const int s = blockIdx.x / a.splits;
  const int split = blockIdx.x % a.splits;
  const int j0 = split * a.blocks_per_wg;
  const int nj = max(0, min(a.nb, j0 + a.blocks_per_wg) - j0);
  RecordStream<NCH, REC> rs;
  rs.arena = a.arena + (uint64_t)s * a.arena_stride;
  rs.limit = (uint32_t)a.arena_stride;
  rs.offs.load(a.off + (int64_t)s * a.off_stride, j0, nj, lane);
  // tokens from the window's first block on (at most nj * B)
  const int rem = (int)max((int64_t)0, imin64(a.n_tokens - (int64_t)j0 * B, (int64_t)nj * B));
  rs.nj = nj;
  rs.lane = lane;
  KB kb;
  kb.init(qs, lane);
  if constexpr (BITS > 4) kb.bits = a.bits;
  bool corrupt = false;

  for (int gq0 = 0; gq0 < a.G; gq0 += GT) {
    kb.set_queries(a.q, s, a.G, gq0);
    auto process = [&](int jj, u32x4 (&pre)[NCH]) __attribute__((always_inline)) {
      const int j = j0 + jj;
      bool rok;
      const uint32_t size = rs.size_of(jj, rok);
      corrupt |= jj < nj && !rok;
      const int n = jj < nj ? min(B, rem - jj * B) : 0;
      wave_sync();
      store_record<NCH>(rec, pre, lane);
      rs.request(jj + 1, pre);
      __builtin_amdgcn_sched_barrier(0);
      wave_sync();
      // range-checked stores: slots past n, absent queries and corrupt
      // records write nothing
      const bool ok = kb.run(rec, size, (n + kR - 1) / kR, [&](int g, int h, float v, bool dok) {
        const uint32_t valid = dok && rok ? (uint32_t)max(0, min(64, n - h * 64)) : 0u;
        const bool gok = gq0 + g < a.G;
        float* row0 = a.scores + ((int64_t)s * a.G + (gok ? gq0 + g : 0)) * a.ld + (int64_t)j * B + h * 64;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), buffer_rsrc(row0, gok ? 4u * valid : 0u),
                                              4 * lane, 0, 0);
      }) && rok;
      corrupt |= rok && !ok;
    };
    u32x4 pre[NCH];
    rs.request(0, pre);
    for (int jj = 0; jj < nj; ++jj) process(jj, pre);
  }
  if (corrupt && lane == 0) latch(a.status, PACKKV_ECORRUPT);
}

// Split-T reduction of the V GEMV and of fused attention: each workgroup
// stores its partial results with device-coherent stores (they go past this
// XCD's L2), waits for them, and takes a ticket from the stream's counter.
// The workgroup that draws the last ticket is the only one that goes on: it
// reads every partial back with device-coherent loads, sums them in split
// order (so the result does not depend on which workgroup it is), and puts
// the counter back to zero for the next call.  No cache write-back or
// invalidation is needed; a release fence in every workgroup (an L2
// write-back on this multi-XCD part) made the V GEMV three times slower.
__device__ __forceinline__ float load_partial(const float* src) {
  return __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool last_to_arrive(uint32_t* ticket, int splits, int lane) {
  __builtin_amdgcn_s_waitcnt(0x0F70);                // vmcnt(0): partials stored
  uint32_t t = 0;
  if (lane == 0) t = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  t = __builtin_amdgcn_readfirstlane(t);
  return t == (uint32_t)splits - 1u;
}
__device__ __forceinline__ void reset_ticket(uint32_t* ticket, int lane) {
  if (lane == 0) __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Occupancy asked of the register allocator: 64-token blocks with one query
// fit 96 VGPRs (5 waves per SIMD), 128-token blocks 168 (3 waves); either
// costs at most a few values kept in scratch outside the block loop
// (D = 128; other head_dims leave the allocator free)
template <int B, int GT, int D>
constexpr int pv_waves_per_eu() { return D != 128 ? 1 : B == 64 && GT == 1 ? 5 : B == 128 ? 3 : 1; }

template <int B, int BITS, int GT, int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(pv_waves_per_eu<B, GT, D>())))
void k_pv_gemv(GemvArgs a) {
  using VB = VSel<B, BITS, GT, D>;
  constexpr int NH = VB::NH;
  constexpr int NA = VB::NA;
  constexpr int REC = max_record_bytes(true, B, BITS, D);
  constexpr int NCH = (REC + 1023) / 1024;
  constexpr int BUF = staging_bytes(REC) > VB::SCRATCH_BYTES ? staging_bytes(REC) : VB::SCRATCH_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t rec[BUF];
  __shared__ __attribute__((aligned(16))) uint32_t dig[VB::LDS_WORDS];

  const int lane = threadIdx.x;
  const int s = blockIdx.x / a.splits;
  const int split = blockIdx.x % a.splits;
  const int j0 = split * a.blocks_per_wg;
  const int nj = max(0, min(a.nb, j0 + a.blocks_per_wg) - j0);
  RecordStream<NCH, REC> rs;
  rs.arena = a.arena + (uint64_t)s * a.arena_stride;
  rs.limit = (uint32_t)a.arena_stride;
  rs.offs.load(a.off + (int64_t)s * a.off_stride, j0, nj, lane);
  // tokens from the window's first block on (at most nj * B)
  const int rem = (int)max((int64_t)0, imin64(a.n_tokens - (int64_t)j0 * B, (int64_t)nj * B));
  rs.nj = nj;
  rs.lane = lane;
  VB vb;
  vb.init(dig, lane);
  if constexpr (BITS > 4) vb.bits = a.bits;
  bool corrupt = false, invalid = false;

  for (int gq0 = 0; gq0 < a.G; gq0 += GT) {
    float acc[GT][NA];
    float pz[GT];
#pragma unroll
    for (int g = 0; g < GT; ++g) {
#pragma unroll
      for (int j = 0; j < NA; ++j) acc[g][j] = 0.f;
      pz[g] = 0.f;
    }
    // weights of the lane's slots (slot h*64 + lane) for block jj; zero past
    // the valid slots, for absent queries and missing blocks
    auto load_p = [&](int jj, float (&pv)[GT][NH]) __attribute__((always_inline)) {
      const bool in = jj < nj;
      const int left = rem - jj * B;
      const uint32_t nbytes = in && left > 0 ? 4u * (uint32_t)min(B, left) : 0u;
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        const bool gok = gq0 + g < a.G;
        const float* src = a.p + ((int64_t)s * a.G + (gok ? gq0 + g : 0)) * a.ld + (int64_t)(in ? j0 + jj : 0) * B;
        const __amdgpu_buffer_rsrc_t r = buffer_rsrc(src, gok ? nbytes : 0u);
#pragma unroll
        for (int h = 0; h < NH; ++h)
          pv[g][h] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, 4 * (h * 64 + lane), 0, 0));
      }
    };
    auto request = [&](int jj, u32x4 (&pre)[NCH], float (&pv)[GT][NH]) __attribute__((always_inline)) {
      rs.request(jj, pre);
      load_p(jj, pv);
    };
    auto process = [&](int jj, u32x4 (&pre)[NCH], float (&pv)[GT][NH]) __attribute__((always_inline)) {
      const int j = j0 + jj;
      bool rok;
      const uint32_t size = rs.size_of(jj, rok);
      corrupt |= jj < nj && !rok;
      const int n = jj < nj ? min(B, rem - jj * B) : 0;
      wave_sync();
      store_record<NCH>(rec, pre, lane);
      float pw[GT][NH];
#pragma unroll
      for (int g = 0; g < GT; ++g)
#pragma unroll
        for (int h = 0; h < NH; ++h) pw[g][h] = pv[g][h];
      // the fixed-point weights need p >= 0 and finite (softmax weights); a
      // block holding any other weight takes no part and latches EINVAL
      bool badp = false;
#pragma unroll
      for (int g = 0; g < GT; ++g)
#pragma unroll
        for (int h = 0; h < NH; ++h) badp |= !(pw[g][h] >= 0.f && pw[g][h] <= __FLT_MAX__);
      const bool pok = __ballot(badp) == 0;
      invalid |= !pok;
      request(jj + 1, pre, pv);
      __builtin_amdgcn_sched_barrier(0);
      wave_sync();
      const bool ok = vb.run(rec, size, (n + kR - 1) / kR, rok && pok, pw, acc, pz);
      corrupt |= rok && pok && !ok;
    };
    // one record (and its weights) in flight
    u32x4 pre[NCH];
    float pv[GT][NH];
    request(0, pre, pv);
    for (int jj = 0; jj < nj; ++jj) process(jj, pre, pv);
    // partial result of this split
    float z[GT];
#pragma unroll
    for (int g = 0; g < GT; ++g) z[g] = wave_sum(pz[g]);
    vb.store(acc, z, [&](int g) -> float* {
      return gq0 + g < a.G ? a.ws + (((int64_t)s * a.G + gq0 + g) * a.splits + split) * D : nullptr;
    });
  }
  if (corrupt && lane == 0) latch(a.status, PACKKV_ECORRUPT);
  if (invalid && lane == 0) latch(a.status, PACKKV_EINVAL);
  if (!last_to_arrive(&a.tickets[s], a.splits, lane)) return;
  // Merge in a fixed order: a half-wave adds up every other split (even
  // splits in half 0, odd in half 1, each in split order) for NPL = D/32
  // channels per lane, then the two halves are added.  The coherent loads
  // of NU splits per half-wave are issued together, so 2 NU splits cost one
  // memory round trip; a split past the last one reads zeros.
  constexpr int NPL = D / 32;
  constexpr int NU = NPL <= 4 ? 8 : 4;
  constexpr uint32_t PB = D * 4;                    // bytes per partial
  const int half = lane >> 5, d0 = (lane & 31) * NPL;
  for (int g = 0; g < a.G; ++g) {
    const float* src = a.ws + ((int64_t)s * a.G + g) * a.splits * D;
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(src, (uint32_t)a.splits * PB);
    float o[NPL];
#pragma unroll
    for (int k = 0; k < NPL; ++k) o[k] = 0.f;
    for (int i0 = 0; i0 < a.splits; i0 += 2 * NU) {
      uint32_t v[NU][NPL];
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const uint32_t off = (uint32_t)(i0 + 2 * u + half) * PB + 4u * (uint32_t)d0;
        if constexpr (NPL == 2) {
          const u32x2 t = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCoherent));
          v[u][0] = t[0];
          v[u][1] = t[1];
        } else {
#pragma unroll
          for (int c = 0; c < NPL; c += 4) {
            const u32x4 t = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 4 * c, 0, kCoherent));
#pragma unroll
            for (int k = 0; k < 4; ++k) v[u][c + k] = t[k];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < NU; ++u)
#pragma unroll
        for (int k = 0; k < NPL; ++k) o[k] += __uint_as_float(v[u][k]);
    }
#pragma unroll
    for (int k = 0; k < NPL; ++k) o[k] += __shfl_xor(o[k], 32, kWave);
    if (half == 0) {
      float* dst = a.out + ((int64_t)s * a.G + g) * D + d0;
#pragma unroll
      for (int c = 0; c < NPL; ++c) dst[c] = o[c];   // out needs only 4-byte alignment
    }
  }
  reset_ticket(&a.tickets[s], lane);
}

// ---------------------------------------------------------------------------
// Fused decode attention:
//
//   out[g] = sum_t softmax_t(scale * q_g . K_hat[t]) V_hat[t]
//
// in one pass over both packed caches, with no scores or weights in HBM.
// A workgroup of two waves takes J consecutive blocks of one stream.  Wave 0
// streams the K records: for each block the K block code gives the scores,
// which go to an LDS slot (block jj & 1).  Wave 1 streams the V records: a
// running-max softmax update turns block jj's scores into weights exp(s - m)
// (earlier sums are rescaled when m grows), and the V block code takes them
// with the V record of the same block.  One workgroup barrier per block hands
// the scores over, so wave 0 scores block jj + 1 while wave 1 finishes block
// jj.  Each split leaves (partial out[D], its max m, its weight sum l); the
// last workgroup of the stream merges the splits with the usual rescaling.
__device__ __forceinline__ float wave_max_f(float v) {
  // fp32 order is the unsigned order of the key bits ^ 0x80000000 (x >= 0)
  // or ~bits (x < 0); a lane without a DPP source reads key 0, the lowest
  const uint32_t b = __float_as_uint(v);
  uint32_t k = b ^ ((uint32_t)((int)b >> 31) | 0x80000000u);
  k = max(k, (uint32_t)dpp_i<0x111>((int)k));
  k = max(k, (uint32_t)dpp_i<0x112>((int)k));
  k = max(k, (uint32_t)dpp_i<0x114>((int)k));
  k = max(k, (uint32_t)dpp_i<0x118>((int)k));
  k = max(k, (uint32_t)dpp_i<0x142, 0xA>((int)k));
  k = max(k, (uint32_t)dpp_i<0x143, 0xC>((int)k));
  const uint32_t r = readlane_u32(k, 63);
  return __uint_as_float(r ^ (r >> 31 ? 0x80000000u : 0xFFFFFFFFu));
}
// 2^x without the range fix-ups of exp2f: arguments here are <= 0 and a
// result that underflows is a weight of 0
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Occupancy asked of the register allocator: 3 waves per SIMD (168 VGPRs)
// for 128-token blocks and 5 (96 VGPRs) for 2-bit 64-token blocks with one
// query, where the few values it has to spill are read once per query group
// (measured: 2-bit 266 -> 249 us; at 4 bits 5 waves gain nothing).  The
// other shapes keep every value in registers.  (Tuned at D = 128; other
// head_dims leave the allocator free.)
template <int B, int BITS, int GT, int D>
constexpr int attn_waves_per_eu() { return D != 128 ? 1 : B == 128 ? 3 : B == 64 && BITS == 2 && GT == 1 ? 5 : 1; }

template <int B, int BITS, int GT, int D, bool PAGED, bool WS = false>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(attn_waves_per_eu<B, BITS, GT, D>())))
void k_attn_decode(AttnArgs a) {
  using KB = KSel<B, BITS, GT, D, WS>;
  using VB = VSel<B, BITS, GT, D, false>;
  constexpr int NH = B / 64;
  constexpr int PF = attn_partial_floats(D);      // floats per split partial
  constexpr int REC_K = max_record_bytes(false, B, BITS, D);
  constexpr int REC_V = max_record_bytes(true, B, BITS, D);
  constexpr int NCH_K = (REC_K + 1023) / 1024;
  constexpr int NCH_V = (REC_V + 1023) / 1024;
  constexpr int BUF_K = staging_bytes(REC_K) > KB::SCRATCH_BYTES ? staging_bytes(REC_K) : KB::SCRATCH_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t rec_k[BUF_K];
  constexpr int BUF_V = staging_bytes(REC_V) > VB::SCRATCH_BYTES ? staging_bytes(REC_V) : VB::SCRATCH_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t rec_v[BUF_V];
  __shared__ __attribute__((aligned(16))) uint8_t qs[KB::QS_BYTES];
  __shared__ __attribute__((aligned(16))) uint32_t dig[VB::LDS_WORDS];
  __shared__ __attribute__((aligned(16))) float ring[2][GT][B];   // scores of blocks jj & 1

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform per wave
  const int lane = threadIdx.x & 63;
  // this workgroup's cache (blockIdx.y) and its slices of q, out and the workspace
  const AttnCache& cache = a.cache[blockIdx.y];
  const uint16_t* q = a.q + blockIdx.y * a.qo_stride;
  float* out = a.out + blockIdx.y * a.qo_stride;
  float* ws = reinterpret_cast<float*>(a.ws + blockIdx.y * a.ws_stride);
  uint32_t* tickets = reinterpret_cast<uint32_t*>(a.tk + blockIdx.y * a.tk_stride);
  const int s = blockIdx.x / a.splits;
  const int split = blockIdx.x % a.splits;
  // the stream's length: one for the cache, or (paged) the stream's own
  int64_t n_tokens = a.n_tokens;
  int nb = a.nb;
  if constexpr (PAGED) {
    n_tokens = __builtin_amdgcn_readfirstlane(cache.lengths[s]);
    nb = (int)((n_tokens + B - 1) / B);
  }
  // the splits divide the blocks evenly: floor or ceil of nb / splits each
  const int j0 = (int)((int64_t)split * nb / a.splits);
  int nj = (int)((int64_t)(split + 1) * nb / a.splits) - j0;
  bool corrupt = false;
  if (PAGED && nj > 64) {                           // a length the launch was not sized for
    nj = 64;
    corrupt = true;
  }
  using Loc = std::conditional_t<PAGED, RecordTable, RecordOffsets>;
  const uint32_t limit = (uint32_t)(PAGED ? a.arena_stride >> 4 : a.arena_stride);
  // tokens from the window's first block on (at most nj * B)
  const int rem = (int)max((int64_t)0, imin64(n_tokens - (int64_t)j0 * B, (int64_t)nj * B));
  const float NEG_INF = -__builtin_huge_valf();

  // Both waves pass the same barriers: one per block and one per query group.
  // With a tile of several queries on the matrix cores the K wave sets the
  // pace of each block; it issues first where the two kinds of wave share a
  // SIMD (measured: four queries -7 %; with one query either order is level
  // or slower, so the vector kernels leave the priority alone).
  if (std::is_same_v<KB, KBlockM<B, BITS, GT>> && wave == 0) __builtin_amdgcn_s_setprio(2);
  if (wave == 0) {
    for (int gq0 = 0; gq0 < a.G; gq0 += GT) {
      // K wave: the scores of every block, handed over through the ring
      // with one workgroup barrier per block
      RecordStream<NCH_K, REC_K, Loc> ks;
      if constexpr (PAGED) {
        ks.arena = cache.k_arena;
        ks.offs.load(cache.k_tab + (int64_t)s * a.off_stride, j0, nj, lane);
      } else {
        ks.arena = cache.k_arena + (uint64_t)s * a.arena_stride;
        ks.offs.load(cache.k_off + (int64_t)s * a.off_stride, j0, nj, lane);
      }
      ks.limit = limit;
      ks.nj = nj;
      ks.lane = lane;
      KB kb;
      kb.init(qs, lane);
      if constexpr (BITS > 4) kb.bits = a.bits;
      kb.set_queries(q, s, a.G, gq0);
      u32x4 pre[NCH_K];
      ks.request(0, pre);
      for (int jj = 0; jj < nj; ++jj) {
        const int n = min(B, rem - jj * B);
        bool rok;
        const uint32_t size = ks.size_of(jj, rok);
        corrupt |= !rok;
        wave_sync();
        store_record<NCH_K>(rec_k, pre, lane);
        ks.request(jj + 1, pre);
        __builtin_amdgcn_sched_barrier(0);
        wave_sync();
        const bool ok = kb.run(rec_k, size, (n + kR - 1) / kR, [&](int g, int h, float v, bool dok) {
          ring[jj & 1][g][h * 64 + lane] = dok && rok && h * 64 + lane < n ? v * a.scale_log2e : NEG_INF;
        }) && rok;
        corrupt |= rok && !ok;
        __syncthreads();                            // block jj goes to the V wave
      }
      __syncthreads();                              // the ring is reused
    }
  } else {
    for (int gq0 = 0; gq0 < a.G; gq0 += GT) {
      // V wave: running-max softmax over the scores, weighted sum of V
      RecordStream<NCH_V, REC_V, Loc> vs;
      if constexpr (PAGED) {
        vs.arena = cache.v_arena;
        vs.offs.load(cache.v_tab + (int64_t)s * a.off_stride, j0, nj, lane);
      } else {
        vs.arena = cache.v_arena + (uint64_t)s * a.arena_stride;
        vs.offs.load(cache.v_off + (int64_t)s * a.off_stride, j0, nj, lane);
      }
      vs.limit = limit;
      vs.nj = nj;
      vs.lane = lane;
      VB vb;
      vb.init(dig, lane);
      if constexpr (BITS > 4) vb.bits = a.bits;
      float m[GT], l[GT], acc[GT][VB::NA], pz[GT];
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        m[g] = NEG_INF;
        l[g] = 0.f;
        pz[g] = 0.f;
#pragma unroll
        for (int j = 0; j < VB::NA; ++j) acc[g][j] = 0.f;
      }
      u32x4 pre[NCH_V];
      vs.request(0, pre);
      for (int jj = 0; jj < nj; ++jj) {
        const int n = min(B, rem - jj * B);
        __syncthreads();                            // block jj's scores are in the ring
        // weights exp(s - m); earlier sums rescaled when m grows
        float w[GT][NH], al[GT];
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          float sc[NH];
#pragma unroll
          for (int h = 0; h < NH; ++h) sc[h] = ring[jj & 1][g][h * 64 + lane];
          float mx = sc[0];
#pragma unroll
          for (int h = 1; h < NH; ++h) mx = fmaxf(mx, sc[h]);
          const float mn = fmaxf(m[g], wave_max_f(mx));
          const float alpha = mn == NEG_INF ? 1.f : fast_exp2(m[g] - mn);
          al[g] = alpha;
          pz[g] *= alpha;
          l[g] *= alpha;
          m[g] = mn;
#pragma unroll
          for (int h = 0; h < NH; ++h) {
            w[g][h] = mn == NEG_INF ? 0.f : fast_exp2(sc[h] - mn);
            l[g] += w[g][h];
          }
        }
        vb.rescale(acc, al);
        bool rok;
        const uint32_t size = vs.size_of(jj, rok);
        corrupt |= !rok;
        wave_sync();
        store_record<NCH_V>(rec_v, pre, lane);
        vs.request(jj + 1, pre);
        __builtin_amdgcn_sched_barrier(0);
        wave_sync();
        const bool ok = vb.run(rec_v, size, (n + kR - 1) / kR, rok, w, acc, pz);
        corrupt |= rok && !ok;
      }
      // this split's partial: out sums, max, weight sum
      float z[GT];
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        z[g] = wave_sum(pz[g]);
        const float lsum = wave_sum(l[g]);
        if (gq0 + g < a.G && lane == 0) {
          float* dst = ws + (((int64_t)s * a.G + gq0 + g) * a.splits + split) * PF;
          store_partial(dst + D, m[g]);
          store_partial(dst + D + 1, lsum);
        }
      }
      vb.store(acc, z, [&](int g) -> float* {
        return gq0 + g < a.G ? ws + (((int64_t)s * a.G + gq0 + g) * a.splits + split) * PF : nullptr;
      });
      __syncthreads();                              // the ring is reused
    }
  }
  if (corrupt && lane == 0) latch(cache.status, PACKKV_ECORRUPT);
  if (wave != 1 || !last_to_arrive(&tickets[s], a.splits, lane)) return;
  // Merge: the largest split max M first (lanes across splits), then each
  // split's sums scaled by 2^(m_i - M).  A half-wave takes every other split
  // (in split order) and a lane NPL = D/32 of the outputs; the loads of NU
  // splits per half-wave are issued together, those of the first NU before
  // the max is known, so that up to 2 NU splits cost two memory round trips.
  constexpr int NPL = D / 32;
  constexpr int NU = NPL <= 4 ? 8 : 4;
  const int half = lane >> 5, d0 = (lane & 31) * NPL;
  constexpr uint32_t PB = PF * 4;                   // bytes per partial
  for (int g = 0; g < a.G; ++g) {
    const float* src = ws + ((int64_t)s * a.G + g) * a.splits * PF;
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(src, (uint32_t)a.splits * PB);
    uint32_t v[NU][NPL];
    u32x2 ml[NU];
    auto load_batch = [&](int i0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const uint32_t off = (uint32_t)(i0 + 2 * u + half) * PB;   // past the end reads zeros
        if constexpr (NPL == 2) {
          const u32x2 t = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off + 4 * d0, 0, kCoherent));
          v[u][0] = t[0];
          v[u][1] = t[1];
        } else {
#pragma unroll
          for (int c = 0; c < NPL; c += 4) {
            const u32x4 t =
                __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 4 * (d0 + c), 0, kCoherent));
#pragma unroll
            for (int k = 0; k < 4; ++k) v[u][c + k] = t[k];
          }
        }
        ml[u] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off + 4 * D, 0, kCoherent));
      }
    };
    load_batch(0);
    float M = NEG_INF;
    for (int i = lane; i < a.splits; i += 64) M = fmaxf(M, load_partial(src + (int64_t)i * PF + D));
    M = wave_max_f(M);
    float L = 0.f, o[NPL];
#pragma unroll
    for (int k = 0; k < NPL; ++k) o[k] = 0.f;
    for (int i0 = 0; i0 < a.splits; i0 += 2 * NU) {
      if (i0 > 0) load_batch(i0);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const bool in = i0 + 2 * u + half < a.splits && M != NEG_INF;
        const float f = in ? fast_exp2(__uint_as_float(ml[u].x) - M) : 0.f;
        L = fmaf(__uint_as_float(ml[u].y), f, L);
#pragma unroll
        for (int k = 0; k < NPL; ++k) o[k] = fmaf(__uint_as_float(v[u][k]), f, o[k]);
      }
    }
    L += __shfl_xor(L, 32, kWave);
#pragma unroll
    for (int k = 0; k < NPL; ++k) o[k] += __shfl_xor(o[k], 32, kWave);
    if (half == 0) {
      // an empty stream (paged) has no weights: its output is zero
      float* dst = out + ((int64_t)s * a.G + g) * D + d0;
#pragma unroll
      for (int c = 0; c < NPL; c += 2)
        *reinterpret_cast<float2*>(dst + c) = float2{L > 0.f ? o[c] / L : 0.f, L > 0.f ? o[c + 1] / L : 0.f};
    }
  }
  reset_ticket(&tickets[s], lane);
}

// ---------------------------------------------------------------------------
// Decompress (test path): mode 0 -> u8 q in slot order, mode 1 -> fp32 x_hat
// in token order.
template <int B, bool IS_V, bool WIDE, int D>
__global__ __launch_bounds__(64) void k_decompress(GemvArgs a, const uint8_t* perm, int64_t perm_stride,
                                                   int mode, void* out) {
  constexpr int NR = B / kR;
  constexpr int NRL = NR * D / 64;
  constexpr int HB = WIDE ? 2 : 1;
  constexpr int REC = max_record_bytes(IS_V, B, WIDE ? 8 : 4, D);
  constexpr int NCH = (REC + 1023) / 1024;
  constexpr int HDR = hdr_offset(IS_V, B, D);
  __shared__ __attribute__((aligned(16))) uint8_t rec[staging_bytes(REC)];
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
  {
    // chunk by chunk (the largest records would not fit one register batch)
    const __amdgpu_buffer_rsrc_t rr = buffer_rsrc(arena + o, size);
    u32x4* dst = reinterpret_cast<u32x4*>(rec);
    for (int k = 0; k < NCH; ++k)
      dst[lane + 64 * k] =
          __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, 16 * (lane + 64 * k), 0, kNonTemporal));
  }
  __syncthreads();
  const int pay = payload_offset(IS_V, B, nr, HB, D);
  int w[NRL];
  uint32_t m[NRL], ro[NRL];
  bool full;
  if (!scan_runs<NRL, HB, D / 64>(rec, HDR, pay, size, nr * D, a.bits, lane, w, m, ro, full,
                                  a.korder == 1)) {
    if (lane == 0) latch(a.status, PACKKV_ECORRUPT);
    return;
  }
  const uint16_t* sc = reinterpret_cast<const uint16_t*>(rec);
  const uint8_t* pm = perm + (int64_t)s * perm_stride + (int64_t)j * B;
#pragma unroll
  for (int k = 0; k < NRL; ++k) {
    const int ri = lane + 64 * k;
    const int r = ri / D, c = ri % D;
    if (r >= nr) continue;
    // the run's containers: nibbles holding q (b <= 4) or bytes holding u
    uint32_t nib[4], byt[8];
    if constexpr (!WIDE) {
      uint32_t wd[4];
      run_words(rec, pay, ro[k], false, wd);
      run_to_nibbles(w[k], m[k], wd, nib);
    } else {
      // a consistent record keeps the run's w words inside the staging
      const uint32_t* pw = reinterpret_cast<const uint32_t*>(rec + pay) + ro[k];
      uint32_t wd[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) wd[i] = i < w[k] ? pw[i] : 0u;
      switch (w[k]) {
        case 0: sliced_to_bytes<0>(wd, byt); break;
        case 1: sliced_to_bytes<1>(wd, byt); break;
        case 2: sliced_to_bytes<2>(wd, byt); break;
        case 3: sliced_to_bytes<3>(wd, byt); break;
        case 4: sliced_to_bytes<4>(wd, byt); break;
        case 5: sliced_to_bytes<5>(wd, byt); break;
        case 6: sliced_to_bytes<6>(wd, byt); break;
        case 7: sliced_to_bytes<7>(wd, byt); break;
        default: sliced_to_bytes<8>(wd, byt); break;
      }
    }
    for (int i = 0; i < kR; ++i) {
      const int sl = r * kR + i;
      if (sl >= n) break;
      uint32_t qv;
      if constexpr (WIDE) {
        qv = m[k] + ((byt[i >> 2] >> (8 * (i & 3))) & 255u);
      } else {
        qv = (nib[i >> 3] >> (4 * (i & 7))) & 15u;
      }
      if (mode == 0) {
        uint8_t* o8 = reinterpret_cast<uint8_t*>(out);
        o8[(((int64_t)s * a.n_tokens) + (int64_t)j * B + sl) * D + c] = (uint8_t)qv;
      } else {
        const float scale = f16_bits_to_float(IS_V ? sc[sl] : sc[c]);
        const float zero = f16_bits_to_float(IS_V ? sc[B + sl] : sc[D + c]);
        float* of = reinterpret_cast<float*>(out);
        const int tok = pm[sl];
        if (tok >= n) {
          latch(a.status, PACKKV_ECORRUPT);
          continue;
        }
        const int64_t t = (int64_t)j * B + tok;
        of[((int64_t)s * a.n_tokens + t) * D + c] = fmaf(scale, (float)qv, zero);
      }
    }
  }
}

// Width histogram and byte counts: one wave per record; the lanes' counts
// are summed over the wave first, so a record costs at most a dozen atomics.
template <int B, bool IS_V, bool WIDE, int D>
__global__ __launch_bounds__(64) void k_stats(GemvArgs a, unsigned long long* out) {
  const int lane = threadIdx.x;
  const int s = blockIdx.y, j = blockIdx.x;
  const uint8_t* arena = a.arena + (uint64_t)s * a.arena_stride;
  const uint32_t* offs = a.off + (int64_t)s * a.off_stride;
  const uint32_t o = offs[j], size = offs[j + 1] - o;
  const int n = (int)imin64(B, a.n_tokens - (int64_t)j * B);
  const int nr = (n + kR - 1) / kR;
  if (!record_ok(o, size, a.arena_stride, max_record_bytes(IS_V, B, WIDE ? 8 : 4, D))) {
    if (lane == 0) latch(a.status, PACKKV_ECORRUPT);
    return;
  }
  const uint8_t* hdr = arena + o + hdr_offset(IS_V, B, D);
  int hist[9] = {0, 0, 0, 0, 0, 0, 0, 0, 0};
  int words = 0;
  for (int ri = lane; ri < nr * D; ri += 64) {
    const int w = WIDE ? reinterpret_cast<const uint16_t*>(hdr)[ri] >> 8 : hdr[ri] >> 4;
#pragma unroll
    for (int i = 0; i < 9; ++i) hist[i] += w == i;
    words += w;
  }
  // widths 0..4 at out[0..4] (K) and out[5..9] (V); 5..8 at out[16..19]
  // (K) and out[20..23] (V)
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    const int h = wave_sum_i(hist[i]);
    if (lane == 0 && h) atomicAdd(&out[i < 5 ? (IS_V ? 5 : 0) + i : (IS_V ? 20 : 16) + i - 5], (unsigned long long)h);
  }
  const int wsum = wave_sum_i(words);
  if (lane == 0) {
    if (wsum) atomicAdd(&out[IS_V ? 13 : 12], (unsigned long long)wsum);
    atomicAdd(&out[IS_V ? 11 : 10], (unsigned long long)size);
    atomicAdd(&out[IS_V ? 15 : 14], (unsigned long long)(nr * D));
  }
}

// Softmax over the first T entries of each row: p = exp(s*scale - max)/sum.
// One workgroup of 1024 threads per row: an online (max, sum) pass, then the
// normalising write pass (k_softmax); few or very long rows are cut into
// chunks instead (k_softmax_chunk_*, below).
__device__ __forceinline__ void online_add(float& m, float& sum, float v) {
  if (v > m) {
    sum = sum * __expf(m - v) + 1.0f;
    m = v;
  } else {
    sum += __expf(v - m);
  }
}
__device__ __forceinline__ void online_merge(float& m, float& sum, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) return;
  sum = sum * __expf(m - M) + s2 * __expf(m2 - M);
  m = M;
}

// Four float4 loads per thread are issued before any of them is used (a row
// is one workgroup, and with few rows the chip's HBM is reached only through
// loads in flight); the running (max, sum) is updated once per 16 values.
constexpr int kSoftmaxUnroll = 4;

__device__ __forceinline__ void online_add16(float& m, float& sum, const float4 (&v)[kSoftmaxUnroll], float scale) {
  float lm = -INFINITY;
#pragma unroll
  for (int u = 0; u < kSoftmaxUnroll; ++u)
    lm = fmaxf(lm, fmaxf(fmaxf(v[u].x, v[u].y), fmaxf(v[u].z, v[u].w)) * scale);
  const float M = fmaxf(m, lm);
  if (M == -INFINITY) return;
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < kSoftmaxUnroll; ++u)
    s += __expf(v[u].x * scale - M) + __expf(v[u].y * scale - M) + __expf(v[u].z * scale - M) +
         __expf(v[u].w * scale - M);
  sum = sum * __expf(m - M) + s;
  m = M;
}

__global__ __launch_bounds__(1024) void k_softmax(const float* scores, float* p, int64_t T, int64_t ld,
                                                  float scale) {
  constexpr int U = kSoftmaxUnroll;
  __shared__ float sm[16], ss[16];
  const float* x = scores + (int64_t)blockIdx.x * ld;
  float* y = p + (int64_t)blockIdx.x * ld;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool vec = ((ld & 3) == 0) && ((reinterpret_cast<uintptr_t>(scores) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(p) & 15) == 0);
  const int64_t T4 = vec ? (T >> 2) : 0;
  const float4* x4 = reinterpret_cast<const float4*>(x);
  float m = -INFINITY, sum = 0.f;
  int64_t i = tid;
  for (; i + (U - 1) * 1024 < T4; i += U * 1024) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = x4[i + u * 1024];
    online_add16(m, sum, v, scale);
  }
  for (; i < T4; i += 1024) {
    const float4 v = x4[i];
    online_add(m, sum, v.x * scale);
    online_add(m, sum, v.y * scale);
    online_add(m, sum, v.z * scale);
    online_add(m, sum, v.w * scale);
  }
  for (int64_t k = 4 * T4 + tid; k < T; k += 1024) online_add(m, sum, x[k] * scale);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, kWave), s2 = __shfl_xor(sum, o, kWave);
    online_merge(m, sum, m2, s2);
  }
  if (lane == 0) { sm[wv] = m; ss[wv] = sum; }
  __syncthreads();
  m = sm[0];
  sum = ss[0];
  for (int k = 1; k < 16; ++k) online_merge(m, sum, sm[k], ss[k]);
  const float inv = 1.0f / sum;
  float4* y4 = reinterpret_cast<float4*>(y);
  i = tid;
  for (; i + (U - 1) * 1024 < T4; i += U * 1024) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = x4[i + u * 1024];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float4 r;
      r.x = __expf(v[u].x * scale - m) * inv;
      r.y = __expf(v[u].y * scale - m) * inv;
      r.z = __expf(v[u].z * scale - m) * inv;
      r.w = __expf(v[u].w * scale - m) * inv;
      y4[i + u * 1024] = r;
    }
  }
  for (; i < T4; i += 1024) {
    const float4 v = x4[i];
    float4 r;
    r.x = __expf(v.x * scale - m) * inv;
    r.y = __expf(v.y * scale - m) * inv;
    r.z = __expf(v.z * scale - m) * inv;
    r.w = __expf(v.w * scale - m) * inv;
    y4[i] = r;
  }
  for (int64_t k = 4 * T4 + tid; k < T; k += 1024) y[k] = __expf(x[k] * scale - m) * inv;
}

// Chunked softmax for long rows that are too few to fill the chip one
// workgroup each.  Row r is cut into nchunks chunks of kSoftmaxChunk entries,
// the last one taking the remainder (so every chunk holds at least two).
// (1) each chunk's (max, sum) goes to the first two entries of its own range
// of p; (2) one wave per row merges them and writes the row's (max, 1/sum)
// over every chunk's pair; (3) each chunk reads its pair, then writes its
// outputs over the whole range.  p must not alias scores.
constexpr int kSoftmaxChunk = 8192;

__device__ __forceinline__ void softmax_chunk_range(int c, int nchunks, int64_t T, int64_t& lo, int64_t& hi) {
  lo = (int64_t)c * kSoftmaxChunk;
  hi = c == nchunks - 1 ? T : lo + kSoftmaxChunk;
}

__global__ __launch_bounds__(256) void k_softmax_chunk_stats(const float* scores, float* p, int64_t T, int64_t ld,
                                                             float scale, int nchunks) {
  constexpr int U = kSoftmaxUnroll;
  __shared__ float sm[4], ss[4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float* x = scores + (int64_t)blockIdx.y * ld;
  int64_t lo, hi;
  softmax_chunk_range(blockIdx.x, nchunks, T, lo, hi);
  const bool vec = ((ld & 3) == 0) && ((reinterpret_cast<uintptr_t>(scores) & 15) == 0);
  // chunk starts are multiples of 4 entries: float4 j covers entries 4j..4j+3
  const int64_t v0 = vec ? lo / 4 : 0, v1 = vec ? hi / 4 : 0;
  const float4* x4 = reinterpret_cast<const float4*>(x);
  float m = -INFINITY, sum = 0.f;
  int64_t i = v0 + tid;
  for (; i + (U - 1) * 256 < v1; i += U * 256) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = x4[i + u * 256];
    online_add16(m, sum, v, scale);
  }
  for (; i < v1; i += 256) {
    const float4 v = x4[i];
    online_add(m, sum, v.x * scale);
    online_add(m, sum, v.y * scale);
    online_add(m, sum, v.z * scale);
    online_add(m, sum, v.w * scale);
  }
  for (int64_t k = (vec ? 4 * v1 : lo) + tid; k < hi; k += 256) online_add(m, sum, x[k] * scale);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, kWave), s2 = __shfl_xor(sum, o, kWave);
    online_merge(m, sum, m2, s2);
  }
  if (lane == 0) { sm[wv] = m; ss[wv] = sum; }
  __syncthreads();
  if (tid == 0) {
    for (int k = 1; k < 4; ++k) online_merge(m, sum, sm[k], ss[k]);
    float* y = p + (int64_t)blockIdx.y * ld + lo;
    y[0] = m;
    y[1] = sum;
  }
}

__global__ __launch_bounds__(64) void k_softmax_merge(float* p, int64_t ld, int nchunks) {
  const int lane = threadIdx.x;
  float* y = p + (int64_t)blockIdx.x * ld;
  float m = -INFINITY, sum = 0.f;
  for (int c = lane; c < nchunks; c += 64) {
    const int64_t lo = (int64_t)c * kSoftmaxChunk;
    online_merge(m, sum, y[lo], y[lo + 1]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float m2 = __shfl_xor(m, o, kWave), s2 = __shfl_xor(sum, o, kWave);
    online_merge(m, sum, m2, s2);
  }
  // every lane holds the row's (max, sum) now; the pairs are overwritten
  // only after all of them were read (one wave, loads before stores)
  const float inv = 1.0f / sum;
  for (int c = lane; c < nchunks; c += 64) {
    const int64_t lo = (int64_t)c * kSoftmaxChunk;
    y[lo] = m;
    y[lo + 1] = inv;
  }
}

__global__ __launch_bounds__(256) void k_softmax_chunk_norm(const float* scores, float* p, int64_t T, int64_t ld,
                                                            float scale, int nchunks) {
  constexpr int U = kSoftmaxUnroll;
  __shared__ float mi[2];
  const int tid = threadIdx.x;
  const float* x = scores + (int64_t)blockIdx.y * ld;
  float* y = p + (int64_t)blockIdx.y * ld;
  int64_t lo, hi;
  softmax_chunk_range(blockIdx.x, nchunks, T, lo, hi);
  if (tid == 0) { mi[0] = y[lo]; mi[1] = y[lo + 1]; }
  __syncthreads();                                   // the pair is read before the chunk is written
  const float m = mi[0], inv = mi[1];
  const bool vec = ((ld & 3) == 0) && ((reinterpret_cast<uintptr_t>(scores) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(p) & 15) == 0);
  const int64_t v0 = vec ? lo / 4 : 0, v1 = vec ? hi / 4 : 0;
  const float4* x4 = reinterpret_cast<const float4*>(x);
  float4* y4 = reinterpret_cast<float4*>(y);
  int64_t i = v0 + tid;
  for (; i + (U - 1) * 256 < v1; i += U * 256) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = x4[i + u * 256];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float4 r;
      r.x = __expf(v[u].x * scale - m) * inv;
      r.y = __expf(v[u].y * scale - m) * inv;
      r.z = __expf(v[u].z * scale - m) * inv;
      r.w = __expf(v[u].w * scale - m) * inv;
      y4[i + u * 256] = r;
    }
  }
  for (; i < v1; i += 256) {
    const float4 v = x4[i];
    float4 r;
    r.x = __expf(v.x * scale - m) * inv;
    r.y = __expf(v.y * scale - m) * inv;
    r.z = __expf(v.z * scale - m) * inv;
    r.w = __expf(v.w * scale - m) * inv;
    y4[i] = r;
  }
  for (int64_t k = (vec ? 4 * v1 : lo) + tid; k < hi; k += 256) y[k] = __expf(x[k] * scale - m) * inv;
}

// ---------------------------------------------------------------------------
// Launchers.  Widths 5..8 share one kernel per shape (BITS = 8), which checks
// the record's widths against the configured b at run time.  Shapes are
// dispatched as (B, width class, D); the paged cache is D = 128 only.
static inline int class_bits_or_narrow(int bits) { return bits > 4 ? 8 : bits; }

// f.template operator()<B, BITS, D>() for the cache's shape
template <class F>
static void dispatch_shape(int B, int bits, int D, F&& f) {
  const int cb = class_bits_or_narrow(bits);
  const int key = (B == 128 ? 100 : 0) + (D == 64 ? 0 : D == 128 ? 10 : 20) + cb;
  switch (key) {
#define PACKKV_SHAPE(BB, DD, BI)     case (BB == 128 ? 100 : 0) + (DD == 64 ? 0 : DD == 128 ? 10 : 20) + BI: f.template operator()<BB, BI, DD>(); break;
#define PACKKV_SHAPES(BB, DD) PACKKV_SHAPE(BB, DD, 2) PACKKV_SHAPE(BB, DD, 3) PACKKV_SHAPE(BB, DD, 4) PACKKV_SHAPE(BB, DD, 8)
    PACKKV_SHAPES(64, 64) PACKKV_SHAPES(64, 128) PACKKV_SHAPES(64, 256)
    PACKKV_SHAPES(128, 64) PACKKV_SHAPES(128, 128) PACKKV_SHAPES(128, 256)
#undef PACKKV_SHAPES
#undef PACKKV_SHAPE
    default: break;
  }
}

hipError_t launch_qk(const GemvArgs& a, int B, int n_streams, hipStream_t st) {
  const dim3 grid(n_streams * a.splits);
  dispatch_shape(B, a.bits, a.D, [&]<int BB, int BI, int DD>() {
    if constexpr (BI <= 4) {
      if (a.korder == 1) {
        if (a.G == 1) hipLaunchKernelGGL((k_qk_gemv<BB, BI, 1, DD, true>), grid, dim3(64), 0, st, a);
        else hipLaunchKernelGGL((k_qk_gemv<BB, BI, 4, DD, true>), grid, dim3(64), 0, st, a);
        return;
      }
    }
    if (a.G == 1) hipLaunchKernelGGL((k_qk_gemv<BB, BI, 1, DD>), grid, dim3(64), 0, st, a);
    else hipLaunchKernelGGL((k_qk_gemv<BB, BI, 4, DD>), grid, dim3(64), 0, st, a);
  });
  return hipGetLastError();
}

hipError_t launch_pv(const GemvArgs& a, int B, int n_streams, hipStream_t st) {
  const dim3 grid(n_streams * a.splits);
  dispatch_shape(B, a.bits, a.D, [&]<int BB, int BI, int DD>() {
    if (a.G == 1) hipLaunchKernelGGL((k_pv_gemv<BB, BI, 1, DD>), grid, dim3(64), 0, st, a);
    else hipLaunchKernelGGL((k_pv_gemv<BB, BI, 4, DD>), grid, dim3(64), 0, st, a);
  });
  return hipGetLastError();
}

// Workgroups of the (contiguous-cache) fused attention kernel for this shape
// that are resident on the current device at once: occupancy per compute
// unit times the compute units; 0 if the runtime cannot say.  Asked once per
// shape.
template <int B, int BITS, int GT, int D>
static int resident_wgs_of() {
  int per_cu = 0, dev = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_attn_decode<B, BITS, GT, D, false>, 128, 0) !=
          hipSuccess ||
      hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return per_cu * cus;
}
int attention_resident_wgs(int B, int bits, int G, int D) {
  // [B == 128][D index][bits class][G > 1]: 0 = not asked yet, -1 = unknown.
  // Host threads may race to fill an entry; they store the same value.
  static std::atomic<int> known[2][3][9][2];
  const int cb = class_bits_or_narrow(bits), b1 = B == 128, g1 = G > 1, di = D == 64 ? 0 : D == 128 ? 1 : 2;
  std::atomic<int>& slot = known[b1][di][cb][g1];
  int r = slot.load(std::memory_order_relaxed);
  if (r == 0) {
    int v = 0;
    dispatch_shape(B, bits, D, [&]<int BB, int BI, int DD>() {
      v = g1 ? resident_wgs_of<BB, BI, 4, DD>() : resident_wgs_of<BB, BI, 1, DD>();
    });
    r = v > 0 ? v : -1;
    slot.store(r, std::memory_order_relaxed);
  }
  return r > 0 ? r : 0;
}

hipError_t launch_attention(const AttnArgs& a, int B, int n_streams, int n_caches, hipStream_t st,
                            bool paged) {
  const dim3 grid(n_streams * a.splits, n_caches);
  if (paged) {
    if (a.D != 128) return hipErrorInvalidValue;
    dispatch_shape(B, a.bits, 128, [&]<int BB, int BI, int DD>() {
      if constexpr (DD == 128) {
        if constexpr (BI <= 4) {
          if (a.korder == 1) {
            if (a.G == 1) hipLaunchKernelGGL((k_attn_decode<BB, BI, 1, DD, true, true>), grid, dim3(128), 0, st, a);
            else hipLaunchKernelGGL((k_attn_decode<BB, BI, 4, DD, true, true>), grid, dim3(128), 0, st, a);
            return;
          }
        }
        if (a.G == 1) hipLaunchKernelGGL((k_attn_decode<BB, BI, 1, DD, true>), grid, dim3(128), 0, st, a);
        else hipLaunchKernelGGL((k_attn_decode<BB, BI, 4, DD, true>), grid, dim3(128), 0, st, a);
      }
    });
  } else {
    dispatch_shape(B, a.bits, a.D, [&]<int BB, int BI, int DD>() {
      if constexpr (BI <= 4) {
        if (a.korder == 1) {
          if (a.G == 1) hipLaunchKernelGGL((k_attn_decode<BB, BI, 1, DD, false, true>), grid, dim3(128), 0, st, a);
          else hipLaunchKernelGGL((k_attn_decode<BB, BI, 4, DD, false, true>), grid, dim3(128), 0, st, a);
          return;
        }
      }
      if (a.G == 1) hipLaunchKernelGGL((k_attn_decode<BB, BI, 1, DD, false>), grid, dim3(128), 0, st, a);
      else hipLaunchKernelGGL((k_attn_decode<BB, BI, 4, DD, false>), grid, dim3(128), 0, st, a);
    });
  }
  return hipGetLastError();
}

hipError_t launch_decompress(const GemvArgs& a, int B, bool is_v, int n_streams, const uint8_t* perm,
                             int64_t perm_stride, int mode, void* out, hipStream_t st) {
  dim3 grid(a.nb, n_streams), block(64);
  dispatch_shape(B, a.bits, a.D, [&]<int BB, int BI, int DD>() {
    constexpr bool W = BI > 4;
    if (is_v) hipLaunchKernelGGL((k_decompress<BB, true, W, DD>), grid, block, 0, st, a, perm, perm_stride, mode, out);
    else hipLaunchKernelGGL((k_decompress<BB, false, W, DD>), grid, block, 0, st, a, perm, perm_stride, mode, out);
  });
  return hipGetLastError();
}

hipError_t launch_stats(const GemvArgs& a, int B, bool is_v, int n_streams, unsigned long long* out,
                        hipStream_t st) {
  dim3 grid(a.nb, n_streams), block(64);
  dispatch_shape(B, a.bits, a.D, [&]<int BB, int BI, int DD>() {
    constexpr bool W = BI > 4;
    if (is_v) hipLaunchKernelGGL((k_stats<BB, true, W, DD>), grid, block, 0, st, a, out);
    else hipLaunchKernelGGL((k_stats<BB, false, W, DD>), grid, block, 0, st, a, out);
  });
  return hipGetLastError();
}

// Streaming-read ceiling (a measurement helper, not part of the method):
// a grid-stride read of the buffer, 16 bytes per thread and step in
// 1024-thread workgroups (the steadiest of the shapes measured on 1.24 GB:
// 7.1 TB/s at every grid from 1024 to 16384 workgroups, where contiguous
// shares per workgroup and deeper unrolling ranged 5.7-7.3 TB/s).  Each
// workgroup folds its words with XOR, so the loads cannot be dropped, and
// stores the result to sink[w].  No atomics: thousands of them on one word
// would serialise at the end of the launch and time themselves instead of
// the reads.
constexpr int kReadGroups = 4096;
__global__ __launch_bounds__(1024) void k_stream_read(const u32x4* buf, uint64_t n16, uint32_t* sink) {
  __shared__ uint32_t part[16];
  const uint64_t stride = (uint64_t)gridDim.x * 1024;
  uint32_t x = 0;
  for (uint64_t i = (uint64_t)blockIdx.x * 1024 + threadIdx.x; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(&buf[i]);
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  for (int o = 32; o > 0; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o, kWave);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t y = 0;
    for (int k = 0; k < 16; ++k) y ^= part[k];
    sink[blockIdx.x] = y;
  }
}

hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t st) {
  const uint64_t n16 = bytes / 16;
  uint64_t blocks = (n16 + 1023) / 1024;
  if (blocks > kReadGroups) blocks = kReadGroups;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)blocks), dim3(1024), 0, st, reinterpret_cast<const u32x4*>(buf),
                     n16, sink);
  return hipGetLastError();
}

hipError_t launch_softmax(const float* scores, float* p, int rows, int64_t T, int64_t ld, float scale,
                          hipStream_t st) {
  // Out of place, with fewer rows than compute units or rows of 64K entries
  // and more: split every row into chunks (three launches).  Measured:
  // 128 rows of 131072 entries 96.7 -> 45.4 us, 256 rows of 65792 56.4 ->
  // 46.2 us; 256 rows of 32768 were slower chunked (31.8 -> 36.2 us).
  const int64_t nchunks = T / kSoftmaxChunk;
  if (scores != p && nchunks >= 2 && (rows < 256 || nchunks >= 8) && rows < 1024) {
    const dim3 grid((unsigned)nchunks, (unsigned)rows);
    hipLaunchKernelGGL(k_softmax_chunk_stats, grid, dim3(256), 0, st, scores, p, T, ld, scale, (int)nchunks);
    hipLaunchKernelGGL(k_softmax_merge, dim3(rows), dim3(64), 0, st, p, ld, (int)nchunks);
    hipLaunchKernelGGL(k_softmax_chunk_norm, grid, dim3(256), 0, st, scores, p, T, ld, scale, (int)nchunks);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_softmax, dim3(rows), dim3(1024), 0, st, scores, p, T, ld, scale);
  return hipGetLastError();
}

}  // namespace packkv
