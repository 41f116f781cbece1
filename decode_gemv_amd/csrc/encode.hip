// PackKV encoder on the GPU: quantise -> reorder tokens -> bit-pack, one
// workgroup per block (Fig. 2 caption, steps (1) and (2); Fig. 5 caption for
// the two quantisation granularities; abstract for the growing cache).
//
// Bit-exact contract with the fp64 oracle:
//   * zero = group minimum (fp16, -0 stored as +0);
//   * scale = smallest positive fp16 h with h * L >= max - min (exact fp64
//     comparisons on fp16 values), 0 for a constant group;
//   * q = the level nearest to (x - min) / scale, ties to even (what rint of
//     the correctly rounded fp64 quotient gives), clamped to [0, L]; found
//     from a reciprocal and an exact residual (quant_level);
//   * permutation = greedy L1 grouping with key (distance, index), or (mode
//     2) the tokens sorted by (total of their K and V ints, index); identity
//     unless the payload shrinks strictly;
//   * run width = bit_length(max - min), u = q - min packed in the sliced
//     order of pack_run below.
// This file must be built without fast-math flags.
#include "kernels.hpp"

namespace packkv {

__device__ bool page_take(const PageAlloc& p, int s, int which, uint32_t need16, uint32_t& start16);

// Smallest positive fp16 pattern h with value(h) * L >= d, for d > 0.
__device__ uint32_t min_f16_step(double d, int L) {
  double y = d / (double)L;
  uint32_t h;
  if (y >= 65504.0) {
    h = 0x7BFFu;
  } else {
    int e;
    (void)frexp(y, &e);
    int E = e - 1;                                   // y in [2^E, 2^(E+1))
    if (E < -14) h = (uint32_t)floor(ldexp(y, 24));  // subnormal range
    else h = ((uint32_t)(E + 15) << 10) | ((uint32_t)floor(ldexp(y, 10 - E)) - 1024u);
  }
  if (h == 0) h = 1;
  while (h < 0x7BFFu && f16_bits_to_double(h) * L < d) ++h;
  while (h > 1u && f16_bits_to_double(h - 1) * L >= d) --h;
  return h;
}

// Order-preserving integer key of an fp16 value (not NaN): -0 and +0 share
// key 0, so comparing keys is comparing values.
__device__ __forceinline__ int f16_key(uint32_t h) {
  return (h & 0x8000u) ? -(int)(h & 0x7FFFu) : (int)(h & 0x7FFFu);
}
__device__ __forceinline__ uint32_t f16_of_key(int k) {
  return k < 0 ? (0x8000u | (uint32_t)(-k)) : (uint32_t)k;   // key 0 -> +0
}

// Step and zero of a group from its min and max keys (the oracle's rule).
struct QuantParams {
  double mn, h, inv, half;                           // inv = 1/h rounded once, half = h/2 exactly
  uint32_t hb, zero;
};
__device__ __forceinline__ QuantParams quant_params(int kmin, int kmax, int L) {
  QuantParams p;
  const uint32_t mnb = f16_of_key(kmin), mxb = f16_of_key(kmax);
  p.mn = f16_bits_to_double(mnb);
  const double d = f16_bits_to_double(mxb) - p.mn;
  p.hb = d > 0.0 ? min_f16_step(d, L) : 0u;
  p.h = f16_bits_to_double(p.hb);
  p.inv = p.hb ? 1.0 / p.h : 0.0;
  p.half = 0.5 * p.h;
  p.zero = mnb;                                      // +0 for a zero minimum
  return p;
}
// Level of one value: the level nearest to the exact quotient d / h
// (d = x - min, an exact fp64 subtraction), ties to even, clamped to [0, L],
// without a division per value.  d is a multiple of 2^-24 and h an fp16, so
// a quotient that is not a tie lies at least 2^-25 / h >= 2^-41 from every
// half-way point, while d * inv is within 2^-44 of it (the quotient is at
// most 255): rint(d * inv) is then the nearest level.  At a tie it may land
// on either neighbour; the residual e = t h - d is exact (t h has at most 20
// significant bits, both terms are multiples of 2^-24 below 2^17), equals
// +-h/2 exactly there, and then the even neighbour is taken.
__device__ __forceinline__ uint32_t quant_level(uint32_t x, const QuantParams& p, int L) {
  if (!p.hb) return 0u;
  const double d = f16_bits_to_double(x) - p.mn;
  const double t = rint(d * p.inv);
  const double e = fma(t, p.h, -d);
  int q = (int)t;
  if (fabs(e) == p.half && (q & 1)) q += e > 0.0 ? -1 : 1;
  return (uint32_t)min(max(q, 0), L);
}

// The ints of run r, channel c in slot order: v[i] = q[order[r*32 + i]][c]
// (0 past the n slots).  The run's 32 order bytes are read first as eight
// words, so the 32 value reads do not wait on one another.
template <int D>
__device__ __forceinline__ void run_values(const uint8_t* q, const uint8_t* order, int r, int c, int n,
                                           uint32_t v[kR]) {
  const int s0 = r * kR;
  const uint32_t* o4 = reinterpret_cast<const uint32_t*>(order + s0);
  uint32_t ow[kR / 4];
#pragma unroll
  for (int k = 0; k < kR / 4; ++k) ow[k] = o4[k];
#pragma unroll
  for (int i = 0; i < kR; ++i) {
    const uint32_t t = (ow[i >> 2] >> (8 * (i & 3))) & 0xFFu;
    v[i] = s0 + i < n ? (uint32_t)q[t * D + c] : 0u;
  }
}

// The W words of a run (out[0 .. W-1]; W = 1 .. CB) in the sliced order the
// decoders read: with CB-bit containers (4 for b <= 4, 8 for b = 5..8), the
// container word k holds slots k*(32/CB) + j in field j; if W divides CB,
// g = CB/W containers share word k/g, container k shifted left by
// W*(k % g); otherwise container k < W is word k's low W bits per field and
// bit p of container k >= W goes to bit k of every field of word p.  u[i]
// < 2^W for every slot.
template <int W, int CB>
__device__ __forceinline__ void pack_run(const uint32_t u[kR], uint32_t out[8]) {
  constexpr int PER = 32 / CB;                       // slots per container word
  constexpr uint32_t rep = CB == 4 ? 0x11111111u : 0x01010101u;
  uint32_t C[CB];
#pragma unroll
  for (int k = 0; k < CB; ++k) {
    uint32_t x = 0u;
#pragma unroll
    for (int j = 0; j < PER; ++j) x |= u[k * PER + j] << (CB * j);
    C[k] = x;
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) out[k] = 0u;
  if constexpr (CB % W == 0) {
    constexpr int g = CB / W;
#pragma unroll
    for (int k = 0; k < CB; ++k) out[k / g] |= C[k] << (W * (k % g));
  } else {
#pragma unroll
    for (int p = 0; p < W; ++p) out[p] = C[p];
#pragma unroll
    for (int k = W; k < CB; ++k)
#pragma unroll
      for (int p = 0; p < W; ++p) out[p] |= ((C[k] >> p) & rep) << k;
  }
}

// Min and width of run r, channel c of the slot-ordered ints q[order[slot]][c].
template <int D>
__device__ __forceinline__ void run_stats(const uint8_t* q, const uint8_t* order, int r, int c,
                                          int n, uint32_t& m, uint32_t& w) {
  uint32_t v[kR];
  run_values<D>(q, order, r, c, n, v);
  const int cnt = min(kR, n - r * kR);
  uint32_t lo = 255, hi = 0;
#pragma unroll
  for (int i = 0; i < kR; ++i) {
    if (i < cnt) {
      lo = min(lo, v[i]);
      hi = max(hi, v[i]);
    }
  }
  m = lo;
  w = 32u - __clz(hi - lo);
}

// Payload order 1 of a K record: a run row's entries go by decreasing width,
// equal widths by channel.  The channel-order word offset of entry (r, c)
// counts the words of the row's channels below c; the sorted one counts
// those of the wider channels and of the equally wide ones below c.
// Returns the difference, from the row's widths wrow[D].
template <int D>
__device__ int32_t width_sorted_shift(const uint8_t* wrow, int c, uint32_t w) {
  int32_t d = 0;
  for (int c2 = 0; c2 < D; ++c2) {
    const uint32_t w2 = wrow[c2];
    const int before_sorted = w2 > w || (w2 == w && c2 < c);
    const int before_channel = c2 < c;
    d += (before_sorted - before_channel) * (int32_t)w2;
  }
  return d;
}

// Block-wide (256 threads) exclusive scan of one value per thread.
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh /*[256]*/, uint32_t* total) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {
    uint32_t a = t >= o ? sh[t - o] : 0u;
    __syncthreads();
    sh[t] += a;
    __syncthreads();
  }
  uint32_t incl = sh[t];
  *total = sh[255];
  __syncthreads();
  return incl - v;
}

template <int B, int D>
__global__ __launch_bounds__(256) void k_encode(EncArgs a) {
  constexpr int NR = B / kR;
  constexpr int NT = 256;
  __shared__ __attribute__((aligned(16))) uint8_t qk[B * D];
  __shared__ __attribute__((aligned(16))) uint8_t qv[B * D];
  __shared__ __attribute__((aligned(16))) uint16_t rawk[B * D];
  __shared__ uint16_t ksc[D], kze[D], vsc[128], vze[128];
  __shared__ __attribute__((aligned(16))) uint8_t order[128];
  __shared__ __attribute__((aligned(16))) uint8_t ident[128];
  __shared__ uint8_t alive[128];
  __shared__ uint32_t key[128];
  __shared__ uint8_t wk[4 * D], mk[4 * D], wv[4 * D], mv[4 * D];
  __shared__ uint32_t scan_sh[NT];
  __shared__ uint32_t red[4];

  const int tid = threadIdx.x;
  const int L = (1 << a.bits) - 1;
  const int s = a.stream0 + (int)blockIdx.y;
  int j = a.mode == kTail ? a.block0 : (int)blockIdx.x;
  int64_t n_tok = a.n_tokens;
  int new_at = a.new_at;
  int32_t len0 = 0;
  if (a.paged) {
    len0 = a.lengths[s];
    if (a.mode == kTail) {
      // one token per stream, at the stream's own position
      j = len0 / B;
      new_at = len0 % B;
      n_tok = (int64_t)len0 + 1;
    } else if (a.mode == kPass2 && len0 != a.n_tokens) {
      return;                                        // its pages were not allocated
    }
  }
  const int64_t t0 = (int64_t)j * B;
  if (t0 >= n_tok) return;
  const int n = (int)imin64(B, n_tok - t0);
  const int nr = (n + kR - 1) / kR;
  // the source holds the launch's streams only
  const uint16_t* ks = a.k + (s - a.stream0) * a.src_stream + (a.mode == kTail ? 0 : j * a.src_block);
  const uint16_t* vs = a.v + (s - a.stream0) * a.src_stream + (a.mode == kTail ? 0 : j * a.src_block);

  // (1) quantise.  K per channel over the block's tokens: the block's raw K
  // is staged through LDS with 16-byte loads by every thread (one memory
  // latency), then thread c reads its channel from there.
  const bool fresh = a.mode == kTail && a.new_k != nullptr;
  {
    const uint4* src = reinterpret_cast<const uint4*>(ks);
    uint4* dst = reinterpret_cast<uint4*>(rawk);
    for (int i = tid; i < n * (D / 8); i += NT) {
      const int t = i / (D / 8);
      if (fresh && t >= new_at) {
        // an appended token: read it from the caller and keep it in the staging
        const uint4 u = reinterpret_cast<const uint4*>(a.new_k + s * a.new_stream + (int64_t)(t - new_at) * D)[i % (D / 8)];
        const_cast<uint4*>(src)[i] = u;
        dst[i] = u;
      } else {
        dst[i] = src[i];
      }
    }
  }
  __syncthreads();
  // an infinite or NaN input (exponent field all ones) is outside the
  // method: it latches EINVAL; the records stay well-formed
  bool nonfinite = false;
  if (tid < D) {
    int kmin = 0x7FFF, kmax = -0x7FFF;
    for (int t = 0; t < n; ++t) {
      const uint32_t x = rawk[t * D + tid];
      nonfinite |= (x & 0x7C00u) == 0x7C00u;
      const int k = f16_key(x);
      kmin = min(kmin, k);
      kmax = max(kmax, k);
    }
    const QuantParams qp = quant_params(kmin, kmax, L);
    ksc[tid] = (uint16_t)qp.hb;
    kze[tid] = (uint16_t)qp.zero;
    for (int t = 0; t < n; ++t) qk[t * D + tid] = (uint8_t)quant_level(rawk[t * D + tid], qp, L);
  }
  // V per token: the D channels of token t are split over TPT neighbouring
  // threads, each loading its CPT values with 16-byte loads; min and max are
  // combined across the TPT threads.
  {
    constexpr int TPT = NT / B;                      // 4 (B = 64) or 2 (B = 128)
    constexpr int CPT = D / TPT;                     // 16 .. 128 channels per thread
    const int t = tid / TPT, part = tid % TPT;
    const bool on = t < n;
    const bool appended = fresh && on && t >= new_at;
    uint32_t w[CPT / 2];                             // CPT fp16, two per word
    uint4* stage = reinterpret_cast<uint4*>(const_cast<uint16_t*>(vs) + (int64_t)(on ? t : 0) * D + part * CPT);
    const uint4* src = appended
        ? reinterpret_cast<const uint4*>(a.new_v + s * a.new_stream + (int64_t)(t - new_at) * D + part * CPT)
        : stage;
#pragma unroll
    for (int i = 0; i < CPT / 8; ++i) {
      {
        const uint4 u = src[i];
        if (appended) stage[i] = u;                  // keep it in the staging
        w[4 * i] = u.x; w[4 * i + 1] = u.y; w[4 * i + 2] = u.z; w[4 * i + 3] = u.w;
      }
    }
    int kmin = 0x7FFF, kmax = -0x7FFF;
#pragma unroll
    for (int i = 0; i < CPT / 2; ++i) {
      {
        nonfinite |= on && (((w[i] & 0x7C00u) == 0x7C00u) || ((w[i] & 0x7C000000u) == 0x7C000000u));
        const int a0 = f16_key(w[i] & 0xFFFFu), a1 = f16_key(w[i] >> 16);
        kmin = min(kmin, min(a0, a1));
        kmax = max(kmax, max(a0, a1));
      }
    }
    for (int o = 1; o < TPT; o <<= 1) {
      kmin = min(kmin, __shfl_xor(kmin, o, TPT));
      kmax = max(kmax, __shfl_xor(kmax, o, TPT));
    }
    if (on) {
      const QuantParams qp = quant_params(kmin, kmax, L);
      if (part == 0) {
        vsc[t] = (uint16_t)qp.hb;
        vze[t] = (uint16_t)qp.zero;
      }
      uint8_t* dst = qv + t * D + part * CPT;
#pragma unroll
      for (int i = 0; i < CPT / 2; ++i) {
        {
          dst[2 * i] = (uint8_t)quant_level(w[i] & 0xFFFFu, qp, L);
          dst[2 * i + 1] = (uint8_t)quant_level(w[i] >> 16, qp, L);
        }
      }
    }
  }
  if (__ballot(nonfinite) != 0 && (tid & 63) == 0) latch(a.status, PACKKV_EINVAL);
  if (tid < 128) ident[tid] = (uint8_t)tid;
  __syncthreads();

  // (2) token order inside the block.
  uint8_t* perm_g = a.perm + s * a.perm_stride + (int64_t)j * B;
  if (a.mode == kPass2) {
    if (tid < n) order[tid] = perm_g[tid];
    __syncthreads();
  } else {
    if (tid < 128) order[tid] = (uint8_t)tid;
    if (a.permute == 2 && n > 1) {
      // sort key: the total of the token's K and V ints (at most
      // 2 * 128 * 15 < 2^12), ties by index; the slot is the key's rank
      if (tid < n) {
        const uint32_t* rt = reinterpret_cast<const uint32_t*>(qk + tid * D);
        const uint32_t* vt = reinterpret_cast<const uint32_t*>(qv + tid * D);
        uint32_t total = 0;
        for (int i = 0; i < D / 4; ++i) {
          total = __builtin_amdgcn_sad_u8(rt[i], 0u, total);
          total = __builtin_amdgcn_sad_u8(vt[i], 0u, total);
        }
        key[tid] = (total << 8) | (uint32_t)tid;
      }
      __syncthreads();
      if (tid < n) {
        const uint32_t mine = key[tid];
        int rank = 0;
        for (int u = 0; u < n; ++u) rank += key[u] < mine;
        order[rank] = (uint8_t)tid;
      }
      __syncthreads();
    }
    if (a.permute == 1 && n > 1) {
      if (tid < 128) alive[tid] = tid < n;
      __syncthreads();
      for (int r = 0; r < nr; ++r) {
        const int base = r * kR;
        // seed = smallest remaining token index (one LDS atomic per wave)
        if (tid == 0) red[0] = 0xFFu;
        __syncthreads();
        {
          const uint64_t b = __ballot(tid < n && alive[tid]);
          if ((tid & 63) == 0 && b != 0) atomicMin(&red[0], (uint32_t)(tid + __builtin_ctzll(b)));
        }
        __syncthreads();
        const int sd = (int)red[0];
        if (tid < n) {
          uint32_t k0 = 0xFFFFFFFFu;
          if (alive[tid]) {
            const uint32_t* rt = reinterpret_cast<const uint32_t*>(qk + tid * D);
            const uint32_t* rs = reinterpret_cast<const uint32_t*>(qk + sd * D);
            const uint32_t* vt = reinterpret_cast<const uint32_t*>(qv + tid * D);
            const uint32_t* vd = reinterpret_cast<const uint32_t*>(qv + sd * D);
            uint32_t dist = 0;
            for (int i = 0; i < D / 4; ++i) {
              dist = __builtin_amdgcn_sad_u8(rt[i], rs[i], dist);
              dist = __builtin_amdgcn_sad_u8(vt[i], vd[i], dist);
            }
            k0 = (dist << 8) | (uint32_t)tid;
          }
          key[tid] = k0;
        }
        __syncthreads();
        if (tid < n && alive[tid]) {
          const uint32_t mine = key[tid];
          int rank = 0;
          for (int u = 0; u < n; ++u) rank += key[u] < mine;
          if (rank < kR) {
            order[base + rank] = (uint8_t)tid;
            alive[tid] = 0;
          }
        }
        __syncthreads();
      }
    }
    if (a.permute && n > 1) {
      // identity fallback: keep the new order only if the payload shrinks.
      if (tid < 2) red[tid] = 0;
      __syncthreads();
      // The statistics of both orders are kept in registers (at most 4
      // (run, channel) entries per thread), and those of the chosen order
      // become the record's widths and minima.
      constexpr int EPT = 2 * NR * D / NT;           // entries per thread: 1 .. 8
      uint32_t gm[EPT], gw[EPT], im[EPT], iw[EPT];
      uint32_t sum_g = 0, sum_i = 0;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int it = tid + e * NT;
        gm[e] = gw[e] = im[e] = iw[e] = 0u;
        if (it < 2 * nr * D) {
          const bool is_v = it >= nr * D;
          const int rc = is_v ? it - nr * D : it;
          const uint8_t* q = is_v ? qv : qk;
          run_stats<D>(q, order, rc / D, rc % D, n, gm[e], gw[e]);
          run_stats<D>(q, ident, rc / D, rc % D, n, im[e], iw[e]);
          sum_g += gw[e];
          sum_i += iw[e];
        }
      }
      // one LDS atomic per wave, not per thread (they serialise on one word)
      const uint32_t wave_g = (uint32_t)wave_sum_i((int)sum_g), wave_i = (uint32_t)wave_sum_i((int)sum_i);
      if ((tid & 63) == 0) {
        atomicAdd(&red[0], wave_g);
        atomicAdd(&red[1], wave_i);
      }
      __syncthreads();
      const bool keep = red[0] < red[1];
      __syncthreads();
      if (!keep && tid < 128) order[tid] = (uint8_t)tid;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int it = tid + e * NT;
        if (it < 2 * nr * D) {
          const bool is_v = it >= nr * D;
          const int rc = is_v ? it - nr * D : it;
          (is_v ? wv : wk)[rc] = (uint8_t)(keep ? gw[e] : iw[e]);
          (is_v ? mv : mk)[rc] = (uint8_t)(keep ? gm[e] : im[e]);
        }
      }
      __syncthreads();
    } else {
      // (3') identity order: per-run minima and widths
      for (int it = tid; it < 2 * nr * D; it += NT) {
        const bool is_v = it >= nr * D;
        const int rc = is_v ? it - nr * D : it;
        uint32_t m, w;
        run_stats<D>(is_v ? qv : qk, order, rc / D, rc % D, n, m, w);
        (is_v ? wv : wk)[rc] = (uint8_t)w;
        (is_v ? mv : mk)[rc] = (uint8_t)m;
      }
      __syncthreads();
    }
  }
  if (a.mode == kPass2) {
    // (3) per-run minima and widths in the stored order
    for (int it = tid; it < 2 * nr * D; it += NT) {
      const bool is_v = it >= nr * D;
      const int rc = is_v ? it - nr * D : it;
      uint32_t m, w;
      run_stats<D>(is_v ? qv : qk, order, rc / D, rc % D, n, m, w);
      (is_v ? wv : wk)[rc] = (uint8_t)w;
      (is_v ? mv : mk)[rc] = (uint8_t)m;
    }
    __syncthreads();
  }

  // payload word offsets of every (run, channel), run-major: up to NR * D
  // per tensor, PT consecutive entries per thread.
  constexpr int PT = (NR * D + NT - 1) / NT;         // 1 .. 4
  uint32_t totk, totv;
  const int nrc = nr * D;
  uint32_t k_in[PT], v_in[PT], k_sum = 0, v_sum = 0;  // exclusive sums inside the thread
#pragma unroll
  for (int e = 0; e < PT; ++e) {
    const int rc = PT * tid + e;
    k_in[e] = k_sum;
    v_in[e] = v_sum;
    k_sum += rc < nrc ? wk[rc] : 0u;
    v_sum += rc < nrc ? wv[rc] : 0u;
  }
  const uint32_t k_ex = block_excl_scan(k_sum, scan_sh, &totk);
  const uint32_t v_ex = block_excl_scan(v_sum, scan_sh, &totv);

  const int hb = hdr_entry_bytes(a.bits);
  const uint32_t k_pay = (uint32_t)payload_offset(false, B, nr, hb, D);
  const uint32_t v_pay = (uint32_t)payload_offset(true, B, nr, hb, D);
  const uint32_t k_size = k_pay + (uint32_t)pad16(4 * (int)totk);
  const uint32_t v_size = v_pay + (uint32_t)pad16(4 * (int)totv);
  uint32_t* koff = a.k_off + s * a.off_stride;
  uint32_t* voff = a.v_off + s * a.off_stride;
  uint2* ktab = a.k_tab + s * a.off_stride;
  uint2* vtab = a.v_tab + s * a.off_stride;

  if (a.mode == kPass1) {
    if (tid < B) perm_g[tid] = tid < n ? order[tid] : (uint8_t)0xFF;
    if (tid == 0) {
      if (a.paged) {
        ktab[j].y = k_size;       // sizes; the allocator then places the records
        vtab[j].y = v_size;
      } else {
        koff[j + 1] = k_size;     // sizes; a later scan turns them into offsets
        voff[j + 1] = v_size;
      }
    }
    return;
  }

  // (4) write the records.
  uint64_t kbase, vbase;
  uint8_t* krec;
  uint8_t* vrec;
  if (a.paged) {
    __shared__ uint32_t base_sh[2];
    if (a.mode == kTail) {
      // a block that this token fills moves to the stream's pages; an open
      // one stays in the stream's tail slots
      if (tid == 0) {
        uint32_t k16 = a.pages.tail16 + 2u * (uint32_t)s * a.pages.slot16, v16 = k16 + a.pages.slot16;
        if (n == B && !(page_take(a.pages, s, 0, k_size >> 4, k16) && page_take(a.pages, s, 1, v_size >> 4, v16)))
          k16 = kNoPage;
        base_sh[0] = k16;
        base_sh[1] = v16;
      }
      __syncthreads();
      if (base_sh[0] == kNoPage) {
        if (tid == 0) latch(a.status, PACKKV_ECAPACITY);
        return;
      }
      kbase = (uint64_t)base_sh[0] << 4;
      vbase = (uint64_t)base_sh[1] << 4;
    } else {
      kbase = (uint64_t)ktab[j].x << 4;
      vbase = (uint64_t)vtab[j].x << 4;
    }
    if (kbase + k_size > a.arena_limit || vbase + v_size > a.arena_limit) {
      if (tid == 0) latch(a.status, PACKKV_ECORRUPT);
      return;
    }
    krec = a.k_arena + kbase;
    vrec = a.v_arena + vbase;
  } else {
    if (a.mode == kTail) {
      if (j == 0) {
        kbase = 0u;
        vbase = 0u;
      } else {
        kbase = koff[j];
        vbase = voff[j];
      }
    } else {
      kbase = koff[j];
      vbase = voff[j];
    }
    if (kbase + k_size > a.arena_limit || vbase + v_size > a.arena_limit) {
      if (tid == 0) latch(a.status, PACKKV_ECAPACITY);
      return;
    }
    krec = a.k_arena + s * a.arena_stride + kbase;
    vrec = a.v_arena + s * a.arena_stride + vbase;
  }

  // params
  if (tid < D) {
    reinterpret_cast<uint16_t*>(krec)[tid] = ksc[tid];
    reinterpret_cast<uint16_t*>(krec)[D + tid] = kze[tid];
  }
  if (tid < B) {
    const bool ok = tid < n;
    reinterpret_cast<uint16_t*>(vrec)[tid] = ok ? vsc[order[tid]] : (uint16_t)0;
    reinterpret_cast<uint16_t*>(vrec)[B + tid] = ok ? vze[order[tid]] : (uint16_t)0;
  }
  // headers and the zero padding up to the payload
  {
    const uint32_t kh = (uint32_t)hdr_offset(false, B, D), vh = (uint32_t)hdr_offset(true, B, D);
    // byte i of the header area: entry i / hb, byte i % hb of it
    for (uint32_t i = tid; i < k_pay - kh; i += NT) {
      const uint32_t e = hb == 2 ? i >> 1 : i;
      const uint32_t h = e < (uint32_t)nrc ? (hb == 2 ? ((uint32_t)wk[e] << 8) | mk[e] : ((uint32_t)wk[e] << 4) | mk[e]) : 0u;
      krec[kh + i] = (uint8_t)(hb == 2 && (i & 1u) ? h >> 8 : h);
    }
    for (uint32_t i = tid; i < v_pay - vh; i += NT) {
      const uint32_t e = hb == 2 ? i >> 1 : i;
      const uint32_t h = e < (uint32_t)nrc ? (hb == 2 ? ((uint32_t)wv[e] << 8) | mv[e] : ((uint32_t)wv[e] << 4) | mv[e]) : 0u;
      vrec[vh + i] = (uint8_t)(hb == 2 && (i & 1u) ? h >> 8 : h);
    }
  }
  // payload: each thread packs its PT (run, channel) entries of K and of V
  for (int e = 0; e < 2 * PT; ++e) {
    const bool is_v = e >= PT;
    const int ei = is_v ? e - PT : e;
    const int rc = PT * tid + ei;
    if (rc >= nrc) continue;
    const uint8_t* q = is_v ? qv : qk;
    const uint32_t w = (is_v ? wv : wk)[rc];
    const uint32_t m = (is_v ? mv : mk)[rc];
    if (w == 0) continue;
    const int r = rc / D, c = rc % D;
    uint32_t woff = is_v ? v_ex + v_in[ei] : k_ex + k_in[ei];
    if (!is_v && a.korder == 1) woff += (uint32_t)width_sorted_shift<D>(wk + r * D, c, w);
    uint32_t v[kR];
    run_values<D>(q, order, r, c, n, v);
#pragma unroll
    for (int i = 0; i < kR; ++i) v[i] = r * kR + i < n ? v[i] - m : 0u;
    uint32_t words[8];
    if (hb == 1) {                                   // nibble containers (b <= 4)
      switch (w) {
        case 1: pack_run<1, 4>(v, words); break;
        case 2: pack_run<2, 4>(v, words); break;
        case 3: pack_run<3, 4>(v, words); break;
        default: pack_run<4, 4>(v, words); break;
      }
    } else {                                         // byte containers (b = 5..8)
      switch (w) {
        case 1: pack_run<1, 8>(v, words); break;
        case 2: pack_run<2, 8>(v, words); break;
        case 3: pack_run<3, 8>(v, words); break;
        case 4: pack_run<4, 8>(v, words); break;
        case 5: pack_run<5, 8>(v, words); break;
        case 6: pack_run<6, 8>(v, words); break;
        case 7: pack_run<7, 8>(v, words); break;
        default: pack_run<8, 8>(v, words); break;
      }
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>((is_v ? vrec + v_pay : krec + k_pay)) + woff;
    for (uint32_t i = 0; i < w; ++i) dst[i] = words[i];
  }
  // zero padding after the payload
  if (tid < 4) {
    uint32_t* kt = reinterpret_cast<uint32_t*>(krec + k_pay) + totk;
    uint32_t* vt = reinterpret_cast<uint32_t*>(vrec + v_pay) + totv;
    if (totk + tid < (k_size - k_pay) / 4) kt[tid] = 0u;
    if (totv + tid < (v_size - v_pay) / 4) vt[tid] = 0u;
  }
  if (a.mode == kTail) {
    if (tid < B) perm_g[tid] = tid < n ? order[tid] : (uint8_t)0xFF;
    if (tid == 0) {
      if (a.paged) {
        ktab[j] = make_uint2((uint32_t)(kbase >> 4), k_size);
        vtab[j] = make_uint2((uint32_t)(vbase >> 4), v_size);
        a.lengths[s] = len0 + 1;
      } else {
        if (j == 0) {
          koff[0] = 0u;
          voff[0] = 0u;
        }
        koff[j + 1] = (uint32_t)kbase + k_size;
        voff[j + 1] = (uint32_t)vbase + v_size;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Paged cache: page allocation, set-up and release.

// Place a K (which = 0) or V (1) record of need16 16-byte units in stream
// s's current page of that kind, or at the start of a page taken from the
// free stack; false if none is left.  Called by one thread per stream at a
// time.
__device__ bool page_take(const PageAlloc& p, int s, int which, uint32_t need16, uint32_t& start16) {
  uint32_t* st = p.state + 2 + 4 * s + 2 * which;
  uint32_t page = st[0], fill = st[1];
  if (page == kNoPage || fill + need16 > p.page16) {
    const int old = atomicSub(reinterpret_cast<int*>(p.state), 1);
    if (old <= 0) {
      atomicAdd(reinterpret_cast<int*>(p.state), 1);
      return false;
    }
    page = p.state[2 + 4 * p.n_streams + old - 1];
    fill = 0;
  }
  start16 = page * p.page16 + fill;
  st[0] = page;
  st[1] = fill + need16;
  return true;
}

// Prefill of n_streams streams from stream0 on, after pass 1 wrote the
// sizes: one thread per stream places the closed blocks' records (block
// order, K and V in pages of their own), points the open block at the tail
// slots and sets the length.
__global__ __launch_bounds__(64) void k_paged_alloc(EncArgs a, int n_streams, int64_t n_tokens) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i >= n_streams) return;
  const int s = a.stream0 + i;
  const int nfull = (int)(n_tokens / a.B), nb = (int)((n_tokens + a.B - 1) / a.B);
  uint2* kt = a.k_tab + s * a.off_stride;
  uint2* vt = a.v_tab + s * a.off_stride;
  for (int j = 0; j < nfull; ++j) {
    uint32_t k16, v16;
    if (!page_take(a.pages, s, 0, kt[j].y >> 4, k16) || !page_take(a.pages, s, 1, vt[j].y >> 4, v16)) {
      latch(a.status, PACKKV_ECAPACITY);
      return;                                        // length stays 0: pass 2 writes nothing
    }
    kt[j].x = k16;
    vt[j].x = v16;
  }
  if (nb > nfull) {
    kt[nfull].x = a.pages.tail16 + 2u * (uint32_t)s * a.pages.slot16;
    vt[nfull].x = kt[nfull].x + a.pages.slot16;
  }
  a.lengths[s] = (int32_t)n_tokens;
}

// Every page free, every stream empty, the status clear.
__global__ __launch_bounds__(256) void k_paged_init(PageAlloc p, int32_t* lengths, int32_t* status) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i == 0) {
    p.state[0] = p.n_pages;
    p.state[1] = 0u;
    *status = 0;
  }
  if (i < p.n_streams) {
    for (int k = 0; k < 4; k += 2) {
      p.state[2 + 4 * i + k] = kNoPage;
      p.state[3 + 4 * i + k] = 0u;
    }
    lengths[i] = 0;
  }
  if (i < (int64_t)p.n_pages) p.state[2 + 4 * p.n_streams + i] = p.n_pages - 1u - (uint32_t)i;
}

// Stream s back to empty: its pages go back on the stack.  Its K records
// fill its K pages in block order (and likewise V), so each page shows up
// in one run of consecutive records of its kind.
__global__ __launch_bounds__(64) void k_paged_release(PageAlloc p, const uint2* k_tab, const uint2* v_tab,
                                                      int64_t tab_stride, int32_t* lengths, int B, int s) {
  if (threadIdx.x != 0) return;
  const int nfull = lengths[s] / B;
  for (int which = 0; which < 2; ++which) {
    const uint2* t = (which ? v_tab : k_tab) + s * tab_stride;
    uint32_t last = kNoPage;
    for (int j = 0; j < nfull; ++j) {
      const uint32_t pg = t[j].x / p.page16;
      if (pg != last) {
        p.state[2 + 4 * p.n_streams + atomicAdd(reinterpret_cast<int*>(p.state), 1)] = pg;
        last = pg;
      }
    }
    p.state[2 + 4 * s + 2 * which] = kNoPage;
    p.state[3 + 4 * s + 2 * which] = 0u;
  }
  lengths[s] = 0;
}

// Per stream: sizes in off[1..nb] -> byte offsets (off[0] = 0).
__global__ __launch_bounds__(256) void k_scan_offsets(uint32_t* k_off, uint32_t* v_off,
                                                      int64_t off_stride, int nb) {
  __shared__ uint32_t sh[256];
  uint32_t* off = (blockIdx.y == 0 ? k_off : v_off) + blockIdx.x * off_stride;
  uint32_t carry = 0;
  for (int base = 0; base < nb; base += 256) {
    const int i = base + threadIdx.x;
    const uint32_t v = i < nb ? off[i + 1] : 0u;
    uint32_t tot;
    const uint32_t ex = block_excl_scan(v, sh, &tot);
    if (i < nb) off[i + 1] = carry + ex + v;
    carry += tot;
  }
  if (threadIdx.x == 0) off[0] = 0u;
}

// Copy `cnt` tokens [S][cnt][D] fp16 into the tail staging at token `at`.
__global__ void k_stage_tail(const uint16_t* k, const uint16_t* v, int64_t src_stream,
                             uint16_t* tk, uint16_t* tv, int B, int D, int at, int cnt) {
  const int s = blockIdx.x;
  for (int i = threadIdx.x; i < cnt * D; i += blockDim.x) {
    tk[(int64_t)s * B * D + (int64_t)at * D + i] = k[s * src_stream + i];
    tv[(int64_t)s * B * D + (int64_t)at * D + i] = v[s * src_stream + i];
  }
}

}  // namespace packkv

// ---------------------------------------------------------------------------
// Launch helpers used by the C ABI layer.
namespace packkv {

hipError_t launch_encode(const EncArgs& a, int n_streams, int n_blocks, hipStream_t st) {
  dim3 grid(a.mode == kTail ? 1 : n_blocks, n_streams);
  switch ((a.B == 64 ? 0 : 3) + (a.D == 64 ? 0 : a.D == 128 ? 1 : 2)) {
    case 0: hipLaunchKernelGGL((k_encode<64, 64>), grid, dim3(256), 0, st, a); break;
    case 1: hipLaunchKernelGGL((k_encode<64, 128>), grid, dim3(256), 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_encode<64, 256>), grid, dim3(256), 0, st, a); break;
    case 3: hipLaunchKernelGGL((k_encode<128, 64>), grid, dim3(256), 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_encode<128, 128>), grid, dim3(256), 0, st, a); break;
    default: hipLaunchKernelGGL((k_encode<128, 256>), grid, dim3(256), 0, st, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_paged_alloc(const EncArgs& a, int n_streams, int64_t n_tokens, hipStream_t st) {
  hipLaunchKernelGGL(k_paged_alloc, dim3((n_streams + 63) / 64), dim3(64), 0, st, a, n_streams, n_tokens);
  return hipGetLastError();
}

hipError_t launch_paged_init(const PageAlloc& p, int32_t* lengths, int32_t* status, hipStream_t st) {
  const int64_t n = p.n_pages > (uint32_t)p.n_streams ? (int64_t)p.n_pages : (int64_t)p.n_streams;
  hipLaunchKernelGGL(k_paged_init, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, lengths, status);
  return hipGetLastError();
}

hipError_t launch_paged_release(const PageAlloc& p, const uint2* k_tab, const uint2* v_tab,
                                int64_t tab_stride, int32_t* lengths, int B, int stream, hipStream_t st) {
  hipLaunchKernelGGL(k_paged_release, dim3(1), dim3(64), 0, st, p, k_tab, v_tab, tab_stride, lengths, B,
                     stream);
  return hipGetLastError();
}

hipError_t launch_scan_offsets(uint32_t* k_off, uint32_t* v_off, int64_t off_stride,
                               int n_streams, int nb, hipStream_t st) {
  hipLaunchKernelGGL(k_scan_offsets, dim3(n_streams, 2), dim3(256), 0, st, k_off, v_off,
                     off_stride, nb);
  return hipGetLastError();
}

hipError_t launch_stage_tail(const uint16_t* k, const uint16_t* v, int64_t src_stream,
                             uint16_t* tk, uint16_t* tv, int B, int D, int at, int cnt,
                             int n_streams, hipStream_t st) {
  hipLaunchKernelGGL(k_stage_tail, dim3(n_streams), dim3(256), 0, st, k, v, src_stream, tk, tv,
                     B, D, at, cnt);
  return hipGetLastError();
}

}  // namespace packkv
