// ddtree_topk: fused log-softmax + top-K over the drafter's per-position
// logits ("DDTree Deep Dive", section 1 and section 2 Lemma 1).
//
// Two launches on one stream:
//   chunk kernel  grid (C chunks, L rows), 256 threads, 4096 logits per
//                 workgroup held in registers (16 per thread, coalesced
//                 dword loads: one HBM pass). Emits the chunk's (max,
//                 sum-exp) pair, a candidate superset of the chunk's top-K
//                 and a lower bound t_c of the chunk's K-th largest logit
//                 (the smallest candidate; -inf for chunks shorter than K).
//   merge kernel  grid L, 1024 threads. Combines the (max, sum) pairs into
//                 lse, keeps the candidates >= tau = max_c t_c (a valid
//                 lower bound of the row's K-th largest, so every top-K
//                 element survives), narrows them to the first-digit bucket
//                 of the K-th largest and above, ranks those exactly in LDS
//                 and writes logp = x - lse and the token ids in rank order.
//
// Selection is a radix select. Its first digit is relative to the reference
// maximum m: digit = bits(fl(m - x) + 1) >> 19, clamped (16 bins per octave
// of the distance below the max), which spreads the few values near the top
// over many bins and keeps LDS atomic contention low; it is monotone in x.
// The boundary bin is refined on the exact fp32 order key (4 x 8 bits) and,
// for exact ties, on the index (smaller id first). The chunk kernel stops
// after the first digit when the candidate set fits its slots ("loose").
// Ranking is by (logit descending, token id ascending) throughout.
#include <type_traits>

#include "common.hpp"

namespace {

constexpr int kChunkThreads = 256;
constexpr int kPerThread = 16;
constexpr int kChunk = kChunkThreads * kPerThread;  // 4096
constexpr int kLooseExtra = 256;                     // slots beyond K per chunk
constexpr int kMergeThreads = 1024;
constexpr int kSurvCap = 16384;                      // survivors selected in LDS (128 KB)
constexpr int kLoadBatchSmall = 8;                   // candidates loaded per thread at once:
constexpr int kLoadBatchLarge = 16;                  // the small batch when it holds all
constexpr int kRankAllMax = 256;                     // survivors ranked all against all
constexpr int kFusedHistK = 64;                      // larger K count digits while gathering
constexpr int kBounds = 7;                           // per-chunk bounds: r = 1, 2, 4, ..., 64

// A workgroup barrier for data exchanged through LDS only: waits for this
// wave's LDS operations, not for its global loads and stores (which
// __syncthreads would wait for as well). Every barrier in these kernels
// exchanges LDS data only.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unchanged
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The 32-bit value of lane (lane ^ J), J a power of two below 64: DPP within
// rows of 16 lanes (every lane written, bound_ctrl), the permlane swaps
// across them (no LDS round trip).
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  const int iv = (int)v;
  const int lane = (int)__lane_id();
  if constexpr (J == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, true);  // quad [1,0,3,2]
  } else if constexpr (J == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, true);  // quad [2,3,0,1]
  } else if constexpr (J == 4) {
    const int up = __builtin_amdgcn_mov_dpp(iv, 0x104, 0xF, 0xF, true);  // lane + 4
    const int dn = __builtin_amdgcn_mov_dpp(iv, 0x114, 0xF, 0xF, true);  // lane - 4
    return (uint32_t)((lane & 4) ? dn : up);
  } else if constexpr (J == 8) {
    return (uint32_t)__builtin_amdgcn_mov_dpp(iv, 0x128, 0xF, 0xF, true);  // row rotate 8
  } else if constexpr (J == 16) {
    // Swapping with itself leaves rows (0, 0, 2, 2) in the first result
    // and rows (1, 1, 3, 3) in the second.
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? r[0] : r[1];
  } else {
    static_assert(J == 32, "lane distance");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32) ? r[0] : r[1];
  }
}

// One compare-exchange stage of a bitonic sort over the wave (largest
// first): blocks of K lanes, partners J apart.
template <int K, int J>
__device__ __forceinline__ uint32_t bitonic_stage(uint32_t v) {
  const int lane = (int)__lane_id();
  const uint32_t p = xor_lane<J>(v);
  const bool keep_max = ((lane & J) == 0) == ((lane & K) == 0);
  return keep_max ? max(v, p) : min(v, p);
}

// The wave's 64 values sorted, largest on lane 0. Sorted as order keys
// (ddt::f32_key): unsigned max and min take the lane move as a DPP operand
// and need no float canonicalisation, three vector instructions a stage
// (0.49 us a sort against 0.76 on floats, at the chunk kernel's occupancy).
// -0 comes back as +0, which compares equal to it.
__device__ __forceinline__ float wave_sort_desc(float x) {
  uint32_t v = ddt::f32_key(x);
  v = bitonic_stage<2, 1>(v);
  v = bitonic_stage<4, 2>(v);
  v = bitonic_stage<4, 1>(v);
  v = bitonic_stage<8, 4>(v);
  v = bitonic_stage<8, 2>(v);
  v = bitonic_stage<8, 1>(v);
  v = bitonic_stage<16, 8>(v);
  v = bitonic_stage<16, 4>(v);
  v = bitonic_stage<16, 2>(v);
  v = bitonic_stage<16, 1>(v);
  v = bitonic_stage<32, 16>(v);
  v = bitonic_stage<32, 8>(v);
  v = bitonic_stage<32, 4>(v);
  v = bitonic_stage<32, 2>(v);
  v = bitonic_stage<32, 1>(v);
  v = bitonic_stage<64, 32>(v);
  v = bitonic_stage<64, 16>(v);
  v = bitonic_stage<64, 8>(v);
  v = bitonic_stage<64, 4>(v);
  v = bitonic_stage<64, 2>(v);
  v = bitonic_stage<64, 1>(v);
  return ddt::key_f32(v);
}

// The q-th largest (q = 1, 2, 4, 8 or 16) of a thread's 16 values, whose
// largest is xmax.
__device__ __forceinline__ float qth_largest(const float (&x)[16], int q, float xmax) {
  if (q == 1) return xmax;
  if (q == 16) {
    float m = x[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) m = fminf(m, x[j]);
    return m;
  }
  // Bitonic sort of the 16 values (largest first), then pick.
  float y[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) y[j] = x[j];
#pragma unroll
  for (int k = 2; k <= 16; k <<= 1)
#pragma unroll
    for (int jj = k >> 1; jj > 0; jj >>= 1)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int l = i ^ jj;
        if (l > i) {
          const float a = y[i], b = y[l];
          const bool desc = (i & k) == 0;
          y[i] = desc ? fmaxf(a, b) : fminf(a, b);
          y[l] = desc ? fminf(a, b) : fmaxf(a, b);
        }
      }
  return q == 2 ? y[1] : q == 4 ? y[3] : y[7];
}

// Larger digit = closer to the reference maximum (monotone in x).
__device__ __forceinline__ uint32_t rel_digit(float ref_max, float x) {
  const float y = (ref_max - x) + 1.0f;
  uint32_t b = (__float_as_uint(y) - 0x3F800000u) >> 19;
  b = b > 255u ? 255u : b;
  return 255u - b;
}

// Radix-select histograms, three of them in rotation: pass p counts into
// hist[p % 3] and clears hist[(p + 1) % 3] for the next pass. The bins are
// then read by every wave (each finds the boundary digit itself), so a pass
// needs one barrier: hist[(p + 1) % 3] was last read in pass p - 2, and
// every wave has passed the barrier of pass p - 1, which follows that read.
struct SelShared {
  uint32_t hist[3][256];
  uint32_t kmax[16], kmin[16];  // per-wave key range of a bucket
  uint32_t out_count;
};

// Zero the first two histograms (before pass 0; a barrier must follow).
__device__ __forceinline__ void init_hists(SelShared& s) {
  for (int i = threadIdx.x; i < 512; i += blockDim.x) (&s.hist[0][0])[i] = 0u;
}
__device__ __forceinline__ void clear_next(SelShared& s, int pass) {
  uint32_t* h = s.hist[(pass + 1) % 3];
  for (int i = threadIdx.x; i < 256; i += blockDim.x) h[i] = 0u;
}

struct DigitSel {
  uint32_t digit;   // digit of the boundary bucket
  uint32_t need;    // how many to take from that bucket
  uint32_t above;   // active elements in buckets above it
  uint32_t in_bin;  // active elements in that bucket
};

// With hist filled (and a barrier passed), the bucket holding the need-th
// largest counted element (need <= the total count). Computed by every wave
// on its own; the result is wave-uniform.
__device__ __forceinline__ DigitSel find_digit(const uint32_t* hist, uint32_t need) {
  const int l = threadIdx.x & 63;
  const uint32_t h0 = hist[4 * l], h1 = hist[4 * l + 1];
  const uint32_t h2 = hist[4 * l + 2], h3 = hist[4 * l + 3];
  const uint32_t lsum = h0 + h1 + h2 + h3;
  uint32_t suf = lsum;  // inclusive suffix sum over lanes (high digits last)
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_down(suf, off, 64);
    if (l + off < 64) suf += o;
  }
  const uint32_t above = suf - lsum;
  const bool here = above < need && need <= suf;
  uint32_t a = above, d, hh;
  if (a + h3 >= need) {
    d = 4 * l + 3; hh = h3;
  } else if (a + h3 + h2 >= need) {
    a += h3; d = 4 * l + 2; hh = h2;
  } else if (a + h3 + h2 + h1 >= need) {
    a += h3 + h2; d = 4 * l + 1; hh = h1;
  } else {
    a += h3 + h2 + h1; d = 4 * l; hh = h0;
  }
  const int src = __ffsll((unsigned long long)ddt::ballot(here)) - 1;
  DigitSel r;
  r.digit = (uint32_t)__shfl((int)d, src, 64);
  r.above = (uint32_t)__shfl((int)a, src, 64);
  r.in_bin = (uint32_t)__shfl((int)hh, src, 64);
  r.need = need - r.above;
  return r;
}

// Exact threshold inside the boundary bucket d0 of the relative digit:
// elements of that bucket are taken iff (key > tkey) or (key == tkey and
// ikey(index) >= tik), where ikey is larger for smaller indices. ACTIVE(i)
// says whether element i is in the bucket; KEY(i), IKEY(i) give its keys.
// Passes continue the rotation from pass number `pass` (whose histogram
// is clear). All threads call this; every thread ends with the result.
template <class Active, class Key, class IKey>
__device__ __forceinline__ void refine_bucket(SelShared& sh, uint32_t need, int n_elems,
                                              int idx_passes, int pass, Active active, Key keyf,
                                              IKey ikeyf, uint32_t& tkey, uint32_t& tik) {
  // The bucket's keys share their high bits: find the highest bit where
  // its largest and smallest keys differ and select digit by digit from
  // there down (the shared bits would otherwise cost whole passes in which
  // every element hits the same histogram bin).
  uint32_t kx = 0u, kn = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 0; i < n_elems; ++i) {
    if (active(i)) {
      const uint32_t k = keyf(i);
      kx = k > kx ? k : kx;
      kn = k < kn ? k : kn;
    }
  }
  kx = ddt::wave_max_u32(kx);
  kn = ~ddt::wave_max_u32(~kn);
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sh.kmax[wave] = kx;
    sh.kmin[wave] = kn;
  }
  lds_barrier();
  kx = 0u;
  kn = 0xFFFFFFFFu;
  for (int w = 0; w < nw; ++w) {
    kx = sh.kmax[w] > kx ? sh.kmax[w] : kx;
    kn = sh.kmin[w] < kn ? sh.kmin[w] : kn;
  }
  const uint32_t diff = kx ^ kn;
  const int hb = diff ? 31 - __builtin_clz(diff) : -1;  // highest differing bit
  const uint32_t low = hb >= 0 ? (uint32_t)((2ull << hb) - 1ull) : 0u;
  uint32_t mask = ~low, prefix = kx & mask, inb = 0u;
  bool counted = false;  // inb holds the bucket's count of keys == prefix
  for (int top = hb; top >= 0; top -= 8, ++pass) {
    const int shift = top >= 7 ? top - 7 : 0;
    const uint32_t dmask = (uint32_t)((2ull << (top - shift)) - 1ull);
    clear_next(sh, pass);
    uint32_t* h = sh.hist[pass % 3];
#pragma unroll
    for (int i = 0; i < n_elems; ++i) {
      if (active(i)) {
        const uint32_t k = keyf(i);
        if ((k & mask) == prefix) atomicAdd(&h[(k >> shift) & dmask], 1u);
      }
    }
    lds_barrier();
    const DigitSel ds = find_digit(h, need);
    prefix |= ds.digit << shift;
    mask |= dmask << shift;
    need = ds.need;
    inb = ds.in_bin;
    counted = true;
  }
  tkey = prefix;
  tik = 0u;
  if (!counted) inb = need + 1u;  // all keys equal: let the index decide
  if (need < inb) {
    uint32_t ip = 0u, im = 0u;
    for (int shift = 8 * (idx_passes - 1); shift >= 0; shift -= 8, ++pass) {
      clear_next(sh, pass);
      uint32_t* h = sh.hist[pass % 3];
#pragma unroll
      for (int i = 0; i < n_elems; ++i) {
        if (active(i) && keyf(i) == tkey) {
          const uint32_t ik = ikeyf(i);
          if ((ik & im) == ip) atomicAdd(&h[(ik >> shift) & 255u], 1u);
        }
      }
      lds_barrier();
      const DigitSel ds = find_digit(h, need);
      ip |= ds.digit << shift;
      im |= 255u << shift;
      need = ds.need;
    }
    tik = ip;
  }
}

__global__ __launch_bounds__(kChunkThreads) void topk_chunk_kernel(
    const float* __restrict__ logits, int64_t stride, int V, int K, int cap, int q,
    float4* __restrict__ stats, float* __restrict__ bounds, int* __restrict__ counts,
    float* __restrict__ cand_x, int* __restrict__ cand_i) {
  __shared__ SelShared sh;
  __shared__ float red[3][4];
  __shared__ float wbound[4][1 + kBounds];  // per wave: the chunk bound's and the r-bounds' parts
  __shared__ float wmin[4][1];              // per wave: the quarter-form part of the chunk bound
  const int chunk = blockIdx.x, row = blockIdx.y, C = gridDim.x;
  const int base = chunk * kChunk;
  const int n = min(kChunk, V - base);
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
  const float* src = logits + (int64_t)row * stride + base;

  float x[kPerThread];
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int e = t + kChunkThreads * j;
    x[j] = e < n ? src[e] : -INFINITY;
  }
  init_hists(sh);
  if (t == 0) sh.out_count = 0u;

  float xmax = -INFINITY;  // the thread's largest value
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) xmax = fmaxf(xmax, x[j]);
  const float mx = ddt::wave_reduce_uniform(xmax, ddt::OpMax());
  if (lane == 0) red[0][wave] = mx;
  lds_barrier();
  const float m = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));

  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (t + kChunkThreads * j < n) s += __expf(x[j] - m);
  s = ddt::wave_reduce_uniform(s, ddt::OpSum());

  // Lower bounds without a histogram. Each thread takes the q-th largest of
  // its 16 values (padding is -inf); sorted over the wave, the r-th largest
  // of those, v_r, has r threads each holding q values >= v_r, so at least
  // q r of the wave's (and the chunk's) values are >= v_r: v_r bounds the
  // chunk's (q r)-th largest from below, and so does the maximum of the
  // four waves' v_r. With q r >= Kc (r = ceil(Kc / q) <= 64) that bound T
  // keeps every element of the chunk's top Kc in {x >= T}, usually not
  // many more. The bounds for r = 1, 2, 4, ..., 64 go to the merge.
  const uint32_t Kc = (uint32_t)min(K, n);
  // Two forms of the bound for q r values: the maximum over the waves of
  // their v_r (one wave holds them all), and the minimum over the waves of
  // their v_(r/4) (each of the four waves holds a quarter), which is the
  // tighter one whenever r >= 4.
  {
    const float sv = wave_sort_desc(qth_largest(x, q, xmax));
    const int r_own = ((int)Kc + q - 1) / q;
    const int r_quarter = (r_own + 3) / 4;
    if (lane == 0) red[1][wave] = s;
    const float own_max = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv), r_own - 1));
    const float own_min = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv), r_quarter - 1));
    if (lane == 0) {
      wbound[wave][0] = own_max;
      wmin[wave][0] = own_min;
    }
#pragma unroll
    for (int b = 0; b < kBounds; ++b) {
      const float vb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv), (1 << b) - 1));
      if (lane == 0) wbound[wave][1 + b] = vb;
    }
  }
  lds_barrier();
  const float T = fmaxf(fmaxf(fmaxf(wbound[0][0], wbound[1][0]), fmaxf(wbound[2][0], wbound[3][0])),
                        fminf(fminf(wmin[0][0], wmin[1][0]), fminf(wmin[2][0], wmin[3][0])));
  if (t < kBounds) {
    // Bound b covers the chunk's (q 2^b)-th largest: one wave's v_(2^b), or
    // for b >= 2 the four waves' v_(2^(b-2)).
    float bb = fmaxf(fmaxf(wbound[0][1 + t], wbound[1][1 + t]), fmaxf(wbound[2][1 + t], wbound[3][1 + t]));
    if (t >= 2)
      bb = fmaxf(bb, fminf(fminf(wbound[0][t - 1], wbound[1][t - 1]),
                           fminf(wbound[2][t - 1], wbound[3][t - 1])));
    bounds[(int64_t)(row * C + chunk) * kBounds + t] = bb;
  }
  const int64_t slot0 = ((int64_t)row * C + chunk) * cap;
  const float ssum = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  {
    // Write {x >= T} straight from registers, each thread's values as one
    // run: an exclusive prefix of the per-thread counts over the wave (five
    // ballots of their bits) and one LDS atomic per wave place the runs.
    // (Staging through LDS for coalesced stores, with positions from one
    // ballot per value, took 0.35 us longer per launch.) The list's order
    // is immaterial: the merge ranks by value and id.
    uint32_t selmask = 0u;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j)
      selmask |= (uint32_t)(t + kChunkThreads * j < n && x[j] >= T) << j;
    const uint32_t nsel = (uint32_t)__popc(selmask);
    uint32_t excl = 0u, tot = 0u;
#pragma unroll
    for (int b = 0; b < 5; ++b) {  // nsel <= 16 fits five bits
      const uint64_t bm = ddt::ballot((nsel >> b) & 1u);
      excl += ddt::lanes_below(bm) << b;
      tot += (uint32_t)__popcll(bm) << b;
    }
    uint32_t wb = 0u;
    if (lane == 0 && tot) wb = atomicAdd(&sh.out_count, tot);
    uint32_t pos = (uint32_t)__builtin_amdgcn_readfirstlane((int)wb) + excl;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      if ((selmask >> j) & 1u) {
        if (pos < (uint32_t)cap) {
          cand_x[slot0 + pos] = x[j];
          cand_i[slot0 + pos] = base + t + kChunkThreads * j;
        }
        ++pos;
      }
    }
  }
  lds_barrier();
  const uint32_t n_fast = sh.out_count;
  if (n_fast <= (uint32_t)cap) {
    // The common case: the list is complete.
    if (t == 0) {
      counts[row * C + chunk] = (int)n_fast;
      stats[row * C + chunk] = make_float4(m, ssum, Kc == (uint32_t)K ? T : -INFINITY, 0.f);
    }
    return;
  }
  // Too many values at or above T (heavy ties or a flat chunk): select by
  // radix instead, starting with the first digit's histogram.
  // Everyone has read out_count; and a full workgroup barrier (release and
  // acquire at workgroup scope) orders the stores above before the
  // select's stores below, which may rewrite the same slots from another
  // wave.
  __syncthreads();
  if (t == 0) sh.out_count = 0u;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (t + kChunkThreads * j < n) atomicAdd(&sh.hist[0][rel_digit(m, x[j])], 1u);  // pass 0
  lds_barrier();

  const DigitSel ds0 = find_digit(sh.hist[0], Kc);
  const uint32_t d0 = ds0.digit;
  const uint32_t need = ds0.need;
  const bool loose = ds0.above + ds0.in_bin <= (uint32_t)cap;
  const bool take_bin = loose || need == ds0.in_bin;
  uint32_t tkey = 0u, tik = 0u;
  if (!take_bin) {
    refine_bucket(
        sh, need, kPerThread, 2, 1,
        [&](int j) { return t + kChunkThreads * j < n && rel_digit(m, x[j]) == d0; },
        [&](int j) { return ddt::f32_key(x[j]); },
        [&](int j) { return 0xFFFFu - (uint32_t)(t + kChunkThreads * j); }, tkey, tik);
  }

  // Selection flags, one LDS atomic per wave for the output base.
  uint32_t selmask = 0u;
  float tmin = INFINITY;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int e = t + kChunkThreads * j;
    bool sel = false;
    if (e < n) {
      const uint32_t d = rel_digit(m, x[j]);
      if (d > d0) {
        sel = true;
      } else if (d == d0) {
        if (take_bin) {
          sel = true;
        } else {
          const uint32_t k = ddt::f32_key(x[j]);
          sel = k > tkey || (k == tkey && (0xFFFFu - (uint32_t)e) >= tik);
        }
      }
    }
    if (sel) {
      selmask |= 1u << j;
      tmin = fminf(tmin, x[j]);
    }
  }
  uint32_t wave_total = 0u;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) wave_total += (uint32_t)__popcll(ddt::ballot((selmask >> j) & 1u));
  uint32_t wbase = 0u;
  if (lane == 0 && wave_total) wbase = atomicAdd(&sh.out_count, wave_total);
  wbase = (uint32_t)__builtin_amdgcn_readfirstlane((int)wbase);
  uint32_t run = 0u;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const bool sel = (selmask >> j) & 1u;
    const uint64_t bm = ddt::ballot(sel);
    if (sel) {
      const uint32_t pos = wbase + run + ddt::lanes_below(bm);
      cand_x[slot0 + pos] = x[j];
      cand_i[slot0 + pos] = base + t + kChunkThreads * j;
    }
    run += (uint32_t)__popcll(bm);
  }
  tmin = ddt::wave_reduce_uniform(tmin, ddt::OpMin());
  if (lane == 0) red[2][wave] = tmin;
  lds_barrier();
  if (t == 0) {
    const float tc = fminf(fminf(red[2][0], red[2][1]), fminf(red[2][2], red[2][3]));
    counts[row * C + chunk] = (int)sh.out_count;
    stats[row * C + chunk] = make_float4(m, ssum, Kc == (uint32_t)K ? tc : -INFINITY, 0.f);
  }
}

struct MergeLds {
  SelShared sh;
  int offs[kMergeThreads + 1];  // exclusive prefix of chunk counts (C <= 1024)
  int cnt[kMergeThreads];       // chunk counts
  float taus[1 + kBounds];      // row thresholds from the chunks' r-bounds
  alignas(16) float sx[kSurvCap];
  alignas(16) int si[kSurvCap];
  alignas(16) float wx[DDTREE_MAX_K];
  alignas(16) int wi[DDTREE_MAX_K];
  alignas(16) uint64_t rk[kMergeThreads];  // rank keys
  int rkc[kMergeThreads / 4];              // ranks counted in parts
  float lse, tau, M;
  int total, slots_per;
  uint32_t nsurv, nkeep, nwin;
};

// The rank order as one unsigned 64-bit key: the logit's order key above,
// the complement of the id below (among equal logits the smaller id ranks
// first). Real keys are nonzero.
__device__ __forceinline__ uint64_t rank_key(float x, int i) {
  return ((uint64_t)ddt::f32_key(x) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
}

// Rank the n pairs in xs/is (n <= kMergeThreads) among themselves, one per
// thread, and write those ranked below K. Each pair's key goes to keys[]
// (padded with zeros, which beat nothing); a thread's rank is the number of
// keys above its own, counted 8 at a time from 16-byte LDS reads. Starts
// with a barrier (after the pairs' writes).
// With n <= kMergeThreads / 4 the keys are counted in four quarters by four
// threads per pair, whose counts meet in ranks[] (LDS atomics).
__device__ __forceinline__ void rank_and_write(const float* xs, const int* is, uint64_t* keys,
                                               int* ranks, int n, int K, float lse,
                                               float* out_lp, int32_t* out_tok) {
  const int t = threadIdx.x;
  constexpr int kParts = 4, kPartThreads = kMergeThreads / kParts;
  const bool split = n <= kPartThreads;
  const int npad = split ? (n + 8 * kParts - 1) & ~(8 * kParts - 1) : (n + 7) & ~7;
  lds_barrier();
  float xt = 0.f;
  int it = 0;
  uint64_t mine = 0;
  if (t < n) {
    xt = xs[t];
    it = is[t];
    mine = rank_key(xt, it);
  }
  if (t < npad) keys[t] = mine;
  if (split && t < kPartThreads) ranks[t] = 0;
  lds_barrier();
  const int c = split ? t % kPartThreads : t;  // the pair this thread counts for
  const int part = split ? t / kPartThreads : 0;
  const int len = split ? npad / kParts : npad;
  if (c < n) {
    const uint64_t key = split ? keys[c] : mine;
    int rank = 0;
    for (int u = part * len; u < (part + 1) * len; u += 8) {
      ulonglong2 a[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) a[k] = *reinterpret_cast<const ulonglong2*>(keys + u + 2 * k);
#pragma unroll
      for (int k = 0; k < 4; ++k) rank += (int)(a[k].x > key) + (int)(a[k].y > key);
    }
    if (split) {
      atomicAdd(&ranks[c], rank);
    } else if (rank < K) {
      out_lp[rank] = xt - lse;
      out_tok[rank] = it;
    }
  }
  if (split) {
    lds_barrier();
    if (t < n) {
      const int rank = ranks[t];
      if (rank < K) {
        out_lp[rank] = xt - lse;
        out_tok[rank] = it;
      }
    }
  }
}

__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(
    int C, int K, int cap, int q, int idx_passes, const float4* __restrict__ stats,
    const float* __restrict__ bounds, const int* __restrict__ counts,
    const float* __restrict__ cand_x, const int* __restrict__ cand_i, float* __restrict__ logp,
    int32_t* __restrict__ token) {
  __shared__ MergeLds s;
  const int row = blockIdx.x, t = threadIdx.x, lane = t & 63;
  const float4* st = stats + (int64_t)row * C;
  const int* cnt = counts + (int64_t)row * C;
  const float* cx = cand_x + (int64_t)row * C * cap;
  const int* ci = cand_i + (int64_t)row * C * cap;

  // Chunk metadata: counts, lse and tau.
  if (t < 64) {
    // One chunk per lane per round; the first round's stats and counts
    // (C <= 64 in the common case) are loaded once and kept.
    const float4 v0 = lane < C ? st[lane] : make_float4(-INFINITY, 0.f, -INFINITY, 0.f);
    const int n0 = lane < C ? cnt[lane] : 0;
    float M = -INFINITY, tau = -INFINITY;
    for (int c0 = 0; c0 < C; c0 += 64) {
      const float4 v = c0 == 0 ? v0
                               : (c0 + lane < C ? st[c0 + lane]
                                                : make_float4(-INFINITY, 0.f, -INFINITY, 0.f));
      M = fmaxf(M, ddt::wave_reduce_uniform(v.x, ddt::OpMax()));
      tau = fmaxf(tau, ddt::wave_reduce_uniform(v.z, ddt::OpMax()));
    }
    float S = 0.f;
    int cmax = 1;
    for (int c0 = 0; c0 < C; c0 += 64) {
      const int c = c0 + lane;
      const float4 v = c0 == 0 ? v0 : (c < C ? st[c] : make_float4(-INFINITY, 0.f, -INFINITY, 0.f));
      S += ddt::wave_reduce_uniform(c < C ? v.y * expf(v.x - M) : 0.f, ddt::OpSum());
      const int x = c0 == 0 ? n0 : (c < C ? cnt[c] : 0);
      if (c < C) s.cnt[c] = x;
      cmax = max(cmax, (int)ddt::wave_reduce_uniform((float)x, ddt::OpMax()));
    }
    if (lane == 0) {
      s.slots_per = cmax;  // the longest list
      s.M = M;
      s.tau = tau;
      s.lse = M + logf(S);
      s.nsurv = 0u;
      s.nkeep = 0u;
      s.nwin = 0u;
      s.sh.out_count = 0u;
    }
  }
  else if (t < 64 * (1 + kBounds)) {
    // Wave b: chunk c holds at least q 2^(b-1) values >= its bound
    // bounds[c][b - 1], so the need-th largest of those bounds over the
    // chunks, need = ceil(K / (q 2^(b-1))), has at least K values of the
    // row at or above it: a lower bound of the row's K-th largest.
    const int b = (t >> 6) - 1;
    const int per = q << b;
    const int need = (K + per - 1) / per;
    float tb = -INFINITY;
    if (C <= 64 && need <= C) {
      const float v = lane < C ? bounds[((int64_t)row * C + lane) * kBounds + b] : -INFINITY;
      const float sv = wave_sort_desc(v);
      tb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sv), need - 1));
    }
    if (lane == 0) s.taus[1 + b] = tb;
  }
  init_hists(s.sh);
  lds_barrier();
  float tau_best = s.tau;
#pragma unroll
  for (int b = 0; b < kBounds; ++b) tau_best = fmaxf(tau_best, s.taus[1 + b]);
  const float tau = tau_best, M = s.M, lse = s.lse;
  float* out_lp = logp + (int64_t)row * K;
  int32_t* out_tok = token + (int64_t)row * K;

  // Candidate i of the row (the chunks' lists concatenated): its chunk is
  // found by binary search over the prefix offsets (made by make_offsets,
  // only on the path that needs them).
  auto cand_at = [&](int i) -> int64_t {
    int lo = 0, hi = C;  // last chunk with offs[c] <= i
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s.offs[mid] <= i) lo = mid; else hi = mid;
    }
    return (int64_t)lo * cap + (i - s.offs[lo]);
  };
  // One pass over the candidates: keep(x) says which to append to sx/si
  // (slots past kSurvCap are dropped, the counter still counts them).
  // Chunk c's list is read by the tpc = floor(1024 / C) threads
  // [c tpc, (c + 1) tpc), thread u of them taking positions u, u + tpc,
  // u + 2 tpc, ...: a thread reads its chunk's count once and then issues
  // a pass of up to NB loads before using any (one pass at K = 64 on the
  // full vocabulary, 38 chunks x <= 137 candidates). NB is 8 when
  // that covers the longest list, else 16 (measured: the 16-wide form is
  // slower at small K although its extra iterations are skipped by uniform
  // branches, and faster at large K, where it saves passes). A thread's kept
  // values go out in one run: an exclusive prefix of the per-thread counts
  // over the wave (five ballots of their bits) and one LDS atomic per wave.
  const int tpc = kMergeThreads / C;
  const int my_c = t / tpc;
  const int my_u = t - my_c * tpc;
  const int my_n = my_c < C ? s.cnt[my_c] : 0;
  const int per_thread = (s.slots_per + tpc - 1) / tpc;
  const float* my_cx = cx + (int64_t)min(my_c, C - 1) * cap;
  const int* my_ci = ci + (int64_t)min(my_c, C - 1) * cap;
  static_assert(kLoadBatchLarge <= 31, "per-thread counts fit five bits");
  auto gather_nb = [&](auto nb_const, uint32_t* counter, auto keep) {
    constexpr int NB = decltype(nb_const)::value;
    for (int r0 = 0; r0 < per_thread; r0 += NB) {
      float xv[NB];
      int iv[NB];
#pragma unroll
      for (int r = 0; r < NB; ++r) {
        const int jj = my_u + tpc * (r0 + r);
        xv[r] = -INFINITY;
        iv[r] = -1;
        if (r0 + r >= per_thread) continue;  // uniform
        if (jj < my_n) {
          xv[r] = my_cx[jj];
          iv[r] = my_ci[jj];
        }
      }
      uint32_t km = 0u, nk = 0u;
#pragma unroll
      for (int r = 0; r < NB; ++r) {
        if (r0 + r >= per_thread) continue;  // uniform
        const bool k = iv[r] >= 0 && keep(xv[r]);
        km |= (uint32_t)k << r;
        nk += (uint32_t)k;
      }
      uint32_t excl = 0u, tot = 0u;
#pragma unroll
      for (int b = 0; b < 5; ++b) {
        const uint64_t bm = ddt::ballot((nk >> b) & 1u);
        excl += ddt::lanes_below(bm) << b;
        tot += (uint32_t)__popcll(bm) << b;
      }
      uint32_t wb = 0u;
      if (lane == 0 && tot) wb = atomicAdd(counter, tot);
      uint32_t pos = (uint32_t)__builtin_amdgcn_readfirstlane((int)wb) + excl;
#pragma unroll
      for (int r = 0; r < NB; ++r) {
        if (r0 + r >= per_thread) continue;  // uniform
        if ((km >> r) & 1u) {
          if (pos < (uint32_t)kSurvCap) {
            s.sx[pos] = xv[r];
            s.si[pos] = iv[r];
          }
          ++pos;
        }
      }
    }
  };

  // Survivors: the candidates >= tau (every top-K element is one). They
  // are counted in the histogram of the first digit relative to the row
  // max, used when there are too many to rank all against all: for
  // K > kFusedHistK as they are gathered (there are usually too many), for
  // smaller K only then, from the survivors in LDS (or, when they overflowed
  // it, by a counting pass over the candidates).
  auto gather = [&](uint32_t* counter, auto keep) {
    if (per_thread <= kLoadBatchSmall)
      gather_nb(std::integral_constant<int, kLoadBatchSmall>{}, counter, keep);
    else
      gather_nb(std::integral_constant<int, kLoadBatchLarge>{}, counter, keep);
  };
  const bool fused_hist = K > kFusedHistK;
  if (fused_hist) {
    gather(&s.nsurv, [&](float x) {
      const bool k = x >= tau;
      if (k) atomicAdd(&s.sh.hist[0][rel_digit(M, x)], 1u);
      return k;
    });
  } else {
    gather(&s.nsurv, [&](float x) { return x >= tau; });
  }
  lds_barrier();
  int nsurv = (int)s.nsurv;
  if (nsurv <= kRankAllMax) {
    // Few survivors: rank each among all of them.
    rank_and_write(s.sx, s.si, s.rk, s.rkc, nsurv, K, lse, out_lp, out_tok);
    return;
  }
  if (!fused_hist) {
    if (nsurv <= kSurvCap) {
      for (int i = t; i < nsurv; i += kMergeThreads)
        atomicAdd(&s.sh.hist[0][rel_digit(M, s.sx[i])], 1u);
    } else {
      gather(&s.nkeep, [&](float x) {  // counts only (appends nothing)
        if (x >= tau) atomicAdd(&s.sh.hist[0][rel_digit(M, x)], 1u);
        return false;
      });
    }
    lds_barrier();
  }

  // The bucket d0 of the row's K-th largest: survivors in it or above it
  // hold the top K (typically K plus a few dozen values).
  const DigitSel ds0 = find_digit(s.sh.hist[0], (uint32_t)K);
  const uint32_t d0 = ds0.digit;
  const uint32_t n_top = ds0.above + ds0.in_bin;
  bool in_lds = nsurv <= kSurvCap;
  if (!in_lds && n_top <= (uint32_t)kSurvCap) {
    // The survivors overflowed LDS (a large K): gather only bucket d0 and
    // above, in a second pass.
    gather(&s.nkeep, [&](float x) { return x >= tau && rel_digit(M, x) >= d0; });
    lds_barrier();
    nsurv = (int)n_top;
    in_lds = true;
  }
  if (n_top <= (uint32_t)kMergeThreads) {
    // Bucket d0 and above fit one per thread (then they are in LDS): move
    // them to wx/wi and rank them among themselves.
    for (int i = t; i < nsurv; i += kMergeThreads) {
      const float x = s.sx[i];
      if (rel_digit(M, x) >= d0) {
        const uint32_t pos = atomicAdd(&s.nwin, 1u);
        s.wx[pos] = x;
        s.wi[pos] = s.si[i];
      }
    }
    rank_and_write(s.wx, s.wi, s.rk, s.rkc, (int)n_top, K, lse, out_lp, out_tok);
    return;
  }

  // Many values in bucket d0 or above (a large K, or a tie-heavy row): exact
  // radix select of the K largest inside bucket d0, over the survivors in
  // LDS, else over the candidates in global memory (those below tau are not
  // survivors there and are skipped), then rank the K winners.
  int total = 0;
  if (!in_lds) {
    // Prefix offsets of the chunks' lists for cand_at (this path only).
    if (t < 64) {
      int carry = 0;
      for (int c0 = 0; c0 < C; c0 += 64) {
        const int c = c0 + lane;
        const int x = c < C ? s.cnt[c] : 0;
        int incl = x;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int o = __shfl_up(incl, off, 64);
          if (lane >= off) incl += o;
        }
        if (c < C) s.offs[c] = carry + incl - x;
        carry += __shfl(incl, 63, 64);
      }
      if (lane == 0) {
        s.offs[C] = carry;
        s.total = carry;
      }
    }
    lds_barrier();
    total = s.total;
  }
  const int n_all = in_lds ? nsurv : total;
  auto elem_x = [&](int i) -> float { return in_lds ? s.sx[i] : cx[cand_at(i)]; };
  auto elem_i = [&](int i) -> int { return in_lds ? s.si[i] : ci[cand_at(i)]; };
  const int per = (n_all + kMergeThreads - 1) / kMergeThreads;
  const uint32_t need = ds0.need;
  const bool take_bin = need == ds0.in_bin;
  uint32_t tkey = 0u, tik = 0u;
  const uint32_t idx_mask = idx_passes >= 4 ? 0xFFFFFFFFu : ((1u << (8 * idx_passes)) - 1u);
  if (!take_bin) {
    refine_bucket(
        s.sh, need, per, idx_passes, 1,
        [&](int r) {
          const int i = t + kMergeThreads * r;
          if (i >= n_all) return false;
          const float x = elem_x(i);
          return x >= tau && rel_digit(M, x) == d0;
        },
        [&](int r) { return ddt::f32_key(elem_x(t + kMergeThreads * r)); },
        [&](int r) { return idx_mask - (uint32_t)elem_i(t + kMergeThreads * r); }, tkey, tik);
  }
  for (int r = 0; r < per; ++r) {
    const int i = t + kMergeThreads * r;
    if (i >= n_all) continue;
    const float x = elem_x(i);
    if (!(x >= tau)) continue;
    const uint32_t d = rel_digit(M, x);
    bool sel = d > d0;
    if (d == d0) {
      if (take_bin) {
        sel = true;
      } else {
        const uint32_t k = ddt::f32_key(x);
        sel = k > tkey || (k == tkey && (idx_mask - (uint32_t)elem_i(i)) >= tik);
      }
    }
    if (sel) {
      const uint32_t pos = atomicAdd(&s.nwin, 1u);
      if (pos < (uint32_t)DDTREE_MAX_K) {
        s.wx[pos] = x;
        s.wi[pos] = elem_i(i);
      }
    }
  }
  rank_and_write(s.wx, s.wi, s.rk, s.rkc, K, K, lse, out_lp, out_tok);
}

}  // namespace

namespace ddt_host {

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

TopkPlan topk_plan(int L, int V, int K) {
  TopkPlan p;
  p.C = (V + kChunk - 1) / kChunk;
  p.cap = K + kLooseExtra;
  int bits = 1;
  while (bits < 31 && ((int64_t)1 << bits) < (int64_t)V) ++bits;
  p.idx_passes = (bits + 7) / 8;
  const size_t LC = (size_t)L * p.C;
  p.q = 1;
  while (p.q < 16 && p.q * 64 < K) p.q <<= 1;
  p.stats_off = 0;
  p.bounds_off = align_up(p.stats_off + LC * sizeof(float4), 256);
  p.counts_off = align_up(p.bounds_off + LC * kBounds * sizeof(float), 256);
  p.candx_off = align_up(p.counts_off + LC * sizeof(int), 256);
  p.candi_off = align_up(p.candx_off + LC * p.cap * sizeof(float), 256);
  p.bytes = align_up(p.candi_off + LC * p.cap * sizeof(int), 256);
  return p;
}

int topk_launch(const float* logits, int64_t stride, int L, int V, int K,
                float* logp, int32_t* token, void* ws, hipStream_t stream) {
  const TopkPlan p = topk_plan(L, V, K);
  if (p.C > kMergeThreads) return DDTREE_ERR_UNSUPPORTED;
  char* w = static_cast<char*>(ws);
  float4* stats = reinterpret_cast<float4*>(w + p.stats_off);
  float* bounds = reinterpret_cast<float*>(w + p.bounds_off);
  int* counts = reinterpret_cast<int*>(w + p.counts_off);
  float* cx = reinterpret_cast<float*>(w + p.candx_off);
  int* ci = reinterpret_cast<int*>(w + p.candi_off);
  hipLaunchKernelGGL(topk_chunk_kernel, dim3(p.C, L), dim3(kChunkThreads), 0, stream,
                     logits, stride, V, K, p.cap, p.q, stats, bounds, counts, cx, ci);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return launch_status(e);
  hipLaunchKernelGGL(topk_merge_kernel, dim3(L), dim3(kMergeThreads), 0, stream,
                     p.C, K, p.cap, p.q, p.idx_passes, stats, bounds, counts, cx, ci, logp, token);
  return launch_status(hipGetLastError());
}

}  // namespace ddt_host
