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
#include "common.hpp"

namespace {

constexpr int kChunkThreads = 256;
constexpr int kPerThread = 16;
constexpr int kChunk = kChunkThreads * kPerThread;  // 4096
constexpr int kLooseExtra = 256;                     // slots beyond K per chunk
constexpr int kMergeThreads = 1024;
constexpr int kSurvCap = 16384;                      // survivors selected in LDS (128 KB)
constexpr int kLoadBatch = 8;                        // candidates loaded per thread at once
constexpr int kRankAllMax = 256;                     // survivors ranked all against all

// Larger digit = closer to the reference maximum (monotone in x).
__device__ __forceinline__ uint32_t rel_digit(float ref_max, float x) {
  const float y = (ref_max - x) + 1.0f;
  uint32_t b = (__float_as_uint(y) - 0x3F800000u) >> 19;
  b = b > 255u ? 255u : b;
  return 255u - b;
}

// a before b in rank order: larger logit first, then smaller id.
__device__ __forceinline__ bool beats(float xa, int ia, float xb, int ib) {
  return xa > xb || (xa == xb && ia < ib);
}

// Rank of (xt, it) among xs/is[0, n) (how many beat it), n a multiple of 16
// (pad with sentinels that beat nothing: -inf logit, largest id). Sixteen
// candidates per iteration with 16-byte LDS reads, so the reads of an
// iteration are in flight together.
__device__ __forceinline__ int rank_among(const float* xs, const int* is, int n, float xt,
                                          int it) {
  int rank = 0;
  for (int u = 0; u < n; u += 16) {
    float4 xa[4];
    int4 ia[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      xa[q] = *reinterpret_cast<const float4*>(xs + u + 4 * q);
      ia[q] = *reinterpret_cast<const int4*>(is + u + 4 * q);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      rank += beats(xa[q].x, ia[q].x, xt, it);
      rank += beats(xa[q].y, ia[q].y, xt, it);
      rank += beats(xa[q].z, ia[q].z, xt, it);
      rank += beats(xa[q].w, ia[q].w, xt, it);
    }
  }
  return rank;
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
  __syncthreads();
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
    __syncthreads();
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
      __syncthreads();
      const DigitSel ds = find_digit(h, need);
      ip |= ds.digit << shift;
      im |= 255u << shift;
      need = ds.need;
    }
    tik = ip;
  }
}

__global__ __launch_bounds__(kChunkThreads) void topk_chunk_kernel(
    const float* __restrict__ logits, int64_t stride, int V, int K, int cap,
    float4* __restrict__ stats, int* __restrict__ counts, float* __restrict__ cand_x,
    int* __restrict__ cand_i) {
  __shared__ SelShared sh;
  __shared__ float red[3][4];
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

  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) mx = fmaxf(mx, x[j]);
  mx = ddt::wave_reduce_uniform(mx, ddt::OpMax());
  if (lane == 0) red[0][wave] = mx;
  __syncthreads();
  const float m = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));

  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    if (t + kChunkThreads * j < n) {
      s += __expf(x[j] - m);
      atomicAdd(&sh.hist[0][rel_digit(m, x[j])], 1u);  // pass 0
    }
  }
  s = ddt::wave_reduce_uniform(s, ddt::OpSum());
  if (lane == 0) red[1][wave] = s;
  __syncthreads();

  const uint32_t Kc = (uint32_t)min(K, n);
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
  const int64_t slot0 = ((int64_t)row * C + chunk) * cap;
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
  __syncthreads();
  if (t == 0) {
    const float ssum = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
    const float tc = fminf(fminf(red[2][0], red[2][1]), fminf(red[2][2], red[2][3]));
    counts[row * C + chunk] = (int)sh.out_count;
    stats[row * C + chunk] = make_float4(m, ssum, Kc == (uint32_t)K ? tc : -INFINITY, 0.f);
  }
}

struct MergeLds {
  SelShared sh;
  int offs[kMergeThreads + 1];  // exclusive prefix of chunk counts (C <= 1024)
  alignas(16) float sx[kSurvCap];
  alignas(16) int si[kSurvCap];
  alignas(16) float wx[DDTREE_MAX_K];
  alignas(16) int wi[DDTREE_MAX_K];
  float lse, tau, M;
  int total;
  uint32_t nsurv, nkeep, nwin;
};

// Rank the n pairs in xs/is (n <= kMergeThreads, arrays padded to a multiple
// of 16 with room) among themselves, one per thread, and write those ranked
// below K. Starts with a barrier (after the pairs' writes).
__device__ __forceinline__ void rank_and_write(float* xs, int* is, int n, int K, float lse,
                                               float* out_lp, int32_t* out_tok) {
  const int t = threadIdx.x;
  const int npad = (n + 15) & ~15;
  __syncthreads();
  if (t >= n && t < npad) {
    xs[t] = -INFINITY;
    is[t] = 0x7FFFFFFF;
  }
  __syncthreads();
  if (t < n) {
    const float xt = xs[t];
    const int it = is[t];
    const int rank = rank_among(xs, is, npad, xt, it);
    if (rank < K) {
      out_lp[rank] = xt - lse;
      out_tok[rank] = it;
    }
  }
}

__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(
    int C, int K, int cap, int idx_passes, const float4* __restrict__ stats,
    const int* __restrict__ counts, const float* __restrict__ cand_x,
    const int* __restrict__ cand_i, float* __restrict__ logp, int32_t* __restrict__ token) {
  __shared__ MergeLds s;
  const int row = blockIdx.x, t = threadIdx.x, lane = t & 63;
  const float4* st = stats + (int64_t)row * C;
  const int* cnt = counts + (int64_t)row * C;
  const float* cx = cand_x + (int64_t)row * C * cap;
  const int* ci = cand_i + (int64_t)row * C * cap;

  // Chunk metadata: prefix offsets of the candidate lists, lse and tau.
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
    int carry = 0;
    for (int c0 = 0; c0 < C; c0 += 64) {
      const int c = c0 + lane;
      const float4 v = c0 == 0 ? v0 : (c < C ? st[c] : make_float4(-INFINITY, 0.f, -INFINITY, 0.f));
      S += ddt::wave_reduce_uniform(c < C ? v.y * expf(v.x - M) : 0.f, ddt::OpSum());
      int x = c0 == 0 ? n0 : (c < C ? cnt[c] : 0);
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
      s.M = M;
      s.tau = tau;
      s.lse = M + logf(S);
      s.nsurv = 0u;
      s.nkeep = 0u;
      s.nwin = 0u;
      s.sh.out_count = 0u;
    }
  }
  init_hists(s.sh);
  __syncthreads();
  const int total = s.total;
  const float tau = s.tau, M = s.M, lse = s.lse;
  float* out_lp = logp + (int64_t)row * K;
  int32_t* out_tok = token + (int64_t)row * K;

  // Candidate i of the row (the chunks' lists concatenated): its chunk is
  // found by binary search over the prefix offsets.
  auto cand_at = [&](int i) -> int64_t {
    int lo = 0, hi = C;  // last chunk with offs[c] <= i
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s.offs[mid] <= i) lo = mid; else hi = mid;
    }
    return (int64_t)lo * cap + (i - s.offs[lo]);
  };
  // One pass over the candidates, kLoadBatch per thread at a time: keep(x)
  // says which to append to sx/si (one LDS atomic per wave on `counter`;
  // slots past kSurvCap are dropped, the counter still counts them).
  auto gather = [&](uint32_t* counter, auto keep) {
    for (int g0 = 0; g0 < total; g0 += kMergeThreads * kLoadBatch) {
      float xv[kLoadBatch];
      int iv[kLoadBatch];
#pragma unroll
      for (int r = 0; r < kLoadBatch; ++r) {
        const int i = g0 + t + kMergeThreads * r;
        xv[r] = -INFINITY;
        iv[r] = -1;
        if (i < total) {
          const int64_t at = cand_at(i);
          xv[r] = cx[at];
          iv[r] = ci[at];
        }
      }
#pragma unroll
      for (int r = 0; r < kLoadBatch; ++r) {
        const bool k = iv[r] >= 0 && keep(xv[r]);
        const uint64_t bm = ddt::ballot(k);
        uint32_t wb = 0u;
        if (lane == 0 && bm) wb = atomicAdd(counter, (uint32_t)__popcll(bm));
        wb = (uint32_t)__builtin_amdgcn_readfirstlane((int)wb);
        if (k) {
          const uint32_t pos = wb + ddt::lanes_below(bm);
          if (pos < (uint32_t)kSurvCap) {
            s.sx[pos] = xv[r];
            s.si[pos] = iv[r];
          }
        }
      }
    }
  };

  // Survivors: the candidates >= tau (every top-K element is one), each also
  // counted in the histogram of the first digit relative to the row max.
  gather(&s.nsurv, [&](float x) {
    const bool k = x >= tau;
    if (k) atomicAdd(&s.sh.hist[0][rel_digit(M, x)], 1u);
    return k;
  });
  __syncthreads();
  int nsurv = (int)s.nsurv;
  if (nsurv <= kRankAllMax) {
    // Few survivors: rank each among all of them.
    rank_and_write(s.sx, s.si, nsurv, K, lse, out_lp, out_tok);
    return;
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
    __syncthreads();
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
    rank_and_write(s.wx, s.wi, (int)n_top, K, lse, out_lp, out_tok);
    return;
  }

  // Many values in bucket d0 or above (a large K, or a tie-heavy row): exact
  // radix select of the K largest inside bucket d0, over the survivors in
  // LDS, else over the candidates in global memory (those below tau are not
  // survivors there and are skipped), then rank the K winners.
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
  rank_and_write(s.wx, s.wi, K, K, lse, out_lp, out_tok);
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
  p.stats_off = 0;
  p.counts_off = align_up(p.stats_off + LC * sizeof(float4), 256);
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
  int* counts = reinterpret_cast<int*>(w + p.counts_off);
  float* cx = reinterpret_cast<float*>(w + p.candx_off);
  int* ci = reinterpret_cast<int*>(w + p.candi_off);
  hipLaunchKernelGGL(topk_chunk_kernel, dim3(p.C, L), dim3(kChunkThreads), 0, stream,
                     logits, stride, V, K, p.cap, stats, counts, cx, ci);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return launch_status(e);
  hipLaunchKernelGGL(topk_merge_kernel, dim3(L), dim3(kMergeThreads), 0, stream,
                     p.C, K, p.cap, p.idx_passes, stats, counts, cx, ci, logp, token);
  return launch_status(hipGetLastError());
}

}  // namespace ddt_host
