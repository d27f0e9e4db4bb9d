// ddtree_topk: fused log-softmax + top-K over the drafter's per-position
// logits ("DDTree Deep Dive", section 1 and section 2 Lemma 1).
//
// Two launches on one stream:
//   chunk kernel  grid (C chunks, L rows), 256 threads, 4096 logits per
//                 workgroup held in registers (16 per thread, coalesced
//                 dword loads: one HBM pass). Emits the chunk's (max,
//                 sum-exp) pair and a candidate superset of the chunk's top-K.
//   merge kernel  grid L, 1024 threads. Combines the (max, sum) pairs into
//                 lse, selects the exact top-K among the candidates, ranks
//                 them and writes logp = x - lse and the token ids.
//
// Selection is a radix select. Its first digit is relative to the reference
// maximum m: digit = bits(fl(m - x) + 1) >> 19, clamped (16 bins per octave
// of the distance below the max), which spreads the few values near the top
// over many bins and keeps LDS atomic contention low. The boundary bin is
// then refined on the exact fp32 order key (4 x 8 bits) and, for exact ties,
// on the token index (smaller id first). The chunk kernel may stop after the
// first digit when the candidate set fits its slots ("loose" mode); the
// merge kernel always resolves exactly.
#include "common.hpp"

namespace {

constexpr int kChunkThreads = 256;
constexpr int kPerThread = 16;
constexpr int kChunk = kChunkThreads * kPerThread;  // 4096
constexpr int kLooseExtra = 256;                     // slots beyond K per chunk
constexpr int kMergeThreads = 1024;

// Larger digit = closer to the reference maximum (monotone in x).
__device__ __forceinline__ uint32_t rel_digit(float ref_max, float x) {
  const float y = (ref_max - x) + 1.0f;
  uint32_t b = (__float_as_uint(y) - 0x3F800000u) >> 19;
  b = b > 255u ? 255u : b;
  return 255u - b;
}

struct SelShared {
  uint32_t hist[256];
  uint32_t digit;   // digit of the boundary bucket
  uint32_t need;    // how many to take from that bucket
  uint32_t above;   // active elements in buckets above it
  uint32_t in_bin;  // active elements in that bucket
  uint32_t out_count;
};

__device__ __forceinline__ void zero_hist(SelShared& s) {
  for (int i = threadIdx.x; i < 256; i += blockDim.x) s.hist[i] = 0u;
}

// With hist filled (and a barrier passed), find the bucket holding the
// need-th largest active element. Ends with a barrier.
__device__ void find_digit(SelShared& s, uint32_t need) {
  if (threadIdx.x < 64) {
    const int l = threadIdx.x;
    const uint32_t h0 = s.hist[4 * l], h1 = s.hist[4 * l + 1];
    const uint32_t h2 = s.hist[4 * l + 2], h3 = s.hist[4 * l + 3];
    const uint32_t lsum = h0 + h1 + h2 + h3;
    uint32_t suf = lsum;  // inclusive suffix sum over lanes (high digits last)
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_down(suf, off, 64);
      if (l + off < 64) suf += o;
    }
    const uint32_t above = suf - lsum;
    if (above < need && need <= suf) {
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
      s.digit = d;
      s.above = a;
      s.in_bin = hh;
      s.need = need - a;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ float block_max_256(float v, float* red) {
  v = ddt::wave_max_f32(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_sum_256(float v, float* red) {
  v = ddt::wave_sum_f32(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const float r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kChunkThreads) void topk_chunk_kernel(
    const float* __restrict__ logits, int64_t stride, int V, int K, int cap,
    float2* __restrict__ stats, int* __restrict__ counts,
    float* __restrict__ cand_x, int* __restrict__ cand_i) {
  __shared__ SelShared sh;
  __shared__ float red[4];
  const int chunk = blockIdx.x, row = blockIdx.y, C = gridDim.x;
  const int base = chunk * kChunk;
  const int n = min(kChunk, V - base);
  const int t = threadIdx.x;
  const float* src = logits + (int64_t)row * stride + base;

  float x[kPerThread];
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const int e = t + kChunkThreads * j;
    x[j] = e < n ? src[e] : -INFINITY;
  }
  if (t == 0) sh.out_count = 0u;

  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) m = fmaxf(m, x[j]);
  m = block_max_256(m, red);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (t + kChunkThreads * j < n) s += __expf(x[j] - m);
  s = block_sum_256(s, red);

  const uint32_t Kc = (uint32_t)min(K, n);

  // Pass 0: distance-to-max digit.
  zero_hist(sh);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (t + kChunkThreads * j < n) atomicAdd(&sh.hist[rel_digit(m, x[j])], 1u);
  __syncthreads();
  find_digit(sh, Kc);
  const uint32_t d0 = sh.digit;
  uint32_t need = sh.need;
  const bool loose = sh.above + sh.in_bin <= (uint32_t)cap;
  bool take_bin = loose || need == sh.in_bin;
  uint32_t tkey = 0u, tik = 0u;
  if (!take_bin) {
    uint32_t prefix = 0u, mask = 0u, inb = 0u;
    for (int shift = 24; shift >= 0; shift -= 8) {
      __syncthreads();
      zero_hist(sh);
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kPerThread; ++j) {
        if (t + kChunkThreads * j < n && rel_digit(m, x[j]) == d0) {
          const uint32_t k = ddt::f32_key(x[j]);
          if ((k & mask) == prefix) atomicAdd(&sh.hist[(k >> shift) & 255u], 1u);
        }
      }
      __syncthreads();
      find_digit(sh, need);
      prefix |= sh.digit << shift;
      mask |= 255u << shift;
      need = sh.need;
      inb = sh.in_bin;
    }
    tkey = prefix;
    if (need < inb) {
      uint32_t ip = 0u, im = 0u;
      for (int shift = 8; shift >= 0; shift -= 8) {
        __syncthreads();
        zero_hist(sh);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
          const int e = t + kChunkThreads * j;
          if (e < n && rel_digit(m, x[j]) == d0 && ddt::f32_key(x[j]) == tkey) {
            const uint32_t ik = 0xFFFFu - (uint32_t)e;
            if ((ik & im) == ip) atomicAdd(&sh.hist[(ik >> shift) & 255u], 1u);
          }
        }
        __syncthreads();
        find_digit(sh, need);
        ip |= sh.digit << shift;
        im |= 255u << shift;
        need = sh.need;
      }
      tik = ip;
    }
  }

  const int64_t slot0 = ((int64_t)row * C + chunk) * cap;
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
    const uint64_t bm = ddt::ballot(sel);
    uint32_t wbase = 0u;
    if ((t & 63) == 0 && bm) wbase = atomicAdd(&sh.out_count, (uint32_t)__popcll(bm));
    wbase = __shfl(wbase, 0, 64);
    if (sel) {
      const uint32_t pos = wbase + ddt::lanes_below(bm);
      cand_x[slot0 + pos] = x[j];
      cand_i[slot0 + pos] = base + e;
    }
  }
  __syncthreads();
  if (t == 0) {
    counts[row * C + chunk] = (int)sh.out_count;
    stats[row * C + chunk] = make_float2(m, s);
  }
}

__global__ __launch_bounds__(kMergeThreads) void topk_merge_kernel(
    int C, int K, int cap, int idx_passes, const float2* __restrict__ stats,
    const int* __restrict__ counts, const float* __restrict__ cand_x,
    const int* __restrict__ cand_i, float* __restrict__ logp,
    int32_t* __restrict__ token) {
  __shared__ SelShared sh;
  __shared__ float wx[DDTREE_MAX_K];
  __shared__ int wi[DDTREE_MAX_K];
  __shared__ float s_lse, s_max;
  const int row = blockIdx.x, t = threadIdx.x;
  const float2* st = stats + (int64_t)row * C;
  const int* cnt = counts + (int64_t)row * C;
  const int64_t slot_row = (int64_t)row * C * cap;

  if (t == 0) {
    float M = -INFINITY;
    for (int c = 0; c < C; ++c) M = fmaxf(M, st[c].x);
    float S = 0.f;
    for (int c = 0; c < C; ++c) S += st[c].y * expf(st[c].x - M);
    s_max = M;
    s_lse = M + logf(S);
    sh.out_count = 0u;
  }
  __syncthreads();
  const float M = s_max;

  // Visit every candidate of the row: f(x, token id).
#define FOR_EACH_CAND(BODY)                                                   \
  for (int c = 0; c < C; ++c) {                                               \
    const int nc = cnt[c];                                                    \
    for (int j = t; j < nc; j += kMergeThreads) {                             \
      const float x = cand_x[slot_row + (int64_t)c * cap + j];                \
      const int id = cand_i[slot_row + (int64_t)c * cap + j];                 \
      BODY                                                                    \
    }                                                                         \
  }

  zero_hist(sh);
  __syncthreads();
  FOR_EACH_CAND({ (void)id; atomicAdd(&sh.hist[rel_digit(M, x)], 1u); })
  __syncthreads();
  find_digit(sh, (uint32_t)K);
  const uint32_t d0 = sh.digit;
  uint32_t need = sh.need;
  const bool take_bin = need == sh.in_bin;
  uint32_t tkey = 0u, tik = 0u;
  const uint32_t idx_mask = idx_passes >= 4 ? 0xFFFFFFFFu : ((1u << (8 * idx_passes)) - 1u);
  if (!take_bin) {
    uint32_t prefix = 0u, mask = 0u, inb = 0u;
    for (int shift = 24; shift >= 0; shift -= 8) {
      __syncthreads();
      zero_hist(sh);
      __syncthreads();
      FOR_EACH_CAND({
        (void)id;
        if (rel_digit(M, x) == d0) {
          const uint32_t k = ddt::f32_key(x);
          if ((k & mask) == prefix) atomicAdd(&sh.hist[(k >> shift) & 255u], 1u);
        }
      })
      __syncthreads();
      find_digit(sh, need);
      prefix |= sh.digit << shift;
      mask |= 255u << shift;
      need = sh.need;
      inb = sh.in_bin;
    }
    tkey = prefix;
    if (need < inb) {
      uint32_t ip = 0u, im = 0u;
      for (int shift = 8 * (idx_passes - 1); shift >= 0; shift -= 8) {
        __syncthreads();
        zero_hist(sh);
        __syncthreads();
        FOR_EACH_CAND({
          if (rel_digit(M, x) == d0 && ddt::f32_key(x) == tkey) {
            const uint32_t ik = idx_mask - (uint32_t)id;
            if ((ik & im) == ip) atomicAdd(&sh.hist[(ik >> shift) & 255u], 1u);
          }
        })
        __syncthreads();
        find_digit(sh, need);
        ip |= sh.digit << shift;
        im |= 255u << shift;
        need = sh.need;
      }
      tik = ip;
    }
  }
  __syncthreads();
  FOR_EACH_CAND({
    const uint32_t d = rel_digit(M, x);
    bool sel = d > d0;
    if (d == d0) {
      if (take_bin) {
        sel = true;
      } else {
        const uint32_t k = ddt::f32_key(x);
        sel = k > tkey || (k == tkey && (idx_mask - (uint32_t)id) >= tik);
      }
    }
    if (sel) {
      const uint32_t pos = atomicAdd(&sh.out_count, 1u);
      wx[pos] = x;
      wi[pos] = id;
    }
  })
#undef FOR_EACH_CAND
  __syncthreads();
  // Rank the K winners: larger logit first, then smaller id.
  if (t < K) {
    const float xt = wx[t];
    const int it = wi[t];
    int rank = 0;
    for (int u = 0; u < K; ++u) {
      const float xu = wx[u];
      rank += (xu > xt) || (xu == xt && wi[u] < it);
    }
    logp[(int64_t)row * K + rank] = xt - s_lse;
    token[(int64_t)row * K + rank] = it;
  }
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
  p.counts_off = align_up(p.stats_off + LC * sizeof(float2), 256);
  p.candx_off = align_up(p.counts_off + LC * sizeof(int), 256);
  p.candi_off = align_up(p.candx_off + LC * p.cap * sizeof(float), 256);
  p.bytes = align_up(p.candi_off + LC * p.cap * sizeof(int), 256);
  return p;
}

int topk_launch(const float* logits, int64_t stride, int L, int V, int K,
                float* logp, int32_t* token, void* ws, hipStream_t stream) {
  const TopkPlan p = topk_plan(L, V, K);
  char* w = static_cast<char*>(ws);
  float2* stats = reinterpret_cast<float2*>(w + p.stats_off);
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
