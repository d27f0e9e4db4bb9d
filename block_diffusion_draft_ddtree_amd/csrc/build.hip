// ddtree_build: best-first selection of the top-B prefixes ("DDTree Deep
// Dive", section 2, Proposition 3) and the tree arrays and ancestor mask
// (sections 3 and 4).
//
// One workgroup of 256 threads; wave 0 runs the serial pops, the other
// waves only help stage the top-K table into LDS and write the outputs.
//
// Heap layout. Proposition 3 pushes, for every popped prefix, its next
// sibling and its first child. Equivalently every popped node (and the
// root) owns exactly one "slot" that holds its next not-yet-popped child:
// popping slot p's candidate creates node b, advances slot p to its next
// sibling rank and opens slot b at child rank 0. So the frontier is an
// array of at most B + 1 slots indexed by node id; slot n lives in lane
// n & 63, register n >> 6 of wave 0, as the 32-bit order key of its
// candidate's fp32 score. A pop is a wave-wide max of the lanes' local
// maxima (shuffle butterfly) plus a ballot; exact score ties fall back to a
// wave-cooperative lexicographic comparison of the rank tuples, which are
// rebuilt from the parent/rank arrays in LDS.
//
// Scores follow the fp32 left-to-right sum: a depth-1 candidate is logp[0][r]
// itself, deeper ones fl(score(parent) + logp[d][r]).
#include "common.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxN = DDTREE_MAX_B + 1;

struct BuildLds {
  float lp[DDTREE_MAX_LK];
  float score[kMaxN];
  float cscore[kMaxN];  // score of the slot's current candidate
  int16_t parent[kMaxN];
  int16_t rank[kMaxN];   // last rank of the node's tuple
  int16_t crank[kMaxN];  // rank of the slot's current candidate
  uint8_t depth[kMaxN];
};

__device__ __forceinline__ void compiler_fence() { __asm__ volatile("" ::: "memory"); }

// Rank at depth `d` (1-based) of the tuple of node `x` (depth(x) >= d).
__device__ __forceinline__ int rank_at(const BuildLds& s, int x, int d) {
  while (s.depth[x] > d) x = s.parent[x];
  return s.rank[x];
}

// Wave-uniform: is the candidate of slot a lexicographically before the
// candidate of slot b? Lane i holds element i of each rank tuple.
__device__ bool cand_lex_less(const BuildLds& s, int a, int b) {
  const int lane = ddt::lane_id();
  const int da = s.depth[a] + 1, db = s.depth[b] + 1;
  int xa = -1, xb = -1;
  if (lane < da) xa = (lane == da - 1) ? (int)s.crank[a] : rank_at(s, a, lane + 1);
  if (lane < db) xb = (lane == db - 1) ? (int)s.crank[b] : rank_at(s, b, lane + 1);
  const uint64_t diff = ddt::ballot(xa != xb);
  if (!diff) return a < b;  // identical tuples cannot occur
  const int f = __ffsll((unsigned long long)diff) - 1;
  if (f >= da) return true;   // a is a proper prefix of b
  if (f >= db) return false;
  return __shfl(xa, f, 64) < __shfl(xb, f, 64);
}

template <int J>
__device__ void pop_loop(BuildLds& s, int L, int K, int B) {
  const int lane = ddt::lane_id();
  uint32_t rk[J];
#pragma unroll
  for (int j = 0; j < J; ++j) rk[j] = 0u;
  if (lane == 0) rk[0] = ddt::f32_key(s.cscore[0]);

  for (int b = 1; b <= B; ++b) {
    // Local maximum over this lane's slots.
    uint32_t lk = 0u;
    int lj = 0;
    bool ltie = false;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (rk[j] > lk) {
        lk = rk[j];
        lj = j;
        ltie = false;
      } else if (rk[j] == lk && lk != 0u) {
        ltie = true;
      }
    }
    const uint32_t kmax = ddt::wave_max_u32(lk);
    const uint64_t hit = ddt::ballot(lk == kmax);
    const uint64_t tie = ddt::ballot(lk == kmax && ltie);
    int p;
    if (__popcll(hit) == 1 && tie == 0) {
      const int wl = __ffsll((unsigned long long)hit) - 1;
      p = __shfl(lane + 64 * lj, wl, 64);
    } else {
      // Several slots share the best score: smallest rank tuple wins.
      p = -1;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        uint64_t m = ddt::ballot(rk[j] == kmax);
        while (m) {
          const int l = __ffsll((unsigned long long)m) - 1;
          m &= m - 1;
          const int cand = l + 64 * j;
          if (p < 0 || cand_lex_less(s, cand, p)) p = cand;
        }
      }
    }
    p = __builtin_amdgcn_readfirstlane(p);

    const int c = s.crank[p];
    const float sc = s.cscore[p];
    const int dp = s.depth[p];
    const int dn = dp + 1;
    // Advance slot p to its next sibling.
    const int c2 = c + 1;
    uint32_t pk = 0u;
    float ps = 0.f;
    if (c2 < K) {
      ps = (dp == 0) ? s.lp[c2] : (s.score[p] + s.lp[dp * K + c2]);
      pk = ddt::f32_key(ps);
    }
    // Open slot b at its first child.
    uint32_t bk = 0u;
    float bs = 0.f;
    if (dn < L) {
      bs = sc + s.lp[dn * K];
      bk = ddt::f32_key(bs);
    }
    compiler_fence();
    if (lane == 0) {
      s.parent[b] = (int16_t)p;
      s.rank[b] = (int16_t)c;
      s.depth[b] = (uint8_t)dn;
      s.score[b] = sc;
      s.crank[p] = (int16_t)c2;
      s.cscore[p] = ps;
      s.crank[b] = 0;
      s.cscore[b] = bs;
    }
    compiler_fence();
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (lane == (p & 63) && j == (p >> 6)) rk[j] = pk;
      if (lane == (b & 63) && j == (b >> 6)) rk[j] = bk;
    }
  }
}

template <int J>
__global__ __launch_bounds__(kThreads) void build_kernel(
    const float* __restrict__ logp, const int32_t* __restrict__ token, int L, int K,
    int B, const int32_t* __restrict__ root_token, int32_t* __restrict__ parent_out,
    int32_t* __restrict__ depth_out, int32_t* __restrict__ tok_out,
    float* __restrict__ score_out, uint32_t* __restrict__ anc, int W) {
  __shared__ BuildLds s;
  const int t = threadIdx.x;
  const int LK = L * K;
  for (int i = t; i < LK; i += kThreads) s.lp[i] = logp[i];
  if (t == 0) {
    s.parent[0] = -1;
    s.rank[0] = 0;
    s.depth[0] = 0;
    s.score[0] = 0.f;
  }
  __syncthreads();
  if (t == 0) {
    s.crank[0] = 0;
    s.cscore[0] = s.lp[0];
  }
  __syncthreads();
  if (t < 64) pop_loop<J>(s, L, K, B);
  __syncthreads();

  const int N = B + 1;
  for (int n = t; n < N; n += kThreads) {
    const int d = s.depth[n];
    parent_out[n] = s.parent[n];
    depth_out[n] = d;
    tok_out[n] = n == 0 ? *root_token : token[(d - 1) * K + s.rank[n]];
    if (score_out) score_out[n] = s.score[n];
    // Ancestor-or-self row, written from the high word down.
    uint32_t* row = anc + (int64_t)n * W;
    int wcur = W - 1;
    const int wn = n >> 5;
    for (; wcur > wn; --wcur) row[wcur] = 0u;
    uint32_t acc = 0u;
    for (int j = n; j != -1; j = s.parent[j]) {
      const int wj = j >> 5;
      while (wj < wcur) {
        row[wcur] = acc;
        acc = 0u;
        --wcur;
      }
      acc |= 1u << (j & 31);
    }
    row[wcur] = acc;
    for (--wcur; wcur >= 0; --wcur) row[wcur] = 0u;
  }
}

}  // namespace

namespace ddt_host {

int build_launch(const float* logp, const int32_t* token, int L, int K, int B,
                 const int32_t* root_token, int32_t* parent, int32_t* depth,
                 int32_t* node_token, float* score, uint32_t* anc, int W,
                 hipStream_t stream) {
  const int N = B + 1;
#define DDT_BUILD(JJ)                                                              \
  hipLaunchKernelGGL(build_kernel<JJ>, dim3(1), dim3(kThreads), 0, stream, logp,   \
                     token, L, K, B, root_token, parent, depth, node_token, score, \
                     anc, W)
  if (N <= 64) DDT_BUILD(1);
  else if (N <= 128) DDT_BUILD(2);
  else if (N <= 256) DDT_BUILD(4);
  else if (N <= 512) DDT_BUILD(8);
  else DDT_BUILD(17);
#undef DDT_BUILD
  return launch_status(hipGetLastError());
}

}  // namespace ddt_host
