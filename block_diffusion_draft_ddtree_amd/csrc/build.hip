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
// array of at most B + 1 slots indexed by node id. Slot n lives in lane
// n & 63, register n >> 6 of wave 0, which keeps everything about it in
// registers: its candidate's order key and fp32 score, the candidate's
// rank, the node's own score, depth, parent and rank, and the log-prob of
// the candidate after the current one (prefetched from LDS so that
// advancing a slot never waits on memory).
//
// A pop: each lane takes the max key over its slots, a DPP max inside each
// 16-lane row plus four readlanes gives the wave max in a scalar register,
// and a ballot finds the owner. Exact score ties fall back to a
// wave-cooperative lexicographic comparison of the rank tuples, which are
// rebuilt from parent/rank arrays kept in LDS.
//
// Scores follow the fp32 left-to-right sum: a depth-1 candidate is logp[0][r]
// itself, deeper ones fl(score(parent) + logp[d][r]).
#include "common.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxN = DDTREE_MAX_B + 1;

struct BuildLds {
  float lp[DDTREE_MAX_LK];
  int16_t parent[kMaxN];
  int16_t rank[kMaxN];
  uint8_t depth[kMaxN];
};

// DPP controls (gfx9 encoding).
constexpr int kQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7 - i within each 8 lanes
constexpr int kRowMirror = 0x140;      // lane i <-> 15 - i within each 16 lanes

__device__ __forceinline__ uint32_t dpp_umax(uint32_t v, int ctrl_id) {
  uint32_t o;
  switch (ctrl_id) {
    case 0: o = __builtin_amdgcn_update_dpp(v, v, kQuadXor1, 0xF, 0xF, false); break;
    case 1: o = __builtin_amdgcn_update_dpp(v, v, kQuadXor2, 0xF, 0xF, false); break;
    case 2: o = __builtin_amdgcn_update_dpp(v, v, kRowHalfMirror, 0xF, 0xF, false); break;
    default: o = __builtin_amdgcn_update_dpp(v, v, kRowMirror, 0xF, 0xF, false); break;
  }
  return o > v ? o : v;
}

// Wave-wide max, returned in a scalar (uniform) register.
__device__ __forceinline__ uint32_t wave_umax_uniform(uint32_t v) {
  v = dpp_umax(v, 0);
  v = dpp_umax(v, 1);
  v = dpp_umax(v, 2);
  v = dpp_umax(v, 3);  // every lane now holds the max of its 16-lane row
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
  return ab > cd ? ab : cd;
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), lane));
}

// Rank at depth `d` (1-based) of the tuple of node `x` (depth(x) >= d).
__device__ __forceinline__ int rank_at(const BuildLds& s, int x, int d) {
  while (s.depth[x] > d) x = s.parent[x];
  return s.rank[x];
}

// Wave-uniform: is candidate (slot a, rank ca) lexicographically before
// candidate (slot b, rank cb)? Lane i holds element i of each rank tuple.
__device__ bool cand_lex_less(const BuildLds& s, int a, int ca, int b, int cb) {
  const int lane = ddt::lane_id();
  const int da = s.depth[a] + 1, db = s.depth[b] + 1;
  int xa = -1, xb = -1;
  if (lane < da) xa = (lane == da - 1) ? ca : rank_at(s, a, lane + 1);
  if (lane < db) xb = (lane == db - 1) ? cb : rank_at(s, b, lane + 1);
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
  // Per-slot state (slot n = lane + 64 * j).
  uint32_t key[J];   // order key of the candidate's score, 0 = no candidate
  float csc[J];      // candidate score
  int crk[J];        // candidate rank
  float nlp[J];      // log-prob of the following sibling candidate
  float nsc[J];      // the node's own score
  int dep[J];        // the node's depth
#pragma unroll
  for (int j = 0; j < J; ++j) {
    key[j] = 0u;
    csc[j] = 0.f;
    crk[j] = 0;
    nlp[j] = 0.f;
    nsc[j] = 0.f;
    dep[j] = 0;
  }
  // Lane d (< L) holds logp[d][0]: the first child's log-prob at depth d + 1.
  const float row0 = lane < L ? s.lp[lane * K] : 0.f;
  if (lane == 0) {
    csc[0] = s.lp[0];
    key[0] = ddt::f32_key(csc[0]);
    nlp[0] = K > 1 ? s.lp[1] : 0.f;
  }

  for (int b = 1; b <= B; ++b) {
    uint32_t lk = 0u;
    int lj = 0;
    bool ltie = false;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (key[j] > lk) {
        lk = key[j];
        lj = j;
        ltie = false;
      } else if (key[j] == lk && lk != 0u) {
        ltie = true;
      }
    }
    const uint32_t kmax = wave_umax_uniform(lk);
    const uint64_t hit = ddt::ballot(lk == kmax);
    const uint64_t tie = ddt::ballot(lk == kmax && ltie);
    int p;
    if (__popcll(hit) == 1 && tie == 0) {
      const int wl = __ffsll((unsigned long long)hit) - 1;
      p = wl + 64 * __builtin_amdgcn_readlane(lj, wl);
    } else {
      // Several slots share the best score: smallest rank tuple wins.
      p = -1;
      int pc = 0;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        uint64_t m = ddt::ballot(key[j] == kmax);
        while (m) {
          const int l = __ffsll((unsigned long long)m) - 1;
          m &= m - 1;
          const int cand = l + 64 * j;
          const int cc = __builtin_amdgcn_readlane(crk[j], l);
          if (p < 0 || cand_lex_less(s, cand, cc, p, pc)) {
            p = cand;
            pc = cc;
          }
        }
      }
    }
    p = __builtin_amdgcn_readfirstlane(p);
    const int pl = p & 63, pj = p >> 6;

    // Gather slot p's state from its owner lane.
    int c = 0, dp = 0;
    float sc = 0.f, nl = 0.f, ps = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (j == pj) {
        c = __builtin_amdgcn_readlane(crk[j], pl);
        dp = __builtin_amdgcn_readlane(dep[j], pl);
        sc = readlane_f(csc[j], pl);
        nl = readlane_f(nlp[j], pl);
        ps = readlane_f(nsc[j], pl);
      }
    }
    const int dn = dp + 1;
    if (lane == 0) {
      s.parent[b] = (int16_t)p;
      s.rank[b] = (int16_t)c;
      s.depth[b] = (uint8_t)dn;
    }
    // Advance slot p to its next sibling (rank c + 1, log-prob prefetched).
    const int c2 = c + 1;
    float ps2 = 0.f;
    uint32_t pk = 0u;
    if (c2 < K) {
      ps2 = (dp == 0) ? nl : (ps + nl);
      pk = ddt::f32_key(ps2);
    }
    const float nl2 = (c2 + 1 < K) ? s.lp[dp * K + c2 + 1] : 0.f;
    // Open slot b at its first child.
    uint32_t bk = 0u;
    float bs = 0.f;
    if (dn < L) {
      bs = sc + readlane_f(row0, dn);
      bk = ddt::f32_key(bs);
    }
    const float bnl = (dn < L && K > 1) ? s.lp[dn * K + 1] : 0.f;
    const int bl = b & 63, bj = b >> 6;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      if (lane == pl && j == pj) {
        key[j] = pk;
        csc[j] = ps2;
        crk[j] = c2;
        nlp[j] = nl2;
      }
      if (lane == bl && j == bj) {
        key[j] = bk;
        csc[j] = bs;
        crk[j] = 0;
        nlp[j] = bnl;
        nsc[j] = sc;
        dep[j] = dn;
      }
    }
  }
  // Node scores to LDS (the lp table is no longer needed; reuse its space).
  float* score_out = s.lp;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int n = lane + 64 * j;
    if (n <= B) score_out[n] = nsc[j];
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
  }
  __syncthreads();
  if (t < 64) pop_loop<J>(s, L, K, B);
  __syncthreads();

  const int N = B + 1;
  const float* nscore = s.lp;
  for (int n = t; n < N; n += kThreads) {
    const int d = s.depth[n];
    parent_out[n] = s.parent[n];
    depth_out[n] = d;
    tok_out[n] = n == 0 ? *root_token : token[(d - 1) * K + s.rank[n]];
    if (score_out) score_out[n] = nscore[n];
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
