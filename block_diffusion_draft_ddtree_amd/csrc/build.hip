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
// n & 63, register n >> 6 of wave 0, which keeps what a pop needs about it
// in registers: its candidate's order key and fp32 score, the candidate's
// rank and the node's depth (one word), the node's own score, and the
// log-prob of the candidate after the current one (prefetched from LDS).
//
// A pop: each lane takes the max key over its slots; a DPP max inside each
// 16-lane row, chained across rows by the two row broadcasts, leaves the
// wave max in lane 63, and a ballot finds the owner. The owner's state is
// read with one readlane per field, and the two slots that change are
// written by selects on all lanes (no divergent branch). Each pop issues
// two LDS reads for the log-probs its slots will need next and applies
// them at the following pop, after that pop's reduction, so their latency
// is off the serial chain. The new node's (parent, rank, depth) record is
// one LDS word. Exact score ties fall back to a wave-cooperative
// lexicographic comparison of the rank tuples, rebuilt from those records.
//
// Scores follow the fp32 left-to-right sum: a depth-1 candidate is logp[0][r]
// itself, deeper ones fl(score(parent) + logp[d][r]).
#include "common.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxN = DDTREE_MAX_B + 1;

// A node's record in one word: parent + 1 (11 bits), rank (10 bits), depth
// (6 bits). The root is the all-zero word.
__device__ __forceinline__ uint32_t pack_node(int parent, int rank, int depth) {
  return (uint32_t)(parent + 1) | ((uint32_t)rank << 11) | ((uint32_t)depth << 21);
}
__device__ __forceinline__ int node_parent(uint32_t w) { return (int)(w & 2047u) - 1; }
__device__ __forceinline__ int node_rank(uint32_t w) { return (int)((w >> 11) & 1023u); }
__device__ __forceinline__ int node_depth(uint32_t w) { return (int)(w >> 21); }

struct BuildLds {
  float lp[DDTREE_MAX_LK];
  uint32_t node[kMaxN + 64];  // node records; [kMaxN, kMaxN + 64) takes the other lanes' writes
};

// DPP controls (gfx9 encoding).
constexpr int kQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;  // lane i <-> 7 - i within each 8 lanes
constexpr int kRowMirror = 0x140;      // lane i <-> 15 - i within each 16 lanes
constexpr int kRowBcast15 = 0x142;     // lane 15 of each row -> the next row
constexpr int kRowBcast31 = 0x143;     // lane 31 -> rows 2 and 3

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

// Wave-wide max of unsigned keys (0 is the identity), returned in a scalar
// register: a max within each 16-lane row, then the rows are chained
// through the row broadcasts so that lane 63 holds the max of all 64.
__device__ __forceinline__ uint32_t wave_umax_uniform(uint32_t v) {
  v = umax(v, __builtin_amdgcn_update_dpp(0u, v, kQuadXor1, 0xF, 0xF, false));
  v = umax(v, __builtin_amdgcn_update_dpp(0u, v, kQuadXor2, 0xF, 0xF, false));
  v = umax(v, __builtin_amdgcn_update_dpp(0u, v, kRowHalfMirror, 0xF, 0xF, false));
  v = umax(v, __builtin_amdgcn_update_dpp(0u, v, kRowMirror, 0xF, 0xF, false));
  v = umax(v, __builtin_amdgcn_update_dpp(0u, v, kRowBcast15, 0xA, 0xF, false));
  v = umax(v, __builtin_amdgcn_update_dpp(0u, v, kRowBcast31, 0xC, 0xF, false));
  return __builtin_amdgcn_readlane(v, 63);
}

constexpr int kRowShr1 = 0x111;        // lane i <- lane i - n within each row
constexpr int kRowShr2 = 0x112;
constexpr int kRowShr4 = 0x114;
constexpr int kRowShr8 = 0x118;
constexpr int kWaveShr1 = 0x138;       // lane i <- lane i - 1 across the wave

// Inclusive prefix max over lanes (shifts 1, 2, 4, 8 within each row, then
// the row broadcasts across rows).
__device__ __forceinline__ uint32_t wave_incl_umax_scan(uint32_t v) {
  v = umax(v, __builtin_amdgcn_update_dpp(0u, v, kRowShr1, 0xF, 0xF, false));
  v = umax(v, __builtin_amdgcn_update_dpp(0u, v, kRowShr2, 0xF, 0xF, false));
  v = umax(v, __builtin_amdgcn_update_dpp(0u, v, kRowShr4, 0xF, 0xF, false));
  v = umax(v, __builtin_amdgcn_update_dpp(0u, v, kRowShr8, 0xF, 0xF, false));
  v = umax(v, __builtin_amdgcn_update_dpp(0u, v, kRowBcast15, 0xA, 0xF, false));
  return umax(v, __builtin_amdgcn_update_dpp(0u, v, kRowBcast31, 0xC, 0xF, false));
}

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), lane));
}

// Rank at depth `d` (1-based) of the tuple of node `x` (depth(x) >= d).
__device__ __forceinline__ int rank_at(const BuildLds& s, int x, int d) {
  uint32_t w = s.node[x];
  while (node_depth(w) > d) w = s.node[node_parent(w)];
  return node_rank(w);
}

// Wave-uniform: is candidate (slot a, rank ca) lexicographically before
// candidate (slot b, rank cb)? Lane i holds element i of each rank tuple.
__device__ bool cand_lex_less(const BuildLds& s, int a, int ca, int b, int cb) {
  const int lane = ddt::lane_id();
  const int da = node_depth(s.node[a]) + 1, db = node_depth(s.node[b]) + 1;
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

// The serial best-first pops, on wave 0. Every update is a select on all
// lanes (no divergent branch), and the two log-prob prefetches of a pop (the popped slot's
// sibling after next, the new slot's second child) are applied at the next
// pop, after its reduction, so their LDS latency stays off the chain.
template <int J>
__device__ void pop_loop(BuildLds& s, int L, int K, int B) {
  const int lane = ddt::lane_id();
  // Per-slot state (slot n = lane + 64 * j).
  uint32_t key[J];  // order key of the candidate's score, 0 = no candidate
  float csc[J];     // the candidate's score (the key merges -0 and +0)
  uint32_t crd[J];  // candidate rank | node depth << 16
  float nlp[J];     // log-prob of the candidate after the current one
  float nsc[J];     // the node's own score
#pragma unroll
  for (int j = 0; j < J; ++j) {
    key[j] = 0u;
    csc[j] = 0.f;
    crd[j] = 0u;
    nlp[j] = 0.f;
    nsc[j] = 0.f;
  }
  // Lane d (< L) holds logp[d][0]: the first child's log-prob at depth d + 1.
  const float row0 = lane < L ? s.lp[lane * K] : 0.f;
  // Root run. The first pops take the root's children in rank order for as
  // long as each beats every first child opened before it (the only other
  // candidates): exactly what the serial pops below would do, a tie
  // included (it stops the run and the loop resolves it). A wave handles 63
  // ranks at once: lane i holds rank c + i, a prefix max over the lanes
  // gives the best child opened before it, and the first lane that fails
  // ends the run. Nodes are numbered in rank order, as the pops number them.
  int b = 1, c = 0;
  {
    uint32_t M = 0u;  // best first-child key opened so far
    const float lc = L > 1 ? readlane_f(row0, 1) : 0.f;
    const float nl1 = L > 1 && K > 1 ? s.lp[K + 1] : 0.f;
    while (b <= B && c < K) {
      const int rcap = min(min(K - c, B - b + 1), 63);
      const float si = s.lp[min(c + lane, K - 1)];  // score of rank c + lane
      const uint32_t ki = ddt::f32_key(si);
      const float ci = si + lc;                     // its first child's score
      const uint32_t ui = L > 1 ? ddt::f32_key(ci) : 0u;
      const uint32_t incl = umax(M, wave_incl_umax_scan(ui));
      const uint32_t excl = umax(M, __builtin_amdgcn_update_dpp(0u, incl, kWaveShr1, 0xF, 0xF, false));
      const bool ok = lane < rcap && ki > (lane == 0 ? M : excl);
      const uint64_t fail = ddt::ballot(!ok);  // never empty: lane rcap fails
      const int R = __ffsll((unsigned long long)fail) - 1;
      if (R == 0) break;
      s.node[lane < R ? b + lane : kMaxN + lane] = pack_node(0, c + lane, 1);
      // Run element i goes to the lane of slot b + i.
      const int from = ((lane - b) & 63) * 4;
      const uint32_t km = (uint32_t)__builtin_amdgcn_ds_bpermute(from, (int)ui);
      const float cm = __int_as_float(__builtin_amdgcn_ds_bpermute(from, __float_as_int(ci)));
      const float sm = __int_as_float(__builtin_amdgcn_ds_bpermute(from, __float_as_int(si)));
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int n = lane + 64 * j;
        const bool inr = n >= b && n < b + R;
        key[j] = inr ? km : key[j];
        csc[j] = inr ? cm : csc[j];
        crd[j] = inr ? (1u << 16) : crd[j];
        nsc[j] = inr ? sm : nsc[j];
        nlp[j] = inr ? nl1 : nlp[j];
      }
      M = __builtin_amdgcn_readlane(incl, R - 1);
      b += R;
      c += R;
      if (R < rcap) break;
    }
  }
  // Prefetches of the previous pop, not yet applied (lane -1: none).
  int pf_pl = -1, pf_pj = 0, pf_bl = -1, pf_bj = 0;
  float pf_pv = 0.f, pf_bv = 0.f;
  // The root slot's candidate is now rank c.
  if (lane == 0) {
    csc[0] = c < K ? s.lp[c] : 0.f;
    key[0] = c < K ? ddt::f32_key(csc[0]) : 0u;
    crd[0] = (uint32_t)c;
    nlp[0] = c + 1 < K ? s.lp[c + 1] : 0.f;
  }
  for (; b <= B; ++b) {
    uint32_t lk = key[0];
    int lj = 0;
    bool ltie = false;
#pragma unroll
    for (int j = 1; j < J; ++j) {
      ltie = key[j] == lk ? (lk != 0u) : (key[j] > lk ? false : ltie);
      lj = key[j] > lk ? j : lj;
      lk = umax(lk, key[j]);
    }
    const uint32_t kmax = wave_umax_uniform(lk);
#pragma unroll
    for (int j = 0; j < J; ++j) {
      nlp[j] = (lane == pf_pl && j == pf_pj) ? pf_pv : nlp[j];
      nlp[j] = (lane == pf_bl && j == pf_bj) ? pf_bv : nlp[j];
    }
    const uint64_t hit = ddt::ballot(lk == kmax);
    const uint64_t tie = ddt::ballot(lk == kmax && ltie);
    int pl, pj;
    if (__popcll(hit) == 1 && tie == 0) {
      pl = __ffsll((unsigned long long)hit) - 1;
      pj = __builtin_amdgcn_readlane(lj, pl);
    } else {
      // Several slots share the best score: smallest rank tuple wins.
      int p = -1, pc = 0;
#pragma unroll
      for (int j = 0; j < J; ++j) {
        uint64_t m = ddt::ballot(key[j] == kmax);
        while (m) {
          const int l = __ffsll((unsigned long long)m) - 1;
          m &= m - 1;
          const int cand = l + 64 * j;
          const int cc = (int)(__builtin_amdgcn_readlane(crd[j], l) & 0xFFFFu);
          if (p < 0 || cand_lex_less(s, cand, cc, p, pc)) {
            p = cand;
            pc = cc;
          }
        }
      }
      p = __builtin_amdgcn_readfirstlane(p);
      pl = p & 63;
      pj = p >> 6;
    }
    // Gather slot p's state from its owner lane.
    uint32_t cd = crd[0];
    float nl = nlp[0], ps = nsc[0], sc = csc[0];
#pragma unroll
    for (int j = 1; j < J; ++j) {
      cd = pj == j ? crd[j] : cd;
      nl = pj == j ? nlp[j] : nl;
      ps = pj == j ? nsc[j] : ps;
      sc = pj == j ? csc[j] : sc;
    }
    cd = __builtin_amdgcn_readlane(cd, pl);
    nl = readlane_f(nl, pl);
    ps = readlane_f(ps, pl);
    sc = readlane_f(sc, pl);  // the popped candidate's score
    const int c = (int)(cd & 0xFFFFu), dp = (int)(cd >> 16), dn = dp + 1;
    const int p = pl + 64 * pj;
    // Node b = (parent p, rank c, depth dn); lane 0 writes the record, the
    // other lanes a spare word each.
    s.node[lane == 0 ? b : kMaxN + lane] = pack_node(p, c, dn);
    // Slot p advances to its next sibling (rank c + 1).
    const int c2 = c + 1;
    uint32_t pk = 0u;
    float ps2 = 0.f;
    if (c2 < K) {
      ps2 = dp == 0 ? nl : ps + nl;
      pk = ddt::f32_key(ps2);
    }
    const float nl2 = c2 + 1 < K ? s.lp[dp * K + c2 + 1] : 0.f;
    // Slot b opens at its first child (rank 0 at depth dn + 1).
    uint32_t bk = 0u;
    float bs = 0.f;
    if (dn < L) {
      bs = sc + readlane_f(row0, dn);
      bk = ddt::f32_key(bs);
    }
    const float bnl = dn < L && K > 1 ? s.lp[dn * K + 1] : 0.f;
    const int bl = b & 63, bj = b >> 6;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const bool isp = lane == pl && j == pj, isb = lane == bl && j == bj;
      key[j] = isb ? bk : (isp ? pk : key[j]);
      csc[j] = isb ? bs : (isp ? ps2 : csc[j]);
      crd[j] = isb ? ((uint32_t)dn << 16) : (isp ? ((uint32_t)c2 | ((uint32_t)dp << 16)) : crd[j]);
      nsc[j] = isb ? sc : nsc[j];
    }
    pf_pl = pl;
    pf_pj = pj;
    pf_pv = nl2;
    pf_bl = bl;
    pf_bj = bj;
    pf_bv = bnl;
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
  // One workgroup per request: request r's table, root and outputs.
  {
    const int r = blockIdx.x;
    const int N = B + 1;
    logp += (int64_t)r * LK;
    token += (int64_t)r * LK;
    root_token += r;
    parent_out += (int64_t)r * N;
    depth_out += (int64_t)r * N;
    tok_out += (int64_t)r * N;
    if (score_out) score_out += (int64_t)r * N;
    anc += (int64_t)r * N * W;
  }
  for (int i = t; i < LK; i += kThreads) s.lp[i] = logp[i];
  if (t == 0) s.node[0] = 0u;  // the root
  __syncthreads();
  if (t < 64) pop_loop<J>(s, L, K, B);
  __syncthreads();

  const int N = B + 1;
  const float* nscore = s.lp;
  for (int n = t; n < N; n += kThreads) {
    const uint32_t rec = s.node[n];
    const int d = node_depth(rec);
    parent_out[n] = node_parent(rec);
    depth_out[n] = d;
    tok_out[n] = n == 0 ? *root_token : token[(d - 1) * K + node_rank(rec)];
    if (score_out) score_out[n] = nscore[n];
    // Ancestor-or-self row, written from the high word down.
    uint32_t* row = anc + (int64_t)n * W;
    int wcur = W - 1;
    const int wn = n >> 5;
    for (; wcur > wn; --wcur) row[wcur] = 0u;
    uint32_t acc = 0u;
    for (int j = n; j != -1; j = node_parent(s.node[j])) {
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

int build_launch(const float* logp, const int32_t* token, int L, int K, int B, int R,
                 const int32_t* root_token, int32_t* parent, int32_t* depth,
                 int32_t* node_token, float* score, uint32_t* anc, int W,
                 hipStream_t stream) {
  const int N = B + 1;
#define DDT_BUILD(JJ)                                                              \
  hipLaunchKernelGGL(build_kernel<JJ>, dim3(R), dim3(kThreads), 0, stream, logp,   \
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
