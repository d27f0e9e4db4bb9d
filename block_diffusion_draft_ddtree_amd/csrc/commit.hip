// Commit stage of a round: the greedy accept walk ("DDTree Deep Dive",
// section 6) and the in-place KV-cache compaction of the accepted path
// (section 5).
#include "common.hpp"

namespace {

// At each step the whole wave scans the nodes after `cur` for the
// child whose token equals the target's choice at `cur` (sibling tokens are
// distinct, so at most one matches; the smallest id is taken regardless).
// One wave per request (blockIdx.x).
__global__ __launch_bounds__(64) void walk_kernel(
    const int32_t* __restrict__ parent, const int32_t* __restrict__ tok, int N, int L,
    const int32_t* __restrict__ tgt, int32_t* __restrict__ acc,
    int32_t* __restrict__ n_acc, int32_t* __restrict__ bonus) {
  const int lane = threadIdx.x;
  {
    const int r = blockIdx.x;
    parent += (int64_t)r * N;
    tok += (int64_t)r * N;
    tgt += (int64_t)r * N;
    acc += (int64_t)r * (L + 1);
    n_acc += r;
    bonus += r;
  }
  int cur = 0, a = 0;
  int mine = 0;  // lane i keeps acc[i] (L <= 32 < 64)
  for (int d = 0; d < L; ++d) {
    const int want = tgt[cur];
    int found = -1;
    for (int n0 = cur + 1; n0 < N; n0 += 64) {
      const int n = n0 + lane;
      const bool hit = n < N && parent[n] == cur && tok[n] == want;
      const uint64_t m = ddt::ballot(hit);
      if (m) {
        found = n0 + __ffsll((unsigned long long)m) - 1;
        break;
      }
    }
    found = __builtin_amdgcn_readfirstlane(found);
    if (found < 0) break;
    cur = found;
    ++a;
    if (lane == a) mine = cur;
  }
  if (lane <= L) acc[lane] = lane <= a ? mine : -1;
  if (lane == 0) {
    *n_acc = a;
    *bonus = tgt[cur];
  }
}

// One workgroup per (layer, K/V half, kv-head) slice. Every accepted row is
// staged in LDS before the barrier and written back after it, so a row that
// is both a source (S + acc[k]) and a destination (S + j) is never
// overwritten before it has been read (the LDS store needs the loaded data,
// so every load has completed before any wave passes the barrier).
// blockIdx.y is the request: its cache starts req_stride elements after the
// previous one's, its prefix length is S.v[r], its walk result acc[r], n_acc[r].
__global__ __launch_bounds__(256) void compact_kernel(
    uint16_t* __restrict__ kv, int64_t req_stride, int S_cap, int D, ReqInts S_of, int L,
    const int32_t* __restrict__ acc, const int32_t* __restrict__ n_acc) {
  __shared__ uint4 stage[DDTREE_MAX_L * 128 / 8];
  const int r = blockIdx.y;
  const int S = S_of.v[r];
  acc += (int64_t)r * (L + 1);
  uint16_t* base = kv + (int64_t)r * req_stride + (int64_t)blockIdx.x * S_cap * D;
  const int a = n_acc[r];
  const int cpr = D / 8;  // 16-byte chunks per row
  const int total = a * cpr;
  for (int e = threadIdx.x; e < total; e += 256) {
    const int k = e / cpr + 1, ch = e % cpr;
    stage[e] = *reinterpret_cast<const uint4*>(base + (int64_t)(S + acc[k]) * D + ch * 8);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < total; e += 256) {
    const int k = e / cpr + 1, ch = e % cpr;
    if (acc[k] != k) *reinterpret_cast<uint4*>(base + (int64_t)(S + k) * D + ch * 8) = stage[e];
  }
}

}  // namespace

namespace ddt_host {

int walk_launch(const int32_t* parent, const int32_t* tok, int N, int L, int R,
                const int32_t* tgt, int32_t* acc, int32_t* n_acc, int32_t* bonus,
                hipStream_t stream) {
  hipLaunchKernelGGL(walk_kernel, dim3(R), dim3(64), 0, stream, parent, tok, N, L, tgt, acc,
                     n_acc, bonus);
  return launch_status(hipGetLastError());
}

int compact_launch(uint16_t* kv, int layers, int Hkv, int S_cap, int D, int R, const int* S,
                   int L, const int32_t* acc, const int32_t* n_acc, hipStream_t stream) {
  const int slices = layers * 2 * Hkv;
  ReqInts s_of{};
  for (int r = 0; r < R; ++r) s_of.v[r] = S[r];
  const int64_t req_stride = (int64_t)slices * S_cap * D;
  hipLaunchKernelGGL(compact_kernel, dim3(slices, R), dim3(256), 0, stream, kv, req_stride,
                     S_cap, D, s_of, L, acc, n_acc);
  return launch_status(hipGetLastError());
}

}  // namespace ddt_host
