// ddtree_budget_select: the node budget that maximises expected tokens per
// unit of round time ("DDTree Deep Dive", section 2, Proposition 1: the
// expected accepted length of a tree under the drafter's factorised
// distribution is the sum of q(u) over its nodes; the autobench
// Qwen3-Coder-30B page: the budget has an optimum where verify cost
// outgrows the acceptance gain, and a cost-aware variant picks it).
//
// Best-first pops come in score order, so the budget-B tree is the first
// B + 1 nodes of one build with the largest budget. One workgroup of 1024
// threads: thread t owns pop t + 1, q = exp(score) in fp64, an inclusive
// fp64 scan over the pops gives E[alpha](B) for every B, and a max-reduce of
// (1 + E[alpha](B)) / (t0 + t1 (B + 1)) over B in [B_min, B_max] (smallest
// B on ties) gives the budget.
#include "common.hpp"

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / ddt::kWave;

struct Cand {
  double obj;
  int b;
};

__device__ __forceinline__ Cand better(Cand a, Cand o) {
  return (o.obj > a.obj || (o.obj == a.obj && o.b < a.b)) ? o : a;
}

__device__ __forceinline__ Cand wave_best(Cand c) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    Cand o{__shfl_xor(c.obj, off, ddt::kWave), __shfl_xor(c.b, off, ddt::kWave)};
    c = better(c, o);
  }
  return c;
}

__global__ __launch_bounds__(kThreads) void budget_kernel(const float* __restrict__ score,
                                                          int B_max, int B_min, double t0,
                                                          double t1, float* __restrict__ expected,
                                                          int32_t* __restrict__ budget) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int n = t + 1;  // the pop this thread owns
  double x = n <= B_max ? exp((double)score[n]) : 0.0;
  // Inclusive scan: waves, then the wave totals.
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double o = __shfl_up(x, off, ddt::kWave);
    if (lane >= off) x += o;
  }
  __shared__ double wsum[kWaves];
  __shared__ Cand wbest[kWaves];
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  double base = 0.0;
  for (int i = 0; i < w; ++i) base += wsum[i];
  const double ea = base + x;  // E[alpha](n)
  if (expected != nullptr) {
    if (t == 0) expected[0] = 0.f;
    if (n <= B_max) expected[n] = (float)ea;
  }
  Cand c{-1.0, 0x7FFFFFFF};  // objectives are > 0, so any real candidate wins
  if (n <= B_max && n >= B_min) c = Cand{(1.0 + ea) / (t0 + t1 * (double)(n + 1)), n};
  if (t == 0 && B_min == 0) c = better(c, Cand{1.0 / (t0 + t1), 0});
  c = wave_best(c);
  if (lane == 0) wbest[w] = c;
  __syncthreads();
  if (t == 0) {
    Cand b = wbest[0];
    for (int i = 1; i < kWaves; ++i) b = better(b, wbest[i]);
    budget[0] = b.b;
  }
}

// Nodes past the budget leave the tree: no parent (no walk reaches them)
// and an empty ancestor row (the attention skips tiles of such rows). One
// thread per mask word.
__global__ __launch_bounds__(256) void prune_kernel(const int32_t* __restrict__ budget, int N,
                                                    int32_t* __restrict__ parent,
                                                    uint32_t* __restrict__ anc, int W) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= N * W) return;
  const int n = i / W;
  if (n <= budget[0]) return;
  anc[i] = 0u;
  if (i % W == 0) parent[n] = -1;
}

}  // namespace

namespace ddt_host {

int prune_launch(const int32_t* budget, int N, int32_t* parent, uint32_t* anc, int W,
                 hipStream_t stream) {
  hipLaunchKernelGGL(prune_kernel, dim3((N * W + 255) / 256), dim3(256), 0, stream, budget, N,
                     parent, anc, W);
  return launch_status(hipGetLastError());
}

int budget_launch(const float* score, int B_max, int B_min, double t0, double t1,
                  float* expected, int32_t* budget, hipStream_t stream) {
  hipLaunchKernelGGL(budget_kernel, dim3(1), dim3(kThreads), 0, stream, score, B_max, B_min, t0,
                     t1, expected, budget);
  return launch_status(hipGetLastError());
}

}  // namespace ddt_host
