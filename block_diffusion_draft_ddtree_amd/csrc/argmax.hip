// ddtree_target_argmax: the verifier's greedy choice after every tree node
// ("DDTree Deep Dive", section 6: the walk follows the child whose token is
// the target's choice, which at temperature 0 is the argmax of the target
// head's logits for that node).
//
// A single streaming pass over the N x V logits (fp32 or bf16), 16-byte
// loads, four in flight per thread. Each row is cut into S contiguous chunks,
// one 256-thread workgroup per chunk, with S chosen so that the whole grid
// holds about eight workgroups per compute unit whatever N is (one row alone
// is 0.3 MB at a 152k vocabulary; a workgroup per row leaves most of the chip
// idle for a 65-node tree).
//
// Each thread keeps its best (order key, token id) packed into one 64-bit
// word, key high and the id's complement low, so that combining two bests is
// a plain unsigned 64-bit max: the larger value (fp32 order, -0 == +0) wins,
// and of equal values the smaller id. A chunk's best goes to its own slot of
// the workspace; a second small kernel (one wave per row) takes the max over
// the row's S slots and writes the token id. The kernel boundary orders the
// two, so no cross-workgroup fence or atomic is needed (a per-row arrival
// counter would need an agent-scope release per workgroup, which writes back
// the L2 and costs far more than the second launch).
#include "common.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int kWavesPerWg = kThreads / 64;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint64_t pack_best(float x, int idx) {
  return ((uint64_t)ddt::f32_key(x) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)idx);
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max(uint64_t b) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = ((uint64_t)(uint32_t)__shfl_xor((int)(b >> 32), off, 64) << 32) |
                       (uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)b, off, 64);
    b = max_u64(b, o);
  }
  return b;
}

__device__ __forceinline__ float elem(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float elem(const uint16_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

// A 16-byte vector's elements, widened to fp32, in index order.
__device__ __forceinline__ void widen(const u32x4& v, float (&x)[4]) {
  x[0] = __uint_as_float(v.x);
  x[1] = __uint_as_float(v.y);
  x[2] = __uint_as_float(v.z);
  x[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void widen(const u32x4& v, float (&x)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

// grid (S, N): blockIdx.x = chunk of the row, blockIdx.y = row.
// part: uint64 [N, S], the chunk bests.
template <class T>
__global__ __launch_bounds__(kThreads) void argmax_part_kernel(const T* __restrict__ logits,
                                                               int64_t row_stride, int V,
                                                               int chunk_vecs,
                                                               uint64_t* __restrict__ part) {
  constexpr int E = 16 / sizeof(T);  // elements per 16-byte vector
  const int s = blockIdx.x, n = blockIdx.y, t = threadIdx.x;
  const T* row = logits + (int64_t)n * row_stride;
  // Elements before the row's first 16-byte boundary, then whole vectors,
  // then the few elements after the last one.
  const int head = (int)min<int64_t>(
      V, ((16 - (reinterpret_cast<uintptr_t>(row) & 15u)) & 15u) / sizeof(T));
  const int nvec = (V - head) / E;
  const int body_end = head + nvec * E;
  uint64_t best = 0u;  // below every real candidate (keys of real values are > 0)
  if (s == 0) {
    if (t < head) best = pack_best(elem(row, t), t);
    if (body_end + t < V) best = max_u64(best, pack_best(elem(row, body_end + t), body_end + t));
  }
  const u32x4* vrow = reinterpret_cast<const u32x4*>(row + head);
  const int c0 = s * chunk_vecs, c1 = min(nvec, c0 + chunk_vecs);
  for (int v0 = c0; v0 < c1; v0 += kThreads * kUnroll) {
    u32x4 raw[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int v = v0 + u * kThreads + t;
      raw[u] = v < c1 ? __builtin_nontemporal_load(vrow + v) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int v = v0 + u * kThreads + t;
      if (v < c1) {
        float x[E];
        widen(raw[u], x);
        // In index order, only a strictly larger key replaces, so the first
        // of equal maxima stays.
        uint32_t bk = 0u;
        int bi = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const uint32_t k = ddt::f32_key(x[e]);
          if (k > bk) {
            bk = k;
            bi = head + v * E + e;
          }
        }
        best = max_u64(best, ((uint64_t)bk << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)bi));
      }
    }
  }
  best = wave_max(best);
  __shared__ uint64_t wbest[kWavesPerWg];
  if ((t & 63) == 0) wbest[t >> 6] = best;
  __syncthreads();
  if (t == 0) {
    uint64_t b = wbest[0];
#pragma unroll
    for (int w = 1; w < kWavesPerWg; ++w) b = max_u64(b, wbest[w]);
    part[(int64_t)n * gridDim.x + s] = b;
  }
}

// One wave per row, four rows per workgroup: the max over the row's S chunk
// bests, turned back into the token id.
__global__ __launch_bounds__(256) void argmax_final_kernel(const uint64_t* __restrict__ part,
                                                           int S, int N,
                                                           int32_t* __restrict__ out) {
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (n >= N) return;
  uint64_t b = 0u;
  for (int s = lane; s < S; s += 64) b = max_u64(b, part[(int64_t)n * S + s]);
  b = wave_max(b);
  if (lane == 0) out[n] = (int32_t)(0xFFFFFFFFu - (uint32_t)b);
}

}  // namespace

namespace ddt_host {

// Chunks per row: about sixteen 256-thread workgroups per compute unit over
// the whole grid, at most 32 per row, each chunk at least two loads per
// thread.
int argmax_splits(int N, int V, int dtype_bytes) {
  const int64_t want = std::min<int64_t>(32, (4096 + N - 1) / N);
  const int64_t most = std::max<int64_t>(1, ((int64_t)V * dtype_bytes / 16) / (kThreads * 2));
  return (int)std::max<int64_t>(1, std::min<int64_t>(want, most));
}

size_t argmax_workspace_bytes(int N, int V, int dtype_bytes) {
  return (size_t)N * argmax_splits(N, V, dtype_bytes) * sizeof(uint64_t);
}

int argmax_launch(const void* logits, int bf16, int64_t row_stride, int N, int V, void* ws,
                  int32_t* out, hipStream_t stream) {
  const int esize = bf16 ? 2 : 4;
  const int S = argmax_splits(N, V, esize);
  // Vectors per chunk from a bound on any row's vector count (a row's head
  // can only shorten its body).
  const int nvec_max = V / (16 / esize);
  const int chunk = std::max(1, (nvec_max + S - 1) / S);
  auto* part = static_cast<uint64_t*>(ws);
  const dim3 grid(S, N);
  if (bf16)
    hipLaunchKernelGGL(argmax_part_kernel<uint16_t>, grid, dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(logits), row_stride, V, chunk, part);
  else
    hipLaunchKernelGGL(argmax_part_kernel<float>, grid, dim3(kThreads), 0, stream,
                       static_cast<const float*>(logits), row_stride, V, chunk, part);
  int st = launch_status(hipGetLastError());
  if (st) return st;
  hipLaunchKernelGGL(argmax_final_kernel, dim3((N + 3) / 4), dim3(256), 0, stream, part, S, N,
                     out);
  return launch_status(hipGetLastError());
}

}  // namespace ddt_host
