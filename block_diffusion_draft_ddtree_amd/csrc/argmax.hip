// ddtree_target_argmax / ddtree_target_sample: the verifier's choice after
// every tree node ("DDTree Deep Dive", section 6: the walk follows the child
// whose token is the target's choice -- the argmax of the target head's
// logits for that node when greedy, a draw from the target's distribution
// at temperature > 0, which keeps the output distributed as the target's).
//
// A single streaming pass over the N x V logits (fp32 or bf16), 16-byte
// loads, four in flight per thread. Each row is cut into S contiguous chunks,
// one 256-thread workgroup per chunk, with S chosen so that the whole grid
// holds about sixteen workgroups per compute unit whatever N is (one row
// alone is 0.3 MB at a 152k vocabulary; a workgroup per row leaves most of
// the chip idle for a 65-node tree).
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
//
// Sampling is the Gumbel-max draw: the argmax over v of x_v / T - ln(-ln u_v)
// with one uniform u_v per (node, token). Here it is taken in base 2, as
// x_v * (log2(e) / T) - log2(-log2 u_v), which differs from the natural-log
// key by a positive factor and a constant, so it has the same argmax. The
// uniforms come from Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC 2011): key (seed low, seed high),
// counter (v >> 2, n, offset low, offset high), word v & 3, and
// u = ((word >> 9) + 0.5) * 2^-23, exact in fp32 and inside (0, 1).
#include "common.hpp"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int kWavesPerWg = kThreads / 64;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// ---- temperature > 0 -------------------------------------------------------

struct SampleArgs {
  float c;              // log2(e) / T
  uint32_t k0, k1;      // Philox key: seed low, seed high
  uint32_t off0, off1;  // counter words 2 and 3: offset low, offset high
};

constexpr uint32_t kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kPhiloxW0 = 0x9E3779B9u, kPhiloxW1 = 0xBB67AE85u;

// Philox4x32-10 on the counter (g, n, off0, off1); the four output words.
__device__ __forceinline__ void philox(uint32_t g, uint32_t n, const SampleArgs& a,
                                       uint32_t (&w)[4]) {
  uint32_t c0 = g, c1 = n, c2 = a.off0, c3 = a.off1, k0 = a.k0, k1 = a.k1;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)kPhiloxM0 * c0;
    const uint64_t p1 = (uint64_t)kPhiloxM1 * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += kPhiloxW0;
    k1 += kPhiloxW1;
  }
  w[0] = c0;
  w[1] = c1;
  w[2] = c2;
  w[3] = c3;
}

// The base-2 Gumbel key of logit x drawn with Philox word `word`.
__device__ __forceinline__ float gumbel_key(float x, uint32_t word, float c) {
  // (word >> 9) * 2^-23 + 2^-24 = (2 (word >> 9) + 1) * 2^-24: exact.
  const float u = __builtin_fmaf((float)(word >> 9), 0x1p-23f, 0x1p-24f);
  const float t = -__builtin_amdgcn_logf(u);  // -log2 u, in (0, 24]
  return __builtin_fmaf(x, c, -__builtin_amdgcn_logf(t));
}

// The key of token `idx` alone (row heads and tails).
__device__ __forceinline__ float sample_key_at(float x, int idx, uint32_t n, const SampleArgs& a) {
  uint32_t w[4];
  philox((uint32_t)idx >> 2, n, a, w);
  const uint32_t j = (uint32_t)idx & 3u;
  const uint32_t word = j == 0 ? w[0] : j == 1 ? w[1] : j == 2 ? w[2] : w[3];
  return gumbel_key(x, word, a.c);
}

// The largest value of the E elements of the vector whose first element is
// token i0 (the logit, or its Gumbel key when sampling) and the position of
// its first occurrence. i0 % 4 == SH, fixed per row, so each row runs one
// instantiation. Values are compared as floats: no NaN reaches here, -0 and
// +0 compare equal (as their order keys do), and only a strictly larger
// value replaces, so the first of equal maxima stays.
template <int E, bool kSample, int SH>
__device__ __forceinline__ void vector_best(const float (&x)[E], int i0, uint32_t n,
                                            const SampleArgs& a, float& bz, int& be) {
  float z[E];
  if constexpr (!kSample) {
#pragma unroll
    for (int e = 0; e < E; ++e) z[e] = x[e];
  } else {
    // Words of the Philox blocks that cover tokens i0 - SH ... i0 + E - 1.
    constexpr int kBlocks = E / 4 + (SH != 0 ? 1 : 0);
    uint32_t w[4 * kBlocks];
    const uint32_t g0 = (uint32_t)i0 >> 2;
#pragma unroll
    for (int j = 0; j < kBlocks; ++j) {
      uint32_t b[4];
      philox(g0 + j, n, a, b);
#pragma unroll
      for (int q = 0; q < 4; ++q) w[4 * j + q] = b[q];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) z[e] = gumbel_key(x[e], w[SH + e], a.c);
  }
  bz = z[0];
  be = 0;
#pragma unroll
  for (int e = 1; e < E; ++e) {
    if (z[e] > bz) {
      bz = z[e];
      be = e;
    }
  }
}

// The best (key, id) over this thread's vectors of chunk [c0, c1).
template <class T, bool kSample, int SH>
__device__ __forceinline__ uint64_t chunk_best(const T* row, int head, int c0, int c1, uint32_t n,
                                               const SampleArgs& a, int t) {
  constexpr int E = 16 / sizeof(T);  // elements per 16-byte vector
  const u32x4* vrow = reinterpret_cast<const u32x4*>(row + head);
  uint64_t best = 0u;
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
        float bz;
        int be;
        vector_best<E, kSample, SH>(x, head + v * E, n, a, bz, be);
        const uint32_t bi = (uint32_t)(head + v * E + be);
        best = max_u64(best, ((uint64_t)ddt::f32_key(bz) << 32) | (uint64_t)(0xFFFFFFFFu - bi));
      }
    }
  }
  return best;
}

// grid (S, N): blockIdx.x = chunk of the row, blockIdx.y = row.
// part: uint64 [N, S], the chunk bests.
template <class T, bool kSample>
__global__ __launch_bounds__(kThreads) void argmax_part_kernel(const T* __restrict__ logits,
                                                               int64_t row_stride, int V,
                                                               int chunk_vecs, SampleArgs a,
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
    auto one = [&](int i) {
      const float x = elem(row, i);
      const float key = kSample ? sample_key_at(x, i, (uint32_t)n, a) : x;
      return ((uint64_t)ddt::f32_key(key) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
    };
    if (t < head) best = one(t);
    if (body_end + t < V) best = max_u64(best, one(body_end + t));
  }
  const int c0 = s * chunk_vecs, c1 = min(nvec, c0 + chunk_vecs);
  if constexpr (kSample) {
    // Vector starts are head + v * E with E a multiple of 4: one residue per row.
    switch (head & 3) {
      case 0: best = max_u64(best, chunk_best<T, true, 0>(row, head, c0, c1, n, a, t)); break;
      case 1: best = max_u64(best, chunk_best<T, true, 1>(row, head, c0, c1, n, a, t)); break;
      case 2: best = max_u64(best, chunk_best<T, true, 2>(row, head, c0, c1, n, a, t)); break;
      default: best = max_u64(best, chunk_best<T, true, 3>(row, head, c0, c1, n, a, t)); break;
    }
  } else {
    best = max_u64(best, chunk_best<T, false, 0>(row, head, c0, c1, n, a, t));
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

static int choice_launch(const void* logits, int bf16, int64_t row_stride, int N, int V,
                         const SampleArgs* sample, void* ws, int32_t* out, hipStream_t stream) {
  const int esize = bf16 ? 2 : 4;
  const int S = argmax_splits(N, V, esize);
  // Vectors per chunk from a bound on any row's vector count (a row's head
  // can only shorten its body).
  const int nvec_max = V / (16 / esize);
  const int chunk = std::max(1, (nvec_max + S - 1) / S);
  auto* part = static_cast<uint64_t*>(ws);
  const SampleArgs a = sample ? *sample : SampleArgs{0.f, 0u, 0u, 0u, 0u};
  const dim3 grid(S, N);
  if (bf16 && sample)
    hipLaunchKernelGGL((argmax_part_kernel<uint16_t, true>), grid, dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(logits), row_stride, V, chunk, a, part);
  else if (bf16)
    hipLaunchKernelGGL((argmax_part_kernel<uint16_t, false>), grid, dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(logits), row_stride, V, chunk, a, part);
  else if (sample)
    hipLaunchKernelGGL((argmax_part_kernel<float, true>), grid, dim3(kThreads), 0, stream,
                       static_cast<const float*>(logits), row_stride, V, chunk, a, part);
  else
    hipLaunchKernelGGL((argmax_part_kernel<float, false>), grid, dim3(kThreads), 0, stream,
                       static_cast<const float*>(logits), row_stride, V, chunk, a, part);
  int st = launch_status(hipGetLastError());
  if (st) return st;
  hipLaunchKernelGGL(argmax_final_kernel, dim3((N + 3) / 4), dim3(256), 0, stream, part, S, N,
                     out);
  return launch_status(hipGetLastError());
}

int argmax_launch(const void* logits, int bf16, int64_t row_stride, int N, int V, void* ws,
                  int32_t* out, hipStream_t stream) {
  return choice_launch(logits, bf16, row_stride, N, V, nullptr, ws, out, stream);
}

int sample_launch(const void* logits, int bf16, int64_t row_stride, int N, int V, float log2e_over_t,
                  uint64_t seed, uint64_t offset, void* ws, int32_t* out, hipStream_t stream) {
  const SampleArgs a{log2e_over_t, (uint32_t)seed, (uint32_t)(seed >> 32), (uint32_t)offset,
                     (uint32_t)(offset >> 32)};
  return choice_launch(logits, bf16, row_stride, N, V, &a, ws, out, stream);
}

}  // namespace ddt_host
