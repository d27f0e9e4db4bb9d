// ddtree_tree_attn: ancestor-only GQA tree attention of one layer ("DDTree
// Deep Dive", section 4: a node sees the cached prefix, the root, its
// ancestors and itself; section 10: grouped-query attention).
//
// Decomposition. For kv-head g the query rows are rho = n * G + i (node n,
// i-th query head of the group); all N * G rows share the same keys, so one
// K/V tile staged in LDS feeds 128 query rows (4 waves x 32). The key range
// [0, S + N) (prefix, then the tree block) is cut into 64-key blocks and the
// blocks into `splits` contiguous ranges; grid = (row tiles, Hkv, splits).
// Prefix blocks are dense; only blocks reaching past S read the mask.
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16, wave64). Each wave computes
// S^T = K Q^T for its 32 query columns: A = 32 keys x 16 dims of K (one
// 16-byte LDS read per lane), B = Q^T held in registers for the whole
// kernel. In the 32x32 accumulator, lane (j, h) = (lane & 31, lane >> 5)
// owns query column j and key rows 8*(r/4) + 4*h + r%4 of register r, so
// the whole online softmax is lane-local except one exchange with lane ^ 32.
// Those same registers, rounded to bf16, are exactly the B operand of
// O^T = V^T P^T once the 16 keys of each MFMA step are taken in the order
// {4h..4h+3, 8+4h..8+4h+3} on lane half h; V is written to LDS transposed
// ([d][key]) with that permutation (bits 2 and 3 of the key index swapped)
// so the A operand is again one 16-byte LDS read per lane.
//
// Splits > 1 write unnormalised partial outputs with their running max and
// sum (base-2 domain) to the workspace; a combine kernel merges them.
#include "common.hpp"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBK = 64;        // keys per block
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerTile = 32 * kWaves;
constexpr int kTargetWorkgroups = 512;

template <int D>
struct Cfg {
  static constexpr int KS = D / 16;     // MFMA k-steps for Q.K
  static constexpr int DT = D / 32;     // 32-wide output tiles of P.V
  static constexpr int KROW = D + 8;    // K tile row stride (bf16), padded
  static constexpr int VROW = kBK + 8;  // V^T tile row stride (bf16), padded
  static constexpr int CH = D / 8;      // 16-byte chunks per K/V row
  static constexpr int PER = kBK * CH / kThreads;
};

__device__ __forceinline__ int vt_pos(int r) {
  return (r & ~15) | (r & 3) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ bf16x8 lds_bf16x8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int D>
__global__ __launch_bounds__(kThreads) void tree_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int S, int S_cap, int N, int Hq, int Hkv,
    float scale_log2, const uint32_t* __restrict__ anc, int W,
    uint16_t* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_ml,
    int blocks_per_split, int rows_pad) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBK * C::KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * C::VROW];

  const int tile = blockIdx.x, g = blockIdx.y, split = blockIdx.z;
  const int G = Hq / Hkv, R = N * G;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j = lane & 31, h = lane >> 5;
  const int rho = tile * kRowsPerTile + wave * 32 + j;
  const bool row_ok = rho < R;
  const int node = row_ok ? rho / G : 0;
  const int hq = g * G + (row_ok ? rho % G : 0);

  bf16x8 qf[C::KS];
  {
    const uint16_t* qrow = q + ((int64_t)node * Hq + hq) * D + 8 * h;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      if (row_ok) {
        qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)0.0f;
      }
    }
  }

  f32x16 o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int KT = S + N;
  const int NB = (KT + kBK - 1) / kBK;
  const int b0 = split * blocks_per_split;
  const int b1 = min(NB, b0 + blocks_per_split);
  const uint16_t* kh = k + (int64_t)g * S_cap * D;
  const uint16_t* vh = v + (int64_t)g * S_cap * D;
  const uint32_t* arow = anc + (int64_t)node * W;

  for (int b = b0; b < b1; ++b) {
    const int key0 = b * kBK;
#pragma unroll
    for (int i = 0; i < C::PER; ++i) {
      const int e = tid + kThreads * i;
      const int r = e / C::CH, c = e % C::CH;
      const int key = key0 + r;
      uint4 kc = make_uint4(0u, 0u, 0u, 0u), vc = make_uint4(0u, 0u, 0u, 0u);
      if (key < KT) {
        kc = *reinterpret_cast<const uint4*>(kh + (int64_t)key * D + 8 * c);
        vc = *reinterpret_cast<const uint4*>(vh + (int64_t)key * D + 8 * c);
      }
      *reinterpret_cast<uint4*>(Ks + r * C::KROW + 8 * c) = kc;
      const int pr = vt_pos(r);
      const uint32_t w4[4] = {vc.x, vc.y, vc.z, vc.w};
#pragma unroll
      for (int t2 = 0; t2 < 4; ++t2) {
        Vt[(8 * c + 2 * t2) * C::VROW + pr] = (uint16_t)(w4[t2] & 0xFFFFu);
        Vt[(8 * c + 2 * t2 + 1) * C::VROW + pr] = (uint16_t)(w4[t2] >> 16);
      }
    }
    __syncthreads();

    f32x16 sacc[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 a = lds_bf16x8(Ks + (32 * kt + j) * C::KROW + 16 * ks + 8 * h);
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[kt], 0, 0, 0);
      }
    }

    const bool need_mask = key0 + kBK > S;
    float bmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float sv = sacc[kt][r] * scale_log2;
        if (need_mask) {
          const int kk = key0 + 32 * kt + 8 * (r >> 2) + 4 * h + (r & 3);
          if (kk >= S) {
            const int tn = kk - S;
            const bool vis = row_ok && tn < N && ((arow[tn >> 5] >> (tn & 31)) & 1u);
            if (!vis) sv = -INFINITY;
          }
        }
        sacc[kt][r] = sv;
        bmax = fmaxf(bmax, sv);
      }
    }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
    const float m_new = fmaxf(m_run, bmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float corr = exp2f(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(sacc[kt][r] - m_use);
        sacc[kt][r] = p;
        psum += p;
      }
    l_run = l_run * corr + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= corr;

#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      bf16x8 bp;
#pragma unroll
      for (int e = 0; e < 8; ++e) bp[e] = (__bf16)sacc[mm >> 1][8 * (mm & 1) + e];
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        const bf16x8 a = lds_bf16x8(Vt + (32 * dt + j) * C::VROW + 16 * mm + 8 * h);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bp, o[dt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!row_ok) return;
  if (gridDim.z == 1) {
    const float inv = 1.0f / l_tot;
    uint16_t* orow = out + ((int64_t)node * Hq + hq) * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int d0 = 32 * dt + 8 * qd + 4 * h;
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16_rne(o[dt][4 * qd] * inv) |
               ((uint32_t)f32_to_bf16_rne(o[dt][4 * qd + 1] * inv) << 16);
        pk.y = (uint32_t)f32_to_bf16_rne(o[dt][4 * qd + 2] * inv) |
               ((uint32_t)f32_to_bf16_rne(o[dt][4 * qd + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + d0) = pk;
      }
  } else {
    const int64_t prow = ((int64_t)split * gridDim.y + g) * rows_pad + rho;
    float* po = part_o + prow * D;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int d0 = 32 * dt + 8 * qd + 4 * h;
        *reinterpret_cast<float4*>(po + d0) =
            make_float4(o[dt][4 * qd], o[dt][4 * qd + 1], o[dt][4 * qd + 2], o[dt][4 * qd + 3]);
      }
    if (h == 0) *reinterpret_cast<float2*>(part_ml + prow * 2) = make_float2(m_run, l_tot);
  }
}

// Merge the per-split partials of each query row: 32 threads per row, each
// handling D / 32 consecutive dims (4 at D = 128, 2 at D = 64).
template <int D>
__global__ __launch_bounds__(256) void tree_attn_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, int splits,
    int N, int Hq, int Hkv, int rows_pad, uint16_t* __restrict__ out) {
  constexpr int PD = D / 32;
  const int G = Hq / Hkv, R = N * G;
  const int row = blockIdx.x * 8 + (threadIdx.x >> 5);  // over Hkv * R
  const int sub = threadIdx.x & 31;
  if (row >= Hkv * R) return;
  const int g = row / R, rho = row % R;
  float M = -INFINITY;
  for (int sp = 0; sp < splits; ++sp)
    M = fmaxf(M, part_ml[(((int64_t)sp * Hkv + g) * rows_pad + rho) * 2]);
  float den = 0.f, acc[PD];
#pragma unroll
  for (int i = 0; i < PD; ++i) acc[i] = 0.f;
  for (int sp = 0; sp < splits; ++sp) {
    const int64_t prow = ((int64_t)sp * Hkv + g) * rows_pad + rho;
    const float m = part_ml[prow * 2], l = part_ml[prow * 2 + 1];
    const float wgt = exp2f(m - M);
    den += wgt * l;
    const float* po = part_o + prow * D + PD * sub;
#pragma unroll
    for (int i = 0; i < PD; ++i) acc[i] += wgt * po[i];
  }
  const float inv = 1.0f / den;
  const int node = rho / G, hq = g * G + rho % G;
  uint16_t* orow = out + ((int64_t)node * Hq + hq) * D + PD * sub;
#pragma unroll
  for (int i = 0; i < PD; ++i) orow[i] = f32_to_bf16_rne(acc[i] * inv);
}

}  // namespace

namespace ddt_host {

AttnPlan attn_plan(int N, int Hq, int Hkv, int D, int S) {
  AttnPlan p;
  const int G = Hq / Hkv, R = N * G;
  p.tiles = (R + kRowsPerTile - 1) / kRowsPerTile;
  p.rows_pad = p.tiles * kRowsPerTile;
  const int NB = (S + N + kBK - 1) / kBK;
  int want = (kTargetWorkgroups + p.tiles * Hkv - 1) / (p.tiles * Hkv);
  want = want < 1 ? 1 : (want > NB ? NB : want);
  p.blocks_per_split = (NB + want - 1) / want;
  p.splits = (NB + p.blocks_per_split - 1) / p.blocks_per_split;
  if (p.splits == 1) {
    p.part_o_off = p.part_ml_off = p.bytes = 0;
  } else {
    const size_t rows = (size_t)p.splits * Hkv * p.rows_pad;
    p.part_o_off = 0;
    p.part_ml_off = rows * D * sizeof(float);
    p.bytes = p.part_ml_off + rows * 2 * sizeof(float);
  }
  return p;
}

int attn_launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, int S, int S_cap, int N,
                int Hq, int Hkv, int D, float scale, const uint32_t* anc, int W, uint16_t* out,
                void* ws, hipStream_t stream) {
  const AttnPlan p = attn_plan(N, Hq, Hkv, D, S);
  float* po = p.splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_o_off) : nullptr;
  float* pml = p.splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_ml_off) : nullptr;
  const float scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid(p.tiles, Hkv, p.splits);
  if (D == 128) {
    hipLaunchKernelGGL(tree_attn_kernel<128>, grid, dim3(kThreads), 0, stream, q, k, v, S, S_cap,
                       N, Hq, Hkv, scale_log2, anc, W, out, po, pml, p.blocks_per_split, p.rows_pad);
  } else {
    hipLaunchKernelGGL(tree_attn_kernel<64>, grid, dim3(kThreads), 0, stream, q, k, v, S, S_cap,
                       N, Hq, Hkv, scale_log2, anc, W, out, po, pml, p.blocks_per_split, p.rows_pad);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return launch_status(e);
  const int rows = Hkv * N * (Hq / Hkv);
  const dim3 cgrid((rows + 7) / 8);
  if (D == 128) {
    hipLaunchKernelGGL(tree_attn_combine_kernel<128>, cgrid, dim3(256), 0, stream, po, pml,
                       p.splits, N, Hq, Hkv, p.rows_pad, out);
  } else {
    hipLaunchKernelGGL(tree_attn_combine_kernel<64>, cgrid, dim3(256), 0, stream, po, pml,
                       p.splits, N, Hq, Hkv, p.rows_pad, out);
  }
  return launch_status(hipGetLastError());
}

}  // namespace ddt_host
