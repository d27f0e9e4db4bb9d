// ddtree_tree_attn: ancestor-only GQA tree attention of one layer ("DDTree
// Deep Dive", section 4: a node sees the cached prefix, the root, its
// ancestors and itself; section 10: grouped-query attention).
//
// Decomposition. For kv-head g the query rows are rho = n * G + i (node n,
// i-th query head of the group); all N * G rows share the same keys, so one
// K/V tile staged in LDS feeds 128 query rows (4 waves x 32). The key range
// [0, S + N) (prefix, then the tree block) is cut into 64-key blocks and the
// blocks into `splits` contiguous ranges. Prefix blocks are dense; only
// blocks reaching past S read the mask.
//
// Grid mapping. Workgroups are dealt to the 8 XCDs round-robin by id, and
// each XCD has its own L2. Ids are decoded so that all row tiles of one
// (kv-head, split) land on the same XCD: the K/V range they share is then
// fetched from HBM once and re-read from that XCD's L2.
//
// Data movement. K and V tiles go from global memory straight into LDS
// (global_load_lds, 16 bytes per lane, no registers), double-buffered: the
// copy of block b + 1 is in flight while block b is computed. A wave's copy
// lands 1 KB contiguously (lane l at +16 l), and each lane fetches whichever
// 16-byte chunk belongs at its slot. K rows are row-major with the chunk
// index XOR-ed by the row (slot = chunk ^ fk(row)), so the 32 rows a K
// operand read touches fall in different banks. V is kept chunk-major inside
// groups of 1 KB (4 keys at D = 128, 8 at D = 64): slot = chunk * rows +
// row, so the 8 keys a transposing read touches sit side by side and every
// operand address is a per-lane base plus compile-time offsets.
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16, wave64). Each wave computes
// S^T = K Q^T for its 32 query columns: A = 32 keys x 16 dims of K (one
// 16-byte LDS read per lane), B = Q^T held in registers for the whole
// kernel. In the 32x32 accumulator, lane (j, h) = (lane & 31, lane >> 5)
// owns query column j and key rows 8*(r/4) + 4*h + r%4 of register r, so
// the online softmax is lane-local except one exchange with lane ^ 32.
// Rounded to bf16, those registers are the B operand of O^T = V^T P^T when
// each 16-key step takes keys {4h..4h+3} then {8+4h..8+4h+3} on lane half h.
// The matching V^T A operand comes from row-major V by two transposing LDS
// reads (ds_read_b64_tr_b16): within each 16-lane group, lane i receives
// element i%4 of the 4-element reads of lanes 4e + i/4, so lanes point at
// (key 4h + e, dims 4*(lane%4) + 16*((lane/16)%2)) and get 4 keys of one dim.
//
// Splits > 1 write unnormalised partial outputs with their running max and
// sum (base-2 domain) to the workspace; a combine kernel merges them.
#include <cstdlib>

#include "common.hpp"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

constexpr int kBK = 64;        // keys per block
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerTile = 32 * kWaves;
constexpr int kXcds = 8;

template <int D>
struct Cfg {
  static constexpr int KS = D / 16;              // MFMA k-steps for Q.K
  static constexpr int DT = D / 32;              // 32-wide output tiles of P.V
  static constexpr int NS = D / 8;               // 16-byte slots per row
  static constexpr int ROWB = 2 * D;             // bytes per row
  static constexpr int TILEB = kBK * ROWB;       // bytes per K or V tile
  static constexpr int ROWS_PER_COPY = 1024 / ROWB;         // rows per 1 KB wave copy
  static constexpr int COPIES = TILEB / 1024 / kWaves;      // copies per wave per tile
  static constexpr int VG = ROWS_PER_COPY;                  // keys per chunk-major V group
};

// K rows are read 32 at a time at one chunk: spread consecutive rows over
// all bank groups.
template <int D>
__device__ __forceinline__ int fk(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Copy the 64-key block starting at key0 of K and V into the tile buffers.
// Rows past the last key (KT - 1) are clamped to it: they are real, finite
// data whose scores are masked and whose weights are exactly 0.
template <int D>
__device__ __forceinline__ void copy_block(const uint16_t* kh, const uint16_t* vh, int key0, int KT,
                                           char* kt_lds, char* vt_lds, int wave, int lane) {
  using C = Cfg<D>;
  const int last = KT - 1;
  const int kslot = lane % C::NS;             // K: row-major, XOR-swizzled
  const int vchunk = lane / C::VG;            // V: chunk-major inside a group
  const int vrow = lane % C::VG;
#pragma unroll
  for (int i = 0; i < C::COPIES; ++i) {
    const int copy = wave * C::COPIES + i;
    const int krow = copy * C::ROWS_PER_COPY + lane / C::NS;
    const int kkey = min(key0 + krow, last);
    const int vkey = min(key0 + copy * C::VG + vrow, last);
    const uint16_t* ksrc = kh + (uint32_t)(kkey * D + 8 * (kslot ^ fk<D>(krow)));
    const uint16_t* vsrc = vh + (uint32_t)(vkey * D + 8 * vchunk);
    __builtin_amdgcn_global_load_lds(ksrc, (lds_void_t*)(kt_lds + copy * 1024), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vsrc, (lds_void_t*)(vt_lds + copy * 1024), 16, 0, 0);
  }
}

// Rescaling of the running output is skipped while no query column's
// maximum has grown by more than this (log2 units): the weights then stay
// below 2^8, which bf16 and fp32 hold exactly enough, and the result is the
// same softmax because numerator and denominator share the stale maximum.
constexpr float kRescaleSlack = 8.0f;

// One 64-key block for this wave's 32 query columns: S^T = K Q^T, online
// softmax, O^T += V^T P^T. Blocks reaching past S hold tree keys: there a
// key S + m is visible to the lane's node only if bit m of its ancestor row
// is set (prefix keys are always visible). The mask is applied by a
// wave-uniform branch that touches only the scores, so the output
// accumulators follow a single path through the loop.
template <int D>
__device__ __forceinline__ void block_step(const char* Kb, const char* Vb,
                                           const bf16x8 (&qf)[Cfg<D>::KS],
                                           f32x16 (&o)[Cfg<D>::DT], float& m_run, float& l_run,
                                           float scale_log2, int lane, int key0, int S, int N,
                                           int wlo, uint32_t mw0, uint32_t mw1, uint32_t mw2) {
  using C = Cfg<D>;
  const int j = lane & 31, h = lane >> 5;
  const bool masked = key0 + kBK > S;
  // S^T = K Q^T as two independent accumulator chains (keys 0-31 and
  // 32-63) interleaved step by step, with the K operand reads kept a few
  // steps ahead so LDS latency hides behind the MFMAs.
  f32x16 sacc[2];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[kt][r] = 0.f;
  {
    const char* krow0 = Kb + j * C::ROWB;
    const int f = fk<D>(j);  // the same for rows j and 32 + j
    constexpr int NSTEP = 2 * C::KS;
    constexpr int AHEAD = 4;
    bf16x8 ka[NSTEP];
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
      const int ks = i >> 1, kt = i & 1;
      ka[i] = *reinterpret_cast<const bf16x8*>(krow0 + kt * 32 * C::ROWB + 16 * ((2 * ks + h) ^ f));
    }
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
      const int ks = i >> 1, kt = i & 1;
      sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i], qf[ks], sacc[kt], 0, 0, 0);
    }
    // Schedule: AHEAD reads, then alternate one MFMA with one read.
    __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
    for (int i = 0; i < NSTEP - AHEAD; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[kt][r] *= scale_log2;
  if (masked) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int tn = key0 + 32 * kt + 8 * (r >> 2) + 4 * h + (r & 3) - S;
        const int wi = (tn >> 5) - wlo;
        const uint32_t word = wi == 0 ? mw0 : (wi == 1 ? mw1 : mw2);
        const uint32_t vis = (uint32_t)(tn < 0) | ((uint32_t)(tn < N) & (word >> (tn & 31)));
        sacc[kt][r] = (vis & 1u) ? sacc[kt][r] : -INFINITY;
      }
  }
  float bmax = -INFINITY;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) bmax = fmaxf(bmax, sacc[kt][r]);
  bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
  // Lazy rescale: move the reference maximum only when some column needs it.
  const bool grow = bmax > m_run + kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(grow)) {
    const float m_new = fmaxf(m_run, bmax);
    const float corr = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 when m_run = -inf
    l_run *= corr;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= corr;
    m_run = m_new;
  }
  // A column that has seen no visible key yet keeps m_run = -inf; use 0 as
  // its reference so that masked weights come out as exp2(-inf) = 0.
  const float m_use = m_run == -INFINITY ? 0.f : m_run;
  float psum = 0.f;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(sacc[kt][r] - m_use);
      sacc[kt][r] = p;
      psum += p;
    }
  l_run += psum;

  // V^T operands from two transposing reads per 16 keys. Pointer lane l
  // covers key 16 mm + 8 half + 4 h + e (e = (l & 15) >> 2) and dims
  // 32 dt + 16 ((l >> 4) & 1) + 4 (l & 3); in the chunk-major V layout that
  // is a per-lane base plus offsets fixed at compile time.
  const int e4 = (lane & 15) >> 2;
  const int c0 = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const char* vbase =
      D == 128 ? Vb + h * 1024 + (c0 * 4 + e4) * 16 + 8 * (lane & 1)
               : Vb + (c0 * 8 + 4 * h + e4) * 16 + 8 * (lane & 1);
  constexpr int kMM = D == 128 ? 4096 : 2048;   // offset per 16 keys
  constexpr int kHalf = D == 128 ? 2048 : 1024; // offset of keys +8
  constexpr int kDT = D == 128 ? 256 : 512;     // offset per 32 dims
#pragma unroll
  for (int mm = 0; mm < 4; ++mm) {
    bf16x8 bp;
#pragma unroll
    for (int e = 0; e < 8; ++e) bp[e] = (__bf16)sacc[mm >> 1][8 * (mm & 1) + e];
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const char* p0 = vbase + mm * kMM + dt * kDT;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p0);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p0 + kHalf));
      const bf16x8 a = __builtin_bit_cast(
          bf16x8, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3],
                                                               hi[0], hi[1], hi[2], hi[3]});
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bp, o[dt], 0, 0, 0);
    }
    // At most one 16-key step of V operands in flight (register budget).
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void tree_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int S, int S_cap, int N, int Hq, int Hkv,
    float scale_log2, const uint32_t* __restrict__ anc, int W,
    uint16_t* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_ml,
    int tiles, int splits, int blocks_per_split, int rows_pad, int xcd_map) {
  using C = Cfg<D>;
  // Two buffers per operand, as distinct arrays: every read and every copy
  // below names a fixed array, so the compiler can tell that reading one
  // buffer never has to wait for the copy in flight into the other.
  __shared__ __attribute__((aligned(1024))) char k0[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char v0[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char k1[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char v1[C::TILEB];

  int tile, g, split;
  {
    const int bid = blockIdx.x;
    int grp;
    if (xcd_map) {
      const int local = bid / kXcds;
      grp = (local / tiles) * kXcds + bid % kXcds;
      tile = local % tiles;
    } else {
      grp = bid / tiles;
      tile = bid % tiles;
    }
    g = grp / splits;
    split = grp % splits;
  }
  const int G = Hq / Hkv, R = N * G;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j = lane & 31, h = lane >> 5;
  const int rho = tile * kRowsPerTile + wave * 32 + j;
  const bool row_ok = rho < R;
  const int node = row_ok ? rho / G : 0;
  const int hq = g * G + (row_ok ? rho % G : 0);

  const int KT = S + N;
  const int NB = (KT + kBK - 1) / kBK;
  const int b0 = split * blocks_per_split;
  const int b1 = min(NB, b0 + blocks_per_split);
  const uint16_t* kh = k + (int64_t)g * S_cap * D;
  const uint16_t* vh = v + (int64_t)g * S_cap * D;
  const uint32_t* arow = anc + (int64_t)node * W;

  // Mask words of a block (the at most 3 words of this lane's node that
  // cover its tree keys) are loaded one block ahead, before that block's
  // copy, so they have always arrived when the block is computed and no wait
  // for them can stall on an in-flight copy.
  int wlo_n = 0;
  uint32_t mw0_n = 0u, mw1_n = 0u, mw2_n = 0u;
  auto fetch_mask = [&](int key0) {
    wlo_n = max(0, key0 - S) >> 5;
    mw0_n = mw1_n = mw2_n = 0u;
    if (key0 + kBK > S && row_ok) {
      mw0_n = wlo_n < W ? arow[wlo_n] : 0u;
      mw1_n = wlo_n + 1 < W ? arow[wlo_n + 1] : 0u;
      mw2_n = wlo_n + 2 < W ? arow[wlo_n + 2] : 0u;
    }
  };
  fetch_mask(b0 * kBK);
  copy_block<D>(kh, vh, b0 * kBK, KT, k0, v0, wave, lane);

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

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // One step: compute block b from (kb, vb) while block b + 1 is copied into
  // (kn, vn); the loop below alternates the buffers, unrolled by two.
  auto step = [&](int b, const char* kb, const char* vb, char* kn, char* vn) {
    const int wlo = wlo_n;
    const uint32_t mw0 = mw0_n, mw1 = mw1_n, mw2 = mw2_n;
    if (b + 1 < b1) {
      fetch_mask((b + 1) * kBK);
      copy_block<D>(kh, vh, (b + 1) * kBK, KT, kn, vn, wave, lane);
    }
    block_step<D>(kb, vb, qf, o, m_run, l_run, scale_log2, lane, b * kBK, S, N, wlo, mw0, mw1,
                  mw2);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
#pragma unroll 1
  for (int b = b0; b < b1; b += 2) {
    step(b, k0, v0, k1, v1);
    if (b + 1 < b1) step(b + 1, k1, v1, k0, v0);
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!row_ok) return;
  if (splits == 1) {
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
    const int64_t prow = ((int64_t)split * Hkv + g) * rows_pad + rho;
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
// handling D / 32 consecutive dims. Loads of several splits are issued
// together (splits are taken in batches of 8) so their latencies overlap.
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
  const int64_t stride = (int64_t)Hkv * rows_pad;  // rows between consecutive splits
  const int64_t row0 = (int64_t)g * rows_pad + rho;
  float den = 0.f, acc[PD];
#pragma unroll
  for (int i = 0; i < PD; ++i) acc[i] = 0.f;
  // Splits are taken 8 at a time: every load of a batch is issued before
  // any of them is used, so their latencies overlap.
  float M = -INFINITY;
  for (int s0 = 0; s0 < splits; s0 += 8) {
    float2 ml[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      ml[u] = s0 + u < splits ? *reinterpret_cast<const float2*>(part_ml + (row0 + (s0 + u) * stride) * 2)
                              : make_float2(-INFINITY, 0.f);
#pragma unroll
    for (int u = 0; u < 8; ++u) M = fmaxf(M, ml[u].x);
  }
  for (int s0 = 0; s0 < splits; s0 += 8) {
    float2 ml[8];
    float po[8][PD];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sp = s0 + u;
      const int64_t prow = row0 + (int64_t)(sp < splits ? sp : 0) * stride;
      ml[u] = *reinterpret_cast<const float2*>(part_ml + prow * 2);
#pragma unroll
      for (int i = 0; i < PD; ++i) po[u][i] = part_o[prow * D + PD * sub + i];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (s0 + u < splits) {
        const float wgt = exp2f(ml[u].x - M);
        den += wgt * ml[u].y;
#pragma unroll
        for (int i = 0; i < PD; ++i) acc[i] += wgt * po[u][i];
      }
    }
  }
  const float inv = 1.0f / den;
  const int node = rho / G, hq = g * G + rho % G;
  uint16_t* orow = out + ((int64_t)node * Hq + hq) * D + PD * sub;
#pragma unroll
  for (int i = 0; i < PD; ++i) orow[i] = f32_to_bf16_rne(acc[i] * inv);
}

int target_workgroups() {
  static const int t = [] {
    const char* s = std::getenv("DDTREE_ATTN_TARGET_WG");
    const int v = s ? std::atoi(s) : 0;
    return v > 0 ? v : 256;
  }();
  return t;
}

}  // namespace

namespace ddt_host {

AttnPlan attn_plan(int N, int Hq, int Hkv, int D, int S) {
  (void)D;
  AttnPlan p;
  const int G = Hq / Hkv, R = N * G;
  p.tiles = (R + kRowsPerTile - 1) / kRowsPerTile;
  p.rows_pad = p.tiles * kRowsPerTile;
  const int NB = (S + N + kBK - 1) / kBK;
  const int target = target_workgroups();
  // Pick blocks per split so that the grid is close to the target size,
  // preferring split counts that allow the XCD-aware mapping.
  int best_bps = NB, best_score = 1 << 30;
  for (int bps = 1; bps <= NB; ++bps) {
    const int splits = (NB + bps - 1) / bps;
    const int wgs = Hkv * p.tiles * splits;
    const bool xcd = (Hkv * splits) % kXcds == 0;
    const int score = (wgs > target ? wgs - target : target - wgs) + (xcd ? 0 : target / 4);
    if (score < best_score) {
      best_score = score;
      best_bps = bps;
    }
  }
  p.blocks_per_split = best_bps;
  p.splits = (NB + best_bps - 1) / best_bps;
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
  const int groups = Hkv * p.splits;
  const int xcd_map = groups % kXcds == 0 ? 1 : 0;
  const dim3 grid(groups * p.tiles);
  if (D == 128) {
    hipLaunchKernelGGL(tree_attn_kernel<128>, grid, dim3(kThreads), 0, stream, q, k, v, S, S_cap,
                       N, Hq, Hkv, scale_log2, anc, W, out, po, pml, p.tiles, p.splits,
                       p.blocks_per_split, p.rows_pad, xcd_map);
  } else {
    hipLaunchKernelGGL(tree_attn_kernel<64>, grid, dim3(kThreads), 0, stream, q, k, v, S, S_cap,
                       N, Hq, Hkv, scale_log2, anc, W, out, po, pml, p.tiles, p.splits,
                       p.blocks_per_split, p.rows_pad, xcd_map);
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
