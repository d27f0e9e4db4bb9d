// ddtree_tree_attn: ancestor-only GQA tree attention of one layer ("DDTree
// Deep Dive", section 4: a node sees the cached prefix, the root, its
// ancestors and itself; section 10: grouped-query attention).
//
// Decomposition. For kv-head g the query rows are rho = n * G + i (node n,
// i-th query head of the group); all N * G rows share the same keys. A
// workgroup owns a tile of query rows (RW waves of 32 rows) and a range of
// keys, and runs 8 / RW key streams side by side: the range is cut into
// superblocks of 32 keys per stream, and stream s computes the 32-key
// block s of every superblock. So a workgroup is 8 waves, two per SIMD:
// while one wave of a SIMD runs its softmax the other keeps the matrix
// core busy. RW = 2 (64-row tiles, 4 streams) below 1024 query rows per
// kv-head, RW = 4 (128-row tiles, 2 streams) from there on, where each K/V
// byte copied into LDS then serves twice the rows and there are tiles
// enough to fill the chip. After the loop the streams' partial results are
// merged through LDS. Blocks before S are dense prefix keys; only blocks
// reaching past S read the ancestor mask.
//
// Splits. The key range [0, S + N) is cut into `splits` runs of superblocks
// so that the grid about fills the chip with one workgroup per CU (LDS
// allows one). Splits > 1 write unnormalised partial outputs with their
// reference maximum and sum (base-2 domain) to the workspace, in the
// accumulator's register layout so that every store and load is 1 KB
// contiguous; a combine kernel merges them.
//
// Grid mapping. Workgroups are dealt to the 8 XCDs round-robin by id, and
// each XCD has its own L2. Ids are decoded so that each XCD receives a
// contiguous run of the (kv-head, split, tile) order: the tiles sharing a
// key range then sit on one XCD, which fetches those K/V rows from HBM once
// and serves the other tiles from its L2.
//
// Data movement. K and V blocks go from global memory straight into LDS
// (buffer loads to LDS, 16 bytes per lane, no registers, bounded by the
// last key), double-buffered: the copies of superblock i + 1 are in flight
// while superblock i is computed, one at a time between products. A
// wave's copy lands 1 KB contiguously (lane l at +16 l), and each lane
// fetches whichever 16-byte chunk belongs at its slot. K and V rows are
// row-major with the chunk index XOR-ed by a function of the row (slot =
// chunk ^ f(row)): for K the 32 rows an operand read touches, for V the 4
// keys x 4 chunks a transposing read touches fall in different banks. The
// XOR only permutes chunks inside aligned groups of four, so every four
// lanes of a copy still fetch one contiguous 64-byte piece (a copy whose
// lanes jump between rows runs at a third of the speed).
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16, wave64). Each wave computes
// S^T = K Q^T for its 32 query columns: A = 32 keys x 16 dims of K (one
// 16-byte LDS read per lane), B = Q^T held in registers for the whole
// kernel. In the 32x32 accumulator, lane (j, h) = (lane & 31, lane >> 5)
// owns query column j and key rows 8*(r/4) + 4*h + r%4 of register r, so
// the online softmax is lane-local except one exchange between the lane
// halves (v_permlane32_swap). Rounded to bf16, those registers are the B
// operand of O^T = V^T P^T when each 16-key step takes keys {4h..4h+3} then
// {8+4h..8+4h+3} on lane half h. The matching V^T A operand comes from V by
// two transposing LDS reads (ds_read_b64_tr_b16): within each 16-lane
// group, lane i receives element i%4 of the 4-element reads of lanes
// 4e + i/4, so lanes point at (key 4h + e, dims 4*(lane%4) +
// 16*((lane/16)%2)) and get 4 keys of one dim.
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <mutex>

#include "common.hpp"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

constexpr int kBK = 32;                       // keys per block (one stream's step)
constexpr int kWaves = 8;                     // waves per workgroup: two per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;
constexpr int kMaxMaskWords = (DDTREE_MAX_B + 1 + 31) / 32;  // words of an ancestor row
// Query rows per kv-head (N * G) from which the tall tile shape is used.
constexpr int kTallRows = 1024;

// Tile shape: RW 32-row query waves x 8 / RW key streams. RW = 2 (64-row
// tiles, 4 streams, 128-key superblocks) for small trees; RW = 4 (128-row
// tiles, 2 streams, 64-key superblocks) from kTallRows rows per kv-head on,
// where each K/V byte copied into LDS then feeds twice the rows.
template <int RW>
struct Shape {
  static_assert(RW == 2 || RW == 4, "row waves");
  static constexpr int kRowWaves = RW;
  static constexpr int kStreams = kWaves / RW;
  static constexpr int kRowsPerTile = 32 * RW;
  static constexpr int kSBK = kBK * kStreams;  // keys per superblock
};

template <int D, int RW = 2>
struct Cfg {
  static constexpr int KS = D / 16;                          // MFMA k-steps for Q.K
  static constexpr int DT = D / 32;                          // 32-wide output tiles of P.V
  static constexpr int NS = D / 8;                           // 16-byte slots per row
  static constexpr int ROWB = 2 * D;                         // bytes per row
  static constexpr int TILEB = kBK * ROWB;                   // bytes per K or V block
  static constexpr int ROWS_PER_COPY = 1024 / ROWB;          // rows per 1 KB wave copy
  static constexpr int COPIES = TILEB / 1024 / RW;           // copies per wave per block
  static constexpr int STAGEB = Shape<RW>::kStreams * TILEB;  // one operand of a superblock
};

// K rows are read 32 at a time at one chunk: spread consecutive rows over
// all bank groups.
template <int D>
__device__ __forceinline__ int fk(int row) {
  return D == 128 ? (row & 15) : ((row >> 1) & 7);
}

// V is read 4 consecutive keys x 4 chunks at a time (per 32 lanes): give
// the 4 keys disjoint sets of 16-byte bank slots.
template <int D>
__device__ __forceinline__ int fv(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 values rounded to fp16 (nearest even), low half first; and back.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const _Float16 x = (_Float16)a, y = (_Float16)b;
  return (uint32_t)__builtin_bit_cast(uint16_t, x) | ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// v_permlane32_swap of a value with itself leaves the low half's values in
// one result and the high half's in the other, on every lane: their max is
// the max over lanes j and j + 32.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// n / d and n mod d for 0 <= n < 2^31, d >= 1 and a quotient below 2^22
// (every use here divides an index by a count it indexes), without the
// integer division routine: the float estimate n * (1 / d) carries a
// relative error below 2^-22 (the reciprocal, the conversion of n and the
// product each round once), so it is within one of the quotient, and one
// comparison of the remainder corrects it.
struct Div {
  int d;
  float rcp;
  __device__ __forceinline__ explicit Div(int d_) : d(d_), rcp(__builtin_amdgcn_rcpf((float)d_)) {}
  __device__ __forceinline__ int quot(int n) const {
    int q = (int)((float)n * rcp);
    const int r = n - q * d;
    q += r < 0 ? -1 : (r >= d ? 1 : 0);
    return q;
  }
  __device__ __forceinline__ int rem(int n, int q) const { return n - q * d; }
};

// Per-lane source offsets of a wave's copies, fixed for the whole kernel:
// copy i of row wave rw fetches rows 4 (rw * COPIES + i) + lane / NS (D =
// 128), each lane the chunk that belongs at its 16-byte slot.
// (fv(row) depends only on the row modulo 4, i.e. on the lane, so the V
// offsets of the copies differ by whole rows.)
template <int D, int RW>
struct CopyLanes {
  uint32_t kb[Cfg<D, RW>::COPIES];  // byte offsets from the block's row 0
  uint32_t vb;                      // V offset of copy 0; copy i adds i rows per copy
};
template <int D, int RW>
__device__ __forceinline__ int copy_row(int rw, int i, int lane) {
  using C = Cfg<D, RW>;
  return (rw * C::COPIES + i) * C::ROWS_PER_COPY + lane / C::NS;
}
template <int D, int RW>
__device__ __forceinline__ CopyLanes<D, RW> copy_lanes(int rw, int lane) {
  using C = Cfg<D, RW>;
  static_assert(C::ROWS_PER_COPY % 4 == 0, "fv is periodic in 4 rows");
  CopyLanes<D, RW> cl;
  const int slot = lane % C::NS;
#pragma unroll
  for (int i = 0; i < C::COPIES; ++i) {
    const int row = copy_row<D, RW>(rw, i, lane);
    cl.kb[i] = (uint32_t)(row * C::ROWB + 16 * (slot ^ fk<D>(row)));
  }
  const int row0 = copy_row<D, RW>(rw, 0, lane);
  cl.vb = (uint32_t)(row0 * C::ROWB + 16 * (slot ^ fv<D>(row0)));
  return cl;
}

// Word 3 of a raw buffer resource (32-bit data format, no swizzle).
constexpr uint32_t kRsrcWord3 = 0x00020000u;

// Buffer resource over the 32-key block of K or V starting at key0 (src:
// the kv-head's row 0), bounded at the last key KT - 1, or empty when the
// block is not wanted. A copy's lanes past the bound are out of range and
// write zeros into LDS, so a block reaching past the last key (or lying
// wholly past it) lands as its real rows followed by zero rows: finite data
// whose scores are masked and whose weights are exactly 0. The fields are
// wave-uniform (scalar registers).
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const uint16_t* src, int key0,
                                                             int KT, bool want) {
  using C = Cfg<D>;
  const int rows = want ? max(0, min(kBK, KT - key0)) : 0;
  const uint64_t a = reinterpret_cast<uint64_t>(rows > 0 ? src + (int64_t)key0 * D : src);
  // Taken through readfirstlane: the compiler cannot always see that these
  // are uniform, and a resource in vector registers costs a loop per copy.
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const int nrec = __builtin_amdgcn_readfirstlane(rows * C::ROWB);
  void* base = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, nrec, kRsrcWord3);
}

// Copy i of this row wave's share of a K or V block into LDS (the RW row
// waves of a stream split a block's copies): 1 KB, lane l to +16 l, each
// lane the chunk that belongs at its slot.
template <int D, int RW, bool IS_V>
__device__ __forceinline__ void copy_part(__amdgpu_buffer_rsrc_t rs, char* dst_lds, int rw,
                                          const CopyLanes<D, RW>& cl, int i) {
  using C = Cfg<D, RW>;
  const uint32_t off = IS_V ? cl.vb + (uint32_t)(i * C::ROWS_PER_COPY * C::ROWB) : cl.kb[i];
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (lds_void_t*)(dst_lds + (rw * C::COPIES + i) * 1024), 16, off, 0, 0, 0);
}

// Rescaling of the running output is skipped while no query column's
// maximum has grown by more than this (log2 units): the weights then stay
// below 2^8, which bf16 and fp32 hold exactly enough, and the result is the
// same softmax because numerator and denominator share the stale maximum.
constexpr float kRescaleSlack = 8.0f;

// Visibility of the 32 keys key0..key0+31 of a block reaching past S, for
// one node: bit t is set iff key key0 + t is visible. Prefix keys are always
// visible; tree key S + m is visible iff bit m of the node's ancestor row is
// set; keys from S + N on do not exist (a block may lie wholly past them).
// mw0, mw1 are the row's words max(key0 - S, 0) / 32 and the next one.
__device__ __forceinline__ uint32_t block_visibility(int key0, int S, int N, uint32_t mw0,
                                                     uint32_t mw1) {
  const int t0 = key0 - S;  // tree index of the block's first key, > -32
  uint32_t vis = t0 >= 0 ? __builtin_amdgcn_alignbit(mw1, mw0, (uint32_t)(t0 & 31))
                         : (mw0 << (-t0)) | ((1u << (-t0)) - 1u);
  const int lim = S + N - key0;  // keys of the block that exist
  if (lim < 32) vis &= lim > 0 ? (1u << lim) - 1u : 0u;
  return vis;
}

// Per-lane offsets of the V^T operand reads. Pointer lane l covers key
// 16 mm + 8 half + 4 h + e (e = (l & 15) >> 2) and dims 32 dt + 16 ((l >> 4)
// & 1) + 4 (l & 3), i.e. chunk 4 dt + c0. Since 16 mm + 8 half + 4 h is a
// multiple of 4, the row's swizzle fv is the lane's own constant fv(e), so
// each dt has a per-lane offset and mm, half add compile-time row offsets.
// The offsets are made opaque so each read is one pointer step from its
// array: the LDS alias analysis follows only a few levels of address
// arithmetic (and the optimiser would split a sum into one level per term);
// a read it cannot attribute to its array has to wait for every copy in
// flight.
template <int D>
struct VLanes {
  int off[Cfg<D>::DT];
};
template <int D>
__device__ __forceinline__ VLanes<D> v_lanes(int lane) {
  using C = Cfg<D>;
  const int h = lane >> 5, e4 = (lane & 15) >> 2;
  const int c0 = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  VLanes<D> vl;
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt) {
    vl.off[dt] = (4 * h + e4) * C::ROWB + 16 * ((4 * dt + c0) ^ fv<D>(e4)) + 8 * (lane & 1);
    asm("" : "+v"(vl.off[dt]));
  }
  return vl;
}

// The softmax weights of one 32-key block as the B operands of its two
// 16-key P.V steps (bf16).
struct PBlock {
  bf16x8 p[2];
};

// V^T operands of one 32-key block: [mm][dt], two transposing reads each.
template <int D>
__device__ __forceinline__ void read_v(const char* Vb, const VLanes<D>& vl,
                                       bf16x8 (&va)[2][Cfg<D>::DT]) {
  using C = Cfg<D>;
  constexpr int kMM = 16 * C::ROWB;   // offset per 16 keys
  constexpr int kHalf = 8 * C::ROWB;  // offset of keys +8
#pragma unroll
  for (int mm = 0; mm < 2; ++mm)
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const char* p0 = Vb + vl.off[dt] + mm * kMM;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p0);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p0 + kHalf));
      va[mm][dt] = __builtin_bit_cast(
          bf16x8, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3],
                                                               hi[0], hi[1], hi[2], hi[3]});
    }
}

__device__ __forceinline__ bf16x8 bf16_ones() {
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
  return ones;
}

// O^T += V^T P^T for one block, and the row sums of its bf16 weights on the
// matrix core (A = all ones): the denominator sums exactly the weights the
// numerator uses.
template <int D>
__device__ __forceinline__ void block_pv(const char* Vb, const VLanes<D>& vl, const PBlock& pb,
                                         f32x16 (&o)[Cfg<D>::DT], f32x16& lsum) {
  using C = Cfg<D>;
  bf16x8 va[2][C::DT];
  read_v<D>(Vb, vl, va);
  const bf16x8 ones = bf16_ones();
#pragma unroll
  for (int mm = 0; mm < 2; ++mm) {
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[mm][dt], pb.p[mm], o[dt], 0, 0, 0);
    lsum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pb.p[mm], lsum, 0, 0, 0);
  }
}

// S^T = K Q^T for this wave's 32 query columns over one 32-key block: one
// chain of products, with the K operand reads kept a few steps ahead and
// the copies kcopy(0 .. COPIES - 1) (of the next block, into the other
// stage) placed between the last products.
template <int D, int RW, class KCopy>
__device__ __forceinline__ f32x16 block_qk(const char* Kb, const bf16x8 (&qf)[Cfg<D>::KS],
                                           int lane, KCopy kcopy) {
  using C = Cfg<D, RW>;
  const int j = lane & 31, h = lane >> 5;
  const char* krow = Kb + j * C::ROWB;
  const int f = fk<D>(j);
  constexpr int AHEAD = C::KS / 2;
  bf16x8 ka[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
    ka[ks] = *reinterpret_cast<const bf16x8*>(krow + 16 * ((2 * ks + h) ^ f));
  f32x16 sacc;
#pragma unroll
  for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks)
    sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], sacc, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < C::COPIES; ++i) kcopy(i);
  // Schedule: AHEAD reads, then alternate one product with one read, then
  // the last products with the copies between them.
  static_assert(C::COPIES <= AHEAD, "one copy per trailing product");
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
  for (int i = 0; i < C::KS - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < C::COPIES) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
  return sacc;
}

// Online softmax of one block's scores (unscaled until the exponent, where
// scale * log2(e) and the reference maximum enter as one fma), fused with
// the P.V products of the previous block when PV: those products do not
// depend on this block's exponentials, so the matrix core works through
// them while the vector ALU computes the exponentials. A rescale (rare:
// lazy, see kRescaleSlack) multiplies the running output and sums before
// the previous block's products are added, so it also scales that block's
// pending weights (they were formed against the old reference maximum).
// For blocks reaching past S, `vis` (block_visibility) masks the scores by
// a wave-uniform branch that touches only the scores.
template <int D, bool PV>
__device__ __forceinline__ void block_softmax_pv(f32x16 sacc, const char* Vprev,
                                                 const VLanes<D>& vl, PBlock& pb,
                                                 f32x16 (&o)[Cfg<D>::DT], float& m_run,
                                                 f32x16& lsum, float c, int lane, bool masked,
                                                 uint32_t vis) {
  using C = Cfg<D>;
  const int h = lane >> 5;
  bf16x8 va[2][C::DT];
  if (PV) read_v<D>(Vprev, vl, va);
  if (masked) {
    const uint32_t vh = vis >> (4 * h);
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (!((vh >> (8 * (r >> 2) + (r & 3))) & 1u)) sacc[r] = -INFINITY;
  }
  float bm = sacc[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) bm = fmaxf(bm, sacc[r]);
  const float bmax = halves_max(bm) * c;  // c > 0: the scaled maximum
  // Lazy rescale: move the reference maximum only when some column needs it.
  const bool grow = bmax > m_run + kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(grow)) {
    const float m_new = fmaxf(m_run, bmax);
    // 0 when only m_run is -inf; 1 for a column that has seen no visible key
    // yet and sees none here either (m_run = m_new = -inf: its output, sum
    // and pending weights are all still 0), where the difference is NaN.
    const float corr = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
    for (int r = 0; r < 16; ++r) lsum[r] *= corr;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= corr;
    if (PV) {
#pragma unroll
      for (int e = 0; e < 16; ++e)
        pb.p[e >> 3][e & 7] = (__bf16)((float)pb.p[e >> 3][e & 7] * corr);
    }
    m_run = m_new;
  }
  __builtin_amdgcn_sched_barrier(0);
  if (PV) {
    const bf16x8 ones = bf16_ones();
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[mm][dt], pb.p[mm], o[dt], 0, 0, 0);
      lsum = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pb.p[mm], lsum, 0, 0, 0);
    }
  }
  // A column that has seen no visible key yet keeps m_run = -inf; use 0 as
  // its reference so that masked weights come out as exp2(-inf) = 0.
  const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    pb.p[r >> 3][r & 7] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[r], c, neg_m));
  if (PV) {
    // Interleave: one product, then a slice of the vector work.
#pragma unroll
    for (int i = 0; i < 2 * C::DT + 2; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 1);
    }
  }
}

// Splits of a request's key range and its first split in the partials,
// from its prefix length and the end of the previous request's workgroups.
template <int RW>
__device__ __forceinline__ int req_splits(int S, int N, int sb_per_split) {
  constexpr int SBK = Shape<RW>::kSBK;
  return ((S + N + SBK - 1) / SBK + sb_per_split - 1) / sb_per_split;
}

// The work of one workgroup: position idx in its request's (kv-head, split,
// tile) order; q, k, v, anc and out already point at the request's slices;
// part_base = the request's first split times Hkv (its partial tiles start
// at part_base * tiles * RW).
template <int D, int RW>
__device__ __forceinline__ void attn_workgroup(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int S, int S_cap, int N, int Hq, int Hkv, float scale_log2,
    const uint32_t* __restrict__ anc, int W, uint16_t* __restrict__ out,
    float* __restrict__ part_o, float* __restrict__ part_ml, int tiles, int splits,
    int part_base, int sb_per_split, int idx) {
  using C = Cfg<D, RW>;
  constexpr int kRowWaves = Shape<RW>::kRowWaves;
  constexpr int kStreams = Shape<RW>::kStreams;
  constexpr int kRowsPerTile = Shape<RW>::kRowsPerTile;
  constexpr int kSBK = Shape<RW>::kSBK;
  // Two stages per operand, as distinct arrays: every read and every copy
  // below names a fixed array, so the compiler can tell that reading one
  // stage never has to wait for the copy in flight into the other. Stream s
  // owns bytes [s * TILEB, (s + 1) * TILEB) of each.
  __shared__ __attribute__((aligned(1024))) char k0[C::STAGEB];
  __shared__ __attribute__((aligned(1024))) char v0[C::STAGEB];
  __shared__ __attribute__((aligned(1024))) char k1[C::STAGEB];
  __shared__ __attribute__((aligned(1024))) char v1[C::STAGEB];
  // Q of the tile: with 4 streams it fits the second K stage (free until
  // step 0 copies into it); with 2 it needs an array of its own.
  constexpr bool kQInK1 = kRowWaves * C::TILEB <= C::STAGEB;
  __shared__ __attribute__((aligned(1024))) char qown[kQInK1 ? 16 : kRowWaves * C::TILEB];
  char* const qs = kQInK1 ? k1 : qown;
  __shared__ float2 mlx[kWaves * 64];
  __shared__ uint32_t mrows[kRowsPerTile * kMaxMaskWords];

  const Div div_tiles(tiles), div_splits(splits);
  const int gs = div_tiles.quot(idx);
  const int tile = div_tiles.rem(idx, gs);
  const int g = div_splits.quot(gs);
  const int split = div_splits.rem(gs, g);

  const Div div_G(Div(Hkv).quot(Hq));
  const int G = div_G.d, R = N * G;
  // The wave index is uniform: keep it (and all that derives from it, such
  // as the LDS destinations of the copies) in scalar registers.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int st = wave / kRowWaves, rw = wave % kRowWaves;
  const int j = lane & 31, h = lane >> 5;
  const int row0 = tile * kRowsPerTile + rw * 32;
  const bool live = row0 < R;  // wave-uniform: the wave has query rows
  const int rho = row0 + j;
  const bool row_ok = rho < R;
  const int rho_n = div_G.quot(rho);
  const int node = row_ok ? rho_n : 0;
  const int hq = g * G + (row_ok ? div_G.rem(rho, rho_n) : 0);

  const int KT = S + N;
  const int NSB = (KT + kSBK - 1) / kSBK;
  const int sb0 = split * sb_per_split;
  const int sb1 = min(NSB, sb0 + sb_per_split);
  // Superblock order: tile t of a split starts at superblock t mod n of the
  // split's n and wraps around. The tiles that share a key range sit on one
  // XCD; in the same order they would all wait on the same lines coming
  // from HBM at every step, in this order they ask for different
  // superblocks at first and later find most lines in the XCD's L2. The
  // online softmax does not depend on the key order.
  const int nsb = sb1 - sb0;
  const int rot = tile - Div(nsb).quot(tile) * nsb;
  auto sb_at = [&](int i) {
    const int r = i + rot;
    return sb0 + (r < nsb ? r : r - nsb);
  };
  const uint16_t* kh = k + (int64_t)g * S_cap * D;
  const uint16_t* vh = v + (int64_t)g * S_cap * D;
  const int soff = st * C::TILEB;

  const CopyLanes<D, RW> cl = copy_lanes<D, RW>(rw, lane);
  // Blocks wholly past the last key are still copied (as zero rows) and
  // computed (every key masked): every wave then runs one straight path,
  // and no stage ever holds data that is not finite.
  const VLanes<D> vl = v_lanes<D>(lane);
  {
    const auto rk = block_rsrc<D>(kh, (sb_at(0) * kStreams + st) * kBK, KT, true);
#pragma unroll
    for (int i = 0; i < C::COPIES; ++i) copy_part<D, RW, false>(rk, k0 + soff, rw, cl, i);
  }
  // Q of the tile goes through LDS too: the 32 rows of row wave rw land in
  // qs laid out like a K block, copied by that row wave's stream waves with
  // whole-row coalesced reads (lanes holding Q^T operands would each touch
  // a different row). Rows past R are clamped to row R - 1: finite data
  // whose results are dropped.
  {
    constexpr int QC = C::TILEB / 1024 / kStreams;  // copies per wave
    char* qdst = qs + rw * C::TILEB;
#pragma unroll
    for (int i = 0; i < QC; ++i) {
      const int copy = st * QC + i;
      const int row = copy * C::ROWS_PER_COPY + lane / C::NS;
      const int rr = min(row0 + row, R - 1);
      const int rn = div_G.quot(rr);
      const int qrow = rn * Hq + g * G + div_G.rem(rr, rn);
      const char* src = reinterpret_cast<const char*>(q + (int64_t)qrow * D) +
                        16 * ((lane % C::NS) ^ fk<D>(row));
      __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(qdst + copy * 1024), 16, 0, 0);
    }
  }
  // Ancestor rows of the tile's query rows (row r: node (tile_row0 + r)
  // / G, clamped to the last row), staged in LDS when the workgroup's key
  // range reaches the tree block, after the copies above are on their way;
  // a masked block then reads its two words from LDS. Only the Wn =
  // ceil(N / 32) words that can hold a node are kept.
  const int Wn = (N + 31) >> 5;
  const int tile_row0 = tile * kRowsPerTile;
  if (sb1 * kSBK > S) {
    const Div div_Wn(Wn);
    for (int i = threadIdx.x; i < kRowsPerTile * Wn; i += kThreads) {
      const int r = div_Wn.quot(i), w = div_Wn.rem(i, r);
      const int rr = min(tile_row0 + r, R - 1);
      mrows[i] = anc[(int64_t)div_G.quot(rr) * W + w];
    }
  }
  // A pruned tree (ddtree_tree_prune) has empty ancestor rows for the nodes
  // it dropped: a tile none of whose nodes keeps its own bit has nothing to
  // compute. The bits load with the prologue's copies and are checked once
  // everything has landed (below).
  uint32_t own = 0u;
  {
    const int n_first = div_G.quot(tile_row0);
    const int n_last = div_G.quot(min(R - 1, tile_row0 + kRowsPerTile - 1));
#pragma unroll
    for (int u = 0; u < kRowsPerTile / 64; ++u) {  // at most kRowsPerTile nodes
      const int n = n_first + 64 * u + lane;
      if (n <= n_last) own |= (anc[(int64_t)n * W + (n >> 5)] >> (n & 31)) & 1u;
    }
  }
  const uint32_t* myrow = mrows + (rw * 32 + j) * Wn;
  auto vis_of = [&](int key0) {
    if (key0 + kBK <= S) return ~0u;
    const int wlo = max(0, key0 - S) >> 5;
    const uint32_t mw0 = wlo < Wn ? myrow[wlo] : 0u;
    const uint32_t mw1 = wlo + 1 < Wn ? myrow[wlo + 1] : 0u;
    return block_visibility(key0, S, N, mw0, mw1);
  };

  f32x16 o[C::DT];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY;
  f32x16 lsum;  // every register holds the running sum of the lane's column
#pragma unroll
  for (int r = 0; r < 16; ++r) lsum[r] = 0.f;

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // Every copy has landed: a tile of pruned nodes only can leave (all its
  // waves see the same bits, so none waits at a later barrier).
  if (!ddt::ballot(own != 0u)) return;
  // Q^T operands of the wave's 32 rows, read like a K operand; then a
  // barrier before step 0 copies into k1.
  bf16x8 qf[C::KS];
  {
    const char* qrow = qs + rw * C::TILEB + j * C::ROWB;
    const int f = fk<D>(j);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ((2 * ks + h) ^ f));
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Software pipeline over superblocks. Step i forms the scores of block i
  // and its softmax weights, and issues the P.V products of block i - 1
  // together with the Q.K products of block i. So the V rows of block i are
  // first read in step i + 1: step i copies K of superblock i + 1 and V of
  // superblock i, each into the stage the step before last finished with
  // (K: i + 1 mod 2; V: i mod 2). The first step (no P.V) and the last P.V
  // are peeled; the loop is unrolled by two so every access names a fixed
  // array.
  PBlock pb;  // weights of the previous block
  auto step = [&](int i, bool first, const char* kc, char* kn, char* vdst, const char* vprev) {
    const int key0 = (sb_at(i) * kStreams + st) * kBK;
    // The copies enter the texture-address unit at about 45 B per clock per
    // CU, and a wave whose copies are queued there cannot issue further;
    // but a copy issued late in the step is still on its way from L2 when
    // the step ends. So V of this superblock goes out at the start of the
    // step, and K of the next one (none after the last) one copy at a time
    // between the last score products. Branch-free: a block not wanted has
    // an empty resource.
    const auto rk = block_rsrc<D>(kh, (sb_at(i + 1) * kStreams + st) * kBK, KT, i + 1 < nsb);
    const auto rv = block_rsrc<D>(vh, key0, KT, true);
#pragma unroll
    for (int c = 0; c < C::COPIES; ++c) copy_part<D, RW, true>(rv, vdst + soff, rw, cl, c);
    auto kcopy = [&](int c) { copy_part<D, RW, false>(rk, kn + soff, rw, cl, c); };
    __builtin_amdgcn_sched_barrier(0);
    const f32x16 sacc = block_qk<D, RW>(kc + soff, qf, lane, kcopy);
    __builtin_amdgcn_sched_barrier(0);
    const bool masked = key0 + kBK > S;
    const uint32_t vis = vis_of(key0);
    if (first)
      block_softmax_pv<D, false>(sacc, vprev + soff, vl, pb, o, m_run, lsum, scale_log2, lane,
                                 masked, vis);
    else
      block_softmax_pv<D, true>(sacc, vprev + soff, vl, pb, o, m_run, lsum, scale_log2, lane,
                                masked, vis);
    // Keep the wait for the copies at the end of the step: the scheduler
    // would otherwise hoist it (and the barrier) above the vector work.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  step(0, true, k0, k1, v0, v1);
#pragma unroll 1
  for (int i = 1; i < nsb; i += 2) {
    step(i, false, k1, k0, v1, v0);
    if (i + 1 < nsb) step(i + 1, false, k0, k1, v0, v1);
  }
  // The last block's P.V: its V went to v0 if the last step was an even
  // number of steps after the first, else to v1.
  block_pv<D>(((nsb - 1) & 1 ? v1 : v0) + soff, vl, pb, o, lsum);
  __syncthreads();

  // Merge the streams. Every wave parks its (reference max, sum) and the
  // fp32 output tiles it does not merge itself in LDS; then the wave of
  // stream s merges the MT 32-dim output tiles [s MT, (s + 1) MT) of its
  // rows over the streams, its own share straight from registers. Wave
  // w = s RW + r parks in stage array w / 2 (k0, v0, k1, v1), at offset
  // (w mod 2) PB. Four streams (MT = 1; with D = 64 streams 2 and 3 merge
  // nothing): a wave's slot holds all DT tiles, its own unused. Two streams
  // (MT = DT / 2): it holds only the DT - MT tiles the other stream merges,
  // so that the eight slots fit the smaller stage arrays.
  constexpr int MT = (C::DT + kStreams - 1) / kStreams;
  constexpr bool kCompact = kStreams == 2;
  constexpr int PB = (kCompact ? C::DT - MT : C::DT) * 4096;
  static_assert(2 * PB <= C::STAGEB, "two waves' parked tiles per stage array");
  auto park_of = [&](int s_, int r_) -> char* {
    const int w = s_ * kRowWaves + r_;
    char* arr = (w >> 1) == 0 ? k0 : (w >> 1) == 1 ? v0 : (w >> 1) == 2 ? k1 : v1;
    return arr + (w & 1) * PB;
  };
  auto pslot = [&](int s_, int d) { return kCompact && d >= s_ * MT ? d - MT : d; };
  const float l_tot = lsum[0];
  {
    float4* ob = reinterpret_cast<float4*>(park_of(st, rw));
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      if (dt >= st * MT && dt < (st + 1) * MT) continue;
      const int ps = pslot(st, dt);
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        ob[(ps * 4 + qd) * 64 + lane] =
            make_float4(o[dt][4 * qd], o[dt][4 * qd + 1], o[dt][4 * qd + 2], o[dt][4 * qd + 3]);
    }
    mlx[wave * 64 + lane] = make_float2(m_run, l_tot);
  }
  __syncthreads();
  if (!live || st * MT >= C::DT) return;
  float ms[kStreams], ls[kStreams];
#pragma unroll
  for (int s = 0; s < kStreams; ++s) {
    const float2 ml = mlx[(s * kRowWaves + rw) * 64 + lane];
    ms[s] = ml.x;
    ls[s] = ml.y;
  }
  float M = ms[0];
#pragma unroll
  for (int s = 1; s < kStreams; ++s) M = fmaxf(M, ms[s]);
  const float Mu = M == -INFINITY ? 0.f : M;
  float L = 0.f, ws_[kStreams];
#pragma unroll
  for (int s = 0; s < kStreams; ++s) {
    ws_[s] = __builtin_amdgcn_exp2f(ms[s] - Mu);
    L += ws_[s] * ls[s];
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int dt = st * MT + mt;
    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int s = 0; s < kStreams; ++s) {
      const float w = ws_[s];
      if (s == st) {
#pragma unroll
        for (int d = 0; d < C::DT; ++d)
          if (d == dt) {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] += w * o[d][r];
          }
        continue;
      }
      const float4* ob = reinterpret_cast<const float4*>(park_of(s, rw));
      const int ps = pslot(s, dt);
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const float4 x = ob[(ps * 4 + qd) * 64 + lane];
        acc[4 * qd] += w * x.x;
        acc[4 * qd + 1] += w * x.y;
        acc[4 * qd + 2] += w * x.z;
        acc[4 * qd + 3] += w * x.w;
      }
    }
    if (!row_ok) continue;
    if (splits == 1) {
      const float inv = 1.0f / L;
      uint16_t* orow = out + ((int64_t)node * Hq + hq) * D;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int d0 = 32 * dt + 8 * qd + 4 * h;
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16_rne(acc[4 * qd] * inv) |
               ((uint32_t)f32_to_bf16_rne(acc[4 * qd + 1] * inv) << 16);
        pk.y = (uint32_t)f32_to_bf16_rne(acc[4 * qd + 2] * inv) |
               ((uint32_t)f32_to_bf16_rne(acc[4 * qd + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + d0) = pk;
      }
    } else {
      // Partial tile wb of this split: the split's output normalised by its
      // own sum, [DT][4][64 lanes] x 4 fp16, plus one fp32 (max, sum) pair
      // per row. Normalised values lie within the V rows' range, so fp16
      // keeps them to 2^-11 relative, well inside the final bf16 rounding;
      // half the bytes of fp32 partials to write here and read back in the
      // combine. Non-temporal stores: the partials are read once, by the
      // combine kernel, and need not sit in L2 (whose dirty lines would
      // otherwise be written back at the end of the kernel).
      const int64_t wb =
          ((int64_t)(part_base + split * Hkv + g) * tiles + tile) * kRowWaves + rw;
      const float inv = L > 0.f ? 1.0f / L : 0.f;  // a split may see no key of a row
      u32x2* po = reinterpret_cast<u32x2*>(part_o) + (wb * C::DT + dt) * 4 * 64;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd)
        __builtin_nontemporal_store(
            u32x2{pack_f16x2(acc[4 * qd] * inv, acc[4 * qd + 1] * inv),
                  pack_f16x2(acc[4 * qd + 2] * inv, acc[4 * qd + 3] * inv)},
            po + qd * 64 + lane);
      if (dt == 0 && h == 0) reinterpret_cast<float2*>(part_ml)[wb * 32 + j] = make_float2(M, L);
    }
  }
}

// Workgroup id -> position in the (request, kv-head, split, tile) order,
// one contiguous run per XCD. Ids past the work exit before any barrier.
__device__ __forceinline__ int xcd_run_index(int per_xcd) {
  return (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
}

// One request: its values are plain arguments.
template <int D, int RW>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void tree_attn_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int S, int S_cap, int N, int Hq, int Hkv, float scale_log2,
    const uint32_t* __restrict__ anc, int W, uint16_t* __restrict__ out,
    float* __restrict__ part_o, float* __restrict__ part_ml, int tiles, int splits,
    int sb_per_split, int wgs, int per_xcd) {
  const int idx = xcd_run_index(per_xcd);
  if (idx >= wgs) return;
  attn_workgroup<D, RW>(q, k, v, S, S_cap, N, Hq, Hkv, scale_log2, anc, W, out, part_o,
                        part_ml, tiles, splits, 0, sb_per_split, idx);
}

// Several requests: prefix lengths and cumulative workgroup ends per
// request; request r's slices start r strides into q, anc, out and
// kv_req_stride elements into k and v.
template <int D, int RW>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void tree_attn_batched_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, int64_t kv_req_stride, ReqInts S_of, ReqInts wg_end,
    int S_cap, int N, int Hq, int Hkv, float scale_log2, const uint32_t* __restrict__ anc, int W,
    uint16_t* __restrict__ out, float* __restrict__ part_o, float* __restrict__ part_ml,
    int tiles, int sb_per_split, int wgs, int per_xcd) {
  const int idx0 = xcd_run_index(per_xcd);
  if (idx0 >= wgs) return;
  int req = 0;  // the first request whose workgroups end past idx0 (uniform)
  while (idx0 >= wg_end.v[req]) ++req;
  const int wg0 = req ? wg_end.v[req - 1] : 0;
  const int S = S_of.v[req];
  const int64_t qo = (int64_t)req * N * Hq * D;
  attn_workgroup<D, RW>(q + qo, k + req * kv_req_stride, v + req * kv_req_stride, S, S_cap, N,
                        Hq, Hkv, scale_log2, anc + (int64_t)req * N * W, W, out + qo, part_o,
                        part_ml, tiles, req_splits<RW>(S, N, sb_per_split), wg0 / tiles,
                        sb_per_split, idx0 - wg0);
}

// Merge the per-split partials. One thread per float4 of a partial tile
// (the same slot in every split), so each load instruction of a wave reads
// 1 KB contiguously; the splits are taken 8 at a time with every load of a
// batch issued before any is used, merged by a running maximum.
template <int D, int RW>
__device__ __forceinline__ void combine_rows(const float* __restrict__ part_o,
                                             const float* __restrict__ part_ml, int splits,
                                             int split_base, int N, int Hq, int Hkv, int tiles,
                                             const uint32_t* __restrict__ anc, int W,
                                             uint16_t* __restrict__ out) {
  constexpr int DT = D / 32;
  constexpr int kRowWaves = Shape<RW>::kRowWaves;
  constexpr int kRowsPerTile = Shape<RW>::kRowsPerTile;
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int lane = t & 63, qd = (t >> 6) & 3;
  const int dt = (t >> 8) % DT;
  const int wbl = t / (256 * DT);  // (kv-head, tile, row wave)
  const int WB = Hkv * tiles * kRowWaves;
  if (wbl >= WB) return;
  const int rw = wbl % kRowWaves;
  const Div div_tiles(tiles), div_G(Div(Hkv).quot(Hq));
  const int g = div_tiles.quot(wbl / kRowWaves);
  const int tile = div_tiles.rem(wbl / kRowWaves, g);
  const int G = div_G.d, R = N * G;
  const int j = lane & 31, h = lane >> 5;
  const int rho = tile * kRowsPerTile + rw * 32 + j;
  if (rho >= R) return;
  // Rows of nodes a pruned tree dropped have no partials (their tile may not
  // have run) and no output. The check's load goes out with the partials'
  // loads and is tested before the store (a dropped row merges whatever the
  // workspace holds and discards it), so it adds no round trip.
  const int node = div_G.quot(rho);
  const uint32_t own_word = anc[(int64_t)node * W + (node >> 5)];
  const uint2* po = reinterpret_cast<const uint2*>(part_o);
  const float2* pml = reinterpret_cast<const float2*>(part_ml);
  float M = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < splits; s0 += 8) {
    float2 ml[8];
    uint2 xh[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t wb = (int64_t)(split_base + min(s0 + u, splits - 1)) * WB + wbl;
      ml[u] = pml[wb * 32 + j];
      xh[u] = po[((wb * DT + dt) * 4 + qd) * 64 + lane];
    }
    float bm = M;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < splits) bm = fmaxf(bm, ml[u].x);
    const float bmu = bm == -INFINITY ? 0.f : bm;
    const float corr = __builtin_amdgcn_exp2f(M - bmu);  // 0 while M = -inf
    L *= corr;
    acc.x *= corr;
    acc.y *= corr;
    acc.z *= corr;
    acc.w *= corr;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (s0 + u < splits) {
        // The split's weight: its sum rescaled to the running maximum.
        const float w = __builtin_amdgcn_exp2f(ml[u].x - bmu) * ml[u].y;
        L += w;
        acc.x += w * f16_lo(xh[u].x);
        acc.y += w * f16_hi(xh[u].x);
        acc.z += w * f16_lo(xh[u].y);
        acc.w += w * f16_hi(xh[u].y);
      }
    }
    M = bm;
  }
  if (!((own_word >> (node & 31)) & 1u)) return;
  const float inv = 1.0f / L;
  const int hq = g * G + div_G.rem(rho, node);
  const int d0 = 32 * dt + 8 * qd + 4 * h;
  uint2 pk;
  pk.x = (uint32_t)f32_to_bf16_rne(acc.x * inv) | ((uint32_t)f32_to_bf16_rne(acc.y * inv) << 16);
  pk.y = (uint32_t)f32_to_bf16_rne(acc.z * inv) | ((uint32_t)f32_to_bf16_rne(acc.w * inv) << 16);
  *reinterpret_cast<uint2*>(out + ((int64_t)node * Hq + hq) * D + d0) = pk;
}

template <int D, int RW>
__global__ __launch_bounds__(256) void tree_attn_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, int splits, int N,
    int Hq, int Hkv, int tiles, const uint32_t* __restrict__ anc, int W,
    uint16_t* __restrict__ out) {
  combine_rows<D, RW>(part_o, part_ml, splits, 0, N, Hq, Hkv, tiles, anc, W, out);
}

// blockIdx.y is the request; one that ran as a single split wrote its
// output directly.
template <int D, int RW>
__global__ __launch_bounds__(256) void tree_attn_batched_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml, ReqInts S_of,
    ReqInts wg_end, int sb_per_split, int N, int Hq, int Hkv, int tiles,
    const uint32_t* __restrict__ anc, int W, uint16_t* __restrict__ out) {
  const int req = blockIdx.y;
  const int splits = req_splits<RW>(S_of.v[req], N, sb_per_split);
  if (splits == 1) return;
  const int split_base = req ? wg_end.v[req - 1] / (Hkv * tiles) : 0;
  combine_rows<D, RW>(part_o, part_ml, splits, split_base, N, Hq, Hkv, tiles,
                      anc + (int64_t)req * N * W, W, out + (int64_t)req * N * Hq * D);
}

// Workgroups resident at once: one per CU (LDS holds one).
constexpr int kSlots = 256;

// The tile shape of a call on the host: row waves, rows per tile, keys per
// superblock and the modelled time of one superblock step (measured: about
// 1.4 us for 128 keys x 64 rows; 64 keys x 128 rows, the same products
// with half the copies, planned at 1.05 us).
struct HostShape {
  int rw, rows, sbk;
  double step_us;
};
inline HostShape host_shape(int N, int Hq, int Hkv) {
  if (N * (Hq / Hkv) >= kTallRows) return {4, Shape<4>::kRowsPerTile, Shape<4>::kSBK, 1.05};
  return {2, Shape<2>::kRowsPerTile, Shape<2>::kSBK, 1.4};
}

// Superblocks of a key range of S + N keys.
inline int n_superblocks(int S, int N, int sbk) { return (S + N + sbk - 1) / sbk; }

// Most splits a request with nsb superblocks may be cut into, when each
// split covers `per_split` workgroups: enough for four waves of workgroups
// over the chip, or one split per 16 superblocks when that is more, never
// more than one per superblock. Non-decreasing in nsb, so a workspace sized
// for a prefix length serves every shorter one.
inline int split_budget(int nsb, int per_split) {
  const int waves4 = (4 * kSlots + per_split - 1) / per_split;
  return std::min(nsb, std::max(waves4, (nsb + 15) / 16));
}

// Launch model constants, measured on the 30B verifier shape: a
// workgroup's fixed work (set-up, merge, write), the partials' HBM rate
// (bytes per microsecond) and the combine launch (the step time is the
// shape's).
constexpr double kWgUs = 4.0, kPartBytesPerUs = 5.0e6, kCombineUs = 3.0;

// Modelled time of the launch with `sbps` superblocks per split. The
// workgroups run in id order; XCD x takes the contiguous id range the kernel
// maps to it, and each of its CUs (slots / 8, one resident workgroup each)
// takes the next workgroup when it frees up. A workgroup lasts its split's
// superblocks times the step time plus kWgUs. Splitting adds the partials'
// round trip through HBM and the combine launch. Returns early (with a
// value at least `cap`) once the bound exceeds cap.
double model_us(int nreq, const int* S, int N, int Hkv, int D, const HostShape& sh, int tiles,
                int rows_pad, int sbps, double cap) {
  const int kSBK = sh.sbk;
  const double kStepUs = sh.step_us;
  const int slots = kSlots;
  const int cus = slots / kXcds;
  int64_t splits_total = 0;
  double work = 0.0, longest = 0.0;
  for (int r = 0; r < nreq; ++r) {
    const int nsb = (S[r] + N + kSBK - 1) / kSBK;
    const int sp = (nsb + sbps - 1) / sbps;
    splits_total += sp;
    work += (double)Hkv * tiles * (nsb * kStepUs + sp * kWgUs);
    longest = std::max(longest, std::min(sbps, nsb) * kStepUs + kWgUs);
  }
  double extra = 0.0;
  if (splits_total > nreq)
    extra = (double)splits_total * Hkv * rows_pad * (2 * D + 8) * 2 / kPartBytesPerUs + kCombineUs;
  const double bound = std::max(work / slots, longest) + extra;
  if (bound >= cap) return bound;
  const int64_t wgs = splits_total * Hkv * tiles;
  const int64_t per_xcd = (wgs + kXcds - 1) / kXcds;
  double worst = 0.0;
  double heap[kSlots / kXcds];  // a min-heap of the XCD's CU free times
  double* const heap_end = heap + cus;
  int r = 0, g = 0, split = 0, tile = 0;  // the workgroup at id 0
  for (int x = 0; x < kXcds; ++x) {
    std::fill(heap, heap_end, 0.0);  // every CU free at time 0
    for (int64_t i = 0; i < per_xcd && x * per_xcd + i < wgs; ++i) {
      const int nsb = (S[r] + N + kSBK - 1) / kSBK;
      const double c = std::min(sbps, nsb - split * sbps) * kStepUs + kWgUs;
      std::pop_heap(heap, heap_end, std::greater<double>());
      heap_end[-1] += c;
      std::push_heap(heap, heap_end, std::greater<double>());
      // Next id: tile fastest, then split, then kv-head, then request.
      if (++tile == tiles) {
        tile = 0;
        if (++split == (nsb + sbps - 1) / sbps) {
          split = 0;
          if (++g == Hkv) {
            g = 0;
            ++r;
          }
        }
      }
    }
    worst = std::max(worst, *std::max_element(heap, heap_end));
    if (worst + extra >= cap) return worst + extra;
  }
  return worst + extra;
}

struct PlanKey {
  int nreq, N, Hq, Hkv, D;
  int S[DDTREE_MAX_REQ];
};

// Superblocks per split with the smallest modelled time; ties keep the
// longer splits. Candidates: every count up to 64 superblocks, beyond that
// the counts that cut the longest request into 1..64 equal splits, keeping
// only those that cut no request into more splits than its split_budget.
// The last choice is kept per thread, so the calls of one round (every
// layer, same prefix lengths) plan once.
int choose_sbps(int nreq, const int* S, int N, int Hq, int Hkv, int D, const HostShape& sh,
                int tiles, int rows_pad) {
  const int kSBK = sh.sbk;
  thread_local PlanKey last{};
  thread_local int last_sbps = 0;
  PlanKey key{};
  key.nreq = nreq;
  key.N = N;
  key.Hq = Hq;
  key.Hkv = Hkv;
  key.D = D;
  for (int r = 0; r < nreq; ++r) key.S[r] = S[r];
  if (last_sbps > 0 && std::memcmp(&key, &last, sizeof(PlanKey)) == 0) return last_sbps;
  int nsb_max = 1;
  for (int r = 0; r < nreq; ++r) nsb_max = std::max(nsb_max, (S[r] + N + kSBK - 1) / kSBK);
  // Shortest split length that keeps every request within its budget.
  int sbps_min = 1;
  for (int r = 0; r < nreq; ++r) {
    const int nsb = n_superblocks(S[r], N, kSBK);
    const int b = split_budget(nsb, Hkv * tiles);
    sbps_min = std::max(sbps_min, (nsb + b - 1) / b);
  }
  // Fixed arrays (no heap allocation on the launch path).
  int cand[64 + 64 + 1];
  int nc = 0;
  for (int c = 1; c <= std::min(nsb_max, 64); ++c) cand[nc++] = c;
  for (int k = 1; k <= 64; ++k) cand[nc++] = (nsb_max + k - 1) / k;
  cand[nc++] = sbps_min;
  for (int i = 0; i < nc; ++i) cand[i] = std::max(cand[i], sbps_min);
  std::sort(cand, cand + nc, std::greater<int>());
  nc = (int)(std::unique(cand, cand + nc) - cand);
  int best = cand[0];
  double best_us = model_us(nreq, S, N, Hkv, D, sh, tiles, rows_pad, best, 1e300);
  for (int i = 1; i < nc; ++i) {
    const double t = model_us(nreq, S, N, Hkv, D, sh, tiles, rows_pad, cand[i], best_us);
    if (t < best_us) {
      best_us = t;
      best = cand[i];
    }
  }
  last = key;
  last_sbps = best;
  return best;
}

}  // namespace

// Split partials of ddtree_tree_attn_noalloc: a device array in the code
// object, one per GPU. Host code never names it except to look up each
// device's copy (the name is only a host-side stand-in there).
static __device__ __align__(256) unsigned char scratch[DDTREE_NOALLOC_SCRATCH_BYTES];

namespace ddt_host {

int attn_static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DDTREE_ERR_HIP;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DDTREE_ERR_HIP;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return DDTREE_OK;
}

AttnPlan attn_plan(int nreq, const int* S, int N, int Hq, int Hkv, int D) {
  AttnPlan p{};
  const int G = Hq / Hkv, R = N * G;
  const HostShape sh = host_shape(N, Hq, Hkv);
  const int kSBK = sh.sbk;
  p.nreq = nreq;
  p.row_waves = sh.rw;
  p.tiles = (R + sh.rows - 1) / sh.rows;
  p.rows_pad = p.tiles * sh.rows;
  const int per_split = Hkv * p.tiles;
  // One superblock count per split for every request, so requests with
  // longer prefixes get proportionally more splits; chosen by simulating
  // the launch (choose_sbps).
  p.sb_per_split = choose_sbps(nreq, S, N, Hq, Hkv, D, sh, p.tiles, p.rows_pad);
  int wg = 0, sp = 0;
  p.any_split = false;
  for (int r = 0; r < DDTREE_MAX_REQ; ++r) {
    if (r < nreq) {
      const int nsb = (S[r] + N + kSBK - 1) / kSBK;
      const int splits = (nsb + p.sb_per_split - 1) / p.sb_per_split;
      p.S.v[r] = S[r];
      p.splits.v[r] = splits;
      p.split_base.v[r] = sp;
      sp += splits;
      wg += per_split * splits;
      p.wg_end.v[r] = wg;
      p.any_split = p.any_split || splits > 1;
    } else {
      p.S.v[r] = 0;
      p.splits.v[r] = 1;
      p.split_base.v[r] = sp;
      p.wg_end.v[r] = 0x7FFFFFFF;
    }
  }
  p.total_splits = sp;
  p.wgs = wg;
  p.per_xcd = (p.wgs + kXcds - 1) / kXcds;
  if (!p.any_split) {
    p.part_o_off = p.part_ml_off = p.bytes = 0;
  } else {
    const size_t rows = (size_t)p.total_splits * Hkv * p.rows_pad;
    p.part_o_off = 0;
    p.part_ml_off = rows * D * sizeof(uint16_t);  // fp16 normalised outputs
    p.bytes = p.part_ml_off + rows * 2 * sizeof(float);
  }
  return p;
}

// The plan cuts request r into at most split_budget(nsb_r) splits and lays
// out partial rows for the sum of its requests' splits, so the sum of the
// budgets bounds it; with no request able to split it needs nothing. Both
// are non-decreasing in every S[r].
size_t attn_workspace_bound(int nreq, const int* S, int N, int Hq, int Hkv, int D) {
  const int G = Hq / Hkv, R = N * G;
  const HostShape sh = host_shape(N, Hq, Hkv);
  const int tiles = (R + sh.rows - 1) / sh.rows;
  size_t splits = 0;
  bool can_split = false;
  for (int r = 0; r < nreq; ++r) {
    const int b = split_budget(n_superblocks(S[r], N, sh.sbk), Hkv * tiles);
    splits += (size_t)b;
    can_split = can_split || b > 1;
  }
  if (!can_split) return 0;
  const size_t rows = splits * Hkv * (size_t)tiles * sh.rows;
  return rows * D * sizeof(uint16_t) + rows * 2 * sizeof(float);
}

// The main and combine launches of a plan with tile shape RW.
template <int D, int RW>
static int attn_launch_shape(const AttnPlan& p, const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, int64_t kv_req_stride, int nreq, int S0,
                             int S_cap, int N, int Hq, int Hkv, float scale_log2,
                             const uint32_t* anc, int W, uint16_t* out, float* po, float* pml,
                             hipStream_t stream) {
  const dim3 grid(kXcds * p.per_xcd);
  if (nreq == 1)
    hipLaunchKernelGGL((tree_attn_kernel<D, RW>), grid, dim3(kThreads), 0, stream, q, k, v, S0,
                       S_cap, N, Hq, Hkv, scale_log2, anc, W, out, po, pml, p.tiles,
                       p.splits.v[0], p.sb_per_split, p.wgs, p.per_xcd);
  else
    hipLaunchKernelGGL((tree_attn_batched_kernel<D, RW>), grid, dim3(kThreads), 0, stream, q, k,
                       v, kv_req_stride, p.S, p.wg_end, S_cap, N, Hq, Hkv, scale_log2, anc, W,
                       out, po, pml, p.tiles, p.sb_per_split, p.wgs, p.per_xcd);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !p.any_split) return launch_status(e);
  const int threads = Hkv * p.tiles * RW * (D / 32) * 4 * 64;
  const dim3 cgrid((threads + 255) / 256, nreq);
  if (nreq == 1)
    hipLaunchKernelGGL((tree_attn_combine_kernel<D, RW>), cgrid, dim3(256), 0, stream, po, pml,
                       p.splits.v[0], N, Hq, Hkv, p.tiles, anc, W, out);
  else
    hipLaunchKernelGGL((tree_attn_batched_combine_kernel<D, RW>), cgrid, dim3(256), 0, stream,
                       po, pml, p.S, p.wg_end, p.sb_per_split, N, Hq, Hkv, p.tiles, anc, W, out);
  return launch_status(hipGetLastError());
}

int attn_launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t kv_req_stride,
                int nreq, const int* S, int S_cap, int N, int Hq, int Hkv, int D, float scale,
                const uint32_t* anc, int W, uint16_t* out, void* ws, hipStream_t stream) {
  const AttnPlan p = attn_plan(nreq, S, N, Hq, Hkv, D);
  float* po = p.any_split ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_o_off) : nullptr;
  float* pml = p.any_split ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.part_ml_off) : nullptr;
  const float scale_log2 = scale * 1.4426950408889634f;
  auto go = [&](auto launch) {
    return launch(p, q, k, v, kv_req_stride, nreq, S[0], S_cap, N, Hq, Hkv, scale_log2, anc, W,
                  out, po, pml, stream);
  };
  if (D == 128)
    return p.row_waves == 4 ? go(attn_launch_shape<128, 4>) : go(attn_launch_shape<128, 2>);
  return p.row_waves == 4 ? go(attn_launch_shape<64, 4>) : go(attn_launch_shape<64, 2>);
}

}  // namespace ddt_host
