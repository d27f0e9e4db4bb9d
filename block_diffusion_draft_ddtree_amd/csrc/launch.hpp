// Host-side launchers of libddtree's kernels (internal; one per .hip file).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ddtree.h"

// One int per request, passed by value in the kernel arguments.
struct ReqInts {
  int v[DDTREE_MAX_REQ];
};

namespace ddt_host {

int launch_status(hipError_t e);

// ddtree_topk: chunk kernel + merge kernel; workspace carve-up.
struct TopkPlan {
  int C, cap, idx_passes, q;
  size_t stats_off, bounds_off, counts_off, candx_off, candi_off, bytes;
};
TopkPlan topk_plan(int L, int V, int K);
int topk_launch(const float* logits, int64_t stride, int L, int V, int K, float* logp,
                int32_t* token, void* ws, hipStream_t stream);

int build_launch(const float* logp, const int32_t* token, int L, int K, int B, int R,
                 const int32_t* root_token, int32_t* parent, int32_t* depth,
                 int32_t* node_token, float* score, uint32_t* anc, int W, hipStream_t stream);

// ddtree_tree_attn: grid shape and split-partial workspace, for nreq
// requests of N nodes each with their own prefix lengths.
struct AttnPlan {
  int nreq;
  int row_waves;          // tile shape: 2 (64-row tiles, 128-key superblocks) or 4 (128, 64)
  int tiles, rows_pad;    // query tiles per kv-head, and their rows
  int sb_per_split;       // superblocks per split, every request
  ReqInts S, splits;      // per request: prefix length, splits of its key range
  ReqInts wg_end;         // per request: end of its workgroup range
  ReqInts split_base;     // per request: its first split in the partials
  int total_splits;
  bool any_split;         // some request runs more than one split
  int wgs, per_xcd;       // workgroups with work; grid = 8 * per_xcd
  size_t part_o_off, part_ml_off, bytes;
};
AttnPlan attn_plan(int nreq, const int* S, int N, int Hq, int Hkv, int D);
// Device address of the static scratch array on the current device (looked
// up once per device); DDTREE_OK or DDTREE_ERR_HIP.
int attn_static_scratch(void** ptr);
// Workspace that serves attn_plan for these prefix lengths and for every
// shorter ones (elementwise): non-decreasing in each S[r].
size_t attn_workspace_bound(int nreq, const int* S, int N, int Hq, int Hkv, int D);
int attn_launch(const uint16_t* q, const uint16_t* k, const uint16_t* v, int64_t kv_req_stride,
                int nreq, const int* S, int S_cap, int N, int Hq, int Hkv, int D, float scale,
                const uint32_t* anc, int W, uint16_t* out, void* ws, hipStream_t stream);

int prune_launch(const int32_t* budget, int N, int32_t* parent, uint32_t* anc, int W,
                 hipStream_t stream);

size_t argmax_workspace_bytes(int N, int V, int dtype_bytes);
int argmax_launch(const void* logits, int bf16, int64_t row_stride, int N, int V, void* ws,
                  int32_t* out, hipStream_t stream);
int sample_launch(const void* logits, int bf16, int64_t row_stride, int N, int V, float log2e_over_t,
                  uint64_t seed, uint64_t offset, void* ws, int32_t* out, hipStream_t stream);

int budget_launch(const float* score, int B_max, int B_min, double t0, double t1,
                  float* expected, int32_t* budget, hipStream_t stream);

int walk_launch(const int32_t* parent, const int32_t* tok, int N, int L, int R,
                const int32_t* tgt, int32_t* acc, int32_t* n_acc, int32_t* bonus,
                hipStream_t stream);
int compact_launch(uint16_t* kv, int layers, int Hkv, int S_cap, int D, int R, const int* S,
                   int L, const int32_t* acc, const int32_t* n_acc, hipStream_t stream);

}  // namespace ddt_host
