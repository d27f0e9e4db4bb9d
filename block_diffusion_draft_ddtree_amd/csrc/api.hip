// C ABI of libddtree: argument validation on the host, then kernel launches.
// Declarations and semantics: include/ddtree.h.
#include <cstdint>

#include "common.hpp"

#define DDT_API extern "C" __attribute__((visibility("default")))

namespace ddt_host {

int launch_status(hipError_t e) { return e == hipSuccess ? DDTREE_OK : DDTREE_ERR_HIP; }

}  // namespace ddt_host

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// sum_{d=1..L} K^d >= B, without overflow.
bool enough_prefixes(int L, int K, int B) {
  int64_t total = 0, pw = 1;
  for (int d = 1; d <= L; ++d) {
    pw *= K;
    total += pw;
    if (total >= B) return true;
  }
  return total >= B;
}

int topk_check(int L, int V, int K) {
  if (L < 1 || V < 1 || K < 1) return DDTREE_ERR_INVALID_ARGUMENT;
  if (K > V) return DDTREE_ERR_INVALID_ARGUMENT;
  if (L > DDTREE_MAX_L * DDTREE_MAX_REQ || K > DDTREE_MAX_K) return DDTREE_ERR_UNSUPPORTED;
  if (V > DDTREE_MAX_V) return DDTREE_ERR_UNSUPPORTED;
  return DDTREE_OK;
}

int attn_check(int N, int Hq, int Hkv, int D, int S) {
  if (N < 1 || Hq < 1 || Hkv < 1 || S < 0) return DDTREE_ERR_INVALID_ARGUMENT;
  if (Hq % Hkv != 0) return DDTREE_ERR_INVALID_ARGUMENT;
  if (N > DDTREE_MAX_B + 1) return DDTREE_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return DDTREE_ERR_UNSUPPORTED;
  if ((int64_t)N * Hq > (int64_t)1 << 30) return DDTREE_ERR_UNSUPPORTED;
  return DDTREE_OK;
}

}  // namespace

DDT_API const char* ddtree_status_string(int status) {
  switch (status) {
    case DDTREE_OK: return "DDTREE_OK";
    case DDTREE_ERR_INVALID_ARGUMENT: return "DDTREE_ERR_INVALID_ARGUMENT";
    case DDTREE_ERR_UNSUPPORTED: return "DDTREE_ERR_UNSUPPORTED";
    case DDTREE_ERR_WORKSPACE_TOO_SMALL: return "DDTREE_ERR_WORKSPACE_TOO_SMALL";
    case DDTREE_ERR_HIP: return "DDTREE_ERR_HIP";
    default: return "DDTREE_ERR_UNKNOWN";
  }
}

DDT_API int ddtree_version(void) { return 100; }

DDT_API int ddtree_topk_workspace_bytes(int L, int V, int K, size_t* bytes) {
  if (!bytes) return DDTREE_ERR_INVALID_ARGUMENT;
  const int st = topk_check(L, V, K);
  if (st) return st;
  *bytes = ddt_host::topk_plan(L, V, K).bytes;
  return DDTREE_OK;
}

DDT_API int ddtree_topk(const float* logits, int64_t row_stride, int L, int V, int K, float* logp,
                        int32_t* token, void* ws, size_t ws_bytes, hipStream_t stream) {
  const int st = topk_check(L, V, K);
  if (st) return st;
  if (!logits || !logp || !token || !ws) return DDTREE_ERR_INVALID_ARGUMENT;
  if (row_stride < V) return DDTREE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < ddt_host::topk_plan(L, V, K).bytes) return DDTREE_ERR_WORKSPACE_TOO_SMALL;
  return ddt_host::topk_launch(logits, row_stride, L, V, K, logp, token, ws, stream);
}

static int build_check(const float* logp, const int32_t* token, int L, int K, int B, int R,
                       const int32_t* root_token, int32_t* parent, int32_t* depth,
                       int32_t* node_token, uint32_t* anc, int mask_words) {
  if (L < 1 || K < 1 || B < 1 || R < 1) return DDTREE_ERR_INVALID_ARGUMENT;
  if (L > DDTREE_MAX_L || K > DDTREE_MAX_K || B > DDTREE_MAX_B) return DDTREE_ERR_UNSUPPORTED;
  if (R > DDTREE_MAX_REQ) return DDTREE_ERR_UNSUPPORTED;
  if ((int64_t)L * K > DDTREE_MAX_LK) return DDTREE_ERR_UNSUPPORTED;
  if (!enough_prefixes(L, K, B)) return DDTREE_ERR_INVALID_ARGUMENT;
  if (!logp || !token || !root_token || !parent || !depth || !node_token || !anc)
    return DDTREE_ERR_INVALID_ARGUMENT;
  if ((int64_t)mask_words * 32 < B + 1) return DDTREE_ERR_INVALID_ARGUMENT;
  return DDTREE_OK;
}

DDT_API int ddtree_build(const float* logp, const int32_t* token, int L, int K, int B,
                         const int32_t* root_token, int32_t* parent, int32_t* depth,
                         int32_t* node_token, float* score, uint32_t* anc, int mask_words,
                         hipStream_t stream) {
  const int st = build_check(logp, token, L, K, B, 1, root_token, parent, depth, node_token, anc,
                             mask_words);
  if (st) return st;
  return ddt_host::build_launch(logp, token, L, K, B, 1, root_token, parent, depth, node_token,
                                score, anc, mask_words, stream);
}

DDT_API int ddtree_build_batched(const float* logp, const int32_t* token, int L, int K, int B,
                                 int R, const int32_t* root_token, int32_t* parent,
                                 int32_t* depth, int32_t* node_token, float* score, uint32_t* anc,
                                 int mask_words, hipStream_t stream) {
  const int st = build_check(logp, token, L, K, B, R, root_token, parent, depth, node_token, anc,
                             mask_words);
  if (st) return st;
  return ddt_host::build_launch(logp, token, L, K, B, R, root_token, parent, depth, node_token,
                                score, anc, mask_words, stream);
}

DDT_API int ddtree_tree_attn_workspace_bytes(int N, int Hq, int Hkv, int D, int S, size_t* bytes) {
  if (!bytes) return DDTREE_ERR_INVALID_ARGUMENT;
  const int st = attn_check(N, Hq, Hkv, D, S);
  if (st) return st;
  *bytes = ddt_host::attn_workspace_bound(1, &S, N, Hq, Hkv, D);
  return DDTREE_OK;
}

static int attn_args_check(const uint16_t* q, const uint16_t* k, const uint16_t* v, int S_cap,
                           int N, float scale, const uint32_t* anc, int mask_words,
                           const uint16_t* out) {
  if (!q || !k || !v || !anc || !out) return DDTREE_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return DDTREE_ERR_INVALID_ARGUMENT;
  if (S_cap < N) return DDTREE_ERR_INVALID_ARGUMENT;
  if ((int64_t)mask_words * 32 < N) return DDTREE_ERR_INVALID_ARGUMENT;
  if (!(scale > 0.f) || scale != scale || scale > 3.0e38f) return DDTREE_ERR_INVALID_ARGUMENT;
  return DDTREE_OK;
}

DDT_API int ddtree_tree_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, int S,
                             int S_cap, int N, int Hq, int Hkv, int D, float scale,
                             const uint32_t* anc, int mask_words, uint16_t* out, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  int st = attn_check(N, Hq, Hkv, D, S);
  if (st) return st;
  st = attn_args_check(q, k, v, S_cap, N, scale, anc, mask_words, out);
  if (st) return st;
  if ((int64_t)S + N > S_cap) return DDTREE_ERR_INVALID_ARGUMENT;
  const size_t need = ddt_host::attn_plan(1, &S, N, Hq, Hkv, D).bytes;
  if (need && (!ws || ws_bytes < need)) return DDTREE_ERR_WORKSPACE_TOO_SMALL;
  return ddt_host::attn_launch(q, k, v, 0, 1, &S, S_cap, N, Hq, Hkv, D, scale, anc, mask_words,
                               out, ws, stream);
}

DDT_API int ddtree_tree_attn_noalloc(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     int S, int S_cap, int N, int Hq, int Hkv, int D, float scale,
                                     const uint32_t* anc, int mask_words, uint16_t* out,
                                     hipStream_t stream) {
  int st = attn_check(N, Hq, Hkv, D, S);
  if (st) return st;
  st = attn_args_check(q, k, v, S_cap, N, scale, anc, mask_words, out);
  if (st) return st;
  if ((int64_t)S + N > S_cap) return DDTREE_ERR_INVALID_ARGUMENT;
  const size_t need = ddt_host::attn_plan(1, &S, N, Hq, Hkv, D).bytes;
  if (need > DDTREE_NOALLOC_SCRATCH_BYTES) return DDTREE_ERR_WORKSPACE_TOO_SMALL;
  void* ws = nullptr;
  if (need) {
    st = ddt_host::attn_static_scratch(&ws);
    if (st) return st;
  }
  return ddt_host::attn_launch(q, k, v, 0, 1, &S, S_cap, N, Hq, Hkv, D, scale, anc, mask_words,
                               out, ws, stream);
}

static int attn_batch_check(int R, const int32_t* S, int N, int Hq, int Hkv, int D) {
  if (R < 1 || !S) return DDTREE_ERR_INVALID_ARGUMENT;
  if (R > DDTREE_MAX_REQ) return DDTREE_ERR_UNSUPPORTED;
  for (int r = 0; r < R; ++r) {
    const int st = attn_check(N, Hq, Hkv, D, S[r]);
    if (st) return st;
  }
  return DDTREE_OK;
}

DDT_API int ddtree_tree_attn_batched_workspace_bytes(int R, const int32_t* S, int N, int Hq,
                                                     int Hkv, int D, size_t* bytes) {
  if (!bytes) return DDTREE_ERR_INVALID_ARGUMENT;
  const int st = attn_batch_check(R, S, N, Hq, Hkv, D);
  if (st) return st;
  *bytes = ddt_host::attn_workspace_bound(R, S, N, Hq, Hkv, D);
  return DDTREE_OK;
}

DDT_API int ddtree_tree_attn_batched(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     int64_t kv_req_stride, int R, const int32_t* S, int S_cap,
                                     int N, int Hq, int Hkv, int D, float scale,
                                     const uint32_t* anc, int mask_words, uint16_t* out,
                                     void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = attn_batch_check(R, S, N, Hq, Hkv, D);
  if (st) return st;
  st = attn_args_check(q, k, v, S_cap, N, scale, anc, mask_words, out);
  if (st) return st;
  for (int r = 0; r < R; ++r)
    if ((int64_t)S[r] + N > S_cap) return DDTREE_ERR_INVALID_ARGUMENT;
  // Each request's K (and V) block [Hkv, S_cap, D] must fit in its stride,
  // and the stride must keep 16-byte alignment.
  if (R > 1 && (kv_req_stride < (int64_t)Hkv * S_cap * D || kv_req_stride % 8 != 0))
    return DDTREE_ERR_INVALID_ARGUMENT;
  const size_t need = ddt_host::attn_plan(R, S, N, Hq, Hkv, D).bytes;
  if (need && (!ws || ws_bytes < need)) return DDTREE_ERR_WORKSPACE_TOO_SMALL;
  return ddt_host::attn_launch(q, k, v, kv_req_stride, R, S, S_cap, N, Hq, Hkv, D, scale, anc,
                               mask_words, out, ws, stream);
}

static int argmax_check(int dtype, int N, int V) {
  if (N < 1 || V < 1) return DDTREE_ERR_INVALID_ARGUMENT;
  if (dtype != DDTREE_DTYPE_F32 && dtype != DDTREE_DTYPE_BF16) return DDTREE_ERR_INVALID_ARGUMENT;
  if (N > DDTREE_MAX_B + 1 || V > DDTREE_MAX_V) return DDTREE_ERR_UNSUPPORTED;
  return DDTREE_OK;
}

DDT_API int ddtree_target_argmax_workspace_bytes(int dtype, int N, int V, size_t* bytes) {
  if (!bytes) return DDTREE_ERR_INVALID_ARGUMENT;
  const int st = argmax_check(dtype, N, V);
  if (st) return st;
  *bytes = ddt_host::argmax_workspace_bytes(N, V, dtype == DDTREE_DTYPE_BF16 ? 2 : 4);
  return DDTREE_OK;
}

DDT_API int ddtree_target_argmax(const void* logits, int dtype, int64_t row_stride, int N,
                                 int V, int32_t* out, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  const int st = argmax_check(dtype, N, V);
  if (st) return st;
  if (!logits || !out || !ws) return DDTREE_ERR_INVALID_ARGUMENT;
  if (row_stride < V) return DDTREE_ERR_INVALID_ARGUMENT;
  const uintptr_t esize = dtype == DDTREE_DTYPE_BF16 ? 2u : 4u;
  if (reinterpret_cast<uintptr_t>(logits) % esize != 0) return DDTREE_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(ws) % 8 != 0) return DDTREE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < ddt_host::argmax_workspace_bytes(N, V, (int)esize))
    return DDTREE_ERR_WORKSPACE_TOO_SMALL;
  return ddt_host::argmax_launch(logits, dtype == DDTREE_DTYPE_BF16, row_stride, N, V, ws, out,
                                 stream);
}

DDT_API int ddtree_target_sample(const void* logits, int dtype, int64_t row_stride, int N, int V,
                                 float temperature, uint64_t seed, uint64_t offset, int32_t* out,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  const int st = argmax_check(dtype, N, V);
  if (st) return st;
  if (!logits || !out || !ws) return DDTREE_ERR_INVALID_ARGUMENT;
  if (row_stride < V) return DDTREE_ERR_INVALID_ARGUMENT;
  const uintptr_t esize = dtype == DDTREE_DTYPE_BF16 ? 2u : 4u;
  if (reinterpret_cast<uintptr_t>(logits) % esize != 0) return DDTREE_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(ws) % 8 != 0) return DDTREE_ERR_INVALID_ARGUMENT;
  // T > 0 and log2(e) / T a finite, normal fp32 number.
  if (!(temperature > 0.f) || !(temperature <= 3.0e38f)) return DDTREE_ERR_INVALID_ARGUMENT;
  const double c = 1.4426950408889634 / (double)temperature;
  if (!(c <= 3.0e38) || c < 1.2e-38) return DDTREE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < ddt_host::argmax_workspace_bytes(N, V, (int)esize))
    return DDTREE_ERR_WORKSPACE_TOO_SMALL;
  return ddt_host::sample_launch(logits, dtype == DDTREE_DTYPE_BF16, row_stride, N, V, (float)c,
                                 seed, offset, ws, out, stream);
}

DDT_API int ddtree_budget_select(const float* score, int B_max, int B_min, double t0, double t1,
                                 float* expected, int32_t* budget, hipStream_t stream) {
  if (B_max < 1 || B_min < 0 || B_min > B_max) return DDTREE_ERR_INVALID_ARGUMENT;
  if (B_max > DDTREE_MAX_B) return DDTREE_ERR_UNSUPPORTED;
  if (!score || !budget) return DDTREE_ERR_INVALID_ARGUMENT;
  if (!(t0 >= 0.0) || !(t1 >= 0.0) || !(t0 <= 1e300) || !(t1 <= 1e300) || !(t0 + t1 > 0.0))
    return DDTREE_ERR_INVALID_ARGUMENT;
  return ddt_host::budget_launch(score, B_max, B_min, t0, t1, expected, budget, stream);
}

DDT_API int ddtree_tree_prune(const int32_t* budget, int N, int32_t* parent, uint32_t* anc,
                              int mask_words, hipStream_t stream) {
  if (N < 1 || !budget || !parent || !anc) return DDTREE_ERR_INVALID_ARGUMENT;
  if (N > DDTREE_MAX_B + 1) return DDTREE_ERR_UNSUPPORTED;
  if ((int64_t)mask_words * 32 < N) return DDTREE_ERR_INVALID_ARGUMENT;
  return ddt_host::prune_launch(budget, N, parent, anc, mask_words, stream);
}

static int walk_check(const int32_t* parent, const int32_t* node_token, int N, int L, int R,
                      const int32_t* target, int32_t* acc, int32_t* n_acc, int32_t* next_bonus) {
  if (N < 1 || L < 1 || R < 1) return DDTREE_ERR_INVALID_ARGUMENT;
  if (L > DDTREE_MAX_L || N > DDTREE_MAX_B + 1 || R > DDTREE_MAX_REQ) return DDTREE_ERR_UNSUPPORTED;
  if (!parent || !node_token || !target || !acc || !n_acc || !next_bonus)
    return DDTREE_ERR_INVALID_ARGUMENT;
  return DDTREE_OK;
}

DDT_API int ddtree_accept_walk(const int32_t* parent, const int32_t* node_token, int N, int L,
                               const int32_t* target_argmax, int32_t* acc, int32_t* n_acc,
                               int32_t* next_bonus, hipStream_t stream) {
  const int st = walk_check(parent, node_token, N, L, 1, target_argmax, acc, n_acc, next_bonus);
  if (st) return st;
  return ddt_host::walk_launch(parent, node_token, N, L, 1, target_argmax, acc, n_acc, next_bonus,
                               stream);
}

DDT_API int ddtree_accept_walk_batched(const int32_t* parent, const int32_t* node_token, int N,
                                       int L, int R, const int32_t* target, int32_t* acc,
                                       int32_t* n_acc, int32_t* next_bonus, hipStream_t stream) {
  const int st = walk_check(parent, node_token, N, L, R, target, acc, n_acc, next_bonus);
  if (st) return st;
  return ddt_host::walk_launch(parent, node_token, N, L, R, target, acc, n_acc, next_bonus,
                               stream);
}

static int compact_check(uint16_t* kv, int layers, int Hkv, int S_cap, int D, int R,
                         const int32_t* S, int N, int L, const int32_t* acc,
                         const int32_t* n_acc) {
  if (layers < 1 || Hkv < 1 || N < 1 || L < 1 || R < 1) return DDTREE_ERR_INVALID_ARGUMENT;
  if (L > DDTREE_MAX_L || R > DDTREE_MAX_REQ) return DDTREE_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return DDTREE_ERR_UNSUPPORTED;
  if (!kv || !acc || !n_acc || !S || !aligned16(kv)) return DDTREE_ERR_INVALID_ARGUMENT;
  for (int r = 0; r < R; ++r)
    if (S[r] < 0 || (int64_t)S[r] + N > S_cap) return DDTREE_ERR_INVALID_ARGUMENT;
  if ((int64_t)layers * 2 * Hkv > 0x7FFFFFFF) return DDTREE_ERR_UNSUPPORTED;
  return DDTREE_OK;
}

DDT_API int ddtree_kv_compact(uint16_t* kv, int layers, int Hkv, int S_cap, int D, int S, int N,
                              int L, const int32_t* acc, const int32_t* n_acc,
                              hipStream_t stream) {
  const int st = compact_check(kv, layers, Hkv, S_cap, D, 1, &S, N, L, acc, n_acc);
  if (st) return st;
  return ddt_host::compact_launch(kv, layers, Hkv, S_cap, D, 1, &S, L, acc, n_acc, stream);
}

DDT_API int ddtree_kv_compact_batched(uint16_t* kv, int layers, int Hkv, int S_cap, int D, int R,
                                      const int32_t* S, int N, int L, const int32_t* acc,
                                      const int32_t* n_acc, hipStream_t stream) {
  const int st = compact_check(kv, layers, Hkv, S_cap, D, R, S, N, L, acc, n_acc);
  if (st) return st;
  return ddt_host::compact_launch(kv, layers, Hkv, S_cap, D, R, S, L, acc, n_acc, stream);
}
