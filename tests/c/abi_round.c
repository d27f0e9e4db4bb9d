/* One DDTree round driven through the C ABI alone (no Python): top-K, tree
 * build, tree attention, accept walk and KV compaction on a small shape
 * (L = 4 positions, V = 1000, K = 8, B = 16, 4 query / 2 kv heads, D = 64,
 * a 128-row prefix), with the structural facts of each step checked on the
 * host ("DDTree Deep Dive", sections 1-6): ranked top-K rows, a
 * prefix-closed tree in score order whose mask rows are ancestor-or-self
 * sets, root-node attention against a direct fp64 evaluation, the walk's
 * path, and the compacted cache rows. Prints "abi_round ok" and exits 0 on
 * success; any failed check prints it and exits 1. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ddtree.h"

enum { L = 4, V = 1000, K = 8, B = 16, N = B + 1, HQ = 4, HKV = 2, D = 64, S = 128 };
enum { S_CAP = S + N, W = (N + 31) / 32, G = HQ / HKV };

static int failures = 0;
#define CHECK(cond, ...)                        \
  do {                                          \
    if (!(cond)) {                              \
      fprintf(stderr, "check failed: " __VA_ARGS__); \
      fprintf(stderr, "\n");                    \
      ++failures;                               \
    }                                           \
  } while (0)
#define HIPOK(x)                                                         \
  do {                                                                   \
    hipError_t e_ = (x);                                                 \
    if (e_ != hipSuccess) {                                              \
      fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                          \
    }                                                                    \
  } while (0)
#define DDOK(x)                                                          \
  do {                                                                   \
    int s_ = (x);                                                        \
    if (s_ != DDTREE_OK) {                                               \
      fprintf(stderr, "%s at line %d\n", ddtree_status_string(s_), __LINE__); \
      return 1;                                                          \
    }                                                                    \
  } while (0)

/* xorshift32 uniform in [0, 1) */
static uint32_t rng_state = 2463534242u;
static float urand(void) {
  rng_state ^= rng_state << 13;
  rng_state ^= rng_state >> 17;
  rng_state ^= rng_state << 5;
  return (float)(rng_state >> 8) * (1.0f / 16777216.0f);
}

static uint16_t to_bf16(float f) { /* round to nearest even */
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
static double from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

int main(void) {
  /* Inputs: drafter logits with a few hot tokens per position (so the tree
   * grows below the root), queries and the cache. */
  static float logits[L * V];
  for (int i = 0; i < L * V; ++i) logits[i] = 4.0f * urand() - 2.0f;
  for (int i = 0; i < L; ++i)
    for (int h = 0; h < 3; ++h) logits[i * V + 37 * (i + 1) + 101 * h] += 9.0f - 2.0f * h;
  static uint16_t q[N * HQ * D], kv[2 * HKV * S_CAP * D], kv0[2 * HKV * S_CAP * D];
  for (int i = 0; i < N * HQ * D; ++i) q[i] = to_bf16(2.0f * urand() - 1.0f);
  for (int i = 0; i < 2 * HKV * S_CAP * D; ++i) kv[i] = kv0[i] = to_bf16(2.0f * urand() - 1.0f);

  float *d_logits, *d_logp, *d_score;
  int32_t *d_token, *d_root, *d_parent, *d_depth, *d_ntok, *d_tgt, *d_acc, *d_nacc, *d_bonus;
  uint32_t* d_anc;
  uint16_t *d_q, *d_kv, *d_out;
  void *d_ws_topk, *d_ws_attn;
  size_t ws_topk = 0, ws_attn = 0;
  DDOK(ddtree_topk_workspace_bytes(L, V, K, &ws_topk));
  DDOK(ddtree_tree_attn_workspace_bytes(N, HQ, HKV, D, S, &ws_attn));
  HIPOK(hipMalloc((void**)&d_logits, sizeof logits));
  HIPOK(hipMalloc((void**)&d_logp, L * K * sizeof(float)));
  HIPOK(hipMalloc((void**)&d_token, L * K * sizeof(int32_t)));
  HIPOK(hipMalloc((void**)&d_root, sizeof(int32_t)));
  HIPOK(hipMalloc((void**)&d_parent, N * sizeof(int32_t)));
  HIPOK(hipMalloc((void**)&d_depth, N * sizeof(int32_t)));
  HIPOK(hipMalloc((void**)&d_ntok, N * sizeof(int32_t)));
  HIPOK(hipMalloc((void**)&d_score, N * sizeof(float)));
  HIPOK(hipMalloc((void**)&d_anc, N * W * sizeof(uint32_t)));
  HIPOK(hipMalloc((void**)&d_q, sizeof q));
  HIPOK(hipMalloc((void**)&d_kv, sizeof kv));
  HIPOK(hipMalloc((void**)&d_out, sizeof q));
  HIPOK(hipMalloc((void**)&d_tgt, N * sizeof(int32_t)));
  HIPOK(hipMalloc((void**)&d_acc, (L + 1) * sizeof(int32_t)));
  HIPOK(hipMalloc((void**)&d_nacc, sizeof(int32_t)));
  HIPOK(hipMalloc((void**)&d_bonus, sizeof(int32_t)));
  HIPOK(hipMalloc(&d_ws_topk, ws_topk > 0 ? ws_topk : 256));
  HIPOK(hipMalloc(&d_ws_attn, ws_attn > 0 ? ws_attn : 256));
  const int32_t root = 7;
  HIPOK(hipMemcpy(d_logits, logits, sizeof logits, hipMemcpyHostToDevice));
  HIPOK(hipMemcpy(d_root, &root, sizeof root, hipMemcpyHostToDevice));
  HIPOK(hipMemcpy(d_q, q, sizeof q, hipMemcpyHostToDevice));
  HIPOK(hipMemcpy(d_kv, kv, sizeof kv, hipMemcpyHostToDevice));

  /* Host-side validation: a bad call is refused before any work. */
  CHECK(ddtree_topk(d_logits, V, L, V, V + 1, d_logp, d_token, d_ws_topk, ws_topk, 0) ==
            DDTREE_ERR_INVALID_ARGUMENT,
        "K > V must be rejected");

  /* 1. top-K */
  DDOK(ddtree_topk(d_logits, V, L, V, K, d_logp, d_token, d_ws_topk, ws_topk, 0));
  float logp[L * K];
  int32_t token[L * K];
  HIPOK(hipMemcpy(logp, d_logp, sizeof logp, hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(token, d_token, sizeof token, hipMemcpyDeviceToHost));
  for (int i = 0; i < L; ++i) {
    double mass = 0.0;
    for (int k = 0; k < K; ++k) {
      const int t = token[i * K + k];
      CHECK(t >= 0 && t < V, "token id range");
      CHECK(logp[i * K + k] <= 0.0f, "log-prob <= 0");
      mass += exp((double)logp[i * K + k]);
      if (k) {
        CHECK(logits[i * V + token[i * K + k - 1]] >= logits[i * V + t], "rank order");
        CHECK(logp[i * K + k - 1] >= logp[i * K + k], "log-probs descend");
      }
      /* logp = x - lse: the gap to the row's first entry is the logit gap */
      CHECK(fabs((logp[i * K] - logp[i * K + k]) - (logits[i * V + token[i * K]] - logits[i * V + t])) < 1e-5,
            "logp differences equal logit differences");
    }
    CHECK(mass <= 1.0 + 1e-5, "top-K mass <= 1");
    /* nothing outside the top-K beats its last entry */
    const float last = logits[i * V + token[i * K + K - 1]];
    int above = 0;
    for (int v = 0; v < V; ++v) above += logits[i * V + v] > last;
    CHECK(above <= K - 1, "top-K set is the K largest");
  }

  /* 2. tree */
  DDOK(ddtree_build(d_logp, d_token, L, K, B, d_root, d_parent, d_depth, d_ntok, d_score, d_anc, W, 0));
  int32_t parent[N], depth[N], ntok[N];
  float score[N];
  uint32_t anc[N * W];
  HIPOK(hipMemcpy(parent, d_parent, sizeof parent, hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(depth, d_depth, sizeof depth, hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(ntok, d_ntok, sizeof ntok, hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(score, d_score, sizeof score, hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(anc, d_anc, sizeof anc, hipMemcpyDeviceToHost));
  CHECK(parent[0] == -1 && depth[0] == 0 && ntok[0] == root, "root node");
  int maxdepth = 0;
  for (int n = 1; n < N; ++n) {
    const int p = parent[n];
    CHECK(p >= 0 && p < n, "parents precede children");
    CHECK(depth[n] == depth[p] + 1 && depth[n] <= L, "depth = parent depth + 1");
    CHECK(score[n] <= score[p], "a child scores at most its parent");
    if (n > 1) CHECK(score[n] <= score[n - 1], "pops in score order");
    int found = 0;
    for (int k = 0; k < K; ++k) found |= token[(depth[n] - 1) * K + k] == ntok[n];
    CHECK(found, "node token is in its position's top-K");
    for (int w = 0; w < W; ++w) {
      uint32_t want = anc[p * W + w];
      if (w == n / 32) want |= 1u << (n % 32);
      CHECK(anc[n * W + w] == want, "mask row = parent row | self");
    }
    if (depth[n] > maxdepth) maxdepth = depth[n];
  }
  CHECK(maxdepth >= 2, "the tree grows below the root");

  /* 3. tree attention; the root attends to the prefix and itself only */
  const float scale = 0.125f; /* 1 / sqrt(64) */
  DDOK(ddtree_tree_attn(d_q, d_kv, d_kv + HKV * S_CAP * D, S, S_CAP, N, HQ, HKV, D, scale, d_anc, W,
                        d_out, d_ws_attn, ws_attn, 0));
  static uint16_t out[N * HQ * D];
  HIPOK(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));
  for (int h = 0; h < HQ; ++h) {
    const int g = h / G;
    double logit[S + 1], mx = -1e300, den = 0.0;
    for (int j = 0; j <= S; ++j) { /* rows 0..S-1 and the root row S */
      double dot = 0.0;
      for (int d = 0; d < D; ++d)
        dot += from_bf16(q[(0 * HQ + h) * D + d]) * from_bf16(kv[(g * S_CAP + j) * D + d]);
      logit[j] = scale * dot;
      if (logit[j] > mx) mx = logit[j];
    }
    for (int j = 0; j <= S; ++j) den += exp(logit[j] - mx);
    for (int d = 0; d < D; ++d) {
      double num = 0.0;
      for (int j = 0; j <= S; ++j)
        num += exp(logit[j] - mx) * from_bf16(kv[(HKV * S_CAP + g * S_CAP + j) * D + d]);
      const double ref = num / den, got = from_bf16(out[(0 * HQ + h) * D + d]);
      CHECK(fabs(got - ref) <= 2e-2 + 1e-2 * fabs(ref), "root attention within tolerance");
    }
  }

  /* 4. walk: the target follows the first child of each node for two steps */
  int32_t tgt[N];
  for (int n = 0; n < N; ++n) tgt[n] = 999;
  int cur = 0, path[L + 1], a_want = 0;
  path[0] = 0;
  for (int step = 0; step < 2; ++step) {
    int child = -1;
    for (int n = cur + 1; n < N && child < 0; ++n)
      if (parent[n] == cur) child = n;
    if (child < 0) break;
    tgt[cur] = ntok[child];
    cur = child;
    path[++a_want] = cur;
  }
  HIPOK(hipMemcpy(d_tgt, tgt, sizeof tgt, hipMemcpyHostToDevice));
  DDOK(ddtree_accept_walk(d_parent, d_ntok, N, L, d_tgt, d_acc, d_nacc, d_bonus, 0));
  int32_t acc[L + 1], n_acc, bonus;
  HIPOK(hipMemcpy(acc, d_acc, sizeof acc, hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(&n_acc, d_nacc, sizeof n_acc, hipMemcpyDeviceToHost));
  HIPOK(hipMemcpy(&bonus, d_bonus, sizeof bonus, hipMemcpyDeviceToHost));
  CHECK(n_acc == a_want, "accepted count");
  for (int k = 0; k <= L; ++k) CHECK(acc[k] == (k <= a_want ? path[k] : -1), "accepted path");
  CHECK(bonus == tgt[cur], "next bonus");

  /* 5. compaction: row S + k takes row S + acc[k], k = 1..a; others stay */
  DDOK(ddtree_kv_compact(d_kv, 1, HKV, S_CAP, D, S, N, L, d_acc, d_nacc, 0));
  HIPOK(hipMemcpy(kv, d_kv, sizeof kv, hipMemcpyDeviceToHost));
  for (int sl = 0; sl < 2 * HKV; ++sl)
    for (int row = 0; row < S_CAP; ++row) {
      const int src = (row > S && row <= S + n_acc) ? S + acc[row - S] : row;
      CHECK(memcmp(&kv[(sl * S_CAP + row) * D], &kv0[(sl * S_CAP + src) * D], D * 2) == 0,
            "compacted row");
    }
  HIPOK(hipDeviceSynchronize());
  if (failures) {
    printf("abi_round: %d checks failed\n", failures);
    return 1;
  }
  printf("abi_round ok: tree depth %d, accepted %d, library version %d\n", maxdepth, n_acc,
         ddtree_version());
  return 0;
}
