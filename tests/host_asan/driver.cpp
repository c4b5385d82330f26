// Host-side checks of the library's C ABI for an AddressSanitizer build:
// every call here runs on the CPU only (configuration and plan checks, the
// tree-expansion and lookahead policies, null-handle calls).  Exit status 0
// when every expectation holds; ASan aborts the process on a memory error.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "spec_verify.h"

static int failures = 0;
#define EXPECT(c)                                                    \
  do {                                                               \
    if (!(c)) {                                                      \
      std::fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #c); \
      ++failures;                                                    \
    }                                                                \
  } while (0)

static spec_config dense(int L, int d, int hq, int hkv, int D, int ff, int V, int wdt, int kvdt, int ctx, int max_k) {
  spec_config c;
  std::memset(&c, 0, sizeof c);
  c.n_layers = L; c.d_model = d; c.n_q_heads = hq; c.n_kv_heads = hkv; c.head_dim = D; c.d_ff = ff; c.vocab = V;
  c.weight_dtype = wdt; c.kv_dtype = kvdt; c.rope_theta = 10000.f; c.rms_eps = 1e-5f;
  c.max_ctx = ctx; c.max_k = max_k;
  return c;
}

// a small linear congruential generator (fixed seed)
static uint32_t lcg_state = 12345u;
static uint32_t lcg() { return lcg_state = lcg_state * 1664525u + 1013904223u; }

int main() {
  char msg[256];
  std::vector<spec_config> good;
  good.push_back(dense(2, 256, 4, 4, 64, 1024, 2048, SPEC_DT_F32, SPEC_DT_F32, 600, 4));
  good.push_back(dense(32, 4096, 32, 32, 128, 11008, 32000, SPEC_DT_BF16, SPEC_DT_BF16, 1700, 15));
  good.push_back(dense(32, 4096, 32, 32, 128, 11008, 32000, SPEC_DT_INT4G128, SPEC_DT_BF16, 2700, 8));
  good.push_back(dense(28, 3584, 28, 4, 128, 18944, 152064, SPEC_DT_BF16, SPEC_DT_BF16, 4800, 10));
  spec_config moe = dense(16, 2048, 16, 4, 128, 0, 32000, SPEC_DT_BF16, SPEC_DT_BF16, 2700, 8);
  moe.n_experts = 64; moe.top_k = 6; moe.n_shared = 1; moe.d_ff_expert = 1408;
  good.push_back(moe);
  spec_config many = good[1];
  many.n_seqs = 8; many.attn_group_pages = 6;
  good.push_back(many);
  for (const spec_config& c : good) {
    EXPECT(spec_config_check(&c, msg, sizeof msg) == SPEC_OK);
    // (small grids only for the small model: a large matrix on a few
    // workgroups exceeds the per-workgroup split-K lists, and is refused)
    for (int g : {1, 7, 64, 256, 304}) {
      if (g < 64 && c.n_layers > 2) continue;
      if (spec_plan_check(&c, g, msg, sizeof msg) != SPEC_OK) {
        std::fprintf(stderr, "plan check (grid %d): %s\n", g, msg);
        ++failures;
      }
    }
  }
  // a large model on one workgroup is refused, not overrun
  EXPECT(spec_plan_check(&good[1], 1, msg, sizeof msg) == SPEC_EINVAL);
  // invalid configurations are refused with a message, short buffers included
  spec_config bad = good[1];
  bad.head_dim = 96;
  EXPECT(spec_config_check(&bad, msg, sizeof msg) == SPEC_EINVAL && std::strlen(msg) > 0);
  EXPECT(spec_config_check(&bad, msg, 1) == SPEC_EINVAL);
  EXPECT(spec_config_check(&bad, nullptr, 0) == SPEC_EINVAL);
  bad = good[1];
  bad.reserved[0] = 1;
  EXPECT(spec_config_check(&bad, msg, sizeof msg) == SPEC_EINVAL);
  bad = good[0];
  bad.attn_group_pages = 6;   // fp32 models take 3-page groups
  EXPECT(spec_config_check(&bad, msg, sizeof msg) == SPEC_EINVAL);
  EXPECT(spec_config_check(nullptr, msg, sizeof msg) == SPEC_EINVAL);
  EXPECT(spec_plan_check(&good[1], 0, msg, sizeof msg) == SPEC_EINVAL);

  // lookahead policy
  for (int max_k = 1; max_k <= 15; ++max_k)
    for (int k = 1; k <= max_k; ++k)
      for (int n = 0; n <= k; ++n) {
        const int nk = spec_adaptive_k(k, n, max_k);
        EXPECT(nk >= 1 && nk <= max_k);
      }
  EXPECT(spec_adaptive_k(0, 0, 5) == -1 && spec_adaptive_k(3, 4, 5) == -1);

  // tree expansion on seeded random candidate sets, every output within bounds
  for (int trial = 0; trial < 2000; ++trial) {
    const int n = (int)(lcg() % 40);
    std::vector<int32_t> parents(n), off(n + 1, 0), ids;
    std::vector<double> p(n), cd(n);
    for (int i = 0; i < n; ++i) {
      parents[i] = i == 0 ? -1 : (int)(lcg() % (unsigned)(i + 1)) - 1;
      p[i] = (lcg() % 1001) / 1000.0;
      cd[i] = (lcg() % 4) * 0.25;
      const int ne = (int)(lcg() % 12);
      for (int j = 0; j < ne; ++j) ids.push_back((int32_t)(lcg() % 300));
      off[i + 1] = (int32_t)ids.size();
    }
    std::vector<int32_t> base;
    for (int j = 0; j < (int)(lcg() % 6); ++j) base.push_back((int32_t)(lcg() % 300));
    const int max_nodes = (int)(lcg() % 16);
    std::vector<int32_t> order(max_nodes > 0 ? max_nodes : 1, -7), rows(max_nodes + 1, -7);
    const int cnt = spec_tree_expand(n, n ? parents.data() : nullptr, n ? p.data() : nullptr, off.data(),
                                     ids.empty() ? nullptr : ids.data(), (int32_t)base.size(),
                                     base.empty() ? nullptr : base.data(), 1.0 + (lcg() % 20), (lcg() % 4) * 0.5,
                                     n ? cd.data() : nullptr, max_nodes, order.data(), rows.data());
    EXPECT(cnt >= 0 && cnt <= max_nodes && cnt <= n);
    if (cnt < 0) continue;
    std::vector<int> seen(n, -1);
    for (int r = 0; r < cnt; ++r) {
      EXPECT(order[r] >= 0 && order[r] < n && seen[order[r]] < 0);
      if (order[r] < 0 || order[r] >= n) continue;
      seen[order[r]] = r;
      const int par = parents[order[r]];
      EXPECT(par < 0 || (seen[par] >= 0 && seen[par] < r));   // a parent is admitted first
      EXPECT(rows[r + 1] >= 0 && rows[r + 1] <= r);
    }
    if (cnt > 0) EXPECT(rows[0] == -1);
  }
  int32_t order1[1];
  EXPECT(spec_tree_expand(-1, nullptr, nullptr, nullptr, nullptr, 0, nullptr, 1.0, 1.0, nullptr, 1, order1,
                          nullptr) == -1);

  // calls on a null handle
  EXPECT(spec_kv_len(nullptr) == -1);
  EXPECT(spec_seq_kv_len(nullptr, 0) == -1);
  EXPECT(spec_last_error(nullptr) != nullptr);
  spec_verify_destroy(nullptr);
  spec_step_result res;
  int32_t tok = 0;
  EXPECT(spec_verify_step(nullptr, &tok, 0, SPEC_ACCEPT_GREEDY, nullptr, nullptr, &res, nullptr) == SPEC_EINVAL);
  EXPECT(spec_kv_commit_rollback(nullptr, 0) == SPEC_EINVAL);

  std::fprintf(stderr, "host checks: %d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
