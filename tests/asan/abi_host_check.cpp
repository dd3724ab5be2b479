// Host-side checks of libcsa2 under AddressSanitizer: argument validation of
// every entry point (rejected before any launch, so no GPU is touched),
// workspace sizing, the launch timer and a randomized block-pool workload
// against a plain reference set.  Exits non-zero on the first failed check;
// ASan aborts on any out-of-bounds access, use after free or leak.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <set>
#include <vector>

#include "../../include/csa2.h"

static int g_fail = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      g_fail = 1;                                                  \
    }                                                              \
  } while (0)

static void validation() {
  void *s = nullptr;
  size_t n = 0;
  CHECK(csa2_abi_version() == CSA2_ABI_VERSION);
  for (int st = 0; st <= 5; ++st) CHECK(csa2_status_string((csa2_status)st) != nullptr);
  CHECK(csa2_fp4_pack(nullptr, 4, 15, nullptr, nullptr, s) == CSA2_ERR_INVALID_ARG);
  CHECK(csa2_fp4_pack(nullptr, 0, 16, nullptr, nullptr, s) == CSA2_OK);
  CHECK(csa2_fp4_unpack(nullptr, nullptr, 3, 16, nullptr, s) == CSA2_ERR_INVALID_ARG);
  CHECK(csa2_topk_workspace_size(1, 100, 0, &n) == CSA2_ERR_INVALID_ARG);
  CHECK(csa2_topk_workspace_size(3, 70000, 2048, &n) == CSA2_OK && n > 0);
  CHECK(csa2_index_select_workspace_size(2, 1 << 20, 2048, 2048, 8, &n) == CSA2_OK && n > 0);
  CHECK(csa2_index_select_workspace_size(2, 1 << 20, 2048, 2049, 8, &n) == CSA2_ERR_INVALID_ARG);
  CHECK(csa2_index_reindex_layers_workspace_size(3, 1, 2048, 2048, 8, &n) == CSA2_OK && n > 0);
  CHECK(csa2_index_reindex_layers_workspace_size(9, 1, 2048, 2048, 8, &n) == CSA2_ERR_INVALID_ARG);
  CHECK(csa2_attn_workspace_size(1, 64, 2048, 512, &n) == CSA2_OK);
  CHECK(csa2_attn_layers_workspace_size(20, 32, 128, 4096, 512, 1, &n) == CSA2_OK && n > 0);
  CHECK(csa2_attn_layers_workspace_size(21, 1, 64, 2048, 512, 0, &n) == CSA2_ERR_INVALID_ARG);
  // at most 65,535 sequences per call (layers x sequences for the layered attention)
  CHECK(csa2_attn_workspace_size(65535, 128, 4096, 512, &n) == CSA2_OK && n > 0);
  CHECK(csa2_attn_workspace_size(65536, 64, 2048, 512, &n) == CSA2_ERR_INVALID_ARG);
  CHECK(csa2_attn_layers_workspace_size(20, 3276, 128, 4096, 512, 1, &n) == CSA2_OK && n > 0);
  CHECK(csa2_attn_layers_workspace_size(20, 3277, 64, 2048, 512, 0, &n) == CSA2_ERR_INVALID_ARG);
  CHECK(csa2_index_select_workspace_size(65535, 1 << 10, 2048, 2048, 8, &n) == CSA2_OK && n > 0);
  CHECK(csa2_index_select_workspace_size(65536, 1 << 10, 2048, 0, 8, &n) == CSA2_ERR_INVALID_ARG);
  CHECK(csa2_workspace_clear(nullptr, 0, s) == CSA2_OK);
  CHECK(csa2_workspace_clear(nullptr, 64, s) == CSA2_ERR_INVALID_ARG);

  // a layer and a batch view that pass the host checks (fake, aligned pointers: nothing is dereferenced)
  uint8_t *fake = reinterpret_cast<uint8_t *>(uintptr_t(1) << 20);
  csa2_kv_layer kv{fake, fake, nullptr, fake, 4, 64, 512, 0, 64, CSA2_BF16, nullptr, 1};
  const int32_t *tab = reinterpret_cast<const int32_t *>(fake);
  csa2_seqs sq{tab, 4, tab, 1, 256};
  CHECK(csa2_index_scores(&kv, &sq, nullptr, nullptr, nullptr, s) == CSA2_ERR_INVALID_ARG);
  kv.block_tokens = 32;
  CHECK(csa2_index_select(&kv, &sq, fake, nullptr, 8, CSA2_FULL, nullptr, nullptr, 0, 0, reinterpret_cast<int32_t *>(fake),
                          fake, 1 << 30, s) == CSA2_ERR_INVALID_ARG);
  kv.block_tokens = 64;
  CHECK(csa2_index_select(&kv, &sq, fake, nullptr, 8, CSA2_FULL, nullptr, nullptr, 0, 0, reinterpret_cast<int32_t *>(fake),
                          fake, 16, s) == CSA2_ERR_WORKSPACE);
  CHECK(csa2_index_select(&kv, &sq, fake, nullptr, 8, CSA2_REINDEX, nullptr, nullptr, 16, 8,
                          reinterpret_cast<int32_t *>(fake), fake, 1 << 30, s) == CSA2_ERR_INVALID_ARG);
  csa2_seqs bad = sq;
  bad.max_seq_len = 257;  // beyond the table's capacity
  CHECK(csa2_sparse_fp4_decode_attn(&kv, &bad, reinterpret_cast<uint16_t *>(fake), 64,
                                    reinterpret_cast<int32_t *>(fake), 64, 0.1f, reinterpret_cast<float *>(fake),
                                    nullptr, fake, 1 << 30, s) == CSA2_ERR_INVALID_ARG);
  CHECK(csa2_sparse_fp4_decode_attn(&kv, &sq, reinterpret_cast<uint16_t *>(fake), 24,
                                    reinterpret_cast<int32_t *>(fake), 64, 0.1f, reinterpret_cast<float *>(fake),
                                    nullptr, fake, 1 << 30, s) == CSA2_ERR_INVALID_ARG);
  // layered calls: one bad layer rejects the whole call
  csa2_attn_layer layers[3];
  for (auto &l : layers)
    l = csa2_attn_layer{&kv, reinterpret_cast<uint16_t *>(fake), reinterpret_cast<int32_t *>(fake),
                        reinterpret_cast<float *>(fake), nullptr, nullptr, nullptr};
  csa2_kv_layer rope = kv;
  rope.rope_dim = 64;
  rope.rope = reinterpret_cast<uint16_t *>(fake);
  layers[2].layer = &rope;
  CHECK(csa2_sparse_fp4_decode_attn_layers(layers, 3, &sq, 64, 64, 0.1f, fake, 1 << 30, s) == CSA2_ERR_INVALID_ARG);
  CHECK(csa2_sparse_fp4_decode_attn_layers(layers, 0, &sq, 64, 64, 0.1f, fake, 1 << 30, s) == CSA2_ERR_INVALID_ARG);
  csa2_reindex_query rq[2] = {{fake, nullptr, reinterpret_cast<int32_t *>(fake)}, {fake, reinterpret_cast<float *>(fake),
                                                                                    reinterpret_cast<int32_t *>(fake)}};
  CHECK(csa2_index_reindex_layers(&kv, &sq, rq, 2, 64, tab, 2048, 8, fake, 1 << 30, s) == CSA2_ERR_INVALID_ARG);
  csa2_append app[2] = {{&kv, reinterpret_cast<float *>(fake), nullptr, fake}, {&kv, reinterpret_cast<float *>(fake),
                                                                                nullptr, nullptr}};
  CHECK(csa2_index_select_append(&kv, &sq, app, 2, fake, nullptr, 8, nullptr, 0, 0, reinterpret_cast<int32_t *>(fake),
                                 fake, 1 << 30, s) == CSA2_ERR_INVALID_ARG);  // two rows write one pool's codes
  CHECK(csa2_index_select_append(&kv, &sq, app, 9, fake, nullptr, 8, nullptr, 0, 0, reinterpret_cast<int32_t *>(fake),
                                 fake, 1 << 30, s) == CSA2_ERR_INVALID_ARG);
  csa2_kv_finish fin{reinterpret_cast<float *>(fake), 0.0f, 10000.0f, nullptr};
  CHECK(csa2_kv_finish_rows(reinterpret_cast<float *>(fake), 4, 1, 0, &fin, fake, fake, nullptr, nullptr, nullptr,
                            nullptr, s) == CSA2_ERR_INVALID_ARG);  // eps must be positive
  csa2_swa_window w{fake, reinterpret_cast<float *>(fake), 1};
  CHECK(csa2_swa_append(&w, tab, 2, reinterpret_cast<float *>(fake), s) == CSA2_ERR_INVALID_ARG);
  // the launch timer: unknown names are refused, NULL disarms
  CHECK(csa2_time_next_launch("no_such_kernel", fake, fake) == CSA2_ERR_INVALID_ARG);
  CHECK(csa2_time_next_launch("sparse_attn", nullptr, fake) == CSA2_ERR_INVALID_ARG);
  CHECK(csa2_time_next_launch(nullptr, nullptr, nullptr) == CSA2_OK);
  CHECK(csa2_timer_pending() == 0);
  CHECK(csa2_debug_flags(nullptr) == CSA2_ERR_INVALID_ARG);
}

static void block_pool() {
  CHECK(csa2_block_pool_create(-1) == nullptr);
  csa2_block_pool *p = csa2_block_pool_create(0);
  CHECK(p != nullptr && csa2_block_pool_num_free(p) == 0);
  int32_t id = 0;
  CHECK(csa2_block_alloc(p, 1, &id) == CSA2_ERR_INVALID_ARG);
  csa2_block_pool_destroy(p);
  csa2_block_pool_destroy(nullptr);

  const int N = 4096;
  p = csa2_block_pool_create(N);
  std::mt19937 rng(7);
  std::set<int32_t> held;
  std::vector<int32_t> buf(N + 8);
  for (int it = 0; it < 20000; ++it) {
    const int op = rng() % 4;
    if (op < 2) {  // take a random count; fails exactly when too few are free
      const int k = rng() % 64;
      const csa2_status st = csa2_block_alloc(p, k, buf.data());
      if (k > N - (int)held.size()) {
        CHECK(st == CSA2_ERR_INVALID_ARG);
      } else {
        CHECK(st == CSA2_OK);
        for (int i = 0; i < k; ++i) {
          CHECK(buf[i] >= 0 && buf[i] < N && held.count(buf[i]) == 0);
          held.insert(buf[i]);
        }
      }
    } else if (op == 2 && !held.empty()) {  // return a random subset
      std::vector<int32_t> v(held.begin(), held.end());
      std::shuffle(v.begin(), v.end(), rng);
      v.resize(1 + rng() % v.size());
      CHECK(csa2_block_free(p, (int32_t)v.size(), v.data()) == CSA2_OK);
      for (int32_t x : v) held.erase(x);
    } else {  // a bad return changes nothing: a free id, an out-of-range id, a duplicate
      int32_t badv[2] = {N, -1};
      CHECK(csa2_block_free(p, 1, badv) == CSA2_ERR_INVALID_ARG);
      CHECK(csa2_block_free(p, 1, badv + 1) == CSA2_ERR_INVALID_ARG);
      if (!held.empty()) {
        const int32_t h = *held.begin();
        int32_t dup[2] = {h, h};
        CHECK(csa2_block_free(p, 2, dup) == CSA2_ERR_INVALID_ARG);
      }
    }
    CHECK(csa2_block_pool_num_free(p) == N - (int)held.size());
  }
  csa2_block_pool_destroy(p);
}

int main() {
  validation();
  block_pool();
  if (g_fail) return 1;
  std::printf("abi host checks ok\n");
  return 0;
}
