// Host-side checks of the C ABI, built together with ra_api.cpp and the launcher stand-ins
// under the sanitizers (see tests/test_host_sanitizers.py). Every call runs its argument
// validation; calls with valid arguments go on to fill the kernel arguments and reach a
// launcher, which reports "no device" (RA_ERR_HIP). The planner counts are compared with
// counts from a direct position rule written here. Exit status 0 when every check holds.
#include <stdio.h>
#include <string.h>

#include <thread>
#include <vector>

#include "ra.h"

static int g_fail = 0;
#define CHECK(cond)                                                    \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                        \
    }                                                                  \
  } while (0)

static void* const FAKE = (void*)0x10000;

// Global position of local row i (contiguous: r*S + i; striped: i*N + r; zigzag: chunks r and
// 2N-1-r of length L/(2N)), written out here independently of the library.
static long long pos(int assign, int n, int r, long long L, long long i) {
  const long long S = L / n, C = L / (2 * n);
  if (assign == RA_STRIPED) return i * n + r;
  if (assign == RA_ZIGZAG) return i < C ? r * C + i : (2LL * n - 1 - r) * C + (i - C);
  return r * S + i;
}

static void planner_counts() {
  const int assigns[3] = {RA_CONTIGUOUS, RA_STRIPED, RA_ZIGZAG};
  const int ns[3] = {1, 3, 4};
  for (int a : assigns)
    for (int n : ns) {
      const long long L = 2LL * n * 24;
      const long long S = L / n;
      for (int r = 0; r < n; ++r)
        for (int src = 0; src < n; ++src) {
          ra_shard q = {a, n, r, L}, k = {a, n, src, L};
          int64_t out[4] = {0, 0, 0, 0};
          CHECK(ra_share_work(&q, &k, S, S, 1, 7, 5, out) == RA_OK);
          long long pairs = 0, full = 0, part = 0, skip = 0;
          for (long long i = 0; i < S; ++i)
            for (long long j = 0; j < S; ++j) pairs += pos(a, n, src, L, j) <= pos(a, n, r, L, i);
          for (long long i0 = 0; i0 < S; i0 += 7)
            for (long long j0 = 0; j0 < S; j0 += 5) {
              long long vis = 0, all = 0;
              for (long long i = i0; i < i0 + 7 && i < S; ++i)
                for (long long j = j0; j < j0 + 5 && j < S; ++j) {
                  ++all;
                  vis += pos(a, n, src, L, j) <= pos(a, n, r, L, i);
                }
              if (vis == 0) ++skip;
              else if (vis == all) ++full;
              else ++part;
            }
          CHECK(out[0] == pairs && out[1] == full && out[2] == part && out[3] == skip);
        }
    }
}

static void validation() {
  // block attention
  CHECK(ra_block_attn_fwd(FAKE, FAKE, FAKE, FAKE, (float*)FAKE, 1, 2, 2, 64, 64, 96, 1, 1, 0, 0, 0, 0.f, 0) ==
        RA_ERR_UNSUPPORTED);
  CHECK(strlen(ra_last_error()) > 0);
  CHECK(ra_block_attn_fwd(FAKE, FAKE, FAKE, FAKE, (float*)FAKE, 1, 6, 4, 64, 64, 128, 1, 1, 0, 0, 0, 0.f, 0) ==
        RA_ERR_SHAPE);
  CHECK(ra_block_attn_fwd(0, 0, 0, 0, 0, 0, 2, 2, 64, 64, 128, 1, 1, 0, 0, 0, 0.f, 0) == RA_OK);
  CHECK(ra_block_attn_fwd(FAKE, FAKE, FAKE, FAKE, (float*)FAKE, 1, 2, 2, 64, 64, 128, 1, 1, 0, 0, 0, 0.f, 0) ==
        RA_ERR_HIP);
  // causal block call: shard descriptors must match the sizes
  ra_shard qs = {RA_ZIGZAG, 4, 1, 256}, ks = {RA_ZIGZAG, 4, 3, 256};
  CHECK(ra_block_attn_fwd(FAKE, FAKE, FAKE, FAKE, (float*)FAKE, 1, 2, 2, 64, 64, 128, 1, 0, 1, &qs, &ks, 0.f, 0) ==
        RA_ERR_HIP);
  ks.global_len = 250;
  CHECK(ra_block_attn_fwd(FAKE, FAKE, FAKE, FAKE, (float*)FAKE, 1, 2, 2, 64, 64, 128, 1, 0, 1, &qs, &ks, 0.f, 0) ==
        RA_ERR_SHAPE);

  // ring share, every ring size up to the limit (fills all per-step slots of the kernel arguments)
  std::vector<const void*> shares(RA_MAX_WORLD + 1, FAKE);
  for (int n = 1; n <= RA_MAX_WORLD; ++n)
    CHECK(ra_ring_share(FAKE, shares.data(), shares.data(), FAKE, (float*)FAKE, 1, 2, 2, 64, 128, n, n - 1,
                        RA_STRIPED, 1, RA_BF16, RA_BF16, 0.f, 0, n, 0, 0, 0) == RA_ERR_HIP);
  CHECK(ra_ring_share(FAKE, shares.data(), shares.data(), FAKE, (float*)FAKE, 1, 2, 2, 64, 128, RA_MAX_WORLD + 1, 0,
                      RA_STRIPED, 1, RA_BF16, RA_BF16, 0.f, 0, RA_MAX_WORLD + 1, 0, 0, 0) == RA_ERR_UNSUPPORTED);
  // a resume needs a state this process stored in the workspace
  const size_t wsb = ra_ring_share_workspace_bytes(1, 2, 64, 128);
  CHECK(ra_ring_share(FAKE, shares.data(), shares.data(), FAKE, (float*)FAKE, 1, 2, 2, 64, 128, 4, 1, RA_ZIGZAG, 1,
                      RA_BF16, RA_BF16, 0.f, 2, 2, FAKE, wsb, 0) == RA_ERR_INVALID_ARG);
  // a partial run that fails to launch stores no state
  CHECK(ra_ring_share(FAKE, shares.data(), shares.data(), FAKE, (float*)FAKE, 1, 2, 2, 64, 128, 4, 1, RA_ZIGZAG, 1,
                      RA_BF16, RA_BF16, 0.f, 0, 2, FAKE, wsb, 0) == RA_ERR_HIP);
  CHECK(ra_ring_share(FAKE, shares.data(), shares.data(), FAKE, (float*)FAKE, 1, 2, 2, 64, 128, 4, 1, RA_ZIGZAG, 1,
                      RA_BF16, RA_BF16, 0.f, 2, 2, FAKE, wsb, 0) == RA_ERR_INVALID_ARG);

  // backward and its allocation-free form
  std::vector<float*> grads(RA_MAX_WORLD, (float*)FAKE);
  CHECK(ra_ring_share_bwd(FAKE, shares.data(), shares.data(), FAKE, (float*)FAKE, FAKE, (float*)FAKE, grads.data(),
                          grads.data(), 1, 2, 2, 64, 128, 8, 3, RA_ZIGZAG, 1, RA_BF16, 0.f, FAKE, 1 << 20, 0) ==
        RA_ERR_HIP);
  CHECK(ra_ring_share_bwd_noalloc(FAKE, shares.data(), shares.data(), FAKE, (float*)FAKE, FAKE, (float*)FAKE,
                                  grads.data(), grads.data(), 1, 64, 64, 65600, 128, 2, 0, RA_CONTIGUOUS, 1, RA_BF16,
                                  0.f, 0) == RA_ERR_UNSUPPORTED);
  CHECK(ra_ring_share_bwd_noalloc(FAKE, shares.data(), shares.data(), FAKE, (float*)FAKE, FAKE, (float*)FAKE,
                                  grads.data(), grads.data(), 1, 2, 2, 64, 128, 8, 3, RA_ZIGZAG, 1, RA_BF16, 0.f, 0) ==
        RA_ERR_HIP);

  // merge and permutes
  CHECK(ra_lse_merge(FAKE, (float*)FAKE, FAKE, (float*)FAKE, 1, 2, 4, 12, 1, 1, 0) == RA_ERR_UNSUPPORTED);
  CHECK(ra_lse_merge(FAKE, (float*)FAKE, FAKE, (float*)FAKE, 1, 2, 4, 16, 1, 0, 0) == RA_ERR_HIP);
  CHECK(ra_seq2head_permute(FAKE, FAKE, 1, 4, 8, 6, 128, 1, 0, 0, 0) == RA_ERR_SHAPE);
  CHECK(ra_seq2head_permute(FAKE, FAKE, 1, 4, 8, 8, 128, 1, -1, 1, 0) == RA_ERR_HIP);
  std::vector<void*> outs(RA_MAX_PERMUTE, FAKE);
  CHECK(ra_seq2head_permute_n(shares.data(), outs.data(), RA_MAX_PERMUTE, 1, 4, 8, 8, 128, 1, 2, 0, 0) == RA_ERR_HIP);
  CHECK(ra_seq2head_permute_n(shares.data(), outs.data(), RA_MAX_PERMUTE + 1, 1, 4, 8, 8, 128, 1, 2, 0, 0) ==
        RA_ERR_INVALID_ARG);

  // debug hooks
  CHECK(ra_debug_tile_count_slots(2, 3, 300) == 3 * 2 * 3 * 32);
  CHECK(ra_debug_tile_counts(FAKE, shares.data(), shares.data(), FAKE, (float*)FAKE, 1, 2, 2, 64, 128, 4, 0,
                             RA_STRIPED, 1, RA_BF16, 0.f, (int32_t*)FAKE, 1, 0) == RA_ERR_INVALID_ARG);
  ra_shard p = {RA_ZIGZAG, 8, 3, 262144};
  CHECK(ra_debug_positions(&p, (int64_t*)FAKE, 0) == RA_ERR_HIP);
  int64_t bm = 0, bn = 0;
  CHECK(ra_tile_shape(RA_BF16, 128, &bm, &bn) == RA_OK && bm == 128 && bn == 64);
}

// The error text is thread-local and the workspace records are shared: hammer both from threads.
static void threads() {
  std::vector<std::thread> ts;
  for (int t = 0; t < 8; ++t)
    ts.emplace_back([t] {
      std::vector<const void*> shares(4, FAKE);
      for (int it = 0; it < 200; ++it) {
        const int rc = ra_block_attn_fwd(FAKE, FAKE, FAKE, FAKE, (float*)FAKE, 1, 2, 2, 64, 64, t % 2 ? 96 : 128, 1,
                                         1, 0, 0, 0, 0.f, 0);
        CHECK(rc == (t % 2 ? RA_ERR_UNSUPPORTED : RA_ERR_HIP));
        CHECK(strlen(ra_last_error()) > 0);
        CHECK(ra_ring_share(FAKE, shares.data(), shares.data(), FAKE, (float*)FAKE, 1, 2, 2, 64, 128, 4, 1,
                            RA_CONTIGUOUS, 1, RA_BF16, RA_BF16, 0.f, 1, 3, (void*)(uintptr_t)(0x100000 * (t + 1)),
                            1 << 20, 0) == RA_ERR_INVALID_ARG);
      }
    });
  for (auto& t : ts) t.join();
}

int main() {
  planner_counts();
  validation();
  threads();
  if (g_fail) fprintf(stderr, "%d checks failed\n", g_fail);
  else printf("abi host checks: all passed\n");
  return g_fail ? 1 : 0;
}
