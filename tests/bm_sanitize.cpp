// Host-only test program for the native block manager under AddressSanitizer and
// UndefinedBehaviorSanitizer (built with g++ by tests/test_block_manager_sanitized.py,
// together with csrc/block_manager.cpp; no GPU code).
//
// A seeded random sequence of operations (add, fork, append batches, release,
// table and export reads, and calls the header defines as errors) runs against
// the C ABI. After every operation the manager's observable state is checked
// against a model kept here: per-block reference counts equal the number of
// live tables holding the block, the free count equals the blocks with count
// zero, a table has ceil(tokens / B) entries, every returned slot lies in its
// sequence's block for that position, and each copy pair names a block that
// was shared and a block that was free. A failed append applies exactly the
// tokens it reports. Exit status 0 and "bm_sanitize: ok" on success.
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>

#include "pa.h"
#include "pa_error.h"

// The library's error recorder lives in api.hip, which is GPU code; this
// host-only build records the detail the same way.
namespace pa {
static char g_err[512];
pa_status fail(pa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}
pa_status ok() {
  g_err[0] = '\0';
  return PA_OK;
}
}  // namespace pa

namespace {

int g_failures = 0;

#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      std::fprintf(stderr, "CHECK failed: %s: ", #cond);   \
      std::fprintf(stderr, __VA_ARGS__);                   \
      std::fprintf(stderr, "\n");                          \
      if (++g_failures > 20) std::exit(1);                 \
    }                                                      \
  } while (0)

struct Model {
  int NB, B, MB;
  std::map<int, int64_t> tokens;   // live sequence -> token count
};

void check_state(pa_block_manager* bm, const Model& md, int step) {
  std::vector<int> users(md.NB, 0);
  std::vector<int32_t> row(md.MB + 1);
  for (const auto& kv : md.tokens) {
    int nb = -1;
    int64_t nt = -1;
    const pa_status st = pa_bm_get_table(bm, kv.first, row.data(), md.MB + 1, &nb, &nt);
    CHECK(st == PA_OK, "step %d: get_table(%d) status %d", step, kv.first, (int)st);
    if (st != PA_OK) continue;
    CHECK(nt == kv.second, "step %d: seq %d tokens %lld, model %lld", step, kv.first,
          (long long)nt, (long long)kv.second);
    CHECK(nb == (int)((kv.second + md.B - 1) / md.B), "step %d: seq %d has %d blocks for %lld tokens",
          step, kv.first, nb, (long long)kv.second);
    for (int j = 0; j < nb; ++j) {
      CHECK(row[j] >= 0 && row[j] < md.NB, "step %d: block %d out of the pool", step, row[j]);
      if (row[j] >= 0 && row[j] < md.NB) users[row[j]] += 1;
    }
  }
  int free_blocks = 0;
  for (int b = 0; b < md.NB; ++b) {
    CHECK(pa_bm_refcount(bm, b) == users[b], "step %d: block %d refcount %d, tables hold it %d times",
          step, b, pa_bm_refcount(bm, b), users[b]);
    free_blocks += users[b] == 0;
  }
  CHECK(pa_bm_num_free(bm) == free_blocks, "step %d: %d free, %d blocks unused", step,
        pa_bm_num_free(bm), free_blocks);
}

void run(uint64_t seed, int NB, int B, int MB, int steps) {
  std::mt19937_64 rng(seed);
  auto pick = [&](int n) { return (int)(rng() % (uint64_t)n); };
  pa_block_manager* bm = nullptr;
  CHECK(pa_bm_create(NB, B, MB, &bm) == PA_OK && bm, "create NB=%d B=%d MB=%d", NB, B, MB);
  if (!bm) return;
  Model md{NB, B, MB, {}};
  std::vector<int32_t> row(MB + 1);
  for (int step = 0; step < steps; ++step) {
    std::vector<int> live;
    for (const auto& kv : md.tokens) live.push_back(kv.first);
    const int op = pick(100);
    if (op < 10 || live.empty()) {   // a new sequence
      int id = -1;
      CHECK(pa_bm_add_sequence(bm, &id) == PA_OK && id >= 0, "step %d: add", step);
      CHECK(!md.tokens.count(id), "step %d: id %d handed out while live", step, id);
      md.tokens[id] = 0;
    } else if (op < 18) {            // fork a live sequence
      const int parent = live[pick((int)live.size())];
      int child = -1;
      CHECK(pa_bm_fork(bm, parent, &child) == PA_OK, "step %d: fork %d", step, parent);
      CHECK(!md.tokens.count(child), "step %d: fork id %d handed out while live", step, child);
      md.tokens[child] = md.tokens[parent];
    } else if (op < 26) {            // release a live sequence
      const int id = live[pick((int)live.size())];
      int freed = -1;
      CHECK(pa_bm_release(bm, id, &freed) == PA_OK && freed >= 0, "step %d: release %d", step, id);
      md.tokens.erase(id);
      CHECK(pa_bm_release(bm, id, &freed) == PA_ERR_STATE, "step %d: second release of %d", step, id);
    } else if (op < 90) {            // append to a batch (a sequence may appear more than once)
      const int n = 1 + pick(12);
      std::vector<int> ids(n);
      for (int i = 0; i < n; ++i) ids[i] = live[pick((int)live.size())];
      const int max_copies = pick(4) == 0 ? pick(2) : n;   // sometimes too little room for copies
      std::vector<int64_t> slots(n, -7);
      std::vector<int32_t> pairs(2 * (max_copies > 0 ? max_copies : 1), -7);
      // model: the block each token will land in, and which blocks are shared
      std::vector<int> refs(NB);
      for (int b = 0; b < NB; ++b) refs[b] = pa_bm_refcount(bm, b);
      int n_copies = -1, n_applied = -1;
      const pa_status st = pa_bm_append_tokens(bm, ids.data(), n, slots.data(),
                                               max_copies > 0 ? pairs.data() : nullptr, max_copies,
                                               &n_copies, &n_applied);
      CHECK(st == PA_OK || st == PA_ERR_EXHAUSTED || st == PA_ERR_STATE || st == PA_ERR_SHAPE,
            "step %d: append status %d", step, (int)st);
      CHECK(n_applied >= 0 && n_applied <= n && (st != PA_OK || n_applied == n),
            "step %d: applied %d of %d, status %d", step, n_applied, n, (int)st);
      CHECK(n_copies >= 0 && n_copies <= (max_copies > 0 ? max_copies : 0), "step %d: %d copies",
            step, n_copies);
      for (int c = 0; c < n_copies; ++c) {
        const int src = pairs[2 * c], dst = pairs[2 * c + 1];
        CHECK(src >= 0 && src < NB && dst >= 0 && dst < NB && src != dst, "step %d: pair (%d, %d)",
              step, src, dst);
        if (src >= 0 && src < NB && dst >= 0 && dst < NB) {
          CHECK(refs[src] > 1, "step %d: copied block %d was not shared", step, src);
          CHECK(refs[dst] == 0, "step %d: copy target %d was in use", step, dst);
          refs[dst] = 1;   // a later pair in this call may not reuse it
          refs[src] -= 1;
        }
      }
      for (int i = 0; i < n_applied; ++i) {
        const int id = ids[i];
        const int64_t t = md.tokens[id];
        md.tokens[id] = t + 1;
        int nb = 0;
        CHECK(pa_bm_get_table(bm, id, row.data(), MB + 1, &nb, nullptr) == PA_OK, "step %d", step);
        const int64_t j = t / B;
        CHECK(j < nb && slots[i] == (int64_t)row[j] * B + t % B,
              "step %d: token %d of seq %d at slot %lld, table entry %lld of %d", step, i, id,
              (long long)slots[i], (long long)j, nb);
      }
    } else if (op < 95) {            // export a batch of live sequences
      const int n = 1 + pick((int)live.size());
      std::vector<int> ids(n);
      for (int i = 0; i < n; ++i) ids[i] = live[pick((int)live.size())];
      const int mb = 1 + pick(MB);
      std::vector<int32_t> tables((size_t)n * mb, -9), lens(n, -9);
      const pa_status st = pa_bm_export(bm, ids.data(), n, tables.data(), mb, lens.data());
      bool fits = true;
      for (int i = 0; i < n; ++i) fits = fits && (md.tokens[ids[i]] + B - 1) / B <= mb;
      CHECK(st == (fits ? PA_OK : PA_ERR_SHAPE), "step %d: export status %d (fits %d)", step,
            (int)st, (int)fits);
      if (st == PA_OK) {
        for (int i = 0; i < n; ++i) {
          int nb = 0;
          CHECK(pa_bm_get_table(bm, ids[i], row.data(), MB + 1, &nb, nullptr) == PA_OK, "step %d", step);
          CHECK(lens[i] == md.tokens[ids[i]], "step %d: exported length", step);
          for (int j = 0; j < mb; ++j)
            CHECK(tables[(size_t)i * mb + j] == (j < nb ? row[j] : -1), "step %d: exported entry", step);
        }
      }
    } else {                         // calls the header defines as errors
      int out = 0, nb = 0;
      int64_t slot = 0;
      int nc = 0, na = 0;
      const int dead = 1000000 + pick(1000);
      CHECK(pa_bm_fork(bm, dead, &out) == PA_ERR_STATE, "step %d: fork of a dead id", step);
      CHECK(pa_bm_append_tokens(bm, &dead, 1, &slot, nullptr, 0, &nc, &na) == PA_ERR_STATE && na == 0,
            "step %d: append to a dead id", step);
      CHECK(pa_bm_get_table(bm, -1, row.data(), MB, &nb, nullptr) == PA_ERR_STATE, "step %d", step);
      CHECK(pa_bm_append_tokens(bm, nullptr, 1, &slot, nullptr, 0, &nc, &na) == PA_ERR_NULL,
            "step %d: null ids", step);
      CHECK(pa_bm_export(bm, &live[0], 1, row.data(), 0, &out) == PA_ERR_SHAPE, "step %d", step);
      CHECK(pa_bm_refcount(bm, NB) == -1 && pa_bm_refcount(bm, -1) == -1, "step %d", step);
    }
    check_state(bm, md, step);
  }
  for (const auto& kv : md.tokens) pa_bm_release(bm, kv.first, nullptr);
  CHECK(pa_bm_num_free(bm) == NB, "all blocks back after releasing every sequence");
  pa_bm_destroy(bm);
}

}  // namespace

int main(int argc, char** argv) {
  const int rounds = argc > 1 ? std::atoi(argv[1]) : 12;
  pa_block_manager* bad = reinterpret_cast<pa_block_manager*>(1);
  CHECK(pa_bm_create(0, 16, 0, &bad) == PA_ERR_SHAPE && bad == nullptr, "create with no blocks");
  CHECK(pa_bm_create(8, 16, 0, nullptr) == PA_ERR_NULL, "create with no out pointer");
  for (int r = 0; r < rounds; ++r) {
    const int NB = 4 + 13 * (r % 5);        // small pools: exhaustion and copy-on-write are common
    const int B = (r % 3 == 0) ? 1 : (r % 3 == 1 ? 4 : 16);
    const int MB = 2 + (r % 7);
    run(1000 + r, NB, B, MB, 4000);
  }
  if (g_failures) {
    std::fprintf(stderr, "bm_sanitize: %d failed checks\n", g_failures);
    return 1;
  }
  std::printf("bm_sanitize: ok (%d rounds)\n", rounds);
  return 0;
}
