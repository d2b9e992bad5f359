// Host block manager: free list, reference counts, on-demand allocation,
// fork, copy-on-write decisions and release. Declared in include/pa.h.
//
// [L] "Paged Attention: OS-Inspired Memory Management for KV Caches":
//     "How PagedAttention works" (prefill takes just enough blocks, new tokens
//     go into the last block, one more block is taken only when a token's slot
//     lies past the last one, blocks go back to the free list when the request
//     ends), "Memory sharing across requests" (a count of users per block;
//     before a token is written into a block that others use, the writer gets
//     a copy of it, its table is repointed and the original's count drops).
//
// A sequence is its block table plus its token count: token t sits in table
// entry t / B at offset t % B, so the slot of the next token, and whether it
// needs a new block, follow from the count alone. Host memory only; no GPU
// call is made here. The device-side copy that a copy-on-write decision
// requires is reported as a (src, dst) pair for pa_copy_blocks.
#include <cstdint>
#include <functional>
#include <new>
#include <queue>
#include <vector>

#include "pa.h"
#include "pa_error.h"

struct pa_block_manager {
  struct Seq {
    bool live = false;
    std::vector<int32_t> table;   // physical block of logical block i
    int64_t tokens = 0;           // tokens written; the next one goes to position `tokens`
  };

  int num_blocks = 0;
  int block_size = 0;
  int max_blocks_per_seq = 0;
  std::vector<int32_t> users;     // sequences using each block (0 = free)
  // free blocks in a ring, oldest first: taken from the head, returned behind
  // the last one (every block is free at most once, so num_blocks slots suffice)
  std::vector<int32_t> ring;
  int64_t head = 0;
  int64_t n_free = 0;
  std::vector<Seq> seqs;
  // released sequence ids, smallest first
  std::priority_queue<int, std::vector<int>, std::greater<int>> spare_ids;

  int32_t take_block() {
    const int32_t b = ring[head];
    head = (head + 1) % num_blocks;
    --n_free;
    users[b] = 1;
    return b;
  }

  void return_block(int32_t b) {
    ring[(head + n_free) % num_blocks] = b;
    ++n_free;
  }

  int new_id() {
    if (!spare_ids.empty()) {
      const int id = spare_ids.top();
      spare_ids.pop();
      return id;
    }
    seqs.emplace_back();
    return (int)seqs.size() - 1;
  }

  bool valid(int id) const { return id >= 0 && id < (int)seqs.size() && seqs[id].live; }
};

namespace {

using pa::fail;
using pa::ok;

// Runs the body of an entry point that may allocate host memory: no C++
// exception crosses the C boundary; running out of memory becomes a status.
template <class F>
pa_status guarded(const char* fn, F&& body) {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    return fail(PA_ERR_EXHAUSTED, "%s: out of host memory", fn);
  } catch (...) {
    return fail(PA_ERR_STATE, "%s: internal error", fn);
  }
}

}  // namespace

extern "C" {

pa_status pa_bm_create(int num_blocks, int block_size, int max_blocks_per_seq,
                       pa_block_manager** out) {
  if (!out) return fail(PA_ERR_NULL, "pa_bm_create: out is NULL");
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0 || max_blocks_per_seq < 0)
    return fail(PA_ERR_SHAPE, "pa_bm_create: num_blocks=%d block_size=%d max_blocks_per_seq=%d",
                num_blocks, block_size, max_blocks_per_seq);
  return guarded("pa_bm_create", [&]() {
    pa_block_manager* bm = new pa_block_manager();
    try {
      bm->num_blocks = num_blocks;
      bm->block_size = block_size;
      bm->max_blocks_per_seq = max_blocks_per_seq > 0 ? max_blocks_per_seq : num_blocks;
      bm->users.assign(num_blocks, 0);
      bm->ring.resize(num_blocks);
      for (int b = 0; b < num_blocks; ++b) bm->ring[b] = b;
      bm->n_free = num_blocks;
    } catch (...) {
      delete bm;
      throw;
    }
    *out = bm;
    return ok();
  });
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

pa_status pa_bm_add_sequence(pa_block_manager* bm, int* seq_id) {
  if (!bm || !seq_id) return fail(PA_ERR_NULL, "pa_bm_add_sequence: null argument");
  return guarded("pa_bm_add_sequence", [&]() {
    const int id = bm->new_id();
    bm->seqs[id] = pa_block_manager::Seq();
    bm->seqs[id].live = true;
    *seq_id = id;
    return ok();
  });
}

pa_status pa_bm_fork(pa_block_manager* bm, int parent, int* child) {
  if (!bm || !child) return fail(PA_ERR_NULL, "pa_bm_fork: null argument");
  if (!bm->valid(parent)) return fail(PA_ERR_STATE, "pa_bm_fork: no live sequence %d", parent);
  return guarded("pa_bm_fork", [&]() {
    // the child is built completely before any reference count changes, so a
    // failed allocation leaves the manager as it was
    pa_block_manager::Seq c;
    c.live = true;
    c.table = bm->seqs[parent].table;
    c.tokens = bm->seqs[parent].tokens;
    const int id = bm->new_id();
    for (int32_t b : c.table) bm->users[b] += 1;
    bm->seqs[id] = std::move(c);
    *child = id;
    return ok();
  });
}

pa_status pa_bm_append_tokens(pa_block_manager* bm, const int* seq_ids, int n, int64_t* slots,
                              int32_t* copy_pairs, int max_copies, int* n_copies,
                              int* n_applied) {
  if (!bm || !n_copies || !n_applied || (n > 0 && (!seq_ids || !slots)))
    return fail(PA_ERR_NULL, "pa_bm_append_tokens: null argument");
  *n_copies = 0;
  *n_applied = 0;
  if (n < 0 || max_copies < 0) return fail(PA_ERR_SHAPE, "pa_bm_append_tokens: n=%d", n);
  if (max_copies > 0 && !copy_pairs)
    return fail(PA_ERR_NULL, "pa_bm_append_tokens: copy_pairs is NULL");
  const int B = bm->block_size;
  return guarded("pa_bm_append_tokens", [&]() {
    for (int i = 0; i < n; ++i) {
      const int id = seq_ids[i];
      if (!bm->valid(id)) return fail(PA_ERR_STATE, "pa_bm_append_tokens: no live sequence %d", id);
      pa_block_manager::Seq& q = bm->seqs[id];
      const int64_t j = q.tokens / B;          // table entry of the new token
      const int32_t off = (int32_t)(q.tokens % B);
      if (j == (int64_t)q.table.size()) {
        // the position lies past the last block: allocate on demand
        if ((int)q.table.size() >= bm->max_blocks_per_seq)
          return fail(PA_ERR_STATE, "pa_bm_append_tokens: sequence %d has %d blocks (maximum)", id,
                      (int)q.table.size());
        if (bm->n_free == 0)
          return fail(PA_ERR_EXHAUSTED, "pa_bm_append_tokens: no free block (token %d)", i);
        q.table.reserve(q.table.size() + 1);   // may throw: before the block leaves the ring
        q.table.push_back(bm->take_block());
      } else if (bm->users[q.table[j]] > 1) {
        // the block is shared: the writer gets its own copy first
        if (bm->n_free == 0)
          return fail(PA_ERR_EXHAUSTED, "pa_bm_append_tokens: no free block for a copy (token %d)", i);
        if (*n_copies >= max_copies)
          return fail(PA_ERR_SHAPE, "pa_bm_append_tokens: more than %d copies", max_copies);
        const int32_t shared = q.table[j];
        const int32_t own = bm->take_block();
        bm->users[shared] -= 1;
        copy_pairs[2 * *n_copies] = shared;
        copy_pairs[2 * *n_copies + 1] = own;
        *n_copies += 1;
        q.table[j] = own;
      }
      slots[i] = (int64_t)q.table[j] * B + off;
      q.tokens += 1;
      *n_applied = i + 1;
    }
    return ok();
  });
}

pa_status pa_bm_release(pa_block_manager* bm, int seq_id, int* n_freed) {
  if (!bm) return fail(PA_ERR_NULL, "pa_bm_release: null manager");
  if (!bm->valid(seq_id)) return fail(PA_ERR_STATE, "pa_bm_release: no live sequence %d", seq_id);
  return guarded("pa_bm_release", [&]() {
    bm->spare_ids.push(seq_id);   // first: a failed push leaves the sequence as it was
    pa_block_manager::Seq& q = bm->seqs[seq_id];
    int freed = 0;
    for (int32_t b : q.table) {
      if (--bm->users[b] == 0) {
        bm->return_block(b);
        ++freed;
      }
    }
    q = pa_block_manager::Seq();
    if (n_freed) *n_freed = freed;
    return ok();
  });
}

pa_status pa_bm_get_table(const pa_block_manager* bm, int seq_id, int32_t* row, int max_len,
                          int* n_blocks, int64_t* num_tokens) {
  if (!bm || !n_blocks) return fail(PA_ERR_NULL, "pa_bm_get_table: null argument");
  if (!bm->valid(seq_id)) return fail(PA_ERR_STATE, "pa_bm_get_table: no live sequence %d", seq_id);
  const pa_block_manager::Seq& q = bm->seqs[seq_id];
  const int nb = (int)q.table.size();
  *n_blocks = nb;
  if (num_tokens) *num_tokens = q.tokens;
  if (!row && max_len == 0) return ok();   // size query
  if (nb > 0 && (!row || max_len < nb))
    return fail(PA_ERR_SHAPE, "pa_bm_get_table: row holds %d entries, table has %d", max_len, nb);
  for (int j = 0; j < nb; ++j) row[j] = q.table[j];
  return ok();
}

pa_status pa_bm_export(const pa_block_manager* bm, const int* seq_ids, int n, int32_t* tables,
                       int MB, int32_t* context_lens) {
  if (!bm || (n > 0 && (!seq_ids || !tables || !context_lens)))
    return fail(PA_ERR_NULL, "pa_bm_export: null argument");
  if (n < 0 || MB <= 0) return fail(PA_ERR_SHAPE, "pa_bm_export: n=%d MB=%d", n, MB);
  for (int i = 0; i < n; ++i) {
    const int id = seq_ids[i];
    if (!bm->valid(id)) return fail(PA_ERR_STATE, "pa_bm_export: no live sequence %d", id);
    const pa_block_manager::Seq& q = bm->seqs[id];
    if ((int)q.table.size() > MB)
      return fail(PA_ERR_SHAPE, "pa_bm_export: sequence %d has %d blocks > MB=%d", id,
                  (int)q.table.size(), MB);
    if (q.tokens > INT32_MAX) return fail(PA_ERR_SHAPE, "pa_bm_export: sequence %d too long", id);
    int32_t* row = tables + (int64_t)i * MB;
    for (int j = 0; j < MB; ++j) row[j] = j < (int)q.table.size() ? q.table[j] : -1;
    context_lens[i] = (int32_t)q.tokens;
  }
  return ok();
}

int pa_bm_num_free(const pa_block_manager* bm) { return bm ? (int)bm->n_free : -1; }

int pa_bm_refcount(const pa_block_manager* bm, int block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->users[block];
}

}  // extern "C"
