// pa_alloc.cpp - host-side reference-counted allocator of a paged pool's physical block ids
// (declared in include/pa.h). Blocks are shared by sequences that fork from one another
// (beam search, parallel sampling) or that share a prompt prefix, and go back to the free
// list when their last sequence lets go (inferensys glossary "vLLM": PagedAttention entry,
// continuous batching entry). The allocator holds only host memory; copying a shared
// block before a write (pa_allocator_writable) and re-arming freed FP4 blocks
// (pa_reset_blocks) are the caller's device work.
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/pa.h"

struct pa_block_allocator {
  std::mutex mu;
  std::vector<int32_t> refs;   // reference count per block id, 0 = free
  std::vector<int32_t> stack;  // free ids; the back is handed out next
};

namespace {

bool in_range(const pa_block_allocator* a, int32_t id) {
  return id >= 0 && (size_t)id < a->refs.size();
}

// Checks ids[0..n) for range and use; with `need` set, also that every block has at least
// as many references as it has occurrences in the list. Returns a pa_status.
int check_ids(pa_block_allocator* a, const int32_t* ids, int32_t n, bool need) {
  for (int32_t i = 0; i < n; ++i) {
    if (!in_range(a, ids[i])) return PA_ERR_SHAPE;
    if (a->refs[ids[i]] == 0) return PA_ERR_STATE;
  }
  if (need) {
    std::vector<int32_t> sorted(ids, ids + n);
    std::sort(sorted.begin(), sorted.end());
    for (size_t i = 0; i < sorted.size();) {
      size_t j = i;
      while (j < sorted.size() && sorted[j] == sorted[i]) ++j;
      if ((int64_t)(j - i) > a->refs[sorted[i]]) return PA_ERR_STATE;
      i = j;
    }
  }
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_allocator_create(int32_t num_blocks, pa_block_allocator** out) {
  if (!out) return PA_ERR_NULL;
  *out = nullptr;
  if (num_blocks < 1) return PA_ERR_SHAPE;
  pa_block_allocator* a = new (std::nothrow) pa_block_allocator();
  if (!a) return PA_ERR_EXHAUSTED;
  try {
    a->refs.assign((size_t)num_blocks, 0);
    a->stack.resize((size_t)num_blocks);
  } catch (...) {
    delete a;
    return PA_ERR_EXHAUSTED;
  }
  for (int32_t i = 0; i < num_blocks; ++i) a->stack[i] = num_blocks - 1 - i;  // 0 on top
  *out = a;
  return PA_OK;
}

int pa_allocator_destroy(pa_block_allocator* a) {
  if (!a) return PA_ERR_NULL;
  delete a;
  return PA_OK;
}

int pa_allocator_alloc(pa_block_allocator* a, int32_t n, int32_t* ids_out) {
  if (!a) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  if (n == 0) return PA_OK;
  if (!ids_out) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(a->mu);
  if ((size_t)n > a->stack.size()) return PA_ERR_EXHAUSTED;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = a->stack.back();
    a->stack.pop_back();
    a->refs[id] = 1;
    ids_out[i] = id;
  }
  return PA_OK;
}

int pa_allocator_share(pa_block_allocator* a, const int32_t* ids, int32_t n) {
  if (!a) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  if (n == 0) return PA_OK;
  if (!ids) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(a->mu);
  int st = check_ids(a, ids, n, false);
  if (st != PA_OK) return st;
  for (int32_t i = 0; i < n; ++i)
    if (a->refs[ids[i]] > INT32_MAX - n) return PA_ERR_SHAPE;  // count would overflow
  for (int32_t i = 0; i < n; ++i) ++a->refs[ids[i]];
  return PA_OK;
}

int pa_allocator_release(pa_block_allocator* a, const int32_t* ids, int32_t n,
                         int32_t* freed_out, int32_t* num_freed) {
  if (!a) return PA_ERR_NULL;
  if (n < 0) return PA_ERR_SHAPE;
  if (num_freed) *num_freed = 0;
  if (n == 0) return PA_OK;
  if (!ids) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(a->mu);
  int st = check_ids(a, ids, n, true);
  if (st != PA_OK) return st;
  int32_t k = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t id = ids[i];
    if (--a->refs[id] == 0) {
      a->stack.push_back(id);
      if (freed_out) freed_out[k] = id;
      ++k;
    }
  }
  if (num_freed) *num_freed = k;
  return PA_OK;
}

int pa_allocator_writable(pa_block_allocator* a, int32_t id, int32_t* id_out) {
  if (!a || !id_out) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(a->mu);
  if (!in_range(a, id)) return PA_ERR_SHAPE;
  if (a->refs[id] == 0) return PA_ERR_STATE;
  if (a->refs[id] == 1) {
    *id_out = id;
    return 0;
  }
  if (a->stack.empty()) return PA_ERR_EXHAUSTED;
  const int32_t fresh = a->stack.back();
  a->stack.pop_back();
  a->refs[fresh] = 1;
  --a->refs[id];
  *id_out = fresh;
  return 1;
}

int pa_allocator_refcount(pa_block_allocator* a, int32_t id) {
  if (!a) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(a->mu);
  if (!in_range(a, id)) return PA_ERR_SHAPE;
  return a->refs[id];
}

int pa_allocator_num_free(pa_block_allocator* a) {
  if (!a) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(a->mu);
  return (int)a->stack.size();
}

}  // extern "C"
