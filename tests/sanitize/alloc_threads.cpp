// Concurrent use of the host block allocator (pa_allocator_*), for ThreadSanitizer: eight
// threads allocate, share, make writable (copy on write) and release blocks of one pool
// at once, as the host side of a serving loop with several scheduler threads would. At the
// end every block is free again and the counts add up. Prints "alloc_threads ok" and exits
// 0 on success. Test infrastructure only.
#include <stdint.h>
#include <stdio.h>

#include <atomic>
#include <thread>
#include <vector>

#include "../../include/pa.h"

int main() {
  const int32_t kBlocks = 4096, kThreads = 8, kRounds = 2000;
  pa_block_allocator* a = nullptr;
  if (pa_allocator_create(kBlocks, &a) != PA_OK) return 1;
  std::atomic<int> failures{0};
  std::vector<std::thread> th;
  for (int t = 0; t < kThreads; ++t) {
    th.emplace_back([&, t] {
      uint32_t x = 12345u + 977u * (uint32_t)t;  // per-thread LCG
      auto next = [&x] { return x = x * 1664525u + 1013904223u; };
      for (int r = 0; r < kRounds; ++r) {
        int32_t n = 1 + (int32_t)(next() % 8);
        int32_t ids[8];
        int st = pa_allocator_alloc(a, n, ids);
        if (st == PA_ERR_EXHAUSTED) continue;
        if (st != PA_OK) { ++failures; continue; }
        // share one block, then make it writable (copy on write): with two owners a new
        // block comes back and the original keeps one reference, which is dropped here
        const int32_t orig = ids[0];
        if (pa_allocator_share(a, &orig, 1) != PA_OK) ++failures;
        int32_t fresh = -1;
        const int w = pa_allocator_writable(a, orig, &fresh);
        if (w == 1) {
          ids[0] = fresh;
          if (pa_allocator_release(a, &orig, 1, nullptr, nullptr) != PA_OK) ++failures;
        } else if (w == PA_ERR_EXHAUSTED) {  // no copy: drop the extra reference instead
          if (pa_allocator_release(a, &orig, 1, nullptr, nullptr) != PA_OK) ++failures;
        } else {
          ++failures;
        }
        if (pa_allocator_refcount(a, ids[0]) < 1) ++failures;
        int32_t freed[8], nf = 0;
        if (pa_allocator_release(a, ids, n, freed, &nf) != PA_OK) ++failures;
        (void)pa_allocator_num_free(a);
      }
    });
  }
  for (auto& t : th) t.join();
  const int free_now = pa_allocator_num_free(a);
  pa_allocator_destroy(a);
  if (free_now != kBlocks) failures += 1000000;
  if (failures.load() != 0) {
    printf("alloc_threads: %d failed calls\n", failures.load());
    return 2;
  }
  printf("alloc_threads ok (%d blocks free of %d)\n", free_now, kBlocks);
  return 0;
}
