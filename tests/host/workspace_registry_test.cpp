// Host test of the split workspace registry (workspace.h) with a fake
// allocator: growth keeps the smaller buffer alive, release frees every
// buffer exactly once, and two threads on one key hold it one after the
// other.  Built with g++ by tests/test_workspace_host.py; prints "ok".
#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <set>
#include <thread>
#include <vector>

#include "workspace.h"

namespace {

struct FakeAlloc {
  std::set<void*>* live;
  int* frees;
  int* fail_next;
  void* alloc(int64_t bytes) {
    if (*fail_next) {
      --*fail_next;
      return nullptr;
    }
    void* p = std::malloc(size_t(bytes));
    live->insert(p);
    return p;
  }
  bool free(void* p) {
    if (!live->erase(p)) {
      std::printf("double or foreign free\n");
      std::exit(1);
    }
    ++*frees;
    std::free(p);
    return true;
  }
};

#define CHECK(c)                                                  \
  do {                                                            \
    if (!(c)) {                                                   \
      std::printf("check failed line %d: %s\n", __LINE__, #c);    \
      std::exit(1);                                               \
    }                                                             \
  } while (0)

}  // namespace

int main() {
  std::set<void*> live;
  int frees = 0, fail_next = 0;
  using Reg = ppa::WorkspaceRegistry<int, FakeAlloc>;
  Reg reg(FakeAlloc{&live, &frees, &fail_next});

  // growth: a larger request gets a new buffer, the old one stays allocated
  void* p1;
  {
    Reg::Lease l;
    CHECK(reg.acquire(7, 1000, &l) && l.held());
    p1 = l.ptr();
  }
  CHECK(reg.capacity(7) == 1000);
  {
    Reg::Lease l;
    CHECK(reg.acquire(7, 500, &l));   // smaller: same buffer
    CHECK(l.ptr() == p1);
  }
  void* p2;
  {
    Reg::Lease l;
    CHECK(reg.acquire(7, 4000, &l));
    p2 = l.ptr();
  }
  CHECK(p2 != p1 && reg.capacity(7) == 4000);
  CHECK(live.count(p1) == 1 && live.count(p2) == 1 && frees == 0);
  CHECK(reg.live_buffers() == 2);

  // a failed allocation leaves the current buffer in place and the lease unheld
  fail_next = 1;
  {
    Reg::Lease l;
    CHECK(!reg.acquire(7, 8000, &l) && !l.held());
  }
  CHECK(reg.capacity(7) == 4000 && live.count(p2) == 1);

  // keys are independent
  {
    Reg::Lease a, b;
    CHECK(reg.acquire(1, 64, &a) && reg.acquire(2, 64, &b));
    CHECK(a.ptr() != b.ptr());
  }

  // two threads on one key: the second waits until the first lease ends, and
  // the first thread's growth does not free what it hands out
  std::atomic<int> phase{0};
  std::atomic<bool> second_got_it_early{false};
  void* first_ptr = nullptr;
  std::thread t1([&] {
    Reg::Lease l;
    CHECK(reg.acquire(9, 100, &l));
    first_ptr = l.ptr();
    phase = 1;
    std::this_thread::sleep_for(std::chrono::milliseconds(200));
    // still the owner: the buffer it holds is still allocated
    CHECK(live.count(first_ptr) == 1);
    phase = 2;
  });
  std::thread t2([&] {
    while (phase.load() < 1) std::this_thread::yield();
    Reg::Lease l;
    CHECK(reg.acquire(9, 100000, &l));   // grows, must wait for t1
    if (phase.load() < 2) second_got_it_early = true;
  });
  t1.join();
  t2.join();
  CHECK(!second_got_it_early.load());
  CHECK(live.count(first_ptr) == 1);   // retired, not freed
  CHECK(reg.capacity(9) == 100000);

  // release frees every buffer (current and retired) exactly once
  const int64_t n = reg.live_buffers();
  CHECK(n == int64_t(live.size()));
  CHECK(reg.release_all());
  CHECK(live.empty() && frees == n);
  CHECK(reg.capacity(7) == 0 && reg.live_buffers() == 0);
  std::printf("ok\n");
  return 0;
}
