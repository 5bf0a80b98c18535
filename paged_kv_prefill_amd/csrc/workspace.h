// Split workspace registry: one grow-only device buffer per (device, stream).
// HIP-free (the allocator is a template parameter) so that its locking and
// lifetime rules are tested on the host with a fake allocator.
//
// Rules:
//  * A call holds its stream's entry (a Lease) from the moment it takes the
//    buffer until its last kernel is enqueued.  Two host threads calling on
//    one stream therefore enqueue whole calls one after the other: one call's
//    split partials are never overwritten by another call's attention kernel
//    before its own merge kernel has read them (the stream runs them in
//    enqueue order).
//  * Growing never frees the smaller buffer: it is retired and kept until
//    release_all().  Work already enqueued, and HIP graphs captured earlier
//    on that stream, keep pointing at memory that stays allocated.
//  * release_all() frees every buffer, retired ones included.  The caller must
//    make sure no stream still runs (or will replay) work that uses them.
#pragma once

#include <stdint.h>

#include <map>
#include <mutex>
#include <utility>
#include <vector>

namespace ppa {

// Alloc provides `void* alloc(int64_t bytes)` (nullptr on failure) and
// `bool free(void* p)`.
template <class Key, class Alloc>
class WorkspaceRegistry {
  struct Entry {
    std::mutex use;              // held by a call from taking the buffer to its last launch
    void* ptr = nullptr;
    int64_t bytes = 0;
    std::vector<void*> retired;  // smaller buffers that earlier calls or captured graphs may use
  };

 public:
  // The stream's buffer, held until destruction (or reset()).
  class Lease {
   public:
    Lease() = default;
    Lease(Lease&&) = default;
    Lease& operator=(Lease&&) = default;
    void* ptr() const { return ptr_; }
    bool held() const { return lock_.owns_lock(); }
    void reset() {
      if (lock_.owns_lock()) lock_.unlock();
      ptr_ = nullptr;
    }

   private:
    friend class WorkspaceRegistry;
    std::unique_lock<std::mutex> lock_;
    void* ptr_ = nullptr;
  };

  explicit WorkspaceRegistry(Alloc alloc = Alloc()) : alloc_(std::move(alloc)) {}

  // Takes the entry of `key` (waiting for a call of another thread on the same
  // key to finish enqueueing), grows its buffer to at least `bytes`, and hands
  // it out in `lease`.  Returns false (lease not held) if the allocation fails.
  bool acquire(const Key& key, int64_t bytes, Lease* lease) {
    Entry* e;
    {
      std::lock_guard<std::mutex> g(map_mutex_);
      e = &entries_[key];   // map nodes never move
    }
    std::unique_lock<std::mutex> lk(e->use);
    if (e->bytes < bytes) {
      void* p = alloc_.alloc(bytes);
      if (!p) return false;
      if (e->ptr) e->retired.push_back(e->ptr);
      e->ptr = p;
      e->bytes = bytes;
    }
    lease->lock_ = std::move(lk);
    lease->ptr_ = e->ptr;
    return true;
  }

  // Current capacity of `key`'s buffer (0 if none).
  int64_t capacity(const Key& key) {
    std::lock_guard<std::mutex> g(map_mutex_);
    auto it = entries_.find(key);
    if (it == entries_.end()) return 0;
    std::lock_guard<std::mutex> u(it->second.use);
    return it->second.bytes;
  }

  // Buffers kept alive (current and retired) over all keys.
  int64_t live_buffers() {
    std::lock_guard<std::mutex> g(map_mutex_);
    int64_t n = 0;
    for (auto& kv : entries_) {
      std::lock_guard<std::mutex> u(kv.second.use);
      n += (kv.second.ptr ? 1 : 0) + int64_t(kv.second.retired.size());
    }
    return n;
  }

  // Frees every buffer (waiting for calls that are still enqueueing).
  // Returns false if any free failed (all entries are dropped regardless).
  bool release_all() {
    std::lock_guard<std::mutex> g(map_mutex_);
    bool ok = true;
    for (auto& kv : entries_) {
      std::lock_guard<std::mutex> u(kv.second.use);
      for (void* p : kv.second.retired) ok &= alloc_.free(p);
      if (kv.second.ptr) ok &= alloc_.free(kv.second.ptr);
    }
    entries_.clear();
    return ok;
  }

 private:
  Alloc alloc_;
  std::mutex map_mutex_;
  std::map<Key, Entry> entries_;
};

}  // namespace ppa
