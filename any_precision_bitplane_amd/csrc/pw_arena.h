// Extent allocator over one caller-owned byte range (the plane arena of the
// weight pager).  Pure host C++ with no HIP dependency, so it is unit-tested on
// the CPU on its own.
//
// "Technical summary: PagedWeight", Core components 1: the page table tracks
// per block a desired and a committed bitwidth, and pages live on the GPU, on
// the CPU or in transfer.  A block committed at q keeps the first q bit planes
// resident; with the plane-major storage format those planes are one contiguous
// prefix, so the block's device pages form one extent of q plane slabs that
// grows or shrinks at its end.  This allocator hands out such extents:
// first-fit over a sorted free list, neighbours merged on release, growth in
// place when the range after an extent is free.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <iterator>
#include <map>

namespace pw {

class ExtentArena {
 public:
  static constexpr size_t kNone = ~(size_t)0;

  ExtentArena(size_t bytes = 0, size_t align = 256) { reset(bytes, align); }

  void reset(size_t bytes, size_t align) {
    align_ = align ? align : 1;
    size_ = bytes / align_ * align_;
    free_.clear();
    if (size_) free_[0] = size_;
    used_ = 0;
  }

  size_t size() const { return size_; }
  size_t used() const { return used_; }
  size_t round(size_t n) const { return (n + align_ - 1) / align_ * align_; }

  // Offset of a new extent of n bytes (rounded up), or kNone if no free range fits.
  size_t alloc(size_t n) {
    n = round(n);
    if (n == 0) return kNone;
    for (auto it = free_.begin(); it != free_.end(); ++it) {
      if (it->second < n) continue;
      const size_t off = it->first, len = it->second;
      free_.erase(it);
      if (len > n) free_[off + n] = len - n;
      used_ += n;
      return off;
    }
    return kNone;
  }

  // Return [off, off + n) to the free list, merging with free neighbours.
  // The range must have come from alloc/grow and not be free already.
  void release(size_t off, size_t n) {
    n = round(n);
    if (n == 0) return;
    used_ -= n;
    auto next = free_.lower_bound(off);
    if (next != free_.begin()) {
      auto prev = std::prev(next);
      if (prev->first + prev->second == off) {
        off = prev->first;
        n += prev->second;
        free_.erase(prev);
      }
    }
    next = free_.lower_bound(off);
    if (next != free_.end() && off + n == next->first) {
      n += next->second;
      free_.erase(next);
    }
    free_[off] = n;
  }

  // Grow the extent [off, off + old_n) to new_n bytes in place if the range
  // right after it is free; returns whether it did.
  bool grow(size_t off, size_t old_n, size_t new_n) {
    old_n = round(old_n);
    new_n = round(new_n);
    if (new_n <= old_n) return true;
    const size_t end = off + old_n, extra = new_n - old_n;
    auto it = free_.find(end);
    if (it == free_.end() || it->second < extra) return false;
    const size_t len = it->second;
    free_.erase(it);
    if (len > extra) free_[end + extra] = len - extra;
    used_ += extra;
    return true;
  }

  size_t free_ranges() const { return free_.size(); }
  size_t largest_free() const {
    size_t m = 0;
    for (const auto& kv : free_) m = kv.second > m ? kv.second : m;
    return m;
  }

 private:
  size_t size_ = 0, align_ = 256, used_ = 0;
  std::map<size_t, size_t> free_;   // offset -> length, disjoint, never adjacent
};

}  // namespace pw
