#include "allocator.hpp"

#include <limits>

namespace pa {

namespace {
int64_t blocks_for(int64_t tokens, int64_t bs) { return (tokens + bs - 1) / bs; }
}  // namespace

BlockAllocator::BlockAllocator(int32_t num_blocks, int32_t block_size)
    : n_(num_blocks), bs_(block_size), ref_(num_blocks, 0) {
  stack_.reserve(num_blocks);
  for (int32_t i = num_blocks - 1; i >= 0; --i) stack_.push_back(i);
}

bool BlockAllocator::set_free_order(const int32_t* order, int32_t n, std::string* err) {
  if (n != n_) {
    *err = "free order must list every block id once";
    return false;
  }
  std::vector<char> seen(n_, 0);
  for (int32_t i = 0; i < n; ++i) {
    int32_t b = order[i];
    if (b < 0 || b >= n_ || seen[b]) {
      *err = "free order must be a permutation of 0..N-1";
      return false;
    }
    seen[b] = 1;
  }
  stack_.clear();
  for (int32_t i = n - 1; i >= 0; --i) stack_.push_back(order[i]);
  return true;
}

int32_t BlockAllocator::create() {
  seqs_.push_back(Seq{});
  seqs_.back().alive = true;
  ++live_count_;
  return static_cast<int32_t>(seqs_.size() - 1);
}

bool BlockAllocator::live(int32_t seq) const {
  return seq >= 0 && static_cast<size_t>(seq) < seqs_.size() && seqs_[seq].alive;
}

AllocResult BlockAllocator::append(int32_t seq, int32_t n_tokens, int32_t* slots_out,
                                   int32_t* cow_pair, int* n_cow, std::string* err) {
  if (n_cow) *n_cow = 0;
  if (!live(seq)) {
    *err = "unknown or released sequence";
    return AllocResult::InvalidArg;
  }
  if (n_tokens < 0) {
    *err = "token count cannot be negative";
    return AllocResult::InvalidArg;
  }
  if (n_tokens == 0) return AllocResult::Ok;
  Seq& s = seqs_[seq];
  const int64_t len0 = s.length, len1 = len0 + n_tokens;
  if (len1 > std::numeric_limits<int32_t>::max() / 2) {
    *err = "sequence length overflow";
    return AllocResult::InvalidArg;
  }
  const int64_t fresh = blocks_for(len1, bs_) - blocks_for(len0, bs_);
  const bool cow = (len0 % bs_) != 0 && ref_[s.table.back()] > 1;
  if (fresh + (cow ? 1 : 0) > static_cast<int64_t>(stack_.size())) {
    *err = "pool exhausted";
    return AllocResult::OutOfBlocks;
  }
  if (cow) {
    const int32_t old_b = s.table.back();
    const int32_t new_b = stack_.back();
    stack_.pop_back();
    --ref_[old_b];
    ref_[new_b] = 1;
    s.table.back() = new_b;
    if (cow_pair) {
      cow_pair[0] = old_b;
      cow_pair[1] = new_b;
    }
    if (n_cow) *n_cow = 1;
    ++cow_copies_;
  }
  for (int64_t i = 0; i < fresh; ++i) {
    const int32_t b = stack_.back();
    stack_.pop_back();
    ref_[b] = 1;
    s.table.push_back(b);
  }
  if (slots_out) {
    for (int64_t p = len0; p < len1; ++p)
      slots_out[p - len0] = s.table[p / bs_] * bs_ + static_cast<int32_t>(p % bs_);
  }
  s.length = static_cast<int32_t>(len1);
  return AllocResult::Ok;
}

AllocResult BlockAllocator::fork(int32_t parent, int32_t* child, std::string* err) {
  if (!live(parent)) {
    *err = "unknown or released parent sequence";
    return AllocResult::InvalidArg;
  }
  for (int32_t b : seqs_[parent].table) ++ref_[b];
  Seq c;
  c.table = seqs_[parent].table;
  c.length = seqs_[parent].length;
  c.alive = true;
  seqs_.push_back(std::move(c));
  ++live_count_;
  *child = static_cast<int32_t>(seqs_.size() - 1);
  return AllocResult::Ok;
}

AllocResult BlockAllocator::release(int32_t seq, std::string* err) {
  if (!live(seq)) {
    *err = "unknown or released sequence";
    return AllocResult::InvalidArg;
  }
  Seq& s = seqs_[seq];
  for (int32_t b : s.table) {
    if (--ref_[b] == 0) stack_.push_back(b);
  }
  s.table.clear();
  s.table.shrink_to_fit();
  s.length = 0;
  s.alive = false;
  --live_count_;
  return AllocResult::Ok;
}

int64_t BlockAllocator::logical_tokens() const {
  int64_t t = 0;
  for (const Seq& s : seqs_)
    if (s.alive) t += s.length;
  return t;
}

int64_t BlockAllocator::tail_slots() const {
  int64_t t = 0;
  for (const Seq& s : seqs_)
    if (s.alive) t += static_cast<int64_t>(s.table.size()) * bs_ - s.length;
  return t;
}

int64_t BlockAllocator::shared_blocks() const {
  int64_t c = 0;
  for (int32_t r : ref_)
    if (r > 1) ++c;
  return c;
}

}  // namespace pa
