#include "allocator.hpp"

#include <algorithm>
#include <limits>

namespace pa {

namespace {
int64_t blocks_for(int64_t tokens, int64_t bs) { return (tokens + bs - 1) / bs; }
}  // namespace

size_t BlockAllocator::KeyHash::operator()(const Key& k) const {
  // FNV-1a over the parent serial and the ids (finds candidates only; keys
  // are compared in full).
  uint64_t h = 1469598103934665603ull;
  auto mix = [&](uint64_t x) {
    for (int i = 0; i < 8; ++i) {
      h ^= (x >> (8 * i)) & 0xffu;
      h *= 1099511628211ull;
    }
  };
  mix(static_cast<uint64_t>(k.parent));
  for (int32_t t : k.ids) mix(static_cast<uint32_t>(t));
  return static_cast<size_t>(h);
}

BlockAllocator::BlockAllocator(int32_t num_blocks, int32_t block_size)
    : n_(num_blocks), bs_(block_size), ref_(num_blocks, 0), serial_(num_blocks, 0), key_of_(num_blocks) {
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

int32_t BlockAllocator::pop_fresh() {
  const int32_t b = stack_.back();
  stack_.pop_back();
  if (serial_[b] != 0) {
    cache_.erase(key_of_[b]);
    serial_[b] = 0;
    key_of_[b].ids.clear();
    ++counts_.evicted;
  }
  return b;
}

AllocResult BlockAllocator::append(int32_t seq, int32_t n_tokens, int32_t* slots_out,
                                   int32_t* cow_pair, int* n_cow, std::string* err) {
  return append_impl(seq, n_tokens, nullptr, slots_out, cow_pair, n_cow, nullptr, err);
}

AllocResult BlockAllocator::append_tokens(int32_t seq, const int32_t* ids, int32_t n_tokens,
                                          int32_t* slots_out, int32_t* cow_pair, int* n_cow,
                                          int* n_cached, std::string* err) {
  if (n_tokens > 0 && !ids) {
    *err = "token ids are NULL";
    if (n_cow) *n_cow = 0;
    if (n_cached) *n_cached = 0;
    return AllocResult::InvalidArg;
  }
  return append_impl(seq, n_tokens, ids, slots_out, cow_pair, n_cow, n_cached, err);
}

AllocResult BlockAllocator::append_impl(int32_t seq, int32_t n_tokens, const int32_t* ids,
                                        int32_t* slots_out, int32_t* cow_pair, int* n_cow,
                                        int* n_cached, std::string* err) {
  if (n_cow) *n_cow = 0;
  if (n_cached) *n_cached = 0;
  if (!resident(seq, err)) return AllocResult::InvalidArg;
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
  // Lookups: whole blocks from a block boundary, up to the first miss.
  std::vector<int32_t> hits;
  int64_t lookups = 0;
  int64_t parent = s.parent;
  if (ids && cache_on_ && s.chain && len0 % bs_ == 0) {
    Key key{0, std::vector<int32_t>(bs_)};
    for (int64_t j = 0; j < n_tokens / bs_; ++j) {
      key.parent = parent;
      key.ids.assign(ids + j * bs_, ids + (j + 1) * bs_);
      ++lookups;
      const auto it = cache_.find(key);
      if (it == cache_.end()) break;
      hits.push_back(it->second);
      parent = serial_[it->second];
    }
  }
  int64_t free_hits = 0;
  for (int32_t b : hits)
    if (ref_[b] == 0) ++free_hits;
  const int64_t fresh = blocks_for(len1, bs_) - blocks_for(len0, bs_) - static_cast<int64_t>(hits.size());
  const bool cow = (len0 % bs_) != 0 && ref_[s.table.back()] > 1;
  if (fresh + (cow ? 1 : 0) > static_cast<int64_t>(stack_.size()) - free_hits) {
    *err = "pool exhausted";
    return AllocResult::OutOfBlocks;
  }
  counts_.lookups += lookups;
  for (int32_t b : hits) {
    if (ref_[b] == 0) {
      for (size_t k = 0; k < stack_.size(); ++k) {
        if (stack_[k] == b) {
          stack_.erase(stack_.begin() + static_cast<std::ptrdiff_t>(k));
          break;
        }
      }
    }
    inc_ref(b);
    s.table.push_back(b);
  }
  counts_.hit_blocks += static_cast<int64_t>(hits.size());
  if (cow) {
    const int32_t old_b = s.table.back();
    const int32_t new_b = pop_fresh();
    dec_ref(old_b);
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
    const int32_t b = pop_fresh();
    ref_[b] = 1;
    s.table.push_back(b);
  }
  const int64_t cached = static_cast<int64_t>(hits.size()) * bs_;
  if (n_cached) *n_cached = static_cast<int>(cached);
  if (slots_out) {
    for (int64_t p = len0; p < len1; ++p)
      slots_out[p - len0] = p - len0 < cached ? -1 : s.table[p / bs_] * bs_ + static_cast<int32_t>(p % bs_);
  }
  s.length = static_cast<int32_t>(len1);
  // Chain state; register the blocks that became full.
  if (!ids || !cache_on_) s.chain = false;
  if (s.chain) {
    s.parent = parent;
    int64_t pos = len0 + cached;
    for (int64_t x = cached; x < n_tokens; ++x) {
      s.tail.push_back(ids[x]);
      ++pos;
      if (pos % bs_ == 0) {
        const int32_t b = s.table[pos / bs_ - 1];
        Key key{s.parent, s.tail};
        const auto it = cache_.find(key);
        if (it != cache_.end()) {
          s.parent = serial_[it->second];
        } else {
          serial_[b] = next_serial_++;
          key_of_[b] = key;
          cache_.emplace(std::move(key), b);
          s.parent = serial_[b];
          ++counts_.registered;
        }
        s.tail.clear();
      }
    }
  } else {
    s.tail.clear();
  }
  return AllocResult::Ok;
}

void BlockAllocator::enable_prefix_cache(bool on) {
  cache_on_ = on;
  if (!on) {
    cache_.clear();
    std::fill(serial_.begin(), serial_.end(), 0);
    for (Key& k : key_of_) k.ids.clear();
    for (Seq& s : seqs_) {
      s.chain = false;
      s.tail.clear();
    }
  }
}

bool BlockAllocator::resident(int32_t seq, std::string* err) const {
  if (!live(seq)) {
    *err = "unknown or released sequence";
    return false;
  }
  if (seqs_[seq].swapped) {
    *err = "sequence is swapped out";
    return false;
  }
  return true;
}

AllocResult BlockAllocator::fork(int32_t parent, int32_t* child, std::string* err) {
  if (!resident(parent, err)) return AllocResult::InvalidArg;
  for (int32_t b : seqs_[parent].table) inc_ref(b);
  Seq c;
  c.table = seqs_[parent].table;
  c.length = seqs_[parent].length;
  c.alive = true;
  c.chain = seqs_[parent].chain;
  c.parent = seqs_[parent].parent;
  c.tail = seqs_[parent].tail;
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
  if (s.swapped) {
    for (int32_t hb : s.host) host_stack_.push_back(hb);
    s.host.clear();
    s.host.shrink_to_fit();
    s.swapped = false;
  } else {
    free_device(s);
  }
  s.table.clear();
  s.table.shrink_to_fit();
  s.tail.clear();
  s.tail.shrink_to_fit();
  s.length = 0;
  s.alive = false;
  --live_count_;
  return AllocResult::Ok;
}

void BlockAllocator::free_device(Seq& s) {
  for (int32_t b : s.table) {
    if (dec_ref(b) == 0) {
      if (cache_on_ && serial_[b] != 0) {
        stack_.insert(stack_.begin(), b);  // cached: reused last
      } else {
        stack_.push_back(b);
      }
    }
  }
}

AllocResult BlockAllocator::host_tier(int32_t num_host_blocks, std::string* err) {
  if (num_host_blocks < 0) {
    *err = "negative host block count";
    return AllocResult::InvalidArg;
  }
  for (const Seq& s : seqs_) {
    if (s.alive && s.swapped) {
      *err = "sequences are swapped out";
      return AllocResult::InvalidArg;
    }
  }
  host_n_ = num_host_blocks;
  host_stack_.clear();
  for (int32_t i = num_host_blocks - 1; i >= 0; --i) host_stack_.push_back(i);
  return AllocResult::Ok;
}

AllocResult BlockAllocator::swap_out(int32_t seq, std::vector<int32_t>* pairs, std::string* err) {
  if (!resident(seq, err)) return AllocResult::InvalidArg;
  Seq& s = seqs_[seq];
  if (s.table.size() > host_stack_.size()) {
    *err = "host tier exhausted";
    return AllocResult::OutOfBlocks;
  }
  pairs->clear();
  s.host.clear();
  for (int32_t b : s.table) {
    const int32_t hb = host_stack_.back();
    host_stack_.pop_back();
    pairs->push_back(b);
    pairs->push_back(hb);
    s.host.push_back(hb);
  }
  free_device(s);
  s.table.clear();
  s.swapped = true;
  return AllocResult::Ok;
}

AllocResult BlockAllocator::swap_in(int32_t seq, std::vector<int32_t>* pairs, std::string* err) {
  if (!live(seq)) {
    *err = "unknown or released sequence";
    return AllocResult::InvalidArg;
  }
  Seq& s = seqs_[seq];
  if (!s.swapped) {
    *err = "sequence is not swapped out";
    return AllocResult::InvalidArg;
  }
  if (s.host.size() > stack_.size()) {
    *err = "pool exhausted";
    return AllocResult::OutOfBlocks;
  }
  pairs->clear();
  s.table.clear();
  for (int32_t hb : s.host) {
    const int32_t b = pop_fresh();
    ref_[b] = 1;
    s.table.push_back(b);
    pairs->push_back(hb);
    pairs->push_back(b);
  }
  for (int32_t hb : s.host) host_stack_.push_back(hb);
  s.host.clear();
  s.swapped = false;
  return AllocResult::Ok;
}

int64_t BlockAllocator::logical_tokens() const {
  int64_t t = 0;
  for (const Seq& s : seqs_)
    if (s.alive && !s.swapped) t += s.length;
  return t;
}

int64_t BlockAllocator::tail_slots() const {
  int64_t t = 0;
  for (const Seq& s : seqs_)
    if (s.alive && !s.swapped) t += static_cast<int64_t>(s.table.size()) * bs_ - s.length;
  return t;
}

void BlockAllocator::inc_ref(int32_t b) {
  if (++ref_[b] == 2) ++shared_count_;
}

int32_t BlockAllocator::dec_ref(int32_t b) {
  if (ref_[b]-- == 2) --shared_count_;
  return ref_[b];
}

}  // namespace pa
