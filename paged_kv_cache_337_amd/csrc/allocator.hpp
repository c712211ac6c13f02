// Host block manager: reference-counted physical blocks, a LIFO free stack,
// per-sequence block tables, fork and block-granular copy-on-write.
//
// Mechanism: "Paged Attention Explained", "How Paged Attention Works", Steps
// 2, 3 and 5 (on-demand blocks, block table, release to the pool) and the
// "KV-Cache Block Manager" component; "PagedAttention: paging the KV cache like
// an OS pages memory", "How it works" (reference counts, copy-on-write when a
// shared block must be modified).
//
// Open policy points, fixed here: the free stack pops in the caller's given
// order first; sequence ids are never reused; fork and release walk tables in
// logical order; at most one copy per append (only the last block can be
// partially filled); every operation validates before it mutates.
//
// Automatic prefix caching ("PagedAttention and KV Cache Compression", "What
// Most People Miss": every block of prompt text gets a fingerprint, and a
// request whose block matches points to the existing block instead of
// processing it again).  A full block is identified exactly by the cache
// serial of the block before it (0 for a sequence's first block) and its
// block_size token ids; the hash only finds candidates.  Lookups run from a
// block boundary over the appended whole blocks and stop at the first miss;
// hits are applied before copy-on-write and fresh blocks.  A block is
// registered when it becomes full with known ids (an existing entry with the
// same key stays).  A registered block popped for new contents is evicted;
// registered blocks freed to count 0 go to the bottom of the free stack, so
// uncached blocks are reused first and cached ones least recently freed
// first.  An append without ids ends the sequence's chain; fork copies it.
//
// Host tier ("Paged Attention Explained", "Hybrid Memory Strategies"): host
// blocks each hold one device block of every layer; their free blocks form a
// LIFO stack (initially ascending ids).  swap_out gives each block of the
// sequence's table, in logical order, the top host block and then releases
// the device blocks as release would (a block shared with another sequence
// stays on the device); swap_in takes fresh device blocks in logical order
// and returns the host blocks in logical order.  A swapped sequence keeps its
// length and prefix-cache chain; it cannot grow or be forked until swapped in.
#pragma once

#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

namespace pa {

enum class AllocResult { Ok, InvalidArg, OutOfBlocks };

class BlockAllocator {
 public:
  BlockAllocator(int32_t num_blocks, int32_t block_size);

  // order: ids in the order they are handed out; empty -> ascending.
  bool set_free_order(const int32_t* order, int32_t n, std::string* err);

  int32_t create();
  AllocResult append(int32_t seq, int32_t n_tokens, int32_t* slots_out, int32_t* cow_pair,
                     int* n_cow, std::string* err);
  // Append tokens by id; slots of tokens served by cached blocks are -1 and
  // their count is *n_cached (a multiple of the block size).
  AllocResult append_tokens(int32_t seq, const int32_t* ids, int32_t n_tokens, int32_t* slots_out,
                            int32_t* cow_pair, int* n_cow, int* n_cached, std::string* err);
  void enable_prefix_cache(bool on);
  AllocResult host_tier(int32_t num_host_blocks, std::string* err);
  // pairs: (device, host) for swap_out, (host, device) for swap_in, [2 * n].
  AllocResult swap_out(int32_t seq, std::vector<int32_t>* pairs, std::string* err);
  AllocResult swap_in(int32_t seq, std::vector<int32_t>* pairs, std::string* err);
  bool swapped(int32_t seq) const { return live(seq) && seqs_[seq].swapped; }
  const std::vector<int32_t>& host_table(int32_t seq) const { return seqs_[seq].host; }
  int32_t host_blocks() const { return host_n_; }
  const std::vector<int32_t>& host_free_stack() const { return host_stack_; }
  bool prefix_cache_enabled() const { return cache_on_; }
  struct CacheCounts {
    int64_t registered = 0, hit_blocks = 0, evicted = 0, lookups = 0;
  };
  const CacheCounts& cache_counts() const { return counts_; }
  int64_t cached_blocks() const { return static_cast<int64_t>(cache_.size()); }
  AllocResult fork(int32_t parent, int32_t* child, std::string* err);
  AllocResult release(int32_t seq, std::string* err);

  bool live(int32_t seq) const;
  const std::vector<int32_t>& table(int32_t seq) const { return seqs_[seq].table; }
  int32_t length(int32_t seq) const { return seqs_[seq].length; }

  int32_t num_blocks() const { return n_; }
  int32_t block_size() const { return bs_; }
  const std::vector<int32_t>& refcounts() const { return ref_; }
  const std::vector<int32_t>& free_stack() const { return stack_; }
  int64_t cow_copies() const { return cow_copies_; }
  int64_t live_seqs() const { return live_count_; }
  int64_t logical_tokens() const;
  int64_t tail_slots() const;
  int64_t shared_blocks() const { return shared_count_; }  // blocks with count > 1

 private:
  struct Seq {
    std::vector<int32_t> table;
    int32_t length = 0;
    bool alive = false;
    bool chain = true;          // every token id so far is known
    int64_t parent = 0;         // cache serial of the last full block
    std::vector<int32_t> tail;  // ids of the partially filled last block
    bool swapped = false;
    std::vector<int32_t> host;  // host blocks while swapped out
  };
  struct Key {
    int64_t parent;
    std::vector<int32_t> ids;
    bool operator==(const Key& o) const { return parent == o.parent && ids == o.ids; }
  };
  struct KeyHash {
    size_t operator()(const Key& k) const;
  };
  AllocResult append_impl(int32_t seq, int32_t n_tokens, const int32_t* ids, int32_t* slots_out,
                          int32_t* cow_pair, int* n_cow, int* n_cached, std::string* err);
  int32_t pop_fresh();
  void free_device(Seq& s);
  bool resident(int32_t seq, std::string* err) const;
  void inc_ref(int32_t b);
  int32_t dec_ref(int32_t b);  // returns the new count

  int32_t n_, bs_;
  std::vector<int32_t> ref_;
  std::vector<int32_t> stack_;  // top = back()
  std::vector<Seq> seqs_;
  int64_t cow_copies_ = 0;
  int64_t live_count_ = 0;
  int64_t shared_count_ = 0;  // blocks with count > 1
  // prefix cache
  bool cache_on_ = false;
  std::unordered_map<Key, int32_t, KeyHash> cache_;
  std::vector<int64_t> serial_;   // per block, 0 = not registered
  std::vector<Key> key_of_;       // per block, valid when registered
  int64_t next_serial_ = 1;
  CacheCounts counts_;
  // host tier
  int32_t host_n_ = 0;
  std::vector<int32_t> host_stack_;  // top = back()
};

}  // namespace pa
