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
#pragma once

#include <cstdint>
#include <string>
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
  int64_t shared_blocks() const;

 private:
  struct Seq {
    std::vector<int32_t> table;
    int32_t length = 0;
    bool alive = false;
  };
  int32_t n_, bs_;
  std::vector<int32_t> ref_;
  std::vector<int32_t> stack_;  // top = back()
  std::vector<Seq> seqs_;
  int64_t cow_copies_ = 0;
  int64_t live_count_ = 0;
};

}  // namespace pa
