// LFU + recency slot table of the bounded expert pool (host side, HIP-free).
//
// Pages: hot experts sit in a bounded pool evicted by LFU plus recency
// (paotong.dev commentary, paragraph on the bounded pool; cheshm.ai news
// article, paragraph on how it works), filled lazily from an empty start
// (alphalab.site field test, section on the 4.3 GB figure). Reading taken
// (moe.h states it in full): per (token, layer) step the selected experts are
// visited in ascending global id; a hit increments the slot's use count and
// stamps the tick; a miss fills the lowest empty slot or evicts the slot with
// the smallest (use count, last tick) not used by the current step.
#pragma once

#include <cstdint>
#include <set>
#include <tuple>
#include <unordered_map>
#include <vector>

namespace moe {

class PoolTable {
 public:
  explicit PoolTable(int64_t n_slots);
  void reset();

  // One step: gids (k distinct values, any order). Writes, per input position,
  // the slot now holding that gid. Appends per-access (ascending gid) hit and
  // victim entries to the trace. Returns, per input position, whether the
  // access missed (needs a copy into its slot).
  void step(const int64_t* gids, int k, int64_t* slot_of_pos, uint8_t* miss_of_pos);

  int64_t n_slots() const { return n_slots_; }
  uint64_t accesses = 0, hits = 0, misses = 0, evictions = 0;
  std::vector<uint8_t> trace_hit;
  std::vector<int64_t> trace_victim;

 private:
  int64_t n_slots_;
  std::vector<int64_t> slot_gid_;
  std::vector<uint64_t> freq_, last_;
  std::vector<uint8_t> pinned_;
  std::unordered_map<int64_t, int64_t> where_;
  std::set<std::tuple<uint64_t, uint64_t, int64_t>> evictable_;
  int64_t next_empty_ = 0;
  uint64_t tick_ = 0;
};

}  // namespace moe
