#include "pool_policy.h"

#include <algorithm>
#include <numeric>

#include "common.h"

namespace moe {

PoolTable::PoolTable(int64_t n_slots) : n_slots_(n_slots) { reset(); }

void PoolTable::reset() {
  slot_gid_.assign((size_t)n_slots_, -1);
  freq_.assign((size_t)n_slots_, 0);
  last_.assign((size_t)n_slots_, 0);
  pinned_.assign((size_t)n_slots_, 0);
  where_.clear();
  evictable_.clear();
  next_empty_ = 0;
  tick_ = 0;
  accesses = hits = misses = evictions = 0;
  trace_hit.clear();
  trace_victim.clear();
}

void PoolTable::step(const int64_t* gids, int k, int64_t* slot_of_pos, uint8_t* miss_of_pos) {
  std::vector<int> order((size_t)k);
  std::iota(order.begin(), order.end(), 0);
  std::sort(order.begin(), order.end(), [&](int a, int b) { return gids[a] < gids[b]; });
  std::vector<int64_t> touched;
  touched.reserve((size_t)k);
  for (int pos : order) {
    const int64_t gid = gids[pos];
    ++tick_;
    ++accesses;
    auto it = where_.find(gid);
    int64_t s;
    if (it != where_.end()) {
      s = it->second;
      if (!pinned_[(size_t)s]) evictable_.erase(std::make_tuple(freq_[(size_t)s], last_[(size_t)s], s));
      freq_[(size_t)s] += 1;
      last_[(size_t)s] = tick_;
      ++hits;
      trace_hit.push_back(1);
      trace_victim.push_back(-1);
      miss_of_pos[pos] = 0;
    } else {
      int64_t victim = -1;
      if (next_empty_ < n_slots_) {
        s = next_empty_++;
      } else {
        auto v = evictable_.begin();  // smallest (freq, last) among unpinned slots
        s = std::get<2>(*v);
        evictable_.erase(v);
        victim = slot_gid_[(size_t)s];
        where_.erase(victim);
        ++evictions;
      }
      slot_gid_[(size_t)s] = gid;
      where_[gid] = s;
      freq_[(size_t)s] = 1;
      last_[(size_t)s] = tick_;
      ++misses;
      trace_hit.push_back(0);
      trace_victim.push_back(victim);
      miss_of_pos[pos] = 1;
    }
    slot_of_pos[pos] = s;
    if (!pinned_[(size_t)s]) {
      pinned_[(size_t)s] = 1;
      touched.push_back(s);
    }
  }
  for (int64_t s : touched) {
    pinned_[(size_t)s] = 0;
    evictable_.insert(std::make_tuple(freq_[(size_t)s], last_[(size_t)s], s));
  }
}

}  // namespace moe

extern "C" moe_status moe_pool_simulate(int64_t n_slots, int32_t k, int64_t n_steps, const int64_t* gids,
                                        uint8_t* hit, int64_t* victim) {
  moe::clear_error();
  if (n_slots < 1 || k < 1 || k > n_slots || n_steps < 0)
    return moe::fail(MOE_EINVAL, "moe_pool_simulate: need 1 <= k <= n_slots and n_steps >= 0");
  if (n_steps > 0 && (!gids || !hit || !victim)) return moe::fail(MOE_EINVAL, "moe_pool_simulate: NULL pointer");
  for (int64_t s = 0; s < n_steps; ++s)
    for (int a = 0; a < k; ++a)
      for (int b = a + 1; b < k; ++b)
        if (gids[s * k + a] == gids[s * k + b])
          return moe::fail(MOE_EINVAL, "moe_pool_simulate: repeated gid within a step");
  moe::PoolTable t(n_slots);
  std::vector<int64_t> slots((size_t)k);
  std::vector<uint8_t> miss((size_t)k);
  for (int64_t s = 0; s < n_steps; ++s) t.step(gids + s * k, k, slots.data(), miss.data());
  std::copy(t.trace_hit.begin(), t.trace_hit.end(), hit);
  std::copy(t.trace_victim.begin(), t.trace_victim.end(), victim);
  return MOE_OK;
}
