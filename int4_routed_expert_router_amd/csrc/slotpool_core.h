// Slot-pool replacement policy (host only, no HIP): residency table, LFU
// counts with lazy aging, recency, pinning.  The policy is spelled out in
// include/moe_slotpool.h.
#pragma once
#include <stdint.h>

#include <vector>

namespace moe {

struct PoolEvent {
  int32_t expert;
  int32_t slot;
  int32_t victim;  // evicted expert or -1
  bool hit;
};

class PoolCore {
 public:
  enum Result { kOk = 0, kFull = 1, kBadInput = 2, kBusy = 3 };

  PoolCore(int layers, int experts, int slots, int aging_period)
      : L_(layers), E_(experts), S_(slots), P_(aging_period),
        slot_of_(static_cast<size_t>(layers) * experts, -1),
        expert_in_(static_cast<size_t>(layers) * slots, -1),
        count_(static_cast<size_t>(layers) * slots, 0),
        last_use_(static_cast<size_t>(layers) * slots, 0),
        pinned_(static_cast<size_t>(layers) * slots, 0),
        epoch_(layers, 0),
        mark_(experts, 0) {}

  // Plans and applies one acquire; events[i] describes experts[i].  On kFull
  // or kBadInput nothing changes.
  Result acquire(int layer, const int32_t* experts, int n, uint64_t step, std::vector<PoolEvent>& events) {
    events.assign(n, PoolEvent{-1, -1, -1, false});
    if (layer < 0 || layer >= L_ || n < 0) return kBadInput;
    int32_t* slot_of = &slot_of_[static_cast<size_t>(layer) * E_];
    const size_t sb = static_cast<size_t>(layer) * S_;
    if (!distinct_in_range(experts, n)) return kBadInput;
    int misses = 0;
    for (int i = 0; i < n; ++i)
      if (slot_of[experts[i]] < 0) ++misses;
    if (misses > 0) {
      int avail = 0;
      for (int s = 0; s < S_; ++s) {
        const int e = expert_in_[sb + s];
        if (e < 0) ++avail;
        else if (!pinned_[sb + s] && !requested(e, experts, n)) ++avail;
      }
      if (misses > avail) return kFull;
    }
    age(layer, step);
    for (int i = 0; i < n; ++i) {
      const int e = experts[i];
      const int s = slot_of[e];
      if (s >= 0) {
        count_[sb + s] += 1;
        last_use_[sb + s] = step;
        pinned_[sb + s] = 1;
        events[i] = PoolEvent{e, s, -1, true};
        ++hits_;
      }
    }
    for (int i = 0; i < n; ++i) {
      const int e = experts[i];
      if (events[i].hit) continue;
      int s = -1, victim = -1;
      for (int k = 0; k < S_; ++k)
        if (expert_in_[sb + k] < 0) {
          s = k;
          break;
        }
      if (s < 0) {
        for (int k = 0; k < S_; ++k) {
          if (pinned_[sb + k]) continue;
          if (s < 0 || better_victim(sb, k, s)) s = k;
        }
        victim = expert_in_[sb + s];
        slot_of[victim] = -1;
        ++evictions_;
      }
      expert_in_[sb + s] = e;
      slot_of[e] = s;
      count_[sb + s] = 1;
      last_use_[sb + s] = step;
      pinned_[sb + s] = 1;
      events[i] = PoolEvent{e, s, victim, false};
      ++misses_;
    }
    return kOk;
  }

  // Best-effort early load of predicted experts (see include/moe_slotpool.h):
  // loaded[k] describes the k-th expert this call brought in (hit = false).
  Result prefetch(int layer, const int32_t* experts, int n, uint64_t step, std::vector<PoolEvent>& loaded) {
    loaded.clear();
    if (layer < 0 || layer >= L_ || n < 0) return kBadInput;
    if (!distinct_in_range(experts, n)) return kBadInput;
    int32_t* slot_of = &slot_of_[static_cast<size_t>(layer) * E_];
    const size_t sb = static_cast<size_t>(layer) * S_;
    age(layer, step);
    for (int i = 0; i < n; ++i) {
      const int e = experts[i];
      if (slot_of[e] >= 0) continue;
      int s = -1, victim = -1;
      for (int k = 0; k < S_; ++k)
        if (expert_in_[sb + k] < 0) {
          s = k;
          break;
        }
      if (s < 0) {
        for (int k = 0; k < S_; ++k) {
          if (pinned_[sb + k] || requested(expert_in_[sb + k], experts, n)) continue;
          if (s < 0 || better_victim(sb, k, s)) s = k;
        }
        if (s < 0) continue;   // every slot is pinned or holds a requested expert
        victim = expert_in_[sb + s];
        slot_of[victim] = -1;
        ++evictions_;
      }
      expert_in_[sb + s] = e;
      slot_of[e] = s;
      count_[sb + s] = 0;
      last_use_[sb + s] = step;
      loaded.push_back(PoolEvent{e, s, victim, false});
      ++prefetches_;
    }
    return kOk;
  }

  void release(int layer) {
    const size_t sb = static_cast<size_t>(layer) * S_;
    for (int s = 0; s < S_; ++s) pinned_[sb + s] = 0;
  }

  Result evict(int layer, int expert) {
    if (layer < 0 || layer >= L_ || expert < 0 || expert >= E_) return kBadInput;
    int32_t& so = slot_of_[static_cast<size_t>(layer) * E_ + expert];
    if (so < 0) return kOk;
    const size_t k = static_cast<size_t>(layer) * S_ + so;
    if (pinned_[k]) return kBusy;
    expert_in_[k] = -1;
    count_[k] = 0;
    last_use_[k] = 0;
    so = -1;
    ++evictions_;
    return kOk;
  }

  uint64_t hits() const { return hits_; }
  uint64_t misses() const { return misses_; }
  uint64_t evictions() const { return evictions_; }
  uint64_t prefetches() const { return prefetches_; }
  int layers() const { return L_; }
  int experts() const { return E_; }
  int slots() const { return S_; }

 private:
  bool distinct_in_range(const int32_t* experts, int n) {
    bool bad = false;
    for (int i = 0; i < n && !bad; ++i) {
      const int e = experts[i];
      if (e < 0 || e >= E_ || mark_[e]) bad = true;
      else mark_[e] = 1;
    }
    for (int i = 0; i < n; ++i)
      if (experts[i] >= 0 && experts[i] < E_) mark_[experts[i]] = 0;
    return !bad;
  }
  static bool requested(int e, const int32_t* experts, int n) {
    for (int i = 0; i < n; ++i)
      if (experts[i] == e) return true;
    return false;
  }
  bool better_victim(size_t sb, int a, int b) const {
    if (count_[sb + a] != count_[sb + b]) return count_[sb + a] < count_[sb + b];
    if (last_use_[sb + a] != last_use_[sb + b]) return last_use_[sb + a] < last_use_[sb + b];
    return expert_in_[sb + a] < expert_in_[sb + b];
  }
  void age(int layer, uint64_t step) {
    if (P_ <= 0) return;
    const uint64_t ep = step / static_cast<uint64_t>(P_);
    if (ep > epoch_[layer]) {
      const uint64_t d = ep - epoch_[layer];
      const int shift = d > 63 ? 63 : static_cast<int>(d);
      const size_t sb = static_cast<size_t>(layer) * S_;
      for (int s = 0; s < S_; ++s) count_[sb + s] >>= shift;
      epoch_[layer] = ep;
    }
  }

  int L_, E_, S_, P_;
  std::vector<int32_t> slot_of_, expert_in_;
  std::vector<uint64_t> count_, last_use_;
  std::vector<uint8_t> pinned_;
  std::vector<uint64_t> epoch_;
  std::vector<uint8_t> mark_;
  uint64_t hits_ = 0, misses_ = 0, evictions_ = 0, prefetches_ = 0;
};

}  // namespace moe
