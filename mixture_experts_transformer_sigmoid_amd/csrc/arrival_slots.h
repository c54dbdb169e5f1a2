// Host-side table of the small-batch router's arrival-count slots (plain C++, no HIP).
//
// The router kernel counts, per 16-token block, the workgroups that have finished, in
// counters the library holds on each GPU; the last workgroup of a block takes the block's
// top-k and puts the counter back to zero.  Calls that may overlap on one GPU must not
// share counters, and such calls need their own workspaces, so each workspace address
// gets a slot of its own: a slot stays with its workspace while that workspace is among
// the kSlots most recently used, and forever once a call on it has been captured into a
// graph (the graph's launches carry the slot number, so it may never be handed to another
// workspace) until the caller releases the workspace.  One table per GPU; the caller
// serialises access.
#pragma once

#include <stdint.h>

#include <unordered_map>

namespace moe {

template <int kSlots>
class ArrivalSlotTable {
 public:
  // The slot of workspace `key`; `pin` (the call is being captured) keeps it until the
  // workspace is released.  Returns -1 when every slot is held by a graph and `key` has none.
  int slot(uintptr_t key, bool pin) {
    ++clock_;
    int i;
    const auto it = slot_of_.find(key);
    if (it != slot_of_.end()) {
      i = it->second;
    } else {
      // a free slot, else the least recently used one that no graph holds
      i = -1;
      for (int j = 0; j < kSlots; ++j) {
        if (!taken_[j]) {
          i = j;
          break;
        }
        if (!pinned_[j] && (i < 0 || used_at_[j] < used_at_[i])) i = j;
      }
      if (i < 0) return -1;
      if (taken_[i]) slot_of_.erase(key_[i]);
      taken_[i] = true;
      key_[i] = key;
      slot_of_[key] = i;
    }
    used_at_[i] = clock_;
    if (pin) pinned_[i] = true;
    return i;
  }

  // Workspace `key` will not be used again: its slot, pinned or not, becomes free.
  void release(uintptr_t key) {
    const auto it = slot_of_.find(key);
    if (it == slot_of_.end()) return;
    const int i = it->second;
    slot_of_.erase(it);
    taken_[i] = false;
    pinned_[i] = false;
  }

 private:
  std::unordered_map<uintptr_t, int> slot_of_;
  uintptr_t key_[kSlots] = {};
  uint64_t used_at_[kSlots] = {};
  bool taken_[kSlots] = {};
  bool pinned_[kSlots] = {};
  uint64_t clock_ = 0;
};

// Frees the slot of workspace `ws` on every GPU (defined with the router; host only).
void arrival_release(const void* ws);

}  // namespace moe
