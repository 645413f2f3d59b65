// Host pack planners: order-preserving next-fit and best-fit-decreasing.
//
// Next-fit follows "Pack sequences without joining their contexts", "Fill only
// the current row" and "Extend the existing storage and decoder": whole items
// only, an oversized item is an error, an exact fill opens no extra row.
// Best-fit-decreasing is the default strategy named in "Packing与
// FlashAttention Varlen", section 2; its tie-breaks are stated in pvb.h.
//
// The best-fit search keeps, for every distinct remaining-room value, the set of
// bins with that room: the tightest bin that fits an item of length L is the
// smallest bin number in the first room bucket >= L.  O(n log n) overall.
#include <algorithm>
#include <cstdint>
#include <map>
#include <set>
#include <vector>

#include "pvb.h"

namespace {

pvb_status validate(const int32_t* lengths, int64_t n, int32_t capacity) {
  if (n < 0 || capacity <= 0) return PVB_E_INVALID_ARG;
  if (n > 0 && lengths == nullptr) return PVB_E_INVALID_ARG;
  if (n > (int64_t(1) << 31)) return PVB_E_OVERFLOW;
  for (int64_t i = 0; i < n; ++i) {
    if (lengths[i] < 0) return PVB_E_INVALID_ARG;
    if (lengths[i] > capacity) return PVB_E_OVERSIZED;
  }
  return PVB_OK;
}

}  // namespace

extern "C" pvb_status pvb_pack_plan_nextfit(const int32_t* lengths, int64_t n, int32_t capacity,
                                            int32_t* row_of, int32_t* start_of, int64_t* n_rows) {
  pvb_status st = validate(lengths, n, capacity);
  if (st != PVB_OK) return st;
  if (n_rows == nullptr || (n > 0 && (row_of == nullptr || start_of == nullptr)))
    return PVB_E_INVALID_ARG;
  if (n == 0) {
    *n_rows = 0;
    return PVB_OK;
  }
  int64_t row = 0, used = 0;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t L = lengths[i];
    if (L > capacity - used) {
      ++row;
      used = 0;
    }
    row_of[i] = static_cast<int32_t>(row);
    start_of[i] = static_cast<int32_t>(used);
    used += L;
  }
  *n_rows = row + 1;
  return PVB_OK;
}

extern "C" pvb_status pvb_pack_plan_bfd(const int32_t* lengths, int64_t n, int32_t capacity,
                                        int32_t* bin_of, int32_t* start_of, int64_t* n_bins,
                                        int32_t* order, int64_t* bin_offsets) {
  pvb_status st = validate(lengths, n, capacity);
  if (st != PVB_OK) return st;
  if (n_bins == nullptr || bin_offsets == nullptr ||
      (n > 0 && (bin_of == nullptr || start_of == nullptr || order == nullptr)))
    return PVB_E_INVALID_ARG;

  // Decreasing length, ties by lower index.
  std::vector<int32_t> sorted(static_cast<size_t>(n));
  for (int64_t i = 0; i < n; ++i) sorted[i] = static_cast<int32_t>(i);
  std::stable_sort(sorted.begin(), sorted.end(),
                   [lengths](int32_t a, int32_t b) { return lengths[a] > lengths[b]; });

  std::map<int64_t, std::set<int32_t>> by_room;  // room -> bins with that room
  std::vector<int64_t> room;                     // room of each bin
  std::vector<std::vector<int32_t>> members;
  for (int64_t s = 0; s < n; ++s) {
    const int32_t i = sorted[s];
    const int64_t L = lengths[i];
    int32_t j;
    auto it = by_room.lower_bound(L);
    if (it != by_room.end()) {
      j = *it->second.begin();
      it->second.erase(it->second.begin());
      if (it->second.empty()) by_room.erase(it);
    } else {
      j = static_cast<int32_t>(room.size());
      room.push_back(capacity);
      members.emplace_back();
    }
    bin_of[i] = j;
    start_of[i] = static_cast<int32_t>(capacity - room[j]);
    room[j] -= L;
    members[j].push_back(i);
    by_room[room[j]].insert(j);
  }
  int64_t pos = 0;
  bin_offsets[0] = 0;
  for (size_t j = 0; j < members.size(); ++j) {
    for (int32_t i : members[j]) order[pos++] = i;
    bin_offsets[j + 1] = pos;
  }
  *n_bins = static_cast<int64_t>(members.size());
  return PVB_OK;
}
