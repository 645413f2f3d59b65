// Host pack planners: order-preserving next-fit and best-fit-decreasing.
//
// Next-fit follows "Pack sequences without joining their contexts", "Fill only
// the current row" and "Extend the existing storage and decoder": whole items
// only, an oversized item is an error, an exact fill opens no extra row.
// Best-fit-decreasing is the default strategy named in "Packing与
// FlashAttention Varlen", section 2; its tie-breaks are stated in pvb.h.
//
// The best-fit search keeps the open bins bucketed by remaining room: the
// tightest bin that fits an item of length L is the smallest bin number in the
// first non-empty room bucket >= L.  For capacities up to kDenseRooms the
// buckets are an array of min-heaps indexed by room with a two-level bitset
// over the non-empty ones; beyond that an ordered map of sets.  O(n log n).
#include <algorithm>
#include <cstdint>
#include <map>
#include <functional>
#include <set>
#include <vector>

#include "pvb.h"

namespace {

constexpr int64_t kDenseRooms = int64_t(1) << 20;

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

namespace {

// Buckets of bins by remaining room, for small capacities.
class DenseRooms {
 public:
  explicit DenseRooms(int64_t capacity)
      : heaps_(static_cast<size_t>(capacity) + 1),
        lo_(static_cast<size_t>((capacity + 64) / 64), 0),
        hi_(static_cast<size_t>((lo_.size() + 63) / 64), 0) {}

  // smallest non-empty room >= L, or -1
  int64_t first_at_least(int64_t L) const {
    size_t w = static_cast<size_t>(L >> 6);
    if (w >= lo_.size()) return -1;
    uint64_t bits = lo_[w] & (~uint64_t(0) << (L & 63));
    if (bits) return int64_t(w) * 64 + __builtin_ctzll(bits);
    size_t hw = (w + 1) >> 6;
    if (hw >= hi_.size()) return -1;
    uint64_t hb = ((w + 1) & 63) ? hi_[hw] & (~uint64_t(0) << ((w + 1) & 63)) : hi_[hw];
    while (!hb) {
      if (++hw >= hi_.size()) return -1;
      hb = hi_[hw];
    }
    const size_t lw = hw * 64 + __builtin_ctzll(hb);
    return int64_t(lw) * 64 + __builtin_ctzll(lo_[lw]);
  }
  int32_t pop_min(int64_t room) {
    auto& h = heaps_[room];
    std::pop_heap(h.begin(), h.end(), std::greater<int32_t>());
    const int32_t j = h.back();
    h.pop_back();
    if (h.empty()) clear_bit(room);
    return j;
  }
  void push(int64_t room, int32_t bin) {
    auto& h = heaps_[room];
    if (h.empty()) set_bit(room);
    h.push_back(bin);
    std::push_heap(h.begin(), h.end(), std::greater<int32_t>());
  }

 private:
  void set_bit(int64_t r) {
    lo_[r >> 6] |= uint64_t(1) << (r & 63);
    hi_[r >> 12] |= uint64_t(1) << ((r >> 6) & 63);
  }
  void clear_bit(int64_t r) {
    lo_[r >> 6] &= ~(uint64_t(1) << (r & 63));
    if (!lo_[r >> 6]) hi_[r >> 12] &= ~(uint64_t(1) << ((r >> 6) & 63));
  }
  std::vector<std::vector<int32_t>> heaps_;
  std::vector<uint64_t> lo_, hi_;
};

// Buckets of bins by remaining room, for any capacity.
class SparseRooms {
 public:
  int64_t first_at_least(int64_t L) const {
    auto it = by_room_.lower_bound(L);
    return it == by_room_.end() ? -1 : it->first;
  }
  int32_t pop_min(int64_t room) {
    auto it = by_room_.find(room);
    const int32_t j = *it->second.begin();
    it->second.erase(it->second.begin());
    if (it->second.empty()) by_room_.erase(it);
    return j;
  }
  void push(int64_t room, int32_t bin) { by_room_[room].insert(bin); }

 private:
  std::map<int64_t, std::set<int32_t>> by_room_;
};

template <class Rooms>
void best_fit(const int32_t* lengths, const std::vector<int32_t>& sorted, int32_t capacity,
              Rooms& rooms, int32_t* bin_of, int32_t* start_of, std::vector<int64_t>& room) {
  for (int32_t i : sorted) {
    const int64_t L = lengths[i];
    int32_t j;
    const int64_t r = rooms.first_at_least(L);
    if (r >= 0) {
      j = rooms.pop_min(r);
    } else {
      j = static_cast<int32_t>(room.size());
      room.push_back(capacity);
    }
    bin_of[i] = j;
    start_of[i] = static_cast<int32_t>(capacity - room[j]);
    room[j] -= L;
    rooms.push(room[j], j);
  }
}

}  // namespace

extern "C" pvb_status pvb_pack_plan_bfd(const int32_t* lengths, int64_t n, int32_t capacity,
                                        int32_t* bin_of, int32_t* start_of, int64_t* n_bins,
                                        int32_t* order, int64_t* bin_offsets) {
  pvb_status st = validate(lengths, n, capacity);
  if (st != PVB_OK) return st;
  if (n_bins == nullptr || bin_offsets == nullptr ||
      (n > 0 && (bin_of == nullptr || start_of == nullptr || order == nullptr)))
    return PVB_E_INVALID_ARG;

  const bool dense = capacity <= kDenseRooms && capacity <= 64 * n + 4096;
  // Decreasing length, ties by lower index (a counting sort when lengths are small).
  std::vector<int32_t> sorted(static_cast<size_t>(n));
  if (dense) {
    std::vector<int64_t> first(static_cast<size_t>(capacity) + 2, 0);
    for (int64_t i = 0; i < n; ++i) ++first[capacity - lengths[i] + 1];
    for (int64_t v = 1; v <= capacity + 1; ++v) first[v] += first[v - 1];
    for (int64_t i = 0; i < n; ++i) sorted[first[capacity - lengths[i]]++] = static_cast<int32_t>(i);
  } else {
    for (int64_t i = 0; i < n; ++i) sorted[i] = static_cast<int32_t>(i);
    std::stable_sort(sorted.begin(), sorted.end(),
                     [lengths](int32_t a, int32_t b) { return lengths[a] > lengths[b]; });
  }

  std::vector<int64_t> room;  // remaining room of each bin
  if (dense) {
    DenseRooms rooms(capacity);
    best_fit(lengths, sorted, capacity, rooms, bin_of, start_of, room);
  } else {
    SparseRooms rooms;
    best_fit(lengths, sorted, capacity, rooms, bin_of, start_of, room);
  }
  // order: bin by bin, each bin in insertion (= sorted) order
  const size_t nb = room.size();
  for (size_t j = 0; j <= nb; ++j) bin_offsets[j] = 0;
  for (int64_t i = 0; i < n; ++i) ++bin_offsets[bin_of[i] + 1];
  for (size_t j = 1; j <= nb; ++j) bin_offsets[j] += bin_offsets[j - 1];
  std::vector<int64_t> fill(bin_offsets, bin_offsets + nb);
  for (int32_t i : sorted) order[fill[bin_of[i]]++] = i;
  *n_bins = static_cast<int64_t>(nb);
  return PVB_OK;
}
