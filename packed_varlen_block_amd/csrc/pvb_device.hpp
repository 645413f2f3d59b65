// Device-side building blocks shared by the gfx950 kernels: vector types, the
// two bf16 MFMA shapes, LDS transpose reads, half-wave exchange and the
// work-item planner used by the attention launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pvb.h"

namespace pvb {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// C[32x32] += A[32x16] * B[16x32]  (bf16 in, fp32 accumulate).
// Lane l holds A[l%32][8*(l/32) + e] and B[8*(l/32) + e][l%32], e = 0..7; the
// result element i of lane l is C[8*(i/4) + 4*(l/32) + i%4][l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Exchange between lanes l and l^32: returns the partner lane's x.
__device__ __forceinline__ float swap_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const bool low = (threadIdx.x & 32) == 0;
  return __uint_as_float(low ? r[1] : r[0]);
}

// Transposed LDS read.  Within each group of 16 lanes, lane i names an 8-byte
// row chunk (4 bf16) at `p`; output lane l' receives element l'%4 of the
// chunks named by lanes l'/4 + 4j, j = 0..3.
__device__ __forceinline__ bf16x4 lds_read_tr(const bf16* p) {
  v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

// 2^x on the transcendental unit (results below 2^-126 flush to 0; -inf -> 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier that orders LDS only: waits for this wave's LDS traffic,
// not for its outstanding global loads, stores or atomics.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Element offset of (row, col) in an LDS tile [rows][D] of bf16 whose 16-byte
// chunks are XOR-swizzled per row.  For D = 128 (16 chunks per 256-byte row,
// 64 banks of 4 bytes) the swizzle f(r) = 4(r%4) + (r/4)%4 makes three access
// patterns bank-conflict free: 16 lanes reading 16 bytes each from 16
// consecutive rows, 32 lanes doing transposed 8-byte reads from 4 consecutive
// rows (r%4 == 0) x 64 bytes, and 16 lanes writing one whole row.
template <int D>
__device__ __forceinline__ int swzf(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((row >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
  return row * D + ((((col >> 3) ^ swzf<D>(row))) << 3) + (col & 7);
}

// Asynchronous 16-byte copy global -> LDS: global_load_lds_dwordx4.  The
// wave's 64 lanes write 64 consecutive 16-byte chunks starting at LDS byte
// address `lds_wave_base` (wave-uniform; lane l at chunk l), reading from
// `gbase + voff` (gbase wave-uniform, voff a per-lane byte offset).
// Completion is tracked by vmcnt only.  The copy is issued from inline
// assembly so that the compiler, which cannot tell which LDS buffer it writes,
// does not add a conservative wait for it before every later LDS read; the
// kernels wait for it explicitly (wait_vmcnt) before a barrier.
__device__ __forceinline__ void copy_to_lds16(const void* gbase, uint32_t voff, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_wave_base), "v"(voff), "s"(gbase)
               : "memory", "m0");
}

// Same, 4 bytes per lane (global_load_lds_dword): 64 consecutive dwords.
__device__ __forceinline__ void copy_to_lds4(const void* gbase, uint32_t voff, uint32_t lds_wave_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(lds_wave_base), "v"(voff), "s"(gbase)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(p);
}

// Stage rows [row0, row0 + ROWS) of a segment-relative [L, D] tensor (row
// stride rs elements) into a swizzled LDS tile [ROWS][D] with 16-byte
// global->LDS copies spread over the NW waves of the workgroup.  Rows at or
// past L are clamped to row L-1 of the same segment, so every staged value is
// finite whenever the segment itself is; callers mask those rows.  Issues
// ROWS * D / 8 / (64 NW) copies per thread.
template <int D, int ROWS, int NW = 4>
__device__ __forceinline__ void stage_rows(const bf16* src, int rs, int row0, int L, bf16* tile, int w,
                                           int lane) {
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;        // rows covered by one wave-wide copy
  constexpr int NI = ROWS / RPI / NW;  // copies per wave
  static_assert(NI * RPI * NW == ROWS, "tile rows must split evenly over the waves");
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const uint32_t tile_base = lds_addr(tile);
#pragma unroll
  for (int r = 0; r < NI; ++r) {
    const int grp = NW * r + wu;
    const int row = grp * RPI + lane / CPR;
    const int c = (lane % CPR) ^ swzf<D>(row);   // logical chunk that lands in this lane's slot
    const int srow = min(row0 + row, L - 1);
    copy_to_lds16(src, (uint32_t)(srow * rs + c * 8) * 2u, tile_base + (uint32_t)(grp * RPI * D * 2));
  }
}

// The same copy pattern for a tile whose rows all lie inside the segment:
// the per-lane byte offsets are computed once (init) and each call only moves
// the wave-uniform source pointer, so a call costs no vector ALU work.
template <int D, int ROWS, int NW = 4>
struct FullTileCopy {
  static constexpr int CPR = D / 8;
  static constexpr int RPI = 64 / CPR;
  static constexpr int NI = ROWS / RPI / NW;
  uint32_t voff[NI];
  int wu;
  __device__ __forceinline__ void init(int rs, int w, int lane) {
    wu = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
    for (int r = 0; r < NI; ++r) {
      const int row = (NW * r + wu) * RPI + lane / CPR;
      const int c = (lane % CPR) ^ swzf<D>(row);
      voff[r] = (uint32_t)(row * rs + c * 8) * 2u;
    }
  }
  // rows [row0, row0 + ROWS) of src (row stride rs), all < L
  __device__ __forceinline__ void issue(const bf16* src, int rs, int row0, bf16* tile) const {
    const bf16* s0 = src + (int64_t)row0 * rs;
    const uint32_t tile_base = lds_addr(tile);
#pragma unroll
    for (int r = 0; r < NI; ++r)
      copy_to_lds16(s0, voff[r], tile_base + (uint32_t)((NW * r + wu) * RPI * D * 2));
  }
};

// Padded LDS tiles.  Rows hold D + 8 bf16 (an odd number of 16-byte chunks),
// and within every 32-row block the rows of an MFMA operand are permuted by
// pi (row-index bits r4 r3 r2 r1 r0 -> r4 r1 r0 r3 r2).  With this layout
//  * 16-byte row reads by 16 lanes from rows pi(0..15) (or pi(16..31)), and
//  * transposed 8-byte reads by 32 lanes from rows b, b+4, b+8, b+12 (64 bytes each)
// are free of bank conflicts, and every address is a per-lane base plus a
// compile-time offset.  C-layout row r of a 32x32 MFMA result computed from
// operand rows pi(0..31) is tile row pi(r), so element i of lane (g, .) sits
// on tile row 16(i>>3) + 4(i&3) + 2((i>>2)&1) + g of its block, and the
// k-slot 8g+e of a 16-deep step kk over those rows is tile row
// 16kk + 4(e&3) + 2(e>>2) + g.
__device__ __forceinline__ int pi32(int r) { return (r & 16) | ((r & 3) << 2) | ((r >> 2) & 3); }
__host__ __device__ constexpr int crow32(int i, int g) {
  return 16 * (i >> 3) + 4 * (i & 3) + 2 * ((i >> 2) & 1) + g;
}

// s_waitcnt with only the vector-memory counter restricted: vmcnt <= n.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <typename T>
__device__ __forceinline__ T out_cast(float x);
template <>
__device__ __forceinline__ float out_cast<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 out_cast<bf16>(float x) { return (bf16)x; }

// ---------------------------------------------------------------------------
// Work-item planner.
//
// A "tile" is (segment b, tile index m) with m < ceil(L_b / TILE); zero-length
// segments have none.  The planner validates cu_seqlens, then writes all tiles
// ordered by m descending, segments in order within a group.  That is heaviest
// first for query tiles (query tile m visits m+1 key tiles); a kernel that
// walks key tiles reads entry (b, m) as key tile ntiles_b - 1 - m, which visits
// m+1 query tiles, so the same list is heaviest first for it too.  Items
// are tile-major with the head fastest, so with H a multiple of 8 every item of
// one head lands on the same XCD (workgroups are dealt to the 8 XCDs round
// robin) and the key/value rows it re-reads stay in that XCD's L2.
// One workgroup of kPlanThreads threads.  LDS holds up to kPlanMaxM groups.
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 1024;
constexpr int kPlanMaxM = 12288;
constexpr int kPlanChunk = 4096;

struct PlanOut {
  int2* tiles;      // [capacity] (b, m)
  int32_t* count;   // [1] number of tiles written
};

__global__ void __launch_bounds__(kPlanThreads)
plan_tiles_kernel(const int32_t* __restrict__ cu, int n_seg, int T, int tile,
                  int2* __restrict__ tiles, int32_t* __restrict__ count, int32_t* __restrict__ status,
                  int report_ok = 1);

// A dispatch packet carries the grid size in work-items as a 32-bit count, so
// a launch of `blocks` workgroups of `threads` work-items must keep the product
// below 2^32; the entry points check this on the host before enqueuing
// anything (PVB_E_UNSUPPORTED), so that no launch fails after an earlier
// kernel of the same call has written PVB_OK to the status word.
inline bool grid_fits(uint64_t blocks, uint32_t threads) { return blocks * threads <= 0xffffffffULL; }

// Host helpers (defined in attn_common.hip).
size_t plan_capacity(int32_t T, int32_t n_seg, int32_t tile);
pvb_status check_host_cu(const int32_t* h_cu, int32_t n_seg, int32_t T);

// Separate key boundaries cu_k (T_k keys) and the key band of each query row
// (see KeyBand): the cross-attention / local-window form of the attention
// entry points.  on = false is causal self-attention over one cu.
struct BandArgs {
  bool on = false;
  const int32_t* cu_k = nullptr;
  int T_k = 0, wl = -1, wr = 0;
};
// Host checks of the cross form: both host mirrors are required (the key
// extents are read by the kernels without a device check), and validated.
pvb_status check_cross_args(const int32_t* h_cu_q, const int32_t* d_cu_k, const int32_t* h_cu_k,
                            int32_t n_seg, int32_t T_q, int32_t T_k, int32_t wl, int32_t wr);

// ---------------------------------------------------------------------------
// In-kernel work-item decode.
//
// For packs of at most kDecodeMaxSeg segments of at most kDecodeMaxM tiles,
// every wave derives its workgroup's item of the planner's list (same order:
// tile index descending, segments in order) straight from cu_seqlens, which
// saves the planner launch and the dependency on it.  The waves of a
// workgroup compute the same result independently, with no LDS and no
// barrier.  With nt_b the tile count of segment b, the items of tile index
// m' >= m number S(m) = sum_b max(0, nt_b - m), so the group of item r is the
// largest m with S(m) > r (binary search), and within it the item is the
// (r - S(m+1))-th segment, in order, with nt_b > m.
// ---------------------------------------------------------------------------
constexpr int kDecodeMaxM = 256;
constexpr int kDecodeMaxSeg = 256;

// Work list handed to the attention kernels: the planner's output, or
// tiles == nullptr when each workgroup decodes its item.  report_ok = false
// (a second list of one call, written after the first) writes the status word
// only on an error, so that it cannot clear the first list's error.
struct WorkList {
  const int2* tiles;
  const int32_t* count;
  int32_t n_seg;
  int32_t* status;
  bool report_ok = true;
};

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off, 64));
  return x;
}

// Item r of the heavy-first list of (segment, TILE-row tile) pairs.  The
// result is wave-uniform and the same in every wave.  Returns false when there
// is no item r or cu_seqlens is invalid; workgroup 0 then, and on success
// when report_ok, writes the status word.
template <int TILE>
__device__ bool decode_work_item(const int32_t* __restrict__ cu, int n_seg, int T, int r, int2* item,
                                 int32_t* __restrict__ status, bool report_ok) {
  constexpr int J = kDecodeMaxSeg / 64;       // segments per lane
  const int lane = threadIdx.x & 63;
  int nt[J];
  bool bad = false;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int b = 64 * j + lane;
    nt[j] = 0;
    if (b < n_seg) {
      const int a = cu[b], c = cu[b + 1];
      if (c < a) bad = true;
      else nt[j] = (int)min(((int64_t)c - a + TILE - 1) / TILE, (int64_t)kDecodeMaxM + 1);
    }
  }
  if (lane == 0 && (cu[0] != 0 || cu[n_seg] != T)) bad = true;
  int M = 0;
#pragma unroll
  for (int j = 0; j < J; ++j) M = max(M, nt[j]);
  M = __builtin_amdgcn_readfirstlane(wave_max(M));
  const bool any_bad = __builtin_amdgcn_ballot_w64(bad) != 0;
  if (blockIdx.x == 0 && threadIdx.x == 0 && (report_ok || any_bad || M > kDecodeMaxM))
    *status = any_bad ? PVB_E_BAD_CU_SEQLENS : M > kDecodeMaxM ? PVB_E_UNSUPPORTED : PVB_OK;
  if (any_bad || M > kDecodeMaxM) return false;
  auto S = [&](int m) {
    int x = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) x += max(0, nt[j] - m);
    return __builtin_amdgcn_readfirstlane(wave_sum(x));
  };
  if (r >= S(0)) return false;
  int lo = 0, hi = M - 1;                       // S(lo) > r holds throughout
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (S(mid) > r) lo = mid;
    else hi = mid - 1;
  }
  int k = r - S(lo + 1);
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const uint64_t mask = __builtin_amdgcn_ballot_w64(nt[j] > lo);
    const int cnt = __builtin_popcountll(mask);
    if (k < cnt) {
      uint64_t mm = mask;
      for (int i = 0; i < k; ++i) mm &= mm - 1;   // drop the k lowest set bits
      // the values are the same in every lane; say so to the compiler, so
      // that what derives from them stays in scalar registers
      *item = make_int2(__builtin_amdgcn_readfirstlane(64 * j + __builtin_ctzll(mm)),
                        __builtin_amdgcn_readfirstlane(lo));
      return true;
    }
    k -= cnt;
  }
  return false;                                  // not reached
}

// Query head h and key/value head hk of head slot r in [0, H) (grouped heads:
// query head h reads key/value head h / (H / Hk)).  Slot r = gi Hk + hk puts
// the query heads of one group Hk slots apart, so with Hk a multiple of 8 a
// group's workgroups land on one XCD (and share its L2) under the
// round-robin dispatch of workgroups over the XCDs.  Hk = H gives h = r.
struct HeadPair {
  int h, hk;
};
__device__ __forceinline__ HeadPair head_of_slot(int r, int H, int Hk) {
  if (Hk == H) return {r, r};   // one query head per key/value head: no division
  const int hk = r % Hk;
  return {hk * (H / Hk) + r / Hk, hk};
}

// The keys that query row r (local) of a slice may use: [lo(r), hi(r)],
// clipped to [0, Lk) when BAND (empty when lo > hi).  delta = Lk - Lq aligns
// the causal clamp to the bottom right; wl / wr < 0 leave that side
// unbounded ("Packing与 FlashAttention Varlen", section 5: the key-block clamp
// (m+1) BM + L_k - L_q + window_right).  Without BAND it is causal
// self-attention, [0, r]; callers still bound keys by Lk themselves.
template <bool BAND>
struct KeyBand {
  int Lk, delta, wl, wr;
  __device__ __forceinline__ int hi(int r) const {
    if constexpr (BAND) return wr < 0 ? Lk - 1 : min(Lk - 1, r + delta + wr);
    else return r;
  }
  __device__ __forceinline__ int lo(int r) const {
    if constexpr (BAND) return wl < 0 ? 0 : max(0, r + delta - wl);
    else return 0;
  }
};

// Work items listed on the host from the host mirror of cu_seqlens and
// handed to the kernel with its launch arguments (read through the scalar
// cache, no dependent memory round trip): item r is the tile m[r] of the
// segment that starts at token seg0[r] and holds len[r] tokens, in the
// planner's order.  Used for small self-attention launches when the mirror is
// given; the kernel then does not read cu_seqlens.
constexpr int kHostItemsMax = 448;
struct HostItems {
  int32_t n;
  int32_t seg0[kHostItemsMax];
  int32_t len_m[kHostItemsMax];   // len << 8 | m  (len <= 32768, m < 256)
};
struct NoHostItems {};

// The item of workgroup tau: from the planner list, or decoded in place.
template <int TILE, bool DECODE>
__device__ __forceinline__ bool work_item(const WorkList& wl, const int32_t* __restrict__ cu, int T, int tau,
                                          int2* item) {
  if constexpr (DECODE) {
    return decode_work_item<TILE>(cu, wl.n_seg, T, tau, item, wl.status, wl.report_ok);
  } else {
    if (tau >= *wl.count) return false;
    *item = wl.tiles[tau];
    return true;
  }
}

// Whether a launch of this shape decodes its items in place: only small
// launches, where the planner's launch and the dependency on it are a
// noticeable share of the call (measured: 20 us of a 60 us short-pack call,
// against 1% extra on a 2048-workgroup launch).
constexpr size_t kDecodeMaxGrid = 1024;
inline bool decode_in_kernel(int32_t T, int32_t n_seg, int32_t tile, size_t grid) {
  return grid > 0 && grid <= kDecodeMaxGrid && n_seg <= kDecodeMaxSeg &&
         ((int64_t)T + tile - 1) / tile <= kDecodeMaxM;
}

}  // namespace pvb
