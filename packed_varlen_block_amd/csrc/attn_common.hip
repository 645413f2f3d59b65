// Work-item planner for the attention launches, and host-side helpers.
//
// The grid of an attention launch is sized from host-known bounds only (T, H,
// n_seg): a device-resident cu_seqlens is never copied back.  This one-workgroup
// kernel turns cu_seqlens into the list of (segment, tile) pairs that carry
// work, heaviest first, so that no workgroup is spent on a tile past the end
// of a short segment (in contrast to a grid sized by the longest segment whose
// surplus blocks exit, as in "Packing与 FlashAttention Varlen", section 5).
#include <algorithm>

#include "pvb_device.hpp"

namespace pvb {

namespace {

// Inclusive sum over the workgroup (kPlanThreads threads); `wsum` is LDS
// scratch of kPlanThreads/64 ints.  Returns the inclusive prefix and the total.
__device__ int block_inclusive_scan(int x, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  if (threadIdx.x < 64) {
    int v = threadIdx.x < kPlanThreads / 64 ? wsum[threadIdx.x] : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int y = __shfl_up(v, off, 64);
      if (lane >= off) v += y;
    }
    if (threadIdx.x < kPlanThreads / 64) wsum[threadIdx.x] = v;
  }
  __syncthreads();
  const int before = w > 0 ? wsum[w - 1] : 0;
  *total = wsum[kPlanThreads / 64 - 1];
  __syncthreads();
  return x + before;
}

}  // namespace

__global__ void __launch_bounds__(kPlanThreads)
plan_tiles_kernel(const int32_t* __restrict__ cu, int n_seg, int T, int tile,
                  int2* __restrict__ tiles, int32_t* __restrict__ count, int32_t* __restrict__ status,
                  int report_ok) {
  __shared__ int s_nt[kPlanChunk];
  __shared__ int s_off[kPlanMaxM];  // counts per group, then their exclusive offsets
  __shared__ int s_wsum[kPlanThreads / 64];
  __shared__ int s_bad, s_maxm;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_bad = 0;
    s_maxm = 0;
  }
  __syncthreads();

  // 1. validate cu_seqlens (first 0, non-decreasing, last T); tiles per segment
  int bad = 0, mx = 0;
  for (int b = tid; b < n_seg; b += kPlanThreads) {
    const int a = cu[b], c = cu[b + 1];
    if (c < a) bad = 1;
    else mx = max(mx, (int)(((int64_t)(c - a) + tile - 1) / tile));
  }
  if (tid == 0 && (cu[0] != 0 || cu[n_seg] != T)) bad = 1;
  if (bad) atomicOr(&s_bad, 1);
  if (mx) atomicMax(&s_maxm, mx);
  __syncthreads();
  const int M = s_maxm;
  if (s_bad || M > kPlanMaxM) {
    if (tid == 0) {
      *status = s_bad ? PVB_E_BAD_CU_SEQLENS : PVB_E_UNSUPPORTED;
      *count = 0;
    }
    return;
  }

  // 2. group m holds the segments with more than m tiles; count them
  for (int m = tid; m < M; m += kPlanThreads) s_off[m] = 0;
  for (int c0 = 0; c0 < n_seg; c0 += kPlanChunk) {
    const int nc = min(kPlanChunk, n_seg - c0);
    __syncthreads();
    for (int i = tid; i < nc; i += kPlanThreads)
      s_nt[i] = (int)(((int64_t)(cu[c0 + i + 1] - cu[c0 + i]) + tile - 1) / tile);
    __syncthreads();
    for (int m = tid; m < M; m += kPlanThreads) {
      int c = 0;
      for (int i = 0; i < nc; ++i) c += s_nt[i] > m;
      s_off[m] += c;
    }
  }
  __syncthreads();

  // 3. exclusive offsets with the largest m first
  int carry = 0;
  for (int j0 = 0; j0 < M; j0 += kPlanThreads) {
    const int j = j0 + tid;
    const int v = j < M ? s_off[M - 1 - j] : 0;
    int total;
    const int incl = block_inclusive_scan(v, s_wsum, &total);
    if (j < M) s_off[M - 1 - j] = carry + incl - v;
    carry += total;
  }
  __syncthreads();
  if (tid == 0) {
    *count = carry;
    if (report_ok) *status = PVB_OK;
  }

  // 4. emit: inside group m, segments in order
  for (int m0 = 0; m0 < M; m0 += kPlanThreads) {
    const int m = m0 + tid;
    int pos = m < M ? s_off[m] : 0;
    for (int c0 = 0; c0 < n_seg; c0 += kPlanChunk) {
      const int nc = min(kPlanChunk, n_seg - c0);
      __syncthreads();
      for (int i = tid; i < nc; i += kPlanThreads)
        s_nt[i] = (int)(((int64_t)(cu[c0 + i + 1] - cu[c0 + i]) + tile - 1) / tile);
      __syncthreads();
      if (m < M) {
        for (int i = 0; i < nc; ++i) {
          const int nt = s_nt[i];
          if (nt > m) tiles[pos++] = make_int2(c0 + i, m);
        }
      }
    }
  }
}

size_t plan_capacity(int32_t T, int32_t n_seg, int32_t tile) {
  // sum_b ceil(L_b / tile) <= (T + n_b * (tile - 1)) / tile over the n_b
  // non-empty segments, and n_b <= min(n_seg, T): zero-length segments add
  // no tiles
  const int64_t nb = std::min<int64_t>(n_seg, T);
  return (size_t)(((int64_t)T + nb * (tile - 1)) / tile);
}

pvb_status check_cross_args(const int32_t* h_cu_q, const int32_t* d_cu_k, const int32_t* h_cu_k,
                            int32_t n_seg, int32_t T_q, int32_t T_k, int32_t wl, int32_t wr) {
  if (h_cu_q == nullptr || h_cu_k == nullptr || d_cu_k == nullptr || T_k < 0 || T_q < 0 || n_seg < 0 ||
      wl < -1 || wr < -1)
    return PVB_E_INVALID_ARG;
  const pvb_status sq = check_host_cu(h_cu_q, n_seg, T_q);
  if (sq != PVB_OK) return sq;
  return check_host_cu(h_cu_k, n_seg, T_k);
}

pvb_status check_host_cu(const int32_t* h_cu, int32_t n_seg, int32_t T) {
  if (h_cu == nullptr) return PVB_OK;
  if (h_cu[0] != 0 || h_cu[n_seg] != T) return PVB_E_BAD_CU_SEQLENS;
  for (int32_t b = 0; b < n_seg; ++b)
    if (h_cu[b + 1] < h_cu[b]) return PVB_E_BAD_CU_SEQLENS;
  return PVB_OK;
}

}  // namespace pvb
