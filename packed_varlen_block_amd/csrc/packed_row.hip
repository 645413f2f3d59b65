// Packed-row metadata on the device: cu_seqlens by a prefix scan of the
// segment lengths, then per-cell local positions and occurrence segment ids
// ("Packing与 FlashAttention Varlen", sections 1-3; "Pack sequences without
// joining their contexts", "Fill only the current row"), with an optional
// next-token gather that keeps every pair inside its own document ("Form pairs
// inside each source range"); and the reverse direction, cu_seqlens compiled
// back from the reset points of a position stream (section 3; section 6 for
// the separate text-position plane that carries the boundaries when the
// rotary coordinates repeat).
#include "pvb_device.hpp"

namespace pvb {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kFillThreads = 256;

// One workgroup scans all lengths in chunks of kScanThreads, carrying the sum.
__global__ void __launch_bounds__(kScanThreads)
scan_lengths_kernel(const int32_t* __restrict__ lengths, int n, int capacity,
                    int32_t* __restrict__ cu, int32_t* __restrict__ max_seqlen,
                    int32_t* __restrict__ status) {
  __shared__ int64_t s_wsum[kScanThreads / 64];
  __shared__ int s_flags, s_max;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) {
    s_flags = 0;
    s_max = 0;
  }
  __syncthreads();
  int64_t carry = 0;
  int flags = 0, mx = 0;
  for (int i0 = 0; i0 < n; i0 += kScanThreads) {
    const int i = i0 + tid;
    int64_t x = 0;
    if (i < n) {
      const int L = lengths[i];
      if (L < 0) flags |= 1;
      else {
        x = L;
        mx = max(mx, L);
      }
    }
    // inclusive scan: within the wave, then across waves
    int64_t y = x;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int64_t t = __shfl_up(y, off, 64);
      if (lane >= off) y += t;
    }
    if (lane == 63) s_wsum[w] = y;
    __syncthreads();
    int64_t before = 0, total = 0;
    for (int k = 0; k < kScanThreads / 64; ++k) {
      if (k < w) before += s_wsum[k];
      total += s_wsum[k];
    }
    const int64_t incl = carry + before + y;
    if (i < n) {
      if (incl > INT32_MAX) flags |= 2;
      else cu[i + 1] = (int32_t)incl;
    }
    carry += total;
    __syncthreads();
  }
  if (flags) atomicOr(&s_flags, flags);
  atomicMax(&s_max, mx);
  __syncthreads();
  if (tid == 0) {
    cu[0] = 0;
    int st = PVB_OK;
    if (s_flags & 1) st = PVB_E_INVALID_ARG;
    else if (s_flags & 2) st = PVB_E_OVERFLOW;
    else if (carry > capacity) st = PVB_E_OVERSIZED;
    *status = st;
    if (max_seqlen != nullptr && st == PVB_OK) *max_seqlen = s_max;
  }
}

// One thread per cell: s(t) = max{b : cu[b] <= t} by binary search.
__global__ void __launch_bounds__(kFillThreads)
fill_row_kernel(const int32_t* __restrict__ cu, int n, int capacity, int base,
                int32_t* __restrict__ pos, int32_t* __restrict__ seg,
                const int32_t* __restrict__ tokens, const int64_t* __restrict__ tok_off,
                int32_t* __restrict__ inputs, int32_t* __restrict__ targets,
                uint8_t* __restrict__ valid, const int32_t* __restrict__ status) {
  const int t = blockIdx.x * kFillThreads + threadIdx.x;
  if (t >= capacity || *status != PVB_OK) return;
  const int total = cu[n];
  if (t < total) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cu[mid] <= t) lo = mid;
      else hi = mid - 1;
    }
    const int j = t - cu[lo];
    pos[t] = j;
    seg[t] = base + lo;
    if (tokens != nullptr) {
      const int64_t off = tok_off[lo] + j;
      if (inputs != nullptr) inputs[t] = tokens[off];
      if (targets != nullptr) targets[t] = tokens[off + 1];
    }
    if (valid != nullptr) valid[t] = 1;
  } else {
    pos[t] = 0;
    seg[t] = -1;
    if (inputs != nullptr) inputs[t] = -1;
    if (targets != nullptr) targets[t] = -1;
    if (valid != nullptr) valid[t] = 0;
  }
}

// Block reductions over kScanThreads threads through LDS (`red` holds one
// int per wave); every thread gets the result.
__device__ int block_sum(int x, int* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  x = wave_sum(x);
  __syncthreads();
  if (lane == 0) red[w] = x;
  __syncthreads();
  int t = 0;
  for (int k = 0; k < kScanThreads / 64; ++k) t += red[k];
  return t;
}
__device__ int block_min(int x, int* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = min(x, __shfl_xor(x, off, 64));
  __syncthreads();
  if (lane == 0) red[w] = x;
  __syncthreads();
  int t = INT32_MAX;
  for (int k = 0; k < kScanThreads / 64; ++k) t = min(t, red[k]);
  return t;
}

// One workgroup: the start tokens of a position stream (position == 0, or ==
// the smallest position), in order, then T, are cu_seqlens; max_seqlen is the
// largest difference.  The stream is read in chunks of kSlices x kScanThreads
// tokens, slice-major (token c0 + k kScanThreads + thread), so every load is
// coalesced and a thread's kSlices loads are in flight together.  Passes: the
// sentinel (min mode); the count, checked against the output capacity before
// anything is written (skipped when the capacity is at least T + 1, which no
// count can exceed); the ordered write, where a start's rank is its lane
// rank in the wave's ballot plus the counts of all earlier (slice, wave)
// pairs; and a read-back of the written boundaries for the largest difference.
constexpr int kSlices = 16;
constexpr int kChunk = kSlices * kScanThreads;
constexpr int kWaves = kScanThreads / 64;

__global__ void __launch_bounds__(kScanThreads)
boundaries_kernel(const int32_t* __restrict__ pos, int T, int use_min, int32_t* __restrict__ cu,
                  int cu_capacity, int32_t* __restrict__ n_seg_out, int32_t* __restrict__ max_seqlen,
                  int32_t* __restrict__ status) {
  __shared__ int red[kWaves];
  __shared__ int s_off[kSlices * kWaves];   // counts, then exclusive offsets, slice-major
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int x[kSlices];
  auto load = [&](const int32_t* src, int c0, int n) {
#pragma unroll
    for (int k = 0; k < kSlices; ++k) {
      const int t = c0 + k * kScanThreads + tid;
      x[k] = t < n ? src[t] : 0;
    }
  };
  int sent = 0;
  if (use_min) {
    int m = INT32_MAX;
    for (int c0 = 0; c0 < T; c0 += kChunk) {
      load(pos, c0, T);
#pragma unroll
      for (int k = 0; k < kSlices; ++k)
        if (c0 + k * kScanThreads + tid < T) m = min(m, x[k]);
    }
    sent = block_min(m, red);
  }
  int st = PVB_OK;
  if (T > 0 && pos[0] != sent) st = PVB_E_BAD_CU_SEQLENS;   // the first token must start a segment
  else if (cu_capacity <= T) {
    int cnt = 0;
    for (int c0 = 0; c0 < T; c0 += kChunk) {
      load(pos, c0, T);
#pragma unroll
      for (int k = 0; k < kSlices; ++k) cnt += c0 + k * kScanThreads + tid < T && x[k] == sent ? 1 : 0;
    }
    if (block_sum(cnt, red) + 1 > cu_capacity) st = PVB_E_OVERSIZED;   // more segments than the output holds
  }
  if (st != PVB_OK) {
    if (tid == 0) *status = st;
    return;
  }
  // ordered write: the r-th start token goes to cu[r]
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int carry = 0;
  for (int c0 = 0; c0 < T; c0 += kChunk) {
    load(pos, c0, T);
    uint64_t mask[kSlices];
#pragma unroll
    for (int k = 0; k < kSlices; ++k) {
      mask[k] = __builtin_amdgcn_ballot_w64(c0 + k * kScanThreads + tid < T && x[k] == sent);
      if (lane == 0) s_off[k * kWaves + w] = __builtin_popcountll(mask[k]);
    }
    __syncthreads();
    // wave 0: exclusive scan of the kSlices * kWaves counts in slice-major order
    if (w == 0) {
      constexpr int PER = kSlices * kWaves / 64;
      int v[PER], sum = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        v[i] = s_off[PER * lane + i];
        sum += v[i];
      }
      int y = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int z = __shfl_up(y, off, 64);
        if (lane >= off) y += z;
      }
      int run = y - sum;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        s_off[PER * lane + i] = run;
        run += v[i];
      }
      if (lane == 63) red[0] = y;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kSlices; ++k)
      if ((mask[k] >> lane) & 1ull)
        cu[carry + s_off[k * kWaves + w] + __builtin_popcountll(mask[k] & below)] = c0 + k * kScanThreads + tid;
    carry += red[0];
    __syncthreads();
  }
  const int n = carry;
  if (tid == 0) cu[n] = T;
  // make this workgroup's writes of cu visible to its own reads below
  __threadfence();
  __syncthreads();
  int mx = 0;
  for (int b = tid; b < n; b += kScanThreads) mx = max(mx, cu[b + 1] - cu[b]);
  mx = -block_min(-mx, red);
  if (tid == 0) {
    *n_seg_out = n;
    if (max_seqlen != nullptr) *max_seqlen = mx;
    *status = PVB_OK;
  }
}

}  // namespace
}  // namespace pvb

extern "C" pvb_status pvb_build_packed_row(const int32_t* d_lengths, int32_t n_seg, int32_t capacity,
                                           int32_t segment_base, int32_t* d_cu, int32_t* d_pos,
                                           int32_t* d_seg, int32_t* d_max_seqlen,
                                           const int32_t* d_tokens, const int64_t* d_tok_off,
                                           int32_t* d_inputs, int32_t* d_targets, uint8_t* d_valid,
                                           int32_t* d_status, void* stream) {
  using namespace pvb;
  if (n_seg < 0 || capacity < 0 || segment_base < 0 || d_cu == nullptr || d_status == nullptr)
    return PVB_E_INVALID_ARG;
  if (n_seg > 0 && d_lengths == nullptr) return PVB_E_INVALID_ARG;
  if (capacity > 0 && (d_pos == nullptr || d_seg == nullptr)) return PVB_E_INVALID_ARG;
  if (n_seg > PVB_MAX_COUNT || capacity > PVB_MAX_COUNT) return PVB_E_OVERFLOW;
  if ((int64_t)segment_base + n_seg > (int64_t)INT32_MAX + 1) return PVB_E_OVERFLOW;
  const bool want_tokens = d_inputs != nullptr || d_targets != nullptr;
  if (want_tokens && (d_tokens == nullptr || d_tok_off == nullptr)) return PVB_E_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  scan_lengths_kernel<<<1, kScanThreads, 0, s>>>(d_lengths, n_seg, capacity, d_cu, d_max_seqlen,
                                                 d_status);
  if (hipGetLastError() != hipSuccess) return PVB_E_HIP;
  if (capacity > 0) {
    const int blocks = (capacity + kFillThreads - 1) / kFillThreads;
    fill_row_kernel<<<blocks, kFillThreads, 0, s>>>(d_cu, n_seg, capacity, segment_base, d_pos,
                                                    d_seg, want_tokens ? d_tokens : nullptr,
                                                    d_tok_off, d_inputs, d_targets, d_valid,
                                                    d_status);
    if (hipGetLastError() != hipSuccess) return PVB_E_HIP;
  }
  return PVB_OK;
}

extern "C" pvb_status pvb_boundaries_from_positions(const int32_t* d_pos, int32_t T, int32_t sentinel,
                                                    int32_t* d_cu, int32_t cu_capacity,
                                                    int32_t* d_n_seg, int32_t* d_max_seqlen,
                                                    int32_t* d_status, void* stream) {
  using namespace pvb;
  if (T < 0 || (T > 0 && d_pos == nullptr) || d_cu == nullptr || cu_capacity < 1 ||
      d_n_seg == nullptr || d_status == nullptr)
    return PVB_E_INVALID_ARG;
  if (sentinel != PVB_SENTINEL_ZERO && sentinel != PVB_SENTINEL_MIN) return PVB_E_INVALID_ARG;
  if (T > PVB_MAX_COUNT) return PVB_E_OVERFLOW;   // also keeps T + 1 boundaries within int32
  hipStream_t s = static_cast<hipStream_t>(stream);
  boundaries_kernel<<<1, kScanThreads, 0, s>>>(d_pos, T, sentinel == PVB_SENTINEL_MIN ? 1 : 0, d_cu,
                                               cu_capacity, d_n_seg, d_max_seqlen, d_status);
  return hipGetLastError() == hipSuccess ? PVB_OK : PVB_E_HIP;
}
