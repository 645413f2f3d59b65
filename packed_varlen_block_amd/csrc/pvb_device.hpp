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
// ordered heaviest first: by m descending when `ascending_work` is false (the
// forward, where q-tile m reads m+1 key tiles) or by (ntiles_b - 1 - m)
// descending when it is true (the backward, where key tile m of segment b
// visits ntiles_b - m query tiles), segments in order within a group.  Items
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
plan_tiles_kernel(const int32_t* __restrict__ cu, int n_seg, int T, int tile, int backward,
                  int2* __restrict__ tiles, int32_t* __restrict__ count, int32_t* __restrict__ status);

// Host helpers (defined in attn_common.hip).
size_t plan_capacity(int32_t T, int32_t n_seg, int32_t tile);
pvb_status check_host_cu(const int32_t* h_cu, int32_t n_seg, int32_t T);

}  // namespace pvb
