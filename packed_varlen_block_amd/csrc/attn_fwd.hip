// Forward block-causal varlen attention on gfx950 matrix cores.
//
// What is computed ("Packing与 FlashAttention Varlen", sections 1 and 5;
// "Pack sequences without joining their contexts", "Permission depends on the
// example"): for every segment [cu[b], cu[b+1]) and head h, query i attends to
// keys j of the same segment with j <= i; O and LSE are written at the
// query's own flat rows.
//
// One workgroup = one work item (segment b, query tile m of 128 rows, head h)
// taken from the planner's heaviest-first list.  Its 4 waves own 32 query rows
// each.  Per K/V tile (64 keys; 32 when segments are short on average):
//   * K and V rows of the segment are copied global -> LDS asynchronously
//     (16-byte copies into a double-buffered, XOR-swizzled tile: the copy of
//     tile n+1 overlaps the math on tile n),
//   * S^T = K Q^T on 32x32x16 bf16 MFMAs with Q held in registers, so that
//     each lane owns one query column and the row max/sum of the online
//     softmax is in-lane plus one half-wave exchange,
//   * O^T += V^T P^T, where V^T fragments come straight from the row-major V
//     tile through the LDS transpose read and P never leaves registers.
// Key tiles wholly above the diagonal are never visited; masking is applied
// only on tiles that cross the diagonal or the segment end.  The running max
// is raised lazily (see kSlack), so most tiles skip the rescale of O.  A bf16 O
// is staged through LDS and stored as whole rows.
#include <algorithm>
#include <type_traits>

#include "pvb_device.hpp"

namespace pvb {
namespace {

constexpr int kFwdBM = 128;   // query rows per work item
constexpr int kFwdThreads = 256;

// BN keys per K/V tile: 64 for long segments; 32 for short ones, where the
// smaller register and LDS footprint lets three workgroups share a CU.
// BAND: separate key boundaries cu_k (T_k keys) and a key band per query row
// (bottom-right causal alignment and local windows, see KeyBand); without it,
// causal self-attention over cu.
// MODE: 0 the planner's list, 1 items decoded in the kernel, 2 items listed
// on the host and passed in `hi` (self-attention only).
template <int D, bool SPLIT, typename OutT, int MODE, int BN, bool BAND>
__global__ void __launch_bounds__(kFwdThreads, BN == 32 ? 3 : 2)
attn_fwd_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                const bf16* __restrict__ v, const int32_t* __restrict__ cu,
                const WorkList wl, int H, int Hk, int T,
                float scale_log2, OutT* __restrict__ o, float* __restrict__ lse,
                const int32_t* __restrict__ cu_k, int T_k, int win_left, int win_right,
                const std::conditional_t<MODE == 2, HostItems, NoHostItems> hi) {
  constexpr int BM = kFwdBM;
  constexpr int NB = BN / 32;    // 32-key blocks per tile
  constexpr int KSTEPS = D / 16;    // k-steps of S^T = K Q^T
  constexpr int DBLK = D / 32;      // 32-wide feature blocks of O^T
  // The running max used for the exponentials is raised only when a tile's
  // max exceeds it by more than kSlack (log2 units), so most tiles skip the
  // rescale of O and the row sum; probabilities stay below 2^kSlack.
  constexpr float kSlack = 8.f;

  __shared__ __attribute__((aligned(16))) bf16 sK[2][BN * D];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][BN * D];

  const int tau = blockIdx.x / H;
  const HeadPair hp = head_of_slot(blockIdx.x - tau * H, H, Hk);
  const int h = hp.h;
  int seg0, L, m_tile, sidx = 0;
  if constexpr (MODE == 2) {
    // the launch holds exactly the listed items; the mirror was checked on the host
    if (blockIdx.x == 0 && threadIdx.x == 0) *wl.status = PVB_OK;
    seg0 = hi.seg0[tau];
    L = hi.len_m[tau] >> 8;
    m_tile = hi.len_m[tau] & 255;
  } else {
    int2 tm;
    if (!work_item<BM, MODE == 1>(wl, cu, T, tau, &tm)) return;
    sidx = tm.x;
    seg0 = cu[sidx];
    L = cu[sidx + 1] - seg0;                   // query rows of the slice
    m_tile = tm.y;
  }
  int seg0k = seg0, Lk = L;                    // its keys
  if constexpr (BAND) {
    static_assert(MODE != 2, "host-listed items are for self-attention");
    // clipped to [0, T_k] so that no access leaves the key tensors (cu_k is
    // validated on the host)
    seg0k = min(max(cu_k[sidx], 0), T_k);
    Lk = min(max(cu_k[sidx + 1] - seg0k, 0), T_k - seg0k);
  }
  const KeyBand<BAND> band{Lk, Lk - L, win_left, win_right};
  const int q0 = m_tile * BM;
  const int rs = H * D;      // row stride of Q and O (elements)
  const int rs_kv = Hk * D;  // row stride of K and V
  const int64_t base = ((int64_t)seg0 * H + h) * D;
  const int64_t base_kv = ((int64_t)seg0k * Hk + hp.hk) * D;
  const bf16* qs = q + base;
  const bf16* ks = k + base_kv;
  const bf16* vs = v + base_kv;

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, lq = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qrow = q0 + 32 * w + lq;     // this lane's query (local index)
  const int wq_first = q0 + 32 * w;      // wave-uniform
  const int wq_last = min(wq_first + 31, L - 1);
  const bool wave_active = wq_first < L;
  const int tr_row = (lane & 15) >> 2;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  bf16x8 qf[KSTEPS];
  if (qrow < L) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = *(const bf16x8*)(qs + qrow * rs + 16 * s + 8 * g);
  } else {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = bf16x8{};
  }

  f32x16 oacc[DBLK];
#pragma unroll
  for (int j = 0; j < DBLK; ++j) oacc[j] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  const int q_last = min(q0 + BM, L) - 1;
  // key tiles holding a key that some row of the tile may use
  int n_lo = 0, n_end = q_last / BN + 1;
  if constexpr (BAND) {
    const int klo = band.lo(q0), khi = band.hi(q_last);
    n_lo = klo / BN;
    n_end = khi >= klo ? khi / BN + 1 : n_lo;
  }
  const int nkv = n_end - n_lo;

  FullTileCopy<D, BN> full;
  full.init(rs_kv, w, lane);
  auto stage = [&](int row0, int b) {
    if (row0 + BN <= Lk) {
      full.issue(ks, rs_kv, row0, sK[b]);
      full.issue(vs, rs_kv, row0, sV[b]);
    } else {
      stage_rows<D, BN>(ks, rs_kv, row0, Lk, sK[b], w, lane);
      stage_rows<D, BN>(vs, rs_kv, row0, Lk, sV[b], w, lane);
    }
  };
  if (nkv > 0) stage(n_lo * BN, 0);
  wait_vmcnt<0>();              // Q fragments and this wave's copies of the first tile
  for (int n = n_lo; n < n_end; ++n) {
    const int b = (n - n_lo) & 1;
    // every wave's copies of tile n have landed, and every wave is done with
    // buffer b^1 (tile n-1), which now receives tile n+1
    lds_barrier();
    if (n + 1 < n_end) stage((n + 1) * BN, b ^ 1);
    const bf16* cK = sK[b];
    const bf16* cV = sV[b];
    const int key0 = n * BN;
    if (wave_active && key0 <= band.hi(wq_last) && key0 + BN - 1 >= band.lo(wq_first)) {
      // S^T = K Q^T: NB 32-key blocks.  The K operands are read kPf k-steps
      // ahead of their MFMAs.
      constexpr int kPf = 2;
      bf16x8 ka[KSTEPS][NB];
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int kb2 = 0; kb2 < NB; ++kb2) ka[s][kb2] = *(const bf16x8*)(cK + swz<D>(32 * kb2 + lq, 16 * s + 8 * g));
      f32x16 st[NB];
#pragma unroll
      for (int kb2 = 0; kb2 < NB; ++kb2) st[kb2] = mfma32(ka[0][kb2], qf[0], f32x16{});
#pragma unroll
      for (int s = 1; s < KSTEPS; ++s)
#pragma unroll
        for (int kb2 = 0; kb2 < NB; ++kb2) st[kb2] = mfma32(ka[s][kb2], qf[s], st[kb2]);
      __builtin_amdgcn_sched_group_barrier(0x100, NB * (kPf + 1), 0);
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);
        if (s + kPf + 1 < KSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, NB, 0);
      }
      // mask keys outside the row's band (later than the query when causal)
      // or past the slice's keys; only tiles that cross a band edge or the end
      if (!(key0 >= band.lo(wq_last) && key0 + BN - 1 <= band.hi(wq_first) && key0 + BN <= Lk)) {
        const int khi = band.hi(qrow), klo = band.lo(qrow);
#pragma unroll
        for (int kb2 = 0; kb2 < NB; ++kb2)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + 32 * kb2 + 8 * (i >> 2) + 4 * g + (i & 3);
            if (key > khi || key < klo || key >= Lk) st[kb2][i] = -INFINITY;
          }
      }
      // online softmax for this lane's query column (in log2 units)
      float mx = -INFINITY;
#pragma unroll
      for (int kb2 = 0; kb2 < NB; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[kb2][i]);
      mx = fmaxf(mx, swap_halves(mx)) * scale_log2;
      if (__builtin_amdgcn_ballot_w64(mx > m_run + kSlack) != 0) {
        const float m_new = fmaxf(m_run, mx);
        // a row with no key so far in a wave that rescales: -inf - -inf would
        // make alpha NaN (only rows of a band can have none)
        float alpha = fast_exp2(m_run - m_new);
        if constexpr (BAND) alpha = m_new == -INFINITY ? 1.f : alpha;
        l_run *= alpha;
#pragma unroll
        for (int j = 0; j < DBLK; ++j)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[j][i] *= alpha;
        m_run = m_new;
      }
      const float m_use = m_run == -INFINITY ? 0.f : m_run;
      float rsum = 0.f;
#pragma unroll
      for (int kb2 = 0; kb2 < NB; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(st[kb2][i] * scale_log2 - m_use);
          st[kb2][i] = p;
          rsum += p;
        }
      l_run += rsum + swap_halves(rsum);

      // O^T += V^T P^T over four 16-key k-steps.  k-slot 8g+e of this lane holds
      // key 16kk + 8(e/4) + 4g + e%4, which is where S^T's C layout put it.
#pragma unroll
      for (int kk = 0; kk < BN / 16; ++kk) {
        bf16x8 ph, pl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = st[kk >> 1][8 * (kk & 1) + e];
          ph[e] = (bf16)p;
          if constexpr (SPLIT) pl[e] = (bf16)(p - (float)ph[e]);
        }
        const int r0 = 16 * kk + 4 * g + tr_row;
#pragma unroll
        for (int j = 0; j < DBLK; ++j) {
          const int c = 32 * j + tr_col;
          const bf16x8 vf = cat(lds_read_tr(cV + swz<D>(r0, c)), lds_read_tr(cV + swz<D>(r0 + 8, c)));
          oacc[j] = mfma32(vf, ph, oacc[j]);
          if constexpr (SPLIT) oacc[j] = mfma32(vf, pl, oacc[j]);
        }
      }
    }
    if (n + 1 < n_end) wait_vmcnt<0>();   // this wave's copies of tile n+1
  }

  if constexpr (sizeof(OutT) == 2) {
    // bf16 O leaves through LDS: each wave stages its 32 rows (waves 0 and 1
    // in the K buffers, 2 and 3 in the V buffers, which every wave is done
    // with after the barrier) and then stores whole rows, 16 bytes per lane,
    // marked non-temporal.  Whole-row stores stream out during the kernel;
    // stored straight from the C layout (16-byte pieces of 32 rows per
    // instruction) O would wait in L2 for the kernel's end.
    lds_barrier();
    bf16* stg = (w < 2 ? &sK[0][0] : &sV[0][0]) + (w & 1) * 32 * D;
    if (!wave_active) return;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int j = 0; j < DBLK; ++j)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 r;
#pragma unroll
        for (int t = 0; t < 4; ++t) r[t] = (bf16)(oacc[j][4 * i4 + t] * inv);
        *(bf16x4*)(stg + swz<D>(lq, 32 * j + 8 * i4 + 4 * g)) = r;
      }
    constexpr int CPR = D / 8, RPI = 64 / CPR;   // 16-byte chunks per row, rows per wave-wide store
#pragma unroll
    for (int it = 0; it < 32 / RPI; ++it) {
      const int rr = it * RPI + lane / CPR, c = lane % CPR;
      const bf16x8 x = *(const bf16x8*)(stg + swz<D>(rr, 8 * c));
      if (wq_first + rr < L)
        __builtin_nontemporal_store(__builtin_bit_cast(f32x4, x),
                                    (f32x4*)(o + base + (int64_t)(wq_first + rr) * rs + 8 * c));
    }
    if (g == 0 && qrow < L) lse[(int64_t)h * T + seg0 + qrow] = (m_run + log2f(l_run)) * kLn2;
    return;
  }
  // fp32 O (its rows would not fit the 32-key kernel's LDS): straight from the C layout
  if (!wave_active || qrow >= L) return;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  OutT* op = o + base + (int64_t)qrow * rs;
#pragma unroll
  for (int j = 0; j < DBLK; ++j)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int col = 32 * j + 8 * i4 + 4 * g;
      *(float4*)(op + col) = make_float4(oacc[j][4 * i4] * inv, oacc[j][4 * i4 + 1] * inv,
                                         oacc[j][4 * i4 + 2] * inv, oacc[j][4 * i4 + 3] * inv);
    }
  if (g == 0) lse[(int64_t)h * T + seg0 + qrow] = (m_run + log2f(l_run)) * kLn2;
}

template <int D, bool SPLIT, typename OutT, int BN, bool BAND>
void launch_fwd_bb(const void* q, const void* k, const void* v, const int32_t* cu, const WorkList& wl,
                   int H, int Hk, int T, size_t grid, float scale_log2, void* o, float* lse,
                   const BandArgs& bd, const HostItems* hi, hipStream_t s) {
  if constexpr (!BAND) {
    if (hi != nullptr) {
      attn_fwd_kernel<D, SPLIT, OutT, 2, BN, false><<<dim3((unsigned)grid), kFwdThreads, 0, s>>>(
          (const bf16*)q, (const bf16*)k, (const bf16*)v, cu, wl, H, Hk, T, scale_log2, (OutT*)o, lse,
          bd.cu_k, bd.T_k, bd.wl, bd.wr, *hi);
      return;
    }
  }
  if (wl.tiles == nullptr)
    attn_fwd_kernel<D, SPLIT, OutT, 1, BN, BAND><<<dim3((unsigned)grid), kFwdThreads, 0, s>>>(
        (const bf16*)q, (const bf16*)k, (const bf16*)v, cu, wl, H, Hk, T, scale_log2, (OutT*)o, lse,
        bd.cu_k, bd.T_k, bd.wl, bd.wr, NoHostItems{});
  else
    attn_fwd_kernel<D, SPLIT, OutT, 0, BN, BAND><<<dim3((unsigned)grid), kFwdThreads, 0, s>>>(
        (const bf16*)q, (const bf16*)k, (const bf16*)v, cu, wl, H, Hk, T, scale_log2, (OutT*)o, lse,
        bd.cu_k, bd.T_k, bd.wl, bd.wr, NoHostItems{});
}

template <int D, bool SPLIT, typename OutT, int BN>
void launch_fwd_bn(const void* q, const void* k, const void* v, const int32_t* cu, const WorkList& wl,
                   int H, int Hk, int T, size_t grid, float scale_log2, void* o, float* lse,
                   const BandArgs& bd, const HostItems* hi, hipStream_t s) {
  if (bd.on) launch_fwd_bb<D, SPLIT, OutT, BN, true>(q, k, v, cu, wl, H, Hk, T, grid, scale_log2, o, lse, bd, hi, s);
  else launch_fwd_bb<D, SPLIT, OutT, BN, false>(q, k, v, cu, wl, H, Hk, T, grid, scale_log2, o, lse, bd, hi, s);
}

template <int D, bool SPLIT, typename OutT>
hipError_t launch_fwd(const void* q, const void* k, const void* v, const int32_t* cu,
                      const WorkList& wl, int H, int Hk, int T, size_t cap, float scale_log2, void* o,
                      float* lse, bool short_keys, const BandArgs& bd, const HostItems* hi, hipStream_t s) {
  // host-listed items: exactly one workgroup per (item, head)
  const size_t grid = (hi != nullptr ? (size_t)hi->n : cap) * (size_t)H;
  if (grid == 0) return hipSuccess;
  if (short_keys) launch_fwd_bn<D, SPLIT, OutT, 32>(q, k, v, cu, wl, H, Hk, T, grid, scale_log2, o, lse, bd, hi, s);
  else launch_fwd_bn<D, SPLIT, OutT, 64>(q, k, v, cu, wl, H, Hk, T, grid, scale_log2, o, lse, bd, hi, s);
  return hipGetLastError();
}

// The work list of a small self-attention launch, from the validated host
// mirror of cu_seqlens, in the planner's order (tile index descending,
// segments in order within a tile index).  False when it does not fit
// HostItems (then the device plans).
bool list_items_on_host(const int32_t* h_cu, int32_t n_seg, int tile, HostItems* out) {
  int mmax = 0;
  for (int32_t b = 0; b < n_seg; ++b) {
    const int32_t L = h_cu[b + 1] - h_cu[b];
    if (L > 32768) return false;
    mmax = std::max(mmax, (L + tile - 1) / tile);
  }
  int n = 0;
  for (int m = mmax - 1; m >= 0; --m)
    for (int32_t b = 0; b < n_seg; ++b) {
      const int32_t L = h_cu[b + 1] - h_cu[b];
      if ((L + tile - 1) / tile <= m) continue;
      if (n >= kHostItemsMax) return false;
      out->seg0[n] = h_cu[b];
      out->len_m[n] = (L << 8) | m;
      ++n;
    }
  out->n = n;
  return true;
}

size_t fwd_workspace(int32_t T, int32_t n_seg) {
  return 256 + plan_capacity(T, n_seg, kFwdBM) * sizeof(int2);
}

}  // namespace

size_t attn_fwd_workspace_bytes(int32_t T, int32_t n_seg) { return fwd_workspace(T, n_seg); }

}  // namespace pvb

namespace pvb {
namespace {
pvb_status fwd_call(const void* d_q, const void* d_k, const void* d_v, const int32_t* d_cu,
                    const int32_t* h_cu, int32_t n_seg, int32_t T, int32_t H, int32_t H_kv, int32_t d,
                    float softmax_scale, void* d_o, int32_t o_dtype, float* d_lse, int32_t precision,
                    void* workspace, size_t workspace_bytes, int32_t* d_status, const BandArgs& bd,
                    void* stream) {
  if (n_seg < 0 || T < 0 || H <= 0 || d_cu == nullptr || d_status == nullptr) return PVB_E_INVALID_ARG;
  if (H_kv <= 0 || H % H_kv != 0) return PVB_E_INVALID_ARG;
  if (n_seg > PVB_MAX_COUNT) return PVB_E_OVERFLOW;
  const int32_t T_k = bd.on ? bd.T_k : T;
  if ((T > 0 && (d_q == nullptr || d_o == nullptr || d_lse == nullptr)) ||
      (T_k > 0 && (d_k == nullptr || d_v == nullptr)))
    return PVB_E_INVALID_ARG;
  if (o_dtype != PVB_BF16 && o_dtype != PVB_F32) return PVB_E_INVALID_ARG;
  if (precision != PVB_PREC_BF16 && precision != PVB_PREC_SPLIT) return PVB_E_INVALID_ARG;
  if (!(softmax_scale > 0.f) || !(softmax_scale < INFINITY)) return PVB_E_INVALID_ARG;
  if (d != 64 && d != 128) return PVB_E_UNSUPPORTED;
  if ((int64_t)T * H * d >= ((int64_t)1 << 31) || (int64_t)T_k * H_kv * d >= ((int64_t)1 << 31))
    return PVB_E_UNSUPPORTED;
  const size_t cap = plan_capacity(T, n_seg, kFwdBM);
  if (!grid_fits(cap * (uint64_t)H, kFwdThreads)) return PVB_E_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < fwd_workspace(T, n_seg)) return PVB_E_WORKSPACE;
  const pvb_status hs = check_host_cu(h_cu, n_seg, T);
  if (hs != PVB_OK) return hs;

  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* count = static_cast<int32_t*>(workspace);
  int2* tiles = reinterpret_cast<int2*>(static_cast<char*>(workspace) + 256);
  // small self-attention packs with the host mirror: the items are listed on
  // the host and passed with the launch; otherwise small packs decode their
  // items in the kernel, and larger ones take the planner's list (the planner
  // writes the list and the status first)
  HostItems hitems;
  const bool host_list = h_cu != nullptr && !bd.on && n_seg <= kDecodeMaxSeg &&
                         list_items_on_host(h_cu, n_seg, kFwdBM, &hitems);
  const bool dec = host_list || decode_in_kernel(T, n_seg, kFwdBM, cap * (size_t)H);
  if (!dec) {
    plan_tiles_kernel<<<1, kPlanThreads, 0, s>>>(d_cu, n_seg, T, kFwdBM, tiles, count, d_status);
    if (hipGetLastError() != hipSuccess) return PVB_E_HIP;
  }
  const WorkList wl{dec ? nullptr : tiles, count, n_seg, d_status};
  // key extents shorter than 512 on average: 32-key tiles, three workgroups per CU
  const bool short_keys = (int64_t)T_k < 512 * (int64_t)n_seg;

  const float sl2 = softmax_scale * kLog2e;
  const bool split = precision == PVB_PREC_SPLIT, f32 = o_dtype == PVB_F32;
  hipError_t e;
#define PVB_FWD(D_, S_, T_) \
  e = launch_fwd<D_, S_, T_>(d_q, d_k, d_v, d_cu, wl, H, H_kv, T, cap, sl2, d_o, d_lse, short_keys, bd, \
                            host_list ? &hitems : nullptr, s)
  if (d == 128) {
    if (split) { if (f32) PVB_FWD(128, true, float); else PVB_FWD(128, true, bf16); }
    else { if (f32) PVB_FWD(128, false, float); else PVB_FWD(128, false, bf16); }
  } else {
    if (split) { if (f32) PVB_FWD(64, true, float); else PVB_FWD(64, true, bf16); }
    else { if (f32) PVB_FWD(64, false, float); else PVB_FWD(64, false, bf16); }
  }
#undef PVB_FWD
  return e == hipSuccess ? PVB_OK : PVB_E_HIP;
}
}  // namespace
}  // namespace pvb

extern "C" pvb_status pvb_varlen_attn_fwd_gqa(const void* d_q, const void* d_k, const void* d_v,
                                              const int32_t* d_cu, const int32_t* h_cu, int32_t n_seg,
                                              int32_t T, int32_t H, int32_t H_kv, int32_t d,
                                              float softmax_scale, void* d_o, int32_t o_dtype, float* d_lse,
                                              int32_t precision, void* workspace, size_t workspace_bytes,
                                              int32_t* d_status, void* stream) {
  return pvb::fwd_call(d_q, d_k, d_v, d_cu, h_cu, n_seg, T, H, H_kv, d, softmax_scale, d_o, o_dtype, d_lse,
                       precision, workspace, workspace_bytes, d_status, pvb::BandArgs{}, stream);
}

extern "C" pvb_status pvb_varlen_cross_attn_fwd(const void* d_q, const void* d_k, const void* d_v,
                                                const int32_t* d_cu_q, const int32_t* h_cu_q,
                                                const int32_t* d_cu_k, const int32_t* h_cu_k, int32_t n_seg,
                                                int32_t T_q, int32_t T_k, int32_t H, int32_t H_kv, int32_t d,
                                                int32_t window_left, int32_t window_right,
                                                float softmax_scale, void* d_o, int32_t o_dtype, float* d_lse,
                                                int32_t precision, void* workspace, size_t workspace_bytes,
                                                int32_t* d_status, void* stream) {
  using namespace pvb;
  const pvb_status hs = check_cross_args(h_cu_q, d_cu_k, h_cu_k, n_seg, T_q, T_k, window_left, window_right);
  if (hs != PVB_OK) return hs;
  const BandArgs bd{true, d_cu_k, T_k, window_left, window_right};
  return fwd_call(d_q, d_k, d_v, d_cu_q, h_cu_q, n_seg, T_q, H, H_kv, d, softmax_scale, d_o, o_dtype, d_lse,
                  precision, workspace, workspace_bytes, d_status, bd, stream);
}

extern "C" pvb_status pvb_varlen_attn_fwd(const void* d_q, const void* d_k, const void* d_v,
                                          const int32_t* d_cu, const int32_t* h_cu, int32_t n_seg,
                                          int32_t T, int32_t H, int32_t d, float softmax_scale,
                                          void* d_o, int32_t o_dtype, float* d_lse, int32_t precision,
                                          void* workspace, size_t workspace_bytes, int32_t* d_status,
                                          void* stream) {
  return pvb_varlen_attn_fwd_gqa(d_q, d_k, d_v, d_cu, h_cu, n_seg, T, H, H, d, softmax_scale, d_o, o_dtype,
                                 d_lse, precision, workspace, workspace_bytes, d_status, stream);
}
