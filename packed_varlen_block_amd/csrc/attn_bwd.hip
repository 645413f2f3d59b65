// Backward of block-causal varlen attention on gfx950 matrix cores.
//
// The gradient is the textbook one for softmax attention, restricted to the
// same per-segment causal ranges as the forward ("Pack sequences without
// joining their contexts", "Extend the existing storage and decoder": the same
// ranges drive forward and backward), so cross-segment derivatives are zero
// by construction:
//   D_i = dO_i . O_i,   P_ij = exp(scale q_i.k_j - LSE_i),   dP_ij = dO_i . v_j,
//   dS_ij = P_ij (dP_ij - D_i),  dV_j = sum_i P_ij dO_i,
//   dK_j = scale sum_i dS_ij q_i, dQ_i = scale sum_j dS_ij k_j.
//
// Kernels
//   bwd_pre   D = rowsum(dO * O) per (token, head); zeroes the fp32 dQ accumulator.
//   bwd_main  one workgroup per (segment, 128-key tile, head), heaviest first.
//             Its 4 waves own 32 keys each with K and V fragments in registers
//             and dK/dV accumulators in registers.  It walks the 64-row query
//             tiles from the diagonal to the segment end:
//               S = Q K^T and dP = dO V^T (Q, dO tiles staged in LDS),
//               P, dS in registers (lane = key column),
//               dV += P^T dO and dK += dS^T Q with dO/Q fragments read
//               transposed from LDS,
//               dS^T -> LDS, then dQ_tile = dS K split over the waves by
//               output block and added into the fp32 accumulator with atomics.
//             The next query tile is prefetched into registers during the
//             current one and lands in the other half of a double-buffered
//             LDS tile; barriers order LDS only, so atomics stay in flight.
//   bwd_dq    dQ accumulator -> bf16 (only for bf16 gradients).
#include "pvb_device.hpp"

namespace pvb {
namespace {

constexpr int kBwdBN = 128;   // keys per work item
constexpr int kBwdBM = 64;    // query rows per step
constexpr int kBwdThreads = 256;
constexpr int kPreThreads = 256;

template <int D, typename OT>
__global__ void __launch_bounds__(kPreThreads)
bwd_pre_kernel(const OT* __restrict__ o, const bf16* __restrict__ dout, int rows, int H, int T,
               float* __restrict__ delta, float* __restrict__ dq_acc,
               const int32_t* __restrict__ status) {
  if (*status != PVB_OK) return;
  constexpr int TPR = D / 8;                     // threads per (token, head) row
  constexpr int RPB = kPreThreads / TPR;         // rows per block
  const int r = blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = (threadIdx.x % TPR) * 8;
  float acc = 0.f;
  if (r < rows) {
    const int64_t off = (int64_t)r * D + c;
    const bf16x8 g = *(const bf16x8*)(dout + off);
    float ov[8];
    if constexpr (sizeof(OT) == 4) {
      const float4 a = *(const float4*)(o + off), b = *(const float4*)(o + off + 4);
      ov[0] = a.x; ov[1] = a.y; ov[2] = a.z; ov[3] = a.w;
      ov[4] = b.x; ov[5] = b.y; ov[6] = b.z; ov[7] = b.w;
    } else {
      const bf16x8 a = *(const bf16x8*)(o + off);
#pragma unroll
      for (int e = 0; e < 8; ++e) ov[e] = (float)a[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)g[e] * ov[e];
    *(float4*)(dq_acc + off) = make_float4(0.f, 0.f, 0.f, 0.f);
    *(float4*)(dq_acc + off + 4) = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int m = TPR / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (r < rows && threadIdx.x % TPR == 0) {
    const int t = r / H, h = r - t * H;
    delta[(int64_t)h * T + t] = acc;
  }
}

template <int D, bool SPLIT, typename GradT>
__global__ void __launch_bounds__(kBwdThreads, 1)
bwd_main_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                const bf16* __restrict__ dout, const float* __restrict__ lse,
                const float* __restrict__ delta, const int32_t* __restrict__ cu,
                const int2* __restrict__ tiles, const int32_t* __restrict__ n_tiles, int H, int T,
                float scale, float scale_log2, float* __restrict__ dq_acc,
                GradT* __restrict__ dk, GradT* __restrict__ dv) {
  constexpr int BN = kBwdBN, BM = kBwdBM;
  constexpr int QP = D + 8;         // pitch of the Q / dO / K tiles (elements)
  constexpr int TP = BM + 8;        // pitch of the dS^T tile [key][query]
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int CPR = D / 8;        // 16-byte chunks per row
  constexpr int QCH = BM * CPR / kBwdThreads;  // chunks per thread per Q (or dO) tile
  constexpr int NSPLIT = SPLIT ? 2 : 1;

  __shared__ __attribute__((aligned(16))) bf16 sQ[2][BM * QP];
  __shared__ __attribute__((aligned(16))) bf16 sdO[2][BM * QP];
  __shared__ __attribute__((aligned(16))) bf16 sK[BN * QP];
  __shared__ __attribute__((aligned(16))) bf16 sdST[NSPLIT][BN * TP];
  __shared__ float sLse[2][BM], sDel[2][BM];

  const int tau = blockIdx.x / H;
  const int h = blockIdx.x - tau * H;
  if (tau >= *n_tiles) return;
  const int2 tm = tiles[tau];
  const int seg0 = cu[tm.x];
  const int L = cu[tm.x + 1] - seg0;
  const int k0 = tm.y * BN;
  const int64_t rs = (int64_t)H * D;
  const int64_t base = ((int64_t)seg0 * H + h) * D;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 5, lq = lane & 31;
  const int kw0 = k0 + 32 * w;          // first key of this wave
  const int kcol = kw0 + lq;            // this lane's key column (local index)
  // transpose-read lane offsets: row (lane&15)>>2 of a 4-row group, column 16((lane>>4)&1) + 4(lane&3)
  const int tr_row = (lane & 15) >> 2;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // K and V fragments (B operands of S = Q K^T and dP = dO V^T)
  bf16x8 kf[KSTEPS], vf[KSTEPS];
  if (kcol < L) {
    const bf16* kp = k + base + kcol * rs + 8 * g;
    const bf16* vp = v + base + kcol * rs + 8 * g;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      kf[s] = *(const bf16x8*)(kp + 16 * s);
      vf[s] = *(const bf16x8*)(vp + 16 * s);
    }
  } else {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) kf[s] = vf[s] = bf16x8{};
  }
  // K tile, row-major, for the dQ product
  for (int c = tid; c < BN * CPR; c += kBwdThreads) {
    const int row = c / CPR, col = (c % CPR) * 8;
    const int key = k0 + row;
    *(uint4*)(sK + row * QP + col) = key < L ? *(const uint4*)(k + base + key * rs + col) : zero4();
  }

  // next query tile, prefetched into registers while the current one is used
  uint4 pq[QCH], pd[QCH];
  float plse = INFINITY, pdel = 0.f;
  auto fetch = [&](int jq) {
    const int qt0 = jq * BM;
#pragma unroll
    for (int r = 0; r < QCH; ++r) {
      const int c = tid + kBwdThreads * r;
      const int row = c / CPR, col = (c % CPR) * 8;
      const int qi = qt0 + row;
      if (qi < L) {
        pq[r] = *(const uint4*)(q + base + qi * rs + col);
        pd[r] = *(const uint4*)(dout + base + qi * rs + col);
      } else {
        pq[r] = zero4();
        pd[r] = zero4();
      }
    }
    if (tid < BM) {
      const int qi = qt0 + tid;
      plse = qi < L ? lse[(int64_t)h * T + seg0 + qi] * kLog2e : INFINITY;
      pdel = qi < L ? delta[(int64_t)h * T + seg0 + qi] : 0.f;
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int r = 0; r < QCH; ++r) {
      const int c = tid + kBwdThreads * r;
      const int row = c / CPR, col = (c % CPR) * 8;
      *(uint4*)(sQ[buf] + row * QP + col) = pq[r];
      *(uint4*)(sdO[buf] + row * QP + col) = pd[r];
    }
    if (tid < BM) {
      sLse[buf][tid] = plse;
      sDel[buf][tid] = pdel;
    }
  };

  f32x16 dkacc[DBLK], dvacc[DBLK];
#pragma unroll
  for (int j = 0; j < DBLK; ++j) dkacc[j] = dvacc[j] = f32x16{};

  const int jq0 = k0 / BM;
  const int jq_end = (L + BM - 1) / BM;
  fetch(jq0);
  stash(0);
  lds_barrier();
  for (int jq = jq0; jq < jq_end; ++jq) {
    const int buf = (jq - jq0) & 1;
    const int qt0 = jq * BM;
    const int qt_last = min(qt0 + BM, L) - 1;
    if (jq + 1 < jq_end) fetch(jq + 1);
    const bf16* cQ = sQ[buf];
    const bf16* cdO = sdO[buf];

    if (kw0 <= qt_last) {   // otherwise every key of this wave is later than every query
      f32x16 sacc[2] = {f32x16{}, f32x16{}}, pacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const bf16x8 qa = *(const bf16x8*)(cQ + (32 * qb + lq) * QP + 16 * s + 8 * g);
          const bf16x8 da = *(const bf16x8*)(cdO + (32 * qb + lq) * QP + 16 * s + 8 * g);
          sacc[qb] = mfma32(qa, kf[s], sacc[qb]);
          pacc[qb] = mfma32(da, vf[s], pacc[qb]);
        }
      }
      // P and dS; element i of block qb is query qt0 + 32qb + 8(i/4) + 4g + i%4
      const bool need_mask = qt0 < kw0 + 31 || qt0 + BM > L || kw0 + 32 > L;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ql = 32 * qb + 8 * (i >> 2) + 4 * g + (i & 3);
          float p = fast_exp2(sacc[qb][i] * scale_log2 - sLse[buf][ql]);
          if (need_mask && (kcol > qt0 + ql || qt0 + ql >= L || kcol >= L)) p = 0.f;
          sacc[qb][i] = p;
          pacc[qb][i] = p * (pacc[qb][i] - sDel[buf][ql]);
        }
      // dV += P^T dO and dK += dS^T Q.  k-slot 8g+e holds query 16kk + 8(e/4) + 4g + e%4.
#pragma unroll
      for (int kk = 0; kk < BM / 16; ++kk) {
        bf16x8 ph, pl, sh, sl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = sacc[kk >> 1][8 * (kk & 1) + e];
          const float ds = pacc[kk >> 1][8 * (kk & 1) + e];
          ph[e] = (bf16)p;
          sh[e] = (bf16)ds;
          if constexpr (SPLIT) {
            pl[e] = (bf16)(p - (float)ph[e]);
            sl[e] = (bf16)(ds - (float)sh[e]);
          }
        }
        const int roff = (16 * kk + 4 * g + tr_row) * QP + tr_col;
#pragma unroll
        for (int j = 0; j < DBLK; ++j) {
          const bf16x8 dof = cat(lds_read_tr(cdO + roff + 32 * j), lds_read_tr(cdO + roff + 8 * QP + 32 * j));
          const bf16x8 qtf = cat(lds_read_tr(cQ + roff + 32 * j), lds_read_tr(cQ + roff + 8 * QP + 32 * j));
          dvacc[j] = mfma32(ph, dof, dvacc[j]);
          dkacc[j] = mfma32(sh, qtf, dkacc[j]);
          if constexpr (SPLIT) {
            dvacc[j] = mfma32(pl, dof, dvacc[j]);
            dkacc[j] = mfma32(sl, qtf, dkacc[j]);
          }
        }
      }
      // dS^T -> LDS: row = this lane's key, four consecutive queries per store
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          bf16x4 hi, lo;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float ds = pacc[qb][4 * i4 + t];
            hi[t] = (bf16)ds;
            if constexpr (SPLIT) lo[t] = (bf16)(ds - (float)hi[t]);
          }
          const int off = (32 * w + lq) * TP + 32 * qb + 8 * i4 + 4 * g;
          *(bf16x4*)(&sdST[0][off]) = hi;
          if constexpr (SPLIT) *(bf16x4*)(&sdST[1][off]) = lo;
        }
    }
    lds_barrier();

    // dQ tile = dS K, one 32x32 output block at a time; only key steps that
    // belong to waves with work are visited
    const int n_ks = min(BN / 16, (qt_last - k0) / 16 + 1);
    for (int blk = w; blk < 2 * DBLK; blk += 4) {
      const int qb = blk & 1, j = blk >> 1;
      f32x16 acc = f32x16{};
      for (int ks = 0; ks < n_ks; ++ks) {
        const int r0 = 16 * ks + 8 * g + tr_row;
        const bf16* kaddr = sK + r0 * QP + 32 * j + tr_col;
        const bf16x8 bk = cat(lds_read_tr(kaddr), lds_read_tr(kaddr + 4 * QP));
#pragma unroll
        for (int p = 0; p < NSPLIT; ++p) {
          const bf16* saddr = &sdST[p][r0 * TP + 32 * qb + tr_col];
          const bf16x8 a = cat(lds_read_tr(saddr), lds_read_tr(saddr + 4 * TP));
          acc = mfma32(a, bk, acc);
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qi = qt0 + 32 * qb + 8 * (i >> 2) + 4 * g + (i & 3);
        if (qi < L) unsafeAtomicAdd(dq_acc + base + qi * rs + 32 * j + lq, acc[i] * scale);
      }
    }
    if (jq + 1 < jq_end) stash(buf ^ 1);
    lds_barrier();
  }

  // dK (scaled) and dV rows of this wave's keys
#pragma unroll
  for (int j = 0; j < DBLK; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kw0 + 8 * (i >> 2) + 4 * g + (i & 3);
      if (key < L) {
        const int64_t off = base + key * rs + 32 * j + lq;
        dk[off] = out_cast<GradT>(dkacc[j][i] * scale);
        dv[off] = out_cast<GradT>(dvacc[j][i]);
      }
    }
}

__global__ void bwd_dq_convert_kernel(const float* __restrict__ acc, bf16* __restrict__ out, int64_t n,
                                      const int32_t* __restrict__ status) {
  if (*status != PVB_OK) return;
  const int64_t i = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i >= n) return;
  const float4 a = *(const float4*)(acc + i), b = *(const float4*)(acc + i + 4);
  bf16x8 r;
  r[0] = (bf16)a.x; r[1] = (bf16)a.y; r[2] = (bf16)a.z; r[3] = (bf16)a.w;
  r[4] = (bf16)b.x; r[5] = (bf16)b.y; r[6] = (bf16)b.z; r[7] = (bf16)b.w;
  *(bf16x8*)(out + i) = r;
}

struct BwdLayout {
  size_t tiles_off, delta_off, dq_off, total;
};

BwdLayout bwd_layout(int32_t T, int32_t H, int32_t d, int32_t n_seg, int32_t grad_dtype) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  BwdLayout l;
  l.tiles_off = 256;
  l.delta_off = up(l.tiles_off + plan_capacity(T, n_seg, kBwdBN) * sizeof(int2));
  l.dq_off = up(l.delta_off + (size_t)H * T * sizeof(float));
  l.total = l.dq_off + (grad_dtype == PVB_F32 ? 0 : (size_t)T * H * d * sizeof(float));
  return l;
}

template <int D, bool SPLIT, typename GradT, typename OT>
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, const int32_t* cu, const int2* tiles, const int32_t* count,
                      int H, int T, size_t cap, float scale, float* delta, float* dq_acc, void* dq,
                      void* dk, void* dv, const int32_t* status, hipStream_t s) {
  const int rows = T * H;
  if (rows > 0) {
    constexpr int RPB = kPreThreads / (D / 8);
    bwd_pre_kernel<D, OT><<<(rows + RPB - 1) / RPB, kPreThreads, 0, s>>>(
        (const OT*)o, (const bf16*)dout, rows, H, T, delta, dq_acc, status);
  }
  const size_t grid = cap * (size_t)H;
  if (grid > 0)
    bwd_main_kernel<D, SPLIT, GradT><<<dim3((unsigned)grid), kBwdThreads, 0, s>>>(
        (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout, lse, delta, cu, tiles,
        count, H, T, scale, scale * kLog2e, dq_acc, (GradT*)dk, (GradT*)dv);
  if constexpr (sizeof(GradT) == 2) {
    const int64_t n = (int64_t)T * H * D;
    if (n > 0)
      bwd_dq_convert_kernel<<<(unsigned)((n / 8 + 255) / 256), 256, 0, s>>>(dq_acc, (bf16*)dq, n, status);
  }
  return hipGetLastError();
}

}  // namespace

size_t attn_bwd_workspace_bytes(int32_t T, int32_t H, int32_t d, int32_t n_seg, int32_t grad_dtype) {
  return bwd_layout(T, H, d, n_seg, grad_dtype).total;
}

}  // namespace pvb

extern "C" pvb_status pvb_varlen_attn_bwd(const void* d_q, const void* d_k, const void* d_v,
                                          const void* d_o, int32_t o_dtype, const void* d_do,
                                          const float* d_lse, const int32_t* d_cu, const int32_t* h_cu,
                                          int32_t n_seg, int32_t T, int32_t H, int32_t d,
                                          float softmax_scale, void* d_dq, void* d_dk, void* d_dv,
                                          int32_t grad_dtype, int32_t precision, void* workspace,
                                          size_t workspace_bytes, int32_t* d_status, void* stream) {
  using namespace pvb;
  if (n_seg < 0 || T < 0 || H <= 0 || d_cu == nullptr || d_status == nullptr) return PVB_E_INVALID_ARG;
  if (T > 0 && (d_q == nullptr || d_k == nullptr || d_v == nullptr || d_o == nullptr ||
                d_do == nullptr || d_lse == nullptr || d_dq == nullptr || d_dk == nullptr ||
                d_dv == nullptr))
    return PVB_E_INVALID_ARG;
  if (o_dtype != PVB_BF16 && o_dtype != PVB_F32) return PVB_E_INVALID_ARG;
  if (grad_dtype != PVB_BF16 && grad_dtype != PVB_F32) return PVB_E_INVALID_ARG;
  if (precision != PVB_PREC_BF16 && precision != PVB_PREC_SPLIT) return PVB_E_INVALID_ARG;
  if (!(softmax_scale > 0.f) || !(softmax_scale < INFINITY)) return PVB_E_INVALID_ARG;
  if (d != 64 && d != 128) return PVB_E_UNSUPPORTED;
  if ((int64_t)T * H * d > (int64_t)1 << 40 || (int64_t)T * H > 0x7fffffffLL) return PVB_E_UNSUPPORTED;
  const size_t cap = plan_capacity(T, n_seg, kBwdBN);
  if (cap * (size_t)H > 0x7fffffffULL) return PVB_E_UNSUPPORTED;
  const BwdLayout lay = bwd_layout(T, H, d, n_seg, grad_dtype);
  if (workspace == nullptr || workspace_bytes < lay.total) return PVB_E_WORKSPACE;
  const pvb_status hs = check_host_cu(h_cu, n_seg, T);
  if (hs != PVB_OK) return hs;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* count = reinterpret_cast<int32_t*>(ws);
  int2* tiles = reinterpret_cast<int2*>(ws + lay.tiles_off);
  float* delta = reinterpret_cast<float*>(ws + lay.delta_off);
  float* dq_acc = grad_dtype == PVB_F32 ? static_cast<float*>(d_dq) : reinterpret_cast<float*>(ws + lay.dq_off);
  plan_tiles_kernel<<<1, kPlanThreads, 0, s>>>(d_cu, n_seg, T, kBwdBN, 1, tiles, count, d_status);
  if (hipGetLastError() != hipSuccess) return PVB_E_HIP;

  const bool split = precision == PVB_PREC_SPLIT, gf32 = grad_dtype == PVB_F32, of32 = o_dtype == PVB_F32;
  hipError_t e = hipSuccess;
#define PVB_BWD(D_, S_, G_, O_)                                                                   \
  e = launch_bwd<D_, S_, G_, O_>(d_q, d_k, d_v, d_o, d_do, d_lse, d_cu, tiles, count, H, T, cap, \
                                 softmax_scale, delta, dq_acc, d_dq, d_dk, d_dv, d_status, s)
#define PVB_BWD_O(D_, S_, G_) \
  if (of32) PVB_BWD(D_, S_, G_, float); else PVB_BWD(D_, S_, G_, bf16)
#define PVB_BWD_G(D_, S_) \
  if (gf32) { PVB_BWD_O(D_, S_, float); } else { PVB_BWD_O(D_, S_, bf16); }
  if (d == 128) {
    if (split) { PVB_BWD_G(128, true); } else { PVB_BWD_G(128, false); }
  } else {
    if (split) { PVB_BWD_G(64, true); } else { PVB_BWD_G(64, false); }
  }
#undef PVB_BWD_G
#undef PVB_BWD_O
#undef PVB_BWD
  return e == hipSuccess ? PVB_OK : PVB_E_HIP;
}
