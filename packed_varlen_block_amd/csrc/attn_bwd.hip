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
// Kernels (one planner list of 128-row tiles serves both):
//   bwd_dq   (runs first) one workgroup per (segment, 128-query tile, head);
//            forms {LSE log2(e), D = rowsum(dO * O)} of its rows for the
//            dK/dV kernel, and is shaped like the forward: Q and dO fragments
//            in registers, K and V tiles copied global -> LDS
//            (double-buffered); S^T, dP^T and dS^T with each lane owning one
//            query column, and dQ^T += K^T dS^T with K^T read transposed from
//            LDS.
//   bwd_kv_pair  one workgroup per (segment, 64-key half of a planner tile,
//            head).  Wave pairs own 32 keys each and walk the 32-row query
//            tiles from the diagonal to the segment end (Q, dO copied
//            global -> LDS into a double-buffered ring, the next tile in flight
//            during the math on the current one).  In a pair one wave forms
//            S, P and dV += P^T dO, the other dP, dS = P (dP - D) with P
//            handed over through LDS, and dK += dS^T Q; the second operands
//            are read transposed from LDS.
// dQ is recomputed rather than accumulated across key tiles with atomics:
// device-scope float atomics are resolved past the per-XCD L2, and their
// traffic (about 4 bytes per permitted edge at 128-key tiles) costs more than
// the two extra matrix products.  Every gradient element is written once, so
// the backward is deterministic.
#include <mutex>

#include "pvb_device.hpp"

namespace pvb {
namespace {

constexpr int kTile = 128;       // rows per planner tile (two 64-key halves for dK/dV, queries for dQ)
constexpr int kKvBM = 32;        // query rows per dK/dV step
constexpr int kDqBN = 64;        // keys per dq step
constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// dK, dV with wave pairs
// ---------------------------------------------------------------------------
// One workgroup per (segment, 64-key tile, head); waves 2p and 2p+1 form pair
// p, owning keys k0 + 32p .. +31.  Per 32-row query step the even wave computes
// S = Q K^T, P = exp2(S scale log2e - LSE log2e) and dV += P^T dO; the odd wave
// computes dP = dO V^T, takes P from its partner through LDS, forms
// dS = P (dP - D) and accumulates dK += dS^T Q.  Each matrix product over the
// permitted (query, key) pairs is done once: S, dP, dV and dK, 16 MFMAs per
// wave and step.  Both roles run the same instruction stream up to role
// selects: first product A x (K or V fragment in registers) with A = Q or dO
// rows from LDS, then (P or dS) x (dO or Q, read transposed from LDS).
// Work items come from the key-side list (cu, T, wl); with BAND the query
// extents come from cu_q (T_q queries) and each key sees the query rows whose
// band holds it.
template <int D, bool SPLIT, typename GradT, bool DECODE, bool BAND>
__global__ void __launch_bounds__(kThreads, 3)
bwd_kv_pair_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                   const bf16* __restrict__ dout, const float2* __restrict__ ld,
                   const int32_t* __restrict__ cu, const WorkList wl, int H, int Hk, int T, float scale,
                   float scale_log2, GradT* __restrict__ dk, GradT* __restrict__ dv,
                   const int32_t* __restrict__ cu_q, int T_q, int win_left, int win_right) {
  constexpr int BN = kTile / 2, BM = kKvBM;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int PB = (D + 8) * 2;                // padded row pitch (bytes)
  constexpr int CP = D / 8 + 1;                  // 16-byte chunks per padded row
  constexpr int CPT = (BM * CP + 63) / 64;       // wave-wide copies per tile
  constexpr int NI = (2 * CPT + 3) / 4;          // copies per wave per stage (Q, dO, spare)
  constexpr int TILE_BYTES = CPT * 1024;
  constexpr int STAGE_BYTES = 4 * NI * 1024;
  constexpr int NST = 2;                         // ring of query tiles
  constexpr int COPIES = NI + 1;                 // + the {LSE, D} record copy

  __shared__ __attribute__((aligned(1024))) char ring[NST][STAGE_BYTES];
  // per ring slot: LSE log2e of the BM rows, then their D, both in C-layout order
  __shared__ __attribute__((aligned(16))) float sLD[NST][2 * BM];
  // P handed from the even to the odd wave of a pair: chunk j of lane l holds
  // its elements 4j .. 4j+3 (same lane, same C-layout position in both waves)
  __shared__ __attribute__((aligned(16))) float4 xbuf[2][4][64];

  // work item: 128-key planner tile tau, its 64-key half, key/value head hk;
  // the walk covers the query tiles of each of the group's G query heads
  const int tau = blockIdx.x / (2 * Hk);
  const int rem = blockIdx.x - tau * 2 * Hk;
  const int half = rem >= Hk ? 1 : 0;
  const int hk = rem - half * Hk;
  const int G = H / Hk;
  int2 tm;
  if (!work_item<kTile, DECODE>(wl, cu, T, tau, &tm)) return;
  const int seg0k = cu[tm.x];
  const int Lk = cu[tm.x + 1] - seg0k;                 // keys of the slice
  int seg0 = seg0k, Lq = Lk;                           // its query rows (clipped to [0, T_q])
  if constexpr (BAND) {
    seg0 = min(max(cu_q[tm.x], 0), T_q);
    Lq = min(max(cu_q[tm.x + 1] - seg0, 0), T_q - seg0);
  }
  const KeyBand<BAND> band{Lk, Lk - Lq, win_left, win_right};
  const int k0 = ((Lk + kTile - 1) / kTile - 1 - tm.y) * kTile + BN * half;
  if (k0 >= Lk) return;                                // empty half of a ragged last tile
  const int rs = H * D;                                // row stride of Q, dO (elements)
  const int rs_kv = Hk * D;                            // row stride of K, V, dK, dV
  const int64_t base_kv = ((int64_t)seg0k * Hk + hk) * D;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 5, lq = lane & 31;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int pair = wu >> 1, role = wu & 1;             // role 0: S, P, dV; role 1: dP, dS, dK
  const int kw0 = k0 + 32 * pair;                      // first key of this pair (wave-uniform)
  const int kcol = kw0 + lq;                           // this lane's key column (local index)
  const int a_off = pi32(lq) * PB + 16 * g;
  const int t_off = (g + 4 * ((lane & 15) >> 2)) * PB + 2 * (16 * ((lane >> 4) & 1) + 4 * (lane & 3));

  // B operand of the first product: K rows (role 0) or V rows (role 1)
  const bf16* fs = (role ? v : k) + base_kv;
  bf16x8 frag[KSTEPS];
  if (kcol < Lk) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) frag[s] = *(const bf16x8*)(fs + kcol * rs_kv + 16 * s + 8 * g);
  } else {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) frag[s] = bf16x8{};
  }
  // the fragment loads must not be left in flight: the compiler would wait for
  // them inside the loop with counts that also cover the asynchronous copies
  wait_vmcnt<0>();

  // where this lane's slot of each copy lands: tile row and 16-byte chunk
  // (spare slots re-read a valid row; the pad chunk of a row gets a copy of
  // its last chunk)
  auto c_row = [&](int i) { return min((64 * ((4 * i + wu) % CPT) + lane) / CP, BM - 1); };
  auto c_col = [&](int i) { return min((64 * ((4 * i + wu) % CPT) + lane) % CP, D / 8 - 1); };
  uint32_t c_off[NI];                             // byte offset of the slot's chunk in a full tile
#pragma unroll
  for (int i = 0; i < NI; ++i) c_off[i] = (uint32_t)(c_row(i) * rs + c_col(i) * 8) * 2u;
  // records in C-layout order: dword j < BM holds the LSE of tile row
  // crow32(j & 15, j >> 4), dword BM + j its D
  auto rec_row = [&]() {
    const int rec = (2 * BM / 4) * w + lane;
    const int slot = rec - (rec >= BM ? BM : 0);
    return crow32(slot & 15, slot >> 4);
  };
  const int rec_kind = (2 * BM / 4) * w + lane >= BM ? 1 : 0;
  const uint32_t rec_off = (uint32_t)(rec_row() * 8 + rec_kind * 4);
  // query rows whose band holds one of this workgroup's keys [k0, k_last]:
  // from the first row whose band reaches k0 to the last whose band starts by k_last
  int jq_lo = k0 / BM, jq_end = (Lq + BM - 1) / BM;
  if constexpr (BAND) {
    const int k_last = min(k0 + BN, Lk) - 1;
    const int q_first = win_right < 0 ? 0 : max(0, k0 - band.delta - win_right);
    const int q_last = win_left < 0 ? Lq - 1 : min(Lq - 1, k_last - band.delta + win_left);
    jq_lo = q_first / BM;
    jq_end = q_last >= q_first ? q_last / BM + 1 : jq_lo;
  }
  const int n_steps = jq_end - jq_lo;                  // query tiles per query head
  // The walk visits query tiles jq_lo.. of query head hk G, then of hk G + 1,
  // and so on.  Staging runs ahead of the math, so it keeps its own cursor
  // (query head sh, tile st), advanced one tile per call.
  int sh = hk * G, st = jq_lo;
  auto stage = [&](int b) {
    const int qt0 = st * BM;
    const int64_t base = ((int64_t)seg0 * H + sh) * D;
    const bf16* qs = q + base;
    const bf16* gs = dout + base;
    const float2* lds_h = ld + (int64_t)sh * T_q + seg0;
    if (++st >= jq_end) {
      st = jq_lo;
      ++sh;
    }
    const uint32_t sb = lds_addr(ring[b]);
    const uint32_t lb = lds_addr(sLD[b]) + (uint32_t)(wu * (2 * BM / 4) * 4);
    if (qt0 + BM <= Lq) {
      const bf16* q0p = qs + (int64_t)qt0 * rs;
      const bf16* g0p = gs + (int64_t)qt0 * rs;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int c = 4 * i + wu;
        copy_to_lds16(c >= CPT && c < 2 * CPT ? g0p : q0p, c_off[i], sb + (uint32_t)c * 1024u);
      }
      if (lane < 2 * BM / 4) copy_to_lds4(lds_h + qt0, rec_off, lb);
    } else {
      // ragged last tile: rows past the end re-read the segment's last row
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int c = 4 * i + wu;
        const bf16* src = c >= CPT && c < 2 * CPT ? gs : qs;
        const int grow = min(qt0 + c_row(i), Lq - 1);
        copy_to_lds16(src, (uint32_t)(grow * rs + c_col(i) * 8) * 2u, sb + (uint32_t)c * 1024u);
      }
      if (lane < 2 * BM / 4)
        copy_to_lds4(lds_h, (uint32_t)(min(qt0 + rec_row(), Lq - 1) * 8 + rec_kind * 4), lb);
    }
  };

  f32x16 acc2[DBLK];
#pragma unroll
  for (int j = 0; j < DBLK; ++j) acc2[j] = f32x16{};
  float4* xb = xbuf[pair][0];

  const int n_walk = G * n_steps;
#pragma unroll
  for (int i = 0; i < NST - 1; ++i)
    if (i < n_walk) stage(i);
  int tq = jq_lo;                                      // query tile of step t
  for (int t = 0; t < n_walk; ++t) {
    const int b = t % NST;
    const int qt0 = tq * BM;
    if (++tq >= jq_end) tq = jq_lo;
    if (t + NST - 2 < n_walk) wait_vmcnt<(NST - 2) * COPIES>();
    else wait_vmcnt<0>();
    // every wave's copies of step t have landed, every wave is done with the
    // slot of step t - 1 (which now receives step t + NST - 1), and the odd
    // waves are done reading the P of step t - 1
    lds_barrier();
    if (t + NST - 1 < n_walk) stage((t + NST - 1) % NST);
    const char* cQ = ring[b];
    const char* cdO = ring[b] + TILE_BYTES;
    const char* a_src = role ? cdO : cQ;         // rows of the first product
    const char* t_src = role ? cQ : cdO;         // transposed operand of the second
    const float* cLD = sLD[b] + role * BM;       // LSE (role 0) or D (role 1)

    // S (role 0) or dP (role 1); element i is query qt0 + crow32(i, g).
    // Operands are read three k-steps ahead of their MFMAs.
    bf16x8 aa[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) aa[s] = *(const bf16x8*)(a_src + a_off + 32 * s);
    f32x16 acc = mfma32(aa[0], frag[0], f32x16{});
#pragma unroll
    for (int s = 1; s < KSTEPS; ++s) acc = mfma32(aa[s], frag[s], acc);
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (s + 3 < KSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    float4 rv[4];
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) rv[kq] = *(const float4*)(cLD + 16 * g + 4 * kq);

    if (role == 0) {
      // P, zero outside the causal ranges; handed to the partner
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = fast_exp2(acc[i] * scale_log2 - rv[i >> 2][i & 3]);
      // wave-uniform: only tiles that cross the diagonal or an end are masked
      if (!(band.hi(qt0) >= kw0 + 31 && band.lo(qt0 + BM - 1) <= kw0 && qt0 + BM <= Lq && kw0 + 32 <= Lk)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qr = qt0 + crow32(i, g);
          if (kcol > band.hi(qr) || kcol < band.lo(qr) || qr >= Lq || kcol >= Lk) acc[i] = 0.f;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xb[64 * j + lane] = make_float4(acc[4 * j], acc[4 * j + 1], acc[4 * j + 2], acc[4 * j + 3]);
    }
    lds_barrier();                               // P of this step is visible to the odd waves
    if (role == 1) {
      // dS = P (dP - D)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 p4 = xb[64 * j + lane];
        acc[4 * j] = p4.x * (acc[4 * j] - rv[j].x);
        acc[4 * j + 1] = p4.y * (acc[4 * j + 1] - rv[j].y);
        acc[4 * j + 2] = p4.z * (acc[4 * j + 2] - rv[j].z);
        acc[4 * j + 3] = p4.w * (acc[4 * j + 3] - rv[j].w);
      }
    }
    // dV += P^T dO (role 0) or dK += dS^T Q (role 1); k-slot 8g+e of step kk
    // is tile row 16kk + 4(e&3) + 2(e>>2) + g, which the transposed reads fetch
#pragma unroll
    for (int kk = 0; kk < BM / 16; ++kk) {
      bf16x8 xh, xl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = acc[8 * kk + e];
        xh[e] = (bf16)x;
        if constexpr (SPLIT) xl[e] = (bf16)(x - (float)xh[e]);
      }
#pragma unroll
      for (int j = 0; j < DBLK; ++j) {
        const int o0 = t_off + 16 * kk * PB + 64 * j;
        const bf16x8 tf = cat(lds_read_tr((const bf16*)(t_src + o0)), lds_read_tr((const bf16*)(t_src + o0 + 2 * PB)));
        acc2[j] = mfma32(xh, tf, acc2[j]);
        if constexpr (SPLIT) acc2[j] = mfma32(xl, tf, acc2[j]);
      }
    }
  }

  // dV (role 0) or scaled dK (role 1) rows of this pair's keys
  GradT* outp = role ? dk : dv;
  const float oscale = role ? scale : 1.f;
#pragma unroll
  for (int j = 0; j < DBLK; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kw0 + 8 * (i >> 2) + 4 * g + (i & 3);
      if (key < Lk) outp[base_kv + (int64_t)key * rs_kv + 32 * j + lq] = out_cast<GradT>(acc2[j][i] * oscale);
    }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
// Also forms the per-row statistics {LSE log2e, D = dO . O} of its queries and
// writes them for the dK/dV kernel, which runs after it.
template <int D, bool SPLIT, typename GradT, bool DECODE, typename OT, bool BAND>
__global__ void __launch_bounds__(kThreads, 2)
bwd_dq_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
              const bf16* __restrict__ dout, const OT* __restrict__ o, const float* __restrict__ lse,
              float2* __restrict__ ld, const int32_t* __restrict__ cu, const WorkList wl, int H, int Hk, int T,
              float scale, float scale_log2, GradT* __restrict__ dq,
              const int32_t* __restrict__ cu_k, int T_k, int win_left, int win_right) {
  constexpr int BM = kTile, BN = kDqBN;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;

  __shared__ __attribute__((aligned(16))) bf16 sK[2][BN * D];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][BN * D];

  const int tau = blockIdx.x / H;
  const HeadPair hp = head_of_slot(blockIdx.x - tau * H, H, Hk);
  const int h = hp.h;
  int2 tm;
  if (!work_item<BM, DECODE>(wl, cu, T, tau, &tm)) return;
  const int seg0 = cu[tm.x];
  const int L = cu[tm.x + 1] - seg0;           // query rows of the slice
  int seg0k = seg0, Lk = L;                    // its keys (clipped to [0, T_k])
  if constexpr (BAND) {
    seg0k = min(max(cu_k[tm.x], 0), T_k);
    Lk = min(max(cu_k[tm.x + 1] - seg0k, 0), T_k - seg0k);
  }
  const KeyBand<BAND> band{Lk, Lk - L, win_left, win_right};
  const int q0 = tm.y * BM;
  const int rs = H * D;       // row stride of Q, dO, O, dQ (elements)
  const int rs_kv = Hk * D;   // row stride of K, V
  const int64_t base = ((int64_t)seg0 * H + h) * D;
  const int64_t base_kv = ((int64_t)seg0k * Hk + hp.hk) * D;
  const bf16* qs = q + base;
  const bf16* ks = k + base_kv;
  const bf16* vs = v + base_kv;
  const bf16* gs = dout + base;

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, lq = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qrow = q0 + 32 * w + lq;
  const int wq_first = q0 + 32 * w;     // wave-uniform
  const int wq_last = min(wq_first + 31, L - 1);
  const bool wave_active = wq_first < L;
  const int tr_row = (lane & 15) >> 2;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  bf16x8 qf[KSTEPS], gf[KSTEPS];
  float2 rl = make_float2(INFINITY, 0.f);   // {LSE log2e, D} of this lane's query
  float dpart = 0.f;                        // this lane's half of dO . O
  if (qrow < L) {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      qf[s] = *(const bf16x8*)(qs + qrow * rs + 16 * s + 8 * g);
      gf[s] = *(const bf16x8*)(gs + qrow * rs + 16 * s + 8 * g);
    }
    const OT* orow = o + base + (int64_t)qrow * rs;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      float ov[8];
      if constexpr (sizeof(OT) == 4) {
        const float4 a = *(const float4*)(orow + 16 * s + 8 * g), b = *(const float4*)(orow + 16 * s + 8 * g + 4);
        ov[0] = a.x; ov[1] = a.y; ov[2] = a.z; ov[3] = a.w;
        ov[4] = b.x; ov[5] = b.y; ov[6] = b.z; ov[7] = b.w;
      } else {
        const bf16x8 a = *(const bf16x8*)(orow + 16 * s + 8 * g);
#pragma unroll
        for (int e = 0; e < 8; ++e) ov[e] = (float)a[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) dpart += (float)gf[s][e] * ov[e];
    }
    rl.x = lse[(int64_t)h * T + seg0 + qrow] * kLog2e;
    // a row with no key (LSE = -inf) takes +inf, so that every P of the row,
    // masked scores included, is exp2(-inf) = 0 rather than NaN
    if constexpr (BAND) rl.x = rl.x == -INFINITY ? INFINITY : rl.x;
  } else {
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = gf[s] = bf16x8{};
  }
  // lanes l and l^32 hold the two halves of one query row
  rl.y = dpart + swap_halves(dpart);
  if (g == 0 && qrow < L) ld[(int64_t)h * T + seg0 + qrow] = rl;

  f32x16 dqacc[DBLK];
#pragma unroll
  for (int j = 0; j < DBLK; ++j) dqacc[j] = f32x16{};

  const int q_last = min(q0 + BM, L) - 1;
  // key tiles holding a key that some row of the tile may use
  int n_lo = 0, n_end = q_last / BN + 1;
  if constexpr (BAND) {
    const int klo = band.lo(q0), khi = band.hi(q_last);
    n_lo = klo / BN;
    n_end = khi >= klo ? khi / BN + 1 : n_lo;
  }
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
  if (n_end > n_lo) stage(n_lo * BN, 0);
  wait_vmcnt<0>();
  for (int n = n_lo; n < n_end; ++n) {
    const int b = (n - n_lo) & 1;
    lds_barrier();
    if (n + 1 < n_end) stage((n + 1) * BN, b ^ 1);
    const bf16* cK = sK[b];
    const bf16* cV = sV[b];
    const int key0 = n * BN;
    if (wave_active && key0 <= band.hi(wq_last) && key0 + BN - 1 >= band.lo(wq_first)) {
      // S^T = K Q^T and dP^T = V dO^T: each lane owns one query column.  The
      // K and V operands are read kPf k-steps ahead of their MFMAs.
      constexpr int kPf = 1;
      bf16x8 ka[KSTEPS][2], va[KSTEPS][2];
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          ka[s][kb2] = *(const bf16x8*)(cK + swz<D>(32 * kb2 + lq, 16 * s + 8 * g));
          va[s][kb2] = *(const bf16x8*)(cV + swz<D>(32 * kb2 + lq, 16 * s + 8 * g));
        }
      f32x16 st[2], dpt[2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        st[kb2] = mfma32(ka[0][kb2], qf[0], f32x16{});
        dpt[kb2] = mfma32(va[0][kb2], gf[0], f32x16{});
      }
#pragma unroll
      for (int s = 1; s < KSTEPS; ++s)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          st[kb2] = mfma32(ka[s][kb2], qf[s], st[kb2]);
          dpt[kb2] = mfma32(va[s][kb2], gf[s], dpt[kb2]);
        }
      __builtin_amdgcn_sched_group_barrier(0x100, 4 * (kPf + 1), 0);
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        if (s + kPf + 1 < KSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      }
      // wave-uniform: only tiles that cross a band edge (the diagonal when
      // causal) or the end of the keys are masked
      const bool need_mask = !(key0 >= band.lo(wq_last) && key0 + BN - 1 <= band.hi(wq_first) && key0 + BN <= Lk);
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) st[kb2][i] = fast_exp2(st[kb2][i] * scale_log2 - rl.x);
      if (need_mask) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + 32 * kb2 + 8 * (i >> 2) + 4 * g + (i & 3);
            if (key > band.hi(qrow) || key < band.lo(qrow) || key >= Lk) st[kb2][i] = 0.f;
          }
      }
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) st[kb2][i] *= dpt[kb2][i] - rl.y;
      // dQ^T += K^T dS^T.  k-slot 8g+e holds key 16kk + 8(e/4) + 4g + e%4.
#pragma unroll
      for (int kk = 0; kk < BN / 16; ++kk) {
        bf16x8 sh, sl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float ds = st[kk >> 1][8 * (kk & 1) + e];
          sh[e] = (bf16)ds;
          if constexpr (SPLIT) sl[e] = (bf16)(ds - (float)sh[e]);
        }
        const int r0 = 16 * kk + 4 * g + tr_row;
#pragma unroll
        for (int j = 0; j < DBLK; ++j) {
          const int c = 32 * j + tr_col;
          const bf16x8 kt = cat(lds_read_tr(cK + swz<D>(r0, c)), lds_read_tr(cK + swz<D>(r0 + 8, c)));
          dqacc[j] = mfma32(kt, sh, dqacc[j]);
          if constexpr (SPLIT) dqacc[j] = mfma32(kt, sl, dqacc[j]);
        }
      }
    }
    if (n + 1 < n_end) wait_vmcnt<0>();
  }

  if (!wave_active || qrow >= L) return;
  GradT* op = dq + base + (int64_t)qrow * rs;
#pragma unroll
  for (int j = 0; j < DBLK; ++j)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int col = 32 * j + 8 * i4 + 4 * g;
      if constexpr (sizeof(GradT) == 4) {
        *(float4*)(op + col) = make_float4(dqacc[j][4 * i4] * scale, dqacc[j][4 * i4 + 1] * scale,
                                           dqacc[j][4 * i4 + 2] * scale, dqacc[j][4 * i4 + 3] * scale);
      } else {
        bf16x4 r;
#pragma unroll
        for (int t = 0; t < 4; ++t) r[t] = (bf16)(dqacc[j][4 * i4 + t] * scale);
        *(bf16x4*)(op + col) = r;
      }
    }
}

struct BwdLayout {
  size_t tiles_off, tiles_k_off, ld_off, total;
};

// Workspace: list counts in [0, 256) (query list at 0, key list at 128), the
// query tile list, the key tile list (cross form only; otherwise the query
// list serves both kernels), then the {LSE log2e, D} records [H][T].
BwdLayout bwd_layout(int32_t T, int32_t H, int32_t n_seg, int32_t T_k = -1) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  BwdLayout l;
  l.tiles_off = 256;
  size_t end = up(l.tiles_off + plan_capacity(T, n_seg, kTile) * sizeof(int2));
  l.tiles_k_off = l.tiles_off;
  if (T_k >= 0) {
    l.tiles_k_off = end;
    end = up(end + plan_capacity(T_k, n_seg, kTile) * sizeof(int2));
  }
  l.ld_off = end;
  l.total = l.ld_off + (size_t)H * T * sizeof(float2);
  return l;
}

template <int D, bool SPLIT, typename GradT, typename OT, bool BAND>
void launch_bwd_kernels(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, const int32_t* cu, const WorkList& wl, const int32_t* cu_kl,
                        const WorkList& wl_k, int H, int Hk, int T, int T_kl, size_t cap, size_t cap_k,
                        float scale, float2* ld, void* dq, void* dk, void* dv, const BandArgs& bd,
                        hipStream_t s) {
  // dQ first: it also writes the {LSE log2e, D} records the dK/dV kernel reads.
  // One dQ workgroup per (query tile, query head); one dK/dV workgroup per
  // (64-key half tile, key/value head), walking the query tiles of the
  // group's heads.
  const unsigned gq = (unsigned)(cap * H), gk = (unsigned)(2 * cap_k * Hk);
  if (gq > 0) {
    if (wl.tiles == nullptr)
      bwd_dq_kernel<D, SPLIT, GradT, true, OT, BAND><<<dim3(gq), kThreads, 0, s>>>(
          (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout, (const OT*)o, lse, ld, cu, wl,
          H, Hk, T, scale, scale * kLog2e, (GradT*)dq, bd.cu_k, bd.T_k, bd.wl, bd.wr);
    else
      bwd_dq_kernel<D, SPLIT, GradT, false, OT, BAND><<<dim3(gq), kThreads, 0, s>>>(
          (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout, (const OT*)o, lse, ld, cu, wl,
          H, Hk, T, scale, scale * kLog2e, (GradT*)dq, bd.cu_k, bd.T_k, bd.wl, bd.wr);
  }
  if (gk > 0) {
    if (wl_k.tiles == nullptr)
      bwd_kv_pair_kernel<D, SPLIT, GradT, true, BAND><<<dim3(gk), kThreads, 0, s>>>(
          (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout, ld, cu_kl, wl_k, H, Hk, T_kl,
          scale, scale * kLog2e, (GradT*)dk, (GradT*)dv, cu, T, bd.wl, bd.wr);
    else
      bwd_kv_pair_kernel<D, SPLIT, GradT, false, BAND><<<dim3(gk), kThreads, 0, s>>>(
          (const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)dout, ld, cu_kl, wl_k, H, Hk, T_kl,
          scale, scale * kLog2e, (GradT*)dk, (GradT*)dv, cu, T, bd.wl, bd.wr);
  }
}

template <int D, bool SPLIT, typename GradT, typename OT>
hipError_t launch_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, const int32_t* cu, const WorkList& wl, const int32_t* cu_kl,
                      const WorkList& wl_k, int H, int Hk, int T, int T_kl, size_t cap, size_t cap_k,
                      float scale, float2* ld, void* dq, void* dk, void* dv, const BandArgs& bd,
                      hipStream_t s) {
  if (bd.on)
    launch_bwd_kernels<D, SPLIT, GradT, OT, true>(q, k, v, o, dout, lse, cu, wl, cu_kl, wl_k, H, Hk, T, T_kl,
                                                  cap, cap_k, scale, ld, dq, dk, dv, bd, s);
  else
    launch_bwd_kernels<D, SPLIT, GradT, OT, false>(q, k, v, o, dout, lse, cu, wl, cu_kl, wl_k, H, Hk, T, T_kl,
                                                   cap, cap_k, scale, ld, dq, dk, dv, bd, s);
  return hipGetLastError();
}

pvb_status bwd_call(const void* d_q, const void* d_k, const void* d_v, const void* d_o, int32_t o_dtype,
                    const void* d_do, const float* d_lse, const int32_t* d_cu, const int32_t* h_cu,
                    int32_t n_seg, int32_t T, int32_t H, int32_t H_kv, int32_t d, float softmax_scale,
                    void* d_dq, void* d_dk, void* d_dv, int32_t grad_dtype, int32_t precision,
                    void* workspace, size_t workspace_bytes, int32_t* d_status, const BandArgs& bd,
                    void* stream) {
  if (n_seg < 0 || T < 0 || H <= 0 || d_cu == nullptr || d_status == nullptr) return PVB_E_INVALID_ARG;
  if (H_kv <= 0 || H % H_kv != 0) return PVB_E_INVALID_ARG;
  if (n_seg > PVB_MAX_COUNT) return PVB_E_OVERFLOW;
  const int32_t T_k = bd.on ? bd.T_k : T;
  if ((T > 0 && (d_q == nullptr || d_o == nullptr || d_do == nullptr || d_lse == nullptr || d_dq == nullptr)) ||
      (T_k > 0 && (d_k == nullptr || d_v == nullptr || d_dk == nullptr || d_dv == nullptr)))
    return PVB_E_INVALID_ARG;
  if (o_dtype != PVB_BF16 && o_dtype != PVB_F32) return PVB_E_INVALID_ARG;
  if (grad_dtype != PVB_BF16 && grad_dtype != PVB_F32) return PVB_E_INVALID_ARG;
  if (precision != PVB_PREC_BF16 && precision != PVB_PREC_SPLIT) return PVB_E_INVALID_ARG;
  if (!(softmax_scale > 0.f) || !(softmax_scale < INFINITY)) return PVB_E_INVALID_ARG;
  if (d != 64 && d != 128) return PVB_E_UNSUPPORTED;
  if ((int64_t)T * H * d >= ((int64_t)1 << 31) || (int64_t)T_k * H_kv * d >= ((int64_t)1 << 31))
    return PVB_E_UNSUPPORTED;
  const size_t cap = plan_capacity(T, n_seg, kTile);
  const size_t cap_k = bd.on ? plan_capacity(T_k, n_seg, kTile) : cap;
  if (!grid_fits(cap * (uint64_t)H, kThreads) || !grid_fits(2 * cap_k * (uint64_t)H_kv, kThreads))
    return PVB_E_UNSUPPORTED;
  const BwdLayout lay = bwd_layout(T, H, n_seg, bd.on ? T_k : -1);
  if (workspace == nullptr || workspace_bytes < lay.total) return PVB_E_WORKSPACE;
  const pvb_status hs = check_host_cu(h_cu, n_seg, T);
  if (hs != PVB_OK) return hs;

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float2* ld = reinterpret_cast<float2*>(ws + lay.ld_off);
  // Small launches decode their items in the kernels (which then write the
  // status); otherwise the planner writes the list and the status first.  The
  // cross form takes one mode for both lists, so that the query list's writer
  // comes first in stream order and the key list's writes only errors.
  bool dec = decode_in_kernel(T, n_seg, kTile, cap * (size_t)H);
  if (bd.on) dec = dec && decode_in_kernel(T_k, n_seg, kTile, 2 * cap_k * (size_t)H_kv);
  auto make_list = [&](const int32_t* c, int32_t Tn, size_t toff, size_t coff, bool first,
                       WorkList* out) -> bool {
    int32_t* count = reinterpret_cast<int32_t*>(ws + coff);
    int2* tiles = reinterpret_cast<int2*>(ws + toff);
    if (!dec) {
      plan_tiles_kernel<<<1, kPlanThreads, 0, s>>>(c, n_seg, Tn, kTile, tiles, count, d_status, first ? 1 : 0);
      if (hipGetLastError() != hipSuccess) return false;
    }
    *out = WorkList{dec ? nullptr : tiles, count, n_seg, d_status, first};
    return true;
  };
  WorkList wl, wl_k;
  if (!make_list(d_cu, T, lay.tiles_off, 0, true, &wl)) return PVB_E_HIP;
  const int32_t* cu_kl = d_cu;
  if (bd.on) {
    cu_kl = bd.cu_k;
    if (!make_list(bd.cu_k, T_k, lay.tiles_k_off, 128, false, &wl_k)) return PVB_E_HIP;
  } else {
    wl_k = wl;
  }

  const bool split = precision == PVB_PREC_SPLIT, gf32 = grad_dtype == PVB_F32, of32 = o_dtype == PVB_F32;
  hipError_t e = hipSuccess;
#define PVB_BWD(D_, S_, G_, O_)                                                                        \
  e = launch_bwd<D_, S_, G_, O_>(d_q, d_k, d_v, d_o, d_do, d_lse, d_cu, wl, cu_kl, wl_k, H, H_kv, T, T_k, \
                                 cap, cap_k, softmax_scale, ld, d_dq, d_dk, d_dv, bd, s)
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

}  // namespace

size_t attn_bwd_workspace_bytes(int32_t T, int32_t H, int32_t d, int32_t n_seg, int32_t grad_dtype) {
  (void)d;
  (void)grad_dtype;
  return bwd_layout(T, H, n_seg).total;
}

size_t cross_bwd_workspace_bytes(int32_t T_q, int32_t T_k, int32_t H, int32_t n_seg) {
  return bwd_layout(T_q, H, n_seg, T_k).total;
}

}  // namespace pvb

extern "C" pvb_status pvb_varlen_attn_bwd_gqa(const void* d_q, const void* d_k, const void* d_v,
                                              const void* d_o, int32_t o_dtype, const void* d_do,
                                              const float* d_lse, const int32_t* d_cu, const int32_t* h_cu,
                                              int32_t n_seg, int32_t T, int32_t H, int32_t H_kv, int32_t d,
                                              float softmax_scale, void* d_dq, void* d_dk, void* d_dv,
                                              int32_t grad_dtype, int32_t precision, void* workspace,
                                              size_t workspace_bytes, int32_t* d_status, void* stream) {
  return pvb::bwd_call(d_q, d_k, d_v, d_o, o_dtype, d_do, d_lse, d_cu, h_cu, n_seg, T, H, H_kv, d,
                       softmax_scale, d_dq, d_dk, d_dv, grad_dtype, precision, workspace, workspace_bytes,
                       d_status, pvb::BandArgs{}, stream);
}

// ---------------------------------------------------------------------------
// The backward without a caller workspace.  Its scratch (the planner's tile
// list and the {LSE log2e, D} records) lives in one fixed device array of the
// library, `scratch`; each GPU holds its own copy of it, at an address taken
// once per device with hipGetSymbolAddress (the array's name on the host is
// only a stand-in and is never passed to a kernel).  Nothing in it has to
// start at zero: the planner writes its count and list, and the dQ kernel
// writes every record, before anything reads them.
// ---------------------------------------------------------------------------
namespace pvb {
namespace {
static __device__ __align__(256) char scratch[PVB_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (nullptr on failure).
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace
}  // namespace pvb

extern "C" pvb_status pvb_varlen_attn_bwd_noalloc(const void* d_q, const void* d_k, const void* d_v,
                                                  const void* d_o, int32_t o_dtype, const void* d_do,
                                                  const float* d_lse, const int32_t* d_cu, const int32_t* h_cu,
                                                  int32_t n_seg, int32_t T, int32_t H, int32_t H_kv, int32_t d,
                                                  float softmax_scale, void* d_dq, void* d_dk, void* d_dv,
                                                  int32_t grad_dtype, int32_t precision, int32_t* d_status,
                                                  void* stream) {
  using namespace pvb;
  if (n_seg < 0 || T < 0 || H <= 0) return PVB_E_INVALID_ARG;
  if (n_seg > PVB_MAX_COUNT) return PVB_E_OVERFLOW;
  // the sizes the scratch can hold, checked before any HIP call
  if (bwd_layout(T, H, n_seg).total > (size_t)PVB_STATIC_SCRATCH_BYTES) return PVB_E_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return PVB_E_HIP;
  return bwd_call(d_q, d_k, d_v, d_o, o_dtype, d_do, d_lse, d_cu, h_cu, n_seg, T, H, H_kv, d, softmax_scale,
                  d_dq, d_dk, d_dv, grad_dtype, precision, ws, (size_t)PVB_STATIC_SCRATCH_BYTES, d_status,
                  BandArgs{}, stream);
}

extern "C" pvb_status pvb_varlen_attn_bwd(const void* d_q, const void* d_k, const void* d_v,
                                          const void* d_o, int32_t o_dtype, const void* d_do,
                                          const float* d_lse, const int32_t* d_cu, const int32_t* h_cu,
                                          int32_t n_seg, int32_t T, int32_t H, int32_t d,
                                          float softmax_scale, void* d_dq, void* d_dk, void* d_dv,
                                          int32_t grad_dtype, int32_t precision, void* workspace,
                                          size_t workspace_bytes, int32_t* d_status, void* stream) {
  return pvb_varlen_attn_bwd_gqa(d_q, d_k, d_v, d_o, o_dtype, d_do, d_lse, d_cu, h_cu, n_seg, T, H, H, d,
                                 softmax_scale, d_dq, d_dk, d_dv, grad_dtype, precision, workspace,
                                 workspace_bytes, d_status, stream);
}

extern "C" pvb_status pvb_varlen_cross_attn_bwd(const void* d_q, const void* d_k, const void* d_v,
                                                const void* d_o, int32_t o_dtype, const void* d_do,
                                                const float* d_lse, const int32_t* d_cu_q,
                                                const int32_t* h_cu_q, const int32_t* d_cu_k,
                                                const int32_t* h_cu_k, int32_t n_seg, int32_t T_q,
                                                int32_t T_k, int32_t H, int32_t H_kv, int32_t d,
                                                int32_t window_left, int32_t window_right,
                                                float softmax_scale, void* d_dq, void* d_dk, void* d_dv,
                                                int32_t grad_dtype, int32_t precision, void* workspace,
                                                size_t workspace_bytes, int32_t* d_status, void* stream) {
  using namespace pvb;
  const pvb_status hs = check_cross_args(h_cu_q, d_cu_k, h_cu_k, n_seg, T_q, T_k, window_left, window_right);
  if (hs != PVB_OK) return hs;
  const BandArgs bd{true, d_cu_k, T_k, window_left, window_right};
  return bwd_call(d_q, d_k, d_v, d_o, o_dtype, d_do, d_lse, d_cu_q, h_cu_q, n_seg, T_q, H, H_kv, d,
                  softmax_scale, d_dq, d_dk, d_dv, grad_dtype, precision, workspace, workspace_bytes, d_status,
                  bd, stream);
}
