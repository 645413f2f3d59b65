// Gated delta rule over a packed token stream, its recurrent state reset at
// every boundary.
//
// "Packing与 FlashAttention Varlen", section 6: the linear-attention
// (Gated DeltaNet) layers of a hybrid model consume the same cumulative
// boundaries as the attention layers, and the boundary keeps the recurrent
// state of one sample out of the next.  The recurrence is the published gated
// delta rule (Yang, Kautz and Hatamizadeh, 2024); per slice and head, with a
// [d_k, d_v] state S:  S <- exp(g_t) S;  u_t = beta_t (v_t - S^T k_t);
// S <- S + k_t u_t^T;  o_t = scale S^T q_t.
//
// Chunked evaluation (the UT transform of the delta rule, Yang et al.,
// "Parallelizing Linear Transformers with the Delta Rule over Sequence
// Length", 2024, with gates): inside a chunk of 64 positions, with gamma_i the
// gate summed from the chunk start and G_i = exp(gamma_i),
//   (I + A) U = diag(beta) (V - diag(G) K S0),   A_ij = beta_i (G_i/G_j) k_i.k_j  (j < i),
//   O = scale (diag(G) Q S0 + P U),               P_ij = (G_i/G_j) q_i.k_j       (j <= i),
//   S_end = G_63 S0 + (diag(G_63/G) K)^T U.
// The chunk products run on the matrix cores; every fp32 operand (the state,
// P, U, T = (I + A)^-1, A's off-diagonal block) is split into bf16 hi + lo
// parts, so the products keep about 16 significant bits (the state update is
// written K^T (diag(G_63/G) U), so that K^T stays exact); the two 32-row
// triangles of the solve are fp32 on the vector unit.
//
// A chain is one workgroup of 4 waves per (slice, value head); the slices are
// independent.  Value head h reads query/key head h / (H / H_k).  Wave w owns
// value columns [32w, 32w + 32) of the state, which stays in its registers (C
// layout of four 32x32 blocks) across the chunks.  Given a workspace, a slice
// is cut into groups of 16 chunks: a chunk maps its starting state affinely,
// so the groups' maps are composed in parallel, walked group by group, and
// every group's chunks then run from their starting state (the forward, and
// both walks of the backward, the state-gradient walk on the transposed maps).
// The backward recomputes each chunk's starting state and U from the inputs;
// a training forward can leave them (with T, T^T and the group maps) in the
// backward's workspace instead, and the backward then skips that walk.
#include <type_traits>

#include "pvb_device.hpp"

namespace pvb {
namespace {

constexpr int kGdD = 128;            // d_k = d_v
constexpr int kGdC = 64;             // chunk length
constexpr int kGdThreads = 256;
// six split A fragments of a 64x64 matrix, [f][hi, lo][lane] x 16 bytes (12 KB)
constexpr size_t kGdTFragFloats = 6 * 2 * 64 * 4;
constexpr int kKP = kGdD + 8;        // bf16 row pitch of the Q, K, V tiles
constexpr int kFP = kGdC + 4;        // fp32 row pitch of A^T and P

struct GdSmem {
  alignas(16) bf16 q[kGdC][kKP];
  alignas(16) bf16 k[kGdC][kKP];
  alignas(16) bf16 v[kGdC][kKP];
  alignas(16) float at[kGdC][kFP];   // A^T: at[j][i] = A[i][j]
  alignas(16) float p[kGdC][kFP];    // P (row i, column j)
  // A operands shared by the four waves, in fragment order [..][lane]: K^T
  // for the state update (key-dim block r, position step s; exact in bf16)
  // and P split once per chunk (row block rb, position step s; rb = 0 stops
  // at s = 2).  Positions inside a step are in the order of the C layout's
  // rows.
  alignas(16) bf16x8 kt[4][4][64];
  alignas(16) bf16x8 ph[6][64], pl[6][64];
  alignas(16) float gl[kGdC];        // gamma_i log2(e)
  alignas(16) float eg[kGdC];        // exp(gamma_i)
  alignas(16) float dec[kGdC];       // exp(gamma_63 - gamma_i)
  alignas(16) float beta[kGdC];
};

// Checkpoint slot of chunk c of the slice that starts at token seg0 and is
// slice number b: seg0/64 + b + c.  Slices before b hold at most
// sum(ceil(L/64)) <= seg0/64 + b chunks, so slots never collide, and
// T/64 + B + 1 slots cover a call.
__host__ __device__ __forceinline__ size_t gd_ckpt_slot(int seg0, int b, int c) {
  return (size_t)(seg0 / 64) + (size_t)b + (size_t)c;
}

// Groups of 16 chunks (1024 tokens) for the grouped forward: group gi of
// slice b (starting at token seg0) has slot seg0/1024 + b + gi, which never
// collide for the same reason as the chunk slots; T/1024 + B + 1 slots.
constexpr int kGdGrpTok = 1024;
constexpr int kGdGrpChunks = kGdGrpTok / 64;
__host__ __device__ __forceinline__ size_t gd_grp_slot(int seg0, int b, int gi) {
  return (size_t)(seg0 / kGdGrpTok) + (size_t)b + (size_t)gi;
}

// Position of element e of a k-step s fragment whose k order follows the C
// layout's rows (lane half hg): 16s + 8(e/4) + 4hg + e%4.
__device__ __forceinline__ int kpos(int s, int e, int hg) { return 16 * s + 8 * (e >> 2) + 4 * hg + (e & 3); }

// hi = bf16(x), lo = bf16(x - hi): hi + lo carries about 16 significant bits.
__device__ __forceinline__ void split8(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hi[e] = (bf16)x[e];
    lo[e] = (bf16)(x[e] - (float)hi[e]);
  }
}

// Row of C-layout element i (lane half hg) inside a 32x32 block.
__device__ __forceinline__ int crow(int i, int hg) { return 8 * (i >> 2) + 4 * hg + (i & 3); }

// CKPT: the recomputation pass of the backward.  Instead of O and the final
// state it stores, for every chunk, the state at the chunk's start and the
// chunk's U (the solved right-hand side) in checkpoint slots (see
// gd_ckpt_slot); the products that only feed O are skipped.
template <typename OutT, bool CKPT, bool GROUPED = false, bool TRAIN = false>
__device__ __forceinline__ void gd_fwd_body(GdSmem& sm, int& s_bad, int blk, const bf16* __restrict__ q,
                                            const bf16* __restrict__ k, const bf16* __restrict__ v,
                                            const float* __restrict__ g, const float* __restrict__ beta,
                                            const int32_t* __restrict__ cu, int n_seg, int T, int H, int Hk, float scale,
                                            const float* __restrict__ h0, OutT* __restrict__ o, float* __restrict__ ht,
                                            int32_t* __restrict__ status, float* __restrict__ ck_s,
                                            float* __restrict__ ck_u, const float* __restrict__ ck_t,
                                            const float* __restrict__ gstate = nullptr) {
  // CKPT: checkpoints only (the backward's recomputation); TRAIN: the forward
  // with O and the final states that also leaves the backward's checkpoints
  constexpr bool STORE = CKPT || TRAIN;               // chunk-start states and U into ck_s, ck_u
  constexpr bool WITH_O = !CKPT;
  constexpr bool USE_T = STORE || GROUPED;            // the solve as U = T rhs, T from pass 0
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, hg = lane >> 5, c = lane & 31;

  // every workgroup checks the whole cu_seqlens before it writes anything
  if (tid == 0) s_bad = 0;
  __syncthreads();
  for (int b = tid; b < n_seg; b += kGdThreads)
    if (cu[b + 1] < cu[b]) atomicOr(&s_bad, 1);
  if (tid == 0 && (cu[0] != 0 || cu[n_seg] != T)) atomicOr(&s_bad, 1);
  __syncthreads();
  if (blk == 0 && tid == 0) *status = s_bad ? PVB_E_BAD_CU_SEQLENS : PVB_OK;
  if (s_bad) return;

  // the (slice, value head) of this workgroup; GROUPED: a group of up to
  // kGdGrpTok tokens of the slice, from its group slot (see gd_grp_slot)
  int b, h, cbeg = 0;
  size_t gslot = 0;
  if constexpr (GROUPED) {
    if (n_seg == 0) return;
    gslot = (size_t)(blk / H);
    h = blk - (blk / H) * H;
    int lo = 0, hi = n_seg - 1;                       // the largest b with cu[b] / kGdGrpTok + b <= gslot
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((size_t)(cu[mid] / kGdGrpTok + mid) <= gslot) lo = mid;
      else hi = mid - 1;
    }
    b = lo;
    const int gi = (int)(gslot - (size_t)(cu[b] / kGdGrpTok + b));
    const int Lb = cu[b + 1] - cu[b];
    if (gi < 0 || (gi > 0 && gi * kGdGrpTok >= Lb)) return;   // an empty slice keeps group 0
    cbeg = gi * kGdGrpTok;
  } else {
    if ((int)blk >= n_seg * H) return;
    b = blk / H;
    h = blk - (blk / H) * H;
  }
  const int hk = h / (H / Hk);                        // the query/key head of value head h
  const int seg0 = cu[b], L = cu[b + 1] - seg0;
  const int cend = GROUPED ? min(L, cbeg + kGdGrpTok) : L;
  const int n0 = 32 * w + c;                          // this lane's value column
  const size_t st_base = (size_t)(b * H + h) * kGdD * kGdD;

  // the state, rows (key dims) 32r + crow(i, hg), column n0; a group after the
  // slice's first starts from the state the group scan left for it
  const float* s_in = h0 ? h0 + st_base : nullptr;
  if constexpr (GROUPED) {
    if (cbeg > 0) s_in = gstate + (gslot * H + h) * kGdD * kGdD;
  }
  f32x16 S[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i) S[r][i] = s_in ? s_in[(size_t)(32 * r + crow(i, hg)) * kGdD + n0] : 0.f;

  // The inputs of chunk c + 1 are loaded into registers while chunk c is
  // computed (and before its outputs are stored, so that waiting for them
  // never waits for those stores).
  uint4 pq[4], pk[4], pv[4];
  // the chunk's T = (I + A)^-1 as its six split A fragments (12 KB, three
  // 16-byte pieces a thread); the backward's slots also hold T^T's after them
  float4 pt0, pt1, pt2;
  float pg = 0.f, pb = 0.f;
  constexpr size_t kTStride = (STORE ? 2 : 1) * kGdTFragFloats;
  auto fetch = [&](int cc0) {
    const int nvv = min(kGdC, L - cc0);
    if constexpr (USE_T) {
      const float* tp = ck_t + (gd_ckpt_slot(seg0, b, cc0 / kGdC) * H + h) * kTStride + 4 * tid;
      pt0 = *(const float4*)tp;
      pt1 = *(const float4*)(tp + 4 * kGdThreads);
      pt2 = *(const float4*)(tp + 8 * kGdThreads);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int ch = tid + kGdThreads * it;           // 16-byte chunk: row ch/16, columns 8(ch%16)..
      const int row = ch >> 4, col = (ch & 15) * 8;
      pq[it] = pk[it] = pv[it] = zero4();
      if (row < nvv) {
        const size_t off_qk = ((size_t)(seg0 + cc0 + row) * Hk + hk) * kGdD + col;
        const size_t off_v = ((size_t)(seg0 + cc0 + row) * H + h) * kGdD + col;
        pq[it] = *(const uint4*)(q + off_qk);
        pk[it] = *(const uint4*)(k + off_qk);
        pv[it] = *(const uint4*)(v + off_v);
      }
    }
    pg = pb = 0.f;
    if (w == 0 && lane < nvv) {
      const size_t idx = (size_t)(seg0 + cc0 + lane) * H + h;
      pg = g[idx];
      pb = beta[idx];
    }
  };
  if (cbeg < cend) fetch(cbeg);

  for (int c0 = cbeg; c0 < cend; c0 += kGdC) {
    const int nv = min(kGdC, L - c0);
    const size_t slot = gd_ckpt_slot(seg0, b, c0 / kGdC);
    if constexpr (STORE) {
      // the lane's offset is made opaque here, so that the 64 store addresses
      // are formed at the stores rather than kept live across the loop
      int lo = 4 * hg * kGdD + n0;
      asm volatile("" : "+v"(lo));
      float* cs = ck_s + (slot * H + h) * kGdD * kGdD + lo;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) cs[(size_t)(32 * r + 8 * (i >> 2) + (i & 3)) * kGdD] = S[r][i];
    }
    __syncthreads();                                  // the previous chunk's reads are done

    // ---- stage Q, K, V (zero past the slice's end) and the gates
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int ch = tid + kGdThreads * it;
      const int row = ch >> 4, col = (ch & 15) * 8;
      *(uint4*)&sm.q[row][col] = pq[it];
      *(uint4*)&sm.k[row][col] = pk[it];
      *(uint4*)&sm.v[row][col] = pv[it];
    }
    if constexpr (USE_T) {                            // T's fragments, as stored, in A^T's place
      float4* tf = reinterpret_cast<float4*>(&sm.at[0][0]);
      tf[tid] = pt0;
      tf[tid + kGdThreads] = pt1;
      tf[tid + 2 * kGdThreads] = pt2;
    }
    if (w == 0) {
      float x = pg;                                   // inclusive sum over the chunk
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      x *= kLog2e;
      const float last = __shfl(x, 63, 64);
      sm.gl[lane] = x;
      sm.eg[lane] = fast_exp2(x);
      sm.dec[lane] = fast_exp2(last - x);
      sm.beta[lane] = pb;
    }
    if (c0 + kGdC < cend) fetch(c0 + kGdC);
    __syncthreads();

    // ---- A (for the solve, stored transposed) and P: the lower 32x32 blocks
    // (0,0), (1,0), (1,1) of K K^T and Q K^T (block (0,1) is never read), two
    // blocks for waves 0 and 1, one for waves 2 and 3
    auto block = [&](auto isq_tag, int bi, int bj) {
      constexpr bool ISQ = decltype(isq_tag)::value;
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < kGdD / 16; ++s) {
        const bf16x8 a = ISQ ? *(const bf16x8*)&sm.q[32 * bi + c][16 * s + 8 * hg]
                             : *(const bf16x8*)&sm.k[32 * bi + c][16 * s + 8 * hg];
        const bf16x8 bk = *(const bf16x8*)&sm.k[32 * bj + c][16 * s + 8 * hg];
        acc = mfma32(a, bk, acc);
      }
      const int pj = 32 * bj + c;
      const float gj = sm.gl[pj];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int p0 = 32 * bi + 8 * m + 4 * hg;      // rows p0 .. p0 + 3
        const float4 gi = *(const float4*)&sm.gl[p0];
        const float gv[4] = {gi.x, gi.y, gi.z, gi.w};
        float bv[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (!ISQ) {
          const float4 b4 = *(const float4*)&sm.beta[p0];
          bv[0] = b4.x; bv[1] = b4.y; bv[2] = b4.z; bv[3] = b4.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int pi = p0 + e;
          const float dcy = fast_exp2(fminf(gv[e] - gj, 0.f));
          if constexpr (ISQ) sm.p[pi][pj] = pj <= pi ? acc[4 * m + e] * dcy : 0.f;
          else sm.at[pj][pi] = pj < pi ? bv[e] * acc[4 * m + e] * dcy : 0.f;
        }
      }
    };
    using KK = std::integral_constant<bool, false>;
    using QK = std::integral_constant<bool, true>;
    if constexpr (!WITH_O) {
      // P only feeds O, and the solve takes T from the workspace
    } else if constexpr (USE_T) {                     // P only: the solve takes T from the workspace
      if (w == 0) block(QK{}, 0, 0);
      else if (w == 1) block(QK{}, 1, 0);
      else if (w == 2) block(QK{}, 1, 1);
    } else {
      if (w == 0) { block(KK{}, 1, 0); block(QK{}, 0, 0); }
      else if (w == 1) { block(QK{}, 1, 0); block(KK{}, 0, 0); }
      else if (w == 2) block(KK{}, 1, 1);
      else block(QK{}, 1, 1);
    }

    // ---- K^T as A fragments (exact in bf16), once for the four waves:
    // fragment (r, s, lane (fc, fh)) of thread tid is r = it, s = w, element
    // e K[kpos(s, e, fh)][32 r + fc]; the gate G_63 / G goes with U instead
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const bf16* kc = &sm.k[16 * w + 4 * hg][32 * it + c];
      bf16x8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = kc[(8 * (e >> 2) + (e & 3)) * kKP];
      sm.kt[it][w][lane] = x;
    }

    // ---- K S0 and Q S0 for this wave's columns.  The state is the B operand
    // straight from its C layout: k-step s takes elements 8(s%2) + e of block
    // s/2, i.e. key dims kpos(s, e, hg), so the K and Q rows are read in that
    // order (two 8-byte pieces).
    f32x16 ks[2] = {}, oacc[2] = {};
#pragma unroll
    for (int s = 0; s < kGdD / 16; ++s) {
      float sv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = S[s >> 1][8 * (s & 1) + e];
      bf16x8 shi, slo;
      split8(sv, shi, slo);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const bf16* kr = &sm.k[32 * rb + c][16 * s + 4 * hg];
        const bf16* qr = &sm.q[32 * rb + c][16 * s + 4 * hg];
        const bf16x8 ka = cat(*(const bf16x4*)kr, *(const bf16x4*)(kr + 8));
        const bf16x8 qa = cat(*(const bf16x4*)qr, *(const bf16x4*)(qr + 8));
        ks[rb] = mfma32(ka, shi, ks[rb]);
        ks[rb] = mfma32(ka, slo, ks[rb]);
        if constexpr (WITH_O) {
          oacc[rb] = mfma32(qa, shi, oacc[rb]);
          oacc[rb] = mfma32(qa, slo, oacc[rb]);
        }
      }
    }

    // ---- right-hand side, in place (rows pos = 32 rb + crow(i, hg)); the
    // state's part of O takes its gate
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int pos = 32 * rb + crow(i, hg);
        const float egp = sm.eg[pos];
        ks[rb][i] = sm.beta[pos] * ((float)sm.v[pos][n0] - egp * ks[rb][i]);
        oacc[rb][i] *= egp;
      }
    __syncthreads();                                  // A and P are complete

    // ---- P as split A fragments, once for the four waves (read after the
    // next barrier): fragment f = (rb, s, lane), rb = 0 with s < 2 only
    for (int f = tid; f < (WITH_O ? 6 * 64 : 0); f += kGdThreads) {
      const int fi = f >> 6, fl = f & 63, fc = fl & 31, fh = fl >> 5;
      const int rb = fi < 2 ? 0 : 1, s = fi < 2 ? fi : fi - 2;
      const float* src = &sm.p[32 * rb + fc][16 * s + 4 * fh];
      const float4 a4 = *(const float4*)src, b4 = *(const float4*)(src + 8);
      const float x[8] = {a4.x, a4.y, a4.z, a4.w, b4.x, b4.y, b4.z, b4.w};
      split8(x, sm.ph[fi][fl], sm.pl[fi][fl]);
    }

    // ---- (I + A) U = rhs, blocked by 32 rows: U_top = solve(A11, R_top);
    // R_bot -= A21 U_top on the matrix cores; U_bot = solve(A22, R_bot).
    // Each triangle is solved in the C layout: lanes c and c + 32 hold
    // column n0 of the block, each in groups of four rows (rows 8m + 4hg ..
    // + 3).  Step j: the lane holding row j (final by then) hands u_j to its
    // partner, and every row group that may lie below row j subtracts its
    // A[row][j] multiple.  A is zero on and above the diagonal, so the rows of
    // row j's own group that are not below it are left as they are.  The A
    // values of step j + 1 are read while step j computes.
    auto triangle = [&](auto rb_tag) {
      constexpr int RB = decltype(rb_tag)::value;
      float4 acur[4], anext[4];
      auto load_a = [&](int jj, float4 (&buf)[4]) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (8 * m + 7 > jj) buf[m] = *(const float4*)&sm.at[32 * RB + jj][32 * RB + 8 * m + 4 * hg];
      };
      load_a(0, acur);
      // fully unrolled: every register index below must be a constant
#pragma clang loop unroll(full)
      for (int jj = 0; jj < 31; ++jj) {
        if (jj + 1 < 31) load_a(jj + 1, anext);
        const int ij = 4 * (jj >> 3) + (jj & 3);      // element index of row jj
        const bool own = ((jj >> 2) & 1) == hg;
        const float x = ks[RB][ij];
        const float other = swap_halves(x);
        const float uj = own ? x : other;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if (8 * m + 7 <= jj) continue;              // the whole group is at or above row jj
          const float4 a4 = acur[m];
          ks[RB][4 * m] -= a4.x * uj;
          ks[RB][4 * m + 1] -= a4.y * uj;
          ks[RB][4 * m + 2] -= a4.z * uj;
          ks[RB][4 * m + 3] -= a4.w * uj;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) acur[m] = anext[m];
      }
    };
    // U as the B operand straight from its C layout (k-step s: elements
    // 8(s%2) + e of row block s/2, positions kpos(s, e, hg)), split
    bf16x8 uh[4], ul[4];
    auto split_u = [&](int s) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = ks[s >> 1][8 * (s & 1) + e];
      split8(x, uh[s], ul[s]);
    };
    if constexpr (USE_T) {
      // U = T rhs: A element e of lane (c, hg) at k-step s is T[32 rb + c][kpos(s, e, hg)]
      // (two runs of four); row block 0 of T has no column past 31
      f32x16 uu[2] = {};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float xb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) xb[e] = ks[s >> 1][8 * (s & 1) + e];
        bf16x8 bh, bl;
        split8(xb, bh, bl);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          if (rb == 0 && s >= 2) continue;
          // fragment f = (rb, s) as pass 0 split it
          const bf16x8* tf = reinterpret_cast<const bf16x8*>(&sm.at[0][0]);
          const int f = rb == 0 ? s : 2 + s;
          const bf16x8 ah = tf[(2 * f) * 64 + lane], al = tf[(2 * f + 1) * 64 + lane];
          uu[rb] = mfma32(ah, bh, uu[rb]);
          uu[rb] = mfma32(ah, bl, uu[rb]);
          uu[rb] = mfma32(al, bh, uu[rb]);
        }
      }
      ks[0] = uu[0];
      ks[1] = uu[1];
      if constexpr (WITH_O) {
#pragma unroll
        for (int s = 0; s < 4; ++s) split_u(s);
      }
    } else {
      triangle(std::integral_constant<int, 0>{});
      split_u(0);
      split_u(1);
  #pragma unroll
      for (int s = 0; s < 2; ++s) {
        float x[8];                                     // -A21 at row 32 + c, positions kpos(s, e, hg)
  #pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = -sm.at[kpos(s, e, hg)][32 + c];
        bf16x8 ah, al;
        split8(x, ah, al);
        ks[1] = mfma32(ah, uh[s], ks[1]);
        ks[1] = mfma32(ah, ul[s], ks[1]);
        ks[1] = mfma32(al, uh[s], ks[1]);
      }
      triangle(std::integral_constant<int, 1>{});
      split_u(2);
      split_u(3);
    }
    if constexpr (STORE) {
      int lo = 4 * hg * kGdD + n0;                    // opaque, as for the state
      asm volatile("" : "+v"(lo));
      float* cuu = ck_u + (slot * H + h) * kGdC * kGdD + lo;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          cuu[(size_t)(32 * rb + 8 * (i >> 2) + (i & 3)) * kGdD] = ks[rb][i];   // zero past the end
        }
    }
    __syncthreads();                                  // the P and key fragments are complete

    // ---- O = scale (diag(G) Q S0 + P U) (row block 0 has no key past 31)
    // and S = G_63 S0 + (diag(G_63 / G) K)^T U: the matrix-core work of both
    // is issued first, then O is staged in the Q/K tiles (free by now) and
    // written with 16-byte stores.
    if constexpr (WITH_O) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (rb == 0 && s >= 2) continue;
          const int fi = rb == 0 ? s : 2 + s;
          const bf16x8 a_hi = sm.ph[fi][lane], a_lo = sm.pl[fi][lane];
          oacc[rb] = mfma32(a_hi, uh[s], oacc[rb]);
          oacc[rb] = mfma32(a_hi, ul[s], oacc[rb]);
          oacc[rb] = mfma32(a_lo, uh[s], oacc[rb]);
        }
    }
    // the state update as K^T (diag(G_63 / G) U): K^T exact, the scaled U
    // split (k-step s: positions kpos(s, e, hg))
    bf16x8 dh[4], dl[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float4 d0 = *(const float4*)&sm.dec[16 * s + 4 * hg];
      const float4 d1 = *(const float4*)&sm.dec[16 * s + 8 + 4 * hg];
      const float dd[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = dd[e] * ks[s >> 1][8 * (s & 1) + e];
      split8(x, dh[s], dl[s]);
    }
    const float glast = sm.eg[kGdC - 1];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int i = 0; i < 16; ++i) S[r][i] *= glast;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 ka = sm.kt[r][s][lane];
        S[r] = mfma32(ka, dh[s], S[r]);
        S[r] = mfma32(ka, dl[s], S[r]);
      }
    }
    if constexpr (!WITH_O) continue;                  // no O in the recomputation pass
    OutT* stg = reinterpret_cast<OutT*>(&sm.q[0][0]) + w * (kGdC * 32);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) stg[(32 * rb + crow(i, hg)) * 32 + c] = out_cast<OutT>(scale * oacc[rb][i]);
    {
      constexpr int kPer = 16 / sizeof(OutT);         // elements per 16-byte piece
      constexpr int kRowPieces = 32 / kPer;           // pieces per 32-column row
#pragma unroll
      for (int it = 0; it < kGdC * kRowPieces / 64; ++it) {
        const int piece = lane + 64 * it;
        const int row = piece / kRowPieces, cp = piece % kRowPieces;
        if (row < nv)
          *(uint4*)(o + ((size_t)(seg0 + c0 + row) * H + h) * kGdD + 32 * w + cp * kPer) =
              *(const uint4*)(stg + row * 32 + cp * kPer);
      }
    }
  }

  if (WITH_O && ht && cend == L) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) ht[st_base + (size_t)(32 * r + crow(i, hg)) * kGdD + n0] = S[r][i];
  }
}


// The forward without a workspace: one chain per (slice, value head).
template <typename OutT>
__global__ void __launch_bounds__(kGdThreads, 1)
gated_delta_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                   const float* __restrict__ g, const float* __restrict__ beta,
                   const int32_t* __restrict__ cu, int n_seg, int T, int H, int Hk, float scale,
                   const float* __restrict__ h0, OutT* __restrict__ o, float* __restrict__ ht,
                   int32_t* __restrict__ status) {
  __shared__ GdSmem sm;
  __shared__ int s_bad;
  gd_fwd_body<OutT, false>(sm, s_bad, blockIdx.x, q, k, v, g, beta, cu, n_seg, T, H, Hk, scale, h0, o, ht, status,
                           nullptr, nullptr, nullptr);
}

}  // namespace
}  // namespace pvb

namespace pvb {
namespace {

// ===========================================================================
// Backward of the gated delta rule over the packed stream.
//
// The gradients of  sum_t o_t . dO_t + <S_final, dS_final>  with respect to
// q, k, v, g, beta and the initial states, slice by slice (nothing crosses a
// boundary), by reverse-mode differentiation of the chunked form above.  With
// n positions in a chunk, gamma the chunk-local cumulative gate, G = exp(gamma),
// G_L its last value, Gam_ij = G_i / G_j, Ah = strict_lower(Gam o K K^T) (so
// A = diag(beta) Ah), P = lower(Gam o Q K^T), S0 the state at the chunk's
// start, U the chunk's solved update, X = V - diag(G) K S0, Kt = diag(G_L / G) K
// and dS the gradient with respect to the state at the chunk's end:
//   dU  = scale P^T dO + Kt dS               dR = (I + A)^-T dU
//   dV  = diag(beta) dR                      dKS = -diag(G) dV
//   dS (for the previous chunk) = K^T dKS + scale Q^T diag(G) dO + G_L dS
//   dA  = -strict_lower(dR U^T)              dP = scale lower(dO U^T)
//   dKt = U dS^T
//   dbeta_i = sum_c dR_ic X_ic + sum_j dA_ij Ah_ij
//   dG_i = -sum_c dV_ic (K S0)_ic + scale sum_c dO_ic (Q S0)_ic
//   M = diag(beta) (Gam o dA),  N = Gam o dP
//   dK = dKS S0^T + N^T Q + (M + M^T) K + diag(G_L / G) dKt
//   dQ = scale diag(G) dO S0^T + N K
//   dgamma = rowsum(dP o P) - colsum(dP o P) + rowsum(dA o A) - colsum(dA o A)
//            + G o dG - rowsum(dKt o Kt);  dgamma_last += sum(dKt o Kt) + G_L <dS, S0>
//   dg_t = sum_{i >= t} dgamma_i  (inside the chunk).
// Only the first three lines form a chain from chunk to chunk, and that chain
// needs neither S0 nor U.  So the call runs three passes:
//   0. T = (I + A)^-1 of every chunk (gd_tmat_kernel), as split fragments of
//      T and T^T;
//   1. the recomputation walk, which stores S0 and U of every chunk into
//      checkpoint slots, and
//   2. the state-gradient walk back over the chunks, which stores dS at every
//      chunk's end and every chunk's dR and writes dV and dh0; both walks run
//      side by side in one launch (gd_bwd_chains_kernel), or, when a slice is
//      longer than one group, on every group at once from the group maps and
//      scans (gd_bwd_grp_chains_kernel);
//   3. the chunk-parallel pass (gd_bwd_chunk_kernel), one workgroup per
//      (chunk, value head): everything else, from the four checkpoints.
// After the training forward (gd_fwd_train_kernel), which leaves T, S0, U and
// the recomputation's group maps in the workspace, passes 0 and 1 are skipped
// and pass 2 runs alone (gd_bwd_cwalk_kernel).
// The products run on the matrix cores with fp32 operands split into bf16
// hi + lo parts (about 16 significant bits); the transposed solve is fp32 on
// the vector unit.  dQ and dK of a query/key head shared by several value
// heads are summed with fp32 atomic adds into buffers cleared first.

// Checkpoint layouts, per slot and value head, row-major fp32: S0 and dS
// [d_k][d_v], U and dR [64][d_v] (all 64 rows written; rows past the chunk's
// end are zero).
constexpr size_t kGdStateFloats = (size_t)kGdD * kGdD;
constexpr size_t kGdChunkFloats = (size_t)kGdC * kGdD;

// Sum over the 32 lanes of a half-wave of each of the 16 C-layout values of
// a lane (rows crow(i, hg) of one 32-column block): a halving exchange, 16
// shuffles.  Lane c of half hg returns the sum of row crow(idx, hg) with
// idx = 8 b4 + 4 b3 + 2 b2 + b1 (b_k bit k of c); lanes c and c ^ 1 agree.
__device__ __forceinline__ float row_sum16(const float (&v)[16], int c, int& idx) {
  float a[8];
  const bool b4 = c & 16, b3 = c & 8, b2 = c & 4, b1 = c & 2;
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = (b4 ? v[j + 8] : v[j]) + __shfl_xor(b4 ? v[j] : v[j + 8], 16, 64);
  float b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = (b3 ? a[j + 4] : a[j]) + __shfl_xor(b3 ? a[j] : a[j + 4], 8, 64);
  float d2[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) d2[j] = (b2 ? b[j + 2] : b[j]) + __shfl_xor(b2 ? b[j] : b[j + 2], 4, 64);
  float e = (b1 ? d2[1] : d2[0]) + __shfl_xor(b1 ? d2[0] : d2[1], 2, 64);
  e += __shfl_xor(e, 1, 64);
  idx = 8 * b4 + 4 * b3 + 2 * b2 + b1;
  return e;
}

// Two 16-byte reads of 8 consecutive fp32 values.
__device__ __forceinline__ void load8f(const float* p, float (&x)[8]) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Shared by the two backward kernels: the chunk's gates (wave 0) and the
// lower 32x32 blocks of Ah and P (block (0, 1) is not formed), from Q and K
// staged in LDS.  Job j of 6: KK (1,0), QK (0,0), QK (1,0), KK (0,0), KK (1,1),
// QK (1,1), handed out as the forward does.
struct GdTiles {
  alignas(16) bf16 q[kGdC][kKP];
  alignas(16) bf16 k[kGdC][kKP];
  alignas(16) bf16 dO[kGdC][kKP];
  alignas(16) float ah[kGdC][kFP];   // Ah (no beta)
  alignas(16) float p[kGdC][kFP];    // P
  alignas(16) float gl[kGdC];        // gamma_i log2(e)
  alignas(16) float eg[kGdC];        // G_i
  alignas(16) float dec[kGdC];       // G_L / G_i
  alignas(16) float beta[kGdC];
};

__device__ __forceinline__ void gd_gates(GdTiles& t, float gx, float bx, int lane) {
  float x = gx;                                       // inclusive sum (zero past the chunk's end)
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  x *= kLog2e;
  const float last = __shfl(x, 63, 64);               // flat past the end: the last position's sum
  t.gl[lane] = x;
  t.eg[lane] = fast_exp2(x);
  t.dec[lane] = fast_exp2(last - x);
  t.beta[lane] = bx;
}

__device__ __forceinline__ void gd_ah_p_block(GdTiles& t, bool isq, int bi, int bj, int c, int hg) {
  f32x16 acc = {};
#pragma unroll
  for (int s = 0; s < kGdD / 16; ++s) {
    const bf16x8 a = isq ? *(const bf16x8*)&t.q[32 * bi + c][16 * s + 8 * hg]
                         : *(const bf16x8*)&t.k[32 * bi + c][16 * s + 8 * hg];
    const bf16x8 bk = *(const bf16x8*)&t.k[32 * bj + c][16 * s + 8 * hg];
    acc = mfma32(a, bk, acc);
  }
  const int pj = 32 * bj + c;
  const float gj = t.gl[pj];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int pi = 32 * bi + crow(i, hg);
    const float dcy = fast_exp2(fminf(t.gl[pi] - gj, 0.f));
    if (isq) t.p[pi][pj] = pj <= pi ? acc[i] * dcy : 0.f;
    else t.ah[pi][pj] = pj < pi ? acc[i] * dcy : 0.f;
  }
}



// Stages rows [t0, t0 + n) of Q and K (query/key head hk) and dO (value head
// h) in the tiles, zero past n: 16-byte pieces, 1024 / NT per thread and tile.
template <int NT>
struct GdStage {
  static constexpr int IT = 1024 / NT;
  uint4 q[IT], k[IT], o[IT];
  float g, b;
  __device__ __forceinline__ void fetch(const bf16* q_, const bf16* k_, const bf16* do_, const float* g_,
                                        const float* beta_, int t0, int n, int H, int Hk, int h, int hk,
                                        int tid) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int ch = tid + NT * it;
      const int row = ch >> 4, col = (ch & 15) * 8;
      q[it] = k[it] = o[it] = zero4();
      if (row < n) {
        const size_t oqk = ((size_t)(t0 + row) * Hk + hk) * kGdD + col;
        const size_t oo = ((size_t)(t0 + row) * H + h) * kGdD + col;
        q[it] = *(const uint4*)(q_ + oqk);
        k[it] = *(const uint4*)(k_ + oqk);
        o[it] = *(const uint4*)(do_ + oo);
      }
    }
    g = b = 0.f;
    if (tid < 64 && tid < n) {
      const size_t idx = (size_t)(t0 + tid) * H + h;
      g = g_[idx];
      b = beta_[idx];
    }
  }
  __device__ __forceinline__ void put(GdTiles& t, int tid) const {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int ch = tid + NT * it;
      const int row = ch >> 4, col = (ch & 15) * 8;
      *(uint4*)&t.q[row][col] = q[it];
      *(uint4*)&t.k[row][col] = k[it];
      *(uint4*)&t.dO[row][col] = o[it];
    }
  }
};

// Every workgroup checks the whole cu_seqlens before it writes anything.
__device__ __forceinline__ bool gd_cu_bad(const int32_t* __restrict__ cu, int n_seg, int T, int* s_bad) {
  if (threadIdx.x == 0) *s_bad = 0;
  __syncthreads();
  for (int b = threadIdx.x; b < n_seg; b += blockDim.x)
    if (cu[b + 1] < cu[b]) atomicOr(s_bad, 1);
  if (threadIdx.x == 0 && (cu[0] != 0 || cu[n_seg] != T)) atomicOr(s_bad, 1);
  __syncthreads();
  return *s_bad != 0;
}

// Every workgroup checks the whole cu_seqlens before it writes anything; the
// same pass finds the slice of checkpoint slot `slot`: the largest b whose
// first slot cu[b] / 64 + b is at most slot (that first slot rises strictly
// with b).
__device__ __forceinline__ bool gd_cu_bad_find(const int32_t* __restrict__ cu, int n_seg, int T, int slot,
                                               int* s_bad, int* s_b) {
  if (threadIdx.x == 0) {
    *s_bad = 0;
    *s_b = 0;
  }
  __syncthreads();
  for (int b = threadIdx.x; b < n_seg; b += blockDim.x) {
    const int c0 = cu[b];
    if (cu[b + 1] < c0) atomicOr(s_bad, 1);
    if (c0 >= 0 && c0 / kGdC + b <= slot) atomicMax(s_b, b);
  }
  if (threadIdx.x == 0 && (cu[0] != 0 || cu[n_seg] != T)) atomicOr(s_bad, 1);
  __syncthreads();
  return *s_bad != 0;
}

struct GdChainSmem {
  GdTiles t;
  // A fragments of K^T and Q^T for the state-gradient update, [d_k block][k-step][lane]:
  // element e of lane (c, hg) is K[kpos(s, e, hg)][32 r + c]
  alignas(16) bf16x8 kt[4][4][64], qt[4][4][64];
};

// Pass 2: the state-gradient chain, chunks from the last to the first.  Wave
// w owns value columns [32w, 32w + 32): dS stays in its registers (C layout
// of four 32x32 blocks, rows = key dims), as the state does in the forward.
// MODE 0: one workgroup per (slice, value head) walks the whole slice from the
// final-state gradient.  MODE 1 and 2 work on a group of 16 chunks (block =
// group slot x H + head, as the grouped forward): dS of a group's start is
// A_g^T dS of its end plus an offset F_g (A_g the forward's map of the group),
// so MODE 1 walks the group from dS = 0 without storing anything and leaves
// F_g in gF (groups after a slice's first); MODE 2 walks it from dS of its end
// (gD, or the final-state gradient for the slice's last group) with every
// store, and writes dh0 for the slice's first group.
template <typename GradT, int MODE = 0>
__device__ __forceinline__ void gd_bwd_chain_body(GdChainSmem& sm, int& s_bad, int blk, const bf16* __restrict__ q,
                                                  const bf16* __restrict__ k, const float* __restrict__ g,
                                                  const float* __restrict__ beta, const int32_t* __restrict__ cu,
                                                  int n_seg, int T, int H, int Hk, float scale,
                                                  const bf16* __restrict__ dout, const float* __restrict__ dht,
                                                  const float* __restrict__ ck_t, float* __restrict__ ck_ds,
                                                  float* __restrict__ ck_dr, GradT* __restrict__ dv,
                                                  float* __restrict__ dh0, float* __restrict__ gF = nullptr,
                                                  const float* __restrict__ gD = nullptr) {
  GdTiles& t = sm.t;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, hg = lane >> 5, c = lane & 31;
  if (gd_cu_bad(cu, n_seg, T, &s_bad)) return;
  int b, h, gi = 0, n_grp = 1;
  size_t gslot = 0;
  if constexpr (MODE == 0) {
    if ((int)blk >= n_seg * H) return;
    b = blk / H;
    h = blk - (blk / H) * H;
  } else {
    if (n_seg == 0) return;
    gslot = (size_t)(blk / H);
    h = blk - (blk / H) * H;
    int lo = 0, hi = n_seg - 1;                       // the largest b with cu[b] / kGdGrpTok + b <= gslot
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((size_t)(cu[mid] / kGdGrpTok + mid) <= gslot) lo = mid;
      else hi = mid - 1;
    }
    b = lo;
    gi = (int)(gslot - (size_t)(cu[b] / kGdGrpTok + b));
    const int Lb = cu[b + 1] - cu[b];
    n_grp = std::max(1, (Lb + kGdGrpTok - 1) / kGdGrpTok);   // an empty slice keeps group 0
    if (gi < 0 || gi >= n_grp || (MODE == 1 && gi == 0)) return;
  }
  const int hk = h / (H / Hk);
  const int seg0 = cu[b], L = cu[b + 1] - seg0;
  const int n0 = 32 * w + c;
  const size_t st_base = (size_t)(b * H + h) * kGdStateFloats;
  const size_t gs_base = (gslot * H + h) * kGdStateFloats;
  // staging rows of this wave for row-piece stores: [64][kSP] fp32 in the Q/K/dO
  // tiles, which hold nothing between a chunk's last product and the next
  // chunk's staging; only this wave touches them
  constexpr int kSP = 36;
  float* stg = reinterpret_cast<float*>(&t.q[0][0]) + w * (kGdC * kSP);
  auto wave_lds_fence = [] { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); };

  const float* ds_in = MODE == 1 ? nullptr : dht ? dht + st_base : nullptr;
  if (MODE == 2 && gi + 1 < n_grp) ds_in = gD + gs_base;
  f32x16 dS[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i) dS[r][i] = ds_in ? ds_in[(size_t)(32 * r + crow(i, hg)) * kGdD + n0] : 0.f;

  // the chunks [c_lo, c_hi) of this walk
  const int n_chunks = (L + kGdC - 1) / kGdC;
  const int c_lo = MODE == 0 ? 0 : gi * kGdGrpChunks;
  const int c_hi = MODE == 0 ? n_chunks : std::min(n_chunks, c_lo + kGdGrpChunks);
  GdStage<kGdThreads> pf;
  float4 ptm0, ptm1, ptm2;                            // the chunk's T^T fragments (12 KB)
  const float* tbase = ck_t + (gd_ckpt_slot(seg0, b, 0) * H + h) * (2 * kGdTFragFloats) + kGdTFragFloats + 4 * tid;
  const size_t tstep = (size_t)H * 2 * kGdTFragFloats;   // one checkpoint slot
  if (c_hi > c_lo) {
    const int c0 = (c_hi - 1) * kGdC;
    pf.fetch(q, k, dout, g, beta, seg0 + c0, L - c0, H, Hk, h, hk, tid);
    const float* tp = tbase + (size_t)(c_hi - 1) * tstep;
    ptm0 = *(const float4*)tp;
    ptm1 = *(const float4*)(tp + 4 * kGdThreads);
    ptm2 = *(const float4*)(tp + 8 * kGdThreads);
  }
  for (int ci = c_hi - 1; ci >= c_lo; --ci) {
    const int t0 = seg0 + ci * kGdC;
    const int n = min(kGdC, L - ci * kGdC);
    const size_t slot = gd_ckpt_slot(seg0, b, ci);
    if constexpr (MODE != 1) {
      // dS at this chunk's end into its checkpoint: 64 rows at a time through
      // this wave's staging rows, written as 32-byte row pieces
      float* dst = ck_ds + (slot * H + h) * kGdStateFloats + 32 * w;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
          for (int i = 0; i < 16; ++i) stg[(32 * r2 + crow(i, hg)) * kSP + c] = dS[2 * half + r2][i];
        wave_lds_fence();
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int pc = lane + 64 * it, row = pc >> 2, q8 = pc & 3;
          const float* src = stg + row * kSP + 8 * q8;
          float* o = dst + (size_t)(64 * half + row) * kGdD + 8 * q8;
          *(float4*)o = *(const float4*)src;
          *(float4*)(o + 4) = *(const float4*)(src + 4);
        }
        wave_lds_fence();
      }
    }
    __syncthreads();                                  // the previous chunk's LDS reads are done
    pf.put(t, tid);
    {                                                 // T^T's fragments, as stored, into Ah's place
      float4* tf = reinterpret_cast<float4*>(&t.ah[0][0]);
      tf[tid] = ptm0;
      tf[tid + kGdThreads] = ptm1;
      tf[tid + 2 * kGdThreads] = ptm2;
    }
    if (w == 0) gd_gates(t, pf.g, pf.b, lane);
    if (ci > c_lo) {
      const int c0 = (ci - 1) * kGdC;
      pf.fetch(q, k, dout, g, beta, seg0 + c0, kGdC, H, Hk, h, hk, tid);
      const float* tp = tbase + (size_t)(ci - 1) * tstep;
      ptm0 = *(const float4*)tp;
      ptm1 = *(const float4*)(tp + 4 * kGdThreads);
      ptm2 = *(const float4*)(tp + 8 * kGdThreads);
    }
    __syncthreads();

    // the lower blocks of P: QK (0,0), (1,0), (1,1)
    if (w < 3) gd_ah_p_block(t, true, w == 0 ? 0 : 1, w == 2 ? 1 : 0, c, hg);
    // K^T and Q^T fragments, once for the four waves
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int f = tid + kGdThreads * it;
      const int r = f >> 8, s = (f >> 6) & 3, fl = f & 63, fc = fl & 31, fh = fl >> 5;
      bf16x8 xk, xq;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xk[e] = t.k[kpos(s, e, fh)][32 * r + fc];
        xq[e] = t.q[kpos(s, e, fh)][32 * r + fc];
      }
      sm.kt[r][s][fl] = xk;
      sm.qt[r][s][fl] = xq;
    }
    // dO of this wave's columns as B fragments (k-step s: positions kpos(s, e, hg))
    bf16x8 dob[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) dob[s][e] = t.dO[kpos(s, e, hg)][n0];
    // K dS for this wave's columns (the state gradient as the B operand straight
    // from its C layout, as the forward's K S0)
    f32x16 du[2] = {}, kds[2] = {};
#pragma unroll
    for (int s = 0; s < kGdD / 16; ++s) {
      float sv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = dS[s >> 1][8 * (s & 1) + e];
      bf16x8 shi, slo;
      split8(sv, shi, slo);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const bf16* kr = &t.k[32 * rb + c][16 * s + 4 * hg];
        const bf16x8 ka = cat(*(const bf16x4*)kr, *(const bf16x4*)(kr + 8));
        kds[rb] = mfma32(ka, shi, kds[rb]);
        kds[rb] = mfma32(ka, slo, kds[rb]);
      }
    }
    __syncthreads();                                  // T, P and the fragments are complete

    // P^T dO: A element e of lane (c, hg) at k-step s is P[kpos(s, e, hg)][32 rb + c];
    // P^T of row block 1 has no position below 32
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (rb == 1 && s < 2) continue;
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = t.p[kpos(s, e, hg)][32 * rb + c];
        bf16x8 ph, pl;
        split8(x, ph, pl);
        du[rb] = mfma32(ph, dob[s], du[rb]);
        du[rb] = mfma32(pl, dob[s], du[rb]);
      }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) du[rb][i] = scale * du[rb][i] + t.dec[32 * rb + crow(i, hg)] * kds[rb][i];

    // ---- dR = (I + A)^-T dU = T^T dU: A element e of lane (c, hg) at k-step s
    // is T[kpos(s, e, hg)][32 rb + c], fragment f = rb == 0 ? s : 2 + s as pass
    // 0 split it; row block 1 of T^T has no column below 32
    {
      f32x16 dr[2] = {};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float xb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) xb[e] = du[s >> 1][8 * (s & 1) + e];
        bf16x8 bh, bl;
        split8(xb, bh, bl);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          if (rb == 1 && s < 2) continue;
          const bf16x8* tf = reinterpret_cast<const bf16x8*>(&t.ah[0][0]);
          const int f = rb == 0 ? s : 2 + s;
          const bf16x8 ah = tf[(2 * f) * 64 + lane], al = tf[(2 * f + 1) * 64 + lane];
          dr[rb] = mfma32(ah, bh, dr[rb]);
          dr[rb] = mfma32(ah, bl, dr[rb]);
          dr[rb] = mfma32(al, bh, dr[rb]);
        }
      }
      du[0] = dr[0];
      du[1] = dr[1];
    }

    // ---- the new dS = G_L dS + K^T dKS + scale Q^T diag(G) dO with
    // dKS = -diag(G beta) dR
    const float gL = t.eg[kGdC - 1];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) dS[r][i] *= gL;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x1[8], x2[8];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {                // positions kpos(s, 4 hf .. 4 hf + 3, hg): four in a row
        const int p0 = kpos(s, 4 * hf, hg);
        const float4 g4 = *(const float4*)&t.eg[p0], b4 = *(const float4*)&t.beta[p0];
        const float gv[4] = {g4.x, g4.y, g4.z, g4.w}, bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int e = 4 * hf + e4;
          x1[e] = -gv[e4] * bv[e4] * du[s >> 1][8 * (s & 1) + e];
          x2[e] = scale * gv[e4] * (float)dob[s][e];
        }
      }
      bf16x8 b1h, b1l, b2h, b2l;
      split8(x1, b1h, b1l);
      split8(x2, b2h, b2l);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bf16x8 ak = sm.kt[r][s][lane], aq = sm.qt[r][s][lane];
        dS[r] = mfma32(ak, b1h, dS[r]);
        dS[r] = mfma32(ak, b1l, dS[r]);
        dS[r] = mfma32(aq, b2h, dS[r]);
        dS[r] = mfma32(aq, b2l, dS[r]);
      }
    }
    // off the chain: dR into its checkpoint and dV = diag(beta) dR, through
    // this wave's staging rows, written as 32-byte row pieces
    if constexpr (MODE != 1) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) stg[(32 * rb + crow(i, hg)) * kSP + c] = du[rb][i];
      wave_lds_fence();
      float* drp = ck_dr + (slot * H + h) * kGdChunkFloats + 32 * w;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int pc = lane + 64 * it, row = pc >> 2, q8 = pc & 3;
        const float* src = stg + row * kSP + 8 * q8;
        const float4 x0 = *(const float4*)src, x1 = *(const float4*)(src + 4);
        float* o = drp + (size_t)row * kGdD + 8 * q8;
        *(float4*)o = x0;
        *(float4*)(o + 4) = x1;
        if (row < n) {
          const float bt = t.beta[row];
          const float x[8] = {bt * x0.x, bt * x0.y, bt * x0.z, bt * x0.w, bt * x1.x, bt * x1.y, bt * x1.z, bt * x1.w};
          GradT* od = dv + ((size_t)(t0 + row) * H + h) * kGdD + 32 * w + 8 * q8;
          if constexpr (std::is_same_v<GradT, float>) {
            *(float4*)od = make_float4(x[0], x[1], x[2], x[3]);
            *(float4*)(od + 4) = make_float4(x[4], x[5], x[6], x[7]);
          } else {
            bf16x8 pk;
#pragma unroll
            for (int e = 0; e < 8; ++e) pk[e] = (bf16)x[e];
            *(bf16x8*)od = pk;
          }
        }
      }
      wave_lds_fence();
    }
  }
  float* ds_out = MODE == 1 ? gF + gs_base : (dh0 && gi == 0) ? dh0 + st_base : nullptr;
  if (ds_out) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) ds_out[(size_t)(32 * r + crow(i, hg)) * kGdD + n0] = dS[r][i];
  }
}

constexpr int kGdChunkThreads = 512;
constexpr int kUP = kGdD + 4;        // fp32 row pitch of the staged U and dR

// Pass 0: T = (I + A)^-1 of every chunk (A = diag(beta) strict_lower(Gam o K K^T),
// which depends on no state), so that both chains apply the solve as a
// product.  Work items are (checkpoint slot, value head) pairs, slot-major;
// each workgroup (one wave) takes a run of `per` consecutive items, `per`
// chosen so that the grid is one round of resident workgroups, and loads the
// next item's K and gates while it computes the current one.  Per
// item: the three lower blocks of K K^T on the matrix cores, the K fragments
// loaded straight into the operand layout (lane (c, hg) holds rows c and
// 32 + c, dims 16 s + 8 hg .. + 7 at k-step s); the diagonal blocks of T by
// forward substitution, T_ij = [i = j] - sum_{l < i} A_il T_lj in fp32, lane j
// taking column j of T11 and lane 32 + j column j of T22; then T21 = -T22 A21
// T11 on the matrix cores.  Rows and columns past the chunk's end give the
// identity.  T is stored as the six split A fragments that U = T rhs takes
// (fragment f = (rb, s): rb = 0, s = f for f < 2, else rb = 1, s = f - 2;
// [f][hi, lo][lane], 12 KB); TT (the backward) adds after them the six of
// T^T that dR = T^T dU takes (rb = 0, s = f for f < 4, else rb = 1, s = f - 2).
constexpr int kGdTmatPerCu = 8;       // resident workgroups per CU (LDS: 8 x 17.9 KB)
struct GdTmatSmem {
  alignas(16) float a[kGdC][kFP];    // A, then T over it
  alignas(16) float gl[kGdC];
  alignas(16) float beta[kGdC];
};

template <bool TT>
__global__ void __launch_bounds__(64, 2)
gd_tmat_kernel(const bf16* __restrict__ k, const float* __restrict__ g, const float* __restrict__ beta,
               const int32_t* __restrict__ cu, int n_seg, int T, int H, int Hk, float* __restrict__ ck_t, int per) {
  __shared__ GdTmatSmem sm;
  __shared__ int s_bad;
  const int lane = threadIdx.x, hg = lane >> 5, c = lane & 31;
  if (gd_cu_bad(cu, n_seg, T, &s_bad) || n_seg == 0) return;
  const int64_t n_items = ((int64_t)T / kGdC + n_seg + 1) * H;
  // run r of workgroup x: consecutive runs on one XCD (x mod 8 with the grid a
  // multiple of 8), so the heads of a slot read its g and beta lines through
  // one L2
  const int64_t run = (int64_t)(blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
  const int64_t it_end = std::min<int64_t>(n_items, (run + 1) * per);
  // the slice of the current slot: the largest b whose first slot cu[b]/64 + b
  // is at most the slot (found once by bisection, then advanced)
  int64_t it = run * per;
  if (it >= it_end) return;
  int b;
  {
    const int64_t slot = it / H;
    int lo = 0, hi = n_seg - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)(cu[mid] / kGdC + mid) <= slot) lo = mid;
      else hi = mid - 1;
    }
    b = lo;
  }
  // the next item at or after `it` whose slot holds a chunk; sets the item's
  // chunk (t0, n) and heads, or it = it_end
  int t0 = 0, n = 0, h = 0, hk = 0;
  int64_t slot = 0;
#define GD_TMAT_NEXT()                                                                                  \
  for (; it < it_end; ++it) {                                                                           \
    slot = it / H;                                                                                      \
    while (b + 1 < n_seg && (int64_t)(cu[b + 1] / kGdC + b + 1) <= slot) ++b;                             \
    const int seg0_ = cu[b], L_ = cu[b + 1] - seg0_;                                                    \
    const int64_t ci_ = slot - (seg0_ / kGdC + b);                                                      \
    if (ci_ >= 0 && ci_ * kGdC < L_) {                                                                  \
      h = (int)(it - slot * H);                                                                         \
      hk = h / (H / Hk);                                                                                \
      t0 = seg0_ + (int)ci_ * kGdC;                                                                     \
      n = min(kGdC, L_ - (int)ci_ * kGdC);                                                              \
      break;                                                                                            \
    }                                                                                                   \
    it = (slot + 1) * H - 1;                          /* an empty slot: skip its heads */               \
  }
  // K fragments and gates of the item, into registers (scalars, not arrays,
  // which the compiler would move to LDS)
  uint4 f00, f01, f02, f03, f04, f05, f06, f07, f10, f11, f12, f13, f14, f15, f16, f17;
  float pg, pb;
#define GD_TMAT_FETCH()                                                                                 \
  {                                                                                                    \
    const bf16* r0_ = k + ((size_t)(t0 + c) * Hk + hk) * kGdD + 8 * hg;                                 \
    const bf16* r1_ = r0_ + (size_t)32 * Hk * kGdD;                                                     \
    const bool v0_ = c < n, v1_ = 32 + c < n;                                                           \
    f00 = v0_ ? *(const uint4*)(r0_ + 0) : zero4();                                                     \
    f01 = v0_ ? *(const uint4*)(r0_ + 16) : zero4();                                                    \
    f02 = v0_ ? *(const uint4*)(r0_ + 32) : zero4();                                                    \
    f03 = v0_ ? *(const uint4*)(r0_ + 48) : zero4();                                                    \
    f04 = v0_ ? *(const uint4*)(r0_ + 64) : zero4();                                                    \
    f05 = v0_ ? *(const uint4*)(r0_ + 80) : zero4();                                                    \
    f06 = v0_ ? *(const uint4*)(r0_ + 96) : zero4();                                                    \
    f07 = v0_ ? *(const uint4*)(r0_ + 112) : zero4();                                                   \
    f10 = v1_ ? *(const uint4*)(r1_ + 0) : zero4();                                                     \
    f11 = v1_ ? *(const uint4*)(r1_ + 16) : zero4();                                                    \
    f12 = v1_ ? *(const uint4*)(r1_ + 32) : zero4();                                                    \
    f13 = v1_ ? *(const uint4*)(r1_ + 48) : zero4();                                                    \
    f14 = v1_ ? *(const uint4*)(r1_ + 64) : zero4();                                                    \
    f15 = v1_ ? *(const uint4*)(r1_ + 80) : zero4();                                                    \
    f16 = v1_ ? *(const uint4*)(r1_ + 96) : zero4();                                                    \
    f17 = v1_ ? *(const uint4*)(r1_ + 112) : zero4();                                                   \
    pg = lane < n ? g[(size_t)(t0 + lane) * H + h] : 0.f;                                               \
    pb = lane < n ? beta[(size_t)(t0 + lane) * H + h] : 0.f;                                            \
  }
  GD_TMAT_NEXT();
  if (it >= it_end) return;
  GD_TMAT_FETCH();
  while (true) {
    const int cur_n = n;
    const int64_t cur_slot = slot;
    const int cur_h = h;
    {
      float x = pg;                                   // inclusive sum (zero past the chunk's end)
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      sm.gl[lane] = x * kLog2e;
      sm.beta[lane] = pb;
    }
    // blocks (0,0), (1,0), (1,1) of K K^T: A operand row block bi, B operand
    // row block bj, both from the fragments as loaded
    f32x16 kk0 = {}, kk1 = {}, kk2 = {};
    {
      const uint4 r0[8] = {f00, f01, f02, f03, f04, f05, f06, f07};
      const uint4 r1[8] = {f10, f11, f12, f13, f14, f15, f16, f17};
#pragma unroll
      for (int s2 = 0; s2 < 8; ++s2) {
        const bf16x8 x0 = __builtin_bit_cast(bf16x8, r0[s2]);
        const bf16x8 x1 = __builtin_bit_cast(bf16x8, r1[s2]);
        kk0 = mfma32(x0, x0, kk0);
        kk1 = mfma32(x1, x0, kk1);
        kk2 = mfma32(x1, x1, kk2);
      }
    }
    // the next item's loads go out while this one is computed
    ++it;
    GD_TMAT_NEXT();
    const bool more = it < it_end;
    if (more) GD_TMAT_FETCH();
    __syncthreads();                                  // the gates are in LDS; the last item's T is stored
    // A = diag(beta) strict_lower(Gam o K K^T) for the three blocks; rows
    // 32 bi + 8 m + 4 hg + e of the C layout
    {
      const f32x16 kk[3] = {kk0, kk1, kk2};
#pragma unroll
      for (int blk = 0; blk < 3; ++blk) {
        const int bi = blk == 0 ? 0 : 1, bj = blk == 2 ? 1 : 0;
        const int pj = 32 * bj + c;
        const float gj = sm.gl[pj];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int p0 = 32 * bi + 8 * m + 4 * hg;
          const float4 gi4 = *(const float4*)&sm.gl[p0];
          const float4 bt4 = *(const float4*)&sm.beta[p0];
          const float gv[4] = {gi4.x, gi4.y, gi4.z, gi4.w};
          const float bv[4] = {bt4.x, bt4.y, bt4.z, bt4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int pi = p0 + e;
            sm.a[pi][pj] = pj < pi ? bv[e] * kk[blk][4 * m + e] * fast_exp2(gv[e] - gj) : 0.f;
          }
        }
      }
    }
    __syncthreads();
    // the two diagonal 32x32 blocks by substitution, side by side: lanes 0-31
    // take the columns of T11, lanes 32-63 those of T22
    {
      const int bb = lane >> 5, jl = lane & 31;
      float tc[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;   // four partial sums shorten the dependent chain
#pragma unroll
        for (int l4 = 0; l4 < i; l4 += 4) {
          const float4 a4 = *(const float4*)&sm.a[32 * bb + i][32 * bb + l4];
          a0 += a4.x * tc[l4];
          if (l4 + 1 < i) a1 += a4.y * tc[l4 + 1];
          if (l4 + 2 < i) a2 += a4.z * tc[l4 + 2];
          if (l4 + 3 < i) a3 += a4.w * tc[l4 + 3];
        }
        tc[i] = (i == jl ? 1.f : 0.f) - ((a0 + a1) + (a2 + a3));
      }
      // T11 and T22 over A11 and A22 (every lane of the one wave has read
      // them); A21 stays until T21 is formed
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        sm.a[32 * bb + i][32 * bb + jl] = tc[i];
        sm.a[i][32 + jl] = 0.f;                         // T12 (written twice, zero)
      }
    }
    __syncthreads();
    // T21 = -T22 (A21 T11): X = A21 T11, A element e of lane (c, hg) at
    // k-step s is A21[c][kpos(s, e, hg)], B element T11[kpos(s, e, hg)][c];
    // then -T22 X with X as the B operand straight from its C layout
    {
      f32x16 x = {};
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const float* ar = &sm.a[32 + c][kpos(s2, 0, hg)];
        const float4 p0 = *(const float4*)ar, p1 = *(const float4*)(ar + 8);
        const float xa[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        float xb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) xb[e] = sm.a[kpos(s2, e, hg)][c];
        bf16x8 ah, al, bh, bl;
        split8(xa, ah, al);
        split8(xb, bh, bl);
        x = mfma32(ah, bh, x);
        x = mfma32(ah, bl, x);
        x = mfma32(al, bh, x);
      }
      f32x16 y = {};
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const float* tr = &sm.a[32 + c][32 + kpos(s2, 0, hg)];
        const float4 p0 = *(const float4*)tr, p1 = *(const float4*)(tr + 8);
        const float xa[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        float xb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) xb[e] = x[8 * s2 + e];
        bf16x8 ah, al, bh, bl;
        split8(xa, ah, al);
        split8(xb, bh, bl);
        y = mfma32(ah, bh, y);
        y = mfma32(ah, bl, y);
        y = mfma32(al, bh, y);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sm.a[32 + crow(i, hg)][c] = -y[i];   // T21 over A21, read for X above
    }
    __syncthreads();
    float* dst = ck_t + ((size_t)cur_slot * H + cur_h) * ((TT ? 2 : 1) * kGdTFragFloats);
    {
      // A element e of lane (c, hg) in fragment (rb, s) is T[32 rb + c][kpos(s, e, hg)]
      bf16x8* fd = reinterpret_cast<bf16x8*>(dst);
#pragma unroll
      for (int f = 0; f < 6; ++f) {
        const int rb = f < 2 ? 0 : 1, s2 = f < 2 ? f : f - 2;
        const float* tr = &sm.a[32 * rb + c][kpos(s2, 0, hg)];
        const float4 p0 = *(const float4*)tr, p1 = *(const float4*)(tr + 8);
        const float xa[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        bf16x8 th, tl;
        split8(xa, th, tl);
        fd[(2 * f) * 64 + lane] = th;
        fd[(2 * f + 1) * 64 + lane] = tl;
      }
    }
    if constexpr (TT) {
      // A element e of lane (c, hg) in fragment (rb, s) of T^T is T[kpos(s, e, hg)][32 rb + c]
      bf16x8* fd = reinterpret_cast<bf16x8*>(dst + kGdTFragFloats);
#pragma unroll
      for (int f = 0; f < 6; ++f) {
        const int rb = f < 4 ? 0 : 1, s2 = f < 4 ? f : f - 2;
        float xa[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) xa[e] = sm.a[kpos(s2, e, hg)][32 * rb + c];
        bf16x8 th, tl;
        split8(xa, th, tl);
        fd[(2 * f) * 64 + lane] = th;
        fd[(2 * f + 1) * 64 + lane] = tl;
      }
    }
    (void)cur_n;
    if (!more) break;
  }
#undef GD_TMAT_FETCH
#undef GD_TMAT_NEXT
}

// ===========================================================================
// The grouped forward: the chain of chunks cut into groups of 16.
//
// With T = (I + A)^-1 from pass 0, a chunk maps its starting state affinely,
//   U = T diag(beta) V - T diag(beta G) K S0 = Ut - W S0,
//   S_end = (G_L I - Kt^T W) S0 + Kt^T Ut = M S0 + B,   Kt = diag(G_L / G) K,
// so a group of chunks maps it as S_out = A_g S_in + Z_g with A_g the product
// of its chunks' M and Z_g the state it reaches from zero.  Pass 1 composes
// (A_g, Z_g) for every group that another group follows, all groups at once;
// pass 2 walks each slice's groups in order, S_(g+1) = A_g S_g + Z_g, leaving
// every group's starting state; pass 3 (the forward kernel in GROUPED mode)
// runs the chunks of every group from its starting state and writes O and
// the final states.  The serial depth of a slice of n chunks goes from n
// chunk steps to 16 + n/16 + 16 steps.  Every product splits its fp32
// operands into bf16 hi + lo parts (three products), as the chunk kernels do.

#ifndef GD_CMP_OCC
#define GD_CMP_OCC 2
#endif
struct GdComposeSmem {
  alignas(16) bf16 k[kGdC][kKP];
  alignas(16) bf16 v[kGdC][kKP];
  alignas(16) bf16x8 tf[12][64];                      // T's split A fragments, as pass 0 stores them
  alignas(16) bf16x8 kt[4][4][64];                    // K^T as A fragments [d_k block][k-step][lane]
  alignas(16) float eg[kGdC], dec[kGdC], beta[kGdC];
};

// Pass 1: two workgroups of 4 waves per (group slot, value head), one for
// Z_g and one for A_g; groups that are the last of their slice (or hold no
// chunk) return at once, except that for the backward (BWD, whose reverse
// walk needs A_g of every group after a slice's first) A_g is formed for every
// group of a slice with more than one, the last group's partial chunks
// included, and T's slots also hold T^T.  Block x n_gs + gslot H + h takes
// map x (0: Z, 1:
// A), n_gs = gslots H, so the pair shares an XCD whenever n_gs is a multiple
// of 8.  Wave w owns columns [32w, 32w + 32) of its map (C layout, rows = key
// dims).  M is never formed: M X = G_L X - Kt^T T diag(beta G) K X, so every
// chunk takes the map through the forward recurrence's own chunk step (K X,
// the right-hand side, U = T rhs, the rank-64 update), Z with V and from
// zero, A without V and from the identity.  The update is written
// K^T (diag(G_L / G) U): K^T is exact in bf16, so only the scaled U is split
// (two products, not three).  With one map per workgroup the registers and
// LDS allow two workgroups per CU.
template <bool BWD>
__global__ void __launch_bounds__(kGdThreads, GD_CMP_OCC)
gd_grp_compose_kernel(const bf16* __restrict__ k, const bf16* __restrict__ v, const float* __restrict__ g,
                      const float* __restrict__ beta, const int32_t* __restrict__ cu, int n_seg, int T, int H,
                      int Hk, const float* __restrict__ ck_t, float* __restrict__ gA, float* __restrict__ gZ,
                      int n_gs) {
  constexpr size_t t_stride = (BWD ? 2 : 1) * kGdTFragFloats;
  __shared__ GdComposeSmem sm;
  __shared__ int s_bad, s_b;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, hg = lane >> 5, c = lane & 31;
  const bool is_a = (int)blockIdx.x >= n_gs;
  const int bx = is_a ? (int)blockIdx.x - n_gs : (int)blockIdx.x;
  const size_t gslot = bx / H;
  const int h = bx - (bx / H) * H;
  if (tid == 0) {
    s_bad = 0;
    s_b = 0;
  }
  __syncthreads();
  for (int b = tid; b < n_seg; b += kGdThreads) {
    const int c0 = cu[b];
    if (cu[b + 1] < c0) atomicOr(&s_bad, 1);
    if (c0 >= 0 && (size_t)(c0 / kGdGrpTok + b) <= gslot) atomicMax(&s_b, b);
  }
  if (tid == 0 && (cu[0] != 0 || cu[n_seg] != T)) atomicOr(&s_bad, 1);
  __syncthreads();
  if (s_bad || n_seg == 0) return;
  const int b = s_b, seg0 = cu[b], L = cu[b + 1] - seg0;
  const int gi = (int)(gslot - gd_grp_slot(seg0, b, 0));
  const int n_grp = (L + kGdGrpTok - 1) / kGdGrpTok;
  if (gi < 0 || n_grp < 2 || gi >= n_grp - ((BWD && is_a) ? 0 : 1)) return;
  // chunks of the group: 16, fewer in a slice's last group, whose last chunk
  // may be partial (its rows past the slice's end load as zero)
  const int nch = BWD ? std::min(kGdGrpChunks, (L + kGdC - 1) / kGdC - gi * kGdGrpChunks) : kGdGrpChunks;
  const int hk = h / (H / Hk);
  const int n0 = 32 * w + c;
  // V enters Z only; both maps take the same path (one loop, not one per map)
  const float vsc = is_a ? 0.f : 1.f;

  f32x16 X[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i) X[r][i] = 32 * r + 8 * (i >> 2) + (i & 3) == n0 - 4 * hg ? 1.f - vsc : 0.f;

  // chunk j + 1's K, V (Z only), T and gates are loaded into registers while
  // chunk j is computed; scalar registers, not arrays, which the compiler
  // would move to LDS.  Thread tid
  // takes rows tid/16 + 16 it, columns 8 (tid % 16) of K and V (it = 0..3)
  // and the 16-byte pieces tid + 256 it of T's fragments (it = 0..2).
  uint4 pk0, pk1, pk2, pk3, pv0, pv1, pv2, pv3;
  float4 pt0, pt1, pt2;
  float pg, pb;
  const int frow = tid >> 4, fcol = (tid & 15) * 8;
#define GD_CMP_FETCH(j_)                                                                                \
  {                                                                                                    \
    const int t0_ = seg0 + (gi * kGdGrpChunks + (j_)) * kGdC;                                           \
    const int nr_ = BWD ? std::min(kGdC, seg0 + L - t0_) : kGdC;                                        \
    const float* tp_ = ck_t + (gd_ckpt_slot(seg0, b, gi * kGdGrpChunks + (j_)) * H + h) * t_stride      \
                       + 4 * tid;                                                                       \
    /* rows past the slice's end (BWD: a last chunk may be partial) load its */                        \
    /* last row and are zeroed when staged: a load under the row test would */                          \
    /* be a branch closed by a full wait, and so would a select right after */                          \
    /* the loads.  o*_ are row offsets from row frow. */                                                \
    const int o0_ = BWD ? std::min(0, nr_ - 1 - frow) : 0, o1_ = BWD ? std::min(16, nr_ - 1 - frow) : 16;  \
    const int o2_ = BWD ? std::min(32, nr_ - 1 - frow) : 32, o3_ = BWD ? std::min(48, nr_ - 1 - frow) : 48; \
    const bf16* kp_ = k + ((size_t)(t0_ + frow) * Hk + hk) * kGdD + fcol;                               \
    const bf16* vp_ = v + ((size_t)(t0_ + frow) * H + h) * kGdD + fcol;                                 \
    pk0 = *(const uint4*)(kp_ + (ptrdiff_t)o0_ * Hk * kGdD);                                            \
    pk1 = *(const uint4*)(kp_ + (ptrdiff_t)o1_ * Hk * kGdD);                                            \
    pk2 = *(const uint4*)(kp_ + (ptrdiff_t)o2_ * Hk * kGdD);                                            \
    pk3 = *(const uint4*)(kp_ + (ptrdiff_t)o3_ * Hk * kGdD);                                            \
    pv0 = *(const uint4*)(vp_ + (ptrdiff_t)o0_ * H * kGdD);                                             \
    pv1 = *(const uint4*)(vp_ + (ptrdiff_t)o1_ * H * kGdD);                                             \
    pv2 = *(const uint4*)(vp_ + (ptrdiff_t)o2_ * H * kGdD);                                             \
    pv3 = *(const uint4*)(vp_ + (ptrdiff_t)o3_ * H * kGdD);                                             \
    pt0 = *(const float4*)tp_;                                                                          \
    pt1 = *(const float4*)(tp_ + 4 * kGdThreads);                                                       \
    pt2 = *(const float4*)(tp_ + 8 * kGdThreads);                                                       \
    const int rl_ = BWD ? std::min(lane, nr_ - 1) : lane;                                                \
    pg = g[(size_t)(t0_ + rl_) * H + h];                                                                \
    pb = beta[(size_t)(t0_ + rl_) * H + h];                                                             \
  }
  GD_CMP_FETCH(0);
  for (int j = 0; j < nch; ++j) {
    // the lane's indices, made opaque per chunk (they shadow the ones above),
    // so that the addresses formed from them are not hoisted out of the loop
    // and kept in registers, which spilled
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, hg = lane >> 5, c = lane & 31;
    const int frow = tid >> 4, fcol = (tid & 15) * 8;
    const int n0 = 32 * w + c;
    // rows of this chunk: 64, fewer in a partial last chunk (BWD only)
    const int nr = BWD ? std::min(kGdC, L - (gi * kGdGrpChunks + j) * kGdC) : kGdC;
    __syncthreads();                                   // the previous chunk's reads of LDS are done
    *(uint4*)&sm.k[frow][fcol] = frow < nr ? pk0 : zero4();
    *(uint4*)&sm.k[frow + 16][fcol] = frow + 16 < nr ? pk1 : zero4();
    *(uint4*)&sm.k[frow + 32][fcol] = frow + 32 < nr ? pk2 : zero4();
    *(uint4*)&sm.k[frow + 48][fcol] = frow + 48 < nr ? pk3 : zero4();
    *(uint4*)&sm.v[frow][fcol] = frow < nr ? pv0 : zero4();
    *(uint4*)&sm.v[frow + 16][fcol] = frow + 16 < nr ? pv1 : zero4();
    *(uint4*)&sm.v[frow + 32][fcol] = frow + 32 < nr ? pv2 : zero4();
    *(uint4*)&sm.v[frow + 48][fcol] = frow + 48 < nr ? pv3 : zero4();
    reinterpret_cast<float4*>(&sm.tf[0][0])[tid] = pt0;
    reinterpret_cast<float4*>(&sm.tf[0][0])[tid + kGdThreads] = pt1;
    reinterpret_cast<float4*>(&sm.tf[0][0])[tid + 2 * kGdThreads] = pt2;
    if (w == 0) {
      float x = lane < nr ? pg : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      x *= kLog2e;
      const float last = __shfl(x, 63, 64);
      sm.eg[lane] = fast_exp2(x);
      sm.dec[lane] = fast_exp2(last - x);
      sm.beta[lane] = lane < nr ? pb : 0.f;
    }
    if (j + 1 < nch) GD_CMP_FETCH(j + 1);
    __syncthreads();
    // K^T as A fragments, once for the four waves (read after the next
    // barrier): element e of fragment (r, s, lane (fc, fh)) is
    // K[kpos(s, e, fh)][32 r + fc]
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int f = tid + kGdThreads * it;
      const int r = f >> 8, s = (f >> 6) & 3, fl = f & 63, fc = fl & 31, fh = fl >> 5;
      bf16x8 x;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = sm.k[kpos(s, e, fh)][32 * r + fc];
      sm.kt[r][s][fl] = x;
    }
    // K X: A element e of lane (c, hg) at k-step s is K[32 rb + c][kpos(s, e,
    // hg)] (exact in bf16, so X alone is split); X is the B operand straight
    // from its C layout
    f32x16 kx[2] = {};
#pragma unroll
    for (int s = 0; s < kGdD / 16; ++s) {
      float xb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) xb[e] = X[s >> 1][8 * (s & 1) + e];
      bf16x8 bh, bl;
      split8(xb, bh, bl);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const bf16* kr = &sm.k[32 * rb + c][16 * s + 4 * hg];
        const bf16x8 ka = cat(*(const bf16x4*)kr, *(const bf16x4*)(kr + 8));
        kx[rb] = mfma32(ka, bh, kx[rb]);
        kx[rb] = mfma32(ka, bl, kx[rb]);
      }
    }
    // right-hand side beta ([V] - G K X), in place
    {
      // rows 32 rb + crow(i, hg): one lane-dependent base and constant offsets
      const float* bp = &sm.beta[4 * hg];
      const float* ep = &sm.eg[4 * hg];
      const bf16* vp = &sm.v[4 * hg][n0];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ro = 32 * rb + 8 * (i >> 2) + (i & 3);
          kx[rb][i] = bp[ro] * (vsc * (float)vp[ro * kKP] - ep[ro] * kx[rb][i]);
        }
    }
    // U = T rhs: A element e of lane (c, hg) at k-step s is T[32 rb + c][kpos(s,
    // e, hg)]; row block 0 of T has no column past 31
    f32x16 uu[2] = {};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float xb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) xb[e] = kx[s >> 1][8 * (s & 1) + e];
      bf16x8 bh, bl;
      split8(xb, bh, bl);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        if (rb == 0 && s >= 2) continue;
        const int f = rb == 0 ? s : 2 + s;              // fragment (rb, s) as pass 0 split it
        const bf16x8 th = sm.tf[2 * f][lane], tl = sm.tf[2 * f + 1][lane];
        uu[rb] = mfma32(th, bh, uu[rb]);
        uu[rb] = mfma32(th, bl, uu[rb]);
        uu[rb] = mfma32(tl, bh, uu[rb]);
      }
    }
    __syncthreads();                                   // the K^T fragments are complete
    // X <- G_L X + K^T (diag(G_L / G) U)
    const float gL = sm.eg[kGdC - 1];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) X[r][i] *= gL;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float4 d0 = *(const float4*)&sm.dec[32 * (s >> 1) + 16 * (s & 1) + 4 * hg];
      const float4 d1 = *(const float4*)&sm.dec[32 * (s >> 1) + 16 * (s & 1) + 8 + 4 * hg];
      const float dd[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
      float xr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) xr[e] = dd[e] * uu[s >> 1][8 * (s & 1) + e];
      bf16x8 rh, rl;
      split8(xr, rh, rl);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bf16x8 ka = sm.kt[r][s][lane];
        X[r] = mfma32(ka, rh, X[r]);
        X[r] = mfma32(ka, rl, X[r]);
      }
    }
  }
#undef GD_CMP_FETCH
  float* px = (is_a ? gA : gZ) + (gslot * H + h) * kGdD * kGdD + (size_t)(4 * hg) * kGdD + n0;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i) px[(32 * r + 8 * (i >> 2) + (i & 3)) * kGdD] = X[r][i];
}

// Pass 2: four workgroups per (slice, value head) with more than one group,
// one per block of 32 value columns (the columns of S_(g+1) = A_g S_g + Z_g
// depend on the same columns of S_g only).  Block cb n_seg H + slice H + h
// takes column block cb, so the four blocks of a (slice, head) share an XCD,
// and its L2 copy of A_g, whenever n_seg H is a multiple of 8.  From the
// initial state (zero when
// absent), each S_(g+1) is stored as group g+1's starting state.  Wave w owns
// rows [32w, 32w + 32) of the column block: its rows of A_g (row-major, the A
// operand) and Z_g are loaded one group ahead, and the whole block of S_g, the
// B operand, passes through LDS, double-buffered so that one barrier a group
// suffices.  C-layout element i of wave w's row block is B element i % 8 of
// k-step 2w + i / 8, so each wave's accumulator goes to LDS as it stands.
// REV (the backward's state-gradient walk): from the final-state gradient,
// D_(g-1) = A_g^T D_g + F_g from the slice's last group back to its second,
// stored as group g-1's end gradient; the A operand then takes A_g's columns.
constexpr int kGdScanPitch = 20;     // floats per lane in the exchange: b128 accesses free of bank conflicts
using GdScanLds = float[2][4][64][kGdScanPitch];
template <bool REV>
__device__ __forceinline__ void gd_grp_scan_body(GdScanLds& xs, int& s_bad, int blk, const int32_t* __restrict__ cu,
                                                 int n_seg, int T, int H, const float* __restrict__ h0,
                                                 const float* __restrict__ gA, const float* __restrict__ gZ,
                                                 float* __restrict__ gS) {
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, hg = lane >> 5, c = lane & 31;
  const int nbh = n_seg * H;
  if (gd_cu_bad(cu, n_seg, T, &s_bad) || nbh == 0) return;
  const int cb = blk / nbh, bh = blk - cb * nbh;
  if (cb >= 4) return;
  const int b = bh / H, h = bh - b * H;
  const int seg0 = cu[b], L = cu[b + 1] - seg0;
  const int n_grp = (L + kGdGrpTok - 1) / kGdGrpTok;
  if (n_grp < 2) return;
  const int n0 = 32 * cb + c;
  const size_t st_base = (size_t)(b * H + h) * kGdD * kGdD;
  {
    f32x16 S0;
#pragma unroll
    for (int i = 0; i < 16; ++i) S0[i] = h0 ? h0[st_base + (size_t)(32 * w + crow(i, hg)) * kGdD + n0] : 0.f;
    float* x = &xs[0][w][lane][0];
#pragma unroll
    for (int q = 0; q < 4; ++q) *(float4*)(x + 4 * q) = make_float4(S0[4 * q], S0[4 * q + 1], S0[4 * q + 2], S0[4 * q + 3]);
  }
  // step j takes group gi = j (forward) or n_grp - 1 - j (REV).  Its A
  // operand: element e of lane (c, hg) at k-step s is A_g[32w + c][kpos(s, e,
  // hg)] (two float4 a k-step), or for REV A_g[kpos(s, e, hg)][32w + c]
#define GD_SCAN_LOAD(j_, ra_, rz_)                                                                        \
  {                                                                                                    \
    const size_t sl_ = gd_grp_slot(seg0, b, REV ? n_grp - 1 - (j_) : (j_));                            \
    const float* pz_ = gZ + (sl_ * H + h) * kGdD * kGdD + (size_t)(32 * w) * kGdD + n0;                 \
    if constexpr (REV) {                                                                               \
      const float* pa_ = gA + (sl_ * H + h) * kGdD * kGdD + (size_t)(4 * hg) * kGdD + 32 * w + c;       \
      _Pragma("unroll") for (int s_ = 0; s_ < 8; ++s_) {                                                \
        const float* p_ = pa_ + (size_t)(16 * s_) * kGdD;                                               \
        ra_[2 * s_] = make_float4(p_[0], p_[kGdD], p_[2 * kGdD], p_[3 * kGdD]);                          \
        ra_[2 * s_ + 1] = make_float4(p_[8 * kGdD], p_[9 * kGdD], p_[10 * kGdD], p_[11 * kGdD]);         \
      }                                                                                                 \
    } else {                                                                                            \
      const float* pa_ = gA + (sl_ * H + h) * kGdD * kGdD + (size_t)(32 * w + c) * kGdD + 4 * hg;       \
      _Pragma("unroll") for (int s_ = 0; s_ < 8; ++s_) {                                                \
        ra_[2 * s_] = *(const float4*)(pa_ + 16 * s_);                                                  \
        ra_[2 * s_ + 1] = *(const float4*)(pa_ + 16 * s_ + 8);                                          \
      }                                                                                                 \
    }                                                                                                   \
    _Pragma("unroll") for (int i_ = 0; i_ < 16; ++i_) rz_[i_] = pz_[(size_t)crow(i_, hg) * kGdD];        \
  }
  float4 ca[16], na[16];
  float cz[16], nz[16];
  GD_SCAN_LOAD(0, ca, cz);
  __syncthreads();
  for (int gi = 0; gi + 1 < n_grp; ++gi) {
    if (gi + 2 < n_grp) GD_SCAN_LOAD(gi + 1, na, nz);
    f32x16 Sn;
#pragma unroll
    for (int i = 0; i < 16; ++i) Sn[i] = cz[i];
#pragma unroll
    for (int s = 0; s < kGdD / 16; ++s) {
      const float* x = &xs[gi & 1][s >> 1][lane][8 * (s & 1)];
      const float4 b0 = *(const float4*)x, b1 = *(const float4*)(x + 4);
      const float xb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      const float xa[8] = {ca[2 * s].x, ca[2 * s].y, ca[2 * s].z, ca[2 * s].w,
                           ca[2 * s + 1].x, ca[2 * s + 1].y, ca[2 * s + 1].z, ca[2 * s + 1].w};
      bf16x8 ah, al, sh, sl;
      split8(xa, ah, al);
      split8(xb, sh, sl);
      Sn = mfma32(ah, sh, Sn);
      Sn = mfma32(ah, sl, Sn);
      Sn = mfma32(al, sh, Sn);
    }
    const size_t so = REV ? gd_grp_slot(seg0, b, n_grp - 2 - gi) : gd_grp_slot(seg0, b, gi) + 1;
    float* ps = gS + (so * H + h) * kGdD * kGdD + (size_t)(32 * w) * kGdD + n0;
#pragma unroll
    for (int i = 0; i < 16; ++i) ps[(size_t)crow(i, hg) * kGdD] = Sn[i];
    float* x = &xs[(gi + 1) & 1][w][lane][0];
#pragma unroll
    for (int q = 0; q < 4; ++q) *(float4*)(x + 4 * q) = make_float4(Sn[4 * q], Sn[4 * q + 1], Sn[4 * q + 2], Sn[4 * q + 3]);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ca[i] = na[i];
      cz[i] = nz[i];
    }
  }
#undef GD_SCAN_LOAD
}

template <bool REV>
__global__ void __launch_bounds__(kGdThreads, 1)
gd_grp_scan_kernel(const int32_t* __restrict__ cu, int n_seg, int T, int H, const float* __restrict__ h0,
                   const float* __restrict__ gA, const float* __restrict__ gZ, float* __restrict__ gS) {
  __shared__ alignas(16) GdScanLds xs;
  __shared__ int s_bad;
  gd_grp_scan_body<REV>(xs, s_bad, (int)blockIdx.x, cu, n_seg, T, H, h0, gA, gZ, gS);
}

// Both walks of the plain backward in one launch: blocks [0, nb) the forward
// walk (starting states), blocks [nb, 2 nb) the reverse walk (end gradients),
// nb = 4 n_seg H.  When n_seg H is a multiple of 8, each walk's four column
// blocks of a (slice, head) stay on one XCD, as in the separate launches.
__global__ void __launch_bounds__(kGdThreads, 1)
gd_grp_scan2_kernel(const int32_t* __restrict__ cu, int n_seg, int T, int H, int nb, const float* __restrict__ h0,
                    const float* __restrict__ gA, const float* __restrict__ gZ, float* __restrict__ gS,
                    const float* __restrict__ dht, const float* __restrict__ gF, float* __restrict__ gD) {
  __shared__ alignas(16) GdScanLds xs;
  __shared__ int s_bad;
  if ((int)blockIdx.x < nb)
    gd_grp_scan_body<false>(xs, s_bad, (int)blockIdx.x, cu, n_seg, T, H, h0, gA, gZ, gS);
  else
    gd_grp_scan_body<true>(xs, s_bad, (int)blockIdx.x - nb, cu, n_seg, T, H, dht, gA, gF, gD);
}

// Pass 3: the forward kernel on every group from its starting state.
template <typename OutT>
__global__ void __launch_bounds__(kGdThreads, 1)
gd_fwd_grouped_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                      const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
                      int n_seg, int T, int H, int Hk, float scale, const float* __restrict__ h0,
                      OutT* __restrict__ o, float* __restrict__ ht, int32_t* __restrict__ status,
                      const float* __restrict__ ck_t, const float* __restrict__ gS) {
  __shared__ GdSmem sm;
  __shared__ int s_bad;
  gd_fwd_body<OutT, false, true>(sm, s_bad, blockIdx.x, q, k, v, g, beta, cu, n_seg, T, H, Hk, scale, h0, o, ht,
                                 status, nullptr, nullptr, ck_t, gS);
}

// CUs of the current device (cached per device; 256 if the query fails).
int gd_cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Pass 0's launch: items per workgroup so that the grid is one round of
// resident workgroups.
struct GdTmatLaunch {
  unsigned grid;
  int per;
};
GdTmatLaunch gd_tmat_launch(size_t slots, int H) {
  const size_t items = slots * (size_t)H;
  const size_t res = (size_t)gd_cu_count() * kGdTmatPerCu;
  const size_t per = std::max<size_t>(1, (items + res - 1) / res);
  const size_t runs = std::max<size_t>(1, (items + per - 1) / per);
  return {(unsigned)((runs + 7) / 8 * 8), (int)per};   // a multiple of 8: runs map to XCDs in blocks
}

struct GdFwdLayout {
  size_t slots, gslots, ck_t, gA, gZ, gS, total;
};
GdFwdLayout gd_fwd_layout(int32_t T, int32_t H, int32_t n_seg) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  GdFwdLayout l;
  l.slots = (size_t)T / kGdC + (size_t)n_seg + 1;
  l.gslots = (size_t)T / kGdGrpTok + (size_t)n_seg + 1;
  const size_t gs = up(l.gslots * H * kGdD * kGdD * sizeof(float));
  l.ck_t = 0;
  l.gA = up(l.slots * H * kGdTFragFloats * sizeof(float));
  l.gZ = l.gA + gs;
  l.gS = l.gZ + gs;
  l.total = l.gS + gs;
  return l;
}

// Passes 1 and 2 in one launch: they do not depend on each other, so the
// recomputation chain of a (slice, head) runs beside its state-gradient chain
// on another CU.  Block 2j is the state-gradient chain of workgroup j, block
// 2j + 1 its recomputation; the two share one LDS allocation.
constexpr size_t kGdChainsLds = sizeof(GdSmem) > sizeof(GdChainSmem) ? sizeof(GdSmem) : sizeof(GdChainSmem);

template <typename GradT>
__global__ void __launch_bounds__(kGdThreads, 1)
gd_bwd_chains_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                     const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
                     int n_seg, int T, int H, int Hk, float scale, const float* __restrict__ h0,
                     int32_t* __restrict__ status, const float* __restrict__ ck_t, float* __restrict__ ck_s,
                     float* __restrict__ ck_u, const bf16* __restrict__ dout, const float* __restrict__ dht,
                     float* __restrict__ ck_ds, float* __restrict__ ck_dr, GradT* __restrict__ dv,
                     float* __restrict__ dh0) {
  __shared__ __align__(16) unsigned char raw[kGdChainsLds];
  __shared__ int s_bad;
  const int j = blockIdx.x >> 1;
  if (blockIdx.x & 1)
    gd_fwd_body<bf16, true>(*reinterpret_cast<GdSmem*>(raw), s_bad, j, q, k, v, g, beta, cu, n_seg, T, H, Hk,
                            scale, h0, (bf16*)nullptr, nullptr, status, ck_s, ck_u, ck_t);
  else
    gd_bwd_chain_body<GradT>(*reinterpret_cast<GdChainSmem*>(raw), s_bad, j, q, k, g, beta, cu, n_seg, T, H, Hk,
                             scale, dout, dht, ck_t, ck_ds, ck_dr, dv, dh0);
}

// The grouped chains (slices longer than one group).  Pass 1b: the offsets F_g
// of the state-gradient walk, one workgroup per (group slot, value head) for
// every group after a slice's first.
__global__ void __launch_bounds__(kGdThreads, 1)
gd_bwd_cgrp_compose_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const float* __restrict__ g,
                           const float* __restrict__ beta, const int32_t* __restrict__ cu, int n_seg, int T, int H,
                           int Hk, float scale, const bf16* __restrict__ dout, const float* __restrict__ ck_t,
                           float* __restrict__ gF) {
  __shared__ GdChainSmem sm;
  __shared__ int s_bad;
  gd_bwd_chain_body<float, 1>(sm, s_bad, blockIdx.x, q, k, g, beta, cu, n_seg, T, H, Hk, scale, dout, nullptr, ck_t,
                              nullptr, nullptr, (float*)nullptr, nullptr, gF, nullptr);
}

// Passes 1 and 2 on groups, side by side: block 2j is the state-gradient walk
// of group slot x head j from its end gradient, block 2j + 1 the
// recomputation of the same group from its starting state.
template <typename GradT>
__global__ void __launch_bounds__(kGdThreads, 1)
gd_bwd_grp_chains_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                         const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
                         int n_seg, int T, int H, int Hk, float scale, const float* __restrict__ h0,
                         int32_t* __restrict__ status, const float* __restrict__ ck_t, float* __restrict__ ck_s,
                         float* __restrict__ ck_u, const bf16* __restrict__ dout, const float* __restrict__ dht,
                         float* __restrict__ ck_ds, float* __restrict__ ck_dr, GradT* __restrict__ dv,
                         float* __restrict__ dh0, const float* __restrict__ gS, const float* __restrict__ gD) {
  __shared__ __align__(16) unsigned char raw[kGdChainsLds];
  __shared__ int s_bad;
  const int j = blockIdx.x >> 1;
  if (blockIdx.x & 1)
    gd_fwd_body<bf16, true, true>(*reinterpret_cast<GdSmem*>(raw), s_bad, j, q, k, v, g, beta, cu, n_seg, T, H, Hk,
                                  scale, h0, (bf16*)nullptr, nullptr, status, ck_s, ck_u, ck_t, gS);
  else
    gd_bwd_chain_body<GradT, 2>(*reinterpret_cast<GdChainSmem*>(raw), s_bad, j, q, k, g, beta, cu, n_seg, T, H, Hk,
                                scale, dout, dht, ck_t, ck_ds, ck_dr, dv, dh0, nullptr, gD);
}

// The training forward's group pass: O and the final states as the grouped
// forward, plus the backward's checkpoints (every chunk's starting state and
// U), with T's fragments in the backward's slots.
template <typename OutT>
__global__ void __launch_bounds__(kGdThreads, 1)
gd_fwd_train_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
                    int n_seg, int T, int H, int Hk, float scale, const float* __restrict__ h0,
                    OutT* __restrict__ o, float* __restrict__ ht, int32_t* __restrict__ status,
                    const float* __restrict__ ck_t, float* __restrict__ ck_s, float* __restrict__ ck_u,
                    const float* __restrict__ gS) {
  __shared__ GdSmem sm;
  __shared__ int s_bad;
  gd_fwd_body<OutT, false, true, true>(sm, s_bad, blockIdx.x, q, k, v, g, beta, cu, n_seg, T, H, Hk, scale, h0, o,
                                       ht, status, ck_s, ck_u, ck_t, gS);
}

// The backward after a training forward: the state-gradient walk alone on
// every group (the recomputation's checkpoints are in the workspace); it
// validates cu_seqlens and writes the status word.
template <typename GradT>
__global__ void __launch_bounds__(kGdThreads, 1)
gd_bwd_cwalk_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const float* __restrict__ g,
                    const float* __restrict__ beta, const int32_t* __restrict__ cu, int n_seg, int T, int H, int Hk,
                    float scale, int32_t* __restrict__ status, const float* __restrict__ ck_t,
                    const bf16* __restrict__ dout, const float* __restrict__ dht, float* __restrict__ ck_ds,
                    float* __restrict__ ck_dr, GradT* __restrict__ dv, float* __restrict__ dh0,
                    const float* __restrict__ gD) {
  __shared__ GdChainSmem sm;
  __shared__ int s_bad;
  const bool bad = gd_cu_bad(cu, n_seg, T, &s_bad);
  if (blockIdx.x == 0 && threadIdx.x == 0) *status = bad ? PVB_E_BAD_CU_SEQLENS : PVB_OK;
  if (bad) return;
  gd_bwd_chain_body<GradT, 2>(sm, s_bad, blockIdx.x, q, k, g, beta, cu, n_seg, T, H, Hk, scale, dout, dht, ck_t,
                              ck_ds, ck_dr, dv, dh0, nullptr, gD);
}

struct GdChunkSmem {
  GdTiles t;                         // Ah and P become M and N in place
  alignas(16) float u[kGdC][kUP];    // U
  alignas(16) float dr[kGdC][kUP];   // dR
  float xr[4][kGdC], gr[4][kGdC], rk[4][kGdC];   // row partials per column quarter
  float rs[6][32], cs[6][32];                    // row and column partials of the dA / dP blocks
  float red[4];
  int slice;
};

// Pass 3: one workgroup of 8 waves per (checkpoint slot, value head); slots
// that hold no chunk return at once.  Wave w works on row block rb = w / 4
// (positions [32 rb, 32 rb + 32)) and quarter cq = w % 4: value columns
// [32 cq, 32 cq + 32) for the row sums through K S0 and Q S0, key dims
// [32 cq, 32 cq + 32) of dK and dQ.  U and dR are staged in LDS once; S0 and
// dS are read from the checkpoints where they are used, one k-step ahead.
__global__ void __launch_bounds__(kGdChunkThreads, 1)
gd_bwd_chunk_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
                    int n_seg, int T, int H, int Hk, float scale, const bf16* __restrict__ dout,
                    const float* __restrict__ ck_s, const float* __restrict__ ck_u,
                    const float* __restrict__ ck_ds, const float* __restrict__ ck_dr, float* __restrict__ dq,
                    float* __restrict__ dk, float* __restrict__ dg, float* __restrict__ dbeta, bool atomic_qk) {
  __shared__ GdChunkSmem sm;
  __shared__ int s_bad;
  GdTiles& t = sm.t;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, hg = lane >> 5, c = lane & 31;
  const int rb = w >> 2, cq = w & 3;
  const int slot = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  if (gd_cu_bad_find(cu, n_seg, T, slot, &s_bad, &sm.slice) || n_seg == 0) return;
  const int b = sm.slice, seg0 = cu[b], L = cu[b + 1] - seg0;
  const int ci = slot - (seg0 / kGdC + b);
  if (ci < 0 || ci * kGdC >= L) return;
  const int hk = h / (H / Hk);
  const int t0 = seg0 + ci * kGdC, n = min(kGdC, L - ci * kGdC);
  const float* S0p = ck_s + ((size_t)slot * H + h) * kGdStateFloats;
  const float* dSp = ck_ds + ((size_t)slot * H + h) * kGdStateFloats;
  const float* Up = ck_u + ((size_t)slot * H + h) * kGdChunkFloats;
  const float* dRp = ck_dr + ((size_t)slot * H + h) * kGdChunkFloats;
  const int n0 = 32 * cq + c;                         // this lane's value column, and key dim

  // this wave's rows of V in its value columns, loaded with the tiles and in
  // flight during the barrier
  float vc[16];
  {
    GdStage<kGdChunkThreads> st;
    st.fetch(q, k, dout, g, beta, t0, n, H, Hk, h, hk, tid);
    float4 xu[4], xd[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {                  // 16-byte pieces: row ch / 32, columns 4 (ch % 32)..
      const int ch = tid + kGdChunkThreads * it;
      xu[it] = *(const float4*)(Up + 4 * ch);
      xd[it] = *(const float4*)(dRp + 4 * ch);
    }
    // rows past the chunk's end read its last row (always in bounds) and are
    // then set to zero: a load under the row test would be a branch, which
    // the compiler closes by waiting for the load, one round trip per row
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 32 * rb + crow(i, hg);
      const float x = (float)v[((size_t)(t0 + min(row, n - 1)) * H + h) * kGdD + n0];
      vc[i] = row < n ? x : 0.f;
    }
    st.put(t, tid);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int ch = tid + kGdChunkThreads * it;
      *(float4*)&sm.u[ch >> 5][4 * (ch & 31)] = xu[it];
      *(float4*)&sm.dr[ch >> 5][4 * (ch & 31)] = xd[it];
    }
    if (w == 0) gd_gates(t, st.g, st.b, lane);
  }
  __syncthreads();
  // the first k-step of S0 and dS for the products after dA and dP (row n0,
  // value columns 16 s + 8 hg ..), in flight during the blocks before them
  float xs[2][8], xds[2][8];
  auto fetch_s = [&](int s, int buf) {
    const int col = 16 * s + 8 * hg;
    load8f(S0p + (size_t)n0 * kGdD + col, xs[buf]);
    load8f(dSp + (size_t)n0 * kGdD + col, xds[buf]);
  };
  fetch_s(0, 0);

  if (w < 6) {
    // Ah and P blocks: KK (1,0), QK (0,0), QK (1,0), KK (0,0), KK (1,1), QK (1,1)
    const bool isq = w == 1 || w == 2 || w == 5;
    const int bi = (w == 1 || w == 3) ? 0 : 1, bj = (w == 4 || w == 5) ? 1 : 0;
    gd_ah_p_block(t, isq, bi, bj, c, hg);
  } else {                                            // block (0, 1) of Ah and P (then M and N) is zero
    for (int e = tid - 384; e < 32 * 32; e += 128) {
      t.ah[e >> 5][32 + (e & 31)] = 0.f;
      t.p[e >> 5][32 + (e & 31)] = 0.f;
    }
  }
  // ---- the row partial sum_c dR V (dbeta) over this wave's value columns;
  // the K S0 and Q S0 terms come later from dR S0^T and dO S0^T:
  // sum_c dR (K S0) = sum_k K o (dR S0^T), sum_c dO (Q S0) = sum_k Q o (dO S0^T)
  {
    float xr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) xr[i] = sm.dr[32 * rb + crow(i, hg)][n0] * vc[i];
    int idx;
    const float sx = row_sum16(xr, c, idx);
    if ((c & 1) == 0) sm.xr[cq][32 * rb + crow(idx, hg)] = sx;
  }
  __syncthreads();                                    // Ah and P are complete

  f32x16 r1 = {}, kt1 = {}, q1 = {};
  // waves 2 and 3 take the S0 phase first, in step with waves 6 and 7 (the
  // same quarters, the other row block), which have no dA / dP block: both row
  // blocks then read the same S0 and dS lines at about the same time
  const bool s0_first = w == 2 || w == 3;
#pragma clang loop unroll(disable)
  for (int ph = 0; ph < 2; ++ph) {
    if ((ph == 0) != s0_first) {
      // ---- dA = -strict_lower(dR U^T) and dP = scale lower(dO U^T), contracted
      // over all value columns (k index = column 16 s + 8 hg + e), one block per
      // wave: its row and column partials of dA o Ah (with beta of the row for the
      // columns) and dP o P, then M = diag(beta) (Gam o dA) and N = Gam o dP
      // written over Ah and P in place (each wave reads and writes its own block).
      if (w < 6) {
        const bool isp = w >= 3;
        const int bi = (w == 1 || w == 3) ? 0 : 1, bj = (w == 2 || w == 5) ? 1 : 0;
        f32x16 acc = {};
    #pragma unroll
        for (int s = 0; s < kGdD / 16; ++s) {
          const int col = 16 * s + 8 * hg;
          float xu[8];
          load8f(&sm.u[32 * bj + c][col], xu);
          bf16x8 uh, ul;
          split8(xu, uh, ul);
          if (isp) {
            const bf16x8 a = *(const bf16x8*)&t.dO[32 * bi + c][col];
            acc = mfma32(a, uh, acc);
            acc = mfma32(a, ul, acc);
          } else {
            float xd[8];
            load8f(&sm.dr[32 * bi + c][col], xd);
            bf16x8 rh, rl;
            split8(xd, rh, rl);
            acc = mfma32(rh, uh, acc);
            acc = mfma32(rh, ul, acc);
            acc = mfma32(rl, uh, acc);
          }
        }
        const int cc = 32 * bj + c;
        const float glc = t.gl[cc];
        float rsum[16], csum = 0.f;
    #pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 32 * bi + crow(i, hg);
          const float gam = fast_exp2(fminf(t.gl[r] - glc, 0.f));
          if (isp) {
            const float dpv = cc <= r ? scale * acc[i] : 0.f;
            const float prod = dpv * t.p[r][cc];
            rsum[i] = prod;
            csum += prod;
            t.p[r][cc] = gam * dpv;
          } else {
            const float dav = cc < r ? -acc[i] : 0.f;
            const float prod = dav * t.ah[r][cc];
            const float br = t.beta[r];
            rsum[i] = prod;
            csum += br * prod;
            t.ah[r][cc] = br * gam * dav;
          }
        }
        int idx;
        const float rsv = row_sum16(rsum, c, idx);
        csum += swap_halves(csum);
        if ((c & 1) == 0) sm.rs[w][crow(idx, hg)] = rsv;
        if (hg == 0) sm.cs[w][c] = csum;
      }

    } else {
      // ---- row block rb, key dims of quarter cq: dR S0^T, U dS^T (= dKt) and
      // dO S0^T contracted over all value columns; <dS, S0> over these key dims
      // (waves of row block 0); the row partials sum_d dKt o Kt, and over these
      // key dims sum_d K o (dR S0^T) = sum_c dR (K S0) and
      // sum_d Q o (dO S0^T) = sum_c dO (Q S0)
      {
        float sdot = 0.f;
    #pragma unroll
        for (int s = 0; s < kGdD / 16; ++s) {
          const int cur = s & 1, col = 16 * s + 8 * hg;
          if (s + 1 < kGdD / 16) fetch_s(s + 1, cur ^ 1);
          if (rb == 0) {
    #pragma unroll
            for (int e = 0; e < 8; ++e) sdot += xs[cur][e] * xds[cur][e];
          }
          float xr[8], xu[8];
          load8f(&sm.dr[32 * rb + c][col], xr);
          load8f(&sm.u[32 * rb + c][col], xu);
          bf16x8 sh, sl, dh, dl, rh, rl, uh, ul;
          split8(xs[cur], sh, sl);
          split8(xds[cur], dh, dl);
          split8(xr, rh, rl);
          split8(xu, uh, ul);
          const bf16x8 oa = *(const bf16x8*)&t.dO[32 * rb + c][col];
          r1 = mfma32(rh, sh, r1);
          r1 = mfma32(rh, sl, r1);
          r1 = mfma32(rl, sh, r1);
          kt1 = mfma32(uh, dh, kt1);
          kt1 = mfma32(uh, dl, kt1);
          kt1 = mfma32(ul, dh, kt1);
          q1 = mfma32(oa, sh, q1);
          q1 = mfma32(oa, sl, q1);
        }
        if (rb == 0) {
    #pragma unroll
          for (int off = 32; off > 0; off >>= 1) sdot += __shfl_xor(sdot, off, 64);
          if (lane == 0) sm.red[cq] = sdot;
        }
        float x[16];
    #pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = 32 * rb + crow(i, hg);
          x[i] = kt1[i] * t.dec[row] * (float)t.k[row][n0];
        }
        float xb[16], xc[16];
    #pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = 32 * rb + crow(i, hg);
          xb[i] = (float)t.k[row][n0] * r1[i];
          xc[i] = (float)t.q[row][n0] * q1[i];
        }
        int idx;
        const float sx = row_sum16(x, c, idx);
        const float sb = row_sum16(xb, c, idx);
        const float sc = row_sum16(xc, c, idx);
        if ((c & 1) == 0) {
          const int row = 32 * rb + crow(idx, hg);
          sm.rk[cq][row] = sx;
          // this wave wrote sm.xr[cq][row] in the first phase (same lane, same row)
          sm.xr[cq][row] -= t.eg[row] * sb;
          sm.gr[cq][row] = -t.beta[row] * sb + scale * sc;
        }
      }
    }
  }
  __syncthreads();                                    // M, N and every partial are complete

  // ---- dbeta and dg of the chunk's positions (wave 0, lane = position).  The
  // dA blocks are waves 0 (1,0), 1 (0,0), 2 (1,1); the dP blocks waves 3 (0,0),
  // 4 (1,0), 5 (1,1).
  if (w == 0) {
    const int i = lane, ii = i & 31;
    const bool up = i >= 32;
    const float rowA = up ? sm.rs[0][ii] + sm.rs[2][ii] : sm.rs[1][ii];
    const float colA = up ? sm.cs[2][ii] : sm.cs[0][ii] + sm.cs[1][ii];
    const float rowP = up ? sm.rs[4][ii] + sm.rs[5][ii] : sm.rs[3][ii];
    const float colP = up ? sm.cs[5][ii] : sm.cs[3][ii] + sm.cs[4][ii];
    float dba = rowA, dG = 0.f, rk = 0.f;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      dba += sm.xr[qq][i];
      dG += sm.gr[qq][i];
      rk += sm.rk[qq][i];
    }
    float dgm = rowP - colP + t.beta[i] * rowA - colA + t.eg[i] * dG - rk;
    float tot = rk;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off, 64);
    if (i == n - 1) dgm += tot + t.eg[i] * (sm.red[0] + sm.red[1] + sm.red[2] + sm.red[3]);
    if (i >= n) dgm = 0.f;
    // dg_i = sum over j >= i of dgamma_j: a reversed inclusive scan
    float x = dgm;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_down(x, off, 64);
      if (i + off < 64) x += y;
    }
    if (i < n) {
      dg[(size_t)(t0 + i) * H + h] = x;
      dbeta[(size_t)(t0 + i) * H + h] = dba;
    }
  }

  // ---- dK = -diag(G beta) dR S0^T + diag(G_L / G) dKt + N^T Q + (M + M^T) K and
  // dQ = scale diag(G) dO S0^T + N K, row block rb, key dims of quarter cq;
  // k index = position 16 s + 8 hg + e
  {
    f32x16 ka = {}, qa = {};
#pragma unroll
    for (int s = 0; s < kGdC / 16; ++s) {
      const int p0 = 16 * s + 8 * hg;
      bf16x8 bq, bk;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bq[e] = t.q[p0 + e][n0];
        bk[e] = t.k[p0 + e][n0];
      }
      bf16x8 hh, ll;
      float x[8];
      if (!(rb == 1 && s < 2)) {                      // N^T and M^T of row block 1 have no position below 32
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = t.p[p0 + e][32 * rb + c];
        split8(x, hh, ll);
        ka = mfma32(hh, bq, ka);
        ka = mfma32(ll, bq, ka);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = t.ah[p0 + e][32 * rb + c];
        split8(x, hh, ll);
        ka = mfma32(hh, bk, ka);
        ka = mfma32(ll, bk, ka);
      }
      if (!(rb == 0 && s >= 2)) {                     // N and M of row block 0 have no position past 31
        load8f(&t.ah[32 * rb + c][p0], x);
        split8(x, hh, ll);
        ka = mfma32(hh, bk, ka);
        ka = mfma32(ll, bk, ka);
        load8f(&t.p[32 * rb + c][p0], x);
        split8(x, hh, ll);
        qa = mfma32(hh, bk, qa);
        qa = mfma32(ll, bk, qa);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 32 * rb + crow(i, hg);
      if (row >= n) continue;
      const float gr = t.eg[row];
      const float kv = -gr * t.beta[row] * r1[i] + t.dec[row] * kt1[i] + ka[i];
      const float qv = scale * gr * q1[i] + qa[i];
      const size_t o = ((size_t)(t0 + row) * Hk + hk) * kGdD + n0;
      if (atomic_qk) {
        atomicAdd(dk + o, kv);
        atomicAdd(dq + o, qv);
      } else {
        dk[o] = kv;
        dq[o] = qv;
      }
    }
  }
}

// Clears dQ and dK before value heads that share a query/key head add into
// them; writes nothing when cu_seqlens is bad (the backward then writes nothing).
__global__ void __launch_bounds__(256)
gd_clear_kernel(float* __restrict__ a, float* __restrict__ b2, int64_t n, const int32_t* __restrict__ cu, int n_seg,
                int T) {
  __shared__ int s_bad;
  if (gd_cu_bad(cu, n_seg, T, &s_bad)) return;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    a[i] = 0.f;
    b2[i] = 0.f;
  }
}

struct GdBwdLayout {
  size_t slots, ck_s, ck_u, ck_ds, ck_dr, ck_t, gslots, gA, gZ, gS, gF, gD, total;
};
GdBwdLayout gd_bwd_layout(int32_t T, int32_t H, int32_t n_seg) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  GdBwdLayout l;
  l.slots = (size_t)T / kGdC + (size_t)n_seg + 1;
  const size_t st = up(l.slots * H * kGdStateFloats * sizeof(float));
  const size_t ch = up(l.slots * H * kGdChunkFloats * sizeof(float));
  l.ck_s = 0;
  l.ck_ds = st;
  l.ck_u = 2 * st;
  l.ck_dr = 2 * st + ch;
  l.ck_t = 2 * st + 2 * ch;
  // per group slot and head: the map A_g, the state Z_g and starting state of
  // the recomputation, the offset F_g and end gradient of the state-gradient walk
  l.gslots = (size_t)T / kGdGrpTok + (size_t)n_seg + 1;
  const size_t gs = up(l.gslots * H * kGdStateFloats * sizeof(float));
  l.gA = l.ck_t + up(l.slots * H * 2 * kGdTFragFloats * sizeof(float));
  l.gZ = l.gA + gs;
  l.gS = l.gZ + gs;
  l.gF = l.gS + gs;
  l.gD = l.gF + gs;
  l.total = l.gD + gs;
  return l;
}

}  // namespace
}  // namespace pvb

extern "C" size_t pvb_gated_delta_bwd_workspace_bytes(int32_t T, int32_t H, int32_t n_seg) {
  if (T < 0 || H <= 0 || n_seg < 0) return 0;
  return pvb::gd_bwd_layout(T, H, n_seg).total;
}

namespace pvb {
namespace {
// after_fwd: the workspace holds pvb_gated_delta_fwd_train's checkpoints for
// the same inputs, so T's pass and the recomputation are skipped.
pvb_status gated_delta_bwd_call(const void* d_q, const void* d_k, const void* d_v, const float* d_g,
                                const float* d_beta, const int32_t* d_cu, const int32_t* h_cu, int32_t n_seg,
                                int32_t T, int32_t H, int32_t H_k, int32_t d, float scale, const float* d_h0,
                                const void* d_dout, const float* d_dht, float* d_dq, float* d_dk, void* d_dv,
                                float* d_dg, float* d_dbeta, float* d_dh0, int32_t grad_dtype, void* workspace,
                                size_t workspace_bytes, int32_t* d_status, void* stream, bool after_fwd) {
  if (n_seg < 0 || T < 0 || H <= 0 || d_cu == nullptr || d_status == nullptr) return PVB_E_INVALID_ARG;
  if (H_k <= 0 || H % H_k != 0) return PVB_E_INVALID_ARG;
  if (n_seg > PVB_MAX_COUNT) return PVB_E_OVERFLOW;
  if (T > 0 && (d_q == nullptr || d_k == nullptr || d_v == nullptr || d_g == nullptr || d_beta == nullptr ||
                d_dout == nullptr || d_dq == nullptr || d_dk == nullptr || d_dv == nullptr || d_dg == nullptr ||
                d_dbeta == nullptr))
    return PVB_E_INVALID_ARG;
  if (grad_dtype != PVB_BF16 && grad_dtype != PVB_F32) return PVB_E_INVALID_ARG;
  if (!(scale > 0.f) || !(scale < INFINITY)) return PVB_E_INVALID_ARG;
  if (d != kGdD) return PVB_E_UNSUPPORTED;
  const GdBwdLayout lay = gd_bwd_layout(T, H, n_seg);
  if ((int64_t)T * H * d >= ((int64_t)1 << 31) || !grid_fits((uint64_t)8 * n_seg * H, kGdThreads) ||
      !grid_fits((uint64_t)lay.slots * H, kGdChunkThreads) || !grid_fits((uint64_t)2 * lay.gslots * H, kGdThreads))
    return PVB_E_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < lay.total) return PVB_E_WORKSPACE;
  const pvb_status hs = check_host_cu(h_cu, n_seg, T);
  if (hs != PVB_OK) return hs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* ck_s = reinterpret_cast<float*>(ws + lay.ck_s);
  float* ck_u = reinterpret_cast<float*>(ws + lay.ck_u);
  float* ck_ds = reinterpret_cast<float*>(ws + lay.ck_ds);
  float* ck_dr = reinterpret_cast<float*>(ws + lay.ck_dr);
  float* ck_t = reinterpret_cast<float*>(ws + lay.ck_t);
  const bool atomic_qk = H != H_k;
  const int64_t nqk = (int64_t)T * H_k * d;
  if (atomic_qk && nqk > 0) {
    const unsigned blocks = (unsigned)std::min<int64_t>((nqk + 255) / 256, 8192);
    gd_clear_kernel<<<blocks, 256, 0, s>>>(d_dq, d_dk, nqk, d_cu, n_seg, T);
  }
  const unsigned grid = (unsigned)std::max<int64_t>(1, (int64_t)n_seg * H);
  // pass 0: T = (I + A)^-1 of every chunk
  if (!after_fwd) {
    const GdTmatLaunch tl = gd_tmat_launch(lay.slots, H);
    gd_tmat_kernel<true><<<tl.grid, 64, 0, s>>>((const bf16*)d_k, d_g, d_beta, d_cu, n_seg, T, H, H_k, ck_t,
                                                tl.per);
  }
  // passes 1 and 2 side by side: the recomputation stores the chunk-start
  // states and the U of every chunk (it also validates cu_seqlens and writes
  // the status word); the state-gradient chain stores dS at every chunk's end
  // and dR, and writes dV and dh0.  A slice longer than one group of 1024
  // tokens is walked in groups (whether one is, is known without the host
  // mirror only on the device): the recomputation's group maps and starting
  // states as in the grouped forward, the state-gradient walk's offsets, its
  // group end gradients by the transposed maps, then both walks on every
  // group at once.
  bool multi = true;
  if (h_cu != nullptr) {
    multi = false;
    for (int32_t b = 0; b < n_seg && !multi; ++b) multi = h_cu[b + 1] - h_cu[b] > kGdGrpTok;
  }
  if (after_fwd) {
    // the state-gradient walk alone, in groups: the recomputation's group maps
    // are in the workspace
    float* gA = reinterpret_cast<float*>(ws + lay.gA);
    float* gF = reinterpret_cast<float*>(ws + lay.gF);
    float* gD = reinterpret_cast<float*>(ws + lay.gD);
    const unsigned ggrid = (unsigned)(lay.gslots * H);
    if (multi) {
      gd_bwd_cgrp_compose_kernel<<<ggrid, kGdThreads, 0, s>>>((const bf16*)d_q, (const bf16*)d_k, d_g, d_beta,
                                                              d_cu, n_seg, T, H, H_k, scale, (const bf16*)d_dout,
                                                              ck_t, gF);
      const unsigned sgrid = (unsigned)std::max<int64_t>(1, 4 * (int64_t)n_seg * H);
      gd_grp_scan_kernel<true><<<sgrid, kGdThreads, 0, s>>>(d_cu, n_seg, T, H, d_dht, gA, gF, gD);
    }
    if (grad_dtype == PVB_F32)
      gd_bwd_cwalk_kernel<float><<<std::max(1u, ggrid), kGdThreads, 0, s>>>(
          (const bf16*)d_q, (const bf16*)d_k, d_g, d_beta, d_cu, n_seg, T, H, H_k, scale, d_status, ck_t,
          (const bf16*)d_dout, d_dht, ck_ds, ck_dr, (float*)d_dv, d_dh0, gD);
    else
      gd_bwd_cwalk_kernel<bf16><<<std::max(1u, ggrid), kGdThreads, 0, s>>>(
          (const bf16*)d_q, (const bf16*)d_k, d_g, d_beta, d_cu, n_seg, T, H, H_k, scale, d_status, ck_t,
          (const bf16*)d_dout, d_dht, ck_ds, ck_dr, (bf16*)d_dv, d_dh0, gD);
  } else if (!multi) {
    if (grad_dtype == PVB_F32)
      gd_bwd_chains_kernel<float><<<2 * grid, kGdThreads, 0, s>>>(
          (const bf16*)d_q, (const bf16*)d_k, (const bf16*)d_v, d_g, d_beta, d_cu, n_seg, T, H, H_k, scale, d_h0,
          d_status, ck_t, ck_s, ck_u, (const bf16*)d_dout, d_dht, ck_ds, ck_dr, (float*)d_dv, d_dh0);
    else
      gd_bwd_chains_kernel<bf16><<<2 * grid, kGdThreads, 0, s>>>(
          (const bf16*)d_q, (const bf16*)d_k, (const bf16*)d_v, d_g, d_beta, d_cu, n_seg, T, H, H_k, scale, d_h0,
          d_status, ck_t, ck_s, ck_u, (const bf16*)d_dout, d_dht, ck_ds, ck_dr, (bf16*)d_dv, d_dh0);
  } else {
    float* gA = reinterpret_cast<float*>(ws + lay.gA);
    float* gZ = reinterpret_cast<float*>(ws + lay.gZ);
    float* gS = reinterpret_cast<float*>(ws + lay.gS);
    float* gF = reinterpret_cast<float*>(ws + lay.gF);
    float* gD = reinterpret_cast<float*>(ws + lay.gD);
    const unsigned ggrid = (unsigned)(lay.gslots * H);
    gd_grp_compose_kernel<true><<<2 * ggrid, kGdThreads, 0, s>>>(
        (const bf16*)d_k, (const bf16*)d_v, d_g, d_beta, d_cu, n_seg, T, H, H_k, ck_t, gA, gZ, (int)ggrid);
    gd_bwd_cgrp_compose_kernel<<<ggrid, kGdThreads, 0, s>>>((const bf16*)d_q, (const bf16*)d_k, d_g, d_beta, d_cu,
                                                            n_seg, T, H, H_k, scale, (const bf16*)d_dout, ck_t, gF);
    const unsigned sgrid = (unsigned)std::max<int64_t>(1, 4 * (int64_t)n_seg * H);
    gd_grp_scan2_kernel<<<2 * sgrid, kGdThreads, 0, s>>>(d_cu, n_seg, T, H, (int)sgrid, d_h0, gA, gZ, gS, d_dht,
                                                         gF, gD);
    if (grad_dtype == PVB_F32)
      gd_bwd_grp_chains_kernel<float><<<2 * ggrid, kGdThreads, 0, s>>>(
          (const bf16*)d_q, (const bf16*)d_k, (const bf16*)d_v, d_g, d_beta, d_cu, n_seg, T, H, H_k, scale, d_h0,
          d_status, ck_t, ck_s, ck_u, (const bf16*)d_dout, d_dht, ck_ds, ck_dr, (float*)d_dv, d_dh0, gS, gD);
    else
      gd_bwd_grp_chains_kernel<bf16><<<2 * ggrid, kGdThreads, 0, s>>>(
          (const bf16*)d_q, (const bf16*)d_k, (const bf16*)d_v, d_g, d_beta, d_cu, n_seg, T, H, H_k, scale, d_h0,
          d_status, ck_t, ck_s, ck_u, (const bf16*)d_dout, d_dht, ck_ds, ck_dr, (bf16*)d_dv, d_dh0, gS, gD);
  }
  // pass 3, chunk-parallel: dQ, dK, dg, dbeta
  gd_bwd_chunk_kernel<<<(unsigned)(lay.slots * H), kGdChunkThreads, 0, s>>>(
      (const bf16*)d_q, (const bf16*)d_k, (const bf16*)d_v, d_g, d_beta, d_cu, n_seg, T, H, H_k, scale,
      (const bf16*)d_dout, ck_s, ck_u, ck_ds, ck_dr, d_dq, d_dk, d_dg, d_dbeta, atomic_qk);
  return hipGetLastError() == hipSuccess ? PVB_OK : PVB_E_HIP;
}
}  // namespace
}  // namespace pvb

extern "C" pvb_status pvb_gated_delta_bwd(const void* d_q, const void* d_k, const void* d_v, const float* d_g,
                                          const float* d_beta, const int32_t* d_cu, const int32_t* h_cu,
                                          int32_t n_seg, int32_t T, int32_t H, int32_t H_k, int32_t d, float scale,
                                          const float* d_h0, const void* d_dout, const float* d_dht, float* d_dq,
                                          float* d_dk, void* d_dv, float* d_dg, float* d_dbeta, float* d_dh0,
                                          int32_t grad_dtype, void* workspace, size_t workspace_bytes,
                                          int32_t* d_status, void* stream) {
  return pvb::gated_delta_bwd_call(d_q, d_k, d_v, d_g, d_beta, d_cu, h_cu, n_seg, T, H, H_k, d, scale, d_h0, d_dout,
                                   d_dht, d_dq, d_dk, d_dv, d_dg, d_dbeta, d_dh0, grad_dtype, workspace,
                                   workspace_bytes, d_status, stream, false);
}

extern "C" pvb_status pvb_gated_delta_bwd_after_fwd(const void* d_q, const void* d_k, const void* d_v,
                                                    const float* d_g, const float* d_beta, const int32_t* d_cu,
                                                    const int32_t* h_cu, int32_t n_seg, int32_t T, int32_t H,
                                                    int32_t H_k, int32_t d, float scale, const float* d_h0,
                                                    const void* d_dout, const float* d_dht, float* d_dq, float* d_dk,
                                                    void* d_dv, float* d_dg, float* d_dbeta, float* d_dh0,
                                                    int32_t grad_dtype, void* workspace, size_t workspace_bytes,
                                                    int32_t* d_status, void* stream) {
  return pvb::gated_delta_bwd_call(d_q, d_k, d_v, d_g, d_beta, d_cu, h_cu, n_seg, T, H, H_k, d, scale, d_h0, d_dout,
                                   d_dht, d_dq, d_dk, d_dv, d_dg, d_dbeta, d_dh0, grad_dtype, workspace,
                                   workspace_bytes, d_status, stream, true);
}

namespace pvb {
namespace {
pvb_status gated_delta_call(const void* d_q, const void* d_k, const void* d_v, const float* d_g,
                            const float* d_beta, const int32_t* d_cu, const int32_t* h_cu, int32_t n_seg,
                            int32_t T, int32_t H, int32_t H_k, int32_t d, float scale, const float* d_h0,
                            void* d_o, int32_t o_dtype, float* d_ht, void* workspace, size_t workspace_bytes,
                            int32_t* d_status, void* stream) {
  if (n_seg < 0 || T < 0 || H <= 0 || d_cu == nullptr || d_status == nullptr) return PVB_E_INVALID_ARG;
  if (H_k <= 0 || H % H_k != 0) return PVB_E_INVALID_ARG;
  if (n_seg > PVB_MAX_COUNT) return PVB_E_OVERFLOW;
  if (T > 0 && (d_q == nullptr || d_k == nullptr || d_v == nullptr || d_g == nullptr || d_beta == nullptr ||
                d_o == nullptr))
    return PVB_E_INVALID_ARG;
  if (o_dtype != PVB_BF16 && o_dtype != PVB_F32) return PVB_E_INVALID_ARG;
  if (!(scale > 0.f) || !(scale < INFINITY)) return PVB_E_INVALID_ARG;
  if (d != kGdD) return PVB_E_UNSUPPORTED;
  const GdFwdLayout lay = gd_fwd_layout(T, H, n_seg);
  if ((int64_t)T * H * d >= ((int64_t)1 << 31) || !grid_fits(4 * (uint64_t)n_seg * H, kGdThreads) ||
      !grid_fits((uint64_t)lay.slots * H, kGdThreads) || !grid_fits(2 * (uint64_t)lay.gslots * H, kGdThreads))
    return PVB_E_UNSUPPORTED;
  const bool grouped = workspace != nullptr || workspace_bytes != 0;
  if (grouped && (workspace == nullptr || workspace_bytes < lay.total)) return PVB_E_WORKSPACE;
  const pvb_status hs = check_host_cu(h_cu, n_seg, T);
  if (hs != PVB_OK) return hs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!grouped) {
    // one chain per (slice, head); with no slice, one workgroup still checks
    // cu_seqlens and writes the status
    const unsigned grid = (unsigned)std::max<int64_t>(1, (int64_t)n_seg * H);
    if (o_dtype == PVB_F32)
      gated_delta_kernel<float><<<grid, kGdThreads, 0, s>>>(
          (const bf16*)d_q, (const bf16*)d_k, (const bf16*)d_v, d_g, d_beta, d_cu, n_seg, T, H, H_k, scale, d_h0,
          (float*)d_o, d_ht, d_status);
    else
      gated_delta_kernel<bf16><<<grid, kGdThreads, 0, s>>>(
          (const bf16*)d_q, (const bf16*)d_k, (const bf16*)d_v, d_g, d_beta, d_cu, n_seg, T, H, H_k, scale, d_h0,
          (bf16*)d_o, d_ht, d_status);
    return hipGetLastError() == hipSuccess ? PVB_OK : PVB_E_HIP;
  }
  char* ws = static_cast<char*>(workspace);
  float* ck_t = reinterpret_cast<float*>(ws + lay.ck_t);
  float* gA = reinterpret_cast<float*>(ws + lay.gA);
  float* gZ = reinterpret_cast<float*>(ws + lay.gZ);
  float* gS = reinterpret_cast<float*>(ws + lay.gS);
  // pass 0: T of every chunk; passes 1 and 2 only when a slice spans more than
  // one group (known without the host mirror only on the device)
  bool multi = true;
  if (h_cu != nullptr) {
    multi = false;
    for (int32_t b = 0; b < n_seg && !multi; ++b) multi = h_cu[b + 1] - h_cu[b] > kGdGrpTok;
  }
  const GdTmatLaunch tl = gd_tmat_launch(lay.slots, H);
  gd_tmat_kernel<false><<<tl.grid, 64, 0, s>>>((const bf16*)d_k, d_g, d_beta, d_cu, n_seg, T, H, H_k, ck_t,
                                               tl.per);
  if (multi) {
    gd_grp_compose_kernel<false><<<(unsigned)(2 * lay.gslots * H), kGdThreads, 0, s>>>(
        (const bf16*)d_k, (const bf16*)d_v, d_g, d_beta, d_cu, n_seg, T, H, H_k, ck_t, gA, gZ,
        (int)(lay.gslots * H));
    gd_grp_scan_kernel<false><<<(unsigned)std::max<int64_t>(1, 4 * (int64_t)n_seg * H), kGdThreads, 0, s>>>(
        d_cu, n_seg, T, H, d_h0, gA, gZ, gS);
  }
  if (o_dtype == PVB_F32)
    gd_fwd_grouped_kernel<float><<<(unsigned)(lay.gslots * H), kGdThreads, 0, s>>>(
        (const bf16*)d_q, (const bf16*)d_k, (const bf16*)d_v, d_g, d_beta, d_cu, n_seg, T, H, H_k, scale, d_h0,
        (float*)d_o, d_ht, d_status, ck_t, gS);
  else
    gd_fwd_grouped_kernel<bf16><<<(unsigned)(lay.gslots * H), kGdThreads, 0, s>>>(
        (const bf16*)d_q, (const bf16*)d_k, (const bf16*)d_v, d_g, d_beta, d_cu, n_seg, T, H, H_k, scale, d_h0,
        (bf16*)d_o, d_ht, d_status, ck_t, gS);
  return hipGetLastError() == hipSuccess ? PVB_OK : PVB_E_HIP;
}

// The training forward: the grouped forward on the backward's workspace, which
// it leaves holding T and T^T of every chunk, every chunk's starting state and
// U, and the group maps, so that the backward can skip their recomputation.
pvb_status gated_delta_train_call(const void* d_q, const void* d_k, const void* d_v, const float* d_g,
                                  const float* d_beta, const int32_t* d_cu, const int32_t* h_cu, int32_t n_seg,
                                  int32_t T, int32_t H, int32_t H_k, int32_t d, float scale, const float* d_h0,
                                  void* d_o, int32_t o_dtype, float* d_ht, void* workspace, size_t workspace_bytes,
                                  int32_t* d_status, void* stream) {
  if (n_seg < 0 || T < 0 || H <= 0 || d_cu == nullptr || d_status == nullptr) return PVB_E_INVALID_ARG;
  if (H_k <= 0 || H % H_k != 0) return PVB_E_INVALID_ARG;
  if (n_seg > PVB_MAX_COUNT) return PVB_E_OVERFLOW;
  if (T > 0 && (d_q == nullptr || d_k == nullptr || d_v == nullptr || d_g == nullptr || d_beta == nullptr ||
                d_o == nullptr))
    return PVB_E_INVALID_ARG;
  if (o_dtype != PVB_BF16 && o_dtype != PVB_F32) return PVB_E_INVALID_ARG;
  if (!(scale > 0.f) || !(scale < INFINITY)) return PVB_E_INVALID_ARG;
  if (d != kGdD) return PVB_E_UNSUPPORTED;
  const GdBwdLayout lay = gd_bwd_layout(T, H, n_seg);
  if ((int64_t)T * H * d >= ((int64_t)1 << 31) || !grid_fits((uint64_t)4 * n_seg * H, kGdThreads) ||
      !grid_fits((uint64_t)lay.slots * H, kGdChunkThreads) || !grid_fits((uint64_t)2 * lay.gslots * H, kGdThreads))
    return PVB_E_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < lay.total) return PVB_E_WORKSPACE;
  const pvb_status hs = check_host_cu(h_cu, n_seg, T);
  if (hs != PVB_OK) return hs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* ck_s = reinterpret_cast<float*>(ws + lay.ck_s);
  float* ck_u = reinterpret_cast<float*>(ws + lay.ck_u);
  float* ck_t = reinterpret_cast<float*>(ws + lay.ck_t);
  float* gA = reinterpret_cast<float*>(ws + lay.gA);
  float* gZ = reinterpret_cast<float*>(ws + lay.gZ);
  float* gS = reinterpret_cast<float*>(ws + lay.gS);
  bool multi = true;
  if (h_cu != nullptr) {
    multi = false;
    for (int32_t b = 0; b < n_seg && !multi; ++b) multi = h_cu[b + 1] - h_cu[b] > kGdGrpTok;
  }
  const GdTmatLaunch tl = gd_tmat_launch(lay.slots, H);
  gd_tmat_kernel<true><<<tl.grid, 64, 0, s>>>((const bf16*)d_k, d_g, d_beta, d_cu, n_seg, T, H, H_k, ck_t, tl.per);
  const unsigned ggrid = (unsigned)std::max<size_t>(1, lay.gslots * H);
  if (multi) {
    // the maps of every group, the last's too (the backward's transposed scan
    // reads them all)
    gd_grp_compose_kernel<true><<<2 * ggrid, kGdThreads, 0, s>>>(
        (const bf16*)d_k, (const bf16*)d_v, d_g, d_beta, d_cu, n_seg, T, H, H_k, ck_t, gA, gZ, (int)ggrid);
    gd_grp_scan_kernel<false><<<(unsigned)std::max<int64_t>(1, 4 * (int64_t)n_seg * H), kGdThreads, 0, s>>>(
        d_cu, n_seg, T, H, d_h0, gA, gZ, gS);
  }
  if (o_dtype == PVB_F32)
    gd_fwd_train_kernel<float><<<ggrid, kGdThreads, 0, s>>>(
        (const bf16*)d_q, (const bf16*)d_k, (const bf16*)d_v, d_g, d_beta, d_cu, n_seg, T, H, H_k, scale, d_h0,
        (float*)d_o, d_ht, d_status, ck_t, ck_s, ck_u, gS);
  else
    gd_fwd_train_kernel<bf16><<<ggrid, kGdThreads, 0, s>>>(
        (const bf16*)d_q, (const bf16*)d_k, (const bf16*)d_v, d_g, d_beta, d_cu, n_seg, T, H, H_k, scale, d_h0,
        (bf16*)d_o, d_ht, d_status, ck_t, ck_s, ck_u, gS);
  return hipGetLastError() == hipSuccess ? PVB_OK : PVB_E_HIP;
}
}  // namespace
}  // namespace pvb

extern "C" size_t pvb_gated_delta_fwd_workspace_bytes(int32_t T, int32_t H, int32_t n_seg) {
  if (T < 0 || H <= 0 || n_seg < 0) return 0;
  return pvb::gd_fwd_layout(T, H, n_seg).total;
}

extern "C" pvb_status pvb_gated_delta_fwd(const void* d_q, const void* d_k, const void* d_v, const float* d_g,
                                          const float* d_beta, const int32_t* d_cu, const int32_t* h_cu,
                                          int32_t n_seg, int32_t T, int32_t H, int32_t d, float scale,
                                          const float* d_h0, void* d_o, int32_t o_dtype, float* d_ht,
                                          void* workspace, size_t workspace_bytes, int32_t* d_status,
                                          void* stream) {
  return pvb::gated_delta_call(d_q, d_k, d_v, d_g, d_beta, d_cu, h_cu, n_seg, T, H, H, d, scale, d_h0, d_o,
                               o_dtype, d_ht, workspace, workspace_bytes, d_status, stream);
}

extern "C" pvb_status pvb_gated_delta_fwd_gqa(const void* d_q, const void* d_k, const void* d_v,
                                              const float* d_g, const float* d_beta, const int32_t* d_cu,
                                              const int32_t* h_cu, int32_t n_seg, int32_t T, int32_t H,
                                              int32_t H_k, int32_t d, float scale, const float* d_h0,
                                              void* d_o, int32_t o_dtype, float* d_ht, void* workspace,
                                              size_t workspace_bytes, int32_t* d_status, void* stream) {
  return pvb::gated_delta_call(d_q, d_k, d_v, d_g, d_beta, d_cu, h_cu, n_seg, T, H, H_k, d, scale, d_h0, d_o,
                               o_dtype, d_ht, workspace, workspace_bytes, d_status, stream);
}

extern "C" pvb_status pvb_gated_delta_fwd_train(const void* d_q, const void* d_k, const void* d_v,
                                                const float* d_g, const float* d_beta, const int32_t* d_cu,
                                                const int32_t* h_cu, int32_t n_seg, int32_t T, int32_t H,
                                                int32_t H_k, int32_t d, float scale, const float* d_h0, void* d_o,
                                                int32_t o_dtype, float* d_ht, void* workspace,
                                                size_t workspace_bytes, int32_t* d_status, void* stream) {
  return pvb::gated_delta_train_call(d_q, d_k, d_v, d_g, d_beta, d_cu, h_cu, n_seg, T, H, H_k, d, scale, d_h0, d_o,
                                     o_dtype, d_ht, workspace, workspace_bytes, d_status, stream);
}
