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
// P, U, the gated keys, A's off-diagonal block) is split into bf16 hi + lo
// parts, so the products keep about 16 significant bits; the two 32-row
// triangles of the solve are fp32 on the vector unit.
//
// One workgroup of 4 waves per (slice, value head); the slices are
// independent.  Value head h reads query/key head h / (H / H_k).  Wave w owns
// value columns [32w, 32w + 32) of the state, which stays in its registers (C
// layout of four 32x32 blocks) across the chunks of the slice.
#include <type_traits>

#include "pvb_device.hpp"

namespace pvb {
namespace {

constexpr int kGdD = 128;            // d_k = d_v
constexpr int kGdC = 64;             // chunk length
constexpr int kGdThreads = 256;
constexpr int kKP = kGdD + 8;        // bf16 row pitch of the Q, K, V tiles
constexpr int kFP = kGdC + 4;        // fp32 row pitch of A^T and P

struct GdSmem {
  alignas(16) bf16 q[kGdC][kKP];
  alignas(16) bf16 k[kGdC][kKP];
  alignas(16) bf16 v[kGdC][kKP];
  alignas(16) float at[kGdC][kFP];   // A^T: at[j][i] = A[i][j]
  alignas(16) float p[kGdC][kFP];    // P (row i, column j)
  // A operands shared by the four waves, split once per chunk, in fragment
  // order [..][lane]: the gated keys for the state update (key-dim block r,
  // position step s) and P (row block rb, position step s; rb = 0 stops at
  // s = 2).  Positions inside a step are in the order of the C layout's rows.
  alignas(16) bf16x8 kth[4][4][64], ktl[4][4][64];
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
template <typename OutT, bool CKPT = false>
__global__ void __launch_bounds__(kGdThreads, 1)
gated_delta_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                   const float* __restrict__ g, const float* __restrict__ beta,
                   const int32_t* __restrict__ cu, int n_seg, int T, int H, int Hk, float scale,
                   const float* __restrict__ h0, OutT* __restrict__ o, float* __restrict__ ht,
                   int32_t* __restrict__ status, float* __restrict__ ck_s = nullptr,
                   float* __restrict__ ck_u = nullptr) {
  __shared__ GdSmem sm;
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, hg = lane >> 5, c = lane & 31;

  // every workgroup checks the whole cu_seqlens before it writes anything
  if (tid == 0) s_bad = 0;
  __syncthreads();
  for (int b = tid; b < n_seg; b += kGdThreads)
    if (cu[b + 1] < cu[b]) atomicOr(&s_bad, 1);
  if (tid == 0 && (cu[0] != 0 || cu[n_seg] != T)) atomicOr(&s_bad, 1);
  __syncthreads();
  if (blockIdx.x == 0 && tid == 0) *status = s_bad ? PVB_E_BAD_CU_SEQLENS : PVB_OK;
  if (s_bad || (int)blockIdx.x >= n_seg * H) return;

  const int b = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  const int hk = h / (H / Hk);                        // the query/key head of value head h
  const int seg0 = cu[b], L = cu[b + 1] - seg0;
  const int n0 = 32 * w + c;                          // this lane's value column
  const size_t st_base = (size_t)(b * H + h) * kGdD * kGdD;

  // the state, rows (key dims) 32r + crow(i, hg), column n0
  f32x16 S[4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      S[r][i] = h0 ? h0[st_base + (size_t)(32 * r + crow(i, hg)) * kGdD + n0] : 0.f;

  // The inputs of chunk c + 1 are loaded into registers while chunk c is
  // computed (and before its outputs are stored, so that waiting for them
  // never waits for those stores).
  uint4 pq[4], pk[4], pv[4];
  float pg = 0.f, pb = 0.f;
  auto fetch = [&](int cc0) {
    const int nvv = min(kGdC, L - cc0);
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
  if (L > 0) fetch(0);

  for (int c0 = 0; c0 < L; c0 += kGdC) {
    const int nv = min(kGdC, L - c0);
    const size_t slot = gd_ckpt_slot(seg0, b, c0 / kGdC);
    if constexpr (CKPT) {
      float* cs = ck_s + (slot * H + h) * kGdD * kGdD;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) cs[(size_t)(32 * r + crow(i, hg)) * kGdD + n0] = S[r][i];
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
    if (c0 + kGdC < L) fetch(c0 + kGdC);
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
    if constexpr (CKPT) {                             // P only feeds O
      if (w == 0) block(KK{}, 1, 0);
      else if (w == 1) block(KK{}, 0, 0);
      else if (w == 2) block(KK{}, 1, 1);
    } else {
      if (w == 0) { block(KK{}, 1, 0); block(QK{}, 0, 0); }
      else if (w == 1) { block(QK{}, 1, 0); block(KK{}, 0, 0); }
      else if (w == 2) block(KK{}, 1, 1);
      else block(QK{}, 1, 1);
    }

    // ---- the gated keys (diag(G_63 / G) K)^T as split A fragments, once for
    // the four waves: fragment f = (r, s, lane) of a thread
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int f = tid + kGdThreads * it;
      const int r = f >> 8, s = (f >> 6) & 3, fl = f & 63, fc = fl & 31, fh = fl >> 5;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int pos = kpos(s, e, fh);
        x[e] = (float)sm.k[pos][32 * r + fc] * sm.dec[pos];
      }
      split8(x, sm.kth[r][s][fl], sm.ktl[r][s][fl]);
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
        if constexpr (!CKPT) {
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
    for (int f = tid; f < (CKPT ? 0 : 6 * 64); f += kGdThreads) {
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
    if constexpr (CKPT) {
      float* cuu = ck_u + (slot * H + h) * kGdC * kGdD;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int pos = 32 * rb + crow(i, hg);
          if (pos < nv) cuu[(size_t)pos * kGdD + n0] = ks[rb][i];
        }
    }
    __syncthreads();                                  // the P and key fragments are complete

    // ---- O = scale (diag(G) Q S0 + P U) (row block 0 has no key past 31)
    // and S = G_63 S0 + (diag(G_63 / G) K)^T U: the matrix-core work of both
    // is issued first, then O is staged in the Q/K tiles (free by now) and
    // written with 16-byte stores.
    if constexpr (!CKPT) {
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
    const float glast = sm.eg[kGdC - 1];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int i = 0; i < 16; ++i) S[r][i] *= glast;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 a_hi = sm.kth[r][s][lane], a_lo = sm.ktl[r][s][lane];
        S[r] = mfma32(a_hi, uh[s], S[r]);
        S[r] = mfma32(a_hi, ul[s], S[r]);
        S[r] = mfma32(a_lo, uh[s], S[r]);
      }
    }
    if constexpr (CKPT) continue;                     // no O in the recomputation pass
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

  if (!CKPT && ht) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) ht[st_base + (size_t)(32 * r + crow(i, hg)) * kGdD + n0] = S[r][i];
  }
}

}  // namespace
}  // namespace pvb

namespace pvb {
namespace {
pvb_status gated_delta_call(const void* d_q, const void* d_k, const void* d_v, const float* d_g,
                            const float* d_beta, const int32_t* d_cu, const int32_t* h_cu, int32_t n_seg,
                            int32_t T, int32_t H, int32_t H_k, int32_t d, float scale, const float* d_h0,
                            void* d_o, int32_t o_dtype, float* d_ht, int32_t* d_status, void* stream) {
  if (n_seg < 0 || T < 0 || H <= 0 || d_cu == nullptr || d_status == nullptr) return PVB_E_INVALID_ARG;
  if (H_k <= 0 || H % H_k != 0) return PVB_E_INVALID_ARG;
  if (n_seg > PVB_MAX_COUNT) return PVB_E_OVERFLOW;
  if (T > 0 && (d_q == nullptr || d_k == nullptr || d_v == nullptr || d_g == nullptr || d_beta == nullptr ||
                d_o == nullptr))
    return PVB_E_INVALID_ARG;
  if (o_dtype != PVB_BF16 && o_dtype != PVB_F32) return PVB_E_INVALID_ARG;
  if (!(scale > 0.f) || !(scale < INFINITY)) return PVB_E_INVALID_ARG;
  if (d != kGdD) return PVB_E_UNSUPPORTED;
  if ((int64_t)T * H * d >= ((int64_t)1 << 31) || !grid_fits((uint64_t)n_seg * H, kGdThreads))
    return PVB_E_UNSUPPORTED;
  const pvb_status hs = check_host_cu(h_cu, n_seg, T);
  if (hs != PVB_OK) return hs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // one workgroup per (slice, head); with no slice, one workgroup still checks
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
}  // namespace
}  // namespace pvb

extern "C" pvb_status pvb_gated_delta_fwd(const void* d_q, const void* d_k, const void* d_v, const float* d_g,
                                          const float* d_beta, const int32_t* d_cu, const int32_t* h_cu,
                                          int32_t n_seg, int32_t T, int32_t H, int32_t d, float scale,
                                          const float* d_h0, void* d_o, int32_t o_dtype, float* d_ht,
                                          int32_t* d_status, void* stream) {
  return pvb::gated_delta_call(d_q, d_k, d_v, d_g, d_beta, d_cu, h_cu, n_seg, T, H, H, d, scale, d_h0, d_o,
                               o_dtype, d_ht, d_status, stream);
}

extern "C" pvb_status pvb_gated_delta_fwd_gqa(const void* d_q, const void* d_k, const void* d_v,
                                              const float* d_g, const float* d_beta, const int32_t* d_cu,
                                              const int32_t* h_cu, int32_t n_seg, int32_t T, int32_t H,
                                              int32_t H_k, int32_t d, float scale, const float* d_h0,
                                              void* d_o, int32_t o_dtype, float* d_ht, int32_t* d_status,
                                              void* stream) {
  return pvb::gated_delta_call(d_q, d_k, d_v, d_g, d_beta, d_cu, h_cu, n_seg, T, H, H_k, d, scale, d_h0, d_o,
                               o_dtype, d_ht, d_status, stream);
}

namespace pvb {
namespace {

// ===========================================================================
// Backward of the gated delta rule over the packed stream.
//
// The gradients of  sum_t o_t . dO_t + <S_final, dS_final>  with respect to
// q, k, v, g, beta and the initial states, slice by slice (nothing crosses a
// boundary), by reverse-mode differentiation of the chunked form above.  A
// recomputation pass (gated_delta_kernel in CKPT mode) stores each chunk's
// starting state S0 and its U; the backward then walks the chunks of every
// (slice, value head) from the last to the first, carrying dS, the gradient
// with respect to the state at the chunk's end.  With n positions in the
// chunk, gamma the chunk-local cumulative gate, G = exp(gamma), G_L its last
// value, Gam_ij = G_i / G_j, Ah = strict_lower(Gam o K K^T) (so A = diag(beta)
// Ah), P = lower(Gam o Q K^T), X = V - diag(G) K S0 and Kt = diag(G_L / G) K:
//   dU  = scale P^T dO + Kt dS               dR = (I + A)^-T dU
//   dV  = diag(beta) dR                      dKS = -diag(G) dV
//   dA  = -strict_lower(dR U^T)              dP = scale lower(dO U^T)
//   dKt = U dS^T
//   dbeta_i = sum_c dR_ic X_ic + sum_j dA_ij Ah_ij
//   dG_i = -sum_c dV_ic (K S0)_ic + scale sum_c dO_ic (Q S0)_ic
//   M = diag(beta) (Gam o dA),  N = Gam o dP
//   dK = dKS S0^T + N^T Q + M K + M^T K + diag(G_L / G) dKt
//   dQ = scale diag(G) dO S0^T + N K
//   dgamma = rowsum(dP o P) - colsum(dP o P) + rowsum(dA o A) - colsum(dA o A)
//            + G o dG - rowsum(dKt o Kt);  dgamma_last += sum(dKt o Kt) + G_L <dS, S0>
//   dg_t = sum_{i >= t} dgamma_i;   dS (for the previous chunk) = K^T dKS + scale Q^T diag(G) dO + G_L dS
// Every product runs on the matrix cores as 32x32 blocks (gd_block_product),
// fp32 operands split into bf16 hi + lo; the chunk's matrices live in a
// per-workgroup global scratch (and Ah, P, M, N in LDS), one wave per output
// block.  dQ and dK of a query/key head shared by several value heads are
// summed with fp32 atomic adds into buffers cleared first.

// Read-only matrix views: element (r, c) at p[r * rs + c * cs], zero outside
// [0, nr) x [0, nc).  FView is fp32 (split into two bf16 parts for the matrix
// cores), HView bf16 (taken as it is), HSView bf16 times a per-row scale.
struct FView {
  const float* p;
  int64_t rs;
  int64_t cs;
  int nr, nc;
  __device__ __forceinline__ float get(int r, int c) const {
    return (r < nr && c < nc) ? p[r * rs + c * cs] : 0.f;
  }
};
struct HView {
  const bf16* p;
  int64_t rs;
  int64_t cs;
  int nr, nc;
  __device__ __forceinline__ float get(int r, int c) const {
    return (r < nr && c < nc) ? (float)p[r * rs + c * cs] : 0.f;
  }
};
struct HSView {
  const bf16* p;
  int64_t rs;
  int64_t cs;
  int nr, nc;
  const float* rsc;
  __device__ __forceinline__ float get(int r, int c) const {
    return (r < nr && c < nc) ? rsc[r] * (float)p[r * rs + c * cs] : 0.f;
  }
};
template <typename V>
struct exact_bf16 : std::false_type {};
template <>
struct exact_bf16<HView> : std::true_type {};

// acc += the 32x32 block (m0, n0) of A B over k < K (a multiple of 16): lane
// l holds A[m0 + l%32][k0 + 8(l/32) + e] and B[k0 + 8(l/32) + e][n0 + l%32];
// result element i of lane l is row m0 + crow(i, l/32), column n0 + l%32.
template <int K, typename VA, typename VB>
__device__ __forceinline__ f32x16 gd_block_product(const VA& a, const VB& b, int m0, int n0, f32x16 acc) {
  const int lane = threadIdx.x & 63, c = lane & 31, hg = lane >> 5;
#pragma unroll 2
  for (int k0 = 0; k0 < K; k0 += 16) {
    float xa[8], xb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      xa[e] = a.get(m0 + c, k0 + 8 * hg + e);
      xb[e] = b.get(k0 + 8 * hg + e, n0 + c);
    }
    bf16x8 ah, al, bh, bl;
    split8(xa, ah, al);
    split8(xb, bh, bl);
    acc = mfma32(ah, bh, acc);
    if constexpr (!exact_bf16<VB>::value) acc = mfma32(ah, bl, acc);
    if constexpr (!exact_bf16<VA>::value) acc = mfma32(al, bh, acc);
  }
  return acc;
}

constexpr int kGdBwdScratch = kGdD * kGdD + 6 * kGdC * kGdD + 2 * kGdC * kGdC;   // floats per workgroup
constexpr int kLP = kGdC + 1;                                                   // LDS row pitch

struct GdBwdSmem {
  float ah[kGdC][kLP];     // Ah (then M)
  float p[kGdC][kLP];      // P (then N)
  float gl[kGdC], eg[kGdC], dec[kGdC], beta[kGdC];
  float dbeta[kGdC], dG[kGdC], dgam[kGdC];
  float red[kGdThreads / 64];
};

template <typename GradT>
__global__ void __launch_bounds__(kGdThreads, 1)
gated_delta_bwd_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                       const float* __restrict__ g, const float* __restrict__ beta,
                       const int32_t* __restrict__ cu, int n_seg, int T, int H, int Hk, float scale,
                       const bf16* __restrict__ dout, const float* __restrict__ dht,
                       const float* __restrict__ ck_s, const float* __restrict__ ck_u, float* __restrict__ scratch,
                       float* __restrict__ dq, float* __restrict__ dk, GradT* __restrict__ dv,
                       float* __restrict__ dg, float* __restrict__ dbeta, float* __restrict__ dh0, bool atomic_qk) {
  __shared__ GdBwdSmem sm;
  __shared__ int s_bad;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, hg = lane >> 5, c = lane & 31;

  // the recomputation pass reported a bad cu_seqlens; every workgroup checks
  // it again before it writes anything
  if (tid == 0) s_bad = 0;
  __syncthreads();
  for (int b = tid; b < n_seg; b += kGdThreads)
    if (cu[b + 1] < cu[b]) atomicOr(&s_bad, 1);
  if (tid == 0 && (cu[0] != 0 || cu[n_seg] != T)) atomicOr(&s_bad, 1);
  __syncthreads();
  if (s_bad || (int)blockIdx.x >= n_seg * H) return;

  const int b = blockIdx.x / H, h = blockIdx.x - (blockIdx.x / H) * H;
  const int hk = h / (H / Hk);
  const int seg0 = cu[b], L = cu[b + 1] - seg0;
  float* sc = scratch + (size_t)blockIdx.x * kGdBwdScratch;
  float* s_dS = sc;                                   // [128][128] gradient of the chunk's end state
  float* s_KS = s_dS + kGdD * kGdD;                   // [64][128] K S0
  float* s_QS = s_KS + kGdC * kGdD;                   // [64][128] Q S0
  float* s_X = s_QS + kGdC * kGdD;                    // [64][128] V - diag(G) K S0
  float* s_dR = s_X + kGdC * kGdD;                    // [64][128] dU, solved in place into dR
  float* s_dKS = s_dR + kGdC * kGdD;                  // [64][128] -diag(G beta) dR
  float* s_dKt = s_dKS + kGdC * kGdD;                 // [64][128] U dS^T
  float* s_dA = s_dKt + kGdC * kGdD;                  // [64][64]
  float* s_dP = s_dA + kGdC * kGdC;                   // [64][64]

  const size_t st_base = (size_t)(b * H + h) * kGdD * kGdD;
  for (int e = tid; e < kGdD * kGdD; e += kGdThreads) s_dS[e] = dht ? dht[st_base + e] : 0.f;

  const int n_chunks = (L + kGdC - 1) / kGdC;
  for (int ci = n_chunks - 1; ci >= 0; --ci) {
    const int t0 = seg0 + ci * kGdC;
    const int n = min(kGdC, L - ci * kGdC);
    const size_t slot = gd_ckpt_slot(seg0, b, ci);
    const float* S0p = ck_s + (slot * H + h) * kGdD * kGdD;
    const float* Up = ck_u + (slot * H + h) * kGdC * kGdD;
    const HView Qv{q + ((size_t)t0 * Hk + hk) * kGdD, (int64_t)Hk * kGdD, 1, n, kGdD};
    const HView Kv{k + ((size_t)t0 * Hk + hk) * kGdD, (int64_t)Hk * kGdD, 1, n, kGdD};
    const HView KTv{Kv.p, 1, (int64_t)Hk * kGdD, kGdD, n};            // K^T [dk][pos]
    const HView QTv{Qv.p, 1, (int64_t)Hk * kGdD, kGdD, n};
    const bf16* Vp = v + ((size_t)t0 * H + h) * kGdD;
    const bf16* dOp = dout + ((size_t)t0 * H + h) * kGdD;
    const HView dOv{dOp, (int64_t)H * kGdD, 1, n, kGdD};
    const FView S0v{S0p, kGdD, 1, kGdD, kGdD};                          // [dk][col]
    const FView S0Tv{S0p, 1, kGdD, kGdD, kGdD};                         // [col][dk]
    const FView Uv{Up, kGdD, 1, n, kGdD};                               // [pos][col]
    const FView UTv{Up, 1, kGdD, kGdD, n};                              // [col][pos]
    const FView dSv{s_dS, kGdD, 1, kGdD, kGdD};
    const FView dSTv{s_dS, 1, kGdD, kGdD, kGdD};

    __syncthreads();                                  // the previous chunk is done with LDS and scratch
    // ---- gates (log2 units), chunk-local
    if (w == 0) {
      float x = lane < n ? g[(size_t)(t0 + lane) * H + h] : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      x *= kLog2e;
      const float last = __shfl(x, n - 1, 64);
      sm.gl[lane] = x;
      sm.eg[lane] = fast_exp2(x);
      sm.dec[lane] = fast_exp2(last - x);
      sm.beta[lane] = lane < n ? beta[(size_t)(t0 + lane) * H + h] : 0.f;
    }
    __syncthreads();

    // ---- Ah, P (LDS) and K S0, Q S0 (scratch): 8 + 16 block jobs
    for (int job = w; job < 24; job += 4) {
      if (job < 8) {
        const bool isq = job >= 4;
        const int jb = job & 3;                       // blocks (0,0), (1,0), (1,1), (0,1)
        const int bi = jb == 0 ? 0 : (jb == 3 ? 0 : 1), bj = jb == 1 ? 0 : (jb == 3 ? 1 : bi);
        float (*dst)[kLP] = isq ? sm.p : sm.ah;
        f32x16 acc = {};
        if (jb != 3) acc = isq ? gd_block_product<kGdD>(Qv, KTv, 32 * bi, 32 * bj, acc)
                               : gd_block_product<kGdD>(Kv, KTv, 32 * bi, 32 * bj, acc);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 32 * bi + crow(i, hg), cc = 32 * bj + c;
          const float gam = fast_exp2(fminf(sm.gl[r] - sm.gl[cc], 0.f));
          const bool keep = isq ? cc <= r : cc < r;
          dst[r][cc] = (jb != 3 && keep) ? gam * acc[i] : 0.f;
        }
      } else {
        const int jj = job - 8, isq = jj >= 8, blk = jj & 7, rb = blk >> 2, cb = blk & 3;
        f32x16 acc = {};
        acc = isq ? gd_block_product<kGdD>(Qv, S0v, 32 * rb, 32 * cb, acc)
                  : gd_block_product<kGdD>(Kv, S0v, 32 * rb, 32 * cb, acc);
        float* dst = isq ? s_QS : s_KS;
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[(32 * rb + crow(i, hg)) * kGdD + 32 * cb + c] = acc[i];
      }
    }
    __syncthreads();

    // ---- X = V - diag(G) K S0 and dU = scale P^T dO + diag(G_L / G) K dS
    {
      const int r = tid >> 2, c0 = (tid & 3) * 32;
      for (int cc = c0; cc < c0 + 32; ++cc)
        s_X[r * kGdD + cc] = r < n ? (float)Vp[(size_t)r * H * kGdD + cc] - sm.eg[r] * s_KS[r * kGdD + cc] : 0.f;
    }
    // dU in registers: wave w holds the two 32-row blocks of its 32 columns in
    // the C layout (rows 32 rb + crow(i, hg), column 32 w + c)
    f32x16 du[2];
    {
      const FView PTv{&sm.p[0][0], 1, kLP, kGdC, kGdC};                 // P^T
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        f32x16 a1 = {}, a2 = {};
        a1 = gd_block_product<kGdC>(PTv, dOv, 32 * rb, 32 * w, a1);
        a2 = gd_block_product<kGdD>(Kv, dSv, 32 * rb, 32 * w, a2);
#pragma unroll
        for (int i = 0; i < 16; ++i) du[rb][i] = scale * a1[i] + sm.dec[32 * rb + crow(i, hg)] * a2[i];
      }
    }

    // ---- dR = (I + A)^-T dU, A = diag(beta) Ah, in the C layout, blocked by
    // 32 rows from the bottom: the lower block's triangle, the upper block's
    // update by the matrix cores, the upper block's triangle.  Inside a block,
    // row jj is final when reached from the block's end; the lane holding it
    // hands it across the half-waves and every row above it subtracts A_(jj, row)
    // times it.
    auto triangle_t = [&](auto rb_tag) {
      constexpr int RB = decltype(rb_tag)::value;
#pragma unroll
      for (int jj = 31; jj > 0; --jj) {
        const int ij = 4 * (jj >> 3) + (jj & 3);    // element index of row jj
        const bool own = ((jj >> 2) & 1) == hg;
        const float x = du[RB][ij];
        const float other = swap_halves(x);
        const float rj = (own ? x : other) * sm.beta[32 * RB + jj];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if (8 * m >= jj) continue;                  // every row of the group is at or below jj
          const float4 a4 = *(const float4*)&sm.ah[32 * RB + jj][32 * RB + 8 * m + 4 * hg];
          const int r0 = 8 * m + 4 * hg;
          if (r0 + 0 < jj) du[RB][4 * m + 0] -= a4.x * rj;
          if (r0 + 1 < jj) du[RB][4 * m + 1] -= a4.y * rj;
          if (r0 + 2 < jj) du[RB][4 * m + 2] -= a4.z * rj;
          if (r0 + 3 < jj) du[RB][4 * m + 3] -= a4.w * rj;
        }
      }
    };
    triangle_t(std::integral_constant<int, 1>{});
    {
      // upper rows i: dU_i -= sum_{j in the lower block} A_ji dR_j; the lower
      // block is the B operand straight from its C layout (k-step s: elements
      // 8s + e, rows 32 + kpos(s, e, hg)), A_ji read in that order
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        float xa[8], xb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = 32 + kpos(s2, e, hg);
          xa[e] = -sm.beta[j] * sm.ah[j][c];
          xb[e] = du[1][8 * s2 + e];
        }
        bf16x8 ah, al, bh, bl;
        split8(xa, ah, al);
        split8(xb, bh, bl);
        du[0] = mfma32(ah, bh, du[0]);
        du[0] = mfma32(ah, bl, du[0]);
        du[0] = mfma32(al, bh, du[0]);
      }
    }
    triangle_t(std::integral_constant<int, 0>{});
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s_dR[(32 * rb + crow(i, hg)) * kGdD + 32 * w + c] = du[rb][i];
    __syncthreads();

    // ---- dV = diag(beta) dR (stored), dKS = -diag(G) dV, and the per-row sums
    // of dbeta (through X) and dG
    {
      const int r = tid >> 2, c0 = (tid & 3) * 32;
      const float br = sm.beta[r], gr = sm.eg[r];
      float sR = 0.f, sG = 0.f;
      for (int cc = c0; cc < c0 + 32; ++cc) {
        const int e = r * kGdD + cc;
        const float dr = s_dR[e], dvv = br * dr;
        const float dov = r < n ? (float)dOp[(size_t)r * H * kGdD + cc] : 0.f;
        sR += dr * s_X[e];
        sG += -dvv * s_KS[e] + scale * dov * s_QS[e];
        s_dKS[e] = -gr * dvv;
        if (r < n) dv[((size_t)(t0 + r) * H + h) * kGdD + cc] = out_cast<GradT>(dvv);
      }
      sR += __shfl_xor(sR, 1, 64);
      sR += __shfl_xor(sR, 2, 64);
      sG += __shfl_xor(sG, 1, 64);
      sG += __shfl_xor(sG, 2, 64);
      if ((tid & 3) == 0) {
        sm.dbeta[r] = sR;
        sm.dG[r] = sG;
      }
    }
    // <dS, S0> over the whole state
    {
      float part = 0.f;
      for (int e = tid; e < kGdD * kGdD; e += kGdThreads) part += s_dS[e] * S0p[e];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off, 64);
      if (lane == 0) sm.red[w] = part;
    }
    __syncthreads();

    // ---- dKt = U dS^T, dA = -strict_lower(dR U^T), dP = scale lower(dO U^T)
    {
      const FView dRv{s_dR, kGdD, 1, kGdC, kGdD};
      for (int job = w; job < 16; job += 4) {
        if (job < 8) {
          const int rb = job >> 2, cb = job & 3;
          f32x16 acc = {};
          acc = gd_block_product<kGdD>(Uv, dSTv, 32 * rb, 32 * cb, acc);
#pragma unroll
          for (int i = 0; i < 16; ++i) s_dKt[(32 * rb + crow(i, hg)) * kGdD + 32 * cb + c] = acc[i];
        } else {
          const int jj = job - 8, isp = jj >= 4, jb = jj & 3;
          const int bi = jb == 0 ? 0 : (jb == 3 ? 0 : 1), bj = jb == 1 ? 0 : (jb == 3 ? 1 : bi);
          f32x16 acc = {};
          if (jb != 3) acc = isp ? gd_block_product<kGdD>(dOv, UTv, 32 * bi, 32 * bj, acc)
                                 : gd_block_product<kGdD>(dRv, UTv, 32 * bi, 32 * bj, acc);
          float* dst = isp ? s_dP : s_dA;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int r = 32 * bi + crow(i, hg), cc = 32 * bj + c;
            const bool keep = jb != 3 && (isp ? cc <= r : cc < r);
            dst[r * kGdC + cc] = keep ? (isp ? scale * acc[i] : -acc[i]) : 0.f;
          }
        }
      }
    }
    __syncthreads();

    // ---- the new dS = K^T dKS + scale Q^T diag(G) dO + G_L dS (its own block
    // of the old dS only), and the gate and write-strength gradients
    {
      const FView dKSv{s_dKS, kGdD, 1, kGdC, kGdD};
      const HSView GdOv{dOp, (int64_t)H * kGdD, 1, n, kGdD, sm.eg};
      const float gL = sm.eg[n - 1];
      for (int job = w; job < 16; job += 4) {
        const int rb = job >> 2, cb = job & 3;
        f32x16 a1 = {}, a2 = {};
        a1 = gd_block_product<kGdC>(KTv, dKSv, 32 * rb, 32 * cb, a1);
        a2 = gd_block_product<kGdC>(QTv, GdOv, 32 * rb, 32 * cb, a2);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int e = (32 * rb + crow(i, hg)) * kGdD + 32 * cb + c;
          s_dS[e] = a1[i] + scale * a2[i] + gL * s_dS[e];
        }
      }
    }
    if (tid < kGdC) {
      const int i = tid;
      const float bi = sm.beta[i];
      float rpa = 0.f, cpa = 0.f, rpp = 0.f, cpp = 0.f, dba = 0.f, kk = 0.f;
      for (int j = 0; j < kGdC; ++j) {
        const float a_ij = s_dA[i * kGdC + j] * sm.ah[i][j];            // dA_ij Ah_ij
        dba += a_ij;
        rpa += bi * a_ij;
        cpa += sm.beta[j] * s_dA[j * kGdC + i] * sm.ah[j][i];
        rpp += s_dP[i * kGdC + j] * sm.p[i][j];
        cpp += s_dP[j * kGdC + i] * sm.p[j][i];
      }
      if (i < n)
        for (int cc = 0; cc < kGdD; ++cc)
          kk += s_dKt[i * kGdD + cc] * sm.dec[i] * (float)k[((size_t)(t0 + i) * Hk + hk) * kGdD + cc];
      sm.dbeta[i] += dba;
      sm.dgam[i] = rpp - cpp + rpa - cpa + sm.eg[i] * sm.dG[i] - kk;
      // kk summed over all rows goes to the last position (with G_L <dS, S0>)
      float tot = kk;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off, 64);
      if (i == 0) sm.red[0] = tot + sm.eg[n - 1] * (sm.red[0] + sm.red[1] + sm.red[2] + sm.red[3]);
    }
    __syncthreads();
    if (tid < kGdC) {
      const int i = tid;
      if (i == n - 1) sm.dgam[i] += sm.red[0];
    }
    __syncthreads();
    if (tid < kGdC) {
      const int i = tid;
      // dg_i = sum over j >= i of dgamma_j (positions of this chunk only)
      float s = 0.f;
      for (int j = i; j < n; ++j) s += sm.dgam[j];
      if (i < n) {
        dg[(size_t)(t0 + i) * H + h] = s;
        dbeta[(size_t)(t0 + i) * H + h] = sm.dbeta[i];
      }
    }
    __syncthreads();
    // ---- M = diag(beta) (Gam o dA) and N = Gam o dP into the LDS of Ah and P
    for (int e = tid; e < kGdC * kGdC; e += kGdThreads) {
      const int i = e / kGdC, j = e - (e / kGdC) * kGdC;
      const float gam = fast_exp2(fminf(sm.gl[i] - sm.gl[j], 0.f));
      sm.ah[i][j] = sm.beta[i] * gam * s_dA[e];
      sm.p[i][j] = gam * s_dP[e];
    }
    __syncthreads();

    // ---- dK = dKS S0^T + N^T Q + M K + M^T K + diag(G_L / G) dKt and
    // dQ = scale diag(G) dO S0^T + N K
    {
      const FView dKSv{s_dKS, kGdD, 1, kGdC, kGdD};
      const FView Mv{&sm.ah[0][0], kLP, 1, kGdC, kGdC}, MTv{&sm.ah[0][0], 1, kLP, kGdC, kGdC};
      const FView Nv{&sm.p[0][0], kLP, 1, kGdC, kGdC}, NTv{&sm.p[0][0], 1, kLP, kGdC, kGdC};
      for (int job = w; job < 16; job += 4) {
        const bool isq = job >= 8;
        const int rb = (job & 7) >> 2, cb = job & 3;
        f32x16 a1 = {}, a2 = {};
        if (isq) {
          a1 = gd_block_product<kGdD>(dOv, S0Tv, 32 * rb, 32 * cb, a1);
          a2 = gd_block_product<kGdC>(Nv, Kv, 32 * rb, 32 * cb, a2);
        } else {
          a1 = gd_block_product<kGdD>(dKSv, S0Tv, 32 * rb, 32 * cb, a1);
          a2 = gd_block_product<kGdC>(NTv, Qv, 32 * rb, 32 * cb, a2);
          a2 = gd_block_product<kGdC>(Mv, Kv, 32 * rb, 32 * cb, a2);
          a2 = gd_block_product<kGdC>(MTv, Kv, 32 * rb, 32 * cb, a2);
        }
        float* outp = isq ? dq : dk;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 32 * rb + crow(i, hg), cc = 32 * cb + c;
          if (r >= n) continue;
          const float val = isq ? scale * sm.eg[r] * a1[i] + a2[i]
                                : a1[i] + a2[i] + sm.dec[r] * s_dKt[r * kGdD + cc];
          float* dst = outp + ((size_t)(t0 + r) * Hk + hk) * kGdD + cc;
          if (atomic_qk) atomicAdd(dst, val);
          else *dst = val;
        }
      }
    }
  }
  __syncthreads();
  if (dh0)
    for (int e = tid; e < kGdD * kGdD; e += kGdThreads) dh0[st_base + e] = s_dS[e];
}

// Clears dQ and dK before value heads that share a query/key head add into
// them; writes nothing when cu_seqlens is bad (the backward then writes nothing).
__global__ void __launch_bounds__(256)
gd_clear_kernel(float* __restrict__ a, float* __restrict__ b2, int64_t n, const int32_t* __restrict__ cu, int n_seg,
                int T) {
  __shared__ int s_bad;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  for (int s = threadIdx.x; s < n_seg; s += blockDim.x)
    if (cu[s + 1] < cu[s]) atomicOr(&s_bad, 1);
  if (threadIdx.x == 0 && (cu[0] != 0 || cu[n_seg] != T)) atomicOr(&s_bad, 1);
  __syncthreads();
  if (s_bad) return;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    a[i] = 0.f;
    b2[i] = 0.f;
  }
}

struct GdBwdLayout {
  size_t ck_s, ck_u, scratch, total;
};
GdBwdLayout gd_bwd_layout(int32_t T, int32_t H, int32_t n_seg) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t slots = (size_t)T / kGdC + (size_t)n_seg + 1;
  GdBwdLayout l;
  l.ck_s = 0;
  l.ck_u = up(slots * H * kGdD * kGdD * sizeof(float));
  l.scratch = l.ck_u + up(slots * H * kGdC * kGdD * sizeof(float));
  l.total = l.scratch + (size_t)std::max<int64_t>(1, (int64_t)n_seg * H) * kGdBwdScratch * sizeof(float);
  return l;
}

}  // namespace
}  // namespace pvb

extern "C" size_t pvb_gated_delta_bwd_workspace_bytes(int32_t T, int32_t H, int32_t n_seg) {
  if (T < 0 || H <= 0 || n_seg < 0) return 0;
  return pvb::gd_bwd_layout(T, H, n_seg).total;
}

extern "C" pvb_status pvb_gated_delta_bwd(const void* d_q, const void* d_k, const void* d_v, const float* d_g,
                                          const float* d_beta, const int32_t* d_cu, const int32_t* h_cu,
                                          int32_t n_seg, int32_t T, int32_t H, int32_t H_k, int32_t d, float scale,
                                          const float* d_h0, const void* d_dout, const float* d_dht, float* d_dq,
                                          float* d_dk, void* d_dv, float* d_dg, float* d_dbeta, float* d_dh0,
                                          int32_t grad_dtype, void* workspace, size_t workspace_bytes,
                                          int32_t* d_status, void* stream) {
  using namespace pvb;
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
  if ((int64_t)T * H * d >= ((int64_t)1 << 31) || !grid_fits((uint64_t)n_seg * H, kGdThreads))
    return PVB_E_UNSUPPORTED;
  const GdBwdLayout lay = gd_bwd_layout(T, H, n_seg);
  if (workspace == nullptr || workspace_bytes < lay.total) return PVB_E_WORKSPACE;
  const pvb_status hs = check_host_cu(h_cu, n_seg, T);
  if (hs != PVB_OK) return hs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* ck_s = reinterpret_cast<float*>(ws + lay.ck_s);
  float* ck_u = reinterpret_cast<float*>(ws + lay.ck_u);
  float* scr = reinterpret_cast<float*>(ws + lay.scratch);
  const bool atomic_qk = H != H_k;
  const int64_t nqk = (int64_t)T * H_k * d;
  if (atomic_qk && nqk > 0) {
    const unsigned blocks = (unsigned)std::min<int64_t>((nqk + 255) / 256, 8192);
    gd_clear_kernel<<<blocks, 256, 0, s>>>(d_dq, d_dk, nqk, d_cu, n_seg, T);
  }
  const unsigned grid = (unsigned)std::max<int64_t>(1, (int64_t)n_seg * H);
  // recomputation pass: the chunk-start states and the U of every chunk (it
  // also validates cu_seqlens and writes the status word)
  gated_delta_kernel<bf16, true><<<grid, kGdThreads, 0, s>>>(
      (const bf16*)d_q, (const bf16*)d_k, (const bf16*)d_v, d_g, d_beta, d_cu, n_seg, T, H, H_k, scale, d_h0,
      (bf16*)nullptr, nullptr, d_status, ck_s, ck_u);
  if (grad_dtype == PVB_F32)
    gated_delta_bwd_kernel<float><<<grid, kGdThreads, 0, s>>>(
        (const bf16*)d_q, (const bf16*)d_k, (const bf16*)d_v, d_g, d_beta, d_cu, n_seg, T, H, H_k, scale,
        (const bf16*)d_dout, d_dht, ck_s, ck_u, scr, d_dq, d_dk, (float*)d_dv, d_dg, d_dbeta, d_dh0, atomic_qk);
  else
    gated_delta_bwd_kernel<bf16><<<grid, kGdThreads, 0, s>>>(
        (const bf16*)d_q, (const bf16*)d_k, (const bf16*)d_v, d_g, d_beta, d_cu, n_seg, T, H, H_k, scale,
        (const bf16*)d_dout, d_dht, ck_s, ck_u, scr, d_dq, d_dk, (bf16*)d_dv, d_dg, d_dbeta, d_dh0, atomic_qk);
  return hipGetLastError() == hipSuccess ? PVB_OK : PVB_E_HIP;
}
