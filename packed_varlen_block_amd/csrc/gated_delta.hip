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

template <typename OutT>
__global__ void __launch_bounds__(kGdThreads, 1)
gated_delta_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
                   const float* __restrict__ g, const float* __restrict__ beta,
                   const int32_t* __restrict__ cu, int n_seg, int T, int H, int Hk, float scale,
                   const float* __restrict__ h0, OutT* __restrict__ o, float* __restrict__ ht,
                   int32_t* __restrict__ status) {
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
    if (w == 0) { block(KK{}, 1, 0); block(QK{}, 0, 0); }
    else if (w == 1) { block(QK{}, 1, 0); block(KK{}, 0, 0); }
    else if (w == 2) block(KK{}, 1, 1);
    else block(QK{}, 1, 1);

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
        oacc[rb] = mfma32(qa, shi, oacc[rb]);
        oacc[rb] = mfma32(qa, slo, oacc[rb]);
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
    for (int f = tid; f < 6 * 64; f += kGdThreads) {
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
    __syncthreads();                                  // the P and key fragments are complete

    // ---- O = scale (diag(G) Q S0 + P U) (row block 0 has no key past 31)
    // and S = G_63 S0 + (diag(G_63 / G) K)^T U: the matrix-core work of both
    // is issued first, then O is staged in the Q/K tiles (free by now) and
    // written with 16-byte stores.
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

  if (ht) {
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
