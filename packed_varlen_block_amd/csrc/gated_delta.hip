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
// P, U, the gated keys) is split into bf16 hi + lo parts, so the products keep
// about 16 significant bits; the triangular solve is fp32 on the vector unit.
//
// One workgroup of 4 waves per (slice, head); the slices are independent.
// Wave w owns value columns [32w, 32w + 32) of the state, which stays in its
// registers (C layout of four 32x32 blocks) across the chunks of the slice.
#include "pvb_device.hpp"

namespace pvb {
namespace {

constexpr int kGdD = 128;            // d_k = d_v
constexpr int kGdC = 64;             // chunk length
constexpr int kGdThreads = 256;
constexpr int kKP = kGdD + 8;        // bf16 row pitch of the Q, K, V tiles
constexpr int kTP = kGdC + 8;        // bf16 row pitch of K^T
constexpr int kFP = kGdC + 4;        // fp32 row pitch of A^T, P and U^T

struct GdSmem {
  alignas(16) bf16 q[kGdC][kKP];
  alignas(16) bf16 k[kGdC][kKP];
  alignas(16) bf16 v[kGdC][kKP];
  alignas(16) bf16 kt[kGdD][kTP];    // K^T: kt[c][pos]
  alignas(16) float at[kGdC][kFP];   // A^T: at[j][i] = A[i][j]
  alignas(16) float p[kGdC][kFP];    // P (row i, column j)
  alignas(16) float ut[kGdD][kFP];   // U, transposed: ut[n][pos]
  alignas(16) float gam[kGdC];       // gamma_i
  alignas(16) float eg[kGdC];        // exp(gamma_i)
  alignas(16) float dec[kGdC];       // exp(gamma_63 - gamma_i)
  alignas(16) float beta[kGdC];
};

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
                   const int32_t* __restrict__ cu, int n_seg, int T, int H, float scale,
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

  for (int c0 = 0; c0 < L; c0 += kGdC) {
    const int nv = min(kGdC, L - c0);
    __syncthreads();                                  // the previous chunk's reads are done

    // ---- stage Q, K, V (zero past the slice's end), K^T, and the gates
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int ch = tid + kGdThreads * it;           // 16-byte chunk: row ch/16, columns 8(ch%16)..
      const int row = ch >> 4, col = (ch & 15) * 8;
      uint4 xq = zero4(), xk = zero4(), xv = zero4();
      if (row < nv) {
        const size_t off = ((size_t)(seg0 + c0 + row) * H + h) * kGdD + col;
        xq = *(const uint4*)(q + off);
        xk = *(const uint4*)(k + off);
        xv = *(const uint4*)(v + off);
      }
      *(uint4*)&sm.q[row][col] = xq;
      *(uint4*)&sm.k[row][col] = xk;
      *(uint4*)&sm.v[row][col] = xv;
      const bf16x8 kk = __builtin_bit_cast(bf16x8, xk);
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.kt[col + e][row] = kk[e];
    }
    if (w == 0) {
      float gg = 0.f, bb = 0.f;
      if (lane < nv) {
        const size_t idx = (size_t)(seg0 + c0 + lane) * H + h;
        gg = g[idx];
        bb = beta[idx];
      }
      float x = gg;                                   // inclusive sum over the chunk
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      const float last = __shfl(x, 63, 64);
      sm.gam[lane] = x;
      sm.eg[lane] = expf(x);
      sm.dec[lane] = expf(last - x);
      sm.beta[lane] = bb;
    }
    __syncthreads();

    // ---- A (for the solve, stored transposed) and P: the lower 32x32 blocks
    // (0,0), (1,0), (1,1) of K K^T and Q K^T; block (0,1) is never read
    for (int item = w; item < 6; item += 4) {
      const bool isq = item >= 3;
      const int blk = isq ? item - 3 : item;
      const int bi = blk == 0 ? 0 : 1, bj = blk == 2 ? 1 : 0;
      f32x16 acc = {};
#pragma unroll
      for (int s = 0; s < kGdD / 16; ++s) {
        const bf16x8 a = isq ? *(const bf16x8*)&sm.q[32 * bi + c][16 * s + 8 * hg]
                             : *(const bf16x8*)&sm.k[32 * bi + c][16 * s + 8 * hg];
        const bf16x8 bk = *(const bf16x8*)&sm.k[32 * bj + c][16 * s + 8 * hg];
        acc = mfma32(a, bk, acc);
      }
      const int pj = 32 * bj + c;
      const float gj = sm.gam[pj];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int pi = 32 * bi + crow(i, hg);
        const float dcy = pj <= pi ? expf(sm.gam[pi] - gj) : 0.f;
        if (isq) sm.p[pi][pj] = acc[i] * dcy;
        else sm.at[pj][pi] = pj < pi ? sm.beta[pi] * acc[i] * dcy : 0.f;
      }
    }

    // ---- K S0 for this wave's columns.  The state is the B operand straight
    // from its C layout: k-step s takes elements 8(s%2) + e of block s/2, i.e.
    // key dims 16s + 8(e/4) + 4hg + e%4, so the K rows are read in that order
    // (two 8-byte pieces).
    f32x16 ks[2] = {};
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
        const bf16x8 ka = cat(*(const bf16x4*)kr, *(const bf16x4*)(kr + 8));
        ks[rb] = mfma32(ka, shi, ks[rb]);
        ks[rb] = mfma32(ka, slo, ks[rb]);
      }
    }

    // ---- right-hand side, in place: rows pos = 32 rb + crow(i, hg)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int pos = 32 * rb + crow(i, hg);
        ks[rb][i] = sm.beta[pos] * ((float)sm.v[pos][n0] - sm.eg[pos] * ks[rb][i]);
      }
    __syncthreads();                                  // A is complete

    // ---- (I + A) U = rhs in the C layout: lanes c and c + 32 hold column
    // n0, each in groups of four rows (rows 8m + 4hg .. + 3 of each 32-row
    // block).  Step j: the lane holding row j (final by then) hands u_j to its
    // partner, and every row group that may lie below row j subtracts its
    // A[row][j] multiple.  A is zero on and above the diagonal, so the rows
    // of row j's own group that are not below it are left as they are.
    // The A values of step j + 1 are read while step j computes.
    float4 acur[2][4], anext[2][4];
    auto load_a = [&](int j, float4 (&buf)[2][4]) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (32 * rb + 8 * m + 7 > j) buf[rb][m] = *(const float4*)&sm.at[j][32 * rb + 8 * m + 4 * hg];
    };
    load_a(0, acur);
#pragma unroll
    for (int j = 0; j < kGdC - 1; ++j) {
      if (j + 1 < kGdC - 1) load_a(j + 1, anext);
      const int rbj = j >> 5, jj = j & 31;
      const int ij = 4 * (jj >> 3) + (jj & 3);        // element index of row j
      const bool own = ((jj >> 2) & 1) == hg;
      const float x = ks[rbj][ij];
      const float other = swap_halves(x);
      const float uj = own ? x : other;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if (32 * rb + 8 * m + 7 <= j) continue;      // the whole group is at or above row j
          const float4 a4 = acur[rb][m];
          ks[rb][4 * m] -= a4.x * uj;
          ks[rb][4 * m + 1] -= a4.y * uj;
          ks[rb][4 * m + 2] -= a4.z * uj;
          ks[rb][4 * m + 3] -= a4.w * uj;
        }
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int m = 0; m < 4; ++m) acur[rb][m] = anext[rb][m];
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sm.ut[n0][32 * rb + crow(i, hg)] = ks[rb][i];

    // ---- Q S0 (the state's part of O), after the solve to keep it short
    f32x16 oacc[2] = {};
#pragma unroll
    for (int s = 0; s < kGdD / 16; ++s) {
      float sv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = S[s >> 1][8 * (s & 1) + e];
      bf16x8 shi, slo;
      split8(sv, shi, slo);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const bf16* qr = &sm.q[32 * rb + c][16 * s + 4 * hg];
        const bf16x8 qa = cat(*(const bf16x4*)qr, *(const bf16x4*)(qr + 8));
        oacc[rb] = mfma32(qa, shi, oacc[rb]);
        oacc[rb] = mfma32(qa, slo, oacc[rb]);
      }
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[rb][i] *= sm.eg[32 * rb + crow(i, hg)];

    // ---- U as the B operand (k = position), split; reused by both products
    bf16x8 uh[4], ul[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float* src = &sm.ut[n0][16 * s + 8 * hg];
      const float4 a4 = *(const float4*)src, b4 = *(const float4*)(src + 4);
      const float x[8] = {a4.x, a4.y, a4.z, a4.w, b4.x, b4.y, b4.z, b4.w};
      split8(x, uh[s], ul[s]);
    }

    // ---- O = scale (diag(G) Q S0 + P U); row block 0 has no key past 31
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (rb == 0 && s >= 2) continue;
        const float* src = &sm.p[32 * rb + c][16 * s + 8 * hg];
        const float4 a4 = *(const float4*)src, b4 = *(const float4*)(src + 4);
        const float x[8] = {a4.x, a4.y, a4.z, a4.w, b4.x, b4.y, b4.z, b4.w};
        bf16x8 ph, pl;
        split8(x, ph, pl);
        oacc[rb] = mfma32(ph, uh[s], oacc[rb]);
        oacc[rb] = mfma32(ph, ul[s], oacc[rb]);
        oacc[rb] = mfma32(pl, uh[s], oacc[rb]);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int pos = 32 * rb + crow(i, hg);
        if (pos < nv) o[((size_t)(seg0 + c0 + pos) * H + h) * kGdD + n0] = out_cast<OutT>(scale * oacc[rb][i]);
      }
    }

    // ---- S = G_63 S0 + (diag(G_63 / G) K)^T U
    const float glast = sm.eg[kGdC - 1];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
#pragma unroll
      for (int i = 0; i < 16; ++i) S[r][i] *= glast;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 k8 = *(const bf16x8*)&sm.kt[32 * r + c][16 * s + 8 * hg];
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (float)k8[e] * sm.dec[16 * s + 8 * hg + e];
        bf16x8 kh, kl;
        split8(x, kh, kl);
        S[r] = mfma32(kh, uh[s], S[r]);
        S[r] = mfma32(kh, ul[s], S[r]);
        S[r] = mfma32(kl, uh[s], S[r]);
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

extern "C" pvb_status pvb_gated_delta_fwd(const void* d_q, const void* d_k, const void* d_v, const float* d_g,
                                          const float* d_beta, const int32_t* d_cu, const int32_t* h_cu,
                                          int32_t n_seg, int32_t T, int32_t H, int32_t d, float scale,
                                          const float* d_h0, void* d_o, int32_t o_dtype, float* d_ht,
                                          int32_t* d_status, void* stream) {
  using namespace pvb;
  if (n_seg < 0 || T < 0 || H <= 0 || d_cu == nullptr || d_status == nullptr) return PVB_E_INVALID_ARG;
  if (T > 0 && (d_q == nullptr || d_k == nullptr || d_v == nullptr || d_g == nullptr || d_beta == nullptr ||
                d_o == nullptr))
    return PVB_E_INVALID_ARG;
  if (o_dtype != PVB_BF16 && o_dtype != PVB_F32) return PVB_E_INVALID_ARG;
  if (!(scale > 0.f) || !(scale < INFINITY)) return PVB_E_INVALID_ARG;
  if (d != kGdD) return PVB_E_UNSUPPORTED;
  if ((int64_t)T * H * d >= ((int64_t)1 << 31) || (int64_t)n_seg * H >= ((int64_t)1 << 31) - 1)
    return PVB_E_UNSUPPORTED;
  const pvb_status hs = check_host_cu(h_cu, n_seg, T);
  if (hs != PVB_OK) return hs;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // one workgroup per (slice, head); with no slice, one workgroup still checks
  // cu_seqlens and writes the status
  const unsigned grid = (unsigned)std::max<int64_t>(1, (int64_t)n_seg * H);
  if (o_dtype == PVB_F32)
    gated_delta_kernel<float><<<grid, kGdThreads, 0, s>>>(
        (const bf16*)d_q, (const bf16*)d_k, (const bf16*)d_v, d_g, d_beta, d_cu, n_seg, T, H, scale, d_h0,
        (float*)d_o, d_ht, d_status);
  else
    gated_delta_kernel<bf16><<<grid, kGdThreads, 0, s>>>(
        (const bf16*)d_q, (const bf16*)d_k, (const bf16*)d_v, d_g, d_beta, d_cu, n_seg, T, H, scale, d_h0,
        (bf16*)d_o, d_ht, d_status);
  return hipGetLastError() == hipSuccess ? PVB_OK : PVB_E_HIP;
}
