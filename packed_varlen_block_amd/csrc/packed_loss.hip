// Token-weighted negative log-likelihood over packed cells, and its logit
// gradient ("Pack sequences without joining their contexts", "Keep the same
// nine-target objective": the loss sum over eligible targets divided once by
// their count N; the mean-loss logit derivative (p_ic - 1[c = y_i]) / N;
// excluded cells contribute exactly zero and are skipped before any
// arithmetic, so NaN or Inf logits in them cannot leak; zero eligible targets
// is an error).  The one-step label shift with a sample-local ignore at each
// sample's last cell ("Packing与 FlashAttention Varlen", section 2) is a data
// rule applied before this call.
//
// Three launches on the caller's stream:
//   nll_count_kernel  one workgroup: N and the target checks (status word);
//   nll_row_kernel    one workgroup per cell: the row's log-sum-exp in one
//                     pass (per-thread running max and rescaled sum, combined
//                     across the workgroup), its NLL, then the gradient row.
//                     Rows of up to kHeld 16-byte vectors per thread stay in
//                     registers between the two passes (the logits are read
//                     from HBM once); longer or unaligned rows are read again;
//   nll_sum_kernel    one workgroup: the loss sum in float64 in a fixed order
//                     (deterministic), and the mean.
#include "pvb_device.hpp"

namespace pvb {
namespace {

constexpr int kCountThreads = 1024;
constexpr int kRowThreads = 256;

__device__ __forceinline__ bool eligible(const int32_t* __restrict__ targets, const uint8_t* __restrict__ mask,
                                         int64_t c) {
  return targets[c] >= 0 && (mask == nullptr || mask[c] != 0);
}

__global__ void __launch_bounds__(kCountThreads)
nll_count_kernel(const int32_t* __restrict__ targets, const uint8_t* __restrict__ mask, int64_t C, int V,
                 int32_t* __restrict__ count, int32_t* __restrict__ status) {
  __shared__ int64_t s_n[kCountThreads / 64];
  __shared__ int s_bad;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  int64_t n = 0;
  int bad = 0;
  for (int64_t c = tid; c < C; c += kCountThreads) {
    if (eligible(targets, mask, c)) {
      ++n;
      if (targets[c] >= V) bad = 1;     // a supervised target must be a class
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) n += __shfl_xor(n, off, 64);
  if (lane == 0) s_n[w] = n;
  if (bad) atomicOr(&s_bad, 1);
  __syncthreads();
  if (tid == 0) {
    int64_t t = 0;
    for (int k = 0; k < kCountThreads / 64; ++k) t += s_n[k];
    int st = PVB_OK;
    if (s_bad) st = PVB_E_INVALID_ARG;
    else if (t == 0) st = PVB_E_NO_TARGETS;
    else if (t > INT32_MAX) st = PVB_E_OVERFLOW;
    *count = (int32_t)(st == PVB_OK ? t : 0);
    *status = st;
  }
}

template <typename T>
__device__ __forceinline__ float load_f(const T* p) { return (float)*p; }

// One workgroup per cell.  VEC elements per load (16 bytes when the row is
// aligned for it, else 1); HELD: the row is held in registers (VEC > 1 and
// V <= kHeld * VEC * kRowThreads).
constexpr int kHeld = 16;
template <typename LT, typename GT, int VEC, bool HELD>
__global__ void __launch_bounds__(kRowThreads)
nll_row_kernel(const LT* __restrict__ logits, int V, const int32_t* __restrict__ targets,
               const uint8_t* __restrict__ mask, const int32_t* __restrict__ count,
               const int32_t* __restrict__ status, float* __restrict__ row_nll, GT* __restrict__ grad) {
  __shared__ float s_m[kRowThreads / 64], s_s[kRowThreads / 64];
  if (*status != PVB_OK) return;
  const int64_t c = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  GT* grow = grad == nullptr ? nullptr : grad + c * (int64_t)V;
  if (!eligible(targets, mask, c)) {
    // excluded: zero loss and a zero gradient row, never computed from the logits
    if (tid == 0) row_nll[c] = 0.f;
    if (grow != nullptr)
      for (int v = tid; v < V; v += kRowThreads) grow[v] = (GT)0.f;
    return;
  }
  const LT* row = logits + c * (int64_t)V;
  const int y = targets[c];
  // pass 1: running max and sum of exp(x - max), per thread, in log2 units
  float m = -INFINITY, s = 0.f;
  auto add = [&](float x) {
    const float xl = x * kLog2e;
    if (xl > m) {
      s = s * fast_exp2(m - xl) + 1.f;
      m = xl;
    } else {
      s += fast_exp2(xl - m);
    }
  };
  const int nv = V / VEC;
  typedef __attribute__((__vector_size__(VEC * sizeof(LT)))) LT vec_t;
  vec_t held[HELD ? kHeld : 1];
  if constexpr (HELD) {
    // every load in flight at once, then the pass over registers.  Each logit
    // and each gradient element is touched once: loads and stores are marked
    // non-temporal.
    typedef int ivec_t __attribute__((vector_size(sizeof(vec_t))));
#pragma unroll
    for (int k = 0; k < kHeld; ++k) {
      const int i = tid + k * kRowThreads;
      if (i < nv)
        held[k] = __builtin_bit_cast(vec_t, __builtin_nontemporal_load((const ivec_t*)(row + (int64_t)i * VEC)));
    }
    // the thread's max, then its sum of exp2(x log2e - max): no rescaling
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < kHeld; ++k)
      if (tid + k * kRowThreads < nv) {
#pragma unroll
        for (int e = 0; e < VEC; ++e) mx = fmaxf(mx, (float)held[k][e]);
      }
    if (mx > -INFINITY) {
      m = mx * kLog2e;
#pragma unroll
      for (int k = 0; k < kHeld; ++k)
        if (tid + k * kRowThreads < nv) {
#pragma unroll
          for (int e = 0; e < VEC; ++e) s += fast_exp2((float)held[k][e] * kLog2e - m);
        }
    }
  } else {
    for (int i = tid; i < nv; i += kRowThreads) {
      if constexpr (VEC == 1) {
        add(load_f(row + i));
      } else {
        const vec_t x = *(const vec_t*)(row + (int64_t)i * VEC);
#pragma unroll
        for (int e = 0; e < VEC; ++e) add((float)x[e]);
      }
    }
    for (int v = nv * VEC + tid; v < V; v += kRowThreads) add(load_f(row + v));
  }
  // combine (m, s) pairs: over the wave, then over the waves
  auto merge = [](float& m1, float& s1, float m2, float s2) {
    const float mm = fmaxf(m1, m2);
    if (mm == -INFINITY) return;
    s1 = s1 * fast_exp2(m1 - mm) + s2 * fast_exp2(m2 - mm);
    m1 = mm;
  };
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float m2 = __shfl_xor(m, off, 64), s2 = __shfl_xor(s, off, 64);
    merge(m, s, m2, s2);
  }
  if (lane == 0) {
    s_m[w] = m;
    s_s[w] = s;
  }
  __syncthreads();
  m = s_m[0];
  s = s_s[0];
  for (int k = 1; k < kRowThreads / 64; ++k) merge(m, s, s_m[k], s_s[k]);
  // log-sum-exp (natural log) in float64 from the float32 partial sums
  const double lse = ((double)m + log2((double)s)) * (double)kLn2;
  if (tid == 0) row_nll[c] = (float)(lse - (double)load_f(row + y));
  if (grow == nullptr) return;
  // pass 2: (p - 1[v = y]) / N, with 1/N folded into the exponent
  const float inv_n = 1.f / (float)*count;
  const float lse2 = (float)(lse * (double)kLog2e);
  const float lse2n = (float)(lse * (double)kLog2e + log2((double)*count));
  if constexpr (HELD) {
    typedef __attribute__((__vector_size__(VEC * sizeof(GT)))) GT gvec_t;
#pragma unroll
    for (int k = 0; k < kHeld; ++k) {
      const int i = tid + k * kRowThreads;
      if (i < nv) {
        gvec_t gv;
#pragma unroll
        for (int e = 0; e < VEC; ++e) gv[e] = (GT)fast_exp2((float)held[k][e] * kLog2e - lse2n);
        if ((unsigned)(y - i * VEC) < (unsigned)VEC)      // this vector holds the target class
          gv[y - i * VEC] = (GT)(fast_exp2((float)held[k][y - i * VEC] * kLog2e - lse2n) - inv_n);
        typedef int givec_t __attribute__((vector_size(sizeof(gvec_t))));
        __builtin_nontemporal_store(__builtin_bit_cast(givec_t, gv), (givec_t*)(grow + (int64_t)i * VEC));
      }
    }
  } else {
    for (int v = tid; v < V; v += kRowThreads) {
      const float p = fast_exp2(load_f(row + v) * kLog2e - lse2);
      grow[v] = (GT)((p - (v == y ? 1.f : 0.f)) * inv_n);
    }
  }
}

__global__ void __launch_bounds__(kCountThreads)
nll_sum_kernel(const float* __restrict__ row_nll, int64_t C, const int32_t* __restrict__ count,
               const int32_t* __restrict__ status, double* __restrict__ loss) {
  __shared__ double s_p[kCountThreads / 64];
  if (*status != PVB_OK) return;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  double p = 0.0;
  for (int64_t c = tid; c < C; c += kCountThreads) p += (double)row_nll[c];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off, 64);
  if (lane == 0) s_p[w] = p;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int k = 0; k < kCountThreads / 64; ++k) t += s_p[k];
    loss[0] = t;
    loss[1] = t / (double)*count;
  }
}

template <typename LT, typename GT>
void launch_rows(const void* logits, int64_t C, int V, const int32_t* targets, const uint8_t* mask,
                 const int32_t* count, const int32_t* status, float* row_nll, void* grad, hipStream_t s) {
  constexpr int VEC = 16 / sizeof(LT);
  const bool vec = (V * sizeof(LT)) % 16 == 0 && ((uintptr_t)logits & 15) == 0 &&
                   (grad == nullptr || ((uintptr_t)grad & 15) == 0);
  const bool held = vec && V <= kHeld * VEC * kRowThreads;
  if (held)
    nll_row_kernel<LT, GT, VEC, true><<<dim3((unsigned)C), kRowThreads, 0, s>>>(
        (const LT*)logits, V, targets, mask, count, status, row_nll, (GT*)grad);
  else if (vec)
    nll_row_kernel<LT, GT, VEC, false><<<dim3((unsigned)C), kRowThreads, 0, s>>>(
        (const LT*)logits, V, targets, mask, count, status, row_nll, (GT*)grad);
  else
    nll_row_kernel<LT, GT, 1, false><<<dim3((unsigned)C), kRowThreads, 0, s>>>(
        (const LT*)logits, V, targets, mask, count, status, row_nll, (GT*)grad);
}

}  // namespace
}  // namespace pvb

extern "C" pvb_status pvb_packed_nll(const void* d_logits, int32_t logits_dtype, int64_t C, int32_t V,
                                     const int32_t* d_targets, const uint8_t* d_mask, float* d_row_nll,
                                     double* d_loss, int32_t* d_count, void* d_grad, int32_t grad_dtype,
                                     int32_t* d_status, void* stream) {
  using namespace pvb;
  if (C < 0 || V <= 0 || d_status == nullptr || d_loss == nullptr || d_count == nullptr) return PVB_E_INVALID_ARG;
  if (C > 0 && (d_logits == nullptr || d_targets == nullptr || d_row_nll == nullptr)) return PVB_E_INVALID_ARG;
  if (logits_dtype != PVB_BF16 && logits_dtype != PVB_F32) return PVB_E_INVALID_ARG;
  if (d_grad != nullptr && grad_dtype != PVB_BF16 && grad_dtype != PVB_F32) return PVB_E_INVALID_ARG;
  if (!grid_fits((uint64_t)C, kRowThreads)) return PVB_E_UNSUPPORTED;   // one workgroup per cell
  if (V > PVB_MAX_COUNT) return PVB_E_OVERFLOW;
  hipStream_t s = static_cast<hipStream_t>(stream);
  nll_count_kernel<<<1, kCountThreads, 0, s>>>(d_targets, d_mask, C, V, d_count, d_status);
  if (C > 0) {
    const bool lb = logits_dtype == PVB_BF16, gb = grad_dtype == PVB_BF16;
    if (lb && gb) launch_rows<bf16, bf16>(d_logits, C, V, d_targets, d_mask, d_count, d_status, d_row_nll, d_grad, s);
    else if (lb) launch_rows<bf16, float>(d_logits, C, V, d_targets, d_mask, d_count, d_status, d_row_nll, d_grad, s);
    else if (gb) launch_rows<float, bf16>(d_logits, C, V, d_targets, d_mask, d_count, d_status, d_row_nll, d_grad, s);
    else launch_rows<float, float>(d_logits, C, V, d_targets, d_mask, d_count, d_status, d_row_nll, d_grad, s);
  }
  nll_sum_kernel<<<1, kCountThreads, 0, s>>>(d_row_nll, C, d_count, d_status, d_loss);
  return hipGetLastError() == hipSuccess ? PVB_OK : PVB_E_HIP;
}
