// matrix_scan_grad.hip: the parts of the matrix-scan gradient that follow the
// adjoint scan, for gfx950.
//
// "Tensor operations", the "matrix-scan" section: the gradient is the same
// scan run backwards on a's transposes. With lam[t] the adjoint of h[t] (that
// scan, run by launch_matrix_scan in adjoint mode), the chain rule through
// h[t] = a[t] @ h[p] + b[t] (p the step before t in scan order) gives
//   grad_b[t] = lam[t],   grad_a[t] = lam[t] @ h[p]^T   (zero at the first step),
// and the "gradient" section gives each gradient its operand's shape: an
// operand broadcast over some dims has its gradient summed over them.
//
// Kernels here:
//   ms_grad_a_kernel  one wave per step: lane (i, jq) forms grad_a[t][i][4jq ..
//                     4jq+3] from row i of lam[t] and rows 4jq .. 4jq+3 of
//                     h[p]; it also stores grad_b[t] when that is lam rounded
//                     to bf16. Bound by HBM (a 1 KiB grad_a block per
//                     step for n = 16).
//   sum_to_partial_kernel / sum_to_final_kernel
//                     the sum over broadcast dims, in two passes (partial sums
//                     over slices of the summed index space, then their sum in
//                     a fixed order), so results do not depend on scheduling.
#include "sx_common.hpp"

namespace sx {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float ld_f(const float* p) { return *p; }
__device__ __forceinline__ float ld_f(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void st_f(float* p, float v) { *p = v; }
__device__ __forceinline__ void st_f(uint16_t* p, float v) { *p = f32_to_bf16_rne(v); }

// TH: element type of h; TA: of grad_a (bf16 only when it is the final result).
template <typename TH, typename TA>
__global__ __launch_bounds__(256) void ms_grad_a_kernel(const GradAParams g) {
  const int64_t s = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);  // the step: a row-major lead index
  if (s >= g.steps) return;
  const int lane = int(threadIdx.x) & 63;
  const int i = lane >> 2, jq = lane & 3;
  const int n = g.n, m = g.m;
  const int64_t t = (s / g.inner) % g.T;
  const bool first = g.reverse ? t == g.T - 1 : t == 0;
  const int64_t prev = first ? s : (g.reverse ? s + g.inner : s - g.inner);  // always a valid step
  const float* lam = g.lam + s * int64_t(n) * m;
  const TH* hp = static_cast<const TH*>(g.h) + prev * int64_t(n) * m;
  const int ic = i < n ? i : n - 1;  // clamped rows: every load is in bounds
  int jc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) jc[q] = 4 * jq + q < n ? 4 * jq + q : n - 1;

  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int k = 0;
  if (m % 4 == 0 && (reinterpret_cast<uintptr_t>(g.lam) & 15) == 0) {  // rows of lam (f32) and of h in fours
    for (; k < m; k += 4) {
      const f32x4 l = *reinterpret_cast<const f32x4*>(lam + int64_t(ic) * m + k);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const TH* hr = hp + int64_t(jc[q]) * m + k;
        acc[q] = fmaf(l[0], ld_f(hr), acc[q]);
        acc[q] = fmaf(l[1], ld_f(hr + 1), acc[q]);
        acc[q] = fmaf(l[2], ld_f(hr + 2), acc[q]);
        acc[q] = fmaf(l[3], ld_f(hr + 3), acc[q]);
      }
    }
  }
  for (; k < m; ++k) {
    const float l = lam[int64_t(ic) * m + k];
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = fmaf(l, ld_f(hp + int64_t(jc[q]) * m + k), acc[q]);
  }
  TA* ga = static_cast<TA*>(g.grad_a) + s * int64_t(n) * n + int64_t(i) * n + 4 * jq;
  if (i < n) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (4 * jq + q < n) st_f(ga + q, first ? 0.0f : acc[q]);
  }
  if (g.grad_b != nullptr && i < n) {  // grad_b = lam rounded to bf16; the row's four lanes split it
    uint16_t* gb = static_cast<uint16_t*>(g.grad_b) + s * int64_t(n) * m + int64_t(i) * m;
    for (int kk = jq; kk < m; kk += 4) st_f(gb + kk, lam[int64_t(i) * m + kk]);
  }
}

// Index of the summed (reduced) space -> offset in the source; target index -> offset of its
// first source element. Both by row-major decoding over their own dims.
__device__ __forceinline__ int64_t decode(int64_t idx, int nd, const int64_t* dim, const int64_t* st) {
  int64_t off = 0;
  for (int d = nd - 1; d >= 0; --d) {
    const int64_t q = idx / dim[d];
    off += (idx - q * dim[d]) * st[d];
    idx = q;
  }
  return off;
}

// partial[split][e] = sum of src over the slice [split * per, (split + 1) * per) of the reduced space.
__global__ __launch_bounds__(256) void sum_to_partial_kernel(const SumToParams p) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t split = blockIdx.y;
  if (e >= p.targets) return;
  const int64_t base = decode(e, p.nd_keep, p.keep_dim, p.keep_st);
  const int64_t lo = split * p.per, hi = lo + p.per < p.reduced ? lo + p.per : p.reduced;
  float acc = 0.0f;
  for (int64_t j = lo; j < hi; ++j) acc += p.src[base + decode(j, p.nd_red, p.red_dim, p.red_st)];
  p.partial[split * p.targets + e] = acc;
}

template <typename TG>
__global__ __launch_bounds__(256) void sum_to_final_kernel(const SumToParams p, void* out) {
  const int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (e >= p.targets) return;
  float acc = 0.0f;
  for (int64_t sp = 0; sp < p.splits; ++sp) acc += p.partial[sp * p.targets + e];
  st_f(static_cast<TG*>(out) + e, acc);
}

}  // namespace

hipError_t launch_grad_a(const GradAParams& g, bool h_bf16, bool grad_a_bf16, hipStream_t stream) {
  if (g.steps <= 0 || g.n <= 0) return hipSuccess;
  const int64_t blocks = (g.steps + 3) / 4;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 grid{unsigned(blocks)}, block{256};
  if (h_bf16) {
    if (grad_a_bf16) hipLaunchKernelGGL((ms_grad_a_kernel<uint16_t, uint16_t>), grid, block, 0, stream, g);
    else hipLaunchKernelGGL((ms_grad_a_kernel<uint16_t, float>), grid, block, 0, stream, g);
  } else {
    if (grad_a_bf16) hipLaunchKernelGGL((ms_grad_a_kernel<float, uint16_t>), grid, block, 0, stream, g);
    else hipLaunchKernelGGL((ms_grad_a_kernel<float, float>), grid, block, 0, stream, g);
  }
  return hipGetLastError();
}

hipError_t launch_sum_to(const SumToParams& p, void* out, bool out_bf16, hipStream_t stream) {
  if (p.targets <= 0) return hipSuccess;
  const int64_t bx = (p.targets + 255) / 256;
  if (bx > 0x7fffffff || p.splits > 65535) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(sum_to_partial_kernel, dim3(unsigned(bx), unsigned(p.splits)), dim3(256), 0, stream, p);
  if (out_bf16) hipLaunchKernelGGL(sum_to_final_kernel<uint16_t>, dim3(unsigned(bx)), dim3(256), 0, stream, p, out);
  else hipLaunchKernelGGL(sum_to_final_kernel<float>, dim3(unsigned(bx)), dim3(256), 0, stream, p, out);
  return hipGetLastError();
}

}  // namespace sx
