// matrix_scan_grad.hip: the parts of the matrix-scan gradient that follow the
// adjoint scan, for gfx950.
//
// "Tensor operations", the "matrix-scan" section: the gradient is a scan in
// the opposite direction over transposed a. With lam[t] the adjoint of h[t] (that
// scan, run by launch_matrix_scan in adjoint mode), the chain rule through
// h[t] = a[t] @ h[p] + b[t] (p the step before t in scan order) gives
//   grad_b[t] = lam[t],   grad_a[t] = lam[t] @ h[p]^T   (zero at the first step),
// and the "gradient" section gives each gradient its operand's shape: an
// operand broadcast over some dims has its gradient summed over them.
//
// Kernels here:
//   ms_grad_a_kernel  the grid's waves stride over the steps: n = 16 with
//                     m = 1, an outer product a step, each lane storing four
//                     consecutive values of one row; m = 16, lam h^T on MFMA
//                     for a run of four steps per wave (every load of the run
//                     issued before its first store); 16 | m, MFMA over
//                     16-column blocks a step; other shapes element by element.
//                     It also stores grad_b[t] when that is lam rounded to
//                     bf16 from an f32 lam. When grad_b is bf16 and has the
//                     result's shape, the scan writes lam straight into it,
//                     rounded, and this kernel reads that rounded lam (one
//                     bf16 stream instead of an f32 one out and back). Bound
//                     by HBM (a 1 KiB grad_a block per step for n = 16, f32).
//   sum_to_partial_kernel / sum_to_final_kernel
//                     the sum over broadcast dims, in two passes (partial sums
//                     over slices of the summed index space, then their sum in
//                     a fixed order), so results do not depend on scheduling.
#include <algorithm>

#include "ms_mfma.hpp"
#include "sx_common.hpp"

namespace sx {
namespace {

__device__ __forceinline__ float ld_f(const float* p) { return *p; }
__device__ __forceinline__ float ld_f(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void st_f(float* p, float v) { *p = v; }
__device__ __forceinline__ void st_f(uint16_t* p, float v) { *p = f32_to_bf16_rne(v); }

// Four consecutive elements as f32 (one 16- or 8-byte load), and back.
__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ f32x4 ld4(const uint16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
               __uint_as_float(u.y & 0xffff0000u)};
}
__device__ __forceinline__ void st4(float* p, f32x4 v) { st_stream(reinterpret_cast<f32x4*>(p), v); }
__device__ __forceinline__ void st4(uint16_t* p, f32x4 v) {
  st_stream(reinterpret_cast<u32x2*>(p), u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
}

// The step before step s in the forward scan order (s itself at the first step).
__device__ __forceinline__ int64_t prev_step(const GradAParams& g, int64_t s, bool& first) {
  const int64_t t = (s / g.inner) % g.T;
  first = g.reverse ? t == g.T - 1 : t == 0;
  return first ? s : (g.reverse ? s + g.inner : s - g.inner);
}

// n = 16, m = 1: grad_a[i][j] = lam[i] h[j]. Lane (i, jq), i = lane / 4, forms
// grad_a[i][4jq .. 4jq+3] and stores it as one piece, so the wave writes the
// step's block contiguously.
template <typename TL, typename TH, typename TA>
__device__ __forceinline__ void grad_a_m1(const GradAParams& g, int64_t s, int lane) {
  const int i = lane >> 2, jq = lane & 3;
  bool first;
  const int64_t p = prev_step(g, s, first);
  const float l = ld_f(static_cast<const TL*>(g.lam) + s * 16 + i);
  const f32x4 hv = ld4(static_cast<const TH*>(g.h) + p * 16 + 4 * jq);
  const f32x4 d = first ? zero4() : l * hv;
  st4(static_cast<TA*>(g.grad_a) + s * 256 + i * 16 + 4 * jq, d);
  if (g.grad_b != nullptr && jq == 0) st_f(static_cast<uint16_t*>(g.grad_b) + s * 16 + i, l);
}

// n = 16, m a multiple of 16: grad_a = lam h^T, K = m, by MFMA. Lane (r, c)
// supplies row c of lam and row c of h (columns 4r .. 4r+3 of each 16-block),
// which are the A and X operands of lam h^T; a quad transpose of the result
// gives each lane four consecutive values of one row to store.
template <typename TL, typename TH, typename TA>
__device__ __forceinline__ void grad_a_tiles(const GradAParams& g, int64_t s, int lane) {
  const int r = lane >> 4, c = lane & 15, m = g.m;
  bool first;
  const int64_t p = prev_step(g, s, first);
  const TL* lr = static_cast<const TL*>(g.lam) + s * 16 * m + int64_t(c) * m + 4 * r;
  const TH* hr = static_cast<const TH*>(g.h) + p * 16 * m + int64_t(c) * m + 4 * r;
  uint16_t* br = g.grad_b ? static_cast<uint16_t*>(g.grad_b) + s * 16 * m + int64_t(c) * m + 4 * r : nullptr;
  f32x4 acc = zero4();
  for (int kb = 0; kb < m; kb += 16) {
    const f32x4 la = ld4(lr + kb);
    acc = mfma_16x16x16(la, ld4(hr + kb), acc);
    if (br) st4(br + kb, la);
  }
  const int j = c & 3;
  const f32x4 row = quad_transpose(first ? zero4() : acc, j);  // grad_a[4r + j][4 (c / 4) ..]
  st4(static_cast<TA*>(g.grad_a) + s * 256 + (4 * r + j) * 16 + 4 * (c >> 2), row);
}

// For m = 16 each wave takes a run of consecutive steps and issues every load
// of the run before the first store: one step at a time, the compiler cannot
// move a later step's loads above an earlier step's store (it does not know
// that grad_a overlaps no input), so each step waited a full load round trip
// (runs of 4: 69 against 78 us for the bf16 [16,16384] gradient). For m = 1 one
// step at a time, neighbouring waves on neighbouring steps, stayed the fastest
// (62 us; runs of 1 to 16 steps: 65-70 us). Steps past the end load the last
// step and store nothing.

// n = 16, m = 16, a run of R steps from s0 (as grad_a_tiles with one 16-column block).
template <int R, typename TL, typename TH, typename TA>
__device__ __forceinline__ void grad_a_t16_run(const GradAParams& g, int64_t s0, int lane) {
  const int r = lane >> 4, c = lane & 15, j = c & 3;
  f32x4 la[R], hb[R];
  bool first[R];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int64_t s = s0 + u < g.steps ? s0 + u : g.steps - 1;
    const int64_t p = prev_step(g, s, first[u]);
    la[u] = ld4(static_cast<const TL*>(g.lam) + s * 256 + c * 16 + 4 * r);
    hb[u] = ld4(static_cast<const TH*>(g.h) + p * 256 + c * 16 + 4 * r);
  }
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int64_t s = s0 + u;
    if (s < g.steps) {
      const f32x4 acc = mfma_16x16x16(la[u], hb[u], zero4());
      if (g.grad_b != nullptr) st4(static_cast<uint16_t*>(g.grad_b) + s * 256 + c * 16 + 4 * r, la[u]);
      const f32x4 row = quad_transpose(first[u] ? zero4() : acc, j);  // grad_a[4r + j][4 (c / 4) ..]
      st4(static_cast<TA*>(g.grad_a) + s * 256 + (4 * r + j) * 16 + 4 * (c >> 2), row);
    }
  }
}

// Steps per run of the m = 16 path (PATH 3).
constexpr int kRunT16 = 4;

// Any n <= 16, m: lane (i, jq) forms grad_a[i][4jq .. 4jq+3] element by element.
template <typename TL, typename TH, typename TA>
__device__ __forceinline__ void grad_a_any(const GradAParams& g, int64_t s, int lane) {
  const int i = lane >> 2, jq = lane & 3;
  const int n = g.n, m = g.m;
  bool first;
  const int64_t p = prev_step(g, s, first);
  const TL* lam = static_cast<const TL*>(g.lam) + s * int64_t(n) * m;
  const TH* hp = static_cast<const TH*>(g.h) + p * int64_t(n) * m;
  const int ic = i < n ? i : n - 1;  // clamped rows: every load is in bounds
  int jc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) jc[q] = 4 * jq + q < n ? 4 * jq + q : n - 1;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int k = 0; k < m; ++k) {
    const float l = ld_f(lam + int64_t(ic) * m + k);
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
    for (int kk = jq; kk < m; kk += 4) st_f(gb + kk, ld_f(lam + int64_t(i) * m + kk));
  }
}

// One wave per step, the waves of the grid striding over the steps.
// TL: element type of lam (bf16 when it was rounded into a bf16 grad_b);
// TH: of h; TA: of grad_a (bf16 only when it is the final result).
template <int PATH, typename TL, typename TH, typename TA>
__global__ __launch_bounds__(256) void ms_grad_a_kernel(const GradAParams g) {
  const int lane = int(threadIdx.x) & 63;
  const int64_t nw = int64_t(gridDim.x) * 4;
  const int64_t w = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if constexpr (PATH == 3) {
    for (int64_t s0 = w * kRunT16; s0 < g.steps; s0 += nw * kRunT16) grad_a_t16_run<kRunT16, TL, TH, TA>(g, s0, lane);
  } else {
    for (int64_t s = w; s < g.steps; s += nw) {
      if constexpr (PATH == 1) grad_a_m1<TL, TH, TA>(g, s, lane);
      else if constexpr (PATH == 2) grad_a_tiles<TL, TH, TA>(g, s, lane);
      else grad_a_any<TL, TH, TA>(g, s, lane);
    }
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

namespace {
template <int PATH, typename TL>
void launch_grad_a_path(const GradAParams& g, bool h_bf16, bool grad_a_bf16, dim3 grid, hipStream_t stream) {
  const dim3 block{256};
  if (h_bf16) {
    if (grad_a_bf16) hipLaunchKernelGGL((ms_grad_a_kernel<PATH, TL, uint16_t, uint16_t>), grid, block, 0, stream, g);
    else hipLaunchKernelGGL((ms_grad_a_kernel<PATH, TL, uint16_t, float>), grid, block, 0, stream, g);
  } else {
    if (grad_a_bf16) hipLaunchKernelGGL((ms_grad_a_kernel<PATH, TL, float, uint16_t>), grid, block, 0, stream, g);
    else hipLaunchKernelGGL((ms_grad_a_kernel<PATH, TL, float, float>), grid, block, 0, stream, g);
  }
}
template <int PATH>
void launch_grad_a_lam(const GradAParams& g, bool h_bf16, bool grad_a_bf16, dim3 grid, hipStream_t stream) {
  if (g.lam_bf16) launch_grad_a_path<PATH, uint16_t>(g, h_bf16, grad_a_bf16, grid, stream);
  else launch_grad_a_path<PATH, float>(g, h_bf16, grad_a_bf16, grid, stream);
}
}  // namespace

hipError_t launch_grad_a(const GradAParams& g, bool h_bf16, bool grad_a_bf16, hipStream_t stream) {
  if (g.steps <= 0 || g.n <= 0) return hipSuccess;
  // enough waves to fill the GPU several times over; each strides over the steps
  const int64_t blocks = std::min<int64_t>((g.steps + 3) / 4, int64_t(device_cu_count()) * 16);
  const dim3 grid{unsigned(blocks)};
  // the fast paths read and write whole 16-byte (f32) or 8-byte (bf16) pieces
  auto aligned = [](const void* q, uintptr_t a) { return q == nullptr || reinterpret_cast<uintptr_t>(q) % a == 0; };
  const bool al = aligned(g.lam, g.lam_bf16 ? 8 : 16) && aligned(g.h, h_bf16 ? 8 : 16) &&
                  aligned(g.grad_a, grad_a_bf16 ? 8 : 16) && aligned(g.grad_b, 8);
  if (g.n == 16 && g.m == 1 && al) launch_grad_a_lam<1>(g, h_bf16, grad_a_bf16, grid, stream);
  else if (g.n == 16 && g.m == 16 && al) launch_grad_a_lam<3>(g, h_bf16, grad_a_bf16, grid, stream);
  else if (g.n == 16 && g.m % 16 == 0 && al) launch_grad_a_lam<2>(g, h_bf16, grad_a_bf16, grid, stream);
  else launch_grad_a_lam<0>(g, h_bf16, grad_a_bf16, grid, stream);
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
