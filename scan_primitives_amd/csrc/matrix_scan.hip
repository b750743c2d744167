// matrix_scan.hip: matrix-scan kernels for gfx950.
//
// "Tensor operations" (SexpGPU docs), Operations table (matrix-scan row) and
// the "matrix-scan" section: h[t] = a[t] @ h[t-1] + b[t] from h = 0, one
// matrix product a step, computed in f32 (bf16 operands widen exactly);
// :reverse runs from the end, h[t] = a[t] @ h[t+1] + b[t] from h[T] = 0.
//
// Kernels here:
//   ms_serial_kernel  one 256-thread block per (batch, 16-column tile of m):
//                     thread (i, j) owns h[i][j]; every step stages a[t] in
//                     LDS and forms row i of a[t] @ h with a k-ordered FMA
//                     chain. Serial in time: correct for every shape, and the
//                     baseline the chunked kernels are checked against.
#include "sx_common.hpp"

namespace sx {
namespace {

__device__ __forceinline__ float load_elem(const float* p) { return *p; }
__device__ __forceinline__ float load_elem(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_elem(uint16_t* p, float v) { *p = f32_to_bf16_rne(v); }

template <typename TIn, typename TOut>
__global__ __launch_bounds__(256) void ms_serial_kernel(const MsParams p) {
  const int col_tiles = (p.m + 15) / 16;
  const int64_t batch = int64_t(blockIdx.x) / col_tiles;
  const int ct = int(int64_t(blockIdx.x) % col_tiles);
  const int i = int(threadIdx.x) >> 4, j = int(threadIdx.x) & 15;
  const int n = p.n, m = p.m;
  const int col = ct * 16 + j;
  const bool in_a = i < n && j < n;
  const bool in_h = i < n && col < m;

  __shared__ float sa[16][17];
  __shared__ float sh[16][17];
  sh[i][j] = 0.0f;

  int64_t off[3];
  index_offsets(p.batch, batch, off);
  const int64_t T = p.T;
  int64_t da = p.t_stride[MS_A], db = p.t_stride[MS_B], dout = p.t_stride[MS_OUT];
  const TIn* ap = static_cast<const TIn*>(p.a) + off[MS_A] + (in_a ? i * n + j : 0);
  const TIn* bp = static_cast<const TIn*>(p.b) + off[MS_B] + (in_h ? int64_t(i) * m + col : 0);
  TOut* op = static_cast<TOut*>(p.out) + off[MS_OUT] + (in_h ? int64_t(i) * m + col : 0);
  if (p.reverse) {
    ap += (T - 1) * da;
    bp += (T - 1) * db;
    op += (T - 1) * dout;
    da = -da;
    db = -db;
    dout = -dout;
  }
  float an = in_a ? load_elem(ap) : 0.0f;
  float bn = in_h ? load_elem(bp) : 0.0f;
  for (int64_t t = 0; t < T; ++t) {
    const float av = an, bv = bn;
    if (t + 1 < T) {  // next step's operands, loaded ahead of this step's product
      an = in_a ? load_elem(ap + da) : 0.0f;
      bn = in_h ? load_elem(bp + db) : 0.0f;
    }
    sa[i][j] = av;
    __syncthreads();
    float acc = bv;
    for (int k = 0; k < n; ++k) acc = fmaf(sa[i][k], sh[k][j], acc);
    __syncthreads();
    sh[i][j] = acc;
    if (in_h) store_elem(op, acc);
    ap += da;
    bp += db;
    op += dout;
  }
}

template <typename TIn, typename TOut>
hipError_t launch_serial(const MsParams& p, hipStream_t stream) {
  const int64_t blocks = p.num_batch * ((p.m + 15) / 16);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((ms_serial_kernel<TIn, TOut>), dim3(unsigned(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t matrix_scan_workspace(const MsParams&) { return 0; }

hipError_t launch_matrix_scan(const MsParams& p, void* /*workspace*/, size_t /*workspace_bytes*/,
                              hipStream_t stream) {
  if (p.num_batch <= 0 || p.T <= 0) return hipSuccess;
  if (p.in_bf16) {
    return p.out_bf16 ? launch_serial<uint16_t, uint16_t>(p, stream) : launch_serial<uint16_t, float>(p, stream);
  }
  return p.out_bf16 ? launch_serial<float, uint16_t>(p, stream) : launch_serial<float, float>(p, stream);
}

}  // namespace sx
