// element_scan.hip: element-scan kernels for gfx950.
//
// The three bodies are those of "Nonlinear element scans" (SexpGPU docs),
// introduction:
//   tanh-affine   h' = tanh(x + a * h)
//   norm-cap      y = a * h + x; h' = y / max(1, |y|)   (vector state)
//   max-plus      h' = max(h - c, x)
// Lanes are independent and trips are serial ("Storage and execution").
//
// Kernels here:
//   es_lane_kernel<BODY>   one thread per lane, trips in sequence, loads of
//                          the next block of trips issued before the current
//                          block is computed. Scalar states, and vector
//                          states of the element-wise bodies (each component
//                          is its own lane).
//   es_normcap_row_kernel  one 16-thread DPP row per lane, one state
//                          component per thread; |y|^2 is reduced across the
//                          row with DPP moves.
#include "sx_common.hpp"

namespace sx {
namespace {

// tanh(z) = 1 - 2 / (e^{2z} + 1), with e^{2z} = 2^{z * 2/ln 2} from the
// hardware base-2 exponential and the hardware reciprocal. Saturates
// correctly: e^{2z} -> inf gives 1, e^{2z} -> 0 gives -1. Absolute error is a
// few 1e-8 (one rounding each in the scale, exp2, add and reciprocal).
__device__ __forceinline__ float tanh_f32(float z) {
  const float e = __builtin_amdgcn_exp2f(z * 2.8853900817779268f);
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
}

template <int BODY>
__device__ __forceinline__ float elementwise_body(float h, float x, float s) {
  if constexpr (BODY == SX_BODY_TANH_AFFINE) {
    return tanh_f32(fmaf(s, h, x));
  } else {
    // exact: one correctly rounded subtraction and a maximum
    return fmaxf(h - s, x);
  }
}

template <int BODY>
__global__ __launch_bounds__(64) void es_lane_kernel(const EsParams p) {
  const int64_t lane = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (lane >= p.num_lanes) return;
  int64_t off[4];
  index_offsets(p.lanes, lane, off);
  const int64_t T = p.T;
  int64_t dx = p.t_stride[ES_X], ds = p.t_stride[ES_S], dout = p.t_stride[ES_OUT];
  const float* xp = p.x + off[ES_X];
  const float* sp = p.s + off[ES_S];
  float* op = p.out + off[ES_OUT];
  if (p.reverse) {
    xp += (T - 1) * dx;
    sp += (T - 1) * ds;
    op += (T - 1) * dout;
    dx = -dx;
    ds = -ds;
    dout = -dout;
  }
  float h = p.init[off[ES_INIT]];

  constexpr int U = 8;
  const int64_t full = T / U * U;
  float cx[U], cs[U];
  if (full > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      cx[u] = xp[u * dx];
      cs[u] = sp[u * ds];
    }
  }
  for (int64_t t = 0; t < full; t += U) {
    float nx[U], ns[U];
    const bool more = t + U < full;
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        nx[u] = xp[(U + u) * dx];
        ns[u] = sp[(U + u) * ds];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      h = elementwise_body<BODY>(h, cx[u], cs[u]);
      op[u * dout] = h;
    }
    xp += U * dx;
    sp += U * ds;
    op += U * dout;
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        cx[u] = nx[u];
        cs[u] = ns[u];
      }
    }
  }
  for (int64_t t = full; t < T; ++t) {
    h = elementwise_body<BODY>(h, *xp, *sp);
    *op = h;
    xp += dx;
    sp += ds;
    op += dout;
  }
}

// DPP move within a 16-lane row; CTRL is the gfx9 dpp_ctrl encoding.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the same
// bits (each step adds two values in either order, and addition commutes).
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]: pairs
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]: quads
  v += dpp_f32<0x141>(v);  // row_half_mirror: halves of 8
  v += dpp_f32<0x140>(v);  // row_mirror: the row of 16
  return v;
}

// One trip of the norm-capped body for this thread's component.
// h / max(1, sqrt(ss)) is h * min(1, rsqrt(ss)): rsqrt(ss) >= 1 exactly when
// ss <= 1, and ss = 0 gives +inf, so the factor is 1 there.
__device__ __forceinline__ float norm_cap_trip(float h, float x, float a) {
  const float y = fmaf(a, h, x);
  const float ss = row_sum16(y * y);
  return y * fminf(1.0f, __builtin_amdgcn_rsqf(ss));
}

__global__ __launch_bounds__(256) void es_normcap_row_kernel(const EsParams p) {
  const int64_t gtid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t lane = gtid >> 4;
  // A whole row (one lane) leaves together, so no DPP read crosses into an exited row.
  if (lane >= p.num_lanes) return;
  const int k = int(threadIdx.x & 15);
  const bool active = k < p.n;
  int64_t off[4];
  index_offsets(p.lanes, lane, off);
  const int64_t T = p.T;
  int64_t dx = p.t_stride[ES_X], ds = p.t_stride[ES_S], dout = p.t_stride[ES_OUT];
  const int kk = active ? k : 0;
  const float* xp = p.x + off[ES_X] + kk * p.n_stride[ES_X];
  const float* sp = p.s + off[ES_S] + kk * p.n_stride[ES_S];
  float* op = p.out + off[ES_OUT] + kk * p.n_stride[ES_OUT];
  if (p.reverse) {
    xp += (T - 1) * dx;
    sp += (T - 1) * ds;
    op += (T - 1) * dout;
    dx = -dx;
    ds = -ds;
    dout = -dout;
  }
  float h = active ? p.init[off[ES_INIT] + kk * p.n_stride[ES_INIT]] : 0.0f;

  constexpr int U = 4;
  const int64_t full = T / U * U;
  float cx[U], ca[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    cx[u] = (full > 0 && active) ? xp[u * dx] : 0.0f;
    ca[u] = (full > 0 && active) ? sp[u * ds] : 0.0f;
  }
  for (int64_t t = 0; t < full; t += U) {
    float nx[U], na[U];
    const bool more = t + U < full && active;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      nx[u] = more ? xp[(U + u) * dx] : 0.0f;
      na[u] = more ? sp[(U + u) * ds] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      h = norm_cap_trip(h, cx[u], ca[u]);
      if (active) op[u * dout] = h;
    }
    xp += U * dx;
    sp += U * ds;
    op += U * dout;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      cx[u] = nx[u];
      ca[u] = na[u];
    }
  }
  for (int64_t t = full; t < T; ++t) {
    const float xv = active ? *xp : 0.0f;
    const float av = active ? *sp : 0.0f;
    h = norm_cap_trip(h, xv, av);
    if (active) *op = h;
    xp += dx;
    sp += ds;
    op += dout;
  }
}

}  // namespace

size_t element_scan_workspace(sx_body, const EsParams&) { return 0; }

hipError_t launch_element_scan(sx_body body, const EsParams& p, hipStream_t stream) {
  if (p.num_lanes <= 0) return hipSuccess;
  if (body == SX_BODY_NORM_CAP) {
    const int64_t blocks = (p.num_lanes * 16 + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(es_normcap_row_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, p);
  } else {
    const int64_t blocks = (p.num_lanes + 63) / 64;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (body == SX_BODY_TANH_AFFINE)
      hipLaunchKernelGGL(es_lane_kernel<SX_BODY_TANH_AFFINE>, dim3(unsigned(blocks)), dim3(64), 0, stream, p);
    else
      hipLaunchKernelGGL(es_lane_kernel<SX_BODY_MAX_PLUS>, dim3(unsigned(blocks)), dim3(64), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace sx
