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
//   es_normcap_chunk_kernel the norm-capped body split along the axis into
//                          chunks that run at once. The body is not
//                          associative but it contracts: a chunk starts W
//                          trips early from h = 0, with W chosen so that the
//                          product of per-trip Lipschitz bounds certifies the
//                          warm-up's distance to the true state below 2^-26
//                          (or W reaching back to the start of the axis,
//                          which is then exact). See norm_cap_lipschitz.
//   es_slab_kernel<BODY>   max-plus (and linear-scan) as a chunked associative
//                          scan. A max-plus trip is the map h -> max(h - c, x);
//                          maps of that form compose into max(h + P, Q) (a
//                          linear trip h -> a h + b composes into P h + Q).
//                          One workgroup of NW waves owns 64 lanes and
//                          sweeps the scan axis in slabs of NW*S trips: each
//                          wave summarises its S
//                          trips into (P, Q), the summaries meet in LDS, each
//                          wave takes its entering state by composing the
//                          summaries before it onto the slab's carry, and
//                          replays its trips from there. The next slab's
//                          loads are in flight meanwhile. Inputs are read
//                          once and no state leaves the workgroup.
#include <algorithm>
#include <type_traits>
#include <utility>

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
  } else if constexpr (BODY == kBodyLinear) {
    return fmaf(s, h, x);  // linear-scan: a * h + b, with b as x and a as s
  } else {
    // exact: one correctly rounded subtraction and a maximum
    return fmaxf(h - s, x);
  }
}

// Element access for the kernels linear-scan shares: f32 or bf16 (uint16_t)
// elements, widened to f32 on load and rounded to nearest even on a bf16 store.
__device__ __forceinline__ float ld_elem(const float* p) { return ld_stream(p); }
__device__ __forceinline__ float ld_elem(const uint16_t* p) { return bf16_to_f32(ld_stream(p)); }
__device__ __forceinline__ void st_elem(float* p, float v) { *p = v; }
__device__ __forceinline__ void st_elem(uint16_t* p, float v) { *p = f32_to_bf16_rne(v); }
__device__ __forceinline__ void st_elem_stream(float* p, float v) { st_stream(p, v); }
__device__ __forceinline__ void st_elem_stream(uint16_t* p, float v) { st_stream(p, f32_to_bf16_rne(v)); }

// TI, TO: element types of the sequences and of out (float unless linear-scan).
// IDX32: every lane offset fits 32 bits (the host checks), so the lane's
// offsets come from 32-bit divisions instead of 64-bit ones, whose expansion
// costs a short lane a large share of its time.
template <int BODY, typename TI = float, typename TO = float, bool IDX32 = false>
__global__ __launch_bounds__(64) void es_lane_kernel(const EsParams p) {
  const int64_t lane = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (lane >= p.num_lanes) return;
  int64_t off[4];
  if constexpr (IDX32) index_offsets32(p.lanes, uint32_t(lane), off);
  else index_offsets(p.lanes, lane, off);
  const int64_t T = p.T;
  int64_t dx = p.t_stride[ES_X], ds = p.t_stride[ES_S], dout = p.t_stride[ES_OUT];
  const TI* xp = reinterpret_cast<const TI*>(p.x) + off[ES_X];
  const TI* sp = reinterpret_cast<const TI*>(p.s) + off[ES_S];
  TO* op = reinterpret_cast<TO*>(p.out) + off[ES_OUT];
  if (p.reverse) {
    xp += (T - 1) * dx;
    sp += (T - 1) * ds;
    op += (T - 1) * dout;
    dx = -dx;
    ds = -ds;
    dout = -dout;
  }
  float h = p.init ? p.init[off[ES_INIT]] : 0.0f;  // no initial: linear-scan starts from zero

  constexpr int U = 16;  // trips per block of loads (8-trip blocks left more of each block's load latency exposed)
  const int64_t full = T / U * U;
  float cx[U], cs[U];
  if (full > 0) {
#pragma unroll
    for (int u = 0; u < U; ++u) cx[u] = ld_elem(xp + u * dx);  // grouped by tensor, as the slab kernels load
#pragma unroll
    for (int u = 0; u < U; ++u) cs[u] = ld_elem(sp + u * ds);
  }
  for (int64_t t = 0; t < full; t += U) {
    float nx[U], ns[U];
    const bool more = t + U < full;
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) nx[u] = ld_elem(xp + (U + u) * dx);
#pragma unroll
      for (int u = 0; u < U; ++u) ns[u] = ld_elem(sp + (U + u) * ds);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      h = elementwise_body<BODY>(h, cx[u], cs[u]);
      st_elem(op + u * dout, h);
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
    h = elementwise_body<BODY>(h, ld_elem(xp), ld_elem(sp));
    st_elem(op, h);
    xp += dx;
    sp += ds;
    op += dout;
  }
}

// Lane N of each 16-lane row, broadcast to the whole row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x150 + N, 0xF, 0xF, false));
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


// Maximum over the 16 lanes of a DPP row, every lane of the row gets it.
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  return v;
}

// A Lipschitz bound of one norm-capped trip h -> P(a*h + x), P the projection
// onto the closed unit ball, over states h in that ball (every state after a
// trip is in it). a*h moves by at most alpha = max|a_i| times |h - h'|; P is
// nonexpansive; and when every reachable y = a*h + x has |y| >= r = |x| - alpha
// > 1, P(y) = y/|y| moves by at most |y - y'| / r (Dunkl-Williams in an inner
// product space: |u/|u| - v/|v|| <= 2|u - v| / (|u| + |v|)). So
// L = alpha / max(1, |x| - alpha). The reductions run across the whole DPP
// row (lanes past n hold zeros; a broadcast gate is read by every lane), so
// all lanes of a row get the same bits and decide together. The hardware
// square root and reciprocal are within 1 ulp each; the few-ulp error of the
// product is far inside the margin between the target 2^-26 and the f32
// rounding (about 2^-24 of |h| <= 1) it protects. Non-finite inputs give a
// non-finite L, which never certifies.
__device__ __forceinline__ float norm_cap_lipschitz(float x, float a, bool scalar_gate) {
  const float xn = __builtin_amdgcn_sqrtf(row_sum16(x * x));
  const float al = scalar_gate ? fabsf(a) : row_max16(fabsf(a));
  return al * __builtin_amdgcn_rcpf(fmaxf(1.0f, xn - al));
}

constexpr float kWarmupBound = 1.0f / 67108864.0f;  // 2^-26, far below f32 rounding of |h| <= 1

// One DPP row (16 threads) per (lane, chunk). Positions are in scan order
// (time T-1-q when reversed). The chunk covers positions [s, e); the row runs
// positions [start, e) and stores [s, e), where start <= s is the warm-up
// start certified by the walk back from s, or 0 (exact, from `initial`).
// Fast path: chunks of at most kChunkFast trips whose warm-up certifies within
// kWarmFast trips run entirely from one batch of loads covering
// [s - kWarmFast, s + kChunkFast).
constexpr int kWarmFast = 24;
constexpr int kChunkFast = 16;

template <bool SCALAR_GATE>
__global__ __launch_bounds__(256) void es_normcap_chunk_kernel(const EsParams p, int64_t chunk_len, int64_t nchunks) {
  const int64_t row = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 4;
  // A whole row leaves together, so no DPP read crosses into an exited row.
  if (row >= p.num_lanes * nchunks) return;
  const int64_t chunk = row / p.num_lanes;
  const int64_t lane = row % p.num_lanes;
  const int k = int(threadIdx.x & 15);
  const bool active = k < p.n;
  const int kk = active ? k : 0;
  int64_t off[4];
  index_offsets(p.lanes, lane, off);
  const float* xl = p.x + off[ES_X] + kk * p.n_stride[ES_X];
  const float* al = p.s + off[ES_S] + kk * p.n_stride[ES_S];
  float* ol = p.out + off[ES_OUT] + kk * p.n_stride[ES_OUT];
  const int64_t sx = p.t_stride[ES_X], sa = p.t_stride[ES_S], so = p.t_stride[ES_OUT];
  const int64_t T = p.T;
  const bool rev = p.reverse != 0;
  auto time_of = [&](int64_t q) -> int64_t {  // clamped into [0, T): loads always read a valid element
    q = q < 0 ? 0 : (q >= T ? T - 1 : q);
    return rev ? T - 1 - q : q;
  };
  const int64_t s = chunk * chunk_len;
  const int64_t e = s + chunk_len < T ? s + chunk_len : T;
  const float h0 = active ? p.init[off[ES_INIT] + kk * p.n_stride[ES_INIT]] : 0.0f;
  constexpr bool scalar_gate = SCALAR_GATE;  // a width-one gate: every lane reads the same value

  if (chunk_len <= kChunkFast) {
    // ---- one batch of loads: buffer slot i holds position s - kWarmFast + i.
    // A width-one gate is the same for the whole row, so the row keeps one copy:
    // lane j of the row holds slot 16 g + j in register g, and a trip takes it
    // with a row broadcast. That keeps the kernel at two waves per SIMD.
    auto fast = [&](auto scalar_c) -> bool {
      constexpr bool kScalar = decltype(scalar_c)::value;
      constexpr int kSlots = kWarmFast + kChunkFast;
      constexpr int kGateRegs = kScalar ? (kSlots + 15) / 16 : kSlots;
      const int64_t q_first = s - kWarmFast;
      float xv[kSlots], gv[kGateRegs];
#pragma unroll
      for (int i = 0; i < kSlots; ++i) {
        const float xr = xl[time_of(q_first + i) * sx];
        xv[i] = active ? xr : 0.0f;
      }
#pragma unroll
      for (int g = 0; g < kGateRegs; ++g) {
        if constexpr (kScalar) {
          gv[g] = al[time_of(q_first + 16 * g + k) * sa];
        } else {
          const float ar = al[time_of(q_first + g) * sa];
          gv[g] = active ? ar : 0.0f;
        }
      }
      auto gate = [&](auto i_c) -> float {
        constexpr int i = decltype(i_c)::value;
        if constexpr (kScalar) return row_bcast<i % 16>(gv[i / 16]);
        else return gv[i];
      };
      // walk back from s - 1 (slot kWarmFast - 1) while the bound is above the target
      int first = -1;  // slot of the certified warm-up start
      bool exact = false;
      if (s == 0) {
        first = kWarmFast;
        exact = true;
      } else {
        // the per-trip bounds do not depend on h: form them all at once, then walk
        float lip[kWarmFast];
        [&]<int... is>(std::integer_sequence<int, is...>) {
          ((lip[is] = norm_cap_lipschitz(xv[is], gate(std::integral_constant<int, is>{}), kScalar)), ...);
        }(std::make_integer_sequence<int, kWarmFast>{});
        float prod = 1.0f;
#pragma unroll
        for (int i = kWarmFast - 1; i >= 0; --i) {
          if (first < 0) {  // row-uniform
            if (s - kWarmFast + i < 0) {
              first = i + 1;  // reached the start of the axis
              exact = true;
            } else {
              prod *= lip[i];
              if (prod <= kWarmupBound) first = i;
            }
          }
        }
      }
      if (first < 0) return false;
      float h = exact ? h0 : 0.0f;
      float* op = ol + time_of(s) * so;
      const int64_t dout = rev ? -so : so;
      [&]<int... is>(std::integer_sequence<int, is...>) {
        (([&] {
           const int64_t q = s - kWarmFast + is;
           if (is >= first && q < e) {  // row-uniform
             h = norm_cap_trip(h, xv[is], gate(std::integral_constant<int, is>{}));
             if (is >= kWarmFast && active) op[(is - kWarmFast) * dout] = h;
           }
         }()),
         ...);
      }(std::make_integer_sequence<int, kSlots>{});
      return true;
    };
    if (fast(std::integral_constant<bool, SCALAR_GATE>{})) return;
  }

  // ---- general path: walk back eight positions per round until certified, then run forward
  int64_t start = 0;
  if (s > 0) {
    float prod = 1.0f;
    int64_t q = s - 1;
    bool done = false;
    while (!done) {  // row-uniform: every lane of the row computes the same bound
      float xv[8], av[8];
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const int64_t t = time_of(q - g);
        const float xr = xl[t * sx], ar = al[t * sa];
        xv[g] = active ? xr : 0.0f;
        av[g] = active || scalar_gate ? ar : 0.0f;
      }
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        if (!done) {
          if (q - g < 0) {
            start = 0;  // reached the start of the axis: run exactly from `initial`
            done = true;
          } else {
            prod *= norm_cap_lipschitz(xv[g], av[g], scalar_gate);
            if (prod <= kWarmupBound) {
              start = q - g;
              done = true;
            }
          }
        }
      }
      q -= 8;
    }
  }
  float h = start == 0 ? h0 : 0.0f;  // from `initial` at position 0, else from 0 (in the unit ball)
  constexpr int U = 8;
  for (int64_t q0 = start; q0 < e; q0 += U) {
    float xv[U], av[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t t = time_of(q0 + u < e ? q0 + u : e - 1);
      const float xr = xl[t * sx], ar = al[t * sa];
      xv[u] = active ? xr : 0.0f;
      av[u] = active ? ar : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t q = q0 + u;
      if (q < e) {  // row-uniform
        h = norm_cap_trip(h, xv[u], av[u]);
        if (active && q >= s) ol[time_of(q) * so] = h;
      }
    }
  }
}

// Trips whose maps compose in closed form. Max-plus: h -> max(h - c, x), and
// a run of them is h -> max(h + P, Q). Linear: h -> a h + b, and a run is
// h -> P h + Q. A trip past the end of the axis is the identity map.
template <int BODY>
struct SlabMap {
  static_assert(BODY == SX_BODY_MAX_PLUS || BODY == kBodyLinear, "no closed-form composition");
  static constexpr bool kMaxPlus = BODY == SX_BODY_MAX_PLUS;
  __device__ static float p0() { return kMaxPlus ? 0.0f : 1.0f; }  // the identity map (P, Q)
  __device__ static float q0() { return kMaxPlus ? -__builtin_huge_valf() : 0.0f; }
  __device__ static float x_pad() { return kMaxPlus ? -__builtin_huge_valf() : 0.0f; }  // x (b) of an identity trip
  __device__ static float s_pad() { return kMaxPlus ? 0.0f : 1.0f; }                     // c (a) of an identity trip
  // the map (P, Q) followed by the trip (x, s)
  __device__ static void fold(float& P, float& Q, float x, float s) {
    if constexpr (kMaxPlus) {
      Q = fmaxf(Q - s, x);
      P = P - s;
    } else {
      Q = fmaf(s, Q, x);
      P = P * s;
    }
  }
  __device__ static float apply(float P, float Q, float h) { return kMaxPlus ? fmaxf(h + P, Q) : fmaf(P, h, Q); }
};

// CS: the second sequence (c, or a) has time stride 0, so it is read once per
// lane rather than at every trip, and a slab holds only x in registers.
template <int BODY, int NW, int S, typename TI = float, typename TO = float, bool CS = false>
__global__ __launch_bounds__(NW * 64) void es_slab_kernel(const EsParams p) {
  using M = SlabMap<BODY>;
  __shared__ float sP[2][NW][64];  // per slab parity: each wave's map (P, Q)
  __shared__ float sQ[2][NW][64];
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);  // wave-uniform: index math stays scalar
  const int l = int(threadIdx.x) & 63;
  const int64_t lane = int64_t(blockIdx.x) * 64 + l;
  const bool live = lane < p.num_lanes;
  int64_t off[4];
  index_offsets(p.lanes, live ? lane : 0, off);
  const int64_t T = p.T;
  const TI* xl = reinterpret_cast<const TI*>(p.x) + off[ES_X];
  const TI* cl = reinterpret_cast<const TI*>(p.s) + off[ES_S];
  TO* ol = reinterpret_cast<TO*>(p.out) + off[ES_OUT];
  const int64_t sx = p.t_stride[ES_X], sc = p.t_stride[ES_S], so = p.t_stride[ES_OUT];
  const bool rev = p.reverse != 0;
  float carry = p.init ? p.init[off[ES_INIT]] : 0.0f;  // no initial: linear-scan starts from zero

  constexpr int64_t kSlab = int64_t(NW) * S;
  const int64_t nslabs = (T + kSlab - 1) / kSlab;
  // Scan position q is time q (forward) or T-1-q (reverse). Positions past the
  // end are identity trips. Loads always read a valid
  // element (the position clamped to the last one; a lane past the end reads
  // lane 0's and computes values it never stores), so no load sits behind a
  // branch and every load of a slab is in flight at once.
  auto time_of = [&](int64_t q) -> int64_t {
    const int64_t qc = q < T ? q : T - 1;
    return rev ? T - 1 - qc : qc;
  };
  const float c_once = CS ? ld_elem(cl) : 0.0f;
  // this wave's trips of the slab starting at position q_slab, into xs (and cs): every x, then every c
  // (grouped by tensor, the requests reach memory in fewer row runs: on one box 143.4 against 146.4 us on
  // max-plus [64,4096,256] and 143.2 against 147.0 on linear-scan, interleaved per trip before; on another,
  // this and the 8-trip slabs together took max-plus from 149.2 to 148.7 us)
  auto load = [&](int64_t q_slab, float (&xs)[S], float (&cs)[CS ? 1 : S]) {
#pragma unroll
    for (int k = 0; k < S; ++k) {
      const int64_t q = q_slab + int64_t(wave) * S + k;
      const float xv = ld_elem(xl + time_of(q) * sx);
      xs[k] = q < T ? xv : M::x_pad();
    }
    if constexpr (!CS) {
#pragma unroll
      for (int k = 0; k < S; ++k) {
        const int64_t q = q_slab + int64_t(wave) * S + k;
        const float cv = ld_elem(cl + time_of(q) * sc);
        cs[k] = q < T ? cv : M::s_pad();
      }
    }
  };
  float cx[S], cc[CS ? 1 : S];
  load(0, cx, cc);
  for (int64_t sl = 0; sl < nslabs; ++sl) {
    const int64_t qw = sl * kSlab + int64_t(wave) * S;  // this wave's first position in the slab
    float nx[S], nc[CS ? 1 : S];
    load((sl + 1) * kSlab, nx, nc);  // the next slab, in flight during this one
    // this slab's c at trip k
    auto c_of = [&](int k) -> float {
      if constexpr (CS) return qw + k < T ? c_once : M::s_pad();
      else return cc[k];
    };
    __builtin_amdgcn_sched_barrier(0);  // keep the next slab's loads issued ahead of this slab's work
    // summary of this wave's trips: their maps composed in scan order
    float P = M::p0(), Q = M::q0();
#pragma unroll
    for (int k = 0; k < S; ++k) M::fold(P, Q, cx[k], c_of(k));
    const int par = int(sl & 1);
    sP[par][wave][l] = P;
    sQ[par][wave][l] = Q;
    __syncthreads();
    // entering state of this wave, and the carry into the next slab (the same in every wave)
    float h = carry, hw = carry;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w == wave) hw = h;
      h = M::apply(sP[par][w][l], sQ[par][w][l], h);
    }
    carry = h;
    // replay from the entering state: each trip is the serial body again
#pragma unroll
    for (int k = 0; k < S; ++k) {
      hw = elementwise_body<BODY>(hw, cx[k], c_of(k));
      const int64_t q = qw + k;
      if (live && q < T) st_elem_stream(ol + time_of(q) * so, hw);
    }
#pragma unroll
    for (int k = 0; k < S; ++k) {
      cx[k] = nx[k];
      if constexpr (!CS) cc[k] = nc[k];
    }
  }
}
// ------------------------------------------------------------------ gradients
//
// The gradient of sum(g * out) runs the trips last to first (in scan order).
// With lam the adjoint of the state a trip produced (g there plus what the
// trip after passed back), each trip's chain rule gives its sequences'
// gradients and the adjoint of the state it started from, hp:
//   tanh-affine  dz = lam (1 - h^2): grad_x = dz, grad_s = dz hp, to hp s dz
//   max-plus     x won (x >= hp - c, ties to x): grad_x = lam, grad_c = 0, to hp 0;
//                else grad_x = 0, grad_c = -lam, to hp lam
//   norm-cap     y = s hp + x; capped (|y| > 1): dy = (lam - u (u . lam)) / |y|
//                with u = y / |y|; else dy = lam: grad_x = dy, grad_s = dy hp,
//                to hp s dy
// For the scalar bodies the adjoint reaching hp is A lam, A = s (1 - h^2) or
// [the carry won], and each gradient is lam times a factor of the trip's own:
// so nu (the adjoint passed to a trip's incoming state) follows the linear
// recurrence nu_q = A_q nu_{q+1} + A_q g_q, scanned like linear-scan, and the
// trip's lam is g_q + nu_{q+1}. The branch decisions use f32 values as the
// forward pass computed them.

// A trip of a scalar body's gradient, reduced to what the sweep needs.
struct VjpTrip {
  float a;   // A: the adjoint reaching hp is a * lam
  float g;   // g at this trip
  float kx;  // grad_x = kx * lam
  float ks;  // grad_s = ks * lam
};

template <int BODY>
__device__ __forceinline__ VjpTrip vjp_trip(float h, float hp, float x, float s, float g) {
  VjpTrip v;
  v.g = g;
  if constexpr (BODY == SX_BODY_TANH_AFFINE) {
    const float d = 1.0f - h * h;
    v.a = s * d;
    v.kx = d;
    v.ks = d * hp;
  } else {
    const bool x_won = x >= hp - s;
    v.a = x_won ? 0.0f : 1.0f;
    v.kx = x_won ? 1.0f : 0.0f;
    v.ks = x_won ? 0.0f : -1.0f;
  }
  return v;
}

// One thread per lane, trips last to first in scan order. Forward scan
// position q is time tq(q); the state before it is h at position q - 1
// (initial at q = 0). Loads of a block of U trips are issued before any of
// its trips is computed.
template <int BODY, bool IDX32 = false>  // IDX32: as in es_lane_kernel
__global__ __launch_bounds__(64) void es_vjp_lane_kernel(const EsVjpParams v) {
  const EsParams& p = v.p;
  const int64_t lane = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (lane >= p.num_lanes) return;
  int64_t off[4];
  if constexpr (IDX32) index_offsets32(p.lanes, uint32_t(lane), off);
  else index_offsets(p.lanes, lane, off);
  const int64_t T = p.T;
  const int64_t sx = p.t_stride[ES_X], ss = p.t_stride[ES_S], so = p.t_stride[ES_OUT];
  const float* xl = p.x + off[ES_X];
  const float* sl = p.s + off[ES_S];
  const float* hl = v.h + off[ES_OUT];
  const float* gl = v.g + off[ES_OUT];
  float* gxl = v.gx + off[ES_OUT];
  float* gsl = v.gs + off[ES_OUT];
  const float init = p.init[off[ES_INIT]];
  auto tq = [&](int64_t q) -> int64_t { return p.reverse ? T - 1 - q : q; };
  // blocks of U trips (q1, q1 - 1, ...), block i + 1's loads in flight while block i is computed
  constexpr int U = 8;
  struct Block {
    float h[U], hp[U], x[U], s[U], g[U];
  };
  auto load = [&](int64_t q1, Block& B) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t q = q1 - u >= 0 ? q1 - u : 0;  // clamped: every load is valid
      const int64_t t = tq(q);
      B.hp[u] = hl[tq(q > 0 ? q - 1 : 0) * so];  // unconditional; initial is selected at the trip
      B.h[u] = hl[t * so];
      B.x[u] = xl[t * sx];
      B.s[u] = sl[t * ss];
      B.g[u] = gl[t * so];
    }
  };
  float nu = 0.0f;
  Block cur, nxt;
  load(T - 1, cur);
  for (int64_t q1 = T - 1; q1 >= 0; q1 -= U) {
    load(q1 - U, nxt);  // always (clamped positions): a load behind a branch would cost a full wait
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (q1 - u >= 0) {
        const VjpTrip tr = vjp_trip<BODY>(cur.h[u], q1 - u > 0 ? cur.hp[u] : init, cur.x[u], cur.s[u], cur.g[u]);
        const int64_t t = tq(q1 - u);
        const float lam = tr.g + nu;
        gxl[t * so] = tr.kx * lam;
        gsl[t * so] = tr.ks * lam;
        nu = tr.a * lam;
      }
    }
    cur = nxt;
  }
  v.ginit[off[ES_INIT]] = nu;
}

// The scalar bodies' gradient as a chunked associative scan over the sweep
// (the trips last to first): the adjoint map of a trip, nu -> A nu + A g,
// composes like a linear-scan trip. One workgroup of NW waves owns 64 lanes;
// each slab of NW*S trips is summarised per wave, the summaries meet in LDS,
// each wave composes the ones before it onto the slab's carry, and replays
// its trips storing both gradients. The next slab's loads are in flight
// meanwhile. Sweep position w is scan position T - 1 - w.
template <int BODY, int NW, int S, bool IDX32 = false>  // IDX32: as in es_lane_kernel
__global__ __launch_bounds__(NW * 64) void es_vjp_slab_kernel(const EsVjpParams v) {
  const EsParams& p = v.p;
  __shared__ float sP[2][NW][64];
  __shared__ float sQ[2][NW][64];
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  const int l = int(threadIdx.x) & 63;
  const int64_t lane = int64_t(blockIdx.x) * 64 + l;
  const bool live = lane < p.num_lanes;
  int64_t off[4];
  if constexpr (IDX32) index_offsets32(p.lanes, uint32_t(live ? lane : 0), off);
  else index_offsets(p.lanes, live ? lane : 0, off);
  const int64_t T = p.T;
  const int64_t sx = p.t_stride[ES_X], ss = p.t_stride[ES_S], so = p.t_stride[ES_OUT];
  const float* xl = p.x + off[ES_X];
  const float* sl = p.s + off[ES_S];
  const float* hl = v.h + off[ES_OUT];
  const float* gl = v.g + off[ES_OUT];
  float* gxl = v.gx + off[ES_OUT];
  float* gsl = v.gs + off[ES_OUT];
  const float init = p.init[off[ES_INIT]];
  // sweep position w -> time; positions past the end are clamped for loading and become identity trips
  auto time_of = [&](int64_t w) -> int64_t {
    const int64_t q = T - 1 - (w < T ? w : T - 1);
    return p.reverse ? T - 1 - q : q;
  };
  // this wave's S trips from sweep position w_first: h and the state before each trip (the two
  // h loads of a trip side by side), then every x, every s and every g, grouped by tensor
  // (max-plus [64,4096,256] 260.4 -> 256.8 us, tanh-affine [4,64,32] 5.46 -> 5.02 us against one
  // trip's five loads at a time)
  auto load_slab = [&](int64_t w_first, float (&raw)[S][5]) {
#pragma unroll
    for (int k = 0; k < S; ++k) {
      raw[k][0] = ld_stream(hl + time_of(w_first + k) * so);
      const float hr = hl[time_of(w_first + k + 1) * so];  // clamped position, unconditional load
      raw[k][1] = w_first + k + 1 < T ? hr : init;            // the state before the trip
    }
#pragma unroll
    for (int k = 0; k < S; ++k) raw[k][2] = ld_stream(xl + time_of(w_first + k) * sx);
#pragma unroll
    for (int k = 0; k < S; ++k) raw[k][3] = ld_stream(sl + time_of(w_first + k) * ss);
#pragma unroll
    for (int k = 0; k < S; ++k) raw[k][4] = ld_stream(gl + time_of(w_first + k) * so);
  };
  constexpr int64_t kSlab = int64_t(NW) * S;
  const int64_t nslabs = (T + kSlab - 1) / kSlab;
  float carry = 0.0f;
  float nraw[S][5];
  load_slab(int64_t(wave) * S, nraw);
  for (int64_t sl_i = 0; sl_i < nslabs; ++sl_i) {
    const int64_t w0 = sl_i * kSlab + int64_t(wave) * S;
    VjpTrip tr[S];
#pragma unroll
    for (int k = 0; k < S; ++k) {
      tr[k] = vjp_trip<BODY>(nraw[k][0], nraw[k][1], nraw[k][2], nraw[k][3], nraw[k][4]);
      if (w0 + k >= T) tr[k] = VjpTrip{1.0f, 0.0f, 0.0f, 0.0f};  // identity trip
    }
    load_slab(w0 + kSlab, nraw);  // the next slab, in flight during this one
    __builtin_amdgcn_sched_barrier(0);
    float P = 1.0f, Q = 0.0f;  // this wave's trips composed: nu -> P nu + Q
#pragma unroll
    for (int k = 0; k < S; ++k) {
      Q = tr[k].a * (Q + tr[k].g);
      P = P * tr[k].a;
    }
    const int par = int(sl_i & 1);
    sP[par][wave][l] = P;
    sQ[par][wave][l] = Q;
    __syncthreads();
    float nu = carry, nw = carry;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w == wave) nw = nu;
      nu = fmaf(sP[par][w][l], nu, sQ[par][w][l]);
    }
    carry = nu;
#pragma unroll
    for (int k = 0; k < S; ++k) {
      const float lam = tr[k].g + nw;
      if (live && w0 + k < T) {
        const int64_t t = time_of(w0 + k);
        st_stream(gxl + t * so, tr[k].kx * lam);
        st_stream(gsl + t * so, tr[k].ks * lam);
      }
      nw = tr[k].a * lam;
    }
  }
  if (live && wave == 0) v.ginit[off[ES_INIT]] = carry;
}

// Norm-cap gradient. A trip starting from hp with y = s hp + x passes back
// dy = (lam - u (u . lam)) / |y| when |y| > 1 (u = y / |y|), else dy = lam,
// where lam is the trip's upstream gradient plus what the next trip passed
// back; grad_x = dy, grad_s = dy hp, and s dy goes on to the trip before. A
// width-one sequence under the vector state gets the sum over the row of its
// gradient, taken here by a row reduction (lanes past n contribute zero).
struct NcOut {
  float* gx;
  float* gs;
  int64_t gx_step, gs_step;  // elements per trip
  bool gx_sum, gs_sum;
  bool active;
  int k;
  // where this row's gradients go: full width in out's layout, or one value per trip
  __device__ NcOut(const EsVjpParams& v, const int64_t* off, int k_, bool active_) : active(active_), k(k_) {
    const EsParams& p = v.p;
    const int64_t so = p.t_stride[ES_OUT];
    const int kk = active ? k : 0;
    gx_sum = v.gx_sum != 0;
    gs_sum = v.gs_sum != 0;
    // out is contiguous with the state last, so its offsets are multiples of n
    gx = gx_sum ? v.gx + off[ES_OUT] / p.n : v.gx + off[ES_OUT] + kk;
    gs = gs_sum ? v.gs + off[ES_OUT] / p.n : v.gs + off[ES_OUT] + kk;
    gx_step = gx_sum ? so / p.n : so;
    gs_step = gs_sum ? so / p.n : so;
  }
  __device__ __forceinline__ void store(int64_t t, float dy, float hp) const {
    const float d = active ? dy : 0.0f, dh = active ? dy * hp : 0.0f;
    const float sx = gx_sum ? row_sum16(d) : d;  // uniform branches
    const float ss = gs_sum ? row_sum16(dh) : dh;
    if (gx_sum ? k == 0 : active) gx[t * gx_step] = sx;
    if (gs_sum ? k == 0 : active) gs[t * gs_step] = ss;
  }
};

// The trip's backward step; nu carries what goes on to the trip before.
__device__ __forceinline__ float nc_back_trip(float hp, float x, float s, float g, float& nu, bool active) {
  const float y = active ? fmaf(s, hp, x) : 0.0f;  // lanes past n hold zero
  const float ir = __builtin_amdgcn_rsqf(row_sum16(y * y));
  const float uy = y * ir;
  const float lam = g + nu;
  const float ul = row_sum16(uy * lam);
  const float dy = ir < 1.0f ? (lam - uy * ul) * ir : lam;  // capped when |y| > 1
  nu = active ? s * dy : 0.0f;
  return dy;
}

// One 16-lane DPP row per state vector, trips last to first.
__global__ __launch_bounds__(256) void es_vjp_normcap_row_kernel(const EsVjpParams v) {
  const EsParams& p = v.p;
  const int64_t gtid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t lane = gtid >> 4;
  if (lane >= p.num_lanes) return;  // a whole row leaves together
  const int k = int(threadIdx.x & 15);
  const bool active = k < p.n;
  const int kk = active ? k : 0;
  int64_t off[4];
  index_offsets(p.lanes, lane, off);
  const int64_t T = p.T;
  const int64_t sx = p.t_stride[ES_X], ss = p.t_stride[ES_S], so = p.t_stride[ES_OUT];
  const float* xl = p.x + off[ES_X] + kk * p.n_stride[ES_X];
  const float* sl = p.s + off[ES_S] + kk * p.n_stride[ES_S];
  const float* hl = v.h + off[ES_OUT] + kk;
  const float* gl = v.g + off[ES_OUT] + kk;
  const NcOut out(v, off, k, active);
  const float init = active ? p.init[off[ES_INIT] + kk * p.n_stride[ES_INIT]] : 0.0f;
  auto tq = [&](int64_t q) -> int64_t { return p.reverse ? T - 1 - q : q; };
  // Blocks of U trips, last to first; block i + 1's loads are issued before block i is
  // computed, so the trip chain does not wait on memory. Positions below 0 are clamped
  // for loading and skipped.
  constexpr int U = 8;  // 32 loads a block: the loads in flight stay countable by vmcnt (at most 63)
  struct Block {  // raw loads; the selects that depend on them wait until the trip is computed
    float hr[U], xv[U], sv[U], gv[U];
  };
  auto load = [&](int64_t q1, Block& B) {
#pragma unroll
    for (int u = 0; u < U; ++u) {  // clamped positions: every load is valid and none is behind a branch
      const int64_t q = q1 - u >= 0 ? q1 - u : 0;
      const int64_t t = tq(q);
      B.hr[u] = hl[tq(q > 0 ? q - 1 : 0) * so];
      B.xv[u] = xl[t * sx];
      B.sv[u] = sl[t * ss];
      B.gv[u] = gl[t * so];
    }
  };
  float nu = 0.0f;
  Block cur, nxt;
  load(T - 1, cur);
  for (int64_t q1 = T - 1; q1 >= 0; q1 -= U) {
    load(q1 - U, nxt);  // always (clamped positions): a load behind a branch would cost a full wait
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (q1 - u >= 0) {  // row-uniform
        const float hp = q1 - u > 0 ? cur.hr[u] : init;  // the state before the trip (initial before the first)
        const float dy = nc_back_trip(hp, cur.xv[u], cur.sv[u], cur.gv[u], nu, active);
        out.store(tq(q1 - u), dy, hp);
      }
    }
    cur = nxt;
  }
  if (active) v.ginit[off[ES_INIT] + kk * p.n_stride[ES_INIT]] = nu;
}

// Norm-cap gradient split along the axis. The adjoint map of a trip,
// nu -> s (J^T nu) with J the Jacobian of the cap, has norm at most the
// forward trip's Lipschitz bound L = alpha / max(1, |x| - alpha) (the states
// are in the unit ball, so |y| >= |x| - alpha), and from nu = 0 before the
// last trip the adjoint stays within B = G L* / (1 - L*) (G the largest |g|
// of the lane, L* its largest L, when L* < 1). A chunk of the sweep may then
// start W trips early from nu = 0: its error entering the chunk is at most
// (product of the W bounds) * B, and W is chosen so that this is below 2^-26 G,
// far inside the f32 rounding of the gradients (which are at least of size G
// where g is). Lanes whose bounds reach 1 run exactly from the sweep's start.
// The bounds of the first trip of the scan assume |initial| <= 1, which may not
// hold; that trip only raises L* (it never lies inside a warm-up, which ends
// before the last trip of the sweep).

// Per state vector: G and L* (non-finite values become +inf: no certificate),
// and per chunk of the sweep the product of its trips' bounds, which lets a
// chunk find its warm-up start a whole chunk at a time. One workgroup per
// state vector; its R rows of 16 threads (R = blockDim.x / 16) take every
// R-th chunk, each in batches of 16 trips. bounds holds G, L* at 2 lane,
// 2 lane + 1 and the product of chunk c at 2 num_lanes + c num_lanes + lane.
template <bool S1>
__global__ __launch_bounds__(1024) void es_vjp_normcap_bound_kernel(const EsVjpParams v, int64_t len,
                                                                   int64_t nchunks) {
  const EsParams& p = v.p;
  const int64_t lane = blockIdx.x;
  const int R = int(blockDim.x >> 4), r = int(threadIdx.x >> 4);
  const int k = int(threadIdx.x & 15);
  const bool active = k < p.n;
  const int kk = active ? k : 0;
  int64_t off[4];
  index_offsets(p.lanes, lane, off);
  const int64_t T = p.T, sx = p.t_stride[ES_X], ss = p.t_stride[ES_S], so = p.t_stride[ES_OUT];
  const float* xl = p.x + off[ES_X] + kk * p.n_stride[ES_X];
  const float* sl = p.s + off[ES_S] + kk * p.n_stride[ES_S];
  const float* gl = v.g + off[ES_OUT] + kk;
  auto time_of_sweep = [&](int64_t w) -> int64_t {  // w in [0, T)
    const int64_t q = T - 1 - w;
    return p.reverse ? T - 1 - q : q;
  };
  float* prods = v.bounds + 2 * p.num_lanes + lane;
  float gmax = 0.0f, lmax = 0.0f;
  constexpr int U = 16;
  for (int64_t c = r; c < nchunks; c += R) {  // row-uniform
    const int64_t w_begin = c * len, w_end = w_begin + len < T ? w_begin + len : T;
    float prod = 1.0f;
    for (int64_t w0 = w_begin; w0 < w_end; w0 += U) {
      float xv[U], gv[U], sv[S1 ? 1 : U];
#pragma unroll
      for (int u = 0; u < U; ++u) {  // clamped positions: every load is valid
        const int64_t t = time_of_sweep(w0 + u < w_end ? w0 + u : w_end - 1);
        xv[u] = xl[t * sx];
        gv[u] = gl[t * so];
        if constexpr (!S1) sv[u] = sl[t * ss];
      }
      if constexpr (S1) sv[0] = sl[time_of_sweep(w0 + k < w_end ? w0 + k : w_end - 1) * ss];  // lane k: trip w0 + k
      [&]<int... us>(std::integer_sequence<int, us...>) {
        (([&] {
           constexpr int u = us;
           if (w0 + u < w_end) {  // row-uniform
             float a;
             if constexpr (S1) a = row_bcast<u>(sv[0]);
             else a = active ? sv[u] : 0.0f;
             const float l = norm_cap_lipschitz(active ? xv[u] : 0.0f, a, S1);
             const float ga = active ? gv[u] : 0.0f;
             const float gn = __builtin_amdgcn_sqrtf(row_sum16(ga * ga));
             prod *= l;
             lmax = l <= 3.0e38f ? fmaxf(lmax, l) : __builtin_huge_valf();  // NaN counts as unbounded
             gmax = gn <= 3.0e38f ? fmaxf(gmax, gn) : __builtin_huge_valf();
           }
         }()),
         ...);
      }(std::make_integer_sequence<int, U>{});
    }
    if (k == 0) prods[c * p.num_lanes] = prod;
  }
  __shared__ float red[2][64];
  if (k == 0) {
    red[0][r] = gmax;
    red[1][r] = lmax;
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    float m = 0.0f;
    for (int i = 0; i < R; ++i) m = fmaxf(m, red[threadIdx.x][i]);  // values are >= 0 or +inf
    v.bounds[2 * lane + threadIdx.x] = m;
  }
}

// One DPP row per (state vector, chunk of the sweep): the warm-up from nu = 0
// at the start of the latest earlier chunk from which the product of the
// chunks' bounds is below the target (or the sweep from its start), then the
// chunk's trips storing both gradients; the chunk that ends the sweep also
// stores grad_initial. Sweep position w is scan position T - 1 - w. The next
// block's loads are issued before a block is computed; a width-one gate is
// kept one trip per lane and taken by row broadcast.
template <bool S1>
__global__ __launch_bounds__(256) void es_vjp_normcap_chunk_kernel(const EsVjpParams v, int64_t len,
                                                                   int64_t nchunks) {
  const EsParams& p = v.p;
  const int64_t row = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 4;
  if (row >= p.num_lanes * nchunks) return;  // whole rows
  const int64_t chunk = row / p.num_lanes, lane = row % p.num_lanes;
  const int k = int(threadIdx.x & 15);
  const bool active = k < p.n;
  const int kk = active ? k : 0;
  int64_t off[4];
  index_offsets(p.lanes, lane, off);
  const int64_t T = p.T, sx = p.t_stride[ES_X], ss = p.t_stride[ES_S], so = p.t_stride[ES_OUT];
  const float* xl = p.x + off[ES_X] + kk * p.n_stride[ES_X];
  const float* sl = p.s + off[ES_S] + kk * p.n_stride[ES_S];
  const float* hl = v.h + off[ES_OUT] + kk;
  const float* gl = v.g + off[ES_OUT] + kk;
  const NcOut out(v, off, k, active);
  const float init = active ? p.init[off[ES_INIT] + kk * p.n_stride[ES_INIT]] : 0.0f;
  auto time_of_sweep = [&](int64_t w) -> int64_t {  // clamped into [0, T): every load reads a valid element
    w = w < 0 ? 0 : (w >= T ? T - 1 : w);
    const int64_t q = T - 1 - w;
    return p.reverse ? T - 1 - q : q;
  };
  const float gmax = v.bounds[2 * lane], lmax = v.bounds[2 * lane + 1];
  const int64_t s0 = chunk * len;
  int64_t e0 = s0 + len < T ? s0 + len : T;
  if (!(lmax < 1.0f) || !(gmax <= 3.0e38f)) {  // row-uniform: no certificate for this lane
    if (chunk != 0) return;  // the first chunk's row runs the lane's whole sweep exactly
    e0 = T;
  }
  // ---- the warm-up start: a whole chunk at a time, four chunk products per round
  int64_t start = 0;
  if (s0 > 0) {  // row-uniform (a lane without a certificate has s0 = 0 here)
    if (lmax == 0.0f || gmax == 0.0f) {
      start = s0;  // every adjoint map or every g is zero: nu is exactly zero entering the chunk
    } else {
      const float target = kWarmupBound * (1.0f - lmax) / lmax;
      const float* prods = v.bounds + 2 * p.num_lanes + lane;
      float prod = 1.0f;
      int64_t c = chunk - 1;
      bool done = false;
      while (!done) {
        float pv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) pv[u] = prods[(c - u >= 0 ? c - u : 0) * p.num_lanes];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (!done) {
            if (c - u < 0) {
              start = 0;  // reached the sweep's start: exact from there
              done = true;
            } else {
              prod *= pv[u];
              if (prod <= target) {
                start = (c - u) * len;
                done = true;
              }
            }
          }
        }
        c -= 4;
      }
    }
  }
  // ---- the sweep over [start, e0): trips before s0 only carry the adjoint
  constexpr int U = S1 ? 16 : 8;  // loads a block: 3 U + 1 or 4 U, countable by vmcnt (at most 63)
  struct Block {
    float hr[U], xv[U], gv[U], sv[S1 ? 1 : U];
  };
  auto load = [&](int64_t w0, Block& B) {
#pragma unroll
    for (int u = 0; u < U; ++u) {  // clamped positions: none behind a branch
      const int64_t w = w0 + u < e0 ? w0 + u : e0 - 1;
      const int64_t t = time_of_sweep(w);
      B.hr[u] = hl[time_of_sweep(w + 1) * so];  // the state before the trip (scan position one earlier)
      B.xv[u] = xl[t * sx];
      B.gv[u] = gl[t * so];
      if constexpr (!S1) B.sv[u] = sl[t * ss];
    }
    if constexpr (S1) B.sv[0] = sl[time_of_sweep(w0 + k < e0 ? w0 + k : e0 - 1) * ss];  // lane k: trip w0 + k
  };
  float nu = 0.0f;
  Block cur, nxt;
  load(start, cur);
  for (int64_t w0 = start; w0 < e0; w0 += U) {
    load(w0 + U, nxt);  // clamped: the last round loads valid elements it does not use
    [&]<int... us>(std::integer_sequence<int, us...>) {
      (([&] {
         constexpr int u = us;
         const int64_t w = w0 + u;
         if (w < e0) {  // row-uniform
           const float hp = w + 1 < T ? cur.hr[u] : init;  // the first trip of the scan starts from initial
           float sg;
           if constexpr (S1) sg = row_bcast<u>(cur.sv[0]);
           else sg = cur.sv[u];
           const float dy = nc_back_trip(hp, active ? cur.xv[u] : 0.0f, sg, cur.gv[u], nu, active);
           if (w >= s0) out.store(time_of_sweep(w), dy, hp);
         }
       }()),
       ...);
    }(std::make_integer_sequence<int, U>{});
    cur = nxt;
  }
  if (e0 == T && active) v.ginit[off[ES_INIT] + kk * p.n_stride[ES_INIT]] = nu;
}

}  // namespace

// The slab kernel wants about one 64-lane workgroup per CU (MI355X: 256) and
// at least a couple of slabs along the axis; below that the lane kernel is used.
constexpr int64_t kSlabMinLanes = 64 * 128;
// Norm-cap chunking: used below kChunkMaxLanes vector lanes (where one row per
// lane leaves most of the GPU idle), aiming at kChunkRows rows of at least
// kChunkMinLen trips each.
constexpr int64_t kChunkMaxLanes = 8192;
constexpr int64_t kChunkRows = 8192;
constexpr int64_t kChunkMinLen = 16;
constexpr int64_t kSlabMinTrips = 512;

size_t element_scan_workspace(sx_body, const EsParams&) { return 0; }

namespace {
// Lanes below 2^31 whose dims, strides and offsets (lane part) all lie below 2^31.
bool lane_offsets_fit32(const EsParams& p) {
  if (p.num_lanes >= (int64_t(1) << 31)) return false;
  for (int k = 0; k < 4; ++k) {
    int64_t span = 0;
    for (int d = 0; d < p.lanes.nd; ++d) {
      const int64_t st = p.lanes.st[k][d] < 0 ? -p.lanes.st[k][d] : p.lanes.st[k][d];
      if (p.lanes.dim[d] >= (int64_t(1) << 31) || st >= (int64_t(1) << 31)) return false;
      span += (p.lanes.dim[d] - 1) * st;
      if (span >= (int64_t(1) << 31)) return false;
    }
  }
  return true;
}
}  // namespace

hipError_t launch_element_scan(sx_body body, const EsParams& p, hipStream_t stream) {
  if (p.num_lanes <= 0) return hipSuccess;
  if (body == SX_BODY_NORM_CAP) {
    // a 16-wide state in aligned memory: four components per thread (normcap_quad.hip)
    if (normcap_quad_forward_eligible(p)) return launch_normcap_quad_forward(p, stream);
    if (p.num_lanes < kChunkMaxLanes && p.T >= 2 * kChunkMinLen) {
      // Few lanes: cut the axis into chunks so that about kChunkRows rows run at once.
      int64_t nchunks = (kChunkRows + p.num_lanes - 1) / p.num_lanes;
      int64_t len = (p.T + nchunks - 1) / nchunks;
      if (len < kChunkMinLen) len = kChunkMinLen;
      nchunks = (p.T + len - 1) / len;
      const int64_t blocks = (p.num_lanes * nchunks * 16 + 255) / 256;
      if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
      if (p.n_stride[ES_S] == 0)  // a width-one gate
        hipLaunchKernelGGL(es_normcap_chunk_kernel<true>, dim3(unsigned(blocks)), dim3(256), 0, stream, p, len, nchunks);
      else
        hipLaunchKernelGGL(es_normcap_chunk_kernel<false>, dim3(unsigned(blocks)), dim3(256), 0, stream, p, len, nchunks);
      return hipGetLastError();
    }
    const int64_t blocks = (p.num_lanes * 16 + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(es_normcap_row_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, p);
  } else {
    const int64_t blocks = (p.num_lanes + 63) / 64;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (body == SX_BODY_TANH_AFFINE) {
      if (lane_offsets_fit32(p))
        hipLaunchKernelGGL((es_lane_kernel<SX_BODY_TANH_AFFINE, float, float, true>), dim3(unsigned(blocks)), dim3(64),
                           0, stream, p);
      else
        hipLaunchKernelGGL(es_lane_kernel<SX_BODY_TANH_AFFINE>, dim3(unsigned(blocks)), dim3(64), 0, stream, p);
    } else if (p.num_lanes >= kSlabMinLanes && p.T >= kSlabMinTrips) {
      // enough 64-lane groups to give every CU a workgroup, and a long enough axis to pay for the summaries;
      // slabs of 8 trips a wave (measured on [64,4096,256], one box: 147.0 us against 149.7 with 16 trips,
      // 147.5 with 6, 155.4 with 4, 149.6 with 12, and 149.1 with 8 trips and two slabs in flight; the gain
      // differs from box to box, see the load order below)
      hipLaunchKernelGGL((es_slab_kernel<SX_BODY_MAX_PLUS, 16, 8>), dim3(unsigned(blocks)), dim3(16 * 64), 0, stream, p);
    } else if (lane_offsets_fit32(p)) {
      hipLaunchKernelGGL((es_lane_kernel<SX_BODY_MAX_PLUS, float, float, true>), dim3(unsigned(blocks)), dim3(64), 0,
                         stream, p);
    } else {
      hipLaunchKernelGGL(es_lane_kernel<SX_BODY_MAX_PLUS>, dim3(unsigned(blocks)), dim3(64), 0, stream, p);
    }
  }
  return hipGetLastError();
}

namespace {
template <typename TI, typename TO>
void launch_linear(const EsParams& p, int64_t blocks, hipStream_t stream) {
  if (p.num_lanes >= kSlabMinLanes && p.T >= kSlabMinTrips && p.t_stride[ES_S] == 0)  // a constant in time
    hipLaunchKernelGGL((es_slab_kernel<kBodyLinear, 16, 32, TI, TO, true>), dim3(unsigned(blocks)), dim3(16 * 64), 0,
                       stream, p);
  else if (p.num_lanes >= kSlabMinLanes && p.T >= kSlabMinTrips)  // 8 trips a wave, as max-plus (147.7 against 150.0 us)
    hipLaunchKernelGGL((es_slab_kernel<kBodyLinear, 16, 8, TI, TO>), dim3(unsigned(blocks)), dim3(16 * 64), 0,
                       stream, p);
  else if (lane_offsets_fit32(p))
    hipLaunchKernelGGL((es_lane_kernel<kBodyLinear, TI, TO, true>), dim3(unsigned(blocks)), dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL((es_lane_kernel<kBodyLinear, TI, TO>), dim3(unsigned(blocks)), dim3(64), 0, stream, p);
}
}  // namespace

hipError_t launch_linear_scan(const EsParams& p, bool in_bf16, bool out_bf16, hipStream_t stream) {
  if (p.num_lanes <= 0 || p.T <= 0) return hipSuccess;
  const int64_t blocks = (p.num_lanes + 63) / 64;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (in_bf16) {
    if (out_bf16) launch_linear<uint16_t, uint16_t>(p, blocks, stream);
    else launch_linear<uint16_t, float>(p, blocks, stream);
  } else {
    if (out_bf16) launch_linear<float, uint16_t>(p, blocks, stream);
    else launch_linear<float, float>(p, blocks, stream);
  }
  return hipGetLastError();
}

// The norm-cap gradient's split along the axis (as the forward pass's): chunk
// length and count, or false when one row per state vector is used.
static bool normcap_vjp_split(const EsParams& p, int64_t* len, int64_t* nchunks) {
  if (!(p.num_lanes > 0 && p.num_lanes < kChunkMaxLanes && p.T >= 2 * kChunkMinLen)) return false;
  int64_t c = (kChunkRows + p.num_lanes - 1) / p.num_lanes;
  int64_t l = (p.T + c - 1) / c;
  if (l < kChunkMinLen) l = kChunkMinLen;
  *len = l;
  *nchunks = (p.T + l - 1) / l;
  return true;
}

int64_t element_scan_backward_bound_words(sx_body body, const EsParams& p) {
  if (body != SX_BODY_NORM_CAP) return 0;
  // enough for either layout: the four-components-per-thread kernels (chosen at launch, by
  // alignment) or the one-component-per-thread ones
  int64_t len = 0, nchunks = 0, words = normcap_quad_bound_words(p);
  if (normcap_vjp_split(p, &len, &nchunks))
    words = std::max(words, 2 * p.num_lanes + nchunks * p.num_lanes);  // G and L* per lane, a product per chunk
  return words;
}

hipError_t launch_element_scan_backward(sx_body body, const EsVjpParams& v, hipStream_t stream) {
  const EsParams& p = v.p;
  if (p.num_lanes <= 0 || p.T <= 0) return hipSuccess;
  if (body == SX_BODY_NORM_CAP) {
    if (normcap_quad_eligible(v)) return launch_normcap_quad_backward(v, stream);
    int64_t len = 0, nchunks = 0;
    if (v.bounds != nullptr && normcap_vjp_split(p, &len, &nchunks)) {
      // few lanes: chunks of the sweep with certified warm-ups, as the forward pass splits its axis
      const int64_t blocks = (p.num_lanes * nchunks * 16 + 255) / 256;
      if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
      int rows = 1;  // rows of the bound kernel's workgroup: one chunk each, at most 64
      while (rows < 64 && rows < nchunks) rows *= 2;
      if (p.n_stride[ES_S] == 0) {  // a width-one gate
        hipLaunchKernelGGL(es_vjp_normcap_bound_kernel<true>, dim3(unsigned(p.num_lanes)), dim3(16 * rows), 0,
                           stream, v, len, nchunks);
        hipLaunchKernelGGL(es_vjp_normcap_chunk_kernel<true>, dim3(unsigned(blocks)), dim3(256), 0, stream, v, len,
                           nchunks);
      } else {
        hipLaunchKernelGGL(es_vjp_normcap_bound_kernel<false>, dim3(unsigned(p.num_lanes)), dim3(16 * rows), 0,
                           stream, v, len, nchunks);
        hipLaunchKernelGGL(es_vjp_normcap_chunk_kernel<false>, dim3(unsigned(blocks)), dim3(256), 0, stream, v, len,
                           nchunks);
      }
      return hipGetLastError();
    }
    const int64_t blocks = (p.num_lanes * 16 + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(es_vjp_normcap_row_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, v);
    return hipGetLastError();
  }
  const int64_t blocks = (p.num_lanes + 63) / 64;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  // The gradient's slab kernel is associative in every case; with few lanes it
  // still takes every load of a slab at once, where the lane kernel would wait
  // on memory each block of trips.
  const bool slab = p.T >= kSlabMinTrips || (p.num_lanes < kSlabMinLanes && p.T >= 64);
  auto launch = [&](auto bodyc, auto idxc) {
    constexpr int B = decltype(bodyc)::value;
    constexpr bool I32 = decltype(idxc)::value;
    if (slab && p.T <= 64)  // one slab of 4 trips a wave: every wave has trips (tanh-affine [4,64,32]: 5.5 against 7.0 us)
      hipLaunchKernelGGL((es_vjp_slab_kernel<B, 16, 4, I32>), dim3(unsigned(blocks)), dim3(1024), 0, stream, v);
    else if (slab)
      hipLaunchKernelGGL((es_vjp_slab_kernel<B, 16, 8, I32>), dim3(unsigned(blocks)), dim3(1024), 0, stream, v);
    else
      hipLaunchKernelGGL((es_vjp_lane_kernel<B, I32>), dim3(unsigned(blocks)), dim3(64), 0, stream, v);
  };
  const bool i32 = lane_offsets_fit32(p);
  using TanhC = std::integral_constant<int, SX_BODY_TANH_AFFINE>;
  using MaxC = std::integral_constant<int, SX_BODY_MAX_PLUS>;
  if (body == SX_BODY_TANH_AFFINE) {
    if (i32) launch(TanhC{}, std::true_type{});
    else launch(TanhC{}, std::false_type{});
  } else {
    if (i32) launch(MaxC{}, std::true_type{});
    else launch(MaxC{}, std::false_type{});
  }
  return hipGetLastError();
}

}  // namespace sx
