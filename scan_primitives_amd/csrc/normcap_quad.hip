// normcap_quad.hip: the norm-capped body with the 16-wide state held four
// components per thread.
//
// "Nonlinear element scans" (SexpGPU docs), introduction: the norm-capped
// body y = a h + x, h' = y / max(1, |y|) over a 16-wide state vector. A quad
// of four threads holds one state vector, components 4j .. 4j + 3 in thread j,
// loaded and stored as 16-byte vectors; |y|^2 and the other dot products are a
// sum within the thread and two DPP steps across the quad (the same bits in
// all four threads, so they decide together). Memory is reached through
// buffer resources with 32-bit offsets: no 64-bit address arithmetic per
// trip, and positions past either end of the axis read as zero or as other
// elements of the tensor (never used) instead of needing clamps.
//
// Both directions cut the axis into chunks that run at once (the body is not
// associative, but it contracts):
//   forward   a chunk starts W trips early from h = 0, W the first count for
//             which the product of the per-trip Lipschitz bounds
//             L = alpha / max(1, |x| - alpha) (alpha the largest |a|) is at
//             most 2^-26, or from `initial` when the walk reaches the start.
//   gradient  the trips are taken last to first. A trip from hp with
//             y = s hp + x passes back dy = (lam - u (u . lam)) / |y| when
//             |y| > 1 (u = y / |y|), else lam, where lam is the trip's upstream
//             gradient plus what the next trip passed back; grad_x = dy,
//             grad_s = dy hp, and s dy goes on (width-one x or s: summed over
//             the state). The adjoint map of a trip has norm at most the same
//             L, so from nu = 0 the adjoint stays within B = G L* / (1 - L*)
//             (G the largest |g| of the vector, L* its largest L). A chunk
//             starts from nu = 0 at an earlier chunk's start once the product
//             of the chunks' bounds in between is at most 2^-26 (1 - L*) / L*:
//             the adjoint entering the chunk is then within 2^-26 G of the
//             exact one. Vectors with L* >= 1 (or non-finite values) run their
//             whole sweep in one quad, exactly. A pre-pass writes G, L* and the
//             chunks' products.
#include <type_traits>
#include <utility>

#include "sx_common.hpp"

namespace sx {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t Rsrc;

constexpr float kCertBound = 1.0f / 67108864.0f;  // 2^-26

template <int CTRL>
__device__ __forceinline__ float quad_dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// Over the four threads of a quad; each step adds two values in either order,
// so all four threads get the same bits.
__device__ __forceinline__ float quad_sum(float v) {
  v += quad_dpp<0xB1>(v);  // quad_perm [1,0,3,2]
  v += quad_dpp<0x4E>(v);  // quad_perm [2,3,0,1]
  return v;
}
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, quad_dpp<0xB1>(v));
  v = fmaxf(v, quad_dpp<0x4E>(v));
  return v;
}
__device__ __forceinline__ float dot4(f4 a, f4 b) {
  return fmaf(a.w, b.w, fmaf(a.z, b.z, fmaf(a.y, b.y, a.x * b.x)));
}
__device__ __forceinline__ float sum4(f4 a) { return (a.x + a.y) + (a.z + a.w); }
__device__ __forceinline__ f4 fma4(f4 a, f4 b, f4 c) {
  return f4{fmaf(a.x, b.x, c.x), fmaf(a.y, b.y, c.y), fmaf(a.z, b.z, c.z), fmaf(a.w, b.w, c.w)};
}
__device__ __forceinline__ f4 splat(float v) { return f4{v, v, v, v}; }
__device__ __forceinline__ f4 as4(float v) { return splat(v); }
__device__ __forceinline__ f4 as4(f4 v) { return v; }

// A width-one value stays one register until used.
template <bool ONE>
using Comp = std::conditional_t<ONE, float, f4>;

// Buffer resource over `bytes` bytes from p (the raw-buffer word 3 of gfx9).
__device__ __forceinline__ Rsrc rsrc(const float* p, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0, bytes, 0x00020000);
}
// Element offsets; past the resource's end a load reads zero and a store is dropped.
template <bool ONE>
__device__ __forceinline__ Comp<ONE> bload(Rsrc r, int32_t elem) {
  if constexpr (ONE) return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, elem * 4, 0, 0));
  else return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, elem * 4, 0, 0));
}
__device__ __forceinline__ void bstore(Rsrc r, int32_t elem, f4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned, v), r,
                                         elem * 4, 0, 0);
}
__device__ __forceinline__ void bstore(Rsrc r, int32_t elem, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, elem * 4, 0, 0);
}

// The forward trip's Lipschitz bound, the same in the four threads.
template <bool S1>
__device__ __forceinline__ float quad_lipschitz(f4 x, f4 s) {
  const float xn = __builtin_amdgcn_sqrtf(quad_sum(dot4(x, x)));
  const float al = S1 ? fabsf(s.x) : quad_max(fmaxf(fmaxf(fabsf(s.x), fabsf(s.y)), fmaxf(fabsf(s.z), fabsf(s.w))));
  return al * __builtin_amdgcn_rcpf(fmaxf(1.0f, xn - al));
}

// A quad's offsets: the element of position w along its direction is
// base + w * step (32-bit: every tensor here spans fewer than 2^31 bytes).
struct Walk {
  int32_t base, step;
};
// Scan positions q (forward: dir = 1) or sweep positions w = T - 1 - q
// (gradient: dir = -1), time t = reverse ? T - 1 - q : q.
__device__ __forceinline__ Walk walk_of(int64_t lane_off, int64_t t_stride, int64_t T, bool reverse, bool sweep) {
  const bool down = reverse != sweep;  // time decreases along the walk
  Walk w;
  w.base = int32_t(lane_off + (down ? (T - 1) * t_stride : 0));
  w.step = int32_t(down ? -t_stride : t_stride);
  return w;
}

// ----------------------------------------------------------------- forward
//
// Rows are chunk-major (a run of rows is a run of chunks of every state
// vector), and the blocks are renumbered per XCD (xcd_block): a chunk's
// warm-up, which reads the chunks just before it, and the data one pass
// leaves for the next then stay in one L2.

// CL > 0: chunks of at most CL trips (len <= CL), each started WB trips
// early. Every load a quad needs, its chunk and the WB trips before it, is
// issued before any arithmetic, so the quad waits for memory once. The
// per-trip bounds of the WB trips are independent, so they are all formed at
// once; the quad is certified when the product over some run of trips ending
// at s - 1 is at most 2^-26. Every trip maps into the unit ball, so running
// all WB trips from 0 is as good as starting where that run starts, and the
// run needs no per-quad start point (chunks within WB trips of the axis start
// run exactly from `initial`). A quad that is not certified within WB trips
// takes the general path below, which walks further back a block of loads at
// a time. CL = 0: the general path only.
template <bool X1, bool S1, int CL, int WB>
__global__ __launch_bounds__(256) void nc_quad_fwd_kernel(const EsParams p, NcQuadSpans sp, int64_t len,
                                                          int64_t nchunks) {
  // rows, lanes, dims and strides all lie below 2^31 here (the launcher checks the row count,
  // and every tensor spans less than 2 GiB), so the index arithmetic is 32-bit
  const uint32_t row = uint32_t((xcd_block() * blockDim.x + threadIdx.x) >> 2);
  const uint32_t nl = uint32_t(p.num_lanes);
  if (row >= nl * uint32_t(nchunks)) return;  // whole quads
  const uint32_t chunk = row / nl, lane = row - chunk * nl;
  const int j = int(threadIdx.x & 3);
  int64_t off[4];
  index_offsets32(p.lanes, lane, off);
  const int64_t T = p.T;
  const bool rev = p.reverse != 0;
  const Rsrc rx = rsrc(p.x, sp.x), rs = rsrc(p.s, sp.s), ro = rsrc(p.out, sp.out);
  const Walk wx = walk_of(off[ES_X] + (X1 ? 0 : 4 * j), p.t_stride[ES_X], T, rev, false);
  const Walk ws = walk_of(off[ES_S] + (S1 ? 0 : 4 * j), p.t_stride[ES_S], T, rev, false);
  const Walk wo = walk_of(off[ES_OUT] + 4 * j, p.t_stride[ES_OUT], T, rev, false);
  const int32_t s = int32_t(chunk * len);
  const int32_t e = int32_t(s + len < T ? s + len : T);
  // one trip from h: y = a h + x, h = y / max(1, |y|)
  auto trip = [&](f4& h, f4 xq, f4 sq) {
    const f4 y = fma4(sq, h, xq);
    const float ss = quad_sum(dot4(y, y));
    h = y * fminf(1.0f, __builtin_amdgcn_rsqf(ss));  // rsqrt(ss) >= 1 exactly when ss <= 1
  };
  auto initial_state = [&]() -> f4 {
    const float* ip = p.init + off[ES_INIT] + 4 * j * p.n_stride[ES_INIT];
    const int64_t is = p.n_stride[ES_INIT];
    return f4{ip[0], ip[is], ip[2 * is], ip[3 * is]};
  };
  if constexpr (CL > 0) {
    // Registers hold positions s - WB .. s + CL - 1 (index i = position - (s - WB)); positions past
    // either end of the axis read zero or another element of the tensor (not used). A width-one
    // gate is the same for the quad's four threads, so thread j loads every fourth position
    // (i = 4k + j) and a quad broadcast hands each out when it is used.
    constexpr int NP = WB + CL;
    const int32_t p0 = s - WB;
    Comp<X1> xa[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) xa[i] = bload<X1>(rx, wx.base + (p0 + i) * wx.step);
    constexpr int NS = S1 ? (NP + 3) / 4 : NP;
    Comp<S1> sa[NS];
#pragma unroll
    for (int k = 0; k < NS; ++k)
      sa[k] = bload<S1>(rs, ws.base + (p0 + (S1 ? 4 * k + j : k)) * ws.step);
    auto gate = [&](auto ic) -> f4 {
      constexpr int i = decltype(ic)::value;
      if constexpr (S1) return splat(quad_dpp<(i & 3) * 0x55>(as4(sa[i >> 2]).x));
      else return as4(sa[i]);
    };
    // Certified when some run of trips ending at s - 1, within the WB kept, has a product of bounds
    // of at most 2^-26 (the bounds are independent, so they are formed at once). Every trip maps into
    // the unit ball, so starting all WB trips early from 0 is as good as starting at that run's start.
    // A chunk within WB trips of the axis start runs exactly from `initial` at position 0 (the
    // warm-up must not start at position 0 from 0: `initial` need not lie in the unit ball).
    const bool from_start = s <= WB;  // uniform over the chunk
    bool certified = from_start;
    if (!from_start) {
      float prod = 1.0f;
      [&]<int... us>(std::integer_sequence<int, us...>) {
        ((prod *= quad_lipschitz<S1>(as4(xa[WB - 1 - us]), gate(std::integral_constant<int, WB - 1 - us>{})),
          certified = certified || prod <= kCertBound),
         ...);
      }(std::make_integer_sequence<int, WB>{});
    }
    if (certified) {  // quad-uniform
      f4 h = from_start ? initial_state() : splat(0.0f);
      // each trip's gate is formed one trip ahead, off the recurrence's path
      f4 gcur = gate(std::integral_constant<int, 0>{});
      [&]<int... is>(std::integer_sequence<int, is...>) {
        (([&] {
           const f4 gnext = gate(std::integral_constant<int, is + 1 < NP ? is + 1 : is>{});
           if constexpr (is < WB) {
             if (p0 + is >= 0) trip(h, as4(xa[is]), gcur);  // uniform over the chunk
           } else {
             if (s + (is - WB) < e) {
               trip(h, as4(xa[is]), gcur);
               bstore(ro, wo.base + (s + (is - WB)) * wo.step, h);
             }
           }
           gcur = gnext;
         }()),
         ...);
      }(std::make_integer_sequence<int, NP>{});
      return;
    }
  }
  constexpr int U = 8;
  // ---- general path: walk back from s - 1 while the bound is above 2^-26
  int32_t start = 0;
  if (s > 0) {  // quad-uniform
    float prod = 1.0f;
    bool done = false;
    for (int32_t q = s - 1; !done; q -= U) {
      Comp<X1> xv[U];
      Comp<S1> sv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {  // positions below 0 read zero (unused)
        xv[u] = bload<X1>(rx, wx.base + (q - u) * wx.step);
        sv[u] = bload<S1>(rs, ws.base + (q - u) * ws.step);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (!done) {
          if (q - u < 0) {
            start = 0;  // reached the start of the axis: exact from `initial`
            done = true;
          } else {
            prod *= quad_lipschitz<S1>(as4(xv[u]), as4(sv[u]));
            if (prod <= kCertBound) {
              start = q - u;
              done = true;
            }
          }
        }
      }
    }
  }
  // ---- from `initial` at position 0, else from 0 (in the unit ball)
  f4 h = splat(0.0f);
  if (start == 0) h = initial_state();
  struct Block {
    Comp<X1> x[U];
    Comp<S1> s[U];
  };
  auto load = [&](int32_t q0, Block& B) {
    int32_t ox = wx.base + q0 * wx.step, os = ws.base + q0 * ws.step;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      B.x[u] = bload<X1>(rx, ox);
      ox += wx.step;
      B.s[u] = bload<S1>(rs, os);
      os += ws.step;
    }
  };
  auto run = [&](int32_t q0, const Block& B) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t q = q0 + u;
      if (q < e) {  // quad-uniform
        trip(h, as4(B.x[u]), as4(B.s[u]));
        if (q >= s) bstore(ro, wo.base + q * wo.step, h);
      }
    }
  };
  Block b0, b1;  // the next block's loads are issued before a block is computed (two in turn)
  load(start, b0);
  for (int32_t q0 = start; q0 < e; q0 += 2 * U) {
    load(q0 + U, b1);
    run(q0, b0);
    if (q0 + U >= e) break;  // quad-uniform
    load(q0 + 2 * U, b0);
    run(q0 + U, b1);
  }
}

// ----------------------------------------------------------------- gradient

// Per state vector and group of chunks: the largest |g| and the largest
// per-trip bound L (non-finite values become +inf: no certificate), and per
// chunk of the sweep the product of its trips' bounds. Block b takes group
// b mod 8 (the chunks the gradient pass runs on the same XCD) of vector b / 8;
// its quads take every R-th chunk of the group (R quads). bounds holds the
// group maxima at 2 (g num_lanes + lane) (G) and + 1 (L*), the product of
// chunk c at 2 kXcds num_lanes + c num_lanes + lane.
template <bool X1, bool S1>
__global__ __launch_bounds__(256) void nc_quad_bound_kernel(const EsVjpParams v, NcQuadSpans sp, int64_t len,
                                                            int64_t nchunks) {
  const EsParams& p = v.p;
  const int64_t group = blockIdx.x % kXcds, lane = blockIdx.x / kXcds;
  const int R = int(blockDim.x >> 2), r = int(threadIdx.x >> 2), j = int(threadIdx.x & 3);
  int64_t off[4];
  index_offsets32(p.lanes, uint32_t(lane), off);  // every tensor spans less than 2 GiB
  const int64_t T = p.T;
  const bool rev = p.reverse != 0;
  const Rsrc rx = rsrc(p.x, sp.x), rs = rsrc(p.s, sp.s), rg = rsrc(v.g, sp.out);
  const Walk wx = walk_of(off[ES_X] + (X1 ? 0 : 4 * j), p.t_stride[ES_X], T, rev, true);
  const Walk ws = walk_of(off[ES_S] + (S1 ? 0 : 4 * j), p.t_stride[ES_S], T, rev, true);
  const Walk wg = walk_of(off[ES_OUT] + 4 * j, p.t_stride[ES_OUT], T, rev, true);
  float* prods = v.bounds + 2 * kXcds * p.num_lanes + lane;
  // the gradient pass's rows of XCD k are chunk-major; its chunks are close to group k's
  const int64_t per = (nchunks + kXcds - 1) / kXcds;
  const int64_t c_begin = group * per, c_end = c_begin + per < nchunks ? c_begin + per : nchunks;
  float gmax = 0.0f, lmax = 0.0f;
  constexpr int U = 8;
  for (int64_t c = c_begin + r; c < c_end; c += R) {  // quad-uniform
    const int32_t w_begin = int32_t(c * len), w_end = int32_t(c * len + len < T ? c * len + len : T);
    float prod = 1.0f;
    for (int32_t w0 = w_begin; w0 < w_end; w0 += U) {
      Comp<X1> xv[U];
      Comp<S1> sv[U];
      f4 gv[U];
      int32_t ox = wx.base + w0 * wx.step, os = ws.base + w0 * ws.step, og = wg.base + w0 * wg.step;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        xv[u] = bload<X1>(rx, ox);
        sv[u] = bload<S1>(rs, os);
        gv[u] = bload<false>(rg, og);
        ox += wx.step;
        os += ws.step;
        og += wg.step;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (w0 + u < w_end) {  // quad-uniform
          const float l = quad_lipschitz<S1>(as4(xv[u]), as4(sv[u]));
          const float gn = __builtin_amdgcn_sqrtf(quad_sum(dot4(gv[u], gv[u])));
          prod *= l;
          lmax = l <= 3.0e38f ? fmaxf(lmax, l) : __builtin_huge_valf();  // NaN counts as unbounded
          gmax = gn <= 3.0e38f ? fmaxf(gmax, gn) : __builtin_huge_valf();
        }
      }
    }
    if (j == 0) prods[c * p.num_lanes] = prod;
  }
  // maxima over the workgroup: across the wave's quads by DPP row mirrors and
  // lane reads (the workgroup is whole waves, so every lane read is a live one),
  // then the waves through LDS
  auto wave_max = [](float m) {
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x141, 0xF, 0xF, false)));
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x140, 0xF, 0xF, false)));
    const int bits = __float_as_int(m);
    const float a = __int_as_float(__builtin_amdgcn_readlane(bits, 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(bits, 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(bits, 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(bits, 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
  };
  const float wg_g = wave_max(gmax), wg_l = wave_max(lmax);  // a quad's threads hold the same values
  __shared__ float red[2][4];
  const int wave = int(threadIdx.x >> 6), nwaves = int((blockDim.x + 63) >> 6);
  if ((threadIdx.x & 63) == 0) {
    red[0][wave] = wg_g;
    red[1][wave] = wg_l;
  }
  __syncthreads();
  if (threadIdx.x < 2) {
    float m = 0.0f;
    for (int i = 0; i < nwaves; ++i) m = fmaxf(m, red[threadIdx.x][i]);  // values are >= 0 or +inf
    v.bounds[2 * (group * p.num_lanes + lane) + threadIdx.x] = m;
  }
}

// One quad per (state vector, chunk of the sweep), or per state vector when
// nchunks is 1 (then bounds is unused and every sweep is exact).
template <bool X1, bool S1>
__global__ __launch_bounds__(256) void nc_quad_grad_kernel(const EsVjpParams v, NcQuadSpans sp, int64_t len,
                                                           int64_t nchunks) {
  const EsParams& p = v.p;
  // 32-bit index arithmetic, as in the forward kernel (the launcher checks the row count)
  const uint32_t row = uint32_t((xcd_block() * blockDim.x + threadIdx.x) >> 2);
  const uint32_t nl = uint32_t(p.num_lanes);
  if (row >= nl * uint32_t(nchunks)) return;  // whole quads
  const uint32_t chunk = row / nl, lane = row - chunk * nl;
  const int j = int(threadIdx.x & 3);
  int64_t off[4];
  index_offsets32(p.lanes, lane, off);
  const int64_t T = p.T;
  const bool rev = p.reverse != 0;
  const Rsrc rx = rsrc(p.x, sp.x), rs = rsrc(p.s, sp.s), rh = rsrc(v.h, sp.out), rg = rsrc(v.g, sp.out);
  const Rsrc rgx = rsrc(v.gx, X1 ? sp.out / 16 : sp.out), rgs = rsrc(v.gs, S1 ? sp.out / 16 : sp.out);
  const Walk wx = walk_of(off[ES_X] + (X1 ? 0 : 4 * j), p.t_stride[ES_X], T, rev, true);
  const Walk ws = walk_of(off[ES_S] + (S1 ? 0 : 4 * j), p.t_stride[ES_S], T, rev, true);
  const Walk wo = walk_of(off[ES_OUT] + 4 * j, p.t_stride[ES_OUT], T, rev, true);
  // width-one gradients: out's shape with 1 for the 16 (out is contiguous, state last)
  const Walk w1 = walk_of(off[ES_OUT] / 16, p.t_stride[ES_OUT] / 16, T, rev, true);
  const Walk wgx = X1 ? w1 : wo, wgs = S1 ? w1 : wo;
  f4 init;
  {
    const float* ip = p.init + off[ES_INIT] + 4 * j * p.n_stride[ES_INIT];
    const int64_t is = p.n_stride[ES_INIT];
    init = f4{ip[0], ip[is], ip[2 * is], ip[3 * is]};
  }
  const int32_t s0 = int32_t(chunk * len);
  int32_t e0 = int32_t(s0 + len < T ? s0 + len : T);
  int32_t start = 0;
  if (nchunks > 1) {
    // over the groups' maxima (8 pairs); a value that is not a finite number >= 0
    // (which the pre-pass does not write) leaves the vector without a certificate
    float gmax = 0.0f, lmax = 0.0f;
#pragma unroll
    for (int g = 0; g < kXcds; ++g) {
      const float gg = v.bounds[2 * (g * p.num_lanes + lane)], gl = v.bounds[2 * (g * p.num_lanes + lane) + 1];
      gmax = gg >= 0.0f && gg <= 3.0e38f ? fmaxf(gmax, gg) : __builtin_huge_valf();
      lmax = gl >= 0.0f && gl <= 3.0e38f ? fmaxf(lmax, gl) : __builtin_huge_valf();
    }
    if (!(lmax < 1.0f) || !(gmax <= 3.0e38f)) {  // quad-uniform: no certificate for this vector
      if (chunk != 0) return;  // the first chunk's quad runs the whole sweep exactly
      e0 = int32_t(T);
    } else if (s0 > 0) {
      if (lmax == 0.0f || gmax == 0.0f) {
        start = s0;  // every adjoint map or every g is zero: nu is exactly zero entering the chunk
      } else {
        const float target = kCertBound * (1.0f - lmax) / lmax;
        const float* prods = v.bounds + 2 * kXcds * p.num_lanes + lane;
        float prod = 1.0f;
        int64_t c = chunk - 1;
        bool done = false;
        while (!done) {  // four chunk products per round
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
                  start = int32_t((c - u) * len);
                  done = true;
                }
              }
            }
          }
          c -= 4;
        }
      }
    }
  }
  // ---- the sweep over [start, e0); trips before s0 only carry the adjoint. The next
  // block's loads are issued before a block is computed (two blocks in turn).
  constexpr int U = 8;
  struct Block {
    f4 h[U], g[U];
    Comp<X1> x[U];
    Comp<S1> s[U];
  };
  auto load = [&](int32_t w0, Block& B) {
    int32_t og = wo.base + w0 * wo.step, ox = wx.base + w0 * wx.step, os = ws.base + w0 * ws.step;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      B.g[u] = bload<false>(rg, og);
      og += wo.step;
      B.h[u] = bload<false>(rh, og);  // the state before the trip: one position further along the sweep
      B.x[u] = bload<X1>(rx, ox);
      ox += wx.step;
      B.s[u] = bload<S1>(rs, os);
      os += ws.step;
    }
  };
  f4 nu = splat(0.0f);
  auto run = [&](int32_t w0, const Block& B) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t w = w0 + u;
      if (w < e0) {  // quad-uniform
        const f4 hp = w + 1 < T ? B.h[u] : init;  // the first trip of the scan starts from initial
        const f4 sv = as4(B.s[u]);
        const f4 y = fma4(sv, hp, as4(B.x[u]));
        const float ir = __builtin_amdgcn_rsqf(quad_sum(dot4(y, y)));
        const f4 uy = y * ir;
        const f4 lam = B.g[u] + nu;
        const float ul = quad_sum(dot4(uy, lam));
        const f4 dy = ir < 1.0f ? (lam - uy * ul) * ir : lam;  // capped when |y| > 1
        nu = sv * dy;
        if (w >= s0) {
          if constexpr (X1) {
            const float sx = quad_sum(sum4(dy));
            if (j == 0) bstore(rgx, wgx.base + w * wgx.step, sx);
          } else {
            bstore(rgx, wgx.base + w * wgx.step, dy);
          }
          if constexpr (S1) {
            const float ss = quad_sum(dot4(dy, hp));
            if (j == 0) bstore(rgs, wgs.base + w * wgs.step, ss);
          } else {
            bstore(rgs, wgs.base + w * wgs.step, dy * hp);
          }
        }
      }
    }
  };
  Block b0, b1;
  load(start, b0);
  for (int32_t w0 = start; w0 < e0; w0 += 2 * U) {
    load(w0 + U, b1);
    run(w0, b0);
    if (w0 + U >= e0) break;  // quad-uniform
    load(w0 + 2 * U, b0);
    run(w0 + U, b1);
  }
  if (e0 == T) {
    float* gi = v.ginit + off[ES_INIT] + 4 * j * p.n_stride[ES_INIT];
    const int64_t is = p.n_stride[ES_INIT];
    gi[0] = nu.x;
    gi[is] = nu.y;
    gi[2 * is] = nu.z;
    gi[3 * is] = nu.w;
  }
}

// ----------------------------------------------------------------- host side

// Quads in flight: about kFwdRows (forward) or kGradRows (gradient) rows, in
// chunks of at least kFwdMinLen or kGradMinLen trips. Measured on [8,1024,16,16]
// and [64,1024,16,16]: more rows help the gradient's longer per-row chains on
// the larger shape and slow the forward there. Forward chunks of at most
// kFwdRegLen trips keep the chunk and kFwdWarm warm-up trips in registers;
// 20 warm-up trips certify every chunk of the standard norm-cap workload
// (|x| about 4, gate in [0.8, 1]: the most any chunk needs is 20).
constexpr int64_t kFwdRows = 16384;
constexpr int64_t kGradRows = 32768;
constexpr int64_t kFwdMinLen = 8;
constexpr int64_t kGradMinLen = 8;
constexpr int kFwdRegLen = 8;
constexpr int kFwdWarm = 20;
constexpr int64_t kMaxSpan = int64_t(1) << 31;  // bytes a buffer resource here may cover

bool split_of(const EsParams& p, int64_t rows, int64_t min_len, int64_t* len, int64_t* nchunks) {
  if (!(p.num_lanes > 0 && p.num_lanes < rows && p.T >= 2 * min_len)) {
    *len = p.T;
    *nchunks = 1;
    return false;
  }
  const int64_t c = (rows + p.num_lanes - 1) / p.num_lanes;
  int64_t l = (p.T + c - 1) / c;
  if (l < min_len) l = min_len;
  *len = l;
  *nchunks = (p.T + l - 1) / l;
  return true;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Bytes from tensor k's base to one past its last element, or -1 when a
// stride is negative; width-one sequences (component stride 0) included.
int64_t span_bytes_of(const EsParams& p, int k) {
  int64_t last = (p.T - 1) * p.t_stride[k];
  if (p.t_stride[k] < 0) return -1;
  for (int d = 0; d < p.lanes.nd; ++d) {
    if (p.lanes.st[k][d] < 0) return -1;
    last += (p.lanes.dim[d] - 1) * p.lanes.st[k][d];
  }
  if (p.n_stride[k] < 0) return -1;
  last += int64_t(p.n - 1) * p.n_stride[k];
  return 4 * (last + 1);
}

// A four-component group of tensor k starts at a multiple of four elements.
bool quad_strides_ok(const EsParams& p, int k) {
  if (p.t_stride[k] % 4 != 0) return false;
  for (int d = 0; d < p.lanes.nd; ++d)
    if (p.lanes.dim[d] > 1 && p.lanes.st[k][d] % 4 != 0) return false;
  return true;
}

bool spans_of(const EsParams& p, NcQuadSpans* sp) {
  if (p.n != 16 || p.n_stride[ES_OUT] != 1 || p.T > 0x7fffffff) return false;
  const int64_t sx = span_bytes_of(p, ES_X), ss = span_bytes_of(p, ES_S), so = span_bytes_of(p, ES_OUT);
  if (sx <= 0 || ss <= 0 || so <= 0 || sx >= kMaxSpan || ss >= kMaxSpan || so >= kMaxSpan) return false;
  // initial (and the gradient's grad_initial, in its layout) is addressed by a pointer, but its lane
  // offsets come from the same 32-bit index arithmetic: they must fit as well
  const int64_t si = span_bytes_of(p, ES_INIT);
  if (si <= 0 || si >= kMaxSpan) return false;
  const bool x1 = p.n_stride[ES_X] == 0, s1 = p.n_stride[ES_S] == 0;
  if (!x1 && (p.n_stride[ES_X] != 1 || !quad_strides_ok(p, ES_X) || !aligned16(p.x))) return false;
  if (!s1 && (p.n_stride[ES_S] != 1 || !quad_strides_ok(p, ES_S) || !aligned16(p.s))) return false;
  if (!quad_strides_ok(p, ES_OUT) || p.t_stride[ES_OUT] % 16 != 0) return false;
  sp->x = int32_t(sx);
  sp->s = int32_t(ss);
  sp->out = int32_t(so);
  return true;
}

template <class F>
void by_widths(const EsParams& p, F&& f) {
  using T_ = std::true_type;
  using F_ = std::false_type;
  const bool x1 = p.n_stride[ES_X] == 0, s1 = p.n_stride[ES_S] == 0;
  if (x1 && s1) f(T_{}, T_{});
  else if (x1) f(T_{}, F_{});
  else if (s1) f(F_{}, T_{});
  else f(F_{}, F_{});
}

}  // namespace

bool normcap_quad_forward_eligible(const EsParams& p) {
  NcQuadSpans sp;
  return spans_of(p, &sp) && aligned16(p.out);
}

hipError_t launch_normcap_quad_forward(const EsParams& p, hipStream_t stream) {
  NcQuadSpans sp;
  if (!spans_of(p, &sp)) return hipErrorInvalidValue;
  int64_t len = 0, nchunks = 1;
  split_of(p, kFwdRows, kFwdMinLen, &len, &nchunks);
  const int64_t blocks = (p.num_lanes * nchunks * 4 + 255) / 256;
  if (blocks * 256 > 0x7fffffff) return hipErrorInvalidConfiguration;  // 32-bit row arithmetic
  by_widths(p, [&](auto x1c, auto s1c) {
    constexpr bool X1 = decltype(x1c)::value, S1 = decltype(s1c)::value;
    if (len <= kFwdRegLen)
      hipLaunchKernelGGL((nc_quad_fwd_kernel<X1, S1, kFwdRegLen, kFwdWarm>), dim3(unsigned(blocks)), dim3(256), 0,
                         stream, p, sp, len, nchunks);
    else
      hipLaunchKernelGGL((nc_quad_fwd_kernel<X1, S1, 0, 1>), dim3(unsigned(blocks)), dim3(256), 0, stream, p, sp, len,
                         nchunks);
  });
  return hipGetLastError();
}

bool normcap_quad_eligible(const EsVjpParams& v) {
  NcQuadSpans sp;
  if (!spans_of(v.p, &sp)) return false;
  const bool x1 = v.p.n_stride[ES_X] == 0, s1 = v.p.n_stride[ES_S] == 0;
  if (!aligned16(v.h) || !aligned16(v.g)) return false;
  if ((!x1 && !aligned16(v.gx)) || (!s1 && !aligned16(v.gs))) return false;
  return true;
}

hipError_t launch_normcap_quad_backward(const EsVjpParams& v, hipStream_t stream) {
  const EsParams& p = v.p;
  NcQuadSpans sp;
  if (!spans_of(p, &sp)) return hipErrorInvalidValue;
  int64_t len = 0, nchunks = 1;
  const bool split = split_of(p, kGradRows, kGradMinLen, &len, &nchunks) && v.bounds != nullptr;
  if (!split) {
    len = p.T;
    nchunks = 1;
  }
  const int64_t blocks = (p.num_lanes * nchunks * 4 + 255) / 256;
  if (blocks * 256 > 0x7fffffff) return hipErrorInvalidConfiguration;  // 32-bit row arithmetic
  const int64_t per_group = (nchunks + kXcds - 1) / kXcds;
  // the bound kernel's quads per workgroup: one chunk of the group each, at most 64, and at
  // least a whole wave (its maxima read every lane of the wave)
  int quads = 16;
  while (quads < 64 && quads < per_group) quads *= 2;
  by_widths(p, [&](auto x1c, auto s1c) {
    constexpr bool X1 = decltype(x1c)::value, S1 = decltype(s1c)::value;
    if (split)
      hipLaunchKernelGGL((nc_quad_bound_kernel<X1, S1>), dim3(unsigned(kXcds * p.num_lanes)), dim3(4 * quads), 0,
                         stream, v, sp, len, nchunks);
    hipLaunchKernelGGL((nc_quad_grad_kernel<X1, S1>), dim3(unsigned(blocks)), dim3(256), 0, stream, v, sp, len,
                       nchunks);
  });
  return hipGetLastError();
}

int64_t normcap_quad_bound_words(const EsParams& p) {
  int64_t len = 0, nchunks = 1;
  if (!split_of(p, kGradRows, kGradMinLen, &len, &nchunks)) return 0;
  return 2 * kXcds * p.num_lanes + nchunks * p.num_lanes;
}

}  // namespace sx
