// matrix_scan.hip: matrix-scan kernels for gfx950.
//
// "Tensor operations" (SexpGPU docs), Operations table (matrix-scan row) and
// the "matrix-scan" section: h[t] = a[t] @ h[t-1] + b[t] from h = 0, one
// matrix product a step, computed in f32 (bf16 operands widen exactly);
// :reverse runs from the end, h[t] = a[t] @ h[t+1] + b[t] from h[T] = 0.
//
// Kernels here:
//   ms_chunk_kernel   the single-pass chunked scan. The scan axis is cut into
//                     chunks of K steps; one wave owns one (batch, 16-column
//                     tile of m, chunk) unit. It keeps the chunk's a and b in
//                     registers, composes the chunk's affine map (A, B) with
//                     MFMA, publishes it, takes the state entering the chunk
//                     from its predecessors by decoupled look-back, and
//                     replays the chunk from that state with MFMA, storing
//                     every h[t]. Inputs are read from HBM once.
//   ms_serial_kernel  one 256-thread block per (batch, 16-column tile of m):
//                     thread (i, j) owns h[i][j]; every step stages a[t] in
//                     LDS and forms row i of a[t] @ h with a k-ordered FMA
//                     chain. Serial in time; used when the look-back state
//                     would not fit the chunked kernel's 32-bit unit ids.
//
// MFMA mapping (v_mfma_f32_16x16x4_f32, wave64; lane l = 16 r + c, r = 0..3):
//   A operand  lane (r, c) gives A[c][k], B operand gives B[k][c], for the
//              instruction's k = 0..3 taken from lane group r;
//   result     lane (r, c) holds D[4r + v][c] in register v = 0..3.
// Four instructions q = 0..3 form a 16x16x16 product. Pairing the k index as
// k = 4r + q, lane (r, c) supplies a[c][4r + q] (four consecutive entries of
// row c: one 16-byte load) and X[4r + q][c], which is exactly register q of
// the previous result. So a chain h <- a[t] @ h + b[t] feeds each result
// straight back as the next B operand, with no data movement between steps.
#include <utility>

#include "sx_common.hpp"

namespace sx {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float load_elem(const float* p) { return *p; }
__device__ __forceinline__ float load_elem(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_elem(uint16_t* p, float v) { *p = f32_to_bf16_rne(v); }

// ------------------------------------------------------------------ serial kernel

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

// ------------------------------------------------------------------ chunked kernel

constexpr uint32_t kFlagAggregate = 1;  // the unit's map (A, B) is published
constexpr uint32_t kFlagInclusive = 2;  // the state leaving the unit is published
constexpr uint32_t kSpinLimit = 1u << 22;

// Look-back state of the chunked kernel, carved out of the caller's workspace.
// Slot s = bt * chunks + chunk: bt is the (batch, 16-column tile) index.
struct MsUnitWs {
  uint32_t* header;  // [0] next unit id, [1] status (nonzero: a look-back gave up)
  uint32_t* flags;   // per slot
  float* P;          // per slot, the unit's A as a row-major 16x16 block
  float* L;          // per slot, the unit's B in result-register order (lane * 4 + v)
  float* H;          // per slot, the state leaving the unit, same order as L
  uint32_t num_units;
  uint32_t chunks;   // units per bt along the scan axis
  int col_tiles;     // ceil(m / 16)
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.0f, 0.0f, 0.0f, 0.0f}; }

__device__ __forceinline__ f32x4 mfma_16x16x16(f32x4 a, f32x4 x, f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], x[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], x[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], x[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], x[3], c, 0, 0, 0);
  return c;
}

__device__ __forceinline__ f32x4 identity_d(int r, int c) {  // I in result-register order
  f32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = (4 * r + q == c) ? 1.0f : 0.0f;
  return v;
}

// a[t] for lane (r, c): a[c][4r .. 4r+3], zero past n, kept as f32 or as four packed bf16.
template <typename TIn>
struct ARow;
template <>
struct ARow<float> {
  f32x4 v;
  __device__ __forceinline__ f32x4 get() const { return v; }
};
template <>
struct ARow<uint16_t> {
  uint2 u;
  __device__ __forceinline__ f32x4 get() const {
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                 __uint_as_float(u.y & 0xffff0000u)};
  }
};

template <typename TIn, bool VEC>
__device__ __forceinline__ ARow<TIn> load_a(const TIn* ap, int n, int r, int c) {
  ARow<TIn> out;
  if constexpr (VEC && sizeof(TIn) == 4) {
    out.v = *reinterpret_cast<const f32x4*>(ap + c * 16 + 4 * r);
  } else if constexpr (VEC) {
    out.u = *reinterpret_cast<const uint2*>(ap + c * 16 + 4 * r);
  } else {
    // clamped indices: every lane loads a valid element, then zeroes what lies past n
    uint16_t h[4];
    float f[4];
    const int row = c < n ? c : n - 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool in = c < n && 4 * r + q < n;
      const int col = 4 * r + q < n ? 4 * r + q : n - 1;
      const TIn v = ap[row * n + col];
      if constexpr (sizeof(TIn) == 4) f[q] = in ? float(v) : 0.0f;
      else h[q] = in ? uint16_t(v) : uint16_t(0);
    }
    if constexpr (sizeof(TIn) == 4) out.v = f32x4{f[0], f[1], f[2], f[3]};
    else out.u = make_uint2(h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16));
  }
  return out;
}

template <typename TIn>
__device__ __forceinline__ ARow<TIn> identity_a(int r, int c) {
  ARow<TIn> out;
  if constexpr (sizeof(TIn) == 4) {
    out.v = identity_d(r, c);  // same pattern: entry 4r + q of row c
  } else {
    const uint32_t one = 0x3f80u;  // bf16 1.0
    out.u = make_uint2((c == 4 * r ? one : 0u) | ((c == 4 * r + 1 ? one : 0u) << 16),
                       (c == 4 * r + 2 ? one : 0u) | ((c == 4 * r + 3 ? one : 0u) << 16));
  }
  return out;
}

// b[t] in result-register order for lane (r, c): rows 4r + v of column cc, zero past n and m.
// f32 keeps four floats; bf16 keeps four bf16 packed into two registers.
template <typename TIn>
struct BCol;
template <>
struct BCol<float> {
  f32x4 v;
  __device__ __forceinline__ f32x4 get() const { return v; }
};
template <>
struct BCol<uint16_t> {
  uint2 u;
  __device__ __forceinline__ f32x4 get() const {
    return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                 __uint_as_float(u.y & 0xffff0000u)};
  }
};

template <typename TIn>
__device__ __forceinline__ BCol<TIn> load_b(const TIn* bp, int n, int m, int r, int cc) {
  // clamped indices: every lane loads a valid element, then zeroes what lies past n and m
  BCol<TIn> out;
  const int col = cc < m ? cc : m - 1;
  TIn v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = bp[int64_t(4 * r + q < n ? 4 * r + q : n - 1) * m + col];
  if constexpr (sizeof(TIn) == 4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) out.v[q] = (4 * r + q < n && cc < m) ? v[q] : 0.0f;
  } else {
    uint32_t h[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) h[q] = (4 * r + q < n && cc < m) ? uint32_t(v[q]) : 0u;
    out.u = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
  }
  return out;
}

template <typename TIn>
__device__ __forceinline__ BCol<TIn> select_b(bool keep, BCol<TIn> v) {
  if constexpr (sizeof(TIn) == 4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) v.v[q] = keep ? v.v[q] : 0.0f;
  } else {
    v.u.x = keep ? v.u.x : 0u;
    v.u.y = keep ? v.u.y : 0u;
  }
  return v;
}

template <typename TIn>
__device__ __forceinline__ ARow<TIn> select_a(bool keep, ARow<TIn> v, ARow<TIn> other) {
  if constexpr (sizeof(TIn) == 4) {
#pragma unroll
    for (int q = 0; q < 4; ++q) v.v[q] = keep ? v.v[q] : other.v[q];
  } else {
    v.u.x = keep ? v.u.x : other.u.x;
    v.u.y = keep ? v.u.y : other.u.y;
  }
  return v;
}

// m == 1: lane (r, c) holds b[step c][4r .. 4r+3] for the wave's 16 steps (one load per lane).
template <typename TIn>
__device__ __forceinline__ f32x4 load_b_col1(const TIn* bp, int n, int r, bool vec) {
  f32x4 v;
  if (vec && sizeof(TIn) == 4) {
    v = *reinterpret_cast<const f32x4*>(bp + 4 * r);
  } else if (vec) {
    const uint2 u = *reinterpret_cast<const uint2*>(bp + 4 * r);
    v = f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
              __uint_as_float(u.y & 0xffff0000u)};
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float e = load_elem(bp + (4 * r + q < n ? 4 * r + q : n - 1));
      v[q] = (4 * r + q < n) ? e : 0.0f;
    }
  }
  return v;
}

// Lane (r, 0) takes lane (r, k)'s four values (DPP row_shl:k); the other lanes get zero.
template <int K>
__device__ __forceinline__ f32x4 col0_from_lane(f32x4 v, int c) {
  f32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float x = v[q];
    if constexpr (K > 0)
      x = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v[q]), 0x100 + K, 0xF, 0xF, false));
    o[q] = c == 0 ? x : 0.0f;
  }
  return o;
}

template <typename TOut>
__device__ __forceinline__ void store_h(TOut* op, f32x4 h, int n, int m, int r, int cc) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (4 * r + q < n && cc < m) store_elem(op + int64_t(4 * r + q) * m + cc, h[q]);
}

// m == 1 output: lane (r, 0) writes out[t][4r .. 4r+3].
template <typename TOut>
__device__ __forceinline__ void store_h_col1(TOut* op, f32x4 h, int n, int r, bool vec) {
  if (vec && sizeof(TOut) == 4) {
    *reinterpret_cast<f32x4*>(op + 4 * r) = h;
  } else if (vec) {
    const uint32_t lo = uint32_t(f32_to_bf16_rne(h[0])) | (uint32_t(f32_to_bf16_rne(h[1])) << 16);
    const uint32_t hi = uint32_t(f32_to_bf16_rne(h[2])) | (uint32_t(f32_to_bf16_rne(h[3])) << 16);
    *reinterpret_cast<uint2*>(op + 4 * r) = make_uint2(lo, hi);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (4 * r + q < n) store_elem(op + 4 * r + q, h[q]);
  }
}

// Device-coherent transfer of look-back data between workgroups, which may sit
// on different XCDs: relaxed agent-scope atomic accesses (coherent by the memory
// model), with the payload's completion awaited before the flag is raised. No
// L2 write-back or invalidate is needed, because no published word is ever
// written or read through the non-coherent path.
__device__ __forceinline__ void dev_store4(float* p, f32x4 v) {
  uint32_t* u = reinterpret_cast<uint32_t*>(p);
#pragma unroll
  for (int q = 0; q < 4; ++q) __hip_atomic_store(u + q, __float_as_uint(v[q]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ f32x4 dev_load4(const float* p) {
  const uint32_t* u = reinterpret_cast<const uint32_t*>(p);
  f32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    v[q] = __uint_as_float(__hip_atomic_load(const_cast<uint32_t*>(u + q), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  return v;
}

__device__ __forceinline__ void raise_flag(uint32_t* flag, uint32_t value, int lane) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // every earlier memory access of this wave has completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (lane == 0) __hip_atomic_store(flag, value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave-private LDS transpose: 16x16 block from result-register order to row-major,
// then read back in A-operand order (row c, entries 4r..4r+3).
__device__ __forceinline__ f32x4 to_a_operand(float* scratch, f32x4 d, int r, int c) {
#pragma unroll
  for (int v = 0; v < 4; ++v) scratch[(4 * r + v) * 16 + c] = d[v];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  return *reinterpret_cast<const f32x4*>(scratch + c * 16 + 4 * r);
}

// One workgroup of NW waves owns one unit: NW*K consecutive scan steps of one
// (batch, column tile). Wave w summarises its K steps into an affine map
// (P_w, L_w) with MFMA; the maps meet in LDS; the last wave composes the
// unit's map, publishes it, takes the state entering the unit by decoupled
// look-back over earlier units of the same (batch, tile), and publishes the
// leaving state. Every wave then applies the maps of the waves before it to
// that state and replays its K steps, storing h at every step.
template <int NW, int K, typename TIn, typename TOut, bool VEC, bool M1>
__global__ __launch_bounds__(NW * 64) void ms_unit_kernel(const MsParams p, const MsUnitWs ws) {
  static_assert(K == 16, "the m == 1 path keeps one step per lane column");
  __shared__ float sP[NW][256];  // wave maps: P row-major (A-operand order readable)
  __shared__ float sL[NW][256];  // wave maps: L in result-register order
  __shared__ float sX[256];      // last wave: transpose scratch, then the unit's entering state
  __shared__ uint32_t sUnit;

  const int tid = int(threadIdx.x);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: index math stays scalar
  const int lane = tid & 63;
  const int r = lane >> 4, c = lane & 15;

  // One counter increment per workgroup, in launch order: every unit this one
  // waits for was taken earlier by a running workgroup, so look-back progresses.
  if (tid == 0) sUnit = __hip_atomic_fetch_add(ws.header, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t unit = __builtin_amdgcn_readfirstlane(sUnit);
  if (unit >= ws.num_units) return;

  const uint32_t num_bt = uint32_t(p.num_batch) * uint32_t(ws.col_tiles);
  const uint32_t chunk = unit / num_bt;  // chunk-major: all tiles' chunk 0 first
  const uint32_t bt = unit % num_bt;
  const int64_t batch = bt / uint32_t(ws.col_tiles);
  const int ct = int(bt % uint32_t(ws.col_tiles));
  const int n = p.n, m = p.m;
  const int cc = ct * 16 + c;
  const int mt = min(16, m - ct * 16);
  const bool live = c < mt;

  int64_t off[3];
  index_offsets(p.batch, batch, off);
  const TIn* a0 = static_cast<const TIn*>(p.a) + off[MS_A];
  const TIn* b0 = static_cast<const TIn*>(p.b) + off[MS_B];
  TOut* o0 = static_cast<TOut*>(p.out) + off[MS_OUT];
  const int64_t T = p.T;
  const int64_t q0 = int64_t(chunk) * (NW * K) + int64_t(wave) * K;  // this wave's first scan position
  const int64_t ta = p.reverse ? -p.t_stride[MS_A] : p.t_stride[MS_A];
  const int64_t tb = p.reverse ? -p.t_stride[MS_B] : p.t_stride[MS_B];
  const int64_t to = p.reverse ? -p.t_stride[MS_OUT] : p.t_stride[MS_OUT];
  const int64_t t0 = p.reverse ? T - 1 - q0 : q0;  // time of scan position q0
  const bool vec_b1 = VEC && M1;                   // b[t] and out[t] are 16 contiguous, aligned values

  // ---- load the wave's K steps (scan position q0 + k is time t0 +/- k). Steps past the end
  // become the identity map; their loads read the last step instead, so that no load sits
  // behind a branch and all of them are in flight together.
  ARow<TIn> A[K];
  BCol<TIn> Bv[M1 ? 1 : K];
  const ARow<TIn> eye = identity_a<TIn>(r, c);
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t kk = q0 + k < T ? int64_t(k) : T - 1 - q0;
    A[k] = select_a(q0 + k < T, load_a<TIn, VEC>(a0 + (t0 * p.t_stride[MS_A] + kk * ta), n, r, c), eye);
    if constexpr (!M1) Bv[k] = select_b(q0 + k < T, load_b(b0 + (t0 * p.t_stride[MS_B] + kk * tb), n, m, r, cc));
  }
  f32x4 b1 = zero4();
  if constexpr (M1) {
    const int64_t kc = q0 + c < T ? int64_t(c) : T - 1 - q0;
    b1 = load_b_col1(b0 + (t0 * p.t_stride[MS_B] + kc * tb), n, r, vec_b1);
    if (q0 + c >= T) b1 = zero4();
  }
  __builtin_amdgcn_sched_barrier(0);  // all loads issued before the first product waits on any of them
  auto bterm = [&](auto kc) -> f32x4 {
    constexpr int k = decltype(kc)::value;
    if constexpr (M1) return col0_from_lane<k>(b1, c);
    else return Bv[k].get();
  };

  // ---- the wave's map: P = a[last] ... a[first], L = the scan of its steps from h = 0
  f32x4 P = identity_d(r, c), L = zero4();
  [&]<int... ks>(std::integer_sequence<int, ks...>) {
    ((P = mfma_16x16x16(A[ks].get(), P, zero4()), L = mfma_16x16x16(A[ks].get(), L, bterm(std::integral_constant<int, ks>{}))), ...);
  }(std::make_integer_sequence<int, K>{});
#pragma unroll
  for (int v = 0; v < 4; ++v) sP[wave][(4 * r + v) * 16 + c] = P[v];
  *reinterpret_cast<f32x4*>(&sL[wave][lane * 4]) = L;
  __syncthreads();

  const uint32_t slot = bt * ws.chunks + chunk;
  if (wave == NW - 1) {
    // the unit's map G = M_{NW-1} o ... o M_0, composed in scan order
    f32x4 G = identity_d(r, c), GL = zero4();
    for (int i = 0; i < NW; ++i) {
      const f32x4 Pa = *reinterpret_cast<const f32x4*>(&sP[i][c * 16 + 4 * r]);
      const f32x4 Li = *reinterpret_cast<const f32x4*>(&sL[i][lane * 4]);
      G = mfma_16x16x16(Pa, G, zero4());
      GL = mfma_16x16x16(Pa, GL, Li);
    }
    f32x4 h_in = zero4();
    if (chunk == 0) {
      if (live) dev_store4(ws.H + size_t(slot) * 256 + lane * 4, GL);  // entering 0: leaving = B
      raise_flag(ws.flags + slot, kFlagInclusive, lane);
    } else {
      const f32x4 GA = to_a_operand(sX, G, r, c);
      dev_store4(ws.P + size_t(slot) * 256 + c * 16 + 4 * r, GA);
      if (live) dev_store4(ws.L + size_t(slot) * 256 + lane * 4, GL);
      raise_flag(ws.flags + slot, kFlagAggregate, lane);

      // Look back: scan up to 64 earlier units at once for the nearest one whose
      // leaving state is published, with every unit in between at least aggregated.
      const uint32_t base = bt * ws.chunks;
      int hi = int(chunk) - 1, j = 0;
      uint32_t spins = 0;
      for (;;) {
        const int cand = hi - lane;
        uint32_t f = 0;
        if (cand >= 0) f = __hip_atomic_load(ws.flags + base + cand, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t inc = __ballot(cand >= 0 && f == kFlagInclusive);
        const uint64_t none = __ballot(cand >= 0 && f == 0);
        if (inc != 0) {
          const int l = __ffsll((unsigned long long)inc) - 1;
          if ((none & ((1ull << l) - 1ull)) == 0) {
            j = hi - l;
            break;
          }
        } else if (none == 0 && hi >= 64) {
          hi -= 64;  // 64 aggregates and no leaving state yet: look further back
          continue;
        }
        __builtin_amdgcn_s_sleep(1);
        if (++spins == kSpinLimit || hi < 0) {  // never hang: record it and go on
          if (lane == 0) __hip_atomic_store(ws.header + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          j = 0;
          break;
        }
      }
      // state leaving unit j, then the maps of units j+1 .. chunk-1 in scan order, four at a time
      if (live) h_in = dev_load4(ws.H + size_t(base + j) * 256 + lane * 4);
      for (int i = j + 1; i < int(chunk); i += 4) {
        f32x4 Pb[4], Lb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          Pb[u] = zero4();
          Lb[u] = zero4();
          if (i + u < int(chunk)) {
            Pb[u] = dev_load4(ws.P + size_t(base + i + u) * 256 + c * 16 + 4 * r);
            if (live) Lb[u] = dev_load4(ws.L + size_t(base + i + u) * 256 + lane * 4);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (i + u < int(chunk)) h_in = mfma_16x16x16(Pb[u], h_in, Lb[u]);
      }
      const f32x4 h_out = mfma_16x16x16(GA, h_in, GL);
      if (live) dev_store4(ws.H + size_t(slot) * 256 + lane * 4, h_out);
      raise_flag(ws.flags + slot, kFlagInclusive, lane);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    *reinterpret_cast<f32x4*>(&sX[lane * 4]) = h_in;
  }
  __syncthreads();

  // ---- this wave's entering state: the unit's, carried through the waves before it
  f32x4 h = *reinterpret_cast<const f32x4*>(&sX[lane * 4]);
  for (int i = 0; i < wave; ++i)
    h = mfma_16x16x16(*reinterpret_cast<const f32x4*>(&sP[i][c * 16 + 4 * r]), h,
                      *reinterpret_cast<const f32x4*>(&sL[i][lane * 4]));

  // ---- replay the wave's steps, storing every h[t]
  [&]<int... ks>(std::integer_sequence<int, ks...>) {
    (([&] {
       if (q0 + ks < T) {
         h = mfma_16x16x16(A[ks].get(), h, bterm(std::integral_constant<int, ks>{}));
         TOut* op = o0 + (t0 * p.t_stride[MS_OUT] + ks * to);
         if constexpr (M1) {
           if (c == 0) store_h_col1(op, h, n, r, vec_b1);
         } else {
           store_h(op, h, n, m, r, cc);
         }
       }
     }()),
     ...);
  }(std::make_integer_sequence<int, K>{});
}

__global__ void fill_u32_kernel(uint32_t* p, size_t count) {
  const size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0u;
}

constexpr int kWaves = 8;
constexpr int kSteps = 16;
constexpr int kUnitSteps = kWaves * kSteps;

struct UnitPlan {
  int col_tiles;
  uint64_t chunks, num_units;
  size_t flags_bytes, block_bytes, total;
};

UnitPlan unit_plan(const MsParams& p) {
  UnitPlan u{};
  u.chunks = uint64_t((p.T + kUnitSteps - 1) / kUnitSteps);
  u.col_tiles = (p.m + 15) / 16;
  u.num_units = u.chunks * uint64_t(p.num_batch) * uint64_t(u.col_tiles);
  u.flags_bytes = (u.num_units * 4 + 255) / 256 * 256;
  u.block_bytes = size_t(u.num_units) * 256 * sizeof(float);
  u.total = 256 + u.flags_bytes + 3 * u.block_bytes;
  return u;
}

template <typename TIn, typename TOut>
hipError_t launch_serial(const MsParams& p, hipStream_t stream) {
  const int64_t blocks = p.num_batch * ((p.m + 15) / 16);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((ms_serial_kernel<TIn, TOut>), dim3(unsigned(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename TIn, typename TOut, bool M1>
void launch_unit_variant(const MsParams& p, const MsUnitWs& ws, bool vec, unsigned blocks, hipStream_t stream) {
  if (vec)
    hipLaunchKernelGGL((ms_unit_kernel<kWaves, kSteps, TIn, TOut, true, M1>), dim3(blocks), dim3(kWaves * 64), 0,
                       stream, p, ws);
  else
    hipLaunchKernelGGL((ms_unit_kernel<kWaves, kSteps, TIn, TOut, false, M1>), dim3(blocks), dim3(kWaves * 64), 0,
                       stream, p, ws);
}

template <typename TIn, typename TOut>
hipError_t launch_chunked(const MsParams& p, void* workspace, hipStream_t stream) {
  const UnitPlan up = unit_plan(p);
  char* base = static_cast<char*>(workspace);
  MsUnitWs ws;
  ws.header = reinterpret_cast<uint32_t*>(base);
  ws.flags = reinterpret_cast<uint32_t*>(base + 256);
  ws.P = reinterpret_cast<float*>(base + 256 + up.flags_bytes);
  ws.L = ws.P + up.num_units * 256;
  ws.H = ws.L + up.num_units * 256;
  ws.num_units = uint32_t(up.num_units);
  ws.chunks = uint32_t(up.chunks);
  ws.col_tiles = up.col_tiles;

  // the unit counter, the status word and every flag start at zero
  const size_t words = (256 + up.flags_bytes) / 4;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(unsigned((words + 255) / 256)), dim3(256), 0, stream, ws.header, words);
  // Vector access needs n == 16 and every a[t] (and, for m == 1, b[t] and out[t]) aligned
  // to four elements' width.
  const int64_t va = 4 * int64_t(sizeof(TIn)), vo = 4 * int64_t(sizeof(TOut));
  bool vec = p.n == 16 && reinterpret_cast<uintptr_t>(p.a) % uintptr_t(va) == 0 &&
             (p.t_stride[MS_A] * int64_t(sizeof(TIn))) % va == 0;
  for (int d = 0; d < p.batch.nd && vec; ++d) vec = (p.batch.st[MS_A][d] * int64_t(sizeof(TIn))) % va == 0;
  const bool m1 = p.m == 1;
  if (m1 && vec) {
    vec = reinterpret_cast<uintptr_t>(p.b) % uintptr_t(va) == 0 && reinterpret_cast<uintptr_t>(p.out) % uintptr_t(vo) == 0 &&
          (p.t_stride[MS_B] * int64_t(sizeof(TIn))) % va == 0 && (p.t_stride[MS_OUT] * int64_t(sizeof(TOut))) % vo == 0;
    for (int d = 0; d < p.batch.nd && vec; ++d)
      vec = (p.batch.st[MS_B][d] * int64_t(sizeof(TIn))) % va == 0 && (p.batch.st[MS_OUT][d] * int64_t(sizeof(TOut))) % vo == 0;
  }
  const unsigned blocks = unsigned(up.num_units);
  if (m1) launch_unit_variant<TIn, TOut, true>(p, ws, vec, blocks, stream);
  else launch_unit_variant<TIn, TOut, false>(p, ws, vec, blocks, stream);
  return hipGetLastError();
}

}  // namespace

size_t matrix_scan_workspace(const MsParams& p) {
  if (p.num_batch <= 0 || p.T <= 0 || p.n == 0 || p.m == 0) return 0;
  const UnitPlan up = unit_plan(p);
  if (up.num_units > 0x7fffffffull) return 0;  // beyond 32-bit unit ids: the serial kernel takes it
  return up.total;
}

hipError_t launch_matrix_scan(const MsParams& p, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (p.num_batch <= 0 || p.T <= 0 || p.n == 0 || p.m == 0) return hipSuccess;
  const size_t need = matrix_scan_workspace(p);
  if (need > 0 && workspace != nullptr && workspace_bytes >= need) {
    if (p.in_bf16)
      return p.out_bf16 ? launch_chunked<uint16_t, uint16_t>(p, workspace, stream)
                        : launch_chunked<uint16_t, float>(p, workspace, stream);
    return p.out_bf16 ? launch_chunked<float, uint16_t>(p, workspace, stream)
                      : launch_chunked<float, float>(p, workspace, stream);
  }
  if (p.in_bf16)
    return p.out_bf16 ? launch_serial<uint16_t, uint16_t>(p, stream) : launch_serial<uint16_t, float>(p, stream);
  return p.out_bf16 ? launch_serial<float, uint16_t>(p, stream) : launch_serial<float, float>(p, stream);
}

}  // namespace sx
