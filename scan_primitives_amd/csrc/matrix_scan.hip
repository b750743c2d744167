// matrix_scan.hip: matrix-scan kernels for gfx950.
//
// "Tensor operations" (SexpGPU docs), Operations table (matrix-scan row) and
// the "matrix-scan" section: h[t] = a[t] @ h[t-1] + b[t] from h = 0, one
// matrix product a step, computed in f32 (bf16 operands widen exactly);
// :reverse runs from the end, h[t] = a[t] @ h[t+1] + b[t] from h[T] = 0.
//
// Kernels here (all single pass: inputs are read from HBM once):
//   ms_lead_kernel    the pipelined scan for n = 16 (m = 1, or bf16 with m a
//                     multiple of 16). Persistent workgroups of six compute
//                     waves, a leader wave and a loader wave take units of 96
//                     scan steps of one (batch, 16-column tile) from a counter.
//                     The loader copies a unit's a and b straight into LDS;
//                     each compute wave summarises its 16 steps into an affine
//                     map with MFMA and composes it onto the maps of the
//                     waves before it; the leader publishes the unit's map,
//                     finds the state entering the unit by decoupled
//                     look-back over earlier units, and hands it back; the
//                     compute waves replay their steps from it, storing every
//                     h[t]. In the gradient's adjoint scan (f32, m = 1) the
//                     replay can also form grad_a[t] = lam[t] h[prev]^T
//                     (template flag FOLD), with h staged beside a and b.
//   ms_unit_kernel    the same scan with one workgroup of eight waves per unit
//                     of 128 steps and inputs loaded into registers; it takes
//                     every shape and alignment the pipelined kernel does not.
//   ms_serial_kernel  one 256-thread block per (batch, 16-column tile of m):
//                     thread (i, j) owns h[i][j]; every step stages a[t] in
//                     LDS and forms row i of a[t] @ h with a k-ordered FMA
//                     chain. Serial in time; used when the look-back state
//                     would not fit 32-bit unit ids.
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
#include <algorithm>
#include <atomic>
#include <mutex>
#include <utility>

#include "ms_mfma.hpp"
#include "sx_common.hpp"

namespace sx {
namespace {


__device__ __forceinline__ float load_elem(const float* p) { return *p; }
__device__ __forceinline__ float load_elem(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void store_elem(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_elem(uint16_t* p, float v) { *p = f32_to_bf16_rne(v); }

// ------------------------------------------------------------------ serial kernel

// ADJ (all kernels here): the step at scan position q multiplies by the
// transpose of a at position q - 1 (position 0 at q = 0, where the state it
// multiplies is zero). That is the adjoint recurrence of a matrix scan.
template <typename TIn, typename TOut, bool ADJ = false>
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
  const TIn* ap = static_cast<const TIn*>(p.a) + off[MS_A] + (in_a ? (ADJ ? j * n + i : i * n + j) : 0);
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
    const int64_t da_next = (ADJ && t == 0) ? 0 : da;  // ADJ: steps 0 and 1 both use position 0
    if (t + 1 < T) {  // next step's operands, loaded ahead of this step's product
      an = in_a ? load_elem(ap + da_next) : 0.0f;
      bn = in_h ? load_elem(bp + db) : 0.0f;
    }
    sa[i][j] = av;
    __syncthreads();
    float acc = bv;
    for (int k = 0; k < n; ++k) acc = fmaf(sa[i][k], sh[k][j], acc);
    __syncthreads();
    sh[i][j] = acc;
    if (in_h) store_elem(op, acc);
    ap += da_next;
    bp += db;
    op += dout;
  }
}

// ------------------------------------------------------------------ chunked kernel

// Look-back state of the chunked kernels, carved out of the caller's workspace.
// Slot s = bt * chunks + chunk: bt is the (batch, 16-column tile) index.
//
// The workspace is zero-filled once by its owner; every call then leaves it
// ready for the next one. Each call works under an epoch, one more than the
// last call's (stored in the header, never 0): a flag counts only if it carries
// this call's epoch (and a fixed bit pattern beside it, so that no leftover
// value of another kind passes for one), so what earlier calls left is never
// mistaken for this one's, and nothing needs clearing between calls. The last
// workgroup to finish resets the unit counter and the finish count and stores
// the epoch. A look-back that gives up (its spin limit) sets the status word,
// which stays set until the host reads and clears it.
//
// A flag is raised only after the stores of what it announces have completed,
// so a reader that sees this call's flag reads this call's values.
constexpr uint32_t kFlagMagic = 0x5a3c0000u;  // low half of a raised flag: magic | kind
constexpr uint32_t kFlagAggregate = 1;        // the unit's map (A, B) is published
constexpr uint32_t kFlagInclusive = 2;        // the state leaving the unit is published

struct MsUnitWs {
  uint32_t* header;  // [0] next unit id, [1] status (nonzero: a look-back gave up), [2] epoch of the last call,
                     // [3] workgroups of this call that have finished
  uint64_t* flags;   // per slot: (epoch << 32) | kFlagMagic | kind
  float* P;          // per slot, the unit's A: row c, entries 4r .. 4r+3 from lane index 4c + r (see pub_store4)
  float* L;          // per slot, the unit's B in result-register order, lane index = lane
  float* H;          // per slot, the state leaving the unit, same order as L
  uint32_t num_units;
  uint32_t chunks;   // units per bt along the scan axis
  int col_tiles;     // ceil(m / 16)
  uint32_t spin_limit;  // polls a look-back makes before it gives up
};

__device__ __forceinline__ uint32_t call_epoch(const MsUnitWs& ws) {
  const uint32_t last = __hip_atomic_load(ws.header + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return last >= 0x3fffffffu ? 1u : last + 1u;
}

// One thread per workgroup, after every wave of the workgroup is done with the
// unit counter: the last workgroup of the call resets the counters and records
// the epoch for the next call.
__device__ __forceinline__ void finish_call(const MsUnitWs& ws, uint32_t epoch) {
  const uint32_t done = __hip_atomic_fetch_add(ws.header + 3, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (done == gridDim.x - 1) {
    __hip_atomic_store(ws.header + 0, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(ws.header + 3, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(ws.header + 2, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The kind of a flag raised in this call, 0 for anything else.
__device__ __forceinline__ uint32_t flag_kind(uint64_t f, uint32_t epoch) {
  return (uint32_t(f >> 32) == epoch && (uint32_t(f) & 0xffff0000u) == kFlagMagic) ? (uint32_t(f) & 3u) : 0u;
}

// Raises a flag once every earlier memory access of this wave has completed.
__device__ __forceinline__ void raise_flag(uint64_t* flag, uint32_t kind, uint32_t epoch, int lane) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (lane == 0)
    __hip_atomic_store(flag, (uint64_t(epoch) << 32) | kFlagMagic | kind, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t read_flag(const uint64_t* flag, uint32_t epoch) {
  return flag_kind(__hip_atomic_load(const_cast<uint64_t*>(flag), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT), epoch);
}

// Four published values of one lane, written and read with relaxed
// agent-scope atomic accesses: workgroups that exchange them may sit on
// different XCDs, whose L2 caches are not coherent with each other, and these
// accesses are (by the memory model), with no cache write-back or invalidate.
// A published 16x16 block holds value q of lane index i at word 64 q + i, so
// that each of the four 32-bit accesses of a wave covers 256 contiguous bytes
// (with the four values of a lane side by side, each access would touch a
// quarter of every 64-byte piece of the block, and each piece would be
// written four times).
__device__ __forceinline__ void pub_store4(float* block, int i, f32x4 v) {
  uint32_t* u = reinterpret_cast<uint32_t*>(block) + i;
#pragma unroll
  for (int q = 0; q < 4; ++q) __hip_atomic_store(u + 64 * q, __float_as_uint(v[q]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ f32x4 pub_load4(const float* block, int i) {
  const uint32_t* u = reinterpret_cast<const uint32_t*>(block) + i;
  f32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    v[q] = __uint_as_float(__hip_atomic_load(const_cast<uint32_t*>(u + 64 * q), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  return v;
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

// a X + C for a staged a: bf16 a on the bf16 MFMA (X split in two halves), f32 a on the f32 MFMA.
template <typename TIn>
__device__ __forceinline__ f32x4 mfma_a(const ARow<TIn>& a, f32x4 x, f32x4 c) {
  if constexpr (sizeof(TIn) == 2) return mfma_16x16x16_bf16a(a.u, x, c);
  else return mfma_16x16x16(a.v, x, c);
}

template <typename TIn, bool VEC, bool ADJ = false>
__device__ __forceinline__ ARow<TIn> load_a(const TIn* ap, int n, int r, int c) {
  ARow<TIn> out;
  if constexpr (ADJ) {
    // row c of the transpose is column c of a: a[4r .. 4r+3][c], clamped indices, zero past n
    uint16_t h[4];
    float f[4];
    const int col = c < n ? c : n - 1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool in = c < n && 4 * r + q < n;
      const int row = 4 * r + q < n ? 4 * r + q : n - 1;
      const TIn v = ap[row * n + col];
      if constexpr (sizeof(TIn) == 4) f[q] = in ? float(v) : 0.0f;
      else h[q] = in ? uint16_t(v) : uint16_t(0);
    }
    if constexpr (sizeof(TIn) == 4) out.v = f32x4{f[0], f[1], f[2], f[3]};
    else out.u = make_uint2(h[0] | (uint32_t(h[1]) << 16), h[2] | (uint32_t(h[3]) << 16));
  } else if constexpr (VEC && sizeof(TIn) == 4) {
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

// Decoupled look-back for the unit at position `chunk` of the slots starting at
// `base` (one (batch, column tile)): finds the nearest earlier unit whose leaving
// state is published, with every unit in between at least aggregated (a window
// of 64 flags per poll, one per lane), then applies the maps of the units in
// between to that state in scan order. Returns the state entering the unit in
// result-register order (zero in lanes past the tile's columns). The spin limit
// bounds the wait: a look-back that reaches it records the give-up in the status
// word and returns whatever it has, so no wave can hang. idle() runs between
// polls that found the look-back unresolved (before the wave sleeps).
struct NoIdle {
  __device__ void operator()() const {}
};
template <typename Idle = NoIdle>
__device__ __forceinline__ f32x4 look_back(const MsUnitWs& ws, uint32_t base, int chunk, bool live, int lane, int r,
                                           int c, uint32_t epoch, Idle&& idle = Idle{}) {
  int hi = chunk - 1, j = 0;
  uint32_t spins = 0;
  bool gave_up = false;
  auto poll = [&]() -> uint32_t {
    const int cand = hi - lane;
    return cand >= 0 ? read_flag(ws.flags + base + cand, epoch) : 0u;
  };
  uint32_t f = poll();
  for (;;) {
    const uint64_t inc = __ballot(hi - lane >= 0 && f == kFlagInclusive);
    const uint64_t none = __ballot(hi - lane >= 0 && f == 0);
    if (inc != 0) {
      const int l = __ffsll((unsigned long long)inc) - 1;
      if ((none & ((1ull << l) - 1ull)) == 0) {
        j = hi - l;
        break;
      }
    } else if (none == 0 && hi >= 64) {
      hi -= 64;  // 64 aggregates and no leaving state yet: look further back
      f = poll();
      continue;
    }
    if (++spins >= ws.spin_limit || hi < 0) {
      gave_up = true;
      j = 0;
      break;
    }
    idle();
    __builtin_amdgcn_s_sleep(1);
    f = poll();
  }
  // the state leaving unit j, then the maps of units j+1 .. chunk-1 in scan order, eight at a time
  f32x4 h = zero4();
  if (live) h = pub_load4(ws.H + size_t(base + j) * 256, lane);
  for (int i = j + 1; i < chunk; i += 8) {
    f32x4 Pb[8], Lb[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      Pb[u] = zero4();
      Lb[u] = zero4();
      if (i + u < chunk) {
        Pb[u] = pub_load4(ws.P + size_t(base + i + u) * 256, 4 * c + r);
        if (live) Lb[u] = pub_load4(ws.L + size_t(base + i + u) * 256, lane);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (i + u < chunk) h = mfma_16x16x16(Pb[u], h, Lb[u]);
  }
  if (gave_up && lane == 0) __hip_atomic_store(ws.header + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return h;
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
template <int NW, int K, typename TIn, typename TOut, bool VEC, bool M1, bool ADJ>
__device__ __forceinline__ void ms_unit_body(const MsParams& p, const MsUnitWs& ws, uint32_t unit, uint32_t epoch,
                                             float (*sP)[256], float (*sL)[256], float* sX) {
  const int tid = int(threadIdx.x);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int r = lane >> 4, c = lane & 15;

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
    int64_t ka = kk;  // a's position, relative to q0
    if constexpr (ADJ) ka = q0 + kk > 0 ? kk - 1 : -q0;
    A[k] = select_a(q0 + k < T, load_a<TIn, VEC, ADJ>(a0 + (t0 * p.t_stride[MS_A] + ka * ta), n, r, c), eye);
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
    ((P = mfma_a<TIn>(A[ks], P, zero4()), L = mfma_a<TIn>(A[ks], L, bterm(std::integral_constant<int, ks>{}))), ...);
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
      if (live) pub_store4(ws.H + size_t(slot) * 256, lane, GL);  // entering 0: leaving = B
      raise_flag(ws.flags + slot, kFlagInclusive, epoch, lane);
    } else {
      const f32x4 GA = to_a_operand(sX, G, r, c);
      pub_store4(ws.P + size_t(slot) * 256, 4 * c + r, GA);
      if (live) pub_store4(ws.L + size_t(slot) * 256, lane, GL);
      raise_flag(ws.flags + slot, kFlagAggregate, epoch, lane);
      h_in = look_back(ws, bt * ws.chunks, int(chunk), live, lane, r, c, epoch);
      const f32x4 h_out = mfma_16x16x16(GA, h_in, GL);
      if (live) pub_store4(ws.H + size_t(slot) * 256, lane, h_out);
      raise_flag(ws.flags + slot, kFlagInclusive, epoch, lane);
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
         h = mfma_a<TIn>(A[ks], h, bterm(std::integral_constant<int, ks>{}));
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

template <int NW, int K, typename TIn, typename TOut, bool VEC, bool M1, bool ADJ = false>
__global__ __launch_bounds__(NW * 64) void ms_unit_kernel(const MsParams p, const MsUnitWs ws) {
  static_assert(K == 16, "the m == 1 path keeps one step per lane column");
  __shared__ float sP[NW][256];  // wave maps: P row-major (A-operand order readable)
  __shared__ float sL[NW][256];  // wave maps: L in result-register order
  __shared__ float sX[256];      // last wave: transpose scratch, then the unit's entering state
  __shared__ uint32_t sUnit;

  const int tid = int(threadIdx.x);
  // One counter increment per workgroup, in launch order: every unit this one
  // waits for was taken earlier by a running workgroup, so look-back progresses.
  if (tid == 0) sUnit = __hip_atomic_fetch_add(ws.header, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t unit = __builtin_amdgcn_readfirstlane(sUnit);
  const uint32_t epoch = call_epoch(ws);
  if (unit < ws.num_units) ms_unit_body<NW, K, TIn, TOut, VEC, M1, ADJ>(p, ws, unit, epoch, sP, sL, sX);
  __syncthreads();
  if (tid == 0) finish_call(ws, epoch);
}


// ------------------------------------------------------------------ pipelined kernel
//
// ms_lead_kernel (below) keeps the unit scheme of ms_unit_kernel (wave maps,
// composed per unit, decoupled look-back) but overlaps everything that waits:
// the inputs of the next unit stream into LDS while the current one is
// computed, and a dedicated leader wave does the look-back of one unit while
// the compute waves summarise the next.
//
// Layout choices that make every LDS read of a stage linear (conflict-free):
//   a (f32):  the 16-byte piece a[c][4r..4r+3] that lane (r, c) reads sits
//             at slot 16 r + c of the step's 1 KB block;
//   a (bf16): the 16-byte piece a[c][8p..8p+7] sits at slot c + 16 p of the
//             step's 512-byte block, and lane (r, c) reads its half r % 2
//             of slot c + 16 (r / 2);
//   b:        the same two patterns, with rows of b (m = 16 tiles) or the
//             16 steps of one wave (m = 1) in place of the rows of a.
// For m a multiple of 16 (bf16 only) b is staged row by row and read back in
// result-register order (rows 4r..4r+3 of column c, four 2-byte reads); the
// output goes the other way through a per-wave LDS slot, so that every lane
// stores 16 contiguous bytes of one row.

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

// The LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const uint32_t* w) {
  return uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const uint32_t*)w));
}

// Cache policy of the input copies: non-temporal (each input is read once).
constexpr int kCopyPolicy = 2;

// Lane i's 16 bytes at src land in LDS at dst + 16 i (dst is the same for the
// whole wave). The copy is counted by vmcnt until its bytes are in LDS.
__device__ __forceinline__ void copy16_to_lds(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds((global_void_ptr)const_cast<void*>(src), (lds_void_ptr)dst, 16, 0, kCopyPolicy);
}

// The same with the LDS destination as a byte address (no generic-pointer
// conversion, hence no null test, on the copy path).
__device__ __forceinline__ void copy16_to_lds_at(const void* src, uint32_t lds_byte) {
  __builtin_amdgcn_global_load_lds((global_void_ptr)const_cast<void*>(src), (lds_void_ptr)(uintptr_t)lds_byte, 16, 0, kCopyPolicy);
}

template <typename TIn, bool M1>
struct PipeStage {
  static constexpr int kA = 16 * 16 * int(sizeof(TIn));                // one a[t]
  static constexpr int kB = M1 ? 16 * int(sizeof(TIn)) : kA;           // one b[t] (a 16-column tile)
  static constexpr int kWave = 16 * (kA + kB);                         // one wave's 16 steps
  static constexpr int kPiecesA = sizeof(TIn) == 4 ? 16 : 8;           // 1 KB copies of a
  static constexpr int kPieces = kPiecesA + (M1 ? 1 : 8);              // ... and of b
};

// Where one wave's 16 steps of a unit live.
struct PipeGeo {
  uint32_t chunk, bt, batch;
  int ct;
  int64_t q0;  // scan position of the wave's first step
  int64_t t0;  // its time index
  int64_t off[3];
};

__device__ __forceinline__ PipeGeo pipe_geo(const MsParams& p, const MsUnitWs& ws, uint32_t unit, int wave, int kUnit) {
  PipeGeo g;
  const uint32_t num_bt = uint32_t(p.num_batch) * uint32_t(ws.col_tiles);
  g.chunk = unit / num_bt;
  g.bt = unit % num_bt;
  g.ct = int(g.bt % uint32_t(ws.col_tiles));
  const uint32_t batch = g.bt / uint32_t(ws.col_tiles);
  g.batch = batch;
  if (p.batch.nd == 1) {  // one leading dimension (the usual case): no 64-bit divisions
#pragma unroll
    for (int t = 0; t < 3; ++t) g.off[t] = int64_t(batch) * p.batch.st[t][0];
  } else {
    index_offsets(p.batch, int64_t(batch), g.off);
  }
  g.q0 = int64_t(g.chunk) * kUnit + int64_t(wave) * 16;
  g.t0 = p.reverse ? p.T - 1 - g.q0 : g.q0;
  return g;
}

// One wave's 16 steps of a (and of b's tile) are copied into its LDS stage by
// kPieces copy instructions of 1 KB (the bf16 m = 1 b piece is 512 bytes).
// Piece i of the stage of the wave whose steps start at g.q0 is started here.
// Steps past the end read the last step instead (they become identity steps
// when the stage is read), so every source address is valid.
// ADJ: a's step blocks are those of positions one earlier (see ms_serial_kernel);
// f32 blocks are laid out for a transposed read (see stage_to_regs): lane L
// copies the piece of row 4 ((L / 4) % 4) + L / 16 at columns 4 (L % 4) ...,
// so that LDS word 64 q + (16 r + c) holds a[4r + q][c].
template <typename TIn, bool M1, bool ADJ>
__device__ __forceinline__ void stage_piece(const MsParams& p, const PipeGeo& g, char* st, int lane, int i) {
  using S = PipeStage<TIn, M1>;
  const TIn* a0 = static_cast<const TIn*>(p.a) + g.off[MS_A] + g.t0 * p.t_stride[MS_A];
  const TIn* b0 = static_cast<const TIn*>(p.b) + g.off[MS_B] + g.t0 * p.t_stride[MS_B];
  const int64_t ta = p.reverse ? -p.t_stride[MS_A] : p.t_stride[MS_A];
  const int64_t tb = p.reverse ? -p.t_stride[MS_B] : p.t_stride[MS_B];
  const int64_t T = p.T, q0 = g.q0;
  auto clamp = [&](int k) -> int64_t { return q0 + k < T ? int64_t(k) : T - 1 - q0; };
  auto clamp_a = [&](int k) -> int64_t {  // a's position for step k, relative to q0
    const int64_t kk = clamp(k);
    if constexpr (ADJ) return q0 + kk > 0 ? kk - 1 : -q0;
    return kk;
  };
  if (i < S::kPiecesA) {
    if constexpr (sizeof(TIn) == 4 && ADJ) {
      copy16_to_lds(a0 + clamp_a(i) * ta + (4 * ((lane >> 2) & 3) + (lane >> 4)) * 16 + 4 * (lane & 3),
                    st + i * S::kA);
    } else if constexpr (sizeof(TIn) == 4) {  // step i; lane 16 r + c takes a[c][4r..4r+3]
      copy16_to_lds(a0 + clamp_a(i) * ta + (lane & 15) * 16 + 4 * (lane >> 4), st + i * S::kA);
    } else {  // steps 2i, 2i+1; lane takes a[c][8p..8p+7] for slot c + 16 p of its step
      copy16_to_lds(a0 + clamp_a(2 * i + (lane >> 5)) * ta + (lane & 15) * 16 + 8 * ((lane >> 4) & 1),
                    st + i * 2 * S::kA);
    }
    return;
  }
  char* sb = st + 16 * S::kA;
  const int c = lane & 15;
  if constexpr (M1) {  // one piece: b of all 16 steps, step c at slot c (+ 16 r or + 16 p)
    if constexpr (sizeof(TIn) == 4) copy16_to_lds(b0 + clamp(c) * tb + 4 * (lane >> 4), sb);
    else if (lane < 32) copy16_to_lds(b0 + clamp(c) * tb + 8 * (lane >> 4), sb);
  } else {  // steps 2j, 2j+1 of the tile: b[c][ct*16 + 8p ..] for slot c + 16 p
    const int j = i - S::kPiecesA;
    copy16_to_lds(b0 + clamp(2 * j + (lane >> 5)) * tb + int64_t(c) * p.m + g.ct * 16 + 8 * ((lane >> 4) & 1),
                  sb + j * 2 * S::kB);
  }
}

// All pieces of one wave's stage. When the wave's 16 steps all lie inside the
// scan (every unit but the last) the sources advance by a fixed stride from
// per-lane offsets computed once: the loader's issue rate is bound by its own
// instruction latency, so the clamped per-piece addressing is kept for the
// last unit only.
template <typename TIn, bool M1, bool ADJ>
__device__ __forceinline__ void stage_wave(const MsParams& p, const PipeGeo& g, char* st, uint32_t st_lds, int lane) {
  using S = PipeStage<TIn, M1>;
  if (g.q0 + 16 > p.T || (ADJ && g.q0 == 0)) {
#pragma unroll
    for (int i = 0; i < S::kPieces; ++i) stage_piece<TIn, M1, ADJ>(p, g, st, lane, i);
    return;
  }
  const int64_t ta = p.reverse ? -p.t_stride[MS_A] : p.t_stride[MS_A];
  const int64_t tb = p.reverse ? -p.t_stride[MS_B] : p.t_stride[MS_B];
  // ADJ: a from one position earlier (q0 >= 1 here)
  const TIn* a0 = static_cast<const TIn*>(p.a) + g.off[MS_A] + g.t0 * p.t_stride[MS_A] - (ADJ ? ta : 0);
  const TIn* b0 = static_cast<const TIn*>(p.b) + g.off[MS_B] + g.t0 * p.t_stride[MS_B];
  const int c = lane & 15;
  if constexpr (sizeof(TIn) == 4) {
    const TIn* src = ADJ ? a0 + (4 * ((lane >> 2) & 3) + (lane >> 4)) * 16 + 4 * (lane & 3) : a0 + c * 16 + 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < S::kPiecesA; ++i) copy16_to_lds_at(src + i * ta, st_lds + i * S::kA);
  } else {
    const TIn* src = a0 + (lane >> 5) * ta + c * 16 + 8 * ((lane >> 4) & 1);
#pragma unroll
    for (int i = 0; i < S::kPiecesA; ++i) copy16_to_lds_at(src + 2 * i * ta, st_lds + i * 2 * S::kA);
  }
  const uint32_t sb = st_lds + 16 * S::kA;
  if constexpr (M1) {
    if constexpr (sizeof(TIn) == 4) copy16_to_lds_at(b0 + c * tb + 4 * (lane >> 4), sb);
    else if (lane < 32) copy16_to_lds_at(b0 + c * tb + 8 * (lane >> 4), sb);
  } else {
    const TIn* src = b0 + (lane >> 5) * tb + int64_t(c) * p.m + g.ct * 16 + 8 * ((lane >> 4) & 1);
#pragma unroll
    for (int j = 0; j < 8; ++j) copy16_to_lds_at(src + 2 * j * tb, sb + j * 2 * S::kB);
  }
}

// FOLD: the forward result h at the positions one after each of the wave's 16
// steps (the step before each in the forward scan), into the wave's h area:
// lane L copies elements 4 (L % 4) .. 4 (L % 4) + 3 of position q0 + 1 + L / 4,
// so that word 16 k + j holds h[position q0 + 1 + k][j] (positions past the end
// read the last one; the replay zeroes them). h has the result's layout (m = 1).
__device__ __forceinline__ void stage_fold_h(const MsParams& p, const PipeGeo& g, uint32_t dst_lds, int lane) {
  const int64_t q = g.q0 + 1 + (lane >> 2);
  const int64_t qc = q < p.T ? q : p.T - 1;
  const int64_t t = p.reverse ? p.T - 1 - qc : qc;
  copy16_to_lds_at(static_cast<const float*>(p.fold_h) + g.off[MS_OUT] + t * p.t_stride[MS_OUT] + 4 * (lane & 3), dst_lds);
}

// A compute wave's inputs for one unit, in registers: a[t] in A-operand order
// (identity past the end) and b[t] in result-register order (zero past the end;
// for m = 1, b of all 16 steps with step c in lane column c).
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

template <typename TIn, bool M1>
struct UnitRegs {
  ARow<TIn> A[16];
  BCol<TIn> Bv[M1 ? 1 : 16];
  f32x4 b1;
  float sc;  // SCALED kernels: lane c holds the factor of the wave's step c (lanes 16 r + c alike)
};

// The factor of step k, the same in every lane (a read of lane k).
template <int k, typename R>
__device__ __forceinline__ float step_scale(const R& regs) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(regs.sc), k));
}

template <typename TIn, bool M1, bool ADJ>
__device__ __forceinline__ void stage_to_regs(UnitRegs<TIn, M1>& R, const char* st, int64_t q0, int64_t T, int lane,
                                              int r, int c) {
  using S = PipeStage<TIn, M1>;
  const ARow<TIn> eye = identity_a<TIn>(r, c);
  // bf16 b tiles: element (R, C) of a step's tile sits at byte 256 (C / 8) + 16 R + 2 (C % 8).
  // A transposing LDS read (ds_read_b64_tr_b16) gives lane (r, c) the column piece b[4r .. 4r+3][c]
  // in one instruction: within each 16-lane row, the 8-byte pieces that lanes 4q .. 4q+3 supply form
  // row q of a 4 x 16 block, and lane j receives column j of that block. So lane (r, c) supplies
  // b[4r + c/4][4 (c%4) .. 4 (c%4) + 3].
  static_assert(M1 || sizeof(TIn) == 2, "the pipelined kernel stages 16-column b tiles for bf16 only");
  uint32_t b_lds = 0;
  if constexpr (!M1)
    b_lds = lds_addr(reinterpret_cast<const uint32_t*>(st + 16 * S::kA)) + 256 * ((c & 3) >> 1) + 16 * (4 * r + (c >> 2)) +
            8 * (c & 1);
  // ADJ, the transpose of a: lane (r, c) needs a[4r .. 4r+3][c]. For f32 the loader laid the
  // block out so that these are LDS words 64 q + lane (four linear reads); a bf16 block has the
  // layout of a bf16 b tile, so the same transposing read gives the column piece.
  const uint32_t a_lds = lds_addr(reinterpret_cast<const uint32_t*>(st)) + 256 * ((c & 3) >> 1) + 16 * (4 * r + (c >> 2)) +
                         8 * (c & 1);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    if constexpr (sizeof(TIn) == 4 && ADJ) {
      const float* w = reinterpret_cast<const float*>(st + k * S::kA) + lane;
      R.A[k].v = f32x4{w[0], w[64], w[128], w[192]};
    } else if constexpr (sizeof(TIn) == 4) {
      R.A[k].v = *reinterpret_cast<const f32x4*>(st + k * S::kA + lane * 16);
    } else if constexpr (ADJ) {
      const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4_ptr>(uintptr_t(a_lds + k * S::kA)));
      R.A[k].u = make_uint2(uint32_t(uint16_t(v[0])) | (uint32_t(uint16_t(v[1])) << 16),
                            uint32_t(uint16_t(v[2])) | (uint32_t(uint16_t(v[3])) << 16));
    } else {
      R.A[k].u = *reinterpret_cast<const uint2*>(st + k * S::kA + 16 * (c + 16 * (r >> 1)) + 8 * (r & 1));
    }
    R.A[k] = select_a(q0 + k < T, R.A[k], eye);
    if constexpr (!M1) {
      const bool in = q0 + k < T;
      const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_s16x4_ptr>(uintptr_t(b_lds + k * S::kB)));
      R.Bv[k].u = make_uint2(in ? uint32_t(uint16_t(v[0])) | (uint32_t(uint16_t(v[1])) << 16) : 0u,
                             in ? uint32_t(uint16_t(v[2])) | (uint32_t(uint16_t(v[3])) << 16) : 0u);
    }
  }
  if constexpr (M1) {
    if constexpr (sizeof(TIn) == 4) {
      R.b1 = *reinterpret_cast<const f32x4*>(st + 16 * S::kA + lane * 16);
    } else {
      const uint2 u = *reinterpret_cast<const uint2*>(st + 16 * S::kA + 16 * (c + 16 * (r >> 1)) + 8 * (r & 1));
      R.b1 = f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                   __uint_as_float(u.y & 0xffff0000u)};
    }
    if (q0 + c >= T) R.b1 = zero4();
  }
}

template <typename TIn, bool M1, int k>
__device__ __forceinline__ f32x4 bterm_of(const UnitRegs<TIn, M1>& R, int c) {
  if constexpr (M1) return col0_from_lane<k>(R.b1, c);
  else return R.Bv[k].get();
}

// m = 1: the vector recurrence x <- a x + b on the VALU. A 16x16 by 16 product
// has no reuse of a, so on the MFMA it would fill one of sixteen columns (a
// sixteenth of the instruction's work); here it is 256 multiply-adds over the
// wave's 64 lanes. a is in A-operand order (lane (r, c) holds a[c][4r .. 4r+3]);
// x is held as lane (r, c) -> x[4r .. 4r+3], the same four values across each
// row of 16 lanes. Lane (r, c) forms row c's products with columns 4r .. 4r+3;
// two cross-row swaps (v_permlane16_swap, v_permlane32_swap) sum the four
// column blocks, so that every lane holds y[c]; a round trip through a wave-
// private LDS area gives lane (r, c) y[4r .. 4r+3] (row r reads its own copy).
template <typename TIn>
__device__ __forceinline__ f32x4 matvec_m1(const ARow<TIn>& A, f32x4 x, f32x4 b, float* sv, int r, int c) {
  const f32x4 a = A.get();
  float p = a[0] * x[0];
  p = fmaf(a[1], x[1], p);
  p = fmaf(a[2], x[2], p);
  p = fmaf(a[3], x[3], p);
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(p), __float_as_uint(p), false, false);
  const float q = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(q), __float_as_uint(q), false, false);
  const float y = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
  sv[16 * r + c] = y;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const f32x4 v = *reinterpret_cast<const f32x4*>(sv + 20 * r);  // words 16 r + 4 r .. +3: y[4r .. 4r+3]
  return v + b;
}

// b of the wave's step k for m = 1 in the layout above: lane (r, k) holds
// b[step k][4r .. 4r+3] (see UnitRegs), and a row broadcast of lane k gives it
// to its whole row.
template <int k>
__device__ __forceinline__ f32x4 b_row_m1(f32x4 b1) {
  f32x4 o;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(b1[q]), 0x150 + k, 0xF, 0xF, false));
  return o;
}

// An L slot (or entering state) of the pipelined kernel in LDS: a 16x16 block
// in result-register order (lane * 4 + v), or, for m = 1, only its live
// column, lanes (r, 0), at 4 r + v: the other lanes read zeros and write
// nothing (the m = 1 blocks are zero there anyway).
template <bool M1>
struct LSlot {
  static constexpr int kW = M1 ? 16 : 256;  // floats per slot
  __device__ static f32x4 load(const float* s, int lane, int r, int c) {
    if constexpr (M1) return c == 0 ? *reinterpret_cast<const f32x4*>(s + 4 * r) : zero4();
    else return *reinterpret_cast<const f32x4*>(s + lane * 4);
  }
  __device__ static void store(float* s, f32x4 v, int lane, int r, int c) {
    if constexpr (M1) {
      if (c == 0) *reinterpret_cast<f32x4*>(s + 4 * r) = v;
    } else {
      *reinterpret_cast<f32x4*>(s + lane * 4) = v;
    }
  }
};

// The wave's map: P = a[last] ... a[first] (written row-major), L = the scan of
// its steps from h = 0 (written in result-register order). issue(k) runs at
// step k: it starts the copies of the next unit, spread over the steps so that
// they never back up the memory pipeline.
// SCALED: each step's result is multiplied by its factor, h[t] = (a[t] h + b[t]) * s[t].
// KEEP (f32, m = 1): every step's prefix product P (the product of the wave's
// steps up to it, result-register order) replaces its a in R.A, and its local
// state L (the scan from zero) goes to lane (r, step) of R.b1, rows 4r .. 4r+3;
// the replay then needs neither a nor b (see replay_prefix_m1).
template <typename TIn, bool M1, bool SCALED, bool KEEP = false, typename Issue>
__device__ __forceinline__ void summarize(UnitRegs<TIn, M1>& R, float* sPw, float* sLw, float* sv, int lane,
                                          int r, int c, Issue&& issue) {
  static_assert(!KEEP || (M1 && sizeof(TIn) == 4), "prefix products are kept for f32 m = 1 only");
  f32x4 P = identity_d(r, c), L = zero4();
  [&]<int... ks>(std::integer_sequence<int, ks...>) {
    (([&] {
       issue(ks);
       P = mfma_a<TIn>(R.A[ks], P, zero4());
       if constexpr (M1) {  // L in the VALU layout of matvec_m1; from L = 0 the first step is b
         if constexpr (ks == 0) L = b_row_m1<ks>(R.b1);
         else L = matvec_m1<TIn>(R.A[ks], L, b_row_m1<ks>(R.b1), sv, r, c);
       } else {
         L = mfma_a<TIn>(R.A[ks], L, bterm_of<TIn, M1, ks>(R, c));
       }
       if constexpr (SCALED) {
         const float sk = step_scale<ks>(R);
         P *= sk;
         L *= sk;
       }
       if constexpr (KEEP) {  // (later steps read b from lanes (r, k > ks) only)
         if constexpr (sizeof(TIn) == 4) R.A[ks].v = P;
#pragma unroll
         for (int v = 0; v < 4; ++v) R.b1[v] = c == ks ? L[v] : R.b1[v];
       }
     }()),
     ...);
  }(std::make_integer_sequence<int, 16>{});
#pragma unroll
  for (int v = 0; v < 4; ++v) sPw[(4 * r + v) * 16 + c] = P[v];
  if constexpr (M1) L = c == 0 ? L : zero4();  // result-register order: column 0 only
  LSlot<M1>::store(sLw, L, lane, r, c);
}

// The replay of a KEEP summary (f32, m = 1): h[t] = P_t h + L_t for the wave's 16
// steps, independent of each other (with SCALED both already carry the steps'
// factors). Lane (r, c) holds P_t[4r+v][c] and multiplies
// it by h[c]; the 64 products of each row of 16 lanes are summed over the row by
// recursive halving, each round pairing lanes whose sets of summed lanes are
// disjoint (row rotation by 8, half-row mirror, quad reversal, quad swap), each
// lane keeping the half of the steps its lane bit picks, so that lane (r, c) ends
// with step c's rows 4r .. 4r+3, the layout of the store.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL, int N>
__device__ __forceinline__ void halve(float (&x)[2 * N], bool upper) {
  // x[i] belongs to the lower half of the steps, x[i + N] to the upper; keep this lane's half
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float keep = upper ? x[i + N] : x[i];
    const float send = upper ? x[i] : x[i + N];
    x[i] = keep + dpp_mov<CTRL>(send);
  }
}

template <typename TOut>
__device__ __forceinline__ void replay_prefix_m1(const UnitRegs<float, true>& R, f32x4 h, const MsParams& p,
                                                 const PipeGeo& g, float* sv, int r, int c) {
  // h arrives in result-register order (lanes (r, 0) hold h[4r .. 4r+3]); every lane needs h[c]
  if (c == 0) *reinterpret_cast<f32x4*>(sv + 4 * r) = h;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const float hc = sv[c];
  // x[4 t + v]: step t, row 4r + v, this lane's column's share
  float x[64];
#pragma unroll
  for (int t = 0; t < 16; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) x[4 * t + v] = R.A[t].v[v] * hc;
  // steps are halved by their bit 3, 2, 1, 0 (index bit 5, 4, 3, 2), against lane bit 3, 2, 1, 0
  halve<0x128, 32>(x, (c & 8) != 0);                                   // row_ror:8 (lane c ^ 8)
  halve<0x141, 16>(reinterpret_cast<float (&)[32]>(x), (c & 4) != 0);  // row_half_mirror (c ^ 7)
  halve<0x1B, 8>(reinterpret_cast<float (&)[16]>(x), (c & 2) != 0);    // quad_perm [3,2,1,0] (c ^ 3)
  halve<0xB1, 4>(reinterpret_cast<float (&)[8]>(x), (c & 1) != 0);     // quad_perm [1,0,3,2] (c ^ 1)
  const f32x4 out = f32x4{x[0], x[1], x[2], x[3]} + R.b1;
  if (g.q0 + c < p.T) {
    TOut* o0 = static_cast<TOut*>(p.out) + g.off[MS_OUT];
    const int64_t to = p.reverse ? -p.t_stride[MS_OUT] : p.t_stride[MS_OUT];
    TOut* op = o0 + (g.t0 * p.t_stride[MS_OUT] + c * to) + 4 * r;
    if constexpr (sizeof(TOut) == 4) st_stream(reinterpret_cast<f32x4*>(op), out);
    else st_stream(reinterpret_cast<u32x2*>(op), u32x2{pack_bf16x2(out[0], out[1]), pack_bf16x2(out[2], out[3])});
  }
}

// Replay of one wave's 16 steps from its entering state h, storing every h[t].
// Outputs leave registers without LDS round trips: for m = 1 each step's state
// (lanes (r, 0)) is moved to lanes (r, step) with a DPP shift and one store per
// lane writes all 16 steps at the end; for m = 16 a quad transpose gives each
// lane four consecutive values of one row, stored as one piece per step.
// FOLD (the gradient's adjoint scan, f32, m = 1): each step also stores
// grad_a[t] = lam[t] h[prev]^T, 16x16, where lam[t] is the state just computed
// and hb holds h at the position after each of the wave's steps (the step
// before it in the forward scan), 16 values per step; there is none after the
// last position, whose grad_a is zero. Lane (r, c) forms lam[4r .. 4r+3] times
// h[prev][c], and a quad transpose gives it four consecutive values of one row,
// so each step's 1 KiB block goes out as one contiguous store.
template <typename TIn, typename TOut, bool M1, bool SCALED, bool FOLD = false>
__device__ __forceinline__ void replay_steps(const UnitRegs<TIn, M1>& R, f32x4 h, const MsParams& p, const PipeGeo& g,
                                             float* sv, int lane, int r, int c, const float* hb = nullptr) {
  const int64_t T = p.T;
  const int m = p.m;
  TOut* o0 = static_cast<TOut*>(p.out) + g.off[MS_OUT];
  const int64_t to = p.reverse ? -p.t_stride[MS_OUT] : p.t_stride[MS_OUT];
  auto out_at = [&](int k) -> TOut* { return o0 + (g.t0 * p.t_stride[MS_OUT] + k * to); };
  // Every unit but the last has all 16 steps inside the scan. For those the
  // steps carry no test and are software-pipelined: step k's MFMA chain is
  // issued from h[k-1], then h[k-1]'s output work (gather or transpose,
  // packing, store), which needs no MFMA result still in flight, runs while
  // that chain executes.
  const bool full = g.q0 + 16 <= T;
  if constexpr (M1) {
    // the recurrence on the VALU (matvec_m1); h arrives in result-register order (column 0:
    // lanes (r, 0)) and a row broadcast of lane 0 puts it in the VALU layout
    f32x4 x;
#pragma unroll
    for (int v = 0; v < 4; ++v) x[v] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(h[v]), 0x150, 0xF, 0xF, false));
    f32x4 acc = zero4();  // lane (r, c) ends up with h[step c][4r .. 4r+3]
    float* ga0 = nullptr;
    int64_t gto = 0;
    if constexpr (FOLD) {
      ga0 = static_cast<float*>(p.fold_grad_a) + 16 * (g.off[MS_OUT] + g.t0 * p.t_stride[MS_OUT]) +
            (4 * r + (c & 3)) * 16 + 4 * (c >> 2);
      gto = 16 * to;
    }
    [&]<int... ks>(std::integer_sequence<int, ks...>) {
      (([&] {
         // steps past the end hold the identity and a zero b: x stays, and is not stored
         x = matvec_m1<TIn>(R.A[ks], x, b_row_m1<ks>(R.b1), sv, r, c);
         if constexpr (SCALED) x *= step_scale<ks>(R);
         if constexpr (FOLD) {
           const float hv = g.q0 + ks + 1 < T ? hb[ks * 16 + c] : 0.0f;
           const f32x4 row = quad_transpose(x * hv, c & 3);  // grad_a[t][4r + c % 4][4 (c / 4) ..]
           if (g.q0 + ks < T) st_stream(reinterpret_cast<f32x4*>(ga0 + ks * gto), row);
         }
#pragma unroll
         for (int v = 0; v < 4; ++v) acc[v] = c == ks ? x[v] : acc[v];
       }()),
       ...);
    }(std::make_integer_sequence<int, 16>{});
    if (g.q0 + c < T) {
      TOut* op = out_at(c) + 4 * r;
      if constexpr (sizeof(TOut) == 4) st_stream(reinterpret_cast<f32x4*>(op), acc);
      else st_stream(reinterpret_cast<u32x2*>(op), u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])});
    }
  } else {
    const int j = c & 3;
    const int64_t row_off = int64_t(4 * r + j) * m + g.ct * 16 + 4 * (c >> 2);  // row 4r+j, columns 4(c/4)..
    auto emit = [&](int ks, const f32x4& hv) {  // h[ks] to memory, four consecutive values of one row per lane
      const f32x4 t = quad_transpose(hv, j);
      TOut* op = out_at(ks) + row_off;
      if constexpr (sizeof(TOut) == 4) st_stream(reinterpret_cast<f32x4*>(op), t);
      else st_stream(reinterpret_cast<u32x2*>(op), u32x2{pack_bf16x2(t[0], t[1]), pack_bf16x2(t[2], t[3])});
    };
    if (full) {
      [&]<int... ks>(std::integer_sequence<int, ks...>) {
        (([&] {
           f32x4 hn = mfma_a<TIn>(R.A[ks], h, R.Bv[ks].get());
           if constexpr (SCALED) hn *= step_scale<ks>(R);
           if constexpr (ks > 0) emit(ks - 1, h);
           h = hn;
         }()),
         ...);
      }(std::make_integer_sequence<int, 16>{});
      emit(15, h);
    } else {
      [&]<int... ks>(std::integer_sequence<int, ks...>) {
        (([&] {
           if (g.q0 + ks < T) {
             h = mfma_a<TIn>(R.A[ks], h, R.Bv[ks].get());
             if constexpr (SCALED) h *= step_scale<ks>(R);
             emit(ks, h);
           }
         }()),
         ...);
      }(std::make_integer_sequence<int, 16>{});
    }
  }
}

// Workgroup-local signalling through LDS words. The waves of ms_lead_kernel do
// not meet at s_barrier: the leader and the compute waves run a unit apart.
// A signal is published after the wave's own earlier LDS accesses have
// completed, and a waiter reads what it waited for only after the wait.
// The signal words are accessed with inline DS instructions: for ordinary LDS
// accesses the compiler cannot tell them from the stages being filled by
// global_load_lds and would first wait for every copy in flight.

__device__ __forceinline__ uint32_t lds_read_u32(const uint32_t* w) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(w)) : "memory");
  return v;
}

__device__ __forceinline__ void lds_signal_add(uint32_t* w, int lane) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's earlier LDS accesses are done
  if (lane == 0) asm volatile("ds_add_u32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(lds_addr(w)), "v"(1u) : "memory");
}

__device__ __forceinline__ void lds_signal_set(uint32_t* w, uint32_t v, int lane) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  if (lane == 0) asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(lds_addr(w)), "v"(v) : "memory");
}

// Waits until *w >= target (unsigned, counts only grow).
__device__ __forceinline__ void lds_wait_at_least(const uint32_t* w, uint32_t target) {
  while (lds_read_u32(w) < target) __builtin_amdgcn_s_sleep(1);
}

// vmcnt(n) alone (expcnt and lgkmcnt left at their maxima), as an s_waitcnt immediate.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }

// ms_lead_kernel: NC compute waves, one leader wave and one loader wave per
// workgroup; a unit is NC * 16 scan steps of one (batch, column tile).
// Workgroups stay resident and take units one after another.
//   - The loader streams each unit's inputs from HBM into the compute waves'
//     LDS stages (global_load_lds, no registers held) as soon as a stage has
//     been read, and signals when a stage has landed. It is the only wave that
//     waits on input copies, so those waits never stall an MFMA chain.
//   - For unit k the compute waves move their stages into registers and
//     summarise their 16 steps each into an affine map (LDS, slot k % 4);
//     wave i then composes its map onto the composition of maps 0 .. i-1 that
//     wave i-1 left in its slot, leaving the composition of maps 0 .. i in
//     its own (so every wave carries the entering state in one step, and the
//     last slot holds the unit's map). Then each replays unit k-1, whose
//     entering state the leader has found in the meantime, storing every
//     h[t]. Each compute wave keeps two units in registers (the one it
//     summarises and the one it replays). For f32 m = 1 the summary keeps
//     each step's prefix product and local state in place of its a and b, and
//     the replay forms h[t] = P_t h + L_t for all 16 steps at once instead of
//     stepping through them.
//   - The leader finds the state entering unit k by decoupled look-back over
//     earlier units of the same (batch, tile), publishing the unit's map
//     while it waits (no compute wave waits for a store), hands that state to
//     the compute waves and publishes the state leaving the unit. Its round
//     trips overlap the summary of the next unit, so a replay never waits for
//     its own look-back.
// The waves run a unit apart and never meet at s_barrier after the start; they
// hand work over through LDS words. Per-unit LDS slots rotate over four
// units. Each compute wave announces its summary of unit k in a word of its
// own (set to k + 1), so the next wave composes onto it as soon as it is
// in. The carry counts that guard slot reuse are kept per slot: a count that
// several waves raise only says "all of unit k are in" if no wave can add for
// a later unit on the same count first. A compute wave summarises unit k into
// slot k % 4 only after every wave's carry of unit k-4 out of that slot; each
// wave carries its units in order and summarises unit k+1 before it carries
// unit k. So when any wave adds its carry of unit k+4 to slot k % 4, every
// wave has already added its carry of unit k there. (With one shared summary
// count, a fast wave's unit-1 summary, which has no carry to wait for, once
// stood in for a slow wave's unit-0 summary not yet written.)
//
// Placement: wave i runs on SIMD i % 4, and a wave that shares a SIMD with a
// wave running MFMA chains gets few issue slots (measured: a copy-issuing wave
// falls from 6.6 to 0.9 TB/s). So the six compute waves are waves 0, 1, 2, 4,
// 5, 6 (SIMDs 0-2, two each) and the leader (wave 3) and the loader (wave 7)
// share SIMD 3, where no MFMA chain runs.
template <int NC, typename TIn, typename TOut, bool M1, bool ADJ = false, bool SCALED = false, bool FOLD = false>
__global__ __launch_bounds__(512) void ms_lead_kernel(const MsParams p, const MsUnitWs ws) {
  static_assert(NC == 6, "compute waves fill SIMDs 0-2, two each");
  static_assert(!FOLD || (M1 && ADJ && !SCALED && sizeof(TIn) == 4 && sizeof(TOut) == 4), "grad_a folds into the f32 m = 1 adjoint");
  constexpr int K = 16, kUnit = NC * K, LEADER = 3, LOADER = 7;
  // f32 m = 1 without the gradient fold: the summary keeps its prefix products and the replay uses them
  constexpr bool kKeep = M1 && sizeof(TIn) == 4 && !FOLD;
  using S = PipeStage<TIn, M1>;
  constexpr int kPieces = S::kPieces + (FOLD ? 1 : 0);  // copies per stage (FOLD: one more, for h)
  static_assert(3 * kPieces <= 63, "the loader keeps up to three stages in flight");
  __shared__ __attribute__((aligned(16))) char sStage[NC][S::kWave];
  // Per-unit LDS slots (wave maps, entering state and their signals) rotate
  // over kBufs units, so that a wave can run up to kBufs - 2 units ahead of
  // the slowest wave's carry before it has to wait.
  constexpr int kBufs = 4;
  __shared__ __attribute__((aligned(16))) float sP[kBufs][NC][256];
  __shared__ __attribute__((aligned(16))) float sL[kBufs][NC][LSlot<M1>::kW];
  __shared__ __attribute__((aligned(16))) float sX[kBufs][LSlot<M1>::kW];
  // FOLD: each compute wave's h values for three units (the one being staged, and the two it holds
  // in registers until their replays): the loader fills unit k's area when the wave frees its stage
  // of unit k-1, which it does after replaying unit k-3, the area's last user.
  __shared__ __attribute__((aligned(16))) float sH[FOLD ? 3 : 1][NC][FOLD ? 256 : 4];
  __shared__ __attribute__((aligned(16))) float sV[NC][M1 ? 64 : 4];  // m = 1: each compute wave's matvec_m1 area
  // Unit ids in a ring of 8. The leader publishes id k+2 as it starts unit k, and
  // it starts unit k once unit k-1's summaries are in, so the readers (the
  // compute waves, the loader) may still need ids from k-1 on: four ids are live
  // at once; the ring leaves room to spare.
  constexpr int kIdRing = 8;
  __shared__ uint32_t sId[kIdRing];
  __shared__ uint32_t sIdCount, sSumDone[NC], sCarryDone[kBufs], sHinIt[kBufs], sLanded[NC], sConsumed[NC];

  const int tid = int(threadIdx.x);
  const int hw_wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // compute waves are numbered 0..NC-1 in unit step order
  const int wave = hw_wave < LEADER ? hw_wave : hw_wave - 1;
  const int lane = tid & 63;
  const int r = lane >> 4, c = lane & 15;
  const int64_t T = p.T;
  const uint32_t NU = ws.num_units;
  const uint32_t epoch = call_epoch(ws);

  if (tid == 0) {
    sIdCount = 0;
    for (int b = 0; b < kBufs; ++b) sCarryDone[b] = sHinIt[b] = 0;
  }
  if (tid < NC) {
    sSumDone[tid] = 0;
    sLanded[tid] = 0;
    sConsumed[tid] = 0;
  }
  __syncthreads();

  // Unit ids come from one counter in take order. The leader takes the id of
  // unit k+2 before it works on unit k, so that the loader can stage unit k+1
  // in time; the smallest unfinished unit is then always the one some leader
  // is working on, whose predecessors are all done, so look-back ends.
  auto unit_id = [&](int k) -> uint32_t {
    lds_wait_at_least(&sIdCount, uint32_t(k) + 1);
    return __builtin_amdgcn_readfirstlane(lds_read_u32(&sId[k % kIdRing]));
  };

  if (hw_wave == LOADER) {
    // ------------------------------------------------------------ loader
    const uint32_t stage_lds = __builtin_amdgcn_readfirstlane(lds_addr(reinterpret_cast<const uint32_t*>(&sStage[0][0])));
    // Stage w of unit k is filled once compute wave w has read unit k-1 from it,
    // in whatever order the compute waves free their stages. Up to three stages
    // are in flight; they are retired in the order they were issued (loads
    // return in order, so vmcnt(n) with n the copies issued after a stage means
    // that stage has landed), each one signalled as soon as it has landed, and
    // the queue carries over from one unit to the next, so the copies in flight
    // never drain to zero while there is a stage to fill.
    int qw[3] = {0, 0, 0}, qk[3] = {0, 0, 0};  // stages in flight, oldest first: wave and unit index
    int head = 0, n_pending = 0;
    auto retire_oldest = [&]() {
      if (n_pending == 3) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kPieces));
      else if (n_pending == 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(kPieces));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      lds_signal_set(&sLanded[qw[head]], uint32_t(qk[head]) + 1, lane);
      head = head == 2 ? 0 : head + 1;
      --n_pending;
    };
    for (int k = 0;; ++k) {
      const uint32_t unit = unit_id(k);
      if (unit >= NU) break;
      uint32_t issued = 0;  // stages of unit k started
      int n_issued = 0;
      while (n_issued < NC) {
        bool progress = false;
        for (int w = 0; w < NC; ++w) {
          if ((issued >> w) & 1u) continue;
          if (lds_read_u32(&sConsumed[w]) < uint32_t(k)) continue;
          if (n_pending == 3) retire_oldest();
          const PipeGeo gw = pipe_geo(p, ws, unit, w, kUnit);
          stage_wave<TIn, M1, ADJ>(p, gw, &sStage[w][0], stage_lds + w * S::kWave, lane);
          if constexpr (FOLD)
            stage_fold_h(p, gw, __builtin_amdgcn_readfirstlane(lds_addr(reinterpret_cast<const uint32_t*>(&sH[k % 3][w][0]))), lane);
          const int tail = head + n_pending >= 3 ? head + n_pending - 3 : head + n_pending;
          qw[tail] = w;
          qk[tail] = k;
          ++n_pending;
          issued |= 1u << w;
          ++n_issued;
          progress = true;
        }
        if (!progress) {
          if (n_pending > 0) retire_oldest();
          else __builtin_amdgcn_s_sleep(1);
        }
      }
    }
    while (n_pending > 0) retire_oldest();
  } else

  if (hw_wave == LEADER) {
    // ------------------------------------------------------------ leader
    __builtin_amdgcn_s_setprio(2);  // its look-back is on every replay's path
    auto publish_id = [&](int k, uint32_t id) {
      lds_signal_set(&sId[k % kIdRing], __builtin_amdgcn_readfirstlane(id), lane);
      lds_signal_set(&sIdCount, uint32_t(k) + 1, lane);
    };
    auto fetch_id = [&]() -> uint32_t {
      return lane == 0 ? __hip_atomic_fetch_add(ws.header, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
    };
    publish_id(0, fetch_id());
    publish_id(1, fetch_id());
    // The id of unit k+2 is published as unit k starts; it was fetched as unit
    // k-1 started, so its round trip is long over and never stalls the leader.
    uint32_t pending = fetch_id();
    for (int k = 0;; ++k) {
      publish_id(k + 2, pending);
      const uint32_t unit = __builtin_amdgcn_readfirstlane(lds_read_u32(&sId[k % kIdRing]));
      if (unit >= NU) break;  // (ids only grow: every later unit is past the end as well)
      pending = fetch_id();
      const PipeGeo g = pipe_geo(p, ws, unit, 0, kUnit);
      const bool live = c < min(16, p.m - g.ct * 16);
      const uint32_t base = g.bt * ws.chunks;
      const int kb = k % kBufs;
      const uint32_t slot = base + g.chunk;
      // The unit's map (the compute waves leave the composition of all their
      // maps in the last slot) goes out as an aggregate while the look-back
      // waits for earlier units, so that later units' look-backs need not wait
      // for this one's leaving state: its stores are issued between two polls
      // once the map is in, and the flag is raised after the next poll, whose
      // wait for its own loads has seen the stores complete as well. No compute
      // wave waits for a store to complete.
      int agg = g.chunk > 0 ? 0 : 2;  // 0: map not yet out, 1: stores issued, 2: flag raised (or not needed)
      auto publish_aggregate = [&]() {
        if (agg == 1) {
          raise_flag(ws.flags + slot, kFlagAggregate, epoch, lane);
          agg = 2;
        } else if (agg == 0 && __builtin_amdgcn_readfirstlane(lds_read_u32(&sSumDone[NC - 1])) >= uint32_t(k) + 1) {
          const f32x4 GA = *reinterpret_cast<const f32x4*>(&sP[kb][NC - 1][c * 16 + 4 * r]);
          const f32x4 GL = LSlot<M1>::load(&sL[kb][NC - 1][0], lane, r, c);
          pub_store4(ws.P + size_t(slot) * 256, 4 * c + r, GA);
          if (live) pub_store4(ws.L + size_t(slot) * 256, lane, GL);
          agg = 1;
        }
      };
      // the state entering the unit, from the units before it, found while the
      // compute waves summarise this one
      f32x4 h_in = zero4();
      if (g.chunk > 0) h_in = look_back(ws, base, int(g.chunk), live, lane, r, c, epoch, publish_aggregate);
      // hand the entering state over once the carries of unit k-4 (same slot) have read theirs
      lds_wait_at_least(&sCarryDone[kb], uint32_t(NC) * uint32_t(k / kBufs));  // unit k-kBufs's carries are done
      LSlot<M1>::store(&sX[kb][0], h_in, lane, r, c);
      lds_signal_set(&sHinIt[kb], uint32_t(k) + 1, lane);
      // the leaving state: the unit's map (the compute waves leave the composition of all
      // its waves' maps in the last slot) applied to the entering state
      lds_wait_at_least(&sSumDone[NC - 1], uint32_t(k) + 1);
      const f32x4 GA = *reinterpret_cast<const f32x4*>(&sP[kb][NC - 1][c * 16 + 4 * r]);
      const f32x4 GL = LSlot<M1>::load(&sL[kb][NC - 1][0], lane, r, c);
      const f32x4 h_out = g.chunk == 0 ? GL : mfma_16x16x16(GA, h_in, GL);
      if (live) pub_store4(ws.H + size_t(slot) * 256, lane, h_out);
      raise_flag(ws.flags + slot, kFlagInclusive, epoch, lane);  // (waits for the stores)
    }
  } else {
  // -------------------------------------------------------------- compute waves
  const char* st = &sStage[wave][0];
  UnitRegs<TIn, M1> RA, RB;
  PipeGeo gA, gB;

  // Unit k: stage -> Rc, summarise unit k. Returns false (doing nothing) when there is no unit k.
  auto step = [&](UnitRegs<TIn, M1>& Rc, PipeGeo& gc, int k) -> bool {
    const uint32_t unit = unit_id(k);
    if (unit >= NU) return false;
    gc = pipe_geo(p, ws, unit, wave, kUnit);
    if constexpr (SCALED) {  // the factors of the wave's 16 steps, loaded while the stage lands
      const int64_t q = gc.q0 + c < T ? gc.q0 + c : T - 1;
      Rc.sc = p.step_scale[int64_t(gc.batch) * T + (p.reverse ? T - 1 - q : q)];
    }
    lds_wait_at_least(&sLanded[wave], uint32_t(k) + 1);
    stage_to_regs<TIn, M1, ADJ>(Rc, st, gc.q0, T, lane, r, c);
    lds_signal_set(&sConsumed[wave], uint32_t(k) + 1, lane);  // (waits for the stage reads first)
    const int kb = k % kBufs;
    lds_wait_at_least(&sCarryDone[kb], uint32_t(NC) * uint32_t(k / kBufs));  // unit k-kBufs's carries are done
    float* sPw = &sP[kb][wave][0];
    float* sLw = &sL[kb][wave][0];
    summarize<TIn, M1, SCALED, kKeep>(Rc, sPw, sLw, &sV[wave][0], lane, r, c, [](int) {});
    if (wave > 0) {
      // this wave's map after the composition of the maps of waves 0 .. wave-1 (left in
      // slot wave-1 by the wave before), written back over this wave's own slot
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const f32x4 PA = *reinterpret_cast<const f32x4*>(sPw + c * 16 + 4 * r);  // own map, A-operand order
      const f32x4 Lw = LSlot<M1>::load(sLw, lane, r, c);
      lds_wait_at_least(&sSumDone[wave - 1], uint32_t(k) + 1);
      const float* sPp = &sP[kb][wave - 1][0];
      f32x4 Gp;
#pragma unroll
      for (int v = 0; v < 4; ++v) Gp[v] = sPp[(4 * r + v) * 16 + c];  // result-register order
      const f32x4 GLp = LSlot<M1>::load(&sL[kb][wave - 1][0], lane, r, c);
      const f32x4 G = mfma_16x16x16(PA, Gp, zero4());
      const f32x4 GL = mfma_16x16x16(PA, GLp, Lw);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int v = 0; v < 4; ++v) sPw[(4 * r + v) * 16 + c] = G[v];
      LSlot<M1>::store(sLw, GL, lane, r, c);
    }
    lds_signal_set(&sSumDone[wave], uint32_t(k) + 1, lane);
    return true;
  };
  // Replay unit k (registers R, geometry g) once the leader has handed over its entering state.
  auto finish = [&](const UnitRegs<TIn, M1>& R, const PipeGeo& g, int k) {
    const int kb = k % kBufs;
    lds_wait_at_least(&sHinIt[kb], uint32_t(k) + 1);
    f32x4 h = LSlot<M1>::load(&sX[kb][0], lane, r, c);
    if (wave > 0)  // slot wave-1 holds the composition of the maps of waves 0 .. wave-1
      h = mfma_16x16x16(*reinterpret_cast<const f32x4*>(&sP[kb][wave - 1][c * 16 + 4 * r]), h,
                        LSlot<M1>::load(&sL[kb][wave - 1][0], lane, r, c));
    lds_signal_add(&sCarryDone[kb], lane);
    if constexpr (kKeep) replay_prefix_m1<TOut>(R, h, p, g, &sV[wave][0], r, c);
    else replay_steps<TIn, TOut, M1, SCALED, FOLD>(R, h, p, g, &sV[wave][0], lane, r, c, FOLD ? &sH[k % 3][wave][0] : nullptr);
  };

  for (int k = 0;; k += 2) {
    if (!step(RA, gA, k)) {
      if (k > 0) finish(RB, gB, k - 1);
      break;
    }
    if (k > 0) finish(RB, gB, k - 1);
    if (!step(RB, gB, k + 1)) {
      finish(RA, gA, k);
      break;
    }
    finish(RA, gA, k);
  }
  }  // compute waves

  __syncthreads();
  if (tid == 0) finish_call(ws, epoch);
}

// ------------------------------------------------------------------ :projective
//
// "Tensor operations", the "matrix-scan" section: the running product P of the
// a's, from the identity, is divided after every step by its largest
// magnitude m, and h by the same number: h = (a[t] h + b[t]) / m (m = 1 when P
// is zero). One wave per (batch, 16-column tile), serial in time: P and h
// advance by MFMA each step (P in result-register order, as h), m is the
// maximum over the wave (lane, DPP row, then the four row leaders), and the
// operands of the next K steps are in flight meanwhile.

// Largest |entry| of a 16x16 tile held four values per lane, the same in every lane.
__device__ __forceinline__ float wave_max_abs(f32x4 v) {
  float x = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
  x = fmaxf(x, dpp_mov<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_mov<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_mov<0x141>(x));  // row_half_mirror
  x = fmaxf(x, dpp_mov<0x140>(x));  // row_mirror: every lane holds its row's maximum
  const int xi = __float_as_int(x);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(xi, 0)), r1 = __int_as_float(__builtin_amdgcn_readlane(xi, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(xi, 32)), r3 = __int_as_float(__builtin_amdgcn_readlane(xi, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

template <typename TIn, typename TOut, bool VEC>
__global__ __launch_bounds__(64) void ms_projective_kernel(const MsParams p) {
  const int lane = int(threadIdx.x);
  const int r = lane >> 4, c = lane & 15;
  const int col_tiles = (p.m + 15) / 16;
  const int64_t batch = int64_t(blockIdx.x) / col_tiles;
  const int ct = int(int64_t(blockIdx.x) % col_tiles);
  const int n = p.n, m = p.m, cc = ct * 16 + c;
  int64_t off[3];
  index_offsets(p.batch, batch, off);
  const int64_t T = p.T;
  const int64_t t0 = p.reverse ? T - 1 : 0;  // time of scan position 0
  const int64_t ta = p.reverse ? -p.t_stride[MS_A] : p.t_stride[MS_A];
  const int64_t tb = p.reverse ? -p.t_stride[MS_B] : p.t_stride[MS_B];
  const int64_t to = p.reverse ? -p.t_stride[MS_OUT] : p.t_stride[MS_OUT];
  const TIn* a0 = static_cast<const TIn*>(p.a) + off[MS_A] + t0 * p.t_stride[MS_A];
  const TIn* b0 = static_cast<const TIn*>(p.b) + off[MS_B] + t0 * p.t_stride[MS_B];
  TOut* o0 = static_cast<TOut*>(p.out) + off[MS_OUT] + t0 * p.t_stride[MS_OUT];
  constexpr int K = 4;  // steps whose operands are in flight
  ARow<TIn> A[K];
  BCol<TIn> B[K];
  auto load = [&](int64_t q, int u) {  // clamped position: every load is valid, none behind a branch
    const int64_t qc = q < T ? q : T - 1;
    A[u] = load_a<TIn, VEC>(a0 + qc * ta, n, r, c);
    B[u] = load_b(b0 + qc * tb, n, m, r, cc);
  };
#pragma unroll
  for (int u = 0; u < K; ++u) load(u, u);
  f32x4 P = identity_d(r, c), h = zero4();
  for (int64_t q0 = 0; q0 < T; q0 += K) {
#pragma unroll
    for (int u = 0; u < K; ++u) {
      const int64_t q = q0 + u;
      if (q < T) {  // wave-uniform
        const f32x4 av = A[u].get();
        P = mfma_16x16x16(av, P, zero4());
        h = mfma_16x16x16(av, h, B[u].get());
        const float big = wave_max_abs(P);
        const float inv = big > 0.0f ? 1.0f / big : 1.0f;
        P *= inv;
        h *= inv;
        store_h(o0 + q * to, h, n, m, r, cc);
      }
      load(q0 + u + K, u);
    }
  }
}

// :projective in parallel. In exact arithmetic the factor of step t is 1/m_t
// with m_t = max|a[t] P'|, P' the product of every a before t (in scan order)
// divided by its largest entry; with the factors known, h is an ordinary
// matrix-scan of a[t] s[t] and b[t] s[t]. Three passes give the factors; the
// first and last run one wave per (batch, chunk of kProjChunk steps):
//   ms_proj_chunk_kernel  the chunk's product (later steps on the left),
//                         divided by its largest entry after every step so
//                         that it stays in range; stored row-major.
//   ms_proj_prefix_kernel one wave per batch: the chunk products composed in
//                         scan order (again divided after every product),
//                         storing the product each chunk starts from.
//   ms_proj_scale_kernel  this chunk's steps from its starting product, each
//                         storing the factor of its step (1 where the product
//                         is zero).
// The pipelined kernel with SCALED then runs the scan.
constexpr int kProjChunk = 128;
constexpr int kProjAhead = 16;  // steps of a in flight in both factor passes
static_assert(kProjChunk % kProjAhead == 0, "the factor passes unroll whole rounds of loads");

template <typename TIn, bool VEC>
__global__ __launch_bounds__(64) void ms_proj_chunk_kernel(const MsParams p, float* prod, int64_t chunks) {
  const int lane = int(threadIdx.x), r = lane >> 4, c = lane & 15;
  const int64_t batch = int64_t(blockIdx.x) / chunks, ch = int64_t(blockIdx.x) % chunks;
  int64_t off[3];
  index_offsets(p.batch, batch, off);
  const int64_t T = p.T;
  const int64_t ta = p.reverse ? -p.t_stride[MS_A] : p.t_stride[MS_A];
  const TIn* a0 = static_cast<const TIn*>(p.a) + off[MS_A] + (p.reverse ? T - 1 : 0) * p.t_stride[MS_A];
  const int64_t q_begin = ch * kProjChunk, q_end = q_begin + kProjChunk < T ? q_begin + kProjChunk : T;
  constexpr int K = kProjAhead;  // steps whose operands are in flight
  ARow<TIn> A[K];
  auto load = [&](int64_t q, int u) { A[u] = load_a<TIn, VEC>(a0 + (q < q_end ? q : q_end - 1) * ta, p.n, r, c); };
#pragma unroll
  for (int u = 0; u < K; ++u) load(q_begin + u, u);
  f32x4 P = identity_d(r, c);
  // unrolled over the whole chunk: each step waits for its own operand only (a
  // loop here would drain every load in flight at its head). Steps past the end
  // are computed and dropped by a select, so no load moves behind a branch.
#pragma unroll
  for (int k = 0; k < kProjChunk; ++k) {
    f32x4 Pn = mfma_a<TIn>(A[k % K], P, zero4());
    const float big = wave_max_abs(Pn);
    Pn *= big > 0.0f ? 1.0f / big : 1.0f;
    const bool on = q_begin + k < q_end;  // wave-uniform
#pragma unroll
    for (int v = 0; v < 4; ++v) P[v] = on ? Pn[v] : P[v];
    if (k + K < kProjChunk) load(q_begin + k + K, k % K);
    __builtin_amdgcn_sched_barrier(0);  // the load stays K steps ahead of its use
  }
  float* dst = prod + (batch * chunks + ch) * 256;
#pragma unroll
  for (int v = 0; v < 4; ++v) dst[(4 * r + v) * 16 + c] = P[v];
}

// Chunk products are stored row-major; lane (r, c) reads row c, columns 4r..4r+3
// (the A operand) and keeps rows 4r..4r+3 of column c of a result.
__global__ __launch_bounds__(64) void ms_proj_prefix_kernel(const float* prod, float* entry, int64_t chunks) {
  const int lane = int(threadIdx.x), r = lane >> 4, c = lane & 15;
  const int64_t batch = blockIdx.x;
  const float* pb = prod + batch * chunks * 256 + c * 16 + 4 * r;
  float* eb = entry + batch * chunks * 256;
  f32x4 P = identity_d(r, c);
  constexpr int KP = 16;  // products in flight (positions past the end read chunk 0's, unused)
  f32x4 R[KP];
  auto load_prod = [&](int64_t j, int u) { R[u] = *reinterpret_cast<const f32x4*>(pb + (j < chunks ? j : 0) * 256); };
#pragma unroll
  for (int u = 0; u < KP; ++u) load_prod(u, u);
  for (int64_t j0 = 0; j0 < chunks; j0 += KP) {
#pragma unroll
    for (int u = 0; u < KP; ++u) {
      const int64_t j = j0 + u;
      if (j < chunks) {  // wave-uniform
#pragma unroll
        for (int v = 0; v < 4; ++v) eb[j * 256 + (4 * r + v) * 16 + c] = P[v];
        P = mfma_16x16x16(R[u], P, zero4());
        const float big = wave_max_abs(P);
        P *= big > 0.0f ? 1.0f / big : 1.0f;
      }
      load_prod(j0 + u + KP, u);
    }
  }
}

template <typename TIn, bool VEC>
__global__ __launch_bounds__(64) void ms_proj_scale_kernel(const MsParams p, const float* entry, float* step_scale,
                                                           int64_t chunks) {
  const int lane = int(threadIdx.x), r = lane >> 4, c = lane & 15;
  const int64_t batch = int64_t(blockIdx.x) / chunks, ch = int64_t(blockIdx.x) % chunks;
  int64_t off[3];
  index_offsets(p.batch, batch, off);
  const int64_t T = p.T;
  // the product this chunk starts from
  const float* eb = entry + (batch * chunks + ch) * 256;
  f32x4 P;
#pragma unroll
  for (int v = 0; v < 4; ++v) P[v] = eb[(4 * r + v) * 16 + c];
  const int64_t ta = p.reverse ? -p.t_stride[MS_A] : p.t_stride[MS_A];
  const TIn* a0 = static_cast<const TIn*>(p.a) + off[MS_A] + (p.reverse ? T - 1 : 0) * p.t_stride[MS_A];
  const int64_t q_begin = ch * kProjChunk, q_end = q_begin + kProjChunk < T ? q_begin + kProjChunk : T;
  float* sc = step_scale + batch * T;
  constexpr int K = kProjAhead;
  ARow<TIn> A[K];
  auto load = [&](int64_t q, int u) { A[u] = load_a<TIn, VEC>(a0 + (q < q_end ? q : q_end - 1) * ta, p.n, r, c); };
#pragma unroll
  for (int u = 0; u < K; ++u) load(q_begin + u, u);
#pragma unroll
  for (int k = 0; k < kProjChunk; ++k) {  // unrolled, as in ms_proj_chunk_kernel
    const int64_t q = q_begin + k;
    if (q < q_end) {  // wave-uniform
      P = mfma_a<TIn>(A[k % K], P, zero4());
      const float big = wave_max_abs(P);
      const float inv = big > 0.0f ? 1.0f / big : 1.0f;
      P *= inv;
      if (lane == 0) sc[p.reverse ? T - 1 - q : q] = inv;
    }
    if (k + K < kProjChunk) load(q + K, k % K);
    __builtin_amdgcn_sched_barrier(0);
  }
}

std::atomic<uint32_t> g_spin_limit{0};
constexpr uint32_t kDefaultSpinLimit = 1u << 22;  // about a tenth of a second of polling

uint32_t lookback_spin_limit() {
  const uint32_t v = g_spin_limit.load(std::memory_order_relaxed);
  return v == 0 ? kDefaultSpinLimit : v;
}

constexpr int kWaves = 8;          // ms_unit_kernel: waves per workgroup
constexpr int kSteps = 16;         // steps per wave (both kernels)
constexpr int kLeadCompute = 6;    // ms_lead_kernel: compute waves per workgroup (plus leader and loader)

struct UnitPlan {
  int col_tiles;
  uint64_t chunks, num_units;
  size_t flags_bytes, block_bytes, total;
};

UnitPlan unit_plan(const MsParams& p, int unit_steps) {
  UnitPlan u{};
  u.chunks = uint64_t((p.T + unit_steps - 1) / unit_steps);
  u.col_tiles = (p.m + 15) / 16;
  u.num_units = u.chunks * uint64_t(p.num_batch) * uint64_t(u.col_tiles);
  u.flags_bytes = (u.num_units * sizeof(uint64_t) + 255) / 256 * 256;
  u.block_bytes = size_t(u.num_units) * 256 * sizeof(float);
  u.total = 256 + u.flags_bytes + 3 * u.block_bytes;
  return u;
}

// The look-back state of a unit plan in a workspace (see MsUnitWs).
MsUnitWs unit_ws(const UnitPlan& up, void* workspace) {
  char* base = static_cast<char*>(workspace);
  MsUnitWs ws;
  ws.header = reinterpret_cast<uint32_t*>(base);
  ws.flags = reinterpret_cast<uint64_t*>(base + 256);
  ws.P = reinterpret_cast<float*>(base + 256 + up.flags_bytes);
  ws.L = ws.P + up.num_units * 256;
  ws.H = ws.L + up.num_units * 256;
  ws.num_units = uint32_t(up.num_units);
  ws.chunks = uint32_t(up.chunks);
  ws.col_tiles = up.col_tiles;
  ws.spin_limit = lookback_spin_limit();
  return ws;
}

template <typename TIn, typename TOut, bool ADJ>
hipError_t launch_serial(const MsParams& p, hipStream_t stream) {
  const int64_t blocks = p.num_batch * ((p.m + 15) / 16);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((ms_serial_kernel<TIn, TOut, ADJ>), dim3(unsigned(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename TIn, typename TOut, bool M1, bool ADJ>
void launch_unit_variant(const MsParams& p, const MsUnitWs& ws, bool vec, unsigned blocks, hipStream_t stream) {
  if (ADJ)  // the transposed loads are element loads: no vector variant
    hipLaunchKernelGGL((ms_unit_kernel<kWaves, kSteps, TIn, TOut, false, M1, ADJ>), dim3(blocks), dim3(kWaves * 64),
                       0, stream, p, ws);
  else if (vec)
    hipLaunchKernelGGL((ms_unit_kernel<kWaves, kSteps, TIn, TOut, true, M1>), dim3(blocks), dim3(kWaves * 64), 0,
                       stream, p, ws);
  else
    hipLaunchKernelGGL((ms_unit_kernel<kWaves, kSteps, TIn, TOut, false, M1>), dim3(blocks), dim3(kWaves * 64), 0,
                       stream, p, ws);
}

// The pipelined kernel covers n = 16 with m = 1 (f32 or bf16 inputs) or m a
// multiple of 16 (bf16 inputs: an f32 b tile would not fit the LDS stage), and
// needs 16-byte aligned steps of a and b (global_load_lds moves 16-byte pieces)
// and aligned output pieces. Everything else takes ms_unit_kernel.
bool pipe_fits(const MsParams& p) {
  if (p.n != 16) return false;
  const bool m1 = p.m == 1;
  if (!m1 && !(p.in_bf16 && p.m % 16 == 0)) return false;
  auto aligned = [&](int t, const void* base, int64_t elem, int64_t to) {
    if (reinterpret_cast<uintptr_t>(base) % uintptr_t(to) != 0 || (p.t_stride[t] * elem) % to != 0) return false;
    for (int d = 0; d < p.batch.nd; ++d)
      if ((p.batch.st[t][d] * elem) % to != 0) return false;
    return true;
  };
  const int64_t si = p.in_bf16 ? 2 : 4, so = p.out_bf16 ? 2 : 4;
  return aligned(MS_A, p.a, si, 16) && aligned(MS_B, p.b, si, 16) && aligned(MS_OUT, p.out, so, m1 ? 4 * so : 16);
}

template <typename TIn, typename TOut, bool ADJ>
void launch_lead_tiles(const MsParams& p, const MsUnitWs& ws, unsigned blocks, hipStream_t stream) {
  if constexpr (sizeof(TIn) == 2)
    hipLaunchKernelGGL((ms_lead_kernel<kLeadCompute, TIn, TOut, false, ADJ>), dim3(blocks), dim3(512), 0, stream, p,
                       ws);
}

template <typename TIn, typename TOut, bool ADJ>
hipError_t launch_chunked(const MsParams& p, void* workspace, hipStream_t stream) {
  const bool pipe = pipe_fits(p);
  const UnitPlan up = unit_plan(p, pipe ? kLeadCompute * kSteps : kWaves * kSteps);
  const MsUnitWs ws = unit_ws(up, workspace);
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
  if (pipe) {
    const unsigned blocks = unsigned(std::min<uint64_t>(up.num_units, uint64_t(device_cu_count())));
    if constexpr (ADJ && sizeof(TIn) == 4 && sizeof(TOut) == 4) {
      if (m1 && p.fold_grad_a != nullptr) {  // the caller checked matrix_scan_folds_grad_a
        hipLaunchKernelGGL((ms_lead_kernel<kLeadCompute, TIn, TOut, true, true, false, true>), dim3(blocks), dim3(512),
                           0, stream, p, ws);
        return hipGetLastError();
      }
    }
    if (m1)
      hipLaunchKernelGGL((ms_lead_kernel<kLeadCompute, TIn, TOut, true, ADJ>), dim3(blocks), dim3(512), 0, stream, p,
                         ws);
    else launch_lead_tiles<TIn, TOut, ADJ>(p, ws, blocks, stream);
    return hipGetLastError();
  }
  const unsigned blocks = unsigned(up.num_units);
  if (m1) launch_unit_variant<TIn, TOut, true, ADJ>(p, ws, vec, blocks, stream);
  else launch_unit_variant<TIn, TOut, false, ADJ>(p, ws, vec, blocks, stream);
  return hipGetLastError();
}

// Room :projective's factor passes take after the scan's own workspace: the
// chunk products, the product each chunk starts from and the factor of every step.
struct ProjPlan {
  int64_t chunks;
  size_t prod_off, entry_off, scale_off, total;
};

ProjPlan proj_plan(const MsParams& p, size_t scan_bytes) {
  ProjPlan q{};
  q.chunks = (p.T + kProjChunk - 1) / kProjChunk;
  const size_t prods = size_t(p.num_batch) * size_t(q.chunks) * 256 * sizeof(float);
  q.prod_off = (scan_bytes + 255) / 256 * 256;
  q.entry_off = q.prod_off + prods;
  q.scale_off = q.entry_off + prods;
  q.total = q.scale_off + (size_t(p.num_batch) * size_t(p.T) * sizeof(float) + 255) / 256 * 256;
  return q;
}

size_t scan_workspace(const MsParams& p) {
  // Shapes only (the size is queried without dtypes or pointers): room for the
  // pipelined kernel's shorter units whenever its shapes apply, which also
  // covers ms_unit_kernel's longer ones.
  const bool pipe_shape = p.n == 16 && (p.m == 1 || p.m % 16 == 0);
  const UnitPlan up = unit_plan(p, pipe_shape ? kLeadCompute * kSteps : kWaves * kSteps);
  if (up.num_units > 0x7fffffffull) return 0;  // beyond 32-bit unit ids: the serial kernel takes it
  return up.total;
}

}  // namespace

size_t matrix_scan_workspace(const MsParams& p) {
  if (p.num_batch <= 0 || p.T <= 0 || p.n == 0 || p.m == 0) return 0;
  const size_t scan = scan_workspace(p);
  if (scan == 0) return 0;
  // with room for :projective's passes where the pipelined kernel runs them (n = 16)
  return p.n == 16 ? proj_plan(p, scan).total : scan;
}

namespace {

template <typename TIn, typename TOut>
hipError_t launch_projective_passes(const MsParams& p0, void* workspace, hipStream_t stream) {
  const size_t scan = scan_workspace(p0);
  const ProjPlan pp = proj_plan(p0, scan);
  char* base = static_cast<char*>(workspace);
  float* prod = reinterpret_cast<float*>(base + pp.prod_off);
  float* entry = reinterpret_cast<float*>(base + pp.entry_off);
  float* scale = reinterpret_cast<float*>(base + pp.scale_off);
  MsParams p = p0;
  p.step_scale = scale;
  const int64_t waves = p.num_batch * pp.chunks;
  if (waves > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int64_t va = 4 * int64_t(sizeof(TIn));
  bool vec = reinterpret_cast<uintptr_t>(p.a) % uintptr_t(va) == 0 && (p.t_stride[MS_A] * int64_t(sizeof(TIn))) % va == 0;
  for (int d = 0; d < p.batch.nd && vec; ++d) vec = (p.batch.st[MS_A][d] * int64_t(sizeof(TIn))) % va == 0;
  const dim3 grid{unsigned(waves)}, block{64};
  if (vec) {
    hipLaunchKernelGGL((ms_proj_chunk_kernel<TIn, true>), grid, block, 0, stream, p, prod, pp.chunks);
    hipLaunchKernelGGL(ms_proj_prefix_kernel, dim3(unsigned(p.num_batch)), block, 0, stream, prod, entry, pp.chunks);
    hipLaunchKernelGGL((ms_proj_scale_kernel<TIn, true>), grid, block, 0, stream, p, entry, scale, pp.chunks);
  } else {
    hipLaunchKernelGGL((ms_proj_chunk_kernel<TIn, false>), grid, block, 0, stream, p, prod, pp.chunks);
    hipLaunchKernelGGL(ms_proj_prefix_kernel, dim3(unsigned(p.num_batch)), block, 0, stream, prod, entry, pp.chunks);
    hipLaunchKernelGGL((ms_proj_scale_kernel<TIn, false>), grid, block, 0, stream, p, entry, scale, pp.chunks);
  }
  // the scan of a[t] s[t], b[t] s[t]: the pipelined kernel with its factors
  const UnitPlan up = unit_plan(p, kLeadCompute * kSteps);
  const MsUnitWs ws = unit_ws(up, workspace);
  const unsigned blocks = unsigned(std::min<uint64_t>(up.num_units, uint64_t(device_cu_count())));
  if (p.m == 1)
    hipLaunchKernelGGL((ms_lead_kernel<kLeadCompute, TIn, TOut, true, false, true>), dim3(blocks), dim3(512), 0, stream,
                       p, ws);
  else if constexpr (sizeof(TIn) == 2)
    hipLaunchKernelGGL((ms_lead_kernel<kLeadCompute, TIn, TOut, false, false, true>), dim3(blocks), dim3(512), 0,
                       stream, p, ws);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_matrix_scan_projective(const MsParams& p, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  if (p.num_batch <= 0 || p.T <= 0 || p.n == 0 || p.m == 0) return hipSuccess;
  // In parallel where the pipelined kernel takes the shape and the workspace has room for it all.
  const size_t scan = scan_workspace(p);
  if (pipe_fits(p) && scan > 0 && workspace != nullptr && workspace_bytes >= proj_plan(p, scan).total) {
    if (p.in_bf16)
      return p.out_bf16 ? launch_projective_passes<uint16_t, uint16_t>(p, workspace, stream)
                        : launch_projective_passes<uint16_t, float>(p, workspace, stream);
    return p.out_bf16 ? launch_projective_passes<float, uint16_t>(p, workspace, stream)
                      : launch_projective_passes<float, float>(p, workspace, stream);
  }
  const int64_t blocks = p.num_batch * ((p.m + 15) / 16);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  // whole 16-byte (f32) or 8-byte (bf16) rows of a for n = 16 with aligned steps
  const int64_t va = 4 * int64_t(p.in_bf16 ? 2 : 4);
  bool vec = p.n == 16 && reinterpret_cast<uintptr_t>(p.a) % uintptr_t(va) == 0 &&
             (p.t_stride[MS_A] * (va / 4)) % va == 0;
  for (int d = 0; d < p.batch.nd && vec; ++d) vec = (p.batch.st[MS_A][d] * (va / 4)) % va == 0;
  const dim3 grid{unsigned(blocks)}, block{64};
  auto go = [&](auto tin, auto tout) {
    using TI = decltype(tin);
    using TO = decltype(tout);
    if (vec) hipLaunchKernelGGL((ms_projective_kernel<TI, TO, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((ms_projective_kernel<TI, TO, false>), grid, block, 0, stream, p);
  };
  if (p.in_bf16) {
    if (p.out_bf16) go(uint16_t{}, uint16_t{});
    else go(uint16_t{}, float{});
  } else {
    if (p.out_bf16) go(float{}, uint16_t{});
    else go(float{}, float{});
  }
  return hipGetLastError();
}

void set_lookback_spin_limit(uint32_t limit) { g_spin_limit.store(limit, std::memory_order_relaxed); }

// The look-back state of sx_matrix_scan_noalloc: a fixed array in device memory,
// one per device the library runs on, held until the process ends. Host code
// reaches it only through the address hipGetSymbolAddress gives on each device
// (the array's name in host code is a stand-in, not a device address).
__device__ __align__(256) unsigned char scratch[kMatrixScanScratchBytes];

hipError_t matrix_scan_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> ptrs[kMaxDevices];
  static std::mutex init_mutex;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* ptr = ptrs[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    std::lock_guard<std::mutex> lock(init_mutex);
    ptr = ptrs[dev].load(std::memory_order_relaxed);
    if (ptr == nullptr) {
      // once per device, with the device current: its address, zero-filled once as every
      // matrix-scan workspace must be; synchronous, so no stream can run ahead of it
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      e = hipMemset(ptr, 0, kMatrixScanScratchBytes);
      if (e == hipSuccess) e = hipDeviceSynchronize();
      if (e != hipSuccess) return e;
      // every call above succeeded; what they may have left in the runtime's
      // last-error slot is not this call's error (launch checks read that slot)
      (void)hipGetLastError();
      ptrs[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return hipSuccess;
}

bool matrix_scan_folds_grad_a(const MsParams& p, const void* workspace, size_t workspace_bytes) {
  if (!p.adjoint || p.in_bf16 || p.out_bf16 || p.n != 16 || p.m != 1 || p.fold_h == nullptr || p.fold_grad_a == nullptr)
    return false;
  if (p.num_batch <= 0 || p.T <= 0) return false;
  const size_t need = matrix_scan_workspace(p);
  if (need == 0 || workspace == nullptr || workspace_bytes < need) return false;  // not the chunked scan
  // h is copied in 16-byte pieces and grad_a stored in 16-byte pieces, at out's offsets (x 16 for grad_a)
  const bool al = reinterpret_cast<uintptr_t>(p.fold_h) % 16 == 0 && reinterpret_cast<uintptr_t>(p.fold_grad_a) % 16 == 0 &&
                  (p.t_stride[MS_OUT] * 4) % 16 == 0;
  return al && pipe_fits(p);
}

hipError_t launch_matrix_scan(const MsParams& p, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (p.num_batch <= 0 || p.T <= 0 || p.n == 0 || p.m == 0) return hipSuccess;
  const size_t need = matrix_scan_workspace(p);
  const bool chunked = need > 0 && workspace != nullptr && workspace_bytes >= need;
  if (p.adjoint) {  // computed in f32; stored in f32, or rounded to bf16 when that is the gradient's dtype
    if (chunked) {
      if (p.in_bf16)
        return p.out_bf16 ? launch_chunked<uint16_t, uint16_t, true>(p, workspace, stream)
                          : launch_chunked<uint16_t, float, true>(p, workspace, stream);
      return p.out_bf16 ? launch_chunked<float, uint16_t, true>(p, workspace, stream)
                        : launch_chunked<float, float, true>(p, workspace, stream);
    }
    if (p.in_bf16)
      return p.out_bf16 ? launch_serial<uint16_t, uint16_t, true>(p, stream) : launch_serial<uint16_t, float, true>(p, stream);
    return p.out_bf16 ? launch_serial<float, uint16_t, true>(p, stream) : launch_serial<float, float, true>(p, stream);
  }
  if (chunked) {
    if (p.in_bf16)
      return p.out_bf16 ? launch_chunked<uint16_t, uint16_t, false>(p, workspace, stream)
                        : launch_chunked<uint16_t, float, false>(p, workspace, stream);
    return p.out_bf16 ? launch_chunked<float, uint16_t, false>(p, workspace, stream)
                      : launch_chunked<float, float, false>(p, workspace, stream);
  }
  if (p.in_bf16)
    return p.out_bf16 ? launch_serial<uint16_t, uint16_t, false>(p, stream)
                      : launch_serial<uint16_t, float, false>(p, stream);
  return p.out_bf16 ? launch_serial<float, uint16_t, false>(p, stream) : launch_serial<float, float, false>(p, stream);
}

}  // namespace sx
