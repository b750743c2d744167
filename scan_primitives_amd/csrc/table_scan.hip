// table_scan.hip: table-scan kernels for gfx950.
//
// "Tensor operations", the "table-scan" section: along one axis of `symbols`
// a deterministic automaton moves to table[previous, symbol] at every symbol,
// from state `start`, and every state is kept. Symbols outside [0, symbols)
// and reached table entries outside [0, states) are clamped into range, as
// the pages' GPU backend does.
//
// Kernels here:
//   ts_wave_kernel   tables of at most 16 states. One wave per sequence; a slab
//                    of 64 * K steps gives each lane K consecutive steps. The
//                    map of a step (state -> next state) is packed as sixteen
//                    4-bit entries in a 64-bit word, one per symbol, in LDS.
//                    Each lane composes the maps of its K steps, a scan of the
//                    lanes' maps (six rounds of composition over cross-lane
//                    moves) gives each lane its entering state from the slab's
//                    carry, and each lane replays its steps, storing every
//                    state. The next slab's symbols are loaded meanwhile.
//   ts_serial_kernel any table: one thread per sequence, serial, the table in
//                    LDS when it fits (the design the pages give for their
//                    GPU backend), loads of the next block of symbols ahead.
#include <algorithm>

#include "sx_common.hpp"

namespace sx {
namespace {

constexpr int kTsK = 16;              // steps per lane per slab in ts_wave_kernel
constexpr int64_t kTsSlab = 64 * kTsK;
constexpr uint64_t kIdentityMap = 0xFEDCBA9876543210ull;  // nibble s holds s

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t nib(uint64_t m, uint32_t s) { return uint32_t(m >> (4 * s)) & 15u; }

// The map "inner, then outer" over the first S states (the others stay fixed).
__device__ __forceinline__ uint64_t compose(uint64_t outer, uint64_t inner, int S) {
  uint64_t r = kIdentityMap;
  for (int s = 0; s < S; ++s) {
    const uint64_t img = nib(outer, nib(inner, uint32_t(s)));
    r = (r & ~(uint64_t(15) << (4 * s))) | (img << (4 * s));
  }
  return r;
}

__device__ __forceinline__ uint64_t shfl_up_u64(uint64_t v, int d) {
  const int lo = __shfl_up(int(uint32_t(v)), d, 64);
  const int hi = __shfl_up(int(uint32_t(v >> 32)), d, 64);
  return (uint64_t(uint32_t(hi)) << 32) | uint32_t(lo);
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), l));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v >> 32)), l));
  return (uint64_t(hi) << 32) | lo;
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// VEC: symbols and states are contiguous along the axis and every sequence
// starts 16-byte aligned, so a lane moves its K steps as K/4 16-byte pieces.
template <bool VEC>
__global__ __launch_bounds__(256) void ts_wave_kernel(const TsParams p) {
  __shared__ uint64_t sMap[kTsMaxSymbolsWave];
  const int S = p.states, X = p.nsym;
  for (int x = int(threadIdx.x); x < X; x += 256) {  // per-symbol maps from the clamped table
    uint64_t m = kIdentityMap;
    for (int s = 0; s < S; ++s) {
      const uint64_t e = uint64_t(clampi(p.table[int64_t(s) * X + x], 0, S - 1));
      m = (m & ~(uint64_t(15) << (4 * s))) | (e << (4 * s));
    }
    sMap[x] = m;
  }
  __syncthreads();
  const int wave = int(threadIdx.x) >> 6, lane = int(threadIdx.x) & 63;
  const int64_t seq = int64_t(blockIdx.x) * 4 + wave;
  if (seq >= p.num_seq) return;  // the whole wave leaves together, after the barrier
  int64_t off[2];
  index_offsets(p.seqs, seq, off);
  const int32_t* xs = p.symbols + off[0];
  int32_t* os = p.out + off[1];
  const int64_t T = p.T, sx = p.t_stride[0], so = p.t_stride[1];
  constexpr int K = kTsK;
  // This lane's K symbols of the slab at q0. Full slabs (VEC): K/4 16-byte pieces, no
  // branch. Otherwise element by element from clamped positions (past the end: the last).
  auto load_vec = [&](int64_t q0, int32_t (&buf)[K]) {
    const i32x4* src = reinterpret_cast<const i32x4*>(xs + q0 + int64_t(lane) * K);
#pragma unroll
    for (int j = 0; j < K / 4; ++j) {
      const i32x4 v = ld_stream(src + j);
      buf[4 * j] = v[0];
      buf[4 * j + 1] = v[1];
      buf[4 * j + 2] = v[2];
      buf[4 * j + 3] = v[3];
    }
  };
  auto load_any = [&](int64_t q0, int32_t (&buf)[K]) {
    const int64_t q = q0 + int64_t(lane) * K;
#pragma unroll
    for (int k = 0; k < K; ++k) buf[k] = xs[(q + k < T ? q + k : T - 1) * sx];
  };
  uint32_t carry = uint32_t(p.start);
  // One slab: compose this lane's maps, scan them over the lanes, replay from the entering state.
  auto slab = [&](int64_t q0, const int32_t (&cur)[K], bool full) {
    const int64_t q = q0 + int64_t(lane) * K;
    uint64_t mk[K];
    uint64_t F = kIdentityMap;  // this lane's steps composed
#pragma unroll
    for (int k = 0; k < K; ++k) {
      mk[k] = (full || q + k < T) ? sMap[clampi(cur[k], 0, X - 1)] : kIdentityMap;  // past the end: identity
      F = compose(mk[k], F, S);
    }
    uint64_t G = F;  // inclusive scan over the lanes: lane l ends with the maps of lanes 0..l composed
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint64_t below = shfl_up_u64(G, d);
      if (lane >= d) G = compose(G, below, S);
    }
    const uint64_t before = shfl_up_u64(G, 1);
    uint32_t st = lane == 0 ? carry : nib(before, carry);
    carry = nib(readlane_u64(G, 63), carry);
    int32_t res[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
      st = nib(mk[k], st);
      res[k] = int32_t(st);
    }
    if (full) {
      i32x4* dst = reinterpret_cast<i32x4*>(os + q);
#pragma unroll
      for (int j = 0; j < K / 4; ++j) st_stream(dst + j, i32x4{res[4 * j], res[4 * j + 1], res[4 * j + 2], res[4 * j + 3]});
    } else {
#pragma unroll
      for (int k = 0; k < K; ++k)
        if (q + k < T) os[(q + k) * so] = res[k];
    }
  };
  int32_t cur[K], nxt[K];
  const int64_t nfull = VEC ? T / kTsSlab : 0;
  if (nfull > 0) {
    load_vec(0, cur);
    for (int64_t i = 0; i < nfull; ++i) {
      load_vec((i + 1 < nfull ? i + 1 : i) * kTsSlab, nxt);  // the next full slab (or this one again), in flight
      slab(i * kTsSlab, cur, true);
#pragma unroll
      for (int k = 0; k < K; ++k) cur[k] = nxt[k];
    }
  }
  int64_t q0 = nfull * kTsSlab;
  if (q0 < T) load_any(q0, cur);
  for (; q0 < T; q0 += kTsSlab) {
    load_any(q0 + kTsSlab, nxt);
    slab(q0, cur, false);
#pragma unroll
    for (int k = 0; k < K; ++k) cur[k] = nxt[k];
  }
}

template <bool IN_LDS>
__global__ __launch_bounds__(256) void ts_serial_kernel(const TsParams p) {
  __shared__ int32_t sTable[kTsMaxTableLds];
  const int S = p.states, X = p.nsym;
  if constexpr (IN_LDS) {
    for (int i = int(threadIdx.x); i < S * X; i += 256) sTable[i] = p.table[i];
    __syncthreads();
  }
  const int64_t seq = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (seq >= p.num_seq) return;
  int64_t off[2];
  index_offsets(p.seqs, seq, off);
  const int32_t* xs = p.symbols + off[0];
  int32_t* os = p.out + off[1];
  const int64_t T = p.T, sx = p.t_stride[0], so = p.t_stride[1];
  constexpr int U = 8;
  int32_t cur[U], nxt[U];
  auto load = [&](int64_t q0, int32_t (&buf)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) buf[u] = xs[(q0 + u < T ? q0 + u : T - 1) * sx];
  };
  int st = p.start;
  load(0, cur);
  for (int64_t q0 = 0; q0 < T; q0 += U) {
    load(q0 + U, nxt);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (q0 + u < T) {
        const int64_t i = int64_t(st) * X + clampi(cur[u], 0, X - 1);
        st = clampi(IN_LDS ? sTable[i] : p.table[i], 0, S - 1);
        os[(q0 + u) * so] = st;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = nxt[u];
  }
}

}  // namespace

hipError_t launch_table_scan(const TsParams& p, hipStream_t stream) {
  if (p.num_seq <= 0 || p.T <= 0) return hipSuccess;
  if (p.states <= 16 && p.nsym <= kTsMaxSymbolsWave) {
    const int64_t blocks = (p.num_seq + 3) / 4;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    // whole 16-byte pieces: contiguous along the axis, every sequence's start aligned
    bool vec = p.t_stride[0] == 1 && p.t_stride[1] == 1 && reinterpret_cast<uintptr_t>(p.symbols) % 16 == 0 &&
               reinterpret_cast<uintptr_t>(p.out) % 16 == 0;
    for (int d = 0; d < p.seqs.nd && vec; ++d) vec = p.seqs.st[0][d] % 4 == 0 && p.seqs.st[1][d] % 4 == 0;
    if (vec) hipLaunchKernelGGL(ts_wave_kernel<true>, dim3(unsigned(blocks)), dim3(256), 0, stream, p);
    else hipLaunchKernelGGL(ts_wave_kernel<false>, dim3(unsigned(blocks)), dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  const int64_t blocks = (p.num_seq + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (int64_t(p.states) * p.nsym <= kTsMaxTableLds)
    hipLaunchKernelGGL(ts_serial_kernel<true>, dim3(unsigned(blocks)), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(ts_serial_kernel<false>, dim3(unsigned(blocks)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sx
