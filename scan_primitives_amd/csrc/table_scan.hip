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
//                    of 64 * K steps gives each lane K consecutive steps
//                    (slabs move between HBM and LDS coalesced). The
//                    map of a step (state -> next state) is kept one byte per
//                    state (8 or 16 bytes), one per symbol, in LDS, and maps
//                    compose by byte gathers (v_perm_b32).
//                    Each lane composes the maps of its K steps, a scan of the
//                    lanes' maps (six rounds of composition over DPP lane
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


typedef int i32x4 __attribute__((ext_vector_type(4)));

// A map of states (state -> next state) with one byte per state: MW 32-bit
// words hold 4 * MW entries (MW = 2: up to 8 states, MW = 4: up to 16).
// Entries past the table's states map to themselves and are never reached.
template <int MW>
struct StateMap {
  uint32_t w[MW];
};

template <int MW>
__device__ __forceinline__ StateMap<MW> identity_map() {
  StateMap<MW> m;
#pragma unroll
  for (int i = 0; i < MW; ++i) m.w[i] = 0x03020100u + 0x04040404u * uint32_t(i);
  return m;
}

// "inner, then outer": entry s is outer[inner[s]], a byte gather. v_perm_b32
// picks each result byte from the 8 bytes {src0 (high), src1 (low)} by the
// selector byte (0-7). Sixteen entries take two gathers (entries 0-7 and
// 8-15) and a byte select on bit 3 of the selector: that bit, moved to bit 2
// of each byte, selects byte 4 (0xFF) or byte 0 (0x00) of {~0, 0} in a third
// gather, which gives the byte mask with full-rate instructions only.
template <int MW>
__device__ __forceinline__ StateMap<MW> compose(const StateMap<MW>& outer, const StateMap<MW>& inner) {
  StateMap<MW> r;
  if constexpr (MW == 2) {
    r.w[0] = __builtin_amdgcn_perm(outer.w[1], outer.w[0], inner.w[0]);
    r.w[1] = __builtin_amdgcn_perm(outer.w[1], outer.w[0], inner.w[1]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t sel = inner.w[j];
      const uint32_t low3 = sel & 0x07070707u;
      const uint32_t lo = __builtin_amdgcn_perm(outer.w[1], outer.w[0], low3);
      const uint32_t hi = __builtin_amdgcn_perm(outer.w[3], outer.w[2], low3);
      const uint32_t high = __builtin_amdgcn_perm(0xFFFFFFFFu, 0u, (sel >> 1) & 0x04040404u);  // 0xFF where 8-15
      r.w[j] = (hi & high) | (lo & ~high);
    }
  }
  return r;
}

// m[s] by byte gathers: byte s of the map moved to byte 0 (a select chain over
// the words is turned by the compiler into an indexed stack access).
template <int MW>
__device__ __forceinline__ uint32_t apply(const StateMap<MW>& m, uint32_t s) {  // m[s]
  if constexpr (MW == 2) {
    return __builtin_amdgcn_perm(m.w[1], m.w[0], s) & 0xFFu;
  } else {
    const uint32_t lo = __builtin_amdgcn_perm(m.w[1], m.w[0], s & 7u);
    const uint32_t hi = __builtin_amdgcn_perm(m.w[3], m.w[2], s & 7u);
    return (s & 8u ? hi : lo) & 0xFFu;
  }
}

// DPP move of a map: lanes whose source lies outside what CTRL allows (or in a
// row left out by ROW_MASK) get the identity map, which composes as a no-op.
template <int CTRL, int ROW_MASK, int MW>
__device__ __forceinline__ StateMap<MW> dpp_map(const StateMap<MW>& m) {
  const StateMap<MW> id = identity_map<MW>();
  StateMap<MW> r;
#pragma unroll
  for (int i = 0; i < MW; ++i)
    r.w[i] = uint32_t(__builtin_amdgcn_update_dpp(int(id.w[i]), int(m.w[i]), CTRL, ROW_MASK, 0xF, false));
  return r;
}

// Inclusive scan of the lanes' maps in lane order (lane l ends with the maps of
// lanes 0..l composed, later ones outermost) with DPP moves only: shifts by 1,
// 2, 4 and 8 within each row of 16 lanes, then lane 15 of each even row into
// the odd row after it, then lane 31 into rows 2 and 3.
template <int MW>
__device__ __forceinline__ StateMap<MW> scan_maps(StateMap<MW> G) {
  G = compose<MW>(G, dpp_map<0x111, 0xF>(G));  // row_shr:1
  G = compose<MW>(G, dpp_map<0x112, 0xF>(G));  // row_shr:2
  G = compose<MW>(G, dpp_map<0x114, 0xF>(G));  // row_shr:4
  G = compose<MW>(G, dpp_map<0x118, 0xF>(G));  // row_shr:8
  G = compose<MW>(G, dpp_map<0x142, 0xA>(G));  // row_bcast:15 into rows 1 and 3
  G = compose<MW>(G, dpp_map<0x143, 0xC>(G));  // row_bcast:31 into rows 2 and 3
  return G;
}

template <int MW>
__device__ __forceinline__ StateMap<MW> readlane_map(const StateMap<MW>& m, int l) {
  StateMap<MW> r;
#pragma unroll
  for (int i = 0; i < MW; ++i) r.w[i] = uint32_t(__builtin_amdgcn_readlane(int(m.w[i]), l));
  return r;
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// A slab of 64 K positions staged in LDS: position w sits at word w + 4 (w / 64).
// Both access patterns are free of bank conflicts (K = 8 or 16): lane l
// writing (or reading) 16 bytes at w = 256 j + 4 l for the coalesced global
// side, and lane l reading (or writing) 16 bytes at w = K l + 4 j for its own
// run of K positions.
__device__ __forceinline__ int slab_word(int w) { return w + 4 * (w >> 6); }

__device__ __forceinline__ void wave_lds_sync() {  // the wave's LDS writes are visible to its later reads
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// VEC: symbols and states are contiguous along the axis and every sequence
// starts 16-byte aligned. Full slabs then move between HBM and LDS as 16-byte
// pieces, coalesced across the wave (lane l takes bytes 16 l + 1024 j), and
// each lane takes its K consecutive positions from LDS.
// K: positions per lane per slab (16 or 32: the scan over the lanes is paid once per 1024 or 2048 positions).
template <bool VEC, int MW, int K>
__global__ __launch_bounds__(256) void ts_wave_kernel(const TsParams p) {
  constexpr int64_t kSlab = 64 * K;
  constexpr int kSlabWords = int(kSlab + kSlab / 16);
  __shared__ StateMap<MW> sMap[kTsMaxSymbolsWave];
  __shared__ __attribute__((aligned(16))) int32_t sSlab[4][VEC ? kSlabWords : 4];
  const int S = p.states, X = p.nsym;
  for (int x = int(threadIdx.x); x < X; x += 256) {  // per-symbol maps from the clamped table
    StateMap<MW> m = identity_map<MW>();
#pragma unroll
    for (int i = 0; i < MW; ++i) {  // fully unrolled: no register array indexed at run time
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int st = 4 * i + b;
        if (st < S) {
          const uint32_t e = uint32_t(clampi(p.table[int64_t(st) * X + x], 0, S - 1));
          m.w[i] = (m.w[i] & ~(0xFFu << (8 * b))) | (e << (8 * b));
        }
      }
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
  uint32_t carry = uint32_t(p.start);
  // One slab: compose this lane's maps, scan them over the lanes, replay from the entering
  // state into res. Positions past `valid` (relative to q0) are identity steps.
  auto slab = [&](const int32_t (&cur)[K], int64_t valid_from_q, int32_t (&res)[K]) {
    StateMap<MW> F = identity_map<MW>();  // this lane's steps composed
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const StateMap<MW> mk = k < valid_from_q ? sMap[clampi(cur[k], 0, X - 1)] : identity_map<MW>();
      F = compose<MW>(mk, F);
    }
    const StateMap<MW> G = scan_maps<MW>(F);  // lane l: the maps of lanes 0..l composed
    const StateMap<MW> before = dpp_map<0x138, 0xF>(G);  // wave_shr:1 (lane 0: the identity)
    uint32_t st = apply<MW>(before, carry);
    carry = apply<MW>(readlane_map<MW>(G, 63), carry);
#pragma unroll
    for (int k = 0; k < K; ++k) {  // the step maps again from LDS (keeping them would spill for 16 states)
      if (k < valid_from_q) st = apply<MW>(sMap[clampi(cur[k], 0, X - 1)], st);
      res[k] = int32_t(st);
    }
  };
  int32_t cur[K], res[K];
  const int64_t nfull = VEC ? T / kSlab : 0;
  if (nfull > 0) {
    int32_t* buf = &sSlab[wave][0];
    i32x4 raw[K / 4], nraw[K / 4];
    auto load_slab = [&](int64_t q0, i32x4 (&r)[K / 4]) {  // coalesced: lane l, piece j at 256 j + 4 l
#pragma unroll
      for (int j = 0; j < K / 4; ++j) r[j] = ld_stream(reinterpret_cast<const i32x4*>(xs + q0 + 256 * j + 4 * lane));
    };
    load_slab(0, raw);
    for (int64_t i = 0; i < nfull; ++i) {
      const int64_t q0 = i * kSlab;
#pragma unroll
      for (int j = 0; j < K / 4; ++j) *reinterpret_cast<i32x4*>(buf + slab_word(256 * j + 4 * lane)) = raw[j];
      wave_lds_sync();
#pragma unroll
      for (int j = 0; j < K / 4; ++j) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(buf + slab_word(K * lane + 4 * j));
        cur[4 * j] = v[0];
        cur[4 * j + 1] = v[1];
        cur[4 * j + 2] = v[2];
        cur[4 * j + 3] = v[3];
      }
      load_slab((i + 1 < nfull ? i + 1 : i) * kSlab, nraw);  // the next full slab (or this one again), in flight
      slab(cur, K, res);
      wave_lds_sync();  // every lane has read its symbols before the buffer takes the states
#pragma unroll
      for (int j = 0; j < K / 4; ++j)
        *reinterpret_cast<i32x4*>(buf + slab_word(K * lane + 4 * j)) =
            i32x4{res[4 * j], res[4 * j + 1], res[4 * j + 2], res[4 * j + 3]};
      wave_lds_sync();
#pragma unroll
      for (int j = 0; j < K / 4; ++j)
        st_stream(reinterpret_cast<i32x4*>(os + q0 + 256 * j + 4 * lane),
                  *reinterpret_cast<const i32x4*>(buf + slab_word(256 * j + 4 * lane)));
      wave_lds_sync();  // the states have left the buffer before the next slab's symbols enter it
#pragma unroll
      for (int j = 0; j < K / 4; ++j) raw[j] = nraw[j];
    }
  }
  // the rest (or everything when not VEC): element by element from clamped positions
  for (int64_t q0 = nfull * kSlab; q0 < T; q0 += kSlab) {
    const int64_t q = q0 + int64_t(lane) * K;
#pragma unroll
    for (int k = 0; k < K; ++k) cur[k] = xs[(q + k < T ? q + k : T - 1) * sx];
    slab(cur, T - q, res);
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (q + k < T) os[(q + k) * so] = res[k];
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
    const dim3 grid{unsigned(blocks)}, block{256};
    if (p.states <= 8) {
      // 32 positions a lane: 101.9 against 106.8 us on [4096,16384] (8: 103.4); 16-state tables keep 16
      // (32 and 8 take 138 and 134 against 118 us there)
      if (vec) hipLaunchKernelGGL((ts_wave_kernel<true, 2, 32>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((ts_wave_kernel<false, 2, 16>), grid, block, 0, stream, p);
    } else {
      if (vec) hipLaunchKernelGGL((ts_wave_kernel<true, 4, 16>), grid, block, 0, stream, p);
      else hipLaunchKernelGGL((ts_wave_kernel<false, 4, 16>), grid, block, 0, stream, p);
    }
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
