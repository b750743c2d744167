// sx_common.hpp: descriptors and small device helpers shared by the host
// dispatch (sx_api.cpp) and the kernels (element_scan.hip, matrix_scan.hip).
// Internal to libsx_scan.so; the public interface is include/sx_scan.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sx_scan.h"

namespace sx {

constexpr int kMaxRank = SX_MAX_RANK;
constexpr int kWave = 64;

// Maps a flat lane (or batch) index to one element offset per tensor.
// Dimensions are row-major: the last one varies fastest, so consecutive
// lanes walk the innermost dimension and loads coalesce when it is
// contiguous. The host merges dimensions whose strides allow it, so the
// device loop below usually runs once or twice.
template <int NT>
struct IndexMap {
  int nd;
  int64_t dim[kMaxRank];
  int64_t st[NT][kMaxRank];
};

template <int NT>
__device__ __forceinline__ void index_offsets(const IndexMap<NT>& m, int64_t idx, int64_t (&off)[NT]) {
#pragma unroll
  for (int k = 0; k < NT; ++k) off[k] = 0;
  for (int d = m.nd - 1; d >= 0; --d) {
    const int64_t dd = m.dim[d];
    const int64_t i = dd == 1 ? 0 : idx % dd;
    idx = dd == 1 ? idx : idx / dd;
#pragma unroll
    for (int k = 0; k < NT; ++k) off[k] += i * m.st[k][d];
  }
}

// The same for an index below 2^31 of a map whose dims and strides all lie
// below 2^31 in magnitude (every tensor of the caller spans less than 2 GiB):
// 32-bit divisions, and the loop unrolled over the largest rank so that every
// dimension's descriptor is loaded before the first is used (a loop over the
// runtime rank waits for each load in turn, which measured slower even though
// the unrolled form holds more descriptors than fit in scalar registers).
template <int NT>
__device__ __forceinline__ void index_offsets32(const IndexMap<NT>& m, uint32_t idx, int64_t (&off)[NT]) {
  int32_t o[NT];
#pragma unroll
  for (int k = 0; k < NT; ++k) o[k] = 0;
#pragma unroll
  for (int d = kMaxRank - 1; d >= 0; --d) {
    if (d < m.nd) {
      const uint32_t dd = uint32_t(m.dim[d]);
      const uint32_t q = dd == 1 ? idx : idx / dd;
      const uint32_t i = idx - q * dd;
      idx = q;
#pragma unroll
      for (int k = 0; k < NT; ++k) o[k] += int32_t(i) * int32_t(m.st[k][d]);
    }
  }
#pragma unroll
  for (int k = 0; k < NT; ++k) off[k] = o[k];
}

// Compute units of the current device (the persistent kernels keep one or two
// workgroups resident on each); cached per device.
int device_cu_count();

// ---------------------------------------------------------------- element-scan

enum EsTensor { ES_X = 0, ES_S = 1, ES_INIT = 2, ES_OUT = 3 };

struct EsParams {
  IndexMap<4> lanes;     // lane -> offsets of x, s, initial, out
  int64_t num_lanes;     // lanes (for NORM_CAP: state vectors, each of n values)
  int64_t T;             // trips along the scan axis (>= 1)
  int64_t t_stride[4];   // stride along the scan axis (initial: 0)
  int64_t n_stride[4];   // stride along the state axis (NORM_CAP only; 0 for width-1 sequences)
  int n;                 // state width for NORM_CAP, 1 otherwise
  int reverse;
  const float* x;
  const float* s;
  const float* init;     // nullptr: every lane starts from zero (linear-scan)
  float* out;
};

hipError_t launch_element_scan(sx_body body, const EsParams& p, hipStream_t stream);
size_t element_scan_workspace(sx_body body, const EsParams& p);

// Gradient of an element scan: p as planned for the forward call (initial
// contiguous), h (the forward result) and g (its gradient) in out's layout;
// gx and gs full-width gradients of the two sequences in out's layout (or,
// norm-cap only, with gx_sum / gs_sum set, the width-one gradient: contiguous,
// out's shape with the state axis of width one); ginit in initial's layout.
struct EsVjpParams {
  EsParams p;
  const float* h;
  const float* g;
  float* gx;
  float* gs;
  float* ginit;
  int gx_sum, gs_sum;    // norm-cap: the sequence has width one, its gradient is summed over the state
  float* bounds;         // norm-cap with few lanes: 2 floats per lane of workspace (nullptr: serial rows)
};
hipError_t launch_element_scan_backward(sx_body body, const EsVjpParams& v, hipStream_t stream);
// workspace words the norm-cap gradient's split along the axis takes
int64_t element_scan_backward_bound_words(sx_body body, const EsParams& p);
// The norm-capped body with four state components per thread (normcap_quad.hip):
// n == 16, unit component strides (or width one), 16-byte alignment,
// non-negative strides and tensors spanning fewer than 2^31 bytes.
struct NcQuadSpans {
  int32_t x, s, out;  // bytes from each base pointer to one past its last element
};
bool normcap_quad_forward_eligible(const EsParams& p);
hipError_t launch_normcap_quad_forward(const EsParams& p, hipStream_t stream);
bool normcap_quad_eligible(const EsVjpParams& v);
hipError_t launch_normcap_quad_backward(const EsVjpParams& v, hipStream_t stream);
int64_t normcap_quad_bound_words(const EsParams& p);

// ---------------------------------------------------------------- table-scan

constexpr int kTsMaxSymbolsWave = 2048;   // per-symbol maps in LDS (8 or 16 bytes each) for tables of <= 16 states
constexpr int kTsMaxTableLds = 12288;     // the serial kernel keeps a table of up to 48 KB in LDS

// A sequence is every index of `symbols` but the axis (offsets of symbols, out).
struct TsParams {
  IndexMap<2> seqs;
  int64_t num_seq;
  int64_t T;             // symbols along the axis
  int64_t t_stride[2];   // along the axis: symbols, out (elements)
  int states, nsym;      // table is [states, nsym], row-major
  int start;
  const int32_t* table;
  const int32_t* symbols;
  int32_t* out;
};
hipError_t launch_table_scan(const TsParams& p, hipStream_t stream);

// linear-scan runs on the element-scan kernels: b as the sequence x, a as the
// second sequence s, init == nullptr (every lane starts from zero), and the
// trip h -> a * h + b, a body of the library's own beside the public three.
// Its x and s point at bf16 (uint16_t) elements when in_bf16, and out at bf16
// elements when out_bf16; strides and offsets count elements either way.
constexpr int kBodyLinear = 3;
hipError_t launch_linear_scan(const EsParams& p, bool in_bf16, bool out_bf16, hipStream_t stream);

// ---------------------------------------------------------------- matrix-scan

enum MsTensor { MS_A = 0, MS_B = 1, MS_OUT = 2 };

struct MsParams {
  IndexMap<3> batch;     // batch index (every leading index but the axis) -> offsets of a, b, out
  int64_t num_batch;
  int64_t T;             // steps along the axis (>= 1)
  int64_t t_stride[3];   // element stride of one step along the axis for a, b, out
  int n, m;              // a is n x n, b and out n x m; matrix dims are row-major contiguous
  int in_bf16;           // a and b are bf16 (else f32)
  int out_bf16;          // out is bf16 (else f32)
  int reverse;
  int adjoint;           // step q multiplies by the transpose of a at position q - 1 (the gradient's scan)
  const float* step_scale;  // :projective's second pass: h[t] = (a[t] h + b[t]) * step_scale[batch * T + t]
  const void* a;
  const void* b;
  void* out;
  // The gradient's adjoint scan may form grad_a[t] = lam[t] h[prev]^T in its replay (f32, n = 16,
  // m = 1, where the pipelined kernel runs: matrix_scan_folds_grad_a says when). fold_h is the
  // forward result, laid out as out; fold_grad_a is contiguous f32, the leading dims + [16, 16].
  // Both nullptr otherwise.
  const void* fold_h;
  void* fold_grad_a;
};

hipError_t launch_matrix_scan(const MsParams& p, void* workspace, size_t workspace_bytes, hipStream_t stream);
// Whether launch_matrix_scan, given p with fold_h and fold_grad_a set and this workspace, forms
// grad_a in the adjoint scan itself (else the caller runs launch_grad_a).
bool matrix_scan_folds_grad_a(const MsParams& p, const void* workspace, size_t workspace_bytes);
// :projective: the running product's largest entry divides P and h every step. In parallel (two passes
// for the factors, then the pipelined scan) when the shape and the workspace allow, else serially.
hipError_t launch_matrix_scan_projective(const MsParams& p, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);
size_t matrix_scan_workspace(const MsParams& p);
// Polls a matrix-scan look-back makes before it gives up (0: the default,
// about a tenth of a second); process-wide, for the calls launched after it.
void set_lookback_spin_limit(uint32_t limit);
// Byte offset, in a matrix-scan workspace, of the status word a look-back
// that gave up sets (a 32-bit word, zero while every look-back completed).
constexpr size_t kMatrixScanStatusOffset = 4;
// sx_matrix_scan_noalloc: the look-back state lives in a fixed device array of
// this many bytes (SX_MATRIX_SCAN_SCRATCH_BYTES); matrix_scan_scratch gives its
// address on the current device, set up (and zero-filled) on first use.
constexpr size_t kMatrixScanScratchBytes = SX_MATRIX_SCAN_SCRATCH_BYTES;
hipError_t matrix_scan_scratch(void** out);

// ---------------------------------------------------------------- matrix-scan gradient

// grad_a[s] = lam[s] @ h[prev(s)]^T for every step s (a row-major index over
// the leading dims; prev(s) is the step before s in the forward scan order),
// zero at the first step; optionally grad_b[s] = lam[s] rounded to bf16.
struct GradAParams {
  int64_t steps;         // product of the leading dims
  int64_t T, inner;      // scan axis length; product of the leading dims after it
  int n, m;
  int reverse;           // of the forward scan
  const void* lam;       // contiguous, leading dims + [n, m]; bf16 when lam_bf16, else f32
  int lam_bf16;
  const void* h;         // the forward result, contiguous, leading dims + [n, m]
  void* grad_a;          // contiguous, leading dims + [n, n]; bf16 when grad_a_bf16, else f32
  void* grad_b;          // nullptr, or contiguous bf16, leading dims + [n, m]
};
hipError_t launch_grad_a(const GradAParams& g, bool h_bf16, bool grad_a_bf16, hipStream_t stream);

// out[e] = sum of src over the dims a broadcast operand was stretched along:
// target element e (row-major over the kept dims) starts at src offset
// decode(e, keep), and the reduced index j adds decode(j, red).
struct SumToParams {
  const float* src;
  float* partial;        // splits x targets floats of workspace
  int64_t targets, reduced, splits, per;
  int nd_keep, nd_red;
  int64_t keep_dim[kMaxRank + 2], keep_st[kMaxRank + 2];
  int64_t red_dim[kMaxRank + 2], red_st[kMaxRank + 2];
};
hipError_t launch_sum_to(const SumToParams& p, void* out, bool out_bf16, hipStream_t stream);

// ---------------------------------------------------------------- streaming loads

// A load of an input that is read exactly once. The non-temporal hint keeps
// the stream from displacing lines in L2 and the last-level cache that the
// kernel's stores and other data still use; on MI355X it raises a two-reads-
// one-write stream from 5.6 to 7.0 TB/s (measured, plain vs hinted loads).
// Workgroups go to the eight XCDs in turn (block b to XCD b mod 8), and each
// XCD has its own L2. xcd_block() renumbers the blocks so that each XCD holds
// one contiguous range of them, so that neighbouring blocks share an L2.
constexpr int kXcds = 8;
__device__ __forceinline__ int64_t xcd_block() {
  const int64_t nb = gridDim.x, b = blockIdx.x;
  const int64_t per = nb / kXcds, rem = nb % kXcds, xcd = b % kXcds, slot = b / kXcds;
  return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) { return __builtin_nontemporal_load(p); }

// A store of an output that is written once and not read back by the kernel.
// With rotating buffers (no cache reuse between calls) the hint takes the
// max-plus scan from 156 to 147 us (measured).
template <typename T>
__device__ __forceinline__ void st_stream(T* p, T v) { __builtin_nontemporal_store(v, p); }

// ---------------------------------------------------------------- bf16 helpers

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// Round to nearest, ties to even. NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

}  // namespace sx
