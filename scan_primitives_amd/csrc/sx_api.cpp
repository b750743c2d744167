// sx_api.cpp: the C ABI of libsx_scan.so (declared in include/sx_scan.h).
//
// Every argument is validated here, on the host, before anything touches the
// device: a rejected call launches nothing and leaves `out` alone. The
// shapes and strides are then reduced to the compact descriptors of
// sx_common.hpp and handed to the launchers in element_scan.hip and
// matrix_scan.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "sx_common.hpp"

namespace sx {

int device_cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev < 64) cached[dev] = cus;
  return cus;
}

}  // namespace sx

namespace {

thread_local std::string g_last_error;

sx_status fail(sx_status st, const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = std::string("error[") + sx_status_name(st) + "]: " + buf;
  return st;
}

sx_status ok() {
  g_last_error.clear();
  return SX_OK;
}

// The integer an enum argument holds. A C caller may pass any int where the
// ABI declares an enum; reading it as the C++ enum type before it is checked
// would be undefined for values outside the enum's range, so every entry point
// checks the bits first.
template <typename E>
int enum_code(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized here");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

bool body_ok(const sx_body& b) {
  const int v = enum_code(b);
  return v == SX_BODY_TANH_AFFINE || v == SX_BODY_NORM_CAP || v == SX_BODY_MAX_PLUS;
}

bool dtype_ok(const sx_dtype& d) {
  const int v = enum_code(d);
  return v == SX_F32 || v == SX_BF16;
}

std::string shape_str(int rank, const int64_t* shape) {
  std::string s = "[";
  for (int i = 0; i < rank; ++i) {
    if (i) s += ", ";
    s += std::to_string(shape[i]);
  }
  return s + "]";
}

const char* dtype_name(int dt) { return dt == SX_F32 ? "f32" : dt == SX_BF16 ? "bf16" : "?"; }

void contiguous_strides(int rank, const int64_t* shape, int64_t* st) {
  int64_t acc = 1;
  for (int i = rank - 1; i >= 0; --i) {
    st[i] = acc;
    acc *= std::max<int64_t>(shape[i], 1);
  }
}

// Checked product; returns false on overflow past 2^62.
bool checked_numel(int rank, const int64_t* shape, int64_t* numel) {
  int64_t n = 1;
  for (int i = 0; i < rank; ++i) {
    if (shape[i] < 0) return false;
    if (shape[i] != 0 && n > (int64_t(1) << 62) / shape[i]) return false;
    n *= shape[i];
  }
  *numel = n;
  return true;
}

// Byte span [lo, hi) that a strided tensor touches (only meaningful when numel > 0).
void span_bytes(const void* base, int rank, const int64_t* shape, const int64_t* st, size_t elem,
                uintptr_t* lo, uintptr_t* hi) {
  int64_t mn = 0, mx = 0;
  for (int i = 0; i < rank; ++i) {
    const int64_t e = (shape[i] - 1) * st[i];
    if (e < 0) mn += e; else mx += e;
  }
  const uintptr_t b = reinterpret_cast<uintptr_t>(base);
  *lo = b + uintptr_t(mn * int64_t(elem));
  *hi = b + uintptr_t((mx + 1) * int64_t(elem));
}

bool overlaps(uintptr_t alo, uintptr_t ahi, uintptr_t blo, uintptr_t bhi) { return alo < bhi && blo < ahi; }

// Builds an IndexMap from per-dimension sizes and strides, dropping size-1
// dims and merging neighbours whose strides nest for every tensor.
template <int NT>
sx::IndexMap<NT> make_index_map(int nd, const int64_t* dims, const int64_t (*st)[sx::kMaxRank]) {
  sx::IndexMap<NT> m{};
  int k = 0;
  for (int d = 0; d < nd; ++d) {
    if (dims[d] == 1) continue;
    bool merge = k > 0;
    for (int t = 0; t < NT && merge; ++t) merge = st[t][d] * dims[d] == m.st[t][k - 1];
    if (merge) {
      m.dim[k - 1] *= dims[d];
      for (int t = 0; t < NT; ++t) m.st[t][k - 1] = st[t][d];
    } else {
      m.dim[k] = dims[d];
      for (int t = 0; t < NT; ++t) m.st[t][k] = st[t][d];
      ++k;
    }
  }
  if (k == 0) {
    m.dim[0] = 1;
    for (int t = 0; t < NT; ++t) m.st[t][0] = 0;
    k = 1;
  }
  m.nd = k;
  return m;
}

sx_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SX_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// ------------------------------------------------------------ element-scan validation

struct EsPlan {
  sx::EsParams p;
  int64_t numel;
};

sx_status plan_element_scan(sx_body body, int rank, const int64_t* shape, int axis, int state_axis,
                            const int64_t* initial_strides, int64_t x_width, const int64_t* x_strides,
                            int64_t s_width, const int64_t* s_strides, EsPlan* plan) {
  if (body != SX_BODY_TANH_AFFINE && body != SX_BODY_NORM_CAP && body != SX_BODY_MAX_PLUS)
    return fail(SX_E_UNSUPPORTED, "element-scan: unknown body %d", int(body));
  if (rank > sx::kMaxRank) return fail(SX_E_UNSUPPORTED, "element-scan: rank %d exceeds %d", rank, sx::kMaxRank);
  if (rank < 1 || shape == nullptr) return fail(SX_E_DIM_001, "element-scan: sequences need at least one axis");
  int64_t numel = 0;
  if (!checked_numel(rank, shape, &numel))
    return fail(SX_E_DIM_001, "element-scan: bad sequence shape %s", shape_str(rank, shape).c_str());
  const int ax = axis < 0 ? axis + rank : axis;
  if (ax < 0 || ax >= rank)
    return fail(SX_E_DIM_001, "element-scan: axis %d out of range for sequences %s f32", axis,
                shape_str(rank, shape).c_str());
  const bool vec = state_axis != SX_STATE_SCALAR;
  if (vec && state_axis != -1 && state_axis != rank - 1)
    return fail(SX_E_DIM_001, "element-scan: :state-axis %d is not the last axis of %s", state_axis,
                shape_str(rank, shape).c_str());
  if (!vec && body == SX_BODY_NORM_CAP)
    return fail(SX_E_DIM_001, "element-scan: the norm-cap body reduces over the state, so it needs :state-axis -1");
  int64_t n = 1;
  if (vec) {
    if (rank < 2 || ax == rank - 1)
      return fail(SX_E_DIM_001, "element-scan: :axis %d is the state axis of %s", axis, shape_str(rank, shape).c_str());
    n = shape[rank - 1];
    if (n < 1 || n > SX_MAX_N)
      return fail(SX_E_DIM_001, "element-scan: state width %lld is outside 1..16", (long long)n);
    if (x_width != 1 && x_width != n)
      return fail(SX_E_DIM_001, "element-scan: sequence x has width %lld, state width is %lld", (long long)x_width, (long long)n);
    if (s_width != 1 && s_width != n)
      return fail(SX_E_DIM_001, "element-scan: second sequence has width %lld, state width is %lld", (long long)s_width, (long long)n);
  }
  const int64_t T = shape[ax];
  if (T < 1)
    return fail(SX_E_DIM_001, "element-scan: axis %d of %s has length 0; it must be at least one", axis,
                shape_str(rank, shape).c_str());

  // Per-tensor shapes and strides (elements).
  int64_t xs[sx::kMaxRank], ss[sx::kMaxRank], is[sx::kMaxRank], os[sx::kMaxRank];
  int64_t xshape[sx::kMaxRank], sshape[sx::kMaxRank], ishape[sx::kMaxRank];
  for (int i = 0; i < rank; ++i) xshape[i] = sshape[i] = shape[i];
  if (vec) { xshape[rank - 1] = x_width; sshape[rank - 1] = s_width; }
  for (int i = 0, j = 0; i < rank; ++i)
    if (i != ax) ishape[j++] = shape[i];
  if (x_strides) std::copy(x_strides, x_strides + rank, xs); else contiguous_strides(rank, xshape, xs);
  if (s_strides) std::copy(s_strides, s_strides + rank, ss); else contiguous_strides(rank, sshape, ss);
  if (initial_strides) std::copy(initial_strides, initial_strides + rank - 1, is); else contiguous_strides(rank - 1, ishape, is);
  contiguous_strides(rank, shape, os);
  if (vec) {  // a width-1 sequence broadcasts over the state vector
    if (x_width == 1) xs[rank - 1] = 0;
    if (s_width == 1) ss[rank - 1] = 0;
  }

  sx::EsParams& p = plan->p;
  p = sx::EsParams{};
  p.T = T;
  p.t_stride[sx::ES_X] = xs[ax];
  p.t_stride[sx::ES_S] = ss[ax];
  p.t_stride[sx::ES_INIT] = 0;
  p.t_stride[sx::ES_OUT] = os[ax];
  p.n = body == SX_BODY_NORM_CAP ? int(n) : 1;
  if (body == SX_BODY_NORM_CAP) {
    p.n_stride[sx::ES_X] = xs[rank - 1];
    p.n_stride[sx::ES_S] = ss[rank - 1];
    p.n_stride[sx::ES_INIT] = is[rank - 2];
    p.n_stride[sx::ES_OUT] = 1;
  }
  // Lane dims: every dim but the axis (and but the state axis for NORM_CAP).
  const int lane_end = body == SX_BODY_NORM_CAP ? rank - 1 : rank;
  int64_t dims[sx::kMaxRank];
  int64_t st[4][sx::kMaxRank];
  int nd = 0;
  for (int i = 0; i < lane_end; ++i) {
    if (i == ax) continue;
    dims[nd] = shape[i];
    st[sx::ES_X][nd] = xs[i];
    st[sx::ES_S][nd] = ss[i];
    st[sx::ES_INIT][nd] = is[i < ax ? i : i - 1];
    st[sx::ES_OUT][nd] = os[i];
    ++nd;
  }
  p.lanes = make_index_map<4>(nd, dims, st);
  p.num_lanes = numel / T / (body == SX_BODY_NORM_CAP ? n : 1);
  plan->numel = numel;

  // Spans for the alias check are computed by the caller once the pointers are known.
  (void)xshape;
  return ok();
}

}  // namespace

extern "C" {

const char* sx_status_name(sx_status status) {
  switch (enum_code(status)) {
    case SX_OK: return "OK";
    case SX_E_DIM_001: return "E-DIM-001";
    case SX_E_DIM_002: return "E-DIM-002";
    case SX_E_DIM_003: return "E-DIM-003";
    case SX_E_UNSUPPORTED: return "E-UNSUPPORTED";
    case SX_E_ALIAS: return "E-ALIAS";
    case SX_E_WORKSPACE: return "E-WORKSPACE";
    case SX_E_DEVICE: return "E-DEVICE";
  }
  return "E-UNKNOWN";
}

const char* sx_last_error(void) { return g_last_error.c_str(); }

const char* sx_version(void) { return "sx_scan 0.1 gfx950"; }

size_t sx_element_scan_workspace_bytes(sx_body body, int rank, const int64_t* shape, int axis, int state_axis) {
  if (!body_ok(body)) return 0;
  EsPlan plan;
  const int64_t w = 1;
  if (plan_element_scan(body, rank, shape, axis, state_axis, nullptr, w, nullptr, w, nullptr, &plan) != SX_OK)
    return 0;
  return sx::element_scan_workspace(body, plan.p);
}

sx_status sx_element_scan(sx_body body, int rank, const int64_t* shape, int axis, int state_axis, int reverse,
                          const float* initial, const int64_t* initial_strides, const float* x, int64_t x_width,
                          const int64_t* x_strides, const float* s, int64_t s_width, const int64_t* s_strides,
                          float* out, void* workspace, size_t workspace_bytes, void* stream) {
  if (!body_ok(body)) return fail(SX_E_UNSUPPORTED, "element-scan: unknown body %d", enum_code(body));
  EsPlan plan;
  sx_status st = plan_element_scan(body, rank, shape, axis, state_axis, initial_strides, x_width, x_strides,
                                   s_width, s_strides, &plan);
  if (st != SX_OK) return st;
  if (plan.numel == 0) return ok();
  if (!x) return fail(SX_E_DIM_003, "element-scan: sequence x is NULL; a tensor was expected");
  if (!s) return fail(SX_E_DIM_003, "element-scan: the second sequence is NULL; a tensor was expected");
  if (!initial) return fail(SX_E_DIM_003, "element-scan: initial is NULL; a tensor was expected");
  if (!out) return fail(SX_E_DIM_003, "element-scan: out is NULL; a tensor was expected");

  // Alias check: out is contiguous over the output shape.
  const bool vec = state_axis != SX_STATE_SCALAR;
  int64_t xshape[sx::kMaxRank], sshape[sx::kMaxRank], ishape[sx::kMaxRank];
  int64_t xs[sx::kMaxRank], ss[sx::kMaxRank], is[sx::kMaxRank];
  const int ax = axis < 0 ? axis + rank : axis;
  for (int i = 0; i < rank; ++i) xshape[i] = sshape[i] = shape[i];
  if (vec) { xshape[rank - 1] = x_width; sshape[rank - 1] = s_width; }
  for (int i = 0, j = 0; i < rank; ++i)
    if (i != ax) ishape[j++] = shape[i];
  if (x_strides) std::copy(x_strides, x_strides + rank, xs); else contiguous_strides(rank, xshape, xs);
  if (s_strides) std::copy(s_strides, s_strides + rank, ss); else contiguous_strides(rank, sshape, ss);
  if (initial_strides) std::copy(initial_strides, initial_strides + rank - 1, is); else contiguous_strides(rank - 1, ishape, is);
  uintptr_t olo = reinterpret_cast<uintptr_t>(out), ohi = olo + uintptr_t(plan.numel) * sizeof(float);
  uintptr_t lo, hi;
  span_bytes(x, rank, xshape, xs, sizeof(float), &lo, &hi);
  if (overlaps(olo, ohi, lo, hi)) return fail(SX_E_ALIAS, "element-scan: out overlaps sequence x");
  span_bytes(s, rank, sshape, ss, sizeof(float), &lo, &hi);
  if (overlaps(olo, ohi, lo, hi)) return fail(SX_E_ALIAS, "element-scan: out overlaps the second sequence");
  span_bytes(initial, rank - 1, ishape, is, sizeof(float), &lo, &hi);
  if (overlaps(olo, ohi, lo, hi)) return fail(SX_E_ALIAS, "element-scan: out overlaps initial");

  const size_t need = sx::element_scan_workspace(body, plan.p);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(SX_E_WORKSPACE, "element-scan: workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(SX_E_WORKSPACE, "element-scan: workspace must be 256-byte aligned");

  plan.p.reverse = reverse ? 1 : 0;
  plan.p.x = x;
  plan.p.s = s;
  plan.p.init = initial;
  plan.p.out = out;
  return device_status(sx::launch_element_scan(body, plan.p, static_cast<hipStream_t>(stream)),
                       "element-scan launch");
}

// ------------------------------------------------------------------ matrix-scan

static sx_status plan_matrix_scan(int a_rank, const int64_t* a_shape, const int64_t* a_strides, int b_rank,
                                  const int64_t* b_shape, const int64_t* b_strides, int axis, sx::MsParams* p,
                                  int64_t* out_shape, int* out_rank, int64_t* out_numel) {
  if (a_rank > sx::kMaxRank || b_rank > sx::kMaxRank)
    return fail(SX_E_UNSUPPORTED, "matrix-scan: rank above %d", sx::kMaxRank);
  if (!a_shape || !b_shape || a_rank < 2 || b_rank < 2)
    return fail(SX_E_DIM_001, "matrix-scan: a must be [.., n, n] and b [.., n, m]");
  int64_t tmp;
  if (!checked_numel(a_rank, a_shape, &tmp) || !checked_numel(b_rank, b_shape, &tmp))
    return fail(SX_E_DIM_001, "matrix-scan: negative or oversized dims in a %s, b %s",
                shape_str(a_rank, a_shape).c_str(), shape_str(b_rank, b_shape).c_str());
  const int64_t n = a_shape[a_rank - 1];
  if (a_shape[a_rank - 2] != n)
    return fail(SX_E_DIM_001, "matrix-scan: a %s is not square", shape_str(a_rank, a_shape).c_str());
  if (b_shape[b_rank - 2] != n)
    return fail(SX_E_DIM_001, "matrix-scan: inner dims differ: a %s, b %s", shape_str(a_rank, a_shape).c_str(),
                shape_str(b_rank, b_shape).c_str());
  if (n > SX_MAX_N)
    return fail(SX_E_DIM_001, "matrix-scan: n = %lld, at most 16 allowed (a %s)", (long long)n,
                shape_str(a_rank, a_shape).c_str());
  const int64_t m = b_shape[b_rank - 1];
  const int la = a_rank - 2, lb = b_rank - 2, L = std::max(la, lb);
  if (L < 1)
    return fail(SX_E_DIM_001, "matrix-scan: no leading dim to scan along (a %s, b %s)",
                shape_str(a_rank, a_shape).c_str(), shape_str(b_rank, b_shape).c_str());
  if (L + 2 > sx::kMaxRank) return fail(SX_E_UNSUPPORTED, "matrix-scan: result rank above %d", sx::kMaxRank);
  int64_t lead[sx::kMaxRank], sa[sx::kMaxRank], sb[sx::kMaxRank];
  int64_t ast[sx::kMaxRank], bst[sx::kMaxRank];
  if (a_strides) std::copy(a_strides, a_strides + a_rank, ast); else contiguous_strides(a_rank, a_shape, ast);
  if (b_strides) std::copy(b_strides, b_strides + b_rank, bst); else contiguous_strides(b_rank, b_shape, bst);
  for (int i = 0; i < L; ++i) {
    const int ia = i - (L - la), ib = i - (L - lb);
    const int64_t da = ia >= 0 ? a_shape[ia] : 1, db = ib >= 0 ? b_shape[ib] : 1;
    if (da != db && da != 1 && db != 1)
      return fail(SX_E_DIM_001, "matrix-scan: leading dims of a %s and b %s do not broadcast",
                  shape_str(a_rank, a_shape).c_str(), shape_str(b_rank, b_shape).c_str());
    lead[i] = da == 1 ? db : da;
    sa[i] = (ia >= 0 && da != 1) ? ast[ia] : 0;
    sb[i] = (ib >= 0 && db != 1) ? bst[ib] : 0;
  }
  const int ax = axis < 0 ? axis + L : axis;
  if (ax < 0 || ax >= L)
    return fail(SX_E_DIM_001, "matrix-scan: axis %d out of range for leading dims %s", axis,
                shape_str(L, lead).c_str());
  if ((n > 1 && (ast[a_rank - 1] != 1 || ast[a_rank - 2] != n)) ||
      (m > 1 && bst[b_rank - 1] != 1) || (n > 1 && m > 0 && bst[b_rank - 2] != m))
    return fail(SX_E_UNSUPPORTED, "matrix-scan: the matrix dims of a and b must be row-major contiguous");

  for (int i = 0; i < L; ++i) out_shape[i] = lead[i];
  out_shape[L] = n;
  out_shape[L + 1] = m;
  *out_rank = L + 2;
  int64_t numel = 0;
  if (!checked_numel(L + 2, out_shape, &numel)) return fail(SX_E_DIM_001, "matrix-scan: result too large");
  *out_numel = numel;
  if (!p) return ok();

  int64_t ost[sx::kMaxRank + 2];
  contiguous_strides(L + 2, out_shape, ost);
  *p = sx::MsParams{};
  p->T = lead[ax];
  p->t_stride[sx::MS_A] = sa[ax];
  p->t_stride[sx::MS_B] = sb[ax];
  p->t_stride[sx::MS_OUT] = ost[ax];
  p->n = int(n);
  p->m = int(m);
  int64_t dims[sx::kMaxRank];
  int64_t st[3][sx::kMaxRank];
  int nd = 0;
  for (int i = 0; i < L; ++i) {
    if (i == ax) continue;
    dims[nd] = lead[i];
    st[sx::MS_A][nd] = sa[i];
    st[sx::MS_B][nd] = sb[i];
    st[sx::MS_OUT][nd] = ost[i];
    ++nd;
  }
  p->batch = make_index_map<3>(nd, dims, st);
  p->num_batch = p->T > 0 ? numel / (p->T * std::max<int64_t>(n * m, 1)) : 0;
  if (n * m == 0) p->num_batch = 0;
  return ok();
}

int sx_matrix_scan_out_shape(int a_rank, const int64_t* a_shape, int b_rank, const int64_t* b_shape,
                             int64_t* out_shape) {
  int64_t shp[sx::kMaxRank + 2];
  int r = 0;
  int64_t numel = 0;
  if (plan_matrix_scan(a_rank, a_shape, nullptr, b_rank, b_shape, nullptr, -1, nullptr, shp, &r, &numel) != SX_OK)
    return -1;
  if (out_shape) std::copy(shp, shp + r, out_shape);
  return r;
}

size_t sx_matrix_scan_workspace_bytes(int a_rank, const int64_t* a_shape, int b_rank, const int64_t* b_shape,
                                      int axis) {
  sx::MsParams p;
  int64_t shp[sx::kMaxRank + 2];
  int r = 0;
  int64_t numel = 0;
  if (plan_matrix_scan(a_rank, a_shape, nullptr, b_rank, b_shape, nullptr, axis, &p, shp, &r, &numel) != SX_OK)
    return 0;
  if (numel == 0) return 0;
  return sx::matrix_scan_workspace(p);
}

}  // extern "C"

namespace {

// sx_matrix_scan, and with scratch = true sx_matrix_scan_noalloc: the look-back
// state then goes to the library's fixed device array instead of `workspace`.
sx_status matrix_scan_call(const sx_dtype& dtype, int a_rank, const int64_t* a_shape, const int64_t* a_strides,
                           const void* a, int b_rank, const int64_t* b_shape, const int64_t* b_strides, const void* b,
                           int axis, int reverse, int projective, const sx_dtype& out_dtype, void* out, void* workspace,
                           size_t workspace_bytes, void* stream, bool scratch) {
  if (!dtype_ok(dtype))
    return fail(SX_E_DIM_002, "matrix-scan: a and b must be f32 or bf16 (dtype code %d)", enum_code(dtype));
  if (!dtype_ok(out_dtype))
    return fail(SX_E_DIM_002, "matrix-scan: out must be f32 or bf16 (dtype code %d)", enum_code(out_dtype));
  sx::MsParams p;
  int64_t shp[sx::kMaxRank + 2];
  int r = 0;
  int64_t numel = 0;
  sx_status st = plan_matrix_scan(a_rank, a_shape, a_strides, b_rank, b_shape, b_strides, axis, &p, shp, &r, &numel);
  if (st != SX_OK) return st;
  if (numel == 0) return ok();
  if (!a) return fail(SX_E_DIM_003, "matrix-scan: a %s %s is NULL; a tensor was expected",
                      shape_str(a_rank, a_shape).c_str(), dtype_name(dtype));
  if (!b) return fail(SX_E_DIM_003, "matrix-scan: b %s %s is NULL; a tensor was expected",
                      shape_str(b_rank, b_shape).c_str(), dtype_name(dtype));
  if (!out) return fail(SX_E_DIM_003, "matrix-scan: out is NULL; a tensor was expected");

  const size_t esz = dtype == SX_BF16 ? 2 : 4, osz = out_dtype == SX_BF16 ? 2 : 4;
  int64_t ast[sx::kMaxRank], bst[sx::kMaxRank];
  if (a_strides) std::copy(a_strides, a_strides + a_rank, ast); else contiguous_strides(a_rank, a_shape, ast);
  if (b_strides) std::copy(b_strides, b_strides + b_rank, bst); else contiguous_strides(b_rank, b_shape, bst);
  uintptr_t olo = reinterpret_cast<uintptr_t>(out), ohi = olo + uintptr_t(numel) * osz, lo, hi;
  int64_t anumel = 0, bnumel = 0;
  checked_numel(a_rank, a_shape, &anumel);
  checked_numel(b_rank, b_shape, &bnumel);
  if (anumel > 0) {
    span_bytes(a, a_rank, a_shape, ast, esz, &lo, &hi);
    if (overlaps(olo, ohi, lo, hi)) return fail(SX_E_ALIAS, "matrix-scan: out overlaps a");
  }
  if (bnumel > 0) {
    span_bytes(b, b_rank, b_shape, bst, esz, &lo, &hi);
    if (overlaps(olo, ohi, lo, hi)) return fail(SX_E_ALIAS, "matrix-scan: out overlaps b");
  }
  const size_t need = sx::matrix_scan_workspace(p);
  if (scratch) {
    if (need > sx::kMatrixScanScratchBytes)
      return fail(SX_E_WORKSPACE,
                  "matrix-scan: a %s by %s scan needs %zu bytes of look-back state, more than the %zu bytes the "
                  "allocation-free entry point keeps; use sx_matrix_scan with a workspace",
                  shape_str(a_rank, a_shape).c_str(), shape_str(b_rank, b_shape).c_str(), need,
                  sx::kMatrixScanScratchBytes);
    workspace_bytes = sx::kMatrixScanScratchBytes;
    workspace = nullptr;
    if (need > 0) {
      const hipError_t e = sx::matrix_scan_scratch(&workspace);
      if (e != hipSuccess) return device_status(e, "matrix-scan: setting up the scratch array");
    }
  }
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(SX_E_WORKSPACE, "matrix-scan: workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(SX_E_WORKSPACE, "matrix-scan: workspace must be 256-byte aligned");
  if (projective) {
    p.in_bf16 = dtype == SX_BF16;
    p.out_bf16 = out_dtype == SX_BF16;
    p.reverse = reverse ? 1 : 0;
    p.a = a;
    p.b = b;
    p.out = out;
    return device_status(
        sx::launch_matrix_scan_projective(p, workspace, workspace_bytes, static_cast<hipStream_t>(stream)),
        "matrix-scan :projective launch");
  }

  p.in_bf16 = dtype == SX_BF16;
  p.out_bf16 = out_dtype == SX_BF16;
  p.reverse = reverse ? 1 : 0;
  p.a = a;
  p.b = b;
  p.out = out;
  return device_status(sx::launch_matrix_scan(p, workspace, workspace_bytes, static_cast<hipStream_t>(stream)),
                       "matrix-scan launch");
}

}  // namespace

extern "C" {

sx_status sx_matrix_scan(sx_dtype dtype, int a_rank, const int64_t* a_shape, const int64_t* a_strides, const void* a,
                         int b_rank, const int64_t* b_shape, const int64_t* b_strides, const void* b, int axis,
                         int reverse, int projective, sx_dtype out_dtype, void* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return matrix_scan_call(dtype, a_rank, a_shape, a_strides, a, b_rank, b_shape, b_strides, b, axis, reverse,
                          projective, out_dtype, out, workspace, workspace_bytes, stream, false);
}

sx_status sx_matrix_scan_noalloc(sx_dtype dtype, int a_rank, const int64_t* a_shape, const int64_t* a_strides,
                                 const void* a, int b_rank, const int64_t* b_shape, const int64_t* b_strides,
                                 const void* b, int axis, int reverse, int projective, sx_dtype out_dtype, void* out,
                                 void* stream) {
  return matrix_scan_call(dtype, a_rank, a_shape, a_strides, a, b_rank, b_shape, b_strides, b, axis, reverse,
                          projective, out_dtype, out, nullptr, 0, stream, true);
}

sx_status sx_matrix_scan_workspace_status(void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace == nullptr)
    return fail(SX_E_DIM_003, "matrix-scan workspace status: the workspace is NULL; a buffer was expected");
  if (workspace_bytes < 256)
    return fail(SX_E_WORKSPACE, "matrix-scan workspace status: %zu bytes is smaller than a workspace header (256)",
                workspace_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* word = static_cast<char*>(workspace) + sx::kMatrixScanStatusOffset;
  uint32_t status = 0;
  hipError_t e = hipMemcpyAsync(&status, word, sizeof status, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return device_status(e, "matrix-scan workspace status: reading the status word");
  if (status == 0) return ok();
  static const uint32_t zero = 0;
  e = hipMemcpyAsync(word, &zero, sizeof zero, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return device_status(e, "matrix-scan workspace status: clearing the status word");
  return fail(SX_E_DEVICE,
              "matrix-scan: a look-back gave up waiting for an earlier unit's published state (spin limit reached); "
              "results of the calls on this workspace since its last check are not valid");
}

void sx_set_lookback_spin_limit(uint32_t limit) { sx::set_lookback_spin_limit(limit); }

}  // extern "C"

// ------------------------------------------------------------------ matrix-scan gradient

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Sum of a contiguous full-shape f32 tensor (rank R) down to a target shape
// (right-aligned, each dim equal or 1): which dims are kept, which summed.
sx::SumToParams sum_to_plan(int R, const int64_t* full, int t_rank, const int64_t* tshape) {
  sx::SumToParams q{};
  int64_t fst[sx::kMaxRank + 2];
  contiguous_strides(R, full, fst);
  q.targets = 1;
  q.reduced = 1;
  for (int d = 0; d < R; ++d) {
    const int e = d - (R - t_rank);
    const bool summed = e < 0 || (tshape[e] == 1 && full[d] != 1);
    if (summed) {
      q.red_dim[q.nd_red] = full[d];
      q.red_st[q.nd_red++] = fst[d];
      q.reduced *= full[d];
    } else {
      q.keep_dim[q.nd_keep] = full[d];
      q.keep_st[q.nd_keep++] = fst[d];
      q.targets *= full[d];
    }
  }
  // slices of the summed space: at least 32 terms each, at most 64 MiB of partial sums
  int64_t splits = std::max<int64_t>(1, std::min<int64_t>(65535, q.reduced / 32));
  if (q.targets > 0) splits = std::max<int64_t>(1, std::min<int64_t>(splits, (int64_t(64) << 20) / 4 / q.targets));
  q.splits = splits;
  q.per = (q.reduced + splits - 1) / splits;
  return q;
}

bool same_shape(int r1, const int64_t* s1, int r2, const int64_t* s2) {
  if (r1 != r2) return false;
  for (int i = 0; i < r1; ++i)
    if (s1[i] != s2[i]) return false;
  return true;
}

struct MsBackPlan {
  sx::MsParams p;                       // the adjoint scan (b = g, out = lam)
  int out_rank;
  int64_t out_shape[sx::kMaxRank + 2];  // lead + [n, m]
  int64_t out_numel, a_full_numel;
  bool lam_direct, ga_direct;           // lam is grad_b itself (f32, or rounded to a bf16 grad_b); grad_a in place
  sx::SumToParams sum_a, sum_b;
  size_t scan_ws, lam_off, ga_off, part_off, total;
};

sx_status plan_matrix_scan_backward(int a_rank, const int64_t* a_shape, const int64_t* a_strides, int b_rank,
                                    const int64_t* b_shape, const int64_t* g_strides, int axis, MsBackPlan* bp) {
  sx::MsParams fwd;
  int64_t numel = 0;
  sx_status st = plan_matrix_scan(a_rank, a_shape, nullptr, b_rank, b_shape, nullptr, axis, &fwd, bp->out_shape,
                                  &bp->out_rank, &numel);
  if (st != SX_OK) return st;
  // the adjoint scan: a as given, the gradient of the result in b's place
  int r = 0;
  int64_t shp[sx::kMaxRank + 2];
  st = plan_matrix_scan(a_rank, a_shape, a_strides, bp->out_rank, bp->out_shape, g_strides, axis, &bp->p, shp, &r,
                        &bp->out_numel);
  if (st != SX_OK) return st;
  const int L = bp->out_rank - 2;
  const int64_t n = bp->out_shape[L];
  int64_t afull[sx::kMaxRank + 2];
  std::copy(bp->out_shape, bp->out_shape + L, afull);
  afull[L] = afull[L + 1] = n;
  checked_numel(L + 2, afull, &bp->a_full_numel);
  // with b at the result's shape, the scan writes lam straight into grad_b: in f32, or rounded to
  // bf16 when the gradients are bf16 (grad_a then forms lam h^T from the rounded lam)
  bp->lam_direct = same_shape(b_rank, b_shape, bp->out_rank, bp->out_shape);
  bp->ga_direct = same_shape(a_rank, a_shape, L + 2, afull);
  bp->sum_a = sum_to_plan(L + 2, afull, a_rank, a_shape);
  bp->sum_b = sum_to_plan(bp->out_rank, bp->out_shape, b_rank, b_shape);
  bp->scan_ws = align_up(sx::matrix_scan_workspace(bp->p));
  size_t off = bp->scan_ws;
  bp->lam_off = off;
  if (!bp->lam_direct) off += align_up(size_t(bp->out_numel) * 4);
  bp->ga_off = off;
  if (!bp->ga_direct) off += align_up(size_t(bp->a_full_numel) * 4);
  bp->part_off = off;
  size_t part = 0;
  if (!bp->ga_direct) part = std::max(part, size_t(bp->sum_a.splits * bp->sum_a.targets) * 4);
  if (!same_shape(b_rank, b_shape, bp->out_rank, bp->out_shape))
    part = std::max(part, size_t(bp->sum_b.splits * bp->sum_b.targets) * 4);
  bp->total = off + align_up(part);
  return ok();
}

}  // namespace

extern "C" {

size_t sx_matrix_scan_backward_workspace_bytes(int a_rank, const int64_t* a_shape, int b_rank, const int64_t* b_shape,
                                               int axis, sx_dtype grad_dtype) {
  MsBackPlan bp;
  if (!dtype_ok(grad_dtype)) return 0;
  if (plan_matrix_scan_backward(a_rank, a_shape, nullptr, b_rank, b_shape, nullptr, axis, &bp) != SX_OK) return 0;
  return bp.total;
}

sx_status sx_matrix_scan_backward(sx_dtype dtype, int a_rank, const int64_t* a_shape, const int64_t* a_strides,
                                  const void* a, int b_rank, const int64_t* b_shape, const void* h,
                                  const int64_t* g_strides, const void* g, int axis, int reverse, sx_dtype grad_dtype,
                                  void* grad_a, void* grad_b, void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(dtype))
    return fail(SX_E_DIM_002, "matrix-scan gradient: a, h and g must be f32 or bf16 (dtype code %d)", enum_code(dtype));
  if (!dtype_ok(grad_dtype))
    return fail(SX_E_DIM_002, "matrix-scan gradient: gradients must be f32 or bf16 (dtype code %d)", enum_code(grad_dtype));
  MsBackPlan bp;
  sx_status st = plan_matrix_scan_backward(a_rank, a_shape, a_strides, b_rank, b_shape, g_strides, axis, &bp);
  if (st != SX_OK) return st;
  int64_t a_numel = 0, b_numel = 0;
  checked_numel(a_rank, a_shape, &a_numel);
  checked_numel(b_rank, b_shape, &b_numel);
  if (a_numel == 0 && b_numel == 0) return ok();
  if (bp.out_numel > 0 || bp.a_full_numel > 0) {
    if (!a) return fail(SX_E_DIM_003, "matrix-scan gradient: a %s %s is NULL; a tensor was expected",
                        shape_str(a_rank, a_shape).c_str(), dtype_name(dtype));
  }
  if (bp.out_numel > 0) {
    if (!h) return fail(SX_E_DIM_003, "matrix-scan gradient: the forward result h %s is NULL; a tensor was expected",
                        shape_str(bp.out_rank, bp.out_shape).c_str());
    if (!g) return fail(SX_E_DIM_003, "matrix-scan gradient: the result's gradient g %s is NULL; a tensor was expected",
                        shape_str(bp.out_rank, bp.out_shape).c_str());
  }
  if (a_numel > 0 && !grad_a) return fail(SX_E_DIM_003, "matrix-scan gradient: grad_a is NULL; a tensor was expected");
  if (b_numel > 0 && !grad_b) return fail(SX_E_DIM_003, "matrix-scan gradient: grad_b is NULL; a tensor was expected");

  // outputs overlap no input and not each other
  const size_t esz = dtype == SX_BF16 ? 2 : 4, gsz = grad_dtype == SX_BF16 ? 2 : 4;
  int64_t ast[sx::kMaxRank], gst[sx::kMaxRank + 2], ost[sx::kMaxRank + 2];
  if (a_strides) std::copy(a_strides, a_strides + a_rank, ast); else contiguous_strides(a_rank, a_shape, ast);
  contiguous_strides(bp.out_rank, bp.out_shape, ost);
  if (g_strides) std::copy(g_strides, g_strides + bp.out_rank, gst); else std::copy(ost, ost + bp.out_rank, gst);
  struct Span { uintptr_t lo, hi; const char* name; };
  Span ins[3];
  int nin = 0;
  uintptr_t lo, hi;
  if (a_numel > 0) { span_bytes(a, a_rank, a_shape, ast, esz, &lo, &hi); ins[nin++] = {lo, hi, "a"}; }
  if (bp.out_numel > 0) {
    span_bytes(h, bp.out_rank, bp.out_shape, ost, esz, &lo, &hi); ins[nin++] = {lo, hi, "h"};
    span_bytes(g, bp.out_rank, bp.out_shape, gst, esz, &lo, &hi); ins[nin++] = {lo, hi, "g"};
  }
  const uintptr_t galo = reinterpret_cast<uintptr_t>(grad_a), gahi = galo + uintptr_t(a_numel) * gsz;
  const uintptr_t gblo = reinterpret_cast<uintptr_t>(grad_b), gbhi = gblo + uintptr_t(b_numel) * gsz;
  for (int i = 0; i < nin; ++i) {
    if (a_numel > 0 && overlaps(galo, gahi, ins[i].lo, ins[i].hi))
      return fail(SX_E_ALIAS, "matrix-scan gradient: grad_a overlaps %s", ins[i].name);
    if (b_numel > 0 && overlaps(gblo, gbhi, ins[i].lo, ins[i].hi))
      return fail(SX_E_ALIAS, "matrix-scan gradient: grad_b overlaps %s", ins[i].name);
  }
  if (a_numel > 0 && b_numel > 0 && overlaps(galo, gahi, gblo, gbhi))
    return fail(SX_E_ALIAS, "matrix-scan gradient: grad_a overlaps grad_b");
  if (bp.total > 0 && (workspace == nullptr || workspace_bytes < bp.total))
    return fail(SX_E_WORKSPACE, "matrix-scan gradient: workspace of %zu bytes given, %zu needed", workspace_bytes,
                bp.total);
  if (bp.total > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(SX_E_WORKSPACE, "matrix-scan gradient: workspace must be 256-byte aligned");

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  void* lam = bp.lam_direct ? grad_b : static_cast<void*>(ws + bp.lam_off);
  const bool lam_bf16 = bp.lam_direct && grad_dtype == SX_BF16;
  // 1. the adjoint: the scan in the other direction over g, on a transposed and shifted a step
  bp.p.in_bf16 = dtype == SX_BF16;
  bp.p.out_bf16 = lam_bf16 ? 1 : 0;
  bp.p.reverse = reverse ? 0 : 1;
  bp.p.adjoint = 1;
  bp.p.a = a;
  bp.p.b = g;
  bp.p.out = lam;
  // f32 with grad_a at a's full shape: the pipelined adjoint scan forms grad_a in its replay
  bool folded = false;
  if (dtype == SX_F32 && grad_dtype == SX_F32 && bp.ga_direct && a_numel > 0 && bp.out_numel > 0) {
    bp.p.fold_h = h;
    bp.p.fold_grad_a = grad_a;
    folded = sx::matrix_scan_folds_grad_a(bp.p, ws, bp.scan_ws);
    if (!folded) bp.p.fold_h = bp.p.fold_grad_a = nullptr;
  }
  hipError_t e = sx::launch_matrix_scan(bp.p, ws, bp.scan_ws, s);
  if (e != hipSuccess) return device_status(e, "matrix-scan gradient: adjoint scan launch");
  // 2. grad_a = lam h[prev]^T per step (and grad_b = lam rounded, when that is all grad_b is), unless
  // the scan formed it (f32 gradients: grad_b is lam itself, at the result's shape or summed below)
  const int L = bp.out_rank - 2;
  const int ax = axis < 0 ? axis + L : axis;
  sx::GradAParams gp{};
  gp.steps = bp.out_numel > 0 ? bp.out_numel / (bp.out_shape[L] * bp.out_shape[L + 1])
                              : (bp.a_full_numel > 0 ? bp.a_full_numel / (bp.out_shape[L] * bp.out_shape[L]) : 0);
  gp.T = bp.out_shape[ax];
  gp.inner = 1;
  for (int i = ax + 1; i < L; ++i) gp.inner *= bp.out_shape[i];
  gp.n = int(bp.out_shape[L]);
  gp.m = int(bp.out_shape[L + 1]);
  gp.reverse = reverse ? 1 : 0;
  gp.lam = lam;
  gp.lam_bf16 = lam_bf16 ? 1 : 0;
  gp.h = h;
  gp.grad_a = bp.ga_direct ? grad_a : static_cast<void*>(ws + bp.ga_off);
  const bool b_full = same_shape(b_rank, b_shape, bp.out_rank, bp.out_shape);
  gp.grad_b = (b_full && !bp.lam_direct) ? grad_b : nullptr;
  if (!folded) {
    e = sx::launch_grad_a(gp, dtype == SX_BF16, grad_dtype == SX_BF16 && bp.ga_direct, s);
    if (e != hipSuccess) return device_status(e, "matrix-scan gradient: grad_a launch");
  }
  // 3. sums over broadcast dims
  if (!bp.ga_direct && a_numel > 0) {
    bp.sum_a.src = reinterpret_cast<const float*>(ws + bp.ga_off);
    bp.sum_a.partial = reinterpret_cast<float*>(ws + bp.part_off);
    e = sx::launch_sum_to(bp.sum_a, grad_a, grad_dtype == SX_BF16, s);
    if (e != hipSuccess) return device_status(e, "matrix-scan gradient: grad_a sum launch");
  }
  if (!b_full && b_numel > 0) {
    bp.sum_b.src = static_cast<const float*>(lam);
    bp.sum_b.partial = reinterpret_cast<float*>(ws + bp.part_off);
    e = sx::launch_sum_to(bp.sum_b, grad_b, grad_dtype == SX_BF16, s);
    if (e != hipSuccess) return device_status(e, "matrix-scan gradient: grad_b sum launch");
  }
  return ok();
}

// ------------------------------------------------------------------ element-scan gradient

size_t sx_element_scan_backward_workspace_bytes(sx_body body, int rank, const int64_t* shape, int axis, int state_axis,
                                                int64_t x_width, int64_t s_width) {
  if (!body_ok(body)) return 0;
  EsPlan plan;
  if (plan_element_scan(body, rank, shape, axis, state_axis, nullptr, x_width, nullptr, s_width, nullptr, &plan) !=
      SX_OK)
    return 0;
  const bool vec = state_axis != SX_STATE_SCALAR;
  const int64_t n = vec ? shape[rank - 1] : 1;
  size_t total = 0, part = 0;
  int64_t seq[sx::kMaxRank];
  std::copy(shape, shape + rank, seq);
  for (int64_t w : {x_width, s_width}) {
    if (!vec || w != 1 || n == 1 || body == SX_BODY_NORM_CAP) continue;  // norm-cap sums in its kernels
    total += align_up(size_t(plan.numel) * 4);  // the full-width gradient before its sum over the state
    seq[rank - 1] = 1;
    const sx::SumToParams q = sum_to_plan(rank, shape, rank, seq);
    part = std::max(part, size_t(q.splits * q.targets) * 4);
  }
  // per-lane bounds of the norm-cap gradient's split along the axis
  const size_t bounds = size_t(sx::element_scan_backward_bound_words(body, plan.p)) * 4;
  return total + align_up(part) + align_up(bounds);
}

sx_status sx_element_scan_backward(sx_body body, int rank, const int64_t* shape, int axis, int state_axis, int reverse,
                                   const float* initial, const float* x, int64_t x_width, const int64_t* x_strides,
                                   const float* s, int64_t s_width, const int64_t* s_strides, const float* h,
                                   const float* g, float* grad_initial, float* grad_x, float* grad_s, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (!body_ok(body)) return fail(SX_E_UNSUPPORTED, "element-scan gradient: unknown body %d", enum_code(body));
  EsPlan plan;
  sx_status st = plan_element_scan(body, rank, shape, axis, state_axis, nullptr, x_width, x_strides, s_width,
                                   s_strides, &plan);
  if (st != SX_OK) return st;
  if (plan.numel == 0) return ok();
  const char* what[] = {"initial", "sequence x", "the second sequence", "the forward result h",
                        "the result's gradient g", "grad_initial", "grad_x", "grad_s"};
  const void* ptrs[] = {initial, x, s, h, g, grad_initial, grad_x, grad_s};
  for (int i = 0; i < 8; ++i)
    if (!ptrs[i]) return fail(SX_E_DIM_003, "element-scan gradient: %s is NULL; a tensor was expected", what[i]);
  const bool vec = state_axis != SX_STATE_SCALAR;
  const int64_t n = vec ? shape[rank - 1] : 1;
  const int ax = axis < 0 ? axis + rank : axis;

  // byte spans: inputs, then outputs (initial, h, g and every gradient are contiguous)
  int64_t xshape[sx::kMaxRank], sshape[sx::kMaxRank], ishape[sx::kMaxRank], xs[sx::kMaxRank], ss[sx::kMaxRank];
  int64_t is[sx::kMaxRank], os[sx::kMaxRank];
  for (int i = 0; i < rank; ++i) xshape[i] = sshape[i] = shape[i];
  if (vec) { xshape[rank - 1] = x_width; sshape[rank - 1] = s_width; }
  int64_t inumel = 1;
  for (int i = 0, j = 0; i < rank; ++i)
    if (i != ax) inumel *= (ishape[j++] = shape[i]);
  if (x_strides) std::copy(x_strides, x_strides + rank, xs); else contiguous_strides(rank, xshape, xs);
  if (s_strides) std::copy(s_strides, s_strides + rank, ss); else contiguous_strides(rank, sshape, ss);
  contiguous_strides(rank - 1, ishape, is);
  contiguous_strides(rank, shape, os);
  int64_t xn = 0, sn = 0;
  checked_numel(rank, xshape, &xn);
  checked_numel(rank, sshape, &sn);
  uintptr_t lo[8], hi[8];
  span_bytes(initial, rank - 1, ishape, is, 4, &lo[0], &hi[0]);
  span_bytes(x, rank, xshape, xs, 4, &lo[1], &hi[1]);
  span_bytes(s, rank, sshape, ss, 4, &lo[2], &hi[2]);
  span_bytes(h, rank, shape, os, 4, &lo[3], &hi[3]);
  span_bytes(g, rank, shape, os, 4, &lo[4], &hi[4]);
  lo[5] = reinterpret_cast<uintptr_t>(grad_initial); hi[5] = lo[5] + uintptr_t(inumel) * 4;
  lo[6] = reinterpret_cast<uintptr_t>(grad_x); hi[6] = lo[6] + uintptr_t(xn) * 4;
  lo[7] = reinterpret_cast<uintptr_t>(grad_s); hi[7] = lo[7] + uintptr_t(sn) * 4;
  for (int o = 5; o < 8; ++o)
    for (int i = 0; i < o; ++i)
      if (overlaps(lo[o], hi[o], lo[i], hi[i]))
        return fail(SX_E_ALIAS, "element-scan gradient: %s overlaps %s", what[o], what[i]);

  // width-one sequences under a vector state: norm-cap's kernels sum their gradients over the
  // state; for the other bodies a full-width gradient goes to the workspace and is summed after
  const bool fused = body == SX_BODY_NORM_CAP;
  const bool x_one = vec && x_width == 1 && n > 1, s_one = vec && s_width == 1 && n > 1;
  const bool x_sum = x_one && !fused, s_sum = s_one && !fused;
  const size_t need = sx_element_scan_backward_workspace_bytes(body, rank, shape, axis, state_axis, x_width, s_width);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(SX_E_WORKSPACE, "element-scan gradient: workspace of %zu bytes given, %zu needed", workspace_bytes,
                need);
  if (need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(SX_E_WORKSPACE, "element-scan gradient: workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  const size_t full = align_up(size_t(plan.numel) * 4);
  float* gx_full = x_sum ? reinterpret_cast<float*>(ws) : grad_x;
  float* gs_full = s_sum ? reinterpret_cast<float*>(ws + (x_sum ? full : 0)) : grad_s;
  float* part = reinterpret_cast<float*>(ws + (x_sum ? full : 0) + (s_sum ? full : 0));
  const size_t bounds_bytes = size_t(sx::element_scan_backward_bound_words(body, plan.p)) * 4;
  float* bounds = bounds_bytes > 0 ? reinterpret_cast<float*>(ws + need - align_up(bounds_bytes)) : nullptr;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  sx::EsVjpParams v{};
  v.p = plan.p;
  v.p.reverse = reverse ? 1 : 0;
  v.p.x = x;
  v.p.s = s;
  v.p.init = initial;
  v.p.out = nullptr;
  v.h = h;
  v.g = g;
  v.gx = gx_full;
  v.gs = gs_full;
  v.ginit = grad_initial;
  v.gx_sum = x_one && fused;
  v.gs_sum = s_one && fused;
  v.bounds = bounds;
  hipError_t e = sx::launch_element_scan_backward(body, v, hs);
  if (e != hipSuccess) return device_status(e, "element-scan gradient launch");
  int64_t seq[sx::kMaxRank];
  std::copy(shape, shape + rank, seq);
  seq[rank - 1] = 1;
  for (int which = 0; which < 2; ++which) {
    if (!(which == 0 ? x_sum : s_sum)) continue;
    sx::SumToParams q = sum_to_plan(rank, shape, rank, seq);
    q.src = which == 0 ? gx_full : gs_full;
    q.partial = part;
    e = sx::launch_sum_to(q, which == 0 ? static_cast<void*>(grad_x) : static_cast<void*>(grad_s), false, hs);
    if (e != hipSuccess) return device_status(e, "element-scan gradient: sum over the state launch");
  }
  return ok();
}

// ------------------------------------------------------------------ table-scan

sx_status sx_table_scan(int states, int nsym, const int32_t* table, int rank, const int64_t* shape,
                        const int64_t* strides, const int32_t* symbols, int axis, int32_t start, int32_t* out,
                        void* stream) {
  if (states < 1 || nsym < 1)
    return fail(SX_E_DIM_001, "table-scan: the table is [states symbols] with at least one of each, got [%d %d]",
                states, nsym);
  if (rank > sx::kMaxRank) return fail(SX_E_UNSUPPORTED, "table-scan: rank %d exceeds %d", rank, sx::kMaxRank);
  if (rank < 1 || shape == nullptr) return fail(SX_E_DIM_001, "table-scan: symbols need at least one axis");
  int64_t numel = 0;
  if (!checked_numel(rank, shape, &numel))
    return fail(SX_E_DIM_001, "table-scan: bad symbols shape %s", shape_str(rank, shape).c_str());
  const int ax = axis < 0 ? axis + rank : axis;
  if (ax < 0 || ax >= rank)
    return fail(SX_E_DIM_001, "table-scan: axis %d out of range for symbols %s :i32", axis,
                shape_str(rank, shape).c_str());
  if (start < 0 || start >= states)
    return fail(SX_E_DIM_001, "table-scan: :start %d is not a state of a [%d %d] table", int(start), states, nsym);
  if (numel == 0) return ok();
  if (!table) return fail(SX_E_DIM_003, "table-scan: table is NULL; a tensor was expected");
  if (!symbols) return fail(SX_E_DIM_003, "table-scan: symbols is NULL; a tensor was expected");
  if (!out) return fail(SX_E_DIM_003, "table-scan: out is NULL; a tensor was expected");
  int64_t xs[sx::kMaxRank], os[sx::kMaxRank];
  if (strides) std::copy(strides, strides + rank, xs); else contiguous_strides(rank, shape, xs);
  contiguous_strides(rank, shape, os);
  uintptr_t lo, hi;
  const uintptr_t olo = reinterpret_cast<uintptr_t>(out), ohi = olo + uintptr_t(numel) * 4;
  span_bytes(symbols, rank, shape, xs, 4, &lo, &hi);
  if (overlaps(olo, ohi, lo, hi)) return fail(SX_E_ALIAS, "table-scan: out overlaps symbols");
  const uintptr_t tlo = reinterpret_cast<uintptr_t>(table), thi = tlo + uintptr_t(int64_t(states) * nsym) * 4;
  if (overlaps(olo, ohi, tlo, thi)) return fail(SX_E_ALIAS, "table-scan: out overlaps the table");

  sx::TsParams p{};
  p.T = shape[ax];
  p.t_stride[0] = xs[ax];
  p.t_stride[1] = os[ax];
  int64_t dims[sx::kMaxRank];
  int64_t st[2][sx::kMaxRank];
  int nd = 0;
  for (int i = 0; i < rank; ++i) {
    if (i == ax) continue;
    dims[nd] = shape[i];
    st[0][nd] = xs[i];
    st[1][nd] = os[i];
    ++nd;
  }
  p.seqs = make_index_map<2>(nd, dims, st);
  p.num_seq = numel / p.T;
  p.states = states;
  p.nsym = nsym;
  p.start = start;
  p.table = table;
  p.symbols = symbols;
  p.out = out;
  return device_status(sx::launch_table_scan(p, static_cast<hipStream_t>(stream)), "table-scan launch");
}

// ------------------------------------------------------------------ linear-scan

// a and b broadcast (NumPy: right-aligned, each dim equal or 1; rank 0 is a
// number) to the result shape; the scan runs along `axis` of that shape.
static sx_status plan_linear_scan(int a_rank, const int64_t* a_shape, const int64_t* a_strides, int b_rank,
                                  const int64_t* b_shape, const int64_t* b_strides, int axis, sx::EsParams* p,
                                  int64_t* out_shape, int* out_rank, int64_t* out_numel) {
  if (a_rank > sx::kMaxRank || b_rank > sx::kMaxRank)
    return fail(SX_E_UNSUPPORTED, "linear-scan: rank above %d", sx::kMaxRank);
  if (a_rank < 0 || b_rank < 0 || (a_rank > 0 && !a_shape) || (b_rank > 0 && !b_shape))
    return fail(SX_E_DIM_001, "linear-scan: invalid rank or missing shape");
  int64_t tmp;
  if (!checked_numel(a_rank, a_shape, &tmp) || !checked_numel(b_rank, b_shape, &tmp))
    return fail(SX_E_DIM_001, "linear-scan: negative or oversized dims in a %s, b %s",
                shape_str(a_rank, a_shape).c_str(), shape_str(b_rank, b_shape).c_str());
  const int L = std::max(a_rank, b_rank);
  if (L < 1)
    return fail(SX_E_DIM_001, "linear-scan: a and b are both numbers; there is no axis to scan along");
  int64_t shp[sx::kMaxRank], sa[sx::kMaxRank], sb[sx::kMaxRank];
  int64_t ast[sx::kMaxRank], bst[sx::kMaxRank];
  if (a_strides) std::copy(a_strides, a_strides + a_rank, ast); else contiguous_strides(a_rank, a_shape, ast);
  if (b_strides) std::copy(b_strides, b_strides + b_rank, bst); else contiguous_strides(b_rank, b_shape, bst);
  for (int i = 0; i < L; ++i) {
    const int ia = i - (L - a_rank), ib = i - (L - b_rank);
    const int64_t da = ia >= 0 ? a_shape[ia] : 1, db = ib >= 0 ? b_shape[ib] : 1;
    if (da != db && da != 1 && db != 1)
      return fail(SX_E_DIM_001, "linear-scan: a %s and b %s do not broadcast", shape_str(a_rank, a_shape).c_str(),
                  shape_str(b_rank, b_shape).c_str());
    shp[i] = da == 1 ? db : da;
    sa[i] = (ia >= 0 && da != 1) ? ast[ia] : 0;
    sb[i] = (ib >= 0 && db != 1) ? bst[ib] : 0;
  }
  const int ax = axis < 0 ? axis + L : axis;
  if (ax < 0 || ax >= L)
    return fail(SX_E_DIM_001, "linear-scan: axis %d out of range for shape %s", axis, shape_str(L, shp).c_str());
  int64_t numel = 0;
  if (!checked_numel(L, shp, &numel)) return fail(SX_E_DIM_001, "linear-scan: result too large");
  std::copy(shp, shp + L, out_shape);
  *out_rank = L;
  *out_numel = numel;
  if (!p) return ok();

  int64_t ost[sx::kMaxRank];
  contiguous_strides(L, shp, ost);
  *p = sx::EsParams{};
  p->T = shp[ax];
  p->t_stride[sx::ES_X] = sb[ax];
  p->t_stride[sx::ES_S] = sa[ax];
  p->t_stride[sx::ES_OUT] = ost[ax];
  p->n = 1;
  int64_t dims[sx::kMaxRank];
  int64_t st[4][sx::kMaxRank];
  int nd = 0;
  for (int i = 0; i < L; ++i) {
    if (i == ax) continue;
    dims[nd] = shp[i];
    st[sx::ES_X][nd] = sb[i];
    st[sx::ES_S][nd] = sa[i];
    st[sx::ES_INIT][nd] = 0;
    st[sx::ES_OUT][nd] = ost[i];
    ++nd;
  }
  p->lanes = make_index_map<4>(nd, dims, st);
  p->num_lanes = p->T > 0 ? numel / p->T : 0;
  return ok();
}

int sx_linear_scan_out_shape(int a_rank, const int64_t* a_shape, int b_rank, const int64_t* b_shape,
                             int64_t* out_shape) {
  int64_t shp[sx::kMaxRank];
  int r = 0;
  int64_t numel = 0;
  if (plan_linear_scan(a_rank, a_shape, nullptr, b_rank, b_shape, nullptr, 0, nullptr, shp, &r, &numel) != SX_OK)
    return -1;
  if (out_shape) std::copy(shp, shp + r, out_shape);
  return r;
}

sx_status sx_linear_scan(sx_dtype dtype, int a_rank, const int64_t* a_shape, const int64_t* a_strides, const void* a,
                         int b_rank, const int64_t* b_shape, const int64_t* b_strides, const void* b, int axis,
                         int reverse, sx_dtype out_dtype, void* out, void* stream) {
  if (!dtype_ok(dtype))
    return fail(SX_E_DIM_002, "linear-scan: a and b must be f32 or bf16 (dtype code %d)", enum_code(dtype));
  if (!dtype_ok(out_dtype))
    return fail(SX_E_DIM_002, "linear-scan: out must be f32 or bf16 (dtype code %d)", enum_code(out_dtype));
  sx::EsParams p;
  int64_t shp[sx::kMaxRank];
  int r = 0;
  int64_t numel = 0;
  sx_status st = plan_linear_scan(a_rank, a_shape, a_strides, b_rank, b_shape, b_strides, axis, &p, shp, &r, &numel);
  if (st != SX_OK) return st;
  if (numel == 0) return ok();
  if (!a) return fail(SX_E_DIM_003, "linear-scan: a %s %s is NULL; a tensor was expected",
                      shape_str(a_rank, a_shape).c_str(), dtype_name(dtype));
  if (!b) return fail(SX_E_DIM_003, "linear-scan: b %s %s is NULL; a tensor was expected",
                      shape_str(b_rank, b_shape).c_str(), dtype_name(dtype));
  if (!out) return fail(SX_E_DIM_003, "linear-scan: out is NULL; a tensor was expected");

  const size_t esz = dtype == SX_BF16 ? 2 : 4, osz = out_dtype == SX_BF16 ? 2 : 4;
  int64_t ast[sx::kMaxRank], bst[sx::kMaxRank];
  if (a_strides) std::copy(a_strides, a_strides + a_rank, ast); else contiguous_strides(a_rank, a_shape, ast);
  if (b_strides) std::copy(b_strides, b_strides + b_rank, bst); else contiguous_strides(b_rank, b_shape, bst);
  uintptr_t olo = reinterpret_cast<uintptr_t>(out), ohi = olo + uintptr_t(numel) * osz, lo, hi;
  span_bytes(a, a_rank, a_shape, ast, esz, &lo, &hi);  // numel > 0: neither operand is empty
  if (overlaps(olo, ohi, lo, hi)) return fail(SX_E_ALIAS, "linear-scan: out overlaps a");
  span_bytes(b, b_rank, b_shape, bst, esz, &lo, &hi);
  if (overlaps(olo, ohi, lo, hi)) return fail(SX_E_ALIAS, "linear-scan: out overlaps b");

  p.reverse = reverse ? 1 : 0;
  p.x = static_cast<const float*>(b);  // element type chosen by launch_linear_scan
  p.s = static_cast<const float*>(a);
  p.init = nullptr;
  p.out = static_cast<float*>(out);
  return device_status(sx::launch_linear_scan(p, dtype == SX_BF16, out_dtype == SX_BF16,
                                              static_cast<hipStream_t>(stream)),
                       "linear-scan launch");
}

}  // extern "C"
