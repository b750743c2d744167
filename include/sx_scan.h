/*
 * sx_scan.h: C ABI of the MI355X (gfx950) scan library, libsx_scan.so.
 *
 * The scans of the SexpGPU documentation pages:
 *
 *   element-scan  "Nonlinear element scans": a nonlinear recurrence along
 *                 one axis, one independent lane per index of the other axes,
 *                 with one of three fixed bodies (tanh-affine, norm-capped
 *                 vector state, max-plus), forward or reverse.
 *   element-scan gradient  the chain rule through those bodies, trips last
 *                 to first.
 *   matrix-scan   "Tensor operations", Operations table (matrix-scan row) and
 *                 the "matrix-scan" section: h[t] = a[t] @ h[t-1] + b[t] from
 *                 h = 0, n <= 16, computed in f32, with :axis, :reverse and
 *                 broadcast leading dims.
 *   matrix-scan gradient  the same section and "gradient": the adjoint scan
 *                 in the other direction on a's transposes, then grad_a.
 *   table-scan    "Tensor operations", the "table-scan" section: a
 *                 deterministic automaton over int32 symbols.
 *   linear-scan   the same section: matrix-scan over one-by-one matrices,
 *                 a and b broadcast to one shape (cumsum: a = 1).
 *
 * Conventions shared by every entry point:
 *
 *  - Pointers to tensor data are DEVICE pointers on the device that is
 *    current on the calling thread. Shapes and strides are HOST arrays of
 *    int64_t, read during the call only. Strides count elements (not bytes),
 *    may be zero (a broadcast dimension) and may be passed as NULL to mean
 *    row-major contiguous. Layouts are row-major, as PyTorch's default.
 *  - The caller owns every buffer. The library keeps no pointer after it
 *    returns and allocates no device memory. Where a workspace is needed,
 *    the caller passes one of at least the queried size. Element-scan
 *    workspaces may hold anything on entry. A matrix-scan workspace (also
 *    those of its gradient and :projective) must be zero-filled once before
 *    its first use; every call then leaves it ready for the next one, on any
 *    later shape, with nothing to clear in between (no extra kernel per
 *    call). Keep it for matrix-scan calls only: other writes to its first
 *    256 bytes invalidate it until it is zero-filled again.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream)
 *    and the call returns without waiting. Results follow stream order.
 *    Concurrent calls that share one workspace race.
 *  - Every argument is checked on the host before anything is enqueued. On
 *    an error status nothing is launched and `out` is untouched;
 *    sx_last_error() then returns a message that names the operands with
 *    their shapes and dtypes, as the pages' error notes do.
 *  - Status codes mirror the pages' error table ("Tensor operations",
 *    Errors): E-DIM-001 for a shape mismatch, E-DIM-002 for mismatched or
 *    unsupported dtypes, E-DIM-003 for a missing tensor.
 */
#ifndef SX_SCAN_H
#define SX_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Largest tensor rank the library accepts. */
#define SX_MAX_RANK 8
/* Largest matrix size n of matrix-scan ("n at most 16") and largest state
 * width of a vector-state element scan ("vectors of 1 to 16 values"). */
#define SX_MAX_N 16
/* `state_axis` value that selects a scalar state (no :state-axis). */
#define SX_STATE_SCALAR INT32_MIN

typedef enum sx_status {
  SX_OK = 0,
  SX_E_DIM_001 = 1,     /* shapes do not fit, axis out of range, n > 16, empty element-scan axis */
  SX_E_DIM_002 = 2,     /* dtypes differ, or a dtype the operand does not allow */
  SX_E_DIM_003 = 3,     /* a tensor was expected: a required pointer is NULL */
  SX_E_UNSUPPORTED = 4, /* well-formed but not provided: rank > 8, strided matrix dims */
  SX_E_ALIAS = 5,       /* `out` overlaps an input */
  SX_E_WORKSPACE = 6,   /* workspace NULL or smaller than the queried size */
  SX_E_DEVICE = 7       /* a HIP call failed; sx_last_error() carries hipGetErrorString */
} sx_status;

typedef enum sx_dtype { SX_F32 = 0, SX_BF16 = 1 } sx_dtype;

/* The three element-scan bodies ("Nonlinear element scans", introduction),
 * each taking (state h, sequence x, sequence s) in the page's order:
 *   SX_BODY_TANH_AFFINE  h' = tanh(x + s * h)              s = decay
 *   SX_BODY_NORM_CAP     y = s * h + x; h' = y / max(1, |y|)  s = decay, |y| over the state vector
 *   SX_BODY_MAX_PLUS     h' = max(h - s, x)                s = cost
 * NORM_CAP reduces over the state vector and so needs a vector state; the
 * other two act on each state component on its own and accept either. */
typedef enum sx_body {
  SX_BODY_TANH_AFFINE = 0,
  SX_BODY_NORM_CAP = 1,
  SX_BODY_MAX_PLUS = 2
} sx_body;

/*
 * sx_element_scan: "Nonlinear element scans", introduction and "Arguments
 * and body".
 *
 * For every lane (every index outside `axis`, and outside the state axis for
 * a vector state) the state starts at `initial` and each trip applies the
 * body: forward h[t] = f(h[t-1], x[t], s[t]) from h[-1] = initial, reverse
 * h[t] = f(h[t+1], x[t], s[t]) from h[T] = initial. out[t] holds the state
 * after trip t. Computation is f32.
 *
 *  body          one of sx_body.
 *  rank, shape   the OUTPUT shape, rank 1..SX_MAX_RANK: the sequences' shape,
 *                whose last axis, for a vector state, is the state width n.
 *  axis          the sequence axis; negative counts from the end. Its length
 *                must be at least one (E-DIM-001 otherwise).
 *  state_axis    SX_STATE_SCALAR for a scalar state; -1 or rank-1 for a state
 *                vector along the last axis (1 <= n <= 16, axis != last);
 *                anything else is E-DIM-001.
 *  reverse       0 forward, nonzero reverse.
 *  initial       f32, shape = `shape` without `axis`; `initial_strides` has
 *                rank-1 entries (or NULL for contiguous).
 *  x, s          f32 sequences. Scalar state: shape = `shape`, widths
 *                ignored. Vector state: shape = `shape` with the last axis
 *                replaced by the sequence's own width, `x_width`/`s_width`,
 *                each 1 (broadcast over the state, a per-trip gate) or n.
 *                Strides have `rank` entries; a width-1 axis's stride is
 *                ignored.
 *  out           f32, contiguous, shape `shape`. Must not overlap an input.
 *  workspace     may be NULL when sx_element_scan_workspace_bytes() is 0.
 *  stream        hipStream_t.
 *
 * A shape with zero lanes returns SX_OK without launching.
 */
sx_status sx_element_scan(sx_body body, int rank, const int64_t* shape, int axis, int state_axis,
                          int reverse, const float* initial, const int64_t* initial_strides,
                          const float* x, int64_t x_width, const int64_t* x_strides, const float* s,
                          int64_t s_width, const int64_t* s_strides, float* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Workspace bytes sx_element_scan needs for these arguments (0 when none);
 * returns 0 as well for arguments sx_element_scan would reject. */
size_t sx_element_scan_workspace_bytes(sx_body body, int rank, const int64_t* shape, int axis,
                                       int state_axis);

/*
 * sx_element_scan_backward: gradients of an element scan. The chain rule
 * through the bodies of "Nonlinear element scans" (introduction), with each
 * gradient in its tensor's shape ("Tensor operations", "gradient" section).
 *
 * Given the forward call's arguments, its result h and the gradient g of a
 * loss with respect to h, writes the loss's gradients with respect to
 * initial, x and the second sequence s. The trips are taken last to first in
 * scan order; with lam the adjoint of the state a trip produced (g there plus
 * what the trip after passed back) and hp the state it started from:
 *   tanh-affine  dz = lam (1 - h^2); grad_x = dz; grad_s = dz hp; to hp: s dz
 *   norm-cap     y = s hp + x; when |y| > 1, u = y / |y| and
 *                dy = (lam - u (u . lam)) / |y|, else dy = lam;
 *                grad_x = dy; grad_s = dy hp; to hp: s dy
 *   max-plus     x won (x >= hp - c; ties to x): grad_x = lam, grad_c = 0,
 *                to hp 0; else grad_x = 0, grad_c = -lam, to hp lam
 * grad_initial is what the first trip passes back. A width-one sequence under
 * a vector state gets the sum over the state of its broadcast gradient. The
 * branch decisions use f32 values computed as the forward pass does.
 *
 *  body .. s_strides  as for sx_element_scan, except that initial must be
 *                contiguous (no strides argument).
 *  h, g          the forward result and its gradient: contiguous, `shape`.
 *  grad_initial, grad_x, grad_s
 *                contiguous, the shapes of initial, x and s. Must not overlap
 *                any input or each other (SX_E_ALIAS).
 *  workspace     at least sx_element_scan_backward_workspace_bytes() bytes
 *                (nonzero for width-one sequences under a vector state with
 *                tanh-affine or max-plus, and for norm-cap with fewer than
 *                8192 state vectors and at least 32 trips, which splits the
 *                axis), 256-byte aligned; may be NULL when that is 0. The
 *                call overwrites it.
 *
 * Errors as sx_element_scan; E-DIM-003 for any NULL tensor.
 */
sx_status sx_element_scan_backward(sx_body body, int rank, const int64_t* shape, int axis, int state_axis,
                                   int reverse, const float* initial, const float* x, int64_t x_width,
                                   const int64_t* x_strides, const float* s, int64_t s_width,
                                   const int64_t* s_strides, const float* h, const float* g, float* grad_initial,
                                   float* grad_x, float* grad_s, void* workspace, size_t workspace_bytes,
                                   void* stream);

/* Workspace bytes sx_element_scan_backward needs (0 when none or for invalid arguments). */
size_t sx_element_scan_backward_workspace_bytes(sx_body body, int rank, const int64_t* shape, int axis,
                                                int state_axis, int64_t x_width, int64_t s_width);

/*
 * sx_matrix_scan: "Tensor operations", Operations table (matrix-scan row)
 * and the "matrix-scan" section.
 *
 * a is [lead_a..., n, n] and b [lead_b..., n, m], n <= 16, one float dtype.
 * The leading dims broadcast (NumPy: right-aligned, each equal or 1) to one
 * shape `lead`, and `axis` indexes them (-1: the last leading dim, next to
 * the matrix dims). For every other leading index the n-by-m state runs
 *   forward  h[t] = a[t] @ h[t-1] + b[t]  from h[-1] = 0  (h[0] = b[0]),
 *   reverse  h[t] = a[t] @ h[t+1] + b[t]  from h[T] = 0  (h[T-1] = b[T-1]),
 * and out[t] = h[t]. Computation is f32 for f32 and bf16 operands alike:
 * bf16 widens to f32 exactly, and with bf16 a each product a[t] @ h is
 * formed exactly (h split into three bf16 parts that sum to it) and summed in
 * f32, as with f32 operands.
 *
 *  dtype         SX_F32 or SX_BF16, shared by a and b.
 *  a_*, b_*      rank (>= 2), shape, strides (NULL = contiguous) and data.
 *                The two matrix dims must be row-major contiguous (strides
 *                [n, 1] and [m, 1] where those dims exceed 1); leading dims may
 *                have any stride, including 0. Otherwise SX_E_UNSUPPORTED.
 *  axis          the scan axis among the broadcast leading dims.
 *  reverse       0 forward, nonzero reverse.
 *  projective    nonzero: the :projective variant of the same section,
 *                meant for chains of projective maps whose plain product
 *                would leave f32's range. Each step multiplies a running
 *                product P (starting at the identity) by that step's a,
 *                P = a[t] @ P, then rescales: with m the entry of P of
 *                largest magnitude (m = 1 for a zero P), both P and the new
 *                state are divided by m, h[t] = (a[t] @ h[prev] + b[t]) / m.
 *                When b vanishes after its first step, every state then
 *                equals the plain scan's state times a positive number of
 *                its own. With n = 16, on the shapes the chunked scan
 *                takes, it runs in parallel in the workspace (passes that
 *                compute every step's factor, then the scan); on other
 *                shapes it runs serially in time.
 *  out_dtype     SX_F32 or SX_BF16. The result is rounded to bf16 to nearest
 *                even on store when SX_BF16.
 *  out           contiguous, shape lead + [n, m] (see sx_matrix_scan_out_shape).
 *  workspace     at least sx_matrix_scan_workspace_bytes() bytes, 256-byte
 *                aligned, zero-filled before its first use (see above); may
 *                be NULL when that size is 0.
 *
 * Time-parallel kernels hand each chunk's entering state on through the
 * workspace; every wait for an earlier chunk is bounded, and one that reaches
 * its bound is recorded in the workspace, not returned here (the call is
 * asynchronous): sx_matrix_scan_workspace_status reports it.
 *
 * An axis of length 0 (or m = 0) returns SX_OK with nothing to write.
 */
sx_status sx_matrix_scan(sx_dtype dtype, int a_rank, const int64_t* a_shape, const int64_t* a_strides,
                         const void* a, int b_rank, const int64_t* b_shape, const int64_t* b_strides,
                         const void* b, int axis, int reverse, int projective, sx_dtype out_dtype,
                         void* out, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device memory sx_matrix_scan_noalloc keeps, per device, for its
 * look-back state. */
#define SX_MATRIX_SCAN_SCRATCH_BYTES (16u << 20)

/*
 * sx_matrix_scan_noalloc: sx_matrix_scan (the same arguments, the same result)
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. It takes no
 * workspace: the look-back state lives in a fixed array of
 * SX_MATRIX_SCAN_SCRATCH_BYTES bytes in device memory, one per device the
 * library runs on, kept until the process ends. It calls no allocation
 * routine. The first call on a device sets the array up (its address, and a
 * synchronous zero-fill): make that first call outside graph capture.
 *
 * Shapes whose look-back state is larger than the array (sx_matrix_scan_workspace_bytes
 * above SX_MATRIX_SCAN_SCRATCH_BYTES: about 5000 units of 96 steps of one
 * 16-column tile, e.g. 32 x 8192 and 16 x 16384 fit) return SX_E_WORKSPACE
 * before anything is launched. Every call on a device shares that device's
 * array and leaves it ready for the next call: calls that overlap on one
 * device (concurrent streams, host threads) race. A look-back give-up is
 * recorded in the array, which sx_matrix_scan_workspace_status cannot reach.
 */
sx_status sx_matrix_scan_noalloc(sx_dtype dtype, int a_rank, const int64_t* a_shape, const int64_t* a_strides,
                                 const void* a, int b_rank, const int64_t* b_shape, const int64_t* b_strides,
                                 const void* b, int axis, int reverse, int projective, sx_dtype out_dtype, void* out,
                                 void* stream);

/* Workspace bytes sx_matrix_scan needs for these shapes (0 for invalid ones),
 * with or without :projective (the size covers both). */
size_t sx_matrix_scan_workspace_bytes(int a_rank, const int64_t* a_shape, int b_rank,
                                      const int64_t* b_shape, int axis);

/* Waits for `stream`, then reads and clears the status a matrix-scan
 * workspace carries ("Tensor operations", Errors: every failure is a reported
 * code). SX_OK when every look-back of the calls on this workspace since the
 * last check completed; SX_E_DEVICE when one gave up waiting for an earlier
 * chunk's published state (its results are then not valid), with the reason
 * in sx_last_error(). SX_E_DIM_003 for a NULL workspace, SX_E_WORKSPACE for
 * one of fewer than 256 bytes. Synchronous: not for use under graph capture. */
sx_status sx_matrix_scan_workspace_status(void* workspace, size_t workspace_bytes, void* stream);

/* Bound on the polls a matrix-scan look-back makes before it gives up and
 * records it (see sx_matrix_scan_workspace_status); 0 restores the default
 * (2^22 polls, about a tenth of a second). Process-wide, for calls launched
 * after it. A diagnostic: a small bound forces give-ups, so that the report
 * path can be tested with every kernel still running to its end. */
void sx_set_lookback_spin_limit(uint32_t limit);

/* Writes the matrix-scan result shape to out_shape (room for SX_MAX_RANK + 2
 * entries) and returns its rank, or -1 for shapes that do not fit. */
int sx_matrix_scan_out_shape(int a_rank, const int64_t* a_shape, int b_rank, const int64_t* b_shape,
                             int64_t* out_shape);

/*
 * sx_matrix_scan_backward: "Tensor operations", the "matrix-scan" section (its
 * gradient is a scan in the opposite direction over transposed a) and the
 * "gradient" section (a gradient has its operand's shape and dtype).
 *
 * Given the forward call's a and b shapes, its result h and the gradient g of
 * a loss with respect to h, writes the gradients of that loss with respect to
 * a and b. With lam[t] the adjoint of h[t] and s / p the steps after / before
 * t in the forward scan order,
 *   lam[t]    = g[t] + a[s]^T @ lam[s]   (no second term at the last step)
 *   grad_b[t] = lam[t]
 *   grad_a[t] = lam[t] @ h[p]^T        (zero at the first step, whose a
 *                                      multiplies the zero state)
 * summed over the dims along which a (or b) was broadcast. lam is computed in
 * f32 by the matrix-scan kernels in the other direction. With bf16 gradients
 * and b of the result's shape, lam is stored rounded into grad_b and grad_a
 * is formed from that rounded lam (a relative change of at most 2^-9 per
 * element of lam, inside bf16's own rounding of the result).
 *
 *  dtype         SX_F32 or SX_BF16: the dtype of a, h and g alike.
 *  a_*           a as passed to sx_matrix_scan (strides as there).
 *  b_rank/shape  b's shape (b's values are not needed).
 *  h             the forward result: contiguous, the shape
 *                sx_matrix_scan_out_shape gives, dtype `dtype`.
 *  g_strides, g  gradient of the result: that shape, dtype `dtype`; strides
 *                NULL for contiguous; its two matrix dims row-major
 *                contiguous (else SX_E_UNSUPPORTED).
 *  axis, reverse those of the forward call.
 *  grad_dtype    SX_F32 or SX_BF16 for grad_a and grad_b (rounded to nearest
 *                even on store).
 *  grad_a/grad_b contiguous, the shapes of a and b. Must not overlap any
 *                input or each other (SX_E_ALIAS).
 *  workspace     at least sx_matrix_scan_backward_workspace_bytes() bytes,
 *                256-byte aligned; may be NULL when that is 0.
 *
 * Errors as sx_matrix_scan (E-DIM-001 shapes, E-DIM-002 dtypes, E-DIM-003 a
 * NULL tensor that has elements). Empty operands return SX_OK; gradients of
 * operands that have elements are written even when the result is empty
 * (they are zero then).
 */
sx_status sx_matrix_scan_backward(sx_dtype dtype, int a_rank, const int64_t* a_shape, const int64_t* a_strides,
                                  const void* a, int b_rank, const int64_t* b_shape, const void* h,
                                  const int64_t* g_strides, const void* g, int axis, int reverse, sx_dtype grad_dtype,
                                  void* grad_a, void* grad_b, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes sx_matrix_scan_backward needs (0 for invalid shapes). */
size_t sx_matrix_scan_backward_workspace_bytes(int a_rank, const int64_t* a_shape, int b_rank,
                                               const int64_t* b_shape, int axis, sx_dtype grad_dtype);

/*
 * sx_linear_scan: "Tensor operations", the "matrix-scan" section, on the
 * prelude's linear-scan: matrix-scan over one-by-one matrices, with a and b
 * (tensors or plain numbers) broadcast together. cumsum is linear-scan with
 * a = 1 (a rank-0 a holding 1).
 *
 * For every index outside `axis` of the broadcast shape the scalar state runs
 *   forward  h[t] = a[t] * h[t-1] + b[t]  from h[-1] = 0  (h[0] = b[0]),
 *   reverse  h[t] = a[t] * h[t+1] + b[t]  from h[T] = 0  (h[T-1] = b[T-1]),
 * and out[t] = h[t]. a[0] (forward) or a[T-1] (reverse) multiplies the zero
 * state, so any finite value there gives the same result (the kernels do form
 * that product: an infinite or NaN entry there gives NaN). Computation is f32
 * for f32 and bf16 operands alike.
 *
 *  dtype         SX_F32 or SX_BF16, shared by a and b (else E-DIM-002).
 *  a_*, b_*      rank (0..SX_MAX_RANK; 0 is a number, its shape may be
 *                NULL), shape, strides (NULL = contiguous; any value,
 *                including 0 and negative) and data. The shapes broadcast
 *                NumPy-style (right-aligned, each dim equal or 1) to the
 *                result shape, of rank max(a_rank, b_rank) >= 1; otherwise
 *                E-DIM-001.
 *  axis          the scan axis of the result shape; negative counts from the
 *                end; out of range is E-DIM-001.
 *  reverse       0 forward, nonzero reverse.
 *  out_dtype     SX_F32 or SX_BF16 (rounded to nearest even on store).
 *  out           contiguous, the broadcast shape (see sx_linear_scan_out_shape);
 *                must not overlap a or b (SX_E_ALIAS).
 *
 * No workspace. A result with no elements returns SX_OK without launching.
 */
sx_status sx_linear_scan(sx_dtype dtype, int a_rank, const int64_t* a_shape, const int64_t* a_strides,
                         const void* a, int b_rank, const int64_t* b_shape, const int64_t* b_strides,
                         const void* b, int axis, int reverse, sx_dtype out_dtype, void* out, void* stream);

/* Writes the broadcast shape of a and b to out_shape (room for SX_MAX_RANK
 * entries) and returns its rank, or -1 for shapes that do not fit. */
int sx_linear_scan_out_shape(int a_rank, const int64_t* a_shape, int b_rank, const int64_t* b_shape,
                             int64_t* out_shape);

/*
 * sx_table_scan: "Tensor operations", the "table-scan" section.
 *
 * Runs a deterministic automaton along `axis` of `symbols`: each symbol
 * moves the state to table[previous, symbol], starting at `start`; out holds every
 * state, in symbols' shape. A symbol outside [0, nsym) is clamped into that
 * range, and so is any table value the run lands on outside [0, states), as the
 * pages' GPU backend does (their CPU backend refuses them instead). States
 * have no gradient.
 *
 *  states, nsym  the table's shape [states, nsym], each at least 1 (E-DIM-001).
 *  table         int32, row-major contiguous [states, nsym], device memory.
 *  rank, shape, strides, symbols
 *                int32 symbols, rank 1..SX_MAX_RANK; strides in elements (NULL
 *                for contiguous).
 *  axis          the scan axis; negative counts from the end (the pages'
 *                default is -1). Out of range: E-DIM-001.
 *  start         the first state; outside [0, states): E-DIM-001.
 *  out           int32, contiguous, symbols' shape; must not overlap symbols
 *                or the table (SX_E_ALIAS).
 *
 * No workspace. Symbols with no elements return SX_OK without launching.
 */
sx_status sx_table_scan(int states, int nsym, const int32_t* table, int rank, const int64_t* shape,
                        const int64_t* strides, const int32_t* symbols, int axis, int32_t start, int32_t* out,
                        void* stream);

/* "E-DIM-001" etc. for a status; "OK" for SX_OK. Static storage. */
const char* sx_status_name(sx_status status);

/* Message of the last failed call on this thread (thread-local storage,
 * valid until the next call on the thread); "" after a success. */
const char* sx_last_error(void);

/* Library version string, e.g. "sx_scan 0.1 gfx950". Static storage. */
const char* sx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SX_SCAN_H */
