/* cgtp.h - Clebsch-Gordan tensor products and the equivariant point
 * convolution built on them, for AMD Instinct MI355X (gfx950).
 *
 * What is computed (citations name the page and its section):
 *  - "E3J: An Efficient and Open-Source Backend for Euclidean Equivariant
 *    Operations on GPU and TPU", sections 3.1.1 (full Clebsch-Gordan tensor
 *    product), 3.1.2 and E.2.2 (message-passing convolution with CSR receiver
 *    aggregation, deterministic, no atomics), E.1 (reverse-mode rules by
 *    transposition), G.1-G.2 (harmonics and CG coefficients by ladder
 *    operators and a triangular eigen-system).
 *  - MolSSI e3nn course, "Curriculum at a glance": lessons 02a (irreps
 *    strings), 02b (spherical harmonics), 03a (CG decomposition, parity rule
 *    p3 = p1 p2), 03b (x (x)_w y, connection modes), 05a (edge vector
 *    r_ij = r_j - r_i), 06a (m_ij = (R(|r_ij|) Y(rhat_ij)) (x)_w h_j).
 *  - e3nn_mlx "Modular v2106 point models": Convolution(edge_src, edge_dst,
 *    radial), sqrt(num_neighbors) normalisation, empty edge lists.
 *
 * Conventions (fixed by this library where the pages leave them open):
 *  - Real spherical harmonics, component-normalised (sum_m Y_lm^2 = 2l+1),
 *    z polar axis, m = -l..l inside a block, l-major blocks: Y_1 = sqrt3 (y,z,x).
 *  - Real CG blocks are orthonormal over (m1, m2) for each m3. Sign per path:
 *    even l1+l2+l3 -> C[0,0,0] > 0; odd -> the first nonzero entry in
 *    lexicographic (m1, m2, m3) order (each m from -l) is positive.
 *  - Connection modes (lesson 03b names uvw and uvu; the formulas are e3nn's).
 *    For path p = (i1, i2, l3), x block i1 of multiplicity u, y block i2 of
 *    multiplicity v, with T_p[z, m3, a, b] = sum_{m1,m2} C_p[m1,m2,m3]
 *    x[z,i1,m1,a] y[z,i2,m2,b]:
 *      "uvu" (channel-wise): out[z, p, m3, a] = sum_b w[(z,) p, a, b] T_p[z,m3,a,b]
 *         (v = 1: out = w[(z,) p, a] C x y, one weight per path and channel)
 *      "uvw" (fully connected): out[z, p, m3, k] = sum_a W[p, a, k] T_p[z,m3,a,0]
 *         with the output multiplicity taken from the first irreps_out entry
 *         of type (l3, p3); y multiplicity 1, shared weights, fp32 or bf16,
 *         multiplicities in multiples of 4.
 *    Paths: every x block i1, every y block i2, every l3 in |l1-l2|..l1+l2
 *    whose (l3, p1*p2) appears in irreps_out; order i1, i2, l3. One output
 *    block per path (not collapsed by degree) unless the plan collapses them.
 *    The convolution, the double backward and cgtp_tp_backward_noalloc take
 *    uvu plans with y multiplicity 1 (others: UNSUPPORTED).
 *  - Row layouts: blocks concatenated in irreps (or path) order; inside a
 *    block [2l+1][mul] (channel index fastest, "ir_mul"). Weights of one row
 *    are [path][mul] concatenated (uvu, v = 1: W = sum_p mul_p elements);
 *    uvu with v > 1: [path][u][v]; uvw: [path][u][w], row-major.
 *
 * Memory and execution:
 *  - Every tensor argument is a DEVICE pointer owned by the caller, of the
 *    plan's dtype unless stated. Indices are int32, sizes int64.
 *  - Plans and graphs are opaque handles owned by the library; they allocate
 *    small device tables (once per device for plans) and are immutable after
 *    creation, so they may be shared between streams and threads.
 *  - `stream` is a hipStream_t (NULL = the default stream). Compute calls are
 *    asynchronous on it; outputs are overwritten, never accumulated into.
 *    A NULL gradient pointer skips that gradient.
 *  - Results are deterministic: every sum has a fixed order, no atomics touch
 *    floating-point data, and repeated calls are bitwise identical.
 *  - Graph capture: a plan's (or linear map's) first compute call on a device
 *    uploads its tables (allocation and a synchronous copy); after it, the
 *    compute calls (tensor product, convolution, harmonics, linear map and
 *    their backward / double backward) only launch kernels on `stream` (fills
 *    by kernel, no memset nodes), so they can be captured in a HIP graph and
 *    replayed. Large calls fork onto library-owned streams and join back by
 *    events, which a capture records as graph dependencies. cgtp_csr_from_coo,
 *    graph create and graph transpose allocate or synchronise and are not
 *    capturable; the destroy calls free device memory, so no plan, graph or
 *    linear map may be destroyed while a capture is open (a hipFree during a
 *    global-mode capture invalidates it).
 *  - Errors are status codes; cgtp_last_error() returns a thread-local
 *    message for the last failure. Nothing else escapes the ABI.
 */
#ifndef CGTP_H
#define CGTP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CGTP_OK = 0,
  CGTP_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad enum, misuse   */
  CGTP_ERR_PARSE = 2,       /* malformed irreps string                         */
  CGTP_ERR_UNSUPPORTED = 3, /* valid request outside what is compiled in       */
  CGTP_ERR_INDEX = 4,       /* graph arrays out of range or not monotone       */
  CGTP_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required      */
  CGTP_ERR_HIP = 6,         /* a HIP runtime call failed                       */
  CGTP_ERR_ALLOC = 7        /* host or device allocation failed                */
} cgtp_status;

typedef enum { CGTP_F32 = 0, CGTP_F64 = 1, CGTP_BF16 = 2 } cgtp_dtype;

/* Weight kinds. SHARED: w is [W]. PER_ROW: w is [rows][W] for the tensor
 * product (rows = B) and [edges][W] in CSR order for the convolution. */
typedef enum { CGTP_W_SHARED = 0, CGTP_W_PER_ROW = 1 } cgtp_wkind;

/* Path selections by parity class (E3J appendix B.1: the Gaunt product covers
 * the symmetric paths, the vector signal product the skew-symmetric ones):
 * SYMMETRIC keeps the paths with l1 + l2 + l3 even, SKEW those with it odd. */
typedef enum { CGTP_PATHS_ALL = 0, CGTP_PATHS_SYMMETRIC = 1, CGTP_PATHS_SKEW = 2 } cgtp_paths;

/* Operations for cgtp_workspace_size. */
typedef enum {
  CGTP_OP_TP_BACKWARD = 1,
  CGTP_OP_CONV_BACKWARD = 2,
  CGTP_OP_TP_DOUBLE_BACKWARD = 3,
  CGTP_OP_CONV_DOUBLE_BACKWARD = 4,
  CGTP_OP_CONV_FORWARD = 5
} cgtp_op;

typedef struct cgtp_plan_s* cgtp_plan;
typedef struct cgtp_graph_s* cgtp_graph;
typedef struct cgtp_linear_s* cgtp_linear;

/* Largest degree compiled into the kernels for x, y and output blocks. */
#define CGTP_LMAX 4

const char* cgtp_status_string(cgtp_status s);
/* Message of the last failing call on this thread ("" if none). */
const char* cgtp_last_error(void);

/* ---------------------------------------------------------------- planning */

/* Build a tensor-product plan (host work only; device tables are uploaded on
 * first use on each device). Irreps strings follow the course's lesson 02a:
 * terms "MxLp" joined by '+', M defaults to 1, p in {e, o}; whitespace is
 * ignored. Path enumeration follows lesson 03a (triangle rule, p3 = p1 p2).
 * CG values are built with the ladder-operator construction of E3J appendix
 * G.2: the highest-weight vector of each l3 solves a triangular system, lower
 * m3 follow by repeated lowering; then the real-basis change and sign rule.
 *   mode   : "uvu" or "uvw" (see Connection modes above).
 *   dtype  : storage type of every float tensor (bf16 computes in fp32).
 *   wkind  : see cgtp_wkind.
 * Errors: PARSE (bad string), UNSUPPORTED (another mode, uvw outside its
 * limits above, uvu with y multiplicity > 1 and collapsed outputs, any
 * l > CGTP_LMAX, no path at all), INVALID_ARG (null pointers). */
cgtp_status cgtp_plan_create(const char* irreps_x, const char* irreps_y, const char* irreps_out,
                             const char* mode, cgtp_dtype dtype, cgtp_wkind wkind, cgtp_plan* out);
/* cgtp_plan_create with a path selection and, if collapse != 0, outputs
 * collapsed by degree (E3J appendix B.1 and B.3: the isomorphic copies of each
 * output irrep are summed). Collapsed layout: one output block [2l3+1][mul] per
 * (l3, p3) that some path reaches, in the order of irreps_out (first
 * occurrence), where every path of that (l3, p3) adds its output; mul is the
 * multiplicity of the x blocks feeding it. The tensor product and the
 * convolution accept collapsed plans (the collapsed convolution forward adds
 * the paths into the output in a fixed order: x block, slot chunk, path; with
 * bf16 storage each addition rounds to bf16).
 * Errors: as cgtp_plan_create; INVALID_ARG for a bad selection; UNSUPPORTED
 * when the x blocks feeding one collapsed output differ in multiplicity or no
 * path is selected. */
cgtp_status cgtp_plan_create_ex(const char* irreps_x, const char* irreps_y, const char* irreps_out,
                                const char* mode, cgtp_dtype dtype, cgtp_wkind wkind, cgtp_paths select,
                                int collapse, cgtp_plan* out);
cgtp_status cgtp_plan_destroy(cgtp_plan plan);

/* Output blocks of a plan into a HOST table [num_outputs][4] of
 * (l3, p3, mul, offset within the output row): one per path in path order, or
 * one per collapsed (l3, p3). host_table may be NULL to query the count only;
 * num_outputs may be NULL. */
cgtp_status cgtp_plan_outputs(cgtp_plan plan, int64_t* num_outputs, int32_t* host_table);

/* Sizes in elements per row: dim_x, dim_y, dim_out, the path count and W
 * (weights per row or per edge). Any output pointer may be NULL. */
cgtp_status cgtp_plan_query(cgtp_plan plan, int64_t* dim_x, int64_t* dim_y, int64_t* dim_out,
                            int64_t* num_paths, int64_t* w_numel);

/* HOST table [num_paths][6] of (i1, i2, l1, l2, l3, p3) in path order. */
cgtp_status cgtp_plan_paths(cgtp_plan plan, int32_t* host_table);

/* Dense real CG block of one path into HOST memory, fp64,
 * [2l1+1][2l2+1][2l3+1] row-major. */
cgtp_status cgtp_plan_cg(cgtp_plan plan, int32_t path, double* host_dense);

/* ---------------------------------------------------------- tensor product */

/* out[B][dim_out] = x[B][dim_x] (x)_w y[B][dim_y] (formula above).
 * w is [W] (SHARED) or [B][W] (PER_ROW). B = 0 is a no-op.
 * Errors: INVALID_ARG (null pointer with B > 0, B < 0). */
cgtp_status cgtp_tp_forward(cgtp_plan plan, int64_t B, const void* x, const void* y, const void* w,
                            void* out, void* stream);

/* Reverse mode by transposition (E3J appendix E.1), with g = grad_out:
 *   grad_x[z,i1,m1,u] = sum_p w sum_{m2,m3} C y[m2] g[m3,u]
 *   grad_y[z,i2,m2]   = sum_p sum_u w sum_{m1,m3} C x[m1,u] g[m3,u]
 *   grad_w[(z,)p,u]   = sum_{(z),m1,m2,m3} C x[m1,u] y[m2] g[m3,u]
 * A SHARED plan sums grad_w over rows in a fixed two-stage order; that needs
 * a workspace of cgtp_workspace_size(plan, NULL, B, CGTP_OP_TP_BACKWARD)
 * bytes (0 for PER_ROW). B = 0 writes a zero grad_w for SHARED plans and is
 * otherwise a no-op. Errors: WORKSPACE if ws is NULL or too small. */
cgtp_status cgtp_tp_backward(cgtp_plan plan, int64_t B, const void* x, const void* y, const void* w,
                             const void* grad_out, void* grad_x, void* grad_y, void* grad_w,
                             void* ws, size_t ws_bytes, void* stream);

/* Bytes of the device scratch array behind cgtp_tp_backward_noalloc (one
 * copy per device, held until the process ends). */
#define CGTP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* cgtp_tp_backward without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The
 * shared-weight grad_w partials live in a file-scope device array of
 * CGTP_NOALLOC_SCRATCH_BYTES bytes on each device (its address is looked up
 * on the first call on a device); rows run in passes of whole 256-row chunks,
 * so the summation order and the results are bitwise those of
 * cgtp_tp_backward. Every call on one device shares that array: calls that
 * overlap on a device (different streams, threads) race, so callers serialise
 * them. PER_ROW plans need no scratch. Errors: WORKSPACE when
 * ceil(B / 256) + min(B, 256) rows of W partials (accumulation type) exceed
 * the array; otherwise as cgtp_tp_backward. */
cgtp_status cgtp_tp_backward_noalloc(cgtp_plan plan, int64_t B, const void* x, const void* y, const void* w,
                                     const void* grad_out, void* grad_x, void* grad_y, void* grad_w,
                                     void* stream);

/* Double backward: the reverse mode of cgtp_tp_backward (needed to train on
 * quantities that are themselves gradients, such as forces). For cotangents
 * (gg_x, gg_y, gg_w) of (grad_x, grad_y, grad_w) it writes the cotangents of
 * (x, y, w, grad_out). The backward's outputs are each linear in the other
 * three tensors (E3J appendix E.1), so with S = <gg_x, grad_x> + <gg_y,
 * grad_y> + <gg_w, grad_w>:
 *   out_grad_out = TP(gg_x, y, w) + TP(x, gg_y, w) + TP(x, y, gg_w)
 *   out_x = back(x, gg_y, w, g).grad_x + back(x, y, gg_w, g).grad_x
 *   out_y = back(gg_x, y, w, g).grad_y + back(x, y, gg_w, g).grad_y
 *   out_w = back(gg_x, y, w, g).grad_w + back(x, gg_y, w, g).grad_w
 * summed in that order. Shapes are those of x, y, w, grad_out (gg_w and out_w
 * are [W] for SHARED plans). A NULL cotangent counts as zero; a NULL output is
 * not computed; outputs no cotangent reaches are written as zeros. Needs
 * cgtp_workspace_size(plan, NULL, B, CGTP_OP_TP_DOUBLE_BACKWARD) bytes of
 * workspace (partial results). B = 0 writes a zero out_w for SHARED plans and
 * is otherwise a no-op. Errors: WORKSPACE, INVALID_ARG (null inputs). */
cgtp_status cgtp_tp_double_backward(cgtp_plan plan, int64_t B, const void* x, const void* y, const void* w,
                                    const void* grad_out, const void* gg_x, const void* gg_y, const void* gg_w,
                                    void* out_x, void* out_y, void* out_w, void* out_grad_out, void* ws,
                                    size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------ graphs */

/* COO -> CSR by destination (E3J E.2.2: the receiver-ordered aggregation
 * streams each destination's edges as one contiguous segment, so one owner
 * sums a receiver without atomics). Sort key (dst, src), ties in input order (so
 * the result is the stable lexicographic sort of the pairs). Outputs (device,
 * caller-owned): row_ptr[N+1], src_sorted[E], perm[E] with perm[k] = input
 * index of CSR edge k. Allocates and frees temporary device memory and
 * synchronises the stream once (to read back a validation flag).
 * Errors: INDEX if any src/dst is outside [0, N). */
cgtp_status cgtp_csr_from_coo(int64_t N, int64_t E, const int32_t* src, const int32_t* dst,
                              int32_t* row_ptr, int32_t* src_sorted, int32_t* perm, void* stream);

/* Wrap a CSR-by-destination graph (E3J E.2.2 for the receiver segments, E.3
 * for the backward's source-side gradient locality; device arrays,
 * caller-owned, must outlive the handle): validates row_ptr (row_ptr[0] = 0, non-decreasing,
 * row_ptr[N] = E) and src (in [0, N)), and builds the source-ordered
 * transpose used by the backward pass (owned by the handle; edges grouped by
 * source, in CSR-position order). It also copies the two arrays to the host
 * once to build a receiver schedule (breadth-first order over the graph) that
 * the convolution kernels walk so that receivers sharing sources run close
 * together; results do not depend on it (each receiver is still summed by one
 * owner in CSR order). Synchronises the stream.
 * Errors: INDEX on invalid arrays, ALLOC if device memory runs out. */
cgtp_status cgtp_graph_create(int64_t N, int64_t E, const int32_t* row_ptr, const int32_t* src,
                              void* stream, cgtp_graph* out);
/* cgtp_graph_create with a padding node (E3J 3.1.2 and 3.2: fixed-shape
 * callers pad the edge list with edges into a shared padding node, whose one
 * CSR segment then holds all of them). pad_node in [0, N), or -1 for none.
 * The edges whose destination is pad_node are padding edges: they are
 * skipped, so out[pad_node] = 0, their grad_sh and grad_w rows are zero, and
 * they add nothing to grad_x; they are left out of the transpose. Other edges
 * (also those whose source is pad_node) are ordinary.
 * Errors: as cgtp_graph_create; INDEX for pad_node outside [-1, N). */
cgtp_status cgtp_graph_create_ex(int64_t N, int64_t E, const int32_t* row_ptr, const int32_t* src,
                                 int32_t pad_node, void* stream, cgtp_graph* out);
cgtp_status cgtp_graph_destroy(cgtp_graph graph);

/* Copy the handle's transpose into caller device buffers col_ptr[N+1] and
 * eid[col_ptr[N]] (eid[k] = CSR position of the k-th source-ordered edge;
 * col_ptr[N] = E minus the padding edges). */
cgtp_status cgtp_graph_transpose(cgtp_graph graph, int32_t* col_ptr, int32_t* eid, void* stream);

/* ------------------------------------------------------------- convolution */

/* out[n] = scale * sum_{e: dst(e)=n} TP(x[src(e)], sh[e], w[e]) over CSR
 * segment n, summed in CSR order (course lesson 06a; E3J 3.1.2, E.2.2).
 *   x [N][dim_x], sh [E][dim_y] and w [E][W] (edge tensors in CSR order),
 *   out [N][dim_out]. The plan must be PER_ROW (one weight row per edge).
 * E = 0 writes zeros; nodes without incoming edges get zero rows. Edge
 * messages never reach memory. Errors: UNSUPPORTED for a SHARED plan. */
cgtp_status cgtp_conv_forward(cgtp_plan plan, cgtp_graph graph, const void* x, const void* sh,
                              const void* w, double scale, void* out, void* stream);

/* cgtp_conv_forward with a workspace (same sum, E3J B.3 for collapsed
 * outputs). With collapsed outputs the x blocks' contributions to one output
 * block are added one x block at a time (one path at a time where the
 * general kernel runs: channels not a multiple of 4, misaligned pointers, y
 * degrees repeated); in bf16 storage cgtp_conv_forward rounds that running
 * sum to bf16 after every step, while with a workspace
 * of cgtp_workspace_size(plan, graph, 0, CGTP_OP_CONV_FORWARD) bytes
 * (N * dim_out fp32 values; 0 for other plans) it stays fp32 and is rounded
 * once. ws may be NULL (then as cgtp_conv_forward); a non-NULL ws must be
 * 16-byte aligned. Errors: WORKSPACE if ws is non-NULL and smaller than that
 * size, INVALID_ARG if misaligned. */
cgtp_status cgtp_conv_forward_ws(cgtp_plan plan, cgtp_graph graph, const void* x, const void* sh,
                                 const void* w, double scale, void* out, void* ws, size_t ws_bytes,
                                 void* stream);

/* Reverse mode of cgtp_conv_forward, with g_e = scale * grad_out[dst(e)]:
 *   grad_sh[e] = d/dsh of <g_e, TP(x[src(e)], sh[e], w[e])>   [E][dim_y]
 *   grad_w[e]  = d/dw  of the same                             [E][W]
 *   grad_x[n]  = sum_{e: src(e)=n} d/dx of the same            [N][dim_x]
 * grad_x is summed over the transpose in fixed order from per-edge partials
 * kept in the workspace (cgtp_workspace_size(plan, graph, 0,
 * CGTP_OP_CONV_BACKWARD) bytes). That size also holds one grad_sh copy per
 * x block in the accumulation type, which lets the x blocks' launches run
 * side by side; grad_sh is then their sum in block order, the order in which
 * the launches accumulate it in place when the workspace only holds the
 * partials (E * dim_x accumulation-type values, required whenever grad_x is
 * requested; without grad_x the workspace may be NULL). Errors: WORKSPACE if
 * grad_x is requested and the workspace cannot hold the partials. */
cgtp_status cgtp_conv_backward(cgtp_plan plan, cgtp_graph graph, const void* x, const void* sh,
                               const void* w, double scale, const void* grad_out, void* grad_x,
                               void* grad_sh, void* grad_w, void* ws, size_t ws_bytes, void* stream);

/* Double backward of the convolution, the reverse mode of
 * cgtp_conv_backward: the same sums as cgtp_tp_double_backward with the
 * convolution's forward and backward (scale included), for cotangents gg_x
 * [N][dim_x], gg_sh [E][dim_y], gg_w [E][W] (CSR order) of (grad_x, grad_sh,
 * grad_w); outputs out_x [N][dim_x], out_sh [E][dim_y], out_w [E][W],
 * out_grad_out [N][dim_out]. NULL cotangents count as zero, NULL outputs are
 * skipped. Workspace: cgtp_workspace_size(plan, graph, 0,
 * CGTP_OP_CONV_DOUBLE_BACKWARD) bytes. */
cgtp_status cgtp_conv_double_backward(cgtp_plan plan, cgtp_graph graph, const void* x, const void* sh,
                                      const void* w, double scale, const void* grad_out, const void* gg_x,
                                      const void* gg_sh, const void* gg_w, void* out_x, void* out_sh, void* out_w,
                                      void* out_grad_out, void* ws, size_t ws_bytes, void* stream);

/* Convolution with the radial network's last layer joined to it: the per-edge
 * weights are w[e, k] = sum_j h[e, j] W2[j, k], formed on the matrix cores
 * inside the kernel and never written to memory (E3J E.4 and F.1: fuse
 * message formation and avoid materialising edge-wise intermediates; xnn "Run
 * Models on Fused GPU Kernels", "What to expect from fast implementations":
 * radial networks above a million edges are recomputed rather than stored).
 * Otherwise as cgtp_conv_forward.
 *   h  [E][hidden] hidden activations of the radial network (CSR order)
 *   W2 [hidden][W] its last layer, row-major (no bias)
 * fp32 plans only; y degrees distinct, outputs not collapsed, x multiplicities
 * in {16, 32, 64, 128, 256}, hidden a multiple of 4 up to 1024; otherwise
 * UNSUPPORTED, as also when a slot chunk's two weight tiles and partial sums
 * exceed the device's LDS (possible at multiplicity 256). Deterministic; the
 * sum over a receiver's edges runs in another order than cgtp_conv_forward's
 * (within rounding). */
cgtp_status cgtp_conv_forward_radial(cgtp_plan plan, cgtp_graph graph, const void* x, const void* sh,
                                     const void* h, int64_t hidden, const void* W2, double scale, void* out,
                                     void* stream);

/* Reverse mode of cgtp_conv_forward_radial: grad_x and grad_sh as in
 * cgtp_conv_backward, grad_h [E][hidden] = grad_w W2^T and grad_W2
 * [hidden][W] = h^T grad_w (summed over edges in a fixed order), where grad_w
 * is the convolution's weight cotangent. Composed through the workspace
 * (w, grad_w, the convolution's and the linear map's partials) of
 * cgtp_conv_radial_workspace_size bytes. NULL gradients are skipped. */
cgtp_status cgtp_conv_backward_radial(cgtp_plan plan, cgtp_graph graph, const void* x, const void* sh,
                                      const void* h, int64_t hidden, const void* W2, double scale,
                                      const void* grad_out, void* grad_x, void* grad_sh, void* grad_h,
                                      void* grad_W2, void* ws, size_t ws_bytes, void* stream);
cgtp_status cgtp_conv_radial_workspace_size(cgtp_plan plan, cgtp_graph graph, int64_t hidden, size_t* bytes);

/* Workspace bytes for op (graph may be NULL for the tensor product, B is
 * ignored for the convolution). */
cgtp_status cgtp_workspace_size(cgtp_plan plan, cgtp_graph graph, int64_t B, int op, size_t* bytes);

/* --------------------------------------------------- spherical harmonics */

/* sh[n][(lmax+1)^2] = Y_l(vec/|vec|), l = 0..lmax, conventions above (course
 * lesson 02b; E3J G.1). vec [n][3]. The zero vector gives Y_0 = 1, rest 0.
 * lmax <= CGTP_LMAX. */
cgtp_status cgtp_sh_forward(int lmax, cgtp_dtype dtype, int64_t n, const void* vec, void* sh,
                            void* stream);

/* grad_vec[n][3] = d/dvec of sum(grad_sh * Y(vec/|vec|)); zero for a zero vec. */
cgtp_status cgtp_sh_backward(int lmax, cgtp_dtype dtype, int64_t n, const void* vec,
                             const void* grad_sh, void* grad_vec, void* stream);

/* ------------------------------------------------- equivariant linear map */

/* Channel mixing within irrep types (E3J appendix A.3 lists linear mixing
 * among the core operations; course lesson 03b on the weights of learnable
 * layers). Every (input block i, output block o) with the same l and parity
 * is a path p with a weight matrix W_p [u_i][v_o] (row-major), paths ordered
 * input-major; for every row z and component m of the block:
 *   out[z, o, m, v] = sum over paths p = (i, o) of sum_u x[z, i, m, u] W_p[u, v]
 * No normalisation factor. Output blocks that no input reaches are zero.
 * Rows of x [B][dim_in] and out [B][dim_out] are ir_mul blocks as above; w is
 * one shared weight vector [w_numel] = the W_p concatenated in path order.
 * A fully connected ("uvw") tensor product with y of multiplicity 1 is this
 * map applied to the path outputs of cgtp_tp_forward with unit weights.
 * Runs on the matrix cores (fp32 MFMA: fp32 products and sums; bf16 storage
 * is widened exactly to fp32). dtype: CGTP_F32 or CGTP_BF16 (CGTP_F64 ->
 * UNSUPPORTED). Errors: PARSE, UNSUPPORTED, INVALID_ARG. */
cgtp_status cgtp_linear_create(const char* irreps_in, const char* irreps_out, cgtp_dtype dtype,
                               cgtp_linear* out);
cgtp_status cgtp_linear_destroy(cgtp_linear lin);
/* Row sizes, path count and weight count (any pointer may be NULL). */
cgtp_status cgtp_linear_query(cgtp_linear lin, int64_t* dim_in, int64_t* dim_out, int64_t* num_paths,
                              int64_t* w_numel);
/* Host table [num_paths][5]: i, o, l, u_i, v_o. */
cgtp_status cgtp_linear_paths(cgtp_linear lin, int32_t* host_table);
/* out [B][dim_out] from x [B][dim_in] and w [w_numel]. B = 0 is a no-op. */
cgtp_status cgtp_linear_forward(cgtp_linear lin, int64_t B, const void* x, const void* w, void* out,
                                void* stream);
/* Reverse mode: grad_x [B][dim_in] = sum_p g_o W_p^T; grad_w [w_numel] = sum
 * over rows and m of x_i^T g_o per path, summed over row chunks in a fixed
 * order from partials kept in ws (cgtp_linear_workspace_size bytes; needed
 * only with grad_w). NULL grad pointers are skipped. Errors: WORKSPACE. */
cgtp_status cgtp_linear_backward(cgtp_linear lin, int64_t B, const void* x, const void* w,
                                 const void* grad_out, void* grad_x, void* grad_w, void* ws, size_t ws_bytes,
                                 void* stream);
cgtp_status cgtp_linear_workspace_size(cgtp_linear lin, int64_t B, size_t* bytes);

#ifdef __cplusplus
}
#endif

#endif /* CGTP_H */
