/*
 * e2v2.h -- C ABI of an MI355X (gfx950) implementation of one E2Former-V2-style
 * node-centric equivariant neighbour-attention layer forward.
 *
 * The layer (E2Former-V2 explainer, "E2Former-V2: breaking the computational
 * bottleneck of equivariant graph neural networks", sections 2-3):
 *   1. neighbour list within a cutoff (section 3.2: one target per work item,
 *      padded neighbours masked; section 5.2: verify the list);
 *   2. per-node projections q = h^0 W_Q, k = h^0 W_K, v^l = h^l W_V[l];
 *   3. source pre-coupling h'_j = v_j (x) Y(r_j) computed with EAAS
 *      (section 2.1 alignment rotation, section 2.2 sparse m re-index with the
 *      even/odd sign rule, section 2.3 Proposition 4.3 exactness);
 *   4. streaming aggregation m_i = sum_j alpha_ij h'_j with an online softmax
 *      over q_i . k_j / sqrt(d) plus a Gaussian-RBF x cosine-envelope distance
 *      bias (section 3.1, section 3.2 Algorithm 1; the bias follows the
 *      FlashSchNet page, section 2.1);
 *   5. target coupling hhat_i = m_i (x) Y(r_i) (section 3.1);
 *   6. output projection out^l = hhat^l W_O[l].
 *
 * Conventions shared by every entry point
 *   - Features are [n][(lmax+1)^2][C], channels fastest; component index of
 *     (l, m) is l*l + l + m, m = -l..l.  Real spherical harmonics of the unit
 *     direction, "component" normalised (sum_m Y_lm^2 = 2l+1, Y_00 = 1), real
 *     form of the complex Condon-Shortley harmonics: Y_1 = sqrt(3) (y, z, x).
 *   - Tensor-product paths (l_in, l_filter, l_out), all l <= lmax with
 *     |l_in - l_f| <= l_out <= l_in + l_f, ordered l_out, then l_in, then l_f
 *     (e2v2_path_table).  Path weights are per path and per channel.
 *   - Position vectors are taken from the coordinate origin.  A zero position
 *     has no direction: its encoding is Y_0 = 1, Y_{l>0} = 0.
 *   - Head h owns channels [h*C/H, (h+1)*C/H) in every component.
 *   - Pointers named "device" are device memory owned by the caller; the
 *     library allocates no device memory and keeps no per-call state.  Every
 *     device pointer must be 16-byte aligned.
 *   - Every call enqueues work on `stream` and returns without waiting, except
 *     where a function says it synchronises.
 *   - Errors are returned as status codes; nothing is enqueued when a call
 *     returns an argument error.  e2v2_last_error() gives a thread-local
 *     message for the last failing call on the calling thread.
 */
#ifndef E2V2_H
#define E2V2_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    E2V2_OK = 0,
    E2V2_ERR_ARG = 1,          /* invalid argument, detected before enqueueing anything        */
    E2V2_ERR_CAPACITY = 2,     /* neighbour storage too small; *nnz_host holds the need          */
    E2V2_ERR_UNSUPPORTED = 3,  /* valid but not implemented shape (e.g. channels per head != 8) */
    E2V2_ERR_HIP = 4           /* a HIP runtime call failed; see e2v2_last_error()               */
} e2v2_status;

typedef enum { E2V2_FP32 = 0, E2V2_BF16 = 1 } e2v2_dtype;

/* One attention layer.  Supported: lmax 0..3; heads 4, 8 or 16 with exactly
 * 8 channels per head (channels = 8 * heads); n_rbf 2..64; cutoff > 0. */
typedef struct {
    int32_t lmax;
    int32_t channels;
    int32_t heads;
    int32_t n_rbf;
    float cutoff;        /* Angstrom; also the RBF range and the envelope's zero */
    int32_t storage;     /* e2v2_dtype of h, W_Q, W_K, W_V and W_O.  The intermediates
                            q and k are fp32; h' and the aggregated message m are
                            fp32 (fp32 storage) or, for bf16 storage, fp16 under one
                            power-of-two scale per node; arithmetic is fp32
                            throughout */
} e2v2_layer_desc;

/* Layer weights (device pointers).
 *   w_q, w_k : [C][C] storage dtype, (in, out) row-major: q = h^0 @ w_q
 *   w_v, w_o : [lmax+1][C][C] storage dtype, one (in, out) matrix per l
 *   w_rbf    : [n_rbf][heads] fp32; bias_h(d) = f_c(d) sum_k w_rbf[k][h] phi_k(d),
 *              phi_k(d) = exp(-(d - mu_k)^2 / (2 D^2)), mu_k = k*cutoff/(n_rbf-1),
 *              D = cutoff/(n_rbf-1), f_c(d) = (cos(pi d / cutoff) + 1) / 2
 *   w_src, w_tgt : [n_paths(lmax)][C] fp32 per-path, per-channel weights of the
 *              source and target tensor products */
typedef struct {
    const void *w_q, *w_k, *w_v, *w_o;
    const float *w_rbf;
    const float *w_src, *w_tgt;
} e2v2_weights;

/* Optional copies of the layer's intermediates (device pointers, 16-byte
 * aligned; any may be NULL) and optional stage timing.  Intended for validation
 * and measurement; production callers pass NULL taps.  For bf16 storage steps 2
 * and 3 run as one kernel (v is projected and coupled in registers), so the
 * events after step 2 and after step 3 are recorded back to back, and steps 5
 * and 6 run as one kernel on whole nodes. */
typedef struct {
    float *q;        /* [n][C] fp32                                         */
    float *k;        /* [n][C] fp32 */
    float *v;        /* [n][(lmax+1)^2][C] fp32                             */
    float *hprime;   /* [n][(lmax+1)^2][C] fp32: h' as the streaming kernel reads it
                        (for bf16 storage: its 16-bit form times the node's scale) */
    float *m;        /* [n][(lmax+1)^2][C] fp32 aggregated message (step 4); for
                        bf16 storage its fp16 form times the node's scale */
    float *hhat;     /* [n][(lmax+1)^2][C] fp32 target-coupled message (step 5) */
    hipEvent_t *events;  /* host array of 5 caller-created events or NULL: recorded on
                            `stream` before step 2, after step 2, after step 3, after
                            the streaming kernel (steps 4-5; step 4 only for bf16
                            storage, whose step 5 runs with step 6) and after step 6 */
} e2v2_taps;

/* ------------------------------------------------------------------------
 * Neighbour list (cell list).  E2Former-V2 explainer section 3.2 (neighbour
 * cap with masked padding), section 5.2 (verify the list); Tessera article
 * (neighbour topology reused between rebuilds).
 *
 * For target i the neighbour set is every j != i with d2 < cutoff^2, where
 * dx = (double)pos[j].x - (double)pos[i].x (likewise y, z) and
 * d2 = (dx*dx + dy*dy) + dz*dz, each operation rounded separately in fp64.
 *   max_neighbors == 0 : CSR.  nbr_start[i] is the exclusive prefix sum of
 *                        nbr_len; nbr_idx holds nnz entries.  Synchronises
 *                        `stream` once to read nnz; *nnz_host receives it.
 *                        If nnz > capacity, returns E2V2_ERR_CAPACITY with
 *                        *nnz_host = nnz and leaves the outputs undefined.
 *   max_neighbors == K : row i lives at nbr_idx[i*K .. i*K+K); the K nearest
 *                        by (d2, j) are kept when more qualify; entries past
 *                        nbr_len[i] are -1.  nbr_start[i] = i*K.  capacity must
 *                        be >= n*K.  Does not synchronise unless nnz_host is
 *                        non-NULL (then it waits and stores sum(nbr_len)).
 * A row lists its neighbours in the builder's scan order (the cell rows the
 * cutoff sphere reaches, by z then y; the cells of a row in index order; atoms
 * ascending within a cell), or, when more than K qualify, the K nearest in
 * (d2, j) order; a row longer than 1,024 candidates comes by ascending j.  The
 * rows and their order are deterministic (the same for the same positions).
 *   pos          device [n][3] fp32 (the positions' fp32 values are the truth)
 *   nbr_start    device [n] int32;  nbr_len device [n] int32
 *   nbr_idx      device [capacity] int32
 *   nnz_host     host, may be NULL for K > 0; required for K == 0
 *   order        device [n] int32 or NULL: receives the targets' Hilbert-curve
 *                processing order, the permutation e2v2_target_order returns
 *                (computed in the builder's own launches, from the same
 *                positions); pass it as target_order to the attention calls.
 *   workspace    device scratch of at least
 *                e2v2_build_neighbors_workspace_bytes(n, max_neighbors) bytes
 * Limits: 0 <= n < 2^31 - 1, cutoff > 0 finite, 0 <= K <= 4096, total entries
 * < 2^31.  Non-finite coordinates never fault; such atoms get no neighbours. */
e2v2_status e2v2_build_neighbors(const float *pos, int32_t n, float cutoff, int32_t max_neighbors,
                                 int32_t *nbr_start, int32_t *nbr_len, int32_t *nbr_idx,
                                 int64_t capacity, int64_t *nnz_host, int32_t *order,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);
size_t e2v2_build_neighbors_workspace_bytes(int32_t n, int32_t max_neighbors);

/* ------------------------------------------------------------------------
 * Processing order of the targets along a Hilbert curve, to pass as target_order
 * to the attention calls.  Targets are independent (FlashSchNet page, section
 * 2.3: one program writes each target's output, in any order); the order only
 * decides which targets run together: the four-target streaming kernel reads the
 * union of four consecutive targets' lists once, and the chip's L2 slices each
 * work on one run of the order.  A Hilbert curve keeps every run compact.
 * The curve: cubic cells of side 2^k over the bounding box of the finite
 * coordinates (lo = its low corner), k the largest integer with
 * 8 n 2^(3k) <= V, V the product of the box's sides in fp64 (each side at least
 * 2^-10 of the longest), raised while the longest side spans 1023 cells or more;
 * cell coordinates q = floor((pos - lo) * 2^-k) in fp32, clamped to 0..1023 (NaN
 * to 0); each atom's key is the 30-bit Hilbert index of (qx, qy, qz) (J.
 * Skilling's transposed form, 10 bits per axis, its bits read from the top
 * level down, first axis first); atoms sorted by key, ties by atom id.  With no extent every key is 0
 * (the order is 0..n-1).  Deterministic.
 *   pos        device [n][3] fp32, 4-byte aligned
 *   order      device [n] int32, 4-byte aligned: receives the permutation
 *   workspace  device scratch of at least e2v2_target_order_workspace_bytes(n)
 *              bytes
 * Runs on `stream` and does not synchronise.  It needs no neighbour list, so it
 * can run beside e2v2_build_neighbors on a second stream.  Its radix sort clears
 * counters with hipMemsetAsync: not for stream capture.
 * Errors: E2V2_ERR_ARG for n < 0 or n = 2^31 - 1, NULL or misaligned pointers, a
 * workspace below the size; E2V2_ERR_HIP for a failed launch.  n = 0 does
 * nothing. */
e2v2_status e2v2_target_order(const float *pos, int32_t n, int32_t *order, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);
size_t e2v2_target_order_workspace_bytes(int32_t n);

/* ------------------------------------------------------------------------
 * EAAS tensor product of features with the encoding of each node's position
 * (explainer section 2.1 pseudocode eaas_forward(h, r_vec); section 2.2 sparse
 * re-index; section 2.3 Proposition 4.3):
 *   y^{l_o}[n][m_o][c] = sum_p path_w[p][c] (x_n (x) Y(r_n))^{(l_i,l_f,l_o)}_{m_o,c}
 * equal to the dense Clebsch-Gordan product, evaluated as: rotate x into the
 * frame whose z axis is r_n, re-index m with the even/odd rule (only the
 * m_f = 0 encoding entry is non-zero there), rotate back.
 *   pos     device [n][3] fp32;  x device [n][(lmax+1)^2][C] in x_dtype
 *   path_w  device [n_paths(lmax)][C] fp32
 *   y       device [n][(lmax+1)^2][C] in y_dtype (fp32, or bf16 rounded to nearest even)
 * Limits: lmax 0..3, 1 <= channels <= 256, channels % 8 == 0. */
e2v2_status e2v2_eaas_couple(const float *pos, const void *x, e2v2_dtype x_dtype, const float *path_w,
                             int32_t n, int32_t lmax, int32_t channels,
                             void *y, e2v2_dtype y_dtype, hipStream_t stream);

/* ------------------------------------------------------------------------
 * One attention layer forward (steps 2-6 above) over a given neighbour list
 * (the format e2v2_build_neighbors writes: target i reads
 * nbr_idx[nbr_start[i] .. nbr_start[i] + nbr_len[i])).  Entries outside
 * [0, n) are skipped, so -1 padding inside a row is harmless.  A target with
 * no neighbours gets m = 0 and therefore out = 0.
 *   target_order  device [n] int32 or NULL: the order in which targets are
 *        processed (a permutation of 0..n-1, e.g. the order written by
 *        e2v2_build_neighbors).  With fp32 storage results do not depend
 *        on it.  With bf16 storage it decides which two targets share a wave
 *        and so the summation order, which can move the fp16-stored message by
 *        a rounding step; a given order always gives bit-identical results.  A
 *        spatially coherent order lets neighbouring targets share cached rows.
 *        Entries outside [0, n) are skipped.
 *   h    device [n][(lmax+1)^2][C] storage dtype
 *   out  device [n][(lmax+1)^2][C] fp32
 *   workspace  device scratch of at least e2v2_attn_workspace_bytes(desc, n)
 * No N x K tensor is formed: the streaming kernel reads each neighbour's key
 * and coupled value at most once per target (for bf16 storage with lmax <= 2,
 * once for two consecutive targets of target_order) and accumulates on chip. */
e2v2_status e2v2_attn_forward(const e2v2_layer_desc *desc, const float *pos, const void *h,
                              const e2v2_weights *w, const int32_t *nbr_start, const int32_t *nbr_len,
                              const int32_t *nbr_idx, const int32_t *target_order, int32_t n, float *out,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): e2v2_attn_forward with
 * no workspace argument.  The workspace is a 64 MiB array inside the library,
 * one per device, held until the process ends; its device address is looked up
 * once per device on the first call with that device current.  The call makes
 * no hipMalloc, hipFree or other allocating call.  Arguments, results and errors
 * as for e2v2_attn_forward, plus E2V2_ERR_CAPACITY (nothing enqueued) when
 * e2v2_attn_workspace_bytes(desc, n) exceeds 64 MiB: about 11,000 atoms at
 * l_max = 2, C = 128 with bf16 storage, about 4,000 with fp32 storage.  All
 * calls on one device share its array: calls that overlap on one device (two
 * streams, two host threads) race and must be ordered by the caller.  Nothing
 * in the array needs to start at zero. */
e2v2_status e2v2_attn_forward_noalloc(const e2v2_layer_desc *desc, const float *pos, const void *h,
                                      const e2v2_weights *w, const int32_t *nbr_start, const int32_t *nbr_len,
                                      const int32_t *nbr_idx, const int32_t *target_order, int32_t n, float *out,
                                      hipStream_t stream);

/* Same as e2v2_attn_forward, also copying intermediates into `taps` (host
 * pointer to a struct of device pointers; NULL behaves like e2v2_attn_forward). */
e2v2_status e2v2_attn_forward_taps(const e2v2_layer_desc *desc, const float *pos, const void *h,
                                   const e2v2_weights *w, const int32_t *nbr_start, const int32_t *nbr_len,
                                   const int32_t *nbr_idx, const int32_t *target_order, int32_t n, float *out,
                                   void *workspace, size_t workspace_bytes, const e2v2_taps *taps,
                                   hipStream_t stream);
size_t e2v2_attn_workspace_bytes(const e2v2_layer_desc *desc, int32_t n);

/* The same forward in two calls that share the workspace, so that the part that
 * needs no neighbour list can overlap e2v2_build_neighbors on another stream.
 * e2v2_attn_prepare runs steps 2-3 (projections q, k, v; source pre-coupling of
 * v by EAAS: E2Former-V2 explainer sections 2.3 and 3.1) and leaves q, k, h', the
 * per-node frames and the packed weights in the workspace.  e2v2_attn_aggregate
 * runs steps 4-6 (streaming attention, target coupling, output projection:
 * sections 3.1-3.2) on that workspace and writes out.  Arguments mean what they
 * mean for e2v2_attn_forward.  The two calls must use the same desc, weights, n
 * and workspace; aggregate must be ordered after prepare (same stream, or an
 * event), and a prepare must not start while an earlier aggregate on the same
 * workspace still runs.  The result equals e2v2_attn_forward's bit for bit.
 * Errors as for e2v2_attn_forward; prepare checks pos, h and the projection
 * and source weights, aggregate the neighbour list, out, w_o, w_rbf, w_tgt. */
e2v2_status e2v2_attn_prepare(const e2v2_layer_desc *desc, const float *pos, const void *h,
                              const e2v2_weights *w, int32_t n, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);
e2v2_status e2v2_attn_aggregate(const e2v2_layer_desc *desc, const e2v2_weights *w, const int32_t *nbr_start,
                                const int32_t *nbr_len, const int32_t *nbr_idx, const int32_t *target_order,
                                int32_t n, float *out, void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* ------------------------------------------------------------------------
 * Gradient of the layer with respect to its input features and positions.
 *
 * For L = sum(grad_out * out), with out the layer output of e2v2_attn_forward
 * for the same arguments, writes grad_h = dL/dh.  Weights and the neighbour
 * list are held fixed.  The chain runs the forward's steps 2-3 again
 * (projections, source coupling: E2Former-V2 explainer sections 2.3 and 3.1),
 * then the adjoint of each step in reverse: the output projection (h-hat^l
 * gradient = grad_out^l W_O[l]^T), the target coupling (the EAAS map with each
 * sparse coefficient taken from output to input: D P^T D^T), the softmax
 * attention of section 3.1 (per-head logit gradient alpha (dalpha - sum alpha
 * dalpha); the distance bias of the FlashSchNet page, section 2.1, has no h
 * dependence), the source coupling, and the input projections.
 *
 * grad_pos (optional, NULL to skip) receives dL/dpos [n][3] fp32 with the
 * neighbour list held fixed: the terms through each node's encoding Y(r_i / |r_i|)
 * in both couplings (dL/dY from the dense real Clebsch-Gordan form, which the EAAS
 * form equals, explainer section 2.3, times the tangent gradient of the
 * harmonics) and through every pair distance in the bias.  A node at the origin
 * has no direction; its encoding is held constant there.  For a potential
 * energy E = L the forces are -grad_pos.
 *
 * pos fp32 [n][3]; h [n][(lmax+1)^2][C] in the storage dtype; grad_out fp32
 * [n][(lmax+1)^2][C]; grad_h fp32 [n][(lmax+1)^2][C] (written whole).  With bf16
 * storage the result is the gradient of the same layer function in fp32
 * arithmetic at the bf16 values of h, W_Q, W_K, W_V and W_O (widened exactly in
 * the workspace): the fp16 storage of h' and m inside the forward kernels is
 * rounding of one evaluation, not part of the function, and is not
 * differentiated (forces at the benched storage: the inputs and weights are the
 * bf16 ones, the arithmetic is fp32).
 * The neighbour list has the layout of e2v2_attn_forward (CSR or K-capped with
 * -1 padding; any list, symmetric or not).  Each source's gradient is gathered
 * over the targets that read it, so no result is written by atomics (FlashSchNet
 * page, section 2.3: the backward works by source).  symmetric = 0: the call
 * builds the transposed list in the workspace (the targets that read each
 * source, in increasing order; about 0.26 ms at 1.6 M entries).  symmetric = 1:
 * the caller guarantees that j is in row i exactly as often as i is in row j,
 * with valid entries only, and the list serves as its own transpose (true of
 * every uncapped list of e2v2_build_neighbors and e2v2_filter_neighbors, whose
 * fp64 predicate is symmetric in i and j; not of capped lists in general).  The
 * results of the two modes on a symmetric list with rows sorted by index are
 * identical (the builder's rows come in its scan order, so on them the two
 * differ only by the order of summation).  max_entries:
 * an upper bound on the list's entries (the length of nbr_idx is one); entries
 * beyond it are dropped from the source side, so a smaller value gives a wrong
 * gradient (never an out-of-bounds access).
 * target_order (optional, a permutation of 0..n-1) only changes the order in
 * which nodes are processed.  Workspace: e2v2_layer_backward_workspace_bytes
 * (n, max_entries).  A wrong symmetric = 1 gives a wrong gradient, never an
 * out-of-bounds access.  reuse_forward = 1 skips the recomputation of q, k, v, h'
 * and the frames: the caller guarantees that e2v2_attn_forward (or
 * e2v2_attn_prepare) last ran with the same desc, pos, h, weights and n on this
 * same workspace pointer (its layout is the first e2v2_attn_workspace_bytes of
 * the gradient's workspace), as a training step does when it keeps the forward's
 * intermediates; fp32 storage only (a bf16 forward keeps h' in fp16).
 * All device pointers 16-byte aligned; asynchronous on `stream`.  Errors:
 * E2V2_ERR_ARG (NULL or misaligned pointer, small workspace, n < 0, max_entries
 * outside 0 .. 2^31 - 2),
 * E2V2_ERR_UNSUPPORTED (head shape, reuse_forward with bf16 storage),
 * E2V2_ERR_HIP (launch failure). */
size_t e2v2_layer_backward_workspace_bytes(const e2v2_layer_desc *desc, int32_t n, int64_t max_entries);
e2v2_status e2v2_layer_backward(const e2v2_layer_desc *desc, const float *pos, const void *h,
                                const e2v2_weights *w, const int32_t *nbr_start, const int32_t *nbr_len,
                                const int32_t *nbr_idx, int64_t max_entries, int32_t symmetric,
                                int32_t reuse_forward, const int32_t *target_order, int32_t n,
                                const float *grad_out, float *grad_h, float *grad_pos, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Lists reused between rebuilds (Tessera article, neighbour reuse: the topology
 * is kept for several steps while distances come from the latest coordinates;
 * the short-range lists are taken from the long-range one).
 *
 * e2v2_filter_neighbors keeps, in each row i of a list in the layout of
 * e2v2_build_neighbors, the entries j in [0, n) with d2 < cutoff^2 -- the fp64
 * predicate of e2v2_build_neighbors, evaluated at `pos` -- in their order.
 * out_len[i] receives the count; out_idx[nbr_start[i] .. + out_len[i]) the
 * entries, and the rest of the input row's range, up to nbr_len[i], is set to -1.
 * Output rows start where input rows start (out_idx has the input's layout), and
 * out_len / out_idx may be nbr_len / nbr_idx (in place).  Filtering the K-nearest
 * list at a larger cutoff gives the list at `cutoff` exactly unless some row has
 * more than K atoms within `cutoff`.
 *   pos device [n][3] fp32; nbr_start, nbr_len, out_len device [n] int32;
 *   nbr_idx, out_idx device int32 covering every row's range
 * Limits: 0 <= n < 2^31 - 1, cutoff > 0 finite. */
e2v2_status e2v2_filter_neighbors(const float *pos, int32_t n, float cutoff, const int32_t *nbr_start,
                                  const int32_t *nbr_len, const int32_t *nbr_idx, int32_t *out_len,
                                  int32_t *out_idx, hipStream_t stream);

/* Largest squared displacement max_i (dx*dx + dy*dy) + dz*dz with dx = pos - ref
 * per coordinate, in fp64 (dx is exact for fp32 inputs, each further operation
 * rounded); a non-finite value counts as +inf, and n = 0 gives 0.
 *   pos, ref device [n][3] fp32;  max_d2 device, one double */
e2v2_status e2v2_max_displacement2(const float *pos, const float *ref, int32_t n, double *max_d2,
                                   hipStream_t stream);

/* ------------------------------------------------------------------------
 * A stack of layers over a moving system (Tessera article: three short-range
 * layers with a 5 A cutoff and one long-range layer with 8 A; the neighbour graph
 * rebuilt every 10 steps, or earlier, by a global synchronisation, when an atom
 * has moved more than 0.25 A).  One call is one model step at positions `pos`:
 *   1. Rebuild decision: on the first call (steps_since_rebuild < 0), when
 *      steps_since_rebuild >= rebuild_every, or when e2v2_max_displacement2(pos,
 *      positions at the last rebuild) > (double)max_displacement^2 (or is not
 *      finite).  The displacement test reads one value back and synchronises
 *      `stream`.
 *   2. On a rebuild: the K-nearest list at the largest layer cutoff
 *      (e2v2_build_neighbors), then for every smaller cutoff the entries of that
 *      list within it (e2v2_filter_neighbors), both at `pos`, which becomes the
 *      reference.
 *   3. Layers l = 0 .. n_layers - 1 in order: e2v2_attn_forward with descs[l],
 *      weights[l] and the list of descs[l].cutoff at the current positions, on h
 *      (l = 0) or the previous layer's output: fp32 storage takes it as written,
 *      bf16 storage rounds it to bf16 (nearest, ties to even).  The last layer
 *      writes out.
 * Between rebuilds the lists are reused as they are: an atom listed at the last
 * rebuild stays a neighbour, with its current distance and direction.
 *   descs, weights   host arrays [n_layers] (1..16); every layer has the same lmax,
 *                    channels and storage, since features flow from layer to layer
 *   h                device [n][(lmax+1)^2][C] storage dtype
 *   out              device [n][(lmax+1)^2][C] fp32
 *   max_neighbors    K (1..4096) of the list at the largest cutoff
 *   policy           host; read and updated by every call
 *   state            device, >= e2v2_stack_state_bytes(...): the lists, the
 *                    reference positions and the target order, kept from call to
 *                    call; the caller leaves it untouched during a run
 *   workspace        device scratch, >= e2v2_stack_workspace_bytes(...)
 * Errors as for the calls above; on an error the policy is left unchanged. */
typedef struct {
    int32_t rebuild_every;        /* rebuild when this many steps have passed since the last one (10) */
    float max_displacement;       /* rebuild earlier when an atom moved more than this, A (0.25) */
    int32_t steps_since_rebuild;  /* state: steps since the last rebuild; negative forces one (start at -1) */
    int32_t rebuilt;              /* out: 1 if this call rebuilt the lists, else 0 */
    int64_t rebuilds;             /* out: rebuilds so far (the caller sets 0 at the start of a run) */
} e2v2_rebuild_policy;

size_t e2v2_stack_state_bytes(int32_t n_layers, const e2v2_layer_desc *descs, int32_t n, int32_t max_neighbors);
size_t e2v2_stack_workspace_bytes(int32_t n_layers, const e2v2_layer_desc *descs, int32_t n, int32_t max_neighbors);
e2v2_status e2v2_stack_forward(int32_t n_layers, const e2v2_layer_desc *descs, const e2v2_weights *weights,
                               const float *pos, const void *h, int32_t n, int32_t max_neighbors,
                               e2v2_rebuild_policy *policy, void *state, size_t state_bytes, float *out,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Gradient of the layer stack: for L = sum(grad_out * out), with
 * out the stack output of the last e2v2_stack_forward call at these positions and
 * features, writes grad_h = dL/dh [n][(lmax+1)^2][C] and, if grad_pos is not
 * NULL, grad_pos = dL/dpos [n][3] summed over the layers (the forces of the model
 * for E = L are -grad_pos).  The neighbour lists and the processing order are
 * those in `state` (left by that forward call), held fixed; each layer's input is
 * recomputed over them, then each layer's gradient (e2v2_layer_backward, over its
 * transposed list) runs in reverse order.  Arguments as for e2v2_stack_forward.
 * With bf16 storage each layer's gradient is taken as in e2v2_layer_backward (fp32
 * arithmetic at the bf16 inputs and weights) and the rounding of a layer's output
 * to the next layer's bf16 input passes the gradient through unchanged.  `policy`
 * is the host policy that forward call updated: with no rebuild recorded
 * (rebuilds < 1) the state holds no lists yet, and the call returns E2V2_ERR_ARG
 * before anything is enqueued.  Workspace: e2v2_stack_backward_workspace_bytes
 * (one transposed list per distinct cutoff).  Asynchronous on `stream`. */
size_t e2v2_stack_backward_workspace_bytes(int32_t n_layers, const e2v2_layer_desc *descs, int32_t n,
                                           int32_t max_neighbors);
e2v2_status e2v2_stack_backward(int32_t n_layers, const e2v2_layer_desc *descs, const e2v2_weights *weights,
                                const float *pos, const void *h, int32_t n, int32_t max_neighbors,
                                const void *state, size_t state_bytes, const e2v2_rebuild_policy *policy,
                                const float *grad_out, float *grad_h, float *grad_pos, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * The exact edge-equivalent form (E2Former-V2 explainer, section 1.2: the
 * Wigner-6j recoupling identity that lets a node-centric evaluation reproduce
 * an edge-centric one).  For each target i:
 *   out_i^l = W_O[l] m_i^l,  m_i = sum_j alpha_ij sum_p w_e[p] (v_j (x) S(x_ij))_p,
 * with x_ij = (r_j - r_i) / cutoff, S^l(x) = |x|^l Y^l(x / |x|) the component-
 * normalised real solid harmonics (S^0 = 1), p = (l_i, l_f, l_o) over the paths
 * of e2v2_path_table, v^l = h^l W_V[l], and alpha_ij the layer's attention
 * weights (q.k / sqrt(C / heads) plus the distance bias, softmax over the row).
 * The result depends on r_j - r_i only (translation invariant).  It is
 * evaluated node by node: each source is coupled once with S of its own
 * position relative to an origin (the centroid of the positions),
 * the stream sums those rows with alpha, and each target couples the sum with S
 * of its own position through the addition theorem of S and 6j recoupling
 * coefficients; the per-edge products are never formed.
 *   w    as for e2v2_attn_forward, except that w->w_src holds the edge weights
 *        w_e [n_paths(lmax)][C] fp32 and w->w_tgt is not read
 *   desc storage must be E2V2_FP32 and lmax <= 2 (E2V2_ERR_UNSUPPORTED
 *        otherwise): the node terms grow like (|r - o| / cutoff)^l_f and cancel
 *        to the edge term, so the fp32 rounding of the result grows like
 *        (R / cutoff)^lmax for atoms R from the centroid (measured: 2e-5 of
 *        the output RMS at R / cutoff = 4, 1,000 atoms)
 *   other arguments as for e2v2_attn_forward; workspace of at least
 *   e2v2_edge_workspace_bytes(desc, n) bytes. */
e2v2_status e2v2_edge_forward(const e2v2_layer_desc *desc, const float *pos, const void *h,
                              const e2v2_weights *w, const int32_t *nbr_start, const int32_t *nbr_len,
                              const int32_t *nbr_idx, const int32_t *target_order, int32_t n, float *out,
                              void *workspace, size_t workspace_bytes, hipStream_t stream);
size_t e2v2_edge_workspace_bytes(const e2v2_layer_desc *desc, int32_t n);
/* Host copy of the edge form's tables, for checking: which = 0 the source terms
 * (idx [k][4] = component of v, of S, of the source row, -1), which = 1 the target
 * terms (path, component of the summed row, of S, of the output), which = 2 the
 * blocks of the source row (l_i, lam, l', first component; val unused).  Writes
 * up to cap entries; returns the count, -1 for lmax outside 0..2. */
int32_t e2v2_edge_coefficients(int32_t lmax, int32_t which, int32_t *idx, double *val, int32_t cap);

/* ------------------------------------------------------------------------
 * Host-side tables (no GPU needed). */
int32_t e2v2_num_paths(int32_t lmax);   /* 1, 5, 15, 34 for lmax 0..3; -1 if out of range */
/* li_lf_lo: host [n_paths][3]. */
e2v2_status e2v2_path_table(int32_t lmax, int32_t *li_lf_lo);
/* EAAS coefficients used by the kernels: coef host [n_paths][7]; entry
 * [p][m_o + l_o] multiplies input m_i = m_o (even l_i+l_f+l_o) or m_i = -m_o
 * (odd) of the aligned-frame features; it equals sqrt(2 l_f + 1) times the
 * real coupling tensor at (m_i, m_f = 0, m_o).  Unused slots are 0. */
e2v2_status e2v2_eaas_coefficients(int32_t lmax, float *coef);
/* Real Wigner-D blocks D^l(R), l = 1..lmax, of the alignment rotation of r
 * (R z = r / |r|; the rotation is R_z(alpha) R_y(beta) with no roll), row-major,
 * concatenated; Y^l(R x) = D^l(R) Y^l(x).  Host reference of what the kernels
 * compute per node, fp64.  d: host [sum_{l=1..lmax} (2l+1)^2]. */
e2v2_status e2v2_alignment_wigner(int32_t lmax, const double *r, double *d);

const char *e2v2_status_string(e2v2_status s);
const char *e2v2_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* E2V2_H */
