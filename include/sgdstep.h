/*
 * sgdstep.h -- C ABI of one data-parallel worker's minibatch SGD step on an
 * AMD Instinct MI355X (gfx950).
 *
 * The step follows the SPRINT report (IPSJ SIG Technical Report
 * Vol.2016-HPC-155 No.8): a worker computes the gradient of one sub-batch
 * (Algorithm 1, ComputeGradient, realised as im2col plus matrix products per
 * the section 3.3 SGEMM table), adds it into its gradient buffer GradBuf, and
 * the buffers are summed and applied to the weights (Algorithm 2, with
 * momentum), or applied by a parameter server with a per-parameter Adagrad
 * rate (DistBelief review: w' = w - eta_i * dw).
 *
 * Conventions shared by every entry point:
 *  - All tensors are caller-owned device memory (float32 unless stated).  The
 *    library allocates no device memory; it owns only the host-side net
 *    handle.  Pointers are plain device addresses.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *    kernels on it and return after launch; they never synchronise.  The
 *    caller synchronises before reading results.
 *  - Return value: SGD_OK (0) or a negative SGD_E* code.  The status covers
 *    argument, shape and launch errors only.  sgd_last_error() returns a
 *    thread-local message for the last failure.  Nothing throws across the ABI.
 *  - Results are deterministic: no floating-point atomics; every reduction
 *    has a fixed order, so two identical calls give bitwise-identical outputs.
 *  - NaN in inputs or weights propagates to the loss and gradients (ReLU
 *    passes NaN through); it is not an error.
 */
#ifndef SGDSTEP_H
#define SGDSTEP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define SGD_OK 0
#define SGD_EINVAL (-1)       /* null pointer, bad enum, bad size            */
#define SGD_ESHAPE (-2)       /* layer list does not describe a valid net   */
#define SGD_EWORKSPACE (-3)   /* workspace smaller than sgd_workspace_bytes */
#define SGD_EDEVICE (-4)      /* a HIP launch or query failed               */
#define SGD_EUNSUPPORTED (-5) /* valid request outside what is implemented  */

/* ---- layer kinds ---- */
#define SGD_CONV 1       /* out = out channels, kernel = c, pad = zero padding P; stride 1 */
#define SGD_RELU 2       /* must directly follow SGD_CONV or SGD_FC                        */
#define SGD_MAXPOOL 3    /* pool = p: p x p windows, stride p; p must divide H and W       */
#define SGD_FC 4         /* out = output width                                             */
#define SGD_SOFTMAX_CE 5 /* last layer; must directly follow an SGD_FC without ReLU        */

/* ---- loss reduction over the sub-batch ---- */
#define SGD_REDUCE_MEAN 0 /* loss and gradient scaled by 1/N (Chainer's softmax_cross_entropy) */
#define SGD_REDUCE_SUM 1  /* unscaled sum over samples (SPRINT eq. (1) sums per-sample grads)  */

/* ---- update rules ---- */
#define SGD_PLAIN 0    /* W = W - eta*G                          (SPRINT eq. (1))           */
#define SGD_MOMENTUM 1 /* V = mu*V - eta*G; W = W + V            (SPRINT Algorithm 2, nu=mu) */
#define SGD_ADAGRAD 2  /* A = A + G*G; W = W - (eta/(sqrt(A)+eps))*G  (DistBelief review)   */
#define SGD_NESTEROV 3 /* V = mu*V - eta*G; W = W + mu*V - eta*G  (PIPE report, appendix A) */

/* ---- tensor-info selectors (sgd_tensor_info) ---- */
#define SGD_T_OUT 0    /* forward output of the layer                                  */
#define SGD_T_DOUT 1   /* gradient of the loss: for conv/fc w.r.t. the pre-activation  */
                       /* (ReLU derivative applied), for maxpool w.r.t. its output     */
#define SGD_T_COL 2    /* conv only: im2col matrix (overwritten by dCol in backward)   */
#define SGD_T_WREP 3   /* conv only: weights repacked to [Co][ky][kx][ci]               */
#define SGD_T_ARGMAX 4 /* maxpool only: uint8 window-local argmax ky*p+kx              */

/* ---- tensor layouts reported by sgd_tensor_info ---- */
#define SGD_LAYOUT_NHWC 1 /* dims = {N, H, W, C}                                      */
#define SGD_LAYOUT_NCHW 2 /* dims = {N, C, H, W}                                      */
#define SGD_LAYOUT_ROWS 3 /* dims = {rows, cols, row stride, 1}, row-major             */

typedef struct sgd_layer {
  int kind;   /* SGD_CONV ... SGD_SOFTMAX_CE                 */
  int out;    /* conv: output channels; fc: output width     */
  int kernel; /* conv: filter width c                        */
  int pad;    /* conv: zero padding P on each side           */
  int pool;   /* maxpool: window p                           */
} sgd_layer;

typedef struct sgd_input {
  int batch;    /* N_Subbatch                                 */
  int channels; /* m_0 (an MLP input is channels=width, h=w=1) */
  int height;
  int width;
} sgd_input;

typedef struct sgd_net sgd_net;

/*
 * Plan a network (host only; no device call).  Shapes follow SPRINT section
 * 3.2 eq. (2), generalised to zero padding: a conv layer maps H to
 * H + 2P - c + 1, a pool layer divides by p, an fc layer flattens its input in
 * (c, h, w) order.  `layers` is copied.  On success *out receives a handle to
 * free with sgd_destroy_net.  Errors: SGD_EINVAL (null pointer, n_layers < 2,
 * bad reduction), SGD_ESHAPE (non-positive sizes, pool not dividing the map,
 * conv output < 1, no final SGD_SOFTMAX_CE), SGD_EUNSUPPORTED (ReLU not after
 * conv/fc, conv after fc, softmax not after an fc).
 */
int sgd_create_net(const sgd_input* input, const sgd_layer* layers, int n_layers, int reduction,
                   sgd_net** out);
void sgd_destroy_net(sgd_net* net);

/*
 * Number of parameters, SPRINT section 3.2 eq. (3):
 *   sum over conv layers of m_l (c^2 m_{l-1} + 1) + sum over fc layers of
 *   m_l (x_{l-1}^2 m_{l-1} + 1).
 * The flat parameter vector W (and every gradient) has this length and holds,
 * per weighted layer in network order, the weight (conv [Co][Ci][c][c], fc
 * [out][in]) followed by the bias.  Returns -1 for a null net.
 */
int64_t sgd_param_count(const sgd_net* net);

/*
 * Element offsets of each weighted layer's weight and bias inside the flat
 * vector, in network order.  Writes min(count, max_layers) entries and
 * returns the number of weighted layers (or a negative error).
 */
int sgd_param_offsets(const sgd_net* net, int64_t* w_off, int64_t* b_off, int max_layers);

/* Bytes of device workspace sgd_compute_gradient needs (0 for a null net). */
size_t sgd_workspace_bytes(const sgd_net* net);

/*
 * Where a layer's intermediate tensor lives inside the workspace after
 * sgd_compute_gradient: byte offset, dims (see SGD_LAYOUT_*) and layout.
 * `layer` indexes the layer list given to sgd_create_net (a ReLU entry
 * reports the tensors of the conv/fc it follows).  Returns SGD_OK, or
 * SGD_EINVAL if that layer has no such tensor.  For inspection and tests.
 */
int sgd_tensor_info(const sgd_net* net, int layer, int which, int64_t* byte_offset, int64_t dims[4],
                    int* layout);

/*
 * One sub-batch gradient (SPRINT Algorithm 1, Grad = ComputeGradient(Weights)).
 *  W     [param_count] weights, flat layout above.
 *  X     [N][C][H][W] images, float32, NCHW.
 *  y     [N] int32 labels in [0, classes).  An out-of-range label is caller
 *        error: the softmax kernel never indexes with it (that row's loss and
 *        logit gradient become NaN, so the loss and gradients are NaN), and
 *        with sgd_set_debug on the call returns SGD_EINVAL before any launch.
 *  grad  [param_count] output: the full gradient (every element written).
 *  loss  device float scalar output: softmax cross-entropy, reduced per the
 *        net's reduction.
 *  ws    device workspace of at least sgd_workspace_bytes(net) bytes,
 *        256-byte aligned; its contents on entry do not matter.
 * The kernel sequence is: forward (im2col + GEMM + bias/ReLU + maxpool per
 * conv layer, GEMM + bias/ReLU per fc layer), softmax-CE, then backward in
 * reverse layer order with the dedw, dedb, dedx_fc and dedx_conv products of
 * SPRINT's section 3.3 table (dedx_conv followed by col2im).  No dedx is
 * computed for the first weighted layer.  Errors: SGD_EINVAL (null pointer),
 * SGD_EWORKSPACE, SGD_EDEVICE.
 */
int sgd_compute_gradient(sgd_net* net, const float* W, const float* X, const int32_t* y, float* grad,
                         float* loss, void* ws, size_t ws_bytes, void* stream);

/*
 * A worker's gradient buffer with SPRINT's empty state (Algorithms 1 and 2).
 * `data` is device memory of n floats; `empty` is kept on the host.
 */
typedef struct sgd_gradbuf {
  float* data;
  int64_t n;
  int empty;
} sgd_gradbuf;

/*
 * The same gradient computation written straight into a gradient buffer:
 * stored if the buffer is empty, added element by element (one rounding per
 * addition, after the gradient is formed in fp32) if not -- SPRINT Algorithm
 * 1's ComputeGradient followed by its GradBuf update, without the separate
 * gradient array.  Bitwise equal to sgd_compute_gradient followed by
 * sgd_accumulate_grad.  gb->n must equal the parameter count; clears
 * gb->empty.  Errors as sgd_compute_gradient, and SGD_EINVAL for a buffer of
 * the wrong length.
 */
int sgd_compute_gradient_into(sgd_net* net, const float* W, const float* X, const int32_t* y, sgd_gradbuf* gb,
                              float* loss, void* ws, size_t ws_bytes, void* stream);

/*
 * sgd_compute_gradient_into with the worker-side scaling of SPRINT Algorithm
 * 1 (the worker stores Grad <- -eta * grad): every gradient value is multiplied
 * by `scale` (one rounding) before it is stored in or added to the buffer.
 * scale = -eta makes the buffer hold the step itself; applying it with
 * sgd_apply_update and eta = -1 then gives bitwise the unscaled path's
 * result (the products -1 * (-eta*g) and eta*g round identically).  scale = 1
 * is sgd_compute_gradient_into.  Errors as sgd_compute_gradient_into, and
 * SGD_EINVAL for a non-finite scale.
 */
int sgd_compute_gradient_into_scaled(sgd_net* net, const float* W, const float* X, const int32_t* y,
                                     sgd_gradbuf* gb, float scale, float* loss, void* ws, size_t ws_bytes,
                                     void* stream);

/*
 * GradBuf <- grad if the buffer is empty, else GradBuf + grad (SPRINT
 * Algorithm 1, the GradBuf update).  Clears `empty`.  grad has gb->n floats.
 * Errors: SGD_EINVAL, SGD_EDEVICE.
 */
int sgd_accumulate_grad(sgd_gradbuf* gb, const float* grad, void* stream);

/*
 * Fold k gradients into the buffer in index order, as SPRINT Algorithm 2
 * folds GradBuf_1..GradBuf_N into SendBuf: the first is copied if the buffer
 * is empty, every later one added, one rounding per addition.  `grads` is a
 * host array of k device pointers; 1 <= k <= 16.  Errors: SGD_EINVAL,
 * SGD_EDEVICE.
 */
int sgd_accumulate_grads(sgd_gradbuf* gb, const float* const* grads, int k, void* stream);

typedef struct sgd_rule {
  int rule;    /* SGD_PLAIN, SGD_MOMENTUM, SGD_ADAGRAD or SGD_NESTEROV  */
  float eta;   /* learning rate                                         */
  float mu;    /* momentum coefficient (SGD_MOMENTUM, SGD_NESTEROV)     */
  float eps;   /* Adagrad denominator offset                            */
  float decay; /* weight decay (0: none); the PIPE report's appendix A
                  trains with 5e-4                                      */
} sgd_rule;

/*
 * Apply the buffered gradient G to W in place, elementwise, one rounding per
 * statement in this order (no fused multiply-add; correctly rounded sqrt and
 * division):
 *   decay != 0 first: wd = decay*W; G = G + wd      (weight decay, any rule)
 *   plain:    t = eta*G;  W = W - t
 *   momentum: t1 = mu*V; t2 = eta*G; V = t1 - t2; W = W + V
 *   adagrad:  A = A + G*G; d = sqrt(A) + eps; r = eta/d; t = r*G; W = W - t
 *   nesterov: t1 = mu*V; t2 = eta*G; V = t1 - t2; t3 = mu*V; u = t3 - t2;
 *             W = W + u
 * `state` is V (momentum, Nesterov) or A (Adagrad), n = gb->n floats; NULL
 * for plain.  An empty GradBuf is a zero gradient (SPRINT Algorithm 2 sends
 * 0 when the first buffer is empty): without decay, plain and Adagrad then
 * leave W unchanged and momentum still decays V; weight decay still applies.
 * Marks the buffer empty afterwards.  Errors: SGD_EINVAL, SGD_EDEVICE.
 */
int sgd_apply_update(float* W, sgd_gradbuf* gb, float* state, const sgd_rule* rule, void* stream);

/*
 * One pass that sums k gradient buffers in index order (a left fold, one
 * rounding per addition) and applies the rule, as the parameter server's
 * SumGradient + update of SPRINT Algorithm 2; bitwise equal to
 * sgd_accumulate_grads into an empty buffer followed by sgd_apply_update.
 * `grads` is a host array of k device pointers, 1 <= k <= 16, each n floats.
 * Errors: SGD_EINVAL, SGD_EDEVICE.
 */
int sgd_apply_fused(float* W, float* state, const float* const* grads, int k, int64_t n,
                    const sgd_rule* rule, void* stream);

/*
 * Memory-traffic reference for the update kernels (measurement only; it is
 * not a step of the method).  For every element i < n:
 * outs[j][i] = ins[0][i] + ... + ins[n_in-1][i] for each j < n_out -- the
 * read and write streams of an update pass (the parameter-server apply
 * reads 8 gradient buffers, W and A and writes W and A: 10 reads, 2 writes)
 * without the rule's arithmetic or the GradBuf semantics.  Supported
 * (n_in, n_out): (1, 1) a copy, (10, 0) reads only, (10, 2).  `groups` is the
 * number of float4 groups per thread: 1 (one float4 per thread) or 4 (the
 * update kernels' block-contiguous layout).  ins and outs are host arrays of
 * device pointers, 16-byte aligned; n a positive multiple of 4; outputs may
 * alias inputs.  Errors: SGD_EINVAL, SGD_EDEVICE.
 */
int sgd_stream_ref(float* const* outs, int n_out, const float* const* ins, int n_in, int64_t n, int groups,
                   void* stream);

/*
 * One fp32 matrix product on the library's matrix-core kernels, the SGEMM of
 * the SPRINT report's section 3.3 table: C[m][n] = op(A) * op(B), row-major
 * C with row stride ldc.
 *   a_t == 0: A stored [m][k] (row stride lda); a_t == 1: A stored [k][m].
 *   b_t == 0: B stored [n][k] (row stride ldb), i.e. C = A * B^T (the
 *             forward form of conv and fc); b_t == 1: B stored [k][n].
 * Results are deterministic (fixed summation order for a given shape and
 * GPU).  `ws` is device scratch of sgd_gemm_workspace_bytes() bytes (may be
 * NULL when that is 0), 256-byte aligned.  All pointers are device memory
 * owned by the caller; the call is asynchronous on `stream`.  It serves the
 * timing model of the SPRINT report's section 3.3 (eq. 6 is fitted over such
 * calls) and any caller that wants one product.  Errors: SGD_EINVAL (null
 * pointer, sizes < 1, strides shorter than a row, 2^22 or more 64 x 64
 * output tiles), SGD_EWORKSPACE, SGD_EDEVICE.  sgd_gemm_workspace_bytes
 * returns 0 for invalid arguments.
 */
typedef struct sgd_gemm_args {
  int m, n, k;
  int a_t, b_t;
  const float* A;
  int64_t lda;
  const float* B;
  int64_t ldb;
  float* C;
  int64_t ldc;
} sgd_gemm_args;
size_t sgd_gemm_workspace_bytes(const sgd_gemm_args* g);
int sgd_gemm(const sgd_gemm_args* g, void* ws, size_t ws_bytes, void* stream);

/*
 * Schedule query for the tile kernels behind sgd_gemm and the step's
 * products (host only: no device work, no device needed; the compute-unit
 * count is the current device's, 256 without one).  For an m x n x k
 * product of the given forms (as sgd_gemm's a_t / b_t; n counts a weight
 * gradient's bias column) it writes the schedule the library picks when the
 * product takes the direct-load tile kernels, not gathered, to
 * out[0..11]: tile rows, tile columns, grid (blocks), tiles done whole
 * first, stream-K k-slices (0: none), block-group tile rows and columns (1
 * and 1: ungrouped), edge-last bits (1: ragged last tile row last, 2: ragged
 * last tile column last), tile rows count, tile columns count, 16-deep
 * k-slices per tile, compute units.  A product can still take another
 * kernel (short reductions, a logits layer's skinny products, unaligned
 * operands); the query describes the tile schedule alone.  It serves tests
 * and tools that check the schedule's invariants (every (tile, k-slice)
 * covered once, stream-K slots in k order) on the CPU; it is not a step of
 * the method.  nout >= 12.  Errors: SGD_EINVAL (sizes < 1, null out,
 * nout < 12, 2^22 or more 64 x 64 output tiles).
 */
int sgd_gemm_plan(int m, int n, int k, int a_t, int b_t, int64_t* out, int nout);

/*
 * Implicit-GEMM convolution (on by default).  A conv layer whose input is
 * an activation of this network with Ci % 16 == 0 gathers the im2col
 * operand of its forward and dedw products straight from that activation
 * (SPRINT section 3.3's im2col matrix is never written), and a conv layer
 * with Co % 16 == 0 (not the first) computes dedx as one gather-form product
 * over its output gradient with the ReLU mask in the epilogue, in place of
 * the dCol product and col2im.  Other layers use the explicit im2col path.
 * Changing the setting re-plans the workspace: query sgd_workspace_bytes
 * again.  The forward and dedw results are bitwise the same either way; dedx
 * sums its terms in another order.  Errors: SGD_EINVAL (null net).
 */
int sgd_set_implicit_conv(sgd_net* net, int enable);

/*
 * Debug mode (off by default).  While it is on, sgd_compute_gradient,
 * sgd_compute_gradient_into(_scaled) and sgd_train_step copy the labels y to
 * the host before launching anything (a synchronous read on `stream`, which
 * therefore waits for the work already queued there) and return SGD_EINVAL,
 * with the first bad row named in sgd_last_error(), when a label lies outside
 * [0, classes); nothing is launched then.  sgd_train_step_graph checks the
 * labels once when it records the step (replays are not checked).  The pages
 * give no error convention; this is the plain C-library choice of validating
 * caller data only on request.  Errors: SGD_EINVAL (null net).
 */
int sgd_set_debug(sgd_net* net, int enable);

/*
 * Backward-pass concurrency.  With overlap on each layer's dedw product runs
 * on a second stream the library owns, forked from the caller's stream once
 * the product's inputs are final and joined back into it before the call's
 * work ends, so a dedw product overlaps the next layer's dedx product
 * (SPRINT section 3.3's products are independent once the layer's output
 * gradient exists).  Results are bitwise identical with overlap off; the
 * caller still sees one stream-ordered operation.
 *
 * enable: 1 on, 0 off, negative: the default, which is on when the net's
 * weight-gradient products total at least 2^30 flops per step (2 m n k
 * summed over the dedw products, dedb's column included) and off below,
 * where the fork and join cost more than the overlap gains.  A graph
 * recorded by sgd_train_step_graph keeps the setting in effect when it was
 * recorded.  Errors: SGD_EINVAL (null net).
 */
int sgd_set_overlap(sgd_net* net, int enable);

/* The overlap setting in effect (after the default is resolved): *on = 1 or
 * 0.  Errors: SGD_EINVAL (null net or output). */
int sgd_get_overlap(const sgd_net* net, int* on);

/*
 * Per-launch kernel timing, for measurement.  While enabled, every kernel
 * sgd_compute_gradient launches is bracketed by a HIP event pair on the
 * stream it is launched on, and its algorithmic work is recorded: flops of the
 * arithmetic the method needs (2mnk for a product of the SPRINT section 3.3
 * table, with k the unpadded reduction length) and bytes it must move
 * through HBM (each operand read once, each result written once).
 *
 * sgd_profile(net, 1) clears the records and starts recording; (net, 0)
 * stops.  sgd_profile_read waits for the recorded events, copies up to
 * max_records entries to `out` (in launch order) and returns the number of
 * records.  `kernel` points to a static string.  Errors: SGD_EINVAL,
 * SGD_EDEVICE.
 */
typedef struct sgd_kernel_time {
  const char* kernel; /* e.g. "gemm_64x128_nt", "im2col", "softmax_ce"     */
  int layer;          /* index in the layer list; -1 for an inserted stage
                         or the one weight-repack launch of all conv layers */
  int phase;          /* 0 forward, 1 backward                              */
  double ms;          /* event-measured duration of the launch              */
  double flops;       /* algorithmic floating-point operations              */
  double bytes;       /* algorithmic HBM bytes                              */
  int m, n, k;        /* the product's shape for GEMM launches (and their
                         fixup / split-reduce passes), else 0               */
  int product;        /* index of that product within the recording (all of
                         its launches share it), -1 for other kernels      */
} sgd_kernel_time;

int sgd_profile(sgd_net* net, int enable);
int sgd_profile_read(sgd_net* net, sgd_kernel_time* out, int max_records);

/*
 * One whole SGD step for the common case of one sub-batch per update: the
 * gradient of (X, y) at W is computed and the rule applied to W in place,
 * each layer's update issued as soon as that layer's gradient is final (in
 * the epilogue of its dedw product), so no gradient array is written or read
 * back.  Bitwise equal to sgd_compute_gradient_into into an empty GradBuf
 * followed by sgd_apply_update with the same rule (SPRINT Algorithm 1's
 * gradient into an empty GradBuf, then the apply).  `state` is V (momentum)
 * or A (Adagrad), param_count floats, updated in place; NULL for plain.
 * Errors as sgd_compute_gradient and sgd_apply_update.
 */
int sgd_train_step(sgd_net* net, float* W, const float* X, const int32_t* y, float* state, const sgd_rule* rule,
                   float* loss, void* ws, size_t ws_bytes, void* stream);

/*
 * sgd_train_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same step, bitwise the same W, state and loss, with no workspace
 * argument.  The workspace lives in a static device array of
 * SGD_NOALLOC_SCRATCH_BYTES (64 MiB) that each GPU the library runs on holds
 * until the process ends; the call makes no hipMalloc / hipFree and creates
 * no stream or event (every dedw product runs on `stream`, which gives the
 * same results as the overlapped step).  The array's address on the current
 * device is looked up once, on the first call on that device.  Every call on
 * one GPU shares that GPU's array and nothing in it needs to start at zero:
 * calls that overlap on one GPU (different streams, threads or processes'
 * shared contexts) race and give undefined results -- serialise them.  Errors:
 * SGD_EWORKSPACE when sgd_workspace_bytes(net) exceeds the array, SGD_EINVAL
 * (null net, bad rule, profiling on), SGD_EDEVICE, and those of
 * sgd_train_step.
 */
#define SGD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int sgd_train_step_noalloc(sgd_net* net, float* W, const float* X, const int32_t* y, float* state,
                           const sgd_rule* rule, float* loss, void* stream);

/*
 * SPRINT on one GPU (SPRINT report section 3.4, Algorithms 1 and 2): worker
 * threads, each with its own HIP stream, copy of the weights, gradient
 * array Grad and gradient buffer GradBuf_t with the empty flag, and one
 * update thread with its own stream, all sharing LatestWeights (W) on one
 * device.
 *
 *   worker t, step i (Algorithm 1): if i % n_fetch == 0 and LatestWeights is
 *     newer than its copy, copy it (the fetch, under the weights lock);
 *     take the next sub-batch (batch index = a shared counter mod n_batches);
 *     Grad <- ComputeGradient, folded into a private sum over n_push steps;
 *     every n_push steps (and at its last step) lock GradBuf_t, copy the sum
 *     in if the buffer is empty, else add it (the push).
 *   updater (Algorithm 2 with one node): wait until at least min_bufs
 *     buffers are non-empty (or every worker has finished); take every
 *     non-empty GradBuf_t in index order, marking it empty; W <- rule(W, sum
 *     of the taken buffers) in one fused pass (the algorithm's momentum is
 *     the rule's state); publish the new version.
 *
 * The locks are host mutexes; the device order behind them is carried by
 * HIP events (a worker's add is complete before the updater reads the
 * buffer; the updater's read before the worker refills it; a fetch copy
 * before the next update overwrites W).  Each worker step ends with a wait
 * for its stream, as a worker thread of the report waits for its GPU.
 *
 * n_fetch and n_push are the DistBelief review's fetch and push intervals
 * (Downpour SGD); n_fetch = n_push = 1 is SPRINT.  min_bufs = 1 is the
 * asynchronous SPRINT updater; with min_bufs = workers and sync = 1 (each
 * worker waits for an update newer than its last push before its next step)
 * the run is bulk-synchronous SGD on workers x N_Subbatch samples per update.
 */
typedef struct sgd_sprint_config {
  int workers;   /* N_GPU worker threads / streams, 1..16                   */
  int iters;     /* gradient steps per worker, >= 1                          */
  int n_fetch;   /* fetch interval (steps), >= 1                             */
  int n_push;    /* push interval (steps), >= 1                              */
  int min_bufs;  /* non-empty buffers an update waits for, 1..workers        */
  int sync;      /* 1: wait for a newer version before each step after a push */
} sgd_sprint_config;

/* One gradient step of one worker, in the log. */
typedef struct sgd_sprint_contrib {
  int worker, iter;      /* which worker, its step index                       */
  int push;              /* index of the worker's push that carried it         */
  int64_t batch;         /* sub-batch index into X / y                          */
  int64_t version;       /* version of W its gradient was computed at (0: the
                            caller's W, v: after v updates)                    */
  int64_t update;        /* the update that applied it (it turned version
                            `update` into `update` + 1), -1 if none           */
} sgd_sprint_contrib;

typedef struct sgd_sprint_stats {
  int64_t updates;       /* updates applied (final version of W)               */
  int64_t steps;         /* worker gradient steps (workers x iters)            */
  int64_t fetches;       /* weight copies made by workers                      */
  double wall_ms;        /* the whole run                                      */
  double t_gpu_ms;       /* mean worker step (T_GPU of eq. 9)                  */
  double t_update_ms;    /* mean time between update completions (T_Update)    */
  double n_minibatch_avg;/* measured: sub-batches applied per update x N_Subbatch */
  double n_minibatch_eq9;/* eq. 9 (one node): workers x N_Subbatch x T_Update / T_GPU */
  double staleness_mean; /* mean over steps of update - version                */
  int64_t staleness_max;
} sgd_sprint_stats;

/* Device bytes sgd_sprint_run needs for `net` (its batch is N_Subbatch) and
 * cfg: per worker the net's workspace, three parameter-sized arrays (weights
 * copy, Grad sum, GradBuf_t) and the loss.  0 for invalid arguments. */
size_t sgd_sprint_workspace_bytes(const sgd_net* net, const sgd_sprint_config* cfg);

/*
 * Run cfg->workers x cfg->iters worker steps with the update thread as
 * above; returns when every step has been applied (the last update drains
 * whatever the buffers hold).  W (param_count floats) is LatestWeights,
 * updated in place; `state` the rule's state (NULL for plain).  X and y hold
 * n_batches sub-batches of the net's batch size, consecutive.  `ws` is
 * device memory of sgd_sprint_workspace_bytes(), 256-byte aligned.  The run
 * starts after the work queued on `stream` and the caller's stream waits
 * for its end; the calling thread blocks until the run ends.  `log` (host,
 * may be NULL) receives up to log_cap records, one per worker step, in
 * (worker, iter) order; `stats` (host, may be NULL) the figures above.  The
 * net's own workspace and streams are not used: each worker plans its own
 * copy of the net.  Errors: SGD_EINVAL (bad config, null pointers,
 * n_batches < 1, rule without its state), SGD_EWORKSPACE, SGD_EDEVICE; the
 * first error of any thread stops the run.
 *
 * For tests of that error path, the environment variable
 * SGD_SPRINT_INJECT_FAILURE makes one thread fail with SGD_EDEVICE from the
 * host, with no GPU fault: "w<t>:<i>" fails worker t at its step i while it
 * holds its buffer, "u:<v>" fails the updater at update v while it holds
 * the weights.  Any other value is ignored.
 */
int sgd_sprint_run(const sgd_net* net, const sgd_sprint_config* cfg, float* W, float* state, const sgd_rule* rule,
                   const float* X, const int32_t* y, int64_t n_batches, void* ws, size_t ws_bytes, void* stream,
                   sgd_sprint_stats* stats, sgd_sprint_contrib* log, int64_t log_cap);

/*
 * sgd_train_step recorded once as a HIP graph, to be replayed with one
 * launch per step: the step's 20-100 kernel launches (and the fork/join of
 * the dedw stream) become graph nodes, which removes the host launch gaps
 * that dominate small networks.  Recording does not run the step.  The graph
 * is bound to the pointers given here: every replay reads X, y and the
 * current contents of W and state, and writes W, state, loss and ws, exactly
 * as sgd_train_step with those arguments would (bitwise).  While a replay is
 * in flight neither the graph's buffers nor the net may be used by another
 * call; the net must outlive the graph.  Profiling must be off.  Errors:
 * as sgd_train_step, SGD_EINVAL (profiling on, null output), SGD_EDEVICE
 * (capture or instantiation failed).
 */
typedef struct sgd_step_graph sgd_step_graph;
int sgd_train_step_graph(sgd_net* net, float* W, const float* X, const int32_t* y, float* state,
                         const sgd_rule* rule, float* loss, void* ws, size_t ws_bytes, sgd_step_graph** out);
/* One replay of the recorded step on `stream` (asynchronous).  Errors: SGD_EINVAL, SGD_EDEVICE. */
int sgd_step_graph_launch(sgd_step_graph* g, void* stream);
void sgd_step_graph_destroy(sgd_step_graph* g);

/* Thread-local message describing the last failed call ("" if none). */
const char* sgd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SGDSTEP_H */
