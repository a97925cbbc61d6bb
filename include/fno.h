/*
 * fno.h - C ABI of the MI355X (gfx950) FNO spectral-convolution library.
 *
 * The operation is the Fourier Neural Operator spectral-convolution layer as
 * the TurboFNO write-up ("TurboFNO: FFT-GEMM-iFFT fusion kernels") describes
 * it: section 1 and sections 2.1-2.3 (real FFT of a [B, C, H, W] field, the
 * per-mode complex contraction einsum("xyij,xyik->xyjk") over the input
 * channel with a learnable weight of shape (modes_x, modes_y, in_ch, out_ch),
 * inverse real FFT), and section 4.3 (a C function on raw device pointers
 * called from a PyTorch autograd Function). Sizes are fixed when a plan is
 * made (section 2.3: the output size is a build-time constant of the fused
 * kernel), and grids are powers of two (section 2.1).
 *
 * For every plane the layer computes
 *   Xh[kx, ky] = (1 / prod(grid)) * sum_n x[n] exp(-2 pi i k.n / grid)
 * on the retained modes only, then Yh[b, o, k] = sum_i Xh[b, i, k] w[k, i, o]
 * (no conjugation), then the inverse real transform from the retained modes
 * (every other mode zero), which keeps the real part of the kz = 0 (2D:
 * ky = 0) term and doubles the others. This equals torch.fft.rfft2 ->
 * per-mode einsum -> torch.fft.irfft2 with the default normalisation.
 *
 * Retained modes. 2D: kx in [0, m1) and [H - m1, H) (two corners), ky in
 * [0, m2) (half spectrum). 3D: kx in [0, m1) and [X - m1, X), ky in [0, m2)
 * and [Y - m2, Y), kz in [0, m3).
 *
 * Layouts (all arrays contiguous, on the plan's device, in the plan's dtype):
 *   x  2D [B][Ci][H][W]          3D [B][Ci][X][Y][Z]   (last axis contiguous)
 *   y  2D [B][Co][H][W]          3D [B][Co][X][Y][Z]
 *   w  2D [2*m1][m2][Ci][Co][2]  3D [2*m1][2*m2][m3][Ci][Co][2]
 *      (re, im interleaved; along a corner axis index a < m selects k = a,
 *       index a >= m selects k = N - 2*m + a, i.e. the low corner first.)
 *
 * Ownership. The caller owns x, w and y and keeps them alive until the work
 * queued on `stream` has finished. The plan owns its twiddle tables and its
 * spectra workspace and, where the backward's adjoint contraction cannot
 * read w directly, a buffer for the conjugate-transposed weights: fp32 plans
 * with an odd c_out, and fp16 / bf16 plans whose adjoint contraction runs
 * off the matrix cores or whose c_out is not a multiple of 4; all allocated
 * by fno_plan_create, freed by fno_plan_destroy.
 * Execution calls allocate nothing.
 *
 * Execution calls are asynchronous on `stream` (a hipStream_t; NULL is the
 * null stream) and return as soon as the kernels are queued. One plan runs
 * one call at a time: concurrent calls on different streams need different
 * plans, because they share the plan's workspace. Results are deterministic
 * run to run (no atomics on the data path).
 *
 * Errors. No function throws. Argument errors are detected on the host
 * before any HIP call. A failed fno_plan_create sets *plan to NULL.
 */
#ifndef FNO_H
#define FNO_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fno_plan_s *fno_plan_t;

/* Storage dtype of x, w and y. Every sum accumulates in fp32; the operands
 * of the products are:
 *   FNO_F32   transforms: fp16 matrix-core products of hi + lo parts (each
 *             fp32 operand split into two fp16, about 22 significant bits);
 *             contraction: fp32 matrix-core products; spectra exchanged
 *             between launches as complex fp32.
 *   FNO_F16, FNO_BF16  transforms: fp16 matrix-core products of inputs,
 *             intermediate row / column results and twiddles, each scaled by
 *             a power of two chosen from a bound so no fp16 operand overflows
 *             or loses precision to the subnormal range. 2D layers on
 *             64..256-wide planes with batch >= 16 exchange the spectra as
 *             fp16 with power-of-two exponents and contract them on matrix
 *             cores: fp16 products of the spectra (brought to one
 *             power-of-two scale per batch row) and fp16 weights as stored,
 *             or bf16 hi + lo products for bf16 weights (exact); the
 *             backward of such layers exchanges its spectra the same way
 *             (K a multiple of 4) and forms grad_w from fp16 products of the
 *             spectra, each channel row brought to one power-of-two scale
 *             over the batch. Other layers and passes exchange
 *             complex fp32 spectra and contract them with
 *             bf16 hi + lo matrix-core products (batch >= 16) or fp32
 *             matrix-core products.
 * Planes below 64 rows or columns take register FFTs in fp32 instead of
 * matrix-core transforms. */
typedef enum { FNO_F32 = 0, FNO_F16 = 1, FNO_BF16 = 2 } fno_dtype_t;

typedef enum {
  FNO_OK = 0,
  FNO_ERR_INVALID_ARG = 1, /* NULL / misaligned / overlapping pointer, bad
                              size, mode out of range, wrong ndim */
  FNO_ERR_UNSUPPORTED = 2, /* valid but outside the built kernels' range */
  FNO_ERR_OUT_OF_MEMORY = 3, /* workspace allocation failed */
  FNO_ERR_DEVICE = 4       /* any HIP runtime error (launch included) */
} fno_status_t;

/* Make a plan for one layer shape.
 *   plan   out: the new plan (NULL on failure)
 *   ndim   2 or 3
 *   batch, c_in, c_out  >= 1
 *   grid   ndim entries (H, W or X, Y, Z): powers of two in [8, 256]
 *   modes  ndim entries (m1, m2 or m1, m2, m3): 1 <= m_d <= grid_d / 2
 *   dtype  storage dtype of x, w, y
 *   device HIP device ordinal
 * UNSUPPORTED when max(next_pow2(m_d)) over the axes of a transformed plane
 * exceeds 32 or half the smallest axis of that plane. Allocates the
 * workspace and twiddle tables on `device`; synchronous. */
fno_status_t fno_plan_create(fno_plan_t *plan, int ndim, int batch, int c_in,
                             int c_out, const int *grid, const int *modes,
                             fno_dtype_t dtype, int device);

/* One 2D layer: y = SpectralConv2d(x; w). x, w, y are device pointers laid
 * out as above, 16-byte aligned; x and y must not overlap. INVALID_ARG on a
 * 3D plan. */
fno_status_t fno_spectral_conv2d(fno_plan_t plan, const void *x, const void *w,
                                 void *y, void *stream);

/* One 3D layer (3D plan only); as fno_spectral_conv2d. */
fno_status_t fno_spectral_conv3d(fno_plan_t plan, const void *x, const void *w,
                                 void *y, void *stream);

/* ---- backward pass -------------------------------------------------------
 * Gradients of a scalar loss L through the layer (TurboFNO write-up,
 * section 4.3: the layer is a PyTorch autograd Function, so its backward
 * returns dL/dx and dL/dw given dL/dy). The layer is linear in x and in w,
 * so, with Gh[b][o][k] = forward spectra of grad_y (scaled as in the
 * forward) and Xh those of x:
 *   grad_x = the layer applied to grad_y with every mode's weight matrix
 *            replaced by its conjugate transpose (c_out -> c_in channels);
 *   grad_w[k][i][o] = prod(grid) * gamma_k * sum_b conj(Xh[b][i][k]) Gh[b][o][k],
 *            gamma_k = 1 when the last-axis mode index of k is 0, else 2.
 * A complex weight's gradient is dL/dRe(w) + i dL/dIm(w) (the PyTorch
 * convention); these equal PyTorch autograd through rfft2 -> einsum ->
 * irfft2.
 *   x      [B][Ci][grid] as in the forward; needed only for grad_w
 *   w      as in the forward; needed only for grad_x
 *   grad_y [B][Co][grid], dL/dy
 *   grad_x [B][Ci][grid] out, or NULL to skip
 *   grad_w same layout as w, out, or NULL to skip
 * All in the plan's dtype (gradients are rounded to it from fp32), 16-byte
 * aligned; outputs must not overlap any other argument. INVALID_ARG when
 * both outputs are NULL or an input an output needs is NULL, or on a plan of
 * the other ndim; UNSUPPORTED when ceil(c_in/32) * ceil(c_out/32) exceeds
 * 65535 (grad_w) or that product times ceil(K/8) (grad_w) or times K
 * (grad_x) exceeds 2^31 - 1, K the retained modes. Uses the plan's workspace (one call in flight per plan,
 * forward or backward); asynchronous on `stream`; allocates nothing. */
fno_status_t fno_spectral_conv2d_backward(fno_plan_t plan, const void *x,
                                          const void *w, const void *grad_y,
                                          void *grad_x, void *grad_w,
                                          void *stream);

/* 3D backward (3D plan only); as fno_spectral_conv2d_backward with the 3D
 * layouts and gamma taken from the kz index. */
fno_status_t fno_spectral_conv3d_backward(fno_plan_t plan, const void *x,
                                          const void *w, const void *grad_y,
                                          void *grad_x, void *grad_w,
                                          void *stream);

/* Saved spectra for the backward pass (TurboFNO write-up, section 4.3: the
 * layer as an autograd Function, whose forward keeps what its backward
 * needs). grad_w needs the retained spectra of x, not x itself: a forward
 * that leaves them in a caller-owned buffer spares the backward the
 * transforms of x (a full read of x) and lets a training step keep
 * B * c_in * K complex modes instead of x.
 *
 * fno_plan_saved_bytes: bytes of that buffer, in *bytes: the spectra of x in
 * the exchange format of the plan's backward (complex fp32, or fp16 pairs
 * and one int exponent per (b, i) plane), each part 256-byte aligned.
 * UNSUPPORTED (and *bytes untouched) for plans whose forward and backward
 * exchange those spectra in different formats: 2D fp16 / bf16 layers on the
 * half exchange whose backward keeps complex fp32 (K not a multiple of 4, or
 * an adjoint contraction off the matrix cores). INVALID_ARG on a NULL
 * argument. */
fno_status_t fno_plan_saved_bytes(fno_plan_t plan, size_t *bytes);

/* The layer (2D or 3D by the plan) computing y as fno_spectral_conv2d / 3d
 * do, with the plan's stand-alone kernels, that also leaves the spectra of
 * x in `saved` (device, 256-byte aligned, fno_plan_saved_bytes long, owned
 * by the caller and not overlapping x, w or y). The contents are valid for
 * fno_spectral_conv_backward_saved on this plan while x is unchanged.
 * INVALID_ARG, UNSUPPORTED as fno_plan_saved_bytes and the forward;
 * asynchronous on `stream`; allocates nothing. */
fno_status_t fno_spectral_conv_forward_save(fno_plan_t plan, const void *x,
                                            const void *w, void *y,
                                            void *saved, void *stream);

/* The backward (2D or 3D by the plan) with the spectra of x read from
 * `saved`, as written by fno_spectral_conv_forward_save on this plan,
 * instead of transformed from x; otherwise as fno_spectral_conv2d_backward
 * (same results). saved may be NULL when grad_w is NULL; outputs must not
 * overlap it. INVALID_ARG also when saved is not 256-byte aligned or the
 * plan has no saved format (fno_plan_saved_bytes UNSUPPORTED). */
fno_status_t fno_spectral_conv_backward_saved(fno_plan_t plan,
                                              const void *saved,
                                              const void *w,
                                              const void *grad_y,
                                              void *grad_x, void *grad_w,
                                              void *stream);

/* Weight layouts of a PyTorch FNO module, for fno_weights_pack / _unpack.
 *
 * FNO_WEIGHTS_SPLIT: the TurboFNO write-up's form (section 2.2: a weight of
 *   shape (modes_x, modes_y, in_ch, out_ch); section 4.3: passed to the
 *   autograd Function as weight_real and weight_imag). Two real arrays,
 *   each shaped like w without its last axis: 2D [2*m1][m2][Ci][Co],
 *   3D [2*m1][2*m2][m3][Ci][Co].
 * FNO_WEIGHTS_CORNERS: one complex array per spectrum corner, channels
 *   first, stacked: 2D [2][Ci][Co][m1][m2][2] with the low kx corner first;
 *   3D [4][Ci][Co][m1][m2][m3][2] with corners (lo, lo), (hi, lo), (lo, hi),
 *   (hi, hi) in (kx, ky). (re, im) interleaved, i.e. the float view of a
 *   complex tensor; the high corner's index 0 is kx = N - m. */
typedef enum { FNO_WEIGHTS_SPLIT = 0, FNO_WEIGHTS_CORNERS = 1 } fno_weight_layout_t;

/* Copy a module's weights into the layer's w (pack) or w back out into the
 * module's layout (unpack; e.g. grad_w of the backward pass). Elements are
 * moved, never converted: all arrays are in the plan's dtype, on its device,
 * and a pack followed by an unpack returns the input bit for bit.
 *   layout  FNO_WEIGHTS_SPLIT: re and im are the two real arrays.
 *           FNO_WEIGHTS_CORNERS: re is the interleaved array, im is NULL.
 *   w       [...][Ci][Co][2] as in the forward; out for pack, in for unpack
 * Asynchronous on `stream`; allocates nothing. INVALID_ARG: NULL plan, w or
 * re; im NULL for the split layout or not NULL for the corner layout; an
 * unknown layout; a pointer not aligned to the element size; w overlapping
 * re or im (unpack: re overlapping im). */
fno_status_t fno_weights_pack(fno_plan_t plan, int layout, const void *src_re,
                              const void *src_im, void *w, void *stream);
fno_status_t fno_weights_unpack(fno_plan_t plan, int layout, const void *w,
                                void *dst_re, void *dst_im, void *stream);

/* ---- allocation-free execution ------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Runs the
 * same kernels as fno_spectral_conv2d / fno_spectral_conv3d (2D or 3D as the
 * plan says) with the same arguments, preconditions and results, but the
 * forward and contracted spectra (and, in 3D, the slab transforms) go
 * through one static device array of FNO_NOALLOC_SCRATCH_BYTES inside the
 * library instead of the plan's workspace. Calls no allocating routine.
 * Each GPU the library runs on holds its own copy of that array until the
 * process ends; every call on one GPU shares it, so calls that overlap in
 * time on one GPU (different streams, or concurrent with another thread's
 * call) race and must be ordered by the caller. Nothing in the array needs
 * to start at zero: every call writes what it reads.
 * UNSUPPORTED when the plan's exchange buffers (complex fp32, each 256-byte
 * aligned: batch*c_in*K + batch*c_out*K values, plus in 3D
 * batch*max(c_in,c_out)*X*2*m2*m3) exceed FNO_NOALLOC_SCRATCH_BYTES;
 * otherwise errors as fno_spectral_conv2d. */
#define FNO_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
fno_status_t fno_spectral_conv_noalloc(fno_plan_t plan, const void *x,
                                       const void *w, void *y, void *stream);

/* Free the plan's device memory after synchronising its device.
 * fno_plan_destroy(NULL) returns FNO_OK. Destroying a plan twice is
 * undefined. */
fno_status_t fno_plan_destroy(fno_plan_t plan);

/* Static string naming a status code. */
const char *fno_status_string(fno_status_t s);

/* ---- inspection and measurement ---------------------------------------- */

/* Bytes of device workspace the plan holds (spectra and staging). */
fno_status_t fno_plan_workspace_bytes(fno_plan_t plan, size_t *bytes);

/* Number of kernel launches one execution call queues, and the name of
 * launch `index` (0-based, in queue order; a static string). */
fno_status_t fno_plan_num_launches(fno_plan_t plan, int *n);
fno_status_t fno_plan_launch_name(fno_plan_t plan, int index,
                                  const char **name);

/* Queue only launch `index` of an execution call, with the same arguments
 * and preconditions as the full call (the launches before it must have
 * produced the workspace contents it reads). Used to time one kernel and to
 * check intermediate spectra. */
fno_status_t fno_plan_run_launch(fno_plan_t plan, int index, const void *x,
                                 const void *w, void *y, void *stream);

/* ---- launch shape --------------------------------------------------------
 * A 2D layer call runs either as three stream-ordered kernels (forward
 * planes, contraction, inverse planes) or as one persistent cooperative
 * launch whose workgroups run the same three phases joined by two grid-wide
 * barriers (TurboFNO write-up, section 3.4: FFT -> GEMM -> iFFT in one fused
 * kernel; section 5.2: the three-kernel split measured as the slower mode).
 * Both agree with the reference to the same tolerance; they split the
 * contraction's input-channel sums differently, so they are not bit for bit
 * equal. A single-launch variant exists for 2D plans with VALU planes whose
 * next_pow2(max mode) is 4, 8 or 16, or matrix-core planes with W of 64 or
 * 128 and at most 16 modes per axis, on devices with cooperative launches.
 * Every plan starts in FNO_LAUNCH_SEPARATE, which measures faster on MI355X
 * at every size the single launch exists for. Calls queued while the stream
 * is being captured into a graph always use the three kernels; backward
 * calls always do.
 *
 * FNO_LAUNCH_FUSED_STALL_TEST exists only to exercise the error path: the
 * barriers wait for one workgroup more than the grid has, every wait gives
 * up after a few hundred polls, the kernel finishes with meaningless output
 * and fno_plan_check then reports FNO_ERR_DEVICE.
 */
typedef enum {
  FNO_LAUNCH_SEPARATE = 0,
  FNO_LAUNCH_FUSED = 1,
  FNO_LAUNCH_FUSED_STALL_TEST = 2
} fno_launch_shape_t;

/* Select the launch shape of the plan's later forward calls. INVALID_ARG:
 * NULL plan or an unknown shape; UNSUPPORTED: a single-launch shape on a plan
 * without a single-launch variant. Not thread-safe against concurrent calls
 * on the same plan. */
fno_status_t fno_plan_set_launch_shape(fno_plan_t plan, int shape);
fno_status_t fno_plan_get_launch_shape(fno_plan_t plan, int *shape);

/* Wait for the plan's device to finish its queued work, then report whether
 * a single-launch call's barrier wait gave up since the last check
 * (FNO_ERR_DEVICE; the barrier state is then reset) or FNO_OK. Synchronous. */
fno_status_t fno_plan_check(fno_plan_t plan);

/* Device pointer to the plan's forward spectra (which = 0, [B][Ci][K],
 * already scaled by 1/prod(grid)) or to the contracted spectra (which = 1,
 * [B][Co][K]); K = 2*m1*m2 (2D) or 4*m1*m2*m3 (3D), modes ordered as in w.
 * Valid after a forward execution call has finished. Their format is what
 * fno_plan_spectra_format reports: 0, complex fp32; 1 (the half exchange of
 * fp16 / bf16 plans), pairs of fp16 (re, im) scaled by powers of two, the
 * exponents at which = 2 (int32 [B][Ci], one per forward plane) and
 * which = 3 (int8 [B][Co][ceil(K/4)], one per group of four contracted
 * modes); a value is the stored pair times 2^-exponent. which 2 and 3 are
 * INVALID_ARG for format 0. */
fno_status_t fno_plan_spectra(fno_plan_t plan, int which, void **ptr);
fno_status_t fno_plan_spectra_format(fno_plan_t plan, int *half);

/* ---- the full FNO2d network ---------------------------------------------
 * The layer inside its model (TurboFNO write-up, sections 1 and 4.3: the
 * fused layer drops into an FNO module): lift Linear, n_layers blocks of
 * GELU(spectral conv + 1x1 conv + bias), projection Linear -> GELU -> Linear.
 * Activations are stored in the storage dtype; sums accumulate in fp32. GELU
 * is the erf form 0.5 v (1 + erf(v / sqrt 2)). With n_layers >= 1 the lift
 * is folded into the first block: its weights are composed with the lift's
 * (spectral weights with P, the 1x1 weights with P, the bias with p through
 * both branches) and the first block runs on the feature channels, so the
 * lifted field is never stored (the same function up to rounding). Blocks
 * run as fno_block2d where the plans allow it (the spectral output is then
 * not stored either), else as fno_spectral_conv2d + fno_channel_mix. */

/* Per-pixel channel mix:
 *   y[b][o][p] = act(sum_i A[o][i] x[b][i][p] + bias[o] + add[b][o][p])
 * x [batch][c_in][pixels], A [c_out][c_in], bias [c_out] (NULL: none),
 * add [batch][c_out][pixels] (NULL: none), y [batch][c_out][pixels]; all in
 * `dtype` on the current device; act: 0 none, 1 GELU. y must not overlap x
 * or add. c_in <= 128. Asynchronous on `stream`. */
fno_status_t fno_channel_mix(const void *x, const void *A, const void *bias,
                             const void *add, void *y, int batch, int c_in,
                             int c_out, long pixels, int act,
                             fno_dtype_t dtype, void *stream);

/* Per-pixel projection:
 *   y[b][c][p] = sum_j Q2[c][j] GELU(sum_i Q1[j][i] x[b][i][p] + q1[j]) + q2[c]
 * Q1 [hidden][c_in], q1 [hidden], Q2 [c_out][hidden], q2 [c_out].
 * c_in <= 64, hidden <= 128, c_out <= 4. */
fno_status_t fno_projection(const void *x, const void *Q1, const void *q1,
                            const void *Q2, const void *q2, void *y, int batch,
                            int c_in, int hidden, int c_out, long pixels,
                            fno_dtype_t dtype, void *stream);

/* One FNO block with the spectral branch finished in its epilogue:
 *   y = act(spectral_conv2d(x, w) + bypass x + bias)
 * x [batch][c_in][H][W] and w as for fno_spectral_conv2d with this 2D plan;
 * bypass [c_out][c_in] (the block's 1x1 convolution), bias [c_out] (NULL:
 * none), y [batch][c_out][H][W], all in the plan's dtype on its device; act:
 * 0 none, 1 GELU (the erf form). The forward planes and the contraction run
 * as in fno_spectral_conv2d; the inverse transform stops after its column
 * stage (rows of fp16 values with one power-of-two scale per plane, in a
 * buffer the plan owns), and one kernel applies the row stage and the 1x1
 * convolution to the same accumulators per image row, then bias and act,
 * so the spectral branch's output is never stored (TurboFNO write-up,
 * sections 1 and 4.3 for the block; the operator-fusion page for the GEMM
 * epilogue). Supported for fp16 / bf16 2D plans on matrix-core planes
 * (H and W of 64, 128 or 256, m1 <= 32, m2 <= 32) with c_in <= 64;
 * otherwise FNO_ERR_UNSUPPORTED and nothing runs. y must
 * not overlap x or w; x, w, y 16-byte aligned. The first call allocates the
 * plan's block buffer (batch*c_out*H*32*ceil(m2/16) halves plus batch*c_out
 * bytes) unless fno_block2d_prepare already did; under stream capture that
 * allocation is refused (FNO_ERR_UNSUPPORTED), so prepare before capturing.
 * Asynchronous on `stream`; the plan's buffers serve one call at a time. */
fno_status_t fno_block2d(fno_plan_t plan, const void *x, const void *w,
                         const void *bypass, const void *bias, int act,
                         void *y, void *stream);

/* Allocate the block buffer fno_block2d needs (idempotent; synchronous). */
fno_status_t fno_block2d_prepare(fno_plan_t plan);

typedef struct fno_model2d_s *fno_model2d_t;

/* Plan of the network on [batch][in_channels][height][width] inputs with
 * `channels` hidden channels, spectral modes (m1, m2) in every block,
 * `proj_channels` hidden units in the projection, `out_channels` outputs.
 * Owns two spectral-conv plans (the first block's from in_channels, the
 * others'), with their fno_block2d buffers where the fused block serves
 * them, two activation buffers of batch*channels*height*width elements (a
 * third for the spectral output of blocks that are not fused), plus the
 * first block's folded weights. */
fno_status_t fno_model2d_create(fno_model2d_t *model, int batch, int height,
                                int width, int in_channels, int channels,
                                int n_layers, int m1, int m2,
                                int proj_channels, int out_channels,
                                fno_dtype_t dtype, int device);

/* Forward pass. features [batch][in_channels][height][width]; out
 * [batch][out_channels][height][width]; params: 2 + 3*n_layers + 4 device
 * pointers in this order: P [channels][in_channels], p [channels], then per
 * block (spectral weights as fno_spectral_conv2d's w, W [channels][channels],
 * b [channels]), then Q1 [proj][channels], q1 [proj], Q2 [out][proj],
 * q2 [out]. params itself is a host array. One call in flight per model. */
fno_status_t fno_model2d_forward(fno_model2d_t model, const void *features,
                                 const void *const *params, void *out,
                                 void *stream);

/* Replay the forward from a HIP graph (on = 1) or queue its kernels on every
 * call (on = 0, the default). With replay on, the first call, and any call
 * whose features, out or params pointers differ from the last capture's,
 * captures the forward on the model's own stream first (synchronous with
 * respect to the host only in that it builds the graph); later calls launch
 * the captured graph on `stream`. Calls queued while `stream` is itself
 * being captured always queue the kernels directly. */
fno_status_t fno_model2d_set_graph(fno_model2d_t model, int on);

/* Free the model (synchronises its device). NULL is a no-op. */
fno_status_t fno_model2d_destroy(fno_model2d_t model);

#ifdef __cplusplus
}
#endif

#endif /* FNO_H */
