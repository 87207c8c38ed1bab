/*
 * fusedconv.h -- C ABI of the MI355X (gfx950) FusedConv library.
 *
 * FusedConv computes, for 1 to 3 spatial dimensions in NCHW / NCDHW layout,
 *
 *     Y = act(conv(X, W; strides, pads or auto_pad, dilations, group) + B + Z)
 *
 * (FusedConv README, "Description", "Inputs", "Outputs", "Attributes";
 * FusedConv manifest.json, "inputs", "outputs", "attributes",
 * "attributeConstraints", "typeConstraints").  B (bias, one value per output
 * channel) and Z (residual, same shape as Y) are optional; both are added
 * before the activation.  The convolution is a cross-correlation: output o
 * reads input o*stride - pad_begin + tap*dilation on every axis, and input
 * coordinates outside the tensor read as zero.  Output channel m reads input
 * channels [g*C/group, (g+1)*C/group) with g = m / (M/group).  Accumulation
 * is fp32 for both element types; an fp16 result is rounded once
 * (round-to-nearest-even) when stored.
 *
 * Lifecycle: fill a fusedconv_desc (start from fusedconv_desc_init), call
 * fusedconv_create -- it validates everything on the host, touches no device
 * and allocates no device memory -- then call fusedconv_run any number of
 * times with device pointers, and finally fusedconv_destroy.
 *
 * Errors: every function returns FUSEDCONV_OK (0) or a negative
 * FUSEDCONV_ERR_* code; nothing is thrown across the boundary.  A failing
 * call leaves a description in fusedconv_last_error() (per thread).  All
 * checks except FUSEDCONV_ERR_LAUNCH happen before any kernel is launched.
 */
#ifndef FUSEDCONV_H
#define FUSEDCONV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FUSEDCONV_MAX_RANK 8

/* Element type T, shared by X, W, B, Z and Y (manifest "typeConstraints"). */
typedef enum fusedconv_dtype {
  FUSEDCONV_F32 = 0,
  FUSEDCONV_F16 = 1
} fusedconv_dtype;

/*
 * Kernel route.  AUTO lets the planner choose; the others force one route
 * (used by tests and tuning).  A forced route that cannot run the problem
 * makes fusedconv_create fail with FUSEDCONV_ERR_ROUTE.
 *   DIRECT     one output element per lane, any problem.
 *   IGEMM      implicit GEMM on MFMA with im2col tiles gathered into LDS,
 *              any problem; supports split-K.
 *   DEPTHWISE  grouped direct kernel with one input channel per group
 *              (C/group == 1), 1 or 2 spatial dims, LDS halo tiles.
 *   IGEMM_HALO implicit GEMM on MFMA, fp16 only, whose input tile is one
 *              channel-last halo box per 32 input channels; needs
 *              C/group >= 16 and at most 64 kernel taps.
 *   SMALLC     implicit GEMM on MFMA, fp16 only, for few input channels per
 *              group (stems, patch embeddings): reduction rows of 8
 *              consecutive kernel columns read from a channel-planar input
 *              box; needs 1 or 2 spatial dims, dilation 1 along the last
 *              axis, C/group < 16 and C/group * KH * ceil(KW/8) <= 24.
 *   POINTWISE  1x1 convolution as a batched GEMM on MFMA, fp16 only (the
 *              FusedConv README's implicit GEMM with one tap, X itself the
 *              reduction operand): needs kernel 1, stride 1, no padding,
 *              C/group % 8 == 0, C/group >= 16 and a pixel count per image
 *              that is a multiple of 8.  Also 2-D 2x2 convolutions with
 *              stride 2, dilation 1 and no padding (patch embeddings,
 *              downsampling) whose W and OW are multiples of 8, with
 *              C/group even and >= 4.
 *   TRANSPOSED the route of transposed convolutions (handles made with
 *              fusedconv_create_transposed), and their only one: one output
 *              element per lane, gathering the input elements and taps that
 *              scatter into it; fp32 and fp16.  fp16 2-D 2x2 stride-2
 *              transposed convolutions with dilation 1, no leading pad, an
 *              output of exactly twice the input, W a multiple of 8 and
 *              C/group a multiple of 8 (>= 16) run instead as an MFMA GEMM
 *              (input pixels x (output channel, 2x2 phase)) with a workspace
 *              for the repacked weights.
 *   IM2COL     explicit im2col, fp16 only (the FusedConv README's
 *              im2col_gemm_tiled_reg_f16_columns variant): the column matrix
 *              [n][group][K rounded up to 8][output pixels rounded up to 8]
 *              is written into the workspace, then multiplied by W on MFMA
 *              by the POINTWISE 1x1 kernel with the fused epilogue.  Any
 *              fp16 forward problem whose output pixels per image are a
 *              multiple of 4 (ViT's 14x14 patch grid is); the planner takes
 *              it for non-overlapping patch convolutions (stride = kernel,
 *              no padding, dilation 1, kernel above 2x2), where the column
 *              matrix is a permutation of X.
 */
typedef enum fusedconv_route {
  FUSEDCONV_ROUTE_AUTO = 0,
  FUSEDCONV_ROUTE_DIRECT = 1,
  FUSEDCONV_ROUTE_IGEMM = 2,
  FUSEDCONV_ROUTE_DEPTHWISE = 3,
  FUSEDCONV_ROUTE_IGEMM_HALO = 4,
  FUSEDCONV_ROUTE_SMALLC = 5,
  FUSEDCONV_ROUTE_POINTWISE = 6,
  FUSEDCONV_ROUTE_TRANSPOSED = 7,
  FUSEDCONV_ROUTE_IM2COL = 8
} fusedconv_route;

/* Shape of one tensor.  present = 0 means the (optional) input is absent. */
typedef struct fusedconv_tensor {
  int32_t present;
  int32_t rank;
  int64_t dims[FUSEDCONV_MAX_RANK];
} fusedconv_tensor;

/*
 * Problem description.  Attribute lists are (pointer, count) pairs; a NULL
 * pointer means the attribute is absent (its default applies), a non-NULL
 * pointer means present with `count` entries, which must match the spatial
 * rank (manifest derive kernelShapeLengthOk, stridesLengthOk,
 * dilationsLengthOk, padsLengthOk).  The library copies everything it needs
 * during fusedconv_create; the caller's arrays and strings need not outlive
 * that call.
 */
typedef struct fusedconv_desc {
  int32_t dtype;              /* fusedconv_dtype */
  fusedconv_tensor x;         /* (N, C, D1..Dn), n = 1..3, required */
  fusedconv_tensor w;         /* (M, C/group, k1..kn), required */
  fusedconv_tensor bias;      /* optional, rank 1, length M */
  fusedconv_tensor z;         /* optional, exactly the shape of Y */
  const char* auto_pad;       /* NULL = "NOTSET"; or SAME_UPPER, SAME_LOWER, VALID */
  int64_t group;              /* default 1 */
  const int64_t* kernel_shape; int32_t n_kernel_shape;  /* must match W if present */
  const int64_t* strides;      int32_t n_strides;       /* default all 1, values >= 1 */
  const int64_t* dilations;    int32_t n_dilations;     /* default all 1, values >= 1 */
  const int64_t* pads;         int32_t n_pads;          /* ONNX order [begins..., ends...],
                                                           values >= 0, only with NOTSET */
  const char* activation;     /* NULL = none; Relu, LeakyRelu, Sigmoid, Tanh, HardSigmoid,
                                 HardSwish, Clip, QuickGelu, Elu, Gelu, FastGelu, Softplus,
                                 ThresholdedRelu, Erf */
  const float* activation_params; int32_t n_activation_params;
                              /* LeakyRelu: exactly [alpha]; HardSigmoid: exactly [alpha, beta];
                                 Clip: exactly [min, max]; QuickGelu, Elu, ThresholdedRelu:
                                 optional [alpha] (defaults 1.702, 1.0, 1.0); Gelu: optional
                                 [approximate] (0 = erf form, nonzero = tanh form); ignored by
                                 the parameter-free activations (README "Attributes",
                                 manifest derive activationParamsOk, actAlpha, actBeta) */
  int32_t route;              /* fusedconv_route; 0 = planner's choice */
  int32_t split_k;            /* 0 = planner's choice; >= 1 forces the K split (IGEMM only) */
} fusedconv_desc;

/* Status codes.  The cited passage is the rule the check enforces. */
enum {
  FUSEDCONV_OK = 0,
  FUSEDCONV_ERR_NULL_ARG = -1,            /* a required pointer is NULL */
  FUSEDCONV_ERR_DTYPE = -2,               /* T not float32/float16 (typeConstraints) */
  FUSEDCONV_ERR_RANK = -3,                /* ranks of X/W/Y differ or spatial rank not 1..3
                                             (derive spatialAttributesOk, *RanksOk) */
  FUSEDCONV_ERR_ATTR_LENGTH = -4,         /* attribute list length (derive *LengthOk) */
  FUSEDCONV_ERR_ATTR_VALUE = -5,          /* stride/dilation < 1, pad < 0, kernel extent < 1
                                             (derive stridesValuesOk, dilationsValuesOk,
                                             padsValuesOk, kernelExtentsOk), bad auto_pad */
  FUSEDCONV_ERR_PADS_WITH_AUTO_PAD = -6,  /* pads given with an automatic mode
                                             (derive explicitPadsOk) */
  FUSEDCONV_ERR_KERNEL_SHAPE = -7,        /* kernel_shape differs from W (kernelShapeMatchesWeights) */
  FUSEDCONV_ERR_GROUP = -8,               /* group < 1, M % group, W.dim1 * group != C (groupOk) */
  FUSEDCONV_ERR_BIAS_SHAPE = -9,          /* bias not rank 1 of length M (biasOk) */
  FUSEDCONV_ERR_Z_SHAPE = -10,            /* Z shape differs from Y (zOk) */
  FUSEDCONV_ERR_ACTIVATION = -11,         /* unknown activation name (activationOk) */
  FUSEDCONV_ERR_ACTIVATION_PARAMS = -12,  /* wrong number of parameters (activationParamsOk) */
  FUSEDCONV_ERR_OUTPUT_SHAPE = -13,       /* an output dim < 1, or a zero-sized input */
  FUSEDCONV_ERR_WORKSPACE = -14,          /* workspace missing or smaller than required */
  FUSEDCONV_ERR_ALIGNMENT = -15,          /* a device pointer is not 16-byte aligned */
  FUSEDCONV_ERR_ROUTE = -16,              /* forced route / split cannot run this problem */
  FUSEDCONV_ERR_LAUNCH = -17,             /* a HIP call or kernel launch failed */
  FUSEDCONV_ERR_DEVICE = -18,             /* current device is not a gfx950 GPU */
  FUSEDCONV_ERR_ALLOC = -19,              /* host allocation of the handle failed */
  FUSEDCONV_ERR_TOO_LARGE = -20           /* a tensor exceeds the library's index limits */
};

typedef struct fusedconv_handle fusedconv_handle;  /* opaque, host memory only */

/* Fill *d with "absent" for every optional field, group = 1, dtype f32. */
void fusedconv_desc_init(fusedconv_desc* d);

/*
 * Validate and resolve the problem and plan the kernels.
 *
 * Defined by: the FusedConv manifest.json "derive" rules, which give every
 * check this call makes (spatialAttributesOk and the *RanksOk ranks; the
 * *LengthOk and *ValuesOk attribute rules; explicitPadsOk;
 * kernelShapeMatchesWeights; groupOk; biasOk; zOk; activationOk;
 * activationParamsOk) and the resolved quantities (samePad* for SAME_UPPER /
 * SAME_LOWER, expectedOutput* for the output dims, actAlpha / actBeta for
 * the activation defaults); the FusedConv README, "Attributes" table, for
 * the attribute meanings and defaults.  The plan (route, tile, K split,
 * workspace bytes) is fixed here, before any device memory exists, as the
 * ExecuTorch WebGPU conv page's im2col GEMM change computes both dispatch
 * grids before allocating any buffer, so that a rejected problem leaks
 * nothing.
 *
 * Host only: no device call, no device allocation.  d and everything it
 * points to are read during the call only.  On success *out owns a new
 * handle (release it with fusedconv_destroy); on failure *out is NULL and
 * the code names the first rule that failed (FUSEDCONV_ERR_*), with details
 * in fusedconv_last_error().
 */
int fusedconv_create(const fusedconv_desc* d, fusedconv_handle** out);

/*
 * Transposed convolution with the same fused epilogue:
 *   Y = act(convT(X, W) + B + Z),
 * convT being the adjoint of the cross-correlation fusedconv_create plans
 * (the transposed form of the aten.convolution entry point the ExecuTorch
 * conv page routes through): every X[n, c, i] adds X[n, c, i] * W[c, m, k]
 * into Y[n, g*(M/group) + m, i*stride - pad_begin + k*dilation], with
 * g = c / (C/group).  d describes X [n, C, in...], W as [C, M/group, k...],
 * B (length M = W.shape[1] * group) and Z (Y's shape), strides, dilations,
 * pads (ONNX order; they trim Y), group, activation; auto_pad must be NULL
 * or "NOTSET" and kernel_shape, if given, must match W.  output_padding:
 * n_output_padding (0 or one per spatial axis) values in [0, stride),
 * appended to Y's end; NULL with 0 means zeros.  Y's extent per axis is
 * stride*(in - 1) + output_padding + (k - 1)*dilation + 1 - pad_begin -
 * pad_end.  route must be FUSEDCONV_ROUTE_AUTO or ..._TRANSPOSED.  The
 * handle is used with every other call below exactly like one from
 * fusedconv_create.  Errors as for fusedconv_create (output_padding out of
 * range: FUSEDCONV_ERR_ATTR_VALUE; wrong count: ..._ATTR_LENGTH).
 */
int fusedconv_create_transposed(const fusedconv_desc* d, const int64_t* output_padding,
                                int32_t n_output_padding, fusedconv_handle** out);

/*
 * Y's shape, inferred from the inputs and attributes as the FusedConv README
 * says outputs are ("Use with @huggingface/kernels": output shapes are
 * inferred and result tensors allocated for the caller; "Outputs": Y has the
 * rank of X).  The spatial dims are the manifest's expectedOutput* values
 * (or, for a transposed handle, the adjoint extent stated at
 * fusedconv_create_transposed); dims[0] = N, dims[1] = M.  *rank = rank of
 * X; dims[0..rank) are filled and the rest set to 0.  The caller allocates
 * Y (and Z, which must have this shape) from it.  Errors: NULL argument.
 */
int fusedconv_output_shape(const fusedconv_handle* h, int64_t dims[FUSEDCONV_MAX_RANK],
                           int32_t* rank);

/*
 * Device workspace bytes fusedconv_run needs (0 if none).  The workspace
 * holds the intermediates the plan chose: the raw fp32 partial sums of a
 * split reduction, which the FusedConv README's split-K variants
 * ("Implementation variants": implicit_im2col_tiled_reg_splitk) write
 * before one combine applies bias and activation, laid out
 * [split][M][N * output pixels]; or a route's repacked weights (see
 * fusedconv_prepare_weights).  The caller allocates it on the device, at
 * least this size and 16-byte aligned.  Errors: NULL argument.
 */
int fusedconv_workspace_size(const fusedconv_handle* h, size_t* bytes);

/*
 * Chosen plan: route (fusedconv_route), K split factor, and a short
 * NUL-terminated kernel name written into name[0..name_len) (may be NULL).
 * The FusedConv README ("Implementation variants") selects one
 * implementation per call from the device, the shapes and the dtypes; this
 * reports which one the planner selected.  Errors: NULL handle.
 */
int fusedconv_plan_info(const fusedconv_handle* h, int32_t* route, int32_t* split_k, char* name,
                        size_t name_len);

/*
 * Compute Y = act(conv(X, W) + B + Z) (FusedConv README, "Description",
 * "Inputs" and "Outputs": B broadcast over each output channel, Z of Y's
 * shape added before the activation; the manifest's "inputs" / "outputs"
 * order x, w, bias, zResidual -> y).  Inputs and outputs are caller-owned
 * device buffers: the library, unlike the README's JavaScript entry point,
 * allocates nothing, so Y is passed in, sized by fusedconv_output_shape.
 *
 * Enqueue the computation on `stream` (a hipStream_t; NULL = the default
 * stream) and return without waiting.  x, w, y: device pointers, contiguous,
 * 16-byte aligned.  bias / z: device pointers iff the descriptor declared
 * them present, else NULL.  workspace: at least fusedconv_workspace_size()
 * bytes of device memory (may be NULL if that is 0), 16-byte aligned, owned
 * by the caller and not used by another run at the same time.  Y must not
 * overlap X, W, B or the workspace; Y may be the same buffer as Z
 * (in-place residual).  The caller owns every buffer and the stream; the
 * library allocates nothing on the device.
 */
int fusedconv_run(const fusedconv_handle* h, const void* x, const void* w, const void* bias,
                  const void* z, void* y, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Weight preparation, for callers whose W stays the same across many runs
 * (inference): fusedconv_prepare_weights enqueues only the route's weight
 * preparation (for IGEMM_HALO a repack of W into the tap-major layout held in
 * the workspace, for SMALLC a repack into rows of 8 kernel columns, for
 * POINTWISE (and the GEMM form of TRANSPOSED) a repack into MFMA fragment
 * order, for IM2COL the same after padding W's rows to a multiple of 8; a
 * no-op for the other routes), and fusedconv_run_ex with
 * FUSEDCONV_RUN_WEIGHTS_PREPARED then skips that step and reads the prepared
 * weights from the workspace.  The caller guarantees that the workspace holds
 * the prepared form of the same W, made with the same handle; otherwise the
 * result is undefined.  Arguments and errors as for fusedconv_run; flags = 0
 * makes fusedconv_run_ex identical to fusedconv_run.
 */
#define FUSEDCONV_RUN_WEIGHTS_PREPARED 1u
int fusedconv_prepare_weights(const fusedconv_handle* h, const void* w, void* workspace,
                              size_t workspace_bytes, void* stream);
int fusedconv_run_ex(const fusedconv_handle* h, const void* x, const void* w, const void* bias,
                     const void* z, void* y, void* workspace, size_t workspace_bytes,
                     unsigned flags, void* stream);

/*
 * fusedconv_run_ex, with the convolution kernels timed by the device: the
 * caller's events (hipEvent_t, made with hipEventCreate, timing not
 * disabled) are recorded by the dispatches themselves, start_event at the
 * begin of the route's first convolution kernel and stop_event at the end
 * of its last one (the K-split combine, if any), so hipEventElapsedTime of
 * the two is the kernels' own duration.  Weight preparation is outside the
 * interval.  This is the measurement hook of the throughput figures (the
 * algorithmic FLOP and bytes of one call divided by this duration); it does
 * not change what is computed.  Both events or neither (then identical to
 * fusedconv_run_ex); one alone gives FUSEDCONV_ERR_NULL_ARG.  Other
 * arguments and errors as for fusedconv_run_ex.
 */
int fusedconv_run_timed(const fusedconv_handle* h, const void* x, const void* w,
                        const void* bias, const void* z, void* y, void* workspace,
                        size_t workspace_bytes, unsigned flags, void* stream, void* start_event,
                        void* stop_event);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same as
 * fusedconv_run (weights prepared on every call), but the workspace is a
 * fixed array inside the library, FUSEDCONV_NOALLOC_SCRATCH_BYTES on each
 * GPU (held until the process ends), so the call allocates nothing and takes
 * no workspace argument.  A plan whose fusedconv_workspace_size exceeds that
 * size is refused with FUSEDCONV_ERR_WORKSPACE before anything is launched.
 * The array is shared by every call on a GPU and keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other threads)
 * race and must be serialized by the caller.  Other arguments and errors as
 * for fusedconv_run.
 */
#define FUSEDCONV_NOALLOC_SCRATCH_BYTES (8u << 20)
int fusedconv_run_noalloc(const fusedconv_handle* h, const void* x, const void* w,
                          const void* bias, const void* z, void* y, void* stream);

/*
 * Backward of the convolution, for training (the tinygrad compare page,
 * tinygrad/codegen/opt/reduce.py: direct_conv_bwd_activation_program runs a
 * 3x3 convolution's input gradient as per-tap GEMMs with the QuickGelu
 * derivative fused into the epilogue, col2im_program assembles the same
 * gradient from per-tap columns with an optional fused activation
 * derivative).  G denotes the gradient of the loss with respect to the
 * convolution's pre-activation output conv(X, W) + B + Z (the caller
 * multiplies a gradient of Y by act'(pre-activation) first, or obtains G
 * from the backward-data call of the layer above, which fuses it).
 *
 * fusedconv_create_backward_data: d describes the FORWARD convolution (x, w,
 * group, strides, dilations, pads / auto_pad, kernel_shape, dtype) with
 * these differences: d->activation and d->activation_params name the
 * activation act_in that produced X from its pre-activation P (NULL:
 * none); d->z present declares a residual gradient R with X's shape; d->bias
 * must be absent.  The handle computes
 *     dP = (conv^T(G, W) + R) * act_in'(P)
 * (conv^T the adjoint of the cross-correlation in X; fp32 accumulation, one
 * rounding; the derivative at the kinks of the piecewise activations is the
 * one-sided value: Relu 0 at 0, LeakyRelu alpha at 0, Clip 1 on [min, max],
 * HardSigmoid alpha strictly inside (0, 1), HardSwish x/3 + 1/2 strictly
 * inside (-3, 3), ThresholdedRelu 0 at alpha).  Planning: with every stride
 * 1 (and pads no larger than dilation*(k - 1)) the gradient is the forward
 * convolution of G with W transposed per group and flipped, run on the
 * IGEMM_HALO (fp16), IGEMM or DIRECT kernel with this epilogue; otherwise
 * the gather kernel of the TRANSPOSED route.  d->route: AUTO, IGEMM_HALO,
 * IGEMM, DIRECT (stride 1 only) or TRANSPOSED; d->split_k as for IGEMM.
 * fusedconv_output_shape reports X's shape, fusedconv_workspace_size the
 * workspace (the flipped W first, then the route's own).  Errors as for
 * fusedconv_create; bias present: FUSEDCONV_ERR_BIAS_SHAPE; z not of X's
 * shape: FUSEDCONV_ERR_Z_SHAPE.
 *
 * fusedconv_backward_data: dy = G (the forward Y's shape), w = W, pre = P
 * (X's shape; required when act_in is set, else ignored), dres = R (X's
 * shape; required iff declared), dx = dP (X's shape, dtype T, may not alias
 * an input).  Device pointers, 16-byte aligned; enqueued on `stream`.
 * A handle from any other create call: FUSEDCONV_ERR_ROUTE.
 */
int fusedconv_create_backward_data(const fusedconv_desc* d, fusedconv_handle** out);
int fusedconv_backward_data(const fusedconv_handle* h, const void* dy, const void* w,
                            const void* pre, const void* dres, void* dx, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * fusedconv_create_backward_weight: d describes the forward convolution as
 * for fusedconv_create; d->bias present requests the bias gradient too;
 * d->z, d->activation and its parameters are ignored.  The handle computes
 *     dW[m, c, k] = sum over n, o of G[n, m, o] * X[n, g*(C/group) + c,
 *                                                   o*stride - pad_begin + k*dilation]
 *     dB[m]       = sum over n, o of G[n, m, o]
 * in fp32 (fp32 accumulation; the fp16 products are exact).  Planning
 * (d->route): AUTO or IM2COL, the column matrix of X (with a row of ones for
 * dB) in the workspace times G on MFMA, image ranges summed by a second
 * kernel; needs the output pixels per image to be a multiple of 4; DIRECT,
 * one reduction per dW element (any problem).  fusedconv_output_shape
 * reports W's shape.
 *
 * fusedconv_backward_weight: x = X, dy = G, dw = float [M][C/group][k...],
 * db = float [M] (required iff the bias gradient was requested, else NULL).
 * Device pointers, 16-byte aligned; enqueued on `stream`.  A handle from any
 * other create call: FUSEDCONV_ERR_ROUTE.
 */
int fusedconv_create_backward_weight(const fusedconv_desc* d, fusedconv_handle** out);
int fusedconv_backward_weight(const fusedconv_handle* h, const void* x, const void* dy,
                              float* dw, float* db, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Release a handle (NULL is allowed).  Host memory only; runs already
 * enqueued with it are unaffected (the kernels received everything by value). */
void fusedconv_destroy(fusedconv_handle* h);

/* Static text for a status code. */
const char* fusedconv_status_string(int status);

/* Detail text of the calling thread's last failing call ("" if none). */
const char* fusedconv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FUSEDCONV_H */
