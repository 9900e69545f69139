/*
 * dcn.h -- C ABI of the MI355X (gfx950) modulated deformable convolution forward.
 *
 * The operation (DCNv2 deform_conv2d; DCNv1 when the mask is absent): for every
 * batch b, output channel o and output pixel (oy, ox)
 *
 *   out[b,o,oy,ox] = bias[o] + sum_{c<Cin} sum_{k<K*K} weight[o,c,i,j] * m_k * S(x[b,c], py_k, px_k)
 *     i = k / K, j = k % K                       kernel point k in row-major order
 *     py_k = oy*stride - pad + i*dilation + offset[b, 2k,   oy, ox]
 *     px_k = ox*stride - pad + j*dilation + offset[b, 2k+1, oy, ox]
 *     m_k  = mask[b, k, oy, ox], or 1 when mask is NULL
 *     S    = bilinear interpolation from the four integer neighbours of (py, px);
 *            a neighbour outside [0,H) x [0,W) contributes zero
 *
 * Sources: the deformable-convolution equation over the regular grid R and the
 * bilinear-interpolation equation (csdn.net tags page "可变形卷积：Deformable
 * ConvNets", part "Deformable Convolutional Networks", sections on deformable
 * convolution and on the PyTorch implementation); the modulation scalar per
 * sampling point (same page, DCNv2 section 3.2; un.csdn.net/5xxxf43i9i, DCNv2
 * formula); the call and its parameters as torchvision's deform_conv2d takes
 * them (agent.csdn.net/6a744b3d10ee7a33f2973402.html, sections 2.1 and 2.2).
 * Offset channel 2k is the row displacement and 2k+1 the column displacement;
 * displacements are in input pixels.  A NaN or infinite displacement makes its
 * sample zero.
 *
 * Conventions for every entry point:
 *  - Tensors are dense, contiguous, row-major, in device memory of the current
 *    device, all of the element type desc->dtype:
 *      x[B,Cin,H,W], offset[B,2K^2,Ho,Wo], mask[B,K^2,Ho,Wo] or NULL,
 *      weight[Cout,Cin,K,K], bias[Cout] or NULL, out[B,Cout,Ho,Wo].
 *  - The caller owns every buffer, including the workspace.  The library keeps
 *    no per-call state and allocates nothing.  Work is queued on `stream`
 *    (asynchronous: no synchronisation, no host<->device copies); buffers must
 *    stay alive until that work completes.  Two calls that share a workspace
 *    must be ordered on one stream.
 *  - Return value: DCN_OK (0) or a negative status.  Every argument is checked
 *    on the host before any HIP call; on an error nothing is launched and out
 *    is not written.  DCN_E_HIP reports a failed kernel launch (the launch's own
 *    return code).  No C++ exception crosses this interface.
 *  - Arithmetic: positions and bilinear weights (times the mask) in fp32; bf16
 *    samples are interpolated in fp32 from their exactly widened corners and
 *    rounded to bf16 (nearest even) before the matrix product; products
 *    accumulate in fp32; out is rounded to dtype.  With at
 *    most 4 input channels and K*K in {1, 4, 9} the column stays in fp32 and is
 *    contracted on fp32 MFMA, and no workspace is needed (dcn_workspace_bytes
 *    returns 0).
 *  - Limits: every tensor (and the staged copy of x) has fewer than 2^31
 *    elements; otherwise DCN_E_UNSUPPORTED.
 *  - Variant choice: a kernel variant is picked from the descriptor.  The
 *    environment variable DCN_VARIANT=<name> (a name dcn_variant_name can
 *    return) pins it, for tile sweeps and tests; a name that does not exist, was
 *    built for the other dtype or cannot run the shape makes every call return
 *    DCN_E_UNSUPPORTED.  DCN_BOX_TILE="fn,TH,TW" restricts the box kernel's tile
 *    to 16*fn pixel slots holding TH x TW output pixels (sweeps only), and
 *    DCN_BOX_ROLES=0|1 pins its placement of consumer and producer waves on the
 *    SIMDs and DCN_BOX_PW=4 its four-producer-wave schedule where it would take
 *    eight (tests and sweeps).  Plans are cached per descriptor and the four
 *    variables' values.
 */
#ifndef DCN_H
#define DCN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum dcn_dtype { DCN_F32 = 0, DCN_BF16 = 1 };

enum dcn_status {
  DCN_OK = 0,
  DCN_E_ARG = -1,          /* NULL required pointer, a dimension out of range, Ho or Wo < 1 */
  DCN_E_UNSUPPORTED = -2,  /* dtype not built, or a tensor at or beyond 2^31 elements */
  DCN_E_WORKSPACE = -3,    /* workspace NULL or smaller than dcn_workspace_bytes() */
  DCN_E_HIP = -4,          /* a kernel launch failed (or, for dcn_forward_noalloc, the
                              device's scratch array could not be located) */
  DCN_E_SCRATCH = -5       /* dcn_forward_noalloc: the problem needs more scratch than
                              DCN_NOALLOC_SCRATCH_BYTES */
};

/* Problem descriptor.  B >= 0 and Cout >= 0 (0 means an empty output: the
 * call succeeds and launches nothing); Cin, H, W, K, stride, dilation >= 1;
 * pad >= 0.  One square kernel, one stride, one pad and one dilation for both
 * axes, as in torchvision's deform_conv2d call.
 *
 * Offset groups (the csdn.net tags page "可变形卷积：Deformable ConvNets",
 * section Deformable Group): the input channels are split into G consecutive
 * groups of Cin/G channels, and group g samples at its own offsets
 * offset[b, 2(g*K*K + k) + {0: dy, 1: dx}] and mask[b, g*K*K + k], so offset has
 * 2*G*K*K channels and mask G*K*K.  offset_groups 0 or 1 means one group (the
 * layout below).  G > 1 needs Cin % G == 0 (else DCN_E_ARG) and Cin/G a multiple
 * of 8 (bf16) or 4 (fp32) (else DCN_E_UNSUPPORTED). */
typedef struct dcn_desc {
  int64_t batch, in_channels, height, width, out_channels;
  int64_t kernel_size, stride, pad, dilation;
  int32_t dtype;          /* enum dcn_dtype */
  int32_t offset_groups;  /* G; 0 or 1 for one group */
} dcn_desc;

/* Output size of the strided, padded, dilated window (as for a regular
 * convolution; the offset and mask are given at this resolution):
 *   Ho = floor((H + 2*pad - dilation*(K-1) - 1) / stride) + 1, likewise Wo.
 * Host only.  DCN_E_ARG if desc is invalid or Ho or Wo would be < 1. */
int dcn_output_hw(const dcn_desc* desc, int64_t* out_h, int64_t* out_w);

/* Bytes of device workspace dcn_forward needs for this descriptor (a staged
 * channels-last copy of x and the weight repacked to [Cout][K^2][Cin]; 0 for
 * variants that read x and weight directly).  Host only; deterministic in the
 * descriptor.  The workspace must be 256-byte aligned. */
int dcn_workspace_bytes(const dcn_desc* desc, size_t* bytes);

/* The forward pass: out = deform_conv2d(x, offset, weight, bias, stride, pad,
 * dilation, mask).  Equivalent to dcn_stage() followed by dcn_forward_staged()
 * on the same stream with the same arguments. */
int dcn_forward(const dcn_desc* desc, const void* x, const void* offset, const void* mask,
                const void* weight, const void* bias, void* out,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* First half of dcn_forward: writes the staged copy of x and the repacked
 * weight into the workspace (the deformable im2col reads channel vectors of x
 * contiguously from it).  Launches nothing for variants with no workspace. */
int dcn_stage(const dcn_desc* desc, const void* x, const void* weight,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Second half of dcn_forward: sampling, interpolation, modulation, the matrix
 * product and the bias epilogue in one kernel, reading the workspace that
 * dcn_stage filled for the same descriptor, x and weight.  Takes the same
 * arguments as dcn_forward (x and weight are read directly by variants with
 * no workspace). */
int dcn_forward_staged(const dcn_desc* desc, const void* x, const void* offset, const void* mask,
                       const void* weight, const void* bias, void* out,
                       const void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of the device array that dcn_forward_noalloc uses as its workspace. */
#define DCN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* dcn_forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  Same arguments and
 * result as dcn_forward without the workspace: the staged copy of x and the repacked
 * weight go to a file-scope device array of DCN_NOALLOC_SCRATCH_BYTES (32 MiB) that
 * each GPU holds from the first call on it until the process ends (located once per
 * device with hipGetSymbolAddress; DCN_E_HIP if that fails).  A descriptor whose
 * dcn_workspace_bytes exceeds that size returns DCN_E_SCRATCH before any launch.
 * Calls no allocating routine.  Every call on one GPU shares that GPU's array and the
 * staging launch of each call writes every byte its fused launch reads, so nothing is
 * carried between calls; calls that overlap in time on one GPU (different streams, or
 * host threads with no ordering) race on the array and must not be issued. */
int dcn_forward_noalloc(const dcn_desc* desc, const void* x, const void* offset, const void* mask,
                        const void* weight, const void* bias, void* out, hipStream_t stream);

/* Name of the kernel variant dcn_forward runs for this descriptor (static
 * string; "invalid" if the descriptor is rejected). */
const char* dcn_variant_name(const dcn_desc* desc);

/* Human-readable description of the plan dcn_forward uses for this descriptor
 * (variant, tile shape, LDS and workspace sizes), written NUL-terminated into
 * buf (at most len bytes).  Host only.  Status as for dcn_workspace_bytes;
 * DCN_E_ARG if buf is NULL or len is 0. */
int dcn_plan_describe(const dcn_desc* desc, char* buf, size_t len);

/* The offset/mask branch of a modulated deformable convolution (csdn.net tags
 * page "可变形卷积：Deformable ConvNets", DCNv2 section 3.2: a separate regular
 * convolution of the same input at the layer's resolution, with 3K^2 outputs per
 * offset group: the first 2K^2 are the offsets, the rest go through a sigmoid and
 * are the modulation scalars).  For the deformable layer `desc` (its out_channels
 * is not used): weight_om [3*G*K*K][Cin][K][K], bias_om [3*G*K*K] or NULL, with the
 * layer's stride, pad and dilation; writes offset [B][2*G*K*K][Ho][Wo] (output
 * channels 0 .. 2GK^2-1, exactly the layout dcn_forward reads) and mask
 * [B][G*K*K][Ho][Wo] (sigmoid of channels 2GK^2 .. 3GK^2-1), in desc's dtype.
 * Device pointers; asynchronous on `stream`; the caller owns every buffer.  The
 * workspace (256-byte aligned) holds its own staged x and repacked weight_om.
 * Errors as for dcn_forward, checked before any launch (outputs untouched). */
int dcn_offset_mask_workspace_bytes(const dcn_desc* desc, size_t* bytes);
int dcn_offset_mask(const dcn_desc* desc, const void* x, const void* weight_om, const void* bias_om,
                    void* offset, void* mask, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The whole DCNv2 layer in one call: the offset/mask branch (as dcn_offset_mask) and
 * then the deformable convolution (as dcn_forward) on the offsets and mask it produced,
 * off one staged channels-last copy of x: x is staged once and both weights are
 * repacked by the same launch (the branch is a convolution of the same input feature
 * map: csdn.net tags page "可变形卷积：Deformable ConvNets", DCNv2 section 3.2).
 * Arguments as for dcn_offset_mask and dcn_forward; offset [B][2*G*K*K][Ho][Wo] and
 * mask [B][G*K*K][Ho][Wo] are written as outputs (the backward needs them) and read by
 * the convolution.  desc->out_channels is the layer's.  Workspace (256-byte aligned):
 * dcn_layer_workspace_bytes.  Where the two paths would stage x differently (for
 * example the direct kernel, which stages nothing), the two calls run one after the
 * other, each on its own part of the workspace.  Errors as for dcn_forward, all
 * checked before any launch. */
int dcn_layer_workspace_bytes(const dcn_desc* desc, size_t* bytes);
int dcn_layer_forward(const dcn_desc* desc, const void* x, const void* weight_om, const void* bias_om,
                      const void* weight, const void* bias, void* offset, void* mask, void* out,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Gradients of dcn_forward (the gradient equation of the csdn.net tags page
 * "可变形卷积：Deformable ConvNets", part "Deformable Convolutional Networks",
 * section on deformable convolution: the offset gradient runs through the
 * derivative of the bilinear kernel; the other gradients follow from the chain rule
 * through the forward sum).  For the layer `desc` and its inputs x, offset, mask
 * (NULL: DCNv1), weight as dcn_forward takes them, and grad_out [B,Cout,Ho,Wo] (the
 * gradient of a loss with respect to out), writes
 *   grad_x [B,Cin,H,W], grad_offset [B,2GK^2,Ho,Wo], grad_mask [B,GK^2,Ho,Wo],
 *   grad_weight [Cout,Cin,K,K], grad_bias [Cout]
 * in desc's dtype.  Any gradient pointer may be NULL (not computed); grad_mask is
 * ignored when mask is NULL.  Where a sampling position is an integer the offset
 * gradient is the derivative from the right.  Arithmetic: positions and bilinear
 * weights in fp32 as in the forward; the two gradient products on MFMA (bf16 data
 * with fp32 accumulation; fp32 data in fp32); the column gradients (W^T grad_out) and
 * the weight gradient's columns rounded to dtype; every other sum accumulates in fp32
 * and is rounded to dtype once.  The weight gradient's split reduction is added in a
 * fixed order; only the bias gradient's per-tile sums (atomic adds) and the terms of
 * each input pixel's gradient (ordered by atomic counters) can be summed in a
 * different order from call to call.  The
 * workspace (256-byte aligned, dcn_backward_workspace_bytes) holds a channels-last copy
 * of x, the transposed weight and grad_out, the columns, the column gradients, the
 * weight gradient's partial sums and the per-pixel lists of (sample, corner) pairs.
 * Device pointers; asynchronous on `stream`; the caller owns every buffer.  Errors as
 * for dcn_forward, checked before any launch (outputs untouched).
 * B == 0 or Cout == 0: the gradients that have elements are written as zeros. */
int dcn_backward_workspace_bytes(const dcn_desc* desc, size_t* bytes);
int dcn_backward(const dcn_desc* desc, const void* x, const void* offset, const void* mask,
                 const void* weight, const void* grad_out, void* grad_x, void* grad_offset,
                 void* grad_mask, void* grad_weight, void* grad_bias, void* workspace,
                 size_t workspace_bytes, hipStream_t stream);

/* Deformable RoI pooling (the csdn.net tags page "可变形卷积：Deformable ConvNets", part
 * (i) section 4 "可变形ROI pooling" and the DCNv2 section 3.2, and part "Deformable
 * Convolutional Networks", section Deformable RoI Pooling; 51itzy.com/kjqy/64159.html,
 * section 二).  Each RoI is split into k x k bins; bin (i, j) is shifted by its own offset,
 * normalised by the RoI's size, and pooled by averaging S x S bilinear samples at the
 * centres of equal sub-cells (a neighbour outside the image contributes zero):
 *   out[r,c,i,j] = m[r,i,j] / S^2 * sum_{u,v<S} S(x[b,c], py, px),  b = rois[r,0],
 *   py = y1 + (i + (u+0.5)/S) * h/k + gamma * h * offset[r,0,i,j],
 *   px = x1 + (j + (v+0.5)/S) * w/k + gamma * w * offset[r,1,i,j],
 *   (x1, y1) = spatial_scale * (rois[r,1], rois[r,2]),
 *   w = spatial_scale * (rois[r,3] - rois[r,1]), h = spatial_scale * (rois[r,4] - rois[r,2]),
 *   m = mask[r,i,j] (1 when mask is NULL).
 * Pixel (y, x) sits at the integer position (y, x), as in the convolution.
 * x [B,C,H,W], offset [R,2,k,k] or NULL (no shift), mask [R,k,k] or NULL, out [R,C,k,k]
 * in desc->dtype; rois [R,5] is always float32 (batch index, x1, y1, x2, y2 in image
 * coordinates).  A RoI whose batch index is not in [0, B) pools zeros.  Bilinear
 * weights and sums in fp32 (sample positions in double for fp32 data, in fp32 for
 * bf16); out rounded to dtype.  Device pointers; asynchronous on
 * `stream`.  bf16 with k <= 16 first writes a channels-last copy of x into the
 * workspace (256-byte aligned, dcn_roi_pool_workspace_bytes; 0 bytes otherwise).
 * DCN_E_ARG for an invalid descriptor or a NULL x, rois or out (R = 0 launches
 * nothing), DCN_E_UNSUPPORTED for another dtype or a tensor at or beyond 2^31
 * elements, DCN_E_WORKSPACE for a missing, short or misaligned workspace, DCN_E_HIP
 * for a failed launch; all checked before any launch. */
typedef struct dcn_roi_desc {
  int64_t batch, channels, height, width;
  int64_t num_rois;      /* R >= 0 */
  int64_t pooled_size;   /* k, 1..1024 */
  int64_t samples;       /* S, samples per bin side, 1..64 */
  float spatial_scale;   /* image -> feature coordinates */
  float gamma;           /* offset scale */
  int32_t dtype;         /* enum dcn_dtype */
  int32_t reserved;      /* 0 */
} dcn_roi_desc;
int dcn_roi_pool_workspace_bytes(const dcn_roi_desc* desc, size_t* bytes);
int dcn_roi_pool(const dcn_roi_desc* desc, const void* x, const float* rois, const void* offset,
                 const void* mask, void* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static text for a status code. */
/* Deformable position-sensitive RoI pooling (the tags page above, part "Deformable
 * Convolutional Networks", section Deformable RoI Pooling: a learnable offset per bin
 * combined with ordinary position-sensitive RoI pooling).  x holds k*k score maps per
 * output channel, and bin (i, j) of output channel c pools only its own map:
 *   out[r,c,i,j] = m[r,i,j] / S^2 * sum_{u,v<S} S(x[b, (c*k + i)*k + j], py, px)
 * with b, py, px, m exactly as for dcn_roi_pool, the offset of bin (i, j) taken from
 * offset[r, 2g + {0: rows, 1: columns}, i, j] for output channel group g = c / (C/G)
 * (G = offset_groups, 0 or 1 meaning one offset per bin shared by every channel).
 * x [B, C*k*k, H, W], offset [R, 2G, k, k] or NULL, mask [R, k, k] or NULL,
 * out [R, C, k, k] in desc->dtype; rois [R, 5] float32.  bf16 with k <= 16, H*W even
 * and G = 1 or (C/G) % 8 == 0 first writes the score maps channels-last and bin-major,
 * [B][H][W][k*k][round_up(C, 8)], into the workspace (256-byte aligned,
 * dcn_ps_roi_pool_workspace_bytes; 0 bytes otherwise), so that a bin's maps of 8
 * channels are one 16-byte read; the others read x directly.  Errors as for
 * dcn_roi_pool (DCN_E_ARG also when C % G != 0), all checked before any launch. */
typedef struct dcn_ps_roi_desc {
  int64_t batch, out_channels, height, width;   /* x has out_channels * k * k channels */
  int64_t num_rois;      /* R >= 0 */
  int64_t pooled_size;   /* k, 1..1024 */
  int64_t samples;       /* S, 1..64 */
  int64_t offset_groups; /* G >= 0; out_channels % G == 0 */
  float spatial_scale;
  float gamma;
  int32_t dtype;
  int32_t reserved;      /* 0 */
} dcn_ps_roi_desc;
int dcn_ps_roi_pool_workspace_bytes(const dcn_ps_roi_desc* desc, size_t* bytes);
int dcn_ps_roi_pool(const dcn_ps_roi_desc* desc, const void* x, const float* rois, const void* offset,
                    const void* mask, void* out, void* workspace, size_t workspace_bytes, hipStream_t stream);

const char* dcn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* DCN_H */
