/*
 * dcn_oracle.h -- CPU oracle for the modulated deformable convolution forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  The product path never calls it and
 * shares no code, header, table or helper with it.
 *
 * What it computes (written out from the pages' definitions):
 *
 *   y[b,o,oy,ox] = bias[o] + sum_{c<Cin} sum_{k<K*K} W[o,c,i,j] * m_k * S(X[b,c], py_k, px_k)
 *      i = k / K, j = k % K            (kernel point k in row-major order)
 *      g = c / (Cin/G)                 (offset group of channel c; G = 1 by default)
 *      py_k = oy*stride - pad + i*dilation + offset[b, 2(g*K*K + k),   oy, ox]
 *      px_k = ox*stride - pad + j*dilation + offset[b, 2(g*K*K + k)+1, oy, ox]
 *      m_k  = mask[b, g*K*K + k, oy, ox]   (1 when mask is NULL: DCNv1)
 *      S(X, py, px) = sum over the four integer neighbours (yy, xx) of (py, px),
 *                     yy in {floor(py), floor(py)+1}, xx in {floor(px), floor(px)+1},
 *                     of (1-|py-yy|)*(1-|px-xx|) * X[yy, xx], where a neighbour
 *                     outside [0,H) x [0,W) contributes zero.
 *
 *   abs_terms[b,o,oy,ox] = |bias[o]| + sum_{c,k} |W[o,c,i,j] * m_k * S(...)|
 *
 * Sources:
 *  - regular grid R and the deformable-convolution equation: csdn.net tags page
 *    "可变形卷积：Deformable ConvNets", part "Deformable Convolutional Networks",
 *    section 可变形卷积 (grid R, regular-conv and deformable-conv equations);
 *  - the modulation scalar per sampling point: same page, DCNv2 section 3.2,
 *    and the DCNv2 formula on un.csdn.net/5xxxf43i9i (section 自行实现方法);
 *  - bilinear interpolation from the four neighbours: same csdn tags page,
 *    section 可变形卷积Pytorch实现, bilinear-interpolation equation (areas S1..S4);
 *  - stride / padding / dilation as in torchvision's deform_conv2d parameter
 *    table on agent.csdn.net/6a744b3d10ee7a33f2973402.html, section 2.1;
 *  - offset groups (channels split along the channel axis into G consecutive
 *    groups, each with its own offset field; 2K^2 * G offset channels): the csdn
 *    tags page, section Deformable Group; the deform_groups argument of the DCN
 *    config on 51itzy.com/kjqy/64159.html (mmdetection section).
 * Readings taken where the pages are silent or disagree: offset channel 2k is
 * the row displacement dy and 2k+1 the column displacement dx; a neighbour
 * outside the image counts as zero (no clamping); the upper neighbour is
 * floor+1 (not ceil, which would lose the sample at integer positions);
 * offsets are in input pixels, never scaled by stride or dilation; group g's
 * offsets are the 2K^2 consecutive channels starting at 2gK^2 (and its mask
 * the K^2 channels from gK^2), in the per-group order of the one-group layout.
 *
 * Arithmetic: inputs arrive as float (already rounded to the element type the
 * caller uses); every position, weight, product and sum is formed in double.
 * Positions are tested against the image with floating compares before any
 * conversion to an integer, so NaN, +-Inf and huge offsets contribute zero.
 *
 * All pointers are host pointers to contiguous row-major arrays:
 *   x[B,Cin,H,W], offset[B,2GK^2,Ho,Wo], mask[B,GK^2,Ho,Wo] or NULL,
 *   weight[Cout,Cin,K,K], bias[Cout] or NULL.
 * Return value: 0 on success, -1 on an invalid argument.
 */
#ifndef DCN_ORACLE_H
#define DCN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct oracle_desc {
  int64_t B, Cin, H, W, Cout, K, stride, pad, dilation;
  int64_t groups;   /* offset groups G (0 means 1); Cin must be a multiple of G */
} oracle_desc;

/* Ho = floor((H + 2*pad - dilation*(K-1) - 1) / stride) + 1, likewise Wo. */
int oracle_output_hw(const oracle_desc* d, int64_t* Ho, int64_t* Wo);

/* Full output grid for output channels [cout_begin, cout_end).
 * out and abs_terms are [B, cout_end-cout_begin, Ho, Wo] doubles.
 * abs_terms may be NULL.  threads <= 0 means the OpenMP default. */
int oracle_forward(const oracle_desc* d, const float* x, const float* offset,
                   const float* mask, const float* weight, const float* bias,
                   int64_t cout_begin, int64_t cout_end,
                   double* out, double* abs_terms, int threads);

/* Individual outputs: points is npts rows of (b, o, oy, ox). */
int oracle_points(const oracle_desc* d, const float* x, const float* offset,
                  const float* mask, const float* weight, const float* bias,
                  const int64_t* points, int64_t npts,
                  double* out, double* abs_terms, int threads);

/* Gradients of y with respect to every input, for an upstream gradient gy =
 * grad_out[B,Cout,Ho,Wo] (the gradient equation of the deformable convolution on
 * the csdn.net tags page "可变形卷积：Deformable ConvNets", part "Deformable
 * Convolutional Networks", section 可变形卷积 (计算梯度): the offset gradient runs
 * through the derivative of the bilinear kernel G; the rest is the chain rule
 * applied to the forward sum above):
 *
 *   Gc[b,c,k,oy,ox]   = sum_o gy[b,o,oy,ox] * W[o,c,i,j]        (gradient of one column entry)
 *   grad_bias[o]      = sum_{b,oy,ox} gy[b,o,oy,ox]
 *   grad_weight[o,c,i,j] = sum_{b,oy,ox} gy[b,o,oy,ox] * m_k * S(X[b,c], py_k, px_k)
 *   grad_mask[b,gk,oy,ox]   = sum_{c in group g} Gc * S(X[b,c], py_k, px_k)
 *   grad_offset[b,2gk,oy,ox]   = sum_{c in group g} Gc * m_k * dS/dpy
 *   grad_offset[b,2gk+1,oy,ox] = sum_{c in group g} Gc * m_k * dS/dpx
 *   grad_x[b,c,yy,xx] = sum_{k,oy,ox} Gc * m_k * (1-|py_k-yy|)*(1-|px_k-xx|)
 *                       over the samples whose neighbours include (yy, xx)
 *
 * dS/dpy = sum over the four neighbours of s_y * (1-|px-xx|) * X[yy,xx], with
 * s_y = -1 for yy = floor(py) and +1 for yy = floor(py)+1 (the derivative of the
 * tent (1-|py-yy|) on the side of yy that py lies on); likewise dS/dpx.  At an
 * integer position this is the derivative from the right, the side floor picks.
 * Neighbours outside the image contribute zero to every term.  The positions are
 * rounded to float (py_k = float(oy*stride - pad + i*dilation) + offset in one
 * float addition) because floor(py) decides which side's derivative is taken:
 * both this oracle and a float implementation then take that integer decision
 * from the same number; everything after the rounding is in double.
 *
 * Outputs are doubles in the layouts of their inputs: grad_x[B,Cin,H,W],
 * grad_offset[B,2GK^2,Ho,Wo], grad_mask[B,GK^2,Ho,Wo] (NULL if mask is NULL),
 * grad_weight[Cout,Cin,K,K], grad_bias[Cout].  Any output may be NULL (not
 * computed).  Each output element is written by one thread, so results do not
 * depend on the thread count. */
int oracle_backward(const oracle_desc* d, const float* x, const float* offset,
                    const float* mask, const float* weight, const float* grad_out,
                    double* grad_x, double* grad_offset, double* grad_mask,
                    double* grad_weight, double* grad_bias, int threads);
/* Deformable RoI pooling (the csdn.net tags page "可变形卷积：Deformable ConvNets",
 * part (i) section 4 "可变形ROI pooling" and part "Deformable Convolutional Networks",
 * section Deformable RoI Pooling; 51itzy.com/kjqy/64159.html section 二; the DCNv2
 * modulated form on the tags page, section 3.2).  The RoI is split into k x k bins;
 * each bin is shifted by its own offset, normalised by the RoI's size, and pooled
 * by averaging bilinear samples (zero outside the image):
 *
 *   y[r,c,i,j] = m[r,i,j] / S^2 * sum_{u,v < S} S(X[b_r, c], py, px)
 *     x1 = rois[r,1]*scale, y1 = rois[r,2]*scale, w = (rois[r,3]-rois[r,1])*scale,
 *     h = (rois[r,4]-rois[r,2])*scale, b_r = rois[r,0]
 *     py = y1 + (i + (u + 0.5)/S) * h/k + gamma * h * offset[r,0,i,j]
 *     px = x1 + (j + (v + 0.5)/S) * w/k + gamma * w * offset[r,1,i,j]
 *     m  = mask[r,i,j], or 1 when mask is NULL
 * Readings where the formulas are missing from the pages: the bin's pixels are an
 * S x S grid of sample points at the centres of equal sub-cells (n_ij = S^2); RoI
 * coordinates are continuous, pixel (y, x) sits at the integer position (y, x) as in
 * the convolution, and no +1 is added to the RoI size; offset channel 0 is the row
 * displacement; the mask scales the bin's average.
 * x[B,C,H,W], rois[R,5] (float), offset[R,2,k,k] or NULL, mask[R,k,k] or NULL,
 * out[R,C,k,k] doubles.  A RoI whose batch index is outside [0, B) gives zeros.
 * abs_out[R,C,k,k] (may be NULL): the sum of the |terms| of each output,
 * |m| / S^2 * sum over the samples and their corners of |corner weight * value|,
 * the denominator of the per-element parity rule. */
typedef struct oracle_roi_desc {
  int64_t B, C, H, W, R, k, S;
  double spatial_scale, gamma;
} oracle_roi_desc;
int oracle_roi_pool(const oracle_roi_desc* d, const float* x, const float* rois, const float* offset,
                    const float* mask, double* out, double* abs_out, int threads);
/* Deformable position-sensitive RoI pooling (the csdn.net tags page "可变形卷积：
 * Deformable ConvNets", part "Deformable Convolutional Networks", section Deformable
 * RoI Pooling: a learnable offset per bin combined with ordinary position-sensitive RoI
 * pooling).  The pages do not spell out position-sensitive pooling; the reading taken
 * is the usual one: the input holds k*k score maps per output channel, and bin (i, j)
 * of output channel c pools only its own map, input channel (c*k + i)*k + j.  Bins,
 * sub-cell samples, offsets (normalised by the RoI size and scaled by gamma) and the
 * modulation scalar are exactly those of oracle_roi_pool.  Offsets may be given per
 * group of output channels ("per class"): the C output channels split into G
 * consecutive groups of C/G, group g using offset channels 2g (rows) and 2g+1
 * (columns); G = 1 shares one offset per bin.
 *
 *   y[r,c,i,j] = m[r,i,j] / S^2 * sum_{u,v < S} S(X[b_r, (c*k + i)*k + j], py, px)
 *     py, px as for oracle_roi_pool with offset[r, 2g + {0, 1}, i, j], g = c / (C/G)
 *
 * x[B, C*k*k, H, W], rois[R,5], offset[R, 2G, k, k] or NULL, mask[R,k,k] or NULL,
 * out[R,C,k,k] and abs_out[R,C,k,k] (may be NULL; as for oracle_roi_pool) doubles. */
typedef struct oracle_ps_roi_desc {
  int64_t B, C, H, W, R, k, S, G;   /* C output channels; x has C*k*k; G offset groups (0 means 1) */
  double spatial_scale, gamma;
} oracle_ps_roi_desc;
int oracle_ps_roi_pool(const oracle_ps_roi_desc* d, const float* x, const float* rois, const float* offset,
                       const float* mask, double* out, double* abs_out, int threads);
/* Number of threads an oracle_forward call with this request would use. */
int oracle_threads(int threads);

#ifdef __cplusplus
}
#endif

#endif
