// dcn_oracle.cpp -- plain CPU oracle for the modulated deformable convolution
// forward.  TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and
// the bench's CPU-baseline leg, never by the product path.
//
// The definition is stated in dcn_oracle.h.  This file writes it out as a
// plain loop over (b, cout, oy, ox, cin, k) with the bilinear sample spelled
// out in the innermost step, in double precision, with no blocking, caching
// or reordering.  OpenMP splits the outermost (b, cout) pairs across threads;
// each output element is produced by exactly one thread, so the result does
// not depend on the thread count.

#include "dcn_oracle.h"

#include <cmath>
#include <cstddef>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

bool valid_desc(const oracle_desc* d) {
  if (d == nullptr) return false;
  if (d->B < 0 || d->Cout < 0) return false;
  if (d->Cin < 1 || d->H < 1 || d->W < 1 || d->K < 1) return false;
  if (d->stride < 1 || d->dilation < 1 || d->pad < 0) return false;
  if (d->groups < 0 || (d->groups > 1 && d->Cin % d->groups != 0)) return false;
  return true;
}

// Output size of a strided, padded, dilated window (torchvision's
// deform_conv2d parameter table: stride, padding and dilation act as in a
// regular convolution).
int64_t out_size(int64_t in, int64_t K, int64_t stride, int64_t pad, int64_t dil) {
  const int64_t span = in + 2 * pad - dil * (K - 1) - 1;
  if (span < 0) return 0;
  return span / stride + 1;
}

// Value of one input plane at the fractional position (py, px): the four
// integer neighbours, each weighted by (1-|py-yy|)*(1-|px-xx|) (the areas of
// the bilinear-interpolation equation), a neighbour outside the plane
// counting as zero.  Returns the sample; inside tests use floating compares
// before any integer conversion, so NaN and infinite positions give zero.  When
// abs_sum is not null, the sum of the |weight * value| of the corners is added to it.
double bilinear_zero_outside(const float* plane, int64_t H, int64_t W, double py, double px,
                             double* abs_sum = nullptr) {
  const double y0 = std::floor(py);
  const double x0 = std::floor(px);
  double acc = 0.0;
  for (int dy = 0; dy < 2; ++dy) {
    const double yy = y0 + dy;
    if (!(yy >= 0.0 && yy <= static_cast<double>(H - 1))) continue;
    for (int dx = 0; dx < 2; ++dx) {
      const double xx = x0 + dx;
      if (!(xx >= 0.0 && xx <= static_cast<double>(W - 1))) continue;
      const double g = (1.0 - std::fabs(py - yy)) * (1.0 - std::fabs(px - xx));
      const int64_t iy = static_cast<int64_t>(yy);
      const int64_t ix = static_cast<int64_t>(xx);
      const double t = g * static_cast<double>(plane[iy * W + ix]);
      acc += t;
      if (abs_sum != nullptr) *abs_sum += std::fabs(t);
    }
  }
  return acc;
}

// One output element y[b,o,oy,ox] and its sum of |terms|.
void one_output(const oracle_desc* d, int64_t Ho, int64_t Wo, const float* x,
                const float* offset, const float* mask, const float* weight,
                const float* bias, int64_t b, int64_t o, int64_t oy, int64_t ox,
                double* y_out, double* abs_out) {
  const int64_t K = d->K, KK = K * K;
  const int64_t G = d->groups > 1 ? d->groups : 1, Cg = d->Cin / G;
  double y = 0.0, a = 0.0;
  if (bias != nullptr) {
    y = static_cast<double>(bias[o]);
    a = std::fabs(y);
  }
  for (int64_t c = 0; c < d->Cin; ++c) {
    const float* plane = x + ((b * d->Cin + c) * d->H) * d->W;
    const int64_t g = c / Cg;   // offset group of this channel
    for (int64_t k = 0; k < KK; ++k) {
      const int64_t i = k / K, j = k % K;
      const int64_t gk = g * KK + k;   // (group, kernel point) index of the offset and mask fields
      const double dy = offset[((b * 2 * KK * G + 2 * gk) * Ho + oy) * Wo + ox];
      const double dx = offset[((b * 2 * KK * G + 2 * gk + 1) * Ho + oy) * Wo + ox];
      const double py = static_cast<double>(oy * d->stride - d->pad + i * d->dilation) + dy;
      const double px = static_cast<double>(ox * d->stride - d->pad + j * d->dilation) + dx;
      const double m = (mask != nullptr) ? static_cast<double>(mask[((b * KK * G + gk) * Ho + oy) * Wo + ox]) : 1.0;
      const double w = weight[((o * d->Cin + c) * K + i) * K + j];
      const double term = w * m * bilinear_zero_outside(plane, d->H, d->W, py, px);
      y += term;
      a += std::fabs(term);
    }
  }
  *y_out = y;
  if (abs_out != nullptr) *abs_out = a;
}

// The sample S at a float position, its derivatives along py and px, and the
// four neighbours with their weights (1-|py-yy|)*(1-|px-xx|); neighbours outside
// the plane have inside = false and contribute nothing.
struct SampleGrad {
  double s, dsy, dsx;
  int64_t iy[4], ix[4];
  double g[4];
  bool inside[4];
};

SampleGrad sample_grad(const float* plane, int64_t H, int64_t W, double py, double px) {
  SampleGrad r{};
  const double y0 = std::floor(py), x0 = std::floor(px);
  for (int n = 0; n < 4; ++n) {
    const int dy = n >> 1, dx = n & 1;
    const double yy = y0 + dy, xx = x0 + dx;
    r.inside[n] = yy >= 0.0 && yy <= static_cast<double>(H - 1) && xx >= 0.0 && xx <= static_cast<double>(W - 1);
    if (!r.inside[n]) continue;
    r.iy[n] = static_cast<int64_t>(yy);
    r.ix[n] = static_cast<int64_t>(xx);
    const double ty = 1.0 - std::fabs(py - yy), tx = 1.0 - std::fabs(px - xx);
    const double v = static_cast<double>(plane[r.iy[n] * W + r.ix[n]]);
    r.g[n] = ty * tx;
    r.s += ty * tx * v;
    r.dsy += (dy == 0 ? -1.0 : 1.0) * tx * v;
    r.dsx += (dx == 0 ? -1.0 : 1.0) * ty * v;
  }
  return r;
}

// Sampling position of kernel point (i, j) at output (oy, ox), rounded to float.
void position_f(const oracle_desc* d, const float* offset, int64_t Ho, int64_t Wo, int64_t b, int64_t gk,
                int64_t i, int64_t j, int64_t oy, int64_t ox, double* py, double* px) {
  const int64_t KKG = d->K * d->K * (d->groups > 1 ? d->groups : 1);
  const float dy = offset[((b * 2 * KKG + 2 * gk) * Ho + oy) * Wo + ox];
  const float dx = offset[((b * 2 * KKG + 2 * gk + 1) * Ho + oy) * Wo + ox];
  const float fy = static_cast<float>(oy * d->stride - d->pad + i * d->dilation) + dy;
  const float fx = static_cast<float>(ox * d->stride - d->pad + j * d->dilation) + dx;
  *py = static_cast<double>(fy);
  *px = static_cast<double>(fx);
}

}  // namespace

extern "C" int oracle_backward(const oracle_desc* d, const float* x, const float* offset, const float* mask,
                               const float* weight, const float* grad_out, double* grad_x, double* grad_offset,
                               double* grad_mask, double* grad_weight, double* grad_bias, int threads) {
  if (!valid_desc(d) || x == nullptr || offset == nullptr || weight == nullptr || grad_out == nullptr) return -1;
  int64_t Ho = 0, Wo = 0;
  if (oracle_output_hw(d, &Ho, &Wo) != 0) return -1;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
  const int64_t B = d->B, Cin = d->Cin, H = d->H, W = d->W, Cout = d->Cout, K = d->K, KK = K * K;
  const int64_t G = d->groups > 1 ? d->groups : 1, Cg = Cin / G, HoWo = Ho * Wo;
  // gradient of the column entry (b, c, k) at output pixel pix
  auto col_grad = [&](int64_t b, int64_t c, int64_t k, int64_t pix) {
    double acc = 0.0;
    for (int64_t o = 0; o < Cout; ++o)
      acc += static_cast<double>(grad_out[(b * Cout + o) * HoWo + pix]) * static_cast<double>(weight[(o * Cin + c) * KK + k]);
    return acc;
  };
  auto mask_of = [&](int64_t b, int64_t gk, int64_t pix) {
    return mask != nullptr ? static_cast<double>(mask[(b * KK * G + gk) * HoWo + pix]) : 1.0;
  };
  if (grad_x != nullptr) {
    // one (b, c) plane per iteration: every write goes to that plane
#pragma omp parallel for schedule(dynamic)
    for (int64_t bc = 0; bc < B * Cin; ++bc) {
      const int64_t b = bc / Cin, c = bc % Cin, g = c / Cg;
      double* gx = grad_x + bc * H * W;
      const float* plane = x + bc * H * W;
      for (int64_t e = 0; e < H * W; ++e) gx[e] = 0.0;
      for (int64_t k = 0; k < KK; ++k)
        for (int64_t oy = 0; oy < Ho; ++oy)
          for (int64_t ox = 0; ox < Wo; ++ox) {
            const int64_t pix = oy * Wo + ox;
            double py, px;
            position_f(d, offset, Ho, Wo, b, g * KK + k, k / K, k % K, oy, ox, &py, &px);
            const SampleGrad sg = sample_grad(plane, H, W, py, px);
            const double t = col_grad(b, c, k, pix) * mask_of(b, g * KK + k, pix);
            for (int n = 0; n < 4; ++n)
              if (sg.inside[n]) gx[sg.iy[n] * W + sg.ix[n]] += t * sg.g[n];
          }
    }
  }
  if (grad_offset != nullptr || (grad_mask != nullptr && mask != nullptr)) {
    // one (b, group, kernel point, pixel) per iteration: its offset pair and mask entry
#pragma omp parallel for schedule(dynamic, 64)
    for (int64_t e = 0; e < B * G * KK * HoWo; ++e) {
      const int64_t pix = e % HoWo, gk = (e / HoWo) % (G * KK), b = e / (HoWo * G * KK);
      const int64_t g = gk / KK, k = gk % KK;
      double py, px;
      position_f(d, offset, Ho, Wo, b, gk, k / K, k % K, pix / Wo, pix % Wo, &py, &px);
      const double m = mask_of(b, gk, pix);
      double gm = 0.0, goy = 0.0, gox = 0.0;
      for (int64_t c = g * Cg; c < (g + 1) * Cg; ++c) {
        const SampleGrad sg = sample_grad(x + (b * Cin + c) * H * W, H, W, py, px);
        const double gc = col_grad(b, c, k, pix);
        gm += gc * sg.s;
        goy += gc * m * sg.dsy;
        gox += gc * m * sg.dsx;
      }
      if (grad_offset != nullptr) {
        grad_offset[(b * 2 * G * KK + 2 * gk) * HoWo + pix] = goy;
        grad_offset[(b * 2 * G * KK + 2 * gk + 1) * HoWo + pix] = gox;
      }
      if (grad_mask != nullptr && mask != nullptr) grad_mask[(b * G * KK + gk) * HoWo + pix] = gm;
    }
  }
  if (grad_weight != nullptr) {
    // one (o, c) pair per iteration: its K*K weights
#pragma omp parallel for schedule(dynamic)
    for (int64_t oc = 0; oc < Cout * Cin; ++oc) {
      const int64_t o = oc / Cin, c = oc % Cin, g = c / Cg;
      for (int64_t k = 0; k < KK; ++k) {
        double acc = 0.0;
        for (int64_t b = 0; b < B; ++b)
          for (int64_t pix = 0; pix < HoWo; ++pix) {
            double py, px;
            position_f(d, offset, Ho, Wo, b, g * KK + k, k / K, k % K, pix / Wo, pix % Wo, &py, &px);
            const SampleGrad sg = sample_grad(x + (b * Cin + c) * H * W, H, W, py, px);
            acc += static_cast<double>(grad_out[(b * Cout + o) * HoWo + pix]) * mask_of(b, g * KK + k, pix) * sg.s;
          }
        grad_weight[oc * KK + k] = acc;
      }
    }
  }
  if (grad_bias != nullptr) {
    for (int64_t o = 0; o < Cout; ++o) {
      double acc = 0.0;
      for (int64_t b = 0; b < B; ++b)
        for (int64_t pix = 0; pix < HoWo; ++pix) acc += static_cast<double>(grad_out[(b * Cout + o) * HoWo + pix]);
      grad_bias[o] = acc;
    }
  }
  return 0;
}

extern "C" int oracle_roi_pool(const oracle_roi_desc* d, const float* x, const float* rois, const float* offset,
                               const float* mask, double* out, double* abs_out, int threads) {
  if (d == nullptr || x == nullptr || rois == nullptr || out == nullptr) return -1;
  if (d->B < 1 || d->C < 1 || d->H < 1 || d->W < 1 || d->R < 0 || d->k < 1 || d->S < 1) return -1;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
  const int64_t k = d->k, S = d->S, C = d->C;
  // one (RoI, channel) pair per iteration: its k x k outputs
#pragma omp parallel for schedule(dynamic)
  for (int64_t rc = 0; rc < d->R * C; ++rc) {
    const int64_t r = rc / C, c = rc % C;
    const float* roi = rois + r * 5;
    const double bi = static_cast<double>(roi[0]);
    const double x1 = static_cast<double>(roi[1]) * d->spatial_scale, y1 = static_cast<double>(roi[2]) * d->spatial_scale;
    const double w = (static_cast<double>(roi[3]) - static_cast<double>(roi[1])) * d->spatial_scale;
    const double h = (static_cast<double>(roi[4]) - static_cast<double>(roi[2])) * d->spatial_scale;
    const bool batch_ok = bi >= 0.0 && bi < static_cast<double>(d->B);
    const int64_t b = batch_ok ? static_cast<int64_t>(bi) : 0;
    const float* plane = x + (b * C + c) * d->H * d->W;
    for (int64_t i = 0; i < k; ++i)
      for (int64_t j = 0; j < k; ++j) {
        double* y = out + (rc * k + i) * k + j;
        double* ya = abs_out != nullptr ? abs_out + (rc * k + i) * k + j : nullptr;
        if (ya != nullptr) *ya = 0.0;
        if (!batch_ok) {
          *y = 0.0;
          continue;
        }
        const double dy = offset != nullptr ? d->gamma * h * static_cast<double>(offset[((r * 2 + 0) * k + i) * k + j]) : 0.0;
        const double dx = offset != nullptr ? d->gamma * w * static_cast<double>(offset[((r * 2 + 1) * k + i) * k + j]) : 0.0;
        const double m = mask != nullptr ? static_cast<double>(mask[(r * k + i) * k + j]) : 1.0;
        double acc = 0.0, acc_abs = 0.0;
        for (int64_t u = 0; u < S; ++u)
          for (int64_t v = 0; v < S; ++v) {
            const double py = y1 + (static_cast<double>(i) + (static_cast<double>(u) + 0.5) / static_cast<double>(S)) * h / static_cast<double>(k) + dy;
            const double px = x1 + (static_cast<double>(j) + (static_cast<double>(v) + 0.5) / static_cast<double>(S)) * w / static_cast<double>(k) + dx;
            acc += bilinear_zero_outside(plane, d->H, d->W, py, px, &acc_abs);
          }
        *y = m * acc / static_cast<double>(S * S);
        if (ya != nullptr) *ya = std::fabs(m) * acc_abs / static_cast<double>(S * S);
      }
  }
  return 0;
}

extern "C" int oracle_ps_roi_pool(const oracle_ps_roi_desc* d, const float* x, const float* rois,
                                  const float* offset, const float* mask, double* out, double* abs_out,
                                  int threads) {
  if (d == nullptr || x == nullptr || rois == nullptr || out == nullptr) return -1;
  if (d->B < 1 || d->C < 1 || d->H < 1 || d->W < 1 || d->R < 0 || d->k < 1 || d->S < 1 || d->G < 0) return -1;
  const int64_t G = d->G > 1 ? d->G : 1;
  if (d->C % G != 0) return -1;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif
  const int64_t k = d->k, S = d->S, C = d->C, Cin = C * k * k, Cg = C / G;
  // one (RoI, output channel) pair per iteration: its k x k outputs
#pragma omp parallel for schedule(dynamic)
  for (int64_t rc = 0; rc < d->R * C; ++rc) {
    const int64_t r = rc / C, c = rc % C, g = c / Cg;
    const float* roi = rois + r * 5;
    const double bi = static_cast<double>(roi[0]);
    const double x1 = static_cast<double>(roi[1]) * d->spatial_scale, y1 = static_cast<double>(roi[2]) * d->spatial_scale;
    const double w = (static_cast<double>(roi[3]) - static_cast<double>(roi[1])) * d->spatial_scale;
    const double h = (static_cast<double>(roi[4]) - static_cast<double>(roi[2])) * d->spatial_scale;
    const bool batch_ok = bi >= 0.0 && bi < static_cast<double>(d->B);
    const int64_t b = batch_ok ? static_cast<int64_t>(bi) : 0;
    for (int64_t i = 0; i < k; ++i)
      for (int64_t j = 0; j < k; ++j) {
        double* y = out + (rc * k + i) * k + j;
        double* ya = abs_out != nullptr ? abs_out + (rc * k + i) * k + j : nullptr;
        *y = 0.0;
        if (ya != nullptr) *ya = 0.0;
        if (!batch_ok) continue;
        // the bin's own score map
        const int64_t ch = (c * k + i) * k + j;
        const float* plane = x + (b * Cin + ch) * d->H * d->W;
        const double dy = offset != nullptr ? d->gamma * h * static_cast<double>(offset[((r * 2 * G + 2 * g) * k + i) * k + j]) : 0.0;
        const double dx = offset != nullptr ? d->gamma * w * static_cast<double>(offset[((r * 2 * G + 2 * g + 1) * k + i) * k + j]) : 0.0;
        const double m = mask != nullptr ? static_cast<double>(mask[(r * k + i) * k + j]) : 1.0;
        double acc = 0.0, acc_abs = 0.0;
        for (int64_t u = 0; u < S; ++u)
          for (int64_t v = 0; v < S; ++v) {
            const double py = y1 + (static_cast<double>(i) + (static_cast<double>(u) + 0.5) / static_cast<double>(S)) * h / static_cast<double>(k) + dy;
            const double px = x1 + (static_cast<double>(j) + (static_cast<double>(v) + 0.5) / static_cast<double>(S)) * w / static_cast<double>(k) + dx;
            acc += bilinear_zero_outside(plane, d->H, d->W, py, px, &acc_abs);
          }
        *y = m * acc / static_cast<double>(S * S);
        if (ya != nullptr) *ya = std::fabs(m) * acc_abs / static_cast<double>(S * S);
      }
  }
  return 0;
}

extern "C" int oracle_output_hw(const oracle_desc* d, int64_t* Ho, int64_t* Wo) {
  if (!valid_desc(d) || Ho == nullptr || Wo == nullptr) return -1;
  const int64_t ho = out_size(d->H, d->K, d->stride, d->pad, d->dilation);
  const int64_t wo = out_size(d->W, d->K, d->stride, d->pad, d->dilation);
  if (ho < 1 || wo < 1) return -1;
  *Ho = ho;
  *Wo = wo;
  return 0;
}

extern "C" int oracle_threads(int threads) {
#ifdef _OPENMP
  return threads > 0 ? threads : omp_get_max_threads();
#else
  (void)threads;
  return 1;
#endif
}

extern "C" int oracle_forward(const oracle_desc* d, const float* x, const float* offset,
                              const float* mask, const float* weight, const float* bias,
                              int64_t cout_begin, int64_t cout_end,
                              double* out, double* abs_terms, int threads) {
  int64_t Ho = 0, Wo = 0;
  if (oracle_output_hw(d, &Ho, &Wo) != 0) return -1;
  if (x == nullptr || offset == nullptr || weight == nullptr || out == nullptr) return -1;
  if (cout_begin < 0 || cout_end > d->Cout || cout_begin > cout_end) return -1;
  const int64_t B = d->B, nO = cout_end - cout_begin;
  const int nthreads = oracle_threads(threads);
  (void)nthreads;
#pragma omp parallel for collapse(2) schedule(dynamic, 1) num_threads(nthreads)
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t oo = 0; oo < nO; ++oo) {
      const int64_t o = cout_begin + oo;
      for (int64_t oy = 0; oy < Ho; ++oy) {
        for (int64_t ox = 0; ox < Wo; ++ox) {
          const int64_t idx = ((b * nO + oo) * Ho + oy) * Wo + ox;
          one_output(d, Ho, Wo, x, offset, mask, weight, bias, b, o, oy, ox,
                     &out[idx], abs_terms != nullptr ? &abs_terms[idx] : nullptr);
        }
      }
    }
  }
  return 0;
}

extern "C" int oracle_points(const oracle_desc* d, const float* x, const float* offset,
                             const float* mask, const float* weight, const float* bias,
                             const int64_t* points, int64_t npts,
                             double* out, double* abs_terms, int threads) {
  int64_t Ho = 0, Wo = 0;
  if (oracle_output_hw(d, &Ho, &Wo) != 0) return -1;
  if (x == nullptr || offset == nullptr || weight == nullptr || out == nullptr) return -1;
  if (npts < 0 || (npts > 0 && points == nullptr)) return -1;
  for (int64_t p = 0; p < npts; ++p) {
    const int64_t* q = points + 4 * p;
    if (q[0] < 0 || q[0] >= d->B || q[1] < 0 || q[1] >= d->Cout || q[2] < 0 || q[2] >= Ho ||
        q[3] < 0 || q[3] >= Wo)
      return -1;
  }
  const int nthreads = oracle_threads(threads);
  (void)nthreads;
#pragma omp parallel for schedule(dynamic, 16) num_threads(nthreads)
  for (int64_t p = 0; p < npts; ++p) {
    const int64_t* q = points + 4 * p;
    one_output(d, Ho, Wo, x, offset, mask, weight, bias, q[0], q[1], q[2], q[3], &out[p],
               abs_terms != nullptr ? &abs_terms[p] : nullptr);
  }
  return 0;
}
