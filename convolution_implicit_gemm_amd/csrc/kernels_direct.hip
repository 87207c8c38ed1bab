// Generic direct convolution: one output element per lane, any rank, group,
// stride, dilation and padding.  The fallback route and the plainest kernel
// of the library: it re-reads the receptive field for every output (the
// "zero cross-thread reuse" the ExecuTorch im2col-GEMM PR describes), so the
// planner only picks it where no tiled kernel applies.
#include <hip/hip_runtime.h>

#include "epilogue.h"
#include "internal.h"
#include "launch.h"

namespace fc {
namespace {

constexpr int kThreads = 256;

template <typename T>
__global__ __launch_bounds__(kThreads) void direct_kernel(const T* __restrict__ x,
                                                          const T* __restrict__ w,
                                                          const T* __restrict__ bias,
                                                          const T* z, const T* pre, T* y,
                                                          ConvParams cp) {
  const int64_t total = cp.n * cp.M * cp.out_sz;
  const int64_t step = (int64_t)gridDim.x * kThreads;
  for (int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x; idx < total; idx += step) {
    const int64_t o = idx % cp.out_sz;
    const int64_t nm = idx / cp.out_sz;
    const int m = (int)(nm % cp.M);
    const int64_t n = nm / cp.M;
    const int ow = (int)(o % cp.OW);
    const int64_t t = o / cp.OW;
    const int oh = (int)(t % cp.OH);
    const int od = (int)(t / cp.OH);
    const int g = m / cp.Mg;
    const T* xg = x + (n * cp.C + (int64_t)g * cp.Cg) * cp.in_sz;
    const T* wm = w + (int64_t)m * cp.K;
    const int id0 = od * cp.sd - cp.pd, ih0 = oh * cp.sh - cp.ph, iw0 = ow * cp.sw - cp.pw;
    float acc = 0.0f;
    for (int c = 0; c < cp.Cg; ++c) {
      const T* xc = xg + (int64_t)c * cp.in_sz;
      const T* wc = wm + (int64_t)c * cp.taps;
      for (int kd = 0; kd < cp.KD; ++kd) {
        const int id = id0 + kd * cp.dd;
        if ((unsigned)id >= (unsigned)cp.D) continue;
        for (int kh = 0; kh < cp.KH; ++kh) {
          const int ih = ih0 + kh * cp.dh;
          if ((unsigned)ih >= (unsigned)cp.H) continue;
          const T* xr = xc + ((int64_t)id * cp.H + ih) * cp.W;
          const T* wr = wc + (kd * cp.KH + kh) * cp.KW;
          for (int kw = 0; kw < cp.KW; ++kw) {
            const int iw = iw0 + kw * cp.dw;
            if ((unsigned)iw >= (unsigned)cp.W) continue;
            acc = fmaf(to_f32(xr[iw]), to_f32(wr[kw]), acc);
          }
        }
      }
    }
    y[idx] = epilogue<T>(acc, m, idx, cp, bias, z, pre);
  }
}

template <typename T>
int launch(const Geometry& g, const RunArgs& a) {
  const ConvParams& cp = g.cp;
  const int64_t total = cp.n * cp.M * cp.out_sz;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > (1 << 22)) blocks = 1 << 22;
  return launch_conv(direct_kernel<T>, dim3((unsigned)blocks), dim3(kThreads), 0, a, kEdgeBoth,
                     (const T*)a.x, (const T*)a.w, (const T*)a.bias, (const T*)a.z,
                     (const T*)a.pre, (T*)a.y, cp);
}

}  // namespace

int launch_direct(const Geometry& g, const Plan&, const RunArgs& a) {
  return g.dtype == FUSEDCONV_F16 ? launch<half_t>(g, a) : launch<float>(g, a);
}

}  // namespace fc
