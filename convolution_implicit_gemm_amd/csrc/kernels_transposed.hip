// Transposed convolution, gather form (the ExecuTorch WebGPU convolution pull
// request, Implementation: the transposed kernel inverts the scatter as a
// gather and reads W un-flipped as [C, M/group, k...]): one output per lane.  Output
// y at position o of channel m (group g) receives X[n, c, i] * W[c, m', k]
// for every input channel c of group g and every kernel tap k whose input
// coordinate i = (o + pad_begin - k*dilation) / stride is an integer inside
// X -- the scatter of the adjoint convolution read backwards, so that every
// output is written once, with the fused epilogue (bias, residual,
// activation; fp32 accumulation, one rounding).  A plain kernel: it
// re-reads X for every output channel and skips the (stride - 1)/stride of
// the taps that do not land.  Transposed 2x2 convolutions with stride 2 (no
// cropping) run as a GEMM on the pointwise kernel instead.
#include <hip/hip_runtime.h>

#include "epilogue.h"
#include "internal.h"
#include "launch.h"

namespace fc {
namespace {

constexpr int kThreads = 256;

// input coordinate of output coordinate o and tap k along one axis, or -1
__device__ __forceinline__ int src_coord(int o, int k, int s, int d, int p, int n) {
  const int t = o + p - k * d;
  if (t < 0) return -1;
  const int i = t / s;
  return (i * s == t && i < n) ? i : -1;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void convt_kernel(const T* __restrict__ x,
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
    const int g = m / cp.Mg, ml = m - g * cp.Mg;
    const T* xg = x + (n * cp.C + (int64_t)g * cp.Cg) * cp.in_sz;
    // W[c][ml][taps] for c in the group
    const T* wg = w + ((int64_t)g * cp.Cg * cp.Mg + ml) * cp.taps;
    float acc = 0.0f;
    for (int kd = 0; kd < cp.KD; ++kd) {
      const int id = src_coord(od, kd, cp.sd, cp.dd, cp.pd, cp.D);
      if (id < 0) continue;
      for (int kh = 0; kh < cp.KH; ++kh) {
        const int ih = src_coord(oh, kh, cp.sh, cp.dh, cp.ph, cp.H);
        if (ih < 0) continue;
        for (int kw = 0; kw < cp.KW; ++kw) {
          const int iw = src_coord(ow, kw, cp.sw, cp.dw, cp.pw, cp.W);
          if (iw < 0) continue;
          const int64_t xi = ((int64_t)id * cp.H + ih) * cp.W + iw;
          const int tap = (kd * cp.KH + kh) * cp.KW + kw;
          for (int c = 0; c < cp.Cg; ++c)
            acc = fmaf(to_f32(xg[(int64_t)c * cp.in_sz + xi]),
                       to_f32(wg[(int64_t)c * cp.Mg * cp.taps + tap]), acc);
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
  return launch_conv(convt_kernel<T>, dim3((unsigned)blocks), dim3(kThreads), 0, a, kEdgeBoth,
                     (const T*)a.x, (const T*)a.w, (const T*)a.bias, (const T*)a.z,
                     (const T*)a.pre, (T*)a.y, cp);
}

}  // namespace

int launch_transposed(const Geometry& g, const Plan& p, const RunArgs& a) {
  if (p.tile == 1) return launch_pointwise(g, p, a);  // 2x2 stride 2: the GEMM form
  return g.dtype == FUSEDCONV_F16 ? launch<half_t>(g, a) : launch<float>(g, a);
}

}  // namespace fc
