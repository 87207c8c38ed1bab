// Grouped convolution with one input channel per group (depthwise, with any
// channel multiplier M/group), 1 or 2 spatial dims.
//
// The work is bandwidth-shaped: each output reads a KHxKW window of one input
// plane, and neighbouring windows overlap, so the plan is to read X from HBM
// once and write Y once (FusedConv manifest grouped_large_kernel_w4 variants:
// input windows shared across columns, several outputs per lane along W,
// fp32 accumulation seeded by the bias).  On gfx950:
//   * one workgroup = one (image, output channel, output tile); the input halo
//     of the tile is loaded with W-contiguous (coalesced) reads into LDS as
//     fp32, zero-filled outside the image;
//   * each lane owns VEC consecutive outputs of one row and walks the taps,
//     reading the window from LDS; weights sit in LDS;
//   * the epilogue (bias, residual, activation) runs in registers before a
//     single store.
#include <hip/hip_runtime.h>

#include "epilogue.h"
#include "internal.h"

namespace fc {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 4;
constexpr int kMaxTileBytes = 64 * 1024;

// LDS row pitch: covers the window of every strip, including the columns of
// the last strip past tile_w (tile_w rounded up to kVec), so no read leaves
// the tile.
__host__ __device__ inline int64_t halo_cols(const ConvParams& cp, int tw) {
  const int64_t twp = (int64_t)(tw + kVec - 1) / kVec * kVec;
  return (twp - 1) * cp.sw + (int64_t)(cp.KW - 1) * cp.dw + 1;
}

int64_t halo_bytes(const ConvParams& cp, int th, int tw) {
  const int64_t rows = (int64_t)(th - 1) * cp.sh + (int64_t)(cp.KH - 1) * cp.dh + 1;
  const int64_t cols = halo_cols(cp, tw);
  return rows * cols * 4 + (int64_t)cp.KH * cp.KW * 4;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void depthwise_kernel(const T* __restrict__ x,
                                                             const T* __restrict__ w,
                                                             const T* __restrict__ bias,
                                                             const T* z, T* y, ConvParams cp,
                                                             int tile_h, int tile_w, int tiles_h,
                                                             int tiles_w) {
  extern __shared__ float smem[];
  const int rows_in = (tile_h - 1) * cp.sh + (cp.KH - 1) * cp.dh + 1;
  const int cols_in = (int)halo_cols(cp, tile_w);
  float* tile = smem;
  float* wl = smem + rows_in * cols_in;

  int64_t b = blockIdx.x;
  const int tx = (int)(b % tiles_w);
  b /= tiles_w;
  const int ty = (int)(b % tiles_h);
  b /= tiles_h;
  const int m = (int)(b % cp.M);
  const int64_t n = b / cp.M;
  const int g = m / cp.Mg;
  const int oh0 = ty * tile_h, ow0 = tx * tile_w;
  const int ih_base = oh0 * cp.sh - cp.ph, iw_base = ow0 * cp.sw - cp.pw;

  const int ntap = cp.KH * cp.KW;
  for (int i = threadIdx.x; i < ntap; i += kThreads) wl[i] = to_f32(w[(int64_t)m * ntap + i]);

  const T* xp = x + (n * cp.C + g) * cp.in_sz;
  for (int i = threadIdx.x; i < rows_in * cols_in; i += kThreads) {
    const int r = i / cols_in, c = i - r * cols_in;
    const int ih = ih_base + r, iw = iw_base + c;
    float v = 0.0f;
    if ((unsigned)ih < (unsigned)cp.H && (unsigned)iw < (unsigned)cp.W)
      v = to_f32(xp[(int64_t)ih * cp.W + iw]);
    tile[i] = v;
  }
  __syncthreads();

  const int spr = (tile_w + kVec - 1) / kVec;  // strips per row
  const int nstrip = tile_h * spr;
  const float bv = cp.has_bias ? to_f32(bias[m]) : 0.0f;
  const int64_t ybase = (n * cp.M + m) * cp.out_sz;
  for (int s = threadIdx.x; s < nstrip; s += kThreads) {
    const int r = s / spr;
    const int c0 = (s - r * spr) * kVec;
    float acc[kVec];
#pragma unroll
    for (int v = 0; v < kVec; ++v) acc[v] = bv;
    for (int kh = 0; kh < cp.KH; ++kh) {
      const float* trow = tile + (r * cp.sh + kh * cp.dh) * cols_in + c0 * cp.sw;
      const float* wrow = wl + kh * cp.KW;
      for (int kw = 0; kw < cp.KW; ++kw) {
        const float wv = wrow[kw];
        const float* tp = trow + kw * cp.dw;
#pragma unroll
        for (int v = 0; v < kVec; ++v) acc[v] = fmaf(wv, tp[v * cp.sw], acc[v]);
      }
    }
    const int oh = oh0 + r;
    if (oh >= cp.OH) continue;
#pragma unroll
    for (int v = 0; v < kVec; ++v) {
      const int ow = ow0 + c0 + v;
      if (c0 + v >= tile_w || ow >= cp.OW) continue;
      const int64_t yi = ybase + (int64_t)oh * cp.OW + ow;
      float val = acc[v];
      if (cp.has_z) val += to_f32(z[yi]);
      y[yi] = from_f32<T>(act_apply(cp.act, val, cp.alpha, cp.beta));
    }
  }
}

template <typename T>
int launch_t(const Geometry& g, const Plan& p, const RunArgs& a) {
  const ConvParams& cp = g.cp;
  const int tiles_h = (cp.OH + p.tile_h - 1) / p.tile_h;
  const int tiles_w = (cp.OW + p.tile_w - 1) / p.tile_w;
  const int64_t blocks = cp.n * cp.M * tiles_h * tiles_w;
  const size_t shmem = (size_t)halo_bytes(cp, p.tile_h, p.tile_w);
  hipLaunchKernelGGL(depthwise_kernel<T>, dim3((unsigned)blocks), dim3(kThreads), shmem,
                     (hipStream_t)a.stream, (const T*)a.x, (const T*)a.w, (const T*)a.bias,
                     (const T*)a.z, (T*)a.y, cp, p.tile_h, p.tile_w, tiles_h, tiles_w);
  return hipPeekAtLastError() == hipSuccess ? FUSEDCONV_OK : FUSEDCONV_ERR_LAUNCH;
}

}  // namespace

bool depthwise_fits(const ConvParams& cp, int32_t& tile_h, int32_t& tile_w) {
  if (cp.Cg != 1 || cp.D != 1 || cp.KD != 1) return false;
  int tw = cp.OW < 256 ? cp.OW : 256;
  int th = 4096 / tw;
  if (th < 1) th = 1;
  if (th > cp.OH) th = cp.OH;
  while (th > 1 && halo_bytes(cp, th, tw) > kMaxTileBytes) th = (th + 1) / 2;
  while (tw > kVec && halo_bytes(cp, th, tw) > kMaxTileBytes) tw = (tw + 1) / 2;
  if (halo_bytes(cp, th, tw) > kMaxTileBytes) return false;
  const int64_t blocks = cp.n * cp.M * (int64_t)((cp.OH + th - 1) / th) * ((cp.OW + tw - 1) / tw);
  if (blocks >= ((int64_t)1 << 31)) return false;
  tile_h = th;
  tile_w = tw;
  return true;
}

int launch_depthwise(const Geometry& g, const Plan& p, const RunArgs& a) {
  return g.dtype == FUSEDCONV_F16 ? launch_t<half_t>(g, p, a) : launch_t<float>(g, p, a);
}

}  // namespace fc
