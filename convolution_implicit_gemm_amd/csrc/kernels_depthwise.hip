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
#include "launch.h"

namespace fc {
namespace {

constexpr int kThreads = 256;
constexpr int kVec = 4;
[[maybe_unused]] constexpr int kMaxTileBytes = 64 * 1024;

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

// ---------------------------------------------------------------------------
// fp16, stride 1, KH x KW in {3, 5, 7}, any dilation: register windows and
// v_dot2_f32_f16.
//
// Each lane owns R x VEC outputs of one plane: rows spaced by dh and columns
// spaced by dw ("dilated lanes"), so the taps kw and kw+1 of every output are
// adjacent once the LDS rows are stored split by column residue mod dw.  A
// lane reads each of its R + KH - 1 input-row windows from LDS once (8-byte
// reads), forms the odd-aligned tap pairs with one v_alignbit per word, and
// accumulates kernel-row pairs (w[kw], w[kw+1]) with v_dot2_f32_f16 (fp16
// products, fp32 sums; an odd KW pairs its last tap with a zero weight).
// Several planes share one 256-thread block.
struct DwFast {
  int r, v;             // output rows / columns per lane (template variant)
  int gr, gc;           // row / column groups per residue class
  int items;            // dh * gr * dw * gc work items per plane
  int tpp, pb;          // threads per plane, planes per block
  int rows, seg, pitch; // LDS tile: rows, halves per column class, halves per row
  int plane_halves;     // rows * pitch
};

// One plan for a given lane block kR x kV; false if it does not fit.
bool dw_fast_try(const ConvParams& cp, int kR, int kV, DwFast& f) {
  const int64_t nr = (cp.OH + cp.dh - 1) / cp.dh, nc = (cp.OW + cp.dw - 1) / cp.dw;
  f.r = kR;
  f.v = kV;
  f.gr = (int)((nr + kR - 1) / kR);
  f.gc = (int)((nc + kV - 1) / kV);
  const int64_t items = (int64_t)cp.dh * f.gr * cp.dw * f.gc;
  const int nwords = (kV + cp.KW + 2) / 2;  // words per row window
  const int64_t rows = (int64_t)(cp.dh - 1) + (int64_t)cp.dh * (kR * f.gr + cp.KH - 2) + 1;
  int64_t seg = (int64_t)kV * (f.gc - 1) + 2 * nwords;
  seg = (seg + 3) / 4 * 4;
  const int64_t pitch = seg * cp.dw;
  const int64_t plane = rows * pitch;
  if (items > (1 << 20) || plane * 2 > 32 * 1024) return false;
  // threads per plane: keep the most lanes busy; planes share the block
  double best = -1.0;
  f.tpp = 0;
  for (int tpp = 32; tpp <= 256; ++tpp) {
    const int pb = 256 / tpp;
    if (pb * plane * 2 > 64 * 1024) continue;
    const int64_t rounds = (items + tpp - 1) / tpp;
    const double util = (double)pb * tpp / 256.0 * (double)items / (double)(rounds * tpp);
    if (util > best + 1e-9) {
      best = util;
      f.tpp = tpp;
    }
  }
  if (f.tpp == 0) return false;
  f.pb = 256 / f.tpp;
  f.items = (int)items;
  f.rows = (int)rows;
  f.seg = (int)seg;
  f.pitch = (int)pitch;
  f.plane_halves = (int)plane;
  return true;
}

// Pick the lane block (rows x columns per lane) with the least padded output
// and then the larger block (fewer windows and index computations per output).
bool dw_fast_plan(const ConvParams& cp, DwFast& f) {
  if (cp.sh != 1 || cp.sw != 1 || !depth_trivial(cp)) return false;
  if (!((cp.KH == 3 || cp.KH == 5 || cp.KH == 7) && cp.KW == cp.KH)) return false;
  // 4 x 4 measured fastest on the 56 x 56 planes (4 x 8 needs ~200 registers
  // and halves occupancy; 8 x 8 does not fully unroll and spills)
  const int shapes[1][2] = {{4, 4}};
  bool found = false;
  double best = 1e30;
  for (const auto& sh : shapes) {
    DwFast c;
    if (!dw_fast_try(cp, sh[0], sh[1], c)) continue;
    const double padded = (double)c.items * c.r * c.v / ((double)cp.OH * cp.OW);
    const double cost = padded * (1.0 + 16.0 / (c.r * c.v));  // per-item overhead share
    if (cost < best - 1e-9) {
      best = cost;
      f = c;
      found = true;
    }
  }
  return found;
}

template <int KS, int kR, int kV, int ACT>
__global__ __launch_bounds__(kThreads) void dw_fast_kernel(const half_t* __restrict__ x,
                                                           const half_t* __restrict__ w,
                                                           const half_t* __restrict__ bias,
                                                           const half_t* z, half_t* y,
                                                           ConvParams cp, DwFast f) {
  constexpr int KH = KS, KW = KS;
  constexpr int NW = (kV + KW + 2) / 2;  // 32-bit words per row window
  constexpr int NP = (KW + 1) / 2;     // tap pairs per kernel row
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  extern __shared__ __attribute__((aligned(16))) half_t tile[];

  const int64_t nplanes = cp.n * cp.M;
  const int64_t plane0 = (int64_t)blockIdx.x * f.pb;

  // ---- load the halo tiles of this block's planes (zero outside the input);
  // column cl of a row is stored at (cl % dw) * seg + cl / dw
  // Zero the tiles, then copy the in-image rows: 16-byte global loads (W a
  // multiple of 8), up to kChunks per lane in flight before they are stored;
  // element at tile column cl lands at (cl % dw) * seg + cl / dw.
  {
    typedef unsigned u4 __attribute__((ext_vector_type(4)));
    const int nz = f.pb * f.plane_halves / 8;
    for (int i = threadIdx.x; i < nz; i += kThreads) ((u4*)tile)[i] = u4{0, 0, 0, 0};
  }
  __syncthreads();
  if ((cp.W & 7) == 0) {
    constexpr int kChunks = 8;
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    const int cpr = cp.W / 8;                 // 8-column chunks per input row
    const int total = f.pb * cp.H * cpr;
    for (int base = 0; base < total; base += kChunks * kThreads) {
      h8 v[kChunks];
      int at[kChunks];
#pragma unroll
      for (int k = 0; k < kChunks; ++k) {
        const int t = base + k * kThreads + threadIdx.x;
        at[k] = -1;
        v[k] = h8{};
        if (t < total) {
          const int row = t / cpr, ch = t - row * cpr;
          const int pi = row / cp.H, ih = row - pi * cp.H;
          const int64_t plane = plane0 + pi;
          if (plane < nplanes) {
            const int64_t nimg = plane / cp.M;
            const int m = (int)(plane - nimg * cp.M);
            v[k] = *(const h8*)(x + (nimg * cp.C + m / cp.Mg) * cp.in_sz + (int64_t)ih * cp.W +
                                ch * 8);
            at[k] = pi * f.plane_halves + (ih + cp.ph) * f.pitch;
          }
        }
      }
#pragma unroll
      for (int k = 0; k < kChunks; ++k) {
        if (at[k] < 0) continue;
        const int t = base + k * kThreads + threadIdx.x;
        const int ch = t % cpr;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int cl = ch * 8 + e + cp.pw;
          const int col = cp.dw == 1 ? cl : (cl % cp.dw) * f.seg + cl / cp.dw;
          tile[at[k] + col] = v[k][e];
        }
      }
    }
  } else {
    // any width: one wave per tile row, lanes along columns
    const int cols = cp.dw * f.seg;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    for (int task = wave; task < f.pb * cp.H; task += kThreads / 64) {
      const int pi = task / cp.H, ih = task - pi * cp.H;
      const int64_t plane = plane0 + pi;
      if (plane >= nplanes) continue;
      const int64_t nimg = plane / cp.M;
      const int m = (int)(plane - nimg * cp.M);
      const half_t* src = x + (nimg * cp.C + m / cp.Mg) * cp.in_sz + (int64_t)ih * cp.W;
      half_t* dst = tile + pi * f.plane_halves + (ih + cp.ph) * f.pitch;
      for (int iw = lane; iw < cp.W; iw += 64) {
        const int cl = iw + cp.pw;
        const int col = cp.dw == 1 ? cl : (cl % cp.dw) * f.seg + cl / cp.dw;
        if (cl < cols) dst[col] = src[iw];
      }
    }
  }
  __syncthreads();

  const int pi = threadIdx.x / f.tpp;
  if (pi >= f.pb) return;
  const int64_t plane = plane0 + pi;
  if (plane >= nplanes) return;
  const int64_t nimg = plane / cp.M;
  const int m = (int)(plane - nimg * cp.M);
  const half_t* tp = tile + pi * f.plane_halves;

  // kernel-row tap pairs (w[kw], w[kw+1]); the last pair of an odd KW is (w, 0)
  h2 wpair[KH][NP];
#pragma unroll
  for (int kh = 0; kh < KH; ++kh)
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const half_t a = w[(int64_t)m * KH * KW + kh * KW + 2 * p];
      const half_t b2 = (2 * p + 1 < KW) ? w[(int64_t)m * KH * KW + kh * KW + 2 * p + 1] : (half_t)0;
      wpair[kh][p] = h2{a, b2};
    }
  const float bv = cp.has_bias ? to_f32(bias[m]) : 0.0f;
  const int64_t ybase = plane * cp.out_sz;
  const int gcc = cp.dw * f.gc;  // column groups over all residue classes

  for (int it = threadIdx.x - pi * f.tpp; it < f.items; it += f.tpp) {
    const int rgi = it / gcc, cgi = it - rgi * gcc;
    const int rres = rgi / f.gr, rk = rgi - rres * f.gr;   // row class, group
    const int cres = cgi / f.gc, ck = cgi - cres * f.gc;   // column class, group
    float acc[kR][kV];
#pragma unroll
    for (int i = 0; i < kR; ++i)
#pragma unroll
      for (int j = 0; j < kV; ++j) acc[i][j] = bv;
    const half_t* rowp = tp + cres * f.seg + kV * ck;
#pragma unroll
    for (int mm = 0; mm < kR + KH - 1; ++mm) {
      const int ir = rres + cp.dh * (kR * rk + mm);
      const unsigned* wp = (const unsigned*)(rowp + ir * f.pitch);
      unsigned wv[NW], sv[NW - 1];
#pragma unroll
      for (int q = 0; q < NW; q += 2) {
        const uint2 d2 = *(const uint2*)(wp + q);
        wv[q] = d2.x;
        if (q + 1 < NW) wv[q + 1] = d2.y;
      }
#pragma unroll
      for (int q = 0; q + 1 < NW; ++q) sv[q] = __builtin_amdgcn_alignbit(wv[q + 1], wv[q], 16);
#pragma unroll
      for (int i = 0; i < kR; ++i) {
        const int kh = mm - i;
        if (kh < 0 || kh >= KH) continue;
#pragma unroll
        for (int j = 0; j < kV; ++j)
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            const unsigned src = (j & 1) ? sv[(j >> 1) + p] : wv[(j >> 1) + p];
            acc[i][j] = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, src), wpair[kh][p],
                                               acc[i][j], false);
          }
      }
    }
    // epilogue: residual, activation, one fp16 rounding
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      const int oh = rres + cp.dh * (kR * rk + i);
      if (oh >= cp.OH) continue;
      const int ow0 = cres + cp.dw * (kV * ck);
      const int64_t yrow = ybase + (int64_t)oh * cp.OW;
#pragma unroll
      for (int j4 = 0; j4 < kV; j4 += 4) {
        const int owq = ow0 + cp.dw * j4;
        act4_t v4 = {acc[i][j4], acc[i][j4 + 1], acc[i][j4 + 2], acc[i][j4 + 3]};
        const bool vec = cp.dw == 1 && (cp.OW & 3) == 0 && owq + 3 < cp.OW;
        if (vec) {
          if (cp.has_z) {
            const h4 zv = *(const h4*)(z + yrow + owq);
#pragma unroll
            for (int j = 0; j < 4; ++j) v4[j] += (float)zv[j];
          }
          v4 = act4<ACT>(v4, cp.alpha, cp.beta);
          h4 out;
#pragma unroll
          for (int j = 0; j < 4; ++j) out[j] = (half_t)v4[j];
          *(h4*)(y + yrow + owq) = out;
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int ow = owq + cp.dw * j;
            if (ow < cp.OW && cp.has_z) v4[j] += to_f32(z[yrow + ow]);
          }
          v4 = act4<ACT>(v4, cp.alpha, cp.beta);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int ow = owq + cp.dw * j;
            if (ow < cp.OW) y[yrow + ow] = (half_t)v4[j];
          }
        }
      }
    }
  }
}

template <int KS, int R, int V>
int launch_fast(const Geometry& g, const DwFast& f, const RunArgs& a) {
  const ConvParams& cp = g.cp;
  const int64_t blocks = (cp.n * cp.M + f.pb - 1) / f.pb;
  const size_t shmem = (size_t)f.pb * f.plane_halves * 2;
  return launch_conv(dw_fast_kernel<KS, R, V, FC_ACT>, dim3((unsigned)blocks), dim3(kThreads), shmem,
                     a, kEdgeBoth, (const half_t*)a.x, (const half_t*)a.w,
                     (const half_t*)a.bias, (const half_t*)a.z, (half_t*)a.y, cp, f);
}

template <typename T>
int launch_t(const Geometry& g, const Plan& p, const RunArgs& a) {
  const ConvParams& cp = g.cp;
  const int tiles_h = (cp.OH + p.tile_h - 1) / p.tile_h;
  const int tiles_w = (cp.OW + p.tile_w - 1) / p.tile_w;
  const int64_t blocks = cp.n * cp.M * tiles_h * tiles_w;
  const size_t shmem = (size_t)halo_bytes(cp, p.tile_h, p.tile_w);
  return launch_conv(depthwise_kernel<T>, dim3((unsigned)blocks), dim3(kThreads), shmem, a,
                     kEdgeBoth, (const T*)a.x, (const T*)a.w, (const T*)a.bias,
                     (const T*)a.z, (T*)a.y, cp, p.tile_h, p.tile_w, tiles_h, tiles_w);
}

}  // namespace

#ifndef FC_ACT
#error "compiled once per activation id: -DFC_ACT=<0..ACT_COUNT-1>"
#endif

// the packed-fp16 depthwise kernel with activation FC_ACT
int FC_CAT(launch_dwfast_act_, FC_ACT)(const Geometry& g, const RunArgs& a) {
  DwFast f;
  if (!dw_fast_plan(g.cp, f)) return FUSEDCONV_ERR_ROUTE;
  switch (g.cp.KH) {
    case 3: return launch_fast<3, 4, 4>(g, f, a);
    case 5: return launch_fast<5, 4, 4>(g, f, a);
    case 7: return launch_fast<7, 4, 4>(g, f, a);
    default: return FUSEDCONV_ERR_ROUTE;
  }
}

#if FC_ACT == 0
FC_ACT_DECLS(launch_dwfast_act_)

bool depthwise_fits(const ConvParams& cp, int32_t& tile_h, int32_t& tile_w) {
  if (cp.Cg != 1 || !depth_trivial(cp)) return false;
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
  if (p.tile == 2) return launch_depthwise_mfma(g, a);
  DwFast f;
  if (p.tile == 1 && g.dtype == FUSEDCONV_F16 && dw_fast_plan(g.cp, f)) {
    static const ActLaunchFn table[ACT_COUNT] = FC_ACT_TABLE(launch_dwfast_act_);
    return table[g.cp.act](g, a);
  }
  return g.dtype == FUSEDCONV_F16 ? launch_t<half_t>(g, p, a) : launch_t<float>(g, p, a);
}

bool depthwise_fast(const ConvParams& cp, int32_t dtype) {
  DwFast f;
  return dtype == FUSEDCONV_F16 && dw_fast_plan(cp, f);
}
#endif

}  // namespace fc
