// Explicit im2col route (fp16): the column matrix is materialised in the
// workspace, then multiplied by W on the matrix cores with the fused
// epilogue.  This is the FusedConv README's "Materialize f16 inputs directly
// into f16 columns, then run the register-tiled GEMM with f32 accumulation"
// variant (im2col_gemm_tiled_reg_f16_columns), here with the GEMM being the
// POINTWISE route's 1x1 kernel: for each group,
//     Y[n, m, p] = act( sum_k W[m, k] * col[n, g, k, p] + B[m] + Z[n, m, p] ),
// col[n, g, k, p] = X[n, g*C/G + c, o(p)*s - pad + tap(k)*d] (0 outside X),
// k = (c, kd, kh, kw) in W's own order, p = the flattened output pixel.
// Columns are stored [n][g][Kp][Pp] (K rounded up to a multiple of 8 with zero
// rows, so the GEMM sees an image of G*Kp channels and P pixels; each row
// padded with zeros to Pp, P rounded up to a multiple of 8, so that the 1x1
// kernel's 8-pixel loads stay in the row), which is the layout the 1x1
// kernel reads; W is used in place when K % 8 == 0, else copied
// to [M][Kp] with zero columns.  For patchify convolutions (stride = kernel,
// no padding, dilation 1) the column matrix is a permutation of X, so the
// route costs one extra write and read of |X| bytes and no gathers in the
// GEMM.  With overlapping windows it costs K/(stride^2) times |X| or more,
// which is where the implicit routes win (the manifest's derive
// implicitTiledWorthIt: stride < kernel).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "epilogue.h"
#include "internal.h"
#include "launch.h"

namespace fc {
namespace {

constexpr int kThreads = 256;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

struct Im2colGeo {
  int Kp;            // K rounded up to a multiple of 8 (and >= 16)
  int64_t P;         // output pixels per image (a multiple of 4)
  int64_t Pp;        // P rounded up to a multiple of 8: the row pitch of col
  size_t frag_ws;    // the 1x1 GEMM's repacked-weight workspace
  size_t w_off;      // byte offset of W padded to [M][Kp] (0 bytes when K % 8 == 0)
  size_t w_bytes;
  size_t col_off;    // byte offset of the column matrix
  size_t col_bytes;
  Geometry gemm;     // the 1x1 GEMM view of the problem
};

// The GEMM view: an image of G*Kp channels and P pixels (1-D), 1x1 kernel,
// whose channel rows are Pp pixels apart.
ConvParams gemm_view(const ConvParams& cp, int Kp, int64_t P, int64_t Pp) {
  ConvParams q = cp;
  q.C = cp.G * Kp;
  q.Cg = Kp;
  q.D = 1; q.H = 1; q.W = (int32_t)P;
  q.OD = 1; q.OH = 1; q.OW = (int32_t)P;
  q.KD = q.KH = q.KW = 1;
  q.sd = q.sh = q.sw = 1;
  q.dd = q.dh = q.dw = 1;
  q.pd = q.ph = q.pw = 0;
  q.taps = 1;
  q.K = Kp;
  q.in_sz = Pp;
  q.out_sz = P;
  q.P = cp.n * P;
  q.transposed = 0;
  q.flat = 1;  // pixel tiles over all images' columns: small images fill whole tiles
              // (the SigLIP grid's 196 pixels: 2 tiles of 128 per image, 77% used, before)
  return q;
}

bool plan_geo(const ConvParams& cp, int32_t dtype, Im2colGeo& ig) {
  if (dtype != FUSEDCONV_F16 || cp.transposed) return false;
  ig.Kp = (int)((cp.K + 7) / 8 * 8);
  if (ig.Kp < 16) ig.Kp = 16;
  ig.P = cp.out_sz;
  if (ig.P % 4 != 0 || ig.P >= ((int64_t)1 << 31) - 8) return false;
  ig.Pp = (ig.P + 7) / 8 * 8;
  ig.gemm.dtype = FUSEDCONV_F16;
  ig.gemm.nsp = 1;
  ig.gemm.y_rank = 3;
  ig.gemm.cp = gemm_view(cp, ig.Kp, ig.P, ig.Pp);
  size_t frag = 0;
  if (!pointwise_fits(ig.gemm.cp, FUSEDCONV_F16, &frag)) {
    ig.gemm.cp.flat = 0;  // per-image pixel tiles when the flat view's offsets overflow
    if (!pointwise_fits(ig.gemm.cp, FUSEDCONV_F16, &frag)) return false;
  }
  ig.frag_ws = align256(frag);
  ig.w_off = ig.frag_ws;
  ig.w_bytes = ig.Kp != cp.K ? align256((size_t)cp.M * ig.Kp * sizeof(half_t)) : 0;
  ig.col_off = ig.w_off + ig.w_bytes;
  ig.col_bytes = (size_t)cp.n * cp.G * ig.Kp * ig.Pp * sizeof(half_t);
  const size_t total = ig.col_off + ig.col_bytes;
  return total < ((size_t)1 << 40);
}

// W [M][K] -> [M][Kp], zero columns k >= K
__global__ __launch_bounds__(kThreads) void pad_w_kernel(const half_t* __restrict__ w,
                                                         half_t* __restrict__ wp, int M, int K,
                                                         int Kp) {
  const int64_t total = (int64_t)M * Kp;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t m = i / Kp;
    const int k = (int)(i - m * Kp);
    wp[i] = k < K ? w[m * K + k] : (half_t)0;
  }
}

// ---- staged form.  Block task = (image n and group g, channel c of the
// group, kernel plane kd, kernel row kh, chunk of L output pixels).  For a
// fixed (c, kd, kh) and output row R = od*OH + oh, every kernel column kw
// reads the same input row (id, ih) = (od*sd - pd + kd*dd, oh*sh - ph +
// kh*dh), and col row k = ((c*KD + kd)*KH + kh)*KW + kw holds the chunk's
// pixels contiguously.  So the block loads the chunk's input rows once
// (16-byte loads when a row is a whole number of them; zero rows outside X)
// into LDS and then writes, for each kw, the chunk's segment of col row k
// as whole pieces of 8 pixels.  LDS element j of a row sits at j + 2*(j >> 6)
// (skew of 2 elements per 64): the 8 pixels of a lane are sw apart, and the
// skew spreads the lanes of a wave over the banks for any stride.  Extra
// blocks (when Kq > K) write the rows k >= K of their chunk: zeros, except
// row K when `ones` (1 for the P valid pixels: the bias-gradient row of the
// weight-gradient GEMM).
struct StagedGeo {
  int L;        // pixels per chunk (multiple of 8)
  int nchunk;   // chunks per col row: ceil(Pp / L)
  int rows;     // LDS rows per block (>= input rows a chunk can span)
  int pitch;    // LDS row pitch in elements
  int64_t main_blocks;
  int64_t blocks;
};

constexpr int kStagedLdsBytes = 32 * 1024;

__device__ __forceinline__ int skew(int j) { return j + 2 * (j >> 6); }

// 8 consecutive elements of T as one store (two 16-byte stores for float)
template <typename T> struct Vec8;
template <> struct Vec8<half_t> {
  half8 v;
  __device__ void set(int e, half_t x) { v[e] = x; }
  __device__ void store(half_t* p) const { *(half8*)p = v; }
};
template <> struct Vec8<float> {
  typedef float float4v_ __attribute__((ext_vector_type(4)));
  float4v_ a, b;
  __device__ void set(int e, float x) {
    if (e < 4) a[e] = x; else b[e - 4] = x;
  }
  __device__ void store(float* p) const {
    *(float4v_*)p = a;
    *(float4v_*)(p + 4) = b;
  }
};

template <typename T>
__global__ __launch_bounds__(kThreads) void im2col_staged_kernel(const T* __restrict__ x,
                                                                 T* __restrict__ col,
                                                                 ConvParams cp, int Kq,
                                                                 int64_t Pp, int ones,
                                                                 StagedGeo sg) {
  extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
  T* rows = (T*)lds_raw;
  const int tid = threadIdx.x;
  const int P = (int)cp.out_sz;
  int64_t t = blockIdx.x;
  if (t >= sg.main_blocks) {
    // rows k = K .. Kq-1 of one (image, group) and chunk
    t -= sg.main_blocks;
    const int chunk = (int)(t % sg.nchunk);
    const int64_t ng = t / sg.nchunk;
    const int P0 = chunk * sg.L;
    const int noct = (int)(min((int64_t)sg.L, Pp - P0) / 8);
    const int nz = Kq - cp.K;
    for (int i = tid; i < nz * noct; i += kThreads) {
      const int k = cp.K + i / noct, o = i % noct;
      Vec8<T> v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v.set(e, (ones && k == cp.K && P0 + 8 * o + e < P) ? (T)1 : (T)0);
      v.store(col + (ng * Kq + k) * Pp + P0 + 8 * o);
    }
    return;
  }
  const int chunk = (int)(t % sg.nchunk);
  t /= sg.nchunk;
  const int kh = (int)(t % cp.KH);
  t /= cp.KH;
  const int kd = (int)(t % cp.KD);
  t /= cp.KD;
  const int c = (int)(t % cp.Cg);
  const int64_t ng = t / cp.Cg;  // n * G + g
  const int64_t n = ng / cp.G;
  const int g = (int)(ng % cp.G);
  const int P0 = chunk * sg.L;
  const int Pend = (int)min((int64_t)P0 + sg.L, Pp);  // chunk end in col (multiple of 8)
  const int Pv = min(Pend, P);                          // ... and in valid pixels (P0 < P)
  const int R0 = P0 / cp.OW;
  const int nrows = (Pv - 1) / cp.OW - R0 + 1;  // <= sg.rows (host)
  const T* xc = x + (n * cp.C + (int64_t)g * cp.Cg + c) * cp.in_sz;

  // stage the input rows of output rows R0 .. R0 + nrows - 1
  auto row_src = [&](int r) -> const T* {
    const int R = R0 + r;
    const int od = R / cp.OH, oh = R - od * cp.OH;
    const int id = od * cp.sd - cp.pd + kd * cp.dd, ih = oh * cp.sh - cp.ph + kh * cp.dh;
    if ((unsigned)id >= (unsigned)cp.D || (unsigned)ih >= (unsigned)cp.H) return nullptr;
    return xc + ((int64_t)id * cp.H + ih) * cp.W;
  };
  constexpr int VE = 16 / sizeof(T);  // elements per 16-byte load
  if (cp.W % VE == 0) {
    typedef T tvec __attribute__((ext_vector_type(VE)));
    const int wv = cp.W / VE;
    for (int i = tid; i < nrows * wv; i += kThreads) {
      const int r = i / wv, j = (i - r * wv) * VE;
      const T* src = row_src(r);
      const tvec v = src ? *(const tvec*)(src + j) : tvec{};
      T* dst = rows + r * sg.pitch + skew(j);  // VE elements stay in one 64-block
#pragma unroll
      for (int e = 0; e < VE; ++e) dst[e] = v[e];
    }
  } else {
    for (int i = tid; i < nrows * cp.W; i += kThreads) {
      const int r = i / cp.W, j = i - r * cp.W;
      const T* src = row_src(r);
      rows[r * sg.pitch + skew(j)] = src ? src[j] : (T)0;
    }
  }
  __syncthreads();

  // col rows k of this (c, kd, kh): one 8-pixel piece per thread and step
  const int noct = (Pend - P0) / 8;
  const int kbase = ((c * cp.KD + kd) * cp.KH + kh) * cp.KW;
  T* colb = col + (ng * Kq + kbase) * Pp + P0;
  for (int i = tid; i < cp.KW * noct; i += kThreads) {
    const int kw = i / noct, o = i - kw * noct;
    const int p0 = P0 + 8 * o;
    int R = p0 / cp.OW, ow = p0 - R * cp.OW;
    const int iw0 = kw * cp.dw - cp.pw;
    Vec8<T> v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      T val = (T)0;
      if (p0 + e < Pv) {
        const int iw = ow * cp.sw + iw0;
        if ((unsigned)iw < (unsigned)cp.W) val = rows[(R - R0) * sg.pitch + skew(iw)];
      }
      v.set(e, val);
      if (++ow == cp.OW) {
        ow = 0;
        ++R;
      }
    }
    v.store(colb + (int64_t)kw * Pp + 8 * o);
  }
}

bool staged_plan(const ConvParams& cp, int Kq, int64_t Pp, int esize, StagedGeo& sg) {
  sg.pitch = cp.W + 2 * (cp.W >> 6) + 2;
  sg.rows = kStagedLdsBytes / (sg.pitch * esize);
  if (sg.rows < 2) return false;
  // a chunk of L pixels starting anywhere spans at most (L - 1) / OW + 2 rows
  const int64_t lmax = (int64_t)(sg.rows - 2) * cp.OW + 1;
  int64_t L = lmax / 8 * 8;
  if (L > 4096) L = 4096;
  if (L > Pp) L = Pp;
  if (L < 8) return false;
  sg.L = (int)L;
  // LDS for the rows a chunk can span, not the whole budget (more blocks per CU)
  sg.rows = (int)std::min<int64_t>(sg.rows, (L - 1) / cp.OW + 2);
  sg.nchunk = (int)((Pp + L - 1) / L);
  sg.main_blocks = cp.n * cp.G * cp.Cg * cp.KD * cp.KH * sg.nchunk;
  sg.blocks = sg.main_blocks + (Kq > cp.K ? cp.n * cp.G * sg.nchunk : 0);
  return sg.blocks < ((int64_t)1 << 31);
}

// ---- gather form (rows too wide to stage): col[((n*G + g)*Kq + k)*Pp + p]
// for 8 consecutive pixels p per thread (one piece of 8; Pp % 8 == 0 so the
// 8 never leave the row of col); rows k >= K as in the staged form
template <typename T>
__global__ __launch_bounds__(kThreads) void im2col_gather_kernel(const T* __restrict__ x,
                                                                 T* __restrict__ col,
                                                                 ConvParams cp, int Kq,
                                                                 int64_t Pp, int ones) {
  const int P = (int)cp.out_sz;
  const int64_t p8 = Pp / 8;
  const int64_t total = cp.n * cp.G * Kq * p8;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    const int pc = (int)(i % p8);
    int64_t r = i / p8;
    const int k = (int)(r % Kq);
    r /= Kq;  // n * G + g
    const int g = (int)(r % cp.G);
    const int64_t n = r / cp.G;
    Vec8<T> v;
    const int p0 = pc * 8;
    if (k < cp.K) {
      // k -> (c, kd, kh, kw) in W's order
      const int kw = k % cp.KW, kh = (k / cp.KW) % cp.KH, kd = (k / (cp.KW * cp.KH)) % cp.KD;
      const int c = k / cp.taps;
      const T* xc = x + (n * cp.C + (int64_t)g * cp.Cg + c) * cp.in_sz;
      int ow = p0 % cp.OW, R = p0 / cp.OW;
      int oh = R % cp.OH, od = R / cp.OH;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        T val = (T)0;
        if (p0 + e < P) {
          const int id = od * cp.sd - cp.pd + kd * cp.dd, ih = oh * cp.sh - cp.ph + kh * cp.dh,
                    iw = ow * cp.sw - cp.pw + kw * cp.dw;
          if ((unsigned)id < (unsigned)cp.D && (unsigned)ih < (unsigned)cp.H &&
              (unsigned)iw < (unsigned)cp.W)
            val = xc[((int64_t)id * cp.H + ih) * cp.W + iw];
        }
        v.set(e, val);
        if (++ow == cp.OW) {
          ow = 0;
          if (++oh == cp.OH) {
            oh = 0;
            ++od;
          }
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v.set(e, (ones && k == cp.K && p0 + e < P) ? (T)1 : (T)0);
    }
    v.store(col + i * 8);
  }
}

unsigned grid_for(int64_t work) {
  int64_t b = (work + kThreads - 1) / kThreads;
  if (b > 8192) b = 8192;
  if (b < 1) b = 1;
  return (unsigned)b;
}

// the 1x1 GEMM's weights: W itself or its zero-padded copy
const void* gemm_w(const Im2colGeo& ig, const ConvParams& cp, const RunArgs& a) {
  return ig.Kp != cp.K ? (const void*)((char*)a.ws + ig.w_off) : a.w;
}

int prepare_weights_impl(const Geometry& g, const Im2colGeo& ig, const RunArgs& a) {
  const ConvParams& cp = g.cp;
  if (ig.Kp != cp.K) {
    hipLaunchKernelGGL(pad_w_kernel, dim3(grid_for((int64_t)cp.M * ig.Kp)), dim3(kThreads), 0,
                       (hipStream_t)a.stream, (const half_t*)a.w, (half_t*)((char*)a.ws + ig.w_off),
                       cp.M, cp.K, ig.Kp);
    if (hipPeekAtLastError() != hipSuccess) return FUSEDCONV_ERR_LAUNCH;
  }
  RunArgs b = a;
  b.w = gemm_w(ig, cp, a);
  Plan pp{};
  return prepare_pointwise(ig.gemm, pp, b);
}

}  // namespace

namespace {
template <typename T>
int launch_columns_t(const ConvParams& cp, const void* x, void* col, int Kq, int64_t Pp, int ones,
                     const RunArgs& a, unsigned edges) {
  StagedGeo sg;
  if (staged_plan(cp, Kq, Pp, (int)sizeof(T), sg))
    return launch_conv(im2col_staged_kernel<T>, dim3((unsigned)sg.blocks), dim3(kThreads),
                       (size_t)sg.rows * sg.pitch * sizeof(T), a, edges, (const T*)x, (T*)col, cp,
                       Kq, Pp, ones, sg);
  return launch_conv(im2col_gather_kernel<T>, dim3(grid_for(cp.n * cp.G * Kq * (Pp / 8))),
                     dim3(kThreads), 0, a, edges, (const T*)x, (T*)col, cp, Kq, Pp, ones);
}
}  // namespace

int launch_columns(const ConvParams& cp, int32_t dtype, const void* x, void* col, int Kq,
                   int64_t Pp, int ones, const RunArgs& a, unsigned edges) {
  return dtype == FUSEDCONV_F16 ? launch_columns_t<half_t>(cp, x, col, Kq, Pp, ones, a, edges)
                                : launch_columns_t<float>(cp, x, col, Kq, Pp, ones, a, edges);
}

bool im2col_fits(const ConvParams& cp, int32_t dtype, size_t* workspace) {
  Im2colGeo ig;
  if (!plan_geo(cp, dtype, ig)) return false;
  if (workspace) *workspace = ig.col_off + ig.col_bytes;
  return true;
}

int prepare_im2col(const Geometry& g, const Plan&, const RunArgs& a) {
  Im2colGeo ig;
  if (!plan_geo(g.cp, g.dtype, ig)) return FUSEDCONV_ERR_ROUTE;
  return prepare_weights_impl(g, ig, a);
}

int launch_im2col(const Geometry& g, const Plan&, const RunArgs& a) {
  const ConvParams& cp = g.cp;
  Im2colGeo ig;
  if (!plan_geo(cp, g.dtype, ig)) return FUSEDCONV_ERR_ROUTE;
  if (!(a.flags & FUSEDCONV_RUN_WEIGHTS_PREPARED)) {
    const int rc = prepare_weights_impl(g, ig, a);
    if (rc != FUSEDCONV_OK) return rc;
  }
  half_t* col = (half_t*)((char*)a.ws + ig.col_off);
  // the column matrix, then the 1x1 GEMM over it: the timed interval of a
  // timed run spans both
  RunArgs ai = a;
  ai.ev_stop = nullptr;
  const int rc = launch_columns(cp, FUSEDCONV_F16, a.x, col, ig.Kp, ig.Pp, 0, ai, kEdgeFirst);
  if (rc != FUSEDCONV_OK) return rc;
  RunArgs b = a;
  b.x = col;
  b.w = gemm_w(ig, cp, a);
  b.flags = a.flags | FUSEDCONV_RUN_WEIGHTS_PREPARED;
  b.ev_start = nullptr;
  Plan pp{};
  return launch_pointwise(ig.gemm, pp, b);
}

}  // namespace fc
