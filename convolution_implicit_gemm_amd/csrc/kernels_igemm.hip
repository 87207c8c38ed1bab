// Implicit-GEMM convolution on MFMA with gathered im2col tiles.
//
// Per group g the convolution is the GEMM  Cmat[m][p] = sum_k A[m][k] * B[k][p]
// with A = W viewed as [M/group][K], K = (C/group)*taps in W's own
// (channel, kd, kh, kw) order, and B = im2col(X) [K][n*OD*OH*OW], gathered on
// the fly: column p = (n, od, oh, ow), row k = (c, kd, kh, kw) reads
// X[n, g*C/group + c, od*sd - pd + kd*dd, oh*sh - ph + kh*dh, ow*sw - pw + kw*dw]
// and reads 0 outside the input (zero padding).  This is the implicit-im2col
// GEMM of the FusedConv manifest's implicit_im2col_* variants and of the
// ExecuTorch conv2d im2col-GEMM PR (M = out channels, N = batch * output
// pixels, K = in channels * taps), re-tiled for gfx950:
//   * 256 threads = 4 wave64s, block tile BM x 128, K tile 32;
//   * A and B tiles are staged in LDS with K contiguous per row (padded rows),
//     double-buffered so the next tile's global loads overlap the MFMAs;
//   * fp16: v_mfma_f32_16x16x32_f16 (fp32 accumulate); fp32:
//     v_mfma_f32_16x16x4_f32;
//   * the epilogue (bias, residual, activation) runs on the accumulators;
//   * split-K (grid z = group * split) writes raw fp32 partials that a second
//     kernel sums and finishes with the same epilogue (FusedConv README,
//     implicit_im2col_tiled_reg_splitk: combine raw partial sums, apply the
//     epilogue once; the combine reassociates the fp32 additions).
#include <hip/hip_runtime.h>

#include "epilogue.h"
#include "internal.h"
#include "launch.h"

namespace fc {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 32;
constexpr int kBN = 128;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

template <typename T> struct Pad;                       // LDS row padding (elements)
template <> struct Pad<half_t> { static constexpr int v = 8; };
template <> struct Pad<float> { static constexpr int v = 4; };

// One wave's MFMA work on one K tile held in LDS.
template <typename T, int TM, int TN, int LDA>
__device__ __forceinline__ void mfma_tile(const T* As, const T* Bs, int lane,
                                          float4v (&acc)[TM][TN]);

template <>
__device__ __forceinline__ void mfma_tile<half_t, 4, 4, kBK + 8>(const half_t* As,
                                                                 const half_t* Bs, int lane,
                                                                 float4v (&acc)[4][4]) {
  constexpr int LD = kBK + 8;
  const int r = lane & 15, q = lane >> 4;
  half8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = *(const half8*)(As + (i * 16 + r) * LD + q * 8);
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = *(const half8*)(Bs + (j * 16 + r) * LD + q * 8);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
}

template <>
__device__ __forceinline__ void mfma_tile<half_t, 4, 2, kBK + 8>(const half_t* As,
                                                                 const half_t* Bs, int lane,
                                                                 float4v (&acc)[4][2]) {
  constexpr int LD = kBK + 8;
  const int r = lane & 15, q = lane >> 4;
  half8 a[4], b[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = *(const half8*)(As + (i * 16 + r) * LD + q * 8);
#pragma unroll
  for (int j = 0; j < 2; ++j) b[j] = *(const half8*)(Bs + (j * 16 + r) * LD + q * 8);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], b[j], acc[i][j], 0, 0, 0);
}

// fp32: each lane reads 4 consecutive k of its row/column and feeds them to
// four 16x16x4 MFMAs; MFMA e then contracts k = {e, 4+e, 8+e, 12+e} of the
// 16-wide group, the same permutation for A and B, so every k is summed once.
template <int TM, int TN>
__device__ __forceinline__ void mfma_tile_f32(const float* As, const float* Bs, int lane,
                                              float4v (&acc)[TM][TN]) {
  constexpr int LD = kBK + 4;
  const int r = lane & 15, q = lane >> 4;
#pragma unroll
  for (int kq = 0; kq < kBK / 16; ++kq) {
    float4v a[TM], b[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) a[i] = *(const float4v*)(As + (i * 16 + r) * LD + kq * 16 + q * 4);
#pragma unroll
    for (int j = 0; j < TN; ++j) b[j] = *(const float4v*)(Bs + (j * 16 + r) * LD + kq * 16 + q * 4);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][e], b[j][e], acc[i][j], 0, 0, 0);
  }
}

template <>
__device__ __forceinline__ void mfma_tile<float, 4, 4, kBK + 4>(const float* As, const float* Bs,
                                                               int lane, float4v (&acc)[4][4]) {
  mfma_tile_f32<4, 4>(As, Bs, lane, acc);
}
template <>
__device__ __forceinline__ void mfma_tile<float, 4, 2, kBK + 4>(const float* As, const float* Bs,
                                                               int lane, float4v (&acc)[4][2]) {
  mfma_tile_f32<4, 2>(As, Bs, lane, acc);
}

// Block tile BM x kBN; waves arranged WGM x WGN, each owning a
// (BM/WGM) x (kBN/WGN) sub-tile = TM x TN MFMA blocks of 16x16.
template <typename T, int BM, int WGM, bool SPLIT>
__global__ __launch_bounds__(kThreads) void igemm_kernel(const T* __restrict__ x,
                                                         const T* __restrict__ w,
                                                         const T* __restrict__ bias,
                                                         const T* z, const T* pre, T* y,
                                                         float* __restrict__ part,
                                                         ConvParams cp, int k_tiles,
                                                         int kt_per_split, int avec) {
  constexpr int WGN = 4 / WGM;
  constexpr int WTM = BM / WGM, WTN = kBN / WGN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr int LD = kBK + Pad<T>::v;
  constexpr int EA = BM * kBK / kThreads;   // A elements per thread per tile
  constexpr int APR = kBK / EA;             // threads per A row
  static_assert(EA == 8 || EA == 16, "A tile split");

  __shared__ __attribute__((aligned(16))) T As[2][BM * LD];
  __shared__ __attribute__((aligned(16))) T Bs[2][kBN * LD];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;

  const int64_t p0 = (int64_t)blockIdx.x * kBN;
  const int m0 = blockIdx.y * BM;
  const int g = (int)(blockIdx.z % cp.G);
  const int sidx = (int)(blockIdx.z / cp.G);
  const int kt0 = sidx * kt_per_split;
  const int kt1 = min(k_tiles, kt0 + kt_per_split);

  // ---- A (weights) loader: row am, k columns [ak, ak + EA) of the tile
  const int am = tid / APR, ak = (tid % APR) * EA;
  const bool arow_ok = (m0 + am) < cp.Mg;
  const T* wrow = w + ((int64_t)g * cp.Mg + m0 + am) * cp.K;

  // ---- B (im2col) loader: this wave gathers k rows [wave*8, wave*8+8) for
  // columns p = lane and lane + 64 of the tile.
  int64_t xbase[2];
  int id0[2], ih0[2], iw0[2];
  bool pok[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t p = p0 + lane + h * 64;
    pok[h] = p < cp.P;
    const int64_t pp = pok[h] ? p : 0;
    const int64_t nimg = pp / cp.out_sz;
    const int64_t o = pp % cp.out_sz;
    const int ow = (int)(o % cp.OW);
    const int64_t t = o / cp.OW;
    const int oh = (int)(t % cp.OH), od = (int)(t / cp.OH);
    xbase[h] = (nimg * cp.C + (int64_t)g * cp.Cg) * cp.in_sz;
    id0[h] = od * cp.sd - cp.pd;
    ih0[h] = oh * cp.sh - cp.ph;
    iw0[h] = ow * cp.sw - cp.pw;
  }
  const int khw = cp.KH * cp.KW;

  T areg[EA];
  T breg[2][8];

  auto load_tile = [&](int kt) {
    const int k0 = kt * kBK;
    // A: contiguous along K
    if (avec) {
#pragma unroll
      for (int v = 0; v < EA; v += 16 / (int)sizeof(T)) {
        const int k = k0 + ak + v;
        typedef T vec_t __attribute__((ext_vector_type(16 / sizeof(T))));
        vec_t val = {};
        if (arow_ok && k < cp.K) val = *(const vec_t*)(wrow + k);
#pragma unroll
        for (int e = 0; e < 16 / (int)sizeof(T); ++e) areg[v + e] = val[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < EA; ++e) {
        const int k = k0 + ak + e;
        areg[e] = (arow_ok && k < cp.K) ? wrow[k] : (T)0;
      }
    }
    // B: gather 8 consecutive k (wave-uniform) for two columns
    int kk = k0 + wave * 8;
    int c = kk / cp.taps;
    int t = kk - c * cp.taps;
    int kd = t / khw;
    int r = t - kd * khw;
    int kh = r / cp.KW;
    int kw = r - kh * cp.KW;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool kok = kk < cp.K;
      const int dd = kd * cp.dd, dh = kh * cp.dh, dw = kw * cp.dw;
      const int64_t coff = (int64_t)c * cp.in_sz;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int id = id0[h] + dd, ih = ih0[h] + dh, iw = iw0[h] + dw;
        const bool ok = kok && pok[h] && (unsigned)id < (unsigned)cp.D &&
                        (unsigned)ih < (unsigned)cp.H && (unsigned)iw < (unsigned)cp.W;
        breg[h][e] = ok ? x[xbase[h] + coff + ((int64_t)id * cp.H + ih) * cp.W + iw] : (T)0;
      }
      // next k: kw fastest, then kh, kd, c
      ++kk;
      if (++kw == cp.KW) {
        kw = 0;
        if (++kh == cp.KH) {
          kh = 0;
          if (++kd == cp.KD) {
            kd = 0;
            ++c;
          }
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
    T* as = As[buf] + am * LD + ak;
#pragma unroll
    for (int e = 0; e < EA; ++e) as[e] = areg[e];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      T* bs = Bs[buf] + (lane + h * 64) * LD + wave * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) bs[e] = breg[h][e];
    }
  };

  float4v acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = float4v{0.0f, 0.0f, 0.0f, 0.0f};

  if (kt0 < kt1) {
    load_tile(kt0);
    store_tile(0);
    __syncthreads();
    int cur = 0;
    for (int kt = kt0; kt < kt1; ++kt) {
      const bool more = kt + 1 < kt1;
      if (more) load_tile(kt + 1);
      mfma_tile<T, TM, TN, LD>(As[cur] + wm * WTM * LD, Bs[cur] + wn * WTN * LD, lane, acc);
      if (more) store_tile(cur ^ 1);
      __syncthreads();
      cur ^= 1;
    }
  }

  // ---- epilogue: lane holds rows 4*(lane/16)+rr, column lane%16 of each block
  const int q = lane >> 4, cl = lane & 15;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t p = p0 + wn * WTN + j * 16 + cl;
    if (p >= cp.P) continue;
    const int64_t nimg = p / cp.out_sz;
    const int64_t o = p % cp.out_sz;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int m = m0 + wm * WTM + i * 16 + q * 4 + rr;
        if (m >= cp.Mg) continue;
        const int gm = g * cp.Mg + m;
        if (SPLIT) {
          part[((int64_t)sidx * cp.M + gm) * cp.P + p] = acc[i][j][rr];
        } else {
          const int64_t yi = (nimg * cp.M + gm) * cp.out_sz + o;
          y[yi] = epilogue<T>(acc[i][j][rr], gm, yi, cp, bias, z, pre);
        }
      }
    }
  }
}

// Sum the split-K partials [split][M][P] and apply the epilogue once.
template <typename T>
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(const float* __restrict__ part,
                                                                 const T* __restrict__ bias,
                                                                 const T* z, const T* pre, T* y,
                                                                 ConvParams cp, int split) {
  const int64_t total = (int64_t)cp.M * cp.P;
  const int64_t step = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += step) {
    float acc = 0.0f;
    for (int s = 0; s < split; ++s) acc += part[(int64_t)s * total + i];
    const int gm = (int)(i / cp.P);
    const int64_t p = i % cp.P;
    const int64_t nimg = p / cp.out_sz, o = p % cp.out_sz;
    const int64_t yi = (nimg * cp.M + gm) * cp.out_sz + o;
    y[yi] = epilogue<T>(acc, gm, yi, cp, bias, z, pre);
  }
}

template <typename T, int BM, int WGM>
int launch_t(const Geometry& g, const Plan& p, const RunArgs& a) {
  const ConvParams& cp = g.cp;
  const bool split = p.split_k > 1;
  dim3 grid((unsigned)((cp.P + kBN - 1) / kBN), (unsigned)((cp.Mg + BM - 1) / BM),
            (unsigned)(cp.G * p.split_k));
  const int avec = (cp.K % (16 / (int)sizeof(T))) == 0;
  if (split) {
    if (launch_conv(igemm_kernel<T, BM, WGM, true>, grid, dim3(kThreads), 0, a, kEdgeFirst,
                    (const T*)a.x, (const T*)a.w, (const T*)a.bias, (const T*)a.z,
                    (const T*)a.pre, (T*)a.y, (float*)a.ws, cp, p.k_tiles, p.k_tiles_per_split,
                    avec) != FUSEDCONV_OK)
      return FUSEDCONV_ERR_LAUNCH;
    int64_t blocks = ((int64_t)cp.M * cp.P + kThreads - 1) / kThreads;
    if (blocks > (1 << 20)) blocks = 1 << 20;
    return launch_conv(splitk_reduce_kernel<T>, dim3((unsigned)blocks), dim3(kThreads), 0, a,
                       kEdgeLast, (const float*)a.ws, (const T*)a.bias, (const T*)a.z,
                       (const T*)a.pre, (T*)a.y, cp, p.split_k);
  }
  return launch_conv(igemm_kernel<T, BM, WGM, false>, grid, dim3(kThreads), 0, a, kEdgeBoth,
                     (const T*)a.x, (const T*)a.w, (const T*)a.bias, (const T*)a.z,
                     (const T*)a.pre, (T*)a.y, (float*)nullptr, cp, p.k_tiles,
                     p.k_tiles_per_split, avec);
}

}  // namespace

int launch_igemm(const Geometry& g, const Plan& p, const RunArgs& a) {
  if (g.dtype == FUSEDCONV_F16)
    return p.tile == IGEMM_BM128_BN128 ? launch_t<half_t, 128, 2>(g, p, a)
                                       : launch_t<half_t, 64, 1>(g, p, a);
  return p.tile == IGEMM_BM128_BN128 ? launch_t<float, 128, 2>(g, p, a)
                                     : launch_t<float, 64, 1>(g, p, a);
}

}  // namespace fc
