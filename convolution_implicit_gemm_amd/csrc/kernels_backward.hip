// Backward kernels of the convolution (fusedconv_create_backward_data /
// _weight), the training side of the FusedConv layer that the tinygrad
// compare page fuses for AMD GPUs (tinygrad/codegen/opt/reduce.py:
// direct_conv_bwd_activation_program, the input gradient of a 3x3
// convolution as per-tap GEMMs with the QuickGelu derivative in the
// epilogue; col2im_program, the same gradient assembled from per-tap columns
// with an optional fused activation derivative).
//
//  * flip_w_kernel: for a stride-1 convolution the input gradient is itself
//    a forward convolution of the output gradient G, with W transposed per
//    group and flipped in every spatial axis, W'[g*C/G + c][m][k] =
//    W[g*M/G + m][c][taps - 1 - k], and begin pads dilation*(k-1) - pad.
//    The forward routes then run it with the backward-data epilogue.
//  * weight gradient dW[m][c, k] = sum_n sum_p G[n][m][p] * col[n][g][c, k][p]
//    with col the column matrix of X (launch_columns), row K of col all ones
//    for the bias gradient: a GEMM whose operands both run along the pixels,
//    so every MFMA operand is a contiguous 16-byte piece of a G row or a
//    col row, loaded straight into registers.  Blocks split the images; the
//    fp32 partials are summed by a second kernel.
//  * wgrad_direct_kernel: the plain reduction, one block per dW element, for
//    problems the GEMM does not take.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "epilogue.h"
#include "internal.h"
#include "launch.h"

namespace fc {
namespace {

typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWM = 256;   // GEMM block tile: output channels
constexpr int kWK = 128;   // GEMM block tile: reduction rows of W (c, k) (+ the ones row)

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

template <typename T>
__global__ __launch_bounds__(kThreads) void flip_w_kernel(const T* __restrict__ w, T* __restrict__ wf,
                                                          int Mg, int Cg, int G, int taps) {
  const int64_t total = (int64_t)G * Cg * Mg * taps;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    // i = ((g*Cg + c)*Mg + m)*taps + t
    const int t = (int)(i % taps);
    int64_t r = i / taps;
    const int m = (int)(r % Mg);
    r /= Mg;
    const int c = (int)(r % Cg);
    const int g = (int)(r / Cg);
    wf[i] = w[(((int64_t)g * Mg + m) * Cg + c) * taps + (taps - 1 - t)];
  }
}

struct WgGeo {
  int Kq;        // col rows: K (+1 for the bias row) rounded up to a multiple of 8
  int64_t Pp;    // col row pitch: P rounded up to a multiple of 8
  int nmt, nkt;  // block tiles along M/group and Kq
  int splits;    // image ranges
  int ipb;       // images per range
  int has_db;
};

// ---- the weight-gradient GEMM.  Block = 4 waves as 2 (channels) x 2
// (reduction rows); a wave owns 128 x 64 outputs = 8 x 4 MFMA tiles.  Lane
// (r16, q) supplies the operand row r16 of each tile and pixels 8q .. 8q+7
// (fp16, v_mfma_f32_16x16x32_f16) or 4q .. 4q+3 (fp32, four
// v_mfma_f32_16x16x4f32 on one element each) of the step.  G rows (P pixels,
// P % 4 == 0) are read as 8-byte (fp16) or 16-byte (fp32) pieces, col rows
// (Pp pixels) as 16-byte pieces; pieces past the row end are zero.  The
// next step's operands are loaded before this step's products.
template <typename T> struct WgOp;
template <> struct WgOp<half_t> {
  static constexpr int kStep = 32;  // pixels per step
  typedef half8 A;
  __device__ static A load_g(const half_t* row, int pix, int P, bool ok) {
    const half4 lo = (ok && pix < P) ? *(const half4*)(row + pix) : half4{};
    const half4 hi = (ok && pix + 4 < P) ? *(const half4*)(row + pix + 4) : half4{};
    return A{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  __device__ static A load_c(const half_t* row, int pix, int64_t Pp, bool ok) {
    return (ok && pix + 8 <= Pp) ? *(const half8*)(row + pix) : half8{};
  }
  __device__ static void mma(float4v& acc, const A& a, const A& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
  }
  static constexpr int kLanePix = 8;
};
template <> struct WgOp<float> {
  static constexpr int kStep = 16;
  typedef float4v A;
  __device__ static A load_g(const float* row, int pix, int P, bool ok) {
    return (ok && pix < P) ? *(const float4v*)(row + pix) : float4v{};
  }
  __device__ static A load_c(const float* row, int pix, int64_t Pp, bool ok) {
    return (ok && pix + 4 <= Pp) ? *(const float4v*)(row + pix) : float4v{};
  }
  __device__ static void mma(float4v& acc, const A& a, const A& b) {
#pragma unroll
    for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], b[t], acc, 0, 0, 0);
  }
  static constexpr int kLanePix = 4;
};

template <typename T>
__global__ __launch_bounds__(kThreads) void wgrad_gemm_kernel(const T* __restrict__ dy,
                                                              const T* __restrict__ col,
                                                              float* __restrict__ part,
                                                              ConvParams cp, WgGeo wg) {
  using Op = WgOp<T>;
  typedef typename Op::A A;
  int64_t t = blockIdx.x;
  const int kt = (int)(t % wg.nkt);
  t /= wg.nkt;
  const int mt = (int)(t % wg.nmt);
  t /= wg.nmt;
  const int g = (int)(t % cp.G);
  const int s = (int)(t / cp.G);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wk = wave >> 1;
  const int r16 = lane & 15, q = lane >> 4;
  const int m0 = mt * kWM + wm * 128, k0 = kt * kWK + wk * 64;
  const int P = (int)cp.out_sz;
  const int64_t n0 = (int64_t)s * wg.ipb;
  const int nimg = (int)std::min<int64_t>(wg.ipb, cp.n - n0);

  bool am[8], bk[4];
#pragma unroll
  for (int i = 0; i < 8; ++i) am[i] = m0 + i * 16 + r16 < cp.Mg;
#pragma unroll
  for (int j = 0; j < 4; ++j) bk[j] = k0 + j * 16 + r16 < wg.Kq;
  const int nps = (int)cdiv(wg.Pp, Op::kStep);
  const int total = nimg * nps;

  auto load = [&](int st, A (&a)[8], A (&b)[4]) __attribute__((always_inline)) {
    const int64_t n = n0 + st / nps;
    const int pix = (st % nps) * Op::kStep + q * Op::kLanePix;
    const T* grow = dy + ((n * cp.M + (int64_t)g * cp.Mg + m0 + r16) * P);
    const T* crow = col + (((n * cp.G + g) * wg.Kq + k0 + r16) * wg.Pp);
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = Op::load_g(grow + (int64_t)i * 16 * P, pix, P, am[i]);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = Op::load_c(crow + (int64_t)j * 16 * wg.Pp, pix, wg.Pp, bk[j]);
  };

  float4v acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float4v{0.f, 0.f, 0.f, 0.f};
  if (total > 0) {
    A ca[8], cb[4], na[8], nb[4];
    load(0, ca, cb);
    for (int st = 0; st < total; ++st) {
      if (st + 1 < total) load(st + 1, na, nb);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) Op::mma(acc[i][j], ca[i], cb[j]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 8; ++i) ca[i] = na[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) cb[j] = nb[j];
    }
  }
  // wait states between the last products and the VALU reads of their
  // accumulators
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  // lane holds rows 4q + r (channels) of column r16 (reduction row) per tile
  float* pb = part + ((int64_t)s * cp.G + g) * cp.Mg * wg.Kq;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = k0 + j * 16 + r16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + i * 16 + q * 4 + r;
        if (m < cp.Mg && k < wg.Kq) pb[(int64_t)m * wg.Kq + k] = acc[i][j][r];
      }
    }
}

// dW[m][k] = sum over the image ranges, k < K; dB[m] from row K
__global__ __launch_bounds__(kThreads) void wgrad_reduce_kernel(const float* __restrict__ part,
                                                                float* __restrict__ dw,
                                                                float* __restrict__ db,
                                                                ConvParams cp, WgGeo wg) {
  const int64_t total = (int64_t)cp.M * wg.Kq;
  const int64_t stride = (int64_t)cp.G * cp.Mg * wg.Kq;  // one image range
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * kThreads) {
    const int k = (int)(i % wg.Kq);
    const int64_t m = i / wg.Kq;  // = g*Mg + ml: part's (g, ml) order is m's
    if (k > cp.K || (k == cp.K && !wg.has_db)) continue;
    float acc = 0.0f;
    for (int s = 0; s < wg.splits; ++s) acc += part[(int64_t)s * stride + i];
    if (k < cp.K) dw[m * cp.K + k] = acc;
    else db[m] = acc;
  }
}

// ---- plain reduction: block b = (m, kk), kk < K a weight, kk == K the bias
template <typename T>
__global__ __launch_bounds__(kThreads) void wgrad_direct_kernel(const T* __restrict__ x,
                                                                const T* __restrict__ dy,
                                                                float* __restrict__ dw,
                                                                float* __restrict__ db,
                                                                ConvParams cp, int has_db) {
  __shared__ float red[kThreads / 64];
  const int kk = (int)(blockIdx.x % (cp.K + has_db));
  const int m = (int)(blockIdx.x / (cp.K + has_db));
  const int g = m / cp.Mg;
  int c = 0, kd = 0, kh = 0, kw = 0;
  if (kk < cp.K) {
    kw = kk % cp.KW;
    kh = (kk / cp.KW) % cp.KH;
    kd = (kk / (cp.KW * cp.KH)) % cp.KD;
    c = kk / cp.taps;
  }
  const int64_t total = cp.n * cp.out_sz;
  float acc = 0.0f;
  for (int64_t i = threadIdx.x; i < total; i += kThreads) {
    const int64_t n = i / cp.out_sz, o = i % cp.out_sz;
    const float gv = to_f32(dy[(n * cp.M + m) * cp.out_sz + o]);
    if (kk == cp.K) {
      acc += gv;
      continue;
    }
    const int ow = (int)(o % cp.OW);
    const int64_t r = o / cp.OW;
    const int oh = (int)(r % cp.OH), od = (int)(r / cp.OH);
    const int id = od * cp.sd - cp.pd + kd * cp.dd, ih = oh * cp.sh - cp.ph + kh * cp.dh,
              iw = ow * cp.sw - cp.pw + kw * cp.dw;
    if ((unsigned)id < (unsigned)cp.D && (unsigned)ih < (unsigned)cp.H && (unsigned)iw < (unsigned)cp.W)
      acc = fmaf(gv, to_f32(x[(n * cp.C + (int64_t)g * cp.Cg + c) * cp.in_sz +
                              ((int64_t)id * cp.H + ih) * cp.W + iw]),
                 acc);
  }
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    float v = 0.0f;
    for (int i = 0; i < kThreads / 64; ++i) v += red[i];
    if (kk < cp.K) dw[(int64_t)m * cp.K + kk] = v;
    else db[m] = v;
  }
}

bool wg_plan(const ConvParams& cp, int32_t dtype, int has_db, WgGeo& wg, size_t* col_bytes,
             size_t* part_bytes) {
  if (cp.transposed || cp.out_sz % 4 != 0 || cp.out_sz >= ((int64_t)1 << 31) - 8) return false;
  const size_t es = dtype == FUSEDCONV_F16 ? 2 : 4;
  wg.has_db = has_db;
  wg.Kq = (int)((cp.K + has_db + 7) / 8 * 8);
  wg.Pp = (cp.out_sz + 7) / 8 * 8;
  wg.nmt = (int)cdiv(cp.Mg, kWM);
  wg.nkt = (int)cdiv(wg.Kq, kWK);
  const int64_t tiles = (int64_t)cp.G * wg.nmt * wg.nkt;
  // about four blocks per CU, at least one image per range
  int64_t splits = std::max<int64_t>(1, std::min<int64_t>(cp.n, cdiv(1024, tiles)));
  wg.ipb = (int)cdiv(cp.n, splits);
  wg.splits = (int)cdiv(cp.n, wg.ipb);
  if (tiles * wg.splits >= ((int64_t)1 << 31)) return false;
  // 32-bit pixel offsets inside a row pair; the pointers are 64-bit
  *col_bytes = align256((size_t)cp.n * cp.G * wg.Kq * wg.Pp * es);
  *part_bytes = (size_t)wg.splits * cp.M * wg.Kq * sizeof(float);
  return true;
}

// ---- shifted-tap weight gradient (fp16, stride 1, 2-D or 1-D, up to 9
// taps, W and OW multiples of 8, C/group a multiple of 16): no column
// matrix.  The tinygrad page runs a 3x3 input gradient as nine per-tap
// GEMMs; here the weight gradient is nine per-tap GEMMs over one staged box
// of X.  Block = 4 waves along 256 output channels x 16 input channels x
// every tap, over a range of images.  Per image and band of output rows:
//   1. KW copies of the band's input rows of the 16 channels go to LDS,
//      copy kw shifted by kw*dw - pw columns (zeros outside X), so that for
//      every tap (kh, kw) the 8 pixels of an MFMA operand are one aligned
//      16-byte LDS read: copy kw, row r + kh*dh, columns ow .. ow+7.  A copy
//      piece is cut in registers out of the three 16-byte pieces of the
//      input row around it (the shift is uniform: one switch case);
//   2. steps of 32 pixels: the G operand (8 pixels of one output channel)
//      arrives through a per-wave LDS ring filled by buffer_load ... lds two
//      steps ahead (across band and image boundaries, so the next image's
//      first steps load during its copies), no registers held; each lane
//      reads back its own 16 bytes after an explicit vmcnt wait.  Per tap one
//      LDS read and 4 MFMAs (v_mfma_f32_16x16x32_f16, reduction = pixels).
// The blocks of channel tile 0 also sum G against an operand of ones (the
// bias gradient).  Partials per image range go to [range][M][K (+1)], summed
// by wgrad_reduce_kernel.  Blocks that share an image range and output
// channels (they differ only in channel tile) are 8 block ids apart: the
// same XCD, so G is read once per XCD's L2.
constexpr int kTapCT = 16;            // input channels per block
constexpr int kTapMaxTaps = 9;
constexpr int kTapRing = 3;           // G steps in the per-wave LDS ring: the current one + 2 ahead
constexpr size_t kTapRingBytes = (size_t)4 * kTapRing * 4 * 64 * 16;  // 4 waves x ring x 4 tiles x 1 KB
constexpr size_t kTapLds = 80 * 1024;  // two blocks per CU

struct TapGeo {
  int BR;        // output rows per band
  int R;         // box rows per band: BR + (KH-1)*dh
  int nband;     // bands per image
  int nct, nmt;  // channel tiles, 256-channel output tiles
  int splits, ipb;
  int Kq;        // partial row: K (+1 bias column)
  int has_db;
  int64_t outer;   // splits * G * nmt
  int64_t blocks;  // outer rounded up to 8, times nct
  size_t lds;      // bytes
};

// Elements 8+S .. 15+S of the 24 halves pc[0] | pc[1] | pc[2] (S compile-time).
template <int S>
__device__ __forceinline__ half8 window_t(const half8 (&pc)[3]) {
  half8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = 8 + S + e;
    r[e] = k < 8 ? pc[0][k & 7] : (k < 16 ? pc[1][k & 7] : pc[2][k & 7]);
  }
  return r;
}

// The same for a shift s in [-8, 8] that is uniform across the block.
__device__ __forceinline__ half8 window(int s, const half8 (&pc)[3]) {
  switch (s) {
#define FC_WIN(S) \
  case S: return window_t<S>(pc);
    FC_WIN(-8) FC_WIN(-7) FC_WIN(-6) FC_WIN(-5) FC_WIN(-4) FC_WIN(-3) FC_WIN(-2) FC_WIN(-1)
    FC_WIN(0) FC_WIN(1) FC_WIN(2) FC_WIN(3) FC_WIN(4) FC_WIN(5) FC_WIN(6) FC_WIN(7) FC_WIN(8)
#undef FC_WIN
    default: return half8{};
  }
}

template <int TAPS>
__global__ __launch_bounds__(kThreads, 2) void wgrad_tap_kernel(const half_t* __restrict__ x,
                                                                const half_t* __restrict__ dy,
                                                                float* __restrict__ part,
                                                                ConvParams cp, TapGeo tg) {
  extern __shared__ __attribute__((aligned(16))) half_t lds[];
  const int64_t b = blockIdx.x;
  const int ct = (int)((b >> 3) % tg.nct);
  const int64_t outer = ((b >> 3) / tg.nct) * 8 + (b & 7);
  if (outer >= tg.outer) return;
  const int mt = (int)(outer % tg.nmt);
  const int64_t t2 = outer / tg.nmt;
  const int g = (int)(t2 % cp.G);
  const int s = (int)(t2 / cp.G);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int m0 = mt * 256 + wave * 64;
  const int c0 = ct * kTapCT;
  const int R = tg.R, W = cp.W, OW = cp.OW;
  const int64_t P = cp.out_sz;
  // [KW][16][CP]: channel planes of R rows x OW, CP = R*OW + 8 halves apart
  // (16 bytes of skew: the 16 channels of an operand read then fall on 16
  // different 4-bank groups)
  const int CP = R * OW + 8;
  half_t* cpy = lds;
  // LDS offset of tap t's operand relative to copy 0, row 0
  int toff[TAPS];
#pragma unroll
  for (int t = 0; t < TAPS; ++t) {
    const int kh = t / cp.KW, kw = t - kh * cp.KW;
    toff[t] = kw * kTapCT * CP + kh * cp.dh * OW;
  }
  const bool do_db = tg.has_db && ct == 0;
  const half8 ones = {1, 1, 1, 1, 1, 1, 1, 1};
  // the wave's G ring: slot k, tile i at ring + (k*4 + i)*512 halves, lane l's
  // 16 bytes at + 8l (buffer_load ... lds writes a wave's 64 pieces in lane order)
  half_t* ring = lds + (tg.lds - kTapRingBytes) / sizeof(half_t) + wave * (kTapRing * 4 * 512);
  const int64_t n0 = (int64_t)s * tg.ipb;
  const int nimg = (int)std::min<int64_t>(tg.ipb, cp.n - n0);
  const int rows_ok = std::max(0, std::min(64, cp.Mg - m0));  // valid G rows of this wave
  // issue pointer: the next (image, band, step) whose G operands are loaded
  int iss_img = 0, iss_band = 0, iss_st = 0, issued = 0;
  auto band_steps = [&](int band) __attribute__((always_inline)) {
    return (std::min(tg.BR, cp.OH - band * tg.BR) * OW + 31) / 32;
  };
  auto issue = [&]() __attribute__((always_inline)) {
    if (iss_img >= nimg) return;
    const int64_t n = n0 + iss_img;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(dy + (n * cp.M + (int64_t)g * cp.Mg + m0) * P), (short)0,
        (int)((int64_t)rows_ok * P * (int64_t)sizeof(half_t)), 0x00020000);
    const int oh0 = iss_band * tg.BR;
    const int bandpix = std::min(tg.BR, cp.OH - oh0) * OW;
    const int p = iss_st * 32 + 8 * q;
    half_t* slot = ring + (issued % kTapRing) * 4 * 512;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = i * 16 + r16;
      const unsigned off = (p < bandpix && row < rows_ok)
                               ? (unsigned)(((int64_t)row * P + (int64_t)oh0 * OW + p) * 2)
                               : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(slot + i * 512), 16, off, 0, 0, 0);
    }
    ++issued;
    if (++iss_st == band_steps(iss_band)) {
      iss_st = 0;
      if (++iss_band == tg.nband) {
        iss_band = 0;
        ++iss_img;
      }
    }
  };
  // before the first copies: their loads hide the first steps' latency
  for (int k = 0; k < kTapRing - 1; ++k) issue();

  float4v acc[4][TAPS], dacc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dacc[i] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < TAPS; ++t) acc[i][t] = float4v{0.f, 0.f, 0.f, 0.f};
  }
  const int W8 = W / 8, OW8 = OW / 8;
  int cur = 0;  // steps consumed
  for (int ii = 0; ii < nimg; ++ii) {
    const int64_t n = n0 + ii;
    const half_t* xg = x + (n * cp.C + (int64_t)g * cp.Cg + c0) * cp.in_sz;
    for (int band = 0; band < tg.nband; ++band) {
      const int oh0 = band * tg.BR;
      // 1. the KW shifted copies of the band's input rows, straight from X:
      // a copy piece (8 output columns) is a window of the three 16-byte
      // pieces of the input row around it (zeros outside X)
      if (band > 0 || ii > 0) __syncthreads();  // the previous products are done
      for (int i = tid; i < kTapCT * R * OW8; i += kThreads) {
        const int c = i / (R * OW8), r2 = i - c * (R * OW8);
        const int rr = r2 / OW8, u = r2 - rr * OW8;
        const int ih = oh0 - cp.ph + rr;
        const bool rok = (unsigned)ih < (unsigned)cp.H;
        const half_t* row = xg + (int64_t)c * cp.in_sz + (int64_t)(rok ? ih : 0) * W;
        half8 pc[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
          const int pu = u - 1 + k;
          pc[k] = (rok && (unsigned)pu < (unsigned)W8) ? *(const half8*)(row + 8 * pu) : half8{};
        }
        half_t* dst = cpy + c * CP + rr * OW + 8 * u;
        for (int kw = 0; kw < cp.KW; ++kw)
          *(half8*)(dst + kw * kTapCT * CP) = window(kw * cp.dw - cp.pw, pc);
      }
      __syncthreads();
      // 2. products over the band's pixels
      const int bandpix = std::min(tg.BR, cp.OH - oh0) * OW;
      const int nst = (bandpix + 31) / 32;
      int r = (8 * q) / OW, ow = 8 * q - r * OW;  // this lane's pixels in the band
      for (int st = 0; st < nst; ++st) {
        // keep two steps ahead in the ring; then wait for this step's four
        // loads (a wave's loads complete in issue order, and nothing but
        // these ring loads is in flight here)
        while (issued < cur + kTapRing && iss_img < nimg) issue();
        __builtin_amdgcn_sched_barrier(0);
        switch (issued - cur - 1) {
          case 0: __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8)); break;
          case 1: __builtin_amdgcn_s_waitcnt(4 | (7 << 4) | (15 << 8)); break;
          default: __builtin_amdgcn_s_waitcnt(8 | (7 << 4) | (15 << 8)); break;
        }
        __builtin_amdgcn_sched_barrier(0);
        half8 a[4];
        const half_t* slot = ring + (cur % kTapRing) * 4 * 512 + lane * 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = *(const half8*)(slot + i * 512);
        const bool ok = st * 32 + 8 * q < bandpix;
        const half_t* cb = cpy + r16 * CP + (ok ? r : 0) * OW + (ok ? ow : 0);
        half8 bv[TAPS];
        if ((st + 1) * 32 <= bandpix) {  // a full step: every lane's pixels are in the band
#pragma unroll
          for (int t = 0; t < TAPS; ++t) bv[t] = *(const half8*)(cb + toff[t]);
        } else {  // the band's last, partial step: zero operands past its end
#pragma unroll
          for (int t = 0; t < TAPS; ++t) bv[t] = ok ? *(const half8*)(cb + toff[t]) : half8{};
        }
#pragma unroll
        for (int t = 0; t < TAPS; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], bv[t], acc[i][t], 0, 0, 0);
        if (do_db) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            dacc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], ones, dacc[i], 0, 0, 0);
        }
        ++cur;
        ow += 32;
        while (ow >= OW) {
          ow -= OW;
          ++r;
        }
      }
    }
  }
  // wait states between the last products and the VALU reads of their
  // accumulators
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  // lane: rows (channels) 4q + r, column r16 (input channel c0 + r16) of
  // every tap's tile; the ones column gives the same sum in every column
  float* pb = part + ((int64_t)s * cp.M + (int64_t)g * cp.Mg) * tg.Kq;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + i * 16 + q * 4 + r;
      if (m >= cp.Mg) continue;
#pragma unroll
      for (int t = 0; t < TAPS; ++t) pb[(int64_t)m * tg.Kq + (c0 + r16) * TAPS + t] = acc[i][t][r];
      if (do_db && r16 == 0) pb[(int64_t)m * tg.Kq + cp.K] = dacc[i][r];
    }
}

bool tap_plan(const ConvParams& cp, int32_t dtype, int has_db, TapGeo& tg, size_t* part_bytes) {
  if (dtype != FUSEDCONV_F16 || cp.transposed || cp.D != 1 || cp.KD != 1 || cp.OD != 1 ||
      cp.pd != 0 || cp.sh != 1 || cp.sw != 1)
    return false;
  if (cp.KH * cp.KW > kTapMaxTaps || cp.W % 8 || cp.OW % 8 || cp.Cg % kTapCT) return false;
  // a copy's column shift kw*dw - pw stays within one 16-byte piece either side
  if (cp.pw > 8 || (int64_t)(cp.KW - 1) * cp.dw - cp.pw > 8) return false;
  if ((int64_t)cp.H * cp.W >= ((int64_t)1 << 31) || cp.out_sz >= ((int64_t)1 << 31)) return false;
  const int span = (cp.KH - 1) * cp.dh;
  // the largest band of output rows whose rows and copies fit the LDS budget
  // copies: KW x 16 channel planes of R*OW + 8 halves
  const size_t per_row = (size_t)kTapCT * cp.KW * cp.OW * sizeof(half_t);
  const size_t skew = (size_t)kTapCT * cp.KW * 8 * sizeof(half_t);
  if (kTapLds < kTapRingBytes + skew) return false;
  const int64_t rmax = (int64_t)((kTapLds - kTapRingBytes - skew) / per_row);
  if (rmax < span + 1) return false;
  tg.BR = (int)std::min<int64_t>(cp.OH, rmax - span);
  tg.R = tg.BR + span;
  tg.nband = (int)cdiv(cp.OH, tg.BR);
  tg.lds = (size_t)tg.R * per_row + skew + kTapRingBytes;
  tg.nct = cp.Cg / kTapCT;
  tg.nmt = (int)cdiv(cp.Mg, 256);
  tg.has_db = has_db;
  tg.Kq = cp.K + has_db;
  const int64_t tiles = (int64_t)cp.G * tg.nmt * tg.nct;
  // about two blocks per CU, at least one image per range
  const int64_t splits = std::max<int64_t>(1, std::min<int64_t>(cp.n, cdiv(512, tiles)));
  tg.ipb = (int)cdiv(cp.n, splits);
  tg.splits = (int)cdiv(cp.n, tg.ipb);
  tg.outer = (int64_t)tg.splits * cp.G * tg.nmt;
  tg.blocks = cdiv(tg.outer, 8) * 8 * tg.nct;
  if (tg.blocks >= ((int64_t)1 << 31)) return false;
  *part_bytes = (size_t)tg.splits * cp.M * tg.Kq * sizeof(float);
  return true;
}

unsigned grid_for(int64_t work, int64_t cap) {
  int64_t b = (work + kThreads - 1) / kThreads;
  return (unsigned)std::max<int64_t>(1, std::min(b, cap));
}

template <typename T>
int launch_wgrad_t(const Geometry& g, const Plan& p, const void* x, const void* dy, float* dw,
                   float* db, void* ws, void* stream) {
  const ConvParams& cp = g.cp;
  RunArgs a{};
  a.stream = stream;
  if (p.route == FUSEDCONV_ROUTE_DIRECT) {
    const int has_db = db != nullptr;
    return launch_conv(wgrad_direct_kernel<T>, dim3((unsigned)((int64_t)cp.M * (cp.K + has_db))),
                       dim3(kThreads), 0, a, kEdgeNone, (const T*)x, (const T*)dy, dw, db, cp,
                       has_db);
  }
  if (p.route == FUSEDCONV_ROUTE_IGEMM_HALO) {
    if constexpr (sizeof(T) != 2) {
      return FUSEDCONV_ERR_ROUTE;
    } else {
      TapGeo tg;
      size_t part_bytes = 0;
      if (!tap_plan(cp, g.dtype, db != nullptr, tg, &part_bytes)) return FUSEDCONV_ERR_ROUTE;
      float* part = (float*)ws;
      int rc = FUSEDCONV_ERR_ROUTE;
      auto go = [&](auto kfn) -> int {
        if (set_max_dynamic_lds((const void*)kfn, (int)kTapLds) != FUSEDCONV_OK)
          return FUSEDCONV_ERR_LAUNCH;
        return launch_conv(kfn, dim3((unsigned)tg.blocks), dim3(kThreads), tg.lds, a, kEdgeNone,
                           (const half_t*)x, (const half_t*)dy, part, cp, tg);
      };
      switch (cp.KH * cp.KW) {
        case 1: rc = go(wgrad_tap_kernel<1>); break;
        case 2: rc = go(wgrad_tap_kernel<2>); break;
        case 3: rc = go(wgrad_tap_kernel<3>); break;
        case 4: rc = go(wgrad_tap_kernel<4>); break;
        case 5: rc = go(wgrad_tap_kernel<5>); break;
        case 6: rc = go(wgrad_tap_kernel<6>); break;
        case 7: rc = go(wgrad_tap_kernel<7>); break;
        case 8: rc = go(wgrad_tap_kernel<8>); break;
        case 9: rc = go(wgrad_tap_kernel<9>); break;
        default: break;
      }
      if (rc != FUSEDCONV_OK) return rc;
      WgGeo wg{};
      wg.Kq = tg.Kq;
      wg.splits = tg.splits;
      wg.has_db = tg.has_db;
      return launch_conv(wgrad_reduce_kernel, dim3(grid_for((int64_t)cp.M * wg.Kq, 8192)),
                         dim3(kThreads), 0, a, kEdgeNone, (const float*)part, dw, db, cp, wg);
    }
  }
  WgGeo wg;
  size_t col_bytes = 0, part_bytes = 0;
  if (!wg_plan(cp, g.dtype, db != nullptr, wg, &col_bytes, &part_bytes)) return FUSEDCONV_ERR_ROUTE;
  T* col = (T*)ws;
  float* part = (float*)((char*)ws + col_bytes);
  int rc = launch_columns(cp, g.dtype, x, col, wg.Kq, wg.Pp, wg.has_db, a, kEdgeNone);
  if (rc != FUSEDCONV_OK) return rc;
  const int64_t blocks = (int64_t)cp.G * wg.nmt * wg.nkt * wg.splits;
  rc = launch_conv(wgrad_gemm_kernel<T>, dim3((unsigned)blocks), dim3(kThreads), 0, a, kEdgeNone,
                   (const T*)dy, (const T*)col, part, cp, wg);
  if (rc != FUSEDCONV_OK) return rc;
  return launch_conv(wgrad_reduce_kernel, dim3(grid_for((int64_t)cp.M * wg.Kq, 8192)),
                     dim3(kThreads), 0, a, kEdgeNone, (const float*)part, dw, db, cp, wg);
}

}  // namespace

int launch_flip_weights(const ConvParams& f, int32_t dtype, const void* w, void* wf, void* stream) {
  const int64_t total = (int64_t)f.M * f.Cg * f.taps;
  const dim3 grid(grid_for(total, 4096)), block(kThreads);
  if (dtype == FUSEDCONV_F16)
    hipLaunchKernelGGL(flip_w_kernel<half_t>, grid, block, 0, (hipStream_t)stream,
                       (const half_t*)w, (half_t*)wf, f.Mg, f.Cg, f.G, f.taps);
  else
    hipLaunchKernelGGL(flip_w_kernel<float>, grid, block, 0, (hipStream_t)stream, (const float*)w,
                       (float*)wf, f.Mg, f.Cg, f.G, f.taps);
  return hipPeekAtLastError() == hipSuccess ? FUSEDCONV_OK : FUSEDCONV_ERR_LAUNCH;
}

bool wgrad_gemm_fits(const ConvParams& cp, int32_t dtype, int has_db, size_t* workspace,
                     int32_t* splits) {
  WgGeo wg;
  size_t col_bytes = 0, part_bytes = 0;
  if (!wg_plan(cp, dtype, has_db, wg, &col_bytes, &part_bytes)) return false;
  if (workspace) *workspace = col_bytes + part_bytes;
  if (splits) *splits = wg.splits;
  return true;
}

bool wgrad_tap_fits(const ConvParams& cp, int32_t dtype, int has_db, size_t* workspace,
                    int32_t* splits) {
  TapGeo tg;
  size_t part_bytes = 0;
  if (!tap_plan(cp, dtype, has_db, tg, &part_bytes)) return false;
  if (workspace) *workspace = part_bytes;
  if (splits) *splits = tg.splits;
  return true;
}

int launch_wgrad(const Geometry& g, const Plan& p, const void* x, const void* dy, float* dw,
                 float* db, void* ws, void* stream) {
  return g.dtype == FUSEDCONV_F16 ? launch_wgrad_t<half_t>(g, p, x, dy, dw, db, ws, stream)
                                  : launch_wgrad_t<float>(g, p, x, dy, dw, db, ws, stream);
}

}  // namespace fc
