// Implicit GEMM on MFMA with channel-last halo boxes (fp16 in, fp32 accumulate).
//
// Same GEMM view as the gathered-im2col route (rows = output pixels p of one
// image tile, columns = output channels m of one group, reduction over
// (input channel, tap)), but the reduction is ordered (channel block of 32,
// tap, channel within block) so that no im2col element is gathered one by
// one:
//   * per channel block, the input box that the tile's windows cover (the
//     tile's "halo", zero outside the image) is copied once into LDS in
//     channel-last layout [position][32 channels]; for tap t every output
//     pixel's 32-channel operand row is then one 64-byte LDS row at
//     position(p) + offset(t), and one lane's 8-channel slice is one
//     ds_read_b128;
//   * the weights are first repacked (every run) into a tap-major layout
//     Wp[g][tap][channel block][m][32] so the operand tile of one (tap,
//     channel block) is a contiguous BM x 64-byte block; it is staged in LDS,
//     double-buffered, one barrier per tap;
//   * v_mfma_f32_16x16x32_f16 with pixels as MFMA rows: each lane ends with 4
//     consecutive pixels of one output channel, so Z is read and Y written in
//     8-byte pieces in the fused epilogue (bias, residual, activation).
// The idea of feeding a matrix unit from an input tile that is staged once
// and re-read per tap is the one the FusedConv manifest's
// implicit_im2col_subgroup_matrix variants and the tinygrad page's shifted
// per-tap WMMA GEMMs use; the layouts and tiling here are gfx950-specific.
#include <hip/hip_runtime.h>

#include <stdlib.h>

#include <algorithm>

#include "epilogue.h"
#include "internal.h"

namespace fc {
namespace {

constexpr int kThreads = 256;
constexpr int kCB = 32;          // channels per block = MFMA K
constexpr int kLDC = kCB + 8;    // LDS row pitch in halves (80 bytes)
constexpr int kMaxItems = 4;     // loader items per thread kept in registers
constexpr size_t kMaxLds = 150 * 1024;  // above 80 KB a CU holds one block

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));

struct HaloTile {
  int TD, TH, TW;      // output tile
  int BD, BH, BW;      // input box
  int tiles_d, tiles_h, tiles_w;
  int ncb;             // channel blocks
  int mgp;             // Wp rows per (tap, channel block): M/group rounded up to BM
  int vec_x;           // W % 8 == 0: 16-byte aligned 8-column groups
  int ltw;             // log2(TW); tiles are one depth slice, TW and TH powers of two
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Dynamic LDS: two input boxes, and at least the epilogue staging area
// (4 waves x 16 channels x (BN/2 + 4) fp32).
size_t lds_bytes(int bpos, int bn) {
  const size_t boxes = (size_t)2 * bpos * kLDC * 2;
  const size_t stage = (size_t)4 * 16 * (bn / 2 + 4) * 4;
  return boxes > stage ? boxes : stage;
}

// Wp[((g*taps + t)*ncb + cb)*mgp + m][c'] = W[g*Mg + m][cb*32 + c'][t]; 0 past
// C/group and for the padding rows m >= M/group.
__global__ __launch_bounds__(kThreads) void repack_w_kernel(const half_t* __restrict__ w,
                                                            half_t* __restrict__ wp,
                                                            ConvParams cp, int ncb, int mgp) {
  const int64_t total = (int64_t)cp.G * cp.taps * ncb * mgp * kCB;
  const int64_t step = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += step) {
    const int cc = (int)(i % kCB);
    int64_t r = i / kCB;
    const int m = (int)(r % mgp);
    r /= mgp;
    const int cb = (int)(r % ncb);
    r /= ncb;
    const int t = (int)(r % cp.taps);
    const int g = (int)(r / cp.taps);
    const int c = cb * kCB + cc;
    wp[i] = (c < cp.Cg && m < cp.Mg) ? w[((int64_t)(g * cp.Mg + m) * cp.Cg + c) * cp.taps + t]
                                     : (half_t)0;
  }
}

// Block tile BN pixels x BM channels, 4 waves as 2 x 2, each owning
// (BN/2) x (BM/2) = TP x TM MFMA blocks of 16x16; two blocks per CU.  Steps
// run over (channel block, tap).  The input box of a channel block sits in
// LDS (double-buffered, one barrier per channel block); weight fragments come
// straight from the repacked buffer into registers one step ahead; input
// fragments are read from LDS at the start of their step.
// PFX: keep the next channel block's input in registers across a whole
// channel block (hides its load latency, costs ~30 registers); without it the
// box is loaded right before it is stored.
template <int BM, int BN, bool PFX>
__global__ __launch_bounds__(kThreads, 2) void halo_kernel(const half_t* __restrict__ x,
                                                           const half_t* __restrict__ wp,
                                                           const half_t* __restrict__ bias,
                                                           const half_t* z, half_t* y,
                                                           ConvParams cp, HaloTile ht) {
  constexpr int TP = BN / 32;
  constexpr int TM = BM / 32;
  extern __shared__ __attribute__((aligned(16))) half_t lds[];
  const int box = ht.BD * ht.BH * ht.BW * kLDC;  // halves per input box

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wpi = wave & 1, wmi = wave >> 1;
  const int r16 = lane & 15, q = lane >> 4;

  // block -> (image, tile), m tile, group
  int64_t b = blockIdx.x;
  const int tw_i = (int)(b % ht.tiles_w);
  b /= ht.tiles_w;
  const int th_i = (int)(b % ht.tiles_h);
  b /= ht.tiles_h;
  const int td_i = (int)(b % ht.tiles_d);
  const int64_t n = b / ht.tiles_d;
  const int m0 = blockIdx.y * BM;
  const int g = blockIdx.z;
  const int od0 = td_i * ht.TD, oh0 = th_i * ht.TH, ow0 = tw_i * ht.TW;
  const int bd0 = od0 * cp.sd - cp.pd, bh0 = oh0 * cp.sh - cp.ph, bw0 = ow0 * cp.sw - cp.pw;

  // ---- zero both input boxes: positions outside the image stay zero
  for (int i = tid; i < 2 * box / 8; i += kThreads) ((half8*)lds)[i] = half8{};

  // ---- input loader items: (channel, d, h, aligned 8-column group) of the
  // in-image part of the box.  The first kMaxItems per thread keep their
  // decoded addresses in registers; further ones are decoded when stored.
  const int d_lo = max(bd0, 0), d_hi = min(bd0 + ht.BD, cp.D);
  const int h_lo = max(bh0, 0), h_hi = min(bh0 + ht.BH, cp.H);
  const int w_lo = max(bw0, 0), w_hi = min(bw0 + ht.BW, cp.W);
  const int g_lo = w_lo >> 3, g_hi = (w_hi + 7) >> 3;
  const int nd = d_hi - d_lo, nh = h_hi - h_lo, ngr = g_hi - g_lo;
  const int nitems = kCB * nd * nh * ngr;
  const half_t* ximg = x + (n * cp.C + (int64_t)g * cp.Cg) * cp.in_sz;
  int it_goff[kMaxItems];   // element offset from the channel block's first channel
  int it_dst[kMaxItems];    // LDS element offset of column 0 of the group, channel c
  int it_cm[kMaxItems];     // channel (bits 8..) and in-box column mask (bits 0..7); -1 none
#pragma unroll
  for (int k = 0; k < kMaxItems; ++k) {
    const int i = tid + k * kThreads;
    it_cm[k] = -1;
    it_goff[k] = it_dst[k] = 0;
    if (i < nitems) {
      int r = i;
      const int gi = r % ngr; r /= ngr;
      const int hh = r % nh; r /= nh;
      const int dd = r % nd;
      const int c = r / nd;
      const int id = d_lo + dd, ih = h_lo + hh, iw = (g_lo + gi) * 8;
      int mask = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (iw + e >= w_lo && iw + e < w_hi) mask |= 1 << e;
      it_cm[k] = (c << 8) | mask;
      it_goff[k] = c * (int)cp.in_sz + (id * cp.H + ih) * cp.W + iw;
      it_dst[k] = (((id - bd0) * ht.BH + (ih - bh0)) * ht.BW + (iw - bw0)) * kLDC + c;
    }
  }
  half8 xreg[kMaxItems];
#define HALO_LOAD_X(CB)                                                        \
  {                                                                            \
    const half_t* xb_ = ximg + (int64_t)(CB) * kCB * cp.in_sz;                 \
    const int cvalid_ = cp.Cg - (CB) * kCB;                                    \
    _Pragma("unroll") for (int k = 0; k < kMaxItems; ++k) {                    \
      half8 v_ = {};                                                           \
      if (it_cm[k] >= 0 && (it_cm[k] >> 8) < cvalid_) {                        \
        const half_t* src_ = xb_ + it_goff[k];                                 \
        if (ht.vec_x) {                                                        \
          v_ = *(const half8*)src_;                                            \
        } else {                                                               \
          _Pragma("unroll") for (int e = 0; e < 8; ++e) if ((it_cm[k] >> e) & 1) v_[e] = src_[e]; \
        }                                                                      \
      }                                                                        \
      xreg[k] = v_;                                                            \
    }                                                                          \
  }
  // store the box of channel block CB (held in xreg) into LDS buffer BUF
  auto store_x = [&](int buf, int cb) {
    half_t* xs = lds + buf * box;
#pragma unroll
    for (int k = 0; k < kMaxItems; ++k) {
      if (it_cm[k] < 0) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if ((it_cm[k] >> e) & 1) xs[it_dst[k] + e * kLDC] = xreg[k][e];
    }
    const half_t* xb = ximg + (int64_t)cb * kCB * cp.in_sz;
    const int cvalid = cp.Cg - cb * kCB;
    for (int i = tid + kMaxItems * kThreads; i < nitems; i += kThreads) {
      int r = i;
      const int gi = r % ngr; r /= ngr;
      const int hh = r % nh; r /= nh;
      const int dd = r % nd;
      const int c = r / nd;
      const int id = d_lo + dd, ih = h_lo + hh, iw = (g_lo + gi) * 8;
      const half_t* src = xb + c * (int)cp.in_sz + (id * cp.H + ih) * cp.W + iw;
      const int dst = (((id - bd0) * ht.BH + (ih - bh0)) * ht.BW + (iw - bw0)) * kLDC + c;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (iw + e >= w_lo && iw + e < w_hi) xs[dst + e * kLDC] = c < cvalid ? src[e] : (half_t)0;
    }
  };

  // ---- weight fragments straight from Wp (rows padded to ht.mgp with zeros):
  // fragment j of step (cb, t) = 16 rows x 64 bytes, each lane reads 16 bytes.
  const half_t* wlane = wp + (int64_t)g * cp.taps * ht.ncb * ht.mgp * kCB +
                        (int64_t)(m0 + wmi * (BM / 2) + r16) * kCB + q * 8;
  const int64_t wstep = (int64_t)ht.mgp * kCB;  // halves per (tap, channel block) tile

  // ---- per-lane LDS offsets (halves) of this lane's operand rows (pixels)
  int aoff[TP];
#pragma unroll
  for (int i = 0; i < TP; ++i) {
    const int pl = wpi * (BN / 2) + i * 16 + r16;
    const int tw = pl % ht.TW, th = (pl / ht.TW) % ht.TH, td = pl / (ht.TW * ht.TH);
    aoff[i] = (((td * cp.sd) * ht.BH + th * cp.sh) * ht.BW + tw * cp.sw) * kLDC + q * 8;
  }

  float4v acc[TP][TM];
#pragma unroll
  for (int i = 0; i < TP; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = float4v{0.0f, 0.0f, 0.0f, 0.0f};

  const int taps = cp.taps, ncb = ht.ncb, nsteps = ncb * taps;
  __syncthreads();  // zero fill done before any box write
  HALO_LOAD_X(0);
  store_x(0, 0);
  if (PFX && ncb > 1) HALO_LOAD_X(1);
  // Step bookkeeping is incremental (uniform, scalar): the weight tile of
  // step (cb, t) is Wp tile t * ncb + cb, the box offset of tap (kd, kh, kw)
  // is ((kd*dd*BH + kh*dh)*BW + kw*dw) positions.
  const int dkw = cp.dw * kLDC;
  const int dkh = (cp.dh * ht.BW - (cp.KW - 1) * cp.dw) * kLDC;
  const int dkd = (cp.dd * ht.BH * ht.BW - (cp.KH - 1) * cp.dh * ht.BW - (cp.KW - 1) * cp.dw) * kLDC;
  const int64_t wtap = (int64_t)ncb * wstep;                 // next tap, same channel block
  const int64_t wcb = wstep - (int64_t)(taps - 1) * ncb * wstep;  // next channel block, tap 0

  // weight fragments: two register sets, prefetch distance one step
  half8 wa[TM], wb[TM];
#pragma unroll
  for (int j = 0; j < TM; ++j) wa[j] = *(const half8*)(wlane + j * 16 * kCB);
  int64_t wnext = (taps > 1) ? wtap : wcb;                   // Wp offset of step 1
  __syncthreads();

  int cb = 0, t = 0, kd = 0, kh = 0, kw = 0, toff = 0;
#define HALO_STEP(WC, WN, HAS_NEXT)                                                      \
  {                                                                                      \
    if (t == taps - 1 && cb + 1 < ncb) {                                                 \
      if (!PFX) HALO_LOAD_X(cb + 1);                                                     \
      store_x((cb + 1) & 1, cb + 1);                                                     \
      __syncthreads();                                                                   \
      if (PFX && cb + 2 < ncb) HALO_LOAD_X(cb + 2);                                      \
    }                                                                                    \
    if (HAS_NEXT) {                                                                      \
      const half_t* sn_ = wlane + wnext;                                                 \
      _Pragma("unroll") for (int j = 0; j < TM; ++j) WN[j] = *(const half8*)(sn_ + j * 16 * kCB); \
    }                                                                                    \
    const half_t* xs_ = lds + (cb & 1) * box + toff;                                     \
    half8 a_[TP];                                                                        \
    _Pragma("unroll") for (int i = 0; i < TP; ++i) a_[i] = *(const half8*)(xs_ + aoff[i]); \
    _Pragma("unroll") for (int i = 0; i < TP; ++i)                                       \
      _Pragma("unroll") for (int j = 0; j < TM; ++j)                                     \
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_[i], WC[j], acc[i][j], 0, 0, 0); \
    /* advance to the next step */                                                       \
    if (++t == taps) {                                                                   \
      t = kd = kh = kw = toff = 0;                                                       \
      ++cb;                                                                              \
    } else if (++kw < cp.KW) {                                                           \
      toff += dkw;                                                                       \
    } else if (kw = 0, ++kh < cp.KH) {                                                   \
      toff += dkh;                                                                       \
    } else {                                                                             \
      kh = 0;                                                                            \
      ++kd;                                                                              \
      toff += dkd;                                                                       \
    }                                                                                    \
    /* Wp offset of the step after the new current one */                               \
    wnext += (t == taps - 1) ? wcb : wtap;                                               \
  }
  int s = 0;
  for (; s + 1 < nsteps; s += 2) {
    HALO_STEP(wa, wb, true);
    HALO_STEP(wb, wa, s + 2 < nsteps);
  }
  if (s < nsteps) HALO_STEP(wa, wb, false);
#undef HALO_STEP
#undef HALO_LOAD_X

  // ---- epilogue.  The accumulators go through LDS (the boxes are dead now)
  // one 16-channel block at a time: staged as 16 rows of consecutive pixels,
  // Z is added into the stage with loads issued a pass ahead, then a rolled
  // loop applies bias and activation and stores Y; consecutive lanes touch
  // consecutive 8-byte pieces of a row.
  __syncthreads();
  constexpr int PW = BN / 2;              // pixels per wave
  constexpr int RP = PW + 4;              // fp32 row pitch (padded)
  constexpr int GPR = PW / 4;             // 4-pixel groups per row
  constexpr int ITER = 16 * GPR / 64;     // groups per lane per pass
  float* stage = (float*)lds + wave * 16 * RP;
  const bool vec_ok = (cp.OW & 3) == 0;
  // per-lane slots of a pass: row (channel within the block) and 4 pixels
  int slot_lds[ITER], slot_nv[ITER];
  int64_t slot_y[ITER];                   // Y offset of the slot for channel block 0
  const int mw = m0 + wmi * (BM / 2);     // first channel of this wave
#pragma unroll
  for (int it = 0; it < ITER; ++it) {
    const int idx = it * 64 + lane;
    const int row = idx / GPR, p4 = (idx % GPR) * 4;
    const int pl = wpi * PW + p4;
    const int tw = pl % ht.TW, th = (pl / ht.TW) % ht.TH, td = pl / (ht.TW * ht.TH);
    const int od = od0 + td, oh = oh0 + th, ow = ow0 + tw;
    const bool ok = od < cp.OD && oh < cp.OH && ow < cp.OW;
    slot_lds[it] = row * RP + p4;
    slot_nv[it] = ok ? min(4, cp.OW - ow) : 0;
    slot_y[it] = (n * cp.M + g * cp.Mg + mw + row) * cp.out_sz +
                 ((int64_t)od * cp.OH + oh) * cp.OW + ow;
  }
  half4 zv[TM][ITER];
  auto load_z = [&](int j) {
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      half4 v = {};
      const int m = mw + j * 16 + (it * 64 + lane) / GPR;
      if (cp.has_z && slot_nv[it] > 0 && m < cp.Mg) {
        const half_t* zp = z + slot_y[it] + (int64_t)j * 16 * cp.out_sz;
        if (vec_ok && slot_nv[it] == 4) {
          v = *(const half4*)zp;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (r < slot_nv[it]) v[r] = zp[r];
        }
      }
      zv[j][it] = v;
    }
  };
  // every Z value of this wave is requested before any is needed
  if (cp.has_z) {
#pragma unroll
    for (int j = 0; j < TM; ++j) load_z(j);
  }
#pragma unroll
  for (int j = 0; j < TM; ++j) {
#pragma unroll
    for (int i = 0; i < TP; ++i) *(float4v*)(stage + r16 * RP + i * 16 + q * 4) = acc[i][j];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (cp.has_z) {
#pragma unroll
      for (int it = 0; it < ITER; ++it) {
        float4v* sp = (float4v*)(stage + slot_lds[it]);
        float4v v = *sp;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] += (float)zv[j][it][r];
        *sp = v;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // rolled: slot coordinates are recomputed with shifts (tile width and
    // height are powers of two), the activation is dispatched per 4 values
    for (int it = 0; it < ITER; ++it) {
      const int idx = it * 64 + lane;
      const int row = idx / GPR, p4 = (idx % GPR) * 4;
      const int m = mw + j * 16 + row;
      const int pl = wpi * PW + p4;
      const int oh = oh0 + (pl >> ht.ltw), ow = ow0 + (pl & (ht.TW - 1));
      if (m >= cp.Mg || oh >= cp.OH || ow >= cp.OW) continue;
      const int nv = min(4, cp.OW - ow);
      const int64_t yi = (n * cp.M + g * cp.Mg + m) * cp.out_sz +
                         ((int64_t)od0 * cp.OH + oh) * cp.OW + ow;
      float4v v4 = *(const float4v*)(stage + row * RP + p4);
      const float bv = cp.has_bias ? to_f32(bias[g * cp.Mg + m]) : 0.0f;
      v4 += bv;
      v4 = act_apply4(cp.act, v4, cp.alpha, cp.beta);
      half4 out;
#pragma unroll
      for (int r = 0; r < 4; ++r) out[r] = (half_t)v4[r];
      if (vec_ok && nv == 4) {
        *(half4*)(y + yi) = out;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (r < nv) y[yi + r] = out[r];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

struct Choice {
  int bm, bn, waves;
  HaloTile ht;
};

// Pick BM, BN and the output tile; false if nothing fits.
bool choose(const ConvParams& cp, Choice& ch) {
  if (cp.Cg < 16) return false;
  // BM = 256 with 4 waves spills registers: 128 output channels per block.
  const int bm = 128;
  const int ncb = (int)cdiv(cp.Cg, kCB);
  const int waves = 4;
  const int tws[] = {16, 32, 64, 128, 256};
  int bn_first = 256;  // FUSEDCONV_HALO_BN=128 restricts the tile to 128 pixels (tuning)
  if (const char* e = getenv("FUSEDCONV_HALO_BN")) bn_first = atoi(e) == 128 ? 128 : 256;
  for (int bn : {256, 128}) {
    if (bn > bn_first) continue;
    // tile widths (multiples of 16; tile = bn / tw rows) in order of padded
    // output area, ties to the wider tile; the first that fits is taken
    int order[5], no = 0;
    double waste[5];
    for (int c : tws) {
      if (c > bn) break;
      waste[no] = (double)cdiv(cp.OH, bn / c) * (bn / c) * cdiv(cp.OW, c) * c /
                  ((double)cp.OH * cp.OW);
      order[no] = c;
      ++no;
    }
    for (int a = 0; a < no; ++a)
      for (int b2 = a + 1; b2 < no; ++b2)
        if (waste[b2] < waste[a] - 1e-9 ||
            (waste[b2] < waste[a] + 1e-9 && order[b2] > order[a])) {
          std::swap(waste[a], waste[b2]);
          std::swap(order[a], order[b2]);
        }
    for (int oi = 0; oi < no; ++oi) {
      const int tw = order[oi], th = bn / tw, td = 1;
      HaloTile ht;
      ht.TD = td; ht.TH = th; ht.TW = tw;
      ht.ltw = 31 - __builtin_clz((unsigned)tw);
      ht.BD = (td - 1) * cp.sd + (cp.KD - 1) * cp.dd + 1;
      ht.BH = (th - 1) * cp.sh + (cp.KH - 1) * cp.dh + 1;
      ht.BW = (tw - 1) * cp.sw + (cp.KW - 1) * cp.dw + 1;
      ht.tiles_d = (int)cdiv(cp.OD, td);
      ht.tiles_h = (int)cdiv(cp.OH, th);
      ht.tiles_w = (int)cdiv(cp.OW, tw);
      ht.ncb = ncb;
      ht.mgp = (int)(cdiv(cp.Mg, bm) * bm);
      ht.vec_x = (cp.W % 8) == 0;
      const int64_t bpos = (int64_t)ht.BD * ht.BH * ht.BW;
      if (bpos > (1 << 20) || lds_bytes((int)bpos, bn) > kMaxLds) continue;
      const int64_t blocks = cp.n * ht.tiles_d * ht.tiles_h * ht.tiles_w;
      if (blocks >= ((int64_t)1 << 31) || cdiv(cp.Mg, bm) > 65535 || cp.G > 65535) continue;
      // the tiles must not be mostly padding
      if ((double)ht.tiles_d * td * ht.tiles_h * th * ht.tiles_w * tw > 2.0 * cp.out_sz) continue;
      ch.bm = bm;
      ch.bn = bn;
      ch.waves = waves;
      ch.ht = ht;
      return true;
    }
  }
  return false;
}

int launch_repack(const ConvParams& cp, const Choice& ch, const RunArgs& a) {
  const int64_t total = (int64_t)cp.G * cp.taps * ch.ht.ncb * ch.ht.mgp * kCB;
  int64_t rblocks = (total + kThreads - 1) / kThreads;
  if (rblocks > 4096) rblocks = 4096;
  hipLaunchKernelGGL(repack_w_kernel, dim3((unsigned)rblocks), dim3(kThreads), 0,
                     (hipStream_t)a.stream, (const half_t*)a.w, (half_t*)a.ws, cp, ch.ht.ncb,
                     ch.ht.mgp);
  return hipPeekAtLastError() == hipSuccess ? FUSEDCONV_OK : FUSEDCONV_ERR_LAUNCH;
}

template <int BM, int BN, bool PFX>
int launch_t(const Geometry& g, const Choice& ch, const RunArgs& a) {
  const ConvParams& cp = g.cp;
  hipStream_t st = (hipStream_t)a.stream;
  const int bpos = ch.ht.BD * ch.ht.BH * ch.ht.BW;
  const size_t lds = lds_bytes(bpos, BN);
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)halo_kernel<BM, BN, PFX>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds) !=
        hipSuccess)
      return FUSEDCONV_ERR_LAUNCH;
    attr_set = true;
  }
  if (!(a.flags & FUSEDCONV_RUN_WEIGHTS_PREPARED)) {
    const int rc = launch_repack(cp, ch, a);
    if (rc != FUSEDCONV_OK) return rc;
  }
  dim3 grid((unsigned)(cp.n * ch.ht.tiles_d * ch.ht.tiles_h * ch.ht.tiles_w),
            (unsigned)cdiv(cp.Mg, BM), (unsigned)cp.G);
  hipLaunchKernelGGL((halo_kernel<BM, BN, PFX>), grid, dim3(kThreads), lds, st, (const half_t*)a.x,
                     (const half_t*)a.ws, (const half_t*)a.bias, (const half_t*)a.z,
                     (half_t*)a.y, cp, ch.ht);
  return hipPeekAtLastError() == hipSuccess ? FUSEDCONV_OK : FUSEDCONV_ERR_LAUNCH;
}

}  // namespace

bool igemm_halo_fits(const ConvParams& cp, int32_t dtype, int32_t& tile_h, int32_t& tile_w,
                     size_t& workspace) {
  if (dtype != FUSEDCONV_F16 || cp.taps > 64) return false;
  Choice ch;
  if (!choose(cp, ch)) return false;
  tile_h = ch.ht.TH;
  tile_w = ch.ht.TW;
  workspace = (size_t)cp.G * cp.taps * ch.ht.ncb * ch.ht.mgp * kCB * sizeof(half_t);
  return true;
}

int prepare_igemm_halo(const Geometry& g, const Plan&, const RunArgs& a) {
  Choice ch;
  if (!choose(g.cp, ch)) return FUSEDCONV_ERR_ROUTE;
  return launch_repack(g.cp, ch, a);
}

int launch_igemm_halo(const Geometry& g, const Plan&, const RunArgs& a) {
  Choice ch;
  if (!choose(g.cp, ch)) return FUSEDCONV_ERR_ROUTE;
  return ch.bn == 256 ? launch_t<128, 256, true>(g, ch, a) : launch_t<128, 128, true>(g, ch, a);
}

}  // namespace fc
