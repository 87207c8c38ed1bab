// Implicit GEMM on the fp32 matrix cores with channel-last halo boxes (fp32
// in, fp32 accumulate, true fp32 products: v_mfma_f32_16x16x4_f32).
//
// The fp16 halo kernel's structure (kernels_halo.hip), re-cut for fp32:
//   * per block of 16 input channels, the input box that a tile's windows
//     cover (zero outside the image) is copied once into LDS, channel-last
//     [position][16 channels + 4 pad], positions split by stride phase, so
//     for tap t every output pixel's 16-channel row is the LDS row at
//     pixel(p) + offset(t);
//   * a lane's operand is 4 consecutive channels of one pixel (one
//     ds_read_b128), fed to four MFMAs: MFMA e contracts channel 4q + e of
//     lane group q, for A (the pixels) and B (the weights) alike, so every
//     channel is summed once;
//   * the weights, repacked tap-major as Wp[g][tap][channel block][m][16]
//     (fusedconv_prepare_weights or at the start of every run), go straight
//     into registers one (channel block, tap) step ahead;
//   * bias seeds the accumulators; Z and the activation follow per lane (4
//     consecutive pixels of one output channel), and where two pixel tiles
//     make 32 whole pixels of a row, lanes 8 apart swap halves so that each
//     store instruction writes whole 128-byte lines.
// The per-element im2col gather of the IGEMM route, whose loads wait at the
// joins of their bounds tests, is gone: X is read once per channel block as
// whole 16-byte rows of the box.
// Depth-stepped form (DS): when a 3-D tile's box, every kernel depth at
// once, does not fit, the box holds one input depth plane and the K loop
// walks (channel block, kernel depth kd, in-plane tap): plane kd of a tile at
// output depth od is input depth od*sd - pd + kd*dd, planes outside the input
// are skipped (their products are zero), and one box buffer per block (two
// blocks per CU) takes the next plane after a barrier.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "epilogue.h"
#include "internal.h"
#include "launch.h"
#include "sync.h"

namespace fc {
namespace {

constexpr int kThreads = 256;   // 4 waves
constexpr int kCB = 16;         // input channels per box
constexpr int kLdc = 20;        // floats per LDS box row (80 bytes: 16 channels + 4 pad)
constexpr size_t kMaxLds = 64 * 1024;  // two boxes; two blocks per CU
constexpr int kMaxTaps = 64;

typedef float float4v __attribute__((ext_vector_type(4)));

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int log2i(int v) { return 31 - __builtin_clz((unsigned)v); }

struct Geo32 {
  int ds;                    // depth-stepped: the box is one input depth plane
  int taps2;                 // taps per box: KH*KW when depth-stepped, else all taps
  int TD, TH, TW, ltw, lth;  // output tile (TW a power of two >= 16)
  int BD, BH, BW;            // input box extents
  int ND, NH, NW;            // positions per stride phase
  int LH, LW;                // LDS pitches in positions
  int box_pos;               // positions per box
  int tiles_d, tiles_h, tiles_w;
  int ntile;
  int nmb, ncb, mgp;         // m blocks, channel blocks, Wp rows per (tap, block)
  int vec;                   // W % 4 == 0: 16-byte row loads
  int tap_off[kMaxTaps];     // LDS row offset (positions) of each tap of a box
};

__device__ __forceinline__ int phase_index(int a, int s, int n) {
  if (s == 1) return a;
  return (a % s) * n + a / s;
}

// Wp[((g*taps + t)*ncb + cb)*mgp + m][c'] = W[g*Mg + m][cb*16 + c'][t]; zero
// past C/group and for rows m >= M/group.
__global__ __launch_bounds__(kThreads) void repack32_kernel(const float* __restrict__ w,
                                                            float* __restrict__ wp, ConvParams cp,
                                                            int ncb, int mgp) {
  const int cpad = ncb * kCB;
  const int total = cp.G * mgp * cpad;
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < total; i += gridDim.x * kThreads) {
    const int c = i % cpad;
    const int r = i / cpad;
    const int m = r % mgp;
    const int g = r / mgp;
    const bool ok = c < cp.Cg && m < cp.Mg;
    const float* src = w + ((int64_t)(g * cp.Mg + (ok ? m : 0)) * cp.Cg + (ok ? c : 0)) * cp.taps;
    float* dst = wp + (((int64_t)g * cp.taps * ncb + c / kCB) * mgp + m) * kCB + c % kCB;
    for (int t = 0; t < cp.taps; ++t) dst[(int64_t)t * ncb * mgp * kCB] = ok ? src[t] : 0.0f;
  }
}

// Block tile: WGP x WGM waves, each 64 pixels x 64 output channels (4 x 4
// MFMA tiles of 16 x 16); BN = 64*WGP pixels, BM = 64*WGM channels.
template <int WGP, bool DS>
__global__ __launch_bounds__(kThreads, 2) void halo32_kernel(const float* __restrict__ x,
                                                             const float* __restrict__ wp,
                                                             const float* __restrict__ bias,
                                                             const float* z, const float* pre,
                                                             float* y, ConvParams cp, Geo32 hg) {
  constexpr int WGM = 4 / WGP;
  constexpr int BM = 64 * WGM;  // the block's channels (its pixels: 64 * WGP)
  extern __shared__ __attribute__((aligned(16))) float lds32[];
  const int box = hg.box_pos * kLdc;  // floats per box

  // ---- block -> (group, m block, tile).  Block b runs on XCD b % 8.  With
  // full-depth boxes, in each whole chunk of 256 block ids XCD x takes the 32
  // consecutive work units 32x .. 32x + 31 of the chunk, so neighbouring
  // tiles, whose boxes share halo columns and rows, run on one XCD at about
  // the same time and read the shared lines from its L2.  Depth-stepped
  // tiles keep the plain order: the tiles of neighbouring output depths,
  // which read the same input planes, are tiles_h * tiles_w ids apart, on one
  // XCD when that is a multiple of 8.
  int bid = blockIdx.x;
  if (!DS && bid < (int)(gridDim.x & ~255u)) bid = (bid & ~255) + (bid & 7) * 32 + ((bid & 255) >> 3);
  const int per_g = hg.ntile * hg.nmb;
  const int g = bid / per_g;
  int rb = bid - g * per_g;
  const int mb = rb % hg.nmb;
  int tile = rb / hg.nmb;
  const int tw_i = tile % hg.tiles_w;
  tile /= hg.tiles_w;
  const int th_i = tile % hg.tiles_h;
  tile /= hg.tiles_h;
  const int td_i = tile % hg.tiles_d;
  const int64_t n = tile / hg.tiles_d;
  const int od0 = td_i * hg.TD, oh0 = th_i * hg.TH, ow0 = tw_i * hg.TW;
  const int bd0 = od0 * cp.sd - cp.pd, bh0 = oh0 * cp.sh - cp.ph, bw0 = ow0 * cp.sw - cp.pw;
  const int m0 = mb * BM;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wpi = wave % WGP, wmi = wave / WGP;
  const int r16 = lane & 15, q = lane >> 4;

  // ---- zero the boxes: positions outside the image stay zero
  constexpr int kBufs = DS ? 1 : 2;
  for (int i = tid; i < kBufs * box / 4; i += kThreads) ((float4v*)lds32)[i] = float4v{0.f, 0.f, 0.f, 0.f};

  // ---- boxes: (channel block cb, kernel depth kd) for bi = cb * nkd + (kd -
  // kd_lo); without depth steps one box per channel block (nkd = 1, kd = 0)
  int kd_lo = 0, nkd = 1;
  if constexpr (DS) {
    const int z0 = od0 * cp.sd - cp.pd;  // input depth of kd = 0
    while (kd_lo < cp.KD && z0 + kd_lo * cp.dd < 0) ++kd_lo;
    int kd_hi = kd_lo;
    while (kd_hi < cp.KD && z0 + kd_hi * cp.dd < cp.D) ++kd_hi;
    nkd = kd_hi - kd_lo;
  }
  const int nbox = hg.ncb * nkd;
  auto box_cb = [&](int bi) __attribute__((always_inline)) { return DS ? bi / nkd : bi; };
  auto box_kd = [&](int bi) __attribute__((always_inline)) { return DS ? kd_lo + bi % nkd : 0; };
  // element offset of box bi's input plane (depth-stepped) from the image base
  auto box_zoff = [&](int bi) __attribute__((always_inline)) {
    return DS ? (int64_t)(od0 * cp.sd - cp.pd + box_kd(bi) * cp.dd) * cp.H * cp.W : (int64_t)0;
  };

  // ---- box loader: item = (channel quad cq, in-image box row, 4-column
  // group): four 16-byte loads (4 channels, same 4 columns), written as up
  // to 4 LDS rows of 4 channels
  const int d_lo = DS ? 0 : max(bd0, 0), d_hi = DS ? 1 : min(bd0 + hg.BD, cp.D);
  const int h_lo = max(bh0, 0), h_hi = min(bh0 + hg.BH, cp.H);
  const int w_lo = max(bw0, 0), w_hi = min(bw0 + hg.BW, cp.W);
  const int g_lo = w_lo >> 2, g_hi = (w_hi + 3) >> 2;
  const int nd = max(d_hi - d_lo, 0), nh = max(h_hi - h_lo, 0), ngr = max(g_hi - g_lo, 0);
  const int nitems = 4 * nd * nh * ngr;
  const float* ximg = x + (n * cp.C + (int64_t)g * cp.Cg) * cp.in_sz;
  // items per thread held across a box: a depth plane of the 3-D conv's
  // 4 x 32 tile has 612 (3 per thread, 247 VGPRs, so none is loaded at the
  // box switch); a full-depth box holds 2 (a 256-pixel 1-D row box has 280)
  constexpr int PF = DS ? 3 : 2;
  struct Item { int goff, ldst, cq, mask, aw0; };
  auto decode = [&](int i) __attribute__((always_inline)) {
    Item it;
    it.cq = i & 3;
    int r = i >> 2;
    const int gi = r % ngr;
    r /= ngr;
    const int hh = r % nh;
    const int dd = r / nh;
    const int id = d_lo + dd, ih = h_lo + hh, iw = (g_lo + gi) * 4;
    int mask = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (iw + e >= w_lo && iw + e < w_hi) mask |= 1 << e;
    it.mask = mask;
    it.goff = (id * cp.H + ih) * cp.W + iw;
    it.ldst = ((DS ? 0 : phase_index(id - bd0, cp.sd, hg.ND)) * hg.LH + phase_index(ih - bh0, cp.sh, hg.NH)) *
              hg.LW;
    it.aw0 = iw - bw0;
    return it;
  };
  Item items[PF];
  float4v xr[PF][4];
  auto load_item = [&](const Item& it, int bi, float4v* v) __attribute__((always_inline)) {
    const int c0 = box_cb(bi) * kCB + it.cq * 4;
    const float* xz = ximg + box_zoff(bi);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = it.mask != 0 && c0 + j < cp.Cg;
      const float* s = ok ? xz + (int64_t)(c0 + j) * cp.in_sz + it.goff : x;
      if (hg.vec) {
        v[j] = *(const float4v*)s;
      } else {
        float4v t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (ok && ((it.mask >> e) & 1)) t[e] = s[e];
        v[j] = t;
      }
    }
  };
  auto store_item = [&](const Item& it, int bi, float* xs, const float4v* v) __attribute__((always_inline)) {
    if (it.mask == 0) return;
    const int cvalid = cp.Cg - box_cb(bi) * kCB - it.cq * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (!((it.mask >> e) & 1)) continue;
      const int col = phase_index(it.aw0 + e, cp.sw, hg.NW);
      float4v u;
#pragma unroll
      for (int j = 0; j < 4; ++j) u[j] = j < cvalid ? v[j][e] : 0.0f;
      *(float4v*)(xs + (it.ldst + col) * kLdc + it.cq * 4) = u;
    }
  };
#pragma unroll
  for (int k = 0; k < PF; ++k) {
    const int i = tid + k * kThreads;
    items[k].mask = 0;
    items[k].goff = items[k].ldst = items[k].cq = items[k].aw0 = 0;
    if (i < nitems) items[k] = decode(i);
  }
  auto prefetch_box = [&](int bi) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < PF; ++k) load_item(items[k], bi, xr[k]);
  };
  auto store_box = [&](int buf, int bi) __attribute__((always_inline)) {
    float* xs = lds32 + buf * box;
#pragma unroll
    for (int k = 0; k < PF; ++k) store_item(items[k], bi, xs, xr[k]);
    for (int i0 = PF * kThreads; i0 < nitems; i0 += kThreads) {  // items beyond the held ones
      const int i = i0 + tid;
      Item it;
      it.mask = 0;
      it.goff = it.ldst = it.cq = it.aw0 = 0;
      if (i < nitems) it = decode(i);
      float4v v[4];
      load_item(it, bi, v);
      store_item(it, bi, xs, v);
    }
  };

  // ---- weights: fragment j of step (cb, t) = 16 rows (channels m) x 16
  // floats; lane (r16, q) reads the 4 floats of channels 4q .. 4q+3
  const float* wg = wp + (int64_t)g * cp.taps * hg.ncb * hg.mgp * kCB;
  const int wl = (m0 + wmi * 64 + r16) * kCB + q * 4;
  const int64_t wstep = (int64_t)hg.mgp * kCB;

  // ---- LDS row (positions) of this lane's pixel in pixel tile i
  int apos[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pu = wpi * 64 + i * 16;  // 16 consecutive pixels of one tile row
    const int tw = pu & (hg.TW - 1), th = (pu >> hg.ltw) & (hg.TH - 1), td = pu >> (hg.ltw + hg.lth);
    apos[i] = (td * hg.LH + th) * hg.LW + tw + r16;
  }

  // ---- accumulators start at the bias (lane column r16 = channel m0 + wmi*64 + 16j + r16)
  float4v acc[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wmi * 64 + j * 16 + r16;
    const float bv = (cp.has_bias && m < cp.Mg) ? bias[g * cp.Mg + m] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][j] = float4v{bv, bv, bv, bv};
  }

  const int taps2 = hg.taps2, ncb = hg.ncb, nsteps = nbox * taps2;
  // step s = (box bi, in-box tap t2) reads Wp tile (kd*taps2 + t2)*ncb + cb
  auto woff = [&](int s) __attribute__((always_inline)) {
    const int bi = s / taps2, t2 = s - bi * taps2;
    return ((int64_t)(box_kd(bi) * taps2 + t2) * ncb + box_cb(bi)) * wstep;
  };
  lds_barrier();  // zero fill done
  if (nbox > 0) {
    prefetch_box(0);
    store_box(0, 0);
  }
  if (nbox > 1) prefetch_box(1);
  float4v wa[4], wb[4];
  auto load_w = [&](int64_t off, float4v* v) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = *(const float4v*)(wg + off + wl + j * 16 * kCB);
  };
  load_w(nsteps > 0 ? woff(0) : 0, wa);
  // lane t holds the LDS row offset of tap t: a step takes its tap's offset
  // with a lane read instead of a scalar memory load (whose wait would also
  // wait for the operand reads in flight)
  int toff_v = 0;
  for (int t = 0; t < taps2; ++t)
    if (lane == t) toff_v = hg.tap_off[t];
  auto tap_base = [&](int bi, int t2) __attribute__((always_inline)) {
    return lds32 + (DS ? 0 : (bi & 1) * box) + __builtin_amdgcn_readlane(toff_v, t2) * kLdc + q * 4;
  };
  lds_barrier();

  // a[i]: this lane's operand (4 channels of one pixel) of pixel tile i for
  // the current step; each is re-read for the next step as soon as the 16
  // products that use it are issued, so the reads land under the step's
  // remaining products
  float4v a[4];
  if (nsteps > 0) {
    const float* xb = tap_base(0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *(const float4v*)(xb + apos[i] * kLdc);
  }
  auto step = [&](int s, const float4v* wc, float4v* wn) __attribute__((always_inline)) {
    const int bi = s / taps2, t2 = s - bi * taps2;
    // the next step's weights (past the last step: the first tile again)
    load_w(s + 1 < nsteps ? woff(s + 1) : 0, wn);
    // the next step's operands, from this box (at the box's last tap these
    // reads of its first tap are discarded and re-read from the next box)
    const float* xn = tap_base(bi, t2 + 1 == taps2 ? 0 : t2 + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][e], wc[j][e], acc[i][j], 0, 0, 0);
      a[i] = *(const float4v*)(xn + apos[i] * kLdc);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (t2 + 1 == taps2 && bi + 1 < nbox) {
      // the next box (held in registers) into the other buffer, whose
      // previous readers (box bi - 1) all passed the last barrier; with one
      // buffer, after every wave is done with this box
      if constexpr (DS) lds_barrier();
      store_box(DS ? 0 : (bi + 1) & 1, bi + 1);
      lds_barrier();
      if (bi + 2 < nbox) prefetch_box(bi + 2);
      const float* xb = tap_base(bi + 1, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *(const float4v*)(xb + apos[i] * kLdc);
    }
  };
  int s = 0;
  for (; s + 2 <= nsteps; s += 2) {
    step(s, wa, wb);
    step(s + 1, wb, wa);
  }
  if (s < nsteps) step(s, wa, wb);

  // wait states between the last products and the VALU reads of their
  // accumulators
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  // ---- epilogue: lane holds pixels 4q .. 4q+3 of pixel tile i (consecutive
  // columns of one tile row) for channel m0 + wmi*64 + 16j + r16
  const bool vec_y = (cp.OW & 3) == 0;
  // bias is in the accumulator; the residual, then the activation (or, for an
  // input gradient, the derivative of the producer's activation)
  auto finish4 = [&](float4v v, int64_t yi) __attribute__((always_inline)) {
    if (cp.has_z) v += *(const float4v*)(z + yi);
    if (cp.bwd) {
      if (cp.act != ACT_NONE) {
        const float4v pv = *(const float4v*)(pre + yi);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] *= dact_apply(cp.act, pv[e], cp.alpha, cp.beta);
      }
    } else {
      v = act_apply4(cp.act, v, cp.alpha, cp.beta);
    }
    return v;
  };
  // one pixel tile, lane by lane (image edges, widths not a multiple of 4)
  auto store_tile = [&](int i) __attribute__((always_inline)) {
    const int pu = wpi * 64 + i * 16 + q * 4;
    const int tw = pu & (hg.TW - 1), th = (pu >> hg.ltw) & (hg.TH - 1), td = pu >> (hg.ltw + hg.lth);
    const int od = od0 + td, oh = oh0 + th, ow = ow0 + tw;
    if (od >= cp.OD || oh >= cp.OH || ow >= cp.OW) return;
    const int nv = min(4, cp.OW - ow);
    const int64_t pix = ((int64_t)od * cp.OH + oh) * cp.OW + ow;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + wmi * 64 + j * 16 + r16;
      if (m >= cp.Mg) continue;
      const int64_t yi = (n * cp.M + (int64_t)g * cp.Mg + m) * cp.out_sz + pix;
      float4v v = acc[i][j];
      if (vec_y && nv == 4) {
        *(float4v*)(y + yi) = finish4(v, yi);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (e >= nv) continue;
          float u = v[e];
          if (cp.has_z) u += z[yi + e];
          if (cp.bwd) {
            if (cp.act != ACT_NONE) u *= dact_apply(cp.act, pre[yi + e], cp.alpha, cp.beta);
          } else {
            u = act_apply(cp.act, u, cp.alpha, cp.beta);
          }
          y[yi + e] = u;
        }
      }
    }
  };
  // Tiles 2k and 2k+1 are 32 consecutive pixels of one tile row when TW >= 32.
  // There a store covers whole 128-byte lines: lanes r16 < 8 of each 16-lane
  // row (one q) swap their tile-2k values of channels r16 + 8 for the
  // tile-(2k+1) values of channels r16 held by lanes r16 + 8 (row shifts by 8
  // lanes), so store A writes channels 0 .. 7 of the 16-channel tile and store
  // B channels 8 .. 15, each over all 32 pixels.
  auto lanes_down8 = [](float4v v) __attribute__((always_inline)) {  // lane r16 takes lane r16 - 8
    float4v r;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      r[e] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v[e]), 0x118, 0xF, 0xF, true));
    return r;
  };
  auto lanes_up8 = [](float4v v) __attribute__((always_inline)) {  // lane r16 takes lane r16 + 8
    float4v r;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      r[e] = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v[e]), 0x108, 0xF, 0xF, true));
    return r;
  };
#pragma unroll
  for (int ip = 0; ip < 4; ip += 2) {
    // the pair's first pixel (the same for every lane of the wave)
    const int pu0 = wpi * 64 + ip * 16;
    const int tw0 = pu0 & (hg.TW - 1), th0 = (pu0 >> hg.ltw) & (hg.TH - 1),
              td0 = pu0 >> (hg.ltw + hg.lth);
    const int od = od0 + td0, oh = oh0 + th0, ow = ow0 + tw0;
    if (!(vec_y && hg.TW >= 32 && od < cp.OD && oh < cp.OH && ow + 32 <= cp.OW)) {
      store_tile(ip);
      store_tile(ip + 1);
      continue;
    }
    const int64_t ybase = (n * cp.M + (int64_t)g * cp.Mg) * cp.out_sz + ((int64_t)od * cp.OH + oh) * cp.OW + ow;
    const bool lo = r16 < 8;
    const int px = lo ? 4 * q : 16 + 4 * q;  // pixel offset of both stores
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int mrow = m0 + wmi * 64 + j * 16;  // the 16-channel tile's first channel
      float4v v0 = acc[ip][j], v1 = acc[ip + 1][j];
      if (mrow + r16 < cp.Mg) {
        const int64_t yi = ybase + (int64_t)(mrow + r16) * cp.out_sz + 4 * q;
        v0 = finish4(v0, yi);
        v1 = finish4(v1, yi + 16);
      }
      const float4v from_lo = lanes_down8(v1), from_hi = lanes_up8(v0);
      const int ca = mrow + (lo ? r16 : r16 - 8), cb = mrow + (lo ? r16 + 8 : r16);
      if (ca < cp.Mg) *(float4v*)(y + ybase + (int64_t)ca * cp.out_sz + px) = lo ? v0 : from_lo;
      if (cb < cp.Mg) *(float4v*)(y + ybase + (int64_t)cb * cp.out_sz + px) = lo ? from_hi : v1;
    }
  }
}

// Tile choice: WGP = 4 (256 pixels x 64 channels) when M/group <= 64, else
// WGP = 2 (128 x 128); tile widths 16 .. 256 in order of padded output
// area; the first whose two boxes fit is taken.
bool choose32_wgp(const ConvParams& cp, int wgp, bool ds, Geo32& hg);

// Full-depth boxes first; for 3-D convs whose box does not fit, the
// depth-stepped form (one input depth plane per box).
bool choose32(const ConvParams& cp, int& wgp, Geo32& hg) {
  if (cp.transposed) return false;
  for (int ds = 0; ds < (cp.KD > 1 ? 2 : 1); ++ds) {
    if ((ds ? cp.KH * cp.KW : cp.taps) > kMaxTaps) continue;  // taps of one box
    wgp = cp.Mg <= 64 ? 4 : 2;
    if (choose32_wgp(cp, wgp, ds, hg)) return true;
    if (wgp == 4 && choose32_wgp(cp, 2, ds, hg)) {  // smaller pixel tiles for small images
      wgp = 2;
      return true;
    }
  }
  return false;
}

bool choose32_wgp(const ConvParams& cp, int wgp, bool ds, Geo32& hg) {
  const int bn = 64 * wgp, bm = 64 * (4 / wgp);
  int order[5], no = 0;
  double waste[5];
  for (int w : {16, 32, 64, 128, 256}) {
    if (w > bn) break;
    const int th = bn / w;
    if (th > 1 && cp.OH == 1 && cp.OD == 1) continue;  // 1-D: one row per tile
    waste[no] = (double)cdiv(cp.OH, th) * th * cdiv(cp.OW, w) * w / ((double)cp.OH * cp.OW);
    order[no++] = w;
  }
  for (int a = 0; a < no; ++a)
    for (int b = a + 1; b < no; ++b)
      if (waste[b] < waste[a] - 1e-9 || (waste[b] < waste[a] + 1e-9 && order[b] > order[a])) {
        std::swap(waste[a], waste[b]);
        std::swap(order[a], order[b]);
      }
  for (int oi = 0; oi < no; ++oi) {
    const int tw = order[oi], th = bn / tw, td = 1;
    Geo32 h{};
    h.ds = ds;
    h.taps2 = ds ? cp.KH * cp.KW : cp.taps;
    h.TD = td; h.TH = th; h.TW = tw;
    h.ltw = log2i(tw);
    h.lth = log2i(th);
    h.BD = ds ? 1 : (td - 1) * cp.sd + (cp.KD - 1) * cp.dd + 1;
    h.BH = (th - 1) * cp.sh + (cp.KH - 1) * cp.dh + 1;
    h.BW = (tw - 1) * cp.sw + (cp.KW - 1) * cp.dw + 1;
    h.ND = ds ? 1 : (int)cdiv(h.BD, cp.sd);
    h.NH = (int)cdiv(h.BH, cp.sh);
    h.NW = (int)cdiv(h.BW, cp.sw);
    h.LH = cp.sh * h.NH;
    h.LW = cp.sw * h.NW;
    const int64_t bpos = (int64_t)(ds ? 1 : cp.sd) * h.ND * h.LH * h.LW;
    if ((size_t)(ds ? 1 : 2) * bpos * kLdc * sizeof(float) > kMaxLds) continue;
    if ((double)cdiv(cp.OD, td) * td * cdiv(cp.OH, th) * th * cdiv(cp.OW, tw) * tw > 2.0 * cp.out_sz)
      continue;
    h.box_pos = (int)bpos;
    h.tiles_d = (int)cdiv(cp.OD, td);
    h.tiles_h = (int)cdiv(cp.OH, th);
    h.tiles_w = (int)cdiv(cp.OW, tw);
    const int64_t ntile = cp.n * h.tiles_d * h.tiles_h * h.tiles_w;
    h.nmb = (int)cdiv(cp.Mg, bm);
    h.ncb = (int)cdiv(cp.Cg, kCB);
    h.mgp = h.nmb * bm;
    if (ntile * h.nmb * cp.G >= ((int64_t)1 << 31)) continue;
    if ((int64_t)cp.G * cp.taps * h.ncb * h.mgp * kCB >= ((int64_t)1 << 31)) continue;
    if (cp.in_sz >= ((int64_t)1 << 31)) continue;
    h.ntile = (int)ntile;
    h.vec = cp.W % 4 == 0;
    for (int t = 0; t < h.taps2; ++t) {
      const int kw = t % cp.KW, kh = (t / cp.KW) % cp.KH, kd = ds ? 0 : t / (cp.KW * cp.KH);
      const int ad = kd * cp.dd, ah = kh * cp.dh, aw = kw * cp.dw;
      h.tap_off[t] = (((ad % cp.sd) * h.ND + ad / cp.sd) * h.LH + (ah % cp.sh) * h.NH + ah / cp.sh) * h.LW +
                     (aw % cp.sw) * h.NW + aw / cp.sw;
    }
    hg = h;
    return true;
  }
  return false;
}

int launch_repack32(const ConvParams& cp, const Geo32& hg, const RunArgs& a) {
  const int64_t total = (int64_t)cp.G * hg.mgp * hg.ncb * kCB;
  int64_t blocks = (total + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(repack32_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     (hipStream_t)a.stream, (const float*)a.w, (float*)a.ws, cp, hg.ncb, hg.mgp);
  return hipPeekAtLastError() == hipSuccess ? FUSEDCONV_OK : FUSEDCONV_ERR_LAUNCH;
}

}  // namespace

bool halo32_fits(const ConvParams& cp, int32_t dtype, size_t* workspace, int32_t* tile_h,
                 int32_t* tile_w, int64_t* blocks) {
  if (dtype != FUSEDCONV_F32) return false;
  int wgp = 0;
  Geo32 hg;
  if (!choose32(cp, wgp, hg)) return false;
  if (blocks) *blocks = (int64_t)hg.ntile * hg.nmb * cp.G;
  if (workspace) *workspace = (size_t)cp.G * cp.taps * hg.ncb * hg.mgp * kCB * sizeof(float);
  if (tile_h) *tile_h = hg.TH;
  if (tile_w) *tile_w = hg.TW;
  return true;
}

int prepare_halo32(const Geometry& g, const Plan&, const RunArgs& a) {
  int wgp = 0;
  Geo32 hg;
  if (!choose32(g.cp, wgp, hg)) return FUSEDCONV_ERR_ROUTE;
  return launch_repack32(g.cp, hg, a);
}

int launch_halo32(const Geometry& g, const Plan&, const RunArgs& a) {
  const ConvParams& cp = g.cp;
  int wgp = 0;
  Geo32 hg;
  if (!choose32(cp, wgp, hg)) return FUSEDCONV_ERR_ROUTE;
  if (!(a.flags & FUSEDCONV_RUN_WEIGHTS_PREPARED)) {
    const int rc = launch_repack32(cp, hg, a);
    if (rc != FUSEDCONV_OK) return rc;
  }
  const unsigned blocks = (unsigned)((int64_t)hg.ntile * hg.nmb * cp.G);
  const size_t lds = (size_t)(hg.ds ? 1 : 2) * hg.box_pos * kLdc * sizeof(float);
  auto go = [&](auto kfn) -> int {
    if (set_max_dynamic_lds((const void*)kfn, (int)kMaxLds) != FUSEDCONV_OK) return FUSEDCONV_ERR_LAUNCH;
    return launch_conv(kfn, dim3(blocks), dim3(kThreads), lds, a, kEdgeBoth, (const float*)a.x,
                       (const float*)a.ws, (const float*)a.bias, (const float*)a.z,
                       (const float*)a.pre, (float*)a.y, cp, hg);
  };
  if (hg.ds) return wgp == 4 ? go(halo32_kernel<4, true>) : go(halo32_kernel<2, true>);
  return wgp == 4 ? go(halo32_kernel<4, false>) : go(halo32_kernel<2, false>);
}

}  // namespace fc
