// Implicit GEMM on MFMA with channel-last halo boxes (fp16 in, fp32 accumulate).
//
// GEMM view per block: rows = BN output pixels of one image tile, columns =
// BM output channels of one group, reduction over (input channel, tap)
// ordered as (channel block of 32, tap, channel within the block), so that no
// im2col element is gathered one by one:
//   * per channel block, the input box that the tile's windows cover (zero
//     outside the image) is copied once into LDS in channel-last layout
//     [position][32 channels].  Positions are split by stride phase along
//     every axis, so for tap t every output pixel's 32-channel operand row is
//     the LDS row at pixel(p) + offset(t), consecutive pixels sit in
//     consecutive rows whatever the stride, and one lane's 8-channel slice is
//     one ds_read_b128;
//   * the weights are repacked into a tap-major layout
//     Wp[g][tap][channel block][m][32] (fusedconv_prepare_weights, or at the
//     start of every run) and loaded straight into registers one step ahead;
//   * v_mfma_f32_16x16x32_f16 with pixels as MFMA rows: each lane ends with 4
//     consecutive pixels of one output channel.
// The fused epilogue of the FusedConv README ("Inputs": B per output channel
// and Z of Y's shape, added before the activation): the accumulators start
// at B; after the K loop they are staged through LDS one 16-channel block at
// a time, Z is added, the activation applied and Y stored once, rounded.
// The idea of feeding a matrix unit from an input tile that is staged once
// and re-read per tap is the one the FusedConv manifest's
// implicit_im2col_subgroup_matrix variants and the tinygrad page's shifted
// per-tap WMMA GEMMs use; the layouts and tiling here are gfx950-specific.
#include <hip/hip_runtime.h>

#include <stdlib.h>

#include <algorithm>
#include <type_traits>

#include "epilogue.h"
#include "internal.h"
#include "launch.h"
#include "sync.h"

namespace fc {
namespace {

constexpr int kThreads = 256;
constexpr int kCB = 32;               // channels per block = MFMA K
// LDS row pitch (halves per box position): 48 (96-byte rows), or 40 when
// two boxes of 48 do not fit.  An operand read is 16 rows at 16-byte column
// offsets; measured on gfx950, such a ds_read_b128 pattern runs at the full
// LDS rate when the row pitch is 16 bytes times 2 mod 4 (96, 160, ...) and
// at half rate for 80 bytes.
constexpr int kLDCFast = kCB + 16;
constexpr int kLDCSmall = kCB + 8;
constexpr int kMaxTaps = 64;
constexpr size_t kLds2 = 80 * 1024;    // two blocks per CU
constexpr size_t kMaxLds = 150 * 1024;  // one block per CU

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned uint2v __attribute__((ext_vector_type(2)));

// Word 3 of a raw buffer resource on gfx9-class GPUs: 32-bit data format,
// untyped access (offsets past num_records read zero and drop writes).
constexpr int kBufferWord3 = 0x00020000;

struct HaloTile {
  int TD, TH, TW;          // output tile
  int BD, BH, BW;          // input box (box-relative coordinates 0..B*-1)
  int ND, NH, NW;          // box positions per stride phase along each axis
  int LH, LW;              // LDS pitches in positions: LH = sh*NH rows, LW = sw*NW columns
  int box_pos;             // positions per LDS box: sd*ND*LH*LW
  int tiles_d, tiles_h, tiles_w;
  int ntile;               // n * tiles_d * tiles_h * tiles_w
  int nmb;                 // m blocks per group
  int remap;               // 1: the m blocks of one tile run back to back on one XCD
  int ncb;                 // input channel blocks
  int mgp;                 // Wp rows per (tap, channel block): M/group rounded up to BM
  int vec_x;               // W % 8 == 0: 16-byte input loads
  int ltw, lth;            // log2(TW), log2(TH)
  int ldc;                 // LDS row pitch in halves (kLDCFast or kLDCSmall)
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Dynamic LDS: two input boxes, or the epilogue staging area (nw waves x 16
// channels x (BN/2 + 4) fp32) if larger.
size_t lds_bytes(int box_pos, int bn, int ldc, int nw) {
  const size_t boxes = (size_t)2 * box_pos * ldc * 2;
  const size_t stage = (size_t)nw * 16 * (bn / 2 + 4) * 4;
  return boxes > stage ? boxes : stage;
}

// Box-relative coordinate a along an axis with stride s and n positions per
// phase -> LDS index (phase-major).
__device__ __forceinline__ int phase_index(int a, int s, int n) {
  if (s == 1) return a;
  const int ph = a % s;
  return ph * n + a / s;
}

// Wp[((g*taps + t)*ncb + cb)*mgp + m][c'] = W[g*Mg + m][cb*32 + c'][t]; 0 past
// C/group and for the padding rows m >= M/group.
__global__ __launch_bounds__(kThreads) void repack_w_kernel(const half_t* __restrict__ w,
                                                            half_t* __restrict__ wp,
                                                            ConvParams cp, int ncb, int mgp) {
  // one thread per (group, row m, channel c): it reads the `taps` weights of
  // (m, c), which are contiguous in W and follow those of (m, c - 1), so a
  // wave reads one contiguous run; it writes one half per tap, and the
  // threads of consecutive channels write consecutive halves of a Wp row.
  // 32-bit index arithmetic.
  const int cpad = ncb * kCB;
  const int total = cp.G * mgp * cpad;
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < total; i += gridDim.x * kThreads) {
    const int c = i % cpad;
    int r = i / cpad;
    const int m = r % mgp;
    const int g = r / mgp;
    const bool ok = c < cp.Cg && m < cp.Mg;
    const half_t* src = w + ((int64_t)(g * cp.Mg + (ok ? m : 0)) * cp.Cg + (ok ? c : 0)) * cp.taps;
    half_t* dst = wp + (((int64_t)g * cp.taps * ncb + c / kCB) * mgp + m) * kCB + c % kCB;
    for (int t = 0; t < cp.taps; ++t)
      dst[(int64_t)t * ncb * mgp * kCB] = ok ? src[t] : (half_t)0;
  }
}

// One work unit: output channels [mb*BM, mb*BM + BM) of group g over the
// output tile at (n, od0, oh0, ow0).
struct Unit {
  int64_t n;
  int g, mb, od0, oh0, ow0;
};

// Block tile BN pixels x BM channels, 2 x NWM waves, each owning
// (BN/2) x (BM/NWM) = TP x TM MFMA blocks of 16x16.  NWM = 2: 4 waves, two
// blocks per CU; NWM = 4: 8 waves sharing one input box, one block per CU
// (two waves per SIMD of the same block, half the box loads per output).
// PF: input-box loader items per thread kept in registers across a channel
// block (each item = 4 channels x 8 columns of one box row, 16 registers);
// items beyond PF * NT are loaded and stored at the channel-block boundary.
// VEC: W % 8 == 0, so an item's 8 columns are one aligned 16-byte load.
template <int BM, int BN, int PF, bool VEC, int NWM, int ACT>
__device__ __forceinline__ void halo_tile(const half_t* __restrict__ x,
                                          const half_t* __restrict__ wp,
                                          const half_t* __restrict__ bias, const half_t* z,
                                          const half_t* pre, half_t* y, const ConvParams& cp,
                                          const HaloTile& ht, const Unit& u) {
  constexpr int NT = 128 * NWM;  // threads
  constexpr int TP = BN / 32;
  constexpr int TM = BM / (16 * NWM);
  extern __shared__ __attribute__((aligned(16))) half_t lds[];
  const int ldc = ht.ldc;
  const int box = ht.box_pos * ldc;  // halves per input box

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wpi = wave & 1, wmi = wave >> 1;
  const int r16 = lane & 15, q = lane >> 4;
  const int g = u.g;
  const int64_t n = u.n;
  const int m0 = u.mb * BM;
  const int od0 = u.od0, oh0 = u.oh0, ow0 = u.ow0;
  const int bd0 = od0 * cp.sd - cp.pd, bh0 = oh0 * cp.sh - cp.ph, bw0 = ow0 * cp.sw - cp.pw;

  // ---- zero both input boxes: positions outside the image stay zero
  for (int i = tid; i < 2 * box / 8; i += NT) ((half8*)lds)[i] = half8{};

  // ---- input loader.  Item i = (row of the in-image part of the box,
  // aligned 8-column group, channel quad cq = i % 8): four 16-byte loads of
  // the same 8 columns in 4 channel planes, written as eight 8-byte LDS rows
  // (4 channels each).  Consecutive lanes cover the 8 quads of one 64-byte
  // LDS row, so the writes are at most 2-way bank conflicted.
  const int d_lo = max(bd0, 0), d_hi = min(bd0 + ht.BD, cp.D);
  const int h_lo = max(bh0, 0), h_hi = min(bh0 + ht.BH, cp.H);
  const int w_lo = max(bw0, 0), w_hi = min(bw0 + ht.BW, cp.W);
  const int g_lo = w_lo >> 3, g_hi = (w_hi + 7) >> 3;
  const int nd = max(d_hi - d_lo, 0), nh = max(h_hi - h_lo, 0), ngr = max(g_hi - g_lo, 0);
  const int nitems = 8 * nd * nh * ngr;
  const int cq = tid & 7;
  const half_t* ximg = x + (n * cp.C + (int64_t)g * cp.Cg + cq * 4) * cp.in_sz;
  // decoded item: element offset of (channel cq*4, row, column group) from the
  // channel block's first plane; LDS half offset of the row (+ cq*4); the
  // box-relative column of the group's first element (+8) and the column mask
  struct Item { int goff, ldst, cm; };
  auto decode = [&](int i) __attribute__((always_inline)) {
    Item it;
    int r = i >> 3;
    const int gi = r % ngr;
    r /= ngr;
    const int hh = r % nh;
    const int dd = r / nh;
    const int id = d_lo + dd, ih = h_lo + hh, iw = (g_lo + gi) * 8;
    int mask = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (iw + e >= w_lo && iw + e < w_hi) mask |= 1 << e;
    it.goff = (id * cp.H + ih) * cp.W + iw;
    it.ldst = ((phase_index(id - bd0, cp.sd, ht.ND) * ht.LH + phase_index(ih - bh0, cp.sh, ht.NH)) *
               ht.LW) * ldc + cq * 4;
    it.cm = ((iw - bw0 + 8) << 8) | mask;
    return it;
  };
  Item items[PF];
#pragma unroll
  for (int k = 0; k < PF; ++k) {
    const int i = tid + k * NT;
    items[k].cm = -1;
    items[k].goff = items[k].ldst = 0;
    if (i < nitems) items[k] = decode(i);
  }
  half8 xreg[PF][4];
  // load item it of channel block cb (4 channel planes) into v
  // Loads are unconditional (an invalid item or channel reads the first
  // element of x instead) and validity is applied when the item is written to
  // LDS: a load under a branch makes the compiler wait for it at the join,
  // which would turn the prefetch into a synchronous HBM round trip.
  auto load_item = [&](const Item& it, int cb, half8* v) __attribute__((always_inline)) {
    const int cvalid = cp.Cg - cb * kCB - cq * 4;  // valid channels of this quad
    const half_t* src = ximg + (int64_t)cb * kCB * cp.in_sz + it.goff;
    int cm = it.cm;
    asm volatile("" : "+v"(cm));  // keep the column tests here, not hoisted
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = cm >= 0 && j < cvalid;
      const half_t* s = ok ? src + j * cp.in_sz : x;
      if constexpr (VEC) {
        v[j] = *(const half8*)s;
      } else {
        half8 t = {};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (ok && ((cm >> e) & 1)) t[e] = s[e];
        v[j] = t;
      }
    }
  };
  // write item it of channel block cb (4 channels in v) into LDS buffer xs:
  // 8 columns x 8 bytes; channels past C/group are written as zeros
  auto store_item = [&](const Item& it, int cb, half_t* xs, const half8* v) __attribute__((always_inline)) {
    int cm = it.cm;
    asm volatile("" : "+v"(cm));  // keep the column tests here, not hoisted
    if (cm < 0) return;
    const int cvalid = cp.Cg - cb * kCB - cq * 4;
    half8 u[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = j < cvalid ? v[j] : half8{};
    const int aw0 = (cm >> 8) - 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (!((cm >> e) & 1)) continue;
      const int col = phase_index(aw0 + e, cp.sw, ht.NW);
      *(half4*)(xs + it.ldst + col * ldc) = half4{u[0][e], u[1][e], u[2][e], u[3][e]};
    }
  };
  auto prefetch_box = [&](int cb) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < PF; ++k) load_item(items[k], cb, xreg[k]);
  };
  // store box cb into buffer buf: the prefetched items, then any further items
  auto store_box = [&](int buf, int cb) __attribute__((always_inline)) {
    half_t* xs = lds + buf * box;
#pragma unroll
    for (int k = 0; k < PF; ++k) store_item(items[k], cb, xs, xreg[k]);
    for (int i0 = PF * NT; i0 < nitems; i0 += PF * NT) {
      Item more[PF];
      half8 v[PF][4];
#pragma unroll
      for (int k = 0; k < PF; ++k) {
        const int i = i0 + tid + k * NT;
        more[k].cm = -1;
        more[k].goff = more[k].ldst = 0;
        if (i < nitems) more[k] = decode(i);
        load_item(more[k], cb, v[k]);
      }
#pragma unroll
      for (int k = 0; k < PF; ++k) store_item(more[k], cb, xs, v[k]);
    }
  };

  // ---- weight fragments straight from Wp (rows padded to ht.mgp with zeros):
  // fragment j of step (cb, t) = 16 rows x 64 bytes, each lane reads 16 bytes
  // at a 32-bit lane offset from the step's (uniform) tile address.
  const half_t* wg = wp + (int64_t)g * cp.taps * ht.ncb * ht.mgp * kCB;
  const int wl = (m0 + wmi * (BM / NWM) + r16) * kCB + q * 8;
  const int64_t wstep = (int64_t)ht.mgp * kCB;  // halves per (tap, channel block) tile

  // ---- LDS offset (halves) of this lane's operand row (pixel) in pixel
  // tile i.  Tiles are TW (a multiple of 16) pixels wide, so pixel tile i of
  // a wave is 16 consecutive pixels of one tile row.
  int aoff[TP];
#pragma unroll
  for (int i = 0; i < TP; ++i) {
    const int pu = wpi * (BN / 2) + i * 16;
    aoff[i] = ((pu >> ht.ltw) * ht.LW + (pu & (ht.TW - 1)) + r16) * ldc + q * 8;
  }
  // ---- LDS offset (halves) of each tap: along every axis the tap's box
  // offset k*dilation splits into stride phase (k*dil % s) and index
  // (k*dil / s).  One int per tap, read once per K step, kept in the unused
  // padding (channels 32..39) of box row t of buffer 0, which neither the
  // box writes nor the MFMA operand reads touch.
  int* const tap_tab = (int*)lds;
  const int tab_stride = ldc / 2;  // ints per LDS row; entry t at int t*tab_stride + 16

  // ---- accumulators start at the bias: lane column r16 is output channel
  // m0 + wmi*BM/NWM + j*16 + r16
  float4v acc[TP][TM];
  {
    const int mw = m0 + wmi * (BM / NWM) + r16;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      float bv = 0.0f;
      if (cp.has_bias && mw + j * 16 < cp.Mg) bv = to_f32(bias[g * cp.Mg + mw + j * 16]);
#pragma unroll
      for (int i = 0; i < TP; ++i) acc[i][j] = float4v{bv, bv, bv, bv};
    }
  }

  const bool vec_y = (cp.OW & 3) == 0;
  const int taps = cp.taps, ncb = ht.ncb, nsteps = ncb * taps;

  lds_barrier();  // zero fill done before any box or table write
  if (tid < cp.taps) {
    const int kw = tid % cp.KW, kh = (tid / cp.KW) % cp.KH, kd = tid / (cp.KW * cp.KH);
    const int ad = kd * cp.dd, ah = kh * cp.dh, aw = kw * cp.dw;
    tap_tab[tid * tab_stride + 16] =
        ((((ad % cp.sd) * ht.ND + ad / cp.sd) * ht.LH + (ah % cp.sh) * ht.NH + ah / cp.sh) * ht.LW +
         (aw % cp.sw) * ht.NW + aw / cp.sw) * ldc;
  }
  prefetch_box(0);
  store_box(0, 0);
  if (ncb > 1) prefetch_box(1);

  // weight fragments: two register sets, prefetch distance one step
  half8 wa[TM], wb[TM];
#pragma unroll
  for (int j = 0; j < TM; ++j) wa[j] = *(const half8*)(wg + wl + j * 16 * kCB);
  lds_barrier();

  // Step s = (cb, t) reads Wp tile t * ncb + cb; wnext is the Wp offset of
  // step s + 1.  After the last step of a channel block the next block's box
  // (held in registers) is written to the other buffer and one barrier
  // separates it from both its readers and the previous readers of that
  // buffer (the steps of channel block cb - 1, all before the last barrier).
  const int64_t wtap = (int64_t)ncb * wstep;                       // next tap, same block
  const int64_t wcb = wstep - (int64_t)(taps - 1) * ncb * wstep;   // next block, tap 0
  int64_t wnext = (taps > 1) ? wtap : wcb;
  int cb = 0, t = 0, s = 0;
  int toff = 0;  // tap 0 is at offset 0
  // Operand rows of pixel tiles 0..TP/2-1 are read one half-step early: a
  // step reads its tiles TP/2..TP-1, runs the MFMAs of tiles 0..TP/2-1,
  // stores the next channel block's box if this was the block's last tap,
  // then reads the next step's tiles 0..TP/2-1 into the registers just freed
  // and runs the rest.  The early read is unconditional (its buffer and tap
  // are selected without a branch) so that it stays between the two halves.
  constexpr int TH = TP / 2;
  half8 a_[TP];
#pragma unroll
  for (int i = 0; i < TH; ++i) a_[i] = *(const half8*)(lds + aoff[i]);
#define HALO_STEP(WC, WN, HAS_NEXT)                                                       \
  {                                                                                       \
    {                                                                                     \
      /* unconditional (a load under a branch is waited for at once); past */             \
      /* the last step it re-reads the first tile */                                      \
      const half_t* sn_ = wg + ((HAS_NEXT) ? wnext : 0);                                  \
      _Pragma("unroll") for (int j = 0; j < TM; ++j) WN[j] = *(const half8*)(sn_ + wl + j * 16 * kCB); \
    }                                                                                     \
    /* keep the loads here, a full step ahead of their use (the scheduler */              \
    /* would otherwise sink them below this step's MFMAs into WC's registers) */          \
    __builtin_amdgcn_sched_barrier(0);                                                    \
    const half_t* xb_ = lds + (cb & 1) * box + toff;                                      \
    _Pragma("unroll") for (int i = TH; i < TP; ++i) a_[i] = *(const half8*)(xb_ + aoff[i]); \
    const bool last_ = t + 1 == taps;                                                     \
    const int tn_ = last_ ? 0 : t + 1;                                                    \
    const int toffn_ = tap_tab[tn_ * tab_stride + 16];                                    \
    _Pragma("unroll") for (int i = 0; i < TH; ++i)                                        \
      _Pragma("unroll") for (int j = 0; j < TM; ++j)                                      \
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_[i], WC[j], acc[i][j], 0, 0, 0); \
    if (last_ && cb + 1 < ncb) {                                                          \
      store_box((cb + 1) & 1, cb + 1);                                                    \
      lds_barrier();                                                                      \
      if (cb + 2 < ncb) prefetch_box(cb + 2);                                             \
    }                                                                                     \
    const int cbn_ = cb + (last_ ? 1 : 0);                                                \
    const half_t* xn_ = lds + (cbn_ & 1) * box + toffn_;                                  \
    _Pragma("unroll") for (int i = 0; i < TH; ++i) a_[i] = *(const half8*)(xn_ + aoff[i]); \
    _Pragma("unroll") for (int i = TH; i < TP; ++i)                                       \
      _Pragma("unroll") for (int j = 0; j < TM; ++j)                                      \
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_[i], WC[j], acc[i][j], 0, 0, 0); \
    t = tn_;                                                                              \
    cb = cbn_;                                                                            \
    toff = toffn_;                                                                        \
    ++s;                                                                                  \
    wnext += (t == taps - 1) ? wcb : wtap;                                                \
  }
  while (s + 1 < nsteps) {
    HALO_STEP(wa, wb, true);
    HALO_STEP(wb, wa, s + 1 < nsteps);
  }
  if (s < nsteps) HALO_STEP(wa, wb, false);
#undef HALO_STEP

  // ---- epilogue: activation and the rounded store.  The accumulators go
  // through LDS (the boxes are dead now) one 16-channel block at a time,
  // staged as 16 rows of consecutive pixels; a rolled loop then applies the
  // activation and stores Y, consecutive lanes writing consecutive 8-byte
  // pieces of a row.
  lds_barrier();
  constexpr int PW = BN / 2;              // pixels per wave
  constexpr int RP = PW + 4;              // fp32 row pitch (padded)
  constexpr int GPR = PW / 4;             // 4-pixel groups per row
  constexpr int ITER = 16 * GPR / 64;     // groups per lane per pass
  float* stage = (float*)lds + wave * 16 * RP;
  const int mw0 = m0 + wmi * (BM / NWM);  // first channel of this wave
  static_assert(64 % GPR == 0, "a lane's 4-pixel group must not change between passes");
  if (vec_y && (int64_t)cp.out_sz * (BM / NWM) * 2 < ((int64_t)1 << 31)) {
    // OW % 4 == 0: pass it of block j gives lane the 4 pixels p4 .. p4+3 of
    // stage row it*RPI + rsub (channel mw0 + 16j + row) -- the same pixels
    // in every pass, so their output offset is computed once.  Residual
    // loads and stores are raw buffer operations: an invalid slot gets an
    // offset past the buffer's range (reads zero, write dropped) and a
    // missing residual is an empty range, so no branch surrounds a memory
    // operation and every residual load is in flight before the first use.
    constexpr int RPI = 64 / GPR;         // stage rows per pass
    constexpr unsigned kOff = 0x80000000u;
    const int p4 = (lane % GPR) * 4, rsub = lane / GPR;
    const int pl = wpi * PW + p4;
    const int tw = pl & (ht.TW - 1), th = (pl >> ht.ltw) & (ht.TH - 1), td = pl >> (ht.ltw + ht.lth);
    const int od = od0 + td, oh = oh0 + th, ow = ow0 + tw;
    const bool pok = od < cp.OD && oh < cp.OH && ow < cp.OW;
    const int pix = (od * cp.OH + oh) * cp.OW + ow;
    const int64_t wbase = (n * cp.M + (int64_t)g * cp.Mg + mw0) * cp.out_sz;
    const __amdgpu_buffer_rsrc_t yb =
        __builtin_amdgcn_make_buffer_rsrc((void*)(y + wbase), (short)0, 0x7fffffff, kBufferWord3);
    const __amdgpu_buffer_rsrc_t zb = __builtin_amdgcn_make_buffer_rsrc(
        cp.has_z ? (void*)(z + wbase) : (void*)y, (short)0, cp.has_z ? 0x7fffffff : 0, kBufferWord3);
    // backward data: the input pre-activation P, read like Z
    const bool dpre = ACT == ACT_NONE && cp.bwd && cp.act != ACT_NONE;
    const __amdgpu_buffer_rsrc_t pb = __builtin_amdgcn_make_buffer_rsrc(
        dpre ? (void*)(pre + wbase) : (void*)y, (short)0, dpre ? 0x7fffffff : 0, kBufferWord3);
    auto voff = [&](int j, int it) __attribute__((always_inline)) {
      const int r = j * 16 + it * RPI + rsub;  // channel relative to mw0
      return (pok && mw0 + r < cp.Mg) ? (unsigned)((r * (int)cp.out_sz + pix) * 2) : kOff;
    };
    uint2v zr[TM][ITER];
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int it = 0; it < ITER; ++it)
        zr[j][it] = __builtin_bit_cast(uint2v, __builtin_amdgcn_raw_buffer_load_b64(zb, voff(j, it), 0, 0));
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      uint2v pr[ITER];
      if constexpr (ACT == ACT_NONE) {
        if (dpre) {
#pragma unroll
          for (int it = 0; it < ITER; ++it)
            pr[it] = __builtin_bit_cast(uint2v, __builtin_amdgcn_raw_buffer_load_b64(pb, voff(j, it), 0, 0));
        }
      }
#pragma unroll
      for (int i = 0; i < TP; ++i) *(float4v*)(stage + r16 * RP + i * 16 + q * 4) = acc[i][j];
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int it = 0; it < ITER; ++it) {
        const float4v sv = *(const float4v*)(stage + (it * RPI + rsub) * RP + p4);
        const half4 zh = __builtin_bit_cast(half4, zr[j][it]);
        act4_t v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = sv[e] + (float)zh[e];
        if constexpr (ACT == ACT_NONE) {
          if (dpre) {  // (acc + Z) * act'(P)
            const half4 ph = __builtin_bit_cast(half4, pr[it]);
            act4_t pv;
#pragma unroll
            for (int e = 0; e < 4; ++e) pv[e] = (float)ph[e];
            v *= dact_apply4(cp.act, pv, cp.alpha, cp.beta);
          }
        }
        v = act4<ACT>(v, cp.alpha, cp.beta);
        half4 out;
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = (half_t)v[e];
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(uint2v, out), yb, voff(j, it), 0, 0);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    return;
  }
  // Z (when OW % 4 == 0, a lane's 4 pixels are all in or all out of the
  // image): every value this wave needs is requested before any is used, as
  // unconditional 8-byte loads (an invalid slot reads z[0..3] and is never
  // stored), so the loads overlap instead of waiting one by one.
  const bool zvec = cp.has_z && vec_y;
  half4 zv[TM][ITER];
  if (zvec) {
#pragma unroll
    for (int j = 0; j < TM; ++j)
#pragma unroll
      for (int it = 0; it < ITER; ++it) {
        const int idx = it * 64 + lane;
        const int row = idx / GPR, p4 = (idx % GPR) * 4;
        const int m = mw0 + j * 16 + row;
        const int pl = wpi * PW + p4;
        const int tw = pl & (ht.TW - 1), th = (pl >> ht.ltw) & (ht.TH - 1), td = pl >> (ht.ltw + ht.lth);
        const int od = od0 + td, oh = oh0 + th, ow = ow0 + tw;
        const bool ok = m < cp.Mg && od < cp.OD && oh < cp.OH && ow < cp.OW;
        const int64_t zi = (n * cp.M + g * cp.Mg + m) * cp.out_sz + ((int64_t)od * cp.OH + oh) * cp.OW + ow;
        zv[j][it] = *(const half4*)(ok ? z + zi : z);
      }
  }
#pragma unroll
  for (int j = 0; j < TM; ++j) {
#pragma unroll
    for (int i = 0; i < TP; ++i) *(float4v*)(stage + r16 * RP + i * 16 + q * 4) = acc[i][j];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (zvec) {  // Z into the stage (unrolled: zv is indexed statically)
#pragma unroll
      for (int it = 0; it < ITER; ++it) {
        const int idx = it * 64 + lane;
        float4v* sp = (float4v*)(stage + (idx / GPR) * RP + (idx % GPR) * 4);
        float4v v = *sp;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] += (float)zv[j][it][r];
        *sp = v;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    // rolled
    for (int it = 0; it < ITER; ++it) {
      const int idx = it * 64 + lane;
      const int row = idx / GPR, p4 = (idx % GPR) * 4;
      const int m = mw0 + j * 16 + row;
      const int pl = wpi * PW + p4;
      const int tw = pl & (ht.TW - 1), th = (pl >> ht.ltw) & (ht.TH - 1), td = pl >> (ht.ltw + ht.lth);
      const int od = od0 + td, oh = oh0 + th, ow = ow0 + tw;
      if (m >= cp.Mg || od >= cp.OD || oh >= cp.OH || ow >= cp.OW) continue;
      const int nv = min(4, cp.OW - ow);
      const int64_t yi = (n * cp.M + g * cp.Mg + m) * cp.out_sz +
                         ((int64_t)od * cp.OH + oh) * cp.OW + ow;
      float4v v4 = *(const float4v*)(stage + row * RP + p4);
      if (cp.has_z && !zvec) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (r < nv) v4[r] += to_f32(z[yi + r]);
      }
      if constexpr (ACT == ACT_NONE) {
        if (cp.bwd && cp.act != ACT_NONE) {  // backward data: (acc + Z) * act'(P)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (r < nv) v4[r] *= dact_apply(cp.act, to_f32(pre[yi + r]), cp.alpha, cp.beta);
        }
      }
      v4 = act4<ACT>(v4, cp.alpha, cp.beta);
      half4 out;
#pragma unroll
      for (int r = 0; r < 4; ++r) out[r] = (half_t)v4[r];
      if (vec_y && nv == 4) {
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

// Block -> work unit (group, tile, m block).  Blocks are dealt to the XCDs
// round-robin; with remap the m blocks of a tile are 8 blocks apart, i.e.
// back to back on the same XCD, so the second reads X from that XCD's L2.
template <int BM, int BN, int PF, bool VEC, int NWM, int ACT>
__global__ __launch_bounds__(128 * NWM, NWM == 2 ? 2 : 1) void halo_kernel(const half_t* __restrict__ x,
                                                           const half_t* __restrict__ wp,
                                                           const half_t* __restrict__ bias,
                                                           const half_t* z, const half_t* pre,
                                                           half_t* y,
                                                           ConvParams cp, HaloTile ht) {
  const int per_g = ht.ntile * ht.nmb;
  Unit u;
  u.g = blockIdx.x / per_g;
  const int rb = blockIdx.x - u.g * per_g;
  int tile;
  if (ht.remap) {
    const int v = rb >> 3;
    u.mb = v % ht.nmb;
    tile = (v / ht.nmb) * 8 + (rb & 7);
  } else {
    u.mb = rb % ht.nmb;
    tile = rb / ht.nmb;
  }
  const int tw_i = tile % ht.tiles_w;
  tile /= ht.tiles_w;
  const int th_i = tile % ht.tiles_h;
  tile /= ht.tiles_h;
  const int td_i = tile % ht.tiles_d;
  u.n = tile / ht.tiles_d;
  u.od0 = td_i * ht.TD;
  u.oh0 = th_i * ht.TH;
  u.ow0 = tw_i * ht.TW;
  halo_tile<BM, BN, PF, VEC, NWM, ACT>(x, wp, bias, z, pre, y, cp, ht, u);
}

struct Choice {
  int bm, bn, nwm;  // block tile BM x BN, waves 2 x nwm
  HaloTile ht;
};

int log2i(int v) { return 31 - __builtin_clz((unsigned)v); }

// Fill the tile-dependent fields; false if the box does not fit.
bool make_tile(const ConvParams& cp, int bm, int bn, int tw, size_t max_lds, int nw, HaloTile& ht) {
  const int th = bn / tw, td = 1;
  ht.TD = td; ht.TH = th; ht.TW = tw;
  ht.ltw = log2i(tw);
  ht.lth = log2i(th);
  ht.BD = (td - 1) * cp.sd + (cp.KD - 1) * cp.dd + 1;
  ht.BH = (th - 1) * cp.sh + (cp.KH - 1) * cp.dh + 1;
  ht.BW = (tw - 1) * cp.sw + (cp.KW - 1) * cp.dw + 1;
  ht.ND = (int)cdiv(ht.BD, cp.sd);
  ht.NH = (int)cdiv(ht.BH, cp.sh);
  ht.NW = (int)cdiv(ht.BW, cp.sw);
  ht.LH = cp.sh * ht.NH;
  ht.LW = cp.sw * ht.NW;
  const int64_t bpos = (int64_t)cp.sd * ht.ND * ht.LH * ht.LW;
  // (the tap table lives in the padding of the first kMaxTaps box rows)
  if (bpos < kMaxTaps || bpos > (1 << 16)) return false;
  if (lds_bytes((int)bpos, bn, kLDCFast, nw) <= max_lds) ht.ldc = kLDCFast;
  else if (lds_bytes((int)bpos, bn, kLDCSmall, nw) <= max_lds) ht.ldc = kLDCSmall;
  else return false;
  ht.box_pos = (int)bpos;
  ht.tiles_d = (int)cdiv(cp.OD, td);
  ht.tiles_h = (int)cdiv(cp.OH, th);
  ht.tiles_w = (int)cdiv(cp.OW, tw);
  const int64_t ntile = cp.n * ht.tiles_d * ht.tiles_h * ht.tiles_w;
  ht.ncb = (int)cdiv(cp.Cg, kCB);
  ht.mgp = (int)(cdiv(cp.Mg, bm) * bm);
  ht.nmb = (int)cdiv(cp.Mg, bm);
  if (ntile * ht.nmb * cp.G >= ((int64_t)1 << 31)) return false;
  if ((int64_t)cp.G * cp.taps * ht.ncb * ht.mgp * (kCB / 8) >= ((int64_t)1 << 31)) return false;
  ht.ntile = (int)ntile;
  ht.remap = (ntile % 8) == 0;
  ht.vec_x = (cp.W % 8) == 0;
  return true;
}

// Pick the block tile and the output tile; false if nothing fits.  In order
// of preference: 8 waves with BM = 256 (one block per CU, both channel halves
// on one input box) when the group has more than 128 output channels, the
// input box has at least twice as many positions as the tile has pixels
// (strided convolutions, where reading X once instead of once per 128
// channels saves the most: measured 15% on the 2x2 stride-2 downsample, no
// gain on stride-1 3x3, which keeps two blocks per CU overlapping their
// epilogues) and there are enough tiles to give every CU one; then BM = 128
// with two blocks per CU; then BM = 128 with one (larger boxes: 3-D, strided
// 3x3).
bool choose(const ConvParams& cp, Choice& ch) {
  if (cp.Cg < 16 || cp.taps > kMaxTaps) return false;
  const int tws[] = {16, 32, 64, 128, 256};
  int bn_first = 256;  // FUSEDCONV_HALO_BN=128 restricts the tile to 128 pixels (tuning)
  if (const char* e = getenv("FUSEDCONV_HALO_BN")) bn_first = atoi(e) == 128 ? 128 : 256;
  struct Cand {
    int bm, nwm;
    size_t max_lds;
  };
  const Cand cands[] = {{256, 4, kMaxLds}, {128, 2, kLds2}, {128, 2, kMaxLds}};
  for (const Cand& c : cands) {
    if (c.bm == 256 && cp.Mg <= 128) continue;
    for (int bn : {256, 128}) {
      if (bn > bn_first) continue;
      // tile widths (multiples of 16; tile = bn / tw rows) in order of padded
      // output area, ties to the wider tile; the first that fits is taken
      int order[5], no = 0;
      double waste[5];
      for (int w : tws) {
        if (w > bn) break;
        waste[no] = (double)cdiv(cp.OH, bn / w) * (bn / w) * cdiv(cp.OW, w) * w /
                    ((double)cp.OH * cp.OW);
        order[no] = w;
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
        HaloTile ht;
        if (!make_tile(cp, c.bm, bn, order[oi], c.max_lds, 2 * c.nwm, ht)) continue;
        // the tiles must not be mostly padding
        if ((double)ht.tiles_d * ht.TD * ht.tiles_h * ht.TH * ht.tiles_w * ht.TW > 2.0 * cp.out_sz)
          continue;
        if (c.bm == 256 && ((int64_t)ht.ntile * cp.G < 256 || ht.box_pos < 2 * bn)) continue;
        ch.bm = c.bm;
        ch.bn = bn;
        ch.nwm = c.nwm;
        ch.ht = ht;
        return true;
      }
    }
  }
  return false;
}

int launch_repack(const ConvParams& cp, const Choice& ch, const RunArgs& a) {
  const int64_t total = (int64_t)cp.G * ch.ht.ncb * ch.ht.mgp * kCB;
  int64_t rblocks = (total + kThreads - 1) / kThreads;
  if (rblocks > 4096) rblocks = 4096;
  hipLaunchKernelGGL(repack_w_kernel, dim3((unsigned)rblocks), dim3(kThreads), 0,
                     (hipStream_t)a.stream, (const half_t*)a.w, (half_t*)a.ws, cp, ch.ht.ncb,
                     ch.ht.mgp);
  return hipPeekAtLastError() == hipSuccess ? FUSEDCONV_OK : FUSEDCONV_ERR_LAUNCH;
}

template <int BM, int BN, int PF, bool VEC, int NWM>
int launch_t(const Geometry& g, const Choice& ch, const RunArgs& a) {
  const ConvParams& cp = g.cp;
  const size_t lds = lds_bytes(ch.ht.box_pos, BN, ch.ht.ldc, 2 * NWM);
  const void* kfn = (const void*)halo_kernel<BM, BN, PF, VEC, NWM, FC_ACT>;
  if (set_max_dynamic_lds(kfn, (int)kMaxLds) != FUSEDCONV_OK) return FUSEDCONV_ERR_LAUNCH;
  if (!(a.flags & FUSEDCONV_RUN_WEIGHTS_PREPARED)) {
    const int rc = launch_repack(cp, ch, a);
    if (rc != FUSEDCONV_OK) return rc;
  }
  const unsigned blocks = (unsigned)((int64_t)ch.ht.ntile * ch.ht.nmb * cp.G);
  return launch_conv(halo_kernel<BM, BN, PF, VEC, NWM, FC_ACT>, dim3(blocks), dim3(128 * NWM), lds, a,
                     kEdgeBoth, (const half_t*)a.x, (const half_t*)a.ws, (const half_t*)a.bias,
                     (const half_t*)a.z, (const half_t*)a.pre, (half_t*)a.y, cp, ch.ht);
}

}  // namespace

#ifndef FC_ACT
#error "compiled once per activation id: -DFC_ACT=<0..ACT_COUNT-1>"
#endif

// the halo route with activation FC_ACT
int FC_CAT(launch_halo_act_, FC_ACT)(const Geometry& g, const RunArgs& a) {
  Choice ch;
  if (!choose(g.cp, ch)) return FUSEDCONV_ERR_ROUTE;
  if (ch.ht.vec_x) {
    if (ch.bm == 256)
      return ch.bn == 256 ? launch_t<256, 256, 1, true, 4>(g, ch, a) : launch_t<256, 128, 1, true, 4>(g, ch, a);
    return ch.bn == 256 ? launch_t<128, 256, 1, true, 2>(g, ch, a) : launch_t<128, 128, 2, true, 2>(g, ch, a);
  }
  if (ch.bm == 256)
    return ch.bn == 256 ? launch_t<256, 256, 1, false, 4>(g, ch, a) : launch_t<256, 128, 1, false, 4>(g, ch, a);
  return ch.bn == 256 ? launch_t<128, 256, 1, false, 2>(g, ch, a) : launch_t<128, 128, 2, false, 2>(g, ch, a);
}

#if FC_ACT == 0
FC_ACT_DECLS(launch_halo_act_)

bool igemm_halo_fits(const ConvParams& cp, int32_t dtype, int32_t& tile_h, int32_t& tile_w,
                     size_t& workspace, int32_t* block_m) {
  if (dtype != FUSEDCONV_F16) return false;
  Choice ch;
  if (!choose(cp, ch)) return false;
  tile_h = ch.ht.TH;
  tile_w = ch.ht.TW;
  if (block_m) *block_m = ch.bm;
  workspace = (size_t)cp.G * cp.taps * ch.ht.ncb * ch.ht.mgp * kCB * sizeof(half_t);
  return true;
}

int prepare_igemm_halo(const Geometry& g, const Plan& p, const RunArgs& a) {
  if (g.dtype == FUSEDCONV_F32) return prepare_halo32(g, p, a);
  Choice ch;
  if (!choose(g.cp, ch)) return FUSEDCONV_ERR_ROUTE;
  return launch_repack(g.cp, ch, a);
}

int launch_igemm_halo(const Geometry& g, const Plan& p, const RunArgs& a) {
  if (g.dtype == FUSEDCONV_F32) return launch_halo32(g, p, a);  // kernels_halo32.hip
  static const ActLaunchFn table[ACT_COUNT] = FC_ACT_TABLE(launch_halo_act_);
  // the backward-data epilogue lives in the activation-free instance
  return table[g.cp.bwd ? ACT_NONE : g.cp.act](g, a);
}
#endif

}  // namespace fc
