// Implicit GEMM on MFMA for few input channels per group (fp16 in, fp32
// accumulate): stems and patch embeddings such as a 7x7 stride-4 conv on 3
// input channels, where C/group is far below the MFMA reduction width.
//
// GEMM view per work unit: rows = 128 output pixels of one image tile,
// columns = 128 output channels of one group, reduction over rows of 8
// consecutive kernel columns: k = ((c*KH + kh)*nchunk + chunk)*8 + j, tap
// kw = chunk*8 + j (taps past KW carry zero weights).  With dilation 1 along
// W, the 8 reduction slots of one row are 8 consecutive input columns of one
// input row, so a lane's MFMA operand (one pixel, 8 slots) is a single
// 16-byte stretch of a channel-planar input box in LDS; for a stride that is
// a multiple of 4 it is 8-byte aligned (two ds_read_b64), otherwise it is
// read as 5 dwords and shifted.
//
// The kernel is bound by HBM (the stem writes 2.7x the bytes it reads), so it
// is organised as a stream with three kinds of waves in one persistent block
// per CU, handing work over through LDS with one barrier per unit:
//   * 2 producer waves load the input box of unit t+2 into registers and
//     write the box of unit t+1 into LDS (zero outside the image);
//   * 8 MFMA waves (32 channels x 64 pixels each, so that every box operand
//     a wave reads from LDS feeds two channel tiles) compute unit t from its
//     box (weights repacked into the row layout Wr[g][m][row][8] by
//     fusedconv_prepare_weights or at the start of every run, held in
//     registers): all of a wave's products first (8 independent accumulator
//     chains), then the fused epilogue (bias seeds the accumulators;
//     residual, activation, one rounding) into an fp16 LDS stage;
//   * 2 store waves write unit t-1's staged results to Y as whole 16-byte
//     pieces, 8 lanes covering 64 consecutive outputs of one row.
// Loads and stores thus sit in different waves: a wave's vector-memory
// counter completes in issue order, so a wave that stored Y before loading
// the next box would wait for its stores to drain before using the box.
// The GEMM formulation is the FusedConv README's implicit-GEMM one; the
// channel-planar row-chunk layout is specific to this kernel.
#include <hip/hip_runtime.h>

#include "epilogue.h"
#include "internal.h"
#include "launch.h"
#include "sync.h"

namespace fc {
namespace {

constexpr int kMfmaWaves = 8;     // 32 output channels x 64 pixels of a unit each
constexpr int kThreads = (kMfmaWaves + 4) * 64;  // + 2 producer waves + 2 store waves
constexpr int kRoleLanes = 128;  // lanes of the producer and of the store role
constexpr int kBM = 128;       // output channels per unit
constexpr int kBN = 128;       // output pixels per unit (8 pixel tiles of 16)
constexpr int kMaxKB = 6;      // reduction blocks of 32 (= 4 rows of 8 taps)
constexpr size_t kMaxLds = 160 * 1024;  // one block per CU
constexpr int kBoxBatch = 12;  // box chunks per producer lane: a box holds up to 1536 chunks
constexpr int kBoxChunks = kRoleLanes * kBoxBatch;
constexpr int kBoxBufs = 3;    // box buffers: unit t computed, t+1 ready, t+2 loading
constexpr int kSP = kBN + 8;   // stage pitch per output channel, halves
constexpr int kPersistentBlocks = 256;  // one block on each of the 256 CUs
// Standard normal CDF table for the erf-form Gelu and Erf activations:
// Phi at x_i = -6 + i/64, i = 0 .. kPhiN, stored with the step to the next
// entry, so Phi(x) = Phi_i + f * (Phi_{i+1} - Phi_i) by linear interpolation.
// Interpolation error <= h^2/8 * max|Phi''| = 7.4e-6 (h = 1/64, max|Phi''| =
// phi(1) = 0.242), so |Gelu error| <= 6 * 7.4e-6 = 4.4e-5 on [-6, 6]; past
// +-6 the table's end values are used (|Gelu(-6)| = 6e-9).  About a third of
// the VALU work of the rational erf approximation, which made this kernel
// VALU-bound: the stem applies Gelu to 151 million outputs.
constexpr int kPhiN = 768;
constexpr float kPhiScale = 64.0f, kPhiOrigin = 384.0f;  // i + f = 64 x + 384
// largest float below kPhiN: i = floor(u) <= kPhiN - 1 and f = u - i < 1; at
// the top (x >= 6) Phi_{kPhiN-1} + f * step differs from Phi_{kPhiN} by 6e-8
// of a step of 1e-10
constexpr float kPhiTop = 767.99994f;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned uint2v __attribute__((ext_vector_type(2)));

struct SmallTile {
  int TH, TW, ltw;      // output tile (TW a power of two >= 16, TH*TW = kBN)
  int BH, BWL;          // input box rows and columns the windows read
  int NCK;              // 8-column chunks per LDS box row (covers any alignment)
  int pitch, plane;     // LDS row pitch (NCK*8) and channel plane, in halves
  int items;            // chunks per box: C/group * BH * NCK
  int nchunk;           // 8-slot chunks per kernel row
  int s;                // tap shift: slot j of chunk holds tap kw = chunk*8 + j - s
  int R, KB;            // reduction rows (C/group * KH * nchunk) and blocks of 4 rows
  int tiles_h, tiles_w, ntile, nmb, mgp;
};

// Word 3 of a raw buffer resource on gfx9-class GPUs: 32-bit data format,
// untyped access (offsets past num_records read zero).
constexpr int kBufferWord3 = 0x00020000;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Wr[((g*mgp + m)*KB*4 + r)*8 + j] = W[g*Mg + m][c][kh][chunk*8 + j - s] with
// r = (c*KH + kh)*nchunk + chunk; zero outside [0, KW), past the R rows and
// for the padding rows m >= M/group.  The shift s puts the first tap of every
// window on a 4-column boundary of the box when the stride is a multiple of
// 4 (window start iw0 - s = 0 mod 4), so that operands are 8-byte aligned.
__global__ __launch_bounds__(kThreads) void repack_rows_kernel(const half_t* __restrict__ w,
                                                               half_t* __restrict__ wr,
                                                               ConvParams cp, SmallTile st) {
  const int64_t rows = (int64_t)st.KB * 4;
  const int64_t total = (int64_t)cp.G * st.mgp * rows * 8;
  const int64_t step = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += step) {
    const int j = (int)(i & 7);
    int64_t t = i >> 3;
    const int r = (int)(t % rows);
    t /= rows;
    const int m = (int)(t % st.mgp);
    const int g = (int)(t / st.mgp);
    half_t v = (half_t)0;
    if (r < st.R && m < cp.Mg) {
      const int chunk = r % st.nchunk, ck = r / st.nchunk;
      const int kh = ck % cp.KH, c = ck / cp.KH;
      const int kw = chunk * 8 + j - st.s;
      if (kw >= 0 && kw < cp.KW) v = w[(((int64_t)(g * cp.Mg + m) * cp.Cg + c) * cp.KH + kh) * cp.KW + kw];
    }
    wr[i] = v;
  }
}

// Work unit u = ((g*n + image)*tiles_h + th)*tiles_w + tw)*nmb + mb.
struct SUnit {
  int64_t n;
  int g, mb, oh0, ow0;
};
__device__ __forceinline__ SUnit decode_unit(int u, const ConvParams& cp, const SmallTile& st) {
  SUnit r;
  r.mb = u % st.nmb;
  u /= st.nmb;
  const int tw_i = u % st.tiles_w;
  u /= st.tiles_w;
  const int th_i = u % st.tiles_h;
  u /= st.tiles_h;
  r.n = u % cp.n;
  r.g = (int)(u / cp.n);
  r.oh0 = th_i * st.TH;
  r.ow0 = tw_i * st.TW;
  return r;
}

// Persistent blocks: block b takes units f, f + gridDim.x, ... (nu of them),
// f a permutation of b (below).
// Box buffers rotate over kBoxBufs = 3: in interval t (t = 0 .. nu, one
// barrier at its end) the MFMA waves compute unit t from box buffer t % 3
// into stage buffer t & 1, the producers fill box buffer (t+2) % 3 with unit
// t+2 (and have unit t+1's box complete before the barrier), and the store
// waves write unit t-1 from stage buffer (t-1) & 1.  A box buffer is refilled
// one interval after its last reader, a stage buffer one interval after.
// Box layout: chunk i = (c*BH + r)*NCK + k (input channel c, box row r =
// input row ih0 + r, input columns bx0 + 8k .. +7 with bx0 = 8 floor(ws / 8),
// ws = iw0 - s the window start) at halves 8i, zero outside the image; the
// windows start delta = ws - bx0 halves into each row.  VEC (W % 8 == 0):
// each chunk is in or out of the image as a whole, and the producers load it
// straight into LDS (buffer_load ... lds; an out-of-range offset for the
// chunks outside the image writes zeros).  Otherwise the producers load
// chunks into registers, zero what is outside and write them.  A4: stride
// % 4 == 0, with s chosen so that delta % 4 == 0: every operand stretch is
// 8-byte aligned (the launcher checks (pw + s) % 4 == 0).  VY: OW % 8 == 0
// (16-byte stores of Y).  HZ: a residual Z is added (no residual code or
// loads otherwise).
template <bool A4, bool VEC, bool VY, bool HZ, int ACT>
__global__ __launch_bounds__(kThreads, 1) void smallc_kernel(const half_t* __restrict__ x,
                                                             const half_t* __restrict__ wr,
                                                             const half_t* __restrict__ bias,
                                                             const half_t* z, half_t* y,
                                                             ConvParams cp, SmallTile st) {
  extern __shared__ __attribute__((aligned(16))) half_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nunits = st.ntile * st.nmb * cp.G;
  constexpr int box = kBoxChunks * 8;  // halves per LDS box buffer
  half_t* const stage0 = lds + kBoxBufs * box;  // two stage buffers of kBM x kSP halves
  // Phi table (erf-form Gelu and Erf): (Phi_i, Phi_{i+1} - Phi_i) pairs
  float2* const phi = (float2*)(stage0 + 2 * kBM * kSP);
  constexpr bool kPhiAct = ACT == ACT_GELU || ACT == ACT_ERF;
  // Block b runs on XCD b % 8.  With a grid of 8k blocks, interval t's units
  // tB .. tB + B - 1 are dealt so that XCD x takes the k consecutive units
  // tB + kx .. tB + kx + k - 1: neighbouring tiles of one image, whose boxes
  // share input rows and columns, run on one XCD at about the same time and
  // read the shared lines from its L2 rather than from HBM once per XCD.
  const int first = (gridDim.x & 7) == 0 ? (int)((blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3))
                                         : (int)blockIdx.x;
  const int nu = first < nunits ? (nunits - 1 - first) / (int)gridDim.x + 1 : 0;
  auto unit_of = [&](int t) __attribute__((always_inline)) {
    return decode_unit(first + t * (int)gridDim.x, cp, st);
  };
  // first input column of the unit's chunks (a multiple of 8) and the
  // window's offset from it
  auto box_x0 = [&](const SUnit& un) __attribute__((always_inline)) {
    const int ws = un.ow0 * cp.sw - cp.pw - st.s;
    return (ws >= 0 ? ws : ws - 7) / 8 * 8;
  };

  if (wave >= kMfmaWaves + 2) {
    // ======================= store waves =======================
    const int sl = tid - (kMfmaWaves + 2) * 64;  // 0 .. 127
    lds_barrier();  // the producers' first box is in LDS
    for (int t = 0; t <= nu; ++t) {
      if (t >= 1) {
        const SUnit cu = unit_of(t - 1);
        const half_t* sb = stage0 + ((t - 1) & 1) * kBM * kSP;
        const int m0 = cu.mb * kBM;
        half_t* yb = y + (cu.n * cp.M + (int64_t)cu.g * cp.Mg + m0) * cp.out_sz;
        // chunk c: channel c / 16, pixels 8 (c % 16) .. +7 of the unit (one
        // tile row); consecutive lanes take consecutive chunks, so 8 lanes
        // write 64 consecutive outputs of a row
#pragma unroll 4
        for (int i = 0; i < kBM * (kBN / 8) / kRoleLanes; ++i) {
          const int c = sl + i * kRoleLanes;
          const int ch = c >> 4, p0 = (c & 15) << 3;
          const int row = p0 >> st.ltw, col = p0 & (st.TW - 1);
          const int oh = cu.oh0 + row, ow = cu.ow0 + col;
          if (m0 + ch >= cp.Mg || oh >= cp.OH || ow >= cp.OW) continue;
          const half8 v = *(const half8*)(sb + ch * kSP + p0);
          half_t* dst = yb + (int64_t)ch * cp.out_sz + oh * cp.OW + ow;
          if (VY && ow + 8 <= cp.OW) {
            *(half8*)dst = v;
          } else {
            const int nv = min(8, cp.OW - ow);
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (e < nv) dst[e] = v[e];
          }
        }
      }
      lds_barrier();
    }
    return;
  }

  if (wave >= kMfmaWaves) {
    // ======================= producer waves =======================
    // Chunk i = u*128 + pl of the box (u < kBoxBatch) is this lane's u-th;
    // its unit-independent element offset (channel, row, 8k) and (r, k) are
    // computed once.
    const int pl = tid - kMfmaWaves * 64;  // 0 .. 127
    int goff[kBoxBatch], rk[kBoxBatch];
#pragma unroll
    for (int u = 0; u < kBoxBatch; ++u) {
      const int i = u * kRoleLanes + pl;
      const int k = i % st.NCK, cr = i / st.NCK;
      const int r = cr % st.BH, c = cr / st.BH;
      const bool ok = i < st.items;
      goff[u] = ok ? c * (int)cp.in_sz + r * cp.W + 8 * k : 0;
      rk[u] = ok ? (r << 16) | k : -1;
    }
    // element offset of chunk u of unit un from the unit's channel-group
    // base, or -1 when the chunk (a whole one: W % 8 == 0) is outside
    auto chunk_off = [&](const SUnit& un, int u) __attribute__((always_inline)) {
      const int ih0 = un.oh0 * cp.sh - cp.ph, bx0 = box_x0(un);
      const int ih = ih0 + (rk[u] >> 16), cc = bx0 + 8 * (rk[u] & 0xffff);
      const bool ok = rk[u] >= 0 && (unsigned)ih < (unsigned)cp.H && cc >= 0 && cc < cp.W;
      return ok ? goff[u] + ih0 * cp.W + bx0 : -1;
    };
    if constexpr (VEC) {
      const int pw = wave - kMfmaWaves;  // 0, 1: chunk blocks of 64 interleave
      // unit t's box into buffer t % 3, straight from global memory; the
      // chunk block of instruction u is 2u + pw (64 chunks, 1 KB)
      auto issue = [&](int t) __attribute__((always_inline)) {
        const SUnit un = unit_of(t);
        const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(x + (un.n * cp.C + (int64_t)un.g * cp.Cg) * cp.in_sz), (short)0,
            (int)(cp.Cg * cp.in_sz * 2), kBufferWord3);
        half_t* bb = lds + (t % kBoxBufs) * box;
#pragma unroll
        for (int u = 0; u < kBoxBatch; ++u) {
          // this lane's chunk of block 2u + pw is chunk (2u + pw)*64 + lane,
          // i.e. u' = u, pl = pw*64 + lane in the numbering above
          const int o = chunk_off(un, u);
          const unsigned voff = o >= 0 ? (unsigned)o * 2u : 0x80000000u;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              xr, (__attribute__((address_space(3))) void*)(bb + (u * kRoleLanes + pw * 64) * 8), 16,
              voff, 0, 0, 0);
        }
      };
      // vmcnt(n) immediate for gfx9: low 4 bits, high 2 bits at 15:14;
      // expcnt and lgkmcnt not waited for
      constexpr int kWaitKeep = (kBoxBatch & 15) | (7 << 4) | (15 << 8) | ((kBoxBatch >> 4) << 14);
      constexpr int kWaitAll = (7 << 4) | (15 << 8);
      if (nu > 0) issue(0);
      if (nu > 1) issue(1);
      // unit 0 complete (unit 1's loads may stay in flight)
      if (nu > 1) __builtin_amdgcn_s_waitcnt(kWaitKeep);
      else __builtin_amdgcn_s_waitcnt(kWaitAll);
      __builtin_amdgcn_s_barrier();
      for (int t = 0; t <= nu; ++t) {
        if (t + 2 < nu) issue(t + 2);
        // unit t+1's box complete before the barrier (unit t+2's in flight)
        if (t + 2 < nu) __builtin_amdgcn_s_waitcnt(kWaitKeep);
        else __builtin_amdgcn_s_waitcnt(kWaitAll);
        __builtin_amdgcn_s_barrier();
      }
    } else {
      half8 bv8[kBoxBatch];
      auto box_load = [&](const SUnit& un) __attribute__((always_inline)) {
        const int ih0 = un.oh0 * cp.sh - cp.ph, bx0 = box_x0(un);
        const int64_t base = (un.n * cp.C + (int64_t)un.g * cp.Cg) * cp.in_sz + (int64_t)ih0 * cp.W + bx0;
#pragma unroll
        for (int u = 0; u < kBoxBatch; ++u) {
          const int ih = ih0 + (rk[u] >> 16), cc = bx0 + 8 * (rk[u] & 0xffff);
          const bool rok = rk[u] >= 0 && (unsigned)ih < (unsigned)cp.H;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const bool ok = rok && cc + e >= 0 && cc + e < cp.W;
            bv8[u][e] = *(ok ? x + base + goff[u] + e : x);
          }
        }
      };
      auto box_store = [&](const SUnit& un, half_t* buf) __attribute__((always_inline)) {
        const int ih0 = un.oh0 * cp.sh - cp.ph, bx0 = box_x0(un);
#pragma unroll
        for (int u = 0; u < kBoxBatch; ++u) {
          if (rk[u] < 0) continue;
          const int ih = ih0 + (rk[u] >> 16), cc = bx0 + 8 * (rk[u] & 0xffff);
          const bool rok = (unsigned)ih < (unsigned)cp.H;
          half8 v = bv8[u];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (!(rok && cc + e >= 0 && cc + e < cp.W)) v[e] = (half_t)0;
          *(half8*)(buf + (u * kRoleLanes + pl) * 8) = v;
        }
      };
      if (nu > 0) {
        box_load(unit_of(0));
        box_store(unit_of(0), lds);
      }
      if (nu > 1) box_load(unit_of(1));
      lds_barrier();
      for (int t = 0; t <= nu; ++t) {
        if (t + 1 < nu) {
          box_store(unit_of(t + 1), lds + ((t + 1) % kBoxBufs) * box);
          if (t + 2 < nu) box_load(unit_of(t + 2));
        }
        lds_barrier();
      }
    }
    return;
  }

  // ======================= MFMA waves =======================
  // wave wmi owns channels [32 wm, +32) (two m tiles) of the unit's 128
  // channels and pixels [64 wp, +64) (four pixel tiles): each box operand it
  // reads serves two channel tiles
  const int wmi = wave;
  const int wm = wmi & 3, wp = wmi >> 2;
  const int r16 = lane & 15, q = lane >> 4;
  // LDS offset (halves) of this lane's reduction row in each block: row
  // kb*4 + q = (c, kh, chunk) -> c*plane + kh*dh*pitch + chunk*8; rows past R
  // read row 0 (their weights are zero)
  int roff[kMaxKB];
#pragma unroll
  for (int kb = 0; kb < kMaxKB; ++kb) {
    const int r = kb * 4 + q;
    int o = 0;
    if (r < st.R) {
      const int chunk = r % st.nchunk, ck = r / st.nchunk;
      const int kh = ck % cp.KH, c = ck / cp.KH;
      o = c * st.plane + kh * cp.dh * st.pitch + chunk * 8;
    }
    roff[kb] = o;
  }
  // weights (KB blocks; lane row kb*4 + q, channel m0 + wmi*16 + r16) and
  // bias of (group, m block); reloaded when a unit changes either.
  // Unconditional loads: blocks past KB re-read block 0 (never used), a
  // missing bias reads wr[0] and is replaced by 0.
  half8 wf[2][kMaxKB];
  float bv[2] = {0.0f, 0.0f};
  int cur_g = -1, cur_mb = -1;
  auto load_weights = [&](int g, int mb) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int m = mb * kBM + (2 * wm + ct) * 16 + r16;
      const half_t* wl = wr + ((int64_t)g * st.mgp + m) * (st.KB * 4 * 8) + q * 8;
#pragma unroll
      for (int kb = 0; kb < kMaxKB; ++kb) wf[ct][kb] = *(const half8*)(wl + (kb < st.KB ? kb * 32 : 0));
      const bool ok = cp.has_bias && m < cp.Mg;
      const float t = to_f32(*(ok ? bias + g * cp.Mg + m : wr));
      bv[ct] = ok ? t : 0.0f;
    }
    cur_g = g;
    cur_mb = mb;
  };

  if constexpr (kPhiAct) {
    // Phi(x_i) = erfc(-x_i / sqrt 2) / 2, in double
    for (int i = tid; i <= kPhiN; i += kMfmaWaves * 64) {
      const double x0 = (i - (double)kPhiOrigin) / kPhiScale;
      const double p0 = 0.5 * erfc(-x0 * 0.70710678118654752440);
      const double p1 = i < kPhiN ? 0.5 * erfc(-(x0 + 1.0 / kPhiScale) * 0.70710678118654752440) : p0;
      phi[i] = float2{(float)p0, (float)(p1 - p0)};
    }
  }
  // Phi by the table at x (clamped to the table's range)
  auto phi_of = [&](float xv) __attribute__((always_inline)) {
    const float u = __builtin_amdgcn_fmed3f(fmaf(xv, kPhiScale, kPhiOrigin), 0.0f, kPhiTop);
    const float2 pe = phi[(int)u];
    return fmaf(__builtin_amdgcn_fractf(u), pe.y, pe.x);
  };
  // operand row of lane r16 in pixel tile pt4: pixel (wp*4 + pt4)*16 + r16
  // of the unit, at this LDS offset from the window start
  int pixb[kBN / 32];
#pragma unroll
  for (int pt4 = 0; pt4 < kBN / 32; ++pt4) {
    const int pa = (wp * (kBN / 32) + pt4) * 16 + r16;
    pixb[pt4] = (pa >> st.ltw) * cp.sh * st.pitch + (pa & (st.TW - 1)) * cp.sw;
  }
  lds_barrier();  // the producers' first box is in LDS; the Phi table is written
  for (int t = 0; t <= nu; ++t) {
    if (t < nu) {
      const SUnit cu = unit_of(t);
      if (cu.g != cur_g || cu.mb != cur_mb) load_weights(cu.g, cu.mb);
      const int delta = cu.ow0 * cp.sw - cp.pw - st.s - box_x0(cu);  // 0 .. 7
      const half_t* buf = lds + (t % kBoxBufs) * box;
      constexpr int kPT = kBN / 32;  // pixel tiles per wave
      // residuals of this lane's 4 pixels in each (pixel tile, channel tile),
      // requested before the products (8-byte loads when OW % 4 == 0, so
      // that a lane's 4 pixels are all in or all out of the row)
      uint2v zr[kPT][2];
#pragma unroll
      for (int pt4 = 0; pt4 < kPT; ++pt4)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          zr[pt4][ct] = uint2v{0u, 0u};
          if (HZ && (cp.OW & 3) == 0) {
            const int pe = (wp * kPT + pt4) * 16 + 4 * q;
            const int m = cu.mb * kBM + (2 * wm + ct) * 16 + r16;
            const int64_t zbase = (cu.n * cp.M + (int64_t)cu.g * cp.Mg + m) * cp.out_sz;
            const int oh = cu.oh0 + (pe >> st.ltw), ow = cu.ow0 + (pe & (st.TW - 1));
            const bool ok = m < cp.Mg && oh < cp.OH && ow < cp.OW;
            zr[pt4][ct] = *(const uint2v*)(ok ? z + zbase + oh * cp.OW + ow : z);
          }
        }
      auto read_a = [&](int pix, int kb) __attribute__((always_inline)) {
        const int o = roff[kb] + pix;
        if constexpr (A4) {
          const uint2v lo = *(const uint2v*)(buf + o);
          const uint2v hi = *(const uint2v*)(buf + o + 4);
          return __builtin_bit_cast(half8, (__attribute__((ext_vector_type(4))) unsigned){lo[0], lo[1], hi[0], hi[1]});
        }
        // any alignment: 5 dwords, shifted
        const unsigned* d = (const unsigned*)buf + (o >> 1);
        const unsigned sh = (o & 1) * 16;
        unsigned w5[5];
#pragma unroll
        for (int k = 0; k < 5; ++k) w5[k] = d[k];
        __attribute__((ext_vector_type(4))) unsigned uu;
#pragma unroll
        for (int k = 0; k < 4; ++k) uu[k] = __builtin_amdgcn_alignbit(w5[k + 1], w5[k], sh);
        return __builtin_bit_cast(half8, uu);
      };
      // the products of all the wave's tiles first (8 independent
      // accumulator chains keep the matrix core busy), then one wait-state
      // gap, then the epilogues (32 independent values)
      float4v acc[kPT][2];
#pragma unroll
      for (int pt4 = 0; pt4 < kPT; ++pt4) {
        const int pix = pixb[pt4] + delta;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) acc[pt4][ct] = float4v{bv[ct], bv[ct], bv[ct], bv[ct]};
#pragma unroll
        for (int kb = 0; kb < kMaxKB; ++kb) {
          if (kb >= st.KB) break;
          const half8 af = read_a(pix, kb);
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
            acc[pt4][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, wf[ct][kb], acc[pt4][ct], 0, 0, 0);
        }
      }
      // The accumulators are read by VALU soon after the last MFMA; the
      // compiler's wait states for v_mfma_f32_16x16x32_f16 results were
      // measured too few on gfx950 (the second half of an accumulator read
      // stale), so 32 wait states are forced here.
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int pt4 = 0; pt4 < kPT; ++pt4)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        // lane holds pixels pt*16 + 4q .. +3 (4 consecutive columns of one
        // tile row) of channel (2 wm + ct)*16 + r16; residual, activation and
        // the rounding here, the store from the stage
        const int pe = (wp * kPT + pt4) * 16 + 4 * q;
        const int m = cu.mb * kBM + (2 * wm + ct) * 16 + r16;
        half_t* sb = stage0 + (t & 1) * kBM * kSP + ((2 * wm + ct) * 16 + r16) * kSP;
        float4v v = acc[pt4][ct];
        if constexpr (HZ) {
          if ((cp.OW & 3) == 0) {
            const half4 zh = __builtin_bit_cast(half4, zr[pt4][ct]);
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] += (float)zh[r];
          } else {
            // OW % 4 != 0: element by element (a lane's 4 pixels may leave the row)
            const int64_t zbase = (cu.n * cp.M + (int64_t)cu.g * cp.Mg + m) * cp.out_sz;
            const int oh = cu.oh0 + (pe >> st.ltw), ow = cu.ow0 + (pe & (st.TW - 1));
            if (m < cp.Mg && oh < cp.OH) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (ow + r < cp.OW) v[r] += to_f32(z[zbase + oh * cp.OW + ow + r]);
            }
          }
        }
        if constexpr (ACT == ACT_GELU) {
          // erf form: x * Phi(x) (a nonzero approximate flag is planned as FastGelu)
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = v[r] * phi_of(v[r]);
        } else if constexpr (ACT == ACT_ERF) {
          // erf(x) = 2 Phi(sqrt 2 x) - 1
#pragma unroll
          for (int r = 0; r < 4; ++r)
            v[r] = v[r] != v[r] ? v[r] : fmaf(2.0f, phi_of(v[r] * 1.41421356237309505f), -1.0f);
        } else {
          v = act4<ACT>(v, cp.alpha, cp.beta);
        }
        half4 out;
#pragma unroll
        for (int r = 0; r < 4; ++r) out[r] = (half_t)v[r];
        *(half4*)(sb + pe) = out;
      }
    }
    lds_barrier();
  }
}

// box buffers, two stage buffers of kBM channels x kSP halves, the Phi table
size_t lds_bytes() {
  return ((size_t)kBoxBufs * kBoxChunks * 8 + (size_t)2 * kBM * kSP) * sizeof(half_t) +
         (size_t)(kPhiN + 1) * 2 * sizeof(float);
}

bool choose(const ConvParams& cp, int32_t dtype, SmallTile& st) {
  if (dtype != FUSEDCONV_F16 || !depth_trivial(cp) || cp.dw != 1 || cp.Cg > 15) return false;
  if (lds_bytes() > kMaxLds) return false;
  // tap shift: with a stride that is a multiple of 4 every window starts at
  // -pw (mod 4); starting the reduction rows s columns earlier puts them on
  // a 4-column boundary (operands 8-byte aligned), if the rows still fit
  st.s = cp.sw % 4 == 0 ? ((-cp.pw) % 4 + 4) % 4 : 0;
  st.nchunk = (cp.KW + st.s + 7) / 8;
  if (cp.Cg * cp.KH * st.nchunk > 4 * kMaxKB && st.s != 0) {
    st.s = 0;
    st.nchunk = (cp.KW + 7) / 8;
  }
  st.R = cp.Cg * cp.KH * st.nchunk;
  st.KB = (st.R + 3) / 4;
  if (st.KB > kMaxKB) return false;
  // tile widths by padded output area, weighted by the input rows the box
  // reads per output row (box rows shared with the neighbouring tiles are
  // read again, from L2); tiles narrower than 64 outputs write Y rows in
  // pieces shorter than a 128-byte line, which costs extra HBM writes
  const int tws[] = {16, 32, 64, 128};  // TW <= kBN, TH = kBN / TW
  int best = -1;
  double best_waste = 1e30, best_cost = 1e30;
  for (int tw : tws) {
    const int th = kBN / tw;
    const double waste = (double)cdiv(cp.OH, th) * th * cdiv(cp.OW, tw) * tw / ((double)cp.OH * cp.OW);
    const int bh = (th - 1) * cp.sh + (cp.KH - 1) * cp.dh + 1;
    const int bwl = (tw - 1) * cp.sw + st.nchunk * 8;
    const int nck = (bwl + 7 + 7) / 8;
    if (cp.Cg * bh * nck > kBoxChunks) continue;  // a box buffer's chunks
    const double reread = (double)bh / (th * cp.sh);
    const double cost = waste * (1.0 + 0.25 * (reread - 1.0)) + (tw < 64 ? 0.1 : 0.0);
    if (cost < best_cost - 1e-9 || (cost < best_cost + 1e-9 && tw > best)) {
      best = tw;
      best_waste = waste;
      best_cost = cost;
    }
  }
  if (best < 0 || best_waste > 2.0) return false;
  st.TW = best;
  st.TH = kBN / best;
  st.ltw = 31 - __builtin_clz((unsigned)best);
  st.BH = (st.TH - 1) * cp.sh + (cp.KH - 1) * cp.dh + 1;
  st.BWL = (st.TW - 1) * cp.sw + st.nchunk * 8;
  // NCK chunks cover delta + BWL columns for any window offset delta < 8;
  // rows are contiguous (pitch NCK*8), so a box is one run of chunks; the
  // 5-dword operand reads end at most 2 halves past a window, inside the
  // buffer (a buffer holds kBoxChunks >= items chunks plus the next buffer
  // or the stage after it)
  st.NCK = (st.BWL + 7 + 7) / 8;
  st.pitch = st.NCK * 8;
  st.plane = st.BH * st.pitch;
  st.items = cp.Cg * st.BH * st.NCK;
  st.tiles_h = (int)cdiv(cp.OH, st.TH);
  st.tiles_w = (int)cdiv(cp.OW, st.TW);
  st.nmb = (int)cdiv(cp.Mg, kBM);
  st.mgp = st.nmb * kBM;
  const int64_t blocks = (int64_t)cp.G * cp.n * st.tiles_h * st.tiles_w * st.nmb;
  if (blocks >= ((int64_t)1 << 31)) return false;
  // 32-bit offsets: a unit's kBM output channels (residual), and one image's
  // channel group of X in bytes (the box loads' buffer range)
  if ((int64_t)kBM * cp.out_sz * 2 >= ((int64_t)1 << 31)) return false;
  if ((int64_t)cp.Cg * cp.in_sz * 2 >= ((int64_t)1 << 31)) return false;
  st.ntile = (int)(cp.n * st.tiles_h * st.tiles_w);
  return true;
}

int launch_repack(const ConvParams& cp, const SmallTile& st, const RunArgs& a) {
  const int64_t total = (int64_t)cp.G * st.mgp * st.KB * 4 * 8;
  int64_t rblocks = (total + kThreads - 1) / kThreads;
  if (rblocks > 4096) rblocks = 4096;
  hipLaunchKernelGGL(repack_rows_kernel, dim3((unsigned)rblocks), dim3(kThreads), 0,
                     (hipStream_t)a.stream, (const half_t*)a.w, (half_t*)a.ws, cp, st);
  return hipPeekAtLastError() == hipSuccess ? FUSEDCONV_OK : FUSEDCONV_ERR_LAUNCH;
}

template <bool A4, bool VEC, bool VY, bool HZ>
int launch_hz(const ConvParams& cp, const SmallTile& st, const RunArgs& a) {
  const void* kfn = (const void*)smallc_kernel<A4, VEC, VY, HZ, FC_ACT>;
  if (set_max_dynamic_lds(kfn, (int)kMaxLds) != FUSEDCONV_OK) return FUSEDCONV_ERR_LAUNCH;
  // persistent: one block per CU (256 CUs), each looping over units
  const int64_t units = (int64_t)cp.G * cp.n * st.tiles_h * st.tiles_w * st.nmb;
  const unsigned blocks = (unsigned)(units < kPersistentBlocks ? units : kPersistentBlocks);
  return launch_conv(smallc_kernel<A4, VEC, VY, HZ, FC_ACT>, dim3(blocks), dim3(kThreads),
                     lds_bytes(), a, kEdgeBoth, (const half_t*)a.x,
                     (const half_t*)a.ws, (const half_t*)a.bias, (const half_t*)a.z, (half_t*)a.y,
                     cp, st);
}

template <bool A4, bool VEC, bool VY>
int launch_t(const ConvParams& cp, const SmallTile& st, const RunArgs& a) {
  return cp.has_z ? launch_hz<A4, VEC, VY, true>(cp, st, a) : launch_hz<A4, VEC, VY, false>(cp, st, a);
}

}  // namespace

#ifndef FC_ACT
#error "compiled once per activation id: -DFC_ACT=<0..ACT_COUNT-1>"
#endif

// the SMALLC route with activation FC_ACT
int FC_CAT(launch_smallc_act_, FC_ACT)(const Geometry& g, const RunArgs& a) {
  SmallTile st;
  if (!choose(g.cp, g.dtype, st)) return FUSEDCONV_ERR_ROUTE;
  if (!(a.flags & FUSEDCONV_RUN_WEIGHTS_PREPARED)) {
    const int rc = launch_repack(g.cp, st, a);
    if (rc != FUSEDCONV_OK) return rc;
  }
  // 8-byte aligned operands: windows start at ow0*sw - pw - s = -(pw + s) (mod 4)
  const bool a4 = g.cp.sw % 4 == 0 && (g.cp.pw + st.s) % 4 == 0;
  const bool vec = g.cp.W % 8 == 0, vy = g.cp.OW % 8 == 0;
  if (a4) {
    if (vec) return vy ? launch_t<true, true, true>(g.cp, st, a) : launch_t<true, true, false>(g.cp, st, a);
    return vy ? launch_t<true, false, true>(g.cp, st, a) : launch_t<true, false, false>(g.cp, st, a);
  }
  if (vec) return vy ? launch_t<false, true, true>(g.cp, st, a) : launch_t<false, true, false>(g.cp, st, a);
  return vy ? launch_t<false, false, true>(g.cp, st, a) : launch_t<false, false, false>(g.cp, st, a);
}

#if FC_ACT == 0
FC_ACT_DECLS(launch_smallc_act_)

bool smallc_fits(const ConvParams& cp, int32_t dtype, int32_t& tile_h, int32_t& tile_w,
                 size_t& workspace) {
  SmallTile st;
  if (!choose(cp, dtype, st)) return false;
  tile_h = st.TH;
  tile_w = st.TW;
  workspace = (size_t)cp.G * st.mgp * st.KB * 4 * 8 * sizeof(half_t);
  return true;
}

int prepare_smallc(const Geometry& g, const Plan&, const RunArgs& a) {
  SmallTile st;
  if (!choose(g.cp, g.dtype, st)) return FUSEDCONV_ERR_ROUTE;
  return launch_repack(g.cp, st, a);
}

int launch_smallc(const Geometry& g, const Plan&, const RunArgs& a) {
  static const ActLaunchFn table[ACT_COUNT] = FC_ACT_TABLE(launch_smallc_act_);
  return table[g.cp.act](g, a);
}
#endif

}  // namespace fc
