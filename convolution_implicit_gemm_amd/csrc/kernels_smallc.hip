// Implicit GEMM on MFMA for few input channels per group (fp16 in, fp32
// accumulate): stems and patch embeddings such as a 7x7 stride-4 conv on 3
// input channels, where C/group is far below the MFMA reduction width.
//
// GEMM view per block: rows = 256 output pixels of one image tile, columns =
// 128 output channels of one group, reduction over rows of 8 consecutive
// kernel columns: k = ((c*KH + kh)*nchunk + chunk)*8 + j, tap kw = chunk*8 + j
// (taps past KW carry zero weights).  With dilation 1 along W, the 8
// reduction slots of one row are 8 consecutive input columns of one input
// row, so a lane's MFMA operand (one pixel, 8 slots) is a single 16-byte
// stretch of a channel-planar input box in LDS; for a stride that is a
// multiple of 4 it is 8-byte aligned (two ds_read_b64), otherwise it is
// read as 5 dwords and shifted.
//   * the block's input box (all C/group channels, zero outside the image) is
//     loaded once into LDS; no im2col element is gathered one by one;
//   * the weights are repacked into the row layout Wr[g][m][row][8]
//     (fusedconv_prepare_weights, or at the start of every run) and each
//     wave keeps its 64 channels x all rows in registers;
//   * each wave streams over 16-pixel tiles: MFMAs, then the fused epilogue
//     (bias seeds the accumulator, residual, activation) and one rounded
//     8-byte store per channel.  Nothing in the loop waits on global memory,
//     so the stores drain while the next tile computes.
// The GEMM formulation is the FusedConv README's implicit-GEMM one; the
// channel-planar row-chunk layout is specific to this kernel.
#include <hip/hip_runtime.h>

#include "epilogue.h"
#include "internal.h"
#include "launch.h"
#include "sync.h"

namespace fc {
namespace {

constexpr int kThreads = 256;
constexpr int kBM = 128;       // output channels per block (4 m tiles per wave)
constexpr int kBN = 256;       // output pixels per block
constexpr int kMaxKB = 6;      // reduction blocks of 32 (= 4 rows of 8 taps)
constexpr size_t kMaxLds = 80 * 1024;  // two box buffers; two blocks per CU
constexpr int kBoxBatch = 8;   // input-box chunks per thread in flight
constexpr int kPersistentBlocks = 2 * 256;  // two blocks on each of the 256 CUs

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned uint2v __attribute__((ext_vector_type(2)));

struct SmallTile {
  int TH, TW, ltw;      // output tile (TW a power of two >= 16, TH*TW = 256)
  int BH, BWL;          // input box rows and columns read
  int pitch, plane;     // LDS row pitch and channel plane, in halves (multiples of 8)
  int nchunk;           // 8-tap chunks per kernel row
  int R, KB;            // reduction rows (C/group * KH * nchunk) and blocks of 4 rows
  int tiles_h, tiles_w, ntile, nmb, mgp;
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Wr[((g*mgp + m)*KB*4 + r)*8 + j] = W[g*Mg + m][c][kh][chunk*8 + j] with
// r = (c*KH + kh)*nchunk + chunk; zero past KW, past the R rows and for the
// padding rows m >= M/group.
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
      const int kw = chunk * 8 + j;
      if (kw < cp.KW) v = w[(((int64_t)(g * cp.Mg + m) * cp.Cg + c) * cp.KH + kh) * cp.KW + kw];
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

// Persistent blocks: block b takes units b, b + gridDim.x, ...  4 waves as
// 2 x 2: wave (wpi, wmi) owns pixels [wpi*128, +128) (8 tiles of 16) and
// channels [wmi*64, +64) (4 m tiles) of each unit.  The next unit's input
// box is loaded into registers while the current unit computes and written
// to the other LDS buffer afterwards (one barrier per unit).  A4: every
// operand stretch is 8-byte aligned (stride % 4 == 0).  VEC: W % 8 == 0
// (16-byte box loads).
template <bool A4, bool VEC, int ACT>
__global__ __launch_bounds__(kThreads, 2) void smallc_kernel(const half_t* __restrict__ x,
                                                             const half_t* __restrict__ wr,
                                                             const half_t* __restrict__ bias,
                                                             const half_t* z, half_t* y,
                                                             ConvParams cp, SmallTile st) {
  extern __shared__ __attribute__((aligned(16))) half_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wpi = wave & 1, wmi = wave >> 1;
  const int r16 = lane & 15, q = lane >> 4;
  const int nunits = st.ntile * st.nmb * cp.G;
  const int box = cp.Cg * st.plane;  // halves per LDS box buffer

  // ---- input box of unit v: box row r of channel c is input row ih0 + r,
  // columns [iw0, iw0 + BWL), zero outside the image.  Loaded as the aligned
  // 8-column chunks of the image rows that overlap the box (16-byte loads
  // when W % 8 == 0); loads are unconditional (an invalid chunk reads
  // x[0..7]) and validity is applied when the chunk is written to LDS, so
  // the loads are only waited for at the write.
  const int nck_max = (st.BWL + 14) / 8;  // chunks per row, any alignment
  const int items_max = cp.Cg * st.BH * nck_max;
  const bool pf = items_max <= kThreads * kBoxBatch;  // whole box fits the prefetch registers
  half8 bv8[kBoxBatch];
  // geometry of item it of unit un's box: LDS row (c*plane + r*pitch, -1 past
  // the box), box column of the chunk's first element, in-image column mask
  struct BoxItem { int dst, col, ok; const half_t* src; };
  auto box_item = [&](const SUnit& un, int it) __attribute__((always_inline)) {
    const int ih0 = un.oh0 * cp.sh - cp.ph, iw0 = un.ow0 * cp.sw - cp.pw;
    const int c0 = (iw0 >= 0 ? iw0 : iw0 - 7) / 8;  // floor(iw0 / 8)
    const int last = iw0 + st.BWL - 1;
    const int nck = (last >= 0 ? last : last - 7) / 8 - c0 + 1;
    const int items = cp.Cg * st.BH * nck;
    const int row = it / nck, k = it - row * nck;
    const int c = row / st.BH, r = row - c * st.BH;
    const int ih = ih0 + r, cc = (c0 + k) * 8;
    const bool rok = it < items && ih >= 0 && ih < cp.H;
    BoxItem bi;
    bi.src = x + (un.n * cp.C + (int64_t)un.g * cp.Cg + c) * cp.in_sz + (int64_t)ih * cp.W + cc;
    int m = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (rok && cc + e >= 0 && cc + e < cp.W) m |= 1 << e;
    bi.ok = m;
    bi.dst = it < items ? c * st.plane + r * st.pitch : -1;
    bi.col = cc - iw0;
    return bi;
  };
  auto box_items = [&](const SUnit& un) __attribute__((always_inline)) {
    const int iw0 = un.ow0 * cp.sw - cp.pw;
    const int c0 = (iw0 >= 0 ? iw0 : iw0 - 7) / 8;
    const int last = iw0 + st.BWL - 1;
    return cp.Cg * st.BH * ((last >= 0 ? last : last - 7) / 8 - c0 + 1);
  };
  // loads only (kept in bv8 across the pixel loop; the geometry is
  // recomputed when the chunks are written, so it holds no registers)
  auto box_load = [&](const SUnit& un, int i0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kBoxBatch; ++u) {
      const BoxItem bi = box_item(un, i0 + u * kThreads + tid);
      if constexpr (VEC) {
        bv8[u] = *(const half8*)(bi.ok ? bi.src : x);  // W % 8 == 0: a chunk is all in or all out
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) bv8[u][e] = *(((bi.ok >> e) & 1) ? bi.src + e : x);
      }
    }
  };
  auto box_store = [&](const SUnit& un, int i0, half_t* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kBoxBatch; ++u) {
      const BoxItem bi = box_item(un, i0 + u * kThreads + tid);
      if (bi.dst < 0) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int col = bi.col + e;
        if (col >= 0 && col < st.BWL) buf[bi.dst + col] = ((bi.ok >> e) & 1) ? bv8[u][e] : (half_t)0;
      }
    }
  };
  // whole box of unit un into buf (batch by batch; used when not prefetched)
  auto box_fill = [&](const SUnit& un, half_t* buf) __attribute__((always_inline)) {
    const int items = box_items(un);
    for (int i0 = 0; i0 < items; i0 += kThreads * kBoxBatch) {
      box_load(un, i0);
      box_store(un, i0, buf);
    }
  };

  // ---- LDS offset (halves) of this lane's reduction row in each block:
  // row kb*4 + q = (c, kh, chunk) -> c*plane + kh*dh*pitch + chunk*8; rows
  // past R read row 0 (their weights are zero)
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

  // ---- weights (4 m tiles x KB blocks; lane row kb*4 + q, channel
  // m0 + wmi*64 + mt*16 + r16) and bias of (group, m block); reloaded when
  // a unit changes either.  Unconditional loads: blocks past KB re-read block
  // 0 (never used), a missing bias reads wr[0] and is replaced by 0.
  half8 wf[4][kMaxKB];
  float bv[4];
  int cur_g = -1, cur_mb = -1;
  auto load_weights = [&](int g, int mb) __attribute__((always_inline)) {
    const int m0 = mb * kBM;
    const half_t* wl = wr + ((int64_t)g * st.mgp + m0 + wmi * 64 + r16) * (st.KB * 4 * 8) + q * 8;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int kb = 0; kb < kMaxKB; ++kb)
        wf[mt][kb] = *(const half8*)(wl + (int64_t)mt * 16 * (st.KB * 32) + (kb < st.KB ? kb * 32 : 0));
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int m = m0 + wmi * 64 + mt * 16 + r16;
      const bool ok = cp.has_bias && m < cp.Mg;
      const float t = to_f32(*(ok ? bias + g * cp.Mg + m : wr));
      bv[mt] = ok ? t : 0.0f;
    }
    cur_g = g;
    cur_mb = mb;
  };

  const bool vec_y = (cp.OW & 3) == 0;
  int u = blockIdx.x;
  if (u >= nunits) return;
  SUnit cu = decode_unit(u, cp, st);
  box_fill(cu, lds);
  load_weights(cu.g, cu.mb);
  lds_barrier();
  for (int it = 0;; ++it) {
    const int un = u + gridDim.x;
    const bool has_next = un < nunits;
    const SUnit nu = decode_unit(has_next ? un : u, cp, st);
    if (pf) box_load(nu, 0);  // next unit's box into registers (the current one if none)
    const half_t* buf = lds + (it & 1) * box;
    const int m0 = cu.mb * kBM;
    const int64_t ybase = (cu.n * cp.M + (int64_t)cu.g * cp.Mg) * cp.out_sz;
    // ---- pixel tiles of the current unit
    for (int pt = 0; pt < 8; ++pt) {
      // operand row of lane r16: pixel wpi*128 + pt*16 + r16
      const int pa = wpi * 128 + pt * 16 + r16;
      const int pix = (pa >> st.ltw) * cp.sh * st.pitch + (pa & (st.TW - 1)) * cp.sw;
      float4v acc[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt] = float4v{bv[mt], bv[mt], bv[mt], bv[mt]};
      auto read_a = [&](int kb) __attribute__((always_inline)) {
        const int o = roff[kb] + pix;
        if constexpr (A4) {
          const uint2v lo = *(const uint2v*)(buf + o);
          const uint2v hi = *(const uint2v*)(buf + o + 4);
          return __builtin_bit_cast(half8, (__attribute__((ext_vector_type(4))) unsigned){lo[0], lo[1], hi[0], hi[1]});
        } else {
          const unsigned* d = (const unsigned*)buf + (o >> 1);
          const unsigned sh = (o & 1) * 16;
          unsigned w5[5];
#pragma unroll
          for (int k = 0; k < 5; ++k) w5[k] = d[k];
          __attribute__((ext_vector_type(4))) unsigned uu;
#pragma unroll
          for (int k = 0; k < 4; ++k) uu[k] = __builtin_amdgcn_alignbit(w5[k + 1], w5[k], sh);
          return __builtin_bit_cast(half8, uu);
        }
      };
      if (st.KB == kMaxKB) {
        // every reduction block used: all operands are read before the first
        // product, so the tile waits for LDS once, not once per block
        half8 af[kMaxKB];
#pragma unroll
        for (int kb = 0; kb < kMaxKB; ++kb) af[kb] = read_a(kb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < kMaxKB; ++kb)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[kb], wf[mt][kb], acc[mt], 0, 0, 0);
      } else {
#pragma unroll
        for (int kb = 0; kb < kMaxKB; ++kb) {
          if (kb >= st.KB) break;
          const half8 a = read_a(kb);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, wf[mt][kb], acc[mt], 0, 0, 0);
        }
      }
      // epilogue: lane holds pixels wpi*128 + pt*16 + 4q .. +3 (4 consecutive
      // columns of one tile row) of channel m0 + wmi*64 + mt*16 + r16
      const int pe = wpi * 128 + pt * 16 + 4 * q;
      const int oh = cu.oh0 + (pe >> st.ltw), ow = cu.ow0 + (pe & (st.TW - 1));
      if (oh >= cp.OH || ow >= cp.OW) continue;
      const int nv = min(4, cp.OW - ow);
      const int64_t pofs = (int64_t)oh * cp.OW + ow;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int m = m0 + wmi * 64 + mt * 16 + r16;
        if (m >= cp.Mg) continue;
        const int64_t yi = ybase + (int64_t)m * cp.out_sz + pofs;
        float4v v = acc[mt];
        if (cp.has_z) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (r < nv) v[r] += to_f32(z[yi + r]);
        }
        v = act4<ACT>(v, cp.alpha, cp.beta);
        half4 out;
#pragma unroll
        for (int r = 0; r < 4; ++r) out[r] = (half_t)v[r];
        if (vec_y && nv == 4) {
          *(half4*)(y + yi) = out;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (r < nv) y[yi + r] = out[r];
        }
      }
    }
    if (!has_next) break;
    // ---- next unit: its box into the other buffer (last read by the unit
    // before this one, whose readers all passed the previous barrier)
    half_t* nbuf = lds + ((it + 1) & 1) * box;
    if (pf) box_store(nu, 0, nbuf);
    else box_fill(nu, nbuf);
    if (nu.g != cur_g || nu.mb != cur_mb) load_weights(nu.g, nu.mb);
    lds_barrier();
    u = un;
    cu = nu;
  }
}

size_t lds_bytes(const ConvParams& cp, const SmallTile& st) {
  return (size_t)2 * cp.Cg * st.plane * sizeof(half_t);  // two box buffers
}

bool choose(const ConvParams& cp, int32_t dtype, SmallTile& st) {
  if (dtype != FUSEDCONV_F16 || !depth_trivial(cp) || cp.dw != 1 || cp.Cg > 15) return false;
  st.nchunk = (cp.KW + 7) / 8;
  st.R = cp.Cg * cp.KH * st.nchunk;
  st.KB = (st.R + 3) / 4;
  if (st.KB > kMaxKB) return false;
  // tile widths in order of padded output area, ties to the wider tile
  const int tws[] = {16, 32, 64, 128, 256};
  int best = -1;
  double best_waste = 1e30;
  for (int tw : tws) {
    const int th = kBN / tw;
    const double waste = (double)cdiv(cp.OH, th) * th * cdiv(cp.OW, tw) * tw / ((double)cp.OH * cp.OW);
    const int bh = (th - 1) * cp.sh + (cp.KH - 1) * cp.dh + 1;
    const int bwl = (tw - 1) * cp.sw + st.nchunk * 8;
    const int pitch = (bwl + 2 + 7) / 8 * 8;
    if ((size_t)2 * cp.Cg * bh * pitch * 2 > kMaxLds) continue;
    if (waste < best_waste - 1e-9 || (waste < best_waste + 1e-9 && tw > best)) {
      best = tw;
      best_waste = waste;
    }
  }
  if (best < 0 || best_waste > 2.0) return false;
  st.TW = best;
  st.TH = kBN / best;
  st.ltw = 31 - __builtin_clz((unsigned)best);
  st.BH = (st.TH - 1) * cp.sh + (cp.KH - 1) * cp.dh + 1;
  st.BWL = (st.TW - 1) * cp.sw + st.nchunk * 8;
  st.pitch = (st.BWL + 2 + 7) / 8 * 8;
  st.plane = st.BH * st.pitch;
  st.tiles_h = (int)cdiv(cp.OH, st.TH);
  st.tiles_w = (int)cdiv(cp.OW, st.TW);
  st.nmb = (int)cdiv(cp.Mg, kBM);
  st.mgp = st.nmb * kBM;
  const int64_t blocks = (int64_t)cp.G * cp.n * st.tiles_h * st.tiles_w * st.nmb;
  if (blocks >= ((int64_t)1 << 31)) return false;
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

template <bool A4, bool VEC>
int launch_t(const ConvParams& cp, const SmallTile& st, const RunArgs& a) {
  const void* kfn = (const void*)smallc_kernel<A4, VEC, FC_ACT>;
  if (set_max_dynamic_lds(kfn, (int)kMaxLds) != FUSEDCONV_OK) return FUSEDCONV_ERR_LAUNCH;
  // persistent: two blocks per CU (256 CUs), each looping over units
  const int64_t units = (int64_t)cp.G * cp.n * st.tiles_h * st.tiles_w * st.nmb;
  const unsigned blocks = (unsigned)(units < kPersistentBlocks ? units : kPersistentBlocks);
  return launch_conv(smallc_kernel<A4, VEC, FC_ACT>, dim3(blocks), dim3(kThreads),
                     lds_bytes(cp, st), a, kEdgeBoth, (const half_t*)a.x,
                     (const half_t*)a.ws, (const half_t*)a.bias, (const half_t*)a.z, (half_t*)a.y,
                     cp, st);
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
  const bool a4 = g.cp.sw % 4 == 0, vec = g.cp.W % 8 == 0;
  if (a4) return vec ? launch_t<true, true>(g.cp, st, a) : launch_t<true, false>(g.cp, st, a);
  return vec ? launch_t<false, true>(g.cp, st, a) : launch_t<false, false>(g.cp, st, a);
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
