// Depthwise convolution (one input channel per group, stride 1, 2 spatial
// dims, fp16) on the matrix cores.
//
// A depthwise output row is a 1-D correlation of input rows with the kernel
// rows: y[oh][ow] = sum_kh sum_kw x[oh + dh*kh][ow + dw*kw] w[kh][kw] (padded
// coordinates).  For one kernel row kh and a block of 16 output columns this
// is a product with a banded (Toeplitz) matrix: with 16 output rows as the
// M side, the input columns of the window as the K side and the 16 output
// columns as the N side,
//     D[r][j] += sum_k  X[oh0 + r + dh*kh][ow0 + k] * T_kh[j][k],
//     T_kh[j][k] = w[kh][(k - j) / dw]   when k - j = dw*kw, 0 <= kw < KW,
// so one v_mfma_f32_16x16x32_f16 per kernel row covers a 16x16 output tile
// when 16 + dw*(KW-1) <= 32.  Only KW of the 32 products per output are
// non-zero, but the matrix cores run ~16x the packed-fp16 VALU rate, which
// leaves the kernel bound by HBM rather than by issue (the VALU form needs
// ~28 v_dot2 per output of a 7x7 kernel).  Products are exact in fp32 and
// the sums are fp32, as in the FusedConv manifest's grouped-kernel variants
// (fp32 accumulation seeded by the bias).
//
// Layout on gfx950:
//   * block b owns channel b % M and walks every k-th image, so the k*M
//     blocks read one compact window of memory at a time; its Toeplitz
//     fragments (KH x 8 halves per lane, from an LDS table of zero-padded
//     kernel rows) are built once;
//   * each input plane is copied into LDS with 16-byte loads and stores at
//     a column shift S that puts input column 0 on an 8-column boundary, so
//     every B fragment is one aligned ds_read_b128; the zero border (the
//     padding) is written once per block and never overwritten;
//   * output tiles start at column -S (their first S columns are dropped);
//   * a wave's work item is 4 interleaved 16 x 16 tiles: output rows
//     64v + 4r + p (p = 0..3) for one 16-column block.  Tile p at kernel row
//     kh reads input rows 64v + 4r + p + dh*kh, so the 4*KH products of the
//     item need only 4 + dh*(KH-1) distinct B fragments (10 instead of 28
//     for a 7x7 kernel), which keeps LDS traffic below the HBM time;
//   * the fp32 results go through an LDS stage so bias, residual Z and the
//     activation run on contiguous 4-element runs with 8-byte global loads
//     and stores; the input is the A operand and the Toeplitz matrix the B
//     operand, so a lane's accumulators are 4 rows of one output column and
//     16 lanes write 16 consecutive stage words;
//   * each lane holds the input of the next 3 planes in registers (3 blocks
//     per CU: ~57 KB in flight per CU for 56 x 56 planes), enough to cover
//     HBM latency at full bandwidth.
// A zero entry of T times an infinite or NaN input would spread that value
// to outputs whose window does not contain it, so a plane holding any
// non-finite input is computed again, after the block's other planes, by an
// exact direct loop whose stores replace the matrix-core ones.
#include <hip/hip_runtime.h>

#include "epilogue.h"
#include "internal.h"
#include "launch.h"
#include "sync.h"

namespace fc {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunks = 2;          // 16-byte input chunks per lane and plane
constexpr int kMaxQuads = 4;           // 4-output quads of y per lane and plane
constexpr int kMaxLds = 64 * 1024;     // bytes per block
constexpr int kRG = 4;                 // interleaved row tiles per work item
constexpr int kPre = 3;                // planes whose input is in flight per block

// Word 3 of a raw buffer resource on gfx9-class GPUs: 32-bit data format,
// untyped access (offsets past num_records read zero and drop writes).
constexpr int kBufferWord3 = 0x00020000;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned uint4v __attribute__((ext_vector_type(4)));
typedef unsigned uint2v __attribute__((ext_vector_type(2)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));

struct DwMfma {
  int TV, TW;        // work items per plane: 64-row groups, 16-column blocks
  int S;             // input column iw sits at LDS column iw + pw + S, pw + S = 0 mod 8
  int G;             // 8-column groups of a B fragment that hold window columns (3 or 4)
  int NR, pitch;     // LDS input rows, halves per row; row R starts at in_row(R)
  int P;             // stage row pitch in floats; output row R starts at stage_row(R)
  int in_halves;     // halves of the input area
  int woff;          // byte offset of the KH*KW weights
  int toff;          // byte offset of the zero-padded kernel rows (2 x KH x 48 halves)
  int foff;          // byte offset of the non-finite plane flags (one word)
  int lds;           // bytes per block
  int k;             // images per step: block b owns channel b % M and images b / M + i k
  int steps;         // steps per block, ceil(n / k) <= 32
  int xch, yq;       // 16-byte chunks of x, 4-output quads of y per plane
};

bool dwm_try(const ConvParams& cp, DwMfma& f) {
  if (cp.Cg != 1 || !depth_trivial(cp) || cp.sh != 1 || cp.sw != 1) return false;
  if (!(cp.KH == 3 || cp.KH == 5 || cp.KH == 7)) return false;
  if (!(cp.dh == 1 || cp.dh == 2)) return false;
  if (cp.W % 8 != 0 || cp.OW % 8 != 0) return false;
  const int span = 16 + cp.dw * (cp.KW - 1);  // K columns a 16-column tile reads
  if (span > 32) return false;
  f.G = (span + 7) / 8;
  f.S = (8 - cp.pw % 8) % 8;
  f.TW = (cp.OW + f.S + 15) / 16;
  f.TV = (cp.OH + 16 * kRG - 1) / (16 * kRG);
  const int need = 16 * (f.TW - 1) + 8 * f.G;
  f.pitch = (need + 7) / 16 * 16 + 8;
  f.NR = 16 * kRG * f.TV + cp.dh * (cp.KH - 1);
  f.in_halves = f.NR * f.pitch + 8 * ((f.NR + 3) / 4);
  f.P = 16 * f.TW + 8;
  // stage rows for every tile row (64 TV), so tile stores need no row test
  const int64_t stage = ((int64_t)64 * f.TV * f.P + 16 * 4 * f.TV) * 4;
  f.woff = f.in_halves * 2 + (int)((stage + 15) / 16 * 16);
  f.toff = f.woff + (cp.KH * cp.KW * 2 + 15) / 16 * 16;
  f.foff = f.toff + 2 * cp.KH * 48 * 2;
  const int64_t lds = f.foff + 16;
  if (lds > kMaxLds) return false;
  f.lds = (int)lds;
  f.xch = (int)(cp.in_sz / 8);
  f.yq = (int)(cp.out_sz / 4);
  if (f.xch > kMaxChunks * kThreads || f.yq > kMaxQuads * kThreads) return false;
  // Block b owns channel b % M (Toeplitz fragments built once) and walks
  // images b / M, b / M + k, ...: at step i the k*M blocks read the planes
  // i*k*M .. (i+1)*k*M - 1 of the image-major order, one compact window of
  // memory (a grid-wide stream rather than k*M scattered ones).  About 3
  // blocks per CU (k*M ~ 768); at most 32 steps (one bit each in the block's
  // non-finite mask).
  int64_t k = (768 + cp.M / 2) / cp.M;
  if (k < 1) k = 1;
  if (k < (cp.n + 31) / 32) k = (cp.n + 31) / 32;
  if (k > cp.n) k = cp.n;
  if (k * cp.M >= ((int64_t)1 << 31)) return false;
  f.k = (int)k;
  f.steps = (int)((cp.n + k - 1) / k);
  return true;
}

// Bit 15 of a half's slot is set in the result when that half is infinite
// or NaN (exponent all ones): adding 1 to an all-ones 5-bit exponent carries
// into bit 15, and no sum leaves its 16-bit slot.
__device__ __forceinline__ unsigned nonfinite_bits(uint4v v) {
  unsigned t = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) t |= (v[i] & 0x7c007c00u) + 0x04000400u;
  return t & 0x80008000u;
}

// LDS input row R starts at in_row(R) halves: 8 extra halves every 4 rows
// so the 16 rows 4r + s (r = 0..15) that one fragment read touches fall on
// distinct banks (pitch/2 is 4 mod 8 dwords, 4*pitch/2 + 4 is 20 mod 32).
__device__ __forceinline__ int in_row(int r, int pitch) { return r * pitch + 8 * (r >> 2); }
// Stage row R starts at stage_row(R) floats (16 extra floats every 16 rows:
// rows 16 apart, written by the same instruction, land 16 banks apart);
// column ow of the output sits at stage column ow + 8.
__device__ __forceinline__ int stage_row(int r, int P) { return r * P + 16 * (r >> 4); }

template <int KH, int DH, int ACT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8)))
void dwm_kernel(const half_t* __restrict__ x, const half_t* __restrict__ w,
                const half_t* __restrict__ bias, const half_t* z, half_t* y, ConvParams cp,
                DwMfma f) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  half_t* xin = (half_t*)smem;
  float* stage = (float*)(smem + f.in_halves * 2);
  half_t* wl = (half_t*)(smem + f.woff);
  half_t* trow = (half_t*)(smem + f.toff);
  unsigned* flags = (unsigned*)(smem + f.foff);  // bit i: step i's plane has a non-finite input
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = (int)(blockIdx.x % (unsigned)cp.M);
  const int n0 = (int)(blockIdx.x / (unsigned)cp.M);
  const int nimg = (int)cp.n;
  // steps of this block: images n0 + i k for i < nst (steps past nst repeat
  // the last image: same results to the same place)
  const int nst = (nimg - n0 + f.k - 1) / f.k;
  const int nlast = n0 + (nst - 1) * f.k;
  const int cw8 = cp.W / 8, ow4 = cp.OW / 4;

  // Chunk c of a plane: input row c / cw8, columns 8 (c % cw8) .. +7.  Lanes
  // past the last chunk repeat it (same data to the same place), so loads,
  // LDS writes and stores carry no branches: a branch around a memory
  // operation makes the compiler drain every outstanding load at the join.
  int xoff[kMaxChunks], xdst[kMaxChunks];
#pragma unroll
  for (int kk = 0; kk < kMaxChunks; ++kk) {
    const int c = tid + kk * kThreads;
    const int cc = c < f.xch ? c : f.xch - 1;
    const int row = cc / cw8, col = cc - row * cw8;
    xoff[kk] = cc * 8;
    xdst[kk] = in_row(row + cp.ph, f.pitch) + col * 8 + cp.pw + f.S;
  }
  // y quad c (4 outputs: row c / ow4, columns 4 (c % ow4) ..): its element
  // offset in the plane and its stage offset (consecutive lanes read
  // consecutive 16-byte stage words: no bank conflicts)
  int yoff[kMaxQuads], soff[kMaxQuads];
#pragma unroll
  for (int kk = 0; kk < kMaxQuads; ++kk) {
    const int c = tid + kk * kThreads;
    const int cc = c < f.yq ? c : f.yq - 1;
    const int row = cc / ow4;
    yoff[kk] = cc * 4;
    soff[kk] = stage_row(row, f.P) + (cc - row * ow4) * 4 + 8;
  }
  // image n: input plane n * C + m / Mg, output plane n * M + m
  const half_t* xm = x + (int64_t)(m / cp.Mg) * cp.in_sz;
  const int64_t xstride = (int64_t)cp.C * cp.in_sz;
  auto image = [&](int i) { return i < nst ? n0 + i * f.k : nlast; };
  auto load_x = [&](int n, uint4v (&r)[kMaxChunks]) __attribute__((always_inline)) {
    const half_t* xp = xm + (int64_t)n * xstride;
#pragma unroll
    for (int kk = 0; kk < kMaxChunks; ++kk) r[kk] = *(const uint4v*)(xp + xoff[kk]);
  };
  // The input of the next kPre planes is in flight in registers (rotating
  // sets), which keeps enough bytes in flight per CU to cover HBM latency.
  uint4v xs[kPre][kMaxChunks];
#pragma unroll
  for (int i = 0; i < kPre; ++i) load_x(image(i), xs[i]);

  // zero the input plane once: its border stays zero for every plane;
  // weights and bias of channel m
  for (int i = tid; i < f.in_halves / 8; i += kThreads) ((uint4v*)xin)[i] = uint4v{0, 0, 0, 0};
  for (int i = tid; i < KH * cp.KW; i += kThreads) wl[i] = w[(int64_t)m * KH * cp.KW + i];
  if (tid == 0) *flags = 0;
  const float bv = cp.has_bias ? to_f32(bias[m]) : 0.0f;
  lds_barrier();
  // zero-padded kernel rows: trow[c][kh][i] = T entry for offset d = i + c - 16
  // (k - j = d), i.e. w[kh][d / dw] when d = dw*kw, 0 <= kw < KW, else 0;
  // copy c = 1 is copy 0 shifted by one half, so every 8-half window starts
  // on a dword in one of the two copies
  for (int idx = tid; idx < 2 * KH * 48; idx += kThreads) {
    const int c = idx / (KH * 48), r = idx - c * KH * 48;
    const int kh = r / 48, d = r - kh * 48 + c - 16;
    half_t v = (half_t)0;
    if (d >= 0) {
      const int kw = d / cp.dw;
      if (kw * cp.dw == d && kw < cp.KW) v = wl[kh * cp.KW + kw];
    }
    trow[idx] = v;
  }
  lds_barrier();

  // Residual of a plane.  A buffer load whose range is empty when there is no
  // residual: the hardware returns zeros without touching memory, with no
  // branch around the load.
  auto load_z = [&](int64_t ybase, uint2v (&zr)[kMaxQuads]) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t zb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(cp.has_z ? z + ybase : x), (short)0, cp.has_z ? (int)(cp.out_sz * 2) : 0,
        kBufferWord3);
#pragma unroll
    for (int kk = 0; kk < kMaxQuads; ++kk)
      zr[kk] = __builtin_bit_cast(uint2v, __builtin_amdgcn_raw_buffer_load_b64(zb, yoff[kk] * 2, 0, 0));
  };
  // bias, residual, activation over the staged plane; 8-byte stores of y
  // (the plane is contiguous: quad c covers y[4c .. 4c+3])
  auto store_plane = [&](int64_t ybase, const uint2v (&zr)[kMaxQuads])
      __attribute__((always_inline)) {
    lds_barrier();
    half_t* yp = y + ybase;
#pragma unroll
    for (int kk = 0; kk < kMaxQuads; ++kk) {
      const float4v s0 = *(const float4v*)(stage + soff[kk]);
      const half4 zh = __builtin_bit_cast(half4, zr[kk]);
      act4_t v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = s0[i] + bv;
      if (cp.has_z) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] += (float)zh[i];
      }
      v = act4<ACT>(v, cp.alpha, cp.beta);
      half4 out;
#pragma unroll
      for (int i = 0; i < 4; ++i) out[i] = (half_t)v[i];
      *(half4*)(yp + yoff[kk]) = out;
    }
  };

  {
    const int j16 = lane & 15, q = lane >> 4;
    // Toeplitz fragments (the B operand): lane holds T_kh[j][8q .. 8q+7],
    // j = lane % 16 the output column of the tile: the 8 halves from
    // i = 16 + 8q - j of the zero-padded row
    half8 tfrag[KH];
    {
      const int i0 = 16 + 8 * q - j16;
      const unsigned* tp = (const unsigned*)(trow + (i0 & 1) * KH * 48) + (i0 >> 1);
#pragma unroll
      for (int kh = 0; kh < KH; ++kh)
        tfrag[kh] = __builtin_bit_cast(
            half8, uint4v{tp[kh * 24], tp[kh * 24 + 1], tp[kh * 24 + 2], tp[kh * 24 + 3]});
    }
    // input fragments (the A operand): lane reads LDS row 64v + 4 r + s
    // (r = lane % 16), columns 16t + 8q .. +7.  Lanes with q >= G meet only
    // zero Toeplitz entries; they read in-bounds LDS input (zero or input
    // values, finite once the plane passed the non-finite test), so their
    // products are exact zeros.
    const int brow = (in_row(4 * j16, f.pitch) + 8 * q) * 2;  // bytes
    const int bstep = f.pitch * 2;                              // bytes per input row
    const int nitem = f.TV * f.TW;

    // step i: image image(i); xr holds its input and receives the input
    // kPre steps ahead
    auto step = [&](int i, uint4v (&xr)[kMaxChunks]) __attribute__((always_inline)) {
      // this plane's input into LDS; flag non-finite values
      unsigned bad = 0;
#pragma unroll
      for (int kk = 0; kk < kMaxChunks; ++kk) {
        *(uint4v*)(xin + xdst[kk]) = xr[kk];
        bad |= nonfinite_bits(xr[kk]);
      }
      const int ir = i < nst ? i : nst - 1;
      if (__builtin_amdgcn_ballot_w64(bad != 0) != 0) atomicOr(flags, 1u << (unsigned)ir);
      const int64_t ybase = ((int64_t)image(i) * cp.M + m) * cp.out_sz;
      uint2v zr[kMaxQuads];
      load_z(ybase, zr);
      lds_barrier();
      // the input kPre steps ahead into the registers just written out
      load_x(image(i + kPre), xr);
      // the plane into the fp32 stage
      for (int it = wave; it < nitem; it += 4) {
        const int v = it / f.TW, t = it - v * f.TW;
        const unsigned char* bp =
            (const unsigned char*)(xin + in_row(64 * v, f.pitch) + 16 * t) + brow;
        float4v acc[kRG];
#pragma unroll
        for (int p = 0; p < kRG; ++p) acc[p] = float4v{0, 0, 0, 0};
#pragma unroll
        for (int s = 0; s < kRG + DH * (KH - 1); ++s) {
          const half8 b = *(const half8*)(bp + s * bstep + 16 * (s >> 2));
#pragma unroll
          for (int kh = 0; kh < KH; ++kh) {
            const int p = s - DH * kh;
            if (p >= 0 && p < kRG)
              acc[p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b, tfrag[kh], acc[p], 0, 0, 0);
          }
          // keep only a few fragments in flight (registers for the prefetch)
          if (s % 3 == 2) __builtin_amdgcn_sched_barrier(0);
        }
        // at least 32 wait states between the last MFMA and the first read of
        // its result (the compiler's count was measured too low on gfx950 for
        // v_mfma_f32_16x16x32_f16 results read soon after)
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 15\n\ts_nop 15" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        // lane holds D[4q + i][j16] of tile p: output row 64v + 4 (4q + i) + p,
        // column 16t - S + j16 (stage column 16t - S + j16 + 8; rows past OH
        // and columns outside the image land in stage rows and margins that
        // are never read)
        float* sq = stage + stage_row(64 * v + 16 * q, f.P) + 16 * t - f.S + j16 + 8;
#pragma unroll
        for (int p = 0; p < kRG; ++p)
#pragma unroll
          for (int e = 0; e < 4; ++e) sq[(4 * e + p) * f.P] = acc[p][e];
      }
      store_plane(ybase, zr);
    };

    for (int i = 0; i < nst; i += kPre) {
#pragma unroll
      for (int u = 0; u < kPre; ++u) step(i + u, xs[u]);
    }
  }

  // Planes with a non-finite input again, by the exact direct loop (only the
  // window's products enter each sum); their stores replace the ones above.
  lds_barrier();
  unsigned badmask = __builtin_amdgcn_readfirstlane(*flags);
  while (badmask != 0) {
    const int i = __builtin_ctz(badmask);
    badmask &= badmask - 1;
    const int n = image(i);
    lds_barrier();  // every lane is done with the stage and the input
    uint4v xr[kMaxChunks];
    load_x(n, xr);
#pragma unroll
    for (int kk = 0; kk < kMaxChunks; ++kk) *(uint4v*)(xin + xdst[kk]) = xr[kk];
    lds_barrier();
    for (int idx = tid; idx < cp.OH * cp.OW; idx += kThreads) {
      const int oh = idx / cp.OW, ow = idx - oh * cp.OW;
      float sum = 0.0f;
      for (int kh = 0; kh < KH; ++kh)
        for (int kw = 0; kw < cp.KW; ++kw)
          sum += (float)xin[in_row(oh + cp.dh * kh, f.pitch) + ow + cp.dw * kw + f.S] *
                 (float)wl[kh * cp.KW + kw];
      stage[stage_row(oh, f.P) + ow + 8] = sum;
    }
    const int64_t ybase = ((int64_t)n * cp.M + m) * cp.out_sz;
    uint2v zr[kMaxQuads];
    load_z(ybase, zr);
    store_plane(ybase, zr);
  }
}

template <int KH, int DH>
int launch_kh(const Geometry& g, const DwMfma& f, const RunArgs& a) {
  const ConvParams& cp = g.cp;
  return launch_conv(dwm_kernel<KH, DH, FC_ACT>, dim3((unsigned)(f.k * cp.M)), dim3(kThreads),
                     (size_t)f.lds, a, kEdgeBoth, (const half_t*)a.x, (const half_t*)a.w,
                     (const half_t*)a.bias, (const half_t*)a.z, (half_t*)a.y, cp, f);
}

}  // namespace

#ifndef FC_ACT
#error "compiled once per activation id: -DFC_ACT=<0..ACT_COUNT-1>"
#endif

int FC_CAT(launch_dwm_act_, FC_ACT)(const Geometry& g, const RunArgs& a) {
  DwMfma f;
  if (g.dtype != FUSEDCONV_F16 || !dwm_try(g.cp, f)) return FUSEDCONV_ERR_ROUTE;
  const int key = g.cp.KH * 4 + g.cp.dh;
  switch (key) {
    case 3 * 4 + 1: return launch_kh<3, 1>(g, f, a);
    case 3 * 4 + 2: return launch_kh<3, 2>(g, f, a);
    case 5 * 4 + 1: return launch_kh<5, 1>(g, f, a);
    case 5 * 4 + 2: return launch_kh<5, 2>(g, f, a);
    case 7 * 4 + 1: return launch_kh<7, 1>(g, f, a);
    case 7 * 4 + 2: return launch_kh<7, 2>(g, f, a);
    default: return FUSEDCONV_ERR_ROUTE;
  }
}

#if FC_ACT == 0
FC_ACT_DECLS(launch_dwm_act_)

bool depthwise_mfma_fits(const ConvParams& cp, int32_t dtype) {
  DwMfma f;
  return dtype == FUSEDCONV_F16 && dwm_try(cp, f);
}

int launch_depthwise_mfma(const Geometry& g, const RunArgs& a) {
  static const ActLaunchFn table[ACT_COUNT] = FC_ACT_TABLE(launch_dwm_act_);
  return table[g.cp.act](g, a);
}
#endif

}  // namespace fc
