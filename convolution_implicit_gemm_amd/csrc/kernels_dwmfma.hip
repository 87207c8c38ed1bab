// Depthwise convolution (one input channel per group, stride 1, 2 spatial
// dims, fp16) on the matrix cores.
//
// A depthwise output row is a 1-D correlation of input rows with the kernel
// rows: y[oh][ow] = sum_kh sum_kw x[oh + dh*kh][ow + dw*kw] w[kh][kw] (padded
// coordinates).  For one kernel row kh and a block of 16 output columns this
// is a product with a banded (Toeplitz) matrix: with the 16 output columns as
// the M side, the input columns of the window as the K side and 16 output
// rows as the N side,
//     D[j][r] += sum_k  T_kh[j][k] * X[oh0 + r + dh*kh][ow0 + k - S],
//     T_kh[j][k] = w[kh][(k - j - S) / dw]   when k - j - S = dw*kw, 0 <= kw < KW,
// so one v_mfma_f32_16x16x32_f16 per kernel row covers a 16x16 output tile
// when S + 16 + dw*(KW-1) <= 32 (S < 8 is the column shift that aligns the
// window, below).  Only KW of the 32 products per output are non-zero, but
// the matrix cores run ~16x the packed-fp16 VALU rate, which leaves the
// kernel bound by memory rather than by issue (the VALU form needs ~28
// v_dot2 per output of a 7x7 kernel).  Products are exact in fp32 and the
// sums are fp32, seeded by the bias, as in the FusedConv manifest's
// grouped-kernel variants (fp32 accumulation).
//
// Layout on gfx950:
//   * block b owns channel b % M and walks every k-th image, so the k*M
//     blocks read one compact window of memory at a time; its Toeplitz
//     fragments (KH x 8 halves per lane, from an LDS table of zero-padded
//     kernel rows) are built once;
//   * input planes go through two LDS buffers: while the waves compute plane
//     i from one, they write plane i+1 (its input loaded kPre planes ahead
//     into registers) into the other, so a plane costs one barrier.  Rows sit
//     at a column shift S that puts input column 0 on an 8-column boundary,
//     so every input fragment is one aligned ds_read_b128; the zero border
//     (the padding) is written once and never overwritten;
//   * a wave's work item is 4 interleaved 16 x 16 tiles: output rows
//     64v + 4r + p (p = 0..3) for the 16 columns 16t .. 16t+15.  Tile p at
//     kernel row kh reads input rows 64v + 4r + p + dh*kh, so the 4*KH
//     products of the item need only 4 + dh*(KH-1) distinct input fragments
//     (10 instead of 28 for a 7x7 kernel);
//   * the Toeplitz matrix is the A operand, so a lane's 4 accumulators are 4
//     consecutive output columns of one output row: bias (the accumulator's
//     start), residual and activation run on them in registers, and the 4
//     fp16 results go to an LDS stage as one 8-byte write;
//   * the stage is double-buffered too: while plane i is computed into one,
//     plane i-1 leaves the other as 16-byte pieces of 8 consecutive outputs,
//     consecutive lanes on consecutive pieces (whole-line global stores).
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
constexpr int kMaxLds = 80 * 1024;     // bytes per block (at least two blocks per CU)
constexpr int kRG = 4;                 // interleaved row tiles per work item
constexpr int kPre = 3;                // planes whose input is in flight per block
constexpr int kTrow = 64;              // halves per zero-padded kernel row
constexpr int kTbase = 24;             // index of offset 0 in a zero-padded kernel row

// Word 3 of a raw buffer resource on gfx9-class GPUs: 32-bit data format,
// untyped access (offsets past num_records read zero and drop writes).
constexpr int kBufferWord3 = 0x00020000;
constexpr unsigned kOff = 0x80000000u;  // an offset past every record

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef unsigned uint4v __attribute__((ext_vector_type(4)));
typedef unsigned uint2v __attribute__((ext_vector_type(2)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));

struct DwMfma {
  int TV, TW;        // work items per plane: 64-row groups, 16-column blocks
  int S;             // input column iw sits at LDS column iw + pw + S, pw + S = 0 mod 8
  int NR, pitch;     // LDS input rows, halves per row; row R starts at in_row(R)
  int bufh;          // halves per input buffer (two of them)
  int sp;            // halves per stage row; stage row R starts at in_row(R, sp)
  int stgh;          // halves per stage buffer (two of them, after the input buffers)
  int no;            // 8-output pieces of a plane
  int woff;          // byte offset of the KH*KW weights
  int toff;          // byte offset of the zero-padded kernel rows (2 x KH x kTrow halves)
  int foff;          // byte offset of the non-finite plane flags (one word)
  int lds;           // bytes per block
  int k;             // images per step: block b owns channel b % M and images b / M + i k
  int steps;         // steps per block, ceil(n / k) <= 32
  int xch;           // 16-byte chunks of x per plane
};

bool dwm_try(const ConvParams& cp, DwMfma& f) {
  if (cp.Cg != 1 || !depth_trivial(cp) || cp.sh != 1 || cp.sw != 1) return false;
  if (!(cp.KH == 3 || cp.KH == 5 || cp.KH == 7)) return false;
  if (!(cp.dh == 1 || cp.dh == 2)) return false;
  if (cp.W % 8 != 0 || cp.OW % 8 != 0) return false;
  f.S = (8 - cp.pw % 8) % 8;
  // window slots a 16-column tile reads, counted from its aligned first slot
  if (f.S + 16 + cp.dw * (cp.KW - 1) > 32) return false;
  f.TW = (cp.OW + 15) / 16;
  f.TV = (cp.OH + 16 * kRG - 1) / (16 * kRG);
  // a fragment read covers 32 halves from column 16t; + 8 halves so that
  // rows 4 apart start on different banks (pitch = 8 mod 16)
  f.pitch = 16 * (f.TW - 1) + 32 + 8;
  if (cp.W + cp.pw + f.S > f.pitch - 8) return false;  // the input row fits
  f.NR = 16 * kRG * f.TV + cp.dh * (cp.KH - 1);
  f.bufh = (f.NR * f.pitch + 8 * ((f.NR + 3) / 4) + 7) / 8 * 8;
  // stage rows for every tile row (64 TV), 16 TW columns; pitch = 8 mod 16 and
  // the 8-half skew every 4 rows keep the 16-byte reads aligned and spread the
  // 8-byte writes of one instruction (rows 4r + p) over distinct banks
  f.sp = 16 * f.TW + 8;
  f.stgh = 64 * f.TV * f.sp + 8 * 16 * f.TV;
  f.no = (int)(cp.out_sz / 8);
  if (f.no > 2 * kThreads) return false;
  f.woff = 2 * f.bufh * 2 + 2 * f.stgh * 2;
  f.toff = f.woff + (cp.KH * cp.KW * 2 + 15) / 16 * 16;
  f.foff = f.toff + 2 * cp.KH * kTrow * 2;
  const int64_t lds = f.foff + 16;
  if (lds > kMaxLds) return false;
  f.lds = (int)lds;
  f.xch = (int)(cp.in_sz / 8);
  if (f.xch > kMaxChunks * kThreads) return false;
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

// LDS input (and stage) row R starts at in_row(R) halves: 8 extra halves
// every 4 rows so the 16 rows 4r + s (r = 0..15) that one fragment read (or
// stage write) touches fall on distinct banks (pitch/2 is 4 mod 8 dwords).
__device__ __forceinline__ int in_row(int r, int pitch) { return r * pitch + 8 * (r >> 2); }

template <int KH, int DH, int ACT, bool HZ>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8)))
void dwm_kernel(const half_t* __restrict__ x, const half_t* __restrict__ w,
                const half_t* __restrict__ bias, const half_t* z, half_t* y, ConvParams cp,
                DwMfma f) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  half_t* xin = (half_t*)smem;  // two input buffers of f.bufh halves
  half_t* stage = xin + 2 * f.bufh;  // two stage buffers of f.stgh halves
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
  const int cw8 = cp.W / 8;

  // Chunk c of a plane: input row c / cw8, columns 8 (c % cw8) .. +7.  Lanes
  // past the last chunk repeat it (same data to the same place), so loads and
  // LDS writes carry no branches: a branch around a memory operation makes
  // the compiler drain every outstanding load at the join.
  int xoff[kMaxChunks], xdst[kMaxChunks];
#pragma unroll
  for (int kk = 0; kk < kMaxChunks; ++kk) {
    const int c = tid + kk * kThreads;
    const int cc = c < f.xch ? c : f.xch - 1;
    const int row = cc / cw8, col = cc - row * cw8;
    xoff[kk] = cc * 8;
    xdst[kk] = in_row(row + cp.ph, f.pitch) + col * 8 + cp.pw + f.S;
  }
  // Piece o of a plane (8 outputs: row o / (OW/8), columns 8 (o % (OW/8)) ..):
  // its stage offset and its byte offset in the output plane (past the
  // records for lanes without a piece: the store is dropped)
  int sof[2];
  unsigned gof[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    const int o = tid + kk * kThreads;
    const int oc = o < f.no ? o : f.no - 1;
    const int row = oc / (cp.OW / 8), col = oc - row * (cp.OW / 8);
    sof[kk] = in_row(row, f.sp) + col * 8;
    gof[kk] = o < f.no ? (unsigned)(oc * 16) : kOff;
  }
  // image n: input plane n * C + m / Mg, output plane n * M + m
  const half_t* xm = x + (int64_t)(m / cp.Mg) * cp.in_sz;
  const int64_t xstride = (int64_t)cp.C * cp.in_sz;
  auto image = [&](int i) { return i < nst ? n0 + i * f.k : nlast; };
  auto load_x = [&](int n, uint4v (&r)[kMaxChunks]) __attribute__((always_inline)) {
    const half_t* xp = xm + (int64_t)n * xstride;
#pragma unroll
    // streamed once: nontemporal (X is not read again by this launch)
    for (int kk = 0; kk < kMaxChunks; ++kk) r[kk] = __builtin_nontemporal_load((const uint4v*)(xp + xoff[kk]));
  };
  // The input of the next kPre planes is in flight in registers (rotating
  // sets: set s holds the planes i = s mod kPre), which keeps enough bytes in
  // flight per CU to cover HBM latency.
  uint4v xs[kPre][kMaxChunks];
#pragma unroll
  for (int i = 0; i < kPre; ++i) load_x(image(i), xs[i]);

  // zero both input buffers once: their borders stay zero for every plane;
  // weights and bias of channel m
  for (int i = tid; i < 2 * f.bufh / 8; i += kThreads) ((uint4v*)xin)[i] = uint4v{0, 0, 0, 0};
  for (int i = tid; i < KH * cp.KW; i += kThreads) wl[i] = w[(int64_t)m * KH * cp.KW + i];
  if (tid == 0) *flags = 0;
  const float bv = cp.has_bias ? to_f32(bias[m]) : 0.0f;
  lds_barrier();
  // zero-padded kernel rows: trow[c][kh][i] = T entry for offset
  // d = i + c - kTbase (d = k - j - S), i.e. w[kh][d / dw] when d = dw*kw,
  // 0 <= kw < KW, else 0; copy c = 1 is copy 0 shifted by one half, so every
  // 8-half window starts on a dword in one of the two copies
  for (int idx = tid; idx < 2 * KH * kTrow; idx += kThreads) {
    const int c = idx / (KH * kTrow), r = idx - c * KH * kTrow;
    const int kh = r / kTrow, d = r - kh * kTrow + c - kTbase;
    half_t v = (half_t)0;
    if (d >= 0) {
      const int kw = d / cp.dw;
      if (kw * cp.dw == d && kw < cp.KW) v = wl[kh * cp.KW + kw];
    }
    trow[idx] = v;
  }

  // a plane's input into buffer b; non-finite values set the plane's flag
  auto put_plane = [&](int i, int b, const uint4v (&xr)[kMaxChunks]) __attribute__((always_inline)) {
    half_t* xb = xin + b * f.bufh;
    unsigned bad = 0;
#pragma unroll
    for (int kk = 0; kk < kMaxChunks; ++kk) {
      *(uint4v*)(xb + xdst[kk]) = xr[kk];
      bad |= nonfinite_bits(xr[kk]);
    }
    const int ir = i < nst ? i : nst - 1;
    if (__builtin_amdgcn_ballot_w64(bad != 0) != 0) atomicOr(flags, 1u << (unsigned)ir);
  };
  put_plane(0, 0, xs[0]);
  load_x(image(kPre), xs[0]);
  lds_barrier();

  {
    const int j16 = lane & 15, q = lane >> 4;
    // Toeplitz fragments (the A operand): lane holds T_kh[j][8q .. 8q+7],
    // j = lane % 16 the output column of the tile: the 8 halves from
    // i = kTbase + 8q - j - S of the zero-padded row
    half8 tfrag[KH];
    {
      const int i0 = kTbase + 8 * q - j16 - f.S;
      const unsigned* tp = (const unsigned*)(trow + (i0 & 1) * KH * kTrow) + (i0 >> 1);
#pragma unroll
      for (int kh = 0; kh < KH; ++kh)
        tfrag[kh] = __builtin_bit_cast(
            half8, uint4v{tp[kh * (kTrow / 2)], tp[kh * (kTrow / 2) + 1], tp[kh * (kTrow / 2) + 2],
                          tp[kh * (kTrow / 2) + 3]});
    }
    // input fragments (the B operand): lane reads LDS row 64v + 4 r + s
    // (r = lane % 16), columns 16t + 8q .. +7; every read stays inside the
    // plane's own buffer, so lanes whose Toeplitz entries are zero multiply
    // finite values (zero border or inputs of a plane that passed the
    // non-finite test) and add exact zeros.
    const int brow = (in_row(4 * j16, f.pitch) + 8 * q) * 2;  // bytes
    const int bstep = f.pitch * 2;                              // bytes per input row
    const int nitem = f.TV * f.TW;

    // plane i's outputs from stage buffer i & 1 to Y
    auto store_out = [&](int i) __attribute__((always_inline)) {
      const int64_t ybase = ((int64_t)image(i) * cp.M + m) * cp.out_sz;
      const __amdgpu_buffer_rsrc_t yb =
          __builtin_amdgcn_make_buffer_rsrc((void*)(y + ybase), (short)0, 0x7fffffff, kBufferWord3);
      const half_t* sb = stage + (i & 1) * f.stgh;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        // cache policy 2 = nt: Y is streamed out, not re-read (measured 3-5 us faster)
        __builtin_amdgcn_raw_buffer_store_b128(*(const uint4v*)(sb + sof[kk]), yb, gof[kk], 0, 2);
    };

    // plane i's outputs; the input kPre planes past plane i+1 is loaded into
    // xr (which held plane i+1's input) before (no residual) or after (with
    // one, whose loads then wait only for older prefetches) the products
    auto step = [&](int i, uint4v (&xr)[kMaxChunks], bool prev) __attribute__((always_inline)) {
      put_plane(i + 1, (i + 1) & 1, xr);
      if constexpr (!HZ) load_x(image(i + 1 + kPre), xr);
      if (prev) store_out(i - 1);
      const int64_t ybase = ((int64_t)image(i) * cp.M + m) * cp.out_sz;
      half_t* sb = stage + (i & 1) * f.stgh;
      const unsigned char* xb = (const unsigned char*)(xin + (i & 1) * f.bufh);
      for (int it = wave; it < nitem; it += 4) {
        const int v = it / f.TW, t = it - v * f.TW;
        // lane's outputs: columns 16t + 4q .. +3 (OW % 4 == 0: all in or
        // all out) of rows 64v + 4 j16 + p
        const int oc = 16 * t + 4 * q;
        uint2v zr[kRG];
        if constexpr (HZ) {
          unsigned off[kRG];
#pragma unroll
          for (int p = 0; p < kRG; ++p) {
            const int r = 64 * v + 4 * j16 + p;
            off[p] = (oc < cp.OW && r < cp.OH) ? (unsigned)((r * cp.OW + oc) * 2) : kOff;
          }
          const __amdgpu_buffer_rsrc_t zb = __builtin_amdgcn_make_buffer_rsrc(
              (void*)(z + ybase), (short)0, 0x7fffffff, kBufferWord3);
#pragma unroll
          for (int p = 0; p < kRG; ++p)
            zr[p] = __builtin_bit_cast(uint2v, __builtin_amdgcn_raw_buffer_load_b64(zb, off[p], 0, 0));
        }
        const unsigned char* bp = xb + (in_row(64 * v, f.pitch) + 16 * t) * 2 + brow;
        float4v acc[kRG];
#pragma unroll
        for (int p = 0; p < kRG; ++p) acc[p] = float4v{bv, bv, bv, bv};
#pragma unroll
        for (int s = 0; s < kRG + DH * (KH - 1); ++s) {
          const half8 b = *(const half8*)(bp + s * bstep + 16 * (s >> 2));
#pragma unroll
          for (int kh = 0; kh < KH; ++kh) {
            const int p = s - DH * kh;
            if (p >= 0 && p < kRG)
              acc[p] = __builtin_amdgcn_mfma_f32_16x16x32_f16(tfrag[kh], b, acc[p], 0, 0, 0);
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
#pragma unroll
        for (int p = 0; p < kRG; ++p) {
          act4_t val;
#pragma unroll
          for (int e = 0; e < 4; ++e) val[e] = acc[p][e];
          if constexpr (HZ) {
            const half4 zh = __builtin_bit_cast(half4, zr[p]);
#pragma unroll
            for (int e = 0; e < 4; ++e) val[e] += (float)zh[e];
          }
          val = act4<ACT>(val, cp.alpha, cp.beta);
          half4 out;
#pragma unroll
          for (int e = 0; e < 4; ++e) out[e] = (half_t)val[e];
          *(half4*)(sb + in_row(64 * v + 4 * j16 + p, f.sp) + oc) = out;
        }
      }
      if constexpr (HZ) load_x(image(i + 1 + kPre), xr);
      // plane i + 1 is in its buffer; every wave is done with plane i's
      lds_barrier();
    };

    // The first kPre steps apart from the loop: entering the loop, the loads
    // in flight are then the ones of a loop iteration, and the compiler's wait
    // counts at the loop head are those of the steady state.
#pragma unroll
    for (int u = 0; u < kPre; ++u) step(u, xs[(u + 1) % kPre], u > 0);
    int i = kPre;
    for (; i < nst; i += kPre) {
#pragma unroll
      for (int u = 0; u < kPre; ++u) step(i + u, xs[(u + 1) % kPre], true);
    }
    store_out(i - 1);
  }

  // Planes with a non-finite input again, by the exact direct loop (only the
  // window's products enter each sum); their stores replace the ones above,
  // which the barrier's release fence has completed.
  __syncthreads();
  unsigned badmask = __builtin_amdgcn_readfirstlane(*flags);
  while (badmask != 0) {
    const int i = __builtin_ctz(badmask);
    badmask &= badmask - 1;
    const int n = image(i);
    uint4v xr[kMaxChunks];
    load_x(n, xr);
#pragma unroll
    for (int kk = 0; kk < kMaxChunks; ++kk) *(uint4v*)(xin + xdst[kk]) = xr[kk];
    lds_barrier();
    const int64_t ybase = ((int64_t)n * cp.M + m) * cp.out_sz;
    for (int idx = tid; idx < cp.OH * cp.OW; idx += kThreads) {
      const int oh = idx / cp.OW, ow = idx - oh * cp.OW;
      float sum = bv;
      for (int kh = 0; kh < KH; ++kh)
        for (int kw = 0; kw < cp.KW; ++kw)
          sum += (float)xin[in_row(oh + cp.dh * kh, f.pitch) + ow + cp.dw * kw + f.S] *
                 (float)wl[kh * cp.KW + kw];
      if constexpr (HZ) sum += to_f32(z[ybase + idx]);
      y[ybase + idx] = (half_t)act_t<ACT>(sum, cp.alpha, cp.beta);
    }
    lds_barrier();  // every lane is done with the buffer
  }
}

template <int KH, int DH, bool HZ>
int launch_one(const Geometry& g, const DwMfma& f, const RunArgs& a) {
  const ConvParams& cp = g.cp;
  return launch_conv(dwm_kernel<KH, DH, FC_ACT, HZ>, dim3((unsigned)(f.k * cp.M)),
                     dim3(kThreads), (size_t)f.lds, a, kEdgeBoth, (const half_t*)a.x,
                     (const half_t*)a.w, (const half_t*)a.bias, (const half_t*)a.z, (half_t*)a.y,
                     cp, f);
}

template <int KH, int DH>
int launch_kh(const Geometry& g, const DwMfma& f, const RunArgs& a) {
  if (g.cp.has_z) return launch_one<KH, DH, true>(g, f, a);
  return launch_one<KH, DH, false>(g, f, a);
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
