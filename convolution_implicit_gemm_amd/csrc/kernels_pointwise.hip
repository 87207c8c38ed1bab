// 1x1 convolution (stride 1, no padding) as a batched GEMM on MFMA (fp16 in,
// fp32 accumulate): Y[n][g*Mg + m][p] = sum_c W[g*Mg + m][c] * X[n][g*Cg + c][p]
// for every pixel p of the flattened spatial extent -- the implicit GEMM of
// the FusedConv README with a single tap, where im2col is the identity and X
// itself is the [C/group x pixels] operand.
//
// GEMM view per block: rows = 128 pixels of one image, columns = 64*NWM
// output channels of one group (128, or 256 when M/group > 128: X is then
// streamed once per pixel tile), reduction over the group's input channels in
// steps of 64.  NCHW stores pixels, not channels, consecutively, while the MFMA
// operand of a lane is 8 consecutive reduction elements, so X is transposed
// on its way into LDS:
//   * two producer waves stream X: a thread loads 4 channels x 8 pixels
//     (four 16-byte loads) per item, keeps three steps of loads in flight in
//     registers and writes each item as eight 8-byte pieces of channel-last
//     LDS rows [pixel][64 channels + 16 pad].  The 16 lanes of a load pass
//     cover 2 channel quads x 8 pixel octets, i.e. whole 128-byte pieces of
//     2 channel rows (a pass over 16 channel rows touches 8 times as many
//     cache lines, and measured 1.3x slower); so that those lanes' transposed
//     writes do not collide in the
//     LDS banks, the 16-byte columns of a row are XOR-swizzled by the row's
//     pixel octet (the operand reads apply the same swizzle and stay
//     conflict free on the 160-byte rows).  A wave's memory counter
//     completes in issue order, so a wave that waited for a weight load
//     issued after long X loads would wait for those too; with the roles
//     split, the producers wait only for X and the MFMA waves only for W;
//   * 2*NWM MFMA waves read the weights, one step ahead, from a copy of W
//     repacked in fragment order (fusedconv_prepare_weights, or at the start
//     of every run): each 16-byte lane piece of an operand is contiguous
//     with its neighbours', zero past C/group and M/group, as register
//     operands: v_mfma_f32_16x16x32_f16 with pixels as rows and
//     output channels as columns, each lane ending with 4 consecutive pixels
//     of one output channel.  One barrier per step hands the two LDS stages
//     between the roles;
//   * the epilogue (bias seeds the accumulators; Z, activation, one rounding)
//     goes through LDS one 16-channel block at a time, so every store writes
//     whole rows of 64 consecutive pixels.
// The same kernel runs 2x2 convolutions with stride 2 and no padding (patch
// embeddings, downsampling): ordered as k = c*4 + kh*2 + kw (W's own memory
// order), the reduction's 4 consecutive elements of one producer item are the
// 4 taps of one input channel, and its 8 output pixels read 16 consecutive
// columns of 2 input rows (two 32-byte pieces per row), split into even (kw 0)
// and odd (kw 1) columns -- the same number of loads as a 1x1 item.
// A third form runs transposed 2x2 convolutions with stride 2 (no pads, the
// output exactly twice the input, e.g. decoder upsampling): output pixel
// (2i + a, 2j + b) of channel m is sum_c W[c][m][a][b] * X[c][i][j], so the
// input pixels are the GEMM rows, the reduction is over the input channels
// (the 1x1 producer as is) and the columns are (m, a, b) = 4m + 2a + b, W's
// own memory order along a row of W.  The epilogue pairs the columns b = 0
// and b = 1 of two neighbouring pixels: each lane stores 4 consecutive
// outputs of one output row.
// Every load is unconditional (invalid X pieces read a valid address and are
// written as zeros; the repacked weights are zero-padded), so the compiler can
// count the loads in flight exactly.
#include <hip/hip_runtime.h>

#include "epilogue.h"
#include "internal.h"
#include "launch.h"
#include "sync.h"

namespace fc {
namespace {

constexpr int kBN = 128;    // pixels per block
constexpr int kBK = 64;     // reduction elements per step (input channels for a 1x1)
constexpr int kLDC = kBK + 16;  // LDS row pitch in halves (160 bytes)
constexpr int kStage = kBN * kLDC;  // halves per LDS stage
constexpr size_t kLds = 2 * kStage * sizeof(half_t);
// word 3 of a raw buffer resource on gfx9-class GPUs (32-bit data format):
// offsets past num_records read zero and drop writes
constexpr int kBufferWord3 = 0x00020000;
constexpr unsigned kOff = 0x80000000u;  // an offset past every range set up here

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef unsigned uint2v __attribute__((ext_vector_type(2)));

struct PwTile {
  int64_t P;       // output pixels per image (flattened spatial extent)
  int kp;          // reduction length per group: C/group * taps (taps 1 or 4)
  int ntile;       // pixel tiles per image
  int nmb;         // output-channel blocks per group
  int ks;          // reduction steps: ceil(kp / 64)
  int nwm;         // MFMA waves along the output channels: 2 (128 per block) or 4 (256)
  int64_t tiles;   // G * n * ntile
  int wt;          // 1: W stored as [C][M/group * 4] (the transposed form)
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Weights in fragment order: Wf[((((g*nmb + mb)*ks + s)*2 + kk)*4 + j)*nwm + wmi]
// [lane][e] = W[g*Mg + m][k] (W as [M][C/group * taps], its memory order) with
// m = mb*64*nwm + wmi*64 + j*16 + lane%16 and k = s*64 + kk*32 + (lane/16)*8 + e;
// zero for m >= M/group or k >= C/group * taps.  The transposed form passes
// M/group * 4 as M/group and reads W[g*Cg + k][m] instead.
constexpr int kFragPerWave = 2 * 4 * 64 * 8;  // halves per (group, m block, step, wave)
__global__ __launch_bounds__(256) void repack_frag_kernel(const half_t* __restrict__ w,
                                                          half_t* __restrict__ wf, ConvParams cp,
                                                          PwTile pt) {
  const int64_t total = (int64_t)cp.G * pt.nmb * pt.ks * kFragPerWave * pt.nwm;
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
    const int e = (int)(i & 7);
    const int lane = (int)((i >> 3) & 63);
    int64_t t = i >> 9;
    const int wmi = (int)(t % pt.nwm);
    t /= pt.nwm;
    const int j = (int)(t & 3);
    t >>= 2;
    const int kk = (int)(t & 1);
    t >>= 1;
    const int s = (int)(t % pt.ks);
    t /= pt.ks;
    const int mb = (int)(t % pt.nmb);
    const int g = (int)(t / pt.nmb);
    const int m = mb * 64 * pt.nwm + wmi * 64 + j * 16 + (lane & 15);
    const int c = s * kBK + kk * 32 + (lane >> 4) * 8 + e;
    const int64_t src = pt.wt ? ((int64_t)g * pt.kp + c) * cp.Mg + m : ((int64_t)g * cp.Mg + m) * pt.kp + c;
    wf[i] = (m < cp.Mg && c < pt.kp) ? w[src] : (half_t)0;
  }
}

// NWM 2: two blocks of 6 waves per CU; NWM 4: one block of 10 waves; either way
// at most 3 waves per SIMD (the launch bound), 168 VGPRs each.
// Block b -> (pixel tile, channel block).  Blocks are dealt to the 8 XCDs
// round-robin (block b on XCD b % 8, the b / 8-th there), so XCD x takes a
// contiguous run of pixel tiles, and each tile's channel blocks back to back:
// the channel blocks of one tile run on one XCD at about the same time and
// all but the first read X from its L2, and so do the line pieces that two
// neighbouring tiles of a channel row share.
template <int ACT, int PATCH, int NWM>
__global__ __launch_bounds__(64 * (2 * NWM + 2), 3) void pw_kernel(const half_t* __restrict__ x,
                                                         const half_t* __restrict__ wf,
                                                         const half_t* __restrict__ bias,
                                                         const half_t* z, half_t* y,
                                                         ConvParams cp, PwTile pt) {
  extern __shared__ __attribute__((aligned(16))) half_t lds[];
  const int b = blockIdx.x;
  const int64_t jx = b >> 3;  // the block's place in its XCD's sequence
  const int mb = (int)(jx % pt.nmb);
  const int64_t tg = (int64_t)(b & 7) * (gridDim.x / (8 * pt.nmb)) + jx / pt.nmb;
  if (tg >= pt.tiles) return;
  const int tile = (int)(tg % pt.ntile);
  const int64_t gn = tg / pt.ntile;       // g * n + image (flat: g)
  const int64_t n = cp.flat ? 0 : gn % cp.n;
  const int g = (int)(cp.flat ? gn : gn / cp.n);
  const int64_t P = pt.P;
  const int64_t p0 = (int64_t)tile * kBN;
  constexpr int BM = 64 * NWM;
  const int m0 = mb * BM;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wpi = wave & 1, wmi = wave >> 1;  // pixel half, channel half
  const int r16 = lane & 15, q = lane >> 4;

  // ---- weight fragments of step s: channel tile j, reduction half kk, one
  // contiguous 1 KB piece of Wf per (step, kk, j, wave) and 16 bytes per lane
  constexpr int kFrag = kFragPerWave * NWM;  // halves per (group, m block, step)
  const half_t* wfb = wf + ((int64_t)g * pt.nmb + mb) * pt.ks * kFrag + wmi * 512 + lane * 8;
  auto load_w = [&](int s, half8 (*f)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        f[j][kk] = *(const half8*)(wfb + (int64_t)s * kFrag + (kk * 4 + j) * (NWM * 512));
  };

  // ---- accumulators start at the bias (lane column r16 = channel
  // m0 + wmi*64 + 16j + r16)
  float4v acc[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wmi * 64 + j * 16 + r16;
    float bv = 0.0f;
    if (cp.has_bias && m < cp.Mg) bv = to_f32(bias[PATCH == 3 ? (g * cp.Mg + m) >> 2 : g * cp.Mg + m]);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][j] = float4v{bv, bv, bv, bv};
  }

  // LDS offset (halves) of this lane's operand in pixel tile i, reduction
  // half kk: row wpi*64 + 16i + r16, 16-byte column 4kk + q swizzled by the
  // row's pixel octet
  int aoff[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wpi * 64 + i * 16 + r16;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) aoff[i][kk] = row * kLDC + (((kk * 4 + q) ^ ((row >> 3) & 7)) * 8);
  }

  auto mfma_step = [&](int s, half8 (*f)[2]) __attribute__((always_inline)) {
    const half_t* st = lds + (s & 1) * kStage;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      half8 a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *(const half8*)(st + aoff[i][kk]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], f[j][kk], acc[i][j], 0, 0, 0);
    }
  };

  const int ks = pt.ks;
  if (wave >= 2 * NWM) {
    // ---- producer: items it = ptid and ptid + 128 of each step, item it =
    // (channel quad cq, pixel octet po) with po = (it & 7) + 8*((it >> 4) & 1),
    // cq = ((it >> 3) & 1) + 2*(it >> 5): channels 4*cq .. +3 of the step,
    // pixels 8*po .. +7 of the tile (a 16-lane pass: 2 quads x 8 octets).
    // Invalid pieces read x[0..7] (unconditional loads) and are written as
    // zeros.  Step s: write X(s) into stage s&1, barrier, load X(s+3)
    // (clamped to the last step) into the freed set.
    const int ptid = tid - 128 * NWM;
    int cq[2], po[2];
    bool pix_ok[2];
    const half_t* xs[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int it = ptid + 128 * k;
      po[k] = (it & 7) + 8 * ((it >> 4) & 1);
      cq[k] = ((it >> 3) & 1) + 2 * (it >> 5);
      int64_t pp = p0 + 8 * po[k];
      // P (and OW for a patch conv) % 8 == 0, or the padded rows of an
      // im2col column matrix: an octet is all in or all out of X
      pix_ok[k] = pp < P;
      int64_t nx = n;
      if (cp.flat) {  // octet of image pp / in_sz (in_sz % 8 == 0: never split)
        nx = pp / cp.in_sz;
        pp -= nx * cp.in_sz;
        pix_ok[k] = nx < cp.n;  // the row padding past P reads the zero columns
      }
      const half_t* img = x + (nx * cp.C + (int64_t)g * cp.Cg) * cp.in_sz;
      if constexpr (PATCH != 2) {
        xs[k] = img + pp;
      } else {  // first input column of the octet's 2x2 patches in input row 2*oh
        const int64_t oh = pp / cp.OW, ow = pp - oh * cp.OW;
        xs[k] = img + (2 * oh) * cp.W + 2 * ow;
      }
    }
    // 1x1: loads j = channels 4*cq + j of the step, 8 pixels each.  2x2: the
    // item is input channel st*16 + cq; loads j = (input row 2*oh + j/2,
    // columns 8*(j%2) .. +7 of the octet's 16)
    auto load_x = [&](int st, half8 (*v)[4]) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (PATCH != 2) {
            const int c = st * kBK + 4 * cq[k] + j;
            const bool ok = pix_ok[k] && c < cp.Cg;
            v[k][j] = *(const half8*)(ok ? xs[k] + (int64_t)c * cp.in_sz : x);
          } else {
            const int c = st * (kBK / 4) + cq[k];
            const bool ok = pix_ok[k] && c < cp.Cg;
            v[k][j] = *(const half8*)(ok ? xs[k] + (int64_t)c * cp.in_sz + (j >> 1) * cp.W + (j & 1) * 8 : x);
          }
        }
    };
    auto store_x = [&](int st, half8 (*v)[4]) __attribute__((always_inline)) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        // row 8*po + e, bytes 8*cq .. +7 of the row's channels, swizzled
        half_t* dst = lds + (st & 1) * kStage + (8 * po[k]) * kLDC + ((8 * cq[k]) ^ ((po[k] & 7) << 4)) / 2;
        half8 u[4];
        if constexpr (PATCH != 2) {
          const int cvalid = cp.Cg - st * kBK - 4 * cq[k];
#pragma unroll
          for (int j = 0; j < 4; ++j) u[j] = pix_ok[k] && j < cvalid ? v[k][j] : half8{};
        } else {
          // reduction rows (kh, kw) = (0,0), (0,1), (1,0), (1,1): even and odd
          // columns of the two input rows
          const bool ok = pix_ok[k] && st * (kBK / 4) + cq[k] < cp.Cg;
#pragma unroll
          for (int kh = 0; kh < 2; ++kh) {
            const half8 a = v[k][2 * kh], b = v[k][2 * kh + 1];
            const half8 ev = {a[0], a[2], a[4], a[6], b[0], b[2], b[4], b[6]};
            const half8 od = {a[1], a[3], a[5], a[7], b[1], b[3], b[5], b[7]};
            u[2 * kh] = ok ? ev : half8{};
            u[2 * kh + 1] = ok ? od : half8{};
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *(half4*)(dst + e * kLDC) = half4{u[0][e], u[1][e], u[2][e], u[3][e]};
      }
    };
    half8 x0[2][4], x1[2][4], x2[2][4];
    load_x(0, x0);
    load_x(min(1, ks - 1), x1);
    load_x(min(2, ks - 1), x2);
#define PW_PROD(S, XS)                  \
  {                                     \
    store_x(S, XS);                     \
    lds_barrier();                      \
    load_x(min((S) + 3, ks - 1), XS);   \
  }
    int st = 0;
    for (; st + 3 <= ks; st += 3) {
      PW_PROD(st, x0);
      PW_PROD(st + 1, x1);
      PW_PROD(st + 2, x2);
    }
    if (st < ks) {
      PW_PROD(st, x0);
      if (st + 1 < ks) PW_PROD(st + 1, x1);
    }
#undef PW_PROD
    lds_barrier();  // the MFMA waves' barrier before their epilogue
    return;
  }

  // ---- MFMA waves: step s waits at the barrier for X(s) in stage s&1,
  // loads W(s+1) (clamped) into the other register set, then multiplies.
  // The loads stay between the previous step's products and this step's
  // (scheduling barriers): a product waits only for W(s), issued a step
  // earlier, and W(s+1) never overwrites registers still being read.
  half8 wa[4][2], wb[4][2];
  load_w(0, wa);
#define PW_STEP(S, WC, WN)                  \
  {                                         \
    lds_barrier();                          \
    __builtin_amdgcn_sched_barrier(0);      \
    load_w(min((S) + 1, ks - 1), WN);       \
    __builtin_amdgcn_sched_barrier(0);      \
    mfma_step(S, WC);                       \
  }
  int s = 0;
  for (; s + 2 <= ks; s += 2) {
    PW_STEP(s, wa, wb);
    PW_STEP(s + 1, wb, wa);
  }
  if (s < ks) PW_STEP(s, wa, wb);
#undef PW_STEP
  lds_barrier();  // every MFMA wave is done with the stages

  // ---- epilogue (the stage buffers are dead now): per 16-channel block,
  // the wave's accumulators go to LDS as 16 rows of its 64 pixels; lane
  // (rsub, p4) then owns pixels p4 .. p4+3 of rows rsub, rsub+4, .., adds
  // Z, applies the activation and stores 8 bytes: 16 lanes cover a row's
  // 128 contiguous bytes.  Raw buffer operations: an invalid slot gets an
  // offset past the range (Z reads zero, the store is dropped).
  constexpr int RP = 64 + 4;  // fp32 stage row pitch
  float* stage = (float*)lds + wave * 16 * RP;
  const int mw0 = m0 + wmi * 64;  // first channel of this wave
  const int p4 = (lane & 15) * 4, rsub = lane >> 4;
  int64_t pg = p0 + wpi * 64 + p4;  // image pixel of this lane
  bool pok = pg < P;
  int64_t imgoff = 0;  // flat: the offset of the lane's image in Y and Z
  if (cp.flat) {       // (in_sz and P multiples of 4: a 4-pixel group is never split)
    const int64_t nq = pg / cp.in_sz;
    pg -= nq * cp.in_sz;
    pok = nq < cp.n && pg < P;
    imgoff = nq * cp.M * P;
  }
  int64_t wbase = (n * cp.M + (int64_t)g * cp.Mg + mw0) * P;
  // transposed form: lane (pr, ah) owns input pixels 2pr, 2pr+1 of the
  // wave's 64 and output row phase a = ah; iteration it of block j is output
  // channel 4j + it of the wave's 16 (columns 16j + 4it + 2ah + b)
  const int pr = lane & 31, ah = lane >> 5;
  const int64_t pp2 = p0 + wpi * 64 + 2 * pr;
  const bool pok2 = pp2 < P;  // P % 8 == 0: a pair is all in or all out
  const int mg_out = cp.Mg >> 2, mo0 = mw0 >> 2;
  int64_t obase = 0;  // output offset of the lane's first value in channel mo0
  if constexpr (PATCH == 3) {
    const int64_t ih = pp2 / cp.W, jw = pp2 - ih * cp.W;
    obase = (2 * ih + ah) * cp.OW + 2 * jw;
    wbase = (n * cp.M + (int64_t)g * mg_out + mo0) * cp.out_sz;
  }
  const __amdgpu_buffer_rsrc_t yb =
      __builtin_amdgcn_make_buffer_rsrc((void*)(y + wbase), (short)0, 0x7fffffff, kBufferWord3);
  const __amdgpu_buffer_rsrc_t zb = __builtin_amdgcn_make_buffer_rsrc(
      cp.has_z ? (void*)(z + wbase) : (void*)y, (short)0, cp.has_z ? 0x7fffffff : 0, kBufferWord3);
  auto voff = [&](int j, int it) __attribute__((always_inline)) {
    if constexpr (PATCH == 3) {
      const int cm = 4 * j + it;  // output channel relative to mo0
      return (pok2 && mo0 + cm < mg_out) ? (unsigned)((cm * cp.out_sz + obase) * 2) : kOff;
    }
    const int r = j * 16 + it * 4 + rsub;  // channel relative to mw0
    return (pok && mw0 + r < cp.Mg) ? (unsigned)((imgoff + r * P + pg) * 2) : kOff;
  };
  uint2v zr[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int it = 0; it < 4; ++it)
      zr[j][it] = __builtin_bit_cast(uint2v, __builtin_amdgcn_raw_buffer_load_b64(zb, voff(j, it), 0, 0));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) *(float4v*)(stage + r16 * RP + i * 16 + q * 4) = acc[i][j];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      float4v sv;
      if constexpr (PATCH == 3) {  // (pixel 2pr, b 0), (2pr, 1), (2pr+1, 0), (2pr+1, 1)
        const float2v s0 = *(const float2v*)(stage + (4 * it + 2 * ah) * RP + 2 * pr);
        const float2v s1 = *(const float2v*)(stage + (4 * it + 2 * ah + 1) * RP + 2 * pr);
        sv = float4v{s0[0], s1[0], s0[1], s1[1]};
      } else {
        sv = *(const float4v*)(stage + (it * 4 + rsub) * RP + p4);
      }
      const half4 zh = __builtin_bit_cast(half4, zr[j][it]);
      act4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = sv[e] + (float)zh[e];
      v = act4<ACT>(v, cp.alpha, cp.beta);
      half4 out;
#pragma unroll
      for (int e = 0; e < 4; ++e) out[e] = (half_t)v[e];
      // cache policy 2 = nt: Y is streamed out (downsample and transposed 2x2
      // measured 4-6% faster than with default stores)
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(uint2v, out), yb, voff(j, it), 0, 2);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// PATCH 1: kernel 1, stride 1, no padding.  PATCH 2: 2-D, kernel 2x2, stride
// 2, dilation 1, no padding, OW % 8 == 0 and W % 8 == 0 (16-byte row pieces).
// PATCH 3: transposed, 2-D, kernel 2x2, stride 2, dilation 1, no leading pad
// and an output of exactly 2H x 2W (trailing pads only crop output_padding),
// W % 8 == 0.
int patch_of(const ConvParams& cp) {
  const bool nopad = cp.pd == 0 && cp.ph == 0 && cp.pw == 0;
  if (cp.transposed)
    return (depth_trivial(cp) && cp.KH == 2 && cp.KW == 2 && cp.sh == 2 && cp.sw == 2 &&
            cp.dh == 1 && cp.dw == 1 && nopad && cp.OH == 2 * cp.H && cp.OW == 2 * cp.W &&
            cp.W % 8 == 0)
               ? 3
               : 0;
  if (cp.KD == 1 && cp.KH == 1 && cp.KW == 1 && cp.sd == 1 && cp.sh == 1 && cp.sw == 1 && nopad &&
      cp.OD == cp.D && cp.OH == cp.H && cp.OW == cp.W)
    return 1;
  if (depth_trivial(cp) && cp.KH == 2 && cp.KW == 2 && cp.sh == 2 && cp.sw == 2 &&
      cp.dh == 1 && cp.dw == 1 && nopad && cp.OH == cp.H / 2 && cp.OW == cp.W / 2 &&
      cp.OW % 8 == 0 && cp.W % 8 == 0)
    return 2;
  return 0;
}

bool choose(const ConvParams& cp, int32_t dtype, PwTile& pt) {
  if (dtype != FUSEDCONV_F16) return false;
  const int patch = patch_of(cp);
  if (patch == 0) return false;
  const bool tr = patch == 3;
  pt.wt = tr ? 1 : 0;
  pt.kp = tr ? cp.Cg : cp.Cg * patch * patch;
  if (pt.kp % 8 != 0 || pt.kp < 16) return false;
  pt.P = tr ? cp.in_sz : cp.out_sz;
  // X rows hold in_sz pixels: for a 1x1 conv in_sz == out_sz, so P % 8 == 0;
  // a column matrix (the explicit im2col route) may pad its rows of P % 4 ==
  // 0 pixels to a multiple of 8 -- the octets straddling P read the padding
  // and the epilogue's 4-pixel groups are all in or all out
  if (patch == 1 ? (cp.in_sz % 8 != 0 || cp.in_sz < pt.P || pt.P % 4 != 0) : pt.P % 8 != 0)
    return false;
  // epilogue offsets: 64 channel planes of one image (16 planes of 4P
  // outputs for the transposed form) in 31-bit byte offsets
  if (pt.P * 64 * 2 * (tr ? 2 : 1) >= ((int64_t)1 << 31)) return false;
  // flat pixel axis: a 1x1 GEMM over padded column rows; Y offsets then span
  // every image (n * M * P outputs) in 31-bit byte offsets
  if (cp.flat && (patch != 1 || cp.n * cp.M * pt.P * 2 >= ((int64_t)1 << 31))) return false;
  const int64_t mg = tr ? 4 * (int64_t)cp.Mg : cp.Mg;  // GEMM columns per group
  if (mg >= ((int64_t)1 << 30)) return false;
  pt.ntile = (int)cdiv(cp.flat ? cp.n * cp.in_sz : pt.P, kBN);
  pt.nwm = mg > 128 ? 4 : 2;
  pt.nmb = (int)cdiv(mg, 64 * pt.nwm);
  pt.ks = (int)cdiv(pt.kp, kBK);
  pt.tiles = (int64_t)cp.G * (cp.flat ? 1 : cp.n) * pt.ntile;
  const int64_t blocks = cdiv(pt.tiles, 8) * 8 * pt.nmb;
  return blocks < ((int64_t)1 << 31);
}

// the parameters the kernels see: the transposed form's GEMM has M/group * 4
// columns per group
ConvParams gemm_params(const ConvParams& cp) {
  ConvParams q = cp;
  if (patch_of(cp) == 3) q.Mg *= 4;
  return q;
}

int launch_repack(const ConvParams& cp, const PwTile& pt, const RunArgs& a) {
  const int64_t total = (int64_t)cp.G * pt.nmb * pt.ks * kFragPerWave * pt.nwm;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(repack_frag_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)a.stream,
                     (const half_t*)a.w, (half_t*)a.ws, cp, pt);
  return hipPeekAtLastError() == hipSuccess ? FUSEDCONV_OK : FUSEDCONV_ERR_LAUNCH;
}

}  // namespace

#ifndef FC_ACT
#error "compiled once per activation id: -DFC_ACT=<0..ACT_COUNT-1>"
#endif

// the POINTWISE route with activation FC_ACT
int FC_CAT(launch_pointwise_act_, FC_ACT)(const Geometry& g, const RunArgs& a) {
  PwTile pt;
  if (!choose(g.cp, g.dtype, pt)) return FUSEDCONV_ERR_ROUTE;
  const ConvParams cq = gemm_params(g.cp);
  if (!(a.flags & FUSEDCONV_RUN_WEIGHTS_PREPARED)) {
    const int rc = launch_repack(cq, pt, a);
    if (rc != FUSEDCONV_OK) return rc;
  }
  const int64_t blocks = cdiv(pt.tiles, 8) * 8 * pt.nmb;
  const int patch = patch_of(g.cp);
  const half_t *x = (const half_t*)a.x, *wf = (const half_t*)a.ws, *b = (const half_t*)a.bias,
               *z = (const half_t*)a.z;
  half_t* y = (half_t*)a.y;
  const dim3 grid((unsigned)blocks);
  int rc;
  if (pt.nwm == 2) {
    if (patch == 1) rc = launch_conv(pw_kernel<FC_ACT, 1, 2>, grid, dim3(384), kLds, a, kEdgeBoth, x, wf, b, z, y, cq, pt);
    else if (patch == 2) rc = launch_conv(pw_kernel<FC_ACT, 2, 2>, grid, dim3(384), kLds, a, kEdgeBoth, x, wf, b, z, y, cq, pt);
    else rc = launch_conv(pw_kernel<FC_ACT, 3, 2>, grid, dim3(384), kLds, a, kEdgeBoth, x, wf, b, z, y, cq, pt);
  } else {
    if (patch == 1) rc = launch_conv(pw_kernel<FC_ACT, 1, 4>, grid, dim3(640), kLds, a, kEdgeBoth, x, wf, b, z, y, cq, pt);
    else if (patch == 2) rc = launch_conv(pw_kernel<FC_ACT, 2, 4>, grid, dim3(640), kLds, a, kEdgeBoth, x, wf, b, z, y, cq, pt);
    else rc = launch_conv(pw_kernel<FC_ACT, 3, 4>, grid, dim3(640), kLds, a, kEdgeBoth, x, wf, b, z, y, cq, pt);
  }
  return rc;
}

#if FC_ACT == 0
FC_ACT_DECLS(launch_pointwise_act_)

bool pointwise_fits(const ConvParams& cp, int32_t dtype, size_t* workspace, int32_t* patch,
                    int32_t* block_m) {
  PwTile pt;
  if (!choose(cp, dtype, pt)) return false;
  if (workspace) *workspace = (size_t)cp.G * pt.nmb * pt.ks * kFragPerWave * pt.nwm * sizeof(half_t);
  if (patch) *patch = patch_of(cp);
  if (block_m) *block_m = 64 * pt.nwm;
  return true;
}

int prepare_pointwise(const Geometry& g, const Plan&, const RunArgs& a) {
  PwTile pt;
  if (!choose(g.cp, g.dtype, pt)) return FUSEDCONV_ERR_ROUTE;
  return launch_repack(gemm_params(g.cp), pt, a);
}

int launch_pointwise(const Geometry& g, const Plan&, const RunArgs& a) {
  static const ActLaunchFn table[ACT_COUNT] = FC_ACT_TABLE(launch_pointwise_act_);
  return table[g.cp.act](g, a);
}
#endif

}  // namespace fc
