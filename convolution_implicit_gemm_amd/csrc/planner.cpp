// Planner: picks the kernel route, tile variant and K split for a resolved
// problem.  Host only.
//
// The pages' planners are tuned for WebGPU adapters (FusedConv manifest.json
// derive implicitTiledWorthIt, tiledSplitK*, preferImplicitSplitK); what
// carries over is the shape of the decision: grouped convs with one input
// channel per group go to a direct halo kernel, dense channel counts go to an
// implicit GEMM (1x1 with stride 1: a plain batched GEMM, POINTWISE; few input
// channels: the row-chunk SMALLC form), and a GEMM
// whose output grid cannot fill the device splits
// its reduction (split-K: raw fp32 partials, then one reduce that applies
// bias, residual and activation once).  Thresholds here are for 256 CUs.
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "internal.h"

namespace fc {
namespace {

constexpr int kBK = 32;                     // IGEMM reduction tile
constexpr int kBN = 128;                    // IGEMM column (output pixel) tile
constexpr int64_t kSplitTargetBlocks = 512; // about two workgroups per CU
constexpr int64_t kSplitMaxBase = 128;      // only split grids this small
constexpr size_t kSplitMaxBytes = (size_t)256 << 20;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Non-overlapping patches: stride = kernel on every axis, no padding, no
// dilation, and a kernel above 1x1 (2x2 with stride 2 has the POINTWISE
// route's patch form).
bool patchify(const ConvParams& cp) {
  if (cp.pd || cp.ph || cp.pw || cp.dd != 1 || cp.dh != 1 || cp.dw != 1) return false;
  if (cp.sd != cp.KD || cp.sh != cp.KH || cp.sw != cp.KW) return false;
  return cp.taps > 4;
}

// Grid limits of the IGEMM launch: x = column tiles, y = row tiles, z = group * split.
bool igemm_grid_ok(const ConvParams& cp, int64_t split) {
  const int bm = cp.Mg > 64 ? 128 : 64;
  return cdiv(cp.P, kBN) < ((int64_t)1 << 31) && cdiv(cp.Mg, bm) <= 65535 &&
         cp.G * split <= 65535;
}

int plan_igemm(const Geometry& g, int32_t split_req, Plan& p, std::string& err) {
  const ConvParams& cp = g.cp;
  const int bm = cp.Mg > 64 ? 128 : 64;
  p.route = FUSEDCONV_ROUTE_IGEMM;
  p.tile = bm == 128 ? IGEMM_BM128_BN128 : IGEMM_BM64_BN128;
  p.k_tiles = (int32_t)cdiv(cp.K, kBK);
  const int64_t base = cdiv(cp.Mg, bm) * cdiv(cp.P, kBN) * cp.G;
  int split = 1;
  if (split_req > 0) {
    if (split_req > p.k_tiles) {
      err = "split_k larger than the number of K tiles";
      return FUSEDCONV_ERR_ROUTE;
    }
    split = split_req;
  } else if (base <= kSplitMaxBase && cp.K >= 8 * kBK) {
    for (int s = 16; s >= 2; s /= 2) {
      if (base * s <= kSplitTargetBlocks && p.k_tiles >= 2 * s &&
          (size_t)s * cp.M * cp.P * 4 <= kSplitMaxBytes) {
        split = s;
        break;
      }
    }
  }
  p.k_tiles_per_split = (int32_t)cdiv(p.k_tiles, split);
  split = (int32_t)cdiv(p.k_tiles, p.k_tiles_per_split);  // no empty slices
  if (!igemm_grid_ok(cp, split)) {
    err = "IGEMM grid exceeds the launch limits (row tiles or group * split above 65535)";
    return FUSEDCONV_ERR_ROUTE;
  }
  p.split_k = split;
  p.workspace = split > 1 ? (size_t)split * cp.M * cp.P * sizeof(float) : 0;
  snprintf(p.name, sizeof(p.name), "igemm_%s_bm%d_bn%d%s", g.dtype == FUSEDCONV_F16 ? "f16" : "f32",
           bm, kBN, split > 1 ? "_splitk" : "");
  return FUSEDCONV_OK;
}

}  // namespace

int make_plan(const Geometry& g, int32_t route, int32_t split_req, Plan& p, std::string& err) {
  memset(&p, 0, sizeof(p));
  p.split_k = 1;
  const ConvParams& cp = g.cp;
  if (split_req < 0) {
    err = "split_k must be >= 0";
    return FUSEDCONV_ERR_ROUTE;
  }
  if (route < FUSEDCONV_ROUTE_AUTO || route > FUSEDCONV_ROUTE_IM2COL) {
    err = "unknown route";
    return FUSEDCONV_ERR_ROUTE;
  }
  if (split_req > 1 && route != FUSEDCONV_ROUTE_IGEMM && route != FUSEDCONV_ROUTE_AUTO) {
    err = "split_k applies to the IGEMM route only";
    return FUSEDCONV_ERR_ROUTE;
  }
  if (cp.transposed || route == FUSEDCONV_ROUTE_TRANSPOSED) {
    if (!cp.transposed || (route != FUSEDCONV_ROUTE_AUTO && route != FUSEDCONV_ROUTE_TRANSPOSED) ||
        split_req > 1) {
      err = "TRANSPOSED is the route of transposed convolutions (fusedconv_create_transposed), "
            "and their only one";
      return FUSEDCONV_ERR_ROUTE;
    }
    p.route = FUSEDCONV_ROUTE_TRANSPOSED;
    size_t ws = 0;
    int32_t bmt = 0;
    if (pointwise_fits(cp, g.dtype, &ws, nullptr, &bmt)) {
      // 2x2 stride 2 without cropping: the pointwise GEMM kernel's transposed form
      p.tile = 1;
      p.workspace = ws;
      snprintf(p.name, sizeof(p.name), "transposed_2x2s2_pointwise_f16_m%d", (int)bmt);
    } else {
      p.tile = 0;
      snprintf(p.name, sizeof(p.name), "transposed_gather_%s",
               g.dtype == FUSEDCONV_F16 ? "f16" : "f32");
    }
    return FUSEDCONV_OK;
  }
  int32_t th = 0, tw = 0;
  size_t halo_ws = 0;
  int32_t bm = 0;  // halo and pointwise routes: output channels per block
  int32_t patch = 1;  // pointwise route: 1 (1x1) or 2 (2x2 with stride 2)
  int64_t hblocks = 0;  // fp32 halo route: its grid
  if (route == FUSEDCONV_ROUTE_AUTO) {
    if (split_req > 1) route = FUSEDCONV_ROUTE_IGEMM;
    else if (cp.Cg == 1 && depthwise_fits(cp, th, tw)) route = FUSEDCONV_ROUTE_DEPTHWISE;
    // 1x1, and 2x2 with stride 2: the pointwise GEMM (measured on MI355X
    // against the halo route: 1x1 at C/group 512 2.6x faster, 256 8-9%, 128 on
    // par)
    else if (pointwise_fits(cp, g.dtype)) route = FUSEDCONV_ROUTE_POINTWISE;
    else if (igemm_halo_fits(cp, g.dtype, th, tw, halo_ws)) route = FUSEDCONV_ROUTE_IGEMM_HALO;
    // fp32: the channel-last halo kernel on the fp32 matrix cores, when its
    // grid fills the chip (a starved grid takes IGEMM, which splits K)
    else if (halo32_fits(cp, g.dtype, nullptr, nullptr, nullptr, &hblocks) && hblocks >= 512)
      route = FUSEDCONV_ROUTE_IGEMM_HALO;
    else if (smallc_fits(cp, g.dtype, th, tw, halo_ws)) route = FUSEDCONV_ROUTE_SMALLC;
    // larger non-overlapping patches (stride = kernel): explicit im2col, whose
    // column matrix is then a permutation of X (the manifest's
    // implicitTiledWorthIt rule: the implicit routes pay off for stride < kernel)
    else if (patchify(cp) && im2col_fits(cp, g.dtype, nullptr)) route = FUSEDCONV_ROUTE_IM2COL;
    else if (cp.K >= 8 && cp.Mg >= 8 && igemm_grid_ok(cp, 1)) route = FUSEDCONV_ROUTE_IGEMM;
    else route = FUSEDCONV_ROUTE_DIRECT;
  }
  switch (route) {
    case FUSEDCONV_ROUTE_DIRECT:
      p.route = route;
      snprintf(p.name, sizeof(p.name), "direct_%s", g.dtype == FUSEDCONV_F16 ? "f16" : "f32");
      return FUSEDCONV_OK;
    case FUSEDCONV_ROUTE_IGEMM:
      return plan_igemm(g, split_req, p, err);
    case FUSEDCONV_ROUTE_DEPTHWISE:
      if (cp.Cg != 1 || !depthwise_fits(cp, th, tw)) {
        err = "DEPTHWISE needs one input channel per group, at most 2 spatial dims and a "
              "halo tile that fits in LDS";
        return FUSEDCONV_ERR_ROUTE;
      }
      p.route = route;
      p.tile_h = th;
      p.tile_w = tw;
      if (depthwise_mfma_fits(cp, g.dtype)) {
        p.tile = 2;  // banded-matrix MFMA kernel
        snprintf(p.name, sizeof(p.name), "depthwise_mfma_f16_k%dx%d", cp.KH, cp.KW);
      } else if (depthwise_fast(cp, g.dtype)) {
        p.tile = 1;  // register-window dot2 kernel
        snprintf(p.name, sizeof(p.name), "depthwise_dot2_f16_k%dx%d", cp.KH, cp.KW);
      } else {
        snprintf(p.name, sizeof(p.name), "depthwise_%s_t%dx%d",
                 g.dtype == FUSEDCONV_F16 ? "f16" : "f32", th, tw);
      }
      return FUSEDCONV_OK;
    case FUSEDCONV_ROUTE_IGEMM_HALO:
      if (g.dtype == FUSEDCONV_F32) {
        if (!halo32_fits(cp, g.dtype, &halo_ws, &th, &tw)) {
          err = "IGEMM_HALO (fp32) needs at most 64 taps per box and two input boxes of a "
                "128- or 256-pixel tile within 64 KB of LDS (3-D: or one box of one input "
                "depth plane)";
          return FUSEDCONV_ERR_ROUTE;
        }
        p.route = route;
        p.tile_h = th;
        p.tile_w = tw;
        p.workspace = halo_ws;
        snprintf(p.name, sizeof(p.name), "igemm_halo_f32_t%dx%d", th, tw);
        return FUSEDCONV_OK;
      }
      if (!igemm_halo_fits(cp, g.dtype, th, tw, halo_ws, &bm)) {
        err = "IGEMM_HALO needs fp16, C/group >= 32, at most 64 taps and a halo box that fits "
              "in LDS";
        return FUSEDCONV_ERR_ROUTE;
      }
      p.route = route;
      p.tile_h = th;
      p.tile_w = tw;
      p.workspace = halo_ws;
      // blocks of 256 output channels (8 waves) are named by it
      if (bm == 256) snprintf(p.name, sizeof(p.name), "igemm_halo_f16_m256_t%dx%d", th, tw);
      else snprintf(p.name, sizeof(p.name), "igemm_halo_f16_t%dx%d", th, tw);
      return FUSEDCONV_OK;
    case FUSEDCONV_ROUTE_SMALLC:
      if (!smallc_fits(cp, g.dtype, th, tw, halo_ws)) {
        err = "SMALLC needs fp16, 1 or 2 spatial dims, dilation 1 along the last axis, "
              "C/group < 16 and C/group * KH * ceil(KW/8) <= 24";
        return FUSEDCONV_ERR_ROUTE;
      }
      p.route = route;
      p.tile_h = th;
      p.tile_w = tw;
      p.workspace = halo_ws;
      snprintf(p.name, sizeof(p.name), "smallc_f16_t%dx%d", th, tw);
      return FUSEDCONV_OK;
    case FUSEDCONV_ROUTE_POINTWISE:
      if (!pointwise_fits(cp, g.dtype, &halo_ws, &patch, &bm)) {
        err = "POINTWISE needs fp16, no padding, and either kernel 1 with stride 1 or a 2-D "
              "2x2 kernel with stride 2 (OW and W multiples of 8); C/group * taps a multiple "
              "of 8 and >= 16, and a pixel count per image that is a multiple of 8";
        return FUSEDCONV_ERR_ROUTE;
      }
      p.route = route;
      p.workspace = halo_ws;
      snprintf(p.name, sizeof(p.name), "pointwise_f16_%sm%d_n128", patch == 2 ? "patch2x2_" : "",
               (int)bm);
      return FUSEDCONV_OK;
    case FUSEDCONV_ROUTE_IM2COL:
      if (!im2col_fits(cp, g.dtype, &halo_ws)) {
        err = "IM2COL needs a forward fp16 problem with a number of output pixels per image that is a multiple of 4";
        return FUSEDCONV_ERR_ROUTE;
      }
      p.route = route;
      p.workspace = halo_ws;
      // K rounded up to a multiple of 8 and at least 16: the GEMM's reduction
      snprintf(p.name, sizeof(p.name), "im2col_f16_k%d", std::max(16, (int)((cp.K + 7) / 8 * 8)));
      return FUSEDCONV_OK;
    default:
      err = "unknown route";
      return FUSEDCONV_ERR_ROUTE;
  }
}

}  // namespace fc
