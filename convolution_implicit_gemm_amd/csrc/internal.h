// Host-side internals: resolver, planner and kernel launchers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "conv_params.h"
#include "fusedconv.h"

namespace fc {

// Result of attribute resolution (everything fusedconv_create validates).
struct Geometry {
  int32_t dtype;        // fusedconv_dtype
  int32_t nsp;          // spatial rank 1..3
  int32_t y_rank;
  int64_t y_dims[FUSEDCONV_MAX_RANK];
  ConvParams cp;
};

// Kernel variants of the IGEMM (gathered im2col) route.
enum IgemmTile : int32_t {
  IGEMM_BM128_BN128 = 0,   // 4 waves as 2x2, 64x64 per wave
  IGEMM_BM64_BN128 = 1,    // 4 waves as 1x4, 64x32 per wave
};

struct Plan {
  int32_t route;         // fusedconv_route (never AUTO)
  int32_t split_k;       // >= 1
  int32_t tile;          // route-specific variant id
  int32_t k_tiles;       // IGEMM: number of BK-wide K tiles
  int32_t k_tiles_per_split;
  // DEPTHWISE / IGEMM_HALO: output tile extents
  int32_t tile_h, tile_w;
  size_t workspace;      // bytes
  char name[64];
};

int resolve(const fusedconv_desc& d, Geometry& g, std::string& err);
int make_plan(const Geometry& g, int32_t route, int32_t split_k, Plan& p, std::string& err);

// Device launchers (kernels_*.hip).  Return 0 or FUSEDCONV_ERR_LAUNCH.
struct RunArgs {
  const void* x;
  const void* w;
  const void* bias;
  const void* z;
  void* y;
  void* ws;
  void* stream;
  unsigned flags;   // FUSEDCONV_RUN_WEIGHTS_PREPARED
};

int launch_direct(const Geometry& g, const Plan& p, const RunArgs& a);
int launch_igemm(const Geometry& g, const Plan& p, const RunArgs& a);
int launch_depthwise(const Geometry& g, const Plan& p, const RunArgs& a);
int launch_igemm_halo(const Geometry& g, const Plan& p, const RunArgs& a);
int prepare_igemm_halo(const Geometry& g, const Plan& p, const RunArgs& a);

// Depthwise planning helper (kernels_depthwise.hip knows its LDS budget).
bool depthwise_fits(const ConvParams& cp, int32_t& tile_h, int32_t& tile_w);
bool depthwise_fast(const ConvParams& cp, int32_t dtype);
bool igemm_halo_fits(const ConvParams& cp, int32_t dtype, int32_t& tile_h, int32_t& tile_w,
                     size_t& workspace);

}  // namespace fc
