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
  // DEPTHWISE / IGEMM_HALO / SMALLC: output tile extents
  int32_t tile_h, tile_w;
  size_t workspace;      // bytes
  char name[64];
};

int resolve(const fusedconv_desc& d, Geometry& g, std::string& err);
// Transposed convolution (fusedconv_create_transposed): d describes X, W as
// [C, M/group, k...], B of length M and Z of Y's shape; output_padding has
// one entry per spatial axis (NULL: zeros).
int resolve_transposed(const fusedconv_desc& d, const int64_t* output_padding,
                       int32_t n_output_padding, Geometry& g, std::string& err);
int make_plan(const Geometry& g, int32_t route, int32_t split_k, Plan& p, std::string& err);

// Device launchers (kernels_*.hip).  Return 0 or FUSEDCONV_ERR_LAUNCH.
struct RunArgs {
  const void* x;
  const void* w;
  const void* bias;
  const void* z;
  const void* pre;  // backward data: the pre-activation P of the convolution's input
  void* y;
  void* ws;
  void* stream;
  unsigned flags;   // FUSEDCONV_RUN_WEIGHTS_PREPARED
  void* ev_start;   // timed run: hipEvent_t recorded at the first convolution kernel's begin
  void* ev_stop;    // and at the last one's end (both NULL otherwise)
};

// Record `msg` as the calling thread's fusedconv_last_error() text; returns code.
int set_last_error(int code, const std::string& msg);
void clear_last_error();

// Raise kernel kfn's dynamic-LDS limit to `bytes` on the current device,
// once per (kernel, device, bytes); safe to call from several threads.
int set_max_dynamic_lds(const void* kfn, int bytes);

int launch_direct(const Geometry& g, const Plan& p, const RunArgs& a);
int launch_igemm(const Geometry& g, const Plan& p, const RunArgs& a);
int launch_depthwise(const Geometry& g, const Plan& p, const RunArgs& a);
int launch_igemm_halo(const Geometry& g, const Plan& p, const RunArgs& a);
int prepare_igemm_halo(const Geometry& g, const Plan& p, const RunArgs& a);
int launch_smallc(const Geometry& g, const Plan& p, const RunArgs& a);
int prepare_smallc(const Geometry& g, const Plan& p, const RunArgs& a);
int launch_pointwise(const Geometry& g, const Plan& p, const RunArgs& a);
int launch_transposed(const Geometry& g, const Plan& p, const RunArgs& a);
int prepare_pointwise(const Geometry& g, const Plan& p, const RunArgs& a);
// Explicit im2col route (kernels_im2col.hip), fp16: fits (with its workspace:
// the GEMM's repacked weights, W padded to a multiple of 8 columns, the
// column matrix), weight preparation and launch.
bool im2col_fits(const ConvParams& cp, int32_t dtype, size_t* workspace);
// The column matrix of cp (a forward problem) in dtype: col[n][g][Kq][Pp],
// rows k < K the im2col of X (zero outside X and at pixels p >= P), row K
// ones at p < P when `ones`, the other rows zero; Kq >= K, Pp >= P, Pp % 8
// == 0.  One kernel, launched with launch_conv's timing edges.
int launch_columns(const ConvParams& cp, int32_t dtype, const void* x, void* col, int Kq,
                   int64_t Pp, int ones, const RunArgs& a, unsigned edges);
int prepare_im2col(const Geometry& g, const Plan& p, const RunArgs& a);
int launch_im2col(const Geometry& g, const Plan& p, const RunArgs& a);

// Backward (kernels_backward.hip).  W of forward problem f, [M][C/G][taps],
// to W' = [C][M/G][taps] flipped in every spatial axis (the weights of the
// stride-1 input gradient as a forward convolution).
int launch_flip_weights(const ConvParams& f, int32_t dtype, const void* w, void* wf, void* stream);
// Weight gradient of forward problem cp as a GEMM over its column matrix:
// fits, with the workspace (column matrix + fp32 partials) and the image
// ranges; launch (plan route IM2COL: the GEMM; DIRECT: the plain reduction).
// dw: float [M][C/G][taps]; db: float [M] or NULL.
bool wgrad_gemm_fits(const ConvParams& cp, int32_t dtype, int has_db, size_t* workspace,
                     int32_t* splits);
// The shifted-tap form (plan route IGEMM_HALO): no column matrix, fp32
// partials only.
bool wgrad_tap_fits(const ConvParams& cp, int32_t dtype, int has_db, size_t* workspace,
                    int32_t* splits);
int launch_wgrad(const Geometry& g, const Plan& p, const void* x, const void* dy, float* dw,
                 float* db, void* ws, void* stream);

// Kernels whose activation is a compile-time parameter: the build compiles
// their source once per activation id (FC_ACT = 0 .. ACT_COUNT-1); unit k
// defines <name>k(g, a), and unit 0 also holds the route's entry points and
// a table of the ACT_COUNT launchers, indexed by the resolved activation.
typedef int (*ActLaunchFn)(const Geometry& g, const RunArgs& a);
#define FC_CAT2(a, b) a##b
#define FC_CAT(a, b) FC_CAT2(a, b)
#define FC_ACT_DECLS(name)                                                                 \
  int name##0(const Geometry&, const RunArgs&); int name##1(const Geometry&, const RunArgs&);   \
  int name##2(const Geometry&, const RunArgs&); int name##3(const Geometry&, const RunArgs&);   \
  int name##4(const Geometry&, const RunArgs&); int name##5(const Geometry&, const RunArgs&);   \
  int name##6(const Geometry&, const RunArgs&); int name##7(const Geometry&, const RunArgs&);   \
  int name##8(const Geometry&, const RunArgs&); int name##9(const Geometry&, const RunArgs&);   \
  int name##10(const Geometry&, const RunArgs&); int name##11(const Geometry&, const RunArgs&); \
  int name##12(const Geometry&, const RunArgs&); int name##13(const Geometry&, const RunArgs&); \
  int name##14(const Geometry&, const RunArgs&);
#define FC_ACT_TABLE(name)                                                                 \
  { name##0, name##1, name##2, name##3, name##4, name##5, name##6, name##7, name##8,        \
    name##9, name##10, name##11, name##12, name##13, name##14 }
static_assert(ACT_COUNT == 15, "FC_ACT_DECLS / FC_ACT_TABLE list every activation id");

// Depthwise planning helper (kernels_depthwise.hip knows its LDS budget).
bool depthwise_fits(const ConvParams& cp, int32_t& tile_h, int32_t& tile_w);
bool depthwise_fast(const ConvParams& cp, int32_t dtype);
// Toeplitz-MFMA depthwise kernel (kernels_dwmfma.hip): fits / launch.
bool depthwise_mfma_fits(const ConvParams& cp, int32_t dtype);
int launch_depthwise_mfma(const Geometry& g, const RunArgs& a);
// Halo route (kernels_halo.hip): fits, with the output tile, the weight
// workspace and (when block_m is given) the block's output channels.
bool igemm_halo_fits(const ConvParams& cp, int32_t dtype, int32_t& tile_h, int32_t& tile_w,
                     size_t& workspace, int32_t* block_m = nullptr);
bool smallc_fits(const ConvParams& cp, int32_t dtype, int32_t& tile_h, int32_t& tile_w,
                 size_t& workspace);
// The fp32 halo kernel (kernels_halo32.hip; route IGEMM_HALO for fp32): fits,
// with the repacked-weight workspace and the output tile; weight repack; launch.
bool halo32_fits(const ConvParams& cp, int32_t dtype, size_t* workspace, int32_t* tile_h,
                 int32_t* tile_w, int64_t* blocks = nullptr);
int prepare_halo32(const Geometry& g, const Plan& p, const RunArgs& a);
int launch_halo32(const Geometry& g, const Plan& p, const RunArgs& a);
// Pointwise route (kernels_pointwise.hip), fp16: 1x1 with stride 1, or 2x2
// with stride 2 (patch 2), no padding; optionally the bytes of its
// repacked-weight workspace, the patch size and the block's output channels.
bool pointwise_fits(const ConvParams& cp, int32_t dtype, size_t* workspace = nullptr,
                    int32_t* patch = nullptr, int32_t* block_m = nullptr);

}  // namespace fc
