// Backward entry points (include/fusedconv.h: fusedconv_create_backward_data,
// fusedconv_backward_data, fusedconv_create_backward_weight,
// fusedconv_backward_weight): planning on the host, launches in
// kernels_backward.hip and the forward routes.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <string.h>

#include <new>
#include <string>

#include "handle.h"
#include "internal.h"

namespace fc {
namespace {

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// The forward problem of a backward descriptor: d without Z (and without B
// for the data gradient); the activation stays (act_in for the data
// gradient, ignored for the weight gradient).
int resolve_forward(const fusedconv_desc& d, bool keep_bias, bool keep_act, Geometry& f,
                    std::string& err) {
  fusedconv_desc fd = d;
  fd.z.present = 0;
  if (!keep_bias) fd.bias.present = 0;
  if (!keep_act) {
    fd.activation = nullptr;
    fd.activation_params = nullptr;
    fd.n_activation_params = 0;
  }
  return resolve(fd, f, err);
}

// Stride 1 and begin/end pads within dilation*(k - 1) on every axis: the
// input gradient is a forward convolution with the flipped kernel.
bool flip_form(const ConvParams& f, int32_t pads_out[3][2]) {
  const int32_t s[3] = {f.sd, f.sh, f.sw}, d[3] = {f.dd, f.dh, f.dw}, k[3] = {f.KD, f.KH, f.KW};
  const int32_t pb[3] = {f.pd, f.ph, f.pw};
  const int64_t in[3] = {f.D, f.H, f.W}, out[3] = {f.OD, f.OH, f.OW};
  for (int i = 0; i < 3; ++i) {
    if (s[i] != 1) return false;
    const int64_t span = (int64_t)d[i] * (k[i] - 1);
    const int64_t pe = out[i] - in[i] - pb[i] + span;  // the forward end pad
    const int64_t b = span - pb[i], e = span - pe;
    if (b < 0 || e < 0) return false;
    pads_out[i][0] = (int32_t)b;
    pads_out[i][1] = (int32_t)e;
  }
  return true;
}

}  // namespace
}  // namespace fc

extern "C" {

int fusedconv_create_backward_data(const fusedconv_desc* d, fusedconv_handle** out) {
  using namespace fc;
  if (out) *out = nullptr;
  if (!d || !out) return set_last_error(FUSEDCONV_ERR_NULL_ARG, "desc and out must not be NULL");
  if (d->bias.present)
    return set_last_error(FUSEDCONV_ERR_BIAS_SHAPE, "the input gradient takes no bias");
  fusedconv_handle* h = new (std::nothrow) fusedconv_handle();
  if (!h) return set_last_error(FUSEDCONV_ERR_ALLOC, "out of host memory");
  std::string err;
  Geometry& f = h->fwd;
  int rc = resolve_forward(*d, false, true, f, err);
  if (rc == FUSEDCONV_OK && d->z.present) {
    bool same = d->z.rank == d->x.rank;
    for (int i = 0; same && i < d->x.rank; ++i) same = d->z.dims[i] == d->x.dims[i];
    if (!same) {
      rc = FUSEDCONV_ERR_Z_SHAPE;
      err = "the residual gradient must have exactly the shape of x";
    }
  }
  if (rc != FUSEDCONV_OK) {
    delete h;
    return set_last_error(rc, err);
  }
  const ConvParams& fp = f.cp;
  Geometry& g = h->geo;
  g.dtype = f.dtype;
  g.nsp = f.nsp;
  g.y_rank = d->x.rank;
  for (int i = 0; i < d->x.rank; ++i) g.y_dims[i] = d->x.dims[i];
  // X and Y swapped: the problem G -> dP
  ConvParams& cp = g.cp;
  cp = fp;
  cp.C = fp.M;
  cp.M = fp.C;
  cp.Cg = fp.Mg;
  cp.Mg = fp.Cg;
  cp.D = fp.OD; cp.H = fp.OH; cp.W = fp.OW;
  cp.OD = fp.D; cp.OH = fp.H; cp.OW = fp.W;
  cp.K = cp.Cg * cp.taps;
  cp.in_sz = fp.out_sz;
  cp.out_sz = fp.in_sz;
  cp.P = fp.n * cp.out_sz;
  cp.has_bias = 0;
  cp.has_z = d->z.present ? 1 : 0;
  cp.bwd = 1;
  int32_t pads[3][2];
  const int32_t route = d->route;
  const bool flip = route != FUSEDCONV_ROUTE_TRANSPOSED && flip_form(fp, pads);
  Plan& p = h->plan;
  if (flip) {
    cp.pd = pads[0][0];
    cp.ph = pads[1][0];
    cp.pw = pads[2][0];
    cp.transposed = 0;
    int32_t r = route;
    if (r == FUSEDCONV_ROUTE_AUTO) {
      int32_t th = 0, tw = 0;
      size_t ws = 0;
      if (d->split_k > 1) r = FUSEDCONV_ROUTE_IGEMM;
      else if (igemm_halo_fits(cp, g.dtype, th, tw, ws)) r = FUSEDCONV_ROUTE_IGEMM_HALO;
      else if (halo32_fits(cp, g.dtype, nullptr, nullptr, nullptr)) r = FUSEDCONV_ROUTE_IGEMM_HALO;
      else if (cp.K >= 8 && cp.Mg >= 8) r = FUSEDCONV_ROUTE_IGEMM;
      else r = FUSEDCONV_ROUTE_DIRECT;
    }
    if (r != FUSEDCONV_ROUTE_IGEMM_HALO && r != FUSEDCONV_ROUTE_IGEMM && r != FUSEDCONV_ROUTE_DIRECT) {
      rc = FUSEDCONV_ERR_ROUTE;
      err = "the input gradient runs on AUTO, IGEMM_HALO, IGEMM, DIRECT or TRANSPOSED";
    } else {
      rc = make_plan(g, r, d->split_k, p, err);
      if (rc == FUSEDCONV_OK && r == FUSEDCONV_ROUTE_IGEMM && p.route != FUSEDCONV_ROUTE_IGEMM)
        rc = FUSEDCONV_ERR_ROUTE;
    }
    if (rc == FUSEDCONV_OK) {
      h->flip_bytes = align256((size_t)fp.M * fp.Cg * fp.taps * (g.dtype == FUSEDCONV_F16 ? 2 : 4));
      p.workspace += h->flip_bytes;
      char name[64];
      snprintf(name, sizeof(name), "bwd_data_flip_%s", p.name);
      memcpy(p.name, name, sizeof(p.name));
      p.name[sizeof(p.name) - 1] = '\0';
    }
  } else if (route != FUSEDCONV_ROUTE_AUTO && route != FUSEDCONV_ROUTE_TRANSPOSED) {
    rc = FUSEDCONV_ERR_ROUTE;
    err = "strided (or over-padded) convolutions: the input gradient runs on TRANSPOSED only";
  } else if (d->split_k > 1) {
    rc = FUSEDCONV_ERR_ROUTE;
    err = "split_k applies to IGEMM only";
  } else {
    // the gather kernel of transposed convolutions: the pads of the forward
    // problem are the begin offsets of its output (= X)
    cp.transposed = 1;
    memset(&p, 0, sizeof(p));
    p.route = FUSEDCONV_ROUTE_TRANSPOSED;
    p.split_k = 1;
    p.tile = 0;
    snprintf(p.name, sizeof(p.name), "bwd_data_gather_%s", g.dtype == FUSEDCONV_F16 ? "f16" : "f32");
  }
  if (rc != FUSEDCONV_OK) {
    delete h;
    return set_last_error(rc, err);
  }
  h->kind = kBackwardData;
  *out = h;
  clear_last_error();
  return FUSEDCONV_OK;
}

int fusedconv_backward_data(const fusedconv_handle* h, const void* dy, const void* w,
                            const void* pre, const void* dres, void* dx, void* workspace,
                            size_t workspace_bytes, void* stream) {
  using namespace fc;
  if (!h || !dy || !w || !dx)
    return set_last_error(FUSEDCONV_ERR_NULL_ARG, "h, dy, w and dx are required");
  if (h->kind != kBackwardData)
    return set_last_error(FUSEDCONV_ERR_ROUTE, "not a fusedconv_create_backward_data handle");
  const ConvParams& cp = h->geo.cp;
  const bool need_pre = cp.act != ACT_NONE;
  if (need_pre && !pre)
    return set_last_error(FUSEDCONV_ERR_NULL_ARG, "pre is required with an input activation");
  if (cp.has_z && !dres) return set_last_error(FUSEDCONV_ERR_NULL_ARG, "dres declared but NULL");
  if (!cp.has_z && dres)
    return set_last_error(FUSEDCONV_ERR_NULL_ARG, "dres given but not declared in the descriptor");
  if (!aligned16(dy) || !aligned16(w) || !aligned16(dx) || (need_pre && !aligned16(pre)) ||
      (dres && !aligned16(dres)) || (workspace && !aligned16(workspace)))
    return set_last_error(FUSEDCONV_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  if (h->plan.workspace > 0 && (!workspace || workspace_bytes < h->plan.workspace))
    return set_last_error(FUSEDCONV_ERR_WORKSPACE,
                          "workspace smaller than fusedconv_workspace_size() reports");
  int rc = check_device(stream);
  if (rc != FUSEDCONV_OK) return rc;
  (void)hipGetLastError();
  RunArgs a{};
  a.x = dy;
  a.w = w;
  a.z = dres;
  a.pre = need_pre ? pre : nullptr;
  a.y = dx;
  a.ws = workspace;
  a.stream = stream;
  if (h->flip_bytes) {
    rc = launch_flip_weights(h->fwd.cp, h->geo.dtype, w, workspace, stream);
    a.w = workspace;
    a.ws = (char*)workspace + h->flip_bytes;
  }
  if (rc == FUSEDCONV_OK) {
    switch (h->plan.route) {
      case FUSEDCONV_ROUTE_IGEMM_HALO: rc = launch_igemm_halo(h->geo, h->plan, a); break;
      case FUSEDCONV_ROUTE_IGEMM: rc = launch_igemm(h->geo, h->plan, a); break;
      case FUSEDCONV_ROUTE_DIRECT: rc = launch_direct(h->geo, h->plan, a); break;
      case FUSEDCONV_ROUTE_TRANSPOSED: rc = launch_transposed(h->geo, h->plan, a); break;
      default: return set_last_error(FUSEDCONV_ERR_ROUTE, "handle has no route");
    }
  }
  if (rc != FUSEDCONV_OK) {
    hipError_t e = hipGetLastError();
    return set_last_error(rc, std::string("kernel launch failed: ") + hipGetErrorString(e));
  }
  return FUSEDCONV_OK;
}

int fusedconv_create_backward_weight(const fusedconv_desc* d, fusedconv_handle** out) {
  using namespace fc;
  if (out) *out = nullptr;
  if (!d || !out) return set_last_error(FUSEDCONV_ERR_NULL_ARG, "desc and out must not be NULL");
  fusedconv_handle* h = new (std::nothrow) fusedconv_handle();
  if (!h) return set_last_error(FUSEDCONV_ERR_ALLOC, "out of host memory");
  std::string err;
  int rc = resolve_forward(*d, true, false, h->fwd, err);
  if (rc != FUSEDCONV_OK) {
    delete h;
    return set_last_error(rc, err);
  }
  h->geo = h->fwd;
  Geometry& g = h->geo;
  g.y_rank = d->w.rank;
  for (int i = 0; i < d->w.rank; ++i) g.y_dims[i] = d->w.dims[i];
  const ConvParams& cp = g.cp;
  h->has_db = d->bias.present ? 1 : 0;
  Plan& p = h->plan;
  memset(&p, 0, sizeof(p));
  p.split_k = 1;
  int32_t route = d->route;
  size_t ws = 0;
  int32_t splits = 1;
  if (route == FUSEDCONV_ROUTE_AUTO)
    route = wgrad_tap_fits(cp, g.dtype, h->has_db, nullptr, nullptr) ? FUSEDCONV_ROUTE_IGEMM_HALO
                                                                     : FUSEDCONV_ROUTE_IM2COL;
  if (cp.transposed) {
    rc = FUSEDCONV_ERR_ROUTE;
    err = "weight gradients of forward convolutions only";
  } else if (route == FUSEDCONV_ROUTE_IGEMM_HALO) {
    if (!wgrad_tap_fits(cp, g.dtype, h->has_db, &ws, &splits)) {
      rc = FUSEDCONV_ERR_ROUTE;
      err = "the shifted-tap weight gradient needs fp16, stride 1, a 1-D or 2-D kernel of at "
            "most 9 taps, W and output W multiples of 8 and C/group a multiple of 16";
    }
  } else if (route == FUSEDCONV_ROUTE_IM2COL) {
    if (!wgrad_gemm_fits(cp, g.dtype, h->has_db, &ws, &splits)) {
      if (d->route == FUSEDCONV_ROUTE_AUTO) {
        route = FUSEDCONV_ROUTE_DIRECT;
      } else {
        rc = FUSEDCONV_ERR_ROUTE;
        err = "the weight-gradient GEMM needs a number of output pixels per image that is a "
              "multiple of 4";
      }
    }
  } else if (route != FUSEDCONV_ROUTE_DIRECT) {
    rc = FUSEDCONV_ERR_ROUTE;
    err = "the weight gradient runs on AUTO, IGEMM_HALO, IM2COL or DIRECT";
  }
  if (rc == FUSEDCONV_OK && route == FUSEDCONV_ROUTE_DIRECT &&
      (int64_t)cp.M * (cp.K + h->has_db) >= ((int64_t)1 << 31)) {
    rc = FUSEDCONV_ERR_TOO_LARGE;
    err = "too many weights for the plain reduction";
  }
  if (rc != FUSEDCONV_OK) {
    delete h;
    return set_last_error(rc, err);
  }
  p.route = route;
  if (route == FUSEDCONV_ROUTE_IGEMM_HALO) {
    p.workspace = ws;
    p.split_k = splits;
    snprintf(p.name, sizeof(p.name), "bwd_weight_taps_f16");
  } else if (route == FUSEDCONV_ROUTE_IM2COL) {
    p.workspace = ws;
    p.split_k = splits;
    snprintf(p.name, sizeof(p.name), "bwd_weight_gemm_%s", g.dtype == FUSEDCONV_F16 ? "f16" : "f32");
  } else {
    snprintf(p.name, sizeof(p.name), "bwd_weight_direct_%s", g.dtype == FUSEDCONV_F16 ? "f16" : "f32");
  }
  h->kind = kBackwardWeight;
  *out = h;
  clear_last_error();
  return FUSEDCONV_OK;
}

int fusedconv_backward_weight(const fusedconv_handle* h, const void* x, const void* dy,
                              float* dw, float* db, void* workspace, size_t workspace_bytes,
                              void* stream) {
  using namespace fc;
  if (!h || !x || !dy || !dw)
    return set_last_error(FUSEDCONV_ERR_NULL_ARG, "h, x, dy and dw are required");
  if (h->kind != kBackwardWeight)
    return set_last_error(FUSEDCONV_ERR_ROUTE, "not a fusedconv_create_backward_weight handle");
  if (h->has_db && !db) return set_last_error(FUSEDCONV_ERR_NULL_ARG, "db requested but NULL");
  if (!h->has_db && db)
    return set_last_error(FUSEDCONV_ERR_NULL_ARG, "db given but the bias gradient was not requested");
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dw) || (db && !aligned16(db)) ||
      (workspace && !aligned16(workspace)))
    return set_last_error(FUSEDCONV_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  if (h->plan.workspace > 0 && (!workspace || workspace_bytes < h->plan.workspace))
    return set_last_error(FUSEDCONV_ERR_WORKSPACE,
                          "workspace smaller than fusedconv_workspace_size() reports");
  int rc = check_device(stream);
  if (rc != FUSEDCONV_OK) return rc;
  (void)hipGetLastError();
  rc = launch_wgrad(h->geo, h->plan, x, dy, dw, db, workspace, stream);
  if (rc != FUSEDCONV_OK) {
    hipError_t e = hipGetLastError();
    return set_last_error(rc, std::string("kernel launch failed: ") + hipGetErrorString(e));
  }
  return FUSEDCONV_OK;
}

}  // extern "C"
