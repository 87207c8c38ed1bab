// C ABI entry points (include/fusedconv.h).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <new>
#include <set>
#include <string>
#include <tuple>

#include "handle.h"
#include "internal.h"

namespace {

thread_local std::string t_last_error;

int set_err(int code, const std::string& msg) {
  t_last_error = msg;
  return code;
}

// Per-device "is gfx950" cache: 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_ok[kMaxDevices];

// The current device must be a gfx950 GPU, and a non-default stream must
// belong to it (kernels are launched for the current device).
int check_device(void* stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return set_err(FUSEDCONV_ERR_DEVICE, "no current HIP device");
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess)
      return set_err(FUSEDCONV_ERR_DEVICE, "hipStreamGetDevice failed for the given stream");
    if (sdev != dev)
      return set_err(FUSEDCONV_ERR_DEVICE, "the stream belongs to device " + std::to_string(sdev) +
                                               ", the current device is " + std::to_string(dev));
  }
  int st = g_dev_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
      return set_err(FUSEDCONV_ERR_DEVICE, "hipGetDeviceProperties failed");
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_ok[dev].store(st, std::memory_order_relaxed);
  }
  if (st != 1) return set_err(FUSEDCONV_ERR_DEVICE, "the current device is not a gfx950 GPU");
  return FUSEDCONV_OK;
}

using fc::aligned16;

}  // namespace

namespace fc {

int set_last_error(int code, const std::string& msg) { return set_err(code, msg); }

int check_device(void* stream) { return ::check_device(stream); }

// the calling thread's last-error text is cleared by a successful create
void clear_last_error() { t_last_error.clear(); }

int set_max_dynamic_lds(const void* kfn, int bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FUSEDCONV_ERR_LAUNCH;
  static std::mutex mu;
  static std::set<std::tuple<const void*, int, int>> done;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(kfn, dev, bytes);
  if (done.count(key)) return FUSEDCONV_OK;
  if (hipFuncSetAttribute(kfn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) != hipSuccess)
    return FUSEDCONV_ERR_LAUNCH;
  done.insert(key);
  return FUSEDCONV_OK;
}

}  // namespace fc

extern "C" {

void fusedconv_desc_init(fusedconv_desc* d) {
  if (!d) return;
  memset(d, 0, sizeof(*d));
  d->dtype = FUSEDCONV_F32;
  d->group = 1;
}

int fusedconv_create(const fusedconv_desc* d, fusedconv_handle** out) {
  if (out) *out = nullptr;
  if (!d || !out) return set_err(FUSEDCONV_ERR_NULL_ARG, "desc and out must not be NULL");
  fusedconv_handle* h = new (std::nothrow) fusedconv_handle();
  if (!h) return set_err(FUSEDCONV_ERR_ALLOC, "out of host memory");
  std::string err;
  int rc = fc::resolve(*d, h->geo, err);
  if (rc == FUSEDCONV_OK) rc = fc::make_plan(h->geo, d->route, d->split_k, h->plan, err);
  if (rc != FUSEDCONV_OK) {
    delete h;
    return set_err(rc, err);
  }
  *out = h;
  t_last_error.clear();
  return FUSEDCONV_OK;
}

int fusedconv_create_transposed(const fusedconv_desc* d, const int64_t* output_padding,
                                int32_t n_output_padding, fusedconv_handle** out) {
  if (out) *out = nullptr;
  if (!d || !out) return set_err(FUSEDCONV_ERR_NULL_ARG, "desc and out must not be NULL");
  fusedconv_handle* h = new (std::nothrow) fusedconv_handle();
  if (!h) return set_err(FUSEDCONV_ERR_ALLOC, "out of host memory");
  std::string err;
  int rc = fc::resolve_transposed(*d, output_padding, n_output_padding, h->geo, err);
  if (rc == FUSEDCONV_OK) rc = fc::make_plan(h->geo, d->route, d->split_k, h->plan, err);
  if (rc != FUSEDCONV_OK) {
    delete h;
    return set_err(rc, err);
  }
  *out = h;
  t_last_error.clear();
  return FUSEDCONV_OK;
}

int fusedconv_output_shape(const fusedconv_handle* h, int64_t dims[FUSEDCONV_MAX_RANK],
                           int32_t* rank) {
  if (!h || !dims || !rank) return set_err(FUSEDCONV_ERR_NULL_ARG, "NULL argument");
  *rank = h->geo.y_rank;
  for (int i = 0; i < FUSEDCONV_MAX_RANK; ++i) dims[i] = i < h->geo.y_rank ? h->geo.y_dims[i] : 0;
  return FUSEDCONV_OK;
}

int fusedconv_workspace_size(const fusedconv_handle* h, size_t* bytes) {
  if (!h || !bytes) return set_err(FUSEDCONV_ERR_NULL_ARG, "NULL argument");
  *bytes = h->plan.workspace;
  return FUSEDCONV_OK;
}

int fusedconv_plan_info(const fusedconv_handle* h, int32_t* route, int32_t* split_k, char* name,
                        size_t name_len) {
  if (!h) return set_err(FUSEDCONV_ERR_NULL_ARG, "NULL handle");
  if (route) *route = h->plan.route;
  if (split_k) *split_k = h->plan.split_k;
  if (name && name_len > 0) {
    strncpy(name, h->plan.name, name_len - 1);
    name[name_len - 1] = '\0';
  }
  return FUSEDCONV_OK;
}

int fusedconv_run(const fusedconv_handle* h, const void* x, const void* w, const void* bias,
                  const void* z, void* y, void* workspace, size_t workspace_bytes,
                  void* stream) {
  return fusedconv_run_ex(h, x, w, bias, z, y, workspace, workspace_bytes, 0u, stream);
}

int fusedconv_prepare_weights(const fusedconv_handle* h, const void* w, void* workspace,
                              size_t workspace_bytes, void* stream) {
  if (!h || !w) return set_err(FUSEDCONV_ERR_NULL_ARG, "h and w are required");
  if (h->kind != fc::kForward)
    return set_err(FUSEDCONV_ERR_ROUTE, "a backward handle: use fusedconv_backward_data / _weight");
  if (!aligned16(w) || (workspace && !aligned16(workspace)))
    return set_err(FUSEDCONV_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  if (h->plan.workspace > 0 && (!workspace || workspace_bytes < h->plan.workspace))
    return set_err(FUSEDCONV_ERR_WORKSPACE,
                   "workspace smaller than fusedconv_workspace_size() reports");
  const bool pw = h->plan.route == FUSEDCONV_ROUTE_POINTWISE ||
                  (h->plan.route == FUSEDCONV_ROUTE_TRANSPOSED && h->plan.tile == 1);
  const bool ic = h->plan.route == FUSEDCONV_ROUTE_IM2COL;
  if (h->plan.route != FUSEDCONV_ROUTE_IGEMM_HALO && h->plan.route != FUSEDCONV_ROUTE_SMALLC && !pw &&
      !ic)
    return FUSEDCONV_OK;
  int rc = check_device(stream);
  if (rc != FUSEDCONV_OK) return rc;
  (void)hipGetLastError();
  fc::RunArgs a{nullptr, w, nullptr, nullptr, nullptr, nullptr, workspace, stream, 0u};
  rc = h->plan.route == FUSEDCONV_ROUTE_SMALLC ? fc::prepare_smallc(h->geo, h->plan, a)
       : pw ? fc::prepare_pointwise(h->geo, h->plan, a)
       : ic ? fc::prepare_im2col(h->geo, h->plan, a)
            : fc::prepare_igemm_halo(h->geo, h->plan, a);
  if (rc != FUSEDCONV_OK) {
    hipError_t e = hipGetLastError();
    return set_err(rc, std::string("kernel launch failed: ") + hipGetErrorString(e));
  }
  return FUSEDCONV_OK;
}

int fusedconv_run_ex(const fusedconv_handle* h, const void* x, const void* w, const void* bias,
                     const void* z, void* y, void* workspace, size_t workspace_bytes,
                     unsigned flags, void* stream) {
  return fusedconv_run_timed(h, x, w, bias, z, y, workspace, workspace_bytes, flags, stream,
                             nullptr, nullptr);
}

int fusedconv_run_timed(const fusedconv_handle* h, const void* x, const void* w,
                        const void* bias, const void* z, void* y, void* workspace,
                        size_t workspace_bytes, unsigned flags, void* stream, void* start_event,
                        void* stop_event) {
  if (!h || !x || !w || !y) return set_err(FUSEDCONV_ERR_NULL_ARG, "h, x, w and y are required");
  if (h->kind != fc::kForward)
    return set_err(FUSEDCONV_ERR_ROUTE, "a backward handle: use fusedconv_backward_data / _weight");
  if (!start_event != !stop_event)
    return set_err(FUSEDCONV_ERR_NULL_ARG, "give both timing events or neither");
  const fc::ConvParams& cp = h->geo.cp;
  if (cp.has_bias && !bias) return set_err(FUSEDCONV_ERR_NULL_ARG, "bias declared but NULL");
  if (!cp.has_bias && bias)
    return set_err(FUSEDCONV_ERR_NULL_ARG, "bias given but not declared in the descriptor");
  if (cp.has_z && !z) return set_err(FUSEDCONV_ERR_NULL_ARG, "z declared but NULL");
  if (!cp.has_z && z) return set_err(FUSEDCONV_ERR_NULL_ARG, "z given but not declared");
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (bias && !aligned16(bias)) ||
      (z && !aligned16(z)) || (workspace && !aligned16(workspace)))
    return set_err(FUSEDCONV_ERR_ALIGNMENT, "device pointers must be 16-byte aligned");
  if (h->plan.workspace > 0 && (!workspace || workspace_bytes < h->plan.workspace))
    return set_err(FUSEDCONV_ERR_WORKSPACE,
                   "workspace smaller than fusedconv_workspace_size() reports");
  int rc = check_device(stream);
  if (rc != FUSEDCONV_OK) return rc;
  (void)hipGetLastError();  // drop a stale error so a launch failure is reported as ours
  if (flags & ~FUSEDCONV_RUN_WEIGHTS_PREPARED)
    return set_err(FUSEDCONV_ERR_ATTR_VALUE, "unknown run flags");
  fc::RunArgs a{x, w, bias, z, nullptr, y, workspace, stream, flags, start_event, stop_event};
  switch (h->plan.route) {
    case FUSEDCONV_ROUTE_DIRECT: rc = fc::launch_direct(h->geo, h->plan, a); break;
    case FUSEDCONV_ROUTE_IGEMM: rc = fc::launch_igemm(h->geo, h->plan, a); break;
    case FUSEDCONV_ROUTE_DEPTHWISE: rc = fc::launch_depthwise(h->geo, h->plan, a); break;
    case FUSEDCONV_ROUTE_IGEMM_HALO: rc = fc::launch_igemm_halo(h->geo, h->plan, a); break;
    case FUSEDCONV_ROUTE_SMALLC: rc = fc::launch_smallc(h->geo, h->plan, a); break;
    case FUSEDCONV_ROUTE_POINTWISE: rc = fc::launch_pointwise(h->geo, h->plan, a); break;
    case FUSEDCONV_ROUTE_TRANSPOSED: rc = fc::launch_transposed(h->geo, h->plan, a); break;
    case FUSEDCONV_ROUTE_IM2COL: rc = fc::launch_im2col(h->geo, h->plan, a); break;
    default: return set_err(FUSEDCONV_ERR_ROUTE, "handle has no route");
  }
  if (rc != FUSEDCONV_OK) {
    hipError_t e = hipGetLastError();
    return set_err(rc, std::string("kernel launch failed: ") + hipGetErrorString(e));
  }
  return FUSEDCONV_OK;
}

void fusedconv_destroy(fusedconv_handle* h) { delete h; }

const char* fusedconv_status_string(int status) {
  switch (status) {
    case FUSEDCONV_OK: return "ok";
    case FUSEDCONV_ERR_NULL_ARG: return "null argument";
    case FUSEDCONV_ERR_DTYPE: return "unsupported dtype";
    case FUSEDCONV_ERR_RANK: return "bad rank";
    case FUSEDCONV_ERR_ATTR_LENGTH: return "bad attribute length";
    case FUSEDCONV_ERR_ATTR_VALUE: return "bad attribute value";
    case FUSEDCONV_ERR_PADS_WITH_AUTO_PAD: return "pads given with auto_pad";
    case FUSEDCONV_ERR_KERNEL_SHAPE: return "kernel_shape does not match w";
    case FUSEDCONV_ERR_GROUP: return "bad group";
    case FUSEDCONV_ERR_BIAS_SHAPE: return "bad bias shape";
    case FUSEDCONV_ERR_Z_SHAPE: return "bad residual shape";
    case FUSEDCONV_ERR_ACTIVATION: return "unknown activation";
    case FUSEDCONV_ERR_ACTIVATION_PARAMS: return "bad activation parameters";
    case FUSEDCONV_ERR_OUTPUT_SHAPE: return "bad output shape";
    case FUSEDCONV_ERR_WORKSPACE: return "workspace too small";
    case FUSEDCONV_ERR_ALIGNMENT: return "misaligned pointer";
    case FUSEDCONV_ERR_ROUTE: return "route cannot run this problem";
    case FUSEDCONV_ERR_LAUNCH: return "launch failed";
    case FUSEDCONV_ERR_DEVICE: return "unsupported device";
    case FUSEDCONV_ERR_ALLOC: return "host allocation failed";
    case FUSEDCONV_ERR_TOO_LARGE: return "tensor too large";
    default: return "unknown status";
  }
}

const char* fusedconv_last_error(void) { return t_last_error.c_str(); }

}  // extern "C"
