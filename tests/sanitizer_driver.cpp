// Host-side sweep run under AddressSanitizer and UndefinedBehaviorSanitizer
// (built by tests/test_sanitizers_cpu.py): the library's resolver, planner
// and C ABI on seeded descriptors, valid and invalid, with no GPU call
// (create, output shape, workspace size, plan info, destroy, for the
// forward, transposed and backward handles), and the oracle's C loop nest on
// tiny problems whose buffers are allocated at exactly their sizes.
// Prints one line per category and exits 0; a sanitizer finding aborts.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "fusedconv.h"

extern "C" {
int oracle_output_dims(int nsp, const int64_t* in, const int64_t* k, const int64_t* strides,
                       const int64_t* dilations, int mode, const int64_t* pads, int64_t* out,
                       int64_t* pad_begin);
int oracle_fusedconv(int nsp, const int64_t* xs, const int64_t* ws, const double* x,
                     const double* w, const double* b, const double* z, int64_t group,
                     const int64_t* strides, const int64_t* dilations, int mode,
                     const int64_t* pads, int act, const double* params, int n_params,
                     int64_t n0, int64_t n1, double* y);
}

namespace {

uint64_t g_state = 0x9e3779b97f4a7c15ull;
uint32_t rnd() {  // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (uint32_t)((g_state * 0x2545f4914f6cdd1dull) >> 32);
}
int64_t pick(int64_t lo, int64_t hi) { return lo + (int64_t)(rnd() % (uint32_t)(hi - lo + 1)); }

const char* kActs[] = {nullptr, "Relu", "LeakyRelu", "Sigmoid", "Tanh", "HardSigmoid",
                       "HardSwish", "Clip", "QuickGelu", "Elu", "Gelu", "FastGelu",
                       "Softplus", "ThresholdedRelu", "Erf", "NotAnActivation"};
const char* kPads[] = {nullptr, "NOTSET", "SAME_UPPER", "SAME_LOWER", "VALID", "BOGUS"};

struct Case {
  fusedconv_desc d;
  int64_t ks[3], st[3], dl[3], pd[6], op[3];
  float ap[3];
  int64_t kshape[3];
};

// A descriptor with shapes that are usually valid; `mess` breaks one thing.
void make_case(Case& c, int mess) {
  fusedconv_desc_init(&c.d);
  const int nsp = (int)pick(1, 3);
  const int64_t group = pick(1, 4);
  const int64_t cg = pick(1, 40), mg = pick(1, 40);
  c.d.dtype = rnd() % 2 ? FUSEDCONV_F16 : FUSEDCONV_F32;
  c.d.x.present = 1;
  c.d.x.rank = nsp + 2;
  c.d.x.dims[0] = pick(1, 3);
  c.d.x.dims[1] = cg * group;
  c.d.w.present = 1;
  c.d.w.rank = nsp + 2;
  c.d.w.dims[0] = mg * group;
  c.d.w.dims[1] = cg;
  for (int i = 0; i < nsp; ++i) {
    c.ks[i] = pick(1, 5);
    c.st[i] = pick(1, 4);
    c.dl[i] = pick(1, 3);
    c.d.x.dims[2 + i] = pick(1, nsp == 3 ? 12 : 40);
    c.d.w.dims[2 + i] = c.ks[i];
    c.pd[i] = pick(0, 3);
    c.pd[nsp + i] = pick(0, 3);
    c.op[i] = pick(0, 2);
    c.kshape[i] = c.ks[i];
  }
  c.d.group = group;
  if (rnd() % 2) { c.d.strides = c.st; c.d.n_strides = nsp; }
  if (rnd() % 2) { c.d.dilations = c.dl; c.d.n_dilations = nsp; }
  c.d.auto_pad = kPads[rnd() % 5];
  if ((!c.d.auto_pad || !strcmp(c.d.auto_pad, "NOTSET")) && rnd() % 2) {
    c.d.pads = c.pd;
    c.d.n_pads = 2 * nsp;
  }
  if (rnd() % 3 == 0) { c.d.kernel_shape = c.kshape; c.d.n_kernel_shape = nsp; }
  const int a = (int)(rnd() % 15);
  c.d.activation = kActs[a];
  c.ap[0] = 0.5f; c.ap[1] = 1.5f; c.ap[2] = 0.25f;
  if (a == 2 || a == 9 || a == 13 || a == 8 || a == 10) { c.d.activation_params = c.ap; c.d.n_activation_params = 1; }
  if (a == 5 || a == 7) { c.d.activation_params = c.ap; c.d.n_activation_params = 2; }
  if (rnd() % 2) {
    c.d.bias.present = 1;
    c.d.bias.rank = 1;
    c.d.bias.dims[0] = c.d.w.dims[0];
  }
  c.d.route = rnd() % 2 ? 0 : (int32_t)(rnd() % 9);  // half the planner's choice, half forced
  c.d.split_k = rnd() % 3 == 0 ? (int32_t)pick(1, 9) : 0;
  switch (mess) {
    case 1: c.d.x.rank = nsp + 3; break;
    case 2: c.d.w.dims[1] += 1; break;
    case 3: if (c.d.strides) c.st[0] = 0; else c.d.group = 0; break;
    case 4: c.d.pads = c.pd; c.d.n_pads = 2 * nsp - 1; break;
    case 5: c.d.activation = kActs[15]; break;
    case 6: c.d.auto_pad = kPads[5]; break;
    case 7: c.d.activation = "Clip"; c.d.activation_params = c.ap; c.d.n_activation_params = 3; break;
    case 8: c.d.x.dims[2] = 0; break;
    default: break;
  }
}

// The queries a created handle answers: output shape, workspace size, plan info.
void probe(fusedconv_handle* h, int& ok_shapes) {
  int64_t dims[FUSEDCONV_MAX_RANK];
  int32_t rank = 0, route = 0, split = 0;
  size_t ws = 0;
  char name[64];
  if (fusedconv_output_shape(h, dims, &rank) == FUSEDCONV_OK && rank >= 3) ++ok_shapes;
  fusedconv_workspace_size(h, &ws);
  fusedconv_plan_info(h, &route, &split, name, (int32_t)sizeof(name));
}

}  // namespace

int main(int argc, char** argv) {
  const int n = argc > 1 ? atoi(argv[1]) : 4000;
  int created = 0, rejected = 0, shapes = 0, tcreated = 0, bcreated = 0;
  for (int i = 0; i < n; ++i) {
    Case c;
    make_case(c, (int)(rnd() % 12));  // 8 of 12 cases are left intact
    fusedconv_handle* h = nullptr;
    int rc = fusedconv_create(&c.d, &h);
    if (rc == FUSEDCONV_OK) {
      ++created;
      probe(h, shapes);
      // a residual of Y's shape, then the same problem again with it
      int64_t dims[FUSEDCONV_MAX_RANK];
      int32_t rank = 0;
      if (fusedconv_output_shape(h, dims, &rank) == FUSEDCONV_OK) {
        fusedconv_desc d2 = c.d;
        d2.z.present = 1;
        d2.z.rank = rank;
        memcpy(d2.z.dims, dims, sizeof(int64_t) * rank);
        fusedconv_handle* h2 = nullptr;
        if (fusedconv_create(&d2, &h2) == FUSEDCONV_OK) {
          probe(h2, shapes);
          fusedconv_destroy(h2);
        }
        // backward handles of the same problem (no bias for the input gradient)
        d2.bias.present = 0;
        d2.z = c.d.x;
        d2.route = 0;
        if (fusedconv_create_backward_data(&d2, &h2) == FUSEDCONV_OK) {
          ++bcreated;
          probe(h2, shapes);
          fusedconv_destroy(h2);
        }
        fusedconv_desc d3 = c.d;
        d3.route = 0;
        d3.z.present = 0;
        if (fusedconv_create_backward_weight(&d3, &h2) == FUSEDCONV_OK) {
          ++bcreated;
          probe(h2, shapes);
          fusedconv_destroy(h2);
        }
      }
      fusedconv_destroy(h);
    } else {
      ++rejected;
      (void)fusedconv_status_string(rc);
      (void)fusedconv_last_error();
    }
    // the transposed form: W is [C, M/group, k...], output_padding per axis
    fusedconv_desc t = c.d;
    t.w.dims[0] = c.d.x.dims[1];
    t.w.dims[1] = c.d.w.dims[0] / (c.d.group > 0 ? c.d.group : 1);
    t.kernel_shape = nullptr;
    t.n_kernel_shape = 0;
    t.route = 0;
    if (fusedconv_create_transposed(&t, (rnd() % 2) ? c.op : nullptr, c.d.x.rank - 2, &h) ==
        FUSEDCONV_OK) {
      ++tcreated;
      probe(h, shapes);
      fusedconv_destroy(h);
    }
  }
  printf("library: %d created, %d rejected, %d transposed, %d backward, %d shapes\n", created,
         rejected, tcreated, bcreated, shapes);

  // the oracle on tiny problems, buffers of exactly the sizes it may touch
  int oracle_runs = 0;
  for (int i = 0; i < n / 20; ++i) {
    const int nsp = (int)pick(1, 3);
    const int64_t group = pick(1, 2), cg = pick(1, 3), mg = pick(1, 3);
    int64_t xs[5], ws[5], st[3], dl[3], pd[6], in[3], k[3], out[3], pb[3];
    xs[0] = pick(1, 2); xs[1] = cg * group;
    ws[0] = mg * group; ws[1] = cg;
    for (int a = 0; a < nsp; ++a) {
      k[a] = ws[2 + a] = pick(1, 3);
      st[a] = pick(1, 3);
      dl[a] = pick(1, 2);
      in[a] = xs[2 + a] = pick(1, 7);
      pd[a] = pick(0, 2);
      pd[nsp + a] = pick(0, 2);
    }
    const int mode = (int)(rnd() % 4);
    if (oracle_output_dims(nsp, in, k, st, dl, mode, pd, out, pb) != 0) continue;
    int64_t xn = xs[0] * xs[1], wn = ws[0] * ws[1], yn = xs[0] * ws[0];
    for (int a = 0; a < nsp; ++a) { xn *= in[a]; wn *= k[a]; yn *= out[a]; }
    std::vector<double> x(xn), w(wn), b(ws[0]), z(yn), y(yn);
    for (auto& v : x) v = (double)(int)(rnd() % 7) - 3.0;
    for (auto& v : w) v = (double)(int)(rnd() % 5) - 2.0;
    for (auto& v : b) v = 0.5;
    for (auto& v : z) v = -0.25;
    const double prm[2] = {0.2, 0.5};
    const int act = (int)(rnd() % 15);
    if (oracle_fusedconv(nsp, xs, ws, x.data(), w.data(), rnd() % 2 ? b.data() : nullptr,
                         rnd() % 2 ? z.data() : nullptr, group, st, dl, mode, pd, act, prm, 2, 0,
                         xs[0], y.data()) == 0)
      ++oracle_runs;
  }
  printf("oracle: %d runs\n", oracle_runs);
  return 0;
}
