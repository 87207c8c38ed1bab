// The opaque handle behind fusedconv_handle (host memory only).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "internal.h"

namespace fc {

enum HandleKind : int32_t {
  kForward = 0,         // fusedconv_create / fusedconv_create_transposed
  kBackwardData = 1,    // fusedconv_create_backward_data
  kBackwardWeight = 2,  // fusedconv_create_backward_weight
};

// Checks shared by the entry points: the current device is a gfx950 GPU and
// a non-default stream belongs to it; 16-byte alignment of device pointers.
int check_device(void* stream);
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace fc

struct fusedconv_handle {
  fc::Geometry geo;     // the problem the planned kernels run
  fc::Plan plan;
  int32_t kind;         // fc::HandleKind
  fc::Geometry fwd;     // backward handles: the forward convolution
  size_t flip_bytes;    // backward data: flipped W at the workspace start (0: none)
  int32_t has_db;       // backward weight: the bias gradient is requested
};
