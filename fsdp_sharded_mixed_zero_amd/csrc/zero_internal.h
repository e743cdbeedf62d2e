// Internal declarations shared by the host partitioner (layout.cpp) and the
// device code (kernels.hip) of libzero_mi355x.so. Not part of the C ABI.
#pragma once

#include <cmath>
#include <cstdint>
#include <vector>

#include "zero.h"

struct zero_layout_s {
  std::vector<int64_t> sizes;
  std::vector<int64_t> offsets;  // flat offset of each tensor
  std::vector<zero_segment> segs;
  zero_layout_info info;
};

namespace zero {

// Record a message for zero_last_error() and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the calling thread's message and return ZERO_OK.
int ok();

// The hyperparameter checks of every update entry point (GPU and host):
// step >= 1, and the argument rules of PyTorch's AdamW (lr >= 0, eps >= 0,
// 0 <= beta1, beta2 < 1, weight_decay >= 0), plus clip_eps >= 0 and a
// max_norm that is a number (<= 0 turns clipping off). A NaN fails them all.
inline int check_adamw_hparams(const zero_adamw_hparams* hp, const char* who) {
  if (hp == nullptr) return fail(ZERO_EINVAL, "%s: NULL hyperparameters", who);
  if (hp->step < 1) return fail(ZERO_EINVAL, "%s: step must be >= 1 (got %lld)", who, (long long)hp->step);
  if (!(hp->lr >= 0.0)) return fail(ZERO_EINVAL, "%s: invalid learning rate %g", who, hp->lr);
  if (!(hp->eps >= 0.0)) return fail(ZERO_EINVAL, "%s: invalid eps %g", who, hp->eps);
  if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0)) return fail(ZERO_EINVAL, "%s: beta1 %g outside [0, 1)", who, hp->beta1);
  if (!(hp->beta2 >= 0.0 && hp->beta2 < 1.0)) return fail(ZERO_EINVAL, "%s: beta2 %g outside [0, 1)", who, hp->beta2);
  if (!(hp->weight_decay >= 0.0))
    return fail(ZERO_EINVAL, "%s: invalid weight decay %g", who, hp->weight_decay);
  if (!(hp->clip_eps >= 0.0)) return fail(ZERO_EINVAL, "%s: invalid clip_eps %g", who, hp->clip_eps);
  if (hp->max_norm != hp->max_norm) return fail(ZERO_EINVAL, "%s: max_norm is NaN", who);
  return ZERO_OK;
}

// The update's constants in fp64, formed from the hyperparameters and the
// 1-based step t as PyTorch's AdamW forms them: beta1, 1 - beta1, beta2,
// 1 - beta2, the decoupled-decay factor 1 - lr*wd, the step size
// lr / (1 - beta1^t), sqrt(1 - beta2^t) and eps. The exact recomputation of
// the GPU kernels and of the host update runs on these values.
struct AdamWExact {
  double beta1, omb1, beta2, omb2, decay, step_size, sqrt_bc2, eps;   // in this order, consecutive
};
static_assert(sizeof(AdamWExact) == 8 * sizeof(double), "AdamWExact holds eight consecutive doubles");

inline void adamw_exact_constants(const zero_adamw_hparams* hp, AdamWExact* x) {
  const double t = double(hp->step);
  x->beta1 = hp->beta1;
  x->omb1 = 1.0 - hp->beta1;
  x->beta2 = hp->beta2;
  x->omb2 = 1.0 - hp->beta2;
  x->decay = 1.0 - hp->lr * hp->weight_decay;
  x->step_size = hp->lr / (1.0 - std::pow(hp->beta1, t));
  x->sqrt_bc2 = std::sqrt(1.0 - std::pow(hp->beta2, t));
  x->eps = hp->eps;
}

}  // namespace zero
