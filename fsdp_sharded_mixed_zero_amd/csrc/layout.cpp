// Host-side partitioner of libzero_mi355x.so: per-tensor size list -> flat
// buffer -> one rank's shard (segments + tail padding) and the per-rank byte
// and communication report.
//
// Sources: notes on "ZeRO: Memory Optimizations Toward Training Trillion
// Parameter Models", sections 2.2 and 5.2 (tensors flattened and fused into a
// contiguous buffer), 4.1-4.3 (state split into N_d equal parts, rank i owns
// part i) and 6 (communication volume); "第 5 课：ZeRO 与 FSDP", sections 2
// (per-rank bytes of each stage, fp32 accumulation note) and 3 (2 Psi / 3 Psi).
// Padding is not on the pages: the buffer is padded at the tail to a multiple
// of n_d * align so every rank owns the same number of elements.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "zero_internal.h"

namespace zero {

static thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return ZERO_OK;
}

static bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }
static bool add_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_add_overflow(a, b, out); }

}  // namespace zero

using zero::fail;

extern "C" const char* zero_last_error(void) { return zero::g_last_error.c_str(); }

extern "C" int zero_layout(const int64_t* sizes, int32_t n_tensors, int32_t n_d, int32_t rank,
                           int64_t align_elems, zero_layout_t* out) {
  if (out == nullptr) return fail(ZERO_EINVAL, "zero_layout: out is NULL");
  *out = nullptr;
  if (sizes == nullptr) return fail(ZERO_EINVAL, "zero_layout: sizes is NULL");
  if (n_tensors < 1) return fail(ZERO_EINVAL, "zero_layout: n_tensors must be >= 1 (got %d)", n_tensors);
  if (n_d < 1) return fail(ZERO_EINVAL, "zero_layout: n_d must be >= 1 (got %d)", n_d);
  if (rank < 0 || rank >= n_d)
    return fail(ZERO_EINVAL, "zero_layout: rank %d outside [0, %d)", rank, n_d);
  if (align_elems < 1) return fail(ZERO_EINVAL, "zero_layout: align_elems must be >= 1");

  zero_layout_s* h = new (std::nothrow) zero_layout_s;
  if (h == nullptr) return fail(ZERO_ENOMEM, "zero_layout: out of host memory");
  try {
    h->sizes.assign(sizes, sizes + n_tensors);
    h->offsets.resize(n_tensors);
  } catch (...) {
    delete h;
    return fail(ZERO_ENOMEM, "zero_layout: out of host memory");
  }

  int64_t psi = 0;
  for (int32_t i = 0; i < n_tensors; ++i) {
    if (sizes[i] < 0) {
      delete h;
      return fail(ZERO_EINVAL, "zero_layout: size of tensor %d is negative", i);
    }
    h->offsets[i] = psi;
    if (!zero::add_ok(psi, sizes[i], &psi)) {
      delete h;
      return fail(ZERO_EINVAL, "zero_layout: total size overflows int64");
    }
  }
  if (psi == 0) {
    delete h;
    return fail(ZERO_EINVAL, "zero_layout: the tensors hold no elements");
  }

  int64_t quantum = 0, padded = 0;
  if (!zero::mul_ok(n_d, align_elems, &quantum) ||
      !zero::mul_ok((psi - 1) / quantum + 1, quantum, &padded)) {
    delete h;
    return fail(ZERO_EINVAL, "zero_layout: padded size overflows int64");
  }
  const int64_t shard = padded / n_d;
  const int64_t lo_rank = int64_t(rank) * shard;
  const int64_t hi_rank = lo_rank + shard;

  // byte report: 16*max(psi, shard)+4*... must fit in int64
  int64_t probe = 0;
  if (!zero::mul_ok(padded, 20, &probe)) {
    delete h;
    return fail(ZERO_EINVAL, "zero_layout: byte report overflows int64");
  }

  // The tensors are sorted by flat offset, so the ones that meet the shard
  // form one contiguous run: find its first member by binary search.
  const auto& off = h->offsets;
  int32_t first = int32_t(std::upper_bound(off.begin(), off.end(), lo_rank) - off.begin()) - 1;
  if (first < 0) first = 0;
  try {
    for (int32_t i = first; i < n_tensors && off[i] < hi_rank; ++i) {
      const int64_t lo = std::max(off[i], lo_rank);
      const int64_t hi = std::min(off[i] + sizes[i], hi_rank);
      if (lo < hi) h->segs.push_back(zero_segment{i, lo - off[i], lo - lo_rank, hi - lo});
    }
  } catch (...) {
    delete h;
    return fail(ZERO_ENOMEM, "zero_layout: out of host memory");
  }

  zero_layout_info& f = h->info;
  std::memset(&f, 0, sizeof f);
  f.n_tensors = n_tensors;
  f.n_d = n_d;
  f.rank = rank;
  f.align = align_elems;
  f.psi = psi;
  f.padded = padded;
  f.shard = shard;
  f.shard_begin = lo_rank;
  f.n_segments = int64_t(h->segs.size());
  const int64_t pad_lo = std::max(psi, lo_rank);
  if (pad_lo < hi_rank) {
    f.pad_begin = pad_lo - lo_rank;
    f.pad_end = shard;
  } else {
    f.pad_begin = f.pad_end = shard;
  }

  // Model-state bytes: 2 B params, 2 B grads, 12 B optimizer per element;
  // stage s splits the optimizer (s>=1), grads (s>=2), params (s>=3).
  for (int s = 0; s < 4; ++s) {
    const int64_t params = 2 * (s >= 3 ? shard : psi);
    const int64_t grads = 2 * (s >= 2 ? shard : psi);
    const int64_t optim = 12 * (s >= 1 ? shard : psi);
    f.bytes_stage[s] = params + grads + optim;
    f.bytes_stage_fp32acc[s] = f.bytes_stage[s] + 4 * (s >= 2 ? shard : psi);
    f.comm_pages[s] = (s == 3 ? 3 : 2) * psi;
    f.comm_exact[s] = (s == 3 ? 3 : 2) * int64_t(n_d - 1) * shard;
  }

  *out = h;
  return zero::ok();
}

extern "C" int zero_layout_query(zero_layout_t h, zero_layout_info* info) {
  if (h == nullptr || info == nullptr) return fail(ZERO_EINVAL, "zero_layout_query: NULL argument");
  *info = h->info;
  return zero::ok();
}

extern "C" int zero_layout_segments(zero_layout_t h, zero_segment* segs, int64_t cap, int64_t* n_out) {
  if (h == nullptr || n_out == nullptr) return fail(ZERO_EINVAL, "zero_layout_segments: NULL argument");
  if (cap < 0) return fail(ZERO_EINVAL, "zero_layout_segments: cap < 0");
  if (cap > 0 && segs == nullptr) return fail(ZERO_EINVAL, "zero_layout_segments: segs is NULL");
  const int64_t n = int64_t(h->segs.size());
  const int64_t k = std::min(n, cap);
  if (k > 0) std::memcpy(segs, h->segs.data(), size_t(k) * sizeof(zero_segment));
  *n_out = n;
  return zero::ok();
}

extern "C" void zero_layout_free(zero_layout_t h) { delete h; }
