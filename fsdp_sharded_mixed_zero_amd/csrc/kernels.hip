// Device code and device-side C ABI of libzero_mi355x.so (gfx950 / CDNA4).
//
// Every kernel here streams HBM; none is a dense contraction, so none uses
// the matrix cores. They are written for 64-lane wavefronts and one rule
// measured on MI355X: every wavefront-wide memory instruction covers one
// contiguous span (lane k takes the k-th 8 or 16 bytes), and the grid is
// one-shot (one unit of work per lane, blocks dispatched in address order),
// so the waves in flight at any moment touch a compact window of each stream.
// Persistent grid-stride loops and lanes that own 32 contiguous bytes (two
// half-filled instructions per stream) both measured 10-20% slower. Loads and
// stores are non-temporal: nothing is reused within a step (the update's
// loads also carry device scope, see "stream loads").
//
//   copy_pieces_kernel<SQ>    pack (tensors -> shard) and unpack (shard ->
//                             tensors); with SQ the pack also sums squares
//   sqnorm_partial_kernel, sqnorm_f32_partial_kernel, sqnorm_final_kernel,
//   sum_rows_kernel           deterministic two-stage sum of squares (fp64);
//                             rows: the final stage of many buckets at once
//   adamw_vec_kernel, adamw_elem_kernel
//                             clip + AdamW + bf16 cast, 28 bytes per element
//   adamw_unpack_vec_kernel, adamw_unpack_elem_kernel
//                             the same, also storing each bf16 parameter at its
//                             tensor position (30 bytes per element)
//   adamw_arrays_vec_kernel, adamw_arrays_elem_kernel
//                             the update over three separate state arrays
//   accumulate_kernel         fp32 gradient accumulation over micro-batches
//   state_convert_kernel      three fp32 arrays <-> the tiled state buffer
//
// Sources for what is computed: "第 5 课：ZeRO 与 FSDP" sections 2-3, notes on
// "ZeRO: Memory Optimizations Toward Training Trillion Parameter Models"
// sections 2.1, 2.2, 3.2.3, 4.1-4.3, 5.2, and "ZeRO-3 核心流程" pitfall 1.
// The update rule and clip coefficient follow PyTorch's AdamW and
// clip_grad_norm_, the pages giving no equations of their own.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <mutex>
#include <vector>

#include "zero_internal.h"

using zero::fail;

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ float bf16_lo(unsigned int w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned int w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even (gfx950 has a hardware convert).
__device__ __forceinline__ unsigned int pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 r = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(unsigned int, r);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// Sum of squares of the 8 bf16 values in a 16-byte word, each square exact in fp64.
__device__ __forceinline__ double sq8(u32x4 w, double acc) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const double a = double(bf16_lo(w[k]));
    const double b = double(bf16_hi(w[k]));
    acc = fma(a, a, acc);
    acc = fma(b, b, acc);
  }
  return acc;
}

// Fixed-order block sum of one double per thread; result valid in thread 0.
// Every thread of the block must call it (it synchronises the block).
template <int THREADS>
__device__ __forceinline__ double block_sum(double x) {
  __shared__ double lds[THREADS / 64];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds[wave] = x;
  __syncthreads();
  double s = 0.0;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 0; w < THREADS / 64; ++w) s += lds[w];
  }
  return s;
}

// ============================================================ pack / unpack
//
// One launch copies up to kCopyMaxPieces contiguous runs ("pieces"). The
// pieces travel in the kernel-argument segment, so no table has to be
// uploaded per call. Blocks are dealt out to pieces by a prefix table; a
// piece whose source and destination have the same address modulo 16 uses
// 16-byte vectors (with a scalar head and tail), any other piece an element
// path. A NULL source writes zeros (padding).
//
// Each wave finds its piece from a 256-entry slot table (the piece holding
// the first block of each run of 2^slot_shift blocks) and a short forward
// step, two or three dependent scalar loads. A binary search over the prefix
// table is a chain of about log2(pieces) + 1 such loads, and on waves that
// live for one load and one store that latency costs 2-3% of the copy rate.

constexpr int kCopyMaxPieces = ZERO_PIECES_PER_LAUNCH;
constexpr int kCopyThreads = 256;      // plain copy: one 16-byte vector per lane
constexpr int kCopySqThreads = 512;    // copy + sum of squares: 2 vectors per lane keep more loads in flight
constexpr int kCopyVecPerThread = 1;
constexpr int kCopySqVecPerThread = 2;
constexpr int64_t kCopyVecPerBlock = int64_t(kCopyThreads) * kCopyVecPerThread;
constexpr int64_t kCopySqVecPerBlock = int64_t(kCopySqThreads) * kCopySqVecPerThread;
constexpr int64_t kCopySqElemPerBlock = kCopySqVecPerBlock * 8;

constexpr int kCopySlots = 256;

struct CopyPieces {
  int32_t n;
  int32_t slot_shift;                        // block b lies in slot b >> slot_shift
  uint64_t vec_mask;                         // bit p: piece p takes the vector path
  int64_t first_block[kCopyMaxPieces + 1];   // prefix of blocks per piece
  uint8_t slot_piece[kCopySlots];            // piece holding the slot's first block
  const uint16_t* src[kCopyMaxPieces];       // NULL: write zeros
  uint16_t* dst[kCopyMaxPieces];
  int64_t len[kCopyMaxPieces];
};
static_assert(kCopyMaxPieces <= 256, "slot_piece holds piece indices in one byte");
static_assert(sizeof(CopyPieces) + sizeof(double*) <= 4096, "kernel arguments fit the 4 KiB segment");

__host__ __device__ inline int64_t copy_head(const void* dst, int64_t len) {
  // elements before dst reaches a 16-byte boundary (dst is 2-byte aligned)
  const int64_t h = int64_t(((16u - (uintptr_t(dst) & 15u)) & 15u) >> 1);
  return h < len ? h : len;
}

// Blocks that a piece of `len` elements at `dst` needs when a block covers
// per_block 16-byte vectors (or per_block * 8 elements on the element path).
__host__ __device__ inline int64_t copy_blocks(const void* dst, int64_t len, bool vec, int64_t per_block) {
  if (vec) {
    const int64_t nvec = (len - copy_head(dst, len)) >> 3;
    const int64_t b = (nvec + per_block - 1) / per_block;
    return b > 0 ? b : 1;
  }
  const int64_t b = (len + per_block * 8 - 1) / (per_block * 8);
  return b > 0 ? b : 1;
}

__device__ __forceinline__ double sq1(uint16_t h, double acc) {
  const double x = double(__uint_as_float(uint32_t(h) << 16));
  return fma(x, x, acc);
}

// SQ: also sum the squares of the values copied (fp64) and write one partial
// per block to partial[blockIdx.x].
template <bool SQ>
__global__ __launch_bounds__(SQ ? kCopySqThreads : kCopyThreads) void copy_pieces_kernel(
    const CopyPieces P, double* __restrict__ partial) {
  constexpr int THREADS = SQ ? kCopySqThreads : kCopyThreads;
  constexpr int VPT = SQ ? kCopySqVecPerThread : kCopyVecPerThread;
  constexpr int64_t VEC_PER_BLOCK = int64_t(THREADS) * VPT;
  const int64_t b = blockIdx.x;
  // the piece this block serves: the last p with first_block[p] <= b. The
  // slot's entry is at most that p, and first_block[n] (the block count)
  // exceeds b, so the walk ends on a piece of this launch.
  int p = P.slot_piece[b >> P.slot_shift];
  while (P.first_block[p + 1] <= b) ++p;
  const int64_t lb = b - P.first_block[p];
  const uint16_t* __restrict__ src = P.src[p];
  uint16_t* __restrict__ dst = P.dst[p];
  const int64_t len = P.len[p];
  const int t = threadIdx.x;
  double acc = 0.0;

  if ((P.vec_mask >> p) & 1u) {
    const int64_t head = copy_head(dst, len);
    const int64_t nvec = (len - head) >> 3;
    const int64_t tail0 = head + nvec * 8;
    if (lb == 0) {
      if (t < head) {
        const uint16_t x = src ? src[t] : uint16_t(0);
        dst[t] = x;
        if (SQ) acc = sq1(x, acc);
      }
      const int64_t k = tail0 + (t - 8);
      if (t >= 8 && k < len) {
        const uint16_t x = src ? src[k] : uint16_t(0);
        dst[k] = x;
        if (SQ) acc = sq1(x, acc);
      }
    }
    const u32x4* __restrict__ s = reinterpret_cast<const u32x4*>(src + head);
    u32x4* __restrict__ d = reinterpret_cast<u32x4*>(dst + head);
    const int64_t base = lb * VEC_PER_BLOCK + t;
    u32x4 r[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int64_t i = base + int64_t(k) * THREADS;
      r[k] = (src && i < nvec) ? __builtin_nontemporal_load(s + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int64_t i = base + int64_t(k) * THREADS;
      if (i < nvec) __builtin_nontemporal_store(r[k], d + i);
      if (SQ) acc = sq8(r[k], acc);   // zero vectors past the end add nothing
    }
  } else {
    const int64_t base = lb * VEC_PER_BLOCK * 8 + t;
    constexpr int kPer = VPT * 8;
#pragma unroll 8
    for (int k = 0; k < kPer; ++k) {
      const int64_t i = base + int64_t(k) * THREADS;
      if (i < len) {
        const uint16_t x = src ? src[i] : uint16_t(0);
        dst[i] = x;
        if (SQ) acc = sq1(x, acc);
      }
    }
  }
  if (SQ) {
    const double s = block_sum<THREADS>(acc);
    if (t == 0) partial[blockIdx.x] = s;
  }
}

struct Piece {
  const uint16_t* src;
  uint16_t* dst;
  int64_t len;
};

// A launch's work-item count must fit in 32 bits: at most 2^31 lanes, so
// 2^23 blocks of the plain copy and 2^22 of the copy with the sum of squares.
constexpr int64_t kCopyMaxLanesPerLaunch = int64_t(1) << 31;
// Pieces are cut to at most 2^34 elements (2^23 plain-copy blocks, 2^21 with
// the sum of squares) so any piece fits one launch.
constexpr int64_t kCopyMaxPieceElems = int64_t(1) << 34;
static_assert(kCopyMaxPieceElems / (kCopyVecPerBlock * 8) <= kCopyMaxLanesPerLaunch / kCopyThreads &&
                  kCopyMaxPieceElems / kCopySqElemPerBlock <= kCopyMaxLanesPerLaunch / kCopySqThreads,
              "a piece of the maximum length fits one launch");

// Launches copying `pieces`, batched by kCopyMaxPieces and by the block limit.
// With `partial` non-NULL the sum-of-squares variant runs and each block writes
// partial[k] (k counts blocks across all launches); *n_partial gets the count.
int launch_pieces(const Piece* pieces, size_t n_pieces, hipStream_t stream, const char* who,
                  double* partial = nullptr, int64_t* n_partial = nullptr) {
  const int64_t per_block = partial ? kCopySqVecPerBlock : kCopyVecPerBlock;
  const int64_t max_blocks = kCopyMaxLanesPerLaunch / (partial ? kCopySqThreads : kCopyThreads);
  size_t i = 0;
  int64_t done = 0;
  while (i < n_pieces) {
    CopyPieces P{};
    int64_t blocks = 0;
    int n = 0;
    for (; i < n_pieces && n < kCopyMaxPieces; ++i, ++n) {
      const Piece& pc = pieces[i];
      const bool vec = pc.src == nullptr ||
                       ((uintptr_t(pc.src) & 15u) == (uintptr_t(pc.dst) & 15u));
      const int64_t nb = copy_blocks(pc.dst, pc.len, vec, per_block);
      if (n > 0 && blocks + nb > max_blocks) break;  // launch what we have first
      P.src[n] = pc.src;
      P.dst[n] = pc.dst;
      P.len[n] = pc.len;
      if (vec) P.vec_mask |= uint64_t(1) << n;
      P.first_block[n] = blocks;
      blocks += nb;
    }
    P.n = n;
    P.first_block[n] = blocks;
    if (blocks > max_blocks) return fail(ZERO_EINVAL, "%s: piece too large for one launch", who);
    // slot table: the smallest power-of-two run of blocks that needs at most
    // kCopySlots slots, and for each slot the piece holding its first block
    int shift = 0;
    while (((blocks + (int64_t(1) << shift) - 1) >> shift) > kCopySlots) ++shift;
    P.slot_shift = shift;
    for (int q = 0, slot = 0; slot < kCopySlots; ++slot) {
      const int64_t first = int64_t(slot) << shift;
      while (q + 1 < n && P.first_block[q + 1] <= first) ++q;
      P.slot_piece[slot] = uint8_t(q);
    }
    if (partial)
      hipLaunchKernelGGL(copy_pieces_kernel<true>, dim3(unsigned(blocks)), dim3(kCopySqThreads), 0, stream, P,
                         partial + done);
    else
      hipLaunchKernelGGL(copy_pieces_kernel<false>, dim3(unsigned(blocks)), dim3(kCopyThreads), 0, stream, P,
                         nullptr);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
    done += blocks;
  }
  if (n_partial) *n_partial = done;
  return zero::ok();
}

int launch_pieces(const std::vector<Piece>& pieces, hipStream_t stream, const char* who,
                  double* partial = nullptr, int64_t* n_partial = nullptr) {
  return launch_pieces(pieces.data(), pieces.size(), stream, who, partial, n_partial);
}

// Upper bound of the blocks the sum-of-squares copy uses for pieces of these
// lengths: ceil(len / elements per block) + 1 each, whatever the alignment.
int64_t pieces_block_bound(const std::vector<int64_t>& lens) {
  int64_t b = 0;
  for (int64_t len : lens) b += (len + kCopySqElemPerBlock - 1) / kCopySqElemPerBlock + 1;
  return b;
}

// Pieces of shard range [begin, begin+count): one per segment overlap, plus
// the padding overlap. `to_shard` selects pack (tensor -> shard) or unpack.
int build_pieces(const zero_layout_s* h, uint16_t* const* tensors, uint16_t* shard, int64_t begin,
                 int64_t count, bool to_shard, std::vector<Piece>* out, const char* who) {
  const int64_t end = begin + count;
  const auto& segs = h->segs;
  // segments are sorted by dst_off: skip to the first that ends after begin
  size_t s = size_t(std::upper_bound(segs.begin(), segs.end(), begin,
                                     [](int64_t v, const zero_segment& g) { return v < g.dst_off + g.len; }) -
                    segs.begin());
  for (; s < segs.size() && segs[s].dst_off < end; ++s) {
    const zero_segment& g = segs[s];
    const int64_t lo = std::max(g.dst_off, begin);
    const int64_t hi = std::min(g.dst_off + g.len, end);
    if (lo >= hi) continue;
    uint16_t* t = tensors[g.tensor];
    if (t == nullptr)
      return fail(ZERO_EINVAL, "%s: pointer of tensor %lld is NULL but the range needs it", who,
                  (long long)g.tensor);
    if (uintptr_t(t) & 1u) return fail(ZERO_EINVAL, "%s: tensor %lld pointer is not 2-byte aligned", who,
                                       (long long)g.tensor);
    for (int64_t a = lo; a < hi; a += kCopyMaxPieceElems) {
      const int64_t n = std::min(kCopyMaxPieceElems, hi - a);
      uint16_t* tp = t + g.src_off + (a - g.dst_off);
      uint16_t* sp = shard + a;
      out->push_back(to_shard ? Piece{tp, sp, n} : Piece{sp, tp, n});
    }
  }
  if (to_shard) {
    const int64_t lo = std::max(h->info.pad_begin, begin);
    const int64_t hi = std::min(h->info.pad_end, end);
    for (int64_t a = lo; a < hi; a += kCopyMaxPieceElems)
      out->push_back(Piece{nullptr, shard + a, std::min(kCopyMaxPieceElems, hi - a)});
  }
  return zero::ok();
}

// The pieces of shard range [begin, begin+count), produced a batch at a time
// into the caller's storage: the pieces build_pieces lists, in its order,
// without allocating memory.
class PieceCursor {
 public:
  PieceCursor(const zero_layout_s* h, uint16_t* const* tensors, uint16_t* shard, int64_t begin, int64_t count,
              bool to_shard)
      : h_(h), tensors_(tensors), shard_(shard), begin_(begin), end_(begin + count), to_shard_(to_shard) {
    const auto& segs = h->segs;
    s_ = size_t(std::upper_bound(segs.begin(), segs.end(), begin,
                                 [](int64_t v, const zero_segment& g) { return v < g.dst_off + g.len; }) -
                segs.begin());
    a_ = begin;
  }

  // Fills up to `cap` pieces; returns how many (0 once the range is done), or
  // a negative error code for a tensor pointer the range needs that is NULL or
  // misaligned.
  int64_t next(Piece* out, int64_t cap, const char* who) {
    const auto& segs = h_->segs;
    int64_t n = 0;
    while (n < cap) {
      if (!in_pad_) {
        if (s_ >= segs.size() || segs[s_].dst_off >= end_) {
          in_pad_ = true;
          a_ = std::max(h_->info.pad_begin, begin_);
          continue;
        }
        const zero_segment& g = segs[s_];
        const int64_t lo = std::max(g.dst_off, begin_), hi = std::min(g.dst_off + g.len, end_);
        if (a_ < lo) a_ = lo;
        if (a_ >= hi) {
          ++s_;
          continue;
        }
        uint16_t* t = tensors_[g.tensor];
        if (t == nullptr)
          return fail(ZERO_EINVAL, "%s: pointer of tensor %lld is NULL but the range needs it", who,
                      (long long)g.tensor);
        if (uintptr_t(t) & 1u)
          return fail(ZERO_EINVAL, "%s: tensor %lld pointer is not 2-byte aligned", who, (long long)g.tensor);
        const int64_t len = std::min(kCopyMaxPieceElems, hi - a_);
        uint16_t* tp = t + g.src_off + (a_ - g.dst_off);
        uint16_t* sp = shard_ + a_;
        out[n++] = to_shard_ ? Piece{tp, sp, len} : Piece{sp, tp, len};
        a_ += len;
      } else {
        const int64_t hi = std::min(h_->info.pad_end, end_);
        if (!to_shard_ || a_ >= hi) return n;   // unpack: padding goes nowhere
        const int64_t len = std::min(kCopyMaxPieceElems, hi - a_);
        out[n++] = Piece{nullptr, shard_ + a_, len};
        a_ += len;
      }
    }
    return n;
  }

 private:
  const zero_layout_s* h_;
  uint16_t* const* tensors_;
  uint16_t* shard_;
  int64_t begin_, end_;
  bool to_shard_;
  size_t s_ = 0;          // the segment being cut
  int64_t a_ = 0;         // next shard element to emit
  bool in_pad_ = false;   // past the segments: the padding overlap
};

int check_range(const zero_layout_s* h, int64_t begin, int64_t count, const char* who) {
  if (begin < 0 || count < 0 || begin > h->info.shard || count > h->info.shard - begin)
    return fail(ZERO_EINVAL, "%s: range [%lld, +%lld) outside the shard of %lld elements", who,
                (long long)begin, (long long)count, (long long)h->info.shard);
  return ZERO_OK;
}

// ============================================================ sum of squares
//
// Stage 1: one-shot blocks (grid-stride only beyond kSqMaxBlocks tiles); each
// lane loads two 16-byte vectors of a 4096-element tile, squares every bf16
// value in fp64 (exact) and accumulates in fp64; the block reduces through
// wavefront shuffles and LDS in a fixed pattern and writes one partial.
// Stage 2: one block adds the partials in a fixed pattern. The number of
// blocks depends only on count and no atomics are used, so results are
// bit-reproducible.

constexpr int kSqThreads = 256;
constexpr int kSqVecPerThread = 2;
constexpr int64_t kSqVecPerBlock = int64_t(kSqThreads) * kSqVecPerThread;  // 4096 bf16
constexpr int64_t kSqMaxBlocks = 65536;
constexpr int kSqFinalThreads = 1024;

int sq_blocks(int64_t count) {
  const int64_t nvec = count >> 3;
  int64_t b = (nvec + kSqVecPerBlock - 1) / kSqVecPerBlock;
  if (b < 1) b = 1;
  if (b > kSqMaxBlocks) b = kSqMaxBlocks;
  return int(b);
}

__global__ __launch_bounds__(kSqThreads) void sqnorm_partial_kernel(const uint16_t* __restrict__ g,
                                                                     int64_t count, int64_t head,
                                                                     double* __restrict__ partial) {
  const int64_t nvec = (count - head) >> 3;
  const u32x4* __restrict__ gv = reinterpret_cast<const u32x4*>(g + head);
  double acc = 0.0;
  for (int64_t tile = blockIdx.x; tile * kSqVecPerBlock < nvec; tile += gridDim.x) {
    const int64_t i0 = tile * kSqVecPerBlock + threadIdx.x;
    u32x4 r[kSqVecPerThread];
#pragma unroll
    for (int k = 0; k < kSqVecPerThread; ++k) {
      const int64_t i = i0 + int64_t(k) * kSqThreads;
      r[k] = i < nvec ? __builtin_nontemporal_load(gv + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < kSqVecPerThread; ++k) acc = sq8(r[k], acc);
  }
  if (blockIdx.x == 0) {
    // scalar head (before the first 16-byte boundary) and tail (< 8 values)
    const int t = threadIdx.x;
    if (t < head) {
      const double x = double(__uint_as_float(uint32_t(g[t]) << 16));
      acc = fma(x, x, acc);
    }
    const int64_t k = head + nvec * 8 + (t - 8);
    if (t >= 8 && k < count) {
      const double x = double(__uint_as_float(uint32_t(g[k]) << 16));
      acc = fma(x, x, acc);
    }
  }
  const double s = block_sum<kSqThreads>(acc);
  if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

// fp32 gradients: the same tiles of kSqVecPerBlock * 8 = 4096 elements per
// block (so the block count and workspace are those of the bf16 kernel), each
// lane loading four 16-byte vectors of 4 floats.
__device__ __forceinline__ double sq4(f32x4 w, double acc) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const double a = double(w[k]);
    acc = fma(a, a, acc);
  }
  return acc;
}

__global__ __launch_bounds__(kSqThreads) void sqnorm_f32_partial_kernel(const float* __restrict__ g, int64_t count,
                                                                         int64_t head, double* __restrict__ partial) {
  constexpr int VPT = 4;
  constexpr int64_t VPB = int64_t(kSqThreads) * VPT;   // 1024 vectors = 4096 floats
  const int64_t nvec = (count - head) >> 2;
  const f32x4* __restrict__ gv = reinterpret_cast<const f32x4*>(g + head);
  double acc = 0.0;
  for (int64_t tile = blockIdx.x; tile * VPB < nvec; tile += gridDim.x) {
    const int64_t i0 = tile * VPB + threadIdx.x;
    f32x4 r[VPT];
#pragma unroll
    for (int k = 0; k < VPT; ++k) {
      const int64_t i = i0 + int64_t(k) * kSqThreads;
      r[k] = i < nvec ? __builtin_nontemporal_load(gv + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int k = 0; k < VPT; ++k) acc = sq4(r[k], acc);
  }
  if (blockIdx.x == 0) {
    const int t = threadIdx.x;
    if (t < head) acc = fma(double(g[t]), double(g[t]), acc);
    const int64_t k = head + nvec * 4 + (t - 4);
    if (t >= 4 && k < count) acc = fma(double(g[k]), double(g[k]), acc);
  }
  const double s = block_sum<kSqThreads>(acc);
  if (threadIdx.x == 0) partial[blockIdx.x] = s;
}

// The fixed-order sum of n doubles by one block of kSqFinalThreads threads;
// every thread calls it, thread 0 writes *out (or adds to it).
__device__ __forceinline__ void final_sum(const double* __restrict__ partial, int64_t n, double* __restrict__ out,
                                          int accumulate) {
  // The partials were just written by blocks on every XCD, so each load is a
  // trip to memory: sixteen independent loads per lane per round keep the
  // rounds few (a 1.7 G-element shard has ~2e5 partials). The accumulators
  // are combined pairwise in a fixed order; the order depends only on n.
  constexpr int T = kSqFinalThreads;
  constexpr int U = 16;
  double acc[U];
#pragma unroll
  for (int u = 0; u < U; ++u) acc[u] = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += int64_t(U) * T) {
    double x[U];                        // past the end: 0, which leaves a sum unchanged
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t k = i + int64_t(u) * T;
      x[u] = k < n ? partial[k] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] += x[u];
  }
#pragma unroll
  for (int w = U / 2; w >= 1; w /= 2) {
#pragma unroll
    for (int u = 0; u < w; ++u) acc[u] += acc[u + w];
  }
  const double s = block_sum<kSqFinalThreads>(acc[0]);
  if (threadIdx.x == 0) *out = accumulate ? *out + s : s;
}

__global__ __launch_bounds__(kSqFinalThreads) void sqnorm_final_kernel(const double* __restrict__ partial,
                                                                        int64_t n, double* __restrict__ out,
                                                                        int accumulate) {
  final_sum(partial, n, out, accumulate);
}

// Rows of partial sums, one block each: out[r] (+)= the sum of row r, in the
// order sqnorm_final_kernel adds the same values.
constexpr int kMaxRowsPerLaunch = 192;

struct Rows {
  int32_t n;
  int64_t begin[kMaxRowsPerLaunch];
  int64_t len[kMaxRowsPerLaunch];
};
static_assert(sizeof(Rows) + 3 * sizeof(void*) <= 4096, "kernel arguments fit the 4 KiB segment");

__global__ __launch_bounds__(kSqFinalThreads) void sum_rows_kernel(const double* __restrict__ partial, const Rows R,
                                                                    double* __restrict__ out, int accumulate) {
  const int r = blockIdx.x;
  final_sum(partial + R.begin[r], R.len[r], out + r, accumulate);
}

// ============================================================ fused AdamW
//
// The fp32 state of an n-element shard is one buffer of 3n floats in tiles of
// kTile elements: tile k covers elements [k*T, k*T + L_k), L_k = min(T, n - k*T),
// and holds master[L_k], then m[L_k], then v[L_k] (the last tile is compact).
// Measured on MI355X, keeping the three state streams within one 96 KiB tile
// raises the update from ~5.6 to ~6.4 TB/s against three separate arrays: the
// waves in flight then touch one compact window of HBM instead of three
// windows hundreds of MB apart.
//
// One lane owns 4 consecutive elements: an 8-byte bf16 gradient load, one
// 16-byte load each of master, m and v, the same three stores back and an
// 8-byte bf16 parameter store: 28 bytes per element, and every wavefront
// instruction covers one contiguous span (512 B or 1 KiB). The grid is
// one-shot, in blocks of one wave: measured on MI355X at the 7.5B shard, the
// fused update takes 553 us in 64-lane blocks, 558 us in 128-lane and 562 us
// in 256-lane ones (a plain copy probe: 83.7 % of 8 TB/s against 81.0 %),
// the dispatcher then placing single waves wherever one has finished. The
// clip coefficient is formed by every lane from the ranks' partial sums
// (uniform loads, fp64), so the step needs no host synchronisation between
// the norm and the update.

constexpr int kAdamThreads = 64;
constexpr int64_t kAdamMaxBlocks = int64_t(1) << 25;   // 2^31 work-items
// A range longer than this is updated in several launches of equal length
// (rounded up to whole tiles). Measured on MI355X over a 1.68 G-element state:
// one launch 7.41 ms, launches of 2^27 or 2^26 elements 7.29-7.30 ms, of 2^25
// 7.33 ms; at 119 M elements one launch and two take the same time. (The copy
// kernels are fastest as one launch: each cut costs them ~3 us.)
constexpr int64_t kAdamLaunchElems = ZERO_ADAMW_LAUNCH_ELEMS;
constexpr int kTileLog2 = 13;
constexpr int64_t kTile = int64_t(1) << kTileLog2;     // ZERO_STATE_TILE
static_assert(kTile == ZERO_STATE_TILE, "state tile size");

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct AdamWArgs {
  const void* g;          // shard element 0 (bf16 bits, or fp32 for the accumulated gradient)
  float* state;           // shard element 0's tile
  uint16_t* param;        // shard element 0
  int64_t n_state;        // elements the state buffer describes
  int64_t begin, end;     // elements to update
  int64_t u_begin, u_end; // 4-element units inside [begin, end)
  const double* rank_sq;
  int32_t n_ranks;
  int32_t clip_on;
  double max_norm;
  double clip_eps;
  float beta1, omb1, beta2, omb2;
  float lr_wd, step_size, inv_sqrt_bc2, eps;
  zero::AdamWExact x;     // the same constants in fp64, for the exact recomputation
};

// The clip coefficient from the ranks' partial sums, formed by every wave
// (all 64 lanes must be active). G is added in a fixed two-level order: lane l
// adds ranks l, l+64, l+128, ... in that order, and the 64 lane sums are then
// added in lane order. With at most 64 ranks each lane holds one rank (the
// others add nothing), so G is the plain rank-order sum, done here by one
// loop of uniform loads. With more, each wave's loads are coalesced rows of 64
// ranks and its dependent chain of fp64 adds is n_ranks/64 + 64 long instead
// of n_ranks (a chain of 1024 made the update 8x slower). The host update
// forms G in the same order.
__device__ __forceinline__ double clip_coefficient(const AdamWArgs& a) {
  if (!a.clip_on) return 1.0;
  double G = 0.0;
  if (a.n_ranks <= 64) {
    for (int r = 0; r < a.n_ranks; ++r) G += a.rank_sq[r];   // uniform loads, rank order
  } else {
    const int lane = threadIdx.x & 63;
    const int rows = a.n_ranks >> 6;
    double run = 0.0;
#pragma unroll 8
    for (int j = 0; j < rows; ++j) run += a.rank_sq[(j << 6) + lane];
    if (lane < a.n_ranks - (rows << 6)) run += a.rank_sq[(rows << 6) + lane];
    const unsigned long long bits = __double_as_longlong(run);
    const int lo = int(unsigned(bits)), hi = int(unsigned(bits >> 32));
#pragma unroll
    for (int l = 0; l < 64; ++l) {   // lane l's sum, read into scalar registers
      const unsigned long long u = (unsigned long long)unsigned(__builtin_amdgcn_readlane(lo, l)) |
                                   ((unsigned long long)unsigned(__builtin_amdgcn_readlane(hi, l)) << 32);
      G += __longlong_as_double((long long)u);
    }
  }
  const double ratio = a.max_norm / (sqrt(G) + a.clip_eps);
  return ratio >= 1.0 ? 1.0 : ratio;  // a NaN ratio stays NaN
}

// One element's update. The fp32 path: c is the clip coefficient rounded to
// fp32, and the step is
//   g' = c*g;  m' = beta1*m + (1-beta1)*g';  v' = beta2*v + (1-beta2)*g'^2
//   p' = (p - lr*wd*p) - (lr/(1-beta1^t)) * m' / (sqrt(v')/sqrt(1-beta2^t) + eps)
// with each line's products and sums as fused multiply-adds, and correctly
// rounded division and square root. Its error stays below 2^-21.6 of
// S = |p - lr*wd*p| + (lr/(1-beta1^t)) * (|beta1*m| + |(1-beta1)*g'|) / denominator
// (the worst seen over 10^8 elements with planted cancellation), so p'
// rounds to within one bf16 step of the exact update's p' as long as
// |p'| >= 2^-13.6 S. Where |p'| < 2^-12 S (the master lands near zero by
// cancellation: about 2e-5 of the elements, in 0.5 % of the waves, on the
// model shards measured) the element is recomputed from its old values in
// fp64 IEEE arithmetic, in PyTorch AdamW's order, with the constants and the
// coefficient in fp64 (adamw_exact); m', v', p' are then the fp32 roundings
// of the exact fp64 evaluation. So every bf16 parameter is within one step
// of the bf16 rounding of the exactly computed master. The host update runs
// the same two paths. (An update entirely in fp64 matches the fp64 oracle bit
// for bit but, measured on MI355X, takes 7-20 % longer: its arithmetic no
// longer hides under the loads.)
constexpr float kCancel = 0x1p-12f;

// The constants are loaded where the branch is taken. Every update kernel
// takes its AdamWArgs as its first argument, at offset 0 of the kernel
// argument segment; the address passes through an empty asm statement in the
// branch, so the compiler cannot hoist the loads to the start of the kernel.
// (Held in scalar registers for the whole kernel, the constants cost the fused
// update one wave per SIMD; the address of the argument itself makes the
// compiler copy the arguments to scratch memory.)
__device__ __forceinline__ void adamw_exact(double c, float g, float& p, float& m, float& v) {
  const char* ka = (const char*)__builtin_amdgcn_kernarg_segment_ptr();
  const zero::AdamWExact* xp = reinterpret_cast<const zero::AdamWExact*>(ka + offsetof(AdamWArgs, x));
  asm volatile("" : "+s"(xp));
  const double beta1 = xp->beta1, omb1 = xp->omb1, beta2 = xp->beta2, omb2 = xp->omb2;
  const double decay = xp->decay, step_size = xp->step_size, sqrt_bc2 = xp->sqrt_bc2, eps = xp->eps;
  const double gh = c * double(g);
  const double m1 = beta1 * double(m) + omb1 * gh;
  const double v1 = beta2 * double(v) + omb2 * (gh * gh);
  const double denom = sqrt(v1) / sqrt_bc2 + eps;
  const double p1 = double(p) * decay - step_size * (m1 / denom);
  p = float(p1);
  m = float(m1);
  v = float(v1);
}

// The fp32 path for one element; returns whether the element must be
// recomputed exactly, i.e. whether (|p'| - 2^-12 |pd|) * denom is below
// 2^-12 * step_size * (|beta1*m| + |(1-beta1)*g'|), pd = p - lr*wd*p. The new
// values go to p1, m1, v1; p, m, v are left as they were.
__device__ __forceinline__ bool adamw_fast(const AdamWArgs& a, float c, float g, float p, float m, float v,
                                           float& p1, float& m1, float& v1) {
  const float gh = g * c;
  const float mg = a.omb1 * gh;
  m1 = fmaf(a.beta1, m, mg);
  v1 = fmaf(a.beta2, v, a.omb2 * (gh * gh));
  const float denom = fmaf(sqrtf(v1), a.inv_sqrt_bc2, a.eps);
  // decoupled decay first, then the step: p - lr*wd*p - step_size*(m/denom),
  // each as one fused multiply-add (the host update runs the same sequence)
  const float pd = fmaf(-a.lr_wd, p, p);
  p1 = fmaf(-a.step_size, m1 / denom, pd);
  return fmaf(-kCancel, fabsf(pd), fabsf(p1)) * denom < (kCancel * a.step_size) * (fabsf(a.beta1 * m) + fabsf(mg));
}

// The update of one element in place.
__device__ __forceinline__ void adamw_one(const AdamWArgs& a, double c64, float c, float g, float& p, float& m,
                                          float& v) {
  float p1, m1, v1;
  if (adamw_fast(a, c, g, p, m, v, p1, m1, v1)) {
    adamw_exact(c64, g, p, m, v);
    return;
  }
  p = p1;
  m = m1;
  v = v1;
}

// Position of element e's master value in the state buffer and its tile length.
__device__ __forceinline__ float* tile_slot(const AdamWArgs& a, int64_t e, int64_t* len) {
  const int64_t k0 = (e >> kTileLog2) << kTileLog2;   // first element of the tile
  const int64_t rest = a.n_state - k0;
  *len = rest < kTile ? rest : kTile;
  return a.state + 3 * k0 + (e - k0);
}

template <typename G>
__device__ __forceinline__ float grad_at(const AdamWArgs& a, int64_t e) {
  if constexpr (sizeof(G) == 2) return __uint_as_float(uint32_t(static_cast<const uint16_t*>(a.g)[e]) << 16);
  else return static_cast<const float*>(a.g)[e];
}

// ------------------------------------------------------------ stream loads
// The vector path loads the gradient and the state with buffer instructions
// carrying the sc1 and nt cache bits (device scope, non-temporal): data read
// once goes to the L2 without passing through the CU's vector L1. Measured at
// the 7.5B shard: the fused update 545 us against 555 us with non-temporal
// global loads. The same bits on the stores made each step ~3 us slower at
// the GPT-2 shard (the write-back at the end of the kernel), so the stores
// stay non-temporal global stores. A buffer resource addresses 32-bit byte
// offsets from its base: each launch gets resources based at its first tile,
// and a launch spans at most kAdamLaunchElems elements (plus rounding to
// whole tiles), whose state fits those offsets.

constexpr int kStreamLoadAux = 16 | 2;        // sc1 | nt
constexpr int kBufferWord3 = 0x00020000;      // raw (untyped) buffer access, gfx9 resource format
static_assert(12 * (kAdamLaunchElems + 3 * kTile) < (int64_t(1) << 31), "a launch's state fits 32-bit offsets");

template <typename G>
struct StreamLoads {
  __amdgpu_buffer_rsrc_t state, grad;
  const float* sbase;   // the state of the launch's first tile
  int64_t e0;           // that tile's first element
};

// The resources of a launch over [a.begin, a.end): the tiles it touches.
template <typename G>
__device__ __forceinline__ StreamLoads<G> stream_loads(const AdamWArgs& a) {
  const int64_t t_lo = (a.begin >> kTileLog2) << kTileLog2;
  const int64_t t_up = ((a.end + kTile - 1) >> kTileLog2) << kTileLog2;
  const int64_t t_hi = t_up < a.n_state ? t_up : a.n_state;
  StreamLoads<G> r;
  r.e0 = t_lo;
  r.sbase = a.state + 3 * t_lo;
  r.state = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(r.sbase), 0, int(12 * (t_hi - t_lo)), kBufferWord3);
  r.grad = __builtin_amdgcn_make_buffer_rsrc(const_cast<G*>(static_cast<const G*>(a.g) + t_lo), 0,
                                             int(int64_t(sizeof(G)) * (t_hi - t_lo)), kBufferWord3);
  return r;
}

// The 4 gradients of the unit at element e (a multiple of 4).
template <typename G>
__device__ __forceinline__ f32x4 grad4(const StreamLoads<G>& ld, int64_t e) {
  const int off = int((e - ld.e0) * int64_t(sizeof(G)));
  if constexpr (sizeof(G) == 2) {
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(ld.grad, off, 0, kStreamLoadAux);
    return f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
  } else {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ld.grad, off, 0, kStreamLoadAux));
  }
}

// The 4 state values at s (a 16-byte aligned master, m or v slot of the launch).
template <typename G>
__device__ __forceinline__ f32x4 state4(const StreamLoads<G>& ld, const float* s) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ld.state, int((s - ld.sbase) * 4), 0,
                                                                         kStreamLoadAux));
}

// One element; returns the bf16 parameter it stores.
template <typename G>
__device__ __forceinline__ uint16_t adamw_scalar(const AdamWArgs& a, double c64, float c, int64_t e) {
  int64_t L;
  float* s = tile_slot(a, e, &L);
  float p = s[0], m = s[L], v = s[2 * L];
  adamw_one(a, c64, c, grad_at<G>(a, e), p, m, v);
  s[0] = p;
  s[L] = m;
  s[2 * L] = v;
  const uint16_t b = to_bf16(p);
  a.param[e] = b;
  return b;
}

template <typename G>
__global__ __launch_bounds__(kAdamThreads) void adamw_vec_kernel(const AdamWArgs a) {
  const double c64 = clip_coefficient(a);
  const float c = float(c64);
  const StreamLoads<G> ld = stream_loads<G>(a);
  const int64_t stride = int64_t(gridDim.x) * kAdamThreads;
  for (int64_t u = a.u_begin + int64_t(blockIdx.x) * kAdamThreads + threadIdx.x; u < a.u_end; u += stride) {
    const int64_t e = u << 2;
    int64_t L;
    float* s = tile_slot(a, e, &L);
    if (L & 3) {   // a compact last tile whose m and v are not 16-byte aligned
      for (int k = 0; k < 4; ++k) adamw_scalar<G>(a, c64, c, e + k);
      continue;
    }
    f32x4* ps = reinterpret_cast<f32x4*>(s);
    f32x4* ms = reinterpret_cast<f32x4*>(s + L);
    f32x4* vs = reinterpret_cast<f32x4*>(s + 2 * L);
    const f32x4 g4 = grad4<G>(ld, e);
    const f32x4 p4 = state4<G>(ld, s);
    const f32x4 m4 = state4<G>(ld, s + L);
    const f32x4 v4 = state4<G>(ld, s + 2 * L);
    float p[4] = {p4[0], p4[1], p4[2], p4[3]};
    float m[4] = {m4[0], m4[1], m4[2], m4[3]};
    float v[4] = {v4[0], v4[1], v4[2], v4[3]};
#pragma unroll
    for (int k = 0; k < 4; ++k) adamw_one(a, c64, c, g4[k], p[k], m[k], v[k]);
    __builtin_nontemporal_store(f32x4{p[0], p[1], p[2], p[3]}, ps);
    __builtin_nontemporal_store(f32x4{m[0], m[1], m[2], m[3]}, ms);
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, vs);
    __builtin_nontemporal_store(u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])},
                                reinterpret_cast<u32x2*>(a.param + e));
  }
  // up to 3 elements before the first unit and after the last one
  if (blockIdx.x == 0) {
    const int t = threadIdx.x;
    const int64_t head_end = 4 * a.u_begin < a.end ? 4 * a.u_begin : a.end;
    if (t < 4 && a.begin + t < head_end) adamw_scalar<G>(a, c64, c, a.begin + t);
    const int64_t k = 4 * a.u_end + (t - 4);
    if (t >= 4 && t < 8 && k >= head_end && k < a.end) adamw_scalar<G>(a, c64, c, k);
  }
}

// Element path for base pointers without the vector path's alignment.
template <typename G>
__global__ __launch_bounds__(kAdamThreads) void adamw_elem_kernel(const AdamWArgs a) {
  const double c64 = clip_coefficient(a);
  const float c = float(c64);
  const int64_t stride = int64_t(gridDim.x) * kAdamThreads;
  for (int64_t e = a.begin + int64_t(blockIdx.x) * kAdamThreads + threadIdx.x; e < a.end; e += stride)
    adamw_scalar<G>(a, c64, c, e);
}

// ------------------------------------------------ AdamW with the unpack fused
//
// The same update, and each new bf16 parameter is also stored at its
// position in the per-tensor parameters: AdamW followed by unpack over the
// same range, in one pass (30 instead of 28 + 4 bytes per element). The
// parameter shard is still written (it is what the all-gather sends). One
// launch carries up to kUnpackMaxPieces pieces of the range in its kernel
// arguments; inside a rank's shard they are contiguous, and padding (after
// the last) has no tensor. Each wave finds the piece of its lowest element
// (uniform loads); when the whole wave lies in it, a lane stores its 4 values
// with one 8-byte store (or 4 scalar stores when the tensor is not 8-byte
// congruent with the shard); a wave across a piece boundary loops over the
// pieces it touches. Every table index is wave-uniform.

constexpr int kUnpackMaxPieces = ZERO_PIECES_PER_LAUNCH;
constexpr int kWave = 64;

constexpr int kUnpackSlots = 256;

struct UnpackPieces {
  int32_t n;                               // pieces (0: no tensor element in the range)
  int32_t slot_shift;                      // element lo[0] + j lies in slot j >> slot_shift
  uint64_t vec_mask;                       // bit p: 4-element stores to piece p are 8-byte aligned
  int64_t lo[kUnpackMaxPieces + 1];        // piece p holds shard elements [lo[p], lo[p+1]); lo[n] ends the last
  uint16_t* dst[kUnpackMaxPieces];         // tensor element of shard element lo[p]
  uint8_t slot_piece[kUnpackSlots];        // piece holding each slot's first element
};
static_assert(sizeof(AdamWArgs) + sizeof(UnpackPieces) <= 4096, "kernel arguments fit the 4 KiB segment");

// The value x holds in the wave's first active lane.
__device__ __forceinline__ int64_t wave_first(int64_t x) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(uint64_t(x)))));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(uint64_t(x) >> 32))));
  return int64_t((uint64_t(hi) << 32) | lo);
}

// The piece holding shard element e (uniform; lo[0] <= e < lo[n]): the last p
// with lo[p] <= e, from the slot table and a short forward step (a binary
// search is a chain of dependent scalar loads at the start of every wave).
__device__ __forceinline__ int unpack_piece(const UnpackPieces& U, int64_t e) {
  int p = U.slot_piece[(e - U.lo[0]) >> U.slot_shift];
  while (U.lo[p + 1] <= e) ++p;
  return p;
}

// Store the bf16 values of this lane's shard elements [e, e + N) (N = 1 or 4;
// for 4, packed in two words) at their tensor positions. The active lanes of
// the wave hold consecutive elements starting at the first active lane's, all
// within W elements of it. (Looking the destination up before the update's
// loads, to overlap its scalar loads with them, measured slower.)
template <int N, int W>
__device__ __forceinline__ void unpack_lane(const UnpackPieces& U, int64_t e, uint32_t w0, uint32_t w1,
                                            int hint = -1) {
  if (U.n == 0) return;
  const int64_t w_lo = wave_first(e);
  if (w_lo >= U.lo[U.n]) return;                     // padding only
  // `hint`: the piece of the block's first element, looked up at the start
  int p = hint >= 0 && w_lo >= U.lo[hint] && w_lo + W <= U.lo[hint + 1] ? hint
          : w_lo < U.lo[0] ? 0 : unpack_piece(U, w_lo);
  if (w_lo >= U.lo[p] && w_lo + W <= U.lo[p + 1]) {  // the whole wave lies in piece p
    uint16_t* d = U.dst[p] + (e - U.lo[p]);
    if constexpr (N == 4) {
      if ((U.vec_mask >> p) & 1) {
        __builtin_nontemporal_store(u32x2{w0, w1}, reinterpret_cast<u32x2*>(d));
      } else {
        d[0] = uint16_t(w0);
        d[1] = uint16_t(w0 >> 16);
        d[2] = uint16_t(w1);
        d[3] = uint16_t(w1 >> 16);
      }
    } else {
      d[0] = uint16_t(w0);
    }
    return;
  }
  for (; p < U.n && U.lo[p] < w_lo + W; ++p) {       // the pieces the wave touches
    const int64_t lo = U.lo[p], hi = U.lo[p + 1];
#pragma unroll
    for (int k = 0; k < N; ++k) {
      const int64_t ek = e + k;
      const uint32_t w = k < 2 ? w0 : w1;
      if (ek >= lo && ek < hi) U.dst[p][ek - lo] = uint16_t(k & 1 ? w >> 16 : w);
    }
  }
}

template <typename G>
__global__ __launch_bounds__(kAdamThreads) void adamw_unpack_vec_kernel(const AdamWArgs a, const UnpackPieces U) {
  // the piece of this block's first element (first pass of the loop), from
  // the block index alone: its scalar loads start before any data is loaded.
  // (Issuing the lane's first loads before the clip coefficient, which every
  // wave forms in a chain of dependent loads and adds, measured 559-563 us at
  // the 7.5B shard against 559-560 us as written: that chain is not what
  // limits the stream. Loading eight ranks' sums per scalar load instead of
  // one took the 24.3 M-element shard from 121 to 119.5 us but the 7.5B
  // shard from 559 to 562 us.)
  const int64_t b_lo = (a.u_begin + int64_t(blockIdx.x) * kAdamThreads) << 2;
  const int hint = U.n > 0 && b_lo >= U.lo[0] && b_lo < U.lo[U.n] ? unpack_piece(U, b_lo) : -1;
  const double c64 = clip_coefficient(a);
  const float c = float(c64);
  const StreamLoads<G> ld = stream_loads<G>(a);
  const int64_t stride = int64_t(gridDim.x) * kAdamThreads;
  for (int64_t u = a.u_begin + int64_t(blockIdx.x) * kAdamThreads + threadIdx.x; u < a.u_end; u += stride) {
    const int64_t e = u << 2;
    int64_t L;
    float* s = tile_slot(a, e, &L);
    if (L & 3) {   // a compact last tile whose m and v are not 16-byte aligned
      for (int k = 0; k < 4; ++k) unpack_lane<1, 4 * kWave>(U, e + k, adamw_scalar<G>(a, c64, c, e + k), 0);
      continue;
    }
    f32x4* ps = reinterpret_cast<f32x4*>(s);
    f32x4* ms = reinterpret_cast<f32x4*>(s + L);
    f32x4* vs = reinterpret_cast<f32x4*>(s + 2 * L);
    const f32x4 g4 = grad4<G>(ld, e);
    const f32x4 p4 = state4<G>(ld, s);
    const f32x4 m4 = state4<G>(ld, s + L);
    const f32x4 v4 = state4<G>(ld, s + 2 * L);
    float p[4] = {p4[0], p4[1], p4[2], p4[3]};
    float m[4] = {m4[0], m4[1], m4[2], m4[3]};
    float v[4] = {v4[0], v4[1], v4[2], v4[3]};
#pragma unroll
    for (int k = 0; k < 4; ++k) adamw_one(a, c64, c, g4[k], p[k], m[k], v[k]);
    __builtin_nontemporal_store(f32x4{p[0], p[1], p[2], p[3]}, ps);
    __builtin_nontemporal_store(f32x4{m[0], m[1], m[2], m[3]}, ms);
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, vs);
    const uint32_t w0 = pack_bf16x2(p[0], p[1]), w1 = pack_bf16x2(p[2], p[3]);
    __builtin_nontemporal_store(u32x2{w0, w1}, reinterpret_cast<u32x2*>(a.param + e));
    unpack_lane<4, 4 * kWave>(U, e, w0, w1, hint);
  }
  // up to 3 elements before the first unit and after the last one
  if (blockIdx.x == 0) {
    const int t = threadIdx.x;
    const int64_t head_end = 4 * a.u_begin < a.end ? 4 * a.u_begin : a.end;
    if (t < 4 && a.begin + t < head_end)
      unpack_lane<1, 4>(U, a.begin + t, adamw_scalar<G>(a, c64, c, a.begin + t), 0);
    const int64_t k = 4 * a.u_end + (t - 4);
    if (t >= 4 && t < 8 && k >= head_end && k < a.end) unpack_lane<1, 4>(U, k, adamw_scalar<G>(a, c64, c, k), 0);
  }
}

template <typename G>
__global__ __launch_bounds__(kAdamThreads) void adamw_unpack_elem_kernel(const AdamWArgs a, const UnpackPieces U) {
  const double c64 = clip_coefficient(a);
  const float c = float(c64);
  const int64_t stride = int64_t(gridDim.x) * kAdamThreads;
  for (int64_t e = a.begin + int64_t(blockIdx.x) * kAdamThreads + threadIdx.x; e < a.end; e += stride)
    unpack_lane<1, kWave>(U, e, adamw_scalar<G>(a, c64, c, e), 0);
}

// ------------------------------------------------ AdamW over three state arrays
//
// The state as the pages hold it: fp32 master, m and v as three arrays of the
// shard's length (K = 12 bytes per parameter, "第 5 课：ZeRO 与 FSDP" section
// 2), for callers that keep them as separate tensors. The arithmetic is
// adamw_one's, so the results are bit-identical to the tiled update's. Each
// launch sees the arrays from a "launch element 0" whose master, m and v are
// 16-byte aligned (and gradient and parameter 8-byte aligned): the host moves
// the pointers back by the arrays' common phase, and the launch's range
// [begin, end) starts at that phase. A lane owns the 4-element unit at 4u:
// one 8-byte gradient load, three 16-byte state loads, the three stores back
// and an 8-byte parameter store, all non-temporal. The first and last units'
// leftover elements (at most 3 each) go to block 0's lanes.
//
// Measured on MI355X at the 7.5B shard (119.4 M elements), this update takes
// 550-558 us (75-76 % of 8 TB/s) against 514 us for the tiled one: the eight
// streams (four read, four written) of three arrays hundreds of MB apart cost
// ~8 % against the tiled state's compact window. Where the three arrays sit
// barely matters (554-568 us over gaps from 0 to 64 MiB between them); two
// units per lane measured 2 % slower, temporal stores 7 %, and the update
// tiles' sc1|nt buffer loads 1 % slower than these loads.

struct StateArrays {
  float* m;   // launch element 0 of m (a.state holds the master's)
  float* v;   // launch element 0 of v
};

// The 4 gradients at element e (a multiple of 4; 8- or 16-byte aligned).
template <typename G>
__device__ __forceinline__ f32x4 grad4_global(const AdamWArgs& a, int64_t e) {
  if constexpr (sizeof(G) == 2) {
    const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(static_cast<const G*>(a.g) + e));
    return f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
  } else {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(static_cast<const G*>(a.g) + e));
  }
}

template <typename G>
__device__ __forceinline__ void adamw_arrays_scalar(const AdamWArgs& a, const StateArrays& sa, double c64, float c,
                                                    int64_t e) {
  float p = a.state[e], m = sa.m[e], v = sa.v[e];
  adamw_one(a, c64, c, grad_at<G>(a, e), p, m, v);
  a.state[e] = p;
  sa.m[e] = m;
  sa.v[e] = v;
  a.param[e] = to_bf16(p);
}

template <typename G>
__global__ __launch_bounds__(kAdamThreads) void adamw_arrays_vec_kernel(const AdamWArgs a, const StateArrays sa) {
  const double c64 = clip_coefficient(a);
  const float c = float(c64);
  const int64_t stride = int64_t(gridDim.x) * kAdamThreads;
  for (int64_t u = a.u_begin + int64_t(blockIdx.x) * kAdamThreads + threadIdx.x; u < a.u_end; u += stride) {
    const int64_t e = u << 2;
    const f32x4 g4 = grad4_global<G>(a, e);
    const f32x4 p4 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(a.state + e));
    const f32x4 m4 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sa.m + e));
    const f32x4 v4 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(sa.v + e));
    float p[4] = {p4[0], p4[1], p4[2], p4[3]};
    float m[4] = {m4[0], m4[1], m4[2], m4[3]};
    float v[4] = {v4[0], v4[1], v4[2], v4[3]};
#pragma unroll
    for (int k = 0; k < 4; ++k) adamw_one(a, c64, c, g4[k], p[k], m[k], v[k]);
    __builtin_nontemporal_store(f32x4{p[0], p[1], p[2], p[3]}, reinterpret_cast<f32x4*>(a.state + e));
    __builtin_nontemporal_store(f32x4{m[0], m[1], m[2], m[3]}, reinterpret_cast<f32x4*>(sa.m + e));
    __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(sa.v + e));
    __builtin_nontemporal_store(u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])},
                                reinterpret_cast<u32x2*>(a.param + e));
  }
  if (blockIdx.x == 0) {
    const int t = threadIdx.x;
    const int64_t head_end = 4 * a.u_begin < a.end ? 4 * a.u_begin : a.end;
    if (t < 4 && a.begin + t < head_end) adamw_arrays_scalar<G>(a, sa, c64, c, a.begin + t);
    const int64_t k = 4 * a.u_end + (t - 4);
    if (t >= 4 && t < 8 && k >= head_end && k < a.end) adamw_arrays_scalar<G>(a, sa, c64, c, k);
  }
}

// Element path, for arrays whose phases differ.
template <typename G>
__global__ __launch_bounds__(kAdamThreads) void adamw_arrays_elem_kernel(const AdamWArgs a, const StateArrays sa) {
  const double c64 = clip_coefficient(a);
  const float c = float(c64);
  const int64_t stride = int64_t(gridDim.x) * kAdamThreads;
  for (int64_t e = a.begin + int64_t(blockIdx.x) * kAdamThreads + threadIdx.x; e < a.end; e += stride)
    adamw_arrays_scalar<G>(a, sa, c64, c, e);
}

// ------------------------------------------------ fp32 gradient accumulation
// acc = (first ? 0 : acc) + g for one micro-batch: an 8-byte bf16 load and a
// 16-byte fp32 load/store per lane (4 elements), fp32 add (round to nearest).

__global__ __launch_bounds__(kAdamThreads) void accumulate_kernel(const uint16_t* __restrict__ g,
                                                                   float* __restrict__ acc, int64_t count,
                                                                   int first, int vec) {
  const int64_t stride = int64_t(gridDim.x) * kAdamThreads;
  const int64_t units = vec ? (count >> 2) : count;
  for (int64_t u = int64_t(blockIdx.x) * kAdamThreads + threadIdx.x; u < units; u += stride) {
    if (vec) {
      const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(g) + u);
      f32x4* ap = reinterpret_cast<f32x4*>(acc) + u;
      const f32x4 x = {bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
      const f32x4 r = first ? x : __builtin_nontemporal_load(ap) + x;
      __builtin_nontemporal_store(r, ap);
    } else {
      const float x = __uint_as_float(uint32_t(g[u]) << 16);
      acc[u] = first ? x : acc[u] + x;
    }
  }
  if (vec && blockIdx.x == 0 && threadIdx.x < (count & 3)) {   // the last count % 4 elements
    const int64_t e = ((count >> 2) << 2) + threadIdx.x;
    const float x = __uint_as_float(uint32_t(g[e]) << 16);
    acc[e] = first ? x : acc[e] + x;
  }
}

// ------------------------------------------------ state layout conversion
// Separate master/m/v arrays <-> the tiled state buffer (a bit copy). One lane
// moves 4 consecutive elements of each array when everything is 16-byte
// aligned and the tile length is a multiple of 4, one element otherwise.

template <bool TO_TILES>
__global__ __launch_bounds__(kAdamThreads) void state_convert_kernel(float* state, float* master, float* m,
                                                                      float* v, int64_t n, int vec) {
  const int64_t stride = int64_t(gridDim.x) * kAdamThreads;
  const int64_t units = vec ? (n >> 2) : n;
  for (int64_t u = int64_t(blockIdx.x) * kAdamThreads + threadIdx.x; u < units; u += stride) {
    const int64_t e0 = vec ? (u << 2) : u;
    const int64_t k0 = (e0 >> kTileLog2) << kTileLog2;
    const int64_t L = (n - k0) < kTile ? (n - k0) : kTile;
    float* s = state + 3 * k0 + (e0 - k0);
    if (vec && !(L & 3)) {
      f32x4* sp = reinterpret_cast<f32x4*>(s);
      f32x4* sm = reinterpret_cast<f32x4*>(s + L);
      f32x4* sv = reinterpret_cast<f32x4*>(s + 2 * L);
      f32x4* xp = reinterpret_cast<f32x4*>(master + e0);
      f32x4* xm = reinterpret_cast<f32x4*>(m + e0);
      f32x4* xv = reinterpret_cast<f32x4*>(v + e0);
      if (TO_TILES) { *sp = *xp; *sm = *xm; *sv = *xv; }
      else { *xp = *sp; *xm = *sm; *xv = *sv; }
    } else {
      const int cnt = vec ? 4 : 1;
      for (int k = 0; k < cnt; ++k) {
        if (TO_TILES) { s[k] = master[e0 + k]; s[L + k] = m[e0 + k]; s[2 * L + k] = v[e0 + k]; }
        else { master[e0 + k] = s[k]; m[e0 + k] = s[L + k]; v[e0 + k] = s[2 * L + k]; }
      }
    }
  }
  if (vec && blockIdx.x == 0 && threadIdx.x < (n & 3)) {   // the last n % 4 elements
    const int64_t e = ((n >> 2) << 2) + threadIdx.x;
    const int64_t k0 = (e >> kTileLog2) << kTileLog2;
    const int64_t L = n - k0 < kTile ? n - k0 : kTile;
    float* s = state + 3 * k0 + (e - k0);
    if (TO_TILES) { s[0] = master[e]; s[L] = m[e]; s[2 * L] = v[e]; }
    else { master[e] = s[0]; m[e] = s[L]; v[e] = s[2 * L]; }
  }
}

bool aligned(const void* p, uintptr_t n) { return (uintptr_t(p) & (n - 1)) == 0; }

}  // namespace

// ======================================================= static scratch
//
// zero_pack_grads_sqnorm_noalloc keeps its block partial sums in this array
// instead of a caller's workspace. Each GPU the library runs on holds its own
// copy, ZERO_NOALLOC_PARTIALS doubles (2 MiB), until the process ends. In
// host code `scratch` only names the array: its device address on the
// current GPU comes from hipGetSymbolAddress, once per device, and only that
// address is passed to kernels.
static __device__ __align__(256) double scratch[ZERO_NOALLOC_PARTIALS];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<double*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of `scratch` on the current device (looked up on the
// first call for each device).
int scratch_address(double** out, const char* who) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ZERO_EHIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ZERO_EINVAL, "%s: device %d is beyond the %d devices the library tracks", who, dev, kMaxDevices);
  double* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess || addr == nullptr)
        return fail(ZERO_EHIP, "%s: hipGetSymbolAddress of the static scratch on device %d: %s", who, dev,
                    hipGetErrorString(e));
      p = static_cast<double*>(addr);
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return ZERO_OK;
}

}  // namespace

// ================================================================== C ABI

extern "C" int zero_pack_grads(zero_layout_t h, const uint16_t* const* tensor_grads, uint16_t* grad_shard,
                               int64_t begin, int64_t count, hipStream_t stream) {
  static const char* who = "zero_pack_grads";
  if (h == nullptr || tensor_grads == nullptr || grad_shard == nullptr)
    return fail(ZERO_EINVAL, "%s: NULL handle, tensor array or shard", who);
  if (int rc = check_range(h, begin, count, who)) return rc;
  if (uintptr_t(grad_shard) & 1u) return fail(ZERO_EINVAL, "%s: shard pointer is not 2-byte aligned", who);
  if (count == 0) return zero::ok();
  std::vector<Piece> pieces;
  if (int rc = build_pieces(h, const_cast<uint16_t* const*>(tensor_grads), grad_shard, begin, count, true,
                            &pieces, who))
    return rc;
  return launch_pieces(pieces, stream, who);
}

// Lengths of the pieces pack would copy for shard range [begin, begin+count).
static std::vector<int64_t> pack_piece_lengths(const zero_layout_s* h, int64_t begin, int64_t count) {
  std::vector<int64_t> lens;
  const int64_t end = begin + count;
  for (const zero_segment& g : h->segs) {
    const int64_t lo = std::max(g.dst_off, begin), hi = std::min(g.dst_off + g.len, end);
    for (int64_t a = lo; a < hi; a += kCopyMaxPieceElems) lens.push_back(std::min(kCopyMaxPieceElems, hi - a));
  }
  const int64_t lo = std::max(h->info.pad_begin, begin), hi = std::min(h->info.pad_end, end);
  for (int64_t a = lo; a < hi; a += kCopyMaxPieceElems) lens.push_back(std::min(kCopyMaxPieceElems, hi - a));
  return lens;
}

extern "C" size_t zero_pack_sqnorm_workspace_bytes(zero_layout_t h, int64_t begin, int64_t count) {
  if (h == nullptr || check_range(h, begin, count, "zero_pack_sqnorm_workspace_bytes") != ZERO_OK) return 0;
  const int64_t blocks = pieces_block_bound(pack_piece_lengths(h, begin, count));
  return size_t(std::max<int64_t>(blocks, 1)) * sizeof(double);
}

extern "C" int zero_pack_grads_sqnorm(zero_layout_t h, const uint16_t* const* tensor_grads, uint16_t* grad_shard,
                                      int64_t begin, int64_t count, double* d_out, int32_t accumulate,
                                      void* d_workspace, size_t ws_bytes, hipStream_t stream) {
  static const char* who = "zero_pack_grads_sqnorm";
  if (h == nullptr || tensor_grads == nullptr || grad_shard == nullptr)
    return fail(ZERO_EINVAL, "%s: NULL handle, tensor array or shard", who);
  if (d_out == nullptr || d_workspace == nullptr) return fail(ZERO_EINVAL, "%s: NULL output or workspace", who);
  if (int rc = check_range(h, begin, count, who)) return rc;
  if (uintptr_t(grad_shard) & 1u) return fail(ZERO_EINVAL, "%s: shard pointer is not 2-byte aligned", who);
  if (uintptr_t(d_workspace) & 7u) return fail(ZERO_EINVAL, "%s: workspace is not 8-byte aligned", who);
  const int64_t bound = std::max<int64_t>(pieces_block_bound(pack_piece_lengths(h, begin, count)), 1);
  if (ws_bytes < size_t(bound) * sizeof(double))
    return fail(ZERO_EINVAL, "%s: workspace of %zu bytes, need %zu", who, ws_bytes, size_t(bound) * sizeof(double));
  std::vector<Piece> pieces;
  if (int rc = build_pieces(h, const_cast<uint16_t* const*>(tensor_grads), grad_shard, begin, count, true,
                            &pieces, who))
    return rc;
  double* part = static_cast<double*>(d_workspace);
  int64_t n_part = 0;
  if (int rc = launch_pieces(pieces, stream, who, part, &n_part)) return rc;
  hipLaunchKernelGGL(sqnorm_final_kernel, dim3(1), dim3(kSqFinalThreads), 0, stream, part, n_part, d_out,
                     accumulate ? 1 : 0);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return zero::ok();
}

extern "C" int zero_pack_grads_sqnorm_noalloc(zero_layout_t h, const uint16_t* const* tensor_grads,
                                              uint16_t* grad_shard, int64_t begin, int64_t count, double* d_out,
                                              int32_t accumulate, hipStream_t stream) {
  static const char* who = "zero_pack_grads_sqnorm_noalloc";
  if (h == nullptr || tensor_grads == nullptr || grad_shard == nullptr)
    return fail(ZERO_EINVAL, "%s: NULL handle, tensor array or shard", who);
  if (d_out == nullptr) return fail(ZERO_EINVAL, "%s: NULL output", who);
  if (int rc = check_range(h, begin, count, who)) return rc;
  if (uintptr_t(grad_shard) & 1u) return fail(ZERO_EINVAL, "%s: shard pointer is not 2-byte aligned", who);
  uint16_t* const* grads = const_cast<uint16_t* const*>(tensor_grads);
  // pass 1: check the tensor pointers and bound the partial sums, as
  // zero_pack_sqnorm_workspace_bytes does
  Piece batch[kCopyMaxPieces];
  int64_t bound = 0;
  {
    PieceCursor cur(h, grads, grad_shard, begin, count, true);
    for (int64_t n; (n = cur.next(batch, kCopyMaxPieces, who)) != 0;) {
      if (n < 0) return int(n);
      for (int64_t i = 0; i < n; ++i) bound += (batch[i].len + kCopySqElemPerBlock - 1) / kCopySqElemPerBlock + 1;
    }
  }
  if (bound > ZERO_NOALLOC_PARTIALS)
    return fail(ZERO_EINVAL,
                "%s: the range [%lld, +%lld) needs up to %lld partial sums; the static scratch holds %d "
                "(split the range, or use zero_pack_grads_sqnorm with a workspace)",
                who, (long long)begin, (long long)count, (long long)bound, ZERO_NOALLOC_PARTIALS);
  double* part = nullptr;
  if (int rc = scratch_address(&part, who)) return rc;
  // pass 2: the launches, each block writing its partial sum to the next slot
  int64_t done = 0;
  PieceCursor cur(h, grads, grad_shard, begin, count, true);
  for (int64_t n; (n = cur.next(batch, kCopyMaxPieces, who)) != 0;) {
    if (n < 0) return int(n);
    int64_t n_part = 0;
    if (int rc = launch_pieces(batch, size_t(n), stream, who, part + done, &n_part)) return rc;
    done += n_part;
  }
  hipLaunchKernelGGL(sqnorm_final_kernel, dim3(1), dim3(kSqFinalThreads), 0, stream, part, done, d_out,
                     accumulate ? 1 : 0);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return zero::ok();
}

extern "C" int zero_unpack_params(zero_layout_t h, const uint16_t* param_shard, uint16_t* const* tensor_params,
                                  int64_t begin, int64_t count, hipStream_t stream) {
  static const char* who = "zero_unpack_params";
  if (h == nullptr || tensor_params == nullptr || param_shard == nullptr)
    return fail(ZERO_EINVAL, "%s: NULL handle, tensor array or shard", who);
  if (int rc = check_range(h, begin, count, who)) return rc;
  if (uintptr_t(param_shard) & 1u) return fail(ZERO_EINVAL, "%s: shard pointer is not 2-byte aligned", who);
  if (count == 0) return zero::ok();
  std::vector<Piece> pieces;
  if (int rc = build_pieces(h, tensor_params, const_cast<uint16_t*>(param_shard), begin, count, false,
                            &pieces, who))
    return rc;
  return launch_pieces(pieces, stream, who);
}

extern "C" size_t zero_sqnorm_workspace_bytes(int64_t count) {
  if (count < 0) count = 0;
  return size_t(sq_blocks(count)) * sizeof(double);
}

extern "C" int zero_shard_sqnorm(const uint16_t* d_grad, int64_t count, double* d_out, int32_t accumulate,
                                 void* d_workspace, size_t ws_bytes, hipStream_t stream) {
  static const char* who = "zero_shard_sqnorm";
  if (count < 0) return fail(ZERO_EINVAL, "%s: count < 0", who);
  if (d_out == nullptr || d_workspace == nullptr) return fail(ZERO_EINVAL, "%s: NULL output or workspace", who);
  if (count > 0 && d_grad == nullptr) return fail(ZERO_EINVAL, "%s: NULL gradient", who);
  if (uintptr_t(d_grad) & 1u) return fail(ZERO_EINVAL, "%s: gradient pointer is not 2-byte aligned", who);
  if (uintptr_t(d_workspace) & 7u) return fail(ZERO_EINVAL, "%s: workspace is not 8-byte aligned", who);
  const int nb = sq_blocks(count);
  if (ws_bytes < size_t(nb) * sizeof(double))
    return fail(ZERO_EINVAL, "%s: workspace of %zu bytes, need %zu", who, ws_bytes, size_t(nb) * sizeof(double));
  double* part = static_cast<double*>(d_workspace);
  const int64_t head = copy_head(d_grad, count);
  hipLaunchKernelGGL(sqnorm_partial_kernel, dim3(nb), dim3(kSqThreads), 0, stream, d_grad, count, head, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  hipLaunchKernelGGL(sqnorm_final_kernel, dim3(1), dim3(kSqFinalThreads), 0, stream, part, nb, d_out,
                     accumulate ? 1 : 0);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return zero::ok();
}

extern "C" int zero_sum_partials(const double* d_partials, int64_t n, double* d_out, int32_t accumulate,
                                 hipStream_t stream) {
  static const char* who = "zero_sum_partials";
  if (n < 0) return fail(ZERO_EINVAL, "%s: n < 0", who);
  if (d_out == nullptr) return fail(ZERO_EINVAL, "%s: NULL output", who);
  if (n > 0 && d_partials == nullptr) return fail(ZERO_EINVAL, "%s: NULL partial sums", who);
  if ((uintptr_t(d_partials) | uintptr_t(d_out)) & 7u) return fail(ZERO_EINVAL, "%s: misaligned pointer", who);
  hipLaunchKernelGGL(sqnorm_final_kernel, dim3(1), dim3(kSqFinalThreads), 0, stream, d_partials, n, d_out,
                     accumulate ? 1 : 0);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return zero::ok();
}

extern "C" int zero_pack_grads_sqnorm_partials(zero_layout_t h, const uint16_t* const* tensor_grads,
                                               uint16_t* grad_shard, int64_t begin, int64_t count,
                                               double* d_partials, size_t cap_bytes, int64_t* n_partials,
                                               hipStream_t stream) {
  static const char* who = "zero_pack_grads_sqnorm_partials";
  if (h == nullptr || tensor_grads == nullptr || grad_shard == nullptr)
    return fail(ZERO_EINVAL, "%s: NULL handle, tensor array or shard", who);
  if (d_partials == nullptr || n_partials == nullptr) return fail(ZERO_EINVAL, "%s: NULL partials or count", who);
  if (int rc = check_range(h, begin, count, who)) return rc;
  if (uintptr_t(grad_shard) & 1u) return fail(ZERO_EINVAL, "%s: shard pointer is not 2-byte aligned", who);
  if (uintptr_t(d_partials) & 7u) return fail(ZERO_EINVAL, "%s: partials are not 8-byte aligned", who);
  const int64_t bound = std::max<int64_t>(pieces_block_bound(pack_piece_lengths(h, begin, count)), 1);
  if (cap_bytes < size_t(bound) * sizeof(double))
    return fail(ZERO_EINVAL, "%s: room for %zu bytes of partial sums, need %zu", who, cap_bytes,
                size_t(bound) * sizeof(double));
  std::vector<Piece> pieces;
  if (int rc = build_pieces(h, const_cast<uint16_t* const*>(tensor_grads), grad_shard, begin, count, true,
                            &pieces, who))
    return rc;
  int64_t n = 0;
  if (int rc = launch_pieces(pieces, stream, who, d_partials, &n)) return rc;
  *n_partials = n;
  return zero::ok();
}

extern "C" int zero_sum_partials_rows(const double* d_partials, const int64_t* row_begin, const int64_t* row_len,
                                      int64_t n_rows, double* d_out, int32_t accumulate, hipStream_t stream) {
  static const char* who = "zero_sum_partials_rows";
  if (n_rows < 0) return fail(ZERO_EINVAL, "%s: n_rows < 0", who);
  if (n_rows == 0) return zero::ok();
  if (d_partials == nullptr || row_begin == nullptr || row_len == nullptr || d_out == nullptr)
    return fail(ZERO_EINVAL, "%s: NULL argument", who);
  if ((uintptr_t(d_partials) | uintptr_t(d_out)) & 7u) return fail(ZERO_EINVAL, "%s: misaligned pointer", who);
  for (int64_t r = 0; r < n_rows; ++r)
    if (row_begin[r] < 0 || row_len[r] < 0)
      return fail(ZERO_EINVAL, "%s: row %lld has a negative start or length", who, (long long)r);
  for (int64_t r0 = 0; r0 < n_rows; r0 += kMaxRowsPerLaunch) {
    Rows R{};
    R.n = int32_t(std::min<int64_t>(kMaxRowsPerLaunch, n_rows - r0));
    for (int32_t i = 0; i < R.n; ++i) {
      R.begin[i] = row_begin[r0 + i];
      R.len[i] = row_len[r0 + i];
    }
    hipLaunchKernelGGL(sum_rows_kernel, dim3(unsigned(R.n)), dim3(kSqFinalThreads), 0, stream, d_partials, R,
                       d_out + r0, accumulate ? 1 : 0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  }
  return zero::ok();
}

// Checks the arguments of an update over [begin, begin+count) and fills the
// kernel arguments (range fields for the whole range). *vec: the pointers
// allow the vector path. With count == 0 it returns OK after the checks
// without filling *out: the caller has nothing to launch.
template <typename G>
static int adamw_args(const G* d_grad, float* d_state, uint16_t* d_param, int64_t n_state, int64_t begin,
                      int64_t count, const zero_adamw_hparams* hp, const double* d_rank_sqnorms, int32_t n_ranks,
                      const char* who, AdamWArgs* out, bool* vec) {
  if (int rc = zero::check_adamw_hparams(hp, who)) return rc;
  if (n_state < 0 || begin < 0 || count < 0 || begin > n_state || count > n_state - begin)
    return fail(ZERO_EINVAL, "%s: range [%lld, +%lld) outside a state of %lld elements", who, (long long)begin,
                (long long)count, (long long)n_state);
  const bool clip = hp->max_norm > 0.0;
  if (clip && (d_rank_sqnorms == nullptr || n_ranks < 1))
    return fail(ZERO_EINVAL, "%s: clipping needs the ranks' sums of squares", who);
  if (count == 0) return zero::ok();
  if (!d_grad || !d_state || !d_param) return fail(ZERO_EINVAL, "%s: NULL buffer", who);
  if ((uintptr_t(d_grad) & (sizeof(G) - 1)) || (uintptr_t(d_param) & 1u) || (uintptr_t(d_state) & 3u))
    return fail(ZERO_EINVAL, "%s: misaligned element pointer", who);

  AdamWArgs a{};
  a.g = d_grad;
  a.state = d_state;
  a.param = d_param;
  a.n_state = n_state;
  a.rank_sq = d_rank_sqnorms;
  a.n_ranks = clip ? n_ranks : 0;
  a.clip_on = clip ? 1 : 0;
  a.max_norm = hp->max_norm;
  a.clip_eps = hp->clip_eps;
  a.beta1 = float(hp->beta1);
  a.omb1 = float(1.0 - hp->beta1);
  a.beta2 = float(hp->beta2);
  a.omb2 = float(1.0 - hp->beta2);
  const double t = double(hp->step);
  const double bc1 = 1.0 - std::pow(hp->beta1, t);
  const double bc2 = 1.0 - std::pow(hp->beta2, t);
  a.lr_wd = float(hp->lr * hp->weight_decay);
  a.step_size = float(hp->lr / bc1);
  a.inv_sqrt_bc2 = float(1.0 / std::sqrt(bc2));
  a.eps = float(hp->eps);
  zero::adamw_exact_constants(hp, &a.x);
  // vector path: 4 gradients (8 or 16 bytes), 4 bf16 params (8 bytes), fp32 state (16 bytes)
  *vec = aligned(d_grad, 4 * sizeof(G)) && aligned(d_param, 8) && aligned(d_state, 16);
  *out = a;
  return zero::ok();
}

// Elements per launch for a range of `count`: the fewest launches of at most
// kAdamLaunchElems, of equal length rounded up to whole tiles.
static int64_t adamw_chunk(int64_t count) {
  if (count <= 0) return kTile;
  const int64_t k = (count + kAdamLaunchElems - 1) / kAdamLaunchElems;
  const int64_t c = (count + k - 1) / k;
  return (c + kTile - 1) / kTile * kTile;
}

// Sets a's range to [r0, r1) and returns the grid for it.
static unsigned adamw_range(AdamWArgs* a, int64_t r0, int64_t r1, bool vec) {
  a->begin = r0;
  a->end = r1;
  a->u_begin = (r0 + 3) >> 2;
  a->u_end = r1 >> 2;
  if (a->u_end < a->u_begin) a->u_end = a->u_begin;   // fewer than 4 elements, all scalar
  const int64_t work = vec ? std::max<int64_t>(a->u_end - a->u_begin, 1) : r1 - r0;
  int64_t blocks = (work + kAdamThreads - 1) / kAdamThreads;
  return unsigned(std::min(std::max<int64_t>(blocks, 1), kAdamMaxBlocks));
}

template <typename G>
static int adamw_launch(const G* d_grad, float* d_state, uint16_t* d_param, int64_t n_state, int64_t begin,
                        int64_t count, const zero_adamw_hparams* hp, const double* d_rank_sqnorms,
                        int32_t n_ranks, hipStream_t stream, const char* who) {
  AdamWArgs a{};
  bool vec = false;
  if (int rc = adamw_args(d_grad, d_state, d_param, n_state, begin, count, hp, d_rank_sqnorms, n_ranks, who, &a,
                          &vec))
    return rc;
  if (count == 0) return zero::ok();
  const int64_t end = begin + count, chunk = adamw_chunk(count);
  for (int64_t r0 = begin; r0 < end;) {
    const int64_t r1 = std::min(end, r0 + chunk);
    const unsigned blocks = adamw_range(&a, r0, r1, vec);
    if (vec)
      hipLaunchKernelGGL(adamw_vec_kernel<G>, dim3(blocks), dim3(kAdamThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(adamw_elem_kernel<G>, dim3(blocks), dim3(kAdamThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
    r0 = r1;
  }
  return zero::ok();
}

// The update with the unpack fused: launches of adamw_chunk(count) elements
// at most and kUnpackMaxPieces pieces, a piece cut by a launch boundary
// continuing in the next launch; the last launch also covers the padding
// after the last piece.
template <typename G>
static int adamw_unpack_launch(const G* d_grad, float* d_state, uint16_t* d_param, int64_t n_state, int64_t begin,
                               int64_t count, const zero_adamw_hparams* hp, const double* d_rank_sqnorms,
                               int32_t n_ranks, zero_layout_t h, uint16_t* const* tensor_params, hipStream_t stream,
                               const char* who) {
  if (h == nullptr || tensor_params == nullptr) return fail(ZERO_EINVAL, "%s: NULL handle or tensor array", who);
  if (n_state != h->info.shard)
    return fail(ZERO_EINVAL, "%s: n_state %lld is not the layout's shard of %lld elements", who,
                (long long)n_state, (long long)h->info.shard);
  AdamWArgs a{};
  bool vec = false;
  if (int rc = adamw_args(d_grad, d_state, d_param, n_state, begin, count, hp, d_rank_sqnorms, n_ranks, who, &a,
                          &vec))
    return rc;
  if (count == 0) return zero::ok();
  std::vector<Piece> pieces;
  if (int rc = build_pieces(h, tensor_params, d_param, begin, count, false, &pieces, who)) return rc;
  const int64_t end = begin + count, chunk = adamw_chunk(count);
  size_t i = 0;                  // the first piece not finished by earlier launches
  for (int64_t r0 = begin; r0 < end;) {
    int64_t r1 = std::min(end, r0 + chunk);
    UnpackPieces U{};
    int n = 0;
    size_t j = i;
    for (; j < pieces.size() && n < kUnpackMaxPieces; ++j, ++n) {
      const int64_t plo = pieces[j].src - d_param;           // the piece's first shard element
      if (plo >= r1) break;
      const int64_t lo = std::max(plo, r0);
      if (lo != (n == 0 ? r0 : U.lo[n]))
        return fail(ZERO_EINVAL, "%s: internal error: pieces not contiguous at element %lld", who, (long long)lo);
      U.lo[n] = lo;
      U.lo[n + 1] = std::min(plo + pieces[j].len, r1);
      U.dst[n] = pieces[j].dst + (lo - plo);
      if (((uintptr_t(U.dst[n]) - 2 * uintptr_t(lo)) & 7u) == 0) U.vec_mask |= uint64_t(1) << n;
    }
    U.n = n;
    // a full table with pieces still starting inside the launch: end it at its last piece
    if (n == kUnpackMaxPieces && j < pieces.size() && pieces[j].src - d_param < r1) r1 = U.lo[n];
    if (n > 0) {   // slot table over [lo[0], lo[n]): the smallest power-of-two slot that needs <= 256 slots
      const int64_t span = U.lo[n] - U.lo[0];
      int shift = 0;
      while (((span + (int64_t(1) << shift) - 1) >> shift) > kUnpackSlots) ++shift;
      U.slot_shift = shift;
      for (int q = 0, slot = 0; slot < kUnpackSlots; ++slot) {
        const int64_t first = U.lo[0] + (int64_t(slot) << shift);
        while (q + 1 < n && U.lo[q + 1] <= first) ++q;
        U.slot_piece[slot] = uint8_t(q);
      }
    }
    const unsigned blocks = adamw_range(&a, r0, r1, vec);
    if (vec)
      hipLaunchKernelGGL(adamw_unpack_vec_kernel<G>, dim3(blocks), dim3(kAdamThreads), 0, stream, a, U);
    else
      hipLaunchKernelGGL(adamw_unpack_elem_kernel<G>, dim3(blocks), dim3(kAdamThreads), 0, stream, a, U);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
    while (i < pieces.size() && pieces[i].src - d_param + pieces[i].len <= r1) ++i;
    r0 = r1;
  }
  return zero::ok();
}

extern "C" int zero_shard_sqnorm_f32(const float* d_grad, int64_t count, double* d_out, int32_t accumulate,
                                     void* d_workspace, size_t ws_bytes, hipStream_t stream) {
  static const char* who = "zero_shard_sqnorm_f32";
  if (count < 0) return fail(ZERO_EINVAL, "%s: count < 0", who);
  if (d_out == nullptr || d_workspace == nullptr) return fail(ZERO_EINVAL, "%s: NULL output or workspace", who);
  if (count > 0 && d_grad == nullptr) return fail(ZERO_EINVAL, "%s: NULL gradient", who);
  if (uintptr_t(d_grad) & 3u) return fail(ZERO_EINVAL, "%s: gradient pointer is not 4-byte aligned", who);
  if (uintptr_t(d_workspace) & 7u) return fail(ZERO_EINVAL, "%s: workspace is not 8-byte aligned", who);
  const int nb = sq_blocks(count);
  if (ws_bytes < size_t(nb) * sizeof(double))
    return fail(ZERO_EINVAL, "%s: workspace of %zu bytes, need %zu", who, ws_bytes, size_t(nb) * sizeof(double));
  double* part = static_cast<double*>(d_workspace);
  // floats before the first 16-byte boundary
  const int64_t head = std::min<int64_t>(count, int64_t(((16u - (uintptr_t(d_grad) & 15u)) & 15u) >> 2));
  hipLaunchKernelGGL(sqnorm_f32_partial_kernel, dim3(nb), dim3(kSqThreads), 0, stream, d_grad, count, head, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  hipLaunchKernelGGL(sqnorm_final_kernel, dim3(1), dim3(kSqFinalThreads), 0, stream, part, int64_t(nb), d_out,
                     accumulate ? 1 : 0);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return zero::ok();
}

extern "C" int zero_adamw_step(const uint16_t* d_grad, float* d_state, uint16_t* d_param, int64_t n_state,
                               int64_t begin, int64_t count, const zero_adamw_hparams* hp,
                               const double* d_rank_sqnorms, int32_t n_ranks, hipStream_t stream) {
  return adamw_launch<uint16_t>(d_grad, d_state, d_param, n_state, begin, count, hp, d_rank_sqnorms, n_ranks,
                                stream, "zero_adamw_step");
}

// Byte ranges [p, p + n) and [q, q + m) overlap.
static bool overlap(const void* p, size_t n, const void* q, size_t m) {
  const uintptr_t a = uintptr_t(p), b = uintptr_t(q);
  return n > 0 && m > 0 && a < b + m && b < a + n;
}

// Element `off` of an array (off may be negative: a launch element 0 before
// the array's first element, never accessed).
template <typename T>
static T* element_at(T* p, int64_t off) {
  return reinterpret_cast<T*>(uintptr_t(p) + uintptr_t(off * int64_t(sizeof(T))));
}

extern "C" int zero_adamw_step_arrays(const uint16_t* d_grad, float* d_master, float* d_m, float* d_v,
                                      uint16_t* d_param, int64_t count, const zero_adamw_hparams* hp,
                                      const double* d_rank_sqnorms, int32_t n_ranks, hipStream_t stream) {
  static const char* who = "zero_adamw_step_arrays";
  AdamWArgs a{};
  bool tiled_vec = false;   // the tiled path's alignment rule, not used here
  if (int rc = adamw_args(d_grad, d_master, d_param, count, 0, count, hp, d_rank_sqnorms, n_ranks, who, &a,
                          &tiled_vec))
    return rc;
  if (count == 0) return zero::ok();
  if (!d_m || !d_v) return fail(ZERO_EINVAL, "%s: NULL buffer", who);
  if ((uintptr_t(d_m) | uintptr_t(d_v)) & 3u) return fail(ZERO_EINVAL, "%s: misaligned element pointer", who);
  const size_t n = size_t(count);
  static const char* names[5] = {"master", "m", "v", "param", "grad"};
  const void* buf[5] = {d_master, d_m, d_v, d_param, d_grad};
  const size_t len[5] = {4 * n, 4 * n, 4 * n, 2 * n, 2 * n};
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 5; ++j)
      if (overlap(buf[i], len[i], buf[j], len[j]))
        return fail(ZERO_EINVAL, "%s: %s and %s overlap", who, names[i], names[j]);
  // The vector path needs the five arrays in one phase: element 0 the same
  // number of elements past a 16-byte (state) or 8-byte (bf16) boundary.
  const int64_t phase = int64_t(uintptr_t(d_master) >> 2) & 3;
  const bool vec = ((uintptr_t(d_m) ^ uintptr_t(d_master)) & 15u) == 0 &&
                   ((uintptr_t(d_v) ^ uintptr_t(d_master)) & 15u) == 0 &&
                   (uintptr_t(d_grad) & 7u) == uintptr_t(2 * phase) &&
                   (uintptr_t(d_param) & 7u) == uintptr_t(2 * phase);
  const int64_t shift = vec ? phase : 0;   // launch element 0 of the first launch is element -shift
  const int64_t vend = shift + count, chunk = adamw_chunk(vend);
  for (int64_t base = 0; base < vend; base += chunk) {
    const int64_t lo = std::max(base, shift), hi = std::min(vend, base + chunk);
    const int64_t off = base - shift;
    a.g = element_at(d_grad, off);
    a.state = element_at(d_master, off);
    a.param = element_at(d_param, off);
    a.n_state = hi - base;
    const StateArrays sa{element_at(d_m, off), element_at(d_v, off)};
    const unsigned blocks = adamw_range(&a, lo - base, hi - base, vec);
    if (vec)
      hipLaunchKernelGGL(adamw_arrays_vec_kernel<uint16_t>, dim3(blocks), dim3(kAdamThreads), 0, stream, a, sa);
    else
      hipLaunchKernelGGL(adamw_arrays_elem_kernel<uint16_t>, dim3(blocks), dim3(kAdamThreads), 0, stream, a, sa);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  }
  return zero::ok();
}

extern "C" int zero_adamw_step_f32grad(const float* d_grad, float* d_state, uint16_t* d_param, int64_t n_state,
                                       int64_t begin, int64_t count, const zero_adamw_hparams* hp,
                                       const double* d_rank_sqnorms, int32_t n_ranks, hipStream_t stream) {
  return adamw_launch<float>(d_grad, d_state, d_param, n_state, begin, count, hp, d_rank_sqnorms, n_ranks,
                             stream, "zero_adamw_step_f32grad");
}

extern "C" int zero_adamw_step_unpack(const uint16_t* d_grad, float* d_state, uint16_t* d_param, int64_t n_state,
                                      int64_t begin, int64_t count, const zero_adamw_hparams* hp,
                                      const double* d_rank_sqnorms, int32_t n_ranks, zero_layout_t h,
                                      uint16_t* const* tensor_params, hipStream_t stream) {
  return adamw_unpack_launch<uint16_t>(d_grad, d_state, d_param, n_state, begin, count, hp, d_rank_sqnorms,
                                       n_ranks, h, tensor_params, stream, "zero_adamw_step_unpack");
}

extern "C" int zero_adamw_step_f32grad_unpack(const float* d_grad, float* d_state, uint16_t* d_param,
                                              int64_t n_state, int64_t begin, int64_t count,
                                              const zero_adamw_hparams* hp, const double* d_rank_sqnorms,
                                              int32_t n_ranks, zero_layout_t h, uint16_t* const* tensor_params,
                                              hipStream_t stream) {
  return adamw_unpack_launch<float>(d_grad, d_state, d_param, n_state, begin, count, hp, d_rank_sqnorms, n_ranks,
                                    h, tensor_params, stream, "zero_adamw_step_f32grad_unpack");
}

extern "C" int zero_accumulate_grads(const uint16_t* d_grad, float* d_acc, int64_t count, int32_t first,
                                     hipStream_t stream) {
  static const char* who = "zero_accumulate_grads";
  if (count < 0) return fail(ZERO_EINVAL, "%s: count < 0", who);
  if (count == 0) return zero::ok();
  if (!d_grad || !d_acc) return fail(ZERO_EINVAL, "%s: NULL buffer", who);
  if ((uintptr_t(d_grad) & 1u) || (uintptr_t(d_acc) & 3u)) return fail(ZERO_EINVAL, "%s: misaligned pointer", who);
  const bool vec = aligned(d_grad, 8) && aligned(d_acc, 16);
  const int64_t units = vec ? std::max<int64_t>(count >> 2, 1) : count;
  const int64_t blocks = std::min(std::max<int64_t>((units + kAdamThreads - 1) / kAdamThreads, 1), kAdamMaxBlocks);
  hipLaunchKernelGGL(accumulate_kernel, dim3(unsigned(blocks)), dim3(kAdamThreads), 0, stream, d_grad, d_acc, count,
                     first ? 1 : 0, vec ? 1 : 0);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return zero::ok();
}

static int state_convert(bool to_tiles, float* state, float* master, float* m, float* v, int64_t n,
                         hipStream_t stream, const char* who) {
  if (n < 0) return fail(ZERO_EINVAL, "%s: n < 0", who);
  if (n == 0) return zero::ok();
  if (!state || !master || !m || !v) return fail(ZERO_EINVAL, "%s: NULL buffer", who);
  if ((uintptr_t(state) | uintptr_t(master) | uintptr_t(m) | uintptr_t(v)) & 3u)
    return fail(ZERO_EINVAL, "%s: misaligned pointer", who);
  const bool vec = aligned(state, 16) && aligned(master, 16) && aligned(m, 16) && aligned(v, 16);
  const int64_t units = vec ? std::max<int64_t>(n >> 2, 1) : n;
  const int64_t blocks = std::min(std::max<int64_t>((units + kAdamThreads - 1) / kAdamThreads, 1), kAdamMaxBlocks);
  if (to_tiles)
    hipLaunchKernelGGL(state_convert_kernel<true>, dim3(unsigned(blocks)), dim3(kAdamThreads), 0, stream, state,
                       master, m, v, n, vec ? 1 : 0);
  else
    hipLaunchKernelGGL(state_convert_kernel<false>, dim3(unsigned(blocks)), dim3(kAdamThreads), 0, stream, state,
                       master, m, v, n, vec ? 1 : 0);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ZERO_EHIP, "%s: launch failed: %s", who, hipGetErrorString(e));
  return zero::ok();
}

extern "C" int zero_state_import(const float* d_master, const float* d_m, const float* d_v, float* d_state,
                                 int64_t n, hipStream_t stream) {
  return state_convert(true, d_state, const_cast<float*>(d_master), const_cast<float*>(d_m),
                       const_cast<float*>(d_v), n, stream, "zero_state_import");
}

extern "C" int zero_state_export(const float* d_state, float* d_master, float* d_m, float* d_v, int64_t n,
                                 hipStream_t stream) {
  return state_convert(false, const_cast<float*>(d_state), d_master, d_m, d_v, n, stream, "zero_state_export");
}
