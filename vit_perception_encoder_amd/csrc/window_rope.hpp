// Token order and positions of the perception encoder's patch grid, on the device.
//
// Window order (vllm.cpp issue #1545, second comment: 32x32 = 1024-patch windows cut
// by the vision tower's sparse permutation; vllm.cpp PR #279, vision-tower commit:
// the tokens are gathered window by window before the blocks, and the inverse
// permutation runs before the final LayerNorm).  The pages name the block walk order
// and the within-block order without stating them; the reading taken here is
// row-major over the win x win blocks of each image (blocks at the right and bottom
// edges clipped to the grid), then row-major inside a block.  Images of a batch are
// concatenated; each keeps its own token range.
//
// 2D rotary position embedding (PR #279, vision-tower commits: width-first, 1-based
// positions).  Reading: the first half of each head's channels is rotated by the
// token's column (width) coordinate + 1, the second half by its row (height)
// coordinate + 1; inside a half, channels 2i and 2i+1 form a pair rotated by angle
// pos * theta^(-4i/d), as multiplication by exp(i * angle) of the complex number
// (x_2i + i x_2i+1).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mgattn {

constexpr int kMaxImages = 64;

struct ImageTable {
  int32_t n;                       // images
  int32_t start[kMaxImages + 1];   // first token of each image (prefix sums of gh*gw)
  int32_t gh[kMaxImages];          // grid height (rows of patches)
  int32_t gw[kMaxImages];          // grid width (columns of patches)
};

// Image holding token t (binary search over the prefix sums).
__device__ inline int image_of(const ImageTable& tb, int t) {
  int lo = 0, hi = tb.n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tb.start[mid] <= t) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// Raster index (y*gw + x) of the token at position p of an image's window order.
// Every block row but the last is win rows tall and spans win*gw tokens; inside a
// block row of height bh, every block but the last is win columns wide and spans
// bh*win tokens.
__device__ inline int window_to_raster(int p, int gh, int gw, int win) {
  // 64-bit products: win may exceed the grid (one block per image)
  const int64_t row_span = static_cast<int64_t>(win) * gw;
  const int by = static_cast<int>(p / row_span);
  const int rem = static_cast<int>(p - by * row_span);
  const int bh = static_cast<int>(min(static_cast<int64_t>(win), static_cast<int64_t>(gh) - static_cast<int64_t>(by) * win));
  const int64_t blk_span = static_cast<int64_t>(bh) * win;
  const int bx = static_cast<int>(rem / blk_span);
  const int rem2 = static_cast<int>(rem - bx * blk_span);
  const int bw = static_cast<int>(min(static_cast<int64_t>(win), static_cast<int64_t>(gw) - static_cast<int64_t>(bx) * win));
  const int y = static_cast<int>(static_cast<int64_t>(by) * win + rem2 / bw);
  const int x = static_cast<int>(static_cast<int64_t>(bx) * win + rem2 % bw);
  return y * gw + x;
}

// dst row p <- src row perm(p) (gather into window order), or dst row perm(p) <- src
// row p (inverse: back to raster order).  One 16-byte piece per thread.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void window_permute_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int32_t pieces_per_row,
                           int32_t win, int32_t inverse, int64_t total_pieces, ImageTable tb) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total_pieces) return;
  const int p = static_cast<int>(i / pieces_per_row);
  const int piece = static_cast<int>(i - static_cast<int64_t>(p) * pieces_per_row);
  const int img = image_of(tb, p);
  const int r = tb.start[img] + window_to_raster(p - tb.start[img], tb.gh[img], tb.gw[img], win);
  const int from = inverse ? p : r, to = inverse ? r : p;
  dst[static_cast<int64_t>(to) * pieces_per_row + piece] = src[static_cast<int64_t>(from) * pieces_per_row + piece];
}

constexpr int kRopeHeadGroup = 4;  // heads per thread: angles computed once for them

struct RopeArgs {
  void* x;
  int64_t ld;          // elements between consecutive tokens
  int32_t H, d;
  int32_t win;         // 0: tokens in raster order; > 0: in window order of this window
  int32_t pieces;      // 16-byte pieces per head (d*elem/16)
  int32_t groups;      // head groups per token: ceil(H / kRopeHeadGroup)
  float inv_freq[32];  // theta^(-4i/d), i < d/4
  ImageTable tb;
};

// One thread = one 16-byte piece (8 bf16 or 4 f32 values: whole pairs inside one half
// of a head, since d/2 is a multiple of 8) of one token, for up to kRopeHeadGroup
// heads: the angles depend on the token and the pair only, so they are computed once
// and applied to each head of the group.  In place.
template <typename T>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void rope2d_kernel(RopeArgs a, int64_t total_threads) {
  constexpr int kPer = 16 / sizeof(T);  // values per piece
  constexpr int kPairs = kPer / 2;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= total_threads) return;
  const int per_token = a.pieces * a.groups;
  const int t = static_cast<int>(i / per_token);
  const int rem = static_cast<int>(i - static_cast<int64_t>(t) * per_token);
  const int grp = rem / a.pieces, piece = rem % a.pieces;
  const int img = image_of(a.tb, t);
  const int p = t - a.tb.start[img];
  const int gw = a.tb.gw[img];
  const int r = a.win > 0 ? window_to_raster(p, a.tb.gh[img], gw, a.win) : p;
  const int c0 = piece * kPer;          // first channel of the piece inside its head
  const int half = a.d / 2;
  const float pos = static_cast<float>(c0 < half ? r % gw + 1 : r / gw + 1);
  const int i0 = (c0 % half) / 2;       // pair index of the piece's first pair
  float cs[kPairs], sn[kPairs];
#pragma unroll
  for (int j = 0; j < kPairs; ++j) sincosf(pos * a.inv_freq[i0 + j], &sn[j], &cs[j]);
  const int h0 = grp * kRopeHeadGroup, h1 = min(a.H, h0 + kRopeHeadGroup);
  T* row = static_cast<T*>(a.x) + static_cast<int64_t>(t) * a.ld + c0;
  uint4 raw[kRopeHeadGroup];
#pragma unroll
  for (int k = 0; k < kRopeHeadGroup; ++k)
    if (h0 + k < h1) raw[k] = *reinterpret_cast<const uint4*>(row + static_cast<int64_t>(h0 + k) * a.d);
#pragma unroll
  for (int k = 0; k < kRopeHeadGroup; ++k) {
    if (h0 + k >= h1) break;
    uint32_t w[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float re = __uint_as_float(w[j] << 16), im = __uint_as_float(w[j] & 0xffff0000u);
        const __bf16 a2 = static_cast<__bf16>(re * cs[j] - im * sn[j]);
        const __bf16 b2 = static_cast<__bf16>(re * sn[j] + im * cs[j]);
        w[j] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a2)) |
               (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b2)) << 16);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float re = __uint_as_float(w[2 * j]), im = __uint_as_float(w[2 * j + 1]);
        w[2 * j] = __float_as_uint(re * cs[j] - im * sn[j]);
        w[2 * j + 1] = __float_as_uint(re * sn[j] + im * cs[j]);
      }
    }
    *reinterpret_cast<uint4*>(row + static_cast<int64_t>(h0 + k) * a.d) = uint4{w[0], w[1], w[2], w[3]};
  }
}

}  // namespace mgattn
