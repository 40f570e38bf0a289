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
// row p (inverse: back to raster order).  One wave per row p: the row's partner
// (image, window order <-> raster) is wave-uniform and computed once; the lanes copy
// the row's 16-byte pieces, four loads in flight per lane before their stores.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void window_permute_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst, int32_t pieces_per_row,
                           int32_t win, int32_t inverse, int32_t n_rows, ImageTable tb) {
  const int p = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * 4 + (threadIdx.x >> 6));
  if (p >= n_rows) return;
  const int lane = threadIdx.x & 63;
  const int img = image_of(tb, p);
  const int r = tb.start[img] + window_to_raster(p - tb.start[img], tb.gh[img], tb.gw[img], win);
  const int from = inverse ? p : r, to = inverse ? r : p;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* __restrict__ s = reinterpret_cast<const u32x4*>(src) + static_cast<int64_t>(from) * pieces_per_row;
  u32x4* __restrict__ d = reinterpret_cast<u32x4*>(dst) + static_cast<int64_t>(to) * pieces_per_row;
  // loads unconditional (lanes past the row end re-read its last piece) and fenced
  // before the first store, so all four are in flight together; stores predicated and
  // non-temporal (nothing in this launch reads them back, and dirty L2 lines would be
  // written back at the kernel's end, delaying the next launch)
  for (int64_t k0 = 0; k0 < pieces_per_row; k0 += 256) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = s[min(k0 + u * 64 + lane, static_cast<int64_t>(pieces_per_row) - 1)];
    asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]));
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (k0 + u * 64 + lane < pieces_per_row) __builtin_nontemporal_store(v[u], d + k0 + u * 64 + lane);
  }
}

struct RopeArgs {
  void* x;
  int64_t ld;          // elements between consecutive tokens
  int32_t H, d;
  int32_t win;         // 0: tokens in raster order; > 0: in window order of this window
  int32_t pieces;      // 16-byte pieces per head (d*elem/16)
  float inv_freq[32];  // theta^(-4i/d), i < d/4
  ImageTable tb;
};

// One wave = one token, in place.  The token's patch position is wave-uniform and
// computed once; lane j < d/2 computes cos and sin of rotation pair j (pairs below d/4
// rotate by the column, the rest by the row, frequency index j mod d/4), and every
// 16-byte piece of the token's H*d values (8 bf16 or 4 f32: whole pairs of one half
// of a head, as d/2 is a multiple of 8) takes its pairs' values from those lanes by
// lane shuffles, made with every lane active before the bounds test.
template <typename T>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void rope2d_kernel(RopeArgs a, int32_t n_tokens) {
  constexpr int kPer = 16 / sizeof(T);  // values per piece
  constexpr int kPairs = kPer / 2;
  const int t = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * 4 + (threadIdx.x >> 6));
  if (t >= n_tokens) return;
  const int lane = threadIdx.x & 63;
  const int img = image_of(a.tb, t);
  const int p = t - a.tb.start[img];
  const int gw = a.tb.gw[img];
  const int r = a.win > 0 ? window_to_raster(p, a.tb.gh[img], gw, a.win) : p;
  const int quarter = a.d / 4;  // pairs per half of a head
  const float f_l = a.inv_freq[lane < 2 * quarter ? lane % quarter : 0];  // loaded before the data
  float c_l = 1.0f, s_l = 0.0f;
  T* row = static_cast<T*>(a.x) + static_cast<int64_t>(t) * a.ld;
  const int total = a.H * a.pieces;
  constexpr int kU = 4;  // pieces per lane loaded together
  for (int j0 = 0; j0 < total; j0 += 64 * kU) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    u32x4 raw[kU];
    int off[kU], pcs[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = min(j0 + u * 64 + lane, total - 1);  // past the end: re-read the last piece
      const int head = j / a.pieces;
      pcs[u] = j - head * a.pieces;
      off[u] = head * a.d + pcs[u] * kPer;
      raw[u] = *reinterpret_cast<const u32x4*>(row + off[u]);
    }
    if (j0 == 0 && lane < 2 * quarter) {  // the angles, while the first loads are in flight
      const float pos = static_cast<float>(lane < quarter ? r % gw + 1 : r / gw + 1);
      sincosf(pos * f_l, &s_l, &c_l);
    }
    asm volatile("" ::"v"(raw[0]), "v"(raw[1]), "v"(raw[2]), "v"(raw[3]));
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float cs[kPairs], sn[kPairs];
#pragma unroll
      for (int k = 0; k < kPairs; ++k) {  // every lane active here
        const int src = (pcs[u] * kPairs + k) & 63;
        cs[k] = __shfl(c_l, src);
        sn[k] = __shfl(s_l, src);
      }
      uint32_t w[4] = {raw[u][0], raw[u][1], raw[u][2], raw[u][3]};
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float re = __uint_as_float(w[k] << 16), im = __uint_as_float(w[k] & 0xffff0000u);
          const __bf16 a2 = static_cast<__bf16>(re * cs[k] - im * sn[k]);
          const __bf16 b2 = static_cast<__bf16>(re * sn[k] + im * cs[k]);
          w[k] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, a2)) |
                 (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, b2)) << 16);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float re = __uint_as_float(w[2 * k]), im = __uint_as_float(w[2 * k + 1]);
          w[2 * k] = __float_as_uint(re * cs[k] - im * sn[k]);
          w[2 * k + 1] = __float_as_uint(re * sn[k] + im * cs[k]);
        }
      }
      if (j0 + u * 64 + lane < total) *reinterpret_cast<u32x4*>(row + off[u]) = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}

}  // namespace mgattn
