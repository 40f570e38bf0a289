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
// bh*win tokens.  The block size is clamped to each side of the image (win may exceed
// the grid: one block per image); blocks are clipped at the edges anyway, so the
// order is the same, and every product below is then at most gh*gw < 2^31, which
// keeps the divisions in 32 bits.
__device__ inline int window_to_raster(int p, int gh, int gw, int win) {
  const uint32_t wh = static_cast<uint32_t>(min(win, gh)), ww = static_cast<uint32_t>(min(win, gw));
  const uint32_t ugh = static_cast<uint32_t>(gh), ugw = static_cast<uint32_t>(gw), up = static_cast<uint32_t>(p);
  const uint32_t row_span = wh * ugw;
  const uint32_t by = up / row_span;
  const uint32_t rem = up - by * row_span;
  const uint32_t bh = min(wh, ugh - by * wh);
  const uint32_t blk_span = bh * ww;
  const uint32_t bx = rem / blk_span;
  const uint32_t rem2 = rem - bx * blk_span;
  const uint32_t bw = min(ww, ugw - bx * ww);
  const uint32_t ry = rem2 / bw;
  return static_cast<int>((by * wh + ry) * ugw + bx * ww + (rem2 - ry * bw));
}

// Patch coordinates (0-based) of batch token t, for tokens in raster order (win == 0)
// or in the window order of window win.
__device__ inline void token_patch(const ImageTable& tb, int win, int t, int* row, int* col) {
  const int img = image_of(tb, t);
  const int p = t - tb.start[img];
  const int gw = tb.gw[img];
  const int r = win > 0 ? window_to_raster(p, tb.gh[img], gw, win) : p;
  *row = r / gw;
  *col = r % gw;
}

// Cosine and sine of one rotation pair at 1-based position pos, frequency f (radians
// per position), for f32 results.
__device__ inline void rope_angle(float pos, float f, float* c, float* s) { sincosf(pos * f, s, c); }

// The same for bf16 results, from the hardware sine and cosine (v_sin_f32 / v_cos_f32
// take the angle in revolutions): the angle pos*f/(2 pi) in f32, reduced to [0, 1) by
// an exact fraction.  The angle carries a relative error of a few 2^-24 (|angle| <
// 2^8 revolutions for positions below ~1600 at f <= 1), far below the 2^-8 rounding of
// the bf16 result.  Every kernel that rotates bf16 (the RoPE pass, the attention
// kernel rotating Q on load) calls this one, so they agree bit for bit.
__device__ inline void rope_angle_bf16(float pos, float f, float* c, float* s) {
  const float rev = __builtin_amdgcn_fractf(pos * f * 0.159154943091895336f);
  *s = __builtin_amdgcn_sinf(rev);
  *c = __builtin_amdgcn_cosf(rev);
}

// One rotation pair stored as two bf16 in a 32-bit word (low half the real part):
// (re + i im) * (c + i s), rounded to bf16.  The products are written out so that every
// kernel that rotates (the RoPE pass, the attention kernel rotating Q on load) rounds
// the same way: fma(re, c, -(im*s)) and fma(re, s, im*c).
__device__ inline uint32_t rope_pair_bf16(uint32_t w, float c, float s) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const float re = __uint_as_float(w << 16), im = __uint_as_float(w & 0xffff0000u);
  const float ims = im * s, imc = im * c;
  // both halves rounded to bf16 (RNE) by one packed conversion
  const bf16x2_t r = {static_cast<__bf16>(__builtin_fmaf(re, c, -ims)), static_cast<__bf16>(__builtin_fmaf(re, s, imc))};
  return __builtin_bit_cast(uint32_t, r);
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
// computed once.  A head's H*d values are P = d*elem/16 pieces of 16 bytes (8 bf16 or 4
// f32: whole pairs of one half of a head, as d/2 is a multiple of 8), and lane l < G*P,
// G = 64/P, always takes piece l mod P of head l/P of each group of G heads, so the
// cosines and sines of its pieces' pairs (pairs below d/4 rotate by the column, the rest
// by the row, frequency index pair mod d/4) are computed once per token in the lane
// that uses them, and a group's G*P pieces are one contiguous stretch of the row.
template <typename T>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void rope2d_kernel(RopeArgs a, int32_t n_tokens) {
  constexpr int kPer = 16 / sizeof(T);  // values per piece
  constexpr int kPairs = kPer / 2;      // rotation pairs per piece
  const int t = __builtin_amdgcn_readfirstlane(static_cast<int>(blockIdx.x) * 4 + (threadIdx.x >> 6));
  if (t >= n_tokens) return;
  const int lane = threadIdx.x & 63;
  const int P = a.pieces, G = 64 / P;  // pieces per head, heads per group (P <= 32)
  const int g = lane / P, pc = lane - g * P;
  const bool active = g < G;
  int prow = 0, pcol = 0;
  token_patch(a.tb, a.win, t, &prow, &pcol);
  const int quarter = a.d / 4;  // pairs per half of a head
  T* row = static_cast<T*>(a.x) + static_cast<int64_t>(t) * a.ld;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  constexpr int kU = 4;  // head groups per trip, their loads in flight together
  float cs[kPairs], sn[kPairs];
  for (int h0 = 0; h0 < a.H; h0 += G * kU) {
    u32x4 raw[kU];
    int off[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int head = min(h0 + u * G + g, a.H - 1);  // inactive lanes and heads past the end re-read a piece
      off[u] = head * a.d + pc * kPer;
      raw[u] = *reinterpret_cast<const u32x4*>(row + off[u]);
    }
    if (h0 == 0) {  // the angles of this lane's pairs, while the first loads are in flight
#pragma unroll
      for (int k = 0; k < kPairs; ++k) {
        const int pair = pc * kPairs + k;
        const float pos = static_cast<float>(pair < quarter ? pcol + 1 : prow + 1);
        const float f = a.inv_freq[pair % quarter];
        if constexpr (sizeof(T) == 2) rope_angle_bf16(pos, f, &cs[k], &sn[k]);
        else rope_angle(pos, f, &cs[k], &sn[k]);
      }
    }
    asm volatile("" ::"v"(raw[0]), "v"(raw[1]), "v"(raw[2]), "v"(raw[3]));
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      uint32_t w[4] = {raw[u][0], raw[u][1], raw[u][2], raw[u][3]};
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = rope_pair_bf16(w[k], cs[k], sn[k]);
      } else {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const float re = __uint_as_float(w[2 * k]), im = __uint_as_float(w[2 * k + 1]);
          const float ims = im * sn[k], imc = im * cs[k];
          w[2 * k] = __float_as_uint(__builtin_fmaf(re, cs[k], -ims));
          w[2 * k + 1] = __float_as_uint(__builtin_fmaf(re, sn[k], imc));
        }
      }
      if (active && h0 + u * G + g < a.H) *reinterpret_cast<u32x4*>(row + off[u]) = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}

}  // namespace mgattn
