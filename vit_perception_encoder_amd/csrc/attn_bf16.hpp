// Single-pass online-softmax attention, bf16 inputs, f32 accumulation, gfx950.
//
// What it computes is the segmented softmax attention of the Muse Glimmer vision
// tower (vllm.cpp issue #1545, sections "Why this one is bad" and "The fix"): each
// segment of cu_seqlens is attended on its own, non-causal unless asked.  The flash
// rung the pages route the tower to (PR #1579, "Numerics, both halves") reaches the
// same function with a running online softmax; this kernel does too, designed for
// CDNA4 rather than after that CUDA kernel.
//
// Layout of the work (one workgroup = 8 waves = one (segment, head, 256-query tile);
// two waves share each SIMD, so one wave's softmax overlaps the other's MFMAs):
//   * Each wave owns 32 queries (one 32-query block).  Scores are computed
//     transposed, S^T = K * Q^T, with v_mfma_f32_32x32x16_bf16: K is the A operand
//     (keys are MFMA rows), Q^T the B operand (queries are MFMA columns).  In the
//     32x32 accumulator a lane then holds ONE query and 16 of the 32 keys (rows
//     8*(r/4) + 4*(lane/32) + r%4), so the row max and row sum are in-lane chains
//     plus a single exchange between lanes l and l^32 (v_permlane32_swap).
//   * head_dim is the contraction of S^T: D/16 MFMA k-steps (96 = 6 x 16).
//   * O^T = V^T * P^T, again 32x32x16: V^T is the A operand, P^T the B operand.  A
//     lane's P^T operand is exactly the 8 probabilities it already holds for one
//     16-key group, converted to bf16 in place: no cross-lane shuffle of P.  The
//     matching V^T operand is read from LDS, where V is stored transposed and with
//     the keys of each 16-key group permuted ([0-3, 8-11 | 4-7, 12-15]) so that
//     those 8 keys are one contiguous 16-byte read.  O^T is D/32 accumulators of
//     32x32 (96 = 3 x 32); a lane holds one query's 16 output channels per tile.
//   * K/V tiles of 128 keys go HBM -> registers -> LDS, double-buffered: the next
//     tile's global loads are in flight during the current tile's MFMA work, and
//     one barrier per tile separates the buffers.  LDS rows are padded (K pitch
//     D+8, V^T pitch 128+8 elements) so every 16-byte MFMA operand read is free of
//     bank conflicts.  A tile is two softmax steps of 64 keys (32 scores per lane).
//   * Softmax uses exp2 with scale*log2(e) folded into one FMA per score, against a
//     reference maximum per query: the first tile's row maximum.  Later tiles do not
//     recompute the maximum.  Exactness does not depend on the reference (numerator
//     and denominator share it); only range does, so a tile whose partial row sum
//     exceeds 2^64 (or is not finite) is redone after refreshing the reference to
//     the true maximum and rescaling O and the row sum (a rare, wave-uniform path).
//   * The row sum adds the bf16-rounded probabilities that feed the PV product
//     (v_dot2 with ones), so the weights stay normalised.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "plan.hpp"

namespace mgattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct KernelArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int32_t H;
  int32_t causal;
  float c;        // |scale| * log2(e)
  int32_t negate; // 1 when scale < 0 (Q is negated in registers; exact)
  SegTable table;
};

template <int D>
struct Bf16Tile {
  static constexpr int kWaves = 8;
  static constexpr int kQBlocks = 1;                     // 32-query blocks per wave
  static constexpr int kBlockM = kWaves * kQBlocks * 32; // queries per workgroup
  static constexpr int kBlockN = 128;                    // keys per LDS tile
  static constexpr int kStepKeys = 64;                   // keys per softmax step
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kKPitch = D + 8;                  // K row pitch (elements)
  static constexpr int kVPitch = kBlockN + 8;            // V^T row pitch (elements)
  static constexpr int kKElems = kBlockN * kKPitch;
  static constexpr int kVElems = D * kVPitch;
  static constexpr int kStageElems = kKElems + kVElems;
  static constexpr int kStages = 2;
  static constexpr int kLdsBytes = kStages * kStageElems * 2;
  static_assert(D % 32 == 0 && D >= 32 && D <= 128, "head_dim must be a multiple of 32 up to 128");
  static_assert(kBlockN % kStepKeys == 0 && kStepKeys % 32 == 0, "LDS tile must hold whole softmax steps");
};

// Exchange with lane l^32 and combine (max or sum) -- one v_permlane32_swap.
__device__ inline float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Key (relative to the 32-key block) held in accumulator register r by lane half hf.
__device__ constexpr int acc_row(int r, int hf) { return 8 * (r >> 2) + 4 * hf + (r & 3); }

// In-place v *= a on every element.  The tied register operand keeps the scaled
// accumulator in the registers it already occupies, so the (rare) rescale branch
// does not force the compiler to copy the accumulators at the branch join.
__device__ inline void scale_in_place(f32x16& v, float a) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float t = v[i];
    asm volatile("v_mul_f32 %0, %0, %1" : "+v"(t) : "v"(a));
    v[i] = t;
  }
}

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void attn_fwd_bf16(KernelArgs a) {
  using TL = Bf16Tile<D>;
  constexpr int BM = TL::kBlockM, BN = TL::kBlockN;
  constexpr int KS = D / 16;   // MFMA k-steps over head_dim
  constexpr int CT = D / 32;   // 32-channel output tiles
  constexpr int NB = TL::kStepKeys / 32;  // 32-key blocks per softmax step
  constexpr int NSTEP = BN / TL::kStepKeys;  // softmax steps per LDS tile
  constexpr int KP = TL::kKPitch, VP = TL::kVPitch;
  constexpr int NT = TL::kThreads;
  constexpr int K_CHUNKS = BN * D / 8;         // 16-byte pieces of a K tile
  constexpr int K_PER_T = (K_CHUNKS + NT - 1) / NT;
  constexpr int V_UNITS = (BN / 4) * (D / 8);  // 4 keys x 8 channels each
  constexpr int V_PER_T = (V_UNITS + NT - 1) / NT;
  // A row's partial sum over one tile above 2^64 means the reference maximum is stale
  // by a wide margin: the tile is redone against a refreshed maximum.
  constexpr float kSumLimit = 18446744073709551616.0f;
  static_assert(TL::kQBlocks == 1, "one 32-query block per wave");

  __shared__ __attribute__((aligned(16))) __bf16 lds[TL::kStages * TL::kStageElems];

  const Tile tile = decode_tile(a.table, a.H, BM, a.causal, blockIdx.x);
  if (!tile.valid) return;
  const int L = a.table.len[tile.slot];
  const int q0 = tile.q0;
  const int rs = a.H * D;  // elements between consecutive tokens
  const size_t base = (static_cast<size_t>(a.table.start[tile.slot]) * a.H + tile.head) * D;
  const __bf16* __restrict__ qg = static_cast<const __bf16*>(a.q) + base;
  const __bf16* __restrict__ kg = static_cast<const __bf16*>(a.k) + base;
  const __bf16* __restrict__ vg = static_cast<const __bf16*>(a.v) + base;
  __bf16* __restrict__ og = static_cast<__bf16*>(a.o) + base;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const float c = a.c;
  const int qr = q0 + wave * 32 + n;  // this lane's query (relative to the segment)
  const int qmin = q0 + wave * 32;    // the wave's first query

  // ---- Q fragments (B operand of S^T): lane holds query qr, channels 16s + 8hf + [0,8)
  bf16x8 qf[KS];
  if (qr < L) {
    const bf16x8* p = reinterpret_cast<const bf16x8*>(qg + static_cast<size_t>(qr) * rs + 8 * hf);
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = p[2 * s];
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = bf16x8{};
  }
  if (a.negate) {
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = -qf[s];
  }

  const int kend = a.causal ? min(L, q0 + BM) : L;
  const int ntiles = (kend + BN - 1) / BN;

  // ---- tile staging: per-thread offsets are fixed, a tile only moves the base
  int k_row[K_PER_T], k_goff[K_PER_T], k_loff[K_PER_T];
#pragma unroll
  for (int i = 0; i < K_PER_T; ++i) {
    const int id = tid + i * NT;
    const int key = id / (D / 8), part = id % (D / 8);
    k_row[i] = (K_CHUNKS % NT == 0 || id < K_CHUNKS) ? key : BN;  // BN: never loaded
    k_goff[i] = key * rs + part * 8;
    k_loff[i] = key * KP + part * 8;
  }
  int v_row[V_PER_T], v_goff[V_PER_T], v_loff[V_PER_T];
#pragma unroll
  for (int i = 0; i < V_PER_T; ++i) {
    const int u = tid + i * NT;
    const int kq = u % (BN / 4), cg = u / (BN / 4);
    // keys 4kq..4kq+3 = 16G + 8a + 4b + [0,4) go to position 16G + 8b + 4a of each V^T row
    const int pos = 16 * (kq >> 2) + 8 * (kq & 1) + 4 * ((kq >> 1) & 1);
    v_row[i] = (V_UNITS % NT == 0 || u < V_UNITS) ? 4 * kq : BN;
    v_goff[i] = 4 * kq * rs + cg * 8;
    v_loff[i] = cg * 8 * VP + pos;
  }
  bf16x8 kreg[K_PER_T];
  bf16x8 vreg[V_PER_T][4];

  auto load_tile = [&](int t) {
    const int kt0 = t * BN;
    const __bf16* kb = kg + static_cast<size_t>(kt0) * rs;
    const __bf16* vb = vg + static_cast<size_t>(kt0) * rs;
    const int lim = L - kt0;  // rows at or past lim are outside the segment
    if (lim >= BN) {
#pragma unroll
      for (int i = 0; i < K_PER_T; ++i)
        if (K_CHUNKS % NT == 0 || k_row[i] < BN) kreg[i] = *reinterpret_cast<const bf16x8*>(kb + k_goff[i]);
#pragma unroll
      for (int i = 0; i < V_PER_T; ++i)
        if (V_UNITS % NT == 0 || v_row[i] < BN) {
#pragma unroll
          for (int j = 0; j < 4; ++j) vreg[i][j] = *reinterpret_cast<const bf16x8*>(vb + v_goff[i] + j * rs);
        }
    } else {
#pragma unroll
      for (int i = 0; i < K_PER_T; ++i)
        kreg[i] = k_row[i] < lim ? *reinterpret_cast<const bf16x8*>(kb + k_goff[i]) : bf16x8{};
#pragma unroll
      for (int i = 0; i < V_PER_T; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          vreg[i][j] = v_row[i] + j < lim ? *reinterpret_cast<const bf16x8*>(vb + v_goff[i] + j * rs) : bf16x8{};
    }
  };

  auto store_tile = [&](int buf) {
    __bf16* ks = lds + buf * TL::kStageElems;
    __bf16* vt = ks + TL::kKElems;
#pragma unroll
    for (int i = 0; i < K_PER_T; ++i)
      if (K_CHUNKS % NT == 0 || k_row[i] < BN) *reinterpret_cast<bf16x8*>(ks + k_loff[i]) = kreg[i];
#pragma unroll
    for (int i = 0; i < V_PER_T; ++i)
      if (V_UNITS % NT == 0 || v_row[i] < BN) {
#pragma unroll
        for (int ch = 0; ch < 8; ++ch) {
          bf16x4 col = {vreg[i][0][ch], vreg[i][1][ch], vreg[i][2][ch], vreg[i][3][ch]};
          *reinterpret_cast<bf16x4*>(vt + v_loff[i] + ch * VP) = col;
        }
      }
  };

  // ---- running state of this lane's query
  f32x16 o[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) o[ct] = f32x16{};
  float m_run = 0.0f, l_run = 0.0f;
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

  load_tile(0);
  store_tile(0);
  __syncthreads();

  // One softmax step of 64 keys: S^T = K Q^T, probabilities against the reference maximum,
  // O^T += V^T P^T.  MASKED is a compile-time flag so interior tiles carry no
  // per-score checks.
  auto tile_step = [&](auto masked_tag, const __bf16* ks, const __bf16* vt, int kb0, int key0, bool first) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    f32x16 s[NB];
    // keys past the segment end, and (causal) keys after the query, take no weight
    auto dead = [&](int b, int r) {
      const int key = key0 + b * 32 + acc_row(r, hf);
      return key >= L || (a.causal && key > qr);
    };
    auto scores = [&]() {
#pragma unroll
      for (int b = 0; b < NB; ++b) s[b] = f32x16{};
#pragma unroll
      for (int st = 0; st < KS; ++st)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ks + ((kb0 + b) * 32 + n) * KP + 16 * st + 8 * hf);
          s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[st], s[b], 0, 0, 0);
        }
      if constexpr (MASKED) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (dead(b, r)) s[b][r] = -INFINITY;
      }
    };
    auto row_max = [&]() {
      float mx = s[0][0];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[b][r]);
      return half_swap_max(mx);
    };
    scores();
    if (first) m_run = row_max();

    // probabilities -> bf16 B operands of the PV product; this lane's share of the
    // row sum, over the same rounded values
    bf16x8 pk[NB][2];
    float lsum;
    auto probabilities = [&]() {
      const float mc = m_run * c;
      lsum = 0.0f;
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          bf16x8 pv;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][8 * h2 + e], c, -mc));
            if constexpr (MASKED) p = dead(b, 8 * h2 + e) ? 0.0f : p;
            pv[e] = static_cast<__bf16>(p);
          }
          pk[b][h2] = pv;
#pragma unroll
          for (int e = 0; e < 8; e += 2)
            lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pv[e], pv[e + 1]}, ones, lsum, false);
        }
    };
    probabilities();
    // A stale maximum shows as a huge (or non-finite) partial sum: recompute the
    // scores, refresh the maximum, rescale, redo.  Recomputing S here (rare) instead
    // of keeping it live keeps the common path inside the register budget.
    if (__builtin_amdgcn_ballot_w64(!(lsum <= kSumLimit))) {
      scores();
      const float m_new = fmaxf(m_run, row_max());
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) scale_in_place(o[ct], alpha);
      probabilities();
    }
    l_run += lsum;

    // O^T += V^T P^T
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const bf16x8 vf =
              *reinterpret_cast<const bf16x8*>(vt + (ct * 32 + n) * VP + (kb0 + b) * 32 + h2 * 16 + 8 * hf);
          o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pk[b][h2], o[ct], 0, 0, 0);
        }
  };

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const __bf16* ks = lds + buf * TL::kStageElems;
    const __bf16* vt = ks + TL::kKElems;
#pragma unroll
    for (int j = 0; j < NSTEP; ++j) {
      const int key0 = t * BN + j * TL::kStepKeys;
      if (key0 >= kend) break;  // workgroup-uniform: the rest of the tile is past the end
      const bool masked = (key0 + TL::kStepKeys > L) || (a.causal && key0 + TL::kStepKeys - 1 > qmin);
      if (masked)
        tile_step(std::true_type{}, ks, vt, j * NB, key0, t == 0 && j == 0);
      else
        tile_step(std::false_type{}, ks, vt, j * NB, key0, t == 0 && j == 0);
    }
    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O / l, bf16 (round to nearest even), rows inside the segment only
  const float inv = 1.0f / half_swap_sum(l_run);
  if (qr < L) {
    __bf16* dst = og + static_cast<size_t>(qr) * rs + 4 * hf;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 val;
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = static_cast<__bf16>(o[ct][4 * r4 + e] * inv);
        *reinterpret_cast<bf16x4*>(dst + ct * 32 + r4 * 8) = val;
      }
  }
}

}  // namespace mgattn
