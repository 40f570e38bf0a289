// One-token decoding of the text decoder's attention (mbext next-steps page,
// "Architecture / Text decoder": grouped key/value heads, a local window of 2048
// tokens, incremental decoding with a KV cache), bf16, split over the keys.
//
// A workgroup = one (sequence, key/value head): the G <= 32 query heads of the group,
// for the sequence's single new token, are the 32 columns of the score tile (S^T =
// K Q^T with v_mfma_f32_32x32x16_bf16, columns >= G zero).  The visible keys (the last
// `window` of the cache, or all of it) are split into contiguous 32-key blocks, and
// wave w takes the w-th eighth of them: each wave runs its own online softmax over
// its keys (K operands loaded straight from HBM one block ahead; V blocks staged by
// LDS DMA into the wave's own double buffer and read transposed with
// ds_read_b64_tr_b16).  At the end the eight partial results (m, l, O) are merged
// through LDS: O = sum_w 2^{(m_w - M) c} O_w / sum_w 2^{(m_w - M) c} l_w.
// K and V of the window are read exactly once.
//
// With few sequences (n_seq * Hkv well below the 256 CUs) the keys are further split
// over nsplit workgroups per (sequence, key/value head), each taking a contiguous
// range of blocks; they write their merged (M, den, O / den) to a caller-provided
// workspace in f32, and attn_decode_combine merges the nsplit partial results the
// same way (weights 2^{(M_s - M) c} den_s) into the bf16 output.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_bf16.hpp"
#include "plan.hpp"

namespace mgattn {

template <int D>
struct DecodeTile {
  static constexpr int kWaves = 8;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBlockElems = 32 * D;                    // one 32-key V block
  static constexpr int kWaveElems = 2 * kBlockElems;             // double buffer per wave
  static constexpr int kVBytes = kWaves * kWaveElems * 2;
  static constexpr int kMergeBytes = kWaves * (D * 32 + 64) * 4;  // O tiles + m, l per wave
  static constexpr int kLdsBytes = kVBytes > kMergeBytes ? kVBytes : kMergeBytes;
  static_assert(kLdsBytes <= 160 * 1024, "LDS of one CU");
  static_assert(D % 32 == 0 && D <= 128, "head_dim must be a multiple of 32 up to 128");
};

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void attn_decode_bf16(KernelArgs a) {
  using TL = DecodeTile<D>;
  constexpr int KS = D / 16;  // MFMA k-steps over head_dim
  constexpr int CT = D / 32;  // 32-channel output tiles
  constexpr int VDMA = 32 * D / 8 / 64;  // LDS DMA instructions per V block
  constexpr float kRescaleLog2 = 8.0f;

  __shared__ __attribute__((aligned(16))) __bf16 lds[TL::kLdsBytes / 2];

  const int Hkv = a.H;  // key/value heads
  const int nsplit = a.nsplit;
  const int wg = blockIdx.x / nsplit, split = blockIdx.x % nsplit;  // wg = (sequence, key/value head)
  const int slot = wg / Hkv, g = wg % Hkv;
  if (slot >= a.table.n) return;
  const int G = a.hq_per_kv;
  const int Lk = a.table.klen[slot];
  const int k_lo = a.window > 0 ? max(0, Lk - a.window) : 0;  // first visible key
  const int nblk_all = (Lk - k_lo + 31) / 32;
  // this workgroup's blocks: [sb0, sb0 + nblk) (possibly none when nsplit > 1)
  const int sb0 = nblk_all * split / nsplit;
  const int nblk = nblk_all * (split + 1) / nsplit - sb0;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;   // score column: query head g*G + n
  const int hf = lane >> 5;
  const float c = a.c;
  // this wave's blocks
  const int b_begin = sb0 + nblk * wave / TL::kWaves, b_end = sb0 + nblk * (wave + 1) / TL::kWaves;

  const __bf16* __restrict__ kg =
      static_cast<const __bf16*>(a.k) + static_cast<size_t>(a.table.kstart[slot]) * a.ldk + static_cast<size_t>(g) * D;
  const __bf16* __restrict__ vg =
      static_cast<const __bf16*>(a.v) + static_cast<size_t>(a.table.kstart[slot]) * a.ldv + static_cast<size_t>(g) * D;

  // Q fragments: column n = query head g*G + n of the sequence's token, channels
  // 16s + 8hf + [0,8); columns >= G are zero.
  bf16x8 qf[KS];
  if (n < G) {
    const bf16x8* p = reinterpret_cast<const bf16x8*>(
        static_cast<const __bf16*>(a.q) + static_cast<size_t>(a.table.start[slot]) * a.ldq +
        static_cast<size_t>(g * G + n) * D + 8 * hf);
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = p[2 * s];
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = bf16x8{};
  }
  if (a.qsign != 1) {
    const __bf16 sg = static_cast<__bf16>(static_cast<float>(a.qsign));
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = qf[s] * sg;
  }

  __bf16* vbuf = lds + wave * TL::kWaveElems;
  auto key_of = [&](int blk, int i) { return min(k_lo + blk * 32 + i, Lk - 1); };  // clamped row
  auto load_k = [&](int blk, bf16x8(&kf)[KS]) {
    const bf16x8* p = reinterpret_cast<const bf16x8*>(kg + static_cast<size_t>(key_of(blk, n)) * a.ldk + 8 * hf);
#pragma unroll
    for (int s = 0; s < KS; ++s) kf[s] = p[2 * s];
  };
  auto issue_v = [&](int blk) {  // V block -> this wave's buffer blk & 1, row-major, pitch D
    __bf16* dst = vbuf + (blk & 1) * TL::kBlockElems;
#pragma unroll
    for (int u = 0; u < VDMA; ++u) {
      const int slot16 = u * 64 + lane;
      dma16(vg + static_cast<size_t>(key_of(blk, slot16 / (D / 8))) * a.ldv + (slot16 % (D / 8)) * 8,
            __builtin_amdgcn_readfirstlane(lds_addr(dst + u * 512)));
    }
  };

  f32x16 o[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) o[ct] = f32x16{};
  float m_run = -1.0e30f, l_run = 0.0f;
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  const int tr_row = ((lane & 15) >> 2) + 4 * hf;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // Two blocks in flight: blocks b and b+1 are loaded before block b is waited for
  // (counted: block b+1's KS K loads and VDMA V copies may still be outstanding), and
  // block b+2 goes out once block b's operands are consumed -- its V into the buffer
  // block b just vacated.
  bf16x8 kcur[KS], knext[KS];
  if (b_begin < b_end) {
    load_k(b_begin, kcur);
    issue_v(b_begin);
  }
  if (b_begin + 1 < b_end) {
    load_k(b_begin + 1, knext);
    issue_v(b_begin + 1);
  }
  for (int blk = b_begin; blk < b_end; ++blk) {
    const bool more = blk + 1 < b_end;
    dma_wait_leave(more ? KS + VDMA : 0);
    // scores of this block
    f32x16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur[0], qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
    for (int st = 1; st < KS; ++st) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kcur[st], qf[st], s, 0, 0, 0);
    const int key0 = k_lo + blk * 32;
    if (key0 + 32 > Lk) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (key0 + acc_row(r, hf) >= Lk) s[r] = -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    const float m_blk = half_swap_max(mx);
    if (__builtin_amdgcn_ballot_w64((m_blk - m_run) * c > kRescaleLog2)) {
      const float m_new = fmaxf(m_run, m_blk);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) o[ct] *= alpha;
    }
    const float mc = m_run * c;
    bf16x8 pk[2];
    float lsum = 0.0f;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pk[h2][e] = static_cast<__bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * h2 + e], c, -mc)));
#pragma unroll
      for (int e = 0; e < 8; e += 2)
        lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pk[h2][e], pk[h2][e + 1]}, ones, lsum, false);
    }
    l_run += lsum;
    const __bf16* vt = vbuf + (blk & 1) * TL::kBlockElems;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const __bf16* vrow = vt + (h2 * 16 + tr_row) * D + tr_col;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const bf16x4 lo = ds_read_tr(vrow + ct * 32);
        const bf16x4 hi = ds_read_tr(vrow + 8 * D + ct * 32);
        o[ct] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7),
                                                         pk[h2], o[ct], 0, 0, 0);
      }
    }
#pragma unroll
    for (int st = 0; st < KS; ++st) kcur[st] = knext[st];
    if (blk + 2 < b_end) {
      load_k(blk + 2, knext);
      issue_v(blk + 2);
    }
  }
  const float l_all = half_swap_sum(l_run);

  // ---- merge the eight partial results through LDS (the V buffers are dead once
  // every wave has passed the barrier).  Each wave stores its O tile as one float4 per
  // lane and (output tile ct, register quad r4): slot [wave][ct][r4][lane], so a lane
  // reads back the same four channels of the same query column from every wave, and
  // the CT*4 slices are shared out over the waves.  Lane (n, hf) of slice (ct, r4)
  // holds channels ct*32 + 8 r4 + 4 hf + [0, 4) of query column n.
  __syncthreads();
  constexpr int NSL = CT * 4;                          // float4 slices per lane
  f32x4* o_w = reinterpret_cast<f32x4*>(lds);          // [wave][NSL][64]
  float* m_w = reinterpret_cast<float*>(o_w + TL::kWaves * NSL * 64);  // [wave][32]
  float* l_w = m_w + TL::kWaves * 32;                  // [wave][32]
  static_assert((TL::kWaves * NSL * 64 * 4 + TL::kWaves * 64) * 4 <= TL::kLdsBytes, "merge buffers inside LDS");
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      o_w[(wave * NSL + ct * 4 + r4) * 64 + lane] =
          f32x4{o[ct][4 * r4], o[ct][4 * r4 + 1], o[ct][4 * r4 + 2], o[ct][4 * r4 + 3]};
  if (hf == 0) {
    m_w[wave * 32 + n] = m_run;
    l_w[wave * 32 + n] = l_all;
  }
  __syncthreads();
  // weights of the eight waves for this lane's column: 2^{(m_w - M) c}, den = sum f_w l_w
  float M = m_w[n];
#pragma unroll
  for (int w = 1; w < TL::kWaves; ++w) M = fmaxf(M, m_w[w * 32 + n]);
  float f[TL::kWaves], den = 0.0f;
#pragma unroll
  for (int w = 0; w < TL::kWaves; ++w) {
    f[w] = __builtin_amdgcn_exp2f((m_w[w * 32 + n] - M) * c);
    den = __builtin_fmaf(f[w], l_w[w * 32 + n], den);
  }
  const bool col_ok = n < G;
  __bf16* og = static_cast<__bf16*>(a.o) + static_cast<size_t>(a.table.start[slot]) * a.ldo +
               static_cast<size_t>(g * G + n) * D + 4 * hf;
  const size_t ps = static_cast<size_t>(wg) * nsplit + split;  // partial-result slot
  // partial result of this split: O / den (0 for a split without keys), M, den
  const float inv = nsplit == 1 ? 1.0f / den : (den > 0.0f ? 1.0f / den : 0.0f);
  for (int sl = wave; sl < NSL; sl += TL::kWaves) {
    f32x4 acc = o_w[sl * 64 + lane] * f[0];
#pragma unroll
    for (int w = 1; w < TL::kWaves; ++w) {
      const f32x4 x = o_w[(w * NSL + sl) * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(x[e], f[w], acc[e]);
    }
    const int ch0 = (sl / 4) * 32 + (sl % 4) * 8;
    if (!col_ok) continue;
    if (nsplit == 1) {
      bf16x4 val;
#pragma unroll
      for (int e = 0; e < 4; ++e) val[e] = static_cast<__bf16>(acc[e] * inv);
      *reinterpret_cast<bf16x4*>(og + ch0) = val;
    } else {
      *reinterpret_cast<f32x4*>(a.part + (ps * 32 + n) * D + ch0 + 4 * hf) = acc * inv;
    }
  }
  if (nsplit > 1 && wave == 0 && hf == 0 && col_ok) {
    float* ml = a.part + static_cast<size_t>(a.table.n) * Hkv * nsplit * 32 * D + ps * 64;
    ml[n] = M;
    ml[32 + n] = den;
  }
}

// The same decoding for groups of G <= 16 query heads (the text decoder's 32 / 2), on
// v_mfma_f32_16x16x32_bf16 (lane l = 16 gq + n), whose 16 columns are the group's heads:
// no zero columns, so half the products, exponentials and merge traffic of the 32-column
// tile above.  S^T = K Q^T per 16-key half of a 32-key block: step s contracts channels
// 32 s + 8 gq + [0, 8) (lane n holds key row n of the half, lane group gq 16 bytes of it,
// so a K load instruction reads 16 rows x 64 bytes), and the accumulator holds keys
// 4 gq + r of the half for head n.  O^T += V^T P^T contracts the 32 keys of the block in
// one step, lane group gq supplying keys 4 gq + [0, 4) and 16 + 4 gq + [0, 4): exactly
// the probabilities its own accumulators hold, so P never leaves its lane; the V^T
// operand comes from two ds_read_b64_tr_b16 (within 16 lanes: a 4-row x 16-column tile
// read row by row, received column by column) at rows 4 gq + [0, 4) and 16 + that.  Row
// maxima and sums combine the four lane groups with two lane swaps (16, then 32).
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void attn_decode_bf16_g16(KernelArgs a) {
  using TL = DecodeTile<D>;
  constexpr int KS = D / 32;  // QK steps over head_dim
  constexpr int CT = D / 16;  // 16-channel output tiles
  constexpr int VDMA = 32 * D / 8 / 64;  // LDS DMA instructions per V block
  constexpr float kRescaleLog2 = 8.0f;

  __shared__ __attribute__((aligned(16))) __bf16 lds[TL::kLdsBytes / 2];

  const int Hkv = a.H;
  const int nsplit = a.nsplit;
  const int wg = blockIdx.x / nsplit, split = blockIdx.x % nsplit;
  const int slot = wg / Hkv, g = wg % Hkv;
  if (slot >= a.table.n) return;
  const int G = a.hq_per_kv;
  const int Lk = a.table.klen[slot];
  const int k_lo = a.window > 0 ? max(0, Lk - a.window) : 0;
  const int nblk_all = (Lk - k_lo + 31) / 32;
  const int sb0 = nblk_all * split / nsplit;
  const int nblk = nblk_all * (split + 1) / nsplit - sb0;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 15;   // head column / key row of a 16-key half
  const int gq = lane >> 4;  // lane group
  const float c = a.c;
  const int b_begin = sb0 + nblk * wave / TL::kWaves, b_end = sb0 + nblk * (wave + 1) / TL::kWaves;

  const __bf16* __restrict__ kg =
      static_cast<const __bf16*>(a.k) + static_cast<size_t>(a.table.kstart[slot]) * a.ldk + static_cast<size_t>(g) * D;
  const __bf16* __restrict__ vg =
      static_cast<const __bf16*>(a.v) + static_cast<size_t>(a.table.kstart[slot]) * a.ldv + static_cast<size_t>(g) * D;

  // Q fragments: head g*G + n, channels 32 s + 8 gq + [0, 8); heads >= G are zero
  bf16x8 qf[KS];
  if (n < G) {
    const bf16x8* p = reinterpret_cast<const bf16x8*>(
        static_cast<const __bf16*>(a.q) + static_cast<size_t>(a.table.start[slot]) * a.ldq +
        static_cast<size_t>(g * G + n) * D + 8 * gq);
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = p[4 * s];
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = bf16x8{};
  }
  if (a.qsign != 1) {
    const __bf16 sg = static_cast<__bf16>(static_cast<float>(a.qsign));
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = qf[s] * sg;
  }

  __bf16* vbuf = lds + wave * TL::kWaveElems;
  auto key_of = [&](int blk, int i) { return min(k_lo + blk * 32 + i, Lk - 1); };  // clamped row
  auto load_k = [&](int blk, bf16x8(&kf)[2][KS]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16x8* p = reinterpret_cast<const bf16x8*>(kg + static_cast<size_t>(key_of(blk, 16 * h + n)) * a.ldk + 8 * gq);
#pragma unroll
      for (int s = 0; s < KS; ++s) kf[h][s] = p[4 * s];
    }
  };
  auto issue_v = [&](int blk) {  // V block -> this wave's buffer blk & 1, row-major, pitch D
    __bf16* dst = vbuf + (blk & 1) * TL::kBlockElems;
#pragma unroll
    for (int u = 0; u < VDMA; ++u) {
      const int slot16 = u * 64 + lane;
      dma16(vg + static_cast<size_t>(key_of(blk, slot16 / (D / 8))) * a.ldv + (slot16 % (D / 8)) * 8,
            __builtin_amdgcn_readfirstlane(lds_addr(dst + u * 512)));
    }
  };

  f32x4 o[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) o[ct] = f32x4{};
  float m_run = -1.0e30f, l_run = 0.0f;
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  // V^T operand rows (keys) 4 gq + n/4 and 16 + that, columns 16 ct + 4 (n % 4)
  const int tr_off = (4 * gq + (n >> 2)) * D + 4 * (n & 3);

  // Two blocks in flight, as in attn_decode_bf16: blocks b and b+1 are loaded before
  // block b is waited for (counted), and block b+2 goes out once block b is consumed.
  bf16x8 kcur[2][KS], knext[2][KS];
  if (b_begin < b_end) {
    load_k(b_begin, kcur);
    issue_v(b_begin);
  }
  if (b_begin + 1 < b_end) {
    load_k(b_begin + 1, knext);
    issue_v(b_begin + 1);
  }
  for (int blk = b_begin; blk < b_end; ++blk) {
    const bool more = blk + 1 < b_end;
    dma_wait_leave(more ? 2 * KS + VDMA : 0);
    f32x4 sc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kcur[h][0], qf[0], f32x4{}, 0, 0, 0);
#pragma unroll
      for (int s = 1; s < KS; ++s) sc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kcur[h][s], qf[s], sc[h], 0, 0, 0);
    }
    const int key0 = k_lo + blk * 32;
    if (key0 + 32 > Lk) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (key0 + 16 * h + 4 * gq + r >= Lk) sc[h][r] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3]));
    mx = fmaxf(mx, fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    const float m_blk = half_swap_max(row16_swap_max(mx));
    if (__builtin_amdgcn_ballot_w64((m_blk - m_run) * c > kRescaleLog2)) {
      const float m_new = fmaxf(m_run, m_blk);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) o[ct] *= alpha;
    }
    const float mc = m_run * c;
    // P^T operand: keys 4 gq + [0, 4) (half 0), then 16 + 4 gq + [0, 4) (half 1)
    bf16x8 pk;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) pk[4 * h + r] = static_cast<__bf16>(__builtin_amdgcn_exp2f(__builtin_fmaf(sc[h][r], c, -mc)));
    float lsum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; e += 2) lsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pk[e], pk[e + 1]}, ones, lsum, false);
    l_run += lsum;
    const __bf16* vt = vbuf + (blk & 1) * TL::kBlockElems + tr_off;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const bf16x4 lo = ds_read_tr(vt + 16 * ct);
      const bf16x4 hi = ds_read_tr(vt + 16 * D + 16 * ct);
      o[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pk, o[ct],
                                                      0, 0, 0);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int s = 0; s < KS; ++s) kcur[h][s] = knext[h][s];
    if (blk + 2 < b_end) {
      load_k(blk + 2, knext);
      issue_v(blk + 2);
    }
  }
  const float l_all = half_swap_sum(row16_swap_sum(l_run));  // over the four lane groups' keys

  // ---- merge the eight partial results through LDS, as in attn_decode_bf16: slot
  // [wave][ct][lane] holds lane (gq, n)'s channels 16 ct + 4 gq + [0, 4) of head n, and
  // wave w merges the slices ct = w, w + 8, ...
  __syncthreads();
  f32x4* o_w = reinterpret_cast<f32x4*>(lds);                        // [wave][CT][64]
  float* m_w = reinterpret_cast<float*>(o_w + TL::kWaves * CT * 64);  // [wave][16]
  float* l_w = m_w + TL::kWaves * 16;                                 // [wave][16]
  static_assert((TL::kWaves * CT * 64 * 4 + TL::kWaves * 32) * 4 <= TL::kLdsBytes, "merge buffers inside LDS");
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) o_w[(wave * CT + ct) * 64 + lane] = o[ct];
  if (gq == 0) {
    m_w[wave * 16 + n] = m_run;
    l_w[wave * 16 + n] = l_all;
  }
  __syncthreads();
  float M = m_w[n];
#pragma unroll
  for (int w = 1; w < TL::kWaves; ++w) M = fmaxf(M, m_w[w * 16 + n]);
  float f[TL::kWaves], den = 0.0f;
#pragma unroll
  for (int w = 0; w < TL::kWaves; ++w) {
    f[w] = __builtin_amdgcn_exp2f((m_w[w * 16 + n] - M) * c);
    den = __builtin_fmaf(f[w], l_w[w * 16 + n], den);
  }
  const bool col_ok = n < G;
  __bf16* og = static_cast<__bf16*>(a.o) + static_cast<size_t>(a.table.start[slot]) * a.ldo +
               static_cast<size_t>(g * G + n) * D + 4 * gq;
  const size_t ps = static_cast<size_t>(wg) * nsplit + split;  // partial-result slot
  const float inv = nsplit == 1 ? 1.0f / den : (den > 0.0f ? 1.0f / den : 0.0f);
  for (int ct = wave; ct < CT; ct += TL::kWaves) {
    f32x4 acc = o_w[ct * 64 + lane] * f[0];
#pragma unroll
    for (int w = 1; w < TL::kWaves; ++w) {
      const f32x4 x = o_w[(w * CT + ct) * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(x[e], f[w], acc[e]);
    }
    if (!col_ok) continue;
    if (nsplit == 1) {
      bf16x4 val;
#pragma unroll
      for (int e = 0; e < 4; ++e) val[e] = static_cast<__bf16>(acc[e] * inv);
      *reinterpret_cast<bf16x4*>(og + 16 * ct) = val;
    } else {
      *reinterpret_cast<f32x4*>(a.part + (ps * 32 + n) * D + 16 * ct + 4 * gq) = acc * inv;
    }
  }
  if (nsplit > 1 && wave == 0 && gq == 0 && col_ok) {
    float* ml = a.part + static_cast<size_t>(a.table.n) * Hkv * nsplit * 32 * D + ps * 64;
    ml[n] = M;
    ml[32 + n] = den;
  }
}

// Merge of the nsplit (<= kMaxSplit) partial results of one (sequence, key/value head):
// one workgroup of 256 threads, a thread per (query head of the group, 8 channels).
constexpr int kMaxSplit = 16;
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256))) void attn_decode_combine(KernelArgs a) {
  const int Hkv = a.H;
  const int nsplit = a.nsplit;
  const int wg = blockIdx.x;
  const int slot = wg / Hkv, g = wg % Hkv;
  if (slot >= a.table.n) return;
  const int G = a.hq_per_kv;
  const float c = a.c;
  const float* part_o = a.part;
  const float* part_ml = a.part + static_cast<size_t>(a.table.n) * Hkv * nsplit * 32 * D;
  __bf16* og = static_cast<__bf16*>(a.o) + static_cast<size_t>(a.table.start[slot]) * a.ldo;
  for (int piece = threadIdx.x; piece < G * D / 8; piece += 256) {
    const int col = piece / (D / 8), ch0 = (piece % (D / 8)) * 8;
    // every load of the piece is issued before any is used (splits unrolled up to the
    // maximum, predicated), so the merge costs one memory round trip
    float Ms[kMaxSplit], dens[kMaxSplit];
    f32x4 x0[kMaxSplit], x1[kMaxSplit];
#pragma unroll
    for (int sp = 0; sp < kMaxSplit; ++sp) {
      if (sp < nsplit) {
        const size_t ps = static_cast<size_t>(wg) * nsplit + sp;
        Ms[sp] = part_ml[ps * 64 + col];
        dens[sp] = part_ml[ps * 64 + 32 + col];
        const f32x4* po = reinterpret_cast<const f32x4*>(part_o + (ps * 32 + col) * D + ch0);
        x0[sp] = po[0];
        x1[sp] = po[1];
      }
    }
    float M = -1.0e30f;
#pragma unroll
    for (int sp = 0; sp < kMaxSplit; ++sp)
      if (sp < nsplit) M = fmaxf(M, Ms[sp]);
    float tot = 0.0f, acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int sp = 0; sp < kMaxSplit; ++sp) {
      if (sp < nsplit) {
        const float F = __builtin_amdgcn_exp2f((Ms[sp] - M) * c) * dens[sp];
        tot += F;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[e] += F * x0[sp][e];
          acc[4 + e] += F * x1[sp][e];
        }
      }
    }
    const float inv = 1.0f / tot;
    bf16x8 val;
#pragma unroll
    for (int e = 0; e < 8; ++e) val[e] = static_cast<__bf16>(acc[e] * inv);
    *reinterpret_cast<bf16x8*>(og + static_cast<size_t>(g * G + col) * D + ch0) = val;
  }
}

}  // namespace mgattn
