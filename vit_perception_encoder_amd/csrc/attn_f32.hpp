// Single-pass online-softmax attention for f32 inputs (f32 MFMA, f32 accumulation).
//
// Same operation and work split as the bf16 kernel (segmented softmax attention,
// vllm.cpp issue #1545, "The fix"), kept in f32 end to end: inputs are never
// rounded to a narrower type.  Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x2_f32; the MFMA contracts two head_dim channels per step, and lane
// half hf supplies channel hf*D/2 + step, so each lane reads one contiguous half row
// of Q and K.  In the 32x32 accumulator a lane holds one query and 16 keys; each
// accumulator register is directly the B operand of one PV step (O^T += V^T P^T,
// two keys per step), so P never leaves its lane.  V stays row-major in LDS, where
// the A operand of a PV step is 32 consecutive channels of one key row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_bf16.hpp"  // KernelArgs, lane helpers
#include "plan.hpp"

namespace mgattn {

template <int D>
struct F32Tile {
  static constexpr int kWaves = 4;
  static constexpr int kBlockM = kWaves * 32;  // one 32-query block per wave
  static constexpr int kThreads = kWaves * 64;
  static constexpr int kBlockN = 32;           // keys per LDS tile
  static constexpr int kPitch = D + 4;         // K and V row pitch (floats)
  static constexpr int kTileElems = kBlockN * kPitch;
  static constexpr int kStageElems = 2 * kTileElems;  // K then V
  static constexpr int kStages = 2;
  static constexpr int kLdsBytes = kStages * kStageElems * 4;
  static_assert(D % 32 == 0 && D >= 32 && D <= 128, "head_dim must be a multiple of 32 up to 128");
  static_assert((kBlockN * D / 4) % (kWaves * 64) == 0, "tile must split evenly over the threads");
};

template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void attn_fwd_f32(KernelArgs a) {
  using TL = F32Tile<D>;
  constexpr int BM = TL::kBlockM, BN = TL::kBlockN, P = TL::kPitch;
  constexpr int HD = D / 2;   // channels per lane half, = MFMA steps for S^T
  constexpr int CT = D / 32;  // 32-channel output tiles
  constexpr int NT = TL::kWaves * 64;
  constexpr int CH = BN * D / 4;  // float4 pieces per K (or V) tile
  constexpr int PER_T = CH / NT;
  constexpr float kRescaleLog2 = 8.0f;

  __shared__ __attribute__((aligned(16))) float lds[TL::kStages * TL::kStageElems];

  const Tile tile = decode_tile(a.table, a.H, BM, a.causal, blockIdx.x);
  if (!tile.valid) return;
  const int L = a.table.len[tile.slot];    // queries of the segment
  const int Lk = a.table.klen[tile.slot];  // keys of the segment
  const int off = Lk - L;                  // position of query 0 among the keys
  const int q0 = tile.q0;
  // Token t, head h of a tensor with leading dimension ld starts at t*ld + h*D; query
  // head h reads key/value head h / hq_per_kv.
  const size_t t0 = static_cast<size_t>(a.table.start[tile.slot]);
  const size_t tk0 = static_cast<size_t>(a.table.kstart[tile.slot]);
  const size_t hoff = static_cast<size_t>(tile.head) * D;
  const size_t kvoff = static_cast<size_t>(tile.head / a.hq_per_kv) * D;
  const float* __restrict__ qg = static_cast<const float*>(a.q) + t0 * a.ldq + hoff;
  const float* __restrict__ kg = static_cast<const float*>(a.k) + tk0 * a.ldk + kvoff;
  const float* __restrict__ vg = static_cast<const float*>(a.v) + tk0 * a.ldv + kvoff;
  float* __restrict__ og = static_cast<float*>(a.o) + t0 * a.ldo + hoff;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const float c = a.c;
  const int qr = q0 + wave * 32 + n;

  // Q: lane holds query qr, channels hf*HD + [0, HD)
  float qf[HD];
  if (qr < L) {
    const f32x4* p = reinterpret_cast<const f32x4*>(qg + static_cast<size_t>(qr) * a.ldq + hf * HD);
#pragma unroll
    for (int j = 0; j < HD / 4; ++j) {
      const f32x4 x = p[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[4 * j + e] = x[e] * static_cast<float>(a.qsign);
    }
  } else {
#pragma unroll
    for (int j = 0; j < HD; ++j) qf[j] = 0.0f;
  }

  // keys this q-tile needs (causal: up to its last query; window: from its first
  // query's window start, whole tiles below it skipped); tile 0 starts at key kb0
  const int kend = a.causal ? min(Lk, off + q0 + BM) : Lk;
  const int kbeg = a.window > 0 ? max(0, off + q0 - a.window + 1) : 0;
  const int kb0 = (kbeg / BN) * BN;
  const int ntiles = (kend - kb0 + BN - 1) / BN;

  f32x4 kreg[PER_T], vreg[PER_T];
  auto load_tile = [&](int t) {
    const int kt0 = kb0 + t * BN;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int id = tid + i * NT;
      const int key = id / (D / 4), part = id % (D / 4);
      const int row = kt0 + key;
      const bool in = row < Lk;
      kreg[i] = in ? *reinterpret_cast<const f32x4*>(kg + static_cast<size_t>(row) * a.ldk + part * 4) : f32x4{};
      vreg[i] = in ? *reinterpret_cast<const f32x4*>(vg + static_cast<size_t>(row) * a.ldv + part * 4) : f32x4{};
    }
  };
  auto store_tile = [&](int buf) {
    float* ks = lds + buf * TL::kStageElems;
    float* vs = ks + TL::kTileElems;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int id = tid + i * NT;
      const int key = id / (D / 4), part = id % (D / 4);
      *reinterpret_cast<f32x4*>(ks + key * P + part * 4) = kreg[i];
      *reinterpret_cast<f32x4*>(vs + key * P + part * 4) = vreg[i];
    }
  };

  f32x16 o[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) o[ct] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const float* ks = lds + buf * TL::kStageElems;
    const float* vs = ks + TL::kTileElems;
    const int kt0 = kb0 + t * BN;

    f32x16 s = f32x16{};
#pragma unroll
    for (int j = 0; j < HD / 4; ++j) {
      const f32x4 kf = *reinterpret_cast<const f32x4*>(ks + n * P + hf * HD + 4 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[e], qf[4 * j + e], s, 0, 0, 0);
    }

    const int pos_lo = off + q0 + wave * 32;  // position of the wave's first query
    const int pos = off + qr;
    const bool masked = (kt0 + BN > Lk) || (a.causal && kt0 + BN - 1 > pos_lo) ||
                        (a.window > 0 && kt0 < pos_lo + 31 - a.window + 1);
    auto is_masked = [&](int key) {
      return key >= Lk || (a.causal && key > pos) || (a.window > 0 && key <= pos - a.window);
    };
    if (masked) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (is_masked(kt0 + acc_row(r, hf))) s[r] = -INFINITY;
    }

    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    const float m_tile = fmaxf(half_swap_max(mx), -1.0e30f);  // finite for rows without keys here
    if (t == 0) {
      m_run = m_tile;
    } else if (__builtin_amdgcn_ballot_w64((m_tile - m_run) * c > kRescaleLog2)) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) o[ct] *= alpha;
    }

    const float mc = m_run * c;
    float lsum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -mc));
      if (masked && is_masked(kt0 + acc_row(r, hf))) p = 0.0f;
      s[r] = p;
      lsum += p;
    }
    l_run += lsum;

    // O^T += V^T P^T, two keys (one per lane half) per MFMA step
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float* vrow = vs + acc_row(r, hf) * P + n;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        o[ct] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[ct * 32], s[r], o[ct], 0, 0, 0);
    }

    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float inv = 1.0f / half_swap_sum(l_run);
  if (qr < L) {
    float* dst = og + static_cast<size_t>(qr) * a.ldo + 4 * hf;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 val;
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = o[ct][4 * r4 + e] * inv;
        *reinterpret_cast<f32x4*>(dst + ct * 32 + r4 * 8) = val;
      }
  }
}

// Key-split variant for dense non-causal calls whose (segment, head, 128-query tile)
// units leave most SIMDs idle (a 256-token segment of 16 heads is 32 workgroups of
// four waves): one 32-query block per workgroup, W waves each taking the 32-key tiles
// t = wave, wave + W, ... of the segment.  A wave's tiles are its own, so K and V go
// straight from global memory into the MFMA operand registers (no LDS staging, no
// barriers in the loop), with the same operand layout as above: lane (n, hf) reads K
// row n, channels hf*D/2 + [0, D/2), and for PV the V element (key, 32ct + n).  Each
// wave runs its own online softmax; at the end waves 1..W-1 write (m, l, O) per lane to
// LDS and wave 0 merges the W states (m = max, weights 2^((m_w - m)c)) and stores.
// Waves per 32-query block of the key-split f32 kernel (four at head_dim 128, where
// eight waves would leave too few registers per wave) and its LDS bytes.
template <int D>
constexpr int f32_split_waves() { return D == 128 ? 4 : 8; }
template <int D>
constexpr long f32_split_lds_bytes() { return (f32_split_waves<D>() - 1) * (D / 32 * 4 + 1) * 64 * 16L; }

template <int D, int W>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * W, 64 * W), amdgpu_waves_per_eu(W >= 8 ? 2 : 1, 2)))
void attn_fwd_f32_split(KernelArgs a) {
  constexpr int BM = 32, BN = 32;
  constexpr int HD = D / 2;
  constexpr int CT = D / 32;
  constexpr int kPart = CT * 4 + 1;  // float4 per lane: O, then (m, l)
  constexpr float kRescaleLog2 = 8.0f;
  __shared__ __attribute__((aligned(16))) f32x4 part[(W - 1) * kPart * 64];
  static_assert(W == f32_split_waves<D>() && sizeof(part) == f32_split_lds_bytes<D>(), "LDS bytes the host reports");

  const Tile tile = decode_tile(a.table, a.H, BM, 0, blockIdx.x);
  if (!tile.valid) return;
  const int L = a.table.len[tile.slot];  // queries = keys of the segment
  const int q0 = tile.q0;
  const size_t t0 = static_cast<size_t>(a.table.start[tile.slot]);
  const size_t hoff = static_cast<size_t>(tile.head) * D;
  const float* __restrict__ qg = static_cast<const float*>(a.q) + t0 * a.ldq + hoff;
  const float* __restrict__ kg = static_cast<const float*>(a.k) + t0 * a.ldk + hoff;
  const float* __restrict__ vg = static_cast<const float*>(a.v) + t0 * a.ldv + hoff;
  float* __restrict__ og = static_cast<float*>(a.o) + t0 * a.ldo + hoff;

  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const float c = a.c;
  const int qr = q0 + n;

  float qf[HD];
  if (qr < L) {
    const f32x4* p = reinterpret_cast<const f32x4*>(qg + static_cast<size_t>(qr) * a.ldq + hf * HD);
#pragma unroll
    for (int j = 0; j < HD / 4; ++j) {
      const f32x4 x = p[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[4 * j + e] = x[e] * static_cast<float>(a.qsign);
    }
  } else {
#pragma unroll
    for (int j = 0; j < HD; ++j) qf[j] = 0.0f;
  }

  const int ntiles = (L + BN - 1) / BN;
  f32x16 o[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) o[ct] = f32x16{};
  float m_run = -INFINITY, l_run = 0.0f;

  for (int t = wave; t < ntiles; t += W) {
    const int kt0 = t * BN;
    // K row kt0 + n (rows past the segment end read as zeros), channels hf*HD + [0, HD)
    f32x4 kq[HD / 4];
    const bool krow = kt0 + n < L;
    const f32x4* kp = reinterpret_cast<const f32x4*>(kg + static_cast<size_t>(kt0 + n) * a.ldk + hf * HD);
#pragma unroll
    for (int j = 0; j < HD / 4; ++j) kq[j] = krow ? kp[j] : f32x4{};
    // V elements (key kt0 + acc_row(r, hf), channel 32ct + n)
    float vv[16][CT];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kt0 + acc_row(r, hf);
      const float* vr = vg + static_cast<size_t>(key) * a.ldv + n;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) vv[r][ct] = key < L ? vr[ct * 32] : 0.0f;
    }
    f32x16 s = f32x16{};
#pragma unroll
    for (int j = 0; j < HD / 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_32x32x2f32(kq[j][e], qf[4 * j + e], s, 0, 0, 0);
    const bool masked = kt0 + BN > L;
    if (masked) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kt0 + acc_row(r, hf) >= L) s[r] = -INFINITY;
    }
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    const float m_tile = fmaxf(half_swap_max(mx), -1.0e30f);
    if (t == wave) {
      m_run = m_tile;
    } else if (__builtin_amdgcn_ballot_w64((m_tile - m_run) * c > kRescaleLog2)) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) o[ct] *= alpha;
    }
    const float mc = m_run * c;
    float lsum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -mc));
      if (masked && kt0 + acc_row(r, hf) >= L) p = 0.0f;
      s[r] = p;
      lsum += p;
    }
    l_run += lsum;
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) o[ct] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv[r][ct], s[r], o[ct], 0, 0, 0);
  }

  // merge: a wave without tiles holds m = -inf, l = 0, O = 0 and weighs nothing
  if (wave > 0) {
    f32x4* pw = part + (wave - 1) * kPart * 64 + lane;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        pw[(ct * 4 + r4) * 64] = f32x4{o[ct][4 * r4], o[ct][4 * r4 + 1], o[ct][4 * r4 + 2], o[ct][4 * r4 + 3]};
    pw[CT * 4 * 64] = f32x4{m_run, l_run, 0.0f, 0.0f};
  }
  __syncthreads();
  if (wave > 0) return;
  float m_all = m_run;
#pragma unroll
  for (int w = 1; w < W; ++w) m_all = fmaxf(m_all, part[(w - 1) * kPart * 64 + CT * 4 * 64 + lane][0]);
  const float f0 = __builtin_amdgcn_exp2f((m_run - m_all) * c);
  l_run *= f0;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) o[ct] *= f0;
#pragma unroll
  for (int w = 1; w < W; ++w) {
    const f32x4* pw = part + (w - 1) * kPart * 64 + lane;
    const f32x4 ml = pw[CT * 4 * 64];
    const float fw = __builtin_amdgcn_exp2f((ml[0] - m_all) * c);
    l_run = __builtin_fmaf(ml[1], fw, l_run);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 v = pw[(ct * 4 + r4) * 64];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[ct][4 * r4 + e] = __builtin_fmaf(v[e], fw, o[ct][4 * r4 + e]);
      }
  }
  const float inv = 1.0f / half_swap_sum(l_run);
  if (qr < L) {
    float* dst = og + static_cast<size_t>(qr) * a.ldo + 4 * hf;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 val;
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = o[ct][4 * r4 + e] * inv;
        *reinterpret_cast<f32x4*>(dst + ct * 32 + r4 * 8) = val;
      }
  }
}

// The same key split with one 16-query block per workgroup, for calls whose 32-query
// blocks still leave CUs idle (a 256-token segment of 16 heads is 128 blocks of 32, 256
// of 16): twice the workgroups, half the products per CU.  v_mfma_f32_16x16x4_f32, lane
// l = 16 g + n (lane group g, column n).  S^T = K Q^T per 16-key block: step s contracts
// channel g*D/4 + s (each lane group supplies a contiguous quarter of the row, so a lane
// reads a contiguous quarter row of K and Q), and the accumulator holds keys 4g + r
// (r = 0..3) of the block for query n.  O^T += V^T P^T per 32-key tile in 8 steps:
// step (b, r) contracts key 16b + 4g + r, whose probability lane (g, n) holds in its own
// register (b, r), so P never leaves its lane; the A operand is V[key][16ct + n].  The
// row maximum combines the four lane groups with two lane swaps (16, then 32), the row
// sum once at the end.  Waves take the 32-key tiles t = wave, wave + W, ...; waves
// 1..W-1 hand (m, l, O) to wave 0 through LDS, as in attn_fwd_f32_split.
template <int D>
constexpr int f32_split16_waves() { return 8; }
template <int D>
constexpr long f32_split16_lds_bytes() { return (f32_split16_waves<D>() - 1) * (D / 16 + 1) * 64 * 16L; }

template <int D, int W>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * W, 64 * W), amdgpu_waves_per_eu(2, 2)))
void attn_fwd_f32_split16(KernelArgs a) {
  constexpr int BM = 16, BN = 32;
  constexpr int QD = D / 4;      // channels per lane group = QK steps per 16-key block
  constexpr int CT = D / 16;     // 16-channel output tiles
  constexpr int kPart = CT + 1;  // float4 per lane: O, then (m, l)
  constexpr float kRescaleLog2 = 8.0f;
  static_assert(QD % 4 == 0, "a lane group's quarter row is whole float4 pieces");
  __shared__ __attribute__((aligned(16))) f32x4 part[(W - 1) * kPart * 64];
  static_assert(W == f32_split16_waves<D>() && sizeof(part) == f32_split16_lds_bytes<D>(), "LDS bytes the host reports");

  const Tile tile = decode_tile(a.table, a.H, BM, 0, blockIdx.x);
  if (!tile.valid) return;
  const int L = a.table.len[tile.slot];  // queries = keys of the segment
  const int q0 = tile.q0;
  const size_t t0 = static_cast<size_t>(a.table.start[tile.slot]);
  const size_t hoff = static_cast<size_t>(tile.head) * D;
  const float* __restrict__ qg = static_cast<const float*>(a.q) + t0 * a.ldq + hoff;
  const float* __restrict__ kg = static_cast<const float*>(a.k) + t0 * a.ldk + hoff;
  const float* __restrict__ vg = static_cast<const float*>(a.v) + t0 * a.ldv + hoff;
  float* __restrict__ og = static_cast<float*>(a.o) + t0 * a.ldo + hoff;

  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;  // query column
  const int g = lane >> 4;  // lane group
  const float c = a.c;
  const int qr = q0 + n;

  float qf[QD];
  if (qr < L) {
    const f32x4* p = reinterpret_cast<const f32x4*>(qg + static_cast<size_t>(qr) * a.ldq + g * QD);
#pragma unroll
    for (int j = 0; j < QD / 4; ++j) {
      const f32x4 x = p[j];
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[4 * j + e] = x[e] * static_cast<float>(a.qsign);
    }
  } else {
#pragma unroll
    for (int j = 0; j < QD; ++j) qf[j] = 0.0f;
  }

  const int ntiles = (L + BN - 1) / BN;
  f32x4 o[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) o[ct] = f32x4{};
  float m_run = -INFINITY, l_run = 0.0f;

  for (int t = wave; t < ntiles; t += W) {
    const int kt0 = t * BN;
    // K rows kt0 + 16b + n (rows past the segment end read as zeros), channels g*QD + [0, QD)
    f32x4 kq[2][QD / 4];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const bool krow = kt0 + 16 * b + n < L;
      const f32x4* kp = reinterpret_cast<const f32x4*>(kg + static_cast<size_t>(kt0 + 16 * b + n) * a.ldk + g * QD);
#pragma unroll
      for (int j = 0; j < QD / 4; ++j) kq[b][j] = krow ? kp[j] : f32x4{};
    }
    // V elements (key kt0 + 16b + 4g + r, channel 16ct + n)
    float vv[2][4][CT];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kt0 + 16 * b + 4 * g + r;
        const float* vr = vg + static_cast<size_t>(key) * a.ldv + n;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) vv[b][r][ct] = key < L ? vr[16 * ct] : 0.0f;
      }
    f32x4 s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = f32x4{};
#pragma unroll
      for (int j = 0; j < QD / 4; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[b] = __builtin_amdgcn_mfma_f32_16x16x4f32(kq[b][j][e], qf[4 * j + e], s[b], 0, 0, 0);
    }
    const bool masked = kt0 + BN > L;
    if (masked) {
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kt0 + 16 * b + 4 * g + r >= L) s[b][r] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3]));
    mx = fmaxf(mx, fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    const float m_tile = fmaxf(half_swap_max(row16_swap_max(mx)), -1.0e30f);
    if (t == wave) {
      m_run = m_tile;
    } else if (__builtin_amdgcn_ballot_w64((m_tile - m_run) * c > kRescaleLog2)) {
      const float m_new = fmaxf(m_run, m_tile);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) o[ct] *= alpha;
    }
    const float mc = m_run * c;
    float lsum = 0.0f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], c, -mc));
        if (masked && kt0 + 16 * b + 4 * g + r >= L) p = 0.0f;
        s[b][r] = p;
        lsum += p;
      }
    l_run += lsum;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) o[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv[b][r][ct], s[b][r], o[ct], 0, 0, 0);
  }

  // merge: a wave without tiles holds m = -inf, l = 0, O = 0 and weighs nothing
  if (wave > 0) {
    f32x4* pw = part + (wave - 1) * kPart * 64 + lane;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) pw[ct * 64] = o[ct];
    pw[CT * 64] = f32x4{m_run, l_run, 0.0f, 0.0f};
  }
  __syncthreads();
  if (wave > 0) return;
  float m_all = m_run;
#pragma unroll
  for (int w = 1; w < W; ++w) m_all = fmaxf(m_all, part[(w - 1) * kPart * 64 + CT * 64 + lane][0]);
  const float f0 = __builtin_amdgcn_exp2f((m_run - m_all) * c);
  l_run *= f0;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) o[ct] *= f0;
#pragma unroll
  for (int w = 1; w < W; ++w) {
    const f32x4* pw = part + (w - 1) * kPart * 64 + lane;
    const f32x4 ml = pw[CT * 64];
    const float fw = __builtin_amdgcn_exp2f((ml[0] - m_all) * c);
    l_run = __builtin_fmaf(ml[1], fw, l_run);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const f32x4 v = pw[ct * 64];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[ct][e] = __builtin_fmaf(v[e], fw, o[ct][e]);
    }
  }
  // the row sum over the four lane groups' keys
  const float inv = 1.0f / half_swap_sum(row16_swap_sum(l_run));
  if (qr < L) {
    float* dst = og + static_cast<size_t>(qr) * a.ldo + 4 * g;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) *reinterpret_cast<f32x4*>(dst + 16 * ct) = o[ct] * inv;
  }
}


}  // namespace mgattn
