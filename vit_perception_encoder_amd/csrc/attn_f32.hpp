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

}  // namespace mgattn
