// Dense segmented attention, bf16 inputs, f32 accumulation, gfx950: the
// software-pipelined main loop.
//
// Same operation as attn_fwd_bf16<D, false> (vllm.cpp issue #1545, sections "Why this
// one is bad" and "The fix": every cu_seqlens segment attended on its own, online
// softmax as in the flash rung of PR #1579, "Numerics, both halves"), same tile
// (8 waves, 256 queries, 32 per wave; S^T = K Q^T and O^T = V^T P^T on
// v_mfma_f32_32x32x16_bf16; K/V tiles of 128 keys in three LDS stages filled by LDS
// DMA), but a different way of keeping the matrix core fed.
//
// On gfx950 one wave issues a VALU instruction at best every ~7 cycles, while the
// SIMD accepts one from another wave in between; transcendentals take about 2.7
// times the issue cost of an FMA.  So the softmax of a 64-key step (~120 VALU
// instructions per wave, 32 of them v_exp_f32) cannot hide behind the other wave's
// 24 MFMAs when one wave runs it alone.  Here every wave runs, per iteration j,
//     PV(j-1)  --  O^T += V^T P(j-1)^T   (12 MFMAs at head_dim 96)
//     QK(j+1)  --  S(j+1)^T = K Q^T      (12 MFMAs)
//     SM(j)    --  online softmax of S(j) into P(j)
// as one instruction stream: MFMA slot k is followed by the LDS operand reads of a
// later slot and by a slice of the softmax, with a scheduling fence after each slot
// so the compiler keeps that interleave.  Both waves of a SIMD do the same, so the
// matrix core always has an MFMA waiting while the two VALU streams share the rest.
// S and P have one register buffer each, shared by two steps: the QK MFMAs write
// S(j+1) into a 32-key block only after the softmax has read S(j) from it, and the
// softmax writes P(j) into a block only after the PV MFMAs have read P(j-1) from it
// (both products run block-major, the softmax slices are placed to match).
//
// LDS: K of step s is read in iteration s-1, V of step s in iteration s+1, so tile t
// (steps 2t, 2t+1) is live in iterations 2t-1 .. 2t+2.  One barrier per tile, at the
// start of odd iteration 2t+1: each wave first waits for its own DMA of tile t+1
// (issued two iterations earlier; tile 1 just after the first barrier), and after the
// barrier tile t-1's stage (last read in iteration 2t) receives tile t+2.  The Q tile
// arrives by DMA in the third stage before tile 2 does.
//
// Rescaling is lazy (the running maximum moves only when a row's maximum grows by more
// than 2^8 in probability terms, decided per wave) and branch-free inside the loop:
// the row sum takes the factor at once; O, which the same iteration's PV MFMAs still
// accumulate into, takes it at the start of the next iteration, before PV(j).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "attn_bf16.hpp"
#include "plan.hpp"
#include "schedule.hpp"

namespace mgattn {

template <int... K, typename F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, K...>, F&& f) {
  (f(std::integral_constant<int, K>{}), ...);
}
// f(integral_constant<int, k>) for k = 0 .. N-1, in order, k a constant expression.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, static_cast<F&&>(f));
}

// Row maxima in the main loop: IEEE maximum (NaN in, NaN out), which gfx950 has as
// v_maximum3_f32.  fmaxf (NaN ignored) makes the compiler quiet every MFMA result
// with a v_max_f32 x, x before it enters a maximum chain: 8 VALU instructions per
// 64-key step that this form does not need.  Finite scores and -inf (masked keys) give
// the same maxima either way; a NaN score makes the row NaN either way.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float half_swap_maximum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Scheduling fence: the compiler moves no instruction across it.
#define MGATTN_FENCE() __builtin_amdgcn_sched_barrier(0)

// Slot plan of one iteration for steps of NB 32-key blocks: 64-key steps (NB = 2, every
// shape but the four-group key split) or 32-key steps (NB = 1).
template <int D, int NB = 2>
struct PipeTile {
  using T = Bf16Tile<D>;
  static constexpr int kNB = NB;                     // 32-key blocks per step
  static constexpr int kStepKeys = 32 * kNB;
  static constexpr int kKS = D / 16;                 // QK k-steps
  static constexpr int kCT = D / 32;                 // 32-channel output tiles
  static constexpr int kNPV = kNB * 2 * kCT;         // PV MFMAs per iteration
  static constexpr int kNQK = kKS * kNB;             // QK MFMAs per iteration
  static constexpr int kNSlot = kNPV + kNQK;
  static constexpr int kDV = 3;                      // V^T read distance (slots)
  static constexpr int kDK = 4;                      // K read distance (slots)
  // Slots 0 .. kNPV-1: PV MFMA i = (32-key block b, 16-key half h2, channel tile ct),
  // block-major, so block 0 of P(j-1) is dead after slot kNPV/2 - 1.
  static constexpr int pv_b(int i) { return i / (2 * kCT); }
  static constexpr int pv_h(int i) { return (i / kCT) % 2; }
  static constexpr int pv_c(int i) { return i % kCT; }
  // Slots kNPV ..: QK MFMA i = (block b, k-step st), block-major, so S(j+1) block 0
  // overwrites S(j) block 0 only after the softmax has read it (slot kNPV on), and
  // block 1 from slot kNPV + kKS on.
  static constexpr int qk_b(int i) { return i / kKS; }
  static constexpr int qk_s(int i) { return i % kKS; }
  // Softmax slices: slots 0..3 the row maxima (64-key steps: block 0 in slots 0-1, block
  // 1 in slots 2-3), slot 4 the running maximum; score pair
  // u (of the lane's 16 NB: block u/8) is exponentiated in slot exp_slot(u) and
  // converted to bf16 and summed one slot later; the row sum takes the step in slot
  // kLSlot.  NB = 2: S and P have one buffer each; block 0's pairs end before slot kNPV
  // and block 1's before kNPV + kKS, and the conversions of block 0 start at slot
  // kNPV/2, after PV(j-1) has read P block 0.  NB = 1: S and P have two buffers,
  // alternating by iteration parity, so the slices only follow the running maximum.
  static constexpr int kBufs = kNB == 2 ? 1 : 2;
  static constexpr int exp_slot(int u) {
    constexpr int tbl2[16] = {5, 6, 7, 8, 9, 10, 11, 11, 12, 13, 13, 14, 15, 16, 16, 17};
    constexpr int tbl1[8] = {5, 6, 7, 7, 8, 9, 9, 10};
    return kNB == 2 ? tbl2[u] : tbl1[u];
  }
  static constexpr int kLSlot = kNB == 2 ? 19 : 11;
  static_assert(D == 96, "the slot plan is laid out for head_dim 96 (6 k-steps, 3 channel tiles)");
  static_assert(kKS == 6 && kNPV == 6 * kNB && kNSlot == 12 * kNB, "slot plan");
  static_assert(kNB == 1 || kNB == 2, "32- or 64-key steps");
  static_assert(T::kStages == 3, "the pipelined loop needs three LDS stages");
  static_assert(T::kBlockN == 2 * T::kStepKeys, "two 64-key steps per LDS tile");
  static_assert(kNPV >= kDK, "K reads start inside the PV slots");
  static_assert(exp_slot(0) - 1 >= 4 && exp_slot(8 * kNB - 1) + 1 <= kLSlot && kLSlot < kNSlot,
                "exponent arguments after the running maximum (slot 4), the row sum after the last conversion");
};

// W waves per workgroup, 32 queries each: 8 for launches that fill the chip, 4 (query
// tiles of 128) when a launch has too few (segment, head, tile) units.  kRope: Q is
// rotated by the 2D RoPE as it is read (mgattn_dense_rope2d); the angles of a lane's 24
// rotation pairs are computed while the prologue's DMA is in flight, and the angles and
// the rotation round exactly as the RoPE pass does (window_rope.hpp), so the result is
// that of rotating q in memory first.
// G > 1: the keys are split between G wave groups of W/G waves (query tiles of 32W/G),
// group g taking keys g*128/G .. (g+1)*128/G - 1 of every 128-key tile (64-key steps
// for two groups, 32-key steps for four), each wave running its own online softmax
// over its part; at the end groups 1.. hand their (m, l, O) to group 0 through LDS,
// which merges them and stores the tile.  For launches whose (segment, head, tile)
// units leave CUs idle: smaller query tiles, fewer steps per wave.  Non-causal only.
template <int D, int W, bool kRope = false, int G = 1>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * W, 64 * W), amdgpu_waves_per_eu(W == 8 ? 2 : 1, 2)))
void attn_fwd_bf16_pipe(KernelArgs a) {
  static_assert(G == 1 || G == 2 || G == 4, "one, two or four key groups");
  constexpr bool kSplit = G > 1;
  using TL = Bf16Tile<D>;
  using PT = PipeTile<D, G == 4 ? 1 : 2>;
  using SG = sched::SplitGeometry<D>;
  constexpr int QB = W / G;          // 32-query blocks
  static_assert(QB * G == W, "whole query blocks per group");
  constexpr int BM = 32 * QB, BN = TL::kBlockN;
  constexpr int SK = PT::kStepKeys;
  static_assert(!kSplit || G * SK == BN, "the groups' steps tile a 128-key tile");
  constexpr int NB = PT::kNB, KS = PT::kKS, CT = PT::kCT;
  constexpr int NPV = PT::kNPV, NQK = PT::kNQK, NSLOT = PT::kNSlot;
  constexpr int DV = PT::kDV, DK = PT::kDK;
  constexpr int NSTEP = BN / SK;
  constexpr int KP = TL::kKPitch, VP = TL::kVPitch, KSL = TL::kKSlots;
  constexpr int KDMA = TL::kKDma, VDMA = TL::kVDma;
  constexpr int KDMA_W = (KDMA + W - 1) / W;
  constexpr int VDMA_W = (VDMA + W - 1) / W;
  constexpr float kRescaleLog2 = 8.0f;

  constexpr int KE = TL::kKElems;
  // Q rows are padded like K rows, so the Q fragment reads are free of bank conflicts
  constexpr int kLdsElems = kSplit ? SG::lds_elems(BM) : sched::pipe_lds_elems<D>(BM);
  static_assert(kLdsElems * 2 <= 160 * 1024, "LDS of one CU");
  __shared__ __attribute__((aligned(16))) __bf16 lds[kLdsElems];
  // K and V of LDS tile t; K and V^T rows of step j (keys 64j.., or for key group g
  // keys 128j + 64g..)
  auto k_tile = [&](int t) { return kSplit ? lds + SG::k_slot_elem(t) : lds + (t % TL::kStages) * TL::kStageElems; };
  auto v_tile = [&](int t) {
    return kSplit ? lds + SG::v_slot_elem(t) : lds + (t % TL::kStages) * TL::kStageElems + KE;
  };

  const Tile tile = decode_tile(a.table, a.H, BM, a.causal, blockIdx.x);
  if (!tile.valid) return;
  const int L = a.table.len[tile.slot];  // tokens of the segment (queries = keys)
  const int q0 = tile.q0;
  const size_t t0 = static_cast<size_t>(a.table.start[tile.slot]);
  const size_t hoff = static_cast<size_t>(tile.head) * D;
  const __bf16* __restrict__ qg = static_cast<const __bf16*>(a.q) + t0 * a.ldq + hoff;
  const __bf16* __restrict__ kg = static_cast<const __bf16*>(a.k) + t0 * a.ldk + hoff;
  const __bf16* __restrict__ vg = static_cast<const __bf16*>(a.v) + t0 * a.ldv + hoff;
  __bf16* __restrict__ og = static_cast<__bf16*>(a.o) + t0 * a.ldo + hoff;
  const int ldk = a.ldk, ldv = a.ldv;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;
  const int hf = lane >> 5;
  const float c = a.c;
  const int grp = kSplit ? wave / QB : 0;  // key group (wave-uniform)
  const int qb = kSplit ? wave % QB : wave;  // 32-query block
  const int qr = q0 + qb * 32 + n;  // this lane's query (relative to the segment)
  const int qmin = q0 + qb * 32;    // the wave's first query

  // keys this q-tile needs: all of the segment, or (causal) up to its last query
  const int kend = a.causal ? min(L, q0 + BM) : L;
  const int ntiles = (kend + BN - 1) / BN;
  const int nsteps = kSplit ? ntiles : (kend + SK - 1) / SK;  // steps of this wave

  // ---- LDS DMA plan (as in attn_fwd_bf16): DMA instruction i of a tile fills 64
  // consecutive 16-byte slots; wave w issues instructions w, w+8, ...  K slot s is row
  // s/KSL, piece s%KSL (the padding piece D/8 repeats piece D/8-1); V slot s is row
  // s/(D/8), piece s%(D/8).  Rows past the segment end are clamped to its last row.
  auto k_row = [&](int u) { return ((wave + W * u) * 64 + lane) / KSL; };
  auto k_off = [&](int u) { return min(((wave + W * u) * 64 + lane) % KSL, D / 8 - 1) * 8; };
  auto v_row = [&](int u) { return ((wave + W * u) * 64 + lane) / (D / 8); };
  auto v_off = [&](int u) { return (((wave + W * u) * 64 + lane) % (D / 8)) * 8; };
  uint32_t k_boff[KDMA_W], v_boff[VDMA_W];
#pragma unroll
  for (int u = 0; u < KDMA_W; ++u)
    k_boff[u] = (static_cast<uint32_t>(k_row(u)) * static_cast<uint32_t>(ldk) + k_off(u)) * 2u;
#pragma unroll
  for (int u = 0; u < VDMA_W; ++u)
    v_boff[u] = (static_cast<uint32_t>(v_row(u)) * static_cast<uint32_t>(ldv) + v_off(u)) * 2u;
  auto issue_tile = [&](int t, int part) {  // part: 1 = K, 2 = V, 3 = both
    const int kt0 = t * BN;
    const int last = L - 1 - kt0;
    const __bf16* kb = kg + static_cast<size_t>(kt0) * ldk;
    const __bf16* vb = vg + static_cast<size_t>(kt0) * ldv;
    __bf16* kl = k_tile(t);
    __bf16* vl = v_tile(t);
    if (last >= BN - 1) {
#pragma unroll
      for (int u = 0; u < KDMA_W; ++u) {
        const int i = wave + W * u;
        if ((part & 1) && (KDMA % W == 0 || i < KDMA))
          dma16s(kb, k_boff[u], __builtin_amdgcn_readfirstlane(lds_addr(kl + i * 512)));
      }
#pragma unroll
      for (int u = 0; u < VDMA_W; ++u) {
        const int i = wave + W * u;
        if ((part & 2) && (VDMA % W == 0 || i < VDMA))
          dma16s(vb, v_boff[u], __builtin_amdgcn_readfirstlane(lds_addr(vl + i * 512)));
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < KDMA_W; ++u) {
      const int i = wave + W * u;
      if ((part & 1) && (KDMA % W == 0 || i < KDMA))
        dma16(kb + static_cast<size_t>(min(k_row(u), last)) * ldk + k_off(u),
              __builtin_amdgcn_readfirstlane(lds_addr(kl + i * 512)));
    }
#pragma unroll
    for (int u = 0; u < VDMA_W; ++u) {
      const int i = wave + W * u;
      if ((part & 2) && (VDMA % W == 0 || i < VDMA))
        dma16(vb + static_cast<size_t>(min(v_row(u), last)) * ldv + v_off(u),
              __builtin_amdgcn_readfirstlane(lds_addr(vl + i * 512)));
    }
  };
  const int my_kdma = KDMA / W + (wave < KDMA % W ? 1 : 0);
  const int my_vdma = VDMA / W + (wave < VDMA % W ? 1 : 0);

  // ---- prologue: Q tile (from the third stage on) and tile 0; Q rows and K of tile 0
  // are waited for before the first barrier, V of tile 0 at the barrier of iteration 1.
  // Tile 1 goes out right after the first barrier (also waited for at iteration 1):
  // issued with the rest, its 50 KB per workgroup share the start-up burst of every
  // workgroup at once and hold back the Q rows and K the first product waits for.
  // Key-split: Q after the K and V rings; K of tiles 0 and 1, then V of tile 0; K of
  // tile 1 is waited for at the barrier of iteration 0.
  // Q slot s (16 bytes) is row s/KSL, piece min(s%KSL, D/8-1), as for K
  constexpr int QDMA = TL::q_pad_dma(BM);
  constexpr int QDMA_W = (QDMA + W - 1) / W;
  static_assert(W == 4 || W == 8, "4 or 8 waves");
  __bf16* ql = kSplit ? lds + SG::kQElem : lds + sched::pipe_q_elem<D>();
  static_assert((kSplit ? SG::kQElem : sched::pipe_q_elem<D>()) + QDMA * 512 <= kLdsElems, "Q DMA inside LDS");
#pragma unroll
  for (int u = 0; u < QDMA_W; ++u) {
    const int i = wave + W * u;
    const int slot = i * 64 + lane;
    const int row = min(q0 + slot / KSL, L - 1);
    if (QDMA % W == 0 || i < QDMA)
      dma16(qg + static_cast<size_t>(row) * a.ldq + min(slot % KSL, D / 8 - 1) * 8,
            __builtin_amdgcn_readfirstlane(lds_addr(ql + i * 512)));
  }
  if constexpr (kSplit) {
    issue_tile(0, 1);
    if (ntiles > 1) issue_tile(1, 1);
    issue_tile(0, 2);
  } else {
    issue_tile(0, 1);
    issue_tile(0, 2);
    static_assert(sched::kPipePrologueTiles == 1, "tile 0 before the first barrier, tile 1 right after it");
  }
  // RoPE angles of this lane's query, computed while the prologue's DMA is in flight:
  // fragment st holds channels 16st + 8hf + [0, 8), i.e. 4 pairs of one half of the
  // head (the width half below D/2, rotated by the column + 1; the height half by the
  // row + 1), pair index (channel mod D/2) / 2; rope_angle_bf16 as in the RoPE pass.
  float rc[KS][4], rs[KS][4];
  if constexpr (kRope) {
    int prow = 0, pcol = 0;
    token_patch(a.rope.tb, a.rope.win, static_cast<int>(t0) + min(qr, L - 1), &prow, &pcol);
#pragma unroll
    for (int st = 0; st < KS; ++st)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int ch = 16 * st + 8 * hf + 2 * k;
        rope_angle_bf16(static_cast<float>(ch >= D / 2 ? prow + 1 : pcol + 1), a.rope.inv_freq[(ch % (D / 2)) / 2],
                        &rc[st][k], &rs[st][k]);
        // keep the angles here, under the DMA wait: left alone, the compiler sinks them
        // past the barrier next to the rotation, onto the path to the first MFMA
        asm volatile("" ::"v"(rc[st][k]), "v"(rs[st][k]));
      }
  }
  if constexpr (kSplit) dma_wait_leave(my_vdma + (ntiles > 1 ? my_kdma : 0));
  else dma_wait_leave(my_vdma);
  __syncthreads();
  if constexpr (!kSplit) {
    if (ntiles > 1) issue_tile(1, 3);
  }

  bf16x8 qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(ql + (qb * 32 + n) * KP + 16 * s + 8 * hf);
  if constexpr (kRope) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      u32x4 w = __builtin_bit_cast(u32x4, qf[st]);
#pragma unroll
      for (int k = 0; k < 4; ++k) w[k] = rope_pair_bf16(w[k], rc[st][k], rs[st][k]);
      qf[st] = __builtin_bit_cast(bf16x8, w);
    }
  }
  if (qr >= L) {
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = bf16x8{};
  }
  if (a.qsign != 1) {
    const __bf16 sg = static_cast<__bf16>(static_cast<float>(a.qsign));
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = qf[s] * sg;
  }

  // ---- running state
  f32x16 o[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) o[ct] = f32x16{};
  float m_run = 0.0f, l_run = 0.0f, alpha = 1.0f;
  int resc = 0;  // O waits for the factor alpha (wave-uniform)
  const bf16x2 ones = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
  // NB = 2: one buffer, S(j) until the softmax has read it, then S(j+1), and P(j-1)
  // until PV(j-1) has read it, then P(j).  NB = 1: iteration j reads S(j) and writes
  // P(j) in buffer j % 2, QK(j+1) writes S(j+1) and PV(j-1) reads P(j-1) in the other.
  constexpr int NBUF = PT::kBufs;
  f32x16 s[NBUF][NB];
  bf16x8 p[NBUF][NB][2];

  // K and V^T rows of this wave's step j.  Key-split: the ring offset goes through
  // readfirstlane, an opaque wave-uniform value, so the compiler forms each operand
  // read as one base plus an immediate instead of re-deriving the ring index per read.
  auto k_step = [&](int j) {
    if constexpr (kSplit)
      return lds + __builtin_amdgcn_readfirstlane(SG::k_slot_elem(j) + grp * SK * KP);
    else
      return k_tile(j / NSTEP) + (j % NSTEP) * SK * KP;
  };
  auto v_step = [&](int j) {
    if constexpr (kSplit)
      return lds + __builtin_amdgcn_readfirstlane(SG::v_slot_elem(j) + grp * SK * VP);
    else
      return v_tile(j / NSTEP) + (j % NSTEP) * SK * VP;
  };
  static_assert(NB * 32 == SK, "a step is NB blocks of 32 keys");
  // V^T transpose-read lane addressing (see attn_bf16.hpp)
  const int tr_row = ((lane & 15) >> 2) + 4 * hf;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // V^T operand of PV MFMA i for step js
  auto read_v = [&](const __bf16* vt, int i) {
    const __bf16* vrow = vt + ((PT::pv_b(i)) * 32 + PT::pv_h(i) * 16 + tr_row) * VP + tr_col + PT::pv_c(i) * 32;
    const bf16x4 lo = ds_read_tr(vrow);
    const bf16x4 hi = ds_read_tr(vrow + 8 * VP);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto read_k = [&](const __bf16* ks, int i) {
    return *reinterpret_cast<const bf16x8*>(ks + (PT::qk_b(i) * 32 + n) * KP + 16 * PT::qk_s(i) + 8 * hf);
  };

  // Scores of step j (in buffer sb) past the segment end or (causal) after the query: -inf.
  auto mask = [&](int j, f32x16 (&sb)[NB]) {
    const int key0 = kSplit ? j * BN + grp * SK : j * SK;
    if ((key0 + SK > L) || (a.causal && key0 + SK - 1 > qmin)) {
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + b * 32 + acc_row(r, hf);
          if (key >= L || (a.causal && key > qr)) sb[b][r] = -INFINITY;
        }
    }
  };

  // One iteration.  HAS_PV: PV(j-1); HAS_QK: QK(j+1); HAS_SM: the softmax of step j;
  // FIRST: the first softmax step (sets the running maximum); PAR: j % 2 (NB = 1).
  auto iteration = [&](int j, auto has_pv, auto has_qk, auto has_sm, auto first, auto par) {
    constexpr bool PV = decltype(has_pv)::value, QK = decltype(has_qk)::value;
    constexpr bool SM = decltype(has_sm)::value, FIRST = decltype(first)::value;
    constexpr int BC = NBUF == 2 ? decltype(par)::value : 0;  // S(j) and P(j)
    constexpr int BN1 = NBUF == 2 ? 1 - BC : 0;               // S(j+1) and P(j-1)
    if constexpr (PV) {
      if (resc) {  // the factor decided in the previous iteration, before PV(j-1) adds in
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) o[ct] *= alpha;
      }
    }
    if constexpr (SM) mask(j, s[BC]);
    const int jv = sched::pipe_v_step(j), jk = sched::pipe_k_step(j);
    const __bf16* vt = PV ? v_step(jv) : lds;
    const __bf16* ks = QK ? k_step(jk) : lds;
    bf16x8 vf[NPV];
    bf16x8 kf[NQK];
    if constexpr (PV) {
      static_for<DV>([&](auto ic) { vf[decltype(ic)::value] = read_v(vt, decltype(ic)::value); });
    }
    float mx[2 * NB];              // partial row maxima: block b, half h at 2b+h
    float mc = 0.0f;
    float lsum[2] = {0.0f, 0.0f};  // two row-sum chains (even and odd score pairs)
    float px[8 * NB][2];           // a score pair between its exponent argument and its conversion
    MGATTN_FENCE();
    static_for<NSLOT>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      // -- the MFMA of slot k
      if constexpr (k < NPV) {
        if constexpr (PV)
          o[PT::pv_c(k)] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[k], p[BN1][PT::pv_b(k)][PT::pv_h(k)],
                                                                   o[PT::pv_c(k)], 0, 0, 0);
      } else {
        constexpr int i = k - NPV;
        if constexpr (QK) {
          if constexpr (PT::qk_s(i) == 0)
            s[BN1][PT::qk_b(i)] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[0], f32x16{}, 0, 0, 0);
          else
            s[BN1][PT::qk_b(i)] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qf[PT::qk_s(i)], s[BN1][PT::qk_b(i)], 0, 0, 0);
        }
      }
      // -- operand reads of later slots
      if constexpr (PV && k + DV < NPV) vf[k + DV] = read_v(vt, k + DV);
      if constexpr (QK && k + DK >= NPV && k + DK < NSLOT) kf[k + DK - NPV] = read_k(ks, k + DK - NPV);
      // -- the softmax slice of slot k
      if constexpr (SM) {
        // slots 0..3: row maximum as 2 NB independent maximum chains over 8 scores each
        const f32x16(&sc)[NB] = s[BC];
        if constexpr (k < 4) {
          static_for<2 * NB>([&](auto cc) {
            constexpr int ch = decltype(cc)::value, b = ch / 2, r0 = 8 * (ch % 2);
            if constexpr (NB == 2) {
              // block b in slots 2b and 2b+1: block 1, completed by the last QK MFMA of the
              // previous iteration, is first read two slots after block 0
              if constexpr (k == 2 * b)
                mx[ch] = vmax(vmax(vmax(vmax(sc[b][r0], sc[b][r0 + 1]), sc[b][r0 + 2]), sc[b][r0 + 3]), sc[b][r0 + 4]);
              if constexpr (k == 2 * b + 1)
                mx[ch] = vmax(vmax(vmax(mx[ch], sc[b][r0 + 5]), sc[b][r0 + 6]), sc[b][r0 + 7]);
            } else {
              if constexpr (k == 0) mx[ch] = vmax(vmax(sc[b][r0], sc[b][r0 + 1]), sc[b][r0 + 2]);
              if constexpr (k == 1) mx[ch] = vmax(vmax(mx[ch], sc[b][r0 + 3]), sc[b][r0 + 4]);
              if constexpr (k == 2) mx[ch] = vmax(vmax(mx[ch], sc[b][r0 + 5]), sc[b][r0 + 6]);
              if constexpr (k == 3) mx[ch] = vmax(mx[ch], sc[b][r0 + 7]);
            }
          });
        }
        if constexpr (k == 4) {
          // a step with no visible key for some rows (causal, or a key group past the
          // segment end) has maximum -inf; the floor keeps the reference finite (those
          // rows get p = 0 and take alpha = 0 at the first step with keys)
          float mxa = vmax(mx[0], mx[1]);
          if constexpr (NB == 2) mxa = vmax(mxa, vmax(mx[2], mx[3]));
          const float m_blk = vmax(half_swap_maximum(mxa), -1.0e30f);
          if constexpr (FIRST) {
            m_run = m_blk;
          } else {
            const bool grow = __builtin_amdgcn_ballot_w64((m_blk - m_run) * c > kRescaleLog2) != 0;
            const float m_new = grow ? vmax(m_run, m_blk) : m_run;
            alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
            resc = grow;
            m_run = m_new;
          }
          mc = m_run * c;
        }
        // probabilities, pair by pair, in three stages one slot apart (no stage waits
        // on the one before it): exponent argument s*c - m*c, p = exp2, then the
        // conversion to bf16 (RNE) and the row sum
        static_for<8 * NB>([&](auto uc) {
          constexpr int u = decltype(uc)::value;
          constexpr int b = u / 8, h2 = (u / 4) % 2, e = 2 * (u % 4);
          constexpr int E = PT::exp_slot(u);
          if constexpr (E + 1 == k) {
            const bf16x2 pr = {static_cast<__bf16>(px[u][0]), static_cast<__bf16>(px[u][1])};
            p[BC][b][h2][e] = pr[0];
            p[BC][b][h2][e + 1] = pr[1];
            lsum[u & 1] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, lsum[u & 1], false);
          }
          if constexpr (E == k) {
            px[u][0] = __builtin_amdgcn_exp2f(px[u][0]);
            px[u][1] = __builtin_amdgcn_exp2f(px[u][1]);
          }
          if constexpr (E - 1 == k) {
            px[u][0] = __builtin_fmaf(sc[b][8 * h2 + e], c, -mc);
            px[u][1] = __builtin_fmaf(sc[b][8 * h2 + e + 1], c, -mc);
          }
        });
        if constexpr (k == PT::kLSlot) {
          if constexpr (FIRST) l_run = lsum[0] + lsum[1];
          else l_run = __builtin_fmaf(l_run, alpha, lsum[0] + lsum[1]);
        }
      }
      MGATTN_FENCE();
    });
    if constexpr (!SM) resc = 0;
  };

  auto tile_sync = [&](int j) {  // start of iteration j
    if constexpr (kSplit) {
      // all of this wave's DMA but V of tile j (the last it issued, read in iteration
      // j+1), so K of tile j+1 and V of tile j-1 are here; after the barrier the slots
      // of K of tile j and V of tile j-2 (last read in iteration j-1) are free
      dma_wait_leave(j < ntiles ? my_vdma : 0);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (sched::split_issue_k(j) < ntiles) issue_tile(sched::split_issue_k(j), 1);
      if (sched::split_issue_v(j) < ntiles) issue_tile(sched::split_issue_v(j), 2);
    } else {  // odd iterations j = 2t+1
      if (!sched::pipe_syncs(j)) return;
      dma_wait();  // this wave's DMA of tile t+1
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const int tn = sched::pipe_issue_tile(j);
      if (tn < ntiles) issue_tile(tn, 3);
    }
  };

  using T_ = std::true_type;
  using F_ = std::false_type;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  // ---- S(0), then iteration 0 (no PV)
  {
    const __bf16* ks = k_step(0);
    static_for<NQK>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const bf16x8 kf = read_k(ks, i);
      if constexpr (PT::qk_s(i) == 0)
        s[0][PT::qk_b(i)] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[0], f32x16{}, 0, 0, 0);
      else
        s[0][PT::qk_b(i)] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[PT::qk_s(i)], s[0][PT::qk_b(i)], 0, 0, 0);
    });
  }
  tile_sync(0);
  if (nsteps > 1) iteration(0, F_{}, T_{}, T_{}, T_{}, P0{});
  else iteration(0, F_{}, F_{}, T_{}, T_{}, P0{});
  // ---- steady state: every part present (two iterations per trip with two buffers)
  int j = 1;
  if constexpr (NBUF == 2) {
    for (; j + 2 < nsteps; j += 2) {
      tile_sync(j);
      iteration(j, T_{}, T_{}, T_{}, F_{}, P1{});
      tile_sync(j + 1);
      iteration(j + 1, T_{}, T_{}, T_{}, F_{}, P0{});
    }
    if (j + 1 < nsteps) {
      tile_sync(j);
      iteration(j, T_{}, T_{}, T_{}, F_{}, P1{});
      ++j;
    }
  } else {
    for (; j + 1 < nsteps; ++j) {
      tile_sync(j);
      iteration(j, T_{}, T_{}, T_{}, F_{}, P0{});
    }
  }
  // ---- the last softmax step (no QK), then PV of the last step
  if (nsteps > 1) {
    tile_sync(nsteps - 1);
    if (NBUF == 2 && ((nsteps - 1) & 1)) iteration(nsteps - 1, T_{}, F_{}, T_{}, F_{}, P1{});
    else iteration(nsteps - 1, T_{}, F_{}, T_{}, F_{}, P0{});
  }
  tile_sync(nsteps);
  if (NBUF == 2 && (nsteps & 1)) iteration(nsteps, T_{}, F_{}, F_{}, F_{}, P1{});
  else iteration(nsteps, T_{}, F_{}, F_{}, F_{}, P0{});
  if (resc) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) o[ct] *= alpha;
  }

  // ---- epilogue (as attn_fwd_bf16): O / l -> bf16 (RNE), staged through the wave's
  // own LDS rows once every wave is done with the K/V stages, stored as whole rows
  // (non-temporal), rows inside the segment only.
  constexpr int OP = D + 8;
  static_assert(QB * 32 * OP <= kLdsElems, "O staging must fit in the K/V stages");
  __syncthreads();
  if constexpr (kSplit) {
    // groups 1..G-1 hand each lane's (O, m, l) -- 13 float4, lane-major, after group 0's
    // staging rows -- to the group-0 wave of the same queries, which merges:
    // m = max_g m_g, O = sum_g O_g 2^((m_g-m)c), l likewise
    constexpr int kPart = CT * 4 + 1;
    static_assert(QB * 32 * OP * 2 % 16 == 0 && QB * 32 * OP * 2 + (G - 1) * QB * kPart * 64 * 16 <= kLdsElems * 2,
                  "merge buffers must fit behind the staging rows");
    f32x4* part = reinterpret_cast<f32x4*>(lds + QB * 32 * OP) + lane;
    auto part_of = [&](int g) { return part + ((g - 1) * QB + qb) * kPart * 64; };
    if (grp > 0) {
      f32x4* pw = part_of(grp);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          pw[(ct * 4 + r4) * 64] = f32x4{o[ct][4 * r4], o[ct][4 * r4 + 1], o[ct][4 * r4 + 2], o[ct][4 * r4 + 3]};
      pw[CT * 4 * 64] = f32x4{m_run, l_run, 0.0f, 0.0f};
    }
    __syncthreads();
    if (grp > 0) return;
    float m_new = m_run;
#pragma unroll
    for (int g = 1; g < G; ++g) m_new = fmaxf(m_new, part_of(g)[CT * 4 * 64][0]);
    const float f0 = __builtin_amdgcn_exp2f((m_run - m_new) * c);
    l_run *= f0;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) o[ct] *= f0;
#pragma unroll
    for (int g = 1; g < G; ++g) {
      const f32x4* pg = part_of(g);
      const f32x4 ml = pg[CT * 4 * 64];
      const float fg = __builtin_amdgcn_exp2f((ml[0] - m_new) * c);
      l_run = __builtin_fmaf(ml[1], fg, l_run);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const f32x4 vg1 = pg[(ct * 4 + r4) * 64];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[ct][4 * r4 + e] = __builtin_fmaf(vg1[e], fg, o[ct][4 * r4 + e]);
        }
    }
  }
  const float inv = 1.0f / half_swap_sum(l_run);
  __bf16* ow = lds + qb * 32 * OP;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      bf16x4 val;
#pragma unroll
      for (int e = 0; e < 4; ++e) val[e] = static_cast<__bf16>(o[ct][4 * r4 + e] * inv);
      *reinterpret_cast<bf16x4*>(ow + n * OP + ct * 32 + r4 * 8 + 4 * hf) = val;
    }
  constexpr int CH = D / 8;
  constexpr int NU = 32 * CH / 64;
  static_assert(32 * CH % 64 == 0, "whole store instructions per wave");
  bf16x8 piece_val[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int cidx = u * 64 + lane;
    piece_val[u] = *reinterpret_cast<const bf16x8*>(ow + (cidx / CH) * OP + (cidx % CH) * 8);
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int cidx = u * 64 + lane;
    const int row = cidx / CH;
    if (qmin + row < L)
      __builtin_nontemporal_store(piece_val[u],
                                  reinterpret_cast<bf16x8*>(og + static_cast<size_t>(qmin + row) * a.ldo + (cidx % CH) * 8));
  }
}

}  // namespace mgattn
