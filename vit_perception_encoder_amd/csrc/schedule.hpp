// LDS staging schedules of the bf16 attention kernels: which K/V tile goes into which
// LDS stage, when its DMA is issued and waited for, and which step's keys and values a
// wave reads in each part of its program.  Plain constexpr functions with no GPU
// dependency, shared by the kernels and by a host model that replays every wave's
// program and checks that no stage is read before its DMA is waited for and published
// by a barrier, and none is overwritten before its last read.
#pragma once

#ifdef __HIPCC__
#define MGATTN_HD __host__ __device__
#else
#define MGATTN_HD
#endif

namespace mgattn {
namespace sched {

constexpr MGATTN_HD int imax(int a, int b) { return a > b ? a : b; }

// Geometry shared by both kernels (bf16, 128-key tiles, 64-key softmax steps).
template <int D>
struct Geometry {
  static constexpr int kBlockN = 128;                    // keys per LDS tile
  static constexpr int kStepKeys = 64;                   // keys per softmax step
  static constexpr int kStepsPerTile = kBlockN / kStepKeys;
  static constexpr int kKSlots = D / 8 + 1;              // 16-byte slots per K row (+1 pad)
  static constexpr int kKPitch = kKSlots * 8;            // K row pitch (elements)
  static constexpr int kVPitch = D;                      // V row pitch (elements)
  static constexpr int kKElems = kBlockN * kKPitch;
  static constexpr int kVElems = kBlockN * kVPitch;
  static constexpr int kStageElems = kKElems + kVElems;
  // three stages when they fit in the 160 KB of a CU (head_dim <= 96), else two
  static constexpr int kStages = (3 * kStageElems * 2 <= 160 * 1024) ? 3 : 2;
  static constexpr int kLdsBytes = kStages * kStageElems * 2;
  // LDS DMA instructions (64 lanes x 16 bytes) per tile
  static constexpr int kKDma = (kBlockN * kKSlots + 63) / 64;
  static constexpr int kVDma = kBlockN * D / 8 / 64;
  // of which wave w of W issues instructions w, w + W, ...
  static constexpr MGATTN_HD int k_dma_of(int w, int W) { return kKDma / W + (w < kKDma % W ? 1 : 0); }
  static constexpr MGATTN_HD int v_dma_of(int w, int W) { return kVDma / W + (w < kVDma % W ? 1 : 0); }
  // Q tile of bm rows, 16 bytes per lane
  static constexpr MGATTN_HD int q_dma(int bm) { return bm * D / 8 / 64; }
  // the same with rows padded like K rows (kKSlots slots of 16 bytes, the last one
  // repeating the row's last piece), as the pipelined kernel stores Q
  static constexpr MGATTN_HD int q_pad_dma(int bm) { return (bm * kKSlots + 63) / 64; }
  static constexpr MGATTN_HD int q_pad_dma_of(int w, int W, int bm) {
    return q_pad_dma(bm) / W + (w < q_pad_dma(bm) % W ? 1 : 0);
  }
  static constexpr MGATTN_HD int q_pad_elems(int bm) { return bm * kKPitch; }
};

// ---- the phased kernel (attn_fwd_bf16): two wave groups one phase apart, a barrier
// closing every phase.  A wave's slots are MFMA(0), VALU(0), MFMA(1), ..., VALU(n-1),
// MFMA(n); the leading group (waves 0..W/2-1) runs slot i in phase i, the trailing one
// in phase i+1.  MFMA(0) reads the Q fragments and K of step 0; VALU(j) reads (part of)
// K of step j+1; MFMA(j) reads the rest of K of step j (head_dim 128) and V of step j-1.
// Tile t (steps 2t, 2t+1 at 64 keys per step) sits in stage t % stages; its DMA is
// issued at the start of phase phased_issue_phase(t) (its V one phase later with three
// stages) and waited for at the end of phase phased_wait_phase(t); the Q tile sits in
// the last stage.  Tile 0 and the Q tile are issued before phase 0: the leading
// group's Q rows and K of tile 0 are waited for before the first barrier, the rest at
// the end of phase 0.
constexpr MGATTN_HD int phased_issue_phase(int t, int steps_per_tile, int stages) {
  return imax(2 * steps_per_tile * t - 4, 2 * steps_per_tile * (t - stages + 1) + 2);
}
constexpr MGATTN_HD int phased_wait_phase(int t, int steps_per_tile) { return 2 * steps_per_tile * t - 2; }

// ---- the pipelined kernel (attn_fwd_bf16_pipe): iteration j runs PV of step j-1, QK
// of step j+1 and the softmax of step j; QK of step 0 runs before iteration 0.  Tile t
// sits in stage t % 3; the Q tile (rows padded like K rows) starts at stage 2 and, for
// 256 rows, runs past its end, until tile 2 arrives.  The Q tile and tile 0 are issued
// before the first barrier, which publishes Q and K of tile 0, and tile 1 right after
// it; odd iterations open with a wait for all of the wave's DMA, a barrier, and the
// issue of tile pipe_issue_tile(j).
constexpr MGATTN_HD int pipe_k_step(int j) { return j + 1; }       // K read by iteration j (QK)
constexpr MGATTN_HD int pipe_v_step(int j) { return j - 1; }       // V read by iteration j (PV)
constexpr MGATTN_HD bool pipe_syncs(int j) { return (j & 1) != 0; }
constexpr MGATTN_HD int pipe_issue_tile(int j) { return (j >> 1) + 2; }
constexpr int kPipePrologueTiles = 1;  // tiles issued before the first barrier (tile 1 follows it)
template <int D>
constexpr MGATTN_HD int pipe_q_elem() { return (Geometry<D>::kStages - 1) * Geometry<D>::kStageElems; }
template <int D>
constexpr MGATTN_HD int pipe_lds_elems(int bm) {
  return imax(Geometry<D>::kStages * Geometry<D>::kStageElems, pipe_q_elem<D>() + Geometry<D>::q_pad_elems(bm));
}

// ---- the key-split pipelined kernel (attn_fwd_bf16_pipe<D, W, R, G> with G = 2 or 4
// key groups), for launches with too few (segment, head, query tile) units to fill the
// chip: the groups share every 128-key tile, group g taking keys g*128/G ..
// (g+1)*128/G - 1 of it, so a wave's step j is that part of tile j and each iteration
// consumes a whole tile.  Iteration j reads K
// of tile j+1 (QK) and V of tile j-1 (PV); K tiles live in a ring of two slots, V
// tiles in a ring of three, the Q tile after them.  Before QK(0): DMA of Q, K of tiles
// 0 and 1 and V of tile 0, a wait for Q and K of tile 0, a barrier.  Every iteration j
// (the closing PV-only one included) opens with a wait for all of the wave's DMA but
// V of tile j (the last it issued), a barrier, and the DMA of K of tile j+2 and V of
// tile j+1 (those that exist), in that order.
template <int D>
struct SplitGeometry : Geometry<D> {
  using G = Geometry<D>;
  static constexpr int kKRing = 2, kVRing = 3;
  static constexpr MGATTN_HD int k_slot_elem(int t) { return (t % kKRing) * G::kKElems; }
  static constexpr MGATTN_HD int v_slot_elem(int t) { return kKRing * G::kKElems + (t % kVRing) * G::kVElems; }
  static constexpr int kQElem = kKRing * G::kKElems + kVRing * G::kVElems;
  static constexpr MGATTN_HD int lds_elems(int bm) { return kQElem + G::q_pad_elems(bm); }
};
constexpr MGATTN_HD int split_issue_k(int j) { return j + 2; }  // K tile issued after iteration j's barrier
constexpr MGATTN_HD int split_issue_v(int j) { return j + 1; }  // V tile issued after it
constexpr MGATTN_HD int split_k_tile(int j) { return j + 1; }   // K tile read by iteration j
constexpr MGATTN_HD int split_v_tile(int j) { return j - 1; }   // V tile read by iteration j

}  // namespace sched
}  // namespace mgattn
