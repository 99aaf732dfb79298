// qknorm_launch.h -- what the host API hands to the gfx950 kernels.
//
// One launch covers up to two "segments": the query rows and the key rows of
// the same tokens (or the single tensor of a split-path call). Each segment
// is processed by teams of `wpr` wavefronts; a team owns one row at a time.
//
// Register layout of a row inside a team ("slots"): the row's 16-byte
// vectors are grouped by column slice. The team's lanes form sub-teams of
// 2^sub_lanes_log2 lanes (a power of two from one lane to the whole team);
// sub-team u takes slices u, u + nsub, u + 2 nsub, ... one after the other
// and deals each slice's vectors over its own lanes from its lane 0. Slot j
// of a lane therefore always lies inside one slice, and a slice's partial sum
// of squares is a reduction over its sub-team's lanes and the slots of that
// slice. With one slice and sub-teams as wide as the team this is the usual
// strided layout (vector v in lane v % team, slot v / team). Sub-teams
// narrower than a wavefront serve many narrow slices: with as many sub-teams
// as slices, each lane holds one slice in all its slots, and a group sum over
// the sub-team's lanes gives the partial.
//
// When every such layout would need too many slots, the kernel falls back to
// the "masked" layout: plain strided vectors, and a per-lane slice index
// selects which partial each vector's squares join.
//
// Headwise rows use the one-slice (strided) layout. A head is a power of two
// of at most 64 vectors, so each head sits in one slot of one aligned group
// of lanes of one wavefront, and lane l always holds the head's vector
// l mod (vectors per head): its weights are the same in every slot.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qknorm.h"

namespace qkn {

enum Mode : int {
  MODE_FWD = 0,    // statistic and scaling in one pass (row stays in registers)
  MODE_STATS = 1,  // statistic only: one fp32 per row to `stats_out` (S, or 1/RMS if emit_rinv)
  MODE_APPLY = 2,  // combine `comb_k` precomputed partials, then scale
  MODE_HEAD = 3,   // headwise: every head of 2^head_log2 vectors has its own statistic
};

constexpr int kMaxSlots = 16;  // slots per lane of the widest compiled variant

// Slot tables: slot j of sub-team 0 starts at vector slot_base[j] of the
// row; slot_lim[j] packs the lanes it covers (low 16 bits) and which of the
// sub-team's slices it belongs to (high 16 bits). Sub-team u adds
// u * slice_vec to the base and owns slices u, u + nsub, u + 2 nsub, ...
// (nsub = team lanes / sub-team lanes).
struct Seg {
  const void* x;          // row 0 of the input
  void* y;                // row 0 of the output (FWD, APPLY, HEAD)
  const void* gamma;      // weights of the columns processed (FWD, APPLY); HEAD: of one head
  const float* stats_in;  // APPLY: partials laid out [comb_k][T]
  float* stats_out;       // STATS: row t's sum goes to stats_out[t]
  int64_t x_stride;       // elements between input rows
  int64_t y_stride;       // elements between output rows
  int32_t wpr_log2;       // log2 of the wavefronts per team
  int32_t sub_lanes_log2; // log2 of the lanes per sub-team (deals one slice at a time)
  int32_t lds_gamma;      // 1: the workgroup stages gamma in LDS and its rows share it
  int32_t rows_per_wg;    // teams per workgroup
  int32_t nwg;            // workgroups covering all T rows
  int32_t nslot;          // slots per lane in use
  uint32_t row_bytes;     // bytes of one row processed (and of its weights)
  int32_t lay_k;          // partial sums per row (slices)
  int32_t comb_k;         // APPLY: partials combined per row
  int32_t masked;         // masked layout (kernels for narrow slices only)
  int32_t slice_vec;      // masked layout: vectors per slice
  float inv_slice_vec;    // masked layout: 1.0f / slice_vec
  float h;                // the mean of squares divides by this width
  uint32_t flush_mask;    // segmented layout: bit j set when slot j ends a slice
  int32_t head_log2;      // HEAD: log2 of the 16-byte vectors per head (0 ... 6)
  float inv_h;            // 1 / h, rounded once (exact for HEAD's power-of-two heads)
  int32_t emit_rinv;      // STATS: write 1 / sqrt(S / h + eps) instead of S
  int32_t rpw;            // rows each one-wavefront team takes at once (1, 2, 4)
  int32_t slot_base[kMaxSlots];
  int32_t slot_lim[kMaxSlots];  // 0 for j >= nslot
};

struct Args {
  Seg seg[2];  // blockIdx.y selects one
  int64_t T;   // rows per segment
  float eps;
};

// The row vector that slot j of team lane `tl` holds, or -1 when the slot is
// empty there. `lim_word` and `base` are the slot's table entries. Used by
// the kernels and by the host-side layout checks.
__host__ __device__ inline int slot_vector(int lim_word, int base, int tl, int wpr_log2, int sub_lanes_log2,
                                           int slice_vec, int K) {
  const int sub = tl >> sub_lanes_log2;             // sub-team within the team
  const int stl = tl & ((1 << sub_lanes_log2) - 1);  // lane within the sub-team
  const int slice = sub + ((lim_word >> 16) << (6 + wpr_log2 - sub_lanes_log2));
  return (stl < (lim_word & 0xffff) && slice < K) ? base + sub * slice_vec + stl : -1;
}

// Compile-time variants a launch picks from.
struct Variant {
  int dtype;     // qknorm_dtype
  int mode;      // Mode
  int vpl;       // slots per lane the kernel is built for (>= what the segments need)
  int nw;        // wavefronts per workgroup: 4 or 16
  bool narrow;   // FWD, STATS: slices narrower than a wavefront (sub-teams of
                 // fewer than 64 lanes, or the masked layout)
  bool nt;       // FWD only: non-temporal row loads and stores
  bool pipe;     // FWD only: persistent workgroups with the next rows prefetched
  int rpw = 1;   // rows per one-wavefront team (1, or 2 / 4 for rows of at most 2 slots)
};

// Slot counts the kernels are compiled for, per workgroup size. In
// 4-wavefront workgroups every count up to 8 has its own body: a row runs
// the smallest body that fits, and slots past its own count still cost
// their loads and arithmetic (an FP8 slot about 80 vector instructions per
// row). 2048 x 5120/1024 FP8 (5 slots): 6.79 -> 6.48 us with the exact
// body; 256 x 5120 bf16 in teams of 4 wavefronts (3 slots): 4.25 -> 4.14 us.
constexpr int kVpl4[] = {1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 16};
constexpr int kVpl16[] = {1, 2, 4, 8};

// Most slots per lane for an element type and workgroup size. An FP8 slot
// holds its 16-byte vector and two 16-byte weight vectors (bf16 weights), so
// FP8 stops at 8 slots (4 in 16-wavefront workgroups, whose wavefronts get
// at most 128 VGPRs) and wider rows take bigger teams instead.
constexpr int max_slots(int dtype, int nw) {
  return dtype == QKNORM_FP8_E4M3 ? (nw == 4 ? 8 : 4) : (nw == 4 ? 16 : 8);
}

// Smallest compiled slot count >= `slots` for `nw` wavefronts per workgroup,
// or 0 when none is large enough.
inline int compiled_vpl(int slots, int nw, int dtype) {
  if (slots > max_slots(dtype, nw)) return 0;
  if (nw == 4) {
    for (int c : kVpl4)
      if (c >= slots) return c;
  } else if (nw == 16) {
    for (int c : kVpl16)
      if (c >= slots) return c;
  }
  return 0;
}

// Enqueue one launch: grid.x workgroups per segment, grid.y segments, with
// `lds_bytes` of dynamic LDS for staged gamma. Returns hipSuccess or the
// launch error. Dispatches on v.dtype to one of the per-type entries below,
// each built in its own translation unit.
hipError_t launch(const Variant& v, const Args& a, dim3 grid, unsigned lds_bytes, hipStream_t stream);
hipError_t launch_f32(const Variant& v, const Args& a, dim3 grid, unsigned lds_bytes, hipStream_t stream);
hipError_t launch_bf16(const Variant& v, const Args& a, dim3 grid, unsigned lds_bytes, hipStream_t stream);
hipError_t launch_fp8(const Variant& v, const Args& a, dim3 grid, unsigned lds_bytes, hipStream_t stream);

}  // namespace qkn
