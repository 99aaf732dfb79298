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
//
// Packed rows: launches over many rows of one slice and at most 32 vectors
// put 64 / 2^pack_log2 rows in each slot of a wavefront, row i of the slot
// over the aligned lanes i * 2^pack_log2 ... (lane l holding vector
// l mod 2^pack_log2), where one row per slot would leave lanes idle.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
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
  // first, together (a paired launch reads nothing else of a segment):
  const void* x;          // row 0 of the input
  void* y;                // row 0 of the output (FWD, APPLY, HEAD)
  const void* gamma;      // weights of the columns processed (FWD, APPLY); HEAD: of one head
  int64_t x_stride;       // elements between input rows
  int64_t y_stride;       // elements between output rows
  uint32_t row_bytes;     // bytes of one row processed (and of its weights)
  float inv_h;            // 1 / h, rounded once (exact for HEAD's power-of-two heads)
  // the rest of the segment
  const float* stats_in;  // APPLY: partials laid out [comb_k][T]
  float* stats_out;       // STATS: row t's sum goes to stats_out[t]
  int32_t wpr_log2;       // log2 of the wavefronts per team
  int32_t sub_lanes_log2; // log2 of the lanes per sub-team (deals one slice at a time)
  int32_t lds_gamma;      // 1: the workgroup stages gamma in LDS and its rows share it
  int32_t rows_per_wg;    // teams per workgroup
  int32_t nwg;            // workgroups covering all T rows
  int32_t nslot;          // slots per lane in use
  int32_t lay_k;          // partial sums per row (slices)
  int32_t comb_k;         // APPLY: partials combined per row
  int32_t masked;         // masked layout (kernels for narrow slices only)
  int32_t slice_vec;      // masked layout: vectors per slice
  float inv_slice_vec;    // masked layout: 1.0f / slice_vec
  float h;                // the mean of squares divides by this width
  uint32_t flush_mask;    // segmented layout: bit j set when slot j ends a slice
  int32_t head_log2;      // HEAD: log2 of the 16-byte vectors per head (0 ... 6)
  int32_t emit_rinv;      // STATS: write 1 / sqrt(S / h + eps) instead of S
  int32_t rpw;            // rows each one-wavefront team takes at once (1, 2, 4)
  int32_t dense;          // 1: no slot needs a lane test (see slot_offset)
  int32_t tail_lanes;     // lanes of the last slot of each slice (the ragged slot when not dense)
  int32_t lds_gamma_vec;  // paired launches: where this segment's staged gamma starts in LDS
                          // (16-byte vectors; 0 for segment 0). The host sizes LDS by it
                          // and the layout checker compares it with the offset the kernel
                          // derives from segment 0's row bytes.
  int32_t slot_base[kMaxSlots];
  int32_t slot_lim[kMaxSlots];  // 0 for j >= nslot
  int32_t pack_log2;            // packed launches: log2 of the lanes per row (rows of <= 32 vectors)
  int32_t pad_[12];             // whole 64-byte lines per segment
};

// T and eps lead, so that they share a 64-byte line with the first fields of
// segment 0, and segment 1's first fields sit in one line of their own: a
// paired launch reads two lines of arguments (arguments are read through
// scalar loads at kernel entry, and every further line costs time; 512
// bytes spread over a launch's entry cost about 1.3 us).
struct Args {
  int64_t T;   // rows per segment
  float eps;
  int32_t pad_;
  Seg seg[2];  // blockIdx.y selects one (paired launches: both, grid.y = 1)
};
static_assert(sizeof(Seg) % 64 == 0, "segments in whole lines");
static_assert(offsetof(Seg, inv_h) + sizeof(float) <= 48, "a segment's first fields fit the rest of a line");
static_assert(offsetof(Args, seg) == 16, "segment 0 right after T and eps");

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

// Byte offset the kernels' raw buffer accesses use for an empty slot: past
// any row, so the hardware range check reads zeros and drops the store.
constexpr uint32_t kOutsideOffset = 0x80000000u;

// The byte offset of slot j's vector for a lane, as the kernels form it:
// `lane_vec` = sub * slice_vec + stl is the lane's vector within its
// sub-team's first slice (computed once per wavefront) and `base` the
// slot's table entry. The result is 16 * slot_vector() when that vector
// exists; otherwise it is kOutsideOffset, or lies at or past the end of the
// row, where the range check drops the access as well: a sub-team with no
// slice in the slot's round (slice >= K) would start at vector
// K * slice_vec, the row's length. Within a slice every slot but the last
// covers the whole sub-team, and the last one (`ends_slice`, its flush bit)
// covers `tail_lanes` lanes, the same for every slice; lanes past that would
// reach into the next slice, so only such ragged slots need the lane test.
// When a segment has none (`dense`: one slice, the masked layout, or slices
// that are whole multiples of the sub-team), every slot is one addition.
__host__ __device__ inline uint32_t slot_offset(int base, int lane_vec, int stl, bool ends_slice, int tail_lanes,
                                                bool dense) {
  return (dense || !ends_slice || stl < tail_lanes) ? static_cast<uint32_t>(base + lane_vec) * 16u
                                                    : kOutsideOffset;
}

// Packed rows: the byte offset of a lane's vector in one slot, from the
// wavefront's first row (`rel`: the slot's first row plus the lane's row
// within the slot), or kOutsideOffset when the lane holds nothing there (a
// vector past the row, or a row past the `span` rows the wavefront has); and
// the byte length of the buffer resource over the wavefront's rows. Used by
// the kernels and by the host-side layout checks.
__host__ __device__ inline uint32_t packed_offset(int64_t rel, int64_t span, int vec, bool vlive,
                                                  int64_t stride_bytes) {
  return (vlive && rel < span) ? static_cast<uint32_t>(rel * stride_bytes) + static_cast<uint32_t>(vec) * 16u
                               : kOutsideOffset;
}
__host__ __device__ inline uint32_t packed_bytes(int64_t span, int64_t stride_bytes, uint32_t row_bytes) {
  return span > 0 ? static_cast<uint32_t>((span - 1) * stride_bytes) + row_bytes : 0u;
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
  bool pair = false;  // FWD: each wavefront takes one token's row of both segments
                      // (segment 0 the wider), grid.y = 1
  int vpl_b = 0;      // paired: the body for segment 1's rows, on the chain vpl, vpl/2, ...
  bool pack = false;  // FWD, STATS, APPLY: rows of one slice and <= 32 vectors, several
                      // per slot (kPackSlots slots per wavefront)
  bool early = false; // paired FP8: the products x gamma formed before the statistic
};

// Paired FP8 rows form the products x gamma early only when the two rows
// hold at most kEarlySlots slots together: the products take 16 VGPRs per
// slot, and wider pairs would need more than 256 registers (one wavefront
// per SIMD).
constexpr int kEarlySlots = 12;

// Slots per wavefront of a packed launch; each holds 64 / 2^pack_log2 rows.
constexpr int kPackSlots = 4;

// The body for `nslot` slots in a kernel built for `vpl`: the smallest of
// vpl, vpl/2, vpl/4, ... that holds them (the kernels' dispatch).
constexpr int body_slots(int vpl, int nslot) {
  int v = vpl;
  while (v > 1 && nslot <= v / 2) v /= 2;
  return v;
}
constexpr bool on_halving_chain(int vpl, int v) {
  for (int c = vpl; c >= 1; c /= 2)
    if (c == v) return true;
  return false;
}

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

// Whether a kernel is compiled for a variant: the launch dispatch
// instantiates exactly these, and the host-side layout checker confirms
// that every variant the planner reaches is among them (and lists any that
// none reaches).
//  - slot counts: those of kVpl4 / kVpl16 up to the type's register cap;
//  - several rows per wavefront (rpw 2 or 4): 4-wavefront workgroups of
//    whole-wavefront sub-teams, streaming, unpipelined; rows of 1 slot (4
//    rows, every mode but the headwise one), or statistics-only passes over
//    rows of 2 slots (2 rows);
//  - the persistent pipelined body: forward passes in 4-wavefront
//    workgroups;
//  - narrow-slice kernels stream (nt) and never serve the headwise form or
//    the split path's apply step, whose layouts hold one slice;
//  - ordinary cached row accesses (nt off): forward passes only;
//  - paired rows (both segments' rows of a token in one wavefront): forward
//    passes in 4-wavefront workgroups, streaming, one row of each segment per
//    wavefront, the second on the chain vpl, vpl/2, ...
//  - packed rows (several narrow rows in each slot): forward, statistics and
//    apply passes in 4-wavefront workgroups, streaming, one slot per row,
//    kPackSlots slots per wavefront;
//  - early products (x gamma formed before the statistic): paired FP8 rows.
constexpr bool compiled_vpl_value(int vpl, int nw, int dtype) {
  if (vpl < 1 || vpl > max_slots(dtype, nw)) return false;
  if (nw == 4) {
    for (int c : kVpl4)
      if (c == vpl) return true;
  } else if (nw == 16) {
    for (int c : kVpl16)
      if (c == vpl) return true;
  }
  return false;
}
constexpr bool compiled(int dtype, int mode, int vpl, int nw, bool narrow, bool nt, bool pipe, int rpw,
                        int pair_b = 0, bool pack = false, bool early = false) {
  if (!compiled_vpl_value(vpl, nw, dtype)) return false;
  if (early && (dtype != QKNORM_FP8_E4M3 || pair_b == 0 || pack || vpl + pair_b > kEarlySlots)) return false;
  if (pack)
    return (mode == MODE_FWD || mode == MODE_STATS || mode == MODE_APPLY) && vpl == 1 && nw == 4 && !narrow && nt &&
           !pipe && rpw == kPackSlots && pair_b == 0;
  if (pair_b != 0)
    return mode == MODE_FWD && nw == 4 && !narrow && nt && !pipe && rpw == 1 && on_halving_chain(vpl, pair_b);
  if (rpw != 1) {
    if (nw != 4 || narrow || !nt || pipe) return false;
    return (vpl == 1 && rpw == 4 && mode != MODE_HEAD) || (mode == MODE_STATS && vpl == 2 && rpw == 2);
  }
  if (narrow && !nt) return false;
  if (pipe && (mode != MODE_FWD || nw != 4)) return false;
  if (!nt && mode != MODE_FWD) return false;
  if (narrow && (mode == MODE_HEAD || mode == MODE_APPLY)) return false;
  return true;
}
inline bool compiled(const Variant& v) {
  return compiled(v.dtype, v.mode, v.vpl, v.nw, v.narrow, v.nt, v.pipe, v.rpw, v.pair ? v.vpl_b : 0, v.pack,
                  v.early);
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
