// qknorm_api.cpp -- the C ABI of libqknorm: argument validation, schedule
// choice and launch. Validation runs entirely on the host and before any HIP
// call, so every error path can be exercised without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>

#include "qknorm.h"
#include "qknorm_launch.h"

struct qknorm_ctx {
  int device;
  int num_cus;
  qknorm_options opt;
};

namespace {

constexpr int64_t kVecBytes = 16;
constexpr int kMaxSlices = 64;
constexpr int64_t kMaxRows = (int64_t{1} << 31) - 1;
constexpr int64_t kMaxTotalWidth = int64_t{1} << 24;  // exact as a float divisor

int elem_bytes(int dtype) { return dtype == QKNORM_F32 ? 4 : dtype == QKNORM_BF16 ? 2 : 1; }
// gamma is bf16 for fp8 rows, else the rows' own type
int gamma_elem_bytes(int dtype) { return dtype == QKNORM_FP8_E4M3 ? 2 : elem_bytes(dtype); }
int64_t vec_elems(int dtype) { return kVecBytes / elem_bytes(dtype); }
bool valid_dtype(int dtype) { return dtype == QKNORM_F32 || dtype == QKNORM_BF16 || dtype == QKNORM_FP8_E4M3; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Byte footprint of `n` rows: row r starts at base + r*stride and is
// `width` bytes long.
struct Rows {
  uintptr_t base;
  int64_t width;
  int64_t stride;
  int64_t n;
};

// Do two row sets share a byte? Exact when their bounding ranges are apart,
// or when they repeat with one period (the same stride, or one of them is a
// single row) and their column windows are disjoint modulo that period, as
// the query and key columns of one packed QKV buffer are. Otherwise
// conservatively "yes".
bool overlap(const Rows& a, const Rows& b) {
  if (a.n <= 0 || b.n <= 0 || a.width <= 0 || b.width <= 0) return false;
  const uintptr_t a_end = a.base + static_cast<uintptr_t>((a.n - 1) * a.stride + a.width);
  const uintptr_t b_end = b.base + static_cast<uintptr_t>((b.n - 1) * b.stride + b.width);
  if (a_end <= b.base || b_end <= a.base) return false;
  int64_t S = 0;
  if (a.n > 1 && b.n > 1)
    S = a.stride == b.stride ? a.stride : 0;
  else
    S = a.n > 1 ? a.stride : b.stride;
  if (S > 0 && a.width <= S && b.width <= S) {
    int64_t d = static_cast<int64_t>(b.base - a.base) % S;
    if (d < 0) d += S;
    if (a.width <= d && d + b.width <= S) return false;
  }
  return true;
}

Rows in_rows(const qknorm_rows& r, int dtype, int64_t T) {
  const int eb = elem_bytes(dtype);
  return Rows{reinterpret_cast<uintptr_t>(r.x), r.width * eb, r.x_stride * eb, T};
}
Rows out_rows(const qknorm_rows& r, int dtype, int64_t T) {
  const int eb = elem_bytes(dtype);
  return Rows{reinterpret_cast<uintptr_t>(r.y), r.width * eb, r.y_stride * eb, T};
}
Rows flat(const void* p, int64_t bytes) {
  return Rows{reinterpret_cast<uintptr_t>(p), bytes, bytes, 1};
}

// One tensor's shape checks (null, shape, alignment), shared by all calls.
int check_rows(const qknorm_rows* r, const void* gamma, int dtype, bool need_y, bool need_gamma) {
  if (r == nullptr || r->x == nullptr || (need_y && r->y == nullptr) ||
      (need_gamma && gamma == nullptr))
    return QKNORM_ERR_NULL;
  if (r->width < 1 || r->x_stride < r->width || (need_y && r->y_stride < r->width))
    return QKNORM_ERR_SHAPE;
  const int64_t ve = vec_elems(dtype);
  if (r->width % ve != 0 || r->x_stride % ve != 0 || (need_y && r->y_stride % ve != 0))
    return QKNORM_ERR_ALIGN;
  if (!aligned16(r->x) || (need_y && !aligned16(r->y)) || (need_gamma && !aligned16(gamma)))
    return QKNORM_ERR_ALIGN;
  return QKNORM_OK;
}

// In place (same pointer, same stride) or disjoint.
bool in_out_ok(const qknorm_rows& r, int dtype, int64_t T) {
  if (r.y == r.x) return r.y_stride == r.x_stride;
  return !overlap(in_rows(r, dtype, T), out_rows(r, dtype, T));
}

bool eps_ok(float eps) { return std::isfinite(eps) && eps >= 0.0f; }

int check_ctx(const qknorm_ctx* ctx) {
  if (ctx == nullptr) return QKNORM_ERR_CONTEXT;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur != ctx->device) return QKNORM_ERR_DEVICE;
  return QKNORM_OK;
}

// Vectors per head when `head_dim` columns make a valid head (a power of two
// of 16-byte vectors, at most one wavefront's 64), else 0.
int head_vectors(int64_t head_dim, int dtype) {
  const int64_t bytes = head_dim * elem_bytes(dtype);
  if (head_dim < 1 || bytes % kVecBytes != 0) return 0;
  const int64_t hv = bytes / kVecBytes;
  return (hv <= 64 && (hv & (hv - 1)) == 0) ? static_cast<int>(hv) : 0;
}

// Validation shared by the two fused calls, after dtype and T: each tensor's
// pointers, shape and alignment, its cut (num_slices equal slices, or heads
// of head_dim columns when `headwise`), eps, then aliasing. gamma has
// `width` weights (layerwise) or `head_dim` (headwise).
int check_fused(int dtype, int64_t T, const qknorm_rows* const* segs, const void* const* gammas, int nseg,
                int num_slices, bool headwise, int64_t head_dim, float eps) {
  const int64_t ve = vec_elems(dtype);
  for (int i = 0; i < nseg; ++i) {
    const int st = check_rows(segs[i], gammas[i], dtype, true, true);
    if (st != QKNORM_OK) return st;
    if (segs[i]->width > qknorm_max_width(dtype)) return QKNORM_ERR_SHAPE;
    if (headwise) {
      if (head_vectors(head_dim, dtype) == 0 || segs[i]->width % head_dim != 0) return QKNORM_ERR_SLICES;
    } else if (num_slices < 1 || num_slices > kMaxSlices || segs[i]->width % num_slices != 0 ||
               (segs[i]->width / num_slices) % ve != 0) {
      return QKNORM_ERR_SLICES;
    }
  }
  if (!eps_ok(eps)) return QKNORM_ERR_EPS;
  const int geb = gamma_elem_bytes(dtype);
  for (int i = 0; i < nseg; ++i) {
    if (!in_out_ok(*segs[i], dtype, T)) return QKNORM_ERR_ALIAS;
    const Rows yi = out_rows(*segs[i], dtype, T);
    for (int j = 0; j < nseg; ++j) {
      const int64_t gw = headwise ? head_dim : segs[j]->width;
      if (overlap(yi, flat(gammas[j], gw * geb))) return QKNORM_ERR_ALIAS;
      if (j == i) continue;
      if (overlap(yi, in_rows(*segs[j], dtype, T)) || overlap(yi, out_rows(*segs[j], dtype, T)))
        return QKNORM_ERR_ALIAS;
    }
  }
  return QKNORM_OK;
}

// How one segment's rows are spread over lanes.
struct Plan {
  int wpr_log2 = 0;        // team: 2^wpr_log2 wavefronts per row
  int sub_lanes_log2 = 6;  // sub-team: 2^sub_lanes_log2 lanes deal one slice at a time
  int slots = 0;
  bool masked = false;
  int min_slots = 0;       // seg_plan: the fewest slots any sub-team layout of this team needs
};

// Slots per lane of the segmented layout: teams of 2^wl wavefronts, split
// into sub-teams of 2^sl lanes that take the row's K slices round-robin;
// each sub-team deals each of its slices over its lanes.
int seg_slots(int64_t slice_vec, int K, int wl, int sl) {
  const int64_t nsub = int64_t{1} << (6 + wl - sl);
  return static_cast<int>(ceil_div(K, nsub) * ceil_div(slice_vec, int64_t{1} << sl));
}
int plain_slots(int64_t nvec, int wl) {
  return static_cast<int>(ceil_div(nvec, int64_t{64} << wl));
}
// The masked layout: plain strided slots over the whole team.
Plan masked_plan(int64_t nvec, int wl) { return Plan{wl, 6 + wl, plain_slots(nvec, wl), true}; }
// Plans served by the kernels for slices narrower than a wavefront.
bool narrow_plan(const Plan& p) { return p.masked || p.sub_lanes_log2 < 6; }

// Relative cost of a layout: its slots, weighted by the length of the
// contiguous run a load instruction reads per sub-team ((sub-team lanes x
// 16) bytes, or a whole wavefront's for sub-teams of whole wavefronts).
// Runs shorter than a 128-byte line cost more than the slots saved; the
// weights (in quarters: 1, 1.25, 2.5, 4 for runs of >= 128, 64, 32 and 16
// bytes) follow what equal-slot layouts measured on MI355X: 16384 x
// 4096/4096 bf16, 64 slices: 260 us with 2-lane sub-teams against 97 us with
// 8-lane ones; 32 slices: 109 against 87 us with 4-lane against 8-lane ones.
int layout_cost(int slots, int sl) { return slots * (sl >= 3 ? 4 : sl == 2 ? 5 : sl == 1 ? 10 : 16); }

// The sub-team size for a team of 2^wl wavefronts. Sub-teams of whole
// wavefronts come first (fewest slots; ties go to the smaller sub-team: fewer
// partials to combine through LDS). Narrower ones serve many narrow slices:
// among those within `cap` slots the least layout_cost wins (ties to the
// narrowest of at least 8 lanes, which takes fewer rounds of group sums), and
// it replaces the whole-wavefront layout only when it costs less.
Plan seg_plan(int64_t slice_vec, int K, int wl, int cap) {
  Plan best{wl, 6, seg_slots(slice_vec, K, wl, 6), false};
  for (int sl = 7; sl <= 6 + wl; ++sl) {
    const int n = seg_slots(slice_vec, K, wl, sl);
    if (n < best.slots) best = Plan{wl, sl, n, false};
  }
  int fewest = best.slots;
  Plan narrow{};
  for (int sl = 5; sl >= 0; --sl) {
    const int n = seg_slots(slice_vec, K, wl, sl);
    fewest = n < fewest ? n : fewest;
    if (n > cap) continue;
    const int c = layout_cost(n, sl);
    const int cn = narrow.slots ? layout_cost(narrow.slots, narrow.sub_lanes_log2) : -1;
    if (cn < 0 || c < cn || (c == cn && sl >= 3)) narrow = Plan{wl, sl, n, false};
  }
  Plan pick = (narrow.slots && layout_cost(narrow.slots, narrow.sub_lanes_log2) < layout_cost(best.slots, 6))
                  ? narrow : best;
  pick.min_slots = fewest;
  return pick;
}

// Choose the team size for one segment by its row width. The smallest team
// whose slice layout fits the register budget wins: narrow rows get one
// wavefront per row (several rows per workgroup, no LDS reduction, no
// barrier), wide rows get several wavefronts per row. `max_wl` is 2 for
// 4-wavefront workgroups and 4 for 16-wavefront ones; `forced_wl` >= 0 pins
// the team.
bool plan_segment(int64_t nvec, int K, int max_wl, int cap, int forced_wl, Plan* out) {
  const int64_t slice_vec = nvec / K;
  const int lo = forced_wl >= 0 ? forced_wl : 0;
  const int hi = forced_wl >= 0 ? forced_wl : max_wl;
  for (int wl = lo; wl <= hi; ++wl) {
    const Plan p = seg_plan(slice_vec, K, wl, cap);
    // slices much narrower than a sub-team leave most of each slot's lanes
    // empty: the masked layout then issues half the loads or fewer
    const int m = plain_slots(nvec, wl);
    if (m <= cap && 2 * m <= p.min_slots) {
      *out = masked_plan(nvec, wl);
      return true;
    }
    if (p.slots <= cap) {
      *out = p;
      return true;
    }
  }
  for (int wl = lo; wl <= hi; ++wl) {
    const int n = plain_slots(nvec, wl);
    if (n <= cap) {
      *out = masked_plan(nvec, wl);
      return true;
    }
  }
  return false;
}

int forced_log2(const qknorm_ctx* ctx) {
  switch (ctx->opt.waves_per_row) {
    case 1: return 0;
    case 2: return 1;
    case 4: return 2;
    case 8: return 3;
    case 16: return 4;
    default: return -1;
  }
}

struct SegIn {
  int64_t nvec;
  int K;
};

// Plans a launch of 1 or 2 segments of T rows each. Returns QKNORM_OK or
// QKNORM_ERR_SHAPE.
//
// The row width sets the smallest team that holds a row in registers. The
// number of rows per SIMD (measured on MI355X over T = 512 ... 32768 for
// 4096/4096 and 5120/1024 rows) then adjusts it:
//  - fewer than 2 rows per SIMD (decode-sized batches): teams widen, up to
//    one workgroup per row, until there are 2 wavefronts per SIMD, so each
//    row's loads are spread over more wavefronts and finish sooner;
//  - 8 or more wavefronts per SIMD, counting each segment's team (long
//    prefill launches, several rounds of wavefronts per SIMD): a row that
//    would take one wavefront 16 or more slots, or 8 or more when every
//    segment's rows would, is shared by two wavefronts, so each holds half
//    a row and its writes start sooner after its reads (bf16 16384 x 4096,
//    8 slots: 3% faster); with fewer slots one wavefront per row stays
//    faster (FP8 16384 x 4096, 4 slots: 47.7 us against 50.7 us with two).
//    Counting wavefronts rather than rows matters when the query rows
//    already take teams: 3632 x 32768/4096 bf16, whose key rows then take
//    two wavefronts instead of one with 8 slots, 100.0 -> 95.3 us;
//  - in between, every row's loads are issued in the first round, and one
//    wavefront per row is fastest.
int plan_launch(const qknorm_ctx* ctx, int dtype, const SegIn* in, int nseg, int64_t T, Plan* plans, int* nw) {
  const int cap4 = qkn::max_slots(dtype, 4), cap16 = qkn::max_slots(dtype, 16);
  const int fl = forced_log2(ctx);
  bool ok = true;
  bool wide = fl > 2;
  if (!wide) {
    for (int i = 0; i < nseg && ok; ++i) ok = plan_segment(in[i].nvec, in[i].K, 2, cap4, fl, &plans[i]);
    if (!ok) wide = fl < 0;  // retry with 16-wavefront workgroups
  }
  if (wide) {
    ok = true;
    for (int i = 0; i < nseg && ok; ++i) ok = plan_segment(in[i].nvec, in[i].K, 4, cap16, fl, &plans[i]);
    *nw = 16;
    if (!ok) return QKNORM_ERR_SHAPE;
    // Rows this wide take teams of up to 16 wavefronts, so the launch makes
    // several rounds of wavefronts even for modest T; a segment whose rows
    // would take 8 or more slots per lane (the key rows beside such query
    // rows) then widens its team while it keeps 2 or more slots. 1808 x
    // 65536/8192 bf16: 121.8 -> 103.9 us (8192-column key rows in teams of
    // 16 wavefronts instead of 2).
    if (fl < 0) {
      const int64_t simds = int64_t{4} * ctx->num_cus;
      int64_t team_waves = 0;
      for (int i = 0; i < nseg; ++i) team_waves += T << plans[i].wpr_log2;
      if (team_waves >= 8 * simds) {
        for (int i = 0; i < nseg; ++i) {
          if (plans[i].masked || plans[i].slots < 8) continue;
          while (plans[i].wpr_log2 < 4 && plans[i].slots >= 2) {
            const Plan p = seg_plan(in[i].nvec / in[i].K, in[i].K, plans[i].wpr_log2 + 1, cap16);
            if (p.slots > cap16 || p.masked) break;
            plans[i] = p;
          }
        }
      }
    }
    return QKNORM_OK;
  }
  *nw = 4;
  if (!ok) return QKNORM_ERR_SHAPE;
  if (fl < 0) {
    const int64_t simds = int64_t{4} * ctx->num_cus;
    int64_t team_waves = 0;
    for (int i = 0; i < nseg; ++i) team_waves += T << plans[i].wpr_log2;
    if (team_waves >= 8 * simds) {
      // rows of 8-15 slots widen only when every segment's rows do (both
      // 8-slot segments of 16384 x 4096/4096 bf16: 86.7 -> 84.3 us); beside
      // key rows that stay with one wavefront they stay too (26208 x
      // 4096/1024 bf16: 88.9 us widened, 85.3 us not); 16 slots always widen
      bool all = true;
      for (int i = 0; i < nseg; ++i) all = all && (plans[i].wpr_log2 != 0 || plans[i].slots >= 8);
      for (int i = 0; i < nseg; ++i) {
        if (plans[i].wpr_log2 != 0 || plans[i].slots < 8) continue;
        if (plans[i].slots < 16 && !all) continue;
        const Plan p = plans[i].masked ? masked_plan(in[i].nvec, 1)
                                       : seg_plan(in[i].nvec / in[i].K, in[i].K, 1, cap4);
        if (p.slots <= cap4) plans[i] = p;
      }
      return QKNORM_OK;
    }
    const int64_t fill = 2 * simds;  // two wavefronts per SIMD
    for (;;) {
      int64_t waves = 0;
      for (int i = 0; i < nseg; ++i) waves += T << plans[i].wpr_log2;
      if (waves >= fill) break;
      bool widened = false;
      for (int i = 0; i < nseg; ++i) {
        const int wl = plans[i].wpr_log2 + 1;
        if (wl > 2) continue;
        plans[i] = plans[i].masked ? masked_plan(in[i].nvec, wl)
                                   : seg_plan(in[i].nvec / in[i].K, in[i].K, wl, cap4);
        widened = true;
      }
      if (!widened) break;
    }
  }
  return QKNORM_OK;
}

// Lay one segment's rows out over the team's lanes (see qknorm_launch.h).
// Segmented: sub-teams take the slices round-robin and deal each slice's
// vectors from their lane 0 again, so every slot lies in one slice; masked:
// plain strided slots over the whole team.
void fill_layout(qkn::Seg* s, const Plan& p, int nw, int64_t nvec, int K, int64_t T) {
  const int wl = p.wpr_log2;
  const int sl = p.sub_lanes_log2;  // the whole team when masked
  const int64_t ns = int64_t{1} << sl;  // lanes per sub-team
  const int64_t nsub = int64_t{1} << (6 + wl - sl);
  const int64_t slice_vec = nvec / K;
  s->wpr_log2 = wl;
  s->sub_lanes_log2 = sl;
  s->masked = p.masked ? 1 : 0;
  s->rows_per_wg = nw >> wl;
  s->nwg = static_cast<int32_t>(ceil_div(T, s->rows_per_wg));
  s->lay_k = K;
  s->row_bytes = static_cast<uint32_t>(nvec * kVecBytes);
  s->slice_vec = static_cast<int32_t>(slice_vec);
  s->inv_slice_vec = 1.0f / static_cast<float>(slice_vec);
  s->lds_gamma = 0;
  s->lds_gamma_vec = 0;
  s->pack_log2 = 0;
  s->flush_mask = 0;
  // no slot needs a lane test (qkn::slot_offset)
  s->dense = (p.masked || K == 1 || slice_vec % ns == 0) ? 1 : 0;
  s->tail_lanes = static_cast<int32_t>(ns);
  for (int j = 0; j < qkn::kMaxSlots; ++j) {
    s->slot_base[j] = 0;
    s->slot_lim[j] = 0;
  }
  if (p.masked) {
    s->nslot = static_cast<int32_t>(ceil_div(nvec, ns));
    for (int j = 0; j < s->nslot; ++j) {
      s->slot_base[j] = static_cast<int32_t>(j * ns);
      s->slot_lim[j] = static_cast<int32_t>(nvec - j * ns < ns ? nvec - j * ns : ns);
    }
    return;
  }
  const int64_t sps = ceil_div(slice_vec, ns);  // slots per slice
  s->nslot = static_cast<int32_t>(ceil_div(K, nsub) * sps);
  s->tail_lanes = static_cast<int32_t>(slice_vec - (sps - 1) * ns);
  for (int j = 0; j < s->nslot; ++j) {
    const int64_t i = j / sps, ij = j % sps;  // the sub-team's i-th slice, its ij-th slot
    const int64_t left = slice_vec - ij * ns;
    s->slot_base[j] = static_cast<int32_t>(i * nsub * slice_vec + ij * ns);
    s->slot_lim[j] = static_cast<int32_t>((left < ns ? left : ns) | (i << 16));
    if (ij == sps - 1) s->flush_mask |= 1u << j;
  }
}

// The width the mean of squares divides by, and its reciprocal (rounded
// once, from double): the kernels form the mean as S * (1/H), exact when H is
// a power of two and otherwise within an ulp of S / H, which keeps a
// division off the path from the statistic to the scaling.
void set_width(qkn::Seg* s, int64_t h) {
  s->h = static_cast<float>(h);
  s->inv_h = static_cast<float>(1.0 / static_cast<double>(h));
}

// Bytes of the weights of one row of `row_bytes` bytes.
uint32_t gamma_bytes(uint32_t row_bytes, int dtype) {
  return row_bytes / static_cast<uint32_t>(elem_bytes(dtype)) * static_cast<uint32_t>(gamma_elem_bytes(dtype));
}

// Several rows per workgroup share one copy of gamma staged in LDS.
constexpr uint32_t kLdsGammaMax = 32768;
void share_gamma(qkn::Seg* s, int dtype) {
  s->lds_gamma = (s->rows_per_wg > 1 && gamma_bytes(s->row_bytes, dtype) <= kLdsGammaMax) ? 1 : 0;
}

// Launches over many narrow rows, one wavefront each (16 or more rows per
// SIMD): each wavefront takes several rows at once, so it keeps several
// times the loads in flight and its fixed costs (argument loads, offsets,
// the weights) serve several rows.
//  - Statistics-only launches (partial sums, inverse RMS) over rows of 1 or
//    2 slots take 4 or 2 rows: a read-only pass has no stores to overlap its
//    load latency with (16384 rows of 1024 bf16 columns 8.16 -> 6.97 us,
//    32768 of 512: 8.52 -> 7.48 us, 16384 of 2048 fp8: 7.49 -> 7.13 us).
//  - Forward and apply launches over rows of 1 slot take 4 rows (MI355X,
//    q and k rows of the same shape: bf16 8192 x 512 6.94 us against 7.98
//    with one row per wavefront, 65536 x 512 44.5 against 45.5, fp32
//    65536 x 256 44.0 against 45.8, fp8 32768 x 1024 25.3 against 27.3;
//    apply on 8192 x 512: 7.0 against 8.5). With 2 slots, 2 rows per
//    wavefront were 0-3% slower (bf16 65536 x 1024: 85.4 against 83.7), so
//    those keep one row per wavefront.
//
// (FP8 forward launches of a single round once took 2 rows of one tensor per
// wavefront: 2048 x 5120/1024 FP8 8.0 -> 7.15 us at the time. Paired rows serve those
// launches better, 6.45 -> 6.34 us, and below 2 paired wavefronts per SIMD one
// row per wavefront is best: 1024 x 5120/1024 4.46 us against 5.57 with two.)
void rows_per_wave(const qknorm_ctx* ctx, qkn::Variant* v, qkn::Args* a, int nseg) {
  for (int i = 0; i < nseg; ++i) a->seg[i].rpw = 1;
  v->rpw = 1;
  if (v->narrow || v->nw != 4 || v->pipe || ctx->opt.max_workgroups > 0 || ctx->opt.waves_per_row != 0) return;
  int slots = 0;
  for (int i = 0; i < nseg; ++i) {
    if (a->seg[i].wpr_log2 != 0) return;
    slots = a->seg[i].nslot > slots ? a->seg[i].nslot : slots;
  }
  const int64_t simds = int64_t{4} * ctx->num_cus;
  int rpw = 1;
  const bool many = a->T * nseg >= 16 * simds;
  if (v->nt && many && (slots == 1 || (slots == 2 && v->mode == qkn::MODE_STATS)) && v->mode != qkn::MODE_HEAD)
    rpw = slots == 1 ? 4 : 2;
  if (rpw == 1) return;
  v->rpw = rpw;
  for (int i = 0; i < nseg; ++i) {
    a->seg[i].rpw = rpw;
    a->seg[i].nwg = static_cast<int32_t>(ceil_div(a->T, int64_t{a->seg[i].rows_per_wg} * rpw));
  }
}

// Paired rows: a forward launch of two segments whose rows are each one
// slice in one wavefront (with staged weights) gives each wavefront one
// token's row of both, up to 4 paired wavefronts per SIMD (one-wavefront
// rows of both tensors already mean at least one; FP8 rows from 2). A
// workgroup then stores only after all four tokens' rows have arrived, so
// the launch issues nearly all its reads before its writes, where separate
// wavefronts let the narrower rows' stores start while most rows are still
// being read; reads and writes mixed in HBM cost more than either alone (24
// MiB each way: 4.99 us read only, 4.78 us write only, 9.87 us as one
// copy). MI355X, gated back to back, bit for bit the unpaired results,
// against the same launch unpaired: 2048 x 5120/1024 bf16 9.77 -> 8.68 us;
// 1792 x 4096/4096 12.49 -> 10.55; 4096 x 2048/512 9.05 -> 8.42; fp32 2048 x
// 2048/512 8.89 -> 7.40; FP8 3072 x 5120/1024 8.98 -> 8.32, FP8 2048 x
// 5120/1024 6.45 (two rows of one tensor per wavefront) -> 6.34. From about five per
// SIMD the other wavefronts already overlap each row's chain and pairing
// mostly loses (8192 x 4096/1024: 28.5 -> 29.4; FP8 6144 x 5120/1024: 15.1
// -> 16.7); FP8 rows below two per SIMD run best unpaired (1536 x
// 4096/4096: 6.33 against 7.04).
bool pair_band(int64_t T, int num_cus, int dtype) {
  const int64_t simds = int64_t{4} * num_cus;
  return T <= 4 * simds && (dtype != QKNORM_FP8_E4M3 || T >= 2 * simds);
}
// Paired FP8 rows form the products x gamma before the statistic when the
// launch has at most 2 paired wavefronts per SIMD: those kernels hold 16
// more VGPRs per slot and keep 2 or 3 wavefronts per SIMD. MI355X, gated
// back to back, against the scaling after the statistic: 2048 tokens 6.47
// -> 6.13 us (5120/1024 columns) and 8.48 -> 8.35 (8192/1024); at 4 per
// SIMD 10.44 -> 11.67 (4096 tokens, 5120/1024) and 12.91 -> 14.49
// (4096/4096), where the launch no longer fits one round.
bool early_products(int64_t T, int num_cus, int dtype) {
  return dtype == QKNORM_FP8_E4M3 && T <= int64_t{2} * 4 * num_cus;
}
void pair_rows(const qknorm_ctx* ctx, qkn::Variant* v, qkn::Args* a, int nseg) {
  v->pair = false;
  if (nseg != 2 || v->mode != qkn::MODE_FWD || v->nw != 4 || v->narrow || !v->nt || v->pipe ||
      ctx->opt.max_workgroups > 0 || ctx->opt.waves_per_row != 0)
    return;
  for (int i = 0; i < 2; ++i)
    if (a->seg[i].wpr_log2 != 0 || a->seg[i].lay_k != 1 || !a->seg[i].lds_gamma) return;
  if (!pair_band(a->T, ctx->num_cus, v->dtype)) return;
  if (a->seg[1].nslot > a->seg[0].nslot) {  // segment 0 is the wider
    const qkn::Seg t = a->seg[0];
    a->seg[0] = a->seg[1];
    a->seg[1] = t;
  }
  for (int i = 0; i < 2; ++i) a->seg[i].rpw = 1;
  v->rpw = 1;
  v->pair = true;
  v->vpl_b = qkn::body_slots(v->vpl, a->seg[1].nslot);
  v->early = early_products(a->T, ctx->num_cus, v->dtype) && v->vpl + v->vpl_b <= qkn::kEarlySlots;
}

// Packed rows: a launch over many rows (16 or more per SIMD, as for several
// rows per wavefront) whose rows are one slice of at most 32 vectors in one
// wavefront puts 64 / 2^pack_log2 of them in each slot (2^pack_log2 lanes
// per row, the vector count rounded up to a power of two), kPackSlots slots
// per wavefront, where one row per slot leaves lanes idle: the loads, the
// arithmetic and the stores of those lanes carry other rows, and the results
// are bit for bit the one-row ones. MI355X, gated back to back, before
// packing: the same bytes as FP8 rows of 32 vectors (16384 x 512 per tensor)
// and of 64 (8192 x 1024) took 5.70 against 5.11 us for the statistics, 9.93
// against 7.79 for the apply step and 9.96 against 7.97 for the forward.
// In apply launches each lane of a row's group fetches one of the row's
// partials, so groups are also at least as wide as the partials are many.
// A wavefront's rows share one buffer resource, so their span must stay
// below 2^31 bytes.
void pack_rows(const qknorm_ctx* ctx, qkn::Variant* v, qkn::Args* a, int nseg) {
  v->pack = false;
  if (v->mode == qkn::MODE_HEAD || v->pair || v->narrow || v->nw != 4 || !v->nt || v->pipe ||
      ctx->opt.max_workgroups > 0 || ctx->opt.waves_per_row != 0)
    return;
  const int64_t simds = int64_t{4} * ctx->num_cus;
  if (a->T * nseg < 16 * simds) return;
  int hl[2] = {0, 0};
  const int64_t eb = elem_bytes(v->dtype);
  for (int i = 0; i < nseg; ++i) {
    const qkn::Seg& s = a->seg[i];
    const int64_t nvec = s.row_bytes / 16;
    if (s.wpr_log2 != 0 || s.sub_lanes_log2 != 6 || s.masked || s.lay_k != 1 || s.nslot != 1 || nvec > 32) return;
    // a group holds the row's vectors, and in apply launches one lane per partial
    const int64_t lanes = v->mode == qkn::MODE_APPLY && s.comb_k > nvec ? s.comb_k : nvec;
    while ((int64_t{1} << hl[i]) < lanes) ++hl[i];
    if (hl[i] > 5) return;
    const int64_t last = (int64_t{qkn::kPackSlots} << (6 - hl[i])) - 1;  // a wavefront's last row, relative
    const int64_t lim = int64_t{1} << 31;
    if (s.x_stride >= lim || last * s.x_stride * eb + s.row_bytes >= lim) return;
    if (v->mode != qkn::MODE_STATS && (s.y_stride >= lim || last * s.y_stride * eb + s.row_bytes >= lim)) return;
  }
  for (int i = 0; i < nseg; ++i) {
    qkn::Seg& s = a->seg[i];
    s.pack_log2 = hl[i];
    s.rpw = qkn::kPackSlots;
    s.lds_gamma = 0;
    s.nwg = static_cast<int32_t>(ceil_div(a->T, int64_t{v->nw} * qkn::kPackSlots << (6 - hl[i])));
  }
  v->rpw = qkn::kPackSlots;
  v->pack = true;
}

// Enqueue `nseg` segments: grid.x covers the larger segment (capped by the
// persistent-grid option), grid.y selects the segment (paired launches: one
// row of both). A capped forward uses the pipelined variant, whose
// workgroups prefetch their next rows.
int run(const qknorm_ctx* ctx, qkn::Variant v, qkn::Args a, int nseg, void* stream) {
  pair_rows(ctx, &v, &a, nseg);
  if (!v.pair) pack_rows(ctx, &v, &a, nseg);
  if (!v.pair && !v.pack) rows_per_wave(ctx, &v, &a, nseg);
  int64_t gx = 0;
  unsigned lds = 0;
  for (int i = 0; i < nseg; ++i) {
    gx = a.seg[i].nwg > gx ? a.seg[i].nwg : gx;
    // whole chunks of one 16-byte vector per thread (see the kernel's gamma_to_lds)
    const unsigned chunk = 16u * 64u * static_cast<unsigned>(v.nw);
    const unsigned need = (gamma_bytes(a.seg[i].row_bytes, v.dtype) + chunk - 1) / chunk * chunk;
    if (v.pair) {
      // segment 1's weights follow segment 0's
      a.seg[i].lds_gamma_vec = static_cast<int32_t>(lds / 16u);
      lds += need;
    } else if (a.seg[i].lds_gamma && need > lds) {
      lds = need;
    }
  }
  if (gx <= 0) return QKNORM_OK;
  const int cap = ctx->opt.max_workgroups;
  if (cap > 0 && gx > cap) {
    gx = cap;
    v.pipe = v.mode == qkn::MODE_FWD && v.nw == 4;
  }
  if (v.pipe) lds = 0;  // the pipelined body keeps gamma in registers
  // a launch holds at most 2^32 - 1 work-items along x; the workgroups'
  // grid-stride loop covers any rows beyond that
  const int64_t hw_cap = int64_t{0xFFFFFFFF} / (int64_t{64} * v.nw);
  if (gx > hw_cap) gx = hw_cap;
  const hipError_t e = qkn::launch(v, a, dim3(static_cast<unsigned>(gx), static_cast<unsigned>(v.pair ? 1 : nseg)),
                                   lds, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QKNORM_OK : QKNORM_ERR_DEVICE;
}

}  // namespace

extern "C" {

const char* qknorm_status_string(int status) {
  switch (status) {
    case QKNORM_OK: return "ok";
    case QKNORM_ERR_NULL: return "a required pointer is NULL";
    case QKNORM_ERR_SHAPE: return "invalid shape: T, width, stride or h_total out of range";
    case QKNORM_ERR_SLICES: return "invalid slicing: num_slices outside [1, 64], width not cut evenly "
                                   "into whole 16-byte vectors, or slice_index out of range";
    case QKNORM_ERR_ALIGN: return "pointer not 16-byte aligned, or width/stride not whole 16-byte vectors";
    case QKNORM_ERR_DTYPE: return "unsupported dtype";
    case QKNORM_ERR_EPS: return "eps must be finite and >= 0";
    case QKNORM_ERR_ALIAS: return "an output overlaps an input without being that same input";
    case QKNORM_ERR_DEVICE: return "no usable gfx950 device, wrong current device, or a HIP call failed";
    case QKNORM_ERR_CONTEXT: return "context is NULL";
    default: return "unknown status";
  }
}

int64_t qknorm_max_width(int dtype) {
  if (!valid_dtype(dtype)) return 0;
  return int64_t{64} * 16 * qkn::max_slots(dtype, 16) * vec_elems(dtype);
}

int qknorm_create_ex(qknorm_ctx** ctx_out, int device, const qknorm_options* opts) {
  if (ctx_out == nullptr) return QKNORM_ERR_NULL;
  *ctx_out = nullptr;
  qknorm_options o{0, 0, 0};
  if (opts != nullptr) {
    o = *opts;
    const int w = o.waves_per_row;
    if (!(w == 0 || w == 1 || w == 2 || w == 4 || w == 8 || w == 16) || o.max_workgroups < 0 ||
        (o.cached_rows != 0 && o.cached_rows != 1))
      return QKNORM_ERR_SHAPE;
  }
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) return QKNORM_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return QKNORM_ERR_DEVICE;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return QKNORM_ERR_DEVICE;
  qknorm_ctx* c = new (std::nothrow) qknorm_ctx{device, prop.multiProcessorCount, o};
  if (c == nullptr) return QKNORM_ERR_DEVICE;
  *ctx_out = c;
  return QKNORM_OK;
}

int qknorm_create(qknorm_ctx** ctx_out, int device) { return qknorm_create_ex(ctx_out, device, nullptr); }

int qknorm_destroy(qknorm_ctx* ctx) {
  delete ctx;
  return QKNORM_OK;
}

int qknorm_forward(qknorm_ctx* ctx, int dtype, int64_t T, const qknorm_rows* q, const qknorm_rows* k,
                   const void* gamma_q, const void* gamma_k, float eps, int num_slices, void* stream) {
  if (!valid_dtype(dtype)) return QKNORM_ERR_DTYPE;
  if (T < 0 || T > kMaxRows) return QKNORM_ERR_SHAPE;
  if (T == 0) return QKNORM_OK;
  const qknorm_rows* segs[2] = {q, k};
  const void* gammas[2] = {gamma_q, gamma_k};
  const int nseg = k != nullptr ? 2 : 1;
  const int64_t ve = vec_elems(dtype);
  int st = check_fused(dtype, T, segs, gammas, nseg, num_slices, false, 0, eps);
  if (st != QKNORM_OK) return st;
  st = check_ctx(ctx);
  if (st != QKNORM_OK) return st;

  SegIn in[2];
  for (int i = 0; i < nseg; ++i) in[i] = SegIn{segs[i]->width / ve, num_slices};
  Plan plans[2];
  int nw = 4;
  st = plan_launch(ctx, dtype, in, nseg, T, plans, &nw);
  if (st != QKNORM_OK) return st;
  // When only one tensor's rows need the narrow-slice kernels, a large pair
  // runs as two launches, so the other tensor keeps the plain kernels (their
  // registers cost the narrow ones 5-9% on wide query rows: 16384 tokens of
  // 16384/2048 bf16 columns in 8 slices, 218 -> 199 us); below 2^23 vectors
  // the second launch costs more than it saves (about 1.5 us).
  if (nseg == 2 && narrow_plan(plans[0]) != narrow_plan(plans[1]) &&
      T * (in[0].nvec + in[1].nvec) >= (int64_t{1} << 23)) {
    st = qknorm_forward(ctx, dtype, T, q, nullptr, gamma_q, nullptr, eps, num_slices, stream);
    if (st != QKNORM_OK) return st;
    return qknorm_forward(ctx, dtype, T, k, nullptr, gamma_k, nullptr, eps, num_slices, stream);
  }

  bool narrow = false;
  for (int i = 0; i < nseg; ++i) narrow = narrow || narrow_plan(plans[i]);
  qkn::Args a{};
  a.T = T;
  a.eps = eps;
  int slots = 0;
  for (int i = 0; i < nseg; ++i) {
    qkn::Seg& s = a.seg[i];
    s.x = segs[i]->x;
    s.y = segs[i]->y;
    s.gamma = gammas[i];
    s.x_stride = segs[i]->x_stride;
    s.y_stride = segs[i]->y_stride;
    // one kernel serves both segments: the kernels for narrow slices when
    // either needs them (they also run the other layouts)
    fill_layout(&s, plans[i], nw, in[i].nvec, num_slices, T);
    share_gamma(&s, dtype);
    set_width(&s, segs[i]->width);
    s.comb_k = 0;
    slots = s.nslot > slots ? s.nslot : slots;
  }
  qkn::Variant v{dtype, qkn::MODE_FWD, qkn::compiled_vpl(slots, nw, dtype), nw, narrow,
                 ctx->opt.cached_rows == 0 || narrow, false};
  if (v.vpl == 0) return QKNORM_ERR_SHAPE;
  return run(ctx, v, a, nseg, stream);
}

int qknorm_forward_headwise(qknorm_ctx* ctx, int dtype, int64_t T, const qknorm_rows* q, const qknorm_rows* k,
                            const void* gamma_q, const void* gamma_k, int64_t head_dim, float eps,
                            void* stream) {
  if (!valid_dtype(dtype)) return QKNORM_ERR_DTYPE;
  if (T < 0 || T > kMaxRows) return QKNORM_ERR_SHAPE;
  if (T == 0) return QKNORM_OK;
  const qknorm_rows* segs[2] = {q, k};
  const void* gammas[2] = {gamma_q, gamma_k};
  const int nseg = k != nullptr ? 2 : 1;
  int st = check_fused(dtype, T, segs, gammas, nseg, 1, true, head_dim, eps);
  if (st != QKNORM_OK) return st;
  st = check_ctx(ctx);
  if (st != QKNORM_OK) return st;

  const int64_t ve = vec_elems(dtype);
  SegIn in[2];
  for (int i = 0; i < nseg; ++i) in[i] = SegIn{segs[i]->width / ve, 1};
  Plan plans[2];
  int nw = 4;
  st = plan_launch(ctx, dtype, in, nseg, T, plans, &nw);
  if (st != QKNORM_OK) return st;
  const int hv = head_vectors(head_dim, dtype);
  int hl = 0;
  while ((1 << hl) < hv) ++hl;
  qkn::Args a{};
  a.T = T;
  a.eps = eps;
  int slots = 0;
  for (int i = 0; i < nseg; ++i) {
    // one slice is never narrow: heads rely on the strided layout
    if (narrow_plan(plans[i])) return QKNORM_ERR_SHAPE;
    qkn::Seg& s = a.seg[i];
    s.x = segs[i]->x;
    s.y = segs[i]->y;
    s.gamma = gammas[i];
    s.x_stride = segs[i]->x_stride;
    s.y_stride = segs[i]->y_stride;
    fill_layout(&s, plans[i], nw, in[i].nvec, 1, T);
    s.head_log2 = hl;
    set_width(&s, head_dim);
    slots = s.nslot > slots ? s.nslot : slots;
  }
  qkn::Variant v{dtype, qkn::MODE_HEAD, qkn::compiled_vpl(slots, nw, dtype), nw, false, true, false};
  if (v.vpl == 0) return QKNORM_ERR_SHAPE;
  return run(ctx, v, a, nseg, stream);
}

int qknorm_inv_rms(qknorm_ctx* ctx, int dtype, int64_t T, const qknorm_rows* q, const qknorm_rows* k, float eps,
                   int num_slices, float* rinv_q, float* rinv_k, void* stream) {
  if (!valid_dtype(dtype)) return QKNORM_ERR_DTYPE;
  if (T < 0 || T > kMaxRows) return QKNORM_ERR_SHAPE;
  if (T == 0) return QKNORM_OK;
  const qknorm_rows* segs[2] = {q, k};
  float* outs[2] = {rinv_q, rinv_k};
  const int nseg = k != nullptr ? 2 : 1;
  const int64_t ve = vec_elems(dtype);
  for (int i = 0; i < nseg; ++i) {
    if (outs[i] == nullptr) return QKNORM_ERR_NULL;
    const int st = check_rows(segs[i], nullptr, dtype, false, false);
    if (st != QKNORM_OK) return st;
    if (segs[i]->width > qknorm_max_width(dtype)) return QKNORM_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(outs[i]) & 3u) != 0) return QKNORM_ERR_ALIGN;
    if (num_slices < 1 || num_slices > kMaxSlices || segs[i]->width % num_slices != 0 ||
        (segs[i]->width / num_slices) % ve != 0)
      return QKNORM_ERR_SLICES;
  }
  if (!eps_ok(eps)) return QKNORM_ERR_EPS;
  for (int i = 0; i < nseg; ++i) {
    const Rows oi = flat(outs[i], T * 4);
    for (int j = 0; j < nseg; ++j) {
      if (overlap(oi, in_rows(*segs[j], dtype, T))) return QKNORM_ERR_ALIAS;
      if (j != i && overlap(oi, flat(outs[j], T * 4))) return QKNORM_ERR_ALIAS;
    }
  }
  int st = check_ctx(ctx);
  if (st != QKNORM_OK) return st;

  SegIn in[2];
  for (int i = 0; i < nseg; ++i) in[i] = SegIn{segs[i]->width / ve, num_slices};
  Plan plans[2];
  int nw = 4;
  st = plan_launch(ctx, dtype, in, nseg, T, plans, &nw);
  if (st != QKNORM_OK) return st;
  bool narrow = false;
  for (int i = 0; i < nseg; ++i) narrow = narrow || narrow_plan(plans[i]);
  qkn::Args a{};
  a.T = T;
  a.eps = eps;
  int slots = 0;
  for (int i = 0; i < nseg; ++i) {
    qkn::Seg& s = a.seg[i];
    s.x = segs[i]->x;
    s.x_stride = segs[i]->x_stride;
    s.stats_out = outs[i];
    fill_layout(&s, plans[i], nw, in[i].nvec, num_slices, T);
    set_width(&s, segs[i]->width);
    s.emit_rinv = 1;
    slots = s.nslot > slots ? s.nslot : slots;
  }
  qkn::Variant v{dtype, qkn::MODE_STATS, qkn::compiled_vpl(slots, nw, dtype), nw, narrow, true, false};
  if (v.vpl == 0) return QKNORM_ERR_SHAPE;
  return run(ctx, v, a, nseg, stream);
}

int qknorm_partial_stats(qknorm_ctx* ctx, int dtype, int64_t T, const void* x_slice, int64_t x_stride,
                         int64_t slice_width, int slice_index, int num_slices, float* stats, void* stream) {
  if (!valid_dtype(dtype)) return QKNORM_ERR_DTYPE;
  if (T < 0 || T > kMaxRows) return QKNORM_ERR_SHAPE;
  if (T == 0) return QKNORM_OK;
  if (x_slice == nullptr) return QKNORM_ERR_NULL;
  const qknorm_rows r{x_slice, nullptr, slice_width, x_stride, slice_width};
  return qknorm_partial_stats_qk(ctx, dtype, T, &r, nullptr, slice_index, num_slices, stats, nullptr, stream);
}

int qknorm_partial_stats_qk(qknorm_ctx* ctx, int dtype, int64_t T, const qknorm_rows* q_slice,
                            const qknorm_rows* k_slice, int slice_index, int num_slices, float* stats_q,
                            float* stats_k, void* stream) {
  if (!valid_dtype(dtype)) return QKNORM_ERR_DTYPE;
  if (T < 0 || T > kMaxRows) return QKNORM_ERR_SHAPE;
  if (T == 0) return QKNORM_OK;
  const qknorm_rows* segs[2] = {q_slice, k_slice};
  float* outs[2] = {stats_q, stats_k};
  const int nseg = k_slice != nullptr ? 2 : 1;
  for (int i = 0; i < nseg; ++i) {
    if (segs[i] == nullptr || outs[i] == nullptr) return QKNORM_ERR_NULL;
    const int st = check_rows(segs[i], nullptr, dtype, false, false);
    if (st != QKNORM_OK) return st;
    if (segs[i]->width > qknorm_max_width(dtype)) return QKNORM_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(outs[i]) & 3u) != 0) return QKNORM_ERR_ALIGN;
  }
  if (num_slices < 1 || num_slices > kMaxSlices || slice_index < 0 || slice_index >= num_slices)
    return QKNORM_ERR_SLICES;
  float* rows_out[2] = {nullptr, nullptr};
  for (int i = 0; i < nseg; ++i) rows_out[i] = outs[i] + static_cast<int64_t>(slice_index) * T;
  for (int i = 0; i < nseg; ++i) {
    const Rows oi = flat(rows_out[i], T * 4);
    for (int j = 0; j < nseg; ++j) {
      if (overlap(oi, in_rows(*segs[j], dtype, T))) return QKNORM_ERR_ALIAS;
      if (j != i && overlap(oi, flat(rows_out[j], T * 4))) return QKNORM_ERR_ALIAS;
    }
  }
  int st = check_ctx(ctx);
  if (st != QKNORM_OK) return st;

  const int64_t ve = vec_elems(dtype);
  SegIn in[2];
  for (int i = 0; i < nseg; ++i) in[i] = SegIn{segs[i]->width / ve, 1};
  Plan plans[2];
  int nw = 4;
  st = plan_launch(ctx, dtype, in, nseg, T, plans, &nw);
  if (st != QKNORM_OK) return st;
  qkn::Args a{};
  a.T = T;
  a.eps = 0.0f;
  int slots = 0;
  for (int i = 0; i < nseg; ++i) {
    qkn::Seg& s = a.seg[i];
    s.x = segs[i]->x;
    s.x_stride = segs[i]->x_stride;
    s.stats_out = rows_out[i];
    fill_layout(&s, plans[i], nw, in[i].nvec, 1, T);
    set_width(&s, segs[i]->width);
    slots = s.nslot > slots ? s.nslot : slots;
  }
  qkn::Variant v{dtype, qkn::MODE_STATS, qkn::compiled_vpl(slots, nw, dtype), nw, false, true, false};
  if (v.vpl == 0) return QKNORM_ERR_SHAPE;
  return run(ctx, v, a, nseg, stream);
}

int qknorm_apply_stats(qknorm_ctx* ctx, int dtype, int64_t T, const qknorm_rows* x_slice,
                       const void* gamma_slice, const float* stats, int num_slices, int64_t h_total,
                       float eps, void* stream) {
  return qknorm_apply_stats_qk(ctx, dtype, T, x_slice, nullptr, gamma_slice, nullptr, stats, nullptr, num_slices,
                               h_total, 0, eps, stream);
}

int qknorm_apply_stats_qk(qknorm_ctx* ctx, int dtype, int64_t T, const qknorm_rows* q_slice,
                          const qknorm_rows* k_slice, const void* gamma_q_slice, const void* gamma_k_slice,
                          const float* stats_q, const float* stats_k, int num_slices, int64_t hq_total,
                          int64_t hk_total, float eps, void* stream) {
  if (!valid_dtype(dtype)) return QKNORM_ERR_DTYPE;
  if (T < 0 || T > kMaxRows) return QKNORM_ERR_SHAPE;
  if (T == 0) return QKNORM_OK;
  const qknorm_rows* segs[2] = {q_slice, k_slice};
  const void* gammas[2] = {gamma_q_slice, gamma_k_slice};
  const float* stats[2] = {stats_q, stats_k};
  const int64_t totals[2] = {hq_total, hk_total};
  const int nseg = k_slice != nullptr ? 2 : 1;
  for (int i = 0; i < nseg; ++i) {
    if (stats[i] == nullptr) return QKNORM_ERR_NULL;
    const int st = check_rows(segs[i], gammas[i], dtype, true, true);
    if (st != QKNORM_OK) return st;
    if (segs[i]->width > qknorm_max_width(dtype) || totals[i] < segs[i]->width || totals[i] > kMaxTotalWidth)
      return QKNORM_ERR_SHAPE;
    if ((reinterpret_cast<uintptr_t>(stats[i]) & 3u) != 0) return QKNORM_ERR_ALIGN;
  }
  if (num_slices < 1 || num_slices > kMaxSlices) return QKNORM_ERR_SLICES;
  if (!eps_ok(eps)) return QKNORM_ERR_EPS;
  const int geb = gamma_elem_bytes(dtype);
  for (int i = 0; i < nseg; ++i) {
    if (!in_out_ok(*segs[i], dtype, T)) return QKNORM_ERR_ALIAS;
    const Rows yi = out_rows(*segs[i], dtype, T);
    for (int j = 0; j < nseg; ++j) {
      if (overlap(yi, flat(stats[j], num_slices * T * 4)) || overlap(yi, flat(gammas[j], segs[j]->width * geb)))
        return QKNORM_ERR_ALIAS;
      if (j == i) continue;
      if (overlap(yi, in_rows(*segs[j], dtype, T)) || overlap(yi, out_rows(*segs[j], dtype, T)))
        return QKNORM_ERR_ALIAS;
    }
  }
  int st = check_ctx(ctx);
  if (st != QKNORM_OK) return st;

  const int64_t ve = vec_elems(dtype);
  SegIn in[2];
  for (int i = 0; i < nseg; ++i) in[i] = SegIn{segs[i]->width / ve, 1};
  Plan plans[2];
  int nw = 4;
  st = plan_launch(ctx, dtype, in, nseg, T, plans, &nw);
  if (st != QKNORM_OK) return st;
  qkn::Args a{};
  a.T = T;
  a.eps = eps;
  int slots = 0;
  for (int i = 0; i < nseg; ++i) {
    qkn::Seg& s = a.seg[i];
    s.x = segs[i]->x;
    s.y = segs[i]->y;
    s.gamma = gammas[i];
    s.stats_in = stats[i];
    s.x_stride = segs[i]->x_stride;
    s.y_stride = segs[i]->y_stride;
    fill_layout(&s, plans[i], nw, in[i].nvec, 1, T);
    share_gamma(&s, dtype);
    s.comb_k = num_slices;
    set_width(&s, totals[i]);
    slots = s.nslot > slots ? s.nslot : slots;
  }
  qkn::Variant v{dtype, qkn::MODE_APPLY, qkn::compiled_vpl(slots, nw, dtype), nw, false, true, false};
  if (v.vpl == 0) return QKNORM_ERR_SHAPE;
  return run(ctx, v, a, nseg, stream);
}

}  // extern "C"
