// Host-side check of the launch planner and the slot tables (no GPU).
//
// Includes the library's host source, replaces the device launch with a
// recorder, and for a grid of row widths, slice counts, row counts and team
// sizes verifies, through the same slot_vector() the kernels use, that:
//  - every vector of a row is held by exactly one (lane, slot) of its team;
//  - each slot of a sub-team lies inside one slice;
//  - a sub-team's slots of one slice are consecutive and the last one has
//    its flush bit set, and the i-th flush is slice sub + i * nsub, which is
//    where the LDS combine looks for it;
//  - the slot count fits a compiled variant, and staged gamma fits the
//    copy loop's bound;
//  - headwise plans keep every head inside one aligned lane group of one
//    wavefront and slot, lane l holding the head's vector l mod (vectors
//    per head);
//  - the kernels' slot offsets (slot_offset) equal the table's vectors, or
//    fall where the buffer range check drops the access;
//  - every public entry point, over shapes, slice counts and every
//    combination of schedule options, asks only for variants that have a
//    kernel (compiled()), and every compiled variant is reached by some
//    call.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <set>
#include <tuple>
#include <vector>

// The entry points ask HIP for the current device before launching; here
// there is none, so the library's call is routed to this stand-in (device 0,
// the fake contexts' device) and every entry point runs its real validation
// and planning up to the launch, which the recorder below replaces.
static hipError_t layout_check_hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
#define hipGetDevice layout_check_hipGetDevice
#include "qknorm_api.cpp"
#undef hipGetDevice

namespace qkn {
static Variant g_v;
static Args g_a;
static dim3 g_grid;
static unsigned g_lds;
using VariantKey = std::tuple<int, int, int, int, bool, bool, bool, int, int, bool, bool>;
static VariantKey key(const Variant& v) {
  return VariantKey{v.dtype, v.mode, v.vpl, v.nw, v.narrow, v.nt, v.pipe, v.rpw, v.pair ? v.vpl_b : 0, v.pack,
                    v.early};
}
static long g_paired, g_packed, g_packed_covered;
static void check_pair_launch(const Variant& v, const Args& a, dim3 grid, unsigned lds);
static void check_pack_launch(const Variant& v, const Args& a, dim3 grid, unsigned lds);
static std::set<VariantKey> g_reached;
static long g_launches, g_uncompiled;
hipError_t launch(const Variant& v, const Args& a, dim3 grid, unsigned lds_bytes, hipStream_t) {
  g_v = v;
  g_a = a;
  g_grid = grid;
  g_lds = lds_bytes;
  g_reached.insert(key(v));
  ++g_launches;
  if (v.pair) check_pair_launch(v, a, grid, lds_bytes);
  if (v.pack) check_pack_launch(v, a, grid, lds_bytes);
  if (!compiled(v)) {
    if (g_uncompiled < 10)
      std::printf("FAIL no kernel for reached variant dtype=%d mode=%d vpl=%d nw=%d narrow=%d nt=%d pipe=%d rpw=%d "
                  "pack=%d\n",
                  v.dtype, v.mode, v.vpl, v.nw, v.narrow, v.nt, v.pipe, v.rpw, v.pack);
    ++g_uncompiled;
    return hipErrorInvalidValue;
  }
  return hipSuccess;
}
}  // namespace qkn

static int failures = 0;
static long g_layouts[3];  // segments laid out with whole-wavefront sub-teams, narrower ones, masked
static long g_dense;       // segments whose slots need no lane test
#define CHECK(c, ...)                          \
  do {                                         \
    if (!(c)) {                                \
      if (failures < 20) {                     \
        std::printf("FAIL %s: ", #c);          \
        std::printf(__VA_ARGS__);              \
        std::printf("\n");                    \
      }                                        \
      ++failures;                              \
    }                                          \
  } while (0)

static int body_slots(int vpl, int nslot) {  // the kernel's dispatch: VPL, VPL/2, ...
  int v = vpl;
  while (v > 1 && nslot <= v / 2) v /= 2;
  return v;
}

// A paired forward launch (both segments' rows of a token in one
// wavefront): one-wavefront teams in both segments with staged weights,
// segment 0 the wider, segment 1 on the body the kernel is built with, the
// same workgroups covering both, one grid row, and segment 1's weights
// placed right after segment 0's in LDS.
void qkn::check_pair_launch(const Variant& v, const Args& a, dim3 grid, unsigned lds) {
  ++g_paired;
  const Seg &s0 = a.seg[0], &s1 = a.seg[1];
  CHECK(v.mode == MODE_FWD && v.nw == 4 && !v.narrow && v.nt && !v.pipe && v.rpw == 1, "paired variant");
  CHECK(s0.wpr_log2 == 0 && s1.wpr_log2 == 0 && s0.rows_per_wg == 4 && s1.rows_per_wg == 4,
        "paired teams %d/%d", s0.wpr_log2, s1.wpr_log2);
  CHECK(s0.lds_gamma && s1.lds_gamma && !s0.masked && !s1.masked && s0.lay_k == 1 && s1.lay_k == 1,
        "paired segments' weights or layout");
  // the kernel lays both rows out as plain strided slots (slot j, lane l:
  // vector 64 j + l, or dropped past the row): the table's layout
  for (int i = 0; i < 2; ++i) {
    const Seg& s = a.seg[i];
    const int nvec = static_cast<int>(s.row_bytes / 16);
    for (int j = 0; j < s.nslot; ++j)
      for (int l = 0; l < 64; ++l) {
        const int v = slot_vector(s.slot_lim[j], s.slot_base[j], l, 0, 6, s.slice_vec, 1);
        const int want = j * 64 + l < nvec ? j * 64 + l : -1;
        CHECK(v == want, "paired segment %d slot %d lane %d: table %d, strided %d", i, j, l, v, want);
      }
  }
  CHECK(s0.nslot >= s1.nslot && s0.nslot <= v.vpl && v.vpl_b == body_slots(v.vpl, s1.nslot),
        "paired slots %d/%d on bodies %d/%d", s0.nslot, s1.nslot, v.vpl, v.vpl_b);
  // early products: FP8 launches of at most 2 paired wavefronts per SIMD (256 compute units)
  CHECK(v.early == (v.dtype == QKNORM_FP8_E4M3 && a.T <= 2 * 4 * 256 && v.vpl + v.vpl_b <= kEarlySlots),
        "paired T=%lld slots %d + %d early=%d", (long long)a.T, v.vpl, v.vpl_b, v.early ? 1 : 0);
  CHECK(s0.nwg == s1.nwg && int64_t{s0.nwg} * 4 >= a.T && int64_t{s0.nwg - 1} * 4 < a.T && grid.x == unsigned(s0.nwg) &&
            grid.y == 1,
        "paired grid %u x %u for %d workgroups", grid.x, grid.y, s0.nwg);
  const unsigned chunk = 16u * 64u * 4u;
  const unsigned need0 = (gamma_bytes(s0.row_bytes, v.dtype) + chunk - 1) / chunk * chunk;
  const unsigned need1 = (gamma_bytes(s1.row_bytes, v.dtype) + chunk - 1) / chunk * chunk;
  CHECK(s0.lds_gamma_vec == 0 && unsigned(s1.lds_gamma_vec) * 16u == need0 && lds == need0 + need1,
        "paired LDS: segment 1 at %d vectors, %u bytes", s1.lds_gamma_vec, lds);
  // the copy loops of the two bodies cover each segment's weights
  for (int i = 0; i < 2; ++i) {
    const int body = i == 0 ? v.vpl : v.vpl_b;
    const int64_t gvec = gamma_bytes(a.seg[i].row_bytes, v.dtype) / 16;
    CHECK(gvec <= int64_t{(body + 1) / 2} * 4 * 64 * (v.dtype == QKNORM_FP8_E4M3 ? 2 : 1),
          "paired segment %d: %lld weight vectors past the copy loop of body %d", i, (long long)gvec, body);
  }
}

// A packed launch (several narrow rows per slot): every segment one slice
// of at most 32 vectors in one-wavefront teams, 2^pack_log2 lanes per row
// (the vector count, or in apply launches the partials if more, rounded up
// to a power of two), no staged weights, the
// workgroups covering all rows, and a wavefront's rows within one buffer
// resource. For up to 20001 rows, the kernel's index arithmetic is run for
// every workgroup, wavefront, slot and lane: each (row, vector) is held by
// exactly one lane, every live offset lies inside the wavefront's resource
// and points at that vector, and every other lane's offset is dropped.
void qkn::check_pack_launch(const Variant& v, const Args& a, dim3 grid, unsigned lds) {
  ++g_packed;
  CHECK((v.mode == MODE_FWD || v.mode == MODE_STATS || v.mode == MODE_APPLY) && v.nw == 4 && v.vpl == 1 &&
            !v.narrow && v.nt && !v.pipe && v.rpw == kPackSlots && !v.pair,
        "packed variant mode %d", v.mode);
  CHECK(lds == 0, "packed launch with %u bytes of LDS", lds);
  const int nseg = static_cast<int>(grid.y);
  CHECK(nseg == 1 || nseg == 2, "packed grid.y %u", grid.y);
  const int64_t T = a.T;
  const int eb = elem_bytes(v.dtype);
  for (int i = 0; i < nseg; ++i) {
    const Seg& s = a.seg[i];
    const int64_t nvec = s.row_bytes / 16;
    const int hl = s.pack_log2;
    CHECK(s.wpr_log2 == 0 && s.sub_lanes_log2 == 6 && !s.masked && s.lay_k == 1 && s.nslot == 1 && !s.lds_gamma &&
              s.rpw == kPackSlots && s.rows_per_wg == 4,
          "packed segment %d layout", i);
    // a group: the row's vectors, and in apply launches a lane per partial
    const int64_t lanes = v.mode == MODE_APPLY && s.comb_k > nvec ? s.comb_k : nvec;
    CHECK(nvec >= 1 && nvec <= 32 && hl >= 0 && hl <= 5 && (int64_t{1} << hl) >= lanes &&
              (hl == 0 || (int64_t{1} << (hl - 1)) < lanes),
          "packed segment %d: %lld vectors (%d partials) in groups of 2^%d lanes", i, (long long)nvec, s.comb_k, hl);
    const int64_t per_wave = int64_t{kPackSlots} << (6 - hl), per_wg = 4 * per_wave;
    CHECK(int64_t{s.nwg} * per_wg >= T && int64_t{s.nwg - 1} * per_wg < T && grid.x >= unsigned(s.nwg),
          "packed segment %d: %d workgroups of %lld rows for T=%lld, grid %u", i, s.nwg, (long long)per_wg,
          (long long)T, grid.x);
    const int64_t xs = s.x_stride * eb, ys = s.y_stride * eb;
    CHECK((per_wave - 1) * xs + s.row_bytes < (int64_t{1} << 31), "packed segment %d: input span", i);
    CHECK(v.mode == MODE_STATS || (per_wave - 1) * ys + s.row_bytes < (int64_t{1} << 31),
          "packed segment %d: output span", i);
    if (T > 20001) continue;
    ++g_packed_covered;
    std::vector<unsigned char> held(static_cast<size_t>(T * nvec), 0);
    for (int64_t gi = 0; gi < s.nwg; ++gi)
      for (int wave = 0; wave < 4; ++wave) {
        const int64_t row0 = ((gi * 4 + wave) * kPackSlots) << (6 - hl);
        int64_t span = T - row0;
        span = span < per_wave ? span : per_wave;
        const uint32_t xbytes = packed_bytes(span, xs, s.row_bytes), ybytes = packed_bytes(span, ys, s.row_bytes);
        for (int j = 0; j < kPackSlots; ++j)
          for (int lane = 0; lane < 64; ++lane) {
            const int sub = lane >> hl, vec = lane & ((1 << hl) - 1);
            const bool vlive = vec < nvec;
            const int64_t rel = (int64_t{j} << (6 - hl)) + sub, row = row0 + rel;
            const uint32_t xo = packed_offset(rel, span, vec, vlive, xs);
            const uint32_t yo = packed_offset(rel, span, vec, vlive, ys);
            if (vlive && row < T) {
              CHECK(xo == static_cast<uint32_t>(rel * xs + 16 * vec) && xo + 16 <= xbytes,
                    "packed segment %d row %lld vector %d: input offset %u of %u", i, (long long)row, vec, xo, xbytes);
              CHECK(v.mode == MODE_STATS ||
                        (yo == static_cast<uint32_t>(rel * ys + 16 * vec) && yo + 16 <= ybytes),
                    "packed segment %d row %lld vector %d: output offset %u of %u", i, (long long)row, vec, yo,
                    ybytes);
              ++held[static_cast<size_t>(row * nvec + vec)];
            } else {
              CHECK(xo == kOutsideOffset && yo == kOutsideOffset, "packed segment %d: empty lane not dropped", i);
            }
          }
      }
    for (size_t k = 0; k < held.size(); ++k)
      CHECK(held[k] == 1, "packed segment %d: row %lld vector %lld held %d times", i,
            (long long)(k / static_cast<size_t>(nvec)), (long long)(k % static_cast<size_t>(nvec)), held[k]);
  }
}

static void check_seg(const qkn::Seg& s, int nw, int vpl, int64_t nvec, int K, bool masked, const char* what) {
  const int wl = s.wpr_log2, m = s.sub_lanes_log2;
  CHECK(m >= 0 && m <= 6 + wl, "%s sub_lanes_log2 %d wpr_log2 %d", what, m, wl);
  CHECK(!masked || m == 6 + wl, "%s masked layout with sub-teams of 2^%d lanes", what, m);
  CHECK(s.nslot >= 1 && s.nslot <= vpl, "%s nslot %d vpl %d", what, s.nslot, vpl);
  CHECK(s.rows_per_wg * (1 << wl) == nw, "%s rows_per_wg", what);
  CHECK(static_cast<int64_t>(s.row_bytes) == nvec * 16, "%s row_bytes", what);
  const int lanes = 64 << wl;
  const int nsub = 1 << (6 + wl - m);
  const int64_t sv = s.slice_vec;
  std::vector<int> count(nvec, 0);
  // slice held by (sub-team, slot); -2 = unset, -1 = empty for this sub-team
  std::vector<std::vector<int>> slot_slice(nsub, std::vector<int>(s.nslot, -2));
  for (int tl = 0; tl < lanes; ++tl) {
    const int sub = tl >> m;
    for (int j = 0; j < s.nslot; ++j) {
      const int v = qkn::slot_vector(s.slot_lim[j], s.slot_base[j], tl, wl, m, s.slice_vec, s.lay_k);
      // the kernels' offset: the same vector, or an access the range check drops
      const int stl = tl & ((1 << m) - 1);
      const uint32_t off = qkn::slot_offset(s.slot_base[j], sub * s.slice_vec + stl, stl, (s.flush_mask >> j) & 1u,
                                            s.tail_lanes, s.dense);
      if (v >= 0)
        CHECK(off == static_cast<uint32_t>(v) * 16u, "%s slot %d lane %d offset %u for vector %d", what, j, tl, off, v);
      else
        CHECK(off >= s.row_bytes, "%s slot %d lane %d empty but offset %u < row bytes %u", what, j, tl, off,
              s.row_bytes);
      if (v < 0) continue;
      CHECK(v < nvec, "%s vector %d >= %lld", what, v, (long long)nvec);
      if (v >= nvec) continue;
      ++count[v];
      const int sl = static_cast<int>(v / sv);
      if (!masked) {
        int& rec = slot_slice[sub][j];
        CHECK(rec == -2 || rec == sl, "%s slot %d mixes slices %d and %d", what, j, rec, sl);
        rec = sl;
      }
    }
  }
  for (int64_t v = 0; v < nvec; ++v) CHECK(count[v] == 1, "%s vector %lld held %d times", what, (long long)v, count[v]);
  for (int j = s.nslot; j < qkn::kMaxSlots; ++j) CHECK(s.slot_lim[j] == 0, "%s unused slot %d not empty", what, j);
  if (!masked) {
    for (int u = 0; u < nsub; ++u) {
      int flushes = 0;
      for (int j = 0; j < s.nslot; ++j) {
        const bool flush = (s.flush_mask >> j) & 1u;
        const int sl = slot_slice[u][j];
        const int next = j + 1 < s.nslot ? slot_slice[u][j + 1] : -3;
        const int expect = u + flushes * nsub;  // the slice the kernel's partial counter stands at
        if (sl >= 0) {
          CHECK(sl == expect, "%s sub %d slot %d holds slice %d, counter at %d", what, u, j, sl, expect);
          CHECK(flush == (next != sl), "%s sub %d slot %d flush bit %d", what, u, j, (int)flush);
        }
        if (flush) ++flushes;
      }
      CHECK(flushes <= 64, "%s too many partials", what);
    }
  }
  if (s.lds_gamma) {
    const int v = body_slots(vpl, s.nslot);
    CHECK(nvec <= static_cast<int64_t>((v + 1) / 2) * nw * 64, "%s staged gamma exceeds the copy loop", what);
    CHECK(s.rows_per_wg > 1, "%s staged gamma with one row per workgroup", what);
  }
}

static void check_heads(const qkn::Seg& s, int hv, const char* what);

static void run_forward(int64_t T, int64_t hq, int64_t hk, int K, int forced_wpr, int dtype) {
  qknorm_ctx ctx{0, 256, qknorm_options{forced_wpr, 0, 0}};
  const int64_t ve = vec_elems(dtype);
  SegIn in[2] = {{hq / ve, K}, {hk / ve, K}};
  const int nseg = hk > 0 ? 2 : 1;
  Plan plans[2];
  int nw = 4;
  const int st = plan_launch(&ctx, dtype, in, nseg, T, plans, &nw);
  if (st != QKNORM_OK) {
    // only a pinned team that cannot hold the row may be refused
    CHECK(forced_wpr != 0, "auto plan refused T=%lld hq=%lld hk=%lld K=%d", (long long)T, (long long)hq,
          (long long)hk, K);
    return;
  }
  bool narrow = false;
  for (int i = 0; i < nseg; ++i) narrow = narrow || narrow_plan(plans[i]);
  int slots = 0;
  qkn::Seg seg[2] = {};
  bool masked[2] = {false, false};
  char what[160];
  std::snprintf(what, sizeof what, "T=%lld hq=%lld hk=%lld K=%d wpr=%d dt=%d", (long long)T, (long long)hq,
                (long long)hk, K, forced_wpr, dtype);
  for (int i = 0; i < nseg; ++i) {
    masked[i] = plans[i].masked;
    fill_layout(&seg[i], plans[i], nw, in[i].nvec, K, T);
    seg[i].x_stride = seg[i].y_stride = i == 0 ? hq : hk;  // contiguous rows
    share_gamma(&seg[i], dtype);
    slots = seg[i].nslot > slots ? seg[i].nslot : slots;
    // the kernels for narrow slices tell the layouts apart by the masked
    // flag and the sub-team width; the others only ever see sub-teams of
    // whole wavefronts
    const int sl = seg[i].sub_lanes_log2;
    CHECK(seg[i].masked == (masked[i] ? 1 : 0), "%s seg %d masked flag", what, i);
    CHECK(!masked[i] || sl == 6 + seg[i].wpr_log2, "%s seg %d masked with sub-teams 2^%d", what, i, sl);
    CHECK(narrow || (!masked[i] && sl >= 6), "%s wavefront kernel, seg %d: sub-teams 2^%d", what, i, sl);
  }
  const int vpl = qkn::compiled_vpl(slots, nw, dtype);
  CHECK(vpl > 0, "%s no compiled variant for %d slots", what, slots);
  if (vpl == 0) return;
  // up to 8 slots in 4-wavefront workgroups, the widest segment runs a body
  // of exactly its slot count (no empty slots)
  CHECK(nw != 4 || slots > 8 || vpl == slots, "%s %d slots run by the %d-slot body", what, slots, vpl);
  // several rows per wavefront: every row covered once, no spare workgroups;
  // paired rows (forward only) as the enqueue step decides them
  for (int mode : {qkn::MODE_STATS, qkn::MODE_FWD}) {
    qkn::Variant v{dtype, mode, vpl, nw, narrow, true, false};
    qkn::Args a{};
    a.T = T;
    for (int i = 0; i < nseg; ++i) a.seg[i] = seg[i];
    pair_rows(&ctx, &v, &a, nseg);
    CHECK(!v.pair || mode == qkn::MODE_FWD, "%s paired rows in mode %d", what, mode);
    CHECK(!v.pair || (forced_wpr == 0 && pair_band(T, 256, dtype) && qkn::compiled(v)),
          "%s paired launch T=%lld", what, (long long)T);
    if (!v.pair) pack_rows(&ctx, &v, &a, nseg);
    CHECK(!v.pack || (forced_wpr == 0 && K == 1 && T * nseg >= 16 * 1024 && qkn::compiled(v)),
          "%s packed launch T=%lld", what, (long long)T);
    if (v.pack) qkn::check_pack_launch(v, a, dim3(a.seg[0].nwg > a.seg[nseg - 1].nwg ? a.seg[0].nwg
                                                                                      : a.seg[nseg - 1].nwg,
                                                  nseg),
                                       0);
    if (!v.pair && !v.pack) rows_per_wave(&ctx, &v, &a, nseg);
    for (int i = 0; i < nseg; ++i) {
      const int64_t per_wg = int64_t{a.seg[i].rows_per_wg} * a.seg[i].rpw << (v.pack ? 6 - a.seg[i].pack_log2 : 0);
      CHECK(a.seg[i].rpw == v.rpw && (v.rpw == 1 || v.rpw == 2 || v.rpw == 4), "%s rpw %d", what, v.rpw);
      CHECK(int64_t{a.seg[i].nwg} * per_wg >= T && int64_t{a.seg[i].nwg - 1} * per_wg < T, "%s nwg %d", what,
            a.seg[i].nwg);
      CHECK(v.rpw == 1 || (a.seg[i].wpr_log2 == 0 && !narrow && nw == 4 &&
                           ((mode == qkn::MODE_STATS && a.seg[i].nslot * v.rpw <= 4) ||
                            (a.seg[i].nslot == 1 && v.rpw == 4))),
            "%s mode %d rpw %d with wpr_log2 %d, %d slots", what, mode, v.rpw, a.seg[i].wpr_log2, a.seg[i].nslot);
    }
  }
  for (int i = 0; i < nseg; ++i) {
    check_seg(seg[i], nw, vpl, in[i].nvec, K, masked[i], what);
    ++g_layouts[masked[i] ? 2 : seg[i].sub_lanes_log2 < 6 ? 1 : 0];
    g_dense += seg[i].dense;
  }
}

// Headwise: each aligned group of hv lanes of one wavefront holds, in each
// slot, either nothing or the hv vectors of one head in order, so lane l
// holds the head's vector l mod hv (the kernel's head sum and weights).
static void check_heads(const qkn::Seg& s, int hv, const char* what) {
  const int wl = s.wpr_log2, m = s.sub_lanes_log2, lanes = 64 << wl;
  for (int j = 0; j < s.nslot; ++j)
    for (int g0 = 0; g0 < lanes; g0 += hv) {
      const int v0 = qkn::slot_vector(s.slot_lim[j], s.slot_base[j], g0, wl, m, s.slice_vec, 1);
      for (int i = 0; i < hv; ++i) {
        const int v = qkn::slot_vector(s.slot_lim[j], s.slot_base[j], g0 + i, wl, m, s.slice_vec, 1);
        if (v0 < 0) {
          CHECK(v < 0, "%s slot %d group %d: lane %d live in an empty group", what, j, g0, i);
          continue;
        }
        CHECK(v == v0 + i && v0 % hv == 0, "%s slot %d group %d: lane %d holds %d (group starts at %d)", what,
              j, g0, i, v, v0);
        CHECK(v < 0 || v % hv == ((g0 + i) & 63) % hv, "%s weights of lane %d", what, g0 + i);
      }
    }
}

static void run_headwise(int64_t T, int64_t hq, int64_t hk, int64_t D, int forced_wpr, int dtype) {
  qknorm_ctx ctx{0, 256, qknorm_options{forced_wpr, 0, 0}};
  const int64_t ve = vec_elems(dtype);
  const int hv = head_vectors(D, dtype);
  SegIn in[2] = {{hq / ve, 1}, {hk / ve, 1}};
  const int nseg = hk > 0 ? 2 : 1;
  Plan plans[2];
  int nw = 4;
  char what[160];
  std::snprintf(what, sizeof what, "headwise T=%lld hq=%lld hk=%lld D=%lld wpr=%d dt=%d", (long long)T,
                (long long)hq, (long long)hk, (long long)D, forced_wpr, dtype);
  CHECK(hv > 0, "%s invalid head", what);
  if (plan_launch(&ctx, dtype, in, nseg, T, plans, &nw) != QKNORM_OK) {
    CHECK(forced_wpr != 0, "%s auto plan refused", what);
    return;
  }
  qkn::Seg seg[2];
  int slots = 0;
  for (int i = 0; i < nseg; ++i) {
    CHECK(!narrow_plan(plans[i]), "%s narrow plan", what);
    fill_layout(&seg[i], plans[i], nw, in[i].nvec, 1, T);
    slots = seg[i].nslot > slots ? seg[i].nslot : slots;
  }
  const int vpl = qkn::compiled_vpl(slots, nw, dtype);
  CHECK(vpl > 0, "%s no compiled variant for %d slots", what, slots);
  if (vpl == 0) return;
  for (int i = 0; i < nseg; ++i) {
    check_seg(seg[i], nw, vpl, in[i].nvec, 1, false, what);
    check_heads(seg[i], hv, what);
  }
}

// The plan of one launch (automatic schedule, 256 compute units) as one
// line: what the tests pin for the benchmark workloads, so that a change of
// the planner that moves one of them shows up.
static void print_plan(const char* name, int dtype, int64_t T, int64_t hq, int64_t hk, int K) {
  qknorm_ctx ctx{0, 256, qknorm_options{0, 0, 0}};
  const int64_t ve = vec_elems(dtype);
  SegIn in[2] = {{hq / ve, K}, {hk / ve, K}};
  Plan plans[2];
  int nw = 4;
  if (plan_launch(&ctx, dtype, in, 2, T, plans, &nw) != QKNORM_OK) {
    std::printf("plan %s: refused\n", name);
    return;
  }
  qkn::Args a{};
  a.T = T;
  bool narrow = false;
  int slots = 0;
  for (int i = 0; i < 2; ++i) {
    narrow = narrow || narrow_plan(plans[i]);
    fill_layout(&a.seg[i], plans[i], nw, in[i].nvec, K, T);
    share_gamma(&a.seg[i], dtype);
    slots = a.seg[i].nslot > slots ? a.seg[i].nslot : slots;
  }
  qkn::Variant v{dtype, qkn::MODE_FWD, qkn::compiled_vpl(slots, nw, dtype), nw, narrow, true, false};
  pair_rows(&ctx, &v, &a, 2);
  if (!v.pair) pack_rows(&ctx, &v, &a, 2);
  if (!v.pair && !v.pack) rows_per_wave(&ctx, &v, &a, 2);
  std::printf("plan %s: nw=%d body=%d narrow=%d rows_per_wave=%d paired=%d early=%d", name, nw, v.vpl,
              narrow ? 1 : 0, v.rpw, v.pair ? v.vpl_b : 0, v.early ? 1 : 0);
  for (int i = 0; i < 2; ++i)
    std::printf(" | %s team=%d sub_lanes=%d slots=%d masked=%d", i ? "k" : "q", 1 << plans[i].wpr_log2,
                1 << plans[i].sub_lanes_log2, plans[i].slots, plans[i].masked ? 1 : 0);
  std::printf("\n");
}

// Every public entry point, over shapes, slice counts and schedule options,
// through the library's own validation and planning: records each variant a
// launch asks for. Fake device addresses, far apart, are never dereferenced.
static long sweep_entry_points() {
  long calls = 0;
  const uintptr_t B = 0x100000000000ull, G = 0x1000000000ull;  // tensors 64 GiB apart
  auto P = [&](int i) { return reinterpret_cast<void*>(B + i * G); };
  std::vector<qknorm_options> opts;
  for (int w : {0, 1, 2, 4, 8, 16})
    for (int cap : {0, 3})
      for (int cached : {0, 1}) opts.push_back(qknorm_options{w, cap, cached});
  // every slot count of one-wavefront rows for each element type (256 fp32,
  // 512 bf16 or 1024 fp8 columns per slot), and wider rows for the teams
  std::vector<int64_t> widths = {8, 64, 200, 1000, 1280, 12288, 24576, 49152, 65536};
  for (int64_t slots = 1; slots <= 32; ++slots)
    for (int64_t per : {256, 512, 1024}) widths.push_back(slots * per);
  const int64_t rows[] = {1, 64, 256, 2048, 3001, 16384, 100000};
  const int ks[] = {1, 2, 4, 8, 64};
  for (const qknorm_options& o : opts) {
    qknorm_ctx ctx{0, 256, o};
    for (int dtype : {QKNORM_BF16, QKNORM_F32, QKNORM_FP8_E4M3})
      for (int64_t hq : widths)
        // key rows as wide as the query rows, or narrower by the grouped-query
        // ratios (the paired kernels pair a wide row with each narrower body)
        for (int64_t hk : {hq, hq / 2, hq / 4, hq / 5, hq / 8, hq / 12, hq / 16}) {
          const int64_t ve = vec_elems(dtype);
          if (hq > qknorm_max_width(dtype) || hk < ve || hk % ve) continue;
          for (int64_t T : rows) {
            qknorm_rows q{P(0), P(1), hq, hq, hq}, k{P(2), P(3), hk, hk, hk};
            for (int K : ks) {
              calls += 3;
              qknorm_forward(&ctx, dtype, T, &q, &k, P(4), P(5), 1e-6f, K, nullptr);
              qknorm_forward(&ctx, dtype, T, &q, nullptr, P(4), nullptr, 1e-6f, K, nullptr);
              qknorm_inv_rms(&ctx, dtype, T, &q, &k, 1e-6f, K, static_cast<float*>(P(6)),
                             static_cast<float*>(P(7)), nullptr);
              if (hq % K || hk % K || (hq / K) % ve || (hk / K) % ve) continue;
              qknorm_rows qs{P(0), P(1), hq / K, hq, hq}, ks_{P(2), P(3), hk / K, hk, hk};
              calls += 4;
              qknorm_partial_stats_qk(&ctx, dtype, T, &qs, &ks_, 0, K, static_cast<float*>(P(6)),
                                      static_cast<float*>(P(7)), nullptr);
              qknorm_partial_stats(&ctx, dtype, T, P(0), hq, hq / K, 0, K, static_cast<float*>(P(6)), nullptr);
              qknorm_apply_stats_qk(&ctx, dtype, T, &qs, &ks_, P(4), P(5), static_cast<const float*>(P(6)),
                                    static_cast<const float*>(P(7)), K, hq, hk, 1e-6f, nullptr);
              qknorm_apply_stats(&ctx, dtype, T, &qs, P(4), static_cast<const float*>(P(6)), K, hq, 1e-6f,
                                 nullptr);
            }
            for (int64_t D = 1; D <= hk; D *= 2) {
              ++calls;
              qknorm_forward_headwise(&ctx, dtype, T, &q, &k, P(4), P(5), D, 1e-6f, nullptr);
            }
          }
        }
  }
  return calls;
}

int main() {
  int cases = 0;
  const int64_t widths[] = {8, 24, 64, 96, 200, 256, 512, 1000, 1024, 1032, 1280, 1536, 2048,
                            4096, 5120, 8192, 12288, 16384, 32768, 65536};
  const int64_t rows[] = {1, 3, 64, 256, 2048, 16384, 20001};
  const int ks[] = {1, 2, 3, 4, 5, 8, 10, 16, 24, 32, 40, 48, 64};
  const int wprs[] = {0, 1, 2, 4, 8, 16};
  for (int dtype : {QKNORM_BF16, QKNORM_F32, QKNORM_FP8_E4M3})
    for (int64_t hq : widths)
      for (int K : ks) {
        const int64_t ve = vec_elems(dtype);
        if (hq > qknorm_max_width(dtype) || hq % K || (hq / K) % ve) continue;
        for (int64_t T : rows)
          for (int w : wprs) {
            run_forward(T, hq, 0, K, w, dtype);
            ++cases;
            // a key segment of a quarter / the same width, when it slices evenly
            for (int64_t hk : {hq / 4, hq}) {
              if (hk < ve || hk % K || (hk / K) % ve) continue;
              run_forward(T, hq, hk, K, w, dtype);
              ++cases;
            }
          }
      }
  for (int dtype : {QKNORM_BF16, QKNORM_F32, QKNORM_FP8_E4M3})
    for (int64_t hq : widths)
      for (int64_t D = 1; D <= hq; D *= 2) {
        if (hq > qknorm_max_width(dtype) || head_vectors(D, dtype) == 0 || hq % D) continue;
        for (int64_t T : rows)
          for (int w : wprs) {
            run_headwise(T, hq, 0, D, w, dtype);
            run_headwise(T, hq, (hq / 4) % D == 0 && hq >= 4 * D ? hq / 4 : D, D, w, dtype);
            cases += 2;
          }
      }
  print_plan("c1 K=1", QKNORM_F32, 4, 256, 256, 1);
  print_plan("c1 K=4", QKNORM_F32, 4, 256, 256, 4);
  print_plan("c2 K=1", QKNORM_BF16, 64, 4096, 4096, 1);
  print_plan("c3 K=4", QKNORM_BF16, 256, 5120, 5120, 4);
  print_plan("c3 K=1", QKNORM_BF16, 256, 5120, 5120, 1);
  print_plan("c4 K=1", QKNORM_BF16, 2048, 5120, 1024, 1);
  print_plan("c5 K=8", QKNORM_BF16, 16384, 4096, 4096, 8);
  print_plan("c5 K=1", QKNORM_BF16, 16384, 4096, 4096, 1);
  print_plan("c4f8 K=1", QKNORM_FP8_E4M3, 2048, 5120, 1024, 1);
  print_plan("c5f8 K=8", QKNORM_FP8_E4M3, 16384, 4096, 4096, 8);
  print_plan("c5f8 K=1", QKNORM_FP8_E4M3, 16384, 4096, 4096, 1);
  std::printf("segments: %ld whole-wavefront sub-teams, %ld narrower sub-teams, %ld masked; %ld dense\n",
              g_layouts[0], g_layouts[1], g_layouts[2], g_dense);
  // the kernels a call can ask for, and the ones compiled for none
  const long calls = sweep_entry_points();
  CHECK(qkn::g_uncompiled == 0, "%ld launches asked for a variant without a kernel", qkn::g_uncompiled);
  long compiled_n = 0;
  std::vector<qkn::VariantKey> unused;
  for (int dtype : {QKNORM_F32, QKNORM_BF16, QKNORM_FP8_E4M3})
    for (int mode = 0; mode < 4; ++mode)
      for (int nw : {4, 16})
        for (int vpl = 1; vpl <= qkn::kMaxSlots; ++vpl)
          for (int narrow = 0; narrow < 2; ++narrow)
            for (int nt = 0; nt < 2; ++nt)
              for (int pipe = 0; pipe < 2; ++pipe)
                for (int rpw : {1, 2, 4})
                  for (int pb = 0; pb <= qkn::kMaxSlots; ++pb)
                    for (int pk = 0; pk < 2; ++pk)
                      for (int ea = 0; ea < 2; ++ea) {
                        if (!qkn::compiled(dtype, mode, vpl, nw, narrow, nt, pipe, rpw, pb, pk != 0, ea != 0))
                          continue;
                        ++compiled_n;
                        const qkn::VariantKey k{dtype, mode, vpl, nw, narrow != 0, nt != 0, pipe != 0, rpw, pb,
                                                pk != 0, ea != 0};
                        if (!qkn::g_reached.count(k)) unused.push_back(k);
                      }
  std::printf("entry points: %ld calls, %ld launches, %zu variants reached, %ld compiled, %zu compiled and "
              "never reached\n", calls, qkn::g_launches, qkn::g_reached.size(), compiled_n, unused.size());
  std::printf("paired launches %ld; packed launches %ld, %ld segments traced lane by lane\n", qkn::g_paired,
              qkn::g_packed, qkn::g_packed_covered);
  CHECK(unused.empty(), "%zu compiled variants that no call reaches", unused.size());
  for (const auto& k : unused)
    std::printf("  unreached: dtype=%d mode=%d vpl=%d nw=%d narrow=%d nt=%d pipe=%d rpw=%d paired=%d packed=%d "
                "early=%d\n",
                std::get<0>(k), std::get<1>(k), std::get<2>(k), std::get<3>(k), (int)std::get<4>(k),
                (int)std::get<5>(k), (int)std::get<6>(k), std::get<7>(k), std::get<8>(k), (int)std::get<9>(k),
                (int)std::get<10>(k));
  std::printf("%d cases, %d failures\n", cases, failures);
  return failures ? 1 : 0;
}
