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
//    per head).
#include "qknorm_api.cpp"

#include <cstdio>
#include <vector>

namespace qkn {
static Variant g_v;
static Args g_a;
static dim3 g_grid;
static unsigned g_lds;
hipError_t launch(const Variant& v, const Args& a, dim3 grid, unsigned lds_bytes, hipStream_t) {
  g_v = v;
  g_a = a;
  g_grid = grid;
  g_lds = lds_bytes;
  return hipSuccess;
}
}  // namespace qkn

static int failures = 0;
static long g_layouts[3];  // segments laid out with whole-wavefront sub-teams, narrower ones, masked
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
  qkn::Seg seg[2];
  bool masked[2] = {false, false};
  char what[160];
  std::snprintf(what, sizeof what, "T=%lld hq=%lld hk=%lld K=%d wpr=%d dt=%d", (long long)T, (long long)hq,
                (long long)hk, K, forced_wpr, dtype);
  for (int i = 0; i < nseg; ++i) {
    masked[i] = plans[i].masked;
    fill_layout(&seg[i], plans[i], nw, in[i].nvec, K, T);
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
  // several rows per wavefront: every row covered once, no spare workgroups
  for (int mode : {qkn::MODE_STATS, qkn::MODE_FWD}) {
    qkn::Variant v{dtype, mode, vpl, nw, narrow, true, false};
    qkn::Args a{};
    a.T = T;
    for (int i = 0; i < nseg; ++i) a.seg[i] = seg[i];
    rows_per_wave(&ctx, &v, &a, nseg);
    for (int i = 0; i < nseg; ++i) {
      const int64_t per_wg = int64_t{a.seg[i].rows_per_wg} * a.seg[i].rpw;
      CHECK(a.seg[i].rpw == v.rpw && (v.rpw == 1 || v.rpw == 2 || v.rpw == 4), "%s rpw %d", what, v.rpw);
      CHECK(int64_t{a.seg[i].nwg} * per_wg >= T && int64_t{a.seg[i].nwg - 1} * per_wg < T, "%s nwg %d", what,
            a.seg[i].nwg);
      CHECK(v.rpw == 1 || (a.seg[i].wpr_log2 == 0 && !narrow && nw == 4 &&
                           (mode == qkn::MODE_STATS ? a.seg[i].nslot * v.rpw <= 4
                                                    : dtype == QKNORM_FP8_E4M3 && v.rpw == 2 && a.seg[i].nslot <= 8)),
            "%s mode %d rpw %d with wpr_log2 %d, %d slots", what, mode, v.rpw, a.seg[i].wpr_log2, a.seg[i].nslot);
    }
  }
  for (int i = 0; i < nseg; ++i) {
    check_seg(seg[i], nw, vpl, in[i].nvec, K, masked[i], what);
    ++g_layouts[masked[i] ? 2 : seg[i].sub_lanes_log2 < 6 ? 1 : 0];
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
  rows_per_wave(&ctx, &v, &a, 2);
  std::printf("plan %s: nw=%d body=%d narrow=%d rows_per_wave=%d", name, nw, v.vpl, narrow ? 1 : 0, v.rpw);
  for (int i = 0; i < 2; ++i)
    std::printf(" | %s team=%d sub_lanes=%d slots=%d masked=%d", i ? "k" : "q", 1 << plans[i].wpr_log2,
                1 << plans[i].sub_lanes_log2, plans[i].slots, plans[i].masked ? 1 : 0);
  std::printf("\n");
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
  std::printf("segments: %ld whole-wavefront sub-teams, %ld narrower sub-teams, %ld masked\n", g_layouts[0],
              g_layouts[1], g_layouts[2]);
  std::printf("%d cases, %d failures\n", cases, failures);
  return failures ? 1 : 0;
}
