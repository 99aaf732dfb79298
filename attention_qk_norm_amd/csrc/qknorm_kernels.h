// qknorm_kernels.h -- gfx950 kernels for layerwise QK-Norm (device templates).
//
// Each element type is instantiated in a translation unit of its own
// (qknorm_kernels_f32.hip, _bf16.hip, _fp8.hip), so the three compile in
// parallel.
//
// Per row (SwiftQK technical review, Eq. 1; the K-slice statistic of section
// 4b, Eqs. 3-6):
//   1. the team loads its row with 16-byte vector loads into VGPRs (the whole
//      row stays resident, so HBM is read once);
//   2. per slice, each lane accumulates its slots' squares in fp32; a
//      wavefront reduction (DPP within rows of 16 lanes, then 4 readlanes)
//      gives the slice's partial, or, for slices narrower than a wavefront,
//      a sum over the slice's aligned group of lanes; teams of several
//      wavefronts add their partials through LDS;
//   3. the partials are summed in ascending slice order (review Eq. 5), then
//      r = 1 / sqrt(S / H + eps) with H the full width (Eq. 6);
//   4. y = (x * gamma) * r in fp32 (for bf16 and e4m3 rows x * gamma is
//      exact, so the fp32 result is rounded once, at the product with r),
//      rounded to the output type, stored with 16-byte vector stores; y may
//      be x.
// The split path reuses the same body: MODE_STATS stops after step 2 and
// writes one fp32 per row (Algorithm 1, Phase A), or after step 3 and writes
// the row's inverse RMS for a consumer that scales the row itself;
// MODE_APPLY skips step 2 and combines precomputed partials instead (Phase
// B's scalar sum, then Phase C). MODE_HEAD is the headwise form.
//
// Element types are traits structs (F32, BF16, FP8): vector width, squares,
// scaling and the weights' type and layout. FP8 rows (OCP E4M3, the review's
// Fig. 2(b) FP8 runs) take bf16 weights.
//
// No matrix cores: the work is a reduction and an elementwise scale, bound by
// HBM bandwidth.
#pragma once

#include "qknorm_launch.h"

#include "qknorm.h"

namespace qkn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Row data move through raw buffer resources: base = the row (or gamma),
// num_records = its byte length. Lanes given an offset past the end read
// zeros and their stores are dropped by the hardware range check, so ragged
// slots, partial teams and rows past T need no branches.
constexpr int kRsrcConfig = 0x00020000;  // raw, untyped, 32-bit data format
constexpr uint32_t kOutside = kOutsideOffset;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcConfig);
}

// aux = 2 sets the non-temporal (streaming) cache policy bit.
template <bool NT>
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT ? 2 : 0);
}

template <bool NT>
__device__ __forceinline__ void store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, NT ? 2 : 0);
}

// Weights stored in the rows' own type: one 16-byte weight vector per row
// vector, at the same byte offset.
struct SameTypeGamma {
  using G = u32x4;
  static constexpr uint32_t kGammaScale = 1;  // weight bytes per row byte
  static __device__ __forceinline__ G load_gamma(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return load16<false>(r, off);
  }
  static __device__ __forceinline__ G gamma_lds(const u32x4* lds, uint32_t v) { return lds[v]; }
};

// binary32 rows: 4 elements per 16-byte vector.
struct F32 : SameTypeGamma {
  static constexpr int kDtype = QKNORM_F32;
  static constexpr int kBytes = 4;
  static __device__ __forceinline__ float sumsq(u32x4 d, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = __uint_as_float(d[i]);
      acc = __builtin_fmaf(v, v, acc);
    }
    return acc;
  }
  // fp32 and bf16 results cannot leave their type's range here, so SAT and
  // the running maximum (for types that saturate) are unused
  static constexpr bool kSaturates = false;
  template <bool SAT>
  static __device__ __forceinline__ u32x4 encode(u32x4 d, u32x4 g, float r, float&) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = __float_as_uint(__uint_as_float(d[i]) * __uint_as_float(g[i]) * r);
    return o;
  }
};

// The element is handed over by value on purpose: this clang lowers
// __builtin_bit_cast applied directly to an ext_vector element (d[i], d.y)
// as a read of element 0, silently.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// bfloat16 rows: 8 elements per 16-byte vector, two per dword. The square
// sums use the bf16 dot-product instruction (fp32 result and accumulator);
// the scaling widens to fp32 and rounds back to nearest-even in one packed
// conversion.
struct BF16 : SameTypeGamma {
  static constexpr int kDtype = QKNORM_BF16;
  static constexpr int kBytes = 2;
  static __device__ __forceinline__ float sumsq(u32x4 d, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2 p = as_bf16x2(d[i]);
      acc = __builtin_amdgcn_fdot2_f32_bf16(p, p, acc, false);
    }
    return acc;
  }
  static constexpr bool kSaturates = false;
  template <bool SAT>
  static __device__ __forceinline__ u32x4 encode(u32x4 d, u32x4 g, float r, float&) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float xl = __uint_as_float(d[i] << 16);
      const float xh = __uint_as_float(d[i] & 0xffff0000u);
      const float gl = __uint_as_float(g[i] << 16);
      const float gh = __uint_as_float(g[i] & 0xffff0000u);
      const f32x2 yv = {xl * gl * r, xh * gh * r};
      o[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(yv, bf16x2));
    }
    return o;
  }
};

// OCP FP8 E4M3 rows (the e4m3 encoding without infinities that gfx950
// converts natively; largest finite value 448): 16 elements per 16-byte
// vector. The weights stay bfloat16, so one row vector takes two weight
// vectors, at twice the row vector's byte offset. Squares accumulate in fp32
// (review section 5); y = (x * gamma) * r in fp32 is rounded to nearest-even
// e4m3, saturating at +-448 (the conversion instruction alone would give NaN
// past 464), while NaN stays NaN.
__device__ __forceinline__ f32x2 fp8_pair(uint32_t w, bool high) {
  return high ? __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true)
              : __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
}

__device__ __forceinline__ float sat_e4m3(float v) {
  return __builtin_fabsf(v) > 448.0f ? __builtin_copysignf(448.0f, v) : v;
}

struct FP8 {
  static constexpr int kDtype = QKNORM_FP8_E4M3;
  static constexpr int kBytes = 1;
  struct G {
    u32x4 lo, hi;  // weights of elements 0-7 and 8-15 of the row vector
  };
  static constexpr uint32_t kGammaScale = 2;
  static __device__ __forceinline__ G load_gamma(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const uint32_t o = off == kOutside ? kOutside : 2u * off;
    return G{load16<false>(r, o), load16<false>(r, o == kOutside ? kOutside : o + 16u)};
  }
  static __device__ __forceinline__ G gamma_lds(const u32x4* lds, uint32_t v) {
    return G{lds[2u * v], lds[2u * v + 1u]};
  }
  // Squares: each pair widens exactly to bf16 (the scaled conversion with
  // scale 1; e4m3 values, subnormals included, are bf16 values) and one
  // bf16 dot product adds both squares to the fp32 accumulator: two
  // instructions per pair instead of a widening to fp32 and two FMAs.
  static __device__ __forceinline__ float sumsq(u32x4 d, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[i], 1.0f, false);
      const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[i], 1.0f, true);
      acc = __builtin_amdgcn_fdot2_f32_bf16(a, a, acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(b, b, acc, false);
    }
    return acc;
  }
  // y = (x gamma) r for the vector's 16 elements, rounded to nearest-even
  // e4m3. SAT: results past 448 (infinities included) become +-448 first.
  // Otherwise `peak` takes the largest |y| (three-operand maxima; a NaN
  // result leaves it unchanged and is encoded as NaN).
  template <bool SAT>
  static __device__ __forceinline__ u32x4 encode(u32x4 d, const G& g, float r, float& peak) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // row dword i holds elements 4i..4i+3; their weights are bf16 words
      // 4i..4i+3, i.e. weight dwords 2i and 2i+1
      const uint32_t g0 = i < 2 ? g.lo[2 * i] : g.hi[2 * i - 4];
      const uint32_t g1 = i < 2 ? g.lo[2 * i + 1] : g.hi[2 * i - 3];
      const uint32_t w8 = d[i];
      const f32x2 a = fp8_pair(w8, false);
      const f32x2 b = fp8_pair(w8, true);
      float y0 = a.x * __uint_as_float(g0 << 16) * r;
      float y1 = a.y * __uint_as_float(g0 & 0xffff0000u) * r;
      float y2 = b.x * __uint_as_float(g1 << 16) * r;
      float y3 = b.y * __uint_as_float(g1 & 0xffff0000u) * r;
      if constexpr (SAT) {
        y0 = sat_e4m3(y0);
        y1 = sat_e4m3(y1);
        y2 = sat_e4m3(y2);
        y3 = sat_e4m3(y3);
      } else {
        peak = __builtin_fmaxf(__builtin_fmaxf(peak, __builtin_fabsf(y0)), __builtin_fabsf(y1));
        peak = __builtin_fmaxf(__builtin_fmaxf(peak, __builtin_fabsf(y2)), __builtin_fabsf(y3));
      }
      // both halves are written, so the word the conversion starts from is
      // immaterial: the input word saves an initialisation
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(y0, y1, static_cast<int>(w8), false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(y2, y3, w, true);
      o[i] = static_cast<uint32_t>(w);
    }
    return o;
  }
  // x gamma for the vector's 16 elements. An e4m3 significand has 4 bits
  // and a bf16 one 8, so each product is exact in fp32 and encode's
  // (x gamma) r rounds once, at the multiplication by r. `peak` takes the
  // largest |x gamma| (NaN products leave it unchanged): rounding is
  // monotonic, so the largest |y| is peak * r rounded, and whether any
  // result passes 448 is known from one product.
  static constexpr int kElems = 16;
  static __device__ __forceinline__ void products(u32x4 d, const G& g, float (&t)[kElems], float& peak) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t g0 = i < 2 ? g.lo[2 * i] : g.hi[2 * i - 4];
      const uint32_t g1 = i < 2 ? g.lo[2 * i + 1] : g.hi[2 * i - 3];
      const f32x2 a = fp8_pair(d[i], false);
      const f32x2 b = fp8_pair(d[i], true);
      t[4 * i] = a.x * __uint_as_float(g0 << 16);
      t[4 * i + 1] = a.y * __uint_as_float(g0 & 0xffff0000u);
      t[4 * i + 2] = b.x * __uint_as_float(g1 << 16);
      t[4 * i + 3] = b.y * __uint_as_float(g1 & 0xffff0000u);
      peak = __builtin_fmaxf(__builtin_fmaxf(peak, __builtin_fabsf(t[4 * i])), __builtin_fabsf(t[4 * i + 1]));
      peak = __builtin_fmaxf(__builtin_fmaxf(peak, __builtin_fabsf(t[4 * i + 2])), __builtin_fabsf(t[4 * i + 3]));
    }
  }
  // encode<SAT>'s result from the products: the same bits
  template <bool SAT>
  static __device__ __forceinline__ u32x4 encode_products(const float (&t)[kElems], float r) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = SAT ? sat_e4m3(t[4 * i + e] * r) : t[4 * i + e] * r;
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w, true);
      o[i] = static_cast<uint32_t>(w);
    }
    return o;
  }
  // The plain encoding saturates nothing (past 464 it gives NaN): rows are
  // encoded plainly, and a lane whose results passed 448 encodes and writes
  // its vectors again with the clamp (encode_store).
  static constexpr bool kSaturates = true;
  // Whether the weights alone keep every result of rows of width h inside
  // the range: |x_j r| <= sqrt(h) since x_j^2 <= S (fp32 rounding of S and of
  // the products stays far inside the 2^-10 margin), so |y_j| <= sqrt(h)
  // max|gamma|. The largest |gamma| is taken on the bf16 bits (non-negative
  // bf16 values order like 16-bit integers; a NaN weight counts as huge),
  // one packed integer maximum per weight dword; uniform over the wavefront.
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ u16x2 magnitudes(uint32_t w) {  // by value, as as_bf16x2
    return __builtin_bit_cast(u16x2, w & 0x7fff7fffu);
  }
  template <int V>
  static __device__ __forceinline__ bool weights_bound(const G (&g)[V], float h) {
    u16x2 m = {0, 0};
#pragma unroll
    for (int j = 0; j < V; ++j) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        m = __builtin_elementwise_max(m, magnitudes(g[j].lo[i]));
        m = __builtin_elementwise_max(m, magnitudes(g[j].hi[i]));
      }
    }
    const uint32_t top = m.x > m.y ? m.x : m.y;
    const float gmax = __uint_as_float(top << 16);
    const bool lane = gmax * __builtin_sqrtf(h) * (1.0f + 0x1p-10f) <= 448.0f;
    return __builtin_amdgcn_ballot_w64(!lane) == 0;
  }
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float lane_value(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// S plus the values of lanes l0, l0 + step, ..., n of them, added one after
// another in that order (every lane gets the same result). The lane reads go
// out four at a time ahead of their additions.
__device__ __forceinline__ float add_lanes_in_order(float S, float v, int l0, int step, int n) {
  int i = 0;
  for (; i + 4 <= n; i += 4) {
    const int l = l0 + i * step;
    const float a = lane_value(v, l), b = lane_value(v, l + step), c = lane_value(v, l + 2 * step),
                e = lane_value(v, l + 3 * step);
    S += a;
    S += b;
    S += c;
    S += e;
  }
  for (; i < n; ++i) S += lane_value(v, l0 + i * step);
  return S;
}

// Sums over the 64 lanes of a wavefront of R independent values at once
// (one per row a wavefront holds); every lane receives the same sums. Each
// step is applied to all R values before the next, so the steps of
// different rows fill each other's pipeline gaps, while every value is
// added in the same order as on its own. Must be called with all 64 lanes
// active.
template <int R>
__device__ __forceinline__ void wave_sums(float (&v)[R]) {
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] += dpp<0xB1>(v[r]);   // quad_perm [1,0,3,2]: pairs
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] += dpp<0x4E>(v[r]);   // quad_perm [2,3,0,1]: quads
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] += dpp<0x141>(v[r]);  // row_half_mirror: 8 lanes
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] += dpp<0x140>(v[r]);  // row_mirror: 16 lanes (row sums)
#pragma unroll
  for (int r = 0; r < R; ++r)
    v[r] = (lane_value(v[r], 0) + lane_value(v[r], 16)) + (lane_value(v[r], 32) + lane_value(v[r], 48));
}

// Sum over the 64 lanes of a wavefront; every lane receives the same value.
__device__ __forceinline__ float wave_sum(float v) {
  float a[1] = {v};
  wave_sums<1>(a);
  return a[0];
}

// Exact v / sv for 0 <= v < 2^20, 1 <= sv < 2^20: a float estimate off by at
// most one, then corrected with integer arithmetic.
__device__ __forceinline__ int slice_of(int v, int sv, float inv_sv) {
  int q = static_cast<int>(static_cast<float>(v) * inv_sv);
  q += ((q + 1) * sv <= v) ? 1 : 0;
  q -= (q * sv > v) ? 1 : 0;
  return q;
}

// Everything a wavefront reads from its segment's kernel arguments, copied
// into scalar registers at kernel entry: the copy sits before any branch, so
// the scalar loads issue together and retire in one round trip.
struct Hot {
  const void* x;
  void* y;
  const void* gamma;
  const float* stats_in;
  float* stats_out;
  int64_t x_stride, y_stride, T;
  int rows_per_wg, nwg, nslot, wpr_log2, sub_lanes_log2, lds_gamma, lay_k, comb_k, masked, slice_vec,
      head_log2, emit_rinv, dense, tail_lanes, pack_log2;
  uint32_t row_bytes, flush_mask;
  float inv_slice_vec, h, inv_h, eps;

  __device__ __forceinline__ Hot(const Args& a, const Seg& s)
      : x(s.x), y(s.y), gamma(s.gamma), stats_in(s.stats_in), stats_out(s.stats_out),
        x_stride(s.x_stride), y_stride(s.y_stride), T(a.T), rows_per_wg(s.rows_per_wg), nwg(s.nwg),
        nslot(s.nslot), wpr_log2(s.wpr_log2), sub_lanes_log2(s.sub_lanes_log2), lds_gamma(s.lds_gamma),
        lay_k(s.lay_k), comb_k(s.comb_k), masked(s.masked), slice_vec(s.slice_vec), head_log2(s.head_log2),
        emit_rinv(s.emit_rinv), dense(s.dense), tail_lanes(s.tail_lanes), pack_log2(s.pack_log2),
        row_bytes(s.row_bytes), flush_mask(s.flush_mask), inv_slice_vec(s.inv_slice_vec), h(s.h),
        inv_h(s.inv_h), eps(a.eps) {}

  // A segment of a paired launch, whose rows are one slice in one
  // wavefront: everything but the first fields of the segment (pointers,
  // strides, row bytes, 1/H) is implied, so only those are loaded. The
  // layout is the plain strided one (slot j, lane l: vector 64 j + l) with
  // its V slots and one flush at the last; slots past the row read zeros,
  // whose squares add nothing, and their stores are dropped.
  template <int V>
  __device__ __forceinline__ void paired_one_slice() {
    wpr_log2 = 0;
    sub_lanes_log2 = 6;
    rows_per_wg = 4;
    masked = 0;
    lds_gamma = 1;
    lay_k = 1;
    dense = 1;
    nslot = V;
    flush_mask = 1u << (V - 1);
    tail_lanes = kWave;
    slice_vec = 0;
    // the few arguments left, pinned here so that their loads issue together
    // at entry (left alone, the compiler sinks some of them past the weight
    // copies, a second and third round trip before the first row load)
    asm volatile("" : "+s"(x), "+s"(y), "+s"(gamma), "+s"(x_stride), "+s"(y_stride), "+s"(row_bytes), "+s"(inv_h),
                 "+s"(T), "+s"(eps));
  }
};

// The segment's slot table (each slot's first vector), read at kernel entry
// with the other arguments.
template <int VPL>
struct Tables {
  int base[VPL];
  __device__ __forceinline__ explicit Tables(const Seg& s) {
#pragma unroll
    for (int j = 0; j < VPL; ++j) base[j] = s.slot_base[j];
    // Pin every entry here, before the dispatch on the slot count: left to
    // itself the compiler sinks the loads of entries only the wider bodies
    // use past that branch, which costs each launch a second round trip to
    // memory before its first row load. The empty asm emits nothing.
#pragma unroll
    for (int j = 0; j < VPL; ++j) asm volatile("" : "+s"(base[j]));
  }
};

// Where this lane's V slots sit in a row of one segment: fixed for the whole
// launch, computed once per wavefront. A team of 2^wpr_log2 wavefronts owns
// a row; it is split into sub-teams of 2^sub_lanes_log2 lanes, and the row's
// slices are dealt to the sub-teams round-robin, so slices narrower than the
// team still keep every lane busy.
template <int V>
struct Layout {
  int wpr_log2, wpr, team, tl;
  uint32_t off[V];  // byte offset of each slot's vector; kOutside, or past the row, when empty
  int base[V];      // vector index of each slot, also when empty (masked layout)

  // One slice, a one-wavefront team: slot j of lane l holds vector 64 j + l
  // (offsets past the row are dropped by the range check).
  __device__ __forceinline__ Layout(int wave, int lane) : wpr_log2(0), wpr(1), team(wave), tl(lane) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      base[j] = j * kWave + lane;
      off[j] = static_cast<uint32_t>(base[j]) * 16u;
    }
  }

  template <int VPL>
  __device__ __forceinline__ Layout(const Tables<VPL>& tb, const Hot& s, int wave, int lane) {
    static_assert(V <= VPL, "layout wider than its table");
    wpr_log2 = s.wpr_log2;
    wpr = 1 << wpr_log2;
    team = wave >> wpr_log2;
    tl = ((wave & (wpr - 1)) << 6) | lane;  // lane within the team
    const int stl = tl & ((1 << s.sub_lanes_log2) - 1);
    const int lane_vec = (tl >> s.sub_lanes_log2) * s.slice_vec + stl;
#pragma unroll
    for (int j = 0; j < V; ++j) base[j] = tb.base[j] + lane_vec;
    // One addition per slot (the lane's offset plus the slot's base), and a
    // lane test only on slots that end a ragged slice: this runs before the
    // first row load.
    if (s.dense) {
#pragma unroll
      for (int j = 0; j < V; ++j) off[j] = slot_offset(tb.base[j], lane_vec, stl, false, 0, true);
    } else {
#pragma unroll
      for (int j = 0; j < V; ++j)
        off[j] = slot_offset(tb.base[j], lane_vec, stl, (s.flush_mask >> j) & 1u, s.tail_lanes, false);
    }
  }
};

// Row `row` of the segment as a buffer resource; rows past T get an empty one.
template <class E>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* p, int64_t stride, int64_t row,
                                                           bool live, uint32_t bytes) {
  return rsrc(static_cast<const char*>(p) + row * stride * E::kBytes, live ? bytes : 0u);
}

template <class E, int VPL, bool NT>
__device__ __forceinline__ void load_row(u32x4 (&d)[VPL], __amdgpu_buffer_rsrc_t r, const Layout<VPL>& L) {
#pragma unroll
  for (int j = 0; j < VPL; ++j) d[j] = load16<NT>(r, L.off[j]);
}

// The weights of this lane's slots, straight from memory (L2 after the
// first row).
template <class E, int VPL>
__device__ __forceinline__ void load_gamma(typename E::G (&g)[VPL], const Hot& s, const Layout<VPL>& L) {
  const auto r = rsrc(s.gamma, s.row_bytes * E::kGammaScale);
#pragma unroll
  for (int j = 0; j < VPL; ++j) g[j] = E::load_gamma(r, L.off[j]);
}

// Sums over aligned groups of 2^hl lanes (hl <= 6), every lane of a group
// receiving the same value: the heads of the headwise form (review,
// "Layerwise vs. headwise QK-Norm"), and the slices of narrow sub-teams.
// Within a row of 16 lanes each butterfly step adds the partner group's sum,
// and the addition is commutative, so the lanes agree bit for bit; groups of
// 32 and 64 lanes add the row sums read from lanes 0, 16, 32 and 48 in a
// fixed order.
template <int V>
__device__ __forceinline__ void head_sums(float (&q)[V], int hl, int lane) {
  if (hl >= 1) {
#pragma unroll
    for (int j = 0; j < V; ++j) q[j] += dpp<0xB1>(q[j]);
  }
  if (hl >= 2) {
#pragma unroll
    for (int j = 0; j < V; ++j) q[j] += dpp<0x4E>(q[j]);
  }
  if (hl >= 3) {
#pragma unroll
    for (int j = 0; j < V; ++j) q[j] += dpp<0x141>(q[j]);
  }
  if (hl >= 4) {
#pragma unroll
    for (int j = 0; j < V; ++j) q[j] += dpp<0x140>(q[j]);
  }
  if (hl == 5) {
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const float lo = lane_value(q[j], 0) + lane_value(q[j], 16);
      const float hi = lane_value(q[j], 32) + lane_value(q[j], 48);
      q[j] = lane < 32 ? lo : hi;
    }
  } else if (hl == 6) {
#pragma unroll
    for (int j = 0; j < V; ++j)
      q[j] = (lane_value(q[j], 0) + lane_value(q[j], 16)) + (lane_value(q[j], 32) + lane_value(q[j], 48));
  }
}

// The row statistic S = sum over slices (ascending) of each slice's sum of
// squares. Teams of several wavefronts add their partials through `part`
// (one barrier, and a second one only when `reuse`: the workgroup goes on to
// combine another row there; uniform over the workgroup); every lane of the
// team returns the same S.
//
// NARROW: the kernels for launches with slices narrower than a wavefront.
// Their segments may have sub-teams of fewer than 64 lanes, sub-teams of
// whole wavefronts, or the masked layout (told apart at run time); the
// other kernels only see sub-teams of whole wavefronts.
template <class E, int VPL, bool NARROW>
__device__ __forceinline__ float row_stat(const u32x4 (&d)[VPL], const Hot& s, const Layout<VPL>& L,
                                          int wave, int lane, float* part, bool reuse) {
  float S = 0.f;
  const int w0 = L.team << L.wpr_log2;
  const bool narrow_subs = NARROW && s.sub_lanes_log2 < 6;
  const bool masked = NARROW && s.masked;
  if (!narrow_subs && !masked) {
    // slots are grouped by slice; a set bit in flush_mask closes a slice
    // (this wavefront's share of it)
    float p = 0.f;
    int slice = 0;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      p = E::sumsq(d[j], p);
      if ((s.flush_mask >> j) & 1u) {
        const float P = wave_sum(p);
        p = 0.f;
        if (L.wpr == 1)
          S += P;
        else if (lane == 0)
          part[wave * kWave + slice] = P;
        ++slice;
      }
    }
  } else if (narrow_subs) {
    // 2^(6-sl) sub-teams per wavefront. A set bit in flush_mask closes a
    // round: every sub-team's current slice (sub-team u's round-i slice is
    // u + i nsub). Group sums over each sub-team's lanes, read from its first
    // lane, are whole slice partials.
    const int sl = s.sub_lanes_log2;
    const int nsw_log2 = 6 - sl;
    float p = 0.f;
    int round = 0;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      p = E::sumsq(d[j], p);
      if ((s.flush_mask >> j) & 1u) {
        float g[1] = {p};
        head_sums<1>(g, sl, lane);
        // this wavefront's sub-teams hold slices k0, k0 + 1, ... this round
        const int k0 = ((wave & (L.wpr - 1)) << nsw_log2) + (round << (nsw_log2 + L.wpr_log2));
        const int last = min(k0 + (1 << nsw_log2), s.lay_k);
        if (L.wpr == 1) {
          // round-major, sub-team-minor: ascending k
          S = add_lanes_in_order(S, g[0], 0, 1 << sl, last - k0);
        } else {
          // the first lane of each sub-team publishes its slice's partial
          const int k = k0 + (lane >> sl);
          if ((lane & ((1 << sl) - 1)) == 0 && k < last) part[w0 * kWave + k] = g[0];
        }
        p = 0.f;
        ++round;
      }
    }
  } else {
    // plain strided slots; each vector's squares join the partial of the
    // slice its index falls in
    float q[VPL];
    int sid[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      q[j] = E::sumsq(d[j], 0.f);
      sid[j] = slice_of(L.base[j], s.slice_vec, s.inv_slice_vec);
    }
    for (int k = 0; k < s.lay_k; ++k) {
      float p = 0.f;
#pragma unroll
      for (int j = 0; j < VPL; ++j) p += (sid[j] == k) ? q[j] : 0.f;
      const float P = wave_sum(p);
      if (L.wpr == 1)
        S += P;
      else if (lane == 0)
        part[wave * kWave + k] = P;
    }
  }
  if (L.wpr > 1) {
    // Sub-teams of whole wavefronts: slice k's partials come from the
    // wavefronts of sub-team k % nsub, at index k / nsub of their partial
    // lists. Narrower sub-teams wrote whole slice partials at index k of the
    // team's first list. Lane k gathers slice k (one LDS round trip for all
    // lanes), then the slices are added in ascending k.
    __syncthreads();
    float Pk = 0.f;
    if (lane < s.lay_k) {
      if (!narrow_subs) {
        // log2 of the wavefronts per sub-team (the whole team when masked)
        const int sub_w = s.sub_lanes_log2 - 6;
        const int nsub_log2 = L.wpr_log2 - sub_w;
        const int w1 = w0 + ((lane & ((1 << nsub_log2) - 1)) << sub_w);
        const int i = lane >> nsub_log2;
        // four reads in flight at a time, added in wavefront order; reads
        // past the sub-team repeat its last wavefront and add zero (partials
        // are sums of squares, never -0, so adding +0 changes nothing)
        const int cnt = 1 << sub_w;
        if (cnt == 1) Pk = part[w1 * kWave + i];
        for (int w = 0; cnt > 1 && w < cnt; w += 4) {
          float x[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) x[u] = part[(w1 + min(w + u, cnt - 1)) * kWave + i];
#pragma unroll
          for (int u = 0; u < 4; ++u) Pk += w + u < cnt ? x[u] : 0.f;
        }
      } else {
        Pk = part[w0 * kWave + lane];
      }
    }
    S = add_lanes_in_order(S, Pk, 0, 1, s.lay_k);
    if (reuse) __syncthreads();  // `part` is free again
  }
  return S;
}

// 1 / sqrt(a) by the hardware reciprocal square root, within one ulp (0.73
// ulp at worst on the MI355X samples checked, against 1.17 for a square root
// followed by a division). The instruction returns infinity for denormal
// arguments, so those are scaled by 2^64 first and the result by 2^32, both
// exact. Zero gives infinity, infinity zero and NaN NaN, as 1 / sqrt does.
__device__ __forceinline__ float rsqrt_full(float a) {
  return a < 0x1p-126f ? __builtin_amdgcn_rsqf(a * 0x1p64f) * 0x1p32f : __builtin_amdgcn_rsqf(a);
}

// The inverse RMS of a row (review Eq. 6): the fused forward and the
// statistic-only output use this same expression, so they agree bit for bit.
// The mean is S times the host's 1/H (exact for a power-of-two H, otherwise
// within an ulp of S / H) with eps added in the same fused multiply-add, so
// no division sits between the statistic and the scaling.
__device__ __forceinline__ float inv_rms(float S, float inv_h, float eps) {
  return rsqrt_full(__builtin_fmaf(S, inv_h, eps));
}

// Scale and store a lane's vectors: vector j with weights gw(j) and inverse
// RMS rw(j). Types that saturate (FP8) are encoded plainly while each
// vector's largest |y| is tracked; a vector with a result past the type's
// range is not stored (its store goes to the dropped offset) but marked,
// and the lanes with marks then load those input vectors again (still
// unwritten, also in place) with their weights gr(j), and store them
// encoded with the clamp. The common case is one straight pass: a compare,
// a select and an OR per vector, and one branch per row.
template <class E, int VPL, bool NT, bool CHECK, class GW, class RW, class GR>
__device__ __forceinline__ void encode_store(const u32x4 (&d)[VPL], GW gw, RW rw, GR gr,
                                             __amdgpu_buffer_rsrc_t xr, __amdgpu_buffer_rsrc_t yr,
                                             const Layout<VPL>& L) {
  uint32_t redo = 0;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    float peak = 0.f;
    const u32x4 o = E::template encode<false>(d[j], gw(j), rw(j), peak);
    if constexpr (CHECK) {
      const bool over = peak > 448.0f;
      redo |= over ? 1u << j : 0u;
      store16<NT>(yr, over ? kOutside : L.off[j], o);
    } else {
      store16<NT>(yr, L.off[j], o);
    }
  }
  if constexpr (CHECK) {
    if (redo != 0) {
      for (int j = 0; j < VPL; ++j) {
        if ((redo >> j) & 1u) {
          float unused = 0.f;
          const u32x4 x = load16<NT>(xr, L.off[j]);
          store16<NT>(yr, L.off[j], E::template encode<true>(x, gr(j), rw(j), unused));
        }
      }
    }
  }
}

// Row `row` scaled by its statistic S and the per-column weights g.
template <class E, int VPL, bool NT, bool CHECK = E::kSaturates>
__device__ __forceinline__ void scale_store(const u32x4 (&d)[VPL], const typename E::G (&g)[VPL], float S,
                                            const Hot& s, int64_t row, bool live, const Layout<VPL>& L) {
  const float r = inv_rms(S, s.inv_h, s.eps);
  const auto grs = rsrc(s.gamma, s.row_bytes * E::kGammaScale);
  encode_store<E, VPL, NT, CHECK>(
      d, [&](int j) -> const typename E::G& { return g[j]; }, [&](int) { return r; },
      [&](int j) { return E::load_gamma(grs, L.off[j]); }, row_rsrc<E>(s.x, s.x_stride, row, live, s.row_bytes),
      row_rsrc<E>(s.y, s.y_stride, row, live, s.row_bytes), L);
}

// FP8 rows whose products x gamma (E::products) were formed while the row's
// statistic was pending: y = t r, encoded as encode_store does. `peak` is
// the lane's largest |t|; when peak * r passes 448 the lane encodes all its
// vectors with the clamp (the same bits as encode_store's redo, which
// clamps only the vectors past the range: the clamp leaves the others as
// they are).
template <class E, int VPL, bool NT>
__device__ __forceinline__ void products_store(const float (&t)[VPL][E::kElems], float peak, float S,
                                               const Hot& s, int64_t row, bool live, const Layout<VPL>& L) {
  const float r = inv_rms(S, s.inv_h, s.eps);
  const auto yr = row_rsrc<E>(s.y, s.y_stride, row, live, s.row_bytes);
  if (peak * r > 448.0f) {
#pragma unroll
    for (int j = 0; j < VPL; ++j) store16<NT>(yr, L.off[j], E::template encode_products<true>(t[j], r));
  } else {
#pragma unroll
    for (int j = 0; j < VPL; ++j) store16<NT>(yr, L.off[j], E::template encode_products<false>(t[j], r));
  }
}

// The split path's precomputed partials of a row (MODE_APPLY): lane k <
// comb_k fetches partial k, laid out [comb_k][T]. Issued with the row's own
// loads, so its round trip overlaps theirs; other modes load nothing.
template <int MODE>
__device__ __forceinline__ float load_partial(const Hot& s, int64_t row, bool live, int lane) {
  if constexpr (MODE == MODE_APPLY)
    return (live && lane < s.comb_k) ? s.stats_in[static_cast<int64_t>(lane) * s.T + row] : 0.f;
  return 0.f;
}
// Loads load_partial adds to a wavefront's count of outstanding loads.
template <int MODE>
constexpr int kPartialLoads = MODE == MODE_APPLY ? 1 : 0;

// Finish one row whose data (and weights) are in registers: statistic (or
// the precomputed partials `pk`, from load_partial), then scale and store,
// or publish the statistic.
template <class E, int VPL, int MODE, bool NARROW, bool NT, bool CHECK = E::kSaturates>
__device__ __forceinline__ void row_finish(const u32x4 (&d)[VPL], const typename E::G (&g)[VPL], const Hot& s,
                                           const Layout<VPL>& L, int64_t row, bool live, int wave,
                                           int lane, float* part, bool reuse, float pk) {
  float S = 0.f;
  if constexpr (MODE == MODE_APPLY) {
    // lane k holds partial k; they are added in ascending k
    S = add_lanes_in_order(S, pk, 0, 1, s.comb_k);
  } else {
    S = row_stat<E, VPL, NARROW>(d, s, L, wave, lane, part, reuse);
  }
  if constexpr (MODE == MODE_STATS) {
    if (live && L.tl == 0) s.stats_out[row] = s.emit_rinv ? inv_rms(S, s.inv_h, s.eps) : S;
  } else {
    scale_store<E, VPL, NT, CHECK>(d, g, S, s, row, live, L);
  }
}

// One row, headwise: each slot's head statistic, then its own inverse RMS
// (the mean divides by the head width) and the head's weights `g`, which
// are the same vector for every slot of this lane.
template <class E, int VPL, bool NT>
__device__ __forceinline__ void head_finish(const u32x4 (&d)[VPL], const typename E::G& g, const Hot& s,
                                            const Layout<VPL>& L, int64_t row, bool live, int lane) {
  float q[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) q[j] = E::sumsq(d[j], 0.f);
  head_sums<VPL>(q, s.head_log2, lane);
  float r[VPL];
#pragma unroll
  for (int j = 0; j < VPL; ++j) r[j] = rsqrt_full(q[j] * s.inv_h + s.eps);
  encode_store<E, VPL, NT, E::kSaturates>(
      d, [&](int) -> const typename E::G& { return g; }, [&](int j) { return r[j]; }, [&](int) { return g; },
      row_rsrc<E>(s.x, s.x_stride, row, live, s.row_bytes), row_rsrc<E>(s.y, s.y_stride, row, live, s.row_bytes), L);
}

// Weights for the team's slots when several rows share a workgroup: the
// workgroup copies gamma into LDS once, by direct buffer-to-LDS loads (no
// VGPRs involved), and every wavefront reads its slots from there. That is
// one global read of gamma per workgroup instead of one per row. The copy is
// issued before the row loads (gamma_to_lds), and waited for after them
// (gamma_from_lds), so it overlaps the row transfer. The LDS block is
// rounded up to whole NW * 64 * 16-byte chunks, so lanes past the end of
// gamma (which read zeros) still write inside it.
template <class E, int VPL, int NW>
__device__ __forceinline__ void gamma_to_lds(const Hot& s, int wave, int lane, u32x4* lds_g) {
  // rows_per_wg > 1 here, so a row has at most VPL * NW * 64 / 2 vectors,
  // and its weights kGammaScale times as many
  constexpr int kChunks = static_cast<int>(E::kGammaScale) * ((VPL + 1) / 2);
  const uint32_t gbytes = s.row_bytes * E::kGammaScale;
  const auto gr = rsrc(s.gamma, gbytes);
  const uint32_t nvec = gbytes >> 4;
#pragma unroll
  for (int k = 0; k < kChunks; ++k) {
    const uint32_t v0 = static_cast<uint32_t>(wave * kWave + k * NW * kWave);
    if (v0 < nvec)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(gr, (__attribute__((address_space(3))) void*)(lds_g + v0), 16,
                                               (v0 + static_cast<uint32_t>(lane)) * 16u, 0, 0, 0);
  }
}

// Wait for this wavefront's copies (issued before its INFLIGHT row loads, so
// at most that many loads may stay in flight), then for the whole
// workgroup's. Empty slots (offsets at or past the row's end) read the last
// weight vector: their rows are zeros and their stores are dropped.
template <class E, int VPL>
__device__ __forceinline__ void gamma_read_lds(typename E::G (&g)[VPL], const Hot& s, const Layout<VPL>& L,
                                               const u32x4* lds_g) {
  const uint32_t last = (s.row_bytes >> 4) - 1u;
#pragma unroll
  for (int j = 0; j < VPL; ++j) g[j] = E::gamma_lds(lds_g, min(L.off[j] >> 4, last));
}

template <int INFLIGHT>
__device__ __forceinline__ void wait_gamma_copies() {
  static_assert(INFLIGHT < 64, "vmcnt holds 6 bits");
  // s_waitcnt with vmcnt = INFLIGHT and the lgkm / exp counters left alone
  __builtin_amdgcn_s_waitcnt((INFLIGHT & 0xF) | ((INFLIGHT >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  __syncthreads();
}

template <class E, int VPL, int INFLIGHT = VPL>
__device__ __forceinline__ void gamma_from_lds(typename E::G (&g)[VPL], const Hot& s, const Layout<VPL>& L,
                                               const u32x4* lds_g) {
  wait_gamma_copies<INFLIGHT>();
  gamma_read_lds<E, VPL>(g, s, L, lds_g);
}

// Persistent workgroups: group gi, gi + G, gi + 2G, ... (G = gridDim.x). The
// next group's rows are loaded before the current group is reduced and
// stored, so reads of later rows overlap writes of earlier ones; gamma is
// loaded once. Every wavefront of a workgroup runs the same number of
// iterations (rows past T are empty), so barriers stay in step.
template <class E, int VPL, bool NARROW, bool NT>
__device__ __forceinline__ void fwd_pipelined(const Hot& s, const Layout<VPL>& L,
                                              int wave, int lane, float* part) {
  const int64_t G = gridDim.x;
  int64_t g0 = blockIdx.x;
  if (g0 >= s.nwg) return;
  u32x4 A[VPL], B[VPL];
  typename E::G g[VPL];
  int64_t ra = g0 * s.rows_per_wg + L.team;
  load_row<E, VPL, NT>(A, row_rsrc<E>(s.x, s.x_stride, ra, ra < s.T, s.row_bytes), L);
  load_gamma<E, VPL>(g, s, L);
  for (;;) {
    const int64_t g1 = g0 + G;
    const int64_t rb = g1 * s.rows_per_wg + L.team;
    load_row<E, VPL, NT>(B, row_rsrc<E>(s.x, s.x_stride, rb, g1 < s.nwg && rb < s.T, s.row_bytes), L);
    float S = row_stat<E, VPL, NARROW>(A, s, L, wave, lane, part, true);
    scale_store<E, VPL, NT>(A, g, S, s, ra, ra < s.T, L);
    if (g1 >= s.nwg) break;
    const int64_t g2 = g1 + G;
    ra = g2 * s.rows_per_wg + L.team;
    load_row<E, VPL, NT>(A, row_rsrc<E>(s.x, s.x_stride, ra, g2 < s.nwg && ra < s.T, s.row_bytes), L);
    S = row_stat<E, VPL, NARROW>(B, s, L, wave, lane, part, true);
    scale_store<E, VPL, NT>(B, g, S, s, rb, rb < s.T, L);
    if (g2 >= s.nwg) break;
    g0 = g2;
  }
}

// The statistic of each of the RPW rows a one-wavefront team holds
// (sub-teams of whole wavefronts): per slice, the lane sums of all rows
// reduce together (wave_sums), then each row adds its slices in ascending
// order, as row_stat does for one row, so the results are the same bits.
template <class E, int V, int RPW>
__device__ __forceinline__ void stat_rows(const u32x4 (&d)[RPW][V], const Hot& s, float (&S)[RPW]) {
  float p[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    S[r] = 0.f;
    p[r] = 0.f;
  }
#pragma unroll
  for (int j = 0; j < V; ++j) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) p[r] = E::sumsq(d[r][j], p[r]);
    if ((s.flush_mask >> j) & 1u) {
      wave_sums<RPW>(p);
#pragma unroll
      for (int r = 0; r < RPW; ++r) {
        S[r] += p[r];
        p[r] = 0.f;
      }
    }
  }
}

// Publish the statistics of RPW consecutive rows (statistics-only passes).
template <int RPW>
__device__ __forceinline__ void store_stats(const float (&S)[RPW], const Hot& s, int64_t row0, int tl) {
#pragma unroll
  for (int r = 0; r < RPW; ++r)
    if (row0 + r < s.T && tl == 0) s.stats_out[row0 + r] = s.emit_rinv ? inv_rms(S[r], s.inv_h, s.eps) : S[r];
}

// One wavefront per row, RPW consecutive rows per wavefront: all their loads
// go out first, then the rows are finished in order, so the work on one row
// overlaps the loads of the next; the rows share one copy of the weights.
// Each row is reduced by the wavefront on its own (no LDS); statistics-only
// passes reduce all the rows together.
template <class E, int V, int NW, int MODE, bool NT, int RPW>
__device__ __forceinline__ void body_rows(const Hot& s, const Layout<V>& L, int wave, int lane, float* part,
                                          u32x4* lds_g) {
  int64_t gi = blockIdx.x;
  int64_t row0 = (gi * s.rows_per_wg + L.team) * RPW;
  u32x4 d[RPW][V];
  float pk[RPW];
  typename E::G g[V];
  const bool staged = MODE != MODE_STATS && s.lds_gamma;
  if (staged) gamma_to_lds<E, V, NW>(s, wave, lane, lds_g);
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    load_row<E, V, NT>(d[r], row_rsrc<E>(s.x, s.x_stride, row0 + r, row0 + r < s.T, s.row_bytes), L);
    pk[r] = load_partial<MODE>(s, row0 + r, row0 + r < s.T, lane);
  }
  if constexpr (MODE != MODE_STATS) {
    if (staged)
      gamma_from_lds<E, V, (V + kPartialLoads<MODE>) * RPW>(g, s, L, lds_g);
    else
      load_gamma<E, V>(g, s, L);
  }
  if constexpr (MODE == MODE_STATS) {
    float S[RPW];
    stat_rows<E, V, RPW>(d, s, S);
    store_stats<RPW>(S, s, row0, L.tl);
    // grids capped at the hardware limit only
    for (gi += gridDim.x; gi < s.nwg; gi += gridDim.x) {
      row0 = (gi * s.rows_per_wg + L.team) * RPW;
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        load_row<E, V, NT>(d[r], row_rsrc<E>(s.x, s.x_stride, row0 + r, row0 + r < s.T, s.row_bytes), L);
      stat_rows<E, V, RPW>(d, s, S);
      store_stats<RPW>(S, s, row0, L.tl);
    }
    return;
  }
  // FP8 forward: when the weights alone bound every result inside the range
  // (checked once for all the wavefront's rows), the rows skip the
  // per-vector test.
  bool check = E::kSaturates;
  if constexpr (E::kSaturates && MODE == MODE_FWD) check = !E::weights_bound(g, s.h);
  if (check) {
#pragma unroll
    for (int r = 0; r < RPW; ++r)
      row_finish<E, V, MODE, false, NT>(d[r], g, s, L, row0 + r, row0 + r < s.T, wave, lane, part, false, pk[r]);
  } else {
#pragma unroll
    for (int r = 0; r < RPW; ++r)
      row_finish<E, V, MODE, false, NT, false>(d[r], g, s, L, row0 + r, row0 + r < s.T, wave, lane, part, false,
                                               pk[r]);
  }
  // grids capped at the hardware limit only
  for (gi += gridDim.x; gi < s.nwg; gi += gridDim.x) {
    row0 = (gi * s.rows_per_wg + L.team) * RPW;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      load_row<E, V, NT>(d[r], row_rsrc<E>(s.x, s.x_stride, row0 + r, row0 + r < s.T, s.row_bytes), L);
      pk[r] = load_partial<MODE>(s, row0 + r, row0 + r < s.T, lane);
    }
    if constexpr (MODE != MODE_STATS) load_gamma<E, V>(g, s, L);
#pragma unroll
    for (int r = 0; r < RPW; ++r)
      row_finish<E, V, MODE, false, NT>(d[r], g, s, L, row0 + r, row0 + r < s.T, wave, lane, part, false, pk[r]);
  }
}

// Packed rows: rows of one slice and at most 32 vectors, SLOTS slots per
// wavefront and 64 / 2^hl rows in each, row i of a slot over the aligned
// lanes i * 2^hl ... (lane l holds the row's vector l mod 2^hl; 2^hl is the
// row's vector count rounded up to a power of two), so no lane idles where
// one row per slot would leave most of the wavefront empty. A row's squares
// are summed over its lane group by the same butterfly steps a whole
// wavefront starts with; in the one-row layout the further steps only add
// the empty lanes' zeros, so the statistic, and everything computed from it,
// has the same bits. The weights are each lane's one vector, the same in
// every slot. A wavefront's rows share one buffer resource spanning them; a
// lane's offset adds its row's distance from the first (the host keeps the
// span below 2^31 bytes).
template <class E, int NW, int MODE, bool NT, int SLOTS>
__device__ __forceinline__ void body_packed(const Hot& s, int wave, int lane) {
  const int hl = s.pack_log2;
  const int rps_log2 = 6 - hl;  // rows per slot
  const int sub = lane >> hl;   // the lane's row within a slot
  const int vec = lane & ((1 << hl) - 1);
  const bool vlive = static_cast<uint32_t>(vec) < (s.row_bytes >> 4);
  const int64_t xs = s.x_stride * E::kBytes, ys = s.y_stride * E::kBytes;
  typename E::G g[1];
  if constexpr (MODE != MODE_STATS)
    g[0] = E::load_gamma(rsrc(s.gamma, s.row_bytes * E::kGammaScale),
                         vlive ? static_cast<uint32_t>(vec) * 16u : kOutside);
  // FP8: the weight bound, as for one-row layouts (forward passes only)
  bool check = E::kSaturates;
  if constexpr (E::kSaturates && MODE == MODE_FWD) check = !E::weights_bound(g, s.h);
  for (int64_t gi = blockIdx.x; gi < s.nwg; gi += gridDim.x) {
    const int64_t row0 = ((gi * NW + wave) * SLOTS) << rps_log2;
    int64_t span = s.T - row0;  // rows of this wavefront
    span = span < (int64_t{SLOTS} << rps_log2) ? span : (int64_t{SLOTS} << rps_log2);
    int64_t row[SLOTS];
    uint32_t xo[SLOTS], yo[SLOTS];
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
      const int64_t rel = (int64_t{j} << rps_log2) + sub;
      row[j] = row0 + rel;
      xo[j] = packed_offset(rel, span, vec, vlive, xs);
      yo[j] = packed_offset(rel, span, vec, vlive, ys);
    }
    const auto xr = rsrc(static_cast<const char*>(s.x) + row0 * xs, packed_bytes(span, xs, s.row_bytes));
    u32x4 d[SLOTS];
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) d[j] = load16<NT>(xr, xo[j]);
    float S[SLOTS];
    if constexpr (MODE == MODE_APPLY) {
      // lane v of a row's group fetches the row's partial v (the host packs
      // apply launches only where a group has a lane for each partial), and
      // the partials are added in ascending order from zero, partial k read
      // from the group's lane k
      float pk[SLOTS];
#pragma unroll
      for (int j = 0; j < SLOTS; ++j)
        pk[j] = (vec < s.comb_k && row[j] < s.T) ? s.stats_in[vec * s.T + row[j]] : 0.f;
      const int group = (sub << hl) * 4;  // ds_bpermute address of the group's first lane
#pragma unroll
      for (int j = 0; j < SLOTS; ++j) S[j] = 0.f;
      for (int k = 0; k < s.comb_k; ++k) {
#pragma unroll
        for (int j = 0; j < SLOTS; ++j)
          S[j] += __int_as_float(__builtin_amdgcn_ds_bpermute(group + 4 * k, __float_as_int(pk[j])));
      }
    } else {
      float q[SLOTS];
#pragma unroll
      for (int j = 0; j < SLOTS; ++j) q[j] = E::sumsq(d[j], 0.f);
      head_sums<SLOTS>(q, hl, lane);
#pragma unroll
      for (int j = 0; j < SLOTS; ++j) S[j] = 0.f + q[j];
    }
    if constexpr (MODE == MODE_STATS) {
#pragma unroll
      for (int j = 0; j < SLOTS; ++j)
        if (vec == 0 && row[j] < s.T) s.stats_out[row[j]] = s.emit_rinv ? inv_rms(S[j], s.inv_h, s.eps) : S[j];
    } else {
      const auto yr = rsrc(static_cast<char*>(s.y) + row0 * ys, packed_bytes(span, ys, s.row_bytes));
      uint32_t redo = 0;
#pragma unroll
      for (int j = 0; j < SLOTS; ++j) {
        const float r = inv_rms(S[j], s.inv_h, s.eps);
        float peak = 0.f;
        const u32x4 o = E::template encode<false>(d[j], g[0], r, peak);
        if (E::kSaturates && check) {
          // as encode_store: a vector with a result past the range is stored
          // again, from the input, with the clamp
          const bool over = peak > 448.0f;
          redo |= over ? 1u << j : 0u;
          store16<NT>(yr, over ? kOutside : yo[j], o);
        } else {
          store16<NT>(yr, yo[j], o);
        }
      }
      if (E::kSaturates && redo != 0) {
        for (int j = 0; j < SLOTS; ++j) {
          if ((redo >> j) & 1u) {
            float unused = 0.f;
            const u32x4 x = load16<NT>(xr, xo[j]);
            store16<NT>(yr, yo[j], E::template encode<true>(x, g[0], inv_rms(S[j], s.inv_h, s.eps), unused));
          }
        }
      }
    }
  }
}

template <class E, int V, int VPL, int NW, int MODE, bool NARROW, bool NT, bool PIPE, int RPW>
__device__ __forceinline__ void body(const Hot& s, const Tables<VPL>& tb, int wave, int lane, float* part,
                                     u32x4* lds_g) {
  const Layout<V> L(tb, s, wave, lane);
  if constexpr (RPW > 1) {
    static_assert(!NARROW && !PIPE && MODE != MODE_HEAD, "several rows per wavefront: wavefront sub-teams only");
    body_rows<E, V, NW, MODE, NT, RPW>(s, L, wave, lane, part, lds_g);
  } else if constexpr (MODE == MODE_HEAD) {
    int64_t gi = blockIdx.x;
    int64_t row = gi * s.rows_per_wg + L.team;
    u32x4 d[V];
    load_row<E, V, NT>(d, row_rsrc<E>(s.x, s.x_stride, row, row < s.T, s.row_bytes), L);
    const typename E::G g = E::load_gamma(rsrc(s.gamma, (16u << s.head_log2) * E::kGammaScale),
                                          static_cast<uint32_t>(lane & ((1 << s.head_log2) - 1)) * 16u);
    head_finish<E, V, NT>(d, g, s, L, row, row < s.T, lane);
    for (gi += gridDim.x; gi < s.nwg; gi += gridDim.x) {
      row = gi * s.rows_per_wg + L.team;
      u32x4 d2[V];
      load_row<E, V, NT>(d2, row_rsrc<E>(s.x, s.x_stride, row, row < s.T, s.row_bytes), L);
      head_finish<E, V, NT>(d2, g, s, L, row, row < s.T, lane);
    }
  } else if constexpr (PIPE) {
    fwd_pipelined<E, V, NARROW, NT>(s, L, wave, lane, part);
  } else {
    // The first group needs no bounds check (a group past the end holds only
    // empty rows), so its loads follow the argument loads directly. Group
    // indices are 64-bit in every body: with up to 2^31 - 1 rows, one
    // workgroup per row and a grid capped at the hardware limit, a
    // grid-stride step passes 2^31.
    int64_t gi = blockIdx.x;
    int64_t row = gi * s.rows_per_wg + L.team;
    bool live = row < s.T;
    u32x4 d[V];
    typename E::G g[V];
    const bool staged = MODE != MODE_STATS && s.lds_gamma;
    if (staged) gamma_to_lds<E, V, NW>(s, wave, lane, lds_g);
    load_row<E, V, NT>(d, row_rsrc<E>(s.x, s.x_stride, row, live, s.row_bytes), L);
    const float pk = load_partial<MODE>(s, row, live, lane);
    if constexpr (MODE != MODE_STATS) {
      if (staged)
        gamma_from_lds<E, V, V + kPartialLoads<MODE>>(g, s, L, lds_g);
      else
        load_gamma<E, V>(g, s, L);
    }
    row_finish<E, V, MODE, NARROW, NT>(d, g, s, L, row, live, wave, lane, part,
                                       gi + static_cast<int64_t>(gridDim.x) < s.nwg, pk);
    // Only grids capped at the hardware limit get here. Reloading gamma each
    // time keeps the first row's registers free of this loop (holding them
    // across it costs about 40 VGPRs).
    for (gi += gridDim.x; gi < s.nwg; gi += gridDim.x) {
      row = gi * s.rows_per_wg + L.team;
      live = row < s.T;
      u32x4 d2[V];
      typename E::G g2[V];
      load_row<E, V, NT>(d2, row_rsrc<E>(s.x, s.x_stride, row, live, s.row_bytes), L);
      const float pk2 = load_partial<MODE>(s, row, live, lane);
      if constexpr (MODE != MODE_STATS) load_gamma<E, V>(g2, s, L);
      row_finish<E, V, MODE, NARROW, NT>(d2, g2, s, L, row, live, wave, lane, part,
                                         gi + static_cast<int64_t>(gridDim.x) < s.nwg, pk2);
    }
  }
}

// The variant is compiled for VPL slots, the widest segment of the launch;
// a narrower segment (the key rows of a grouped-query layout) runs the
// smallest of the bodies for VPL, VPL/2, VPL/4, ... slots (rounded down)
// that holds its slots, chosen by uniform branches, so key rows of half the
// query width or less skip the query rows' extra slots.
template <class E, int V, int VPL, int NW, int MODE, bool NARROW, bool NT, bool PIPE, int RPW>
__device__ __forceinline__ void dispatch(const Hot& s, const Tables<VPL>& tb, int wave, int lane,
                                         float* part, u32x4* lds_g) {
  if constexpr (V > 1) {
    if (s.nslot <= V / 2) {
      dispatch<E, V / 2, VPL, NW, MODE, NARROW, NT, PIPE, RPW>(s, tb, wave, lane, part, lds_g);
      return;
    }
  }
  body<E, V, VPL, NW, MODE, NARROW, NT, PIPE, RPW>(s, tb, wave, lane, part, lds_g);
}

// Paired rows: each one-wavefront team takes token t's row of segment a (the
// wider, VA slots) and of segment b (VB slots), one slice each, and the
// workgroup stages both weight vectors in LDS (b's after a's). Every row load
// goes out before the first wait, and each row is finished exactly as on its
// own (the same strided layout, the same order of operations, so the same
// bits). Launches of one or a few rounds of wavefronts then issue nearly all
// their reads before their writes: a workgroup stores only after all its
// tokens' rows have arrived (a barrier precedes its first store), where
// separate wavefronts for the two segments let the narrow rows' stores start
// while most rows are still being read.
template <class E, int VA, int VB, int NW, bool NT, bool EARLY>
__device__ __forceinline__ void body_pair(const Hot& sa, const Hot& sb, int wave, int lane, float* part,
                                          u32x4* lds_g) {
  const Layout<VA> La(wave, lane);
  const Layout<VB> Lb(wave, lane);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * NW + wave;
  const bool live = row < sa.T;
  u32x4 da[VA], db[VB];
  typename E::G ga[VA], gb[VB];
  // segment b's weights follow segment a's copy, rounded up to whole chunks
  // of one vector per thread as the copy loop writes them
  constexpr uint32_t kChunkVec = NW * kWave;
  const uint32_t a_vec = (sa.row_bytes * E::kGammaScale) >> 4;
  u32x4* const lds_b = lds_g + (a_vec + kChunkVec - 1) / kChunkVec * kChunkVec;
  gamma_to_lds<E, VA, NW>(sa, wave, lane, lds_g);
  gamma_to_lds<E, VB, NW>(sb, wave, lane, lds_b);
  load_row<E, VA, NT>(da, row_rsrc<E>(sa.x, sa.x_stride, row, live, sa.row_bytes), La);
  load_row<E, VB, NT>(db, row_rsrc<E>(sb.x, sb.x_stride, row, live, sb.row_bytes), Lb);
  wait_gamma_copies<VA + VB>();
  gamma_read_lds<E, VA>(ga, sa, La, lds_g);
  gamma_read_lds<E, VB>(gb, sb, Lb, lds_b);
  // Both statistics before any store, and the workgroup's barrier before
  // its first store: the workgroup writes only after all its tokens' rows
  // have landed (the scheduling barrier keeps the compiler from moving the
  // narrow row's stores up between the statistics).
  if constexpr (EARLY) {
    // FP8: the products x gamma are formed as the row vectors land, while
    // the statistics still wait for the rest, so after them only y = t r
    // and the encoding remain (one slice per row: the lane's squares in
    // slot order, then one wavefront sum each, as row_stat forms them).
    // MI355X, gated back to back, 2048 tokens of 5120/1024 columns: FP8
    // 6.20 -> 5.99 us; the same for bf16 rows, whose scaling is lighter,
    // 8.48 -> 8.57 us. The products hold 16 VGPRs per slot, so these
    // kernels keep 2 or 3 wavefronts per SIMD; they are built for rows of at
    // most kEarlySlots slots together, and the planner takes them for
    // launches of at most 2 paired wavefronts per SIMD.
    static_assert(E::kSaturates, "early products: FP8 rows");
    float ta[VA][E::kElems], tb[VB][E::kElems];
    float p[2] = {0.f, 0.f}, peak_a = 0.f, peak_b = 0.f;
#pragma unroll
    for (int j = 0; j < VA; ++j) {
      p[0] = E::sumsq(da[j], p[0]);
      E::products(da[j], ga[j], ta[j], peak_a);
    }
#pragma unroll
    for (int j = 0; j < VB; ++j) {
      p[1] = E::sumsq(db[j], p[1]);
      E::products(db[j], gb[j], tb[j], peak_b);
    }
    wave_sums<2>(p);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    products_store<E, VB, NT>(tb, peak_b, p[1], sb, row, live, Lb);
    products_store<E, VA, NT>(ta, peak_a, p[0], sa, row, live, La);
  } else {
    const float Sb = row_stat<E, VB, false>(db, sb, Lb, wave, lane, part, false);
    const float Sa = row_stat<E, VA, false>(da, sa, La, wave, lane, part, false);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    scale_store<E, VB, NT>(db, gb, Sb, sb, row, live, Lb);
    scale_store<E, VA, NT>(da, ga, Sa, sa, row, live, La);
  }
}

// blockIdx.y selects the segment (query rows, key rows), so everything a
// wavefront needs from the kernel arguments is one round of scalar loads;
// a paired launch reads both segments in that round.
template <class E, int VPL, int NW, int MODE, bool NARROW, bool NT, bool PIPE, int RPW = 1, int PAIRB = 0,
          bool PACK = false, bool EARLY = false>
__global__ void __launch_bounds__(NW * kWave) qknorm_kernel(const Args a) {
  __shared__ float part[NW * kWave];  // per-wavefront slice partials (teams of > 1 wave)
  extern __shared__ u32x4 lds_g[];    // staged gamma (dynamic size: the launch's widest row)
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  if constexpr (PACK) {
    static_assert(VPL == 1 && NW == 4 && !NARROW && NT && !PIPE && RPW == kPackSlots && PAIRB == 0,
                  "packed rows: one 4-slot body");
    const Hot s(a, a.seg[blockIdx.y]);
    body_packed<E, NW, MODE, NT, RPW>(s, wave, lane);
  } else if constexpr (PAIRB > 0) {
    // paired rows: segment 1 runs the body of PAIRB slots (each pairing its
    // own kernel, so a narrow second row does not carry a wide one's registers)
    static_assert(MODE == MODE_FWD && NW == 4 && !NARROW && NT && !PIPE && RPW == 1, "paired forward rows only");
    Hot sa(a, a.seg[0]), sb(a, a.seg[1]);
    sa.paired_one_slice<VPL>();
    sb.paired_one_slice<PAIRB>();
    body_pair<E, VPL, PAIRB, NW, NT, EARLY>(sa, sb, wave, lane, part, lds_g);
  } else {
    const Seg& seg = a.seg[blockIdx.y];
    const Hot s(a, seg);
    const Tables<VPL> tb(seg);
    dispatch<E, VPL, VPL, NW, MODE, NARROW, NT, PIPE, RPW>(s, tb, wave, lane, part, lds_g);
  }
}

// The launch dispatch: the run-time variant picks one of the kernels the
// compiled() table names; any other combination instantiates nothing and is
// refused.
template <class E, int VPL, int NW, int MODE, bool NARROW, bool NT, bool PIPE, int RPW, int PAIRB = 0,
          bool PACK = false, bool EARLY = false>
hipError_t launch_one(const Args& a, dim3 gd, unsigned lds, hipStream_t st) {
  if constexpr (compiled(E::kDtype, MODE, VPL, NW, NARROW, NT, PIPE, RPW, PAIRB, PACK, EARLY)) {
    hipLaunchKernelGGL((qknorm_kernel<E, VPL, NW, MODE, NARROW, NT, PIPE, RPW, PAIRB, PACK, EARLY>), gd,
                       dim3(NW * kWave), lds, st, a);
    return hipGetLastError();
  } else {
    return hipErrorInvalidValue;
  }
}

// Paired launches: segment 1's body, down the chain VPL, VPL/2, ...
template <class E, int VPL, int NW, int MODE, bool NARROW, bool NT, bool PIPE, int VB>
hipError_t by_pair_b(const Variant& v, const Args& a, dim3 gd, unsigned lds, hipStream_t st) {
  if (v.vpl_b == VB)
    return v.early ? launch_one<E, VPL, NW, MODE, NARROW, NT, PIPE, 1, VB, false, true>(a, gd, lds, st)
                   : launch_one<E, VPL, NW, MODE, NARROW, NT, PIPE, 1, VB>(a, gd, lds, st);
  if constexpr (VB > 1) return by_pair_b<E, VPL, NW, MODE, NARROW, NT, PIPE, VB / 2>(v, a, gd, lds, st);
  return hipErrorInvalidValue;
}

template <class E, int VPL, int NW, int MODE, bool NARROW, bool NT, bool PIPE>
hipError_t by_rpw(const Variant& v, const Args& a, dim3 gd, unsigned lds, hipStream_t st) {
  switch (v.rpw) {
    case 1:
      return v.pair ? by_pair_b<E, VPL, NW, MODE, NARROW, NT, PIPE, VPL>(v, a, gd, lds, st)
                    : launch_one<E, VPL, NW, MODE, NARROW, NT, PIPE, 1>(a, gd, lds, st);
    case 2: return launch_one<E, VPL, NW, MODE, NARROW, NT, PIPE, 2>(a, gd, lds, st);
    case 4:
      return v.pack ? launch_one<E, VPL, NW, MODE, NARROW, NT, PIPE, 4, 0, true>(a, gd, lds, st)
                    : launch_one<E, VPL, NW, MODE, NARROW, NT, PIPE, 4>(a, gd, lds, st);
    default: return hipErrorInvalidValue;
  }
}

template <class E, int VPL, int NW, int MODE, bool NARROW, bool NT>
hipError_t by_pipe(const Variant& v, const Args& a, dim3 gd, unsigned lds, hipStream_t st) {
  return v.pipe ? by_rpw<E, VPL, NW, MODE, NARROW, NT, true>(v, a, gd, lds, st)
                : by_rpw<E, VPL, NW, MODE, NARROW, NT, false>(v, a, gd, lds, st);
}

template <class E, int VPL, int NW, int MODE, bool NARROW>
hipError_t by_nt(const Variant& v, const Args& a, dim3 gd, unsigned lds, hipStream_t st) {
  return v.nt ? by_pipe<E, VPL, NW, MODE, NARROW, true>(v, a, gd, lds, st)
              : by_pipe<E, VPL, NW, MODE, NARROW, false>(v, a, gd, lds, st);
}

template <class E, int VPL, int NW, int MODE>
hipError_t by_narrow(const Variant& v, const Args& a, dim3 gd, unsigned lds, hipStream_t st) {
  return v.narrow ? by_nt<E, VPL, NW, MODE, true>(v, a, gd, lds, st)
                  : by_nt<E, VPL, NW, MODE, false>(v, a, gd, lds, st);
}

template <class E, int VPL, int NW>
hipError_t launch_vpl(const Variant& v, const Args& a, dim3 gd, unsigned lds, hipStream_t st) {
  switch (v.mode) {
    case MODE_FWD: return by_narrow<E, VPL, NW, MODE_FWD>(v, a, gd, lds, st);
    case MODE_STATS: return by_narrow<E, VPL, NW, MODE_STATS>(v, a, gd, lds, st);
    case MODE_APPLY: return by_narrow<E, VPL, NW, MODE_APPLY>(v, a, gd, lds, st);
    case MODE_HEAD: return by_narrow<E, VPL, NW, MODE_HEAD>(v, a, gd, lds, st);
    default: return hipErrorInvalidValue;
  }
}

template <class E>
hipError_t launch_dtype(const Variant& v, const Args& a, dim3 grid, unsigned lds, hipStream_t st) {
  if (!compiled(v) || v.dtype != E::kDtype) return hipErrorInvalidValue;
  if (v.nw == 4) {
    switch (v.vpl) {
      case 1: return launch_vpl<E, 1, 4>(v, a, grid, lds, st);
      case 2: return launch_vpl<E, 2, 4>(v, a, grid, lds, st);
      case 3: return launch_vpl<E, 3, 4>(v, a, grid, lds, st);
      case 4: return launch_vpl<E, 4, 4>(v, a, grid, lds, st);
      case 5: return launch_vpl<E, 5, 4>(v, a, grid, lds, st);
      case 6: return launch_vpl<E, 6, 4>(v, a, grid, lds, st);
      case 7: return launch_vpl<E, 7, 4>(v, a, grid, lds, st);
      case 8: return launch_vpl<E, 8, 4>(v, a, grid, lds, st);
      case 10: return launch_vpl<E, 10, 4>(v, a, grid, lds, st);
      case 12: return launch_vpl<E, 12, 4>(v, a, grid, lds, st);
      case 16: return launch_vpl<E, 16, 4>(v, a, grid, lds, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (v.vpl) {
    case 1: return launch_vpl<E, 1, 16>(v, a, grid, lds, st);
    case 2: return launch_vpl<E, 2, 16>(v, a, grid, lds, st);
    case 4: return launch_vpl<E, 4, 16>(v, a, grid, lds, st);
    case 8: return launch_vpl<E, 8, 16>(v, a, grid, lds, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace qkn
