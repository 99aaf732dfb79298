// qknorm_kernels.hip -- gfx950 kernels for layerwise QK-Norm.
//
// Per row (SwiftQK technical review, Eq. 1; the K-slice statistic of section
// 4b, Eqs. 3-6):
//   1. the team loads its row with 16-byte vector loads into VGPRs (the whole
//      row stays resident, so HBM is read once);
//   2. per slice, each lane accumulates its slots' squares in fp32; a
//      wavefront reduction (DPP within rows of 16 lanes, then 4 readlanes)
//      gives the slice's partial; teams of several wavefronts add their
//      partials through LDS;
//   3. the partials are summed in ascending slice order (review Eq. 5), then
//      r = 1 / sqrt(S / H + eps) with H the full width (Eq. 6);
//   4. y = (x * r) * gamma (Eq. 1 order), rounded to the output type, stored
//      with 16-byte vector stores; y may be x.
// The split path reuses the same body: MODE_STATS stops after step 2 and
// writes one fp32 per row (Algorithm 1, Phase A); MODE_APPLY skips step 2 and
// combines precomputed partials instead (Phase B's scalar sum, then Phase C).
//
// No matrix cores: the work is a reduction and an elementwise scale, bound by
// HBM bandwidth.
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
constexpr uint32_t kOutside = 0x80000000u;

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

// binary32 rows: 4 elements per 16-byte vector.
struct F32 {
  static constexpr int kBytes = 4;
  static __device__ __forceinline__ float sumsq(u32x4 d, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = __uint_as_float(d[i]);
      acc = __builtin_fmaf(v, v, acc);
    }
    return acc;
  }
  static __device__ __forceinline__ u32x4 scale(u32x4 d, u32x4 g, float r) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = __float_as_uint(__uint_as_float(d[i]) * r * __uint_as_float(g[i]));
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
struct BF16 {
  static constexpr int kBytes = 2;
  static __device__ __forceinline__ float sumsq(u32x4 d, float acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x2 p = as_bf16x2(d[i]);
      acc = __builtin_amdgcn_fdot2_f32_bf16(p, p, acc, false);
    }
    return acc;
  }
  static __device__ __forceinline__ u32x4 scale(u32x4 d, u32x4 g, float r) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float xl = __uint_as_float(d[i] << 16);
      const float xh = __uint_as_float(d[i] & 0xffff0000u);
      const float gl = __uint_as_float(g[i] << 16);
      const float gh = __uint_as_float(g[i] & 0xffff0000u);
      const f32x2 yv = {xl * r * gl, xh * r * gh};
      o[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(yv, bf16x2));
    }
    return o;
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

// Sum over the 64 lanes of a wavefront; every lane receives the same value.
// Must be called with all 64 lanes active.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]: pairs
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]: quads
  v += dpp<0x141>(v);  // row_half_mirror: 8 lanes
  v += dpp<0x140>(v);  // row_mirror: 16 lanes (every lane of a row holds the row sum)
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
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
  int rows_per_wg, nwg, nslot, wpr_log2, lay_k, comb_k, slice_vec;
  uint32_t row_bytes, flush_mask;
  float inv_slice_vec, h, eps;

  __device__ __forceinline__ Hot(const Args& a, const Seg& s)
      : x(s.x), y(s.y), gamma(s.gamma), stats_in(s.stats_in), stats_out(s.stats_out),
        x_stride(s.x_stride), y_stride(s.y_stride), T(a.T), rows_per_wg(s.rows_per_wg), nwg(s.nwg),
        nslot(s.nslot), wpr_log2(s.wpr_log2),
        lay_k(s.lay_k), comb_k(s.comb_k), slice_vec(s.slice_vec), row_bytes(s.row_bytes),
        flush_mask(s.flush_mask), inv_slice_vec(s.inv_slice_vec), h(s.h), eps(a.eps) {}
};

// The segment's slot table, read at kernel entry with the other arguments.
template <int VPL>
struct Tables {
  int lim[VPL];
  int base[VPL];
  __device__ __forceinline__ explicit Tables(const Seg& s) {
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      lim[j] = s.slot_lim[j];
      base[j] = s.slot_base[j];
    }
  }
};

// Where this lane's V slots sit in a row of one segment: fixed for the whole
// launch, computed once per wavefront.
template <int V>
struct Layout {
  int wpr_log2, wpr, team, tl;
  uint32_t off[V];  // byte offset of each slot's vector; kOutside when empty
  int base[V];      // vector index of each slot (masked layout)

  template <int VPL>
  __device__ __forceinline__ Layout(const Tables<VPL>& tb, int wl, int wave, int lane) {
    static_assert(V <= VPL, "layout wider than its table");
    wpr_log2 = wl;
    wpr = 1 << wpr_log2;
    team = wave >> wpr_log2;
    tl = ((wave & (wpr - 1)) << 6) | lane;  // lane within the team
#pragma unroll
    for (int j = 0; j < V; ++j) {
      base[j] = tb.base[j];
      const uint32_t o = static_cast<uint32_t>(tb.base[j] + tl) * 16u;
      off[j] = tl < tb.lim[j] ? o : kOutside;
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

// The row statistic S = sum over slices (ascending) of each slice's sum of
// squares. Teams of several wavefronts add their partials through `part`
// (one barrier); every lane of the team returns the same S.
template <class E, int VPL, bool MASKED>
__device__ __forceinline__ float row_stat(const u32x4 (&d)[VPL], const Hot& s, const Layout<VPL>& L,
                                          int wave, int lane, float* part) {
  float S = 0.f;
  if constexpr (!MASKED) {
    // slots are grouped by slice; a set bit in flush_mask closes a slice
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
  } else {
    // plain strided slots; each vector's squares join the partial of the
    // slice its index falls in
    float q[VPL];
    int sid[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      q[j] = E::sumsq(d[j], 0.f);
      sid[j] = slice_of(L.base[j] + L.tl, s.slice_vec, s.inv_slice_vec);
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
    __syncthreads();
    const int w0 = L.team << L.wpr_log2;
    for (int k = 0; k < s.lay_k; ++k) {
      float P = 0.f;
      for (int w = 0; w < L.wpr; ++w) P += part[(w0 + w) * kWave + k];
      S += P;
    }
    __syncthreads();  // `part` is free again
  }
  return S;
}

template <class E, int VPL, bool NT>
__device__ __forceinline__ void scale_store(const u32x4 (&d)[VPL], const u32x4 (&g)[VPL], float S,
                                            float h, float eps, __amdgpu_buffer_rsrc_t yr,
                                            const Layout<VPL>& L) {
  const float r = 1.0f / __builtin_sqrtf(S / h + eps);
#pragma unroll
  for (int j = 0; j < VPL; ++j) store16<NT>(yr, L.off[j], E::scale(d[j], g[j], r));
}

// One row per team: load, statistic, scale, store.
template <class E, int VPL, int MODE, bool MASKED, bool NT>
__device__ __forceinline__ void row_pass(const Hot& s, const Layout<VPL>& L, int gi, int wave, int lane,
                                         float* part) {
  // rows past T read and write nothing (their buffer resources are empty);
  // no branch here, so nothing delays the first loads
  const int64_t row = static_cast<int64_t>(gi) * s.rows_per_wg + L.team;
  const bool live = row < s.T;

  u32x4 d[VPL];
  u32x4 g[VPL];
  load_row<E, VPL, NT>(d, row_rsrc<E>(s.x, s.x_stride, row, live, s.row_bytes), L);
  if constexpr (MODE != MODE_STATS) load_row<E, VPL, false>(g, rsrc(s.gamma, s.row_bytes), L);

  float S = 0.f;
  if constexpr (MODE == MODE_APPLY) {
    // lane k fetches partial k; then they are added in ascending k
    float pk = 0.f;
    if (live && lane < s.comb_k) pk = s.stats_in[static_cast<int64_t>(lane) * s.T + row];
    for (int k = 0; k < s.comb_k; ++k) S += lane_value(pk, k);
  } else {
    S = row_stat<E, VPL, MASKED>(d, s, L, wave, lane, part);
  }

  if constexpr (MODE == MODE_STATS) {
    if (live && L.tl == 0) s.stats_out[row] = S;
  } else {
    scale_store<E, VPL, NT>(d, g, S, s.h, s.eps, row_rsrc<E>(s.y, s.y_stride, row, live, s.row_bytes), L);
  }
}

// Persistent workgroups: group gi, gi + G, gi + 2G, ... (G = gridDim.x). The
// next group's rows are loaded before the current group is reduced and
// stored, so reads of later rows overlap writes of earlier ones; gamma is
// loaded once. Every wavefront of a workgroup runs the same number of
// iterations (rows past T are empty), so barriers stay in step.
template <class E, int VPL, bool MASKED, bool NT>
__device__ __forceinline__ void fwd_pipelined(const Hot& s, const Layout<VPL>& L,
                                              int wave, int lane, float* part) {
  const int G = gridDim.x;
  int g0 = blockIdx.x;
  if (g0 >= s.nwg) return;
  u32x4 A[VPL], B[VPL], g[VPL];
  int64_t ra = static_cast<int64_t>(g0) * s.rows_per_wg + L.team;
  load_row<E, VPL, NT>(A, row_rsrc<E>(s.x, s.x_stride, ra, ra < s.T, s.row_bytes), L);
  load_row<E, VPL, false>(g, rsrc(s.gamma, s.row_bytes), L);
  for (;;) {
    const int g1 = g0 + G;
    const int64_t rb = static_cast<int64_t>(g1) * s.rows_per_wg + L.team;
    load_row<E, VPL, NT>(B, row_rsrc<E>(s.x, s.x_stride, rb, g1 < s.nwg && rb < s.T, s.row_bytes), L);
    float S = row_stat<E, VPL, MASKED>(A, s, L, wave, lane, part);
    scale_store<E, VPL, NT>(A, g, S, s.h, s.eps, row_rsrc<E>(s.y, s.y_stride, ra, ra < s.T, s.row_bytes), L);
    if (g1 >= s.nwg) break;
    const int g2 = g1 + G;
    ra = static_cast<int64_t>(g2) * s.rows_per_wg + L.team;
    load_row<E, VPL, NT>(A, row_rsrc<E>(s.x, s.x_stride, ra, g2 < s.nwg && ra < s.T, s.row_bytes), L);
    S = row_stat<E, VPL, MASKED>(B, s, L, wave, lane, part);
    scale_store<E, VPL, NT>(B, g, S, s.h, s.eps, row_rsrc<E>(s.y, s.y_stride, rb, rb < s.T, s.row_bytes), L);
    if (g2 >= s.nwg) break;
    g0 = g2;
  }
}

template <class E, int V, int VPL, int MODE, bool MASKED, bool NT, bool PIPE>
__device__ __forceinline__ void body(const Hot& s, const Tables<VPL>& tb, int wave, int lane, float* part) {
  const Layout<V> L(tb, s.wpr_log2, wave, lane);
  if constexpr (PIPE) {
    fwd_pipelined<E, V, MASKED, NT>(s, L, wave, lane, part);
  } else {
    // the first group needs no bounds check (a group past the end holds only
    // empty rows), so its loads can follow the argument loads directly
    int gi = blockIdx.x;
    do {
      row_pass<E, V, MODE, MASKED, NT>(s, L, gi, wave, lane, part);
      gi += gridDim.x;
    } while (gi < s.nwg);
  }
}

// The variant is compiled for VPL slots, the widest segment of the launch;
// a narrower segment (the key rows of a grouped-query layout) runs the body
// for VPL/2, VPL/4, ... slots instead, chosen by one uniform branch, so it
// issues no instructions for slots it does not have.
template <class E, int V, int VPL, int MODE, bool MASKED, bool NT, bool PIPE>
__device__ __forceinline__ void dispatch(const Hot& s, const Tables<VPL>& tb, int wave, int lane,
                                         float* part) {
  if constexpr (V > 1) {
    if (s.nslot <= V / 2) {
      dispatch<E, V / 2, VPL, MODE, MASKED, NT, PIPE>(s, tb, wave, lane, part);
      return;
    }
  }
  body<E, V, VPL, MODE, MASKED, NT, PIPE>(s, tb, wave, lane, part);
}

// blockIdx.y selects the segment (query rows, key rows), so everything a
// wavefront needs from the kernel arguments is one round of scalar loads.
template <class E, int VPL, int NW, int MODE, bool MASKED, bool NT, bool PIPE>
__global__ void __launch_bounds__(NW * kWave) qknorm_kernel(const Args a) {
  __shared__ float part[NW * kWave];  // per-wavefront slice partials (teams of > 1 wave)
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  const Seg& seg = a.seg[blockIdx.y];
  const Hot s(a, seg);
  const Tables<VPL> tb(seg);
  dispatch<E, VPL, VPL, MODE, MASKED, NT, PIPE>(s, tb, wave, lane, part);
}

template <class E, int VPL, int NW>
hipError_t launch_vpl(const Variant& v, const Args& a, dim3 gd, hipStream_t st) {
  const dim3 bd(NW * kWave);
  if (v.mode == MODE_FWD) {
    if constexpr (NW == 4) {
      if (v.pipe) {
        if (v.masked)
          hipLaunchKernelGGL((qknorm_kernel<E, VPL, NW, MODE_FWD, true, true, true>), gd, bd, 0, st, a);
        else if (v.nt)
          hipLaunchKernelGGL((qknorm_kernel<E, VPL, NW, MODE_FWD, false, true, true>), gd, bd, 0, st, a);
        else
          hipLaunchKernelGGL((qknorm_kernel<E, VPL, NW, MODE_FWD, false, false, true>), gd, bd, 0, st, a);
        return hipGetLastError();
      }
    }
    if (v.masked)
      hipLaunchKernelGGL((qknorm_kernel<E, VPL, NW, MODE_FWD, true, true, false>), gd, bd, 0, st, a);
    else if (v.nt)
      hipLaunchKernelGGL((qknorm_kernel<E, VPL, NW, MODE_FWD, false, true, false>), gd, bd, 0, st, a);
    else
      hipLaunchKernelGGL((qknorm_kernel<E, VPL, NW, MODE_FWD, false, false, false>), gd, bd, 0, st, a);
  } else if (v.mode == MODE_STATS) {
    hipLaunchKernelGGL((qknorm_kernel<E, VPL, NW, MODE_STATS, false, true, false>), gd, bd, 0, st, a);
  } else {
    hipLaunchKernelGGL((qknorm_kernel<E, VPL, NW, MODE_APPLY, false, true, false>), gd, bd, 0, st, a);
  }
  return hipGetLastError();
}

template <class E>
hipError_t launch_dtype(const Variant& v, const Args& a, dim3 grid, hipStream_t st) {
  if (v.nw == 4) {
    switch (v.vpl) {
      case 1: return launch_vpl<E, 1, 4>(v, a, grid, st);
      case 2: return launch_vpl<E, 2, 4>(v, a, grid, st);
      case 4: return launch_vpl<E, 4, 4>(v, a, grid, st);
      case 6: return launch_vpl<E, 6, 4>(v, a, grid, st);
      case 8: return launch_vpl<E, 8, 4>(v, a, grid, st);
      case 10: return launch_vpl<E, 10, 4>(v, a, grid, st);
      case 12: return launch_vpl<E, 12, 4>(v, a, grid, st);
      case 16: return launch_vpl<E, 16, 4>(v, a, grid, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (v.nw == 16) {
    switch (v.vpl) {
      case 1: return launch_vpl<E, 1, 16>(v, a, grid, st);
      case 2: return launch_vpl<E, 2, 16>(v, a, grid, st);
      case 4: return launch_vpl<E, 4, 16>(v, a, grid, st);
      case 8: return launch_vpl<E, 8, 16>(v, a, grid, st);
      default: return hipErrorInvalidValue;
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

int compiled_vpl(int slots, int nw) {
  static const int k4[] = {1, 2, 4, 6, 8, 10, 12, 16};
  static const int k16[] = {1, 2, 4, 8};
  if (nw == 4) {
    for (int c : k4)
      if (c >= slots) return c;
  } else if (nw == 16) {
    for (int c : k16)
      if (c >= slots) return c;
  }
  return 0;
}

hipError_t launch(const Variant& v, const Args& a, dim3 grid, hipStream_t stream) {
  if (v.dtype == QKNORM_F32) return launch_dtype<F32>(v, a, grid, stream);
  if (v.dtype == QKNORM_BF16) return launch_dtype<BF16>(v, a, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace qkn
