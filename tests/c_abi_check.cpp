// A C++ caller of libqknorm through include/qknorm.h alone (no Python): device
// buffers from hipMalloc, then every entry point the header declares on fp32
// rows (the fused forward with default and forced options, the headwise
// form, the inverse RMS, the split path one tensor at a time and both
// tensors at once), checked element by element against the fp64 oracle
// (oracle/qknorm_oracle.c, linked as test infrastructure), plus error codes,
// status strings and width limits. Prints "c_abi_check: ok" and exits 0 on
// success.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "qknorm.h"

extern "C" void oracle_forward(const float* x, int64_t T, int64_t H, int64_t ldx, const float* gamma, double eps,
                               int K, double* P, double* y, int64_t ldy);
extern "C" void oracle_inv_rms(const float* x, int64_t T, int64_t H, int64_t ldx, int K, double eps, double* P,
                               double* r);
extern "C" void oracle_headwise(const float* x, int64_t T, int64_t H, int64_t ldx, int64_t D, const float* gamma,
                                double eps, double* y, int64_t ldy);

static int failures = 0;
#define EXPECT(c, ...)                  \
  do {                                  \
    if (!(c)) {                         \
      std::printf("FAIL %s: ", #c);     \
      std::printf(__VA_ARGS__);         \
      std::printf("\n");                \
      ++failures;                       \
    }                                   \
  } while (0)
#define HIP(x)                                                                     \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);   \
      return 2;                                                                    \
    }                                                                              \
  } while (0)

// a fixed, seedless pattern: values of both signs and several magnitudes
static float value(int64_t t, int64_t j, int which) {
  const double u = std::sin(0.37 * (double)(j + 1) + 1.3 * (double)t + 0.5 * which);
  return (float)(u * (1.0 + (double)((j + 3 * t) % 7)));
}

static bool close_f32(double got, double want) { return std::fabs(got - want) <= 1e-5 * std::fabs(want); }

int main() {
  const int64_t T = 37, Hq = 1024, Hk = 256;
  const int K = 4;
  const float eps = 1e-6f;
  std::vector<float> q(T * Hq), k(T * Hk), gq(Hq), gk(Hk);
  for (int64_t t = 0; t < T; ++t) {
    for (int64_t j = 0; j < Hq; ++j) q[t * Hq + j] = value(t, j, 0);
    for (int64_t j = 0; j < Hk; ++j) k[t * Hk + j] = value(t, j, 1);
  }
  for (int64_t j = 0; j < Hq; ++j) gq[j] = 0.5f + (float)(j % 11) / 10.0f;
  for (int64_t j = 0; j < Hk; ++j) gk[j] = 1.5f - (float)(j % 5) / 8.0f;

  float *dq, *dk, *dyq, *dyk, *dgq, *dgk, *dstats, *drq, *drk;
  HIP(hipMalloc(&dq, q.size() * 4));
  HIP(hipMalloc(&dk, k.size() * 4));
  HIP(hipMalloc(&dyq, q.size() * 4));
  HIP(hipMalloc(&dyk, k.size() * 4));
  HIP(hipMalloc(&dgq, gq.size() * 4));
  HIP(hipMalloc(&dgk, gk.size() * 4));
  HIP(hipMalloc(&dstats, K * T * 4));
  HIP(hipMalloc(&drq, T * 4));
  HIP(hipMalloc(&drk, T * 4));
  HIP(hipMemcpy(dq, q.data(), q.size() * 4, hipMemcpyHostToDevice));
  HIP(hipMemcpy(dk, k.data(), k.size() * 4, hipMemcpyHostToDevice));
  HIP(hipMemcpy(dgq, gq.data(), gq.size() * 4, hipMemcpyHostToDevice));
  HIP(hipMemcpy(dgk, gk.data(), gk.size() * 4, hipMemcpyHostToDevice));

  qknorm_ctx* ctx = nullptr;
  EXPECT(qknorm_create(&ctx, 0) == QKNORM_OK, "create");
  EXPECT(qknorm_create(nullptr, 0) == QKNORM_ERR_NULL, "create(NULL)");
  qknorm_ctx* bad = nullptr;
  EXPECT(qknorm_create(&bad, 1000) == QKNORM_ERR_DEVICE && bad == nullptr, "create on a missing device");
  hipStream_t stream;
  HIP(hipStreamCreate(&stream));

  qknorm_rows rq{dq, dyq, Hq, Hq, Hq}, rk{dk, dyk, Hk, Hk, Hk};
  EXPECT(qknorm_forward(ctx, QKNORM_F32, T, &rq, &rk, dgq, dgk, eps, K, stream) == QKNORM_OK, "forward");
  EXPECT(qknorm_inv_rms(ctx, QKNORM_F32, T, &rq, &rk, eps, K, drq, drk, stream) == QKNORM_OK, "inv_rms");
  // error paths: nothing is enqueued
  EXPECT(qknorm_forward(ctx, 7, T, &rq, &rk, dgq, dgk, eps, K, stream) == QKNORM_ERR_DTYPE, "dtype");
  EXPECT(qknorm_forward(ctx, QKNORM_F32, T, &rq, &rk, dgq, dgk, eps, 3, stream) == QKNORM_ERR_SLICES, "slices");
  EXPECT(qknorm_forward(ctx, QKNORM_F32, T, &rq, &rk, dgq, dgk, -1.0f, K, stream) == QKNORM_ERR_EPS, "eps");
  EXPECT(qknorm_forward(nullptr, QKNORM_F32, T, &rq, &rk, dgq, dgk, eps, K, stream) == QKNORM_ERR_CONTEXT, "ctx");
  EXPECT(qknorm_forward(ctx, QKNORM_F32, 0, nullptr, nullptr, nullptr, nullptr, eps, K, stream) == QKNORM_OK,
         "T = 0");
  HIP(hipStreamSynchronize(stream));

  std::vector<float> yq(q.size()), yk(k.size()), gotr(T);
  HIP(hipMemcpy(yq.data(), dyq, yq.size() * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(yk.data(), dyk, yk.size() * 4, hipMemcpyDeviceToHost));
  std::vector<double> P(K * T), refq(q.size()), refk(k.size()), refr(T);
  oracle_forward(q.data(), T, Hq, Hq, gq.data(), (double)eps, K, P.data(), refq.data(), Hq);
  oracle_forward(k.data(), T, Hk, Hk, gk.data(), (double)eps, K, P.data(), refk.data(), Hk);
  int bad_q = 0, bad_k = 0;
  for (size_t i = 0; i < yq.size(); ++i) bad_q += !close_f32(yq[i], refq[i]);
  for (size_t i = 0; i < yk.size(); ++i) bad_k += !close_f32(yk[i], refk[i]);
  EXPECT(bad_q == 0, "%d query elements outside 1e-5", bad_q);
  EXPECT(bad_k == 0, "%d key elements outside 1e-5", bad_k);
  HIP(hipMemcpy(gotr.data(), drq, T * 4, hipMemcpyDeviceToHost));
  oracle_inv_rms(q.data(), T, Hq, Hq, K, (double)eps, P.data(), refr.data());
  for (int64_t t = 0; t < T; ++t) EXPECT(close_f32(gotr[t], refr[t]), "rinv[%lld]", (long long)t);

  // split path over the query rows: K partial-sum calls, then K applies in place
  const int64_t w = Hq / K;
  for (int s = 0; s < K; ++s)
    EXPECT(qknorm_partial_stats(ctx, QKNORM_F32, T, dq + s * w, Hq, w, s, K, dstats, stream) == QKNORM_OK, "stats");
  for (int s = 0; s < K; ++s) {
    qknorm_rows r{dq + s * w, dq + s * w, w, Hq, Hq};
    EXPECT(qknorm_apply_stats(ctx, QKNORM_F32, T, &r, dgq + s * w, dstats, K, Hq, eps, stream) == QKNORM_OK,
           "apply");
  }
  HIP(hipStreamSynchronize(stream));
  HIP(hipMemcpy(yq.data(), dq, yq.size() * 4, hipMemcpyDeviceToHost));
  bad_q = 0;
  for (size_t i = 0; i < yq.size(); ++i) bad_q += !close_f32(yq[i], refq[i]);
  EXPECT(bad_q == 0, "%d split-path elements outside 1e-5", bad_q);

  // headwise: heads of 64 columns, weights shared by the heads of a tensor
  const int64_t D = 64;
  std::vector<float> hq(D), hk(D);
  for (int64_t j = 0; j < D; ++j) {
    hq[j] = 0.75f + (float)(j % 9) / 16.0f;
    hk[j] = 1.25f - (float)(j % 3) / 4.0f;
  }
  float *dhq, *dhk;
  HIP(hipMalloc(&dhq, D * 4));
  HIP(hipMalloc(&dhk, D * 4));
  HIP(hipMemcpy(dhq, hq.data(), D * 4, hipMemcpyHostToDevice));
  HIP(hipMemcpy(dhk, hk.data(), D * 4, hipMemcpyHostToDevice));
  HIP(hipMemcpy(dq, q.data(), q.size() * 4, hipMemcpyHostToDevice));  // the split path above wrote in place
  EXPECT(qknorm_forward_headwise(ctx, QKNORM_F32, T, &rq, &rk, dhq, dhk, D, eps, stream) == QKNORM_OK, "headwise");
  EXPECT(qknorm_forward_headwise(ctx, QKNORM_F32, T, &rq, &rk, dhq, dhk, 48, eps, stream) == QKNORM_ERR_SLICES,
         "headwise with a head that is not a power of two of vectors");
  HIP(hipStreamSynchronize(stream));
  HIP(hipMemcpy(yq.data(), dyq, yq.size() * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(yk.data(), dyk, yk.size() * 4, hipMemcpyDeviceToHost));
  std::vector<double> hrefq(q.size()), hrefk(k.size());
  oracle_headwise(q.data(), T, Hq, Hq, D, hq.data(), (double)eps, hrefq.data(), Hq);
  oracle_headwise(k.data(), T, Hk, Hk, D, hk.data(), (double)eps, hrefk.data(), Hk);
  bad_q = bad_k = 0;
  for (size_t i = 0; i < yq.size(); ++i) bad_q += !close_f32(yq[i], hrefq[i]);
  for (size_t i = 0; i < yk.size(); ++i) bad_k += !close_f32(yk[i], hrefk[i]);
  EXPECT(bad_q == 0 && bad_k == 0, "headwise: %d query, %d key elements outside 1e-5", bad_q, bad_k);

  // split path over both tensors at once: K statistics launches, K applies
  // (out of place), each taking a query slice and a key slice
  float *dstats_k;
  HIP(hipMalloc(&dstats_k, K * T * 4));
  const int64_t wk = Hk / K;
  for (int s = 0; s < K; ++s) {
    qknorm_rows sq{dq + s * w, nullptr, w, Hq, 0}, sk{dk + s * wk, nullptr, wk, Hk, 0};
    EXPECT(qknorm_partial_stats_qk(ctx, QKNORM_F32, T, &sq, &sk, s, K, dstats, dstats_k, stream) == QKNORM_OK,
           "stats_qk");
  }
  for (int s = 0; s < K; ++s) {
    qknorm_rows aq{dq + s * w, dyq + s * w, w, Hq, Hq}, ak{dk + s * wk, dyk + s * wk, wk, Hk, Hk};
    EXPECT(qknorm_apply_stats_qk(ctx, QKNORM_F32, T, &aq, &ak, dgq + s * w, dgk + s * wk, dstats, dstats_k, K, Hq,
                                 Hk, eps, stream) == QKNORM_OK,
           "apply_qk");
  }
  {
    qknorm_rows sq{dq, nullptr, w, Hq, 0};
    EXPECT(qknorm_partial_stats_qk(ctx, QKNORM_F32, T, &sq, nullptr, K, K, dstats, nullptr, stream) ==
               QKNORM_ERR_SLICES,
           "stats_qk with a slice index past the last slice");
  }
  HIP(hipStreamSynchronize(stream));
  HIP(hipMemcpy(yq.data(), dyq, yq.size() * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(yk.data(), dyk, yk.size() * 4, hipMemcpyDeviceToHost));
  bad_q = bad_k = 0;
  for (size_t i = 0; i < yq.size(); ++i) bad_q += !close_f32(yq[i], refq[i]);
  for (size_t i = 0; i < yk.size(); ++i) bad_k += !close_f32(yk[i], refk[i]);
  EXPECT(bad_q == 0 && bad_k == 0, "split path, both tensors: %d query, %d key elements outside 1e-5", bad_q, bad_k);

  // a context with forced options: two wavefronts per row, a capped grid
  qknorm_options opts{2, 7, 0};
  qknorm_ctx* ctx2 = nullptr;
  EXPECT(qknorm_create_ex(&ctx2, 0, &opts) == QKNORM_OK, "create_ex");
  qknorm_options bad_opts{3, 0, 0};
  qknorm_ctx* ctx3 = nullptr;
  EXPECT(qknorm_create_ex(&ctx3, 0, &bad_opts) != QKNORM_OK && ctx3 == nullptr, "create_ex with 3 waves per row");
  EXPECT(qknorm_forward(ctx2, QKNORM_F32, T, &rq, &rk, dgq, dgk, eps, K, stream) == QKNORM_OK, "forward, forced");
  HIP(hipStreamSynchronize(stream));
  HIP(hipMemcpy(yq.data(), dyq, yq.size() * 4, hipMemcpyDeviceToHost));
  HIP(hipMemcpy(yk.data(), dyk, yk.size() * 4, hipMemcpyDeviceToHost));
  bad_q = bad_k = 0;
  for (size_t i = 0; i < yq.size(); ++i) bad_q += !close_f32(yq[i], refq[i]);
  for (size_t i = 0; i < yk.size(); ++i) bad_k += !close_f32(yk[i], refk[i]);
  EXPECT(bad_q == 0 && bad_k == 0, "forced options: %d query, %d key elements outside 1e-5", bad_q, bad_k);
  EXPECT(qknorm_destroy(ctx2) == QKNORM_OK, "destroy ctx2");

  // status strings and width limits
  for (int st : {(int)QKNORM_OK, (int)QKNORM_ERR_NULL, (int)QKNORM_ERR_DTYPE, (int)QKNORM_ERR_SLICES,
                 (int)QKNORM_ERR_CONTEXT, -12345})
    EXPECT(qknorm_status_string(st) != nullptr && qknorm_status_string(st)[0] != 0, "status string %d", st);
  EXPECT(qknorm_max_width(QKNORM_F32) == 32768 && qknorm_max_width(QKNORM_BF16) == 65536 &&
             qknorm_max_width(QKNORM_FP8_E4M3) == 65536 && qknorm_max_width(7) == 0,
         "max widths");

  HIP(hipFree(dhq));
  HIP(hipFree(dhk));
  HIP(hipFree(dstats_k));
  EXPECT(qknorm_destroy(ctx) == QKNORM_OK, "destroy");
  EXPECT(qknorm_destroy(nullptr) == QKNORM_OK, "destroy(NULL)");
  HIP(hipStreamDestroy(stream));
  for (float* p : {dq, dk, dyq, dyk, dgq, dgk, dstats, drq, drk}) HIP(hipFree(p));
  if (failures) {
    std::printf("c_abi_check: %d failures\n", failures);
    return 1;
  }
  std::printf("c_abi_check: ok\n");
  return 0;
}
