// Host-side memory and undefined-behaviour check, built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py (CPU only).
//
// Part A runs the CPU oracle (oracle/moe_oracle.c) on small random inputs of
// every function it exports and checks a few invariants.  Part B drives the
// host code of the C ABI (argument checks, workspace sizes, the weight-
// gradient split plan) over valid, edge and invalid shapes; no call in it
// reaches a kernel launch, so no GPU is needed.  Exit code 0 = clean.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "../include/moe.h"

extern "C" {
uint16_t oracle_f64_to_bf16(double v);
void oracle_route(int64_t T, int d, int E, int k, const uint16_t* x, const float* w_router,
                  const float* bias, int32_t* idx, float* gate, float* margin, float* scores,
                  int nthreads);
void oracle_seq_balance(int64_t T, int E, int k, int S, const float* scores, const int32_t* idx,
                        double alpha, double* L);
void oracle_permute(int64_t T, int E, int k, const int32_t* idx, int32_t* counts, int32_t* offsets,
                    int32_t* perm_src, int32_t* pos);
void oracle_grouped_ffn(int64_t T, int d, int E, int k, int H, int Hs, const uint16_t* x,
                        const int32_t* perm_src, const int32_t* offsets, const uint16_t* w1,
                        const uint16_t* w3, const uint16_t* w2, const uint16_t* ws1,
                        const uint16_t* ws3, const uint16_t* ws2, uint16_t* y_perm,
                        uint16_t* y_shared, int nthreads);
void oracle_combine(int64_t T, int d, int E, int k, const uint16_t* y_perm, const uint16_t* y_shared,
                    const float* gate, const int32_t* idx, const int32_t* pos,
                    const uint16_t* residual, uint16_t* out);
void oracle_dense_masked(int64_t T, int d, int E, int k, int H, int Hs, const uint16_t* x,
                         const float* gate, const int32_t* idx, const uint16_t* w1,
                         const uint16_t* w3, const uint16_t* w2, const uint16_t* ws1,
                         const uint16_t* ws3, const uint16_t* ws2, const uint16_t* residual,
                         uint16_t* out, int nthreads);
void oracle_rmsnorm(int64_t T, int d, const uint16_t* x, const float* g, double eps, uint16_t* out);
void oracle_update_bias(int64_t T, int E, int k, const int32_t* counts, float* bias, float gamma);
void oracle_moe_backward(int64_t T, int d, int E, int k, int H, int Hs, int S, double alpha,
                         const double* x, const double* wr, const int32_t* idx, const double* w1,
                         const double* w3, const double* w2, const double* ws1, const double* ws3,
                         const double* ws2, const double* dout, int round_storage, double* dx,
                         double* dwr, double* dw1, double* dw3, double* dw2, double* dws1,
                         double* dws3, double* dws2, int nthreads);
void oracle_moe_forward_f64(int64_t T, int d, int E, int k, int H, int Hs, int S, double alpha,
                            const double* x, const double* wr, const int32_t* idx,
                            const double* w1, const double* w3, const double* w2,
                            const double* ws1, const double* ws3, const double* ws2, double* out,
                            double* loss_bal);
}

namespace {
int failures = 0;
#define CHECK(cond)                                                    \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

std::mt19937_64 rng(51);
std::vector<uint16_t> bf16s(size_t n, double scale) {
  std::normal_distribution<double> nd(0.0, scale);
  std::vector<uint16_t> v(n);
  for (auto& e : v) e = oracle_f64_to_bf16(nd(rng));
  return v;
}
std::vector<float> f32s(size_t n, double scale) {
  std::normal_distribution<double> nd(0.0, scale);
  std::vector<float> v(n);
  for (auto& e : v) e = static_cast<float>(nd(rng));
  return v;
}
std::vector<double> f64s(size_t n, double scale) {
  std::normal_distribution<double> nd(0.0, scale);
  std::vector<double> v(n);
  for (auto& e : v) e = nd(rng);
  return v;
}

void oracle_part() {
  const int64_t T = 36;
  const int d = 16, E = 5, k = 2, H = 8, Hs = 8, S = 12;
  auto x = bf16s(T * d, 1.0);
  auto wr = f32s(static_cast<size_t>(d) * E, 0.3);
  auto bias = f32s(E, 0.05);
  std::vector<int32_t> idx(T * k), counts(E), offsets(E + 1), perm(T * k), pos(T * k);
  std::vector<float> gate(T * k), margin(T), scores(T * E);
  oracle_route(T, d, E, k, x.data(), wr.data(), bias.data(), idx.data(), gate.data(), margin.data(),
               scores.data(), 2);
  for (int64_t t = 0; t < T; ++t) {
    double s = 0;
    for (int j = 0; j < k; ++j) s += gate[t * k + j];
    CHECK(std::fabs(s - 1.0) < 1e-5);
  }
  std::vector<double> L(T / S);  // one value per sequence
  oracle_seq_balance(T, E, k, S, scores.data(), idx.data(), 1e-4, L.data());
  for (double v : L) CHECK(std::isfinite(v));
  oracle_permute(T, E, k, idx.data(), counts.data(), offsets.data(), perm.data(), pos.data());
  CHECK(offsets[E] == T * k);
  auto w1 = bf16s(static_cast<size_t>(E) * H * d, 0.2), w3 = bf16s(static_cast<size_t>(E) * H * d, 0.2);
  auto w2 = bf16s(static_cast<size_t>(E) * d * H, 0.2);
  auto ws1 = bf16s(static_cast<size_t>(Hs) * d, 0.2), ws3 = bf16s(static_cast<size_t>(Hs) * d, 0.2);
  auto ws2 = bf16s(static_cast<size_t>(d) * Hs, 0.2);
  std::vector<uint16_t> y_perm(T * k * d), y_shared(T * d), out(T * d), dense(T * d);
  oracle_grouped_ffn(T, d, E, k, H, Hs, x.data(), perm.data(), offsets.data(), w1.data(), w3.data(),
                     w2.data(), ws1.data(), ws3.data(), ws2.data(), y_perm.data(), y_shared.data(), 2);
  oracle_combine(T, d, E, k, y_perm.data(), y_shared.data(), gate.data(), idx.data(), pos.data(),
                 x.data(), out.data());
  oracle_dense_masked(T, d, E, k, H, Hs, x.data(), gate.data(), idx.data(), w1.data(), w3.data(),
                      w2.data(), ws1.data(), ws3.data(), ws2.data(), x.data(), dense.data(), 2);
  CHECK(std::memcmp(out.data(), dense.data(), out.size() * 2) == 0);
  std::vector<float> g(d, 1.0f);
  std::vector<uint16_t> xn(T * d);
  oracle_rmsnorm(T, d, x.data(), g.data(), 1e-6, xn.data());
  auto b2 = bias;
  oracle_update_bias(T, E, k, counts.data(), b2.data(), 1e-3f);
  // backward and the fp64 forward, with and without the shared expert
  for (int hs : {Hs, 0}) {
    auto xd = f64s(T * d, 1.0), wrd = f64s(static_cast<size_t>(d) * E, 0.3);
    auto w1d = f64s(static_cast<size_t>(E) * H * d, 0.2), w3d = f64s(static_cast<size_t>(E) * H * d, 0.2);
    auto w2d = f64s(static_cast<size_t>(E) * d * H, 0.2), dout = f64s(T * d, 1.0);
    auto ws1d = f64s(static_cast<size_t>(Hs) * d, 0.2), ws3d = f64s(static_cast<size_t>(Hs) * d, 0.2);
    auto ws2d = f64s(static_cast<size_t>(d) * Hs, 0.2);
    std::vector<double> dx(T * d), dwr(static_cast<size_t>(d) * E), dw1(w1d.size()), dw3(w3d.size()),
        dw2(w2d.size()), dws1(ws1d.size()), dws3(ws3d.size()), dws2(ws2d.size()), o(T * d);
    const double* s1 = hs ? ws1d.data() : nullptr;
    const double* s3 = hs ? ws3d.data() : nullptr;
    const double* s2 = hs ? ws2d.data() : nullptr;
    for (int round = 0; round < 2; ++round)
      oracle_moe_backward(T, d, E, k, H, hs, S, 0.3, xd.data(), wrd.data(), idx.data(), w1d.data(),
                          w3d.data(), w2d.data(), s1, s3, s2, dout.data(), round, dx.data(), dwr.data(),
                          dw1.data(), dw3.data(), dw2.data(), hs ? dws1.data() : nullptr,
                          hs ? dws3.data() : nullptr, hs ? dws2.data() : nullptr, 2);
    double lb = 0;
    oracle_moe_forward_f64(T, d, E, k, H, hs, S, 0.3, xd.data(), wrd.data(), idx.data(), w1d.data(),
                           w3d.data(), w2d.data(), s1, s3, s2, o.data(), &lb);
    CHECK(std::isfinite(lb) && std::isfinite(dx[0]));
  }
}

moe_shape shape_of(int64_t T, int d, int E, int k, int H, int Hs, int S) {
  moe_shape s;
  s.tokens = T;
  s.d_model = d;
  s.n_experts = E;
  s.top_k = k;
  s.hidden = H;
  s.shared_hidden = Hs;
  s.seq_len = S;
  return s;
}

void abi_part() {
  // workspace sizes over valid and edge shapes (the split plan included)
  const moe_shape shapes[] = {
      shape_of(0, 64, 1, 1, 64, 0, 0),          shape_of(1, 64, 1, 1, 64, 64, 1),
      shape_of(2048, 384, 16, 4, 256, 256, 256), shape_of(8192, 384, 16, 4, 256, 256, 256),
      shape_of(4096, 7168, 256, 8, 2048, 2048, 4096), shape_of(64, 7168, 256, 8, 2048, 2048, 0),
      shape_of(4096, 7168, 32, 8, 2048, 2048, 4096), shape_of(4096, 384, 8, 2, 256, 256, 128),
      shape_of(18000, 7168, 256, 8, 2048, 2048, 0), shape_of(100000, 64, 1024, 32, 64, 64, 0),
      shape_of(1600, 128, 4, 2, 128, 192, 320)};
  for (const moe_shape& s : shapes) {
    size_t fw = 0, bw = 0;
    CHECK(moe_workspace_bytes(&s, &fw) == MOE_OK);
    CHECK(moe_backward_workspace_bytes(&s, &bw) == MOE_OK);
    CHECK(fw % 256 == 0 && bw % 256 == 0);
  }
  // invalid shapes
  const moe_shape bad[] = {shape_of(-1, 64, 4, 2, 64, 64, 0), shape_of(8, 0, 4, 2, 64, 64, 0),
                           shape_of(8, 64, 4, 5, 64, 64, 0), shape_of(9, 64, 4, 2, 64, 64, 4),
                           shape_of(8, 60, 4, 2, 64, 64, 0), shape_of(8, 64, 2000, 2, 64, 64, 0),
                           shape_of(149797, 7168, 256, 8, 2048, 2048, 0)};
  for (const moe_shape& s : bad) {
    size_t b = 0;
    CHECK(moe_workspace_bytes(&s, &b) != MOE_OK);
    CHECK(moe_backward_workspace_bytes(&s, &b) != MOE_OK);
  }
  {  // x_perm and h beyond 2 GiB: the forward takes it, the backward does not
    const moe_shape wide = shape_of(20000, 7168, 256, 8, 2048, 2048, 0);
    size_t b = 0;
    CHECK(moe_workspace_bytes(&wide, &b) == MOE_OK && b % 256 == 0);
    CHECK(moe_backward_workspace_bytes(&wide, &b) == MOE_ERR_UNSUPPORTED);
  }
  size_t b = 0;
  CHECK(moe_workspace_bytes(nullptr, &b) == MOE_ERR_INVALID_ARGUMENT);
  CHECK(moe_workspace_bytes(&shapes[2], nullptr) == MOE_ERR_INVALID_ARGUMENT);
  CHECK(std::strlen(moe_status_str(MOE_ERR_SCRATCH_LIMIT)) > 0);
  CHECK(std::strlen(moe_status_str(12345)) > 0);
  // every entry point refuses missing arguments before touching a device
  const moe_shape& s = shapes[2];
  alignas(256) static unsigned char buf[1 << 12];
  void* p = buf;
  auto u16 = static_cast<uint16_t*>(p);
  auto f32 = static_cast<float*>(p);
  auto i32 = static_cast<int32_t*>(p);
  const uint16_t* odd = reinterpret_cast<const uint16_t*>(buf + 2);
  CHECK(moe_route(&s, nullptr, f32, f32, i32, f32, f32, f32, 1e-4f, p, sizeof buf, nullptr) ==
        MOE_ERR_INVALID_ARGUMENT);
  CHECK(moe_route(&s, odd, f32, f32, i32, f32, f32, f32, 1e-4f, p, sizeof buf, nullptr) != MOE_OK);
  CHECK(moe_route(&s, u16, f32, f32, i32, f32, f32, f32, 1e-4f, p, 16, nullptr) == MOE_ERR_WORKSPACE);
  CHECK(moe_permute(&s, i32, nullptr, i32, i32, i32, nullptr, nullptr, p, sizeof buf, nullptr) ==
        MOE_ERR_INVALID_ARGUMENT);
  CHECK(moe_permute_noalloc(&s, i32, nullptr, i32, i32, i32, nullptr, nullptr, nullptr) ==
        MOE_ERR_INVALID_ARGUMENT);
  const moe_shape huge = shape_of(1000000, 64, 1024, 1, 64, 64, 0);
  CHECK(moe_permute_noalloc(&huge, i32, i32, i32, i32, i32, nullptr, nullptr, nullptr) ==
        MOE_ERR_SCRATCH_LIMIT);
  CHECK(moe_grouped_ffn(&s, u16, nullptr, i32, i32, nullptr, u16, u16, u16, u16, u16, u16, u16, p,
                        sizeof buf, nullptr) == MOE_ERR_INVALID_ARGUMENT);
  CHECK(moe_combine(&s, nullptr, u16, f32, i32, nullptr, u16, nullptr) == MOE_ERR_INVALID_ARGUMENT);
  CHECK(moe_rmsnorm(&s, u16, f32, -1.0f, u16, nullptr) == MOE_ERR_INVALID_ARGUMENT);
  CHECK(moe_update_bias(&s, nullptr, f32, 1e-3f, nullptr) == MOE_ERR_INVALID_ARGUMENT);
  CHECK(moe_combine_backward(&s, u16, nullptr, f32, i32, u16, f32, nullptr) ==
        MOE_ERR_INVALID_ARGUMENT);
  CHECK(moe_grouped_ffn_backward(&s, u16, u16, i32, u16, u16, u16, u16, u16, u16, u16, u16, u16,
                                 u16, nullptr, f32, f32, f32, f32, f32, p, sizeof buf, nullptr) ==
        MOE_ERR_INVALID_ARGUMENT);
  CHECK(moe_grouped_ffn_backward(&s, u16, u16, i32, u16, u16, u16, u16, u16, u16, u16, u16, u16,
                                 u16, f32, f32, f32, f32, f32, f32, p, 16, nullptr) ==
        MOE_ERR_WORKSPACE);
  CHECK(moe_route_backward(&s, u16, f32, i32, f32, f32, -1.0f, u16, u16, i32, nullptr, u16, f32, p,
                           sizeof buf, nullptr) == MOE_ERR_INVALID_ARGUMENT);
}
}  // namespace

int main() {
  oracle_part();
  abi_part();
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("host sanitizer check: clean\n");
  return 0;
}
