// abi_sanitize.cpp -- host-side checks of the C ABI's validation paths and of
// the oracle, built with AddressSanitizer and UndefinedBehaviorSanitizer on
// the host code (no kernel is ever launched: every call below is refused
// before a launch or is host-only).
// Run by tests/test_sanitize.py; exits non-zero (or the sanitizer aborts) on
// the first failure.

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "dcn.h"
#include "dcn_oracle.h"

#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #c); \
      return 1;                                                         \
    }                                                                   \
  } while (0)

namespace {

dcn_desc desc(int B, int C, int H, int W, int O, int kh, int kw, int ph, int pw,
              int dt = DCN_F32, int lay = DCN_OUT_NCHW, int odt = DCN_F32) {
  return dcn_desc{B, C, H, W, O, kh, kw, ph, pw, dt, odt, lay};
}

int abi_checks() {
  void* const fake = reinterpret_cast<void*>(0x10000);
  void* const odd = reinterpret_cast<void*>(0x10004);
  // descriptors
  const dcn_desc good[] = {desc(1, 64, 16, 16, 64, 3, 3, 1, 1), desc(0, 8, 4, 4, 8, 1, 1, 0, 0),
                           desc(2, 8, 5, 7, 300, 2, 4, 0, 1, DCN_BF16, DCN_OUT_NHWC),
                           desc(1, 64, 128, 128, 64, 7, 7, 3, 3)};
  for (const dcn_desc& d : good) {
    dcn_plan p = nullptr;
    CHECK(dcn_create(&d, &p) == DCN_OK && p != nullptr);
    size_t ws = 0, pw = 0, bw = 0;
    int32_t ho = 0, wo = 0;
    CHECK(dcn_workspace_bytes(p, &ws) == DCN_OK);
    CHECK(dcn_packed_weight_bytes(p, &pw) == DCN_OK && pw <= ws && pw % 256 == 0);
    CHECK(dcn_backward_workspace_bytes(p, &bw) == DCN_OK && bw > 0);
    CHECK(dcn_output_size(p, &ho, &wo) == DCN_OK && ho > 0 && wo > 0);
    if (d.batch > 0) {
      // refused before any launch: NULL / misaligned pointers, short workspaces
      CHECK(dcn_forward_packed(p, nullptr, fake, nullptr, fake, ws, nullptr, fake, nullptr) ==
            DCN_E_NULL);
      CHECK(dcn_forward_packed(p, fake, fake, nullptr, fake, pw - 1, nullptr, fake, nullptr) ==
            DCN_E_WORKSPACE);
      CHECK(dcn_forward_packed(p, odd, fake, nullptr, fake, ws, nullptr, fake, nullptr) ==
            DCN_E_ALIGN);
      CHECK(dcn_forward_rows(p, -1, 1, fake, fake, nullptr, fake, ws, nullptr, fake, nullptr) ==
            DCN_E_SHAPE);
      CHECK(dcn_forward_rows(p, 0, ho + 1, fake, fake, nullptr, fake, ws, nullptr, fake,
                             nullptr) == DCN_E_SHAPE);
      CHECK(dcn_pack_weight(p, nullptr, fake, ws, nullptr) == DCN_E_NULL);
      CHECK(dcn_pack_weight(p, fake, fake, pw - 1, nullptr) == DCN_E_WORKSPACE);
      CHECK(dcn_backward(p, nullptr, fake, nullptr, fake, fake, nullptr, nullptr, nullptr,
                         nullptr, nullptr, fake, bw, nullptr) != DCN_OK);
      CHECK(dcn_backward(p, fake, fake, nullptr, fake, fake, nullptr, nullptr, nullptr, nullptr,
                         nullptr, fake, bw - 1, nullptr) != DCN_OK);
      CHECK(dcn_debug_coords(p, nullptr, nullptr, nullptr, nullptr) == DCN_E_NULL);
      CHECK(dcn_debug_corner_table(p, fake, fake, nullptr, fake, ws, nullptr, fake, nullptr,
                                   nullptr, nullptr) == DCN_E_NULL);
    }
    dcn_plan plans[2] = {p, p};
    const void* offs[2] = {fake, fake};
    CHECK(dcn_forward_multi(9, plans, fake, offs, nullptr, offs, &ws, nullptr, nullptr,
                            nullptr) == DCN_E_UNSUPPORTED);
    CHECK(dcn_forward_multi(2, plans, fake, nullptr, nullptr, offs, &ws, nullptr, nullptr,
                            nullptr) == DCN_E_NULL);
    CHECK(dcn_destroy(p) == DCN_OK);
  }
  const dcn_desc bad[] = {desc(-1, 8, 4, 4, 8, 1, 1, 0, 0), desc(1, 0, 4, 4, 8, 1, 1, 0, 0),
                          desc(1, 8, 2, 2, 8, 5, 5, 1, 1), desc(1, 6, 4, 4, 8, 1, 1, 0, 0),
                          desc(1, 12, 4, 4, 8, 1, 1, 0, 0, DCN_BF16), desc(1, 8, 4, 4, 8, 1, 1, 0, 0, 7),
                          desc(1, 8, 4, 4, 8, 1, 1, 0, 0, DCN_F32, 9),
                          desc(1, 8, 4, 4, 8, 1, 1, 0, 0, DCN_F32, DCN_OUT_NCHW, DCN_BF16),
                          desc(1024, 4, 1024, 1024, 4, 1, 1, 0, 0)};
  for (const dcn_desc& d : bad) {
    dcn_plan p = reinterpret_cast<dcn_plan>(fake);
    CHECK(dcn_create(&d, &p) != DCN_OK && p == nullptr);
    CHECK(std::strlen(dcn_last_error()) > 0);
  }
  CHECK(dcn_create(nullptr, nullptr) == DCN_E_NULL);
  CHECK(dcn_destroy(nullptr) == DCN_OK);
  for (int s = 0; s <= 9; ++s) CHECK(dcn_status_string(static_cast<dcn_status>(s)) != nullptr);
  CHECK(dcn_version() > 0);
  CHECK(dcn_nchw_to_nhwc(fake, fake, 1, -4, 4, 4, DCN_F32, nullptr) == DCN_E_SHAPE);
  CHECK(dcn_nchw_to_nhwc(odd, fake, 1, 4, 4, 4, DCN_BF16, nullptr) == DCN_E_ALIGN);

  // multi-scale deformable attention
  const int32_t hw[4] = {8, 8, 4, 4};
  dcn_msda_desc md = {2, 10, 8, 32, 2, 4, DCN_BF16, 1};
  dcn_msda_plan mp = nullptr;
  CHECK(dcn_msda_create(&md, hw, &mp) == DCN_OK);
  int32_t S = 0;
  CHECK(dcn_msda_value_positions(mp, &S) == DCN_OK && S == 80);
  CHECK(dcn_msda_forward(mp, nullptr, fake, fake, fake, nullptr) == DCN_E_NULL);
  CHECK(dcn_msda_forward(mp, fake, reinterpret_cast<void*>(0x10001), fake, fake, nullptr) ==
        DCN_E_ALIGN);
  CHECK(dcn_msda_destroy(mp) == DCN_OK);
  md.head_dim = 12;  // not a multiple of 8 for bf16
  CHECK(dcn_msda_create(&md, hw, &mp) == DCN_E_UNSUPPORTED && mp == nullptr);

  // single-scale deformable sampling
  dcn_dsample_desc dd = {1, 4, 16, 32, 32, 3, 3, 1, 1, DCN_F32, 1, DCN_OUT_NHWC};
  dcn_dsample_plan dp = nullptr;
  CHECK(dcn_dsample_create(&dd, &dp) == DCN_OK);
  int32_t dho = 0, dwo = 0;
  CHECK(dcn_dsample_output_size(dp, &dho, &dwo) == DCN_OK && dho == 32 && dwo == 32);
  CHECK(dcn_dsample_forward(dp, nullptr, fake, fake, fake, nullptr) == DCN_E_NULL);
  CHECK(dcn_dsample_forward(dp, odd, fake, fake, fake, nullptr) == DCN_E_ALIGN);
  CHECK(dcn_dsample_destroy(dp) == DCN_OK);
  dd.group_ch = 6;
  CHECK(dcn_dsample_create(&dd, &dp) == DCN_E_UNSUPPORTED && dp == nullptr);
  return 0;
}

int oracle_checks() {
  std::mt19937 rng(7);
  std::normal_distribution<float> n01(0.f, 1.f);
  auto fill = [&](std::vector<float>& v, float s) {
    for (float& e : v) e = n01(rng) * s;
  };
  // forward, coords, backward on a small padded 3x3 problem
  dcn_oracle_shape s = {2, 4, 5, 6, 3, 3, 3, 1, 1};
  const int64_t K = 9, Ho = 5, Wo = 6, P = 2 * Ho * Wo;
  std::vector<float> x(2 * 5 * 6 * 4), off(2 * 2 * K * Ho * Wo), m(2 * K * Ho * Wo),
      w(3 * 4 * K), b(3), g(2 * 3 * Ho * Wo);
  fill(x, 1.f);
  fill(off, 3.f);
  fill(m, 1.f);
  fill(w, 0.3f);
  fill(b, 0.1f);
  fill(g, 1.f);
  off[0] = 1e30f;  // a point far outside
  std::vector<double> out(P * 3), norm(P * 3);
  CHECK(dcn_oracle_forward(&s, x.data(), off.data(), m.data(), w.data(), b.data(), nullptr, P,
                           out.data(), norm.data(), 3) == 0);
  for (int64_t e = 0; e < P * 3; ++e) CHECK(std::isfinite(out[e]) && norm[e] >= 0.0);
  std::vector<int32_t> yx(2 * K * Ho * Wo * 2);
  std::vector<uint8_t> v4(2 * K * Ho * Wo);
  CHECK(dcn_oracle_coords(&s, off.data(), yx.data(), v4.data(), 2) == 0);
  CHECK(v4[0] == 0);
  std::vector<double> gx(x.size()), go(off.size()), gm(m.size()), gw(w.size()), gb(3);
  std::vector<double> nx(x.size()), no(off.size()), nm(m.size()), nw(w.size()), nb(3);
  CHECK(dcn_oracle_backward(&s, x.data(), off.data(), m.data(), w.data(), g.data(), gx.data(),
                            go.data(), gm.data(), gw.data(), gb.data(), nx.data(), no.data(),
                            nm.data(), nw.data(), nb.data(), 2) == 0);
  CHECK(dcn_oracle_backward(&s, x.data(), off.data(), nullptr, w.data(), g.data(), nullptr,
                            nullptr, nullptr, gw.data(), nullptr, nullptr, nullptr, nullptr,
                            nullptr, nullptr, 1) == 0);
  // multi-scale deformable attention: 2 levels, softmax
  const int64_t shapes[4] = {4, 5, 2, 3};
  const int64_t Bq = 1, Sv = 26, G = 2, D = 4, Q = 3, L = 2, Kp = 2;
  std::vector<float> val(Bq * Sv * G * D), loc(Bq * Q * G * L * Kp * 2), aw(Bq * Q * G * L * Kp);
  fill(val, 1.f);
  for (float& e : loc) e = std::fabs(n01(rng)) * 0.6f;
  fill(aw, 1.f);
  std::vector<double> mo(Bq * Q * G * D), mn(Bq * Q * G * D);
  CHECK(dcn_oracle_msda(Bq, Sv, G, D, Q, L, Kp, shapes, val.data(), loc.data(), aw.data(), 1,
                        mo.data(), mn.data(), 2) == 0);
  // single-scale sampling: 2 groups of 4 channels
  dcn_oracle_ds_shape ds = {1, 2, 4, 5, 6, 3, 3, 1, 1};
  // x [1, 5, 6, G*D], offset [1, G*2K, Ho, Wo], weights [1, G*K, Ho, Wo]
  std::vector<float> dx(5 * 6 * 8), doff(2 * 2 * K * Ho * Wo), dw(2 * K * Ho * Wo);
  fill(dx, 1.f);
  fill(doff, 2.f);
  fill(dw, 1.f);
  std::vector<double> dout(Ho * Wo * 8), dnorm(Ho * Wo * 8);
  CHECK(dcn_oracle_dsample(&ds, dx.data(), doff.data(), dw.data(), 1, dout.data(), dnorm.data(),
                           2) == 0);
  // refused shapes
  dcn_oracle_shape bad = {1, 4, 2, 2, 3, 5, 5, 0, 0};
  CHECK(dcn_oracle_forward(&bad, x.data(), off.data(), nullptr, w.data(), nullptr, nullptr, 0,
                           out.data(), nullptr, 1) == 2);
  return 0;
}

}  // namespace

int main() {
  if (abi_checks() != 0) return 1;
  if (oracle_checks() != 0) return 1;
  std::puts("sanitize ok");
  return 0;
}
