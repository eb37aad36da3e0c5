// oracle_sanitize_main.cpp -- drives every entry point of the fp64 oracle on
// tiny layers of each storage format (fp32, bf16, fp8 with block scales, MXFP4,
// MX FP8, MX FP8 expert inputs), plus the argument checks, so that a build of
// the oracle with AddressSanitizer and UndefinedBehaviorSanitizer sees every
// loop it runs.  Exit status 0 when every call returns what it should.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "oracle.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint32_t next_u32() {  // xorshift64*: test inputs only
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (uint32_t)((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}
float uniform_pm1() { return (float)((next_u32() >> 8) * (2.0 / 16777216.0) - 1.0); }

int g_fail = 0;
void check(bool ok, const char *what) {
  if (!ok) {
    std::fprintf(stderr, "FAIL: %s\n", what);
    g_fail = 1;
  }
}

// One matrix stack in a given storage format, with the bytes kept alive.
struct Store {
  std::vector<uint8_t> data, scale;
  orc_mat m{};
  Store(int32_t dtype, int64_t n, int64_t rows, int64_t cols) {
    const int64_t el = n * rows * cols;
    m.dtype = dtype;
    m.n_mats = n;
    m.rows = rows;
    m.cols = cols;
    switch (dtype) {
      case ORC_F32: {
        data.resize(el * 4);
        float *p = reinterpret_cast<float *>(data.data());
        for (int64_t i = 0; i < el; ++i) p[i] = uniform_pm1() / std::sqrt((float)cols);
        break;
      }
      case ORC_BF16: {
        data.resize(el * 2);
        uint16_t *p = reinterpret_cast<uint16_t *>(data.data());
        for (int64_t i = 0; i < el; ++i) {
          float f = uniform_pm1();
          uint32_t u;
          std::memcpy(&u, &f, 4);
          p[i] = (uint16_t)(u >> 16);
        }
        break;
      }
      case ORC_FP8E4M3: {
        data.resize(el);
        for (auto &b : data) b = (uint8_t)(next_u32() % 0x7E) | (next_u32() & 0x80);
        scale.resize(n * (rows / 128) * (cols / 128) * 4);
        float *s = reinterpret_cast<float *>(scale.data());
        for (size_t i = 0; i < scale.size() / 4; ++i) s[i] = 1.0f / 256.0f;
        break;
      }
      case ORC_MXFP4:
        data.resize(el / 2);
        for (auto &b : data) b = (uint8_t)next_u32();
        scale.resize(n * rows * (cols / 32));
        for (auto &b : scale) b = (uint8_t)(120 + next_u32() % 4);
        break;
      case ORC_MXFP8:
        data.resize(el);
        for (auto &b : data) b = (uint8_t)(next_u32() % 0x7E) | (next_u32() & 0x80);
        scale.resize(n * rows * (cols / 32));
        for (auto &b : scale) b = (uint8_t)(118 + next_u32() % 4);
        break;
    }
    m.data = data.data();
    m.scale = scale.empty() ? nullptr : scale.data();
  }
};

void run_layer(int32_t dense_dt, int32_t expert_dt, int64_t mx_block, int64_t mx_exact,
               int32_t cutoff) {
  const bool big = dense_dt == ORC_FP8E4M3;  // fp8 blocks are 128 x 128
  orc_shape s{};
  s.d = big ? 256 : 64;
  s.latent = big ? 128 : 32;
  s.n_experts = 8;
  s.top_k = 2;
  s.expert_inter = big ? 128 : 64;
  s.n_shared = 2;
  s.shared_inter = big ? 128 : 32;
  s.beta = 4.0;
  s.beta_u = 25.0;
  s.rms_eps = 1e-6;
  s.act_mx_block = mx_block;
  s.act_mx_exact = mx_exact;
  const int64_t bt = 13, E = s.n_experts, k = s.top_k, P = bt * k;
  const int32_t rdt = dense_dt == ORC_FP8E4M3 ? ORC_BF16 : dense_dt;
  Store wr(rdt, 1, E, s.d), wdp(dense_dt, 1, s.latent, s.d);
  Store wg(expert_dt, E, s.expert_inter, s.latent), wu(expert_dt, E, s.expert_inter, s.latent);
  Store wd(expert_dt, E, s.latent, s.expert_inter), wup(dense_dt, 1, s.d, s.latent);
  Store sg(dense_dt, s.n_shared, s.shared_inter, s.d), su(dense_dt, s.n_shared, s.shared_inter, s.d);
  Store sd(dense_dt, s.n_shared, s.d, s.shared_inter);
  Store x(rdt, 1, bt, s.d);
  std::vector<float> bias(E), gamma(s.latent, 1.0f), alpha(E, 0.0f);
  for (auto &b : bias) b = 0.5f * uniform_pm1();
  orc_weights w{wr.m, bias.data(), wdp.m, wg.m, wu.m, wd.m, gamma.data(), wup.m,
                sg.m, su.m, sd.m};
  std::vector<float> z32(bt * E), zeta(E);
  std::vector<int32_t> idx(P), counts(E), offsets(E + 1), perm(P), inv(P);
  std::vector<double> wts(P), y(bt * s.d);
  const int rc = orc_forward(&s, &w, &x.m, bt, cutoff, alpha.data(), z32.data(), zeta.data(),
                             idx.data(), wts.data(), counts.data(), offsets.data(), perm.data(),
                             inv.data(), y.data());
  check(rc == 0, "orc_forward");
  check(offsets[E] == P, "dispatch covers every pair");
  for (double v : y) check(std::isfinite(v), "finite output");
  // the step functions on one token
  std::vector<double> z64(E), xl(s.latent), o(k * s.latent), ylat(s.latent), n(s.latent),
      yt(s.d), xt(s.d), sh(s.d);
  const int64_t row = 5;
  check(orc_router_logits(&s, &w, &x.m, &row, 1, z64.data()) == 0, "router logits");
  for (int64_t c = 0; c < s.d; ++c) xt[c] = orc_decode(&x.m, 0, row, c);
  orc_matvec(&wdp.m, 0, xt.data(), xl.data());
  for (int64_t j = 0; j < k; ++j)
    check(orc_expert(&s, &wg.m, &wu.m, &wd.m, idx[row * k + j], xl.data(),
                     o.data() + j * s.latent) == 0, "expert");
  check(orc_combine_norm(&s, o.data(), wts.data() + row * k, gamma.data(), ylat.data(),
                         n.data()) == 0, "combine");
  check(orc_shared(&s, &w, xt.data(), sh.data()) == 0, "shared");
  check(orc_output(&s, &w, n.data(), xt.data(), yt.data()) == 0, "output");
}

}  // namespace

int main() {
  orc_set_threads(2);
  check(orc_get_threads() == 2, "thread count");
  for (int32_t cutoff : {ORC_CUTOFF_GIVEN, ORC_CUTOFF_BATCH}) {
    run_layer(ORC_F32, ORC_F32, 0, 0, cutoff);
    run_layer(ORC_BF16, ORC_BF16, 0, 0, cutoff);
  }
  run_layer(ORC_FP8E4M3, ORC_FP8E4M3, 0, 0, ORC_CUTOFF_BATCH);
  run_layer(ORC_BF16, ORC_MXFP4, 0, 0, ORC_CUTOFF_BATCH);
  run_layer(ORC_BF16, ORC_MXFP4, 32, 0, ORC_CUTOFF_BATCH);
  run_layer(ORC_BF16, ORC_MXFP4, 32, 1, ORC_CUTOFF_BATCH);
  run_layer(ORC_BF16, ORC_MXFP8, 32, 0, ORC_CUTOFF_BATCH);

  // dense FFN on one row
  {
    orc_shape s{};
    s.d = 64;
    s.expert_inter = 96;
    s.beta = 4.0;
    s.beta_u = 25.0;
    s.rms_eps = 1e-6;
    Store g(ORC_BF16, 1, 96, 64), u(ORC_BF16, 1, 96, 64), dn(ORC_BF16, 1, 64, 96);
    std::vector<double> xr(64), r(64), yr(64);
    for (auto &v : xr) v = uniform_pm1();
    for (auto &v : r) v = uniform_pm1();
    check(orc_dense_ffn(&s, &g.m, &u.m, &dn.m, nullptr, xr.data(), r.data(), yr.data()) == 0,
          "dense ffn");
    check(orc_dense_ffn(&s, &dn.m, &u.m, &g.m, nullptr, xr.data(), r.data(), yr.data()) != 0,
          "dense ffn rejects mismatched shapes");
  }
  // MX FP8 quantiser and the encoders, over extreme values
  {
    std::vector<double> v(96);
    for (size_t i = 0; i < v.size(); ++i) v[i] = std::ldexp(uniform_pm1(), (int)(i % 40) - 20);
    v[0] = 0.0;
    v[1] = 1e300;
    v[2] = -1e-300;
    std::vector<uint8_t> codes(96), sc(3);
    check(orc_mx8_quantize(v.data(), 96, 32, codes.data(), sc.data()) == 0, "mx8 quantize");
    check(orc_mx8_quantize(v.data(), 95, 32, codes.data(), sc.data()) != 0, "mx8 rejects n");
    for (int c = 0; c < 256; ++c) {
      (void)orc_e4m3_to_double((uint8_t)c);
      (void)orc_e2m1_to_double((uint8_t)c);
      (void)orc_e8m0_to_double((uint8_t)c);
      (void)orc_double_to_e4m3(std::ldexp((double)c, -12));
      (void)orc_bf16_to_double((uint16_t)(c * 257));
    }
    for (double d : {0.0, -0.0, 1e-45, 3.5e38, -2.5e-40, 1.0 + 1.0 / 256})
      (void)orc_round_bf16(d);
  }
  // argument checks: rank out of range, ids out of range, k > E
  {
    std::vector<float> z(4 * 3, 0.5f), zeta(3);
    check(orc_quantile(z.data(), 4, 3, 0, zeta.data()) != 0, "quantile rejects m = 0");
    check(orc_quantile(z.data(), 4, 3, 5, zeta.data()) != 0, "quantile rejects m > bt");
    std::vector<int32_t> idx = {0, 7, 1, 2}, c(3), off(4), pm(4), iv(4);
    check(orc_dispatch(idx.data(), 2, 2, 3, c.data(), off.data(), pm.data(), iv.data()) != 0,
          "dispatch rejects an out-of-range id");
    std::vector<int32_t> ix(8);
    std::vector<double> wt(8);
    check(orc_topk(z.data(), nullptr, nullptr, 4, 3, 4, ix.data(), wt.data()) != 0,
          "topk rejects k > E");
  }
  if (g_fail) return 1;
  std::printf("oracle sanitizer run ok\n");
  return 0;
}
