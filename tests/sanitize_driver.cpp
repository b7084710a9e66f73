// Host-only driver for the sanitizer build of the oracle (oracle/oracle.cpp,
// included below so its internal structs are visible) and the storage tier
// (sparse_moe_decode_amd/csrc/store.cpp, linked). Built with
// -fsanitize=address,undefined by tests/test_sanitize.py, it runs every
// exported oracle routine on small shapes, including the error returns, and
// the storage tier's threaded reads (buffered and O_DIRECT where the file
// system allows it, many tickets in flight, unaligned destinations, bad ids,
// a missing file). Prints "ok" and returns 0 when every check holds; a
// sanitizer report aborts the run.

#include "../oracle/oracle.cpp"

#include <fcntl.h>
#include <unistd.h>

#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "sparse_moe_decode.h"

// store.cpp reports errors through this hook (defined by the library's
// boundary code in the product build).
static std::string g_msg;
int smd_report(int code, const char* msg) {
  g_msg = msg;
  return code;
}

#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      return 1;                                                      \
    }                                                                \
  } while (0)

namespace {

struct Lcg {
  uint64_t s;
  uint32_t u32() {
    s = s * 6364136223846793005ULL + 1442695040888963407ULL;
    return (uint32_t)(s >> 32);
  }
  double sym() { return (u32() / 4294967296.0) * 2.0 - 1.0; }
};

uint16_t h16(double v) {
  uint16_t o;
  orc_f16_round(&v, 1, &o);
  return o;
}

int oracle_part() {
  const int d = 128, E = 16, K = 4, I = 64, Is = 64, G = 32, r = 4, P = 64;
  const int F = d + 2 * E;
  Lcg rng{7};
  auto words = [&](size_t n) {
    std::vector<uint32_t> v(n);
    for (auto& x : v) x = rng.u32();
    return v;
  };
  auto scales = [&](size_t n) {
    std::vector<uint16_t> v(n);
    for (auto& x : v) x = h16(0.01 + 0.01 * std::fabs(rng.sym()));
    return v;
  };
  auto halfs = [&](size_t n, double a) {
    std::vector<uint16_t> v(n);
    for (auto& x : v) x = h16(a * rng.sym());
    return v;
  };
  // fp16 round trip over every pattern
  for (uint32_t b = 0; b < 65536; ++b) {
    const uint16_t bits = (uint16_t)b;
    double v;
    orc_f16_decode(&bits, 1, &v);
    if (v == v) CHECK(h16(v) == bits || (v == 0.0));
  }
  auto gq = words((size_t)E * I * d / 8), uq = words((size_t)E * I * d / 8),
       dq = words((size_t)E * d * I / 8);
  auto gs = scales((size_t)E * I * d / G), us = scales((size_t)E * I * d / G),
       ds = scales((size_t)E * d * I / G);
  auto sgq = words((size_t)Is * d / 8), suq = words((size_t)Is * d / 8),
       sdq = words((size_t)d * Is / 8);
  auto sgs = scales((size_t)Is * d / G), sus = scales((size_t)Is * d / G),
       sds = scales((size_t)d * Is / G);
  auto ag = halfs((size_t)r * d, 0.05), bg = halfs((size_t)Is * r, 0.05),
       au = halfs((size_t)r * d, 0.05), bu = halfs((size_t)Is * r, 0.05),
       ad = halfs((size_t)r * Is, 0.05), bd = halfs((size_t)d * r, 0.05);
  auto x16 = halfs(d, 1.0);
  std::vector<double> x(d), y(d), y2(d);
  orc_f16_decode(x16.data(), d, x.data());

  std::vector<double> deq((size_t)I * d);
  orc_q4_dequant(gq.data(), gs.data(), I, d, G, deq.data());
  std::vector<double> mv(I), z(I), zs(I), zg(I);
  orc_q4_matvec(gq.data(), gs.data(), I, d, G, x.data(), mv.data());
  for (int i = 0; i < I; ++i) z[i] = mv[i] - 3.0;
  orc_silu(z.data(), I, zs.data());
  orc_gelu_erf(z.data(), I, zg.data());
  std::vector<double> nrm(d);
  orc_rmsnorm(x.data(), d, 1e-6, nrm.data());

  orc_expert(gq.data(), gs.data(), uq.data(), us.data(), dq.data(), ds.data(), d, I, G, x.data(),
             y.data());
  orc_shared_expert(sgq.data(), sgs.data(), suq.data(), sus.data(), sdq.data(), sds.data(),
                    ag.data(), bg.data(), au.data(), bu.data(), ad.data(), bd.data(), d, Is, G, r,
                    8.0, x.data(), y.data());
  orc_shared_expert(sgq.data(), sgs.data(), suq.data(), sus.data(), sdq.data(), sds.data(),
                    nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, d, Is, G, 0, 0.0,
                    x.data(), y2.data());
  std::vector<double> acc(d, 0.0);
  orc_lora_delta(ad.data(), bd.data(), Is, d, r, 2.0, x.data(), acc.data());

  orc_moe m{};
  m.d = d; m.E = E; m.K = K; m.I = I; m.Is = Is; m.group = G; m.r = r; m.alpha = 8.0;
  m.gate_q = gq.data(); m.up_q = uq.data(); m.down_q = dq.data();
  m.gate_s = gs.data(); m.up_s = us.data(); m.down_s = ds.data();
  m.sh_gate_q = sgq.data(); m.sh_up_q = suq.data(); m.sh_down_q = sdq.data();
  m.sh_gate_s = sgs.data(); m.sh_up_s = sus.data(); m.sh_down_s = sds.data();
  m.a_gate = ag.data(); m.b_gate = bg.data(); m.a_up = au.data(); m.b_up = bu.data();
  m.a_down = ad.data(); m.b_down = bd.data();
  int32_t idx[K] = {3, 0, 15, 7};
  double w[K] = {0.4, 0.3, 0.2, 0.1};
  CHECK(orc_moe_decode(&m, x16.data(), idx, w, y.data()) == 0);
  int32_t bad[K] = {3, 0, 16, 7};
  CHECK(orc_moe_decode(&m, x16.data(), bad, w, y.data()) == -1);

  std::vector<double> lg(E), bias(E, 0.01), sel(E), grp(4);
  for (auto& v : lg) v = 2.0 * rng.sym();
  lg[5] = lg[9];  // a tie
  int32_t ri[K];
  double rw[K];
  int32_t tk[E];
  CHECK(orc_topk(lg.data(), nullptr, E, E, tk) == E);
  CHECK(orc_route_softmax_topk(lg.data(), E, K, 1, ri, rw) == 0);
  CHECK(orc_route_softmax_topk(lg.data(), E, K, 0, ri, rw) == 0);
  CHECK(orc_route_softmax_topk(lg.data(), E, E + 1, 1, ri, rw) == -1);
  CHECK(orc_route_sigmoid_group(lg.data(), bias.data(), E, K, 4, 2, 2.5, ri, rw, sel.data(),
                                grp.data()) == 0);
  CHECK(orc_route_sigmoid_group(lg.data(), nullptr, E, K, 5, 2, 1.0, ri, rw, nullptr,
                                nullptr) == -1);
  orc_routing rt{1, E, K, 1, 4, 2, 2.5};
  float bias32[E];
  for (int e = 0; e < E; ++e) bias32[e] = 0.02f * (float)rng.sym();
  CHECK(orc_route(&rt, lg.data(), bias32, ri, rw) == 0);

  auto fc1 = halfs((size_t)P * F, 0.05), fc2 = halfs((size_t)E * P, 0.05),
       lin = halfs((size_t)E * F, 0.05);
  int32_t cur[K] = {1, 2, 3, 4}, prev[K] = {4, 5, 6, 7}, dup[K] = {1, 1, 2, 3};
  std::vector<double> hl(E), hl0(E);
  CHECK(orc_head_logits(fc1.data(), fc2.data(), lin.data(), d, E, P, K, x16.data(), cur, prev,
                        1, hl.data()) == 0);
  CHECK(orc_head_logits(fc1.data(), fc2.data(), lin.data(), d, E, P, K, x16.data(), cur, nullptr,
                        0, hl0.data()) == 0);
  CHECK(orc_head_logits(fc1.data(), fc2.data(), lin.data(), d, E, P, K, x16.data(), dup, prev,
                        1, hl.data()) != 0);

  auto attn = halfs(d, 0.1), router = halfs((size_t)E * d, 0.05), h = halfs(d, 1.0);
  orc_layer L{};
  L.moe = m;
  L.rt = orc_routing{0, E, K, 1, 1, 1, 1.0};
  L.eps = 1e-6;
  L.attn = attn.data();
  L.router = router.data();
  L.router_bias = nullptr;
  L.fc1 = fc1.data(); L.fc2 = fc2.data(); L.lin = lin.data();
  L.head_bias = nullptr;
  L.P = P;
  std::vector<double> hout(d), rlog(E), hlog(E);
  std::vector<uint16_t> xout(d);
  int32_t ei[K], pi[K];
  double ew[K], pw[K];
  CHECK(orc_layer_step(&L, h.data(), nullptr, nullptr, nullptr, prev, hout.data(), xout.data(), ei,
                       ew, rlog.data(), hlog.data(), pi, pw) == 0);
  L.router = nullptr;
  const float rwf[K] = {0.4f, 0.3f, 0.2f, 0.1f};
  CHECK(orc_layer_step(&L, h.data(), xout.data(), idx, rwf, nullptr, hout.data(), nullptr, ei,
                       ew, nullptr, nullptr, pi, pw) == 0);
  CHECK(orc_layer_step(&L, h.data(), nullptr, bad, rwf, nullptr, hout.data(), nullptr, ei, ew,
                       nullptr, nullptr, pi, pw) == -1);

  const int S = 2 * K;
  std::vector<int32_t> slot_of(E, -1), slot_expert(S, -1), ce(S), cs(S);
  CHECK(orc_slot_policy(E, S, K, slot_of.data(), slot_expert.data(), nullptr, idx, ce.data(),
                        cs.data()) == K);
  int32_t nxt[K] = {7, 8, 9, 3};
  CHECK(orc_slot_policy(E, S, K, slot_of.data(), slot_expert.data(), idx, nxt, ce.data(),
                        cs.data()) == 2);
  int32_t big[K] = {10, 11, 12, 13};
  CHECK(orc_slot_policy(E, K, K, slot_of.data(), slot_expert.data(), nxt, big, ce.data(),
                        cs.data()) == -1);
  return 0;
}

int store_part(const char* dir) {
  const int L = 2, E = 6;
  const int64_t bundle = 8192;
  std::vector<std::string> paths;
  std::vector<std::vector<unsigned char>> data(L);
  for (int l = 0; l < L; ++l) {
    paths.push_back(std::string(dir) + "/layer" + std::to_string(l) + ".bin");
    data[l].resize((size_t)E * bundle);
    for (size_t i = 0; i < data[l].size(); ++i) data[l][i] = (unsigned char)(i * 131 + l * 7 + (i >> 13));
    FILE* f = std::fopen(paths[l].c_str(), "wb");
    CHECK(f != nullptr);
    CHECK(std::fwrite(data[l].data(), 1, data[l].size(), f) == data[l].size());
    std::fclose(f);
  }
  const char* cp[L] = {paths[0].c_str(), paths[1].c_str()};
  for (int direct = 0; direct < 2; ++direct) {
    e0_store* st = nullptr;
    const int rc = e0_store_open(cp, L, E, bundle, 3, direct, &st);
    if (direct && rc != E0_OK) continue;  // O_DIRECT not supported by this file system
    CHECK(rc == E0_OK);
    // many tickets in flight; destinations one byte off alignment
    std::vector<unsigned char> buf((size_t)L * E * bundle + 1);
    std::vector<int64_t> tickets;
    for (int l = 0; l < L; ++l) {
      int32_t ids[E];
      void* dst[E];
      for (int e = 0; e < E; ++e) {
        ids[e] = (e * 5 + l) % E;
        dst[e] = buf.data() + 1 + ((size_t)l * E + e) * bundle;
      }
      for (int half = 0; half < 2; ++half) {
        int64_t t = -1;
        CHECK(e0_store_read(st, l, ids + 3 * half, 3, dst + 3 * half, &t) == E0_OK);
        tickets.push_back(t);
      }
    }
    for (int64_t t : tickets) {
      double blocked = 0, rd = 0;
      CHECK(e0_store_wait(st, t, &blocked, &rd) == E0_OK);
    }
    for (int l = 0; l < L; ++l)
      for (int e = 0; e < E; ++e) {
        const int id = (e * 5 + l) % E;
        CHECK(std::memcmp(buf.data() + 1 + ((size_t)l * E + e) * bundle,
                          data[l].data() + (size_t)id * bundle, bundle) == 0);
      }
    CHECK(e0_store_bytes(st) == (int64_t)L * E * bundle);
    int32_t badid[1] = {E};
    void* d0[1] = {buf.data()};
    int64_t t = -1;
    CHECK(e0_store_read(st, 0, badid, 1, d0, &t) == E0_ERR_RANGE);
    CHECK(e0_store_read(st, L, badid, 0, d0, &t) != E0_OK);
    e0_store_close(st);
  }
  const std::string missing = std::string(dir) + "/missing.bin";
  const char* mp[1] = {missing.c_str()};
  e0_store* st = nullptr;
  CHECK(e0_store_open(mp, 1, E, bundle, 1, 0, &st) == E0_ERR_IO);
  CHECK(e0_store_open(cp, L, E, 1000, 1, 1, &st) == E0_ERR_ALIGN);
  for (auto& p : paths) unlink(p.c_str());
  return 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc < 2) {
    std::fprintf(stderr, "usage: %s <scratch directory>\n", argv[0]);
    return 2;
  }
  if (oracle_part()) return 1;
  if (store_part(argv[1])) return 1;
  std::printf("ok\n");
  return 0;
}
