// Host-only driver of the library's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer (any finding aborts the run).  It calls every
// path that runs on the host without a GPU: status strings and sizes, the
// planner over a grid of shapes (valid, ragged, extreme and invalid), the EC
// scheduler and its selection step on random inputs, and the argument checks
// of the device entry points, which must reject their inputs before anything
// is enqueued.  Each check that fails prints its case and exits non-zero.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>
#include <vector>

#include "spear_w4ec.h"

extern "C" int spear_test_status_names(void);   // sanitizer_status.c

namespace {

int g_failures = 0;

#define CHECK(cond, ...)                          \
  do {                                            \
    if (!(cond)) {                                \
      std::fprintf(stderr, "FAIL %s: ", #cond);   \
      std::fprintf(stderr, __VA_ARGS__);          \
      std::fprintf(stderr, "\n");                 \
      ++g_failures;                               \
    }                                             \
  } while (0)

// SplitMix64 (Steele, Lea and Flood) as the driver's own random source.
struct Rng {
  uint64_t s;
  uint64_t next() {
    uint64_t x = (s += 0x9E3779B97F4A7C15ull);
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
  }
  int pick(int n) { return (int)(next() % (uint64_t)n); }
  double unit() { return (double)(next() >> 11) * (1.0 / 9007199254740992.0); }
};

const int32_t kBig = std::numeric_limits<int32_t>::max();

void statuses() {
  CHECK(spear_test_status_names() == 1, "status names of -5..39");
  for (int c = SPEAR_OK; c <= SPEAR_ERR_INVALID_ARGUMENT; ++c) {
    const char* s = spear_status_str((spear_status_t)c);
    CHECK(s != nullptr && s[0] != '\0', "status %d", c);
  }
  CHECK(spear_abi_version() == SPEAR_ABI_VERSION, "abi");
}

void sizes() {
  const int32_t ks[] = {-8, 0, 7, 8, 16, 120, 128, 136, 4096, 14336, kBig - 7, kBig};
  const int32_t ns[] = {-1, 0, 1, 15, 16, 17, 4096, 14336, kBig};
  const int32_t ranks[] = {-1, 0, 1, 32, 64, 112, 113, 128, 256, 257};
  for (int32_t K : ks)
    for (int32_t N : ns) {
      size_t b = 0;
      spear_status_t st = spear_packed_bytes(K, N, &b);
      if (st == SPEAR_OK) CHECK((double)b >= (double)K * N / 2, "packed_bytes K=%d N=%d", K, N);
      CHECK(spear_packed_bytes(K, N, nullptr) != SPEAR_OK, "packed_bytes null K=%d N=%d", K, N);
      for (int32_t r : ranks) {
        st = spear_ec_init_workspace_bytes(K, N, r, &b);
        if (st == SPEAR_OK) CHECK((double)b >= (double)K * N * 4, "ec_init bytes K=%d N=%d r=%d: %zu", K, N, r, b);
      }
    }
  const int32_t ms[] = {-1, 0, 1, 16, 2048, 65536, kBig};
  for (int32_t M : ms)
    for (int32_t K : ks)
      for (int32_t r : ranks) {
        size_t b = 0;
        const spear_status_t st = spear_ec_workspace_bytes(M, K, r, &b);
        if (st == SPEAR_OK) CHECK((double)b >= (double)(M > 0 ? M : 0) * r * 4, "ec ws M=%d K=%d r=%d", M, K, r);
      }
}

bool plan_is_sane(const spear_linear_desc_t& d, const spear_plan_t& p) {
  if (p.abi_version != SPEAR_ABI_VERSION || p.M != d.M || p.K != d.K || p.N != d.N) return false;
  if (p.variant < SPEAR_VARIANT_FUSED || p.variant > SPEAR_VARIANT_NO_EC) return false;
  if (d.M > 0 && (p.grid < 1 || p.tile_m < 1 || p.tile_n < 1 || p.split_k < 1)) return false;
  if (!(std::isfinite(p.predicted_us) && p.predicted_us >= 0.0f)) return false;
  if (!(std::isfinite(p.predicted_no_ec_us) && p.predicted_no_ec_us >= 0.0f)) return false;
  if (p.workspace_bytes > ((size_t)1 << 44)) return false;
  return true;
}

void plans(Rng& rng) {
  const int32_t ms[] = {-1, 0, 1, 2, 3, 4, 5, 8, 15, 16, 17, 31, 32, 63, 64, 65, 127, 128, 255, 256, 257,
                        511, 512, 1000, 1024, 2048, 4096, 65536, 1 << 24, kBig};
  const int32_t ks[] = {-8, 0, 7, 8, 16, 24, 120, 128, 136, 1024, 4096, 8192, 14336, 65536, 1 << 24, kBig - 7};
  const int32_t ns[] = {-1, 0, 1, 2, 15, 16, 17, 200, 392, 4096, 14336, 65536, 1 << 24, kBig};
  const int32_t ranks[] = {-1, 0, 1, 3, 4, 8, 31, 32, 64, 100, 128, 256, 257};
  const int32_t variants[] = {-1, SPEAR_VARIANT_AUTO, SPEAR_VARIANT_FUSED, SPEAR_VARIANT_SPLIT, SPEAR_VARIANT_NO_EC, 4};
  const int32_t groups[] = {0, SPEAR_GROUP_SIZE, 64, -1};
  const int32_t cus[] = {-1, 1, 7, 64, 256, 304, 1024};
  const float taus[] = {0.0f, 0.05f, 1.0f, 1.5f, -0.1f, std::numeric_limits<float>::quiet_NaN()};
  long ok = 0, total = 0;
  for (int i = 0; i < 60000; ++i) {
    spear_linear_desc_t d{};
    d.M = ms[rng.pick(sizeof ms / sizeof *ms)];
    d.K = ks[rng.pick(sizeof ks / sizeof *ks)];
    d.N = ns[rng.pick(sizeof ns / sizeof *ns)];
    d.rank = ranks[rng.pick(sizeof ranks / sizeof *ranks)];
    d.variant = variants[rng.pick(sizeof variants / sizeof *variants)];
    d.group_size = groups[rng.pick(sizeof groups / sizeof *groups)];
    d.device_cus = cus[rng.pick(sizeof cus / sizeof *cus)];
    d.skip_tau = taus[rng.pick(sizeof taus / sizeof *taus)];
    d.gate_bias = (float)(rng.unit() * 20.0 - 10.0);
    if (d.device_cus == 0) d.device_cus = 256;   // never query a device here
    spear_plan_t p{};
    const spear_status_t st = spear_dispatch_plan(&d, &p);
    ++total;
    if (st == SPEAR_OK) {
      ++ok;
      CHECK(plan_is_sane(d, p), "plan M=%d K=%d N=%d r=%d v=%d g=%d cus=%d -> variant %d grid %d tile %dx%d split %d "
            "predicted %g / %g us, workspace %zu", d.M, d.K, d.N, d.rank, d.variant, d.group_size, d.device_cus,
            p.variant, p.grid, p.tile_m, p.tile_n, p.split_k, p.predicted_us, p.predicted_no_ec_us, p.workspace_bytes);
    }
  }
  // Ragged and aligned shapes in full, on the planner's common paths.
  for (int32_t M : {1, 3, 16, 17, 64, 130, 256, 2048})
    for (int32_t K : {8, 136, 4096, 14336})
      for (int32_t N : {1, 17, 392, 4096})
        for (int32_t r : {0, 4, 36, 64})
          for (int32_t v : {SPEAR_VARIANT_AUTO, SPEAR_VARIANT_FUSED, SPEAR_VARIANT_SPLIT, SPEAR_VARIANT_NO_EC})
            for (int32_t g : {0, SPEAR_GROUP_SIZE}) {
              spear_linear_desc_t d{M, K, N, r, -1.0f, 0.0f, v, 256, g};
              spear_plan_t p{};
              if (spear_dispatch_plan(&d, &p) == SPEAR_OK) {
                ++ok;
                CHECK(plan_is_sane(d, p), "grid plan M=%d K=%d N=%d r=%d v=%d g=%d", M, K, N, r, v, g);
              }
              ++total;
            }
  CHECK(ok > total / 20, "only %ld of %ld plans accepted", ok, total);
  spear_plan_t p{};
  CHECK(spear_dispatch_plan(nullptr, &p) == SPEAR_ERR_NULL_POINTER, "null desc");
  spear_linear_desc_t d{16, 4096, 4096, 32, -1.0f, 0.0f, SPEAR_VARIANT_AUTO, 256, 0};
  CHECK(spear_dispatch_plan(&d, nullptr) == SPEAR_ERR_NULL_POINTER, "null plan");
  std::printf("plans: %ld of %ld accepted\n", ok, total);
}

void scheduler(Rng& rng) {
  for (int t = 0; t < 3000; ++t) {
    const int n = rng.pick(41);
    std::vector<double> extra(n);
    std::vector<float> w(n);
    for (int i = 0; i < n; ++i) {
      extra[i] = rng.pick(8) == 0 ? -1.0 : rng.unit() * 50.0;
      w[i] = rng.pick(6) == 0 ? 0.0f : (float)rng.unit();
    }
    const double slack = rng.pick(10) == 0 ? -5.0 : rng.pick(10) == 0 ? 1e30 : rng.unit() * 200.0;
    std::vector<uint8_t> on(n + 1, 7);
    double added = -1.0;
    const spear_status_t st = spear_schedule_ec_costs(extra.data(), w.data(), n, slack, on.data(), &added);
    CHECK(st == SPEAR_OK, "costs n=%d slack=%g status %d", n, slack, (int)st);
    double sum = 0.0;
    for (int i = 0; i < n; ++i) {
      CHECK(on[i] <= 1, "ec_on value");
      if (on[i]) {
        CHECK(extra[i] >= 0.0 && w[i] > 0.0f, "chose a layer without an EC or weight");
        sum += extra[i];
      }
    }
    CHECK(on[n] == 7, "wrote past ec_on");
    if (slack >= 0.0) CHECK(sum <= slack * (1.0 + 1e-9) + 1e-6, "over the slack: %g > %g", sum, slack);
  }
  {  // the largest instance: the coarse grid and the bit table at full size
    const int n = 4096;
    std::vector<double> extra(n);
    std::vector<float> w(n);
    for (int i = 0; i < n; ++i) {
      extra[i] = rng.unit();
      w[i] = (float)(0.1 + rng.unit());
    }
    std::vector<uint8_t> on(n + 1, 7);
    double added = 0.0;
    CHECK(spear_schedule_ec_costs(extra.data(), w.data(), n, 1000.0, on.data(), &added) == SPEAR_OK, "n = 4096");
    CHECK(on[n] == 7 && added <= 1000.0 * (1.0 + 1e-9), "n = 4096 outputs");
  }
  double e1[2] = {1.0, std::numeric_limits<double>::quiet_NaN()};
  float w1[2] = {1.0f, 1.0f};
  uint8_t on1[2];
  CHECK(spear_schedule_ec_costs(e1, w1, 2, 10.0, on1, nullptr) == SPEAR_ERR_INVALID_ARGUMENT, "nan extra");
  CHECK(spear_schedule_ec_costs(e1, w1, -1, 10.0, on1, nullptr) == SPEAR_ERR_INVALID_SHAPE, "n < 0");
  CHECK(spear_schedule_ec_costs(e1, w1, 5000, 10.0, on1, nullptr) == SPEAR_ERR_INVALID_SHAPE, "n too large");
  CHECK(spear_schedule_ec_costs(nullptr, w1, 2, 10.0, on1, nullptr) == SPEAR_ERR_NULL_POINTER, "null extra");

  for (int t = 0; t < 300; ++t) {
    const int n = 1 + rng.pick(12);
    std::vector<spear_sched_layer_t> layers(n);
    for (auto& l : layers) {
      l.K = 8 * (1 + rng.pick(2048));
      l.N = 1 + rng.pick(16384);
      l.rank = rng.pick(4) == 0 ? 0 : 4 * (1 + rng.pick(32));
      l.group_size = rng.pick(2) ? 0 : SPEAR_GROUP_SIZE;
      l.weight = (float)rng.unit();
    }
    const int32_t M = 1 + rng.pick(4096);
    const double slo = rng.unit() * 2000.0;
    std::vector<uint8_t> on(n + 1, 7);
    double pred = 0.0;
    const spear_status_t st = spear_schedule_ec(layers.data(), n, M, slo, 256, on.data(), &pred);
    CHECK(st == SPEAR_OK, "schedule n=%d M=%d status %d", n, M, (int)st);
    CHECK(on[n] == 7 && std::isfinite(pred), "schedule outputs");
    for (int i = 0; i < n; ++i) CHECK(on[i] <= 1 && (layers[i].rank > 0 || on[i] == 0), "ec_on of layer %d", i);
  }
  spear_sched_layer_t bad{7, 16, 8, 0, 1.0f};
  uint8_t on2[1];
  CHECK(spear_schedule_ec(&bad, 1, 4, 100.0, 256, on2, nullptr) == SPEAR_ERR_INVALID_SHAPE, "bad layer");
  CHECK(spear_schedule_ec(&bad, -1, 4, 100.0, 256, on2, nullptr) == SPEAR_ERR_INVALID_SHAPE, "n < 0");
  CHECK(spear_schedule_ec(nullptr, 1, 4, 100.0, 256, on2, nullptr) == SPEAR_ERR_NULL_POINTER, "null layers");
}

void argument_checks() {
  // Pointers that are never dereferenced on the host: each call must fail its
  // checks before anything is enqueued.
  char* base = reinterpret_cast<char*>((uintptr_t)1 << 20);
  const void* X = base;
  spear_linear_desc_t d{4, 4096, 4096, 32, -1.0f, 0.0f, SPEAR_VARIANT_AUTO, 256, 0};
  spear_plan_t p{};
  CHECK(spear_dispatch_plan(&d, &p) == SPEAR_OK, "plan for the argument checks");
  CHECK(spear_w4ec_linear(nullptr, &p, X, X, X, X, X, X, base, base, 1 << 30, nullptr) == SPEAR_ERR_NULL_POINTER,
        "null desc");
  CHECK(spear_w4ec_linear(&d, &p, nullptr, X, X, X, X, X, base, base, 1 << 30, nullptr) == SPEAR_ERR_NULL_POINTER,
        "null X");
  CHECK(spear_w4ec_linear(&d, &p, base + 2, X, X, X, X, X, base, base, 1 << 30, nullptr) == SPEAR_ERR_MISALIGNED,
        "misaligned X");
  if (p.workspace_bytes > 0)
    CHECK(spear_w4ec_linear(&d, &p, X, X, X, X, X, X, base, base, p.workspace_bytes - 1, nullptr) ==
              SPEAR_ERR_WORKSPACE_TOO_SMALL,
          "small workspace");
  spear_plan_t other = p;
  other.N = 1024;
  CHECK(spear_w4ec_linear(&d, &other, X, X, X, X, X, X, base, base, 1 << 30, nullptr) == SPEAR_ERR_INVALID_PLAN,
        "plan of another shape");
  spear_linear_desc_t bad = d;
  bad.K = 12;
  CHECK(spear_w4ec_linear(&bad, nullptr, X, X, X, X, X, X, base, base, 1 << 30, nullptr) == SPEAR_ERR_INVALID_SHAPE,
        "K not a multiple of 8");
  CHECK(spear_w4ec_linear_noalloc(nullptr, nullptr, X, X, X, X, X, X, base, nullptr) == SPEAR_ERR_NULL_POINTER,
        "noalloc null desc");
  CHECK(spear_pack_w4(nullptr, 128, 16, base, base, nullptr) == SPEAR_ERR_NULL_POINTER, "pack null");
  CHECK(spear_pack_w4(X, 12, 16, base, base, nullptr) == SPEAR_ERR_INVALID_SHAPE, "pack K");
  CHECK(spear_pack_w4_grouped(X, 128, 16, 64, base, base, nullptr) == SPEAR_ERR_UNSUPPORTED, "pack group 64");
  CHECK(spear_debug_unpack_w4(nullptr, 128, 16, base, nullptr) == SPEAR_ERR_NULL_POINTER, "unpack null");
  CHECK(spear_ec_project(4, 4096, 0, X, X, X, -1.0f, 0.0f, base, base, base, 1 << 20, nullptr) ==
            SPEAR_ERR_INVALID_SHAPE,
        "ec_project rank 0");
  CHECK(spear_ec_init(X, X, X, 4096, 4096, 0, 113, 0, base, base, base, (size_t)1 << 40, nullptr) ==
            SPEAR_ERR_INVALID_SHAPE || spear_ec_init(X, X, X, 4096, 4096, 0, 113, 0, base, base, base,
                                                     (size_t)1 << 40, nullptr) == SPEAR_ERR_UNSUPPORTED,
        "ec_init rank 113");
  CHECK(spear_ec_init(X, X, X, 4096, 4096, 0, 32, 65, base, base, base, (size_t)1 << 40, nullptr) ==
            SPEAR_ERR_INVALID_ARGUMENT,
        "ec_init iterations");
  CHECK(spear_ec_init(X, X, X, 4096, 4096, 0, 32, 0, base, base, base, 16, nullptr) ==
            SPEAR_ERR_WORKSPACE_TOO_SMALL,
        "ec_init workspace");
  uint32_t code = 0;
  char buf[64];
  CHECK(spear_take_error(buf, 1024, &code, nullptr) == SPEAR_ERR_WORKSPACE_TOO_SMALL, "take_error small");
  CHECK(spear_debug_stream_read(nullptr, 64, 1, buf, nullptr) == SPEAR_ERR_NULL_POINTER, "stream_read null");
  double flops = 0.0;
  CHECK(spear_debug_mfma_rate(0, 1, 10, nullptr, nullptr, &flops) == SPEAR_ERR_NULL_POINTER, "mfma_rate null");
  CHECK(spear_debug_mfma_rate(2, 1, 10, buf, nullptr, &flops) == SPEAR_ERR_INVALID_ARGUMENT, "mfma_rate shape");
  CHECK(spear_debug_mfma_rate(0, 1, 1 << 21, buf, nullptr, &flops) == SPEAR_ERR_INVALID_ARGUMENT,
        "mfma_rate iterations");
  spear_debug_set_spin_limit(0);
  spear_debug_set_spin_limit(-1);
  spear_debug_fail_waits(1);
  spear_debug_fail_waits(0);
}

}  // namespace

int main() {
  Rng rng{12345};
  statuses();
  sizes();
  plans(rng);
  scheduler(rng);
  argument_checks();
  if (g_failures) {
    std::fprintf(stderr, "%d check(s) failed\n", g_failures);
    return 1;
  }
  std::printf("sanitizer driver: all checks passed\n");
  return 0;
}
