// Drives every host-side entry point of libmlora (mlora_host.cpp: routes,
// adapter maps, table packing, windows, tile count, row token) through edge
// cases, capacity and NULL errors and a seeded fuzz, so that a build with
// AddressSanitizer and UndefinedBehaviorSanitizer reports any out-of-bounds
// access, leak, overflow or other undefined behaviour. Results are also
// checked against the plain rules; exit status 0 means clean.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "mlora.h"

static int g_failures = 0;
#define CHECK(c)                                                     \
  do {                                                               \
    if (!(c)) {                                                      \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      ++g_failures;                                                  \
    }                                                                \
  } while (0)

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(uint32_t n) {  // xorshift64*, seeded
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (uint32_t)((g_state * 0x2545F4914F6CDD1Dull) >> 33) % (n ? n : 1);
}

static void routes() {
  for (int s = -3; s < 6; ++s)
    for (int a = -1; a < 4; ++a)
      for (int h = 0; h < 2; ++h) {
        const int r = mlora_resolve_moe_lora_route(s, a, h);
        CHECK(r == (!h ? MLORA_ROUTE_FOLD : s < 0 ? MLORA_ROUTE_SKIP
                                                  : s == a ? MLORA_ROUTE_FOLD : MLORA_ROUTE_REFUSE));
        CHECK(mlora_ensure_decode_route_servable(r) ==
              (r == MLORA_ROUTE_REFUSE ? MLORA_ERR_REFUSE : MLORA_OK));
        const int m = mlora_resolve_moe_lora_route_multi(s, a);
        CHECK(m == (s < 0 ? MLORA_ROUTE_SKIP : s < a ? MLORA_ROUTE_FOLD : MLORA_ROUTE_REFUSE));
      }
  CHECK(mlora_ensure_decode_route_servable(99) == MLORA_ERR_INVALID);
  CHECK(mlora_last_error()[0] != '\0');
}

static void maps() {
  // host map: valid, rejected and capacity-limited inputs
  const int32_t cu_ok[] = {0, 3, 3, 7}, slots3[] = {1, -1, 2};
  int64_t total = -1;
  CHECK(mlora_build_moe_row_adapter_host(cu_ok, 4, slots3, 3, nullptr, 0, &total) ==
        MLORA_ERR_CAPACITY);
  CHECK(total == 7);
  std::vector<int32_t> out(7, 99);
  CHECK(mlora_build_moe_row_adapter_host(cu_ok, 4, slots3, 3, out.data(), 7, &total) == MLORA_OK);
  CHECK(out[0] == 1 && out[2] == 1 && out[3] == 2 && out[6] == 2);
  const int32_t cu_bad[] = {0, 4, 2}, slots2[] = {1, 1};
  std::vector<int32_t> small(2, 42);
  CHECK(mlora_build_moe_row_adapter_host(cu_bad, 3, slots2, 2, small.data(), 2, &total) ==
        MLORA_NONE);
  CHECK(small[0] == 42 && small[1] == 42);
  CHECK(mlora_build_moe_row_adapter_host(cu_ok, 1, slots3, 0, nullptr, 0, &total) == MLORA_NONE);
  CHECK(mlora_build_moe_row_adapter_host(cu_ok, 4, slots3, 2, nullptr, 0, &total) == MLORA_NONE);
  CHECK(mlora_build_moe_row_adapter_host(nullptr, 4, slots3, 3, nullptr, 0, &total) ==
        MLORA_ERR_INVALID);
  // decode maps, padding and truncation
  const int32_t dslots[] = {1, -1, 2, 1, 0};
  std::vector<int32_t> d(8, 7);
  CHECK(mlora_build_moe_row_adapter_decode(dslots, 5, 8, 1, 1, d.data()) == MLORA_OK);
  CHECK(d[0] == 1 && d[1] == -1 && d[2] == -1 && d[3] == 1 && d[4] == -1 && d[7] == -1);
  CHECK(mlora_build_moe_row_adapter_decode(dslots, 5, 3, 1, 0, d.data()) == MLORA_OK);
  CHECK(mlora_build_moe_row_adapter_decode(dslots, 5, 0, 1, 1, nullptr) == MLORA_OK);
  CHECK(mlora_build_moe_row_adapter_decode(nullptr, 5, 4, 1, 1, d.data()) == MLORA_ERR_INVALID);
  CHECK(mlora_build_moe_row_adapter_decode_multi(dslots, 5, 8, 2, d.data()) == MLORA_OK);
  CHECK(d[0] == 1 && d[2] == -1 && d[4] == 0 && d[6] == -1);
  CHECK(mlora_build_moe_row_adapter_decode_multi(dslots, 5, -1, 2, d.data()) ==
        MLORA_ERR_INVALID);
  // fuzz: random boundaries (sometimes decreasing), random slots
  for (int it = 0; it < 2000; ++it) {
    const int batch = (int)rnd(9);
    std::vector<int32_t> cu(batch + 1), sl(batch);
    cu[0] = rnd(10) == 0 ? (int32_t)rnd(3) : 0;
    for (int b = 0; b < batch; ++b) {
      cu[b + 1] = cu[b] + (int32_t)rnd(6) - (rnd(20) == 0 ? 7 : 0);
      sl[b] = (int32_t)rnd(5) - 1;
    }
    int64_t n = -1;
    const int rc = mlora_build_moe_row_adapter_host(cu.data(), batch + 1, sl.data(), batch,
                                                    nullptr, 0, &n);
    if (rc == MLORA_ERR_CAPACITY || (rc == MLORA_OK && n == 0)) {
      std::vector<int32_t> m(n > 0 ? n : 1, -9);
      CHECK(mlora_build_moe_row_adapter_host(cu.data(), batch + 1, sl.data(), batch, m.data(),
                                             n, &n) == MLORA_OK);
      for (int b = 0; b < batch; ++b)
        for (int t = cu[b]; t < cu[b + 1]; ++t) CHECK(m[t] == sl[b]);
    } else {
      CHECK(rc == MLORA_NONE);
    }
    const int padded = (int)rnd(12);
    std::vector<int32_t> dm(padded + 1);
    CHECK(mlora_build_moe_row_adapter_decode(sl.data(), batch, padded, (int32_t)rnd(3),
                                             (int32_t)rnd(2), dm.data()) == MLORA_OK);
    CHECK(mlora_build_moe_row_adapter_decode_multi(sl.data(), batch, padded, (int32_t)rnd(4),
                                                   dm.data()) == MLORA_OK);
  }
}

static void packing() {
  int32_t n = -1, na = -1, ne = -1;
  CHECK(mlora_pack_expert_tables(nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr,
                                 nullptr, 0, &n) == MLORA_NONE);
  const int32_t bad_ids[] = {3, -1};
  const uint64_t ad[] = {16, 32}, bd[] = {48, 64};
  const float sc[] = {1.f, 2.f};
  CHECK(mlora_pack_expert_tables(bad_ids, ad, bd, sc, 2, nullptr, nullptr, nullptr, 0, &n) ==
        MLORA_ERR_INVALID);
  for (int it = 0; it < 2000; ++it) {
    const int m = 1 + (int)rnd(20);
    std::vector<int32_t> ids(m), slots(m);
    std::vector<uint64_t> a(m), b(m);
    std::vector<float> s(m);
    for (int i = 0; i < m; ++i) {
      ids[i] = (int32_t)rnd(40);
      slots[i] = (int32_t)rnd(5);
      a[i] = rnd(4) ? 16ull * (1 + rnd(1000)) : 0;
      b[i] = rnd(4) ? 16ull * (1 + rnd(1000)) : 0;
      s[i] = (float)rnd(100) / 8.f;
    }
    CHECK(mlora_pack_expert_tables(ids.data(), a.data(), b.data(), s.data(), m, nullptr,
                                   nullptr, nullptr, 0, &n) == MLORA_ERR_CAPACITY);
    std::vector<uint64_t> at(n), bt(n);
    std::vector<float> st(n);
    CHECK(mlora_pack_expert_tables(ids.data(), a.data(), b.data(), s.data(), m, at.data(),
                                   bt.data(), st.data(), n, &n) == MLORA_OK);
    for (int i = 0; i < m; ++i) {  // the last entry for each id wins
      bool later = false;
      for (int j = i + 1; j < m; ++j) later |= ids[j] == ids[i];
      if (!later) CHECK(at[ids[i]] == a[i] && bt[ids[i]] == b[i] && st[ids[i]] == s[i]);
    }
    CHECK(mlora_pack_expert_tables_multi(slots.data(), ids.data(), a.data(), b.data(), s.data(),
                                         m, nullptr, nullptr, nullptr, 0, &na, &ne) ==
          MLORA_ERR_CAPACITY);
    const int64_t cells = (int64_t)na * ne;
    std::vector<uint64_t> am(cells), bm(cells);
    std::vector<float> sm(cells);
    CHECK(mlora_pack_expert_tables_multi(slots.data(), ids.data(), a.data(), b.data(), s.data(),
                                         m, am.data(), bm.data(), sm.data(), cells, &na,
                                         &ne) == MLORA_OK);
    for (int i = 0; i < m; ++i) {
      bool later = false;
      for (int j = i + 1; j < m; ++j) later |= ids[j] == ids[i] && slots[j] == slots[i];
      if (!later) CHECK(am[(int64_t)slots[i] * ne + ids[i]] == a[i]);
    }
  }
}

static void windows() {
  int64_t nw = -1;
  CHECK(mlora_grouped_down_windows(10, 0, nullptr, nullptr, 0, &nw) == MLORA_ERR_INVALID);
  CHECK(mlora_grouped_down_windows(0, 5, nullptr, nullptr, 0, &nw) == MLORA_OK && nw == 0);
  for (int it = 0; it < 2000; ++it) {
    const int64_t total = rnd(5000), cap = 1 + rnd(700);
    const int rc = mlora_grouped_down_windows(total, cap, nullptr, nullptr, 0, &nw);
    CHECK(rc == (total ? MLORA_ERR_CAPACITY : MLORA_OK));
    std::vector<int64_t> s(nw + 1), e(nw + 1);
    CHECK(mlora_grouped_down_windows(total, cap, s.data(), e.data(), nw, &nw) == MLORA_OK);
    int64_t at = 0;
    for (int64_t w = 0; w < nw; ++w) {
      CHECK(s[w] == at && e[w] > s[w] && e[w] - s[w] <= cap);
      at = e[w];
      CHECK(mlora_grouped_down_wc(s[w], e[w]) ==
            (uint32_t)((e[w] - s[w] + MLORA_MLG_M_TILE - 1) / MLORA_MLG_M_TILE));
    }
    CHECK(at == total);
  }
  CHECK(mlora_grouped_down_wc(7, 7) == 1);
  CHECK(mlora_gather_row_token(17, 8) == 2 && mlora_gather_row_token(-1, 8) == -1 &&
        mlora_gather_row_token(5, 0) == -1);
  CHECK(mlora_m_tile() == MLORA_MLG_M_TILE);
}

int main() {
  routes();
  maps();
  packing();
  windows();
  if (g_failures) std::fprintf(stderr, "%d checks failed\n", g_failures);
  else std::printf("host sanitize: clean\n");
  return g_failures ? 1 : 0;
}
