// Host checks of the static step plan (kd_plan.h), built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py. The plan is integer arithmetic
// that the packer and every workgroup repeat, so a wrong partition or an overflow would send a
// workgroup to the wrong rows; each check below states a property the kernels rely on.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "kd_plan.h"

static int g_fail = 0;
#define CHECK(cond, ...)                                      \
  do {                                                        \
    if (!(cond)) {                                            \
      std::fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond); \
      std::fprintf(stderr, __VA_ARGS__);                      \
      std::fprintf(stderr, "\n");                             \
      if (++g_fail > 20) std::exit(1);                        \
    }                                                         \
  } while (0)

using namespace kd;

// part_lo cuts n items into `parts` contiguous runs; part_of names the run that holds an item.
static void check_partition(int64_t n, int64_t parts) {
  CHECK(part_lo(n, parts, 0) == 0 && part_lo(n, parts, parts) == n, "n=%lld parts=%lld", (long long)n, (long long)parts);
  for (int64_t i = 0; i < parts; ++i) CHECK(part_lo(n, parts, i) <= part_lo(n, parts, i + 1), "monotone i=%lld", (long long)i);
  for (int64_t u = 0; u < n; ++u) {
    const int64_t w = part_of(n, parts, u);
    CHECK(w >= 0 && w < parts && part_lo(n, parts, w) <= u && u < part_lo(n, parts, w + 1),
          "part_of n=%lld parts=%lld u=%lld -> %lld", (long long)n, (long long)parts, (long long)u, (long long)w);
  }
}

// wave_lo splits n items over the 8 waves: runs in order, covering 0..n, the older waves of a
// SIMD (0-3) never with fewer items than the younger ones (4-7).
static void check_waves(int64_t n) {
  CHECK(wave_lo(n, 0) == 0 && wave_lo(n, kWaves) == n, "n=%lld", (long long)n);
  for (int v = 0; v < kWaves; ++v) CHECK(wave_lo(n, v) <= wave_lo(n, v + 1), "n=%lld v=%d", (long long)n, v);
  for (int v = 0; v < 4; ++v) {
    const int64_t a = wave_lo(n, v + 1) - wave_lo(n, v), b = wave_lo(n, v + 5) - wave_lo(n, v + 4);
    CHECK(a + 1 >= b, "n=%lld v=%d older %lld younger %lld", (long long)n, v, (long long)a, (long long)b);
  }
}

struct Shape {
  const char* name;
  int L, d, hq, hkv, hd, F, V, max_seq, wbytes, kvbytes;
};

static void check_shape(const Shape& s, int nwg) {
  const Dims m = make_dims(s.L, s.d, s.hq, s.hkv, s.hd, s.F, s.V, s.max_seq, nwg, s.wbytes, s.kvbytes);
  // the cache holds every position a step may touch, and the last packet of a chunk may run 7 past
  CHECK(m.S >= s.max_seq + 7 && m.S % 16 == 0, "%s S=%d", s.name, m.S);
  CHECK(m.lpp * m.ppp == 64 && m.lpp * m.kv_vpl == m.hd, "%s lanes per position", s.name);
  // packed blob: regions in order and back to back
  CHECK(m.off_o - m.off_qkv == (int64_t)m.nqkv * m.d && m.off_gu - m.off_o == (int64_t)m.d * m.qdim &&
            m.off_d - m.off_gu == (int64_t)2 * m.F * m.d && m.layer_elems - m.off_d == (int64_t)m.d * m.F &&
            m.blob_elems == m.off_lm + (int64_t)m.V * m.d,
        "%s blob layout", s.name);
  // row scales: one per output row of the seven matrices, then the LM head
  const ScaleLayout sc = scale_layout(m);
  CHECK(sc.layer == (int64_t)m.nqkv + m.d + 2 * (int64_t)m.F + m.d && sc.total == (int64_t)m.L * sc.layer + m.V,
        "%s scale layout", s.name);
  // FFN slices: whole units, in order, every workgroup at least one unit when the shape allows it
  const int64_t fu = ffn_unit(m), U = m.F / fu;
  CHECK(m.F % fu == 0, "%s ffn unit", s.name);
  CHECK(ffn_lo(m, 0) == 0 && ffn_lo(m, nwg) == m.F, "%s ffn ends", s.name);
  for (int w = 0; w < nwg; ++w) {
    const int64_t a = ffn_lo(m, w), b = ffn_lo(m, w + 1);
    CHECK(a % fu == 0 && b > a - 1 && (U < nwg || b > a), "%s ffn slice %d [%lld, %lld)", s.name, w, (long long)a, (long long)b);
    CHECK(down_wg_off(m, w) == (int64_t)m.d * a, "%s down offset", s.name);
  }
  check_partition(U, nwg);
  check_partition(m.nqkv, nwg);
  check_partition(m.V, nwg);
  // exchange words: disjoint regions in order, even offsets, each as large as its vector
  const LLLayout l = ll_layout(m);
  const int64_t at[] = {l.qkv, l.attp, l.o, l.xp, l.dp, l.x, l.lm, l.total};
  const int64_t need[] = {m.nqkv, (int64_t)m.hq * max_chunks(m) * (m.hd + 2), m.qdim, m.d, (int64_t)nwg * m.d, m.d, 2 * (int64_t)nwg};
  for (int i = 0; i < 7; ++i) CHECK(at[i] % 2 == 0 && at[i + 1] - at[i] >= need[i], "%s ll region %d", s.name, i);
  // attention split at every position: chunks of whole packets, no empty chunk, scores that fit
  // a wave's LDS share, partials that fit their buffer, merge slices that divide the head
  for (int32_t p = 0; p < s.max_seq; ++p) {
    const AttPlan a = att_plan(m, p);
    const int64_t pk = ceil_div(a.CH, m.ppp);
    CHECK(a.P == p + 1 && a.CH > 0 && a.CH % m.ppp == 0, "%s p=%d CH=%d", s.name, p, a.CH);
    CHECK((int64_t)a.NC * a.CH >= a.P && (int64_t)(a.NC - 1) * a.CH < a.P, "%s p=%d NC=%d CH=%d", s.name, p, a.NC, a.CH);
    CHECK(a.NC <= max_chunks(m) && a.units == a.NC * m.hkv && ceil_div(a.units, nwg) <= kMaxUnits, "%s p=%d units", s.name, p);
    CHECK(ceil_div(pk, kWaves) * m.ppp <= kScorePos, "%s p=%d scores per wave", s.name, p);
    CHECK(m.hd % a.MS == 0 && a.MS % 2 == 0 && (int64_t)a.NC * (a.MS + 2) <= kMergeWords &&
              a.nmerge == m.hq * (m.hd / a.MS),
          "%s p=%d merge MS=%d", s.name, p, a.MS);
  }
  // tags: one step's tags never reach the next step's
  CHECK(ll_tag(0, m.L, kLM) < tag_stride(m), "%s tags", s.name);
}

int main() {
  const int nwg = 256;
  for (int64_t n : {1, 2, 3, 7, 8, 9, 63, 64, 100, 255, 256, 257, 1000, 1792, 6144, 32000})
    for (int64_t parts : {1, 2, 3, 7, 8, 64, 255, 256, 257}) check_partition(n, parts);
  for (int64_t n = 0; n < 4096; ++n) check_waves(n);
  check_waves((int64_t)1 << 40);
  const std::vector<Shape> shapes = {
      {"tiny f32", 2, 256, 4, 4, 64, 1024, 1024, 96, 4, 4},
      {"2B bf16", 26, 2048, 16, 4, 128, 8192, 32000, 1024, 2, 2},
      {"2B bf16 long", 26, 2048, 16, 4, 128, 8192, 32000, 32768 + 136, 2, 2},
      {"8B bf16", 32, 4096, 32, 8, 128, 14336, 128256, 1280, 2, 2},
      {"8B one-byte", 32, 4096, 32, 8, 128, 14336, 128256, 1280, 1, 2},
      {"2B one-byte", 26, 2048, 16, 4, 128, 8192, 32000, 1024, 1, 2},
      {"hd64 bf16 G2", 2, 1024, 16, 8, 64, 2048, 4096, 520, 2, 2},
      {"hd128 f32 G3", 2, 1536, 12, 4, 128, 4096, 4096, 520, 4, 4},
  };
  for (const Shape& s : shapes) check_shape(s, nwg);
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("plan checks passed (%zu shapes)\n", shapes.size());
  return 0;
}
