// Host-side property harness for the library's CPU code (rate tables, codebooks, rate
// allocation, head layouts, plan construction and the decode kernel's K-block slot
// order), built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitize.py. Randomized over seeds; every check aborts with a message.
// It links the host source alone (no GPU code, no device calls).
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "gtq_internal.h"

using namespace gtq;

static int g_checks = 0;
#define CHECK(c, ...)                                              \
  do {                                                             \
    ++g_checks;                                                    \
    if (!(c)) {                                                    \
      fprintf(stderr, "CHECK failed at line %d: %s: ", __LINE__, #c); \
      fprintf(stderr, __VA_ARGS__);                                \
      fprintf(stderr, "\n");                                       \
      abort();                                                     \
    }                                                              \
  } while (0)

// splitmix64
struct Rng {
  uint64_t s;
  explicit Rng(uint64_t seed) : s(seed) {}
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
  int below(int n) { return (int)(next() % (uint64_t)n); }
  double unit() { return (double)(next() >> 11) * (1.0 / 9007199254740992.0); }
  float normal() {  // Box-Muller
    const double u = unit() + 1e-300, v = unit();
    return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v));
  }
};

// rates in [lo, hi] per block summing to `budget` (lo * 64 <= budget <= hi * 64)
static void random_rates(Rng& r, int lo, int hi, int budget, uint8_t* out) {
  int total = 0;
  for (int j = 0; j < kJ; ++j) {
    out[j] = (uint8_t)lo;
    total += lo;
  }
  // a skewed mix: some draws favour a few blocks, others spread evenly
  const int mode = r.below(3);
  while (total < budget) {
    int j = mode == 0 ? r.below(kJ) : mode == 1 ? r.below(8) * 8 + r.below(8) % 2 : r.below(kJ / 4) * 4;
    for (int t = 0; t < kJ && out[j] >= hi; ++t) j = (j + 1) % kJ;
    ++out[j];
    ++total;
  }
}

static void check_tables() {
  double d[5];
  CHECK(gtq_rate_distortion(4, d) == GTQ_OK, "%s", gtq_last_error());
  CHECK(fabs(d[0] - 1.0) < 1e-12, "D(0) = %.17g", d[0]);
  for (int b = 1; b <= 4; ++b) {
    CHECK(d[b] < d[b - 1] && d[b] > 0.0, "D not decreasing at %d", b);
    // the Panter-Dite high-rate bound sqrt(3) pi / 2 * 4^-b is an upper estimate for b >= 1
    CHECK(d[b] <= 2.73 * pow(4.0, -b), "D(%d) = %g above the high-rate estimate", b, d[b]);
  }
  for (int b = 2; b <= 4; ++b)  // convex in b: the marginal gains shrink
    CHECK(d[b - 2] - d[b - 1] > d[b - 1] - d[b], "D not convex at %d", b);
  CHECK(gtq_rate_distortion(0, d) == GTQ_EINVAL, "b_max 0 accepted");
  CHECK(gtq_rate_distortion(5, d) == GTQ_EINVAL, "b_max 5 accepted");
  CHECK(gtq_rate_distortion(4, nullptr) == GTQ_EINVAL, "NULL accepted");
  for (int b = 1; b <= 4; ++b) {
    float c[16], t[16];
    memset(t, 0, sizeof(t));
    CHECK(gtq_codebook(b, c, t) == GTQ_OK, "%s", gtq_last_error());
    const int n = 1 << b;
    for (int k = 0; k < n; ++k) {
      CHECK(c[k] == -c[n - 1 - k], "codebook %d not symmetric at %d", b, k);
      CHECK(k == 0 || c[k] > c[k - 1], "codebook %d not ascending at %d", b, k);
      CHECK((float)(_Float16)c[k] == c[k], "centroid %d/%d not binary16", b, k);
    }
    for (int k = 0; k + 1 < n; ++k)
      CHECK(c[k] < t[k] && t[k] < c[k + 1], "threshold %d/%d not between its centroids", b, k);
  }
  float c[16], t[16];
  CHECK(gtq_codebook(0, c, t) == GTQ_EINVAL && gtq_codebook(5, c, t) == GTQ_EINVAL, "bad bits accepted");
}

// the allocation: rates in [b_min, b_max] summing to the budget, and no single bit moved
// from one block to another lowers the proxy sum_j s_j D(b_j) (with D convex this local
// condition is the global optimum of the separable problem)
static void check_alloc(Rng& r) {
  double d[5];
  gtq_rate_distortion(4, d);
  const int nq = 1 + r.below(6), nk = 1 + r.below(9);
  std::vector<float> q((size_t)nq * kD), k((size_t)nk * kD);
  std::vector<float> scale(kD);
  for (int i = 0; i < kD; ++i) scale[i] = (float)exp(4.0 * (r.unit() - 0.5));  // energy spread
  for (int i = 0; i < nq * kD; ++i) q[i] = r.normal() * scale[i % kD];
  for (int i = 0; i < nk * kD; ++i) k[i] = r.normal() * scale[(i * 7) % kD];
  const int b_min = 1 + r.below(4), b_max = b_min + r.below(5 - b_min);
  const int budget = kJ * b_min + r.below(kJ * (b_max - b_min) + 1);
  const int layout = r.below(2) ? GTQ_ROPE_HALF : GTQ_ROPE_INTERLEAVED;
  uint8_t rates[kJ];
  double s[kJ], proxy = -1.0;
  CHECK(gtq_alloc_rates(q.data(), nq, k.data(), nk, kD, layout, b_min, b_max, budget, rates, s, &proxy) == GTQ_OK,
        "%s", gtq_last_error());
  int sum = 0;
  double p = 0.0;
  for (int j = 0; j < kJ; ++j) {
    CHECK(rates[j] >= b_min && rates[j] <= b_max, "rate %d of block %d outside [%d, %d]", rates[j], j, b_min, b_max);
    CHECK(s[j] >= 0.0 && isfinite(s[j]), "score %d = %g", j, s[j]);
    sum += rates[j];
    p += s[j] * d[rates[j]];
  }
  CHECK(sum == budget, "rates sum to %d, budget %d", sum, budget);
  CHECK(fabs(p - proxy) <= 1e-9 * fabs(p) + 1e-300, "proxy %g vs %g", proxy, p);
  for (int i = 0; i < kJ; ++i) {
    if (rates[i] <= b_min) continue;
    for (int j = 0; j < kJ; ++j) {
      if (j == i || rates[j] >= b_max) continue;
      const double delta = s[i] * (d[rates[i] - 1] - d[rates[i]]) - s[j] * (d[rates[j]] - d[rates[j] + 1]);
      CHECK(delta >= -1e-12 * (fabs(p) + 1e-300), "moving a bit from %d to %d lowers the proxy by %g", i, j, -delta);
    }
  }
  // argument errors leave no partial state and name themselves
  CHECK(gtq_alloc_rates(q.data(), nq, k.data(), nk, kD, layout, b_min, b_max, kJ * b_max + 1, rates, s, &proxy) ==
            GTQ_EINVAL,
        "budget above 64 b_max accepted");
  CHECK(gtq_alloc_rates(nullptr, nq, k.data(), nk, kD, layout, 1, 4, 128, rates, nullptr, nullptr) == GTQ_EINVAL,
        "NULL accepted");
  CHECK(gtq_alloc_rates(q.data(), 0, k.data(), nk, kD, layout, 1, 4, 128, rates, nullptr, nullptr) == GTQ_EINVAL,
        "n_q 0 accepted");
  CHECK(gtq_alloc_rates(q.data(), nq, k.data(), nk, 64, layout, 1, 4, 128, rates, nullptr, nullptr) ==
            GTQ_EUNSUPPORTED,
        "head_dim 64 accepted");
  CHECK(strlen(gtq_last_error()) > 0, "empty error message");
}

// a head's layout and the decode kernel's tables describe the same record
static void check_head(const uint8_t* rates, int layout, const gtq_head_layout& lay, const DevHead& dh, int n1,
                       int n4) {
  int dims = 0, bits = 0;
  bool seen[kD] = {};
  for (int g = 0; g < lay.n_groups; ++g) {
    CHECK(g == 0 || lay.rate[g] > lay.rate[g - 1], "groups not ascending");
    int cnt = 0;
    for (int j = 0; j < kJ; ++j) cnt += rates[j] == lay.rate[g];
    CHECK(lay.dim[g] == 2 * cnt, "group %d dim %d for %d blocks", g, lay.dim[g], cnt);
    CHECK(lay.bit_offset[g] == bits, "group %d bit offset", g);
    bits += lay.dim[g] * lay.rate[g];
    for (int i = 0; i < lay.dim[g]; ++i) {
      const int c = lay.coord[dims + i];
      CHECK(c >= 0 && c < kD && !seen[c], "coordinate %d repeated or out of range", c);
      seen[c] = true;
      // the coordinate belongs to a block of this group's rate
      const int j = layout == GTQ_ROPE_HALF ? c % kJ : c / 2;
      CHECK(rates[j] == lay.rate[g], "coordinate %d in the wrong group", c);
      CHECK(dh.coord[dims + i] == c, "device coord table differs");
    }
    dims += lay.dim[g];
  }
  CHECK(dims == kD, "group dims sum to %d", dims);
  CHECK(lay.k_words == (bits + 31) / 32, "k_words %d for %d bits", lay.k_words, bits);
  CHECK(dh.n_groups == lay.n_groups && dh.nkb <= kMaxKB - 1, "nkb %d", dh.nkb);
  // slot order: n1 rate-1 slots of group 0, then n4 rate-4 slots of the last group
  for (int s = 0; s < n1; ++s) CHECK((dh.kb_rg[s] & 0xFF) == 1 && (dh.kb_rg[s] >> 8) == 0, "slot %d not rate 1", s);
  for (int s = n1; s < n1 + n4; ++s)
    CHECK((dh.kb_rg[s] & 0xFF) == 4 && (dh.kb_rg[s] >> 8) == dh.n_groups - 1, "slot %d not rate 4", s);
  for (int s = dh.nkb; s < kMaxKB; ++s)
    CHECK(dh.kb_rg[s] == dh.kb_rg[0] && dh.kb_bit[s] == dh.kb_bit[0], "unused slot %d not slot 0", s);
  // every record position maps to a distinct operand entry of a slot of its group, and the
  // slot's first bit plus rate x entry is the position's bit in the record
  bool used[kMaxKB * kKB] = {};
  for (int g = 0; g < dh.n_groups; ++g)
    for (int i = 0; i < dh.dim[g]; ++i) {
      const int kp = dh.kp_pos[dh.pos_off[g] + i];
      const int s = kp / kKB, e = kp % kKB;
      CHECK(s < dh.nkb && !used[kp], "position %d of group %d: entry %d reused or past the slots", i, g, kp);
      used[kp] = true;
      CHECK((dh.kb_rg[s] & 0xFF) == dh.rate[g] && (dh.kb_rg[s] >> 8) == g, "position %d in a slot of another group",
            i);
      CHECK(dh.kb_bit[s] + e * dh.rate[g] == dh.bit_off[g] + i * dh.rate[g], "position %d: bit %d, slot gives %d",
            i, dh.bit_off[g] + i * dh.rate[g], dh.kb_bit[s] + e * dh.rate[g]);
    }
}

static void check_plans(Rng& r) {
  const int L = 1 + r.below(3), H = 1 + r.below(4), g = 1 + r.below(4);
  const int budget = 16 * (4 + r.below(13));  // 64 .. 256
  const int layout = r.below(2) ? GTQ_ROPE_HALF : GTQ_ROPE_INTERLEAVED;
  std::vector<uint8_t> rates((size_t)L * H * kJ);
  // some plans share one head's rates across a layer (the specialized slots then cover
  // every head), others draw each head apart
  const bool shared = r.below(2);
  for (int l = 0; l < L; ++l)
    for (int h = 0; h < H; ++h) {
      uint8_t* dst = &rates[((size_t)l * H + h) * kJ];
      if (shared && h > 0) memcpy(dst, &rates[(size_t)l * H * kJ], kJ);
      else random_rates(r, 1, 4, budget, dst);
    }
  size_t krot = 0;
  for (size_t hh = 0; hh < (size_t)L * H; ++hh) {
    gtq_head_layout lay;
    CHECK(gtq_head_layout_from_rates(&rates[hh * kJ], layout, &lay) == GTQ_OK, "%s", gtq_last_error());
    for (int gg = 0; gg < lay.n_groups; ++gg) krot += (size_t)lay.dim[gg] * lay.dim[gg];
  }
  std::vector<float> k_rot(krot), v_rot((size_t)L * H * kD * kD);
  for (auto& x : k_rot) x = r.normal() * 0.1f;
  for (auto& x : v_rot) x = r.normal() * 0.1f;
  gtq_plan_desc d{};
  d.n_layers = L;
  d.n_kv_heads = H;
  d.n_q_heads = H * g;
  d.head_dim = kD;
  d.rope_layout = layout;
  d.k_budget = budget;
  d.v_bits = 1 + r.below(4);
  d.flags = GTQ_PLAN_HOST_ONLY;
  d.k_rates = rates.data();
  d.k_rot = k_rot.data();
  d.v_rot = v_rot.data();
  gtq_plan p;
  CHECK(plan_build_host(&d, &p) == GTQ_OK, "%s", gtq_last_error());
  CHECK(p.k_words == 2 * budget / 32, "plan k_words");
  for (int l = 0; l < L; ++l) {
    const int n1 = p.layer_n1[l], n4 = p.layer_n4[l];
    CHECK(n1 >= 0 && n4 >= 0 && n1 <= 3 && n4 <= 3 && n1 + n4 <= 4, "layer %d: n1 %d n4 %d", l, n1, n4);
    for (int h = 0; h < H; ++h) {
      const size_t hh = (size_t)l * H + h;
      const DevHead& dh = p.heads[hh];
      check_head(&rates[hh * kJ], layout, p.layouts[hh], dh, n1, n4);
      CHECK(n1 <= (dh.rate[0] == 1 ? dh.nkb_g[0] : 0), "n1 past the rate-1 blocks");
      CHECK(n4 <= (dh.rate[dh.n_groups - 1] == 4 ? dh.nkb_g[dh.n_groups - 1] : 0), "n4 past the rate-4 blocks");
    }
    // the specialized counts are the largest that every head of the layer supports
    // (within the caps)
    int m1 = 3, m4 = 3;
    for (int h = 0; h < H; ++h) {
      const DevHead& dh = p.heads[(size_t)l * H + h];
      m1 = std::min(m1, dh.rate[0] == 1 ? dh.nkb_g[0] : 0);
      m4 = std::min(m4, dh.rate[dh.n_groups - 1] == 4 ? dh.nkb_g[dh.n_groups - 1] : 0);
    }
    CHECK(n1 == m1 && n4 == std::min(m4, 4 - m1), "layer %d: counts not maximal", l);
  }
  // the transposed V rotations and the split rotations: 16 Pi = hi + lo to binary16 accuracy
  for (size_t hh = 0; hh < (size_t)L * H; ++hh) {
    const DevHead& dh = p.heads[hh];
    const float* v = p.rot.data() + dh.vrot_off;
    const float* vt = p.rot.data() + dh.vrot_t_off;
    for (int i = 0; i < kD; i += 17)
      for (int j = 0; j < kD; j += 13) CHECK(vt[j * kD + i] == v[i * kD + j], "V^T entry (%d, %d)", i, j);
    for (int i = 0; i < kD; i += 11)
      for (int j = 0; j < kD; j += 7) {
        _Float16 hi, lo;
        memcpy(&hi, &p.rsplit[dh.rsv_off + i * kD + j], 2);
        memcpy(&lo, &p.rsplit[dh.rsv_off + kD * kD + i * kD + j], 2);
        const double want = 16.0 * v[i * kD + j];
        // hi takes 11 significant bits, lo the next 11 (its binary16 subnormal step is 2^-24)
        CHECK(fabs((double)(float)hi + (double)(float)lo - want) <= ldexp(fabs(want), -21) + ldexp(1.0, -24),
              "split V rotation (%d, %d): %.9g + %.9g vs %.9g", i, j, (double)(float)hi, (double)(float)lo, want);
      }
  }
  // cache sizes follow the record layout
  gtq_cache_sizes cs;
  CHECK(gtq_cache_bytes(&p, 3, 64, &cs) == GTQ_OK, "%s", gtq_last_error());
  CHECK(cs.k_codes_bytes == (size_t)3 * H * 64 * p.k_words * 4, "k_codes bytes");
  CHECK(cs.v_codes_bytes == (size_t)3 * H * (64 / GTQ_VBLOCK) * 32 * d.v_bits * 4, "v_codes bytes");
  CHECK(cs.logical_bits_per_token == 2 * budget + kD * d.v_bits, "logical bits");
  CHECK(gtq_cache_bytes(&p, 3, 65, &cs) == GTQ_EINVAL, "capacity 65 accepted");
  gtq_head_layout out;
  CHECK(gtq_plan_layout(&p, L, 0, &out) == GTQ_EINVAL, "layer out of range accepted");
  CHECK(gtq_plan_layout(&p, L - 1, H - 1, &out) == GTQ_OK, "%s", gtq_last_error());
  // invalid descriptions fail with a message
  gtq_plan bad;
  gtq_plan_desc e = d;
  e.k_budget = budget + 16 > 256 ? budget - 16 : budget + 16;  // rates no longer sum to it
  CHECK(plan_build_host(&e, &bad) == GTQ_EINVAL, "rates not summing to k_budget accepted");
  e = d;
  e.n_q_heads = H * g + 1;
  CHECK(H == 1 || plan_build_host(&e, &bad) == GTQ_EINVAL, "n_q not a multiple of n_kv accepted");
  e = d;
  e.k_budget = 100;
  CHECK(plan_build_host(&e, &bad) == GTQ_EINVAL, "k_budget 100 accepted");
  e = d;
  e.v_rot = nullptr;
  CHECK(plan_build_host(&e, &bad) == GTQ_EINVAL, "NULL v_rot accepted");
  e = d;
  e.flags = 1 << 20;
  CHECK(plan_build_host(&e, &bad) == GTQ_EINVAL, "unknown flag accepted");
}

int main(int argc, char** argv) {
  const int trials = argc > 1 ? atoi(argv[1]) : 200;
  const uint64_t seed = argc > 2 ? strtoull(argv[2], nullptr, 10) : 1;
  check_tables();
  Rng r(seed);
  for (int t = 0; t < trials; ++t) check_alloc(r);
  for (int t = 0; t < trials; ++t) check_plans(r);
  // every rate mix with one rate-1 group of 1..3 K-blocks and a rate-4 group
  for (int n1b = 1; n1b <= 31; ++n1b) {
    uint8_t rt[kJ];
    for (int j = 0; j < kJ; ++j) rt[j] = j < n1b ? 1 : j < 64 - n1b ? 2 : 4;
    gtq_head_layout lay;
    DevHead dh;
    build_head(rt, GTQ_ROPE_HALF, &lay, &dh);
    const int a1 = std::min(3, dh.nkb_g[0]);
    const int a4 = std::min(std::min(3, dh.nkb_g[dh.n_groups - 1]), 4 - a1);
    order_kblocks(&dh, a1, a4);
    check_head(rt, GTQ_ROPE_HALF, lay, dh, a1, a4);
  }
  printf("host_sanitize: %d checks passed (%d trials, seed %llu)\n", g_checks, trials, (unsigned long long)seed);
  return 0;
}
