// Host-side part of libgtq: error reporting, Lloyd-Max codebooks, energy scores,
// largest-marginal-gain allocation, group layouts and host validation of plans.
// Nothing here touches the GPU.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "gtq_internal.h"

namespace gtq {

static thread_local std::string g_last_error;

gtq_status fail(gtq_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}
gtq_status ok() {
  g_last_error.clear();
  return GTQ_OK;
}

// ---------------------------------------------------------------- Lloyd-Max
// MSE-optimal scalar quantizer of a unit Gaussian (TurboQuant diagram, "paper"
// column, per-coordinate MSE scalar quantization), by Lloyd's alternation of the
// nearest-neighbour cells (edges at centroid midpoints) and the centroid
// condition (each centroid is the conditional mean of its cell).
static double pdf(double x) {
  if (isinf(x)) return 0.0;
  return exp(-0.5 * x * x) / sqrt(2.0 * M_PI);
}
static double cell_mass(double a, double b) {  // P(a < X < b)
  const double r2 = sqrt(2.0);
  if (a >= 0.0) return 0.5 * (erfc(a / r2) - erfc(b / r2));
  if (b <= 0.0) return 0.5 * (erfc(-b / r2) - erfc(-a / r2));
  return 1.0 - 0.5 * erfc(-a / r2) - 0.5 * erfc(b / r2);
}

void lloyd_max(int bits, double* c, double* mse) {
  const int n = 1 << bits;
  double edge[17];
  for (int k = 0; k < n; ++k) c[k] = 2.0 * (-1.0 + (2.0 * k + 1.0) / n);
  for (int it = 0; it < 200000; ++it) {
    edge[0] = -INFINITY;
    edge[n] = INFINITY;
    for (int k = 1; k < n; ++k) edge[k] = 0.5 * (c[k - 1] + c[k]);
    double delta = 0.0;
    for (int k = 0; k < n; ++k) {
      double nk = (pdf(edge[k]) - pdf(edge[k + 1])) / cell_mass(edge[k], edge[k + 1]);
      delta = std::max(delta, fabs(nk - c[k]));
      c[k] = nk;
    }
    if (delta < 1e-15) break;
  }
  edge[0] = -INFINITY;
  edge[n] = INFINITY;
  for (int k = 1; k < n; ++k) edge[k] = 0.5 * (c[k - 1] + c[k]);
  double s = 0.0;
  for (int k = 0; k < n; ++k) s += cell_mass(edge[k], edge[k + 1]) * c[k] * c[k];
  *mse = 1.0 - s;
}

struct Tables {
  double mse[5];
  float cent[5][16];
  float thr[5][16];
};

// binary16 round-to-nearest-even of a double, returned as float (exact).
static float round_to_half(double x) {
  _Float16 h = (_Float16)x;  // IEEE conversion, round to nearest even
  return (float)h;
}

static const Tables& tables() {
  static Tables t;
  static std::once_flag once;
  std::call_once(once, [] {
    t.mse[0] = 1.0;
    memset(t.cent, 0, sizeof(t.cent));
    memset(t.thr, 0, sizeof(t.thr));
    for (int b = 1; b <= 4; ++b) {
      double c[16];
      lloyd_max(b, c, &t.mse[b]);
      const int n = 1 << b;
      for (int k = 0; k < n; ++k) t.cent[b][k] = round_to_half(c[k]);
      // midpoint of two binary16 values is exact in fp32
      for (int k = 0; k + 1 < n; ++k)
        t.thr[b][k] = (float)(0.5 * ((double)t.cent[b][k] + (double)t.cent[b][k + 1]));
    }
  });
  return t;
}

static uint32_t half_bits(float x) {
  const _Float16 h = (_Float16)x;  // exact: the centroids are binary16 values
  uint16_t u;
  memcpy(&u, &h, 2);
  return u;
}

void fill_codebook(DevCodebook* cb) {
  const Tables& t = tables();
  memcpy(cb->c, t.cent, sizeof(cb->c));
  memcpy(cb->t, t.thr, sizeof(cb->t));
  memset(cb->pair, 0, sizeof(cb->pair));
  for (int b = 1; b <= 4; ++b) {
    const int base = ((1 << (2 * b)) - 4) / 3, m = (1 << b) - 1;
    for (int x = 0; x < (1 << (2 * b)); ++x)
      cb->pair[base + x] = half_bits(t.cent[b][x & m]) | (half_bits(t.cent[b][x >> b]) << 16);
  }
  for (int x = 0; x < 256; ++x) {
    for (int j = 0; j < 4; ++j) cb->oct1[x][j] = cb->pair[0 + ((x >> (2 * j)) & 3)];
    for (int j = 0; j < 2; ++j) cb->quad2[x][j] = cb->pair[4 + ((x >> (4 * j)) & 15)];
  }
}

// ---------------------------------------------------------------- layouts
static inline void block_coords(int j, int layout, int* a, int* b) {
  if (layout == GTQ_ROPE_HALF) {
    *a = j;
    *b = j + kJ;
  } else {
    *a = 2 * j;
    *b = 2 * j + 1;
  }
}

// Equal-rate groups in ascending rate (Block-GTQ abstract, 5th sentence) and the
// decode kernel's K-block table. Rates must already be validated in [1, 4].
void build_head(const uint8_t* rates, int layout, gtq_head_layout* lay, DevHead* dh) {
  memset(lay, 0, sizeof(*lay));
  memset(dh, 0, sizeof(*dh));
  int pos = 0, bit = 0, kp = 0, kb = 0, rot = 0;
  for (int r = 1; r <= 4; ++r) {
    int count = 0;
    for (int j = 0; j < kJ; ++j) count += (rates[j] == r);
    if (!count) continue;
    const int g = lay->n_groups++;
    const int d = 2 * count;
    lay->rate[g] = r;
    lay->dim[g] = d;
    lay->bit_offset[g] = bit;
    lay->rot_offset[g] = rot;
    dh->rate[g] = r;
    dh->dim[g] = d;
    dh->bit_off[g] = bit;
    dh->pos_off[g] = pos;
    dh->kp_off[g] = kp;
    dh->krot_off[g] = rot;  // relative; made absolute by the plan
    const int nk = (d + kKB - 1) / kKB;
    dh->nkb_g[g] = nk;
    for (int i = 0; i < nk; ++i) {
      dh->kb_bit[kb + i] = bit + i * kKB * r;
      dh->kb_rg[kb + i] = r | (g << 8);
    }
    for (int j = 0; j < kJ; ++j) {
      if (rates[j] != r) continue;
      int a, b;
      block_coords(j, layout, &a, &b);
      lay->coord[pos] = a;
      dh->coord[pos] = (uint8_t)a;
      ++pos;
      lay->coord[pos] = b;
      dh->coord[pos] = (uint8_t)b;
      ++pos;
    }
    bit += d * r;
    kp += nk * kKB;
    kb += nk;
    rot += d * d;
  }
  dh->n_groups = lay->n_groups;
  dh->nkb = kb;
  for (int i = kb; i < kMaxKB; ++i) {  // unused slots: valid reads, multiplied by zero
    dh->kb_bit[i] = dh->kb_bit[0];
    dh->kb_rg[i] = dh->kb_rg[0];
  }
  dh->krot_floats = rot;
  lay->k_words = (bit + 31) / 32;
  for (int g = 0; g < dh->n_groups; ++g)
    for (int i = 0; i < dh->dim[g]; ++i) dh->kp_pos[dh->pos_off[g] + i] = (uint8_t)(dh->kp_off[g] + i);
}

// Puts a head's K-blocks in the slot order the decode kernel specializes on: the first
// n1 blocks of the rate-1 group (group 0), then the first n4 blocks of the rate-4 group
// (the last group), then the remaining blocks in group order. Every head of a layer
// gets the layer's (n1, n4), so that these slots have the same rate in every head.
void order_kblocks(DevHead* dh, int n1, int n4) {
  int src[kMaxKB], ns = 0;
  int first[kMaxGroups], k = 0;
  for (int g = 0; g < dh->n_groups; ++g) {
    first[g] = k;
    k += dh->nkb_g[g];
  }
  const int gl = dh->n_groups - 1;
  for (int i = 0; i < n1; ++i) src[ns++] = first[0] + i;
  for (int i = 0; i < n4; ++i) src[ns++] = first[gl] + i;
  for (int g = 0; g < dh->n_groups; ++g)
    for (int i = (g == 0 ? n1 : 0) + (g == gl ? n4 : 0); i < dh->nkb_g[g]; ++i) src[ns++] = first[g] + i;
  int bit[kMaxKB], rg[kMaxKB], slot_of[kMaxKB];
  for (int s = 0; s < ns; ++s) {
    bit[s] = dh->kb_bit[src[s]];
    rg[s] = dh->kb_rg[src[s]];
    slot_of[src[s]] = s;
  }
  for (int s = 0; s < kMaxKB; ++s) {
    dh->kb_bit[s] = s < ns ? bit[s] : bit[0];
    dh->kb_rg[s] = s < ns ? rg[s] : rg[0];
  }
  for (int g = 0; g < dh->n_groups; ++g)
    for (int i = 0; i < dh->dim[g]; ++i)
      dh->kp_pos[dh->pos_off[g] + i] = (uint8_t)(kKB * slot_of[first[g] + i / kKB] + i % kKB);
}

}  // namespace gtq

using namespace gtq;

extern "C" {

const char* gtq_last_error(void) { return g_last_error.c_str(); }

gtq_status gtq_rate_distortion(int32_t b_max, double* d_out) {
  if (!d_out) return fail(GTQ_EINVAL, "gtq_rate_distortion: d_out is NULL");
  if (b_max < 1 || b_max > 4) return fail(GTQ_EINVAL, "gtq_rate_distortion: b_max must be in [1, 4]");
  const Tables& t = tables();
  for (int b = 0; b <= b_max; ++b) d_out[b] = t.mse[b];
  return ok();
}

gtq_status gtq_codebook(int32_t bits, float* centroids, float* thresholds) {
  if (bits < 1 || bits > 4) return fail(GTQ_EINVAL, "gtq_codebook: bits must be in [1, 4]");
  const Tables& t = tables();
  const int n = 1 << bits;
  if (centroids)
    for (int k = 0; k < n; ++k) centroids[k] = t.cent[bits][k];
  if (thresholds)
    for (int k = 0; k + 1 < n; ++k) thresholds[k] = t.thr[bits][k];
  return ok();
}

gtq_status gtq_alloc_rates(const float* q_cal, int64_t n_q, const float* k_cal, int64_t n_k,
                           int32_t head_dim, int32_t rope_layout, int32_t b_min, int32_t b_max,
                           int32_t budget, uint8_t* rates_out, double* scores_out,
                           double* proxy_out) {
  if (!q_cal || !k_cal || !rates_out) return fail(GTQ_EINVAL, "gtq_alloc_rates: NULL pointer");
  if (head_dim != kD) return fail(GTQ_EUNSUPPORTED, "gtq_alloc_rates: head_dim must be 128");
  if (n_q < 1 || n_k < 1) return fail(GTQ_EINVAL, "gtq_alloc_rates: n_q and n_k must be >= 1");
  if (rope_layout != GTQ_ROPE_HALF && rope_layout != GTQ_ROPE_INTERLEAVED)
    return fail(GTQ_EINVAL, "gtq_alloc_rates: bad rope_layout");
  if (!(1 <= b_min && b_min <= b_max && b_max <= 4))
    return fail(GTQ_EINVAL, "gtq_alloc_rates: need 1 <= b_min <= b_max <= 4");
  if (budget < kJ * b_min || budget > kJ * b_max)
    return fail(GTQ_EINVAL, "gtq_alloc_rates: budget outside [64*b_min, 64*b_max]");

  // Energy score per RoPE block (abstract, 3rd sentence): mean query block energy
  // times mean key block energy, fp64 with compensated (Neumaier) summation.
  double s[kJ];
  for (int j = 0; j < kJ; ++j) {
    int a, b;
    block_coords(j, rope_layout, &a, &b);
    double e[2];
    const float* src[2] = {q_cal, k_cal};
    const int64_t cnt[2] = {n_q, n_k};
    for (int w = 0; w < 2; ++w) {
      double sum = 0.0, comp = 0.0;
      for (int64_t r = 0; r < cnt[w]; ++r) {
        const double x = src[w][r * kD + a], y = src[w][r * kD + b];
        const double v = x * x + y * y;
        const double t = sum + v;
        comp += (fabs(sum) >= fabs(v)) ? (sum - t) + v : (v - t) + sum;
        sum = t;
      }
      e[w] = (sum + comp) / (double)cnt[w];
    }
    s[j] = e[0] * e[1];
    if (!isfinite(s[j])) return fail(GTQ_EINVAL, "gtq_alloc_rates: non-finite calibration data");
  }
  // Largest marginal gain (abstract, 4th sentence): repeatedly give one bit to the
  // block whose proxy sum_j s_j D(b_j) drops most; ties go to the smallest block.
  const Tables& t = tables();
  int rate[kJ];
  int total = 0;
  for (int j = 0; j < kJ; ++j) {
    rate[j] = b_min;
    total += b_min;
  }
  while (total < budget) {
    int best = -1;
    double best_gain = -INFINITY;
    for (int j = 0; j < kJ; ++j) {
      if (rate[j] >= b_max) continue;
      const double gain = s[j] * (t.mse[rate[j]] - t.mse[rate[j] + 1]);
      if (gain > best_gain) {
        best_gain = gain;
        best = j;
      }
    }
    ++rate[best];
    ++total;
  }
  double proxy = 0.0;
  for (int j = 0; j < kJ; ++j) {
    rates_out[j] = (uint8_t)rate[j];
    if (scores_out) scores_out[j] = s[j];
    proxy += s[j] * t.mse[rate[j]];
  }
  if (proxy_out) *proxy_out = proxy;
  return ok();
}

gtq_status gtq_head_layout_from_rates(const uint8_t* rates, int32_t rope_layout,
                                      gtq_head_layout* out) {
  if (!rates || !out) return fail(GTQ_EINVAL, "gtq_head_layout_from_rates: NULL pointer");
  if (rope_layout != GTQ_ROPE_HALF && rope_layout != GTQ_ROPE_INTERLEAVED)
    return fail(GTQ_EINVAL, "gtq_head_layout_from_rates: bad rope_layout");
  for (int j = 0; j < kJ; ++j)
    if (rates[j] < 1 || rates[j] > 4)
      return fail(GTQ_EINVAL, "gtq_head_layout_from_rates: rates must be in [1, 4]");
  DevHead dh;
  build_head(rates, rope_layout, out, &dh);
  return ok();
}

gtq_status gtq_plan_layout(const gtq_plan* plan, int32_t layer, int32_t kv_head,
                           gtq_head_layout* out) {
  if (!plan || !out) return fail(GTQ_EINVAL, "gtq_plan_layout: NULL pointer");
  if (layer < 0 || layer >= plan->n_layers || kv_head < 0 || kv_head >= plan->n_kv)
    return fail(GTQ_EINVAL, "gtq_plan_layout: layer or kv_head out of range");
  *out = plan->layouts[(size_t)layer * plan->n_kv + kv_head];
  return ok();
}

gtq_status gtq_cache_bytes(const gtq_plan* plan, int32_t batch, int64_t capacity,
                           gtq_cache_sizes* out) {
  if (!plan || !out) return fail(GTQ_EINVAL, "gtq_cache_bytes: NULL pointer");
  if (batch < 1 || capacity < 1 || capacity % GTQ_SEQ_ALIGN)
    return fail(GTQ_EINVAL, "gtq_cache_bytes: batch >= 1 and capacity a positive multiple of 32");
  const size_t bh = (size_t)batch * plan->n_kv;
  out->k_words = plan->k_words;
  out->v_words_per_block = 32 * plan->v_bits;
  out->k_codes_bytes = bh * capacity * plan->k_words * 4;
  out->k_norms_bytes = bh * capacity * kNS * 4;
  out->v_codes_bytes = bh * (capacity / GTQ_VBLOCK) * 32 * plan->v_bits * 4;
  out->v_norms_bytes = bh * capacity * 4;
  out->logical_bits_per_token = 2 * plan->k_budget + kD * plan->v_bits + ((plan->flags & GTQ_PLAN_QJL) ? kD : 0);
  out->bytes_per_token = plan->k_words * 4 + kNS * 4 + 16 * plan->v_bits + 4;
  return ok();
}

}  // extern "C"

namespace gtq {
// Host validation and construction of a plan (everything except the device copy).
gtq_status plan_build_host(const gtq_plan_desc* d, gtq_plan* p) {
  if (!d) return fail(GTQ_EINVAL, "gtq_plan_create: desc is NULL");
  if (d->head_dim != kD) return fail(GTQ_EUNSUPPORTED, "gtq_plan_create: head_dim must be 128");
  if (d->n_layers < 1 || d->n_kv_heads < 1 || d->n_q_heads < 1)
    return fail(GTQ_EINVAL, "gtq_plan_create: layer and head counts must be >= 1");
  if (d->n_q_heads % d->n_kv_heads)
    return fail(GTQ_EINVAL, "gtq_plan_create: n_q_heads must be a multiple of n_kv_heads");
  if (d->rope_layout != GTQ_ROPE_HALF && d->rope_layout != GTQ_ROPE_INTERLEAVED)
    return fail(GTQ_EINVAL, "gtq_plan_create: bad rope_layout");
  if (d->v_bits < 1 || d->v_bits > 4) return fail(GTQ_EINVAL, "gtq_plan_create: v_bits must be in [1, 4]");
  if (d->k_budget < kJ || d->k_budget > 4 * kJ || d->k_budget % 16)
    return fail(GTQ_EINVAL, "gtq_plan_create: k_budget must be a multiple of 16 in [64, 256]");
  if (d->flags & ~(GTQ_PLAN_HOST_ONLY | GTQ_PLAN_NORM_CORRECT | GTQ_PLAN_QJL))
    return fail(GTQ_EINVAL, "gtq_plan_create: unknown flags");
  if (!d->k_rates || !d->k_rot || !d->v_rot) return fail(GTQ_EINVAL, "gtq_plan_create: NULL table");
  const bool qjl = (d->flags & GTQ_PLAN_QJL) != 0;
  if (qjl != (d->qjl != nullptr))
    return fail(GTQ_EINVAL, "gtq_plan_create: GTQ_PLAN_QJL and the qjl matrices go together");
  if (qjl && 2 * d->k_budget / 32 + 5 > 16)
    return fail(GTQ_EUNSUPPORTED, "gtq_plan_create: QJL needs k_budget <= 176 (records of at most 16 words)");
  p->n_layers = d->n_layers;
  p->n_kv = d->n_kv_heads;
  p->n_q = d->n_q_heads;
  p->rope_layout = d->rope_layout;
  p->k_budget = d->k_budget;
  p->v_bits = d->v_bits;
  p->k_words = 2 * d->k_budget / 32 + (qjl ? 5 : 0);  // MSE words, then the sketch and gamma
  p->flags = d->flags;
  const size_t nh = (size_t)d->n_layers * d->n_kv_heads;
  p->heads.resize(nh);
  p->layouts.resize(nh);
  size_t krot_total = 0;
  for (size_t h = 0; h < nh; ++h) {
    const uint8_t* r = d->k_rates + h * kJ;
    int sum = 0;
    for (int j = 0; j < kJ; ++j) {
      if (r[j] < 1 || r[j] > 4) return fail(GTQ_EINVAL, "gtq_plan_create: rates must be in [1, 4]");
      sum += r[j];
    }
    if (sum != d->k_budget)
      return fail(GTQ_EINVAL, "gtq_plan_create: a head's rates do not sum to k_budget (head " +
                                  std::to_string(h) + ")");
    build_head(r, d->rope_layout, &p->layouts[h], &p->heads[h]);
    krot_total += p->heads[h].krot_floats;
  }
  // per layer: how many leading rate-1 and rate-4 K-blocks every head has (at most 3
  // each and 4 together: the decode kernel is compiled for these counts)
  p->layer_n1.assign(d->n_layers, 0);
  p->layer_n4.assign(d->n_layers, 0);
  for (int l = 0; l < d->n_layers; ++l) {
    int n1 = 3, n4 = 3;
    for (int h = 0; h < d->n_kv_heads; ++h) {
      const DevHead& dh = p->heads[(size_t)l * d->n_kv_heads + h];
      n1 = std::min(n1, dh.rate[0] == 1 ? dh.nkb_g[0] : 0);
      n4 = std::min(n4, dh.rate[dh.n_groups - 1] == 4 ? dh.nkb_g[dh.n_groups - 1] : 0);
    }
    n4 = std::min(n4, 4 - n1);
    p->layer_n1[l] = n1;
    p->layer_n4[l] = n4;
    for (int h = 0; h < d->n_kv_heads; ++h) order_kblocks(&p->heads[(size_t)l * d->n_kv_heads + h], n1, n4);
  }
  // rotation pool: all K group rotations (as given), all V rotations, then the V
  // rotations transposed (read column-wise by the attention kernel's last step)
  const size_t vsz = (size_t)kD * kD;
  try {
    p->rot.resize(krot_total + (qjl ? 3 : 2) * nh * vsz);  // (and the sketch matrices)
  } catch (...) {
    return fail(GTQ_ENOMEM, "gtq_plan_create: host allocation failed");
  }
  memcpy(p->rot.data(), d->k_rot, krot_total * sizeof(float));
  memcpy(p->rot.data() + krot_total, d->v_rot, nh * vsz * sizeof(float));
  for (size_t h = 0; h < nh; ++h) {
    const float* src = d->v_rot + h * vsz;
    float* dst = p->rot.data() + krot_total + nh * vsz + h * vsz;
    for (int i = 0; i < kD; ++i)
      for (int j = 0; j < kD; ++j) dst[(size_t)j * kD + i] = src[(size_t)i * kD + j];
  }
  size_t off = 0;
  for (size_t h = 0; h < nh; ++h) {
    DevHead& dh = p->heads[h];
    for (int g = 0; g < dh.n_groups; ++g) dh.krot_off[g] += (int64_t)off;
    off += dh.krot_floats;
    dh.vrot_off = (int64_t)(krot_total + h * vsz);
    dh.vrot_t_off = (int64_t)(krot_total + nh * vsz + h * vsz);
    dh.mse_words = 2 * d->k_budget / 32;
    dh.qjl = qjl ? 1 : 0;
    dh.qjl_off = qjl ? (int64_t)(krot_total + 2 * nh * vsz + h * vsz) : 0;
    if (qjl) {
      const float* src = d->qjl + h * vsz;
      for (size_t e = 0; e < vsz; ++e)
        if (!isfinite(src[e])) return fail(GTQ_EINVAL, "gtq_plan_create: non-finite QJL matrix");
      memcpy(p->rot.data() + dh.qjl_off, src, vsz * sizeof(float));
    }
    // a randomized Hadamard Pi_V: every entry is +-c, c = fp32(1/sqrt(128)), with the
    // Sylvester sign pattern times a per-column sign (read off row 0)
    {
      const float c = 0.0883883461356163f;  // fp32 nearest to 1/sqrt(128)
      const float* v = d->v_rot + h * vsz;
      bool had = true;
      for (int j = 0; j < kD && had; ++j) had = (v[j] == c || v[j] == -c);
      for (int i = 0; i < kD && had; ++i)
        for (int j = 0; j < kD && had; ++j) {
          const float sj = v[j] > 0.f ? 1.f : -1.f;
          const float hij = (__builtin_popcount((unsigned)(i & j)) & 1) ? -1.f : 1.f;
          had = v[(size_t)i * kD + j] == sj * hij * c;
        }
      dh.v_hadamard = had ? 1 : 0;
      for (int j = 0; j < kD; ++j) dh.vsign[j] = v[j] > 0.f ? 1.f : -1.f;
      p->layouts[h].v_hadamard = dh.v_hadamard;
    }
    for (size_t i = 0; i < (size_t)dh.krot_floats; ++i)
      if (!isfinite(p->rot[dh.krot_off[0] + i]))
        return fail(GTQ_EINVAL, "gtq_plan_create: non-finite K rotation");
  }
  // split rotations: 16 Pi = hi + lo + O(2^-24), both binary16, as 128 x 128 matrices
  // (the key groups' Pi_g on the diagonal blocks of record position order, zeros across
  // groups), so that the append's MFMA tiles of 16 outputs need no per-group padding
  {
    size_t total = 0;
    for (size_t h = 0; h < nh; ++h) {
      DevHead& dh = p->heads[h];
      dh.rsk_off = (int64_t)total;
      total += 2 * vsz;
      dh.rsv_off = (int64_t)total;
      total += 2 * vsz;
    }
    try {
      p->rsplit.assign(total, 0);
    } catch (...) {
      return fail(GTQ_ENOMEM, "gtq_plan_create: host allocation failed");
    }
    // Pi (d x d, row-major) into rows and columns [p0, p0 + d) of the 128 x 128 pair at off
    auto put = [&](const float* src, int d, int p0, size_t off) {
      for (int i = 0; i < d; ++i)
        for (int j = 0; j < d; ++j) {
          const float x = kRotSplitScale * src[(size_t)i * d + j];
          const _Float16 hi = (_Float16)x;
          const _Float16 lo = (_Float16)(x - (float)hi);
          const size_t e = (size_t)(p0 + i) * kD + (p0 + j);
          memcpy(&p->rsplit[off + e], &hi, 2);
          memcpy(&p->rsplit[off + vsz + e], &lo, 2);
        }
    };
    for (size_t h = 0; h < nh; ++h) {
      const DevHead& dh = p->heads[h];
      for (int g = 0; g < dh.n_groups; ++g)
        put(p->rot.data() + dh.krot_off[g], dh.dim[g], dh.pos_off[g], dh.rsk_off);
      put(p->rot.data() + dh.vrot_off, kD, 0, dh.rsv_off);
    }
  }
  fill_codebook(&p->cb);
  return ok();
}
}  // namespace gtq
