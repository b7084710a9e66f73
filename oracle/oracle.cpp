// Scalar CPU oracle for the streaming-MoE per-layer decode step.
//
// TEST INFRASTRUCTURE ONLY. This file is the parity reference for the HIP
// library. Only the test suite, the package smoke check and the benchmark's
// CPU-baseline leg may load it. The product path never calls it, and it shares
// no code, header, table or constant with the HIP kernels.
//
// Style: plain loops, fp64 arithmetic, fp16 rounding (round-to-nearest-even)
// only where the precision contract puts it: the RMS-normed activation that
// feeds the GEMVs. Everything else stays in double.
//
// Citations name the source pages by these tags:
//   [MW]  "The Other Half of the Memory Wall: Serving 35B MoEs from SSD with
//         Trained Routing Prediction" (arXiv 2609.18063, HTML).
//   [RG]  the xyznot.com reading guide of the same paper.
//   [IE]  "Inside Edge0-35B: Running a 35B Sparse MoE in Under 3 GiB RAM via
//         SSD Offload and Prerouter Speculation" (orbital.net.in blog).
//   [CB]  "Edge0 streams a 35B MoE off SSD. I counted the bytes it can't
//         stream." (ai.thesatyajit.com audit).
//
// Readings where the pages are silent (each is listed in the design notes):
//   * int4 layout: element i of a row sits in 32-bit word i/8 at bits
//     4*(i%8) (low nibble first) and is a two's-complement value in [-8, 7];
//     the weight is fp16 scale[row][i/group] times that integer.
//   * top-K order: descending score, exact ties go to the lower expert id.
//   * sigmoid-group: groups are contiguous blocks of E/n experts and the
//     group score sums the two largest *biased* scores.
//   * RMSNorm: gain 1, eps added to the mean square.
//   * shared expert: added to the routed combine with no gate.
//   * slot policy: see orc_slot_policy.
//
// Pins: every function here is checked by tests/test_oracle_*.py against
// closed forms, library routines, brute force or the pages' printed numbers.

#include <cfenv>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>

namespace {

// ----------------------------------------------------------------- fp16 --

// Exact decode of an IEEE binary16 bit pattern.
double f16_to_f64(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int expo = (h >> 10) & 31;
  const int mant = h & 1023;
  double v;
  if (expo == 0) {
    v = std::ldexp(static_cast<double>(mant), -24);
  } else if (expo == 31) {
    v = mant ? NAN : INFINITY;
  } else {
    v = std::ldexp(static_cast<double>(1024 + mant), expo - 25);
  }
  return sign ? -v : v;
}

// Round a double to binary16 with round-to-nearest, ties to even.
uint16_t f64_to_f16(double v) {
  if (std::isnan(v)) return 0x7E00;
  uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  double a = std::fabs(v);
  if (a == 0.0) return sign;
  // Values at or above 65520 round to infinity (65504 is the largest finite).
  if (a >= 65520.0) return sign | 0x7C00;
  if (a < std::ldexp(1.0, -14)) {
    // Subnormal range: integer multiple of 2^-24. A result of 1024 is the
    // smallest normal number, whose bit pattern is 0x0400, so no special case.
    double m = std::nearbyint(std::ldexp(a, 24));
    return sign | static_cast<uint16_t>(m);
  }
  int ex;
  std::frexp(a, &ex);  // a = f * 2^ex, f in [0.5, 1)
  int e = ex - 1;      // a in [2^e, 2^(e+1))
  double m = std::nearbyint(std::ldexp(a, 10 - e));  // in [1024, 2048]
  if (m >= 2048.0) {
    m = 1024.0;
    e += 1;
  }
  int biased = e + 15;
  if (biased >= 31) return sign | 0x7C00;
  return sign | static_cast<uint16_t>((biased << 10) | (static_cast<int>(m) - 1024));
}

// ----------------------------------------------------------------- int4 --

// Signed value of element i of one packed row (layout reading above).
int q4_value(const uint32_t* rowq, int i) {
  uint32_t word = rowq[i / 8];
  int nib = static_cast<int>((word >> (4 * (i % 8))) & 15u);
  return nib >= 8 ? nib - 16 : nib;
}

// Weight (row o, column i) of an int4 matrix with `cols` inputs.
double q4_weight(const uint32_t* q, const uint16_t* s, int cols, int group, int o, int i) {
  const uint32_t* rowq = q + static_cast<int64_t>(o) * (cols / 8);
  double scale = f16_to_f64(s[static_cast<int64_t>(o) * (cols / group) + i / group]);
  return scale * q4_value(rowq, i);
}

// y[o] = sum_i W[o][i] x[i] with W the dequantised int4 matrix.
void q4_matvec(const uint32_t* q, const uint16_t* s, int rows, int cols, int group,
               const double* x, double* y) {
  for (int o = 0; o < rows; ++o) {
    double acc = 0.0;
    for (int i = 0; i < cols; ++i) acc += q4_weight(q, s, cols, group, o, i) * x[i];
    y[o] = acc;
  }
}

// y[o] = sum_i W[o][i] x[i] for a row-major fp16 matrix [rows, cols].
void f16_matvec(const uint16_t* W, int rows, int cols, const double* x, double* y) {
  for (int o = 0; o < rows; ++o) {
    double acc = 0.0;
    const uint16_t* row = W + static_cast<int64_t>(o) * cols;
    for (int i = 0; i < cols; ++i) acc += f16_to_f64(row[i]) * x[i];
    y[o] = acc;
  }
}

// ----------------------------------------------------------- activations --

// SiLU, the gate nonlinearity of the SwiGLU expert [MW §3.1 Math contract].
double silu(double z) { return z / (1.0 + std::exp(-z)); }

// Exact (erf) GELU used between the two head layers [MW §3.2 Head].
double gelu_erf(double z) { return 0.5 * z * (1.0 + std::erf(z / std::sqrt(2.0))); }

// ---------------------------------------------------------------- top-K --

// Indices of the k largest scores among allowed entries, in descending score
// order; equal scores go to the lower index. Returns the count found.
int topk(const double* score, const uint8_t* allowed, int n, int k, int32_t* idx) {
  std::vector<uint8_t> taken(n, 0);
  int found = 0;
  for (int slot = 0; slot < k; ++slot) {
    int best = -1;
    for (int e = 0; e < n; ++e) {
      if (taken[e] || (allowed && !allowed[e])) continue;
      if (best < 0 || score[e] > score[best]) best = e;
    }
    if (best < 0) break;
    taken[best] = 1;
    idx[slot] = best;
    ++found;
  }
  return found;
}

}  // namespace

extern "C" {

// ------------------------------------------------------ exported helpers --

void orc_f16_round(const double* in, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f64_to_f16(in[i]);
}

void orc_f16_decode(const uint16_t* in, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = f16_to_f64(in[i]);
}

// Full dequantised matrix [rows, cols] (row-major) of a packed int4 matrix.
void orc_q4_dequant(const uint32_t* q, const uint16_t* s, int rows, int cols, int group,
                    double* w) {
  for (int o = 0; o < rows; ++o)
    for (int i = 0; i < cols; ++i)
      w[static_cast<int64_t>(o) * cols + i] = q4_weight(q, s, cols, group, o, i);
}

void orc_q4_matvec(const uint32_t* q, const uint16_t* s, int rows, int cols, int group,
                   const double* x, double* y) {
  q4_matvec(q, s, rows, cols, group, x, y);
}

void orc_silu(const double* z, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = silu(z[i]);
}

void orc_gelu_erf(const double* z, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = gelu_erf(z[i]);
}

// RMSNorm with unit gain: out = h / sqrt(mean(h^2) + eps).
void orc_rmsnorm(const double* h, int d, double eps, double* out) {
  double ss = 0.0;
  for (int i = 0; i < d; ++i) ss += h[i] * h[i];
  double inv = 1.0 / std::sqrt(ss / d + eps);
  for (int i = 0; i < d; ++i) out[i] = h[i] * inv;
}

int orc_topk(const double* score, const uint8_t* allowed, int n, int k, int32_t* idx) {
  return topk(score, allowed, n, k, idx);
}

// Softmax-top-K routing [MW App. A "Softmax-topk"]: g = softmax(logits) over
// all E experts, the K largest g are selected, and with `norm` set the
// selected probabilities are renormalised to sum to one (norm_topk_prob, as
// the 35B MoESpec sets it [CB "A3B describes a model ..."]).
int orc_route_softmax_topk(const double* logits, int E, int K, int norm, int32_t* idx,
                           double* w) {
  if (K < 1 || K > E) return -1;
  double m = logits[0];
  for (int e = 1; e < E; ++e) m = std::fmax(m, logits[e]);
  std::vector<double> g(E);
  double z = 0.0;
  for (int e = 0; e < E; ++e) {
    g[e] = std::exp(logits[e] - m);
    z += g[e];
  }
  for (int e = 0; e < E; ++e) g[e] /= z;
  if (topk(g.data(), nullptr, E, K, idx) != K) return -1;
  double sel = 0.0;
  for (int k = 0; k < K; ++k) sel += g[idx[k]];
  for (int k = 0; k < K; ++k) w[k] = norm ? g[idx[k]] / sel : g[idx[k]];
  return 0;
}

// Sigmoid-group routing [MW App. A "Sigmoid-group"]: sigma = sigmoid(logits);
// selection uses the biased score sigma + bias; a group's score is the sum of
// its two largest biased scores; the best `topk_groups` groups survive; the K
// largest biased scores among survivors are selected; weights are
// scale * sigma[sel] / (sum sigma[sel] + 1e-20) on the raw sigmoid.
// Optional outputs: the biased scores [E] and the group scores [n_groups].
int orc_route_sigmoid_group(const double* logits, const double* bias, int E, int K,
                            int n_groups, int topk_groups, double scale, int32_t* idx,
                            double* w, double* sel_out, double* group_out) {
  if (n_groups < 1 || E % n_groups != 0 || topk_groups < 1 || topk_groups > n_groups)
    return -1;
  const int per = E / n_groups;
  if (per < 2 || K < 1 || K > topk_groups * per) return -1;
  std::vector<double> sig(E), sel(E);
  for (int e = 0; e < E; ++e) {
    sig[e] = 1.0 / (1.0 + std::exp(-logits[e]));
    sel[e] = sig[e] + (bias ? bias[e] : 0.0);
  }
  std::vector<double> gscore(n_groups);
  for (int g = 0; g < n_groups; ++g) {
    int32_t top2[2];
    topk(sel.data() + g * per, nullptr, per, 2, top2);
    gscore[g] = sel[g * per + top2[0]] + sel[g * per + top2[1]];
  }
  std::vector<int32_t> kept(topk_groups);
  topk(gscore.data(), nullptr, n_groups, topk_groups, kept.data());
  std::vector<uint8_t> allowed(E, 0);
  for (int j = 0; j < topk_groups; ++j)
    for (int e = 0; e < per; ++e) allowed[kept[j] * per + e] = 1;
  if (topk(sel.data(), allowed.data(), E, K, idx) != K) return -1;
  double sum = 0.0;
  for (int k = 0; k < K; ++k) sum += sig[idx[k]];
  for (int k = 0; k < K; ++k) w[k] = scale * sig[idx[k]] / (sum + 1e-20);
  if (sel_out)
    for (int e = 0; e < E; ++e) sel_out[e] = sel[e];
  if (group_out)
    for (int g = 0; g < n_groups; ++g) group_out[g] = gscore[g];
  return 0;
}

// One routed SwiGLU expert [MW §3.1 Math contract; IE "Architectural Deep
// Dive"]: y = down(silu(gate(x)) * up(x)). Gate/up are [I, d], down is [d, I],
// all int4 with fp16 group scales. The intermediate is not rounded.
void orc_expert(const uint32_t* gate_q, const uint16_t* gate_s, const uint32_t* up_q,
                const uint16_t* up_s, const uint32_t* down_q, const uint16_t* down_s, int d,
                int I, int group, const double* x, double* y) {
  std::vector<double> g(I), u(I), h(I);
  q4_matvec(gate_q, gate_s, I, d, group, x, g.data());
  q4_matvec(up_q, up_s, I, d, group, x, u.data());
  for (int i = 0; i < I; ++i) h[i] = silu(g[i]) * u[i];
  q4_matvec(down_q, down_s, d, I, group, h.data(), y);
}

// Unmerged LoRA delta [MW §3.3; RG "Unmerged Adapter Execution"]:
// y_acc += scale * B (A x), with A [r, in] and B [out, r] fp16 row-major.
void orc_lora_delta(const uint16_t* A, const uint16_t* B, int in, int out, int r, double scale,
                    const double* x, double* y_acc) {
  std::vector<double> ax(r);
  f16_matvec(A, r, in, x, ax.data());
  for (int o = 0; o < out; ++o) {
    double acc = 0.0;
    for (int j = 0; j < r; ++j) acc += f16_to_f64(B[static_cast<int64_t>(o) * r + j]) * ax[j];
    y_acc[o] += scale * acc;
  }
}

// Shared expert with an unmerged LoRA delta on each of its three projections
// (each projection is W_int4 x + (alpha/r) B A x). LoRA pointers may be null.
void orc_shared_expert(const uint32_t* gate_q, const uint16_t* gate_s, const uint32_t* up_q,
                       const uint16_t* up_s, const uint32_t* down_q, const uint16_t* down_s,
                       const uint16_t* a_gate, const uint16_t* b_gate, const uint16_t* a_up,
                       const uint16_t* b_up, const uint16_t* a_down, const uint16_t* b_down,
                       int d, int Is, int group, int r, double alpha, const double* x,
                       double* y) {
  const double c = r > 0 ? alpha / r : 0.0;
  std::vector<double> g(Is), u(Is), h(Is);
  q4_matvec(gate_q, gate_s, Is, d, group, x, g.data());
  q4_matvec(up_q, up_s, Is, d, group, x, u.data());
  if (a_gate && b_gate) orc_lora_delta(a_gate, b_gate, d, Is, r, c, x, g.data());
  if (a_up && b_up) orc_lora_delta(a_up, b_up, d, Is, r, c, x, u.data());
  for (int i = 0; i < Is; ++i) h[i] = silu(g[i]) * u[i];
  q4_matvec(down_q, down_s, d, Is, group, h.data(), y);
  if (a_down && b_down) orc_lora_delta(a_down, b_down, Is, d, r, c, h.data(), y);
}

// Inputs of one MoE layer for the oracle. Pools are stacked by expert id.
struct orc_moe {
  int d, E, K, I, Is, group, r;
  double alpha;
  const uint32_t *gate_q, *up_q, *down_q;  // [E, I, d/8], [E, I, d/8], [E, d, I/8]
  const uint16_t *gate_s, *up_s, *down_s;  // [E, I, d/G], [E, I, d/G], [E, d, I/G]
  const uint32_t *sh_gate_q, *sh_up_q, *sh_down_q;  // shared expert, Is rows/cols
  const uint16_t *sh_gate_s, *sh_up_s, *sh_down_s;
  const uint16_t *a_gate, *b_gate, *a_up, *b_up, *a_down, *b_down;  // nullable
};

// Routed combine plus shared expert for one token: y = sum_k w_k E_{idx_k}(x)
// + S(x) [CB "The mechanism" (shared_experts=1 in the MoESpec); MW Fig. 1 sum
// node]. x is the fp16 activation. Returns -1 on an out-of-range id.
int orc_moe_decode(const orc_moe* m, const uint16_t* x16, const int32_t* idx, const double* w,
                   double* y) {
  const int d = m->d, I = m->I, G = m->group;
  std::vector<double> x(d), ye(d);
  for (int i = 0; i < d; ++i) x[i] = f16_to_f64(x16[i]);
  for (int i = 0; i < d; ++i) y[i] = 0.0;
  for (int k = 0; k < m->K; ++k) {
    int e = idx[k];
    if (e < 0 || e >= m->E) return -1;
    const int64_t gu_q = static_cast<int64_t>(e) * I * (d / 8);
    const int64_t gu_s = static_cast<int64_t>(e) * I * (d / G);
    const int64_t dn_q = static_cast<int64_t>(e) * d * (I / 8);
    const int64_t dn_s = static_cast<int64_t>(e) * d * (I / G);
    orc_expert(m->gate_q + gu_q, m->gate_s + gu_s, m->up_q + gu_q, m->up_s + gu_s,
               m->down_q + dn_q, m->down_s + dn_s, d, I, G, x.data(), ye.data());
    for (int i = 0; i < d; ++i) y[i] += w[k] * ye[i];
  }
  if (m->sh_gate_q) {
    orc_shared_expert(m->sh_gate_q, m->sh_gate_s, m->sh_up_q, m->sh_up_s, m->sh_down_q,
                      m->sh_down_s, m->a_gate, m->b_gate, m->a_up, m->b_up, m->a_down,
                      m->b_down, d, m->Is, G, m->r, m->alpha, x.data(), ye.data());
    for (int i = 0; i < d; ++i) y[i] += ye[i];
  }
  return 0;
}

// Prerouter head [MW §3.2 Head; RG "Prerouter Head Architecture"; CB "The
// mechanism" (PrerouterHead)]: f = [x ; onehot(cur) ; onehot(prev)] of length
// d + 2E, logits = lin f + fc2 gelu_erf(fc1 f), no biases. fc1 [P, d+2E],
// fc2 [E, P], lin [E, d+2E], fp16 row-major. prev == nullptr is the all-zero
// one-hot. form 0 builds the dense concatenated feature; form 1 adds the
// gathered one-hot columns instead. Returns -1 on a bad or repeated id.
int orc_head_logits(const uint16_t* fc1, const uint16_t* fc2, const uint16_t* lin, int d, int E,
                    int P, int K, const uint16_t* x16, const int32_t* cur, const int32_t* prev,
                    int form, double* logits) {
  const int F = d + 2 * E;
  std::vector<uint8_t> seen_c(E, 0), seen_p(E, 0);
  for (int k = 0; k < K; ++k) {
    if (cur[k] < 0 || cur[k] >= E || seen_c[cur[k]]) return -1;
    seen_c[cur[k]] = 1;
    if (prev) {
      if (prev[k] < 0 || prev[k] >= E || seen_p[prev[k]]) return -1;
      seen_p[prev[k]] = 1;
    }
  }
  std::vector<double> z(P), a(P), lo(E);
  if (form == 0) {
    std::vector<double> f(F, 0.0);
    for (int i = 0; i < d; ++i) f[i] = f16_to_f64(x16[i]);
    for (int e = 0; e < E; ++e) {
      f[d + e] = seen_c[e] ? 1.0 : 0.0;
      f[d + E + e] = seen_p[e] ? 1.0 : 0.0;
    }
    f16_matvec(fc1, P, F, f.data(), z.data());
    f16_matvec(lin, E, F, f.data(), lo.data());
  } else {
    std::vector<double> x(d);
    for (int i = 0; i < d; ++i) x[i] = f16_to_f64(x16[i]);
    for (int p = 0; p < P; ++p) {
      const uint16_t* row = fc1 + static_cast<int64_t>(p) * F;
      double acc = 0.0;
      for (int i = 0; i < d; ++i) acc += f16_to_f64(row[i]) * x[i];
      for (int k = 0; k < K; ++k) {
        acc += f16_to_f64(row[d + cur[k]]);
        if (prev) acc += f16_to_f64(row[d + E + prev[k]]);
      }
      z[p] = acc;
    }
    for (int e = 0; e < E; ++e) {
      const uint16_t* row = lin + static_cast<int64_t>(e) * F;
      double acc = 0.0;
      for (int i = 0; i < d; ++i) acc += f16_to_f64(row[i]) * x[i];
      for (int k = 0; k < K; ++k) {
        acc += f16_to_f64(row[d + cur[k]]);
        if (prev) acc += f16_to_f64(row[d + E + prev[k]]);
      }
      lo[e] = acc;
    }
  }
  for (int p = 0; p < P; ++p) a[p] = gelu_erf(z[p]);
  f16_matvec(fc2, E, P, a.data(), logits);
  for (int e = 0; e < E; ++e) logits[e] += lo[e];
  return 0;
}

// Routing parameters of one predicted layer (router family of the tier).
struct orc_routing {
  int kind;  // 0 softmax-top-K, 1 sigmoid-group
  int E, K, norm_topk, n_groups, topk_groups;
  double scale;
};

int orc_route(const orc_routing* rt, const double* logits, const float* bias32, int32_t* idx,
              double* w) {
  if (rt->kind == 0) return orc_route_softmax_topk(logits, rt->E, rt->K, rt->norm_topk, idx, w);
  std::vector<double> bias(rt->E, 0.0);
  if (bias32)
    for (int e = 0; e < rt->E; ++e) bias[e] = bias32[e];
  return orc_route_sigmoid_group(logits, bias.data(), rt->E, rt->K, rt->n_groups,
                                 rt->topk_groups, rt->scale, idx, w, nullptr, nullptr);
}

// One decode layer-step [MW §3.2 Motivation, Head, Prediction-as-routing,
// Feature drift]:
//   h_attn = h + attn                    (fixed residual update for attention)
//   x      = fp16(RMSNorm(h_attn))       (post-attention norm output)
//   routing: router layers run their own router W_r x (fp16 [E, d]);
//            predicted layers take (route_idx, route_w) as given
//   y      = routed combine + shared expert (orc_moe_decode)
//   h_out  = h_attn + y                  (returned unrounded)
//   head (if the layer owns one): logits over f = [x; onehot(executed set);
//            onehot(previous token's set)], routed with the next layer's
//            routing family -> prediction for the next layer, next token.
struct orc_layer {
  orc_moe moe;
  orc_routing rt;
  double eps;
  const uint16_t* attn;         // [d] fp16 residual update, nullable
  const uint16_t* router;       // [E, d] fp16, nullable (predicted layer)
  const float* router_bias;     // [E] fp32 sigmoid-group bias, nullable
  const uint16_t *fc1, *fc2, *lin;  // head, nullable (layer owns no head)
  const float* head_bias;       // [E] bias of the predicted layer's routing
  int P;
};

// x_in (nullable): an fp16 rounding of RMSNorm(h_attn) to use instead of the
// oracle's own; x_out always receives the oracle's own rounding.
int orc_layer_step(const orc_layer* L, const uint16_t* h16, const uint16_t* x_in,
                   const int32_t* route_idx, const float* route_w, const int32_t* prev_idx,
                   double* h_out, uint16_t* x_out, int32_t* exec_idx, double* exec_w,
                   double* router_logits, double* head_logits, int32_t* pred_idx,
                   double* pred_w) {
  const int d = L->moe.d, E = L->moe.E, K = L->moe.K;
  std::vector<double> ha(d), xn(d), x(d), y(d);
  for (int i = 0; i < d; ++i) ha[i] = f16_to_f64(h16[i]) + (L->attn ? f16_to_f64(L->attn[i]) : 0.0);
  orc_rmsnorm(ha.data(), d, L->eps, xn.data());
  std::vector<uint16_t> x16(d);
  for (int i = 0; i < d; ++i) x16[i] = f64_to_f16(xn[i]);
  if (x_out)
    for (int i = 0; i < d; ++i) x_out[i] = x16[i];
  if (x_in)
    for (int i = 0; i < d; ++i) x16[i] = x_in[i];
  for (int i = 0; i < d; ++i) x[i] = f16_to_f64(x16[i]);
  std::vector<double> w(K);
  if (L->router) {
    std::vector<double> lg(E);
    f16_matvec(L->router, E, d, x.data(), lg.data());
    if (router_logits)
      for (int e = 0; e < E; ++e) router_logits[e] = lg[e];
    if (orc_route(&L->rt, lg.data(), L->router_bias, exec_idx, w.data()) != 0) return -2;
  } else {
    for (int k = 0; k < K; ++k) {
      exec_idx[k] = route_idx[k];
      w[k] = route_w[k];
    }
  }
  for (int k = 0; k < K; ++k) exec_w[k] = w[k];
  if (orc_moe_decode(&L->moe, x16.data(), exec_idx, w.data(), y.data()) != 0) return -1;
  for (int i = 0; i < d; ++i) h_out[i] = ha[i] + y[i];
  if (L->fc1) {
    std::vector<double> lg(E);
    if (orc_head_logits(L->fc1, L->fc2, L->lin, d, E, L->P, K, x16.data(), exec_idx, prev_idx,
                        1, lg.data()) != 0)
      return -3;
    if (head_logits)
      for (int e = 0; e < E; ++e) head_logits[e] = lg[e];
    if (orc_route(&L->rt, lg.data(), L->head_bias, pred_idx, pred_w) != 0) return -4;
  }
  return 0;
}

// Slot policy for the staged HBM slot pool of one layer [MW §3.1 Executor
// paths "staged" (fixed slots, only changed experts rewritten); IE "Fixed-Slot
// Decoding"]. The pages give no policy; this is the reading used:
//   * `in_use` (K ids, or null for none) is the set the running token uses and
//     `next` (K ids) is the set to stage.
//   * an id of `next` that already has a slot keeps it (a hit, no copy);
//   * misses, in ascending id, take free slots in ascending slot index, where
//     a slot is free unless it holds an id of in_use or next; the previous
//     occupant is evicted.
// With n_slots >= 2K a free slot always exists. Writes the (expert, slot)
// copy list and returns its length, or -1 if the pool would overflow / an id
// is out of range.
int orc_slot_policy(int E, int n_slots, int K, int32_t* slot_of, int32_t* slot_expert,
                    const int32_t* in_use, const int32_t* next, int32_t* copy_expert,
                    int32_t* copy_slot) {
  std::vector<uint8_t> keep(E, 0), want(E, 0);
  for (int k = 0; k < K; ++k) {
    if (next[k] < 0 || next[k] >= E) return -1;
    want[next[k]] = 1;
    keep[next[k]] = 1;
    if (in_use) {
      if (in_use[k] < 0 || in_use[k] >= E) return -1;
      keep[in_use[k]] = 1;
    }
  }
  std::vector<int32_t> misses;
  for (int e = 0; e < E; ++e)
    if (want[e] && slot_of[e] < 0) misses.push_back(e);
  std::vector<int32_t> free_slots;
  for (int s = 0; s < n_slots; ++s)
    if (slot_expert[s] < 0 || !keep[slot_expert[s]]) free_slots.push_back(s);
  if (free_slots.size() < misses.size()) return -1;
  for (size_t j = 0; j < misses.size(); ++j) {
    int s = free_slots[j], e = misses[j];
    if (slot_expert[s] >= 0) slot_of[slot_expert[s]] = -1;
    slot_expert[s] = e;
    slot_of[e] = s;
    copy_expert[j] = e;
    copy_slot[j] = s;
  }
  return static_cast<int>(misses.size());
}

}  // extern "C"
