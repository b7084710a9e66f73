// Per-phase HIP kernels of the decode step (gfx950, wave64).
//
// GEMV scheme shared by every weight-streaming kernel: a row of the weight
// matrix is owned by an aligned group of LG lanes; each lane reads 16-byte
// chunks at stride LG (so one wave instruction covers 64/LG rows with fully
// used cache lines), keeps the matching activations in registers, and the
// group is reduced with DPP at the end. Int4 rows are dequantised in
// registers (q4_dot8); fp16 rows use v_dot2_f32_f16 directly. All sums are
// fp32; fp32 activations meet fp16 weights as an fp16 hi/lo pair.
//
// Page tags: [MW] "The Other Half of the Memory Wall: Serving 35B MoEs from
// SSD with Trained Routing Prediction"; [CB] "Edge0 streams a 35B MoE off
// SSD. I counted the bytes it can't stream."; [IE] "Inside Edge0-35B".

#include "device.h"
#include "gemv.h"
#include "internal.h"

namespace smd {

namespace {

constexpr int kBlock = 128;  // threads per block of the GEMV kernels (2 waves)

// ------------------------------------------------------------- gate / up --

struct GateUpArgs {
  Dims dm;
  Pool pool;
  SharedW sh;
  const uint16_t* x;  // [B][d]
  const int32_t* idx; // [B][K]
  float* gu;          // [B][K+1][imax]
  const float* ax;    // [B][3][rmax]
  int imax, rmax;
  int32_t* flags;
};

// SwiGLU gate/up of one expert slot (routed k < K, shared k == K) for one
// token: h[row] = silu(Wg[row] . x (+ LoRA)) * (Wu[row] . x (+ LoRA))
// [MW §3.1 Math contract; IE "Architectural Deep Dive"]. grid = (row blocks,
// K+1, B).
// AFF: affine codec (bf16 scale and bias per group, unsigned nibbles); the
// bias terms use the sums of the activation's 32-element chunks (LDS).
template <int LG, int CPL, bool AFF>
__global__ __launch_bounds__(kBlock) void k_gate_up(GateUpArgs a) {
  extern __shared__ uint16_t xs[];  // [d] pair-permuted; affine: then xsum [d/32] fp32
  const Dims& dm = a.dm;
  const int b = blockIdx.z, k = blockIdx.y;
  const bool shared = (k == dm.K);
  if (shared && !a.sh.present) return;
  const int rows = shared ? dm.Is : dm.I;
  const int d = dm.d;

  const uint32_t *gq, *uq;
  const uint16_t *gs, *us, *gb = nullptr, *ub = nullptr;
  if (shared) {
    gq = a.sh.gate.q; gs = a.sh.gate.s; uq = a.sh.up.q; us = a.sh.up.s;
    gb = a.sh.gate.b; ub = a.sh.up.b;
  } else {
    const int64_t ent = resolve_entry(a.pool, dm.E, a.idx[b * dm.K + k]);
    if (ent < 0) {
      if (threadIdx.x == 0 && blockIdx.x == 0) atomicOr(&a.flags[FLAG_RANGE], 1);
      return;
    }
    gq = (const uint32_t*)entry_ptr(a.pool.gate.q, ent, a.pool.stride_q);
    uq = (const uint32_t*)entry_ptr(a.pool.up.q, ent, a.pool.stride_q);
    gs = (const uint16_t*)entry_ptr(a.pool.gate.s, ent, a.pool.stride_s);
    us = (const uint16_t*)entry_ptr(a.pool.up.s, ent, a.pool.stride_s);
    if (AFF) {
      gb = (const uint16_t*)entry_ptr(a.pool.gate.b, ent, a.pool.stride_s);
      ub = (const uint16_t*)entry_ptr(a.pool.up.b, ent, a.pool.stride_s);
    }
  }

  const uint16_t* xb = a.x + (int64_t)b * d;
  for (int i = threadIdx.x; i < d; i += blockDim.x) xs[perm8(i)] = xb[i];
  float* xsum = reinterpret_cast<float*>(xs + d);
  if (AFF) {
    for (int c = threadIdx.x; c < d / 32; c += blockDim.x) {
      float sum = 0.0f;
      for (int i = 0; i < 32; ++i) sum += h2f(xb[32 * c + i]);
      xsum[c] = sum;
    }
  }
  __syncthreads();

  constexpr int kRowsPerWave = 64 / LG;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane % LG, grp = lane / LG;
  const int row = blockIdx.x * (kBlock / 64) * kRowsPerWave + wave * kRowsPerWave + grp;
  if (row >= rows) return;  // whole aligned lane groups leave together

  const int wpr = d / 8, spr = d / dm.G;
  const uint32_t* grow = gq + (int64_t)row * wpr;
  const uint32_t* urow = uq + (int64_t)row * wpr;
  const uint16_t* gsr = gs + (int64_t)row * spr;
  const uint16_t* usr = us + (int64_t)row * spr;

  float ag, au;
  if (AFF)
    gateup_rowpair_aff<LG, CPL>(grow, urow, gsr, usr, gb + (int64_t)row * spr,
                                ub + (int64_t)row * spr, dm.G, xs, xsum, li, ag, au);
  else
    gateup_rowpair<LG, CPL>(grow, urow, gsr, usr, dm.G, xs, li, ag, au);
  if (shared && a.sh.bg) {
    const float* axb = a.ax + (int64_t)b * 3 * a.rmax;
    float lg = 0.0f, lu = 0.0f;
    for (int t = li; t < dm.r; t += LG) {
      lg += h2f(a.sh.bg[(int64_t)row * dm.r + t]) * axb[t];
      lu += h2f(a.sh.bu[(int64_t)row * dm.r + t]) * axb[a.rmax + t];
    }
    ag += dm.lora_scale * lg;
    au += dm.lora_scale * lu;
  }
  ag = group_sum<LG>(ag);
  au = group_sum<LG>(au);
  if (li == 0) a.gu[((int64_t)b * (dm.K + 1) + k) * a.imax + row] = silu(ag) * au;
}

// ------------------------------------------------------------------ down --

struct DownArgs {
  Dims dm;
  Pool pool;
  SharedW sh;
  const int32_t* idx;  // [B][K]
  const float* w;      // [B][K]
  const float* gu;     // [B][K+1][imax]
  int imax;
  const float* ax;     // [B][3][rmax]
  int rmax;
  const float* resid;  // [B][d] or null
  uint16_t* y;         // [B][d]
  int32_t* flags;
};

// Down projections with the weighted combine and the shared expert:
// y[row] = sum_k w_k Wd_k[row] . h_k + Wd_s[row] . h_s (+ down LoRA)
// [MW §3.1 Math contract; CB "The mechanism" (shared_experts = 1)].
// Output fp16(resid + y). grid = (row blocks of d, B).
template <int LG, int CPL, bool AFF>
__global__ __launch_bounds__(kBlock) void k_down(DownArgs a) {
  extern __shared__ uint16_t hs[];  // [nexp][2][I] pair-permuted hi / lo; affine: then
                                    // hsum [nexp][I/32] fp32 (chunk sums of hi + lo)
  __shared__ float coef[16];
  __shared__ int64_t ent_s[16];
  __shared__ float red[4];
  const Dims& dm = a.dm;
  const int b = blockIdx.y;
  const int I = dm.I, d = dm.d;
  const int nexp = dm.K + (a.sh.present ? 1 : 0);

  for (int k = 0; k < nexp; ++k) {
    const float* src = a.gu + ((int64_t)b * (dm.K + 1) + k) * a.imax;
    const float m = block_absmax(src, I, red);
    const int e = hilo_exponent(m);
    const float inv = ldexpf(1.0f, -e);
    uint16_t* hh = hs + (int64_t)k * 2 * I;
    for (int i = threadIdx.x; i < I; i += blockDim.x) {
      f16 hi, lo;
      split_hilo(src[i], inv, hi, lo);
      hh[perm8(i)] = __builtin_bit_cast(uint16_t, hi);
      hh[I + perm8(i)] = __builtin_bit_cast(uint16_t, lo);
    }
    if (threadIdx.x == 0) {
      if (k < dm.K) {
        const int64_t ent = resolve_entry(a.pool, dm.E, a.idx[b * dm.K + k]);
        if (ent < 0 && blockIdx.x == 0) atomicOr(&a.flags[FLAG_RANGE], 1);
        ent_s[k] = ent;
        coef[k] = ent < 0 ? 0.0f : a.w[b * dm.K + k] * ldexpf(1.0f, e);
      } else {
        ent_s[k] = 0;
        coef[k] = ldexpf(1.0f, e);
      }
    }
  }
  __syncthreads();
  float* hsum = reinterpret_cast<float*>(hs + (int64_t)nexp * 2 * I);
  if (AFF) {
    // the pair permutation stays inside 8-element blocks, so positions
    // 32c .. 32c+31 hold exactly chunk c
    for (int j = threadIdx.x; j < nexp * (I / 32); j += blockDim.x) {
      const int k = j / (I / 32), c = j % (I / 32);
      const uint16_t* hh = hs + (int64_t)k * 2 * I + 32 * c;
      float sum = 0.0f;
      for (int i = 0; i < 32; ++i) sum += h2f(hh[i]) + h2f(hh[I + i]);
      hsum[j] = sum;
    }
    __syncthreads();
  }

  constexpr int kRowsPerWave = 64 / LG;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane % LG, grp = lane / LG;
  const int row = blockIdx.x * (kBlock / 64) * kRowsPerWave + wave * kRowsPerWave + grp;
  if (row >= d) return;

  const int wpr = I / 8, spr = I / dm.G;
  float acc = 0.0f;
  for (int k = 0; k < nexp; ++k) {
    if (k < dm.K && ent_s[k] < 0) continue;
    const uint32_t* q;
    const uint16_t *s, *bq = nullptr;
    if (k < dm.K) {
      q = (const uint32_t*)entry_ptr(a.pool.down.q, ent_s[k], a.pool.stride_q);
      s = (const uint16_t*)entry_ptr(a.pool.down.s, ent_s[k], a.pool.stride_s);
      if (AFF) bq = (const uint16_t*)entry_ptr(a.pool.down.b, ent_s[k], a.pool.stride_s);
    } else {
      q = a.sh.down.q;
      s = a.sh.down.s;
      bq = a.sh.down.b;
    }
    const uint16_t* hh = hs + (int64_t)k * 2 * I;
    float part;
    if (AFF)
      part = down_row_hl_aff<LG, CPL>(q + (int64_t)row * wpr, s + (int64_t)row * spr,
                                      bq + (int64_t)row * spr, dm.G, hh, hh + I,
                                      hsum + (int64_t)k * (I / 32), li);
    else
      part = down_row_hl<LG, CPL>(q + (int64_t)row * wpr, s + (int64_t)row * spr, dm.G, hh,
                                  hh + I, li);
    acc += coef[k] * part;
  }
  if (a.sh.present && a.sh.bd) {
    const float* axd = a.ax + (int64_t)b * 3 * a.rmax + 2 * a.rmax;
    float l = 0.0f;
    for (int t = li; t < dm.r; t += LG) l += h2f(a.sh.bd[(int64_t)row * dm.r + t]) * axd[t];
    acc += dm.lora_scale * l;
  }
  acc = group_sum<LG>(acc);
  if (li == 0) {
    const float base = a.resid ? a.resid[(int64_t)b * d + row] : 0.0f;
    a.y[(int64_t)b * d + row] = f2h(base + acc);
  }
}

// ------------------------------------------------------------ fp16 GEMV --

struct Gemv16Args {
  const uint16_t* W;
  int rows, cols;
  int64_t ld;
  const uint16_t* x16;
  const float* xf;
  int64_t x_stride;
  const int32_t *cur, *prev;
  int K, E, gcol0;
  int epi;
  const float* addv;
  float* y;
  int64_t y_stride;
};

// y[b][row] = W[row, :cols] . x[b] (+ one-hot gathered columns) with an
// epilogue. Used for the router, the LoRA A products and the three head
// matrices [MW §3.2 Head; CB "The mechanism" (PrerouterHead)].
// grid = (row blocks, B); 16 lanes per row.
template <bool XF32>
__global__ __launch_bounds__(kBlock) void k_gemv16(Gemv16Args a) {
  extern __shared__ uint16_t xs16[];  // [cols] or hi [cols] + lo [cols]
  __shared__ float red[4];
  const int b = blockIdx.y;
  const int cols = a.cols;
  float scale = 1.0f;
  if constexpr (XF32) {
    const float* xb = a.xf + (int64_t)b * a.x_stride;
    const int e = hilo_exponent(block_absmax(xb, cols, red));
    const float inv = ldexpf(1.0f, -e);
    scale = ldexpf(1.0f, e);
    for (int i = threadIdx.x; i < cols; i += blockDim.x) {
      f16 hi, lo;
      split_hilo(xb[i], inv, hi, lo);
      xs16[i] = __builtin_bit_cast(uint16_t, hi);
      xs16[cols + i] = __builtin_bit_cast(uint16_t, lo);
    }
  } else {
    const uint16_t* xb = a.x16 + (int64_t)b * a.x_stride;
    for (int i = threadIdx.x; i < cols; i += blockDim.x) xs16[i] = xb[i];
  }
  __syncthreads();

  constexpr int LG = 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane % LG, grp = lane / LG;
  const int row = blockIdx.x * (kBlock / LG) + wave * (64 / LG) + grp;
  if (row >= a.rows) return;

  const uint16_t* wrow = a.W + (int64_t)row * a.ld;
  float acc;
  if constexpr (XF32) {
    acc = f16_row_dot_hl<LG>(wrow, cols, xs16, xs16 + cols, li);
  } else {
    acc = f16_row_dot<LG>(wrow, cols, xs16, li);
  }
  acc *= scale;
  if (a.cur) {
    // One-hot blocks of the head feature: each selected expert adds one
    // weight column (the one-hot entry is exactly 1).
    for (int kk = li; kk < 2 * a.K; kk += LG) {
      int col = -1;
      if (kk < a.K) {
        const int e = a.cur[(int64_t)b * a.K + kk];
        if (e >= 0 && e < a.E) col = a.gcol0 + e;
      } else if (a.prev) {
        const int e = a.prev[(int64_t)b * a.K + kk - a.K];
        if (e >= 0 && e < a.E) col = a.gcol0 + a.E + e;
      }
      if (col >= 0) acc += h2f(wrow[col]);
    }
  }
  acc = group_sum<LG>(acc);
  if (li == 0) {
    float v = acc;
    if (a.epi == 1) v = gelu_erf(v);
    else if (a.epi == 2) v += a.addv[(int64_t)b * a.y_stride + row];
    a.y[(int64_t)b * a.y_stride + row] = v;
  }
}

// ------------------------------------------------------------ LoRA B ------

__global__ __launch_bounds__(256) void k_lora_b(const uint16_t* Bm, int out_dim, int r,
                                                float scale, const float* ax, int ax_stride,
                                                float* y_acc) {
  const int b = blockIdx.y;
  const int o = blockIdx.x * blockDim.x + threadIdx.x;
  if (o >= out_dim) return;
  const float* axb = ax + (int64_t)b * ax_stride;
  float s = 0.0f;
  for (int t = 0; t < r; ++t) s += h2f(Bm[(int64_t)o * r + t]) * axb[t];
  y_acc[(int64_t)b * out_dim + o] += scale * s;
}

// --------------------------------------------------------------- routing --

struct RouteArgs {
  Dims dm;
  const float* logits;  // [B][E]
  const float* bias;    // [E] or null (sigmoid-group)
  int32_t* idx;         // [B][K]
  float* w;             // [B][K]
  int32_t* flags;
};

// Routing of one token's fp32 logits (one wave per token) [MW App. A].
__global__ __launch_bounds__(64) void k_route(RouteArgs a) {
  __shared__ RouteScratch rs;
  const int b = blockIdx.x;
  route_wave(a.dm, a.logits + (int64_t)b * a.dm.E, a.bias, rs, a.idx + (int64_t)b * a.dm.K,
             a.w + (int64_t)b * a.dm.K, a.flags);
}

// --------------------------------------------------------------- prepare --

struct PrepArgs {
  Dims dm;
  const uint16_t* h;
  const uint16_t* attn;
  float* hattn;
  uint16_t* xn;
  const int32_t* cidx;
  const float* cw;
  int32_t* eidx;
  float* ew;
};

// h_a = h + attn (fp32), x = fp16(h_a / sqrt(mean(h_a^2) + eps)): the
// post-attention RMSNorm the head and the experts read [MW §3.2 Motivation].
__global__ __launch_bounds__(256) void k_prep(PrepArgs a) {
  __shared__ float red[4];
  const int b = blockIdx.x, d = a.dm.d;
  const uint16_t* hb = a.h + (int64_t)b * d;
  float ss = 0.0f;
  for (int i = threadIdx.x; i < d; i += blockDim.x) {
    const float v = h2f(hb[i]) + (a.attn ? h2f(a.attn[i]) : 0.0f);
    a.hattn[(int64_t)b * d + i] = v;
    ss += v * v;
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
  for (int j = 0; j < (int)(blockDim.x >> 6); ++j) tot += red[j];
  const float inv = 1.0f / sqrtf(tot / d + a.dm.eps);
  for (int i = threadIdx.x; i < d; i += blockDim.x)
    a.xn[(int64_t)b * d + i] = f2h(a.hattn[(int64_t)b * d + i] * inv);
  if (a.cidx && threadIdx.x < a.dm.K) {
    a.eidx[(int64_t)b * a.dm.K + threadIdx.x] = a.cidx[(int64_t)b * a.dm.K + threadIdx.x];
    a.ew[(int64_t)b * a.dm.K + threadIdx.x] = a.cw[(int64_t)b * a.dm.K + threadIdx.x];
  }
}

}  // namespace

// ---------------------------------------------------------- launchers --

static bool q4_shape(int cols, int& lg, int& cpl) {
  if (cols % 32) return false;
  const int nch = cols / 32;
  if (nch % 16 == 0 && nch / 16 <= 8) {
    lg = 16;
    cpl = nch / 16;
  } else if (nch <= 8) {
    lg = 1;
    cpl = nch;
  } else {
    return false;
  }
  return cpl == 1 || cpl == 2 || cpl == 3 || cpl == 4 || cpl == 6 || cpl == 8;
}

bool q4_shape_ok(int cols) {
  int lg, cpl;
  return q4_shape(cols, lg, cpl);
}

// Calls Op<LG, CPL>::run(args...) for the supported instantiations.
template <template <int, int> class Op, typename... A>
static hipError_t q4_dispatch(int lg, int cpl, A&&... args) {
  if (lg == 16) {
    switch (cpl) {
      case 1: Op<16, 1>::run(args...); break;
      case 2: Op<16, 2>::run(args...); break;
      case 3: Op<16, 3>::run(args...); break;
      case 4: Op<16, 4>::run(args...); break;
      case 6: Op<16, 6>::run(args...); break;
      case 8: Op<16, 8>::run(args...); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (cpl) {
      case 1: Op<1, 1>::run(args...); break;
      case 2: Op<1, 2>::run(args...); break;
      case 3: Op<1, 3>::run(args...); break;
      case 4: Op<1, 4>::run(args...); break;
      case 6: Op<1, 6>::run(args...); break;
      case 8: Op<1, 8>::run(args...); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

template <int LG, int CPL>
struct GateUpOp {
  static void run(dim3 grid, size_t lds, hipStream_t st, const GateUpArgs& a) {
    if (a.dm.affine)
      k_gate_up<LG, CPL, true><<<grid, kBlock, lds, st>>>(a);
    else
      k_gate_up<LG, CPL, false><<<grid, kBlock, lds, st>>>(a);
  }
};

template <int LG, int CPL>
struct DownOp {
  static void run(dim3 grid, size_t lds, hipStream_t st, const DownArgs& a) {
    if (a.dm.affine)
      k_down<LG, CPL, true><<<grid, kBlock, lds, st>>>(a);
    else
      k_down<LG, CPL, false><<<grid, kBlock, lds, st>>>(a);
  }
};

static int imax_of(const Dims& dm) { return dm.I > dm.Is ? dm.I : dm.Is; }
static int rmax_of(const Dims& dm) { return dm.r > 1 ? dm.r : 1; }

hipError_t launch_gate_up(const Dims& dm, const Pool& pool, const SharedW& sh,
                          const uint16_t* x, const int32_t* idx, int B, const Scratch& s,
                          hipStream_t st) {
  int lg, cpl;
  if (!q4_shape(dm.d, lg, cpl)) return hipErrorInvalidValue;
  GateUpArgs a{dm, pool, sh, x, idx, s.gu, s.ax, imax_of(dm), rmax_of(dm), s.flags};
  const int rows = imax_of(dm);
  const int rpb = (kBlock / 64) * (64 / lg);
  dim3 grid((rows + rpb - 1) / rpb, dm.K + 1, B);
  const size_t lds = (size_t)dm.d * sizeof(uint16_t) + (dm.affine ? (size_t)dm.d / 32 * 4 : 0);
  return q4_dispatch<GateUpOp>(lg, cpl, grid, lds, st, a);
}

hipError_t launch_down(const Dims& dm, const Pool& pool, const SharedW& sh,
                       const int32_t* idx, const float* w, int B, const float* resid,
                       uint16_t* y16, const Scratch& s, hipStream_t st) {
  int lg, cpl;
  if (!q4_shape(dm.I, lg, cpl)) return hipErrorInvalidValue;
  DownArgs a{dm, pool, sh, idx, w, s.gu, imax_of(dm), s.ax, rmax_of(dm), resid, y16, s.flags};
  const int rpb = (kBlock / 64) * (64 / lg);
  dim3 grid((dm.d + rpb - 1) / rpb, B);
  const int nexp = dm.K + (sh.present ? 1 : 0);
  const size_t lds = (size_t)nexp * 2 * dm.I * sizeof(uint16_t) +
                     (dm.affine ? (size_t)nexp * (dm.I / 32) * 4 : 0);
  return q4_dispatch<DownOp>(lg, cpl, grid, lds, st, a);
}

hipError_t launch_gemv16(const uint16_t* W, int rows, int cols, int64_t ld,
                         const uint16_t* x16, const float* xf32, int64_t x_stride, int B,
                         const int32_t* cur, const int32_t* prev, int K, int E, int gcol0,
                         int epi, const float* addv, float* y, int64_t y_stride,
                         hipStream_t st) {
  if (cols % 8 || ld % 8) return hipErrorInvalidValue;
  Gemv16Args a{W, rows, cols, ld, x16, xf32, x_stride, cur, prev, K, E, gcol0, epi, addv, y,
               y_stride};
  dim3 grid((rows + (kBlock / 16) - 1) / (kBlock / 16), B);
  if (xf32) {
    hipLaunchKernelGGL(k_gemv16<true>, grid, dim3(kBlock), (size_t)cols * 4, st, a);
  } else {
    hipLaunchKernelGGL(k_gemv16<false>, grid, dim3(kBlock), (size_t)cols * 2, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_lora_a(int n_mats, const uint16_t* const* A, const int* slots, int in_dim,
                         int r, const uint16_t* x16, const float* xf32, int64_t x_stride,
                         int B, float* ax, int ax_stride, hipStream_t st) {
  for (int m = 0; m < n_mats; ++m) {
    hipError_t e = launch_gemv16(A[m], r, in_dim, in_dim, x16, xf32, x_stride, B, nullptr,
                                 nullptr, 0, 0, 0, 0, nullptr, ax + slots[m], ax_stride, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_lora_b(const uint16_t* Bm, int out_dim, int r, float scale, const float* ax,
                         int ax_stride, float* y_acc, int B, hipStream_t st) {
  dim3 grid((out_dim + 255) / 256, B);
  hipLaunchKernelGGL(k_lora_b, grid, dim3(256), 0, st, Bm, out_dim, r, scale, ax, ax_stride,
                     y_acc);
  return hipGetLastError();
}

hipError_t launch_route(const Dims& dm, const float* logits, const float* bias, int B,
                        int32_t* idx, float* w, int32_t* flags, hipStream_t st) {
  if (dm.E > kMaxE || dm.K > 8 || dm.n_groups > 64) return hipErrorInvalidValue;
  RouteArgs a{dm, logits, bias, idx, w, flags};
  hipLaunchKernelGGL(k_route, dim3(B), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_prep(const Dims& dm, const uint16_t* h, const uint16_t* attn, int B,
                       float* hattn, uint16_t* xn, const int32_t* cidx, const float* cw,
                       int32_t* eidx, float* ew, hipStream_t st) {
  PrepArgs a{dm, h, attn, hattn, xn, cidx, cw, eidx, ew};
  hipLaunchKernelGGL(k_prep, dim3(B), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace smd
