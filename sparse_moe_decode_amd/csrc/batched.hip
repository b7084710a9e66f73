// Batched decode chunk (16..32 tokens): grouped int4 GEMMs on MFMA.
//
// Source: "The Other Half of the Memory Wall" §3.1 Executor paths (batched
// chunks take the whole-layer path: experts are grouped so each expert's
// weights are read once for all tokens routed to it) and Math contract (one
// quantized kernel computing down(silu(gate(x)) * up(x)) per expert).
//
// Steps, all on the caller's stream:
//   1. k_mb_group: the B*K (token, slot) entries sorted by expert (ascending
//      expert, then entry order), the union of experts with each expert's run.
//   2. k_mb_xperm: x copied in the pair-permuted fp16 order the int4 dequant
//      produces ([x0 x4 x1 x5 x2 x6 x3 x7] per block of 8).
//   3. k_mb_gate_up: one wave per (expert of the union, 32 rows of I); the
//      expert's tokens are the 32 columns of v_mfma_f32_32x32x16_f16 tiles.
//      int4 words are dequantised in registers to exact fp16 integers; each
//      group of 64 inputs is accumulated on its own and scaled in fp32 by the
//      row's group scale (q*s is never rounded). SwiGLU in the epilogue. The
//      shared expert runs as the last "expert" with all tokens, its LoRA B
//      terms added in the epilogue.
//   4. k_mb_hsplit: each (token, slot) SwiGLU output -> fp16 hi + lo with a
//      power-of-two scale (about 22 bits kept); A_down . h of the shared one.
//   5. k_mb_down: as 3 for the down rows, hi and lo accumulated together.
//   6. k_mb_combine: y = sum_k w_k y_k + y_shared + down LoRA, in a fixed
//      order (no atomics, deterministic), rounded to fp16.

#include "gemv.h"
#include "internal.h"

namespace smd {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kCols = 32;  // tokens per MFMA column block

// Grouping tables in s.grp (int32): [0] union size; then sorted entries
// (b*K + k) [BK]; expert, first sorted position and run length per union
// member [BK] each.
struct Groups {
  int32_t* n_union;
  int32_t* sorted;
  int32_t* uexp;
  int32_t* ustart;
  int32_t* ucount;
};

__host__ __device__ inline Groups groups(int32_t* g, int BK) {
  return {g, g + 1, g + 1 + BK, g + 1 + 2 * BK, g + 1 + 3 * BK};
}

__global__ __launch_bounds__(256) void k_mb_group(int E, int K, int B, const int32_t* idx,
                                                  int32_t* grp, int32_t* flags) {
  __shared__ int cnt[kMaxE];
  __shared__ int off[kMaxE];
  const int BK = B * K;
  Groups g = groups(grp, BK);
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int i = threadIdx.x;
  int e = -1;
  if (i < BK) {
    e = idx[i];
    if (e < 0 || e >= E) {
      atomicOr(&flags[FLAG_RANGE], 1);
      e = -1;
    } else {
      atomicAdd(&cnt[e], 1);  // integer counts: order-independent
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int o = 0, u = 0;
    for (int x = 0; x < E; ++x) {
      off[x] = o;
      if (cnt[x]) {
        g.uexp[u] = x;
        g.ustart[u] = o;
        g.ucount[u] = cnt[x];
        ++u;
      }
      o += cnt[x];
    }
    *g.n_union = u;
  }
  __syncthreads();
  if (e >= 0) {
    int rank = 0;  // earlier entries routed to the same expert
    for (int j = 0; j < i; ++j) rank += idx[j] == e;
    g.sorted[off[e] + rank] = i;
  }
}

__global__ __launch_bounds__(256) void k_mb_xperm(const uint16_t* x, int d, uint16_t* xp) {
  const int b = blockIdx.x;
  for (int c = threadIdx.x; c < d / 8; c += blockDim.x) {
    const uint4 v = ldg(reinterpret_cast<const uint4*>(x + (int64_t)b * d + 8 * c));
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint16_t e[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      e[2 * q] = (uint16_t)(w[q] & 0xFFFF);
      e[2 * q + 1] = (uint16_t)(w[q] >> 16);
    }
    *reinterpret_cast<uint4*>(xp + (int64_t)b * d + 8 * c) =
        make_uint4(e[0] | ((uint32_t)e[4] << 16), e[1] | ((uint32_t)e[5] << 16),
                   e[2] | ((uint32_t)e[6] << 16), e[3] | ((uint32_t)e[7] << 16));
  }
}

// Eight int4 weights of one word as exact fp16 integers, in the order
// q0 q4 q1 q5 q2 q6 q3 q7 (matching the pair-permuted activations).
__device__ __forceinline__ h8 q4_to_h8(uint32_t w) {
  const uint32_t u = w ^ 0x88888888u;
  const uint32_t v = u >> 8;
  const f16x2 k1032 = {(f16)1032.0f, (f16)1032.0f};
  const f16x2 k16 = {(f16)0.0625f, (f16)0.0625f};
  const f16x2 k72 = {(f16)72.0f, (f16)72.0f};
  const f16x2 p0 = as_h2((u & 0x000F000Fu) | 0x64006400u) - k1032;
  const f16x2 p1 = as_h2((u & 0x00F000F0u) | 0x64006400u) * k16 - k72;
  const f16x2 p2 = as_h2((v & 0x000F000Fu) | 0x64006400u) - k1032;
  const f16x2 p3 = as_h2((v & 0x00F000F0u) | 0x64006400u) * k16 - k72;
  h8 r;
  r[0] = p0.x; r[1] = p0.y; r[2] = p1.x; r[3] = p1.y;
  r[4] = p2.x; r[5] = p2.y; r[6] = p3.x; r[7] = p3.y;
  return r;
}

__device__ __forceinline__ h8 as_h8(uint4 v) { return __builtin_bit_cast(h8, v); }

// Row held in accumulator register r by a lane of half kh (MFMA 32x32 layout).
__device__ __forceinline__ int acc_row(int r, int kh) { return 8 * (r >> 2) + 4 * kh + (r & 3); }

// One 32-row tile of an int4 matrix against 32 activation columns, over
// n_in inputs: acc (fp32) += sum over groups of scale[row][group] *
// (q . x)_group. `act(g, j)` returns the lane's 8 activations (pair-permuted
// fp16) for MFMA j of input block g (64 inputs).
template <typename Act>
__device__ __forceinline__ void tile_mma(const uint32_t* rows, int wpr, const uint16_t* sc_lds,
                                         int n_groups_s, int G, int n_in, Act act, f32x16& acc) {
  const int l = threadIdx.x & 63, lm = l & 31, kh = l >> 5;
  const uint32_t* arow = rows + (int64_t)lm * wpr;
  for (int g = 0; g < n_in / 64; ++g) {
    const uint4 wv = ldg(reinterpret_cast<const uint4*>(arow + 8 * g + 4 * kh));
    const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
    f32x16 c = {};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      c = __builtin_amdgcn_mfma_f32_32x32x16_f16(q4_to_h8(ww[j]), act(g, j), c, 0, 0, 0);
    const int s = (64 * g) / G;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] += h2f(sc_lds[s * 32 + acc_row(r, kh)]) * c[r];
  }
  (void)n_groups_s;
}

// Scales of rows [m0, m0+32) of an int4 matrix into LDS as [group][row].
__device__ __forceinline__ void load_tile_scales(const uint16_t* s, int n_groups_s, int m0,
                                                 uint16_t* dst) {
  for (int i = threadIdx.x; i < 32 * n_groups_s; i += blockDim.x) {
    const int rr = i / n_groups_s, gg = i % n_groups_s;
    dst[gg * 32 + rr] = ldg(s + (int64_t)(m0 + rr) * n_groups_s + gg);
  }
}

struct MbArgs {
  Dims dm;
  Pool pool;
  SharedW sh;
  int B;
  const uint16_t* xp;    // [B][d] pair-permuted
  const int32_t* grp;
  const int32_t* idx;    // [B][K]
  const float* w;        // [B][K]
  const float* ax;       // [B][3*rmax] LoRA A products (gate, up, down)
  int rmax;
  float* H;              // [B][K+1][imax] SwiGLU outputs
  uint16_t* hh;          // [B][K+1][imax] fp16 hi, pair-permuted
  uint16_t* hl;
  float* hexp;           // [B][K+1] power-of-two scale of hh/hl
  float* Y;              // [B][K+1][d] per-slot down outputs
  float* axd;            // ax, written: A_down . h_shared
  uint16_t* y;           // [B][d]
  int32_t* flags;
};

// Column n of a column block: its token and output slot; `valid` false for
// padding columns (they compute on token 0 and are not stored).
__device__ __forceinline__ void column(const MbArgs& a, bool shared, int start, int count, int cb,
                                       int n, int& b, int& k, bool& valid) {
  const int K = a.dm.K;
  const Groups g = groups(const_cast<int32_t*>(a.grp), a.B * K);
  valid = cb + n < count;
  if (shared) {
    b = valid ? cb + n : 0;
    k = K;
  } else {
    const int ent = g.sorted[start + (valid ? cb + n : 0)];
    b = ent / K;
    k = ent % K;
  }
}

__global__ __launch_bounds__(64) void k_mb_gate_up(MbArgs a) {
  __shared__ uint16_t sg[32 * 64], su[32 * 64];  // [group][row], d/G <= 64
  const Dims& dm = a.dm;
  const int K = dm.K, d = dm.d, I = dm.I;
  const int imax = dm.I > dm.Is ? dm.I : dm.Is;
  const Groups gv = groups(const_cast<int32_t*>(a.grp), a.B * K);
  const int nu = *gv.n_union;
  const int u = blockIdx.y;
  const bool shared = u == nu;
  if (u > nu || (shared && !a.sh.present)) return;
  const int m0 = blockIdx.x * 32;
  const int rows_total = shared ? dm.Is : I;
  if (m0 >= rows_total) return;
  const uint32_t *gq, *uq;
  const uint16_t *gs, *us;
  int start = 0, count = a.B;
  if (shared) {
    gq = a.sh.gate.q; uq = a.sh.up.q; gs = a.sh.gate.s; us = a.sh.up.s;
  } else {
    const int e = gv.uexp[u];
    start = gv.ustart[u];
    count = gv.ucount[u];
    const int64_t ent = resolve_entry(a.pool, dm.E, e);
    if (ent < 0) {
      if (threadIdx.x == 0) atomicOr(&a.flags[FLAG_RANGE], 1);
      return;
    }
    gq = (const uint32_t*)entry_ptr(a.pool.gate.q, ent, a.pool.stride_q);
    uq = (const uint32_t*)entry_ptr(a.pool.up.q, ent, a.pool.stride_q);
    gs = (const uint16_t*)entry_ptr(a.pool.gate.s, ent, a.pool.stride_s);
    us = (const uint16_t*)entry_ptr(a.pool.up.s, ent, a.pool.stride_s);
  }
  const int ngs = d / dm.G, wpr = d / 8;
  load_tile_scales(gs, ngs, m0, sg);
  load_tile_scales(us, ngs, m0, su);
  __syncthreads();
  const int l = threadIdx.x, n = l & 31, kh = l >> 5;
  const float c = dm.lora_scale;
  for (int cb = 0; cb < count; cb += kCols) {
    int b, k;
    bool valid;
    column(a, shared, start, count, cb, n, b, k, valid);
    const uint16_t* xrow = a.xp + (int64_t)b * d + 32 * kh;
    auto act = [&](int g, int j) {
      return as_h8(ldg(reinterpret_cast<const uint4*>(xrow + 64 * g + 8 * j)));
    };
    f32x16 ag = {}, au = {};
    tile_mma(gq + (int64_t)m0 * wpr, wpr, sg, ngs, dm.G, d, act, ag);
    tile_mma(uq + (int64_t)m0 * wpr, wpr, su, ngs, dm.G, d, act, au);
    if (!valid) continue;
    float* hrow = a.H + ((int64_t)b * (K + 1) + k) * imax;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + acc_row(r, kh);
      float gg = ag[r], uu = au[r];
      if (shared && a.sh.ag) {
        const float* axb = a.ax + (int64_t)b * 3 * a.rmax;
        float lg = 0.0f, lu = 0.0f;
        for (int q = 0; q < dm.r; ++q) {
          lg += h2f(ldg(a.sh.bg + (int64_t)row * dm.r + q)) * axb[q];
          lu += h2f(ldg(a.sh.bu + (int64_t)row * dm.r + q)) * axb[a.rmax + q];
        }
        gg += c * lg;
        uu += c * lu;
      }
      hrow[row] = silu(gg) * uu;
    }
  }
}

// One wave per (token, slot): hi/lo copies of the SwiGLU output; for the
// shared slot also A_down . h.
__global__ __launch_bounds__(64) void k_mb_hsplit(MbArgs a) {
  const Dims& dm = a.dm;
  const int K = dm.K;
  const int imax = dm.I > dm.Is ? dm.I : dm.Is;
  const int b = blockIdx.x / (K + 1), k = blockIdx.x % (K + 1);
  const int n = k < K ? dm.I : dm.Is;
  bool valid;
  if (k < K) {
    valid = resolve_entry(a.pool, dm.E, a.idx[b * K + k]) >= 0;
  } else {
    valid = a.sh.present != 0;
  }
  if (!valid) return;
  const int lane = threadIdx.x;
  const float* h = a.H + ((int64_t)b * (K + 1) + k) * imax;
  float m = 0.0f;
  for (int i = lane; i < n; i += 64) m = fmaxf(m, fabsf(h[i]));
  m = wave_max_rows(m);
  const int e = hilo_exponent(m);
  const float inv = ldexpf(1.0f, -e);
  uint16_t* hh = a.hh + ((int64_t)b * (K + 1) + k) * imax;
  uint16_t* hl = a.hl + ((int64_t)b * (K + 1) + k) * imax;
  for (int i = lane; i < n; i += 64) {
    f16 hi, lo;
    split_hilo(h[i], inv, hi, lo);
    hh[perm8(i)] = __builtin_bit_cast(uint16_t, hi);
    hl[perm8(i)] = __builtin_bit_cast(uint16_t, lo);
  }
  if (lane == 0) a.hexp[(int64_t)b * (K + 1) + k] = ldexpf(1.0f, e);
  if (k == K && a.sh.ad) {
    for (int q = 0; q < dm.r; ++q) {
      float s = 0.0f;
      for (int i = lane; i < n; i += 64) s += h2f(ldg(a.sh.ad + (int64_t)q * n + i)) * h[i];
      s = wave_sum_rows(s);
      if (lane == 0) a.axd[(int64_t)b * 3 * a.rmax + 2 * a.rmax + q] = s;
    }
  }
}

__global__ __launch_bounds__(64) void k_mb_down(MbArgs a) {
  __shared__ uint16_t sd[32 * 64];  // [group][row], I/G <= 64
  const Dims& dm = a.dm;
  const int K = dm.K, d = dm.d;
  const int imax = dm.I > dm.Is ? dm.I : dm.Is;
  const Groups gv = groups(const_cast<int32_t*>(a.grp), a.B * K);
  const int nu = *gv.n_union;
  const int u = blockIdx.y;
  const bool shared = u == nu;
  if (u > nu || (shared && !a.sh.present)) return;
  const int m0 = blockIdx.x * 32;
  const uint32_t* dq;
  const uint16_t* ds;
  int start = 0, count = a.B;
  const int nin = shared ? dm.Is : dm.I;
  if (shared) {
    dq = a.sh.down.q; ds = a.sh.down.s;
  } else {
    const int e = gv.uexp[u];
    start = gv.ustart[u];
    count = gv.ucount[u];
    const int64_t ent = resolve_entry(a.pool, dm.E, e);
    if (ent < 0) return;  // flagged by the gate/up step
    dq = (const uint32_t*)entry_ptr(a.pool.down.q, ent, a.pool.stride_q);
    ds = (const uint16_t*)entry_ptr(a.pool.down.s, ent, a.pool.stride_s);
  }
  const int ngs = nin / dm.G, wpr = nin / 8;
  load_tile_scales(ds, ngs, m0, sd);
  __syncthreads();
  const int l = threadIdx.x, n = l & 31, kh = l >> 5;
  for (int cb = 0; cb < count; cb += kCols) {
    int b, k;
    bool valid;
    column(a, shared, start, count, cb, n, b, k, valid);
    const int64_t slot = (int64_t)b * (K + 1) + k;
    const uint16_t* hrow = a.hh + slot * imax + 32 * kh;
    const uint16_t* lrow = a.hl + slot * imax + 32 * kh;
    // hi and lo halves go through the same weights: two MFMA passes per block
    auto act_hi = [&](int g, int j) {
      return as_h8(ldg(reinterpret_cast<const uint4*>(hrow + 64 * g + 8 * j)));
    };
    auto act_lo = [&](int g, int j) {
      return as_h8(ldg(reinterpret_cast<const uint4*>(lrow + 64 * g + 8 * j)));
    };
    f32x16 acc = {};
    tile_mma(dq + (int64_t)m0 * wpr, wpr, sd, ngs, dm.G, nin, act_hi, acc);
    tile_mma(dq + (int64_t)m0 * wpr, wpr, sd, ngs, dm.G, nin, act_lo, acc);
    if (!valid) continue;
    const float sc = a.hexp[slot];
    float* yrow = a.Y + slot * d;
#pragma unroll
    for (int r = 0; r < 16; ++r) yrow[m0 + acc_row(r, kh)] = acc[r] * sc;
  }
}

__global__ __launch_bounds__(256) void k_mb_combine(MbArgs a) {
  const Dims& dm = a.dm;
  const int K = dm.K, d = dm.d, b = blockIdx.x;
  const float c = dm.lora_scale;
  const float* axb = a.axd + (int64_t)b * 3 * a.rmax + 2 * a.rmax;
  for (int j = threadIdx.x; j < d; j += blockDim.x) {
    float acc = 0.0f;
    for (int k = 0; k < K; ++k) {
      if (resolve_entry(a.pool, dm.E, a.idx[b * K + k]) < 0) continue;
      acc += a.w[b * K + k] * a.Y[((int64_t)b * (K + 1) + k) * d + j];
    }
    if (a.sh.present) {
      acc += a.Y[((int64_t)b * (K + 1) + K) * d + j];
      if (a.sh.bd) {
        float ls = 0.0f;
        for (int q = 0; q < dm.r; ++q) ls += h2f(ldg(a.sh.bd + (int64_t)j * dm.r + q)) * axb[q];
        acc += c * ls;
      }
    }
    a.y[(int64_t)b * d + j] = f2h(acc);
  }
}

}  // namespace

bool batched_supported(const Dims& dm) {
  return dm.G % 64 == 0 && dm.d % 64 == 0 && dm.I % 64 == 0 && dm.d / dm.G <= 64 &&
         dm.I / dm.G <= 64 && dm.K * kCols <= 256 && dm.E <= kMaxE &&
         (dm.Is == 0 || dm.Is == dm.I);
}

hipError_t launch_batched(const Dims& dm, const Pool& pool, const SharedW& sh, const uint16_t* x,
                          const int32_t* idx, const float* w, int B, uint16_t* y,
                          const Scratch& s, hipStream_t st) {
  if (B < 1 || B > kCols || !batched_supported(dm)) return hipErrorInvalidValue;
  MbArgs a;
  a.dm = dm;
  a.pool = pool;
  a.sh = sh;
  a.B = B;
  a.xp = s.xn;
  a.grp = s.grp;
  a.idx = idx;
  a.w = w;
  a.ax = s.ax;
  a.rmax = dm.r > 1 ? dm.r : 1;
  a.H = s.gu;
  a.hh = s.hh;
  a.hl = s.hl;
  a.hexp = s.hexp;
  a.Y = s.yk;
  a.axd = s.ax;
  a.y = y;
  a.flags = s.flags;
  hipLaunchKernelGGL(k_mb_group, dim3(1), dim3(256), 0, st, dm.E, dm.K, B, idx, s.grp, s.flags);
  hipLaunchKernelGGL(k_mb_xperm, dim3(B), dim3(256), 0, st, x, dm.d, s.xn);
  const int ny = B * dm.K + 1;  // union members + the shared expert
  const int imax = dm.I > dm.Is ? dm.I : dm.Is;
  hipLaunchKernelGGL(k_mb_gate_up, dim3(imax / 32, ny), dim3(64), 0, st, a);
  hipLaunchKernelGGL(k_mb_hsplit, dim3(B * (dm.K + 1)), dim3(64), 0, st, a);
  hipLaunchKernelGGL(k_mb_down, dim3(dm.d / 32, ny), dim3(64), 0, st, a);
  hipLaunchKernelGGL(k_mb_combine, dim3(B), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace smd
