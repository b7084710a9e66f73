// Persistent whole-token decode kernel: one launch runs a token through a
// range of layers on every CU of the chip.
//
// Per layer l (source: "The Other Half of the Memory Wall" §3.1 Math contract,
// §3.2 Motivation / Head / Prediction-as-routing / Feature drift, §3.3; the
// head layout as listed in "I counted the bytes it can't stream"):
//   1. every workgroup gathers h_l, adds the attention stand-in and computes
//      the RMS norm itself (x is replicated, never exchanged);
//   2. routing: the layer's own router (rows spread over the chip, logits
//      exchanged, top-K recomputed identically everywhere) or the prediction
//      the previous token's head wrote;
//   3. gate/up rows of the routed experts and the shared expert, and the
//      LoRA A products of the shared gate/up, spread over the chip;
//   4. head fc1 (erf-GELU) and linear-path rows, spread over the chip;
//   5. every workgroup gathers the SwiGLU outputs, finishes the shared
//      expert (LoRA B of gate/up, SwiGLU, LoRA A of down) redundantly;
//   6. down rows with the weighted combine, shared expert and down LoRA;
//      h_{l+1} = fp16(h_a + y) is published;
//   7. head fc2 rows; the routing of the head logits runs after the last
//      layer and writes the prediction read by the next token.
//
// Cross-workgroup data moves as 8-byte words (32-bit payload, 32-bit epoch)
// written and polled with agent-scope relaxed atomics (coherent across the
// XCDs' L2s without cache write-back or invalidation): an aligned 8-byte
// access is single-copy atomic, so a word carrying the current launch's epoch
// carries that launch's payload. Buffers are per layer, so no word is written
// twice in one launch. Every wait is bounded by a wall-clock limit; on expiry
// the kernel raises FLAG_SYNC and runs to completion.

#include "gemv.h"
#include "internal.h"

namespace smd {

namespace {

constexpr int kThreads = 256;
constexpr int kLG = 16;
constexpr int kGroups = kThreads / kLG;
constexpr uint64_t kSpinLimit = 20000000ull;  // 0.2 s of the 100 MHz wall clock

__device__ __forceinline__ uint64_t ld64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void ll_put(uint64_t* p, uint32_t v, uint32_t ep) {
  __hip_atomic_store(p, ((uint64_t)ep << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t fbits(float v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float bitsf(uint32_t v) { return __builtin_bit_cast(float, v); }

// Give up waiting: after a wait of this workgroup timed out, or any
// workgroup raised the sync flag, later waits return at once (the results of
// the launch are then reported as invalid through FLAG_SYNC).
typedef volatile __attribute__((address_space(3))) int lds_int;

__device__ __forceinline__ bool wait_expired(uint64_t t0, int32_t* flags, int* abort_lds,
                                             uint32_t& polls) {
  lds_int* ab = (lds_int*)abort_lds;
  if (*ab) return true;
  if ((++polls & 63u) == 0 &&
      __hip_atomic_load(&flags[FLAG_SYNC], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    *ab = 1;
    return true;
  }
  if (wall_clock64() - t0 > kSpinLimit) {
    atomicOr(&flags[FLAG_SYNC], 1);
    *ab = 1;
    return true;
  }
  return false;
}

// All threads of the block gather n words src[0..n) of epoch ep into dst.
template <int U>
__device__ void ll_gather(const uint64_t* src, int n, uint32_t ep, uint32_t* dst,
                          int32_t* flags, int* abort_lds) {
  const uint64_t t0 = wall_clock64();
  uint32_t polls = 0;
  for (int b0 = 0; b0 < n; b0 += U * kThreads) {
    uint64_t v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int i = b0 + j * kThreads + (int)threadIdx.x;
      v[j] = i < n ? ld64(src + i) : ((uint64_t)ep << 32);
    }
    for (;;) {
      bool ok = true;
#pragma unroll
      for (int j = 0; j < U; ++j) ok = ok && ((uint32_t)(v[j] >> 32) == ep);
      if (ok) break;
      if (wait_expired(t0, flags, abort_lds, polls)) break;
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int i = b0 + j * kThreads + (int)threadIdx.x;
        if (i < n && (uint32_t)(v[j] >> 32) != ep) v[j] = ld64(src + i);
      }
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int i = b0 + j * kThreads + (int)threadIdx.x;
      if (i < n) dst[i] = (uint32_t)v[j];
    }
  }
}

// Phase timestamp of this workgroup (thread 0) when tracing is on.
__device__ __forceinline__ void stamp(const StackArgs& a, int l, int k) {
  if (a.trace && threadIdx.x == 0)
    a.trace[((int64_t)blockIdx.x * a.L + l) * kTracePoints + k] = wall_clock64();
}

enum { XH = 0, XG = 1, XR = 2, XA = 3, XL = 4 };

__device__ __forceinline__ uint32_t* flag_row(const StackArgs& a, int l, int x) {
  return a.fl + ((int64_t)l * kExchanges + x) * gridDim.x;
}

// This workgroup has issued its words of exchange x for layer l.
__device__ __forceinline__ void post(const StackArgs& a, int l, int x) {
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(flag_row(a, l, x) + blockIdx.x, a.epoch, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every workgroup posted exchange x of layer l. Wave 0 polls the
// packed flags (a few coalesced loads per round); the others wait at the
// barrier. The words themselves are still epoch-checked when gathered.
__device__ __forceinline__ void wait_all(const StackArgs& a, int l, int x, int* abort_lds) {
  if ((threadIdx.x >> 6) == 0) {
    const uint32_t* f = flag_row(a, l, x);
    const int lane = threadIdx.x & 63;
    const int G = (int)gridDim.x;
    const uint64_t t0 = wall_clock64();
    uint32_t polls = 0;
    uint32_t v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = lane + 64 * j;
      v[j] = i < G ? __hip_atomic_load(f + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : a.epoch;
    }
    for (;;) {
      bool ok = true;
#pragma unroll
      for (int j = 0; j < 8; ++j) ok = ok && v[j] == a.epoch;
      if (__all(ok)) break;
      if (wait_expired(t0, a.flags, abort_lds, polls)) break;
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = lane + 64 * j;
        if (i < G && v[j] != a.epoch)
          v[j] = __hip_atomic_load(f + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  __syncthreads();
}

__device__ __forceinline__ void split(int n, int G, int c, int& beg, int& end) {
  beg = (int)((int64_t)n * c / G);
  end = (int)((int64_t)n * (c + 1) / G);
}

// Block-wide sum (all threads return the total).
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float t = 0.0f;
  for (int j = 0; j < kThreads / 64; ++j) t += red[j];
  return t;
}

constexpr int kMaxL = 64;      // layers per launch (routing tables in LDS)
constexpr int kNR = 4;         // fp16 rows per workgroup per job (router, head, fc2, LoRA A)
constexpr int kLoraRegs = 12;  // 16-byte chunks per thread of the LoRA matrices (Is*r <= 8192)

// Small per-layer values kept in LDS.
struct Misc {
  int32_t ridx[8];
  float rw[8];
  int64_t ent[16];
  float coef[16];
  float emax[16];
  float ad[64];
  float red[4 * kNR];
  float rows[kNR];   // results of the block fp16 row jobs
  float gath[kNR * 16];
  float ha_scale;
  int abort;
  uint16_t hstage[512];  // h_out rows of this workgroup (<= 512)
  int32_t ridx_all[kMaxL * 8];
  float rw_all[kMaxL * 8];
  int32_t pidx_all[kMaxL * 8];
  int64_t ent_all[kMaxL * 8];
  RouteScratch rs;
};

struct Lds {
  // byte offsets into dynamic LDS
  int hattn, xperm, xnat, land, hk, ha, lora, misc;
  int bytes;
};

__host__ __device__ inline Lds lds_layout(const Dims& dm, int ng) {
  auto up = [](int b) { return (b + 15) & ~15; };
  Lds o;
  int off = 0;
  o.hattn = off; off += up(dm.d * 4);
  o.xperm = off; off += up(dm.d * 2);
  o.xnat = off; off += up(dm.d * 2);
  int land = ng;
  if (dm.d / 2 > land) land = dm.d / 2;
  if (dm.E > land) land = dm.E;
  if (dm.P + dm.E > land) land = dm.P + dm.E;
  o.land = off; off += up(land * 4);
  o.hk = off; off += up((dm.K + 1) * 2 * dm.I * 2);
  o.ha = off; off += up(dm.P * 2 * 2);
  o.lora = off; off += up(3 * dm.Is * dm.r * 2);
  o.misc = off; off += up((int)sizeof(Misc));
  o.bytes = off;
  return o;
}

// ---- block fp16 row jobs: thread t < cols/8 holds 16-byte chunk t of each row
template <int NR>
struct F16Rows {
  uint4 w[NR];
};

template <int NR>
__device__ __forceinline__ void f16rows_issue(F16Rows<NR>& R, const uint16_t* const* rp, int nr,
                                              int cols) {
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    R.w[j] = make_uint4(0, 0, 0, 0);
    if (j < nr && t < cols / 8) R.w[j] = ldg(reinterpret_cast<const uint4*>(rp[j] + 8 * t));
  }
}

__device__ __forceinline__ float dot8_h(uint4 w, uint4 x, float acc) {
  acc = dot2(as_h2(w.x), as_h2(x.x), acc);
  acc = dot2(as_h2(w.y), as_h2(x.y), acc);
  acc = dot2(as_h2(w.z), as_h2(x.z), acc);
  acc = dot2(as_h2(w.w), as_h2(x.w), acc);
  return acc;
}

// Reduce p[j] over the block into ms.rows[j] (visible to all threads on return).
template <int NR>
__device__ __forceinline__ void block_rows_reduce(float (&p)[NR], int nr, Misc& ms) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < NR; ++j)
    if (j < nr) p[j] = wave_sum(p[j]);
  if (lane == 0)
#pragma unroll
    for (int j = 0; j < NR; ++j) ms.red[wave * NR + j] = p[j];
  __syncthreads();
  if (threadIdx.x < NR) {
    float s = 0.0f;
    for (int w = 0; w < kThreads / 64; ++w) s += ms.red[w * NR + threadIdx.x];
    ms.rows[threadIdx.x] = s;
  }
  __syncthreads();
}

// rows . x with x fp16 (natural order) in LDS.
template <int NR>
__device__ __forceinline__ void f16rows_finish(const F16Rows<NR>& R, int nr, int cols,
                                               const uint16_t* xs, Misc& ms) {
  const int t = threadIdx.x;
  const uint4 xv = t < cols / 8 ? *reinterpret_cast<const uint4*>(xs + 8 * t) : make_uint4(0, 0, 0, 0);
  float p[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) p[j] = dot8_h(R.w[j], xv, 0.0f);
  block_rows_reduce<NR>(p, nr, ms);
}

// rows . (xh + xl) with an fp16 hi/lo activation in LDS.
template <int NR>
__device__ __forceinline__ void f16rows_finish_hl(const F16Rows<NR>& R, int nr, int cols,
                                                  const uint16_t* xh, const uint16_t* xl,
                                                  Misc& ms) {
  const int t = threadIdx.x;
  const bool in = t < cols / 8;
  const uint4 a = in ? *reinterpret_cast<const uint4*>(xh + 8 * t) : make_uint4(0, 0, 0, 0);
  const uint4 b = in ? *reinterpret_cast<const uint4*>(xl + 8 * t) : make_uint4(0, 0, 0, 0);
  float p[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) p[j] = dot8_h(R.w[j], b, dot8_h(R.w[j], a, 0.0f));
  block_rows_reduce<NR>(p, nr, ms);
}

// ---- gate/up items of one lane group (IPG items per group) ---------------
template <int CPL, int IPG>
struct GuRegs {
  uint4 wg[IPG][CPL], wu[IPG][CPL];
  uint16_t sg[IPG][CPL], su[IPG][CPL];
};

struct GuPlan {
  int ib, ie;  // item range of this workgroup
};

__device__ __forceinline__ bool gu_item(const LayerDev& Ly, const Dims& dm, const Misc& ms,
                                        int n_rt, int it, const uint32_t*& gq,
                                        const uint32_t*& uq, const uint16_t*& gs,
                                        const uint16_t*& us, int& row) {
  const bool routed = it < n_rt;
  if (routed) {
    const int k = it / dm.I;
    row = it % dm.I;
    const int64_t ent = ms.ent[k];
    const int64_t e = ent >= 0 ? ent : 0;
    gq = (const uint32_t*)entry_ptr(Ly.pool.gate.q, e, Ly.pool.stride_q);
    uq = (const uint32_t*)entry_ptr(Ly.pool.up.q, e, Ly.pool.stride_q);
    gs = (const uint16_t*)entry_ptr(Ly.pool.gate.s, e, Ly.pool.stride_s);
    us = (const uint16_t*)entry_ptr(Ly.pool.up.s, e, Ly.pool.stride_s);
    return ent >= 0;
  }
  row = it - n_rt;
  gq = Ly.sh.gate.q;
  uq = Ly.sh.up.q;
  gs = Ly.sh.gate.s;
  us = Ly.sh.up.s;
  return true;
}

template <int CPL, int IPG>
__device__ __forceinline__ void gu_issue(GuRegs<CPL, IPG>& R, const LayerDev& Ly, const Dims& dm,
                                         const Misc& ms, int n_rt, const GuPlan& pl, int grp,
                                         int li) {
#pragma unroll
  for (int j = 0; j < IPG; ++j) {
    const int it = pl.ib + grp + kGroups * j;
    if (it >= pl.ie) continue;
    const uint32_t *gq, *uq;
    const uint16_t *gs, *us;
    int row;
    if (!gu_item(Ly, dm, ms, n_rt, it, gq, uq, gs, us, row)) continue;
    const int wpr = dm.d / 8, spr = dm.d / dm.G;
    const uint32_t* grow = gq + (int64_t)row * wpr;
    const uint32_t* urow = uq + (int64_t)row * wpr;
#pragma unroll
    for (int c2 = 0; c2 < CPL; ++c2) {
      const int c = li + kLG * c2;
      R.wg[j][c2] = ldg(reinterpret_cast<const uint4*>(grow + 4 * c));
      R.wu[j][c2] = ldg(reinterpret_cast<const uint4*>(urow + 4 * c));
      R.sg[j][c2] = ldg(gs + (int64_t)row * spr + (32 * c) / dm.G);
      R.su[j][c2] = ldg(us + (int64_t)row * spr + (32 * c) / dm.G);
    }
  }
}

template <int CPL, int IPG>
__device__ __forceinline__ void gu_finish(const GuRegs<CPL, IPG>& R, const LayerDev& Ly,
                                          const Dims& dm, const Misc& ms, int n_rt, int Is,
                                          const GuPlan& pl, int grp, int li,
                                          const uint16_t* xperm, uint64_t* xg, uint32_t ep) {
#pragma unroll
  for (int j = 0; j < IPG; ++j) {
    const int it = pl.ib + grp + kGroups * j;
    if (it >= pl.ie) continue;  // uniform over the lane group
    const bool routed = it < n_rt;
    const bool ok = !routed || ms.ent[it / dm.I] >= 0;
    float ag = 0.0f, au = 0.0f;
    if (ok) {
#pragma unroll
      for (int c2 = 0; c2 < CPL; ++c2) {
        f16x2 xr[16];
        load_xchunk(xperm, li + kLG * c2, xr);
        ag += h2f(R.sg[j][c2]) * q4_dot32(R.wg[j][c2], xr);
        au += h2f(R.su[j][c2]) * q4_dot32(R.wu[j][c2], xr);
      }
    }
    ag = group_sum<kLG>(ag);
    au = group_sum<kLG>(au);
    if (li == 0) {
      if (routed) {
        ll_put(xg + it, fbits(ok ? silu(ag) * au : 0.0f), ep);
      } else {
        ll_put(xg + n_rt + (it - n_rt), fbits(ag), ep);
        ll_put(xg + n_rt + Is + (it - n_rt), fbits(au), ep);
      }
    }
  }
}

// ---- down rows: every expert's chunk of one row per lane group ------------
constexpr int kMaxExp = 9;

struct DownRegs {
  uint4 w[kMaxExp];
  uint16_t s[kMaxExp];
  uint4 bd[4];  // LoRA B of the down projection, r fp16 = r/8 chunks (r <= 32)
};

// Pending loads of phase A (before the h exchange).
template <int CPL, int IPG>
struct PhaseA {
  F16Rows<kNR> router, head, ax;
  int n_router, n_head, n_ax;
  GuRegs<CPL, IPG> gu;
  bool gu_loaded;
  uint4 attn;  // this thread's 8 elements of the attention update
};

template <int CPL_D, int IPG>
__global__ __launch_bounds__(kThreads) void k_stack(StackArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const Dims& dm = a.dm;
  const int d = dm.d, E = dm.E, K = dm.K, I = dm.I, P = dm.P, G = (int)gridDim.x;
  const int cu = (int)blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int li = lane % kLG, grp = t / kLG;
  const uint32_t ep = a.epoch;
  const int cur = a.token & 1, nxt = (a.token + 1) & 1;
  const Lds lo = lds_layout(dm, a.ng);
  float* hattn = (float*)(smem + lo.hattn);
  uint16_t* xperm = (uint16_t*)(smem + lo.xperm);
  uint16_t* xnat = (uint16_t*)(smem + lo.xnat);
  uint32_t* land = (uint32_t*)(smem + lo.land);
  uint16_t* hk = (uint16_t*)(smem + lo.hk);
  uint16_t* ha = (uint16_t*)(smem + lo.ha);
  uint16_t* lora = (uint16_t*)(smem + lo.lora);
  Misc& ms = *(Misc*)(smem + lo.misc);
  const int nL = a.l1 - a.l0;
  const int F = d + 2 * E;

  // Routing tables of every layer of the launch: the prediction consumed at
  // this token, the previous token's sets, and pool entries of predicted layers.
  if (t == 0) ms.abort = 0;
  for (int i = t; i < nL * K; i += kThreads) {
    const int l = a.l0 + i / K, k = i % K;
    ms.ridx_all[i] = a.route_idx[((int64_t)cur * a.L + l) * K + k];
    ms.rw_all[i] = a.route_w[((int64_t)cur * a.L + l) * K + k];
    ms.pidx_all[i] = a.token > 0 ? a.exec_idx[((int64_t)nxt * a.L + l) * K + k] : -1;
  }
  __syncthreads();
  for (int i = t; i < nL * K; i += kThreads) {
    const int l = a.l0 + i / K;
    ms.ent_all[i] = a.layers[l].router ? 0 : resolve_entry(a.layers[l].pool, E, ms.ridx_all[i]);
  }
  __syncthreads();

  // Issue every load of layer l that does not depend on its activations.
  auto issue_a = [&](int l, PhaseA<CPL_D, IPG>& A) {
    const LayerDev& Ly = a.layers[l];
    const bool has_sh = Ly.sh.present != 0;
    const int Is = has_sh ? dm.Is : 0;
    const int r2 = (has_sh && Ly.sh.ag) ? 2 * dm.r : 0;
    const uint16_t* rp[kNR];
    int b, e;
    A.n_router = 0;
    if (Ly.router) {
      split(E, G, cu, b, e);
      A.n_router = e - b;
      for (int j = 0; j < kNR; ++j) rp[j] = Ly.router + (int64_t)(b + (j < A.n_router ? j : 0)) * d;
      f16rows_issue<kNR>(A.router, rp, A.n_router, d);
    }
    split(r2, G, cu, b, e);
    A.n_ax = e - b;
    for (int j = 0; j < kNR; ++j) {
      const int tt = b + (j < A.n_ax ? j : 0);
      rp[j] = (tt < dm.r ? Ly.sh.ag : Ly.sh.au) + (int64_t)(tt % (dm.r > 0 ? dm.r : 1)) * d;
    }
    if (A.n_ax) f16rows_issue<kNR>(A.ax, rp, A.n_ax, d);
    A.n_head = 0;
    if (Ly.head.fc1) {
      split(P + E, G, cu, b, e);
      A.n_head = e - b;
      for (int j = 0; j < kNR; ++j) {
        const int it = b + (j < A.n_head ? j : 0);
        rp[j] = it < P ? Ly.head.fc1 + (int64_t)it * F : Ly.head.lin + (int64_t)(it - P) * F;
      }
      f16rows_issue<kNR>(A.head, rp, A.n_head, d);
    }
    A.attn = make_uint4(0, 0, 0, 0);
    if (Ly.attn && t < d / 8) A.attn = ldg(reinterpret_cast<const uint4*>(Ly.attn + 8 * t));
    A.gu_loaded = false;
    if (!Ly.router) {
      // routing known: entries from the tables
      if (t < 16) ms.ent[t] = t < K ? ms.ent_all[(l - a.l0) * K + t] : 0;
      __syncthreads();
      GuPlan pl;
      split(K * I + Is, G, cu, pl.ib, pl.ie);
      gu_issue<CPL_D, IPG>(A.gu, Ly, dm, ms, K * I, pl, grp, li);
      A.gu_loaded = true;
    }
  };

  PhaseA<CPL_D, IPG> A;
  issue_a(a.l0, A);

  for (int l = a.l0; l < a.l1; ++l) {
    const LayerDev& Ly = a.layers[l];
    const int step = l - a.l0;
    const bool has_sh = Ly.sh.present != 0;
    const int Is = has_sh ? dm.Is : 0;
    const int r2 = (has_sh && Ly.sh.ag) ? 2 * dm.r : 0;
    const int nexp = K + (has_sh ? 1 : 0);
    const int n_rt = K * I;
    uint64_t* xg = a.xg + (int64_t)l * a.ng;
    const bool head = Ly.head.fc1 != nullptr;

    // ---- 1. h_l, attention stand-in, RMSNorm ---------------------------
    stamp(a, l, 0);
    if (step > 0) {
      wait_all(a, l - 1, XH, &ms.abort);
      ll_gather<4>(a.xh + (int64_t)(l - 1) * (d / 2), d / 2, ep, land, a.flags, &ms.abort);
    }
    __syncthreads();
    stamp(a, l, 1);
    {
      // thread t owns elements 8t..8t+7 (one pair-permutation block)
      float v[8];
      float ss = 0.0f;
      if (t < d / 8) {
        uint32_t hw[4];
        if (step == 0) {
          const uint4 hv = *reinterpret_cast<const uint4*>(a.h + 8 * t);
          hw[0] = hv.x; hw[1] = hv.y; hw[2] = hv.z; hw[3] = hv.w;
        } else {
          const uint4 hv = *reinterpret_cast<const uint4*>(land + 4 * t);
          hw[0] = hv.x; hw[1] = hv.y; hw[2] = hv.z; hw[3] = hv.w;
        }
        const uint32_t aw[4] = {A.attn.x, A.attn.y, A.attn.z, A.attn.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[2 * q] = h2f((uint16_t)(hw[q] & 0xFFFF)) + h2f((uint16_t)(aw[q] & 0xFFFF));
          v[2 * q + 1] = h2f((uint16_t)(hw[q] >> 16)) + h2f((uint16_t)(aw[q] >> 16));
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) ss += v[q] * v[q];
        *reinterpret_cast<float4*>(hattn + 8 * t) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(hattn + 8 * t + 4) = make_float4(v[4], v[5], v[6], v[7]);
      }
      const float tot = block_sum(ss, ms.red);
      const float inv = 1.0f / sqrtf(tot / d + dm.eps);
      if (t < d / 8) {
        uint16_t xv[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) xv[q] = f2h(v[q] * inv);
        const uint4 nat = make_uint4(xv[0] | ((uint32_t)xv[1] << 16), xv[2] | ((uint32_t)xv[3] << 16),
                                     xv[4] | ((uint32_t)xv[5] << 16), xv[6] | ((uint32_t)xv[7] << 16));
        // pair permutation [x0 x4 x1 x5 x2 x6 x3 x7]
        const uint4 per = make_uint4(xv[0] | ((uint32_t)xv[4] << 16), xv[1] | ((uint32_t)xv[5] << 16),
                                     xv[2] | ((uint32_t)xv[6] << 16), xv[3] | ((uint32_t)xv[7] << 16));
        *reinterpret_cast<uint4*>(xnat + 8 * t) = nat;
        *reinterpret_cast<uint4*>(xperm + 8 * t) = per;
        if (cu == 0 && a.x_trace) *reinterpret_cast<uint4*>(a.x_trace + (int64_t)l * d + 8 * t) = nat;
      }
    }
    __syncthreads();
    stamp(a, l, 2);

    // ---- 2. routing ----------------------------------------------------
    int32_t* eidx = a.exec_idx + ((int64_t)cur * a.L + l) * K;
    float* ew = a.exec_w + ((int64_t)cur * a.L + l) * K;
    if (Ly.router) {
      int rb, re;
      split(E, G, cu, rb, re);
      f16rows_finish<kNR>(A.router, A.n_router, d, xnat, ms);
      if (t < A.n_router) ll_put(a.xr + (int64_t)l * E + rb + t, fbits(ms.rows[t]), ep);
      post(a, l, XR);
      wait_all(a, l, XR, &ms.abort);
      ll_gather<2>(a.xr + (int64_t)l * E, E, ep, land, a.flags, &ms.abort);
      __syncthreads();
      if (wave == 0) route_wave(dm, (const float*)land, Ly.router_bias, ms.rs, ms.ridx, ms.rw, a.flags);
      __syncthreads();
      if (t < 16) {
        int64_t ent = 0;
        if (t < K) ent = resolve_entry(Ly.pool, E, ms.ridx[t]);
        ms.ent[t] = ent;
        if (ent < 0 && cu == 0) atomicOr(&a.flags[FLAG_RANGE], 1);
      }
      __syncthreads();
    } else {
      if (t < K) {
        ms.ridx[t] = ms.ridx_all[step * K + t];
        ms.rw[t] = ms.rw_all[step * K + t];
        if (ms.ent[t] < 0 && cu == 0) atomicOr(&a.flags[FLAG_RANGE], 1);
      }
      __syncthreads();
    }
    if (t < K && cu == 0) {
      eidx[t] = ms.ridx[t];
      ew[t] = ms.rw[t];
    }
    stamp(a, l, 3);

    // ---- 3. gate/up rows, shared bases, LoRA A of gate/up ----------------
    {
      GuPlan pl;
      split(n_rt + Is, G, cu, pl.ib, pl.ie);
      if (!A.gu_loaded) gu_issue<CPL_D, IPG>(A.gu, Ly, dm, ms, n_rt, pl, grp, li);
      gu_finish<CPL_D, IPG>(A.gu, Ly, dm, ms, n_rt, Is, pl, grp, li, xperm, xg, ep);
      if (A.n_ax) {
        int b, e;
        split(r2, G, cu, b, e);
        f16rows_finish<kNR>(A.ax, A.n_ax, d, xnat, ms);
        if (t < A.n_ax) ll_put(xg + n_rt + 2 * Is + b + t, fbits(ms.rows[t]), ep);
      }
      post(a, l, XG);
    }
    stamp(a, l, 4);

    // ---- 4. head fc1 / linear path ----------------------------------------
    if (head) {
      int hb, he;
      split(P + E, G, cu, hb, he);
      // one-hot columns of the executed set and of the previous token's set
      if (t < A.n_head * 2 * K) {
        const int j = t / (2 * K), kk = t % (2 * K);
        const int it = hb + j;
        const uint16_t* wrow = it < P ? Ly.head.fc1 + (int64_t)it * F : Ly.head.lin + (int64_t)(it - P) * F;
        int col = -1;
        if (kk < K) {
          const int e = ms.ridx[kk];
          if (e >= 0 && e < E) col = d + e;
        } else {
          const int e = ms.pidx_all[step * K + kk - K];
          if (e >= 0 && e < E) col = d + E + e;
        }
        ms.gath[t] = col >= 0 ? h2f(ldg(wrow + col)) : 0.0f;
      }
      f16rows_finish<kNR>(A.head, A.n_head, d, xnat, ms);
      if (t < A.n_head) {
        float acc = ms.rows[t];
        for (int kk = 0; kk < 2 * K; ++kk) acc += ms.gath[t * 2 * K + kk];
        const int it = hb + t;
        ll_put(a.xa + (int64_t)l * (P + E) + it, fbits(it < P ? gelu_erf(acc) : acc), ep);
      }
      post(a, l, XA);
    }
    stamp(a, l, 5);

    // ---- phase B loads: down rows, shared-expert LoRA matrices, fc2 rows ----
    int db, de;
    {
      int wb, we;
      split(d / 2, G, cu, wb, we);
      db = 2 * wb;
      de = 2 * we;
    }
    DownRegs D;
    const int drow = db + grp;
    if (drow < de) {
      const int wpr = I / 8, spr = I / dm.G;
#pragma unroll
      for (int k = 0; k < kMaxExp; ++k) {
        D.w[k] = make_uint4(0, 0, 0, 0);
        D.s[k] = 0;
        if (k >= nexp || (k < K && ms.ent[k] < 0)) continue;
        const uint32_t* q = k < K ? (const uint32_t*)entry_ptr(Ly.pool.down.q, ms.ent[k], Ly.pool.stride_q) : Ly.sh.down.q;
        const uint16_t* sc = k < K ? (const uint16_t*)entry_ptr(Ly.pool.down.s, ms.ent[k], Ly.pool.stride_s) : Ly.sh.down.s;
        D.w[k] = ldg(reinterpret_cast<const uint4*>(q + (int64_t)drow * wpr + 4 * li));
        D.s[k] = ldg(sc + (int64_t)drow * spr + (32 * li) / dm.G);
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        D.bd[c] = make_uint4(0, 0, 0, 0);
        if (has_sh && Ly.sh.bd && c * 8 < dm.r && li == 0)
          D.bd[c] = ldg(reinterpret_cast<const uint4*>(Ly.sh.bd + (int64_t)drow * dm.r + 8 * c));
      }
    }
    // LoRA matrices of the shared expert: B_gate, B_up [Is, r], A_down [r, Is]
    uint4 lr[kLoraRegs];
    const int n_lora16 = has_sh && dm.r > 0 ? (3 * Is * dm.r) / 8 : 0;
    const bool lora_gu = has_sh && Ly.sh.bg;
    const bool lora_d = has_sh && Ly.sh.ad;
#pragma unroll
    for (int j = 0; j < kLoraRegs; ++j) {
      lr[j] = make_uint4(0, 0, 0, 0);
      const int c = t + kThreads * j;
      if (c >= n_lora16) continue;
      const int per = Is * dm.r / 8;  // chunks per matrix
      const int m = c / per, off = c % per;
      const uint16_t* src = m == 0 ? Ly.sh.bg : (m == 1 ? Ly.sh.bu : Ly.sh.ad);
      if ((m < 2 && lora_gu) || (m == 2 && lora_d)) lr[j] = ldg(reinterpret_cast<const uint4*>(src + 8 * off));
    }
    F16Rows<kNR> fc2r;
    int n_fc2 = 0, fb = 0, fe = 0;
    if (head) {
      split(E, G, cu, fb, fe);
      n_fc2 = fe - fb;
      const uint16_t* rp[kNR];
      for (int j = 0; j < kNR; ++j) rp[j] = Ly.head.fc2 + (int64_t)(fb + (j < n_fc2 ? j : 0)) * P;
      f16rows_issue<kNR>(fc2r, rp, n_fc2, P);
    }

    // ---- 5. gather SwiGLU outputs; finish the shared expert ----------------
    stamp(a, l, 6);
    const int ng_l = n_rt + 2 * Is + r2;
    wait_all(a, l, XG, &ms.abort);
    ll_gather<16>(xg, ng_l, ep, land, a.flags, &ms.abort);
#pragma unroll
    for (int j = 0; j < kLoraRegs; ++j) {
      const int c = t + kThreads * j;
      if (c < n_lora16) *reinterpret_cast<uint4*>(lora + 8 * c) = lr[j];
    }
    __syncthreads();
    stamp(a, l, 7);
    if (has_sh) {
      const float c = dm.lora_scale;
      const float* axg = (const float*)land + n_rt + 2 * Is;
      const int r = dm.r;
      const uint16_t* Bg = lora;
      const uint16_t* Bu = lora + Is * r;
      const uint16_t* Ad = lora + 2 * Is * r;
      for (int i = t; i < Is; i += kThreads) {
        float g = bitsf(land[n_rt + i]), u = bitsf(land[n_rt + Is + i]);
        if (r2) {
          float lg = 0.0f, lu = 0.0f;
          for (int q = 0; q < r; ++q) {
            lg += h2f(Bg[i * r + q]) * axg[q];
            lu += h2f(Bu[i * r + q]) * axg[r + q];
          }
          g += c * lg;
          u += c * lu;
        }
        land[n_rt + i] = fbits(silu(g) * u);  // the shared SwiGLU output replaces the gate base
      }
      __syncthreads();
      if (lora_d) {
        const float* hsh = (const float*)land + n_rt;
        for (int q = grp; q < r; q += kGroups) {
          float acc = 0.0f;
          for (int i = li; i < Is; i += kLG) acc += h2f(Ad[q * Is + i]) * hsh[i];
          acc = group_sum<kLG>(acc);
          if (li == 0) ms.ad[q] = acc;
        }
      }
    }
    // fp16 hi/lo copies of each expert's SwiGLU output for the down GEMVs
    for (int k = wave; k < nexp; k += kThreads / 64) {
      const float* src = (const float*)land + (k < K ? k * I : n_rt);
      float m = 0.0f;
      for (int i = lane; i < I; i += 64) m = fmaxf(m, fabsf(src[i]));
      m = wave_max(m);
      if (lane == 0) ms.emax[k] = m;
    }
    __syncthreads();
    for (int idx = t; idx < nexp * (I / 8); idx += kThreads) {
      const int k = idx / (I / 8), blk = idx % (I / 8);
      const float* src = (const float*)land + (k < K ? k * I : n_rt) + 8 * blk;
      const int e = hilo_exponent(ms.emax[k]);
      const float inv = ldexpf(1.0f, -e);
      uint16_t hi[8], lo2[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        f16 h_, l_;
        split_hilo(src[q], inv, h_, l_);
        hi[q] = __builtin_bit_cast(uint16_t, h_);
        lo2[q] = __builtin_bit_cast(uint16_t, l_);
      }
      uint16_t* hh = hk + (int64_t)k * 2 * I + 8 * blk;
      *reinterpret_cast<uint4*>(hh) = make_uint4(hi[0] | ((uint32_t)hi[4] << 16), hi[1] | ((uint32_t)hi[5] << 16),
                                                 hi[2] | ((uint32_t)hi[6] << 16), hi[3] | ((uint32_t)hi[7] << 16));
      *reinterpret_cast<uint4*>(hh + I) = make_uint4(lo2[0] | ((uint32_t)lo2[4] << 16), lo2[1] | ((uint32_t)lo2[5] << 16),
                                                     lo2[2] | ((uint32_t)lo2[6] << 16), lo2[3] | ((uint32_t)lo2[7] << 16));
      if (blk == 0)
        ms.coef[k] = k < K ? (ms.ent[k] < 0 ? 0.0f : ms.rw[k] * ldexpf(1.0f, e)) : ldexpf(1.0f, e);
    }
    __syncthreads();
    stamp(a, l, 8);

    // ---- 6. down rows: combine, shared expert, down LoRA, residual ---------
    if (drow < de) {
      float acc = 0.0f;
#pragma unroll
      for (int k = 0; k < kMaxExp; ++k) {
        if (k >= nexp || (k < K && ms.ent[k] < 0)) continue;
        const uint16_t* hh = hk + (int64_t)k * 2 * I;
        f16x2 xh[16], xl[16];
        load_xchunk(hh, li, xh);
        load_xchunk(hh + I, li, xl);
        acc += ms.coef[k] * (h2f(D.s[k]) * q4_dot32_hl(D.w[k], xh, xl));
      }
      if (has_sh && Ly.sh.bd && li == 0) {
        float lsum = 0.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (c * 8 >= dm.r) continue;
          const uint32_t bw[4] = {D.bd[c].x, D.bd[c].y, D.bd[c].z, D.bd[c].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            lsum += h2f((uint16_t)(bw[q] & 0xFFFF)) * ms.ad[8 * c + 2 * q];
            lsum += h2f((uint16_t)(bw[q] >> 16)) * ms.ad[8 * c + 2 * q + 1];
          }
        }
        acc += dm.lora_scale * lsum;
      }
      acc = group_sum<kLG>(acc);
      if (li == 0) {
        const uint16_t hv = f2h(hattn[drow] + acc);
        a.h[(int64_t)(step + 1) * d + drow] = hv;
        ms.hstage[drow - db] = hv;
      }
    }
    __syncthreads();
    for (int j = db / 2 + t; j < de / 2; j += kThreads) {
      const int r0 = 2 * j - db;
      const uint32_t pr = (uint32_t)ms.hstage[r0] | ((uint32_t)ms.hstage[r0 + 1] << 16);
      ll_put(a.xh + (int64_t)l * (d / 2) + j, pr, ep);
    }
    post(a, l, XH);
    stamp(a, l, 9);

    // next layer's activation-independent loads go out before the fc2 work
    if (l + 1 < a.l1) issue_a(l + 1, A);

    // ---- 7. head fc2 rows ----------------------------------------------------
    if (head) {
      wait_all(a, l, XA, &ms.abort);
      ll_gather<4>(a.xa + (int64_t)l * (P + E), P + E, ep, land, a.flags, &ms.abort);
      __syncthreads();
      {
        float m = 0.0f;
        for (int i = t; i < P; i += kThreads) m = fmaxf(m, fabsf(bitsf(land[i])));
        m = wave_max(m);
        if (lane == 0) ms.red[wave] = m;
        __syncthreads();
        float mx = 0.0f;
        for (int j = 0; j < kThreads / 64; ++j) mx = fmaxf(mx, ms.red[j]);
        const int e = hilo_exponent(mx);
        const float inv = ldexpf(1.0f, -e);
        for (int i = t; i < P; i += kThreads) {
          f16 hi, lo2;
          split_hilo(bitsf(land[i]), inv, hi, lo2);
          ha[i] = __builtin_bit_cast(uint16_t, hi);
          ha[P + i] = __builtin_bit_cast(uint16_t, lo2);
        }
        if (t == 0) ms.ha_scale = ldexpf(1.0f, e);
      }
      __syncthreads();
      f16rows_finish_hl<kNR>(fc2r, n_fc2, P, ha, ha + P, ms);
      if (t < n_fc2) {
        const int e = fb + t;
        const float logit = ms.rows[t] * ms.ha_scale + bitsf(land[P + e]);
        ll_put(a.xl + (int64_t)l * E + e, fbits(logit), ep);
        if (a.head_logits) a.head_logits[(int64_t)l * E + e] = logit;
      }
      post(a, l, XL);
    }
    __syncthreads();
  }

  // ---- routing of each head's logits: the next token's prediction ----------
  for (int l = a.l0 + cu; l < a.l1; l += G) {
    const LayerDev& Ly = a.layers[l];
    if (!Ly.head.fc1) continue;
    wait_all(a, l, XL, &ms.abort);
    ll_gather<2>(a.xl + (int64_t)l * E, E, ep, land, a.flags, &ms.abort);
    __syncthreads();
    int32_t* pidx = l + 1 < a.L ? a.route_idx + ((int64_t)nxt * a.L + l + 1) * K : a.sink_idx;
    float* pw = l + 1 < a.L ? a.route_w + ((int64_t)nxt * a.L + l + 1) * K : a.sink_w;
    if (wave == 0) route_wave(dm, (const float*)land, Ly.head.bias, ms.rs, pidx, pw, a.flags);
    __syncthreads();
  }
}

template <int CPL_D, int IPG>
hipError_t launch_stack_t(const StackArgs& a, int grid, hipStream_t st) {
  const Lds lo = lds_layout(a.dm, a.ng);
  static bool attr_set = false;
  if (!attr_set) {
    hipFuncSetAttribute((const void*)k_stack<CPL_D, IPG>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr_set = true;
  }
  hipLaunchKernelGGL((k_stack<CPL_D, IPG>), dim3(grid), dim3(kThreads), (size_t)lo.bytes, st, a);
  return hipGetLastError();
}

}  // namespace

int stack_lds_bytes(const Dims& dm, int ng) { return lds_layout(dm, ng).bytes; }

bool stack_supported(const Dims& dm) {
  if (dm.d % 512 || dm.I != 512 || dm.K > 8 || dm.E > kMaxE || dm.r > 16) return false;
  if (dm.Is != 0 && dm.Is != dm.I) return false;
  if (3 * dm.Is * dm.r / 8 > kLoraRegs * kThreads) return false;
  if (dm.P % 8 || dm.P > 2048) return false;
  const int cpl = dm.d / 512;
  return cpl == 3 || cpl == 4;
}

hipError_t launch_stack(const StackArgs& a, int grid, hipStream_t st) {
  const Dims& dm = a.dm;
  // Work per workgroup must fit the fixed per-thread plans.
  const int gu_items = dm.K * dm.I + dm.Is;
  const int ipg = (gu_items + grid - 1) / grid;
  if (a.l1 - a.l0 > kMaxL || grid < 1 || grid > 512 || !a.fl) return hipErrorInvalidValue;
  if ((dm.E + grid - 1) / grid > kNR || (dm.P + dm.E + grid - 1) / grid > kNR ||
      (2 * dm.r + grid - 1) / grid > kNR || 2 * ((dm.d / 2 + grid - 1) / grid) > kGroups ||
      2 * dm.K * kNR > kNR * 16)
    return hipErrorInvalidValue;
  const int cpl = dm.d / 512;
  if (ipg <= kGroups) {
    if (cpl == 3) return launch_stack_t<3, 1>(a, grid, st);
    if (cpl == 4) return launch_stack_t<4, 1>(a, grid, st);
  } else if (ipg <= 2 * kGroups) {
    if (cpl == 3) return launch_stack_t<3, 2>(a, grid, st);
    if (cpl == 4) return launch_stack_t<4, 2>(a, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace smd
