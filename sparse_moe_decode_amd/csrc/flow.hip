// Wave-specialised persistent decode kernel: one launch runs one token through
// a range of layers, with the weight stream decoupled from the dependent chain.
//
// What one layer computes ("The Other Half of the Memory Wall" §3.1 Math
// contract, §3.2 Motivation / Head / Prediction-as-routing, §3.3; head
// layout as listed in "I counted the bytes it can't stream"):
//   x = fp16(RMSNorm(h + a)); routing (own router, or the previous token's
//   prediction); SwiGLU of the K routed experts and the shared expert (with
//   its unmerged LoRA); weighted down projections; h' = fp16(h + a + y); and,
//   on head layers, the prerouter head over [x; onehot(S_cur); onehot(S_prev)]
//   whose top-K becomes the next token's routing of the next layer.
//
// Layout of the work on the chip:
//   * gate/up CUs [0, ng): gather h_l, norm it (every one of them), own a
//     contiguous range of (expert, row) SwiGLU items and publish their
//     outputs; the first E/4 also own four router rows each, the next 2r one
//     LoRA A row each (the shared expert's gate/up A products); in the wait
//     for the next layer they compute their share of the head's fc1 and
//     linear-path rows;
//   * down CUs [ng, ng + nd): gather all SwiGLU outputs, own a contiguous
//     range of output row pairs (every expert slot, the down LoRA, the
//     residual) and publish h_{l+1}; in the wait for the next layer they
//     compute their share of the previous head's fc2 rows, and one of them
//     ranks the head before that into the next token's prediction.
// Every CU runs four compute waves and three loader waves. The loaders
// stream a layer's rows into one of two LDS layer slots with direct-to-LDS
// loads (their own vector memory counters, no registers), a layer ahead of
// the compute; the third streams router and head rows into their own
// buffers. Routed rows of a predicted layer are known at launch; on a router
// layer they are issued as soon as the CU has ranked its own logits.
// Loaders and compute waves meet only through LDS flags; the compute waves
// synchronise among themselves with an LDS counter.
//
// Cross-CU data moves as 8-byte words (32-bit payload, 32-bit launch epoch)
// stored and polled with agent-scope relaxed atomics (single-copy atomic, so
// a word with the current epoch carries this launch's payload). Each
// producer owns whole 64-byte blocks (no line is written by two CUs), and
// consumers poll with 16-byte coherent loads. Every wait is bounded by the
// wall clock; on expiry the kernel raises FLAG_SYNC and runs to completion.

#include "gemv.h"
#include "internal.h"

namespace smd {

namespace {

constexpr int kFC = 256;                  // compute threads (four waves)
constexpr int kFW = kFC / 64;
constexpr int kFL = 3;                    // loader waves
constexpr int kFThreads = kFC + 64 * kFL;
constexpr int kGL = 16;                   // lanes per group
constexpr int kGN = kFC / kGL;            // groups
constexpr int kFRank = 16;
constexpr int kFI = 512;
constexpr int kFMaxL = 64;
constexpr uint64_t kFSpin = 20000000ull;  // 0.2 s of the 100 MHz wall clock
constexpr int kRouterRows = 4;
constexpr int kBlk = 8;                   // words of a small exchange block

// LDS flag words (loader <-> compute handshakes, compute barrier).
enum {
  FL_READY = 0,    // [2] layer slot landed (step + 1)
  FL_PRE = 2,      // [2] the part of the slot that needs no routing landed
  FL_FREED = 4,    // [2][4] slot released by compute wave w (step + 1)
  FL_ROUTE = 12,   // routing of this step known (step + 1)
  FL_RREADY = 13,  // router rows landed (step + 1)
  FL_RFREED = 14,  // [4] router rows consumed by wave w (step + 1)
  FL_HREADY = 18,  // head rows / fc2 rows landed (step + 1)
  FL_HFREED = 19,  // [4] consumed by wave w (step + 1)
  FL_CBAR = 23,
  FL_ABORT = 24,
  FL_N = 32
};

// per-step layer flags
enum { LF_ROUTER = 1, LF_HEAD = 2, LF_SHARED = 4, LF_LORA = 8, LF_LORAD = 16, LF_ATTN = 32 };

__shared__ __align__(16) unsigned char s_mem[kFlowLds];
__shared__ int s_fl[FL_N];

typedef __attribute__((address_space(3))) void lds_v;
typedef __attribute__((address_space(1))) void glb_v;
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int fl_ld(int i) {
  return __hip_atomic_load(&s_fl[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void fl_st(int i, int v) {
  __hip_atomic_store(&s_fl[i], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

struct Waiter {
  uint64_t t0;
  uint32_t polls;
};

// A wait gives up once this CU has given up, any CU raised the sync flag, or
// 0.2 s passed (then it raises the flag itself).
__device__ __forceinline__ bool expired(Waiter& w, int32_t* gflags) {
  if (fl_ld(FL_ABORT)) return true;
  if ((++w.polls & 63u) == 0 &&
      __hip_atomic_load(&gflags[FLAG_SYNC], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    fl_st(FL_ABORT, 1);
    return true;
  }
  if (wall_clock64() - w.t0 > kFSpin) {
    atomicOr(&gflags[FLAG_SYNC], 1);
    fl_st(FL_ABORT, 1);
    return true;
  }
  return false;
}

// Wait until flag i reaches v.
__device__ __forceinline__ void fl_wait(int i, int v, int32_t* gflags) {
  if (fl_ld(i) >= v) return;
  Waiter w{(uint64_t)wall_clock64(), 0};
  while (fl_ld(i) < v) {
    if (expired(w, gflags)) return;
    __builtin_amdgcn_s_sleep(1);
  }
}

// Wait until flags i .. i+n-1 all reach v.
__device__ __forceinline__ void fl_wait_all(int i, int n, int v, int32_t* gflags) {
  for (int q = 0; q < n; ++q) fl_wait(i + q, v, gflags);
}

// Barrier of the compute waves (the loader waves never join it).
__device__ __forceinline__ void cbar(int& phase, int32_t* gflags) {
  phase += kFW;
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
  asm volatile("" ::: "memory");
  if ((threadIdx.x & 63) == 0)
    __hip_atomic_fetch_add(&s_fl[FL_CBAR], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  fl_wait(FL_CBAR, phase, gflags);
  asm volatile("" ::: "memory");
}

// Release a flag after this wave's LDS reads of the resource completed.
__device__ __forceinline__ void release(int i, int v) {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  if ((threadIdx.x & 63) == 0) fl_st(i, v);
}

// Loader: all direct-to-LDS loads of this wave have landed.
__device__ __forceinline__ void dma_drain() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void xput(uint64_t* p, uint32_t v, uint32_t ep) {
  __hip_atomic_store(p, ((uint64_t)ep << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t fbits(float v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float bitsf(uint32_t v) { return __builtin_bit_cast(float, v); }

// Threads [0, nthr) poll words [0, n) of an exchange region (n even, region
// 16-byte aligned) with 16-byte coherent loads until every word carries the
// epoch; sink(word, payload) then sees each word once.
template <int U, typename Sink>
__device__ __forceinline__ void xgather(const uint64_t* base, int n, uint32_t ep, int tid, int nthr,
                                        int32_t* gflags, Sink&& sink) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, n * 8, 0x00020000);
  const int np = n >> 1;
  for (int b0 = 0; b0 < np; b0 += U * nthr) {
    u32x4v v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int p = b0 + j * nthr + tid;
      v[j] = p < np ? __builtin_amdgcn_raw_buffer_load_b128(rs, p * 16, 0, 16)
                    : (u32x4v){0u, ep, 0u, ep};
    }
    Waiter w{0, 0};
    bool started = false;
    for (;;) {
      bool ok = true;
#pragma unroll
      for (int j = 0; j < U; ++j) ok = ok && v[j].y == ep && v[j].w == ep;
      if (ok) break;
      if (!started) {
        w.t0 = wall_clock64();
        started = true;
      }
      if (expired(w, gflags)) break;
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int p = b0 + j * nthr + tid;
        if (p < np && (v[j].y != ep || v[j].w != ep))
          v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, p * 16, 0, 16);
      }
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int p = b0 + j * nthr + tid;
      if (p < np) {
        sink(2 * p, v[j].x);
        sink(2 * p + 1, v[j].z);
      }
    }
  }
}

// Packed exchange words: two floats rounded to 28 bits (sign, exponent and
// 19 mantissa bits, round half away from zero on the magnitude) under an
// 8-bit tag: bits 0-27 the first, 28-55 the second, 56-63 the tag. The tag is
// the launch epoch mod 255, plus 1; the host clears the words before a tag
// could come round again (every 255 launches), so a word with the current
// tag was written by this launch.
__device__ __forceinline__ uint32_t pk_tag(uint32_t epoch) { return epoch % 255u + 1u; }
__device__ __forceinline__ uint64_t q28(float v) { return (uint64_t)((fbits(v) + 8u) >> 4); }
__device__ __forceinline__ void xput2(uint64_t* p, float v0, float v1, uint32_t tag) {
  const uint64_t w = ((uint64_t)tag << 56) | (q28(v1) << 28) | q28(v0);
  __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Gather of n packed words (n even; 16-byte polls, U in flight per thread):
// sink(word index, first value, second value) once per word.
template <int U, typename Sink>
__device__ __forceinline__ void xgather2(const uint64_t* base, int n, uint32_t tag, int tid,
                                         int nthr, int32_t* gflags, Sink&& sink) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, n * 8, 0x00020000);
  const int np = n >> 1;
  const uint32_t want = tag << 24;
  for (int b0 = 0; b0 < np; b0 += U * nthr) {
    u32x4v v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int p = b0 + j * nthr + tid;
      v[j] = p < np ? __builtin_amdgcn_raw_buffer_load_b128(rs, p * 16, 0, 16)
                    : (u32x4v){0u, want, 0u, want};
    }
    Waiter w{0, 0};
    bool started = false;
    for (;;) {
      bool ok = true;
#pragma unroll
      for (int j = 0; j < U; ++j)
        ok = ok && (v[j].y & 0xFF000000u) == want && (v[j].w & 0xFF000000u) == want;
      if (ok) break;
      if (!started) {
        w.t0 = wall_clock64();
        started = true;
      }
      if (expired(w, gflags)) break;
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int p = b0 + j * nthr + tid;
        if (p < np && ((v[j].y & 0xFF000000u) != want || (v[j].w & 0xFF000000u) != want))
          v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, p * 16, 0, 16);
      }
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int p = b0 + j * nthr + tid;
      if (p < np) {
        sink(2 * p, bitsf(v[j].x << 4), bitsf(((v[j].y << 8) | (v[j].x >> 24)) & 0xFFFFFFF0u));
        sink(2 * p + 1, bitsf(v[j].z << 4), bitsf(((v[j].w << 8) | (v[j].z >> 24)) & 0xFFFFFFF0u));
      }
    }
  }
}

template <typename Sink>
__device__ __forceinline__ void xgather_any(const uint64_t* base, int n, uint32_t ep, int tid,
                                            int nthr, int32_t* gflags, Sink&& sink) {
  xgather<8>(base, n, ep, tid, nthr, gflags, sink);
}

// Loader: npieces 16-byte pieces into LDS dst (piece q at dst + 16 q) from
// addr(q); lanes whose piece is invalid (ok(q) false) or past the end load
// nothing.
template <typename Addr, typename Ok>
__device__ __forceinline__ void dma16(unsigned char* dst, int npieces, Addr&& addr, Ok&& ok) {
  const int lane = threadIdx.x & 63;
  for (int i = 0; i < npieces; i += 64) {
    const int q = i + lane;
    if (q < npieces && ok(q))
      __builtin_amdgcn_global_load_lds((glb_v*)addr(q), (lds_v*)(dst + 16 * i), 16, 0, 0);
  }
}

template <typename Addr>
__device__ __forceinline__ void dma4(unsigned char* dst, int npieces, Addr&& addr) {
  const int lane = threadIdx.x & 63;
  for (int i = 0; i < npieces; i += 64) {
    const int q = i + lane;
    if (q < npieces)
      __builtin_amdgcn_global_load_lds((glb_v*)addr(q), (lds_v*)(dst + 4 * i), 4, 0, 0);
  }
}

__device__ __forceinline__ const char* cptr(const void* p) { return (const char*)p; }

// The launch's arguments, read in place from the kernel-argument segment
// with scalar loads. The role functions below are separate functions: a
// reference parameter would make the compiler copy the arguments to scratch,
// and the segment pointer is only defined in the kernel itself, so the
// kernel passes its address and the callee makes it wave-uniform again.
typedef const __attribute__((address_space(4))) FlowArgs KA;
typedef const __attribute__((address_space(4))) FlowPlan KP;
typedef const __attribute__((address_space(4))) Dims KD;
__device__ __forceinline__ KA& args_at(uint64_t p) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)p);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(p >> 32));
  return *(KA*)((((uint64_t)hi) << 32) | lo);
}
// A private copy of the dimensions (for helpers taking an ordinary reference).
__device__ __forceinline__ Dims dims_of(KD& k) {
  Dims d;
  d.d = k.d; d.E = k.E; d.K = k.K; d.I = k.I; d.Is = k.Is; d.P = k.P; d.G = k.G; d.r = k.r;
  d.lora_scale = k.lora_scale;
  d.router_kind = k.router_kind; d.norm_topk = k.norm_topk; d.n_groups = k.n_groups;
  d.topk_groups = k.topk_groups;
  d.route_scale = k.route_scale; d.eps = k.eps;
  d.affine = k.affine;
  return d;
}

// Contiguous share [beg, end) of n items for part c of G.
__device__ __forceinline__ int share_b(int n, int G, int c) {
  return (int)((uint32_t)n * (uint32_t)c / (uint32_t)G);  // n * c < 2^32
}

__device__ __forceinline__ void stamp(KA& a, int row, int k) {
  if (a.trace && threadIdx.x == 0)
    a.trace[((int64_t)blockIdx.x * (a.L + 1) + row) * kTracePoints + k] = wall_clock64();
}

__device__ __forceinline__ float dot8_h(uint4 w, uint4 x, float acc) {
  acc = dot2(as_h2(w.x), as_h2(x.x), acc);
  acc = dot2(as_h2(w.y), as_h2(x.y), acc);
  acc = dot2(as_h2(w.z), as_h2(x.z), acc);
  acc = dot2(as_h2(w.w), as_h2(x.w), acc);
  return acc;
}

template <typename T>
__device__ __forceinline__ T* lds_at(int off) {
  return reinterpret_cast<T*>(s_mem + off);
}

// Routing tables of the launch in LDS ([nL][K] each), per-step layer flags,
// and the work split: first routed item of routed CU c (ibr[c], c <= ngr),
// first shared row of shared CU c (ibs[c], c <= ng - ngr), first row pair of
// down CU j (pb[j], j <= nd), first head row of gate/up CU c (hb[c],
// c <= ng), first fc2 row of down CU j (fb[j]).
struct RT {
  int32_t* idx;
  float* w;
  int32_t* prev;
  int32_t* ent;
  int32_t* lf;
  int32_t *ibr, *ibs, *pb, *hb, *fb;
};

template <typename P>
__device__ __forceinline__ RT rt_at(int off, int nL, int K, P& p) {
  RT t;
  t.idx = lds_at<int32_t>(off);
  t.w = lds_at<float>(off + nL * K * 4);
  t.prev = lds_at<int32_t>(off + 2 * nL * K * 4);
  t.ent = lds_at<int32_t>(off + 3 * nL * K * 4);
  t.lf = lds_at<int32_t>(off + 4 * nL * K * 4);
  t.ibr = t.lf + nL;
  t.ibs = t.ibr + p.ngr + 1;
  t.pb = t.ibs + (p.ng - p.ngr) + 1;
  t.hb = t.pb + p.nd + 1;
  t.fb = t.hb + p.ng + 1;
  return t;
}

// A wave-uniform float in a scalar register.
__device__ __forceinline__ float uniform_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// Dot of a wave's fp16 row (LDS, natural order, d columns) with x (LDS,
// natural fp16): lane takes 8-element chunks lane + 64 m.
template <int CPL>
__device__ __forceinline__ float wave_row_dot(const uint16_t* row, const uint16_t* x) {
  const int lane = threadIdx.x & 63;
  float pm[CPL];
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const int c = lane + 64 * m;
    pm[m] = dot8_h(*reinterpret_cast<const uint4*>(row + 8 * c),
                   *reinterpret_cast<const uint4*>(x + 8 * c), 0.0f);
  }
  float acc = 0.0f;
#pragma unroll
  for (int m = 0; m < CPL; ++m) acc += pm[m];
  return acc;
}

// fp16 bits of v, saturated to the largest finite fp16 (NaN stays NaN).
__device__ __forceinline__ uint16_t f2h_sat(float v) {
  return f2h(v == v ? fminf(fmaxf(v, -65504.0f), 65504.0f) : v);
}

// Loader waves stamp trace points from their first lane.
__device__ __forceinline__ void lstamp(KA& a, int row, int k) {
  if (a.trace && (threadIdx.x & 63) == 0)
    a.trace[((int64_t)blockIdx.x * (a.L + 1) + row) * kTracePoints + k] = wall_clock64();
}

// Item range of gate/up CU cu: routed CUs own routed items (global index
// it = k*I + row), shared CUs rows of the shared expert.
struct Items {
  bool shared;
  int b, e;  // routed: item indices; shared: shared-expert rows
};

template <typename P>
__device__ __forceinline__ Items items_of(const RT& rt, P& p, int cu) {
  Items r;
  r.shared = cu >= p.ngr;
  if (r.shared) {
    r.b = rt.ibs[cu - p.ngr];
    r.e = rt.ibs[cu - p.ngr + 1];
  } else {
    r.b = rt.ibr[cu];
    r.e = rt.ibr[cu + 1];
  }
  return r;
}

// ============================================================ gate/up CUs ==

template <int CPL, int KM>
__device__ __attribute__((noinline)) void gu_loader(uint64_t kap, int lw) {
  KA& a = args_at(kap);
  KP& p = a.pl;
  constexpr int d = 512 * CPL;
  const int K = a.dm.K, E = a.dm.E, r = a.dm.r, I = kFI;
  const int nL = a.l1 - a.l0;
  const int cu = blockIdx.x;
  const RT rt = rt_at(p.g_rt, nL, K, p);
  const Items it = items_of(rt, p, cu);
  const int ipc = it.e - it.b;
  const int aq = (cu >= p.ca0 && cu < p.ca0 + 2 * r) ? cu - p.ca0 : -1;
  int32_t* gf = a.flags;
  if (lw < 2) {
    for (int step = lw; step < nL; step += 2) {
      const int slot = lw;
      const int l = a.l0 + step;
      if (step >= 2) fl_wait_all(FL_FREED + 4 * slot, kFW, step - 1, gf);
      lstamp(a, l, 10 + slot);
      const LayerDev& Ly = a.layers[l];
      const int lf = rt.lf[step];
      unsigned char* S = s_mem + slot * p.g_slot;
      if (lf & LF_ATTN)
        dma16(S + p.g_at, d / 8, [&](int q) { return cptr(Ly.attn) + 16 * q; },
              [](int) { return true; });
      if (aq >= 0 && (lf & LF_LORA)) {
        const uint16_t* A = (aq < r ? Ly.sh.ag : Ly.sh.au) + (int64_t)(aq % r) * d;
        dma16(S + p.g_ar, d / 8, [&](int q) { return cptr(A) + 16 * q; }, [](int) { return true; });
      }
      // items: gate/up rows (d/32 pieces each), then their scales (d/512 each)
      const int pr = d / 32, ps = d / 512;
      auto item_dma = [&]() {
        auto base = [&](int jj, int pj, bool sc) -> const char* {
          if (it.shared) {
            const int row = it.b + jj;
            const Q4& q4 = pj ? Ly.sh.up : Ly.sh.gate;
            return sc ? cptr(q4.s) + (int64_t)row * (d / 32) : cptr(q4.q) + (int64_t)row * (d / 2);
          }
          const int gi = it.b + jj, k = gi / I, row = gi % I;
          const int ent = rt.ent[step * K + k];
          const Q4& q4 = pj ? Ly.pool.up : Ly.pool.gate;
          return sc ? cptr(q4.s) + ent * Ly.pool.stride_s + (int64_t)row * (d / 32)
                    : cptr(q4.q) + ent * Ly.pool.stride_q + (int64_t)row * (d / 2);
        };
        auto valid = [&](int jj) {
          return it.shared ? (lf & LF_SHARED) != 0 : rt.ent[step * K + (it.b + jj) / I] >= 0;
        };
        dma16(S + p.g_gq, ipc * 2 * pr,
              [&](int q) {
                const int jj = q / (2 * pr), rem = q % (2 * pr);
                return base(jj, rem / pr, false) + 16 * (rem % pr);
              },
              [&](int q) { return valid(q / (2 * pr)); });
        dma16(S + p.g_gs, ipc * 2 * ps,
              [&](int q) {
                const int jj = q / (2 * ps), rem = q % (2 * ps);
                return base(jj, rem / ps, true) + 16 * (rem % ps);
              },
              [&](int q) { return valid(q / (2 * ps)); });
      };
      const bool known = it.shared || !(lf & LF_ROUTER);
      if (known) item_dma();
      dma_drain();
      fl_st(FL_PRE + slot, step + 1);
      if (!known) {
        fl_wait(FL_ROUTE, step + 1, gf);
        lstamp(a, l, 12);
        item_dma();
        dma_drain();
      }
      fl_st(FL_READY + slot, step + 1);
      lstamp(a, l, 13);
    }
    return;
  }
  // router rows and head rows
  const bool rcu = cu < p.nrc;
  const int r0 = kRouterRows * cu, r1 = min(r0 + kRouterRows, E);
  const int hb = rt.hb[cu], he = rt.hb[cu + 1];
  const int P = a.dm.P, F = d + 2 * E;
  int prev_r = 0, prev_h = 0;
  for (int step = 0; step < nL; ++step) {
    const int l = a.l0 + step;
    const int lf = rt.lf[step];
    const LayerDev& Ly = a.layers[l];
    if ((lf & LF_ROUTER) && rcu && r1 > r0) {
      fl_wait_all(FL_RFREED, kFW, prev_r, gf);
      dma16(s_mem + p.g_rb, (r1 - r0) * (d / 8),
            [&](int q) { return cptr(Ly.router) + ((int64_t)(r0 + q / (d / 8)) * d) * 2 + 16 * (q % (d / 8)); },
            [](int) { return true; });
      dma_drain();
      fl_st(FL_RREADY, step + 1);
      prev_r = step + 1;
    }
    if (lf & LF_HEAD) {
      fl_wait_all(FL_HFREED, kFW, prev_h, gf);
      auto hrow = [&](int hr) -> const char* {
        return hr < P ? cptr(Ly.head.fc1) + (int64_t)hr * F * 2 : cptr(Ly.head.lin) + (int64_t)(hr - P) * F * 2;
      };
      if (he > hb) {
        dma16(s_mem + p.g_hb, (he - hb) * (d / 8),
              [&](int q) { return hrow(hb + q / (d / 8)) + 16 * (q % (d / 8)); },
              [](int) { return true; });
        if (lf & LF_ROUTER) fl_wait(FL_ROUTE, step + 1, gf);
        dma4(s_mem + p.g_hc, (he - hb) * 2 * K, [&](int q) {
          const int rr = q / (2 * K), kk = q % (2 * K);
          const int e = kk < K ? rt.idx[step * K + kk] : rt.prev[step * K + kk - K];
          const int col = (e >= 0 && e < E) ? (kk < K ? d + e : d + E + e) : d;
          return hrow(hb + rr) + (col & ~1) * 2;
        });
      }
      dma_drain();
      fl_st(FL_HREADY, step + 1);
      prev_h = step + 1;
    }
  }
}

template <int CPL, int KM>
__device__ __attribute__((noinline)) void gu_compute(uint64_t kap) {
  KA& a = args_at(kap);
  KP& p = a.pl;
  constexpr int d = 512 * CPL;
  const Dims dm = dims_of(a.dm);
  const int K = dm.K, E = dm.E, r = dm.r, I = kFI, P = dm.P;
  const int nL = a.l1 - a.l0;
  const int cu = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int li = t % kGL, grp = t / kGL;
  const uint32_t ep = a.epoch;
  const int cur = a.token & 1;
  int32_t* gf = a.flags;
  const RT rt = rt_at(p.g_rt, nL, K, p);
  const Items it = items_of(rt, p, cu);
  const int ipc = it.e - it.b;
  const int aq = (cu >= p.ca0 && cu < p.ca0 + 2 * r) ? cu - p.ca0 : -1;
  const bool rcu = cu < p.nrc;
  const int r0 = kRouterRows * cu, r1 = min(r0 + kRouterRows, E);
  const int hb = rt.hb[cu], he = rt.hb[cu + 1];
  const int bir = 1 << p.lbr, hs = 1 << p.lhs;
  const uint32_t tag = pk_tag(ep);
  uint16_t* hbuf = lds_at<uint16_t>(p.g_h);
  uint16_t* xn = lds_at<uint16_t>(p.g_xn);
  uint16_t* xp = lds_at<uint16_t>(p.g_xp);
  float* lg = lds_at<float>(p.g_lg);
  RouteScratch& rs = *lds_at<RouteScratch>(p.g_rs);
  int phase = 0;

  for (int step = 0; step < nL; ++step) {
    const int l = a.l0 + step;
    const int slot = step & 1;
    const int lf = rt.lf[step];
    const unsigned char* S = s_mem + slot * p.g_slot;
    uint64_t* X = a.xbuf + (int64_t)l * p.xlayer;
    uint64_t* XB = X + p.o_xb;
    const LayerDev& Ly = a.layers[l];
    stamp(a, l, 0);
    fl_wait(FL_PRE + slot, step + 1, gf);

    // ---- h_l ---------------------------------------------------------------
    if (step == 0) {
      if (t < d / 8)
        *reinterpret_cast<uint4*>(hbuf + 8 * t) = ldg(reinterpret_cast<const uint4*>(a.h + 8 * t));
    } else {
      const uint64_t* XA = a.xbuf + (int64_t)(l - 1) * p.xlayer + p.o_xa;
      uint32_t* h32 = reinterpret_cast<uint32_t*>(hbuf);
      const int lba = p.lba;
      if (p.direct & 4) {  // every down CU owns 1 << lba row pairs: word w is pair w
        xgather_any(XA, p.nd << lba, ep, t, kFC, gf, [&](int wi, uint32_t v) { h32[wi] = v; });
      } else {
        xgather_any(XA, p.nd << lba, ep, t, kFC, gf, [&](int wi, uint32_t v) {
          const int jd = wi >> lba, o = wi & ((1 << lba) - 1);
          const int pb = rt.pb[jd];
          if (o < rt.pb[jd + 1] - pb) h32[pb + o] = v;
        });
      }
    }
    cbar(phase, gf);
    stamp(a, l, 1);

    // ---- RMSNorm: every wave sums the squares itself -------------------------
    {
      const uint16_t* at = reinterpret_cast<const uint16_t*>(S + p.g_at);
      const bool att = (lf & LF_ATTN) != 0;
      float ssq[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int m = 0; m < CPL; ++m) {
        const int c = lane + 64 * m;
        const uint4 hv = *reinterpret_cast<const uint4*>(hbuf + 8 * c);
        const uint4 av = att ? *reinterpret_cast<const uint4*>(at + 8 * c) : make_uint4(0, 0, 0, 0);
        const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w}, aw[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float v0 = h2f((uint16_t)(hw[q] & 0xFFFF)) + h2f((uint16_t)(aw[q] & 0xFFFF));
          const float v1 = h2f((uint16_t)(hw[q] >> 16)) + h2f((uint16_t)(aw[q] >> 16));
          ssq[q] = fmaf(v0, v0, ssq[q]);
          ssq[q] = fmaf(v1, v1, ssq[q]);
        }
      }
      const float tot = wave_sum_rows((ssq[0] + ssq[1]) + (ssq[2] + ssq[3]));
      const float inv = 1.0f / sqrtf(tot / d + dm.eps);
      if (t < d / 8) {
        const uint4 hv = *reinterpret_cast<const uint4*>(hbuf + 8 * t);
        const uint4 av = att ? *reinterpret_cast<const uint4*>(at + 8 * t) : make_uint4(0, 0, 0, 0);
        const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w}, aw[4] = {av.x, av.y, av.z, av.w};
        uint16_t xv[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xv[2 * q] = f2h((h2f((uint16_t)(hw[q] & 0xFFFF)) + h2f((uint16_t)(aw[q] & 0xFFFF))) * inv);
          xv[2 * q + 1] = f2h((h2f((uint16_t)(hw[q] >> 16)) + h2f((uint16_t)(aw[q] >> 16))) * inv);
        }
        const uint4 nat = make_uint4(xv[0] | ((uint32_t)xv[1] << 16), xv[2] | ((uint32_t)xv[3] << 16),
                                     xv[4] | ((uint32_t)xv[5] << 16), xv[6] | ((uint32_t)xv[7] << 16));
        const uint4 per = make_uint4(xv[0] | ((uint32_t)xv[4] << 16), xv[1] | ((uint32_t)xv[5] << 16),
                                     xv[2] | ((uint32_t)xv[6] << 16), xv[3] | ((uint32_t)xv[7] << 16));
        *reinterpret_cast<uint4*>(xn + 8 * t) = nat;
        *reinterpret_cast<uint4*>(xp + 8 * t) = per;
        if (cu == 0 && a.x_trace) *reinterpret_cast<uint4*>(a.x_trace + (int64_t)l * d + 8 * t) = nat;
      }
    }
    cbar(phase, gf);
    stamp(a, l, 2);

    // ---- LoRA A row of the shared gate/up, router rows --------------------------
    if (aq >= 0 && wave == 0) {
      float v = 0.0f;
      if (lf & LF_LORA) v = wave_sum_rows(wave_row_dot<CPL>(reinterpret_cast<const uint16_t*>(S + p.g_ar), xn));
      if (lane < kBlk) xput2(XB + p.xb_a + aq * kBlk + lane, lane == 0 ? v : 0.0f, 0.0f, tag);
    }
    if ((lf & LF_ROUTER) && rcu) {
      fl_wait(FL_RREADY, step + 1, gf);
      const int nr = r1 - r0;
      if (wave < nr) {
        const float v = wave_sum_rows(wave_row_dot<CPL>(lds_at<uint16_t>(p.g_rb) + wave * d, xn));
        if (lane == 0) xput(X + p.o_xr + cu * kBlk + wave, fbits(v), ep);
      }
      if (wave == 0 && lane >= nr && lane < kBlk) xput(X + p.o_xr + cu * kBlk + lane, 0u, ep);
      release(FL_RFREED + wave, step + 1);
    }

    // ---- routing -----------------------------------------------------------
    if (lf & LF_ROUTER) {
      if (wave == 0) {
        xgather_any(X + p.o_xr, p.nrc * kBlk, ep, lane, 64, gf, [&](int wi, uint32_t v) {
          const int c = wi >> 3, o = wi & 7, e = kRouterRows * c + o;
          if (o < kRouterRows && e < E) lg[e] = bitsf(v);
        });
        wave_lds_sync();
        route_wave(dm, lg, Ly.router_bias, rs, rt.idx + step * K, rt.w + step * K, gf);
        wave_lds_sync();
        if (lane < K) {
          const int64_t ent = resolve_entry(Ly.pool, E, rt.idx[step * K + lane]);
          rt.ent[step * K + lane] = (int32_t)ent;
          if (ent < 0 && cu == 0) atomicOr(&gf[FLAG_RANGE], 1);
        }
        release(FL_ROUTE, step + 1);
      } else {
        fl_wait(FL_ROUTE, step + 1, gf);
      }
    } else if (cu == 0 && wave == 0 && lane < K && rt.ent[step * K + lane] < 0) {
      atomicOr(&gf[FLAG_RANGE], 1);
    }
    if (cu == 0 && wave == 0 && lane < K) {
      a.exec_idx[((int64_t)cur * a.L + l) * K + lane] = rt.idx[step * K + lane];
      a.exec_w[((int64_t)cur * a.L + l) * K + lane] = rt.w[step * K + lane];
    }
    stamp(a, l, 3);

    // ---- gate/up items ---------------------------------------------------------
    fl_wait(FL_READY + slot, step + 1, gf);
    stamp(a, l, 6);
    {
      // the lane's activation chunks li + 16 m (pair-permuted fp16)
      f16x2 xr[CPL][16];
#pragma unroll
      for (int m = 0; m < CPL; ++m) load_xchunk(xp, li + kGL * m, xr[m]);
      stamp(a, l, 7);
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) {
        const int jj = grp + kGN * j2;
        bool ok = jj < ipc;  // uniform over the group
        if (ok) ok = it.shared ? (lf & LF_SHARED) != 0 : rt.ent[step * K + (it.b + jj) / I] >= 0;
        float ag = 0.0f, au = 0.0f;
        if (ok) {
          const uint4* gq = reinterpret_cast<const uint4*>(S + p.g_gq + (2 * jj) * (d / 2));
          const uint4* uq = reinterpret_cast<const uint4*>(S + p.g_gq + (2 * jj + 1) * (d / 2));
          const uint16_t* gs = reinterpret_cast<const uint16_t*>(S + p.g_gs + (2 * jj) * (d / 32));
          const uint16_t* us = reinterpret_cast<const uint16_t*>(S + p.g_gs + (2 * jj + 1) * (d / 32));
          float pg[CPL], pu[CPL];
#pragma unroll
          for (int m = 0; m < CPL; ++m) {
            const int c = li + kGL * m;
            pg[m] = h2f(gs[c >> 1]) * q4_dot32_ilp(gq[c], xr[m]);
            pu[m] = h2f(us[c >> 1]) * q4_dot32_ilp(uq[c], xr[m]);
          }
#pragma unroll
          for (int m = 0; m < CPL; ++m) {
            ag += pg[m];
            au += pu[m];
          }
        }
        ag = group_sum<kGL>(ag);
        au = group_sum<kGL>(au);
        if (it.shared) {
          // the shared expert's raw sums, (g, u) in one word: the down CUs
          // add the LoRA terms and take the SwiGLU
          if (li == 0 && jj < ipc) xput2(XB + p.xb_s + ((cu - p.ngr) << p.lhs) + jj, ag, au, tag);
        } else {
          // items 2o and 2o + 1 share word o: the odd group hands its value to
          // the even one 16 lanes below
          const float sv = ok ? silu(ag) * au : 0.0f;
          const float sn = __shfl_xor(sv, kGL, 64);
          if (li == 0 && (grp & 1) == 0 && jj < ipc) xput2(XB + (cu << p.lbr) + (jj >> 1), sv, sn, tag);
        }
      }
      stamp(a, l, 8);
      if (it.shared) {
        if (t >= ipc && t < hs) xput2(XB + p.xb_s + ((cu - p.ngr) << p.lhs) + t, 0.0f, 0.0f, tag);
      } else if (t >= (ipc + 1) / 2 && t < bir) {
        xput2(XB + (cu << p.lbr) + t, 0.0f, 0.0f, tag);
      }
      release(FL_FREED + 4 * slot + wave, step + 1);
    }
    stamp(a, l, 4);

    // ---- head: fc1 and linear-path rows --------------------------------------------
    if (lf & LF_HEAD) {
      fl_wait(FL_HREADY, step + 1, gf);
      const int nh = he - hb;
      for (int rr = wave; rr < nh; rr += kFW) {
        const int hr = hb + rr;
        float acc = wave_row_dot<CPL>(lds_at<uint16_t>(p.g_hb) + rr * d, xn);
        if (lane < 2 * K) {
          const int e = lane < K ? rt.idx[step * K + lane] : rt.prev[step * K + lane - K];
          if (e >= 0 && e < E) {
            const int col = lane < K ? d + e : d + E + e;
            const uint32_t wv = lds_at<uint32_t>(p.g_hc)[rr * 2 * K + lane];
            acc += h2f((uint16_t)((col & 1) ? wv >> 16 : wv & 0xFFFF));
          }
        }
        acc = wave_sum_rows(acc);
        if (lane == 0) xput(X + p.o_xh1 + cu * kBlk + rr, fbits(hr < P ? gelu_erf(acc) : acc), ep);
      }
      if (wave == 0 && lane >= nh && lane < kBlk) xput(X + p.o_xh1 + cu * kBlk + lane, 0u, ep);
      release(FL_HFREED + wave, step + 1);
    }
    stamp(a, l, 5);
  }
}

// ============================================================== down CUs ==

template <int CPL, int KM>
__device__ __attribute__((noinline)) void dn_loader(uint64_t kap, int lw) {
  KA& a = args_at(kap);
  KP& p = a.pl;
  (void)CPL;
  const int K = a.dm.K, r = a.dm.r, I = kFI, P = a.dm.P;
  const int nL = a.l1 - a.l0;
  const int j = blockIdx.x - p.ng;
  const RT rt = rt_at(p.d_rt, nL, K, p);
  const int pb = rt.pb[j], pe = rt.pb[j + 1];
  const int rpc = 2 * (pe - pb);
  const int KX = p.KX;
  int32_t* gf = a.flags;
  if (lw < 2) {
    for (int step = lw; step < nL; step += 2) {
      const int slot = lw;
      const int l = a.l0 + step;
      if (step >= 2) fl_wait_all(FL_FREED + 4 * slot, kFW, step - 1, gf);
      lstamp(a, l, 10 + slot);
      const LayerDev& Ly = a.layers[l];
      const int lf = rt.lf[step];
      unsigned char* S = s_mem + slot * p.d_slot;
      if (lf & LF_ATTN) dma4(S + p.d_at, rpc / 2, [&](int q) { return cptr(Ly.attn) + (int64_t)(pb + q) * 4; });
      // rows of expert slot k: [k][rr][I/2 bytes], scales [k][rr][16 bytes]
      auto exp_dma = [&](int k0, int k1) {
        if (k1 <= k0) return;
        auto qbase = [&](int k, int rr, bool sc) -> const char* {
          const int row = 2 * pb + rr;
          if (k < K) {
            const int ent = rt.ent[step * K + k];
            return sc ? cptr(Ly.pool.down.s) + ent * Ly.pool.stride_s + (int64_t)row * 16
                      : cptr(Ly.pool.down.q) + ent * Ly.pool.stride_q + (int64_t)row * (I / 2);
          }
          return sc ? cptr(Ly.sh.down.s) + (int64_t)row * 16 : cptr(Ly.sh.down.q) + (int64_t)row * (I / 2);
        };
        auto valid = [&](int k) { return k < K ? rt.ent[step * K + k] >= 0 : (lf & LF_SHARED) != 0; };
        constexpr int pq = kFI / 32;  // pieces of a row
        dma16(S + p.d_dq + 16 * (k0 * rpc * pq), (k1 - k0) * rpc * pq,
              [&](int q) {
                const int k = k0 + q / (rpc * pq), rem = q % (rpc * pq);
                return qbase(k, rem / pq, false) + 16 * (rem % pq);
              },
              [&](int q) { return valid(k0 + q / (rpc * pq)); });
        dma16(S + p.d_ds + 16 * (k0 * rpc), (k1 - k0) * rpc,
              [&](int q) { return qbase(k0 + q / rpc, q % rpc, true); },
              [&](int q) { return valid(k0 + q / rpc); });
      };
      if (KX > K) {
        exp_dma(K, KX);
        if (lf & LF_LORAD)
          dma16(S + p.d_bd, rpc * 2,
                [&](int q) { return cptr(Ly.sh.bd) + ((int64_t)(2 * pb + q / 2) * r) * 2 + 16 * (q % 2); },
                [](int) { return true; });
      }
      const bool routed_known = !(lf & LF_ROUTER);
      if (routed_known) exp_dma(0, K);
      dma_drain();
      fl_st(FL_PRE + slot, step + 1);
      if (!routed_known) {
        fl_wait(FL_ROUTE, step + 1, gf);
        lstamp(a, l, 12);
        exp_dma(0, K);
        dma_drain();
      }
      fl_st(FL_READY + slot, step + 1);
      lstamp(a, l, 13);
    }
    return;
  }
  // fc2 rows of each head
  const int fb = rt.fb[j], fe = rt.fb[j + 1];
  int prev = 0;
  for (int step = 0; step < nL; ++step) {
    const int lf = rt.lf[step];
    if (!(lf & LF_HEAD)) continue;
    const LayerDev& Ly = a.layers[a.l0 + step];
    fl_wait_all(FL_HFREED, kFW, prev, gf);
    const int pr = P / 8;
    dma16(s_mem + p.d_f2, (fe - fb) * pr,
          [&](int q) { return cptr(Ly.head.fc2) + ((int64_t)(fb + q / pr) * P) * 2 + 16 * (q % pr); },
          [](int) { return true; });
    dma_drain();
    fl_st(FL_HREADY, step + 1);
    prev = step + 1;
  }
}

// fc2 rows of the head on layer a.l0 + hs, in the wait for a later layer or
// after the last one.
template <int CPL, int KM>
__device__ __attribute__((noinline)) int dn_head_fc2(uint64_t kap, int hs, int phase) {
  KA& a = args_at(kap);
  KP& p = a.pl;
  const Dims dm = dims_of(a.dm);
  const int E = dm.E, P = dm.P;
  const int lh = a.l0 + hs;
  const int j = blockIdx.x - p.ng;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const uint32_t ep = a.epoch;
  int32_t* gf = a.flags;
  uint64_t* X = a.xbuf + (int64_t)lh * p.xlayer;
  float* ab = lds_at<float>(p.d_ab);
  const RT rt = rt_at(p.d_rt, a.l1 - a.l0, dm.K, p);
  xgather_any(X + p.o_xh1, p.ng * kBlk, ep, t, kFC, gf, [&](int wi, uint32_t v) {
    const int c = wi >> 3, o = wi & 7;
    const int hb = rt.hb[c];
    if (o < rt.hb[c + 1] - hb) ab[hb + o] = bitsf(v);
  });
  cbar(phase, gf);
  fl_wait(FL_HREADY, hs + 1, gf);
  const int fb = rt.fb[j], fe = rt.fb[j + 1];
  const uint16_t* f2 = lds_at<uint16_t>(p.d_f2);
  for (int rr = wave; rr < fe - fb; rr += kFW) {
    const int e = fb + rr;
    float acc = 0.0f;
    if (8 * lane < P) {
      const uint4 wv = *reinterpret_cast<const uint4*>(f2 + rr * P + 8 * lane);
      const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
      const float4 a0 = *reinterpret_cast<const float4*>(ab + 8 * lane);
      const float4 a1 = *reinterpret_cast<const float4*>(ab + 8 * lane + 4);
      const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      float a2 = 0.0f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc = fmaf(h2f((uint16_t)(ww[q] & 0xFFFF)), av[2 * q], acc);
        a2 = fmaf(h2f((uint16_t)(ww[q] >> 16)), av[2 * q + 1], a2);
      }
      acc += a2;
    }
    acc = wave_sum_rows(acc);
    const float logit = acc + ab[P + e];
    if (lane == 0) {
      xput(X + p.o_xh2 + j * kBlk + rr, fbits(logit), ep);
      if (a.head_logits) a.head_logits[(int64_t)lh * E + e] = logit;
    }
  }
  if (wave == 0 && lane >= fe - fb && lane < kBlk) xput(X + p.o_xh2 + j * kBlk + lane, 0u, ep);
  release(FL_HFREED + wave, hs + 1);
  return phase;
}

// Ranking of the head on layer lh into the next token's routing of layer
// lh+1 (wave 0 of the designated down CU).
template <int CPL, int KM>
__device__ __attribute__((noinline)) void dn_head_topk(uint64_t kap, int lh) {
  KA& a = args_at(kap);
  KP& p = a.pl;
  const Dims dm = dims_of(a.dm);
  const int K = dm.K;
  const int nxt = (a.token + 1) & 1;
  const uint32_t ep = a.epoch;
  int32_t* gf = a.flags;
  const int lane = threadIdx.x & 63;
  uint64_t* X = a.xbuf + (int64_t)lh * p.xlayer;
  float* lg = lds_at<float>(p.d_lg);
  RouteScratch& rs = *lds_at<RouteScratch>(p.d_rs);
  const RT rt = rt_at(p.d_rt, a.l1 - a.l0, K, p);
  xgather_any(X + p.o_xh2, p.nd * kBlk, ep, lane, 64, gf, [&](int wi, uint32_t v) {
    const int jd = wi >> 3, o = wi & 7;
    const int fb = rt.fb[jd];
    if (o < rt.fb[jd + 1] - fb) lg[fb + o] = bitsf(v);
  });
  wave_lds_sync();
  int32_t* pidx = lh + 1 < a.L ? a.route_idx + ((int64_t)nxt * a.L + lh + 1) * K : a.sink_idx;
  float* pw = lh + 1 < a.L ? a.route_w + ((int64_t)nxt * a.L + lh + 1) * K : a.sink_w;
  route_wave(dm, lg, a.layers[lh].head.bias, rs, pidx, pw, gf);
}

template <int CPL, int KM>
__device__ __attribute__((noinline)) void dn_compute(uint64_t kap) {
  KA& a = args_at(kap);
  KP& p = a.pl;
  constexpr int d = 512 * CPL;
  const Dims dm = dims_of(a.dm);
  const int K = dm.K, E = dm.E, r = dm.r, I = kFI;
  const int nL = a.l1 - a.l0;
  const int j = blockIdx.x - p.ng;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int li = t % kGL, grp = t / kGL;
  const uint32_t ep = a.epoch;
  int32_t* gf = a.flags;
  const RT rt = rt_at(p.d_rt, nL, K, p);
  const int pb = rt.pb[j], pe = rt.pb[j + 1];
  const int npairs = pe - pb, rpc = 2 * npairs;
  const int KX = p.KX, KI = K * I;
  const int Is = KX > K ? I : 0;
  const int ngs = p.ng - p.ngr;
  float* sb = lds_at<float>(p.d_sb);   // SwiGLU outputs [KX][I]; the shared slot first holds raw g
  float* su = lds_at<float>(p.d_su);   // the shared expert's raw u [I]
  float* ax = lds_at<float>(p.d_ax);   // LoRA A products: A_gate x, then A_up x
  uint16_t* hk = lds_at<uint16_t>(p.d_hk);
  float* csc = lds_at<float>(p.d_cs);
  float* vv = lds_at<float>(p.d_v);
  float* coef = lds_at<float>(p.d_co);
  uint16_t* ho = lds_at<uint16_t>(p.d_ho);
  float* lg = lds_at<float>(p.d_lg);
  RouteScratch& rs = *lds_at<RouteScratch>(p.d_rs);
  int phase = 0;

  if (t < rpc) ho[t] = ldg(a.h + 2 * pb + t);

  for (int step = 0; step < nL; ++step) {
    const int l = a.l0 + step;
    const int slot = step & 1;
    const int lf = rt.lf[step];
    const unsigned char* S = s_mem + slot * p.d_slot;
    uint64_t* X = a.xbuf + (int64_t)l * p.xlayer;
    const LayerDev& Ly = a.layers[l];
    stamp(a, l, 0);

    // LoRA matrices of the shared expert, fetched ahead into registers:
    // rows t and t + 256 of B_gate and B_up, and rank t/16's A_down columns
    // 32 (t%16) .. 32 (t%16) + 31
    const bool lora = (lf & LF_SHARED) && (lf & LF_LORA) && Is;
    const bool lorad = (lf & LF_SHARED) && (lf & LF_LORAD) && Is;
    uint4 bgr[2][2], bur[2][2], adr[4];
    if (lora) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bgr[q][h] = ldg(reinterpret_cast<const uint4*>(Ly.sh.bg + (int64_t)(t + 256 * q) * r + 8 * h));
          bur[q][h] = ldg(reinterpret_cast<const uint4*>(Ly.sh.bu + (int64_t)(t + 256 * q) * r + 8 * h));
        }
    }
    if (lorad) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        adr[c] = ldg(reinterpret_cast<const uint4*>(Ly.sh.ad + (int64_t)(t >> 4) * I + 32 * (t & 15) + 8 * c));
    }

    // ---- routing of a router layer: ranked here as well -----------------------
    if ((lf & LF_ROUTER) && wave == 0) {
      xgather_any(X + p.o_xr, p.nrc * kBlk, ep, lane, 64, gf, [&](int wi, uint32_t v) {
        const int c = wi >> 3, o = wi & 7, e = kRouterRows * c + o;
        if (o < kRouterRows && e < E) lg[e] = bitsf(v);
      });
      wave_lds_sync();
      route_wave(dm, lg, Ly.router_bias, rs, rt.idx + step * K, rt.w + step * K, gf);
      wave_lds_sync();
      if (lane < K) rt.ent[step * K + lane] = (int32_t)resolve_entry(Ly.pool, E, rt.idx[step * K + lane]);
      release(FL_ROUTE, step + 1);
    }
    if (wave == 0 && lane < KX) {
      float cv = 0.0f;
      if (lane < K) cv = rt.ent[step * K + lane] >= 0 ? rt.w[step * K + lane] : 0.0f;
      else cv = (lf & LF_SHARED) ? 1.0f : 0.0f;
      coef[lane] = cv;
    }

    // ---- SwiGLU outputs, the shared expert's sums, LoRA A products -------------
    {
      const int lbr = p.lbr, lhs = p.lhs;
      if ((p.direct & 3) == 3) {
        // whole blocks everywhere: routed word w holds items 2w, 2w + 1, shared
        // word w row w
        xgather2<8>(X + p.o_xb, p.xb_n, pk_tag(ep), t, kFC, gf, [&](int wi, float v0, float v1) {
          if (wi < p.xb_s) {
            sb[2 * wi] = v0;
            sb[2 * wi + 1] = v1;
          } else if (wi < p.xb_a) {
            sb[KI + wi - p.xb_s] = v0;
            su[wi - p.xb_s] = v1;
          } else if (((wi - p.xb_a) & 7) == 0) {
            ax[(wi - p.xb_a) >> 3] = v0;
          }
        });
      } else {
        xgather2<8>(X + p.o_xb, p.xb_n, pk_tag(ep), t, kFC, gf, [&](int wi, float v0, float v1) {
          if (wi < p.xb_s) {
            // SwiGLU outputs of items 2o and 2o + 1 of routed CU c
            const int c = wi >> lbr, o = wi & ((1 << lbr) - 1);
            const int b = rt.ibr[c], n = rt.ibr[c + 1] - b;
            if (2 * o < n) sb[b + 2 * o] = v0;
            if (2 * o + 1 < n) sb[b + 2 * o + 1] = v1;
          } else if (wi < p.xb_a) {
            // the shared expert's raw g and u of row o of shared CU c
            const int w2 = wi - p.xb_s, c = w2 >> lhs, o = w2 & ((1 << lhs) - 1);
            const int b = rt.ibs[c];
            if (c < ngs && o < rt.ibs[c + 1] - b) {
              sb[KI + b + o] = v0;
              su[b + o] = v1;
            }
          } else {
            const int w3 = wi - p.xb_a;
            if ((w3 & 7) == 0) ax[w3 >> 3] = v0;
          }
        });
      }
    }
    cbar(phase, gf);
    stamp(a, l, 1);
    // the shared expert: LoRA B terms, then the SwiGLU
    if (Is && (lf & LF_SHARED)) {
      // the A products are the same for every lane: one vector read of all
      // of them, then scalar registers, so the B terms wait on no LDS read
      float axs[2 * kFRank];
      if (lora) {
#pragma unroll
        for (int c = 0; c < 2 * kFRank / 4; ++c) {
          const float4 v = reinterpret_cast<const float4*>(ax)[c];
          axs[4 * c] = v.x;
          axs[4 * c + 1] = v.y;
          axs[4 * c + 2] = v.z;
          axs[4 * c + 3] = v.w;
        }
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int i = t + 256 * q;
        float g = sb[KI + i], u = su[i];
        if (lora) {
          float lg2 = 0.0f, lu2 = 0.0f;
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t gw[4] = {bgr[q][h].x, bgr[q][h].y, bgr[q][h].z, bgr[q][h].w};
            const uint32_t uw[4] = {bur[q][h].x, bur[q][h].y, bur[q][h].z, bur[q][h].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              lg2 = fmaf(h2f((uint16_t)(gw[e] & 0xFFFF)), axs[8 * h + 2 * e], lg2);
              lg2 = fmaf(h2f((uint16_t)(gw[e] >> 16)), axs[8 * h + 2 * e + 1], lg2);
              lu2 = fmaf(h2f((uint16_t)(uw[e] & 0xFFFF)), axs[kFRank + 8 * h + 2 * e], lu2);
              lu2 = fmaf(h2f((uint16_t)(uw[e] >> 16)), axs[kFRank + 8 * h + 2 * e + 1], lu2);
            }
          }
          g = fmaf(dm.lora_scale, lg2, g);
          u = fmaf(dm.lora_scale, lu2, u);
        }
        sb[KI + i] = silu(g) * u;
      }
    }
    cbar(phase, gf);
    stamp(a, l, 14);
    // fp16 hi + lo copies (pair-permuted) with a power-of-two scale per 32 elements
#pragma unroll
    for (int k = 0; k < KM + 1; ++k) {
      if (k < KX) {
        const float2 v = *reinterpret_cast<const float2*>(sb + k * I + 32 * grp + 2 * li);
        const float sc = hilo_pair(v.x, v.y, grp, li, hk + k * 2 * I, I);
        if (li == 0) csc[k * (I / 32) + grp] = sc;
      }
    }
    stamp(a, l, 15);
    // A_down . h_shared: group g takes rank g, lane li its 32 columns
    {
      float part = 0.0f;
      if (lorad) {
        const float* hsv = sb + KI + 32 * li;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t aw[4] = {adr[c].x, adr[c].y, adr[c].z, adr[c].w};
          const float4 h0 = *reinterpret_cast<const float4*>(hsv + 8 * c);
          const float4 h1 = *reinterpret_cast<const float4*>(hsv + 8 * c + 4);
          float p2 = 0.0f;
          part = fmaf(h2f((uint16_t)(aw[0] & 0xFFFF)), h0.x, part);
          p2 = fmaf(h2f((uint16_t)(aw[0] >> 16)), h0.y, p2);
          part = fmaf(h2f((uint16_t)(aw[1] & 0xFFFF)), h0.z, part);
          p2 = fmaf(h2f((uint16_t)(aw[1] >> 16)), h0.w, p2);
          part = fmaf(h2f((uint16_t)(aw[2] & 0xFFFF)), h1.x, part);
          p2 = fmaf(h2f((uint16_t)(aw[2] >> 16)), h1.y, p2);
          part = fmaf(h2f((uint16_t)(aw[3] & 0xFFFF)), h1.z, part);
          p2 = fmaf(h2f((uint16_t)(aw[3] >> 16)), h1.w, p2);
          part += p2;
        }
      }
      part = group_sum<kGL>(part);
      if (li == 0) vv[grp] = part;
    }
    cbar(phase, gf);
    stamp(a, l, 2);

    // ---- down rows: every expert slot, down LoRA, residual -----------------------
    fl_wait(FL_READY + slot, step + 1, gf);
    stamp(a, l, 6);
    if (grp < npairs) {
      const int rr0 = 2 * grp;
      constexpr int pq = kFI / 32;
      float p0[KM + 1], p1[KM + 1];
#pragma unroll
      for (int k = 0; k < KM + 1; ++k) {
        p0[k] = p1[k] = 0.0f;
        // slots past KX, unresolved experts and a missing shared expert carry
        // a zero coefficient (uniform over the CU)
        if (k < KX && coef[k] != 0.0f) {
          f16x2 xh[16], xl[16];
          load_xchunk(hk + k * 2 * I, li, xh);
          load_xchunk(hk + k * 2 * I + I, li, xl);
          const float f = coef[k] * csc[k * (I / 32) + li];
          const uint4* dq = reinterpret_cast<const uint4*>(S + p.d_dq) + (k * rpc + rr0) * pq;
          const uint16_t* ds = reinterpret_cast<const uint16_t*>(S + p.d_ds + 16 * (k * rpc + rr0));
          p0[k] = f * (h2f(ds[li >> 1]) * q4_dot32_hl_ilp(dq[li], xh, xl));
          p1[k] = f * (h2f(ds[8 + (li >> 1)]) * q4_dot32_hl_ilp(dq[pq + li], xh, xl));
        }
      }
      float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
      for (int k = 0; k < KM + 1; ++k) {
        acc0 += p0[k];
        acc1 += p1[k];
      }
      stamp(a, l, 7);
      if (lorad) {
        const uint16_t* bd = reinterpret_cast<const uint16_t*>(S + p.d_bd) + rr0 * r;
        acc0 = fmaf(dm.lora_scale, h2f(bd[li]) * vv[li], acc0);
        acc1 = fmaf(dm.lora_scale, h2f(bd[r + li]) * vv[li], acc1);
      }
      acc0 = group_sum<kGL>(acc0);
      acc1 = group_sum<kGL>(acc1);
      if (li == 0) {
        float a0 = 0.0f, a1 = 0.0f;
        if (lf & LF_ATTN) {
          const uint32_t aw = reinterpret_cast<const uint32_t*>(S + p.d_at)[grp];
          a0 = h2f((uint16_t)(aw & 0xFFFF));
          a1 = h2f((uint16_t)(aw >> 16));
        }
        const uint16_t o0 = f2h((h2f(ho[rr0]) + a0) + acc0);
        const uint16_t o1 = f2h((h2f(ho[rr0 + 1]) + a1) + acc1);
        ho[rr0] = o0;
        ho[rr0 + 1] = o1;
        const int row = 2 * (pb + grp);
        *reinterpret_cast<uint32_t*>(a.h + (int64_t)(step + 1) * d + row) = o0 | ((uint32_t)o1 << 16);
        xput(X + p.o_xa + (j << p.lba) + grp, o0 | ((uint32_t)o1 << 16), ep);
      }
    }
    stamp(a, l, 8);
    if (t >= npairs && t < (1 << p.lba)) xput(X + p.o_xa + (j << p.lba) + t, 0u, ep);
    release(FL_FREED + 4 * slot + wave, step + 1);
    stamp(a, l, 3);

    // ---- heads in the wait for the next layer ----------------------------------
    if (step >= 1 && (rt.lf[step - 1] & LF_HEAD)) phase = dn_head_fc2<CPL, KM>(kap, step - 1, phase);
    stamp(a, l, 4);
    if (step >= 2 && (rt.lf[step - 2] & LF_HEAD) && (l - 2) % p.nd == j && wave == 0)
      dn_head_topk<CPL, KM>(kap, l - 2);
    stamp(a, l, 5);
  }
  if (nL >= 1 && (rt.lf[nL - 1] & LF_HEAD)) phase = dn_head_fc2<CPL, KM>(kap, nL - 1, phase);
  for (int hs = (nL >= 2 ? nL - 2 : 0); hs < nL; ++hs)
    if ((rt.lf[hs] & LF_HEAD) && (a.l0 + hs) % p.nd == j && wave == 0)
      dn_head_topk<CPL, KM>(kap, a.l0 + hs);
  stamp(a, a.L, 0);
}

template <int CPL, int KM>
__global__ __launch_bounds__(kFThreads) void k_flow(FlowArgs a) {
  const FlowPlan& p = a.pl;
  const int K = a.dm.K, E = a.dm.E;
  const int nL = a.l1 - a.l0;
  const bool gu = (int)blockIdx.x < p.ng;
  const int cur = a.token & 1, nxt = (a.token + 1) & 1;
  const int t = threadIdx.x;
  if (t < FL_N) s_fl[t] = 0;
  // routing tables of the launch, per-step layer flags, the work split
  const RT rt = rt_at(gu ? p.g_rt : p.d_rt, nL, K, p);
  for (int i = t; i < nL * K; i += kFThreads) {
    const int l = a.l0 + i / K, k = i % K;
    const LayerDev& Ly = a.layers[l];
    const int e = a.route_idx[((int64_t)cur * a.L + l) * K + k];
    rt.idx[i] = e;
    rt.w[i] = a.route_w[((int64_t)cur * a.L + l) * K + k];
    rt.prev[i] = a.token > 0 ? a.exec_idx[((int64_t)nxt * a.L + l) * K + k] : -1;
    rt.ent[i] = Ly.router ? -1 : (int32_t)resolve_entry(Ly.pool, E, e);
  }
  const int ngs = p.ng - p.ngr;
  for (int i = t; i <= p.ngr; i += kFThreads) rt.ibr[i] = share_b(K * kFI, p.ngr, i);
  for (int i = t; i <= ngs; i += kFThreads) rt.ibs[i] = ngs ? share_b(a.dm.Is, ngs, i) : 0;
  for (int i = t; i <= p.ng; i += kFThreads) rt.hb[i] = share_b(p.hrn, p.ng, i);
  for (int i = t; i <= p.nd; i += kFThreads) {
    rt.pb[i] = share_b(a.dm.d / 2, p.nd, i);
    rt.fb[i] = share_b(E, p.nd, i);
  }
  for (int s = t; s < nL; s += kFThreads) {
    const LayerDev& Ly = a.layers[a.l0 + s];
    int lf = 0;
    if (Ly.router) lf |= LF_ROUTER;
    if (Ly.head.fc1) lf |= LF_HEAD;
    if (Ly.sh.present) lf |= LF_SHARED;
    if (Ly.sh.present && Ly.sh.ag) lf |= LF_LORA;
    if (Ly.sh.present && Ly.sh.ad) lf |= LF_LORAD;
    if (Ly.attn) lf |= LF_ATTN;
    rt.lf[s] = lf;
  }
  __syncthreads();
  const int w = t >> 6;
  const uint64_t kap = (uint64_t)__builtin_amdgcn_kernarg_segment_ptr();
  if (w >= kFW) {
    if (gu) gu_loader<CPL, KM>(kap, w - kFW);
    else dn_loader<CPL, KM>(kap, w - kFW);
    dma_drain();
    return;
  }
  if (gu) gu_compute<CPL, KM>(kap);
  else dn_compute<CPL, KM>(kap);
}

template <int CPL, int KM>
hipError_t launch_flow_t(const FlowArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((k_flow<CPL, KM>), dim3(a.pl.ng + a.pl.nd), dim3(kFThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

// ------------------------------------------------------------------ plan --

static int rup16(int x) { return (x + 15) & ~15; }
static int cdiv(int a, int b) { return (a + b - 1) / b; }
static int log2ceil(int x, int lo) {
  int l = lo;
  while ((1 << l) < x) ++l;
  return l;
}

bool flow_supported(const Dims& dm) {
  if (dm.affine) return false;
  if (dm.d != 1536 && dm.d != 2048) return false;
  if (dm.I != kFI || dm.G != 64 || dm.K < 1 || dm.K > 8 || dm.E > 256 || dm.E < dm.K) return false;
  if (dm.Is != 0 && dm.Is != kFI) return false;
  if (dm.r != 0 && dm.r != kFRank) return false;
  if (dm.P < 64 || dm.P > 512 || dm.P % 64) return false;
  return true;
}

static FlowPlan flow_plan_t(const Dims& dm, int ng, int nd, int nL, bool snap) {
  FlowPlan p{};
  p.ok = 0;
  if (!flow_supported(dm) || ng < 2 || nd < 1 || nL < 1 || nL > kFMaxL) return p;
  const int d = dm.d, K = dm.K, E = dm.E, I = dm.I, r = dm.r, P = dm.P, Is = dm.Is;
  const int KI = K * I;
  p.ng = ng;
  p.nd = nd;
  p.KX = K + (Is ? 1 : 0);
  // routed and shared gate/up CUs in proportion to their items
  p.ngr = ng;
  if (Is) {
    p.ngr = (int)(((int64_t)ng * KI + (KI + Is) / 2) / (KI + Is));
    if (p.ngr > ng - 1) p.ngr = ng - 1;
    if (p.ngr < 1) p.ngr = 1;
  }
  {
    // a power-of-two share of routed items per CU (16 or more: whole 64-byte
    // blocks of two items a word) lets the down CUs store the exchange
    // words straight into place; taken when it keeps at least 80% of the CUs
    int ipr = 2;
    while (ipr * p.ngr < KI) ipr *= 2;
    if (snap && ipr >= 16 && KI % ipr == 0 && 5 * (KI / ipr) >= 4 * p.ngr) p.ngr = KI / ipr;
  }
  const int ngs = ng - p.ngr;
  p.ipr_max = cdiv(KI, p.ngr);
  p.ips_max = Is ? cdiv(Is, ngs) : 0;
  p.ipc_max = p.ipr_max > p.ips_max ? p.ipr_max : p.ips_max;
  p.lbr = log2ceil(cdiv(p.ipr_max, 2), 3);  // two items a word
  p.lhs = log2ceil(p.ips_max, 3);            // (g, u) of one row a word
  p.pairs_max = cdiv(d / 2, nd);
  p.lba = log2ceil(p.pairs_max, 3);
  p.nrc = cdiv(E, kRouterRows);
  // the LoRA A rows go to the shared CUs when there are enough of them
  p.ca0 = (Is && ngs >= 2 * r) ? p.ngr : p.nrc;
  p.hrn = P + E;
  p.hr_max = cdiv(p.hrn, ng);
  p.f2_max = cdiv(E, nd);
  if (p.ipc_max > 2 * kGN || p.pairs_max > kGN || p.hr_max > kBlk || p.f2_max > kBlk) return p;
  if (p.ngr < p.nrc || (p.ca0 == p.nrc && p.ngr < p.nrc + 2 * r)) return p;
  p.direct = 0;
  if (p.ipr_max == (2 << p.lbr) && KI == p.ngr * p.ipr_max) p.direct |= 1;
  if (!Is || Is == (ngs << p.lhs)) p.direct |= 2;
  if (d / 2 == (nd << p.lba)) p.direct |= 4;
  // exchange words of a layer (every region starts on a 128-byte line)
  int o = 0;
  auto region = [&](int n) {
    const int at = o;
    o += (n + 15) & ~15;
    return at;
  };
  p.o_xa = region(nd << p.lba);
  p.xb_s = p.ngr << p.lbr;
  p.xb_a = p.xb_s + (Is ? ngs << p.lhs : 0);
  p.xb_n = p.xb_a + 2 * r * kBlk;
  p.o_xb = region(p.xb_n);
  p.o_xr = region(p.nrc * kBlk);
  p.o_xh1 = region(ng * kBlk);
  p.o_xh2 = region(nd * kBlk);
  p.xlayer = o;
  // routing tables, layer flags and split tables
  const int rtb = nL * K * 16 + nL * 4 + (p.ngr + 1 + ngs + 1 + nd + 1 + ng + 1 + nd + 1) * 4;
  // gate/up CU LDS
  {
    const int ipc = p.ipc_max;
    int s = 0;
    p.g_at = s; s = rup16(s + d * 2);
    p.g_gq = s; s = rup16(s + ipc * 2 * (d / 2));
    p.g_gs = s; s = rup16(s + ipc * 2 * (d / 32));
    p.g_ar = s; s = rup16(s + d * 2);
    p.g_slot = s;
    int off = 2 * s;
    p.g_rb = off; off = rup16(off + kRouterRows * d * 2);
    p.g_hb = off; off = rup16(off + p.hr_max * d * 2);
    p.g_hc = off; off = rup16(off + p.hr_max * 2 * K * 4);
    p.g_h = off; off = rup16(off + d * 2);
    p.g_xn = off; off = rup16(off + d * 2);
    p.g_xp = off; off = rup16(off + d * 2);
    p.g_lg = off; off = rup16(off + E * 4);
    p.g_rs = off; off = rup16(off + (int)sizeof(RouteScratch));
    p.g_rt = off; off = rup16(off + rtb);
    p.g_end = off;
  }
  // down CU LDS
  {
    const int rpc = 2 * p.pairs_max, KX = p.KX;
    int s = 0;
    p.d_dq = s; s = rup16(s + KX * rpc * (I / 2));
    p.d_ds = s; s = rup16(s + KX * rpc * 16);
    p.d_bd = s; s = rup16(s + rpc * r * 2);
    p.d_at = s; s = rup16(s + p.pairs_max * 4);
    p.d_slot = s;
    int off = 2 * s;
    p.d_f2 = off; off = rup16(off + p.f2_max * P * 2);
    p.d_sb = off; off = rup16(off + KX * I * 4);
    p.d_su = off; off = rup16(off + I * 4);
    p.d_ax = off; off = rup16(off + 2 * kFRank * 4);
    p.d_hk = off; off = rup16(off + KX * 2 * I * 2);
    p.d_cs = off; off = rup16(off + KX * (I / 32) * 4);
    p.d_v = off; off = rup16(off + kGN * 4);
    p.d_co = off; off = rup16(off + 16 * 4);
    p.d_ho = off; off = rup16(off + rpc * 2);
    p.d_ab = off; off = rup16(off + (P + E) * 4);
    p.d_lg = off; off = rup16(off + E * 4);
    p.d_rs = off; off = rup16(off + (int)sizeof(RouteScratch));
    p.d_rt = off; off = rup16(off + rtb);
    p.d_end = off;
  }
  if (p.g_end > kFlowLds || p.d_end > kFlowLds) return p;
  p.ok = 1;
  return p;
}

FlowPlan flow_plan(const Dims& dm, int ng, int nd, int nL) {
  const FlowPlan p = flow_plan_t(dm, ng, nd, nL, true);
  return p.ok ? p : flow_plan_t(dm, ng, nd, nL, false);
}

// Default split of `grid` CUs: as many down CUs as it takes to give each at
// most 16 row pairs and a layer slot that fits, the rest gate/up.
bool flow_default_roles(const Dims& dm, int grid, int nL, int& ng, int& nd) {
  if (!flow_supported(dm)) return false;
  const int pairs = dm.d / 2;
  for (int cand_nd = cdiv(pairs, kGN); cand_nd < grid; ++cand_nd) {
    const int cand_ng = grid - cand_nd;
    const FlowPlan p = flow_plan(dm, cand_ng, cand_nd, nL);
    if (p.ok) {
      ng = cand_ng;
      nd = cand_nd;
      return true;
    }
  }
  return false;
}

namespace {
__global__ __launch_bounds__(256) void k_fill0(uint64_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    p[i] = 0;
}
}  // namespace

// Zero n exchange words (a plain kernel, so a captured stream records no memset).
hipError_t launch_flow_clear(uint64_t* words, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(k_fill0, dim3((unsigned)blocks), dim3(256), 0, st, words, n);
  return hipGetLastError();
}

hipError_t launch_flow(const FlowArgs& a, hipStream_t st) {
  if (!a.pl.ok) return hipErrorInvalidValue;
  const int cpl = a.dm.d / 512;
  if (a.dm.K <= 4) {
    if (cpl == 4) return launch_flow_t<4, 4>(a, st);
    if (cpl == 3) return launch_flow_t<3, 4>(a, st);
  } else {
    if (cpl == 4) return launch_flow_t<4, 8>(a, st);
    if (cpl == 3) return launch_flow_t<3, 8>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace smd
