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
//   3. gate/up rows of the routed experts and the shared expert spread over
//      the chip; the LoRA A products of the shared gate/up (published right
//      after the norm) let the owners of shared rows add the LoRA B terms, so
//      every gate/up row leaves its owner as a finished SwiGLU output;
//   4. every workgroup gathers the SwiGLU outputs and forms the shared
//      expert's down-LoRA A product itself;
//   5. down rows with the weighted combine, shared expert and down LoRA;
//      h_{l+1} = fp16(h_a + y) is published.
// The prerouter heads are not on this chain: a head's output is consumed by
// the next token only. Each workgroup keeps x_l of the few head layers whose
// rows it owns; after the last layer every workgroup streams its share of
// all heads' fc1 and linear-path rows, then of their fc2 rows, and the
// routing of each head's logits writes the next token's prediction.
//
// Cross-workgroup data moves as 8-byte words (32-bit payload, 32-bit epoch)
// written and polled with agent-scope relaxed atomics (coherent across the
// XCDs' L2s without cache write-back or invalidation): an aligned 8-byte
// access is single-copy atomic, so a word carrying the current launch's epoch
// carries that launch's payload, and a consumer polls the words themselves
// (no separate arrival flag, so one fabric round trip per exchange). Buffers
// are per layer, so no word is written twice in one launch. Every wait is
// bounded by a wall-clock limit; on expiry the kernel raises FLAG_SYNC and
// runs to completion.

#include "gemv.h"
#include "internal.h"

namespace smd {

namespace {

constexpr int kThreads = 256;
constexpr int kLG = 16;
constexpr int kGroups = kThreads / kLG;
constexpr uint64_t kSpinLimit = 20000000ull;  // 0.2 s of the 100 MHz wall clock
constexpr int kMaxL = 64;      // layers per launch (routing tables in LDS)
constexpr int kNR = 4;         // fp16 rows per workgroup per block job (router, LoRA A)
constexpr int kMaxExp = 9;     // experts per down row: K <= 8 routed + the shared expert
constexpr int kEp = 9;         // base addresses per expert slot (q, s, b of gate, up, down)
constexpr int kRank = 16;      // LoRA rank of this kernel (or no LoRA at all)
static_assert(kRank == 16, "one lane group per rank of the down LoRA A product");
constexpr int kStackI = 512;   // expert intermediate width of this kernel
constexpr int kHX = 4;         // head layers one workgroup keeps x / fc2 activations of
constexpr int kF2R = 4;        // fc2 rounds (kGroups rows each) per workgroup
constexpr int kCPF = 4;        // 16-byte chunks per lane of an fc2 row (P <= 512)

// Stand-in row for loads whose row does not exist (an unresolved expert, an
// item past the workgroup's share, a layer without that matrix): every load of
// the layer loop is issued unconditionally, from its row or from here, so that
// each lands in the register it is consumed from. A conditional load merged
// with a default value makes the compiler copy the register at the merge,
// which waits for the load there instead of where the value is used. Never
// written; 8 KB covers every such load (offsets < d * 2 bytes, d <= 2048).
__device__ __align__(16) uint32_t g_zrow[2048];

// The row's address is made opaque to the compiler, which could otherwise
// fold the loads to zeros and turn them back into conditional loads.
__device__ __forceinline__ const void* zrow() {
  const void* p = g_zrow;
  asm("" : "+s"(p));
  return p;
}

// p when v, else the zero row. The choice is hidden from the compiler too, so
// that it cannot split the load into two conditional ones.
template <typename T>
__device__ __forceinline__ const T* pick(bool v, const T* p) {
  const T* q = v ? p : (const T*)zrow();
  asm("" : "+v"(q));
  return q;
}

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
__device__ __forceinline__ void ll_gather(const uint64_t* src, int n, uint32_t ep, uint32_t* dst,
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

// ll_gather with 16-byte polls: two words per load, U loads per thread in
// flight (agent-scope buffer loads, so a poll is one request for both
// words). src 16-byte aligned and n even; otherwise the 8-byte gather.
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
// PAD: word i goes to dst[pad32(i)] (four words of padding after every 32),
// so 16-lane groups reading 32 consecutive words per lane hit distinct banks.
// The padded gather has no 8-byte fallback: its callers pass an even n and a
// 16-byte aligned src (the SwiGLU outputs: I == 512, even exchange rows).
__device__ __forceinline__ int pad32(int i) { return i + 4 * (i >> 5); }

template <int U, bool PAD = false>
__device__ __forceinline__ void ll_gather2(const uint64_t* src, int n, uint32_t ep, uint32_t* dst,
                                           int32_t* flags, int* abort_lds) {
  if (!PAD && ((n & 1) || (reinterpret_cast<uintptr_t>(src) & 15))) {
    ll_gather<2 * U>(src, n, ep, dst, flags, abort_lds);
    return;
  }
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, n * 8, 0x00020000);
  const uint64_t t0 = wall_clock64();
  uint32_t polls = 0;
  const int np = n >> 1;
  for (int b0 = 0; b0 < np; b0 += U * kThreads) {
    u32x4v v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int p = b0 + j * kThreads + (int)threadIdx.x;
      v[j] = p < np ? __builtin_amdgcn_raw_buffer_load_b128(rs, p * 16, 0, 16)
                    : (u32x4v){0u, ep, 0u, ep};
    }
    for (;;) {
      bool ok = true;
#pragma unroll
      for (int j = 0; j < U; ++j) ok = ok && v[j].y == ep && v[j].w == ep;
      if (ok) break;
      if (wait_expired(t0, flags, abort_lds, polls)) break;
      __builtin_amdgcn_s_sleep(1);
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const int p = b0 + j * kThreads + (int)threadIdx.x;
        if (p < np && (v[j].y != ep || v[j].w != ep))
          v[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, p * 16, 0, 16);
      }
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int p = b0 + j * kThreads + (int)threadIdx.x;
      if (p < np) {
        const int i = PAD ? pad32(2 * p) : 2 * p;
        dst[i] = v[j].x;
        dst[i + 1] = v[j].z;
      }
    }
  }
}

// Phase timestamp of this workgroup (thread 0) when tracing is on. Rows
// 0..L-1 are layers, row L the head phase after the last layer.
__device__ __forceinline__ void stamp(const StackArgs& a, int row, int k) {
  if (a.trace && threadIdx.x == 0)
    a.trace[((int64_t)blockIdx.x * (a.L + 1) + row) * kTracePoints + k] = wall_clock64();
}

// Wait for every outstanding vector memory operation. Placed only where all
// of them are already known to be complete (their results were consumed),
// so it costs nothing; it keeps the compiler's conservative tracking of
// possibly pending loads across the layer loop from adding a wait later at a
// point where exchange stores or prefetches are in flight (vector memory
// operations retire in order, so such a wait would stall on all of them).
__device__ __forceinline__ void vm_drained() { __builtin_amdgcn_s_waitcnt(0x0F70); }


// A struct of 8-byte fields from global memory by vector loads (per-lane
// addresses allowed).
template <typename T>
__device__ __forceinline__ T ldg_struct(const T* p) {
  static_assert(sizeof(T) % 8 == 0, "struct size");
  const uint64_t* w = reinterpret_cast<const uint64_t*>(p);
  uint64_t buf[sizeof(T) / 8];
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 8); ++i) buf[i] = ldg(w + i);
  return __builtin_bit_cast(T, buf);
}

// Contiguous share [beg, end) of n items for workgroup c of G (n * G < 2^32).
__device__ __forceinline__ void split(int n, int G, int c, int& beg, int& end) {
  beg = (int)((uint32_t)n * (uint32_t)c / (uint32_t)G);
  end = (int)((uint32_t)n * (uint32_t)(c + 1) / (uint32_t)G);
}

// LoRA A rows of workgroup c: one each on the first r2 workgroups (whose
// SwiGLU items are routed ones, so no shared-expert owner computes them), or
// spread over all G when G < r2.
__device__ __forceinline__ void ax_share(int r2, int G, int c, int& beg, int& end) {
  if (G >= r2) {
    beg = c < r2 ? c : r2;
    end = c < r2 ? c + 1 : r2;
  } else {
    split(r2, G, c, beg, end);
  }
}

// Router rows of workgroup c: kNR each on the first E / kNR workgroups, so
// the logits exchange waits on fewer producers (stack_launchable requires
// E <= kNR * G).
__device__ __forceinline__ void router_share(int E, int G, int c, int& beg, int& end) {
  const int np = (E + kNR - 1) / kNR;
  beg = c < np ? kNR * c : E;
  end = c < np ? min(kNR * c + kNR, E) : E;
  if (np > G) split(E, G, c, beg, end);
}

// Block-wide sum (all threads return the total).
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum_rows(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return (red[0] + red[1]) + (red[2] + red[3]);
}

// Small per-layer values kept in LDS.
struct Misc {
  // down-projection bases and combine weight of expert slot k (routed k < K,
  // shared k == K); null / 0 when the slot is unused or its id did not resolve
  const uint32_t* dq[kMaxExp];
  const uint16_t* dsc[kMaxExp];
  float coef[16];
  float ad[kRank];             // A_down . h_shared
  float axgu[2 * kRank];       // A_gate x then A_up x (rows of the shared expert)
  // base addresses of a layer's experts (slot k < K routed, k == K shared;
  // null when unused or unresolved): gate q, up q, down q, gate s, up s,
  // down s, then (affine codec) gate b, up b, down b. Two sets by layer
  // parity: the next layer's is written while the current one is read.
  const void* eptr[2][kMaxExp][kEp];
  // affine codec: sums of the normed x over each 32-element chunk (the
  // gate/up bias terms b * sum)
  float xsum[64];
  float hsc[kHX][16];          // scales of the fc2 activation chunks (per lane)
  float red[4 * kNR];
  float rows[kNR];             // results of the block fp16 row jobs
  int abort;
  int n_heads;
  uint16_t hstage[512];        // h_out rows of this workgroup (<= 512)
  int32_t hl_list[kMaxL];      // layer of head h (launch order)
  const uint16_t* hfc1[kMaxL];  // weights of head h
  const uint16_t* hlin[kMaxL];
  const uint16_t* hfc2[kMaxL];
  const float* hbias[kMaxL];
  int32_t hidx_of[kMaxL];      // head index of layer step s, or -1
  int32_t ridx_all[kMaxL * 8];
  float rw_all[kMaxL * 8];
  int32_t pidx_all[kMaxL * 8];
  int64_t ent_all[kMaxL * 8];
  RouteScratch rs;
};

struct Lds {
  // byte offsets into dynamic LDS
  int hattn, xperm, xnat, land, ha, hx, misc, lay;
  int bytes;
};

// nl: layers of the launch; their device-table entries are copied to LDS so
// that no pointer of the table is read from global memory inside the layer
// loop (such a read would wait on every load issued before it).
__host__ __device__ inline Lds lds_layout(const Dims& dm, int ng, int nl) {
  auto up = [](int b) { return (b + 15) & ~15; };
  Lds o;
  int off = 0;
  o.hattn = off; off += up(dm.d * 4);
  o.xperm = off; off += up(dm.d * 2);
  o.xnat = off; off += up(dm.d * 2);
  int land = ng + ng / 8;  // the SwiGLU outputs land padded (pad32)
  if (dm.d / 2 > land) land = dm.d / 2;
  if (dm.E > land) land = dm.E;
  if (kHX * (dm.P + dm.E) > land) land = kHX * (dm.P + dm.E);
  o.land = off; off += up(land * 4);
  o.ha = off; off += up(kHX * 2 * dm.P * 2);
  o.hx = off; off += up(kHX * dm.d * 2);
  o.misc = off; off += up((int)sizeof(Misc));
  o.lay = off; off += up(nl * (int)sizeof(LayerDev));
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
    R.w[j] = ldg(pick(j < nr && t < cols / 8, reinterpret_cast<const uint4*>(rp[j] + 8 * t)));
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
    if (j < nr) p[j] = wave_sum_rows(p[j]);
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

// Base addresses of expert slot k of a layer into ep[k] (see Misc::eptr);
// ent: the slot's pool entry (routed slots, k < K).
// Biases (affine codec) sit at the scales' entry offsets: stride_s apart.
__device__ __forceinline__ void fill_slot(const void* (&ep)[kEp], const LayerDev& Ly, int K, int k,
                                          int64_t ent) {
  const void* p[kEp] = {nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, nullptr, nullptr, nullptr};
  if (k < K && ent >= 0) {
    p[0] = entry_ptr(Ly.pool.gate.q, ent, Ly.pool.stride_q);
    p[1] = entry_ptr(Ly.pool.up.q, ent, Ly.pool.stride_q);
    p[2] = entry_ptr(Ly.pool.down.q, ent, Ly.pool.stride_q);
    p[3] = entry_ptr(Ly.pool.gate.s, ent, Ly.pool.stride_s);
    p[4] = entry_ptr(Ly.pool.up.s, ent, Ly.pool.stride_s);
    p[5] = entry_ptr(Ly.pool.down.s, ent, Ly.pool.stride_s);
    if (Ly.pool.gate.b) {
      p[6] = entry_ptr(Ly.pool.gate.b, ent, Ly.pool.stride_s);
      p[7] = entry_ptr(Ly.pool.up.b, ent, Ly.pool.stride_s);
      p[8] = entry_ptr(Ly.pool.down.b, ent, Ly.pool.stride_s);
    }
  } else if (k == K && Ly.sh.present) {
    p[0] = Ly.sh.gate.q;
    p[1] = Ly.sh.up.q;
    p[2] = Ly.sh.down.q;
    p[3] = Ly.sh.gate.s;
    p[4] = Ly.sh.up.s;
    p[5] = Ly.sh.down.s;
    p[6] = Ly.sh.gate.b;
    p[7] = Ly.sh.up.b;
    p[8] = Ly.sh.down.b;
  }
#pragma unroll
  for (int i = 0; i < kEp; ++i) ep[i] = p[i];
}

// ---- gate/up items of one lane group (IPG items per group) ---------------
template <int CPL, int IPG>
struct GuRegs {
  uint4 wg[IPG][CPL], wu[IPG][CPL];
  // group scales of the item's row, two per lane (lane li: scales 2li, 2li+1;
  // a row has d/G <= 32 of them); a chunk's scale is fetched from its lane
  uint32_t sg[IPG], su[IPG];
  uint32_t bg[IPG], bu[IPG];  // affine codec: the group biases, packed like the scales
  uint16_t lbg[IPG], lbu[IPG];  // shared items: element li of the row of LoRA B_gate / B_up
};

struct GuPlan {
  int ib, ie;  // item range of this workgroup
};

// Gate/up rows of the group's items, addressed through the layer's slot
// table ep (LDS); items of unresolved routed slots are skipped.
template <int CPL, int IPG, bool AFF>
__device__ __forceinline__ void gu_issue(GuRegs<CPL, IPG>& R, const LayerDev& Ly, const Dims& dm,
                                         const void* const (*ep)[kEp], int n_rt, const GuPlan& pl,
                                         int grp, int li, bool known) {
#pragma unroll
  for (int j = 0; j < IPG; ++j) {
    // every load is issued; a missing row reads the zero row (see zrow)
    const int it = pl.ib + grp + kGroups * j;
    const bool routed = it < n_rt;
    const int k = it >= pl.ie ? 0 : routed ? it / kStackI : dm.K;
    const int row = it >= pl.ie ? 0 : routed ? it % kStackI : it - n_rt;
    const uint32_t* gq = (const uint32_t*)ep[k][0];
    const bool v = known && it < pl.ie && gq != nullptr;
    const uint32_t* uq = (const uint32_t*)ep[k][1];
    const uint16_t* gs = (const uint16_t*)ep[k][3];
    const uint16_t* us = (const uint16_t*)ep[k][4];
    const bool lb = v && !routed && Ly.sh.ag != nullptr;
    R.lbg[j] = ldg(pick(lb, Ly.sh.bg + (int64_t)row * kRank + li));
    R.lbu[j] = ldg(pick(lb, Ly.sh.bu + (int64_t)row * kRank + li));
    const int gsh = __builtin_ctz(dm.G);  // G is a power of two
    const int wpr = dm.d / 8, spr = dm.d >> gsh;
#pragma unroll
    for (int c2 = 0; c2 < CPL; ++c2) {
      const int c = li + kLG * c2;
      R.wg[j][c2] = ldg(pick(v, reinterpret_cast<const uint4*>(gq + (int64_t)row * wpr + 4 * c)));
      R.wu[j][c2] = ldg(pick(v, reinterpret_cast<const uint4*>(uq + (int64_t)row * wpr + 4 * c)));
    }
    // spr is even and rows start 4-byte aligned: one 4-byte load per lane
    const bool vs = v && 2 * li < spr;
    R.sg[j] = ldg(pick(vs, reinterpret_cast<const uint32_t*>(gs + (int64_t)row * spr) + li));
    R.su[j] = ldg(pick(vs, reinterpret_cast<const uint32_t*>(us + (int64_t)row * spr) + li));
    if (AFF) {
      const uint16_t* gb = (const uint16_t*)ep[k][6];
      const uint16_t* ub = (const uint16_t*)ep[k][7];
      R.bg[j] = ldg(pick(vs, reinterpret_cast<const uint32_t*>(gb + (int64_t)row * spr) + li));
      R.bu[j] = ldg(pick(vs, reinterpret_cast<const uint32_t*>(ub + (int64_t)row * spr) + li));
    }
  }
}

// Gate and up dot products of the group's items. Routed items publish
// silu(g) u at once; a shared item's sums are returned in sg_out / su_out
// for gu_finish_shared (its LoRA terms need the layer's A products).
// Scale (32 c) >> gsh of a row whose scales the lane group holds two per
// lane (the group's lanes are active together).
// BF16: the packed values are bf16 (affine codec) rather than fp16.
template <bool BF16 = false>
__device__ __forceinline__ float row_scale(uint32_t packed, int c, int gsh) {
  const int idx = (32 * c) >> gsh;
  const int base = (int)(threadIdx.x & 63) & ~(kLG - 1);
  const uint32_t v = (uint32_t)__shfl((int)packed, base + (idx >> 1));
  const uint16_t b = (uint16_t)((idx & 1) ? v >> 16 : v & 0xFFFFu);
  return BF16 ? bf2f(b) : h2f(b);
}

// AFF: affine items add b * (sum of the chunk's x), xsum per 32 elements.
template <int CPL, int IPG, bool AFF>
__device__ __forceinline__ void gu_finish(const GuRegs<CPL, IPG>& R, const int64_t* ent_k,
                                          int n_rt, const GuPlan& pl, int grp, int li, int gsh,
                                          const uint16_t* xperm, const float* xsum, uint64_t* xg,
                                          uint32_t ep, float (&sg_out)[IPG], float (&su_out)[IPG]) {
#pragma unroll
  for (int j = 0; j < IPG; ++j) {
    const int it = pl.ib + grp + kGroups * j;
    if (it >= pl.ie) continue;  // uniform over the lane group
    const bool routed = it < n_rt;
    const bool ok = !routed || ent_k[it / kStackI] >= 0;
    float ag = 0.0f, au = 0.0f;
    if (ok) {
#pragma unroll
      for (int c2 = 0; c2 < CPL; ++c2) {
        f16x2 xr[16];
        load_xchunk(xperm, li + kLG * c2, xr);
        const int c = li + kLG * c2;
        if (AFF) {
          const float xs = xsum[c];
          ag += row_scale<true>(R.sg[j], c, gsh) * q4_dot32<true>(R.wg[j][c2], xr) +
                row_scale<true>(R.bg[j], c, gsh) * xs;
          au += row_scale<true>(R.su[j], c, gsh) * q4_dot32<true>(R.wu[j][c2], xr) +
                row_scale<true>(R.bu[j], c, gsh) * xs;
        } else {
          ag += row_scale(R.sg[j], c, gsh) * q4_dot32(R.wg[j][c2], xr);
          au += row_scale(R.su[j], c, gsh) * q4_dot32(R.wu[j][c2], xr);
        }
      }
    }
    ag = group_sum<kLG>(ag);
    au = group_sum<kLG>(au);
    sg_out[j] = ag;
    su_out[j] = au;
    if (routed && li == 0) ll_put(xg + it, fbits(ok ? silu(ag) * au : 0.0f), ep);
  }
}

// Shared items: g += c B_gate[row] . (A_gate x), u likewise (lane li takes
// rank li; axgu holds the r gate then r up A products, or null without
// LoRA), then silu(g) u is published after the routed outputs.
template <int CPL, int IPG>
__device__ __forceinline__ void gu_finish_shared(const GuRegs<CPL, IPG>& R, float cl, int n_rt,
                                                 const GuPlan& pl, int grp, int li,
                                                 const float* axgu, const float (&sg_in)[IPG],
                                                 const float (&su_in)[IPG], uint64_t* xg,
                                                 uint32_t ep) {
#pragma unroll
  for (int j = 0; j < IPG; ++j) {
    const int it = pl.ib + grp + kGroups * j;
    if (it >= pl.ie || it < n_rt) continue;  // uniform over the lane group
    float g = sg_in[j], u = su_in[j];
    if (axgu) {
      const float lg = group_sum<kLG>(h2f(R.lbg[j]) * axgu[li]);
      const float lu = group_sum<kLG>(h2f(R.lbu[j]) * axgu[kRank + li]);
      g = fmaf(cl, lg, g);
      u = fmaf(cl, lu, u);
    }
    if (li == 0) ll_put(xg + it, fbits(silu(g) * u), ep);
  }
}

// ---- down rows: every expert's chunk of one row per lane group ------------
template <int NX>
struct DownRegs {
  uint4 w[NX];
  uint16_t s[NX];
  uint16_t b[NX];  // affine codec: the chunk's group bias
  uint4 bd[kRank / 8];  // LoRA B of the down projection, row drow (lane 0 of the group)
};

// Shared-expert LoRA A_down ([r, Is]): lane group g takes rank g (kRank ==
// kGroups), lane li its columns 32 li .. 32 li + 31 (Is == 16 * 32).
struct LoraRegs {
  uint4 ad[4];
};

// Loads of a layer issued ahead of its activations: router and LoRA A rows,
// attention update, and, once the routing is known, gate/up rows (phase A)
// and down rows with the shared-expert LoRA matrices (phase B).
template <int CPL, int IPG, int NX>
struct PhaseA {
  F16Rows<kNR> router, ax;
  int n_router, n_ax;
  GuRegs<CPL, IPG> gu;
  bool gu_loaded;
  uint4 attn;  // this thread's 8 elements of the attention update
  DownRegs<NX> D;
  LoraRegs LR;
};

// CPL_D: 16-byte chunks per lane of a d-wide int4 row; IPG: gate/up items
// per lane group; NX: expert slots per down row (K routed + shared); AFF:
// the affine int4 codec (bf16 scales and biases, unsigned nibbles).
template <int CPL_D, int IPG, int NX, bool AFF>
__global__ __launch_bounds__(kThreads) void k_stack(StackArgs a) {
  constexpr int CPH = 4 * CPL_D;  // 16-byte chunks per lane of a d-wide fp16 head row
  extern __shared__ __align__(16) unsigned char smem[];
  const Dims& dm = a.dm;
  constexpr int I = kStackI;
  const int d = dm.d, E = dm.E, K = dm.K, P = dm.P, G = (int)gridDim.x;
  const int cu = (int)blockIdx.x;
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int li = lane % kLG, grp = t / kLG;
  const uint32_t ep = a.epoch;
  const int cur = a.token & 1, nxt = (a.token + 1) & 1;
  const int nL = a.l1 - a.l0;
  const Lds lo = lds_layout(dm, a.ng, nL);
  float* hattn = (float*)(smem + lo.hattn);
  uint16_t* xperm = (uint16_t*)(smem + lo.xperm);
  uint16_t* xnat = (uint16_t*)(smem + lo.xnat);
  uint32_t* land = (uint32_t*)(smem + lo.land);
  uint16_t* ha = (uint16_t*)(smem + lo.ha);
  uint16_t* hx = (uint16_t*)(smem + lo.hx);
  Misc& ms = *(Misc*)(smem + lo.misc);
  LayerDev* lay = (LayerDev*)(smem + lo.lay);
  const int F = d + 2 * E;
  const int PE = P + E;

  {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(a.layers + a.l0);
    uint32_t* dst = reinterpret_cast<uint32_t*>(lay);
    const int nw = nL * (int)(sizeof(LayerDev) / 4);
    for (int i = t; i < nw; i += kThreads) dst[i] = ldg(src + i);
  }
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
  // (the layer table is in LDS now: no further global reads of it)
  if (wave == 0) {  // head list (nL <= 64: one lane per layer)
    const HeadW hw = lay[lane < nL ? lane : 0].head;
    const bool has = lane < nL && hw.fc1 != nullptr;
    const uint64_t m = __ballot(has);
    const int before = __popcll(m & ((1ull << lane) - 1ull));
    if (lane < nL) ms.hidx_of[lane] = has ? before : -1;
    if (has) {
      ms.hl_list[before] = a.l0 + lane;
      ms.hfc1[before] = hw.fc1;
      ms.hlin[before] = hw.lin;
      ms.hfc2[before] = hw.fc2;
      ms.hbias[before] = hw.bias;
    }
    if (lane == 0) ms.n_heads = __popcll(m);
  }
  for (int i = t; i < nL * K; i += kThreads) {
    const LayerDev& Ls = lay[i / K];
    ms.ent_all[i] = Ls.router ? 0 : resolve_entry(Ls.pool, E, ms.ridx_all[i]);
  }
  __syncthreads();
  // slot table of the first layer (a router layer fills its own once routed)
  if (t <= K) fill_slot(ms.eptr[0][t], lay[0], K, t, t < K ? ms.ent_all[t] : 0);
  __syncthreads();
  const int nH = ms.n_heads;
  // This workgroup's share of the heads' fc1 / linear rows (head-major), and
  // the heads whose x it keeps for them.
  int g0, g1;
  split(nH * PE, G, cu, g0, g1);
  const int hx0 = g0 / PE, hx1 = g1 > g0 ? (g1 - 1) / PE : -1;

  // down rows of this workgroup: [db, de), one per lane group
  int db, de;
  {
    int wb, we;
    split(d / 2, G, cu, wb, we);
    db = 2 * wb;
    de = 2 * we;
  }
  const int drow = db + grp;

  // Phase B loads of a layer whose routed entries are ent_k[0..K): down rows
  // [drow] of every expert slot, LoRA B_down row, the shared expert's A_down.
  // Issued once this workgroup's gate/up outputs are published, so that
  // issuing them overlaps the wait for everyone else's.
  auto issue_b = [&](const LayerDev& Ly, const void* const (*ep_k)[kEp], PhaseA<CPL_D, IPG, NX>& A) {
    const bool has_sh = Ly.sh.present != 0;
    const int Is = has_sh ? dm.Is : 0;
    const bool lora_d = has_sh && Ly.sh.ad != nullptr;
    // every load is issued; a missing row reads the zero row (see zrow)
    const bool rv = drow < de;
    const int gsh = __builtin_ctz(dm.G);
    const int wpr = I / 8, spr = I >> gsh;
    const uint32_t* q[NX];
    const uint16_t* sc[NX];
    const uint16_t* bb[NX];
#pragma unroll
    for (int k = 0; k < NX; ++k) {
      q[k] = k <= K ? (const uint32_t*)ep_k[k][2] : nullptr;
      sc[k] = k <= K ? (const uint16_t*)ep_k[k][5] : nullptr;
      bb[k] = AFF && k <= K ? (const uint16_t*)ep_k[k][8] : nullptr;
    }
#pragma unroll
    for (int k = 0; k < NX; ++k) {
      const bool v = rv && q[k] != nullptr;
      A.D.w[k] = ldg(pick(v, reinterpret_cast<const uint4*>(q[k] + (int64_t)drow * wpr + 4 * li)));
      A.D.s[k] = ldg(pick(v, sc[k] + (int64_t)drow * spr + ((32 * li) >> gsh)));
      if (AFF) A.D.b[k] = ldg(pick(v, bb[k] + (int64_t)drow * spr + ((32 * li) >> gsh)));
    }
    const bool vb = rv && lora_d && li == 0;
#pragma unroll
    for (int c = 0; c < kRank / 8; ++c)
      A.D.bd[c] = ldg(pick(vb, reinterpret_cast<const uint4*>(Ly.sh.bd + (int64_t)drow * kRank + 8 * c)));
#pragma unroll
    for (int c = 0; c < 4; ++c)
      A.LR.ad[c] = ldg(pick(lora_d, reinterpret_cast<const uint4*>(Ly.sh.ad + (int64_t)grp * Is +
                                                                   32 * li + 8 * c)));
  };

  // Issue the loads of layer l that its gate/up step needs and that do not
  // depend on its activations.
  int rt0, rt1;  // this workgroup's router rows (the same on every router layer)
  router_share(E, G, cu, rt0, rt1);
  auto issue_a = [&](int l, const LayerDev& Ly, PhaseA<CPL_D, IPG, NX>& A) {
    const bool has_sh = Ly.sh.present != 0;
    const int Is = has_sh ? dm.Is : 0;
    const int r2 = (has_sh && Ly.sh.ag) ? 2 * kRank : 0;
    // straight-line: every load is issued, missing rows from the zero row
    // (see zrow), so that no load result is merged at a branch
    const uint16_t* rp[kNR];
    int b, e;
    b = rt0;
    e = rt1;
    A.n_router = Ly.router ? e - b : 0;
    for (int j = 0; j < kNR; ++j) rp[j] = Ly.router + (int64_t)(b + (j < A.n_router ? j : 0)) * d;
    f16rows_issue<kNR>(A.router, rp, A.n_router, d);
    ax_share(r2, G, cu, b, e);
    A.n_ax = e - b;
    for (int j = 0; j < kNR; ++j) {
      const int tt = b + (j < A.n_ax ? j : 0);
      rp[j] = (tt < kRank ? Ly.sh.ag : Ly.sh.au) + (int64_t)(tt % kRank) * d;
    }
    f16rows_issue<kNR>(A.ax, rp, A.n_ax, d);
    A.attn = ldg(pick(Ly.attn != nullptr && t < d / 8, reinterpret_cast<const uint4*>(Ly.attn + 8 * t)));
    // routing known unless this is a router layer: entries from the tables
    A.gu_loaded = !Ly.router;
    GuPlan pl;
    split(K * I + Is, G, cu, pl.ib, pl.ie);
    gu_issue<CPL_D, IPG, AFF>(A.gu, Ly, dm, ms.eptr[(l - a.l0) & 1], K * I, pl, grp, li,
                              A.gu_loaded);
  };

  for (int l = a.l0; l < a.l1; ++l) {
    // Loads of layer l that need no activations go out first; they are in
    // flight while h_l is gathered (their registers live within one layer).
    stamp(a, l, 0);
    const LayerDev& Ly = lay[l - a.l0];
    PhaseA<CPL_D, IPG, NX> A;
    issue_a(l, Ly, A);
    const int step = l - a.l0;
    const bool has_sh = Ly.sh.present != 0;
    const int Is = has_sh ? dm.Is : 0;
    const int r2 = (has_sh && Ly.sh.ag) ? 2 * kRank : 0;
    const bool lora_d = has_sh && Ly.sh.ad != nullptr;
    const int n_rt = K * I;
    uint64_t* xg = a.xg + (int64_t)l * a.ng;
    const int hid = ms.hidx_of[step];
    const bool keep_x = hid >= hx0 && hid <= hx1;

    // ---- 1. h_l, attention stand-in, RMSNorm ---------------------------
    stamp(a, l, 9);
    if (step > 0) {
      ll_gather2<2>(a.xh + (int64_t)(l - 1) * (d / 2), d / 2, ep, land, a.flags, &ms.abort);
    }
    vm_drained();
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
        const bool att = Ly.attn != nullptr;
        const uint32_t aw[4] = {att ? A.attn.x : 0u, att ? A.attn.y : 0u, att ? A.attn.z : 0u,
                                att ? A.attn.w : 0u};
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
        if (AFF) {
          // chunk c (32 elements) is held by threads 4c .. 4c+3; d / 8 is a
          // multiple of 64, so whole waves take this branch
          float sx = 0.0f;
#pragma unroll
          for (int q = 0; q < 8; ++q) sx += h2f(xv[q]);
          sx += __shfl_xor(sx, 1);
          sx += __shfl_xor(sx, 2);
          if ((t & 3) == 0) ms.xsum[t >> 2] = sx;
        }
        if (keep_x) *reinterpret_cast<uint4*>(hx + (hid - hx0) * d + 8 * t) = nat;
        if (cu == 0 && a.x_trace) *reinterpret_cast<uint4*>(a.x_trace + (int64_t)l * d + 8 * t) = nat;
      }
    }
    __syncthreads();
    // LoRA A products of the shared gate/up (rows spread over the chip),
    // published now: the workgroups that own shared-expert rows need them at
    // the end of step 3 for the LoRA B terms.
    if (A.n_ax) {
      int b, e;
      ax_share(r2, G, cu, b, e);
      f16rows_finish<kNR>(A.ax, A.n_ax, d, xnat, ms);
      if (t < A.n_ax) ll_put(xg + n_rt + Is + b + t, fbits(ms.rows[t]), ep);
    }
    stamp(a, l, 2);

    // ---- 2. routing ----------------------------------------------------
    int32_t* eidx = a.exec_idx + ((int64_t)cur * a.L + l) * K;
    float* ew = a.exec_w + ((int64_t)cur * a.L + l) * K;
    if (Ly.router) {
      const int rb = rt0;
      f16rows_finish<kNR>(A.router, A.n_router, d, xnat, ms);
      stamp(a, l, 10);
      if (t < A.n_router) ll_put(a.xr + (int64_t)l * E + rb + t, fbits(ms.rows[t]), ep);
      stamp(a, l, 11);
      ll_gather2<1>(a.xr + (int64_t)l * E, E, ep, land, a.flags, &ms.abort);
      __syncthreads();
      stamp(a, l, 13);
      // the executed set (this layer's head reads it too) and its weights go
      // straight into the launch's routing tables
      if (wave == 0)
        route_wave(dm, (const float*)land, Ly.router_bias, ms.rs, &ms.ridx_all[step * K],
                   &ms.rw_all[step * K], a.flags);
      __syncthreads();
      stamp(a, l, 14);
      if (t < K) {
        const int64_t ent = resolve_entry(Ly.pool, E, ms.ridx_all[step * K + t]);
        ms.ent_all[step * K + t] = ent;
        fill_slot(ms.eptr[step & 1][t], Ly, K, t, ent);
        if (ent < 0 && cu == 0) atomicOr(&a.flags[FLAG_RANGE], 1);
      }
      __syncthreads();
    } else if (t < K && ms.ent_all[step * K + t] < 0 && cu == 0) {
      atomicOr(&a.flags[FLAG_RANGE], 1);
    }
    const int64_t* ent_k = &ms.ent_all[step * K];
    if (t < K && cu == 0) {
      eidx[t] = ms.ridx_all[step * K + t];
      ew[t] = ms.rw_all[step * K + t];
    }
    stamp(a, l, 3);

    // ---- 3. gate/up rows, shared bases, LoRA A of gate/up ----------------
    {
      GuPlan pl;
      split(n_rt + Is, G, cu, pl.ib, pl.ie);
      if (!A.gu_loaded)
        gu_issue<CPL_D, IPG, AFF>(A.gu, Ly, dm, ms.eptr[step & 1], n_rt, pl, grp, li, true);
      vm_drained();  // gate/up rows, router and LoRA A rows have arrived
      float shg[IPG], shu[IPG];
      gu_finish<CPL_D, IPG, AFF>(A.gu, ent_k, n_rt, pl, grp, li, __builtin_ctz(dm.G), xperm,
                                 ms.xsum, xg, ep, shg, shu);
      if (pl.ie > n_rt) {  // this workgroup owns rows of the shared expert
        const float* axgu = nullptr;
        if (r2) {
          ll_gather2<1>(xg + n_rt + Is, r2, ep, reinterpret_cast<uint32_t*>(ms.axgu), a.flags,
                        &ms.abort);
          __syncthreads();
          axgu = ms.axgu;
        }
        gu_finish_shared<CPL_D, IPG>(A.gu, dm.lora_scale, n_rt, pl, grp, li, axgu, shg, shu, xg,
                                     ep);
      }
      __syncthreads();  // the down-projection table of this layer is visible
    }
    stamp(a, l, 4);

    // ---- phase B loads: down rows, shared-expert LoRA -----------------------
    issue_b(Ly, ms.eptr[step & 1], A);
    const DownRegs<NX>& D = A.D;
    const LoraRegs& LR = A.LR;
    stamp(a, l, 5);

    // slot table of the next layer (its routing is known unless it is a
    // router layer, which fills its own once routed), written while this
    // layer's SwiGLU outputs are still in flight
    if (step + 1 < nL && t <= K)
      fill_slot(ms.eptr[(step + 1) & 1][t], lay[step + 1], K, t,
                t < K ? ms.ent_all[(step + 1) * K + t] : 0);
    // this layer's down bases and combine weights (read after the gather)
    if (t < NX) {
      const uint32_t* q = t <= K ? (const uint32_t*)ms.eptr[step & 1][t][2] : nullptr;
      ms.dq[t] = q;
      ms.dsc[t] = t <= K ? (const uint16_t*)ms.eptr[step & 1][t][5] : nullptr;
      ms.coef[t] = !q ? 0.0f : t < K ? ms.rw_all[step * K + t] : 1.0f;
    }

    // ---- 4. gather SwiGLU outputs; finish the shared expert ----------------
    const int ng_l = n_rt + Is;
    ll_gather2<8, true>(xg, ng_l, ep, land, a.flags, &ms.abort);
    vm_drained();
    __syncthreads();
    stamp(a, l, 6);
    {
      const float* lf = (const float*)land;
      if (has_sh) {
        // the shared expert's SwiGLU outputs, LoRA terms included
        if (lora_d) {
          // rank grp of A_down h: the lane's 32 columns, then the group's sum
          const float4* hp = reinterpret_cast<const float4*>(lf + pad32(n_rt + 32 * li));
          float p = 0.0f;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float4 v0 = hp[2 * c], v1 = hp[2 * c + 1];
            const float hv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            const uint32_t aw[4] = {LR.ad[c].x, LR.ad[c].y, LR.ad[c].z, LR.ad[c].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              p = fmaf(h2f((uint16_t)(aw[e] & 0xFFFF)), hv[2 * e], p);
              p = fmaf(h2f((uint16_t)(aw[e] >> 16)), hv[2 * e + 1], p);
            }
          }
          p = group_sum<kLG>(p);
          if (li == 0) ms.ad[grp] = p;
        }
      }
      // The down rows read the fp32 outputs in place (unresolved experts'
      // outputs are zeros, never used: their down rows are zero too).
      __syncthreads();
    }
    stamp(a, l, 7);

    // ---- 5. down rows: combine, shared expert, down LoRA, residual ---------
    if (drow < de) {
      float acc = 0.0f;
      // Slots without an expert (unresolved ids, no shared expert, k > K)
      // hold zero weights and a zero coefficient; with K == NX - 1 the loop
      // runs without branches so that the slots' LDS reads interleave.
      const float* lf = (const float*)land;
      if (K == NX - 1 && has_sh) {
#pragma unroll
        for (int k = 0; k < NX; ++k) {
          if (AFF) {
            float xs;
            const float dq = q4_dot32_f32<true>(D.w[k], lf + pad32(k * I + 32 * li), &xs);
            acc += ms.coef[k] * (bf2f(D.s[k]) * dq + bf2f(D.b[k]) * xs);
          } else {
            acc += ms.coef[k] * (h2f(D.s[k]) * q4_dot32_f32(D.w[k], lf + pad32(k * I + 32 * li)));
          }
        }
      } else {
#pragma unroll
        for (int k = 0; k < NX; ++k) {
          if (!ms.dq[k]) continue;
          if (AFF) {
            float xs;
            const float dq = q4_dot32_f32<true>(D.w[k], lf + pad32(k * I + 32 * li), &xs);
            acc += ms.coef[k] * (bf2f(D.s[k]) * dq + bf2f(D.b[k]) * xs);
          } else {
            acc += ms.coef[k] * (h2f(D.s[k]) * q4_dot32_f32(D.w[k], lf + pad32(k * I + 32 * li)));
          }
        }
      }
      if (lora_d && li == 0) {
        float lsum = 0.0f;
#pragma unroll
        for (int c = 0; c < kRank / 8; ++c) {
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
      vm_drained();
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
    stamp(a, l, 8);
  }

  if (nH == 0) return;

  // ---- heads: fc1 / linear rows, fc2 rows, routing of the logits ------------
  const int hrow = a.L;
  stamp(a, hrow, 0);
  // fc2 rows of this workgroup (head-major); they do not depend on the
  // hidden activations, so they are loaded first.
  int f0, f1;
  split(nH * E, G, cu, f0, f1);
  const int nf = f1 - f0;
  const int cpf = P / 128;
  uint4 w2[kF2R][kCPF];
#pragma unroll
  for (int r = 0; r < kF2R; ++r) {
    int f = f0 + r * kGroups + grp;
    f = f < f1 ? f : f1 - 1;
    const int h = nf > 0 ? f / E : 0, e = nf > 0 ? f % E : 0;
    const uint16_t* wrow = ms.hfc2[h] + (int64_t)e * P;
#pragma unroll
    for (int j = 0; j < kCPF; ++j) {
      w2[r][j] = make_uint4(0, 0, 0, 0);
      if (nf > 0 && r * kGroups < nf && j < cpf)
        w2[r][j] = ldg(reinterpret_cast<const uint4*>(wrow + 8 * (li + kLG * j)));
    }
  }

  // fc1 / linear rows: lane group grp takes row g0 + r*kGroups + grp of round
  // r; two rounds in flight. Lanes li < 2K also fetch the row's one-hot
  // column of the executed set (li < K) or of the previous token's set.
  {
    const int nrow = g1 - g0;
    const int R1 = (nrow + kGroups - 1) / kGroups;
    auto h1_issue = [&](uint4 (&w)[CPH], uint16_t& gv, int r) {
      int g = g0 + r * kGroups + grp;
      g = g < g1 ? g : g1 - 1;
      const int h = g / PE, it = g % PE;
      const int s = ms.hl_list[h] - a.l0;
      const uint16_t* wrow = it < P ? ms.hfc1[h] + (int64_t)it * F : ms.hlin[h] + (int64_t)(it - P) * F;
#pragma unroll
      for (int j = 0; j < CPH; ++j) w[j] = ldg(reinterpret_cast<const uint4*>(wrow + 8 * (li + kLG * j)));
      int col = d;  // an in-row column whose value is dropped
      if (li < K) {
        const int e = ms.ridx_all[s * K + li];
        if (e >= 0 && e < E) col = d + e;
      } else if (li < 2 * K) {
        const int e = ms.pidx_all[s * K + li - K];
        if (e >= 0 && e < E) col = d + E + e;
      }
      gv = ldg(wrow + col);
    };
    auto h1_finish = [&](const uint4 (&w)[CPH], uint16_t gv, int r) {
      const int graw = g0 + r * kGroups + grp;
      const int g = graw < g1 ? graw : g1 - 1;
      const int h = g / PE, it = g % PE;
      const int l = ms.hl_list[h], s = l - a.l0;
      const uint16_t* xs = hx + (h - hx0) * d;
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < CPH; ++j)
        acc = dot8_h(w[j], *reinterpret_cast<const uint4*>(xs + 8 * (li + kLG * j)), acc);
      bool use = false;
      if (li < K) {
        const int e = ms.ridx_all[s * K + li];
        use = e >= 0 && e < E;
      } else if (li < 2 * K) {
        const int e = ms.pidx_all[s * K + li - K];
        use = e >= 0 && e < E;
      }
      if (use) acc += h2f(gv);
      acc = group_sum<kLG>(acc);
      if (li == 0 && graw < g1)
        ll_put(a.xa + (int64_t)l * PE + it, fbits(it < P ? gelu_erf(acc) : acc), ep);
    };
    uint4 wa[CPH], wb[CPH];
    uint16_t ga = 0, gb = 0;
    if (nrow > 0) {
      h1_issue(wa, ga, 0);
      for (int r = 0; r < R1; r += 2) {
        if (r + 1 < R1) h1_issue(wb, gb, r + 1);
        h1_finish(wa, ga, r);
        if (r + 1 < R1) {
          if (r + 2 < R1) h1_issue(wa, ga, r + 2);
          h1_finish(wb, gb, r + 1);
        }
      }
    }
  }
  __syncthreads();
  stamp(a, hrow, 1);

  // fc2: hidden activations and linear path of the heads of this workgroup's
  // fc2 rows, as fp16 hi + lo with a power-of-two scale per lane chunk.
  const int hf0 = nf > 0 ? f0 / E : 0, hf1 = nf > 0 ? (f1 - 1) / E : -1;
  for (int h = hf0; h <= hf1; ++h)
    ll_gather2<2>(a.xa + (int64_t)ms.hl_list[h] * PE, PE, ep, land + (h - hf0) * PE, a.flags,
                  &ms.abort);
  __syncthreads();
  stamp(a, hrow, 2);
  if (t < (hf1 - hf0 + 1) * kLG) {
    const int s = t / kLG, lc = t % kLG;
    const float* act = (const float*)land + s * PE;
    float m = 0.0f;
    for (int j = 0; j < cpf; ++j) {
      const float4 u = *reinterpret_cast<const float4*>(act + 8 * (lc + kLG * j));
      const float4 v = *reinterpret_cast<const float4*>(act + 8 * (lc + kLG * j) + 4);
      m = fmaxf(m, fmaxf(fmaxf(fabsf(u.x), fabsf(u.y)), fmaxf(fabsf(u.z), fabsf(u.w))));
      m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    const int e = hilo_exponent(m);
    const float inv = ldexpf(1.0f, -e);
    for (int j = 0; j < cpf; ++j) {
      const int c = lc + kLG * j;
      uint16_t hi[8], lo2[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        f16 h_, l_;
        split_hilo(act[8 * c + q], inv, h_, l_);
        hi[q] = __builtin_bit_cast(uint16_t, h_);
        lo2[q] = __builtin_bit_cast(uint16_t, l_);
      }
      uint16_t* dst = ha + s * 2 * P + 8 * c;
      *reinterpret_cast<uint4*>(dst) =
          make_uint4(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16),
                     hi[4] | ((uint32_t)hi[5] << 16), hi[6] | ((uint32_t)hi[7] << 16));
      *reinterpret_cast<uint4*>(dst + P) =
          make_uint4(lo2[0] | ((uint32_t)lo2[1] << 16), lo2[2] | ((uint32_t)lo2[3] << 16),
                     lo2[4] | ((uint32_t)lo2[5] << 16), lo2[6] | ((uint32_t)lo2[7] << 16));
    }
    ms.hsc[s][lc] = ldexpf(1.0f, e);
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kF2R; ++r) {
    if (r * kGroups >= nf) continue;  // uniform
    const int fraw = f0 + r * kGroups + grp;
    const int f = fraw < f1 ? fraw : f1 - 1;
    const int h = f / E, e = f % E, s = h - hf0;
    const uint16_t* xh_ = ha + s * 2 * P;
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < kCPF; ++j) {
      if (j >= cpf) continue;
      const int c = li + kLG * j;
      const uint4 xa = *reinterpret_cast<const uint4*>(xh_ + 8 * c);
      const uint4 xb = *reinterpret_cast<const uint4*>(xh_ + P + 8 * c);
      acc = dot8_h(w2[r][j], xb, dot8_h(w2[r][j], xa, acc));
    }
    acc *= ms.hsc[s][li];
    acc = group_sum<kLG>(acc);
    if (li == 0 && fraw < f1) {
      const int l = ms.hl_list[h];
      const float logit = acc + bitsf(land[s * PE + P + e]);
      ll_put(a.xl + (int64_t)l * E + e, fbits(logit), ep);
      if (a.head_logits) a.head_logits[(int64_t)l * E + e] = logit;
    }
  }
  __syncthreads();
  stamp(a, hrow, 3);

  // routing of each head's logits: the next token's prediction
  for (int h = cu; h < nH; h += G) {
    const int l = ms.hl_list[h];
    ll_gather2<1>(a.xl + (int64_t)l * E, E, ep, land, a.flags, &ms.abort);
    __syncthreads();
    int32_t* pidx = l + 1 < a.L ? a.route_idx + ((int64_t)nxt * a.L + l + 1) * K : a.sink_idx;
    float* pw = l + 1 < a.L ? a.route_w + ((int64_t)nxt * a.L + l + 1) * K : a.sink_w;
    if (wave == 0) route_wave(dm, (const float*)land, ms.hbias[h], ms.rs, pidx, pw, a.flags);
    __syncthreads();
  }
  stamp(a, hrow, 4);
}

template <int CPL_D, int IPG, int NX, bool AFF>
hipError_t launch_stack_t(const StackArgs& a, int grid, hipStream_t st) {
  const Lds lo = lds_layout(a.dm, a.ng, a.l1 - a.l0);
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)k_stack<CPL_D, IPG, NX, AFF>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr_set = true;
  }
  hipLaunchKernelGGL((k_stack<CPL_D, IPG, NX, AFF>), dim3(grid), dim3(kThreads), (size_t)lo.bytes,
                     st, a);
  return hipGetLastError();
}

template <int CPL_D, int IPG, int NX>
hipError_t launch_stack_c(const StackArgs& a, int grid, hipStream_t st) {
  return a.dm.affine ? launch_stack_t<CPL_D, IPG, NX, true>(a, grid, st)
                     : launch_stack_t<CPL_D, IPG, NX, false>(a, grid, st);
}

// Largest number of consecutive blocks of size `block` that a contiguous
// range of at most `per` items can touch.
int span(int per, int block) { return per <= 0 ? 0 : (per - 1) / block + 2; }

}  // namespace

bool stack_supported(const Dims& dm) {
  if (dm.d % 512 || dm.I != kStackI || dm.K > 8 || dm.E > kMaxE) return false;
  if (dm.G < 32 || (dm.G & (dm.G - 1)) || dm.d % dm.G || dm.d / dm.G > 32) return false;
  if (dm.Is != 0 && dm.Is != dm.I) return false;
  if (dm.r != 0 && dm.r != kRank) return false;
  if (dm.P % 128 || dm.P > 128 * kCPF) return false;
  const int cpl = dm.d / 512;
  return cpl == 3 || cpl == 4;
}

bool stack_launchable(const StackArgs& a, int grid) {
  const Dims& dm = a.dm;
  const int n_heads = a.n_heads;
  if (!stack_supported(dm) || a.l1 - a.l0 > kMaxL || a.l1 <= a.l0 || grid < 1 || grid > 512)
    return false;
  if (lds_layout(dm, a.ng, a.l1 - a.l0).bytes > 160 * 1024) return false;
  // Work per workgroup must fit the fixed per-thread plans.
  const int gu_items = dm.K * dm.I + dm.Is;
  const int ipg = (gu_items + grid - 1) / grid;
  if (ipg > 2 * kGroups) return false;
  if ((dm.E + grid - 1) / grid > kNR || (2 * dm.r + grid - 1) / grid > kNR ||
      2 * ((dm.d / 2 + grid - 1) / grid) > kGroups)
    return false;
  const int PE = dm.P + dm.E;
  const int h1 = (n_heads * PE + grid - 1) / grid, f2 = (n_heads * dm.E + grid - 1) / grid;
  if (span(h1, PE) > kHX || span(f2, dm.E) > kHX || f2 > kF2R * kGroups) return false;
  return true;
}

int stack_lds_bytes(const Dims& dm, int ng, int n_layers) { return lds_layout(dm, ng, n_layers).bytes; }

hipError_t launch_stack(const StackArgs& a, int grid, hipStream_t st) {
  if (!stack_launchable(a, grid)) return hipErrorInvalidValue;
  const Dims& dm = a.dm;
  const int gu_items = dm.K * dm.I + dm.Is;
  const int ipg = (gu_items + grid - 1) / grid;
  const int cpl = dm.d / 512;
  // instantiated shapes: top-4 (5 expert slots) with one gate/up item per
  // lane group, top-8 (9 slots) with up to two
  if (dm.K <= 4 && ipg <= kGroups) {
    if (cpl == 3) return launch_stack_c<3, 1, 5>(a, grid, st);
    if (cpl == 4) return launch_stack_c<4, 1, 5>(a, grid, st);
  } else if (ipg <= 2 * kGroups) {
    if (cpl == 3) return launch_stack_c<3, 2, 9>(a, grid, st);
    if (cpl == 4) return launch_stack_c<4, 2, 9>(a, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace smd
