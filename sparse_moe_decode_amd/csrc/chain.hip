// Persistent whole-token decode kernel with a layer-ahead weight slot in LDS.
//
// One launch runs one decode token through a range of layers on every CU
// (one workgroup of 512 threads per CU). The step of a layer is the one of
// "The Other Half of the Memory Wall" §3.1 Math contract (RMSNorm, routed
// SwiGLU experts with a weighted combine, the shared expert with its
// unmerged LoRA of §3.3, residual), with the routing source of §3.2
// (Prediction-as-routing): a router layer ranks its own logits, every other
// layer runs the set the previous token's head predicted for it. The heads
// (§3.2 Head; the head layout as listed in "I counted the bytes it can't
// stream") are not on the layer chain and run after the last layer.
//
// Why this shape. At batch 1 a token is a chain of layers, each with two
// chip-wide exchanges (h, then the SwiGLU outputs), and the time per layer is
// latency, not bandwidth. Three things set that latency on gfx950:
//  * Vector memory operations of one wave retire in order, so a poll issued
//    after a wave's weight loads waits for them too. Group B (waves 4-7)
//    does every poll of the layer chain and never loads weights; group A
//    (waves 0-3) loads the weights and never polls.
//  * A compute unit keeps only so many loads in flight, so the issue of a
//    layer's ~35 KB of weights stalls the issuing waves for a memory round
//    trip or two. Group A issues them where it would wait anyway: the down
//    rows while group B forms x, the gate/up rows while group B gathers the
//    SwiGLU outputs.
//  * One wave per SIMD leaves the VALU idle between dependent instructions.
//    All eight waves compute, reading weights and activations from LDS.
//
// The layer-ahead slot. The weights a layer reads (its share of gate/up rows
// and scales, the shared items' LoRA B rows and A_down columns, down rows and
// scales, the down LoRA B rows) come from one LDS slot. Group A loads layer
// l+1's into registers during layer l (on predicted layers the experts are
// known a token ahead, §3.2 Motivation) and writes them into the slot while
// group B gathers h_{l+1}. On a router layer the routed experts are known only
// once routed: their rows are loaded then.
//
// Per layer l:
//   1. group B polls its eight elements of h_l, adds the attention update
//      (held in registers since the previous layer) and forms the RMS norm
//      (block sum); x_l is replicated in LDS. Group A writes the slot;
//   2. group A: the workgroup's fp16 row jobs (router rows, the shared
//      expert's LoRA A rows), published at once, then the issue of layer
//      l+1's down rows. All waves: one gate/up row per wave per round; wave 7
//      polls the LoRA A products meanwhile when this workgroup owns rows of
//      the shared expert;
//   3. group A publishes the routed SwiGLU outputs and issues layer l+1's
//      gate/up rows; group B publishes the shared expert's (LoRA B terms
//      added) and their partial A_down products, then gathers every SwiGLU
//      output and partial product;
//   4. all waves: one expert slot per wave, lanes over (row, column block),
//      each q * s formed in fp32 (v_fma_mix); the A_down partials are summed;
//   5. group B: combine, down LoRA, residual; h_{l+1} published as fp16 pairs.
//
// Exchange words are 8 bytes (32-bit payload, 32-bit launch epoch), written
// with agent-scope relaxed atomics and polled 16 bytes at a time with
// agent-scope buffer loads (coherent across the XCDs' L2s). Buffers are per
// layer, so no word is written twice in one launch. Every wait is bounded by
// a wall-clock limit; on expiry the kernel raises FLAG_SYNC and runs to
// completion, and every loop has a bound that every wave reaches.

#include "gemv.h"
#include "internal.h"

namespace smd {

namespace {

constexpr int kT = 512;        // threads per workgroup
constexpr int kTA = 256;       // group A: threads [0, 256); group B: [256, 512)
constexpr int kMaxL = 64;      // layers per launch
constexpr int kRank = 16;      // LoRA rank (or none)
constexpr int kI = 512;        // expert intermediate width
constexpr int kGq = 64;        // int4 group size
constexpr int kMaxX = 9;       // expert slots per down row: K <= 8 routed + the shared expert
constexpr int kJobs = 4;       // fp16 row jobs per workgroup (one per group-A wave)
constexpr int kHX = 4;         // head layers one workgroup keeps x of
constexpr int kG16 = kT / 16;  // 16-lane groups of the workgroup
constexpr int kF2R = 2;        // fc2 rounds (kG16 rows each) per workgroup
constexpr int kCPF = 4;        // 16-byte chunks per lane of an fc2 row (P <= 512)
constexpr int kSO = kChainSO;  // workgroups owning shared-expert rows, at most
constexpr uint64_t kSpin = 20000000ull;  // 0.2 s of the 100 MHz wall clock

// Shapes of one instantiation: CPR 16-byte chunks per d-wide int4 row (d =
// 32 CPR), NX expert slots per down row.
template <int CPR, int NX>
struct Shp {
  static constexpr int D = 32 * CPR;
  static constexpr int MI = NX == 5 ? 12 : 21;        // gate/up items per workgroup
  static constexpr int MR = CPR == 64 ? 10 : 8;       // down rows per workgroup
  static constexpr int NGU = (2 * MI * CPR + kTA - 1) / kTA;        // 16-byte gate/up pieces per A lane
  static constexpr int NGS = (2 * MI * (CPR / 4) + kTA - 1) / kTA;  // 4-byte gate/up scale pieces
  static constexpr int NLB = (MI * 4 + kTA - 1) / kTA;              // 16-byte LoRA B pieces
  static constexpr int NLD = (kRank * MI + kTA - 1) / kTA;          // 2-byte A_down pieces
  static constexpr int NDN = (MR * NX * 16 + kTA - 1) / kTA;        // 16-byte down pieces
  static constexpr int NDS = (MR * NX * 4 + kTA - 1) / kTA;         // 4-byte down-scale pieces
  static constexpr int JC = D / 512;                  // 16-byte pieces per lane of a row job
  static constexpr int GUR = (2 * MI + 7) / 8;        // gate/up rounds (one row per wave)
  static constexpr int NP = MR * NX;                  // down pairs (row, expert slot)
  static constexpr int DT = (MR * NX + kG16 - 1) / kG16;  // down rounds (one pair per 16-lane group)
  static constexpr int NW = NX * kI + 16 * kSO;       // SwiGLU and A_down partial words, at most
  static constexpr int JS = (NW / 4 + kTA - 1) / kTA;  // pairs of packed words per B thread
};

// Index of word w in the padded SwiGLU buffer: four floats of padding after
// every 64, so that lanes reading 64-element blocks apart hit different LDS
// banks.
__device__ __forceinline__ int svp(int w) { return w + 4 * (w >> 6); }

// Stand-in for rows that do not exist: every weight load is issued, from its
// row or from here (a load under a branch whose result merges with a default
// value makes the compiler wait for it at the merge). Never written; every
// such load reads offset 0 of it.
__device__ __align__(16) uint32_t g_czero[64];

__device__ __forceinline__ const void* czero() {
  const void* p = g_czero;
  asm("" : "+s"(p));
  return p;
}

template <typename T>
__device__ __forceinline__ const T* pk(bool v, const T* p) {
  const T* q = v ? p : (const T*)czero();
  asm("" : "+v"(q));
  return q;
}

__device__ __forceinline__ void put(uint64_t* p, uint32_t v, uint32_t ep) {
  __hip_atomic_store(p, ((uint64_t)ep << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t fb(float v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ float bf(uint32_t v) { return __builtin_bit_cast(float, v); }

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef volatile __attribute__((address_space(3))) int lds_vi;

// Give up waiting once this workgroup has given up, any workgroup raised the
// sync flag, or the wall-clock limit passed (then raise it).
__device__ __forceinline__ bool expired(uint64_t t0, int32_t* flags, int* abort_lds,
                                       uint32_t& polls) {
  lds_vi* ab = (lds_vi*)abort_lds;
  if (*ab) return true;
  if ((++polls & 63u) == 0 &&
      __hip_atomic_load(&flags[FLAG_SYNC], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    *ab = 1;
    return true;
  }
  if (wall_clock64() - t0 > kSpin) {
    atomicOr(&flags[FLAG_SYNC], 1);
    *ab = 1;
    return true;
  }
  return false;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t xrsrc(const uint64_t* base, int nwords) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, nwords * 8, 0x00020000);
}

// 16-byte agent-scope poll of word pair p (words 2p, 2p+1).
__device__ __forceinline__ v4u poll16(__amdgpu_buffer_rsrc_t rs, int p) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, p * 16, 0, 16);
}

// Poll U pairs per thread (pairs p0 + j * stride, j < U, p < np) until every
// word carries epoch ep; payloads to dst (word w at dst[w], or at dst[svp(w)]
// with PAD).
template <int U, bool PAD = false>
__device__ __forceinline__ void gather_pairs(const uint64_t* base, int np, int p0, int stride,
                                             uint32_t ep, uint32_t* dst, int32_t* flags,
                                             int* abort_lds) {
  const __amdgpu_buffer_rsrc_t rs = xrsrc(base, 2 * np);
  v4u v[U];
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int p = p0 + j * stride;
    v[j] = p < np ? poll16(rs, p) : (v4u){0u, ep, 0u, ep};
  }
  const uint64_t t0 = wall_clock64();
  uint32_t polls = 0;
  for (;;) {
    bool ok = true;
#pragma unroll
    for (int j = 0; j < U; ++j) ok = ok && v[j].y == ep && v[j].w == ep;
    if (ok) break;
    if (expired(t0, flags, abort_lds, polls)) break;
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int p = p0 + j * stride;
      if (p < np && (v[j].y != ep || v[j].w != ep)) v[j] = poll16(rs, p);
    }
  }
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int p = p0 + j * stride;
    if (p < np) {
      const int w = PAD ? svp(2 * p) : 2 * p;  // a pair never straddles a 64-word block
      *reinterpret_cast<uint2*>(dst + w) = make_uint2(v[j].x, v[j].z);
    }
  }
}

__device__ __forceinline__ bool tagged(v4u v, uint32_t tag) {
  return (v.y >> 24) == tag && (v.w >> 24) == tag;
}

// Poll U pairs of packed words per thread (pairs p0 + j * stride, j < U,
// p < np) until every word carries tag; the four values of pair p go to
// dst[svp(4p) .. + 3].
template <int U>
__device__ __forceinline__ void gather_packed(const uint64_t* base, int np, int p0, int stride,
                                              uint32_t tag, float* dst, int32_t* flags,
                                              int* abort_lds) {
  const __amdgpu_buffer_rsrc_t rs = xrsrc(base, 2 * np);
  v4u v[U];
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int p = p0 + j * stride;
    v[j] = p < np ? poll16(rs, p) : (v4u){0u, tag << 24, 0u, tag << 24};
  }
  const uint64_t t0 = wall_clock64();
  uint32_t polls = 0;
  for (;;) {
    bool ok = true;
#pragma unroll
    for (int j = 0; j < U; ++j) ok = ok && tagged(v[j], tag);
    if (ok) break;
    if (expired(t0, flags, abort_lds, polls)) break;
    __builtin_amdgcn_s_sleep(1);
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int p = p0 + j * stride;
      if (p < np && !tagged(v[j], tag)) v[j] = poll16(rs, p);
    }
  }
#pragma unroll
  for (int j = 0; j < U; ++j) {
    const int p = p0 + j * stride;
    if (p < np) {
      const float2 a = unpack2(v[j].x, v[j].y), b = unpack2(v[j].z, v[j].w);
      *reinterpret_cast<float4*>(dst + svp(4 * p)) = make_float4(a.x, a.y, b.x, b.y);
    }
  }
}

// Poll word pair p until both words carry epoch ep.
__device__ __forceinline__ v4u poll_pair(const uint64_t* base, int np, int p, uint32_t ep,
                                         int32_t* flags, int* abort_lds) {
  const __amdgpu_buffer_rsrc_t rs = xrsrc(base, 2 * np);
  v4u v = poll16(rs, p);
  if (v.y == ep && v.w == ep) return v;
  const uint64_t t0 = wall_clock64();
  uint32_t polls = 0;
  while (!(v.y == ep && v.w == ep)) {
    if (expired(t0, flags, abort_lds, polls)) break;
    __builtin_amdgcn_s_sleep(1);
    v = poll16(rs, p);
  }
  return v;
}

// Group B (four waves): each thread waits until its probe pair (the last
// word pair a producer writes) is present, or has none (has false); then the
// four waves meet on an LDS counter (gen: this thread's count of meetings
// times four). A full gather after this mostly takes one round: polls that
// find nothing are kept to one 16-byte load per producer and round.
// packed: the words carry an 8-bit tag (ep) rather than the epoch.
__device__ __forceinline__ void probe_meet(const uint64_t* base, int np, int p, bool has,
                                          uint32_t ep, int* cnt, int& gen, int32_t* flags,
                                          int* abort_lds, bool packed = false) {
  if (has && packed) {
    const __amdgpu_buffer_rsrc_t rs = xrsrc(base, 2 * np);
    v4u v = poll16(rs, p);
    const uint64_t t0 = wall_clock64();
    uint32_t polls = 0;
    while (!tagged(v, ep)) {
      if (expired(t0, flags, abort_lds, polls)) break;
      __builtin_amdgcn_s_sleep(1);
      v = poll16(rs, p);
    }
  } else if (has) {
    (void)poll_pair(base, np, p, ep, flags, abort_lds);
  }
  gen += 4;
  if ((threadIdx.x & 63) == 0)
    __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  if (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= gen) return;
  const uint64_t t0 = wall_clock64();
  uint32_t polls = 0;
  while (__hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < gen) {
    if (expired(t0, flags, abort_lds, polls)) break;
    __builtin_amdgcn_s_sleep(1);
  }
}

// Contiguous share [beg, end) of n items for workgroup c of G.
__device__ __host__ __forceinline__ void share(int n, int G, int c, int& beg, int& end) {
  beg = (int)((uint32_t)n * (uint32_t)c / (uint32_t)G);
  end = (int)((uint32_t)n * (uint32_t)(c + 1) / (uint32_t)G);
}

// Gate/up items of workgroup c of G: whole pairs, so that each packed
// exchange word (two items) has one producer.
__device__ __host__ __forceinline__ void share_items(int n, int G, int c, int& beg, int& end) {
  share(n / 2, G, c, beg, end);
  beg *= 2;
  end *= 2;
}

// First workgroup of G whose share of n items reaches past item m (m < n):
// the workgroups owning items of [m, n) are [first_past(n, G, m), G).
__device__ __host__ __forceinline__ int first_past(int n, int G, int m) {
  return (int)(((int64_t)(m + 1) * G + n - 1) / n) - 1;
}

__device__ __forceinline__ void stampc(const StackArgs& a, int row, int k, bool who) {
  if (a.trace && who)
    a.trace[((int64_t)blockIdx.x * (a.L + 1) + row) * kTracePoints + k] = wall_clock64();
}

__device__ __forceinline__ float dot8h(uint4 w, uint4 x, float acc) {
  acc = dot2(as_h2(w.x), as_h2(x.x), acc);
  acc = dot2(as_h2(w.y), as_h2(x.y), acc);
  acc = dot2(as_h2(w.z), as_h2(x.z), acc);
  acc = dot2(as_h2(w.w), as_h2(x.w), acc);
  return acc;
}

// Small per-launch and per-layer values in LDS.
struct CMisc {
  // base addresses of expert slot k (k < K routed, k == K shared; null when
  // unused or unresolved): gate q, up q, down q, gate s, up s, down s; by
  // layer parity
  const void* eptr[2][kMaxX][6];
  float coef[2][16];           // combine weight of each expert slot (0 when unused), by parity
  float ad[kRank];             // A_down . s_shared
  float axgu[2 * kRank];       // A_gate x, then A_up x
  float shs[64];               // this workgroup's shared-expert SwiGLU outputs (by item)
  float red[8];
  float hsc[kHX][kG16];        // head phase: scales of the fc2 activation chunks
  int abort;
  int bmeet;                   // group B's meeting counter (probe_meet)
  int n_heads;
  int32_t hl_list[kMaxL];
  int32_t hidx_of[kMaxL];
  const uint16_t* hfc1[kMaxL];
  const uint16_t* hlin[kMaxL];
  const uint16_t* hfc2[kMaxL];
  const float* hbias[kMaxL];
  RouteScratch rs;
};

// Byte offsets into dynamic LDS.
struct CLds {
  int lay, ridx, rw, pidx, ent, misc, tab;
  int gu, gs, lb, ld, dn, ds, bd;  // the slot (bd by layer parity)
  int xperm, xnat, hattn, sv, gpart, dpart, hx;
  int land, ha;  // head phase (over the slot)
  int bytes;
};

template <int CPR, int NX>
__host__ __device__ inline CLds chain_layout(const Dims& dm, int nL) {
  using S = Shp<CPR, NX>;
  auto up = [](int b) { return (b + 15) & ~15; };
  CLds o;
  int off = 0;
  o.lay = off; off += up(nL * (int)sizeof(LayerDev));
  o.ridx = off; off += up(nL * dm.K * 4);
  o.rw = off; off += up(nL * dm.K * 4);
  o.pidx = off; off += up(nL * dm.K * 4);
  o.ent = off; off += up(nL * dm.K * 8);
  o.misc = off; off += up((int)sizeof(CMisc));
  o.tab = off; off += up(3 * (S::NP + 2 * S::MI) * 16);
  o.gu = off; off += up(2 * S::MI * CPR * 16);
  o.gs = off; off += up(2 * S::MI * CPR);  // CPR / 2 fp16 scales per row
  o.lb = off; off += up(2 * S::MI * 64);         // by layer parity
  o.ld = off; off += up(2 * kRank * S::MI * 2);  // by layer parity
  o.dn = off; off += up(S::NP * 272);      // a pair's 256 bytes, then 16 bytes of padding
  o.ds = off; off += up(S::NP * 16);
  o.bd = off; off += up(2 * S::MR * kRank * 2);
  o.xperm = off; off += up(S::D * 2);
  o.xnat = off; off += up(S::D * 2);
  o.hattn = off; off += up(S::D * 4);
  o.sv = off; off += up((S::NW + S::NW / 16 + 8) * 4);
  o.gpart = off; off += up(2 * S::MI * 4 * 4);
  o.dpart = off; off += up(S::NP * 4);
  o.hx = off; off += up(kHX * S::D * 2);
  o.bytes = off;
  // head phase, after the layer loop: over the slot
  o.land = o.gu;
  o.ha = o.gu + up(kHX * (dm.P + dm.E) * 4);
  return o;
}

// Registers of group A holding layer l+1's slot while layer l runs: the
// gate/up part (rows, scales, the shared items' LoRA B rows and A_down
// columns) and the down part (rows, scales, down LoRA B rows). Lane tA holds
// pieces tA + 256 j of each region.
template <int CPR, int NX>
struct Pref {
  using S = Shp<CPR, NX>;
  uint4 gu[S::NGU];
  uint32_t gs[S::NGS];
  uint4 lb[S::NLB];
  uint16_t ld[S::NLD];
  uint4 dn[S::NDN];
  uint32_t ds[S::NDS];
  uint4 bd;
};

// A row's (or a down pair's) address and its scales' address; 0: no load.
struct Tab {
  uint64_t q, s;
};

// Which experts' pieces a fill covers: the routed experts (known only once a
// router layer has routed), the rest (shared expert, LoRA), or both.
enum { F_ROUTED = 1, F_STATIC = 2, F_ALL = 3 };

template <int CPR, int NX>
__global__ __launch_bounds__(kT) void k_chain(StackArgs a) {
  using S = Shp<CPR, NX>;
  constexpr int D = S::D;
  constexpr int HC = CPR / 2;  // scales per d-wide row
  extern __shared__ __align__(16) unsigned char smem[];
  const Dims& dm = a.dm;
  const int E = dm.E, K = dm.K, P = dm.P;
  const int nwg = (int)gridDim.x, cu = (int)blockIdx.x;
  const int t = threadIdx.x, wave = t >> 6;
  const bool isA = t < kTA;
  const uint32_t ep = a.epoch;
  const int cur = a.token & 1, nxt = (a.token + 1) & 1;
  const int nL = a.l1 - a.l0;
  const CLds lo = chain_layout<CPR, NX>(dm, nL);
  LayerDev* lay = (LayerDev*)(smem + lo.lay);
  int32_t* ridx_all = (int32_t*)(smem + lo.ridx);
  float* rw_all = (float*)(smem + lo.rw);
  int32_t* pidx_all = (int32_t*)(smem + lo.pidx);
  int64_t* ent_all = (int64_t*)(smem + lo.ent);
  CMisc& ms = *(CMisc*)(smem + lo.misc);
  unsigned char* s_gu = smem + lo.gu;
  uint16_t* s_gs = (uint16_t*)(smem + lo.gs);
  uint16_t* s_lb = (uint16_t*)(smem + lo.lb);
  uint16_t* s_ld = (uint16_t*)(smem + lo.ld);
  unsigned char* s_dn = smem + lo.dn;
  uint16_t* s_ds = (uint16_t*)(smem + lo.ds);
  uint16_t* s_bd = (uint16_t*)(smem + lo.bd);
  uint16_t* xperm = (uint16_t*)(smem + lo.xperm);
  uint16_t* xnat = (uint16_t*)(smem + lo.xnat);
  float* hattn = (float*)(smem + lo.hattn);
  float* sv = (float*)(smem + lo.sv);
  float* gpart = (float*)(smem + lo.gpart);
  float* dpart = (float*)(smem + lo.dpart);
  uint16_t* hx = (uint16_t*)(smem + lo.hx);
  const int PE = P + E;
  const int F = D + 2 * E;
  const int n_rt = K * kI;

  // ---- launch tables -------------------------------------------------------
  {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(a.layers + a.l0);
    uint32_t* dst = reinterpret_cast<uint32_t*>(lay);
    const int nw = nL * (int)(sizeof(LayerDev) / 4);
    for (int i = t; i < nw; i += kT) dst[i] = ldg(src + i);
  }
  if (t == 0) {
    ms.abort = 0;
    ms.bmeet = 0;
  }
  for (int i = t; i < nL * K; i += kT) {
    const int l = a.l0 + i / K, k = i % K;
    ridx_all[i] = a.route_idx[((int64_t)cur * a.L + l) * K + k];
    rw_all[i] = a.route_w[((int64_t)cur * a.L + l) * K + k];
    pidx_all[i] = a.token > 0 ? a.exec_idx[((int64_t)nxt * a.L + l) * K + k] : -1;
  }
  __syncthreads();
  if (wave == 0) {  // head list (nL <= 64: one lane per layer)
    const int lane = t & 63;
    const LayerDev* Lm = a.layers + a.l0 + (lane < nL ? lane : 0);
    const HeadW hw = {ldg(&Lm->head.fc1), ldg(&Lm->head.fc2), ldg(&Lm->head.lin),
                      ldg(&Lm->head.bias)};
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
  for (int i = t; i < nL * K; i += kT) {
    const LayerDev& Ls = lay[i / K];
    ent_all[i] = Ls.router ? 0 : resolve_entry(Ls.pool, E, ridx_all[i]);
  }
  __syncthreads();
  const int nH = ms.n_heads;
  int g0, g1;  // this workgroup's share of the heads' fc1 / linear rows
  share(nH * PE, nwg, cu, g0, g1);
  const int hx0 = g0 / PE, hx1 = g1 > g0 ? (g1 - 1) / PE : -1;
  int db, de;  // down rows [db, de)
  {
    int wb, we;
    share(D / 2, nwg, cu, wb, we);
    db = 2 * wb;
    de = 2 * we;
  }
  const int nR = de - db;

  // Slot table (expert base addresses, combine weights) of step s2 into
  // parity s2 & 1, by threads k <= K. The routed slots of a router layer are
  // filled once it has routed.
  auto fill_table = [&](int s2, int k, bool routed_known) {
    const LayerDev& Ly = lay[s2];
    const void* p[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
    float c = 0.0f;
    if (k < K) {
      const int64_t ent = ent_all[s2 * K + k];
      if (routed_known && ent >= 0) {
        p[0] = entry_ptr(Ly.pool.gate.q, ent, Ly.pool.stride_q);
        p[1] = entry_ptr(Ly.pool.up.q, ent, Ly.pool.stride_q);
        p[2] = entry_ptr(Ly.pool.down.q, ent, Ly.pool.stride_q);
        p[3] = entry_ptr(Ly.pool.gate.s, ent, Ly.pool.stride_s);
        p[4] = entry_ptr(Ly.pool.up.s, ent, Ly.pool.stride_s);
        p[5] = entry_ptr(Ly.pool.down.s, ent, Ly.pool.stride_s);
        c = rw_all[s2 * K + k];
      }
    } else if (k == K && Ly.sh.present) {
      p[0] = Ly.sh.gate.q;
      p[1] = Ly.sh.up.q;
      p[2] = Ly.sh.down.q;
      p[3] = Ly.sh.gate.s;
      p[4] = Ly.sh.up.s;
      p[5] = Ly.sh.down.s;
      c = 1.0f;
    }
#pragma unroll
    for (int i = 0; i < 6; ++i) ms.eptr[s2 & 1][k][i] = p[i];
    ms.coef[s2 & 1][k] = c;
  };

  // ---- slot fills: issue into group A's registers, then write into LDS ----
  // Address tables of a fill (set z: the parity of the layer ahead, or 2
  // for a router layer's own routed rows), built by one wave: per gate/up row
  // and per down pair the row's and its scales' addresses, 0 where the fill
  // loads nothing.
  Tab* tabs = (Tab*)(smem + lo.tab);
  auto tab_g = [&](int z) { return tabs + z * (S::NP + 2 * S::MI); };
  auto tab_d = [&](int z) { return tabs + z * (S::NP + 2 * S::MI) + 2 * S::MI; };
  auto build_tables = [&](int s2, int mode, int z, int lane) {
    const LayerDev& Ly = lay[s2];
    const void* const(*ept)[6] = ms.eptr[s2 & 1];
    int ib, ie;
    share_items(n_rt + (Ly.sh.present ? kI : 0), nwg, cu, ib, ie);
    const int nI = ie - ib;
    const bool rt = (mode & F_ROUTED) != 0, st = (mode & F_STATIC) != 0;
    if (lane < 2 * S::MI) {
      const int r = lane;
      const int it = ib + (r >> 1), gu = r & 1;
      const bool routed = it < n_rt;
      const int k = routed ? it / kI : K;
      const int row = routed ? it % kI : it - n_rt;
      uint64_t q = 0, sc = 0;
      if (r < 2 * nI && k <= K && (routed ? rt : st)) {
        const char* bq = (const char*)ept[k][gu];
        const char* bs = (const char*)ept[k][3 + gu];
        if (bq && bs) {
          q = (uint64_t)(bq + (int64_t)row * (D / 2));
          sc = (uint64_t)(bs + (int64_t)row * HC * 2);
        }
      }
      tab_g(z)[r] = Tab{q, sc};
    }
    for (int p = lane; p < S::NP; p += 64) {
      const int rr = p / NX, k = p % NX;
      uint64_t q = 0, sc = 0;
      if (rr < nR && k <= K && (k < K ? rt : st)) {
        const char* bq = (const char*)ept[k][2];
        const char* bs = (const char*)ept[k][5];
        if (bq && bs) {
          q = (uint64_t)(bq + (int64_t)(db + rr) * (kI / 2));
          sc = (uint64_t)(bs + (int64_t)(db + rr) * (kI / kGq) * 2);
        }
      }
      tab_d(z)[p] = Tab{q, sc};
    }
  };
  Pref<CPR, NX> pf;
  // Gate/up part of step s2 (tables z): rows and scales of this workgroup's
  // items, the shared items' LoRA B rows (gate, up) and A_down columns.
  // part 0: the first half of the rows; part 1: the rest; part 2: all.
  auto issue_g = [&](int s2, int z, int mode, int tA, int part) {
    const LayerDev& Ly = lay[s2];
    const Tab* tg = tab_g(z);
    int ib, ie;
    share_items(n_rt + (Ly.sh.present ? kI : 0), nwg, cu, ib, ie);
    const bool st = (mode & F_STATIC) != 0;
    constexpr int H0 = (S::NGU + 1) / 2;
#pragma unroll
    for (int j = 0; j < S::NGU; ++j) {
      if ((part == 0 && j >= H0) || (part == 1 && j < H0)) continue;
      const int q = tA + kTA * j;
      const int r = q / CPR, c = q % CPR;
      const uint64_t b = r < 2 * S::MI ? tg[r].q : 0;
      pf.gu[j] = ldg(pk(b != 0, reinterpret_cast<const uint4*>(b + 16 * c)));
    }
    if (part == 0) return;
#pragma unroll
    for (int j = 0; j < S::NGS; ++j) {
      const int q = tA + kTA * j;
      const int r = q / (HC / 2), w = q % (HC / 2);
      const uint64_t b = r < 2 * S::MI ? tg[r].s : 0;
      pf.gs[j] = ldg(pk(b != 0, reinterpret_cast<const uint32_t*>(b + 4 * w)));
    }
#pragma unroll
    for (int j = 0; j < S::NLB; ++j) {
      // item i: gate row halves, then up row halves
      const int q = tA + kTA * j;
      const int i = q >> 2, which = (q >> 1) & 1, half = q & 1;
      const int it = ib + i;
      const bool v = st && i < S::MI && it >= n_rt && it < ie && Ly.sh.bg != nullptr;
      const uint16_t* src = (which ? Ly.sh.bu : Ly.sh.bg) + (int64_t)(it - n_rt) * kRank + 8 * half;
      pf.lb[j] = ldg(pk(v, reinterpret_cast<const uint4*>(src)));
    }
#pragma unroll
    for (int j = 0; j < S::NLD; ++j) {
      // A_down[rank][item]: rank q / MI, item q % MI
      const int q = tA + kTA * j;
      const int rk = q / S::MI, i = q % S::MI;
      const int it = ib + i;
      const bool v = st && rk < kRank && it >= n_rt && it < ie && Ly.sh.ad != nullptr;
      pf.ld[j] = ldg(pk(v, Ly.sh.ad + (int64_t)rk * kI + (it - n_rt)));
    }
  };
  // Down part of step s2 (tables z): this workgroup's rows of every expert
  // slot with their scales (pair p = row * NX + slot), and the down LoRA B rows.
  auto issue_d = [&](int s2, int z, int mode, int tA) {
    const LayerDev& Ly = lay[s2];
    const Tab* td = tab_d(z);
    const bool st = (mode & F_STATIC) != 0;
#pragma unroll
    for (int j = 0; j < S::NDN; ++j) {
      const int q = tA + kTA * j;
      const int p = q >> 4, c = q & 15;
      const uint64_t b = p < S::NP ? td[p].q : 0;
      pf.dn[j] = ldg(pk(b != 0, reinterpret_cast<const uint4*>(b + 16 * c)));
    }
#pragma unroll
    for (int j = 0; j < S::NDS; ++j) {
      const int q = tA + kTA * j;
      const int p = q >> 2, w = q & 3;
      const uint64_t b = p < S::NP ? td[p].s : 0;
      pf.ds[j] = ldg(pk(b != 0, reinterpret_cast<const uint32_t*>(b + 4 * w)));
    }
    {
      const int rr = tA >> 1, half = tA & 1;
      const bool v = st && rr < nR && Ly.sh.present && Ly.sh.ad != nullptr;
      pf.bd = ldg(pk(v, reinterpret_cast<const uint4*>(Ly.sh.bd + (int64_t)(db + rr) * kRank + 8 * half)));
    }
  };
  // Write the pieces a fill of this mode loaded; the others stay in place.
  auto commit_g = [&](int s2, int mode, int tA) {
    int ib, ie;
    share_items(n_rt + (lay[s2].sh.present ? kI : 0), nwg, cu, ib, ie);
    const bool rt = (mode & F_ROUTED) != 0, st = (mode & F_STATIC) != 0;
#pragma unroll
    for (int j = 0; j < S::NGU; ++j) {
      const int q = tA + kTA * j;
      const int r = q / CPR;
      const bool sel = r < 2 * S::MI && (ib + (r >> 1) < n_rt ? rt : st);
      if (sel) *reinterpret_cast<uint4*>(s_gu + 16 * q) = pf.gu[j];
    }
#pragma unroll
    for (int j = 0; j < S::NGS; ++j) {
      const int q = tA + kTA * j;
      const int r = q / (HC / 2);
      const bool sel = r < 2 * S::MI && (ib + (r >> 1) < n_rt ? rt : st);
      if (sel) reinterpret_cast<uint32_t*>(s_gs)[q] = pf.gs[j];
    }
    if (st) {
#pragma unroll
      for (int j = 0; j < S::NLB; ++j) {
        const int q = tA + kTA * j;
        if (q < S::MI * 4) *reinterpret_cast<uint4*>(s_lb + (s2 & 1) * S::MI * 32 + 8 * q) = pf.lb[j];
      }
#pragma unroll
      for (int j = 0; j < S::NLD; ++j) {
        const int q = tA + kTA * j;
        if (q < kRank * S::MI) s_ld[(s2 & 1) * kRank * S::MI + q] = pf.ld[j];
      }
    }
  };
  auto commit_d = [&](int s2, int mode, int tA) {
    const bool rt = (mode & F_ROUTED) != 0, st = (mode & F_STATIC) != 0;
#pragma unroll
    for (int j = 0; j < S::NDN; ++j) {
      const int q = tA + kTA * j;
      const int p = q >> 4, k = p % NX;
      const bool sel = q < S::NP * 16 && (k < K ? rt : st);
      if (sel) *reinterpret_cast<uint4*>(s_dn + 272 * p + 16 * (q & 15)) = pf.dn[j];
    }
#pragma unroll
    for (int j = 0; j < S::NDS; ++j) {
      const int q = tA + kTA * j;
      const int k = (q >> 2) % NX;
      const bool sel = q < S::NP * 4 && (k < K ? rt : st);
      if (sel) reinterpret_cast<uint32_t*>(s_ds)[q] = pf.ds[j];
    }
    if (st && tA < S::MR * 2)
      *reinterpret_cast<uint4*>(s_bd + (s2 & 1) * S::MR * kRank + 8 * tA) = pf.bd;
  };

  // fp16 row jobs of step s2 (router rows, then the shared expert's LoRA A
  // rows): job w in A wave w, lane l holding columns 8 (l + 64 i) .. + 7.
  uint4 jr[S::JC];
  auto jobs_of = [&](int s2, int& nrr, int& nax, int& rb, int& xb) {
    const LayerDev& Ly = lay[s2];
    int re, xe;
    share(E, nwg, cu, rb, re);
    nrr = Ly.router ? re - rb : 0;
    const int r2 = (Ly.sh.present && Ly.sh.ag) ? 2 * kRank : 0;
    share(r2, nwg, cu, xb, xe);
    nax = xe - xb;
  };
  auto jobs_issue = [&](int s2, int lane) {
    const LayerDev& Ly = lay[s2];
    int nrr, nax, rb, xb;
    jobs_of(s2, nrr, nax, rb, xb);
    const int j = wave;  // A waves only
    const uint16_t* row = nullptr;
    if (j < nrr) row = Ly.router + (int64_t)(rb + j) * D;
    else if (j < nrr + nax) {
      const int tt = xb + j - nrr;
      row = (tt < kRank ? Ly.sh.ag : Ly.sh.au) + (int64_t)(tt % kRank) * D;
    }
#pragma unroll
    for (int i = 0; i < S::JC; ++i)
      jr[i] = ldg(pk(row != nullptr, reinterpret_cast<const uint4*>(row + 8 * (lane + 64 * i))));
  };
  // What the fill of step s2 ahead of its layer covers (its routed experts
  // only when they are known).
  auto ahead_mode = [&](int s2) { return lay[s2].router ? F_STATIC : F_ALL; };

  // The attention update of a step: group B thread tB holds elements
  // 8 tB .. 8 tB + 7.
  uint4 attn = make_uint4(0, 0, 0, 0);
  auto attn_load = [&](int s2, int tB) {
    const LayerDev& Ly = lay[s2];
    attn = ldg(pk(Ly.attn != nullptr && tB < D / 8, reinterpret_cast<const uint4*>(Ly.attn + 8 * tB)));
  };

  // ---- first layer's slot, synchronously -----------------------------------
  if (wave == 3) {
    const int lane = t & 63;
    if (lane <= K) fill_table(0, lane, !lay[0].router);
    wave_lds_sync();
    build_tables(0, ahead_mode(0), 0, lane);
  }
  __syncthreads();
  if (isA) {
    const int m0 = ahead_mode(0);
    issue_g(0, 0, m0, t, 2);
    issue_d(0, 0, m0, t);
    jobs_issue(0, t & 63);
    commit_g(0, m0, t);
    commit_d(0, m0, t);
  } else {
    attn_load(0, t - kTA);
  }
  __syncthreads();
  int gmode = 0, dmode = 0;  // what the registers hold for the next step
  int bgen = 0;              // group B: meetings so far, times four

  for (int l = a.l0; l < a.l1; ++l) {
    // The thread index, opaque to the compiler inside the layer loop: the
    // per-thread offsets of the fills and the compute are recomputed each
    // layer (a few integer instructions) instead of being hoisted out of the
    // loop and held in registers across it.
    int tx = t;
    asm volatile("" : "+v"(tx));
    const int tA = tx, tB = tx - kTA, lane = tx & 63, li = tx & 15;
    const int s = l - a.l0;
    const int cp = s & 1;
    const LayerDev& Ly = lay[s];
    const bool router = Ly.router != nullptr;
    const bool has_sh = Ly.sh.present != 0;
    const bool lora = has_sh && Ly.sh.ag != nullptr;
    const bool lora_d = has_sh && Ly.sh.ad != nullptr;
    const int Is = has_sh ? kI : 0;
    const int n_gu = n_rt + Is;
    // the workgroups owning shared-expert items publish partial A_down products
    // exchange words of the layer (packed: two values each): SwiGLU outputs
    // [0, n_gu / 2), then 8 words of partial A_down products from each
    // workgroup owning shared items; the LoRA A products (plain words) after
    // room for kSO such workgroups
    const int so0 = lora_d ? first_past(n_gu / 2, nwg, n_rt / 2) : nwg;
    const int n_so = nwg - so0;
    const int ax_off = n_gu / 2 + (lora_d ? 8 * kSO : 0);
    const uint32_t tag = 1u + ep % 255u;
    uint64_t* xg = a.xg + (int64_t)l * a.ng;
    const int hid = ms.hidx_of[s];
    const bool keep_x = hid >= hx0 && hid <= hx1;
    int ib, ie;
    share_items(n_gu, nwg, cu, ib, ie);
    const int nI = ie - ib;
    const bool ahead = s + 1 < nL;
    stampc(a, l, 0, t == 0);

    // ---- 1. B: h_l, attention update, RMSNorm; A: the slot ----------------
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = 0.0f;
    if (!isA) {
      if (s > 0) {
        // probe: the last h pair of producer tB
        int wb, we;
        share(D / 2, nwg, tB < nwg ? tB : 0, wb, we);
        probe_meet(a.xh + (int64_t)(l - 1) * (D / 2), D / 4, (we - 1) >> 1, tB < nwg && we > wb, ep,
                   &ms.bmeet, bgen, a.flags, &ms.abort);
      }
      if (tB < D / 8) {  // elements 8 tB .. 8 tB + 7
        uint32_t hw[4];
        if (s == 0) {
          const uint4 hv = ldg(reinterpret_cast<const uint4*>(a.h + 8 * tB));
          hw[0] = hv.x; hw[1] = hv.y; hw[2] = hv.z; hw[3] = hv.w;
        } else {
          const uint64_t* xb = a.xh + (int64_t)(l - 1) * (D / 2);
          const v4u p0 = poll_pair(xb, D / 4, 2 * tB, ep, a.flags, &ms.abort);
          const v4u p1 = poll_pair(xb, D / 4, 2 * tB + 1, ep, a.flags, &ms.abort);
          hw[0] = p0.x; hw[1] = p0.z; hw[2] = p1.x; hw[3] = p1.z;
        }
        const uint32_t aw[4] = {attn.x, attn.y, attn.z, attn.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[2 * q] = h2f((uint16_t)(hw[q] & 0xFFFF)) + h2f((uint16_t)(aw[q] & 0xFFFF));
          v[2 * q + 1] = h2f((uint16_t)(hw[q] >> 16)) + h2f((uint16_t)(aw[q] >> 16));
        }
        *reinterpret_cast<float4*>(hattn + 8 * tB) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(hattn + 8 * tB + 4) = make_float4(v[4], v[5], v[6], v[7]);
      }
      float ss = 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) ss = fmaf(v[q], v[q], ss);
      ss = wave_sum_rows(ss);
      if (lane == 0) ms.red[wave - 4] = ss;
      stampc(a, l, 1, tB == 0);
    } else {
      if (s > 0) {
        commit_g(s, gmode, tA);
        commit_d(s, dmode, tA);
      }
      // the next layer's slot table and fill tables (a router layer fills
      // its routed slots itself once routed); the last readers of this
      // parity and of tables 0 were in layer l-1
      if (wave == 3 && ahead) {
        if (lane <= K) fill_table(s + 1, lane, !lay[s + 1].router);
        wave_lds_sync();
        build_tables(s + 1, ahead_mode(s + 1), (s + 1) & 1, lane);
      }
      stampc(a, l, 12, t == 0);
    }
    __syncthreads();
    if (!isA) {
      const float tot = (ms.red[0] + ms.red[1]) + (ms.red[2] + ms.red[3]);
      const float inv = 1.0f / sqrtf(tot / D + dm.eps);
      if (tB < D / 8) {
        uint16_t xv[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) xv[q] = f2h(v[q] * inv);
        const uint4 nat = make_uint4(xv[0] | ((uint32_t)xv[1] << 16), xv[2] | ((uint32_t)xv[3] << 16),
                                     xv[4] | ((uint32_t)xv[5] << 16), xv[6] | ((uint32_t)xv[7] << 16));
        // pair permutation [x0 x4 x1 x5 x2 x6 x3 x7]
        const uint4 per = make_uint4(xv[0] | ((uint32_t)xv[4] << 16), xv[1] | ((uint32_t)xv[5] << 16),
                                     xv[2] | ((uint32_t)xv[6] << 16), xv[3] | ((uint32_t)xv[7] << 16));
        *reinterpret_cast<uint4*>(xnat + 8 * tB) = nat;
        *reinterpret_cast<uint4*>(xperm + 8 * tB) = per;
        if (keep_x) *reinterpret_cast<uint4*>(hx + (hid - hx0) * D + 8 * tB) = nat;
        if (cu == 0 && a.x_trace) *reinterpret_cast<uint4*>(a.x_trace + (int64_t)l * D + 8 * tB) = nat;
      }
    } else if (!router && ahead) {
      // the next layer's down part: it drains while x_l is formed and the
      // gate/up rows run, before group B polls again (a router layer issues
      // it later: its routed rows pass through the same registers first)
      dmode = ahead_mode(s + 1);
      issue_d(s + 1, (s + 1) & 1, dmode, tA);
    }
    __syncthreads();
    stampc(a, l, 2, t == 0);

    // ---- 2. row jobs, routing, gate/up -----------------------------------
    int nrr, nax, rb, xb;
    jobs_of(s, nrr, nax, rb, xb);
    if (isA && wave < nrr + nax) {
      float acc = 0.0f;
#pragma unroll
      for (int i = 0; i < S::JC; ++i)
        acc = dot8h(jr[i], *reinterpret_cast<const uint4*>(xnat + 8 * (lane + 64 * i)), acc);
      acc = wave_sum_rows(acc);
      if (lane == 0) {
        if (wave < nrr) put(a.xr + (int64_t)l * E + rb + wave, fb(acc), ep);
        else put(xg + ax_off + xb + wave - nrr, fb(acc), ep);
      }
    }
    stampc(a, l, 3, t == 0);
    int32_t* eidx = a.exec_idx + ((int64_t)cur * a.L + l) * K;
    float* ew = a.exec_w + ((int64_t)cur * a.L + l) * K;
    if (router) {
      // router layer: gather the logits, rank them, resolve the entries,
      // then load the routed experts' rows into the slot
      if (!isA)
        gather_pairs<1>(a.xr + (int64_t)l * E, E / 2, tB, 0, ep, (uint32_t*)sv, a.flags, &ms.abort);
      __syncthreads();
      stampc(a, l, 10, t == 0);
      if (wave == 4)
        route_wave(dm, sv, Ly.router_bias, ms.rs, &ridx_all[s * K], &rw_all[s * K], a.flags);
      __syncthreads();
      if (wave == 3) {
        if (lane < K) {
          const int64_t ent = resolve_entry(Ly.pool, E, ridx_all[s * K + lane]);
          ent_all[s * K + lane] = ent;
          if (ent < 0 && cu == 0) atomicOr(&a.flags[FLAG_RANGE], 1);
        }
        wave_lds_sync();
        if (lane <= K) fill_table(s, lane, true);
        wave_lds_sync();
        build_tables(s, F_ROUTED, 2, lane);
      }
      __syncthreads();
      if (isA) {
        issue_g(s, 2, F_ROUTED, tA, 2);
        issue_d(s, 2, F_ROUTED, tA);
        commit_g(s, F_ROUTED, tA);
        commit_d(s, F_ROUTED, tA);
      }
      __syncthreads();
      stampc(a, l, 11, t == 0);
    } else if (t < K && cu == 0 && ent_all[s * K + t] < 0) {
      atomicOr(&a.flags[FLAG_RANGE], 1);
    }
    if (t < K && cu == 0) {
      eidx[t] = ridx_all[s * K + t];
      ew[t] = rw_all[s * K + t];
    }
    const bool need_ax = lora && ie > n_rt;
    {
      // gate/up rows: wave w takes rows w, w + 8, ...; lane c holds x chunk c
      // (32 elements, pair-permuted)
      f16x2 xr[16];
      const bool lv = lane < CPR;
      if (lv) load_xchunk(xperm, lane, xr);
      else {
#pragma unroll
        for (int q = 0; q < 16; ++q) xr[q] = (f16x2){(f16)0.0f, (f16)0.0f};
      }
      float pr[S::GUR];
#pragma unroll
      for (int rr = 0; rr < S::GUR; ++rr) {
        const int r = wave + 8 * rr;
        pr[rr] = 0.0f;
        if (r < 2 * nI && lv) {
          const uint4 w = *reinterpret_cast<const uint4*>(s_gu + 16 * (r * CPR + lane));
          const float sc = h2f(s_gs[r * HC + (lane >> 1)]);
          pr[rr] = sc * q4_dot32(w, xr);
        }
      }
#pragma unroll
      for (int rr = 0; rr < S::GUR; ++rr) {
        const int r = wave + 8 * rr;
        const float g = group_sum<16>(pr[rr]);
        if (r < 2 * nI && li == 0) gpart[4 * r + (lane >> 4)] = g;
      }
    }
    if (need_ax && wave == 7)
      gather_pairs<1>(xg + ax_off, kRank, lane, 0, ep, reinterpret_cast<uint32_t*>(ms.axgu), a.flags,
                      &ms.abort);
    __syncthreads();
    stampc(a, l, 4, t == 0);

    // ---- 3. SwiGLU outputs and A_down partials out; B gathers them -------
    if (isA) {
      if (2 * tA < nI && ib + 2 * tA < n_rt) {
        // routed items 2w, 2w + 1 (one expert: I is even) as one packed word
        const int it = ib + 2 * tA;
        const float4* gp = reinterpret_cast<const float4*>(gpart + 4 * (4 * tA));
        const float4 g0 = gp[0], u0 = gp[1], g1 = gp[2], u1 = gp[3];
        const bool ok = ms.eptr[cp][it / kI][0] != nullptr;
        const float a0 = silu((g0.x + g0.y) + (g0.z + g0.w)) * ((u0.x + u0.y) + (u0.z + u0.w));
        const float a1 = silu((g1.x + g1.y) + (g1.z + g1.w)) * ((u1.x + u1.y) + (u1.z + u1.w));
        put2(xg + it / 2, ok ? a0 : 0.0f, ok ? a1 : 0.0f, tag);
      }
      // the first half of the next layer's gate/up rows and its row jobs:
      // they drain at the start of group B's wait for the SwiGLU outputs
      if (ahead) {
        gmode = ahead_mode(s + 1);
        issue_g(s + 1, (s + 1) & 1, gmode, tA, 0);
        jobs_issue(s + 1, lane);
      }
      stampc(a, l, 13, t == 0);
    } else {
      if (wave == 4 && ie > n_rt) {
        // this workgroup's shared items (nI <= 64: one wave)
        const int i0 = n_rt > ib ? n_rt - ib : 0;
        if (lane >= i0 && lane < nI) {
          const float4 gp = *reinterpret_cast<const float4*>(gpart + 4 * (2 * lane));
          const float4 up_ = *reinterpret_cast<const float4*>(gpart + 4 * (2 * lane + 1));
          float g = (gp.x + gp.y) + (gp.z + gp.w), u = (up_.x + up_.y) + (up_.z + up_.w);
          if (lora) {
            const uint4* bq = reinterpret_cast<const uint4*>(s_lb + cp * S::MI * 32 + lane * 32);
            const float4* ax = reinterpret_cast<const float4*>(ms.axgu);
            float lg = 0.0f, lu = 0.0f;
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const uint4 wg = bq[c], wu = bq[2 + c];
              const float4 a0 = ax[2 * c], a1 = ax[2 * c + 1];
              const float4 b0 = ax[4 + 2 * c], b1 = ax[4 + 2 * c + 1];
              const uint32_t g4[4] = {wg.x, wg.y, wg.z, wg.w}, u4[4] = {wu.x, wu.y, wu.z, wu.w};
              const float ag[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
              const float au[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                lg = fmaf(h2f((uint16_t)(g4[e] & 0xFFFF)), ag[2 * e], lg);
                lg = fmaf(h2f((uint16_t)(g4[e] >> 16)), ag[2 * e + 1], lg);
                lu = fmaf(h2f((uint16_t)(u4[e] & 0xFFFF)), au[2 * e], lu);
                lu = fmaf(h2f((uint16_t)(u4[e] >> 16)), au[2 * e + 1], lu);
              }
            }
            g = fmaf(dm.lora_scale, lg, g);
            u = fmaf(dm.lora_scale, lu, u);
          }
          ms.shs[lane] = silu(g) * u;
        }
        wave_lds_sync();
        // shared items, two to a packed word (i0 is even)
        if (2 * lane >= i0 && 2 * lane < nI)
          put2(xg + (ib + 2 * lane) / 2, ms.shs[2 * lane], ms.shs[2 * lane + 1], tag);
        if (lora_d) {
          // partial A_down . s_shared over this workgroup's items; rank = lane
          if (lane < kRank) {
            float acc = 0.0f;
            for (int i = i0; i < nI; ++i)
              acc = fmaf(h2f(s_ld[cp * kRank * S::MI + lane * S::MI + i]), ms.shs[i], acc);
            ms.shs[32 + lane] = acc;
          }
          wave_lds_sync();
          if (lane < kRank / 2)
            put2(xg + n_gu / 2 + 8 * (cu - so0) + lane, ms.shs[32 + 2 * lane],
                 ms.shs[32 + 2 * lane + 1], tag);
        }
      }
      stampc(a, l, 5, tB == 0);
      const int nw = n_gu / 2 + 8 * n_so;  // packed words to gather (even)
      {
        // probe: the last word producer tB writes (its last A_down partial,
        // else its last SwiGLU output)
        const int c = tB < nwg ? tB : 0;
        int cb, ce;
        share_items(n_gu, nwg, c, cb, ce);
        const int last = c >= so0 ? n_gu / 2 + 8 * (c - so0) + 7 : ce / 2 - 1;
        probe_meet(xg, nw / 2, last >> 1, tB < nwg && (ce > cb || c >= so0), tag, &ms.bmeet, bgen,
                   a.flags, &ms.abort, true);
      }
      gather_packed<S::JS>(xg, nw / 2, tB, kTA, tag, sv, a.flags, &ms.abort);
      stampc(a, l, 6, tB == 0);
      if (ahead) attn_load(s + 1, tB);
    }
    __syncthreads();
    stampc(a, l, 7, t == 0);

    // ---- 4. down: every wave; the A_down sum ------------------------------
    {
      // one 32-element chunk of one (row, expert slot) pair per lane and
      // round: lane groups of 16 cover a pair's 512 columns; pairs k-major
      const int np = nR * (K + 1);
      const int g16 = tx >> 4;
#pragma unroll
      for (int dr = 0; dr < S::DT; ++dr) {
        const int u = g16 + kG16 * dr;  // pair index, uniform over the group
        if (u >= np) continue;
        const int k = u / nR, rr = u - k * nR;
        const int p = rr * NX + k;
        const float cf = ms.coef[cp][k];
        float acc = 0.0f;
        if (cf != 0.0f) {
          const uint4 w = *reinterpret_cast<const uint4*>(s_dn + 272 * p + 16 * li);
          const float sc = h2f(s_ds[p * 8 + (li >> 1)]);
          acc = (cf * sc) * q4_dot32_f32(w, sv + svp(k * kI + 32 * li));
        }
        acc = group_sum<16>(acc);
        if (li == 0) dpart[p] = acc;
      }
      // A_down . s_shared: rank lane / 4 summed over every fourth partial,
      // on the last wave (it has the fewest pairs)
      if (lora_d && wave == 7) {
        const int rk = lane >> 2, qq = lane & 3;
        float acc = 0.0f;
#pragma unroll 4
        for (int c = qq; c < n_so; c += 4) acc += sv[svp(n_gu + 16 * c + rk)];
        acc = group_sum<4>(acc);
        if (qq == 0) ms.ad[rk] = acc;
      }
    }
    __syncthreads();
    stampc(a, l, 8, t == 0);

    // ---- 5. B: combine, down LoRA, residual; publish h_{l+1} -------------
    // A: the rest of the next layer's gate/up part (and, after a router
    // layer, its down part): they drain at the start of the wait for h
    if (isA && ahead) {
      issue_g(s + 1, (s + 1) & 1, gmode, tA, 1);
      if (router) {
        dmode = gmode;
        issue_d(s + 1, (s + 1) & 1, dmode, tA);
      }
      stampc(a, l, 14, t == 0);
    }
    if (wave == 4) {
      const int r = lane;
      float y = 0.0f;
      if (r < nR) {
        float pk_[NX];
#pragma unroll
        for (int k = 0; k < NX; ++k) pk_[k] = k <= K ? dpart[r * NX + k] : 0.0f;
#pragma unroll
        for (int k = 0; k < NX; ++k) y += pk_[k];
        if (lora_d) {
          const uint4* bq = reinterpret_cast<const uint4*>(s_bd + cp * S::MR * kRank + r * kRank);
          const float4* ad = reinterpret_cast<const float4*>(ms.ad);
          float ls = 0.0f;
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const uint4 bw = bq[c];
            const float4 a0 = ad[2 * c], a1 = ad[2 * c + 1];
            const uint32_t b4[4] = {bw.x, bw.y, bw.z, bw.w};
            const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ls = fmaf(h2f((uint16_t)(b4[e] & 0xFFFF)), av[2 * e], ls);
              ls = fmaf(h2f((uint16_t)(b4[e] >> 16)), av[2 * e + 1], ls);
            }
          }
          y = fmaf(dm.lora_scale, ls, y);
        }
      }
      const uint32_t h16 = r < nR ? f2h(hattn[db + r] + y) : 0u;
      const uint32_t hn = (uint32_t)__shfl_xor((int)h16, 1);
      if (r < nR && !(r & 1)) {
        const uint32_t word = h16 | (hn << 16);
        *reinterpret_cast<uint32_t*>(a.h + (int64_t)(s + 1) * D + db + r) = word;
        put(a.xh + (int64_t)l * (D / 2) + db / 2 + r / 2, word, ep);
      }
      stampc(a, l, 9, tB == 0);
    }
  }
  __syncthreads();

  if (nH == 0) return;
  const int lane = t & 63, li = t & 15, grp = t >> 4;
  (void)lane;

  // ---- heads: fc1 / linear rows, fc2 rows, routing of the logits ------------
  uint32_t* land = (uint32_t*)(smem + lo.land);
  uint16_t* ha = (uint16_t*)(smem + lo.ha);
  constexpr int CPH = D / 128;  // 16-byte chunks per lane of a d-wide fp16 row (16 lanes)
  const int hrow = a.L;
  stampc(a, hrow, 0, t == 0);
  int f0, f1;  // fc2 rows of this workgroup (head-major)
  share(nH * E, nwg, cu, f0, f1);
  const int nf = f1 - f0;
  const int cpf = P / 128;
  uint4 w2[kF2R][kCPF];
#pragma unroll
  for (int r = 0; r < kF2R; ++r) {
    int f = f0 + r * kG16 + grp;
    f = f < f1 ? f : f1 - 1;
    const int h = nf > 0 ? f / E : 0, e = nf > 0 ? f % E : 0;
    const uint16_t* wrow = ms.hfc2[h] + (int64_t)e * P;
#pragma unroll
    for (int j = 0; j < kCPF; ++j)
      w2[r][j] = ldg(pk(nf > 0 && r * kG16 < nf && j < cpf,
                        reinterpret_cast<const uint4*>(wrow + 8 * (li + 16 * j))));
  }
  {
    const int nrow = g1 - g0;
    const int R1 = (nrow + kG16 - 1) / kG16;
    auto h1_issue = [&](uint4 (&w)[CPH], uint16_t& gv, int r) {
      int g = g0 + r * kG16 + grp;
      g = g < g1 ? g : g1 - 1;
      const int h = g / PE, it = g % PE;
      const int s = ms.hl_list[h] - a.l0;
      const uint16_t* wrow = it < P ? ms.hfc1[h] + (int64_t)it * F : ms.hlin[h] + (int64_t)(it - P) * F;
#pragma unroll
      for (int j = 0; j < CPH; ++j) w[j] = ldg(reinterpret_cast<const uint4*>(wrow + 8 * (li + 16 * j)));
      int col = D;  // an in-row column whose value is dropped
      if (li < K) {
        const int e = ridx_all[s * K + li];
        if (e >= 0 && e < E) col = D + e;
      } else if (li < 2 * K) {
        const int e = pidx_all[s * K + li - K];
        if (e >= 0 && e < E) col = D + E + e;
      }
      gv = ldg(wrow + col);
    };
    auto h1_finish = [&](const uint4 (&w)[CPH], uint16_t gv, int r) {
      const int graw = g0 + r * kG16 + grp;
      const int g = graw < g1 ? graw : g1 - 1;
      const int h = g / PE, it = g % PE;
      const int l = ms.hl_list[h], s = l - a.l0;
      const uint16_t* xs = hx + (h - hx0) * D;
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < CPH; ++j)
        acc = dot8h(w[j], *reinterpret_cast<const uint4*>(xs + 8 * (li + 16 * j)), acc);
      bool use = false;
      if (li < K) {
        const int e = ridx_all[s * K + li];
        use = e >= 0 && e < E;
      } else if (li < 2 * K) {
        const int e = pidx_all[s * K + li - K];
        use = e >= 0 && e < E;
      }
      if (use) acc += h2f(gv);
      acc = group_sum<16>(acc);
      if (li == 0 && graw < g1)
        put(a.xa + (int64_t)l * PE + it, fb(it < P ? gelu_erf(acc) : acc), ep);
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
  stampc(a, hrow, 1, t == 0);

  // fc2: hidden activations and linear path of the heads of this workgroup's
  // fc2 rows, as fp16 hi + lo with a power-of-two scale per lane chunk.
  const int hf0 = nf > 0 ? f0 / E : 0, hf1 = nf > 0 ? (f1 - 1) / E : -1;
  for (int h = hf0; h <= hf1; ++h) {
    const int np = PE / 2;
    const uint64_t* base = a.xa + (int64_t)ms.hl_list[h] * PE;
    uint32_t* dst = land + (h - hf0) * PE;
    for (int p0 = 0; p0 < np; p0 += kT)
      gather_pairs<1>(base, np, p0 + t, 0, ep, dst, a.flags, &ms.abort);
  }
  __syncthreads();
  stampc(a, hrow, 2, t == 0);
  if (t < (hf1 - hf0 + 1) * 16) {
    const int s = t / 16, lc = t % 16;
    const float* act = (const float*)land + s * PE;
    float m = 0.0f;
    for (int j = 0; j < cpf; ++j) {
      const float4 u = *reinterpret_cast<const float4*>(act + 8 * (lc + 16 * j));
      const float4 w = *reinterpret_cast<const float4*>(act + 8 * (lc + 16 * j) + 4);
      m = fmaxf(m, fmaxf(fmaxf(fabsf(u.x), fabsf(u.y)), fmaxf(fabsf(u.z), fabsf(u.w))));
      m = fmaxf(m, fmaxf(fmaxf(fabsf(w.x), fabsf(w.y)), fmaxf(fabsf(w.z), fabsf(w.w))));
    }
    const int e = hilo_exponent(m);
    const float inv = ldexpf(1.0f, -e);
    for (int j = 0; j < cpf; ++j) {
      const int c = lc + 16 * j;
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
    if (r * kG16 >= nf) continue;  // uniform
    const int fraw = f0 + r * kG16 + grp;
    const int f = fraw < f1 ? fraw : f1 - 1;
    const int h = f / E, e = f % E, s = h - hf0;
    const uint16_t* xh_ = ha + s * 2 * P;
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < kCPF; ++j) {
      if (j >= cpf) continue;
      const int c = li + 16 * j;
      const uint4 xa = *reinterpret_cast<const uint4*>(xh_ + 8 * c);
      const uint4 xb2 = *reinterpret_cast<const uint4*>(xh_ + P + 8 * c);
      acc = dot8h(w2[r][j], xb2, dot8h(w2[r][j], xa, acc));
    }
    acc *= ms.hsc[s][li];
    acc = group_sum<16>(acc);
    if (li == 0 && fraw < f1) {
      const int l = ms.hl_list[h];
      const float logit = acc + bf(land[s * PE + P + e]);
      put(a.xl + (int64_t)l * E + e, fb(logit), ep);
      if (a.head_logits) a.head_logits[(int64_t)l * E + e] = logit;
    }
  }
  __syncthreads();
  stampc(a, hrow, 3, t == 0);

  // routing of each head's logits: the next token's prediction
  for (int h = cu; h < nH; h += nwg) {
    const int l = ms.hl_list[h];
    float* lg = (float*)land;
    if (t < E / 2) gather_pairs<1>(a.xl + (int64_t)l * E, E / 2, t, 0, ep, (uint32_t*)lg, a.flags, &ms.abort);
    __syncthreads();
    int32_t* pidx = l + 1 < a.L ? a.route_idx + ((int64_t)nxt * a.L + l + 1) * K : a.sink_idx;
    float* pw = l + 1 < a.L ? a.route_w + ((int64_t)nxt * a.L + l + 1) * K : a.sink_w;
    if (wave == 0) route_wave(dm, lg, ms.hbias[h], ms.rs, pidx, pw, a.flags);
    __syncthreads();
  }
  stampc(a, hrow, 4, t == 0);
}

template <int CPR, int NX>
hipError_t launch_t(const StackArgs& a, int grid, hipStream_t st) {
  const CLds lo = chain_layout<CPR, NX>(a.dm, a.l1 - a.l0);
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void*)k_chain<CPR, NX>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    attr_set = true;
  }
  hipLaunchKernelGGL((k_chain<CPR, NX>), dim3(grid), dim3(kT), (size_t)lo.bytes, st, a);
  return hipGetLastError();
}

int span_of(int per, int block) { return per <= 0 ? 0 : (per - 1) / block + 2; }

template <int CPR, int NX>
bool fits(const StackArgs& a, int grid) {
  using S = Shp<CPR, NX>;
  const Dims& dm = a.dm;
  const int nL = a.l1 - a.l0;
  if (chain_layout<CPR, NX>(dm, nL).bytes > 160 * 1024) return false;
  const int items = dm.K * dm.I + dm.Is;
  if (2 * ((items / 2 + grid - 1) / grid) > S::MI) return false;
  if (2 * ((dm.d / 2 + grid - 1) / grid) > S::MR) return false;
  if ((dm.E + grid - 1) / grid + (2 * dm.r + grid - 1) / grid > kJobs) return false;
  // the workgroups owning shared-expert items, each publishing 16 partial
  // A_down products
  if (dm.Is && grid - first_past((dm.K * dm.I + dm.Is) / 2, grid, dm.K * dm.I / 2) > kSO) return false;
  const int PE = dm.P + dm.E;
  const int h1 = (a.n_heads * PE + grid - 1) / grid, f2 = (a.n_heads * dm.E + grid - 1) / grid;
  if (span_of(h1, PE) > kHX || span_of(f2, dm.E) > kHX || f2 > kF2R * kG16) return false;
  return true;
}

}  // namespace

bool chain_launchable(const StackArgs& a, int grid) {
  const Dims& dm = a.dm;
  if (dm.affine || dm.I != kI || dm.G != kGq || dm.K < 1 || dm.K > 8) return false;
  if (dm.d != 2048 && dm.d != 1536) return false;
  if (dm.Is != 0 && dm.Is != kI) return false;
  if (dm.r != 0 && dm.r != kRank) return false;
  if (dm.P % 128 || dm.P > 128 * kCPF || dm.E > kMaxE || (dm.E & 1)) return false;
  const int nL = a.l1 - a.l0;
  if (nL < 1 || nL > kMaxL || grid < 1 || grid > 1024) return false;
  const int cpr = dm.d / 32;
  if (cpr == 64) return dm.K <= 4 ? fits<64, 5>(a, grid) : fits<64, 9>(a, grid);
  return dm.K <= 4 ? fits<48, 5>(a, grid) : fits<48, 9>(a, grid);
}

hipError_t launch_chain(const StackArgs& a, int grid, hipStream_t st) {
  if (!chain_launchable(a, grid)) return hipErrorInvalidValue;
  const int cpr = a.dm.d / 32;
  if (cpr == 64) return a.dm.K <= 4 ? launch_t<64, 5>(a, grid, st) : launch_t<64, 9>(a, grid, st);
  return a.dm.K <= 4 ? launch_t<48, 5>(a, grid, st) : launch_t<48, 9>(a, grid, st);
}

}  // namespace smd
