// Internal types shared by the HIP kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sparse_moe_decode.h"

namespace smd {

// Device view of one int4 matrix (b: affine biases, null for symmetric).
struct Q4 {
  const uint32_t* q;
  const uint16_t* s;
  const uint16_t* b;
};

// Device view of a routed pool: entry j of projection p sits at
// p.q + j*stride_q bytes (scales p.s + j*stride_s). Expert ids map to
// entries directly, or through slot_of when it is set.
struct Pool {
  Q4 gate, up, down;
  int64_t stride_q, stride_s;
  int32_t count;
  const int32_t* slot_of;
};

struct SharedW {
  Q4 gate, up, down;
  const uint16_t *ag, *bg, *au, *bu, *ad, *bd;  // LoRA A/B per projection, nullable
  int32_t present;
};

struct HeadW {
  const uint16_t *fc1, *fc2, *lin;
  const float* bias;
};

// One layer of a stack as the persistent kernel reads it (device table).
struct LayerDev {
  Pool pool;
  SharedW sh;
  const uint16_t* router;
  const float* router_bias;
  HeadW head;
  const uint16_t* attn;
};

// Tier dimensions as the kernels use them.
struct Dims {
  int32_t d, E, K, I, Is, P, G, r;
  float lora_scale;  // alpha / r
  int32_t router_kind, norm_topk, n_groups, topk_groups;
  float route_scale, eps;
  int32_t affine;  // E0_QUANT_AFFINE codec
};

// Flags the kernels raise (device int32 array).
enum { FLAG_RANGE = 0, FLAG_SYNC = 1, N_FLAGS = 4 };

// Per-context device scratch, sized for max_tokens tokens.
struct Scratch {
  int32_t max_tokens;
  float* gu;      // [B][K+1][Imax] SwiGLU outputs (routed experts, then shared)
  float* ax;      // [B][3][rmax]   LoRA A products: gate, up, down
  float* hattn;   // [B][d]         h + attention update (fp32); the batched path's
                  //                affine input sums [B][d/64]
  uint16_t* xn;   // [B][d]         fp16 RMS-normed activation
  float* hact;    // [B][P]         head hidden activation erf_gelu(fc1 f)
  float* hlin;    // [B][E]         head linear path lin f
  float* logits;  // [B][E]         router / head logits
  int32_t* sink_idx;  // [B][K]     prediction with no consumer layer
  float* sink_w;      // [B][K]
  int32_t* flags; // [N_FLAGS]
  // batched path (B >= 16 tokens)
  int32_t* grp;   // [batched_grp_ints] experts of the batch, their token runs,
                  //                work tiles and tile descriptors (T = batched_max_tiles)
  float* axp;     // [kLoraSlices][B][2 rmax] shared gate/up LoRA A products
                  //                over slices of the inputs
  float* yk;      // [B][K+1][d]    per-slot down outputs
};

// Input slices of the batched path's LoRA A products (summed in order later).
constexpr int kLoraSlices = 8;

// ---- launchers (kernels.hip) ------------------------------------------------
// All return hipSuccess or the launch error; shapes are validated by callers.

// SwiGLU gate/up for the K routed experts of each token (expert k reads
// routing idx[b*K + k]) and, when sh.present, the shared expert (slot K).
hipError_t launch_gate_up(const Dims& dm, const Pool& pool, const SharedW& sh,
                          const uint16_t* x, const int32_t* idx, int B, const Scratch& s,
                          hipStream_t st);
// Down projections + weighted combine + shared expert + down LoRA.
// Output y16[b][d] = fp16(resid[b][d] + y) (resid may be null).
hipError_t launch_down(const Dims& dm, const Pool& pool, const SharedW& sh,
                       const int32_t* idx, const float* w, int B, const float* resid,
                       uint16_t* y16, const Scratch& s, hipStream_t st);
// LoRA A products: ax[b][slot][t] = sum_i A[t][i] x[b][i] for up to 3 A's.
// x is fp16 ([B][in], stride x_stride) or fp32 when xf32 != nullptr.
hipError_t launch_lora_a(int n_mats, const uint16_t* const* A, const int* slots, int in_dim,
                         int r, const uint16_t* x16, const float* xf32, int64_t x_stride,
                         int B, float* ax, int ax_stride, hipStream_t st);
// y_acc[b][o] += scale * sum_t Bm[o][t] ax[b][t]
hipError_t launch_lora_b(const uint16_t* Bm, int out_dim, int r, float scale, const float* ax,
                         int ax_stride, float* y_acc, int B, hipStream_t st);
// Dense fp16 GEMV: y[b][o] = W[o, 0:cols] . x[b] (+ gathered one-hot columns
// W[o, gcol0 + cur[b][k]] and W[o, gcol0 + E + prev[b][k]]) with epilogue:
// epi 0 none, 1 erf-GELU, 2 add addv[b][o]. x is fp16, or fp32 if xf32.
hipError_t launch_gemv16(const uint16_t* W, int rows, int cols, int64_t ld,
                         const uint16_t* x16, const float* xf32, int64_t x_stride, int B,
                         const int32_t* cur, const int32_t* prev, int K, int E, int gcol0,
                         int epi, const float* addv, float* y, int64_t y_stride,
                         hipStream_t st);
// Routing of fp32 logits [B][E] with the tier's family -> idx/w [B][K].
hipError_t launch_route(const Dims& dm, const float* logits, const float* bias, int B,
                        int32_t* idx, float* w, int32_t* flags, hipStream_t st);
// h_attn = h + attn, xn = fp16(RMSNorm(h_attn)); optionally copies a routing
// (cidx/cw [B][K]) into exec (eidx/ew).
hipError_t launch_prep(const Dims& dm, const uint16_t* h, const uint16_t* attn, int B,
                       float* hattn, uint16_t* xn, const int32_t* cidx, const float* cw,
                       int32_t* eidx, float* ew, hipStream_t st);

// Batch of B tokens through grouped int4 GEMMs on MFMA (batched.hip):
// y[b] = fp16(sum_k w[b,k] E_idx(x[b]) + S(x[b])). Work is split into tiles of
// up to 32 tokens of one expert (the union of the batch's experts, plus the
// shared expert over all B tokens).
bool batched_supported(const Dims& dm);
// Upper bound on the work tiles of a batch: sum over members of
// ceil(count/32) <= B*K/32 + members, members <= min(B*K, E), plus the
// shared expert's ceil(B/32).
inline int batched_max_tiles(int B, int K, int E) {
  const int BK = B * K;
  return (B + 31) / 32 + (BK < E ? BK : E) + (BK + 31) / 32;
}
// The grouping tables (int32): counts, sorted entries, union members and
// their runs [2 + 4 B K], the tiles [2 T]; then, from this 16-byte aligned
// offset, one int4 descriptor per tile [4 T].
__host__ __device__ inline int batched_desc_offset(int BK, int ny) { return (2 + 4 * BK + 2 * ny + 3) & ~3; }
inline size_t batched_grp_ints(int B, int K, int E) {
  const int ny = batched_max_tiles(B, K, E);
  return (size_t)batched_desc_offset(B * K, ny) + 4 * (size_t)ny;
}
hipError_t launch_batched(const Dims& dm, const Pool& pool, const SharedW& sh, const uint16_t* x,
                          const int32_t* idx, const float* w, int B, uint16_t* y,
                          const Scratch& s, hipStream_t st);

// Persistent whole-token kernel (stack.hip). Exchange buffers hold 8-byte
// (payload, epoch) words per layer: xh [L][d/2] h_out fp16 pairs, xg [L][ng]
// SwiGLU outputs + shared bases + LoRA A products, xr [L][E] router logits,
// xa [L][P+E] head hidden + linear path, xl [L][E] head logits.
struct StackArgs {
  Dims dm;
  const LayerDev* layers;
  int32_t L, l0, l1, token, ng;
  int32_t n_heads;  // layers of [l0, l1) with a head
  uint32_t epoch;
  int32_t* route_idx;
  float* route_w;
  int32_t* exec_idx;
  float* exec_w;
  float* head_logits;
  uint16_t* x_trace;
  uint16_t* h;
  uint64_t *xh, *xg, *xr, *xa, *xl;
  int32_t* sink_idx;
  float* sink_w;
  int32_t* flags;
  uint64_t* trace;  // optional [G][L+1][kTracePoints] wall-clock stamps (100 MHz)
};
constexpr int kTracePoints = 16;
bool stack_supported(const Dims& dm);
// Whether one launch over [l0, l1) (with a.n_heads head layers) fits the
// kernel's fixed per-workgroup plans on `grid` workgroups.
bool stack_launchable(const StackArgs& a, int grid);
int stack_lds_bytes(const Dims& dm, int ng, int n_layers);
hipError_t launch_stack(const StackArgs& a, int grid, hipStream_t st);
// Persistent kernel with a layer-ahead weight slot (chain.hip): the same
// arguments and exchange buffers; whether [l0, l1) on `grid` workgroups fits
// its plans. Its SwiGLU exchange of a layer with a down LoRA also carries 16
// partial A_down products from each of at most kChainSO workgroups (the ones
// owning shared-expert rows), after the shared expert's words; the LoRA A
// products of the gate/up follow them.
constexpr int kChainSO = 64;
bool chain_launchable(const StackArgs& a, int grid);
hipError_t launch_chain(const StackArgs& a, int grid, hipStream_t st);


// Wave-specialised persistent kernel (flow.hip): gate/up CUs [0, ng) and down
// CUs [ng, ng + nd), four compute and three loader waves each. The plan holds
// the work split, the exchange layout of a layer (8-byte words) and the LDS
// layout of both roles (byte offsets); host and kernel read the same plan.
constexpr int kFlowLds = 156 * 1024;
struct FlowPlan {
  int32_t ok, ng, nd, KX;
  int32_t direct;  // exchange words map to LDS without tables: 1 routed, 2 shared, 4 h
  // gate/up CUs [0, ngr) own the routed items (K*I, ipr_max at most each),
  // [ngr, ng) the shared expert's rows (ips_max at most each)
  int32_t ngr, ipr_max, ips_max, ipc_max;
  int32_t lbr, lhs;  // routed block 1 << lbr words; shared block 2 << lhs (g, then u)
  int32_t pairs_max, lba, nrc, ca0, hrn, hr_max, f2_max;
  // exchange words of a layer: h_out, SwiGLU outputs (routed blocks, shared
  // blocks, LoRA A-product blocks: one region), router logits, head hidden
  // and linear path, head logits
  int32_t o_xa, o_xb, xb_n, xb_s, xb_a, o_xr, o_xh1, o_xh2, xlayer;
  // gate/up CU LDS (bytes): layer slot (attention update, item rows, scales,
  // LoRA A row), router rows, head rows, head one-hot words, work
  int32_t g_at, g_gq, g_gs, g_ar, g_slot, g_rb, g_hb, g_hc, g_h, g_xn, g_xp, g_lg, g_rs, g_rt,
      g_end;
  // down CU LDS: layer slot (down rows, scales, LoRA B_down rows, attention
  // pairs), fc2 rows, work
  int32_t d_dq, d_ds, d_bd, d_at, d_slot, d_f2, d_sb, d_su, d_ax, d_hk, d_cs, d_v, d_co, d_ho,
      d_ab, d_lg, d_rs, d_rt, d_end;
};
struct FlowArgs {
  Dims dm;
  FlowPlan pl;
  const LayerDev* layers;
  int32_t L, l0, l1, token;
  uint32_t epoch;
  int32_t* route_idx;
  float* route_w;
  int32_t* exec_idx;
  float* exec_w;
  float* head_logits;
  uint16_t* x_trace;
  uint16_t* h;
  int32_t* sink_idx;
  float* sink_w;
  int32_t* flags;
  uint64_t* xbuf;   // [L][pl.xlayer] exchange words
  uint64_t* trace;  // optional [grid][L+1][kTracePoints] wall-clock stamps
};
bool flow_supported(const Dims& dm);
// Plan of one launch over nL layers on ng + nd workgroups (ok == 0: does not fit).
FlowPlan flow_plan(const Dims& dm, int ng, int nd, int nL);
// Default split of grid workgroups into gate/up and down CUs.
bool flow_default_roles(const Dims& dm, int grid, int nL, int& ng, int& nd);
hipError_t launch_flow(const FlowArgs& a, hipStream_t st);
// Zero the streaming kernel's exchange words (its packed words carry an
// 8-bit tag that comes round every 255 launches).
hipError_t launch_flow_clear(uint64_t* words, int64_t n, hipStream_t st);

// Staging: device-side slot policy for one layer, then a gather-copy of the
// missing bundles from (device-mapped) pinned host memory into HBM slots.
// Cross-layer hot-expert cache (stage.hip): largest cache and layers per call.
constexpr int kMaxCacheEntries = 4096;
constexpr int kMaxCacheLayers = 64;
hipError_t launch_cache_stage(int E, int C, int K, int layer0, int n_layers, int tick,
                              int32_t* slot_of, int32_t* owner, int32_t* stamp,
                              const int32_t* next, int32_t* copy_list, int32_t* n_copies,
                              unsigned long long* total, const char* host, int64_t host_stride,
                              char* cache, int64_t bundle, int32_t* flags, hipStream_t st);
hipError_t launch_stage(int E, int n_slots, int K, int n_layers, int32_t* slot_of,
                        int32_t* slot_expert, const int32_t* in_use, const int32_t* next,
                        int32_t* copy_list, int32_t* n_copies, unsigned long long* total,
                        const char* host, int64_t host_stride, char* hbm, int64_t hbm_stride,
                        int64_t bundle, int32_t* flags, hipStream_t st);
// Workgroups of the staging copy kernel (it occupies at most this many
// compute units).
constexpr int kCopyBlocks = 16;

}  // namespace smd
