// Batched tokens (B >= 16, decode chunks up to prefill-sized batches):
// grouped int4 GEMMs on MFMA.
//
// Source: "The Other Half of the Memory Wall" §3.1 Executor paths (batched
// chunks take the whole-layer path: experts are grouped so each expert's
// weights are read once for all tokens routed to it) and Math contract (one
// quantized kernel computing down(silu(gate(x)) * up(x)) per expert).
//
// Steps, all on the caller's stream:
//   1. k_mb_prep: the B*K (token, slot) entries sorted by expert (ascending
//      expert, then entry order) with the union of experts and each one's run;
//      x copied in the pair-permuted fp16 order the int4 dequant produces
//      ([x0 x4 x1 x5 x2 x6 x3 x7] per block of 8); LoRA A.x of the shared
//      expert's gate and up.
//   2. k_mb_gate_up: per (union member, 32 rows of I), eight waves: gate and
//      up rows, each over a quarter of the inputs. On
//      v_mfma_f32_32x32x16_f16 the member's tokens are operand A (rows) and
//      32 weight rows operand B, so each lane owns one weight row and its
//      group scales. int4 words are dequantised in registers to exact fp16
//      integers; each group of 64 inputs is accumulated on its own and scaled
//      in fp32 by the row's group scale (q*s is never rounded). SwiGLU and
//      the shared expert's LoRA B terms in the epilogue; fp32 output.
//   3. k_mb_down: per (union member, 128 output rows); the member's SwiGLU
//      outputs are staged in LDS as fp16 hi + lo under a power-of-two scale
//      per token (about 22 bits kept) and both halves go through the same
//      dequantised weights; also A_down . h of the shared expert.
//   4. k_mb_combine: y = sum_k w_k y_k + y_shared + down LoRA, in a fixed
//      order (no atomics, deterministic), rounded to fp16.
// Steps 2 and 3 run over a work list of tiles: one per 32 tokens of each
// union member (the MFMA column block), the shared expert's tiles first
// (dispatched first, they have the most tokens). A batch of any size B is
// one launch of each step; each expert's weights are read once per 32 of its
// tokens, so B = 32 reads every expert with routed tokens at most once.
// From 16 entries per expert on average the prefill kernels take over
// (k_pf_gate_up, k_pf_down: 64-token tiles, below). Every kernel has an
// affine-codec variant (AFF): unsigned nibbles, bf16 scales, and the bias
// added in fp32 as b times the token's sum over the group.

#include "gemv.h"
#include "internal.h"

namespace smd {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kCols = 32;  // tokens per MFMA column block
constexpr int kMaxR = 32;  // largest LoRA rank of the shared expert

__device__ __forceinline__ h8 as_h8(uint4 v) { return __builtin_bit_cast(h8, v); }

// Grouping tables in s.grp (int32): [0] union size, [1] number of tiles;
// then sorted entries (b*K + k) [BK]; expert, first sorted position and run
// length per union member [BK] each; the work tiles as (member, tile) pairs
// (member -1 = the shared expert, whose tokens are all B), one per up to 32
// of a member's tokens.
struct Groups {
  int32_t* n_union;
  int32_t* n_tiles;
  int32_t* sorted;
  int32_t* uexp;
  int32_t* ustart;
  int32_t* ucount;
  int32_t* tiles;
};

__host__ __device__ inline Groups groups(int32_t* g, int BK) {
  return {g, g + 1, g + 2, g + 2 + BK, g + 2 + 2 * BK, g + 2 + 3 * BK, g + 2 + 4 * BK};
}

// Work tile descriptors after the tables above (16-byte aligned), one int4
// per tile of the launch grids (ny of them): member (-1 the shared expert),
// first entry, token count (0: no tile), and the member's pool entry (-1
// when its id does not resolve). k_mb_prep writes them where it forms the
// tiles, so a gate/up or down workgroup reads everything it needs before
// its weight loads in one load.
__host__ __device__ inline int4* tile_descs(int32_t* g, int BK, int ny) {
  return reinterpret_cast<int4*>(g + batched_desc_offset(BK, ny));
}

struct MbArgs {
  Dims dm;
  Pool pool;
  SharedW sh;
  int B;
  const uint16_t* x;     // [B][d] input, natural order
  uint16_t* xp;          // [B][d] pair-permuted copy
  int32_t* grp;
  int tile;              // tokens per work tile: 32 (chunk kernels) or 64 (prefill kernels)
  int ny;                // work tiles the launch grids cover (an upper bound on the tiles)
  const int32_t* idx;    // [B][K]
  const float* w;        // [B][K]
  float* ax;             // [B][3*rmax] LoRA A products (down in slot 2)
  float* axp;            // [n_sl][B][2*rmax] gate/up LoRA A products per input slice
  int n_sl;              // input slices (divides d/64)
  int rmax;
  float* H;              // [B][K+1][imax] SwiGLU outputs
  float* Y;              // [B][K+1][d] per-slot down outputs
  float* xsum;           // affine codec: [B][d/64] sums of each token's x per input group
  int ctok;              // tokens per combine workgroup
  uint16_t* y;           // [B][d]
  int32_t* flags;
};

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off);
    if (l >= off) v += t;
  }
  return v;
}

// Block 0 of k_mb_prep: the B*K entries sorted by expert (ascending expert
// id, then entry order), the union of experts with each member's run, and
// the work tiles. Integer counting only, so nothing depends on thread timing.
// Each wave owns a contiguous quarter of the entries:
//   1. it counts its quarter per expert (LDS atomics: order-independent);
//   2. thread t takes experts 2t and 2t+1: offsets, union positions and tile
//      positions by prefix sums, and each wave's cursor for them (the
//      expert's offset plus its entries in earlier quarters);
//   3. each wave walks its quarter 64 entries at a time, in order, with no
//      block barrier: lanes that hold the same expert find each other with
//      one ballot per bit of the id, an entry lands at the wave's cursor plus
//      its rank among them, and their first lane advances the cursor.
// kMaxE = 512 ids take nine bits. Each lane keeps kGrpDepth loads in flight.
constexpr int kGrpDepth = 16;

__device__ void group_entries(const MbArgs& a) {
  __shared__ int wcnt[4][kMaxE];  // counts of wave w's quarter, then its cursors
  __shared__ int wtot[3][4];
  const int E = a.dm.E, K = a.dm.K, BK = a.B * K;
  const Groups g = groups(a.grp, BK);
  const int t = threadIdx.x, nt = blockDim.x;
  const int wv = t >> 6, lane = t & 63;
  const int cpw = ((BK + 63) / 64 + 3) / 4;  // 64-entry chunks per quarter
  const int q0 = min(BK, wv * cpw * 64), q1 = min(BK, (wv + 1) * cpw * 64);
  for (int e = t; e < 4 * kMaxE; e += nt) (&wcnt[0][0])[e] = 0;
  __syncthreads();
  for (int i0 = q0 + lane; i0 < q1; i0 += kGrpDepth * 64) {
    int ev[kGrpDepth];
#pragma unroll
    for (int u = 0; u < kGrpDepth; ++u) ev[u] = i0 + 64 * u < q1 ? a.idx[i0 + 64 * u] : -2;
#pragma unroll
    for (int u = 0; u < kGrpDepth; ++u) {
      if (ev[u] == -2) continue;
      if (ev[u] < 0 || ev[u] >= E)
        atomicOr(&a.flags[FLAG_RANGE], 1);
      else
        atomicAdd(&wcnt[wv][ev[u]], 1);
    }
  }
  __syncthreads();
  int cw0[4], cw1[4], c0 = 0, c1 = 0;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    cw0[v] = wcnt[v][2 * t];
    cw1[v] = wcnt[v][2 * t + 1];
    c0 += cw0[v];
    c1 += cw1[v];
  }
  const int n0 = (c0 + a.tile - 1) / a.tile, n1 = (c1 + a.tile - 1) / a.tile;
  int ps = wave_incl_scan(c0 + c1);
  int pu = wave_incl_scan((c0 > 0) + (c1 > 0));
  int pt = wave_incl_scan(n0 + n1);
  if (lane == 63) {
    wtot[0][wv] = ps;
    wtot[1][wv] = pu;
    wtot[2][wv] = pt;
  }
  __syncthreads();  // also: every count has been read before it becomes a cursor
  for (int v = 0; v < wv; ++v) {
    ps += wtot[0][v];
    pu += wtot[1][v];
    pt += wtot[2][v];
  }
  const int n_sh = a.sh.present ? (a.B + a.tile - 1) / a.tile : 0;
  const int off0 = ps - c0 - c1;
  int u = pu - (c0 > 0) - (c1 > 0);
  int tp = n_sh + pt - n0 - n1;
  int4* td = tile_descs(a.grp, BK, a.ny);
  if (c0) {
    g.uexp[u] = 2 * t;
    g.ustart[u] = off0;
    g.ucount[u] = c0;
    const int ent = (int)resolve_entry(a.pool, E, 2 * t);
    for (int j = 0; j < n0; ++j) {
      g.tiles[2 * tp] = u;
      g.tiles[2 * tp + 1] = j;
      td[tp] = make_int4(u, off0 + a.tile * j, min(a.tile, c0 - a.tile * j), ent);
      ++tp;
    }
    ++u;
  }
  if (c1) {
    g.uexp[u] = 2 * t + 1;
    g.ustart[u] = off0 + c0;
    g.ucount[u] = c1;
    const int ent = (int)resolve_entry(a.pool, E, 2 * t + 1);
    for (int j = 0; j < n1; ++j) {
      g.tiles[2 * tp] = u;
      g.tiles[2 * tp + 1] = j;
      td[tp] = make_int4(u, off0 + c0 + a.tile * j, min(a.tile, c1 - a.tile * j), ent);
      ++tp;
    }
  }
  for (int j = t; j < n_sh; j += blockDim.x) {
    g.tiles[2 * j] = -1;
    g.tiles[2 * j + 1] = j;
    td[j] = make_int4(-1, a.tile * j, min(a.tile, a.B - a.tile * j), 0);
  }
  // tiles of the grids past the last one: no work
  for (int y = n_sh + (wtot[2][0] + wtot[2][1]) + (wtot[2][2] + wtot[2][3]) + t; y < a.ny;
       y += blockDim.x)
    td[y] = make_int4(0, 0, 0, -1);
  if (t == blockDim.x - 1) {
    *g.n_union = pu;
    *g.n_tiles = n_sh + pt;
  }
  {
    int o0 = off0, o1 = off0 + c0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      wcnt[v][2 * t] = o0;
      wcnt[v][2 * t + 1] = o1;
      o0 += cw0[v];
      o1 += cw1[v];
    }
  }
  __syncthreads();
  int* cur = wcnt[wv];
  const uint64_t below = (1ull << lane) - 1;
  for (int c = q0; c < q1; c += kGrpDepth * 64) {
    int ev[kGrpDepth];
#pragma unroll
    for (int v = 0; v < kGrpDepth; ++v)
      ev[v] = c + 64 * v + lane < q1 ? a.idx[c + 64 * v + lane] : -1;
#pragma unroll
    for (int v = 0; v < kGrpDepth; ++v) {
      if (c + 64 * v >= q1) break;  // uniform over the wave
      const int i = c + 64 * v + lane;
      const int e = ev[v] >= 0 && ev[v] < E ? ev[v] : -1;
      uint64_t same = __ballot(e >= 0);
#pragma unroll
      for (int bit = 0; bit < 9; ++bit) {
        const bool set = (e >> bit) & 1;
        const uint64_t m = __ballot(set);
        same &= set ? m : ~m;
      }
      const int rank = __popcll(same & below), n_same = __popcll(same);
      if (e >= 0) g.sorted[cur[e] + rank] = i;
      // every lane has read its cursor before the first lanes advance them
      __builtin_amdgcn_wave_barrier();
      if (e >= 0 && rank == 0) cur[e] += n_same;
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// Blocks 0..B-1 of k_mb_prep: token b's pair-permuted x; for the affine
// codec also its sum over each 64-input group (fp32 over the fp16 values:
// chunk c of 8 values is thread c, and a group's 8 chunks are 8 adjacent
// lanes).
__device__ void prep_token(const MbArgs& a, int b) {
  const int d = a.dm.d;
  const uint16_t* xb = a.x + (int64_t)b * d;
  for (int c0 = 0; c0 < d / 8; c0 += blockDim.x) {  // uniform over the block
    const int c = c0 + threadIdx.x;
    float sum = 0.0f;
    if (c < d / 8) {
      const uint4 v = ldg(reinterpret_cast<const uint4*>(xb + 8 * c));
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint16_t e[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        e[2 * q] = (uint16_t)(w[q] & 0xFFFF);
        e[2 * q + 1] = (uint16_t)(w[q] >> 16);
      }
      *reinterpret_cast<uint4*>(a.xp + (int64_t)b * d + 8 * c) =
          make_uint4(e[0] | ((uint32_t)e[4] << 16), e[1] | ((uint32_t)e[5] << 16),
                     e[2] | ((uint32_t)e[6] << 16), e[3] | ((uint32_t)e[7] << 16));
#pragma unroll
      for (int q = 0; q < 8; ++q) sum += h2f(e[q]);
    }
    if (a.dm.affine) {
      sum = group_sum<8>(sum);
      if (c < d / 8 && (c & 7) == 0) a.xsum[(int64_t)b * (d / 64) + (c >> 3)] = sum;
    }
  }
}

// LoRA blocks of k_mb_prep: partial (A_gate x_b, A_up x_b) over one slice of
// the inputs for 32 tokens b0.. per block, on MFMA: tokens are operand A
// (rows), the 2r LoRA rows operand B (columns, gate rows then up rows, 32 per
// column block); the four waves take a quarter of the slice each and meet in
// LDS (fixed order). The slices are summed in order by the gate/up step.
// Products of fp16 values are exact; sums are fp32.
__device__ void prep_lora(const MbArgs& a, int lb) {
  __shared__ float red[4][16][64];
  const int d = a.dm.d, r = a.dm.r, b0 = (lb / a.n_sl) * kCols, sl = lb % a.n_sl;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, n = l & 31, kh = l >> 5;
  const int nb = min(kCols, a.B - b0);
  const int q = d / a.n_sl / 4, k0 = sl * (d / a.n_sl) + wave * q;
  float* out = a.axp + (int64_t)sl * a.B * 2 * a.rmax;
  // token rows past the batch read a valid row (their outputs are not stored)
  const uint16_t* xrow = a.x + (int64_t)(b0 + (n < nb ? n : nb - 1)) * d + k0 + 8 * kh;
  for (int cb = 0; cb < 2 * r; cb += 32) {
    const int o = cb + n;
    const bool col_ok = o < 2 * r;
    const uint16_t* arow =
        (o < r ? a.sh.ag : a.sh.au) + (int64_t)((col_ok ? o : 0) % r) * d + k0 + 8 * kh;
    f32x16 acc = {};
#pragma unroll 4
    for (int k = 0; k < q; k += 16) {
      const uint4 xv = ldg(reinterpret_cast<const uint4*>(xrow + k));
      const uint4 av = col_ok ? ldg(reinterpret_cast<const uint4*>(arow + k)) : make_uint4(0, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(xv), as_h8(av), acc, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) red[wave][i][l] = acc[i];
    __syncthreads();
    // thread (register i, lane l) sums the four quarters in order
    for (int e = threadIdx.x; e < 16 * 64; e += blockDim.x) {
      const int i = e >> 6, ll = e & 63;
      const int t = 8 * (i >> 2) + 4 * (ll >> 5) + (i & 3), oo = cb + (ll & 31);
      if (t < nb && oo < 2 * r) {
        const float v = (red[0][i][ll] + red[1][i][ll]) + (red[2][i][ll] + red[3][i][ll]);
        out[(int64_t)(b0 + t) * 2 * a.rmax + oo] = v;
      }
    }
    __syncthreads();
  }
}

// Grid: the grouping block first (the longest, so it starts at once), B
// token blocks, then ceil(B/32) x n_sl LoRA blocks when the shared expert has
// LoRA.
__global__ __launch_bounds__(256) void k_mb_prep(MbArgs a) {
  const int bx = blockIdx.x;
  if (bx == 0)
    group_entries(a);
  else if (bx <= a.B)
    prep_token(a, bx - 1);
  else
    prep_lora(a, bx - a.B - 1);
}

// Eight int4 weights of one word as exact fp16 integers, in the order
// q0 q4 q1 q5 q2 q6 q3 q7 (matching the pair-permuted activations); AFF:
// unsigned nibbles (the affine codec) rather than two's complement.
template <bool AFF = false>
__device__ __forceinline__ h8 q4_to_h8(uint32_t w) {
  f16x2 p0, p1, p2, p3;
  q4_pairs<AFF>(w, p0, p1, p2, p3);
  h8 r;
  r[0] = p0.x; r[1] = p0.y; r[2] = p1.x; r[3] = p1.y;
  r[4] = p2.x; r[5] = p2.y; r[6] = p3.x; r[7] = p3.y;
  return r;
}

__device__ __forceinline__ uint32_t word(const uint4& v, int j) {
  return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// Pins an accumulator in registers at this point: without it the compiler
// sinks the per-group scale-adds into the conditional stores at the end and
// keeps every group's partial alive until then.
__device__ __forceinline__ void keep(f32x16& v) { asm volatile("" : "+v"(v)); }

// MFMA 32x32x16 layout with the chunk's tokens as operand A and 32 weight rows
// as operand B: lane l supplies token row l%32 and weight row l%32 over the
// k-slice 8*(l/32)..+8; accumulator register r of lane l holds token row
// tok_row(r, l/32) of weight row l%32.
__device__ __forceinline__ int tok_row(int r, int kh) { return 8 * (r >> 2) + 4 * kh + (r & 3); }

// A group scale or bias: fp16 (symmetric codec) or bf16 (affine codec).
template <bool AFF>
__device__ __forceinline__ float sb2f(uint16_t v) { return AFF ? bf2f(v) : h2f(v); }

// acc[r] += s * c[r] for the NR registers that can hold a valid token: count
// tokens occupy rows 0..count-1, i.e. registers r < NR = 4*ceil(count/8).
template <int NR>
__device__ __forceinline__ void scale_add(f32x16& acc, const f32x16& c, float s) {
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r] = fmaf(s, c[r], acc[r]);
}

// Multiply-accumulate of one wave: NG groups of 64 inputs, weights wv (one
// word per lane per MFMA), activations xv of the lane's token row
// (pair-permuted fp16), group scales sv.
// Groups i0 .. i0 + NH - 1 of the NG, accumulated into acc; the activations
// xv of those NH groups only.
template <int NG, int NH, int NR, bool AFF>
__device__ __forceinline__ void gu_mma(f32x16& acc, const uint4 (&wv)[NG], const float (&sv)[NG],
                                       const uint4 (&xv)[NH][4], int i0) {
#pragma unroll
  for (int i = 0; i < NH; ++i) {
    f32x16 c = {};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      c = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(xv[i][j]),
                                                q4_to_h8<AFF>(word(wv[i0 + i], j)), c, 0, 0, 0);
    scale_add<NR>(acc, c, sv[i0 + i]);
    keep(acc);
  }
}

// Down multiply-accumulate: hi and lo activation rows (in LDS) through the
// same dequantised weights.
template <int NG, int NR, bool AFF>
__device__ __forceinline__ f32x16 dn_mma(const uint4 (&wq)[NG], const float (&sc)[NG],
                                         const uint16_t* hrow, const uint16_t* lrow) {
  f32x16 acc = {};
#pragma unroll
  for (int i = 0; i < NG; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    f32x16 c = {};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 hv = *reinterpret_cast<const uint4*>(hrow + 64 * i + 8 * j);
      const uint4 lv = *reinterpret_cast<const uint4*>(lrow + 64 * i + 8 * j);
      const h8 w8 = q4_to_h8<AFF>(word(wq[i], j));
      c = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(hv), w8, c, 0, 0, 0);
      c = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(lv), w8, c, 0, 0, 0);
    }
    scale_add<NR>(acc, c, sc[i]);
    keep(acc);
  }
  return acc;
}

// Token and output slot of token row t of a tile: the shared expert's tiles
// run over tokens start.., a member's over its sorted entries start...
__device__ __forceinline__ void entry_of(const MbArgs& a, bool shared, int start, int t, int& b,
                                         int& k) {
  const int K = a.dm.K;
  if (shared) {
    b = start + t;
    k = K;
  } else {
    const Groups g = groups(a.grp, a.B * K);
    const int ent = g.sorted[start + t];
    b = ent / K;
    k = ent % K;
  }
}

// Work tile y: the shared expert (dispatched first, it has the most tokens)
// or a union member, with its first entry and token count (<= a.tile).
// u: the member's pool entry (-1 when its id did not resolve; 0 for the
// shared expert). One 16-byte read of the tile's descriptor.
__device__ __forceinline__ bool tile_of(const MbArgs& a, int y, bool& shared, int& u, int& start,
                                        int& count) {
  const uint4 v = ldg(reinterpret_cast<const uint4*>(tile_descs(a.grp, a.B * a.dm.K, a.ny) + y));
  if ((int)v.z <= 0) return false;
  shared = (int)v.x < 0;
  start = (int)v.y;
  count = (int)v.z;
  u = (int)v.w;
  return true;
}

// Work item of this workgroup in the (row block, tile) grid. The natural
// order is kept: renumbering so that one XCD takes all row blocks of a tile
// (sharing its activations in that XCD's L2) measured slower, since the
// shared expert's full tiles then crowd onto one XCD.
__device__ __forceinline__ bool tile_block(const MbArgs& a, int& bx, bool& shared, int& u,
                                           int& start, int& count) {
  bx = blockIdx.x;
  return tile_of(a, blockIdx.y, shared, u, start, count);
}

// Gate/up of one union member (or the shared expert) for 32 rows. Eight
// waves: waves 0-3 the gate rows, 4-7 the up rows, each over a quarter of
// the inputs (NG groups); partials meet in LDS. A wave issues all its loads
// (weight words, scales, activations of its valid token rows) before the
// first multiply. AFF (affine codec): each wave adds b * (the token's sum of
// x over the group) for its groups, from sums staged in LDS.
// (The affine variant's bias terms need more registers: it keeps one
// workgroup per compute unit.)
constexpr int kXsTok = 8;            // tiles of up to this many tokens stage x in LDS
typedef __attribute__((address_space(3))) void lptr_v;
typedef __attribute__((address_space(1))) void gptr_v;
constexpr int kXsRow = 2048 + 8;     // staged row stride (fp16; 16-byte pad against bank conflicts)

template <int NG, bool AFF>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(AFF ? 2 : 4)))
void k_mb_gate_up(MbArgs a) {
  __shared__ float red[2][4][16][64];
  __shared__ float axs[kCols][2][kMaxR];
  __shared__ float xss[AFF ? kCols : 1][32];  // [tile token][input group]
  __shared__ uint16_t xsl[kXsTok * kXsRow];  // the tile's activations (count <= kXsTok)
  const Dims& dm = a.dm;
  const int K = dm.K, d = dm.d;
  const int imax = dm.I > dm.Is ? dm.I : dm.Is;
  bool shared;
  int u, start, count;
  int bx;
  if (!tile_block(a, bx, shared, u, start, count)) return;
  const int m0 = bx * 32;
  if (m0 >= (shared ? dm.Is : dm.I)) return;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, n = l & 31, kh = l >> 5;
  const int mat = wave >> 2, quarter = wave & 3;  // 0 gate, 1 up
  const uint32_t* wq;
  const uint16_t* ws;
  const uint16_t* wb = nullptr;
  const bool lora = shared && a.sh.ag;
  if (shared) {
    wq = mat ? a.sh.up.q : a.sh.gate.q;
    ws = mat ? a.sh.up.s : a.sh.gate.s;
    if (AFF) wb = mat ? a.sh.up.b : a.sh.gate.b;
    if (lora) {  // LoRA A products of this tile's tokens: the slices in order
      for (int i = threadIdx.x; i < count * 2 * dm.r; i += blockDim.x) {
        const int tt = i / (2 * dm.r), j = i % (2 * dm.r);
        const float* p = a.axp + (int64_t)(start + tt) * 2 * a.rmax + j;
        float v = 0.0f;
        for (int sl = 0; sl < a.n_sl; ++sl) v += p[(int64_t)sl * a.B * 2 * a.rmax];
        axs[tt][j / dm.r][j % dm.r] = v;
      }
    }
  } else {
    const int64_t ent = u;
    if (ent < 0) {
      if (threadIdx.x == 0) atomicOr(&a.flags[FLAG_RANGE], 1);
      return;
    }
    const Q4& m = mat ? a.pool.up : a.pool.gate;
    wq = (const uint32_t*)entry_ptr(m.q, ent, a.pool.stride_q);
    ws = (const uint16_t*)entry_ptr(m.s, ent, a.pool.stride_s);
    if (AFF) wb = (const uint16_t*)entry_ptr(m.b, ent, a.pool.stride_s);
  }
  const int ngs = d / dm.G, g0 = quarter * NG, wpr = d / 8;
  if (AFF) {
    for (int i = threadIdx.x; i < count * ngs; i += blockDim.x) {
      const int tt = i / ngs, gg = i % ngs;
      int b, k;
      entry_of(a, shared, start, tt, b, k);
      xss[tt][gg] = a.xsum[(int64_t)b * ngs + gg];
    }
    __syncthreads();
  }
  const int nr = 4 * ((count + 7) >> 3);
  const uint32_t* qrow = wq + (int64_t)(m0 + n) * wpr + 4 * kh;
  const uint16_t* srow = ws + (int64_t)(m0 + n) * ngs;
  // Small tiles (most of a decode chunk's) stage their token rows in LDS
  // (direct-to-LDS loads, issued before the weight loads), so a wave reads
  // its activations there instead of loading them per lane.
  const bool xlds = count <= kXsTok && d + 8 <= kXsRow;
  // Token rows past count read a valid row (the last one): their outputs
  // land in accumulator rows that are never stored.
  int bt, kt;
  if (!xlds) entry_of(a, shared, start, n < count ? n : count - 1, bt, kt);
  const uint16_t* xrow = xlds ? nullptr : a.xp + (int64_t)bt * d + 32 * kh + 64 * g0;
  if (xlds) {
    // each wave stages its own quarter of every token row (the gate and the
    // up wave of a quarter write the same bytes), so a wave waits only for
    // its own loads: one instruction per row, 16 bytes a lane, issued before
    // the weight words
    const int qw = 64 * NG;  // inputs of a quarter
    for (int tt = 0; tt < count; ++tt) {
      int b, k;
      entry_of(a, shared, start, tt, b, k);
      if (8 * l < qw)
        __builtin_amdgcn_global_load_lds((gptr_v*)(a.xp + (int64_t)b * d + qw * quarter + 8 * l),
                                         (lptr_v*)(xsl + tt * kXsRow + qw * quarter), 16, 0, 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  uint4 wv[NG];
  float sv[NG], bv[NG];
#pragma unroll
  for (int i = 0; i < NG; ++i) wv[i] = ldg(reinterpret_cast<const uint4*>(qrow + 8 * (g0 + i)));
#pragma unroll
  for (int i = 0; i < NG; ++i) sv[i] = sb2f<AFF>(ldg(srow + g0 + i));
  if (AFF) {
    const uint16_t* brow = wb + (int64_t)(m0 + n) * ngs;
#pragma unroll
    for (int i = 0; i < NG; ++i) bv[i] = bf2f(ldg(brow + g0 + i));
  }
  // the activations in two halves of the quarter's groups (each half's loads
  // together), which keeps a wave within 128 registers: two workgroups share
  // a compute unit, so one's loads overlap the other's MFMAs and epilogue
  constexpr int NH = NG / 2;
  f32x16 acc = {};
  if (xlds) {
    // the staged rows are in once at most NG loads (the weight words issued
    // after them) are outstanding; the MFMAs then wait for each group's word
    __builtin_amdgcn_s_waitcnt(0x0F70 | NG);
    const uint16_t* xl = xsl + (n < count ? n : count - 1) * kXsRow + 32 * kh + 64 * g0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 xv[NH][4];
#pragma unroll
      for (int i = 0; i < NH; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xv[i][j] = *reinterpret_cast<const uint4*>(xl + 64 * (NH * h + i) + 8 * j);
      gu_mma<NG, NH, 16, AFF>(acc, wv, sv, xv, NH * h);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint4 xv[NH][4];
#pragma unroll
      for (int i = 0; i < NH; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xv[i][j] = ldg(reinterpret_cast<const uint4*>(xrow + 64 * (NH * h + i) + 8 * j));
      // one variant for all counts: a second (fewer registers scaled) costs
      // the register allocator more than it saves
      gu_mma<NG, NH, 16, AFF>(acc, wv, sv, xv, NH * h);
    }
  }
  if (AFF) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float* xsr = xss[tok_row(r, kh)] + g0;  // rows past count: never stored
      float bsum = 0.0f;
#pragma unroll
      for (int i = 0; i < NG; ++i) bsum = fmaf(bv[i], xsr[i], bsum);
      acc[r] += bsum;
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (r < nr) red[mat][quarter][r][l] = acc[r];
  __syncthreads();
  // wave w finishes registers r = w, w+8 (fixed summation order)
  const float c = dm.lora_scale;
  const int row = m0 + n;
  for (int r = wave; r < nr; r += 8) {
    const int t = tok_row(r, kh);
    if (t >= count) continue;
    float gg = (red[0][0][r][l] + red[0][1][r][l]) + (red[0][2][r][l] + red[0][3][r][l]);
    float uu = (red[1][0][r][l] + red[1][1][r][l]) + (red[1][2][r][l] + red[1][3][r][l]);
    int b, k;
    entry_of(a, shared, start, t, b, k);
    if (lora) {
      float lg = 0.0f, lu = 0.0f;
      for (int q = 0; q < dm.r; q += 8) {
        const uint4 bgv = ldg(reinterpret_cast<const uint4*>(a.sh.bg + (int64_t)row * dm.r + q));
        const uint4 buv = ldg(reinterpret_cast<const uint4*>(a.sh.bu + (int64_t)row * dm.r + q));
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const f16x2 g2 = as_h2(word(bgv, p)), u2 = as_h2(word(buv, p));
          lg = fmaf((float)g2.x, axs[t][0][q + 2 * p], lg);
          lg = fmaf((float)g2.y, axs[t][0][q + 2 * p + 1], lg);
          lu = fmaf((float)u2.x, axs[t][1][q + 2 * p], lu);
          lu = fmaf((float)u2.y, axs[t][1][q + 2 * p + 1], lu);
        }
      }
      gg = fmaf(c, lg, gg);
      uu = fmaf(c, lu, uu);
    }
    a.H[((int64_t)b * (K + 1) + k) * imax + row] = silu(gg) * uu;
  }
}

// Down projection. A workgroup takes kDnWaves * 32 output rows of one union
// member (or the shared expert); its waves take 32 rows each over all NG
// input groups (eight waves: the staging below is shared by twice the rows,
// and at up to 128 registers two workgroups still share a compute unit). The member's fp32 SwiGLU outputs (count tokens x NG*64) are staged
// once in LDS as fp16 hi + lo under a power-of-two scale per token (about 22
// bits of each value kept); hi and lo then go through the same dequantised
// weights. Workgroups of the shared expert also form A_down . h for the down
// LoRA, two tokens each. AFF (affine codec): the staging also forms each
// token's sum of hi + lo over every input group, and the epilogue adds
// b * that sum per group.
constexpr int kDnPad = 8;    // fp16 padding per staged row (spreads LDS banks)
constexpr int kDnWaves = 8;  // waves (32 output rows each) per workgroup

template <int NG, bool AFF>
__global__ __launch_bounds__(64 * kDnWaves) __attribute__((amdgpu_waves_per_eu(AFF ? 2 : 4)))
void k_mb_down(MbArgs a) {
  extern __shared__ __align__(16) uint16_t hs[];  // [count][2][NG*64 + kDnPad]
  __shared__ float hx[kCols];                      // per-token power-of-two scale
  __shared__ float hss[AFF ? kCols : 1][8];        // [token][input group] sums of hi + lo
  constexpr int nin = NG * 64, stride = nin + kDnPad, wpr = NG * 8;
  const Dims& dm = a.dm;
  const int K = dm.K, d = dm.d;
  const int imax = dm.I > dm.Is ? dm.I : dm.Is;
  bool shared;
  int u, start, count;
  int bx;
  if (!tile_block(a, bx, shared, u, start, count)) return;
  const uint32_t* dq;
  const uint16_t* ds;
  const uint16_t* db = nullptr;
  if (shared) {
    dq = a.sh.down.q; ds = a.sh.down.s;
    if (AFF) db = a.sh.down.b;
  } else {
    const int64_t ent = u;
    if (ent < 0) return;  // flagged by the gate/up step
    dq = (const uint32_t*)entry_ptr(a.pool.down.q, ent, a.pool.stride_q);
    ds = (const uint16_t*)entry_ptr(a.pool.down.s, ent, a.pool.stride_s);
    if (AFF) db = (const uint16_t*)entry_ptr(a.pool.down.b, ent, a.pool.stride_s);
  }
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, n = l & 31, kh = l >> 5;
  const int m0 = (bx * kDnWaves + wave) * 32;
  const bool rows_ok = m0 < d;
  uint4 wq[NG];
  float sc[NG], bd[NG];
  if (rows_ok) {
    const uint32_t* qrow = dq + (int64_t)(m0 + n) * wpr + 4 * kh;
    const uint16_t* srow = ds + (int64_t)(m0 + n) * NG;
#pragma unroll
    for (int i = 0; i < NG; ++i) wq[i] = ldg(reinterpret_cast<const uint4*>(qrow + 8 * i));
#pragma unroll
    for (int i = 0; i < NG; ++i) sc[i] = sb2f<AFF>(ldg(srow + i));
    if (AFF) {
      const uint16_t* brow = db + (int64_t)(m0 + n) * NG;
#pragma unroll
      for (int i = 0; i < NG; ++i) bd[i] = bf2f(ldg(brow + i));
    }
  }
  // stage: wave w takes tokens w, w+4, ...; lane l the 8 values of chunk l
  for (int t = wave; t < count; t += kDnWaves) {
    int b, k;
    entry_of(a, shared, start, t, b, k);
    const float* h = a.H + ((int64_t)b * (K + 1) + k) * imax + 8 * l;
    float v[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if (l < NG * 8) {
      const float4 v0 = *reinterpret_cast<const float4*>(h);
      const float4 v1 = *reinterpret_cast<const float4*>(h + 4);
      v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
      v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    const int e = hilo_exponent(wave_max_rows(m));
    const float inv = ldexpf(1.0f, -e);
    float psum = 0.0f;
    if (l < NG * 8) {
      uint16_t hi[8], lo[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        f16 th, tl;
        split_hilo(v[i], inv, th, tl);
        hi[i] = __builtin_bit_cast(uint16_t, th);
        lo[i] = __builtin_bit_cast(uint16_t, tl);
        if (AFF) psum += (float)th + (float)tl;
      }
      // pair-permuted order [0 4 1 5 2 6 3 7]
      *reinterpret_cast<uint4*>(hs + (t * 2) * stride + 8 * l) =
          make_uint4(hi[0] | ((uint32_t)hi[4] << 16), hi[1] | ((uint32_t)hi[5] << 16),
                     hi[2] | ((uint32_t)hi[6] << 16), hi[3] | ((uint32_t)hi[7] << 16));
      *reinterpret_cast<uint4*>(hs + (t * 2 + 1) * stride + 8 * l) =
          make_uint4(lo[0] | ((uint32_t)lo[4] << 16), lo[1] | ((uint32_t)lo[5] << 16),
                     lo[2] | ((uint32_t)lo[6] << 16), lo[3] | ((uint32_t)lo[7] << 16));
    }
    if (AFF) {
      psum = group_sum<8>(psum);  // lanes 8g .. 8g+7 hold group g's chunks
      if (l < NG * 8 && (l & 7) == 0) hss[t][l >> 3] = psum;
    }
    if (l == 0) hx[t] = ldexpf(1.0f, e);
  }
  if (shared && a.sh.ad) {
    // A_down . h_shared[t] for tokens t = bx, bx + gridDim.x, ...;
    // wave w takes ranks q = w, w+4, ...
    for (int t = bx; t < count; t += gridDim.x) {
      const int b = start + t;
      const float* h = a.H + ((int64_t)b * (K + 1) + K) * imax + 8 * l;
      float v[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
      if (l < NG * 8) {
        const float4 v0 = *reinterpret_cast<const float4*>(h);
        const float4 v1 = *reinterpret_cast<const float4*>(h + 4);
        v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
        v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
      }
      for (int q = wave; q < dm.r; q += kDnWaves) {
        float sacc = 0.0f;
        if (l < NG * 8) {
          const uint4 av = ldg(reinterpret_cast<const uint4*>(a.sh.ad + (int64_t)q * nin + 8 * l));
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const f16x2 ah = as_h2(word(av, p));
            sacc = fmaf((float)ah.x, v[2 * p], sacc);
            sacc = fmaf((float)ah.y, v[2 * p + 1], sacc);
          }
        }
        sacc = wave_sum_rows(sacc);
        if (l == 0) a.ax[(int64_t)b * 3 * a.rmax + 2 * a.rmax + q] = sacc;
      }
    }
  }
  __syncthreads();
  if (!rows_ok) return;
  const int nr = 4 * ((count + 7) >> 3);
  // token rows past count read the last valid row (never stored)
  const int tc = n < count ? n : count - 1;
  const uint16_t* hrow = hs + (tc * 2) * stride + 32 * kh;
  const uint16_t* lrow = hrow + stride;
  f32x16 acc;
  if (nr == 4)
    acc = dn_mma<NG, 4, AFF>(wq, sc, hrow, lrow);
  else
    acc = dn_mma<NG, 16, AFF>(wq, sc, hrow, lrow);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int t = tok_row(r, kh);
    if (r < nr && t < count) {
      int b, k;
      entry_of(a, shared, start, t, b, k);
      const int64_t slot = (int64_t)b * (K + 1) + k;
      float v = acc[r];
      if (AFF) {
#pragma unroll
        for (int i = 0; i < NG; ++i) v = fmaf(bd[i], hss[t][i], v);
      }
      a.Y[slot * d + m0 + n] = v * hx[t];
    }
  }
}

// y[b] = sum_k w_k y_k + y_shared + down LoRA, in a fixed order (no atomics),
// rounded to fp16. Grid (ceil(B / ctok), ceil(d / 1024)); thread j takes
// columns 4j..4j+3 of ctok consecutive tokens (16-byte loads): it reads the
// four columns' down-LoRA rows once (16-byte words) and then each token's
// slot outputs. ctok = 1 for small batches (more workgroups), more for large
// ones (fewer reads of the LoRA rows).
constexpr int kCombTokMax = 4;
constexpr int kCombK = 8;  // routed slots a token's loads cover (K <= 8)

// Token b's routed slot outputs (four columns from j0), its shared slot's and
// its K weights, all issued together with no condition, so one memory latency
// covers them. Slots k >= K read the shared slot's row and weights k >= K the
// last one: in bounds (Y holds K + 1 rows per token, w K), never used.
struct CombRow {
  float4 y[kCombK];
  float4 ysh;
  float w[kCombK];
};

__device__ __forceinline__ void comb_load(const MbArgs& a, int b, int j0, CombRow& r) {
  const int K = a.dm.K, d = a.dm.d;
  const float* yb = a.Y + (int64_t)b * (K + 1) * d + j0;
#pragma unroll
  for (int k = 0; k < kCombK; ++k)
    r.y[k] = *reinterpret_cast<const float4*>(yb + (int64_t)(k < K ? k : K) * d);
  r.ysh = *reinterpret_cast<const float4*>(yb + (int64_t)K * d);
#pragma unroll
  for (int k = 0; k < kCombK; ++k) r.w[k] = a.w[b * K + (k < K ? k : K - 1)];
}

__global__ __launch_bounds__(256) void k_mb_combine(MbArgs a) {
  __shared__ int ok[kCombTokMax][kCombK];
  __shared__ float axd[kCombTokMax][kMaxR];
  const Dims& dm = a.dm;
  const int K = dm.K, d = dm.d, b0 = blockIdx.x * a.ctok;
  const int nb = min(a.ctok, a.B - b0);
  const bool lora = a.sh.present && a.sh.bd;
  const int j0 = 4 * (blockIdx.y * blockDim.x + threadIdx.x);
  // d % 128 == 0: a thread's four columns are all in range or all out; the
  // loads of out-of-range threads read column 0 and are dropped
  const bool act = j0 < d;
  const int jl = act ? j0 : 0;
  // the first token's rows and the LoRA rows do not depend on the tables
  // below: issued first, so their latency overlaps the table lookups
  CombRow row;
  comb_load(a, b0, jl, row);
  uint4 bv[4][kMaxR / 8];  // the four columns' down-LoRA rows (fp16, r <= kMaxR)
  if (lora) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int q = 0; q < kMaxR / 8; ++q)
        if (8 * q < dm.r)
          bv[jj][q] = ldg(reinterpret_cast<const uint4*>(a.sh.bd + (int64_t)(jl + jj) * dm.r + 8 * q));
  }
  for (int i = threadIdx.x; i < nb * K; i += blockDim.x) {
    const int tb = i / K, k = i % K;
    ok[tb][k] = resolve_entry(a.pool, dm.E, a.idx[(b0 + tb) * K + k]) >= 0;
  }
  if (lora)
    for (int i = threadIdx.x; i < nb * dm.r; i += blockDim.x) {
      const int tb = i / dm.r, q = i % dm.r;
      axd[tb][q] = a.ax[(int64_t)(b0 + tb) * 3 * a.rmax + 2 * a.rmax + q];
    }
  __syncthreads();
  if (!act) return;
  const float c = dm.lora_scale;
  for (int tb = 0; tb < nb; ++tb) {
    const int b = b0 + tb;
    if (tb > 0) comb_load(a, b, j0, row);
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < kCombK; ++k) {
      if (k >= K || !ok[tb][k]) continue;
      const float wk = row.w[k];
      const float4 v = row.y[k];
      acc[0] += wk * v.x;
      acc[1] += wk * v.y;
      acc[2] += wk * v.z;
      acc[3] += wk * v.w;
    }
    if (a.sh.present) {
      const float4 v = row.ysh;
      acc[0] += v.x;
      acc[1] += v.y;
      acc[2] += v.z;
      acc[3] += v.w;
      if (lora) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          float ls = 0.0f;
#pragma unroll
          for (int q = 0; q < kMaxR / 8; ++q) {
            if (8 * q >= dm.r) break;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const f16x2 h = as_h2(word(bv[jj][q], p));
              ls = fmaf((float)h.x, axd[tb][8 * q + 2 * p], ls);
              ls = fmaf((float)h.y, axd[tb][8 * q + 2 * p + 1], ls);
            }
          }
          acc[jj] += c * ls;
        }
      }
    }
    const uint32_t lo = (uint32_t)f2h(acc[0]) | ((uint32_t)f2h(acc[1]) << 16);
    const uint32_t hi = (uint32_t)f2h(acc[2]) | ((uint32_t)f2h(acc[3]) << 16);
    *reinterpret_cast<uint2*>(a.y + (int64_t)b * d + j0) = make_uint2(lo, hi);
  }
}

// ---------------------------------------------------------------------------
// Prefill-sized batches: 64-token tiles through GEMM-shaped kernels. A
// workgroup keeps its tile's activations in LDS and streams the weight rows
// it owns past them, so each dequantised weight word feeds the tile's two
// 32-token MFMA column blocks.

constexpr int kPfTok = 64;        // tokens per tile
constexpr int kPfSG = 4;          // 64-input groups per LDS stage (gate/up)
// Batches with at least this many entries per expert on average (B*K >= 16 E)
// take the prefill kernels; measured on the 35B tier (K = 4), the chunk
// kernels are faster up to about 900 tokens.
constexpr int kPrefillPerExpert = 16;

// LDS layout of the staged activations: token t's 16-byte chunk c sits in
// slot c * ROW + t, ROW = tokens + 1. Rows of one chunk are padded by one
// slot, so one token's chunks (written by a wave) spread over the banks as
// one chunk of 32 tokens (an MFMA operand read) does, and a lane's read
// address is its own base plus a constant offset per (group, step).

// Gate/up of one tile: eight waves, each the same 32 rows of I of both the
// gate and the up matrix (256 rows per workgroup) over all d inputs, for the
// tile's 64 tokens (four accumulators), so SwiGLU is formed in registers.
// Activations are staged through LDS kPfSG groups at a time (double-buffered,
// one barrier per stage); a wave reloads each weight word for the next stage
// as soon as it has dequantised it. Each 64-input group is accumulated on
// its own and scaled in fp32 by the row's group scale, as in the chunk
// kernels. Two waves per SIMD overlap one wave's loads with the other's
// MFMAs.
constexpr int kPfGuRows = 256;  // rows of I per gate/up workgroup

// SiLU through the hardware exp2 and reciprocal: relative error about 1e-6,
// far below the fp16 rounding of the layer output.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// AFF (affine codec): the epilogue adds b * (the token's sum of x over the
// group) for every group, from sums staged in LDS.
// TB: 32-token blocks per workgroup (grid z: the tile's 64 / (32 TB) parts);
// with TB = 1 two workgroups share a compute unit.
template <bool AFF, int TB>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4 / TB)))
void k_pf_gate_up(MbArgs a) {
  constexpr int TOK = 32 * TB, ROW = TOK + 1;  // tokens per part; LDS row (one pad slot)
  __shared__ __align__(16) uint4 xs[2][kPfSG * 8 * ROW];
  __shared__ float axs[TOK][2][kMaxR];
  __shared__ __align__(16) float xss[AFF ? 32 : 1][TOK];  // [input group][part token]
  __shared__ int tokb[TOK], tokk[TOK];
  const Dims& dm = a.dm;
  const int K = dm.K, d = dm.d;
  const int imax = dm.I > dm.Is ? dm.I : dm.Is;
  bool shared;
  int u, start, count;
  int bx;
  if (!tile_block(a, bx, shared, u, start, count)) return;
  // this part's tokens: t0 .. t0 + count - 1 of the tile
  const int t0 = TOK * (int)blockIdx.z;
  count -= t0;
  if (count <= 0) return;
  if (count > TOK) count = TOK;
  start += t0;  // tiles run over consecutive tokens (shared) or sorted entries
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, n = l & 31, kh = l >> 5;
  const int row = bx * kPfGuRows + wave * 32 + n;  // I % 256 == 0
  const bool lora = shared && a.sh.ag;
  const uint32_t *gq, *uq;
  const uint16_t *gs, *us, *gb = nullptr, *ub = nullptr;
  if (shared) {
    gq = a.sh.gate.q; uq = a.sh.up.q; gs = a.sh.gate.s; us = a.sh.up.s;
    if (AFF) {
      gb = a.sh.gate.b;
      ub = a.sh.up.b;
    }
  } else {
    const int64_t ent = u;
    if (ent < 0) {
      if (threadIdx.x == 0) atomicOr(&a.flags[FLAG_RANGE], 1);
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
  if (threadIdx.x < TOK) {
    // rows past count repeat the last token (their outputs are never stored)
    int b, k;
    entry_of(a, shared, start, threadIdx.x < count ? threadIdx.x : count - 1, b, k);
    tokb[threadIdx.x] = b;
    tokk[threadIdx.x] = k;
  }
  if (lora) {  // LoRA A products of this tile's tokens: the slices in order
    for (int i = threadIdx.x; i < count * 2 * dm.r; i += blockDim.x) {
      const int tt = i / (2 * dm.r), j = i % (2 * dm.r);
      const float* p = a.axp + (int64_t)(start + tt) * 2 * a.rmax + j;
      float v = 0.0f;
      for (int sl = 0; sl < a.n_sl; ++sl) v += p[(int64_t)sl * a.B * 2 * a.rmax];
      axs[tt][j / dm.r][j % dm.r] = v;
    }
  }
  __syncthreads();
  const int wpr = d / 8, ngs = d / 64, ns = d / (64 * kPfSG);
  const uint32_t* gro = gq + (int64_t)row * wpr + 4 * kh;
  const uint32_t* uro = uq + (int64_t)row * wpr + 4 * kh;
  const uint16_t* gsr = gs + (int64_t)row * ngs;
  const uint16_t* usr = us + (int64_t)row * ngs;
  constexpr int kXr = kPfSG * 8 * TOK / 512;  // 16-byte chunks per thread per stage
  uint4 xr[kXr];
  auto load_x = [&](int st) {
#pragma unroll
    for (int it = 0; it < kXr; ++it) {
      const int flat = it * 512 + threadIdx.x, tt = flat / (kPfSG * 8), c = flat % (kPfSG * 8);
      xr[it] = ldg(reinterpret_cast<const uint4*>(a.xp + (int64_t)tokb[tt] * d +
                                                  64 * kPfSG * st + 8 * c));
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int it = 0; it < kXr; ++it) {
      const int flat = it * 512 + threadIdx.x, tt = flat / (kPfSG * 8), c = flat % (kPfSG * 8);
      xs[buf][c * ROW + tt] = xr[it];
    }
  };
  uint4 wg[kPfSG], wu[kPfSG];
  float sg[kPfSG], su[kPfSG];
#pragma unroll
  for (int i = 0; i < kPfSG; ++i) {
    wg[i] = ldg(reinterpret_cast<const uint4*>(gro + 8 * i));
    wu[i] = ldg(reinterpret_cast<const uint4*>(uro + 8 * i));
    sg[i] = sb2f<AFF>(ldg(gsr + i));
    su[i] = sb2f<AFF>(ldg(usr + i));
  }
  load_x(0);
  if (AFF)
    for (int i = threadIdx.x; i < ngs * TOK; i += blockDim.x) {
      const int gg = i / TOK, tt = i % TOK;
      xss[gg][tt] = a.xsum[(int64_t)tokb[tt] * ngs + gg];
    }
  store_x(0);
  __syncthreads();
  f32x16 ag[TB], au[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) ag[tb] = au[tb] = f32x16{};
  for (int st = 0; st < ns; ++st) {
    const bool more = st + 1 < ns;
    if (more) load_x(st + 1);
    const uint4* xb = xs[st & 1];
#pragma unroll
    for (int g = 0; g < kPfSG; ++g) {
      __builtin_amdgcn_sched_barrier(0);  // one group's operands live at a time
      const uint4 cwg = wg[g], cwu = wu[g];
      const float csg = sg[g], csu = su[g];
      if (more) {  // the same group of the next stage, into the freed registers
        const int gn = kPfSG * (st + 1) + g;
        wg[g] = ldg(reinterpret_cast<const uint4*>(gro + 8 * gn));
        wu[g] = ldg(reinterpret_cast<const uint4*>(uro + 8 * gn));
        sg[g] = sb2f<AFF>(ldg(gsr + gn));
        su[g] = sb2f<AFF>(ldg(usr + gn));
      }
      f32x16 cg[TB], cu[TB];
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) cg[tb] = cu[tb] = f32x16{};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = 8 * g + 4 * kh + j;
        const h8 w_g = q4_to_h8<AFF>(word(cwg, j)), w_u = q4_to_h8<AFF>(word(cwu, j));
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          const h8 xv = as_h8(xb[c * ROW + 32 * tb + n]);
          cg[tb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xv, w_g, cg[tb], 0, 0, 0);
          cu[tb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xv, w_u, cu[tb], 0, 0, 0);
        }
      }
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        scale_add<16>(ag[tb], cg[tb], csg);
        scale_add<16>(au[tb], cu[tb], csu);
        keep(ag[tb]);
        keep(au[tb]);
      }
    }
    if (more) store_x((st + 1) & 1);
    __syncthreads();
  }
  if (AFF) {
    // bias terms: the lane's row, every group; four consecutive tile tokens
    // per 16-byte read of the sums
    const uint16_t* gbr = gb + (int64_t)row * ngs;
    const uint16_t* ubr = ub + (int64_t)row * ngs;
#pragma unroll 4
    for (int g = 0; g < ngs; ++g) {
      const float bg = bf2f(ldg(gbr + g)), bu = bf2f(ldg(ubr + g));
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float4 x4 = *reinterpret_cast<const float4*>(&xss[g][32 * tb + 8 * j + 4 * kh]);
          const float xa[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            ag[tb][4 * j + q] = fmaf(bg, xa[q], ag[tb][4 * j + q]);
            au[tb][4 * j + q] = fmaf(bu, xa[q], au[tb][4 * j + q]);
          }
        }
    }
  }
  // epilogue: shared-expert LoRA B terms, SwiGLU, fp32 store
  const float cl = dm.lora_scale;
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = 32 * tb + tok_row(r, kh);
      if (t >= count) continue;
      float gg = ag[tb][r];
      float uu = au[tb][r];
      if (lora) {
        float lg = 0.0f, lu = 0.0f;
        for (int q = 0; q < dm.r; q += 8) {
          const uint4 bgv = ldg(reinterpret_cast<const uint4*>(a.sh.bg + (int64_t)row * dm.r + q));
          const uint4 buv = ldg(reinterpret_cast<const uint4*>(a.sh.bu + (int64_t)row * dm.r + q));
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const f16x2 g2 = as_h2(word(bgv, p)), u2 = as_h2(word(buv, p));
            lg = fmaf((float)g2.x, axs[t][0][q + 2 * p], lg);
            lg = fmaf((float)g2.y, axs[t][0][q + 2 * p + 1], lg);
            lu = fmaf((float)u2.x, axs[t][1][q + 2 * p], lu);
            lu = fmaf((float)u2.y, axs[t][1][q + 2 * p + 1], lu);
          }
        }
        gg = fmaf(cl, lg, gg);
        uu = fmaf(cl, lu, uu);
      }
      a.H[((int64_t)tokb[t] * (K + 1) + tokk[t]) * imax + row] = silu_fast(gg) * uu;
    }
  }
}

// Down projection of TB 32-token blocks of a tile (grid z: the tile's
// 64 / (32 TB) parts): eight waves, 32 output rows each (256 per workgroup)
// over all NG input groups. The part's fp32 SwiGLU outputs (32 TB tokens x
// NG*64) are staged once in LDS as fp16 hi + lo under a power-of-two scale
// per token; each dequantised weight word feeds 2 TB MFMAs (hi and lo of each
// 32-token block). With TB = 1 the staged part takes half the LDS, so two
// workgroups share a compute unit and one's loads overlap the other's
// MFMAs. Workgroups of the shared
// expert's tiles also form A_down . h for the down LoRA. AFF (affine
// codec): the staging also forms each token's sum of hi + lo over every input
// group, and the epilogue adds b * that sum per group.
template <int NG, bool AFF, int TB>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4 / TB)))
void k_pf_down(MbArgs a) {
  constexpr int TOK = 32 * TB, ROW = TOK + 1;  // tokens per part; LDS row (one pad slot)
  extern __shared__ __align__(16) uint4 hsp[];  // [NG*8 chunks][hi, lo] x ROW slots
  __shared__ float hx[TOK];
  __shared__ __align__(16) float hss[AFF ? NG : 1][TOK];  // [input group][part token]
  __shared__ int tokb[TOK], tokk[TOK];
  constexpr int nin = NG * 64, nch = NG * 8;
  const Dims& dm = a.dm;
  const int K = dm.K, d = dm.d;
  const int imax = dm.I > dm.Is ? dm.I : dm.Is;
  bool shared;
  int u, start, count;
  int bx;
  if (!tile_block(a, bx, shared, u, start, count)) return;
  // this part's tokens: t0 .. t0 + count - 1 of the tile
  const int t0 = TOK * (int)blockIdx.z;
  count -= t0;
  if (count <= 0) return;
  if (count > TOK) count = TOK;
  const uint32_t* dq;
  const uint16_t* ds;
  const uint16_t* db = nullptr;
  if (shared) {
    dq = a.sh.down.q;
    ds = a.sh.down.s;
    if (AFF) db = a.sh.down.b;
  } else {
    const int64_t ent = u;
    if (ent < 0) return;  // flagged by the gate/up step
    dq = (const uint32_t*)entry_ptr(a.pool.down.q, ent, a.pool.stride_q);
    ds = (const uint16_t*)entry_ptr(a.pool.down.s, ent, a.pool.stride_s);
    if (AFF) db = (const uint16_t*)entry_ptr(a.pool.down.b, ent, a.pool.stride_s);
  }
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63, n = l & 31, kh = l >> 5;
  const int row = bx * 256 + wave * 32 + n;  // d % 256 == 0
  uint4 wq[NG];
  float sc[NG], bd[NG];
  {
    const uint32_t* qrow = dq + (int64_t)row * (nin / 8) + 4 * kh;
    const uint16_t* srow = ds + (int64_t)row * NG;
#pragma unroll
    for (int i = 0; i < NG; ++i) wq[i] = ldg(reinterpret_cast<const uint4*>(qrow + 8 * i));
#pragma unroll
    for (int i = 0; i < NG; ++i) sc[i] = sb2f<AFF>(ldg(srow + i));
    if (AFF) {
      const uint16_t* brow = db + (int64_t)row * NG;
#pragma unroll
      for (int i = 0; i < NG; ++i) bd[i] = bf2f(ldg(brow + i));
    }
  }
  if (threadIdx.x < TOK) {
    int b = 0, k = 0;
    if ((int)threadIdx.x < count) entry_of(a, shared, start, t0 + threadIdx.x, b, k);
    tokb[threadIdx.x] = b;
    tokk[threadIdx.x] = k;
  }
  __syncthreads();
  // stage: wave w takes tokens w, w+8, ...; lane c the 8 values of chunk c.
  // All of the wave's loads are issued before the first token is split.
  constexpr int kTpw = TOK / 8, kCpl = (nch + 63) / 64;
  float4 hv[kTpw][kCpl][2];
#pragma unroll
  for (int i = 0; i < kTpw; ++i) {
    const int t = wave + 8 * i;
    const float* h = a.H + ((int64_t)tokb[t] * (K + 1) + tokk[t]) * imax;
#pragma unroll
    for (int cc = 0; cc < kCpl; ++cc) {
      const int c = l + 64 * cc;
      hv[i][cc][0] = hv[i][cc][1] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (t < count && c < nch) {  // rows past count: zeros (never stored)
        hv[i][cc][0] = *reinterpret_cast<const float4*>(h + 8 * c);
        hv[i][cc][1] = *reinterpret_cast<const float4*>(h + 8 * c + 4);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kTpw; ++i) {
    const int t = wave + 8 * i;
    float v[kCpl][8];
    float m = 0.0f;
#pragma unroll
    for (int cc = 0; cc < kCpl; ++cc) {
      const float4 v0 = hv[i][cc][0], v1 = hv[i][cc][1];
      v[cc][0] = v0.x; v[cc][1] = v0.y; v[cc][2] = v0.z; v[cc][3] = v0.w;
      v[cc][4] = v1.x; v[cc][5] = v1.y; v[cc][6] = v1.z; v[cc][7] = v1.w;
#pragma unroll
      for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(v[cc][q]));
    }
    const int e = hilo_exponent(wave_max_rows(m));
    const float inv = ldexpf(1.0f, -e);
#pragma unroll
    for (int cc = 0; cc < kCpl; ++cc) {
      const int c = l + 64 * cc;
      float psum = 0.0f;
      uint16_t hi[8], lo[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        f16 th, tl;
        split_hilo(v[cc][q], inv, th, tl);
        hi[q] = __builtin_bit_cast(uint16_t, th);
        lo[q] = __builtin_bit_cast(uint16_t, tl);
        if (AFF) psum += (float)th + (float)tl;
      }
      if (AFF) {
        // lanes 8g .. 8g+7 hold group g's chunks (uniform over the wave;
        // chunks past nch hold zeros)
        psum = group_sum<8>(psum);
        if (c < nch && (c & 7) == 0) hss[c >> 3][t] = psum;
      }
      if (c >= nch) continue;
      // pair-permuted order [0 4 1 5 2 6 3 7]
      hsp[(2 * c) * ROW + t] =
          make_uint4(hi[0] | ((uint32_t)hi[4] << 16), hi[1] | ((uint32_t)hi[5] << 16),
                     hi[2] | ((uint32_t)hi[6] << 16), hi[3] | ((uint32_t)hi[7] << 16));
      hsp[(2 * c + 1) * ROW + t] =
          make_uint4(lo[0] | ((uint32_t)lo[4] << 16), lo[1] | ((uint32_t)lo[5] << 16),
                     lo[2] | ((uint32_t)lo[6] << 16), lo[3] | ((uint32_t)lo[7] << 16));
    }
    if (l == 0) hx[t] = t < count ? ldexpf(1.0f, e) : 0.0f;
  }
  if (shared && a.sh.ad) {
    // A_down . h_shared[t] for the part's tokens t = bx, bx + gridDim.x, ...;
    // wave w takes ranks q = w, w+8, ...
    for (int t = bx; t < count; t += gridDim.x) {
      const int b = start + t0 + t;
      const float* h = a.H + ((int64_t)b * (K + 1) + K) * imax;
      for (int q = wave; q < dm.r; q += 8) {
        float sacc = 0.0f;
        for (int c = l; c < nch; c += 64) {
          const float4 v0 = *reinterpret_cast<const float4*>(h + 8 * c);
          const float4 v1 = *reinterpret_cast<const float4*>(h + 8 * c + 4);
          const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
          const uint4 av = ldg(reinterpret_cast<const uint4*>(a.sh.ad + (int64_t)q * nin + 8 * c));
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const f16x2 ah = as_h2(word(av, p));
            sacc = fmaf((float)ah.x, v[2 * p], sacc);
            sacc = fmaf((float)ah.y, v[2 * p + 1], sacc);
          }
        }
        sacc = wave_sum_rows(sacc);
        if (l == 0) a.ax[(int64_t)b * 3 * a.rmax + 2 * a.rmax + q] = sacc;
      }
    }
  }
  __syncthreads();
  f32x16 acc[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) acc[tb] = f32x16{};
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    __builtin_amdgcn_sched_barrier(0);  // one group's operands live at a time
    f32x16 cc[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) cc[tb] = f32x16{};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 8 * g + 4 * kh + j;
      const h8 w8 = q4_to_h8<AFF>(word(wq[g], j));
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        cc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(hsp[(2 * c) * ROW + 32 * tb + n]), w8,
                                                        cc[tb], 0, 0, 0);
        cc[tb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(hsp[(2 * c + 1) * ROW + 32 * tb + n]),
                                                        w8, cc[tb], 0, 0, 0);
      }
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      scale_add<16>(acc[tb], cc[tb], sc[g]);
      keep(acc[tb]);
    }
  }
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int t = 32 * tb + tok_row(r, kh);
      if (t < count) {
        float v = acc[tb][r];
        if (AFF) {
#pragma unroll
          for (int i = 0; i < NG; ++i) v = fmaf(bd[i], hss[i][t], v);
        }
        a.Y[((int64_t)tokb[t] * (K + 1) + tokk[t]) * d + row] = v * hx[t];
      }
    }
  }
}

}  // namespace

bool batched_supported(const Dims& dm) {
  const int gu_groups = dm.G > 0 ? dm.d / dm.G : 0, dn_groups = dm.G > 0 ? dm.I / dm.G : 0;
  return dm.G == 64 && dm.d % 128 == 0 && dm.I % 64 == 0 && gu_groups % 8 == 0 &&
         gu_groups <= 32 && dn_groups % 2 == 0 && dn_groups <= 8 && dm.K <= 8 &&
         dm.E <= kMaxE && dm.r % 8 == 0 && dm.r <= kMaxR && (dm.Is == 0 || dm.Is == dm.I);
}

// Shapes the prefill kernels take: 256 rows of I per gate/up workgroup,
// 256 output rows per down workgroup, whole LDS stages of kPfSG groups.
static bool prefill_supported(const Dims& dm) {
  return batched_supported(dm) && dm.I % kPfGuRows == 0 && dm.d % 256 == 0 &&
         dm.d % (64 * kPfSG) == 0;
}

namespace {

template <int NG>
void launch_gate_up_ng(const MbArgs& a, dim3 grid, hipStream_t st) {
  if (a.dm.affine)
    hipLaunchKernelGGL((k_mb_gate_up<NG, true>), grid, dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((k_mb_gate_up<NG, false>), grid, dim3(512), 0, st, a);
}

// 32-token blocks per prefill workgroup (1: two workgroups per compute unit).
constexpr int kPfDownTB = 1;
constexpr int kPfGuTB = 2;  // one part of 32 tokens needs over 128 registers (scratch spills)

template <int NG, bool AFF>
hipError_t launch_pf_down_t(const MbArgs& a, dim3 grid, hipStream_t st) {
  constexpr int TB = kPfDownTB;
  const size_t lds = (size_t)NG * 8 * 2 * (32 * TB + 1) * sizeof(uint4);
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)k_pf_down<NG, AFF, TB>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  grid.z = kPfTok / (32 * TB);
  hipLaunchKernelGGL((k_pf_down<NG, AFF, TB>), grid, dim3(512), lds, st, a);
  return hipSuccess;
}

template <int NG>
hipError_t launch_pf_down_ng(const MbArgs& a, dim3 grid, hipStream_t st) {
  return a.dm.affine ? launch_pf_down_t<NG, true>(a, grid, st)
                     : launch_pf_down_t<NG, false>(a, grid, st);
}

template <int NG>
void launch_down_ng(const MbArgs& a, dim3 grid, hipStream_t st) {
  const size_t lds = (size_t)(a.B < kCols ? a.B : kCols) * 2 * (NG * 64 + kDnPad) * sizeof(uint16_t);
  if (a.dm.affine)
    hipLaunchKernelGGL((k_mb_down<NG, true>), grid, dim3(64 * kDnWaves), lds, st, a);
  else
    hipLaunchKernelGGL((k_mb_down<NG, false>), grid, dim3(64 * kDnWaves), lds, st, a);
}

}  // namespace

hipError_t launch_batched(const Dims& dm, const Pool& pool, const SharedW& sh, const uint16_t* x,
                          const int32_t* idx, const float* w, int B, uint16_t* y,
                          const Scratch& s, hipStream_t st) {
  if (B < 1 || !batched_supported(dm)) return hipErrorInvalidValue;
  MbArgs a;
  a.dm = dm;
  a.pool = pool;
  a.sh = sh;
  a.B = B;
  a.x = x;
  a.xp = s.xn;
  a.grp = s.grp;
  a.idx = idx;
  a.w = w;
  a.ax = s.ax;
  a.axp = s.axp;
  a.rmax = dm.r > 1 ? dm.r : 1;
  a.n_sl = 1;  // largest slice count <= kLoraSlices with whole 16-input MFMA steps per wave
  while (a.n_sl < kLoraSlices && (dm.d / 64) % (2 * a.n_sl) == 0) a.n_sl *= 2;
  a.H = s.gu;
  a.Y = s.yk;
  a.xsum = s.hattn;  // unused by this path otherwise; [B][d] floats >= [B][d/64]
  a.ctok = B >= 512 ? kCombTokMax : 1;
  a.y = y;
  a.flags = s.flags;
  const bool pf = (int64_t)B * dm.K >= (int64_t)kPrefillPerExpert * dm.E && prefill_supported(dm);
  a.tile = pf ? kPfTok : kCols;
  // an upper bound for either tile size; tiles past n_tiles exit at once
  const int ny = batched_max_tiles(B, dm.K, dm.E);
  a.ny = ny;
  const int imax = dm.I > dm.Is ? dm.I : dm.Is;
  const int lora_blocks = sh.present && sh.ag ? (B + kCols - 1) / kCols * a.n_sl : 0;
  hipLaunchKernelGGL(k_mb_prep, dim3(B + 1 + lora_blocks), dim3(256), 0, st, a);
  if (pf) {
    const dim3 gu_grid(imax / kPfGuRows, ny, kPfTok / (32 * kPfGuTB));
    if (dm.affine)
      hipLaunchKernelGGL((k_pf_gate_up<true, kPfGuTB>), gu_grid, dim3(512), 0, st, a);
    else
      hipLaunchKernelGGL((k_pf_gate_up<false, kPfGuTB>), gu_grid, dim3(512), 0, st, a);
    const dim3 grid(dm.d / 256, ny);
    hipError_t e;
    switch (dm.I / dm.G) {
      case 2: e = launch_pf_down_ng<2>(a, grid, st); break;
      case 4: e = launch_pf_down_ng<4>(a, grid, st); break;
      case 6: e = launch_pf_down_ng<6>(a, grid, st); break;
      default: e = launch_pf_down_ng<8>(a, grid, st); break;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_mb_combine, dim3((B + a.ctok - 1) / a.ctok, (dm.d + 1023) / 1024),
                       dim3(256), 0, st, a);
    return hipGetLastError();
  }
  const dim3 gu_grid(imax / 32, ny);
  switch (dm.d / dm.G / 4) {
    case 2: launch_gate_up_ng<2>(a, gu_grid, st); break;
    case 4: launch_gate_up_ng<4>(a, gu_grid, st); break;
    case 6: launch_gate_up_ng<6>(a, gu_grid, st); break;
    default: launch_gate_up_ng<8>(a, gu_grid, st); break;
  }
  const dim3 dn_grid((dm.d + 32 * kDnWaves - 1) / (32 * kDnWaves), ny);
  switch (dm.I / dm.G) {
    case 2: launch_down_ng<2>(a, dn_grid, st); break;
    case 4: launch_down_ng<4>(a, dn_grid, st); break;
    case 6: launch_down_ng<6>(a, dn_grid, st); break;
    default: launch_down_ng<8>(a, dn_grid, st); break;
  }
  hipLaunchKernelGGL(k_mb_combine, dim3((B + a.ctok - 1) / a.ctok, (dm.d + 1023) / 1024),
                       dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace smd
