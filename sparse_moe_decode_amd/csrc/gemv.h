// Device building blocks shared by the per-phase kernels and the persistent
// whole-token kernel, so that both compute identical sums in identical order.
#pragma once

#include "device.h"
#include "internal.h"

namespace smd {

__device__ __forceinline__ const void* entry_ptr(const void* base, int64_t entry, int64_t stride) {
  return (const char*)base + entry * stride;
}

// Resolve routed expert id -> pool entry (through the slot table if any);
// -1 if the id or the slot is out of range.
__device__ __forceinline__ int64_t resolve_entry(const Pool& p, int E, int e) {
  if (e < 0 || e >= E) return -1;
  int64_t ent = e;
  if (p.slot_of) ent = ldg(p.slot_of + e);
  if (ent < 0 || ent >= p.count) return -1;
  return ent;
}

// Load the pair-permuted fp16 activation chunk c (32 elements) from LDS.
__device__ __forceinline__ void load_xchunk(const uint16_t* xs, int c, f16x2* xr) {
  const uint4* src = reinterpret_cast<const uint4*>(xs + 32 * c);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    uint4 v = src[m];
    xr[4 * m + 0] = as_h2(v.x);
    xr[4 * m + 1] = as_h2(v.y);
    xr[4 * m + 2] = as_h2(v.z);
    xr[4 * m + 3] = as_h2(v.w);
  }
}

// One 16-byte chunk (32 int4 weights) against 32 activations.
template <bool AFF = false>
__device__ __forceinline__ float q4_dot32(uint4 wv, const f16x2* xr) {
  float p = 0.0f;
  p = q4_dot8<AFF>(wv.x, xr + 0, p);
  p = q4_dot8<AFF>(wv.y, xr + 4, p);
  p = q4_dot8<AFF>(wv.z, xr + 8, p);
  p = q4_dot8<AFF>(wv.w, xr + 12, p);
  return p;
}

// Same with an fp16 hi/lo activation pair (dequantises each word once).
template <bool AFF = false>
__device__ __forceinline__ float q4_dot8_hl(uint32_t w, const f16x2* xh, const f16x2* xl,
                                            float acc) {
  f16x2 p0, p1, p2, p3;
  q4_pairs<AFF>(w, p0, p1, p2, p3);
  acc = dot2(p0, xh[0], acc);
  acc = dot2(p1, xh[1], acc);
  acc = dot2(p2, xh[2], acc);
  acc = dot2(p3, xh[3], acc);
  acc = dot2(p0, xl[0], acc);
  acc = dot2(p1, xl[1], acc);
  acc = dot2(p2, xl[2], acc);
  acc = dot2(p3, xl[3], acc);
  return acc;
}

template <bool AFF = false>
__device__ __forceinline__ float q4_dot32_hl(uint4 wv, const f16x2* xh, const f16x2* xl) {
  float p = 0.0f;
  p = q4_dot8_hl<AFF>(wv.x, xh + 0, xl + 0, p);
  p = q4_dot8_hl<AFF>(wv.y, xh + 4, xl + 4, p);
  p = q4_dot8_hl<AFF>(wv.z, xh + 8, xl + 8, p);
  p = q4_dot8_hl<AFF>(wv.w, xh + 12, xl + 12, p);
  return p;
}

// The same sums with independent partial sums per packed word (and per hi /
// lo half), so that a single wave's dependent v_dot2 chains are four (eight)
// times shorter; the partials are added in a fixed tree.
__device__ __forceinline__ float q4_dot32_ilp(uint4 wv, const f16x2* xr) {
  const float p0 = q4_dot8(wv.x, xr + 0, 0.0f), p1 = q4_dot8(wv.y, xr + 4, 0.0f);
  const float p2 = q4_dot8(wv.z, xr + 8, 0.0f), p3 = q4_dot8(wv.w, xr + 12, 0.0f);
  return (p0 + p1) + (p2 + p3);
}

__device__ __forceinline__ float q4_dot8_split(uint32_t w, const f16x2* xh, const f16x2* xl) {
  f16x2 p0, p1, p2, p3;
  q4_pairs(w, p0, p1, p2, p3);
  float h = dot2(p0, xh[0], 0.0f), l = dot2(p0, xl[0], 0.0f);
  h = dot2(p1, xh[1], h);
  l = dot2(p1, xl[1], l);
  h = dot2(p2, xh[2], h);
  l = dot2(p2, xl[2], l);
  h = dot2(p3, xh[3], h);
  l = dot2(p3, xl[3], l);
  return h + l;
}

__device__ __forceinline__ float q4_dot32_hl_ilp(uint4 wv, const f16x2* xh, const f16x2* xl) {
  const float p0 = q4_dot8_split(wv.x, xh + 0, xl + 0), p1 = q4_dot8_split(wv.y, xh + 4, xl + 4);
  const float p2 = q4_dot8_split(wv.z, xh + 8, xl + 8), p3 = q4_dot8_split(wv.w, xh + 12, xl + 12);
  return (p0 + p1) + (p2 + p3);
}

// 32 int4 weights of one 16-byte chunk against 32 fp32 activations (natural
// order, 16-byte aligned in LDS): each product q * s is formed and
// accumulated in fp32 (v_fma_mix takes the exact fp16 q).
// AFF: unsigned nibbles (the affine codec); with xsum non-null the sum of
// the 32 activations is written there as well (the bias term's factor).
template <bool AFF = false>
__device__ __forceinline__ float q4_dot32_f32(uint4 wv, const float* s, float* xsum = nullptr) {
  const uint32_t w4[4] = {wv.x, wv.y, wv.z, wv.w};
  float a0 = 0.0f, a1 = 0.0f, sx = 0.0f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    f16x2 p0, p1, p2, p3;
    q4_pairs<AFF>(w4[m], p0, p1, p2, p3);
    const float4 x0 = *reinterpret_cast<const float4*>(s + 8 * m);
    const float4 x1 = *reinterpret_cast<const float4*>(s + 8 * m + 4);
    a0 = fmaf((float)p0.x, x0.x, a0);
    a1 = fmaf((float)p0.y, x1.x, a1);
    a0 = fmaf((float)p1.x, x0.y, a0);
    a1 = fmaf((float)p1.y, x1.y, a1);
    a0 = fmaf((float)p2.x, x0.z, a0);
    a1 = fmaf((float)p2.y, x1.z, a1);
    a0 = fmaf((float)p3.x, x0.w, a0);
    a1 = fmaf((float)p3.y, x1.w, a1);
    if (xsum) sx += ((x0.x + x0.y) + (x0.z + x0.w)) + ((x1.x + x1.y) + (x1.z + x1.w));
  }
  if (xsum) *xsum = sx;
  return a0 + a1;
}

// Block-wide max of |v| over a strided range (kBlock threads).
__device__ __forceinline__ float block_absmax(const float* v, int n, float* red) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < n; i += blockDim.x) m = fmaxf(m, fabsf(v[i]));
  m = wave_max(m);
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = m;
  __syncthreads();
  float r = 0.0f;
  for (int j = 0; j < nw; ++j) r = fmaxf(r, red[j]);
  return r;
}

// Power-of-two exponent e with max|v| * 2^-e < 2^14 (0 for an all-zero vector).
__device__ __forceinline__ int hilo_exponent(float absmax) {
  if (!(absmax > 0.0f)) return 0;
  int ex;
  frexpf(absmax, &ex);  // absmax < 2^ex
  return ex - 14;
}


// Lane li of a 16-lane group holds elements 32c + 2li and 32c + 2li + 1 of an
// I-vector. The group converts chunk c to fp16 hi + lo scaled by a power of
// two 2^-e chosen from the chunk's max |v|, written pair-permuted to dst (hi
// at dst[0, I), lo at dst[I, 2I)); returns 2^e. With hsum non-null, lane 0
// writes there the chunk's sum of hi + lo (for the affine bias terms). All 16
// lanes must be active.
__device__ __forceinline__ float hilo_pair(float v0, float v1, int c, int li, uint16_t* dst,
                                           int I, float* hsum = nullptr) {
  const float m = group_max<16>(fmaxf(fabsf(v0), fabsf(v1)));
  const int e = hilo_exponent(m);
  const float inv = ldexpf(1.0f, -e);
  f16 h0, l0, h1, l1;
  split_hilo(v0, inv, h0, l0);
  split_hilo(v1, inv, h1, l1);
  const int i0 = 32 * c + 2 * li;
  const int p0 = perm8(i0), p1 = perm8(i0 + 1);
  dst[p0] = __builtin_bit_cast(uint16_t, h0);
  dst[p1] = __builtin_bit_cast(uint16_t, h1);
  dst[I + p0] = __builtin_bit_cast(uint16_t, l0);
  dst[I + p1] = __builtin_bit_cast(uint16_t, l1);
  if (hsum) {
    const float sum = group_sum<16>(((float)h0 + (float)l0) + ((float)h1 + (float)l1));
    if (li == 0) *hsum = sum;
  }
  return ldexpf(1.0f, e);
}

// ---------------------------------------------------------- row kernels --
// One aligned group of LG lanes computes one row; li is the lane's index in
// the group. Each returns the lane's partial sum; the caller reduces over the
// group with group_sum<LG>.

// Gate and up rows of one expert against the pair-permuted fp16 x in LDS
// (d = 32 * LG * CPL columns): partial Wg[row] . x and Wu[row] . x.
template <int LG, int CPL>
__device__ __forceinline__ void gateup_rowpair(const uint32_t* grow, const uint32_t* urow,
                                               const uint16_t* gsr, const uint16_t* usr, int G,
                                               const uint16_t* xs, int li, float& ag,
                                               float& au) {
  uint4 wg[CPL], wu[CPL];
  uint16_t sg[CPL], su[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = li + LG * j;
    wg[j] = ldg(reinterpret_cast<const uint4*>(grow + 4 * c));
    wu[j] = ldg(reinterpret_cast<const uint4*>(urow + 4 * c));
    sg[j] = ldg(gsr + (32 * c) / G);
    su[j] = ldg(usr + (32 * c) / G);
  }
  ag = 0.0f;
  au = 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    f16x2 xr[16];
    load_xchunk(xs, li + LG * j, xr);
    ag += h2f(sg[j]) * q4_dot32(wg[j], xr);
    au += h2f(su[j]) * q4_dot32(wu[j], xr);
  }
}

// One int4 row ([I] inputs) against an activation held as pair-permuted fp16
// hi and lo halves in LDS: partial row . (hi + lo).
template <int LG, int CPL>
__device__ __forceinline__ float down_row_hl(const uint32_t* qrow, const uint16_t* srow, int G,
                                             const uint16_t* hh, const uint16_t* hl, int li) {
  uint4 wv[CPL];
  uint16_t sv[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = li + LG * j;
    wv[j] = ldg(reinterpret_cast<const uint4*>(qrow + 4 * c));
    sv[j] = ldg(srow + (32 * c) / G);
  }
  float part = 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    f16x2 xh[16], xl[16];
    load_xchunk(hh, li + LG * j, xh);
    load_xchunk(hl, li + LG * j, xl);
    part += h2f(sv[j]) * q4_dot32_hl(wv[j], xh, xl);
  }
  return part;
}

// Affine gate/up rows: w = s q + b with bf16 s, b per group and unsigned q.
// A 32-element chunk c contributes s (q . x) + b xsum[c], xsum[c] the sum of
// the chunk's activations (fp32, in LDS).
template <int LG, int CPL>
__device__ __forceinline__ void gateup_rowpair_aff(const uint32_t* grow, const uint32_t* urow,
                                                   const uint16_t* gsr, const uint16_t* usr,
                                                   const uint16_t* gbr, const uint16_t* ubr,
                                                   int G, const uint16_t* xs, const float* xsum,
                                                   int li, float& ag, float& au) {
  uint4 wg[CPL], wu[CPL];
  uint16_t sg[CPL], su[CPL], bg[CPL], bu[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = li + LG * j;
    wg[j] = ldg(reinterpret_cast<const uint4*>(grow + 4 * c));
    wu[j] = ldg(reinterpret_cast<const uint4*>(urow + 4 * c));
    sg[j] = ldg(gsr + (32 * c) / G);
    su[j] = ldg(usr + (32 * c) / G);
    bg[j] = ldg(gbr + (32 * c) / G);
    bu[j] = ldg(ubr + (32 * c) / G);
  }
  ag = 0.0f;
  au = 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = li + LG * j;
    f16x2 xr[16];
    load_xchunk(xs, c, xr);
    ag += bf2f(sg[j]) * q4_dot32<true>(wg[j], xr) + bf2f(bg[j]) * xsum[c];
    au += bf2f(su[j]) * q4_dot32<true>(wu[j], xr) + bf2f(bu[j]) * xsum[c];
  }
}

// Affine down row against hi/lo activations; hsum[c] = sum of the chunk's
// hi + lo values.
template <int LG, int CPL>
__device__ __forceinline__ float down_row_hl_aff(const uint32_t* qrow, const uint16_t* srow,
                                                 const uint16_t* brow, int G, const uint16_t* hh,
                                                 const uint16_t* hl, const float* hsum, int li) {
  uint4 wv[CPL];
  uint16_t sv[CPL], bv[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = li + LG * j;
    wv[j] = ldg(reinterpret_cast<const uint4*>(qrow + 4 * c));
    sv[j] = ldg(srow + (32 * c) / G);
    bv[j] = ldg(brow + (32 * c) / G);
  }
  float part = 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = li + LG * j;
    f16x2 xh[16], xl[16];
    load_xchunk(hh, c, xh);
    load_xchunk(hl, c, xl);
    part += bf2f(sv[j]) * q4_dot32_hl<true>(wv[j], xh, xl) + bf2f(bv[j]) * hsum[c];
  }
  return part;
}

// fp16 row [cols] against fp16 x (natural order) in LDS: partial dot product
// over the 8-element chunks li, li + LG, ...
template <int LG>
__device__ __forceinline__ float f16_row_dot(const uint16_t* wrow, int cols, const uint16_t* xs,
                                             int li) {
  float acc = 0.0f;
  const int nch = cols / 8;
  for (int c = li; c < nch; c += LG) {
    const uint4 wv = ldg(reinterpret_cast<const uint4*>(wrow + 8 * c));
    const uint4 xv = *reinterpret_cast<const uint4*>(xs + 8 * c);
    acc = dot2(as_h2(wv.x), as_h2(xv.x), acc);
    acc = dot2(as_h2(wv.y), as_h2(xv.y), acc);
    acc = dot2(as_h2(wv.z), as_h2(xv.z), acc);
    acc = dot2(as_h2(wv.w), as_h2(xv.w), acc);
  }
  return acc;
}

// Same with an fp16 hi/lo activation pair (natural order).
template <int LG>
__device__ __forceinline__ float f16_row_dot_hl(const uint16_t* wrow, int cols,
                                                const uint16_t* xh, const uint16_t* xl, int li) {
  float acc = 0.0f;
  const int nch = cols / 8;
  for (int c = li; c < nch; c += LG) {
    const uint4 wv = ldg(reinterpret_cast<const uint4*>(wrow + 8 * c));
    const uint4 a = *reinterpret_cast<const uint4*>(xh + 8 * c);
    const uint4 b = *reinterpret_cast<const uint4*>(xl + 8 * c);
    acc = dot2(as_h2(wv.x), as_h2(a.x), acc);
    acc = dot2(as_h2(wv.y), as_h2(a.y), acc);
    acc = dot2(as_h2(wv.z), as_h2(a.z), acc);
    acc = dot2(as_h2(wv.w), as_h2(a.w), acc);
    acc = dot2(as_h2(wv.x), as_h2(b.x), acc);
    acc = dot2(as_h2(wv.y), as_h2(b.y), acc);
    acc = dot2(as_h2(wv.z), as_h2(b.z), acc);
    acc = dot2(as_h2(wv.w), as_h2(b.w), acc);
  }
  return acc;
}

constexpr int kMaxE = 512;

// LDS written by some lanes of a wave and read by others: the wave's LDS
// operations complete in issue order, so only compiler reordering must be
// prevented.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct RouteScratch {
  float sel[kMaxE];  // sigmoid-group selection scores
  int keep[64];      // sigmoid-group: group kept
};

// Routing of one token's fp32 logits by the tier's family [MW App. A]:
// softmax-top-K (select the K largest logits, which are the K largest
// probabilities; weights renormalised over the K, or the full softmax when
// norm_topk is 0) or sigmoid-group (biased scores, top-2-sum group ranking,
// top-K inside surviving groups, weights s * sigma / (sum sigma + 1e-20)).
// Ties go to the lower id (lower group id for groups).
//
// One full wave (all 64 lanes active). Lane l holds candidates l + 64j as
// 64-bit keys (order-preserving score bits, then the complemented id, so
// the maximum key is the best score with the lowest id), sorted once per
// lane. Each of the K rounds takes the wave maximum of the lanes' best keys
// (DPP inside rows, four readlanes) and the winner's lane drops it. Lane k
// keeps the k-th selection, computes its weight and writes idx[k] / w[k].
template <int PER>
__device__ __forceinline__ void route_wave_t(const Dims& dm, const float* lg, const float* bias,
                                             RouteScratch& rs, int32_t* out_idx, float* out_w,
                                             int32_t* flags) {
  const int lane = threadIdx.x & 63;
  const int E = dm.E, K = dm.K;
  const bool sg = dm.router_kind == E0_ROUTER_SIGMOID_GROUP;

  if (sg) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = lane + 64 * j;
      if (e < E) rs.sel[e] = 1.0f / (1.0f + expf(-lg[e])) + (bias ? ldg(bias + e) : 0.0f);
    }
    wave_lds_sync();
    // group score: sum of the two best selection scores of the group
    const int gsize = E / dm.n_groups;
    uint64_t gkey = 0;
    if (lane < dm.n_groups) {
      float m1 = -INFINITY, m2 = -INFINITY;
      for (int i = 0; i < gsize; ++i) {
        const float v = rs.sel[lane * gsize + i];
        if (v > m1) { m2 = m1; m1 = v; } else if (v > m2) { m2 = v; }
      }
      gkey = ((uint64_t)f2key(m1 + m2) << 32) | (0xFFFFFFFFu - (uint32_t)lane);
    }
    bool kept = false;
    for (int r = 0; r < dm.topk_groups; ++r) {
      const uint64_t g = wave_max_key(gkey);
      if (gkey == g && g != 0) {
        kept = true;
        gkey = 0;
      }
    }
    if (lane < dm.n_groups) rs.keep[lane] = kept ? 1 : 0;
    wave_lds_sync();
  }

  // Keys: order-preserving score bits over (inverted) id, so ties go to the
  // lower id and every key is unique; 0 = no candidate. Each lane sorts its
  // PER keys once; a round then takes the wave maximum of the lanes' heads
  // and the winning lane shifts its list.
  uint64_t key[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    key[j] = 0;
    const int e = lane + 64 * j;
    if (e < E) {
      bool ok = true;
      float score = lg[e];
      if (sg) {
        ok = rs.keep[e / (E / dm.n_groups)] != 0;
        score = rs.sel[e];
      }
      if (ok) key[j] = ((uint64_t)f2key(score) << 32) | (0xFFFFFFFFu - (uint32_t)e);
    }
  }
#pragma unroll
  for (int i = 1; i < PER; ++i)
#pragma unroll
    for (int j = i; j > 0; --j) {
      const uint64_t hi = key[j] > key[j - 1] ? key[j] : key[j - 1];
      const uint64_t lo = key[j] > key[j - 1] ? key[j - 1] : key[j];
      key[j - 1] = hi;
      key[j] = lo;
    }
  int mine = -1;  // lane k < K: the k-th selection
  int first = 0;
  for (int k = 0; k < K; ++k) {
    const uint64_t g = wave_max_key(key[0]);
    int e = 0;
    if (g == 0) {  // no candidate left (rejected shapes make this unreachable)
      if (lane == 0) atomicOr(&flags[FLAG_RANGE], 4);
    } else {
      e = (int)(0xFFFFFFFFu - (uint32_t)g);
    }
    if (k == 0) first = e;
    if (lane == k) mine = e;
    if (key[0] == g) {
#pragma unroll
      for (int j = 0; j + 1 < PER; ++j) key[j] = key[j + 1];
      key[PER - 1] = 0;
    }
  }
  // softmax shift: the largest logit is the first selection
  const float mx = lg[first];
  float full = 0.0f;
  if (!sg && !dm.norm_topk) {
    float z = 0.0f;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = lane + 64 * j;
      if (e < E) z += expf(lg[e] - mx);
    }
    full = wave_sum_rows(z);
  }
  float wk = 0.0f;
  if (lane < K) {
    const float l = lg[mine];
    wk = sg ? 1.0f / (1.0f + expf(-l)) : expf(l - mx);
  }
  float denom = wave_sum_rows(wk);
  if (sg) denom += 1e-20f;
  else if (!dm.norm_topk) denom = full;
  if (lane < K) {
    out_idx[lane] = mine;
    const float ww = wk / denom;
    out_w[lane] = sg ? dm.route_scale * ww : ww;
  }
}

__device__ __forceinline__ void route_wave(const Dims& dm, const float* lg, const float* bias,
                                           RouteScratch& rs, int32_t* out_idx, float* out_w,
                                           int32_t* flags) {
  if (dm.E <= 256)
    route_wave_t<4>(dm, lg, bias, rs, out_idx, out_w, flags);
  else
    route_wave_t<8>(dm, lg, bias, rs, out_idx, out_w, flags);
}

}  // namespace smd
