// Expert staging: the slot policy runs on the device, then the missing
// expert bundles are gathered from pinned host memory (mapped into the GPU
// address space) into the layer's HBM slots over PCIe. Everything runs on
// the caller's side stream, so the predicted ids never travel to the host.
//
// Source: "The Other Half of the Memory Wall" §3.1 Executor paths (staged
// fixed slots, only changed experts rewritten) and §3.2 Prediction-as-routing
// (staged set equals routed set); "Inside Edge0-35B", Fixed-Slot Decoding.

#include "internal.h"

namespace smd {

namespace {

constexpr int kMaxE = 512;
constexpr int kMaxSlots = 64;
constexpr int kCopyThreads = 1024;

// Slot policy, one workgroup per layer of the call (single thread; E <= 512,
// K <= 8, slots <= 64): ids of `next` with a slot keep it; misses in
// ascending id take, in ascending slot order, the slots holding no id of
// in_use or next. Writes (expert, slot) pairs to copy_list and the count to
// n_copies, and adds the count to the stager's running total.
__global__ __launch_bounds__(64) void k_slot_policy(int E, int n_slots, int K,
                                                    int32_t* slot_of, int32_t* slot_expert,
                                                    const int32_t* in_use, const int32_t* next,
                                                    int32_t* copy_list, int32_t* n_copies,
                                                    unsigned long long* total, int32_t* flags) {
  __shared__ uint32_t keep[kMaxE / 32];
  const int l = blockIdx.x;
  slot_of += (int64_t)l * E;
  slot_expert += (int64_t)l * n_slots;
  next += (int64_t)l * K;
  if (in_use) in_use += (int64_t)l * K;
  copy_list += (int64_t)l * 16;
  n_copies += l;
  if (threadIdx.x < kMaxE / 32) keep[threadIdx.x] = 0;
  __syncthreads();
  if (threadIdx.x != 0) return;
  // 1. every id in range, else nothing is staged
  for (int k = 0; k < K; ++k) {
    const bool bad = next[k] < 0 || next[k] >= E || (in_use && (in_use[k] < 0 || in_use[k] >= E));
    if (bad) {
      atomicOr(&flags[FLAG_RANGE], 1);
      *n_copies = 0;
      return;
    }
  }
  // 2. ids that must stay resident: the set in use and the new set
  for (int k = 0; k < K; ++k) {
    keep[next[k] >> 5] |= 1u << (next[k] & 31);
    if (in_use) keep[in_use[k] >> 5] |= 1u << (in_use[k] & 31);
  }
  // 3. misses of the new set, ascending and without repeats
  int misses[8];
  int nm = 0;
  for (int k = 0; k < K; ++k) {
    const int e = next[k];
    if (slot_of[e] >= 0) continue;
    bool dup = false;
    for (int i = 0; i < nm; ++i) dup |= (misses[i] == e);
    if (dup) continue;
    int i = nm++;
    while (i > 0 && misses[i - 1] > e) {
      misses[i] = misses[i - 1];
      --i;
    }
    misses[i] = e;
  }
  // 4. free slots in ascending order take the misses; occupants are evicted
  int nc = 0;
  for (int s = 0; s < n_slots && nc < nm; ++s) {
    const int old = slot_expert[s];
    const bool held = old >= 0 && old < E;
    if (held && (keep[old >> 5] & (1u << (old & 31)))) continue;
    const int e = misses[nc];
    if (held) slot_of[old] = -1;
    slot_expert[s] = e;
    slot_of[e] = s;
    copy_list[2 * nc] = e;
    copy_list[2 * nc + 1] = s;
    ++nc;
  }
  if (nc < nm) atomicOr(&flags[FLAG_RANGE], 2);  // pool too small for the set
  *n_copies = nc;
  atomicAdd(total, (unsigned long long)nc);
}

// Gather-copy of every listed bundle of the call's layers, host-mapped
// memory -> HBM slots, in 16-byte units. A few large workgroups stride over
// each bundle in turn (four loads in flight per thread): enough reads in
// flight for the host link, while occupying at most kCopyBlocks compute
// units so that a persistent kernel on the rest of the chip keeps running.
__global__ __launch_bounds__(kCopyThreads) void k_stage_copy(
    const char* host, int64_t host_stride, char* hbm, int64_t hbm_stride, int64_t bundle,
    int n_layers, const int32_t* copy_list, const int32_t* n_copies) {
  const int64_t n16 = bundle / 16;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int l = 0; l < n_layers; ++l) {
    const int nc = n_copies[l];
    for (int j = 0; j < nc; ++j) {
      const int e = copy_list[16 * l + 2 * j], s = copy_list[16 * l + 2 * j + 1];
      const uint4* src = reinterpret_cast<const uint4*>(host + l * host_stride + (int64_t)e * bundle);
      uint4* dst = reinterpret_cast<uint4*>(hbm + l * hbm_stride + (int64_t)s * bundle);
      int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
      for (; i + 3 * step < n16; i += 4 * step) {
        uint4 a = src[i], b = src[i + step], c = src[i + 2 * step], d = src[i + 3 * step];
        dst[i] = a;
        dst[i + step] = b;
        dst[i + 2 * step] = c;
        dst[i + 3 * step] = d;
      }
      for (; i < n16; i += step) dst[i] = src[i];
    }
  }
}

constexpr int kCacheThreads = 1024;

// Cross-layer hot-expert cache policy [MW §3.1 Executor paths, "hot":
// LRU-resident experts; Table 1: a shared LRU of expert bundles across
// layers; IE "The Streaming Subsystem": a hit skips the read], one workgroup
// for all layers of the call. State: slot_of [L][E] (cache entry of
// (layer, id), or -1), owner [C] (layer * E + id, or -1 for empty), stamp
// [C] (tick of the entry's last staging, -1 never). Staging the sets of
// layers layer0 .. layer0 + n_layers - 1 at tick T: ids already cached are
// hits and their entries' stamp becomes T; the misses, in ascending
// (layer, id), take the entries that are empty or were last staged before
// T - 1 (the running token and the sets already staged for T keep theirs),
// least recently staged first, ties to the lower index; the previous owner
// loses the entry. The entry table is worked on in LDS (one bitonic sort of
// the free entries by (stamp, index)) and written back at the end. Writes
// the per-layer (id, entry) copy lists. With too few free entries nothing
// but the hit stamps changes and the range flag gets bit 2.
__global__ __launch_bounds__(kCacheThreads) void k_cache_policy(
    int E, int C, int K, int layer0, int n_layers, int tick, int32_t* slot_of, int32_t* owner,
    int32_t* stamp, const int32_t* next, int32_t* copy_list, int32_t* n_copies,
    unsigned long long* total, int32_t* flags) {
  __shared__ uint64_t key[kMaxCacheEntries];
  __shared__ int32_t own_l[kMaxCacheEntries], stm_l[kMaxCacheEntries];
  __shared__ int32_t mis[kMaxCacheLayers * 8];
  __shared__ int32_t nmis[kMaxCacheLayers], moff[kMaxCacheLayers + 1];
  __shared__ int bad;
  const int t = threadIdx.x, nt = blockDim.x, nk = n_layers * K;
  if (t == 0) bad = 0;
  for (int c = t; c < C; c += nt) {
    own_l[c] = owner[c];
    stm_l[c] = stamp[c];
  }
  __syncthreads();
  for (int i = t; i < nk; i += nt)
    if (next[i] < 0 || next[i] >= E) bad = 1;
  __syncthreads();
  if (bad) {
    if (t == 0) atomicOr(&flags[FLAG_RANGE], 1);
    for (int l = t; l < n_layers; l += nt) n_copies[l] = 0;
    return;
  }
  // hits: refresh the entry's stamp (every writer stores the same value)
  for (int i = t; i < nk; i += nt) {
    const int c = slot_of[(int64_t)(layer0 + i / K) * E + next[i]];
    if (c >= 0) stm_l[c] = tick;
  }
  // misses of each layer, ascending and without repeats (a thread per layer)
  if (t < n_layers) {
    const int64_t row = (int64_t)(layer0 + t) * E;
    int m[8];
    int nm = 0;
    for (int k = 0; k < K; ++k) {
      const int e = next[t * K + k];
      if (slot_of[row + e] >= 0) continue;
      bool dup = false;
      for (int i = 0; i < nm; ++i) dup |= (m[i] == e);
      if (dup) continue;
      int i = nm++;
      while (i > 0 && m[i - 1] > e) {
        m[i] = m[i - 1];
        --i;
      }
      m[i] = e;
    }
    for (int i = 0; i < nm; ++i) mis[t * 8 + i] = m[i];
    nmis[t] = nm;
  }
  __syncthreads();
  if (t == 0) {
    moff[0] = 0;
    for (int l = 0; l < n_layers; ++l) moff[l + 1] = moff[l] + nmis[l];
  }
  // free entries keyed by (stamp, index) (stamp + 1 >= 0); others sort last
  int P = 1;
  while (P < C) P <<= 1;
  for (int c = t; c < P; c += nt) {
    uint64_t kk = ~0ull;
    if (c < C && (own_l[c] < 0 || stm_l[c] < tick - 1))
      kk = ((uint64_t)(uint32_t)(stm_l[c] + 1) << 32) | (uint32_t)c;
    key[c] = kk;
  }
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = t; i < P; i += nt) {
        const int x = i ^ j;
        if (x > i) {
          const uint64_t a = key[i], b = key[x];
          if ((a > b) == ((i & k) == 0)) {
            key[i] = b;
            key[x] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  const int m_total = moff[n_layers];
  const bool overflow = m_total > C || (m_total > 0 && key[m_total - 1] == ~0ull);
  if (!overflow) {
    for (int j = t; j < m_total; j += nt) {
      int li = 0;
      while (moff[li + 1] <= j) ++li;
      const int r = j - moff[li], e = mis[li * 8 + r];
      const int c = (int)(uint32_t)key[j];
      const int old = own_l[c];
      if (old >= 0) slot_of[old] = -1;  // old = layer * E + id
      own_l[c] = (layer0 + li) * E + e;
      stm_l[c] = tick;
      slot_of[(int64_t)(layer0 + li) * E + e] = c;
      copy_list[li * 16 + 2 * r] = e;
      copy_list[li * 16 + 2 * r + 1] = c;
    }
  }
  for (int l = t; l < n_layers; l += nt) n_copies[l] = overflow ? 0 : nmis[l];
  if (t == 0) {
    if (overflow)
      atomicOr(&flags[FLAG_RANGE], 2);
    else
      atomicAdd(total, (unsigned long long)m_total);
  }
  __syncthreads();
  for (int c = t; c < C; c += nt) {
    owner[c] = own_l[c];
    stamp[c] = stm_l[c];
  }
}

}  // namespace

hipError_t launch_cache_stage(int E, int C, int K, int layer0, int n_layers, int tick,
                              int32_t* slot_of, int32_t* owner, int32_t* stamp,
                              const int32_t* next, int32_t* copy_list, int32_t* n_copies,
                              unsigned long long* total, const char* host, int64_t host_stride,
                              char* cache, int64_t bundle, int32_t* flags, hipStream_t st) {
  if (E > kMaxE || C < 1 || C > kMaxCacheEntries || K > 8 || n_layers < 1 ||
      n_layers > kMaxCacheLayers || bundle % 16)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_cache_policy, dim3(1), dim3(kCacheThreads), 0, st, E, C, K, layer0,
                     n_layers, tick, slot_of, owner, stamp, next, copy_list, n_copies, total,
                     flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // copies: host pool of the call's layers -> cache entries (one pool, no
  // per-layer stride on the device side)
  hipLaunchKernelGGL(k_stage_copy, dim3(kCopyBlocks), dim3(kCopyThreads), 0, st, host,
                     host_stride, cache, (int64_t)0, bundle, n_layers, copy_list, n_copies);
  return hipGetLastError();
}

hipError_t launch_stage(int E, int n_slots, int K, int n_layers, int32_t* slot_of,
                        int32_t* slot_expert, const int32_t* in_use, const int32_t* next,
                        int32_t* copy_list, int32_t* n_copies, unsigned long long* total,
                        const char* host, int64_t host_stride, char* hbm, int64_t hbm_stride,
                        int64_t bundle, int32_t* flags, hipStream_t st) {
  if (E > kMaxE || n_slots > kMaxSlots || K > 8 || bundle % 16 || n_layers < 1)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_slot_policy, dim3(n_layers), dim3(64), 0, st, E, n_slots, K, slot_of,
                     slot_expert, in_use, next, copy_list, n_copies, total, flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_stage_copy, dim3(kCopyBlocks), dim3(kCopyThreads), 0, st, host,
                     host_stride, hbm, hbm_stride, bundle, n_layers, copy_list, n_copies);
  return hipGetLastError();
}

}  // namespace smd
