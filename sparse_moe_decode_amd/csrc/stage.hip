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

}  // namespace

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
