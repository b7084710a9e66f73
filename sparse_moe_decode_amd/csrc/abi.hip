// C-ABI entry points: argument validation, device scratch, and the launch
// sequences of the decode step. Declarations and documentation are in
// include/sparse_moe_decode.h.

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "internal.h"

namespace smd {
bool q4_shape_ok(int cols);
}  // namespace smd

using namespace smd;

namespace {

// Token count from which moe_int4_decode groups tokens by expert and runs
// grouped int4 GEMMs on MFMA (tiles of up to 32 or 64 of an expert's tokens).
constexpr int kBatchedMin = 16;

thread_local std::string g_err = "no error";

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(E0_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

// The error channel of e0_last_error for the other translation units.
int smd_report(int code, const char* msg) { return fail(code, "%s", msg); }

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

struct e0_ctx {
  e0_spec spec;
  Dims dm;
  int device;
  Scratch s;
  void* block;
};

struct e0_model {
  e0_ctx* ctx;
  std::vector<e0_layer> layers;
  LayerDev* dev_table;  // device copy of the layer table (persistent kernel)
  void* xbuf;           // exchange words of the persistent kernel (one block)
  uint64_t *xh, *xg, *xr, *xa, *xl;
  int32_t ng;
  uint32_t epoch;
  int32_t path;
  int32_t grid;  // workgroups of the persistent kernels (one per compute unit)
  int32_t cus;   // compute units of the device
  uint64_t* trace;
  int32_t trace_grid;  // grid the trace buffer was sized for
  // streaming kernel: exchange words [L][xlayer] and the role split
  uint64_t* fxbuf;
  int64_t fxwords;
  uint32_t fx_clean;  // every exchange word is zero or was written after this epoch
  uint32_t cx_clean;  // the same for the packed words of the layer-ahead slot kernel (in xg)
  int32_t fng, fnd;  // explicit split (0, 0: automatic)
};

namespace {

// Gate/up and down workgroups of the streaming kernel for a launch of nL
// layers on the model's grid; false when it does not fit.
bool flow_roles(const e0_model* m, int nL, int& ng, int& nd) {
  const Dims& dm = m->ctx->dm;
  if (!flow_supported(dm) || m->grid < 2) return false;
  if (m->fng > 0 && m->fnd > 0) {
    if (m->fng + m->fnd != m->grid) return false;
    ng = m->fng;
    nd = m->fnd;
    return flow_plan(dm, ng, nd, nL).ok != 0;
  }
  return flow_default_roles(dm, m->grid, nL, ng, nd);
}

// Size the streaming kernel's exchange words for the current split.
hipError_t flow_alloc(e0_model* m) {
  int ng, nd;
  const int L = (int)m->layers.size();
  if (!flow_roles(m, L < 64 ? L : 64, ng, nd)) return hipSuccess;
  const FlowPlan p = flow_plan(m->ctx->dm, ng, nd, L < 64 ? L : 64);
  const int64_t need = (int64_t)L * p.xlayer;
  if (need <= m->fxwords) return hipSuccess;
  if (m->fxbuf) (void)hipFree(m->fxbuf);
  m->fxbuf = nullptr;
  m->fxwords = 0;
  hipError_t e = hipMalloc(&m->fxbuf, need * 8);
  if (e == hipSuccess) e = hipMemset(m->fxbuf, 0, need * 8);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) {
    m->fxwords = need;
    m->fx_clean = m->epoch;
  }
  return e;
}

// Validates a tier description and fills the kernels' dimensions.
int spec_dims(const e0_spec& p, Dims& dm) {
  if (p.d_model <= 0 || p.n_experts <= 0 || p.top_k < 1 || p.top_k > 8 ||
      p.top_k > p.n_experts || p.inter <= 0 || p.group <= 0)
    return fail(E0_ERR_ARG, "spec: bad dimensions");
  if (p.quant != E0_QUANT_SYMMETRIC && p.quant != E0_QUANT_AFFINE)
    return fail(E0_ERR_ARG, "spec: unknown int4 codec %d", p.quant);
  if (p.group % 32 || p.d_model % p.group || p.inter % p.group)
    return fail(E0_ERR_SHAPE, "spec: group %d must be a multiple of 32 dividing d and I",
                p.group);
  if (!q4_shape_ok(p.d_model) || !q4_shape_ok(p.inter))
    return fail(E0_ERR_SHAPE, "spec: d=%d or I=%d not supported by the int4 kernels",
                p.d_model, p.inter);
  if (p.shared_inter != 0 && p.shared_inter != p.inter)
    return fail(E0_ERR_SHAPE, "spec: shared_inter must be 0 or equal to inter");
  if (p.lora_rank < 0 || p.lora_rank > 64) return fail(E0_ERR_SHAPE, "spec: rank > 64");
  if (p.n_experts > 512) return fail(E0_ERR_SHAPE, "spec: more than 512 experts");
  if (p.head_hidden < 0 || p.head_hidden % 8 || (p.d_model + 2 * p.n_experts) % 8)
    return fail(E0_ERR_SHAPE, "spec: head dims must be multiples of 8");
  if (p.router_kind == E0_ROUTER_SIGMOID_GROUP) {
    if (p.n_groups < 1 || p.n_groups > 64 || p.n_experts % p.n_groups ||
        p.n_experts / p.n_groups < 2 || p.topk_groups < 1 || p.topk_groups > p.n_groups ||
        p.top_k > p.topk_groups * (p.n_experts / p.n_groups))
      return fail(E0_ERR_SHAPE, "spec: bad sigmoid-group parameters");
  } else if (p.router_kind != E0_ROUTER_SOFTMAX_TOPK) {
    return fail(E0_ERR_ARG, "spec: unknown router kind");
  }
  dm = Dims{};
  dm.d = p.d_model; dm.E = p.n_experts; dm.K = p.top_k; dm.I = p.inter; dm.Is = p.shared_inter;
  dm.P = p.head_hidden; dm.G = p.group; dm.r = p.lora_rank;
  dm.lora_scale = p.lora_rank > 0 ? p.lora_alpha / (float)p.lora_rank : 0.0f;
  dm.router_kind = p.router_kind; dm.norm_topk = p.norm_topk; dm.n_groups = p.n_groups;
  dm.topk_groups = p.topk_groups; dm.route_scale = p.route_scale;
  dm.eps = p.rms_eps > 0 ? p.rms_eps : 1e-6f;
  dm.affine = p.quant == E0_QUANT_AFFINE;
  return E0_OK;
}

// Byte size of the scratch for B tokens; with base != nullptr also carves
// the buffers of *s out of [base, base + size) (every buffer 256-byte aligned).
size_t scratch_layout(const Dims& dm, int B, char* base, Scratch* s) {
  const int imax = dm.I > dm.Is ? dm.I : dm.Is;
  const int rmax = dm.r > 1 ? dm.r : 1;
  const size_t n_gu = (size_t)B * (dm.K + 1) * imax;
  const size_t n_ax = (size_t)B * 3 * rmax;
  const size_t n_d = (size_t)B * dm.d;
  const size_t n_p = (size_t)B * (dm.P > 0 ? dm.P : 1);
  const size_t n_e = (size_t)B * dm.E;
  const size_t n_grp = batched_grp_ints(B, dm.K, dm.E);
  const size_t n_slot = (size_t)B * (dm.K + 1);
  const size_t n_axp = (size_t)kLoraSlices * B * 2 * rmax;
  auto up = [](size_t bytes) { return (bytes + 255) & ~(size_t)255; };
  const size_t sizes[] = {up(n_gu * 4), up(n_ax * 4), up(n_d * 4), up(n_d * 2), up(n_p * 4),
                          up(n_e * 4), up(n_e * 4), up((size_t)B * dm.K * 4),
                          up((size_t)B * dm.K * 4), up(N_FLAGS * 4), up(n_grp * 4),
                          up(n_axp * 4), up(n_slot * dm.d * 4)};
  size_t total = 0;
  for (size_t z : sizes) total += z;
  if (base) {
    char* q = base;
    void* ptrs[13];
    for (int i = 0; i < 13; ++i) {
      ptrs[i] = q;
      q += sizes[i];
    }
    s->max_tokens = B;
    s->gu = (float*)ptrs[0];
    s->ax = (float*)ptrs[1];
    s->hattn = (float*)ptrs[2];
    s->xn = (uint16_t*)ptrs[3];
    s->hact = (float*)ptrs[4];
    s->hlin = (float*)ptrs[5];
    s->logits = (float*)ptrs[6];
    s->sink_idx = (int32_t*)ptrs[7];
    s->sink_w = (float*)ptrs[8];
    s->flags = (int32_t*)ptrs[9];
    s->grp = (int32_t*)ptrs[10];
    s->axp = (float*)ptrs[11];
    s->yk = (float*)ptrs[12];
  }
  return total;
}

}  // namespace

extern "C" {

const char* e0_last_error(void) { return g_err.c_str(); }

int e0_create(const e0_spec* spec, int32_t max_tokens, e0_ctx** out) {
  if (!spec || !out) return fail(E0_ERR_ARG, "e0_create: null argument");
  *out = nullptr;
  if (max_tokens < 1 || max_tokens > 8192)
    return fail(E0_ERR_ARG, "e0_create: max_tokens %d outside [1, 8192]", max_tokens);
  Dims dm;
  int rc;
  if ((rc = spec_dims(*spec, dm))) return rc;
  e0_ctx* c = new e0_ctx();
  c->spec = *spec;
  c->dm = dm;
  if (hipGetDevice(&c->device) != hipSuccess) {
    delete c;
    return fail(E0_ERR_HIP, "e0_create: no current HIP device");
  }
  const size_t bytes = scratch_layout(dm, max_tokens, nullptr, nullptr);
  hipError_t e = hipMalloc(&c->block, bytes);
  if (e != hipSuccess) {
    delete c;
    return hip_fail(e, "e0_create: hipMalloc");
  }
  e = hipMemset(c->block, 0, bytes);
  if (e != hipSuccess) {
    (void)hipFree(c->block);
    delete c;
    return hip_fail(e, "e0_create: hipMemset");
  }
  scratch_layout(dm, max_tokens, (char*)c->block, &c->s);
  *out = c;
  return E0_OK;
}

void e0_destroy(e0_ctx* ctx) {
  if (!ctx) return;
  (void)hipFree(ctx->block);
  delete ctx;
}

int e0_device_status(e0_ctx* ctx, void* stream) {
  if (!ctx) return fail(E0_ERR_ARG, "e0_device_status: null ctx");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "e0_device_status: sync");
  int32_t flags[N_FLAGS];
  e = hipMemcpy(flags, ctx->s.flags, sizeof(flags), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "e0_device_status: copy");
  e = hipMemset(ctx->s.flags, 0, sizeof(flags));
  if (e != hipSuccess) return hip_fail(e, "e0_device_status: clear");
  if (flags[FLAG_SYNC]) return fail(E0_ERR_SYNC, "a device-side wait hit its spin limit");
  if (flags[FLAG_RANGE]) return fail(E0_ERR_RANGE, "an expert id or slot was out of range");
  return E0_OK;
}

}  // extern "C"

namespace {

int check_q4(const e0_q4& m, bool affine, const char* what) {
  if (!m.q || !m.s) return fail(E0_ERR_ARG, "%s: null int4 matrix", what);
  if (affine != (m.b != nullptr))
    return fail(E0_ERR_ARG, "%s: biases must be given for the affine codec and only for it",
                what);
  if (!aligned(m.q, 16) || !aligned(m.s, 2) || (m.b && !aligned(m.b, 2)))
    return fail(E0_ERR_ALIGN, "%s: packed words must be 16-byte aligned", what);
  return E0_OK;
}

int make_pool(const Dims& dm, const e0_experts* ex, const int32_t* slot_of, Pool& p) {
  if (!ex) return fail(E0_ERR_ARG, "routed pool is null");
  int rc;
  const bool af = dm.affine != 0;
  if ((rc = check_q4(ex->gate, af, "routed gate")) || (rc = check_q4(ex->up, af, "routed up")) ||
      (rc = check_q4(ex->down, af, "routed down")))
    return rc;
  p.gate = {ex->gate.q, ex->gate.s, ex->gate.b};
  p.up = {ex->up.q, ex->up.s, ex->up.b};
  p.down = {ex->down.q, ex->down.s, ex->down.b};
  p.stride_q = ex->stride_q ? ex->stride_q : (int64_t)dm.I * dm.d / 2;
  p.stride_s = ex->stride_s ? ex->stride_s : (int64_t)2 * dm.I * (dm.d / dm.G);
  if (p.stride_q % 16 || p.stride_s % 2) return fail(E0_ERR_ALIGN, "pool strides misaligned");
  p.count = ex->count;
  if (p.count < 1) return fail(E0_ERR_ARG, "routed pool count must be >= 1");
  p.slot_of = slot_of;
  return E0_OK;
}

int make_shared(const Dims& dm, const e0_shared* sh, SharedW& w) {
  std::memset(&w, 0, sizeof(w));
  if (!sh) return E0_OK;
  if (dm.Is == 0) return fail(E0_ERR_ARG, "shared expert given but shared_inter = 0");
  int rc;
  const bool af = dm.affine != 0;
  if ((rc = check_q4(sh->gate, af, "shared gate")) || (rc = check_q4(sh->up, af, "shared up")) ||
      (rc = check_q4(sh->down, af, "shared down")))
    return rc;
  w.gate = {sh->gate.q, sh->gate.s, sh->gate.b};
  w.up = {sh->up.q, sh->up.s, sh->up.b};
  w.down = {sh->down.q, sh->down.s, sh->down.b};
  const bool lg = sh->lgate.a && sh->lgate.b, lu = sh->lup.a && sh->lup.b,
             ld = sh->ldown.a && sh->ldown.b;
  if ((lg || lu || ld) && dm.r == 0) return fail(E0_ERR_ARG, "LoRA given but rank = 0");
  if (lg != lu) return fail(E0_ERR_ARG, "gate and up LoRA must be given together");
  for (const uint16_t* a : {sh->lgate.a, sh->lup.a, sh->ldown.a})
    if (a && !aligned(a, 16)) return fail(E0_ERR_ALIGN, "LoRA A must be 16-byte aligned");
  if (lg) { w.ag = sh->lgate.a; w.bg = sh->lgate.b; w.au = sh->lup.a; w.bu = sh->lup.b; }
  if (ld) { w.ad = sh->ldown.a; w.bd = sh->ldown.b; }
  w.present = 1;
  return E0_OK;
}

// Shared-expert LoRA A products for the gate/up (input x fp16).
hipError_t lora_a_x(const Dims& dm, const Scratch& s, const SharedW& sh, const uint16_t* x,
                    int B, hipStream_t st) {
  if (!sh.present || !sh.ag) return hipSuccess;
  const int rmax = dm.r > 1 ? dm.r : 1;
  const uint16_t* A[2] = {sh.ag, sh.au};
  const int slots[2] = {0, rmax};
  return launch_lora_a(2, A, slots, dm.d, dm.r, x, nullptr, dm.d, B, s.ax, 3 * rmax, st);
}

// Down LoRA A product on the shared expert's fp32 SwiGLU output.
hipError_t lora_a_down(const Dims& dm, const Scratch& s, const SharedW& sh, int B,
                       hipStream_t st) {
  if (!sh.present || !sh.ad) return hipSuccess;
  const int rmax = dm.r > 1 ? dm.r : 1;
  const int imax = dm.I > dm.Is ? dm.I : dm.Is;
  const uint16_t* A[1] = {sh.ad};
  const int slots[1] = {2 * rmax};
  return launch_lora_a(1, A, slots, dm.Is, dm.r, nullptr, s.gu + (int64_t)dm.K * imax,
                       (int64_t)(dm.K + 1) * imax, B, s.ax, 3 * rmax, st);
}

// The routed experts and the shared expert of n_tokens tokens on scratch s
// (sized for at least n_tokens).
int moe_run(const Dims& dm, const Scratch& s, const e0_experts* routed, const int32_t* slot_of,
            const e0_shared* shared, const uint16_t* x, const int32_t* idx, const float* w,
            int n_tokens, uint16_t* y, hipStream_t st) {
  Pool pool;
  SharedW sh;
  int rc;
  if ((rc = make_pool(dm, routed, slot_of, pool)) || (rc = make_shared(dm, shared, sh))) return rc;
  hipError_t e;
  if (n_tokens >= kBatchedMin && batched_supported(dm)) {
    // the whole batch through the grouped MFMA path: each expert's weights
    // are read once for all of its tokens
    if ((e = launch_batched(dm, pool, sh, x, idx, w, n_tokens, y, s, st)) != hipSuccess)
      return hip_fail(e, "batched");
    return E0_OK;
  }
  if ((e = lora_a_x(dm, s, sh, x, n_tokens, st)) != hipSuccess) return hip_fail(e, "lora A");
  if ((e = launch_gate_up(dm, pool, sh, x, idx, n_tokens, s, st)) != hipSuccess)
    return hip_fail(e, "gate/up");
  if ((e = lora_a_down(dm, s, sh, n_tokens, st)) != hipSuccess) return hip_fail(e, "lora A down");
  if ((e = launch_down(dm, pool, sh, idx, w, n_tokens, nullptr, y, s, st)) != hipSuccess)
    return hip_fail(e, "down");
  return E0_OK;
}

}  // namespace

extern "C" {

int moe_int4_decode(e0_ctx* ctx, const e0_experts* routed, const int32_t* slot_of,
                    const e0_shared* shared, const uint16_t* x, const int32_t* idx,
                    const float* w, int32_t n_tokens, uint16_t* y, void* stream) {
  if (!ctx || !x || !idx || !w || !y) return fail(E0_ERR_ARG, "moe_int4_decode: null argument");
  if (n_tokens == 0) return E0_OK;
  if (n_tokens < 0 || n_tokens > ctx->s.max_tokens)
    return fail(E0_ERR_ARG, "moe_int4_decode: n_tokens %d outside [0, %d]", n_tokens,
                ctx->s.max_tokens);
  return moe_run(ctx->dm, ctx->s, routed, slot_of, shared, x, idx, w, n_tokens, y,
                 (hipStream_t)stream);
}

int lora_delta(e0_ctx* ctx, const uint16_t* A, const uint16_t* Bm, int32_t in_dim,
               int32_t out_dim, int32_t rank, float scale, const uint16_t* x, float* y_acc,
               int32_t n_tokens, void* stream) {
  if (!ctx || !A || !Bm || !x || !y_acc) return fail(E0_ERR_ARG, "lora_delta: null argument");
  if (n_tokens == 0) return E0_OK;
  if (n_tokens < 0 || n_tokens > ctx->s.max_tokens)
    return fail(E0_ERR_ARG, "lora_delta: n_tokens out of range");
  if (rank < 1 || rank > 64 || in_dim < 8 || in_dim % 8 || out_dim < 1)
    return fail(E0_ERR_SHAPE, "lora_delta: rank in [1, 64], in_dim a multiple of 8");
  if (!aligned(A, 16) || !aligned(x, 16))
    return fail(E0_ERR_ALIGN, "lora_delta: A and x must be 16-byte aligned");
  const int rmax = ctx->dm.r > 1 ? ctx->dm.r : 1;
  if (rank > 3 * rmax) return fail(E0_ERR_SHAPE, "lora_delta: rank larger than the context's");
  hipStream_t st = (hipStream_t)stream;
  const int slots[1] = {0};
  hipError_t e = launch_lora_a(1, &A, slots, in_dim, rank, x, nullptr, in_dim, n_tokens,
                               ctx->s.ax, 3 * rmax, st);
  if (e != hipSuccess) return hip_fail(e, "lora_delta A");
  e = launch_lora_b(Bm, out_dim, rank, scale, ctx->s.ax, 3 * rmax, y_acc, n_tokens, st);
  if (e != hipSuccess) return hip_fail(e, "lora_delta B");
  return E0_OK;
}

}  // extern "C"

namespace {

int check_head(const e0_ctx* ctx, const e0_head* hd) {
  if (!hd || !hd->fc1 || !hd->fc2 || !hd->lin) return fail(E0_ERR_ARG, "head: null weights");
  if (ctx->dm.P <= 0) return fail(E0_ERR_SHAPE, "head: head_hidden is 0");
  if (!aligned(hd->fc1, 16) || !aligned(hd->fc2, 16) || !aligned(hd->lin, 16))
    return fail(E0_ERR_ALIGN, "head: weights must be 16-byte aligned");
  return E0_OK;
}

// fc1 (+GELU) and lin on [x; onehot(cur); onehot(prev)], then fc2 + lin,
// then routing. logits_out may alias the scratch logits.
hipError_t head_launch(const e0_ctx* ctx, const e0_head* hd, const uint16_t* x,
                       const int32_t* cur, const int32_t* prev, int B, float* logits_out,
                       int32_t* out_idx, float* out_w, hipStream_t st) {
  const Dims& dm = ctx->dm;
  const Scratch& s = ctx->s;
  const int64_t F = (int64_t)dm.d + 2 * dm.E;
  hipError_t e = launch_gemv16(hd->fc1, dm.P, dm.d, F, x, nullptr, dm.d, B, cur, prev, dm.K,
                               dm.E, dm.d, 1, nullptr, s.hact, dm.P, st);
  if (e != hipSuccess) return e;
  e = launch_gemv16(hd->lin, dm.E, dm.d, F, x, nullptr, dm.d, B, cur, prev, dm.K, dm.E, dm.d, 0,
                    nullptr, s.hlin, dm.E, st);
  if (e != hipSuccess) return e;
  float* lg = logits_out ? logits_out : s.logits;
  e = launch_gemv16(hd->fc2, dm.E, dm.P, dm.P, nullptr, s.hact, dm.P, B, nullptr, nullptr, 0,
                    0, 0, 2, s.hlin, lg, dm.E, st);
  if (e != hipSuccess) return e;
  return launch_route(dm, lg, hd->bias, B, out_idx, out_w, s.flags, st);
}

}  // namespace

extern "C" {

int prerouter_forward(e0_ctx* ctx, const e0_head* head, const uint16_t* x,
                      const int32_t* cur_idx, const int32_t* prev_idx, int32_t n_tokens,
                      float* logits, int32_t* out_idx, float* out_w, void* stream) {
  if (!ctx || !x || !cur_idx || !out_idx || !out_w)
    return fail(E0_ERR_ARG, "prerouter_forward: null argument");
  int rc = check_head(ctx, head);
  if (rc) return rc;
  if (n_tokens == 0) return E0_OK;
  if (n_tokens < 0 || n_tokens > ctx->s.max_tokens)
    return fail(E0_ERR_ARG, "prerouter_forward: n_tokens out of range");
  if (!aligned(x, 16)) return fail(E0_ERR_ALIGN, "prerouter_forward: x must be 16-byte aligned");
  hipError_t e = head_launch(ctx, head, x, cur_idx, prev_idx, n_tokens, logits, out_idx, out_w,
                             (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "prerouter_forward");
  return E0_OK;
}

int e0_model_create(e0_ctx* ctx, const e0_layer* layers, int32_t n_layers, e0_model** out) {
  if (!ctx || !layers || !out || n_layers < 1)
    return fail(E0_ERR_ARG, "e0_model_create: bad argument");
  *out = nullptr;
  for (int l = 0; l < n_layers; ++l) {
    const e0_layer& L = layers[l];
    Pool p;
    SharedW sw;
    int rc;
    if ((rc = make_pool(ctx->dm, &L.experts, L.slot_of, p)) ||
        (rc = make_shared(ctx->dm, L.shared.gate.q ? &L.shared : nullptr, sw)))
      return fail(rc, "layer %d: %s", l, g_err.c_str());
    if (L.head.fc1 && (rc = check_head(ctx, &L.head)))
      return fail(rc, "layer %d: %s", l, g_err.c_str());
    if (L.router && !aligned(L.router, 16))
      return fail(E0_ERR_ALIGN, "layer %d: router must be 16-byte aligned", l);
  }
  e0_model* m = new e0_model();
  m->ctx = ctx;
  m->layers.assign(layers, layers + n_layers);
  m->dev_table = nullptr;
  m->xbuf = nullptr;
  m->xh = m->xg = m->xr = m->xa = m->xl = nullptr;
  m->epoch = 0;
  m->path = E0_PATH_AUTO;
  m->grid = 0;
  m->trace = nullptr;
  m->trace_grid = 0;
  m->fxbuf = nullptr;
  m->fxwords = 0;
  m->fng = m->fnd = 0;
  m->fx_clean = 0;
  m->cx_clean = 0;
  const Dims& dm = ctx->dm;
  // Device table of the layers for the persistent kernel.
  std::vector<LayerDev> table(n_layers);
  int ng = 0;
  for (int l = 0; l < n_layers; ++l) {
    const e0_layer& L = layers[l];
    LayerDev& t = table[l];
    make_pool(ctx->dm, &L.experts, L.slot_of, t.pool);
    make_shared(ctx->dm, L.shared.gate.q ? &L.shared : nullptr, t.sh);
    t.router = L.router;
    t.router_bias = L.router_bias;
    t.head = HeadW{L.head.fc1, L.head.fc2, L.head.lin, L.head.bias};
    if (!L.head.fc1) t.head = HeadW{nullptr, nullptr, nullptr, nullptr};
    t.attn = L.attn;
    const int Is = t.sh.present ? dm.Is : 0;
    const int r2 = (t.sh.present && t.sh.ag) ? 2 * dm.r : 0;
    // exchange words of a layer: routed SwiGLU outputs, shared SwiGLU
    // outputs, (layer-ahead slot kernel, down LoRA) partial A_down products,
    // the shared gate/up LoRA A products
    const int n_ad = (t.sh.present && t.sh.ad) ? 16 * kChainSO : 0;
    const int n = dm.K * dm.I + Is + n_ad + r2;
    if (n > ng) ng = n;
  }
  m->ng = (ng + 1) & ~1;  // layer rows of xg stay 16-byte aligned (16-byte polls)
  if (stack_supported(dm)) {
    hipError_t e = hipMalloc(&m->dev_table, sizeof(LayerDev) * n_layers);
    if (e == hipSuccess)
      e = hipMemcpy(m->dev_table, table.data(), sizeof(LayerDev) * n_layers,
                    hipMemcpyHostToDevice);
    const size_t wh = (size_t)n_layers * (dm.d / 2), wg = (size_t)n_layers * ng,
                 wr = (size_t)n_layers * dm.E, wa = (size_t)n_layers * (dm.P + dm.E),
                 wl = (size_t)n_layers * dm.E;
    int dev = 0, cus = 0;
    if (e == hipSuccess) e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const size_t words = wh + wg + wr + wa + wl;
    if (e == hipSuccess) e = hipMalloc(&m->xbuf, words * 8);
    if (e == hipSuccess) e = hipMemset(m->xbuf, 0, words * 8);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      e0_model_destroy(m);
      return hip_fail(e, "e0_model_create: persistent-kernel buffers");
    }
    uint64_t* w = (uint64_t*)m->xbuf;
    m->xh = w; w += wh;
    m->xg = w; w += wg;
    m->xr = w; w += wr;
    m->xa = w; w += wa;
    m->xl = w; w += wl;
    m->grid = cus;
    m->cus = cus;
    if ((e = flow_alloc(m)) != hipSuccess) {
      e0_model_destroy(m);
      return hip_fail(e, "e0_model_create: streaming-kernel buffers");
    }
  }
  *out = m;
  return E0_OK;
}

void e0_model_destroy(e0_model* model) {
  if (!model) return;
  if (model->dev_table) (void)hipFree(model->dev_table);
  if (model->xbuf) (void)hipFree(model->xbuf);
  if (model->fxbuf) (void)hipFree(model->fxbuf);
  delete model;
}

int e0_model_set_trace(e0_model* model, uint64_t* trace) {
  if (!model) return fail(E0_ERR_ARG, "e0_model_set_trace: null model");
  model->trace = trace;
  model->trace_grid = trace ? model->grid : 0;
  return E0_OK;
}

int32_t e0_model_trace_shape(e0_model* model, int32_t* grid, int32_t* rows, int32_t* points) {
  if (!model) return fail(E0_ERR_ARG, "e0_model_trace_shape: null model");
  if (grid) *grid = model->grid;
  if (rows) *rows = (int32_t)model->layers.size() + 1;
  if (points) *points = kTracePoints;
  return E0_OK;
}

int e0_model_set_grid(e0_model* model, int32_t grid) {
  if (!model || grid < 0) return fail(E0_ERR_ARG, "e0_model_set_grid: bad argument");
  if (!model->dev_table)
    return fail(E0_ERR_SHAPE, "e0_model_set_grid: shapes not supported by the persistent kernel");
  if (grid > model->cus)
    return fail(E0_ERR_ARG, "e0_model_set_grid: %d workgroups exceed the %d compute units", grid,
                model->cus);
  model->grid = grid == 0 ? model->cus : grid;
  if (model->trace && model->grid > model->trace_grid) {
    model->trace = nullptr;  // sized for a smaller grid: dropped
    model->trace_grid = 0;
  }
  if (model->fng + model->fnd != model->grid) model->fng = model->fnd = 0;
  const hipError_t e = flow_alloc(model);
  if (e != hipSuccess) return hip_fail(e, "e0_model_set_grid: streaming-kernel buffers");
  return E0_OK;
}

int e0_model_set_roles(e0_model* model, int32_t n_gate_up, int32_t n_down) {
  if (!model || n_gate_up < 0 || n_down < 0)
    return fail(E0_ERR_ARG, "e0_model_set_roles: bad argument");
  if (!model->dev_table || !flow_supported(model->ctx->dm))
    return fail(E0_ERR_SHAPE, "e0_model_set_roles: shapes not supported by the streaming kernel");
  if ((n_gate_up == 0) != (n_down == 0))
    return fail(E0_ERR_ARG, "e0_model_set_roles: give both counts or neither");
  if (n_gate_up && n_gate_up + n_down != model->grid)
    return fail(E0_ERR_ARG, "e0_model_set_roles: %d + %d workgroups differ from the grid %d",
                n_gate_up, n_down, model->grid);
  const int L = (int)model->layers.size();
  if (n_gate_up && !flow_plan(model->ctx->dm, n_gate_up, n_down, L < 64 ? L : 64).ok)
    return fail(E0_ERR_SHAPE, "e0_model_set_roles: split %d + %d does not fit the kernel",
                n_gate_up, n_down);
  model->fng = n_gate_up;
  model->fnd = n_down;
  const hipError_t e = flow_alloc(model);
  if (e != hipSuccess) return hip_fail(e, "e0_model_set_roles: streaming-kernel buffers");
  return E0_OK;
}

int e0_model_set_path(e0_model* model, int32_t path) {
  if (!model || path < E0_PATH_AUTO || path > E0_PATH_CHAIN)
    return fail(E0_ERR_ARG, "e0_model_set_path: bad argument");
  if ((path == E0_PATH_PERSISTENT || path == E0_PATH_CHAIN) && !model->dev_table)
    return fail(E0_ERR_SHAPE, "e0_model_set_path: shapes not supported by the persistent kernel");
  if (path == E0_PATH_FLOW && (!model->dev_table || !flow_supported(model->ctx->dm)))
    return fail(E0_ERR_SHAPE, "e0_model_set_path: shapes not supported by the streaming kernel");
  model->path = path;
  return E0_OK;
}

int layer_step(e0_ctx* ctx, e0_model* model, int32_t layer_begin, int32_t layer_end,
               const e0_state* state, int32_t token, uint16_t* h, void* stream) {
  if (!ctx || !model || !state || !h) return fail(E0_ERR_ARG, "layer_step: null argument");
  const int L = (int)model->layers.size();
  if (layer_begin < 0 || layer_end > L || layer_begin >= layer_end || token < 0)
    return fail(E0_ERR_ARG, "layer_step: bad layer range or token");
  if (!state->route_idx || !state->route_w || !state->exec_idx || !state->exec_w)
    return fail(E0_ERR_ARG, "layer_step: state buffers are null");
  if (state->n_layers != L)
    return fail(E0_ERR_ARG, "layer_step: state sized for %d layers, the model has %d",
                state->n_layers, L);
  if (!aligned(h, 16) || (ctx->dm.d * 2) % 16)
    return fail(E0_ERR_ALIGN, "layer_step: h must be 16-byte aligned");
  const Dims& dm = ctx->dm;
  const Scratch& s = ctx->s;
  hipStream_t st = (hipStream_t)stream;
  const int K = dm.K;
  const int cur = token & 1, nxt = (token + 1) & 1;
  if (model->trace && model->grid > model->trace_grid)
    return fail(E0_ERR_ARG, "layer_step: the trace buffer is sized for a smaller grid");
  const int nL = layer_end - layer_begin;
  // The streaming kernel, when the layer range fits it: sets `launched`.
  auto run_flow = [&](bool& launched) -> int {
    launched = false;
    if (!model->dev_table) return E0_OK;
    int ng = 0, nd = 0;
    FlowArgs a;
    bool ok = flow_roles(model, nL, ng, nd);
    if (ok) {
      a.pl = flow_plan(dm, ng, nd, nL);
      ok = a.pl.ok && (int64_t)L * a.pl.xlayer <= model->fxwords;
    }
    if (!ok) return E0_OK;
    a.dm = dm;
    a.layers = model->dev_table;
    a.L = L;
    a.l0 = layer_begin;
    a.l1 = layer_end;
    a.token = token;
    a.epoch = ++model->epoch;
    if (a.epoch == 0) a.epoch = ++model->epoch;  // 0 marks never-written words
    a.route_idx = state->route_idx;
    a.route_w = state->route_w;
    a.exec_idx = state->exec_idx;
    a.exec_w = state->exec_w;
    a.head_logits = state->head_logits;
    a.x_trace = state->x_trace;
    a.h = h;
    a.sink_idx = s.sink_idx;
    a.sink_w = s.sink_w;
    a.flags = s.flags;
    a.xbuf = model->fxbuf;
    a.trace = model->trace;
    launched = true;
    // packed words carry the epoch mod 255: clear them before a tag repeats
    if (a.epoch - model->fx_clean >= 255u) {
      hipError_t e = launch_flow_clear(model->fxbuf, model->fxwords, st);
      if (e != hipSuccess) return hip_fail(e, "layer_step (exchange clear)");
      model->fx_clean = a.epoch - 1;
    }
    hipError_t e = launch_flow(a, st);
    if (e != hipSuccess) return hip_fail(e, "layer_step (streaming kernel)");
    return E0_OK;
  };
  if (model->path == E0_PATH_FLOW) {
    bool launched;
    const int rc = run_flow(launched);
    if (!launched) return fail(E0_ERR_SHAPE, "layer_step: this layer range does not fit the streaming kernel");
    return rc;
  }
  if (model->path != E0_PATH_PHASES && model->dev_table) {
    StackArgs a;
    a.n_heads = 0;
    for (int l = layer_begin; l < layer_end; ++l)
      if (model->layers[l].head.fc1) ++a.n_heads;
    a.dm = dm;
    a.layers = model->dev_table;
    a.L = L;
    a.l0 = layer_begin;
    a.l1 = layer_end;
    a.token = token;
    a.ng = model->ng;
    a.epoch = ++model->epoch;
    if (a.epoch == 0) a.epoch = ++model->epoch;  // 0 marks never-written words
    a.route_idx = state->route_idx;
    a.route_w = state->route_w;
    a.exec_idx = state->exec_idx;
    a.exec_w = state->exec_w;
    a.head_logits = state->head_logits;
    a.x_trace = state->x_trace;
    a.h = h;
    a.xh = model->xh;
    a.xg = model->xg;
    a.xr = model->xr;
    a.xa = model->xa;
    a.xl = model->xl;
    a.sink_idx = s.sink_idx;
    a.sink_w = s.sink_w;
    a.flags = s.flags;
    a.trace = model->trace;
    if (model->path == E0_PATH_CHAIN && chain_launchable(a, model->grid)) {
      // its packed exchange words carry the epoch mod 255: clear them before
      // a tag can recur
      if (a.epoch - model->cx_clean >= 255u) {
        hipError_t e = launch_flow_clear(model->xg, (int64_t)L * model->ng, st);
        if (e != hipSuccess) return hip_fail(e, "layer_step (exchange clear)");
        model->cx_clean = a.epoch - 1;
      }
      hipError_t e = launch_chain(a, model->grid, st);
      if (e != hipSuccess) return hip_fail(e, "layer_step (layer-ahead slot kernel)");
      return E0_OK;
    }
    if (model->path == E0_PATH_CHAIN)
      return fail(E0_ERR_SHAPE, "layer_step: this layer range does not fit the layer-ahead slot kernel");
    if (stack_launchable(a, model->grid)) {
      hipError_t e = launch_stack(a, model->grid, st);
      if (e != hipSuccess) return hip_fail(e, "layer_step (persistent kernel)");
      return E0_OK;
    }
    if (model->path == E0_PATH_PERSISTENT)
      return fail(E0_ERR_SHAPE, "layer_step: this layer range does not fit the persistent kernel");
  }
  if (model->path == E0_PATH_AUTO) {
    bool launched;
    const int rc = run_flow(launched);
    if (launched) return rc;
  }
  for (int l = layer_begin; l < layer_end; ++l) {
    const e0_layer& Ly = model->layers[l];
    Pool pool;
    SharedW sh;
    make_pool(ctx->dm, &Ly.experts, Ly.slot_of, pool);
    make_shared(ctx->dm, Ly.shared.gate.q ? &Ly.shared : nullptr, sh);
    const uint16_t* hin = h + (int64_t)(l - layer_begin) * dm.d;
    uint16_t* hout = h + (int64_t)(l - layer_begin + 1) * dm.d;
    int32_t* eidx = state->exec_idx + ((int64_t)cur * L + l) * K;
    float* ew = state->exec_w + ((int64_t)cur * L + l) * K;
    const int32_t* ridx = state->route_idx + ((int64_t)cur * L + l) * K;
    const float* rw = state->route_w + ((int64_t)cur * L + l) * K;
    hipError_t e;
    const bool routed_here = Ly.router != nullptr;
    uint16_t* xn = state->x_trace ? state->x_trace + (int64_t)l * dm.d : s.xn;
    e = launch_prep(dm, hin, Ly.attn, 1, s.hattn, xn, routed_here ? nullptr : ridx,
                    routed_here ? nullptr : rw, eidx, ew, st);
    if (e != hipSuccess) return hip_fail(e, "layer_step prep");
    if (routed_here) {
      e = launch_gemv16(Ly.router, dm.E, dm.d, dm.d, xn, nullptr, dm.d, 1, nullptr, nullptr,
                        0, 0, 0, 0, nullptr, s.logits, dm.E, st);
      if (e == hipSuccess) e = launch_route(dm, s.logits, Ly.router_bias, 1, eidx, ew, s.flags, st);
      if (e != hipSuccess) return hip_fail(e, "layer_step router");
    }
    if ((e = lora_a_x(ctx->dm, ctx->s, sh, xn, 1, st)) != hipSuccess) return hip_fail(e, "lora A");
    if ((e = launch_gate_up(dm, pool, sh, xn, eidx, 1, s, st)) != hipSuccess)
      return hip_fail(e, "gate/up");
    if ((e = lora_a_down(ctx->dm, ctx->s, sh, 1, st)) != hipSuccess) return hip_fail(e, "lora A down");
    if ((e = launch_down(dm, pool, sh, eidx, ew, 1, s.hattn, hout, s, st)) != hipSuccess)
      return hip_fail(e, "down");
    if (Ly.head.fc1) {
      const int32_t* prev = token > 0 ? state->exec_idx + ((int64_t)nxt * L + l) * K : nullptr;
      float* lg = state->head_logits ? state->head_logits + (int64_t)l * dm.E : nullptr;
      int32_t* pidx;
      float* pw;
      if (l + 1 < L) {
        pidx = state->route_idx + ((int64_t)nxt * L + l + 1) * K;
        pw = state->route_w + ((int64_t)nxt * L + l + 1) * K;
      } else {
        // The last layer's head has no consumer; its routing goes to a sink.
        pidx = s.sink_idx;
        pw = s.sink_w;
      }
      e = head_launch(ctx, &Ly.head, xn, eidx, prev, 1, lg, pidx, pw, st);
      if (e != hipSuccess) return hip_fail(e, "layer_step head");
    }
  }
  return E0_OK;
}

}  // extern "C"

// ------------------------------------------------------------- staging --

struct e0_stager {
  e0_ctx* ctx;
  const char* host_dev;  // device-side address of the pinned host pool
  int32_t L, n_slots;
  char* hbm;
  int32_t* slot_of;
  int32_t* slot_expert;
  int64_t bundle;
  int32_t* copy_list;  // [L][2*8]
  int32_t* n_copies;   // [L]
  unsigned long long* total;  // bundles copied since creation
};

extern "C" {

int64_t e0_bundle_bytes(const e0_spec* spec) {
  if (!spec || spec->group <= 0) return -1;
  const int64_t Id = (int64_t)spec->inter * spec->d_model;
  const int64_t per_group = spec->quant == E0_QUANT_AFFINE ? 2 : 1;  // scale (+ bias)
  return 3 * (Id / 2) + 3 * 2 * per_group * (Id / spec->group);
}

int e0_stager_create(e0_ctx* ctx, const void* host_pool, int32_t n_layers, int32_t n_slots,
                     void* hbm_slots, int32_t* slot_of, int32_t* slot_expert,
                     e0_stager** out) {
  if (!ctx || !host_pool || !hbm_slots || !slot_of || !slot_expert || !out)
    return fail(E0_ERR_ARG, "e0_stager_create: null argument");
  *out = nullptr;
  const Dims& dm = ctx->dm;
  if (n_layers < 1 || n_slots < 2 * dm.K || n_slots > 64)
    return fail(E0_ERR_ARG, "e0_stager_create: need 2K <= n_slots <= 64 and n_layers >= 1");
  if (!aligned(host_pool, 16) || !aligned(hbm_slots, 16))
    return fail(E0_ERR_ALIGN, "e0_stager_create: pools must be 16-byte aligned");
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, host_pool);
  if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return fail(E0_ERR_ARG, "e0_stager_create: host pool is not pinned host memory");
  }
  void* dev = nullptr;
  e = hipHostGetDevicePointer(&dev, const_cast<void*>(host_pool), 0);
  if (e != hipSuccess || !dev) return hip_fail(e, "e0_stager_create: device address of pool");
  e0_stager* s = new e0_stager();
  s->ctx = ctx;
  s->host_dev = (const char*)dev;
  s->L = n_layers;
  s->n_slots = n_slots;
  s->hbm = (char*)hbm_slots;
  s->slot_of = slot_of;
  s->slot_expert = slot_expert;
  s->bundle = e0_bundle_bytes(&ctx->spec);
  e = hipMalloc(&s->copy_list, (size_t)n_layers * 16 * sizeof(int32_t));
  if (e == hipSuccess) e = hipMalloc(&s->n_copies, (size_t)n_layers * sizeof(int32_t));
  if (e == hipSuccess) e = hipMalloc(&s->total, sizeof(unsigned long long));
  if (e == hipSuccess) e = hipMemset(s->total, 0, sizeof(unsigned long long));
  if (e == hipSuccess) e = hipMemset(slot_of, 0xFF, (size_t)n_layers * dm.E * sizeof(int32_t));
  if (e == hipSuccess)
    e = hipMemset(slot_expert, 0xFF, (size_t)n_layers * n_slots * sizeof(int32_t));
  if (e == hipSuccess) e = hipMemset(s->n_copies, 0, (size_t)n_layers * sizeof(int32_t));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    e0_stager_destroy(s);
    return hip_fail(e, "e0_stager_create");
  }
  *out = s;
  return E0_OK;
}

void e0_stager_destroy(e0_stager* st) {
  if (!st) return;
  if (st->copy_list) (void)hipFree(st->copy_list);
  if (st->n_copies) (void)hipFree(st->n_copies);
  if (st->total) (void)hipFree(st->total);
  delete st;
}

int e0_stager_copies(e0_stager* st, int64_t* out) {
  if (!st || !out) return fail(E0_ERR_ARG, "e0_stager_copies: null argument");
  unsigned long long v = 0;
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(&v, st->total, sizeof(v), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "e0_stager_copies");
  *out = (int64_t)v;
  return E0_OK;
}

int stage_experts_n(e0_stager* st, int32_t layer, int32_t n_layers, const int32_t* new_idx,
                    const int32_t* in_use_idx, void* side_stream, void* done_event) {
  if (!st || !new_idx) return fail(E0_ERR_ARG, "stage_experts: null argument");
  if (n_layers < 1 || layer < 0 || layer + n_layers > st->L)
    return fail(E0_ERR_ARG, "stage_experts: layers [%d, %d) outside [0, %d)", layer,
                layer + n_layers, st->L);
  const Dims& dm = st->ctx->dm;
  hipStream_t ss = (hipStream_t)side_stream;
  hipError_t e = launch_stage(
      dm.E, st->n_slots, dm.K, n_layers, st->slot_of + (int64_t)layer * dm.E,
      st->slot_expert + (int64_t)layer * st->n_slots, in_use_idx, new_idx,
      st->copy_list + (int64_t)layer * 16, st->n_copies + layer, st->total,
      st->host_dev + (int64_t)layer * dm.E * st->bundle, (int64_t)dm.E * st->bundle,
      st->hbm + (int64_t)layer * st->n_slots * st->bundle, (int64_t)st->n_slots * st->bundle,
      st->bundle, st->ctx->s.flags, ss);
  if (e != hipSuccess) return hip_fail(e, "stage_experts");
  if (done_event) {
    e = hipEventRecord((hipEvent_t)done_event, ss);
    if (e != hipSuccess) return hip_fail(e, "stage_experts: event");
  }
  return E0_OK;
}

int stage_experts(e0_stager* st, int32_t layer, const int32_t* new_idx,
                  const int32_t* in_use_idx, void* side_stream, void* done_event) {
  return stage_experts_n(st, layer, 1, new_idx, in_use_idx, side_stream, done_event);
}

}  // extern "C"

struct e0_cache {
  e0_ctx* ctx;
  const char* host_dev;  // device-side address of the pinned host pool
  int32_t L, C;
  char* hbm;
  int32_t* slot_of;
  int32_t* owner;
  int32_t* stamp;
  int64_t bundle;
  int32_t* copy_list;  // [L][2*8]
  int32_t* n_copies;   // [L]
  unsigned long long* total;
};

extern "C" {

int e0_cache_create(e0_ctx* ctx, const void* host_pool, int32_t n_layers, int32_t n_entries,
                    void* hbm_cache, int32_t* slot_of, int32_t* owner, int32_t* stamp,
                    e0_cache** out) {
  if (!ctx || !host_pool || !hbm_cache || !slot_of || !owner || !stamp || !out)
    return fail(E0_ERR_ARG, "e0_cache_create: null argument");
  *out = nullptr;
  const Dims& dm = ctx->dm;
  if (n_layers < 1 || n_entries < 1 || n_entries > kMaxCacheEntries)
    return fail(E0_ERR_ARG, "e0_cache_create: need n_layers >= 1 and 1 <= n_entries <= %d",
                kMaxCacheEntries);
  if (!aligned(host_pool, 16) || !aligned(hbm_cache, 16))
    return fail(E0_ERR_ALIGN, "e0_cache_create: pools must be 16-byte aligned");
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, host_pool);
  if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return fail(E0_ERR_ARG, "e0_cache_create: host pool is not pinned host memory");
  }
  void* dev = nullptr;
  e = hipHostGetDevicePointer(&dev, const_cast<void*>(host_pool), 0);
  if (e != hipSuccess || !dev) return hip_fail(e, "e0_cache_create: device address of pool");
  e0_cache* c = new e0_cache();
  c->ctx = ctx;
  c->host_dev = (const char*)dev;
  c->L = n_layers;
  c->C = n_entries;
  c->hbm = (char*)hbm_cache;
  c->slot_of = slot_of;
  c->owner = owner;
  c->stamp = stamp;
  c->bundle = e0_bundle_bytes(&ctx->spec);
  c->copy_list = nullptr;
  c->n_copies = nullptr;
  c->total = nullptr;
  e = hipMalloc(&c->copy_list, (size_t)n_layers * 16 * sizeof(int32_t));
  if (e == hipSuccess) e = hipMalloc(&c->n_copies, (size_t)n_layers * sizeof(int32_t));
  if (e == hipSuccess) e = hipMalloc(&c->total, sizeof(unsigned long long));
  if (e == hipSuccess) e = hipMemset(c->total, 0, sizeof(unsigned long long));
  if (e == hipSuccess) e = hipMemset(slot_of, 0xFF, (size_t)n_layers * dm.E * sizeof(int32_t));
  if (e == hipSuccess) e = hipMemset(owner, 0xFF, (size_t)n_entries * sizeof(int32_t));
  if (e == hipSuccess) e = hipMemset(stamp, 0xFF, (size_t)n_entries * sizeof(int32_t));
  if (e == hipSuccess) e = hipMemset(c->n_copies, 0, (size_t)n_layers * sizeof(int32_t));
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    e0_cache_destroy(c);
    return hip_fail(e, "e0_cache_create");
  }
  *out = c;
  return E0_OK;
}

void e0_cache_destroy(e0_cache* c) {
  if (!c) return;
  (void)hipFree(c->copy_list);
  (void)hipFree(c->n_copies);
  (void)hipFree(c->total);
  delete c;
}

int64_t e0_cache_copies(e0_cache* c) {
  if (!c) return -1;
  unsigned long long v = 0;
  if (hipMemcpy(&v, c->total, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return -1;
  return (int64_t)v;
}

int stage_experts_cached(e0_cache* c, int32_t layer, int32_t n_layers, const int32_t* new_idx,
                         int32_t tick, void* side_stream, void* done_event) {
  if (!c || !new_idx) return fail(E0_ERR_ARG, "stage_experts_cached: null argument");
  if (n_layers < 1 || n_layers > kMaxCacheLayers || layer < 0 || layer + n_layers > c->L)
    return fail(E0_ERR_ARG, "stage_experts_cached: layers [%d, %d) outside [0, %d) or more than %d",
                layer, layer + n_layers, c->L, kMaxCacheLayers);
  if (tick < 0) return fail(E0_ERR_ARG, "stage_experts_cached: negative tick");
  const Dims& dm = c->ctx->dm;
  hipStream_t ss = (hipStream_t)side_stream;
  hipError_t e = launch_cache_stage(
      dm.E, c->C, dm.K, layer, n_layers, tick, c->slot_of, c->owner, c->stamp, new_idx,
      c->copy_list + (int64_t)layer * 16, c->n_copies + layer, c->total,
      c->host_dev + (int64_t)layer * dm.E * c->bundle, (int64_t)dm.E * c->bundle, c->hbm,
      c->bundle, c->ctx->s.flags, ss);
  if (e != hipSuccess) return hip_fail(e, "stage_experts_cached");
  if (done_event) {
    e = hipEventRecord((hipEvent_t)done_event, ss);
    if (e != hipSuccess) return hip_fail(e, "stage_experts_cached: event");
  }
  return E0_OK;
}

int stage_layer(e0_ctx* ctx, const void* host_layer, void* hbm_layer, void* stream,
                void* done_event) {
  if (!ctx || !host_layer || !hbm_layer) return fail(E0_ERR_ARG, "stage_layer: null argument");
  if (!aligned(host_layer, 16) || !aligned(hbm_layer, 16))
    return fail(E0_ERR_ALIGN, "stage_layer: pools must be 16-byte aligned");
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, host_layer);
  if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();
    return fail(E0_ERR_ARG, "stage_layer: host pool is not pinned host memory");
  }
  const size_t bytes = (size_t)ctx->dm.E * (size_t)e0_bundle_bytes(&ctx->spec);
  hipStream_t st = (hipStream_t)stream;
  e = hipMemcpyAsync(hbm_layer, host_layer, bytes, hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "stage_layer: copy");
  if (done_event) {
    e = hipEventRecord((hipEvent_t)done_event, st);
    if (e != hipSuccess) return hip_fail(e, "stage_layer: event");
  }
  return E0_OK;
}

}  // extern "C"

// ---- moe_int4_decode_static: the same step on a workspace the library
// never allocates ------------------------------------------------------------

namespace {

// Workspace of moe_int4_decode_static. Each GPU the library runs on holds its
// own copy until the process ends; in host code `scratch` names a host-side
// stand-in, so only the address from hipGetSymbolAddress reaches kernels.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
char* g_static_ptr[kMaxDevices];

// Device address of the current device's copy (looked up once per device).
int static_scratch(int dev, char** out) {
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "moe_int4_decode_static: hipGetSymbolAddress");
    g_static_ptr[dev] = (char*)ptr;
  }
  *out = g_static_ptr[dev];
  return E0_OK;
}

}  // namespace

extern "C" {

int moe_int4_decode_static(const e0_spec* spec, const e0_experts* routed, const int32_t* slot_of,
                           const e0_shared* shared, const uint16_t* x, const int32_t* idx,
                           const float* w, int32_t n_tokens, uint16_t* y, int32_t* flags,
                           void* stream) {
  if (!spec || !x || !idx || !w || !y)
    return fail(E0_ERR_ARG, "moe_int4_decode_static: null argument");
  if (n_tokens < 0) return fail(E0_ERR_ARG, "moe_int4_decode_static: n_tokens %d < 0", n_tokens);
  if (n_tokens == 0) return E0_OK;
  Dims dm;
  int rc;
  if ((rc = spec_dims(*spec, dm))) return rc;
  const size_t need = scratch_layout(dm, n_tokens, nullptr, nullptr);
  if (need > kStaticScratchBytes)
    return fail(E0_ERR_SHAPE,
                "moe_int4_decode_static: %d tokens of this tier need %zu bytes of workspace; "
                "the static workspace holds %zu",
                n_tokens, need, kStaticScratchBytes);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(E0_ERR_HIP, "moe_int4_decode_static: no device");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(E0_ERR_ARG, "moe_int4_decode_static: device %d beyond %d", dev, kMaxDevices);
  char* base = nullptr;
  if ((rc = static_scratch(dev, &base))) return rc;
  Scratch s;
  scratch_layout(dm, n_tokens, base, &s);
  if (flags) s.flags = flags;
  return moe_run(dm, s, routed, slot_of, shared, x, idx, w, n_tokens, y, (hipStream_t)stream);
}

}  // extern "C"
