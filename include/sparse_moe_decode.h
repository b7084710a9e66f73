/*
 * sparse_moe_decode.h — C ABI of the MI355X (gfx950) streaming-MoE decode step.
 *
 * The library implements one decode layer-step of a mixture-of-experts model
 * whose routing is predicted one token ahead by a small per-layer head, as
 * described on these pages (cited by tag below):
 *   [MW] "The Other Half of the Memory Wall: Serving 35B MoEs from SSD with
 *        Trained Routing Prediction" (arXiv 2609.18063).
 *   [RG] the xyznot.com reading guide of the same paper.
 *   [IE] "Inside Edge0-35B: Running a 35B Sparse MoE in Under 3 GiB RAM via
 *        SSD Offload and Prerouter Speculation".
 *   [CB] "Edge0 streams a 35B MoE off SSD. I counted the bytes it can't stream."
 *
 * Conventions for every call:
 *   - Pointers to tensors are DEVICE pointers owned by the caller, unless a
 *     comment says "host". The library never frees caller memory.
 *   - fp16 tensors are passed as uint16_t bit patterns (IEEE binary16).
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls are
 *     asynchronous on that stream and do not synchronise the host unless the
 *     comment says so.
 *   - Return 0 on success or a negative E0_ERR_* code; e0_last_error() gives a
 *     thread-local message. No C++ exception crosses this boundary.
 *   - Expert ids read from device memory are range-checked inside the
 *     kernels. An out-of-range id contributes nothing and raises a device
 *     error flag that e0_device_status() reports (E0_ERR_RANGE).
 *
 * Int4 matrix layout (e0_q4): a matrix W [rows, cols] is stored as
 *   q: uint32 [rows, cols/8]; element i of row o is in word o*(cols/8) + i/8
 *      at bits 4*(i%8) (low nibble first), a two's-complement value in [-8, 7];
 *   s: fp16   [rows, cols/G]; the weight is s[o][i/G] * q.
 * This is the packed shape the pages give for the stacked expert tensors
 * ([IE "Architectural Deep Dive"]: uint32 [E, out, in/8], eight values per
 * word; [CB "Counting the bytes"]) with symmetric values and no bias; nibble
 * order and signedness are this library's reading (the pages are silent).
 * Alignment: q and s base pointers 16-byte aligned; cols % 32 == 0 and
 * G % 32 == 0; G divides cols.
 */
#ifndef SPARSE_MOE_DECODE_H
#define SPARSE_MOE_DECODE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  E0_OK = 0,
  E0_ERR_ARG = -1,    /* null pointer / bad argument */
  E0_ERR_SHAPE = -2,  /* dimensions the kernels do not support */
  E0_ERR_ALIGN = -3,  /* misaligned pointer */
  E0_ERR_HIP = -4,    /* a HIP runtime call failed */
  E0_ERR_RANGE = -5,  /* an expert id read on the device was out of range */
  E0_ERR_SYNC = -6,   /* a device-side wait hit its spin limit */
  E0_ERR_STATE = -7,  /* object used in a state it does not allow */
  E0_ERR_IO = -8      /* a file could not be opened or read */
};

enum { E0_ROUTER_SOFTMAX_TOPK = 0, E0_ROUTER_SIGMOID_GROUP = 1 };

/* Int4 codec of the expert matrices. Symmetric: a two's-complement nibble q
 * in [-8, 7] times an fp16 group scale, w = s q. Affine (the pages' MLX
 * format [MW §3.1, "int4 affine group-64", every projection with its scales
 * and biases]): an unsigned nibble q in [0, 15], with a bf16 group scale
 * and bias, w = s q + b. Both pack element i of a row in word i/8 at bits
 * 4 (i % 8). */
enum { E0_QUANT_SYMMETRIC = 0, E0_QUANT_AFFINE = 1 };

/* Model dimensions and routing family of one tier ([CB "A3B describes a model
 * that isn't the one serving"], MoESpec; [MW App. A]). */
typedef struct e0_spec {
  int32_t d_model;      /* d: hidden size */
  int32_t n_experts;    /* E: routed experts per layer */
  int32_t top_k;        /* K: experts per token (1..8) */
  int32_t inter;        /* I: routed expert intermediate size */
  int32_t shared_inter; /* Is: shared expert intermediate size (0 = none) */
  int32_t head_hidden;  /* P: prerouter head hidden width */
  int32_t group;        /* G: int4 quantisation group along the input dim */
  int32_t lora_rank;    /* r: LoRA rank on the shared expert (0 = none) */
  float lora_alpha;     /* alpha: LoRA scale is alpha / r */
  int32_t router_kind;  /* E0_ROUTER_SOFTMAX_TOPK or E0_ROUTER_SIGMOID_GROUP */
  int32_t norm_topk;    /* softmax-top-K: renormalise the K selected probs */
  int32_t n_groups;     /* sigmoid-group: n groups of E/n contiguous experts */
  int32_t topk_groups;  /* sigmoid-group: groups kept */
  float route_scale;    /* sigmoid-group: scale s on the weights */
  float rms_eps;        /* RMSNorm epsilon (gain is 1) */
  int32_t quant;        /* E0_QUANT_SYMMETRIC or E0_QUANT_AFFINE */
} e0_spec;

typedef struct e0_q4 {
  const uint32_t* q; /* packed nibbles [rows, cols/8] */
  const uint16_t* s; /* group scales [rows, cols/G]: fp16 (symmetric), bf16 (affine) */
  const uint16_t* b; /* affine: bf16 group biases [rows, cols/G]; symmetric: NULL */
} e0_q4;

/* A pool of `count` routed experts (or staged slots). Entry j's gate/up
 * matrices ([I, d]) start at gate.q + j*stride_q bytes (scales at
 * gate.s + j*stride_s, affine biases at gate.b + j*stride_s), its down
 * matrix ([d, I]) likewise. stride_q / stride_s = 0 selects dense stacking
 * ([count, I, d/8] u32 and [count, I, d/G] 16-bit), i.e. I*d/2 and 2*I*d/G
 * bytes. Entries are
 * addressed by expert id, or through a slot table; ids and slots at or
 * beyond `count` are rejected on the device. */
typedef struct e0_experts {
  e0_q4 gate, up, down;
  int64_t stride_q; /* bytes between consecutive entries' packed words */
  int64_t stride_s; /* bytes between consecutive entries' scales */
  int32_t count;    /* entries in the pool */
} e0_experts;

/* Unmerged LoRA pair of one projection [MW §3.3]: A fp16 [r, in], B fp16
 * [out, r]; the projection becomes W x + (alpha/r) B (A x). NULL = none. */
typedef struct e0_lora {
  const uint16_t* a;
  const uint16_t* b;
} e0_lora;

/* Shared expert (gate/up [Is, d], down [d, Is]) with LoRA on each projection. */
typedef struct e0_shared {
  e0_q4 gate, up, down;
  e0_lora lgate, lup, ldown;
} e0_shared;

/* Prerouter head [MW §3.2 Head; CB "The mechanism"]: fc1 fp16 [P, d+2E],
 * fc2 fp16 [E, P], lin fp16 [E, d+2E] (nn.Linear weights, no bias).
 * bias: fp32 [E] selection bias of the predicted layer's sigmoid-group
 * routing (NULL = zero; unused for softmax-top-K). */
typedef struct e0_head {
  const uint16_t* fc1;
  const uint16_t* fc2;
  const uint16_t* lin;
  const float* bias;
} e0_head;

typedef struct e0_ctx e0_ctx;

/* Create a context for one tier. Allocates the device scratch the entry
 * points share, sized for up to `max_tokens` tokens per call (1..8192; a
 * prefill batch of B tokens holds about B*(K+1)*(4d + 4I) bytes of it), on
 * the current HIP device. Calls on one context must not overlap in time. */
int e0_create(const e0_spec* spec, int32_t max_tokens, e0_ctx** out);
void e0_destroy(e0_ctx* ctx);

/* Thread-local text of the last error (never NULL). */
const char* e0_last_error(void);

/* Synchronise `stream`, then return and clear the device-side error flags
 * (E0_ERR_RANGE for a bad expert id, E0_ERR_SYNC for a spin-limit exit). */
int e0_device_status(e0_ctx* ctx, void* stream);

/* ---------------------------------------------------------------------------
 * moe_int4_decode — routed experts plus shared expert for B tokens.
 * [MW §3.1 Math contract]: each routed expert is down(silu(gate x) * up x);
 * [CB "The mechanism", MoESpec shared_experts=1; MW Fig. 1 sum node]: the
 * output is sum_k w[b][k] E_{idx[b][k]}(x_b) + S(x_b), S the shared expert
 * with its unmerged LoRA deltas (omitted when shared == NULL).
 *   routed   host struct of device pointers; expert idx is read from
 *            routed->... at slot slot_of[idx] when slot_of != NULL (the
 *            staged slot table [MW §3.1 "staged"]), else at idx.
 *   slot_of  device int32 [E] or NULL.
 *   x        fp16 [B, d] activations (already RMS-normed).
 *   idx, w   int32 / fp32 [B, K] routing (ids in [0, E)).
 *   y        fp16 [B, d] output (round-to-nearest-even of the fp32 sum).
 * B <= max_tokens. Internal sums are fp32; q*s is never rounded to fp16 and
 * the SwiGLU intermediate keeps fp32 precision. B < 16 runs one GEMV per
 * (token, expert); B >= 16 groups the B*K entries by expert in one launch
 * and runs int4 x fp16 MFMA tiles of up to 32 of an expert's tokens (64 from
 * 16 entries per expert on average, B*K >= 16 E), fp32 group scales applied
 * to fp32 partials, each expert's weights read once per tile [MW §3.1
 * Executor paths: batched chunks and prefill take the whole-layer path].
 * Either codec runs on both paths; the affine biases enter as b times the
 * fp32 sum of the group's inputs. Both paths are deterministic. */
int moe_int4_decode(e0_ctx* ctx, const e0_experts* routed, const int32_t* slot_of,
                    const e0_shared* shared, const uint16_t* x, const int32_t* idx,
                    const float* w, int32_t n_tokens, uint16_t* y, void* stream);

/* ---------------------------------------------------------------------------
 * moe_int4_decode_static — moe_int4_decode for callers that cannot allocate
 * device memory at call time (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). Same arguments and result as
 * moe_int4_decode, with the tier given by its spec instead of a context, and
 * no allocation, free or allocating library call of any kind: the kernels'
 * workspace is a library-owned static device array of 16 MiB per GPU, held
 * until the process ends, whose address is looked up (not allocated) on the
 * first call on each device.
 *   spec     the tier (validated as in e0_create).
 *   flags    device int32 [4] or NULL: the kernels OR error bits into
 *            flags[0] (an expert id out of range, as e0_device_status
 *            reports them for moe_int4_decode); the library never clears it.
 * E0_ERR_SHAPE when n_tokens tokens of this tier need more than the 16 MiB
 * (35B shapes with K = 4: up to about 240 tokens; K = 8: about 150).
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (two streams, two host threads) race and must be serialised by the
 * caller. Each call rewrites all of the workspace it reads. */
int moe_int4_decode_static(const e0_spec* spec, const e0_experts* routed, const int32_t* slot_of,
                           const e0_shared* shared, const uint16_t* x, const int32_t* idx,
                           const float* w, int32_t n_tokens, uint16_t* y, int32_t* flags,
                           void* stream);

/* ---------------------------------------------------------------------------
 * lora_delta — y_acc[b] += scale * B (A x[b]) for B tokens [MW §3.3; RG
 * "Unmerged Adapter Execution"]. A fp16 [rank, in], Bm fp16 [out, rank],
 * x fp16 [B, in], y_acc fp32 [B, out] (read-modify-write). rank <= 64. */
int lora_delta(e0_ctx* ctx, const uint16_t* A, const uint16_t* Bm, int32_t in_dim,
               int32_t out_dim, int32_t rank, float scale, const uint16_t* x, float* y_acc,
               int32_t n_tokens, void* stream);

/* ---------------------------------------------------------------------------
 * prerouter_forward — the head owned by layer N on B tokens [MW §3.2 Head,
 * Prediction-as-routing; CB "The mechanism"]:
 *   f = [x ; onehot(cur) ; onehot(prev)]  (length d + 2E),
 *   logits = lin f + fc2 erf_gelu(fc1 f),
 * then the tier's routing function [MW App. A] on the fp32 logits gives layer
 * N+1's routing for the next token.
 *   x        fp16 [B, d] post-attention-norm activations of layer N.
 *   cur_idx  int32 [B, K] the set layer N executed (K distinct ids).
 *   prev_idx int32 [B, K] the set at the previous token, or NULL for the
 *            all-zero one-hot (first token).
 *   logits   fp32 [B, E] or NULL.
 *   out_idx  int32 [B, K] selected ids, descending score, ties to lower id.
 *   out_w    fp32 [B, K] routing weights. */
int prerouter_forward(e0_ctx* ctx, const e0_head* head, const uint16_t* x,
                      const int32_t* cur_idx, const int32_t* prev_idx, int32_t n_tokens,
                      float* logits, int32_t* out_idx, float* out_w, void* stream);

/* ---------------------------------------------------------------------------
 * Stack description for layer_step. One e0_layer per layer (host struct of
 * device pointers; copied into a device table by e0_model_create).
 *   experts    routed pool indexed by id, or by slot through slot_of.
 *   slot_of    device int32 [E] id -> slot table, or NULL.
 *   router     fp16 [E, d] own router (layers not routed by a prediction),
 *              NULL on layers that consume a prediction.
 *   router_bias fp32 [E] sigmoid-group selection bias, or NULL.
 *   head       prerouter head owned by this layer (fc1 == NULL: none). Its
 *              prediction routes layer+1 at the next token.
 *   attn       fp16 [d] fixed residual update standing in for attention. */
typedef struct e0_layer {
  e0_experts experts;
  const int32_t* slot_of;
  e0_shared shared;
  const uint16_t* router;
  const float* router_bias;
  e0_head head;
  const uint16_t* attn;
} e0_layer;

typedef struct e0_model e0_model;

int e0_model_create(e0_ctx* ctx, const e0_layer* layers, int32_t n_layers, e0_model** out);
void e0_model_destroy(e0_model* model);

/* How layer_step executes. E0_PATH_AUTO (default) takes the first of these
 * that the shapes and the layer range allow: the persistent whole-token
 * kernel (E0_PATH_PERSISTENT: d a multiple of 512 up to 2048, I = 512; both
 * int4 codecs), the wave-specialised streaming kernel (E0_PATH_FLOW:
 * symmetric int4, d 1536 or 2048, I = 512, group 64, K <= 8, E <= 256, rank 0
 * or 16, at most 64 layers per launch), one kernel per phase
 * (E0_PATH_PHASES, any shape). E0_PATH_CHAIN, taken only when asked for, is
 * a persistent kernel that loads the next layer's weights while the current
 * layer's exchanges run (symmetric int4, d 1536 or 2048, I = 512, group 64,
 * K <= 8, E <= 512 and even, rank 0 or 16, at most 64 layers per launch, and
 * per-workgroup shares that fit its plans); its exchange words carry the
 * SwiGLU outputs rounded to 28 bits. Forcing CHAIN, FLOW or PERSISTENT fails
 * with E0_ERR_SHAPE when the shapes or the range do not fit it. All compute
 * the same step. */
enum { E0_PATH_AUTO = 0, E0_PATH_PHASES = 1, E0_PATH_PERSISTENT = 2, E0_PATH_FLOW = 3,
       E0_PATH_CHAIN = 4 };
int e0_model_set_path(e0_model* model, int32_t path);

/* Workgroups of the persistent kernels: one per compute unit by default (grid
 * 0 restores that). A smaller grid leaves compute units free, so kernels on
 * other streams (the staging copies of stage_experts) run concurrently with
 * layer_step instead of between its launches; the work is spread over the
 * grid either way. E0_ERR_ARG when grid exceeds the compute units (every
 * workgroup must be resident at once), E0_ERR_SHAPE when the model's shapes do
 * not fit a persistent kernel. The trace shape follows the grid; a trace
 * buffer set for a smaller grid is dropped. */
int e0_model_set_grid(e0_model* model, int32_t grid);

/* Split of the FLOW kernel's grid: n_gate_up workgroups own the SwiGLU items
 * and the head's fc1 / linear rows, n_down the output rows and the head's fc2
 * rows; n_gate_up + n_down must equal the grid. 0, 0 (default) picks the
 * split from the shapes. E0_ERR_SHAPE when the split does not fit the
 * kernel's per-workgroup limits. */
int e0_model_set_roles(e0_model* model, int32_t n_gate_up, int32_t n_down);

/* Phase tracing of the persistent kernels (observability; off by default).
 * trace: device uint64 [grid][rows][points] (shape from e0_model_trace_shape;
 * rows = L + 1), or NULL to turn tracing off. It serves launches on at most
 * the grid it was set for. Thread 0 of each workgroup writes the 100 MHz wall
 * clock at phase boundaries of row l < L (a layer):
 *   PERSISTENT: 0 layer start, 9 activation-independent loads issued, 1 h
 *     gathered, 2 x normed, 3 routed, 4 gate/up published, 5 down and LoRA
 *     loads issued, 6 SwiGLU outputs gathered, 7 shared expert and hi/lo
 *     copies done, 8 h_out published; a layer with its own router also 10
 *     logits reduced, 11 logits published, 13 logits gathered, 14 routed. Row
 *     L (the heads, after the last layer): 0 start, 1 fc1/linear rows
 *     published, 2 activations gathered, 3 fc2 rows published, 4 head routing.
 *   FLOW, gate/up workgroups: 0 layer start, 1 h gathered, 2 x normed, 3
 *     routed, 4 SwiGLU items published, 5 head rows published. Down
 *     workgroups: 0 layer start, 1 SwiGLU outputs gathered, 2 hi/lo copies, 3
 *     h_out published, 4 previous head's fc2 published, 5 ranking of the head
 *     before done; row L point 0: end of the launch. */
int e0_model_set_trace(e0_model* model, uint64_t* trace);
int32_t e0_model_trace_shape(e0_model* model, int32_t* grid, int32_t* rows, int32_t* points);

/* Device-resident decode state, caller-owned, L = number of model layers:
 *   route_idx / route_w  int32 / fp32 [2][L][K]: routing consumed at token t
 *        is read from buffer t&1; a head owned by layer l at token t writes
 *        layer l+1's prediction into buffer (t+1)&1. The caller fills buffer
 *        0 for the first token.
 *   exec_idx / exec_w    int32 / fp32 [2][L][K]: the set each layer executed
 *        at token t (buffer t&1); buffer (t+1)&1 holds token t-1's set, the
 *        head's "previous token" input.
 *   head_logits          fp32 [L][E] or NULL: logits of each layer's head.
 *   x_trace              fp16 [L][d] or NULL: each layer's normed activation
 *        x (the input of its experts and head) at the last token.
 *   n_layers             L, the layer count the buffers were sized for; it
 *        must equal the model's (E0_ERR_ARG otherwise). */
typedef struct e0_state {
  int32_t* route_idx;
  float* route_w;
  int32_t* exec_idx;
  float* exec_w;
  float* head_logits;
  uint16_t* x_trace;
  int32_t n_layers;
} e0_state;

/* ---------------------------------------------------------------------------
 * layer_step — one decode token through layers [layer_begin, layer_end)
 * [MW §3.2 Motivation, Head, Prediction-as-routing, Feature drift]. Per layer l:
 *   h_a = h + attn[l];  x = fp16(RMSNorm(h_a));
 *   routing = own router on x (router != NULL) or the prediction in
 *             route_*[t&1][l];
 *   y = moe_int4_decode(x, routing);  h' = fp16(h_a + y);
 *   if l owns a head: prerouter_forward(x, exec set, previous set) ->
 *             route_*[(t+1)&1][l+1] (when l+1 < L).
 * h: fp16 [layer_end - layer_begin + 1, d]; h[0] is the input, h[i+1] the
 * output of layer layer_begin + i (every layer's residual is kept).
 * token: t >= 0 (t == 0 means no previous set). */
int layer_step(e0_ctx* ctx, e0_model* model, int32_t layer_begin, int32_t layer_end,
               const e0_state* state, int32_t token, uint16_t* h, void* stream);

/* ---------------------------------------------------------------------------
 * Expert staging [MW §3.1 Executor paths "staged"; §3.2 (staged set equals the
 * routed set); IE "Fixed-Slot Decoding"]: a pinned host pool of expert
 * bundles is copied into an HBM slot pool, keyed by the predicted set, on a
 * side stream.
 * Bundle layout of one expert (bytes, in order): gate q [I, d/8] u32,
 * up q, down q [d, I/8] u32, gate s [I, d/G] 16-bit, up s, down s, and for
 * the affine codec gate b, up b, down b (bf16, shaped as the scales);
 * bundle size e0_bundle_bytes(spec) (35B shapes: 1,671,168 bytes symmetric,
 * 1,769,472 affine, the pages' "1.77 MB" per expert). An e0_experts view of a pool of bundles has
 * stride_q = stride_s = bundle bytes.
 *   host_pool  HOST pointer, pinned (hipHostMalloc), [n_layers][E] bundles.
 *   hbm_slots  device pointer, [n_layers][n_slots] bundles.
 *   slot_of    device int32 [n_layers][E], slot_expert [n_layers][n_slots];
 *              the stager initialises both to -1 (empty).
 * Slot policy (the pages give none; this is the library's reading): ids of
 * the new set that already hold a slot keep it; misses, in ascending id, take
 * the lowest slots not holding an id of the set in use or of the new set.
 * n_slots >= 2K guarantees a free slot. */
typedef struct e0_stager e0_stager;

int64_t e0_bundle_bytes(const e0_spec* spec);

int e0_stager_create(e0_ctx* ctx, const void* host_pool, int32_t n_layers, int32_t n_slots,
                     void* hbm_slots, int32_t* slot_of, int32_t* slot_expert,
                     e0_stager** out);
void e0_stager_destroy(e0_stager* st);

/* stage_experts — make layer `layer`'s slots hold the K ids in new_idx
 * (device int32 [K]) while the K ids in in_use_idx (device, or NULL for none)
 * stay resident. Runs the slot policy on the device and copies each missing
 * bundle from the host pool over PCIe into its slot, all on `side_stream`,
 * then records `done_event` (a hipEvent_t, may be NULL) on that stream.
 * Expert ids never travel to the host. The copy kernel runs 16 workgroups,
 * so it occupies at most 16 compute units; a persistent layer_step kernel
 * sized to leave that many free (e0_model_set_grid) runs beside it. */
int stage_experts(e0_stager* st, int32_t layer, const int32_t* new_idx,
                  const int32_t* in_use_idx, void* side_stream, void* done_event);

/* stage_experts for the n_layers consecutive layers layer .. layer+n_layers-1
 * in one pass (one policy launch, one copy launch): new_idx and in_use_idx
 * (or NULL) are device int32 [n_layers][K], row i for layer layer+i. */
int stage_experts_n(e0_stager* st, int32_t layer, int32_t n_layers, const int32_t* new_idx,
                    const int32_t* in_use_idx, void* side_stream, void* done_event);

/* ---------------------------------------------------------------------------
 * stage_layer — whole-layer staging for prefill-sized batches [MW §3.1
 * Executor paths, "whole-layer": a prefill loads every expert of a layer at
 * once, and the load of the next layer overlaps the current layer's GPU
 * work]. Copies one layer's E expert bundles as a single DMA transfer on
 * `stream`, then records done_event (a hipEvent_t, may be NULL) there.
 *   host_layer  HOST pointer, pinned (hipHostMalloc), E bundles in the bundle
 *               layout above (E * e0_bundle_bytes bytes, contiguous, expert e
 *               at e * bundle).
 *   hbm_layer   device pointer, the same size. An e0_experts view of it with
 *               stride_q = stride_s = bundle bytes (no slot table) feeds
 *               moe_int4_decode.
 * The caller owns both buffers and orders the copy against the kernels that
 * read hbm_layer (events). Errors: E0_ERR_ARG for a null pointer or a host
 * pointer that is not pinned, E0_ERR_ALIGN unless both are 16-byte aligned,
 * E0_ERR_HIP if the copy cannot be queued. */
int stage_layer(e0_ctx* ctx, const void* host_layer, void* hbm_layer, void* stream,
                void* done_event);

/* ---------------------------------------------------------------------------
 * Cross-layer hot-expert cache [MW §3.1 Executor paths, "hot": LRU-resident
 * hot experts; MW Table 1: a shared LRU of expert bundles across layers
 * (64 -> 1024 bundles); IE "The Streaming Subsystem": a hit skips the read
 * from the slower tier]. One HBM pool of n_entries bundles serves every
 * layer of a pinned host pool: a layer's slot table maps its ids to cache
 * entries, so a hit costs no copy and an id evicted from one layer's set can
 * be refilled for another layer.
 *   host_pool  HOST pointer, pinned (hipHostMalloc), [n_layers][E] bundles.
 *   hbm_cache  device pointer, [n_entries] bundles; an e0_experts view of it
 *              (stride_q = stride_s = bundle bytes, count = n_entries) with
 *              slot_of = slot_of[l] is layer l's routed pool.
 *   slot_of    device int32 [n_layers][E]: cache entry of (layer, id), -1;
 *   owner      device int32 [n_entries]: layer * E + id held, -1 (empty);
 *   stamp      device int32 [n_entries]: tick of the last staging, -1.
 *              The cache initialises all three to -1 and owns their
 *              contents afterwards; the caller owns the memory.
 * Replacement (the pages say LRU and give no detail; this is the library's
 * reading): staging the sets of token T (tick T), ids already cached are
 * hits and their entries get stamp T; the misses, in ascending (layer, id),
 * take the entries that are empty or were last staged before T - 1 (the
 * running token T - 1 and the sets already staged for T keep theirs), least
 * recently staged first, ties to the lower entry index. n_entries >= 2 K
 * n_layers guarantees a free entry. n_entries <= 4096. */
typedef struct e0_cache e0_cache;

int e0_cache_create(e0_ctx* ctx, const void* host_pool, int32_t n_layers, int32_t n_entries,
                    void* hbm_cache, int32_t* slot_of, int32_t* owner, int32_t* stamp,
                    e0_cache** out);
void e0_cache_destroy(e0_cache* c);

/* stage_experts_cached — stage the sets new_idx (device int32 [n_layers][K],
 * row i for layer layer+i, n_layers <= 64) at tick `tick` (the index of the
 * token that will use them, >= 0): runs the replacement on the device, then
 * copies each missing bundle from the host pool over PCIe into its entry,
 * all on side_stream, then records done_event (may be NULL). Ids out of
 * range: nothing is staged and device_status reports E0_ERR_RANGE; too few
 * free entries: only the hit stamps change, also reported as E0_ERR_RANGE.
 * The copy kernel occupies at most 16 compute units, as stage_experts. */
int stage_experts_cached(e0_cache* c, int32_t layer, int32_t n_layers, const int32_t* new_idx,
                         int32_t tick, void* side_stream, void* done_event);

/* Bundles copied from the host pool since the cache was created (a
 * synchronous device read; -1 on error). */
int64_t e0_cache_copies(e0_cache* c);

/* ---------------------------------------------------------------------------
 * Storage tier under the pinned pool [MW §3.1: expert weights stay on SSD
 * as per-layer stacked files and stream on demand by byte range; §5.3:
 * reads issued one token ahead move the load time off the critical path].
 * Layer l's file (paths[l]) holds its E bundles back to back, bundle e at
 * byte e * bundle_bytes (the bundle layout above). io_threads host threads
 * serve the reads; direct != 0 opens the files with O_DIRECT (page cache
 * bypassed; bundle_bytes a multiple of 4096), so every
 * read reaches the device (each I/O thread reads into its own page-aligned
 * buffer and copies the bundle to its destination, since the driver's
 * pinned pages cannot take a direct read). Host code only: no GPU call.
 *   e0_store_read   queue one pread per id of `ids` (host int32 [n]) into
 *                   dst[i] (host pointers, typically into a pinned pool);
 *                   returns at once with a ticket.
 *   e0_store_wait   block until the ticket's reads are done; blocked_s (may
 *                   be NULL) gets the time this call waited, read_s the time
 *                   from queueing to the last read's completion. E0_ERR_IO if
 *                   any read failed; a ticket is waited on once.
 *   e0_store_bytes  bytes read since opening.
 * Errors: E0_ERR_ARG (bad argument), E0_ERR_ALIGN (O_DIRECT bundle size),
 * E0_ERR_RANGE (id outside [0, E)), E0_ERR_IO (open or read failed). */
typedef struct e0_store e0_store;

int e0_store_open(const char* const* paths, int32_t n_layers, int32_t n_experts,
                  int64_t bundle_bytes, int32_t io_threads, int32_t direct, e0_store** out);
void e0_store_close(e0_store* s);
int e0_store_read(e0_store* s, int32_t layer, const int32_t* ids, int32_t n, void* const* dst,
                  int64_t* ticket);
int e0_store_wait(e0_store* s, int64_t ticket, double* blocked_s, double* read_s);
int64_t e0_store_bytes(e0_store* s);

/* Bundles copied by this stager's stage_experts calls since it was created
 * (observability: host-link bytes = count x e0_bundle_bytes). Synchronises
 * the device; E0_ERR_HIP if a copy fails. */
int e0_stager_copies(e0_stager* st, int64_t* out);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_MOE_DECODE_H */
