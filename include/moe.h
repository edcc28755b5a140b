/*
 * moe.h -- C ABI of libmoe.so: the routed-expert MoE layer forward on one
 * AMD Instinct MI355X (gfx950).
 *
 * The layer, as the pages describe it: a router scores every expert for every
 * token and keeps a few ("Mixture of experts VRAM: total vs active parameters",
 * section "How current MoE models route each token"); tokens that chose the
 * same expert are grouped so one read of the expert's weights serves all of
 * them ("Understanding MoE Inference Costs on Galactus", section "Prompt
 * processing is a different phase"); each expert is a gate/up/down FFN with a
 * SiLU gate (pith.science verdict on FloE, arXiv 2505.05950,
 * referee_report.summary); 4-bit experts are held in memory and computed at
 * higher precision (Mixture of experts VRAM..., same section, last paragraph);
 * results are collected back per token (same page, "Expert parallelism on RTX
 * PRO 6000 and H200 NVL"); expert weights that do not fit device memory are
 * paged in from host memory on demand through stable logical slots ("What
 * expert offloading actually costs", section "Inside expert paging").
 *
 * Conventions for every call:
 *  - Buffers are caller-owned.  "device" pointers are HIP device memory,
 *    "host" pointers ordinary host memory.  Nothing here keeps a pointer after
 *    the call returns, except moe_cache_* (see there).
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Device
 *    calls only enqueue work on it and return; results are ready when the
 *    stream reaches them.  No call synchronises the device.
 *  - Return value: MOE_OK (0) or a negative moe_status; on error nothing was
 *    enqueued and moe_last_error() holds a message (thread-local).
 *  - Row-major everywhere; "[A][B]" means A rows of B contiguous elements.
 *  - Sizes: T >= 0 tokens, H hidden, E experts (1..1024), k top-k (1..min(E,16)),
 *    I expert intermediate size.  H and I must be multiples of 32.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID = -1,     /* bad argument: null pointer, size out of range, k > E ... */
  MOE_ERR_UNSUPPORTED = -2, /* valid but not supported: H or I not a multiple of 32, dtype mix ... */
  MOE_ERR_HIP = -3,         /* a HIP runtime call failed (message from hipGetErrorString) */
  MOE_ERR_CAPACITY = -4,    /* expert cache: one lookup group needs more slots than exist */
  MOE_ERR_NOT_PINNED = -5,  /* expert cache: host bank is not page-locked HIP host memory */
  MOE_ERR_WORKSPACE = -6    /* workspace pointer null or smaller than the size query returned */
} moe_status;

/* activation / output element types */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/*
 * Expert weight formats (the "logical" form handed to moe_pack_expert):
 *  MOE_W_F32, MOE_W_BF16: plain [rows][K] matrices.
 *  MOE_W_MXFP4: OCP Microscaling MXFP4 -- E2M1 elements, two per byte, element 2i in the
 *    low nibble; one E8M0 scale byte per 32 consecutive elements along K ([rows][K/32]).
 *  MOE_W_INT4G32: symmetric INT4, two's-complement nibbles, element 2i in the low nibble;
 *    one bf16 scale per 32 consecutive elements along K ([rows][K/32], uint16 bit patterns).
 * For every format K is the contraction dimension: H for gate/up, I for down.
 */
typedef enum { MOE_W_F32 = 0, MOE_W_BF16 = 1, MOE_W_MXFP4 = 2, MOE_W_INT4G32 = 3 } moe_wfmt;

typedef enum { MOE_FFN_AUTO = 0, MOE_FFN_DECODE = 1, MOE_FFN_PREFILL = 2 } moe_ffn_mode;

/* Message of the last failing call on this thread ("" if none). Never NULL. */
const char* moe_last_error(void);

/* ------------------------------------------------------------------ router */

/*
 * Router: logits[t][e] = sum_h x[t][h] * w_router[e][h] + bias[e] (fp32 accumulation),
 * then for each token the k largest logits in descending order (equal logits:
 * lower expert id first) and their gate weights
 *     topk_w[t][j] = exp(l_j - l_0) / sum_{i<k} exp(l_i - l_0),
 * i.e. the softmax over all E logits renormalised over the chosen k.
 *   x         device [T][H], element type xdt
 *   w_router  device [E][H], element type xdt
 *   bias      device [E] fp32, or NULL for none
 *   topk_ids  device [T][k] int32 (out);  topk_w device [T][k] fp32 (out)
 *   logits    device [T][E] fp32 (out), or NULL
 *   ws        device workspace of ws_bytes >= moe_route_workspace(T, H, E, xdt) bytes (may be NULL if 0)
 * Errors: MOE_ERR_INVALID for null x/w_router/topk_ids/topk_w (when T > 0), E out of
 * 1..1024, k out of 1..min(E,16), H <= 0; MOE_ERR_WORKSPACE if the workspace is too small.
 */
int moe_route(const void* x, int xdt, int T, int H, const void* w_router, const float* bias, int E, int k,
              int32_t* topk_ids, float* topk_w, float* logits, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes moe_route needs (device, 256-byte aligned; 0 when none).  bf16 batches with
 * T*E <= 2^20 spread the router over many workgroups and keep partial logits there; larger bf16
 * batches with E a multiple of 16 keep the router matrix repacked into MFMA fragments
 * (E*H*2 bytes), the [T][E] fp32 logits and the row-tile plan of the MFMA kernel there. */
size_t moe_route_workspace(int T, int H, int E, int xdt);

/* ------------------------------------------------------------- permutation */

/*
 * Workspace bytes moe_permute needs: 0 when T*k <= 8192 (one workgroup does the grouping),
 * else 8 * ceil(T*k / 2048) * E (per-block expert counts and starting cursors of the
 * block-parallel path); device memory, 4-byte aligned, owned by the caller.
 */
size_t moe_permute_workspace(int T, int k, int E);

/*
 * Group the T*k (token, slot) pairs by expert, stably:
 *   counts[e]   number of pairs routed to e                      device [E] int32 (out)
 *   offsets[e]  exclusive prefix sum of counts, offsets[E] = T*k device [E+1] int32 (out)
 *   perm_src[p] flat index t*k+j of the p-th pair in expert-major order, ascending
 *               flat index inside an expert                       device [T*k] int32 (out)
 *   inv_perm[i] position p of flat index i (perm_src[inv_perm[i]] == i) device [T*k] int32 (out)
 *   topk_ids    device [T][k] int32, every id in [0, E)
 * Errors: MOE_ERR_INVALID for null pointers (T > 0), E out of 1..1024, k < 1,
 * T*k > 1<<24; MOE_ERR_WORKSPACE if ws_bytes < moe_permute_workspace(T, k, E).
 * Ids outside [0, E) are a caller error with undefined (but memory-safe) results.
 */
int moe_permute(const int32_t* topk_ids, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------- expert weight packages */

/*
 * One expert's gate, up and down matrices (plus block scales for the 4-bit formats) live
 * in one contiguous device "package" in the layout the kernels stream.  Its size counts
 * every byte the expert's weights occupy, scales included ("Understanding MoE Inference
 * Costs on Galactus", section "What a smaller quantization can change"):
 *   f32 12HI, bf16 6HI, MXFP4 3HI/2 + 3HI/32, INT4-g32 3HI/2 + 3HI/16.
 * Returns 0 for an unsupported (H, I, fmt).
 */
size_t moe_package_bytes(int H, int I, int fmt);

/*
 * Host, offline: repack one expert from the logical layout into a package.
 *   gate, up  host [I][H] (f32 / bf16 elements, or [I][H/2] nibble bytes for 4-bit)
 *   down      host [H][I] (or [H][I/2] nibble bytes)
 *   *_scales  host [rows][K/32] (E8M0 bytes for MXFP4, bf16 bits for INT4); NULL for f32/bf16
 *   package   host, package_bytes >= moe_package_bytes(H, I, fmt) (out)
 * Errors: MOE_ERR_INVALID (null pointers, small package); MOE_ERR_UNSUPPORTED if H or I is not a
 * multiple of 32, or (INT4) a scale is not exactly representable in binary16, the precision the
 * kernels compute INT4 experts in.
 */
int moe_pack_expert(int H, int I, int fmt, const void* gate, const void* gate_scales, const void* up,
                    const void* up_scales, const void* down, const void* down_scales, void* package,
                    size_t package_bytes);

/*
 * Test hook: decode a package on the device back to the logical layout in fp32:
 * out = [gate I*H][up I*H][down H*I] (device, 3*H*I floats).  Every value is exact.
 */
int moe_dequant_expert(const void* package, int H, int I, int fmt, float* out, void* stream);

/* --------------------------------------------------------------- expert FFN */

typedef struct {
  int H, I, E;
  int fmt;                       /* moe_wfmt of every package */
  const void* packages;          /* device: package of logical expert e at packages + slot(e) * pkg_stride */
  size_t pkg_stride;             /* bytes between packages, >= moe_package_bytes, multiple of 256 */
  const int32_t* slot_of_expert; /* device [E] stable logical -> physical slot, or NULL for slot(e) = e */
  int n_slots;                   /* packages available at `packages` when slot_of_expert is set (>= 1);
                                    an expert whose slot is outside [0, n_slots) is skipped (its rows of
                                    y_perm are not written); ignored when slot_of_expert is NULL */
} moe_experts;

/* Workspace bytes moe_expert_ffn needs for these experts, T tokens and top-k: the activations
 * cast to the MFMA operand type when they differ from it, h [T*k][I], and the row-tile plans
 * (with the work counters of the persistent prefill kernels).  A workspace serves one call at a
 * time: calls in flight together (on different streams) need workspaces of their own. */
size_t moe_ffn_workspace(const moe_experts* w, int T, int k, int mode);

/*
 * Grouped SwiGLU expert FFN over the permuted pairs:
 *   for every expert e and p in [offsets[e], offsets[e+1]):
 *     r = x[perm_src[p] / k]
 *     y_perm[p] = W_down_e (SiLU(W_gate_e r) * (W_up_e r)),  SiLU(z) = z / (1 + e^-z)
 *   x        device [T][H], element type xdt
 *   offsets  device [E+1], perm_src device [T*k] (from moe_permute)
 *   y_perm   device [T*k][H] fp32 (out)
 * Precision: MFMA products of exactly decoded weights (bf16 / MXFP4 -> bf16 operands,
 * INT4 -> fp16 operands with fp16 activations) accumulated in fp32; the intermediate
 * SiLU(g)*u is rounded once to the operand type; f32 experts run in fp32 throughout.
 * A shared (always-on) expert is the same call with E = 1, offsets = {0, T}, k = 1 and
 * perm_src = {0, 1, ..., T-1}.
 * Errors: MOE_ERR_INVALID (null pointers, sizes), MOE_ERR_UNSUPPORTED (H, I not multiples
 * of 32), MOE_ERR_WORKSPACE (ws smaller than moe_ffn_workspace).
 */
int moe_expert_ffn(const moe_experts* w, const void* x, int xdt, int T, int k, const int32_t* offsets,
                   const int32_t* perm_src, float* y_perm, int mode, void* ws, size_t ws_bytes, void* stream);

/*
 * Profiling hook.  While set (on the calling thread), every moe_expert_ffn call records, on its
 * stream, events[0] right before the gate/up GEMM kernel(s) (after any activation cast and
 * row-tile planning), events[1] after the gate/up kernel(s) (before the down kernel(s)) and
 * events[2] after the down kernel(s).  `events` points to 3 hipEvent_t passed as void*; the
 * array is read at each call, so it must stay valid while set.  NULL turns it off.
 */
int moe_ffn_trace_events(void* const* events);

/* ------------------------------------------------------------------ combine */

/*
 * Weighted combine back to token order:
 *   out[t] = sum_{j<k} topk_w[t][j] * y_perm[inv_perm[t*k+j]]  (+ shared_y[t])
 * fp32 sum in slot order j = 0..k-1, then the shared expert's output with weight 1,
 * then one rounding (nearest-even) to odt.  Deterministic: no atomics.
 *   y_perm device [T*k][H] fp32; topk_w device [T][k] fp32; inv_perm device [T*k] int32
 *   shared_y device [T][H] fp32 or NULL; out device [T][H] of type odt (out)
 */
int moe_combine(const float* y_perm, const float* topk_w, const int32_t* inv_perm, int T, int k, int H,
                const float* shared_y, void* out, int odt, void* stream);

/* -------------------------------------------------------------- expert cache */

/*
 * HBM residency cache for an expert bank that lives in host memory ("What expert
 * offloading actually costs", "Inside expert paging": stable logical slots over moving
 * physical residency; theflow.svmpsp.dev related-abstracts list: an LRU cache serves
 * most expert lookups).  Keys are (layer, expert); one global pool of `capacity` slots.
 * Lookups come in groups (one layer of one step; group g = the g-th moe_cache_plan call,
 * from 0); duplicate ids in a group count once; a distinct id found resident is a hit;
 * every id of the group gets tick g.  The cache starts empty.  A miss evicts a resident key
 * not in the current group:
 *   MOE_CACHE_LRU (0): the one with the smallest (tick, layer*E + expert);
 *   MOE_CACHE_LFU_DECAY (1): every key carries a use count; at the start of group g, when
 *     decay_period > 0, g > 0 and g % decay_period == 0, every count is halved (integer
 *     shift); then every key of the group gains 1024; the victim is the one with the
 *     smallest (count, tick, layer*E + expert).  Under a skewed, slowly drifting expert
 *     popularity this keeps the popular experts resident through bursts of one-off lookups.
 *
 * The cache object keeps the two pointers of its descriptor (it does not own them) and is
 * host-side state with a single owner (not thread-safe).
 */
typedef struct moe_cache moe_cache_t;

typedef struct {
  const void* host_bank; /* host, page-locked (hipHostMalloc): [L][E] packages, pkg_bytes apart */
  size_t pkg_bytes;      /* bytes per package (copy size and bank stride) */
  int L, E;              /* layers, experts per layer */
  void* device_pool;     /* device: capacity slots, slot_stride bytes apart */
  size_t slot_stride;    /* >= pkg_bytes, multiple of 256 */
  int capacity;          /* number of slots (1 .. L*E) */
  int policy;            /* MOE_CACHE_LRU or MOE_CACHE_LFU_DECAY */
  int decay_period;      /* LFU_DECAY: groups between halvings of the counts (0: never) */
} moe_cache_desc;

enum { MOE_CACHE_LRU = 0, MOE_CACHE_LFU_DECAY = 1 };

typedef struct {
  int layer;
  int n_ids;          /* distinct expert ids looked up */
  int n_hits, n_misses;
  int32_t miss_ids[1024];  /* experts to fetch (ascending) */
  int32_t miss_slots[1024]; /* slot each of them goes to */
  int32_t slot_of_expert[1024]; /* host copy of this layer's expert -> slot table (-1 = absent) */
} moe_cache_plan_t;

typedef struct {
  int64_t lookups, hits, misses, evictions;
  int64_t bytes_fetched;
} moe_cache_stats_t;

/*
 * Create a cache over desc (pointers kept, not owned).
 * Errors: MOE_ERR_INVALID (null pointers, sizes); MOE_ERR_NOT_PINNED if host_bank is not
 * page-locked HIP host memory (checked with hipPointerGetAttributes).
 */
int moe_cache_create(const moe_cache_desc* desc, moe_cache_t** out);

/*
 * Host only, synchronous: look up the n expert ids host_ids[0..n) of `layer` (the ids a
 * router chose, already copied to the host), update the policy state and fill *plan.
 * Errors: MOE_ERR_INVALID (bad layer, id outside [0, E), n < 0), MOE_ERR_CAPACITY if the
 * group has more distinct ids than the cache has slots (state is then unchanged).
 */
int moe_cache_plan(moe_cache_t* c, int layer, const int32_t* host_ids, int n, moe_cache_plan_t* plan);

/*
 * Enqueue on copy_stream one host->device copy per miss of *plan (bank package ->
 * its slot), then the copy of plan->slot_of_expert to dev_slot_of_expert (device [E],
 * usable as moe_experts.slot_of_expert with packages = device_pool), then record `done`
 * (a hipEvent_t as void*, may be NULL) so the compute stream can wait on it.
 * The plan's table is copied from the plan object: keep *plan alive until done.
 */
int moe_cache_fetch(moe_cache_t* c, const moe_cache_plan_t* plan, int32_t* dev_slot_of_expert, void* copy_stream,
                    void* done);

int moe_cache_stats(const moe_cache_t* c, moe_cache_stats_t* out);
void moe_cache_destroy(moe_cache_t* c);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
