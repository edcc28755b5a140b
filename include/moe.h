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

/*
 * moe_expert_ffn variants: AUTO picks per expert from its row count (weight streaming for few rows, the
 * MFMA tile kernel for many); DECODE streams every expert; PREFILL tiles every expert.
 * DECODE_MX (MXFP4 experts only) streams every expert on the block-scaled matrix cores
 * (v_mfma_scale_f32_16x16x128_f8f6f4): the FP4 weights and their E8M0 scales enter the MFMA as stored,
 * and the activations (x, then h) are first rounded to two MXFP8 (E4M3) terms per 32-element block,
 * x = 2^e hi + 2^(e-4) lo, which holds each element to within 2^-8 of its magnitude.
 */
typedef enum { MOE_FFN_AUTO = 0, MOE_FFN_DECODE = 1, MOE_FFN_PREFILL = 2, MOE_FFN_DECODE_MX = 3 } moe_ffn_mode;

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
 * Logits that are not finite: +inf and -inf order as numbers, NaN below -inf; a token always gets
 * k distinct ids in [0, E) (a token whose logits are all NaN gets ids 0..k-1), and a NaN among its
 * chosen logits (or infinities of both signs) makes that token's gate weights NaN; other tokens
 * are not affected.
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
 *   offsets[e]  exclusive prefix sum of counts; offsets[E] = the number of pairs placed
 *               (T*k when every id is valid)                      device [E+1] int32 (out)
 *   perm_src[p] flat index t*k+j of the p-th pair in expert-major order, ascending
 *               flat index inside an expert, p < offsets[E]       device [T*k] int32 (out)
 *   inv_perm[i] position p of flat index i (perm_src[inv_perm[i]] == i), or -1 for a
 *               dropped pair                                      device [T*k] int32 (out)
 *   topk_ids    device [T][k] int32
 * A pair whose id lies outside [0, E) is dropped: not counted, not placed, inv_perm -1 (the
 * combine then skips it).  moe_route never produces such ids.
 * Errors: MOE_ERR_INVALID for null pointers (T > 0), E out of 1..1024, k < 1,
 * T*k > 1<<24; MOE_ERR_WORKSPACE if ws_bytes < moe_permute_workspace(T, k, E).
 */
int moe_permute(const int32_t* topk_ids, int T, int k, int E, int32_t* counts, int32_t* offsets, int32_t* perm_src,
                int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream);

/* --------------------------------------------------- router + permutation */

/*
 * moe_route followed by moe_permute on its ids, in one call: the same outputs, bit for bit, as
 * those two calls (arguments as there).  Decode batches in bf16 (T <= 16, T*k <= 1024, T*E <= 2^20,
 * H a multiple of 32) take two launches instead of three: the router's partial logits, then one
 * workgroup that sums them, selects the top k of every token and groups the pairs.  Other
 * batches run the two calls' kernels one after the other.  (The routing and grouping steps are
 * those of "Mixture of experts VRAM: total vs active parameters", section "How current MoE models
 * route each token", and of "Understanding MoE Inference Costs on Galactus", section "Prompt
 * processing is a different phase".)
 *   ws  device workspace of ws_bytes >= moe_route_permute_workspace(T, H, E, k, xdt) bytes
 * Errors: those of moe_route and moe_permute; MOE_ERR_WORKSPACE if the workspace is too small.
 */
int moe_route_permute(const void* x, int xdt, int T, int H, const void* w_router, const float* bias, int E, int k,
                      int32_t* topk_ids, float* topk_w, float* logits, int32_t* counts, int32_t* offsets,
                      int32_t* perm_src, int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes moe_route_permute needs (device, 256-byte aligned): the router's partial logits
 * on the fused path, else moe_route_workspace and moe_permute_workspace, each rounded up to 256. */
size_t moe_route_permute_workspace(int T, int H, int E, int k, int xdt);

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
 * multiple of 32, or (INT4) a nonzero scale s lies outside [2^-14, 65504/8] in magnitude: the
 * kernels compute INT4 experts on binary16 operands, where every q * s (q in [-8, 7]) is then an
 * exact finite normal-range value (subnormal or NaN scales, and scales whose products overflow,
 * are refused rather than rounded).
 */
int moe_pack_expert(int H, int I, int fmt, const void* gate, const void* gate_scales, const void* up,
                    const void* up_scales, const void* down, const void* down_scales, void* package,
                    size_t package_bytes);

/*
 * Test hook: decode a package on the device back to the logical layout in fp32:
 * out = [gate I*H][up I*H][down H*I] (device, 3*H*I floats).  Every value is exact.
 */
int moe_dequant_expert(const void* package, int H, int I, int fmt, float* out, void* stream);

/* ------------------------------------------------- lossless package compression */

/*
 * A tier of losslessly compressed experts in GPU memory and in host memory ("What expert
 * offloading actually costs", section "Inside expert paging": compressed GPU memory beside host
 * DRAM, lossless so that no output bit changes).  The pages name no codec; this one is an
 * exponent-window code for bf16 packages, decoded on the GPU into a plain package that the FFN
 * kernels read as usual:
 *  - the package is read as little-endian bf16 values in chunks of 512 (1024 bytes; the package
 *    size must be a multiple of 1024, as every bf16 package is);
 *  - per chunk, M = the largest exponent field, window base b = max(M - 14, 0); a value whose
 *    exponent e lies in [b, b + 14] gets the 4-bit code e - b + 1, any other value the code 0
 *    and an escape byte holding e;
 *  - a coded chunk is 512 bytes (sign << 7 | 7-bit mantissa, value order), 256 bytes of codes
 *    (value 2t in the low nibble of byte t, value 2t+1 in the high one), the escape bytes in
 *    value order, zeros to a multiple of 16: 768 + 16 ceil(escapes / 16) bytes; a chunk for which
 *    that is 1024 or more is stored raw;
 *  - the blob: a 64-byte header (u32 magic 0x31345758, u32 chunk count n, u64 package bytes,
 *    u64 data offset, u64 blob bytes, zeros), u32 chunk offsets off[0..n] relative to the data
 *    offset, u8 window bases (0 for raw chunks), zeros up to the data offset (the first multiple
 *    of 256 past the tables), then the chunks back to back; a chunk of off[i+1] - off[i] = 1024
 *    bytes is raw.
 * bf16 weights around zero compress to about 75% (12 bits per value).  4-bit packages are not
 * compressed: their codes carry 3.6-3.9 bits of entropy each, which no fixed-width code can use.
 */

/* Largest blob for a package of raw_bytes bytes (0 if raw_bytes is not a multiple of 1024). */
size_t moe_compress_bound(size_t raw_bytes);

/*
 * Host, offline: encode one package.
 *   raw   host, raw_bytes (a multiple of 1024, below 4 GiB)
 *   blob  host, cap >= moe_compress_bound(raw_bytes) bytes (out); *blob_bytes = its size (out)
 * Errors: MOE_ERR_INVALID (size, null pointers, small cap).
 */
int moe_compress_package(const void* raw, size_t raw_bytes, void* blob, size_t cap, size_t* blob_bytes);

/*
 * Decode n blobs into packages on the device, in one launch:
 *   src_base   device, blob j at src_base + pairs[2j] * src_stride (src_stride a multiple of 256)
 *   dst_base   device, its package at dst_base + pairs[2j+1] * dst_stride (dst_stride a multiple
 *              of 16, >= raw_bytes)
 *   pairs      device [n][2] int32 {source slot, destination slot}; a pair with a negative slot
 *              is skipped (so one slot table can serve several passes)
 *   raw_bytes  every package's size (a multiple of 1024)
 * The blobs must come from moe_compress_package (the decoder trusts their tables).
 * Errors: MOE_ERR_INVALID (sizes, strides, n out of 0..65535, null pointers when n > 0).
 */
int moe_decompress_packages(const void* src_base, size_t src_stride, void* dst_base, size_t dst_stride,
                            const int32_t* pairs, int n, size_t raw_bytes, void* stream);

/*
 * A second lossless code, for any package (4-bit ones included): an order-0 rANS code of its bytes.
 *  - the package of n bytes is cut at byte `split` into two regions (its codes, then its scales),
 *    each coded on its own;
 *  - region model: h[s] = occurrences of byte s in the region (m bytes); f[s] = max(1, floor(4096
 *    h[s] / m)) for present s, else 0; while the f sum to more than 4096 the largest (smallest s
 *    among equals) loses one, while they sum to less the largest gains the rest; c[s] = f[0] + ...
 *    + f[s-1];
 *  - region byte j is symbol j div 32768 of stream j mod 32768.  A stream is coded from state
 *    x = 2^16, last symbol first: before symbol s, if x >= 2^20 f[s] the low 16 bits of x are a
 *    word and x shifts right by 16; then x = 4096 (x div f[s]) + (x mod f[s]) + c[s]; the final x
 *    is the stream's state.  Decoding: s is the symbol with c[s] <= x mod 4096 < c[s] + f[s], then
 *    x = f[s] (x div 4096) + (x mod 4096) - c[s], and if x < 2^16, x = 2^16 x + the next word;
 *  - streams 64g .. 64g+63 share one word sequence, in decoding order: per symbol index, the words
 *    the streams read after it, in stream order;
 *  - blob: a 64-byte header (u32 magic 0x31534E52, u32 32768, u64 n, u64 split, u64 blob bytes,
 *    zeros), then per region: u16 f[256], u32 states[32768], u32 word offsets off[0..512] (group g:
 *    words off[g] .. off[g+1]-1), the u16 words, zeros up to a multiple of 16 bytes.
 * GLM-shaped INT4 packages take 88.5% of their bytes, gpt-oss-shaped MXFP4 ones 92.7%.
 */

/* Largest rANS blob for a package of raw_bytes bytes. */
size_t moe_compress_rans_bound(size_t raw_bytes);

/*
 * Host, offline: encode one package, cut into regions at byte `split` (<= raw_bytes < 4 GiB).
 *   blob  host, cap >= moe_compress_rans_bound(raw_bytes) bytes (out); *blob_bytes = its size
 * Errors: MOE_ERR_INVALID (sizes, null pointers, small cap).
 */
int moe_compress_rans(const void* raw, size_t raw_bytes, size_t split, void* blob, size_t cap, size_t* blob_bytes);

/*
 * Decode n rANS blobs into packages on the device, in one launch (slots and pairs as for
 * moe_decompress_packages; src_stride a multiple of 256, dst_stride >= raw_bytes).  A blob whose
 * header names another package size is skipped (nothing written).  The blobs must come from
 * moe_compress_rans (the decoder trusts their tables).
 * Errors: MOE_ERR_INVALID (strides, n out of 0..65535, null pointers when n > 0).
 */
int moe_decompress_rans(const void* src_base, size_t src_stride, void* dst_base, size_t dst_stride,
                        const int32_t* pairs, int n, size_t raw_bytes, void* stream);

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
 * INT4 -> fp16 operands) accumulated in fp32; f32 experts run in fp32 throughout.
 * Activations: fp32 input for bf16 / MXFP4 experts is rounded to bf16.  For INT4 experts each
 * token's row is divided by a power of two s_t that puts its largest finite magnitude in [4, 8)
 * and then rounded to fp16 (so any finite activation magnitude is safe; elements more than 2^19
 * times smaller than the row's largest lose bits); the gate is evaluated on the unscaled value.
 * The intermediate SiLU(g)*u is rounded once to the operand type; for INT4 it is SiLU(g)*u / s_t^2
 * in fp16, bounded by 64 * |W_gate row|_1 * |W_up row|_1 whatever the activations (finite when that
 * bound is below 65504; typical values are about H times smaller), and the down result is
 * multiplied back by s_t^2 in fp32.
 * A shared (always-on) expert is the same call with E = 1, offsets = {0, T}, k = 1 and
 * perm_src = {0, 1, ..., T-1}.
 * Errors: MOE_ERR_INVALID (null pointers, sizes), MOE_ERR_UNSUPPORTED (H, I not multiples
 * of 32; INT4 experts with activations not 16-byte aligned; MOE_FFN_DECODE_MX with experts that
 * are not MXFP4), MOE_ERR_WORKSPACE (ws smaller than moe_ffn_workspace for this mode).
 */
int moe_expert_ffn(const moe_experts* w, const void* x, int xdt, int T, int k, const int32_t* offsets,
                   const int32_t* perm_src, float* y_perm, int mode, void* ws, size_t ws_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under stream capture, serving loops and
 * harnesses that forbid hipMalloc): moe_expert_ffn with its workspace taken from a static device
 * array of MOE_FFN_NOALLOC_MAX_WORKSPACE bytes that the library holds on every device it runs on
 * until the process ends.  Same arguments, semantics and results as moe_expert_ffn (the same
 * kernels); the call allocates nothing.  The array's device address is looked up on the first call
 * made with a device current.  All calls on one device share its array and nothing of it survives
 * a call: calls in flight together on one device (several streams or host threads) race on it and
 * must be serialised by the caller.
 * Errors: as moe_expert_ffn; MOE_ERR_WORKSPACE when moe_ffn_workspace(w, T, k, mode) exceeds
 * MOE_FFN_NOALLOC_MAX_WORKSPACE (use moe_expert_ffn with a caller workspace then).
 */
#define MOE_FFN_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)
int moe_expert_ffn_noalloc(const moe_experts* w, const void* x, int xdt, int T, int k, const int32_t* offsets,
                           const int32_t* perm_src, float* y_perm, int mode, void* stream);

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
 * then one rounding (nearest-even) to odt.  Deterministic: no atomics.  A pair with
 * inv_perm -1 (dropped by moe_permute) contributes nothing.
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
 * Pinned keys (moe_cache_pin) are never evicted; a key a prefetch brought in has tick -1 until a
 * demand lookup uses it (moe_cache_prefetch).
 *
 * The cache object keeps the two pointers of its descriptor (it does not own them) and is
 * host-side state with a single owner (not thread-safe).
 */
typedef struct moe_cache moe_cache_t;

/* A copy engine: enqueue (or perform) a copy of `bytes` from src to dst on `stream`; return 0 on
 * success, nonzero on failure.  The default engine is hipMemcpyAsync host -> device. */
typedef int (*moe_copy_fn)(void* ctx, void* dst, const void* src, size_t bytes, void* stream);

typedef struct {
  const void* host_bank; /* host, page-locked (hipHostMalloc): [L][E] packages, pkg_bytes apart */
  size_t pkg_bytes;      /* bytes per package (copy size and bank stride) */
  int L, E;              /* layers, experts per layer */
  void* device_pool;     /* device: capacity slots, slot_stride bytes apart */
  size_t slot_stride;    /* >= pkg_bytes, multiple of 256 */
  int capacity;          /* number of slots (1 .. L*E) */
  int policy;            /* MOE_CACHE_LRU or MOE_CACHE_LFU_DECAY */
  int decay_period;      /* LFU_DECAY: groups between halvings of the counts (0: never) */
  moe_copy_fn copy;      /* NULL: hipMemcpyAsync (host_bank must then be page-locked); otherwise every
                            package and slot-table copy of moe_cache_fetch goes through it, and host_bank
                            and device_pool are whatever memory it understands (not checked) */
  void* copy_ctx;        /* first argument of `copy` */
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
  int64_t lookups, hits, misses, evictions; /* demand lookups (moe_cache_plan) and all evictions */
  int64_t bytes_fetched;                    /* package bytes of every fetch planned (demand, prefetch,
                                               pin), less those a failed fetch rolled back; with a
                                               rANS bank read by hipMemcpyAsync, each fetched blob's
                                               own bytes */
  int64_t prefetch_fetches;                 /* packages a prefetch brought in */
  int64_t prefetch_hits;                    /* demand hits on such a package before its eviction */
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
 * Host only, synchronous: fetch ahead of use (best effort).  Makes the experts host_ids[0..n) of
 * `layer` resident if slots allow, without counting demand lookups: each absent one takes a free
 * slot or evicts the policy's first candidate that is neither in this set nor in the latest demand
 * group (whose FFN may still be reading its slots); when no such candidate is left the remaining
 * ones are skipped.  A prefetched expert enters as the first eviction candidate (last use "never",
 * use count unchanged) until a demand lookup uses it; experts already resident are left as they
 * are.  *plan lists the fetches (n_hits = already resident); enqueue them with moe_cache_fetch on
 * the same copy stream as the demand fetches, so that a later demand fetch's event covers them.
 * The intended use (predictor-free, "Understanding MoE Inference Costs on Galactus" and the Edge0
 * abstract of the theflow.svmpsp.dev list): while layer l computes, prefetch what layer l + 1 used
 * at the previous step, or its most used experts.
 * Errors: MOE_ERR_INVALID (bad layer or id).
 */
int moe_cache_prefetch(moe_cache_t* c, int layer, const int32_t* host_ids, int n, moe_cache_plan_t* plan);

/*
 * Host only, synchronous: pin the experts host_ids[0..n) of `layer`: they become resident (absent
 * ones take free slots or evict as a prefetch would) and are never evicted afterwards; demand
 * lookups find them as hits.  A static pin of the popular experts beside the cache policy for the
 * rest (theflow.svmpsp.dev list, the router-locality study: static-pin hit rate).  *plan lists the
 * fetches; enqueue them with moe_cache_fetch.
 * Errors: MOE_ERR_INVALID (bad layer or id); MOE_ERR_CAPACITY if the absent ones do not fit the
 * free and evictable slots (state unchanged).  moe_cache_plan fails with MOE_ERR_CAPACITY for a
 * group whose misses do not fit the slots left unpinned.
 */
int moe_cache_pin(moe_cache_t* c, int layer, const int32_t* host_ids, int n, moe_cache_plan_t* plan);

/*
 * Enqueue on copy_stream one host->device copy per miss of *plan (bank package ->
 * its slot), then the copy of plan->slot_of_expert to dev_slot_of_expert (device [E],
 * usable as moe_experts.slot_of_expert with packages = device_pool), then record `done`
 * (a hipEvent_t as void*, may be NULL) so the compute stream can wait on it.
 * The plan's table is copied from the plan object: keep *plan alive until done.
 * A copy that fails to enqueue rolls the plan back from that miss on: those experts are no longer
 * resident (their slots are free again, and the next lookup of them misses and fetches them
 * again); the call returns MOE_ERR_HIP and the plan's slot table must not be used.
 */
int moe_cache_fetch(moe_cache_t* c, const moe_cache_plan_t* plan, int32_t* dev_slot_of_expert, void* copy_stream,
                    void* done);

/*
 * Declare the bank's packages rANS blobs (moe_compress_rans, one per bank slot of pkg_bytes) of
 * packages of raw_bytes bytes (<= slot_stride): the host tier holds the compressed bytes and the
 * pool plain packages ("Understanding MoE Inference Costs on Galactus": compressed memory beside
 * host DRAM as the cheaper tier), so a miss moves the blob (GLM-shaped INT4 experts: 88.5% of the
 * package) and hits cost nothing extra.  From then on moe_cache_fetch copies each miss's blob into
 * one of `staging_slots` device staging slots (staging: device, staging_slots * staging_stride
 * bytes, staging_stride >= pkg_bytes and a multiple of 256; the cache uses it, the caller owns it)
 * and a decode stream created here (on the current device, default priority) decodes it into the
 * pool slot while the copy stream moves on to the next blob; before `done` the copy stream waits
 * for the fetch's last decode, so `done` (and any later event of the copy stream) covers the
 * decoded packages.  A staging slot is rewritten only after the decode that read it.  With the
 * default copy engine only the blob's own bytes cross the link, and a bank slot whose header is
 * not a rANS blob of raw_bytes fails the fetch (MOE_ERR_INVALID, rolled back as a failed copy).
 * Call once, before the first fetch; moe_cache_destroy waits for the decode stream.
 * Errors: MOE_ERR_INVALID (null pointers, sizes, a planning-only cache, a second call);
 * MOE_ERR_HIP (stream or event creation).
 */
int moe_cache_set_rans(moe_cache_t* c, void* staging, size_t staging_stride, int staging_slots, size_t raw_bytes);

int moe_cache_stats(const moe_cache_t* c, moe_cache_stats_t* out);
void moe_cache_destroy(moe_cache_t* c);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
