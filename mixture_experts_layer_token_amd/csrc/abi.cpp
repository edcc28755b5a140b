// C-ABI entry points of libmoe.so: argument validation, then the launches.  No entry point
// allocates device memory or synchronises the device.
#include "common.hpp"

namespace moe {

static thread_local void* const* g_trace = nullptr;

void* const* trace_events() { return g_trace; }

bool fmt_valid(int fmt) { return fmt >= MOE_W_F32 && fmt <= MOE_W_INT4G32; }
bool dtype_valid(int dt) { return dt == MOE_F32 || dt == MOE_BF16; }

static int check_experts(const moe_experts* w, const char* fn) {
  if (!w) return fail(MOE_ERR_INVALID, "%s: null moe_experts", fn);
  if (!fmt_valid(w->fmt)) return fail(MOE_ERR_INVALID, "%s: bad weight format %d", fn, w->fmt);
  if (w->E < 1 || w->E > 1024) return fail(MOE_ERR_INVALID, "%s: E=%d out of 1..1024", fn, w->E);
  if (w->H <= 0 || w->I <= 0) return fail(MOE_ERR_INVALID, "%s: H=%d I=%d", fn, w->H, w->I);
  if (w->H % 32 || w->I % 32)
    return fail(MOE_ERR_UNSUPPORTED, "%s: H=%d and I=%d must be multiples of 32", fn, w->H, w->I);
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_ffn_trace_events(void* const* events) {
  g_trace = events;
  return MOE_OK;
}

extern "C" size_t moe_route_workspace(int T, int H, int E, int xdt) {
  if (T < 0 || H <= 0 || E < 1 || E > 1024 || !dtype_valid(xdt)) return 0;
  return route_workspace(T, H, E, xdt);
}

extern "C" int moe_route(const void* x, int xdt, int T, int H, const void* w_router, const float* bias, int E, int k,
                         int32_t* topk_ids, float* topk_w, float* logits, void* ws, size_t ws_bytes, void* stream) {
  if (!dtype_valid(xdt)) return fail(MOE_ERR_INVALID, "moe_route: bad dtype %d", xdt);
  if (T < 0 || H <= 0) return fail(MOE_ERR_INVALID, "moe_route: T=%d H=%d", T, H);
  if (E < 1 || E > 1024) return fail(MOE_ERR_INVALID, "moe_route: E=%d out of 1..1024", E);
  if (k < 1 || k > E || k > 16) return fail(MOE_ERR_INVALID, "moe_route: k=%d out of 1..min(E,16)", k);
  if (T > 0 && (!x || !w_router || !topk_ids || !topk_w)) return fail(MOE_ERR_INVALID, "moe_route: null pointer");
  return launch_route(x, xdt, T, H, w_router, bias, E, k, topk_ids, topk_w, logits, ws, ws_bytes,
                      (hipStream_t)stream);
}

extern "C" size_t moe_permute_workspace(int T, int k, int E) {
  if (T < 0 || k < 1 || E < 1) return 0;
  return permute_workspace(T, k, E);
}

extern "C" int moe_permute(const int32_t* topk_ids, int T, int k, int E, int32_t* counts, int32_t* offsets,
                           int32_t* perm_src, int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k < 1 || k > 16) return fail(MOE_ERR_INVALID, "moe_permute: T=%d k=%d", T, k);
  if (E < 1 || E > 1024) return fail(MOE_ERR_INVALID, "moe_permute: E=%d out of 1..1024", E);
  if ((long long)T * k > (1LL << 24)) return fail(MOE_ERR_INVALID, "moe_permute: T*k too large");
  if (!counts || !offsets) return fail(MOE_ERR_INVALID, "moe_permute: null counts/offsets");
  if (T > 0 && (!topk_ids || !perm_src || !inv_perm)) return fail(MOE_ERR_INVALID, "moe_permute: null pointer");
  if (ws_bytes < moe_permute_workspace(T, k, E)) return fail(MOE_ERR_WORKSPACE, "moe_permute: workspace too small");
  return launch_permute(topk_ids, T, k, E, counts, offsets, perm_src, inv_perm, ws, ws_bytes, (hipStream_t)stream);
}

extern "C" size_t moe_route_permute_workspace(int T, int H, int E, int k, int xdt) {
  if (T < 0 || H <= 0 || E < 1 || E > 1024 || k < 1 || !dtype_valid(xdt)) return 0;
  return route_permute_workspace(T, H, E, k, xdt);
}

extern "C" int moe_route_permute(const void* x, int xdt, int T, int H, const void* w_router, const float* bias, int E,
                                 int k, int32_t* topk_ids, float* topk_w, float* logits, int32_t* counts,
                                 int32_t* offsets, int32_t* perm_src, int32_t* inv_perm, void* ws, size_t ws_bytes,
                                 void* stream) {
  if (!dtype_valid(xdt)) return fail(MOE_ERR_INVALID, "moe_route_permute: bad dtype %d", xdt);
  if (T < 0 || H <= 0) return fail(MOE_ERR_INVALID, "moe_route_permute: T=%d H=%d", T, H);
  if (E < 1 || E > 1024) return fail(MOE_ERR_INVALID, "moe_route_permute: E=%d out of 1..1024", E);
  if (k < 1 || k > E || k > 16) return fail(MOE_ERR_INVALID, "moe_route_permute: k=%d out of 1..min(E,16)", k);
  if ((long long)T * k > (1LL << 24)) return fail(MOE_ERR_INVALID, "moe_route_permute: T*k too large");
  if (!counts || !offsets) return fail(MOE_ERR_INVALID, "moe_route_permute: null counts/offsets");
  if (T > 0 && (!x || !w_router || !topk_ids || !topk_w || !perm_src || !inv_perm))
    return fail(MOE_ERR_INVALID, "moe_route_permute: null pointer");
  return launch_route_permute(x, xdt, T, H, w_router, bias, E, k, topk_ids, topk_w, logits, counts, offsets, perm_src,
                              inv_perm, ws, ws_bytes, (hipStream_t)stream);
}

extern "C" size_t moe_ffn_workspace(const moe_experts* w, int T, int k, int mode) {
  if (check_experts(w, "moe_ffn_workspace") != MOE_OK || T < 0 || k < 1) return 0;
  return ffn_workspace(w, T, k, mode);
}

extern "C" int moe_expert_ffn(const moe_experts* w, const void* x, int xdt, int T, int k, const int32_t* offsets,
                              const int32_t* perm_src, float* y_perm, int mode, void* ws, size_t ws_bytes,
                              void* stream) {
  return expert_ffn(w, x, xdt, T, k, offsets, perm_src, y_perm, mode, ws, ws_bytes, stream, true);
}

int moe::expert_ffn(const moe_experts* w, const void* x, int xdt, int T, int k, const int32_t* offsets,
                    const int32_t* perm_src, float* y_perm, int mode, void* ws, size_t ws_bytes, void* stream,
                    bool helper_stream) {
  int rc = check_experts(w, "moe_expert_ffn");
  if (rc != MOE_OK) return rc;
  if (!dtype_valid(xdt)) return fail(MOE_ERR_INVALID, "moe_expert_ffn: bad dtype %d", xdt);
  if (T < 0 || k < 1 || k > 16) return fail(MOE_ERR_INVALID, "moe_expert_ffn: T=%d k=%d", T, k);
  if ((long long)T * k > (1LL << 24)) return fail(MOE_ERR_INVALID, "moe_expert_ffn: T*k too large");
  if (mode < MOE_FFN_AUTO || mode > MOE_FFN_DECODE_MX) return fail(MOE_ERR_INVALID, "moe_expert_ffn: mode %d", mode);
  if (mode == MOE_FFN_DECODE_MX && w->fmt != MOE_W_MXFP4)
    return fail(MOE_ERR_UNSUPPORTED, "moe_expert_ffn: the block-scaled mode takes MXFP4 experts (format %d)", w->fmt);
  size_t need = moe_package_bytes(w->H, w->I, w->fmt);
  if (w->pkg_stride < need || w->pkg_stride % 256)
    return fail(MOE_ERR_INVALID, "moe_expert_ffn: pkg_stride %zu (need >= %zu, multiple of 256)", w->pkg_stride, need);
  if (T > 0 && (!w->packages || !x || !offsets || !perm_src || !y_perm))
    return fail(MOE_ERR_INVALID, "moe_expert_ffn: null pointer");
  if (w->slot_of_expert && w->n_slots < 1)
    return fail(MOE_ERR_INVALID, "moe_expert_ffn: n_slots=%d with a slot table", w->n_slots);
  return launch_ffn(w, x, xdt, T, k, offsets, perm_src, y_perm, mode, ws, ws_bytes, (hipStream_t)stream,
                    helper_stream);
}

extern "C" int moe_combine(const float* y_perm, const float* topk_w, const int32_t* inv_perm, int T, int k, int H,
                           const float* shared_y, void* out, int odt, void* stream) {
  if (!dtype_valid(odt)) return fail(MOE_ERR_INVALID, "moe_combine: bad dtype %d", odt);
  if (T < 0 || k < 1 || k > 16 || H <= 0) return fail(MOE_ERR_INVALID, "moe_combine: T=%d k=%d H=%d", T, k, H);
  if (T > 0 && (!y_perm || !topk_w || !inv_perm || !out)) return fail(MOE_ERR_INVALID, "moe_combine: null pointer");
  return launch_combine(y_perm, topk_w, inv_perm, T, k, H, shared_y, out, odt, (hipStream_t)stream);
}

extern "C" int moe_dequant_expert(const void* package, int H, int I, int fmt, float* out, void* stream) {
  if (!fmt_valid(fmt)) return fail(MOE_ERR_INVALID, "moe_dequant_expert: bad format %d", fmt);
  if (H <= 0 || I <= 0) return fail(MOE_ERR_INVALID, "moe_dequant_expert: H=%d I=%d", H, I);
  if (H % 32 || I % 32) return fail(MOE_ERR_UNSUPPORTED, "moe_dequant_expert: H, I must be multiples of 32");
  if (!package || !out) return fail(MOE_ERR_INVALID, "moe_dequant_expert: null pointer");
  return launch_dequant(package, H, I, fmt, out, (hipStream_t)stream);
}
