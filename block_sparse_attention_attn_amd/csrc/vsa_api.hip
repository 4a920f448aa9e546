// vsa_api.hip -- the extern "C" entry points of libvsa.so declared in include/vsa.h: host-side
// validation (no device reads), workspace sizing and the stream-ordered launch chains. Nothing
// here allocates, frees or synchronizes.
//
// The backward chain follows the FastVideo backward launch header (its launch function:
// support check -> preprocess -> order when nb >= 1024 and no order was given -> main ->
// postprocess, every launch on the caller's stream and checked right after), minus the TMA
// descriptor set-up and the transposed Q/dO copies, which gfx950 does not need: its main kernel
// reads transposed operands from LDS with ds_read_b64_tr_b16.
#include <cmath>
#include <cstdio>
#include <string>

#include "../../include/vsa.h"
#include "vsa_kernels.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(VSA_ELAUNCH, std::string(what) + ": " + hipGetErrorString(e));
  return VSA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr size_t kMaxElems = (size_t)1 << 40;  // guard against size_t overflow in products

bool dims_ok(int batch, int heads, int seqlen, int nb) {
  if (batch < 1 || heads < 1 || nb < 1) return false;
  if ((long long)seqlen != (long long)nb * vsa::BLOCK) return false;
  const long long bh = (long long)batch * heads;
  if (bh * nb >= (1LL << 31)) return false;  // item ids are int32
  if ((size_t)bh * (size_t)seqlen * vsa::HEAD_DIM >= kMaxElems) return false;
  return true;
}

}  // namespace

extern "C" {

const char* vsa_status_string(int status) {
  switch (status) {
    case VSA_OK: return "VSA_OK";
    case VSA_EINVAL: return "VSA_EINVAL: invalid argument";
    case VSA_EUNSUPPORTED: return "VSA_EUNSUPPORTED: unsupported configuration";
    case VSA_ELAUNCH: return "VSA_ELAUNCH: kernel launch failed";
    default: return "VSA: unknown status";
  }
}

const char* vsa_last_error(void) { return g_last_error.c_str(); }

// ------------------------------------------------------------------------------------------------
// invert_indices
// ------------------------------------------------------------------------------------------------

size_t vsa_invert_workspace_bytes(int batch, int heads, int nq, int nkv) {
  if (batch < 1 || heads < 1 || nq < 1 || nkv < 1) return 0;
  return align256(vsa::invert_bitmap_bytes(batch * heads, nq, nkv));
}

int vsa_invert_indices(const int32_t* q2k_idx, const int32_t* q2k_num, int batch, int heads,
                       int nq, int topk, int nkv, int32_t* k2q_idx, int32_t* k2q_num,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if (batch < 1 || heads < 1 || nq < 1 || topk < 1 || nkv < 1)
    return fail(VSA_EINVAL, "vsa_invert_indices: batch, heads, nq, topk and nkv must be >= 1");
  if ((long long)batch * heads * nkv >= (1LL << 31) ||
      (size_t)batch * heads * (size_t)nkv * (size_t)nq >= kMaxElems ||
      (size_t)batch * heads * (size_t)nq * (size_t)topk >= kMaxElems)
    return fail(VSA_EINVAL, "vsa_invert_indices: sizes too large");
  if (!q2k_idx || !q2k_num || !k2q_idx || !k2q_num || !workspace)
    return fail(VSA_EINVAL, "vsa_invert_indices: null pointer");
  const size_t need = vsa_invert_workspace_bytes(batch, heads, nq, nkv);
  if (workspace_bytes < need)
    return fail(VSA_EINVAL, "vsa_invert_indices: workspace of " + std::to_string(workspace_bytes) +
                                " bytes, need " + std::to_string(need));
  vsa::launch_invert(q2k_idx, q2k_num, batch * heads, nq, topk, nkv, k2q_idx, k2q_num,
                     (uint32_t*)workspace, (hipStream_t)stream);
  return launch_status("vsa_invert_indices");
}

// ------------------------------------------------------------------------------------------------
// forward
// ------------------------------------------------------------------------------------------------

int vsa_fwd_check(const vsa_fwd_args* a) {
  if (!a) return fail(VSA_EINVAL, "vsa_fwd: null argument struct");
  if (a->head_dim != vsa::HEAD_DIM)
    return fail(VSA_EUNSUPPORTED, "vsa_fwd: head_dim must be 128, got " + std::to_string(a->head_dim));
  if (!dims_ok(a->batch, a->heads, a->seqlen, a->num_kv_blocks))
    return fail(VSA_EINVAL, "vsa_fwd: need batch, heads, num_kv_blocks >= 1 and seqlen == 64 * "
                            "num_kv_blocks (got seqlen " + std::to_string(a->seqlen) +
                                ", num_kv_blocks " + std::to_string(a->num_kv_blocks) + ")");
  if (a->q2k_stride < 1) return fail(VSA_EINVAL, "vsa_fwd: q2k_stride must be >= 1");
  if (!std::isfinite(a->sm_scale)) return fail(VSA_EINVAL, "vsa_fwd: sm_scale must be finite");
  if (!a->q || !a->k || !a->v || !a->q2k_idx || !a->q2k_num || !a->vbs || !a->o || !a->lse)
    return fail(VSA_EINVAL, "vsa_fwd: null pointer");
  return VSA_OK;
}

int vsa_fwd(const vsa_fwd_args* a, void* stream) {
  const int st = vsa_fwd_check(a);
  if (st != VSA_OK) return st;
  vsa::FwdParams p;
  p.q = (const vsa::bf16*)a->q;
  p.k = (const vsa::bf16*)a->k;
  p.v = (const vsa::bf16*)a->v;
  p.q2k_idx = a->q2k_idx;
  p.q2k_num = a->q2k_num;
  p.vbs = a->vbs;
  p.o = (vsa::bf16*)a->o;
  p.lse = a->lse;
  p.BH = a->batch * a->heads;
  p.S = a->seqlen;
  p.nb = a->num_kv_blocks;
  p.q2k_stride = a->q2k_stride;
  p.scale_log2 = a->sm_scale * 1.4426950408889634f;
  vsa::launch_fwd(p, (hipStream_t)stream);
  return launch_status("vsa_fwd");
}

// ------------------------------------------------------------------------------------------------
// backward
// ------------------------------------------------------------------------------------------------

void vsa_bwd_workspace_layout(int batch, int heads, int seqlen, size_t* dqacc_off,
                              size_t* delta_off, size_t* order_off) {
  const size_t rows = (size_t)(batch < 0 ? 0 : batch) * (size_t)(heads < 0 ? 0 : heads) *
                      (size_t)(seqlen < 0 ? 0 : seqlen);
  const size_t dq = align256(rows * vsa::HEAD_DIM * sizeof(float));
  const size_t delta = align256(rows * sizeof(float));
  if (dqacc_off) *dqacc_off = 0;
  if (delta_off) *delta_off = dq;
  if (order_off) *order_off = dq + delta;
}

size_t vsa_bwd_workspace_bytes(int batch, int heads, int seqlen) {
  if (batch < 1 || heads < 1 || seqlen < vsa::BLOCK) return 0;
  size_t order_off = 0;
  vsa_bwd_workspace_layout(batch, heads, seqlen, nullptr, nullptr, &order_off);
  const size_t items = (size_t)batch * heads * (size_t)(seqlen / vsa::BLOCK);
  return order_off + align256(items * sizeof(int32_t));
}

int vsa_bwd_check(const vsa_bwd_args* a) {
  if (!a) return fail(VSA_EINVAL, "vsa_bwd: null argument struct");
  if (a->head_dim != vsa::HEAD_DIM)
    return fail(VSA_EUNSUPPORTED, "vsa_bwd: head_dim must be 128, got " + std::to_string(a->head_dim));
  if (!dims_ok(a->batch, a->heads, a->seqlen, a->num_kv_blocks))
    return fail(VSA_EINVAL, "vsa_bwd: need batch, heads, num_kv_blocks >= 1 and seqlen == 64 * "
                            "num_kv_blocks (got seqlen " + std::to_string(a->seqlen) +
                                ", num_kv_blocks " + std::to_string(a->num_kv_blocks) + ")");
  if (a->max_q_blocks < 1) return fail(VSA_EINVAL, "vsa_bwd: max_q_blocks must be >= 1");
  if ((size_t)a->batch * a->heads * (size_t)a->num_kv_blocks * (size_t)a->max_q_blocks >= kMaxElems)
    return fail(VSA_EINVAL, "vsa_bwd: k2q_idx too large");
  if (!std::isfinite(a->sm_scale)) return fail(VSA_EINVAL, "vsa_bwd: sm_scale must be finite");
  if (!a->q || !a->k || !a->v || !a->o || !a->dout || !a->lse)
    return fail(VSA_EINVAL, "vsa_bwd: null input pointer");
  if (!a->k2q_idx || !a->k2q_num || !a->vbs)
    return fail(VSA_EINVAL, "vsa_bwd: null index pointer");
  if (!a->dq || !a->dk || !a->dv) return fail(VSA_EINVAL, "vsa_bwd: null output pointer");
  if (!a->workspace) return fail(VSA_EINVAL, "vsa_bwd: null workspace");
  const size_t need = vsa_bwd_workspace_bytes(a->batch, a->heads, a->seqlen);
  if (a->workspace_bytes < need)
    return fail(VSA_EINVAL, "vsa_bwd: workspace of " + std::to_string(a->workspace_bytes) +
                                " bytes, need " + std::to_string(need));
  return VSA_OK;
}

int vsa_bwd_order(const int32_t* k2q_num, int batch, int heads, int num_kv_blocks, int bin_width,
                  int32_t* order, void* stream) {
  if (!k2q_num || !order) return fail(VSA_EINVAL, "vsa_bwd_order: null pointer");
  if (batch < 1 || heads < 1 || num_kv_blocks < 1 || bin_width < 1)
    return fail(VSA_EINVAL, "vsa_bwd_order: batch, heads, num_kv_blocks, bin_width must be >= 1");
  if (num_kv_blocks > VSA_ORDER_MAX_KV_BLOCKS)
    return fail(VSA_EUNSUPPORTED, "vsa_bwd_order: num_kv_blocks above " +
                                      std::to_string(VSA_ORDER_MAX_KV_BLOCKS));
  if ((long long)batch * heads * num_kv_blocks >= (1LL << 31))
    return fail(VSA_EINVAL, "vsa_bwd_order: too many items");
  vsa::launch_bwd_order(k2q_num, batch * heads, num_kv_blocks, bin_width, order,
                        (hipStream_t)stream);
  return launch_status("vsa_bwd_order");
}

namespace {

bool uses_device_order(const vsa_bwd_args* a) {
  return !a->order && a->num_kv_blocks >= VSA_ORDER_MIN_KV_BLOCKS &&
         a->num_kv_blocks <= VSA_ORDER_MAX_KV_BLOCKS;
}

int run_stage(const vsa_bwd_args* a, int stage, hipStream_t s) {
  const int BH = a->batch * a->heads;
  const int nb = a->num_kv_blocks;
  size_t dq_off, delta_off, order_off;
  vsa_bwd_workspace_layout(a->batch, a->heads, a->seqlen, &dq_off, &delta_off, &order_off);
  char* ws = (char*)a->workspace;
  float* dqaccum = (float*)(ws + dq_off);
  float* delta = (float*)(ws + delta_off);
  int32_t* order_ws = (int32_t*)(ws + order_off);

  switch (stage) {
    case VSA_BWD_PREPROCESS: {
      vsa::BwdPreParams pre;
      pre.o = (const vsa::bf16*)a->o;
      pre.dout = (const vsa::bf16*)a->dout;
      pre.k2q_num = a->k2q_num;
      pre.delta = delta;
      pre.dqaccum = dqaccum;
      pre.dk = (vsa::bf16*)a->dk;
      pre.dv = (vsa::bf16*)a->dv;
      pre.BH = BH;
      pre.S = a->seqlen;
      pre.nb = nb;
      vsa::launch_bwd_pre(pre, s);
      return launch_status("vsa_bwd preprocess");
    }
    case VSA_BWD_ORDER:
      if (!uses_device_order(a)) return VSA_OK;
      vsa::launch_bwd_order(a->k2q_num, BH, nb, 8, order_ws, s);
      return launch_status("vsa_bwd order");
    case VSA_BWD_MAIN: {
      vsa::BwdMainParams m;
      m.q = (const vsa::bf16*)a->q;
      m.k = (const vsa::bf16*)a->k;
      m.v = (const vsa::bf16*)a->v;
      m.dout = (const vsa::bf16*)a->dout;
      m.lse = a->lse;
      m.delta = delta;
      m.k2q_idx = a->k2q_idx;
      m.k2q_num = a->k2q_num;
      m.vbs = a->vbs;
      m.order = a->order ? a->order : (uses_device_order(a) ? order_ws : nullptr);
      m.dqaccum = dqaccum;
      m.dk = (vsa::bf16*)a->dk;
      m.dv = (vsa::bf16*)a->dv;
      m.S = a->seqlen;
      m.nb = nb;
      m.max_q_blocks = a->max_q_blocks;
      m.total_items = BH * nb;
      m.items_per_xcd = (m.total_items + 7) / 8;
      m.sm_scale = a->sm_scale;
      m.scale_log2 = a->sm_scale * 1.4426950408889634f;
      vsa::launch_bwd_main(m, s);
      return launch_status("vsa_bwd main");
    }
    case VSA_BWD_POSTPROCESS:
      vsa::launch_bwd_post(dqaccum, (vsa::bf16*)a->dq, (size_t)BH * a->seqlen * vsa::HEAD_DIM,
                           a->sm_scale, s);
      return launch_status("vsa_bwd postprocess");
    default:
      return fail(VSA_EINVAL, "vsa_bwd_stage: unknown stage " + std::to_string(stage));
  }
}

}  // namespace

int vsa_bwd_stage(const vsa_bwd_args* a, int stage, void* stream) {
  const int st = vsa_bwd_check(a);
  if (st != VSA_OK) return st;
  if (stage < VSA_BWD_PREPROCESS || stage > VSA_BWD_POSTPROCESS)
    return fail(VSA_EINVAL, "vsa_bwd_stage: unknown stage " + std::to_string(stage));
  return run_stage(a, stage, (hipStream_t)stream);
}

int vsa_bwd(const vsa_bwd_args* a, void* stream) {
  const int st = vsa_bwd_check(a);
  if (st != VSA_OK) return st;
  for (int stage = VSA_BWD_PREPROCESS; stage <= VSA_BWD_POSTPROCESS; ++stage) {
    const int r = run_stage(a, stage, (hipStream_t)stream);
    if (r != VSA_OK) return r;
  }
  return VSA_OK;
}

}  // extern "C"
