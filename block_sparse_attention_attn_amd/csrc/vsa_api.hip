// vsa_api.hip -- the extern "C" entry points of libvsa.so declared in include/vsa.h: host-side
// validation (no device reads), workspace sizing and the stream-ordered launch chains. Nothing
// here allocates, frees or synchronizes.
//
// The backward chain follows the FastVideo backward launch header (its launch function:
// support check -> preprocess -> order when nb >= 1024 and no order was given -> main ->
// postprocess, every launch on the caller's stream and checked right after), with four
// differences made for gfx950: no TMA descriptors or transposed Q/dO copies (the kernels read
// transposed operands from LDS with ds_read_b64_tr_b16); the main step is two atomic-free
// kernels (kv-major dK/dV, q-major dQ) because fp32 atomics cannot carry the per-pair dQ
// partials at MFMA speed on this chip; the dQ postprocess is the q-major kernel's epilogue; and
// the length-binned order starts at VSA_ORDER_MIN_KV_BLOCKS with bin VSA_ORDER_BIN_WIDTH (it
// keeps the items running together on one XCD in step, for L2 reuse of Q/dO).
#include <cmath>
#include <cstdio>
#include <mutex>
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

// blocks per chunk of the main kernels for nb kv blocks and the caller's chunk_blocks (0: the
// library's choice, < 0: off); 0 when they run as one launch each
int chunk_blocks_of(int nb, int chunk_blocks, int dq_mode) {
  if (chunk_blocks < 0) return 0;
  // the library's width: narrower with the spill, whose workspace holds one chunk's tiles (at
  // 524288 tokens, 512 gave 978 ms against 1023 ms for 1024 and 1057 ms for 256)
  const int dflt = dq_mode == VSA_DQ_SPILL ? VSA_SPILL_CHUNK_BLOCKS : VSA_CHUNK_BLOCKS;
  const int cb = chunk_blocks > 0 ? chunk_blocks : (nb >= VSA_CHUNK_MIN_KV_BLOCKS ? dflt : 0);
  return cb > 0 && cb < nb ? cb : 0;  // one chunk covering every block is no chunk
}
// the recomputing q-major kernel runs in chunks only when the caller asks for them (chunk_blocks
// > 0): at 524288 tokens, chunks of 1024 kv blocks left it unchanged and 2048 gained 3 %
int dq_chunk_blocks_of(int nb, int chunk_blocks, int dq_mode) {
  return dq_mode == VSA_DQ_RECOMPUTE && chunk_blocks > 0 ? chunk_blocks_of(nb, chunk_blocks, dq_mode)
                                                         : 0;
}

// q blocks per chunk of a chunked dS spill (spill mode whose kv-major kernel runs in chunks): the
// spill then holds one chunk's tiles at a time, the q-major kernel running after each kv-major
// launch; 0 when the spill holds every pair's tile
int spill_chunk_blocks_of(int nb, int chunk_blocks, int dq_mode) {
  return dq_mode == VSA_DQ_SPILL ? chunk_blocks_of(nb, chunk_blocks, dq_mode) : 0;
}

// sm_scale * log2(e) in fp32: the factor that turns q.k into the base-2 exponent of the softmax
float scale_log2(float sm_scale) { return sm_scale * 1.4426950408889634f; }

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

}  // extern "C"

// helpers: C++ linkage, internal to this file
namespace {

// kv blocks per kv-range chunk of the forward (0: one launch), like chunk_q_blocks
int fwd_chunk_kv_blocks(int nb, int kv_chunk_blocks) {
  if (kv_chunk_blocks < 0) return 0;
  const int ck = kv_chunk_blocks > 0
                     ? kv_chunk_blocks
                     : (nb >= VSA_FWD_CHUNK_MIN_KV_BLOCKS ? VSA_FWD_CHUNK_KV_BLOCKS : 0);
  return ck > 0 && ck < nb ? ck : 0;
}

size_t fwd_bounds_bytes(size_t items, int nchunks) {
  return align256(items * (size_t)(nchunks + 1) * sizeof(int32_t));
}

// The forward workspace starts with the V pre-pass: each head's max |v| bits, then the fp16 copy
// of v ([B, H, S, 128], 2 bytes per element).
size_t fwd_amax_bytes(size_t bh, int seqlen) {  // per head, then per 64-row tile
  return align256(bh * sizeof(uint32_t)) +
         align256(bh * (size_t)(seqlen / vsa::BLOCK) * sizeof(uint32_t));
}
size_t fwd_v16_bytes(size_t bh, int seqlen) {
  return align256(bh * (size_t)seqlen * vsa::HEAD_DIM * 2);
}
size_t fwd_state_bytes(size_t items) {
  return align256(items * 4 * (size_t)vsa::FWD_STATE_FLOATS * sizeof(float));
}
// with kv-range chunks the items are ordered per chunk by the length of their list's part in it,
// where the sort fits one workgroup (the backward's order limits)
bool fwd_chunk_orders(int nb) {
  return nb >= VSA_ORDER_MIN_KV_BLOCKS && nb <= VSA_ORDER_MAX_KV_BLOCKS;
}

}  // namespace

extern "C" {

size_t vsa_fwd_workspace_bytes(int batch, int heads, int seqlen, int kv_chunk_blocks) {
  if (!dims_ok(batch, heads, seqlen, seqlen / vsa::BLOCK)) return 0;
  const int nb = seqlen / vsa::BLOCK;
  const size_t bh = (size_t)batch * heads;
  const size_t v16 = fwd_amax_bytes(bh, seqlen) + fwd_v16_bytes(bh, seqlen);
  const int ck = fwd_chunk_kv_blocks(nb, kv_chunk_blocks);
  if (ck == 0) return v16;
  const size_t items = bh * nb;
  return v16 + fwd_bounds_bytes(items, (nb + ck - 1) / ck) + fwd_state_bytes(items) +
         (fwd_chunk_orders(nb) ? align256(items * sizeof(int32_t)) : 0);
}

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
  const size_t need =
      vsa_fwd_workspace_bytes(a->batch, a->heads, a->seqlen, a->kv_chunk_blocks);
  if (!a->workspace || a->workspace_bytes < need)
    return fail(VSA_EINVAL, "vsa_fwd: workspace of " + std::to_string(a->workspace_bytes) +
                                " bytes, need " + std::to_string(need));
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
  p.items_per_xcd = (p.BH * p.nb + 7) / 8;
  p.scale_log2 = scale_log2(a->sm_scale);
  const int ck = fwd_chunk_kv_blocks(p.nb, a->kv_chunk_blocks);
  p.nchunks = ck > 0 ? (p.nb + ck - 1) / ck : 0;
  p.chunk = 0;
  p.chunk_bounds = nullptr;
  p.state = nullptr;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)a->workspace;
  uint32_t* amax = (uint32_t*)ws;
  uint32_t* tmax = (uint32_t*)(ws + align256((size_t)p.BH * sizeof(uint32_t)));
  vsa::f16* v16 = (vsa::f16*)(ws + fwd_amax_bytes(p.BH, p.S));
  p.v_amax = amax;
  p.v16 = v16;
  vsa::launch_v16(p.v, p.BH, p.S, amax, tmax, v16, s);
  {
    const int r = launch_status("vsa_fwd v pre-pass");
    if (r != VSA_OK) return r;
  }
  ws += fwd_amax_bytes(p.BH, p.S) + fwd_v16_bytes(p.BH, p.S);
  int32_t* order = nullptr;
  if (p.nchunks > 0) {
    const size_t items = (size_t)p.BH * p.nb;
    int32_t* bounds = (int32_t*)ws;
    p.chunk_bounds = bounds;
    p.state = (float*)(ws + fwd_bounds_bytes(items, p.nchunks));
    if (fwd_chunk_orders(p.nb))
      order = (int32_t*)(ws + fwd_bounds_bytes(items, p.nchunks) + fwd_state_bytes(items));
    vsa::launch_chunk_bounds(a->q2k_idx, a->q2k_num, a->q2k_stride, (int)items, p.nchunks, ck,
                             bounds, s);
    const int r = launch_status("vsa_fwd chunk bounds");
    if (r != VSA_OK) return r;
  }
  const int launches = p.nchunks > 0 ? p.nchunks : 1;
  for (int c = 0; c < launches; ++c) {
    p.chunk = c;
    if (order) {  // this chunk's items binned by the length of their list's part in it
      vsa::launch_chunk_order(p.chunk_bounds, a->q2k_num, a->q2k_stride, p.BH, p.nb, p.nchunks, c,
                              VSA_ORDER_BIN_WIDTH, order, s);
      const int r = launch_status("vsa_fwd chunk work order");
      if (r != VSA_OK) return r;
      p.order = order;
    }
    vsa::launch_fwd(p, s);
    const int r = launch_status("vsa_fwd");
    if (r != VSA_OK) return r;
  }
  return VSA_OK;
}

// ------------------------------------------------------------------------------------------------
// backward
// ------------------------------------------------------------------------------------------------

size_t vsa_bwd_workspace_offset(int batch, int heads, int seqlen, int q2k_stride, int dq_mode,
                                int chunk_blocks, int region) {
  if (batch < 1 || heads < 1 || seqlen < vsa::BLOCK || q2k_stride < 0 ||
      (dq_mode != VSA_DQ_RECOMPUTE && dq_mode != VSA_DQ_SPILL) || region < VSA_WS_LSE_DELTA ||
      region > VSA_WS_END)
    return 0;
  const size_t bh = (size_t)batch * (size_t)heads;
  const size_t nb = (size_t)seqlen / vsa::BLOCK;
  const bool derive = q2k_stride == 0;
  const bool spill = dq_mode == VSA_DQ_SPILL;
  const size_t kq = derive ? nb : (size_t)q2k_stride;  // q2k row width
  const int cq = chunk_blocks_of((int)nb, chunk_blocks, dq_mode);
  const size_t nchunks = cq > 0 ? (nb + cq - 1) / cq : 0;
  const int cqq = dq_chunk_blocks_of((int)nb, chunk_blocks, dq_mode);
  const size_t dq_nchunks = cqq > 0 ? (nb + cqq - 1) / cqq : 0;
  // a chunked spill keeps one chunk's slot bases per chunk and one chunk's tiles (at most
  // chunk width x q2k row width per head)
  const int cs = spill_chunk_blocks_of((int)nb, chunk_blocks, dq_mode);
  const size_t kbase_rows = cs > 0 ? nchunks : 1;
  const size_t ds_qblocks = cs > 0 ? (size_t)cs : nb;
  const size_t sizes[VSA_WS_END] = {
      align256(bh * (size_t)seqlen * 2 * sizeof(float)),                      // lse, Delta
      align256(bh * nb * sizeof(int32_t)),                                    // kv order
      align256(bh * nb * sizeof(int32_t)),                                    // q order
      derive ? align256(bh * nb * sizeof(int32_t)) : 0,                       // q2k_num
      derive ? align256(bh * nb * nb * sizeof(int32_t)) : 0,                  // q2k_idx
      derive ? align256(vsa::invert_bitmap_bytes((int)bh, (int)nb, (int)nb)) : 0,  // bitmap
      spill ? align256(kbase_rows * bh * nb * sizeof(int32_t)) : 0,           // kbase
      spill ? align256(bh * nb * kq * sizeof(int64_t)) : 0,                   // qent
      spill ? align256(bh * ds_qblocks * kq * (size_t)(vsa::BLOCK * vsa::BLOCK) * 2) : 0,  // dS
      nchunks ? align256(bh * nb * (nchunks + 1) * sizeof(int32_t)) : 0,          // bounds
      nchunks ? align256(bh * nb * 2 * (size_t)(vsa::BLOCK * vsa::HEAD_DIM) * sizeof(float))
              : 0,                                                                 // dK/dV
      dq_nchunks ? align256(bh * nb * (dq_nchunks + 1) * sizeof(int32_t)) : 0,     // dq bounds
      dq_nchunks ? align256(bh * nb * (size_t)(vsa::BLOCK * vsa::HEAD_DIM) * sizeof(float))
                 : 0,                                                              // dQ
      align256(bh * nb * vsa::STAT_WORDS * sizeof(uint32_t)),                     // block stats
      align256(bh * vsa::HEAD_SCALE_WORDS * sizeof(int32_t)),                     // head scales
      align256(bh * (size_t)seqlen * vsa::HEAD_DIM * 2),                          // q16
      align256(bh * (size_t)seqlen * vsa::HEAD_DIM * 2),                          // k16
      align256(bh * (size_t)seqlen * vsa::HEAD_DIM * 2),                          // do16
      spill ? 0 : align256(bh * (size_t)seqlen * vsa::HEAD_DIM * 2),              // v16
  };
  size_t off = 0;
  for (int r = 0; r < region; ++r) off += sizes[r];
  return off;
}

size_t vsa_bwd_workspace_bytes(int batch, int heads, int seqlen, int q2k_stride, int dq_mode,
                               int chunk_blocks) {
  return vsa_bwd_workspace_offset(batch, heads, seqlen, q2k_stride, dq_mode, chunk_blocks,
                                  VSA_WS_END);
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
  const size_t items = (size_t)a->batch * a->heads * (size_t)a->num_kv_blocks;
  if (items * (size_t)a->max_q_blocks >= kMaxElems || items * (size_t)a->num_kv_blocks >= kMaxElems)
    return fail(VSA_EINVAL, "vsa_bwd: index metadata too large");
  if (!std::isfinite(a->sm_scale)) return fail(VSA_EINVAL, "vsa_bwd: sm_scale must be finite");
  // the statistics records hold (pp - lse) / (scale_log2 2^(eq + ek)), finite only for a scale
  // not too close to 0
  if (!(std::fabs(scale_log2(a->sm_scale)) >= 0x1p-120f))
    return fail(VSA_EINVAL, "vsa_bwd: |sm_scale * log2(e)| must be at least 2^-120");
  if (!a->q || !a->k || !a->v || !a->o || !a->dout || !a->lse)
    return fail(VSA_EINVAL, "vsa_bwd: null input pointer");
  if (!a->k2q_idx || !a->k2q_num || !a->vbs)
    return fail(VSA_EINVAL, "vsa_bwd: null index pointer");
  if ((a->q2k_idx == nullptr) != (a->q2k_num == nullptr))
    return fail(VSA_EINVAL, "vsa_bwd: give both q2k_idx and q2k_num, or neither");
  if (a->q2k_idx && a->q2k_stride < 1)
    return fail(VSA_EINVAL, "vsa_bwd: q2k_stride must be >= 1 when q2k lists are given");
  if (!a->dq || !a->dk || !a->dv) return fail(VSA_EINVAL, "vsa_bwd: null output pointer");
  if (!a->workspace) return fail(VSA_EINVAL, "vsa_bwd: null workspace");
  if (a->dq_mode != VSA_DQ_RECOMPUTE && a->dq_mode != VSA_DQ_SPILL)
    return fail(VSA_EINVAL, "vsa_bwd: dq_mode must be VSA_DQ_RECOMPUTE or VSA_DQ_SPILL, got " +
                                std::to_string(a->dq_mode));
  if (a->dq_mode == VSA_DQ_SPILL) {
    const long long kq = a->q2k_idx ? a->q2k_stride : a->num_kv_blocks;
    if (a->num_kv_blocks > 65535)
      return fail(VSA_EUNSUPPORTED, "vsa_bwd: VSA_DQ_SPILL supports at most 65535 kv blocks");
    if ((long long)a->num_kv_blocks * kq >= (1LL << 31))
      return fail(VSA_EUNSUPPORTED, "vsa_bwd: VSA_DQ_SPILL needs num_kv_blocks * q2k row width "
                                    "below 2^31");
  }
  const size_t need = vsa_bwd_workspace_bytes(a->batch, a->heads, a->seqlen,
                                              a->q2k_idx ? a->q2k_stride : 0, a->dq_mode,
                                              a->chunk_blocks);
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

}  // extern "C"

// helpers: C++ linkage, internal to this file
namespace {

// Rounds of the kv-major kernel's XCD mapping: the Q and dO tiles of the heads that run at once
// (each head's q window: its q blocks, or one chunk's) should fit half of the 256 MB
// memory-side cache all XCDs share. One round runs one head per XCD (8 heads at once when
// B*H >= 8); R rounds run 8/R heads at once, each shared by R XCDs. Measured on the dK/dV
// kernel: 65536 tokens, 8 heads (256 MiB of Q/dO): 4.73 ms in one round, 4.55 ms in two, 4.67 ms
// in four; 32768 tokens (128 MiB): 2.19, 2.21 and 2.25 ms.
int kv_rounds_of(int bh, int window_q_blocks) {
  const double live = (double)bh * window_q_blocks * (2.0 * vsa::BLOCK * vsa::HEAD_DIM * 2);
  const double budget = 128.0 * 1024 * 1024;
  int r = (int)std::ceil(live / budget);
  return r < 1 ? 1 : (r > 8 ? 8 : r);
}

bool uses_device_order(const vsa_bwd_args* a) {
  return a->num_kv_blocks >= VSA_ORDER_MIN_KV_BLOCKS && a->num_kv_blocks <= VSA_ORDER_MAX_KV_BLOCKS;
}

struct WsView {
  float* lse_delta;
  int32_t* kv_order;
  int32_t* q_order;
  int32_t* q2k_num;
  int32_t* q2k_idx;
  uint32_t* bitmap;
  int32_t* kbase;
  int64_t* qent;
  vsa::f16* ds;
  int32_t* chunk_bounds;
  float* part;
  int32_t* dq_bounds;
  float* dq_part;
  uint32_t* stats;
  int32_t* scales;
  vsa::f16* q16;
  vsa::f16* k16;
  vsa::f16* do16;
  vsa::f16* v16;
};

WsView ws_view(const vsa_bwd_args* a) {
  char* ws = (char*)a->workspace;
  const int kq = a->q2k_idx ? a->q2k_stride : 0;
  auto at = [&](int r) {
    return ws + vsa_bwd_workspace_offset(a->batch, a->heads, a->seqlen, kq, a->dq_mode,
                                         a->chunk_blocks, r);
  };
  return WsView{(float*)at(VSA_WS_LSE_DELTA), (int32_t*)at(VSA_WS_KV_ORDER),
                (int32_t*)at(VSA_WS_Q_ORDER),  (int32_t*)at(VSA_WS_Q2K_NUM),
                (int32_t*)at(VSA_WS_Q2K_IDX),  (uint32_t*)at(VSA_WS_BITMAP),
                (int32_t*)at(VSA_WS_KBASE),    (int64_t*)at(VSA_WS_QENT),
                (vsa::f16*)at(VSA_WS_DS),      (int32_t*)at(VSA_WS_CHUNK_BOUNDS),
                (float*)at(VSA_WS_DKV_PART),   (int32_t*)at(VSA_WS_DQ_BOUNDS),
                (float*)at(VSA_WS_DQ_PART),    (uint32_t*)at(VSA_WS_STATS),
                (int32_t*)at(VSA_WS_SCALES),   (vsa::f16*)at(VSA_WS_Q16),
                (vsa::f16*)at(VSA_WS_K16),     (vsa::f16*)at(VSA_WS_DO16),
                a->dq_mode == VSA_DQ_SPILL ? nullptr : (vsa::f16*)at(VSA_WS_V16)};
}

vsa::BwdParams main_params(const vsa_bwd_args* a, const WsView& ws) {
  vsa::BwdParams m;
  const bool derive = a->q2k_idx == nullptr;
  m.v = (const vsa::bf16*)a->v;
  m.q16 = ws.q16;
  m.k16 = ws.k16;
  m.v16 = ws.v16;
  m.do16 = ws.do16;
  m.scales = ws.scales;
  m.lse = a->lse;
  m.lse_delta = ws.lse_delta;
  m.k2q_idx = a->k2q_idx;
  m.k2q_num = a->k2q_num;
  m.q2k_idx = derive ? ws.q2k_idx : a->q2k_idx;
  m.q2k_num = derive ? ws.q2k_num : a->q2k_num;
  m.vbs = a->vbs;
  m.kv_order = a->order ? a->order : (uses_device_order(a) ? ws.kv_order : nullptr);
  m.q_order = uses_device_order(a) ? ws.q_order : nullptr;
  m.dq = (vsa::bf16*)a->dq;
  m.dk = (vsa::bf16*)a->dk;
  m.dv = (vsa::bf16*)a->dv;
  m.S = a->seqlen;
  m.nb = a->num_kv_blocks;
  m.k2q_stride = a->max_q_blocks;
  m.q2k_stride = derive ? a->num_kv_blocks : a->q2k_stride;
  const bool spill = a->dq_mode == VSA_DQ_SPILL;
  m.kbase = spill ? ws.kbase : nullptr;
  m.qent = spill ? ws.qent : nullptr;
  m.ds = spill ? ws.ds : nullptr;
  m.qent_stride = m.q2k_stride;
  const int cs = spill_chunk_blocks_of(a->num_kv_blocks, a->chunk_blocks, a->dq_mode);
  m.cap = spill ? (cs > 0 ? cs : a->num_kv_blocks) * m.q2k_stride : 0;
  m.total_items = a->batch * a->heads * a->num_kv_blocks;
  m.items_per_xcd = (m.total_items + 7) / 8;
  m.sm_scale = a->sm_scale;
  const int cq = chunk_blocks_of(a->num_kv_blocks, a->chunk_blocks, a->dq_mode);
  m.nchunks = cq > 0 ? (a->num_kv_blocks + cq - 1) / cq : 0;
  m.kv_rounds = kv_rounds_of(a->batch * a->heads, cq > 0 ? cq : a->num_kv_blocks);
  m.chunk = 0;
  m.chunk_bounds = m.nchunks ? ws.chunk_bounds : nullptr;
  m.part = m.nchunks ? ws.part : nullptr;
  return m;
}

int run_stage(const vsa_bwd_args* a, int stage, hipStream_t s) {
  const int BH = a->batch * a->heads;
  const int nb = a->num_kv_blocks;
  const WsView ws = ws_view(a);
  switch (stage) {
    case VSA_BWD_PREPROCESS: {
      vsa::BwdPreParams pre;
      pre.q = (const vsa::bf16*)a->q;
      pre.k = (const vsa::bf16*)a->k;
      pre.v = (const vsa::bf16*)a->v;
      pre.o = (const vsa::bf16*)a->o;
      pre.dout = (const vsa::bf16*)a->dout;
      pre.k2q_num = a->k2q_num;
      pre.lse = a->lse;
      pre.lse_delta = ws.lse_delta;
      pre.stats = ws.stats;
      pre.scales = ws.scales;
      pre.q16 = ws.q16;
      pre.k16 = ws.k16;
      pre.do16 = ws.do16;
      pre.v16 = ws.v16;
      pre.dk = (vsa::bf16*)a->dk;
      pre.dv = (vsa::bf16*)a->dv;
      pre.BH = BH;
      pre.S = a->seqlen;
      pre.nb = nb;
      pre.scale_log2 = scale_log2(a->sm_scale);
      vsa::launch_bwd_pre(pre, s);
      return launch_status("vsa_bwd preprocess");
    }
    case VSA_BWD_INDEX: {
      const bool derive = a->q2k_idx == nullptr;
      if (derive) {
        // k2q rows list q blocks per kv block; inverting them lists kv blocks per q block
        vsa::launch_invert(a->k2q_idx, a->k2q_num, BH, nb, a->max_q_blocks, nb, ws.q2k_idx,
                           ws.q2k_num, ws.bitmap, s);
        const int r = launch_status("vsa_bwd q2k derivation");
        if (r != VSA_OK) return r;
      }
      // chunk bounds of the kv-major kernel's q-range chunks (a chunked spill numbers its tiles by
      // them)
      const int cb = chunk_blocks_of(nb, a->chunk_blocks, a->dq_mode);
      const int nchunks = cb > 0 ? (nb + cb - 1) / cb : 0;
      if (cb > 0) {
        vsa::launch_chunk_bounds(a->k2q_idx, a->k2q_num, a->max_q_blocks, BH * nb, nchunks, cb,
                                 ws.chunk_bounds, s);
        const int r = launch_status("vsa_bwd chunk bounds");
        if (r != VSA_OK) return r;
      }
      const int cs = spill_chunk_blocks_of(nb, a->chunk_blocks, a->dq_mode);
      // the work orders and the dS slot bases: independent per-head tasks, one launch
      vsa::IndexTasks tasks{};
      if (uses_device_order(a)) {
        // (with q-range chunks the DKDV stage orders the items per chunk instead)
        if (!a->order && cb == 0)
          tasks.task[tasks.count++] = {vsa::IndexTask::ORDER, a->k2q_num, ws.kv_order};
        tasks.task[tasks.count++] = {vsa::IndexTask::ORDER, derive ? ws.q2k_num : a->q2k_num,
                                     ws.q_order};
      }
      if (a->dq_mode == VSA_DQ_SPILL && cs == 0)
        tasks.task[tasks.count++] = {vsa::IndexTask::KBASE, a->k2q_num, ws.kbase};
      if (tasks.count > 0) {
        vsa::launch_index_tasks(tasks, BH, nb, VSA_ORDER_BIN_WIDTH, a->max_q_blocks, s);
        const int r = launch_status("vsa_bwd work orders / dS slot bases");
        if (r != VSA_OK) return r;
      }
      if (cs > 0) {
        vsa::launch_chunk_kbase(ws.chunk_bounds, a->k2q_num, a->max_q_blocks, BH, nb, nchunks,
                                ws.kbase, s);
        const int r = launch_status("vsa_bwd per-chunk dS slot bases");
        if (r != VSA_OK) return r;
      }
      if (a->dq_mode == VSA_DQ_SPILL) {
        const vsa::BwdParams m = main_params(a, ws);
        vsa::launch_spill_qent(m.q2k_idx, m.q2k_num, m.q2k_stride, a->k2q_idx, a->k2q_num,
                               a->max_q_blocks, ws.kbase, a->vbs, BH, nb, m.cap,
                               cs > 0 ? ws.chunk_bounds : nullptr, nchunks, cs, ws.qent, s);
        const int r = launch_status("vsa_bwd dS slot table");
        if (r != VSA_OK) return r;
      }
      const int cbq = dq_chunk_blocks_of(nb, a->chunk_blocks, a->dq_mode);
      if (cbq > 0) {
        const vsa::BwdParams m = main_params(a, ws);
        vsa::launch_chunk_bounds(m.q2k_idx, m.q2k_num, m.q2k_stride, BH * nb,
                                 (nb + cbq - 1) / cbq, cbq, ws.dq_bounds, s);
        const int r = launch_status("vsa_bwd dq chunk bounds");
        if (r != VSA_OK) return r;
      }
      return VSA_OK;
    }
    case VSA_BWD_DKDV: {
      vsa::BwdParams m = main_params(a, ws);
      // the kv-major launch covers 8 XCDs x kv_rounds slices of ceil(items / (8 rounds)) ids
      const int per_slice = (m.total_items + 8 * m.kv_rounds - 1) / (8 * m.kv_rounds);
      m.items_per_xcd = m.kv_rounds * per_slice;
      const int launches = m.nchunks > 0 ? m.nchunks : 1;
      // a chunked spill: each kv-major launch writes its chunk's tiles from slot 0 and the q-major
      // kernel turns them into dq for the chunk's q blocks before the next launch reuses them
      const int cs = spill_chunk_blocks_of(nb, a->chunk_blocks, a->dq_mode);
      // with chunks the library's work order bins the items by the part of their list inside
      // each chunk, so the items that run together walk parts of equal length
      const bool chunk_orders = m.nchunks > 0 && !a->order && uses_device_order(a);
      for (int c = 0; c < launches; ++c) {
        m.chunk = c;
        if (chunk_orders) {
          vsa::launch_chunk_order(ws.chunk_bounds, a->k2q_num, a->max_q_blocks, BH, nb, m.nchunks,
                                  c, VSA_ORDER_BIN_WIDTH, ws.kv_order, s);
          const int r = launch_status("vsa_bwd chunk work order");
          if (r != VSA_OK) return r;
        }
        if (cs > 0) {
          m.kbase = ws.kbase + (size_t)c * BH * nb;
          m.ds_chunk_local = 1;
        }
        vsa::launch_bwd_dkdv(m, s);
        int r = launch_status("vsa_bwd dk/dv kernel");
        if (r != VSA_OK) return r;
        if (cs > 0) {
          vsa::BwdParams q = main_params(a, ws);
          q.q_first = c * cs;
          q.q_count = nb - q.q_first < cs ? nb - q.q_first : cs;
          q.items_per_xcd = (BH * q.q_count + 7) / 8;
          vsa::launch_bwd_dq_spill(q, s);
          r = launch_status("vsa_bwd dq kernel");
          if (r != VSA_OK) return r;
        }
      }
      return VSA_OK;
    }
    case VSA_BWD_DQ: {
      vsa::BwdParams m = main_params(a, ws);
      if (spill_chunk_blocks_of(nb, a->chunk_blocks, a->dq_mode) > 0)
        return VSA_OK;  // a chunked spill computed dq in the DKDV stage
      if (a->dq_mode == VSA_DQ_SPILL) {
        vsa::launch_bwd_dq_spill(m, s);
        return launch_status("vsa_bwd dq kernel");
      }
      const int cbq = dq_chunk_blocks_of(nb, a->chunk_blocks, a->dq_mode);
      m.nchunks = cbq > 0 ? (nb + cbq - 1) / cbq : 0;
      m.chunk_bounds = m.nchunks ? ws.dq_bounds : nullptr;
      m.part = m.nchunks ? ws.dq_part : nullptr;
      const int launches = m.nchunks > 0 ? m.nchunks : 1;
      for (int c = 0; c < launches; ++c) {
        m.chunk = c;
        vsa::launch_bwd_dq(m, s);
        const int r = launch_status("vsa_bwd dq kernel");
        if (r != VSA_OK) return r;
      }
      return VSA_OK;
    }
    default:
      return fail(VSA_EINVAL, "vsa_bwd_stage: unknown stage " + std::to_string(stage));
  }
}

}  // namespace

extern "C" {

int vsa_bwd_stage(const vsa_bwd_args* a, int stage, void* stream) {
  const int st = vsa_bwd_check(a);
  if (st != VSA_OK) return st;
  if (stage < VSA_BWD_PREPROCESS || stage > VSA_BWD_DQ)
    return fail(VSA_EINVAL, "vsa_bwd_stage: unknown stage " + std::to_string(stage));
  return run_stage(a, stage, (hipStream_t)stream);
}

int vsa_bwd(const vsa_bwd_args* a, void* stream) {
  const int st = vsa_bwd_check(a);
  if (st != VSA_OK) return st;
  for (int stage = VSA_BWD_PREPROCESS; stage <= VSA_BWD_DQ; ++stage) {
    const int r = run_stage(a, stage, (hipStream_t)stream);
    if (r != VSA_OK) return r;
  }
  return VSA_OK;
}

}  // extern "C"

// ------------------------------------------------------------------------------------------------
// backward without a caller workspace
// ------------------------------------------------------------------------------------------------

// The workspace of vsa_bwd_noalloc: device memory of this code object, one copy per GPU that
// loads the library, held until the process ends. Host code never uses this name as an address
// (on the host it is only a stand-in); the device address comes from hipGetSymbolAddress, per
// device, below.
static __device__ __align__(256) char scratch[VSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's device address on the current device, resolved on the first call there.
int scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(VSA_ELAUNCH, std::string("vsa_bwd_noalloc: hipGetDevice: ") +
                                                    hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(VSA_EUNSUPPORTED, "vsa_bwd_noalloc: device id " + std::to_string(dev) +
                                      " above the supported " + std::to_string(kMaxDevices - 1));
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(VSA_ELAUNCH, std::string("vsa_bwd_noalloc: hipGetSymbolAddress: ") +
                                   hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return VSA_OK;
}

}  // namespace

extern "C" {

int vsa_bwd_noalloc(const vsa_bwd_args* a, void* stream) {
  if (!a) return fail(VSA_EINVAL, "vsa_bwd_noalloc: null argument struct");
  const size_t need = vsa_bwd_workspace_bytes(a->batch, a->heads, a->seqlen,
                                              a->q2k_idx ? a->q2k_stride : 0, a->dq_mode,
                                              a->chunk_blocks);
  if (need > (size_t)VSA_NOALLOC_SCRATCH_BYTES)
    return fail(VSA_EUNSUPPORTED,
                "vsa_bwd_noalloc: this call needs " + std::to_string(need) +
                    " bytes of workspace, above the static scratch of " +
                    std::to_string((size_t)VSA_NOALLOC_SCRATCH_BYTES) +
                    " bytes; use vsa_bwd with a workspace");
  void* ws = nullptr;
  const int r = scratch_of_current_device(&ws);
  if (r != VSA_OK) return r;
  vsa_bwd_args b = *a;
  b.workspace = ws;
  b.workspace_bytes = VSA_NOALLOC_SCRATCH_BYTES;
  return vsa_bwd(&b, stream);
}

}  // extern "C"
