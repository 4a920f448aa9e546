/* vsa.h -- C ABI of the MI355X (gfx950) 64-token block-sparse attention library, libvsa.so.
 *
 * The operation is VSA-style block-sparse attention as the FastVideo pages describe it
 * (the sm_100a backward commit message; the backward launch header's argument struct and launch
 * chain; the backward torch binding; the Python backward module; the backward test page's
 * masked-dense reference and invert helper; the forward module docstring): every 64-token q block
 * attends to a chosen list of 64-token kv blocks, keys at or past variable_block_sizes[kv block]
 * are masked, the softmax scale is sm_scale, head_dim is 128, activations are bf16 with fp32
 * accumulation.
 *
 * Conventions for every entry point:
 *   - Activations (q, k, v, o, dout, dq, dk, dv) are bf16, contiguous [B, H, S, 128] (BHSD),
 *     S = 64 * num_kv_blocks. lse and Delta are fp32 [B, H, S]. Index metadata is int32,
 *     contiguous.
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library allocates nothing,
 *     frees nothing and never synchronizes: it validates on the host (reading no tensor contents),
 *     enqueues kernels on `stream` (a hipStream_t; NULL = the null stream) and returns. Inputs must
 *     stay alive and unmodified until the enqueued work has run.
 *   - Outputs are fully written (including exact zeros), so they may be uninitialised memory.
 *   - Return value: VSA_OK, or a vsa_status code; vsa_status_string() names it and
 *     vsa_last_error() gives the detailed message of the calling thread's last failure. On a
 *     validation failure nothing is enqueued.
 *   - Index values out of range (a kv id outside [0, num_kv_blocks), a count above the row
 *     width) violate the caller contract; the kernels skip such entries rather than read out of
 *     bounds, and the results are then unspecified. Duplicate kv ids in one q2k row count once.
 */
#ifndef VSA_H
#define VSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VSA_OK = 0,
  VSA_EINVAL = 1,        /* a null pointer, a size out of range, a workspace too small */
  VSA_EUNSUPPORTED = 2,  /* a shape this library does not implement (head_dim != 128, ...) */
  VSA_ELAUNCH = 3        /* a HIP launch failed; vsa_last_error() holds the HIP message */
} vsa_status;

/* Name of a status code (static string). */
const char* vsa_status_string(int status);

/* Detailed message of the calling thread's last failing call ("" if none). */
const char* vsa_last_error(void);

/* ------------------------------------------------------------------------------------------ */
/* invert_indices (FastVideo backward Python module: the k2q inversion before the backward;
 * backward test page, invert_indices_torch).
 *
 * q2k_idx [B, H, nq, topk]: row (b, h, qb) lists kv block ids; only the first q2k_num[b, h, qb]
 * entries count. Output k2q_idx [B, H, nkv, nq]: row (b, h, kb) lists, ascending, every q block
 * that selects kb; entries past k2q_num[b, h, kb] are 0. k2q_num [B, H, nkv]. The result is
 * bit-exact and deterministic. Workspace: vsa_invert_workspace_bytes() bytes of device memory
 * (a bitmap), contents on entry irrelevant. */
size_t vsa_invert_workspace_bytes(int batch, int heads, int nq, int nkv);
int vsa_invert_indices(const int32_t* q2k_idx, const int32_t* q2k_num, int batch, int heads,
                       int nq, int topk, int nkv, int32_t* k2q_idx, int32_t* k2q_num,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------ */
/* Forward (FastVideo sm_100a forward module docstring): o = softmax(q k^T * sm_scale over the
 * selected, unmasked keys) v, rounded to bf16; lse = max(q k^T * sm_scale * log2(e)) + log2(l)
 * ("M form", fp32 [B, H, S]). A q row with no valid key gets o = 0 and lse = -inf. */
typedef struct {
  const void* q;          /* bf16 [B, H, S, 128] */
  const void* k;          /* bf16 [B, H, S, 128] */
  const void* v;          /* bf16 [B, H, S, 128] */
  const int32_t* q2k_idx; /* [B, H, num_kv_blocks, q2k_stride] */
  const int32_t* q2k_num; /* [B, H, num_kv_blocks] */
  const int32_t* vbs;     /* variable_block_sizes [num_kv_blocks], each in [0, 64] */
  void* o;                /* bf16 [B, H, S, 128], output */
  float* lse;             /* fp32 [B, H, S], output */
  int batch, heads, seqlen, head_dim, num_kv_blocks, q2k_stride;
  float sm_scale;
} vsa_fwd_args;

int vsa_fwd_check(const vsa_fwd_args* a);
int vsa_fwd(const vsa_fwd_args* a, void* stream);

/* ------------------------------------------------------------------------------------------ */
/* Backward (FastVideo backward launch header: argument struct, workspace helpers, support
 * predicate and the preprocess -> order -> main -> postprocess chain; backward torch binding).
 *
 * Gradients of L = sum(o * dout): dq and dk carry sm_scale, dv does not. kv blocks that no q
 * block selects get exact-zero dk/dv rows, and so do kv rows at or past vbs. lse is the forward's
 * M-form log-sum-exp; o is the forward's bf16 output (Delta = rowsum(o * dout) uses it).
 *
 * Work order: `order` (optional, [B*H*num_kv_blocks] int32 item ids (b*H + h)*nb + kv, a
 * permutation) fixes the order in which items are launched. NULL lets the library choose: the
 * identity below VSA_ORDER_MIN_KV_BLOCKS kv blocks per sequence, else the length-binned order
 * (vsa_bwd_order with bin width 8) computed into the workspace. Any order gives the same dk/dv
 * bits; dq differs only by fp32 summation order.
 *
 * Workspace (device, vsa_bwd_workspace_bytes() bytes, contents on entry irrelevant):
 *   [0, dqacc)        fp32 dQ accumulator [B, H, S, 128]
 *   [dqacc, +delta)   fp32 Delta [B, H, S]   (left holding Delta after the call)
 *   [.., +order)      int32 work order [B*H*nb] (when the library computes it)
 * each region starting at a 256-byte boundary; vsa_bwd_workspace_layout() gives the offsets. */
#define VSA_ORDER_MIN_KV_BLOCKS 1024
#define VSA_ORDER_MAX_KV_BLOCKS 16384

typedef struct {
  const void* q;          /* bf16 [B, H, S, 128] */
  const void* k;
  const void* v;
  const void* o;          /* forward output, bf16 */
  const void* dout;       /* gradient of o, bf16 */
  const float* lse;       /* fp32 [B, H, S], M form */
  const int32_t* k2q_idx; /* [B, H, num_kv_blocks, max_q_blocks] ascending q block ids */
  const int32_t* k2q_num; /* [B, H, num_kv_blocks], 0 allowed */
  const int32_t* vbs;     /* [num_kv_blocks] valid kv tokens per block, in [0, 64] */
  const int32_t* order;   /* optional work order, see above; NULL = library's choice */
  void* dq;               /* bf16 outputs [B, H, S, 128] */
  void* dk;
  void* dv;
  void* workspace;
  size_t workspace_bytes;
  int batch, heads, seqlen, head_dim, num_kv_blocks, max_q_blocks;
  float sm_scale;
} vsa_bwd_args;

size_t vsa_bwd_workspace_bytes(int batch, int heads, int seqlen);
/* Byte offsets of the dQ accumulator, Delta and order regions inside the workspace. */
void vsa_bwd_workspace_layout(int batch, int heads, int seqlen, size_t* dqacc_off,
                              size_t* delta_off, size_t* order_off);
/* Host-only validation of a backward call; reads no device memory. */
int vsa_bwd_check(const vsa_bwd_args* a);
int vsa_bwd(const vsa_bwd_args* a, void* stream);

/* The backward's stages one at a time, for callers that time or interleave them. Each call
 * validates like vsa_bwd. Run on one stream in the order PREPROCESS, ORDER, MAIN, POSTPROCESS,
 * they enqueue exactly the kernels vsa_bwd enqueues and produce the same results. ORDER is a no-op
 * when a->order is given or num_kv_blocks is outside [VSA_ORDER_MIN_KV_BLOCKS,
 * VSA_ORDER_MAX_KV_BLOCKS]; MAIN then uses a->order, the workspace order, or the identity, as
 * vsa_bwd does. */
typedef enum {
  VSA_BWD_PREPROCESS = 0,  /* Delta, dQ accumulator zeroing, zero dk/dv rows of empty kv blocks */
  VSA_BWD_ORDER = 1,       /* length-binned work order into the workspace */
  VSA_BWD_MAIN = 2,        /* dk, dv and the dQ partials */
  VSA_BWD_POSTPROCESS = 3  /* dq = bf16(sm_scale * dQ accumulator) */
} vsa_bwd_stage_id;
int vsa_bwd_stage(const vsa_bwd_args* a, int stage, void* stream);

/* Work order alone: for each (b, h), its kv items ranked by bin = k2q_num / bin_width (larger bin
 * first, then ascending kv id); writes item ids (b*H + h)*nb + kv to order [B*H*nb]. nb may be at
 * most VSA_ORDER_MAX_KV_BLOCKS; bin_width >= 1. */
int vsa_bwd_order(const int32_t* k2q_num, int batch, int heads, int num_kv_blocks, int bin_width,
                  int32_t* order, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VSA_H */
