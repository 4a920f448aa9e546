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
 * ("M form", fp32 [B, H, S]). A q row with no valid key gets o = 0 and lse = -inf.
 *
 * kv-range chunks (kv_chunk_blocks; 0 = the library's choice): with R = kv_chunk_blocks (> 0), or
 * R = VSA_FWD_CHUNK_KV_BLOCKS from VSA_FWD_CHUNK_MIN_KV_BLOCKS kv blocks on when it is 0, the forward
 * runs as C = ceil(nb / R) launches; launch c takes, of every q2k list, the positions from the
 * first entry >= c*R to the first entry >= (c+1)*R (the kv blocks in [c*R, (c+1)*R) when the
 * list is ascending) and carries each wave's running O, max and sum to the next launch in fp32
 * in the workspace, exactly: the results are bitwise those of one launch. The workgroups running
 * together on one XCD then share a window of R kv blocks, so their K/V tiles stay in its L2.
 * Any list order is correct; ascending lists give the locality. With num_kv_blocks in
 * [VSA_ORDER_MIN_KV_BLOCKS, VSA_ORDER_MAX_KV_BLOCKS] each launch also orders its items by the
 * length of their list's part in its chunk (length bins of VSA_ORDER_BIN_WIDTH), so the items
 * running together walk parts of equal length; the order never changes the results.
 * kv_chunk_blocks < 0: never chunk. The forward chunks from fewer kv blocks than the backward:
 * at 65536 tokens (1024 kv blocks, top-k 128) two ordered chunks of 512 took it from 3.21 to
 * 2.69 ms, while at 32768 tokens chunks of 256 were slower (1.285 against 1.215 ms).
 *
 * The P v product runs on fp16 operands (same MFMA rate as bf16, 8x finer rounding of P): a
 * pre-pass writes an fp16 copy of v into the workspace, each head scaled by the power of two that
 * brings its largest |v| into [2^14, 2^15), so every bf16 value of v with |v| >= 2^-28 * max|v|
 * of its head is copied exactly; o is scaled back exactly. Workspace (vsa_fwd_workspace_bytes,
 * 256-byte aligned regions): uint32 [B*H] per-head and [B*H*nb] per-tile max |v| bits, fp16
 * [B, H, S, 128] scaled copy of v, then with chunks int32 [B*H*nb, C+1] chunk bounds, fp32
 * [B*H*nb, 4, 66, 64] per-wave state and (when the items are ordered per chunk) the int32
 * [B*H*nb] work order. */
#define VSA_FWD_CHUNK_KV_BLOCKS 512
#define VSA_FWD_CHUNK_MIN_KV_BLOCKS 1024
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
  float sm_scale;         /* finite; negative and zero are allowed (zero acts as 2^-126) */
  void* workspace;        /* see above; at least vsa_fwd_workspace_bytes */
  size_t workspace_bytes;
  int kv_chunk_blocks;    /* kv-range chunks, see above; 0 = default */
} vsa_fwd_args;

/* Bytes of forward workspace for these sizes and kv_chunk_blocks (0 for an invalid shape). */
size_t vsa_fwd_workspace_bytes(int batch, int heads, int seqlen, int kv_chunk_blocks);
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
 * Arithmetic: every GEMM runs on fp16 operands with fp32 accumulation (v_mfma_f32_32x32x16_f16,
 * the rate of the bf16 form). The preprocess scales each head's q and k by powers of two into
 * [2^14, 2^15) and v and dout into [1, 2) (exact copies of the bf16 values down to 2^-28 times
 * the head's largest one) and P, dS by powers of two chosen so that dS stays within fp16's range
 * (a bound from the row norms of dout and v and the largest |Delta|); P and dS then carry 11
 * significant bits instead of bf16's 8, and the epilogues take the scales back out exactly. A head
 * whose scores q.k * sm_scale * log2 e are all far below 2^-100 (or above 2^100) in size gives up
 * fp16 precision in its q, k copies.
 *
 * The main step runs as two kernels without atomics: a kv-major one (one work item per
 * (b, h, kv block), walking the k2q list) for dk and dv, and a q-major one (one item per
 * (b, h, q block), walking the q2k list) for dq. All three outputs are bitwise reproducible run
 * to run, whatever the work order. The q-major kernel gets dS in one of two ways (dq_mode):
 *   VSA_DQ_RECOMPUTE  it recomputes S and dP for each pair from Q, K, V, dO, lse and Delta
 *                     (three GEMMs per pair; an fp16 copy of v in the workspace);
 *   VSA_DQ_SPILL      the kv-major kernel writes every pair's dS (fp16, scaled, the same values
 *                     its dK GEMM uses) into the workspace and dq is one block-sparse GEMM dS K per
 *                     pair, reading 8 KiB of dS per pair from HBM. This needs 8 KiB of workspace
 *                     per possible pair (B*H*nb*q2k_stride of them, nb*nb when q2k is derived)
 *                     and k2q rows in ascending order (as vsa_invert_indices writes them); it
 *                     supports num_kv_blocks <= 65535. When the kv-major kernel runs in chunks
 *                     of R q blocks (below), the spill is chunked too: it holds the tiles of one
 *                     chunk (B*H*R*q2k_stride possible pairs), and the q-major kernel runs after
 *                     each kv-major launch, over that chunk's q blocks.
 *
 * q2k lists (optional): the forward's q2k_idx [B, H, num_kv_blocks, q2k_stride] / q2k_num, which
 * must describe the same selection as k2q (each pair once). NULL: the library derives them from
 * k2q into the workspace (the inversion kernel of vsa_invert_indices).
 *
 * Work order: `order` (optional, [B*H*num_kv_blocks] int32 item ids (b*H + h)*nb + kv, a
 * permutation) fixes the launch order of the kv-major items. NULL lets the library choose: the
 * identity below VSA_ORDER_MIN_KV_BLOCKS kv blocks per sequence, else the length-binned order
 * (vsa_bwd_order, bin width VSA_ORDER_BIN_WIDTH) computed into the workspace; the q-major items
 * get the same treatment from the q2k counts. The pages sort from 1024 kv blocks with bin
 * parameter 8 (the launch header's order kernel). Here the order also keeps the items that run
 * together on one XCD at equal list lengths, so their ascending walks over Q/dO stay in step and
 * share that XCD's L2; on MI355X that pays from a few hundred kv blocks on, and a narrower bin
 * keeps the walks closer. When the kv-major kernel runs in chunks (below), the library orders
 * its items again before each chunk's launch, by the lengths of their lists' parts inside that
 * chunk (a caller's order is used as given for every chunk). The order never changes the
 * results, which are bitwise identical for any order.
 *
 * Workspace (device, vsa_bwd_workspace_bytes() bytes, contents on entry irrelevant), regions in
 * this order, each at a 256-byte boundary (vsa_bwd_workspace_offset() gives the offsets); a
 * region the call does not use has size 0. K' below is q2k_stride, or nb when q2k is derived.
 *   VSA_WS_LSE_DELTA fp32 [B, H, nb, 2, 64]: per q block, (pp - lse) / c of its 64 rows (fp32
 *                    subtraction, then division), then -Delta * 2^-(eo + ev) of its 64 rows,
 *                    with the head's pp, c, eo, ev from VSA_WS_SCALES; left holding them after
 *                    the call
 *   VSA_WS_KV_ORDER  int32 [B*H*nb] kv-major work order (when the library computes it; with
 *                    q-range chunks the DKDV stage rewrites it before each chunk's launch, by
 *                    the lengths of the lists' parts in that chunk)
 *   VSA_WS_Q_ORDER   int32 [B*H*nb] q-major work order (when the library computes it)
 * only when the q2k lists are derived (q2k_stride argument 0):
 *   VSA_WS_Q2K_NUM   int32 [B, H, nb]
 *   VSA_WS_Q2K_IDX   int32 [B, H, nb, nb]
 *   VSA_WS_BITMAP    the inversion's bitmap
 * only in VSA_DQ_SPILL mode:
 *   VSA_WS_KBASE     int32 [B, H, nb]: per kv block, the first dS slot of its head's pairs
 *                    (exclusive prefix sum of k2q_num inside the head); with a chunked spill
 *                    [C, B, H, nb], the same over each chunk's pairs
 *   VSA_WS_QENT      int64 [B, H, nb, K']: per q2k entry, its dS slot | kv block << 32 |
 *                    vbs[kv block] << 48
 *   VSA_WS_DS        fp16 [B, H, nb*K', 64, 64]: the dS tiles (dS * 2^es), slot-major; with a
 *                    chunked spill [B, H, R*K', 64, 64], one chunk's tiles
 * only when the main kernels run in chunks (below), with C chunks:
 *   VSA_WS_CHUNK_BOUNDS int32 [B*H*nb, C+1]: per kv item, the position in its k2q list of the
 *                    first q block of each chunk (the last entry is the list length)
 *   VSA_WS_DKV_PART  fp32 [B*H*nb, 2, 64, 128]: per kv item, dV then dK (unscaled) summed over
 *                    the chunks so far
 *   VSA_WS_DQ_BOUNDS int32 [B*H*nb, C+1]: per q item, the same for its q2k list and kv blocks
 *                    (VSA_DQ_RECOMPUTE mode with chunk_blocks > 0)
 *   VSA_WS_DQ_PART   fp32 [B*H*nb, 64, 128]: per q item, dQ (unscaled) summed over the chunks so
 *                    far (VSA_DQ_RECOMPUTE mode with chunk_blocks > 0)
 * always (the partial sums above are in the scaled units these define):
 *   VSA_WS_STATS     uint32 [B, H, nb, 8]: per 64-row block, fp32 bit patterns of max |q|, max |k|,
 *                    max |v|, max |dout|, max row |v|^2, max row |dout|^2, max |Delta|, 0
 *   VSA_WS_SCALES    int32 [B, H, 8]: per head eq, ek, ev, eo, pp, es = pp - eo - ev, c (fp32 bits)
 *                    = fp32(sm_scale * log2 e) * 2^(eq + ek), 0. The fp16 operands are
 *                    q * 2^-eq, k * 2^-ek, v * 2^-ev, dout * 2^-eo, P * 2^pp and dS * 2^es
 *   VSA_WS_Q16       fp16 [B, H, S, 128]: q * 2^-eq
 *   VSA_WS_K16       fp16 [B, H, S, 128]: k * 2^-ek
 *   VSA_WS_DO16      fp16 [B, H, S, 128]: dout * 2^-eo
 *   VSA_WS_V16       fp16 [B, H, S, 128]: v * 2^-ev (VSA_DQ_RECOMPUTE mode only)
 *
 * Chunks (chunk_blocks argument; 0 = the library's choice): with R = chunk_blocks (> 0) each
 * main kernel runs as C = ceil(nb / R) launches; with 0, the kv-major kernel alone does, with
 * R = VSA_CHUNK_BLOCKS (VSA_SPILL_CHUNK_BLOCKS in VSA_DQ_SPILL mode), from VSA_CHUNK_MIN_KV_BLOCKS
 * kv blocks per sequence on (at 524288 tokens its chunks saved 7-12 %, while the recomputing
 * q-major kernel gained at most 3 %). Launch c of the kv-major kernel takes, of every
 * k2q list, the q blocks in [c*R, (c+1)*R); launch c of the recomputing q-major kernel takes, of
 * every q2k list, the positions from the first entry >= c*R to the first entry >= (c+1)*R (the kv
 * blocks in [c*R, (c+1)*R) for an ascending list; any order is correct). Each carries its
 * partial sums to the next launch in fp32 in the workspace. The items running together on one
 * XCD then walk a window of R blocks at a time, so the tiles they share stay in its L2; without
 * chunks, ascending walks of thousands of entries drift apart and almost every Q/dO (K/V) tile
 * comes from HBM (the pages' long-sequence cache-locality mode serves the same purpose).
 * chunk_blocks < 0: never chunk. Chunking changes only the fp32 summation order of the chunked
 * sums. In VSA_DQ_SPILL mode the chunks also bound the spill: the dS-reading q-major kernel runs
 * once per chunk, over that chunk's q blocks, right after the kv-major launch that wrote their
 * tiles; its results are bitwise those of the unchunked spill. At 524288 tokens with top-k 2048
 * (B*H = 8) the chunked spill with R = 512 holds 64 GiB of tiles and took the backward from
 * 1139 ms (recompute) to 978 ms. */
#define VSA_CHUNK_MIN_KV_BLOCKS 4096
#define VSA_CHUNK_BLOCKS 1024
#define VSA_SPILL_CHUNK_BLOCKS 512
#define VSA_ORDER_MIN_KV_BLOCKS 64
#define VSA_ORDER_BIN_WIDTH 4
#define VSA_ORDER_MAX_KV_BLOCKS 16384

typedef enum {
  VSA_WS_LSE_DELTA = 0,
  VSA_WS_KV_ORDER = 1,
  VSA_WS_Q_ORDER = 2,
  VSA_WS_Q2K_NUM = 3,
  VSA_WS_Q2K_IDX = 4,
  VSA_WS_BITMAP = 5,
  VSA_WS_KBASE = 6,
  VSA_WS_QENT = 7,
  VSA_WS_DS = 8,
  VSA_WS_CHUNK_BOUNDS = 9,
  VSA_WS_DKV_PART = 10,
  VSA_WS_DQ_BOUNDS = 11,
  VSA_WS_DQ_PART = 12,
  VSA_WS_STATS = 13,
  VSA_WS_SCALES = 14,
  VSA_WS_Q16 = 15,
  VSA_WS_K16 = 16,
  VSA_WS_DO16 = 17,
  VSA_WS_V16 = 18,
  VSA_WS_END = 19
} vsa_bwd_ws_region;

typedef enum { VSA_DQ_RECOMPUTE = 0, VSA_DQ_SPILL = 1 } vsa_dq_mode;

typedef struct {
  const void* q;          /* bf16 [B, H, S, 128] */
  const void* k;
  const void* v;
  const void* o;          /* forward output, bf16 */
  const void* dout;       /* gradient of o, bf16 */
  const float* lse;       /* fp32 [B, H, S], M form */
  const int32_t* k2q_idx; /* [B, H, num_kv_blocks, max_q_blocks] ascending q block ids */
  const int32_t* k2q_num; /* [B, H, num_kv_blocks], 0 allowed */
  const int32_t* q2k_idx; /* optional [B, H, num_kv_blocks, q2k_stride] kv block ids */
  const int32_t* q2k_num; /* optional [B, H, num_kv_blocks] */
  const int32_t* vbs;     /* [num_kv_blocks] valid kv tokens per block, in [0, 64] */
  const int32_t* order;   /* optional kv-major work order, see above; NULL = library's choice */
  void* dq;               /* bf16 outputs [B, H, S, 128] */
  void* dk;
  void* dv;
  void* workspace;
  size_t workspace_bytes;
  int batch, heads, seqlen, head_dim, num_kv_blocks, max_q_blocks, q2k_stride;
  float sm_scale;         /* finite, |sm_scale * log2 e| >= 2^-120 (the records divide lse by it) */
  int dq_mode;            /* vsa_dq_mode */
  int chunk_blocks;       /* blocks per chunk of the main kernels, see above; 0 = default */
} vsa_bwd_args;

/* Bytes of workspace for a backward call. q2k_stride: the row width of the q2k lists the call
 * passes, or 0 when q2k_idx/q2k_num are NULL (derived); dq_mode: a vsa_dq_mode; chunk_blocks:
 * as in vsa_bwd_args. 0 for an invalid shape. */
size_t vsa_bwd_workspace_bytes(int batch, int heads, int seqlen, int q2k_stride, int dq_mode,
                               int chunk_blocks);
/* Byte offset of a workspace region (vsa_bwd_ws_region) for the same arguments; VSA_WS_END gives
 * the total. */
size_t vsa_bwd_workspace_offset(int batch, int heads, int seqlen, int q2k_stride, int dq_mode,
                                int chunk_blocks, int region);
/* Host-only validation of a backward call; reads no device memory. */
int vsa_bwd_check(const vsa_bwd_args* a);
int vsa_bwd(const vsa_bwd_args* a, void* stream);

/* The backward's stages one at a time, for callers that time or interleave them. Each call
 * validates like vsa_bwd. Run on one stream in the order PREPROCESS, INDEX, DKDV, DQ, they
 * enqueue exactly the kernels vsa_bwd enqueues and produce the same results. INDEX derives the
 * q2k lists when they are not given, computes the work orders when num_kv_blocks is in
 * [VSA_ORDER_MIN_KV_BLOCKS, VSA_ORDER_MAX_KV_BLOCKS] (with q-range chunks, DKDV orders the
 * kv-major items per chunk instead), builds the dS slot tables in
 * VSA_DQ_SPILL mode and the chunk bounds when the kv-major kernel runs in q-range chunks;
 * otherwise it enqueues nothing. In VSA_DQ_RECOMPUTE mode DKDV and DQ only read
 * what PREPROCESS and INDEX wrote and may run in either order; in VSA_DQ_SPILL mode DQ reads the
 * dS tiles DKDV writes and must follow it, and with a chunked spill DKDV runs the q-major launches
 * too (each after the kv-major launch of its chunk) and DQ enqueues nothing. */
typedef enum {
  VSA_BWD_PREPROCESS = 0,  /* operand scales and fp16 copies, Delta, the records; zero dk/dv
                              rows of kv blocks with an empty k2q list */
  VSA_BWD_INDEX = 1,       /* q2k derivation (if needed), the length-binned work orders, in
                              VSA_DQ_SPILL mode the dS slot tables, with q-range chunks the
                              chunk bounds */
  VSA_BWD_DKDV = 2,        /* kv-major kernel (one launch per chunk, each after its chunk's
                              work order when the library orders the items): dk, dv (and the
                              dS tiles in VSA_DQ_SPILL mode) */
  VSA_BWD_DQ = 3           /* q-major kernel (VSA_DQ_RECOMPUTE: one launch per chunk):
                              dq = bf16(sm_scale * dS K) */
} vsa_bwd_stage_id;
int vsa_bwd_stage(const vsa_bwd_args* a, int stage, void* stream);

/* vsa_bwd for callers that cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same validation, kernels and results as vsa_bwd, with the
 * workspace taken from a static device array of VSA_NOALLOC_SCRATCH_BYTES inside the library
 * (one per GPU, held until the process ends) instead of a->workspace, which is ignored along with
 * a->workspace_bytes. The caller still passes every input and output. A call whose
 * vsa_bwd_workspace_bytes exceeds the scratch returns VSA_EUNSUPPORTED (the workspace holds about
 * 65 KiB per q block for the fp16 operand copies and records, so recompute mode fits up to about
 * 8100 q blocks per call (B*H*nb), e.g. 8 heads of 32768 tokens; the dS spill, 8 KiB per
 * possible pair, fits only small problems). Calls on one GPU share its scratch: calls that
 * overlap there (different streams, no ordering between them) race and give undefined results.
 * The chain writes every scratch region it reads within the call, so no clearing is needed
 * between calls. The first call on a device resolves the scratch address there
 * (hipGetSymbolAddress); no call allocates or frees memory. */
#define VSA_NOALLOC_SCRATCH_BYTES (512u << 20)
int vsa_bwd_noalloc(const vsa_bwd_args* a, void* stream);

/* Work order alone: for each (b, h), its kv items ranked by bin = k2q_num / bin_width (larger bin
 * first, then ascending kv id); writes item ids (b*H + h)*nb + kv to order [B*H*nb]. nb may be at
 * most VSA_ORDER_MAX_KV_BLOCKS; bin_width >= 1. */
int vsa_bwd_order(const int32_t* k2q_num, int batch, int heads, int num_kv_blocks, int bin_width,
                  int32_t* order, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* VSA_H */
