// vsa_kernels.h -- internal launch interface between the C-ABI entry points (vsa_api.hip) and the
// gfx950 kernels. Not part of the public ABI. All pointers are device pointers; every launcher
// enqueues on `stream` and returns without synchronizing.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "vsa_device.h"

namespace vsa {

// ---- invert_indices: q2k -> k2q, sorted ascending, bit-exact ----
void launch_invert(const int32_t* q2k_idx, const int32_t* q2k_num, int BH, int nq, int topk,
                   int nkv, int32_t* k2q_idx, int32_t* k2q_num, uint32_t* bitmap,
                   hipStream_t stream);
size_t invert_bitmap_bytes(int BH, int nq, int nkv);

// ---- forward: o (bf16) and lse (fp32, base-2 M form) ----
struct FwdParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const int32_t* q2k_idx;  // [BH, nq, q2k_stride]
  const int32_t* q2k_num;  // [BH, nq]
  const int32_t* vbs;      // [nkv]
  bf16* o;
  float* lse;
  // fp16 copy of v, each head scaled by 2^-e with e = f16_head_exponent(v_amax[bh]) (the P V
  // product runs in fp16: see launch_v16)
  const f16* v16;
  const uint32_t* v_amax;  // [BH]: bits of each head's max |v|
  int BH, S, nb, q2k_stride;
  int items_per_xcd;  // ceil(BH * nb / 8): workgroup ids map XCD-first onto (bh, q block) items
  float scale_log2;
  // kv-range chunks (nchunks 0: one launch): this launch takes list positions
  // [bounds[item][chunk], bounds[item][chunk+1]) and carries each wave's state in `state`
  // (defaults: one launch, so a caller that predates the chunks cannot leave them undefined)
  const int32_t* chunk_bounds = nullptr;  // [BH * nb, nchunks + 1]
  float* state = nullptr;                 // [BH * nb, 4 waves, FWD_STATE_FLOATS]
  int chunk = 0, nchunks = 0;
  // work order of this launch: a permutation of the BH * nb item ids (nullptr: identity)
  const int32_t* order = nullptr;
};
// per wave: 64 lane-major rows of O^T accumulator elements, then the running max and sum rows
constexpr int FWD_STATE_FLOATS = 66 * 64;
void launch_fwd(const FwdParams& p, hipStream_t stream);
// The forward's V pre-pass: tmax[bh * S/64 + t] = bits of max |v| over 64-row tile t, amax[bh]
// = their max over the head, then v16 = fp16(v * 2^-e) with e = f16_head_exponent(amax[bh]).
// Three launches; v and v16 are [BH, S, 128].
void launch_v16(const bf16* v, int BH, int S, uint32_t* amax, uint32_t* tmax, f16* v16,
                hipStream_t stream);

// ---- backward preprocess: operand scaling, Delta, records, zero dK/dV rows of empty kv blocks ----
// The backward's MFMAs run in fp16 (v_mfma_f32_32x32x16_f16, the bf16 rate): P and dS keep 11
// significant bits instead of 8. Every operand is an fp16 copy scaled by a per-head power of two,
// so each GEMM's sum has one exact scale per head that the epilogues take back out:
//   q16 = q 2^-eq, k16 = k 2^-ek      (max |.| in [2^14, 2^15): exact copies of the bf16 values)
//   v16 = v 2^-ev, do16 = dO 2^-eo    (max |.| in [1, 2))
//   P'  = P 2^pp,  dS' = dS 2^es with es = pp - eo - ev
// pp is the largest exponent (at most 15) with 2^pp * bound(|dP - Delta|) <= 2^15 in the scaled
// units, so |dS'| <= |P'| |dP' - Delta'| stays inside fp16's range; the bound is
// 1.0625 (max_i |dO_i| max_j |v_j| + max |Delta|) with row 2-norms (Cauchy-Schwarz).
// Per head, as int32 words (c as fp32 bits):
enum HeadScaleWord { SC_EQ = 0, SC_EK, SC_EV, SC_EO, SC_PP, SC_ES, SC_C, HEAD_SCALE_WORDS = 8 };
// SC_C = scale_log2 * 2^(eq + ek): the base-2 softmax exponent per unit of q16 . k16.
// Per (bh, 64-row block), fp32 bit patterns of non-negative values (integer max = value max):
enum StatWord {
  ST_Q = 0, ST_K, ST_V, ST_DO,  // max |x| over the block's rows
  ST_V2, ST_DO2,                // max row |x|^2
  ST_DELTA,                     // max |Delta|
  STAT_WORDS = 8
};
// The main kernels read a q block's row statistics as one record of LD_RECORD_FLOATS floats per
// (bh, q block): (pp - lse) / c of its 64 rows, then -Delta 2^-(eo + ev) of its 64 rows. The
// kv-major kernel loads them straight into its S and dP accumulators as the initial values, so
// the MFMAs produce S' + (pp - lse) / c and dP' - Delta' with no per-element subtraction, and
// P' = exp2(c acc).
constexpr int LD_RECORD_FLOATS = 2 * BLOCK;
struct BwdPreParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const bf16* dout;
  const float* lse;        // [BH, S]
  const int32_t* k2q_num;  // [BH, nb]
  float* lse_delta;        // [BH * nb, LD_RECORD_FLOATS]
  uint32_t* stats;         // [BH * nb, STAT_WORDS]
  int32_t* scales;         // [BH, HEAD_SCALE_WORDS]
  f16* q16;                // fp16 copies [BH, S, 128]
  f16* k16;
  f16* do16;
  f16* v16;                // nullptr: not needed (only the recomputing dQ kernel reads it)
  bf16* dk;
  bf16* dv;
  int BH, S, nb;
  float scale_log2;
};
// Three launches: block statistics (and Delta), per-head scales, then the copies and records.
void launch_bwd_pre(const BwdPreParams& p, hipStream_t stream);

// ---- work order: per (b, h) a length-binned permutation of its items ----
constexpr int ORDER_MAX_KV_BLOCKS = 16384; // LDS holds one 32-bit key per block
void launch_bwd_order(const int32_t* num, int BH, int nb, int bin_width, int32_t* order,
                      hipStream_t stream);
// The work order of chunk c of chunked launches: items binned by the length of their list's
// part inside the chunk (bounds from launch_chunk_bounds over the lists num / stride: k2q for the
// kv-major kernel, q2k for the forward), one permutation per (b, h).
void launch_chunk_order(const int32_t* bounds, const int32_t* num, int stride, int BH, int nb,
                        int nchunks, int c, int bin_width, int32_t* order, hipStream_t stream);
// Up to three per-head tasks of the index stage in one launch (one 1024-thread workgroup per
// head and task): ORDER writes the work order of `num` (counts per item) to `out`; KBASE writes
// the dS slot bases (exclusive prefix sum of the clamped k2q counts `num`) to `out`.
struct IndexTask {
  enum Kind { ORDER = 0, KBASE = 1 };
  int kind;
  const int32_t* num;
  int32_t* out;
};
struct IndexTasks {
  IndexTask task[3];
  int count;
};
void launch_index_tasks(const IndexTasks& t, int BH, int nb, int bin_width, int k2q_stride,
                        hipStream_t stream);

// ---- the two main backward kernels (kv-major dK/dV, q-major dQ) ----
struct BwdParams {
  const bf16* v;           // bf16 v (the kv-major kernel converts its tile in registers)
  const f16* q16;          // the preprocess's scaled fp16 copies
  const f16* k16;
  const f16* v16;          // recompute mode only
  const f16* do16;
  const int32_t* scales;   // [BH, HEAD_SCALE_WORDS]
  const float* lse;        // [BH, S] base-2 M-form lse (the dQ kernel's)
  const float* lse_delta;  // [BH*nb, LD_RECORD_FLOATS]: the q blocks' records (see above)
  const int32_t* k2q_idx;  // [BH*nb, k2q_stride]
  const int32_t* k2q_num;  // [BH*nb]
  const int32_t* q2k_idx;  // [BH*nb, q2k_stride]
  const int32_t* q2k_num;  // [BH*nb]
  const int32_t* vbs;
  const int32_t* kv_order;  // nullptr: identity
  const int32_t* q_order;   // nullptr: identity
  bf16* dq;
  bf16* dk;
  bf16* dv;
  // dS spill (nullptr ds: recompute mode): slot tables from the index stage and the tiles
  const int32_t* kbase;  // [BH*nb]: first slot of each kv block's pairs inside its head
  const int64_t* qent;   // [BH*nb, qent_stride]: slot | kv << 32 | vbs[kv] << 48
  f16* ds;               // [BH, cap, 64*64]: dS' tiles
  int cap, qent_stride;  // slots per head (nb * K'), q2k row width K'
  // q-range chunks of the kv-major kernel (nchunks 0: one launch over whole lists): this launch
  // takes list positions [bounds[item][chunk], bounds[item][chunk+1]) and carries dV, dK
  // (unscaled fp32, [item][2][64][128]) in part from chunk to chunk
  // (defaults: one launch, so a caller that predates the chunks cannot leave them undefined);
  // partial sums are in the scaled units of the fp16 operands
  const int32_t* chunk_bounds = nullptr;  // [total_items, nchunks + 1]
  float* part = nullptr;
  int chunk = 0, nchunks = 0;
  // chunked dS spill (spill mode with chunks): the kv-major kernel numbers each launch's tiles
  // from 0 (kbase then points at that chunk's slot bases), and the q-major kernel runs once per
  // chunk over q blocks [q_first, q_first + q_count) of every head (q_count 0: all items)
  int ds_chunk_local = 0;
  int q_first = 0, q_count = 0;
  int S, nb, k2q_stride, q2k_stride, total_items, items_per_xcd;
  // rounds of the kv-major kernel's XCD mapping (xcd_work_id); items_per_xcd is a multiple
  int kv_rounds = 1;
  float sm_scale;
};
void launch_bwd_dkdv(const BwdParams& p, hipStream_t stream);
void launch_bwd_dq(const BwdParams& p, hipStream_t stream);
void launch_bwd_dq_spill(const BwdParams& p, hipStream_t stream);

// ---- chunk bounds of block lists (k2q rows for the kv-major kernel, q2k rows for the
// forward): bounds[item][c] = the binary-search position of c * width in the item's list (the
// first entry >= c * width when the list is ascending), for c = 0 .. nchunks - 1, and
// bounds[item][nchunks] = the list length clamped to [0, stride]. Non-decreasing in c for any
// list, so the chunks partition the list. ----
void launch_chunk_bounds(const int32_t* idx, const int32_t* num, int stride, int total_items,
                         int nchunks, int width, int32_t* bounds, hipStream_t stream);

// ---- dS slot tables (spill mode) ----
// kbase[bh, kv] = sum of min(max(k2q_num, 0), k2q_stride) over the kv blocks before kv in head bh:
// an IndexTask::KBASE task.
// qent[bh, q, s] for s < q2k_num[bh, q]: the slot of pair (q, kv = q2k_idx[bh, q, s]), i.e.
// kbase[bh, kv] + (position of q in the ascending k2q row of kv), packed with kv and vbs[kv].
// With chunks (bounds non-null, the kv-major chunk bounds; nchunks chunks of `width` q blocks), the
// tiles are numbered per chunk: kbase holds [nchunks][BH * nb] slot bases and the pair of q block q
// takes slot kbase[q / width][bh, kv] + (its position) - bounds[bh, kv][q / width].
void launch_spill_qent(const int32_t* q2k_idx, const int32_t* q2k_num, int q2k_stride,
                       const int32_t* k2q_idx, const int32_t* k2q_num, int k2q_stride,
                       const int32_t* kbase, const int32_t* vbs, int BH, int nb, int cap,
                       const int32_t* bounds, int nchunks, int width, int64_t* qent,
                       hipStream_t stream);
// Per-chunk dS slot bases: kbase[c][bh * nb + kv] = sum over the kv blocks before kv in head bh of
// their pair counts in chunk c (bounds[item][c + 1] - bounds[item][c], clamped as the kv-major
// kernel clamps them against min(max(k2q_num, 0), k2q_stride)). One launch, (BH, nchunks)
// workgroups.
void launch_chunk_kbase(const int32_t* bounds, const int32_t* k2q_num, int k2q_stride, int BH,
                        int nb, int nchunks, int32_t* kbase, hipStream_t stream);

}  // namespace vsa
