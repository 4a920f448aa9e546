// bwd_aux.hip -- the streaming kernels around the backward's main kernels (gfx950):
//   preprocess  Delta = rowsum(bf16(o) * dO) in fp32, and the exact-zero dK/dV rows of kv blocks
//               that no q block selects (FastVideo sm_100a backward commit message, the
//               preprocess sentence; launch header, the delta field of the argument struct);
//               here also the per-head power-of-two scales and scaled fp16 copies of q, k, dO
//               (and v) that let the main kernels run their GEMMs on fp16 operands (the backward
//               test page's tolerance block measures the result against bf16-rounded
//               references: fp16 P and dS carry 11 significant bits where bf16 carries 8).
//               Delta and lse go into a 512-byte record per q block, the initial accumulator
//               values of the kv-major kernel's S and dP MFMAs;
//   order       the per-(b, h) length-binned permutation of work items that the launch header
//               computes on device from 1024 kv blocks on (its order-kernel launch and the
//               ORDER_MIN_KV_BLOCKS comment); used for the kv-major and the q-major kernel;
//   slot tables for the dS spill: where each (q block, kv block) pair's dS tile goes (kv-major
//               order, contiguous per kv block) and, per q2k entry, where to find it.
// The preprocess streams with 16-byte accesses, consecutive lanes on consecutive 16-byte chunks
// of a row. (The pages' dQ postprocess -- scale by sm_scale, round to bf16 -- is fused into the
// q-major dQ kernels' epilogues here.)
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace vsa {

namespace {

// Max over the 64 lanes of a wave, then over the four waves through LDS; every thread gets it.
// Values are non-negative fp32 bit patterns, so the integer max is the value max.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();  // red may still be read from the previous call
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return max(max(red[0], red[1]), max(red[2], red[3]));
}

// Sum of the 16 lanes that share a row (fixed order), every lane of the group gets it.
__device__ __forceinline__ float row_sum16(float a) {
  a += __shfl_xor(a, 8, 64);
  a += __shfl_xor(a, 4, 64);
  a += __shfl_xor(a, 2, 64);
  a += __shfl_xor(a, 1, 64);
  return a;
}

__device__ __forceinline__ float fbits(uint32_t u) { return __uint_as_float(u); }

// ceil(log2(b)) for a positive normal fp32 value
__device__ __forceinline__ int ceil_log2(float b) {
  const uint32_t u = __float_as_uint(b);
  const int ex = (int)((u >> 23) & 0xFF) - 127;
  return (u & 0x7FFFFF) ? ex + 1 : ex;
}

}  // namespace

// Pass 1, grid (nb, BH), 256 threads (each pass of four covers 16 rows x 16 chunks of 8
// elements): the block's maxima of |q|, |k|, |v|, |dO|, of the row norms |v_j|^2, |dO_i|^2 and of
// |Delta_i|; Delta_i = rowsum(bf16(o) * dO) in fp32 goes (negated) into the dP half of the record;
// the exact-zero dK/dV rows of a kv block that no q block selects.
__global__ void __launch_bounds__(256) bwd_stats_kernel(BwdPreParams p) {
  __shared__ uint32_t red[4];
  const int blk = blockIdx.x;
  const int bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int rr = tid >> 4;  // row inside the pass
  const int c = tid & 15;   // 16-byte chunk of the row
  const size_t row0 = (size_t)bh * p.S + (size_t)blk * BLOCK;
  // (a negative count, a caller-contract violation, also gets zero rows: the kv-major kernel
  // skips items whose clamped count is 0)
  const bool empty = p.k2q_num[(size_t)bh * p.nb + blk] <= 0;
  float* rec = p.lse_delta + ((size_t)bh * p.nb + blk) * LD_RECORD_FLOATS;
  uint32_t mq = 0, mk = 0, mv = 0, mo = 0;
  float n2v = 0.0f, n2o = 0.0f, md = 0.0f;
  // the stores come after every load: as far as the compiler knows they may alias the inputs,
  // and a load placed after a store would wait for it
  float dl[4];
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const size_t row = row0 + pass * 16 + rr;
    const size_t at = row * HEAD_DIM + c * 8;
    const bf16x8 q = *(const bf16x8*)(p.q + at);
    const bf16x8 k = *(const bf16x8*)(p.k + at);
    const bf16x8 v = *(const bf16x8*)(p.v + at);
    const bf16x8 o = *(const bf16x8*)(p.o + at);
    const bf16x8 d = *(const bf16x8*)(p.dout + at);
    mq = max(mq, absmax_bits8(q));
    mk = max(mk, absmax_bits8(k));
    mv = max(mv, absmax_bits8(v));
    mo = max(mo, absmax_bits8(d));
    float delta = 0.0f, sv = 0.0f, so = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      delta = __builtin_fmaf((float)o[e], (float)d[e], delta);
      sv = __builtin_fmaf((float)v[e], (float)v[e], sv);
      so = __builtin_fmaf((float)d[e], (float)d[e], so);
    }
    delta = row_sum16(delta);
    n2v = fmaxf(n2v, row_sum16(sv));
    n2o = fmaxf(n2o, row_sum16(so));
    md = fmaxf(md, fabsf(delta));
    dl[pass] = delta;
  }
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    if (c == 0) rec[BLOCK + pass * 16 + rr] = -dl[pass];
    if (empty) {
      const size_t at = (row0 + pass * 16 + rr) * HEAD_DIM + c * 8;
      *(bf16x8*)(p.dk + at) = bf16x8{};
      *(bf16x8*)(p.dv + at) = bf16x8{};
    }
  }
  // (max over NaN: fmaxf drops it and integer max keeps the larger pattern; a NaN input
  // propagates through the kernels' arithmetic either way)
  uint32_t out[7] = {mq, mk, mv, mo, __float_as_uint(n2v), __float_as_uint(n2o),
                     __float_as_uint(md)};
  uint32_t* st = p.stats + ((size_t)bh * p.nb + blk) * STAT_WORDS;
#pragma unroll
  for (int i = 0; i < 7; ++i) {
    const uint32_t m = block_max_u32(out[i], red);
    if (tid == 0) st[i] = m;
  }
  if (tid == 0) st[7] = 0;
}

// Pass 2, one 256-thread workgroup per head: reduce the block statistics, derive the exponents.
__global__ void __launch_bounds__(256) bwd_scales_kernel(BwdPreParams p) {
  __shared__ uint32_t red[4];
  const int bh = blockIdx.x;
  const uint32_t* st = p.stats + (size_t)bh * p.nb * STAT_WORDS;
  uint32_t m[7] = {0, 0, 0, 0, 0, 0, 0};
  for (int b = threadIdx.x; b < p.nb; b += 256) {
#pragma unroll
    for (int i = 0; i < 7; ++i) m[i] = max(m[i], st[(size_t)b * STAT_WORDS + i]);
  }
#pragma unroll
  for (int i = 0; i < 7; ++i) m[i] = block_max_u32(m[i], red);
  if (threadIdx.x != 0) return;
  // q16, k16 exponents, moved (equally) where needed so that c = scale_log2 * 2^(eq + ek) stays
  // within [2^-101, 2^102]: only a head whose scores are all far below fp32 resolution (or
  // beyond its range) gets there, and then loses fp16 precision in q16, k16
  int eq = f16_exponent(m[ST_Q], 14);
  int ek = f16_exponent(m[ST_K], 14);
  {
    const int l = (int)((__float_as_uint(p.scale_log2) >> 23) & 0xFF) - 127;  // normal: >= 2^-120
    const int t = l + eq + ek;
    const int d = t < -100 ? -100 - t : (t > 100 ? 100 - t : 0);
    eq += d / 2;
    ek += d - d / 2;
  }
  const int ev = f16_exponent(m[ST_V], 0);
  const int eo = f16_exponent(m[ST_DO], 0);
  // |dP_ij - Delta_i| in the scaled units, with margin for the fp32 sums
  const float nv = __builtin_ldexpf(sqrtf(fbits(m[ST_V2])), -ev);
  const float no = __builtin_ldexpf(sqrtf(fbits(m[ST_DO2])), -eo);
  const float dm = __builtin_ldexpf(__builtin_ldexpf(fbits(m[ST_DELTA]), -eo), -ev);
  const float b = 1.0625f * (no * nv + dm);
  int pp = 15;
  if (!(b <= 3.0e38f)) pp = -30;                 // inf or NaN inputs
  else if (b >= 0x1p-126f) pp = 15 - ceil_log2(b);
  pp = pp > 15 ? 15 : (pp < -30 ? -30 : pp);
  int32_t* out = p.scales + (size_t)bh * HEAD_SCALE_WORDS;
  out[SC_EQ] = eq;
  out[SC_EK] = ek;
  out[SC_EV] = ev;
  out[SC_EO] = eo;
  out[SC_PP] = pp;
  out[SC_ES] = pp - eo - ev;
  out[SC_C] = (int32_t)__float_as_uint(__builtin_ldexpf(p.scale_log2, eq + ek));
  out[7] = 0;
}

// Pass 3, grid (nb, BH), 256 threads: the fp16 copies of block blk's rows of q, k, dO (and v when
// asked), and the record: (pp - lse) / c (IEEE fp32 subtraction and division), -Delta 2^-(eo+ev).
__global__ void __launch_bounds__(256) bwd_convert_kernel(BwdPreParams p) {
  const int blk = blockIdx.x;
  const int bh = blockIdx.y;
  const int tid = threadIdx.x;
  const int rr = tid >> 4;
  const int c = tid & 15;
  const int32_t* sc = p.scales + (size_t)bh * HEAD_SCALE_WORDS;
  const int eq = ld_const(sc, SC_EQ), ek = ld_const(sc, SC_EK), ev = ld_const(sc, SC_EV);
  const int eo = ld_const(sc, SC_EO), pp = ld_const(sc, SC_PP);
  const float cc = __uint_as_float((uint32_t)ld_const(sc, SC_C));
  const size_t row0 = (size_t)bh * p.S + (size_t)blk * BLOCK;
  float* rec = p.lse_delta + ((size_t)bh * p.nb + blk) * LD_RECORD_FLOATS;
  // every load before any store: the copies may alias the inputs as far as the compiler knows,
  // so a load placed after a store would wait for it
  bf16x8 xq[4], xk[4], xd[4], xv[4];
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const size_t at = (row0 + pass * 16 + rr) * HEAD_DIM + c * 8;
    xq[pass] = *(const bf16x8*)(p.q + at);
    xk[pass] = *(const bf16x8*)(p.k + at);
    xd[pass] = *(const bf16x8*)(p.dout + at);
    if (p.v16) xv[pass] = *(const bf16x8*)(p.v + at);
  }
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const size_t row = row0 + pass * 16 + rr;
    const size_t at = row * HEAD_DIM + c * 8;
    *(f16x8*)(p.q16 + at) = bf16x8_to_f16x8(xq[pass], eq);
    *(f16x8*)(p.k16 + at) = bf16x8_to_f16x8(xk[pass], ek);
    *(f16x8*)(p.do16 + at) = bf16x8_to_f16x8(xd[pass], eo);
    if (p.v16) *(f16x8*)(p.v16 + at) = bf16x8_to_f16x8(xv[pass], ev);
    if (c == 0) {
      const int r = pass * 16 + rr;
      rec[r] = ((float)pp - p.lse[row]) / cc;
      rec[BLOCK + r] = __builtin_ldexpf(__builtin_ldexpf(rec[BLOCK + r], -eo), -ev);
    }
  }
}

void launch_bwd_pre(const BwdPreParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(bwd_stats_kernel, dim3(p.nb, p.BH), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(bwd_scales_kernel, dim3(p.BH), dim3(256), 0, stream, p);
  hipLaunchKernelGGL(bwd_convert_kernel, dim3(p.nb, p.BH), dim3(256), 0, stream, p);
}

// Work order of one (b, h) (one 1024-thread workgroup): bitonic sort of 32-bit keys (inverted
// bin << 14 | kv) in LDS, so the result is larger bins first and ascending kv inside a bin -- a
// deterministic permutation. bin = cnt(kv) / bin_width, clamped to 18 bits.
template <typename Cnt>
__device__ void order_block_of(Cnt cnt, int nb, int bin_width, int32_t* __restrict__ order,
                               int bh) {
  __shared__ uint32_t keys[ORDER_MAX_KV_BLOCKS];
  const int tid = threadIdx.x;
  int P = 1;
  while (P < nb) P <<= 1;
  for (int i = tid; i < P; i += 1024) {
    uint32_t key = 0xFFFFFFFFu;
    if (i < nb) {
      int num = cnt(i);
      num = num < 0 ? 0 : num;
      uint32_t bin = (uint32_t)(num / bin_width);
      bin = bin > 0x3FFFFu ? 0x3FFFFu : bin;
      key = ((0x3FFFFu - bin) << 14) | (uint32_t)i;
    }
    keys[i] = key;
  }
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = tid; i < P; i += 1024) {
        const int ixj = i ^ jj;
        if (ixj > i) {
          const uint32_t a = keys[i], b = keys[ixj];
          const bool up = (i & k) == 0;
          if ((a > b) == up) {
            keys[i] = b;
            keys[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int r = tid; r < nb; r += 1024)
    order[(size_t)bh * nb + r] = bh * nb + (int)(keys[r] & 0x3FFFu);
}

__device__ void order_block(const int32_t* __restrict__ num_in, int nb, int bin_width,
                            int32_t* __restrict__ order, int bh) {
  order_block_of([&](int i) { return num_in[(size_t)bh * nb + i]; }, nb, bin_width, order, bh);
}

// Exclusive prefix sum of cnt(0 .. nb-1) into out[0 .. nb-1] (one 1024-thread workgroup). Thread t
// sums a contiguous chunk of ceil(nb / 1024) counts, the 1024 chunk sums are scanned in LDS, and
// each thread writes its chunk's prefixes.
template <typename Cnt>
__device__ void prefix_block(Cnt cnt, int nb, int32_t* __restrict__ out) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int chunk = (nb + 1023) / 1024;
  const int lo = tid * chunk;
  const int hi = lo + chunk < nb ? lo + chunk : nb;
  int sum = 0;
  for (int i = lo; i < hi; ++i) sum += cnt(i);
  part[tid] = sum;
  __syncthreads();
  // Hillis-Steele inclusive scan of the chunk sums
  for (int d = 1; d < 1024; d <<= 1) {
    const int v = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - sum;  // exclusive prefix of this chunk
  for (int i = lo; i < hi; ++i) {
    out[i] = run;
    run += cnt(i);
  }
}

// dS slot bases of one head: exclusive prefix sum of the clamped k2q counts.
__device__ void kbase_block(const int32_t* __restrict__ num, int nb, int stride,
                            int32_t* __restrict__ kbase, int bh) {
  const int32_t* row = num + (size_t)bh * nb;
  prefix_block(
      [&](int i) {
        const int c = row[i];
        return c < 0 ? 0 : (c > stride ? stride : c);
      },
      nb, kbase + (size_t)bh * nb);
}

// Per-chunk slot bases, workgroup (bh, c): the counts are each kv item's positions in chunk c,
// with the bounds clamped exactly as the kv-major kernel clamps them.
__global__ void __launch_bounds__(1024) chunk_kbase_kernel(const int32_t* __restrict__ bounds,
                                                           const int32_t* __restrict__ k2q_num,
                                                           int k2q_stride, int nb, int BH,
                                                           int nchunks, int32_t* __restrict__ kbase) {
  const int bh = blockIdx.x, c = blockIdx.y;
  prefix_block(
      [&](int j) {
        const size_t item = (size_t)bh * nb + j;
        int n = k2q_num[item];
        n = n < 0 ? 0 : (n > k2q_stride ? k2q_stride : n);
        const int32_t* cb = bounds + item * (nchunks + 1) + c;
        int b0 = cb[0], b1 = cb[1];
        b0 = b0 < 0 ? 0 : (b0 > n ? n : b0);
        b1 = b1 < b0 ? b0 : (b1 > n ? n : b1);
        return b1 - b0;
      },
      nb, kbase + ((size_t)c * BH + bh) * nb);
}

void launch_chunk_kbase(const int32_t* bounds, const int32_t* k2q_num, int k2q_stride, int BH,
                        int nb, int nchunks, int32_t* kbase, hipStream_t stream) {
  hipLaunchKernelGGL(chunk_kbase_kernel, dim3(BH, nchunks), dim3(1024), 0, stream, bounds,
                     k2q_num, k2q_stride, nb, BH, nchunks, kbase);
}

__global__ void __launch_bounds__(1024) bwd_order_kernel(const int32_t* __restrict__ num_in, int nb,
                                                         int bin_width, int32_t* __restrict__ order) {
  order_block(num_in, nb, bin_width, order, blockIdx.x);
}

void launch_bwd_order(const int32_t* num, int BH, int nb, int bin_width, int32_t* order,
                      hipStream_t stream) {
  hipLaunchKernelGGL(bwd_order_kernel, dim3(BH), dim3(1024), 0, stream, num, nb, bin_width, order);
}

// The work order of chunk c of chunked launches (the kv-major kernel over k2q lists, the forward
// over q2k lists): items binned by the length of their list's part inside the chunk (the
// positions chunk_bounds gives, clamped as both kernels clamp them), so the items that run
// together on an XCD walk parts of equal length. One 1024-thread workgroup per (b, h).
__global__ void __launch_bounds__(1024) chunk_order_kernel(const int32_t* __restrict__ bounds,
                                                           const int32_t* __restrict__ num,
                                                           int stride, int nb, int nchunks,
                                                           int c, int bin_width,
                                                           int32_t* __restrict__ order) {
  const int bh = blockIdx.x;
  auto cnt = [&](int i) {
    const size_t item = (size_t)bh * nb + i;
    int n = num[item];
    n = n > stride ? stride : n;
    if (n <= 0) return 0;
    const int32_t* cb = bounds + item * (nchunks + 1) + c;
    int b0 = cb[0], b1 = cb[1];
    b0 = b0 < 0 ? 0 : (b0 > n ? n : b0);
    b1 = b1 < b0 ? b0 : (b1 > n ? n : b1);
    return b1 - b0;
  };
  order_block_of(cnt, nb, bin_width, order, bh);
}

void launch_chunk_order(const int32_t* bounds, const int32_t* num, int stride, int BH, int nb,
                        int nchunks, int c, int bin_width, int32_t* order, hipStream_t stream) {
  hipLaunchKernelGGL(chunk_order_kernel, dim3(BH), dim3(1024), 0, stream, bounds, num, stride, nb,
                     nchunks, c, bin_width, order);
}

// The index stage's per-head tasks in one launch: workgroup (bh, task) runs task blockIdx.y of the
// list for head bh (a work order or the dS slot bases); the tasks are independent.
__global__ void __launch_bounds__(1024) index_tasks_kernel(IndexTasks t, int nb, int bin_width,
                                                           int k2q_stride) {
  const IndexTask& task = t.task[blockIdx.y];
  if (task.kind == IndexTask::ORDER)
    order_block(task.num, nb, bin_width, task.out, blockIdx.x);
  else
    kbase_block(task.num, nb, k2q_stride, task.out, blockIdx.x);
}

void launch_index_tasks(const IndexTasks& t, int BH, int nb, int bin_width, int k2q_stride,
                        hipStream_t stream) {
  if (t.count <= 0) return;
  hipLaunchKernelGGL(index_tasks_kernel, dim3(BH, t.count), dim3(1024), 0, stream, t, nb,
                     bin_width, k2q_stride);
}


// One thread per q2k entry (bh, q, s): binary search of q in the ascending k2q row of its kv
// block (with chunks, only between the bounds of q's chunk in that row). A q missing from that
// row (a caller-contract violation: k2q is not the inverse of q2k, or not ascending) gets the
// first slot of the row (of its chunk's part), so every slot stays inside the head's range. With
// chunks the slot is numbered inside the chunk of q (launch_spill_qent). The kernel is bound by
// the latency of its dependent loads, so the independent ones are issued together: the entry
// with its row's count, then the kv block's list length, slot base, chunk bound and size.
__global__ void __launch_bounds__(256) spill_qent_kernel(
    const int32_t* __restrict__ q2k_idx, const int32_t* __restrict__ q2k_num, int q2k_stride,
    const int32_t* __restrict__ k2q_idx, const int32_t* __restrict__ k2q_num, int k2q_stride,
    const int32_t* __restrict__ kbase, const int32_t* __restrict__ vbs, int nb, int cap,
    const int32_t* __restrict__ bounds, int nchunks, int width, int64_t* __restrict__ qent) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;  // entry within the head
  const int bh = blockIdx.y;
  if (e >= (size_t)nb * q2k_stride) return;
  const int q = (int)(e / q2k_stride);
  const int s = (int)(e - (size_t)q * q2k_stride);
  const size_t qrow = (size_t)bh * nb + q;
  int n = q2k_num[qrow];
  int kv = q2k_idx[qrow * q2k_stride + s];  // inside the row; used only when s < n
  n = n < 0 ? 0 : (n > q2k_stride ? q2k_stride : n);
  if (s >= n) return;
  kv = kv < 0 ? 0 : (kv >= nb ? nb - 1 : kv);
  const size_t krow = (size_t)bh * nb + kv;
  int c = 0;
  if (bounds) {
    c = q / width;
    c = c < nchunks ? c : nchunks - 1;
  }
  int m = k2q_num[krow];
  const int base = bounds ? kbase[(size_t)c * gridDim.y * nb + krow] : kbase[krow];
  const int b0raw = bounds ? bounds[krow * (nchunks + 1) + c] : 0;
  const int b1raw = bounds ? bounds[krow * (nchunks + 1) + c + 1] : 0;
  int vb = vbs[kv];
  m = m < 0 ? 0 : (m > k2q_stride ? k2q_stride : m);
  // with chunks, q (in chunk c) sits between the chunk's bounds in the row, clamped as the
  // kv-major kernel clamps them
  const int b0 = bounds ? (b0raw < 0 ? 0 : (b0raw > m ? m : b0raw)) : 0;
  const int b1 = bounds ? (b1raw < b0 ? b0 : (b1raw > m ? m : b1raw)) : m;
  const int32_t* list = k2q_idx + krow * k2q_stride;
  // first position in [b0, b1) with list[pos] >= q; vhi is the value at hi once hi has moved
  // (q >= 0, so -1 never matches), which spares a last dependent load
  int lo = b0, hi = b1, vhi = -1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const int v = list[mid];
    if (v < q) {
      lo = mid + 1;
    } else {
      hi = mid;
      vhi = v;
    }
  }
  const int t = (lo < b1 && vhi == q) ? lo : b0;
  int slot = base + t - b0;
  slot = slot < 0 ? 0 : (slot >= cap ? cap - 1 : slot);
  vb = vb < 0 ? 0 : (vb > BLOCK ? BLOCK : vb);
  qent[qrow * q2k_stride + s] =
      (int64_t)(uint32_t)slot | ((int64_t)kv << 32) | ((int64_t)vb << 48);
}

// One thread per (item, chunk boundary c = 0 .. nchunks): a binary search of the list.
__global__ void __launch_bounds__(256) chunk_bounds_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ num, int stride,
    int total_items, int nchunks, int width, int32_t* __restrict__ bounds) {
  const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (size_t)total_items * (nchunks + 1)) return;
  const size_t item = e / (nchunks + 1);
  const int c = (int)(e - item * (nchunks + 1));
  int m = num[item];
  m = m < 0 ? 0 : (m > stride ? stride : m);
  int lo = c == 0 ? 0 : m;  // the chunks always cover positions 0 .. m - 1
  if (c > 0 && c < nchunks) {
    const long long lim = (long long)c * width;
    const int32_t* list = idx + item * stride;
    int hi = m;
    lo = 0;
    while (lo < hi) {  // first position with list[pos] >= lim (for an ascending list)
      const int mid = (lo + hi) >> 1;
      if ((long long)list[mid] < lim) lo = mid + 1; else hi = mid;
    }
  }
  bounds[e] = lo;
}

void launch_chunk_bounds(const int32_t* idx, const int32_t* num, int stride, int total_items,
                         int nchunks, int width, int32_t* bounds, hipStream_t stream) {
  const size_t n = (size_t)total_items * (nchunks + 1);
  hipLaunchKernelGGL(chunk_bounds_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     idx, num, stride, total_items, nchunks, width, bounds);
}

void launch_spill_qent(const int32_t* q2k_idx, const int32_t* q2k_num, int q2k_stride,
                       const int32_t* k2q_idx, const int32_t* k2q_num, int k2q_stride,
                       const int32_t* kbase, const int32_t* vbs, int BH, int nb, int cap,
                       const int32_t* bounds, int nchunks, int width, int64_t* qent,
                       hipStream_t stream) {
  const size_t per_head = (size_t)nb * q2k_stride;
  hipLaunchKernelGGL(spill_qent_kernel, dim3((unsigned)((per_head + 255) / 256), BH), dim3(256), 0,
                     stream, q2k_idx, q2k_num, q2k_stride, k2q_idx, k2q_num, k2q_stride, kbase,
                     vbs, nb, cap, bounds, nchunks, width, qent);
}

}  // namespace vsa
