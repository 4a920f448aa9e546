// bwd_dq_spill.hip -- dQ of the 64-token block-sparse attention backward from spilled dS tiles
// (gfx950): the q-major half of the backward's main step when the kv-major kernel has written
// every pair's dS to the workspace.
//
// What it computes (the gradient of the FastVideo backward test page's masked-dense reference;
// launch header argument struct: dq carries sm_scale): for one q block i of (b, h),
//     dQ_i = sum over kv blocks j in its q2k list of dS_ij K_j,    dq_i = bf16(sm_scale * dQ_i)
// with dS_ij the tile the kv-major kernel used for dK_j (so dq and dk see the same dS), kv rows
// at or past vbs[j] excluded. Operands are fp16: the spilled dS' = dS 2^es and the preprocess's
// k16 = K 2^-ek, so the sum is dQ 2^(es-ek) and the epilogue scales back by 2^(ek-es). A q block with an empty list gets zero rows. This is the
// pages' dQ accumulation and postprocess, reorganised as a per-q-block sum so that no atomics
// and no fp32 accumulator are needed; it does one GEMM per pair instead of the three of the
// recomputing kernel (bwd_dq.hip) and streams 8 KiB of dS per pair from HBM, which bounds it.
//
// gfx950 design: one 256-thread workgroup per q block, walking its slot-table row (VSA_WS_QENT:
// dS slot, kv block and vbs per entry). Wave w computes dQ^T rows d = 32w .. 32w+31 for both q
// halves: dQ^T += K^T dS^T with v_mfma_f32_32x32x16_f16, four k-steps of 16 kv per pair. K_j
// (16 KiB) and the dS tile (8 KiB) of each pair arrive by global_load_lds_dwordx4 into two LDS
// rings of 80 KiB together, so two workgroups share a CU: dS, streamed from HBM, is fetched three
// steps before it is read; K, mostly L2 hits, two steps before. Both operands come out of LDS
// through ds_read_b64_tr_b16, one pair ahead of their MFMAs. A pair of a ragged kv block has its
// padded kv slots masked to zero in both operands (so neither stale K rows nor the dS values of
// masked keys can reach dQ).
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace vsa {

namespace {

// Two rings per workgroup: dS tiles (from HBM) in SD stages, K tiles (mostly L2 hits) in SK
// stages; the tile of pair t goes to stage t % SD (t % SK). 4 x 8 KiB + 3 x 16 KiB = 80 KiB, so two
// workgroups share a CU and each covers the other's barrier and issue gaps.
constexpr int SD = 4;
constexpr int SK = 3;
constexpr int UNROLL = 12;      // a multiple of SD and SK: stage offsets are constants
static_assert(SD >= SK && SK >= 3 && UNROLL % SD == 0 && UNROLL % SK == 0 && UNROLL % 2 == 0, "");
constexpr int K_BYTES = 16384;  // one [64][128] fp16 K tile, swizzled
constexpr int S_BYTES = 8192;   // one dS tile, as the kv-major kernel stored it
constexpr int DMA_K = 4;        // per wave per pair: four 1-KiB slices of K
constexpr int DMA_S = 2;        // ... and two of dS

// A workgroup barrier that does not wait for this wave's LDS reads: the reads in flight at each
// barrier are of stages no DMA issued after it writes.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_dq_spill_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) char s_ring[SD * S_BYTES];
  __shared__ __attribute__((aligned(1024))) char k_ring[SK * K_BYTES];

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int kh = lane >> 5;     // k half of the MFMA operands
  const int grp = lane >> 4;    // 16-lane group
  const int t16 = lane & 15;
  const int gc = grp & 1;       // column half inside a 32-lane half

  const int wid = (blockIdx.x & 7) * p.items_per_xcd + (blockIdx.x >> 3);
  int item;  // (b, h, q block)
  if (p.q_count > 0) {  // one chunk of a chunked spill: q blocks [q_first, q_first + q_count)
    const int heads = p.total_items / p.nb;
    if (wid >= heads * p.q_count) return;
    const int bh_c = wid / p.q_count;
    item = bh_c * p.nb + p.q_first + (wid - bh_c * p.q_count);
  } else {
    if (wid >= p.total_items) return;
    item = p.q_order ? ld_const(p.q_order, wid) : wid;
  }
  if (item < 0 || item >= p.total_items) return;
  int n = ld_const(p.q2k_num, item);
  n = n < 0 ? 0 : (n > p.qent_stride ? p.qent_stride : n);
  const int bh = item / p.nb;
  const int i = item - bh * p.nb;
  const size_t head = (size_t)bh * p.S * HEAD_DIM;
  bf16* __restrict__ dq_blk = p.dq + head + (size_t)i * BLOCK * HEAD_DIM;
  if (n == 0) {  // no selected kv block: zero rows
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *(i32x4*)((char*)dq_blk + (c * 256 + threadIdx.x) * 16) = i32x4{};
    return;
  }
  const f16* __restrict__ kh_ptr = p.k16 + head;
  const char* __restrict__ ds_head = (const char*)p.ds + (size_t)bh * p.cap * S_BYTES;
  const int64_t* __restrict__ ent = p.qent + (size_t)item * p.qent_stride;
  auto entry = [&](int t) { return (uint64_t)ld_const(ent, t < n ? t : n - 1); };
  auto kv_of = [&](uint64_t e) {
    const int kv = (int)((e >> 32) & 0xFFFF);
    return kv < p.nb ? kv : p.nb - 1;
  };
  auto slot_of = [&](uint64_t e) {
    const int s = (int)(uint32_t)e;
    return s < 0 ? 0 : (s >= p.cap ? p.cap - 1 : s);
  };
  auto vb_of = [&](uint64_t e) { return (int)((e >> 48) & 0xFF); };

  uint32_t toff[4];
  tile_offsets_wave(toff, lane, w);
  const uint32_t k_lds = lds_addr((VSA_LDS char*)k_ring) + 4096 * w;
  const uint32_t s_lds = lds_addr((VSA_LDS char*)s_ring) + 2048 * w;
  const uint32_t s_off = 16 * lane;
  auto k_src = [&](uint64_t e) { return (const void*)(kh_ptr + (size_t)kv_of(e) * BLOCK * HEAD_DIM); };
  auto s_src = [&](uint64_t e) {
    return (const void*)(ds_head + (size_t)slot_of(e) * S_BYTES + 2048 * w);
  };
  auto issue_k = [&](const void* src, int sk) __attribute__((always_inline)) {
    dma_tile(src, toff, k_lds + sk * K_BYTES);
  };
  auto issue_s = [&](const void* src, int sd) __attribute__((always_inline)) {
    dma_lin2_nt(src, s_off, s_lds + sd * S_BYTES);
  };

  // Operands of one pair. A = K^T: lane holds d = 32w + lane%32 and kv 16ks + 8kh + j. B = dS^T
  // for q half qh: lane holds q column n = lane%32 (the record layout's order, see the epilogue)
  // and the same kv. Each is two transposed reads of four kv rows.
  struct Ops {
    f16x8 a[4];
    f16x8 b[2][4];
  };
  auto read_ops = [&](int sk, int sd, Ops& o) __attribute__((always_inline)) {
    VSA_LDS char* kt = (VSA_LDS char*)k_ring + sk * K_BYTES;
    VSA_LDS char* sb = (VSA_LDS char*)s_ring + sd * S_BYTES;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k0 = 16 * ks + 8 * kh;  // first kv of this lane's k slots
      const int col = 32 * w + 16 * gc + 4 * (t16 & 3);
      o.a[ks] = join_f16(lds_read_tr(kt + tile_elem_byte(k0 + (t16 >> 2), col)),
                         lds_read_tr(kt + tile_elem_byte(k0 + 4 + (t16 >> 2), col)));
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        s16x4 h2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int kk = k0 + 4 * u;  // record rows kk .. kk+3: kv half kk/32, rows kk%32 ..
          const int rec = ((qh + 2 * (kk >> 5)) * 8 + ((kk & 31) >> 2)) * 256 + 128 * gc +
                          32 * (t16 >> 2) + 8 * (t16 & 3);
          h2[u] = lds_read_tr(sb + rec);
        }
        o.b[qh][ks] = join_f16(h2[0], h2[1]);
      }
    }
  };
  // Padded kv slots of a ragged block (kv >= vb) to zero, in both operands.
  auto mask_ops = [&](int vb, Ops& o) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k0 = 16 * ks + 8 * kh;
      union {
        i32x4 m;
        f16x8 v;
      } mk;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        mk.m[d] = (k0 + 2 * d < vb ? 0xFFFF : 0) | (k0 + 2 * d + 1 < vb ? (int)0xFFFF0000u : 0);
      auto andv = [&](f16x8& x) {
        union {
          i32x4 m;
          f16x8 v;
        } u;
        u.v = x;
        u.m &= mk.m;
        x = u.v;
      };
      andv(o.a[ks]);
      andv(o.b[0][ks]);
      andv(o.b[1][ks]);
    }
  };

  // ---- prologue ----
  // In the steady state step u issues K of pair u+SK and then dS of pair u+SD. The prologue runs
  // the virtual steps u = -SD .. -1 of that sequence (skipping K of negative pairs), so the DMA
  // order, and with it every wait count below, is the same from the first step on.
  uint64_t e0[SD];
#pragma unroll
  for (int u = 0; u < SD; ++u) e0[u] = entry(u);
  uint64_t ek[SK];  // entries of the pairs whose K tiles are in the k ring (pair p: ek[p % SK])
#pragma unroll
  for (int u = 0; u < SK; ++u) ek[u] = e0[u];
#pragma unroll
  for (int u = -SD; u < 0; ++u) {
    if (u + SK >= 0) issue_k(k_src(e0[u + SK]), u + SK);
    issue_s(s_src(e0[u + SD]), u + SD);
  }
  // pairs 0 and 1 landed: after K of pair 1 come its step's dS and SK - 2 whole steps
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(DMA_S + (SK - 2) * (DMA_K + DMA_S)));
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), visible to the compiler
  barrier_only();                      // ... everyone's
  uint64_t nk = entry(SK), ns = entry(SD);  // the next step's K and dS entries

  f32x16 acc[2] = {f32x16{}, f32x16{}};
  Ops x, y;
  read_ops(0, 0, x);
  if (vb_of(ek[0]) < BLOCK) mask_ops(vb_of(ek[0]), x);

  // Step t (pair t: k stage t % SK, s stage t % SD). First everything this wave asked of LDS and
  // of the scalar cache is in: pair t's operands and the entries loaded last step. Then pair t+1's
  // operands are read while pair t's MFMAs run. Once K and dS of pair t+2 have landed (own DMAs,
  // then the barrier: everyone's), everyone is done with pair t's stages: K of pair t+SK and dS
  // of pair t+SD go there.
  auto step = [&](int t, int u, Ops& cur, Ops& nxt) __attribute__((always_inline)) {
    const int sk = u % SK, sd = u % SD;                // stages of pair t
    const int sk1 = (u + 1) % SK, sd1 = (u + 1) % SD;  // stages of pair t+1
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0), visible to the compiler
    const void* kn = k_src(nk);
    const void* sn = s_src(ns);
    asm volatile("" ::"s"(kn), "s"(sn));  // source addresses ready before the MFMAs
    read_ops(sk1, sd1, nxt);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      acc[0] = mfma32_f16(cur.a[ks], cur.b[0][ks], acc[0]);
      acc[1] = mfma32_f16(cur.a[ks], cur.b[1][ks], acc[1]);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // three transposed reads
    }
    __builtin_amdgcn_sched_barrier(0);
    // K of pair t+2 was issued SK-2 steps ago; after it come its step's dS and SK-3 whole steps
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(DMA_S + (SK - 3) * (DMA_K + DMA_S)));
    barrier_only();
    issue_k(kn, sk);
    issue_s(sn, sd);
    const int vb1 = vb_of(ek[sk1]);
    ek[sk] = nk;
    nk = entry(t + SK + 1);  // the next step's; waited for at its top
    ns = entry(t + SD + 1);
    if (vb1 < BLOCK) mask_ops(vb1, nxt);  // rare: a ragged kv block
  };
  for (int t = 0; t < n; t += UNROLL) {
#pragma unroll
    for (int u = 0; u < UNROLL; u += 2) {
      if (t + u < n) step(t + u, u, x, y);
      if (t + u + 1 < n) step(t + u + 1, u + 1, y, x);
    }
  }
  // no DMA may still be writing this workgroup's LDS when it ends
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));

  // ---- epilogue: dq = bf16(sm_scale * dQ' 2^(ek - es)). acc[qh] element e of this lane is d = 32w +
  // 8(e/4) + 4kh + e%4 and q = 32qh + q(n), n = lane%32, where the record layout puts column
  // n = 16g + c at q = 16(c/8) + 8((c%8)/4) + 4g + c%4 ----
  const int nn = lane & 31;
  const int cq = nn & 15, gq = nn >> 4;
  const int qoff = 16 * (cq >> 3) + 8 * ((cq & 7) >> 2) + 4 * gq + (cq & 3);
  const float sc = p.sm_scale;
  const int32_t* hs = p.scales + (size_t)bh * HEAD_SCALE_WORDS;
  const int oexp = ld_const(hs, SC_EK) - ld_const(hs, SC_ES);
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    bf16* row = dq_blk + (size_t)(32 * qh + qoff) * HEAD_DIM + 32 * w + 4 * kh;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      union {
        bf16 b[4];
        s16x4 s;
      } r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r.b[e] = (bf16)__builtin_ldexpf(acc[qh][4 * c + e] * sc, oexp);
      *(s16x4*)(row + 8 * c) = r.s;
    }
  }
}

void launch_bwd_dq_spill(const BwdParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(bwd_dq_spill_kernel, dim3(p.items_per_xcd * 8), dim3(256), 0, stream, p);
}

}  // namespace vsa
