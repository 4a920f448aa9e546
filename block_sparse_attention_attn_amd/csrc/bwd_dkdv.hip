// bwd_dkdv.hip -- dK and dV of the 64-token block-sparse attention backward on gfx950 (the kv-major
// half of the backward's main step).
//
// What it computes (FastVideo sm_100a backward commit message: one work item per (batch, head,
// kv64 block); launch header argument struct: k2q lists, variable_block_sizes, dk carries
// sm_scale and dv does not; the gradient is the textbook softmax-attention gradient of the
// backward test page's reference): for one item (b, h, kv block j) and every q block i in its
// k2q list,
//     S    = Q_i K_j^T                       (recomputed scores, 64 x 64)
//     P    = exp2(S * scale_log2 - lse_i)     (lse in base-2 "M form"; kv rows >= vbs[j] -> 0)
//     dP   = dO_i V_j^T
//     dS   = P * (dP - Delta_i)
//     dV_j += P^T dO_i,   dK_j += dS^T Q_i
// then dk_j = bf16(sm_scale * dK_j), dv_j = bf16(dV_j). Items with an empty list do no work here:
// the preprocess wrote their zero rows. dQ is computed by the q-major kernel (bwd_dq.hip), so
// this kernel issues no atomics and its results are bitwise reproducible.
//
// Every GEMM runs on fp16 operands (v_mfma_f32_32x32x16_f16): the preprocess's per-head scaled
// copies q16, k16, do16, v converted to v 2^-ev in LDS, P' = P 2^pp and dS' = dS 2^es in
// fp16 (11 significant bits where bf16 has 8). The accumulators hold S' = S 2^-(eq+ek),
// dP' = dP 2^-(eo+ev), dV' = dV 2^(pp-eo) and dK' = dK 2^(es-eq); the epilogue scales back by
// exact powers of two (vsa_kernels.h, HeadScaleWord).
//
// gfx950 design:
//   * one 256-thread workgroup (4 waves, one per SIMD) per item; wave w owns q rows 32*(w&1)..
//     of every q block and kv rows 32*(w>>1).. of the item, so each 64x64x128 GEMM is eight
//     v_mfma_f32_32x32x16_bf16 per wave;
//   * K_j and V_j fragments (the B operands of S and dP) live in registers for the whole item,
//     with padded kv rows zeroed there. They arrive by DMA through LDS like everything else, so
//     every vector memory operation of the kernel is an LDS DMA whose completion is counted by
//     hand;
//   * Q_i, dO_i and the q block's 512-byte statistics record ((pp - lse_i) / c and -Delta'_i,
//     written by the preprocess) stream through a four-stage ring of XOR-swizzled LDS tiles,
//     fetched by global_load_lds_dwordx4 two steps before their first use; one barrier per q
//     block, between the two phases of a step;
//   * the S and dP accumulators start from the record's values, so the MFMAs deliver
//     S' + (pp - lse) / c and dP' - Delta' directly: P' = exp2(c * acc), dS' = P' * acc';
//   * software pipeline across q blocks: phase B of step t runs the S/dP MFMAs of q block t+1
//     interleaved with the exp2/convert work of q block t and its transposed reads; phase C runs
//     the dV/dK MFMAs of q block t interleaved with the row and record reads of q block t+2, so
//     every MFMA's LDS operands were requested a phase before it issues;
//   * P and dS never leave registers: the D layout of S/dP feeds the A operand of dV/dK directly
//     (the contraction index is permuted to match); the partner operands dO_i^T and Q_i^T come
//     from ds_read_b64_tr_b16 transposed reads;
//   * dV and dK are accumulated per q half and the halves are summed through LDS once per item;
//   * work ids map XCD-first: workgroup ids go round-robin over the 8 XCDs, so XCD x runs a
//     contiguous slice of the (ordered) item list -- one head per XCD when B*H = 8 -- and that
//     head's Q/dO traffic stays in one XCD's L2; when the Q/dO of the heads running at once
//     would overflow half of the shared memory-side cache, the slices run in rounds in which
//     XCD pairs share a head (xcd_work_id), so fewer heads are live at a time;
//   * long lists run in q-range chunks, one launch each: the items take the part of their list
//     inside the chunk's q range and carry dK, dV between launches as fp32 partial sums, so the
//     items on an XCD walk one window of q blocks at a time and keep sharing its L2.
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace vsa {

namespace {

constexpr int STAGES = 4;                        // ring depth: stage t%4 holds q block t
constexpr int STAGE_BYTES = 16384;               // one [64][128] tile of 16-bit values
constexpr int LD_BYTES = LD_RECORD_FLOATS * 4;   // one q block's statistics record
constexpr int DMA_PER_BLOCK = 9;                 // vector memory operations per wave per q block
constexpr int STORES_PER_BLOCK = 2;              // dS stores per wave per q block (spill mode)

__device__ __forceinline__ void barrier_lds() {
  // Wait for this wave's LDS traffic, then meet the other waves. Vector memory traffic (the next
  // tiles' DMA) stays in flight across the barrier.
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The same barrier, with `v` (a scalar load's result) required in its register first: the load
// is issued just before and waited for by the barrier's own lgkmcnt(0).
__device__ __forceinline__ void barrier_lds_with(int v) {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::"s"(v) : "memory");
}

}  // namespace

// SPILL: also write each pair's dS tile (bf16, the A operand of the dK GEMM) to the spill buffer
// for the q-major dQ GEMM (bwd_dq_spill.hip).
template <bool SPILL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_dkdv_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) char q_ring[STAGES * STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char do_ring[STAGES * STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) char ld_ring[STAGES * LD_BYTES];

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int wq = w & 1;   // q half of every q block
  const int wk = w >> 1;  // kv half of the item
  const int g = lane >> 5;
  const int l32 = lane & 31;
  const int grp = lane >> 4;  // 16-lane group
  const int t16 = lane & 15;  // lane inside the group

  // XCD-first work id: blockIdx.x % 8 is the XCD the dispatcher sends the workgroup to.
  const int wid = xcd_work_id(p.items_per_xcd, p.kv_rounds);
  if (wid >= p.total_items) return;
  const int item = p.kv_order ? ld_const(p.kv_order, wid) : wid;
  if (item < 0 || item >= p.total_items) return;  // a malformed order entry: skip, never fault
  int n = ld_const(p.k2q_num, item);
  n = n > p.k2q_stride ? p.k2q_stride : n;
  if (n <= 0) return;
  // q-range chunk: this launch takes list positions [start, start + n) and adds to (first: starts)
  // the fp32 partial sums of the chunks before, which the last chunk turns into dk, dv
  int start = 0;
  bool first = true, last = true;
  if (p.nchunks > 0) {
    const int32_t* cb = p.chunk_bounds + (size_t)item * (p.nchunks + 1) + p.chunk;
    int b0 = ld_const(cb, 0), b1 = ld_const(cb, 1);
    b0 = b0 < 0 ? 0 : (b0 > n ? n : b0);
    b1 = b1 < b0 ? b0 : (b1 > n ? n : b1);
    start = b0;
    n = b1 - b0;
    first = p.chunk == 0;
    last = p.chunk == p.nchunks - 1;
    if (n == 0 && !first && !last) return;  // nothing to add, nothing to finish
  }
  const int bh = item / p.nb;
  const int j = item - bh * p.nb;
  const int vb = ld_const(p.vbs, j);
  const size_t head = (size_t)bh * p.S * HEAD_DIM;
  const f16* __restrict__ qh = p.q16 + head;
  const f16* __restrict__ doh = p.do16 + head;
  const int32_t* __restrict__ hs = p.scales + (size_t)bh * HEAD_SCALE_WORDS;
  const float* __restrict__ recs = p.lse_delta + (size_t)bh * p.nb * LD_RECORD_FLOATS;
  const int* __restrict__ list = p.k2q_idx + (size_t)item * p.k2q_stride + start;
  // q block ids outside [0, nb) violate the caller contract; clamp them so no access leaves the
  // tensors (the result is then unspecified, but nothing faults)
  auto clampq = [&](int qb) { return qb < 0 ? 0 : (qb >= p.nb ? p.nb - 1 : qb); };
  auto entry = [&](int t) { return ld_const(list, t < n ? t : n - 1); };  // raw, in the list

  VSA_LDS char* const qr = (VSA_LDS char*)q_ring;
  VSA_LDS char* const dr = (VSA_LDS char*)do_ring;
  VSA_LDS char* const lr = (VSA_LDS char*)ld_ring;
  uint32_t toff[4];
  tile_offsets_wave(toff, lane, w);
  const uint32_t roff = 16 * lane + 128 * w;  // this wave's quarter of a record (lanes 0..7)
  const uint32_t q_lds = lds_addr(qr) + 4096 * w;  // this wave's slices 4w .. 4w+3
  const uint32_t do_lds = lds_addr(dr) + 4096 * w;
  const uint32_t ld_lds = lds_addr(lr) + 128 * w;
  auto issue = [&](int qb, int st) __attribute__((always_inline)) {
    const size_t tile = (size_t)qb * BLOCK * HEAD_DIM;
    dma_tile_pair_rec(qh + tile, doh + tile, recs + (size_t)qb * LD_RECORD_FLOATS, toff, roff,
                      q_lds + st * STAGE_BYTES, do_lds + st * STAGE_BYTES, ld_lds + st * LD_BYTES);
  };

  f32x16 dv_acc[4], dk_acc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    dv_acc[nt] = f32x16{};
    dk_acc[nt] = f32x16{};
  }
  // An empty chunk (first or last of several) only starts or finishes the partial sums.
  if (n > 0) {
    // ---- prologue ----
    // K_j, V_j into stage 3 of the rings; q blocks 0, 1, 2 into stages 0, 1, 2.
    {
      const size_t tile = (size_t)j * BLOCK * HEAD_DIM;
      dma_tile_pair(p.k16 + head + tile, p.v + head + tile, toff, q_lds + 3 * STAGE_BYTES,
                    do_lds + 3 * STAGE_BYTES);
    }
    {
      const int e0 = entry(0), e1 = entry(1), e2 = entry(2);
      issue(clampq(e0), 0);
      issue(clampq(e1), 1);  // (past the end of the list: repeats of the last q block)
      issue(clampq(e2), 2);
    }
    // dS tiles (spill mode): q block t of this item goes to slot kbase[item] + t of its head. A
    // lane stores its 16 dS' values (two f16x8) as one 32-byte record; the records of a wave's
    // 32 kv rows are laid out so that the q-major kernel's transposed reads of two record groups
    // fall on disjoint banks: record (w, g, l32) at ((8w + l32/4) * 256 + 128g + 32(l32%4)) bytes.
    char* ds_item = nullptr;
    int slot0 = 0;
    const uint32_t ds_rec = ((8 * w + (l32 >> 2)) * 256 + 128 * g + 32 * (l32 & 3));
    auto ds_tile = [&](int t) {
      int slot = slot0 + t;
      slot = slot < p.cap ? slot : p.cap - 1;  // inconsistent counts: stay inside the head
      return ds_item + (size_t)slot * (BLOCK * BLOCK * 2);
    };
    if (SPILL) {
      ds_item = (char*)p.ds + (size_t)bh * p.cap * (BLOCK * BLOCK * 2);
      // (chunked spill: the launch's own tiles, numbered from the chunk's slot bases)
      slot0 = ld_const(p.kbase, item) + (p.ds_chunk_local ? 0 : start);
      // Two stores of zeros into q block 0's tile (rewritten at step 0: one wave's stores to one
      // address land in order), so that every wait below counts the same two stores between the
      // DMA groups of consecutive q blocks.
      char* d = ds_tile(0) + ds_rec;
      *(f16x8*)d = f16x8{};
      *(f16x8*)(d + 16) = f16x8{};
    }
    const int e3 = entry(3);
    // K/V and q blocks 0, 1 landed (own DMAs); q block 2's may still be in flight
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(DMA_PER_BLOCK + (SPILL ? STORES_PER_BLOCK : 0)));
    barrier_lds_with(e3);  // ... everyone's
    int raw = entry(4);    // the list entry step 0 fetches; in by step 0's barrier
    // V_j to fp16 (v 2^-ev, exact like the preprocess's copies) in place in LDS, 16 bytes at a
    // time, then meet again. (Converting the register fragments instead keeps more registers live
    // through the main loop.)
    {
      const int ev = ld_const(hs, SC_EV);
      VSA_LDS bf16x8* vt = (VSA_LDS bf16x8*)(dr + 3 * STAGE_BYTES);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int idx = c * 256 + (int)threadIdx.x;
        const bf16x8 x = vt[idx];
        *(VSA_LDS f16x8*)&vt[idx] = bf16x8_to_f16x8(x, ev);
      }
      barrier_lds();
    }

    // B operand of S = Q K^T and dP = dO V^T: lane holds kv row 32*wk + l32, d = 16*s + 8*g + 0..7
    const int kv_l = 32 * wk + l32;
    const bool kv_valid = kv_l < vb;
    f16x8 kf[8], vf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int b = 3 * STAGE_BYTES + tile_byte(kv_l, 2 * s + g);
      kf[s] = *(const VSA_LDS f16x8*)(qr + b);
      vf[s] = *(const VSA_LDS f16x8*)(dr + b);
    }
    if (!kv_valid) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        kf[s] = f16x8{};
        vf[s] = f16x8{};
      }
    }

    const float cexp = __uint_as_float((uint32_t)ld_const(hs, SC_C));
    const int qrow = 32 * wq + l32;

    // A operands of S = Q K^T and dP = dO V^T for the q block in stage st: q rows 32*wq + l32,
    // d = 16*s + 8*g + 0..7
    f16x8 qa[8], da[8];
    auto load_rows = [&](int st, int sb) __attribute__((always_inline)) {  // steps sb .. sb+3
      VSA_LDS char* qt = qr + st * STAGE_BYTES;
      VSA_LDS char* dt = dr + st * STAGE_BYTES;
#pragma unroll
      for (int s = sb; s < sb + 4; ++s) {
        qa[s] = *(const VSA_LDS f16x8*)(qt + tile_byte(qrow, 2 * s + g));
        da[s] = *(const VSA_LDS f16x8*)(dt + tile_byte(qrow, 2 * s + g));
      }
    };
    // Initial accumulators of the q block in stage st from its record: element i of S / dP is
    // q row 32*wq + 8*(i/4) + 4*g + i%4.
    auto load_init = [&](int st, f32x16& sa_, f32x16& pa_) __attribute__((always_inline)) {
      const VSA_LDS float* ld = (const VSA_LDS float*)(lr + st * LD_BYTES);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int q = 32 * wq + 8 * c + 4 * g;
        const f32x4 a = *(const VSA_LDS f32x4*)(ld + q);
        const f32x4 b = *(const VSA_LDS f32x4*)(ld + BLOCK + q);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sa_[4 * c + e] = a[e];
          pa_[4 * c + e] = b[e];
        }
      }
    };

    // LDS byte addresses of the transposed reads below, one per (column group nt, row half h) and
    // ring: the q half (16 rows), the stage and the ring base differ only by constants, which the
    // reads carry as immediate offsets (the empty asm keeps the compiler from re-deriving the dO
    // addresses from the Q ones, which would cost an add per read: the dO ring starts at 64 KiB,
    // past the reach of an immediate).
    uint32_t trq[4][2], trd[4][2];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int off = tile_elem_byte(32 * wq + 4 * (grp >> 1) + (t16 >> 2) + 8 * h,
                                       32 * nt + 16 * (grp & 1) + 4 * (t16 & 3));
        trq[nt][h] = lds_addr(qr) + off;
        trd[nt][h] = lds_addr(dr) + off;
        asm volatile("" : "+v"(trq[nt][h]), "+v"(trd[nt][h]));
      }
    }
    auto rd_tr = [](uint32_t a) { return lds_read_tr((const VSA_LDS void*)(uintptr_t)a); };

    f32x16 s0, p0, s1, p1;
    load_rows(0, 0);
    load_rows(0, 4);
    load_init(0, s0, p0);
    barrier_lds();  // everyone has read K/V out of stage 3
    // q block 3's record and Q tile; step 0's phase B issues its dO tile (see the step below)
    {
      const int qb3 = clampq(e3);
      dma_rec128(recs + (size_t)qb3 * LD_RECORD_FLOATS, roff, ld_lds + 3 * LD_BYTES);
      dma_tile(qh + (size_t)qb3 * BLOCK * HEAD_DIM, toff, q_lds + 3 * STAGE_BYTES);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      s0 = mfma32_f16(qa[s], kf[s], s0);
      p0 = mfma32_f16(da[s], vf[s], p0);
    }
    load_rows(1, 0);  // a repeat of q block 0 when n == 1
    load_rows(1, 4);
    load_init(1, s1, p1);

    // Step t (q block t in stage st = t % 4): on entry (sc, pc) hold S' + (pp - lse) / c and
    // dP' - Delta' of q block t, (sn, pn) the initial values of q block t+1 and (qa, da) its rows.
    //   phase B: the dO DMA of q block t+3, then the S/dP MFMAs of t+1, interleaved with the
    //            transposed dO^T, Q^T reads of t and P, dS of t;
    //   mid:     q block t+2 has landed (own DMAs, then the barrier: everyone's) and everyone is
    //            done with stage st, which then receives q block t+4;
    //   phase C: dV/dK MFMAs of t, interleaved with the record and row reads of t+2 into (sc, pc)
    //            and (qa, da) and the record and Q DMAs of q block t+4.
    // The last steps compute throwaway S/dP from repeated q blocks, which keeps the body free of
    // branches. The loop is unrolled by four so stage offsets are constants.
    int qb_carry = clampq(e3);  // the q block whose dO tile the next phase B fetches
    auto step = [&](int t, int st, f32x16& sc, f32x16& pc, f32x16& sn, f32x16& pn)
                    __attribute__((always_inline)) {
      const int st2 = (st + 2) & 3;
      // dO tile of q block t+3 into stage (t+3)%4, the second half of the DMA group whose record
      // and Q tile phase C of the previous step issued (both after the barrier that freed the
      // stage). Issued here, ahead of the transposed reads, it spreads the group's nine operations
      // over two phases; all of phase C it costs about 1 % more.
      dma_tile(doh + (size_t)qb_carry * BLOCK * HEAD_DIM, toff,
               do_lds + ((st + 3) & 3) * STAGE_BYTES);

      // ---- phase B ----
      // transposed B operands of dV/dK for q block t: k slot jj of step s2 is q row
      // 32*wq + 16*s2 + 8*(jj/4) + 4*g + jj%4, matching the D layout of S
      f16x8 db[2][4], qbt[2][4];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const uint32_t o = st * STAGE_BYTES + s2 * 16 * 256;  // stage, then 16 rows further down
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          db[s2][nt] = join_f16(rd_tr(trd[nt][0] + o), rd_tr(trd[nt][1] + o));
          qbt[s2][nt] = join_f16(rd_tr(trq[nt][0] + o), rd_tr(trq[nt][1] + o));
        }
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        sn = mfma32_f16(qa[s], kf[s], sn);
        pn = mfma32_f16(da[s], vf[s], pn);
      }
      // P' and dS' of q block t, half h (elements 8h .. 8h+7: q rows 32*wq + 16h + ..) in fp16. A
      // padded kv column (zero K/V fragment) gets some finite or non-finite P'; it only feeds that
      // kv row of dV/dK, which the epilogue overwrites with 0.
      f16x8 pa[2], sa[2];
      auto softmax_half = [&](int h) __attribute__((always_inline)) {
        float pv[8], dsv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(sc[8 * h + e] * cexp);
          dsv[e] = pv[e] * pc[8 * h + e];
        }
        pa[h] = pack8_f16(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
        sa[h] = pack8_f16(dsv[0], dsv[1], dsv[2], dsv[3], dsv[4], dsv[5], dsv[6], dsv[7]);
      };
      // Under the S/dP MFMAs; the empty asm keeps this arithmetic in this phase (it is otherwise
      // free to sink next to its use after the barrier).
      softmax_half(0);
      softmax_half(1);
      asm volatile("" : "+v"(pa[0]), "+v"(sa[0]), "+v"(pa[1]), "+v"(sa[1]));
      // (three VALU per MFMA, the rest of the softmax after them: 1.2 % faster than five per MFMA
      // in the same GPU call; one, two or four were no better)
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two transposed reads
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // three VALU
      }
      __builtin_amdgcn_sched_barrier(0);

      // ---- mid ----
      // Every step issues one q block's DMA group (past the end of the list: a repeat of the last
      // q block, into a stage nobody reads again), so the group of t+3 is always the newest and
      // nine outstanding operations mean q block t+2 has landed: the group of t+2 ends with its dO
      // tile (phase B of step t-1), and after it come the record, Q and dO of t+3. No branch splits
      // the step. (In spill mode the two dS stores of step t-1 sit between the groups of t+2 and
      // t+3.)
      // The list entry of q block t+4 was loaded after the previous barrier; the compiler-visible
      // lgkmcnt(0) tells the compiler that every LDS read issued so far is complete, so the scalar
      // load issued below for the next step adds no wait for them.
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(DMA_PER_BLOCK + (SPILL ? STORES_PER_BLOCK : 0)));
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
      // The dS tile of q block t (spill mode) goes out here, between this wave's wait and the
      // barrier, where the wave would otherwise idle until the others arrive; stores issued inside
      // phase C delay its MFMAs and DMAs.
      if (SPILL) {  // streamed past the caches: read once, by the q-major kernel
        char* d = ds_tile(t) + ds_rec;
        __builtin_nontemporal_store(sa[0], (f16x8*)d);
        __builtin_nontemporal_store(sa[1], (f16x8*)(d + 16));
      }
      barrier_lds_with(raw);  // ... everyone's; everyone is done with stage st
      const int qb = clampq(raw);
      qb_carry = qb;
      raw = entry(t + 5);     // in by the next step's barrier

      // ---- phase C ----
      // dV/dK MFMAs of t. Record and row reads of q block t+2 (records first: they seed the first
      // MFMAs of the next step), with q block t+4's record and Q tile DMAs into stage st placed
      // between them: the asm blocks keep their order relative to the reads, so the DMAs spread
      // over the phase instead of reaching the address unit together.
      {
        const size_t tile = (size_t)qb * BLOCK * HEAD_DIM;
        load_init(st2, sc, pc);
        dma_rec128(recs + (size_t)qb * LD_RECORD_FLOATS, roff, ld_lds + st * LD_BYTES);
        load_rows(st2, 0);
        dma_tile(qh + tile, toff, q_lds + st * STAGE_BYTES);
        load_rows(st2, 4);
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        dv_acc[nt] = mfma32_f16(pa[0], db[0][nt], dv_acc[nt]);
        dk_acc[nt] = mfma32_f16(sa[0], qbt[0][nt], dk_acc[nt]);
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        dv_acc[nt] = mfma32_f16(pa[1], db[1][nt], dv_acc[nt]);
        dk_acc[nt] = mfma32_f16(sa[1], qbt[1][nt], dk_acc[nt]);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // three record / row reads
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int t = 0; t < n; t += 4) {
      step(t, 0, s0, p0, s1, p1);
      if (t + 1 < n) step(t + 1, 1, s1, p1, s0, p0);
      if (t + 2 < n) step(t + 2, 2, s0, p0, s1, p1);
      if (t + 3 < n) step(t + 3, 3, s1, p1, s0, p0);
    }
  }  // n > 0

  // ---- sum the two q halves of dV/dK through LDS, scale, round, store ----
  // the repeats issued by the last four steps are still in flight: wait, then meet
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  barrier_lds();  // every wave is past its last LDS read of the rings
  // wave wq=1 hands over its dV half, wave wq=0 its dK half (16 KiB each, lane-native order);
  // kv half 0 uses the first two q stages, kv half 1 the first two dO stages
  VSA_LDS char* xbase = wk == 0 ? qr : dr;
  VSA_LDS f32x4* dv_x = (VSA_LDS f32x4*)xbase;
  VSA_LDS f32x4* dk_x = (VSA_LDS f32x4*)(xbase + STAGE_BYTES);
  VSA_LDS f32x4* mine_out = wq == 1 ? dv_x : dk_x;
  VSA_LDS f32x4* theirs = wq == 1 ? dk_x : dv_x;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x16& src = wq == 1 ? dv_acc[nt] : dk_acc[nt];
      mine_out[(nt * 4 + c) * 64 + lane] = f32x4{src[4 * c], src[4 * c + 1], src[4 * c + 2], src[4 * c + 3]};
    }
  }
  barrier_lds();
  bf16* outp = (wq == 0 ? p.dv : p.dk) + head + (size_t)j * BLOCK * HEAD_DIM;
  // dv = dV' 2^(eo - pp), dk = sm_scale dK' 2^(eq - es)
  const float oscale = wq == 0 ? 1.0f : p.sm_scale;
  const int oexp = wq == 0 ? ld_const(hs, SC_EO) - ld_const(hs, SC_PP)
                           : ld_const(hs, SC_EQ) - ld_const(hs, SC_ES);
  // this wave's tensor (dV for wq 0, dK for wq 1) in the chunk partial sums: [64][128] fp32
  float* part = p.part ? p.part + ((size_t)item * 2 + wq) * (BLOCK * HEAD_DIM) : nullptr;
  // the chunks before: all of this lane's partial sums are loaded before any store below (a
  // store to the partial sums may alias a later load, which would otherwise wait for it: one
  // memory round trip per group of four)
  float prev[4][4][4];
  if (!first) {
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          prev[nt][c][e] = part[(32 * wk + 8 * c + 4 * g + e) * HEAD_DIM + 32 * nt + l32];
  }
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int d = 32 * nt + l32;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f32x4 o = theirs[(nt * 4 + c) * 64 + lane];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float mine = wq == 0 ? dv_acc[nt][4 * c + e] : dk_acc[nt][4 * c + e];
        const int kv = 32 * wk + 8 * c + 4 * g + e;
        float sum = mine + o[e];
        if (!first) sum += prev[nt][c][e];
        if (last)  // padded kv rows are exactly zero by definition
          outp[(size_t)kv * HEAD_DIM + d] =
              kv < vb ? (bf16)__builtin_ldexpf(sum * oscale, oexp) : (bf16)0.0f;
        else
          part[kv * HEAD_DIM + d] = sum;
      }
    }
  }
}

void launch_bwd_dkdv(const BwdParams& p, hipStream_t stream) {
  if (p.ds)
    hipLaunchKernelGGL(bwd_dkdv_kernel<true>, dim3(p.items_per_xcd * 8), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(bwd_dkdv_kernel<false>, dim3(p.items_per_xcd * 8), dim3(256), 0, stream, p);
}

}  // namespace vsa
