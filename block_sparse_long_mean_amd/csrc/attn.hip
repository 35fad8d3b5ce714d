// Exact softmax attention over the selected blocks.
//
// "MiniMax released MSA ..." (news.hamidun.com), sections "How MSA Works" and
// "Why Long Context is Hard to Scale": the main branch attends exactly, with
// no approximation, over only the selected blocks.  One softmax spans all
// selected keys of a query; it is evaluated block by block with running
// (max, sum) statistics and merged with log-sum-exp weights, which is exact
// up to rounding.
//
// Schedule (bf16):
//  * attn_gather: KV-major.  A work item is one (b, kv head, block) bucket and
//    a tile of up to 128 query rows that chose it (the causal own block is one
//    of the chosen blocks, attended with the per-key causal mask).  The
//    block's keys and values are staged in LDS (V transposed) in 64-key tiles
//    and kept there across consecutive items of the same bucket; each wave
//    holds 32 gathered query rows.  S^T = K Q^T and O^T += V^T P^T run on
//    v_mfma_f32_32x32x16_bf16 with fp32 accumulation; the result per
//    (row, slot) is an unnormalised partial output sum_k p_k v_k (bf16) with
//    p_k = 2^(s_k * scale * log2(e) - m) and its pair (m, l = sum_k p_k) in
//    fp32.  Persistent workgroups walk contiguous item ranges and prefetch
//    the next item's row metadata and queries during the current item's
//    MFMAs.
//  * attn_merge: streaming.  D/8 lanes per output row read the row's
//    partials (8 head dims each), merge them with weights 2^(m_s - max m)
//    and write o (and lse).
#include <math.h>

#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

constexpr int KT = 64;  // keys per LDS tile
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr int VTS = KT + 4;  // V^T row stride: 136 bytes keeps 16 lanes' 8-byte reads on distinct banks

template <int D>
struct AttnSmem {
  uint16_t k[KT * (D + 8)];
  uint16_t vt[D * VTS];
};

// Per-wave LDS staging area, used twice per work item:
//  * the next item's query rows: for each 16-column chunk s, lane l's 16
//    bytes land at elements [(s*64 + l)*8, +8) (global_load_lds_dwordx4
//    writes lane l's data at the wave's LDS base + 16*l);
//  * the finished partial outputs, row-major with rows padded by 8 bytes, so
//    that every global store instruction writes whole 256-byte rows.
template <int D, int W>
struct QStage {
  static constexpr int QELEMS = (D / 16) * 64 * 8;
  static constexpr int RS = D + 4;  // padded output row (bf16 elements)
  static constexpr int OELEMS = 32 * RS;
  static constexpr int ELEMS = QELEMS > OELEMS ? QELEMS : OELEMS;
  uint16_t buf[W][ELEMS];
  int64_t dst[W][32];  // destination element offset of each of the wave's 32 rows
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// LDS reads of the staged key / value tiles go through inline asm that waits
// for its own data inside the same asm block.  While a global_load_lds copy
// of the next item's queries is in flight, the compiler cannot tell these
// reads from that copy's LDS area and would make each of them wait for the
// copy (and, in order, for every vector store issued before it).  Each block
// issues the reads of two (keys) or four (values) MFMA steps from one base
// address with immediate offsets, so that their latencies overlap.
typedef const __attribute__((address_space(3))) void* lds_cptr_t;
BSA_DEV uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)(lds_cptr_t)p; }

// Work-item records are read-only while the gather runs: reading them through
// the constant address space makes them scalar loads, whose wait does not
// also wait for the partial-output stores still in flight (vector memory
// operations complete in order).
typedef const __attribute__((address_space(4))) int* const_int_ptr;
BSA_DEV int4 load_item(const_int_ptr items, int i) {
  return make_int4(items[4 * i], items[4 * i + 1], items[4 * i + 2], items[4 * i + 3]);
}
// Entry word of a lane's row for the item whose entries start at e_item.
// With R >= 4 rows per entry a wave's 32 rows use at most 8 entries: they are
// read with scalar loads (a wave-uniform address) and each lane picks its
// own, so waiting for them does not wait for the vector stores in flight;
// otherwise (R < 4) each lane loads its entry.
template <bool SCALAR>
BSA_DEV uint32_t next_entry(const uint32_t* entries, int e_item, int wave, int lane, int lgR) {
  if constexpr (SCALAR) {
    const const_int_ptr ents = (const const_int_ptr)entries;
    const int e0 = e_item + ((wave * 32) >> lgR);
    const int sel = (lane & 31) >> lgR;
    int v = ents[e0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
      const int x = ents[e0 + i];
      v = sel == i ? x : v;
    }
    return (uint32_t)v;
  }
  return entries[e_item + ((wave * 32 + (lane & 31)) >> lgR)];
}

template <int D, int W>
BSA_DEV void prefetch_q_lds(QStage<D, W>& st, const uint16_t* qrow, bool ok) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (ok) {
    // byte offset of the lane's half row, 16 * (lane >> 5): derived here, in
    // asm, so that it is not held live (and spilled) across the item loop
    uint32_t hb;
    asm volatile("v_and_b32 %0, 32, %1\n\tv_lshrrev_b32 %0, 1, %0" : "=v"(hb) : "v"(lane_id()));
    const char* src = reinterpret_cast<const char*>(qrow) + hb;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      __builtin_amdgcn_global_load_lds((const void*)(src + 32 * s), (lds_ptr_t)(&st.buf[w][s * 64 * 8]), 16, 0, 0);
  }
}

// Rows past the item's end read whatever the staging area holds; their
// result columns are never stored.
template <int D, int W>
BSA_DEV void read_q_lds(const QStage<D, W>& st, bf16x8 (&qf)[D / 16]) {
  const int w = threadIdx.x >> 6, l = lane_id();
#pragma unroll
  for (int s = 0; s < D / 16; ++s) qf[s] = as_bf(*reinterpret_cast<const u16x8*>(&st.buf[w][(s * 64 + l) * 8]));
}

// O^T tile of the wave's 32 rows -> bf16 rows in LDS -> global:
// D/8 lanes write one row's D elements (16 bytes each), 64*8/D rows per
// store instruction.  Rows [nvalid, 32) of the wave are not written; row r's
// destination element offset is held by lane r.
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));

template <int D>
BSA_DEV void pack_partials(const f32x16 (&o)[D / 32], u16x4_t (&pk)[D / 8]) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int gg = 0; gg < 4; ++gg)
      pk[dt * 4 + gg] = u16x4_t{f2bf(o[dt][4 * gg]), f2bf(o[dt][4 * gg + 1]), f2bf(o[dt][4 * gg + 2]),
                                f2bf(o[dt][4 * gg + 3])};
}

// Stores rows N*RPI + lr (N = 0..NMAX-1) of the wave's staged partial rows:
// the LDS reads (destination offset, 16 bytes of the row) go through asm with
// immediate offsets from two base addresses, so the stores of earlier rows
// stay in flight (see the key / value tile reads).
template <int N, int NMAX, int RPI, int RS>
BSA_DEV void store_rows(uint32_t dst_base, uint32_t row_base, int lr, int nvalid, uint16_t* part_o) {
  if constexpr (N < NMAX) {
    if (N * RPI + lr < nvalid) {
      int64_t dst;
      u16x4_t a, b;
      asm volatile(
          "ds_read_b64 %0, %3 offset:%5\n\tds_read_b64 %1, %4 offset:%6\n\tds_read_b64 %2, %4 offset:%7\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=v"(dst), "=v"(a), "=v"(b)
          : "v"(dst_base), "v"(row_base), "n"(N * RPI * 8), "n"(N * RPI * RS * 2), "n"(N * RPI * RS * 2 + 8)
          : "memory");
      const u16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      // streaming store: partials are read once, by the merge, long after
      __builtin_nontemporal_store(v, reinterpret_cast<u16x8*>(part_o + dst));
    }
    store_rows<N + 1, NMAX, RPI, RS>(dst_base, row_base, lr, nvalid, part_o);
  }
}

template <int D, int W>
BSA_DEV void store_partials(QStage<D, W>& st, const u16x4_t (&pk)[D / 8], int64_t dst_mine, int nvalid,
                            uint16_t* part_o) {
  const int w = threadIdx.x >> 6, lane = lane_id(), r = lane & 31, h = lane >> 5;
  constexpr int RS = QStage<D, W>::RS;
  uint16_t* sb = st.buf[w];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) *reinterpret_cast<u16x4_t*>(sb + r * RS + dt * 32 + 8 * gg + 4 * h) = pk[dt * 4 + gg];
  if (h == 0) st.dst[w][r] = dst_mine;
  __builtin_amdgcn_wave_barrier();
  constexpr int CPR = D / 8, RPI = 64 / CPR;
  const int c = lane % CPR, lr = lane / CPR;
  store_rows<0, 32 / RPI, RPI, RS>(lds_addr(&st.dst[w][lr]), lds_addr(sb + lr * RS + c * 8), lr, nvalid,
                                    part_o + c * 8);
}

// Stage keys [key0, key0 + KT) of one kv head (zero past n_valid) into LDS:
// K row-major, V transposed.
template <int D, int NT>
BSA_DEV void stage_kv(AttnSmem<D>& sm, const uint16_t* kb, int64_t ks_t, const uint16_t* vb, int64_t vs_t,
                      int key0, int n_valid) {
  const int tid = threadIdx.x;
  constexpr int CH = D / 8;
  for (int idx = tid; idx < KT * CH; idx += NT) {
    const int kr = idx / CH, ch = idx % CH;
    u16x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
    if (kr < n_valid) x = ld16(kb + (int64_t)(key0 + kr) * ks_t + ch * 8);
    st16(&sm.k[kr * (D + 8) + ch * 8], x);
  }
  // V: a thread takes 4 consecutive keys x 8 head dims and writes them
  // transposed; consecutive lanes take consecutive key quads so that their
  // LDS writes of one V^T row are contiguous
  for (int idx = tid; idx < (KT / 4) * CH; idx += NT) {
    const int kq = idx % (KT / 4), ch = idx / (KT / 4);
    u16x8 r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kr = kq * 4 + i;
      r[i] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (kr < n_valid) r[i] = ld16(vb + (int64_t)(key0 + kr) * vs_t + ch * 8);
    }
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      u16x4 col = {r[0][d], r[1][d], r[2][d], r[3][d]};
      *reinterpret_cast<u16x4*>(&sm.vt[(ch * 8 + d) * VTS + kq * 4]) = col;
    }
  }
}

// Blocks longer than one key tile: the next tile's keys and values are
// copied global -> LDS by DMA in their natural layout (rows of D elements)
// while the current tile is computed, then repacked LDS -> LDS into the
// padded key rows and the transposed values the MFMA reads.  Rows past
// n_valid copy row 0 of the tile (in bounds); the repack zeroes them.
template <int D, int NT>
BSA_DEV void dma_kv(uint16_t* nat, const uint16_t* kb, int64_t ks_t, const uint16_t* vb, int64_t vs_t, int key0,
                    int n_valid) {
  constexpr int CPR = D / 8;       // 16-byte pieces per row
  constexpr int RPI = 64 / CPR;    // rows per DMA instruction (64 lanes x 16 bytes)
  constexpr int NW = NT / 64;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  const int r_in = lane / CPR, c = lane % CPR;
  for (int i = w; i < KT / RPI; i += NW) {
    const int r = i * RPI + r_in;
    const int rr = r < n_valid ? r : 0;
    __builtin_amdgcn_global_load_lds((const void*)(kb + (int64_t)(key0 + rr) * ks_t + c * 8),
                                     (lds_ptr_t)(nat + i * RPI * D), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((const void*)(vb + (int64_t)(key0 + rr) * vs_t + c * 8),
                                     (lds_ptr_t)(nat + KT * D + i * RPI * D), 16, 0, 0);
  }
}

template <int D, int NT>
BSA_DEV void repack_kv(AttnSmem<D>& sm, const uint16_t* nat, int n_valid) {
  const int tid = threadIdx.x;
  constexpr int CH = D / 8;
  for (int idx = tid; idx < KT * CH; idx += NT) {
    const int kr = idx / CH, ch = idx % CH;
    u16x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
    if (kr < n_valid) x = *reinterpret_cast<const u16x8*>(nat + kr * D + ch * 8);
    st16(&sm.k[kr * (D + 8) + ch * 8], x);
  }
  // values transposed as stage_kv writes them
  for (int idx = tid; idx < (KT / 4) * CH; idx += NT) {
    const int kq = idx % (KT / 4), ch = idx / (KT / 4);
    u16x8 r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kr = kq * 4 + i;
      r[i] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (kr < n_valid) r[i] = *reinterpret_cast<const u16x8*>(nat + KT * D + kr * D + ch * 8);
    }
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      u16x4 col = {r[0][d], r[1][d], r[2][d], r[3][d]};
      *reinterpret_cast<u16x4*>(&sm.vt[(ch * 8 + d) * VTS + kq * 4]) = col;
    }
  }
}

// Score steps S and S+1 (head dims 16S .. 16S+31) of qk_tile, then the rest.
// base = LDS byte address of this lane's 16 bytes in key row r, step 0.
template <int S, int D>
BSA_DEV void qk_steps(uint32_t base, const bf16x8 (&qf)[D / 16], f32x16& s0, f32x16& s1) {
  if constexpr (S < D / 16) {
    constexpr int R32 = 32 * (D + 8) * 2;  // byte distance from key row r to r + 32
    u16x8 a0, a1, b0, b1;
    asm volatile(
        "ds_read_b128 %0, %4 offset:%5\n\tds_read_b128 %1, %4 offset:%6\n\t"
        "ds_read_b128 %2, %4 offset:%7\n\tds_read_b128 %3, %4 offset:%8\n\ts_waitcnt lgkmcnt(0)"
        : "=v"(a0), "=v"(a1), "=v"(b0), "=v"(b1)
        : "v"(base), "n"(S * 32), "n"(R32 + S * 32), "n"(S * 32 + 32), "n"(R32 + S * 32 + 32)
        : "memory");
    s0 = mfma32(as_bf(a0), qf[S], s0);
    s1 = mfma32(as_bf(a1), qf[S], s1);
    s0 = mfma32(as_bf(b0), qf[S + 1], s0);
    s1 = mfma32(as_bf(b1), qf[S + 1], s1);
    qk_steps<S + 2, D>(base, qf, s0, s1);
  }
}

// S^T (64 keys x 32 queries) for this wave: s0 keys 0..31, s1 keys 32..63.
template <int D>
BSA_DEV void qk_tile(const AttnSmem<D>& sm, const bf16x8 (&qf)[D / 16], f32x16& s0, f32x16& s1) {
  const int lane = lane_id();
  const int r = lane & 31, h = lane >> 5;
  s0 = f32x16{};
  s1 = f32x16{};
  qk_steps<0, D>(lds_addr(&sm.k[r * (D + 8) + 8 * h]), qf, s0, s1);
}

// Head-dim tile DT (rows 32 DT + r of V^T) of pv_tile over the tile's 64
// keys, then the rest.  base = LDS byte address of V^T row r, key 4h.
template <int DT, int D>
BSA_DEV void pv_steps(uint32_t base, const bf16x8 (&pb)[4], f32x16 (&o)[D / 32], bool first) {
  if constexpr (DT < D / 32) {
    constexpr int OFF = DT * 32 * VTS * 2;
    u16x4 x0, x1, x2, x3, x4, x5, x6, x7;
    // keys 16kk + 4h .. +3 and 16kk + 8 + 4h .. +3 for kk = 0..3
    asm volatile(
        "ds_read_b64 %0, %8 offset:%9\n\tds_read_b64 %1, %8 offset:%10\n\t"
        "ds_read_b64 %2, %8 offset:%11\n\tds_read_b64 %3, %8 offset:%12\n\t"
        "ds_read_b64 %4, %8 offset:%13\n\tds_read_b64 %5, %8 offset:%14\n\t"
        "ds_read_b64 %6, %8 offset:%15\n\tds_read_b64 %7, %8 offset:%16\n\ts_waitcnt lgkmcnt(0)"
        : "=v"(x0), "=v"(x1), "=v"(x2), "=v"(x3), "=v"(x4), "=v"(x5), "=v"(x6), "=v"(x7)
        : "v"(base), "n"(OFF), "n"(OFF + 16), "n"(OFF + 32), "n"(OFF + 48), "n"(OFF + 64), "n"(OFF + 80),
          "n"(OFF + 96), "n"(OFF + 112)
        : "memory");
    const u16x8 a0 = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    const u16x8 a1 = {x2[0], x2[1], x2[2], x2[3], x3[0], x3[1], x3[2], x3[3]};
    const u16x8 a2 = {x4[0], x4[1], x4[2], x4[3], x5[0], x5[1], x5[2], x5[3]};
    const u16x8 a3 = {x6[0], x6[1], x6[2], x6[3], x7[0], x7[1], x7[2], x7[3]};
    o[DT] = first ? mfma32(as_bf(a0), pb[0], f32x16{}) : mfma32(as_bf(a0), pb[0], o[DT]);
    o[DT] = mfma32(as_bf(a1), pb[1], o[DT]);
    o[DT] = mfma32(as_bf(a2), pb[2], o[DT]);
    o[DT] = mfma32(as_bf(a3), pb[3], o[DT]);
    pv_steps<DT + 1, D>(base, pb, o, first);
  }
}

// O^T (D x 32 queries) += V^T P^T for one 64-key tile; p0/p1 hold P^T in the
// S^T result layout.  With `first` the accumulators start from zero.  The
// tile's per-query sum of the (bf16) probabilities -- the same weights the
// product uses -- comes from four more MFMAs with an all-ones A operand and is
// added to l.
template <int D>
BSA_DEV void pv_tile(const AttnSmem<D>& sm, const f32x16& p0, const f32x16& p1, f32x16 (&o)[D / 32], bool first,
                     float& l) {
  const int lane = lane_id();
  const int r = lane & 31, h = lane >> 5;
  bf16x8 pb[4];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    pb[0][e] = (__bf16)p0[e];
    pb[1][e] = (__bf16)p0[8 + e];
    pb[2][e] = (__bf16)p1[e];
    pb[3][e] = (__bf16)p1[8 + e];
  }
  {
    const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                         (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
    f32x16 rsum = mfma32(ones, pb[0], f32x16{});
#pragma unroll
    for (int kk = 1; kk < 4; ++kk) rsum = mfma32(ones, pb[kk], rsum);
    l += rsum[0];
  }
  pv_steps<0, D>(lds_addr(&sm.vt[r * VTS + 4 * h]), pb, o, first);
}

// key index (within a 64-key tile) held by result register i of this lane
BSA_DEV int krow(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// Online-softmax update of one lane's query column.  s0/s1 hold raw scores
// (masked entries already -inf); sl2 = softmax scale * log2(e) is applied
// inside the exponent.  On return s0/s1 hold the probabilities P (0 where
// masked) and the running sum l and accumulators o are rescaled to the new
// max; the tile's own sum of P is added by pv_tile.  `first` skips rescaling
// the still-zero state.
template <int D>
BSA_DEV void softmax_update(f32x16& s0, f32x16& s1, float& m, float& l, f32x16 (&o)[D / 32], float sl2,
                            bool first) {
  float tmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, fmaxf(s0[i], s1[i]));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
  const float mnew = fmaxf(m, tmax * sl2);
  if (mnew == -INFINITY) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = 0.f;
      s1[i] = 0.f;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    s0[i] = __builtin_amdgcn_exp2f(fmaf(s0[i], sl2, -mnew));
    s1[i] = __builtin_amdgcn_exp2f(fmaf(s1[i], sl2, -mnew));
  }
  if (!first) {
    const float corr = __builtin_amdgcn_exp2f(m - mnew);
    l *= corr;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] *= corr;
  }
  m = mnew;
}

template <int D>
BSA_DEV void load_qf(const uint16_t* qrow, bool ok, bf16x8 (&qf)[D / 16]) {
  const int h = lane_id() >> 5;
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u16x8 x = {0, 0, 0, 0, 0, 0, 0, 0};
    if (ok) x = ld16(qrow + 16 * s + 8 * h);
    qf[s] = as_bf(x);
  }
}

// ---------------------------------------------------------------------------
// Row metadata of one lane's query row in a work item.  An item record holds
// {bucket, first entry, rows, tile}; lr is the row's index inside the item.
struct GRow {
  int t, slot, qh, hs, rr;
  int valid;  // an int, not a bool: a padded struct's copy keeps a private-memory temporary
};

// raw entry word of row lr of item `rec` (speculative load guarded by validity)
BSA_DEV uint32_t entry_of(const AttnParams& p, int4 rec, int lr) {
  return lr < rec.z ? p.entries[rec.y + (lr >> p.lgR)] : 0u;
}

// entry word = slot | head-in-group << sh_h | token << sh_t; record w = b << 16 | hk
BSA_DEV GRow grow_of(const AttnParams& p, int4 rec, uint32_t ent, int lr) {
  GRow g;
  const int hk = rec.w & 0xFFFF;
  g.valid = lr < rec.z;
  g.rr = g.valid ? lr & ((1 << p.lgR) - 1) : 0;
  g.slot = (int)(ent & ((1u << p.sh_h) - 1u));
  const int hh = (int)((ent >> p.sh_h) & ((1u << (p.sh_t - p.sh_h)) - 1u));
  g.t = g.valid ? (int)(ent >> p.sh_t) : 0;
  g.qh = p.per_group ? hk * p.G + g.rr : hk * p.G + hh;
  g.hs = p.per_group ? hk : hk * p.G + hh;
  return g;
}

template <int D>
BSA_DEV const uint16_t* q_row(const AttnParams& p, int4 rec, const GRow& g) {
  const int b = rec.w >> 16;
  return p.q + (int64_t)b * p.qs_b + (int64_t)g.t * p.qs_t + (int64_t)g.qh * p.qs_h;
}

// Software pipeline per workgroup (its sequence of items): the next item's
// record and entry word are loaded at the top of the current item, and its
// queries are staged global -> LDS after the current item's first score
// tile, to be read back once the current item's last PV tile is issued.
// SE: entry words through scalar loads (requires R >= 4)
template <int D, int W, bool SE>
__global__ __launch_bounds__(64 * W, 8 / W) void attn_gather_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) AttnSmem<D> sm;
  __shared__ __attribute__((aligned(16))) QStage<D, W> qst;
  // natural-layout keys + values of the next tile (blocks longer than a tile)
  __shared__ __attribute__((aligned(16))) uint16_t s_nat[W == 8 ? 2 * KT * D : 8];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hq = lane >> 5;
  // work items of this launch's chunks (buckets c0*Nb .. c1*Nb)
  const int it_lo = p.tile_off[(int64_t)p.c0 * p.Nb];
  const int nitems = p.tile_off[(int64_t)p.c1 * p.Nb] - it_lo;
  // XCD x owns items [off_x, end_x); its workgroups take runs of run_items
  // consecutive items round-robin, so that at any time the XCD works on a
  // narrow window of buckets (one query chunk: its query rows are re-read
  // by every block they chose, from the memory-side cache while the window
  // stays on the chunk) and consecutive items of a run mostly share a bucket.
  const int x = blockIdx.x & 7, wi = blockIdx.x >> 3, nw = gridDim.x >> 3;
  const int per = nitems >> 3, rem = nitems & 7;
  const int off_x = it_lo + x * per + (x < rem ? x : rem);
  const int end_x = off_x + per + (x < rem ? 1 : 0);
  // runs no longer than an even share, so that small launches still spread
  // over every workgroup
  const int share = max(1, (end_x - off_x + nw - 1) / nw);
  const int RUN = p.run_items > 0 ? min(p.run_items, share) : share;
  int it = off_x + wi * RUN;
  if (it >= end_x) return;  // uniform for the workgroup
  int run_end = min(it + RUN, end_x);

  const int lrow = w * 32 + (lane & 31);
  int staged = -1;  // bucket whose single key tile sits in LDS

  const const_int_ptr items = (const_int_ptr)p.items;
  int4 rec = load_item(items, it);
  GRow g = grow_of(p, rec, entry_of(p, rec, lrow), lrow);
  // the first item's queries take the same LDS path as every later item's,
  // so that the query registers never wait on a vector load (a wait on one
  // would also wait for the partial stores issued before it)
  bf16x8 qf[D / 16];
  prefetch_q_lds<D, W>(qst, q_row<D>(p, rec, g), g.valid);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
  read_q_lds<D, W>(qst, qf);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");

  while (true) {
    const int bucket = rec.x;
    const int hk = rec.w & 0xFFFF;
    const int b = rec.w >> 16;
    const int cid = bucket / p.Nb;  // chunk id
    const int j = bucket - cid * p.Nb;
    const int t_base = (cid % p.NC) * p.CT;
    const int64_t prow_base = (int64_t)(cid - p.c0) * p.Gs;
    const bool wave_on = w * 32 < rec.z;
    // next item: within the run the next one; after it the first of the
    // workgroup's next run
    const bool in_run = it + 1 < run_end;
    const int it_n = in_run ? it + 1 : it + 1 + (nw - 1) * RUN;
    const bool has_next = it_n < end_x;
    // its record, and its entry word: within a run, items cover contiguous
    // entries, so the next item starts right after this one's (read
    // speculatively; the entries array is padded); a new run starts where its
    // record says
    const int4 rec_n = has_next ? load_item(items, it_n) : rec;
    const int w_u = __builtin_amdgcn_readfirstlane(w);
    const int e_n = in_run ? rec.y + ((rec.z + (1 << p.lgR) - 1) >> p.lgR) : rec_n.y;
    const uint32_t ent_n = has_next ? next_entry<SE>(p.entries, e_n, w_u, lane, p.lgR) : 0u;
    GRow g_n = g;

    const int qpos = p.Lk - p.Lq + g.t;
    float m = -INFINITY, l = 0.f;
    f32x16 o[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
    const int key0 = j * p.block;
    const int n_keys = min(p.block, p.Lk - key0);
    const uint16_t* kb = p.k + (int64_t)b * p.ks_b + (int64_t)hk * p.ks_h;
    const uint16_t* vb = p.v + (int64_t)b * p.vs_b + (int64_t)hk * p.vs_h;
    for (int kt0 = 0; kt0 < n_keys; kt0 += KT) {
      const bool single = n_keys <= KT;
      if (W == 8 && !single) {
        // tile kt0 arrives by DMA (issued during the previous tile, or now
        // for the first), is repacked, and the next tile's DMA starts
        if (kt0 == 0) dma_kv<D, 64 * W>(s_nat, kb, p.ks_t, vb, p.vs_t, key0, n_keys);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        repack_kv<D, 64 * W>(sm, s_nat, n_keys - kt0);
        __syncthreads();
        if (kt0 + KT < n_keys) dma_kv<D, 64 * W>(s_nat, kb, p.ks_t, vb, p.vs_t, key0 + kt0 + KT, n_keys - kt0 - KT);
        staged = -1;
      } else if (!(single && staged == bucket)) {
        __syncthreads();
        stage_kv<D, 64 * W>(sm, kb, p.ks_t, vb, p.vs_t, key0 + kt0, n_keys - kt0);
        __syncthreads();
        staged = single ? bucket : -1;
      }
      f32x16 s0, s1;
      if (wave_on) qk_tile<D>(sm, qf, s0, s1);
      if (kt0 == 0 && has_next) {
        // queries of the next item into this wave's LDS staging area
        g_n = grow_of(p, rec_n, ent_n, lrow);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // earlier reads of the staging area are done
        prefetch_q_lds<D, W>(qst, q_row<D>(p, rec_n, g_n), g_n.valid);
      }
      if (wave_on) {
        // mask only where a key can be past the end or after the query
        // (ragged last tile, or the query's own block); wave-uniform test
        const int lim = min(n_keys - kt0, p.causal ? qpos - key0 - kt0 + 1 : KT);
        if (__ballot(g.valid && lim < KT) != 0ull) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kr = krow(i, hq);
            s0[i] = kr < lim ? s0[i] : -INFINITY;
            s1[i] = kr + 32 < lim ? s1[i] : -INFINITY;
          }
        }
        softmax_update<D>(s0, s1, m, l, o, p.sl2, kt0 == 0);
        pv_tile<D>(sm, s0, s1, o, kt0 == 0, l);
      }
    }
    // epilogue: pack this item's outputs, take the next item's queries out of
    // the staging area, then reuse the area to write whole partial rows
    u16x4_t pk[D / 8];
    pack_partials<D>(o, pk);
    if (has_next) {
      __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
      read_q_lds<D, W>(qst, qf);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    {
      const int hsel = p.per_group ? 0 : g.hs - hk * p.G;
      const int64_t prow = (prow_base + hsel) * p.CT + (g.t - t_base);
      const int64_t pidx = (prow * p.kslot + g.slot) * p.R + g.rr;
      if (wave_on) store_partials<D, W>(qst, pk, pidx * D, min(32, rec.z - w * 32), p.part_o);
      if (g.valid && hq == 0) {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        __builtin_nontemporal_store(f32x2{m, l}, reinterpret_cast<f32x2*>(&p.part_ml[pidx]));
      }
    }
    if (!has_next) break;
    if (!in_run) run_end = min(it_n + RUN, end_x);
    it = it_n;
    rec = rec_n;
    g = g_n;
  }
}

// ---------------------------------------------------------------------------
// Gather for sparse buckets (a few rows per selected block, as when a short
// query chunk selects from a very long memory): the MFMA gather would stage
// each block for one or two rows.  Here one wave takes one work item and
// streams its block's keys and values straight from HBM, flash-decoding
// style, with no workgroup barrier (so many items per CU are in flight):
// lane k scores key k of a 64-key pass against the rows' queries (read from
// LDS by broadcast), an fp32 online softmax per row runs across the wave, and
// for the weighted values each lane owns D/64 head dims and takes every key's
// probability by v_readlane.  Rows go two at a time; the partials have the
// gather's format.
template <int D>
__global__ __launch_bounds__(256) void attn_sparse_kernel(AttnParams p) {
  constexpr int NR = 2;        // rows per pass (most sparse buckets hold one or two)
  constexpr int DPL = D / 64;  // head dims per lane (values)
  __shared__ __attribute__((aligned(16))) float s_q[4][NR][D];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int it_lo = p.tile_off[(int64_t)p.c0 * p.Nb];
  const int nitems = p.tile_off[(int64_t)p.c1 * p.Nb] - it_lo;
  const int item = (int)blockIdx.x * 4 + w;
  if (item >= nitems) return;  // wave-uniform; no workgroup barrier follows
  const int4 rec = load_item((const_int_ptr)p.items, it_lo + item);
  const int bucket = rec.x, hk = rec.w & 0xFFFF, b = rec.w >> 16;
  const int cid = bucket / p.Nb;
  const int j = bucket - cid * p.Nb;
  const int t_base = (cid % p.NC) * p.CT;
  const int64_t prow_base = (int64_t)(cid - p.c0) * p.Gs;
  const int key0 = j * p.block;
  const int n_keys = min(p.block, p.Lk - key0);
  const uint16_t* kb = p.k + (int64_t)b * p.ks_b + (int64_t)hk * p.ks_h;
  const uint16_t* vb = p.v + (int64_t)b * p.vs_b + (int64_t)hk * p.vs_h;
  for (int r0 = 0; r0 < rec.z; r0 += NR) {
    const int nr = min(NR, rec.z - r0);
    GRow g[NR];
    int qpos[NR];
#pragma unroll
    for (int a = 0; a < NR; ++a) {
      const int lr = r0 + (a < nr ? a : 0);
      g[a] = grow_of(p, rec, entry_of(p, rec, lr), lr);
      qpos[a] = p.causal ? p.Lk - p.Lq + g[a].t : 0x7FFFFFFF;
    }
    __builtin_amdgcn_wave_barrier();  // the previous rows' queries are no longer read
#pragma unroll
    for (int a = 0; a < NR; ++a) {
      const uint16_t* qr = q_row<D>(p, rec, g[a]);
#pragma unroll
      for (int d = lane; d < D; d += 64) s_q[w][a][d] = a < nr ? bf2f(qr[d]) : 0.f;
    }
    __builtin_amdgcn_wave_barrier();
    float m[NR], l[NR], acc[NR][DPL];
#pragma unroll
    for (int a = 0; a < NR; ++a) {
      m[a] = -INFINITY;
      l[a] = 0.f;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[a][e] = 0.f;
    }
    for (int k0 = 0; k0 < n_keys; k0 += 64) {
      asm volatile("" ::: "memory");  // the query reads below stay in the pass (not hoisted: NR rows x D floats)
      const int key = k0 + lane;
      const bool kv = key < n_keys;
      const uint16_t* krow = kb + (int64_t)(key0 + (kv ? key : 0)) * p.ks_t;
      // scores of this lane's key against the rows, 8 head dims at a time
      float sc[NR];
#pragma unroll
      for (int a = 0; a < NR; ++a) sc[a] = 0.f;
      // four 16-byte pieces of the key row at a time, the next four in flight
      u16x8 kx[4], kn[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) kx[c] = kv ? ld16(krow + c * 8) : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll 1
      for (int c0 = 0; c0 < D / 8; c0 += 4) {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          kn[c] = (kv && c0 + 4 < D / 8) ? ld16(krow + (c0 + 4 + c) * 8) : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
          for (int a = 0; a < NR; ++a) {
            const f32x4 q0 = *reinterpret_cast<const f32x4*>(&s_q[w][a][(c0 + c) * 8]);
            const f32x4 q1 = *reinterpret_cast<const f32x4*>(&s_q[w][a][(c0 + c) * 8 + 4]);
            float part = sc[a];
#pragma unroll
            for (int e = 0; e < 4; ++e) part = fmaf(q0[e], bf2f(kx[c][e]), part);
#pragma unroll
            for (int e = 0; e < 4; ++e) part = fmaf(q1[e], bf2f(kx[c][4 + e]), part);
            sc[a] = part;
          }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) kx[c] = kn[c];
      }
      // this pass's values: lane owns head dims lane*DPL .. +DPL-1 of every key
      const int nk = min(64, n_keys - k0);
      float pr[NR];
#pragma unroll
      for (int a = 0; a < NR; ++a) {
        const float x = (kv && key0 + key <= qpos[a]) ? sc[a] * p.sl2 : -INFINITY;
        const float mnew = fmaxf(m[a], wave_max(x));
        const float e0 = mnew == -INFINITY ? 0.f : exp2f(x - mnew);
        const float c = mnew == -INFINITY ? 1.f : exp2f(m[a] - mnew);
        l[a] = l[a] * c + wave_sum(e0);
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[a][e] *= c;
        m[a] = mnew;
        pr[a] = e0;
      }
      for (int kk0 = 0; kk0 < nk; kk0 += 16) {
        uint32_t vx[16];
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
          const int kq = kk0 + kk;
          const uint16_t* vr = vb + (int64_t)(key0 + k0 + (kq < nk ? kq : 0)) * p.vs_t + lane * DPL;
          vx[kk] = kq < nk ? (DPL == 2 ? *reinterpret_cast<const uint32_t*>(vr) : (uint32_t)*vr) : 0u;
        }
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
          const int kq = kk0 + kk;
          if (kq < nk) {  // wave-uniform
            const float v0 = bf2f((uint16_t)(vx[kk] & 0xFFFFu)), v1 = bf2f((uint16_t)(vx[kk] >> 16));
#pragma unroll
            for (int a = 0; a < NR; ++a) {
              const float pw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pr[a]), kq));
              acc[a][0] = fmaf(pw, v0, acc[a][0]);
              if constexpr (DPL == 2) acc[a][1] = fmaf(pw, v1, acc[a][1]);
            }
          }
        }
      }
    }
    // partial rows: lane writes its head dims; lane 0 writes (m, l)
    for (int a = 0; a < nr; ++a) {
      const int hsel = p.per_group ? 0 : g[a].hs - hk * p.G;
      const int64_t prow = (prow_base + hsel) * p.CT + (g[a].t - t_base);
      const int64_t pidx = (prow * p.kslot + g[a].slot) * p.R + g[a].rr;
      uint16_t* dst = p.part_o + pidx * D + lane * DPL;
      if constexpr (DPL == 2) {
        const uint32_t packed = (uint32_t)f2bf(acc[a][0]) | ((uint32_t)f2bf(acc[a][1]) << 16);
        __builtin_nontemporal_store(packed, reinterpret_cast<uint32_t*>(dst));
      } else {
        __builtin_nontemporal_store(f2bf(acc[a][0]), dst);
      }
      if (lane == 0) {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        __builtin_nontemporal_store(f32x2{m[a], l[a]}, reinterpret_cast<f32x2*>(&p.part_ml[pidx]));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Merge: output row (b, t, h) <- LSE-weighted sum of its selection row's
// partials (the slots of its sel row, own block included).  D/8 lanes per
// row, 8 head dims per lane; slots are read eight at a time so their loads
// are in flight together.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnParams p) {
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int RPW = 64 / LPR;       // rows per wave
  constexpr int SB = 8;               // slots per batch
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int li = lane % LPR;
  // rows of this launch: (chunk - c0, token in chunk, head in group), so a
  // token's G output heads are adjacent
  const int64_t nrows = (int64_t)(p.c1 - p.c0) * p.CT * p.G;
  const int64_t row = ((int64_t)blockIdx.x * 4 + w) * RPW + lane / LPR;
  const int64_t rr_ = row < nrows ? row : 0;
  const int hh = (int)(rr_ % p.G);
  const int t_loc = (int)((rr_ / p.G) % p.CT);
  const int c_rel = (int)(rr_ / ((int64_t)p.G * p.CT));
  const int cid = p.c0 + c_rel;
  const int bh = cid / p.NC;
  const int t = (cid % p.NC) * p.CT + t_loc;
  const bool ok = row < nrows && t < p.Lq;
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const int h = hk * p.G + hh;
  const int hs = p.per_group ? hk : h;
  const int rr = p.per_group ? hh : 0;
  const int64_t prow = ((int64_t)c_rel * p.Gs + (p.per_group ? 0 : hh)) * p.CT + t_loc;
  const int64_t srow = ((int64_t)b * p.Hs + hs) * p.Lq + (ok ? t : 0);
  const int32_t* sr = p.sel + srow * p.sel_w;
  // number of valid slots (valid entries come first, -1 after): the row's
  // lanes count a strided share each, then sum across the row's lanes
  int n = 0;
  if (ok) {
    for (int s = li; s < p.sel_w; s += LPR) n += sr[s] >= 0 ? 1 : 0;
  }
#pragma unroll
  for (int m2 = 1; m2 < LPR; m2 <<= 1) n += __shfl_xor(n, m2, 64);
  // partial s holds sum_k p_k v_k with p = 2^(score*sl2 - m_s) and sum_k p_k = l_s
  float M = -INFINITY, W = 0.f;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int s0 = 0; s0 < n; s0 += SB) {
    float2 ml[SB];
    u16x8 ov[SB];
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int s = s0 + u;
      ml[u] = make_float2(-INFINITY, 0.f);
      ov[u] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (s < n) {
        const int64_t pidx = (prow * p.kslot + s) * p.R + rr;
        // streaming loads: every partial is read exactly once
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        const f32x2 v2 = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(&p.part_ml[pidx]));
        ml[u] = make_float2(v2[0], v2[1]);
        ov[u] = __builtin_nontemporal_load(reinterpret_cast<const u16x8*>(p.part_o + pidx * D + li * 8));
      }
    }
    float mb = M;
#pragma unroll
    for (int u = 0; u < SB; ++u) mb = fmaxf(mb, ml[u].x);
    const float c = __builtin_amdgcn_exp2f(M - mb);
    W *= c;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= c;
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const float wu = __builtin_amdgcn_exp2f(ml[u].x - mb);  // 0 for unused slots
      W = fmaf(wu, ml[u].y, W);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(wu, bf2f(ov[u][e]), acc[e]);
    }
    M = mb;
  }
  if (!ok) return;
  const float inv = W > 0.f ? 1.0f / W : 0.f;
  u16x8 out;
#pragma unroll
  for (int e = 0; e < 8; ++e) out[e] = f2bf(acc[e] * inv);
  // streaming store: the output is written once and not read back here
  __builtin_nontemporal_store(out, reinterpret_cast<u16x8*>(p.o + (int64_t)b * p.os_b + (int64_t)t * p.os_t +
                                                            (int64_t)h * p.os_h + li * 8));
  if (p.lse_out && li == 0)
    p.lse_out[((int64_t)b * p.Hq + h) * p.Lq + t] = W > 0.f ? (M + log2f(W)) * 0.69314718055994530942f : -INFINITY;
}

// Persistent grid = the workgroups the device holds at once (a multiple of 8,
// one range per XCD).
template <int D, int W, bool SE>
static int gather_grid() {
  static int cached = 0;
  if (cached) return cached;
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, attn_gather_kernel<D, W, SE>, 64 * W, 0) != hipSuccess || per < 1)
    return 2048 / W;
  cached = ((cus * per + 7) / 8) * 8;
  return cached;
}

// Work items hold 32 * gather_waves rows: 4 waves for blocks of one 64-key
// tile (a workgroup keeps the tile staged across consecutive items of the
// same block), 8 waves for longer blocks (every item re-stages the block's
// tiles, so a larger item stages them for twice the rows).
int gather_waves(int block) { return block > KT ? 8 : 4; }

template <int D, int W>
static void launch_gather_dw(const AttnParams& p, hipStream_t s) {
  if (p.lgR >= 2)
    hipLaunchKernelGGL((attn_gather_kernel<D, W, true>), dim3(gather_grid<D, W, true>()), dim3(64 * W), 0, s, p);
  else
    hipLaunchKernelGGL((attn_gather_kernel<D, W, false>), dim3(gather_grid<D, W, false>()), dim3(64 * W), 0, s, p);
}

bool launch_attn_gather(const AttnParams& p, hipStream_t s) {
  if (p.sparse_items > 0) {
    LaunchScope ls("attn_gather", s, 2);
    const unsigned grid = (unsigned)((p.sparse_items + 3) / 4);  // one wave per item
    if (p.D == 128)
      hipLaunchKernelGGL(attn_sparse_kernel<128>, dim3(grid), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(attn_sparse_kernel<64>, dim3(grid), dim3(256), 0, s, p);
    return launch_ok("attn_gather");
  }
  {
    LaunchScope ls("attn_gather", s, 2);
    const int W = p.rows_item / 32;
    if (p.D == 128) {
      if (W == 8) launch_gather_dw<128, 8>(p, s);
      else launch_gather_dw<128, 4>(p, s);
    } else {
      if (W == 8) launch_gather_dw<64, 8>(p, s);
      else launch_gather_dw<64, 4>(p, s);
    }
  }
  return launch_ok("attn_gather");
}

bool launch_attn_merge(const AttnParams& p, hipStream_t s) {
  const int64_t nrows = (int64_t)(p.c1 - p.c0) * p.CT * p.G;
  const int rpw = 64 / (p.D / 8);
  const int64_t grid = (nrows + 4 * rpw - 1) / (4 * rpw);
  {
    LaunchScope ls("attn_merge", s, 2);
    if (p.D == 128)
      hipLaunchKernelGGL(attn_merge_kernel<128>, dim3((unsigned)grid), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(attn_merge_kernel<64>, dim3((unsigned)grid), dim3(256), 0, s, p);
  }
  return launch_ok("attn_merge");
}

// ---------------------------------------------------------------------------
// fp32 path: one wave per (b, t, h) query row, all its selected blocks, fp32
// arithmetic throughout (keys on lanes for the scores, head dims on lanes for
// the weighted sum).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_rowwise_f32_kernel(AttnF32Params p) {
  __shared__ float s_q[4][128];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t nrows = (int64_t)p.B * p.Lq * p.Hq;
  const int64_t row = (int64_t)blockIdx.x * 4 + w;
  if (row >= nrows) return;  // wave-uniform; no workgroup barrier follows
  const int h = (int)(row % p.Hq);
  const int t = (int)((row / p.Hq) % p.Lq);
  const int b = (int)(row / ((int64_t)p.Hq * p.Lq));
  const int hk = h / p.G;
  const int hs = p.per_group ? hk : h;
  const float* qr = p.q + (int64_t)b * p.qs_b + (int64_t)t * p.qs_t + (int64_t)h * p.qs_h;
  for (int d = lane; d < p.D; d += 64) s_q[w][d] = qr[d];
  __builtin_amdgcn_wave_barrier();
  const int64_t qpos = (int64_t)p.Lk - p.Lq + t;
  const int64_t cur = qpos / p.block;
  const int32_t* srow = p.sel + (((int64_t)b * p.Hs + hs) * p.Lq + t) * p.sel_w;
  const float* kb = p.k + (int64_t)b * p.ks_b + (int64_t)hk * p.ks_h;
  const float* vb = p.v + (int64_t)b * p.vs_b + (int64_t)hk * p.vs_h;
  float m = -INFINITY, l = 0.f, a0 = 0.f, a1 = 0.f;
  for (int s = 0; s < p.sel_w; ++s) {
    const int j = srow[s];
    if (j < 0) break;
    const int64_t ka = (int64_t)j * p.block;
    int64_t ke = min<int64_t>(ka + p.block, p.Lk);
    if (p.causal && j == cur) ke = min<int64_t>(ke, qpos + 1);
    for (int64_t k0 = ka; k0 < ke; k0 += 64) {
      const int64_t key = k0 + lane;
      float sc = -INFINITY;
      if (key < ke) {
        const float* kr = kb + key * p.ks_t;
        float acc = 0.f;
        for (int d = 0; d < p.D; ++d) acc = fmaf(s_q[w][d], kr[d], acc);
        sc = acc * p.scale;
      }
      const float mnew = fmaxf(m, wave_max(sc));
      const float corr = expf(m - mnew);
      const float pk = key < ke ? expf(sc - mnew) : 0.f;
      l = l * corr + wave_sum(pk);
      a0 *= corr;
      a1 *= corr;
      const int nk = (int)min<int64_t>(64, ke - k0);
      for (int kk = 0; kk < nk; ++kk) {
        const float pv = __shfl(pk, kk, 64);
        const float* vr = vb + (k0 + kk) * p.vs_t;
        if (lane < p.D) a0 = fmaf(pv, vr[lane], a0);
        if (lane + 64 < p.D) a1 = fmaf(pv, vr[lane + 64], a1);
      }
      m = mnew;
    }
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  float* orow = p.o + (int64_t)b * p.os_b + (int64_t)t * p.os_t + (int64_t)h * p.os_h;
  if (lane < p.D) orow[lane] = a0 * inv;
  if (lane + 64 < p.D) orow[lane + 64] = a1 * inv;
  if (p.lse_out && lane == 0) p.lse_out[((int64_t)b * p.Hq + h) * p.Lq + t] = l > 0.f ? m + logf(l) : -INFINITY;
}

bool launch_attn_rowwise_f32(const AttnF32Params& p, hipStream_t s) {
  const int64_t nrows = (int64_t)p.B * p.Lq * p.Hq;
  {
    LaunchScope ls("attn_rowwise_f32", s);
    hipLaunchKernelGGL(attn_rowwise_f32_kernel, dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, s, p);
  }
  return launch_ok("attn_rowwise_f32");
}

// ---------------------------------------------------------------------------
// Backward through the fixed selection.  A bucket's entries (one query
// chunk's rows that chose one (b, kv head, block)) are sorted first and cut
// into work items of consecutive rows, so every sum over the rows that chose
// a block runs in a fixed order.
// ---------------------------------------------------------------------------

// delta[b, h, t] = dout . o of each output row, fp32 (D/8 lanes per row)
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(AttnParams p, int64_t nrows) {
  constexpr int LPR = D / 8;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
  const int li = threadIdx.x % LPR;
  const int64_t rr = row < nrows ? row : 0;  // rows (b, t, h), h fastest
  const int h = (int)(rr % p.Hq);
  const int t = (int)((rr / p.Hq) % p.Lq);
  const int b = (int)(rr / ((int64_t)p.Hq * p.Lq));
  const u16x8 g = ld16(p.dout + (int64_t)b * p.dos_b + (int64_t)t * p.dos_t + (int64_t)h * p.dos_h + li * 8);
  const u16x8 o = ld16(p.o + (int64_t)b * p.os_b + (int64_t)t * p.os_t + (int64_t)h * p.os_h + li * 8);
  float acc = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = fmaf(bf2f(g[e]), bf2f(o[e]), acc);
#pragma unroll
  for (int m2 = 1; m2 < LPR; m2 <<= 1) acc += __shfl_xor(acc, m2, 64);
  if (row < nrows && li == 0) p.delta[((int64_t)b * p.Hq + h) * p.Lq + t] = acc;
}

// Sort each bucket's entry words ascending (bitonic, in LDS); buckets hold at
// most kBwdSortCap entries by construction of the query chunks.
__global__ __launch_bounds__(256) void bwd_sort_kernel(AttnParams p, int nbk) {
  __shared__ uint32_t s_e[kBwdSortCap];
  const int bk = blockIdx.x;
  if (bk >= nbk) return;
  const int a = p.bucket_off[bk];
  const int n = p.bucket_off[bk + 1] - a;
  if (n <= 1 || n > kBwdSortCap) return;  // uniform (larger buckets cannot arise from a valid selection)
  int n2 = 2;
  while (n2 < n) n2 <<= 1;
  uint32_t* ent = const_cast<uint32_t*>(p.entries) + a;
  for (int i = threadIdx.x; i < n2; i += 256) s_e[i] = i < n ? ent[i] : 0xFFFFFFFFu;
  __syncthreads();
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n2; i += 256) {
        const int l = i ^ j;
        if (l > i) {
          const uint32_t x = s_e[i], y = s_e[l];
          const bool up = (i & k) == 0;
          if ((x > y) == up) {
            s_e[i] = y;
            s_e[l] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < n; i += 256) ent[i] = s_e[i];
}

// One workgroup per work item: for each 64-key tile of the block, stage K
// (fp32, LDS), then take the item's rows sixteen at a time.
// Wave w owns keys 16w .. 16w+15 of the tile; lane (key, quarter) forms
// quarter dot products q.k and g.v, completes them across the key's four
// lanes, and accumulates dk and dv for its key and quarter in registers.
// The rows' ds values go through LDS for dq = sum_u ds_u k_u, which each
// (row, slot) partial accumulates over the block's tiles.
template <int D>
__global__ __launch_bounds__(256, 2) void attn_bwd_kernel(AttnParams p) {
  constexpr int KT = 64, RB = 16, DQ = D / 4, KP = D + 4;
  __shared__ __attribute__((aligned(16))) float s_k[KT * KP];
  __shared__ __attribute__((aligned(16))) float s_q[RB][D];
  __shared__ __attribute__((aligned(16))) float s_g[RB][D];
  __shared__ float s_ds[RB][KT];
  __shared__ float s_lse2[RB], s_dl[RB];
  __shared__ int s_qpos[RB];
  __shared__ int64_t s_pidx[RB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int item = blockIdx.x;
  if (item >= p.tile_off[(int64_t)p.B * p.Hkv * p.NC * p.Nb]) return;  // past the built items; uniform
  const int4 rec = load_item((const_int_ptr)p.items, item);
  const int bucket = rec.x, hk = rec.w & 0xFFFF, b = rec.w >> 16;
  const int cid = bucket / p.Nb;
  const int j = bucket - cid * p.Nb;
  const int t_base = (cid % p.NC) * p.CT;
  const int64_t prow_base = (int64_t)cid * p.Gs;
  const int key0 = j * p.block;
  const int n_keys = min(p.block, p.Lk - key0);
  const uint16_t* kb = p.k + (int64_t)b * p.ks_b + (int64_t)hk * p.ks_h;
  const uint16_t* vb = p.v + (int64_t)b * p.vs_b + (int64_t)hk * p.vs_h;
  const int ku = 16 * w + (lane >> 2), qc = lane & 3;  // this lane's key in the tile and quarter
  float* dst = p.dkv_part + (int64_t)item * 2 * p.block * D;
  const float L2E = 1.4426950408889634f;
  for (int t0 = 0; t0 < n_keys; t0 += KT) {
    const int nt = min(KT, n_keys - t0);
    __syncthreads();  // the previous tile's K / V are no longer read
    for (int i = tid; i < KT * (D / 8); i += 256) {
      const int u = i / (D / 8), c8 = i % (D / 8);
      u16x8 kx = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      if (u < nt) kx = ld16(kb + (int64_t)(key0 + t0 + u) * p.ks_t + c8 * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) s_k[u * KP + c8 * 8 + e] = bf2f(kx[e]);
    }
    float dk[DQ], dv[DQ];
#pragma unroll
    for (int e = 0; e < DQ; ++e) dk[e] = dv[e] = 0.f;
    const int key = key0 + t0 + ku;
    __syncthreads();  // the tile is staged
    // this lane's quarter of its key (LDS) and value (straight from memory),
    // held for every row of the item
    float kr[DQ], vr[DQ];
#pragma unroll
    for (int e = 0; e < DQ; e += 8) {
      const f32x4 k0 = *reinterpret_cast<const f32x4*>(&s_k[ku * KP + qc * DQ + e]);
      const f32x4 k1 = *reinterpret_cast<const f32x4*>(&s_k[ku * KP + qc * DQ + e + 4]);
      const u16x8 vx = ku < nt ? ld16(vb + (int64_t)key * p.vs_t + qc * DQ + e) : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        kr[e + x] = k0[x];
        kr[e + 4 + x] = k1[x];
      }
#pragma unroll
      for (int x = 0; x < 8; ++x) vr[e + x] = bf2f(vx[x]);
    }
    for (int r0 = 0; r0 < rec.z; r0 += RB) {
      const int nr = min(RB, rec.z - r0);
      __syncthreads();  // the previous rows' q, g and ds are no longer read
      // stage the batch's rows: q, g (fp32), lse (log2), delta, position, partial index
      for (int i = tid; i < RB * (D / 8); i += 256) {
        const int r = i / (D / 8), c8 = i % (D / 8);
        u16x8 qx = u16x8{0, 0, 0, 0, 0, 0, 0, 0}, gx = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (r < nr) {
          const GRow g = grow_of(p, rec, entry_of(p, rec, r0 + r), r0 + r);
          qx = ld16(q_row<D>(p, rec, g) + c8 * 8);
          gx = ld16(p.dout + (int64_t)b * p.dos_b + (int64_t)g.t * p.dos_t + (int64_t)g.qh * p.dos_h + c8 * 8);
          if (c8 == 0) {
            const int64_t orow = ((int64_t)b * p.Hq + g.qh) * p.Lq + g.t;
            s_lse2[r] = p.lse_in[orow] * L2E;
            s_dl[r] = p.delta[orow];
            s_qpos[r] = p.causal ? p.Lk - p.Lq + g.t : 0x7FFFFFFF;
            const int hsel = p.per_group ? 0 : g.hs - hk * p.G;
            const int64_t prow = (prow_base + hsel) * p.CT + (g.t - t_base);
            s_pidx[r] = (prow * p.kslot + g.slot) * p.R + g.rr;
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s_q[r][c8 * 8 + e] = bf2f(qx[e]);
          s_g[r][c8 * 8 + e] = bf2f(gx[e]);
        }
      }
      __syncthreads();
      for (int r = 0; r < nr; ++r) {
        float sc = 0.f, dp = 0.f;
        float qv[DQ], gv[DQ];  // the row's quarter of q and g, read once for both passes
#pragma unroll
        for (int e = 0; e < DQ; e += 4) {
          const f32x4 qq = *reinterpret_cast<const f32x4*>(&s_q[r][qc * DQ + e]);
          const f32x4 gq = *reinterpret_cast<const f32x4*>(&s_g[r][qc * DQ + e]);
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            qv[e + x] = qq[x];
            gv[e + x] = gq[x];
            sc = fmaf(qq[x], kr[e + x], sc);
            dp = fmaf(gq[x], vr[e + x], dp);
          }
        }
        // complete the dot products across the key's four lanes (a DPP quad; every lane runs it)
        sc += __uint_as_float(dpp32<0xB1>(__float_as_uint(sc), __float_as_uint(sc)));
        dp += __uint_as_float(dpp32<0xB1>(__float_as_uint(dp), __float_as_uint(dp)));
        sc += __uint_as_float(dpp32<0x4E>(__float_as_uint(sc), __float_as_uint(sc)));
        dp += __uint_as_float(dpp32<0x4E>(__float_as_uint(dp), __float_as_uint(dp)));
        const bool ok = ku < nt && key <= s_qpos[r];
        const float pr = ok ? exp2f(sc * p.sl2 - s_lse2[r]) : 0.f;
        const float ds = pr * (dp - s_dl[r]);
#pragma unroll
        for (int e = 0; e < DQ; ++e) {
          dk[e] = fmaf(ds, qv[e], dk[e]);
          dv[e] = fmaf(pr, gv[e], dv[e]);
        }
        if (qc == 0) s_ds[r][ku] = ds;
      }
      __syncthreads();
      // dq partials: thread (row, D/16 head dims) sums ds_u k_u over the tile
      {
        constexpr int DPT = D / 16;
        const int r = tid >> 4, d0 = (tid & 15) * DPT;
        if (r < nr) {
          float acc[DPT];
#pragma unroll
          for (int e = 0; e < DPT; ++e) acc[e] = 0.f;
          for (int u = 0; u < nt; ++u) {
            const float dsu = s_ds[r][u];
#pragma unroll
            for (int e = 0; e < DPT; ++e) acc[e] = fmaf(dsu, s_k[u * KP + d0 + e], acc[e]);
          }
          float* dqp = p.dq_part + s_pidx[r] * D + d0;
#pragma unroll
          for (int e = 0; e < DPT; ++e) dqp[e] = t0 == 0 ? acc[e] : dqp[e] + acc[e];
        }
      }
    }
    // this item's dk / dv sums for the tile's keys
    if (ku < nt) {
      float* dkp = dst + (int64_t)(t0 + ku) * D + qc * DQ;
      float* dvp = dst + (int64_t)(p.block + t0 + ku) * D + qc * DQ;
#pragma unroll
      for (int e = 0; e < DQ; e += 4) {
        *reinterpret_cast<f32x4*>(dkp + e) = f32x4{dk[e], dk[e + 1], dk[e + 2], dk[e + 3]};
        *reinterpret_cast<f32x4*>(dvp + e) = f32x4{dv[e], dv[e + 1], dv[e + 2], dv[e + 3]};
      }
    }
  }
}

// dq row (b, t, h) = scale * sum of its selection row's slot partials, in slot
// order (D/4 lanes per row, four head dims each)
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_reduce_kernel(AttnParams p, int64_t nrows) {
  constexpr int LPR = D / 4;
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPR;
  if (row >= nrows) return;
  const int li = threadIdx.x % LPR;
  const int h = (int)(row % p.Hq);
  const int t = (int)((row / p.Hq) % p.Lq);
  const int b = (int)(row / ((int64_t)p.Hq * p.Lq));
  const int hk = h / p.G, hh = h % p.G;
  const int hs = p.per_group ? hk : h;
  const int c = t / p.CT;
  const int64_t cid = ((int64_t)b * p.Hkv + hk) * p.NC + c;
  const int64_t prow = (cid * p.Gs + (p.per_group ? 0 : hh)) * p.CT + (t - c * p.CT);
  const int rr = p.per_group ? hh : 0;
  const int32_t* sr = p.sel + (((int64_t)b * p.Hs + hs) * p.Lq + t) * p.sel_w;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int sl = 0; sl < p.sel_w; ++sl) {
    const int jj = sr[sl];
    if (jj < 0 || jj >= p.Nb) continue;
    const int64_t pidx = (prow * p.kslot + sl) * p.R + rr;
    acc += *reinterpret_cast<const f32x4*>(p.dq_part + pidx * D + li * 4);
  }
  *reinterpret_cast<f32x4*>(p.dq + row * D + li * 4) = acc * p.scale;
}

// dk / dv of one (b, kv head, block): the items of its buckets summed in
// (query chunk, item) order; blocks nobody chose get zeros
template <int D>
__global__ __launch_bounds__(256) void bwd_dkv_reduce_kernel(AttnParams p) {
  const int64_t blk = blockIdx.x;  // (b * Hkv + hk) * Nb + j
  const int j = (int)(blk % p.Nb);
  const int64_t bh = blk / p.Nb;
  const int hk = (int)(bh % p.Hkv), b = (int)(bh / p.Hkv);
  const int key0 = j * p.block;
  const int n_keys = min(p.block, p.Lk - key0);
  for (int i = threadIdx.x; i < n_keys * (D / 4); i += 256) {
    const int u = i / (D / 4), d4 = (i % (D / 4)) * 4;
    f32x4 ak = f32x4{0.f, 0.f, 0.f, 0.f}, av = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c = 0; c < p.NC; ++c) {
      const int64_t bk = (bh * p.NC + c) * p.Nb + j;
      if (p.grid == 0 || p.counts[bk] == 0) continue;  // no selection entries at all: nothing was built
      for (int it = p.tile_off[bk]; it < p.tile_off[bk + 1]; ++it) {
        const float* src = p.dkv_part + (int64_t)it * 2 * p.block * D;
        ak += *reinterpret_cast<const f32x4*>(src + (int64_t)u * D + d4);
        av += *reinterpret_cast<const f32x4*>(src + (int64_t)(p.block + u) * D + d4);
      }
    }
    const int64_t orow = (((int64_t)b * p.Lk + key0 + u) * p.Hkv + hk) * D + d4;
    *reinterpret_cast<f32x4*>(p.dk + orow) = ak * p.scale;
    *reinterpret_cast<f32x4*>(p.dv + orow) = av;
  }
}

bool launch_attn_backward(const AttnParams& p, int64_t nrows_out, hipStream_t s) {
  const int nbk = p.B * p.Hkv * p.NC * p.Nb;
  {
    LaunchScope ls("bwd_delta", s);
    const int64_t thr = nrows_out * (p.D / 8);
    const unsigned grid = (unsigned)((thr + 255) / 256);
    if (p.D == 128) hipLaunchKernelGGL(bwd_delta_kernel<128>, dim3(grid), dim3(256), 0, s, p, nrows_out);
    else hipLaunchKernelGGL(bwd_delta_kernel<64>, dim3(grid), dim3(256), 0, s, p, nrows_out);
  }
  if (!launch_ok("bwd_delta")) return false;
  if (p.grid > 0) {
    LaunchScope ls("bwd_sort", s);
    hipLaunchKernelGGL(bwd_sort_kernel, dim3((unsigned)nbk), dim3(256), 0, s, p, nbk);
  }
  if (!launch_ok("bwd_sort")) return false;
  if (p.grid > 0) {
    LaunchScope ls("attn_bwd", s);
    // grid = the bound on the item count (items are built on the device);
    // workgroups past the built items exit at once
    const unsigned grid = (unsigned)p.grid;
    if (p.D == 128) hipLaunchKernelGGL(attn_bwd_kernel<128>, dim3(grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(attn_bwd_kernel<64>, dim3(grid), dim3(256), 0, s, p);
  }
  if (!launch_ok("attn_bwd")) return false;
  {
    LaunchScope ls("bwd_dq_reduce", s);
    const int64_t thr = nrows_out * (p.D / 4);
    const unsigned grid = (unsigned)((thr + 255) / 256);
    if (p.D == 128) hipLaunchKernelGGL(bwd_dq_reduce_kernel<128>, dim3(grid), dim3(256), 0, s, p, nrows_out);
    else hipLaunchKernelGGL(bwd_dq_reduce_kernel<64>, dim3(grid), dim3(256), 0, s, p, nrows_out);
  }
  if (!launch_ok("bwd_dq_reduce")) return false;
  {
    LaunchScope ls("bwd_dkv_reduce", s);
    const unsigned grid = (unsigned)((int64_t)p.B * p.Hkv * p.Nb);
    if (p.D == 128) hipLaunchKernelGGL(bwd_dkv_reduce_kernel<128>, dim3(grid), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(bwd_dkv_reduce_kernel<64>, dim3(grid), dim3(256), 0, s, p);
  }
  return launch_ok("bwd_dkv_reduce");
}

}  // namespace bsa
