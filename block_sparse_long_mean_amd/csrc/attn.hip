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
//    (row, slot) is an unnormalised partial output sum_k p_k v_k with
//    p_k = 2^(s_k * scale * log2(e) - m), stored as 16-bit integers with one
//    binary exponent per row, and its pair (m, l = sum_k p_k) in fp32 (the
//    exponent folded in).  Persistent workgroups walk contiguous item ranges and prefetch
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

// One staged 64-key tile of a block.  Keys row-major with rows padded by 16
// bytes (16 lanes reading one 16-byte piece of 16 consecutive rows hit
// distinct banks); values row-major as stored, with the 16-byte pieces of a
// row permuted (piece c of row r at c ^ vswz(r)) so that the transposing
// reads of the P.V operand (four rows x 32 bytes per 16 lanes) hit distinct
// banks.
template <int D>
struct AttnSmem {
  uint16_t k[KT * (D + 8)];
  uint16_t v[KT * D];
};

// piece permutation of value row r (16-byte pieces; D / 8 per row)
template <int D>
BSA_DEV int vswz(int r) {
  if constexpr (D == 128) return 4 * (r & 3);
  else return 4 * ((r >> 1) & 1);
}

// Per-wave LDS staging area, used twice per work item:
//  * the next item's query rows: for each 16-column chunk s, lane l's 16
//    bytes land at elements [(s*64 + l)*8, +8) (global_load_lds_dwordx4
//    writes lane l's data at the wave's LDS base + 16*l);
//  * the finished partial outputs, row-major with rows padded by 8 bytes, so
//    that every global store instruction writes whole 256-byte rows.
template <int D, int W>
struct QStage {
  static constexpr int QELEMS = (D / 16) * 64 * 8;
  static constexpr int RS = D + 4;  // padded output row (16-bit elements)
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

// O^T tile of the wave's 32 rows -> 16-bit rows in LDS -> global:
// D/8 lanes write one row's D elements (16 bytes each), 64*8/D rows per
// store instruction.  Rows [nvalid, 32) of the wave are not written; row r's
// destination element offset is held by lane r.
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));

// Partial outputs are stored as 16-bit integers with one binary exponent per
// row: q = round(32767 * x * 2^-E), with 2^E above the row's largest |x|, so
// every element carries an error of at most 2^(E-16) -- about 2^-15 of the
// row's largest value, where a bf16 element would carry up to 2^-8 of its
// own.  The exponent is folded into the row's (m, l): m' = m + E and
// l' = l * 2^-E leave the merge's weights 2^(m' - M) l' and its log-sum-exp
// unchanged while scaling the stored q back by 2^E (the merge divides by
// 32767 at the end).  E is kept at or above kPartMinExp so that the
// exponents of one row's partials stay within the fp32 range of their
// weights.
constexpr int kPartMinExp = -20;
typedef short s16x2 __attribute__((ext_vector_type(2)));

BSA_DEV int part_exponent(float absmax) { return max(__builtin_amdgcn_frexp_expf(absmax), kPartMinExp); }

BSA_DEV uint32_t pack_norm2(float a, float b, int ex) {
  const s16x2 r = __builtin_amdgcn_cvt_pknorm_i16(__builtin_amdgcn_ldexpf(a, -ex), __builtin_amdgcn_ldexpf(b, -ex));
  return __builtin_bit_cast(uint32_t, r);
}

// Packs this lane's share of the wave's 32 partial rows (lanes l and l + 32
// hold the same query column, so the row's exponent takes both); returns E.
template <int D>
BSA_DEV int pack_partials(const f32x16 (&o)[D / 32], u16x4_t (&pk)[D / 8]) {
  float mx = 0.f;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(o[dt][i]));
  mx = max_halves(mx);
  const int ex = part_exponent(mx);
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int gg = 0; gg < 4; ++gg) {
      const uint32_t a = pack_norm2(o[dt][4 * gg], o[dt][4 * gg + 1], ex);
      const uint32_t b = pack_norm2(o[dt][4 * gg + 2], o[dt][4 * gg + 3], ex);
      pk[dt * 4 + gg] = u16x4_t{(uint16_t)a, (uint16_t)(a >> 16), (uint16_t)b, (uint16_t)(b >> 16)};
    }
  return ex;
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
          : "=&v"(dst), "=&v"(a), "=&v"(b)
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

// Stage keys [key0, key0 + KT) of one kv head into LDS through registers
// (rows past n_valid zero).
template <int D, int NT>
BSA_DEV void stage_kv(AttnSmem<D>& sm, const uint16_t* kb, int64_t ks_t, const uint16_t* vb, int64_t vs_t,
                      int key0, int n_valid) {
  const int tid = threadIdx.x;
  constexpr int CH = D / 8;
  for (int idx = tid; idx < KT * CH; idx += NT) {
    const int kr = idx / CH, ch = idx % CH;
    u16x8 x = {0, 0, 0, 0, 0, 0, 0, 0}, y = {0, 0, 0, 0, 0, 0, 0, 0};
    if (kr < n_valid) {
      x = ld16(kb + (int64_t)(key0 + kr) * ks_t + ch * 8);
      y = ld16(vb + (int64_t)(key0 + kr) * vs_t + ch * 8);
    }
    st16(&sm.k[kr * (D + 8) + ch * 8], x);
    st16(&sm.v[kr * D + ((ch ^ vswz<D>(kr)) * 8)], y);
  }
}

// The same tile copied global -> LDS by DMA (global_load_lds: 64 lanes x 16
// bytes land at consecutive LDS addresses per instruction), straight into
// the layout above: an LDS position that is row padding loads a piece of its
// own row; rows past n_valid load row 0 of the tile (finite values, masked
// out of the scores).  Every thread issues its share; the caller waits.
template <int D, int NT>
BSA_DEV void dma_kv(AttnSmem<D>& sm, const uint16_t* kb, int64_t ks_t, const uint16_t* vb, int64_t vs_t, int key0,
                    int n_valid) {
  constexpr int KP = D / 8 + 1;  // 16-byte pieces per padded key row
  constexpr int VP = D / 8;      // pieces per value row
  constexpr int NW = NT / 64;
  constexpr int NK = (KT * KP + 63) / 64;  // DMA instructions for the keys
  constexpr int NV = KT * VP / 64;         // and for the values
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = lane_id();
  for (int i = w; i < NK + NV; i += NW) {
    if (i < NK) {
      const int P = i * 64 + lane;  // piece position in the padded key tile
      int r = P / KP, c = P % KP;
      if (c == KP - 1 || r >= KT) c = 0;  // padding (or past the tile): a piece of an in-bounds row
      if (r >= KT) r = 0;
      const int rr = r < n_valid ? r : 0;
      __builtin_amdgcn_global_load_lds((const void*)(kb + (int64_t)(key0 + rr) * ks_t + c * 8),
                                       (lds_ptr_t)(sm.k + i * 512), 16, 0, 0);
    } else {
      const int P = (i - NK) * 64 + lane;
      const int r = P / VP, pos = P % VP;
      const int rr = r < n_valid ? r : 0;
      const int c = pos ^ vswz<D>(r);
      __builtin_amdgcn_global_load_lds((const void*)(vb + (int64_t)(key0 + rr) * vs_t + c * 8),
                                       (lds_ptr_t)(sm.v + (i - NK) * 512), 16, 0, 0);
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
        : "=&v"(a0), "=&v"(a1), "=&v"(b0), "=&v"(b1)
        : "v"(base), "n"(S * 32), "n"(R32 + S * 32), "n"(S * 32 + 32), "n"(R32 + S * 32 + 32)
        : "memory");
    s0 = mfma32(as_bf(a0), qf[S], s0);
    s1 = mfma32(as_bf(a1), qf[S], s1);
    s0 = mfma32(as_bf(b0), qf[S + 1], s0);
    s1 = mfma32(as_bf(b1), qf[S + 1], s1);
    qk_steps<S + 2, D>(base, qf, s0, s1);
  }
}

// A . B^T for a padded 64-row tile A (rows of D elements, row stride D + 8)
// and this wave's 32 columns B (qf: lane l holds head dims 16s + 8(l/32) ..
// +7 of column l%32 in qf[s]): s0 = tile rows 0..31, s1 = rows 32..63.
template <int D>
BSA_DEV void qk_tile_pad(const uint16_t* tile, const bf16x8 (&qf)[D / 16], f32x16& s0, f32x16& s1) {
  const int lane = lane_id();
  const int r = lane & 31, h = lane >> 5;
  s0 = f32x16{};
  s1 = f32x16{};
  qk_steps<0, D>(lds_addr(&tile[r * (D + 8) + 8 * h]), qf, s0, s1);
}

// S^T (64 keys x 32 queries) for this wave: s0 keys 0..31, s1 keys 32..63.
template <int D>
BSA_DEV void qk_tile(const AttnSmem<D>& sm, const bf16x8 (&qf)[D / 16], f32x16& s0, f32x16& s1) {
  qk_tile_pad<D>(sm.k, qf, s0, s1);
}

// Head-dim tile DT of pv_tile: O^T rows 32 DT .. 32 DT + 31 over the tile's
// 64 keys.  The A operand (V^T: 8 keys of one head dim per lane) comes from
// the row-major value tile by transposing reads (ds_read_b64_tr_b16): in
// each group of 16 lanes, lane i receives element i%4 of the 8 bytes that
// lane i/4 + 4e addresses (e = 0..3), so a lane s that addresses
// V[k0 + s/4][d0 + 4(s%4)] hands lane i the keys k0 .. k0+3 of head dim
// d0 + i.  The keys follow the P operand's order: 16kk + 4h .. +3, then
// 16kk + 8 + 4h .. +3 (h = lane / 32).  vbase[DT] = LDS byte address this
// lane addresses for head-dim tile DT in key row 4h + s/4; the key steps are
// immediate offsets.
template <int DT, int D>
BSA_DEV void pv_steps(const uint32_t (&vbase)[D / 32], const bf16x8 (&pb)[4], f32x16 (&o)[D / 32], bool first) {
  if constexpr (DT < D / 32) {
    constexpr int RB = D * 2;  // bytes per value row
    u16x4 x0, x1, x2, x3, x4, x5, x6, x7;
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%9\n\tds_read_b64_tr_b16 %1, %8 offset:%10\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:%11\n\tds_read_b64_tr_b16 %3, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:%13\n\tds_read_b64_tr_b16 %5, %8 offset:%14\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:%15\n\tds_read_b64_tr_b16 %7, %8 offset:%16\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3), "=&v"(x4), "=&v"(x5), "=&v"(x6), "=&v"(x7)
        : "v"(vbase[DT]), "n"(0), "n"(8 * RB), "n"(16 * RB), "n"(24 * RB), "n"(32 * RB), "n"(40 * RB),
          "n"(48 * RB), "n"(56 * RB)
        : "memory");
    const u16x8 a0 = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    const u16x8 a1 = {x2[0], x2[1], x2[2], x2[3], x3[0], x3[1], x3[2], x3[3]};
    const u16x8 a2 = {x4[0], x4[1], x4[2], x4[3], x5[0], x5[1], x5[2], x5[3]};
    const u16x8 a3 = {x6[0], x6[1], x6[2], x6[3], x7[0], x7[1], x7[2], x7[3]};
    o[DT] = first ? mfma32(as_bf(a0), pb[0], f32x16{}) : mfma32(as_bf(a0), pb[0], o[DT]);
    o[DT] = mfma32(as_bf(a1), pb[1], o[DT]);
    o[DT] = mfma32(as_bf(a2), pb[2], o[DT]);
    o[DT] = mfma32(as_bf(a3), pb[3], o[DT]);
    pv_steps<DT + 1, D>(vbase, pb, o, first);
  }
}

// LDS byte addresses of pv_steps for a 64-row tile in the permuted layout
// (the value tile of AttnSmem)
template <int D>
BSA_DEV void pv_bases(const uint16_t* tile, uint32_t (&vbase)[D / 32]) {
  const int lane = lane_id();
  const int s = lane & 15, g = lane >> 4, h = lane >> 5;
  const int row = 4 * h + (s >> 2);
  const uint32_t b0 = lds_addr(tile) + (uint32_t)(row * D * 2 + 8 * (s & 1));
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const int piece = 4 * dt + 2 * (g & 1) + ((s & 3) >> 1);
    vbase[dt] = b0 + (uint32_t)((piece ^ vswz<D>(row)) * 16);
  }
}

// O^T (D x 32 queries) += V^T P^T for one 64-key tile; p0/p1 hold P^T in the
// S^T result layout.  With `first` the accumulators start from zero.  The
// tile's per-query sum of the (bf16) probabilities -- the same weights the
// product uses -- comes from four more MFMAs with an all-ones A operand and is
// added to l.
template <int D>
BSA_DEV void pv_tile(const uint16_t* vt, const f32x16& p0, const f32x16& p1, f32x16 (&o)[D / 32], bool first,
                     float& l) {
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
  uint32_t vbase[D / 32];
  pv_bases<D>(vt, vbase);
  pv_steps<0, D>(vbase, pb, o, first);
}

// key index (within a 64-key tile) held by result register i of this lane
BSA_DEV int krow(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }
// the same less the lane's 4h: a constant for an unrolled i, so that masks
// compare against limit - 4h instead of holding 16 row indices per lane
BSA_DEV constexpr int krow0(int i) { return 8 * (i >> 2) + (i & 3); }

// Scores of the tile's keys at or past `lim` (tile-relative) -> -inf.
BSA_DEV void mask_tile(f32x16& s0, f32x16& s1, int lim, int h) {
  const int l2 = lim - 4 * h;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    s0[i] = krow0(i) < l2 ? s0[i] : -INFINITY;
    s1[i] = krow0(i) + 32 < l2 ? s1[i] : -INFINITY;
  }
}

// Online-softmax update of one lane's query column.  s0/s1 hold raw scores
// (masked entries already -inf); sl2 = softmax scale * log2(e) is applied
// inside the exponent.  On return s0/s1 hold the probabilities
// P = 2^(s * sl2 - m) (0 where masked).  The running max m is set by the
// first tile and afterwards moves only when a score passes it by more than
// kRescaleLog2 (then l and the accumulators are rescaled, in a branch the
// wave takes only when one of its rows needs it): P stays at most 2^8, and
// the (m, l) the partial is stored with is whatever m ended up as.  The
// tile's own sum of P is added by pv_tile.
constexpr float kRescaleLog2 = 8.0f;

template <int D>
BSA_DEV void softmax_update(f32x16& s0, f32x16& s1, float& m, float& l, f32x16 (&o)[D / 32], float sl2,
                            bool first) {
  float tmax = max_raw(s0[0], s1[0]);
#pragma unroll
  for (int i = 1; i < 16; ++i) tmax = max3_raw(tmax, s0[i], s1[i]);
  tmax = max_halves(tmax);
  const float tm = tmax * sl2;
  if (first) {
    m = tm;
  } else {
    const bool grow = tm > m + kRescaleLog2;
    if (__ballot(grow) != 0ull) {
      const float mnew = grow ? tm : m;
      const float corr = __builtin_amdgcn_exp2f(m - mnew);
      l *= corr;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) o[dt] *= corr;
      m = mnew;
    }
  }
  if (m == -INFINITY) {
    // no visible key yet in this row
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = 0.f;
      s1[i] = 0.f;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    s0[i] = __builtin_amdgcn_exp2f(fmaf(s0[i], sl2, -m));
    s1[i] = __builtin_amdgcn_exp2f(fmaf(s1[i], sl2, -m));
  }
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
  // two tile buffers for blocks longer than a tile (the next tile is copied
  // by DMA while the current one is computed); one otherwise
  __shared__ __attribute__((aligned(16))) AttnSmem<D> sm[W == 8 ? 2 : 1];
  __shared__ __attribute__((aligned(16))) QStage<D, W> qst;
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
  int staged = -1;  // bucket whose single key tile sits in LDS (in sm[cur])
  int tb = 0;       // the buffer the next tile goes to (alternating across items)
  int cur = 0;      // the buffer holding the tile being computed

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
        // for the first: its buffer was last read two tiles ago, before the
        // previous tile's barrier), then the next tile's DMA goes to the
        // other buffer, which every wave is done with past this barrier
        if (kt0 == 0) dma_kv<D, 64 * W>(sm[tb], kb, p.ks_t, vb, p.vs_t, key0, n_keys);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        cur = tb;
        tb ^= 1;
        if (kt0 + KT < n_keys) dma_kv<D, 64 * W>(sm[tb], kb, p.ks_t, vb, p.vs_t, key0 + kt0 + KT, n_keys - kt0 - KT);
        staged = -1;
      } else if (!(single && staged == bucket)) {
        __syncthreads();
        stage_kv<D, 64 * W>(sm[tb], kb, p.ks_t, vb, p.vs_t, key0 + kt0, n_keys - kt0);
        __syncthreads();
        cur = tb;
        if (W == 8) tb ^= 1;
        staged = single ? bucket : -1;
      }
      // keys of the tile this row may see (past n_keys or after the query: none)
      const int lim = min(n_keys - kt0, p.causal ? qpos - key0 - kt0 + 1 : KT);
      // a wave whose rows all lie before this tile (the query's own block)
      // skips it
      const bool tile_on = wave_on && __ballot(g.valid && lim > 0) != 0ull;
      f32x16 s0, s1;
      // the MFMA phases (scores, P.V) issue at a raised wave priority: a wave
      // of the SIMD that is in its softmax (VALU) then fills the issue slots
      // the other wave's MFMAs leave, instead of both waves contending for
      // the same unit in lockstep after each tile barrier
      if (tile_on) {
        __builtin_amdgcn_s_setprio(1);
        qk_tile<D>(sm[cur], qf, s0, s1);
        __builtin_amdgcn_s_setprio(0);
      }
      if (kt0 == 0 && has_next) {
        // queries of the next item into this wave's LDS staging area
        g_n = grow_of(p, rec_n, ent_n, lrow);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // earlier reads of the staging area are done
        prefetch_q_lds<D, W>(qst, q_row<D>(p, rec_n, g_n), g_n.valid);
      }
      if (tile_on) {
        // mask only where a key can be past the end or after the query
        // (ragged last tile, or the query's own block); wave-uniform test
        if (__ballot(g.valid && lim < KT) != 0ull) mask_tile(s0, s1, lim, hq);
        softmax_update<D>(s0, s1, m, l, o, p.sl2, kt0 == 0);
        __builtin_amdgcn_s_setprio(1);
        pv_tile<D>(sm[cur].v, s0, s1, o, kt0 == 0, l);
        __builtin_amdgcn_s_setprio(0);
      }
    }
    // epilogue: pack this item's outputs, take the next item's queries out of
    // the staging area, then reuse the area to write whole partial rows
    u16x4_t pk[D / 8];
    const int pex = pack_partials<D>(o, pk);
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
        __builtin_nontemporal_store(f32x2{m + (float)pex, __builtin_amdgcn_ldexpf(l, -pex)},
                                    reinterpret_cast<f32x2*>(&p.part_ml[pidx]));
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
// each block in LDS for one or two rows of a 32-row tile.  Here one wave takes
// one work item and streams its block from HBM as the decode attention does:
// v_mfma_f32_16x16x32_bf16 with the block's keys as the A operand of
// S^T = K Q^T, loaded straight into registers (lane l: key 16 kt + l % 16,
// head dims 32 ks + 8 (l / 16) ..), the item's rows as the 16 columns (its
// query rows, 16 at a time; most items hold one or two), and each 64-key
// tile of values copied by DMA into LDS and read transposed for
// O^T += V^T P^T (keys 32 s + 4 g + i and 32 s + 16 + 4 g + i of the B
// operand P^T, g = lane / 16, as in the decode attention).  Online softmax
// per column with the lazy rescale of the MFMA gather; per-key causal masks.
// The partials have the gather's format (16-bit with a row exponent, and
// (m', l') in the log2 domain).  No workgroup barrier, so many items per CU
// are in flight: two waves per SIMD (226 registers at D = 128; three spill),
// 16 KB of LDS per wave.
// DMA of a 64-row tile of consecutive rows (defined with the backward)
template <int D, bool PAD>
BSA_DEV void dma_rows(uint16_t* tile, const uint16_t* base, int64_t rs, int row0, int n_valid, int i);

template <int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void attn_sparse_kernel(AttnParams p) {
  constexpr int KS = D / 32;  // 32-dim steps of a key row
  constexpr int DT = D / 16;  // 16-dim tiles of the output
  constexpr int RB = 2 * D;   // bytes per value row in LDS
  constexpr int NV = KT * D / 8 / 64;  // DMA instructions per value tile
  __shared__ __attribute__((aligned(16))) uint16_t s_v[KT * D];
  const int it_lo = p.tile_off[(int64_t)p.c0 * p.Nb];
  const int nitems = p.tile_off[(int64_t)p.c1 * p.Nb] - it_lo;
  const int item = (int)blockIdx.x;
  if (item >= nitems) return;  // uniform
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
  const int lane = lane_id(), col = lane & 15, g = lane >> 4;
  // LDS byte address of this lane's transposing reads (see the decode
  // attention): row 4 g + col / 4, head dims 16 dt + 4 (col % 4) ..
  const int vrow = 4 * g + (col >> 2);
  const uint32_t vbase = lds_addr(s_v) + (uint32_t)(vrow * RB + 8 * (col & 1));
  const int vpc = (col & 3) >> 1;
  const int vsw = vswz<D>(vrow);
  for (int r0 = 0; r0 < rec.z; r0 += 16) {
    // column col = row r0 + col of the item
    const int lr = r0 + col;
    const bool cv = lr < rec.z;
    const GRow gr = grow_of(p, rec, entry_of(p, rec, lr), lr);
    const int qpos = (p.causal && cv) ? p.Lk - p.Lq + gr.t : 0x7FFFFFFF;
    bf16x8 qf[KS];
    {
      const uint16_t* qr = q_row<D>(p, rec, gr) + 8 * g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf(cv ? ld16(qr + 32 * ks) : u16x8{0, 0, 0, 0, 0, 0, 0, 0});
    }
    float m = -INFINITY, l = 0.f;
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int t0 = 0; t0 < n_keys; t0 += KT) {
      const int nt = min(KT, n_keys - t0);
      // values by DMA into LDS (the previous tile's P.V waited for its own
      // reads), keys straight into the A operands, all in flight together
#pragma unroll
      for (int i = 0; i < NV; ++i) dma_rows<D, false>(s_v, vb, p.vs_t, key0 + t0, nt, i);
      bf16x8 kf[4][KS];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const int key = 16 * kt + col;
        const uint16_t* kr = kb + (int64_t)(key0 + t0 + (key < nt ? key : 0)) * p.ks_t + 8 * g;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kf[kt][ks] = as_bf(key < nt ? ld16(kr + 32 * ks) : u16x8{0, 0, 0, 0, 0, 0, 0, 0});
      }
      f32x4 sc[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        sc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sc[kt] = mfma16(kf[kt][ks], qf[ks], sc[kt]);
      }
      // keys past the block or after the column's query -> -inf (key
      // t0 + 16 kt + 4 g + i of the block)
      const int rel = qpos - (key0 + t0);  // the column's query, relative to the tile
      const int lim = rel >= nt - 1 ? nt : rel + 1;
      if (lim < KT) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[kt][i] = 16 * kt + 4 * g + i < lim ? sc[kt][i] : -INFINITY;
      }
      float tmax = max_raw(sc[0][0], sc[0][1]);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = (kt == 0 ? 2 : 0); i < 4; i += 2) tmax = max3_raw(tmax, sc[kt][i], sc[kt][i + 1]);
      tmax = max_raw(tmax, __shfl_xor(tmax, 16, 64));
      tmax = max_raw(tmax, __shfl_xor(tmax, 32, 64));
      const float tm = tmax * p.sl2;
      if (t0 == 0) {
        m = tm;
      } else {
        const bool grow = tm > m + kRescaleLog2;
        if (__ballot(grow) != 0ull) {
          const float mnew = grow ? tm : m;
          const float corr = __builtin_amdgcn_exp2f(m - mnew);
          l *= corr;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[dt] *= corr;
          m = mnew;
        }
      }
      bf16x8 pb[2];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pr = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(fmaf(sc[kt][i], p.sl2, -m));
          pb[kt >> 1][4 * (kt & 1) + i] = (__bf16)pr;
        }
      {
        const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                             (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
        f32x4 rsum = mfma16(ones, pb[0], f32x4{0.f, 0.f, 0.f, 0.f});
        rsum = mfma16(ones, pb[1], rsum);
        l += rsum[0];
      }
      // the values' copy must have landed (see the decode attention)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const uint32_t va = vbase + (uint32_t)(((2 * dt + vpc) ^ vsw) * 16);
        u16x4 x0, x1, x2, x3;
        asm volatile(
            "ds_read_b64_tr_b16 %0, %4 offset:0\n\tds_read_b64_tr_b16 %1, %4 offset:%5\n\t"
            "ds_read_b64_tr_b16 %2, %4 offset:%6\n\tds_read_b64_tr_b16 %3, %4 offset:%7\n\ts_waitcnt lgkmcnt(0)"
            : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3)
            : "v"(va), "n"(16 * RB), "n"(32 * RB), "n"(48 * RB)
            : "memory");
        const u16x8 a0 = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        const u16x8 a1 = {x2[0], x2[1], x2[2], x2[3], x3[0], x3[1], x3[2], x3[3]};
        o[dt] = mfma16(as_bf(a0), pb[0], o[dt]);
        o[dt] = mfma16(as_bf(a1), pb[1], o[dt]);
      }
    }
    // partial row of column col: 16-bit with the row's exponent (its D dims
    // sit in the four lanes col, col + 16, col + 32, col + 48), then (m', l')
    float mx = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(o[dt][i]));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const int ex = part_exponent(mx);
    if (cv) {
      const int hsel = p.per_group ? 0 : gr.hs - hk * p.G;
      const int64_t prow = (prow_base + hsel) * p.CT + (gr.t - t_base);
      const int64_t pidx = (prow * p.kslot + gr.slot) * p.R + gr.rr;
      uint16_t* dst = p.part_o + pidx * D + 4 * g;
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const u32x2 pk = {pack_norm2(o[dt][0], o[dt][1], ex), pack_norm2(o[dt][2], o[dt][3], ex)};
        __builtin_nontemporal_store(pk, reinterpret_cast<u32x2*>(dst + 16 * dt));
      }
      if (g == 0) {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        __builtin_nontemporal_store(f32x2{m + (float)ex, __builtin_amdgcn_ldexpf(l, -ex)},
                                    reinterpret_cast<f32x2*>(&p.part_ml[pidx]));
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
  // token's G output heads are adjacent; every index fits 32 bits (the plan
  // bounds the query rows below 2^31), so the divisions are 32-bit ones
  const unsigned nrows = (unsigned)(p.c1 - p.c0) * (unsigned)p.CT * (unsigned)p.G;
  const unsigned row = (blockIdx.x * 4u + (unsigned)w) * RPW + (unsigned)(lane / LPR);
  const unsigned rr_ = row < nrows ? row : 0u;
  const unsigned q_g = rr_ / (unsigned)p.G;
  const int hh = (int)(rr_ - q_g * (unsigned)p.G);
  const unsigned c_rel_u = q_g / (unsigned)p.CT;
  const int t_loc = (int)(q_g - c_rel_u * (unsigned)p.CT);
  const int c_rel = (int)c_rel_u;
  const int cid = p.c0 + c_rel;
  const int bh = (int)((unsigned)cid / (unsigned)p.NC);
  const int t = (cid - bh * p.NC) * p.CT + t_loc;
  const bool ok = row < nrows && t < p.Lq;
  const int b = (int)((unsigned)bh / (unsigned)p.Hkv), hk = bh - b * p.Hkv;
  const int h = hk * p.G + hh;
  const int rr = p.per_group ? hh : 0;
  const int64_t prow = ((int64_t)c_rel * p.Gs + (p.per_group ? 0 : hh)) * p.CT + t_loc;
  // number of valid slots: the gate keeps min(topk, candidates) blocks, then
  // the forced own block when causal (the valid entries of a selection row
  // come first), so the count follows from the token's position alone
  int n = 0;
  if (ok) {
    const int ncand = p.causal ? min((p.Lk - p.Lq + t) / p.block, p.Nb) : p.Nb;
    n = min(p.topk, ncand) + (p.causal ? 1 : 0);
  }
  // the row's slot 0; slot s is s * R records further
  const int64_t pidx0 = prow * p.kslot * p.R + rr;
  const float2* ml0 = p.part_ml + pidx0;
  const uint16_t* o0 = p.part_o + pidx0 * D + li * 8;
  // partial s holds q_s = 32767 * 2^-E_s * sum_k p_k v_k with p = 2^(score*sl2 - m_s), and
  // (m_s + E_s, 2^-E_s * sum_k p_k)
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
        // streaming loads: every partial is read exactly once
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        const f32x2 v2 = __builtin_nontemporal_load(reinterpret_cast<const f32x2*>(ml0 + s * p.R));
        ml[u] = make_float2(v2[0], v2[1]);
        ov[u] = __builtin_nontemporal_load(reinterpret_cast<const u16x8*>(o0 + (int64_t)(s * p.R) * D));
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
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(wu, (float)(int16_t)ov[u][e], acc[e]);
    }
    M = mb;
  }
  if (!ok) return;
  // the stored partials are 32767 * (partial) * 2^-E; E is folded into (m', l')
  const float inv = W > 0.f ? 1.0f / (W * 32767.0f) : 0.f;
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
    const unsigned grid = (unsigned)p.sparse_items;  // one wave per item
    if (p.D == 128)
      hipLaunchKernelGGL(attn_sparse_kernel<128>, dim3(grid), dim3(64), 0, s, p);
    else
      hipLaunchKernelGGL(attn_sparse_kernel<64>, dim3(grid), dim3(64), 0, s, p);
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
// Backward through the fixed selection, on bf16 MFMA with fp32 accumulation.
// With the forward's log-sum-exp lse_r of row r and delta_r = dout_r . o_r:
//   p_rk = exp(scale q_r . k_k - lse_r),  dp_rk = dout_r . v_k,
//   ds_rk = p_rk (dp_rk - delta_r),
//   dq_r = scale sum_k ds_rk k_k,  dk_k = scale sum_r ds_rk q_r,
//   dv_k = sum_r p_rk dout_r,
// the sums running over the (row, key) pairs the forward attended.  A
// bucket's entries (one query chunk's rows that chose one (b, kv head,
// block)) are sorted first, so every sum runs in a fixed order and two calls
// give the same bits.
//  * attn_bwd_dkv: one workgroup per (b, kv head, block, 32W keys).  Wave w
//    holds keys 32w .. 32w+31 of the unit (their k and v rows as MFMA
//    operands in registers) and their dk^T, dv^T accumulators; the workgroup
//    walks every row that chose the block -- the block's buckets in query
//    chunk order, each bucket's sorted entries -- 64 rows at a time.  A batch
//    of gathered q and dout rows is copied by DMA into LDS twice: padded
//    rows for S = Q K^T and dP = dO V^T, and rows with permuted pieces for the
//    transposing reads of dV^T += dO^T P and dK^T += Q^T dS.  The next
//    batch's copy runs during the current batch's MFMAs.  dk and dv are
//    written once per key.
//  * attn_bwd_dq: the forward's work items (a bucket's rows, 32 per wave);
//    a wave holds its rows' q and dout as MFMA operands, the block streams
//    through LDS in 64-key tiles (keys padded and permuted, values padded),
//    and S^T = K Q^T, dP^T = V dO^T, dQ^T += K^T dS^T.  One fp32 partial per
//    (row, slot); bwd_dq_reduce sums a row's slots in slot order.
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

// One batch of 64 gathered rows of the dk / dv kernel.
template <int D>
struct BwdRows {
  uint16_t qp[64 * (D + 8)];  // q rows, padded (row-wise operand reads)
  uint16_t gp[64 * (D + 8)];  // dout rows, padded
  uint16_t qs[64 * D];        // q rows, pieces permuted (transposing reads)
  uint16_t gs[64 * D];        // dout rows, pieces permuted
  float lse[64];              // the rows' log-sum-exp (natural log)
  float dl[64];               // the rows' delta
  uint32_t ent[64];           // the rows' entry words (0 past the batch's rows)
};
static_assert(offsetof(BwdRows<128>, dl) == offsetof(BwdRows<128>, lse) + 256 &&
                  offsetof(BwdRows<128>, ent) == offsetof(BwdRows<128>, lse) + 512 &&
                  offsetof(BwdRows<64>, dl) == offsetof(BwdRows<64>, lse) + 256 &&
                  offsetof(BwdRows<64>, ent) == offsetof(BwdRows<64>, lse) + 512,
              "bwd_row_stats reads lse, dl and ent at fixed distances");

// DMA instruction i of a 64-row tile of gathered rows: row r's first
// 16-byte piece sits at piece offset `off` of `base`, held by lane r of the
// wave.  PAD: rows of D + 8 elements (a padding piece loads piece 0 of its
// row); otherwise rows of D elements with piece c of row r at c ^ vswz(r).
template <int D, bool PAD>
BSA_DEV void dma_gathered(uint16_t* tile, const uint16_t* base, uint32_t off, int i) {
  constexpr int RP = PAD ? D / 8 + 1 : D / 8;
  const int P = i * 64 + lane_id();
  const int r = P / RP;
  int c = P % RP;
  if constexpr (PAD) c = c == RP - 1 ? 0 : c;
  else c ^= vswz<D>(r);
  const uint32_t ro = (uint32_t)__shfl((int)off, r, 64);
  __builtin_amdgcn_global_load_lds((const void*)(base + ((int64_t)ro << 3) + c * 8), (lds_ptr_t)(tile + i * 512), 16,
                                   0, 0);
}

// DMA instruction i of a 64-row tile of consecutive rows row0 .. row0+63 of
// `base` (row stride rs elements); rows past n_valid load row row0.
template <int D, bool PAD>
BSA_DEV void dma_rows(uint16_t* tile, const uint16_t* base, int64_t rs, int row0, int n_valid, int i) {
  constexpr int RP = PAD ? D / 8 + 1 : D / 8;
  const int P = i * 64 + lane_id();
  const int r = P / RP;
  int c = P % RP;
  if constexpr (PAD) c = c == RP - 1 ? 0 : c;
  else c ^= vswz<D>(r);
  const int rr = r < n_valid ? r : 0;
  __builtin_amdgcn_global_load_lds((const void*)(base + (int64_t)(row0 + rr) * rs + c * 8),
                                   (lds_ptr_t)(tile + i * 512), 16, 0, 0);
}

// pv_steps over a permuted 64-row tile with the B operand taken from two
// 32x32 result tiles (rows 0..31 in x0, 32..63 in x1), rounded to bf16
template <int D>
BSA_DEV void pv_acc(const uint16_t* tile, const f32x16& x0, const f32x16& x1, f32x16 (&o)[D / 32]) {
  bf16x8 pb[4];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    pb[0][e] = (__bf16)x0[e];
    pb[1][e] = (__bf16)x0[8 + e];
    pb[2][e] = (__bf16)x1[e];
    pb[3][e] = (__bf16)x1[8 + e];
  }
  uint32_t vbase[D / 32];
  pv_bases<D>(tile, vbase);
  pv_steps<0, D>(vbase, pb, o, false);
}

BSA_DEV float lse_log2(float lse) {
  // rows with no visible key carry lse = -inf: no probability anywhere
  return lse == -INFINITY ? INFINITY : lse * 1.4426950408889634f;
}

// Stores a 32x32 result tile set (rows 32dt + krow(i, h) of column lane%32)
// as fp32 rows: dst points at the column's row of D elements.
template <int D>
BSA_DEV void store_cols(float* dst, const f32x16 (&o)[D / 32], float mul) {
  const int h = lane_id() >> 5;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<f32x4*>(dst + 32 * dt + 8 * q + 4 * h) =
          f32x4{o[dt][4 * q], o[dt][4 * q + 1], o[dt][4 * q + 2], o[dt][4 * q + 3]} * mul;
}

// lse and delta of the lane's 32 result rows of a batch, rows
// 8(q&3) + 4h + 32(q>>2) .. +3 in ls[q] / dl[q] (base = address of lse[4h]);
// LDS reads through asm, as for the key / value tiles, so that they do not
// wait for the next batch's copy
BSA_DEV void bwd_row_stats(uint32_t base, f32x4 (&ls)[8], f32x4 (&dl)[8]) {
  asm volatile(
      "ds_read_b128 %0, %16 offset:0\n\tds_read_b128 %1, %16 offset:32\n\t"
      "ds_read_b128 %2, %16 offset:64\n\tds_read_b128 %3, %16 offset:96\n\t"
      "ds_read_b128 %4, %16 offset:128\n\tds_read_b128 %5, %16 offset:160\n\t"
      "ds_read_b128 %6, %16 offset:192\n\tds_read_b128 %7, %16 offset:224\n\t"
      "ds_read_b128 %8, %16 offset:256\n\tds_read_b128 %9, %16 offset:288\n\t"
      "ds_read_b128 %10, %16 offset:320\n\tds_read_b128 %11, %16 offset:352\n\t"
      "ds_read_b128 %12, %16 offset:384\n\tds_read_b128 %13, %16 offset:416\n\t"
      "ds_read_b128 %14, %16 offset:448\n\tds_read_b128 %15, %16 offset:480\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(ls[0]), "=&v"(ls[1]), "=&v"(ls[2]), "=&v"(ls[3]), "=&v"(ls[4]), "=&v"(ls[5]), "=&v"(ls[6]), "=&v"(ls[7]),
        "=&v"(dl[0]), "=&v"(dl[1]), "=&v"(dl[2]), "=&v"(dl[3]), "=&v"(dl[4]), "=&v"(dl[5]), "=&v"(dl[6]), "=&v"(dl[7])
      : "v"(base)
      : "memory");
}

// the rows' entry words, in the same arrangement (ent follows dl)
BSA_DEV void bwd_row_ents(uint32_t base, u32x4 (&en)[8]) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:512\n\tds_read_b128 %1, %8 offset:544\n\t"
      "ds_read_b128 %2, %8 offset:576\n\tds_read_b128 %3, %8 offset:608\n\t"
      "ds_read_b128 %4, %8 offset:640\n\tds_read_b128 %5, %8 offset:672\n\t"
      "ds_read_b128 %6, %8 offset:704\n\tds_read_b128 %7, %8 offset:736\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(en[0]), "=&v"(en[1]), "=&v"(en[2]), "=&v"(en[3]), "=&v"(en[4]), "=&v"(en[5]), "=&v"(en[6]), "=&v"(en[7])
      : "v"(base)
      : "memory");
}

// Batch cursor of the dk / dv kernel (wave-uniform): query chunk c (NC =
// done), first row of the batch within the bucket, the bucket's rows and its
// first entry.
struct BwdCursor {
  int c, start, rows, eoff;
};

BSA_DEV void bwd_seek(const AttnParams& p, int64_t bh, int j, int c, BwdCursor& s) {
  const const_int_ptr off = (const const_int_ptr)p.bucket_off;
  for (; p.grid > 0 && c < p.NC; ++c) {  // grid 0: no selection entries, nothing built
    const int64_t bk = (bh * p.NC + c) * p.Nb + j;
    const int a = off[bk];
    const int n = (off[bk + 1] - a) << p.lgR;
    if (n > 0) {
      s = BwdCursor{c, 0, n, a};
      return;
    }
  }
  s = BwdCursor{p.NC, 0, 0, 0};
}

BSA_DEV void bwd_advance(const AttnParams& p, int64_t bh, int j, BwdCursor& s) {
  if (s.start + 64 < s.rows) s.start += 64;
  else bwd_seek(p, bh, j, s.c + 1, s);
}

// entry word of this lane's row (row = lane) of the cursor's batch; rows
// past the bucket's end read the batch's first row
BSA_DEV uint32_t bwd_entry(const AttnParams& p, const BwdCursor& s) {
  if (s.c >= p.NC) return 0u;
  const int lr = s.start + lane_id();
  const int lrc = lr < s.rows ? lr : s.start;
  return p.entries[s.eoff + (lrc >> p.lgR)];
}

template <int D, int W>
BSA_DEV void bwd_issue_batch(const AttnParams& p, BwdRows<D>& buf, const BwdCursor& s, uint32_t ent, int b, int hk) {
  const int lane = lane_id();
  const int wu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = s.start + lane;
  const bool valid = lr < s.rows;
  const int lrc = valid ? lr : s.start;
  const int rr = lrc & ((1 << p.lgR) - 1);
  const int t = (int)(ent >> p.sh_t);
  const int hh = (int)((ent >> p.sh_h) & ((1u << (p.sh_t - p.sh_h)) - 1u));
  const int qh = p.per_group ? hk * p.G + rr : hk * p.G + hh;
  const uint32_t qo = (uint32_t)(((int64_t)b * p.qs_b + (int64_t)t * p.qs_t + (int64_t)qh * p.qs_h) >> 3);
  const uint32_t go = (uint32_t)(((int64_t)b * p.dos_b + (int64_t)t * p.dos_t + (int64_t)qh * p.dos_h) >> 3);
  const int64_t orow = ((int64_t)b * p.Hq + qh) * p.Lq + t;
  constexpr int NP = D / 8 + 1, NS = D / 8, N = 2 * NP + 2 * NS + 2;
  for (int i = wu; i < N; i += W) {
    if (i < NP) dma_gathered<D, true>(buf.qp, p.q, qo, i);
    else if (i < 2 * NP) dma_gathered<D, true>(buf.gp, p.dout, go, i - NP);
    else if (i < 2 * NP + NS) dma_gathered<D, false>(buf.qs, p.q, qo, i - 2 * NP);
    else if (i < 2 * NP + 2 * NS) dma_gathered<D, false>(buf.gs, p.dout, go, i - 2 * NP - NS);
    else if (i == 2 * NP + 2 * NS)
      __builtin_amdgcn_global_load_lds((const void*)(p.lse_in + orow), (lds_ptr_t)buf.lse, 4, 0, 0);
    else __builtin_amdgcn_global_load_lds((const void*)(p.delta + orow), (lds_ptr_t)buf.dl, 4, 0, 0);
  }
  if (wu == 0) buf.ent[lane] = valid ? ent : 0u;
}

template <int D, int W>
__global__ __launch_bounds__(64 * W, 1) void attn_bwd_dkv_kernel(AttnParams p, int nkt) {
  __shared__ __attribute__((aligned(16))) BwdRows<D> rb[2];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, h = lane >> 5;
  // unit groups (j, bh), group g = j * BH + bh, each of nkt key slices:
  // group g runs on XCD g % 8 (workgroup i runs on XCD i % 8), so that the
  // slices of one block share its rows through that XCD's L2, and every XCD
  // takes the groups in order of j -- low blocks first (under causal
  // selection they collect the most rows) and the heavy ones spread over
  // all XCDs
  const int BH = p.B * p.Hkv;
  const int slot = blockIdx.x >> 3;
  const int64_t grp = (int64_t)(slot / nkt) * 8 + (blockIdx.x & 7);
  if (grp >= (int64_t)p.Nb * BH) return;  // padding of the grid; uniform
  const int kt = slot % nkt;
  const int bh = (int)(grp % BH);
  const int j = (int)(grp / BH);
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const int key0 = j * p.block + kt * 32 * W;
  const int n_keys = min(min(32 * W, p.block - kt * 32 * W), p.Lk - key0);
  if (n_keys <= 0) return;  // a slice past the end of a ragged last block; uniform
  const bool wave_on = 32 * w < n_keys;
  // this lane's key (column lane%32 of the wave's tiles) as B operands
  const int kcol = 32 * w + (lane & 31);
  const int key = key0 + kcol;
  bf16x8 kf[D / 16], vf[D / 16];
  load_qf<D>(p.k + (int64_t)b * p.ks_b + (int64_t)key * p.ks_t + (int64_t)hk * p.ks_h, kcol < n_keys, kf);
  load_qf<D>(p.v + (int64_t)b * p.vs_b + (int64_t)key * p.vs_t + (int64_t)hk * p.vs_h, kcol < n_keys, vf);
  // a row sees this key when its token t >= key - (Lk - Lq), i.e. when its
  // entry word is at least tk << sh_t
  const int tk = key - (p.Lk - p.Lq);
  const uint32_t ent_min = (p.causal && tk > 0) ? (uint32_t)tk << p.sh_t : 0u;
  // the wave's last key: a batch whose first (lowest) token sees it needs no mask
  const int tk_last = min(key0 + 32 * w + 31, key0 + n_keys - 1) - (p.Lk - p.Lq);
  f32x16 dkt[D / 32], dvt[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dkt[dt] = dvt[dt] = f32x16{};

  BwdCursor nx;
  bwd_seek(p, bh, j, 0, nx);
  bool have = nx.c < p.NC;
  int nv = have ? min(64, nx.rows - nx.start) : 0;
  if (have) {
    const uint32_t e0 = bwd_entry(p, nx);
    bwd_issue_batch<D, W>(p, rb[0], nx, e0, b, hk);
    bwd_advance(p, bh, j, nx);
  }
  uint32_t ent_n = bwd_entry(p, nx);
  for (int n = 0; have; ++n) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // batch n is in rb[n & 1]; every wave is done with rb[(n + 1) & 1]
    const bool have_n = nx.c < p.NC;
    int nv_n = 0;
    if (have_n) {
      bwd_issue_batch<D, W>(p, rb[(n + 1) & 1], nx, ent_n, b, hk);
      nv_n = min(64, nx.rows - nx.start);
      bwd_advance(p, bh, j, nx);
      ent_n = bwd_entry(p, nx);
    }
    if (wave_on) {
      const BwdRows<D>& bf = rb[n & 1];
      f32x16 s0, s1, d0, d1;
      qk_tile_pad<D>(bf.qp, kf, s0, s1);
      qk_tile_pad<D>(bf.gp, vf, d0, d1);
      // the batch's rows are sorted by token: the first has the lowest
      const uint32_t sbase = lds_addr(&bf.lse[4 * h]);
      uint32_t ent0;
      asm volatile("ds_read_b32 %0, %1 offset:%2\n\ts_waitcnt lgkmcnt(0)"
                   : "=&v"(ent0)
                   : "v"(lds_addr(bf.ent)), "n"(0)
                   : "memory");
      const bool msk = nv < 64 || (p.causal && (int)(ent0 >> p.sh_t) < tk_last);
      f32x4 ls[8], dl[8];
      bwd_row_stats(sbase, ls, dl);
      u32x4 en[8];
      if (msk) bwd_row_ents(sbase, en);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int r0 = 8 * (q & 3) + 4 * h + 32 * (q >> 2);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f32x16& s = q < 4 ? s0 : s1;
          f32x16& d = q < 4 ? d0 : d1;
          const int i = 4 * (q & 3) + e;
          float pr = __builtin_amdgcn_exp2f(fmaf(s[i], p.sl2, -lse_log2(ls[q][e])));
          if (msk && !(r0 + e < nv && en[q][e] >= ent_min)) pr = 0.f;
          s[i] = pr;
          d[i] = pr * (d[i] - dl[q][e]);
        }
      }
      pv_acc<D>(bf.gs, s0, s1, dvt);
      pv_acc<D>(bf.qs, d0, d1, dkt);
    }
    have = have_n;
    nv = nv_n;
  }
  if (kcol < n_keys) {
    const int64_t orow = (((int64_t)b * p.Lk + key) * p.Hkv + hk) * D;
    store_cols<D>(p.dk + orow, dkt, p.scale);
    store_cols<D>(p.dv + orow, dvt, 1.f);
  }
}

// One 64-key tile of the dq kernel
template <int D>
struct BwdKv {
  uint16_t kp[KT * (D + 8)];  // keys, padded
  uint16_t vp[KT * (D + 8)];  // values, padded
  uint16_t ks[KT * D];        // keys, pieces permuted
};

template <int D, int W>
BSA_DEV void dma_bwd_kv(BwdKv<D>& sm, const uint16_t* kb, int64_t ks_t, const uint16_t* vb, int64_t vs_t, int row0,
                        int n_valid) {
  constexpr int NP = D / 8 + 1, NS = D / 8;
  const int wu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int i = wu; i < 2 * NP + NS; i += W) {
    if (i < NP) dma_rows<D, true>(sm.kp, kb, ks_t, row0, n_valid, i);
    else if (i < 2 * NP) dma_rows<D, true>(sm.vp, vb, vs_t, row0, n_valid, i - NP);
    else dma_rows<D, false>(sm.ks, kb, ks_t, row0, n_valid, i - 2 * NP);
  }
}

template <int D, int W>
__global__ __launch_bounds__(64 * W, 1) void attn_bwd_dq_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(16))) BwdKv<D> sm[2];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, h = lane >> 5;
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
  const int lrow = w * 32 + (lane & 31);
  const GRow g = grow_of(p, rec, entry_of(p, rec, lrow), lrow);
  bf16x8 qf[D / 16], gf[D / 16];
  load_qf<D>(q_row<D>(p, rec, g), g.valid, qf);
  load_qf<D>(p.dout + (int64_t)b * p.dos_b + (int64_t)g.t * p.dos_t + (int64_t)g.qh * p.dos_h, g.valid, gf);
  const int64_t orow = ((int64_t)b * p.Hq + g.qh) * p.Lq + g.t;
  const float lse2 = g.valid ? lse_log2(p.lse_in[orow]) : INFINITY;
  const float dl = g.valid ? p.delta[orow] : 0.f;
  const int qpos = p.Lk - p.Lq + g.t;
  const bool wave_on = w * 32 < rec.z;
  f32x16 dqt[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) dqt[dt] = f32x16{};
  int tb = 0;
  for (int kt0 = 0; kt0 < n_keys; kt0 += KT) {
    // tile kt0 arrives by DMA (issued during the previous tile, or now for
    // the first), then the next tile's DMA goes to the other buffer, which
    // every wave is done with past this barrier
    if (kt0 == 0) dma_bwd_kv<D, W>(sm[0], kb, p.ks_t, vb, p.vs_t, key0, n_keys);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int cur = tb;
    tb ^= 1;
    if (kt0 + KT < n_keys) dma_bwd_kv<D, W>(sm[tb], kb, p.ks_t, vb, p.vs_t, key0 + kt0 + KT, n_keys - kt0 - KT);
    const int lim = min(n_keys - kt0, p.causal ? qpos - key0 - kt0 + 1 : KT);
    if (wave_on && __ballot(g.valid && lim > 0) != 0ull) {
      f32x16 s0, s1, d0, d1;
      qk_tile_pad<D>(sm[cur].kp, qf, s0, s1);
      qk_tile_pad<D>(sm[cur].vp, gf, d0, d1);
      const int l2 = lim - 4 * h;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p0 = krow0(i) < l2 ? __builtin_amdgcn_exp2f(fmaf(s0[i], p.sl2, -lse2)) : 0.f;
        const float p1 = krow0(i) + 32 < l2 ? __builtin_amdgcn_exp2f(fmaf(s1[i], p.sl2, -lse2)) : 0.f;
        d0[i] = p0 * (d0[i] - dl);
        d1[i] = p1 * (d1[i] - dl);
      }
      pv_acc<D>(sm[cur].ks, d0, d1, dqt);
    }
  }
  if (g.valid) {
    const int hsel = p.per_group ? 0 : g.hs - hk * p.G;
    const int64_t prow = (prow_base + hsel) * p.CT + (g.t - t_base);
    const int64_t pidx = (prow * p.kslot + g.slot) * p.R + g.rr;
    store_cols<D>(p.dq_part + pidx * D, dqt, 1.f);
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
  {
    // every (b, kv head, block) unit runs, so that keys nobody attended get zeros
    LaunchScope ls("attn_bwd_dkv", s);
    constexpr int W = kBwdKeyWaves;
    const int nkt = (p.block + 32 * W - 1) / (32 * W);
    const int64_t groups = (int64_t)p.B * p.Hkv * p.Nb;  // (block, b, kv head); 8 per round, one per XCD
    const unsigned grid = (unsigned)((groups + 7) / 8 * 8 * nkt);
    if (p.D == 128) hipLaunchKernelGGL((attn_bwd_dkv_kernel<128, W>), dim3(grid), dim3(64 * W), 0, s, p, nkt);
    else hipLaunchKernelGGL((attn_bwd_dkv_kernel<64, W>), dim3(grid), dim3(64 * W), 0, s, p, nkt);
  }
  if (!launch_ok("attn_bwd_dkv")) return false;
  if (p.grid > 0) {
    LaunchScope ls("attn_bwd_dq", s);
    // grid = the bound on the item count (items are built on the device);
    // workgroups past the built items exit at once
    constexpr int W = kBwdItemRows / 32;
    if (p.D == 128) hipLaunchKernelGGL((attn_bwd_dq_kernel<128, W>), dim3((unsigned)p.grid), dim3(64 * W), 0, s, p);
    else hipLaunchKernelGGL((attn_bwd_dq_kernel<64, W>), dim3((unsigned)p.grid), dim3(64 * W), 0, s, p);
  }
  if (!launch_ok("attn_bwd_dq")) return false;
  {
    LaunchScope ls("bwd_dq_reduce", s);
    const int64_t thr = nrows_out * (p.D / 4);
    const unsigned grid = (unsigned)((thr + 255) / 256);
    if (p.D == 128) hipLaunchKernelGGL(bwd_dq_reduce_kernel<128>, dim3(grid), dim3(256), 0, s, p, nrows_out);
    else hipLaunchKernelGGL(bwd_dq_reduce_kernel<64>, dim3(grid), dim3(256), 0, s, p, nrows_out);
  }
  return launch_ok("bwd_dq_reduce");
}

// ---------------------------------------------------------------------------
// Decode attention on MFMA: one wave per distinct (b, kv head, block) of the
// decode's union, for every query head of the group at once, on
// v_mfma_f32_16x16x32_bf16 (at most 8 of its 16 columns are query heads, so
// the accumulators, scores and operands stay small enough for two or more
// waves per SIMD: one wave's loads are in flight while another computes).
//  * S^T = K Q^T per 16-key tile kt: the A operand is the keys themselves --
//    lane l loads 16 bytes of key row 16 kt + l % 16 (head dims 32 ks +
//    8 (l / 16) ..), straight from the cache into registers -- and B the
//    group's query heads as columns.  Lane l then holds column l % 16 and
//    keys 16 kt + 4 (l / 16) + i, i < 4.
//  * O^T += V^T P^T per 32-key step s: the B operand (P^T) of lane l takes
//    its own probabilities of keys 32 s + 4 g + i and 32 s + 16 + 4 g + i
//    (g = l / 16), rounded to bf16; the A operand (V^T) must list the same
//    keys for head dim 16 dt + l % 16.  Each 64-key tile of values is copied
//    by DMA into LDS (row-major, 16-byte pieces permuted as in the gather)
//    and read with ds_read_b64_tr_b16: in a group of 16 lanes, lane i gets
//    element i % 4 of the 8 bytes that lane i / 4 + 4 e addresses (e < 4),
//    so lane c addressing V[k0 + c / 4][d0 + 4 (c % 4)] hands lane i keys
//    k0 .. k0 + 3 of head dim d0 + i.
//  * Online softmax per column with the gather's lazy rescale; the row sum l
//    comes from the same bf16 probabilities through an all-ones A operand.
// Writes each chosen head's normalised partial and its log2-domain
// log-sum-exp, as the combine reads them.  Three waves per SIMD (168
// registers at D = 128; left to itself the compiler takes 206, two waves).
template <int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(3))) void decode_attend_mfma_kernel(DecodeAttnParams p) {
  constexpr int KS = D / 32;  // 32-dim steps of a key row
  constexpr int DT = D / 16;  // 16-dim tiles of the output
  constexpr int RB = 2 * D;   // bytes per value row in LDS
  __shared__ __attribute__((aligned(16))) uint16_t s_v[KT * D];
  const int bh = blockIdx.x / p.umax, u = blockIdx.x % p.umax;
  if (u >= p.ucount[bh]) return;  // uniform
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const int ent = p.ulist[(int64_t)bh * p.umax + u];
  const int j = ent >> 8, mask = ent & 255;
  int n = p.lens ? p.lens[b] : p.Lc;
  n = n < 1 ? 1 : (n > p.Lc ? p.Lc : n);
  const int ka = j * p.block;
  int nk = min(p.block, n - ka);
  int64_t ko, vo;
  if (p.table) {
    const int pg = p.table[(int64_t)b * p.table_w + j];
    if (pg < 0 || pg >= p.num_pages) nk = 0;  // no keys: nothing is read
    ko = (int64_t)pg * p.ks_b;
    vo = (int64_t)pg * p.vs_b;
  } else {
    ko = (int64_t)b * p.ks_b + (int64_t)ka * p.ks_t;
    vo = (int64_t)b * p.vs_b + (int64_t)ka * p.vs_t;
  }
  // the block's first key and value row
  const uint16_t* kb = p.k + ko + (int64_t)hk * p.ks_h;
  const uint16_t* vb = p.v + vo + (int64_t)hk * p.vs_h;
  const int lane = lane_id(), col = lane & 15, g = lane >> 4;
  // B operand of the scores: column col = query head hk * G + col (zero past G)
  bf16x8 qf[KS];
  {
    const uint16_t* qr = p.q + (int64_t)b * p.qs_b + (int64_t)(hk * p.G + (col < p.G ? col : 0)) * p.qs_h + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf(col < p.G ? ld16(qr + 32 * ks) : u16x8{0, 0, 0, 0, 0, 0, 0, 0});
  }
  // LDS byte address this lane reads for head-dim tile dt of a value tile:
  // row 4 g + col / 4 (+ 16 and + 32 keys as immediate offsets), head dims
  // 16 dt + 4 (col % 4) ..; the piece permutation of a row depends only on
  // the row's low bits, equal for every key offset used
  const int vrow = 4 * g + (col >> 2);
  const uint32_t vbase = lds_addr(s_v) + (uint32_t)(vrow * RB + 8 * (col & 1));
  const int vpc = (col & 3) >> 1;  // piece within the dim tile's two
  const int vsw = vswz<D>(vrow);
  float m = -INFINITY, l = 0.f;
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int NV = KT * D / 8 / 64;  // DMA instructions per value tile
  for (int t0 = 0; t0 < nk; t0 += KT) {
    const int nt = min(KT, nk - t0);
    // the tile's values by DMA into LDS (the previous tile's P.V, which read
    // the buffer, waited for its own reads) and its keys straight into the A
    // operands, all in flight together
#pragma unroll
    for (int i = 0; i < NV; ++i) dma_rows<D, false>(s_v, vb, p.vs_t, t0, nt, i);
    bf16x8 kf[4][KS];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int key = 16 * kt + col;
      const uint16_t* kr = kb + (int64_t)(t0 + (key < nt ? key : 0)) * p.ks_t + 8 * g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[kt][ks] = as_bf(key < nt ? ld16(kr + 32 * ks) : u16x8{0, 0, 0, 0, 0, 0, 0, 0});
    }
    f32x4 sc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sc[kt] = mfma16(kf[kt][ks], qf[ks], sc[kt]);
    }
    // keys at or past nt -> -inf (key 16 kt + 4 g + i)
    if (nt < KT) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[kt][i] = 16 * kt + 4 * g + i < nt ? sc[kt][i] : -INFINITY;
    }
    // column maximum over the tile: the lane's 16 scores, then the four
    // lane groups holding the column
    float tmax = max_raw(sc[0][0], sc[0][1]);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = (kt == 0 ? 2 : 0); i < 4; i += 2) tmax = max3_raw(tmax, sc[kt][i], sc[kt][i + 1]);
    tmax = max_raw(tmax, __shfl_xor(tmax, 16, 64));
    tmax = max_raw(tmax, __shfl_xor(tmax, 32, 64));
    const float tm = tmax * p.sl2;
    if (t0 == 0) {
      m = tm;
    } else {
      const bool grow = tm > m + kRescaleLog2;
      if (__ballot(grow) != 0ull) {
        const float mnew = grow ? tm : m;
        const float corr = __builtin_amdgcn_exp2f(m - mnew);
        l *= corr;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= corr;
        m = mnew;
      }
    }
    // probabilities 2^(s sl2 - m) as the B operands of the two 32-key steps
    bf16x8 pb[2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pr = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(fmaf(sc[kt][i], p.sl2, -m));
        pb[kt >> 1][4 * (kt & 1) + i] = (__bf16)pr;
      }
    {
      const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                           (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
      f32x4 rsum = mfma16(ones, pb[0], f32x4{0.f, 0.f, 0.f, 0.f});
      rsum = mfma16(ones, pb[1], rsum);
      l += rsum[0];
    }
    // the values' copy must have landed: the compiler may order the copy
    // after the key loads, so their wait does not cover it
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint32_t va = vbase + (uint32_t)(((2 * dt + vpc) ^ vsw) * 16);
      u16x4 x0, x1, x2, x3;
      asm volatile(
          "ds_read_b64_tr_b16 %0, %4 offset:0\n\tds_read_b64_tr_b16 %1, %4 offset:%5\n\t"
          "ds_read_b64_tr_b16 %2, %4 offset:%6\n\tds_read_b64_tr_b16 %3, %4 offset:%7\n\ts_waitcnt lgkmcnt(0)"
          : "=&v"(x0), "=&v"(x1), "=&v"(x2), "=&v"(x3)
          : "v"(va), "n"(16 * RB), "n"(32 * RB), "n"(48 * RB)
          : "memory");
      const u16x8 a0 = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
      const u16x8 a1 = {x2[0], x2[1], x2[2], x2[3], x3[0], x3[1], x3[2], x3[3]};
      o[dt] = mfma16(as_bf(a0), pb[0], o[dt]);
      o[dt] = mfma16(as_bf(a1), pb[1], o[dt]);
    }
  }
  if (col < p.G && ((mask >> col) & 1)) {
    const int64_t pidx = ((int64_t)bh * p.umax + u) * p.G + col;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* dst = p.part_o + pidx * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) *reinterpret_cast<f32x4*>(dst + 16 * dt) = o[dt] * inv;
    if (g == 0) p.part_lse[pidx] = l > 0.f ? m + __log2f(l) : -INFINITY;
  }
}

bool launch_decode_attend_mfma(const DecodeAttnParams& p, hipStream_t s) {
  const unsigned grid = (unsigned)(p.B * p.Hkv * p.umax);
  {
    LaunchScope ls("decode_attend", s);
    if (p.D == 128) hipLaunchKernelGGL(decode_attend_mfma_kernel<128>, dim3(grid), dim3(64), 0, s, p);
    else hipLaunchKernelGGL(decode_attend_mfma_kernel<64>, dim3(grid), dim3(64), 0, s, p);
  }
  return launch_ok("decode_attend");
}

}  // namespace bsa
