// Gate: score every candidate block's summary with the gate query and keep
// the top-k per selection row.
//
// MoBA repo card (ross.abutalabs.com/products/moba.json), card.what_it_is:
// MoE-style top-k gating over KV blocks.  "MiniMax released MSA ..."
// (news.hamidun.com), section "How MSA Works": a light index branch picks the
// top-k blocks per query and per GQA group.  Readings where the pages are
// silent: score = dot(gate query, block mean); per group the heads' scores are
// summed, which equals scoring with the summed query; in causal mode only
// blocks before the query's own block compete; ties go to the lower index.
//
// Scores run on bf16 MFMA (16x16x32).  Operands that are not exact in bf16
// are split into hi + lo bf16 parts and the product is formed as
// hi.hi + hi.lo + lo.hi, which is within a few fp32 ulps of the fp32 dot
// product -- enough to reproduce a float64 ranking up to near-ties.
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

struct RowInfo {
  int t, hh;
};

BSA_DEV RowInfo row_to_th(int row, const GateParams& p) {
  RowInfo r;
  if (p.per_group) {
    r.t = row;
    r.hh = 0;
  } else {
    r.t = row / p.G;
    r.hh = row % p.G;
  }
  return r;
}

// Absolute key position of query token t of sequence b.
BSA_DEV int64_t qpos_of(const GateParams& p, int b, int t) {
  int64_t Lk = p.Lk;
  if (p.lens) {
    int n = p.lens[b];
    n = n < 1 ? 1 : (n > p.Lk ? p.Lk : n);
    Lk = n;
  }
  return Lk - p.Lq + t;
}

// candidate blocks of query token t: [0, ncand)
BSA_DEV int ncand_of(const GateParams& p, int b, int t) {
  if (!p.causal) return p.Nb;
  const int64_t cur = qpos_of(p, b, t) / p.block;
  return (int)(cur < p.Nb ? cur : p.Nb);
}

// Load the 8 gate-query elements [d0, d0+8) of one row and split them.
template <int QK>
BSA_DEV void load_gate_q(const GateParams& p, int b, int hk, RowInfo ri, bool ok, int d0, bf16x8& hi, bf16x8& lo) {
  float x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = 0.f;
  if (ok) {
    if constexpr (QK == 0 || QK == 2) {
      const uint16_t* base = reinterpret_cast<const uint16_t*>(p.q) + (int64_t)b * p.qs_b + (int64_t)ri.t * p.qs_t;
      const int nh = (QK == 2) ? p.G : 1;
      const int h0 = (QK == 2) ? hk * p.G : hk * p.G + ri.hh;
      for (int g = 0; g < nh; ++g) {
        u16x8 v = ld16(base + (int64_t)(h0 + g) * p.qs_h + d0);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] += bf2f(v[e]);
      }
    } else {
      const float* base = reinterpret_cast<const float*>(p.q) + (int64_t)b * p.qs_b + (int64_t)ri.t * p.qs_t;
      const int h = p.per_group ? -1 : hk * p.G + ri.hh;
      if (h >= 0) {
        const f32x4* r = reinterpret_cast<const f32x4*>(base + (int64_t)h * p.qs_h + d0);
        f32x4 a = r[0], c = r[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = a[e];
          x[4 + e] = c[e];
        }
      } else {
        for (int g = 0; g < p.G; ++g) {
          const f32x4* r = reinterpret_cast<const f32x4*>(base + (int64_t)(hk * p.G + g) * p.qs_h + d0);
          f32x4 a = r[0], c = r[1];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] += a[e];
            x[4 + e] += c[e];
          }
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    __bf16 h, l;
    split_bf(x[e], h, l);
    hi[e] = h;
    lo[e] = l;
  }
}

// Writes one finished row: top-k (desc keys in buf[0..cnt)) -> output.
template <int V>
BSA_DEV void emit_row(const GateParams& p, const uint64_t* buf, int cnt, int b, int hs, int t, int split) {
  const int lane = lane_id();
  const int64_t srow = ((int64_t)b * p.Hs + hs) * p.Lq + t;
  if (p.nsplit == 1) {
    int idx = lane < cnt ? (int)key_index(buf[lane]) : 0x7FFFFFFF;
    idx = wave_sort_asc_i32(idx);
    int32_t* out = p.sel + srow * p.sel_w;
    const int cur = p.causal ? (int)(qpos_of(p, b, t) / p.block) : -1;
    for (int e = lane; e < p.sel_w; e += 64) {
      int val = -1;
      if (e < cnt) val = idx;
      else if (e == cnt && p.causal) val = cur;
      out[e] = val;
    }
  } else {
    uint64_t* out = p.part + (srow * p.nsplit + split) * p.topk;
    for (int e = lane; e < p.topk; e += 64) out[e] = e < cnt ? buf[e] : 0ull;
  }
}

// ---------------------------------------------------------------------------
// Running top-k held in registers.  In the 16x16 MFMA result layout the 16
// lanes of lane group g = lane/16 hold rows 4g..4g+3, each row's candidates
// spread over those 16 lanes.  Each row keeps its best k keys in the same 16
// lanes: element e = 16*m + (lane % 16) lives in register m, sorted
// descending; unused elements are 0.  New candidates are merged 16 at a time
// with a bitonic merge; all four lane groups merge into their own rows at once.
// ---------------------------------------------------------------------------
// Bitonic sort, ascending, of the 16 keys a 16-lane group holds (one per
// lane); every group sorts its own keys.
BSA_DEV uint64_t group_sort16_asc(uint64_t v, int li) {
#pragma unroll
  for (int size = 2; size <= 16; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const uint64_t o = row_xor64_any(v, stride, li);
      const bool lower = (li & stride) == 0;
      const bool asc = (li & size) == 0 || size == 16;
      v = cx_keep(v, o, lower != asc);
    }
  }
  return v;
}

// Merges up to 16 keys per lane group (b, one per lane, any order, 0 = none)
// into the group's list L (16*KR keys, element e = 16m + li in register m,
// descending, elements >= topk zero) and keeps the best topk.  With b sorted
// ascending, max(L[e], b[e - (16KR - 16)]) over the last register is a
// bitonic sequence holding the 16KR best keys of both; a bitonic merge sorts
// it descending.
template <int KR>
BSA_DEV void list_merge16(uint64_t (&L)[KR], uint64_t b, int li, int topk) {
  static_assert(KR == 1 || KR == 2 || KR == 4, "the bitonic merge needs 16 * KR a power of two");
  b = group_sort16_asc(b, li);
  L[KR - 1] = L[KR - 1] > b ? L[KR - 1] : b;
#pragma unroll
  for (int stride = 8 * KR; stride > 0; stride >>= 1) {
    if (stride >= 16) {
      const int rs = stride >> 4;
#pragma unroll
      for (int r = 0; r < KR; ++r) {
        const int q = r ^ rs;
        if (q > r) {
          const uint64_t a = L[r], c = L[q];
          L[r] = a > c ? a : c;
          L[q] = a > c ? c : a;
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < KR; ++r) {
        const uint64_t o = row_xor64_any(L[r], stride, li);
        const bool lower = (li & stride) == 0;
        L[r] = cx_keep(L[r], o, lower);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < KR; ++m)
    if (m * 16 + li >= topk) L[m] = 0ull;
}

// Ascending bitonic sort of the 16*NR ints a 16-lane group holds (element
// e = 16*r + lane%16 in register r); every group sorts its own row.
template <int NR>
BSA_DEV void group_sort_asc(int (&v)[NR], int li) {
#pragma unroll
  for (int size = 2; size <= 16 * NR; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= 16) {
        const int rs = stride >> 4;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int q = r ^ rs;
          if (q > r) {
            const bool asc = ((r * 16 + li) & size) == 0;
            const int a = v[r], b = v[q];
            const bool sw = asc ? (a > b) : (a < b);
            v[r] = sw ? b : a;
            v[q] = sw ? a : b;
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const int o = row_xor32_any(v[r], stride, li);
          const bool lower = (li & stride) == 0;
          const bool asc = ((r * 16 + li) & size) == 0;
          v[r] = cx_keep_i32(v[r], o, lower != asc);
        }
      }
    }
  }
}

// k-th best key of the row held by this lane's group (0 while fewer than k)
template <int KR>
BSA_DEV uint64_t list_kth(const uint64_t (&L)[KR], int lane, int topk) {
  const int e = topk - 1;
  uint64_t v = 0ull;
#pragma unroll
  for (int m = 0; m < KR; ++m)
    if (m == (e >> 4)) v = L[m];
  return shfl64(v, (lane & 48) + (e & 15));
}

// Largest key held by the 16 lanes of this lane's group (butterfly over the
// row through DPP; every lane of the group ends with it).
BSA_DEV uint64_t group_max64(uint64_t v, int li) {
#pragma unroll
  for (int st = 1; st < 16; st <<= 1) {
    const uint64_t o = row_xor64_any(v, st, li);
    v = o > v ? o : v;
  }
  return v;
}

// At most kSmallK best keys of a row whose candidates all sit in one staged
// chunk are taken by repeated group maxima (each round's winner removed from
// its lane) instead of the list merge: a few DPP butterflies per chosen key.
constexpr int kSmallK = 4;

// DMA instruction i of a chunk of 64 summary rows into the padded LDS layout
// (rows of DG + 8 elements): global_load_lds puts lane l's 16 bytes at the
// wave-uniform LDS base + 16 l, so the lanes walk the padded positions in
// order; a lane whose position is a row's padding loads piece 0 of that row
// again, and rows past n_valid load the chunk's first row (finite values whose
// keys are masked out).  DG / 8 + 1 instructions cover a chunk.
typedef __attribute__((address_space(3))) void* gate_lds_ptr_t;
template <int DG>
BSA_DEV void gate_dma_rows(uint16_t* tile, const uint16_t* base, int64_t rs, int row0, int n_valid, int i) {
  constexpr int RP = DG / 8 + 1;
  const int P = i * 64 + lane_id();
  const int r = P / RP;
  int c = P % RP;
  c = c == RP - 1 ? 0 : c;
  const int rr = r < n_valid ? r : 0;
  __builtin_amdgcn_global_load_lds((const void*)(base + (int64_t)(row0 + rr) * rs + c * 8),
                                   (gate_lds_ptr_t)(tile + i * 512), 16, 0, 0);
}

// FS: the summaries come as fp32 (p_f32) and are split into the hi / lo
// planes as each chunk is staged in LDS (LO is then true)
// Occupancy requested per instantiation (workgroups of W waves per CU), set
// to what its register use reaches: four waves per SIMD for one 16-key list
// over 64-wide summaries, three over 128-wide ones, no request otherwise.
template <int W, int DG, int KR>
constexpr int gate_min_blocks() {
  return W == 4 && KR == 1 ? (DG == 64 ? 4 : 3) : 1;
}

template <int W, int DG, int KR, int QK, bool LO, bool FS>
__global__ __launch_bounds__(64 * W, (gate_min_blocks<W, DG, KR>())) void gate_kernel(GateParams p) {
  constexpr int ROWS = 16 * W;
  constexpr int PADR = DG + 8;  // padded LDS row (bf16 elements)
  constexpr int KS = DG / 32;
  constexpr int CPR = DG / 8;                       // 16-byte chunks per summary row
  constexpr int NPF = (64 * CPR + 64 * W - 1) / (64 * W);  // chunks per thread per plane
  constexpr int STAGE_BYTES = (LO ? 2 : 1) * 64 * PADR * 2;
  // bf16 planes are copied by DMA straight into the stage buffer, the next
  // chunk's copy issued once every wave has scored the current one, so that
  // it is in flight during the top-k work, with no registers held for it
  // (lists of 32 or 64 keys: the registers then allow three waves per SIMD);
  // fp32 summaries, and the instantiations with an occupancy request, go
  // through registers
  constexpr bool DMA = !FS && gate_min_blocks<W, DG, KR>() == 1;
  constexpr int SMEM = STAGE_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char smem[SMEM];
  // per (wave, lane group): the chunk's candidates that beat the row's k-th key
  __shared__ uint64_t s_cand[W][4][80];  // < 16 left over + up to 64 new
  uint16_t* s_hi = reinterpret_cast<uint16_t*>(smem);
  uint16_t* s_lo = s_hi + 64 * PADR;

  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int tile_l = lid % p.ntiles;
  const int rest = lid / p.ntiles;
  const int split = rest % p.nsplit;
  const int bh = rest / p.nsplit;
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  // causal rows late in the sequence have the most candidates: start them first
  const int tile = p.causal ? (p.ntiles - 1 - tile_l) : tile_l;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, kh = lane >> 4;
  const int rbase = tile * ROWS + w * 16;

  // gate-query fragments (A operand) of row rbase + r16
  bf16x8 qh[KS], ql[KS];
  {
    const int row = rbase + r16;
    const bool ok = row < p.rows_per_bh;
    const RowInfo ri = row_to_th(ok ? row : 0, p);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) load_gate_q<QK>(p, b, hk, ri, ok, ks * 32 + kh * 8, qh[ks], ql[ks]);
  }
  // candidate counts of the 4 result rows this lane holds (rows 4*kh + i)
  int ncand[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = rbase + 4 * kh + i;
    ncand[i] = row < p.rows_per_bh ? ncand_of(p, b, row_to_th(row, p).t) : 0;
  }
  // the tile's last row has the most candidates
  const int last_row = min(tile * ROWS + ROWS, p.rows_per_bh) - 1;
  const int nc_max = ncand_of(p, b, row_to_th(last_row, p).t);
  const int c_lo = split * p.span;
  const int c_hi = p.topk > 0 ? min(c_lo + p.span, nc_max) : c_lo;

  const uint16_t* phi = FS ? nullptr : p.p_hi + (int64_t)b * p.ps_b + (int64_t)hk * p.ps_h;
  const uint16_t* plo = (LO && !FS) ? p.p_lo + (int64_t)b * p.ps_b + (int64_t)hk * p.ps_h : nullptr;
  const float* pf32 = FS ? p.p_f32 + (int64_t)b * p.ps_b + (int64_t)hk * p.ps_h : nullptr;

  uint64_t L[4][KR];
  uint64_t thr[4], left[4];
  int nleft[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    thr[i] = 0ull;
    left[i] = 0ull;
    nleft[i] = 0;
#pragma unroll
    for (int m = 0; m < KR; ++m) L[i][m] = 0ull;
  }

  // register prefetch of one chunk of summaries (hi and lo planes, or fp32)
  u16x8 pf_h[FS ? 1 : NPF], pf_l[(LO && !FS) ? NPF : 1];
  f32x4 pf_a[FS ? NPF : 1], pf_b[FS ? NPF : 1];
  auto fetch = [&](int c0) {
#pragma unroll
    for (int n = 0; n < NPF; ++n) {
      const int idx = tid + n * 64 * W;
      const int jr = idx / CPR, ch = idx % CPR;
      const int j = c0 + jr;
      if constexpr (FS) {
        pf_a[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        pf_b[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (idx < 64 * CPR && j < c_hi) {
          const float* src = pf32 + (int64_t)j * p.ps_j + ch * 8;
          pf_a[n] = *reinterpret_cast<const f32x4*>(src);
          pf_b[n] = *reinterpret_cast<const f32x4*>(src + 4);
        }
      } else {
        pf_h[n] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if constexpr (LO) pf_l[n] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (idx < 64 * CPR && j < c_hi) {
          pf_h[n] = ld16(phi + (int64_t)j * p.ps_j + ch * 8);
          if constexpr (LO) pf_l[n] = ld16(plo + (int64_t)j * p.ps_j + ch * 8);
        }
      }
    }
  };
  // the DMA form: a wave's share of the copy instructions of one chunk
  auto dma_chunk = [&](int c0) {
    for (int i = w; i < DG / 8 + 1; i += W) {
      gate_dma_rows<DG>(s_hi, phi, p.ps_j, c0, c_hi - c0, i);
      if constexpr (LO) gate_dma_rows<DG>(s_lo, plo, p.ps_j, c0, c_hi - c0, i);
    }
  };
  if (c_lo < c_hi) {
    if constexpr (DMA) dma_chunk(c_lo);
    else fetch(c_lo);
  }

  for (int c0 = c_lo; c0 < c_hi; c0 += 64) {
    if constexpr (DMA) {
      // this chunk's copy has landed (every wave waits for its own share)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    } else {
    __syncthreads();
#pragma unroll
    for (int n = 0; n < NPF; ++n) {
      const int idx = tid + n * 64 * W;
      if (idx < 64 * CPR) {
        const int jr = idx / CPR, ch = idx % CPR;
        if constexpr (FS) {
          u16x8 h8, l8;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            __bf16 hv, lv;
            split_bf(e < 4 ? pf_a[n][e] : pf_b[n][e - 4], hv, lv);
            h8[e] = __builtin_bit_cast(uint16_t, hv);
            l8[e] = __builtin_bit_cast(uint16_t, lv);
          }
          st16(&s_hi[jr * PADR + ch * 8], h8);
          st16(&s_lo[jr * PADR + ch * 8], l8);
        } else {
          st16(&s_hi[jr * PADR + ch * 8], pf_h[n]);
          if constexpr (LO) st16(&s_lo[jr * PADR + ch * 8], pf_l[n]);
        }
      }
    }
    __syncthreads();
    if (c0 + 64 < c_hi) fetch(c0 + 64);
    }
    f32x4 acc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 bh16 = as_bf(ld16(&s_hi[(ct * 16 + r16) * PADR + ks * 32 + kh * 8]));
        acc[ct] = mfma16(qh[ks], bh16, acc[ct]);
        if constexpr (LO) {
          const bf16x8 bl16 = as_bf(ld16(&s_lo[(ct * 16 + r16) * PADR + ks * 32 + kh * 8]));
          acc[ct] = mfma16(qh[ks], bl16, acc[ct]);
        }
        if constexpr (QK != 0) acc[ct] = mfma16(ql[ks], bh16, acc[ct]);
      }
    }
    if constexpr (DMA) {
      // every wave has read the chunk (its MFMAs consumed the reads): the
      // next chunk's copy overwrites it during the top-k work below
      __syncthreads();
      if (c0 + 64 < c_hi) dma_chunk(c0 + 64);
    }
    if (KR == 1 && p.topk <= kSmallK && c_lo + 64 >= c_hi) {
      // the row's only chunk and a small k: the k best keys directly, in
      // descending order, into list elements 0 .. k-1
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint64_t key[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int j = c0 + ct * 16 + r16;
          key[ct] = (j < c_hi && j < ncand[i]) ? make_key(acc[ct][i], (uint32_t)j) : 0ull;
        }
        uint64_t res = 0ull;
        for (int r = 0; r < p.topk; ++r) {
          uint64_t bst = key[0];
#pragma unroll
          for (int ct = 1; ct < 4; ++ct) bst = key[ct] > bst ? key[ct] : bst;
          bst = group_max64(bst, r16);
          if (r16 == r) res = bst;
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) key[ct] = key[ct] == bst ? 0ull : key[ct];
        }
        L[i][0] = res;
      }
      continue;
    }
    // merge this chunk into the running lists: each lane group appends its
    // row's candidates that beat the row's k-th key to an LDS list (after the
    // fewer than 16 left over from earlier chunks, which wait in a register),
    // then merges the list into the row's top-k 16 keys at a time.  The k-th
    // key is refreshed after each merge; candidates that pass a stale one are
    // simply merged and dropped.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint64_t key[4];
      int pend = 0;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int j = c0 + ct * 16 + r16;
        const bool ok = j < c_hi && j < ncand[i];
        key[ct] = ok ? make_key(acc[ct][i], (uint32_t)j) : 0ull;
      }
      if (KR == 1 && c0 == c_lo) {
        // first chunk, k <= 16: the smallest of the 16 lanes' maxima is a
        // lower bound of the row's k-th best key (16 distinct keys reach it)
        uint64_t lm = key[0];
#pragma unroll
        for (int ct = 1; ct < 4; ++ct) lm = key[ct] > lm ? key[ct] : lm;
#pragma unroll
        for (int st = 1; st < 16; st <<= 1) {
          const uint64_t o = row_xor64_any(lm, st, r16);
          lm = o < lm ? o : lm;
        }
        if (lm > 0ull) thr[i] = lm - 1ull;
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        if (key[ct] > thr[i]) pend |= 1 << ct;
      if (__ballot(pend != 0) == 0ull) continue;  // nothing new in any group
      // slots: exclusive scan of the per-lane counts over the 16-lane group
      const int n_me = __popc(pend);
      int inc = n_me;
      inc += (int)dpp32<0x111>((uint32_t)inc);  // row_shr:1
      inc += (int)dpp32<0x112>((uint32_t)inc);  // row_shr:2
      inc += (int)dpp32<0x114>((uint32_t)inc);  // row_shr:4
      inc += (int)dpp32<0x118>((uint32_t)inc);  // row_shr:8
      // group totals (lane 15 of each group)
      const int n0 = __builtin_amdgcn_readlane(inc, 15), n1 = __builtin_amdgcn_readlane(inc, 31);
      const int n2 = __builtin_amdgcn_readlane(inc, 47), n3 = __builtin_amdgcn_readlane(inc, 63);
      const int ng = kh == 0 ? n0 : kh == 1 ? n1 : kh == 2 ? n2 : n3;
      uint64_t* lst = s_cand[w][kh];
      if (r16 < nleft[i]) lst[r16] = left[i];
      int slot = nleft[i] + inc - n_me;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        if (pend & (1 << ct)) lst[slot++] = key[ct];
      const int cnt = nleft[i] + ng;
      const int m0 = __builtin_amdgcn_readlane(cnt, 0), m1 = __builtin_amdgcn_readlane(cnt, 16);
      const int m2 = __builtin_amdgcn_readlane(cnt, 32), m3 = __builtin_amdgcn_readlane(cnt, 48);
      const int nb = max(max(m0, m1), max(m2, m3)) >> 4;  // whole batches of the fullest list
      for (int q = 0; q < nb; ++q)
        list_merge16<KR>(L[i], 16 * q + r16 < cnt ? lst[16 * q + r16] : 0ull, r16, p.topk);
      nleft[i] = max(0, cnt - 16 * nb);
      left[i] = r16 < nleft[i] ? lst[16 * nb + r16] : 0ull;
      if (nb > 0) thr[i] = list_kth<KR>(L[i], lane, p.topk);
    }
  }
  // the candidates still waiting
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (__ballot(nleft[i] > 0) != 0ull) list_merge16<KR>(L[i], left[i], r16, p.topk);
  // emit: each lane group finishes its four rows from registers -- chosen
  // block ids sorted ascending inside the group, the forced block after them
  constexpr int NR = KR;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = rbase + 4 * kh + i;
    const bool row_ok = row < p.rows_per_bh;
    int cnt = 0;
#pragma unroll
    for (int m = 0; m < KR; ++m) {
      const bool valid = m * 16 + r16 < p.topk && L[i][m] != 0ull;
      cnt += __popc((uint32_t)(__ballot(valid) >> (16 * kh)) & 0xFFFFu);
    }
    const RowInfo ri = row_to_th(row_ok ? row : 0, p);
    const int hs = p.per_group ? hk : hk * p.G + ri.hh;
    const int64_t srow = ((int64_t)b * p.Hs + hs) * p.Lq + ri.t;
    if (p.nsplit == 1) {
      int idx[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r)
        idx[r] = (r < KR && r * 16 + r16 < cnt) ? (int)key_index(L[i][r < KR ? r : 0]) : 0x7FFFFFFF;
      group_sort_asc<NR>(idx, r16);
      if (row_ok) {
        int32_t* out = p.sel + srow * p.sel_w;
        const int cur = p.causal ? (int)(qpos_of(p, b, ri.t) / p.block) : -1;
        // cnt <= topk <= 16 * NR, so the chosen blocks and the forced one sit
        // in the first NR + 1 groups of 16 slots; every later slot of the row
        // (a requested topk above the number of blocks) is padding
#pragma unroll
        for (int r = 0; r <= NR; ++r) {
          const int e = r * 16 + r16;
          if (e < p.sel_w) out[e] = e < cnt ? idx[r < NR ? r : 0] : (e == cnt && p.causal ? cur : -1);
        }
        for (int e = (NR + 1) * 16 + r16; e < p.sel_w; e += 16) out[e] = -1;
      }
    } else if (row_ok) {
      uint64_t* out = p.part + (srow * p.nsplit + split) * p.topk;
#pragma unroll
      for (int m = 0; m < KR; ++m) {
        const int e = m * 16 + r16;
        if (e < p.topk) out[e] = e < cnt ? L[i][m] : 0ull;
      }
    }
  }
}

// Merge the per-split top-k lists of one selection row (one wave per row).
template <int V>
__global__ __launch_bounds__(256) void gate_merge_kernel(GateParams p) {
  constexpr int CAP = 64 * V;
  __shared__ uint64_t s_buf[4][CAP];
  __shared__ int s_cnt[4];
  __shared__ uint64_t s_thr[4];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t nrows = (int64_t)p.B * p.Hs * p.Lq;
  const int64_t srow = (int64_t)blockIdx.x * 4 + w;
  if (srow >= nrows) return;  // wave-uniform; no workgroup barrier follows
  const int t = (int)(srow % p.Lq);
  const int hs = (int)((srow / p.Lq) % p.Hs);
  const int b = (int)(srow / ((int64_t)p.Lq * p.Hs));
  if (lane == 0) {
    s_cnt[w] = 0;
    s_thr[w] = 0ull;
  }
  __builtin_amdgcn_wave_barrier();
  for (int sp = 0; sp < p.nsplit; ++sp) {
    const uint64_t* src = p.part + (srow * p.nsplit + sp) * p.topk;
    for (int e0 = 0; e0 < p.topk; e0 += 64) {
      const uint64_t key = (e0 + lane < p.topk) ? src[e0 + lane] : 0ull;
      const bool hit = key > s_thr[w];
      const uint64_t m = __ballot(hit);
      const int c = s_cnt[w];
      const int pos = c + __popcll(m & ((1ull << lane) - 1ull));
      if (hit) s_buf[w][pos] = key;
      __builtin_amdgcn_wave_barrier();
      if (lane == 0) s_cnt[w] = c + __popcll(m);
      __builtin_amdgcn_wave_barrier();
      if (s_cnt[w] > CAP - 64) row_compact<V>(s_buf[w], &s_cnt[w], &s_thr[w], p.topk);
    }
  }
  row_compact<V>(s_buf[w], &s_cnt[w], &s_thr[w], p.topk);
  GateParams q = p;
  q.nsplit = 1;
  emit_row<V>(q, s_buf[w], s_cnt[w], b, hs, t, 0);
}

// ---------------------------------------------------------------------------
// Small candidate sets (MoBA-style gating over a few dozen blocks): every
// row's candidates fit one chunk of 64 summaries and k <= kSmallK, per-head
// gate queries.  The chunk is staged in LDS once per workgroup; each of its
// W waves then walks `tpw` tiles of 16 rows, the next tile's gate queries in
// flight while it scores the current one and takes its k best by repeated
// group maxima (the rule of gate_kernel's single-chunk path), then writes the
// rows.  Workgroup g of a (b, kv head) owns rows [RT tpw g, RT tpw (g + 1))
// with RT = 16 W; wave w takes its tiles w, w + W, w + 2W, ...  Row indices
// are tracked as (token, head) pairs advanced without divisions.
// ---------------------------------------------------------------------------
template <int KS, int QK>
struct GateQRaw {
  u16x8 h[QK == 0 ? KS : 1];
  f32x4 a[QK == 1 ? KS : 1], c[QK == 1 ? KS : 1];
};

// Gate-query fragment of token t, head hh of the group (ok false: zeros).
template <int KS, int QK>
BSA_DEV void gate_q_fetch(const GateParams& p, int b, int hk, int t, int hh, bool ok, GateQRaw<KS, QK>& r) {
  const int d_lane = (lane_id() >> 4) * 8;
  if constexpr (QK == 0) {
    const uint16_t* base = reinterpret_cast<const uint16_t*>(p.q) + (int64_t)b * p.qs_b + (int64_t)t * p.qs_t +
                           (int64_t)(hk * p.G + hh) * p.qs_h + d_lane;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) r.h[ks] = ok ? ld16(base + ks * 32) : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
  } else {
    const float* base = reinterpret_cast<const float*>(p.q) + (int64_t)b * p.qs_b + (int64_t)t * p.qs_t +
                        (int64_t)(hk * p.G + hh) * p.qs_h + d_lane;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      r.a[ks] = ok ? *reinterpret_cast<const f32x4*>(base + ks * 32) : f32x4{0.f, 0.f, 0.f, 0.f};
      r.c[ks] = ok ? *reinterpret_cast<const f32x4*>(base + ks * 32 + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
}

// (token, head) of a per-head row advanced by n rows: dt = n / G, dh = n % G.
BSA_DEV void rows_advance(int& t, int& hh, int G, int dt, int dh) {
  t += dt;
  hh += dh;
  if (hh >= G) {
    hh -= G;
    ++t;
  }
}

// MFMA operands of the fetched fragment: exact bf16 queries are the operand
// as loaded (no low part); fp32 ones are split into hi + lo.
template <int KS, int QK>
BSA_DEV void gate_q_split(const GateQRaw<KS, QK>& r, bf16x8 (&hi)[KS], bf16x8 (&lo)[KS]) {
  if constexpr (QK == 0) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      hi[ks] = __builtin_bit_cast(bf16x8, r.h[ks]);
      lo[ks] = __builtin_bit_cast(bf16x8, u16x8{0, 0, 0, 0, 0, 0, 0, 0});
    }
    return;
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x;
      if constexpr (QK == 0) x = bf2f(r.h[ks][e]);
      else x = e < 4 ? r.a[ks][e] : r.c[ks][e - 4];
      __bf16 h, l;
      split_bf(x, h, l);
      hi[ks][e] = h;
      lo[ks][e] = l;
    }
  }
}

template <int W, int DG, int QK, bool LO, bool FS>
__global__ __launch_bounds__(64 * W) void gate_small_kernel(GateParams p, int tpw, int nwg) {
  constexpr int PADR = DG + 8;
  constexpr int KS = DG / 32;
  constexpr int CPR = DG / 8;
  static_assert(QK == 0 || QK == 1, "per-head gate queries only");
  __shared__ __attribute__((aligned(16))) uint16_t s_hi[64 * PADR];
  __shared__ __attribute__((aligned(16))) uint16_t s_lo[LO ? 64 * PADR : 8];

  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int wg = lid % nwg, bh = lid / nwg;
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r16 = lane & 15, kh = lane >> 4;
  constexpr int RT = 16 * W;  // rows of one round of tiles (one per wave)
  const int row0 = wg * RT * tpw;
  const int row_end = min(row0 + RT * tpw, p.rows_per_bh);
  // candidates of the workgroup's last row (the most of any of its rows; <= 64)
  const int nc = ncand_of(p, b, row_to_th(row_end - 1, p).t);

  // Row bookkeeping in 32-bit integers, advanced without divisions: the
  // fetched row (this lane's A-operand row) and the lane group's first result
  // row, each as (token, head of the group); rows advance by RT per tile.
  const int G = p.G, dt = RT / G, dh = RT % G;
  const int qbase = p.Lk - p.Lq;  // key position of query token 0
  int frow = row0 + 16 * w + r16;
  int ft = frow / G, fh = frow - (frow / G) * G;
  int rrow = row0 + 16 * w + 4 * kh;
  int rt = rrow / G, rh = rrow - (rrow / G) * G;
  int32_t* sel_b = p.sel + (int64_t)b * p.Hs * p.Lq * p.sel_w;

  // the first tile's gate queries, then the chunk of summaries j < nc
  GateQRaw<KS, QK> nxt;
  gate_q_fetch<KS, QK>(p, b, hk, ft, fh, frow < p.rows_per_bh, nxt);
  for (int idx = tid; idx < 64 * CPR; idx += 64 * W) {
    const int jr = idx / CPR, ch = idx % CPR;
    u16x8 h8 = u16x8{0, 0, 0, 0, 0, 0, 0, 0}, l8 = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    if (jr < nc) {
      if constexpr (FS) {
        const float* src = p.p_f32 + (int64_t)b * p.ps_b + (int64_t)hk * p.ps_h + (int64_t)jr * p.ps_j + ch * 8;
        const f32x4 fa = *reinterpret_cast<const f32x4*>(src), fb = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          __bf16 hv, lv;
          split_bf(e < 4 ? fa[e] : fb[e - 4], hv, lv);
          h8[e] = __builtin_bit_cast(uint16_t, hv);
          l8[e] = __builtin_bit_cast(uint16_t, lv);
        }
      } else {
        const int64_t off = (int64_t)b * p.ps_b + (int64_t)hk * p.ps_h + (int64_t)jr * p.ps_j + ch * 8;
        h8 = ld16(p.p_hi + off);
        if constexpr (LO) l8 = ld16(p.p_lo + off);
      }
    }
    st16(&s_hi[jr * PADR + ch * 8], h8);
    if constexpr (LO) st16(&s_lo[jr * PADR + ch * 8], l8);
  }
  __syncthreads();

  for (int u = 0; u < tpw; ++u) {
    const int rbase = row0 + 16 * w + RT * u;
    if (rbase >= row_end) break;  // wave-uniform; no workgroup barrier follows
    bf16x8 qh[KS], ql[KS];
    gate_q_split<KS, QK>(nxt, qh, ql);
    frow += RT;
    rows_advance(ft, fh, G, dt, dh);
    if (u + 1 < tpw && rbase + RT < row_end) gate_q_fetch<KS, QK>(p, b, hk, ft, fh, frow < p.rows_per_bh, nxt);
    f32x4 acc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 bh16 = as_bf(ld16(&s_hi[(ct * 16 + r16) * PADR + ks * 32 + kh * 8]));
        acc[ct] = mfma16(qh[ks], bh16, acc[ct]);
        if constexpr (LO) {
          const bf16x8 bl16 = as_bf(ld16(&s_lo[(ct * 16 + r16) * PADR + ks * 32 + kh * 8]));
          acc[ct] = mfma16(qh[ks], bl16, acc[ct]);
        }
        if constexpr (QK != 0) acc[ct] = mfma16(ql[ks], bh16, acc[ct]);
      }
    }
    // lane group kh holds rows rrow + i (i < 4): token t[i], head hh[i], own
    // block cur[i] = (qbase + t) / block
    int t[4], hh[4], cur[4], ncand[4];
    {
      int tt = rt, h = rh;
      int c = p.causal ? (qbase + tt) / p.block : 0;
      int crem = p.causal ? (qbase + tt) - c * p.block : 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i > 0 && ++h == G) {
          h = 0;
          ++tt;
          if (++crem == p.block) {
            crem = 0;
            ++c;
          }
        }
        t[i] = tt;
        hh[i] = h;
        cur[i] = c;
        ncand[i] = rrow + i < row_end ? (p.causal ? min(c, p.Nb) : p.Nb) : 0;
      }
    }
    // each row's k best keys by repeated group maxima; the four rows' chains
    // are independent and interleave
    uint64_t key[4][4], res[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      res[i] = 0ull;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int j = ct * 16 + r16;
        const uint64_t kk = make_key(acc[ct][i], (uint32_t)j);
        key[i][ct] = j < ncand[i] ? kk : 0ull;
      }
    }
    for (int r = 0; r < p.topk; ++r) {
      uint64_t bst[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        bst[i] = key[i][0];
#pragma unroll
        for (int ct = 1; ct < 4; ++ct) bst[i] = key[i][ct] > bst[i] ? key[i][ct] : bst[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) bst[i] = group_max64(bst[i], r16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        res[i] = r16 == r ? bst[i] : res[i];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) key[i][ct] = key[i][ct] == bst[i] ? 0ull : key[i][ct];
      }
    }
    // lanes 0 .. cnt-1 of the group hold a row's chosen blocks; each takes
    // its rank among them (the first quad of the group reads its four
    // lanes), which is its slot in the ascending list; the forced block
    // follows
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool valid = r16 < p.topk && res[i] != 0ull;
      const int cnt = __popc((uint32_t)(__ballot(valid) >> (16 * kh)) & 0xFFFFu);
      const uint32_t my = key_index(res[i]);
      const uint32_t v0 = dpp32<0x00>(my), v1 = dpp32<0x55>(my);
      const uint32_t v2 = dpp32<0xAA>(my), v3 = dpp32<0xFF>(my);
      const int rank = (cnt > 0 && v0 < my) + (cnt > 1 && v1 < my) + (cnt > 2 && v2 < my) + (cnt > 3 && v3 < my);
      if (rrow + i < row_end) {
        int32_t* out = sel_b + ((hk * G + hh[i]) * p.Lq + t[i]) * p.sel_w;
        const int e = r16 < cnt ? rank : r16;
        const int val = r16 < cnt ? (int)my : (r16 == cnt && p.causal ? cur[i] : -1);
        if (e < p.sel_w) out[e] = val;
        // cnt <= topk <= kSmallK: every slot from 16 on (a requested topk
        // above the number of blocks) is padding
        for (int e2 = 16 + r16; e2 < p.sel_w; e2 += 16) out[e2] = -1;
      }
    }
    rrow += RT;
    rows_advance(rt, rh, G, dt, dh);
  }
}

// Host check and launch of the small-candidate path; false when it does not
// apply.  About 2048 workgroups (eight per CU), at most kSmallTiles tiles per
// wave.
constexpr int kSmallTiles = 16;
constexpr int kSmallWaves = 8;  // waves per workgroup (4: 0.152 ms, 8: 0.143 ms on the MoBA-style 32K gate)

static bool gate_small_applies(const GateParams& p) {
  if (p.nsplit != 1 || p.topk < 1 || p.topk > kSmallK || p.lens || p.per_group) return false;
  if (p.qkind != 0 && p.qkind != 1) return false;
  if (p.rows_per_bh <= 16) return false;
  // row offsets inside one sequence's selection in 32-bit integers
  if ((int64_t)p.Hs * p.Lq * p.sel_w >= ((int64_t)1 << 31)) return false;
  const int64_t maxc = p.causal ? std::min<int64_t>(p.Nb, ((int64_t)p.Lk - 1) / p.block) : p.Nb;
  return maxc <= 64;
}

template <int DG>
static void gate_small_launch(const GateParams& p, hipStream_t s) {
  const int64_t nbh = (int64_t)p.B * p.Hkv;
  const int64_t rows = nbh * p.rows_per_bh;
  constexpr int RT = 16 * kSmallWaves;
  const int tpw = (int)std::max<int64_t>(1, std::min<int64_t>(kSmallTiles, rows / (2048 * RT)));
  const int nwg = (p.rows_per_bh + RT * tpw - 1) / (RT * tpw);
  const dim3 grid((unsigned)(nbh * nwg));
  const bool lo = p.p_lo != nullptr;
#define BSA_GATE_SMALL(QK, LO, FS) \
  hipLaunchKernelGGL((gate_small_kernel<kSmallWaves, DG, QK, LO, FS>), grid, dim3(64 * kSmallWaves), 0, s, p, tpw, nwg);
  if (p.p_f32) {
    if (p.qkind == 0) { BSA_GATE_SMALL(0, true, true) } else { BSA_GATE_SMALL(1, true, true) }
  } else if (p.qkind == 0) {
    if (lo) { BSA_GATE_SMALL(0, true, false) } else { BSA_GATE_SMALL(0, false, false) }
  } else {
    if (lo) { BSA_GATE_SMALL(1, true, false) } else { BSA_GATE_SMALL(1, false, false) }
  }
#undef BSA_GATE_SMALL
}

template <int W, int DG, int KR>
static void gate_dispatch_q(const GateParams& p, hipStream_t s, int grid) {
  const bool lo = p.p_lo != nullptr;
#define BSA_GATE_CASE(QK, LO, FS)                                                               \
  hipLaunchKernelGGL((gate_kernel<W, DG, KR, QK, LO, FS>), dim3(grid), dim3(64 * W), 0, s, p);
  if (p.p_f32) {
    if (p.qkind == 0) { BSA_GATE_CASE(0, true, true) }
    else if (p.qkind == 1) { BSA_GATE_CASE(1, true, true) }
    else { BSA_GATE_CASE(2, true, true) }
  } else if (p.qkind == 0) {
    if (lo) { BSA_GATE_CASE(0, true, false) } else { BSA_GATE_CASE(0, false, false) }
  } else if (p.qkind == 1) {
    if (lo) { BSA_GATE_CASE(1, true, false) } else { BSA_GATE_CASE(1, false, false) }
  } else {
    if (lo) { BSA_GATE_CASE(2, true, false) } else { BSA_GATE_CASE(2, false, false) }
  }
#undef BSA_GATE_CASE
}

// Registers per row list: the bitonic merge in list_merge16 needs 16 * KR to
// be a power of two, so a top-k above 32 takes four registers (64 keys).
template <int W, int DG>
static void gate_dispatch_k(const GateParams& p, hipStream_t s, int grid) {
  const int kr = p.topk <= 16 ? 1 : p.topk <= 32 ? 2 : 4;
  if (kr == 1) gate_dispatch_q<W, DG, 1>(p, s, grid);
  else if (kr == 2) gate_dispatch_q<W, DG, 2>(p, s, grid);
  else gate_dispatch_q<W, DG, 4>(p, s, grid);
}

int gate_cap_v(int topk) { return (2 * topk + 64) <= 128 ? 2 : 4; }
int gate_waves(const GateParams& p) { return p.rows_per_bh <= 16 ? 1 : 4; }

bool launch_gate(const GateParams& p, hipStream_t s) {
  const int W = gate_waves(p);
  const int grid = p.B * p.Hkv * p.nsplit * p.ntiles;
  {
    LaunchScope ls(p.tag && p.tag[0] == 'd' ? "decode_gate" : "gate_topk", s);
    if (W == 4 && gate_small_applies(p)) {
      if (p.Dg == 128) gate_small_launch<128>(p, s);
      else gate_small_launch<64>(p, s);
    } else if (p.Dg == 128) {
      if (W == 4) gate_dispatch_k<4, 128>(p, s, grid);
      else gate_dispatch_k<1, 128>(p, s, grid);
    } else {
      if (W == 4) gate_dispatch_k<4, 64>(p, s, grid);
      else gate_dispatch_k<1, 64>(p, s, grid);
    }
  }
  return launch_ok(p.tag && p.tag[0] == 'd' ? "decode_gate" : "gate_topk");
}

bool launch_gate_merge(const GateParams& p, hipStream_t s) {
  const int64_t nrows = (int64_t)p.B * p.Hs * p.Lq;
  const int grid = (int)((nrows + 3) / 4);
  {
    LaunchScope ls(p.tag && p.tag[0] == 'd' ? "decode_gate_merge" : "gate_merge", s);
    if (gate_cap_v(p.topk) == 2)
      hipLaunchKernelGGL(gate_merge_kernel<2>, dim3(grid), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(gate_merge_kernel<4>, dim3(grid), dim3(256), 0, s, p);
  }
  return launch_ok(p.tag && p.tag[0] == 'd' ? "decode_gate_merge" : "gate_merge");
}

// ---------------------------------------------------------------------------
// fp32 gate: one wave per selection row, scores in plain fp32 FMA against the
// fp32 summaries, same buffer/compaction top-k.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gate_f32_kernel(GateF32Params p) {
  constexpr int V = 2, CAP = 128;
  __shared__ uint64_t s_buf[4][CAP];
  __shared__ int s_cnt[4];
  __shared__ uint64_t s_thr[4];
  __shared__ float s_q[4][128];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t nrows = (int64_t)p.B * p.Hs * p.Lq;
  const int64_t srow = (int64_t)blockIdx.x * 4 + w;
  if (srow >= nrows) return;  // wave-uniform
  const int t = (int)(srow % p.Lq);
  const int hs = (int)((srow / p.Lq) % p.Hs);
  const int b = (int)(srow / ((int64_t)p.Lq * p.Hs));
  const int hk = p.per_group ? hs : hs / p.G;
  for (int d = lane; d < p.Dg; d += 64) {
    float x = 0.f;
    if (p.per_group) {
      for (int g = 0; g < p.G; ++g) x += p.q[(int64_t)b * p.qs_b + (int64_t)t * p.qs_t + (int64_t)(hk * p.G + g) * p.qs_h + d];
    } else {
      x = p.q[(int64_t)b * p.qs_b + (int64_t)t * p.qs_t + (int64_t)hs * p.qs_h + d];
    }
    s_q[w][d] = x;
  }
  if (lane == 0) {
    s_cnt[w] = 0;
    s_thr[w] = 0ull;
  }
  __builtin_amdgcn_wave_barrier();
  const int64_t qpos = (int64_t)p.Lk - p.Lq + t;
  const int cur = (int)(qpos / p.block);
  const int ncand = p.causal ? min(cur, p.Nb) : p.Nb;
  for (int c0 = 0; c0 < ncand; c0 += 64) {
    const int j = c0 + lane;
    uint64_t key = 0ull;
    if (j < ncand) {
      const float* pr = p.pooled + (((int64_t)b * p.Nb + j) * p.Hkv + hk) * p.Dg;
      float s = 0.f;
      for (int d = 0; d < p.Dg; ++d) s = fmaf(s_q[w][d], pr[d], s);
      key = make_key(s, (uint32_t)j);
    }
    const bool hit = key > s_thr[w];
    const uint64_t m = __ballot(hit);
    const int c = s_cnt[w];
    const int pos = c + __popcll(m & ((1ull << lane) - 1ull));
    if (hit) s_buf[w][pos] = key;
    __builtin_amdgcn_wave_barrier();
    if (lane == 0) s_cnt[w] = c + __popcll(m);
    __builtin_amdgcn_wave_barrier();
    if (s_cnt[w] > CAP - 64) row_compact<V>(s_buf[w], &s_cnt[w], &s_thr[w], p.topk);
  }
  row_compact<V>(s_buf[w], &s_cnt[w], &s_thr[w], p.topk);
  const int cnt = s_cnt[w];
  int idx = lane < cnt ? (int)key_index(s_buf[w][lane]) : 0x7FFFFFFF;
  idx = wave_sort_asc_i32(idx);
  int32_t* out = p.sel + srow * p.sel_w;
  for (int e = lane; e < p.sel_w; e += 64) {
    int val = -1;
    if (e < cnt) val = idx;
    else if (e == cnt && p.causal) val = cur;
    out[e] = val;
  }
}

bool launch_gate_f32(const GateF32Params& p, hipStream_t s) {
  const int64_t nrows = (int64_t)p.B * p.Hs * p.Lq;
  const int grid = (int)((nrows + 3) / 4);
  {
    LaunchScope ls("gate_f32", s);
    hipLaunchKernelGGL(gate_f32_kernel, dim3(grid), dim3(256), 0, s, p);
  }
  return launch_ok("gate_f32");
}

}  // namespace bsa
