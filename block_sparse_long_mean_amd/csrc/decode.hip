// Decode: one new token per sequence against a long cached KV sequence.
//
// The gate streams the routing keys (block summaries) from HBM -- they are
// the light keys kept in GPU memory in "100 Millionen Token: Gedaechtnis oder
// Trugbild?" (aitalk.it), section "Das Gehirn mit zwei Geschwindigkeiten" --
// and keeps the top-k blocks plus the token's own block.  The attention then
// gathers only those blocks (flash-decoding style: split over blocks, merged
// by log-sum-exp).  The G query heads that share a KV head are served by one
// pass over each distinct block they selected, so a block chosen by several
// heads is read from HBM once.
#include <math.h>

#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

BSA_DEV int dec_len(const DecodeAttnParams& p, int b) {
  if (!p.lens) return p.Lc;
  const int n = p.lens[b];
  return n < 1 ? 1 : (n > p.Lc ? p.Lc : n);
}

// ---------------------------------------------------------------------------
// Decode gate, pass 1: stream the routing keys once and keep, per selection
// row, the top-k of each share of kDecShare candidates.  One workgroup per
// (share, b, kv head): its waves score 64 summary rows per step on 16x16x32
// bf16 MFMAs -- A = 16 rows x 32 head dims (lanes read 16-byte pieces, four
// lanes per row per step), B = the group's query heads as columns (G of 16
// used; per group their fp32 sum, split into bf16 hi + lo).  bf16 summaries
// times bf16 queries are exact products; fp32 summaries are split into hi +
// lo as well.  The scores stay in LDS; a wave per row then keeps the share's
// best keys by (score desc, index asc) -- a threshold filter (the k-th best
// of the lanes' maxima bounds the share's k-th best from below) plus an LDS
// buffer compacted by a wave-wide bitonic sort -- and writes them, sorted,
// to the workspace.
constexpr int kDecCap = 128;     // key buffer per wave: topk (<= 64) kept + 64 new

template <int V>
BSA_DEV void lds_row_topk(const float* sc, int j0, int nc, uint64_t* buf, int* cnt, uint64_t* thr, int topk) {
  constexpr int U = kDecShare / 64;
  const int lane = lane_id();
  float sv[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = u * 64 + lane;
    sv[u] = i < nc ? sc[i] : 0.f;
  }
  // starting threshold: the k-th best of the 64 lanes' maxima
  uint64_t lm[1] = {0ull};
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = u * 64 + lane;
    const uint64_t key = i < nc ? make_key(sv[u], (uint32_t)(j0 + i)) : 0ull;
    lm[0] = key > lm[0] ? key : lm[0];
  }
  wave_sort_desc<1>(lm);
  const uint64_t tk = shfl64(lm[0], topk - 1);
  const uint64_t thr0 = tk > 0ull ? tk - 1ull : 0ull;
  // the keys above the threshold, placed in one pass: each lane's count, its
  // place from a wave prefix sum formed bit by bit from ballots, then one
  // compaction -- unless more than the buffer holds pass (only when the best
  // keys crowd into few lanes), which takes the incremental path below
  uint32_t hitm = 0u;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = u * 64 + lane;
    const uint64_t key = i < nc ? make_key(sv[u], (uint32_t)(j0 + i)) : 0ull;
    hitm |= (key > thr0 ? 1u : 0u) << u;
  }
  const int nh = __popc(hitm);
  const uint64_t below = (1ull << lane) - 1ull;
  int before = 0, total = 0;
#pragma unroll
  for (int bit = 0; (1 << bit) <= U; ++bit) {
    const uint64_t mb = __ballot((nh >> bit) & 1);
    before += __popcll(mb & below) << bit;
    total += __popcll(mb) << bit;
  }
  if (total <= kDecCap) {
    int e = before;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if ((hitm >> u) & 1u) {
        buf[e] = make_key(sv[u], (uint32_t)(j0 + u * 64 + lane));
        ++e;
      }
    }
    if (lane == 0) {
      *cnt = total;
      *thr = thr0;
    }
    __builtin_amdgcn_wave_barrier();
    if (total <= 64) row_compact<1>(buf, cnt, thr, topk);  // one key per lane: a shorter sort
    else row_compact<V>(buf, cnt, thr, topk);
    return;
  }
  if (lane == 0 && tk > 0ull) *thr = tk - 1ull;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int i = u * 64 + lane;
    const uint64_t key = i < nc ? make_key(sv[u], (uint32_t)(j0 + i)) : 0ull;
    const bool hit = key > *thr;
    const uint64_t m = __ballot(hit);
    if (m) {
      const int c = *cnt;
      if (hit) buf[c + __popcll(m & ((1ull << lane) - 1ull))] = key;
      __builtin_amdgcn_wave_barrier();
      if (lane == 0) *cnt = c + __popcll(m);
      __builtin_amdgcn_wave_barrier();
      if (*cnt > kDecCap - 64) row_compact<V>(buf, cnt, thr, topk);
    }
  }
  row_compact<V>(buf, cnt, thr, topk);
}

template <typename PT, int D, int NR>
__global__ __launch_bounds__(256) void decode_scores_kernel(DecodeGateParams p) {
  constexpr int KS = D / 32;
  __shared__ float s_sc[NR][kDecShare];
  __shared__ uint64_t s_buf[4][kDecCap];
  __shared__ int s_cnt[4];
  __shared__ uint64_t s_thr[4];
  const int bh = blockIdx.y, share = blockIdx.x;
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, kq = lane >> 4;
  const int nq = p.per_group ? 1 : p.G;
  int n = p.lens ? p.lens[b] : p.Lc;
  n = n < 1 ? 1 : (n > p.Lc ? p.Lc : n);
  const int cur = (n - 1) / p.block;  // candidates: blocks before the token's own
  const int j0 = share * kDecShare;
  const int nc = min(kDecShare, cur - j0);
  if (nc <= 0 || p.topk <= 0) return;  // uniform
  // B operand: column `col` = query head (or the group sum) for k = 8*kq + 32*ks
  // (each lane's 8 consecutive head dims come in one 16-byte load per head)
  bf16x8 qh[KS], ql[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.f;
    const int d0 = ks * 32 + kq * 8;
    if (col < nq) {
      if (p.per_group) {
        for (int g = 0; g < p.G; ++g) {
          const u16x8 v = ld16(p.q + (int64_t)b * p.qs_b + (int64_t)(hk * p.G + g) * p.qs_h + d0);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] += bf2f(v[e]);
        }
      } else {
        const u16x8 v = ld16(p.q + (int64_t)b * p.qs_b + (int64_t)(hk * p.G + col) * p.qs_h + d0);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = bf2f(v[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16 h, l;
      split_bf(x[e], h, l);
      qh[ks][e] = h;
      ql[ks][e] = l;
    }
  }
  const PT* base = reinterpret_cast<const PT*>(p.pooled) + (int64_t)b * p.ps_b + (int64_t)hk * p.ps_h;
  // wave w scores 64-row steps w, w + 4, ... of the share; the A operands
  // of the next step (4 row tiles) are loaded while the current one is
  // computed
  u32x4 raw[4][KS][sizeof(PT) / 2], nxt[4][KS][sizeof(PT) / 2];
  auto fetch = [&](int c0, u32x4 (&dst)[4][KS][sizeof(PT) / 2]) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      const int i = c0 + rt * 16 + col;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int hpart = 0; hpart < (int)(sizeof(PT) / 2); ++hpart) {
          dst[rt][ks][hpart] = u32x4{0u, 0u, 0u, 0u};
          if (i < nc)
            dst[rt][ks][hpart] =
                *reinterpret_cast<const u32x4*>(base + (int64_t)(j0 + i) * p.ps_j + ks * 32 + kq * 8 + hpart * 4);
        }
    }
  };
  if (w * 64 < nc) fetch(w * 64, nxt);
  for (int c0 = w * 64; c0 < nc; c0 += 256) {
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int hpart = 0; hpart < (int)(sizeof(PT) / 2); ++hpart) raw[rt][ks][hpart] = nxt[rt][ks][hpart];
    if (c0 + 256 < nc) fetch(c0 + 256, nxt);
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (sizeof(PT) == 2) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, raw[rt][ks][0]);
          acc = mfma16(a, qh[ks], acc);
          if (p.per_group) acc = mfma16(a, ql[ks], acc);
        } else {
          bf16x8 ah, al;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float x = __uint_as_float(raw[rt][ks][e >> 2][e & 3]);
            __bf16 h, l;
            split_bf(x, h, l);
            ah[e] = h;
            al[e] = l;
          }
          acc = mfma16(ah, qh[ks], acc);
          acc = mfma16(al, qh[ks], acc);
          if (p.per_group) acc = mfma16(ah, ql[ks], acc);
        }
      }
      // result: lane holds column `col` (query head) of rows 4*kq + i
      if (col < nq) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s_sc[col][c0 + rt * 16 + 4 * kq + i] = acc[i];
      }
    }
  }
  __syncthreads();
  // the share's top-k of each row: wave w takes rows w, w + 4
  for (int r = w; r < nq; r += 4) {
    if (lane == 0) {
      s_cnt[w] = 0;
      s_thr[w] = 0ull;
    }
    __builtin_amdgcn_wave_barrier();
    lds_row_topk<2>(s_sc[r], j0, nc, s_buf[w], &s_cnt[w], &s_thr[w], p.topk);
    const int cnt = s_cnt[w];
    const int64_t row = (int64_t)b * p.Hs + (p.per_group ? hk : hk * p.G + r);
    const int64_t li = row * p.nshare + share;
    for (int e = lane; e < cnt; e += 64) p.skeys[li * p.topk + e] = s_buf[w][e];
    if (lane == 0) p.scnt[li] = cnt;
  }
}

// whether the ascending ids row[0 .. w) (then -1 padding) hold j
BSA_DEV bool row_has(const int32_t* row, int w, int j) {
  int lo = 0, hi = w;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const int x = row[mid];
    if (x >= 0 && x < j) lo = mid + 1;
    else hi = mid;
  }
  return lo < w && row[lo] == j;
}

// Union of the selection rows of one (b, kv head), by the whole workgroup:
// rows r < nrow of sel hold ascending block ids, then -1.  Each distinct id
// once, ascending, with the bit mask of the rows (query heads) that chose it,
// packed (j << 8 | mask).  An id counts at the row that holds it first; its
// place is the number of such first ids below it.  Returns the count.
template <int NT>
BSA_DEV int unite_rows(const int32_t (*sel)[65], int nrow, int w, int G, bool per_group, int32_t* s_first,
                       int* s_total, int32_t* out) {
  const int tid = threadIdx.x;
  const int n = nrow * w;
  if (tid == 0) *s_total = 0;
  for (int e = tid; e < n; e += NT) {
    const int r = e / w;
    const int j = sel[r][e % w];
    bool first = j >= 0;
    for (int r2 = 0; first && r2 < r; ++r2) first = !row_has(sel[r2], w, j);
    s_first[e] = first ? j : -1;
  }
  __syncthreads();
  for (int e = tid; e < n; e += NT) {
    const int j = s_first[e];
    if (j < 0) continue;
    const int r = e / w;
    int mask = per_group ? (1 << G) - 1 : 1 << r;
    if (!per_group)
      for (int r2 = r + 1; r2 < nrow; ++r2)
        if (row_has(sel[r2], w, j)) mask |= 1 << r2;
    int rank = 0;
    for (int e2 = 0; e2 < n; ++e2) {
      const int x = s_first[e2];
      rank += (x >= 0 && x < j) ? 1 : 0;
    }
    out[rank] = (j << 8) | mask;
    atomicAdd(s_total, 1);
  }
  __syncthreads();
  return *s_total;
}

// Decode gate, pass 2, and the union, for one (b, kv head) per workgroup:
// wave w merges the share lists of rows w, w + 4 (appended into its LDS
// buffer, compacted to the best k whenever the next list might not fit),
// writes each row ascending with the forced own block last, -1 padded; then
// every thread helps unite the rows' blocks for the attention.
__global__ __launch_bounds__(256) void decode_select_kernel(DecodeGateParams p) {
  __shared__ uint64_t s_buf[4][kDecCap];
  __shared__ int s_cnt[4];
  __shared__ uint64_t s_thr[4];
  __shared__ int32_t s_sel[8][65];
  __shared__ int32_t s_first[512];
  __shared__ int s_total;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bh = blockIdx.x;
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const int nrow = p.per_group ? 1 : p.G;
  int n = p.lens ? p.lens[b] : p.Lc;
  n = n < 1 ? 1 : (n > p.Lc ? p.Lc : n);
  const int cur = (n - 1) / p.block;
  const int nsh = p.topk > 0 ? (cur + kDecShare - 1) / kDecShare : 0;
  for (int r = w; r < nrow; r += 4) {
    const int64_t row = (int64_t)b * p.Hs + (p.per_group ? hk : hk * p.G + r);
    if (lane == 0) {
      s_cnt[w] = 0;
      s_thr[w] = 0ull;
    }
    __builtin_amdgcn_wave_barrier();
    if (nsh * p.topk <= kDecCap) {
      // every share's list at once -- entry e of their concatenation is rank
      // e % k of share e / k, loaded beside that share's count and kept when
      // the rank is below it (a real key is never 0) -- then one sort
      uint64_t v[2] = {0ull, 0ull};
      if (nsh > 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int e = i * 64 + lane;
          const int sh = e / p.topk, rk = e - sh * p.topk;
          if (sh < nsh) {
            const int64_t li = row * p.nshare + sh;
            const uint64_t kk = p.skeys[li * p.topk + rk];
            v[i] = rk < p.scnt[li] ? kk : 0ull;
          }
        }
      }
      const int nk = __popcll(__ballot(v[0] != 0ull)) + __popcll(__ballot(v[1] != 0ull));
      wave_sort_desc<2>(v);
      const int keep = nk < p.topk ? nk : p.topk;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int e = i * 64 + lane;
        if (e < keep) s_buf[w][e] = v[i];
      }
      if (lane == 0) s_cnt[w] = keep;
      __builtin_amdgcn_wave_barrier();
    } else {
      for (int sh = 0; sh < nsh; ++sh) {
        const int64_t li = row * p.nshare + sh;
        const int c = p.scnt[li];
        if (s_cnt[w] + c > kDecCap) row_compact<2>(s_buf[w], &s_cnt[w], &s_thr[w], p.topk);
        const int base = s_cnt[w];
        for (int e = lane; e < c; e += 64) s_buf[w][base + e] = p.skeys[li * p.topk + e];
        __builtin_amdgcn_wave_barrier();
        if (lane == 0) s_cnt[w] = base + c;
        __builtin_amdgcn_wave_barrier();
      }
      row_compact<2>(s_buf[w], &s_cnt[w], &s_thr[w], p.topk);
    }
    const int cnt = s_cnt[w];
    int idx = lane < cnt ? (int)key_index(s_buf[w][lane]) : 0x7FFFFFFF;
    idx = wave_sort_asc_i32(idx);
    int32_t* out = p.sel + row * p.sel_w;
    for (int e = lane; e < p.sel_w; e += 64) {
      const int val = e < cnt ? idx : (e == cnt ? cur : -1);
      out[e] = val;
      s_sel[r][e] = val;
    }
  }
  __syncthreads();
  const int total = unite_rows<256>(s_sel, nrow, p.sel_w, p.G, p.per_group != 0, s_first, &s_total,
                                    p.ulist + (int64_t)bh * p.umax);
  if (threadIdx.x == 0) p.ucount[bh] = total;
}

bool launch_decode_gate(const DecodeGateParams& p, hipStream_t s) {
  {
    LaunchScope ls("decode_scores", s);
    const dim3 grid((unsigned)p.nshare, (unsigned)(p.B * p.Hkv));
    const int nr = p.per_group ? 1 : (p.G <= 4 ? 4 : 8);
#define BSA_DEC_SCORES(PT, DD)                                                                               \
  do {                                                                                                       \
    if (nr == 1) hipLaunchKernelGGL((decode_scores_kernel<PT, DD, 1>), grid, dim3(256), 0, s, p);            \
    else if (nr == 4) hipLaunchKernelGGL((decode_scores_kernel<PT, DD, 4>), grid, dim3(256), 0, s, p);       \
    else hipLaunchKernelGGL((decode_scores_kernel<PT, DD, 8>), grid, dim3(256), 0, s, p);                    \
  } while (0)
    if (p.pooled_bf16) {
      if (p.D == 128) BSA_DEC_SCORES(uint16_t, 128);
      else BSA_DEC_SCORES(uint16_t, 64);
    } else {
      if (p.D == 128) BSA_DEC_SCORES(float, 128);
      else BSA_DEC_SCORES(float, 64);
    }
#undef BSA_DEC_SCORES
  }
  if (!launch_ok("decode_scores")) return false;
  {
    LaunchScope ls("decode_select", s);
    hipLaunchKernelGGL(decode_select_kernel, dim3((unsigned)(p.B * p.Hkv)), dim3(256), 0, s, p);
  }
  return launch_ok("decode_select");
}

// One wave per (b, query head): LSE-merge the partials of its blocks.
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeAttnParams p) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + w;
  if (row >= p.B * p.Hq) return;
  const int b = row / p.Hq, h = row % p.Hq;
  const int hk = h / p.G, hh = h % p.G;
  const int bh = b * p.Hkv + hk;
  const int n = p.ucount[bh];
  float m = -INFINITY, l = 0.f, a0 = 0.f, a1 = 0.f;
  const int32_t* ul = p.ulist + (int64_t)bh * p.umax;
  for (int u0 = 0; u0 < n; u0 += 64) {
    // which of the next 64 union entries this head chose
    const int u = u0 + lane;
    const bool mine = u < n && ((ul[u] & 255) & (1 << hh));
    uint64_t bm = __ballot(mine);
    while (bm) {
      int us[8];
      int k = 0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        us[t] = -1;
        if (bm) {
          us[t] = u0 + __ffsll((unsigned long long)bm) - 1;
          bm &= bm - 1;
          ++k;
        }
      }
      float ls[8], x0[8], x1[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        ls[t] = -INFINITY;
        x0[t] = x1[t] = 0.f;
        if (us[t] >= 0) {
          const int64_t pidx = ((int64_t)bh * p.umax + us[t]) * p.G + hh;
          ls[t] = p.part_lse[pidx];
          const float* src = p.part_o + pidx * p.D;
          x0[t] = lane < p.D ? src[lane] : 0.f;
          x1[t] = lane + 64 < p.D ? src[lane + 64] : 0.f;
        }
      }
      float mb = m;
#pragma unroll
      for (int t = 0; t < 8; ++t) mb = fmaxf(mb, ls[t]);
      const float c1 = __builtin_amdgcn_exp2f(m - mb);
      a0 *= c1;
      a1 *= c1;
      l *= c1;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float c2 = __builtin_amdgcn_exp2f(ls[t] - mb);
        a0 = fmaf(c2, x0[t], a0);
        a1 = fmaf(c2, x1[t], a1);
        l += c2;
      }
      m = mb;
      (void)k;
    }
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  uint16_t* dst = p.o + (int64_t)b * p.os_b + (int64_t)h * p.os_h;
  if (lane < p.D) dst[lane] = f2bf(a0 * inv);
  if (lane + 64 < p.D) dst[lane + 64] = f2bf(a1 * inv);
  if (p.lse_out && lane == 0)
    p.lse_out[(int64_t)b * p.Hq + h] = l > 0.f ? (m + log2f(l)) * 0.69314718055994530942f : -INFINITY;
}

// the attention itself runs on MFMA (decode_attend_mfma_kernel, attn.hip)
bool launch_decode_attend(const DecodeAttnParams& p, hipStream_t s) { return launch_decode_attend_mfma(p, s); }

bool launch_decode_combine(const DecodeAttnParams& p, hipStream_t s) {
  {
    LaunchScope ls("decode_combine", s);
    hipLaunchKernelGGL(decode_combine_kernel, dim3((p.B * p.Hq + 3) / 4), dim3(256), 0, s, p);
  }
  return launch_ok("decode_combine");
}

}  // namespace bsa
