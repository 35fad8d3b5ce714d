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
// Decode gate, pass 1: stream the routing keys once.  A wave scores 16
// summary rows per step on a 16x16x32 bf16 MFMA: A = 16 rows x 32 head dims
// (lanes read 16-byte pieces, four lanes per row per step), B = the group's
// query heads as columns (G of 16 used; per group their fp32 sum, split into
// bf16 hi + lo).  bf16 summaries times bf16 queries are exact products; fp32
// summaries are split into hi + lo as well.  Writes fp32 scores [B, Hs, Nb].
template <typename PT, int D>
__global__ __launch_bounds__(256) void decode_scores_kernel(DecodeGateParams p) {
  constexpr int KS = D / 32;
  constexpr int ROWS_PER_WAVE = 64;  // 4 MFMA row tiles
  const int bh = blockIdx.y;
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 15, kq = lane >> 4;
  const int nq = p.per_group ? 1 : p.G;
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
  const int j0 = (blockIdx.x * 4 + w) * ROWS_PER_WAVE;
  const PT* base = reinterpret_cast<const PT*>(p.pooled) + (int64_t)b * p.ps_b + (int64_t)hk * p.ps_h;
  // A operands for 4 row tiles, all loads issued before the MFMAs
  u32x4 raw[4][KS][sizeof(PT) / 2];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int j = j0 + rt * 16 + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int hpart = 0; hpart < (int)(sizeof(PT) / 2); ++hpart) {
        raw[rt][ks][hpart] = u32x4{0u, 0u, 0u, 0u};
        if (j < p.Nb)
          raw[rt][ks][hpart] = *reinterpret_cast<const u32x4*>(base + (int64_t)j * p.ps_j + ks * 32 + kq * 8 + hpart * 4);
      }
  }
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
      const int hs = p.per_group ? hk : hk * p.G + col;
      float* out = p.scores + ((int64_t)b * p.Hs + hs) * p.Nb;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + rt * 16 + 4 * kq + i;
        if (j < p.Nb) out[j] = acc[i];
      }
    }
  }
}

// Union of the selections of one (b, kv head) by one wave: sel[r][s] for
// rows r < nrow, slots s < w (-1 = none) -> distinct block ids ascending,
// each with a bit mask of the heads that chose it, packed (j << 8 | mask).
BSA_DEV int unite_rows(const int32_t (*sel)[65], int nrow, int w, int G, bool per_group, uint64_t* s_v,
                       int32_t* out) {
  constexpr int V = 8;  // up to 512 (head, block) pairs
  const int lane = lane_id();
  uint64_t v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = i * 64 + lane;
    uint64_t key = 0ull;
    if (e < nrow * w) {
      const int hh = e / w, sl = e % w;
      const int j = sel[hh][sl];
      if (j >= 0) key = ~(((uint64_t)(uint32_t)j << 8) | (uint64_t)hh);  // descending ~val = ascending val
    }
    v[i] = key;
  }
  wave_sort_desc<V>(v);
#pragma unroll
  for (int i = 0; i < V; ++i) s_v[i * 64 + lane] = v[i];
  __builtin_amdgcn_wave_barrier();
  // element e starts a run of equal block ids when its id differs from
  // element e-1's; a run holds at most G entries (one per head)
  int total = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = i * 64 + lane;
    const uint64_t key = s_v[e];
    bool head = false;
    int val = 0;
    if (key != 0ull) {
      const int j = (int)((~key) >> 8);
      head = e == 0 || (int)((~s_v[e - 1]) >> 8) != j;
      if (head) {
        int mask = 0;
        for (int f = e; f < 64 * V && f < e + 8; ++f) {
          const uint64_t kf = s_v[f];
          if (kf == 0ull || (int)((~kf) >> 8) != j) break;
          mask |= per_group ? ((1 << G) - 1) : (1 << (int)((~kf) & 255));
        }
        val = (j << 8) | mask;
      }
    }
    const uint64_t hm = __ballot(head);
    if (head) out[total + __popcll(hm & ((1ull << lane) - 1ull))] = val;
    total += __popcll(hm);
  }
  return total;
}

// Decode gate, pass 2, and the union, for one (b, kv head) per workgroup.
// Its 16 waves split the candidates j < cur of the selection rows (G rows
// per head, one per group): each wave keeps the top-k of its share by (score
// desc, index asc) -- a threshold filter plus an LDS buffer compacted by a
// wave-wide bitonic sort -- the shares of a row are merged pairwise, each row
// is written ascending with the forced own block last, -1 padded, and wave 0
// unites the rows' blocks for the attention.
template <int V>
__global__ __launch_bounds__(1024) void decode_select_kernel(DecodeGateParams p) {
  constexpr int CAP = 64 * V;
  constexpr int NW = 16;
  __shared__ uint64_t s_buf[NW][CAP];
  __shared__ int s_cnt[NW];
  __shared__ uint64_t s_thr[NW];
  __shared__ int32_t s_sel[8][65];
  __shared__ uint64_t s_v[512];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int bh = blockIdx.x;
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const int nrow = p.per_group ? 1 : p.G;
  const int wpr = NW / nrow;  // waves per row
  const int r = w / wpr, q = w % wpr;
  const bool active = r < nrow;
  int n = p.lens ? p.lens[b] : p.Lc;
  n = n < 1 ? 1 : (n > p.Lc ? p.Lc : n);
  const int cur = (n - 1) / p.block;
  const int hs = p.per_group ? hk : hk * p.G + (active ? r : 0);
  const int64_t row = (int64_t)b * p.Hs + hs;
  if (lane == 0) {
    s_cnt[w] = 0;
    s_thr[w] = 0ull;
  }
  __builtin_amdgcn_wave_barrier();
  if (active) {
    const float* sc = p.scores + row * p.Nb;
    constexpr int U = 32;  // chunks of 64 candidates loaded together
    for (int c0 = q * 64 * U; c0 < cur; c0 += wpr * 64 * U) {
      float sv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = c0 + u * 64 + lane;
        sv[u] = j < cur ? sc[j] : 0.f;
      }
      if (c0 == q * 64 * U && p.topk > 0) {
        // starting threshold: the k-th best of the 64 lanes' maxima is a
        // lower bound of the share's k-th best key (k distinct keys reach
        // it), so only keys at or above it need to enter the buffer
        uint64_t lm[1] = {0ull};
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int j = c0 + u * 64 + lane;
          const uint64_t key = j < cur ? make_key(sv[u], (uint32_t)j) : 0ull;
          lm[0] = key > lm[0] ? key : lm[0];
        }
        wave_sort_desc<1>(lm);
        const uint64_t tk = shfl64(lm[0], p.topk - 1);
        if (lane == 0 && tk > 0ull) s_thr[w] = tk - 1ull;
        __builtin_amdgcn_wave_barrier();
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int j = c0 + u * 64 + lane;
        const uint64_t key = j < cur ? make_key(sv[u], (uint32_t)j) : 0ull;
        const bool hit = key > s_thr[w];
        const uint64_t m = __ballot(hit);
        if (m) {
          const int c = s_cnt[w];
          if (hit) s_buf[w][c + __popcll(m & ((1ull << lane) - 1ull))] = key;
          __builtin_amdgcn_wave_barrier();
          if (lane == 0) s_cnt[w] = c + __popcll(m);
          __builtin_amdgcn_wave_barrier();
          if (s_cnt[w] > CAP - 64) row_compact<V>(s_buf[w], &s_cnt[w], &s_thr[w], p.topk);
        }
      }
    }
    row_compact<V>(s_buf[w], &s_cnt[w], &s_thr[w], p.topk);
  }
  // pairwise merges of a row's shares: wave q absorbs wave q + st (at most
  // 2k keys, within the buffer), keeps the best k
  for (int st = 1; st < wpr; st <<= 1) {
    __syncthreads();
    if (active && (q % (2 * st)) == 0 && q + st < wpr) {
      const int c = s_cnt[w], co = s_cnt[w + st];
      for (int e = lane; e < co; e += 64) s_buf[w][c + e] = s_buf[w + st][e];
      __builtin_amdgcn_wave_barrier();
      if (lane == 0) s_cnt[w] = c + co;
      __builtin_amdgcn_wave_barrier();
      row_compact<V>(s_buf[w], &s_cnt[w], &s_thr[w], p.topk);
    }
  }
  if (active && q == 0) {
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
  if (w == 0) {
    const int total = unite_rows(s_sel, nrow, p.sel_w, p.G, p.per_group != 0, s_v, p.ulist + (int64_t)bh * p.umax);
    if (lane == 0) p.ucount[bh] = total;
  }
}

bool launch_decode_gate(const DecodeGateParams& p, hipStream_t s) {
  {
    LaunchScope ls("decode_scores", s);
    const dim3 grid((unsigned)((p.Nb + 255) / 256), (unsigned)(p.B * p.Hkv));  // 4 waves x 64 rows
    if (p.pooled_bf16) {
      if (p.D == 128) hipLaunchKernelGGL((decode_scores_kernel<uint16_t, 128>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((decode_scores_kernel<uint16_t, 64>), grid, dim3(256), 0, s, p);
    } else {
      if (p.D == 128) hipLaunchKernelGGL((decode_scores_kernel<float, 128>), grid, dim3(256), 0, s, p);
      else hipLaunchKernelGGL((decode_scores_kernel<float, 64>), grid, dim3(256), 0, s, p);
    }
  }
  if (!launch_ok("decode_scores")) return false;
  {
    LaunchScope ls("decode_select", s);
    const unsigned grid = (unsigned)(p.B * p.Hkv);
    if (2 * p.topk + 64 <= 128)
      hipLaunchKernelGGL(decode_select_kernel<2>, dim3(grid), dim3(1024), 0, s, p);
    else
      hipLaunchKernelGGL(decode_select_kernel<4>, dim3(grid), dim3(1024), 0, s, p);
  }
  return launch_ok("decode_select");
}

// One workgroup per (b, kv head, distinct block): scores for the heads that
// chose the block, softmax over its keys, weighted sum of its values.
template <int D, int NH>
__global__ __launch_bounds__(256) void decode_attend_kernel(DecodeAttnParams p) {
  constexpr int KC = 64;  // keys per pass (a small pass keeps registers low: 4 waves per SIMD)
  constexpr int CH = D / 8;
  constexpr int KG = 256 / CH;  // key groups in the value pass
  __shared__ float s_q[8][D];
  __shared__ float s_s[8][KC];
  __shared__ float s_m[8], s_l[8], s_c[8];
  __shared__ float s_red[KG][D];
  __shared__ int s_heads[8];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int bh = blockIdx.x / p.umax, u = blockIdx.x % p.umax;
  if (u >= p.ucount[bh]) return;  // uniform for the workgroup, before any barrier
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const int ent = p.ulist[(int64_t)bh * p.umax + u];
  const int j = ent >> 8, mask = ent & 255;
  int nh = 0;
  for (int hh = 0; hh < p.G; ++hh)
    if (mask & (1 << hh)) nh++;
  if (tid == 0) {
    int c = 0;
    for (int hh = 0; hh < p.G; ++hh)
      if (mask & (1 << hh)) s_heads[c++] = hh;
  }
  __syncthreads();
  for (int idx = tid; idx < nh * D; idx += 256) {
    const int a = idx / D, d = idx % D;
    const int hq = hk * p.G + s_heads[a];
    s_q[a][d] = bf2f(p.q[(int64_t)b * p.qs_b + (int64_t)hq * p.qs_h + d]);
  }
  if (tid < 8) {
    s_m[tid] = -INFINITY;
    s_l[tid] = 0.f;
  }
  const int n = dec_len(p, b);
  const int ka = j * p.block;
  int ke = min(ka + p.block, n);
  // kb / vb: the block's first key and value row (token ka of sequence b)
  int64_t ko, vo;
  if (p.table) {
    const int pg = p.table[(int64_t)b * p.table_w + j];
    if (pg < 0 || pg >= p.num_pages) ke = ka;  // no keys: the sequence's output is undefined, nothing is read
    ko = (int64_t)pg * p.ks_b;
    vo = (int64_t)pg * p.vs_b;
  } else {
    ko = (int64_t)b * p.ks_b + (int64_t)ka * p.ks_t;
    vo = (int64_t)b * p.vs_b + (int64_t)ka * p.vs_t;
  }
  const uint16_t* kb = p.k + ko + (int64_t)hk * p.ks_h;
  const uint16_t* vb = p.v + vo + (int64_t)hk * p.vs_h;
  const int dc = tid % CH, kg = tid / CH;
  float acc[NH][8];
#pragma unroll
  for (int a = 0; a < NH; ++a)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[a][e] = 0.f;
  __syncthreads();

  constexpr int KPG = KC / KG;
  for (int k0 = ka; k0 < ke; k0 += KC) {
    const int nk = min(KC, ke - k0);
    // this chunk's values, loaded now so they are in flight with the keys
    u16x8 vx[KPG];
#pragma unroll
    for (int kk = 0; kk < KPG; ++kk) {
      const int key = kg * KPG + kk;
      vx[kk] = key < nk ? ld16(vb + (int64_t)(k0 - ka + key) * p.vs_t + dc * 8) : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
    // scores: 16 lanes per key row (8 head dims each), 16 rows per pass;
    // the partial dot products are summed across the row's 16 lanes
    {
      constexpr int CPR = D / 8;   // lanes per key row
      constexpr int RPP = 256 / CPR;  // rows per pass
      const int c = tid % CPR, rsub = tid / CPR;
      float qv[NH][8];
#pragma unroll
      for (int a = 0; a < NH; ++a)
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[a][e] = a < nh ? s_q[a][c * 8 + e] : 0.f;
      u16x8 kx[KC / RPP];
#pragma unroll
      for (int ps = 0; ps < KC / RPP; ++ps) {
        const int key = ps * RPP + rsub;
        kx[ps] = key < nk ? ld16(kb + (int64_t)(k0 - ka + key) * p.ks_t + c * 8) : u16x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
#pragma unroll
      for (int ps = 0; ps < KC / RPP; ++ps) {
        const int key = ps * RPP + rsub;
        float part[NH];
#pragma unroll
        for (int a = 0; a < NH; ++a) {
          part[a] = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) part[a] = fmaf(qv[a][e], bf2f(kx[ps][e]), part[a]);
        }
#pragma unroll
        for (int a = 0; a < NH; ++a) {
          if (a < nh) {
            float tot = part[a];
#pragma unroll
            for (int m2 = 1; m2 < CPR; m2 <<= 1) tot += __shfl_xor(tot, m2, 64);
            if (c == 0) s_s[a][key] = key < nk ? tot * p.sl2 : -INFINITY;
          }
        }
      }
    }
    __syncthreads();
    // softmax statistics per head (wave a handles heads a, a+4)
    for (int a = w; a < nh; a += 4) {
      const float x0 = lane < KC ? s_s[a][lane] : -INFINITY;
      const float x1 = KC > 64 ? s_s[a][(lane + 64) % KC] : -INFINITY;
      const float mx = wave_max(fmaxf(x0, x1));
      const float mold = s_m[a];
      const float mnew = fmaxf(mold, mx);
      const float e0 = exp2f(x0 - mnew), e1 = exp2f(x1 - mnew);
      if (lane < KC) s_s[a][lane] = e0;
      if (KC > 64) s_s[a][(lane + 64) % KC] = e1;
      const float sum = wave_sum(e0 + e1);
      if (lane == 0) {
        const float c = exp2f(mold - mnew);
        s_c[a] = c;
        s_l[a] = s_l[a] * c + sum;
        s_m[a] = mnew;
      }
    }
    __syncthreads();
    // weighted values: thread = (key group kg, 8-wide d chunk dc)
    {
#pragma unroll
      for (int a = 0; a < NH; ++a) {
        if (a < nh) {
          const float c = s_c[a];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[a][e] *= c;
        }
      }
#pragma unroll
      for (int kk = 0; kk < KPG; ++kk) {
        const int key = kg * KPG + kk;
        if (key < nk) {
          const u16x8 x = vx[kk];
#pragma unroll
          for (int a = 0; a < NH; ++a) {
            if (a < nh) {
              const float pw = s_s[a][key];
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[a][e] = fmaf(pw, bf2f(x[e]), acc[a][e]);
            }
          }
        }
      }
    }
    __syncthreads();
  }
  // reduce the key groups and write the per-head partials
#pragma unroll
  for (int a = 0; a < NH; ++a) {
    if (a >= nh) break;  // nh is uniform across the workgroup
#pragma unroll
    for (int e = 0; e < 8; ++e) s_red[kg][dc * 8 + e] = acc[a][e];
    __syncthreads();
    if (tid < D) {
      float sum = 0.f;
      for (int g = 0; g < KG; ++g) sum += s_red[g][tid];
      const int hh = s_heads[a];
      const int64_t pidx = ((int64_t)bh * p.umax + u) * p.G + hh;
      p.part_o[pidx * D + tid] = sum / s_l[a];
      if (tid == 0) p.part_lse[pidx] = s_m[a] + log2f(s_l[a]);
    }
    __syncthreads();
  }
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

bool launch_decode_attend(const DecodeAttnParams& p, hipStream_t s) {
  const int grid = p.B * p.Hkv * p.umax;
  {
    LaunchScope ls("decode_attend", s);
    if (p.D == 128) {
      if (p.G <= 4) hipLaunchKernelGGL((decode_attend_kernel<128, 4>), dim3(grid), dim3(256), 0, s, p);
      else hipLaunchKernelGGL((decode_attend_kernel<128, 8>), dim3(grid), dim3(256), 0, s, p);
    } else {
      if (p.G <= 4) hipLaunchKernelGGL((decode_attend_kernel<64, 4>), dim3(grid), dim3(256), 0, s, p);
      else hipLaunchKernelGGL((decode_attend_kernel<64, 8>), dim3(grid), dim3(256), 0, s, p);
    }
  }
  return launch_ok("decode_attend");
}

bool launch_decode_combine(const DecodeAttnParams& p, hipStream_t s) {
  {
    LaunchScope ls("decode_combine", s);
    hipLaunchKernelGGL(decode_combine_kernel, dim3((p.B * p.Hq + 3) / 4), dim3(256), 0, s, p);
  }
  return launch_ok("decode_combine");
}

}  // namespace bsa
