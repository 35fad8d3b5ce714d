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

// Union of the selections of the heads of one (b, kv head): distinct block ids
// ascending, each with a bit mask of the heads that chose it.
__global__ __launch_bounds__(64) void decode_union_kernel(DecodeAttnParams p) {
  constexpr int V = 8;  // up to 512 (head, block) pairs
  __shared__ uint64_t s_v[64 * V];
  const int lane = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const int nrow = p.per_group ? 1 : p.G;
  const int w = p.topk + 1;
  uint64_t v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = i * 64 + lane;
    uint64_t key = 0ull;
    if (e < nrow * w) {
      const int hh = e / w, s = e % w;
      const int hs = p.per_group ? hk : hk * p.G + hh;
      const int j = p.sel[((int64_t)b * p.Hs + hs) * w + s];
      if (j >= 0) {
        const uint64_t val = ((uint64_t)(uint32_t)j << 8) | (uint64_t)hh;
        key = ~val;  // descending sort of ~val = ascending val; empty slots (0) last
      }
    }
    v[i] = key;
  }
  wave_sort_desc<V>(v);
#pragma unroll
  for (int i = 0; i < V; ++i) s_v[i * 64 + lane] = v[i];
  __builtin_amdgcn_wave_barrier();
  __syncthreads();
  if (lane == 0) {
    int n = 0;
    int lastj = -1, mask = 0;
    int32_t* out = p.ulist + (int64_t)bh * p.umax;
    for (int e = 0; e < 64 * V; ++e) {
      const uint64_t key = s_v[e];
      if (key == 0ull) break;
      const uint64_t val = ~key;
      const int j = (int)(val >> 8), hh = (int)(val & 255);
      const int bits = p.per_group ? ((1 << p.G) - 1) : (1 << hh);
      if (j != lastj) {
        if (lastj >= 0) out[n++] = (lastj << 8) | mask;
        lastj = j;
        mask = 0;
      }
      mask |= bits;
    }
    if (lastj >= 0) out[n++] = (lastj << 8) | mask;
    p.ucount[bh] = n;
  }
}

// One workgroup per (b, kv head, distinct block): scores for the heads that
// chose the block, softmax over its keys, weighted sum of its values.
template <int D>
__global__ __launch_bounds__(256) void decode_attend_kernel(DecodeAttnParams p) {
  constexpr int KC = 128;  // keys per pass
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
  const int ke = min(ka + p.block, n);
  const uint16_t* kb = p.k + (int64_t)b * p.ks_b + (int64_t)hk * p.ks_h;
  const uint16_t* vb = p.v + (int64_t)b * p.vs_b + (int64_t)hk * p.vs_h;
  const int dc = tid % CH, kg = tid / CH;
  float acc[8][8];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[a][e] = 0.f;
  __syncthreads();

  for (int k0 = ka; k0 < ke; k0 += KC) {
    const int nk = min(KC, ke - k0);
    // scores: two threads per key, each half of the head dimension
    {
      const int key = tid >> 1, half = tid & 1;
      float part[8];
#pragma unroll
      for (int a = 0; a < 8; ++a) part[a] = 0.f;
      if (key < nk) {
        const uint16_t* kr = kb + (int64_t)(k0 + key) * p.ks_t + half * (D / 2);
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          const u16x8 x = ld16(kr + c * 8);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float kv = bf2f(x[e]);
            const int d = half * (D / 2) + c * 8 + e;
#pragma unroll
            for (int a = 0; a < 8; ++a)
              if (a < nh) part[a] = fmaf(s_q[a][d], kv, part[a]);
          }
        }
      }
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        if (a < nh) {
          const float tot = part[a] + __shfl_xor(part[a], 1, 64);
          if (half == 0 && key < KC) s_s[a][key] = key < nk ? tot * p.sl2 : -INFINITY;
        }
      }
    }
    __syncthreads();
    // softmax statistics per head (wave a handles heads a, a+4)
    for (int a = w; a < nh; a += 4) {
      const float x0 = s_s[a][lane], x1 = s_s[a][lane + 64];
      const float mx = wave_max(fmaxf(x0, x1));
      const float mold = s_m[a];
      const float mnew = fmaxf(mold, mx);
      const float e0 = exp2f(x0 - mnew), e1 = exp2f(x1 - mnew);
      s_s[a][lane] = e0;
      s_s[a][lane + 64] = e1;
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
      constexpr int KPG = KC / KG;
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        if (a < nh) {
          const float c = s_c[a];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[a][e] *= c;
        }
      }
      for (int kk = 0; kk < KPG; ++kk) {
        const int key = kg * KPG + kk;
        if (key < nk) {
          const u16x8 x = ld16(vb + (int64_t)(k0 + key) * p.vs_t + dc * 8);
#pragma unroll
          for (int a = 0; a < 8; ++a) {
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
  for (int a = 0; a < 8; ++a) {
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
  for (int u = 0; u < n; ++u) {
    const int ent = p.ulist[(int64_t)bh * p.umax + u];
    if (!((ent & 255) & (1 << hh))) continue;
    const int64_t pidx = ((int64_t)bh * p.umax + u) * p.G + hh;
    const float ls = p.part_lse[pidx];
    const float mnew = fmaxf(m, ls);
    const float c1 = exp2f(m - mnew), c2 = exp2f(ls - mnew);
    const float* src = p.part_o + pidx * p.D;
    a0 = a0 * c1 + c2 * (lane < p.D ? src[lane] : 0.f);
    a1 = a1 * c1 + c2 * (lane + 64 < p.D ? src[lane + 64] : 0.f);
    l = l * c1 + c2;
    m = mnew;
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  uint16_t* dst = p.o + (int64_t)b * p.os_b + (int64_t)h * p.os_h;
  if (lane < p.D) dst[lane] = f2bf(a0 * inv);
  if (lane + 64 < p.D) dst[lane + 64] = f2bf(a1 * inv);
  if (p.lse_out && lane == 0)
    p.lse_out[(int64_t)b * p.Hq + h] = l > 0.f ? (m + log2f(l)) * 0.69314718055994530942f : -INFINITY;
}

bool launch_decode_union(const DecodeAttnParams& p, hipStream_t s) {
  {
    LaunchScope ls("decode_union", s);
    hipLaunchKernelGGL(decode_union_kernel, dim3(p.B * p.Hkv), dim3(64), 0, s, p);
  }
  return launch_ok("decode_union");
}

bool launch_decode_attend(const DecodeAttnParams& p, hipStream_t s) {
  const int grid = p.B * p.Hkv * p.umax;
  {
    LaunchScope ls("decode_attend", s);
    if (p.D == 128)
      hipLaunchKernelGGL(decode_attend_kernel<128>, dim3(grid), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(decode_attend_kernel<64>, dim3(grid), dim3(256), 0, s, p);
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
