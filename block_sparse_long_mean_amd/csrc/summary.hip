// Per-document positions, document-wise RoPE and per-block key summaries.
//
// Document-wise RoPE: "100 Millionen Token: Gedaechtnis oder Trugbild?"
// (aitalk.it), section "Das Gehirn mit zwei Geschwindigkeiten" -- the position
// counter restarts at 0 at every document start.  Block summaries (the
// routing keys of the same section) are the mean of each block's keys; the
// pages leave the summary function open and the mean is this library's
// reading.
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

// ---------------------------------------------------------------------------
// positions: pos[t] = t - (first index of the run of equal doc ids holding t)
// Two passes over fixed chunks of kPosChunk tokens: the last run start inside
// each chunk, then per token the latest run start at or before it.
// ---------------------------------------------------------------------------
constexpr int kPosPerThread = kPosChunk / 256;  // 16

__device__ int block_max_i32(int v, int* red) {
  for (int m = 32; m > 0; m >>= 1) v = max(v, __shfl_xor(v, m, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  int r = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = max(r, red[i]);
  return r;
}

__global__ __launch_bounds__(256) void doc_chunk_last_kernel(const int32_t* __restrict__ doc, int L, int nchunk,
                                                             int32_t* __restrict__ chunk_last) {
  __shared__ int red[4];
  const int b = blockIdx.y, c = blockIdx.x;
  const int32_t* d = doc + (int64_t)b * L;
  const int t0 = c * kPosChunk + threadIdx.x * kPosPerThread;
  int best = -1;
  for (int e = 0; e < kPosPerThread; ++e) {
    const int t = t0 + e;
    if (t < L && (t == 0 || d[t] != d[t - 1])) best = t;
  }
  best = block_max_i32(best, red);
  if (threadIdx.x == 0) chunk_last[(int64_t)b * nchunk + c] = best;
}

__global__ __launch_bounds__(256) void doc_positions_kernel(const int32_t* __restrict__ doc, int L, int nchunk,
                                                            const int32_t* __restrict__ chunk_last,
                                                            int32_t* __restrict__ pos) {
  __shared__ int red[4];
  __shared__ int wtot[4];
  const int b = blockIdx.y, c = blockIdx.x;
  const int32_t* d = doc + (int64_t)b * L;
  // latest run start in the chunks before this one
  int prev = -1;
  for (int i = threadIdx.x; i < c; i += 256) prev = max(prev, chunk_last[(int64_t)b * nchunk + i]);
  prev = block_max_i32(prev, red);
  // per thread: run starts inside its 16 tokens
  const int t0 = c * kPosChunk + threadIdx.x * kPosPerThread;
  int st[kPosPerThread];
  int run = -1;
  for (int e = 0; e < kPosPerThread; ++e) {
    const int t = t0 + e;
    if (t < L && (t == 0 || d[t] != d[t - 1])) run = t;
    st[e] = run;
  }
  // exclusive max-scan of the threads' last run start
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = run;
  for (int m = 1; m < 64; m <<= 1) {
    const int o = __shfl_up(incl, m, 64);
    if (lane >= m) incl = max(incl, o);
  }
  if (lane == 63) wtot[w] = incl;
  __syncthreads();
  int before = prev;
  for (int i = 0; i < w; ++i) before = max(before, wtot[i]);
  int ex = __shfl_up(incl, 1, 64);
  if (lane == 0) ex = -1;
  before = max(before, ex);
  int32_t* pp = pos + (int64_t)b * L;
  for (int e = 0; e < kPosPerThread; ++e) {
    const int t = t0 + e;
    if (t < L) pp[t] = t - max(before, st[e]);
  }
}

bool launch_doc_positions(const int32_t* doc, int B, int L, int32_t* chunk_last, int32_t* pos, hipStream_t s) {
  const int nc = pos_chunks(L);
  dim3 grid(nc, B);
  {
    LaunchScope ls("doc_chunk_last", s);
    hipLaunchKernelGGL(doc_chunk_last_kernel, grid, dim3(256), 0, s, doc, L, nc, chunk_last);
  }
  if (!launch_ok("doc_chunk_last")) return false;
  {
    LaunchScope ls("doc_positions", s);
    hipLaunchKernelGGL(doc_positions_kernel, grid, dim3(256), 0, s, doc, L, nc, chunk_last, pos);
  }
  return launch_ok("doc_positions");
}

// ---------------------------------------------------------------------------
// block summary
// One workgroup per (b, block j, group of hpw heads).  A "unit" is one head's
// pair of 16-byte chunks (elements [c*E, c*E+E) and [D/2 + c*E, ...)), so the
// two halves of every RoPE pair land in the same thread.  256 threads cover
// TP = 256 / U tokens per pass with U = hpw * D / (2E) units per token, so a
// wave reads whole contiguous key rows.
// ---------------------------------------------------------------------------
template <typename T>
struct Elt;
template <>
struct Elt<uint16_t> {
  static constexpr int E = 8;
  typedef u16x8 Raw;
  static BSA_DEV Raw raw(const uint16_t* p) { return ld16(p); }
  static BSA_DEV void cvt(Raw v, float* x) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = bf2f(v[e]);
  }
  static BSA_DEV void load(const uint16_t* p, float* x) { cvt(raw(p), x); }
  static BSA_DEV void store(uint16_t* p, const float* x) {
    u16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = f2bf(x[e]);
    st16(p, v);
  }
};
template <>
struct Elt<float> {
  static constexpr int E = 4;
  typedef f32x4 Raw;
  static BSA_DEV Raw raw(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
  static BSA_DEV void cvt(Raw v, float* x) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = v[e];
  }
  static BSA_DEV void load(const float* p, float* x) { cvt(raw(p), x); }
  static BSA_DEV void store(float* p, const float* x) {
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = x[e];
    *reinterpret_cast<f32x4*>(p) = v;
  }
};

template <typename T, int D, bool ROPE>
__global__ __launch_bounds__(256) void block_summary_kernel(SummaryParams p, int hpw) {
  typedef typename Elt<T>::Raw Raw;
  constexpr int E = Elt<T>::E;
  constexpr int UPH = D / (2 * E);
  constexpr int HALF = D / 2;
  constexpr int SUB = 64;  // tokens per rotation table
  constexpr int UNR = 4;   // passes whose rows are loaded together
  // the rotation table and the closing reduction share the LDS (a barrier
  // separates the table's last read from the reduction's first write)
  __shared__ union {
    struct {
      float cs[ROPE ? SUB : 1][ROPE ? HALF : 1];
      float sn[ROPE ? SUB : 1][ROPE ? HALF : 1];
    } tab;
    float red[2 * E][256];
  } s_mem;
  auto& s_cos = s_mem.tab.cs;
  auto& s_sin = s_mem.tab.sn;
  auto& s_red = s_mem.red;
  const int U = hpw * UPH;
  const int TP = 256 / U;
  const int tid = threadIdx.x;
  const int u = tid % U, tl = tid / U;
  const int hh = u / UPH, c = u % UPH;
  const int bj = blockIdx.x;
  const int b = bj / p.Nb, j = bj % p.Nb;
  const int h = blockIdx.y * hpw + hh;
  const int t0 = j * p.block;
  const int n = min(p.block, p.L - t0);
  const T* kb = reinterpret_cast<const T*>(p.k) + (int64_t)b * p.ks_b + (int64_t)h * p.ks_h;
  float acc[2 * E];
#pragma unroll
  for (int e = 0; e < 2 * E; ++e) acc[e] = 0.f;

  // rows of passes p0 .. p0 + UNR - 1 (token p0*TP + q*TP + tl of the sub-block)
  auto load_rows = [&](int tbase, int lim, Raw (&lo)[UNR], Raw (&hi)[UNR]) {
#pragma unroll
    for (int q = 0; q < UNR; ++q) {
      const int tt = tbase + q * TP + tl;
      lo[q] = Raw{};
      hi[q] = Raw{};
      if (tt < lim) {
        const T* row = kb + (int64_t)(t0 + tt) * p.ks_t;
        lo[q] = Elt<T>::raw(row + c * E);
        hi[q] = Elt<T>::raw(row + HALF + c * E);
      }
    }
  };
  // Sub-blocks of SUB tokens: the next rows are loaded before the rotation
  // table is built and before the current rows are used, so that every
  // thread keeps 2*UNR row loads in flight.
  for (int s0 = 0; s0 < n; s0 += SUB) {
    const int ns = min(SUB, n - s0);
    Raw lo[UNR], hi[UNR];
    load_rows(s0, s0 + ns, lo, hi);
    if constexpr (ROPE) {
      __syncthreads();  // the previous sub-block's table is no longer read
      // the rotation table, 16 tokens per wave: lane i of wave w walks tokens
      // 16w .. 16w + 15 of the sub-block for frequency i in double precision
      // -- the first token's angle reduced and evaluated directly, every next
      // one by a rotation through omega_i when its position is the previous
      // one + 1 (exactly 1, 0 at a document start, directly again after any
      // other jump) -- and rounds each (cos, sin) to fp32 once
      {
        constexpr int TPW = SUB / 4;
        const int wv = tid >> 6, ln = tid & 63;
        const int tb = wv * TPW;
        // lane l of the wave holds token tb + l's position (l < TPW)
        const int pl = (ln < TPW && tb + ln < ns) ? p.pos[(int64_t)b * p.L + t0 + s0 + tb + ln] : 0;
        if (ln < HALF && tb < ns) {
          const int te = min(tb + TPW, ns);
          const int i = ln;
          const double om = p.omega[i];
          double sd, cd;
          sincos(om, &sd, &cd);
          double cv, sv;
          int prev = __builtin_amdgcn_readfirstlane(pl);
          rope_sincos_d(prev, om, cv, sv);
          s_cos[tb][i] = (float)cv;
          s_sin[tb][i] = (float)sv;
          for (int tt = tb + 1; tt < te; ++tt) {
            const int ps = __builtin_amdgcn_readlane(pl, tt - tb);
            if (ps == prev + 1) {
              const double c2 = cv * cd - sv * sd;
              sv = fma(sv, cd, cv * sd);
              cv = c2;
            } else if (ps == 0) {
              cv = 1.0;
              sv = 0.0;
            } else {
              rope_sincos_d(ps, om, cv, sv);
            }
            prev = ps;
            s_cos[tt][i] = (float)cv;
            s_sin[tt][i] = (float)sv;
          }
        }
      }
      __syncthreads();
    }
    for (int p0 = 0; p0 < ns; p0 += UNR * TP) {
      Raw nlo[UNR], nhi[UNR];
      load_rows(s0 + p0 + UNR * TP, s0 + ns, nlo, nhi);
#pragma unroll
      for (int q = 0; q < UNR; ++q) {
        const int tt = p0 + q * TP + tl;  // token within the sub-block
        if (tt < ns) {
          float xl[E], xh[E];
          Elt<T>::cvt(lo[q], xl);
          Elt<T>::cvt(hi[q], xh);
          if constexpr (ROPE) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const float cs = s_cos[tt][c * E + e], sn = s_sin[tt][c * E + e];
              const float a = xl[e], bb = xh[e];
              xl[e] = a * cs - bb * sn;
              xh[e] = a * sn + bb * cs;
            }
            if (p.k_rot) {
              T* kr = reinterpret_cast<T*>(p.k_rot) + (((int64_t)b * p.L + t0 + s0 + tt) * p.H + h) * D;
              Elt<T>::store(kr + c * E, xl);
              Elt<T>::store(kr + HALF + c * E, xh);
            }
          }
#pragma unroll
          for (int e = 0; e < E; ++e) {
            acc[e] += xl[e];
            acc[E + e] += xh[e];
          }
        }
      }
#pragma unroll
      for (int q = 0; q < UNR; ++q) {
        lo[q] = nlo[q];
        hi[q] = nhi[q];
      }
    }
  }
  if constexpr (ROPE) __syncthreads();  // every thread is done with the table
#pragma unroll
  for (int e = 0; e < 2 * E; ++e) s_red[e][tid] = acc[e];
  __syncthreads();
  if (tl == 0) {
    for (int q = 1; q < TP; ++q) {
#pragma unroll
      for (int e = 0; e < 2 * E; ++e) acc[e] += s_red[e][q * U + u];
    }
    float mean[2 * E];
#pragma unroll
    for (int e = 0; e < 2 * E; ++e) mean[e] = acc[e] / (float)n;
    const int64_t pub = (((int64_t)b * p.Nb + j) * p.H + h) * D;
    const int64_t pln = (((int64_t)b * p.H + h) * p.Nb + j) * D;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int d0 = half * HALF + c * E;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float x = mean[half * E + e];
        if (p.pooled_f32) p.pooled_f32[pub + d0 + e] = x;
        if (p.pooled_bf16) p.pooled_bf16[pub + d0 + e] = f2bf(x);
        if (p.plane_hi) {
          __bf16 hi, lo;
          split_bf(x, hi, lo);
          p.plane_hi[pln + d0 + e] = __builtin_bit_cast(uint16_t, hi);
          p.plane_lo[pln + d0 + e] = __builtin_bit_cast(uint16_t, lo);
        }
      }
    }
  }
}

template <typename T, int D, bool ROPE>
static void run_summary(const SummaryParams& p, hipStream_t s) {
  constexpr int UPH = D / (2 * Elt<T>::E);
  // all heads in one workgroup when there are enough blocks to fill the chip
  int hpw = 1;
  if ((int64_t)p.B * p.Nb >= 2048 && (256 % (p.H * UPH)) == 0) hpw = p.H;
  dim3 grid(p.B * p.Nb, p.H / hpw);
  hipLaunchKernelGGL((block_summary_kernel<T, D, ROPE>), grid, dim3(256), 0, s, p, hpw);
}

bool launch_block_summary(const SummaryParams& p, hipStream_t s) {
  {
    LaunchScope ls("block_summary", s);
    const bool rope = p.pos != nullptr;
    if (p.is_bf16) {
      if (p.D == 128) rope ? run_summary<uint16_t, 128, true>(p, s) : run_summary<uint16_t, 128, false>(p, s);
      else rope ? run_summary<uint16_t, 64, true>(p, s) : run_summary<uint16_t, 64, false>(p, s);
    } else {
      if (p.D == 128) rope ? run_summary<float, 128, true>(p, s) : run_summary<float, 128, false>(p, s);
      else rope ? run_summary<float, 64, true>(p, s) : run_summary<float, 64, false>(p, s);
    }
  }
  return launch_ok("block_summary");
}

// ---------------------------------------------------------------------------
// RoPE on queries: one thread per (b, t, h, pair chunk of 4 pairs)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void rope_q_kernel(RopeQParams p) {
  const int half = p.D / 2;
  const int cpr = half / 4;  // 4-pair chunks per row
  const int64_t total = (int64_t)p.B * p.L * p.H * cpr;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int c = (int)(idx % cpr);
    int64_t r = idx / cpr;
    const int h = (int)(r % p.H);
    r /= p.H;
    const int t = (int)(r % p.L);
    const int b = (int)(r / p.L);
    const T* row = reinterpret_cast<const T*>(p.q) + (int64_t)b * p.qs_b + (int64_t)t * p.qs_t + (int64_t)h * p.qs_h;
    const int ps = p.pos[(int64_t)b * p.L + t];
    const int64_t ob = (((int64_t)b * p.L + t) * p.H + h) * p.D;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = c * 4 + e;
      float xa, xb;
      if constexpr (sizeof(T) == 2) {
        xa = bf2f(row[i]);
        xb = bf2f(row[i + half]);
      } else {
        xa = row[i];
        xb = row[i + half];
      }
      float cs, sn;
      rope_sincos(ps, p.omega[i], cs, sn);
      const float ya = xa * cs - xb * sn, yb = xa * sn + xb * cs;
      if (p.out32) {
        p.out32[ob + i] = ya;
        p.out32[ob + i + half] = yb;
      }
      if (p.out16) {
        p.out16[ob + i] = f2bf(ya);
        p.out16[ob + i + half] = f2bf(yb);
      }
    }
  }
}

bool launch_rope_q(const RopeQParams& p, hipStream_t s) {
  const int64_t total = (int64_t)p.B * p.L * p.H * (p.D / 8);
  const int grid = (int)std::min<int64_t>((total + 255) / 256, 65536);
  {
    LaunchScope ls("rope_q", s);
    if (p.is_bf16)
      hipLaunchKernelGGL(rope_q_kernel<uint16_t>, dim3(grid), dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(rope_q_kernel<float>, dim3(grid), dim3(256), 0, s, p);
  }
  return launch_ok("rope_q");
}

// ---------------------------------------------------------------------------
// caller-supplied summaries -> gate planes
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void pooled_to_planes_kernel(const void* pooled, int is_bf16, int64_t ps_b,
                                                               int64_t ps_j, int64_t ps_h, int B, int Nb, int H,
                                                               int D, uint16_t* hi, uint16_t* lo) {
  const int64_t total = (int64_t)B * Nb * H * D;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (int64_t)gridDim.x * 256) {
    const int d = (int)(idx % D);
    int64_t r = idx / D;
    const int j = (int)(r % Nb);
    r /= Nb;
    const int h = (int)(r % H);
    const int b = (int)(r / H);
    const int64_t src = (int64_t)b * ps_b + (int64_t)j * ps_j + (int64_t)h * ps_h + d;
    const float x = is_bf16 ? bf2f(reinterpret_cast<const uint16_t*>(pooled)[src])
                            : reinterpret_cast<const float*>(pooled)[src];
    __bf16 a, c;
    split_bf(x, a, c);
    hi[idx] = __builtin_bit_cast(uint16_t, a);
    if (lo) lo[idx] = __builtin_bit_cast(uint16_t, c);
  }
}

bool launch_pooled_to_planes(const void* pooled, int is_bf16, int64_t ps_b, int64_t ps_j, int64_t ps_h, int B,
                             int Nb, int H, int D, uint16_t* hi, uint16_t* lo, hipStream_t s) {
  const int64_t total = (int64_t)B * Nb * H * D;
  const int grid = (int)std::min<int64_t>((total + 255) / 256, 65536);
  {
    LaunchScope ls("pooled_to_planes", s);
    hipLaunchKernelGGL(pooled_to_planes_kernel, dim3(grid), dim3(256), 0, s, pooled, is_bf16, ps_b, ps_j, ps_h, B,
                       Nb, H, D, hi, lo);
  }
  return launch_ok("pooled_to_planes");
}

}  // namespace bsa
