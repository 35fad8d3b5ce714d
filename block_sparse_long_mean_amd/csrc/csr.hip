// Selection inversion.  The gate gives, per selection row, a list of blocks;
// the gathered attention wants, per (b, kv head, block), the list of rows
// that chose the block, so that one block's keys and values are staged once
// for every row that needs them.  This is an implementation step, not part
// of the method: counting sort into buckets (histogram, exclusive scan,
// scatter), then one work item per (bucket, tile of rows).
//
// Order of entries inside a bucket follows atomic arrival and may vary run to
// run; every row's arithmetic is independent of which other rows share its
// tile, so outputs stay bitwise deterministic.
#include "bsa_device.h"
#include "bsa_internal.h"

namespace bsa {

constexpr int kScanChunk = 4096;  // elements per workgroup in the scans

// two ints (count total, tile total) per chunk
int64_t scan_tmp_len(int64_t n) { return 2 * ((n + kScanChunk - 1) / kScanChunk + 1); }

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

// Every valid entry of a selection row (the gate's blocks, then the forced own
// block when causal) becomes one bucket entry; slot = position in the row.
struct SelEntry {
  bool valid;
  int bucket;
  uint32_t packed;
};

BSA_DEV SelEntry decode_sel(const CsrParams& p, int64_t idx) {
  SelEntry r;
  r.valid = false;
  r.bucket = 0;
  r.packed = 0;
  const int slot = (int)(idx % p.sel_w);
  if (slot >= p.kslot) return r;
  const int64_t srow = idx / p.sel_w;
  const int j = p.sel[idx];
  if (j < 0 || j >= p.Nb) return r;
  const int t = (int)(srow % p.Lq);
  const int hs = (int)((srow / p.Lq) % p.Hs);
  const int b = (int)(srow / ((int64_t)p.Lq * p.Hs));
  const int hk = p.per_group ? hs : hs / p.G;
  const int hh = p.per_group ? 0 : hs % p.G;
  r.valid = true;
  r.bucket = ((b * p.Hkv + hk) * p.NC + t / p.CT) * p.Nb + j;
  r.packed = ((uint32_t)t << p.sh_t) | ((uint32_t)hh << p.sh_h) | (uint32_t)slot;
  return r;
}

__global__ __launch_bounds__(256) void csr_count_kernel(CsrParams p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const SelEntry e = decode_sel(p, i);
    if (e.valid) atomicAdd(&p.counts[e.bucket], 1);
  }
}

__global__ __launch_bounds__(256) void csr_scatter_kernel(CsrParams p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const SelEntry e = decode_sel(p, i);
    if (e.valid) {
      const int pos = p.bucket_off[e.bucket] + atomicAdd(&p.cursor[e.bucket], 1);
      p.entries[pos] = e.packed;
    }
  }
}

// LDS-histogram variants.  A segment is the run of selection rows of one
// (b, kv head, head of the group, chunk): consecutive tokens of one selection
// head whose entries all land in the chunk's Nb buckets.  A workgroup takes up
// to kRowsPerWG rows of a segment, counts its entries per block in LDS, and
// touches global counters once per block it saw.
constexpr int kHistMax = 8192;   // blocks per (b, kv head) handled in LDS
constexpr int kRowsPerWG = 1024; // selection rows per workgroup

// A workgroup's piece of a segment: rows [ra, ra + nrows) of sel (tokens
// t0 ..), the segment's first bucket and head-in-group field.
struct SegPiece {
  int64_t ra;
  int nrows, t0, base, hh;
};

BSA_DEV bool seg_rows(const CsrParams& p, int seg, int piece, SegPiece& sp) {
  const int c = seg % p.NC;
  int rest = seg / p.NC;
  const int hh = rest % p.Gs;
  rest /= p.Gs;
  const int hk = rest % p.Hkv;
  const int b = rest / p.Hkv;
  const int hs = p.per_group ? hk : hk * p.G + hh;
  const int t0 = c * p.CT + piece * kRowsPerWG;
  const int t1 = min(min(t0 + kRowsPerWG, c * p.CT + p.CT), p.Lq);
  sp.ra = ((int64_t)b * p.Hs + hs) * p.Lq + t0;
  sp.nrows = t1 - t0;
  sp.t0 = t0;
  sp.base = ((b * p.Hkv + hk) * p.NC + c) * p.Nb;
  sp.hh = p.per_group ? 0 : hh;
  return t0 < t1;
}

// Entry li (row li / sel_w, slot li % sel_w) of a piece; the quotient comes
// from a float reciprocal corrected by one step (li < 2^24).
BSA_DEV bool piece_entry(const CsrParams& p, const SegPiece& sp, int li, float inv_w, int& bucket, uint32_t& packed) {
  int lr = (int)((float)li * inv_w);
  if (lr * p.sel_w > li) --lr;
  else if ((lr + 1) * p.sel_w <= li) ++lr;
  const int slot = li - lr * p.sel_w;
  if (slot >= p.kslot) return false;
  const int j = p.sel[sp.ra * p.sel_w + li];
  if (j < 0 || j >= p.Nb) return false;
  bucket = sp.base + j;
  packed = ((uint32_t)(sp.t0 + lr) << p.sh_t) | ((uint32_t)sp.hh << p.sh_h) | (uint32_t)slot;
  return true;
}

__global__ __launch_bounds__(256) void csr_count_lds_kernel(CsrParams p) {
  __shared__ int hist[kHistMax];
  SegPiece sp;
  if (!seg_rows(p, blockIdx.x, blockIdx.y, sp)) return;  // uniform
  for (int j = threadIdx.x; j < p.Nb; j += 256) hist[j] = 0;
  __syncthreads();
  const float inv_w = 1.0f / (float)p.sel_w;
  const int ne = sp.nrows * p.sel_w;
  for (int li = threadIdx.x; li < ne; li += 256) {
    int bucket;
    uint32_t packed;
    if (piece_entry(p, sp, li, inv_w, bucket, packed)) atomicAdd(&hist[bucket - sp.base], 1);
  }
  __syncthreads();
  for (int j = threadIdx.x; j < p.Nb; j += 256)
    if (hist[j]) atomicAdd(&p.counts[sp.base + j], hist[j]);
}

__global__ __launch_bounds__(256) void csr_scatter_lds_kernel(CsrParams p) {
  __shared__ int hist[kHistMax];
  SegPiece sp;
  if (!seg_rows(p, blockIdx.x, blockIdx.y, sp)) return;  // uniform
  for (int j = threadIdx.x; j < p.Nb; j += 256) hist[j] = 0;
  __syncthreads();
  const float inv_w = 1.0f / (float)p.sel_w;
  const int ne = sp.nrows * p.sel_w;
  for (int li = threadIdx.x; li < ne; li += 256) {
    int bucket;
    uint32_t packed;
    if (piece_entry(p, sp, li, inv_w, bucket, packed)) atomicAdd(&hist[bucket - sp.base], 1);
  }
  __syncthreads();
  // reserve this workgroup's range in every bucket it touches
  for (int j = threadIdx.x; j < p.Nb; j += 256) {
    const int c = hist[j];
    if (c) hist[j] = p.bucket_off[sp.base + j] + atomicAdd(&p.cursor[sp.base + j], c);
  }
  __syncthreads();
  for (int li = threadIdx.x; li < ne; li += 256) {
    int bucket;
    uint32_t packed;
    if (piece_entry(p, sp, li, inv_w, bucket, packed)) p.entries[atomicAdd(&hist[bucket - sp.base], 1)] = packed;
  }
}

BSA_DEV int tiles_of(const CsrParams& p, int count) {
  const int rows = count * p.R;
  return (rows + p.rows_item - 1) / p.rows_item;
}

// --- exclusive scans of counts (-> bucket_off) and tiles (-> tile_off) -----
// phase 1: per-chunk totals of both quantities
__global__ __launch_bounds__(256) void scan_reduce_kernel(CsrParams p) {
  __shared__ int red[2][4];
  const int c = blockIdx.x;
  int a = 0, t = 0;
  for (int i = threadIdx.x; i < kScanChunk; i += 256) {
    const int64_t g = (int64_t)c * kScanChunk + i;
    if (g < p.nbk) {
      const int v = p.counts[g];
      a += v;
      t += tiles_of(p, v);
    }
  }
  for (int m = 32; m > 0; m >>= 1) {
    a += __shfl_xor(a, m, 64);
    t += __shfl_xor(t, m, 64);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][w] = a;
    red[1][w] = t;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    p.scan_tmp[2 * c] = red[0][0] + red[0][1] + red[0][2] + red[0][3];
    p.scan_tmp[2 * c + 1] = red[1][0] + red[1][1] + red[1][2] + red[1][3];
  }
}

// phase 2: exclusive scan of the chunk totals (single workgroup, sequential
// per thread segment); writes the grand totals at index nbk.
__global__ __launch_bounds__(256) void scan_chunks_kernel(CsrParams p, int nchunk) {
  __shared__ int sa[256], st[256];
  const int per = (nchunk + 255) / 256;
  const int i0 = threadIdx.x * per;
  int a = 0, t = 0;
  for (int i = i0; i < min(i0 + per, nchunk); ++i) {
    a += p.scan_tmp[2 * i];
    t += p.scan_tmp[2 * i + 1];
  }
  sa[threadIdx.x] = a;
  st[threadIdx.x] = t;
  __syncthreads();
  if (threadIdx.x == 0) {
    int ra = 0, rt = 0;
    for (int i = 0; i < 256; ++i) {
      const int xa = sa[i], xt = st[i];
      sa[i] = ra;
      st[i] = rt;
      ra += xa;
      rt += xt;
    }
    p.bucket_off[p.nbk] = ra;
    p.tile_off[p.nbk] = rt;
  }
  __syncthreads();
  int ra = sa[threadIdx.x], rt = st[threadIdx.x];
  for (int i = i0; i < min(i0 + per, nchunk); ++i) {
    const int xa = p.scan_tmp[2 * i], xt = p.scan_tmp[2 * i + 1];
    p.scan_tmp[2 * i] = ra;
    p.scan_tmp[2 * i + 1] = rt;
    ra += xa;
    rt += xt;
  }
}

// phase 3: per chunk, exclusive scan with the chunk base
__global__ __launch_bounds__(256) void scan_apply_kernel(CsrParams p) {
  __shared__ int wa[4], wt[4];
  const int c = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  constexpr int PER = kScanChunk / 256;  // 16 consecutive elements per thread
  const int64_t g0 = (int64_t)c * kScanChunk + threadIdx.x * PER;
  int va[PER], vt[PER];
  int a = 0, t = 0;
  for (int e = 0; e < PER; ++e) {
    const int64_t g = g0 + e;
    const int v = g < p.nbk ? p.counts[g] : 0;
    va[e] = v;
    vt[e] = g < p.nbk ? tiles_of(p, v) : 0;
    a += va[e];
    t += vt[e];
  }
  int ia = a, it = t;
  for (int m = 1; m < 64; m <<= 1) {
    const int oa = __shfl_up(ia, m, 64), ot = __shfl_up(it, m, 64);
    if (lane >= m) {
      ia += oa;
      it += ot;
    }
  }
  if (lane == 63) {
    wa[w] = ia;
    wt[w] = it;
  }
  __syncthreads();
  int ba = p.scan_tmp[2 * c] + ia - a, bt = p.scan_tmp[2 * c + 1] + it - t;
  for (int i = 0; i < w; ++i) {
    ba += wa[i];
    bt += wt[i];
  }
  for (int e = 0; e < PER; ++e) {
    const int64_t g = g0 + e;
    if (g < p.nbk) {
      p.bucket_off[g] = ba;
      p.tile_off[g] = bt;
    }
    ba += va[e];
    bt += vt[e];
  }
}

// one thread per bucket: write its work items {bucket, first entry, rows, b << 16 | kv head}
__global__ __launch_bounds__(256) void expand_items_kernel(CsrParams p) {
  const int ept = p.rows_item / p.R;  // entries per tile
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < p.nbk; g += (int64_t)gridDim.x * 256) {
    const int t0 = p.tile_off[g], t1 = p.tile_off[g + 1];
    const int e0 = p.bucket_off[g];
    const int rows = (p.bucket_off[g + 1] - e0) * p.R;
    for (int t = t0; t < t1; ++t) {
      const int k = t - t0;
      const int bh = (int)(g / ((int64_t)p.NC * p.Nb));
      p.items[t] = make_int4((int)g, e0 + k * ept, min(p.rows_item, rows - k * p.rows_item),
                             ((bh / p.Hkv) << 16) | (bh % p.Hkv));
    }
  }
}

static int grid_for(int64_t n) { return (int)std::max<int64_t>(1, std::min<int64_t>((n + 255) / 256, 16384)); }

bool launch_csr(const CsrParams& p, hipStream_t s) {
  const int64_t nsel = (int64_t)p.B * p.Hs * p.Lq * p.sel_w;
  const int nchunk = (int)((p.nbk + kScanChunk - 1) / kScanChunk);
  {
    LaunchScope ls("csr_fill", s);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(grid_for(p.nbk)), dim3(256), 0, s, p.counts, (int64_t)p.nbk, 0);
    hipLaunchKernelGGL(fill_i32_kernel, dim3(grid_for(p.nbk)), dim3(256), 0, s, p.cursor, (int64_t)p.nbk, 0);
  }
  if (!launch_ok("csr_fill")) return false;
  const int64_t nseg = (int64_t)p.B * p.Hkv * p.Gs * p.NC;
  const int pieces = (std::min(p.CT, p.Lq) + kRowsPerWG - 1) / kRowsPerWG;
  const dim3 lgrid((unsigned)nseg, (unsigned)pieces);
  const bool lds = p.Nb <= kHistMax && pieces <= 65535 && nseg < ((int64_t)1 << 31);
  {
    LaunchScope ls("csr_count", s);
    if (lds)
      hipLaunchKernelGGL(csr_count_lds_kernel, lgrid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(csr_count_kernel, dim3(grid_for(nsel)), dim3(256), 0, s, p, nsel);
  }
  if (!launch_ok("csr_count")) return false;
  {
    LaunchScope ls("csr_scan", s);
    hipLaunchKernelGGL(scan_reduce_kernel, dim3(nchunk), dim3(256), 0, s, p);
    hipLaunchKernelGGL(scan_chunks_kernel, dim3(1), dim3(256), 0, s, p, nchunk);
    hipLaunchKernelGGL(scan_apply_kernel, dim3(nchunk), dim3(256), 0, s, p);
  }
  if (!launch_ok("csr_scan")) return false;
  {
    LaunchScope ls("csr_scatter", s);
    if (lds)
      hipLaunchKernelGGL(csr_scatter_lds_kernel, lgrid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(csr_scatter_kernel, dim3(grid_for(nsel)), dim3(256), 0, s, p, nsel);
    hipLaunchKernelGGL(expand_items_kernel, dim3(grid_for(p.nbk)), dim3(256), 0, s, p);
  }
  return launch_ok("csr_scatter");
}

}  // namespace bsa
