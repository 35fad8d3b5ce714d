// C ABI of libbsa: argument validation, workspace layout and launch order.
#include <math.h>
#include <stdio.h>

#include <algorithm>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "bsa.h"
#include "bsa_internal.h"

#define BSA_API extern "C" __attribute__((visibility("default")))

namespace bsa {

// ---------------------------------------------------------------------------
// errors
// ---------------------------------------------------------------------------
static thread_local std::string g_err;
void set_error(const std::string& msg) { g_err = msg; }

static bsa_status fail(bsa_status st, const std::string& msg) {
  set_error(msg);
  return st;
}

bool launch_ok(const char* name) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error(std::string("launch of ") + name + " failed: " + hipGetErrorString(e));
    return false;
  }
  return true;
}

// ---------------------------------------------------------------------------
// launch timer
// ---------------------------------------------------------------------------
struct TimerRec {
  std::string name;
  hipEvent_t a, b;
};
static int g_timer_level = 0;
static std::vector<TimerRec> g_timer;

LaunchScope::LaunchScope(const char* n, hipStream_t s, int level) : name(n), stream(s), slot(-1) {
  if (g_timer_level < level) return;
  TimerRec r;
  r.name = n;
  if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) return;
  (void)hipEventRecord(r.a, s);
  g_timer.push_back(r);
  slot = (int)g_timer.size() - 1;
}
LaunchScope::~LaunchScope() {
  if (slot >= 0) (void)hipEventRecord(g_timer[slot].b, stream);
}

static void timer_clear() {
  for (auto& r : g_timer) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_timer.clear();
}

// ---------------------------------------------------------------------------
// workspace carving
// ---------------------------------------------------------------------------
struct Carver {
  size_t off = 0;
  char* base = nullptr;
  template <typename T>
  T* take(int64_t n) {
    off = (off + 255) & ~(size_t)255;
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += (size_t)std::max<int64_t>(n, 0) * sizeof(T);
    return p;
  }
};

static void omega_table(double theta, int D, double* out) {
  for (int i = 0; i < D / 2; ++i) out[i] = pow(theta, -2.0 * (double)i / (double)D);
}

static bool dim_ok(int D) { return D == 64 || D == 128; }

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// Every tensor may be device memory or pinned host memory mapped into the
// device's address space at the same address (hipHostMalloc, a pinned
// tensor); kernels then read the host copy over the host link.  This is how a
// memory's content keys and values stay in host RAM while its routing keys
// stay in HBM ("100 Millionen Token ...", section "Das Gehirn mit zwei
// Geschwindigkeiten").  Pageable host memory cannot be read by a kernel: it
// is rejected before anything is enqueued.
static bool resident_one(const void* p) {
  if (!p) return true;
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();  // the failed query must not surface as a later launch error
    return false;
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged || at.isManaged) return true;
  if (at.type != hipMemoryTypeHost || !at.devicePointer || !at.hostPointer) return false;
  const char* dev = (const char*)at.devicePointer + ((const char*)p - (const char*)at.hostPointer);
  return dev == (const char*)p;
}

static bsa_status resident(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (!resident_one(p))
      return fail(BSA_ERR_INVALID_ARG, "a tensor is neither device memory nor pinned host memory mapped for the device");
  return BSA_OK;
}

static bool strides_ok(const int64_t* s, int n, int D, int elt) {
  for (int i = 0; i < n; ++i)
    if (s[i] < 0 || ((s[i] * elt) & 15) != 0) return false;
  (void)D;
  return true;
}

// ---------------------------------------------------------------------------
// prefill plan
// ---------------------------------------------------------------------------
struct PrefillPlan {
  int Nb, Hs, G, Dg, topk, kslot, sel_w, R, Gs, nbk;
  bool bf16, per_group, use_index, rope_q, rope_k, have_pooled;
  int nsplit, span, gate_qkind, ntiles, rows_per_bh;
  int64_t nsel_rows, max_entries, max_items;
  int attn_grid;
  int NC, CT, CPL;  // query chunks per (b, kv head), tokens per chunk, chunks per attention pass
  // workspace pointers
  int32_t *pos_q, *pos_k, *chunk_q, *chunk_k;
  uint16_t *q16, *k16;
  float *q32, *k32;
  uint16_t *p_hi, *p_lo;
  float* pooled32;
  uint64_t* part_keys;
  int32_t* sel;
  int32_t *counts, *cursor, *bucket_off, *tile_off, *scan_tmp;
  uint32_t* entries;
  int4* items;
  uint16_t* part_o;
  float2* part_ml;
  int sh_h, sh_t, lgR;
  size_t bytes;
};

// consecutive work items a gather workgroup takes at a time (runs are dealt
// round-robin to the workgroups of an XCD).  Blocks of one 64-key tile stay
// staged across consecutive items of a bucket, so their workgroups take long
// runs; longer blocks are re-staged by every item, and single items dealt
// round-robin keep the XCD's workgroups on the same few blocks at once (their
// keys and values then come from the XCD's L2).
constexpr int kGatherRun = 64;
// below this many rows per selected (b, kv head, block) on average, the
// gather takes the sparse-bucket kernel
constexpr int kSparseRows = 8;
// query bytes of one (b, kv head) chunk of the default chunk size
constexpr int64_t kChunkQueryBytes = (int64_t)64 << 20;

static int ceil_log2(int x) {
  int b = 0;
  while ((1 << b) < x) ++b;
  return b;
}

static int gate_waves_for(int rows_per_bh, int topk) {
  (void)topk;
  return rows_per_bh <= 16 ? 1 : 4;
}

static bsa_status plan_prefill(const bsa_prefill_args* a, PrefillPlan& P, char* ws, bool gate_only) {
  if (!a) return fail(BSA_ERR_INVALID_ARG, "args is NULL");
  if (a->dtype != BSA_DTYPE_F32 && a->dtype != BSA_DTYPE_BF16) return fail(BSA_ERR_INVALID_ARG, "dtype");
  if (a->B < 1 || a->Lq < 1 || a->Lk < 1 || a->Hq < 1 || a->Hkv < 1) return fail(BSA_ERR_INVALID_ARG, "sizes must be >= 1");
  if (a->Hq % a->Hkv) return fail(BSA_ERR_INVALID_ARG, "Hq must be a multiple of Hkv");
  if (!dim_ok(a->D)) return fail(BSA_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  if (a->block < 1) return fail(BSA_ERR_INVALID_ARG, "block must be >= 1");
  if (a->topk < 0) return fail(BSA_ERR_INVALID_ARG, "topk must be >= 0");
  if (a->causal != 0 && a->causal != 1) return fail(BSA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (a->causal && a->Lq > a->Lk) return fail(BSA_ERR_INVALID_ARG, "causal needs Lq <= Lk");
  if (a->gate_mode != BSA_GATE_PER_HEAD && a->gate_mode != BSA_GATE_PER_GROUP) return fail(BSA_ERR_INVALID_ARG, "gate_mode");
  if (!a->q || !a->k) return fail(BSA_ERR_INVALID_ARG, "q and k are required");
  if (!gate_only && (!a->v || !a->o)) return fail(BSA_ERR_INVALID_ARG, "v and o are required");
  if (gate_only && !a->sel_out) return fail(BSA_ERR_INVALID_ARG, "sel_out is required for bsa_select_blocks");
  if ((a->index_q == nullptr) != (a->index_k == nullptr)) return fail(BSA_ERR_INVALID_ARG, "index_q and index_k go together");
  if (a->pooled && !aligned16(a->pooled)) return fail(BSA_ERR_INVALID_ARG, "pooled must be 16-byte aligned");
  if ((a->pooled_hi == nullptr) != (a->pooled_lo == nullptr))
    return fail(BSA_ERR_INVALID_ARG, "pooled_hi and pooled_lo go together");
  if (a->pooled_hi) {
    if (a->pooled) return fail(BSA_ERR_INVALID_ARG, "give pooled or pooled_hi / pooled_lo, not both");
    if (a->dtype != BSA_DTYPE_BF16) return fail(BSA_ERR_UNSUPPORTED, "pooled_hi / pooled_lo are for bf16 inputs");
    if (!aligned16(a->pooled_hi) || !aligned16(a->pooled_lo))
      return fail(BSA_ERR_INVALID_ARG, "pooled_hi / pooled_lo must be 16-byte aligned");
  }
  const int elt = a->dtype == BSA_DTYPE_BF16 ? 2 : 4;
  if (!aligned16(a->q) || !aligned16(a->k) || (a->v && !aligned16(a->v)) || (a->o && !aligned16(a->o)))
    return fail(BSA_ERR_INVALID_ARG, "tensor base pointers must be 16-byte aligned");
  if (!strides_ok(a->q_stride, 3, a->D, elt) || !strides_ok(a->k_stride, 3, a->D, elt) ||
      (!gate_only && (!strides_ok(a->v_stride, 3, a->D, elt) || !strides_ok(a->o_stride, 3, a->D, elt))))
    return fail(BSA_ERR_INVALID_ARG, "strides must be non-negative and keep rows 16-byte aligned");
  P.bf16 = a->dtype == BSA_DTYPE_BF16;
  P.per_group = a->gate_mode == BSA_GATE_PER_GROUP;
  P.use_index = a->index_q != nullptr;
  P.G = a->Hq / a->Hkv;
  P.Nb = (int)(((int64_t)a->Lk + a->block - 1) / a->block);
  P.Hs = P.per_group ? a->Hkv : a->Hq;
  P.Dg = P.use_index ? a->Di : a->D;
  if (P.use_index) {
    if (!dim_ok(a->Di)) return fail(BSA_ERR_UNSUPPORTED, "index dim must be 64 or 128");
    if (!aligned16(a->index_q) || !aligned16(a->index_k) || !strides_ok(a->iq_stride, 3, a->Di, elt) ||
        !strides_ok(a->ik_stride, 3, a->Di, elt))
      return fail(BSA_ERR_INVALID_ARG, "index tensor alignment/strides");
  }
  if (a->topk > BSA_MAX_TOPK) return fail(BSA_ERR_UNSUPPORTED, "topk above BSA_MAX_TOPK");
  P.topk = std::min(a->topk, P.Nb);
  P.sel_w = a->topk + (a->causal ? 1 : 0);
  P.kslot = std::max(P.sel_w, 1);  // one partial slot per selection entry (own block included)
  P.R = P.per_group ? P.G : 1;
  P.Gs = P.per_group ? 1 : P.G;
  P.rope_q = a->doc_ids_q != nullptr;
  P.rope_k = a->doc_ids_k != nullptr;
  P.have_pooled = a->pooled != nullptr || a->pooled_hi != nullptr;
  if (P.per_group && P.G > 8 && !P.bf16) {
    // fp32 path sums in the gate kernel, no restriction; keep for symmetry
  }
  P.nsel_rows = (int64_t)a->B * P.Hs * a->Lq;
  if (P.nsel_rows * P.sel_w >= (int64_t)1 << 31) return fail(BSA_ERR_UNSUPPORTED, "too many selection entries");
  P.sh_h = ceil_log2(P.kslot);
  P.sh_t = P.sh_h + ceil_log2(P.Gs);
  P.lgR = ceil_log2(P.R);
  if (P.sh_t >= 31 || (int64_t)(a->Lq - 1) >= ((int64_t)1 << (32 - P.sh_t)))
    return fail(BSA_ERR_UNSUPPORTED, "Lq too large for the packed selection entries");
  if ((int64_t)a->B * a->Hkv * P.Nb >= (int64_t)1 << 30) return fail(BSA_ERR_UNSUPPORTED, "too many KV blocks");
  if (a->chunk_tokens < 0) return fail(BSA_ERR_INVALID_ARG, "chunk_tokens must be >= 0");
  if (a->chunks_per_pass < 0) return fail(BSA_ERR_INVALID_ARG, "chunks_per_pass must be >= 0");
  {
    // Query tokens of one (b, kv head) are attended in chunks of CT tokens:
    // the gather works through its items chunk by chunk, and a chunk's query
    // rows (re-read once per block they chose) stay in the memory-side cache
    // while it does.  The default chunk holds about 64 MiB of queries.
    // Chunks run in passes (gather + merge) whose partial outputs fit a
    // workspace budget; the budget is large, one pass over everything is
    // fastest (the cache does not keep the gather's written partials for
    // the merge), so it only bounds the workspace of very long inputs.
    const int64_t per_tok = (int64_t)P.G * P.kslot * (2 * a->D + 8);  // partial bytes per (token, kv head)
    const int64_t budget = (int64_t)40 << 30;
    const int64_t nbh = (int64_t)a->B * a->Hkv;
    if (a->chunk_tokens > 0) {
      P.CT = std::min(a->chunk_tokens, a->Lq);
    } else {
      const int64_t q_bytes = (int64_t)P.G * a->D * 2;  // query bytes per (token, kv head)
      int64_t ct = 1024;
      while (ct * 2 * q_bytes <= kChunkQueryBytes && ct * 2 * per_tok <= budget) ct *= 2;
      P.CT = (int)std::min<int64_t>(ct, a->Lq);
    }
    P.NC = (a->Lq + P.CT - 1) / P.CT;
    const int64_t fit = std::max<int64_t>(1, budget / std::max<int64_t>(1, per_tok * P.CT));
    P.CPL = (int)std::min<int64_t>(nbh * P.NC, a->chunks_per_pass > 0 ? a->chunks_per_pass : fit);
    if (nbh * P.NC * P.Nb >= (int64_t)1 << 30) return fail(BSA_ERR_UNSUPPORTED, "too many (chunk, block) buckets");
    if (nbh * P.NC * P.CT * P.G >= (int64_t)1 << 31) return fail(BSA_ERR_UNSUPPORTED, "too many query rows");
  }
  P.nbk = a->B * a->Hkv * P.NC * P.Nb;
  P.max_entries = P.nsel_rows * (P.topk + (a->causal ? 1 : 0));
  if (P.per_group && (128 % P.G) != 0) return fail(BSA_ERR_UNSUPPORTED, "per-group gating needs G dividing 128");
  const int rows_item = 32 * gather_waves(a->block);
  P.max_items = (P.max_entries * P.R + rows_item - 1) / rows_item + std::min<int64_t>(P.nbk, P.max_entries);
  // gate geometry
  P.rows_per_bh = P.per_group ? a->Lq : a->Lq * P.G;
  const int W = gate_waves_for(P.rows_per_bh, P.topk);
  P.ntiles = (P.rows_per_bh + 16 * W - 1) / (16 * W);
  const int64_t base_wg = (int64_t)a->B * a->Hkv * P.ntiles;
  const int ncand_max = P.Nb;
  P.nsplit = 1;
  if (P.bf16 && P.topk > 0 && base_wg < 2048) {
    // Too few row tiles to fill the chip: split the candidates, aiming at the
    // workgroups the device holds at once -- three per CU for lists of more
    // than 16 keys (their summaries staged by DMA, three waves per SIMD), two
    // otherwise.  Each split pays for its own top-k warm-up and merge
    // entries, so more splits than that cost more than they gain: the 10M-token
    // memory's 512-query chunk (256 row tiles, top-64) measured its gate at
    // 3.37 ms with 3 splits and 3.77 with 2 (gate + merge with registers
    // staging the summaries: 4.07 ms with 2, 4.6 with 4, 5.2 with 8, 5.7 with 1).
    const int fill = P.topk > 16 ? 768 : 512;
    const int want = (int)std::min<int64_t>((fill + base_wg - 1) / base_wg, (ncand_max + 255) / 256);
    P.nsplit = std::max(1, want);
  }
  P.span = (ncand_max + P.nsplit - 1) / P.nsplit;
  P.span = (P.span + 63) / 64 * 64;
  P.nsplit = (ncand_max + P.span - 1) / P.span;
  if (P.nsplit < 1) P.nsplit = 1;
  P.attn_grid = 256 * 8;  // persistent: 8 workgroups per CU

  Carver c;
  c.base = ws;
  const int64_t B = a->B, Lq = a->Lq, Lk = a->Lk;
  P.pos_q = P.rope_q ? c.take<int32_t>(B * Lq) : nullptr;
  P.chunk_q = P.rope_q ? c.take<int32_t>(B * pos_chunks((int)Lq)) : nullptr;
  P.pos_k = P.rope_k ? c.take<int32_t>(B * Lk) : nullptr;
  P.chunk_k = P.rope_k ? c.take<int32_t>(B * pos_chunks((int)Lk)) : nullptr;
  P.q16 = (P.rope_q && P.bf16) ? c.take<uint16_t>(B * Lq * a->Hq * a->D) : nullptr;
  P.q32 = (P.rope_q && (!P.bf16 || !P.use_index)) ? c.take<float>(B * Lq * a->Hq * a->D) : nullptr;
  P.k16 = (P.rope_k && P.bf16) ? c.take<uint16_t>(B * Lk * a->Hkv * a->D) : nullptr;
  P.k32 = (P.rope_k && !P.bf16) ? c.take<float>(B * Lk * a->Hkv * a->D) : nullptr;
  const int64_t npool = (int64_t)a->B * a->Hkv * P.Nb * P.Dg;
  if (P.bf16) {
    // caller-provided fp32 summaries are read by the gate directly
    P.p_hi = P.have_pooled ? nullptr : c.take<uint16_t>(npool);
    P.p_lo = P.have_pooled ? nullptr : c.take<uint16_t>(npool);
    P.pooled32 = nullptr;
  } else {
    P.p_hi = P.p_lo = nullptr;
    P.pooled32 = P.have_pooled ? nullptr : c.take<float>(npool);
  }
  P.part_keys = (P.nsplit > 1) ? c.take<uint64_t>(P.nsel_rows * P.nsplit * P.topk) : nullptr;
  P.sel = a->sel_out ? a->sel_out : c.take<int32_t>(P.nsel_rows * P.sel_w);
  if (P.bf16 && !gate_only) {
    P.counts = c.take<int32_t>(P.nbk);
    P.cursor = c.take<int32_t>(P.nbk);
    P.bucket_off = c.take<int32_t>(P.nbk + 1);
    P.tile_off = c.take<int32_t>(P.nbk + 1);
    P.scan_tmp = c.take<int32_t>(scan_tmp_len(P.nbk));
    P.entries = c.take<uint32_t>(P.max_entries + 256);  // speculative reads past the end stay inside
    P.items = c.take<int4>(P.max_items);
    const int64_t part_rows = (int64_t)P.CPL * P.Gs * P.CT * P.kslot * P.R;
    P.part_o = c.take<uint16_t>(part_rows * a->D);
    P.part_ml = c.take<float2>(part_rows);
  } else {
    P.counts = P.cursor = P.bucket_off = P.tile_off = P.scan_tmp = nullptr;
    P.entries = nullptr;
    P.items = nullptr;
    P.part_o = nullptr;
    P.part_ml = nullptr;
  }
  P.bytes = c.off + 256;
  return BSA_OK;
}

static bsa_status run_prefill(const bsa_prefill_args* a, void* ws, size_t ws_bytes, void* stream, bool gate_only) {
  PrefillPlan P;
  bsa_status st = plan_prefill(a, P, nullptr, gate_only);
  if (st != BSA_OK) return st;
  if (!ws || ws_bytes < P.bytes) return fail(BSA_ERR_WORKSPACE, "workspace smaller than bsa_prefill_workspace_bytes");
  if (((uintptr_t)ws & 255) != 0) return fail(BSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  st = resident({a->q, a->k, a->v, a->o, a->index_q, a->index_k, a->doc_ids_q, a->doc_ids_k, a->pooled, a->pooled_hi, a->pooled_lo, a->sel_out,
                 a->lse_out, ws});
  if (st != BSA_OK) return st;
  plan_prefill(a, P, reinterpret_cast<char*>(ws), gate_only);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const double theta = a->rope_theta > 0.f ? (double)a->rope_theta : 10000.0;
  const int elt = P.bf16 ? 2 : 4;
  (void)elt;

  // 1. positions and RoPE
  const void* q_att = a->q;
  int64_t qa_s[3] = {a->q_stride[0], a->q_stride[1], a->q_stride[2]};
  const void* k_att = a->k;
  int64_t ka_s[3] = {a->k_stride[0], a->k_stride[1], a->k_stride[2]};
  const int64_t qc_s[3] = {(int64_t)a->Lq * a->Hq * a->D, (int64_t)a->Hq * a->D, a->D};
  const int64_t kc_s[3] = {(int64_t)a->Lk * a->Hkv * a->D, (int64_t)a->Hkv * a->D, a->D};
  if (P.rope_q) {
    if (!launch_doc_positions(a->doc_ids_q, a->B, a->Lq, P.chunk_q, P.pos_q, s)) return BSA_ERR_HIP;
    RopeQParams rp;
    rp.is_bf16 = P.bf16;
    rp.B = a->B; rp.L = a->Lq; rp.H = a->Hq; rp.D = a->D;
    rp.q = a->q; rp.qs_b = a->q_stride[0]; rp.qs_t = a->q_stride[1]; rp.qs_h = a->q_stride[2];
    rp.pos = P.pos_q;
    omega_table(theta, a->D, rp.omega);
    rp.out16 = P.q16;
    rp.out32 = P.q32;
    if (!launch_rope_q(rp, s)) return BSA_ERR_HIP;
    q_att = P.bf16 ? (const void*)P.q16 : (const void*)P.q32;
    for (int i = 0; i < 3; ++i) qa_s[i] = qc_s[i];
  }
  const bool summarize = !P.have_pooled;
  if (P.rope_k) {
    if (!launch_doc_positions(a->doc_ids_k, a->B, a->Lk, P.chunk_k, P.pos_k, s)) return BSA_ERR_HIP;
  }
  // 2. block summaries (+ rotated keys)
  {
    SummaryParams sp;
    sp.is_bf16 = P.bf16;
    sp.B = a->B; sp.L = a->Lk; sp.H = a->Hkv; sp.block = a->block; sp.Nb = P.Nb;
    sp.pooled_f32 = nullptr; sp.pooled_bf16 = nullptr; sp.plane_hi = nullptr; sp.plane_lo = nullptr; sp.k_rot = nullptr;
    omega_table(theta, a->D, sp.omega);
    if (P.use_index) {
      // index keys drive the gate; keys for attention are rotated separately
      if (summarize) {
        sp.D = a->Di; sp.k = a->index_k;
        sp.ks_b = a->ik_stride[0]; sp.ks_t = a->ik_stride[1]; sp.ks_h = a->ik_stride[2];
        sp.pos = nullptr;
        if (P.bf16) { sp.plane_hi = P.p_hi; sp.plane_lo = P.p_lo; } else sp.pooled_f32 = P.pooled32;
        if (!launch_block_summary(sp, s)) return BSA_ERR_HIP;
      }
      if (P.rope_k && !gate_only) {
        SummaryParams kr = sp;
        kr.D = a->D; kr.k = a->k; kr.ks_b = a->k_stride[0]; kr.ks_t = a->k_stride[1]; kr.ks_h = a->k_stride[2];
        kr.pos = P.pos_k; kr.plane_hi = kr.plane_lo = nullptr; kr.pooled_f32 = nullptr; kr.pooled_bf16 = nullptr;
        kr.k_rot = P.bf16 ? (void*)P.k16 : (void*)P.k32;
        if (!launch_block_summary(kr, s)) return BSA_ERR_HIP;
      }
    } else if (summarize || (P.rope_k && !gate_only)) {
      sp.D = a->D; sp.k = a->k;
      sp.ks_b = a->k_stride[0]; sp.ks_t = a->k_stride[1]; sp.ks_h = a->k_stride[2];
      sp.pos = P.pos_k;
      if (summarize) {
        if (P.bf16) { sp.plane_hi = P.p_hi; sp.plane_lo = P.p_lo; } else sp.pooled_f32 = P.pooled32;
      }
      if (P.rope_k && !gate_only) sp.k_rot = P.bf16 ? (void*)P.k16 : (void*)P.k32;
      if (!launch_block_summary(sp, s)) return BSA_ERR_HIP;
    }
    if (P.rope_k) {
      k_att = P.bf16 ? (const void*)P.k16 : (const void*)P.k32;
      for (int i = 0; i < 3; ++i) ka_s[i] = kc_s[i];
    }
  }
  // 3. gate + top-k
  // gate query source: index q, else (rotated) q
  const void* gq = P.use_index ? a->index_q : (P.rope_q ? (P.bf16 ? (const void*)P.q32 : (const void*)P.q32) : a->q);
  int64_t gq_s[3];
  if (P.use_index) { for (int i = 0; i < 3; ++i) gq_s[i] = a->iq_stride[i]; }
  else if (P.rope_q) { for (int i = 0; i < 3; ++i) gq_s[i] = qc_s[i]; }
  else { for (int i = 0; i < 3; ++i) gq_s[i] = a->q_stride[i]; }
  const bool gq_f32 = !P.bf16 || (P.rope_q && !P.use_index);
  if (P.bf16) {
    GateParams g;
    g.B = a->B; g.Lq = a->Lq; g.Lk = a->Lk; g.Hkv = a->Hkv; g.G = P.G; g.Hs = P.Hs; g.per_group = P.per_group;
    g.rows_per_bh = P.rows_per_bh; g.ntiles = P.ntiles;
    g.q = gq; g.qs_b = gq_s[0]; g.qs_t = gq_s[1]; g.qs_h = gq_s[2];
    g.qkind = gq_f32 ? 1 : (P.per_group ? 2 : 0);
    g.Dg = P.Dg;
    if (a->pooled_hi) {
      // the caller's planes [B, Hkv, Nb, Dg], laid out as the library's own
      g.p_hi = a->pooled_hi; g.p_lo = a->pooled_lo; g.p_f32 = nullptr;
      g.ps_h = (int64_t)P.Nb * P.Dg; g.ps_b = (int64_t)a->Hkv * g.ps_h; g.ps_j = P.Dg;
    } else if (P.have_pooled) {
      // the caller's fp32 summaries [B, Nb, Hkv, Dg], split into bf16 hi + lo as the gate stages them
      g.p_hi = g.p_lo = nullptr;
      g.p_f32 = reinterpret_cast<const float*>(a->pooled);
      g.ps_h = P.Dg; g.ps_j = (int64_t)a->Hkv * P.Dg; g.ps_b = (int64_t)P.Nb * g.ps_j;
    } else {
      g.p_hi = P.p_hi; g.p_lo = P.p_lo; g.p_f32 = nullptr;
      g.ps_h = (int64_t)P.Nb * P.Dg; g.ps_b = (int64_t)a->Hkv * g.ps_h; g.ps_j = P.Dg;
    }
    g.Nb = P.Nb; g.causal = a->causal; g.block = a->block; g.lens = nullptr;
    g.topk = P.topk; g.nsplit = P.nsplit; g.span = P.span;
    g.sel = P.sel; g.sel_w = P.sel_w; g.part = P.part_keys; g.tag = "gate";
    if (!launch_gate(g, s)) return BSA_ERR_HIP;
    if (P.nsplit > 1 && !launch_gate_merge(g, s)) return BSA_ERR_HIP;
  } else {
    GateF32Params g;
    g.B = a->B; g.Lq = a->Lq; g.Lk = a->Lk; g.Hkv = a->Hkv; g.G = P.G; g.Hs = P.Hs; g.per_group = P.per_group;
    g.Dg = P.Dg;
    g.q = reinterpret_cast<const float*>(gq); g.qs_b = gq_s[0]; g.qs_t = gq_s[1]; g.qs_h = gq_s[2];
    g.pooled = P.have_pooled ? a->pooled : P.pooled32;
    g.Nb = P.Nb; g.causal = a->causal; g.block = a->block; g.topk = P.topk;
    g.sel = P.sel; g.sel_w = P.sel_w;
    if (!launch_gate_f32(g, s)) return BSA_ERR_HIP;
  }
  if (gate_only) return BSA_OK;

  // 4. attention
  const float scale = a->scale != 0.f ? a->scale : (float)(1.0 / sqrt((double)a->D));
  if (!P.bf16) {
    AttnF32Params f;
    f.B = a->B; f.Lq = a->Lq; f.Lk = a->Lk; f.Hq = a->Hq; f.Hkv = a->Hkv; f.G = P.G; f.D = a->D; f.block = a->block;
    f.Hs = P.Hs; f.per_group = P.per_group; f.causal = a->causal;
    f.q = reinterpret_cast<const float*>(q_att); f.qs_b = qa_s[0]; f.qs_t = qa_s[1]; f.qs_h = qa_s[2];
    f.k = reinterpret_cast<const float*>(k_att); f.ks_b = ka_s[0]; f.ks_t = ka_s[1]; f.ks_h = ka_s[2];
    f.v = reinterpret_cast<const float*>(a->v); f.vs_b = a->v_stride[0]; f.vs_t = a->v_stride[1]; f.vs_h = a->v_stride[2];
    f.scale = scale;
    f.sel = P.sel; f.sel_w = P.sel_w;
    f.o = reinterpret_cast<float*>(a->o); f.os_b = a->o_stride[0]; f.os_t = a->o_stride[1]; f.os_h = a->o_stride[2];
    f.lse_out = a->lse_out;
    if (!launch_attn_rowwise_f32(f, s)) return BSA_ERR_HIP;
    return BSA_OK;
  }
  AttnParams ap;
  ap.B = a->B; ap.Lq = a->Lq; ap.Lk = a->Lk; ap.Hq = a->Hq; ap.Hkv = a->Hkv; ap.G = P.G; ap.D = a->D;
  ap.block = a->block; ap.Nb = P.Nb; ap.Hs = P.Hs; ap.per_group = P.per_group; ap.Gs = P.Gs; ap.R = P.R;
  ap.kslot = P.kslot; ap.causal = a->causal; ap.topk = P.topk;
  ap.sh_h = P.sh_h; ap.sh_t = P.sh_t; ap.lgR = P.lgR;
  ap.q = reinterpret_cast<const uint16_t*>(q_att); ap.qs_b = qa_s[0]; ap.qs_t = qa_s[1]; ap.qs_h = qa_s[2];
  ap.k = reinterpret_cast<const uint16_t*>(k_att); ap.ks_b = ka_s[0]; ap.ks_t = ka_s[1]; ap.ks_h = ka_s[2];
  ap.v = reinterpret_cast<const uint16_t*>(a->v); ap.vs_b = a->v_stride[0]; ap.vs_t = a->v_stride[1]; ap.vs_h = a->v_stride[2];
  ap.sl2 = (float)((double)scale * 1.4426950408889634074);
  ap.entries = P.entries; ap.bucket_off = P.bucket_off; ap.tile_off = P.tile_off; ap.items = P.items;
  ap.NC = P.NC; ap.CT = P.CT;
  ap.grid = P.attn_grid;
  ap.rows_item = 32 * gather_waves(a->block);
  ap.run_items = gather_waves(a->block) > 4 ? 1 : kGatherRun;
  // a few rows per selected block on average (a short query chunk over a very
  // long memory): the sparse-bucket gather streams each block from HBM
  // instead of staging it for an MFMA tile of mostly empty rows.  The test
  // counts blocks per (b, kv head), not buckets, so that the query chunking
  // (a scheduling choice) never changes which kernel computes a result.
  const double blocks = (double)a->B * a->Hkv * P.Nb;
  ap.sparse_items = (double)P.max_entries * P.R < kSparseRows * blocks && P.max_items < ((int64_t)1 << 31)
                        ? P.max_items : 0;
  ap.part_o = P.part_o; ap.part_ml = P.part_ml;
  ap.sel = P.sel; ap.sel_w = P.sel_w;
  ap.o = reinterpret_cast<uint16_t*>(a->o); ap.os_b = a->o_stride[0]; ap.os_t = a->o_stride[1]; ap.os_h = a->o_stride[2];
  ap.lse_out = a->lse_out;
  if (P.max_entries > 0) {
    CsrParams cp;
    cp.B = a->B; cp.Lq = a->Lq; cp.Lk = a->Lk; cp.Hkv = a->Hkv; cp.G = P.G; cp.Hs = P.Hs; cp.per_group = P.per_group;
    cp.Nb = P.Nb; cp.block = a->block; cp.causal = a->causal;
    cp.Gs = P.Gs; cp.NC = P.NC; cp.CT = P.CT;
    cp.sel = P.sel; cp.sel_w = P.sel_w; cp.kslot = P.kslot; cp.R = P.R; cp.rows_item = 32 * gather_waves(a->block);
    cp.sh_h = P.sh_h; cp.sh_t = P.sh_t;
    cp.counts = P.counts; cp.cursor = P.cursor; cp.bucket_off = P.bucket_off; cp.tile_off = P.tile_off;
    cp.scan_tmp = P.scan_tmp; cp.entries = P.entries; cp.items = P.items; cp.nbk = P.nbk;
    if (!launch_csr(cp, s)) return BSA_ERR_HIP;
  }
  // attention passes: gather then merge, CPL chunks at a time
  LaunchScope phase("attn", s);
  const int nchunks = a->B * a->Hkv * P.NC;
  for (int c0 = 0; c0 < nchunks; c0 += P.CPL) {
    ap.c0 = c0;
    ap.c1 = std::min(nchunks, c0 + P.CPL);
    if (P.max_entries > 0 && !launch_attn_gather(ap, s)) return BSA_ERR_HIP;
    if (!launch_attn_merge(ap, s)) return BSA_ERR_HIP;
  }
  return BSA_OK;
}

// ---------------------------------------------------------------------------
// decode plan
// ---------------------------------------------------------------------------
struct DecodePlan {
  int Nb, Hs, G, topk, umax, sel_w, nshare;
  uint64_t* skeys;
  int32_t* scnt;
  int32_t* sel;
  int32_t *ulist, *ucount;
  float *part_o, *part_lse;
  size_t bytes;
};

static bsa_status plan_decode(const bsa_decode_args* a, DecodePlan& P, char* ws) {
  if (!a) return fail(BSA_ERR_INVALID_ARG, "args is NULL");
  if (a->dtype != BSA_DTYPE_BF16) return fail(BSA_ERR_UNSUPPORTED, "decode supports bf16 q/k/v");
  if (a->B < 1 || a->Lc < 1 || a->Hq < 1 || a->Hkv < 1) return fail(BSA_ERR_INVALID_ARG, "sizes must be >= 1");
  if (a->Hq % a->Hkv) return fail(BSA_ERR_INVALID_ARG, "Hq must be a multiple of Hkv");
  if (!dim_ok(a->D)) return fail(BSA_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  if (a->block < 1) return fail(BSA_ERR_INVALID_ARG, "block must be >= 1");
  if (a->topk < 0) return fail(BSA_ERR_INVALID_ARG, "topk must be >= 0");
  if (a->topk > BSA_MAX_TOPK) return fail(BSA_ERR_UNSUPPORTED, "topk above BSA_MAX_TOPK");
  if (a->gate_mode != BSA_GATE_PER_HEAD && a->gate_mode != BSA_GATE_PER_GROUP) return fail(BSA_ERR_INVALID_ARG, "gate_mode");
  if (a->pooled_dtype != BSA_DTYPE_BF16 && a->pooled_dtype != BSA_DTYPE_F32) return fail(BSA_ERR_INVALID_ARG, "pooled_dtype");
  if (!a->q || !a->kcache || !a->vcache || !a->pooled || !a->o) return fail(BSA_ERR_INVALID_ARG, "q, kcache, vcache, pooled and o are required");
  P.G = a->Hq / a->Hkv;
  if (P.G > 8) return fail(BSA_ERR_UNSUPPORTED, "decode supports at most 8 query heads per KV head");
  if (a->block_table && a->num_pages < 1) return fail(BSA_ERR_INVALID_ARG, "num_pages must be >= 1 with a block table");
  if (a->block_table && ((uintptr_t)a->block_table & 3)) return fail(BSA_ERR_INVALID_ARG, "block_table must be 4-byte aligned");
  if (a->block > (1 << 22)) return fail(BSA_ERR_UNSUPPORTED, "block too large");
  P.Nb = (int)(((int64_t)a->Lc + a->block - 1) / a->block);
  if (P.Nb >= (1 << 23)) return fail(BSA_ERR_UNSUPPORTED, "too many blocks for decode");
  if (a->block_table && a->table_w < P.Nb) return fail(BSA_ERR_INVALID_ARG, "table_w must be >= ceil(Lc / block)");
  const bool per_group = a->gate_mode == BSA_GATE_PER_GROUP;
  P.Hs = per_group ? a->Hkv : a->Hq;
  P.topk = std::min(a->topk, P.Nb);
  P.sel_w = a->topk + 1;
  if ((per_group ? 1 : P.G) * P.sel_w > 512) return fail(BSA_ERR_UNSUPPORTED, "G * (topk + 1) above 512");
  P.umax = (per_group ? 1 : P.G) * P.sel_w;
  if (!aligned16(a->q) || !aligned16(a->kcache) || !aligned16(a->vcache) || !aligned16(a->pooled) || !aligned16(a->o))
    return fail(BSA_ERR_INVALID_ARG, "tensor base pointers must be 16-byte aligned");
  const int pe = a->pooled_dtype == BSA_DTYPE_BF16 ? 2 : 4;
  if (!strides_ok(a->q_stride, 2, a->D, 2) || !strides_ok(a->k_stride, 3, a->D, 2) || !strides_ok(a->v_stride, 3, a->D, 2) ||
      !strides_ok(a->o_stride, 2, a->D, 2) || !strides_ok(a->p_stride, 3, a->D, pe))
    return fail(BSA_ERR_INVALID_ARG, "strides must be non-negative and keep rows 16-byte aligned");
  Carver c;
  c.base = ws;
  const int64_t nrows = (int64_t)a->B * P.Hs;
  P.nshare = (P.Nb + kDecShare - 1) / kDecShare;
  P.skeys = c.take<uint64_t>(nrows * P.nshare * std::max(P.topk, 1));
  P.scnt = c.take<int32_t>(nrows * P.nshare);
  P.sel = a->sel_out ? a->sel_out : c.take<int32_t>(nrows * P.sel_w);
  P.ulist = c.take<int32_t>((int64_t)a->B * a->Hkv * P.umax);
  P.ucount = c.take<int32_t>((int64_t)a->B * a->Hkv);
  P.part_o = c.take<float>((int64_t)a->B * a->Hkv * P.umax * P.G * a->D);
  P.part_lse = c.take<float>((int64_t)a->B * a->Hkv * P.umax * P.G);
  P.bytes = c.off + 256;
  return BSA_OK;
}

// own_ws: the workspace is the library's own scratch array (device memory by
// construction), left out of the residency check
static bsa_status run_decode(const bsa_decode_args* a, void* ws, size_t ws_bytes, void* stream, bool own_ws = false) {
  DecodePlan P;
  bsa_status st = plan_decode(a, P, nullptr);
  if (st != BSA_OK) return st;
  if (!ws || ws_bytes < P.bytes) return fail(BSA_ERR_WORKSPACE, "workspace smaller than bsa_decode_workspace_bytes");
  if (((uintptr_t)ws & 255) != 0) return fail(BSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  st = resident({a->q, a->kcache, a->vcache, a->pooled, a->cache_lens, a->o, a->sel_out, a->lse_out, a->block_table,
                 own_ws ? nullptr : ws});
  if (st != BSA_OK) return st;
  plan_decode(a, P, reinterpret_cast<char*>(ws));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool per_group = a->gate_mode == BSA_GATE_PER_GROUP;
  DecodeGateParams g;
  g.B = a->B; g.Lc = a->Lc; g.Hq = a->Hq; g.Hkv = a->Hkv; g.G = P.G; g.D = a->D; g.block = a->block; g.Nb = P.Nb;
  g.Hs = P.Hs; g.per_group = per_group; g.topk = P.topk; g.sel_w = P.sel_w; g.lens = a->cache_lens;
  g.q = reinterpret_cast<const uint16_t*>(a->q); g.qs_b = a->q_stride[0]; g.qs_h = a->q_stride[1];
  g.pooled = a->pooled; g.pooled_bf16 = a->pooled_dtype == BSA_DTYPE_BF16;
  g.ps_b = a->p_stride[0]; g.ps_j = a->p_stride[1]; g.ps_h = a->p_stride[2];
  g.nshare = P.nshare; g.skeys = P.skeys; g.scnt = P.scnt; g.sel = P.sel; g.ulist = P.ulist; g.ucount = P.ucount; g.umax = P.umax;
  if (!launch_decode_gate(g, s)) return BSA_ERR_HIP;
  DecodeAttnParams d;
  d.B = a->B; d.Lc = a->Lc; d.Hq = a->Hq; d.Hkv = a->Hkv; d.G = P.G; d.D = a->D; d.block = a->block; d.Hs = P.Hs;
  d.per_group = per_group; d.topk = a->topk; d.umax = P.umax; d.lens = a->cache_lens;
  d.table = a->block_table; d.table_w = a->table_w; d.num_pages = a->num_pages;
  d.q = reinterpret_cast<const uint16_t*>(a->q); d.qs_b = a->q_stride[0]; d.qs_h = a->q_stride[1];
  d.k = reinterpret_cast<const uint16_t*>(a->kcache); d.ks_b = a->k_stride[0]; d.ks_t = a->k_stride[1]; d.ks_h = a->k_stride[2];
  d.v = reinterpret_cast<const uint16_t*>(a->vcache); d.vs_b = a->v_stride[0]; d.vs_t = a->v_stride[1]; d.vs_h = a->v_stride[2];
  const float scale = a->scale != 0.f ? a->scale : (float)(1.0 / sqrt((double)a->D));
  d.sl2 = (float)((double)scale * 1.4426950408889634074);
  d.sel = P.sel; d.ulist = P.ulist; d.ucount = P.ucount; d.part_o = P.part_o; d.part_lse = P.part_lse;
  d.o = reinterpret_cast<uint16_t*>(a->o); d.os_b = a->o_stride[0]; d.os_h = a->o_stride[1];
  d.lse_out = a->lse_out;
  if (!launch_decode_attend(d, s)) return BSA_ERR_HIP;
  if (!launch_decode_combine(d, s)) return BSA_ERR_HIP;
  return BSA_OK;
}

// ---------------------------------------------------------------------------
// backward plan
// ---------------------------------------------------------------------------
struct BackwardPlan {
  int G, Nb, Hs, Gs, R, kslot, sh_h, sh_t, lgR, NC, CT, rows_item;
  int64_t nsel_rows, max_entries, max_items, nbk;
  int32_t *counts, *cursor, *bucket_off, *tile_off, *scan_tmp;
  uint32_t* entries;
  int4* items;
  float *delta, *dq_part;
  size_t bytes;
};

static bsa_status plan_backward(const bsa_backward_args* a, BackwardPlan& P, char* ws) {
  if (!a) return fail(BSA_ERR_INVALID_ARG, "args is NULL");
  if (a->dtype != BSA_DTYPE_BF16) return fail(BSA_ERR_UNSUPPORTED, "backward supports bf16 q/k/v");
  if (a->B < 1 || a->Lq < 1 || a->Lk < 1 || a->Hq < 1 || a->Hkv < 1) return fail(BSA_ERR_INVALID_ARG, "sizes must be >= 1");
  if (a->Hq % a->Hkv) return fail(BSA_ERR_INVALID_ARG, "Hq must be a multiple of Hkv");
  if (!dim_ok(a->D)) return fail(BSA_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  if (a->block < 1) return fail(BSA_ERR_INVALID_ARG, "block must be >= 1");
  if (a->causal != 0 && a->causal != 1) return fail(BSA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (a->causal && a->Lq > a->Lk) return fail(BSA_ERR_INVALID_ARG, "causal needs Lq <= Lk");
  if (a->gate_mode != BSA_GATE_PER_HEAD && a->gate_mode != BSA_GATE_PER_GROUP) return fail(BSA_ERR_INVALID_ARG, "gate_mode");
  if (a->sel_w < 0 || a->sel_w > BSA_MAX_TOPK + 1) return fail(BSA_ERR_INVALID_ARG, "sel_w must be in [0, BSA_MAX_TOPK + 1]");
  if (!a->q || !a->k || !a->v || !a->o || !a->dout || !a->lse || (!a->sel && a->sel_w > 0) || !a->dq || !a->dk || !a->dv)
    return fail(BSA_ERR_INVALID_ARG, "q, k, v, o, dout, lse, sel, dq, dk and dv are required");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o) || !aligned16(a->dout) ||
      !aligned16(a->dq) || !aligned16(a->dk) || !aligned16(a->dv))
    return fail(BSA_ERR_INVALID_ARG, "tensor base pointers must be 16-byte aligned");
  if (!strides_ok(a->q_stride, 3, a->D, 2) || !strides_ok(a->k_stride, 3, a->D, 2) || !strides_ok(a->v_stride, 3, a->D, 2) ||
      !strides_ok(a->o_stride, 3, a->D, 2) || !strides_ok(a->do_stride, 3, a->D, 2))
    return fail(BSA_ERR_INVALID_ARG, "strides must be non-negative and keep rows 16-byte aligned");
  const bool per_group = a->gate_mode == BSA_GATE_PER_GROUP;
  P.G = a->Hq / a->Hkv;
  if (per_group && (128 % P.G) != 0) return fail(BSA_ERR_UNSUPPORTED, "per-group gating needs G dividing 128");
  P.Nb = (int)(((int64_t)a->Lk + a->block - 1) / a->block);
  P.Hs = per_group ? a->Hkv : a->Hq;
  P.Gs = per_group ? 1 : P.G;
  P.R = per_group ? P.G : 1;
  P.kslot = std::max(a->sel_w, 1);
  P.sh_h = ceil_log2(P.kslot);
  P.sh_t = P.sh_h + ceil_log2(P.Gs);
  P.lgR = ceil_log2(P.R);
  P.nsel_rows = (int64_t)a->B * P.Hs * a->Lq;
  if (P.nsel_rows * std::max(a->sel_w, 1) >= (int64_t)1 << 31) return fail(BSA_ERR_UNSUPPORTED, "too many selection entries");
  if (P.sh_t >= 31 || (int64_t)(a->Lq - 1) >= ((int64_t)1 << (32 - P.sh_t)))
    return fail(BSA_ERR_UNSUPPORTED, "Lq too large for the packed selection entries");
  // Query chunks: a (chunk, block) bucket's entries are sorted in LDS (at
  // most CT * Gs of them); the longest chunks the sort holds.
  P.CT = std::min(a->Lq, kBwdSortCap / P.Gs);
  P.NC = (a->Lq + P.CT - 1) / P.CT;
  P.nbk = (int64_t)a->B * a->Hkv * P.NC * P.Nb;
  if (P.nbk >= (int64_t)1 << 30) return fail(BSA_ERR_UNSUPPORTED, "too many (chunk, block) buckets");
  // dq work items: consecutive runs of up to kBwdItemRows rows of a bucket
  // (each (row, slot) partial is summed inside one item, so any split keeps
  // the sums in a fixed order)
  P.rows_item = kBwdItemRows;
  P.max_entries = P.nsel_rows * a->sel_w;
  P.max_items = (P.max_entries * P.R + P.rows_item - 1) / P.rows_item + std::min<int64_t>(P.nbk, P.max_entries);
  if (P.max_items >= (int64_t)1 << 31) return fail(BSA_ERR_UNSUPPORTED, "too many work items");
  Carver c;
  c.base = ws;
  P.counts = c.take<int32_t>(P.nbk);
  P.cursor = c.take<int32_t>(P.nbk);
  P.bucket_off = c.take<int32_t>(P.nbk + 1);
  P.tile_off = c.take<int32_t>(P.nbk + 1);
  P.scan_tmp = c.take<int32_t>(scan_tmp_len(P.nbk));
  P.entries = c.take<uint32_t>(P.max_entries + 256);
  P.items = c.take<int4>(std::max<int64_t>(P.max_items, 1));
  P.delta = c.take<float>((int64_t)a->B * a->Hq * a->Lq);
  // partial rows per (b, kv head, chunk, head of the group): CT each, the last chunk padded
  P.dq_part = c.take<float>((int64_t)a->B * a->Hkv * P.NC * P.Gs * P.CT * P.kslot * P.R * a->D);
  P.bytes = c.off + 256;
  return BSA_OK;
}

static bsa_status run_backward(const bsa_backward_args* a, void* ws, size_t ws_bytes, void* stream) {
  BackwardPlan P;
  bsa_status st = plan_backward(a, P, nullptr);
  if (st != BSA_OK) return st;
  if (!ws || ws_bytes < P.bytes) return fail(BSA_ERR_WORKSPACE, "workspace smaller than bsa_backward_workspace_bytes");
  if (((uintptr_t)ws & 255) != 0) return fail(BSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  st = resident({a->q, a->k, a->v, a->o, a->dout, a->lse, a->sel, a->dq, a->dk, a->dv, ws});
  if (st != BSA_OK) return st;
  plan_backward(a, P, reinterpret_cast<char*>(ws));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool per_group = a->gate_mode == BSA_GATE_PER_GROUP;
  const float scale = a->scale != 0.f ? a->scale : (float)(1.0 / sqrt((double)a->D));
  AttnParams ap{};
  ap.B = a->B; ap.Lq = a->Lq; ap.Lk = a->Lk; ap.Hq = a->Hq; ap.Hkv = a->Hkv; ap.G = P.G; ap.D = a->D;
  ap.block = a->block; ap.Nb = P.Nb; ap.Hs = P.Hs; ap.per_group = per_group; ap.Gs = P.Gs; ap.R = P.R;
  ap.kslot = P.kslot; ap.causal = a->causal; ap.sh_h = P.sh_h; ap.sh_t = P.sh_t; ap.lgR = P.lgR;
  ap.q = reinterpret_cast<const uint16_t*>(a->q); ap.qs_b = a->q_stride[0]; ap.qs_t = a->q_stride[1]; ap.qs_h = a->q_stride[2];
  ap.k = reinterpret_cast<const uint16_t*>(a->k); ap.ks_b = a->k_stride[0]; ap.ks_t = a->k_stride[1]; ap.ks_h = a->k_stride[2];
  ap.v = reinterpret_cast<const uint16_t*>(a->v); ap.vs_b = a->v_stride[0]; ap.vs_t = a->v_stride[1]; ap.vs_h = a->v_stride[2];
  ap.o = const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(a->o));
  ap.os_b = a->o_stride[0]; ap.os_t = a->o_stride[1]; ap.os_h = a->o_stride[2];
  ap.dout = reinterpret_cast<const uint16_t*>(a->dout);
  ap.dos_b = a->do_stride[0]; ap.dos_t = a->do_stride[1]; ap.dos_h = a->do_stride[2];
  ap.sl2 = (float)((double)scale * 1.4426950408889634074);
  ap.scale = scale;
  ap.entries = P.entries; ap.bucket_off = P.bucket_off; ap.tile_off = P.tile_off; ap.items = P.items;
  ap.counts = P.counts;
  ap.NC = P.NC; ap.CT = P.CT; ap.c0 = 0; ap.c1 = a->B * a->Hkv * P.NC;
  ap.rows_item = P.rows_item;
  ap.grid = P.max_entries > 0 ? (int)P.max_items : 0;
  ap.sel = a->sel; ap.sel_w = a->sel_w;
  ap.lse_in = a->lse; ap.delta = P.delta; ap.dq_part = P.dq_part;
  ap.dq = a->dq; ap.dk = a->dk; ap.dv = a->dv;
  CsrParams cp;
  cp.B = a->B; cp.Lq = a->Lq; cp.Lk = a->Lk; cp.Hkv = a->Hkv; cp.G = P.G; cp.Hs = P.Hs; cp.per_group = per_group;
  cp.Nb = P.Nb; cp.block = a->block; cp.causal = a->causal;
  cp.Gs = P.Gs; cp.NC = P.NC; cp.CT = P.CT;
  cp.sel = a->sel; cp.sel_w = a->sel_w; cp.kslot = P.kslot; cp.R = P.R; cp.rows_item = P.rows_item;
  cp.sh_h = P.sh_h; cp.sh_t = P.sh_t;
  cp.counts = P.counts; cp.cursor = P.cursor; cp.bucket_off = P.bucket_off; cp.tile_off = P.tile_off;
  cp.scan_tmp = P.scan_tmp; cp.entries = P.entries; cp.items = P.items; cp.nbk = (int)P.nbk;
  if (P.max_entries > 0 && !launch_csr(cp, s)) return BSA_ERR_HIP;
  if (!launch_attn_backward(ap, (int64_t)a->B * a->Lq * a->Hq, s)) return BSA_ERR_HIP;
  return BSA_OK;
}

// ---------------------------------------------------------------------------
// summary
// ---------------------------------------------------------------------------
static bsa_status plan_summary(const bsa_summary_args* a, int32_t** chunk, int32_t** pos, char* ws, size_t* bytes) {
  if (!a) return fail(BSA_ERR_INVALID_ARG, "args is NULL");
  if (a->dtype != BSA_DTYPE_F32 && a->dtype != BSA_DTYPE_BF16) return fail(BSA_ERR_INVALID_ARG, "dtype");
  if (a->B < 1 || a->L < 1 || a->H < 1 || a->block < 1) return fail(BSA_ERR_INVALID_ARG, "sizes must be >= 1");
  if (!dim_ok(a->D)) return fail(BSA_ERR_UNSUPPORTED, "head dim must be 64 or 128");
  if (!a->k || !a->pooled) return fail(BSA_ERR_INVALID_ARG, "k and pooled are required");
  if (a->pooled_dtype != BSA_DTYPE_F32 && a->pooled_dtype != BSA_DTYPE_BF16) return fail(BSA_ERR_INVALID_ARG, "pooled_dtype");
  if ((a->k_rot || a->pos_out) && !a->doc_ids) return fail(BSA_ERR_INVALID_ARG, "k_rot/pos_out need doc_ids");
  if ((a->plane_hi == nullptr) != (a->plane_lo == nullptr)) return fail(BSA_ERR_INVALID_ARG, "plane_hi and plane_lo go together");
  const int elt = a->dtype == BSA_DTYPE_BF16 ? 2 : 4;
  if (!aligned16(a->k) || !strides_ok(a->k_stride, 3, a->D, elt)) return fail(BSA_ERR_INVALID_ARG, "k alignment/strides");
  if ((int64_t)a->B * ((a->L + a->block - 1) / a->block) >= (int64_t)1 << 31) return fail(BSA_ERR_UNSUPPORTED, "too many blocks");
  Carver c;
  c.base = ws;
  *pos = nullptr;
  *chunk = nullptr;
  if (a->doc_ids) {
    *chunk = c.take<int32_t>((int64_t)a->B * pos_chunks(a->L));
    *pos = a->pos_out ? a->pos_out : c.take<int32_t>((int64_t)a->B * a->L);
  }
  *bytes = c.off + 256;
  return BSA_OK;
}

static bsa_status run_summary(const bsa_summary_args* a, void* ws, size_t ws_bytes, void* stream) {
  int32_t *chunk, *pos;
  size_t need;
  bsa_status st = plan_summary(a, &chunk, &pos, nullptr, &need);
  if (st != BSA_OK) return st;
  if (a->doc_ids) {
    if (!ws || ws_bytes < need) return fail(BSA_ERR_WORKSPACE, "workspace smaller than bsa_summary_workspace_bytes");
    if (((uintptr_t)ws & 255) != 0) return fail(BSA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    plan_summary(a, &chunk, &pos, reinterpret_cast<char*>(ws), &need);
  }
  st = resident({a->k, a->doc_ids, a->pooled, a->k_rot, a->pos_out, a->plane_hi, a->plane_lo, a->doc_ids ? ws : nullptr});
  if (st != BSA_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (a->doc_ids && !launch_doc_positions(a->doc_ids, a->B, a->L, chunk, pos, s)) return BSA_ERR_HIP;
  SummaryParams sp;
  sp.is_bf16 = a->dtype == BSA_DTYPE_BF16;
  sp.B = a->B; sp.L = a->L; sp.H = a->H; sp.D = a->D; sp.block = a->block;
  sp.Nb = (a->L + a->block - 1) / a->block;
  sp.k = a->k; sp.ks_b = a->k_stride[0]; sp.ks_t = a->k_stride[1]; sp.ks_h = a->k_stride[2];
  sp.pos = a->doc_ids ? pos : nullptr;
  omega_table(a->rope_theta > 0.f ? (double)a->rope_theta : 10000.0, a->D, sp.omega);
  sp.pooled_f32 = a->pooled_dtype == BSA_DTYPE_F32 ? reinterpret_cast<float*>(a->pooled) : nullptr;
  sp.pooled_bf16 = a->pooled_dtype == BSA_DTYPE_BF16 ? reinterpret_cast<uint16_t*>(a->pooled) : nullptr;
  sp.plane_hi = a->plane_hi;
  sp.plane_lo = a->plane_lo;
  sp.k_rot = a->k_rot;
  return launch_block_summary(sp, s) ? BSA_OK : BSA_ERR_HIP;
}

}  // namespace bsa

// ---------------------------------------------------------------------------
// exported symbols
// ---------------------------------------------------------------------------
using namespace bsa;

BSA_API size_t bsa_prefill_workspace_bytes(const bsa_prefill_args* a) {
  PrefillPlan P;
  return plan_prefill(a, P, nullptr, false) == BSA_OK ? P.bytes : 0;
}

BSA_API bsa_status bsa_sparse_attn_prefill(const bsa_prefill_args* a, void* ws, size_t ws_bytes, void* stream) {
  return run_prefill(a, ws, ws_bytes, stream, false);
}

BSA_API bsa_status bsa_select_blocks(const bsa_prefill_args* a, void* ws, size_t ws_bytes, void* stream) {
  return run_prefill(a, ws, ws_bytes, stream, true);
}

BSA_API size_t bsa_decode_workspace_bytes(const bsa_decode_args* a) {
  DecodePlan P;
  return plan_decode(a, P, nullptr) == BSA_OK ? P.bytes : 0;
}

BSA_API bsa_status bsa_sparse_attn_decode(const bsa_decode_args* a, void* ws, size_t ws_bytes, void* stream) {
  return run_decode(a, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// decode without allocation: the workspace is a file-scope device array
// ---------------------------------------------------------------------------
// Every GPU the library runs on holds its own copy of `scratch` from module
// load until the process ends.  In host code the array's name is only a
// stand-in for the device symbol: its device address, which differs per GPU,
// comes from hipGetSymbolAddress on the first call on each device and is the
// only form ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[BSA_DECODE_NOALLOC_MAX_BYTES];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static bsa_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(BSA_ERR_HIP, "hipGetDevice failed");
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(BSA_ERR_UNSUPPORTED, "device index above the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(BSA_ERR_HIP, std::string("hipGetSymbolAddress of the decode scratch failed: ") + hipGetErrorString(e));
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BSA_OK;
}

BSA_API bsa_status bsa_sparse_attn_decode_noalloc(const bsa_decode_args* a, void* stream) {
  DecodePlan P;
  const bsa_status st = plan_decode(a, P, nullptr);
  if (st != BSA_OK) return st;
  if (P.bytes > (size_t)BSA_DECODE_NOALLOC_MAX_BYTES)
    return fail(BSA_ERR_WORKSPACE, "decode needs " + std::to_string(P.bytes) +
                                       " bytes of workspace, above the no-allocation limit of " +
                                       std::to_string((size_t)BSA_DECODE_NOALLOC_MAX_BYTES) +
                                       " (BSA_DECODE_NOALLOC_MAX_BYTES): call bsa_sparse_attn_decode with a workspace");
  void* ws = nullptr;
  const bsa_status sst = scratch_of_current_device(&ws);
  if (sst != BSA_OK) return sst;
  return run_decode(a, ws, (size_t)BSA_DECODE_NOALLOC_MAX_BYTES, stream, true);
}

BSA_API size_t bsa_backward_workspace_bytes(const bsa_backward_args* a) {
  BackwardPlan P;
  return plan_backward(a, P, nullptr) == BSA_OK ? P.bytes : 0;
}

BSA_API bsa_status bsa_sparse_attn_backward(const bsa_backward_args* a, void* ws, size_t ws_bytes, void* stream) {
  return run_backward(a, ws, ws_bytes, stream);
}

BSA_API size_t bsa_summary_workspace_bytes(const bsa_summary_args* a) {
  int32_t *c, *p;
  size_t n = 0;
  return plan_summary(a, &c, &p, nullptr, &n) == BSA_OK ? n : 0;
}

BSA_API bsa_status bsa_block_summary(const bsa_summary_args* a, void* ws, size_t ws_bytes, void* stream) {
  return run_summary(a, ws, ws_bytes, stream);
}

BSA_API const char* bsa_last_error(void) { return g_err.c_str(); }

BSA_API int32_t bsa_version(void) { return 200; }  // 0.2.0

#ifndef BSA_BUILD_DIGEST
#define BSA_BUILD_DIGEST "unknown"
#endif
BSA_API const char* bsa_build_digest(void) { return BSA_BUILD_DIGEST; }

BSA_API void bsa_timer_enable(int32_t level) { g_timer_level = level < 0 ? 0 : level; }

BSA_API void bsa_timer_reset(void) { timer_clear(); }

BSA_API bsa_status bsa_timer_report(const char* kernel, double* total_ms, int64_t* launches) {
  if (!kernel || !total_ms || !launches) return fail(BSA_ERR_INVALID_ARG, "null argument");
  double tot = 0.0;
  int64_t n = 0;
  for (auto& r : g_timer) {
    if (r.name != kernel) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return fail(BSA_ERR_HIP, "event synchronize failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return fail(BSA_ERR_HIP, "event elapsed failed");
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return BSA_OK;
}
