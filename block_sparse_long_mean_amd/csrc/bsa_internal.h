// Host-side interfaces between the C ABI layer and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace bsa {

// ---- launch bookkeeping (timer + error capture), defined in api.hip -------
struct LaunchScope {
  // level: the timer level from which this scope records (1 = every level)
  LaunchScope(const char* name, hipStream_t s, int level = 1);
  ~LaunchScope();
  const char* name;
  hipStream_t stream;
  int slot;
};
bool launch_ok(const char* name);  // checks hipGetLastError, records the message

// ---- positions ----------------------------------------------------------
constexpr int kPosChunk = 4096;
inline int pos_chunks(int L) { return (L + kPosChunk - 1) / kPosChunk; }
bool launch_doc_positions(const int32_t* doc, int B, int L, int32_t* chunk_last, int32_t* pos,
                          hipStream_t s);

// ---- block summary --------------------------------------------------------
struct SummaryParams {
  int is_bf16;
  int B, L, H, D, block, Nb;
  const void* k;
  int64_t ks_b, ks_t, ks_h;
  const int32_t* pos;  // per-document positions [B, L] or null (no RoPE)
  double omega[64];    // RoPE frequencies theta^(-2i/D)
  float* pooled_f32;   // public layout [B, Nb, H, D] or null
  uint16_t* pooled_bf16;  // public layout or null
  uint16_t* plane_hi;  // gate layout [B, H, Nb, D] hi/lo split, or null
  uint16_t* plane_lo;
  void* k_rot;         // [B, L, H, D] contiguous rotated keys or null
};
bool launch_block_summary(const SummaryParams& p, hipStream_t s);

struct RopeQParams {
  int is_bf16;
  int B, L, H, D;
  const void* q;
  int64_t qs_b, qs_t, qs_h;
  const int32_t* pos;
  double omega[64];
  uint16_t* out16;  // [B, L, H, D] bf16 or null
  float* out32;     // [B, L, H, D] f32 or null
};
bool launch_rope_q(const RopeQParams& p, hipStream_t s);

// fp32 or bf16 [B, Nb, H, D] (strided) -> hi/lo planes [B, H, Nb, D]
bool launch_pooled_to_planes(const void* pooled, int is_bf16, int64_t ps_b, int64_t ps_j, int64_t ps_h,
                             int B, int Nb, int H, int D, uint16_t* hi, uint16_t* lo, hipStream_t s);

// ---- gate + top-k --------------------------------------------------------
struct GateParams {
  int B, Lq, Lk, Hkv, G, Hs, per_group;
  int rows_per_bh;  // selection rows per (b, kv head)
  int ntiles;       // row tiles per (b, kv head)
  const void* q;    // gate query source
  int64_t qs_b, qs_t, qs_h;
  int qkind;        // 0 bf16 (exact), 1 f32 (split), 2 bf16 summed over the group (split)
  int Dg;
  const uint16_t* p_hi;
  const uint16_t* p_lo;  // may be null (summaries exact in bf16)
  const float* p_f32;    // or fp32 summaries, split into hi / lo while staged (then p_hi, p_lo unused)
  int64_t ps_b, ps_h, ps_j;
  int Nb;
  int causal, block;
  const int32_t* lens;  // decode: per-sequence cache lengths or null
  int topk, nsplit, span;
  int32_t* sel;
  int sel_w;
  uint64_t* part;  // [rows][nsplit][topk] when nsplit > 1
  const char* tag;  // launch name prefix for the timer ("gate" or "decode_gate")
};
bool launch_gate(const GateParams& p, hipStream_t s);
bool launch_gate_merge(const GateParams& p, hipStream_t s);

// fp32 path: gate scored in fp32 against fp32 summaries [B, Nb, Hkv, Dg]
struct GateF32Params {
  int B, Lq, Lk, Hkv, G, Hs, per_group, Dg;
  const float* q;
  int64_t qs_b, qs_t, qs_h;
  const float* pooled;  // [B, Nb, Hkv, Dg] contiguous
  int Nb, causal, block, topk;
  int32_t* sel;
  int sel_w;
};
bool launch_gate_f32(const GateF32Params& p, hipStream_t s);

// ---- selection inversion (CSR) --------------------------------------------
// Query tokens of one (b, kv head) are attended in chunks of CT tokens (NC
// chunks; chunk id = (b * Hkv + hk) * NC + c).  Buckets are per (chunk id,
// block): bucket = chunk id * Nb + j, so a chunk's work items are contiguous.
struct CsrParams {
  int B, Lq, Lk, Hkv, G, Hs, per_group, Nb, block, causal;
  int Gs;         // selection rows per (b, kv head, token): G per head, 1 per group
  int NC, CT;     // chunks per (b, kv head) and tokens per chunk
  const int32_t* sel;
  int sel_w;
  int kslot;      // partial slots per selection row
  int sh_h, sh_t; // entry bit fields: slot | head << sh_h | token << sh_t
  int R;          // attention rows per entry (G per group, else 1)
  int rows_item;  // attention rows per work item
  int32_t* counts;      // [nbk]
  int32_t* cursor;      // [nbk]
  int32_t* bucket_off;  // [nbk + 1]
  int32_t* tile_off;    // [nbk + 1]
  int32_t* scan_tmp;    // [scan_tmp_len]
  uint32_t* entries;
  int4* items;
  int nbk;
};
int64_t scan_tmp_len(int64_t n);
bool launch_csr(const CsrParams& p, hipStream_t s);

// ---- attention ------------------------------------------------------------
struct AttnParams {
  int B, Lq, Lk, Hq, Hkv, G, D, block, Nb, Hs, per_group, Gs, R, kslot, causal;
  int sh_h, sh_t, lgR;  // entry bit fields; R = 1 << lgR
  int topk;             // gate-chosen blocks per row before the candidate count caps it: min(topk, Nb)
  const uint16_t* q;
  int64_t qs_b, qs_t, qs_h;
  const uint16_t* k;
  int64_t ks_b, ks_t, ks_h;
  const uint16_t* v;
  int64_t vs_b, vs_t, vs_h;
  float sl2;  // softmax scale * log2(e)
  const uint32_t* entries;
  const int32_t* bucket_off;
  const int32_t* tile_off;
  const int4* items;  // {bucket, first entry, rows, b << 16 | kv head}
  int NC, CT;              // query chunks per (b, kv head), tokens per chunk
  int c0, c1;              // chunk ids of this launch; its partial buffer holds c1 - c0 chunks
  int grid;                // persistent workgroups
  int rows_item;           // rows per work item: 32 per wave of a gather workgroup
  int run_items;           // consecutive items a gather workgroup takes at a time
  int64_t sparse_items;    // > 0: sparse-bucket gather, one workgroup per item (grid = this bound)
  // partials of the launch's chunks, row ((c - c0) * Gs + head-sel) * CT + token-in-chunk
  uint16_t* part_o;        // [rows * kslot * R, D] int16: 32767 * 2^-E * sum_k p_k v_k, p = 2^(s*sl2 - m)
  float2* part_ml;         // (m + E, 2^-E * l): log2-domain running max and sum of p, row exponent E folded in
  // combine
  const int32_t* sel;
  int sel_w;
  uint16_t* o;
  int64_t os_b, os_t, os_h;
  float* lse_out;  // natural log, [B, Hq, Lq] or null
  // backward through the fixed selection (buckets' entries sorted)
  const uint16_t* dout;
  int64_t dos_b, dos_t, dos_h;
  const float* lse_in;      // [B, Hq, Lq] natural log
  float* delta;             // [B, Hq, Lq]: dout . o per row
  float* dq_part;           // [rows * kslot * R, D]: sum over the slot's keys of ds * k
  const int32_t* counts;    // entries per bucket
  float* dq;                // [B, Lq, Hq, D]
  float* dk;                // [B, Lk, Hkv, D]
  float* dv;
  float scale;
};
int gather_waves(int block);  // waves per gather workgroup for this block size
bool launch_attn_gather(const AttnParams& p, hipStream_t s);
bool launch_attn_merge(const AttnParams& p, hipStream_t s);
// backward: delta, per-bucket entry sort, dk / dv per key, dq partials per
// (row, slot), the ordered dq reduction
constexpr int kBwdSortCap = 8192;  // entries per bucket the LDS sort holds
constexpr int kBwdKeyWaves = 4;    // dk / dv workgroups: 32 keys per wave
constexpr int kBwdItemRows = 256;  // dq work items: 32 rows per wave of 8
bool launch_attn_backward(const AttnParams& p, int64_t nrows_out, hipStream_t s);

struct AttnF32Params {
  int B, Lq, Lk, Hq, Hkv, G, D, block, Hs, per_group, causal;
  const float* q;
  int64_t qs_b, qs_t, qs_h;
  const float* k;
  int64_t ks_b, ks_t, ks_h;
  const float* v;
  int64_t vs_b, vs_t, vs_h;
  float scale;
  const int32_t* sel;
  int sel_w;
  float* o;
  int64_t os_b, os_t, os_h;
  float* lse_out;
};
bool launch_attn_rowwise_f32(const AttnF32Params& p, hipStream_t s);

// ---- decode ---------------------------------------------------------------
struct DecodeAttnParams {
  int B, Lc, Hq, Hkv, G, D, block, Hs, per_group, topk, umax;
  const int32_t* lens;
  const int32_t* table;  // paged caches: [B, table_w] page per logical block, or null
  int table_w, num_pages;
  const uint16_t* q;
  int64_t qs_b, qs_h;
  const uint16_t* k;
  int64_t ks_b, ks_t, ks_h;  // with a table, ks_b is the page stride
  const uint16_t* v;
  int64_t vs_b, vs_t, vs_h;
  float sl2;
  const int32_t* sel;  // [B, Hs, topk + 1]
  int32_t* ulist;      // [B * Hkv, umax] packed (j << 8 | head mask)
  int32_t* ucount;     // [B * Hkv]
  float* part_o;       // [B * Hkv * umax * G, D]
  float* part_lse;
  uint16_t* o;
  int64_t os_b, os_h;
  float* lse_out;
};
struct DecodeGateParams {
  int B, Lc, Hq, Hkv, G, D, block, Nb, Hs, per_group, topk, sel_w;
  const int32_t* lens;
  const uint16_t* q;
  int64_t qs_b, qs_h;
  const void* pooled;  // [B, Nb, Hkv, D] summaries, bf16 or fp32
  int pooled_bf16;
  int64_t ps_b, ps_j, ps_h;
  int nshare;          // candidate shares of kDecShare blocks (over the longest sequence)
  uint64_t* skeys;     // [B, Hs, nshare, topk] each share's best keys, descending (workspace)
  int32_t* scnt;       // [B, Hs, nshare] their counts
  int32_t* sel;   // [B, Hs, sel_w]
  int32_t* ulist;  // [B * Hkv, umax] union of a (b, kv head)'s rows (j << 8 | head mask)
  int32_t* ucount; // [B * Hkv]
  int umax;
};
constexpr int kDecShare = 2048;  // decode gate: candidate blocks per pass-1 workgroup
bool launch_decode_gate(const DecodeGateParams& p, hipStream_t s);
bool launch_decode_attend(const DecodeAttnParams& p, hipStream_t s);
bool launch_decode_attend_mfma(const DecodeAttnParams& p, hipStream_t s);  // attn.hip
bool launch_decode_combine(const DecodeAttnParams& p, hipStream_t s);

void set_error(const std::string& msg);

}  // namespace bsa
