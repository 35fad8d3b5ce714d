/*
 * bsa.h -- C ABI of libbsa, block-sparse attention for AMD MI355X (gfx950).
 *
 * The method (what the calls compute):
 *   - Every query (per query head), or every GQA group, scores per-block key
 *     summaries and keeps the top-k KV blocks; exact softmax attention then
 *     runs over only the kept blocks.  MoBA repo card
 *     (ross.abutalabs.com/products/moba.json), card.what_it_is: MoE-style
 *     top-k gating over KV blocks, switchable to full attention; "MiniMax
 *     released MSA ..." (news.hamidun.com), section "How MSA Works": an index
 *     branch picks the top-k blocks per query and GQA group, a main branch
 *     attends exactly over them.
 *   - Block summaries are routing keys kept in GPU memory ("100 Millionen
 *     Token: Gedaechtnis oder Trugbild?", aitalk.it, section "Das Gehirn mit
 *     zwei Geschwindigkeiten"); this library forms them as the mean of the
 *     block's keys.  The same section gives document-wise RoPE: positions
 *     restart at 0 at each document start.
 *   Readings where the pages are silent (causal masking, the forced own
 *   block, the tie rule, the RoPE form) are stated at each call below.
 *
 * Conventions for every call:
 *   - Every pointer in an args struct is DEVICE memory unless marked HOST,
 *     or pinned host memory mapped into the device's address space at the
 *     same address (hipHostMalloc, a pinned tensor), which the kernels then
 *     read over the host link.  This is the host content tier: a memory's
 *     keys and values (prefill k / v, decode kcache / vcache) stay in host
 *     RAM and only the chosen blocks cross the link, while the routing keys
 *     (pooled) stay in GPU memory ("100 Millionen Token ...", section "Das
 *     Gehirn mit zwei Geschwindigkeiten").  Other memory (pageable host
 *     memory) fails validation with BSA_ERR_INVALID_ARG before anything is
 *     enqueued.
 *     The caller owns all buffers, including the workspace; the library never
 *     allocates or frees device memory and keeps no state across calls other
 *     than the last error message and the optional launch timer.
 *   - Tensors are addressed by element strides for their outer dimensions;
 *     the innermost (head) dimension is contiguous and each row starts on a
 *     16-byte boundary.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream).  Inputs must stay valid until the stream reaches the
 *     call's end.  No host synchronisation happens inside a call.
 *   - Arguments are validated before anything is enqueued: a call that
 *     returns an error has enqueued nothing (BSA_ERR_HIP excepted, which
 *     reports a failed launch).  No C++ exception crosses the ABI.
 *   - Results are bitwise deterministic for identical inputs and shapes.
 *   - NaN or Inf inputs give undefined results.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t bsa_status;
#define BSA_OK 0
#define BSA_ERR_INVALID_ARG 1 /* a null required pointer, a bad size or stride */
#define BSA_ERR_UNSUPPORTED 2 /* a valid request outside what the kernels handle */
#define BSA_ERR_WORKSPACE 3   /* workspace missing, too small or misaligned */
#define BSA_ERR_HIP 4         /* the HIP runtime rejected a launch */

#define BSA_DTYPE_F32 0
#define BSA_DTYPE_BF16 1

#define BSA_GATE_PER_HEAD 0  /* one selection per query head (MoBA card) */
#define BSA_GATE_PER_GROUP 1 /* one per GQA group, head scores summed (MiniMax page) */

#define BSA_MAX_TOPK 64

/*
 * Prefill.  q [B, Lq, Hq, D], k and v [B, Lk, Hkv, D], Hq a multiple of Hkv
 * (G = Hq / Hkv query heads share a KV head); D is 64 or 128.
 *
 * Block j holds key tokens [j*block, min((j+1)*block, Lk)); Nb = ceil(Lk/block).
 * Causal mode: query i sits at key position p = Lk - Lq + i; its own block
 * cur = p / block is always attended with keys <= p and is not counted in
 * topk; only blocks j < cur compete.  Non-causal: every block competes and
 * nothing is forced.  The gate keeps min(topk, #candidates) blocks by score,
 * breaking ties toward the lower block index; topk >= #candidates attends
 * every candidate (full attention).
 *
 * Gate score of block j: (gate query) . (summary of block j), where the
 * summary is the mean of block j's keys (index_k's when given, else k's,
 * after RoPE when doc_ids_k is given) and the gate query is the query head's
 * vector (index_q's when given, else q's after RoPE), or for
 * BSA_GATE_PER_GROUP the sum of the group's G head vectors.
 *
 * Output o[b, i, h] = sum_u softmax_u(scale * q.k_u) v_u over the union of
 * the selected blocks' keys (one softmax over all of them); an empty key set
 * gives o = 0 and lse = -inf.
 */
typedef struct bsa_prefill_args {
    int32_t dtype;                 /* BSA_DTYPE_*: element type of q, k, v, o, index_q, index_k */
    int32_t B, Lq, Lk, Hq, Hkv, D; /* Lq <= Lk when causal */
    const void* q;  int64_t q_stride[3];   /* (b, t, h) element strides */
    const void* k;  int64_t k_stride[3];
    const void* v;  int64_t v_stride[3];
    void* o;        int64_t o_stride[3];   /* output, same element type as q */
    int32_t block;                 /* tokens per KV block, >= 1 */
    int32_t topk;                  /* 0 <= topk <= BSA_MAX_TOPK (clamped to Nb) */
    int32_t causal;                /* 0 or 1 */
    int32_t gate_mode;             /* BSA_GATE_* */
    const void* index_q; int64_t iq_stride[3]; /* optional [B, Lq, Hq, Di]; both or neither with index_k */
    const void* index_k; int64_t ik_stride[3]; /* optional [B, Lk, Hkv, Di] */
    int32_t Di;                    /* index dimension (64 or 128) when index tensors are given */
    const int32_t* doc_ids_q;      /* optional [B, Lq] contiguous: rotate q by document-wise RoPE */
    const int32_t* doc_ids_k;      /* optional [B, Lk] contiguous: rotate k by document-wise RoPE */
    float rope_theta;              /* RoPE base; <= 0 means 10000 (pairs (i, i+D/2)) */
    float scale;                   /* softmax scale; 0 means 1/sqrt(D) */
    const float* pooled;           /* optional precomputed summaries [B, Nb, Hkv, Dg] fp32
                                      contiguous, 16-byte aligned; when given the summary step
                                      is skipped and the gate reads them as they are */
    int32_t* sel_out;              /* optional [B, Hs, Lq, topk + causal] int32, Hs = Hq (per head)
                                      or Hkv (per group): chosen blocks ascending, the forced
                                      block last when causal, -1 padded */
    float* lse_out;                /* optional [B, Hq, Lq] natural-log softmax normaliser */
    int32_t chunk_tokens;          /* scheduling only, results do not depend on it: query tokens
                                      of one (b, kv head) per chunk (the attention works through
                                      its blocks chunk by chunk); 0 lets the library pick (about
                                      64 MiB of queries per chunk), > 0 forces that many */
    int32_t chunks_per_pass;       /* scheduling only: chunks per attention pass (one gather and
                                      one merge launch); 0 = as many as a 40 GiB partial-output
                                      budget holds, > 0 forces that many (the last pass may hold
                                      fewer) */
    /* optional, bf16 prefill only, instead of `pooled`: the summaries as the
       gate's two bf16 planes, each [B, Hkv, Nb, Dg] contiguous and 16-byte
       aligned, with hi = bf16(s) and lo = bf16(s - hi) (round to nearest even)
       for the fp32 summary s -- the planes bsa_block_summary writes.  Both or
       neither; the gate stages them as they are, so a memory queried many
       times is split once, when it is encoded.  Results equal those with
       `pooled` = s. */
    const uint16_t* pooled_hi;
    const uint16_t* pooled_lo;
} bsa_prefill_args;

/* Workspace bytes bsa_sparse_attn_prefill needs for `a` (0 if `a` is invalid;
 * bsa_last_error() then says why).  The workspace must be 256-byte aligned. */
size_t bsa_prefill_workspace_bytes(const bsa_prefill_args* a);

/* Runs the whole prefill: [positions + RoPE] -> block summaries -> gate and
 * top-k -> selection inversion -> gathered attention -> combine.
 * Errors: BSA_ERR_INVALID_ARG / BSA_ERR_UNSUPPORTED for bad or unsupported
 * arguments (among the latter, 2^31 or more query rows -- B * Hq times Lq
 * rounded up to whole query chunks -- or 2^30 or more (query chunk, block)
 * buckets), BSA_ERR_WORKSPACE if ws_bytes is below the query's answer,
 * BSA_ERR_HIP if a launch fails. */
bsa_status bsa_sparse_attn_prefill(const bsa_prefill_args* a, void* workspace, size_t ws_bytes, void* stream);

/* Gate and top-k only (writes a->sel_out, which is then required; o and v
 * are not touched and may be NULL).  Same workspace query as prefill. */
bsa_status bsa_select_blocks(const bsa_prefill_args* a, void* workspace, size_t ws_bytes, void* stream);

/*
 * Decode: one new token per sequence.  q [B, Hq, D]; kcache, vcache
 * [B, Lc, Hkv, D]; pooled [B, Nb, Hkv, D] block summaries of the cache
 * (Nb = ceil(Lc / block)), as produced by bsa_block_summary or any other
 * source: routing keys kept in GPU memory ("100 Millionen Token ...",
 * section "Das Gehirn mit zwei Geschwindigkeiten").  Sequence b holds
 * n_b = cache_lens[b] tokens (Lc when cache_lens is NULL; values are clamped
 * to [1, Lc]); the new token is already cached at position n_b - 1, so its
 * block cur = (n_b - 1) / block is forced (keys up to n_b - 1) and blocks
 * 0..cur-1 compete for topk slots, ties to the lower index.
 *
 * Paged caches (block_table != NULL): kcache and vcache hold num_pages pages
 * of `block` tokens each, strides (page, token in page, head); block j of
 * sequence b (tokens j*block .. j*block + block - 1) is page
 * block_table[b * table_w + j].  table_w >= Nb; pages may be shared or in
 * any order, and only the pages of chosen blocks are read.  An entry outside
 * [0, num_pages) reads nothing and leaves that sequence's output undefined.
 * Lc is then the logical capacity (Nb = ceil(Lc / block) routing keys); the
 * gate and the cache lengths work on logical blocks exactly as above.
 */
typedef struct bsa_decode_args {
    int32_t dtype;                 /* BSA_DTYPE_BF16 (q, caches, o) */
    int32_t B, Lc, Hq, Hkv, D;
    const void* q;      int64_t q_stride[2];   /* (b, h) */
    const void* kcache; int64_t k_stride[3];   /* (b, t, h) */
    const void* vcache; int64_t v_stride[3];
    const void* pooled; int64_t p_stride[3];   /* (b, j, h) */
    int32_t pooled_dtype;          /* BSA_DTYPE_BF16 or BSA_DTYPE_F32 */
    const int32_t* cache_lens;     /* optional [B] */
    int32_t block, topk, gate_mode;
    float scale;                   /* 0 means 1/sqrt(D) */
    void* o;            int64_t o_stride[2];   /* [B, Hq, D] output */
    int32_t* sel_out;              /* optional [B, Hs, topk + 1]: chosen ascending, forced last, -1 padded */
    float* lse_out;                /* optional [B, Hq] */
    const int32_t* block_table;    /* optional [B, table_w] page of each logical block (device) */
    int32_t table_w, num_pages;    /* used only with block_table */
} bsa_decode_args;

size_t bsa_decode_workspace_bytes(const bsa_decode_args* a);
bsa_status bsa_sparse_attn_decode(const bsa_decode_args* a, void* workspace, size_t ws_bytes, void* stream);

/*
 * Decode without allocation, for callers that cannot allocate device memory
 * around the call: code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation.  Same arguments, kernels and results as
 * bsa_sparse_attn_decode, but no workspace argument: the workspace is a
 * library-owned device array of BSA_DECODE_NOALLOC_MAX_BYTES bytes, one per
 * GPU, held from library load until the process ends.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); its first
 * call on a device looks up that device's array (the device current on the
 * calling thread, which must be the device of `stream` and of the tensors).
 * Errors: as bsa_sparse_attn_decode, plus BSA_ERR_WORKSPACE when
 * bsa_decode_workspace_bytes(a) exceeds BSA_DECODE_NOALLOC_MAX_BYTES (the
 * 16 x 1,048,576-token, 32/8-head, block-128, top-32 decode needs about
 * 52 MB).  Every call on one GPU shares that GPU's array: calls whose
 * execution overlaps on one GPU (two streams, two threads) race and give
 * undefined results; calls serialised on one stream are safe.  No part of
 * the array needs to start zeroed.
 */
#define BSA_DECODE_NOALLOC_MAX_BYTES ((size_t)64 << 20)
bsa_status bsa_sparse_attn_decode_noalloc(const bsa_decode_args* a, void* stream);

/*
 * Block summaries (the offline encoding of a memory): pooled[b, j, h, :] =
 * mean of the keys of block j (a short last block averages the tokens it
 * has), after document-wise RoPE when doc_ids is given.  Positions restart
 * at 0 at every change of doc id ("100 Millionen Token ...", section "Das
 * Gehirn mit zwei Geschwindigkeiten"); the rotation pairs (i, i + D/2) with
 * angle pos * theta^(-2i/D), formed in double precision.  Sums are fp32.
 */
typedef struct bsa_summary_args {
    int32_t dtype;                 /* element type of k (and k_rot) */
    int32_t B, L, H, D, block;
    const void* k; int64_t k_stride[3];        /* (b, t, h) */
    const int32_t* doc_ids;        /* optional [B, L] contiguous */
    float rope_theta;              /* <= 0 means 10000 */
    void* pooled;                  /* [B, Nb, H, D] contiguous output */
    int32_t pooled_dtype;          /* BSA_DTYPE_F32 or BSA_DTYPE_BF16 (round to nearest even) */
    void* k_rot;                   /* optional [B, L, H, D] contiguous rotated keys (k's dtype);
                                      needs doc_ids */
    int32_t* pos_out;              /* optional [B, L] per-document positions; needs doc_ids */
    /* optional [B, H, Nb, D] contiguous outputs (both or neither): the fp32
       summaries split into the prefill gate's bf16 planes, hi = bf16(s),
       lo = bf16(s - hi) (bsa_prefill_args pooled_hi / pooled_lo) */
    uint16_t* plane_hi;
    uint16_t* plane_lo;
} bsa_summary_args;

size_t bsa_summary_workspace_bytes(const bsa_summary_args* a);
bsa_status bsa_block_summary(const bsa_summary_args* a, void* workspace, size_t ws_bytes, void* stream);

/*
 * Backward of the prefill's attention through its block selection: the
 * method is trained end to end (MoBA card, card.what_it_is; "MSA: Memory
 * Sparse Attention", "Key Points"), and a top-k choice has no gradient, so
 * with the selection held fixed the gradient is that of exact softmax
 * attention over the chosen keys.  For query row (b, t, h) with weights p_u
 * over the keys it attended (own block masked after the query when causal,
 * query t at absolute position Lk - Lq + t) and g = dL/do:
 *   dv_u += p_u g,  ds_u = p_u (g . v_u - g . o),
 *   dq = scale * sum_u ds_u k_u,  dk_u += scale * ds_u q.
 * q and k are the attended tensors (after RoPE when the forward applied it;
 * the rotation's own backward is the caller's).  o, lse and sel are the
 * forward call's outputs (sel entries -1 or in [0, Nb); entries outside that
 * range are skipped).  bf16 inputs, fp32 outputs; the five products run on
 * bf16 MFMA with fp32 accumulation (p and ds rounded to bf16 as operands),
 * the softmax terms in fp32.  Outputs are bitwise deterministic: the rows
 * that chose a block are summed in a fixed order (query chunk, then the
 * sorted selection entries), a row's slots in slot order.
 */
typedef struct bsa_backward_args {
    int32_t dtype;                 /* BSA_DTYPE_BF16 */
    int32_t B, Lq, Lk, Hq, Hkv, D; /* D 64 or 128 */
    const void* q;    int64_t q_stride[3];   /* (b, t, h) element strides, as in prefill */
    const void* k;    int64_t k_stride[3];
    const void* v;    int64_t v_stride[3];
    const void* o;    int64_t o_stride[3];   /* the forward's output */
    const void* dout; int64_t do_stride[3];  /* dL/do, same shape as o */
    const float* lse;              /* [B, Hq, Lq] the forward's lse_out (natural log) */
    const int32_t* sel;            /* [B, Hs, Lq, sel_w] the forward's sel_out */
    int32_t sel_w;                 /* the forward's topk + causal */
    int32_t block, causal, gate_mode;
    float scale;                   /* 0 means 1/sqrt(D) */
    float* dq;                     /* [B, Lq, Hq, D] contiguous fp32 */
    float* dk;                     /* [B, Lk, Hkv, D] contiguous fp32 */
    float* dv;                     /* [B, Lk, Hkv, D] contiguous fp32 */
} bsa_backward_args;

size_t bsa_backward_workspace_bytes(const bsa_backward_args* a);
bsa_status bsa_sparse_attn_backward(const bsa_backward_args* a, void* workspace, size_t ws_bytes, void* stream);

/* Message for the last non-OK status returned on the calling thread. */
const char* bsa_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
int32_t bsa_version(void);
/* Digest of the sources the library was built from (16 hex digits, a static
 * string): the build hashes every file of the kernel sources and this header,
 * so a caller can tell a library that no longer matches its sources. */
const char* bsa_build_digest(void);

/*
 * Optional launch timer (off by default; host-side state, not thread-safe).
 * Level 1: every kernel launch is bracketed by HIP events recorded on the
 * launch stream, except inside the prefill's attention passes, which are
 * bracketed as one phase named "attn" (gathers and merges of every pass, so
 * that hundreds of short launches are not each charged the events' cost).
 * Level 2: every launch, the attention passes' "attn_gather" / "attn_merge"
 * launches included (and "attn" as well).  0 turns it off.
 * bsa_timer_report synchronises on the events and returns, for the kernel or
 * phase named `kernel` (HOST string), the summed duration in milliseconds and
 * the launch count since the last reset.
 */
void bsa_timer_enable(int32_t level);
void bsa_timer_reset(void);
bsa_status bsa_timer_report(const char* kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* BSA_H */
