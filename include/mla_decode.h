/*
 * mla_decode.h - C ABI of the MI355X (gfx950) MLA / MLRA-4 latent-KV decode library.
 *
 * One decode step (one new token per sequence, or a few: num_queries) of Multi-head Latent
 * Attention over a
 * cache that holds, per token, only the compressed joint latent c_KV and a decoupled
 * rotary key ("超越 GQA 的推理革命…MLA…", sections 鍵值聯合低秩壓縮 and 解耦旋轉位置編碼).
 * The step is computed with matrix absorption (same page, section 矩陣吸收): W_UK is folded
 * into the query, scores are q_lat . c_KV + q_rope . k_rope, the softmax-weighted sum is
 * taken over the latent itself, and W_UV is applied once afterwards.  Mathematically this
 * equals the un-absorbed form (up-project the latent to per-head K and V, then attend;
 * "MLA (Multi-head Latent Attention) 是什么", section 核心机制 step 3).  MLRA-4 splits the
 * latent into four independent branches that attend separately and are summed with a
 * scale ("[ICLR 2025] MLRA…", sections 2.1 and 2.2).
 *
 * Conventions for every entry point
 *  - Pointers named as device pointers must be device memory of the current HIP device;
 *    host pointers are read only during the call.
 *  - The caller owns every buffer, including out and workspace.  The library never
 *    allocates or frees memory and never synchronises the stream; calls are asynchronous
 *    on `stream` (a hipStream_t; NULL = the default stream) and may be made concurrently from
 *    several host threads (mla_decode_noalloc: see its note on overlapping calls).
 *  - Arguments are validated on the host before anything is launched; a failed check
 *    returns a non-zero mla_status and launches nothing.  Values that live in device memory
 *    (seqlens, block_table entries) are not validated by default: seqlens[b] must lie in
 *    [0, max_seqlen] and every block_table entry for a page a sequence uses must index an
 *    existing page; otherwise the behaviour is undefined.  With MLA_FLAG_DEVICE_CHECKS set in
 *    mla_params.flags the device checks both and records what it finds in the error word of
 *    the workspace (see "Split plan" below).
 *  - Device properties (the compute-unit count that sizes the split plan) are queried once
 *    per device and cached; with mla_decode_noalloc's static scratch array and its cached
 *    device address this is the only state the library keeps.
 *  - A kernel launch failure is reported as MLA_ERR_HIP.
 *  - No C++ exception crosses this interface.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP stream type, declared exactly as hip_runtime_api.h declares it (so this header
 * can be included with or without the HIP headers). */
typedef struct ihipStream_t* hipStream_t;

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,        /* a required pointer is NULL                               */
  MLA_ERR_SHAPE = 2,       /* a size, stride or bound is negative or inconsistent      */
  MLA_ERR_UNSUPPORTED = 3, /* valid request this build has no kernel for (dims, page)  */
  MLA_ERR_WORKSPACE = 4,   /* workspace_bytes smaller than mla_workspace_size()        */
  MLA_ERR_DTYPE = 5,       /* unknown dtype                                            */
  MLA_ERR_HIP = 6,         /* a HIP runtime call or kernel launch failed               */
  MLA_ERR_ALIGN = 7        /* pointer or stride not aligned as the dtype requires      */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

/* Page size of the paged latent cache, in tokens. */
#define MLA_PAGE_SIZE 64

/* mla_params.flags: check seqlens and the used block_table entries on the device and record
 * violations in the workspace's error word (costs one extra pass over the block table). */
#define MLA_FLAG_DEVICE_CHECKS 1

/* mla_params.flags: folded query.  W_UK has been folded offline into the query's own
 * projection (the yololab MLA page, section 矩陣吸收: the key up-projection is absorbed into
 * the query projection), so the q_nope argument holds the latent-space query
 * q_lat [B, H, NB * d_latent] (branch br's part at columns br*d_latent ..), scored directly
 * against c_KV: s_t = softmax_scale * (q_lat_br . c_{br,t} + q_r . k_t).  w_uk is not read
 * (may be NULL) and d_nope is not used (any value >= 1). */
#define MLA_FLAG_QUERY_LATENT 2

/* mla_params.flags: latent output.  W_UV is left to the output projection it can be folded
 * into (same section: the value up-projection moves past the attention), so out receives
 * out_scale * [o_0 | .. | o_{NB-1}] [B, H, NB * d_latent], o_br = sum_t softmax(s_br)_t c_{br,t},
 * the branch outputs side by side in latent space.  w_uv is not read (may be NULL) and d_v is
 * not used (any value >= 1).  Not available with a gate. */
#define MLA_FLAG_OUTPUT_LATENT 4

/* mla_params.latent_format: the latent part of the cache (not the rotary key) is stored as
 * OCP FP8 E4M3 codes ("e4m3fn": 4 exponent bits with bias 7, 3 mantissa bits, no infinity)
 * with one per-tensor scale, latent_scale; the element strides of the latent cache then count
 * bytes.  The rotary key, the queries, the weights and the output stay in dtype, which must
 * be MLA_BF16.  The kernels widen the codes to bf16 exactly (E4M3 fits in bf16) and fold the
 * scale into the absorbed query and the output scale; arithmetic is as for a bf16 cache.
 * (Quantised latent caches: the yunthe MLA page, section 一.) */
#define MLA_LATENT_FP8 1

/* Error-word bits (workspace int32 hdr[4], written by every call). */
#define MLA_DEVERR_SEQLEN 1   /* some seqlens[b] outside [0, max_seqlen]; clamped into it   */
#define MLA_DEVERR_BLOCK 2    /* some used block_table entry outside [0, num_pages)         */

typedef struct mla_params {
  int32_t batch;              /* B >= 1 sequences, one query token each                    */
  int32_t num_heads;          /* H query heads                                             */
  int32_t num_branches;       /* NB: 1 = MLA, 4 = MLRA-4                                   */
  int32_t d_nope;             /* per-head query/key content dim before absorption          */
  int32_t d_v;                /* per-head value / output dim                               */
  int32_t d_latent;           /* latent dim per branch d_cb; total latent d_c = NB * d_cb  */
  int32_t d_rope;             /* decoupled rotary key dim (even)                           */
  int32_t page_size;          /* 0 = contiguous cache, MLA_PAGE_SIZE = paged cache         */
  int32_t max_pages_per_seq;  /* paged: block_table columns in use, >= ceil(max_seqlen/64) */
  int32_t max_seqlen;         /* host-side bound on every seqlens[b]; sizes the workspace  */
  int32_t num_splits;         /* 0 = balanced split plan (below); n > 0 = at most n splits
                                 per sequence, each ceil(ceil(max_seqlen/64)/n) pages      */
  int32_t dtype;              /* mla_dtype of q, caches, weights and out                   */
  int32_t flags;              /* 0, or MLA_FLAG_DEVICE_CHECKS | MLA_FLAG_QUERY_LATENT |
                                 MLA_FLAG_OUTPUT_LATENT, in any combination                */
  int32_t num_pages;          /* paged: pages in the pool (bound for the device checks);
                                 0 = not given (block ids are then not checked)            */
  int32_t num_queries;        /* s_q new tokens per sequence decoded in this step (0 or 1:
                                 one); see "Several query tokens" below                    */
  int32_t latent_format;      /* 0: the latent cache holds dtype elements; MLA_LATENT_FP8:
                                 OCP FP8 E4M3 codes (see latent_scale)                     */
  int64_t latent_stride_tok;  /* elements between consecutive tokens of the latent cache   */
  int64_t latent_stride_seq;  /* contiguous: elements between sequences; paged: pages      */
  int64_t rope_stride_tok;    /* same two strides for the rotary-key cache                 */
  int64_t rope_stride_seq;
  int64_t block_table_stride; /* elements between rows of block_table (>= max_pages)      */
  float softmax_scale;        /* score scale, usually 1/sqrt(d_nope + d_rope)              */
  float out_scale;            /* scale on the (branch-summed) output: 1 MLA, 0.5 MLRA-4    */
  float rope_theta;           /* RoPE base, e.g. 10000                                     */
  float latent_scale;         /* MLA_LATENT_FP8: latent value = decoded code * latent_scale
                                 (finite, > 0); otherwise unused                           */
} mla_params;

/*
 * Supported shapes in this build (anything else returns MLA_ERR_UNSUPPORTED):
 *  - MLA_BF16, NB = 1: d_latent = 512 (MLA) or 128 (one MLRA branch on its own, a
 *    tensor-parallel shard of MLRA-4), d_rope = 64, d_nope = 128, d_v = 128, H % 32 == 0.
 *  - MLA_BF16, NB = 4: d_latent = 128, d_rope = 64, d_nope = 128, d_v = 128, H % 32 == 0.
 *  - MLA_F32 (generic SIMT path): NB in {1, 4}, NB*d_latent <= 512, d_rope even <= 64,
 *    d_nope <= 256, d_v <= 256, any H >= 1.
 *  - page_size in {0, 64}.
 * Alignment: bf16 latent, rope, q_nope, w_uk, w_uv, gate and out pointers 16-byte aligned
 * and the cache strides multiples of 8 elements; other pointers aligned to their element size.
 * num_splits is at most 512 and at most ceil(max_seqlen / 64).  flags holds only the
 * MLA_FLAG_* bits above; num_pages >= 0; 0 <= num_queries <= 16 (s_q * H must meet the
 * head rule, and every 32-head group must belong to one query token: H % 32 == 0 on bf16);
 * latent_format is 0 or MLA_LATENT_FP8 (bf16 only; latent pointer and strides then 16-byte
 * aligned in bytes).  With MLA_FLAG_QUERY_LATENT the d_nope rule does not
 * apply, with MLA_FLAG_OUTPUT_LATENT the d_v rule does not.
 *
 * Split plan.  The attention over each sequence is split into work items of whole 64-token
 * pages (split-K over the sequence) whose partial results are merged afterwards.  The plan is
 * made on the device from seqlens at the start of every call, so it follows the actual
 * lengths: with p_b = ceil(seqlens[b] / 64) pages, every sequence is cut into ceil(p_b / c)
 * items of c pages (the last one ragged; an empty sequence gets none), one item per dispatch
 * slot.  With num_splits = 0, c is the smallest page count for which the batch's items fit
 * the workgroups that fill the GPU once (one per compute unit for bf16 MLA whose query rows,
 * s_q * H, are a multiple of 128 with a bf16 latent; four per compute unit for d_latent = 128
 * with NB = 1; else two; divided by the workgroups per item, which is the query rows / 128 or
 * / 32 on bf16 and the query rows on fp32; the device's compute-unit count is queried once
 * per device, at most 256); when no c does, c = max_b p_b.  With num_splits = n, c = ceil(ceil(max_seqlen / 64) / n).
 * After a call has completed on its stream, the workspace starts with that plan (for
 * inspection; nothing reads it after the call):
 *   int32 hdr[8] at byte 0: { W = number of items, c, slots, item
 *         target (0 when forced), error bits (MLA_DEVERR_*; 0 without device checks), first
 *         sequence with an error (-1: none), its first bad block-table column (-1: none),
 *         items_cap }
 *   int32 work[slots][4] at byte 32: { b, t_begin, t_end, item } of the item of each
 *         dispatch slot of the main kernels, b = -1 for a slot without one
 *   int32 slot_end[slots] next: item + 1 for each slot with an item, else 0
 *   int32 items[items_cap][4] next: { b, t_begin, t_end, slot } of every item; items are
 *         numbered sequence-major, item i of sequence b covering tokens [t_begin, t_end)
 *   int32 split_off[B + 1] next: items of sequence b are split_off[b] .. split_off[b+1] - 1,
 *         split_off[B] = W.
 * With MLA_FLAG_DEVICE_CHECKS, a used block-table entry outside [0, num_pages) makes a plan
 * with no items (every output zero, nothing read from the pool); out-of-range seqlens are
 * clamped into [0, max_seqlen] as always and only reported.
 */

/*
 * Several query tokens (num_queries = s_q > 1): the step decodes s_q new tokens of every
 * sequence at once, all of them already in the cache (seqlens[b] = L counts them).  Token i
 * (0 .. s_q - 1) sits at position L - s_q + i, its rotary query is rotated there, and it
 * attends causally to the L_i = L - s_q + 1 + i tokens up to and including itself (a row
 * with L_i <= 0 is zero).  The query-side and output arrays gain a token axis before the
 * head axis: q_nope [B, s_q, H, NB, d_nope] (or [B, s_q, H, NB*d_latent] folded), q_rope
 * [B, s_q, H, d_rope], gate and out [B, s_q, H, ...]; the weights keep their H heads.  Every
 * (token, head) pair is one row of the split plan's work, so the workspace grows with s_q.
 * (The yololab MLA page, section 繁榮背後的代價: several query rows per cache read move the
 * step from memory-bound towards compute-bound.)
 */

/*
 * Bytes of device workspace mla_decode / mlra_decode need for *p (written to *bytes, a
 * host pointer).  Depends only on the fields of *p (sized for devices of up to 256 compute
 * units; needs no device).  The workspace holds the split plan, the
 * absorbed queries, the per-item partial results (running max, running sum and latent-space
 * output of each work item) and, for fp32, the merged latent-space output.
 */
mla_status mla_workspace_size(const mla_params* p, size_t* bytes);

/* Most work items (splits) one sequence can be cut into for *p (written to *splits, host), on
 * a device of up to 256 compute units: n when num_splits = n > 0, else
 * min(ceil(max_seqlen / 64), item target). */
mla_status mla_num_splits(const mla_params* p, int32_t* splits);

/*
 * MLA decode step (NB = 1), absorbed form.  Defined by the yololab MLA page (sections
 * 鍵值聯合低秩壓縮, 解耦旋轉位置編碼, 矩陣吸收) and the interview Q&A (核心机制 step 3).
 *
 * For each sequence b with L = seqlens[b] and each head h:
 *   q_lat  = W_UK[h]^T q_nope[b,h]                         (d_c)
 *   q_r    = RoPE(q_rope[b,h], position L-1)               (d_rope)
 *   s_t    = softmax_scale * (q_lat . c_t + q_r . k_t)      t = 0..L-1
 *   o_lat  = sum_t softmax(s)_t c_t                          (d_c)
 *   out[b,h] = out_scale * W_UV[h]^T o_lat                   (d_v)
 * where c_t is the latent row and k_t the cached rotary key of token t, the latter already
 * rotated at its own position t (see mla_rope_rotate).  L = 0 writes zeros.
 *
 * Arguments (device pointers unless noted; element type = p->dtype unless noted):
 *   q_nope      [B, H, NB, d_nope] contiguous ([B, H, NB*d_latent] with MLA_FLAG_QUERY_LATENT)
 *   q_rope      [B, H, d_rope] contiguous, NOT rotated (rotated here at position L-1)
 *   latent      contiguous: element (b, t, j) at latent[b*latent_stride_seq + t*latent_stride_tok + j]
 *               paged: element (b, t, j) at latent[pg*latent_stride_seq + (t%64)*latent_stride_tok + j]
 *               with pg = block_table[b*block_table_stride + t/64];  j < NB*d_latent
 *   rope        rotated keys, addressed like latent with the rope strides; j < d_rope
 *               (the usual fused row [c_KV | k_rope] is rope = latent + NB*d_latent)
 *   seqlens     int32 [B], 0 <= seqlens[b] <= max_seqlen
 *   block_table int32 [B, block_table_stride] when page_size = 64, else ignored (may be NULL)
 *   w_uk        [NB, H, d_nope, d_latent]   (K = w_uk[br,h] c); unused with MLA_FLAG_QUERY_LATENT
 *   w_uv        [NB, H, d_latent, d_v]      (V = w_uv[br,h]^T c); unused with MLA_FLAG_OUTPUT_LATENT
 *   out         [B, H, d_v] contiguous, written ([B, H, NB*d_latent] with MLA_FLAG_OUTPUT_LATENT)
 *   workspace   >= mla_workspace_size(p) bytes, 256-byte aligned, contents need no
 *               initialisation and are overwritten
 *   stream      hipStream_t
 * Returns MLA_ERR_UNSUPPORTED if p->num_branches != 1.
 */
mla_status mla_decode(const mla_params* p, const void* q_nope, const void* q_rope,
                      const void* latent, const void* rope, const int32_t* seqlens,
                      const int32_t* block_table, const void* w_uk, const void* w_uv, void* out,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * MLRA-4 decode step: the latent row is [c_0 | c_1 | c_2 | c_3] (4 x d_latent) and every
 * branch br attends on its own with its own W_UK[br], W_UV[br] and a shared rotary key
 * ("[ICLR 2025] MLRA…", section 2.1):
 *   s_{br,t} = softmax_scale * (q_lat_br . c_{br,t} + q_r . k_t)
 *   out[b,h] = out_scale * sum_br W_UV[br,h]^T (sum_t softmax(s_br)_t c_{br,t})
 * out_scale is the branch-sum calibration of section 2.2 (0.5 for four branches).
 * Same arguments and layouts as mla_decode; returns MLA_ERR_UNSUPPORTED unless
 * p->num_branches == 4.
 */
mla_status mlra_decode(const mla_params* p, const void* q_nope, const void* q_rope,
                       const void* latent, const void* rope, const int32_t* seqlens,
                       const int32_t* block_table, const void* w_uk, const void* w_uv, void* out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Gated output: mla_decode / mlra_decode whose result is multiplied elementwise by
 * sigmoid(gate), as gated attention does on MLRA-4 ("[ICLR 2025] MLRA…", section 4):
 *   out[b,h,v] = (out_scale * sum_br W_UV[br,h]^T o_br)[v] * 1 / (1 + exp(-gate[b,h,v]))
 *   gate  [B, H, d_v] contiguous, element type p->dtype, the gate logits (the projection that
 *         makes them is the model's); bf16: 16-byte aligned.
 * Other arguments, layouts and flags as mla_decode (gated) / mlra_decode (mlra_decode_gated).
 * Returns MLA_ERR_NULL for a NULL gate and MLA_ERR_UNSUPPORTED with MLA_FLAG_OUTPUT_LATENT.
 */
mla_status mla_decode_gated(const mla_params* p, const void* q_nope, const void* q_rope,
                            const void* latent, const void* rope, const int32_t* seqlens,
                            const int32_t* block_table, const void* w_uk, const void* w_uv,
                            const void* gate, void* out, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);
mla_status mlra_decode_gated(const mla_params* p, const void* q_nope, const void* q_rope,
                             const void* latent, const void* rope, const int32_t* seqlens,
                             const int32_t* block_table, const void* w_uk, const void* w_uv,
                             const void* gate, void* out, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * Tracing variants: identical to mla_decode / mlra_decode, and additionally record five
 * caller-created HIP events (hipEvent_t values passed as void*) on `stream` at the stage
 * boundaries: events[0] before the prologue (whose launch also makes the split plan),
 * events[1] before the split-K main loop, events[2] before the combine, events[3] before the
 * epilogue, events[4] after it.  For bf16 the combine and the epilogue run as one kernel
 * between events[2] and events[3], and events[4] follows events[3] directly.  With events == NULL they behave exactly like the
 * plain entry points.  A failed hipEventRecord returns MLA_ERR_HIP.
 */
mla_status mla_decode_timed(const mla_params* p, const void* q_nope, const void* q_rope,
                            const void* latent, const void* rope, const int32_t* seqlens,
                            const int32_t* block_table, const void* w_uk, const void* w_uv,
                            void* out, void* workspace, size_t workspace_bytes, hipStream_t stream,
                            void* const* events);
mla_status mlra_decode_timed(const mla_params* p, const void* q_nope, const void* q_rope,
                             const void* latent, const void* rope, const int32_t* seqlens,
                             const int32_t* block_table, const void* w_uk, const void* w_uv,
                             void* out, void* workspace, size_t workspace_bytes, hipStream_t stream,
                             void* const* events);

/*
 * Allocation-free variant of mla_decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, semantics and results as mla_decode (NB = 1), bit for bit, minus the
 * workspace: the call uses a static device array of MLA_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends (its device address is looked
 * up once per device, on the first call made with that device current).  Nothing in it
 * needs clearing: every call writes its plan, queries and partials before reading them.
 * Returns MLA_ERR_WORKSPACE, before anything is launched, when mla_workspace_size(p) exceeds
 * MLA_NOALLOC_SCRATCH_BYTES (e.g. B = 256 sequences at H = 128).  Calls no hipMalloc /
 * hipFree or allocating routine.  All calls on one GPU share that GPU's array: two calls
 * that overlap in time on one GPU (different streams, or different host threads without
 * ordering) race on it; calls ordered on one stream do not.  After a call has completed,
 * the array's start holds its split plan as described above (for inspection).
 */
#define MLA_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)
mla_status mla_decode_noalloc(const mla_params* p, const void* q_nope, const void* q_rope,
                              const void* latent, const void* rope, const int32_t* seqlens,
                              const int32_t* block_table, const void* w_uk, const void* w_uv,
                              void* out, hipStream_t stream);

/*
 * Rotate rows of a rotary-key cache in place (the write-side step that gives the decoupled
 * key its position; RoFormer rotation, cited by the interview Q&A).  Row i starts at
 * x + i*row_stride (elements, dtype) and has d_rope elements; pairs (x_{2k}, x_{2k+1})
 * are rotated by angle pos[i] * theta^(-2k/d_rope) (product and reduction mod 2*pi in fp64,
 * sine/cosine of the reduced angle in fp32).  Rows with
 * pos[i] < 0 are left unchanged.  x: device, [n_rows] rows; pos: device int32 [n_rows].
 * d_rope even, 2..256; n_rows >= 0 (0 launches nothing).
 */
mla_status mla_rope_rotate(void* x, int64_t row_stride, const int32_t* pos, int64_t n_rows,
                           int32_t d_rope, float theta, int32_t dtype, hipStream_t stream);

/*
 * Cache append: the write side of the same cache, one decode step's new token per sequence
 * ("超越 GQA 的推理革命…MLA…", section 鍵值聯合低秩壓縮: at write time the token's key and
 * value information is compressed into the joint low-rank latent; section 解耦旋轉位置編碼:
 * the position part is a separate uncompressed key carrying RoPE).  For every sequence b,
 * with t = seqlens[b] (the new token's position; the cache then holds t + 1 tokens):
 *   c_KV   = h_b W_DKV                     (d_latent)
 *   k_rope = RoPE(h_b W_KR, position t)    (d_rope, stored rotated, as mla_decode reads it)
 * and the row [c_KV | k_rope] goes to position t of sequence b, after which seqlens[b] = t + 1.
 * MLRA-4's four branches are column blocks of the same projection, so its rows (d_latent =
 * 4 x 128) are written alike; one branch alone is d_latent = 128.
 * Paged cache: when t is a multiple of 64 the token starts a new page.  The sequences that
 * need one are ranked in batch order, the k-th takes free_pages[k], and it is entered at
 * block_table[b, t / 64]; *pages_used (device) receives min(pages needed, n_free), so the
 * caller can advance its free list.  A sequence that needs a page when the list is exhausted,
 * or whose position lies outside the cache (t < 0, t / 64 >= max_pages_per_seq, or
 * t >= capacity for a contiguous cache), is left untouched (no row, same length).
 * Accumulation fp32, storage bf16 (round to nearest even); angles reduced in fp64.
 *
 * Arguments (device pointers unless noted):
 *   hidden      bf16 [B, d_model], the new tokens' hidden states, 16-byte aligned
 *   w_dkv       bf16 [d_model, d_latent] (row = input feature), 16-byte aligned
 *   w_kr        bf16 [d_model, d_rope], 16-byte aligned
 *   latent/rope the cache, addressed as in mla_decode with the strides below (written)
 *   seqlens     int32 [B] (read and written); block_table int32 [B, block_table_stride]
 *               (paged: read and written; may be NULL for a contiguous cache)
 *   free_pages  int32 [n_free] page ids (may be NULL when n_free = 0)
 *   pages_used  int32 [1] (written)
 *   workspace   >= mla_append_workspace_size(p) bytes, 256-byte aligned
 * Supported: MLA_BF16, d_latent 512 or 128, d_rope 64, d_model a multiple of 256 up to
 * 65536, page_size 0 or 64.  Same conventions as the decode entry points (host validation,
 * no allocation, asynchronous on stream).
 */
typedef struct mla_append_params {
  int32_t batch;              /* B sequences, one new token each                           */
  int32_t d_model;            /* hidden size of the new tokens                             */
  int32_t d_latent;           /* latent width of a row (NB * d_cb)                         */
  int32_t d_rope;             /* rotary key width                                          */
  int32_t page_size;          /* 0 = contiguous cache, MLA_PAGE_SIZE = paged cache         */
  int32_t max_pages_per_seq;  /* paged: usable block_table columns                         */
  int32_t capacity;           /* contiguous: token rows per sequence                       */
  int32_t dtype;              /* mla_dtype                                                 */
  int64_t latent_stride_tok, latent_stride_seq, rope_stride_tok, rope_stride_seq;
  int64_t block_table_stride;
  float rope_theta;
  int32_t latent_format;      /* 0: latent rows in dtype; MLA_LATENT_FP8: the latent part is
                                 written as OCP FP8 E4M3 codes of value / latent_scale
                                 (nearest, ties to even, saturating at +-448; strides then
                                 count bytes), for a cache mla_decode reads with the same
                                 latent_format and latent_scale                            */
  float latent_scale;         /* MLA_LATENT_FP8: finite, > 0                               */
} mla_append_params;

/* Workspace bytes mla_cache_append needs for *p (host pointer *bytes). */
mla_status mla_append_workspace_size(const mla_append_params* p, size_t* bytes);

mla_status mla_cache_append(const mla_append_params* p, const void* hidden, const void* w_dkv,
                            const void* w_kr, void* latent, void* rope, int32_t* seqlens,
                            int32_t* block_table, const int32_t* free_pages, int32_t n_free,
                            int32_t* pages_used, void* workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * Prefill: many new tokens per sequence in one step, computed un-absorbed.  With s_q query
 * tokens against L cached ones the absorbed form scores every query over the 576-wide
 * latent row and sums the 512-wide latent (1088 multiply-adds per query, key and head);
 * up-projecting the cached latents once per head to keys and values costs 192 + 128 per pair
 * after that, the better trade once s_q reaches the hundreds (the interview Q&A "MLA … 是什么",
 * section 核心机制 step 3: the latent is up-projected with W_K_up / W_V_up at inference; the
 * yololab MLA page, section 繁榮背後的代價, on the compute-heavy regime).
 *
 * Same definition, arguments and layouts as mla_decode with p->num_queries = s_q ("Several
 * query tokens" above), s_q >= 1 and not bounded by 16 here: for each sequence b with L =
 * seqlens[b], query token i at position P = L - s_q + i and head h,
 *   K_t    = W_UK[h] c_t                       (d_nope)   V_t = W_UV[h]^T c_t   (d_v)
 *   s_t    = softmax_scale * (q_nope[b,i,h] . K_t + RoPE(q_rope[b,i,h], P) . k_t),  t <= P
 *   out[b,i,h] = out_scale * sum_{t <= P} softmax(s)_t V_t    (zero when P < 0)
 *   q_nope [B, s_q, H, NB, 128], q_rope [B, s_q, H, 64], out [B, s_q, H, 128], caches, seqlens,
 *   block_table and weights exactly as mla_decode (w_uk [NB, H, 128, d_latent], w_uv
 *   [NB, H, d_latent, 128]).
 * MLRA-4 (num_branches 4, d_latent 128 per branch; "[ICLR 2025] MLRA…", sections 2.1 and
 * 2.2) as in mlra_decode: branch br up-projects its own latent slice with W_UK[br] and
 * W_UV[br], scores its own query q_nope[b,i,h,br] plus the shared rotary term, takes its own
 * softmax, and out = out_scale * the sum of the branch outputs.
 * Supported: MLA_BF16, num_branches 1 with d_latent 512 (MLA) or 128 (one MLRA branch cached
 * on its own, the tensor-parallel shard) or num_branches 4 with d_latent 128, d_rope 64,
 * d_nope 128, d_v 128, any H in [1, 4096], batch <= 65535, page_size 0 or 64, flags 0,
 * latent_format 0 (otherwise MLA_ERR_UNSUPPORTED).  num_splits is not used.  Pointers of q_nope, q_rope, latent, rope,
 * w_uk, w_uv and out 16-byte aligned, cache strides multiples of 8 elements (MLA_ERR_ALIGN).
 * The workspace (>= mla_prefill_workspace_size bytes, 256-byte aligned, no initialisation)
 * receives the up-projected keys and values (B x H x NB x L_pad x 128 bf16 each, L_pad =
 * max_seqlen rounded up to a multiple of 256) and a copy of the rotary keys (B x L_pad x 64
 * bf16), in an internal tiled order, and with NB = 4 the branch outputs (B x s_q x H x 4 x
 * 128 bf16).  Kernels on `stream`: the up-projection (a GEMM of the cached latents against
 * W_UK and W_UV, which also copies the rotary keys), a causal flash-attention pass per
 * (head, branch), and with NB = 4 the scaled branch sum.  The up-projection's 256-token tiles,
 * B x H x NB x L_pad / 256, must number below 2^31 (MLA_ERR_SHAPE); it runs one workgroup per
 * compute unit, the count asked of the current device once (MLA_ERR_HIP if that fails).
 */
mla_status mla_prefill_workspace_size(const mla_params* p, size_t* bytes);
mla_status mla_prefill(const mla_params* p, const void* q_nope, const void* q_rope,
                       const void* latent, const void* rope, const int32_t* seqlens,
                       const int32_t* block_table, const void* w_uk, const void* w_uv, void* out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);
/* Tracing variant of mla_prefill: also records three caller-created HIP events (hipEvent_t
 * values passed as void*) on `stream`: events[0] before the up-projection, events[1] between
 * it and the attention, events[2] after the attention (and, with NB = 4, the branch sum).
 * A failed hipEventRecord returns MLA_ERR_HIP. */
mla_status mla_prefill_timed(const mla_params* p, const void* q_nope, const void* q_rope,
                             const void* latent, const void* rope, const int32_t* seqlens,
                             const int32_t* block_table, const void* w_uk, const void* w_uv,
                             void* out, void* workspace, size_t workspace_bytes,
                             hipStream_t stream, void* const* events);

/* Static, human-readable name of a status code. */
const char* mla_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
