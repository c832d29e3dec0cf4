/*
 * mla_decode.h - C ABI of the MI355X (gfx950) MLA / MLRA-4 latent-KV decode library.
 *
 * One decode step (one query token per sequence) of Multi-head Latent Attention over a
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
 *    allocates or frees memory, never synchronises the stream, and keeps no mutable
 *    global state; calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream) and may be made concurrently from several host threads.
 *  - Arguments are validated on the host before anything is launched; a failed check
 *    returns a non-zero mla_status and launches nothing.  Values that live in device memory
 *    (seqlens, block_table entries) are not validated: seqlens[b] must lie in
 *    [0, max_seqlen] and every block_table entry for a page a sequence uses must index an
 *    existing page; otherwise the behaviour is undefined.
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

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,        /* a required pointer is NULL                               */
  MLA_ERR_SHAPE = 2,       /* a size, stride or bound is negative or inconsistent      */
  MLA_ERR_UNSUPPORTED = 3, /* valid request this build has no kernel for (dims, page)  */
  MLA_ERR_WORKSPACE = 4,   /* workspace_bytes smaller than mla_workspace_size()        */
  MLA_ERR_DTYPE = 5,       /* unknown dtype                                            */
  MLA_ERR_ALIGN = 6,       /* pointer or stride not aligned as the dtype requires      */
  MLA_ERR_HIP = 7          /* a HIP runtime call or kernel launch failed               */
} mla_status;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1 } mla_dtype;

/* Page size of the paged latent cache, in tokens. */
#define MLA_PAGE_SIZE 64

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
  int64_t latent_stride_tok;  /* elements between consecutive tokens of the latent cache   */
  int64_t latent_stride_seq;  /* contiguous: elements between sequences; paged: pages      */
  int64_t rope_stride_tok;    /* same two strides for the rotary-key cache                 */
  int64_t rope_stride_seq;
  int64_t block_table_stride; /* elements between rows of block_table (>= max_pages)      */
  float softmax_scale;        /* score scale, usually 1/sqrt(d_nope + d_rope)              */
  float out_scale;            /* scale on the (branch-summed) output: 1 MLA, 0.5 MLRA-4    */
  float rope_theta;           /* RoPE base, e.g. 10000                                     */
} mla_params;

/*
 * Supported shapes in this build (anything else returns MLA_ERR_UNSUPPORTED):
 *  - MLA_BF16, NB = 1: d_latent = 512, d_rope = 64, d_nope = 128, d_v = 128, H % 32 == 0.
 *  - MLA_BF16, NB = 4: d_latent = 128, d_rope = 64, d_nope = 128, d_v = 128, H % 32 == 0.
 *  - MLA_F32 (generic SIMT path): NB in {1, 4}, NB*d_latent <= 512, d_rope even <= 64,
 *    d_nope <= 256, d_v <= 256, any H >= 1.
 *  - page_size in {0, 64}.
 * Alignment: bf16 latent, rope, q_nope, w_uk and w_uv pointers 16-byte aligned and the
 * cache strides multiples of 8 elements; other pointers aligned to their element size.
 * num_splits is at most 512 and at most ceil(max_seqlen / 64).
 *
 * Split plan.  The attention over each sequence is split into work items of whole 64-token
 * pages (split-K over the sequence) whose partial results are merged afterwards.  The plan is
 * made on the device from seqlens at the start of every call, so it follows the actual
 * lengths: with p_b = ceil(seqlens[b] / 64) pages, every sequence is cut into
 * ceil(p_b / c) items of c pages (the last one ragged; an empty sequence gets none).  With
 * num_splits = 0, c is the smallest page count for which the batch's items fit the number of
 * workgroups that fill the GPU once (256 items for bf16 MLA with H % 128 == 0, else 512 /
 * workgroups per item); when no c does, c = max_b p_b.  With num_splits = n,
 * c = ceil(ceil(max_seqlen / 64) / n).
 * After a call has completed on its stream, the workspace starts with that plan (for
 * inspection; nothing reads it after the call):
 *   int32 hdr[4] at byte 0: { W = number of items, c, slots, item target (0 when forced) }
 *   int32 work[slots][4] at byte 16: { b, t_begin, t_end, item } per dispatch slot of the
 *         main kernels, b = -1 for a slot without an item; items are numbered
 *         sequence-major, item i of sequence b covering tokens [t_begin, t_end)
 *   int32 split_off[B + 1] at byte 16 + 16 * slots: items of sequence b are
 *         split_off[b] .. split_off[b + 1] - 1, split_off[B] = W.
 */

/*
 * Bytes of device workspace mla_decode / mlra_decode need for *p (written to *bytes, a
 * host pointer).  Depends only on the fields of *p.  The workspace holds the split plan, the
 * absorbed queries, the per-item partial results (running max, running sum and latent-space
 * output of each work item) and, for fp32, the merged latent-space output.
 */
mla_status mla_workspace_size(const mla_params* p, size_t* bytes);

/* Most work items (splits) one sequence can be cut into for *p (written to *splits, host):
 * n when num_splits = n > 0, else min(ceil(max_seqlen / 64), item target). */
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
 *   q_nope      [B, H, NB, d_nope] contiguous
 *   q_rope      [B, H, d_rope] contiguous, NOT rotated (rotated here at position L-1)
 *   latent      contiguous: element (b, t, j) at latent[b*latent_stride_seq + t*latent_stride_tok + j]
 *               paged: element (b, t, j) at latent[pg*latent_stride_seq + (t%64)*latent_stride_tok + j]
 *               with pg = block_table[b*block_table_stride + t/64];  j < NB*d_latent
 *   rope        rotated keys, addressed like latent with the rope strides; j < d_rope
 *               (the usual fused row [c_KV | k_rope] is rope = latent + NB*d_latent)
 *   seqlens     int32 [B], 0 <= seqlens[b] <= max_seqlen
 *   block_table int32 [B, block_table_stride] when page_size = 64, else ignored (may be NULL)
 *   w_uk        [NB, H, d_nope, d_latent]   (K = w_uk[br,h] c)
 *   w_uv        [NB, H, d_latent, d_v]      (V = w_uv[br,h]^T c)
 *   out         [B, H, d_v] contiguous, written
 *   workspace   >= mla_workspace_size(p) bytes, 256-byte aligned, contents need no
 *               initialisation and are overwritten
 *   stream      hipStream_t
 * Returns MLA_ERR_UNSUPPORTED if p->num_branches != 1.
 */
mla_status mla_decode(const mla_params* p, const void* q_nope, const void* q_rope,
                      const void* latent, const void* rope, const int32_t* seqlens,
                      const int32_t* block_table, const void* w_uk, const void* w_uv, void* out,
                      void* workspace, size_t workspace_bytes, void* stream);

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
                       void* workspace, size_t workspace_bytes, void* stream);

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
                            void* out, void* workspace, size_t workspace_bytes, void* stream,
                            void* const* events);
mla_status mlra_decode_timed(const mla_params* p, const void* q_nope, const void* q_rope,
                             const void* latent, const void* rope, const int32_t* seqlens,
                             const int32_t* block_table, const void* w_uk, const void* w_uv,
                             void* out, void* workspace, size_t workspace_bytes, void* stream,
                             void* const* events);

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
                           int32_t d_rope, float theta, int32_t dtype, void* stream);

/* Static, human-readable name of a status code. */
const char* mla_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
