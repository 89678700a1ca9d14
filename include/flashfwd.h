/*
 * libflashfwd -- fused, tiled attention forward pass for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every tensor argument is a device pointer owned by the caller; the
 * library never allocates, frees or synchronises, and keeps no mutable global
 * state apart from a per-device cache of the compute-unit count and of the address
 * of attn_fwd_splitkv_noalloc's static device buffer.  Each call checks all of its
 * arguments before enqueueing anything: on a non-zero return nothing was enqueued
 * and no output was touched.  On success the work is enqueued on `stream` (a
 * hipStream_t; NULL means the null stream) and runs asynchronously; device faults
 * surface at the caller's next synchronisation with that stream.  Calls are
 * re-entrant, except that overlapping attn_fwd_splitkv_noalloc calls on one GPU share
 * its buffer (see there).  There is no fallback path: an
 * unsupported shape is an error, never a slower route.  Diagnostics: with the
 * environment variable FLASHFWD_LOG set (to anything but "0"), every launch prints
 * one line on stderr naming its kernel, grid and tile or split plan.
 *
 * Layouts (the pages' [batch, seqlen, heads, head_dim] convention: "flash
 * attention V2 code walk-through", tensor-shape table), all row-major and
 * contiguous:
 *   q        bf16 [B, Sq, Hq, d]
 *   k, v     bf16 [B, Sk, Hkv, d]
 *   o        fp32 [B, Sq, Hq, d]
 *   lse      fp32 [B, Hq, Sq]           natural-log logsumexp of the scaled scores
 *   o_accum  fp32 [S, B, Hq, Sq, d]     per-split normalised partial outputs
 *   lse_accum fp32 [S, B, Hq, Sq]       per-split logsumexp
 * Query head h attends with key/value head h / (Hq / Hkv) (grouped-query
 * attention; Hq must be a multiple of Hkv).
 *
 * Semantics shared by all entry points.  For query row i of head h:
 *   s_j = scale * <q_i, k_j>;  key j is visible iff !causal or j <= i + Sk - Sq
 *   (causal mask aligned to the bottom-right corner: "03 forward CUDA kernel",
 *   section 8, and the walk-through's Is_causal pictures);
 *   O_i = sum_j softmax(s)_j v_j over visible keys, LSE_i = log sum_j exp(s_j);
 *   a row with no visible key gets O_i = 0 and LSE_i = -inf (explainer's
 *   one-row loop; forward-kernel page section 7.3).
 * S and P are never written to memory ("FlashAttention 1, 2, 3" explainer,
 * tiling section; forward-kernel page sections 3-6).  Arithmetic: bf16 inputs,
 * bf16 matrix-core products with fp32 accumulation, fp32 softmax state.
 *
 * Limits checked on every call: B, Sq, Sk >= 1; d in {64, 128}; Hq, Hkv >= 1;
 * every pointer 16-byte aligned; scale finite and > 0; each tensor below 2^31
 * elements.
 */
#ifndef FLASHFWD_H
#define FLASHFWD_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FF_OK = 0,
  FF_ERR_NULL = 1,     /* a required pointer is NULL */
  FF_ERR_SHAPE = 2,    /* B, Sq, Sk, Hq or Hkv < 1, or a size over the limits */
  FF_ERR_HEADDIM = 3,  /* d not in {64, 128} */
  FF_ERR_GQA = 4,      /* Hq not a multiple of Hkv */
  FF_ERR_ALIGN = 5,    /* a pointer not 16-byte aligned */
  FF_ERR_SPLITS = 6,   /* num_splits outside [1, FF_MAX_SPLITS] */
  FF_ERR_SCALE = 7,    /* scale not finite or not > 0 */
  FF_ERR_HIP = 8,      /* the HIP runtime reported an error (device query or launch) */
  FF_ERR_ALIAS = 9,    /* an output overlaps an input */
  FF_ERR_OPTION = 10,  /* a mask/bias option out of range (the _ex entry points) */
  FF_ERR_SCRATCH = 11  /* attn_fwd_splitkv_noalloc: the partials exceed the library's buffer */
} ff_status;

#define FF_MAX_SPLITS 128
/* Key granularity of the split-KV partition: split s of S covers key blocks
 * [s*ceil(nb/S), min((s+1)*ceil(nb/S), nb)) with nb = ceil(Sk / FF_SPLIT_BLOCK_N). */
#define FF_SPLIT_BLOCK_N 128

/* Fused forward pass (the prefill kernel): one workgroup per (query tile,
 * batch, head) streams key/value tiles through LDS, updates the online-softmax
 * state and accumulates O, then writes O = o / l and LSE = m + log l
 * (forward-kernel page sections 2-6; explainer, online-softmax and one-row
 * loop sections).  Writes o and lse in full. */
int attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
             int B, int Sq, int Sk, int Hq, int Hkv, int d, int causal, float scale,
             void* stream);

/* attn_fwd with the mask and bias variants ("flash attention V2 code walk-through", the
 * split-KV kernel's template flags Is_local, Has_alibi and Is_softcap, and its
 * n_block_min / n_block_max clipping).  With diag = i + Sk - Sq, the key aligned with
 * query row i:
 *   window_left, window_right: key j is visible iff
 *     diag - window_left <= j <= diag + window_right; -1 means no limit on that side.
 *     With causal set, j <= diag holds as well (causal is the window (-1, 0)).
 *   alibi_slopes: NULL, or fp32 device slopes; query head h of batch b uses
 *     alibi_slopes[b * alibi_batch_stride + h] (alibi_batch_stride 0: one slope per head,
 *     [Hq]; Hq: one per batch and head, [B, Hq]).  -slope * |diag - j| is added to the
 *     score of key j.
 *   softcap: 0 for none; c > 0 maps each scaled score s to c * tanh(s / c) before the
 *     ALiBi bias and the mask (the page gives no formula; this is the plain tanh limit).
 * The LSE is the logsumexp of the resulting logits.  With no option set (windows -1,
 * no slopes, softcap 0) this is attn_fwd, bit for bit.  A row whose window holds no key
 * gets O = 0, LSE = -inf.  Errors: FF_ERR_OPTION for a window below -1, a negative or
 * non-finite softcap, or a batch stride other than 0 or Hq; FF_ERR_ALIGN for slopes not
 * 4-byte aligned; FF_ERR_ALIAS if an output overlaps the slopes; otherwise as attn_fwd. */
int attn_fwd_ex(const void* q, const void* k, const void* v, float* o, float* lse,
                int B, int Sq, int Sk, int Hq, int Hkv, int d, int causal,
                int window_left, int window_right, const float* alibi_slopes,
                int alibi_batch_stride, float softcap, float scale, void* stream);

/* Forward over a variable-length batch ("03 forward CUDA kernel" section 8: sequences
 * concatenated without padding, boundaries given by prefix sums; "flash attention V2
 * code walk-through", Flash_fwd_params: cu_seqlens_q / cu_seqlens_k, q as
 * (total_q, num_heads, head_size)).  Sequence b owns query rows cu_seqlens_q[b] ..
 * cu_seqlens_q[b+1]-1 and key/value rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1; each
 * sequence is attended on its own, causal bottom-right aligned within the sequence.
 *   q [total_q,Hq,d], k, v [total_k,Hkv,d]: bf16; o [total_q,Hq,d], lse [Hq,total_q]: fp32
 *   cu_seqlens_q, cu_seqlens_k: device int32 [B+1], non-decreasing, starting at 0 and
 *     ending at total_q / total_k; max_seqlen_q: the longest query sequence
 * The prefix sums live on the device and are not checked on the host; the kernel clamps
 * them to [0, total] so that no access leaves the tensors (a malformed sum yields
 * unspecified values for the sequences it touches).  A sequence without keys gets O = 0,
 * LSE = -inf.  Other argument rules and errors as for attn_fwd; the prefix sums need
 * 4-byte alignment. */
int attn_fwd_varlen(const void* q, const void* k, const void* v, float* o, float* lse,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int max_seqlen_q,
                    int total_q, int total_k, int Hq, int Hkv, int d, int causal, float scale,
                    void* stream);

/* Split count for attn_fwd_splitkv.  The rule is the forward-kernel page's
 * (section 7.2): the smallest split count whose wave efficiency is at least 85%
 * of the best, where efficiency(S) = w / ceil(w) and w = units * S / slots.
 * Here units = B * Hkv * ceil(Sq * (Hq/Hkv) / 16) workgroups per split and
 * slots = num_cus (one split workgroup per CU), and S is capped so every
 * split keeps at least 4 key blocks of FF_SPLIT_BLOCK_N.  num_cus <= 0 queries
 * the current device.  Pure host arithmetic apart from that query.  For benchmark
 * sweeps only, the environment variable FLASHFWD_NUM_SPLITS = n (an integer in
 * [1, FF_MAX_SPLITS]) replaces the rule's choice; other values are ignored.
 * Returns S >= 1, or the negated ff_status on invalid arguments. */
int attn_splitkv_num_splits(int B, int Sq, int Sk, int Hq, int Hkv, int d, int num_cus);

/* The efficiency rule alone, for `units` workgroups per split on `slots`
 * concurrent workgroup slots, searching S in [1, max_splits].  With units = 48,
 * slots = 108 it returns 2 (efficiencies 0.89 at S = 2 and 0.67 at S = 3, the
 * page's worked example).  Returns the negated FF_ERR_SHAPE if an argument < 1. */
int attn_splits_efficiency_rule(int units, int slots, int max_splits);

/* Split-KV forward (the decode kernel).  The key range is cut into num_splits
 * contiguous ranges of FF_SPLIT_BLOCK_N-key blocks (walk-through, split-KV
 * block range); each workgroup computes one range for up to 16 query rows of
 * one key/value head, the Hq/Hkv query heads sharing that head folded into the
 * row dimension (forward-kernel page section 7.4; the fold is a stride view, no
 * copy).  num_splits == 1: writes o and lse directly (o_accum, lse_accum may be
 * NULL).  num_splits > 1: writes o_accum and lse_accum only (o, lse may be
 * NULL); a split with no visible key writes O_s = 0 and LSE_s = -inf.  With
 * Sq == 1 every key is visible whatever `causal` says (the query sits at
 * position Sk - 1). */
int attn_fwd_splitkv(const void* q, const void* k, const void* v,
                     float* o_accum, float* lse_accum, float* o, float* lse,
                     int B, int Sq, int Sk, int Hq, int Hkv, int d, int causal, float scale,
                     int num_splits, void* stream);

/* LSE-weighted combine of attn_fwd_splitkv's partials (forward-kernel page
 * section 7.3): per row, LSE = log sum_s exp(LSE_s) and O = sum_s exp(LSE_s -
 * LSE) O_s; splits with LSE_s = -inf weigh 0; a row whose splits are all -inf
 * gets O = 0, LSE = -inf.  Writes o [B,Sq,Hq,d] and lse [B,Hq,Sq]. */
int attn_splitkv_combine(const float* o_accum, const float* lse_accum, float* o, float* lse,
                         int B, int Sq, int Hq, int d, int num_splits, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): attn_fwd_splitkv followed, for
 * num_splits > 1, by attn_splitkv_combine, with the split partials kept in a device
 * buffer the library owns instead of caller buffers.  The buffer is a static array of
 * FF_NOALLOC_SCRATCH_FLOATS floats (16 MiB), one per GPU, held until the process ends;
 * the call allocates nothing and frees nothing.  It needs num_splits * B * Hq * Sq *
 * (d + 1) floats of it (num_splits > 1; none for one split) and returns FF_ERR_SCRATCH
 * when that is larger.  Every call on a GPU uses that GPU's one buffer: calls that
 * overlap in time on one GPU (different streams, or other threads) race on it, so
 * callers serialise them (one stream, say).  Arguments, layouts, outputs and the other
 * errors as attn_fwd_splitkv and attn_splitkv_combine; all checks are made before
 * anything is enqueued.  FF_ERR_HIP if the buffer's device address cannot be obtained. */
#define FF_NOALLOC_SCRATCH_FLOATS (4 << 20)
int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, float* o, float* lse,
                             int B, int Sq, int Sk, int Hq, int Hkv, int d, int causal,
                             float scale, int num_splits, void* stream);

/* Split-KV forward against a key/value cache (the decode path of "03 forward CUDA
 * kernel" section 8, which sends cached attention through the split-KV kernel; "flash
 * attention V2 code walk-through": block_table in Flash_fwd_params, the paged row offsets
 * of the split-KV kernel's data preparation, and k_offset with leftpad_k in BlockInfo).
 *   q [B,Sq,Hq,d] bf16; outputs as for attn_fwd_splitkv (o [B,Sq,Hq,d], lse [B,Hq,Sq];
 *     or the partials for attn_splitkv_combine when num_splits > 1).
 *   Paged (block_table != NULL): k_cache, v_cache [num_blocks, page_size, Hkv, d] bf16;
 *     block_table [B, max_blocks_per_seq] int32: logical position t of batch b lives in
 *     block block_table[b][t / page_size], row t % page_size.  page_size must be a
 *     multiple of 32.
 *   Contiguous (block_table == NULL): k_cache, v_cache [B, page_size, Hkv, d], page_size
 *     being the capacity; num_blocks and max_blocks_per_seq are ignored.
 *   cache_seqlens [B] int32: batch b's keys end at position cache_seqlens[b] + new_keys
 *     (new_keys >= 0: rows written by attn_kvcache_append just before, or 0).
 *   cache_leftpad [B] int32 or NULL: batch b's keys start at position cache_leftpad[b]
 *     (left padding; NULL = 0).
 * Causal masking is bottom-right aligned: query i sees key position j iff
 * j <= i + end_b - Sq.  Each split takes an equal share of its batch's keys, so a short
 * sequence in a long cache does not leave splits idle.  The device arrays are not read
 * on the host; the kernel clamps lengths to [0, capacity], left padding to [0, length]
 * and block numbers to [0, num_blocks - 1], so no access leaves the caches (bad values
 * give unspecified results for their batch).  A batch without keys gets O = 0,
 * LSE = -inf.  Errors: FF_ERR_SHAPE also for page_size not a multiple of 32 (paged) and
 * capacities of 2^31 positions or more; int32 arrays need 4-byte alignment.  The caches
 * are read only. */
int attn_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache,
                     const int* cache_seqlens, const int* cache_leftpad, const int* block_table,
                     float* o_accum, float* lse_accum, float* o, float* lse, int B, int Sq,
                     int Hq, int Hkv, int d, int num_blocks, int page_size,
                     int max_blocks_per_seq, int new_keys, int causal, float scale,
                     int num_splits, void* stream);

/* attn_fwd_kvcache with the mask and bias variants of attn_fwd_ex.  diag = i + n_b - Sq
 * for batch b, with n_b = cache_seqlens[b] + new_keys its key count (positions left of
 * cache_leftpad[b] stay invisible).  The window narrows the keys the splits share, so
 * num_splits splits cover only the visible range.  Arguments, errors and outputs
 * otherwise as attn_fwd_kvcache and attn_fwd_ex. */
int attn_fwd_kvcache_ex(const void* q, const void* k_cache, const void* v_cache,
                        const int* cache_seqlens, const int* cache_leftpad,
                        const int* block_table, float* o_accum, float* lse_accum, float* o,
                        float* lse, int B, int Sq, int Hq, int Hkv, int d, int num_blocks,
                        int page_size, int max_blocks_per_seq, int new_keys, int causal,
                        int window_left, int window_right, const float* alibi_slopes,
                        int alibi_batch_stride, float softcap, float scale, int num_splits,
                        void* stream);

/* In-place append of new keys and values to a cache ("03 forward CUDA kernel" section 8;
 * the walk-through's Append_KV case, new k/v given as knew/vnew): k_new[b][t] and
 * v_new[b][t] ([B, S_new, Hkv, d] bf16) are written at logical position
 * cache_seqlens[b] + t of batch b, with the cache layout, block table and clamping of
 * attn_fwd_kvcache; positions at or past the capacity are dropped.  cache_seqlens is not
 * updated: pass new_keys = S_new to attn_fwd_kvcache on the same stream.  Batches whose
 * block tables share a block race on it.  Errors as for attn_fwd_kvcache; the new rows
 * must not overlap the caches. */
int attn_kvcache_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                        const int* cache_seqlens, const int* block_table, int B, int S_new,
                        int Hkv, int d, int num_blocks, int page_size, int max_blocks_per_seq,
                        void* stream);

/* FP8 quantization ("FlashAttention 1, 2, 3" explainer, FlashAttention-3 precision
 * section: a scale per block, carried into the computation; Q and K may first go through
 * a matching orthogonal transform, which keeps QK^T).
 *   x [B,S,H,d] bf16 -> x_fp8 [B,S,H,d] OCP FP8 E4M3 bytes and scales [B,H,ceil(S/128)]
 *   fp32: for each (b, h, block of 128 rows) scale = amax / 448 over the block (1 for an
 *   all-zero block) and code = round-to-nearest-even E4M3 of x / scale (IEEE division).
 *   rotate != 0 first applies the normalized Walsh-Hadamard transform along d (fp32
 *   butterflies of distance 1, 2, ..., d/2, then times fp32(1/sqrt(d))); rotate Q and K
 *   both or neither, never V.
 * Errors: FF_ERR_NULL, FF_ERR_SHAPE (B, S, H < 1 or 2^31 elements), FF_ERR_HEADDIM,
 * FF_ERR_ALIGN (16 bytes), FF_ERR_ALIAS (outputs overlapping x or each other). */
int attn_quantize_fp8(const void* x, void* x_fp8, float* scales, int B, int S, int H, int d,
                      int rotate, void* stream);

/* FP8 forward: attention on the dequantized tensors code * scale (scales as
 * attn_quantize_fp8 writes them: q_scale [B,Hq,ceil(Sq/128)], k_scale and v_scale
 * [B,Hkv,ceil(Sk/128)], positive and finite).  q [B,Sq,Hq,d], k, v [B,Sk,Hkv,d] are E4M3
 * bytes; o [B,Sq,Hq,d] and lse [B,Hq,Sq] fp32; causal and scale as for attn_fwd.  Both
 * products run on the fp8 matrix cores with fp32 accumulation; the softmax state is fp32;
 * the probabilities are rounded to E4M3 for the PV product (the error bound follows from
 * that rounding, relative 2^-4 per probability).  Errors as for attn_fwd, plus
 * FF_ERR_NULL for a missing scale array and FF_ERR_ALIAS for outputs overlapping them. */
int attn_fwd_fp8(const void* q, const void* k, const void* v, const float* q_scale,
                 const float* k_scale, const float* v_scale, float* o, float* lse, int B,
                 int Sq, int Sk, int Hq, int Hkv, int d, int causal, float scale, void* stream);

/* Size of attn_bwd's workspace, in floats: 2 * B * Hq * roundup(Sq, 64).  Returns the
 * count, or the negated ff_status (FF_ERR_SHAPE) for B, Sq or Hq below 1. */
long long attn_bwd_workspace_floats(int B, int Sq, int Hq);

/* Backward of attn_fwd: dQ, dK, dV from the forward's saved LSE ("FlashAttention 1, 2, 3"
 * explainer, sections "backward: from the softmax derivative", "training: backward
 * recomputation" and "backward: back to Q, K, V").  P is recomputed as
 * exp(scale * q.k - LSE), and with D = sum_c dO_c O_c per row:
 *   dV = P^T dO,  dP = dO V^T,  dS = P (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
 * Masked pairs (causal, bottom-right aligned as in attn_fwd) contribute nothing.  With
 * GQA, dK and dV of a key/value head sum over its Hq/Hkv query heads.
 *   q, k, v, dout: bf16, q and dout [B,Sq,Hq,d], k and v [B,Sk,Hkv,d]
 *   o, lse: fp32 [B,Sq,Hq,d] and [B,Hq,Sq], as attn_fwd wrote them for the same inputs
 *   dq: fp32 [B,Sq,Hq,d]; dk, dv: fp32 [B,Sk,Hkv,d]; all three written in full
 *   ws: fp32 workspace of attn_bwd_workspace_floats(B, Sq, Hq) floats, owned by the
 *       caller and overwritten (D and the LSE in base 2 per row; not part of the
 *       interface after the call returns)
 * P and dS are rounded to bf16 as matrix-core operands; all accumulation is fp32.  The
 * result is bitwise deterministic (no atomics).  Argument rules and errors as for
 * attn_fwd (dq, dk, dv and ws must not overlap each other or any input:
 * FF_ERR_ALIAS).  Enqueues two kernels on `stream`. */
int attn_bwd(const void* q, const void* k, const void* v, const float* o, const float* lse,
             const void* dout, float* dq, float* dk, float* dv, float* ws, int B, int Sq, int Sk,
             int Hq, int Hkv, int d, int causal, float scale, void* stream);

/* attn_bwd for the mask and bias variants of attn_fwd_ex: the sliding window
 * (window_left, window_right; -1 = no limit on that side) and ALiBi slopes (fp32 on the
 * device, [Hq] with alibi_batch_stride 0 or [B, Hq] with stride Hq), with the same
 * meaning as there; o and lse must come from attn_fwd_ex with the same options.  A pair
 * outside the window has P = 0, and the ALiBi bias does not depend on q or k, so the
 * formulas of attn_bwd stand.  softcap must be 0 (the soft cap's backward is not
 * provided): anything else returns FF_ERR_OPTION, as do out-of-range options.  The
 * slopes must not overlap dq, dk, dv or ws (FF_ERR_ALIAS).  Otherwise as attn_bwd. */
int attn_bwd_ex(const void* q, const void* k, const void* v, const float* o, const float* lse,
                const void* dout, float* dq, float* dk, float* dv, float* ws, int B, int Sq,
                int Sk, int Hq, int Hkv, int d, int causal, int window_left, int window_right,
                const float* alibi_slopes, int alibi_batch_stride, float softcap, float scale,
                void* stream);

/* Static description of a status code. */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FLASHFWD_H */
