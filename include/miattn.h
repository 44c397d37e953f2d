/* miattn -- exact IO-aware attention for MI355X (gfx950), C ABI.
 *
 * What is computed: exact scaled dot-product attention
 *     O = softmax(scale * Q K^T) V
 * ("Attention Mechanism Optimization for Efficient LLM Inference",
 * "Background: Scaled Dot-Product Attention"), evaluated tile by tile with the
 * running-max / running-sum softmax so the score and probability matrices are
 * never stored ("플래시어텐션: 메모리를 아끼는 정확한 어텐션", §2 타일링 and §3
 * 알고리즘, Theorem 1). Alongside O the library returns the per-row
 * log-sum-exp LSE = m + ln(l) of the scaled scores (natural log), the only
 * statistic the method keeps besides O (same page, §4 재계산).
 *
 * Conventions common to every entry point
 *  - Pointers marked "device" are HIP device pointers; the caller owns them.
 *    The library allocates nothing, frees nothing and keeps no mutable global
 *    state, so calls on different streams may run concurrently -- except
 *    attn_decode_noalloc, whose calls share a static scratch per device.
 *  - Layout is [batch, seq, heads, d] ("Multi-Query Attention (MQA)",
 *    "Comparison"), d contiguous (stride 1). Other strides are given in
 *    elements through miattn_strides; NULL means packed.
 *  - Head groups: query head h reads KV head h / (Hq / Hkv)
 *    ("Grouped-Query Attention (GQA)": contiguous groups; Hkv = 1 is MQA,
 *    Hkv = Hq is MHA). Hq must be a multiple of Hkv.
 *  - Arguments are validated on the host before anything is launched; a
 *    nonzero status means nothing was enqueued. Kernels are enqueued on
 *    `stream` (a hipStream_t; NULL = the null stream) and the call returns
 *    without synchronising. MIATTN_ERR_HIP reports a launch error; faults
 *    inside kernels surface at the caller's next synchronisation.
 *  - No atomics: the same inputs and arguments give bitwise identical outputs.
 *  - A call enqueues kernels only (no memset, copy or allocation), so it can be
 *    captured in a HIP graph and replayed; what a call keeps in its workspace
 *    is rewritten by its own kernels on every launch or replay.
 *  - No C++ exception crosses this interface.
 */
#ifndef MIATTN_H
#define MIATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  MIATTN_OK = 0,
  MIATTN_ERR_NULL = 1,        /* a required pointer is NULL                  */
  MIATTN_ERR_SHAPE = 2,       /* sizes inconsistent or out of range          */
  MIATTN_ERR_UNSUPPORTED = 3, /* valid request the library does not implement */
  MIATTN_ERR_WORKSPACE = 4,   /* workspace missing or smaller than required  */
  MIATTN_ERR_HIP = 5,         /* a HIP runtime call or launch failed         */
  MIATTN_ERR_ARG = 6          /* a scalar argument is invalid (scale, mode)  */
};

/* Element types. */
enum { MIATTN_BF16 = 0, MIATTN_F32 = 1 };

/* Mask kinds (bit flags; CAUSAL | BLOCK combines both rules). */
enum { MIATTN_MASK_NONE = 0, MIATTN_MASK_CAUSAL = 1, MIATTN_MASK_BLOCK = 2 };

/* Softmax evaluation ("TPU attention 최적화 실전 가이드", 4단계; "Online-
 * Softmax"). ONLINE keeps a running row max and rescales. FIXED_MAX subtracts
 * a per-row upper bound on the row's logits fixed before the key loop, by
 * Cauchy-Schwarz over the keys the row can see: the keys of each (batch, KV
 * head) are cut into blocks (the block mask's block_k, else 256 keys); a
 * block the row sees whole bounds its logits by scale * |q_i| * max |k_j|, a
 * block the causal rule cuts by the same over the keys the row sees.
 * FIXED_MAX_CENTERED bounds a whole block by scale * (q_i . c + |q_i| * max
 * |k_j - c|) around the block's mean key c (rounded to bf16); cut blocks as in
 * FIXED_MAX. The bound's distance to the row max is at most the gap between
 * it and the matching lower bound (|q_i| * max|k_j| below zero, or q_i . c -
 * |q_i| * max|k_j - c|); a row whose gap could exceed 64 nats falls back to
 * ONLINE, so exp never underflows the row. Every decision is made per row
 * from the keys that row sees, so keys a mask excludes never change a row's
 * output bits. The result is the same exact attention in every mode. */
enum {
  MIATTN_SOFTMAX_ONLINE = 0,
  MIATTN_SOFTMAX_FIXED_MAX = 1,
  MIATTN_SOFTMAX_FIXED_MAX_CENTERED = 2
};

/* Element strides of a [B, S, H, d] view (d has stride 1). */
typedef struct {
  int64_t b, s, h;
} miattn_strides;

/* Bytes of device workspace attn_fwd needs for these arguments (the same
 * meaning as in attn_fwd; block_q and block_k are read only when mask_kind has
 * BLOCK). Zero for ONLINE without a block mask. Returns 0 for negative sizes.
 * The workspace holds, in this order, each part starting at a multiple of 256
 * bytes:
 *  - fixed-max modes: the key statistics, float [B*Hkv][Nk] (prefix maxima
 *    of |k| within each key block), then the per-row decisions, uint8
 *    [B][Hq][Nq]: 1 where the row took the fixed max, 0 where it fell back
 *    to the running max (readable after the call; for inspection and tests);
 *    centred mode adds float [B*Hkv][nkb] radii and bf16 [B*Hkv][nkb][d]
 *    block centres (nkb = Nk / block_k, or ceil(Nk / 256) without a mask);
 *  - a BLOCK mask whose block_q is not a multiple of 32: a table of row
 *    segments (runs of block rows with identical mask rows, cut into pieces
 *    of at most 32 rows), built on the stream before the attention kernel. */
size_t attn_fwd_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int d, int mask_kind,
                                int block_q, int block_k, int softmax_mode);

/* Prefill / full-sequence attention.
 *
 * q      device, [B, Nq, Hq, d], dtype          (read)
 * k, v   device, [B, Nk, Hkv, d], dtype         (read)
 * o      device, [B, Nq, Hq, d], dtype          (written)
 * lse    device, float [B, Hq, Nq] or NULL      (written: m + ln l, natural log)
 * dtype  MIATTN_BF16 (bf16 MFMA, fp32 accumulation; P rounded to bf16 for the
 *        P V product) or MIATTN_F32 (fp32 throughout)
 * d      64 or 128
 * scale  > 0 and finite; usually 1/sqrt(d)
 * mask_kind  MIATTN_MASK_* flags.
 *        CAUSAL: key j is visible to query i iff j <= i + (Nk - Nq) (rows
 *        aligned at the end, so a single query sees every key).
 *        BLOCK: block_mask (device, uint8 [Nq/block_q, Nk/block_k], row-major,
 *        shared by every batch and head); pairs in a zero block are excluded,
 *        pairs in a nonzero block are included ("플래시어텐션..." §6 블록 희소).
 *        block_q and block_k must be multiples of 16 dividing Nq and Nk, so
 *        no block is partial ("TPU attention 최적화 실전 가이드", 3단계), and
 *        Nk / block_k <= 4096.
 * softmax_mode  MIATTN_SOFTMAX_*
 * strides  NULL (packed) or an array of 4: q, k, v, o
 * workspace, workspace_bytes  device scratch of at least
 *        attn_fwd_workspace_bytes(B, Hq, Hkv, Nq, Nk, d, mask_kind, block_q,
 *        block_k, softmax_mode) bytes (may be NULL / 0 when that is 0); owned by the
 *        caller, overwritten by the call, free for reuse once the call's work
 *        on the stream has finished
 * stream   hipStream_t
 * A query row with no visible key yields O = 0 and LSE = -inf. Finite values
 * at positions a mask excludes never change a bit of the result, in every
 * softmax mode. Inf and NaN at excluded positions never reach a row that
 * cannot see them either; at visible positions they propagate (IEEE). (Under
 * the causal rule such a value can reach a hidden row's accumulator through
 * a zero weight; a wave whose accumulators turn non-finite recomputes its
 * rows pair by pair, which only inputs with such values pay for.) */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int dtype, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
             int mask_kind, const uint8_t* block_mask, int block_q, int block_k,
             int softmax_mode, const miattn_strides* strides,
             void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace attn_decode needs for the split-K partials
 * (0 when the sizes are invalid). Independent of max_len and kv_splits. */
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int max_len, int d, int kv_splits);

/* Decode: one new query token per sequence against a contiguous KV cache
 * ("Role of KV Cache"; "Two Phases of Inference", Decode): query token b
 * attends to the first seqlens[b] cached keys of its sequence.
 *
 * The cached rows of all sequences, laid end to end, are cut into kv_splits
 * equal ranges, so every workgroup streams the same number of rows whatever
 * the length mix. Each range writes a normalised output and LSE for every
 * sequence it touches to the workspace, and a second kernel merges them with
 * the block rule of "플래시어텐션..." §2 타일링 (weights exp(LSE_c - LSE)).
 *
 * q        device, [B, Hq, d] bf16, packed       (read)
 * k_cache, v_cache  device, [B, max_len, Hkv, d] bf16 (read; rows at or past
 *          seqlens[b] are never read)
 * seqlens  device, int32 [B], each in [0, max_len]. The values live on the
 *          device, so the host cannot check them; the kernels clamp each to
 *          [0, max_len] as they read it (a longer length acts as max_len, a
 *          negative one as 0), so no length reads outside the cache
 * o        device, [B, Hq, d] bf16, packed        (written)
 * lse      device, float [B, Hq] or NULL          (written)
 * dtype    MIATTN_BF16
 * d        64 or 128; Hq / Hkv <= 16
 * kv_splits  number of ranges, 1..4096, or 0 for automatic (enough to
 *          fill every CU of the current device)
 * cache_strides  NULL (packed) or an array of 2: k_cache, v_cache
 * workspace  device, at least attn_decode_workspace_bytes(...) bytes
 * A sequence of length 0 yields O = 0 and LSE = -inf. */
int attn_decode(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* seqlens, void* o, float* lse, int dtype, int B,
                int Hq, int Hkv, int max_len, int d, float scale, int kv_splits,
                const miattn_strides* cache_strides, void* workspace,
                size_t workspace_bytes, void* stream);

/* attn_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. Same arguments, meaning and result as attn_decode
 * (bitwise equal to it for the same kv_splits); the split-K partials go to a
 * static 32 MiB array in the library's device code, one per device, held
 * until the process ends. The call allocates nothing (no hipMalloc, no
 * allocating library routine); on its first call on a device it looks up that
 * device's copy of the array (the device must be current, as for any launch
 * on `stream`). The partials take (S + B) * Hq * (d + 1) * 4 bytes (each of
 * the two parts rounded up to 256 bytes), with S = kv_splits or the automatic
 * count (eight 64-lane waves per CU of the device; 256 ranges on 256 CUs for
 * Hkv = 8); a call that needs more than 32 MiB returns MIATTN_ERR_WORKSPACE
 * and launches nothing. Every call on a device shares that device's array:
 * calls that overlap on one device (on different streams, or from different
 * threads without ordering) race and may return wrong results; calls ordered
 * on one stream are safe, since each call writes every partial it reads. */
int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seqlens, void* o, float* lse, int dtype, int B, int Hq,
                        int Hkv, int max_len, int d, float scale, int kv_splits,
                        const miattn_strides* cache_strides, void* stream);

/* Bytes of device workspace attn_decode_multi needs (0 when the sizes are
 * invalid). Independent of max_len and kv_splits. */
size_t attn_decode_multi_workspace_bytes(int B, int n_new, int Hq, int Hkv, int max_len, int d,
                                         int kv_splits);

/* Decode of several new tokens per sequence at once (for example the draft
 * tokens of speculative or multi-token decoding): n_new query rows per
 * sequence whose own keys and values are already the last n_new cached rows,
 * causal among themselves. Row t (0-based) of sequence b attends to cached
 * rows 0 .. seqlens[b] - n_new + t -- the causal rule of attn_fwd with the
 * rows aligned at the end ("Two Phases of Inference", Decode, one token at a
 * time; the same rule for several). All rows of a sequence share one read of
 * the cache: the n_new x (Hq/Hkv) rows of a KV head fill the 16-wide side of
 * the matrix products. Same split-K and merge as attn_decode.
 *
 * q        device, [B, n_new, Hq, d] bf16, packed  (read)
 * o        device, [B, n_new, Hq, d] bf16, packed  (written)
 * lse      device, float [B, n_new, Hq] or NULL     (written)
 * n_new    >= 1 with n_new * (Hq / Hkv) <= 16
 * other arguments as in attn_decode; workspace at least
 * attn_decode_multi_workspace_bytes(...) bytes. A row that sees no cached row
 * (seqlens[b] - n_new + t < 0) yields O = 0 and LSE = -inf. An Inf or NaN in
 * a later new token's own row never reaches an earlier token (a range whose
 * accumulators turn non-finite is recomputed pair by pair). */
int attn_decode_multi(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* seqlens, void* o, float* lse, int dtype, int B, int n_new,
                      int Hq, int Hkv, int max_len, int d, float scale, int kv_splits,
                      const miattn_strides* cache_strides, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Decode (one or several new tokens per sequence, as attn_decode_multi)
 * against a paged KV cache. The pages name paged caches without fixing a
 * layout ("Attention Mechanism Optimization for Efficient LLM Inference",
 * closing section); this one is:
 *
 * k_pages, v_pages  device, [num_pages, page_size, Hkv, d] bf16 (read); with
 *          page_strides (an array of 2, k then v) "b" is the stride from page
 *          to page, "s" from row to row, "h" from head to head, in elements
 * block_table  device, int32 [B, max_pages]: cached row r of sequence b is
 *          row r % page_size of page block_table[b * max_pages + r / page_size]
 *          (precondition, not checked: entries < num_pages for every row
 *          below seqlens[b]; the library is not told num_pages)
 * seqlens  device, int32 [B], each in [0, page_size * max_pages] (clamped
 *          to that range on the device, as in attn_decode)
 * page_size  a power of two >= 16
 * q, o, lse, n_new, workspace  as in attn_decode_multi (workspace size from
 *          attn_decode_multi_workspace_bytes) */
int attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                      const int32_t* block_table, const int32_t* seqlens, void* o, float* lse,
                      int dtype, int B, int n_new, int Hq, int Hkv, int page_size, int max_pages,
                      int d, float scale, int kv_splits, const miattn_strides* page_strides,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace attn_bwd needs: two fp32 rows of Nq rounded up
 * to 64 per (batch, query head) -- the forward LSE in base-2 units and
 * D_i = dO_i . O_i -- then a 256-byte slot holding a flag. 0 when Nq is 0
 * and for invalid sizes. */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Nq);

/* Backward pass by recomputation ("플래시어텐션: 메모리를 아끼는 정확한 어텐션",
 * §4 재계산): from Q, K, V, the forward output O, its per-row LSE and the
 * upstream gradient dO, the gradients of O = softmax(scale * Q K^T + mask) V
 * with respect to Q, K and V. S and P are rebuilt tile by tile from Q, K, V
 * and the LSE; no N x N matrix is stored. With GQA the gradient of a KV head
 * is the sum over the query heads that read it.
 *
 * q, o, dout  device, [B, Nq, Hq, d] bf16        (read)
 * k, v        device, [B, Nk, Hkv, d] bf16       (read)
 * lse         device, float [B, Hq, Nq]          (read: attn_fwd's LSE for
 *             the same q, k, v and mask, natural log)
 * dq          device, [B, Nq, Hq, d] bf16        (written)
 * dk, dv      device, [B, Nk, Hkv, d] bf16       (written; keys no query
 *             sees get 0)
 * dtype       MIATTN_BF16 (bf16 MFMA inputs, fp32 accumulation; P and dS are
 *             rounded to bf16 for the products that consume them)
 * d           64 or 128
 * scale       > 0 and finite, the forward's scale
 * mask_kind, block_mask, block_q, block_k  the forward's mask, same meaning
 *             and limits as in attn_fwd (block sizes multiples of 16 dividing
 *             Nq and Nk); pairs it excludes get no gradient
 * strides     NULL (packed) or an array of 8: q, k, v, o, dout, dq, dk, dv
 * workspace   device, at least attn_bwd_workspace_bytes(B, Hq, Nq) bytes,
 *             owned by the caller, overwritten by the call
 * stream      hipStream_t
 * A query row with no visible key gets dQ = 0 and adds nothing to dK, dV.
 * Inf or NaN in an input reaches only the gradient entries that a pair the
 * mask allows connects it to: with a mask, a wave whose accumulators turn
 * non-finite sets the workspace flag, and a last kernel then recomputes
 * every gradient row holding an Inf or NaN from the visible pairs alone
 * (slow; only on that path).
 * Outputs must not overlap the inputs. */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int dtype, int B, int Hq,
             int Hkv, int Nq, int Nk, int d, float scale, int mask_kind,
             const uint8_t* block_mask, int block_q, int block_k,
             const miattn_strides* strides, void* workspace, size_t workspace_bytes,
             void* stream);

/* Static description of a status code. */
const char* attn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MIATTN_H */
