/*
 * attn.h -- C ABI of the MI355X (gfx950) causal attention library libattn.so.
 *
 * Computes causal scaled dot-product multi-head attention
 *     O = softmax(Q K^T * scale + M) V        per (batch, query head)
 * with the grouped-query K/V head map, an optional sliding window, the
 * KV-cache decode step, chunked prefill against a cache, the cache append,
 * key-padding masks, rotary position embedding and the backward pass.  The operation is the one defined in the attention chapter of the
 * LLM-architecture textbook ("Механизм внимания", sections "Scaled
 * dot-product attention", "Маскирование", "Виды по числу голов K/V",
 * "Скользящее окно", "KV-кэш", "Prefill и decode" and "Прямой проход по
 * шагам").
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers to dense row-major (contiguous)
 *     buffers owned by the caller.  The library never allocates, frees,
 *     synchronises or keeps a pointer after the call returns; the caller keeps
 *     every buffer alive until the stream has passed the call.  The library's
 *     own device memory is attn_decode_noalloc's fixed scratch array (see
 *     there) and up to 256 sets of 9 work counters per device, one per
 *     stream, for the causal bf16 prefills without a window or cache whose
 *     grid covers the chip four or more times (the last quarter of such a
 *     grid is handed out at run time).  A
 *     stream's launches run one after another, and each launch leaves its
 *     set cleared for the next.  A launch into hipStreamPerThread, into a
 *     stream being captured into a graph or belonging to another device than
 *     the current one, or from a stream beyond the 256th takes a fixed order;
 *     the results are the same bits either way.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *     Work is enqueued asynchronously on it.
 *   - Return value: ATTN_OK (0) or a negative attn_status.  Argument errors
 *     are detected on the host before anything is enqueued and leave the
 *     outputs untouched.  ATTN_EHIP reports a HIP launch error.
 *   - Head map: query head h reads K/V head h / (Nq / Nkv) (integer
 *     division), so consecutive query heads share a K/V head; Nq must be a
 *     multiple of Nkv (MHA: Nkv == Nq, MQA: Nkv == 1).
 *   - Element types: ATTN_BF16 (inputs and O in bfloat16, accumulation in
 *     fp32) or ATTN_F32.  LSE is always fp32.
 *   - The library is re-entrant.  Its state is that scratch array, which
 *     calls of attn_decode_noalloc on one device share, and the per-stream
 *     work-counter sets (their stream map is guarded by a lock).
 */
#ifndef TCH_ATTN_H
#define TCH_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_EINVAL = -1,        /* null pointer, non-positive size, bad flag/scale  */
  ATTN_EGQA = -2,          /* Nq is not a multiple of Nkv                      */
  ATTN_EUNSUPPORTED = -3,  /* dtype or head size outside what is implemented,
                              or a head too long for the bf16 MFMA kernels      */
  ATTN_EWORKSPACE = -4,    /* workspace missing or smaller than required       */
  ATTN_EHIP = -5,          /* HIP runtime reported an error at launch          */
  ATTN_ESCRATCH = -6       /* attn_decode_noalloc: the call needs more scratch
                              than ATTN_NOALLOC_SCRATCH_BYTES                   */
} attn_status;

typedef enum { ATTN_BF16 = 0, ATTN_F32 = 1 } attn_dtype;

/*
 * attn_prefill -- attention of S queries against the same S keys.
 *
 *   Q   [B, Nq,  S, Dh]   queries
 *   K   [B, Nkv, S, Dh]   keys
 *   V   [B, Nkv, S, Dh]   values
 *   O   [B, Nq,  S, Dh]   output, same element type as Q
 *   LSE [B, Nq,  S]       fp32 natural-log log-sum-exp of the scaled, masked
 *                         score row (m + ln l); may be NULL
 *   causal   1: query i sees keys j <= i (mask aligned at the top-left);
 *            0: every key is visible
 *   window   <= 0: no window; > 0: query i sees only keys with i - j < window,
 *            i.e. keys max(0, i-window+1) .. i; requires causal == 1
 *   scale    multiplier of Q K^T; > 0 and finite.  The standard definition
 *            uses 1/sqrt(Dh) (the head size).
 *   dtype    attn_dtype of Q, K, V and O.
 * Supported: Dh in 1..256 for both dtypes; bf16 with Dh in {64, 128, 256}
 * takes the MFMA kernel, the rest a general kernel.  B, Nq, Nkv, S >= 1.
 * The MFMA kernel addresses one head through a 31-bit byte range: it needs
 * S * Dh * 2 < 2^31 (S <= 8388607 at Dh = 128); longer heads return
 * ATTN_EUNSUPPORTED before anything is launched.
 * Errors: ATTN_EINVAL, ATTN_EGQA, ATTN_EUNSUPPORTED, ATTN_EHIP.
 */
int attn_prefill(const void* Q, const void* K, const void* V, void* O, float* LSE,
                 int B, int Nq, int Nkv, int S, int Dh,
                 int causal, int window, float scale,
                 int dtype, void* stream);

/*
 * attn_prefill_cache -- chunked prefill: Sq new queries per sequence against
 * a KV cache that already holds their keys (textbook, "Prefill и decode": a
 * long prompt filled chunk by chunk, with the causal mask inside the chunk;
 * "Прямой проход по шагам": mask rows start at the first new position).
 *
 *   Q       [B, Nq, Sq, Dh]      the chunk's queries
 *   Kcache  [B, Nkv, Tcap, Dh]   keys; rows 0 .. lens[b]-1 hold sequence b's
 *                                keys, the chunk's own Sq keys last
 *   Vcache  [B, Nkv, Tcap, Dh]   values, same layout
 *   lens    [B] int32, DEVICE    keys of each sequence including the chunk;
 *                                must satisfy Sq <= lens[b] <= Tcap
 *   O       [B, Nq, Sq, Dh]      output, same element type as Q
 *   LSE     [B, Nq, Sq] fp32 or NULL
 *   window   <= 0: none; > 0: only keys with pos - j < window are visible
 *   scale    > 0 and finite (1/sqrt(Dh) for the standard definition)
 * Query i of sequence b sits at position lens[b] - Sq + i (the mask is aligned
 * at the bottom-right corner) and sees keys j <= its position.  Cache rows at
 * or past lens[b] are never read.  With Sq == lens[b] this is attn_prefill.
 * lens lives on the device: values above Tcap are clamped to Tcap, and a
 * value below Sq leaves rows with no visible key (NaN).
 * Supported: as attn_prefill (bf16 Dh in {64, 128, 256} takes the MFMA kernel,
 * which needs Tcap * Dh * 2 < 2^31, else ATTN_EUNSUPPORTED).
 * Errors: ATTN_EINVAL (also Sq > Tcap), ATTN_EGQA, ATTN_EUNSUPPORTED, ATTN_EHIP.
 */
int attn_prefill_cache(const void* Q, const void* Kcache, const void* Vcache,
                       const int32_t* lens, void* O, float* LSE,
                       int B, int Nq, int Nkv, int Sq, int Dh, int Tcap,
                       int window, float scale, int dtype, void* stream);

/*
 * attn_decode_workspace_bytes -- bytes of device workspace attn_decode needs
 * for these dimensions (0 when the chosen kernel needs none).  Pure host
 * function; returns 0 for invalid arguments.
 */
size_t attn_decode_workspace_bytes(int B, int Nq, int Nkv, int Dh, int Tcap, int dtype);

/*
 * attn_decode -- one generation step: each sequence's single new query row
 * against its KV cache (the textbook's decode phase: a 1 x t score row).
 *
 *   q       [B, Nq, Dh]          the new token's queries
 *   Kcache  [B, Nkv, Tcap, Dh]   keys; rows 0 .. lens[b]-1 of sequence b hold
 *                                its cached keys, the new token's included
 *   Vcache  [B, Nkv, Tcap, Dh]   values, same layout
 *   lens    [B] int32, DEVICE    cached length of each sequence, counting the
 *                                new token; must satisfy 1 <= lens[b] <= Tcap
 *   O       [B, Nq, Dh]          output, same element type as q
 *   LSE     [B, Nq] fp32 or NULL
 *   workspace / workspace_bytes  device scratch of at least
 *                                attn_decode_workspace_bytes(...) bytes
 *                                (may be NULL when that is 0)
 * The scale is 1/sqrt(Dh).  No mask applies beyond the length; cache rows at
 * or past lens[b] are never read.  bf16 with Dh in {64, 128, 256} and at most
 * 32 query heads per K/V head takes the split-K MFMA kernels (and needs the
 * workspace); other shapes take a general kernel.
 * lens lives on the device, so the host cannot check it: a value above Tcap
 * is clamped to Tcap, and a value below 1 yields a NaN output row.
 * Errors: ATTN_EINVAL, ATTN_EGQA, ATTN_EUNSUPPORTED, ATTN_EWORKSPACE, ATTN_EHIP.
 */
int attn_decode(const void* q, const void* Kcache, const void* Vcache,
                const int32_t* lens, void* O,
                int B, int Nq, int Nkv, int Dh, int Tcap,
                float* LSE, void* workspace, size_t workspace_bytes,
                int dtype, void* stream);

/*
 * attn_decode_noalloc -- attn_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without the workspace, the same
 * kernels and the same result bit for bit.  The split-K partials go to a
 * scratch array of ATTN_NOALLOC_SCRATCH_BYTES that the library holds on each
 * device it runs on, from the first call on that device until the process
 * ends; the call itself allocates and frees nothing.
 *   Limit: attn_decode_workspace_bytes(B, Nq, Nkv, Dh, Tcap, dtype) must not
 *   exceed ATTN_NOALLOC_SCRATCH_BYTES (the 64-sequence, 32/8-head, 32768-slot
 *   cache at Dh 128 needs 20.2 MB); larger calls return ATTN_ESCRATCH before
 *   anything is enqueued.  Shapes that need no workspace (fp32, the general
 *   kernel) use no scratch.
 *   Concurrency: every call on one device shares that device's scratch and
 *   leaves its contents behind (nothing in it needs clearing: each call
 *   writes every partial it reads).  Calls that overlap on one device -- on
 *   two streams, or from two host threads without ordering -- race on it;
 *   order them on one stream.
 * Errors: as attn_decode, with ATTN_ESCRATCH in place of ATTN_EWORKSPACE.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int attn_decode_noalloc(const void* q, const void* Kcache, const void* Vcache,
                        const int32_t* lens, void* O,
                        int B, int Nq, int Nkv, int Dh, int Tcap,
                        float* LSE, int dtype, void* stream);

/*
 * attn_decode_window -- attn_decode with a sliding window and an explicit
 * scale (textbook, "Скользящее окно": with a window the new token sees only
 * the recent past).  Arguments as attn_decode, plus
 *   window   <= 0: every cached key; > 0: keys lens[b]-window .. lens[b]-1
 *   scale    > 0 and finite
 * The workspace must hold attn_decode_window_workspace_bytes(..., window, ...)
 * bytes (a short window splits into shorter chunks, so the size depends on it).
 * A rolling-buffer cache of capacity W (see attn_kv_append) holds exactly
 * the last W positions in some slot order; the softmax does not depend on
 * that order, so it is decoded with lens = min(position + 1, W) and no
 * window.
 * Errors: as attn_decode.
 */
int attn_decode_window(const void* q, const void* Kcache, const void* Vcache,
                       const int32_t* lens, void* O,
                       int B, int Nq, int Nkv, int Dh, int Tcap, int window, float scale,
                       float* LSE, void* workspace, size_t workspace_bytes,
                       int dtype, void* stream);

/*
 * attn_decode_window_workspace_bytes -- bytes of device workspace
 * attn_decode_window needs for these dimensions and this window (0 when the
 * chosen kernel needs none; window <= 0 gives attn_decode_workspace_bytes).
 * Pure host function; returns 0 for invalid arguments.
 */
size_t attn_decode_window_workspace_bytes(int B, int Nq, int Nkv, int Dh, int Tcap, int window,
                                          int dtype);

/*
 * attn_kv_append -- write the new tokens' K and V rows into the caches
 * (textbook, "Прямой проход по шагам": the new K and V follow the cached
 * ones; "Скользящее окно": a cache bounded by the window keeps only the last
 * positions -- Mistral's rolling buffer).
 *
 *   Knew, Vnew      [B, Nkv, Snew, Dh]   new rows
 *   Kcache, Vcache  [B, Nkv, Tcap, Dh]   caches, updated in place
 *   pos     [B] int32, DEVICE   position of each sequence's first new token
 *                               (its token count before the append)
 *   rolling  0: row i goes to cache row pos[b] + i, which must be < Tcap;
 *            1: row i goes to row (pos[b] + i) mod Tcap; when Snew > Tcap
 *            only the last Tcap new rows are written
 *   dtype    element type of all four buffers
 * The caller updates its own lengths afterwards.  pos lives on the device: a
 * negative value skips that sequence, and linear rows that would land at or
 * past Tcap are dropped.
 * Errors: ATTN_EINVAL (also rolling == 0 with Snew > Tcap), ATTN_EUNSUPPORTED
 * (dtype, Dh > 256), ATTN_EHIP.
 */
int attn_kv_append(const void* Knew, const void* Vnew, void* Kcache, void* Vcache,
                   const int32_t* pos, int B, int Nkv, int Snew, int Dh, int Tcap,
                   int rolling, int dtype, void* stream);

/*
 * attn_backward_workspace_bytes -- bytes of device workspace attn_backward
 * and attn_backward_padded need (two fp32 per query row: dO . O and the LSE
 * in log2 units).  Pure host function; 0 for invalid arguments.
 */
size_t attn_backward_workspace_bytes(int B, int Nq, int Nkv, int S, int Dh, int dtype);

/*
 * attn_backward -- gradients of attn_prefill's output with respect to Q, K and
 * V (training).  The weights are recomputed from the stored LSE instead of
 * being read (textbook, "Эффективные реализации": FlashAttention recomputes
 * the weight matrix by blocks on the backward pass); the softmax Jacobian is
 * p_i (delta_ij - p_j) ("Почему делить на корень из d_h").  With
 * P = exp(scale Q K^T + M - LSE):
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),
 *   dQ = scale dS K,  dK = scale dS^T Q;
 * a K/V head shared by G query heads receives the sum of their gradients.
 *
 *   Q, O, dO, dQ  [B, Nq,  S, Dh]   forward input, forward output, dL/dO, dL/dQ
 *   K, V, dK, dV  [B, Nkv, S, Dh]   forward inputs and their gradients
 *   LSE           [B, Nq,  S] fp32  the LSE attn_prefill returned for this O
 *   causal, window, scale, dtype    as passed to attn_prefill
 *   workspace / workspace_bytes     device scratch of at least
 *                                   attn_backward_workspace_bytes(...) bytes
 * dQ, dK, dV are written in the element type of the inputs (accumulation in
 * fp32); they are overwritten, not accumulated into.  bf16 with Dh 64, 128 or
 * 256 runs the MFMA kernels, which need S * Dh * 2 < 2^31 (else
 * ATTN_EUNSUPPORTED).
 * Errors: ATTN_EINVAL, ATTN_EGQA, ATTN_EUNSUPPORTED, ATTN_EWORKSPACE, ATTN_EHIP.
 */
int attn_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                  const float* LSE, void* dQ, void* dK, void* dV,
                  int B, int Nq, int Nkv, int S, int Dh,
                  int causal, int window, float scale,
                  void* workspace, size_t workspace_bytes, int dtype, void* stream);

/*
 * attn_backward_padded -- attn_backward for a forward pass that ran with a
 * key-padding mask (attn_prefill_padded, textbook "Паддинг"): the same
 * key_bits [B, ceil(S / 64)] uint64, DEVICE, bit j % 64 of word j / 64 set
 * for a real key j.  A padding key has weight 0 in every row, so its dK and
 * dV rows are 0; a query row that saw no key (LSE = -inf, O = 0) passes no
 * gradient and gets dQ = 0.  key_bits == NULL is attn_backward.  Every other
 * argument, the workspace and the errors are those of attn_backward.
 */
int attn_backward_padded(const void* Q, const void* K, const void* V, const uint64_t* key_bits,
                         const void* O, const void* dO, const float* LSE, void* dQ, void* dK,
                         void* dV, int B, int Nq, int Nkv, int S, int Dh, int causal,
                         int window, float scale, void* workspace, size_t workspace_bytes,
                         int dtype, void* stream);

/*
 * attn_decode_append -- one decode step that also appends the new token's K
 * and V (textbook, "Prefill и decode" and the generation walk-through: each
 * step appends k, v to the cache and then attends over it), in one launch on
 * the bf16 split-K path: the new rows are written to cache row slot[b] and the
 * chunk that holds that row reads them from knew / vnew.
 *
 *   knew, vnew [B, Nkv, Dh]   the new token's K and V rows (already rotated,
 *                             when RoPE is used)
 *   slot [B] int32, DEVICE    cache row of the new token: lens[b] - 1 for a
 *                             linear cache, position mod Tcap for a rolling
 *                             buffer; rows outside [0, Tcap) are not written
 *   lens [B] int32, DEVICE    keys the query sees, counting the new one
 * The query must see row slot[b] (lens[b] - window <= slot[b] < lens[b]) for
 * its own key to enter the softmax.  Every other argument, the workspace
 * (attn_decode_window_workspace_bytes) and the errors are those of
 * attn_decode_window.  fp32, head sizes other than 64/128/256, more than 32
 * query heads per K/V head, or new rows not 16-byte aligned take two launches
 * (attn_kv_append's kernel, then the decode) with the same result.
 */
int attn_decode_append(const void* q, const void* knew, const void* vnew, void* Kcache,
                       void* Vcache, const int32_t* lens, const int32_t* slot, void* O,
                       int B, int Nq, int Nkv, int Dh, int Tcap, int window, float scale,
                       float* LSE, void* workspace, size_t workspace_bytes, int dtype,
                       void* stream);

/*
 * Key-padding masks (textbook, "Паддинг" under "Прямой проход по шагам": the
 * padding's key mask is added to the causal mask and the window, one mask per
 * batch row).  The attention entry points below take the mask as BITS: for a
 * sequence of T keys (T = S for a prefill, Tcap for a cache) its row holds
 * ceil(T / 64) uint64 words, and bit j % 64 of word j / 64 is key j's flag
 * (1 = real token, 0 = padding).  A hidden key gets weight exactly 0, so its
 * K and V must still hold finite values.  A query row that sees no key at all
 * (a left-padding query, say) gets O = 0 and LSE = -inf.
 *
 * attn_pack_key_mask -- bytes -> bits.
 *   mask      [B, T] uint8, DEVICE   nonzero = real token
 *   key_bits  [B, ceil(T / 64)] uint64, DEVICE, written
 * Errors: ATTN_EINVAL, ATTN_EHIP.
 */
int attn_pack_key_mask(const uint8_t* mask, int B, int T, uint64_t* key_bits, void* stream);

/*
 * attn_prefill_padded / attn_prefill_cache_padded / attn_decode_padded --
 * attn_prefill, attn_prefill_cache and attn_decode_window with a key-padding
 * mask, key_bits [B, ceil(S / 64)] (prefill) or [B, ceil(Tcap / 64)] (the
 * cache forms, indexed by cache row), DEVICE.  key_bits == NULL is the
 * unmasked call.  Every other argument, the workspace size and the errors
 * are those of the unpadded entry point.
 */
int attn_prefill_padded(const void* Q, const void* K, const void* V, const uint64_t* key_bits,
                        void* O, float* LSE, int B, int Nq, int Nkv, int S, int Dh,
                        int causal, int window, float scale, int dtype, void* stream);
int attn_prefill_cache_padded(const void* Q, const void* Kcache, const void* Vcache,
                              const int32_t* lens, const uint64_t* key_bits, void* O, float* LSE,
                              int B, int Nq, int Nkv, int Sq, int Dh, int Tcap, int window,
                              float scale, int dtype, void* stream);
int attn_decode_padded(const void* q, const void* Kcache, const void* Vcache,
                       const int32_t* lens, const uint64_t* key_bits, void* O,
                       int B, int Nq, int Nkv, int Dh, int Tcap, int window, float scale,
                       float* LSE, void* workspace, size_t workspace_bytes,
                       int dtype, void* stream);

/*
 * Rotary position embedding, RoPE (textbook, "Как в attention попадает
 * позиция": q and k are rotated by a position-dependent angle so that
 * q_i . k_j depends only on i - j, V is not; step 4 of "Прямой проход по
 * шагам": with padding the rotation takes explicit positions; the layer-cache
 * section: K enters the cache already rotated).  The formula is RoFormer's,
 * which the page cites: pair m is turned by p * theta_m, theta_m =
 * base^(-2m/Dh), (a, b) -> (a cos - b sin, a sin + b cos).
 *
 * attn_rope_cos_sin -- build the angle table.
 *   table [P, Dh] fp32, DEVICE, written: column m holds cos(p theta_m),
 *         column Dh/2 + m holds sin(p theta_m), for positions p = 0 .. P-1
 *   base  > 1 (10000 in RoFormer and LLaMA); Dh even
 * Computed in double precision and rounded once to fp32.
 * Errors: ATTN_EINVAL, ATTN_EHIP.
 */
int attn_rope_cos_sin(float* table, int P, int Dh, double base, void* stream);

/*
 * attn_rope -- rotate X [B, H, S, Dh] into Y (Y == X allowed: in place).
 *   positions [B, S] int32, DEVICE, or NULL: token (b, s) is at positions[b, s]
 *   start     [B] int32, DEVICE, or NULL: with positions NULL, token (b, s) is
 *             at start[b] + s (the first new token's position), or at s
 *   table     from attn_rope_cos_sin with this Dh; positions are clamped to
 *             [0, P - 1]
 *   style     0: pairs (x[2m], x[2m+1]) (RoFormer);
 *             1: halves (x[m], x[m + Dh/2]) (GPT-NeoX, LLaMA in the Hugging
 *             Face layout)
 *   dtype     of X and Y; the rotation is computed in fp32
 * Errors: ATTN_EINVAL (also odd Dh, bad style), ATTN_EUNSUPPORTED, ATTN_EHIP.
 */
int attn_rope(const void* X, void* Y, const int32_t* positions, const int32_t* start,
              const float* table, int P, int B, int H, int S, int Dh, int style, int dtype,
              void* stream);

/*
 * attn_kv_append_rope -- attn_kv_append with the new keys rotated on their
 * way into the cache (one pass over the new rows): key row i of sequence b is
 * rotated at positions[b, i] ([B, Snew] int32, DEVICE) or, with positions
 * NULL, at pos[b] + i, then written where attn_kv_append writes it; V rows are
 * copied unchanged.  table, P, style as for attn_rope; the rest as for
 * attn_kv_append.
 * Errors: ATTN_EINVAL, ATTN_EUNSUPPORTED, ATTN_EHIP.
 */
int attn_kv_append_rope(const void* Knew, const void* Vnew, void* Kcache, void* Vcache,
                        const int32_t* pos, const int32_t* positions, const float* table, int P,
                        int B, int Nkv, int Snew, int Dh, int Tcap, int rolling, int style,
                        int dtype, void* stream);

/*
 * Attention with the queries rotated as they are loaded (RoPE fused into the
 * attention step: the textbook's "Как в attention попадает позиция" and
 * step 4 of "Прямой проход по шагам" -- q and k are turned before their dot
 * product).  The keys must already be rotated: by attn_kv_append_rope on
 * their way into a cache, or by attn_rope for a plain prefill.  Each entry
 * point takes the arguments of its unrotated form (with a key-padding mask,
 * NULL for none), plus
 *   table, P   the angle table from attn_rope_cos_sin ([P, Dh] fp32, DEVICE)
 *   positions  DEVICE int32, or NULL: the rotation position of each query
 *              row -- [B, S] (prefill), [B, Sq] (chunked prefill), [B] (decode)
 *   start      DEVICE int32 [B], or NULL (prefill forms only): with positions
 *              NULL, query row i of sequence b is at start[b] + i
 *   style      0: pairs (x[2m], x[2m+1]); 1: halves (x[m], x[m + Dh/2])
 * Without positions and start a query row is turned at its own position:
 * row i of a prefill at i, row i of a chunk at lens[b] - Sq + i, a decode
 * step's query at lens[b] - 1 (a rolling-buffer cache passes its positions).
 * Positions are clamped to [0, P - 1].  The rotation is the one attn_rope
 * computes (fp32, rounded once to the input type), so the result is that of
 * attn_rope on q followed by the unrotated call, without the extra pass over
 * q.  Errors: those of the unrotated form, and ATTN_EINVAL for a NULL table,
 * P < 1, an odd Dh or a bad style.
 */
int attn_prefill_rope(const void* Q, const void* K, const void* V, const uint64_t* key_bits,
                      void* O, float* LSE, int B, int Nq, int Nkv, int S, int Dh, int causal,
                      int window, float scale, const float* table, int P,
                      const int32_t* positions, const int32_t* start, int style, int dtype,
                      void* stream);
int attn_prefill_cache_rope(const void* Q, const void* Kcache, const void* Vcache,
                            const int32_t* lens, const uint64_t* key_bits, void* O, float* LSE,
                            int B, int Nq, int Nkv, int Sq, int Dh, int Tcap, int window,
                            float scale, const float* table, int P, const int32_t* positions,
                            const int32_t* start, int style, int dtype, void* stream);
int attn_decode_rope(const void* q, const void* Kcache, const void* Vcache, const int32_t* lens,
                     const uint64_t* key_bits, void* O, int B, int Nq, int Nkv, int Dh, int Tcap,
                     int window, float scale, const float* table, int P,
                     const int32_t* positions, int style, float* LSE, void* workspace,
                     size_t workspace_bytes, int dtype, void* stream);

/* attn_strerror -- static description of an attn_status value. */
const char* attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* TCH_ATTN_H */
