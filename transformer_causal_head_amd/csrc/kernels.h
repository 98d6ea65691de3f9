// Internal launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// Rotation of the queries (RoPE) applied by the attention kernels as they
// load q: table [P, Dh] fp32 (cos in columns 0 .. Dh/2 - 1, sin after),
// style 0 pairs (x[2m], x[2m+1]), 1 halves (x[m], x[m + Dh/2]).  Query row i
// of sequence b is turned at positions[b * rows + i] when positions is given,
// else at start[b] + i when start is given, else at the row's own position
// (i for a prefill, lens[b] - rows + i against a cache, lens[b] - 1 for a
// decode step), clamped to [0, P - 1].  Same fp32 arithmetic and rounding to
// the input type as launch_rope, so the attention sees the same q bits.
struct RopeQ {
  const float* table;
  int P;
  const int32_t* positions;
  const int32_t* start;
  int style;
};

// Key-padding masks are passed as bits: word j / 64 of a sequence's row holds
// key j at bit j % 64 (1 = a real token); a row of T keys has this many words.
inline int key_mask_words(int T) { return (T + 63) / 64; }

// bf16 MFMA prefill, head size 64, 128 or 256.  S query rows per head; K/V
// heads of kv_rows rows.  lens == nullptr: plain prefill (S keys, query i at
// position i).  Otherwise sequence b has lens[b] keys and query i sits at
// position lens[b] - S + i (chunked prefill against a cache).  kbits: key-
// padding mask over the kv_rows keys of each sequence, or nullptr.
bool prefill_bf16_supported(int Dh);
hipError_t launch_prefill_bf16(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               int B, int Nq, int Nkv, int S, int Dh, int kv_rows,
                               const int32_t* lens, const uint64_t* kbits, int causal, int window,
                               float scale, hipStream_t stream, const RopeQ* rope = nullptr);

// General row kernel: one wavefront per output row (b, h, i), any Dh in
// 1..256, bf16 (is_bf16 = 1) or fp32.  Same row/key convention as the MFMA
// prefill; a decode step is S = 1 with lens (its query sees keys
// lens[b] - window .. lens[b] - 1, or all of them without a window).
hipError_t launch_rows_general(const void* Q, const void* K, const void* V, void* O,
                               float* LSE, int B, int Nq, int Nkv, int S, int Dh,
                               int kv_rows, const int32_t* lens, const uint64_t* kbits,
                               int causal, int window, float scale, int is_bf16,
                               hipStream_t stream, const RopeQ* rope = nullptr);

// bf16 split-K decode (partials + log-sum-exp merge), head size 64, 128 or
// 256, up to 32 query heads per K/V head.  The query of sequence b sees keys
// max(0, lens[b] - window) .. lens[b] - 1 (window 0: all of them).
bool decode_bf16_supported(int Nq, int Nkv, int Dh);
int decode_bf16_chunk(int B, int Nkv, int L, int G);
size_t decode_bf16_workspace(int B, int Nq, int Nkv, int Dh, int Tcap, int window);
// With knew / vnew / slot (no key mask then): the new token's K and V rows
// [B, Nkv, Dh] are written to cache row slot[b] in the same launch (16-byte
// aligned rows), and the chunk that holds that row reads them from knew/vnew.
hipError_t launch_decode_bf16(const void* q, const void* Kc, const void* Vc, const int32_t* lens,
                              void* O, float* LSE, int B, int Nq, int Nkv, int Dh, int Tcap,
                              int window, float scale, const uint64_t* kbits, void* ws,
                              hipStream_t stream, const void* knew = nullptr,
                              const void* vnew = nullptr, const int32_t* slot = nullptr,
                              const RopeQ* rope = nullptr);

// The allocation-free decode's fixed device scratch: its size, and its address
// on the current device (looked up on the first call per device).
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
hipError_t decode_scratch(void** ptr);

// Copy Snew new K and V rows per (sequence, K/V head) into the caches at
// positions pos[b] .. pos[b] + Snew - 1, or at those positions modulo Tcap
// (rolling buffer).  elem_bytes: 2 (bf16) or 4 (fp32).
hipError_t launch_kv_append(const void* Knew, const void* Vnew, void* Kc, void* Vc,
                            const int32_t* pos, int B, int Nkv, int Snew, int Dh, int Tcap,
                            int rolling, int elem_bytes, hipStream_t stream);

// bytes (nonzero = real token) [B, T] -> bits [B, key_mask_words(T)]
hipError_t launch_pack_key_mask(const uint8_t* mask, int B, int T, uint64_t* bits,
                                hipStream_t stream);

// RoPE: cos/sin table [P, Dh] (cos of p * base^(-2m/Dh) in column m, sin in
// column Dh/2 + m); rotation of X [B, H, S, Dh] into Y (may alias X) at
// positions[b, s], or start[b] + s, or s; style 0: pairs (2m, 2m+1), 1:
// halves (m, m + Dh/2).  Positions are clamped to [0, P).
hipError_t launch_rope_table(float* table, int P, int Dh, double base, hipStream_t stream);
hipError_t launch_rope(const void* X, void* Y, const int32_t* positions, const int32_t* start,
                       const float* table, int P, int B, int H, int S, int Dh, int style,
                       int elem_bytes, hipStream_t stream);
// launch_kv_append with the new K rows rotated (at positions[b, i], or
// pos[b] + i) on their way into the cache; V rows copied unchanged
hipError_t launch_kv_append_rope(const void* Knew, const void* Vnew, void* Kc, void* Vc,
                                 const int32_t* pos, const int32_t* positions, const float* table,
                                 int P, int B, int Nkv, int Snew, int Dh, int Tcap, int rolling,
                                 int style, int elem_bytes, hipStream_t stream);

// Backward pass of prefill attention.  The workspace holds Delta
// [B, Nq, S] fp32 (dO . O per row), then the rows' LSE in log2 units
// [B, Nq, S] fp32 (+inf for a row that saw no key).  kbits: key-padding mask
// [B, key_mask_words(S)] or null.
size_t backward_workspace(int B, int Nq, int S);
hipError_t launch_backward_general(const void* Q, const void* K, const void* V, const void* O,
                                   const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                                   int B, int Nq, int Nkv, int S, int Dh, int causal, int window,
                                   float scale, void* ws, int is_bf16, const uint64_t* kbits,
                                   hipStream_t stream);
// Delta_i = dO_i . O_i for `rows` rows of Dh elements (and, if lse2 is not
// null, lse2_i = LSE_i log2(e), +inf where LSE_i = -inf)
hipError_t launch_backward_delta(const void* O, const void* dO, const float* LSE, float* delta,
                                 float* lse2, long long rows, int Dh, int is_bf16,
                                 hipStream_t stream);
// bf16 MFMA backward (Dh 64, 128 or 256): Delta, then the dQ and dK/dV kernels
bool backward_bf16_supported(int Dh);
hipError_t launch_backward_bf16(const void* Q, const void* K, const void* V, const void* O,
                                const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                                int B, int Nq, int Nkv, int S, int Dh, int causal, int window,
                                float scale, void* ws, const uint64_t* kbits, hipStream_t stream);

}  // namespace attn
