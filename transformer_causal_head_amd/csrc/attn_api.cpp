// C ABI of libattn.so: argument validation, kernel choice, launch.
// Every check runs on the host before anything is enqueued.

#include <hip/hip_runtime.h>
#include <math.h>

#include "../../include/attn.h"
#include "kernels.h"

namespace {

bool positive(int x) { return x > 0; }

int validate_common(int B, int Nq, int Nkv, int Dh, int dtype) {
  if (!positive(B) || !positive(Nq) || !positive(Nkv) || !positive(Dh)) return ATTN_EINVAL;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_EUNSUPPORTED;
  if (Nq % Nkv != 0) return ATTN_EGQA;
  if (Dh > 256) return ATTN_EUNSUPPORTED;
  return ATTN_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_EHIP; }

// The bf16 MFMA kernels address one head of a tensor (rows x Dh bf16 values)
// through a buffer descriptor with a 31-bit byte range.
bool mfma_head_fits(long long rows, int Dh) { return rows * Dh * 2 <= 0x7fffffffLL; }

}  // namespace

// rotation arguments of the _rope entry points: a table, its rows, a style
static int validate_rope(const float* table, int P, int Dh, int style) {
  if (!table || !positive(P) || Dh % 2 != 0 || (style != 0 && style != 1)) return ATTN_EINVAL;
  return ATTN_OK;
}

static int prefill_impl(const void* Q, const void* K, const void* V, const uint64_t* kbits,
                        void* O, float* LSE, int B, int Nq, int Nkv, int S, int Dh, int causal,
                        int window, float scale, int dtype, void* stream,
                        const attn::RopeQ* rope = nullptr) {
  if (!Q || !K || !V || !O) return ATTN_EINVAL;
  int st = validate_common(B, Nq, Nkv, Dh, dtype);
  if (st != ATTN_OK) return st;
  if (!positive(S)) return ATTN_EINVAL;
  if (causal != 0 && causal != 1) return ATTN_EINVAL;
  if (window > 0 && !causal) return ATTN_EINVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return ATTN_EINVAL;
  if (window < 0) window = 0;
  if (dtype == ATTN_BF16 && attn::prefill_bf16_supported(Dh) && !mfma_head_fits(S, Dh))
    return ATTN_EUNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == ATTN_BF16 && attn::prefill_bf16_supported(Dh))
    return from_hip(attn::launch_prefill_bf16(Q, K, V, O, LSE, B, Nq, Nkv, S, Dh, S, nullptr,
                                              kbits, causal, window, scale, s, rope));
  return from_hip(attn::launch_rows_general(Q, K, V, O, LSE, B, Nq, Nkv, S, Dh, S, nullptr,
                                            kbits, causal, window, scale, dtype == ATTN_BF16, s,
                                            rope));
}

static int prefill_cache_impl(const void* Q, const void* Kcache, const void* Vcache,
                              const int32_t* lens, const uint64_t* kbits, void* O, float* LSE,
                              int B, int Nq, int Nkv, int Sq, int Dh, int Tcap, int window,
                              float scale, int dtype, void* stream,
                              const attn::RopeQ* rope = nullptr) {
  if (!Q || !Kcache || !Vcache || !lens || !O) return ATTN_EINVAL;
  int st = validate_common(B, Nq, Nkv, Dh, dtype);
  if (st != ATTN_OK) return st;
  if (!positive(Sq) || !positive(Tcap) || Sq > Tcap) return ATTN_EINVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return ATTN_EINVAL;
  if (window < 0) window = 0;
  if (dtype == ATTN_BF16 && attn::prefill_bf16_supported(Dh) && !mfma_head_fits(Tcap, Dh))
    return ATTN_EUNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == ATTN_BF16 && attn::prefill_bf16_supported(Dh))
    return from_hip(attn::launch_prefill_bf16(Q, Kcache, Vcache, O, LSE, B, Nq, Nkv, Sq, Dh,
                                              Tcap, lens, kbits, 1, window, scale, s, rope));
  return from_hip(attn::launch_rows_general(Q, Kcache, Vcache, O, LSE, B, Nq, Nkv, Sq, Dh, Tcap,
                                            lens, kbits, 1, window, scale, dtype == ATTN_BF16, s,
                                            rope));
}

extern "C" {

int attn_prefill(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                 int Nq, int Nkv, int S, int Dh, int causal, int window, float scale,
                 int dtype, void* stream) {
  return prefill_impl(Q, K, V, nullptr, O, LSE, B, Nq, Nkv, S, Dh, causal, window, scale, dtype,
                      stream);
}

int attn_prefill_padded(const void* Q, const void* K, const void* V, const uint64_t* key_bits,
                        void* O, float* LSE, int B, int Nq, int Nkv, int S, int Dh, int causal,
                        int window, float scale, int dtype, void* stream) {
  return prefill_impl(Q, K, V, key_bits, O, LSE, B, Nq, Nkv, S, Dh, causal, window, scale, dtype,
                      stream);
}

int attn_prefill_cache(const void* Q, const void* Kcache, const void* Vcache,
                       const int32_t* lens, void* O, float* LSE, int B, int Nq, int Nkv,
                       int Sq, int Dh, int Tcap, int window, float scale, int dtype,
                       void* stream) {
  return prefill_cache_impl(Q, Kcache, Vcache, lens, nullptr, O, LSE, B, Nq, Nkv, Sq, Dh, Tcap,
                            window, scale, dtype, stream);
}

int attn_prefill_cache_padded(const void* Q, const void* Kcache, const void* Vcache,
                              const int32_t* lens, const uint64_t* key_bits, void* O, float* LSE,
                              int B, int Nq, int Nkv, int Sq, int Dh, int Tcap, int window,
                              float scale, int dtype, void* stream) {
  return prefill_cache_impl(Q, Kcache, Vcache, lens, key_bits, O, LSE, B, Nq, Nkv, Sq, Dh, Tcap,
                            window, scale, dtype, stream);
}

size_t attn_decode_window_workspace_bytes(int B, int Nq, int Nkv, int Dh, int Tcap, int window,
                                          int dtype) {
  if (validate_common(B, Nq, Nkv, Dh, dtype) != ATTN_OK || !positive(Tcap)) return 0;
  if (dtype == ATTN_BF16 && attn::decode_bf16_supported(Nq, Nkv, Dh))
    return attn::decode_bf16_workspace(B, Nq, Nkv, Dh, Tcap, window > 0 ? window : 0);
  return 0;
}

size_t attn_decode_workspace_bytes(int B, int Nq, int Nkv, int Dh, int Tcap, int dtype) {
  return attn_decode_window_workspace_bytes(B, Nq, Nkv, Dh, Tcap, 0, dtype);
}

static int decode_check(const void* q, const void* Kcache, const void* Vcache,
                        const int32_t* lens, const void* O, int B, int Nq, int Nkv, int Dh,
                        int Tcap, float scale, int dtype) {
  if (!q || !Kcache || !Vcache || !lens || !O) return ATTN_EINVAL;
  int st = validate_common(B, Nq, Nkv, Dh, dtype);
  if (st != ATTN_OK) return st;
  if (!positive(Tcap)) return ATTN_EINVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return ATTN_EINVAL;
  return ATTN_OK;
}

static int decode_impl(const void* q, const void* Kcache, const void* Vcache,
                       const int32_t* lens, const uint64_t* kbits, void* O, int B, int Nq,
                       int Nkv, int Dh, int Tcap,
                       int window, float scale, float* LSE, void* workspace,
                       size_t workspace_bytes, int dtype, void* stream,
                       const attn::RopeQ* rope = nullptr) {
  int st = decode_check(q, Kcache, Vcache, lens, O, B, Nq, Nkv, Dh, Tcap, scale, dtype);
  if (st != ATTN_OK) return st;
  if (window < 0) window = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t need = attn_decode_window_workspace_bytes(B, Nq, Nkv, Dh, Tcap, window, dtype);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return ATTN_EWORKSPACE;
    return from_hip(attn::launch_decode_bf16(q, Kcache, Vcache, lens, O, LSE, B, Nq, Nkv, Dh,
                                             Tcap, window, scale, kbits, workspace, s, nullptr,
                                             nullptr, nullptr, rope));
  }
  return from_hip(attn::launch_rows_general(q, Kcache, Vcache, O, LSE, B, Nq, Nkv, 1, Dh, Tcap,
                                            lens, kbits, 1, window, scale, dtype == ATTN_BF16, s,
                                            rope));
}

int attn_decode(const void* q, const void* Kcache, const void* Vcache, const int32_t* lens,
                void* O, int B, int Nq, int Nkv, int Dh, int Tcap, float* LSE, void* workspace,
                size_t workspace_bytes, int dtype, void* stream) {
  const float scale = Dh > 0 ? 1.0f / sqrtf((float)Dh) : 1.0f;
  return decode_impl(q, Kcache, Vcache, lens, nullptr, O, B, Nq, Nkv, Dh, Tcap, 0, scale, LSE,
                     workspace, workspace_bytes, dtype, stream);
}

int attn_decode_noalloc(const void* q, const void* Kcache, const void* Vcache,
                        const int32_t* lens, void* O, int B, int Nq, int Nkv, int Dh, int Tcap,
                        float* LSE, int dtype, void* stream) {
  const float scale = Dh > 0 ? 1.0f / sqrtf((float)Dh) : 1.0f;
  int st = decode_check(q, Kcache, Vcache, lens, O, B, Nq, Nkv, Dh, Tcap, scale, dtype);
  if (st != ATTN_OK) return st;
  const size_t need = attn_decode_workspace_bytes(B, Nq, Nkv, Dh, Tcap, dtype);
  static_assert(attn::kDecodeScratchBytes == ATTN_NOALLOC_SCRATCH_BYTES, "header and library");
  if (need > attn::kDecodeScratchBytes) return ATTN_ESCRATCH;
  void* ws = nullptr;
  if (need > 0 && attn::decode_scratch(&ws) != hipSuccess) return ATTN_EHIP;
  return decode_impl(q, Kcache, Vcache, lens, nullptr, O, B, Nq, Nkv, Dh, Tcap, 0, scale, LSE, ws,
                     need > 0 ? attn::kDecodeScratchBytes : 0, dtype, stream);
}

int attn_decode_window(const void* q, const void* Kcache, const void* Vcache,
                       const int32_t* lens, void* O, int B, int Nq, int Nkv, int Dh, int Tcap,
                       int window, float scale, float* LSE, void* workspace,
                       size_t workspace_bytes, int dtype, void* stream) {
  return decode_impl(q, Kcache, Vcache, lens, nullptr, O, B, Nq, Nkv, Dh, Tcap, window, scale, LSE,
                     workspace, workspace_bytes, dtype, stream);
}

int attn_decode_padded(const void* q, const void* Kcache, const void* Vcache,
                       const int32_t* lens, const uint64_t* key_bits, void* O, int B, int Nq,
                       int Nkv, int Dh, int Tcap, int window, float scale, float* LSE,
                       void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  return decode_impl(q, Kcache, Vcache, lens, key_bits, O, B, Nq, Nkv, Dh, Tcap, window, scale,
                     LSE, workspace, workspace_bytes, dtype, stream);
}

int attn_decode_append(const void* q, const void* knew, const void* vnew, void* Kcache,
                       void* Vcache, const int32_t* lens, const int32_t* slot, void* O, int B,
                       int Nq, int Nkv, int Dh, int Tcap, int window, float scale, float* LSE,
                       void* workspace, size_t workspace_bytes, int dtype, void* stream) {
  if (!q || !knew || !vnew || !Kcache || !Vcache || !lens || !slot || !O) return ATTN_EINVAL;
  int st = validate_common(B, Nq, Nkv, Dh, dtype);
  if (st != ATTN_OK) return st;
  if (!positive(Tcap)) return ATTN_EINVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return ATTN_EINVAL;
  if (window < 0) window = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t need = attn_decode_window_workspace_bytes(B, Nq, Nkv, Dh, Tcap, window, dtype);
  const int elem = dtype == ATTN_BF16 ? 2 : 4;
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return ATTN_EWORKSPACE;
    if ((((uintptr_t)knew | (uintptr_t)vnew) % 16) == 0)  // one launch: append inside the decode
      return from_hip(attn::launch_decode_bf16(q, Kcache, Vcache, lens, O, LSE, B, Nq, Nkv, Dh,
                                               Tcap, window, scale, nullptr, workspace, s, knew,
                                               vnew, slot));
    hipError_t e = attn::launch_kv_append(knew, vnew, Kcache, Vcache, slot, B, Nkv, 1, Dh, Tcap, 0,
                                          elem, s);
    if (e != hipSuccess) return ATTN_EHIP;
    return from_hip(attn::launch_decode_bf16(q, Kcache, Vcache, lens, O, LSE, B, Nq, Nkv, Dh, Tcap,
                                             window, scale, nullptr, workspace, s));
  }
  // general kernels: the append, then the decode rows
  hipError_t e = attn::launch_kv_append(knew, vnew, Kcache, Vcache, slot, B, Nkv, 1, Dh, Tcap, 0,
                                        elem, s);
  if (e != hipSuccess) return ATTN_EHIP;
  return from_hip(attn::launch_rows_general(q, Kcache, Vcache, O, LSE, B, Nq, Nkv, 1, Dh, Tcap, lens,
                                            nullptr, 1, window, scale, dtype == ATTN_BF16, s));
}

int attn_prefill_rope(const void* Q, const void* K, const void* V, const uint64_t* key_bits,
                      void* O, float* LSE, int B, int Nq, int Nkv, int S, int Dh, int causal,
                      int window, float scale, const float* table, int P,
                      const int32_t* positions, const int32_t* start, int style, int dtype,
                      void* stream) {
  const int st = validate_rope(table, P, Dh, style);
  if (st != ATTN_OK) return st;
  const attn::RopeQ rope{table, P, positions, start, style};
  return prefill_impl(Q, K, V, key_bits, O, LSE, B, Nq, Nkv, S, Dh, causal, window, scale, dtype,
                      stream, &rope);
}

int attn_prefill_cache_rope(const void* Q, const void* Kcache, const void* Vcache,
                            const int32_t* lens, const uint64_t* key_bits, void* O, float* LSE,
                            int B, int Nq, int Nkv, int Sq, int Dh, int Tcap, int window,
                            float scale, const float* table, int P, const int32_t* positions,
                            const int32_t* start, int style, int dtype, void* stream) {
  const int st = validate_rope(table, P, Dh, style);
  if (st != ATTN_OK) return st;
  const attn::RopeQ rope{table, P, positions, start, style};
  return prefill_cache_impl(Q, Kcache, Vcache, lens, key_bits, O, LSE, B, Nq, Nkv, Sq, Dh, Tcap,
                            window, scale, dtype, stream, &rope);
}

int attn_decode_rope(const void* q, const void* Kcache, const void* Vcache, const int32_t* lens,
                     const uint64_t* key_bits, void* O, int B, int Nq, int Nkv, int Dh, int Tcap,
                     int window, float scale, const float* table, int P,
                     const int32_t* positions, int style, float* LSE, void* workspace,
                     size_t workspace_bytes, int dtype, void* stream) {
  const int st = validate_rope(table, P, Dh, style);
  if (st != ATTN_OK) return st;
  const attn::RopeQ rope{table, P, positions, nullptr, style};
  return decode_impl(q, Kcache, Vcache, lens, key_bits, O, B, Nq, Nkv, Dh, Tcap, window, scale, LSE,
                     workspace, workspace_bytes, dtype, stream, &rope);
}

int attn_pack_key_mask(const uint8_t* mask, int B, int T, uint64_t* key_bits, void* stream) {
  if (!mask || !key_bits || !positive(B) || !positive(T)) return ATTN_EINVAL;
  return from_hip(attn::launch_pack_key_mask(mask, B, T, key_bits,
                                             static_cast<hipStream_t>(stream)));
}

int attn_rope_cos_sin(float* table, int P, int Dh, double base, void* stream) {
  if (!table || !positive(P) || !positive(Dh) || Dh % 2 != 0) return ATTN_EINVAL;
  if (!(base > 1.0) || !isfinite(base)) return ATTN_EINVAL;
  return from_hip(attn::launch_rope_table(table, P, Dh, base, static_cast<hipStream_t>(stream)));
}

int attn_rope(const void* X, void* Y, const int32_t* positions, const int32_t* start,
              const float* table, int P, int B, int H, int S, int Dh, int style, int dtype,
              void* stream) {
  if (!X || !Y || !table) return ATTN_EINVAL;
  if (!positive(P) || !positive(B) || !positive(H) || !positive(S) || !positive(Dh))
    return ATTN_EINVAL;
  if (Dh % 2 != 0 || (style != 0 && style != 1)) return ATTN_EINVAL;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_EUNSUPPORTED;
  return from_hip(attn::launch_rope(X, Y, positions, start, table, P, B, H, S, Dh, style,
                                    dtype == ATTN_BF16 ? 2 : 4, static_cast<hipStream_t>(stream)));
}

int attn_kv_append_rope(const void* Knew, const void* Vnew, void* Kcache, void* Vcache,
                        const int32_t* pos, const int32_t* positions, const float* table, int P,
                        int B, int Nkv, int Snew, int Dh, int Tcap, int rolling, int style,
                        int dtype, void* stream) {
  if (!Knew || !Vnew || !Kcache || !Vcache || !pos || !table) return ATTN_EINVAL;
  if (!positive(B) || !positive(Nkv) || !positive(Snew) || !positive(Dh) || !positive(Tcap) ||
      !positive(P))
    return ATTN_EINVAL;
  if (Dh % 2 != 0 || (style != 0 && style != 1)) return ATTN_EINVAL;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_EUNSUPPORTED;
  if (rolling != 0 && rolling != 1) return ATTN_EINVAL;
  if (!rolling && Snew > Tcap) return ATTN_EINVAL;
  return from_hip(attn::launch_kv_append_rope(Knew, Vnew, Kcache, Vcache, pos, positions, table, P,
                                              B, Nkv, Snew, Dh, Tcap, rolling, style,
                                              dtype == ATTN_BF16 ? 2 : 4,
                                              static_cast<hipStream_t>(stream)));
}

int attn_kv_append(const void* Knew, const void* Vnew, void* Kcache, void* Vcache,
                   const int32_t* pos, int B, int Nkv, int Snew, int Dh, int Tcap, int rolling,
                   int dtype, void* stream) {
  if (!Knew || !Vnew || !Kcache || !Vcache || !pos) return ATTN_EINVAL;
  if (!positive(B) || !positive(Nkv) || !positive(Snew) || !positive(Dh) || !positive(Tcap))
    return ATTN_EINVAL;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_EUNSUPPORTED;
  if (Dh > 256) return ATTN_EUNSUPPORTED;
  if (rolling != 0 && rolling != 1) return ATTN_EINVAL;
  if (!rolling && Snew > Tcap) return ATTN_EINVAL;
  return from_hip(attn::launch_kv_append(Knew, Vnew, Kcache, Vcache, pos, B, Nkv, Snew, Dh, Tcap,
                                         rolling, dtype == ATTN_BF16 ? 2 : 4,
                                         static_cast<hipStream_t>(stream)));
}

size_t attn_backward_workspace_bytes(int B, int Nq, int Nkv, int S, int Dh, int dtype) {
  if (validate_common(B, Nq, Nkv, Dh, dtype) != ATTN_OK || !positive(S)) return 0;
  return attn::backward_workspace(B, Nq, S);
}

static int backward_impl(const void* Q, const void* K, const void* V, const uint64_t* key_bits,
                         const void* O, const void* dO, const float* LSE, void* dQ, void* dK,
                         void* dV, int B, int Nq, int Nkv, int S, int Dh, int causal, int window,
                         float scale, void* workspace, size_t workspace_bytes, int dtype,
                         void* stream) {
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV) return ATTN_EINVAL;
  int st = validate_common(B, Nq, Nkv, Dh, dtype);
  if (st != ATTN_OK) return st;
  if (!positive(S)) return ATTN_EINVAL;
  if (causal != 0 && causal != 1) return ATTN_EINVAL;
  if (window > 0 && !causal) return ATTN_EINVAL;
  if (!(scale > 0.f) || !isfinite(scale)) return ATTN_EINVAL;
  if (window < 0) window = 0;
  if (dtype == ATTN_BF16 && attn::backward_bf16_supported(Dh) && !mfma_head_fits(S, Dh))
    return ATTN_EUNSUPPORTED;
  const size_t need = attn_backward_workspace_bytes(B, Nq, Nkv, S, Dh, dtype);
  if (workspace == nullptr || workspace_bytes < need) return ATTN_EWORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == ATTN_BF16 && attn::backward_bf16_supported(Dh))
    return from_hip(attn::launch_backward_bf16(Q, K, V, O, dO, LSE, dQ, dK, dV, B, Nq, Nkv, S, Dh,
                                               causal, window, scale, workspace, key_bits, s));
  return from_hip(attn::launch_backward_general(Q, K, V, O, dO, LSE, dQ, dK, dV, B, Nq, Nkv, S,
                                                Dh, causal, window, scale, workspace,
                                                dtype == ATTN_BF16, key_bits, s));
}

int attn_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                  const float* LSE, void* dQ, void* dK, void* dV, int B, int Nq, int Nkv, int S,
                  int Dh, int causal, int window, float scale, void* workspace,
                  size_t workspace_bytes, int dtype, void* stream) {
  return backward_impl(Q, K, V, nullptr, O, dO, LSE, dQ, dK, dV, B, Nq, Nkv, S, Dh, causal,
                       window, scale, workspace, workspace_bytes, dtype, stream);
}

int attn_backward_padded(const void* Q, const void* K, const void* V, const uint64_t* key_bits,
                         const void* O, const void* dO, const float* LSE, void* dQ, void* dK,
                         void* dV, int B, int Nq, int Nkv, int S, int Dh, int causal, int window,
                         float scale, void* workspace, size_t workspace_bytes, int dtype,
                         void* stream) {
  return backward_impl(Q, K, V, key_bits, O, dO, LSE, dQ, dK, dV, B, Nq, Nkv, S, Dh, causal,
                       window, scale, workspace, workspace_bytes, dtype, stream);
}

const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_EINVAL: return "invalid argument (null pointer, non-positive size, bad flag or scale)";
    case ATTN_EGQA: return "number of query heads is not a multiple of the number of K/V heads";
    case ATTN_EUNSUPPORTED:
      return "unsupported element type or head size, or a head too long for the MFMA kernels";
    case ATTN_EWORKSPACE: return "workspace missing or too small";
    case ATTN_EHIP: return "HIP runtime error at launch";
    case ATTN_ESCRATCH:
      return "the call needs more scratch than the allocation-free entry point's fixed buffer";
    default: return "unknown status";
  }
}

}  // extern "C"
