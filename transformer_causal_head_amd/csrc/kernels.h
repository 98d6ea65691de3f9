// Internal launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// bf16, Dh == 128 MFMA prefill.
hipError_t launch_prefill_bf16_d128(const void* Q, const void* K, const void* V, void* O,
                                    float* LSE, int B, int Nq, int Nkv, int S, int causal,
                                    int window, float scale, hipStream_t stream);

// General row kernel: one wavefront per output row, any Dh in 1..256,
// bf16 (is_bf16 = 1) or fp32.  Prefill when lens == nullptr (rows (b,h,i),
// K/V heads of S rows); decode otherwise (rows (b,h), K/V heads of kv_rows
// rows, sequence b reads keys 0..lens[b]-1).
hipError_t launch_rows_general(const void* Q, const void* K, const void* V, void* O,
                               float* LSE, int B, int Nq, int Nkv, int S, int Dh,
                               int kv_rows, const int32_t* lens, int causal, int window,
                               float scale, int is_bf16, hipStream_t stream);

// bf16, Dh == 128 split-K decode (partials + log-sum-exp merge).
int decode_bf16_d128_chunk(int B, int Nkv, int Tcap);
size_t decode_bf16_d128_workspace(int B, int Nq, int Nkv, int Tcap);
bool decode_bf16_d128_supported(int Nq, int Nkv);
hipError_t launch_decode_bf16_d128(const void* q, const void* Kc, const void* Vc,
                                   const int32_t* lens, void* O, float* LSE, int B, int Nq,
                                   int Nkv, int Tcap, void* ws, hipStream_t stream);

}  // namespace attn
