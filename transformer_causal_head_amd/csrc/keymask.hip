// Key-padding mask: one byte per key (nonzero = a real token) packed into
// one bit per key, the form the attention kernels read.
//
// The textbook's forward pass ("Паддинг" under "Прямой проход по шагам")
// adds each batch row's key mask to the causal mask and the window.  The
// kernels test a whole tile of keys against one 64-bit word: bit j % 64 of
// word j / 64 of sequence b is key j's flag; bits past the last key are 0.

#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

// one wavefront per word: lane j reads key 64 * w + j, the ballot is the word
__global__ __launch_bounds__(256) void pack_key_mask_kernel(const uint8_t* mask, int T, int words,
                                                            long long n_words, uint64_t* bits) {
  const long long wid = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wid >= n_words) return;
  const long long b = wid / words;
  const int j = (int)(wid % words) * 64 + lane;
  const bool on = j < T && mask[b * T + j] != 0;
  const uint64_t word = __builtin_amdgcn_ballot_w64(on);
  if (lane == 0) bits[wid] = word;
}

}  // namespace

hipError_t launch_pack_key_mask(const uint8_t* mask, int B, int T, uint64_t* bits,
                                hipStream_t stream) {
  const int words = key_mask_words(T);
  const long long n = (long long)B * words;
  const long long blocks = (n + 3) / 4;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(pack_key_mask_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, mask, T,
                     words, n, bits);
  return hipGetLastError();
}

}  // namespace attn
