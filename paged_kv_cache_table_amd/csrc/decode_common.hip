// Decode dispatch over format combinations, and the merge pass.
#include "decode_impl.hpp"

namespace pkv {

hipError_t launch_decode_split_f32(const AttnArgs&, int, int, int, hipStream_t, bool*);
hipError_t launch_decode_split_f16(const AttnArgs&, int, int, int, hipStream_t, bool*);
hipError_t launch_decode_split_q8h(const AttnArgs&, int, int, int, hipStream_t, bool*);
hipError_t launch_decode_split_q8f(const AttnArgs&, int, int, int, hipStream_t, bool*);

hipError_t launch_decode_split(const AttnArgs& a, int combo, int hd, int bs, int g, hipStream_t st,
                               bool* found) {
  switch (combo) {
    case kComboF32: return launch_decode_split_f32(a, hd, bs, g, st, found);
    case kComboF16: return launch_decode_split_f16(a, hd, bs, g, st, found);
    case kComboQ8H: return launch_decode_split_q8h(a, hd, bs, g, st, found);
    case kComboQ8F: return launch_decode_split_q8f(a, hd, bs, g, st, found);
    default: *found = false; return hipSuccess;
  }
}

hipError_t launch_decode_merge(const AttnArgs& a, int hd, hipStream_t st) {
  const dim3 grid((unsigned)((a.n_q_heads * hd + 255) / 256), a.n_seqs);
  switch (hd) {
    case 64: hipLaunchKernelGGL(decode_merge_kernel<64>, grid, dim3(256), 0, st, a); break;
    case 128: hipLaunchKernelGGL(decode_merge_kernel<128>, grid, dim3(256), 0, st, a); break;
    case 256: hipLaunchKernelGGL(decode_merge_kernel<256>, grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

__global__ void zero_words_kernel(int32_t* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_zero_words(int32_t* p, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_words_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace pkv
