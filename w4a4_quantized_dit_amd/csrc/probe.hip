// Memory-system probe for the benchmark (not part of the layer): a plain streaming kernel that
// reads `read_bytes` from src and writes `write_bytes` to dst in the same pass, with 16-byte
// nontemporal loads and 16-byte stores over a grid-stride loop, so that the activation kernels
// can be compared with a copy of their own read/write byte mix.  Built into its own library
// (libsvdq_probe.so); the layer's library does not contain it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

__global__ __launch_bounds__(256) void k_stream(const u32x4_t* __restrict__ src, int64_t n_read,
                                                u32x4_t* __restrict__ dst, int64_t n_write) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  // written piece i depends on the read pieces i, i + n_out, i + 2 n_out, ... (consecutive
  // threads touch consecutive 16-byte pieces on both sides)
  const int64_t n_out = n_write > 0 ? n_write : n_read;
  const int64_t per = (n_read + n_out - 1) / n_out;
  u32x4_t acc = u32x4_t{0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_out; i += stride) {
    for (int64_t j = 0; j < per; ++j) {
      const int64_t k = i + j * n_out;
      if (k < n_read) acc ^= __builtin_nontemporal_load(src + k);
    }
    if (n_write > 0) dst[i] = acc;
  }
  // a pure read keeps its loads by a store that no input makes
  if (n_write == 0 && acc[0] == 0x9E3779B9u && acc[1] == 0x7F4A7C15u) dst[0] = acc;
}

}  // namespace

extern "C" int svdq_probe_stream(const void* src, int64_t read_bytes, void* dst,
                                 int64_t write_bytes, hipStream_t stream) {
  if (!src || !dst || read_bytes < 0 || write_bytes < 0 || (read_bytes | write_bytes) & 15)
    return 1;
  const int64_t nr = read_bytes / 16, nw = write_bytes / 16;
  const int64_t n = nw > 0 ? nw : nr;
  if (n == 0) return 0;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;   // 16 workgroups per CU, grid-stride beyond
  if (blocks < 1) blocks = 1;
  k_stream<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(
      reinterpret_cast<const u32x4_t*>(src), nr, reinterpret_cast<u32x4_t*>(dst), nw);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
