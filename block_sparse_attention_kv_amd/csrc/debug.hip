// debug.hip -- run the kernels' own NVFP4 / FP8 decoders (fmt.hpp) over flat
// buffers so that tests can check them bit for bit against every code; and
// a plain streaming read of device memory, the attainable read bandwidth
// that the decode kernels' rates are read against.
#include "fmt.hpp"
#include "msa_internal.hpp"

namespace msa {

namespace {

__device__ __forceinline__ uint32_t load_u32_bytes(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

__device__ __forceinline__ void store_f16x8(float* out, u32x4 v) {
  const f16x8 h = __builtin_bit_cast(f16x8, v);
#pragma unroll
  for (int e = 0; e < 8; e++) out[e] = (float)h[e];
}

// One 16-element group per thread: elements 0..7 through the shared-scale
// decoder used for K, elements 8..15 through the per-element-scale decoder
// used for V.
__global__ void debug_nvfp4_kernel(const uint8_t* codes, const uint8_t* scales, int64_t n_groups, float* out) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n_groups) return;
  const uint32_t w0 = load_u32_bytes(codes + 8 * g);
  const uint32_t w1 = load_u32_bytes(codes + 8 * g + 4);
  const uint32_t sb = scales[g];
  const uint32_t s2 = fp8x2_f16x2<false>(sb | (sb << 8));
  store_f16x8(out + 16 * g, nvfp4x8_f16(w0, bcast_lo16(s2)));
  const uint32_t s8 = sb * 0x01010101u;
  const u32x4 each = fp8x8_f16(s8, s8);
  store_f16x8(out + 16 * g + 8, nvfp4x8_f16_each(w1, each));
}

// Eight E4M3 codes per thread through the bf16 decoder used for indexer keys.
__global__ void debug_fp8_kernel(const uint8_t* codes, int64_t n, float* out) {
  const int64_t i0 = 8 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
  if (i0 >= n) return;
  uint8_t by[8];
#pragma unroll
  for (int e = 0; e < 8; e++) by[e] = (i0 + e < n) ? codes[i0 + e] : 0;
  const u32x4 v = fp8x8_bf16(load_u32_bytes(by), load_u32_bytes(by + 4));
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const uint32_t w = v[e >> 1];
    if (i0 + e < n) out[i0 + e] = bf16_bits_to_f32((e & 1) ? (w >> 16) : (w & 0xFFFFu));
  }
}

// Reads n16 16-byte words with nontemporal loads: each wave takes 4 KB of
// contiguous memory per step (four 1 KB loads in flight), the waves of the
// grid striding over the buffer. (Lanes whose four loads lie a grid stride
// apart instead reach about 20% less on a 1 GiB stream.) The XOR of all words
// is stored only when it equals `magic` (a value from the host), so the
// loads cannot be dropped and nothing is written in practice.
__global__ __launch_bounds__(256) void read_bw_kernel(const u32x4* p, int64_t n16, uint32_t* out, uint32_t magic) {
  const int lane = threadIdx.x & 63;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t base = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 256; base < n16; base += nwaves * 256) {
    u32x4 v[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int64_t i = base + 64 * j + lane;
      v[j] = i < n16 ? __builtin_nontemporal_load(p + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 4; j++) acc ^= v[j];
  }
  const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == magic) out[0] = x;
}

}  // namespace

hipError_t launch_debug_read(const void* buf, int64_t bytes, uint32_t* out, int cus, hipStream_t s) {
  if (bytes <= 0) return hipSuccess;
  const int64_t n16 = bytes / 16;
  int64_t blocks = (int64_t)4 * cus;  // 16 waves per compute unit
  const int64_t need = (n16 + 1023) / 1024;  // 4 KB per wave and step
  if (blocks > need) blocks = need;
  read_bw_kernel<<<dim3((unsigned)blocks), 256, 0, s>>>(static_cast<const u32x4*>(buf), n16, out, 0x9E3779B9u);
  return hipGetLastError();
}

hipError_t launch_debug_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t n_groups, float* out,
                              hipStream_t s) {
  if (n_groups <= 0) return hipSuccess;
  const int64_t blocks = (n_groups + 255) / 256;
  debug_nvfp4_kernel<<<dim3((unsigned)blocks), 256, 0, s>>>(codes, scales, n_groups, out);
  return hipGetLastError();
}

hipError_t launch_debug_fp8(const uint8_t* codes, int64_t n, float* out, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 8 * 256 - 1) / (8 * 256);
  debug_fp8_kernel<<<dim3((unsigned)blocks), 256, 0, s>>>(codes, n, out);
  return hipGetLastError();
}

}  // namespace msa
