// Weight repack: canonical Q4_32 / Q8_32 / F32 matrices -> the tiled layout of common.h, and
// small set-up kernels (the RoPE table).
#include "common.h"

namespace dfl {

// One thread per (source n-tile, k-block, lane): writes that lane's 16 (Q4) or 2x16 (Q8)
// code bytes, and lanes < 16 write their row's four f16 scales.
__global__ void k_pack_q(int fmt, const uint8_t* __restrict__ codes, const uint16_t* __restrict__ scales, int rows,
                         int cols, uint8_t* __restrict__ out, long tile_off, long tile_stride) {
  const long KB = cols / 128, T = rows / 16;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * KB * 64) return;
  const int lane = (int)(idx & 63);
  const long tk = idx >> 6;
  const long kb = tk % KB, t = tk / KB;
  const long n = t * 16 + (lane & 15);
  const int quarter = lane >> 4;
  const long dst_tile = tile_off + t * tile_stride;
  const int SB = fmt == Q4 ? SB_Q4 : SB_Q8;
  uint8_t* sb = out + (dst_tile * KB + kb) * SB;
  for (int j = 0; j < 4; j++) {
    const long k0 = 32 * (4 * kb + j) + 8 * quarter;
    if (fmt == Q4) {
      const uint8_t* row = codes + n * (cols / 2);
      uint32_t word = 0;
      for (int b = 0; b < 4; b++) {
        const long klo = k0 + b, khi = k0 + 4 + b;
        uint32_t lo = (klo & 1) ? (row[klo >> 1] >> 4) : (row[klo >> 1] & 15);
        uint32_t hi = (khi & 1) ? (row[khi >> 1] >> 4) : (row[khi >> 1] & 15);
        word |= (lo | (hi << 4)) << (8 * b);
      }
      *(uint32_t*)(sb + 16 * lane + 4 * j) = word;
    } else {
      const uint8_t* row = codes + n * cols;
      uint8_t* dst = sb + (j < 2 ? 0 : 1024) + 16 * lane + 8 * (j & 1);
      for (int b = 0; b < 8; b++) dst[b] = row[k0 + b];
    }
  }
  if (lane < 16) {
    uint16_t* dsc = (uint16_t*)(sb + (fmt == Q4 ? SB_SCALES_Q4 : SB_SCALES_Q8) + 8 * lane);
    for (int j = 0; j < 4; j++) dsc[j] = scales[n * (cols / 32) + 4 * kb + j];
  }
}

// F32: row r of the source goes to row (tile_off + (r/16)*tile_stride)*16 + r%16.
__global__ void k_pack_f32(const float* __restrict__ src, int rows, int cols, float* __restrict__ out, long tile_off,
                           long tile_stride) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)rows * cols) return;
  const long r = idx / cols, c = idx % cols;
  const long dr = (tile_off + (r / 16) * tile_stride) * 16 + (r % 16);
  out[dr * cols + c] = src[idx];
}

hipError_t launch_pack(int fmt, const void* codes, const void* scales, int rows, int cols, void* out, long tile_off,
                       long tile_stride, hipStream_t st) {
  if (fmt == F32) {
    const long total = (long)rows * cols;
    hipLaunchKernelGGL(k_pack_f32, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, (const float*)codes,
                       rows, cols, (float*)out, tile_off, tile_stride);
  } else {
    const long total = (long)(rows / 16) * (cols / 128) * 64;
    hipLaunchKernelGGL(k_pack_q, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, fmt,
                       (const uint8_t*)codes, (const uint16_t*)scales, rows, cols, (uint8_t*)out, tile_off,
                       tile_stride);
  }
  return hipGetLastError();
}

size_t max_dynamic_lds() {
  static size_t cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 64 * 1024;
  if (!cached[dev]) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || v <= 0)
      v = 64 * 1024;
    cached[dev] = (size_t)v;
  }
  return cached[dev];
}

hipError_t allow_lds(const void* kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  if (bytes > max_dynamic_lds()) return hipErrorInvalidValue;
  return hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

// inv_freq[i] = theta^(-2i/hd) in f64, stored f32 (cortiq-engine dflash.rs, Drafter::new).
__global__ void k_inv_freq(double theta, int hd, float* out) {
  const int i = threadIdx.x;
  if (i < hd / 2) out[i] = (float)pow(theta, -(2.0 * i) / (double)hd);
}

hipError_t launch_inv_freq(double theta, int hd, float* out, hipStream_t st) {
  hipLaunchKernelGGL(k_inv_freq, dim3(1), dim3(128), 0, st, theta, hd, out);
  return hipGetLastError();
}

}  // namespace dfl
