// Lossless re-layout of grouped 4-bit weights into MFMA tiles.
//
// Canonical layout (as stored in a checkpoint): codes [G][N][K/2] (two E2M1 codes per
// byte, element 2j in the low nibble), scales [G][N][K/16] (one E4M3 code per 16
// weights along K).
//
// Tiled layout (what the expert FFN kernels read): the matrix is cut into tiles of
// 16 rows x 128 columns. Tile (g, b, s) covers rows 16b..16b+15 and columns
// 128s..128s+127 of expert g and is stored at index ((g * N/16) + b) * K/128 + s:
//   codes  1024 bytes: lane l = rn + 16*kq (rn = l % 16, kq = l / 16) owns bytes
//          16l..16l+15 = canonical bytes of row 16b+rn, columns 128s+32kq .. +31;
//   scales  128 bytes: lane l owns bytes 2l, 2l+1 = the scales of the same row for
//          column groups 8s+2kq and 8s+2kq+1.
// So a wave reads a tile with one contiguous 1 KB load (16 B per lane) plus one
// contiguous 128 B load, and every lane then holds exactly the 32 codes and two
// scales of the 16x16x32 MFMA operands it feeds. Bytes are only moved, never
// changed; the total size is the canonical size.
#include "device.hpp"
#include "launch.hpp"

namespace moe4 {

namespace {

// One thread per 16-byte code chunk (and its 2 scale bytes).
__global__ __launch_bounds__(256) void prepack_kernel(const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ scales, int G, int N,
                                                      int K, uint8_t* __restrict__ tcodes,
                                                      uint8_t* __restrict__ tscales) {
  const long long nb = N / 16, ns = K / 128;
  const long long total = (long long)G * nb * ns * 64;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int l = (int)(i & 63);
    const long long tile = i >> 6;
    const long long s = tile % ns;
    const long long gb = tile / ns;  // g * nb + b
    const long long b = gb % nb, g = gb / nb;
    const int rn = l & 15, kq = l >> 4;
    const long long row = g * N + b * 16 + rn;
    const uint4 v = *reinterpret_cast<const uint4*>(codes + row * (K / 2) + s * 64 + kq * 16);
    *reinterpret_cast<uint4*>(tcodes + tile * 1024 + l * 16) = v;
    const uint8_t* sc = scales + row * (K / 16) + s * 8 + kq * 2;
    tscales[tile * 128 + l * 2] = sc[0];
    tscales[tile * 128 + l * 2 + 1] = sc[1];
  }
}

}  // namespace

hipError_t launch_prepack(const uint8_t* codes, const uint8_t* scales, int G, int N, int K,
                          uint8_t* tcodes, uint8_t* tscales, hipStream_t s) {
  const long long total = (long long)G * (N / 16) * (K / 128) * 64;
  if (total == 0) return hipSuccess;
  const long long blocks = (total + 255) / 256;
  const int grid = (int)(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(prepack_kernel, dim3(grid), dim3(256), 0, s, codes, scales, G, N, K, tcodes,
                     tscales);
  return hipGetLastError();
}

}  // namespace moe4
