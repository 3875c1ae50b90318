// kv_write: rotate (x U on MFMA, then Walsh-Hadamard and bit reversal),
// clip, quantize to INT2 and pack new K/V tokens into the paged cache.
//
// Method: the Italian page "OSCAR: Come Together AI Comprime la KV Cache a
// 2-bit per LLM", sections "I tre fattori della rotazione" (R = U H_Had P_br)
// and "Architettura del Sistema di Serving e Layout di Memoria" (each token is
// rotated, clipped and quantized at write time; sink and recent tokens stay
// BF16); the Spanish summary "Resumen Tecnico: OSCAR ...", section 2.2 B.
//
// Work decomposition: 256-thread blocks per (KV head, K-or-V), about three per
// CU over the whole grid (43 KB of LDS and 3 waves per SIMD each); each walks
// groups of four 16-token tiles (one per wave) strided by the grid.  The block
// stages U^T in LDS once; each wave reads its MFMA A-fragments from there.  Per tile of 16
// tokens the wave computes y^T = U^T x^T with 32 v_mfma_f32_16x16x32_bf16;
// lane l then owns token l%16 and channels 16*mt + 4*(l/16) + r (mt<8, r<4),
// so five of the seven butterfly stages are in registers and two cross lanes.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "kv_write_body.h"

namespace oscar {

namespace {

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void kv_write_kernel(KvWriteArgs a) {
  __shared__ KvWriteSmem sm;
  kv_write_block(a, sm, blockIdx.x, gridDim.x, blockIdx.y, blockIdx.z);
}

}  // namespace

int device_cus() {   // compute units of the current device (cached per device)
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

int launch_kv_write(const KvWriteLaunch& L, hipStream_t stream) {
  KvWriteArgs a{};
  dim3 grid;
  if (!kv_write_setup(L, device_cus(), a, grid)) return 0;   // nothing to write
  hipLaunchKernelGGL(kv_write_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace oscar
