// Measurement helper, not part of libringattn: the sustained rate of
// v_mfma_f32_32x32x16_bf16 on this device, with operands held in registers,
// so that the attention kernel's throughput can be read against what the
// matrix cores deliver under the same power and clock conditions.
//
// Every wave runs four independent accumulation chains; operands are either
// all zeros or N(0, 1)-like bf16 values (sum of two uniforms), since the
// matrix core's power draw, and with it the clock the chip holds, depends on
// the operand bits.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(512) void mfma_loop(float* out, int iters, int random_operands,
                                                 unsigned long long* clk) {
  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  bf16x8 a[4], b[4];
  for (int j = 0; j < 4; ++j)
    for (int i = 0; i < 8; ++i) {
      float va = 0.f, vb = 0.f;
      if (random_operands) {
        const uint32_t h = mix(threadIdx.x * 131u + blockIdx.x * 7919u + j * 8u + i);
        va = ((h & 0xffff) / 65536.0f - 0.5f) * 3.4f;
        vb = ((h >> 16) / 65536.0f - 0.5f) * 3.4f;
      }
      a[j][i] = (__bf16)va;
      b[j][i] = (__bf16)vb;
    }
  f32x16 c[4] = {};
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[(j + r) & 3], c[j], 0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < 4; ++j)
    for (int i = 0; i < 16; ++i) s += c[j][i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clk[0] = __builtin_amdgcn_s_memtime() - c0;
    clk[1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
}

}  // namespace

// Runs `iters` MFMA per wave (a multiple of 4) on `grid` workgroups of 512
// threads, twice, and reports the second run: wall time, FLOP/s and the
// shader clock of workgroup 0 (s_memtime against the 100 MHz s_memrealtime).
// Returns 0, or the HIP error code.
extern "C" int ra_probe_mfma_bf16(int grid, int iters, int random_operands, double* ms, double* tflops,
                                  double* clock_ghz) {
  float* out = nullptr;
  unsigned long long* clk = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t err = hipMalloc(&out, (size_t)grid * 512 * sizeof(float));
  if (err == hipSuccess) err = hipMalloc(&clk, 2 * sizeof(unsigned long long));
  if (err == hipSuccess) err = hipEventCreate(&e0);
  if (err == hipSuccess) err = hipEventCreate(&e1);
  float t = 0.f;
  unsigned long long h[2] = {0, 0};
  for (int rep = 0; rep < 2 && err == hipSuccess; ++rep) {
    err = hipEventRecord(e0, nullptr);
    if (err == hipSuccess) {
      hipLaunchKernelGGL(mfma_loop, dim3(grid), dim3(512), 0, nullptr, out, iters & ~3, random_operands, clk);
      err = hipGetLastError();
    }
    if (err == hipSuccess) err = hipEventRecord(e1, nullptr);
    if (err == hipSuccess) err = hipEventSynchronize(e1);
    if (err == hipSuccess) err = hipEventElapsedTime(&t, e0, e1);
  }
  if (err == hipSuccess) err = hipMemcpy(h, clk, sizeof(h), hipMemcpyDeviceToHost);
  if (err == hipSuccess) {
    const double flop = (double)grid * 8 * (iters & ~3) * 4 * 32768.0;  // 8 waves, 4 chains
    *ms = t;
    *tflops = flop / (t * 1e-3) / 1e12;
    *clock_ghz = h[1] ? (double)h[0] / ((double)h[1] * 10.0) : 0.0;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (clk) (void)hipFree(clk);
  if (out) (void)hipFree(out);
  return (int)err;
}
