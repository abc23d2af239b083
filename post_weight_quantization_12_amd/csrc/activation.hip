// Gated activation between the MLP layers of a Llama-style block:
// A = SiLU(G) * U elementwise, SiLU(g) = g / (1 + e^-g).
//
// The layer-wise method quantizes one layer at a time and takes each
// layer's calibration inputs from the block with its earlier layers already
// quantized (glossary entry "gptq", paragraph "Method" (1)).  In a Llama MLP
// the input of the down projection is this product of the gate and up
// projections' outputs.  Evaluated in fp32 (expf), rounded once to fp16.
// HBM-bound: 6 bytes per element.
#include "common.hpp"

namespace gptq {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ inline float silu_mul1(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Grid: (ceil(cols / 2048), rows): 256 threads, 8 elements each.
__global__ void __launch_bounds__(256)
silu_mul_kernel(const _Float16* __restrict__ G, int64_t ldg, const _Float16* __restrict__ U,
                int64_t ldu, int64_t cols, _Float16* __restrict__ A, int64_t lda, int vec) {
  const int64_t r = blockIdx.y;
  const int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (c0 >= cols) return;
  const _Float16* g = G + r * ldg + c0;
  const _Float16* u = U + r * ldu + c0;
  _Float16* a = A + r * lda + c0;
  if (vec && c0 + 8 <= cols) {
    const uint4 gv = *reinterpret_cast<const uint4*>(g);
    const uint4 uv = *reinterpret_cast<const uint4*>(u);
    const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w}, uw[4] = {uv.x, uv.y, uv.z, uv.w};
    uint32_t aw[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const half2_t gh = __builtin_bit_cast(half2_t, gw[j]);
      const half2_t uh = __builtin_bit_cast(half2_t, uw[j]);
      const half2_t ah = {(_Float16)silu_mul1((float)gh.x, (float)uh.x),
                          (_Float16)silu_mul1((float)gh.y, (float)uh.y)};
      aw[j] = __builtin_bit_cast(uint32_t, ah);
    }
    *reinterpret_cast<uint4*>(a) = make_uint4(aw[0], aw[1], aw[2], aw[3]);
    return;
  }
  for (int j = 0; j < 8 && c0 + j < cols; ++j)
    a[j] = (_Float16)silu_mul1((float)g[j], (float)u[j]);
}

}  // namespace

hipError_t run_silu_mul(const void* G, int64_t ldg, const void* U, int64_t ldu, int64_t rows,
                        int64_t cols, void* A, int64_t lda, hipStream_t s) {
  const bool vec = ((reinterpret_cast<uintptr_t>(G) | reinterpret_cast<uintptr_t>(U) |
                     reinterpret_cast<uintptr_t>(A)) & 15) == 0 &&
                   ldg % 8 == 0 && ldu % 8 == 0 && lda % 8 == 0;
  for (int64_t r0 = 0; r0 < rows; r0 += 65535) {  // grid y limit
    const int64_t nr = rows - r0 < 65535 ? rows - r0 : 65535;
    dim3 grid((unsigned)((cols + 2047) / 2048), (unsigned)nr);
    hipLaunchKernelGGL(silu_mul_kernel, grid, dim3(256), 0, s,
                       static_cast<const _Float16*>(G) + r0 * ldg, ldg,
                       static_cast<const _Float16*>(U) + r0 * ldu, ldu, cols,
                       static_cast<_Float16*>(A) + r0 * lda, lda, vec ? 1 : 0);
    GPTQ_HIP_TRY(hipGetLastError());
  }
  return hipSuccess;
}

}  // namespace gptq
