// Storage form of a quantized layer's group parameters.
//
// The pages save a quantized model as safetensors with a quantize_config.json
// ("AutoGPTQ" catalogue page, Safetensors Support; "GPTQ > Using AutoGPTQ in
// Practice", saving the quantized model).  The codes are already dense
// (qweight); for storage the group parameters shrink too: scales to fp16 and
// zero-points to the same dense b-bit stream as the codes, here along the
// output channels: row g of qzeros is the little-endian b-bit stream of
// zeros[g][0 .. out-1] cut into 32-bit words (zero r at bits [r b, (r+1) b)).
// HBM-bound: 8 bytes in, 2 + b/8 bytes out per (group, channel).
#include "common.hpp"

namespace gptq {
namespace {

// Thread t converts scale t and builds qzeros word t (row t / wpr, word
// t % wpr) from the zeros whose bit ranges overlap it.
template <int B>
__global__ void __launch_bounds__(256)
export_kernel(const float* __restrict__ scales, const int32_t* __restrict__ zeros,
              int64_t G, int64_t out, _Float16* __restrict__ s16,
              uint32_t* __restrict__ qz, int64_t wpr) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < G * out) s16[t] = (_Float16)scales[t];
  if (t >= G * wpr) return;
  const int64_t g = t / wpr, w = t % wpr;
  const int64_t bit0 = w * 32;
  const int64_t r0 = bit0 / B, r1 = (bit0 + 31) / B;  // zeros touching this word
  uint32_t v = 0;
  for (int64_t r = r0; r <= r1 && r < out; ++r) {
    const uint32_t z = (uint32_t)zeros[g * out + r] & ((1u << B) - 1u);
    const int64_t sh = r * B - bit0;  // position of zero r relative to the word
    if (sh >= 0)
      v |= sh < 32 ? z << sh : 0u;
    else
      v |= z >> (-sh);
  }
  qz[g * wpr + w] = v;
}

// zeros[g][r] from qzeros (inverse of the packing above).
template <int B>
__global__ void __launch_bounds__(256)
unpack_zeros_kernel(const uint32_t* __restrict__ qz, int64_t G, int64_t out, int64_t wpr,
                    int32_t* __restrict__ zeros) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= G * out) return;
  const int64_t g = t / out, r = t % out;
  const int64_t bit = r * B, w = bit / 32;
  const int off = (int)(bit % 32);
  uint32_t v = qz[g * wpr + w] >> off;
  if (off + B > 32) v |= qz[g * wpr + w + 1] << (32 - off);
  zeros[t] = (int32_t)(v & ((1u << B) - 1u));
}

}  // namespace

hipError_t run_export(const float* scales, const int32_t* zeros, int64_t G, int64_t out, int bits,
                      void* scales_f16, int32_t* qzeros, hipStream_t s) {
  const int64_t wpr = out * bits / 32;
  const int64_t n = G * out > G * wpr ? G * out : G * wpr;
  const dim3 grid((unsigned)((n + 255) / 256));
  _Float16* s16 = static_cast<_Float16*>(scales_f16);
  uint32_t* qz = reinterpret_cast<uint32_t*>(qzeros);
  switch (bits) {
    case 2: hipLaunchKernelGGL(export_kernel<2>, grid, dim3(256), 0, s, scales, zeros, G, out, s16, qz, wpr); break;
    case 3: hipLaunchKernelGGL(export_kernel<3>, grid, dim3(256), 0, s, scales, zeros, G, out, s16, qz, wpr); break;
    case 8: hipLaunchKernelGGL(export_kernel<8>, grid, dim3(256), 0, s, scales, zeros, G, out, s16, qz, wpr); break;
    default: hipLaunchKernelGGL(export_kernel<4>, grid, dim3(256), 0, s, scales, zeros, G, out, s16, qz, wpr); break;
  }
  return hipGetLastError();
}

hipError_t run_unpack_zeros(const int32_t* qzeros, int64_t G, int64_t out, int bits,
                            int32_t* zeros, hipStream_t s) {
  const int64_t wpr = out * bits / 32;
  const dim3 grid((unsigned)((G * out + 255) / 256));
  const uint32_t* qz = reinterpret_cast<const uint32_t*>(qzeros);
  switch (bits) {
    case 2: hipLaunchKernelGGL(unpack_zeros_kernel<2>, grid, dim3(256), 0, s, qz, G, out, wpr, zeros); break;
    case 3: hipLaunchKernelGGL(unpack_zeros_kernel<3>, grid, dim3(256), 0, s, qz, G, out, wpr, zeros); break;
    case 8: hipLaunchKernelGGL(unpack_zeros_kernel<8>, grid, dim3(256), 0, s, qz, G, out, wpr, zeros); break;
    default: hipLaunchKernelGGL(unpack_zeros_kernel<4>, grid, dim3(256), 0, s, qz, G, out, wpr, zeros); break;
  }
  return hipGetLastError();
}

}  // namespace gptq
