// Hessian accumulation H(upper) += 2 X^T X on the gfx950 matrix cores.
//
// The Hessian of the layer reconstruction loss with respect to the layer's
// weights is 2 * sum_t x_t x_t^T over calibration tokens (glossary entry
// "gptq", "Algorithm" step (1)).  X arrives tokens x features, row-major, so
// both MFMA operands are column panels of X: the contraction runs over tokens,
// which are the strided dimension in memory.  Each thread loads an 8-token x
// 8-feature block with 16-byte loads, transposes it in registers and stores
// feature-major rows (8 consecutive tokens per 16 bytes) into LDS, from which
// every MFMA operand is one ds_read_b128.
//
// Tiles: T x T output tiles of the upper triangle only; K (tokens) is staged
// BK = 64 at a time, double-buffered in LDS.  MFMA: v_mfma_f32_32x32x16_{f16,bf16}
// (fp16/bf16 products are exact in fp32; accumulation is fp32).
#include "common.hpp"

namespace gptq {
namespace {

constexpr int BK = 64;        // tokens per LDS stage
constexpr int LDSK = BK + 8;  // padded row (halves): 144 B, conflict-free b128 reads

template <int T>
struct SyrkCfg {
  static constexpr int NT = T * BK / 32;  // threads: one 8x8 block per thread per operand
  static constexpr int WM = 2;
  static constexpr int WN = (NT / 64) / WM;
  static constexpr int FM = T / WM / 32;  // 32x32 fragments per wave along M
  static constexpr int FN = T / WN / 32;
  static constexpr size_t LDS = (size_t)4 * T * LDSK * sizeof(uint16_t);  // 2 stages x (A, B)
};

__device__ inline uint32_t lo16pair(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ inline uint32_t hi16pair(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

__device__ inline uint32_t comp(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Transpose an 8 (tokens) x 8 (features) block of 16-bit values:
// r[t] holds features 0..7 of token t; o[f] receives tokens 0..7 of feature f.
__device__ inline void transpose8x8(const uint4 (&r)[8], uint4 (&o)[8]) {
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    uint32_t d[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t a = comp(r[2 * p], f >> 1), b = comp(r[2 * p + 1], f >> 1);
      d[p] = (f & 1) ? hi16pair(a, b) : lo16pair(a, b);
    }
    o[f] = make_uint4(d[0], d[1], d[2], d[3]);
  }
}

template <bool BF16>
__device__ inline f32x16_t mfma16(const uint4& a, const uint4& b, f32x16_t c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  }
}

template <int T, bool BF16, bool VEC>
__global__ void __launch_bounds__(SyrkCfg<T>::NT)
syrk_upper_kernel(float* __restrict__ H, int64_t n, const uint16_t* __restrict__ X,
                  int64_t ntok, int64_t ldx, int nt) {
  using C = SyrkCfg<T>;
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* sA = smem;                       // [2][T][LDSK]
  uint16_t* sB = smem + 2 * T * LDSK;        // [2][T][LDSK]

  // Upper-triangle tile (ti <= tj) from the linear block index.
  const int b = blockIdx.x;
  int tj = (int)((sqrtf(8.0f * (float)b + 1.0f) - 1.0f) * 0.5f);
  while ((tj + 1) * (tj + 2) / 2 <= b) ++tj;
  while (tj * (tj + 1) / 2 > b) --tj;
  const int ti = b - tj * (tj + 1) / 2;
  (void)nt;
  const int64_t i0 = (int64_t)ti * T, j0 = (int64_t)tj * T;

  const int tid = threadIdx.x;
  const int which = tid / T;          // 0: A panel (features i0..), 1: B panel (features j0..)
  const int local = tid % T;
  // Lanes take consecutive token blocks first: a 16-lane pass of the 16-byte
  // LDS stores then covers tb = 0..7 (16-byte steps) times two feature blocks
  // (144*8 B apart = 128 B mod 256), i.e. 16 distinct bank groups.
  const int tb = local % (BK / 8), fb = local / (BK / 8);
  const int64_t col = (which ? j0 : i0) + fb * 8;
  uint16_t* sdst = which ? sB : sA;

  uint4 r[8];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int64_t tok = k0 + tb * 8 + t;
      if constexpr (VEC) {
        if (tok < ntok && col < n) {
          r[t] = *reinterpret_cast<const uint4*>(X + tok * ldx + col);
        } else {
          r[t] = make_uint4(0, 0, 0, 0);
        }
      } else {
        uint32_t d[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          uint32_t lo = 0, hi = 0;
          if (tok < ntok && col + 2 * p < n) lo = X[tok * ldx + col + 2 * p];
          if (tok < ntok && col + 2 * p + 1 < n) hi = X[tok * ldx + col + 2 * p + 1];
          d[p] = lo | (hi << 16);
        }
        r[t] = make_uint4(d[0], d[1], d[2], d[3]);
      }
    }
  };
  auto lstore = [&](int buf) {
    uint4 o[8];
    transpose8x8(r, o);
    uint16_t* base = sdst + (size_t)buf * T * LDSK;
#pragma unroll
    for (int f = 0; f < 8; ++f)
      *reinterpret_cast<uint4*>(base + (fb * 8 + f) * LDSK + tb * 8) = o[f];
  };

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave % C::WM, wn = wave / C::WM;
  f32x16_t acc[C::FM][C::FN];
#pragma unroll
  for (int a = 0; a < C::FM; ++a)
#pragma unroll
    for (int c = 0; c < C::FN; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][c][v] = 0.0f;

  const int nk = (int)((ntok + BK - 1) / BK);
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((int64_t)(kt + 1) * BK);
    const uint16_t* a_base = sA + (size_t)cur * T * LDSK;
    const uint16_t* b_base = sB + (size_t)cur * T * LDSK;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int koff = ks * 16 + (lane >> 5) * 8;
      uint4 af[C::FM], bfr[C::FN];
#pragma unroll
      for (int a = 0; a < C::FM; ++a)
        af[a] = *reinterpret_cast<const uint4*>(
            a_base + (wm * C::FM * 32 + a * 32 + (lane & 31)) * LDSK + koff);
#pragma unroll
      for (int c = 0; c < C::FN; ++c)
        bfr[c] = *reinterpret_cast<const uint4*>(
            b_base + (wn * C::FN * 32 + c * 32 + (lane & 31)) * LDSK + koff);
#pragma unroll
      for (int a = 0; a < C::FM; ++a)
#pragma unroll
        for (int c = 0; c < C::FN; ++c) acc[a][c] = mfma16<BF16>(af[a], bfr[c], acc[a][c]);
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: H[i][j] += 2 * acc for i <= j (upper triangle), in bounds.
#pragma unroll
  for (int a = 0; a < C::FM; ++a)
#pragma unroll
    for (int c = 0; c < C::FN; ++c) {
      const int64_t j = j0 + wn * C::FN * 32 + c * 32 + (lane & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t i = i0 + wm * C::FM * 32 + a * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        if (i < n && j < n && i <= j) {
          float* p = H + i * n + j;
          *p = *p + 2.0f * acc[a][c][v];
        }
      }
    }
}

template <int T, bool BF16, bool VEC>
hipError_t launch_t(float* H, int64_t n, const uint16_t* X, int64_t ntok, int64_t ldx,
                    hipStream_t s) {
  const int nt = (int)((n + T - 1) / T);
  const int64_t tiles = (int64_t)nt * (nt + 1) / 2;
  const size_t lds = SyrkCfg<T>::LDS;
  auto kern = syrk_upper_kernel<T, BF16, VEC>;
  GPTQ_HIP_TRY(hipFuncSetAttribute((const void*)kern,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  hipLaunchKernelGGL(kern, dim3((unsigned)tiles), dim3(SyrkCfg<T>::NT), lds, s, H, n, X, ntok,
                     ldx, nt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_syrk(float* H, int64_t n, const void* X, int dtype, int64_t ntok,
                       int64_t ldx, hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(X);
  const bool vec = (n % 8 == 0) && (ldx % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
  const bool bf = dtype == 1;
  // 256 x 256 tiles (8 waves) halve the operand traffic per flop against 128 x 128.
  constexpr int T = 256;
  if (bf) {
    return vec ? launch_t<T, true, true>(H, n, x, ntok, ldx, s)
               : launch_t<T, true, false>(H, n, x, ntok, ldx, s);
  }
  return vec ? launch_t<T, false, true>(H, n, x, ntok, ldx, s)
             : launch_t<T, false, false>(H, n, x, ntok, ldx, s);
}

}  // namespace gptq
