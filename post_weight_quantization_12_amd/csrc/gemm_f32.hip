// fp32 GEMM on the gfx950 matrix cores (v_mfma_f32_32x32x2_f32):
//     C[M x N] = alpha * op(A) op(B) + beta * C, row-major operands.
//
// Used by the factorization (triangular products and the symmetric rank-k
// update of the recursive Cholesky/inverse) and by the lazy trailing update
// of the quantization sweep (W[:, right] -= E[:, left] * U'[left, right]).
// fp32 operands keep the sweep's accumulated error at fp32 level.
//
// Tiles BM x BN (128 or 64), BK = 16, 256 threads = 2 x 2 waves.  Both
// operands are staged k-contiguous in LDS (rows of 16 floats + 4 pad, so each
// lane's 8 k-values are two conflict-free ds_read_b128).  In one 32x32x2 MFMA
// the two lane halves carry two different k; over the 8 MFMAs of a stage,
// lane half h carries k = 8h + u for MFMA u.  Any fixed assignment of k to
// (MFMA, half) gives the same sum as long as A and B use the same one.
#include "common.hpp"

namespace gptq {
namespace {

constexpr int BK = 16;
constexpr int LDK = BK + 4;

template <int BM, int BN, bool TA, bool TB, bool VEC>
__global__ void __launch_bounds__(256)
gemm_f32_kernel(int64_t M, int64_t N, int64_t K, const float* __restrict__ A, int64_t lda,
                const float* __restrict__ B, int64_t ldb, float* __restrict__ C, int64_t ldc,
                float alpha, float beta, int kmode, int lower_only) {
  constexpr int FM = BM / 64, FN = BN / 64;
  __shared__ __align__(16) float sA[2][BM * LDK];
  __shared__ __align__(16) float sB[2][BN * LDK];

  const int64_t i0 = (int64_t)blockIdx.y * BM, j0 = (int64_t)blockIdx.x * BN;
  if (lower_only && j0 >= i0 + BM) return;

  int64_t kbeg = 0, kend = K;
  if (kmode == KR_LE_COL) kend = j0 + BN < K ? j0 + BN : K;
  else if (kmode == KR_GE_COL) kbeg = j0;
  else if (kmode == KR_LE_ROW) kend = i0 + BM < K ? i0 + BM : K;
  kbeg = kbeg / BK * BK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int c = 0; c < FN; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][c][v] = 0.0f;

  if (kend > kbeg) {
    constexpr int NA = BM / 64, NB = BN / 64;  // float4 per thread per stage
    float4 ra[NA], rb[NB];

    // op(A)[i][k] for the tile: !TA -> A[i*lda + k] (vector along k); TA -> A[k*lda + i].
    auto loadA = [&](int64_t k0) {
#pragma unroll
      for (int p = 0; p < NA; ++p) {
        const int idx = tid + p * 256;
        int64_t r, c;  // memory row / column of the first element
        if constexpr (!TA) { r = i0 + idx / 4; c = k0 + (idx % 4) * 4; }
        else { r = k0 + idx / (BM / 4); c = i0 + (idx % (BM / 4)) * 4; }
        const int64_t rlim = TA ? K : M, clim = TA ? M : K;
        if constexpr (VEC) {
          ra[p] = (r < rlim && c < clim) ? *reinterpret_cast<const float4*>(A + r * lda + c)
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
        } else {
          float t[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) t[e] = (r < rlim && c + e < clim) ? A[r * lda + c + e] : 0.f;
          ra[p] = make_float4(t[0], t[1], t[2], t[3]);
        }
      }
    };
    // op(B)[k][j]: !TB -> B[k*ldb + j] (vector along j); TB -> B[j*ldb + k] (vector along k).
    auto loadB = [&](int64_t k0) {
#pragma unroll
      for (int p = 0; p < NB; ++p) {
        const int idx = tid + p * 256;
        int64_t r, c;
        if constexpr (TB) { r = j0 + idx / 4; c = k0 + (idx % 4) * 4; }
        else { r = k0 + idx / (BN / 4); c = j0 + (idx % (BN / 4)) * 4; }
        const int64_t rlim = TB ? N : K, clim = TB ? K : N;
        if constexpr (VEC) {
          rb[p] = (r < rlim && c < clim) ? *reinterpret_cast<const float4*>(B + r * ldb + c)
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
        } else {
          float t[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) t[e] = (r < rlim && c + e < clim) ? B[r * ldb + c + e] : 0.f;
          rb[p] = make_float4(t[0], t[1], t[2], t[3]);
        }
      }
    };
    auto store = [&](int buf, int64_t k0) {
#pragma unroll
      for (int p = 0; p < NA; ++p) {
        const int idx = tid + p * 256;
        if constexpr (!TA) {
          *reinterpret_cast<float4*>(&sA[buf][(idx / 4) * LDK + (idx % 4) * 4]) = ra[p];
        } else {
          const int k = idx / (BM / 4), i = (idx % (BM / 4)) * 4;
          sA[buf][(i + 0) * LDK + k] = ra[p].x;
          sA[buf][(i + 1) * LDK + k] = ra[p].y;
          sA[buf][(i + 2) * LDK + k] = ra[p].z;
          sA[buf][(i + 3) * LDK + k] = ra[p].w;
        }
      }
#pragma unroll
      for (int p = 0; p < NB; ++p) {
        const int idx = tid + p * 256;
        if constexpr (TB) {
          *reinterpret_cast<float4*>(&sB[buf][(idx / 4) * LDK + (idx % 4) * 4]) = rb[p];
        } else {
          const int k = idx / (BN / 4), j = (idx % (BN / 4)) * 4;
          sB[buf][(j + 0) * LDK + k] = rb[p].x;
          sB[buf][(j + 1) * LDK + k] = rb[p].y;
          sB[buf][(j + 2) * LDK + k] = rb[p].z;
          sB[buf][(j + 3) * LDK + k] = rb[p].w;
        }
      }
      (void)k0;
    };

    const int nk = (int)((kend - kbeg + BK - 1) / BK);
    loadA(kbeg);
    loadB(kbeg);
    store(0, kbeg);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const int64_t knext = kbeg + (int64_t)(kt + 1) * BK;
      if (kt + 1 < nk) { loadA(knext); loadB(knext); }
      const int h = lane >> 5;
      float av[FM][8], bv[FN][8];
#pragma unroll
      for (int a = 0; a < FM; ++a) {
        const float* p = &sA[cur][(wm * (BM / 2) + a * 32 + (lane & 31)) * LDK + h * 8];
        const float4 x0 = *reinterpret_cast<const float4*>(p);
        const float4 x1 = *reinterpret_cast<const float4*>(p + 4);
        av[a][0] = x0.x; av[a][1] = x0.y; av[a][2] = x0.z; av[a][3] = x0.w;
        av[a][4] = x1.x; av[a][5] = x1.y; av[a][6] = x1.z; av[a][7] = x1.w;
      }
#pragma unroll
      for (int c = 0; c < FN; ++c) {
        const float* p = &sB[cur][(wn * (BN / 2) + c * 32 + (lane & 31)) * LDK + h * 8];
        const float4 x0 = *reinterpret_cast<const float4*>(p);
        const float4 x1 = *reinterpret_cast<const float4*>(p + 4);
        bv[c][0] = x0.x; bv[c][1] = x0.y; bv[c][2] = x0.z; bv[c][3] = x0.w;
        bv[c][4] = x1.x; bv[c][5] = x1.y; bv[c][6] = x1.z; bv[c][7] = x1.w;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
          for (int c = 0; c < FN; ++c)
            acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a][u], bv[c][u], acc[a][c], 0, 0, 0);
      if (kt + 1 < nk) store(cur ^ 1, knext);
      __syncthreads();
    }
  }

  // Epilogue.  32x32 accumulator layout: lane l, element v -> row (v/4)*8 + (l/32)*4 + v%4,
  // column l%32.
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int c = 0; c < FN; ++c) {
      const int64_t j = j0 + wn * (BN / 2) + c * 32 + (lane & 31);
      if (j >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t i = i0 + wm * (BM / 2) + a * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        if (i < M) {
          float* p = C + i * ldc + j;
          const float r = alpha * acc[a][c][v];
          *p = beta == 0.0f ? r : r + beta * *p;
        }
      }
    }
}

template <int BM, int BN, bool TA, bool TB>
hipError_t launch_shape(const GemmArgs& g, bool vec, hipStream_t s) {
  dim3 grid((unsigned)((g.N + BN - 1) / BN), (unsigned)((g.M + BM - 1) / BM));
  if (vec) {
    hipLaunchKernelGGL((gemm_f32_kernel<BM, BN, TA, TB, true>), grid, dim3(256), 0, s, g.M, g.N,
                       g.K, g.A, g.lda, g.B, g.ldb, g.C, g.ldc, g.alpha, g.beta, g.kmode,
                       (int)g.lower_only);
  } else {
    hipLaunchKernelGGL((gemm_f32_kernel<BM, BN, TA, TB, false>), grid, dim3(256), 0, s, g.M, g.N,
                       g.K, g.A, g.lda, g.B, g.ldb, g.C, g.ldc, g.alpha, g.beta, g.kmode,
                       (int)g.lower_only);
  }
  return hipGetLastError();
}

template <int BM, int BN>
hipError_t launch_tile(const GemmArgs& g, bool vec, hipStream_t s) {
  if (!g.transA && !g.transB) return launch_shape<BM, BN, false, false>(g, vec, s);
  if (!g.transA && g.transB) return launch_shape<BM, BN, false, true>(g, vec, s);
  if (g.transA && !g.transB) return launch_shape<BM, BN, true, false>(g, vec, s);
  return launch_shape<BM, BN, true, true>(g, vec, s);
}

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_gemm_f32(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const bool vec = al16(g.A) && al16(g.B) && g.lda % 4 == 0 && g.ldb % 4 == 0 &&
                   g.M % 4 == 0 && g.N % 4 == 0 && g.K % 4 == 0;
  // 128x128 tiles when that still fills the chip, else 64x64.
  const int64_t big = ((g.M + 127) / 128) * ((g.N + 127) / 128);
  if (big >= 512) return launch_tile<128, 128>(g, vec, s);
  return launch_tile<64, 64>(g, vec, s);
}

}  // namespace gptq
