// fp32 GEMM on the gfx950 matrix cores (v_mfma_f32_32x32x2_f32):
//     C[M x N] = alpha * op(A) op(B) + beta * C, row-major operands.
//
// Used by the factorization (triangular products and the symmetric rank-k
// update of the recursive Cholesky/inverse) and by the lazy trailing update
// of the quantization sweep (W[:, right] -= E[:, left] * U'[left, right]).
// fp32 operands keep the sweep's accumulated error at fp32 level.
//
// Two kernels:
//  * gemm_f32_dma (16-byte aligned operands, K a multiple of 32): both
//    operands go straight from memory to LDS with buffer_load ... lds (no
//    register staging), NS-stage ring, 32 k per stage.  Each operand keeps its
//    memory layout in LDS: a k-contiguous operand (A not transposed, B
//    transposed) as rows of 32 floats whose 16-byte chunks are XOR-swizzled
//    by row % 8, read 4 k at a time with ds_read_b128; an m/n-contiguous
//    operand as 32 rows of k, read one float per lane (a half-wave reads 128
//    contiguous bytes).  Masked output elements get buffer offsets past the
//    descriptor's range, so the epilogue is branch-free.
//  * gemm_f32_kernel (anything else): register-staged double buffer, BK = 16.
//
// In one 32x32x2 MFMA the two lane halves carry two different k.  Any fixed
// assignment of k to (MFMA, half) gives the same sum as long as A and B use
// the same one.
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

// ---------------------------------------------------------------------------
// Direct-to-LDS kernel.
constexpr int DK = 32;  // k per stage

// LDS image of one operand tile for one stage: R rows (of M or N) x DK.
// K-contiguous: [R][8 chunks of 4 floats], chunk c of row r at c ^ (r % 8).
// MN-contiguous: [DK][R].
template <int R, bool KC>
struct OpTile {
  static constexpr int FLOATS = R * DK;
  static constexpr int IPW = R / 32;  // buffer_load_lds per wave (4 waves, 64 x 16 B each)
  // Byte offset (from the operand's stage base) lane `lane` of instruction q of
  // wave `wave` loads; the instruction's LDS destination is chunk (wave*IPW+q)*64.
  __device__ static uint32_t voff(int wave, int q, int lane, int64_t ld) {
    const int slot = (wave * IPW + q) * 64 + lane;
    if constexpr (KC) {
      const int row = slot >> 3, lch = (slot & 7) ^ (row & 7);
      return (uint32_t)(((int64_t)row * ld + lch * 4) * 4);
    } else {
      const int krow = slot / (R / 4), ch = slot % (R / 4);
      return (uint32_t)(((int64_t)krow * ld + ch * 4) * 4);
    }
  }
  // The 16 k values (k = 16 h + u, u < 16) of row/column `r` for lane half h.
  __device__ static void frag(const float* t, int r, int h, float (&v)[16]) {
    if constexpr (KC) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 x = *reinterpret_cast<const float4*>(t + r * DK + (((4 * h + c) ^ (r & 7)) * 4));
        v[4 * c + 0] = x.x; v[4 * c + 1] = x.y; v[4 * c + 2] = x.z; v[4 * c + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = t[(16 * h + u) * R + r];
    }
  }
};

// LDS destination of a direct load (generic -> LDS address space).
#define GPTQ_LDS(p) \
  ((__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) char*)(char*)(p)))

__device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int num = bytes <= 0 ? 0 : bytes > 0x7FFFFFFFLL ? 0x7FFFFFFF : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, num, 0x00020000);
}

// 16 fp32 values -> fp16 high parts and fp16 remainders, as two 8-element
// MFMA operands each.  hi = x with the mantissa cut to 10 bits (exact in
// fp16 in its normal range), lo = x - hi (exact in fp32) rounded toward zero
// to fp16: |x - hi - lo| <= 2^-20 |x| there, and <= 2^-24 in absolute terms
// below it.  Three VALU ops per value (and, sub, half of two packed cvts).
__device__ __attribute__((always_inline)) inline void split16(const float (&v)[16], half8_t (&hi)[2],
                                                              half8_t (&lo)[2]) {
#pragma unroll
  for (int e = 0; e < 16; e += 2) {
    const float h0 = __uint_as_float(__float_as_uint(v[e]) & 0xFFFFE000u);
    const float h1 = __uint_as_float(__float_as_uint(v[e + 1]) & 0xFFFFE000u);
    const auto hp = __builtin_amdgcn_cvt_pkrtz(h0, h1);
    const auto lp = __builtin_amdgcn_cvt_pkrtz(v[e] - h0, v[e + 1] - h1);
    hi[e >> 3][e & 7] = hp[0];
    hi[e >> 3][(e & 7) + 1] = hp[1];
    lo[e >> 3][e & 7] = lp[0];
    lo[e >> 3][(e & 7) + 1] = lp[1];
  }
}

// IPW direct loads of 64 x 16 bytes from `base` (byte extent `bytes`; 0 = all
// zeros) into consecutive 1 KiB pieces of LDS starting at `lds`.
template <int IPW>
__device__ __attribute__((always_inline)) inline void issue_stage(const char* base, int64_t bytes,
                                                                  const uint32_t* voff,
                                                                  float* lds) {
  __amdgpu_buffer_rsrc_t rs = rsrc(base, bytes);
#pragma unroll
  for (int q = 0; q < IPW; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, GPTQ_LDS(lds + q * 256), 16, voff[q], 0, 0, 0);
}

// One workgroup's tile of a product: block b of the product's nb blocks,
// the stage buffers st0..st2 (LDS objects of the calling kernel, one per
// stage, STAGE floats each; st2 unused with two stages).
template <int BM, int BN, bool TA, bool TB>
struct DmaShape {
  using TA_ = OpTile<BM, !TA>;
  using TB_ = OpTile<BN, TB>;
  static constexpr int STAGE = TA_::FLOATS + TB_::FLOATS;
};
template <int BM, int BN, int NS, bool TA, bool TB, bool X3>
__device__ __attribute__((always_inline)) inline void gemm_f32_dma_tile(
    int b, int nb, int64_t M, int64_t N, int64_t K, const float* __restrict__ A, int64_t lda,
    const float* __restrict__ B, int64_t ldb, float* __restrict__ C, int64_t ldc, float alpha,
    float beta, int kmode, int lower_only, int tiles_n, float* st0, float* st1, float* st2) {
  constexpr bool AKC = !TA, BKC = TB;  // k-contiguous in memory
  using TA_ = OpTile<BM, AKC>;
  using TB_ = OpTile<BN, BKC>;
  constexpr int FM = BM / 64, FN = BN / 64;
  constexpr int IPW = TA_::IPW + TB_::IPW;
  static_assert(NS == 2 || NS == 3, "2 or 3 stages");

  // Tile order.  Full K: XCD-contiguous runs of the row-major order (blocks
  // are dispatched to the 8 XCDs round-robin, so neighbouring tiles share an
  // L2).  Triangular K ranges: the tiles with the most k go first (longest
  // processing time first), so the last wave is not a few long tiles.
  const int tiles_m = nb / tiles_n;
  int ti, tj;
  if (kmode == KR_LE_COL) {
    tj = tiles_n - 1 - b / tiles_m; ti = b % tiles_m;
  } else if (kmode == KR_GE_COL) {
    tj = b / tiles_m; ti = b % tiles_m;
  } else if (kmode == KR_LE_ROW) {
    ti = tiles_m - 1 - b / tiles_n; tj = b % tiles_n;
  } else {
    const int t = (nb % 8 == 0) ? (b % 8) * (nb / 8) + b / 8 : b;
    ti = t / tiles_n; tj = t % tiles_n;
  }
  const int64_t i0 = (int64_t)ti * BM, j0 = (int64_t)tj * BN;
  if (lower_only && j0 >= i0 + BM) return;

  int64_t kbeg = 0, kend = K;
  if (kmode == KR_LE_COL) kend = j0 + BN < K ? j0 + BN : K;
  else if (kmode == KR_GE_COL) kbeg = j0;
  else if (kmode == KR_LE_ROW) kend = i0 + BM < K ? i0 + BM : K;
  kbeg = kbeg / DK * DK;
  const int nk = kend > kbeg ? (int)((kend - kbeg + DK - 1) / DK) : 0;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  // Operand bases at k = kbeg and their byte extents (rows/columns past the
  // matrix read as zero or only feed masked outputs).
  const float* abase = AKC ? A + i0 * lda + kbeg : A + kbeg * lda + i0;
  const int64_t aext = AKC ? ((M - i0 - 1) * lda + (K - kbeg)) * 4 : ((K - kbeg - 1) * lda + (M - i0)) * 4;
  const float* bbase = BKC ? B + j0 * ldb + kbeg : B + kbeg * ldb + j0;
  const int64_t bext = BKC ? ((N - j0 - 1) * ldb + (K - kbeg)) * 4 : ((K - kbeg - 1) * ldb + (N - j0)) * 4;
  const int64_t astep = AKC ? DK * 4 : DK * lda * 4;  // bytes per stage
  const int64_t bstep = BKC ? DK * 4 : DK * ldb * 4;

  uint32_t va[TA_::IPW], vb[TB_::IPW];
#pragma unroll
  for (int q = 0; q < TA_::IPW; ++q) va[q] = TA_::voff(wave, q, lane, lda);
#pragma unroll
  for (int q = 0; q < TB_::IPW; ++q) vb[q] = TB_::voff(wave, q, lane, ldb);

  auto issue = [&](int s, float* stage) __device__ __attribute__((always_inline)) {
    const bool live = s < nk;
    issue_stage<TA_::IPW>(live ? (const char*)abase + s * astep : (const char*)A,
                          live ? aext - s * astep : 0, va, stage + wave * TA_::IPW * 256);
    issue_stage<TB_::IPW>(live ? (const char*)bbase + s * bstep : (const char*)B,
                          live ? bext - s * bstep : 0, vb, stage + TA_::FLOATS + wave * TB_::IPW * 256);
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int a = 0; a < FM; ++a)
#pragma unroll
    for (int c = 0; c < FN; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][c][v] = 0.0f;

  const int h = lane >> 5;
  auto compute = [&](const float* stage) __device__ __attribute__((always_inline)) {
    float av[FM][16], bv[FN][16];
#pragma unroll
    for (int a = 0; a < FM; ++a) TA_::frag(stage, wm * (BM / 2) + a * 32 + (lane & 31), h, av[a]);
#pragma unroll
    for (int c = 0; c < FN; ++c)
      TB_::frag(stage + TA_::FLOATS, wn * (BN / 2) + c * 32 + (lane & 31), h, bv[c]);
    if constexpr (!X3) {
#pragma unroll
      for (int u = 0; u < 16; ++u)
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
          for (int c = 0; c < FN; ++c)
            acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[a][u], bv[c][u], acc[a][c], 0, 0, 0);
    } else {
      // Split fp16 products: x = hi + lo (split16), a b ~ a_hi b_hi +
      // a_hi b_lo + a_lo b_hi with fp32 accumulation.  MFMA
      // k-step q (16 k) takes this lane's values 8q..8q+7 (k = 16h + 8q + e).
      half8_t ah[FM][2], al[FM][2], bh[FN][2], bl[FN][2];
#pragma unroll
      for (int a = 0; a < FM; ++a) split16(av[a], ah[a], al[a]);
#pragma unroll
      for (int c = 0; c < FN; ++c) split16(bv[c], bh[c], bl[c]);
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int a = 0; a < FM; ++a)
#pragma unroll
          for (int c = 0; c < FN; ++c) {
            acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[a][q], bh[c][q], acc[a][c], 0, 0, 0);
            acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[a][q], bl[c][q], acc[a][c], 0, 0, 0);
            acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[a][q], bh[c][q], acc[a][c], 0, 0, 0);
          }
    }
  };
  // Stage k: own loads of k landed, barrier (everyone's landed, everyone is
  // done reading k - 1), refill k - 1's buffer with k + NS - 1, compute k.
  auto step = [&](int k, const float* cur, float* prev) __device__ __attribute__((always_inline)) {
    wait_vmcnt<(NS - 2) * IPW>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    issue(k + NS - 1, prev);
    compute(cur);
  };

  if (nk > 0) {
    issue(0, st0);
    if constexpr (NS == 3) issue(1, st1);
    int kt = 0;
    if constexpr (NS == 2) {
      for (; kt + 2 <= nk; kt += 2) {
        step(kt, st0, st1);
        step(kt + 1, st1, st0);
      }
      if (kt < nk) step(kt, st0, st1);
    } else {
      for (; kt + 3 <= nk; kt += 3) {
        step(kt, st0, st2);
        step(kt + 1, st1, st0);
        step(kt + 2, st2, st1);
      }
      if (kt < nk) step(kt, st0, st2);
      if (kt + 1 < nk) step(kt + 1, st1, st0);
    }
    wait_vmcnt<0>();
  }

  // Epilogue: C tile through a buffer descriptor, 16 elements per 32 x 32 block.
  const int64_t cext = ((M - i0 - 1) * ldc + (N - j0)) * 4;
  __amdgpu_buffer_rsrc_t rc = rsrc(C + i0 * ldc + j0, cext);
  const bool rd = beta != 0.0f;
#pragma unroll
  for (int a = 0; a < FM; ++a) {
#pragma unroll
    for (int c = 0; c < FN; ++c) {
      const int jl = wn * (BN / 2) + c * 32 + (lane & 31);
      uint32_t off[16];
      float cv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int il = wm * (BM / 2) + a * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        const bool in = i0 + il < M && j0 + jl < N;
        off[v] = in ? (uint32_t)(((int64_t)il * ldc + jl) * 4) : 0x80000000u;
        cv[v] = rd ? __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rc, (int)off[v], 0, 0))
                   : 0.0f;
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float r = alpha * acc[a][c][v];
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(rd ? r + beta * cv[v] : r), rc,
                                              (int)off[v], 0, 0);
      }
    }
  }
}

template <int BM, int BN, int NS, bool TA, bool TB, bool X3>
__global__ void __launch_bounds__(256)
gemm_f32_dma(int64_t M, int64_t N, int64_t K, const float* __restrict__ A, int64_t lda,
             const float* __restrict__ B, int64_t ldb, float* __restrict__ C, int64_t ldc,
             float alpha, float beta, int kmode, int lower_only, int tiles_n) {
  constexpr int STAGE = DmaShape<BM, BN, TA, TB>::STAGE;
  __shared__ __align__(16) float st0[STAGE];
  __shared__ __align__(16) float st1[STAGE];
  __shared__ __align__(16) float st2[NS == 3 ? STAGE : 4];
  gemm_f32_dma_tile<BM, BN, NS, TA, TB, X3>(blockIdx.x, gridDim.x, M, N, K, A, lda, B, ldb, C,
                                            ldc, alpha, beta, kmode, lower_only, tiles_n, st0,
                                            st1, st2);
}

// Two independent products in one launch (blocks [0, nb1) take the first,
// the rest the second), both with A not transposed, sharing the stage
// buffers; the first takes its B transposed, the second not.  Each block
// computes exactly what it would in a launch of its own.
struct DmaProblem {
  int64_t M, N, K;
  const float* A; int64_t lda;
  const float* B; int64_t ldb;
  float* C; int64_t ldc;
  float alpha, beta;
  int kmode, lower_only, tiles_n, nb;
};
template <int BM, int BN, int NS, bool X3>
__global__ void __launch_bounds__(256)
gemm_f32_dma_pair(DmaProblem p, DmaProblem q) {
  constexpr int S1 = DmaShape<BM, BN, false, true>::STAGE, S2 = DmaShape<BM, BN, false, false>::STAGE;
  constexpr int STAGE = S1 > S2 ? S1 : S2;
  __shared__ __align__(16) float st0[STAGE];
  __shared__ __align__(16) float st1[STAGE];
  __shared__ __align__(16) float st2[NS == 3 ? STAGE : 4];
  const int b = blockIdx.x;
  if (b < p.nb)
    gemm_f32_dma_tile<BM, BN, NS, false, true, X3>(b, p.nb, p.M, p.N, p.K, p.A, p.lda, p.B,
                                                   p.ldb, p.C, p.ldc, p.alpha, p.beta, p.kmode,
                                                   p.lower_only, p.tiles_n, st0, st1, st2);
  else
    gemm_f32_dma_tile<BM, BN, NS, false, false, X3>(b - p.nb, q.nb, q.M, q.N, q.K, q.A, q.lda,
                                                    q.B, q.ldb, q.C, q.ldc, q.alpha, q.beta,
                                                    q.kmode, q.lower_only, q.tiles_n, st0, st1,
                                                    st2);
}

// ---------------------------------------------------------------------------
// Error-update GEMM of the column sweep, on errors the sweep stored already
// split:
//   C[M x N] -= sum over the K range's sweep blocks b (32 SPB columns each) of
//               einv[b][r] * (Ehi_b + Elo_b) (Vhi_b + Vlo_b)^T
//   E   the sweep's errors, each row and block scaled by 1 / einv (a power of
//       two), in place of the block's fp32 columns: per 16 columns, 16 fp16
//       high parts then 16 fp16 remainders (64 bytes; row stride lde floats);
//   V   fp16 [N x K] (k-contiguous: U' transposed, rounded to nearest once);
//   Vl  fp16 remainders of U' - V (VLO: a third product, Ehi Vl; else unused);
//   einv fp32 [blocks][eld]: the block's inverse row scales.
// Every product is exact in the fp32 accumulator of its block; a block's sum
// is multiplied by its (exact) power of two and added to the tile's total, so
// rows and blocks of very different magnitude keep their relative precision.
//
// 128 x BN tiles (BN = 256: eight waves; 128: four), each wave a 64 x 64
// block (2 x 2 accumulators plus the total), 32 k per stage, four stages of
// direct-to-LDS loads in flight behind the one being read.  Every stage
// buffer is an LDS object of its own and the loop is unrolled over the four,
// so the compiler tracks each buffer's direct loads separately and waits
// only for the stage it reads (with one indexed array it waits for every
// load in flight before each read, and nothing overlaps).  A stage holds the
// E rows (128 bytes each, 16-byte chunk c of row r at c ^ ((r >> 1) & 7)),
// the V rows (64 bytes, chunk c at c ^ ((r >> 2) & 3)): a 16-lane pass of
// 16-byte reads of 16 consecutive rows covers all 64 banks).  The inverse
// scales of all the call's blocks (at most EH_KB_MAX) are put in LDS before
// the loop: loads into registers inside it, or direct loads into LDS read
// back, made the compiler wait for every stage in flight.
constexpr int EH_BM = 128, EH_NS = 4, EH_KB_MAX = 48;

template <bool VLO, int BN>
struct EhStage {
  static constexpr int NW = 2 * BN / 64;           // waves (2 x BN/64 of 64 x 64): 2 BN threads
  static constexpr int A = EH_BM * DK * 4;         // E image (hi + lo): 16 KiB
  static constexpr int B = BN * DK * 2;            // V image
  static constexpr int BYTES = A + (VLO ? 2 : 1) * B;
  static constexpr int AIPW = A / 1024 / NW;       // 16-byte direct loads per wave
  static constexpr int BIPW = B / 1024 / NW;
  static constexpr int IPW = AIPW + (VLO ? 2 : 1) * BIPW;
};

// 16 bytes from LDS through an LDS-typed pointer (the waitcnt pass then keeps
// its reads apart from the direct loads into the other stage buffers).
__device__ inline half8_t lds_read_h8(const char* p) {
  return *(const __attribute__((address_space(3))) half8_t*)(
      (const __attribute__((address_space(3))) char*)(p));
}

__device__ inline f32x4_t lds_read_f4(const char* base, int off) {
  return *(const __attribute__((address_space(3))) f32x4_t*)(
      (const __attribute__((address_space(3))) char*)(base) + off);
}

template <bool VLO, int SPB, int BN>
__global__ void __launch_bounds__(2 * BN)
gemm_eh_dma(int64_t M, int64_t N, int64_t K, const float* __restrict__ A, int64_t lda,
            const _Float16* __restrict__ B, const _Float16* __restrict__ Bl, int64_t ldb,
            float* __restrict__ C, int64_t ldc, const float* __restrict__ einv, int64_t eld) {
  using S = EhStage<VLO, BN>;
  static_assert(4 % SPB == 0 && EH_NS == 4, "a block of stages ends on a stage buffer");
  __shared__ __align__(16) char st0[S::BYTES];
  __shared__ __align__(16) char st1[S::BYTES];
  __shared__ __align__(16) char st2[S::BYTES];
  __shared__ __align__(16) char st3[S::BYTES];
  __shared__ __align__(16) float scl[EH_KB_MAX * EH_BM];  // inverse scales, [block][tile row]
  constexpr int OB = S::A, OBL = S::A + S::B;

  // Tile order: each XCD (block b -> XCD b % 8) takes a contiguous run of a
  // grouped order (bands of 8 row tiles, column by column, the band's rows
  // inside a column), so the tiles an XCD runs together share A rows and V
  // columns in its L2.
  const int nb = gridDim.x, b = blockIdx.x;
  const int tiles_n = (int)((N + BN - 1) / BN), tiles_m = nb / tiles_n;
  int ti, tj;
  {
    const int x = b % 8, r = b / 8, q = nb / 8, rem = nb % 8;
    const int t = x * q + (x < rem ? x : rem) + r;
    const int band = t / (8 * tiles_n), w = t % (8 * tiles_n);
    const int rows = tiles_m - 8 * band < 8 ? tiles_m - 8 * band : 8;
    tj = w / rows;
    ti = 8 * band + w % rows;
  }
  const int64_t i0 = (int64_t)ti * EH_BM, j0 = (int64_t)tj * BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1, h = lane >> 5;

  const char* abase = reinterpret_cast<const char*>(A + i0 * lda);
  const int64_t aext = ((M - i0 - 1) * lda + K) * 4;
  const char* bbase = reinterpret_cast<const char*>(B + j0 * ldb);
  const char* blbase = VLO ? reinterpret_cast<const char*>(Bl + j0 * ldb) : nullptr;
  const int64_t bext = ((N - j0 - 1) * ldb + K) * 2;
  const int nk = (int)(K / DK);
  uint32_t va[S::AIPW], vb[S::BIPW];
#pragma unroll
  for (int q = 0; q < S::AIPW; ++q) {
    const int slot = (wave * S::AIPW + q) * 64 + lane;
    const int row = slot >> 3, lch = (slot & 7) ^ ((row >> 1) & 7);
    va[q] = (uint32_t)(((int64_t)row * lda + lch * 4) * 4);
  }
#pragma unroll
  for (int q = 0; q < S::BIPW; ++q) {
    const int slot = (wave * S::BIPW + q) * 64 + lane;
    const int row = slot >> 2, lch = (slot & 3) ^ ((row >> 2) & 3);
    vb[q] = (uint32_t)(((int64_t)row * ldb + lch * 8) * 2);
  }
  // (the direct loads go through issue_stage: a load builtin written in
  // the lambda itself keeps the host compiler from emitting the kernel)
  auto issue = [&](int st, char* stage) __device__ __attribute__((always_inline)) {
    const bool live = st < nk;
    issue_stage<S::AIPW>(live ? abase + (int64_t)st * DK * 4 : (const char*)A,
                         live ? aext - (int64_t)st * DK * 4 : 0, va,
                         reinterpret_cast<float*>(stage + wave * S::AIPW * 1024));
    issue_stage<S::BIPW>(live ? bbase + (int64_t)st * DK * 2 : (const char*)B,
                         live ? bext - (int64_t)st * DK * 2 : 0, vb,
                         reinterpret_cast<float*>(stage + OB + wave * S::BIPW * 1024));
    if constexpr (VLO)
      issue_stage<S::BIPW>(live ? blbase + (int64_t)st * DK * 2 : (const char*)Bl,
                           live ? bext - (int64_t)st * DK * 2 : 0, vb,
                           reinterpret_cast<float*>(stage + OBL + wave * S::BIPW * 1024));
  };

  f32x16_t acc[2][2], tot[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        acc[a][c][v] = 0.0f;
        tot[a][c][v] = 0.0f;
      }

  // MFMA k-step q takes k = 16 q + 8 h + e (e < 8): E chunks 4q + h (high
  // parts) and 4q + 2 + h (remainders), V chunk 2q + h.  first: the stage
  // opens a block (its sums start from zero); last: it closes one (tot +=
  // einv * acc).
  // This lane's LDS byte offsets inside a stage buffer, computed once (a
  // single offset from the buffer keeps every read attributable to its LDS
  // object, which is what lets the compiler wait only for that stage).
  int offah[2][2], offal[2][2], offb[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int row = wm * 64 + a * 32 + (lane & 31), sw = (row >> 1) & 7;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      offah[a][q] = row * 128 + (((4 * q + h) ^ sw) * 16);
      offal[a][q] = row * 128 + (((4 * q + 2 + h) ^ sw) * 16);
    }
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int row = wn * 64 + c * 32 + (lane & 31), sw = (row >> 2) & 3;
#pragma unroll
    for (int q = 0; q < 2; ++q) offb[c][q] = OB + row * 64 + (((2 * q + h) ^ sw) * 16);
  }
  auto compute = [&](const char* stage, int kb, bool first, bool last) __device__ __attribute__((always_inline)) {
    half8_t ah[2][2], al[2][2], bh[2][2], bl[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        ah[a][q] = lds_read_h8(stage + offah[a][q]);
        al[a][q] = lds_read_h8(stage + offal[a][q]);
      }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        bh[c][q] = lds_read_h8(stage + offb[c][q]);
        if constexpr (VLO) bl[c][q] = lds_read_h8(stage + (offb[c][q] + (OBL - OB)));
      }
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          f32x16_t x = acc[a][c];
          if (first && q == 0) {
#pragma unroll
            for (int v = 0; v < 16; ++v) x[v] = 0.0f;
          }
          if constexpr (VLO) x = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[a][q], bl[c][q], x, 0, 0, 0);
          x = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[a][q], bh[c][q], x, 0, 0, 0);
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[a][q], bh[c][q], x, 0, 0, 0);
        }
    if (last) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          // one opaque offset per read: constant parts split off into
          // further address steps hide the LDS object from the waitcnt pass
          int o = (kb * EH_BM + wm * 64 + a * 32 + g * 8 + h * 4) * 4;
          asm volatile("" : "+v"(o));
          const f32x4_t s4 = lds_read_f4(reinterpret_cast<const char*>(scl), o);
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            tot[a][c][4 * g + 0] = fmaf(s4[0], acc[a][c][4 * g + 0], tot[a][c][4 * g + 0]);
            tot[a][c][4 * g + 1] = fmaf(s4[1], acc[a][c][4 * g + 1], tot[a][c][4 * g + 1]);
            tot[a][c][4 * g + 2] = fmaf(s4[2], acc[a][c][4 * g + 2], tot[a][c][4 * g + 2]);
            tot[a][c][4 * g + 3] = fmaf(s4[3], acc[a][c][4 * g + 3], tot[a][c][4 * g + 3]);
          }
        }
      }
    }
  };
  // Stage kt (buffer kt % 4): own loads of kt landed, barrier (everyone's
  // landed, nobody reads kt - 1 any more), refill kt - 1's buffer with
  // kt + 3, compute kt.  Stages past K read zeros (zero-size descriptor):
  // whole rounds of four stages, no data-dependent branches.
  auto step = [&](int kt, const char* cur, char* prev, int u) __device__ __attribute__((always_inline)) {
    const int kb = kt / SPB;
    wait_vmcnt<(EH_NS - 2) * S::IPW>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    issue(kt + EH_NS - 1, prev);
    compute(cur, kb, u % SPB == 0, u % SPB == SPB - 1);
  };
  // Every block's inverse scales of the tile's rows (rows past M: 0) are
  // loaded before the first stages (so waiting for them does not wait for
  // the stages) and stored to LDS after; the first step's barrier makes
  // them visible.
  constexpr int SPT = EH_KB_MAX * EH_BM / (S::NW * 64);  // scales per thread, at most
  float sv[SPT];
#pragma unroll
  for (int u = 0; u < SPT; ++u) {
    const int e = tid + u * S::NW * 64;
    const int64_t r = i0 + (e % EH_BM);
    sv[u] = (e < (nk / SPB) * EH_BM && r < M) ? einv[(int64_t)(e / EH_BM) * eld + r] : 0.0f;
  }
  issue(0, st0);
  issue(1, st1);
  issue(2, st2);
#pragma unroll
  for (int u = 0; u < SPT; ++u) scl[tid + u * S::NW * 64] = sv[u];
  for (int kt = 0; kt < nk; kt += 4) {
    step(kt + 0, st0, st3, 0);
    step(kt + 1, st1, st0, 1);
    step(kt + 2, st2, st1, 2);
    step(kt + 3, st3, st2, 3);
  }
  wait_vmcnt<0>();

  // C -= tot, through a buffer descriptor (outside rows / columns dropped)
  const int64_t cext = ((M - i0 - 1) * ldc + (N - j0)) * 4;
  __amdgpu_buffer_rsrc_t rc = rsrc(C + i0 * ldc + j0, cext);
#pragma unroll
  for (int a = 0; a < 2; ++a) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int jl = wn * 64 + c * 32 + (lane & 31);
      uint32_t off[16];
      float cv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int il = wm * 64 + a * 32 + (v >> 2) * 8 + h * 4 + (v & 3);
        const bool in = i0 + il < M && j0 + jl < N;
        off[v] = in ? (uint32_t)(((int64_t)il * ldc + jl) * 4) : 0x80000000u;
        cv[v] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rc, (int)off[v], 0, 0));
      }
#pragma unroll
      for (int v = 0; v < 16; ++v)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(cv[v] - tot[a][c][v]), rc,
                                              (int)off[v], 0, 0);
    }
  }
}

template <int BM, int BN, int NS, bool TA, bool TB, bool X3>
hipError_t launch_dma(const GemmArgs& g, hipStream_t s) {
  const int64_t tm = (g.M + BM - 1) / BM, tn = (g.N + BN - 1) / BN;
  hipLaunchKernelGGL((gemm_f32_dma<BM, BN, NS, TA, TB, X3>), dim3((unsigned)(tm * tn)), dim3(256),
                     0, s, g.M, g.N, g.K, g.A, g.lda, g.B, g.ldb, g.C, g.ldc, g.alpha, g.beta,
                     g.kmode, (int)g.lower_only, (int)tn);
  return hipGetLastError();
}

template <int BM, int BN, int NS, bool X3>
hipError_t launch_dma_t(const GemmArgs& g, hipStream_t s) {
  if (!g.transA && !g.transB) return launch_dma<BM, BN, NS, false, false, X3>(g, s);
  if (!g.transA && g.transB) return launch_dma<BM, BN, NS, false, true, X3>(g, s);
  if (g.transA && !g.transB) return launch_dma<BM, BN, NS, true, false, X3>(g, s);
  return launch_dma<BM, BN, NS, true, true, X3>(g, s);
}

}  // namespace

hipError_t launch_gemm_eh(int64_t M, int64_t N, int64_t K, const float* E, int64_t lde,
                          const _Float16* V, const _Float16* Vl, int64_t ldv, float* C,
                          int64_t ldc, const float* einv, int64_t eld, int kb, hipStream_t s) {
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  if (K % kb != 0 || (kb != 32 && kb != 64 && kb != 128) || lde % 4 != 0 || ldv % 8 != 0 ||
      !al16(E) || (reinterpret_cast<uintptr_t>(V) & 15) != 0 ||
      (Vl && (reinterpret_cast<uintptr_t>(Vl) & 15) != 0) || (reinterpret_cast<uintptr_t>(einv) & 3))
    return hipErrorInvalidValue;
  if (K > (int64_t)EH_KB_MAX * kb) {  // sequential launches of at most EH_KB_MAX blocks each
    for (int64_t k0 = 0; k0 < K; k0 += (int64_t)EH_KB_MAX * kb) {
      const int64_t kc = K - k0 < (int64_t)EH_KB_MAX * kb ? K - k0 : (int64_t)EH_KB_MAX * kb;
      GPTQ_HIP_TRY(launch_gemm_eh(M, N, kc, E + k0, lde, V + k0, Vl ? Vl + k0 : nullptr, ldv, C,
                                  ldc, einv + (k0 / kb) * eld, eld, kb, s));
    }
    return hipSuccess;
  }
  const int64_t tm = (M + EH_BM - 1) / EH_BM;
  // 128 x 256 tiles from half a round of them on (C3's 4096 x 2688 x 2816:
  // 194 -> 173 us, 4096 x 1408 x 1408: 63 -> 47 us; a third of a round, at
  // 4096 x 640 x 768, 21 -> 25 us), for two-product 128-column blocks (the
  // per-stage block sums of smaller blocks do not fit the registers of eight
  // waves); else 128 x 128
  const bool wide = !Vl && kb == 128 && tm * ((N + 255) / 256) >= 128;
  const int bn = wide ? 256 : 128;
  const dim3 grid((unsigned)(tm * ((N + bn - 1) / bn)));
#define GPTQ_EH(VL, SPB, BN)                                                                    \
  hipLaunchKernelGGL((gemm_eh_dma<VL, SPB, BN>), grid, dim3(EhStage<VL, BN>::NW * 64), 0, s, M, \
                     N, K, E, lde, V, Vl, ldv, C, ldc, einv, eld)
  if (Vl) {
    if (kb == 32) GPTQ_EH(true, 1, 128);
    else if (kb == 64) GPTQ_EH(true, 2, 128);
    else GPTQ_EH(true, 4, 128);
  } else if (wide) {
    GPTQ_EH(false, 4, 256);
  } else {
    if (kb == 32) GPTQ_EH(false, 1, 128);
    else if (kb == 64) GPTQ_EH(false, 2, 128);
    else GPTQ_EH(false, 4, 128);
  }
#undef GPTQ_EH
  return hipGetLastError();
}

// The conditions under which launch_gemm_f32 takes 64 x 64 tiles, three
// stages and split fp16 products for g.
bool dma64_split(const GemmArgs& g) {
  const bool vec = al16(g.A) && al16(g.B) && g.lda % 4 == 0 && g.ldb % 4 == 0 &&
                   g.M % 4 == 0 && g.N % 4 == 0 && g.K % 4 == 0;
  const int64_t big = ((g.M + 127) / 128) * ((g.N + 127) / 128);
  return g.M > 0 && g.N > 0 && vec && g.K % DK == 0 && g.K > 0 && g.split16 && big < 256;
}

hipError_t launch_gemm_f32_pair(const GemmArgs& g1, const GemmArgs& g2, hipStream_t s) {
  if (!(dma64_split(g1) && dma64_split(g2) && !g1.transA && g1.transB && !g2.transA &&
        !g2.transB)) {
    GPTQ_HIP_TRY(launch_gemm_f32(g1, s));
    return launch_gemm_f32(g2, s);
  }
  auto prob = [](const GemmArgs& g) {
    const int64_t tm = (g.M + 63) / 64, tn = (g.N + 63) / 64;
    return DmaProblem{g.M, g.N, g.K, g.A, g.lda, g.B, g.ldb, g.C, g.ldc, g.alpha, g.beta,
                      g.kmode, (int)g.lower_only, (int)tn, (int)(tm * tn)};
  };
  const DmaProblem p = prob(g1), q = prob(g2);
  hipLaunchKernelGGL((gemm_f32_dma_pair<64, 64, 3, true>), dim3((unsigned)(p.nb + q.nb)), dim3(256),
                     0, s, p, q);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  const bool vec = al16(g.A) && al16(g.B) && g.lda % 4 == 0 && g.ldb % 4 == 0 &&
                   g.M % 4 == 0 && g.N % 4 == 0 && g.K % 4 == 0;
  const int64_t big = ((g.M + 127) / 128) * ((g.N + 127) / 128);
  if (vec && g.K % DK == 0 && g.K > 0) {
    // 128x128 tiles when that still fills the chip, else 64x64.
    if (g.split16) {
      if (big >= 256) return launch_dma_t<128, 128, 2, true>(g, s);
      return launch_dma_t<64, 64, 3, true>(g, s);
    }
    if (big >= 256) return launch_dma_t<128, 128, 2, false>(g, s);
    return launch_dma_t<64, 64, 3, false>(g, s);
  }
  if (big >= 512) return launch_tile<128, 128>(g, vec, s);
  return launch_tile<64, 64>(g, vec, s);
}

}  // namespace gptq
