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

template <int BM, int BN, int NS, bool TA, bool TB, bool X3>
__global__ void __launch_bounds__(256)
gemm_f32_dma(int64_t M, int64_t N, int64_t K, const float* __restrict__ A, int64_t lda,
             const float* __restrict__ B, int64_t ldb, float* __restrict__ C, int64_t ldc,
             float alpha, float beta, int kmode, int lower_only, int tiles_n,
             const float* __restrict__ row_scale) {
  constexpr bool AKC = !TA, BKC = TB;  // k-contiguous in memory
  using TA_ = OpTile<BM, AKC>;
  using TB_ = OpTile<BN, BKC>;
  constexpr int FM = BM / 64, FN = BN / 64;
  constexpr int IPW = TA_::IPW + TB_::IPW;
  constexpr int STAGE = TA_::FLOATS + TB_::FLOATS;
  static_assert(NS == 2 || NS == 3, "2 or 3 stages");
  __shared__ __align__(16) float st0[STAGE];
  __shared__ __align__(16) float st1[STAGE];
  __shared__ __align__(16) float st2[NS == 3 ? STAGE : 4];

  // Tile order.  Full K: XCD-contiguous runs of the row-major order (blocks
  // are dispatched to the 8 XCDs round-robin, so neighbouring tiles share an
  // L2).  Triangular K ranges: the tiles with the most k go first (longest
  // processing time first), so the last wave is not a few long tiles.
  const int nb = gridDim.x, b = blockIdx.x;
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
  // Per-row scale of this lane's A fragment rows (X3 with row_scale only).
  float rsa[FM];
#pragma unroll
  for (int a = 0; a < FM; ++a) {
    const int64_t r = i0 + wm * (BM / 2) + a * 32 + (lane & 31);
    rsa[a] = (X3 && row_scale != nullptr && r < M) ? row_scale[r] : 1.0f;
  }
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
      for (int a = 0; a < FM; ++a) {
#pragma unroll
        for (int u = 0; u < 16; ++u) av[a][u] *= rsa[a];
        split16(av[a], ah[a], al[a]);
      }
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
    float ralpha[16];  // alpha / row_scale of each accumulator row
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t r = i0 + wm * (BM / 2) + a * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
      ralpha[v] = (X3 && row_scale != nullptr && r < M) ? alpha / row_scale[r] : alpha;
    }
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
        const float r = ralpha[v] * acc[a][c][v];
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(rd ? r + beta * cv[v] : r), rc,
                                              (int)off[v], 0, 0);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Error-update GEMM of the column sweep: C -= E V^T on two fp16 products.
//   E  fp32 [M x K] (row-major, k-contiguous; each row scaled by a power of
//      two first, from the sweeps' per-row error maxima over the K range),
//      split x = hi + lo as split16 does;
//   V  fp16 [N x K] (k-contiguous: the coefficient matrix stored transposed
//      and rounded to nearest fp16 once);
//   C  fp32 [M x N] -= (E_hi V + E_lo V) / scale.
// 128 x 128 tiles, four 64 x 64 waves, 32 k per stage, three stages of
// direct-to-LDS loads.  The fp16 rows of V are 64 bytes per stage: chunk c
// of row r sits at c ^ ((r >> 2) & 3), so a 16-lane pass of 16-byte reads of
// 16 consecutive rows covers all 64 banks.
constexpr int E2_BM = 128, E2_BN = 128, E2_NS = 3;  // 72 KiB of LDS: two workgroups per CU
constexpr int E2_AIPW = E2_BM / 32;      // fp32 A: 4 KiB per wave-wide load round
constexpr int E2_BIPW = E2_BN / 64;      // fp16 B: 64 rows x 64 bytes per round
constexpr int E2_AF = E2_BM * DK;        // floats per A stage
constexpr int E2_BH = E2_BN * DK;        // halves per B stage

__global__ void __launch_bounds__(256)
gemm_e2_dma(int64_t M, int64_t N, int64_t K, const float* __restrict__ A, int64_t lda,
            const _Float16* __restrict__ B, int64_t ldb, float* __restrict__ C, int64_t ldc,
            const float* __restrict__ emax, int64_t eld, int64_t eb0, int64_t eb1) {
  __shared__ __align__(16) float sa[E2_NS][E2_AF];
  __shared__ __align__(16) _Float16 sb[E2_NS][E2_BH];
  __shared__ float rsl[E2_BM];
  using TA_ = OpTile<E2_BM, true>;
  static_assert(TA_::IPW == E2_AIPW, "A loads per wave");

  const int nb = gridDim.x, b = blockIdx.x;
  const int tiles_n = (int)((N + E2_BN - 1) / E2_BN);
  const int t = (nb % 8 == 0) ? (b % 8) * (nb / 8) + b / 8 : b;
  const int ti = t / tiles_n, tj = t % tiles_n;
  const int64_t i0 = (int64_t)ti * E2_BM, j0 = (int64_t)tj * E2_BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1, h = lane >> 5;

  // Row scales of the tile: 2^(14 - e) for the rows' largest error m = f 2^e
  // (f in [0.5, 1)) over the K range's blocks, so every scaled error is below
  // 2^14.  Two threads per row, each every second block, eight loads in
  // flight (a K range holds up to in / block blocks).
  {
    const int rr = tid & (E2_BM - 1), half = tid >> 7;
    const int64_t r = i0 + rr;
    float m = 0.0f;
    if (r < M) {
      int64_t k = eb0 + half;
      for (; k + 14 < eb1; k += 16) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = emax[(k + 2 * u) * eld + r];
#pragma unroll
        for (int u = 0; u < 8; ++u) m = fmaxf(m, v[u]);
      }
      for (; k < eb1; k += 2) m = fmaxf(m, emax[k * eld + r]);
    }
    if (half) rsl[rr] = m;
    __syncthreads();
    if (!half) {
      m = fmaxf(m, rsl[rr]);
      int e = 0;
      (void)frexpf(m, &e);
      rsl[rr] = (m > 0.0f && m < INFINITY) ? ldexpf(1.0f, 14 - e) : 1.0f;
    }
  }

  const float* abase = A + i0 * lda;
  const int64_t aext = ((M - i0 - 1) * lda + K) * 4;
  const _Float16* bbase = B + j0 * ldb;
  const int64_t bext = ((N - j0 - 1) * ldb + K) * 2;
  const int nk = (int)(K / DK);
  uint32_t va[E2_AIPW], vb[E2_BIPW];
#pragma unroll
  for (int q = 0; q < E2_AIPW; ++q) va[q] = TA_::voff(wave, q, lane, lda);
#pragma unroll
  for (int q = 0; q < E2_BIPW; ++q) {
    const int slot = (wave * E2_BIPW + q) * 64 + lane;
    const int row = slot >> 2, lch = (slot & 3) ^ ((row >> 2) & 3);
    vb[q] = (uint32_t)(((int64_t)row * ldb + lch * 8) * 2);
  }
  auto issue = [&](int st, int buf) __device__ __attribute__((always_inline)) {
    const bool live = st < nk;
    issue_stage<E2_AIPW>(live ? (const char*)abase + (int64_t)st * DK * 4 : (const char*)A,
                         live ? aext - (int64_t)st * DK * 4 : 0, va,
                         &sa[buf][0] + wave * E2_AIPW * 256);
    __amdgpu_buffer_rsrc_t rs = rsrc(live ? (const char*)bbase + (int64_t)st * DK * 2 : (const char*)B,
                                     live ? bext - (int64_t)st * DK * 2 : 0);
#pragma unroll
    for (int q = 0; q < E2_BIPW; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, GPTQ_LDS(&sb[buf][0] + (wave * E2_BIPW + q) * 512), 16, vb[q], 0, 0, 0);
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][c][v] = 0.0f;

#pragma unroll
  for (int st = 0; st + 1 < E2_NS; ++st) issue(st, st);
  __syncthreads();  // row scales
  float rsa[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) rsa[a] = rsl[wm * 64 + a * 32 + (lane & 31)];

  auto compute = [&](int buf) __device__ __attribute__((always_inline)) {
    float av[2][16];
#pragma unroll
    for (int a = 0; a < 2; ++a) TA_::frag(&sa[buf][0], wm * 64 + a * 32 + (lane & 31), h, av[a]);
    half8_t bq[2][2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = wn * 64 + c * 32 + (lane & 31);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int ph = (2 * h + q) ^ ((row >> 2) & 3);
        bq[c][q] = *reinterpret_cast<const half8_t*>(&sb[buf][row * DK + ph * 8]);
      }
    }
    half8_t ah[2][2], al[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int u = 0; u < 16; ++u) av[a][u] *= rsa[a];
      split16(av[a], ah[a], al[a]);
    }
    // MFMA k-step q takes this lane's k = 16 h + 8 q + e (e < 8) of A and B
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(al[a][q], bq[c][q], acc[a][c], 0, 0, 0);
          acc[a][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah[a][q], bq[c][q], acc[a][c], 0, 0, 0);
        }
  };
  constexpr int IPW = E2_AIPW + E2_BIPW;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt % E2_NS;
    wait_vmcnt<(E2_NS - 2) * IPW>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    issue(kt + E2_NS - 1, (kt + E2_NS - 1) % E2_NS);
    compute(buf);
  }
  wait_vmcnt<0>();

  // C += -acc / scale, through a buffer descriptor (outside rows / columns dropped)
  const int64_t cext = ((M - i0 - 1) * ldc + (N - j0)) * 4;
  __amdgpu_buffer_rsrc_t rc = rsrc(C + i0 * ldc + j0, cext);
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    float ralpha[16];
#pragma unroll
    for (int v = 0; v < 16; ++v)
      ralpha[v] = -1.0f / rsl[wm * 64 + a * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3)];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int jl = wn * 64 + c * 32 + (lane & 31);
      uint32_t off[16];
      float cv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int il = wm * 64 + a * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        const bool in = i0 + il < M && j0 + jl < N;
        off[v] = in ? (uint32_t)(((int64_t)il * ldc + jl) * 4) : 0x80000000u;
        cv[v] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rc, (int)off[v], 0, 0));
      }
#pragma unroll
      for (int v = 0; v < 16; ++v)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(fmaf(ralpha[v], acc[a][c][v], cv[v])),
                                              rc, (int)off[v], 0, 0);
    }
  }
}

template <int BM, int BN, int NS, bool TA, bool TB, bool X3>
hipError_t launch_dma(const GemmArgs& g, hipStream_t s) {
  const int64_t tm = (g.M + BM - 1) / BM, tn = (g.N + BN - 1) / BN;
  hipLaunchKernelGGL((gemm_f32_dma<BM, BN, NS, TA, TB, X3>), dim3((unsigned)(tm * tn)), dim3(256),
                     0, s, g.M, g.N, g.K, g.A, g.lda, g.B, g.ldb, g.C, g.ldc, g.alpha, g.beta,
                     g.kmode, (int)g.lower_only, (int)tn, g.row_scale);
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

hipError_t launch_gemm_e2(int64_t M, int64_t N, int64_t K, const float* E, int64_t lde,
                          const _Float16* V, int64_t ldv, float* C, int64_t ldc,
                          const float* emax, int64_t eld, int64_t eb0, int64_t eb1,
                          hipStream_t s) {
  if (M <= 0 || N <= 0 || K <= 0) return hipSuccess;
  if (K % DK != 0 || lde % 4 != 0 || ldv % 8 != 0 || !al16(E) ||
      (reinterpret_cast<uintptr_t>(V) & 15) != 0)
    return hipErrorInvalidValue;
  const int64_t tiles = ((M + E2_BM - 1) / E2_BM) * ((N + E2_BN - 1) / E2_BN);
  hipLaunchKernelGGL(gemm_e2_dma, dim3((unsigned)tiles), dim3(256), 0, s, M, N, K, E, lde, V, ldv,
                     C, ldc, emax, eld, eb0, eb1);
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
