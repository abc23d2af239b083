// gptq_prepare: damping, desc_act column order and U = upper Cholesky factor
// of the inverse damped Hessian, in quantization order.
//
//   damp_percent ("GPTQ > Using AutoGPTQ in Practice", Key Parameters):
//       H_d = H + damp * mean(diag H) * I   (a zero diagonal entry counts as 1)
//   desc_act (same list): quantization order by decreasing diag(H), stable.
//   factor: the sweep adjusts remaining weights using H^-1 (glossary "gptq",
//       "Algorithm" step (2)); the object it needs is U with U^T U = H_p^-1.
//
// Route on the GPU (half the flops of "invert, then factor"): with J the
// index reversal, factor A = J H_p J = L L^T (ordinary lower Cholesky), then
// R = J L J is upper with H_p = R R^T, so H_p^-1 = R^-T R^-1 and U = R^-1 =
// J L^-1 J.  L and L^-1 are computed together by one recursion
//     [A11 .  ]    L11 = chol(A11), X11 = L11^-1            (recursive)
//     [A21 A22] -> L21 = A21 X11^T,  A22 -= L21 L21^T       (MFMA GEMMs)
//                  T2 = L21 X11                             (MFMA GEMM)
//                  L22 = chol(A22), X22 = L22^-1            (recursive)
//                  X21 = -X22 T2                            (MFMA GEMM)
// whose leaves (<= 128 columns) run in one workgroup out of LDS.  X = L^-1 is
// built directly in the output buffer and finally moved in place to
// U[i][j] = X[n-1-i][n-1-j].
//
// Scaling: the recursion runs on A' = D A D with D = diag(2^-e_i) chosen so
// that A'_ii lies in [0.5, 2) (exact: powers of two).  Then L' = D L, every
// |L'_ij| < 1.5, and X' = L'^-1 = X D^-1, so X = X' D is recovered exactly.
// With entries of order one the recursion's products can run as split fp16
// MFMAs (three fp16 products per fp32 product, fp32 accumulation).
#include "common.hpp"

namespace gptq {
namespace {

constexpr int NB = 128;  // leaf order of the recursion

__global__ void fill_f32_kernel(float* p, int64_t count, float v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

__device__ inline uint32_t order_key(float d) {
  // Monotone map float -> uint32 (ascending).  -0 counts as +0; NaN sorts lowest.
  if (d != d) return 0u;
  if (d == 0.0f) d = 0.0f;
  const uint32_t u = __float_as_uint(d);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One workgroup: keys of the raw diagonal, mean of the (dead-fixed) diagonal,
// damp_add = damp * mean; clears info and the rank counters.
__global__ void __launch_bounds__(1024)
diag_stats_kernel(const float* __restrict__ H, int64_t n, float damp, uint32_t* __restrict__ keys,
                  int32_t* __restrict__ rank, float* __restrict__ damp_add,
                  int32_t* __restrict__ info) {
  __shared__ double red[1024];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
    const float d = H[i * n + i];
    keys[i] = order_key(d);
    rank[i] = 0;
    s += (double)(d == 0.0f ? 1.0f : d);
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    *damp_add = (float)((double)damp * (red[0] / (double)n));
    *info = 0;
  }
}

// rank(i) = #{j : key_j > key_i, or key_j == key_i and j < i}: decreasing
// key, ties by index (stable).  Block (x, y) counts, for its 256 keys i, the
// keys j of chunk y (RANK_CHUNK of them) and adds the count to rank[i]
// (integer adds: the result does not depend on their order).
constexpr int RANK_CHUNK = 1024;
__global__ void __launch_bounds__(256)
rank_count_kernel(const uint32_t* __restrict__ keys, int64_t n, int desc,
                  int32_t* __restrict__ rank) {
  __shared__ __align__(16) uint32_t sk[RANK_CHUNK];
  if (!desc) return;
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t c0 = (int64_t)blockIdx.y * RANK_CHUNK;
  const int64_t cn = n - c0 < RANK_CHUNK ? n - c0 : RANK_CHUNK;
  for (int64_t t = threadIdx.x; t < RANK_CHUNK; t += blockDim.x)
    sk[t] = t < cn ? keys[c0 + t] : 0u;
  __syncthreads();
  if (i >= n) return;
  const uint32_t ki = keys[i];
  int cnt = 0;
  if (c0 + cn <= i) {  // every j of the chunk precedes i: ties count
#pragma unroll 4
    for (int t = 0; t < RANK_CHUNK; t += 4) {
      const uint4 k4 = *reinterpret_cast<const uint4*>(sk + t);
      cnt += (k4.x >= ki) + (k4.y >= ki) + (k4.z >= ki) + (k4.w >= ki);
    }
    cnt -= (int)(RANK_CHUNK - cn) * (ki == 0u);  // padding keys are 0
  } else if (c0 > i) {  // every j follows i: strict only
#pragma unroll 4
    for (int t = 0; t < RANK_CHUNK; t += 4) {
      const uint4 k4 = *reinterpret_cast<const uint4*>(sk + t);
      cnt += (k4.x > ki) + (k4.y > ki) + (k4.z > ki) + (k4.w > ki);
    }
  } else {
    for (int t = 0; t < (int)cn; ++t) {
      const uint32_t kj = sk[t];
      cnt += (kj > ki) | ((kj == ki) & (c0 + t < i));
    }
  }
  if (cnt) atomicAdd(rank + i, cnt);
}

// perm[rank(i)] = i (desc_act) or perm[i] = i.
__global__ void rank_scatter_kernel(const int32_t* __restrict__ rank, int64_t n, int desc,
                                    int32_t* __restrict__ perm) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n) return;
  perm[desc ? rank[i] : i] = (int32_t)i;
}

// S = H with the lower triangle mirrored from the upper (S fully symmetric).
// Grid: (nb, nb) 64 x 64 tiles, the workgroups of tiles below the diagonal
// exit at once; tile (bi, bj), bi <= bj, of H's upper part is read once
// (coalesced) and written twice: as is, and transposed through LDS into tile
// (bj, bi) (a diagonal tile mirrors its own upper part).
constexpr int SYM_T = 64;
__global__ void __launch_bounds__(256)
symmetrize_kernel(const float* __restrict__ H, int64_t n, float* __restrict__ S) {
  __shared__ float t[SYM_T][SYM_T + 1];
  const int64_t bi = blockIdx.y, bj = blockIdx.x;
  if (bi > bj) return;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4
  for (int r = ty; r < SYM_T; r += 4) {
    const int64_t i = bi * SYM_T + r, j = bj * SYM_T + tx;
    const float v = (i < n && j < n) ? H[i * n + j] : 0.0f;
    t[r][tx] = v;
    if (bi < bj && i < n && j < n) S[i * n + j] = v;
  }
  __syncthreads();
  for (int r = ty; r < SYM_T; r += 4) {
    const int64_t i = bj * SYM_T + r, j = bi * SYM_T + tx;
    if (i < n && j < n) S[i * n + j] = (bi < bj || r > tx) ? t[tx][r] : t[r][tx];
  }
}

// dsc[a] = 2^-floor(E/2) where d = m 2^E (m in [0.5, 1)) is the damped,
// dead-fixed diagonal entry at position a of A (q(a) = perm[n-1-a]), so that
// d * dsc^2 lies in [0.5, 2).
__global__ void scale_kernel(const float* __restrict__ H, int64_t n,
                             const int32_t* __restrict__ perm, const float* __restrict__ damp_add,
                             float* __restrict__ dsc) {
  const int64_t a = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (a >= n) return;
  const int64_t q = perm[n - 1 - a];
  const float h = H[q * n + q];
  const float d = (h == 0.0f ? 1.0f : h) + *damp_add;
  int e = 0;
  (void)frexpf(d, &e);
  dsc[a] = (d > 0.0f && d < INFINITY) ? ldexpf(1.0f, -(e >> 1)) : 1.0f;
}

// A[a][b] (b <= a) = dsc[a] dsc[b] S[q(a)][q(b)] with q(a) = perm[n-1-a];
// diagonal: dead fix + damp before scaling.  256 threads; 512 where the
// staged row leaves room for at most four workgroups per compute unit (n
// above 8192), 1024 where it leaves room for at most two (n above 16384), so
// that enough loads are in flight.
__global__ void __launch_bounds__(1024)
gather_kernel(const float* __restrict__ S, int64_t n, const int32_t* __restrict__ perm,
              const float* __restrict__ damp_add, const float* __restrict__ dsc,
              float* __restrict__ A) {
  extern __shared__ __align__(16) float row[];
  const int64_t a = blockIdx.x;
  const int64_t src = perm[n - 1 - a];
  // Stage the source row, 4 float4 loads per thread in flight.
  if (((n & 3) | (reinterpret_cast<uintptr_t>(S) & 15)) == 0) {
    const float4* s4 = reinterpret_cast<const float4*>(S + src * n);
    float4* r4 = reinterpret_cast<float4*>(row);
    const int64_t n4 = n / 4;
    for (int64_t t0 = threadIdx.x; t0 < n4; t0 += 4 * (int64_t)blockDim.x) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t t = t0 + u * (int64_t)blockDim.x;
        v[u] = t < n4 ? s4[t] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t t = t0 + u * (int64_t)blockDim.x;
        if (t < n4) r4[t] = v[u];
      }
    }
  } else {
    for (int64_t t = threadIdx.x; t < n; t += blockDim.x) row[t] = S[src * n + t];
  }
  __syncthreads();
  const float dadd = *damp_add, da = dsc[a];
  // 8 elements per thread in flight (the loop is latency-bound otherwise).
  for (int64_t b0 = threadIdx.x; b0 <= a; b0 += 8 * (int64_t)blockDim.x) {
    int32_t q[8];
    float sc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t b = b0 + u * (int64_t)blockDim.x;
      q[u] = b <= a ? perm[n - 1 - b] : 0;
      sc[u] = b <= a ? dsc[b] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t b = b0 + u * (int64_t)blockDim.x;
      if (b <= a) {
        float v = row[q[u]];
        if (b == a) v = (v == 0.0f ? 1.0f : v) + dadd;
        A[a * n + b] = (v * da) * sc[u];
      }
    }
  }
}

// Leaf of the recursion: X = L^-1 for the m x m (m <= NB) diagonal block at
// `off` (lower part of A, leading dimension n), in one workgroup of 8 waves
// out of LDS, blocked by 16 columns.  Per 16-column step c:
//   (a) wave 0 factors the 16 x 16 diagonal block in registers (readlane
//       broadcasts, one rsqrt per pivot);
//   (b) every row below is solved against the new block by forward
//       substitution (one thread per row);
//   (c) the trailing lower block is updated in 16 x 16 tiles on the matrix
//       cores (v_mfma_f32_16x16x4f32).
// Then the eight diagonal blocks are inverted, one per wave, all at once
// (inside the step loop the inversion of the previous block on a second wave
// took longer than the factorization and held up every step: 4.9 k against
// 3.9 k cycles), and the off-diagonal blocks of X are formed by doubling
// (blocks of 32, 64, 128):
//   T = L21 X11, X21 = -X22 T, again in 16 x 16 MFMA tiles over all waves.
// Rows >= m are padded with the identity (so every pivot is defined).  Only
// X is written back (lower part, rows and columns < m): the recursion never
// reads L again.  L and X share one LDS array: L in the strict lower
// triangle, X transposed in the upper one and on the diagonal
// (X[i][j], i >= j, at [j][i]; L's own diagonal is not read once the
// reciprocals 1 / L_jj are kept).  68 KiB instead of 135: the leaf then fits
// on a compute unit beside a GEMM workgroup of the helper streams, instead
// of waiting for one to drain (leaves waited 15 us on average at n = 11008
// and 65 us at n = 28672 with L and X apart).
constexpr int LP = NB + 4;  // padded LDS row (16-byte aligned rows)
constexpr int LEAF_THREADS = 512;
constexpr int NSTEP = NB / 16;

__device__ inline float bcast(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// d += c[lane o of this 16-lane row] * ng in one instruction (v_fmac_f32
// with a DPP row_newbcast source; o must be a constant after unrolling).
// "first" puts two wait states in front: DPP may not read a register that
// a VALU instruction wrote less than two instructions before, and c is
// computed just before the first use.
#define GPTQ_FMAC_BCAST(O)                                                          \
  case O:                                                                           \
    if (first)                                                                      \
      asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:" #O            \
                   " row_mask:0xf bank_mask:0xf"                                    \
                   : "+v"(d)                                                        \
                   : "v"(c), "v"(ng));                                              \
    else                                                                            \
      asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:" #O                     \
                   " row_mask:0xf bank_mask:0xf"                                    \
                   : "+v"(d)                                                        \
                   : "v"(c), "v"(ng));                                              \
    break;
__device__ inline void fmac_bcast(float& d, float c, float ng, int o, bool first) {
  switch (o) {
    GPTQ_FMAC_BCAST(0) GPTQ_FMAC_BCAST(1) GPTQ_FMAC_BCAST(2) GPTQ_FMAC_BCAST(3)
    GPTQ_FMAC_BCAST(4) GPTQ_FMAC_BCAST(5) GPTQ_FMAC_BCAST(6) GPTQ_FMAC_BCAST(7)
    GPTQ_FMAC_BCAST(8) GPTQ_FMAC_BCAST(9) GPTQ_FMAC_BCAST(10) GPTQ_FMAC_BCAST(11)
    GPTQ_FMAC_BCAST(12) GPTQ_FMAC_BCAST(13) GPTQ_FMAC_BCAST(14) GPTQ_FMAC_BCAST(15)
    default: break;
  }
}
#undef GPTQ_FMAC_BCAST

// acc += sgn * sum_{k<K} a(r, k) b(k, c) for one 16 x 16 tile (v_mfma_f32_16x16x4f32:
// lane l supplies a(l%16, k0 + l/16) and b(k0 + l/16, l%16) and holds rows
// 4(l/16)..+3 of column l%16).  a(r, k) = A[r*LP + k]; b(k, c) = BT ? B[c*LP + k] : B[k*LP + c].
// All operands are read first and the K/4 products go to up to four
// accumulators in turn, so neither the LDS latency nor the MFMA latency
// serializes the loop.
template <bool BT, int K>
__device__ inline f32x4_t tile16(const float* A, const float* B, f32x4_t acc, float sgn,
                                  int lane) {
  const int r = lane & 15, kq = lane >> 4;
  constexpr int NK = K / 4, NA = NK < 4 ? NK : 4;
  float a[NK], b[NK];
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    a[i] = sgn * A[r * LP + 4 * i + kq];
    b[i] = BT ? B[r * LP + 4 * i + kq] : B[(4 * i + kq) * LP + r];
  }
  f32x4_t part[NA];
  part[0] = acc;
#pragma unroll
  for (int p = 1; p < NA; ++p) part[p] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < NK; ++i)
    part[i % NA] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], part[i % NA], 0, 0, 0);
#pragma unroll
  for (int p = 1; p < NA; ++p) part[0] += part[p];
  return part[0];
}
__device__ inline f32x4_t load_tile(const float* C, int lane) {
  f32x4_t v;
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = C[(4 * (lane >> 4) + q) * LP + (lane & 15)];
  return v;
}
__device__ inline void store_tile(float* C, f32x4_t v, int lane) {
#pragma unroll
  for (int q = 0; q < 4; ++q) C[(4 * (lane >> 4) + q) * LP + (lane & 15)] = v[q];
}

// One doubling level of the leaf's inverse: for each pair of SZ-blocks on the
// diagonal, T = L21 X11 (into the X21 area), then X21 = -X22 T.  X (and T)
// are read and written transposed in the upper triangle of Ls; the zeros of
// the triangular X11 and X22 (whose places hold L) are supplied by masks.
// Tiles as tile16: lane l supplies a(l%16, k) and b(k, l%16) for k = 4i + l/16
// and holds rows 4(l/16)..+3 of column l%16; the K/4 products go to up to four
// accumulators in turn.
template <int SZ>
__device__ inline void doubling_level(float* Ls, int wave, int lane) {
  constexpr int PER = (SZ / 16) * (SZ / 16), TILES = (NB / (2 * SZ)) * PER;
  constexpr int NWAVE = LEAF_THREADS / 64, HOLD = (TILES + NWAVE - 1) / NWAVE;
  constexpr int NK = SZ / 4, NA = NK < 4 ? NK : 4;
  const int r = lane & 15, kq = lane >> 4;
  auto mma = [&](const float (&a)[NK], const float (&b)[NK]) {
    f32x4_t part[NA];
#pragma unroll
    for (int p = 0; p < NA; ++p) part[p] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NK; ++i)
      part[i % NA] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], part[i % NA], 0, 0, 0);
#pragma unroll
    for (int p = 1; p < NA; ++p) part[0] += part[p];
    return part[0];
  };
  // element (4(l/16) + q, l%16) of the tile at rows/columns (ri, cj) of the
  // X21 area (block rows o+SZ.., columns o..), stored transposed
  auto store_t = [&](int o, int ri, int cj, f32x4_t v) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      Ls[(o + cj + r) * LP + o + SZ + ri + 4 * kq + q] = v[q];
  };
  for (int t = wave; t < TILES; t += NWAVE) {
    const int o = (t / PER) * 2 * SZ, ti = (t % PER) / (SZ / 16), tj = (t % PER) % (SZ / 16);
    // T[16ti + .][16tj + c] = sum_k L[o+SZ+16ti+.][o+k] X11[k][16tj + c]   (X11[k][c] = 0 for k < c)
    float a[NK], b[NK];
    const int c = 16 * tj + r;
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      const int k = 4 * i + kq;
      a[i] = Ls[(o + SZ + 16 * ti + r) * LP + o + k];
      b[i] = k >= c ? Ls[(o + c) * LP + o + k] : 0.0f;
    }
    store_t(o, 16 * ti, 16 * tj, mma(a, b));
  }
  __syncthreads();
  f32x4_t res[HOLD];
#pragma unroll
  for (int h = 0; h < HOLD; ++h) {
    const int t = wave + h * NWAVE;
    res[h] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    if (t < TILES) {
      const int o = (t / PER) * 2 * SZ, ti = (t % PER) / (SZ / 16), tj = (t % PER) % (SZ / 16);
      // X21[16ti + i][.] = -sum_k X22[16ti + i][k] T[k][.]   (X22[i][k] = 0 for k > i)
      float a[NK], b[NK];
      const int ri = 16 * ti + r;
#pragma unroll
      for (int i = 0; i < NK; ++i) {
        const int k = 4 * i + kq;
        a[i] = k <= ri ? -Ls[(o + SZ + k) * LP + o + SZ + ri] : 0.0f;
        b[i] = Ls[(o + 16 * tj + r) * LP + o + SZ + k];
      }
      res[h] = mma(a, b);
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < HOLD; ++h) {
    const int t = wave + h * NWAVE;
    if (t < TILES) {
      const int o = (t / PER) * 2 * SZ, ti = (t % PER) / (SZ / 16), tj = (t % PER) % (SZ / 16);
      store_t(o, 16 * ti, 16 * tj, res[h]);
    }
  }
  __syncthreads();
}

__global__ void __launch_bounds__(LEAF_THREADS)
cholinv_leaf_kernel(const float* __restrict__ A, float* __restrict__ X, int64_t n, int64_t off,
                    int m, int32_t* __restrict__ info) {
  __shared__ __align__(16) float Ls[NB * LP];  // L lower, X transposed upper and diagonal
  __shared__ float rinv_s[NB];  // 1 / L_jj
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15;

  // Whole blocks with 16-byte aligned rows move as float4 (all eight loads
  // of a thread in flight at once); ragged or unaligned blocks element-wise.
  const bool vec = m == NB && (n & 3) == 0 && (off & 3) == 0;
  if (vec) {
    constexpr int PER4 = NB * NB / 4 / LEAF_THREADS;
    float4 v[PER4];
#pragma unroll
    for (int u = 0; u < PER4; ++u) {
      const int e = tid + LEAF_THREADS * u, i = e / (NB / 4), j = 4 * (e % (NB / 4));
      v[u] = *reinterpret_cast<const float4*>(A + (off + i) * n + off + j);
    }
#pragma unroll
    for (int u = 0; u < PER4; ++u) {
      const int e = tid + LEAF_THREADS * u, i = e / (NB / 4), j = 4 * (e % (NB / 4));
      float4 l;
      l.x = j + 0 <= i ? v[u].x : 0.0f;
      l.y = j + 1 <= i ? v[u].y : 0.0f;
      l.z = j + 2 <= i ? v[u].z : 0.0f;
      l.w = j + 3 <= i ? v[u].w : 0.0f;
      *reinterpret_cast<float4*>(Ls + i * LP + j) = l;
    }
  } else {
    // 8 loads per thread in flight (addresses of masked-out elements are
    // clamped to the block's first element).
    constexpr int PER = NB * NB / LEAF_THREADS;
#pragma unroll
    for (int q0 = 0; q0 < PER; q0 += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = tid + LEAF_THREADS * (q0 + u), i = e / NB, j = e % NB;
        const bool ok = i < m && j <= i;
        v[u] = A[ok ? (off + i) * n + off + j : off * n + off];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = tid + LEAF_THREADS * (q0 + u), i = e / NB, j = e % NB;
        const bool ok = i < m && j <= i;
        Ls[i * LP + j] = ok ? v[u] : (i == j ? 1.0f : 0.0f);
      }
    }
  }
  __syncthreads();

  // Y = (diagonal block b of L)^-1, by one wave (lanes 0..15 hold rows):
  // row k of Y = (e_k - sum_{j<k} L_kj Y_j) / L_kk, rows broadcast by readlane;
  // stored transposed into the block's upper part and diagonal.
  auto invert_block = [&](int b) {
    const int c = 16 * b;
    float d[16], y[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      d[j] = j < li ? Ls[(c + li) * LP + c + j] : 0.0f;
      y[j] = j == li ? 1.0f : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if (li == k) {
        const float rk = rinv_s[c + k];
#pragma unroll
        for (int j = 0; j <= k; ++j) y[j] *= rk;
      }
      const float g = li > k ? d[k] : 0.0f;
#pragma unroll
      for (int j = 0; j <= k; ++j) y[j] = fmaf(-g, bcast(y[j], k), y[j]);
    }
    if (lane < 16) {
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j <= li) Ls[(c + j) * LP + c + li] = y[j];
    }
  };

  // Trailing update of the lower part after the panel of columns cp..cp+15,
  // one 16 x 16 tile (ti, tj) on the matrix cores:
  //     A[r][s] -= sum_q L[r][cp+q] L[s][cp+q]   (r >= s >= cp + 16)
  auto tile_update = [&](int cp, int ti, int tj) {
    const int base = cp + 16;
    float* C = Ls + (base + 16 * ti) * LP + base + 16 * tj;
    f32x4_t acc = load_tile(C, lane);
    acc = tile16<true, 16>(Ls + (base + 16 * ti) * LP + cp, Ls + (base + 16 * tj) * LP + cp, acc,
                           -1.0f, lane);
    store_tile(C, acc, lane);
  };

  // Right-looking over 16-column steps with a lookahead of one: each step's
  // trailing update is split into the next column block (tj = 0), which the
  // next diagonal block and panel need at once, and the rest, which waves
  // 1.. apply while wave 0 factors the next diagonal block.
#pragma unroll 1
  for (int step = 0; step < NSTEP; ++step) {
    const int c = 16 * step;
    if (wave == 0) {
      // (a) 16 x 16 diagonal block: Cholesky in registers.  The first bad
      // pivot and the reciprocals are recorded after the loop (no branches
      // inside it).
      float d[16], rv[16];
      const float* rowp = Ls + (c + li) * LP + c;
#pragma unroll
      for (int j = 0; j < 16; j += 4) {
        const float4 v = *reinterpret_cast<const float4*>(rowp + j);
        d[j] = v.x; d[j + 1] = v.y; d[j + 2] = v.z; d[j + 3] = v.w;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) d[j] = j <= li ? d[j] : 0.0f;
      // Pivot k: column k of L is c = d[k] / sqrt(d_kk) in the rows >= k
      // (0 above, where the lanes hold upper-triangle entries); every lane
      // then takes d[j] -= c * c_j for j > k, c_j arriving from lane j by a
      // DPP broadcast fused into the FMA.  Lane k also updates its own
      // upper entries (k, j > k): garbage that the store masks.
      int fail = -1;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float dk = bcast(d[k], k);
        if (fail < 0 && !(dk > 0.0f && dk < INFINITY) && c + k < m) fail = k;
        const float r = __builtin_amdgcn_rsqf(dk);
        rv[k] = r;  // 1 / L[k][k]
        const float ck = li >= k ? d[k] * r : 0.0f;
        d[k] = ck;
        const float ng = -ck;
#pragma unroll
        for (int j = k + 1; j < 16; ++j) fmac_bcast(d[j], ck, ng, j, j == k + 1);
        // two wait states before the next pivot's broadcast of d[k + 1]
        asm volatile("s_nop 1");
      }
      if (lane < 16) {
        float* wrow = Ls + (c + li) * LP + c;
#pragma unroll
        for (int j = 0; j < 16; j += 4)
          *reinterpret_cast<float4*>(wrow + j) = make_float4(j + 0 <= li ? d[j] : 0.0f, j + 1 <= li ? d[j + 1] : 0.0f,
                                                           j + 2 <= li ? d[j + 2] : 0.0f, j + 3 <= li ? d[j + 3] : 0.0f);
      }
      if (lane == 0) {
        if (fail >= 0) atomicCAS(info, 0, (int32_t)(n - (off + c + fail)));  // quantization-order column
#pragma unroll
        for (int k = 0; k < 16; ++k) rinv_s[c + k] = rv[k];
      }
    } else if (step > 0) {
      // (c2) the previous step's update beyond its next column block:
      // tiles 1 <= tj <= ti < nt, over waves 1..
      const int cp = c - 16, nt = (NB - cp - 16) / 16;
      for (int t = wave - 1; t < (nt - 1) * nt / 2; t += LEAF_THREADS / 64 - 1) {
        int u = 0;
        while ((u + 1) * (u + 2) / 2 <= t) ++u;
        tile_update(cp, u + 1, t - u * (u + 1) / 2 + 1);
      }
    }
    __syncthreads();
    const int rows = NB - c - 16;
    if (rows > 0) {
      // (b) L[i][c+j] = (A[i][c+j] - sum_{q<j} L[i][c+q] L[c+j][c+q]) / L[c+j][c+j]
      if (tid < rows) {
        float* row = Ls + (c + 16 + tid) * LP + c;
        float x[16];
#pragma unroll
        for (int q = 0; q < 16; q += 4) {
          const float4 v = *reinterpret_cast<const float4*>(row + q);
          x[q] = v.x; x[q + 1] = v.y; x[q + 2] = v.z; x[q + 3] = v.w;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float* lj = Ls + (c + j) * LP + c;  // same address in every lane
          float sacc = x[j];
#pragma unroll
          for (int q = 0; q < j; ++q) sacc = fmaf(-x[q], lj[q], sacc);
          x[j] = sacc * rinv_s[c + j];
        }
#pragma unroll
        for (int q = 0; q < 16; q += 4)
          *reinterpret_cast<float4*>(row + q) = make_float4(x[q], x[q + 1], x[q + 2], x[q + 3]);
      }
      __syncthreads();
      // (c1) this step's update of the next column block: tiles (ti, 0)
      for (int t = wave; t < rows / 16; t += LEAF_THREADS / 64) tile_update(c, t, 0);
      __syncthreads();
    }
  }
  static_assert(NSTEP <= LEAF_THREADS / 64, "one diagonal block per wave");
  if (wave < NSTEP) invert_block(wave);
  __syncthreads();

  // Off-diagonal blocks of X by doubling: for blocks of 2s (s = 16, 32, 64)
  //   T = L21 X11 (into the X21 area), X21 = -X22 T,
  // with every level's tiles spread over the 8 waves (16 x 16 MFMA tiles).
  doubling_level<16>(Ls, wave, lane);
  doubling_level<32>(Ls, wave, lane);
  doubling_level<64>(Ls, wave, lane);
  static_assert(NB == 128, "three doubling levels");

  if (vec) {
    // whole rows of the block, zeros above the diagonal
#pragma unroll
    for (int u = 0; u < NB * NB / 4 / LEAF_THREADS; ++u) {
      const int e = tid + LEAF_THREADS * u, i = e / (NB / 4), j = 4 * (e % (NB / 4));
      float4 v;
      v.x = j + 0 <= i ? Ls[(j + 0) * LP + i] : 0.0f;
      v.y = j + 1 <= i ? Ls[(j + 1) * LP + i] : 0.0f;
      v.z = j + 2 <= i ? Ls[(j + 2) * LP + i] : 0.0f;
      v.w = j + 3 <= i ? Ls[(j + 3) * LP + i] : 0.0f;
      *reinterpret_cast<float4*>(X + (off + i) * n + off + j) = v;
    }
  } else {
    for (int i = tid / NB; i < m; i += LEAF_THREADS / NB) {
      const int j = tid % NB;
      if (j <= i) X[(off + i) * n + off + j] = Ls[j * LP + i];
    }
  }
}


// In place: U[i][j] = X[n-1-i][n-1-j] for i <= j, 0 below the diagonal, where
// X = X' D (column b of the computed X' times dsc[b]).  X' is lower
// triangular, so every strictly lower (a, b) moves to the strictly upper
// (n-1-a, n-1-b) (which holds 0) and diagonal entries swap in pairs.
// Workgroup r takes the source rows r and c = n-1-r: the strictly lower part
// of each lands in the strictly upper part of the other, so the two rows
// hold n-1 moved entries together (every workgroup the same work) and no
// other workgroup touches them; the diagonal pair (r, r), (c, c) is swapped
// by one thread.  For n a multiple of 4 the whole 4-column chunks left of
// the diagonal move as 16-byte loads and stores when U and dsc are 16-byte
// aligned (chunk k of row a lands, reversed, in chunk n/4-1-k of row n-1-a),
// four chunks per thread in flight; the rest column by column.
__global__ void __launch_bounds__(256)
reverse_inplace_kernel(float* __restrict__ U, int64_t n, const float* __restrict__ dsc) {
  const int64_t r = blockIdx.x, c = n - 1 - r;
  if (r > c) return;
  for (int side = 0; side < (r < c ? 2 : 1); ++side) {
    const int64_t a = side ? c : r;
    float* __restrict__ src = U + a * n;
    float* __restrict__ dst = U + (n - 1 - a) * n;
    int64_t b0 = 0;
    if (((n & 3) | (reinterpret_cast<uintptr_t>(U) & 15) | (reinterpret_cast<uintptr_t>(dsc) & 15)) ==
        0) {
      const int64_t full = a >> 2, n4 = n >> 2;  // chunks k with 4k + 3 < a
      float4* s4 = reinterpret_cast<float4*>(src);
      float4* d4 = reinterpret_cast<float4*>(dst);
      const float4* c4 = reinterpret_cast<const float4*>(dsc);
      for (int64_t k0 = threadIdx.x; k0 < full; k0 += 4 * (int64_t)blockDim.x) {
        float4 v[4], sc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t k = k0 + u * (int64_t)blockDim.x;
          if (k < full) {
            v[u] = s4[k];
            sc[u] = c4[k];
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t k = k0 + u * (int64_t)blockDim.x;
          if (k < full) {
            d4[n4 - 1 - k] = make_float4(v[u].w * sc[u].w, v[u].z * sc[u].z, v[u].y * sc[u].y,
                                         v[u].x * sc[u].x);
            s4[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          }
        }
      }
      b0 = full << 2;
    }
    for (int64_t b = b0 + threadIdx.x; b < a; b += blockDim.x) {
      const float v = src[b] * dsc[b];
      dst[n - 1 - b] = v;
      src[b] = 0.0f;
    }
  }
  if (threadIdx.x == 0) {
    if (r < c) {
      const float v = U[r * n + r] * dsc[r];
      U[r * n + r] = U[c * n + c] * dsc[c];
      U[c * n + c] = v;
    } else {
      U[r * n + r] *= dsc[r];
    }
  }
}

struct PrepCtx {
  float* A;
  float* X;
  float* T;    // L21 of the node being processed (reused by every level)
  float* T2;   // stack of L21 X11 blocks, one per recursion depth
  int64_t n;
  int32_t* info;
  hipStream_t s;
};

hipError_t gemm(PrepCtx& c, int64_t M, int64_t N, int64_t K, const float* Am, int64_t lda, bool ta,
                const float* Bm, int64_t ldb, bool tb, float* Cm, int64_t ldc, float alpha,
                float beta, int kmode, bool lower) {
  GemmArgs g{M, N, K, Am, lda, ta, Bm, ldb, tb, Cm, ldc, alpha, beta, kmode, lower};
  g.split16 = true;  // operands are O(1) after the scaling
  return launch_gemm_f32(g, c.s);
}

// Node [off, off + m) with its L21 X11 block at t2 (room for m2 x m1, and
// below it the stack of the deeper levels).  The left child only leaves
// X11 behind for this node; L21 is needed only by the two products issued
// before the right child runs, so it lives in the shared T, and the right
// child's result X22 meets T2 = L21 X11 afterwards.
hipError_t cholinv(PrepCtx& c, int64_t off, int64_t m, float* t2) {
  const int64_t n = c.n;
  if (m <= NB) {
    hipLaunchKernelGGL(cholinv_leaf_kernel, dim3(1), dim3(LEAF_THREADS), 0, c.s, c.A, c.X, n, off,
                       (int)m, c.info);
    return hipGetLastError();
  }
  const int64_t m1 = ((m / 2 + NB - 1) / NB) * NB;
  const int64_t m2 = m - m1;
  float* A21 = c.A + (off + m1) * n + off;
  float* A22 = c.A + (off + m1) * n + off + m1;
  float* X11 = c.X + off * n + off;
  float* X21 = c.X + (off + m1) * n + off;
  float* X22 = c.X + (off + m1) * n + off + m1;
  float* next = t2 + m2 * m1;  // deeper levels
  GPTQ_HIP_TRY(cholinv(c, off, m1, next));
  // L21 = A21 * X11^T  (X11 lower: op(B)[k][j] = X11[j][k] vanishes for k > j)
  GPTQ_HIP_TRY(gemm(c, m2, m1, m1, A21, n, false, X11, n, true, c.T, m1, 1.0f, 0.0f, KR_LE_COL,
                    false));
  // A22 -= L21 L21^T (lower tiles) and T2 = L21 * X11 (X11[k][j] vanishes
  // for k < j): both read only L21 and X11, so one launch carries both
  GemmArgs upd{m2, m2, m1, c.T, m1, false, c.T, m1, true, A22, n, -1.0f, 1.0f, KR_FULL, true};
  GemmArgs t2p{m2, m1, m1, c.T, m1, false, X11, n, false, t2, m1, 1.0f, 0.0f, KR_GE_COL, false};
  upd.split16 = t2p.split16 = true;  // operands are O(1) after the scaling
  GPTQ_HIP_TRY(launch_gemm_f32_pair(upd, t2p, c.s));
  GPTQ_HIP_TRY(cholinv(c, off + m1, m2, next));
  // X21 = -X22 * T2 (X22[i][k] vanishes for k > i)
  GPTQ_HIP_TRY(gemm(c, m2, m1, m2, X22, n, false, t2, m1, false, X21, n, -1.0f, 0.0f, KR_LE_ROW,
                    false));
  return hipSuccess;
}

// Blocked right-looking Cholesky with inversion, W-column blocks j (W from
// outer_width; a block is factored by the recursion above, one leaf when
// W = NB):
//   diag:   L_jj, X_jj = L_jj^-1                        (main stream)
//   panel:  P_j^T = X_jj A[j+1:, j]^T into the unused upper triangle,
//           row block j (so L below the diagonal is kept transposed there)
//   next:   block column j+1 -= P_j P_j[j+1]^T          (main stream)
//   rest:   A[j+2:, j+2:] -= P_j P_j^T, lower tiles     (update stream)
//   inv:    X[j, :j] = -X_jj T_j, T_j = L[j, :j] X[:j, :j]
//                                                       (inverse stream)
// The main stream carries only the diagonal blocks and the two skinny
// products each one needs; the trailing update of step j runs while block
// j+1 factors, and the off-diagonal blocks of X follow on their own
// stream.  Lookahead of one block: "next" of step j+1 waits for "rest" of
// step j (it updates the first columns "rest" wrote).  Products in the
// upper triangle of diagonal tiles (lower-only GEMMs compute whole tiles)
// land in the diagonal blocks' upper parts, which nothing reads.
// Columns per block of the blocked schedule: single leaves up to n = 4096;
// above, the skinny K = 128 products of the update and inverse streams cost
// more than they hide, and wider blocks (factored by the recursion) are
// faster; the trailing update re-reads the trailing matrix once per block,
// about n^3 / (3 W) * 8 bytes, so the largest layers take the widest
// (measured: n = 4096: 2.32 ms at 128, 2.40 at 256; n = 11008: 13.5 ms at
// 128, 10.2 at 512, 10.3 at 1024; n = 28672: 99 ms at 512, 84.8 at 1024,
// 83.9 at 2048, 87.5 at 4096).
constexpr int64_t OUTER_MAX = 2048;
int64_t outer_width(int64_t n) { return n <= 4096 ? NB : n <= 12288 ? 512 : OUTER_MAX; }
hipError_t cholinv_blocked(PrepCtx& c, float* tbuf) {
  const int64_t n = c.n;
  const int64_t W = outer_width(n);
  std::lock_guard<std::mutex> lock(helper_mutex());
  HelperStreams* hs = nullptr;
  GPTQ_HIP_TRY(helper_streams(hs));
  const hipStream_t M = c.s, UPD = hs->a, INV = hs->b;
  hipEvent_t ev_fork = hs->ev[0], ev_step = hs->ev[1], ev_upd = hs->ev[2],
             ev_join_upd = hs->ev[4], ev_join_inv = hs->ev[5];
  PrepCtx cu = c, ci = c;
  cu.s = UPD;
  ci.s = INV;
  GPTQ_HIP_TRY(hipEventRecord(ev_fork, M));
  GPTQ_HIP_TRY(hipStreamWaitEvent(UPD, ev_fork, 0));
  GPTQ_HIP_TRY(hipStreamWaitEvent(INV, ev_fork, 0));
  // One event record and at most one wait per block on the caller's stream
  // (each costs several microseconds of queue latency on the critical
  // chain): the record after the next-block update releases both helper
  // streams.
  // Inverse stream, block j = [o, o + m) once its diagonal block and panel
  // are done: X[j, :j] = -X_jj T_j with T_j = L[j, :j] X[:j, :j].
  // Up to 512-column blocks T is accumulated right-looking,
  // T[j+1:, :j+1] += L[j+1:, j] X[j, :j+1] after block j, so each T_j is
  // complete when its block comes and the work of the late blocks is spread
  // over the schedule (kept transposed in the strict upper triangle of X,
  // zero at the start and free until the reversal: T_j^T = X[:o, o:o+m]).
  // Wider blocks form T_j whole when block j comes (one o x o x m product,
  // into tbuf): there the right-looking updates, each a pass over the
  // trailing part of T, slow the diagonal chain more than the late products
  // cost (measured: n = 11008 8.80 -> 8.45 ms right-looking, n = 4096
  // 2.07 -> 1.99 ms, n = 28672 91 -> 95 ms).
  const bool right_looking = W <= 512;
  auto inverse_step = [&](int64_t o, int64_t m, int64_t rest) -> hipError_t {
    if (!right_looking && o == 0) return hipSuccess;
    GPTQ_HIP_TRY(hipStreamWaitEvent(INV, ev_step, 0));
    if (!right_looking) {
      // T = L[j, :j] X[:j, :j] = (U[:o, o:o+m])^T X[:o, :o]   (X lower: k >= col)
      GPTQ_HIP_TRY(gemm(ci, m, o, o, c.A + o, n, true, c.X, n, false, tbuf, o, 1.0f, 0.0f,
                        KR_GE_COL, false));
      // X[j, :j] = -X_jj T   (X_jj lower: k <= row)
      return gemm(ci, m, o, m, c.X + o * n + o, n, false, tbuf, o, false, c.X + o * n, n, -1.0f,
                  0.0f, KR_LE_ROW, false);
    }
    // X[j, :j] = -X_jj T_j   (X_jj lower: k <= row)
    if (o > 0)
      GPTQ_HIP_TRY(gemm(ci, m, o, m, c.X + o * n + o, n, false, c.X + o, n, true, c.X + o * n, n,
                        -1.0f, 0.0f, KR_LE_ROW, false));
    if (rest == 0) return hipSuccess;
    // T^T[:o+m, o+m:] += X[j, :o+m]^T P_j^T, P_j^T = L[o+m:, j]^T (row block j of A's upper part)
    return gemm(ci, o + m, rest, m, c.X + o * n, n, true, c.A + o * n + o + m, n, false,
                c.X + o + m, n, 1.0f, 1.0f, KR_FULL, false);
  };
  bool pending_rest = false;
  for (int64_t o = 0; o < n; o += W) {
    const int64_t m = n - o < W ? n - o : W;
    const int64_t rest = n - o - m;
    GPTQ_HIP_TRY(cholinv(c, o, m, c.T2));
    if (rest == 0) {
      if (o > 0) {
        GPTQ_HIP_TRY(hipEventRecord(ev_step, M));
        GPTQ_HIP_TRY(inverse_step(o, m, 0));
      }
      break;
    }
    float* U_j = c.A + o * n + o + m;
    // P_j^T = X_jj A[o+m:, o:o+m]^T
    GPTQ_HIP_TRY(gemm(c, m, rest, m, c.X + o * n + o, n, false, c.A + (o + m) * n + o, n, true,
                      U_j, n, 1.0f, 0.0f, KR_LE_ROW, false));
    if (pending_rest) GPTQ_HIP_TRY(hipStreamWaitEvent(M, ev_upd, 0));
    const int64_t m2 = rest < W ? rest : W;
    // block column j+1 (rows o+m..n, m2 columns) -= P_j P_j[0:m2]^T
    GPTQ_HIP_TRY(gemm(c, rest, m2, m, U_j, n, true, U_j, n, false, c.A + (o + m) * n + o + m, n,
                      -1.0f, 1.0f, KR_FULL, true));
    GPTQ_HIP_TRY(hipEventRecord(ev_step, M));
    pending_rest = false;
    GPTQ_HIP_TRY(inverse_step(o, m, rest));
    if (rest > m2) {
      GPTQ_HIP_TRY(hipStreamWaitEvent(UPD, ev_step, 0));
      const int64_t r2 = rest - m2;
      float* C = c.A + (o + m + m2) * n + o + m + m2;
      // the rest of the trailing matrix -= P_j P_j^T (lower tiles)
      GPTQ_HIP_TRY(gemm(cu, r2, r2, m, U_j + m2, n, true, U_j + m2, n, false, C, n, -1.0f, 1.0f,
                        KR_FULL, true));
      GPTQ_HIP_TRY(hipEventRecord(ev_upd, UPD));
      pending_rest = true;
    }
  }
  GPTQ_HIP_TRY(hipEventRecord(ev_join_upd, UPD));
  GPTQ_HIP_TRY(hipEventRecord(ev_join_inv, INV));
  GPTQ_HIP_TRY(hipStreamWaitEvent(M, ev_join_upd, 0));
  GPTQ_HIP_TRY(hipStreamWaitEvent(M, ev_join_inv, 0));
  return hipSuccess;
}

// Floats of the T2 stack for a node of order m (its own block plus the
// deeper levels' largest chain).
int64_t t2_floats(int64_t m) {
  if (m <= NB) return 0;
  const int64_t m1 = ((m / 2 + NB - 1) / NB) * NB;
  const int64_t m2 = m - m1;
  const int64_t a = t2_floats(m1), b = t2_floats(m2);
  return m2 * m1 + (a > b ? a : b);
}

struct PrepLayout {
  float* A;
  float* T;
  float* T2;
  float* TB;
  uint32_t* keys;
  int32_t* rank;
  float* damp_add;
  float* dsc;
  size_t bytes;
};

PrepLayout carve(void* ws, int64_t n) {
  Carver c(ws);
  PrepLayout l;
  // the recursion factors diagonal blocks of at most w columns
  const int64_t w = n < outer_width(n) ? n : outer_width(n);
  const int64_t m1max = ((w / 2 + NB - 1) / NB) * NB;
  l.A = c.take<float>((size_t)n * n);
  // every internal node has m2 <= m1 <= m1max, so m1max^2 holds any L21 block
  l.T = c.take<float>((size_t)(m1max > 0 ? m1max * m1max : 1));
  l.T2 = c.take<float>((size_t)(t2_floats(w) > 0 ? t2_floats(w) : 1));
  // T = L[j, :j] X[:j, :j] of the inverse stream for blocks wider than 512:
  // at most w x n
  l.TB = c.take<float>(w > 512 ? (size_t)w * (size_t)n : 1);
  l.keys = c.take<uint32_t>((size_t)n);
  l.rank = c.take<int32_t>((size_t)n);
  l.damp_add = c.take<float>(1);
  l.dsc = c.take<float>((size_t)n);
  l.bytes = c.used;
  return l;
}

}  // namespace

size_t prepare_workspace_bytes(int64_t n) { return carve(nullptr, n).bytes; }

hipError_t launch_stable_order_desc(const uint32_t* keys, int64_t n, int32_t* rank,
                                    int32_t* order, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const unsigned nb256 = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(fill_f32_kernel, dim3(nb256 < 2048 ? nb256 : 2048), dim3(256), 0, s,
                     reinterpret_cast<float*>(rank), n, 0.0f);  // all-zero bits: int 0
  GPTQ_HIP_TRY(hipGetLastError());
  hipLaunchKernelGGL(rank_count_kernel, dim3(nb256, (unsigned)((n + RANK_CHUNK - 1) / RANK_CHUNK)),
                     dim3(256), 0, s, keys, n, 1, rank);
  GPTQ_HIP_TRY(hipGetLastError());
  hipLaunchKernelGGL(rank_scatter_kernel, dim3(nb256), dim3(256), 0, s, rank, n, 1, order);
  return hipGetLastError();
}

hipError_t run_prepare(const float* H, int64_t n, float damp, int desc_act, float* U,
                       int32_t* perm, int32_t* info, void* ws, hipStream_t s) {
  PrepLayout l = carve(ws, n);
  hipLaunchKernelGGL(diag_stats_kernel, dim3(1), dim3(1024), 0, s, H, n, damp, l.keys, l.rank,
                     l.damp_add, info);
  GPTQ_HIP_TRY(hipGetLastError());
  const unsigned nb256 = (unsigned)((n + 255) / 256);
  if (desc_act) {
    hipLaunchKernelGGL(rank_count_kernel, dim3(nb256, (unsigned)((n + RANK_CHUNK - 1) / RANK_CHUNK)),
                       dim3(256), 0, s, l.keys, n, desc_act, l.rank);
    GPTQ_HIP_TRY(hipGetLastError());
  }
  hipLaunchKernelGGL(rank_scatter_kernel, dim3(nb256), dim3(256), 0, s, l.rank, n, desc_act, perm);
  GPTQ_HIP_TRY(hipGetLastError());
  // S (symmetric H) is staged in the output buffer, gathered into A, then the
  // output buffer is cleared and receives L^-1.
  const unsigned nbs = (unsigned)((n + SYM_T - 1) / SYM_T);
  hipLaunchKernelGGL(symmetrize_kernel, dim3(nbs, nbs), dim3(256), 0, s, H, n, U);
  GPTQ_HIP_TRY(hipGetLastError());
  const size_t lds = (size_t)n * sizeof(float);
  GPTQ_HIP_TRY(hipFuncSetAttribute((const void*)gather_kernel,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
  hipLaunchKernelGGL(scale_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, H, n, perm,
                     l.damp_add, l.dsc);
  GPTQ_HIP_TRY(hipGetLastError());
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)n), dim3(lds > 64 * 1024 ? 1024 : lds > 32 * 1024 ? 512 : 256), lds, s, U,
                     n, perm, l.damp_add, l.dsc, l.A);
  GPTQ_HIP_TRY(hipGetLastError());
  hipLaunchKernelGGL(fill_f32_kernel, dim3(2048), dim3(256), 0, s, U, n * n, 0.0f);
  GPTQ_HIP_TRY(hipGetLastError());
  PrepCtx c{l.A, U, l.T, l.T2, n, info, s};
  GPTQ_HIP_TRY(cholinv_blocked(c, l.TB));
  hipLaunchKernelGGL(reverse_inplace_kernel, dim3((unsigned)((n + 1) / 2)), dim3(256), 0, s, U, n,
                     l.dsc);
  return hipGetLastError();
}

}  // namespace gptq
