// gptq_quantize_layer: the column sweep with error compensation, lazy block
// updates on the matrix cores, and dense b-bit packing.
//
// Glossary entry "gptq", "Algorithm" step (2): for each weight in order,
// quantize it, compute its error, adjust the remaining weights of the row to
// compensate.  With U' = diag(U)^-1 U (U the upper Cholesky factor of the
// inverse damped Hessian in quantization order) the adjustment after column j
// is  w_k -= e_j * U'_jk  for k > j.  Rows never interact.
//
// Blocking: columns are swept in blocks of B (32/64/128).  Inside a block a
// workgroup owns a slab of 32 rows; each row is spread over the 4 lanes of a
// quad, lane q holding block columns 4r + q in registers (r < B/4), and U' of
// the block sits in LDS, lane-interleaved so each lane reads its own
// coefficients as float4.  Per column: the owning lane's value is broadcast
// with a quad DPP move, all 4 lanes decide the code identically, and each lane
// updates its remaining registers.  Group scale/zero ("gptq" agent skill page,
// "Group-wise quantization") are taken at the group's first column from the
// group's current values with two quad DPP reductions.
//
// Across blocks, the updates from a finished range of columns to the columns
// right of it are applied as one GEMM (W[:, right] -= E[:, left] U'[left,
// right], fp32 accumulation) on a recursive halving schedule: the left half is
// swept, one GEMM carries all its updates to the right half, then the right
// half is swept.  Each pair (j < k) is updated exactly once, before column k
// is read.
#include "common.hpp"

namespace gptq {
namespace {

constexpr int SW_THREADS = 128;            // 2 waves
constexpr int SW_ROWS = SW_THREADS / 4;    // rows per workgroup

__device__ inline float dpp_bcast(float v, int lane_in_quad) {
  // quad_perm [o, o, o, o]
  int r;
  switch (lane_in_quad) {
    case 0: r = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x00, 0xF, 0xF, false); break;
    case 1: r = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0x55, 0xF, 0xF, false); break;
    case 2: r = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0xAA, 0xF, 0xF, false); break;
    default: r = __builtin_amdgcn_mov_dpp(__float_as_int(v), 0xFF, 0xF, 0xF, false); break;
  }
  return __int_as_float(r);
}
__device__ inline float dpp_xor1(float v) {  // quad_perm [1, 0, 3, 2]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ inline float dpp_xor2(float v) {  // quad_perm [2, 3, 0, 1]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// Scale / zero of a group from its (row-wide) lo / hi, with 0 already included.
__device__ inline void grid_params(float lo, float hi, int bits, int sym, float& s, float& z) {
  const float maxq = (float)((1 << bits) - 1);
  if (sym) {
    hi = fmaxf(-lo, hi);
    lo = -hi;
  }
  // A degenerate range (an all-zero group-row) becomes [-1, 1]; its zero
  // rint(1 / s) = rint(maxq / 2) is an exact tie that rounds to the even
  // 2^(b-1).  It is set directly: in fp32, 1 / fl(2 / maxq) falls just below
  // the tie for 3, 4 and 8 bits and would round down.
  const bool flat = lo == hi;
  if (flat) {
    lo = -1.0f;
    hi = 1.0f;
  }
  s = (hi - lo) / maxq;
  z = (sym || flat) ? (float)(1 << (bits - 1)) : rintf(-lo / s);
}

// Row scale of a block's errors for the trailing GEMMs: 2^(14 - e) for the
// row's largest |error| m = f 2^e (f in [0.5, 1)), so every scaled error is
// below 2^14 (the exponent capped at 126); 1 for an all-zero or non-finite
// row.
__device__ inline float error_row_scale(float m) {
  if (!(m > 0.0f && m < INFINITY)) return 1.0f;
  int e = 0;
  (void)frexpf(m, &e);
  return ldexpf(1.0f, min(14 - e, 126));
}

// Eight consecutive errors of a row (src, 16-byte aligned), scaled by rsc and
// split for the trailing GEMMs: x = hi + lo with hi = x rounded toward zero
// to fp16 and lo = x - hi (exact in fp32) rounded toward zero to fp16, so
// |x - hi - lo| <= 2^-21 |x| in the fp16 normal range.  grp is the row's
// 16-column group (64 bytes: 16 high parts, then 16 remainders); hh picks the
// group's first or second eight columns.
__device__ inline void store_split8(const float* src, float rsc, float* grp, int hh) {
  const float4 a = *reinterpret_cast<const float4*>(src);
  const float4 b = *reinterpret_cast<const float4*>(src + 4);
  const float x[8] = {a.x * rsc, a.y * rsc, a.z * rsc, a.w * rsc,
                      b.x * rsc, b.y * rsc, b.z * rsc, b.w * rsc};
  half8_t hi, lo;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const auto hp = __builtin_amdgcn_cvt_pkrtz(x[e], x[e + 1]);
    const auto lp = __builtin_amdgcn_cvt_pkrtz(x[e] - (float)hp[0], x[e + 1] - (float)hp[1]);
    hi[e] = hp[0];
    hi[e + 1] = hp[1];
    lo[e] = lp[0];
    lo[e + 1] = lp[1];
  }
  *reinterpret_cast<half8_t*>(grp + 4 * hh) = hi;
  *reinterpret_cast<half8_t*>(grp + 8 + 4 * hh) = lo;
}

template <typename T>
__device__ inline float to_f32(T v);
template <>
__device__ inline float to_f32<float>(float v) { return v; }
template <>
__device__ inline float to_f32<_Float16>(_Float16 v) { return (float)v; }
template <>
__device__ inline float to_f32<uint16_t>(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Wp[r][j] = W[r][perm[j]] as fp32 (perm == nullptr: identity).  256
// threads; 512 where the staged row leaves room for at most four workgroups
// per compute unit (in above 8192), 1024 where it leaves room for at most two
// (in above 16384), so that enough loads are in flight.
template <typename T>
__global__ void __launch_bounds__(1024)
gather_w_kernel(const T* __restrict__ W, int64_t out, int64_t in, const int32_t* __restrict__ perm,
                float* __restrict__ Wp) {
  extern __shared__ __align__(16) float rowbuf[];
  const int64_t r = blockIdx.x;
  const T* src = W + r * in;
  float* dst = Wp + r * in;
  const bool vec = (reinterpret_cast<uintptr_t>(W) & 15) == 0;  // rows then are too (in % 32 == 0)
  if (!vec) {
    for (int64_t j = threadIdx.x; j < in; j += blockDim.x) rowbuf[j] = to_f32<T>(src[j]);
  } else {
    // Stage the row as fp32, 4 x 16-byte loads per thread in flight.
    constexpr int PER = 16 / sizeof(T);  // elements per 16-byte load
    const uint4* s16 = reinterpret_cast<const uint4*>(src);
    const int64_t nv = in / PER;
    for (int64_t t0 = threadIdx.x; t0 < nv; t0 += 4 * (int64_t)blockDim.x) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t t = t0 + u * (int64_t)blockDim.x;
        v[u] = t < nv ? s16[t] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t t = t0 + u * (int64_t)blockDim.x;
        if (t < nv) {
          const T* e = reinterpret_cast<const T*>(&v[u]);
#pragma unroll
          for (int q = 0; q < PER; ++q) rowbuf[t * PER + q] = to_f32<T>(e[q]);
        }
      }
    }
  }
  __syncthreads();
  if (perm == nullptr) {
    for (int64_t j = threadIdx.x; j < in; j += blockDim.x) dst[j] = rowbuf[j];
    return;
  }
  // 8 elements per thread in flight (the loop is latency-bound otherwise).
  for (int64_t j0 = threadIdx.x; j0 < in; j0 += 8 * (int64_t)blockDim.x) {
    int32_t p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t j = j0 + u * (int64_t)blockDim.x;
      p[u] = j < in ? perm[j] : 0;
      if ((uint32_t)p[u] >= (uint32_t)in) p[u] = 0;  // never read outside the row
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t j = j0 + u * (int64_t)blockDim.x;
      if (j < in) dst[j] = rowbuf[p[u]];
    }
  }
}

// The forms of U' = diag(U)^-1 U the later kernels read, from U (upper, n x n
// fp32) in one pass:
//   Ub[b][j][k] = U'[bB + j][bB + k] for the sweep's diagonal B x B blocks
//               (k > j; 0 for k <= j);
//   Vt[c][r] = fp16(U'[r][c]) (round to nearest) and Vl[c][r] = the
//   remainder U'[r][c] - Vt[c][r] (exact in fp32) rounded toward zero to
//   fp16, for r < c: U' transposed for the trailing GEMMs, which read it
//   k-contiguous (null when the layer has no trailing GEMM).
// 64 x 64 tiles of U through LDS; tiles below the diagonal exit (the parts
// of a diagonal block they cover are never read: a sweep row's window
// starts at most 15 columns left of its diagonal, inside the same tile).
// Whole tiles with 16-byte aligned rows move 4 columns per access (16-byte
// loads of U and stores of Ub, 8-byte stores of Vt and Vl); ragged or
// unaligned tiles element by element.  Both give the same values.
__global__ void __launch_bounds__(256)
uprime_split_kernel(const float* __restrict__ U, int64_t n, int B, float* __restrict__ Ub,
                    _Float16* __restrict__ Vt, _Float16* __restrict__ Vl) {
  __shared__ float tile[64][65];
  __shared__ float dg[64];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  if (r0 > c0 + 63) return;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  if (threadIdx.x < 64) {
    const int64_t r = r0 + threadIdx.x;
    dg[threadIdx.x] = r < n ? U[r * n + r] : 1.0f;
  }
  __syncthreads();
  const bool vec = (n & 3) == 0 && c0 + 64 <= n &&
                   ((reinterpret_cast<uintptr_t>(U) | reinterpret_cast<uintptr_t>(Ub)) & 15) == 0 &&
                   ((reinterpret_cast<uintptr_t>(Vt) | reinterpret_cast<uintptr_t>(Vl)) & 7) == 0;
  const int q4 = 4 * (threadIdx.x & 15), g = threadIdx.x >> 4;  // 16 x 16 threads
  if (vec) {
    // rows g, g + 16, ...; columns q4 .. q4 + 3 (r0 + 64 <= c0 + 64 <= n)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = g + 16 * u;
      const int64_t r = r0 + i, c = c0 + q4;
      const float4 x = *reinterpret_cast<const float4*>(U + r * n + c);
      const float d = dg[i];
      float4 v;
      v.x = r < c ? x.x / d : 0.0f;
      v.y = r < c + 1 ? x.y / d : 0.0f;
      v.z = r < c + 2 ? x.z / d : 0.0f;
      v.w = r < c + 3 ? x.w / d : 0.0f;
      tile[i][q4] = v.x;
      tile[i][q4 + 1] = v.y;
      tile[i][q4 + 2] = v.z;
      tile[i][q4 + 3] = v.w;
      if (r / B == c / B)  // B is a multiple of 4: the chunk lies in one block
        *reinterpret_cast<float4*>(Ub + (r / B) * B * B + (r % B) * B + (c % B)) = v;
    }
  } else {
    for (int i = ty; i < 64; i += 4) {
      const int64_t r = r0 + i, c = c0 + tx;
      if (r >= n || c >= n) continue;
      const float v = r < c ? U[r * n + c] / dg[i] : 0.0f;
      tile[i][tx] = v;
      if (r / B == c / B) Ub[(r / B) * B * B + (r % B) * B + (c % B)] = v;
    }
  }
  __syncthreads();
  if (Vt == nullptr) return;
  if (vec) {
    // Vt[c][r .. r + 3] for c = c0 + g + 16u, r = r0 + q4
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = g + 16 * u;
      const int64_t c = c0 + i, r = r0 + q4;
      if (r + 3 < c) {
        _Float16 hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = tile[q4 + e][i];
          hi[e] = (_Float16)x;
          lo[e] = __builtin_amdgcn_cvt_pkrtz(x - (float)hi[e], 0.0f)[0];
        }
        *reinterpret_cast<uint2*>(Vt + c * n + r) = *reinterpret_cast<const uint2*>(hi);
        *reinterpret_cast<uint2*>(Vl + c * n + r) = *reinterpret_cast<const uint2*>(lo);
      } else {
        for (int e = 0; e < 4 && r + e < c; ++e) {
          const float x = tile[q4 + e][i];
          const _Float16 hi = (_Float16)x;
          Vt[c * n + r + e] = hi;
          Vl[c * n + r + e] = __builtin_amdgcn_cvt_pkrtz(x - (float)hi, 0.0f)[0];
        }
      }
    }
  } else {
    for (int i = ty; i < 64; i += 4) {
      const int64_t c = c0 + i, r = r0 + tx;
      if (c < n && r < n && r < c) {
        const float u = tile[tx][i];
        const _Float16 hi = (_Float16)u;
        Vt[c * n + r] = hi;
        Vl[c * n + r] = __builtin_amdgcn_cvt_pkrtz(u - (float)hi, 0.0f)[0];
      }
    }
  }
}

// pinv[perm[j]] = j;  g_idx[perm[j]] = j / gs (0 for one group per row).
__global__ void perm_tables_kernel(const int32_t* __restrict__ perm, int64_t in, int gs,
                                   int32_t* __restrict__ pinv, int32_t* __restrict__ g_idx) {
  const int64_t j = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (j >= in) return;
  int32_t p = perm ? perm[j] : (int32_t)j;
  if ((uint32_t)p >= (uint32_t)in) p = 0;
  pinv[p] = (int32_t)j;
  g_idx[p] = gs > 0 ? (int32_t)(j / gs) : 0;
}

// One group per row: scale/zero from the whole original row.
__global__ void __launch_bounds__(256)
row_params_kernel(const float* __restrict__ Wp, int64_t out, int64_t in, int bits, int sym,
                  float* __restrict__ scales, int32_t* __restrict__ zeros) {
  __shared__ float slo[256], shi[256];
  const int64_t r = blockIdx.x;
  float lo = 0.0f, hi = 0.0f;
  for (int64_t j = threadIdx.x; j < in; j += blockDim.x) {
    const float v = Wp[r * in + j];
    lo = fminf(lo, v);
    hi = fmaxf(hi, v);
  }
  slo[threadIdx.x] = lo;
  shi[threadIdx.x] = hi;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      slo[threadIdx.x] = fminf(slo[threadIdx.x], slo[threadIdx.x + w]);
      shi[threadIdx.x] = fmaxf(shi[threadIdx.x], shi[threadIdx.x + w]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    float s, z;
    grid_params(slo[0], shi[0], bits, sym, s, z);
    scales[r] = s;
    zeros[r] = (int32_t)z;
  }
}

// Sweep of block columns [c0, c0 + width) for a slab of 32 rows.
// GS: group size (divides B, multiple of 4) or 0 = one group per row
// (scales[0][r] / zeros[0][r] precomputed).
//
// Lane q of a row's quad holds block columns 4r + q.  The registers form a
// sliding window: at quad-step R (block columns 4R .. 4R+3), w[t] holds column
// 4(R + t) + q, so the columns being quantized are always in w[0] and every
// register index is a compile-time constant while the loop over R stays
// rolled.  U' rows are stored pre-shifted to the same window:
//     Ul[j][q][t] = U'[c0 + j][c0 + 4(j/4 + t) + q]   (0 outside the block),
// which is 0 wherever that column is not right of j (U' is strictly upper).
template <int B>
struct SweepSmem {
  static constexpr int NR = B / 4, PITCH = NR + 4, EP = B + 4;
  static constexpr size_t UL = (size_t)B * 4 * PITCH;          // floats
  static constexpr size_t ES = (size_t)SW_ROWS * EP;            // floats
  static constexpr size_t BYTES = (UL + ES) * sizeof(float) + (size_t)SW_ROWS * B;
};

template <int B, int GS>
__global__ void __launch_bounds__(SW_THREADS)
sweep_kernel(float* __restrict__ Wp, const float* __restrict__ Ub, int64_t out, int64_t in,
             int64_t c0, int width, int bits, int sym, float* __restrict__ scales,
             int32_t* __restrict__ zeros, uint8_t* __restrict__ codes,
             float* __restrict__ einv) {
  using SM = SweepSmem<B>;
  constexpr int NR = SM::NR, PITCH = SM::PITCH, EP = SM::EP;
  extern __shared__ __align__(16) float smem[];
  float* Ul = smem;
  float* Es = smem + SM::UL;
  uint8_t* Cs = reinterpret_cast<uint8_t*>(Es + SM::ES);

  const int tid = threadIdx.x;
  const int q = tid & 3, rl = tid >> 2;
  const int64_t row0 = (int64_t)blockIdx.x * SW_ROWS;
  const int64_t row = row0 + rl;
  const bool live = row < out;

  // Pre-shifted U' window: item (j, t) is the float4 of columns 4(j/4 + t) .. +3.
  {
    constexpr int ITEMS = B * NR / SW_THREADS;
    float4 v[ITEMS];
#pragma unroll
    for (int p = 0; p < ITEMS; ++p) {
      const int e = tid + p * SW_THREADS;
      const int j = e / NR, t = e % NR;
      const int c = 4 * (j / 4 + t);
      v[p] = (j < width && c < width)
                 ? *reinterpret_cast<const float4*>(Ub + j * B + c)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int p = 0; p < ITEMS; ++p) {
      const int e = tid + p * SW_THREADS;
      const int j = e / NR, t = e % NR;
      float* d = Ul + j * 4 * PITCH + t;
      d[0 * PITCH] = v[p].x;
      d[1 * PITCH] = v[p].y;
      d[2 * PITCH] = v[p].z;
      d[3 * PITCH] = v[p].w;
    }
  }

  float w[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int col = 4 * r + q;
    w[r] = (live && col < width) ? Wp[row * in + c0 + col] : 0.0f;
  }

  const float maxq = (float)((1 << bits) - 1);
  float s = 1.0f, z = 0.0f;
  if constexpr (GS == 0) {
    if (live) {
      s = scales[row];
      z = (float)zeros[row];
    }
  }
  __syncthreads();

  const int nquads = width / 4;
  for (int R = 0; R < nquads; ++R) {
    if constexpr (GS > 0) {
      if ((4 * R) % GS == 0) {
        // range of the group's current values, 0 included
        float lo = 0.0f, hi = 0.0f;
#pragma unroll
        for (int t = 0; t < GS / 4; ++t) {
          lo = fminf(lo, w[t]);
          hi = fmaxf(hi, w[t]);
        }
        lo = fminf(lo, dpp_xor1(lo));
        hi = fmaxf(hi, dpp_xor1(hi));
        lo = fminf(lo, dpp_xor2(lo));
        hi = fmaxf(hi, dpp_xor2(hi));
        grid_params(lo, hi, bits, sym, s, z);
        if (live && q == 0) {
          const int64_t g = (c0 + 4 * R) / GS;
          scales[g * out + row] = s;
          zeros[g * out + row] = (int32_t)z;
        }
      }
    }
#pragma unroll
    for (int o = 0; o < 4; ++o) {
      const int j = 4 * R + o;
      const float wj = dpp_bcast(w[0], o);
      const float qf = fminf(fmaxf(rintf(wj / s) + z, 0.0f), maxq);
      const float err = wj - s * (qf - z);
      if (q == o) {
        Es[rl * EP + j] = err;
        Cs[rl * B + j] = (uint8_t)qf;
      }
      const float* urow = Ul + j * 4 * PITCH + q * PITCH;
#pragma unroll
      for (int t = 0; t < NR; t += 4) {
        const float4 u = *reinterpret_cast<const float4*>(urow + t);
        w[t + 0] = fmaf(-err, u.x, w[t + 0]);
        if (t + 1 < NR) w[t + 1] = fmaf(-err, u.y, w[t + 1]);
        if (t + 2 < NR) w[t + 2] = fmaf(-err, u.z, w[t + 2]);
        if (t + 3 < NR) w[t + 3] = fmaf(-err, u.w, w[t + 3]);
      }
    }
#pragma unroll
    for (int t = 0; t + 1 < NR; ++t) w[t] = w[t + 1];
    w[NR - 1] = 0.0f;
  }
  __syncthreads();

  // The block's errors for the trailing GEMMs, in place of its columns of
  // Wp: each row scaled by error_row_scale of its largest |error| (einv
  // keeps the inverse) and split by store_split8; lane q of a row's quad
  // writes the eight-column pieces q, q + 4, ...
  {
    float m = 0.0f;
    for (int c = q; c < width; c += 4) m = fmaxf(m, fabsf(Es[rl * EP + c]));
    m = fmaxf(m, dpp_xor1(m));
    m = fmaxf(m, dpp_xor2(m));
    const float rsc = error_row_scale(m);
    if (live) {
      if (q == 0) einv[(c0 / B) * out + row] = 1.0f / rsc;
      for (int p = q; 8 * p < width; p += 4)
        store_split8(Es + rl * EP + 8 * p, rsc, Wp + row * in + c0 + 16 * (p >> 1), p & 1);
    }
  }
  const int w16 = width / 16;
  for (int e = tid; e < SW_ROWS * w16; e += SW_THREADS) {
    const int r = e / w16, c = (e % w16) * 16;
    if (row0 + r < out)
      *reinterpret_cast<uint4*>(codes + (row0 + r) * in + c0 + c) =
          *reinterpret_cast<const uint4*>(Cs + r * B + c);
  }
}

// qweight[u*bits + t][r]: word t of the 32-code unit u of row r (original
// column order).  A workgroup stages R rows of codes (quantization order) in
// LDS, rows PACK_PAD bytes longer than the codes so that the R rows of a
// column fall in different LDS banks, then packs (unit, row) pairs with the R
// rows of a unit on neighbouring threads: each thread takes its unit's 32
// pinv entries from memory (the R threads of a unit read the same 128 bytes),
// the permuted code reads hit LDS, and the word stores of a unit cover R
// consecutive rows.
constexpr int PACK_PAD = 16;
__global__ void __launch_bounds__(256)
pack_kernel(const uint8_t* __restrict__ codes, const int32_t* __restrict__ pinv, int64_t out,
            int64_t in, int bits, int R, int32_t* __restrict__ qweight) {
  extern __shared__ __align__(16) uint8_t cl[];
  const int64_t cp = in + PACK_PAD;  // LDS row pitch (16-byte aligned: in is a multiple of 32)
  const int64_t r0 = (int64_t)blockIdx.x * R;
  const int rows = (int)(out - r0 < R ? out - r0 : R);
  const int64_t v16 = in / 16;
  for (int64_t e0 = threadIdx.x; e0 < rows * v16; e0 += 4 * (int64_t)blockDim.x) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t e = e0 + u * (int64_t)blockDim.x;
      v[u] = e < rows * v16 ? *reinterpret_cast<const uint4*>(codes + r0 * in + e * 16)
                            : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t e = e0 + u * (int64_t)blockDim.x;
      if (e < rows * v16)
        *reinterpret_cast<uint4*>(cl + (e / v16) * cp + (e % v16) * 16) = v[u];
    }
  }
  __syncthreads();
  const int64_t units = in / 32;
  for (int64_t t = threadIdx.x; t < units * R; t += blockDim.x) {
    const int64_t u = t / R;
    const int rr = (int)(t % R);
    if (rr >= rows) continue;
    int32_t pu[32];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int4 v = *reinterpret_cast<const int4*>(pinv + u * 32 + 4 * q);
      pu[4 * q + 0] = v.x; pu[4 * q + 1] = v.y; pu[4 * q + 2] = v.z; pu[4 * q + 3] = v.w;
    }
    const uint8_t* crow = cl + (int64_t)rr * cp;
    uint64_t acc = 0;
    int nb = 0, w = 0;
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      const int32_t p = (uint32_t)pu[c] < (uint32_t)in ? pu[c] : 0;  // never read outside the row
      acc |= (uint64_t)crow[p] << nb;
      nb += bits;
      if (nb >= 32) {
        qweight[(u * bits + w) * out + r0 + rr] = (int32_t)(uint32_t)acc;
        acc >>= 32;
        nb -= 32;
        ++w;
      }
    }
  }
}

// Sweep with 16 lanes per row (group sizes that are multiples of 16, or one
// group per row): lane q of a row's 16-lane DPP row holds block columns
// 16r + q (r < B/16) as a sliding window (w[t] = column 16(R + t) + q at step
// R), the owning lane's value is broadcast with DPP row_newbcast (one VALU
// op), group min/max reduce over the 16 lanes with DPP, and the U' window is
// stored pre-shifted per lane:
//     Ul[j][q][t] = U'[c0 + j][c0 + 16(j/16 + t) + q]   (0 unless right of j).
// Four times the lanes of the quad layout per row: 4x fewer updates per lane
// and per column, and 4x the rows in flight.
constexpr int S16_THREADS = 256;
constexpr int S16_ROWS = S16_THREADS / 16;

template <int B>
struct Sweep16Smem {
  static constexpr int NR = B / 16, PITCH = (NR + 4 + 3) / 4 * 4, EP = B + 4;
  static constexpr size_t UL = (size_t)B * 16 * PITCH;  // floats
  static constexpr size_t ES = (size_t)S16_ROWS * EP;    // floats
  static constexpr size_t BYTES = (UL + ES) * sizeof(float) + (size_t)S16_ROWS * B;
};

// Value of lane o of each 16-lane row, to every lane of the row (o constant
// after unrolling).
__device__ inline float row_bcast16(float v, int o) {
  const int x = __float_as_int(v);
  int r;
  switch (o) {
    case 0: r = __builtin_amdgcn_mov_dpp(x, 0x150, 0xF, 0xF, true); break;
    case 1: r = __builtin_amdgcn_mov_dpp(x, 0x151, 0xF, 0xF, true); break;
    case 2: r = __builtin_amdgcn_mov_dpp(x, 0x152, 0xF, 0xF, true); break;
    case 3: r = __builtin_amdgcn_mov_dpp(x, 0x153, 0xF, 0xF, true); break;
    case 4: r = __builtin_amdgcn_mov_dpp(x, 0x154, 0xF, 0xF, true); break;
    case 5: r = __builtin_amdgcn_mov_dpp(x, 0x155, 0xF, 0xF, true); break;
    case 6: r = __builtin_amdgcn_mov_dpp(x, 0x156, 0xF, 0xF, true); break;
    case 7: r = __builtin_amdgcn_mov_dpp(x, 0x157, 0xF, 0xF, true); break;
    case 8: r = __builtin_amdgcn_mov_dpp(x, 0x158, 0xF, 0xF, true); break;
    case 9: r = __builtin_amdgcn_mov_dpp(x, 0x159, 0xF, 0xF, true); break;
    case 10: r = __builtin_amdgcn_mov_dpp(x, 0x15A, 0xF, 0xF, true); break;
    case 11: r = __builtin_amdgcn_mov_dpp(x, 0x15B, 0xF, 0xF, true); break;
    case 12: r = __builtin_amdgcn_mov_dpp(x, 0x15C, 0xF, 0xF, true); break;
    case 13: r = __builtin_amdgcn_mov_dpp(x, 0x15D, 0xF, 0xF, true); break;
    case 14: r = __builtin_amdgcn_mov_dpp(x, 0x15E, 0xF, 0xF, true); break;
    default: r = __builtin_amdgcn_mov_dpp(x, 0x15F, 0xF, 0xF, true); break;
  }
  return __int_as_float(r);
}
// Min / max over a 16-lane row (quad swaps, then rotations by 4 and 8).
__device__ inline float row_min16(float v) {
  v = fminf(v, dpp_xor1(v));
  v = fminf(v, dpp_xor2(v));
  v = fminf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false)));
  v = fminf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false)));
  return v;
}
__device__ inline float row_max16(float v) {
  v = fmaxf(v, dpp_xor1(v));
  v = fmaxf(v, dpp_xor2(v));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false)));
  return v;
}

// One block of the sweep for the workgroup's 16 rows (smem16: the
// workgroup's Sweep16Smem<B>).  delta (LDS, [16 rows][B], or null): an
// update of the block's columns still to be subtracted from the values
// loaded from Wp.
template <int B, int GS>
__device__ __attribute__((always_inline)) inline void sweep16_body(
    float* smem16, float* __restrict__ Wp, const float* __restrict__ Ub, int64_t out, int64_t in,
    int64_t c0, int width, int bits, int sym, float* __restrict__ scales,
    int32_t* __restrict__ zeros, uint8_t* __restrict__ codes, float* __restrict__ einv,
    const float* delta) {
  using SM = Sweep16Smem<B>;
  constexpr int NR = SM::NR, PITCH = SM::PITCH, EP = SM::EP;
  static_assert(GS % 16 == 0, "group size a multiple of 16 (0: one group per row)");
  float* Ul = smem16;
  float* Es = smem16 + SM::UL;
  uint8_t* Cs = reinterpret_cast<uint8_t*>(Es + SM::ES);

  const int tid = threadIdx.x;
  const int q = tid & 15, rl = tid >> 4;
  const int64_t row0 = (int64_t)blockIdx.x * S16_ROWS;
  const int64_t row = row0 + rl;
  const bool live = row < out;

  // This lane's columns of its row (issued first: their HBM latency overlaps
  // the U' loads below).
  float w[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int col = 16 * r + q;
    w[r] = (live && col < width) ? Wp[row * in + c0 + col] : 0.0f;
  }

  // Pre-shifted U' window.  Item (j, t, h): the float4 of block columns
  // 16(j/16 + t) + 4h .. +3 of U' row c0 + j, spread to lanes 4h .. 4h+3;
  // columns not right of j are stored as 0.  All of a thread's loads are in
  // flight together (one round trip, not one per batch).
  {
    constexpr int ITEMS = B * NR * 4;
    constexpr int PER = ITEMS / S16_THREADS;
    static_assert(ITEMS % S16_THREADS == 0, "whole items per thread");
    float4 v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + u * S16_THREADS;
      const int j = e / (NR * 4), t = (e / 4) % NR, h = e % 4;
      const int c = 16 * (j / 16 + t) + 4 * h;
      v[u] = (j < width && c < width)
                 ? *reinterpret_cast<const float4*>(Ub + j * B + c)
                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int e = tid + u * S16_THREADS;
      const int j = e / (NR * 4), t = (e / 4) % NR, h = e % 4;
      const int c = 16 * (j / 16 + t) + 4 * h;
      float* d = Ul + (j * 16 + 4 * h) * PITCH + t;
      d[0 * PITCH] = c + 0 > j ? v[u].x : 0.0f;
      d[1 * PITCH] = c + 1 > j ? v[u].y : 0.0f;
      d[2 * PITCH] = c + 2 > j ? v[u].z : 0.0f;
      d[3 * PITCH] = c + 3 > j ? v[u].w : 0.0f;
    }
  }

  const float maxq = (float)((1 << bits) - 1);
  float s = 1.0f, z = 0.0f;
  if constexpr (GS == 0) {
    if (live) {
      s = scales[row];
      z = (float)zeros[row];
    }
  }
  float rs = 1.0f / s;
  __syncthreads();
  if (delta != nullptr) {
#pragma unroll
    for (int r = 0; r < NR; ++r) w[r] -= delta[rl * B + 16 * r + q];
  }

  // U' rows of the step's 16 columns, each replaced by the same column of
  // the next step once used, so the LDS latency (16 columns ahead) stays off
  // the column-to-column dependency chain.  (Widths are multiples of 16.)
  constexpr int NU = (NR + 3) / 4, COL = 16 * PITCH;  // floats per column
  const float* ulane = Ul + q * PITCH;
  auto load_u = [&](const float* urow, float4* dst) {
#pragma unroll
    for (int t = 0; t < NU; ++t) dst[t] = *reinterpret_cast<const float4*>(urow + 4 * t);
  };
  float4 ur[16][NU];
  if (width >= 16) {
#pragma unroll
    for (int o = 0; o < 16; ++o) load_u(ulane + o * COL, ur[o]);
  }

  const int nsteps = width / 16;
  for (int R = 0; R < nsteps; ++R) {
    if constexpr (GS > 0) {
      if ((16 * R) % GS == 0) {
        // range of the group's current values, 0 included
        float lo = 0.0f, hi = 0.0f;
#pragma unroll
        for (int t = 0; t < GS / 16; ++t) {
          lo = fminf(lo, w[t]);
          hi = fmaxf(hi, w[t]);
        }
        lo = row_min16(lo);
        hi = row_max16(hi);
        grid_params(lo, hi, bits, sym, s, z);
        rs = 1.0f / s;
        if (live && q == 0) {
          const int64_t g = (c0 + 16 * R) / GS;
          scales[g * out + row] = s;
          zeros[g * out + row] = (int32_t)z;
        }
      }
    }
    float my_err = 0.0f, my_code = 0.0f;  // this lane's column of the step
    // rint(wj / s) with the quotient correctly rounded, without the division
    // on the column-to-column dependency chain: y = wj * (1/s) is within
    // |y| 2^-22 of the rounded quotient, so rint(y) is the same integer
    // unless y lies that close to a half-integer (|y - rint(y)| +
    // |y| 2^-20 >= 1/2 flags it, with margin for the rounding of that test),
    // or 1/s is zero or not finite.  A flag only raises the step's maximum;
    // after the 16 columns a wave with a flag sweeps them again from the
    // saved state with true divisions (a branch per column on the chain cost
    // about a third of the sweep).  Non-finite w gives the same code either
    // way.
    float w_in[NR];
#pragma unroll
    for (int t = 0; t < NR; ++t) w_in[t] = w[t];
    float flag = fabsf(rs) < INFINITY && rs != 0.0f ? 0.0f : 1.0f;
    // next step's rows (past the last step: rows in range, not used)
    const float* unext = ulane + (R + 1 < nsteps ? 16 * (R + 1) * COL : 0);
    auto columns = [&](const bool exact) {
#pragma unroll
      for (int o = 0; o < 16; ++o) {
        float4 ub[NU];
        if (exact) {
          load_u(ulane + (16 * R + o) * COL, ub);  // the ring holds the next step
        } else {
#pragma unroll
          for (int t = 0; t < NU; ++t) ub[t] = ur[o][t];
          load_u(unext + o * COL, ur[o]);
        }
        const float wj = row_bcast16(w[0], o);
        float qz;
        if (exact) {
          qz = __builtin_amdgcn_fmed3f(rintf(wj / s), -z, maxq - z);
        } else {
          const float y = wj * rs;
          const float qr = rintf(y);
          // clamp(qr + z, 0, maxq) - z in one step (small integers: exact)
          qz = __builtin_amdgcn_fmed3f(qr, -z, maxq - z);
          flag = fmaxf(flag, fmaf(fabsf(y), 0x1p-20f, fabsf(y - qr)));
        }
        const float err = wj - s * qz;
        my_err = q == o ? err : my_err;
        my_code = q == o ? qz : my_code;
#pragma unroll
        for (int t = 0; t < NR; t += 4) {
          const float4 u = ub[t / 4];
          w[t + 0] = fmaf(-err, u.x, w[t + 0]);
          if (t + 1 < NR) w[t + 1] = fmaf(-err, u.y, w[t + 1]);
          if (t + 2 < NR) w[t + 2] = fmaf(-err, u.z, w[t + 2]);
          if (t + 3 < NR) w[t + 3] = fmaf(-err, u.w, w[t + 3]);
        }
      }
    };
    columns(false);
    if (__builtin_amdgcn_ballot_w64(flag >= 0.5f) != 0) {
#pragma unroll
      for (int t = 0; t < NR; ++t) w[t] = w_in[t];
      columns(true);
    }
    my_code += z;
    Es[rl * EP + 16 * R + q] = my_err;
    Cs[rl * B + 16 * R + q] = (uint8_t)my_code;
#pragma unroll
    for (int t = 0; t + 1 < NR; ++t) w[t] = w[t + 1];
    w[NR - 1] = 0.0f;
  }
  __syncthreads();

  // The block's errors for the trailing GEMMs, in place of its columns of
  // Wp: each row scaled by error_row_scale of its largest |error| (einv
  // keeps the inverse) and split by store_split8; lane q of a row writes
  // the eight-column piece q.
  {
    float m = 0.0f;
    for (int c = q; c < width; c += 16) m = fmaxf(m, fabsf(Es[rl * EP + c]));
    m = row_max16(m);
    const float rsc = error_row_scale(m);
    if (live) {
      if (q == 0) einv[(c0 / B) * out + row] = 1.0f / rsc;
      if (8 * q < width)
        store_split8(Es + rl * EP + 8 * q, rsc, Wp + row * in + c0 + 16 * (q >> 1), q & 1);
    }
  }
  const int w16 = width / 16;
  for (int e = tid; e < S16_ROWS * w16; e += S16_THREADS) {
    const int r = e / w16, c = (e % w16) * 16;
    if (row0 + r < out)
      *reinterpret_cast<uint4*>(codes + (row0 + r) * in + c0 + c) =
          *reinterpret_cast<const uint4*>(Cs + r * B + c);
  }
}

template <int B, int GS>
__global__ void __launch_bounds__(S16_THREADS)
sweep16_kernel(float* __restrict__ Wp, const float* __restrict__ Ub, int64_t out, int64_t in,
               int64_t c0, int width, int bits, int sym, float* __restrict__ scales,
               int32_t* __restrict__ zeros, uint8_t* __restrict__ codes,
               float* __restrict__ einv) {
  extern __shared__ __align__(16) float smem16[];
  sweep16_body<B, GS>(smem16, Wp, Ub, out, in, c0, width, bits, sym, scales, zeros, codes, einv,
                      nullptr);
}

// Two adjacent full 128-column blocks in one launch: the first block's sweep,
// its update of the second block for the workgroup's rows, the second
// block's sweep.  The update (the trailing product of the pair, otherwise a
// GEMM launch of its own between two sweep launches) runs on the matrix
// cores in fp32: the first block's fp32 errors (still in LDS) times U' of
// the pair, rebuilt in fp32 from its fp16 parts (Vt + Vl, U' transposed) and
// staged in the space of the sweep's U' window.
constexpr int PAIR_B = 128;
template <int GS>
__global__ void __launch_bounds__(S16_THREADS)
sweep16_pair_kernel(float* __restrict__ Wp, const float* __restrict__ Ub,
                    const _Float16* __restrict__ Vt, const _Float16* __restrict__ Vl, int64_t out,
                    int64_t in, int64_t c0, int bits, int sym, float* __restrict__ scales,
                    int32_t* __restrict__ zeros, uint8_t* __restrict__ codes,
                    float* __restrict__ einv) {
  constexpr int B = PAIR_B;
  using SM = Sweep16Smem<B>;
  constexpr int UP = B + 4;  // pitch of the staged U' block (rows 4 banks apart)
  static_assert(SM::UL >= (size_t)B * UP, "the pair's U' block fits the window's space");
  extern __shared__ __align__(16) float smem16[];
  float* delta = smem16 + (SM::BYTES / sizeof(float));  // [16 rows][B]
  sweep16_body<B, GS>(smem16, Wp, Ub, out, in, c0, B, bits, sym, scales, zeros, codes, einv,
                      nullptr);
  __syncthreads();  // the window and the first block's errors are final
  const int tid = threadIdx.x;
  float* Us = smem16;                 // Us[k * UP + j] = U'[c0 + k][c0 + B + j]
  const float* Es = smem16 + SM::UL;  // the first block's errors, [16 rows][EP]
  {
    const int j = tid >> 1, kh = (tid & 1) * (B / 2);
    const _Float16* vt = Vt + (c0 + B + j) * in + c0 + kh;
    const _Float16* vl = Vl + (c0 + B + j) * in + c0 + kh;
    half8_t hv[B / 16], lv[B / 16];
#pragma unroll
    for (int u = 0; u < B / 16; ++u) {
      hv[u] = *reinterpret_cast<const half8_t*>(vt + 8 * u);
      lv[u] = *reinterpret_cast<const half8_t*>(vl + 8 * u);
    }
#pragma unroll
    for (int u = 0; u < B / 16; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) Us[(kh + 8 * u + e) * UP + j] = (float)hv[u][e] + (float)lv[u][e];
  }
  __syncthreads();
  {
    // v_mfma_f32_16x16x4f32: lane l supplies E[l % 16][k + l / 16] and
    // U'[k + l / 16][j + l % 16] and holds rows 4 (l / 16) .. +3 of column
    // j + l % 16; wave v takes columns 32 v .. 32 v + 31.
    const int l = tid & 63, v = tid >> 6;
    f32x4_t d[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) d[t][i] = 0.0f;
#pragma unroll 4
    for (int k = 0; k < B; k += 4) {
      const float a = Es[(l & 15) * SM::EP + k + (l >> 4)];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        d[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(
            a, Us[(k + (l >> 4)) * UP + 32 * v + 16 * t + (l & 15)], d[t], 0, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) delta[(4 * (l >> 4) + i) * B + 32 * v + 16 * t + (l & 15)] = d[t][i];
  }
  __syncthreads();
  sweep16_body<B, GS>(smem16, Wp, Ub + B * B, out, in, c0 + B, B, bits, sym, scales, zeros, codes,
                      einv, delta);
}

template <int B, int GS>
hipError_t launch_sweep16(float* Wp, const float* Ub, int64_t out, int64_t in, int64_t c0,
                          int width, int bits, int sym, float* scales, int32_t* zeros,
                          uint8_t* codes, float* einv, hipStream_t s) {
  auto k = sweep16_kernel<B, GS>;
  const size_t lds = Sweep16Smem<B>::BYTES;
  GPTQ_HIP_TRY(hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)lds));
  hipLaunchKernelGGL(k, dim3((unsigned)((out + S16_ROWS - 1) / S16_ROWS)), dim3(S16_THREADS), lds,
                     s, Wp, Ub, out, in, c0, width, bits, sym, scales, zeros, codes, einv);
  return hipGetLastError();
}

template <int GS>
hipError_t launch_sweep16_pair(float* Wp, const float* Ub, const _Float16* Vt, const _Float16* Vl,
                               int64_t out, int64_t in, int64_t c0, int bits, int sym,
                               float* scales, int32_t* zeros, uint8_t* codes, float* einv,
                               hipStream_t s) {
  auto k = sweep16_pair_kernel<GS>;
  const size_t lds = Sweep16Smem<PAIR_B>::BYTES + (size_t)S16_ROWS * PAIR_B * sizeof(float);
  GPTQ_HIP_TRY(hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)lds));
  hipLaunchKernelGGL(k, dim3((unsigned)((out + S16_ROWS - 1) / S16_ROWS)), dim3(S16_THREADS), lds,
                     s, Wp, Ub, Vt, Vl, out, in, c0, bits, sym, scales, zeros, codes, einv);
  return hipGetLastError();
}

template <int B>
hipError_t launch_sweep(int gs, float* Wp, const float* Ub, int64_t out, int64_t in, int64_t c0,
                        int width, int bits, int sym, float* scales, int32_t* zeros,
                        uint8_t* codes, float* einv, hipStream_t s) {
  if (gs > B) return hipErrorInvalidValue;
  // 16 lanes per row where the group size allows it.
  switch (gs > 0 ? gs : 0) {
    case 0: return launch_sweep16<B, 0>(Wp, Ub, out, in, c0, width, bits, sym, scales, zeros,
                                        codes, einv, s);
    case 16: return launch_sweep16<B, 16>(Wp, Ub, out, in, c0, width, bits, sym, scales, zeros,
                                          codes, einv, s);
    case 32: return launch_sweep16<B, 32>(Wp, Ub, out, in, c0, width, bits, sym, scales, zeros,
                                          codes, einv, s);
    case 64:
      if constexpr (B >= 64)
        return launch_sweep16<B, (B >= 64 ? 64 : 16)>(Wp, Ub, out, in, c0, width, bits, sym,
                                                       scales, zeros, codes, einv, s);
      break;
    case 128:
      if constexpr (B >= 128)
        return launch_sweep16<B, (B >= 128 ? 128 : 16)>(Wp, Ub, out, in, c0, width, bits, sym,
                                                         scales, zeros, codes, einv, s);
      break;
    default:
      break;
  }
  dim3 grid((unsigned)((out + SW_ROWS - 1) / SW_ROWS)), block(SW_THREADS);
  const size_t lds = SweepSmem<B>::BYTES;
#define GPTQ_SWEEP_CASE(G)                                                                     \
  case G: {                                                                                    \
    auto k = sweep_kernel<B, (G > 0 ? G : 0)>;                                                 \
    GPTQ_HIP_TRY(hipFuncSetAttribute((const void*)k,                                           \
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));   \
    hipLaunchKernelGGL(k, grid, block, lds, s, Wp, Ub, out, in, c0, width, bits, sym, scales,  \
                       zeros, codes, einv);                                                    \
    break;                                                                                     \
  }
  switch (gs > 0 ? gs : 0) {
    GPTQ_SWEEP_CASE(0)
    GPTQ_SWEEP_CASE(4)
    GPTQ_SWEEP_CASE(8)
    GPTQ_SWEEP_CASE(16)
    GPTQ_SWEEP_CASE(32)
    case 64:
      if constexpr (B >= 64) {
        auto k = sweep_kernel<B, (B >= 64 ? 64 : 4)>;
        GPTQ_HIP_TRY(hipFuncSetAttribute((const void*)k,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
        hipLaunchKernelGGL(k, grid, block, lds, s, Wp, Ub, out, in, c0, width, bits, sym, scales,
                           zeros, codes, einv);
      }
      break;
    case 128:
      if constexpr (B >= 128) {
        auto k = sweep_kernel<B, (B >= 128 ? 128 : 4)>;
        GPTQ_HIP_TRY(hipFuncSetAttribute((const void*)k,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
        hipLaunchKernelGGL(k, grid, block, lds, s, Wp, Ub, out, in, c0, width, bits, sym, scales,
                           zeros, codes, einv);
      }
      break;
    default:
      return hipErrorInvalidValue;
  }
#undef GPTQ_SWEEP_CASE
  return hipGetLastError();
}

struct QCtx {
  float* Wp;
  const float* Ub;     // U' diagonal blocks, [ceil(in / block)][block][block]
  const _Float16* Vt;  // U' transposed, rounded to fp16
  const _Float16* Vl;  // remainders U' - Vt, rounded toward zero to fp16
  int64_t out, in;
  int bits, gs, sym, block;
  float* scales;
  int32_t* zeros;
  uint8_t* codes;
  float* einv;  // [ceil(in / block)][out] inverse row scales of the stored errors
  hipStream_t s;
};

hipError_t sweep_block(QCtx& c, int64_t a, int64_t b) {
  const int width = (int)(b - a);
  switch (c.block) {
    case 32: return launch_sweep<32>(c.gs, c.Wp, c.Ub + (a / 32) * 32 * 32, c.out, c.in, a, width, c.bits, c.sym,
                                     c.scales, c.zeros, c.codes, c.einv, c.s);
    case 64: return launch_sweep<64>(c.gs, c.Wp, c.Ub + (a / 64) * 64 * 64, c.out, c.in, a, width, c.bits, c.sym,
                                     c.scales, c.zeros, c.codes, c.einv, c.s);
    default: return launch_sweep<128>(c.gs, c.Wp, c.Ub + (a / 128) * 128 * 128, c.out, c.in, a, width, c.bits, c.sym,
                                      c.scales, c.zeros, c.codes, c.einv, c.s);
  }
}

// Columns [a, b): sweep the left half, carry its updates to the right half
// with one GEMM, then the right half.  The GEMMs read the errors the sweeps
// stored split into two fp16 parts (per row and block scaled by a power of
// two) and multiply them by U' rounded once to fp16 (two products per term),
// plus its fp16 remainder (a third product) where the rounding of U' would
// move pre-rounding values too far: for GEMMs over fewer than SPLIT_MIN_K
// error columns (the pairs of nearby columns, cheap in flops), and in layers
// wider than TWO_PRODUCT_MAX_IN.  The rounding of U' moves a pre-rounding
// value by a sum over every earlier column, which grows with the layer width:
// largest shifts measured in a CPU emulation of the two-product form were
// 3.5e-4 code units at 4096 columns, 4.2e-4 at 11008 and 1.1e-3 at 28672,
// against a 1e-3 boundary window; three products keep 9e-6 at 28672.
constexpr int64_t SPLIT_MIN_K = 512;
constexpr int64_t TWO_PRODUCT_MAX_IN = 16384;
// Two full 128-column blocks in one launch (sweep16_pair_kernel), for the
// group sizes the 16-lane sweep takes.
hipError_t sweep_pair(QCtx& c, int64_t a) {
  const float* Ub = c.Ub + (a / PAIR_B) * PAIR_B * PAIR_B;
  switch (c.gs > 0 ? c.gs : 0) {
#define GPTQ_PAIR_CASE(G)                                                                     \
  case G:                                                                                     \
    return launch_sweep16_pair<G>(c.Wp, Ub, c.Vt, c.Vl, c.out, c.in, a, c.bits, c.sym,        \
                                  c.scales, c.zeros, c.codes, c.einv, c.s);
    GPTQ_PAIR_CASE(0)
    GPTQ_PAIR_CASE(16)
    GPTQ_PAIR_CASE(32)
    GPTQ_PAIR_CASE(64)
    GPTQ_PAIR_CASE(128)
#undef GPTQ_PAIR_CASE
    default:
      return hipErrorInvalidValue;
  }
}
bool pair_fits(const QCtx& c) {
  const int g = c.gs > 0 ? c.gs : 0;
  return c.block == PAIR_B && c.Vt != nullptr &&
         (g == 0 || g == 16 || g == 32 || g == 64 || g == 128);
}

hipError_t process(QCtx& c, int64_t a, int64_t b) {
  const int64_t B = c.block;
  if (b - a <= B) return sweep_block(c, a, b);
  if (b - a == 2 * B && pair_fits(c)) return sweep_pair(c, a);
  const int64_t nblk = (b - a + B - 1) / B;
  // Where the pair kernel applies, split on pair boundaries (the left part
  // an even number of blocks), so the leaves are pairs wherever the block
  // count allows and single blocks stay rare; else halve by blocks.
  int64_t m = a + B * ((nblk + 1) / 2);
  if (pair_fits(c)) {
    const int64_t mp = a + 2 * B * (((nblk + 1) / 2 + 1) / 2);
    if (mp < b) m = mp;
  }
  GPTQ_HIP_TRY(process(c, a, m));
  const bool three = m - a < SPLIT_MIN_K || c.in > TWO_PRODUCT_MAX_IN;
  GPTQ_HIP_TRY(launch_gemm_eh(c.out, b - m, m - a, c.Wp + a, c.in, c.Vt + m * c.in + a,
                              three ? c.Vl + m * c.in + a : nullptr, c.in, c.Wp + m, c.in,
                              c.einv + (a / B) * c.out, c.out, (int)B, c.s));
  return process(c, m, b);
}

struct QLayout {
  float* Wp;
  float* Ub;
  _Float16* Vt;
  _Float16* Vl;
  uint8_t* codes;
  int32_t* pinv;
  float* einv;
  size_t bytes;
};

QLayout carve(void* ws, int64_t out, int64_t in, int block) {
  Carver c(ws);
  QLayout l;
  l.Wp = c.take<float>((size_t)out * in);
  const int64_t nblk = (in + block - 1) / block;
  l.Ub = c.take<float>((size_t)nblk * block * block);
  // the trailing GEMMs (only when the layer is wider than one block)
  const bool gemms = in > block;
  l.Vt = gemms ? c.take<_Float16>((size_t)in * in) : nullptr;
  l.Vl = gemms ? c.take<_Float16>((size_t)in * in) : nullptr;
  l.codes = c.take<uint8_t>((size_t)out * in);
  l.pinv = c.take<int32_t>((size_t)in);
  l.einv = c.take<float>((size_t)out * (size_t)((in + block - 1) / block));
  l.bytes = c.used;
  return l;
}

}  // namespace

size_t quantize_workspace_bytes(int64_t out, int64_t in, int, int, int block) {
  return carve(nullptr, out, in, block).bytes;
}

hipError_t run_quantize(const void* W, int wdtype, int64_t out, int64_t in, const float* U,
                        const int32_t* perm, int bits, int gs, int sym, int block,
                        int32_t* qweight, float* scales, int32_t* zeros, int32_t* g_idx,
                        void* ws, hipStream_t s) {
  QLayout l = carve(ws, out, in, block);
  const size_t lds = (size_t)in * sizeof(float);
  const unsigned gw_threads = lds > 64 * 1024 ? 1024 : lds > 32 * 1024 ? 512 : 256;
  if (wdtype == 0) {
    auto k = gather_w_kernel<_Float16>;
    GPTQ_HIP_TRY(hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds));
    hipLaunchKernelGGL(k, dim3((unsigned)out), dim3(gw_threads), lds, s,
                       static_cast<const _Float16*>(W), out, in, perm, l.Wp);
  } else if (wdtype == 1) {
    auto k = gather_w_kernel<uint16_t>;
    GPTQ_HIP_TRY(hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds));
    hipLaunchKernelGGL(k, dim3((unsigned)out), dim3(gw_threads), lds, s,
                       static_cast<const uint16_t*>(W), out, in, perm, l.Wp);
  } else {
    auto k = gather_w_kernel<float>;
    GPTQ_HIP_TRY(hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds));
    hipLaunchKernelGGL(k, dim3((unsigned)out), dim3(gw_threads), lds, s, static_cast<const float*>(W),
                       out, in, perm, l.Wp);
  }
  GPTQ_HIP_TRY(hipGetLastError());
  {
    const unsigned nt = (unsigned)((in + 63) / 64);
    hipLaunchKernelGGL(uprime_split_kernel, dim3(nt, nt), dim3(256), 0, s, U, in, block, l.Ub, l.Vt,
                       l.Vl);
    GPTQ_HIP_TRY(hipGetLastError());
  }
  hipLaunchKernelGGL(perm_tables_kernel, dim3((unsigned)((in + 255) / 256)), dim3(256), 0, s, perm,
                     in, gs, l.pinv, g_idx);
  GPTQ_HIP_TRY(hipGetLastError());
  if (gs <= 0) {
    hipLaunchKernelGGL(row_params_kernel, dim3((unsigned)out), dim3(256), 0, s, l.Wp, out, in,
                       bits, sym, scales, zeros);
    GPTQ_HIP_TRY(hipGetLastError());
  }
  QCtx c{l.Wp, l.Ub, l.Vt, l.Vl, out, in, bits, gs, sym, block, scales, zeros, l.codes, l.einv,
         s};
  GPTQ_HIP_TRY(process(c, 0, in));
  // rows per packing workgroup: 4 (several workgroups per compute unit to
  // cover the latency of the per-unit pinv reads; 16 rows per workgroup
  // took 117 us against 99 at 4096 x 11008), fewer if 4 rows do not fit
  int R = 4;
  while (R > 1 && (size_t)R * (in + PACK_PAD) > 160 * 1024) --R;
  const size_t plds = (size_t)R * (in + PACK_PAD);
  GPTQ_HIP_TRY(hipFuncSetAttribute((const void*)pack_kernel,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)plds));
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((out + R - 1) / R)), dim3(256), plds, s, l.codes,
                     l.pinv, out, in, bits, R, qweight);
  return hipGetLastError();
}

}  // namespace gptq
