// The attention half of a Llama-style decoder block, for the layer-wise
// calibration forward.
//
// The layer-wise method quantizes one layer at a time and takes each layer's
// calibration inputs from the block with the layers before it already
// quantized (glossary entry "gptq", paragraph "Method" (1) and (3)).  The
// input of the output projection is the attention of the (quantized) query,
// key and value projections; the input of the MLP is the normalized residual
// stream after the (quantized) output projection.  Two kernels:
//
//   attn_fwd_kernel: causal multi-head attention per sequence,
//       O[t] = sum_{s <= t} softmax_s(Q[t] . K[s] / sqrt(hd)) V[s],
//     fp16 Q, K, V in, fp32 scores, softmax and accumulation, fp16 O out.
//     One workgroup = 128 queries of one head of one sequence, eight waves
//     of 16 queries; key blocks of 64 are staged in LDS (double-buffered)
//     and walked with an online softmax; under the causal mask a wave skips
//     the 16-key tiles past its last query.  The matrix cores compute
//     S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_f16 (gfx950's
//     full-rate 16 x 16 fp16 product; k slot j of lane group g pairs A and B
//     alike): in that orientation the S^T accumulator of a lane (query
//     l % 16, keys 4 (l / 16) + 0..3 of a 16-key tile) is exactly its part of
//     the B operand of the second product (two tiles per product: k slots
//     0..3 the first, 4..7 the second), and the O^T accumulator of a lane
//     belongs to the same query as the softmax statistics the lane holds, so
//     nothing is moved between lanes except the max / sum reductions over
//     keys.
//
//   residual_rmsnorm_kernel: Hs = X + A (the residual stream, fp16) and
//     U = Hs / sqrt(mean(Hs^2) + eps) * gamma (fp16), one row per workgroup.
#include "common.hpp"

#include <cmath>

namespace gptq {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));

constexpr int AW = 8;         // waves per workgroup
constexpr int AQ = 16 * AW;   // queries per workgroup (16 per wave)
constexpr int AK = 64;        // keys per staged block

__device__ inline float4_t mfma16(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ inline half8_t cat8(half4_t lo, half4_t hi) {
  return (half8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ds_read_b64_tr_b16: in each 16-lane group, lane j receives element j % 4
// of the 8-byte reads of lanes j / 4 + 4 i (i < 4).  A lane pointing at
// (row r0 + j / 4, columns c0 + 4 (j % 4) ..) therefore receives column
// c0 + j of rows r0 .. r0 + 3.
__device__ inline half4_t ds_read_tr16(const _Float16* p) {
  const v4i16_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (v4i16_t __attribute__((address_space(3)))*)(
          (__attribute__((address_space(3))) _Float16*)(p)));
  return __builtin_bit_cast(half4_t, v);
}

// Max / sum over the four 16-lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48),
// with gfx950's row swaps: v_permlane16_swap of a register with itself
// leaves lane l's value in one result and lane l ^ 16's in the other (which
// one depends on the row), so a symmetric operation on the two is the pair's
// reduction; v_permlane32_swap likewise for l ^ 32.  (VALU only; a shuffle
// through ds_bpermute put an LDS round trip on the softmax's critical path.)
__device__ inline float vmax(float a, float b) { return __builtin_fmaxf(a, b); }
__device__ inline float group4_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return vmax(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ inline float group4_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Grid: (ceil(seq_len / 128), heads, seqs); 512 threads.  Q, K, V, O rows are
// tokens (sequence b occupies rows b * seq_len ...), head h the columns
// h * HD .. h * HD + HD - 1; every row start and ld a multiple of 8 halves.
// K and V blocks are staged row-major (16-byte stores) in two buffers: the
// next block's global loads are in flight while the current one is used.
// K rows are HD + 8 halves apart (a wave's 8-byte reads of 16 rows cover
// all banks), V rows HD + 16 (the transposing reads of 8 rows do).
template <int HD>
__global__ void __launch_bounds__(512)
attn_fwd_kernel(const _Float16* __restrict__ Q, int64_t ldq, const _Float16* __restrict__ K,
                int64_t ldk, const _Float16* __restrict__ V, int64_t ldv,
                _Float16* __restrict__ O, int64_t ldo, int seq_len, float scale_log2e,
                int causal) {
  constexpr int KP = HD + 8, VP = HD + 16;
  constexpr int NS = HD / 16;                      // 16-wide slices of the head dimension
  constexpr int NS2 = HD / 32;                     // 32-wide slices (k of the S^T product)
  constexpr int CH = AK * HD / 8;                  // 16-byte chunks of a K (or V) block
  constexpr int PT = CH / (AW * 64);               // chunks per thread
  static_assert(CH % (AW * 64) == 0, "whole chunks per thread");
  __shared__ __align__(16) _Float16 Ks[2][AK * KP];
  __shared__ __align__(16) _Float16 Vs[2][AK * VP];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.y;
  const int64_t tok0 = (int64_t)blockIdx.z * seq_len;       // first token of the sequence
  const int qb0 = blockIdx.x * AQ;                          // first query of the workgroup
  const int qw0 = qb0 + wave * 16;                          // first query of the wave
  const int qw = qw0 + (lane & 15);                         // this lane's query
  const int g = lane >> 4, kq = 4 * g;                      // lane group, its 4-slot offset

  // Q^T as B operands, one per 32-wide slice: (query qw, dims 32 s + 8 g ..).
  half8_t qf[NS2];
#pragma unroll
  for (int s = 0; s < NS2; ++s) {
    if (qw < seq_len) {
      const uint4 v =
          *reinterpret_cast<const uint4*>(Q + (tok0 + qw) * ldq + h * HD + 32 * s + 8 * g);
      qf[s] = __builtin_bit_cast(half8_t, v);
    } else {
      qf[s] = (half8_t){0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  float4_t oacc[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) oacc[s] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
  float m = -INFINITY, l = 0.0f;

  const int qlast = qb0 + AQ - 1 < seq_len - 1 ? qb0 + AQ - 1 : seq_len - 1;
  const int kend = causal ? qlast + 1 : seq_len;            // keys [0, kend)
  const int wlast = qw0 + 15 < seq_len - 1 ? qw0 + 15 : seq_len - 1;  // the wave's last query

  uint4 kr[PT], vr[PT];
  auto fetch = [&](int kb) {
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int c = tid + u * AW * 64;
      const int r = c / (HD / 8), d0 = (c % (HD / 8)) * 8;
      const int key = kb + r;
      kr[u] = vr[u] = make_uint4(0, 0, 0, 0);
      if (key < seq_len) {
        kr[u] = *reinterpret_cast<const uint4*>(K + (tok0 + key) * ldk + h * HD + d0);
        vr[u] = *reinterpret_cast<const uint4*>(V + (tok0 + key) * ldv + h * HD + d0);
      }
    }
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int c = tid + u * AW * 64;
      const int r = c / (HD / 8), d0 = (c % (HD / 8)) * 8;
      *reinterpret_cast<uint4*>(&Ks[buf][r * KP + d0]) = kr[u];
      *reinterpret_cast<uint4*>(&Vs[buf][r * VP + d0]) = vr[u];
    }
  };

  fetch(0);
  stage(0);
  __syncthreads();
  for (int kb = 0, buf = 0; kb < kend; kb += AK, buf ^= 1) {
    const bool more = kb + AK < kend;  // uniform
    if (more) fetch(kb + AK);
    // 16-key tiles of this block the wave needs (causal: keys <= its last query)
    const int nt = causal ? (wlast - kb >= AK - 1 ? 4 : wlast >= kb ? (wlast - kb) / 16 + 1 : 0) : 4;
    if (nt > 0) {
      const _Float16* ks = Ks[buf];
      const _Float16* vs = Vs[buf];
      // S^T (16 t + key, query) tiles
      float4_t sacc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        sacc[t] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
        if (t < nt) {
#pragma unroll
          for (int s = 0; s < NS2; ++s) {
            const half8_t kf = __builtin_bit_cast(
                half8_t,
                *reinterpret_cast<const uint4*>(&ks[(16 * t + (lane & 15)) * KP + 32 * s + 8 * g]));
            sacc[t] = mfma16(kf, qf[s], sacc[t]);
          }
        }
      }
      // mask (causal, past the sequence, tiles not computed) where the block
      // is not wholly visible to every query of the wave; block max
      const bool whole = kb + AK <= seq_len && (!causal || kb + AK - 1 <= qw0);  // uniform
      float bmax = -INFINITY;
      if (!whole) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = kb + 16 * t + kq + i;
            const bool ok = t < nt && key < seq_len && (!causal || key <= qw);
            sacc[t][i] = ok ? sacc[t][i] : -INFINITY;
          }
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) bmax = vmax(bmax, sacc[t][i]);
      bmax = group4_max(bmax);
      const float mnew = vmax(m, bmax);
      const float mref = mnew == -INFINITY ? 0.0f : mnew;   // a query with no key yet
      // v_exp_f32 directly (exp2(-inf) = 0 on the first block; results below
      // 2^-126 flush to zero, which the sums cannot feel)
      const float alpha = __builtin_amdgcn_exp2f((m - mref) * scale_log2e);
      const float mc = mref * scale_log2e;
      float psum = 0.0f;
      half4_t pf[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = __builtin_amdgcn_exp2f(fmaf(sacc[t][i], scale_log2e, -mc));
          psum += p[i];
        }
        pf[t] = (half4_t){(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
      }
      l = alpha * l + group4_sum(psum);
      m = mnew;
      // the running maximum rarely moves after the first blocks: rescale O
      // only when it did for some query of the wave
      const bool rescale = __builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0;
      // O^T (HD x 16 queries) = alpha O^T + V^T P^T, 32 keys (tiles 2u, 2u + 1)
      // per product; the A operand (dims 16 s + j, keys 16 t + kq ..) from
      // row-major V by transposing reads.  A tile past the wave's last one
      // (odd nt) has P = 0.
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        float4_t o = rescale ? oacc[s] * alpha : oacc[s];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          if (2 * u < nt) {
            const half4_t v0 = ds_read_tr16(
                &vs[(32 * u + kq + ((lane & 15) >> 2)) * VP + 16 * s + 4 * (lane & 3)]);
            const half4_t v1 = ds_read_tr16(
                &vs[(32 * u + 16 + kq + ((lane & 15) >> 2)) * VP + 16 * s + 4 * (lane & 3)]);
            o = mfma16(cat8(v0, v1), cat8(pf[2 * u], pf[2 * u + 1]), o);
          }
        }
        oacc[s] = o;
      }
    }
    if (more) {
      stage(buf ^ 1);  // the other buffer: everyone finished it before the last barrier
    }
    __syncthreads();
  }
  if (qw >= seq_len) return;
  const float inv = 1.0f / l;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const half4_t ov = {(_Float16)(oacc[s][0] * inv), (_Float16)(oacc[s][1] * inv),
                        (_Float16)(oacc[s][2] * inv), (_Float16)(oacc[s][3] * inv)};
    *reinterpret_cast<uint2*>(O + (tok0 + qw) * ldo + h * HD + 16 * s + kq) =
        __builtin_bit_cast(uint2, ov);
  }
}

// One row per workgroup (256 threads): Hs = fp16(X + A), then
// U = fp16(Hs * rsqrt(mean(Hs^2) + eps) * gamma), sums in fp32.
__global__ void __launch_bounds__(256)
residual_rmsnorm_kernel(const _Float16* __restrict__ X, int64_t ldx, const _Float16* __restrict__ A,
                        int64_t lda, const _Float16* __restrict__ gamma, int64_t d, float eps,
                        _Float16* __restrict__ Hs, int64_t ldh, _Float16* __restrict__ U,
                        int64_t ldu) {
  __shared__ float red[4];
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  float ss = 0.0f;
  for (int64_t c = tid; c < d; c += 256) {
    const _Float16 hv = (_Float16)((float)X[r * ldx + c] + (float)A[r * lda + c]);
    Hs[r * ldh + c] = hv;
    const float f = (float)hv;
    ss = fmaf(f, f, ss);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float rs = 1.0f / sqrtf(tot / (float)d + eps);
  // each thread re-reads only the values it wrote itself (same thread, program order)
  for (int64_t c = tid; c < d; c += 256)
    U[r * ldu + c] = (_Float16)((float)Hs[r * ldh + c] * rs * (float)gamma[c]);
}

}  // namespace

hipError_t run_attention(const void* Q, int64_t ldq, const void* K, int64_t ldk, const void* V,
                         int64_t ldv, void* O, int64_t ldo, int64_t seqs, int64_t seq_len,
                         int heads, int head_dim, int causal, hipStream_t s) {
  const float scale_log2e = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
  dim3 grid((unsigned)((seq_len + AQ - 1) / AQ), (unsigned)heads, (unsigned)seqs);
  auto q = static_cast<const _Float16*>(Q);
  auto k = static_cast<const _Float16*>(K);
  auto v = static_cast<const _Float16*>(V);
  auto o = static_cast<_Float16*>(O);
  if (head_dim == 64)
    hipLaunchKernelGGL(attn_fwd_kernel<64>, grid, dim3(AW * 64), 0, s, q, ldq, k, ldk, v, ldv, o,
                       ldo, (int)seq_len, scale_log2e, causal);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<128>, grid, dim3(AW * 64), 0, s, q, ldq, k, ldk, v, ldv, o,
                       ldo, (int)seq_len, scale_log2e, causal);
  return hipGetLastError();
}

hipError_t run_residual_rmsnorm(const void* X, int64_t ldx, const void* A, int64_t lda,
                                const void* gamma, int64_t rows, int64_t d, float eps, void* Hs,
                                int64_t ldh, void* U, int64_t ldu, hipStream_t s) {
  for (int64_t r0 = 0; r0 < rows; r0 += 1 << 30) {
    const int64_t nr = rows - r0 < (1 << 30) ? rows - r0 : (1 << 30);
    hipLaunchKernelGGL(residual_rmsnorm_kernel, dim3((unsigned)nr), dim3(256), 0, s,
                       static_cast<const _Float16*>(X) + r0 * ldx, ldx,
                       static_cast<const _Float16*>(A) + r0 * lda, lda,
                       static_cast<const _Float16*>(gamma), d, eps,
                       static_cast<_Float16*>(Hs) + r0 * ldh, ldh,
                       static_cast<_Float16*>(U) + r0 * ldu, ldu);
    GPTQ_HIP_TRY(hipGetLastError());
  }
  return hipSuccess;
}

}  // namespace gptq
