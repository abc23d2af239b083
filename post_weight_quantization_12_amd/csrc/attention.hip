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
//     One workgroup = 64 queries of one head of one sequence, four waves of
//     16 queries; key blocks of 64 are staged in LDS (K as is, V transposed)
//     and walked with an online softmax.  The matrix cores compute
//     S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x16_f16: in that
//     orientation the S^T accumulator of a lane (query l % 16, keys
//     4 (l / 16) + 0..3 of a 16-key slice) is exactly its B operand for the
//     second product, and the O^T accumulator of a lane belongs to the same
//     query as the softmax statistics the lane holds, so nothing is moved
//     between lanes except the max / sum reductions over keys.
//
//   residual_rmsnorm_kernel: Hs = X + A (the residual stream, fp16) and
//     U = Hs / sqrt(mean(Hs^2) + eps) * gamma (fp16), one row per workgroup.
#include "common.hpp"

#include <cmath>

namespace gptq {
namespace {

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int AQ = 64;   // queries per workgroup (16 per wave)
constexpr int AK = 64;   // keys per staged block

__device__ inline float4_t mfma16(half4_t a, half4_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// Max / sum over the four 16-lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48).
__device__ inline float group4_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}
__device__ inline float group4_sum(float v) {
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
}

// Grid: (ceil(seq_len / 64), heads, seqs); 256 threads.  Q, K, V, O rows are
// tokens (sequence b occupies rows b * seq_len ...), head h the columns
// h * HD .. h * HD + HD - 1; every row start and ld a multiple of 8 halves.
template <int HD>
__global__ void __launch_bounds__(256)
attn_fwd_kernel(const _Float16* __restrict__ Q, int64_t ldq, const _Float16* __restrict__ K,
                int64_t ldk, const _Float16* __restrict__ V, int64_t ldv,
                _Float16* __restrict__ O, int64_t ldo, int seq_len, float scale_log2e,
                int causal) {
  constexpr int KP = HD + 8;   // K rows in LDS (halves): 8-byte reads spread over the banks
  constexpr int VP = AK + 8;   // V^T rows in LDS (halves)
  constexpr int NS = HD / 16;  // 16-wide slices of the head dimension
  __shared__ __align__(16) _Float16 Ks[AK * KP];
  __shared__ __align__(16) _Float16 Vt[HD * VP];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = blockIdx.y;
  const int64_t tok0 = (int64_t)blockIdx.z * seq_len;       // first token of the sequence
  const int qb0 = blockIdx.x * AQ;                          // first query of the workgroup
  const int qw = qb0 + wave * 16 + (lane & 15);             // this lane's query
  const int kq = 4 * (lane >> 4);                           // this lane's 4-slot offset

  // Q^T as B operands, one per 16-wide slice: (query qw, dims 16 s + kq ..).
  half4_t qf[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (qw < seq_len) {
      const uint2 v = *reinterpret_cast<const uint2*>(Q + (tok0 + qw) * ldq + h * HD + 16 * s + kq);
      qf[s] = __builtin_bit_cast(half4_t, v);
    } else {
      qf[s] = (half4_t){0, 0, 0, 0};
    }
  }
  float4_t oacc[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) oacc[s] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
  float m = -INFINITY, l = 0.0f;

  const int qlast = qb0 + AQ - 1 < seq_len - 1 ? qb0 + AQ - 1 : seq_len - 1;
  const int kend = causal ? qlast + 1 : seq_len;            // keys [0, kend)
  for (int kb = 0; kb < kend; kb += AK) {
    __syncthreads();  // the previous block's LDS reads are done
    // stage K (row-major) and V^T: 64 keys x HD dims, 16-byte chunks
    for (int c = tid; c < AK * HD / 8; c += 256) {
      const int r = c / (HD / 8), d0 = (c % (HD / 8)) * 8;
      const int key = kb + r;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (key < seq_len) {
        kv = *reinterpret_cast<const uint4*>(K + (tok0 + key) * ldk + h * HD + d0);
        vv = *reinterpret_cast<const uint4*>(V + (tok0 + key) * ldv + h * HD + d0);
      }
      *reinterpret_cast<uint4*>(&Ks[r * KP + d0]) = kv;
      const uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Vt[(d0 + 2 * j) * VP + r] = __builtin_bit_cast(_Float16, (uint16_t)(w[j] & 0xFFFFu));
        Vt[(d0 + 2 * j + 1) * VP + r] = __builtin_bit_cast(_Float16, (uint16_t)(w[j] >> 16));
      }
    }
    __syncthreads();

    // S^T (64 keys x 16 queries) in four 16 x 16 tiles
    float4_t sacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sacc[t] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const half4_t kf = __builtin_bit_cast(
            half4_t, *reinterpret_cast<const uint2*>(&Ks[(16 * t + (lane & 15)) * KP + 16 * s + kq]));
        sacc[t] = mfma16(kf, qf[s], sacc[t]);
      }
    }
    // mask (causal, past the sequence), block max over this lane's keys
    float bmax = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb + 16 * t + kq + i;
        const bool ok = key < seq_len && (!causal || key <= qw);
        sacc[t][i] = ok ? sacc[t][i] : -INFINITY;
        bmax = fmaxf(bmax, sacc[t][i]);
      }
    bmax = group4_max(bmax);
    const float mnew = fmaxf(m, bmax);
    const float mref = mnew == -INFINITY ? 0.0f : mnew;     // a query with no key yet
    const float alpha = exp2f((m - mref) * scale_log2e);    // exp2(-inf) = 0 on the first block
    float psum = 0.0f;
    half4_t pf[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = exp2f((sacc[t][i] - mref) * scale_log2e);
        psum += p[i];
      }
      pf[t] = (half4_t){(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3]};
    }
    l = alpha * l + group4_sum(psum);
    m = mnew;
    // O^T (HD x 16 queries) = alpha O^T + V^T P^T
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      float4_t o = oacc[s] * alpha;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const half4_t vf = __builtin_bit_cast(
            half4_t, *reinterpret_cast<const uint2*>(&Vt[(16 * s + (lane & 15)) * VP + 16 * t + kq]));
        o = mfma16(vf, pf[t], o);
      }
      oacc[s] = o;
    }
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
    hipLaunchKernelGGL(attn_fwd_kernel<64>, grid, dim3(256), 0, s, q, ldq, k, ldk, v, ldv, o, ldo,
                       (int)seq_len, scale_log2e, causal);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<128>, grid, dim3(256), 0, s, q, ldq, k, ldk, v, ldv, o,
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
