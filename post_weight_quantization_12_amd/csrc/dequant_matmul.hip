// Dequantize-on-the-fly matmul Y = X W^T from the packed layer on gfx950.
//
// The glossary entry "gptq" (paragraph "Inference") applies a quantized
// layer by dequantizing its weights during the computation and multiplying.
// The layer arrives as gptq_quantize_layer writes it: qweight int32
// [in * b / 32 x out] (row r's codes form a little-endian b-bit stream along
// the input dimension, word j of that stream in qweight[j][r]), scales fp32
// and zeros int32 [n_groups x out], g_idx int32 [in]:
//     W[r][k] = scales[g_idx[k]][r] * (code[r][k] - zeros[g_idx[k]][r]).
// A 32-code chunk of a row's stream is exactly b words, so every kernel here
// walks the input dimension 32 k at a time, whatever b is.
//
// Two kernels:
//   * few tokens (M <= 8, decode): HBM-bound on qweight.  Lane = output
//     column (a wave's 64 columns read 256 contiguous bytes per word row),
//     the four waves of a workgroup take interleaved chunks of the
//     workgroup's input range; per chunk, exact (q - z) code pairs in fp16
//     meet X pairs in v_dot2_f32_f16 (fp32 sums, up to 8 token rows held
//     in registers) and the sum is scaled once; X's slice of the input range
//     is staged in LDS as fp16 pairs.  The input dimension is split over
//     several workgroups (grid >= 2 per compute unit); their partial sums go
//     to the workspace and a second kernel adds them in a fixed order.
//   * many tokens (prefill): 256 x 256 tiles from 256 tokens on, 128 x 128
//     below, on v_mfma_f32_32x32x16_f16.
//     Per 32-k chunk the X tile goes to LDS as is (k contiguous: an MFMA A
//     operand is one 16-byte read) and the weight tile is dequantized into
//     LDS as fp16 column-major (k contiguous: a B operand is one 16-byte
//     read): a code pair becomes the half2 (1024 + q0, 1024 + q1) by OR-ing
//     it into 0x6400 0x6400, minus (1024 + z) (exact: integers below 2048),
//     times the scale split into two fp16 parts s = sh + sl (sh = fp16(s),
//     sl = fp16(s - sh)) as one fused (q - z) sh + fl((q - z) sl): close to
//     the fp16 rounding of the exact weight.  A scale rounded to fp16 alone
//     would scale a whole group-row of weights by the same factor (1 + d),
//     |d| <= 2^-11, an error that does not average out over the group.
#include "common.hpp"

#include <type_traits>

namespace gptq {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

constexpr int DQ_CHUNK = 32;   // k per chunk
constexpr int SMALL_COLS = 64; // output columns per small-M workgroup
constexpr int SMALL_LDS_MAX = 64 * 1024;
constexpr int SMALL_DEPTH = 4;  // chunks whose words a lane loads ahead

// Code k (0..31, a constant after unrolling) of a chunk whose B words are
// w[0..B-1] (w[B] == 0).
template <int B>
__device__ inline uint32_t chunk_code(const uint32_t* w, int k) {
  const int pos = k * B, wi = pos / 32, off = pos % 32;
  const uint32_t lo = w[wi] >> off;
  const uint32_t v = off + B <= 32 ? lo : (lo | (w[wi + 1] << (32 - off)));
  return v & ((1u << B) - 1u);
}

// Code pairs.  A chunk's 32 codes form 16 pairs whose two b-bit fields sit
// at the same offsets of the two halves of one word (for b = 2, 4, 8), so
// one shift and one AND extract a pair as (lo, hi) 16-bit lanes:
//   b = 4: pair p = (code 8j + i, code 8j + i + 4), j = p / 4, i = p % 4
//   b = 8: pair p = (code 4j + i, code 4j + i + 2), j = p / 2, i = p % 2
//   b = 2: pair p = (code 16j + i, code 16j + i + 8), j = p / 8, i = p % 8
//   b = 3: pair p = (code 2p, code 2p + 1), fields gathered one by one.
template <int B>
__host__ __device__ constexpr int pair_code(int p, int hi) {
  return B == 4 ? 8 * (p / 4) + p % 4 + 4 * hi
       : B == 8 ? 4 * (p / 2) + p % 2 + 2 * hi
       : B == 2 ? 16 * (p / 8) + p % 8 + 8 * hi
       : 2 * p + hi;
}
// (a & m) | o in one VALU op.  gfx950's three-operand encoding takes no
// literal, so the masks live in registers the caller keeps.
__device__ inline uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(m), "v"(o));
  return d;
}
// Pair p of a chunk whose words are w, as the fp16 pair (1024 + lo, 1024 + hi).
// m = the pair mask of B (0x000F000F for B = 4, ...), o = 0x64006400.
template <int B>
__device__ inline uint32_t pair_magic(const uint32_t* w, int p, uint32_t m, uint32_t o) {
  if constexpr (B == 4) return and_or(w[p / 4] >> (4 * (p % 4)), m, o);
  if constexpr (B == 8) return and_or(w[p / 2] >> (8 * (p % 2)), m, o);
  if constexpr (B == 2) return and_or(w[p / 8] >> (2 * (p % 8)), m, o);
  return chunk_code<B>(w, 2 * p) | (chunk_code<B>(w, 2 * p + 1) << 16) | 0x64006400u;
}
template <int B>
__host__ __device__ constexpr uint32_t pair_mask() {
  return B == 4 ? 0x000F000Fu : B == 8 ? 0x00FF00FFu : B == 2 ? 0x00030003u : 0u;
}

// ---------------------------------------------------------------- small M --
// Grid: (ceil(out / (64 CPL)), nsplit).  Workgroup (bx, by) covers columns
// [64 CPL bx, 64 CPL (bx + 1)) and chunks [by * cps, min((by + 1) * cps, in / 32));
// lane l of every wave owns the CPL adjacent columns from 64 CPL bx + CPL l
// (CPL = 4: one 16-byte load per word row), and the four waves take
// interleaved chunks of the range.  MB = token rows held per lane (>= M, a
// power of two up to 8).
// LDS: xp[pair][MB], the X slice as fp16 pairs in the chunks' pair order
// (pair p of chunk c at 16 c + p), then cg[cps]: the group of each chunk of
// the slice when all its 32 k share one, else -1.
//
// A single-group chunk is summed as s * sum_k x_k (q_k - z): each pair
// (q_a - z, q_b - z) is formed exactly in fp16 (0x6400 | q is 1024 + q,
// minus 1024 + z: integers below 2048) and v_dot2_f32_f16 multiplies it with
// the X pair into an fp32 sum (products of fp16 values are exact in fp32);
// the chunk's sum is scaled by s once.  Mixed-group chunks dequantize each
// weight in fp32 as s (q - z).
template <int B, int CPL>
__host__ __device__ constexpr int small_depth() {
  // chunks per prefetched block: about 16 words per column group in flight
  return CPL == 1 ? SMALL_DEPTH : B == 8 ? 1 : B == 2 ? 4 : 2;
}

template <int B, int MB, int CPL>
__global__ void __launch_bounds__(256)
dq_small_kernel(const _Float16* __restrict__ X, int64_t M, int64_t in, int64_t ldx,
                const uint32_t* __restrict__ qw, const float* __restrict__ scales,
                const int32_t* __restrict__ zeros, const int32_t* __restrict__ g_idx,
                const int32_t* __restrict__ x_order, int64_t out, int64_t cps,
                float* __restrict__ part, void* __restrict__ Y, int y_f16, int64_t ldy) {
  constexpr int D = small_depth<B, CPL>();
  constexpr int COLS = 64 * CPL;
  constexpr int NP = CPL == 1 ? 2 : 1;  // partial sums per (column, row)
  extern __shared__ __align__(16) uint32_t xp[];
  const int tid = threadIdx.x, lane = tid & 63;
  // uniform: the chunk index, g_idx reads and the group test stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t colb = (int64_t)blockIdx.x * COLS + (int64_t)lane * CPL;
  // loads stay in bounds, unconditional (CPL = 4 implies out % 4 == 0)
  const int64_t colc = colb + CPL <= out ? colb : out - CPL;
  const int64_t nch = in / DQ_CHUNK;
  const int64_t c0 = (int64_t)blockIdx.y * cps;
  const int64_t c1 = c0 + cps < nch ? c0 + cps : nch;
  const int ncl = (int)(c1 - c0);
  int* cg = reinterpret_cast<int*>(xp + (size_t)ncl * 16 * MB);
  // Chunks c0 + wave, + 4, + 8, ... in blocks of D.  The words of the next
  // block, and the scales and zeros of each of its single-group chunks, are
  // loaded before the current block is used, so the memory latency overlaps
  // the arithmetic.
  struct Blk {
    uint32_t w[D][B][CPL];
    float s[D][CPL];
    int32_t z[D][CPL];
    int g[D];
  };
  auto load_words = [&](int64_t cb, Blk& k) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int64_t c = cb + 4 * d < c1 ? cb + 4 * d : c0;  // past the end: a valid dummy, unused
#pragma unroll
      for (int i = 0; i < B; ++i) {
        const uint32_t* src = qw + (c * B + i) * out + colc;
        if constexpr (CPL == 4) {
          const uint4 v = *reinterpret_cast<const uint4*>(src);
          k.w[d][i][0] = v.x; k.w[d][i][1] = v.y; k.w[d][i][2] = v.z; k.w[d][i][3] = v.w;
        } else {
          k.w[d][i][0] = *src;
        }
      }
    }
  };
  auto load_groups = [&](int64_t cb, Blk& k) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int64_t c = cb + 4 * d < c1 ? cb + 4 * d : c0;
      k.g[d] = __builtin_amdgcn_readfirstlane(cg[c - c0]);
      const int64_t gi = k.g[d] >= 0 ? k.g[d] : 0;
      if constexpr (CPL == 4) {
        const float4 sv = *reinterpret_cast<const float4*>(scales + gi * out + colc);
        const int4 zv = *reinterpret_cast<const int4*>(zeros + gi * out + colc);
        k.s[d][0] = sv.x; k.s[d][1] = sv.y; k.s[d][2] = sv.z; k.s[d][3] = sv.w;
        k.z[d][0] = zv.x; k.z[d][1] = zv.y; k.z[d][2] = zv.z; k.z[d][3] = zv.w;
      } else {
        k.s[d][0] = scales[gi * out + colc];
        k.z[d][0] = zeros[gi * out + colc];
      }
    }
  };
  Blk cur, nxt;
  // the first block's words are independent of the staging below: in flight
  // while it runs
  load_words(c0 + wave, cur);
  // X slice: one thread per (row, chunk): 32 halves in, 16 pairs out
  for (int e = tid; e < MB * ncl; e += 256) {
    const int m = e / ncl, c = e % ncl;
    _Float16 xv[DQ_CHUNK];
    if (m >= M) {
#pragma unroll
      for (int k = 0; k < DQ_CHUNK; ++k) xv[k] = (_Float16)0.0f;
    } else if (x_order) {
      const int32_t* xo = x_order + (c0 + c) * DQ_CHUNK;
#pragma unroll
      for (int k = 0; k < DQ_CHUNK; ++k) xv[k] = X[m * ldx + xo[k]];
    } else {
      const uint4* src = reinterpret_cast<const uint4*>(X + m * ldx + (c0 + c) * DQ_CHUNK);
#pragma unroll
      for (int q = 0; q < DQ_CHUNK / 8; ++q) {
        const uint4 v = src[q];
        const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const half2_t h = __builtin_bit_cast(half2_t, u[j]);
          xv[8 * q + 2 * j] = h.x;
          xv[8 * q + 2 * j + 1] = h.y;
        }
      }
    }
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const half2_t h = {xv[pair_code<B>(p, 0)], xv[pair_code<B>(p, 1)]};
      xp[(16 * c + p) * MB + m] = __builtin_bit_cast(uint32_t, h);
    }
  }
  // chunk groups: a wave reads 64 consecutive g_idx (two chunks) per step
  for (int c2 = 2 * wave; c2 < ncl; c2 += 8) {
    const int k = 32 * c2 + lane;
    const int g = k < 32 * ncl ? g_idx[c0 * DQ_CHUNK + k] : 0;
    const int g0 = __shfl(g, lane & 32);
    const uint64_t diff = __ballot(g != g0);
    if ((lane & 31) == 0 && k < 32 * ncl)
      cg[c2 + (lane >> 5)] = ((lane ? (diff >> 32) : (diff & 0xffffffffull)) == 0) ? g0 : -1;
  }
  __syncthreads();

  float acc[CPL][MB];
#pragma unroll
  for (int j = 0; j < CPL; ++j)
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[j][m] = 0.0f;
  const uint32_t pm = pair_mask<B>(), pmagic = 0x64006400u;
  load_groups(c0 + wave, cur);
  auto process = [&](int64_t cb, const Blk& cur) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int64_t c = cb + 4 * d;
      if (c >= c1) break;  // uniform
      const uint32_t* xc = xp + (size_t)(c - c0) * 16 * MB;
      if (cur.g[d] >= 0) {
        half2_t zz[CPL];
        uint32_t wj[CPL][B + 1];
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          const _Float16 zf = (_Float16)(1024 + cur.z[d][j]);
          zz[j] = (half2_t){zf, zf};
#pragma unroll
          for (int i = 0; i < B; ++i) wj[j][i] = cur.w[d][i][j];
          wj[j][B] = 0u;
        }
        float cs[CPL][NP][MB];
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
          for (int q = 0; q < NP; ++q)
#pragma unroll
            for (int m = 0; m < MB; ++m) cs[j][q][m] = 0.0f;
#pragma unroll
        for (int p4 = 0; p4 < 16; p4 += 4) {
          uint32_t xv[4 * MB];
#pragma unroll
          for (int q = 0; q < MB; ++q) {
            const uint4 v = *reinterpret_cast<const uint4*>(xc + p4 * MB + 4 * q);
            xv[4 * q] = v.x; xv[4 * q + 1] = v.y; xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
          }
#pragma unroll
          for (int pp = 0; pp < 4; ++pp)
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
              const half2_t h =
                  __builtin_bit_cast(half2_t, pair_magic<B>(wj[j], p4 + pp, pm, pmagic)) - zz[j];
#pragma unroll
              for (int m = 0; m < MB; ++m)
                cs[j][pp % NP][m] = __builtin_amdgcn_fdot2(
                    h, __builtin_bit_cast(half2_t, xv[pp * MB + m]), cs[j][pp % NP][m], false);
            }
        }
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
          for (int m = 0; m < MB; ++m)
            acc[j][m] = fmaf(cur.s[d][j], NP == 2 ? cs[j][0][m] + cs[j][NP - 1][m] : cs[j][0][m],
                             acc[j][m]);
      } else {
        // the chunk's groups (uniform), one scale and zero per k
        const int64_t kb = c * DQ_CHUNK;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          uint32_t wj[B + 1];
#pragma unroll
          for (int i = 0; i < B; ++i) wj[i] = cur.w[d][i][j];
          wj[B] = 0u;
#pragma unroll 4
          for (int p = 0; p < 16; ++p) {
#pragma unroll
            for (int hi = 0; hi < 2; ++hi) {
              const int k = pair_code<B>(p, hi);
              const int64_t g = g_idx[kb + k];
              const float sc = scales[g * out + colc + j];
              const float wv =
                  sc * (float)((int)chunk_code<B>(wj, k) - zeros[g * out + colc + j]);
#pragma unroll
              for (int m = 0; m < MB; ++m) {
                const half2_t xh = __builtin_bit_cast(half2_t, xc[p * MB + m]);
                acc[j][m] = fmaf((float)(hi ? xh.y : xh.x), wv, acc[j][m]);
              }
            }
          }
        }
      }
    }
  };
  // two buffers in turn; a block past the end is neither loaded nor used
  for (int64_t cb = c0 + wave; cb < c1; cb += 8 * D) {
    if (cb + 4 * D < c1) {
      load_words(cb + 4 * D, nxt);
      load_groups(cb + 4 * D, nxt);
    }
    process(cb, cur);
    if (cb + 4 * D >= c1) break;
    if (cb + 8 * D < c1) {
      load_words(cb + 8 * D, cur);
      load_groups(cb + 8 * D, cur);
    }
    process(cb + 4 * D, nxt);
  }
  // the four waves' sums, in wave order
  __syncthreads();
  float* red = reinterpret_cast<float*>(xp);  // [4][MB][COLS]
#pragma unroll
  for (int j = 0; j < CPL; ++j)
#pragma unroll
    for (int m = 0; m < MB; ++m) red[(wave * MB + m) * COLS + lane * CPL + j] = acc[j][m];
  __syncthreads();
  for (int e = tid; e < MB * COLS; e += 256) {
    const int m = e / COLS, l = e % COLS;
    const int64_t cc = (int64_t)blockIdx.x * COLS + l;
    if (m >= M || cc >= out) continue;
    const float v = ((red[(0 * MB + m) * COLS + l] + red[(1 * MB + m) * COLS + l]) +
                     red[(2 * MB + m) * COLS + l]) + red[(3 * MB + m) * COLS + l];
    if (gridDim.y > 1) {
      part[((int64_t)blockIdx.y * M + m) * out + cc] = v;
    } else if (y_f16) {
      static_cast<_Float16*>(Y)[m * ldy + cc] = (_Float16)v;
    } else {
      static_cast<float*>(Y)[m * ldy + cc] = v;
    }
  }
}

// Y = sum of the nsplit partials, in split order.
__global__ void __launch_bounds__(256)
dq_reduce_kernel(const float* __restrict__ part, int nsplit, int64_t M, int64_t out,
                 void* __restrict__ Y, int y_f16, int64_t ldy) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= M * out) return;
  const int64_t m = e / out, cc = e % out, stride = M * out;
  float v = part[e];
  int s = 1;
  for (; s + 8 <= nsplit; s += 8) {  // eight loads in flight, added in split order
    float t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = part[(int64_t)(s + j) * stride + e];
#pragma unroll
    for (int j = 0; j < 8; ++j) v += t[j];
  }
  for (; s < nsplit; ++s) v += part[(int64_t)s * stride + e];
  if (y_f16)
    static_cast<_Float16*>(Y)[m * ldy + cc] = (_Float16)v;
  else
    static_cast<float*>(Y)[m * ldy + cc] = v;
}

// ---------------------------------------------------------------- MFMA path --
constexpr int TN = 128;          // tile columns (outputs); rows (tokens): TM = 128 or 256
constexpr int XP = DQ_CHUNK + 8; // LDS pitch in halves (80 bytes, 16-byte aligned rows)

// Grid: (ceil(out / 128), ceil(M / TM), nsplit); 8 waves, TM / 64 x
// 512 / TM of them, each a 64 x (TM / 4) block (64 x 64 for TM = 256,
// 64 x 32 for TM = 128, which fits fewer tokens).  Split z covers chunks [z cps, min((z + 1) cps, in / 32));
// with more than one split the fp32 sums go to part[z][M][out] for
// dq_reduce_kernel.  Two LDS buffers: while the matrix cores work on chunk
// c, the X tile and the weight words of chunk c + 1 (and the scale and zero
// of its group) are in flight; they are dequantized into the other buffer
// afterwards, and one barrier per chunk separates the two.  g_idx is read
// two chunks ahead.  A 256-row tile halves the dequantization per matrix-core
// flop against 128 rows: each thread dequantizes 8 codes of one column.
template <int B, int TM>
__global__ void __launch_bounds__(512)
dq_mfma_kernel(const _Float16* __restrict__ X, int64_t M, int64_t in, int64_t ldx,
               const uint32_t* __restrict__ qw, const float* __restrict__ scales,
               const int32_t* __restrict__ zeros, const int32_t* __restrict__ g_idx,
               int64_t out, int64_t cps, float* __restrict__ part, void* __restrict__ Y,
               int y_f16, int64_t ldy) {
  __shared__ __align__(16) _Float16 Xs[2][TM * XP];  // TM: template parameter
  __shared__ __align__(16) _Float16 Ws[2][TN * XP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int WMN = TM / 64;          // waves along the rows
  constexpr int FB = TM == 256 ? 2 : 1; // 32-column blocks per wave
  const int wm = wave % WMN, wn = wave / WMN;
  const int64_t m0 = (int64_t)blockIdx.y * TM, n0 = (int64_t)blockIdx.x * TN;
  // weight dequantization: column wc, codes 8 wq .. 8 wq + 7 of each chunk
  const int wc = tid % TN;
  const int wq = __builtin_amdgcn_readfirstlane(tid / TN);  // uniform within a wave
  const int64_t wcol = n0 + wc;
  const int64_t wcolc = wcol < out ? wcol : out - 1;  // in-bounds loads; columns >= out never stored
  // the (at most two) words holding the thread's 8 codes: bits [8 wq B, 8 wq B + 8 B)
  const int wbit = 8 * wq * B;
  const int wlo = wbit / 32, woff = wbit % 32;
  const bool two = woff + 8 * B > 32;  // uniform
  const int64_t nch_all = in / DQ_CHUNK;
  const int64_t cbeg = (int64_t)blockIdx.z * cps;
  const int64_t nch = cbeg + cps < nch_all ? cbeg + cps : nch_all;  // end of this split

  f32x16_t acc[2][FB];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < FB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  constexpr int XI = TM / 128;
  uint4 xr[XI];       // X tile part: rows tid / 4 + 128 i, k-octet tid % 4
  uint32_t w0, w1;    // the weight words of column wc holding its 8 codes
  int gA[8], gB[8];   // groups of the staged chunk's 8 k, and of the chunk after
  float sA;           // scale and zero of gA[0]
  int32_t zA;
  bool oneA;
  auto load_g = [&](int64_t c, int* g) {
    const int64_t cc = c < nch ? c : nch - 1;
#pragma unroll
    for (int k = 0; k < 8; ++k) g[k] = g_idx[cc * DQ_CHUNK + 8 * wq + k];
  };
  auto fetch = [&](int64_t c) {
    const int64_t kb = c * DQ_CHUNK;
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int r = tid / 4 + 128 * i, o = 8 * (tid % 4);
      xr[i] = make_uint4(0u, 0u, 0u, 0u);
      if (m0 + r < M) xr[i] = *reinterpret_cast<const uint4*>(X + (m0 + r) * ldx + kb + o);
    }
    w0 = qw[(c * B + wlo) * out + wcolc];
    w1 = two ? qw[(c * B + wlo + 1) * out + wcolc] : 0u;
    bool one = true;
#pragma unroll
    for (int k = 1; k < 8; ++k) one = one && gA[k] == gA[0];
    oneA = one;
    sA = scales[(int64_t)gA[0] * out + wcolc];
    zA = zeros[(int64_t)gA[0] * out + wcolc];
  };
  auto stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XI; ++i) {
      const int r = tid / 4 + 128 * i, o = 8 * (tid % 4);
      *reinterpret_cast<uint4*>(&Xs[buf][r * XP + o]) = xr[i];
    }
    half2_t sh[4], sl[4], zz[4];
    // s = hi + lo in fp16: s - hi is exact in fp32, lo its fp16 rounding
    auto lo16 = [](float s, _Float16 h) { return (_Float16)(s - (float)h); };
    if (oneA) {
      const _Float16 h = (_Float16)sA;
      const half2_t s2 = {h, h};
      const _Float16 l = lo16(sA, h);
      const half2_t l2 = {l, l};
      const half2_t z2 = {(_Float16)(1024.0f + (float)zA), (_Float16)(1024.0f + (float)zA)};
#pragma unroll
      for (int p = 0; p < 4; ++p) { sh[p] = s2; sl[p] = l2; zz[p] = z2; }
    } else {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float s0 = scales[(int64_t)gA[2 * p] * out + wcolc];
        const float s1 = scales[(int64_t)gA[2 * p + 1] * out + wcolc];
        const float z0 = (float)zeros[(int64_t)gA[2 * p] * out + wcolc];
        const float z1 = (float)zeros[(int64_t)gA[2 * p + 1] * out + wcolc];
        const _Float16 h0 = (_Float16)s0, h1 = (_Float16)s1;
        sh[p] = (half2_t){h0, h1};
        sl[p] = (half2_t){lo16(s0, h0), lo16(s1, h1)};
        zz[p] = (half2_t){(_Float16)(1024.0f + z0), (_Float16)(1024.0f + z1)};
      }
    }
    // the 8 codes: a 64-bit window of the column's stream starting at woff
    const uint64_t win = (((uint64_t)w1 << 32) | w0) >> woff;
    constexpr uint32_t mask = (1u << B) - 1u;
    uint32_t packed[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t q0 = (uint32_t)(win >> (2 * p * B)) & mask;
      const uint32_t q1 = (uint32_t)(win >> ((2 * p + 1) * B)) & mask;
      const uint32_t q2 = q0 | (q1 << 16) | 0x64006400u;
      const half2_t qz = __builtin_bit_cast(half2_t, q2) - zz[p];
      // one rounding of (q - z) sh + fl((q - z) sl): the large product is
      // exact inside the fused operation
      const half2_t d = __builtin_elementwise_fma(qz, sh[p], qz * sl[p]);
      packed[p] = __builtin_bit_cast(uint32_t, d);
    }
    *reinterpret_cast<uint4*>(&Ws[buf][wc * XP + 8 * wq]) =
        make_uint4(packed[0], packed[1], packed[2], packed[3]);
  };

  load_g(cbeg, gA);
  load_g(cbeg + 1, gB);
  fetch(cbeg);
  stage(0);
  __syncthreads();
  for (int64_t c = cbeg; c < nch; ++c) {
    const int buf = (int)((c - cbeg) & 1);
    const bool more = c + 1 < nch;  // uniform
    if (more) {
#pragma unroll
      for (int k = 0; k < 8; ++k) gA[k] = gB[k];
      fetch(c + 1);
      load_g(c + 2, gB);
    }
#pragma unroll
    for (int kk = 0; kk < DQ_CHUNK; kk += 16) {
      const int ko = kk + 8 * (lane >> 5);
      half8_t af[2], bf[FB];
#pragma unroll
      for (int a = 0; a < 2; ++a)
        af[a] = *reinterpret_cast<const half8_t*>(
            &Xs[buf][(wm * 64 + a * 32 + (lane & 31)) * XP + ko]);
#pragma unroll
      for (int b = 0; b < FB; ++b)
        bf[b] = *reinterpret_cast<const half8_t*>(
            &Ws[buf][(wn * 32 * FB + b * 32 + (lane & 31)) * XP + ko]);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < FB; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[a], bf[b], acc[a][b], 0, 0, 0);
    }
    if (more) stage(buf ^ 1);
    __syncthreads();
  }
  // 32 x 32 block layout: element v of lane l is row 8 (v / 4) + 4 (l / 32) + v % 4,
  // column l % 32
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < FB; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t r = m0 + wm * 64 + a * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int64_t cc = n0 + wn * 32 * FB + b * 32 + (lane & 31);
        if (r < M && cc < out) {
          if (gridDim.z > 1)
            part[((int64_t)blockIdx.z * M + r) * out + cc] = acc[a][b][v];
          else if (y_f16)
            static_cast<_Float16*>(Y)[r * ldy + cc] = (_Float16)acc[a][b][v];
          else
            static_cast<float*>(Y)[r * ldy + cc] = acc[a][b][v];
        }
      }
}

// ------------------------------------------------------- 256 x 256 tiles --
// Prefill from 256 tokens on.  Workgroup tile: 256 tokens x 256 outputs, 8
// waves as 2 x 4 blocks of 128 tokens x 64 outputs (4 x 2 blocks of 32 x 32,
// 8 MFMAs per 16 k).  A stage is one 32-k chunk of two 16-k substeps.
//   * X goes from memory straight into LDS (buffer_load ... lds), and so do
//     the weight words, scales and zeros: all of stage s + 6 at the middle
//     of stage s, into a ring of six stage slots.  A stage's loads are 16 X
//     pieces, b word rows and the scale and zero rows, 1 KiB each, dealt
//     round-robin to the 8 waves: wave w issues loads w, w + 8, ... (K or
//     K - 1 of them, K = 3, 4 for 8 bits; a direct-to-LDS load costs the
//     compute unit about 44 cycles whatever its size, so none is issued
//     for nothing).  Loads complete in issue order, so "the loads of stage
//     s + 1 have landed" is vmcnt <= 4 K_w at the middle of stage s.
//   * The A operands (X) are read from LDS: per MFMA 512 bytes (128-token
//     blocks).  The B operands never touch LDS as weights: each lane reads
//     the one to three words holding its 8 codes (column, 8-k group) and
//     the column's scale and zero, and dequantizes them in registers (the
//     two-part scale of the 128 x 128 kernel, bit-identical weights); the
//     two waves that share a column range both do so.  A substep's
//     dequantization runs between the MFMAs of the substep before it, so
//     the matrix cores keep running while it executes.
//   * X rows are 64 bytes, four 16-byte chunks; chunk q of row r sits at
//     position q ^ swz(r), swz(r) = (r >> 2) & 3: the 16-byte reads of 16
//     adjacent lanes (rows) hit distinct banks of the 64.  Token rows past
//     M read as zeros (buffer range).
//   * Each chunk's group (or -1 where its 32 g_idx entries differ) comes
//     from a table a small kernel writes first; a mixed chunk takes scale
//     and zero per weight from memory (after the one-group result, which it
//     replaces).
//   * One barrier per stage, between its two substeps (s_barrier with
//     explicit waits: a fence would drain the loads in flight).
//   * Needs out % 4 == 0 and 16-byte aligned qweight, scales and zeros (the
//     launcher falls back to the 128 x 128 kernel otherwise); buffer offsets
//     are 32-bit (the argument check bounds qweight, scales and zeros below
//     2 GiB and, from 9 tokens on, ldx by 2^22).
// Tiles: a 1-D grid over (token tile, split, column tile), column tiles
// fastest; block b runs logical tile (b % 8) per_xcd + b / 8, so each XCD
// (blocks dispatched round-robin) walks a contiguous run and its ~32
// resident workgroups share one X tile in its L2.
constexpr int QT = 256;
constexpr int QT_L = 6;  // ring slots
template <int B>
__host__ __device__ constexpr int qt_loads_per_wave() { return B == 8 ? 4 : 3; }
constexpr int QT_STAGE = QT * DQ_CHUNK * 2;  // bytes of one 256 x 32 fp16 tile

// 16 lanes of a 16-byte LDS access are served together from 64 banks
// (256 bytes): rows r and r + 4 k share banks unless their chunks differ.
__device__ inline int qt_swz(int r) { return (r >> 2) & 3; }

__device__ inline void qt_dma(__amdgpu_buffer_rsrc_t rs, uint32_t voff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) char*)lds),
      16, voff, 0, 0, 0);
}

// cgroup[c] = the group of chunk c when its 32 g_idx entries are equal, else -1.
__global__ void __launch_bounds__(256)
dq_chunk_group_kernel(const int32_t* __restrict__ g_idx, int64_t nch, int32_t* __restrict__ cgroup) {
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= nch) return;
  const int32_t* g = g_idx + c * DQ_CHUNK;
  const int32_t g0 = g[0];
  int diff = 0;
  for (int k = 1; k < DQ_CHUNK; ++k) diff |= g[k] ^ g0;
  cgroup[c] = diff == 0 ? g0 : -1;
}

// Codes 8 kg .. 8 kg + 7 of a chunk (a lane's B operand) from the chunk's
// word rows wq[i * QT + col]: the 1 - 3 words holding them, as a window
// with code j at bits B j.
template <int B>
__device__ inline uint64_t qt_window(const uint32_t* wq, int col, int kg) {
  constexpr int bit0 = 0;
  (void)bit0;
  const int bit = 8 * kg * B, w = bit >> 5, off = bit & 31;
  if constexpr (B == 4) {
    return wq[kg * QT + col];
  } else if constexpr (B == 8) {
    return (uint64_t)wq[(2 * kg) * QT + col] | ((uint64_t)wq[(2 * kg + 1) * QT + col] << 32);
  } else if constexpr (B == 2) {
    return wq[(kg >> 1) * QT + col] >> (16 * (kg & 1));
  } else {  // B == 3: 24 bits at bit 24 kg, in words w and w + 1 (w + 1 <= 2)
    const uint32_t lo = wq[w * QT + col];
    const uint32_t hi = w + 1 < 3 ? wq[(w + 1) * QT + col] : 0u;
    return ((((uint64_t)hi << 32) | lo) >> off);
  }
}

// The 8 weights s (q - z) of a lane, rounded as the 128 x 128 kernel rounds
// them ((q - z) sh + fl((q - z) sl) in one fused fp16 rounding), in k order.
// pm = pair_mask<B>() and pmagic = 0x64006400 live in registers (and_or).
template <int B>
__device__ inline half8_t qt_dequant8(uint64_t win, half2_t sh, half2_t sl, half2_t zz,
                                      uint32_t pm, uint32_t pmagic) {
  const uint32_t magic = pmagic;
  half2_t q[4];  // (1024 + code, 1024 + code) pairs
  if constexpr (B == 4 || B == 2) {
    // pairs (j, j + 4): one AND-OR each on the (for b = 2: doubled) window
    uint32_t v = (uint32_t)win;
    if constexpr (B == 2) v = (v & 0xFFFFu) | ((v & 0xFFFFu) << 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) q[j] = __builtin_bit_cast(half2_t, and_or(v >> (B * j), pm, pmagic));
  } else if constexpr (B == 8) {
    // pairs (j, j + 2) of each word
    const uint32_t w0 = (uint32_t)win, w1 = (uint32_t)(win >> 32);
    q[0] = __builtin_bit_cast(half2_t, and_or(w0, pm, pmagic));
    q[1] = __builtin_bit_cast(half2_t, and_or(w0 >> 8, pm, pmagic));
    q[2] = __builtin_bit_cast(half2_t, and_or(w1, pm, pmagic));
    q[3] = __builtin_bit_cast(half2_t, and_or(w1 >> 8, pm, pmagic));
  } else {  // B == 3: pairs (2j, 2j + 1)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t a = (uint32_t)(win >> (6 * j)) & 7u, b = (uint32_t)(win >> (6 * j + 3)) & 7u;
      q[j] = __builtin_bit_cast(half2_t, a | (b << 16) | magic);
    }
  }
  half2_t d[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const half2_t qz = q[j] - zz;
    d[j] = __builtin_elementwise_fma(qz, sh, qz * sl);
  }
  // k order
  if constexpr (B == 4 || B == 2) {  // d[j] = (k j, k j + 4)
    return (half8_t){d[0][0], d[1][0], d[2][0], d[3][0], d[0][1], d[1][1], d[2][1], d[3][1]};
  } else if constexpr (B == 8) {  // d[0] = (0, 2), d[1] = (1, 3), d[2] = (4, 6), d[3] = (5, 7)
    return (half8_t){d[0][0], d[1][0], d[0][1], d[1][1], d[2][0], d[3][0], d[2][1], d[3][1]};
  } else {
    return (half8_t){d[0][0], d[0][1], d[1][0], d[1][1], d[2][0], d[2][1], d[3][0], d[3][1]};
  }
}

template <int B>
__global__ void __launch_bounds__(512)
dq_tile_kernel(const _Float16* __restrict__ X, int64_t M, int64_t in, int64_t ldx,
               const uint32_t* __restrict__ qw, const float* __restrict__ scales,
               const int32_t* __restrict__ zeros, const int32_t* __restrict__ g_idx,
               const int32_t* __restrict__ cgroup, int64_t out, int64_t cps, int ntn, int ns,
               int64_t total, float* __restrict__ part, void* __restrict__ Y, int y_f16,
               int64_t ldy) {
  // One LDS object per ring slot: the stage's X tile, its weight words,
  // scale and zero rows, and the pad for the spare loads.  The compiler
  // tracks direct-to-LDS loads per object (up to eight), so with one object
  // per slot it can tell that the slot read is not the target of a load in
  // flight.
  constexpr int L = QT_L, K = qt_loads_per_wave<B>();
  constexpr int WOFF = QT_STAGE, PAD = QT_STAGE + (B + 2) * QT * 4;
  constexpr int SLOT = PAD;
  static_assert(L * SLOT <= 160 * 1024, "LDS");
  static_assert(16 + B + 2 <= 8 * K && 16 + B + 2 > 8 * (K - 1), "loads per stage");
  __shared__ __align__(16) char sl0[SLOT];
  __shared__ __align__(16) char sl1[SLOT];
  __shared__ __align__(16) char sl2[SLOT];
  __shared__ __align__(16) char sl3[SLOT];
  __shared__ __align__(16) char sl4[SLOT];
  __shared__ __align__(16) char sl5[SLOT];
  const int64_t per_xcd = (total + 7) / 8;
  const int64_t o = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (o >= total) return;
  const int tn = (int)(o % ntn);
  const int64_t rest = o / ntn;
  const int z = (int)(rest % ns);
  const int64_t tm = rest / ns;
  const int64_t m0 = tm * QT, n0 = (int64_t)tn * QT;
  const int64_t nch_all = in / DQ_CHUNK;
  const int64_t cb = (int64_t)z * cps;
  const int64_t ce = cb + cps < nch_all ? cb + cps : nch_all;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // 128-token half, 64-output quarter
  const int l32 = lane & 31, hi8 = lane >> 5;

  // ---- loads
  const int64_t rows = M - m0 < QT ? M - m0 : QT;
  const int64_t cols = out - n0 < QT ? out - n0 : QT;  // a multiple of 4
  uint32_t voff[2];  // X pieces wave and wave + 8
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = 16 * (wave + 8 * q) + (lane >> 2), pos = lane & 3;
    voff[q] = (uint32_t)(((int64_t)r * ldx + 8 * (pos ^ qt_swz(r))) * 2);
  }
  const uint32_t loff = (uint32_t)lane * 16;  // 4 columns of a word, scale or zero row
  // load t of a stage (wave w issues t = w + 8 j, j < K): X piece t (rows
  // 16 t .. 16 t + 15) for t < 16, then word row t - 16, then the scale and
  // the zero row, then pads
  auto issue = [&](int64_t c, int grp, char* sd) {
    const bool live = c < ce;
#pragma unroll
    for (int j = 0; j < K; ++j) {
      const int t = wave + 8 * j;  // wave-uniform
      const void* base = X;
      int bytes = 0;
      uint32_t vo = loff;
      int dst = PAD;
      if (j < 2) {  // t < 16 (wave < 8)
        vo = voff[j];
        dst = t * 1024;
        if (live) {
          base = X + m0 * ldx + c * DQ_CHUNK;
          bytes = (int)(((rows - 1) * ldx + (in - c * DQ_CHUNK)) * 2);
        }
      } else if (t < 16 + B) {
        dst = WOFF + (t - 16) * QT * 4;
        if (live) {
          base = qw + (c * B + (t - 16)) * out + n0;
          bytes = (int)(cols * 4);
        }
      } else if (t < 18 + B) {
        dst = WOFF + (t - 16) * QT * 4;
        if (live && grp >= 0) {
          base = t == 16 + B ? (const void*)(scales + grp * out + n0)
                             : (const void*)(zeros + grp * out + n0);
          bytes = (int)(cols * 4);
        }
      }
      if (t < 18 + B) {  // a pad when not (each costs as much as a real load)
        __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, 0x00020000);
        qt_dma(rs, vo, sd + dst);
      }
    }
  };
  // the loads of stage s + 1 have landed: L - 2 stages were issued after
  // them, K or K - 1 loads each (waves whose last load would be a pad)
  const bool full = wave + 8 * (K - 1) < 18 + B;
  auto wait_next = [&]() {
    if (full)
      wait_vmcnt<(L - 2) * K>();
    else
      wait_vmcnt<(L - 2) * (K - 1)>();
  };
  // the chunk's group (cgroup: one group, or -1), one scalar load
  auto group_of = [&](int64_t c) -> int {
    return __builtin_amdgcn_readfirstlane(cgroup[c < ce ? c : ce - 1]);
  };

  // ---- operands
  const int rsw = qt_swz(l32);
  const uint32_t pm = pair_mask<B>(), pmagic = 0x64006400u;
  struct AFr {
    half8_t a[4];
  };
  struct BFr {
    half8_t b[2];
  };
  struct Scl {
    half2_t sh[2], sl[2], zz[2];
  };
  auto load_a = [&](AFr& F, const char* xb, int sub) {
    const int cpos = ((2 * sub + hi8) ^ rsw) * 16;
#pragma unroll
    for (int a = 0; a < 4; ++a)
      F.a[a] = *reinterpret_cast<const half8_t*>(xb + (wm * 128 + a * 32 + l32) * 64 + cpos);
  };
  // column of block b of this lane (local), and its global index for the
  // per-weight path
  auto colb = [&](int b) { return wn * 64 + b * 32 + l32; };
  auto scales_of = [&](const char* wd, Scl& S) {
    const uint32_t* sz = reinterpret_cast<const uint32_t*>(wd) + B * QT;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const float s = __uint_as_float(sz[colb(b)]);
      const int32_t zi = (int32_t)sz[QT + colb(b)];
      const _Float16 hs = (_Float16)s, ls = (_Float16)(s - (float)hs);
      const _Float16 zh = (_Float16)(1024.0f + (float)zi);
      S.sh[b] = (half2_t){hs, hs};
      S.sl[b] = (half2_t){ls, ls};
      S.zz[b] = (half2_t){zh, zh};
    }
  };
  auto dequant_b = [&](BFr& F, const char* wd, const Scl& S, int sub) {
    const uint32_t* wq = reinterpret_cast<const uint32_t*>(wd);
#pragma unroll
    for (int b = 0; b < 2; ++b)
      F.b[b] = qt_dequant8<B>(qt_window<B>(wq, colb(b), 2 * sub + hi8), S.sh[b], S.sl[b], S.zz[b],
                              pm, pmagic);
  };
  // several groups in the chunk: scale and zero per weight from memory
  auto dequant_b_mixed = [&](BFr& F, const char* wd, int64_t c, int sub) {
    const uint32_t* wq = reinterpret_cast<const uint32_t*>(wd);
    const int kg = 2 * sub + hi8;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int64_t col = n0 + colb(b) < out ? n0 + colb(b) : out - 1;
      const uint64_t win = qt_window<B>(wq, colb(b), kg);
      half8_t r;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t g = g_idx[c * DQ_CHUNK + 8 * kg + j];
        const float s = scales[g * out + col];
        const _Float16 hs = (_Float16)s, ls = (_Float16)(s - (float)hs);
        const _Float16 qz = (_Float16)((float)((win >> (B * j)) & ((1u << B) - 1u)) -
                                       (float)zeros[g * out + col]);
        r[j] = __builtin_elementwise_fma(qz, hs, qz * ls);
      }
      F.b[b] = r;
    }
    wait_vmcnt<0>();  // this path's own loads (the compiler's waits assume none in flight)
  };
  f32x16_t acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
  auto mma = [&](const AFr& A, const BFr& Bf) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A.a[a], Bf.b[b], acc[a][b], 0, 0, 0);
  };
  // interleave: the substep's VALU work between its 8 MFMAs
  auto interleave = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // LDS reads first
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // six VALU
    }
  };

  // ---- prologue: loads of stages cb .. cb + L - 1 issued, stage cb's
  // landed and its first substep operands ready
  int g0 = group_of(cb), g1 = group_of(cb + 1), g2 = group_of(cb + 2);
  int g3 = group_of(cb + 3), g4 = group_of(cb + 4), g5 = group_of(cb + 5);
  issue(cb + 0, g0, sl0);
  issue(cb + 1, g1, sl1);
  issue(cb + 2, g2, sl2);
  issue(cb + 3, g3, sl3);
  issue(cb + 4, g4, sl4);
  issue(cb + 5, g5, sl5);
  wait_vmcnt<(L - 1) * K>();  // stage cb landed; the rest stays in flight
  __builtin_amdgcn_s_barrier();
  AFr A0, A1;
  BFr B0, B1;
  Scl S;
  load_a(A0, sl0, 0);
  scales_of(sl0 + WOFF, S);
  dequant_b(B0, sl0 + WOFF, S, 0);
  if (g0 < 0) dequant_b_mixed(B0, sl0 + WOFF, cb, 0);

  // Stage c in slot xc (group gcur), the next stage in slot xn (group
  // gnxt); gi: group of stage c + L, whose loads go to slot xc at the
  // middle of stage c.
  int64_t c = cb;
  auto step = [&](char* xc, int gcur, char* xn, int gnxt, int gi)
      __attribute__((always_inline)) {
    const char* wcs = xc + WOFF;
    const char* wns = xn + WOFF;
    // substep 0: MFMAs on A0/B0 while substep 1's operands are formed
    load_a(A1, xc, 1);
    mma(A0, B0);
    dequant_b(B1, wcs, S, 1);
    interleave();
    if (gcur < 0) dequant_b_mixed(B1, wcs, c, 1);
    // stage c + 1 landed and visible; stage c's slot free after the barrier
    wait_next();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    issue(c + L, gi, xc);
    // substep 1: MFMAs on A1/B1 while stage c + 1's first operands are formed
    load_a(A0, xn, 0);
    scales_of(wns, S);
    mma(A1, B1);
    dequant_b(B0, wns, S, 0);
    interleave();
    if (gnxt < 0 && c + 1 < ce) dequant_b_mixed(B0, wns, c + 1, 0);
    ++c;
  };
  // g0 .. g(L-1): groups of stages c .. c + L - 1.  Whole rounds of L
  // stages run in a loop with one exit, the rest one stage at a time after
  // it: with an exit after every stage the compiler loses track of the
  // loads in flight at the loop head and waits for all of them there.
  int gn;
#define GPTQ_QT_STEP(XC, XN)                             \
  gn = group_of(c + L);                                 \
  step(XC, g0, XN, g1, gn);                             \
  g0 = g1; g1 = g2; g2 = g3; g3 = g4; g4 = g5; g5 = gn;
  while (c + 6 <= ce) {
    GPTQ_QT_STEP(sl0, sl1)
    GPTQ_QT_STEP(sl1, sl2)
    GPTQ_QT_STEP(sl2, sl3)
    GPTQ_QT_STEP(sl3, sl4)
    GPTQ_QT_STEP(sl4, sl5)
    GPTQ_QT_STEP(sl5, sl0)
  }
  if (c < ce) { GPTQ_QT_STEP(sl0, sl1) }
  if (c < ce) { GPTQ_QT_STEP(sl1, sl2) }
  if (c < ce) { GPTQ_QT_STEP(sl2, sl3) }
  if (c < ce) { GPTQ_QT_STEP(sl3, sl4) }
  if (c < ce) { GPTQ_QT_STEP(sl4, sl5) }
#undef GPTQ_QT_STEP
  wait_vmcnt<0>();  // no load may land in LDS after the workgroup ends
  wait_lgkm0();

  // 32 x 32 block layout: element v of lane l is row 8 (v / 4) + 4 (l / 32) + v % 4,
  // column l % 32
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t r = m0 + wm * 128 + a * 32 + 8 * (v >> 2) + 4 * hi8 + (v & 3);
        const int64_t cc = n0 + colb(b);
        if (r < M && cc < out) {
          if (ns > 1)
            part[((int64_t)z * M + r) * out + cc] = acc[a][b][v];
          else if (y_f16)
            static_cast<_Float16*>(Y)[r * ldy + cc] = (_Float16)acc[a][b][v];
          else
            static_cast<float*>(Y)[r * ldy + cc] = acc[a][b][v];
        }
      }
}

// Splits of the input range: about 512 workgroups for the 128 x 128 kernel
// (two per compute unit), 256 for the 256 x 256 one (one per compute unit),
// each split at least 8 chunks.  The 256 x 256 tiles take 256 tokens on.
constexpr int64_t QT_MIN_M = 256;
int64_t mfma_chunks_per_split(int64_t M, int64_t in, int64_t out, bool big) {
  const int64_t nch = in / DQ_CHUNK;
  const int64_t tm = big ? QT : 128, tn = big ? QT : TN, want = big ? 256 : 512;
  const int64_t tiles = ((out + tn - 1) / tn) * ((M + tm - 1) / tm);
  int64_t ns = (want + tiles - 1) / tiles;
  if (ns > nch / 8) ns = nch / 8;
  if (ns < 1) ns = 1;
  return (nch + ns - 1) / ns;
}
size_t mfma_partial_bytes(int64_t M, int64_t in, int64_t out, bool big) {
  const int64_t cps = mfma_chunks_per_split(M, in, out, big);
  const int64_t ns = (in / DQ_CHUNK + cps - 1) / cps;
  return ns > 1 ? align_up((size_t)ns * M * out * sizeof(float)) : 0;
}

// ------------------------------------------------------------ group order --
// Xp[m][p] = X[m][x_order[p]] (the matrix-core path's X in packed order).
// A workgroup copies rows m0 .. m0 + R - 1 of X into LDS with 16-byte loads
// (R in <= 32768 halves), then each thread takes 8 consecutive positions p:
// one read of their x_order entries serves every staged row, and the 8
// gathered values leave as one 16-byte store per row.  (A thread per
// position and row read 2 bytes from scattered columns: 1.4 TB/s.)
constexpr int64_t GATHER_LDS_HALVES = 32768;
constexpr int64_t GATHER_MAX_IN = 65536;  // one 128 KiB row; wider: a thread per column
int gather_rows(int64_t in) {
  const int64_t r = GATHER_LDS_HALVES / in;
  return (int)(r >= 8 ? 8 : r < 1 ? 1 : r);
}
__global__ void __launch_bounds__(256)
dq_gather_x_kernel(const _Float16* __restrict__ X, int64_t M, int64_t in, int64_t ldx,
                   const int32_t* __restrict__ x_order, int R, _Float16* __restrict__ Xp) {
  extern __shared__ __align__(16) _Float16 xrows[];  // [R][in]
  const int64_t m0 = (int64_t)blockIdx.x * R;
  const int nr = M - m0 < R ? (int)(M - m0) : R;
  for (int r = 0; r < nr; ++r)
    for (int64_t c = (int64_t)threadIdx.x * 8; c < in; c += 256 * 8)
      *reinterpret_cast<uint4*>(&xrows[r * in + c]) =
          *reinterpret_cast<const uint4*>(X + (m0 + r) * ldx + c);
  __syncthreads();
  for (int64_t p = (int64_t)threadIdx.x * 8; p < in; p += 256 * 8) {
    int idx[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) idx[j] = x_order[p + j];
    for (int r = 0; r < nr; ++r) {
      const _Float16* row = xrows + r * in;
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = (uint32_t)__builtin_bit_cast(uint16_t, row[idx[2 * j]]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, row[idx[2 * j + 1]]) << 16);
      *reinterpret_cast<uint4*>(Xp + (m0 + r) * in + p) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}
// Rows longer than GATHER_MAX_IN: one thread per position, rows strided.
__global__ void __launch_bounds__(256)
dq_gather_x_cols_kernel(const _Float16* __restrict__ X, int64_t M, int64_t in, int64_t ldx,
                        const int32_t* __restrict__ x_order, _Float16* __restrict__ Xp) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p >= in) return;
  const int64_t k = x_order[p];
  for (int64_t m = blockIdx.y; m < M; m += gridDim.y) Xp[m * in + p] = X[m * ldx + k];
}

// keys[k] = ~g_idx[k]: decreasing key = increasing group.
__global__ void dq_group_keys_kernel(const int32_t* __restrict__ g_idx, int64_t in,
                                     uint32_t* __restrict__ keys) {
  const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (k < in) keys[k] = ~(uint32_t)g_idx[k];
}

__global__ void dq_gather_i32_kernel(const int32_t* __restrict__ src,
                                     const int32_t* __restrict__ idx, int64_t n,
                                     int32_t* __restrict__ dst) {
  const int64_t p = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (p < n) dst[p] = src[idx[p]];
}

// qs: column col's codes in x_order, re-packed.  Grid (ceil(out / 256), in / 32):
// thread = one column, one chunk of 32 sorted positions (= B output words).
template <int B>
__global__ void __launch_bounds__(256)
dq_repack_kernel(const uint32_t* __restrict__ qw, const int32_t* __restrict__ x_order,
                 int64_t out, uint32_t* __restrict__ qs) {
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (col >= out) return;
  const int64_t c = blockIdx.y;
  uint32_t w[B + 1];
#pragma unroll
  for (int i = 0; i <= B; ++i) w[i] = 0u;
#pragma unroll
  for (int j = 0; j < DQ_CHUNK; ++j) {
    const int64_t bit = (int64_t)x_order[c * DQ_CHUNK + j] * B;
    const int64_t wi = bit >> 5;
    const int off = (int)(bit & 31);
    uint32_t v = qw[wi * out + col] >> off;
    if (off + B > 32) v |= qw[(wi + 1) * out + col] << (32 - off);
    v &= (1u << B) - 1u;
    const int pos = j * B, pw = pos >> 5, po = pos & 31;
    w[pw] |= v << po;
    if (po + B > 32) w[pw + 1] |= v >> (32 - po);
  }
#pragma unroll
  for (int i = 0; i < B; ++i) qs[(c * B + i) * out + col] = w[i];
}

// ------------------------------------------------------------------- plan --
struct SmallPlan {
  int mb;        // token rows per lane
  int cpl;       // columns per lane
  int64_t cps;   // chunks per split
  int nsplit;
  size_t lds;    // bytes
};
// cpl 4 needs out % 4 == 0 and 16-byte aligned qweight, scales and zeros;
// it is taken for up to 4 token rows.
SmallPlan small_plan(int64_t M, int64_t in, int64_t out, int cpl) {
  SmallPlan p;
  p.mb = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : 8;
  p.cpl = cpl;
  const int64_t nch = in / DQ_CHUNK;
  const int64_t cols = 64 * (int64_t)cpl;
  const int64_t ncolwg = (out + cols - 1) / cols;
  // about 512 workgroups, each wave at least two blocks of chunks (cpl 1)
  // or two chunks (cpl 4), X slice and the final reduction within LDS
  int64_t ns = (512 + ncolwg - 1) / ncolwg;
  const int64_t ns_max = cpl == 1 ? nch / (8 * SMALL_DEPTH) : nch / 8;
  if (ns > ns_max) ns = ns_max;
  if (ns < 1) ns = 1;
  int64_t cps = (nch + ns - 1) / ns;
  const int64_t cps_max = SMALL_LDS_MAX / (((int64_t)p.mb * 16 + 1) * 4);
  if (cps > cps_max) cps = cps_max;
  p.cps = cps;
  p.nsplit = (int)((nch + cps - 1) / cps);
  const size_t xsb = ((size_t)p.mb * cps * 16 + cps) * 4;
  const size_t redb = (size_t)4 * p.mb * cols * 4;
  p.lds = xsb > redb ? xsb : redb;
  return p;
}
bool cpl4_ok(int64_t M, int64_t out) { return M <= 4 && out % 4 == 0; }

template <int B, int MB, int CPL>
hipError_t launch_small_t(const SmallPlan& p, const _Float16* X, int64_t M, int64_t in,
                          int64_t ldx, const uint32_t* qw, const float* scales,
                          const int32_t* zeros, const int32_t* g_idx, const int32_t* xo,
                          int64_t out, float* part, void* Y, int y_f16, int64_t ldy,
                          hipStream_t s) {
  auto k = dq_small_kernel<B, MB, CPL>;
  GPTQ_HIP_TRY(hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)p.lds));
  dim3 grid((unsigned)((out + 64 * CPL - 1) / (64 * CPL)), (unsigned)p.nsplit);
  hipLaunchKernelGGL(k, grid, dim3(256), p.lds, s, X, M, in, ldx, qw, scales, zeros, g_idx, xo,
                     out, p.cps, part, Y, y_f16, ldy);
  return hipGetLastError();
}
template <int B>
hipError_t launch_small_b(const SmallPlan& p, const _Float16* X, int64_t M, int64_t in,
                          int64_t ldx, const uint32_t* qw, const float* scales,
                          const int32_t* zeros, const int32_t* g_idx, const int32_t* xo,
                          int64_t out, float* part, void* Y, int y_f16, int64_t ldy,
                          hipStream_t s) {
  if (p.cpl == 4) {
    switch (p.mb) {
      case 1: return launch_small_t<B, 1, 4>(p, X, M, in, ldx, qw, scales, zeros, g_idx, xo, out, part, Y, y_f16, ldy, s);
      case 2: return launch_small_t<B, 2, 4>(p, X, M, in, ldx, qw, scales, zeros, g_idx, xo, out, part, Y, y_f16, ldy, s);
      default: return launch_small_t<B, 4, 4>(p, X, M, in, ldx, qw, scales, zeros, g_idx, xo, out, part, Y, y_f16, ldy, s);
    }
  }
  switch (p.mb) {
    case 1: return launch_small_t<B, 1, 1>(p, X, M, in, ldx, qw, scales, zeros, g_idx, xo, out, part, Y, y_f16, ldy, s);
    case 2: return launch_small_t<B, 2, 1>(p, X, M, in, ldx, qw, scales, zeros, g_idx, xo, out, part, Y, y_f16, ldy, s);
    case 4: return launch_small_t<B, 4, 1>(p, X, M, in, ldx, qw, scales, zeros, g_idx, xo, out, part, Y, y_f16, ldy, s);
    default: return launch_small_t<B, 8, 1>(p, X, M, in, ldx, qw, scales, zeros, g_idx, xo, out, part, Y, y_f16, ldy, s);
  }
}

}  // namespace

size_t dequant_matmul_workspace_bytes(int64_t M, int64_t in, int64_t out, int has_order) {
  if (M > DQ_SMALL_M_MAX) {
    // [gathered X when has_order][split partials when more than one split];
    // from 256 tokens either tile kernel may run (alignment decides): the
    // larger need
    size_t parts = mfma_partial_bytes(M, in, out, false);
    if (M >= QT_MIN_M && out % 4 == 0) {  // + the chunk group table
      const size_t b = align_up((size_t)(in / DQ_CHUNK) * sizeof(int32_t)) +
                       mfma_partial_bytes(M, in, out, true);
      parts = b > parts ? b : parts;
    }
    return (has_order ? align_up((size_t)M * in * sizeof(_Float16)) : 0) + parts;
  }
  // either column layout may run (alignment decides): the larger need
  size_t need = 0;
  for (int cpl = 1; cpl <= (cpl4_ok(M, out) ? 4 : 1); cpl += 3) {
    const SmallPlan p = small_plan(M, in, out, cpl);
    if (p.nsplit > 1) {
      const size_t b = align_up((size_t)p.nsplit * M * out * sizeof(float));
      need = b > need ? b : need;
    }
  }
  return need;
}

hipError_t run_dequant_matmul(const void* X, int64_t M, int64_t in, int64_t ldx,
                              const int32_t* qweight, const float* scales, const int32_t* zeros,
                              const int32_t* g_idx, const int32_t* x_order, int64_t out, int bits,
                              void* Y, int y_f16, int64_t ldy, void* ws, size_t ws_bytes,
                              hipStream_t s) {
  const _Float16* x = static_cast<const _Float16*>(X);
  const uint32_t* qw = reinterpret_cast<const uint32_t*>(qweight);
  const int32_t* xo = x_order;
  if (M <= DQ_SMALL_M_MAX) {
    const bool aligned = ((reinterpret_cast<uintptr_t>(qweight) | reinterpret_cast<uintptr_t>(scales) |
                           reinterpret_cast<uintptr_t>(zeros)) & 15) == 0;
    const SmallPlan p = small_plan(M, in, out, cpl4_ok(M, out) && aligned ? 4 : 1);
    float* part = static_cast<float*>(ws);
    hipError_t e;
    switch (bits) {
      case 2: e = launch_small_b<2>(p, x, M, in, ldx, qw, scales, zeros, g_idx, xo, out, part, Y, y_f16, ldy, s); break;
      case 3: e = launch_small_b<3>(p, x, M, in, ldx, qw, scales, zeros, g_idx, xo, out, part, Y, y_f16, ldy, s); break;
      case 8: e = launch_small_b<8>(p, x, M, in, ldx, qw, scales, zeros, g_idx, xo, out, part, Y, y_f16, ldy, s); break;
      default: e = launch_small_b<4>(p, x, M, in, ldx, qw, scales, zeros, g_idx, xo, out, part, Y, y_f16, ldy, s); break;
    }
    GPTQ_HIP_TRY(e);
    if (p.nsplit > 1) {
      const int64_t total = M * out;
      hipLaunchKernelGGL(dq_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                         part, p.nsplit, M, out, Y, y_f16, ldy);
      GPTQ_HIP_TRY(hipGetLastError());
    }
    return hipSuccess;
  }
  if (ws_bytes < dequant_matmul_workspace_bytes(M, in, out, xo ? 1 : 0)) return hipErrorInvalidValue;
  char* wsp = static_cast<char*>(ws);
  if (xo) {
    // X in packed order into the workspace, then the plain product on it
    _Float16* xp = reinterpret_cast<_Float16*>(wsp);
    if (in <= GATHER_MAX_IN) {
      const int R = gather_rows(in);
      const size_t lds = (size_t)R * in * sizeof(_Float16);
      if (lds > 64 * 1024)
        GPTQ_HIP_TRY(hipFuncSetAttribute((const void*)dq_gather_x_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
      hipLaunchKernelGGL(dq_gather_x_kernel, dim3((unsigned)((M + R - 1) / R)), dim3(256), lds, s,
                         x, M, in, ldx, xo, R, xp);
    } else {
      hipLaunchKernelGGL(dq_gather_x_cols_kernel, dim3((unsigned)((in + 255) / 256),
                         (unsigned)(M < 1024 ? M : 1024)), dim3(256), 0, s, x, M, in, ldx, xo, xp);
    }
    GPTQ_HIP_TRY(hipGetLastError());
    x = xp;
    ldx = in;
    wsp += align_up((size_t)M * in * sizeof(_Float16));
  }
  const bool big = M >= QT_MIN_M && out % 4 == 0 &&
                   ((reinterpret_cast<uintptr_t>(qweight) | reinterpret_cast<uintptr_t>(scales) |
                     reinterpret_cast<uintptr_t>(zeros)) & 15) == 0;
  const int64_t cps = mfma_chunks_per_split(M, in, out, big);
  const int64_t ns = (in / DQ_CHUNK + cps - 1) / cps;
  float* part = ns > 1 ? reinterpret_cast<float*>(wsp) : nullptr;
  if (big) {
    int32_t* cgroup = reinterpret_cast<int32_t*>(wsp);
    const int64_t nch = in / DQ_CHUNK;
    part = ns > 1 ? reinterpret_cast<float*>(wsp + align_up((size_t)nch * sizeof(int32_t))) : nullptr;
    hipLaunchKernelGGL(dq_chunk_group_kernel, dim3((unsigned)((nch + 255) / 256)), dim3(256), 0, s,
                       g_idx, nch, cgroup);
    GPTQ_HIP_TRY(hipGetLastError());
    const int64_t ntn = (out + QT - 1) / QT, total = ((M + QT - 1) / QT) * ns * ntn;
    const dim3 grid((unsigned)(8 * ((total + 7) / 8)));
#define GPTQ_DQ_TILE(BB)                                                                     \
  hipLaunchKernelGGL((dq_tile_kernel<BB>), grid, dim3(512), 0, s, x, M, in, ldx, qw, scales, \
                     zeros, g_idx, cgroup, out, cps, (int)ntn, (int)ns, total, part, Y, y_f16,  \
                     ldy)
    switch (bits) {
      case 2: GPTQ_DQ_TILE(2); break;
      case 3: GPTQ_DQ_TILE(3); break;
      case 8: GPTQ_DQ_TILE(8); break;
      default: GPTQ_DQ_TILE(4); break;
    }
#undef GPTQ_DQ_TILE
  } else {
    dim3 grid((unsigned)((out + TN - 1) / TN), (unsigned)((M + 127) / 128), (unsigned)ns);
#define GPTQ_DQ_MFMA(BB)                                                                     \
  hipLaunchKernelGGL((dq_mfma_kernel<BB, 128>), grid, dim3(512), 0, s, x, M, in, ldx, qw,    \
                     scales, zeros, g_idx, out, cps, part, Y, y_f16, ldy)
    switch (bits) {
      case 2: GPTQ_DQ_MFMA(2); break;
      case 3: GPTQ_DQ_MFMA(3); break;
      case 8: GPTQ_DQ_MFMA(8); break;
      default: GPTQ_DQ_MFMA(4); break;
    }
  }
#undef GPTQ_DQ_MFMA
  GPTQ_HIP_TRY(hipGetLastError());
  if (ns > 1) {
    const int64_t total = M * out;
    hipLaunchKernelGGL(dq_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       part, (int)ns, M, out, Y, y_f16, ldy);
    GPTQ_HIP_TRY(hipGetLastError());
  }
  return hipSuccess;
}

size_t dequant_group_order_workspace_bytes(int64_t in) {
  return 2 * align_up((size_t)in * sizeof(int32_t));
}

hipError_t run_dequant_group_order(const int32_t* qweight, const int32_t* g_idx, int64_t in,
                                   int64_t out, int bits, int32_t* qweight_sorted,
                                   int32_t* g_idx_sorted, int32_t* x_order, void* ws,
                                   hipStream_t s) {
  uint32_t* keys = static_cast<uint32_t*>(ws);
  int32_t* rank = reinterpret_cast<int32_t*>(static_cast<char*>(ws) +
                                             align_up((size_t)in * sizeof(int32_t)));
  const unsigned nb = (unsigned)((in + 255) / 256);
  hipLaunchKernelGGL(dq_group_keys_kernel, dim3(nb), dim3(256), 0, s, g_idx, in, keys);
  GPTQ_HIP_TRY(hipGetLastError());
  GPTQ_HIP_TRY(launch_stable_order_desc(keys, in, rank, x_order, s));
  hipLaunchKernelGGL(dq_gather_i32_kernel, dim3(nb), dim3(256), 0, s, g_idx, x_order, in,
                     g_idx_sorted);
  GPTQ_HIP_TRY(hipGetLastError());
  const uint32_t* qw = reinterpret_cast<const uint32_t*>(qweight);
  uint32_t* qs = reinterpret_cast<uint32_t*>(qweight_sorted);
  dim3 grid((unsigned)((out + 255) / 256), (unsigned)(in / DQ_CHUNK));
  switch (bits) {
    case 2: hipLaunchKernelGGL(dq_repack_kernel<2>, grid, dim3(256), 0, s, qw, x_order, out, qs); break;
    case 3: hipLaunchKernelGGL(dq_repack_kernel<3>, grid, dim3(256), 0, s, qw, x_order, out, qs); break;
    case 8: hipLaunchKernelGGL(dq_repack_kernel<8>, grid, dim3(256), 0, s, qw, x_order, out, qs); break;
    default: hipLaunchKernelGGL(dq_repack_kernel<4>, grid, dim3(256), 0, s, qw, x_order, out, qs); break;
  }
  return hipGetLastError();
}

}  // namespace gptq
