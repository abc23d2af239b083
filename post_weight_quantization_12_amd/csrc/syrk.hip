// Hessian accumulation H(upper) += 2 X^T X on the gfx950 matrix cores.
//
// The Hessian of the layer reconstruction loss with respect to the layer's
// weights is 2 * sum_t x_t x_t^T over calibration tokens (glossary entry
// "gptq", "Algorithm" step (1)).  X arrives tokens x features, row-major, so
// both MFMA operands are column panels of X: the contraction runs over tokens,
// which are the strided dimension in memory.
//
// Main kernel (syrk_dma_kernel, rows 16-byte aligned): 256 x 256 output tiles
// of the upper triangle; 32-token stages of the two column panels are copied
// straight from memory into LDS (buffer_load ... lds, five stages in flight)
// and read transposed into MFMA operands (ds_read_b64_tr_b16);
// v_mfma_f32_32x32x16_{f16,bf16} (products exact in fp32, fp32 accumulation).
// Three schedules, chosen per call:
//   * whole tiles, one launch per 32768 tokens, when the tiles fill the
//     workgroup rounds (n = 11008: 990 tiles, 3.9 rounds of 256);
//   * token split (a workspace, long calls, few tiles): every XCD works on
//     its own block of tokens, tiles round by round, partial tiles summed by
//     a second kernel;
//   * stream-K (a workspace, short calls, few tiles): equal runs of (tile,
//     stage) units, split tiles summed by a second kernel.
// Rows that are not 16-byte aligned use syrk_upper_kernel: each thread
// gathers an 8-token x 8-feature block (element loads), transposes it in
// registers and stores feature-major rows into LDS (64-token stages, double
// buffered), from which every MFMA operand is one ds_read_b128.
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

// ---------------------------------------------------------------------------
// Main path: direct-to-LDS loads + transposing LDS reads (gfx950).
//
// X panels stay in their natural token-major layout.  Each 16-byte chunk (8
// features of one token) is copied straight from HBM into LDS by
// buffer_load ... lds (no VGPR staging), 5 stages deep (the whole 160 KiB LDS),
// so ~4 stages of loads are in flight while one is consumed.  A stage holds 32 tokens x 256 features
// of each operand panel; chunk (t, c) is stored at physical slot
// t*32 + (c ^ 4*(t%4)) so that the transposing reads below hit 16 distinct
// bank groups per 32-lane pass.
//
// MFMA operands come from ds_read_b64_tr_b16: within a 16-lane group, lane j
// receives element j%4 of the 8-byte reads issued by lanes j/4 + 4i (i<4).
// Lane L pointing at (token t0 + L/4, features f0 + 4*(L%4)) therefore gets
// feature f0 + L at tokens t0..t0+3 -- one k-slot quarter of an A/B fragment.
// Out-of-range tokens read as 0 through the buffer descriptor's size check.
// Waves split the 256 x 256 tile into 64 x 128 or 128 x 128 blocks (SyrkShape).
constexpr int DT = 256, DBK = 32, DS = 5;
constexpr int PANEL_BYTES = DBK * DT * 2;       // 16 KiB
constexpr int STAGE_BYTES = 2 * PANEL_BYTES;    // A + B
typedef short v4i16_t __attribute__((ext_vector_type(4)));

__device__ inline v4i16_t ds_read_tr16(const char* lds_byte_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (v4i16_t __attribute__((address_space(3)))*)(
          (__attribute__((address_space(3))) char*)(lds_byte_ptr)));
}

template <bool BF16>
__device__ inline f32x16_t mfma_tr(v4i16_t lo, v4i16_t hi, v4i16_t blo, v4i16_t bhi, f32x16_t c) {
  typedef short v8i16_t __attribute__((ext_vector_type(8)));
  v8i16_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  v8i16_t b = __builtin_shufflevector(blo, bhi, 0, 1, 2, 3, 4, 5, 6, 7);
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
}

// Tile order for the upper triangle (ti <= tj), L2-aware.  Workgroups are
// dispatched to the 8 XCDs round-robin (block b -> XCD b % 8) and each XCD has
// its own L2, so block b takes logical tile (b % 8) * per_xcd + b / 8: every
// XCD walks its own contiguous run of the logical order.  The logical order
// visits row groups of G tile rows; inside a group it goes column by column,
// so the ~32 tiles one XCD runs at a time share G row panels and a few
// column panels, and those panels are read from HBM once per XCD.
constexpr int TILE_GROUP = 8;
// Logical tile o (< nt(nt+1)/2) of the grouped order -> (ti, tj).
__device__ inline void tile_of(int64_t o, int nt, int& ti, int& tj) {
  ti = tj = 0;
  for (int g0 = 0; g0 < nt; g0 += TILE_GROUP) {
    const int gsz = nt - g0 < TILE_GROUP ? nt - g0 : TILE_GROUP;
    const int64_t tri = (int64_t)gsz * (gsz + 1) / 2;
    const int64_t cnt = tri + (int64_t)gsz * (nt - g0 - gsz);
    if (o < cnt) {
      if (o < tri) {  // triangle: column g0 + d holds d + 1 tiles
        int d = 0;
        while ((int64_t)(d + 1) * (d + 2) / 2 <= o) ++d;
        tj = g0 + d;
        ti = g0 + (int)(o - (int64_t)d * (d + 1) / 2);
      } else {
        const int64_t r = o - tri;
        tj = g0 + gsz + (int)(r / gsz);
        ti = g0 + (int)(r % gsz);
      }
      return;
    }
    o -= cnt;
  }
}
__device__ inline bool syrk_tile(int b, int nt, int& ti, int& tj) {
  const int64_t total = (int64_t)nt * (nt + 1) / 2;
  const int64_t per_xcd = (total + 7) / 8;
  const int64_t o = (int64_t)(b % 8) * per_xcd + b / 8;
  if (o >= total) return false;
  tile_of(o, nt, ti, tj);
  ti = __builtin_amdgcn_readfirstlane(ti);  // uniform: keeps tile addressing in SGPRs
  tj = __builtin_amdgcn_readfirstlane(tj);
  return true;
}

// Stream-K bookkeeping (used when the tiles alone cannot fill the chip): the
// (tile, 32-token stage) units are cut into nwg equal contiguous runs, one per
// workgroup.  units <= nk, so a run touches at most two tiles.  A tile done
// whole by one run is added to H directly; a tile split between runs leaves
// one partial 256 x 256 accumulator per contributor in the workspace (slot 0
// if the run starts in that tile, slot 1 if it ends there), and a second
// kernel adds them to H in run order, so the sum order, and the result, do
// not depend on timing.
struct StreamK {
  float* partial;   // [nwg][2][256 * 256], row-major tiles
  int64_t units;    // units per workgroup
  int nwg;          // workgroups (a multiple of 8)
  int ks;           // > 0: token-split schedule with ks token blocks (below)
};
constexpr int PART_FLOATS = DT * DT;

// Token-split schedule.  The tokens are cut into S blocks (S = 1, 2, 4, 8);
// XCD x works on block x % S, and the tiles are divided evenly among the
// 8 / S XCDs that share a block.  Inside an XCD the C workgroups take the
// XCD's tiles round by round, all over the same token range, so the ~C tiles
// of a round read the same token rows together and share them in the XCD's
// L2.  The tiles left after the whole rounds are cut along the tokens into
// s = C / r pieces each, so the last round is as long as the others divided
// by s and no workgroup idles.  Every (tile, block, piece) item leaves one
// partial; a second kernel adds a tile's partials to H in a fixed order.
struct KsXcd {
  int64_t t0, tn;   // tiles [t0, t0 + tn) of the grouped order
  int64_t base;     // first partial slot of this XCD
  int64_t items;    // q * C + r * s
  int q, r, sp;     // whole rounds, tiles left, pieces per tile left
};
__host__ __device__ inline KsXcd ks_xcd(int x, int S, int C, int64_t T) {
  const int G = 8 / S;
  KsXcd k{0, 0, 0, 0, 0, 0, 0};
  for (int y = 0; y <= x; ++y) {
    const int g = y / S;
    const int64_t t0 = T * g / G, t1 = T * (g + 1) / G, tn = t1 - t0;
    const int q = (int)(tn / C), r = (int)(tn % C), sp = r > 0 ? C / r : 0;
    const int64_t items = (int64_t)q * C + (int64_t)r * sp;
    if (y == x) {
      k.t0 = t0; k.tn = tn; k.q = q; k.r = r; k.sp = sp; k.items = items;
    } else {
      k.base += items;
    }
  }
  return k;
}
// Token stages [k0, k1) of item i of an XCD on block b; tile o (grouped order).
__device__ inline void ks_item(const KsXcd& k, int64_t i, int b, int S, int C, int nk,
                               int64_t& o, int& k0, int& k1) {
  const int bk = (nk + S - 1) / S;
  const int lo = b * bk < nk ? b * bk : nk, hi = (b + 1) * bk < nk ? (b + 1) * bk : nk;
  const int64_t whole = (int64_t)k.q * C;
  if (i < whole) {
    o = k.t0 + i;
    k0 = lo;
    k1 = hi;
  } else {
    const int64_t j = i - whole;
    const int p = (int)(j % k.sp);
    o = k.t0 + whole + j / k.sp;
    const int len = hi - lo;
    k0 = lo + (int)((int64_t)len * p / k.sp);
    k1 = lo + (int)((int64_t)len * (p + 1) / k.sp);
  }
}

// Waves per workgroup: 8, two per SIMD, each a 64 x 128 block (8
// accumulators): the second wave on a SIMD keeps its matrix pipe busy while
// the first waits at a barrier or on LDS (6-7 % faster on whole tiles than
// one 128 x 128 wave per SIMD, 11 % under stream-K at n = 4096).
template <bool STREAMK>
struct SyrkShape {
  static constexpr int NW = 8;                    // waves
  static constexpr int WM = NW / 2;               // row blocks
  static constexpr int FA = DT / WM / 32;         // 32-row A fragments per wave
  static constexpr int FB = 4;                    // 32-column B fragments per wave
  static constexpr int DMA = 2 * DT * DBK * 2 / 16 / 64 / NW;  // 16-byte loads per wave per stage
};

// One substep's MFMAs (8 per wave) with the other substep's 12 transposing
// LDS reads spread between them: two reads after each of the first six
// MFMAs, the last two MFMAs alone (so the reads have landed before the
// barrier that follows; 1-3 % faster than reads spread over all eight).
// A macro: the scheduling builtins need literal group ids.
#define GPTQ_SYRK_INTERLEAVE(FA, ID)                                  \
  do {                                                                \
    static_assert((FA) == 2, "schedule written for 64 x 128 blocks"); \
    _Pragma("unroll") for (int i_ = 0; i_ < 6; ++i_) {                \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, ID);             \
      __builtin_amdgcn_sched_group_barrier(0x100, 2, ID);             \
    }                                                                 \
    _Pragma("unroll") for (int i_ = 0; i_ < 2; ++i_) {                \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, ID);             \
    }                                                                 \
  } while (0)

template <bool BF16, bool STREAMK>
__global__ void __launch_bounds__(SyrkShape<STREAMK>::NW * 64)
syrk_dma_kernel(float* __restrict__ H, int64_t n, const uint16_t* __restrict__ X, int64_t ntok,
                int64_t ldx, StreamK sk) {
  // One LDS object per stage: the compiler then tracks each stage's direct
  // loads separately and only waits for the stage being read.
  __shared__ __align__(16) char st0[STAGE_BYTES];
  __shared__ __align__(16) char st1[STAGE_BYTES];
  __shared__ __align__(16) char st2[STAGE_BYTES];
  __shared__ __align__(16) char st3[STAGE_BYTES];
  __shared__ __align__(16) char st4[STAGE_BYTES];
  static_assert(DS == 5, "five stage buffers (160 KiB, the whole LDS)");

  const int nt = (int)((n + DT - 1) / DT);
  const int nk = (int)((ntok + DBK - 1) / DBK);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  using SS = SyrkShape<STREAMK>;
  constexpr int FA = SS::FA, FB = SS::FB, DMA_PER_WAVE = SS::DMA, RW = DT / SS::WM;
  static_assert(FA == 2 && FB == 4 && DMA_PER_WAVE == 4, "array sizes below");
  const int wm = wave % SS::WM, wn = wave / SS::WM;

  // Transposing-read byte offsets within a panel, per lane (substep 0, first 4 tokens).
  const int g = lane >> 4, L = lane & 15;
  const int trow = 8 * (g >> 1) + (L >> 2);               // token row within the substep
  const int cx = 2 * (g & 1) + ((L & 3) >> 1);            // chunk within a 32-feature fragment
  const int half8 = (L & 1) * 8;
  const int xsw = 4 * (L >> 2);                           // = 4 * (trow % 4)
  // Arrays have literal sizes: with sizes that depend on the template
  // parameter the host compiler emits no kernel.
  int aoff[2], boff[4];
#pragma unroll
  for (int f = 0; f < FA; ++f)
    aoff[f] = (trow * 32 + ((wm * (RW / 8) + f * 4 + cx) ^ xsw)) * 16 + half8;
#pragma unroll
  for (int f = 0; f < FB; ++f)
    boff[f] = PANEL_BYTES + (trow * 32 + ((wn * 16 + f * 4 + cx) ^ xsw)) * 16 + half8;

  f32x16_t acc[2][4];
  uint32_t voff[4];
  int64_t tok_end = ntok;

  // Logical stage st of the current segment [seg_k0, seg_k1) reads token
  // stage st, or seg_k0 + seg_k1 - 1 - st when the segment runs descending.
  int seg_k0 = 0, seg_k1 = nk;
  bool seg_desc = false;
  auto issue = [&](int st, char* stage) {
    const int phys = seg_desc ? seg_k0 + seg_k1 - 1 - st : st;
    const int64_t k0 = (int64_t)phys * DBK;
    const uint16_t* base = X + k0 * ldx;
    const int64_t rem = st < seg_k1 ? (tok_end - k0) * ldx * 2 : 0;
    const uint32_t num = rem <= 0 ? 0u : rem > 0xFFFFFFFFLL ? 0xFFFFFFFFu : (uint32_t)rem;
    const uint16_t* rbase = rem <= 0 ? X : base;  // nothing is read past the segment
    __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)rbase, (short)0, (int)num, 0x00020000);
#pragma unroll
    for (int q = 0; q < DMA_PER_WAVE; ++q) {
      const int gq = wave * DMA_PER_WAVE + q, panel = gq / 16, cb = gq % 16;
      char* dst = stage + panel * PANEL_BYTES + cb * 64 * 16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) char*)dst),
          16, voff[q], 0, 0, 0);
    }
  };

  // Operands of one 16-token substep: 4 A and 4 B fragments, two 4-token
  // halves each.
  struct Frags {
    v4i16_t alo[2], ahi[2], blo[4], bhi[4];
  };
  auto load = [&](Frags& F, const char* stage, int sub) {
    const int so = sub * 16 * 32 * 16;  // 16 token rows
#pragma unroll
    for (int f = 0; f < FA; ++f) {
      F.alo[f] = ds_read_tr16(stage + so + aoff[f]);
      F.ahi[f] = ds_read_tr16(stage + so + aoff[f] + 4 * 32 * 16);
    }
#pragma unroll
    for (int f = 0; f < FB; ++f) {
      F.blo[f] = ds_read_tr16(stage + so + boff[f]);
      F.bhi[f] = ds_read_tr16(stage + so + boff[f] + 4 * 32 * 16);
    }
  };
  auto mma = [&](const Frags& F) {
#pragma unroll
    for (int a = 0; a < FA; ++a)
#pragma unroll
      for (int c = 0; c < FB; ++c)
        acc[a][c] = mfma_tr<BF16>(F.alo[a], F.ahi[a], F.blo[c], F.bhi[c], acc[a][c]);
  };
  // Software pipeline.  Per stage k (buffer `cur`, next stage in `nxt`):
  //   read substep 1 of k | MFMAs of substep 0 of k
  //   wait: own LDS reads done, own loads of stage k+1 landed (three later
  //   stages may still be in flight); barrier: everyone's stage k+1 is visible
  //   and nobody reads stage k any more -> refill `cur` with stage k+5
  //   read substep 0 of k+1 | MFMAs of substep 1 of k
  // Stages past the segment are loaded through a zero-size descriptor (they
  // read as zeros and add nothing), so the loop has no data-dependent branches
  // and the compiler tracks each stage buffer's loads exactly.
  Frags F0, F1;
  // Each substep's transposing LDS reads are issued between the other
  // substep's MFMAs, so the wave never sits on a block of reads while its
  // matrix pipe drains (4 % at n = 11008).
  auto stage_step = [&](int k, char* cur, const char* nxt) {
    load(F1, cur, 1);
    mma(F0);
    GPTQ_SYRK_INTERLEAVE(FA, 0);
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkm0();
    wait_vmcnt<(DS - 2) * DMA_PER_WAVE>();
    __builtin_amdgcn_s_barrier();
    issue(k + DS, cur);
    __builtin_amdgcn_sched_barrier(0);
    load(F0, nxt, 0);
    mma(F1);
    GPTQ_SYRK_INTERLEAVE(FA, 1);
    __builtin_amdgcn_sched_barrier(0);
  };

  // acc = sum over token stages [k0, k1) of the 256 x 256 tile at (i0, j0),
  // taken in descending stage order when desc is set.
  auto run = [&](int64_t i0, int64_t j0, int k0, int k1, bool desc) {
    seg_k0 = k0;
    seg_k1 = k1;
    seg_desc = desc;
#pragma unroll
    for (int q = 0; q < DMA_PER_WAVE; ++q) {
      const int gq = wave * DMA_PER_WAVE + q, panel = gq / 16, cb = gq % 16;
      const int p = cb * 64 + lane;
      const int t = p / 32, c = (p % 32) ^ (4 * (t % 4));
      const int64_t col = (panel ? j0 : i0) + 8 * c;
      voff[q] = (uint32_t)((t * ldx + col) * 2);
    }
    tok_end = (int64_t)k1 * DBK < ntok ? (int64_t)k1 * DBK : ntok;
#pragma unroll
    for (int a = 0; a < FA; ++a)
#pragma unroll
      for (int c = 0; c < FB; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[a][c][v] = 0.0f;
    issue(k0 + 0, st0);
    issue(k0 + 1, st1);
    issue(k0 + 2, st2);
    issue(k0 + 3, st3);
    issue(k0 + 4, st4);
    wait_vmcnt<(DS - 1) * DMA_PER_WAVE>();
    __builtin_amdgcn_s_barrier();
    load(F0, st0, 0);
    for (int kt = k0; kt < k1; kt += DS) {
      stage_step(kt + 0, st0, st1);
      stage_step(kt + 1, st1, st2);
      stage_step(kt + 2, st2, st3);
      stage_step(kt + 3, st3, st4);
      stage_step(kt + 4, st4, st0);
    }
    wait_vmcnt<0>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();  // every wave is done with the stage buffers
  };

  // H[i][j] += 2 * acc for i <= j (upper triangle), in bounds.  Buffer loads
  // and stores: an element outside the triangle gets an offset past the
  // descriptor's range (the load returns 0, the store is dropped), so the
  // epilogue has no branches and each 32 x 32 block's 16 loads are in flight
  // together instead of one round trip per element.
  auto store_h = [&](int64_t i0, int64_t j0) __attribute__((always_inline)) {
    const int64_t rem = ((n - i0) * n - j0) * 4;  // bytes from H[i0][j0] to the end of H
    const int num = rem < 0x7FFFFFF0LL ? (int)rem : 0x7FFFFFF0;
    __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(H + i0 * n + j0), (short)0, num, 0x00020000);
    // Under stream-K, an opaque copy of the lane index: inside the loop over
    // segments the compiler would otherwise hoist all 128 element offsets
    // (loop invariant) above the loop and spill them.
    int ln = lane;
    if constexpr (STREAMK) asm volatile("" : "+v"(ln));
#pragma unroll
    for (int a = 0; a < FA; ++a)
#pragma unroll
      for (int c = 0; c < FB; ++c) {
        const int jl = wn * 128 + c * 32 + (ln & 31);
        uint32_t off[16];
        float hv[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int il = wm * RW + a * 32 + (v >> 2) * 8 + (ln >> 5) * 4 + (v & 3);
          const bool in = i0 + il < n && j0 + jl < n && i0 + il <= j0 + jl;
          off[v] = in ? (uint32_t)(((int64_t)il * n + jl) * 4) : 0x80000000u;
          hv[v] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (int)off[v], 0, 0));
        }
#pragma unroll
        for (int v = 0; v < 16; ++v)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(hv[v] + 2.0f * acc[a][c][v]), rs,
                                                (int)off[v], 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
  };
  // A partial tile: acc stored row-major (256 x 256) to `part`.
  auto store_part = [&](float* part) __attribute__((always_inline)) {
    int ln = lane;  // opaque, as in store_h
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int a = 0; a < FA; ++a)
#pragma unroll
      for (int c = 0; c < FB; ++c) {
        const int jl = wn * 128 + c * 32 + (ln & 31);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int il = wm * RW + a * 32 + (v >> 2) * 8 + (ln >> 5) * 4 + (v & 3);
          part[il * DT + jl] = acc[a][c][v];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
  };

  if constexpr (!STREAMK) {
    int ti, tj;
    if (!syrk_tile(blockIdx.x, nt, ti, tj)) return;
    run((int64_t)ti * DT, (int64_t)tj * DT, 0, nk, false);
    store_h((int64_t)ti * DT, (int64_t)tj * DT);
  } else if (sk.ks > 0) {
    const int S = sk.ks, C = sk.nwg / 8, x = blockIdx.x % 8;
    const KsXcd k = ks_xcd(x, S, C, (int64_t)nt * (nt + 1) / 2);
#pragma nounroll
    for (int64_t i = blockIdx.x / 8; i < k.items; i += C) {
      int64_t o;
      int k0, k1;
      ks_item(k, i, x % S, S, C, nk, o, k0, k1);
      int ti, tj;
      tile_of(o, nt, ti, tj);
      ti = __builtin_amdgcn_readfirstlane(ti);
      tj = __builtin_amdgcn_readfirstlane(tj);
      run((int64_t)ti * DT, (int64_t)tj * DT, k0, k1, false);
      store_part(sk.partial + (k.base + i) * PART_FLOATS);
    }
  } else {
    const int64_t total = (int64_t)nt * (nt + 1) / 2 * nk;
    const int lam = (blockIdx.x % 8) * (sk.nwg / 8) + blockIdx.x / 8;  // XCD-contiguous runs
    const int64_t s0 = (int64_t)lam * sk.units;
    const int64_t s1 = s0 + sk.units < total ? s0 + sk.units : total;
#pragma nounroll
    for (int64_t pos = s0; pos < s1;) {
      const int64_t tile = pos / nk;
      const int k0 = (int)(pos % nk);
      const int k1 = (int)(k0 + (s1 - pos) < nk ? k0 + (s1 - pos) : nk);
      int ti, tj;
      tile_of(tile, nt, ti, tj);
      ti = __builtin_amdgcn_readfirstlane(ti);
      tj = __builtin_amdgcn_readfirstlane(tj);
      // A run's first segment, when it starts inside a tile, walks its
      // stages downwards from the last one: runs start at staggered token
      // offsets, and this way the concurrently running segments of one XCD
      // meet the same token stages at the same time instead of each
      // streaming its own part of X through the shared L2 (about 3 % faster
      // at n = 4096, where every run holds less than one tile).
      run((int64_t)ti * DT, (int64_t)tj * DT, k0, k1, k1 == nk && k0 > 0);
      if (k0 == 0 && k1 == nk)
        store_h((int64_t)ti * DT, (int64_t)tj * DT);
      else
        store_part(sk.partial + ((int64_t)lam * 2 + (pos == s0 ? 0 : 1)) * PART_FLOATS);
      pos += k1 - k0;
    }
  }
}

// H += 2 * (sum of a split tile's partials, in run order).  Grid: (tiles,
// DT / FIX_ROWS); thread = tile column, FIX_ROWS rows per workgroup.
constexpr int FIX_ROWS = 16;
__global__ void __launch_bounds__(DT)
syrk_streamk_fixup(float* __restrict__ H, int64_t n, int nk, const float* __restrict__ partial,
                   int64_t units) {
  const int nt = (int)((n + DT - 1) / DT);
  const int64_t tile = blockIdx.x;
  // Launched only when units < nk: then every tile has two or more contributors.
  const int64_t first = tile * nk / units, lastw = ((tile + 1) * nk - 1) / units;
  int ti, tj;
  tile_of(tile, nt, ti, tj);
  const int r0 = blockIdx.y * FIX_ROWS, jl = threadIdx.x;
  float sum[FIX_ROWS];
  for (int64_t w = first; w <= lastw; ++w) {
    const int64_t seg0 = w * units > tile * nk ? w * units : tile * nk;
    const float* part = partial + (w * 2 + (seg0 == w * units ? 0 : 1)) * (int64_t)PART_FLOATS +
                        (int64_t)r0 * DT + jl;
#pragma unroll
    for (int r = 0; r < FIX_ROWS; ++r) {
      const float x = part[r * DT];
      sum[r] = w == first ? x : sum[r] + x;
    }
  }
  const int64_t j = (int64_t)tj * DT + jl;
#pragma unroll
  for (int r = 0; r < FIX_ROWS; ++r) {
    const int64_t i = (int64_t)ti * DT + r0 + r;
    if (i < n && j < n && i <= j) H[i * n + j] += 2.0f * sum[r];
  }
}

// Token-split schedule: H += 2 * (sum of a tile's partials: blocks in order,
// pieces in order).  Grid: (tiles, DT / FIX_ROWS); thread (rq, jx) sums rows
// r0 + 4 rq .. +3 at columns 4 jx .. +3 with 16-byte loads of the partials.
__global__ void __launch_bounds__(DT)
syrk_ksplit_fixup(float* __restrict__ H, int64_t n, int S, int C, const float* __restrict__ partial) {
  static_assert(FIX_ROWS == 4 * (DT / 64), "four rows per thread");
  const int nt = (int)((n + DT - 1) / DT);
  const int64_t T = (int64_t)nt * (nt + 1) / 2;
  const int64_t o = blockIdx.x;
  int ti, tj;
  tile_of(o, nt, ti, tj);
  const int rq = threadIdx.x / 64, jx = threadIdx.x % 64;
  const int r0 = blockIdx.y * FIX_ROWS + 4 * rq;
  float4 sum[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) sum[r] = make_float4(0.f, 0.f, 0.f, 0.f);
  const int G = 8 / S;
  const int g = (int)((o * G + G - 1) / T);  // first group whose range holds o
  int gg = g;
  while (gg > 0 && T * gg / G > o) --gg;
  while (T * (gg + 1) / G <= o) ++gg;
  for (int b = 0; b < S; ++b) {
    const KsXcd k = ks_xcd(gg * S + b, S, C, T);
    const int64_t lt = o - k.t0, whole = (int64_t)k.q * C;
    const int64_t first = lt < whole ? lt : whole + (lt - whole) * k.sp;
    const int cnt = lt < whole ? 1 : k.sp;
    for (int p = 0; p < cnt; ++p) {
      const float* part =
          partial + (k.base + first + p) * (int64_t)PART_FLOATS + (int64_t)r0 * DT + 4 * jx;
      float4 v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = *reinterpret_cast<const float4*>(part + r * DT);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sum[r].x += v[r].x;
        sum[r].y += v[r].y;
        sum[r].z += v[r].z;
        sum[r].w += v[r].w;
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t i = (int64_t)ti * DT + r0 + r;
    const int64_t j = (int64_t)tj * DT + 4 * jx;
    const float e[4] = {sum[r].x, sum[r].y, sum[r].z, sum[r].w};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (i < n && j + c < n && i <= j + c) H[i * n + j + c] += 2.0f * e[c];
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

namespace {
// Compute units of the current device, rounded down to whole rounds over the
// 8 XCDs (the stream-K grid), at most MAX_SK_WG.
constexpr int MAX_SK_WG = 512;
int sk_workgroups() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  cus = cus >= 8 ? cus / 8 * 8 : 8;
  return cus < MAX_SK_WG ? cus : MAX_SK_WG;
}
size_t partial_bytes(int nwg) { return align_up((size_t)nwg * 2 * PART_FLOATS * sizeof(float)); }

// Whole-tile launches cover at most this many tokens.
constexpr int64_t WHOLE_CHUNK = 32768;
// The token-split schedule needs at least this many 32-token stages per
// block: shorter items pay the pipeline fill, the partial store and the
// fix-up for too little work (measured at n = 4096: 4 % faster than
// stream-K at 256 stages per block, 11 % slower at 128, 17 % faster at 1024).
constexpr int KS_MIN_STAGES = 256;
// The split schedules are used when whole tiles leave the last round less
// than 90 % full (at n = 4096, 136 tiles on 256 workgroups; at n = 8192,
// 528 tiles: 2.06 rounds).
inline bool split_schedules(int64_t T, int nwg) {
  const int64_t rounds = (T + nwg - 1) / nwg;
  return 10 * T < 9 * rounds * (int64_t)nwg;
}
// Token blocks for T tiles on nwg workgroups: enough blocks that each XCD
// has at least four rounds of items, at most 8.
int ks_blocks(int64_t T, int nwg) {
  const int C = nwg / 8;
  int S = 1;
  while (S < 8 && T * S / 8 < 4 * (int64_t)C) S *= 2;
  return S;
}
size_t ks_bytes(int64_t n, int nwg) {
  const int nt = (int)((n + DT - 1) / DT);
  const int64_t T = (int64_t)nt * (nt + 1) / 2;
  const int S = ks_blocks(T, nwg), C = nwg / 8;
  int64_t items = 0;
  for (int x = 0; x < 8; ++x) items += ks_xcd(x, S, C, T).items;
  return align_up((size_t)items * PART_FLOATS * sizeof(float));
}
}  // namespace

size_t syrk_workspace_bytes(int64_t n) {
  const int nwg = sk_workgroups();
  const int nt = (int)((n + DT - 1) / DT);
  const int64_t T = (int64_t)nt * (nt + 1) / 2;
  if (!split_schedules(T, nwg)) return 0;  // whole tiles only
  const size_t a = 4 * T < 3 * (int64_t)nwg ? partial_bytes(nwg) : 0, b = ks_bytes(n, nwg);
  return a > b ? a : b;
}

hipError_t launch_syrk(float* H, int64_t n, const void* X, int dtype, int64_t ntok,
                       int64_t ldx, void* ws, size_t ws_bytes, hipStream_t s) {
  const uint16_t* x = static_cast<const uint16_t*>(X);
  const bool aligned = (ldx % 8 == 0) && ((reinterpret_cast<uintptr_t>(X) & 15) == 0);
  const bool bf = dtype == 1;
  if (aligned) {
    // direct-to-LDS pipeline (16-byte chunks need 16-byte aligned rows)
    const int nt = (int)((n + DT - 1) / DT);
    const int64_t tiles = (int64_t)nt * (nt + 1) / 2;
    const int nwg = sk_workgroups();
    const int nk = (int)((ntok + DBK - 1) / DBK);
    StreamK sk{static_cast<float*>(ws), 0, nwg, 0};
    auto kern_sk = bf ? syrk_dma_kernel<true, true> : syrk_dma_kernel<false, true>;
    const bool have_ws = ws != nullptr && ws_bytes >= syrk_workspace_bytes(n);
    if (have_ws && split_schedules(tiles, nwg)) {
      const int S = ks_blocks(tiles, nwg);
      if (nk / S >= KS_MIN_STAGES) {
        sk.ks = S;
        hipLaunchKernelGGL(kern_sk, dim3((unsigned)nwg), dim3(SyrkShape<true>::NW * 64), 0, s, H,
                           n, x, ntok, ldx, sk);
        GPTQ_HIP_TRY(hipGetLastError());
        hipLaunchKernelGGL(syrk_ksplit_fixup, dim3((unsigned)tiles, DT / FIX_ROWS), dim3(DT), 0,
                           s, H, n, S, nwg / 8, sk.partial);
        return hipGetLastError();
      }
      if (4 * tiles < 3 * (int64_t)nwg) {
        sk.units = (tiles * nk + nwg - 1) / nwg;
        hipLaunchKernelGGL(kern_sk, dim3((unsigned)nwg), dim3(SyrkShape<true>::NW * 64), 0, s, H,
                           n, x, ntok, ldx, sk);
        GPTQ_HIP_TRY(hipGetLastError());
        if (sk.units < nk)
          hipLaunchKernelGGL(syrk_streamk_fixup, dim3((unsigned)tiles, DT / FIX_ROWS), dim3(DT), 0,
                             s, H, n, nk, sk.partial, sk.units);
        return hipGetLastError();
      }
    }
    // Whole tiles, one launch per WHOLE_CHUNK tokens: all workgroups of a
    // launch start at the same token stage and stay close, so the X rows they
    // read together stay in L2 (one launch over 262144 tokens is 5-7 % slower).
    const int64_t blocks = (tiles + 7) / 8 * 8;  // whole rounds over the 8 XCDs
    auto kern = bf ? syrk_dma_kernel<true, false> : syrk_dma_kernel<false, false>;
    for (int64_t t0 = 0; t0 < ntok; t0 += WHOLE_CHUNK) {
      const int64_t len = ntok - t0 < WHOLE_CHUNK ? ntok - t0 : WHOLE_CHUNK;
      hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(SyrkShape<false>::NW * 64), 0, s, H, n,
                         x + t0 * ldx, len, ldx, sk);
      GPTQ_HIP_TRY(hipGetLastError());
    }
    return hipSuccess;
  }
  // Unaligned rows: register-staged kernel with element loads.
  constexpr int T = 256;
  return bf ? launch_t<T, true, false>(H, n, x, ntok, ldx, s)
            : launch_t<T, false, false>(H, n, x, ntok, ldx, s);
}

}  // namespace gptq
