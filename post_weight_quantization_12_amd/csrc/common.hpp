// Shared declarations of the gfx950 GPTQ library (host side and device helpers).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <mutex>
#include <string>

namespace gptq {

// Vector types used with the gfx950 matrix-core builtins.
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// s_waitcnt with vmcnt <= N and the other counters left alone (gfx9 encoding:
// vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// s_waitcnt lgkmcnt(0) (LDS reads and writes of this wave done), vmcnt untouched.
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0x3 << 14) | 0xF); }

// Helper streams of one device for calls that spread their work: two
// non-blocking streams (default priority) and six timing-free events,
// created on first use and kept until the process ends.  A call takes
// helper_mutex() before helper_streams() and holds it while it enqueues, so
// calls from several host threads never interleave their event records and
// waits; it forks from and joins back into the caller's stream.
struct HelperStreams {
  hipStream_t a = nullptr, b = nullptr;
  hipEvent_t ev[6] = {};
};
std::mutex& helper_mutex();
hipError_t helper_streams(HelperStreams*& out);

// Error reporting to the C ABI (per host thread).
void set_error(const std::string& msg);
void clear_error();

// Workspace carving: every piece 256-byte aligned.
inline size_t align_up(size_t v, size_t a = 256) { return (v + a - 1) / a * a; }

struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* p) : base(static_cast<char*>(p)) {}
  template <typename T>
  T* take(size_t count) {
    T* p = reinterpret_cast<T*>(base ? base + used : nullptr);
    used += align_up(count * sizeof(T));
    return p;
  }
};

// ---------------------------------------------------------------------------
// fp32 matrix-core GEMM on row-major operands:
//     C[M x N] = alpha * op(A) * op(B) + beta * C
// op(A) is A [M x K] (transA = false) or A^T with A stored [K x M];
// op(B) is B [K x N] (transB = false) or B^T with B stored [N x K].
// kmode restricts each output tile's K range to where a triangular operand
// can be nonzero (entries outside must still be zero in memory if read):
enum KRange : int {
  KR_FULL = 0,    // all of [0, K)
  KR_LE_COL = 1,  // op(B)[k][j] == 0 for k > j  -> k < j0 + tile_n
  KR_GE_COL = 2,  // op(B)[k][j] == 0 for k < j  -> k >= j0
  KR_LE_ROW = 3,  // op(A)[i][k] == 0 for k > i  -> k < i0 + tile_m
};
struct GemmArgs {
  int64_t M, N, K;
  const float* A; int64_t lda; bool transA;
  const float* B; int64_t ldb; bool transB;
  float* C; int64_t ldc;
  float alpha, beta;
  int kmode;
  bool lower_only;  // compute only tiles that touch the lower triangle (i >= j)
  // Products as three fp16 MFMAs on split operands (x = hi + lo, both fp16;
  // the lo*lo term dropped), fp32 accumulation: about 2^-20 relative per
  // operand for values of magnitude ~1 (values must stay below 65504 and are
  // resolved down to ~2^-24 absolute).  Used only where the operands are
  // scaled to that range; falls back to fp32 MFMAs on unaligned shapes.
  bool split16 = false;
};
hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t s);
// Two independent products (no operand of one is written by the other) in
// one launch where both take the 64 x 64 split-fp16 tiles, the first with B
// transposed and the second not (A not transposed in either); otherwise two
// launches.  Each result is what launch_gemm_f32 gives.
hipError_t launch_gemm_f32_pair(const GemmArgs& a, const GemmArgs& b, hipStream_t s);
// Error-update GEMM of the column sweep on the errors the sweep stored split:
//   C[M x N] -= sum over sweep blocks b (kb columns each) of
//               einv[b][r] * (Ehi + Elo)_b (V + Vl)_b^T
// E: per 16 columns of a row, 16 fp16 high parts then 16 fp16 remainders of
// the errors scaled by 1 / einv (row stride lde floats, 16-byte aligned);
// V, Vl: fp16 [N x K], k-contiguous (ldv a multiple of 8); Vl == nullptr
// drops the third product (Ehi Vl); einv fp32 [K / kb][eld]; kb 32, 64 or
// 128 dividing K.
hipError_t launch_gemm_eh(int64_t M, int64_t N, int64_t K, const float* E, int64_t lde,
                          const _Float16* V, const _Float16* Vl, int64_t ldv, float* C,
                          int64_t ldc, const float* einv, int64_t eld, int kb, hipStream_t s);

// Hessian SYRK: H(upper) += 2 X^T X.  ws (optional) enables the stream-K schedule.
size_t syrk_workspace_bytes(int64_t n);
hipError_t launch_syrk(float* H, int64_t n, const void* X, int dtype, int64_t ntok,
                       int64_t ldx, void* ws, size_t ws_bytes, hipStream_t s);

// gptq_prepare pipeline.
size_t prepare_workspace_bytes(int64_t n);
hipError_t run_prepare(const float* H, int64_t n, float damp, int desc_act, float* U,
                       int32_t* perm, int32_t* info, void* ws, hipStream_t s);

// order[r] = the index i of rank r when the n keys are sorted by decreasing
// value, ties by increasing index (a stable sort).  rank: n ints of scratch.
hipError_t launch_stable_order_desc(const uint32_t* keys, int64_t n, int32_t* rank,
                                    int32_t* order, hipStream_t s);

// gptq_quantize_layer pipeline.
size_t quantize_workspace_bytes(int64_t out, int64_t in, int bits, int gs, int block);
hipError_t run_quantize(const void* W, int wdtype, int64_t out, int64_t in, const float* U,
                        const int32_t* perm, int bits, int gs, int sym, int block,
                        int32_t* qweight, float* scales, int32_t* zeros, int32_t* g_idx,
                        void* ws, hipStream_t s);

// Dequantize-on-the-fly matmul Y = X W^T from the packed layer.  Up to
// DQ_SMALL_M_MAX token rows take the HBM-bound kernel (its workspace holds
// the split input range's partial sums), more the MFMA tiles.
// With x_order, packed position p reads input column x_order[p]; the
// matrix-core path gathers X into its workspace first.
constexpr int DQ_SMALL_M_MAX = 8;  // measured: the tiles win from 9 tokens on
size_t dequant_matmul_workspace_bytes(int64_t M, int64_t in, int64_t out, int has_order);
hipError_t run_dequant_matmul(const void* X, int64_t M, int64_t in, int64_t ldx,
                              const int32_t* qweight, const float* scales, const int32_t* zeros,
                              const int32_t* g_idx, const int32_t* x_order, int64_t out, int bits,
                              void* Y, int y_f16, int64_t ldy, void* ws, size_t ws_bytes,
                              hipStream_t s);
// Host-side argument checks of the dequantize-on-the-fly entry points: a
// gptq_status_t (GPTQ_OK, or the failure with gptq_last_error_message set).
int dequant_check(const void* X, int x_dtype, int64_t M, int64_t in, int64_t ldx,
                  const int32_t* qweight, const float* scales, const int32_t* zeros,
                  const int32_t* g_idx, int64_t n_groups, int64_t out, int bits, const void* Y,
                  int y_dtype, int64_t ldy);
// Storage form of the group parameters: fp16 scales, zeros packed b-bit
// along the output channels (out * bits % 32 == 0), and the inverse.
hipError_t run_export(const float* scales, const int32_t* zeros, int64_t G, int64_t out, int bits,
                      void* scales_f16, int32_t* qzeros, hipStream_t s);
hipError_t run_unpack_zeros(const int32_t* qzeros, int64_t G, int64_t out, int bits,
                            int32_t* zeros, hipStream_t s);

// A = SiLU(G) * U elementwise, fp16 in and out, fp32 arithmetic.
hipError_t run_silu_mul(const void* G, int64_t ldg, const void* U, int64_t ldu, int64_t rows,
                        int64_t cols, void* A, int64_t lda, hipStream_t s);

// Causal (or full) multi-head attention per sequence, fp16 in and out, fp32
// softmax and accumulation; head_dim 64 or 128.
hipError_t run_attention(const void* Q, int64_t ldq, const void* K, int64_t ldk, const void* V,
                         int64_t ldv, void* O, int64_t ldo, int64_t seqs, int64_t seq_len,
                         int heads, int head_dim, int causal, hipStream_t s);
// Hs = X + A and U = RMSNorm(Hs) * gamma, rows of d fp16 values.
hipError_t run_residual_rmsnorm(const void* X, int64_t ldx, const void* A, int64_t lda,
                                const void* gamma, int64_t rows, int64_t d, float eps, void* Hs,
                                int64_t ldh, void* U, int64_t ldu, hipStream_t s);

// The layer's input positions re-ordered by group (stable), repacked.
size_t dequant_group_order_workspace_bytes(int64_t in);
hipError_t run_dequant_group_order(const int32_t* qweight, const int32_t* g_idx, int64_t in,
                                   int64_t out, int bits, int32_t* qweight_sorted,
                                   int32_t* g_idx_sorted, int32_t* x_order, void* ws,
                                   hipStream_t s);

}  // namespace gptq

#define GPTQ_HIP_TRY(expr)                  \
  do {                                      \
    hipError_t _e = (expr);                 \
    if (_e != hipSuccess) return _e;        \
  } while (0)
