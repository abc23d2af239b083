// extern "C" entry points of the gfx950 GPTQ library: argument validation
// (before anything is enqueued), workspace checks, status strings.
#include <cmath>
#include <map>
#include <string>

#include "../../include/gptq.h"
#include "common.hpp"

namespace gptq {
namespace {
thread_local std::string g_last_error;
}
void set_error(const std::string& msg) { g_last_error = msg; }
void clear_error() { g_last_error.clear(); }
const char* last_error_c() { return g_last_error.c_str(); }

std::mutex& helper_mutex() {
  static std::mutex mu;
  return mu;
}
hipError_t helper_streams(HelperStreams*& out) {
  static std::map<int, HelperStreams> per_dev;  // guarded by helper_mutex()
  int dev = 0;
  GPTQ_HIP_TRY(hipGetDevice(&dev));
  auto it = per_dev.find(dev);
  if (it == per_dev.end()) {
    HelperStreams h;
    GPTQ_HIP_TRY(hipStreamCreateWithFlags(&h.a, hipStreamNonBlocking));
    GPTQ_HIP_TRY(hipStreamCreateWithFlags(&h.b, hipStreamNonBlocking));
    for (hipEvent_t& e : h.ev) GPTQ_HIP_TRY(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    it = per_dev.emplace(dev, h).first;
  }
  out = &it->second;
  return hipSuccess;
}

// Host-side checks shared by the dequantize-on-the-fly entry points;
// GPTQ_OK or the failing status with its message set.
int dequant_check(const void* X, int x_dtype, int64_t M, int64_t in, int64_t ldx,
                  const int32_t* qweight, const float* scales, const int32_t* zeros,
                  const int32_t* g_idx, int64_t n_groups, int64_t out, int bits, const void* Y,
                  int y_dtype, int64_t ldy) {
  auto bad = [](int status, const char* msg) {
    set_error(msg);
    return status;
  };
  if (!X) return bad(GPTQ_ERR_INVALID_ARG, "X is NULL");
  if (!qweight || !scales || !zeros || !g_idx)
    return bad(GPTQ_ERR_INVALID_ARG, "qweight, scales, zeros or g_idx is NULL");
  if (!Y) return bad(GPTQ_ERR_INVALID_ARG, "Y is NULL");
  if (M < 0) return bad(GPTQ_ERR_INVALID_ARG, "M must be >= 0");
  if (in < 32 || in % 32 != 0) return bad(GPTQ_ERR_INVALID_ARG, "in must be a positive multiple of 32");
  if (out < 1) return bad(GPTQ_ERR_INVALID_ARG, "out must be >= 1");
  if (n_groups < 1) return bad(GPTQ_ERR_INVALID_ARG, "n_groups must be >= 1");
  if (ldx < in) return bad(GPTQ_ERR_INVALID_ARG, "ldx must be >= in");
  if (ldy < out) return bad(GPTQ_ERR_INVALID_ARG, "ldy must be >= out");
  if (x_dtype != GPTQ_F16) return bad(GPTQ_ERR_UNSUPPORTED, "x_dtype must be GPTQ_F16");
  if (y_dtype != GPTQ_F16 && y_dtype != GPTQ_F32)
    return bad(GPTQ_ERR_INVALID_ARG, "y_dtype must be GPTQ_F16 or GPTQ_F32");
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return bad(GPTQ_ERR_UNSUPPORTED, "bits must be 2, 3, 4 or 8");
  if (ldx % 8 != 0 || (reinterpret_cast<uintptr_t>(X) & 15) != 0)
    return bad(GPTQ_ERR_UNSUPPORTED, "X rows must be 16-byte aligned (ldx a multiple of 8)");
  // the matrix-core kernels address qweight, scales, zeros and a 256-row X
  // tile with 32-bit buffer offsets
  if ((in / 32) * bits * out > (int64_t(1) << 29) || n_groups * out > (int64_t(1) << 29))
    return bad(GPTQ_ERR_UNSUPPORTED, "qweight, scales and zeros must each be below 2 GiB");
  if (M > 8 && ldx > (int64_t(1) << 22))
    return bad(GPTQ_ERR_UNSUPPORTED, "from 9 tokens on, ldx must be at most 2^22");
  return GPTQ_OK;
}
}  // namespace gptq

using namespace gptq;

namespace {

int fail(int status, const std::string& msg) {
  set_error(msg);
  return status;
}

int hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return GPTQ_OK;
  return fail(GPTQ_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

bool valid_group(int gs, int block) {
  if (gs == -1) return true;
  return gs >= 4 && gs % 4 == 0 && gs <= block && block % gs == 0;
}

}  // namespace

extern "C" {

size_t gptq_hessian_workspace_bytes(int64_t n) {
  if (n < 1) return 0;
  return syrk_workspace_bytes(n);
}

int gptq_hessian_accumulate(float* H, int64_t n, const void* X, int x_dtype, int64_t ntok,
                            int64_t ldx, void* workspace, size_t workspace_bytes,
                            void* stream) {
  clear_error();
  if (!H) return fail(GPTQ_ERR_INVALID_ARG, "H is NULL");
  if (!X) return fail(GPTQ_ERR_INVALID_ARG, "X is NULL");
  if (n < 1) return fail(GPTQ_ERR_INVALID_ARG, "n must be >= 1");
  if (ntok < 0) return fail(GPTQ_ERR_INVALID_ARG, "ntok must be >= 0");
  if (ldx < n) return fail(GPTQ_ERR_INVALID_ARG, "ldx must be >= n");
  if (x_dtype != GPTQ_F16 && x_dtype != GPTQ_BF16)
    return fail(GPTQ_ERR_UNSUPPORTED, "x_dtype must be GPTQ_F16 or GPTQ_BF16");
  const int64_t nt = (n + 127) / 128;
  if (nt * (nt + 1) / 2 > 0x7FFFFFFFLL) return fail(GPTQ_ERR_UNSUPPORTED, "n too large");
  if (workspace != nullptr && workspace_bytes < syrk_workspace_bytes(n))
    return fail(GPTQ_ERR_WORKSPACE,
                "workspace smaller than gptq_hessian_workspace_bytes(n) = " +
                    std::to_string(syrk_workspace_bytes(n)) + " (or pass NULL)");
  if (ntok == 0) return GPTQ_OK;
  return hip_status(launch_syrk(H, n, X, x_dtype, ntok, ldx, workspace, workspace_bytes,
                                static_cast<hipStream_t>(stream)),
                    "gptq_hessian_accumulate");
}

size_t gptq_prepare_workspace_bytes(int64_t n) {
  if (n < 1 || n > GPTQ_MAX_PREPARE_N) return 0;
  return prepare_workspace_bytes(n);
}

int gptq_prepare(const float* H, int64_t n, float damp_percent, int desc_act, float* Hinv_chol,
                 int32_t* perm, int32_t* info, void* workspace, size_t workspace_bytes,
                 void* stream) {
  clear_error();
  if (!H) return fail(GPTQ_ERR_INVALID_ARG, "H is NULL");
  if (!Hinv_chol) return fail(GPTQ_ERR_INVALID_ARG, "Hinv_chol is NULL");
  if (!perm) return fail(GPTQ_ERR_INVALID_ARG, "perm is NULL");
  if (!info) return fail(GPTQ_ERR_INVALID_ARG, "info is NULL");
  if (n < 1) return fail(GPTQ_ERR_INVALID_ARG, "n must be >= 1");
  if (n > GPTQ_MAX_PREPARE_N)
    return fail(GPTQ_ERR_UNSUPPORTED, "n exceeds GPTQ_MAX_PREPARE_N (32768)");
  if (!(damp_percent >= 0.0f) || !std::isfinite(damp_percent))
    return fail(GPTQ_ERR_INVALID_ARG, "damp_percent must be finite and >= 0");
  if (static_cast<const void*>(H) == static_cast<const void*>(Hinv_chol))
    return fail(GPTQ_ERR_INVALID_ARG, "H and Hinv_chol must not alias");
  const size_t need = prepare_workspace_bytes(n);
  if (!workspace) return fail(GPTQ_ERR_INVALID_ARG, "workspace is NULL");
  if (workspace_bytes < need)
    return fail(GPTQ_ERR_WORKSPACE, "workspace smaller than gptq_prepare_workspace_bytes(n) = " +
                                        std::to_string(need));
  return hip_status(run_prepare(H, n, damp_percent, desc_act ? 1 : 0, Hinv_chol, perm, info,
                                workspace, static_cast<hipStream_t>(stream)),
                    "gptq_prepare");
}

size_t gptq_quantize_workspace_bytes(int64_t out, int64_t in, int bits, int group_size,
                                     int block) {
  if (out < 1 || in < 32 || in % 32 != 0 || in > GPTQ_MAX_PREPARE_N) return 0;
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8) return 0;
  if (block != 32 && block != 64 && block != 128) return 0;
  if (!valid_group(group_size, block)) return 0;
  return quantize_workspace_bytes(out, in, bits, group_size, block);
}

int gptq_quantize_layer(const void* W, int w_dtype, int64_t out, int64_t in,
                        const float* Hinv_chol, const int32_t* perm, int bits, int group_size,
                        int sym, int block, int32_t* qweight, float* scales, int32_t* zeros,
                        int32_t* g_idx, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  if (!W) return fail(GPTQ_ERR_INVALID_ARG, "W is NULL");
  if (!Hinv_chol) return fail(GPTQ_ERR_INVALID_ARG, "Hinv_chol is NULL");
  if (!qweight || !scales || !zeros || !g_idx)
    return fail(GPTQ_ERR_INVALID_ARG, "an output pointer (qweight/scales/zeros/g_idx) is NULL");
  if (w_dtype != GPTQ_F16 && w_dtype != GPTQ_BF16 && w_dtype != GPTQ_F32)
    return fail(GPTQ_ERR_INVALID_ARG, "w_dtype must be GPTQ_F16, GPTQ_BF16 or GPTQ_F32");
  if (out < 1) return fail(GPTQ_ERR_INVALID_ARG, "out must be >= 1");
  if (out > 0x7FFFFFFFLL) return fail(GPTQ_ERR_UNSUPPORTED, "out too large");
  if (in < 32 || in % 32 != 0)
    return fail(GPTQ_ERR_INVALID_ARG, "in must be a positive multiple of 32");
  if (in > GPTQ_MAX_PREPARE_N) return fail(GPTQ_ERR_UNSUPPORTED, "in exceeds 32768");
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return fail(GPTQ_ERR_UNSUPPORTED, "bits must be 2, 3, 4 or 8");
  if (block != 32 && block != 64 && block != 128)
    return fail(GPTQ_ERR_UNSUPPORTED, "block must be 32, 64 or 128");
  if (!valid_group(group_size, block))
    return fail(GPTQ_ERR_INVALID_ARG,
                "group_size must be -1 or a multiple of 4 that divides block");
  if (sym != 0 && sym != 1) return fail(GPTQ_ERR_INVALID_ARG, "sym must be 0 or 1");
  const size_t need = quantize_workspace_bytes(out, in, bits, group_size, block);
  if (!workspace) return fail(GPTQ_ERR_INVALID_ARG, "workspace is NULL");
  if (workspace_bytes < need)
    return fail(GPTQ_ERR_WORKSPACE,
                "workspace smaller than gptq_quantize_workspace_bytes(...) = " +
                    std::to_string(need));
  return hip_status(run_quantize(W, w_dtype, out, in, Hinv_chol, perm, bits, group_size, sym,
                                 block, qweight, scales, zeros, g_idx, workspace,
                                 static_cast<hipStream_t>(stream)),
                    "gptq_quantize_layer");
}

size_t gptq_dequant_matmul_workspace_bytes(int64_t M, int64_t in, int64_t out, int has_order) {
  if (M < 1 || in < 32 || in % 32 != 0 || out < 1) return 0;
  return dequant_matmul_workspace_bytes(M, in, out, has_order ? 1 : 0);
}

int gptq_dequant_matmul(const void* X, int x_dtype, int64_t M, int64_t in, int64_t ldx,
                        const int32_t* qweight, const float* scales, const int32_t* zeros,
                        const int32_t* g_idx, const int32_t* x_order, int64_t n_groups,
                        int64_t out, int bits, void* Y, int y_dtype, int64_t ldy,
                        void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  const int st = dequant_check(X, x_dtype, M, in, ldx, qweight, scales, zeros, g_idx, n_groups,
                               out, bits, Y, y_dtype, ldy);
  if (st != GPTQ_OK || M == 0) return st;
  const size_t need = dequant_matmul_workspace_bytes(M, in, out, x_order ? 1 : 0);
  if (need > 0 && !workspace) return fail(GPTQ_ERR_INVALID_ARG, "workspace is NULL");
  if (workspace_bytes < need)
    return fail(GPTQ_ERR_WORKSPACE,
                "workspace smaller than gptq_dequant_matmul_workspace_bytes(...) = " +
                    std::to_string(need));
  return hip_status(run_dequant_matmul(X, M, in, ldx, qweight, scales, zeros, g_idx, x_order, out,
                                       bits, Y, y_dtype == GPTQ_F16 ? 1 : 0, ldy, workspace,
                                       workspace_bytes, static_cast<hipStream_t>(stream)),
                    "gptq_dequant_matmul");
}

size_t gptq_dequant_group_order_workspace_bytes(int64_t in) {
  if (in < 1) return 0;
  return dequant_group_order_workspace_bytes(in);
}

int gptq_dequant_group_order(const int32_t* qweight, const int32_t* g_idx, int64_t in,
                             int64_t out, int bits, int32_t* qweight_sorted,
                             int32_t* g_idx_sorted, int32_t* x_order, void* workspace,
                             size_t workspace_bytes, void* stream) {
  clear_error();
  if (!qweight || !g_idx) return fail(GPTQ_ERR_INVALID_ARG, "qweight or g_idx is NULL");
  if (!qweight_sorted || !g_idx_sorted || !x_order)
    return fail(GPTQ_ERR_INVALID_ARG, "qweight_sorted, g_idx_sorted or x_order is NULL");
  if (qweight_sorted == qweight)
    return fail(GPTQ_ERR_INVALID_ARG, "qweight_sorted must not alias qweight");
  if (in < 32 || in % 32 != 0)
    return fail(GPTQ_ERR_INVALID_ARG, "in must be a positive multiple of 32");
  if (out < 1) return fail(GPTQ_ERR_INVALID_ARG, "out must be >= 1");
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return fail(GPTQ_ERR_UNSUPPORTED, "bits must be 2, 3, 4 or 8");
  const size_t need = dequant_group_order_workspace_bytes(in);
  if (!workspace) return fail(GPTQ_ERR_INVALID_ARG, "workspace is NULL");
  if (workspace_bytes < need)
    return fail(GPTQ_ERR_WORKSPACE,
                "workspace smaller than gptq_dequant_group_order_workspace_bytes(in) = " +
                    std::to_string(need));
  return hip_status(run_dequant_group_order(qweight, g_idx, in, out, bits, qweight_sorted,
                                            g_idx_sorted, x_order, workspace,
                                            static_cast<hipStream_t>(stream)),
                    "gptq_dequant_group_order");
}

int gptq_silu_mul(const void* G, int64_t ldg, const void* U, int64_t ldu, int64_t rows,
                  int64_t cols, void* A, int64_t lda, void* stream) {
  clear_error();
  if (!G || !U || !A) return fail(GPTQ_ERR_INVALID_ARG, "G, U or A is NULL");
  if (rows < 0 || cols < 0) return fail(GPTQ_ERR_INVALID_ARG, "rows and cols must be >= 0");
  if (ldg < cols || ldu < cols || lda < cols)
    return fail(GPTQ_ERR_INVALID_ARG, "leading dimensions must be >= cols");
  if (rows == 0 || cols == 0) return GPTQ_OK;
  return hip_status(run_silu_mul(G, ldg, U, ldu, rows, cols, A, lda,
                                 static_cast<hipStream_t>(stream)),
                    "gptq_silu_mul");
}

int gptq_attention_forward(const void* Q, int64_t ldq, const void* K, int64_t ldk, const void* V,
                           int64_t ldv, void* O, int64_t ldo, int64_t seqs, int64_t seq_len,
                           int heads, int head_dim, int causal, void* stream) {
  clear_error();
  if (!Q || !K || !V || !O) return fail(GPTQ_ERR_INVALID_ARG, "Q, K, V or O is NULL");
  if (seqs < 0 || seq_len < 0) return fail(GPTQ_ERR_INVALID_ARG, "seqs and seq_len must be >= 0");
  if (heads < 1 || heads > 65535) return fail(GPTQ_ERR_INVALID_ARG, "heads must be in [1, 65535]");
  if (head_dim != 64 && head_dim != 128)
    return fail(GPTQ_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  const int64_t w = (int64_t)heads * head_dim;
  if (ldq < w || ldk < w || ldv < w || ldo < w)
    return fail(GPTQ_ERR_INVALID_ARG, "leading dimensions must be >= heads * head_dim");
  if (ldq % 8 || ldk % 8 || ldv % 8 || ldo % 8 ||
      ((reinterpret_cast<uintptr_t>(Q) | reinterpret_cast<uintptr_t>(K) |
        reinterpret_cast<uintptr_t>(V) | reinterpret_cast<uintptr_t>(O)) & 15))
    return fail(GPTQ_ERR_UNSUPPORTED,
                "Q, K, V, O must be 16-byte aligned with leading dimensions a multiple of 8");
  if (seqs > 65535) return fail(GPTQ_ERR_UNSUPPORTED, "seqs must be <= 65535 per call");
  if (seq_len > (int64_t)1 << 30) return fail(GPTQ_ERR_UNSUPPORTED, "seq_len must be <= 2^30");
  if (seqs == 0 || seq_len == 0) return GPTQ_OK;
  return hip_status(run_attention(Q, ldq, K, ldk, V, ldv, O, ldo, seqs, seq_len, heads, head_dim,
                                  causal ? 1 : 0, static_cast<hipStream_t>(stream)),
                    "gptq_attention_forward");
}

int gptq_residual_rmsnorm(const void* X, int64_t ldx, const void* A, int64_t lda,
                          const void* gamma, int64_t rows, int64_t d, float eps, void* Hs,
                          int64_t ldh, void* U, int64_t ldu, void* stream) {
  clear_error();
  if (!X || !A || !gamma || !Hs || !U)
    return fail(GPTQ_ERR_INVALID_ARG, "X, A, gamma, Hs or U is NULL");
  if (rows < 0 || d < 1) return fail(GPTQ_ERR_INVALID_ARG, "rows must be >= 0 and d >= 1");
  if (ldx < d || lda < d || ldh < d || ldu < d)
    return fail(GPTQ_ERR_INVALID_ARG, "leading dimensions must be >= d");
  if (!(eps >= 0.0f) || !std::isfinite(eps))
    return fail(GPTQ_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (rows == 0) return GPTQ_OK;
  return hip_status(run_residual_rmsnorm(X, ldx, A, lda, gamma, rows, d, eps, Hs, ldh, U, ldu,
                                         static_cast<hipStream_t>(stream)),
                    "gptq_residual_rmsnorm");
}

int gptq_export_params(const float* scales, const int32_t* zeros, int64_t n_groups, int64_t out,
                       int bits, void* scales_f16, int32_t* qzeros, void* stream) {
  clear_error();
  if (!scales || !zeros || !scales_f16 || !qzeros)
    return fail(GPTQ_ERR_INVALID_ARG, "scales, zeros, scales_f16 or qzeros is NULL");
  if (n_groups < 1 || out < 1) return fail(GPTQ_ERR_INVALID_ARG, "n_groups and out must be >= 1");
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return fail(GPTQ_ERR_UNSUPPORTED, "bits must be 2, 3, 4 or 8");
  if ((out * bits) % 32 != 0)
    return fail(GPTQ_ERR_UNSUPPORTED, "out * bits must be a multiple of 32");
  return hip_status(run_export(scales, zeros, n_groups, out, bits, scales_f16, qzeros,
                               static_cast<hipStream_t>(stream)),
                    "gptq_export_params");
}

int gptq_unpack_zeros(const int32_t* qzeros, int64_t n_groups, int64_t out, int bits,
                      int32_t* zeros, void* stream) {
  clear_error();
  if (!qzeros || !zeros) return fail(GPTQ_ERR_INVALID_ARG, "qzeros or zeros is NULL");
  if (n_groups < 1 || out < 1) return fail(GPTQ_ERR_INVALID_ARG, "n_groups and out must be >= 1");
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return fail(GPTQ_ERR_UNSUPPORTED, "bits must be 2, 3, 4 or 8");
  if ((out * bits) % 32 != 0)
    return fail(GPTQ_ERR_UNSUPPORTED, "out * bits must be a multiple of 32");
  return hip_status(run_unpack_zeros(qzeros, n_groups, out, bits, zeros,
                                     static_cast<hipStream_t>(stream)),
                    "gptq_unpack_zeros");
}

const char* gptq_status_string(int status) {
  switch (status) {
    case GPTQ_OK: return "GPTQ_OK";
    case GPTQ_ERR_INVALID_ARG: return "GPTQ_ERR_INVALID_ARG: invalid argument";
    case GPTQ_ERR_UNSUPPORTED: return "GPTQ_ERR_UNSUPPORTED: unsupported request";
    case GPTQ_ERR_WORKSPACE: return "GPTQ_ERR_WORKSPACE: workspace too small";
    case GPTQ_ERR_HIP: return "GPTQ_ERR_HIP: HIP runtime error";
    default: return "unknown gptq status";
  }
}

const char* gptq_last_error_message(void) { return gptq::last_error_c(); }

}  // extern "C"
