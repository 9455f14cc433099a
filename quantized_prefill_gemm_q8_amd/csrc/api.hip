// Host side of the C ABI declared in include/qgemm.h: argument checks,
// workspace carving and kernel dispatch.  No allocation, no global mutable
// state apart from a once-per-device architecture check and the trace switch
// read once from the environment.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "common.h"

namespace {

constexpr int64_t kMaxDevices = 64;

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int64_t padded_rows(int64_t M) { return (M + qg::kRowPad - 1) / qg::kRowPad * qg::kRowPad; }

// Byte offsets of the workspace sections, each 256-byte aligned.
struct Layout {
  int64_t Mp, q_off, dx_off, dxt_off, ds_off, dsp_off, total;
};

bool layout_for(int64_t M, int64_t K, Layout* L) {
  if (M < 1 || K < 256 || K % 256 != 0) return false;
  const int64_t Mp = padded_rows(M);
  // overflow guard: Mp*K and the scale arrays must fit comfortably in int64
  if (Mp > (INT64_C(1) << 40) / K) return false;
  L->Mp = Mp;
  L->q_off = 0;
  L->dx_off = Mp * K;                          // every section is a multiple of 256 bytes
  L->dxt_off = L->dx_off + Mp * (K / 32) * 4;
  L->ds_off = L->dxt_off + Mp * (K / 32) * 4;
  L->dsp_off = L->ds_off + Mp * (K / 32) * 4;
  L->total = L->dsp_off + Mp * (K / 32) * 3 * 2;
  return true;
}

// gfx950 check, cached per device (atomic so concurrent first calls are fine).
std::atomic<int> g_arch_ok[kMaxDevices];

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QG_EDEVICE;
  if (dev < 0 || dev >= kMaxDevices) return QG_EDEVICE;
  int st = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return QG_EDEVICE;
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? QG_OK : QG_EDEVICE;
}

int check_common(const void* W, int fmt, int64_t N, int64_t K) {
  if (!W) return QG_EINVAL;
  if (fmt != QG_Q4_K && fmt != QG_Q5_K && fmt != QG_Q6_K && fmt != QG_Q8_0) return QG_EFMT;
  if (N < 1 || K < 256 || K % 256 != 0) return QG_EINVAL;
  if (N > (INT64_C(1) << 40) / K) return QG_EINVAL;
  if (!aligned(W, 16)) return QG_EALIGN;
  return QG_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? QG_OK : QG_ELAUNCH; }

// QGEMM_TRACE=1 in the environment: one line on stderr per accepted GEMM call
// naming the entry point, the problem and the kernel it launches (which path
// a call took is otherwise invisible to the caller).
bool trace_on() {
  static const bool on = [] {
    const char* v = getenv("QGEMM_TRACE");
    return v != nullptr && v[0] != '\0' && strcmp(v, "0") != 0;
  }();
  return on;
}

const char* fmt_name(int fmt) {
  switch (fmt) {
    case QG_Q4_K: return "Q4_K";
    case QG_Q6_K: return "Q6_K";
    case QG_Q5_K: return "Q5_K";
    case QG_Q8_0: return "Q8_0";
    default: return "?";
  }
}

// (callers test trace_on() first, so the kernel-name lookup costs nothing
// when tracing is off)
void trace(const char* entry, int fmt, int64_t M, int64_t N, int64_t K, const char* path,
           const char* kernel) {
  fprintf(stderr, "qgemm: %s fmt=%s M=%lld N=%lld K=%lld path=%s kernel=%s\n", entry, fmt_name(fmt),
          static_cast<long long>(M), static_cast<long long>(N), static_cast<long long>(K), path,
          kernel ? kernel : "?");
}

// The tiled kernels of each format.
hipError_t launch_tiled(const uint8_t* W, int fmt, const QgWorkspace& ws, int64_t M, int64_t N, int64_t K,
                        float* y, hipStream_t s) {
  if (fmt == QG_Q4_K) return qg_launch_gemm_q4k(W, ws, M, N, K, y, s);
  if (fmt == QG_Q5_K) return qg_launch_gemm_q5k(W, ws, M, N, K, y, s);
  if (fmt == QG_Q8_0) return qg_launch_gemm_q80(W, ws, M, N, K, y, s);
  return qg_launch_gemm_q6k(W, ws, M, N, K, y, s);
}

// QG_PATH_AUTO: the skinny kernel for Q6_K and Q8_0 problems of M <= 8 rows
// (ahead of their tiled kernels up to 8 rows).  For Q4_K and Q5_K the
// small-grid kernel takes over from a row count that depends on the shape,
// measured on cold weights (each call reading them from HBM) over the decode
// projections 1024->4096, 1024->7168, 3584->1024, 2560->9728, 9728->2560 and
// 4096->24576: the small-grid kernel runs one wavefront per 32 weight rows
// and K-group, so few weight rows leave it short of wavefronts (N <= 1024:
// skinny up to 8 rows); the skinny kernel's per-row work grows with M, most
// at K <= 1024 where a wavefront decodes four weight rows per step (skinny up
// to 4 rows for N <= 4096, 2 above); otherwise up to 6 rows for N <= 12288
// and 4 above.
bool auto_skinny(int fmt, int64_t M, int64_t N, int64_t K) {
  if (fmt == QG_Q6_K || fmt == QG_Q8_0) return M <= QG_SKINNY_MAX_M;
  int64_t mmax;
  if (N <= 1024) mmax = 8;
  else if (K <= 1024) mmax = N <= 4096 ? 4 : 2;
  else mmax = N <= 12288 ? 6 : 4;
  return M <= mmax;
}

}  // namespace

extern "C" {

size_t qgemm_workspace_bytes(int64_t M, int64_t K) {
  Layout L;
  if (!layout_for(M, K, &L)) return 0;
  return static_cast<size_t>(L.total);
}

static QgWorkspace carve(void* workspace, const Layout& L) {
  uint8_t* base = static_cast<uint8_t*>(workspace);
  QgWorkspace ws;
  ws.q = reinterpret_cast<int8_t*>(base + L.q_off);
  ws.dx = reinterpret_cast<float*>(base + L.dx_off);
  ws.dxT = reinterpret_cast<float*>(base + L.dxt_off);
  ws.dS = reinterpret_cast<float*>(base + L.ds_off);
  ws.dsp = reinterpret_cast<uint16_t*>(base + L.dsp_off);
  ws.Mp = L.Mp;
  return ws;
}

static int check_workspace(const void* workspace, size_t workspace_bytes, const Layout& L) {
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < static_cast<size_t>(L.total))
    return QG_EWORKSPACE;
  return QG_OK;
}

int qgemm_quantize_workspace(const void* x, int x_dtype, int64_t M, int64_t K, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!x || M < 1) return QG_EINVAL;
  if (x_dtype != QG_F32 && x_dtype != QG_BF16) return QG_EDTYPE;
  Layout L;
  if (!layout_for(M, K, &L)) return QG_EINVAL;
  int rc = check_workspace(workspace, workspace_bytes, L);
  if (rc) return rc;
  if (!aligned(x, 16)) return QG_EALIGN;
  rc = check_device();
  if (rc) return rc;
  const QgWorkspace ws = carve(workspace, L);
  return launch_status(qg_launch_act_quant_ws(x, x_dtype, M, K, ws, static_cast<hipStream_t>(stream)));
}

int qgemm_gemm_quantized(const void* q_weights, int fmt, const void* workspace,
                         size_t workspace_bytes, int64_t M, int64_t N, int64_t K, float* y,
                         void* stream, int path) {
  int rc = check_common(q_weights, fmt, N, K);
  if (rc) return rc;
  if (!y || M < 1) return QG_EINVAL;
  if (path != QG_PATH_AUTO && path != QG_PATH_TILED && path != QG_PATH_SKINNY) return QG_EINVAL;
  if (path == QG_PATH_SKINNY && M > QG_SKINNY_MAX_M) return QG_EINVAL;
  Layout L;
  if (!layout_for(M, K, &L)) return QG_EINVAL;
  if (M > (INT64_C(1) << 40) / N) return QG_EINVAL;
  rc = check_workspace(workspace, workspace_bytes, L);
  if (rc) return rc;
  if (!aligned(y, 16)) return QG_EALIGN;
  rc = check_device();
  if (rc) return rc;
  const QgWorkspace ws = carve(const_cast<void*>(workspace), L);
  const bool skinny = path == QG_PATH_SKINNY || (path == QG_PATH_AUTO && auto_skinny(fmt, M, N, K));
  const uint8_t* W = static_cast<const uint8_t*>(q_weights);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (trace_on())
    trace("gemm", fmt, M, N, K, skinny ? "skinny" : "tiled",
        qgemm_kernel_name(fmt, M, N, K, skinny ? QG_PATH_SKINNY : QG_PATH_TILED));
  if (skinny) return launch_status(qg_launch_gemm_skinny(W, fmt, ws, M, N, K, y, s));
  return launch_status(launch_tiled(W, fmt, ws, M, N, K, y, s));
}

int qgemm_prefill_ex(const void* q_weights, int fmt, const void* x, int x_dtype, int64_t M,
                     int64_t N, int64_t K, float* y, void* workspace, size_t workspace_bytes,
                     void* stream, int path) {
  // validate everything the GEMM half checks before launching the quantiser
  int rc = check_common(q_weights, fmt, N, K);
  if (rc) return rc;
  if (!x || !y || M < 1) return QG_EINVAL;
  if (x_dtype != QG_F32 && x_dtype != QG_BF16) return QG_EDTYPE;
  if (path != QG_PATH_AUTO && path != QG_PATH_TILED && path != QG_PATH_SKINNY) return QG_EINVAL;
  if (path == QG_PATH_SKINNY && M > QG_SKINNY_MAX_M) return QG_EINVAL;
  Layout L;
  if (!layout_for(M, K, &L)) return QG_EINVAL;
  if (M > (INT64_C(1) << 40) / N) return QG_EINVAL;
  rc = check_workspace(workspace, workspace_bytes, L);
  if (rc) return rc;
  if (!aligned(x, 16) || !aligned(y, 16)) return QG_EALIGN;
  rc = qgemm_quantize_workspace(x, x_dtype, M, K, workspace, workspace_bytes, stream);
  if (rc) return rc;
  return qgemm_gemm_quantized(q_weights, fmt, workspace, workspace_bytes, M, N, K, y, stream, path);
}

int qgemm_prefill(const void* q_weights, int fmt, const void* x, int x_dtype, int64_t M,
                  int64_t N, int64_t K, float* y, void* workspace, size_t workspace_bytes,
                  void* stream) {
  return qgemm_prefill_ex(q_weights, fmt, x, x_dtype, M, N, K, y, workspace, workspace_bytes,
                          stream, QG_PATH_AUTO);
}

int qgemm_lm_head(const void* q_weights, int fmt, const void* x_row, int x_dtype, int64_t N,
                  int64_t K, float* y, void* workspace, size_t workspace_bytes, void* stream) {
  return qgemm_prefill_ex(q_weights, fmt, x_row, x_dtype, 1, N, K, y, workspace, workspace_bytes,
                          stream, QG_PATH_AUTO);
}

const char* qgemm_kernel_name(int fmt, int64_t M, int64_t N, int64_t K, int path) {
  if (fmt != QG_Q4_K && fmt != QG_Q5_K && fmt != QG_Q6_K && fmt != QG_Q8_0) return NULL;
  if (M < 1 || N < 1 || K < 256 || K % 256 != 0) return NULL;
  if (path != QG_PATH_AUTO && path != QG_PATH_TILED && path != QG_PATH_SKINNY) return NULL;
  if (path == QG_PATH_SKINNY && M > QG_SKINNY_MAX_M) return NULL;
  const bool skinny = path == QG_PATH_SKINNY || (path == QG_PATH_AUTO && auto_skinny(fmt, M, N, K));
  if (skinny) return qg_gemm_skinny_kernel_name(fmt, M, N, K);
  if (fmt == QG_Q5_K) return qg_gemm_q5k_kernel_name(M, N, K);
  if (fmt == QG_Q8_0) return qg_gemm_q80_kernel_name(M, N, K);
  return fmt == QG_Q4_K ? qg_gemm_q4k_kernel_name(M, N, K) : qg_gemm_q6k_kernel_name(M, N, K);
}

const char* qgemm_strerror(int code) {
  switch (code) {
    case QG_OK: return "success";
    case QG_EINVAL: return "invalid argument (null pointer, size < 1, K not a multiple of 256, size overflow or bad path)";
    case QG_EFMT: return "unsupported weight format (QG_Q4_K, QG_Q5_K, QG_Q6_K, QG_Q8_0; the per-256 entry points take Q4_K only, the fp16 branch Q4_K and Q6_K)";
    case QG_EDTYPE: return "unsupported activation type (expected QG_F32 or QG_BF16)";
    case QG_EWORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case QG_EALIGN: return "pointer not 16-byte aligned";
    case QG_ELAUNCH: return "kernel launch failed";
    case QG_EDEVICE: return "current device is not a gfx950 (MI355X) GPU";
    case QG_ENOSCRATCH: return "problem too large for qgemm_prefill_noalloc's static scratch (QG_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown error code";
  }
}

int qgemm_quantize_act(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* q, float* d,
                       int32_t* S, void* stream) {
  if (!x || !q || !d || !S || M < 1 || K < 32 || K % 32 != 0) return QG_EINVAL;
  if (M > (INT64_C(1) << 40) / K) return QG_EINVAL;
  if (x_dtype != QG_F32 && x_dtype != QG_BF16) return QG_EDTYPE;
  if (!aligned(x, 16) || !aligned(q, 8) || !aligned(d, 4) || !aligned(S, 4)) return QG_EALIGN;
  int rc = check_device();
  if (rc) return rc;
  return launch_status(qg_launch_act_quant_hook(x, x_dtype, M, K, q, d, S,
                                                static_cast<hipStream_t>(stream)));
}

int qgemm_dequant(const void* q_weights, int fmt, int64_t N, int64_t K, float* w, void* stream) {
  int rc = check_common(q_weights, fmt, N, K);
  if (rc) return rc;
  if (!w) return QG_EINVAL;
  rc = check_device();
  if (rc) return rc;
  return launch_status(qg_launch_dequant(static_cast<const uint8_t*>(q_weights), fmt, N, K, w,
                                         static_cast<hipStream_t>(stream)));
}

int qgemm_block_partials(const void* q_weights, int fmt, const int8_t* qx, int64_t M, int64_t N,
                         int64_t K, int32_t* out, void* stream) {
  int rc = check_common(q_weights, fmt, N, K);
  if (rc) return rc;
  if (!qx || !out || M < 1) return QG_EINVAL;
  if (M > (INT64_C(1) << 34) / N / (K / 16)) return QG_EINVAL;
  if (!aligned(qx, 16)) return QG_EALIGN;
  rc = check_device();
  if (rc) return rc;
  return launch_status(qg_launch_block_partials(static_cast<const uint8_t*>(q_weights), fmt, qx,
                                                M, N, K, out, static_cast<hipStream_t>(stream)));
}

// ---- per-256 activation scales ----

int qgemm_quantize_workspace_a256(const void* x, int x_dtype, int64_t M, int64_t K, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (!x || M < 1) return QG_EINVAL;
  if (x_dtype != QG_F32 && x_dtype != QG_BF16) return QG_EDTYPE;
  Layout L;
  if (!layout_for(M, K, &L)) return QG_EINVAL;
  int rc = check_workspace(workspace, workspace_bytes, L);
  if (rc) return rc;
  if (!aligned(x, 16)) return QG_EALIGN;
  rc = check_device();
  if (rc) return rc;
  const QgWorkspace ws = carve(workspace, L);
  return launch_status(qg_launch_act_quant256_ws(x, x_dtype, M, K, ws, static_cast<hipStream_t>(stream)));
}

int qgemm_gemm_quantized_a256(const void* q_weights, int fmt, const void* workspace,
                              size_t workspace_bytes, int64_t M, int64_t N, int64_t K, float* y,
                              void* stream) {
  int rc = check_common(q_weights, fmt, N, K);
  if (rc) return rc;
  if (fmt != QG_Q4_K) return QG_EFMT;
  if (!y || M < 1) return QG_EINVAL;
  Layout L;
  if (!layout_for(M, K, &L)) return QG_EINVAL;
  if (M > (INT64_C(1) << 40) / N) return QG_EINVAL;
  rc = check_workspace(workspace, workspace_bytes, L);
  if (rc) return rc;
  if (!aligned(y, 16)) return QG_EALIGN;
  rc = check_device();
  if (rc) return rc;
  const QgWorkspace ws = carve(const_cast<void*>(workspace), L);
  const uint8_t* W = static_cast<const uint8_t*>(q_weights);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (trace_on())
    trace("gemm_a256", fmt, M, N, K, auto_skinny(fmt, M, N, K) ? "skinny" : "tiled",
        qgemm_kernel_name_a256(fmt, M, N, K));
  // the skinny and small-grid kernels read the per-block scales, which the
  // per-256 workspace holds too
  if (auto_skinny(fmt, M, N, K)) return launch_status(qg_launch_gemm_skinny(W, fmt, ws, M, N, K, y, s));
  return launch_status(qg_launch_gemm_q4k(W, ws, M, N, K, y, s, true));
}

int qgemm_prefill_a256(const void* q_weights, int fmt, const void* x, int x_dtype, int64_t M,
                       int64_t N, int64_t K, float* y, void* workspace, size_t workspace_bytes,
                       void* stream) {
  int rc = check_common(q_weights, fmt, N, K);
  if (rc) return rc;
  if (fmt != QG_Q4_K) return QG_EFMT;
  if (!x || !y || M < 1) return QG_EINVAL;
  if (x_dtype != QG_F32 && x_dtype != QG_BF16) return QG_EDTYPE;
  Layout L;
  if (!layout_for(M, K, &L)) return QG_EINVAL;
  if (M > (INT64_C(1) << 40) / N) return QG_EINVAL;
  rc = check_workspace(workspace, workspace_bytes, L);
  if (rc) return rc;
  if (!aligned(x, 16) || !aligned(y, 16)) return QG_EALIGN;
  rc = qgemm_quantize_workspace_a256(x, x_dtype, M, K, workspace, workspace_bytes, stream);
  if (rc) return rc;
  return qgemm_gemm_quantized_a256(q_weights, fmt, workspace, workspace_bytes, M, N, K, y, stream);
}

const char* qgemm_kernel_name_a256(int fmt, int64_t M, int64_t N, int64_t K) {
  if (fmt != QG_Q4_K || M < 1 || N < 1 || K < 256 || K % 256 != 0) return NULL;
  if (auto_skinny(fmt, M, N, K)) return qg_gemm_skinny_kernel_name(fmt, M, N, K);
  return qg_gemm_q4k_kernel_name(M, N, K, true);
}

int qgemm_quantize_act_a256(const void* x, int x_dtype, int64_t M, int64_t K, int8_t* q, float* d,
                            int32_t* S, void* stream) {
  if (!x || !q || !d || !S || M < 1 || K < 256 || K % 256 != 0) return QG_EINVAL;
  if (M > (INT64_C(1) << 40) / K) return QG_EINVAL;
  if (x_dtype != QG_F32 && x_dtype != QG_BF16) return QG_EDTYPE;
  if (!aligned(x, 16) || !aligned(q, 8) || !aligned(d, 4) || !aligned(S, 4)) return QG_EALIGN;
  int rc = check_device();
  if (rc) return rc;
  return launch_status(qg_launch_act_quant256_hook(x, x_dtype, M, K, q, d, S,
                                                   static_cast<hipStream_t>(stream)));
}

// ---- the dequantise-to-fp16 branch ----

size_t qgemm_deq_f16_workspace_bytes(int64_t M, int64_t K) {
  if (M < 1 || K < 256 || K % 256 != 0 || M > (INT64_C(1) << 39) / K) return 0;  // 2*M*K <= 2^40
  return static_cast<size_t>((M * K * 2 + 255) / 256 * 256);
}

int qgemm_to_f16(const void* x, int x_dtype, int64_t M, int64_t K, uint16_t* x16, void* stream) {
  if (!x || !x16 || M < 1 || K < 8 || K % 8 != 0) return QG_EINVAL;
  if (M > (INT64_C(1) << 40) / K) return QG_EINVAL;
  if (x_dtype != QG_F32 && x_dtype != QG_BF16) return QG_EDTYPE;
  if (!aligned(x, 16) || !aligned(x16, 16)) return QG_EALIGN;
  int rc = check_device();
  if (rc) return rc;
  return launch_status(qg_launch_to_f16(x, x_dtype, M, K, x16, static_cast<hipStream_t>(stream)));
}

int qgemm_dequant_f16(const void* q_weights, int fmt, int64_t N, int64_t K, uint16_t* w16,
                      void* stream) {
  if (fmt == QG_Q5_K || fmt == QG_Q8_0) return QG_EFMT;
  int rc = check_common(q_weights, fmt, N, K);
  if (rc) return rc;
  if (!w16) return QG_EINVAL;
  if (!aligned(w16, 16)) return QG_EALIGN;
  rc = check_device();
  if (rc) return rc;
  return launch_status(qg_launch_dequant_f16(static_cast<const uint8_t*>(q_weights), fmt, N, K, w16,
                                             static_cast<hipStream_t>(stream)));
}

int qgemm_prefill_deq_f16(const void* q_weights, int fmt, const void* x, int x_dtype, int64_t M,
                          int64_t N, int64_t K, float* y, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (fmt == QG_Q5_K || fmt == QG_Q8_0) return QG_EFMT;
  int rc = check_common(q_weights, fmt, N, K);
  if (rc) return rc;
  if (!x || !y || M < 1) return QG_EINVAL;
  if (x_dtype != QG_F32 && x_dtype != QG_BF16) return QG_EDTYPE;
  const size_t need = qgemm_deq_f16_workspace_bytes(M, K);
  if (need == 0 || M > (INT64_C(1) << 40) / N) return QG_EINVAL;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need) return QG_EWORKSPACE;
  if (!aligned(x, 16) || !aligned(y, 16)) return QG_EALIGN;
  rc = check_device();
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (trace_on())
    trace("prefill_deq_f16", fmt, M, N, K, "f16", qgemm_deq_f16_kernel_name(fmt, M, N, K));
  uint16_t* x16 = static_cast<uint16_t*>(workspace);
  rc = launch_status(qg_launch_to_f16(x, x_dtype, M, K, x16, s));
  if (rc) return rc;
  return launch_status(qg_launch_gemm_deq_f16(static_cast<const uint8_t*>(q_weights), fmt, x16, M, N, K,
                                              y, s));
}

const char* qgemm_deq_f16_kernel_name(int fmt, int64_t M, int64_t N, int64_t K) {
  if ((fmt != QG_Q4_K && fmt != QG_Q6_K) || M < 1 || N < 1 || K < 256 || K % 256 != 0) return NULL;
  return qg_gemm_deq_f16_kernel_name(fmt, M, N, K);
}

// ---- fusions either side of the GEMM: RMSNorm -> quantiser, SwiGLU epilogue ----

static int check_rms(const void* x, int x_dtype, const float* g, float eps, int64_t M, int64_t K) {
  if (!x || !g || M < 1 || M > INT64_C(0x7FFFFFFF)) return QG_EINVAL;  // one workgroup per row
  if (x_dtype != QG_F32 && x_dtype != QG_BF16) return QG_EDTYPE;
  if (K < 256 || K % 256 != 0 || K > kRmsMaxK) return QG_EINVAL;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return QG_EINVAL;  // NaN, negative or infinite eps
  if (!aligned(x, 16) || !aligned(g, 16)) return QG_EALIGN;
  return QG_OK;
}

int qgemm_rmsnorm_quantize_workspace(const void* x, int x_dtype, const float* g, float eps, int64_t M,
                                     int64_t K, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_rms(x, x_dtype, g, eps, M, K);
  if (rc) return rc;
  Layout L;
  if (!layout_for(M, K, &L)) return QG_EINVAL;
  rc = check_workspace(workspace, workspace_bytes, L);
  if (rc) return rc;
  rc = check_device();
  if (rc) return rc;
  const QgWorkspace ws = carve(workspace, L);
  return launch_status(qg_launch_rmsnorm_quant_ws(x, x_dtype, g, eps, M, K, ws, static_cast<hipStream_t>(stream)));
}

int qgemm_rmsnorm_quantize_act(const void* x, int x_dtype, const float* g, float eps, int64_t M, int64_t K,
                               int8_t* q, float* d, int32_t* S, void* stream) {
  int rc = check_rms(x, x_dtype, g, eps, M, K);
  if (rc) return rc;
  if (!q || !d || !S) return QG_EINVAL;
  if (M > (INT64_C(1) << 40) / K) return QG_EINVAL;
  if (!aligned(q, 8) || !aligned(d, 4) || !aligned(S, 4)) return QG_EALIGN;
  rc = check_device();
  if (rc) return rc;
  return launch_status(qg_launch_rmsnorm_quant_hook(x, x_dtype, g, eps, M, K, q, d, S,
                                                    static_cast<hipStream_t>(stream)));
}

// The gate+up GEMM with the SwiGLU epilogue runs fused for Q4_K, Q5_K and Q8_0
// weights on the LDS-tiled kernels; otherwise the plain GEMM writes the fp32 gate+up output
// into the workspace after the quantised activations and the SwiGLU kernel
// reads it from there.
static bool swiglu_fused(int fmt, int64_t M, int64_t F, int64_t K) {
  return fmt != QG_Q6_K && !auto_skinny(fmt, M, 2 * F, K) && qg_swiglu_fusable(fmt, M, F, K);
}

static bool swiglu_layout(int fmt, int64_t M, int64_t F, int64_t K, Layout* L, int64_t* total) {
  if (F < 1 || F > (INT64_C(1) << 39) / K) return false;  // 2F * K <= 2^40
  if (!layout_for(M, K, L)) return false;
  if (M > (INT64_C(1) << 38) / F) return false;             // M * 2F * 4 bytes <= 2^41
  *total = L->total + (swiglu_fused(fmt, M, F, K) ? 0 : (M * 2 * F * 4 + 255) / 256 * 256);
  return true;
}

size_t qgemm_swiglu_workspace_bytes(int fmt, int64_t M, int64_t F, int64_t K) {
  if (fmt != QG_Q4_K && fmt != QG_Q5_K && fmt != QG_Q6_K && fmt != QG_Q8_0) return 0;
  Layout L;
  int64_t total;
  if (!swiglu_layout(fmt, M, F, K, &L, &total)) return 0;
  return static_cast<size_t>(total);
}

int qgemm_gemm_quantized_swiglu(const void* q_weights, int fmt, const void* workspace,
                                size_t workspace_bytes, int64_t M, int64_t F, int64_t K, uint16_t* h,
                                void* stream) {
  if (F < 1 || F > (INT64_C(1) << 39) / 256) return QG_EINVAL;
  int rc = check_common(q_weights, fmt, 2 * F, K);
  if (rc) return rc;
  if (!h || M < 1) return QG_EINVAL;
  Layout L;
  int64_t total;
  if (!swiglu_layout(fmt, M, F, K, &L, &total)) return QG_EINVAL;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < static_cast<size_t>(total)) return QG_EWORKSPACE;
  if (!aligned(h, 16)) return QG_EALIGN;
  rc = check_device();
  if (rc) return rc;
  const QgWorkspace ws = carve(const_cast<void*>(workspace), L);
  const uint8_t* W = static_cast<const uint8_t*>(q_weights);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (trace_on())
    trace("gemm_swiglu", fmt, M, 2 * F, K, swiglu_fused(fmt, M, F, K) ? "fused" : "gemm+swiglu",
        qgemm_kernel_name_swiglu(fmt, M, F, K));
  if (swiglu_fused(fmt, M, F, K)) return launch_status(qg_launch_gemm_swiglu(W, fmt, ws, M, F, K, h, s));
  float* y = reinterpret_cast<float*>(static_cast<uint8_t*>(const_cast<void*>(workspace)) + L.total);
  if (auto_skinny(fmt, M, 2 * F, K)) rc = launch_status(qg_launch_gemm_skinny(W, fmt, ws, M, 2 * F, K, y, s));
  else rc = launch_status(launch_tiled(W, fmt, ws, M, 2 * F, K, y, s));
  if (rc) return rc;
  return launch_status(qg_launch_swiglu(y, M, F, h, s));
}

int qgemm_prefill_swiglu(const void* q_weights, int fmt, const void* x, int x_dtype, int64_t M, int64_t F,
                         int64_t K, uint16_t* h, void* workspace, size_t workspace_bytes, void* stream) {
  // validate everything the GEMM half checks before launching the quantiser
  if (F < 1 || F > (INT64_C(1) << 39) / 256) return QG_EINVAL;
  int rc = check_common(q_weights, fmt, 2 * F, K);
  if (rc) return rc;
  if (!x || !h || M < 1) return QG_EINVAL;
  if (x_dtype != QG_F32 && x_dtype != QG_BF16) return QG_EDTYPE;
  Layout L;
  int64_t total;
  if (!swiglu_layout(fmt, M, F, K, &L, &total)) return QG_EINVAL;
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < static_cast<size_t>(total)) return QG_EWORKSPACE;
  if (!aligned(x, 16) || !aligned(h, 16)) return QG_EALIGN;
  rc = qgemm_quantize_workspace(x, x_dtype, M, K, workspace, workspace_bytes, stream);
  if (rc) return rc;
  return qgemm_gemm_quantized_swiglu(q_weights, fmt, workspace, workspace_bytes, M, F, K, h, stream);
}

const char* qgemm_kernel_name_swiglu(int fmt, int64_t M, int64_t F, int64_t K) {
  if ((fmt != QG_Q4_K && fmt != QG_Q5_K && fmt != QG_Q6_K && fmt != QG_Q8_0) || M < 1 || F < 1 || K < 256 || K % 256 != 0)
    return NULL;
  if (F > (INT64_C(1) << 39) / K) return NULL;
  if (swiglu_fused(fmt, M, F, K)) return qg_gemm_swiglu_kernel_name(fmt, M, F, K);
  return qgemm_kernel_name(fmt, M, 2 * F, K, QG_PATH_AUTO);
}

int qgemm_swiglu(const float* y, int64_t M, int64_t F, uint16_t* h, void* stream) {
  if (!y || !h || M < 1 || F < 1 || M > (INT64_C(1) << 38) / F) return QG_EINVAL;
  if (!aligned(y, 16) || !aligned(h, 16)) return QG_EALIGN;
  int rc = check_device();
  if (rc) return rc;
  return launch_status(qg_launch_swiglu(y, M, F, h, static_cast<hipStream_t>(stream)));
}

// ---- diagnostics ----

int qgemm_test_plant_delay(int kernel, int sleeps) {
  if (kernel != QG_PLANT_QUANTIZE || sleeps < 0 || sleeps > QG_PLANT_MAX_SLEEPS) return QG_EINVAL;
  qg_set_planted_quant_sleeps(sleeps);
  return QG_OK;
}

int qgemm_sclk_probe(uint64_t* ticks, int iters, void* stream) {
  if (!ticks || iters < 1 || iters > (1 << 24)) return QG_EINVAL;
  if (!aligned(ticks, 8)) return QG_EALIGN;
  int rc = check_device();
  if (rc) return rc;
  return launch_status(qg_launch_sclk_probe(ticks, iters, static_cast<hipStream_t>(stream)));
}

int qgemm_read_probe(const void* src, int64_t bytes, void* stream) {
  if (bytes < 0 || bytes % 16 != 0 || (bytes > 0 && !src)) return QG_EINVAL;
  if (!aligned(src, 16)) return QG_EALIGN;
  int rc = check_device();
  if (rc) return rc;
  return launch_status(qg_launch_read_probe(src, bytes, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
