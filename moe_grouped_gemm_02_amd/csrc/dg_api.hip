// C ABI of libdg: argument validation, error reporting, CU-count control and
// dispatch to the gfx950 kernels.  Every check that can be made on the host
// is made before anything is enqueued; nothing here allocates device memory
// or synchronises the host.

#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "dg.h"
#include "dg_internal.h"

namespace {

thread_local char g_last_error[512] = "";
std::atomic<int> g_num_cus_override{0};

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_last_error[0] = '\0';
  return DG_SUCCESS;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// count * stride * elem < lim, for count, stride >= 0 and elem, lim > 0,
// decided without forming the product (strides come from the caller).
bool below(int64_t count, int64_t stride, int64_t elem, int64_t lim) {
  if (count == 0 || stride == 0) return true;
  return stride <= (lim - 1) / elem / count;
}

int env_num_cus() {
  const char* s = getenv("DG_NUM_CUS");
  if (!s || !*s) return 0;
  const int v = atoi(s);
  return v > 0 ? (v < 4096 ? v : 4096) : 0;
}

// CU count the persistent schedule is sized to; negative on failure.
int resolve_num_cus() {
  const int forced = g_num_cus_override.load();
  if (forced > 0) return forced;
  const int env = env_num_cus();
  if (env > 0) return env;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DG_ERR_HIP;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return DG_ERR_HIP;
  return cus;
}

bool debug_enabled() {
  const char* s = getenv("DG_DEBUG");
  return s && *s && strcmp(s, "0") != 0;
}

const char* layout_name(int layout) {
  switch (layout) {
    case dg::kDense: return "dense";
    case dg::kContiguous: return "contiguous";
    case dg::kMasked: return "masked";
    default: return "k_grouped";
  }
}

// Shared checks for the three GEMM entry points.  rows = the rows of the
// layout's row space (M, M_total or M_max).
int check_gemm_common(const uint8_t* a, const void* sfa, const uint8_t* b, const void* sfb,
                      const uint16_t* d, int rows, int n, int k, int64_t lda, int64_t ldb,
                      int64_t ldd, int64_t ld_sfa) {
  if (rows < 0 || n < 0 || k < 0) return fail(DG_ERR_INVALID_VALUE, "negative dimension (m=%d n=%d k=%d)", rows, n, k);
  if (k % 128 != 0) return fail(DG_ERR_UNSUPPORTED_SHAPE, "k=%d is not a multiple of 128", k);
  // With k == 0 nothing of A, B or the scales is read, so only d must be valid.
  if (!d || (k > 0 && (!a || !sfa || !b || !sfb)))
    return fail(DG_ERR_INVALID_VALUE, "null pointer argument");
  if (!aligned16(a) || !aligned16(b) || !aligned16(d) || !aligned16(sfa) || !aligned16(sfb))
    return fail(DG_ERR_MISALIGNED, "a, b, d, sfa and sfb must be 16-byte aligned");
  if (lda < k || ldb < k) return fail(DG_ERR_INVALID_VALUE, "lda/ldb smaller than k");
  if (ldd < n) return fail(DG_ERR_INVALID_VALUE, "ldd smaller than n");
  if (lda % 16 || ldb % 16) return fail(DG_ERR_MISALIGNED, "lda and ldb must be multiples of 16 bytes");
  if (ldd % 8) return fail(DG_ERR_MISALIGNED, "ldd must be a multiple of 8 elements");
  if (ld_sfa < rows || ld_sfa < 4) return fail(DG_ERR_INVALID_VALUE, "ld_sfa=%lld smaller than rows (%d) or 4", (long long)ld_sfa, rows);
  if (ld_sfa % 4) return fail(DG_ERR_MISALIGNED, "ld_sfa must be a multiple of 4");
  // The kernels address each operand (per group) with 32-bit byte offsets.
  const int64_t lim = (int64_t)1 << 32;
  if (!below(rows, lda, 1, lim) || !below(n, ldb, 1, lim) || !below(k / 128, ld_sfa, 4, lim))
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "operand of 4 GiB or more (per group)");
  return DG_SUCCESS;
}

int check_workspace(const dg::GemmConfig& cfg, int layout, int rows, int n, int groups,
                    void* ws, size_t ws_bytes) {
  const size_t need = dg::workspace_bytes_for(cfg, layout, rows, n, groups);
  if (need == 0) return DG_SUCCESS;
  if (!ws || ws_bytes < need)
    return fail(DG_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  if (!aligned16(ws)) return fail(DG_ERR_MISALIGNED, "workspace must be 16-byte aligned");
  return DG_SUCCESS;
}

int run_gemm(int layout, dg::GemmParams& p, int rows, int groups, void* ws, size_t ws_bytes,
             void* stream, int expected_m = 0) {
  if (!dg::plannable(layout, rows, p.n, groups))
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "too many output tiles (m=%d n=%d groups=%d)", rows, p.n, groups);
  const int cus = resolve_num_cus();
  if (cus < 0) return fail(DG_ERR_HIP, "cannot query the device's compute-unit count");
  const bool qout = p.dq != nullptr;
  const bool narrow_ok = !p.sf_ue8m0 && !p.majors && layout != dg::kKGrouped;
  const dg::GemmConfig cfg = dg::choose_config(layout, rows, p.n, p.k, groups, cus, expected_m, qout, narrow_ok);
  if (layout == dg::kKGrouped && !dg::kgrouped_variant_built(cfg.variant))
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "tile variant %d is not built for the K-grouped layout", cfg.variant);
  if (p.majors && !dg::majors_variant_built(cfg.variant))
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "tile variant %d is not built for MN-major operands", cfg.variant);
  if (p.sf_ue8m0 && !dg::ue8m0_variant_built(cfg.variant))
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "tile variant %d is not built for UE8M0 scales", cfg.variant);
  if (qout && !dg::variant_quantises_output(cfg.variant))
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "tile variant %d cannot quantise its output (columns not whole 128-blocks)",
                cfg.variant);
  int st = check_workspace(cfg, layout, rows, p.n, groups, ws, ws_bytes);
  if (st != DG_SUCCESS) return st;
  p.workspace = static_cast<float*>(ws);
  p.counters = nullptr;
  if (debug_enabled())
    fprintf(stderr, "[dg] %s m=%d n=%d k=%d groups=%d: bm=%d bn=%d stream_k=%d grid=%d tiles=%d variant=%d cus=%d\n",
            layout_name(layout), rows, p.n, p.k, groups, cfg.bm, cfg.bn, cfg.stream_k, cfg.grid,
            cfg.tiles, cfg.variant, cus);
  const hipError_t e = dg::launch_gemm(layout, p, cfg, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DG_ERR_HIP, "GEMM launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Optional quantised copy of the output (the *_qout entry points).
struct QOut {
  uint8_t* dq;
  void* dsf;
  int64_t ld_dsf;
  bool ue8m0;  // exponent-byte output scales
};

// Checks of the quantised-output arguments; rows = the rows of one group.
int check_qout(const QOut* q, int rows, int n, int groups) {
  if (!q) return DG_SUCCESS;
  if (!q->dq || !q->dsf) return fail(DG_ERR_INVALID_VALUE, "null dq or dsf");
  if (!aligned16(q->dq) || !aligned16(q->dsf)) return fail(DG_ERR_MISALIGNED, "dq and dsf must be 16-byte aligned");
  if (n % 128) return fail(DG_ERR_UNSUPPORTED_SHAPE, "n=%d is not a multiple of 128 (quantised output)", n);
  if (q->ld_dsf < rows || q->ld_dsf < 4) return fail(DG_ERR_INVALID_VALUE, "ld_dsf smaller than the rows or 4");
  if (q->ld_dsf % 4) return fail(DG_ERR_MISALIGNED, "ld_dsf must be a multiple of 4");
  if ((int64_t)rows * n > (((int64_t)1 << 40) - 1) / groups) return fail(DG_ERR_UNSUPPORTED_SHAPE, "quantised output too large");
  if (!below((int64_t)groups * (n / 128), q->ld_dsf, 4, (int64_t)1 << 40))
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "output scales too large");
  return DG_SUCCESS;
}

void set_qout(dg::GemmParams& p, const QOut* q, int rows, int n) {
  if (!q) return;
  p.dq = q->dq;
  p.dsf = static_cast<float*>(q->dsf);
  p.dq_ue8m0 = q->ue8m0 ? 1 : 0;
  p.ld_dsf = q->ld_dsf;
  p.dq_gstride = (int64_t)rows * n;
  p.dsf_gstride = (int64_t)(n / 128) * q->ld_dsf;
}

// Scale-format fields of GemmParams.  fp32: weight scales [G][ceil(N/128)][K/128].
// UE8M0: exponent bytes, weights MN-major [G][K/128][ld_sfb].
void set_scales(dg::GemmParams& p, const void* sfa, const void* sfb, int n, int k, bool ue8m0) {
  p.sfa = static_cast<const float*>(sfa);
  p.sfb = static_cast<const float*>(sfb);
  p.sf_ue8m0 = ue8m0 ? 1 : 0;
  p.ld_sfb = ue8m0 ? ((((int64_t)n + 127) / 128 + 3) / 4 * 4) : 0;
  p.sfb_gstride = ue8m0 ? (int64_t)(k / 128) * p.ld_sfb : (((int64_t)n + 127) / 128) * (k / 128);
}

int gemm_nt_impl(const uint8_t* a, const void* sfa, const uint8_t* b, const void* sfb, uint16_t* d,
                 int m, int n, int k, int64_t lda, int64_t ldb, int64_t ldd, int64_t ld_sfa,
                 void* workspace, size_t workspace_bytes, void* stream, bool ue8m0,
                 const QOut* qo = nullptr) {
  int st = check_gemm_common(a, sfa, b, sfb, d, m, n, k, lda, ldb, ldd, ld_sfa);
  if (st == DG_SUCCESS) st = check_qout(qo, m, n, 1);
  if (st != DG_SUCCESS) return st;
  if (m == 0 || n == 0) return ok();
  dg::GemmParams p{};
  p.a = a; p.b = b; p.d = d;
  set_scales(p, sfa, sfb, n, k, ue8m0);
  set_qout(p, qo, m, n);
  p.m = m; p.n = n; p.k = k; p.num_groups = 1;
  p.lda = lda; p.ldb = ldb; p.ldd = ldd; p.ld_sfa = ld_sfa;
  return run_gemm(dg::kDense, p, m, 1, workspace, workspace_bytes, stream);
}

// Dense GEMM with MN-major operands.  majors bit 0: A is stored M-major as
// [K][lda] (lda >= m, m % 16 == 0); bit 1: B is stored N-major as [K][ldb]
// (ldb >= n, n % 16 == 0).  Scales keep the K-major (NT) layouts.
int gemm_majors_impl(int majors, const uint8_t* a, const void* sfa, const uint8_t* b, const void* sfb,
                     uint16_t* d, int m, int n, int k, int64_t lda, int64_t ldb, int64_t ldd, int64_t ld_sfa,
                     void* workspace, size_t workspace_bytes, void* stream, bool ue8m0) {
  const bool at = (majors & 1) != 0, bt = (majors & 2) != 0;
  // The common checks see a K-major leading dimension for a transposed
  // operand; its own rules follow.
  int st = check_gemm_common(a, sfa, b, sfb, d, m, n, k, at ? k : lda, bt ? k : ldb, ldd, ld_sfa);
  if (st != DG_SUCCESS) return st;
  const int64_t lim = (int64_t)1 << 32;
  if (at) {
    if (m % 16) return fail(DG_ERR_UNSUPPORTED_SHAPE, "m=%d is not a multiple of 16 (M-major A)", m);
    if (lda < m) return fail(DG_ERR_INVALID_VALUE, "lda smaller than m (M-major A)");
    if (lda % 16) return fail(DG_ERR_MISALIGNED, "lda must be a multiple of 16 bytes");
    if (!below(k, lda, 1, lim)) return fail(DG_ERR_UNSUPPORTED_SHAPE, "operand of 4 GiB or more");
  }
  if (bt) {
    if (n % 16) return fail(DG_ERR_UNSUPPORTED_SHAPE, "n=%d is not a multiple of 16 (N-major B)", n);
    if (ldb < n) return fail(DG_ERR_INVALID_VALUE, "ldb smaller than n (N-major B)");
    if (ldb % 16) return fail(DG_ERR_MISALIGNED, "ldb must be a multiple of 16 bytes");
    if (!below(k, ldb, 1, lim)) return fail(DG_ERR_UNSUPPORTED_SHAPE, "operand of 4 GiB or more");
  }
  if (m == 0 || n == 0) return ok();
  dg::GemmParams p{};
  p.a = a; p.b = b; p.d = d;
  set_scales(p, sfa, sfb, n, k, ue8m0);
  p.m = m; p.n = n; p.k = k; p.num_groups = 1;
  p.lda = lda; p.ldb = ldb; p.ldd = ldd; p.ld_sfa = ld_sfa;
  p.majors = majors;
  return run_gemm(dg::kDense, p, m, 1, workspace, workspace_bytes, stream);
}

int contiguous_impl(const uint8_t* a, const void* sfa, const uint8_t* b, const void* sfb, uint16_t* d,
                    const int32_t* m_indices, int m_total, int n, int k, int num_groups, int64_t ld_sfa,
                    void* workspace, size_t workspace_bytes, void* stream, bool ue8m0,
                    const QOut* qo = nullptr) {
  if (num_groups < 1) return fail(DG_ERR_INVALID_VALUE, "num_groups must be >= 1");
  int st = check_gemm_common(a, sfa, b, sfb, d, m_total, n, k, k, k, n, ld_sfa);
  if (st == DG_SUCCESS) st = check_qout(qo, m_total, n, 1);
  if (st != DG_SUCCESS) return st;
  if (!m_indices) return fail(DG_ERR_INVALID_VALUE, "null m_indices");
  if (m_total % 128) return fail(DG_ERR_UNSUPPORTED_SHAPE, "m_total=%d is not a multiple of 128", m_total);
  if (n % 8) return fail(DG_ERR_MISALIGNED, "n must be a multiple of 8 (rows of d are packed)");
  if (m_total == 0 || n == 0) return ok();
  dg::GemmParams p{};
  p.a = a; p.b = b; p.d = d; p.m_indices = m_indices;
  set_scales(p, sfa, sfb, n, k, ue8m0);
  set_qout(p, qo, m_total, n);
  p.m = m_total; p.n = n; p.k = k; p.num_groups = num_groups;
  p.lda = k; p.ldb = k; p.ldd = n; p.ld_sfa = ld_sfa;
  p.b_gstride = (int64_t)n * k;
  return run_gemm(dg::kContiguous, p, m_total, num_groups, workspace, workspace_bytes, stream);
}

int masked_impl(const uint8_t* a, const void* sfa, const uint8_t* b, const void* sfb, uint16_t* d,
                const int32_t* masked_m, int num_groups, int m_max, int n, int k, int expected_m,
                int64_t ld_sfa, void* workspace, size_t workspace_bytes, void* stream, bool ue8m0,
                const QOut* qo = nullptr) {
  if (num_groups < 1) return fail(DG_ERR_INVALID_VALUE, "num_groups must be >= 1");
  if (expected_m < 0) return fail(DG_ERR_INVALID_VALUE, "expected_m must be >= 0");
  int st = check_gemm_common(a, sfa, b, sfb, d, m_max, n, k, k, k, n, ld_sfa);
  if (st == DG_SUCCESS) st = check_qout(qo, m_max, n, num_groups);
  if (st != DG_SUCCESS) return st;
  if (!masked_m) return fail(DG_ERR_INVALID_VALUE, "null masked_m");
  if (n % 8) return fail(DG_ERR_MISALIGNED, "n must be a multiple of 8 (rows of d are packed)");
  if (num_groups > 65535) return fail(DG_ERR_UNSUPPORTED_SHAPE, "too many groups");
  if (m_max == 0 || n == 0) return ok();
  dg::GemmParams p{};
  p.a = a; p.b = b; p.d = d; p.masked_m = masked_m;
  set_scales(p, sfa, sfb, n, k, ue8m0);
  set_qout(p, qo, m_max, n);
  p.m = m_max; p.n = n; p.k = k; p.num_groups = num_groups;
  p.lda = k; p.ldb = k; p.ldd = n; p.ld_sfa = ld_sfa;
  p.a_gstride = (int64_t)m_max * k;
  p.sfa_gstride = (int64_t)(k / 128) * ld_sfa;
  p.b_gstride = (int64_t)n * k;
  p.d_gstride = (int64_t)m_max * n;
  return run_gemm(dg::kMasked, p, m_max, num_groups, workspace, workspace_bytes, stream, expected_m);
}

int k_grouped_impl(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb, uint16_t* d,
                   const int32_t* k_offsets, int num_groups, int m, int n, int k, int64_t ld_sfa,
                   int64_t ld_sfb, void* workspace, size_t workspace_bytes, void* stream) {
  if (num_groups < 1) return fail(DG_ERR_INVALID_VALUE, "num_groups must be >= 1");
  int st = check_gemm_common(a, sfa, b, sfb, d, m, n, k, k, k, n, ld_sfa);
  if (st != DG_SUCCESS) return st;
  if (!k_offsets) return fail(DG_ERR_INVALID_VALUE, "null k_offsets");
  if (n % 8) return fail(DG_ERR_MISALIGNED, "n must be a multiple of 8 (rows of d are packed)");
  if (ld_sfb < n || ld_sfb < 4) return fail(DG_ERR_INVALID_VALUE, "ld_sfb=%lld smaller than n (%d) or 4", (long long)ld_sfb, n);
  if (ld_sfb % 4) return fail(DG_ERR_MISALIGNED, "ld_sfb must be a multiple of 4");
  if (!below(k / 128, ld_sfb, 4, (int64_t)1 << 32)) return fail(DG_ERR_UNSUPPORTED_SHAPE, "sfb of 4 GiB or more");
  if ((((int64_t)m + 63) / 64) * (((int64_t)n + 63) / 64) > (((int64_t)1 << 31) - 1) / num_groups)
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "too many output tiles");
  if (m == 0 || n == 0) return ok();
  dg::GemmParams p{};
  p.a = a; p.b = b; p.d = d; p.k_offsets = k_offsets;
  p.sfa = sfa; p.sfb = sfb; p.ld_sfb = ld_sfb;
  p.m = m; p.n = n; p.k = k; p.num_groups = num_groups;
  p.lda = k; p.ldb = k; p.ldd = n; p.ld_sfa = ld_sfa;
  p.d_gstride = (int64_t)m * n;
  return run_gemm(dg::kKGrouped, p, m, num_groups, workspace, workspace_bytes, stream);
}

int quant_1x128_impl(const uint16_t* x, uint8_t* q, void* sf, int rows, int cols, int64_t ld_sf,
                     int num_groups, bool pow2, void* stream) {
  if (rows < 0 || cols < 0 || num_groups < 1) return fail(DG_ERR_INVALID_VALUE, "bad sizes (rows=%d cols=%d groups=%d)", rows, cols, num_groups);
  if (cols % 128) return fail(DG_ERR_UNSUPPORTED_SHAPE, "cols=%d is not a multiple of 128", cols);
  if (ld_sf < rows) return fail(DG_ERR_INVALID_VALUE, "ld_sf smaller than rows");
  if (ld_sf % 4) return fail(DG_ERR_MISALIGNED, "ld_sf must be a multiple of 4");
  if ((int64_t)num_groups * rows > INT32_MAX) return fail(DG_ERR_UNSUPPORTED_SHAPE, "num_groups * rows exceeds 2^31 - 1");
  if (!x || !q || !sf) return fail(DG_ERR_INVALID_VALUE, "null pointer argument");
  if (!aligned16(x) || !aligned16(q) || !aligned16(sf)) return fail(DG_ERR_MISALIGNED, "x, q and sf must be 16-byte aligned");
  if (cols == 0 || ld_sf == 0) return ok();
  const hipError_t e = dg::launch_quant_1x128(x, q, sf, rows, cols, ld_sf, num_groups, pow2,
                                              static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DG_ERR_HIP, "quant_1x128 launch failed: %s", hipGetErrorString(e));
  return ok();
}

int quant_1x128_mn_impl(const uint16_t* x, uint8_t* q, void* sf, int rows, int cols, int64_t ld_sf,
                        bool pow2, void* stream) {
  if (rows < 0 || cols < 0) return fail(DG_ERR_INVALID_VALUE, "bad sizes (rows=%d cols=%d)", rows, cols);
  if (rows % 128) return fail(DG_ERR_UNSUPPORTED_SHAPE, "rows=%d (K) is not a multiple of 128", rows);
  if (cols % 8) return fail(DG_ERR_UNSUPPORTED_SHAPE, "cols=%d is not a multiple of 8", cols);
  if (ld_sf < cols) return fail(DG_ERR_INVALID_VALUE, "ld_sf smaller than cols");
  if (ld_sf % 4) return fail(DG_ERR_MISALIGNED, "ld_sf must be a multiple of 4");
  if (rows / 128 > 65535) return fail(DG_ERR_UNSUPPORTED_SHAPE, "too many K blocks");
  if (!x || !q || !sf) return fail(DG_ERR_INVALID_VALUE, "null pointer argument");
  if (!aligned16(x) || !aligned16(q) || !aligned16(sf)) return fail(DG_ERR_MISALIGNED, "x, q and sf must be 16-byte aligned");
  if (rows == 0 || ld_sf == 0) return ok();
  const hipError_t e = dg::launch_quant_1x128_mn(x, q, sf, rows, cols, ld_sf, pow2, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DG_ERR_HIP, "quant_1x128_mn launch failed: %s", hipGetErrorString(e));
  return ok();
}

int quant_128x128_impl(const uint16_t* w, uint8_t* q, void* sf, int rows, int cols, int num_groups,
                       bool pow2, void* stream) {
  if (rows < 0 || cols < 0 || num_groups < 1) return fail(DG_ERR_INVALID_VALUE, "bad sizes (rows=%d cols=%d groups=%d)", rows, cols, num_groups);
  if (cols % 128) return fail(DG_ERR_UNSUPPORTED_SHAPE, "cols=%d is not a multiple of 128", cols);
  if (!w || !q || !sf) return fail(DG_ERR_INVALID_VALUE, "null pointer argument");
  if (!aligned16(w) || !aligned16(q) || !aligned16(sf)) return fail(DG_ERR_MISALIGNED, "w, q and sf must be 16-byte aligned");
  if (num_groups > 65535 || rows > 65535 * 128) return fail(DG_ERR_UNSUPPORTED_SHAPE, "too many blocks");
  if (rows == 0 || cols == 0) return ok();
  const hipError_t e = dg::launch_quant_128x128(w, q, sf, rows, cols, num_groups, pow2,
                                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(DG_ERR_HIP, "quant_128x128 launch failed: %s", hipGetErrorString(e));
  return ok();
}

// ------------------------------------------------- no-allocation dense GEMM --
// Device scratch of dg_fp8_gemm_nt_noalloc, for callers that cannot allocate:
// the stream-K arrival counters (the first kStreamKCounterBytes) and fp32
// partial tiles of one call.  The array lives in the loaded code object, one
// copy per GPU, until the process ends.  Host code never uses the array's
// name as an address: each device's copy is looked up once with
// hipGetSymbolAddress and kept in g_scratch.
constexpr size_t kNoAllocScratchBytes = dg::kStreamKCounterBytes + ((size_t)32 << 20);
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

__global__ void clear_words(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// This device's scratch address; on the first call for a device, also
// enqueues (on `stream`) a kernel that clears the counter region.  Every
// GEMM call leaves the counters it used at zero, so later calls need no
// clearing.  Returns DG_SUCCESS or an error status.
int noalloc_scratch(void* stream, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(DG_ERR_HIP, "cannot query the current device");
  if (dev < 0 || dev >= kMaxDevices) return fail(DG_ERR_HIP, "device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return fail(DG_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    const int words = (int)(dg::kStreamKCounterBytes / 4);
    hipLaunchKernelGGL(clear_words, dim3(words / 256), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint32_t*>(ptr), words);
    const hipError_t le = hipGetLastError();
    if (le != hipSuccess) return fail(DG_ERR_HIP, "scratch clear launch failed: %s", hipGetErrorString(le));
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return DG_SUCCESS;
}

}  // namespace

extern "C" {

int dg_fp8_gemm_nt_noalloc(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                           uint16_t* d, int m, int n, int k, int64_t lda, int64_t ldb, int64_t ldd,
                           int64_t ld_sfa, void* stream) {
  int st = check_gemm_common(a, sfa, b, sfb, d, m, n, k, lda, ldb, ldd, ld_sfa);
  if (st != DG_SUCCESS) return st;
  if (m == 0 || n == 0) return ok();
  if (!dg::plannable(dg::kDense, m, n, 1))
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "too many output tiles (m=%d n=%d)", m, n);
  const int cus = resolve_num_cus();
  if (cus < 0) return fail(DG_ERR_HIP, "cannot query the device's compute-unit count");
  const dg::GemmConfig cfg = dg::choose_config(dg::kDense, m, n, k, 1, cus);
  const size_t need = dg::workspace_bytes_for(cfg, dg::kDense, m, n, 1);
  if (need > kNoAllocScratchBytes)
    return fail(DG_ERR_WORKSPACE, "m=%d n=%d k=%d needs %zu bytes of scratch; the no-allocation GEMM holds %zu",
                m, n, k, need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    st = noalloc_scratch(stream, &ws);
    if (st != DG_SUCCESS) return st;
  }
  return gemm_nt_impl(a, sfa, b, sfb, d, m, n, k, lda, ldb, ldd, ld_sfa, ws, need > 0 ? kNoAllocScratchBytes : 0,
                      stream, false);
}

int dg_fp8_gemm_nt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   uint16_t* d, int m, int n, int k, int64_t lda, int64_t ldb, int64_t ldd,
                   int64_t ld_sfa, void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_nt_impl(a, sfa, b, sfb, d, m, n, k, lda, ldb, ldd, ld_sfa, workspace, workspace_bytes,
                      stream, false);
}

int dg_fp8_gemm_nn(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   uint16_t* d, int m, int n, int k, int64_t lda, int64_t ldb, int64_t ldd,
                   int64_t ld_sfa, void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_majors_impl(2, a, sfa, b, sfb, d, m, n, k, lda, ldb, ldd, ld_sfa, workspace, workspace_bytes, stream,
                          false);
}

int dg_fp8_gemm_nn_ue8m0(const uint8_t* a, const uint8_t* sfa, const uint8_t* b, const uint8_t* sfb,
                         uint16_t* d, int m, int n, int k, int64_t lda, int64_t ldb, int64_t ldd,
                         int64_t ld_sfa, void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_majors_impl(2, a, sfa, b, sfb, d, m, n, k, lda, ldb, ldd, ld_sfa, workspace, workspace_bytes, stream,
                          true);
}

int dg_fp8_gemm_tn(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   uint16_t* d, int m, int n, int k, int64_t lda, int64_t ldb, int64_t ldd,
                   int64_t ld_sfa, void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_majors_impl(3, a, sfa, b, sfb, d, m, n, k, lda, ldb, ldd, ld_sfa, workspace, workspace_bytes, stream,
                          false);
}

int dg_fp8_gemm_tn_ue8m0(const uint8_t* a, const uint8_t* sfa, const uint8_t* b, const uint8_t* sfb,
                         uint16_t* d, int m, int n, int k, int64_t lda, int64_t ldb, int64_t ldd,
                         int64_t ld_sfa, void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_majors_impl(3, a, sfa, b, sfb, d, m, n, k, lda, ldb, ldd, ld_sfa, workspace, workspace_bytes, stream,
                          true);
}

int dg_fp8_gemm_tt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                   uint16_t* d, int m, int n, int k, int64_t lda, int64_t ldb, int64_t ldd,
                   int64_t ld_sfa, void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_majors_impl(1, a, sfa, b, sfb, d, m, n, k, lda, ldb, ldd, ld_sfa, workspace, workspace_bytes, stream,
                          false);
}

int dg_fp8_gemm_tt_ue8m0(const uint8_t* a, const uint8_t* sfa, const uint8_t* b, const uint8_t* sfb,
                         uint16_t* d, int m, int n, int k, int64_t lda, int64_t ldb, int64_t ldd,
                         int64_t ld_sfa, void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_majors_impl(1, a, sfa, b, sfb, d, m, n, k, lda, ldb, ldd, ld_sfa, workspace, workspace_bytes, stream,
                          true);
}

int dg_fp8_gemm_nt_ue8m0(const uint8_t* a, const uint8_t* sfa, const uint8_t* b,
                         const uint8_t* sfb, uint16_t* d, int m, int n, int k, int64_t lda,
                         int64_t ldb, int64_t ldd, int64_t ld_sfa, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return gemm_nt_impl(a, sfa, b, sfb, d, m, n, k, lda, ldb, ldd, ld_sfa, workspace, workspace_bytes,
                      stream, true);
}

int dg_grouped_contiguous(const uint8_t* a, const float* sfa, const uint8_t* b,
                          const float* sfb, uint16_t* d, const int32_t* m_indices,
                          int m_total, int n, int k, int num_groups, int64_t ld_sfa,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return contiguous_impl(a, sfa, b, sfb, d, m_indices, m_total, n, k, num_groups, ld_sfa, workspace,
                         workspace_bytes, stream, false);
}

int dg_grouped_contiguous_ue8m0(const uint8_t* a, const uint8_t* sfa, const uint8_t* b,
                                const uint8_t* sfb, uint16_t* d, const int32_t* m_indices,
                                int m_total, int n, int k, int num_groups, int64_t ld_sfa,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return contiguous_impl(a, sfa, b, sfb, d, m_indices, m_total, n, k, num_groups, ld_sfa, workspace,
                         workspace_bytes, stream, true);
}

int dg_grouped_masked(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                      uint16_t* d, const int32_t* masked_m, int num_groups, int m_max, int n,
                      int k, int expected_m, int64_t ld_sfa, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return masked_impl(a, sfa, b, sfb, d, masked_m, num_groups, m_max, n, k, expected_m, ld_sfa,
                     workspace, workspace_bytes, stream, false);
}

int dg_grouped_masked_ue8m0(const uint8_t* a, const uint8_t* sfa, const uint8_t* b,
                            const uint8_t* sfb, uint16_t* d, const int32_t* masked_m,
                            int num_groups, int m_max, int n, int k, int expected_m,
                            int64_t ld_sfa, void* workspace, size_t workspace_bytes,
                            void* stream) {
  return masked_impl(a, sfa, b, sfb, d, masked_m, num_groups, m_max, n, k, expected_m, ld_sfa,
                     workspace, workspace_bytes, stream, true);
}

int dg_fp8_gemm_nt_qout(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                        uint16_t* d, uint8_t* dq, float* dsf, int m, int n, int k, int64_t lda,
                        int64_t ldb, int64_t ldd, int64_t ld_sfa, int64_t ld_dsf, void* workspace,
                        size_t workspace_bytes, void* stream) {
  const QOut q{dq, dsf, ld_dsf, false};
  return gemm_nt_impl(a, sfa, b, sfb, d, m, n, k, lda, ldb, ldd, ld_sfa, workspace, workspace_bytes,
                      stream, false, &q);
}

int dg_fp8_gemm_nt_ue8m0_qout(const uint8_t* a, const uint8_t* sfa, const uint8_t* b, const uint8_t* sfb,
                              uint16_t* d, uint8_t* dq, uint8_t* dsf, int m, int n, int k, int64_t lda,
                              int64_t ldb, int64_t ldd, int64_t ld_sfa, int64_t ld_dsf, void* workspace,
                              size_t workspace_bytes, void* stream) {
  const QOut q{dq, dsf, ld_dsf, true};
  return gemm_nt_impl(a, sfa, b, sfb, d, m, n, k, lda, ldb, ldd, ld_sfa, workspace, workspace_bytes,
                      stream, true, &q);
}

int dg_grouped_contiguous_qout(const uint8_t* a, const float* sfa, const uint8_t* b,
                               const float* sfb, uint16_t* d, uint8_t* dq, float* dsf,
                               const int32_t* m_indices, int m_total, int n, int k, int num_groups,
                               int64_t ld_sfa, int64_t ld_dsf, void* workspace,
                               size_t workspace_bytes, void* stream) {
  const QOut q{dq, dsf, ld_dsf, false};
  return contiguous_impl(a, sfa, b, sfb, d, m_indices, m_total, n, k, num_groups, ld_sfa, workspace,
                         workspace_bytes, stream, false, &q);
}

int dg_grouped_contiguous_ue8m0_qout(const uint8_t* a, const uint8_t* sfa, const uint8_t* b,
                                     const uint8_t* sfb, uint16_t* d, uint8_t* dq, uint8_t* dsf,
                                     const int32_t* m_indices, int m_total, int n, int k, int num_groups,
                                     int64_t ld_sfa, int64_t ld_dsf, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  const QOut q{dq, dsf, ld_dsf, true};
  return contiguous_impl(a, sfa, b, sfb, d, m_indices, m_total, n, k, num_groups, ld_sfa, workspace,
                         workspace_bytes, stream, true, &q);
}

int dg_grouped_masked_qout(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb,
                           uint16_t* d, uint8_t* dq, float* dsf, const int32_t* masked_m,
                           int num_groups, int m_max, int n, int k, int expected_m, int64_t ld_sfa,
                           int64_t ld_dsf, void* workspace, size_t workspace_bytes, void* stream) {
  const QOut q{dq, dsf, ld_dsf, false};
  return masked_impl(a, sfa, b, sfb, d, masked_m, num_groups, m_max, n, k, expected_m, ld_sfa,
                     workspace, workspace_bytes, stream, false, &q);
}

int dg_grouped_masked_ue8m0_qout(const uint8_t* a, const uint8_t* sfa, const uint8_t* b, const uint8_t* sfb,
                                 uint16_t* d, uint8_t* dq, uint8_t* dsf, const int32_t* masked_m,
                                 int num_groups, int m_max, int n, int k, int expected_m, int64_t ld_sfa,
                                 int64_t ld_dsf, void* workspace, size_t workspace_bytes, void* stream) {
  const QOut q{dq, dsf, ld_dsf, true};
  return masked_impl(a, sfa, b, sfb, d, masked_m, num_groups, m_max, n, k, expected_m, ld_sfa,
                     workspace, workspace_bytes, stream, true, &q);
}

int dg_k_grouped_nt(const uint8_t* a, const float* sfa, const uint8_t* b, const float* sfb, uint16_t* d,
                    const int32_t* k_offsets, int num_groups, int m, int n, int k, int64_t ld_sfa,
                    int64_t ld_sfb, void* workspace, size_t workspace_bytes, void* stream) {
  return k_grouped_impl(a, sfa, b, sfb, d, k_offsets, num_groups, m, n, k, ld_sfa, ld_sfb, workspace,
                        workspace_bytes, stream);
}

int dg_quant_1x128(const uint16_t* x, uint8_t* q, float* sf, int rows, int cols,
                   int64_t ld_sf, int num_groups, void* stream) {
  return quant_1x128_impl(x, q, sf, rows, cols, ld_sf, num_groups, false, stream);
}

int dg_quant_1x128_mn(const uint16_t* x, uint8_t* q, float* sf, int rows, int cols, int64_t ld_sf,
                      void* stream) {
  return quant_1x128_mn_impl(x, q, sf, rows, cols, ld_sf, false, stream);
}

int dg_quant_1x128_mn_ue8m0(const uint16_t* x, uint8_t* q, uint8_t* sf, int rows, int cols, int64_t ld_sf,
                            void* stream) {
  return quant_1x128_mn_impl(x, q, sf, rows, cols, ld_sf, true, stream);
}

int dg_quant_1x128_ue8m0(const uint16_t* x, uint8_t* q, uint8_t* sf, int rows, int cols,
                         int64_t ld_sf, int num_groups, void* stream) {
  return quant_1x128_impl(x, q, sf, rows, cols, ld_sf, num_groups, true, stream);
}

int dg_quant_128x128(const uint16_t* w, uint8_t* q, float* sf, int rows, int cols,
                     int num_groups, void* stream) {
  return quant_128x128_impl(w, q, sf, rows, cols, num_groups, false, stream);
}

int dg_quant_128x128_ue8m0(const uint16_t* w, uint8_t* q, uint8_t* sf, int rows, int cols,
                           int num_groups, void* stream) {
  return quant_128x128_impl(w, q, sf, rows, cols, num_groups, true, stream);
}

int64_t dg_get_ue8m0_sfb_leading_dim(int n) {
  if (n < 0) return -1;
  return (((int64_t)n + 127) / 128 + 3) / 4 * 4;
}

size_t dg_get_workspace_size(int m, int n, int k, int num_groups) {
  if (m <= 0 || n <= 0 || k <= 0 || num_groups < 1) return 0;
  int cus = resolve_num_cus();
  if (cus < 0) cus = 256;
  // The largest need over the layouts, with and without a quantised output,
  // and, for the masked layout, over the tile shapes its expected_m hint can
  // select.
  size_t worst = 0;
  const int hints[] = {0, 1, 64, 65, 128, 129, 256, 257};
  for (int narrow = 0; narrow <= 1; ++narrow)
    for (int qout = 0; qout <= 1; ++qout)
      for (int layout = dg::kDense; layout <= dg::kMasked; ++layout)
        for (int h : hints) {
          if ((h && layout != dg::kMasked) || !dg::plannable(layout, m, n, num_groups)) break;
          const dg::GemmConfig c = dg::choose_config(layout, m, n, k, num_groups, cus, h, qout != 0, narrow != 0);
          const size_t need = dg::workspace_bytes_for(c, layout, m, n, num_groups);
          if (need > worst) worst = need;
        }
  return worst;
}

int dg_get_num_cus(void) {
  const int v = resolve_num_cus();
  if (v < 0) return fail(DG_ERR_HIP, "cannot query the device's compute-unit count");
  return v;
}

int dg_set_num_cus(int num_cus) {
  if (num_cus < 0 || num_cus > 4096) return fail(DG_ERR_INVALID_VALUE, "num_cus must be in [0, 4096]");
  g_num_cus_override.store(num_cus);
  return ok();
}

int dg_get_m_alignment_for_contiguous_layout(void) { return 128; }

int64_t dg_get_sf_leading_dim(int m) {
  if (m < 0) return -1;
  return ((int64_t)m + 3) / 4 * 4;
}

const char* dg_get_last_error_string(void) { return g_last_error; }

int dg_describe_config(int layout, int m, int n, int k, int num_groups, int expected_m,
                       int num_cus, char* buf, size_t len) {
  const bool qout = (layout & 8) != 0;  // configuration of the *_qout entry points
  layout &= ~8;
  if (layout < dg::kDense || layout > dg::kKGrouped || m < 0 || n < 0 || k < 0 ||
      num_groups < 1 || expected_m < 0 || num_cus < 1 || !buf || len == 0)
    return fail(DG_ERR_INVALID_VALUE, "bad arguments to dg_describe_config");
  if (!dg::plannable(layout, m, n, num_groups))
    return fail(DG_ERR_UNSUPPORTED_SHAPE, "too many output tiles (m=%d n=%d groups=%d)", m, n, num_groups);
  const dg::GemmConfig c = dg::choose_config(layout, m, n, k, num_groups, num_cus, expected_m, qout);
  snprintf(buf, len, "layout=%s bm=%d bn=%d stream_k=%d sk_split=%d grid=%d tiles=%d variant=%d k_rotate=%d workspace=%zu",
           layout_name(layout), c.bm, c.bn, c.stream_k, c.sk_split, c.grid, c.tiles, c.variant, c.k_rotate,
           dg::workspace_bytes_for(c, layout, m, n, num_groups));
  return ok();
}

}  // extern "C"
