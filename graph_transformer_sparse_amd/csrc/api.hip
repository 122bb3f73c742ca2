// The C ABI of libgtattn (declared in include/gt_attn.h): argument checks,
// workspace layout, per-thread error detail and optional event timing.
// Every check runs on the host before anything is enqueued; a call that
// fails one returns its status without touching the device.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <utility>
#include <vector>

#include "device.hpp"
#include "host.hpp"
#include "layout.hpp"

namespace gt {

bool shape_supported(gt_dtype dt, int heads, int head_dim);
gt_status launch_fwd(const gt_graph *g, int heads, int head_dim, gt_dtype dt, float scale,
                     const void *Q, const void *K, const void *V, const float *bias, void *Y,
                     float *lse, float *part, hipStream_t st);
gt_status launch_bwd(const gt_graph *g, int heads, int head_dim, gt_dtype dt, float scale,
                     const void *Q, const void *K, const void *V, const float *bias,
                     const void *Y, const float *lse, const void *dY, void *dQ, void *dK,
                     void *dV, float *dbias, float *rowstat, float *fixstat, float *part_rows,
                     float *part_cols, hipStream_t st);

static thread_local char g_err[512];

gt_status fail(gt_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_err[0] = 0; }

// ---- event timing --------------------------------------------------------
namespace {
struct Prof {
  std::mutex mu;
  int32_t mask = 0;                                     // kernels being timed
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;  // reusable event pairs
  std::vector<int> kind;                                // kernel of pool[i] in use
  size_t used = 0;
};
Prof &prof() {
  static Prof p;
  return p;
}
const char *const kPkNames[PK_COUNT] = {"fwd",      "fwd_merge",      "bwd_rows",
                                        "bwd_rows_merge", "bwd_cols", "bwd_cols_merge",
                                        "bwd_dbias"};
}  // namespace

int prof_begin(ProfKernel k, hipStream_t s) {
  Prof &p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  if (!(p.mask & (1 << k))) return -1;
  if (p.used == p.pool.size()) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess) return -1;
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      return -1;
    }
    p.pool.push_back({a, b});
    p.kind.push_back(-1);
  }
  const int tok = (int)p.used++;
  p.kind[tok] = k;
  if (hipEventRecord(p.pool[tok].first, s) != hipSuccess) p.kind[tok] = -1;
  return tok;
}

void prof_end(int tok, hipStream_t s) {
  if (tok < 0) return;
  Prof &p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  if (hipEventRecord(p.pool[tok].second, s) != hipSuccess) p.kind[tok] = -1;
}

}  // namespace gt

using namespace gt;

namespace {

struct WorkLayout {
  size_t part_fwd;                                 // forward
  size_t rowstat, fixstat, part_rows, part_cols;   // backward
  size_t fwd_total, bwd_total, total;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

WorkLayout work_layout(const gt_graph *g, int heads, int head_dim) {
  WorkLayout w;
  const size_t D = (size_t)heads * head_dim;
  const size_t sr = (size_t)g->rows.n_items, sc = (size_t)g->cols.n_items;
  w.part_fwd = 0;
  w.fwd_total = align256(sr * (size_t)fwd_slot_floats(D, heads) * sizeof(float));
  w.rowstat = 0;
  w.fixstat = align256((size_t)g->n_rows * heads * 2 * sizeof(float));
  w.part_rows = w.fixstat + align256((size_t)g->n_rows * heads * 2 * sizeof(float));
  w.part_cols = w.part_rows + align256(sr * (size_t)rows_slot_floats(D, heads) * sizeof(float));
  w.bwd_total = w.part_cols + align256(sc * (size_t)cols_slot_floats(D, heads) * sizeof(float));
  w.total = std::max<size_t>(std::max(w.fwd_total, w.bwd_total), 256);
  return w;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

gt_status check_common(const gt_graph *g, int heads, int head_dim, gt_dtype dt) {
  if (!g) return fail(GT_E_NULL, "graph is NULL");
  if (dt != GT_F32 && dt != GT_BF16) return fail(GT_E_DTYPE, "unknown dtype %d", (int)dt);
  if (!shape_supported(dt, heads, head_dim))
    return fail(GT_E_SHAPE, "heads %d x head_dim %d not supported for dtype %d", heads, head_dim,
                (int)dt);
  if (g->n_rows < 0 || g->n_cols < 0 || g->nnz < 0)
    return fail(GT_E_ARG, "graph has negative sizes");
  if (!g->indptr || (g->nnz > 0 && !g->indices) || !g->indptr_t || !g->rows.order ||
      !g->cols.order || !g->rows.spans || !g->cols.spans)
    return fail(GT_E_NULL, "graph is not prepared");
  return GT_OK;
}

gt_status check_feat(const void *p, const char *name, bool need) {
  if (!p) return need ? fail(GT_E_NULL, "%s is NULL", name) : GT_OK;
  if (!aligned16(p)) return fail(GT_E_ALIGN, "%s is not 16-byte aligned", name);
  return GT_OK;
}

#define TRY(x)                  \
  do {                          \
    gt_status s_ = (x);         \
    if (s_ != GT_OK) return s_; \
  } while (0)

}  // namespace

extern "C" size_t gt_attn_work_bytes(const gt_graph *g, int32_t heads, int32_t head_dim) {
  if (!g || heads <= 0 || head_dim <= 0) return 0;
  return work_layout(g, heads, head_dim).total;
}

extern "C" gt_status gt_attn_fwd(const gt_graph *g, int32_t heads, int32_t head_dim, gt_dtype dt,
                                 float scale, const void *Q, const void *K, const void *V,
                                 const float *bias, void *Y, float *lse, void *work,
                                 size_t work_bytes, void *stream) {
  clear_error();
  TRY(check_common(g, heads, head_dim, dt));
  const bool rows = g->n_rows > 0, cols = g->n_cols > 0;
  TRY(check_feat(Q, "Q", rows));
  TRY(check_feat(K, "K", cols));
  TRY(check_feat(V, "V", cols));
  TRY(check_feat(Y, "Y", rows));
  if (rows && !lse) return fail(GT_E_NULL, "lse is NULL");
  if (lse && !aligned4(lse)) return fail(GT_E_ALIGN, "lse is not 4-byte aligned");
  if (bias && !aligned4(bias)) return fail(GT_E_ALIGN, "bias is not 4-byte aligned");
  const WorkLayout w = work_layout(g, heads, head_dim);
  if (!work) return fail(GT_E_NULL, "work is NULL");
  if (!aligned16(work)) return fail(GT_E_ALIGN, "work is not 16-byte aligned");
  if (work_bytes < w.fwd_total)
    return fail(GT_E_WORKSPACE, "work has %zu bytes, needs %zu", work_bytes, w.fwd_total);
  char *wb = (char *)work;
  return launch_fwd(g, heads, head_dim, dt, scale, Q, K, V, bias, Y, lse,
                    (float *)(wb + w.part_fwd), (hipStream_t)stream);
}

// ---- forward without a caller workspace ------------------------------------
// The piece states of split rows live in a file-scope device array instead
// of the caller's work buffer.  Host code never uses the array's name as an
// address: on the first call on a device (with that device current) its
// device address is looked up with hipGetSymbolAddress and kept per device.
static __device__ __align__(256) unsigned char scratch[GT_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
std::vector<void *> g_scratch_at;   // device address of `scratch`, per device id

gt_status scratch_address(void **out) {
  int dev = 0;
  GT_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if ((size_t)dev >= g_scratch_at.size()) g_scratch_at.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_at[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(GT_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_at[dev] = p;
  }
  *out = g_scratch_at[dev];
  return GT_OK;
}
}  // namespace

extern "C" gt_status gt_attn_fwd_noalloc(const gt_graph *g, int32_t heads, int32_t head_dim,
                                         gt_dtype dt, float scale, const void *Q, const void *K,
                                         const void *V, const float *bias, void *Y, float *lse,
                                         void *stream) {
  clear_error();
  TRY(check_common(g, heads, head_dim, dt));
  const bool rows = g->n_rows > 0, cols = g->n_cols > 0;
  TRY(check_feat(Q, "Q", rows));
  TRY(check_feat(K, "K", cols));
  TRY(check_feat(V, "V", cols));
  TRY(check_feat(Y, "Y", rows));
  if (rows && !lse) return fail(GT_E_NULL, "lse is NULL");
  if (lse && !aligned4(lse)) return fail(GT_E_ALIGN, "lse is not 4-byte aligned");
  if (bias && !aligned4(bias)) return fail(GT_E_ALIGN, "bias is not 4-byte aligned");
  const WorkLayout w = work_layout(g, heads, head_dim);
  if (w.fwd_total > (size_t)GT_NOALLOC_SCRATCH_BYTES)
    return fail(GT_E_WORKSPACE, "the forward needs %zu bytes of scratch; the static maximum is %zu",
                w.fwd_total, (size_t)GT_NOALLOC_SCRATCH_BYTES);
  void *ptr = nullptr;
  TRY(scratch_address(&ptr));
  return launch_fwd(g, heads, head_dim, dt, scale, Q, K, V, bias, Y, lse,
                    (float *)((char *)ptr + w.part_fwd), (hipStream_t)stream);
}

extern "C" gt_status gt_attn_bwd(const gt_graph *g, int32_t heads, int32_t head_dim, gt_dtype dt,
                                 float scale, const void *Q, const void *K, const void *V,
                                 const float *bias, const void *Y, const float *lse,
                                 const void *dY, void *dQ, void *dK, void *dV, float *dbias,
                                 void *work, size_t work_bytes, void *stream) {
  clear_error();
  TRY(check_common(g, heads, head_dim, dt));
  if ((bias == nullptr) != (dbias == nullptr))
    return fail(GT_E_UNSUPPORTED, "bias and dbias must be given together");
  const bool rows = g->n_rows > 0, cols = g->n_cols > 0;
  TRY(check_feat(Q, "Q", rows));
  TRY(check_feat(K, "K", cols));
  TRY(check_feat(V, "V", cols));
  TRY(check_feat(Y, "Y", rows && bias != nullptr));
  TRY(check_feat(dY, "dY", rows));
  TRY(check_feat(dQ, "dQ", rows));
  TRY(check_feat(dK, "dK", cols));
  TRY(check_feat(dV, "dV", cols));
  if (rows && !lse) return fail(GT_E_NULL, "lse is NULL");
  if (lse && !aligned4(lse)) return fail(GT_E_ALIGN, "lse is not 4-byte aligned");
  if (bias && (!aligned4(bias) || !aligned4(dbias)))
    return fail(GT_E_ALIGN, "bias / dbias not 4-byte aligned");
  const WorkLayout w = work_layout(g, heads, head_dim);
  if (!work) return fail(GT_E_NULL, "work is NULL");
  if (!aligned16(work)) return fail(GT_E_ALIGN, "work is not 16-byte aligned");
  if (work_bytes < w.bwd_total)
    return fail(GT_E_WORKSPACE, "work has %zu bytes, needs %zu", work_bytes, w.bwd_total);
  char *wb = (char *)work;
  return launch_bwd(g, heads, head_dim, dt, scale, Q, K, V, bias, Y, lse, dY, dQ, dK, dV, dbias,
                    (float *)(wb + w.rowstat), (float *)(wb + w.fixstat),
                    (float *)(wb + w.part_rows), (float *)(wb + w.part_cols),
                    (hipStream_t)stream);
}

extern "C" gt_status gt_prof_enable(int32_t kernel_mask) {
  Prof &p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  p.mask = kernel_mask & ((1 << PK_COUNT) - 1);
  return GT_OK;
}

extern "C" gt_status gt_prof_reset(void) {
  Prof &p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  p.used = 0;
  return GT_OK;
}

extern "C" gt_status gt_prof_query(const char *kernel, double *total_ms, int64_t *launches) {
  clear_error();
  if (!kernel || !total_ms || !launches) return fail(GT_E_NULL, "NULL argument");
  int k = -1;
  for (int i = 0; i < PK_COUNT; ++i)
    if (strcmp(kernel, kPkNames[i]) == 0) k = i;
  if (k < 0) return fail(GT_E_ARG, "unknown kernel name '%s'", kernel);
  Prof &p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  double ms = 0.0;
  int64_t n = 0;
  for (size_t i = 0; i < p.used; ++i) {
    if (p.kind[i] != k) continue;
    GT_HIP(hipEventSynchronize(p.pool[i].second));
    float t = 0.f;
    GT_HIP(hipEventElapsedTime(&t, p.pool[i].first, p.pool[i].second));
    ms += t;
    ++n;
  }
  *total_ms = ms;
  *launches = n;
  return GT_OK;
}

extern "C" const char *gt_status_str(gt_status s) {
  switch (s) {
    case GT_OK: return "ok";
    case GT_E_NULL: return "a required pointer is NULL";
    case GT_E_ARG: return "argument out of range";
    case GT_E_DTYPE: return "unknown dtype";
    case GT_E_SHAPE: return "heads/head_dim not supported";
    case GT_E_ALIGN: return "misaligned pointer";
    case GT_E_UNSUPPORTED: return "bias and dbias must be given together";
    case GT_E_WORKSPACE: return "workspace too small";
    case GT_E_CSR: return "malformed CSR";
    case GT_E_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

extern "C" const char *gt_last_error(void) { return g_err; }

extern "C" int32_t gt_version(void) { return 104; }
