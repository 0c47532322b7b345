// C ABI of the LiteAttention step library (declared in include/lite_attn.h): argument
// validation, error reporting and kernel dispatch. No device memory is allocated here (the
// persistent launches' tile queues are static device memory of the library).

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <utility>

#include "lite_attn.h"
#include "lite_attn_internal.h"

struct lite_attn_s {
  lite_attn_config cfg;
  int64_t sb, sh, sn;
  int Tq, Tk, W;
  float scale;
  lite_attn::FwdLauncher fwd;
};

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tile queue of a stream for persistent launches. Each (device, stream) pair gets one of the
// device's kQueueSlots queues for the life of the process; launches on one stream run one after
// another, so a queue is never used by two launches at once. Returns nullptr (the launch then
// takes one workgroup per tile) when the stream belongs to another device than the current
// one, for the per-thread default stream (one handle value, many streams), or when every queue
// of the device is taken.
struct QueueTable {
  std::mutex mu;
  std::map<std::pair<int, uintptr_t>, int> slot;
  std::map<int, int> used;
  std::map<int, int> cus;
  std::map<int, uint32_t*> base;   // queue 0 of each device
};

QueueTable& queue_table() {
  static QueueTable* t = new QueueTable;   // never destroyed: usable during static teardown
  return *t;
}

uint32_t* stream_queue(hipStream_t st, int* n_cu) {
  *n_cu = 0;
  if (st == hipStreamPerThread) return nullptr;
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (st != nullptr) {
    int dev = -1;
    if (hipStreamGetDevice(st, &dev) != hipSuccess || dev != cur) return nullptr;
  }
  QueueTable& t = queue_table();
  std::lock_guard<std::mutex> lock(t.mu);
  auto c = t.cus.find(cur);
  if (c == t.cus.end()) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, cur) != hipSuccess)
      return nullptr;
    c = t.cus.emplace(cur, n).first;
  }
  const auto key = std::make_pair(cur, reinterpret_cast<uintptr_t>(st));
  auto it = t.slot.find(key);
  if (it == t.slot.end()) {
    int& used = t.used[cur];
    if (used >= lite_attn::kQueueSlots) return nullptr;
    it = t.slot.emplace(key, used++).first;
  }
  auto b = t.base.find(cur);
  if (b == t.base.end()) {
    uint32_t* q0 = nullptr;
    if (lite_attn::tile_queue_address(0, &q0) != hipSuccess) return nullptr;
    b = t.base.emplace(cur, q0).first;
  }
  *n_cu = c->second;
  return b->second + 2 * it->second;
}

}  // namespace

extern "C" {

const char* lite_attn_status_string(int status) {
  switch (status) {
    case LITE_ATTN_OK: return "ok";
    case LITE_ATTN_ERR_INVALID_ARG: return "invalid argument";
    case LITE_ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case LITE_ATTN_ERR_HIP: return "HIP runtime error";
    case LITE_ATTN_ERR_NO_MEMORY: return "out of host memory";
    default: return "unknown status";
  }
}

const char* lite_attn_last_error(void) { return g_last_error.c_str(); }

int lite_attn_create(const lite_attn_config* cfg, lite_attn_t* out) {
  try {
    if (out) *out = nullptr;
    if (!cfg || !out) return fail(LITE_ATTN_ERR_INVALID_ARG, "create: NULL argument");
    const lite_attn_config& c = *cfg;
    if (c.abi_version != LITE_ATTN_ABI_VERSION)
      return fail(LITE_ATTN_ERR_INVALID_ARG, "create: abi_version %d, library is %d",
                  c.abi_version, LITE_ATTN_ABI_VERSION);
    if (c.batch < 0 || c.heads < 0 || c.seq_len < 0)
      return fail(LITE_ATTN_ERR_INVALID_ARG, "create: negative size (B=%d H=%d N=%d)", c.batch,
                  c.heads, c.seq_len);
    if (c.head_dim <= 0 || c.tile_q <= 0 || c.tile_k <= 0)
      return fail(LITE_ATTN_ERR_INVALID_ARG, "create: head_dim and tiles must be positive");
    if (c.order != LITE_ATTN_ORDER_ASC && c.order != LITE_ATTN_ORDER_ALT)
      return fail(LITE_ATTN_ERR_INVALID_ARG, "create: unknown order %d", c.order);
    if (c.dtype != LITE_ATTN_BF16 && c.dtype != LITE_ATTN_FP32)
      return fail(LITE_ATTN_ERR_INVALID_ARG, "create: unknown dtype %d", c.dtype);
    if (c.dense_prefix < 0 || c.dense_prefix > c.seq_len)
      return fail(LITE_ATTN_ERR_INVALID_ARG, "create: dense_prefix %d outside [0, %d]",
                  c.dense_prefix, c.seq_len);
    if (!(std::isfinite(c.softmax_scale)))
      return fail(LITE_ATTN_ERR_INVALID_ARG, "create: softmax_scale is not finite");
    if ((c.options & ~(uint32_t)LITE_ATTN_OPT_IN_STEP_SKIP) != 0u || c.reserved != 0u)
      return fail(LITE_ATTN_ERR_INVALID_ARG, "create: unknown option bits 0x%x or reserved %u",
                  c.options, c.reserved);

    int64_t sb = c.stride_b, sh = c.stride_h, sn = c.stride_n;
    if (sb == 0 && sh == 0 && sn == 0) {
      sn = c.head_dim;
      sh = (int64_t)c.seq_len * sn;
      sb = (int64_t)c.heads * sh;
    }
    if (sb < 0 || sh < 0 || sn < c.head_dim || sb % 8 || sh % 8 || sn % 8 || sn >= (1 << 24))
      return fail(LITE_ATTN_ERR_INVALID_ARG,
                  "create: strides (%lld, %lld, %lld) must be non-negative multiples of 8 "
                  "elements with head_dim <= stride_n < 2^24",
                  (long long)sb, (long long)sh, (long long)sn);

    if (c.tile_k != lite_attn::kTileK)
      return fail(LITE_ATTN_ERR_UNSUPPORTED, "create: tile_k %d not built (only %d)", c.tile_k,
                  lite_attn::kTileK);
    const bool in_step = (c.options & LITE_ATTN_OPT_IN_STEP_SKIP) != 0u;
    lite_attn::FwdLauncher fwd = lite_attn::get_fwd_launcher(c.dtype, c.head_dim, c.tile_q, in_step);
    if (!fwd)
      return fail(LITE_ATTN_ERR_UNSUPPORTED,
                  "create: no kernel for dtype=%d head_dim=%d tile_q=%d (built: head_dim 64/128,"
                  " tile_q 64/128, tile_k 64)",
                  c.dtype, c.head_dim, c.tile_q);
    const int64_t tq = ceil_div(c.seq_len, c.tile_q);
    const int64_t tk = ceil_div(c.seq_len, c.tile_k);
    if (tk > lite_attn::kMaxTilesK)
      return fail(LITE_ATTN_ERR_UNSUPPORTED, "create: %lld key tiles exceed the limit %d",
                  (long long)tk, lite_attn::kMaxTilesK);
    if ((int64_t)c.batch * c.heads * tq > 0x7fffffffLL)
      return fail(LITE_ATTN_ERR_UNSUPPORTED, "create: too many query tiles for one launch");

    lite_attn_s* hnd = new (std::nothrow) lite_attn_s;
    if (!hnd) return fail(LITE_ATTN_ERR_NO_MEMORY, "create: out of host memory");
    hnd->cfg = c;
    hnd->sb = sb;
    hnd->sh = sh;
    hnd->sn = sn;
    hnd->Tq = (int)tq;
    hnd->Tk = (int)tk;
    hnd->W = (int)ceil_div(tk, 32);
    hnd->scale = c.softmax_scale > 0.f ? c.softmax_scale : 1.0f / std::sqrt((float)c.head_dim);
    hnd->fwd = fwd;
    *out = hnd;
    return LITE_ATTN_OK;
  } catch (...) {
    return fail(LITE_ATTN_ERR_NO_MEMORY, "create: unexpected exception");
  }
}

int lite_attn_destroy(lite_attn_t handle) {
  delete handle;
  return LITE_ATTN_OK;
}

size_t lite_attn_mask_bytes(lite_attn_t h) {
  if (!h) return 0;
  return (size_t)h->cfg.batch * h->cfg.heads * h->Tq * h->W * sizeof(uint32_t);
}

int lite_attn_mask_geometry(lite_attn_t h, int32_t* tiles_q, int32_t* tiles_k,
                            int32_t* words_per_row) {
  if (!h) return fail(LITE_ATTN_ERR_INVALID_ARG, "mask_geometry: NULL handle");
  if (tiles_q) *tiles_q = h->Tq;
  if (tiles_k) *tiles_k = h->Tk;
  if (words_per_row) *words_per_row = h->W;
  return LITE_ATTN_OK;
}

}  // extern "C"

namespace {

// Shared body of lite_attn_step and lite_attn_step_scheduled.
int step_impl(const char* who, lite_attn_t h, const void* q, const void* k, const void* v,
              void* out, uint32_t* mask, float log_eps_t, int32_t step, void* workspace,
              bool scheduled, float* tile_stats, float refresh_delta, bool refresh,
              void* stream) {
  try {
    if (!h) return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: NULL handle", who);
    if (std::isnan(log_eps_t) || log_eps_t > 0.f)
      return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: log_eps_t must be in [-inf, 0], got %g", who,
                  (double)log_eps_t);
    if (step < 0) return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: negative step %d", who, step);
    const lite_attn_config& c = h->cfg;
    if ((int64_t)c.batch * c.heads * c.seq_len == 0) return LITE_ATTN_OK;
    if (!q || !k || !v || !out || !mask)
      return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: NULL tensor or mask pointer", who);
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(mask, 4))
      return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: misaligned pointer (tensors need 16 B)", who);
    if (out == q || out == k || out == v)
      return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: out aliases an input", who);
    if (scheduled && (!workspace || !aligned(workspace, 256)))
      return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: NULL or not 256-byte aligned workspace", who);
    if (refresh && (!tile_stats || !aligned(tile_stats, 4)))
      return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: NULL or misaligned tile_stats", who);
    if (refresh && !(refresh_delta >= 0.f))
      return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: refresh_delta must be >= 0, got %g", who,
                  (double)refresh_delta);

    const hipStream_t st = static_cast<hipStream_t>(stream);
    lite_attn::FwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.mask = mask;
    p.sb = h->sb;
    p.sh = h->sh;
    p.sn = h->sn;
    p.B = c.batch;
    p.H = c.heads;
    p.N = c.seq_len;
    p.Tq = h->Tq;
    p.Tk = h->Tk;
    p.W = h->W;
    p.scale = h->scale;
    p.scale_log2 = h->scale * 1.4426950408889634f;
    p.log_eps = log_eps_t;
    p.descending = (c.order == LITE_ATTN_ORDER_ALT && (step & 1)) ? 1 : 0;
    p.dense_prefix = c.dense_prefix;
    p.perm = nullptr;
    p.stats = refresh ? tile_stats : nullptr;
    p.refresh_delta = refresh_delta;
    p.queue = c.dtype == LITE_ATTN_BF16 ? stream_queue(st, &p.n_cu) : nullptr;   // persistent
    if (!p.queue) p.n_cu = 0;
    if (scheduled) {
      const int n = c.batch * c.heads * h->Tq;
      const hipError_t e = lite_attn::launch_plan(mask, n, h->W, h->Tk, workspace, st);
      if (e != hipSuccess)
        return fail(LITE_ATTN_ERR_HIP, "%s: schedule launch failed: %s", who,
                    hipGetErrorString(e));
      p.perm = static_cast<const uint32_t*>(workspace);
    }
    const hipError_t e = h->fwd(p, st);
    if (e != hipSuccess)
      return fail(LITE_ATTN_ERR_HIP, "%s: kernel launch failed: %s", who, hipGetErrorString(e));
    return LITE_ATTN_OK;
  } catch (...) {
    return fail(LITE_ATTN_ERR_HIP, "%s: unexpected exception", who);
  }
}

}  // namespace

extern "C" {

int lite_attn_step(lite_attn_t h, const void* q, const void* k, const void* v, void* out,
                   uint32_t* mask, float log_eps_t, int32_t step, void* stream) {
  return step_impl("step", h, q, k, v, out, mask, log_eps_t, step, nullptr, false, nullptr, 0.f,
                   false, stream);
}

int lite_attn_step_refresh(lite_attn_t h, const void* q, const void* k, const void* v,
                           void* out, uint32_t* mask, float* tile_stats, float refresh_delta,
                           float log_eps_t, int32_t step, void* stream) {
  return step_impl("step_refresh", h, q, k, v, out, mask, log_eps_t, step, nullptr, false,
                   tile_stats, refresh_delta, true, stream);
}

size_t lite_attn_workspace_bytes(lite_attn_t h) {
  if (!h) return 0;
  return lite_attn::plan_workspace_bytes((int64_t)h->cfg.batch * h->cfg.heads * h->Tq);
}

int lite_attn_step_scheduled(lite_attn_t h, const void* q, const void* k, const void* v,
                             void* out, uint32_t* mask, float log_eps_t, int32_t step,
                             void* workspace, void* stream) {
  return step_impl("step_scheduled", h, q, k, v, out, mask, log_eps_t, step, workspace, true,
                   nullptr, 0.f, false, stream);
}

int lite_attn_reset_mask(lite_attn_t h, uint32_t* mask, void* stream) {
  if (!h) return fail(LITE_ATTN_ERR_INVALID_ARG, "reset_mask: NULL handle");
  const size_t words = lite_attn_mask_bytes(h) / sizeof(uint32_t);
  if (words == 0) return LITE_ATTN_OK;
  if (!mask || !aligned(mask, 4))
    return fail(LITE_ATTN_ERR_INVALID_ARG, "reset_mask: NULL or misaligned mask");
  const hipError_t e =
      lite_attn::launch_mask_fill_zero(mask, words, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(LITE_ATTN_ERR_HIP, "reset_mask: launch failed: %s", hipGetErrorString(e));
  return LITE_ATTN_OK;
}

int lite_attn_mask_popcount(lite_attn_t h, const uint32_t* mask, uint32_t* counts,
                            void* stream) {
  if (!h) return fail(LITE_ATTN_ERR_INVALID_ARG, "mask_popcount: NULL handle");
  const int heads_total = h->cfg.batch * h->cfg.heads;
  if (heads_total == 0) return LITE_ATTN_OK;
  if (!counts || !aligned(counts, 4))
    return fail(LITE_ATTN_ERR_INVALID_ARG, "mask_popcount: NULL or misaligned counts");
  if (h->Tq == 0) {
    const hipError_t e = lite_attn::launch_mask_fill_zero(counts, (size_t)heads_total,
                                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LITE_ATTN_OK
                           : fail(LITE_ATTN_ERR_HIP, "mask_popcount: %s", hipGetErrorString(e));
  }
  if (!mask || !aligned(mask, 4))
    return fail(LITE_ATTN_ERR_INVALID_ARG, "mask_popcount: NULL or misaligned mask");
  const hipError_t e = lite_attn::launch_mask_popcount(mask, counts, heads_total, h->Tq, h->Tk,
                                                       h->W, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(LITE_ATTN_ERR_HIP, "mask_popcount: launch failed: %s", hipGetErrorString(e));
  return LITE_ATTN_OK;
}

}  // extern "C"
