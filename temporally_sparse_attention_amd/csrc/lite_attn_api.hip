// C ABI of the LiteAttention step library (declared in include/lite_attn.h): argument
// validation, error reporting and kernel dispatch. No device memory is allocated here (the
// persistent launches' tile queues and the workspace of lite_attn_step_scheduled_static are
// static device memory of the library).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "lite_attn.h"
#include "lite_attn_aux.h"
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

// Tile queue of a persistent launch. Two launches that share a queue must not overlap: each
// takes tile positions from it, and the last workgroup of each puts it back to zero.
// - An eager launch uses the queue of its (device, stream) pair, one of the device's first
//   kEagerQueueSlots queues, assigned on first use and kept for the life of the process.
//   Launches on one stream run one after another.
// - A launch captured into a graph gets a queue of its own, never given to anything else: a
//   graph may be replayed on any stream, concurrently with other work (two guidance branches
//   captured on one capture stream and replayed on two streams, say).
// Returns nullptr (the launch then takes one workgroup per query tile) when the stream belongs
// to another device than the current one, for the per-thread default stream (one handle value,
// many streams), or when the pool the launch draws from is used up.
struct QueueTable {
  std::mutex mu;
  std::map<std::pair<int, uintptr_t>, int> slot;
  std::map<int, int> used;        // eager queues handed out, per device
  std::map<int, int> captured;    // captured-launch queues handed out, per device
  std::map<int, int> cus;
  std::map<int, uint32_t*> base;  // queue 0 of each device
};

QueueTable& queue_table() {
  static QueueTable* t = new QueueTable;   // never destroyed: usable during static teardown
  return *t;
}

uint32_t* launch_queue(hipStream_t st, int* n_cu, int* slot_out) {
  *n_cu = 0;
  *slot_out = -1;
  if (st == hipStreamPerThread) return nullptr;
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (st != nullptr) {
    int dev = -1;
    if (hipStreamGetDevice(st, &dev) != hipSuccess || dev != cur) return nullptr;
    if (hipStreamIsCapturing(st, &capture) != hipSuccess) return nullptr;
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
  auto b = t.base.find(cur);
  if (b == t.base.end()) {
    uint32_t* q0 = nullptr;
    if (lite_attn::tile_queue_address(0, &q0) != hipSuccess) return nullptr;
    b = t.base.emplace(cur, q0).first;
  }
  int slot;
  if (capture == hipStreamCaptureStatusActive) {
    int& n = t.captured[cur];
    if (n >= lite_attn::kQueueSlots - lite_attn::kEagerQueueSlots) return nullptr;
    slot = lite_attn::kEagerQueueSlots + n++;
  } else {
    const auto key = std::make_pair(cur, reinterpret_cast<uintptr_t>(st));
    auto it = t.slot.find(key);
    if (it == t.slot.end()) {
      int& used = t.used[cur];
      if (used >= lite_attn::kEagerQueueSlots) return nullptr;
      it = t.slot.emplace(key, used++).first;
    }
    slot = it->second;
  }
  *n_cu = c->second;
  *slot_out = slot;
  return b->second + 2 * slot;
}

// Compute units of the current device (cached), for a launch that took no tile queue; 0 when the
// device cannot be queried.
int device_cus() {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return 0;
  QueueTable& t = queue_table();
  std::lock_guard<std::mutex> lock(t.mu);
  auto c = t.cus.find(cur);
  if (c == t.cus.end()) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, cur) != hipSuccess)
      return 0;
    c = t.cus.emplace(cur, n).first;
  }
  return c->second;
}

// The most recent attention launch of the calling thread (lite_attn_last_launch).
thread_local int32_t g_last_grid = 0;
thread_local int32_t g_last_queue = -1;

// out is written through the strides it shares with q, k and v, so the map from (b, h, n, d)
// to an element offset must be one to one: every dimension with more than one index needs a
// nonzero stride, and, taken in increasing stride order, each stride must reach past the span
// of the dimension before it (the head dimension is the innermost, stride 1).
bool strides_one_to_one(int64_t B, int64_t H, int64_t N, int64_t D, int64_t sb, int64_t sh,
                        int64_t sn) {
  struct Dim {
    int64_t extent, stride;
  } dims[4] = {{D, 1}, {N, sn}, {H, sh}, {B, sb}};
  Dim live[4];
  int n = 0;
  for (const Dim& d : dims) {
    if (d.extent <= 1) continue;
    if (d.stride <= 0) return false;
    live[n++] = d;
  }
  for (int i = 1; i < n; ++i)   // insertion sort by stride
    for (int j = i; j > 0 && live[j].stride < live[j - 1].stride; --j) std::swap(live[j], live[j - 1]);
  for (int i = 1; i < n; ++i) {
    const __int128 span = (__int128)live[i - 1].stride * live[i - 1].extent;
    if ((__int128)live[i].stride < span) return false;
  }
  return true;
}

// Workspace of lite_attn_step_scheduled_static, for callers that cannot allocate: file-scope
// device memory, one copy per device, held until the process ends. Host code never uses this
// name as an address: the device address is taken once per device, with that device current,
// and passed to the kernels like a caller's workspace. Every call on a device shares the one
// array, so calls that overlap on a device race.
constexpr size_t kStaticWorkspaceBytes = size_t(1) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];

struct ScratchTable {
  std::mutex mu;
  std::map<int, void*> ptr;   // device -> address of its copy of `scratch`
};

ScratchTable& scratch_table() {
  static ScratchTable* t = new ScratchTable;   // never destroyed: usable during static teardown
  return *t;
}

// Device address of `scratch` on the current device (taken on the first call per device).
hipError_t static_workspace(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  ScratchTable& t = scratch_table();
  std::lock_guard<std::mutex> lock(t.mu);
  auto it = t.ptr.find(dev);
  if (it == t.ptr.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    it = t.ptr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return hipSuccess;
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

int lite_attn_last_launch(int32_t* workgroups, int32_t* queue) {
  if (workgroups) *workgroups = g_last_grid;
  if (queue) *queue = g_last_queue;
  return LITE_ATTN_OK;
}

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
    if (!strides_one_to_one(c.batch, c.heads, c.seq_len, c.head_dim, sb, sh, sn))
      return fail(LITE_ATTN_ERR_INVALID_ARG,
                  "create: strides (%lld, %lld, %lld) map two (b, h, n) rows of out to "
                  "overlapping memory",
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
    // The bf16 kernels address one head's K and V rows through a 32-bit buffer offset.
    if (c.dtype == LITE_ATTN_BF16 && c.seq_len > 0 &&
        ((int64_t)c.seq_len - 1) * sn * 2 + (int64_t)c.head_dim * 2 >= (int64_t(1) << 31))
      return fail(LITE_ATTN_ERR_UNSUPPORTED,
                  "create: one head spans %lld bytes with stride_n %lld; the bf16 kernels "
                  "need it below 2^31",
                  (long long)(((int64_t)c.seq_len - 1) * sn * 2 + c.head_dim * 2), (long long)sn);
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
    int slot = -1;
    p.queue = c.dtype == LITE_ATTN_BF16 ? launch_queue(st, &p.n_cu, &slot) : nullptr;
    if (!p.queue) p.n_cu = 0;
    if (scheduled) {
      const int n = c.batch * c.heads * h->Tq;
      // short tiles at the end of the queue: about eight per workgroup slot (two per CU)
      const int tail_max = 16 * (p.n_cu > 0 ? p.n_cu : device_cus());
      const hipError_t e = lite_attn::launch_plan(mask, n, h->Tq, h->W, h->Tk, p.descending,
                                                  tail_max, workspace, st);
      if (e != hipSuccess)
        return fail(LITE_ATTN_ERR_HIP, "%s: schedule launch failed: %s", who,
                    hipGetErrorString(e));
      p.perm = static_cast<const uint32_t*>(workspace);
    }
    unsigned grid = 0;
    const hipError_t e = h->fwd(p, st, &grid);
    if (e != hipSuccess)
      return fail(LITE_ATTN_ERR_HIP, "%s: kernel launch failed: %s", who, hipGetErrorString(e));
    g_last_grid = (int32_t)grid;
    g_last_queue = p.queue ? slot : -1;
    return LITE_ATTN_OK;
  } catch (...) {
    return fail(LITE_ATTN_ERR_HIP, "%s: unexpected exception", who);
  }
}

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Bytes spanned by one output tensor under the handle's strides, rounded up to 256.
size_t output_span_bytes(lite_attn_t h) {
  const lite_attn_config& c = h->cfg;
  if ((int64_t)c.batch * c.heads * c.seq_len == 0) return 0;
  const int64_t elems = (int64_t)(c.batch - 1) * h->sb + (int64_t)(c.heads - 1) * h->sh +
                        (int64_t)(c.seq_len - 1) * h->sn + c.head_dim;
  return round256((size_t)elems * (c.dtype == LITE_ATTN_BF16 ? 2 : 4));
}

int max_abs_diff_impl(const char* who, lite_attn_t h, const void* a, const void* b,
                      float* result, hipStream_t st) {
  const lite_attn_config& c = h->cfg;
  const hipError_t e = lite_attn::launch_output_max_abs_diff(
      a, b, c.dtype == LITE_ATTN_BF16, c.batch, c.heads, c.seq_len, c.head_dim, h->sb, h->sh,
      h->sn, result, st);
  return e == hipSuccess ? LITE_ATTN_OK
                         : fail(LITE_ATTN_ERR_HIP, "%s: reduction launch failed: %s", who,
                                hipGetErrorString(e));
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

int lite_attn_step_scheduled_static(lite_attn_t h, const void* q, const void* k,
                                    const void* v, void* out, uint32_t* mask, float log_eps_t,
                                    int32_t step, void* stream) {
  static const char* who = "step_scheduled_static";
  try {
    if (!h) return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: NULL handle", who);
    const size_t need = lite_attn_workspace_bytes(h);
    if (need > kStaticWorkspaceBytes)
      return fail(LITE_ATTN_ERR_UNSUPPORTED,
                  "%s: the schedule needs %zu bytes of workspace (%lld query tiles); the static "
                  "workspace holds %zu: use lite_attn_step_scheduled with a caller workspace",
                  who, need, (long long)h->cfg.batch * h->cfg.heads * h->Tq,
                  kStaticWorkspaceBytes);
    if ((int64_t)h->cfg.batch * h->cfg.heads * h->cfg.seq_len == 0) return LITE_ATTN_OK;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (st != nullptr && st != hipStreamPerThread) {
      int cur = -1, dev = -2;
      if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(st, &dev) != hipSuccess ||
          dev != cur)
        return fail(LITE_ATTN_ERR_INVALID_ARG,
                    "%s: the stream must belong to the current device (the static workspace "
                    "used is the current device's)", who);
    }
    void* ws = nullptr;
    const hipError_t e = static_workspace(&ws);
    if (e != hipSuccess)
      return fail(LITE_ATTN_ERR_HIP, "%s: static workspace address: %s", who,
                  hipGetErrorString(e));
    return step_impl(who, h, q, k, v, out, mask, log_eps_t, step, ws, true, nullptr, 0.f, false,
                     stream);
  } catch (...) {
    return fail(LITE_ATTN_ERR_HIP, "%s: unexpected exception", who);
  }
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

int lite_attn_output_max_abs_diff(lite_attn_t h, const void* a, const void* b, float* result,
                                  void* stream) {
  static const char* who = "output_max_abs_diff";
  if (!h) return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: NULL handle", who);
  if (!result || !aligned(result, 4))
    return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: NULL or misaligned result", who);
  const lite_attn_config& c = h->cfg;
  if ((int64_t)c.batch * c.heads * c.seq_len > 0 &&
      (!a || !b || !aligned(a, 16) || !aligned(b, 16)))
    return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: NULL or misaligned tensor (16 B needed)", who);
  return max_abs_diff_impl(who, h, a, b, result, static_cast<hipStream_t>(stream));
}

size_t lite_attn_calibrate_workspace_bytes(lite_attn_t h) {
  if (!h) return 0;
  return 4 * output_span_bytes(h) + 2 * round256(lite_attn_mask_bytes(h)) + 256;
}

int lite_attn_calibrate(lite_attn_t h, const void* const* q, const void* const* k,
                        const void* const* v, int32_t steps, const float* error_budgets,
                        const float* candidates, int32_t n_candidates, float* log_eps,
                        float* errors, void* workspace, void* stream) {
  static const char* who = "calibrate";
  try {
    if (!h) return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: NULL handle", who);
    if (steps < 0) return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: negative steps %d", who, steps);
    if (steps == 0) return LITE_ATTN_OK;
    if (!q || !k || !v || !error_budgets || !log_eps || !errors)
      return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: NULL host array", who);
    if (n_candidates < 0 || (n_candidates > 0 && !candidates))
      return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: bad candidate list", who);
    for (int t = 0; t < steps; ++t)
      if (std::isnan(error_budgets[t]))
        return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: error budget %d is NaN", who, t);
    std::vector<float> cands(candidates, candidates + n_candidates);
    for (float x : cands)
      if (std::isnan(x) || x > 0.f)
        return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: candidate %g is not in [-inf, 0]", who,
                    (double)x);
    std::sort(cands.begin(), cands.end(), [](float a, float b) { return a > b; });
    cands.erase(std::unique(cands.begin(), cands.end()), cands.end());  // loosest first

    const hipStream_t st = static_cast<hipStream_t>(stream);
    const lite_attn_config& c = h->cfg;
    const bool empty = (int64_t)c.batch * c.heads * c.seq_len == 0;  // no device call at all
    if (!empty) {
      if (!workspace || !aligned(workspace, 256))
        return fail(LITE_ATTN_ERR_INVALID_ARG, "%s: NULL or not 256-byte aligned workspace",
                    who);
      hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
      if (hipStreamIsCapturing(st, &capture) != hipSuccess)
        return fail(LITE_ATTN_ERR_HIP, "%s: cannot query the stream's capture status", who);
      if (capture != hipStreamCaptureStatusNone)
        return fail(LITE_ATTN_ERR_INVALID_ARG,
                    "%s: the stream is capturing; calibration reads its errors back and cannot "
                    "be recorded into a graph", who);
    }

    const size_t ob = output_span_bytes(h);
    const size_t mask_bytes = lite_attn_mask_bytes(h);
    const size_t mb = round256(mask_bytes);
    uint8_t* w = static_cast<uint8_t*>(workspace);
    void* out_try = w;                 // output of a trial step (discarded)
    void* out_next = w + ob;           // next step's output under a trial mask
    void* dense_cur = w + 2 * ob;      // dense output of the current step
    void* dense_next = w + 3 * ob;     // dense output of the next step
    uint32_t* mask = empty ? nullptr : reinterpret_cast<uint32_t*>(w + 4 * ob);
    uint32_t* m_try = empty ? nullptr : reinterpret_cast<uint32_t*>(w + 4 * ob + mb);
    float* res = empty ? nullptr : reinterpret_cast<float*>(w + 4 * ob + 2 * mb);
    const size_t words = mask_bytes / sizeof(uint32_t);

    auto run = [&](int t, uint32_t* m, float eps, void* out) {
      return step_impl(who, h, q[t], k[t], v[t], out, m, eps, t, nullptr, false, nullptr, 0.f,
                       false, stream);
    };
    auto hip_ok = [&](hipError_t e, const char* what) {
      return e == hipSuccess ? LITE_ATTN_OK
                             : fail(LITE_ATTN_ERR_HIP, "%s: %s: %s", who, what,
                                    hipGetErrorString(e));
    };
    // dense attention of step t (nothing skipped) into out
    auto dense = [&](int t, void* out) {
      int r = hip_ok(lite_attn::launch_mask_fill_zero(m_try, words, st), "mask clear");
      return r != LITE_ATTN_OK ? r : run(t, m_try, -INFINITY, out);
    };
    auto error = [&](const void* a, const void* b, float* err) {
      *err = 0.f;
      if (empty) return (int)LITE_ATTN_OK;
      int r = max_abs_diff_impl(who, h, a, b, res, st);
      if (r != LITE_ATTN_OK) return r;
      r = hip_ok(hipMemcpyAsync(err, res, sizeof(float), hipMemcpyDeviceToHost, st), "read-back");
      return r != LITE_ATTN_OK ? r : hip_ok(hipStreamSynchronize(st), "synchronize");
    };
#define CALIB_TRY(x)                     \
  do {                                   \
    const int r_ = (x);                  \
    if (r_ != LITE_ATTN_OK) return r_;   \
  } while (0)

    // the generation starts with nothing skipped
    CALIB_TRY(hip_ok(lite_attn::launch_mask_fill_zero(mask, words, st), "mask clear"));
    CALIB_TRY(dense(0, dense_cur));
    for (int t = 0; t < steps; ++t) {
      float pick = -INFINITY;
      if (t + 1 < steps) {
        // step t's flags first change step t+1's output: take the loosest candidate whose flags,
        // added to the mask so far, keep step t+1 within its budget
        CALIB_TRY(dense(t + 1, dense_next));
        for (float eps : cands) {
          if (words)
            CALIB_TRY(hip_ok(hipMemcpyAsync(m_try, mask, mask_bytes, hipMemcpyDeviceToDevice, st),
                             "mask copy"));
          CALIB_TRY(run(t, m_try, eps, out_try));
          CALIB_TRY(run(t + 1, m_try, -INFINITY, out_next));
          float err = 0.f;
          CALIB_TRY(error(out_next, dense_next, &err));
          if (err <= error_budgets[t + 1]) {
            pick = eps;
            break;
          }
        }
      } else if (t > 0) {
        pick = log_eps[t - 1];  // the last step's flags change no output
      }
      CALIB_TRY(run(t, mask, pick, out_try));
      CALIB_TRY(error(out_try, dense_cur, &errors[t]));
      log_eps[t] = pick;
      std::swap(dense_cur, dense_next);
    }
#undef CALIB_TRY
    return LITE_ATTN_OK;
  } catch (...) {
    return fail(LITE_ATTN_ERR_NO_MEMORY, "%s: out of host memory", who);
  }
}

}  // extern "C"
