// gfx950 bookkeeping kernels of the LiteAttention step library, kept apart from the attention
// kernel: mask clearing and counting, the schedule of a scheduled step, and the output error of
// the budget calibration.
//
// Method: "LiteAttention: Temporal Sparse Attention for Diffusion Transformers", page 1
// "Architecture Overview" (bitmask or skip list, accumulated-error calibration).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lite_attn_aux.h"

namespace lite_attn {

namespace {

// Bits of mask word w that correspond to real key tiles (< Tk).
__device__ __forceinline__ uint32_t valid_bits(int w, int Tk) {
  const int rem = Tk - 32 * w;
  return rem >= 32 ? 0xffffffffu : (rem <= 0 ? 0u : ((1u << rem) - 1u));
}

// ---------------------------------------------------------------------------------------
// mask bookkeeping kernels
// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) mask_fill_zero(uint32_t* mask, size_t words) {
  for (size_t w = (size_t)blockIdx.x * blockDim.x + threadIdx.x; w < words;
       w += (size_t)gridDim.x * blockDim.x)
    mask[w] = 0u;
}

// Schedule of a step from its visit counts (LiteAttention, page 1 "Architecture Overview": a skip
// list for high sparsity; its list lengths are the per-tile work). A first kernel counts, per
// query tile, the key tiles it will visit. A single workgroup of 1024 threads then orders the
// tiles for the persistent launch in three parts:
//  1. heavy tiles first, in natural order: a tile is heavy when it visits at least half of all
//     key tiles and at least four times the mean count (a dense-prefix row in a sparse step);
//  2. then the middle tiles head by head, heads in decreasing order of their middle work (ties by
//     index), and within a head in the direction of the step's key traversal;
//  3. last, the short tiles, in the step's traversal order: the non-heavy tiles whose count is
//     below a cut, the largest cut that leaves at most min(tail_max, non-heavy / 4) of them.
// Long work starts first, and the launch ends on short tiles, so the workgroups finish close
// together; neighbouring query tiles of a head (which share K/V through the caches) still run
// together in parts 2 and 3. With more than kPlanHeads heads the middle keeps the natural order.
constexpr int kPlanThreads = 1024;
constexpr int kPlanHeads = 1024;
constexpr int kPlanBins = 2 * kPlanThreads;   // visit counts 0 .. 2047 (kMaxTilesK = 2048)

// Per query tile: the number of key tiles it will visit (one thread per tile).
__global__ void __launch_bounds__(256) plan_count(const uint32_t* mask, int n, int W, int Tk,
                                                  uint16_t* count) {
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (x >= n) return;
  const uint32_t* row = mask + (size_t)x * W;
  int c = 0;
  for (int w = 0; w < W; ++w) c += __popc(~row[w] & valid_bits(w, Tk));
  count[x] = (uint16_t)c;
}

// Exclusive scan of v over the 1024 threads of the workgroup (s: kPlanThreads words of LDS).
__device__ uint32_t plan_exclusive_scan(uint32_t v, uint32_t* s) {
  const int t = threadIdx.x;
  s[t] = v;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const uint32_t u = t >= off ? s[t - off] : 0u;
    __syncthreads();
    s[t] += u;
    __syncthreads();
  }
  const uint32_t incl = s[t];
  __syncthreads();
  return incl - v;
}

__global__ void __launch_bounds__(kPlanThreads) plan_order(const uint16_t* count, int n, int Tq,
                                                           int Tk, int descending, int tail_max,
                                                           uint32_t* perm) {
  __shared__ uint32_t s_scan[kPlanThreads];
  __shared__ uint32_t s_hist[kPlanBins];              // counts of the non-heavy tiles
  __shared__ unsigned long long s_work[kPlanHeads];   // middle work per head
  __shared__ uint32_t s_pre[kPlanHeads + 1];          // middle tiles before each head's first
  __shared__ uint32_t s_base[kPlanHeads];             // rank -> head, then head -> first position
  __shared__ unsigned long long s_total;
  __shared__ uint32_t s_heavy, s_cut, s_short;
  const int t = threadIdx.x;
  const int heads = n / Tq;
  const bool by_work = heads <= kPlanHeads;
  // every thread walks a contiguous range of tiles (natural order) in each pass
  const int per = (n + kPlanThreads - 1) / kPlanThreads;
  const int lo = min(n, t * per), hi = min(n, lo + per);
  if (t == 0) {
    s_total = 0ull;
    s_cut = 0u;
  }
  for (int h = t; h < kPlanHeads; h += kPlanThreads) s_work[h] = 0ull;
  for (int c = t; c < kPlanBins; c += kPlanThreads) s_hist[c] = 0u;
  __syncthreads();
  unsigned long long sum = 0ull;
  for (int x = lo; x < hi; ++x) sum += count[x];
  atomicAdd(&s_total, sum);
  __syncthreads();
  // heavy: c >= Tk / 2 and c * n >= 4 * total (exact integer form of "4 x the mean")
  const unsigned long long total = s_total;
  auto heavy = [&](int c) {
    return 2 * c >= Tk && (unsigned long long)c * (unsigned long long)n >= 4ull * total;
  };
  // 1. heavy tiles in natural order; histogram of the others' counts
  uint32_t nh = 0u;
  for (int x = lo; x < hi; ++x) {
    const int c = count[x];
    if (heavy(c)) ++nh;
    else if (c < kPlanBins) atomicAdd(&s_hist[c], 1u);
  }
  uint32_t at = plan_exclusive_scan(nh, s_scan);
  if (t == kPlanThreads - 1) s_heavy = at + nh;
  for (int x = lo; x < hi; ++x)
    if (heavy(count[x])) perm[at++] = (uint32_t)x;
  __syncthreads();
  const uint32_t n_heavy = s_heavy;
  // the cut: the largest c whose tiles below it number at most k
  const uint32_t k = min((uint32_t)max(tail_max, 0), ((uint32_t)n - n_heavy) / 4u);
  {
    const uint32_t h0 = s_hist[2 * t], h1 = s_hist[2 * t + 1];
    const uint32_t below = plan_exclusive_scan(h0 + h1, s_scan);   // tiles with count < 2t
    uint32_t cut = 0u;
    if (below <= k) cut = 2u * t;
    if (below + h0 <= k) cut = 2u * t + 1u;
    if (t == kPlanThreads - 1 && below + h0 + h1 <= k) cut = kPlanBins;
    atomicMax(&s_cut, cut);
  }
  __syncthreads();
  const int cut = (int)s_cut;
  auto is_short = [&](int c) { return c < cut && !heavy(c); };
  // 3. short tiles last, in traversal order
  uint32_t ns = 0u, nm = 0u;
  for (int x = lo; x < hi; ++x) {
    const int c = count[x];
    if (is_short(c)) ++ns;
    else if (!heavy(c)) ++nm;
  }
  uint32_t sp = plan_exclusive_scan(ns, s_scan);
  if (t == kPlanThreads - 1) s_short = sp + ns;
  __syncthreads();
  const uint32_t n_short = s_short;
  for (int x = lo; x < hi; ++x)
    if (is_short(count[x])) {
      const uint32_t idx = sp++;
      perm[(uint32_t)n - n_short + (descending ? n_short - 1u - idx : idx)] = (uint32_t)x;
    }
  auto middle = [&](int c) { return !heavy(c) && !is_short(c); };
  // 2. the middle tiles: their natural-order prefix count, per-head starts and work
  uint32_t pre = plan_exclusive_scan(nm, s_scan);
  const uint32_t pre_lo = pre;
  if (!by_work) {   // natural head order
    for (int x = lo; x < hi; ++x)
      if (middle(count[x])) perm[n_heavy + pre++] = (uint32_t)x;
    return;
  }
  {
    unsigned long long w = 0ull;
    int h_cur = lo < hi ? lo / Tq : 0;
    for (int x = lo; x < hi; ++x) {
      const int h = x / Tq;
      if (h != h_cur) {
        atomicAdd(&s_work[h_cur], w);
        w = 0ull;
        h_cur = h;
      }
      if (x == h * Tq) s_pre[h] = pre;
      const int c = count[x];
      if (middle(c)) {
        w += (unsigned long long)c;
        ++pre;
      }
    }
    if (lo < hi) atomicAdd(&s_work[h_cur], w);
    if (hi == n && lo < hi) s_pre[heads] = pre;
    if (n == 0 && t == 0) s_pre[0] = 0u;
  }
  __syncthreads();
  // rank of each head: heavier first, ties by index
  for (int h = t; h < heads; h += kPlanThreads) {
    const unsigned long long w = s_work[h];
    uint32_t rank = 0u;
    for (int g = 0; g < heads; ++g) {
      const unsigned long long wg = s_work[g];
      rank += (wg > w || (wg == w && g < h)) ? 1u : 0u;
    }
    s_base[rank] = (uint32_t)h;   // rank -> head
  }
  __syncthreads();
  uint32_t my_head = 0u, my_rest = 0u;
  if (t < heads) {
    my_head = s_base[t];
    my_rest = s_pre[my_head + 1] - s_pre[my_head];
  }
  __syncthreads();
  const uint32_t before = plan_exclusive_scan(my_rest, s_scan);
  if (t < heads) s_base[my_head] = n_heavy + before;   // head -> first position
  __syncthreads();
  // each head's middle tiles in the direction of the step's key traversal
  pre = pre_lo;
  for (int x = lo; x < hi; ++x) {
    if (!middle(count[x])) continue;
    const int h = x / Tq;
    const uint32_t within = pre++ - s_pre[h];
    const uint32_t rest = s_pre[h + 1] - s_pre[h];
    perm[s_base[h] + (descending ? rest - 1u - within : within)] = (uint32_t)x;
  }
}

__global__ void __launch_bounds__(256) mask_popcount(const uint32_t* mask, uint32_t* counts,
                                                     int Tq, int Tk, int W) {
  __shared__ uint32_t s_sum;
  if (threadIdx.x == 0) s_sum = 0u;
  __syncthreads();
  const size_t words = (size_t)Tq * W;
  const uint32_t* base = mask + (size_t)blockIdx.x * words;
  uint32_t acc = 0u;
  for (size_t w = threadIdx.x; w < words; w += blockDim.x)
    acc += __popc(base[w] & valid_bits((int)(w % (size_t)W), Tk));
  atomicAdd(&s_sum, acc);
  __syncthreads();
  if (threadIdx.x == 0) counts[blockIdx.x] = s_sum;
}

// Largest |a - b| over the valid elements of two outputs laid out by the shared strides, the
// error measure of the per-step budget calibration (LiteAttention, page 1 "Architecture
// Overview": accumulated-error calibration). Each difference is taken in fp32; |d| is compared
// as its bit pattern, which orders non-negative floats like their values and puts NaN above
// +inf, so a NaN anywhere is reported as NaN. *result must hold 0 before the launch.
template <bool BF16>
__global__ void __launch_bounds__(256) output_max_abs_diff(const uint4* a, const uint4* b,
                                                           int64_t chunks, int per_row, int H,
                                                           int N, int64_t sb, int64_t sh,
                                                           int64_t sn, uint32_t* result) {
  constexpr int kElems = BF16 ? 8 : 4;  // elements per 16-byte chunk
  uint32_t m = 0u;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = c / per_row;
    const int part = (int)(c - row * per_row);
    const int n = (int)(row % N);
    const int64_t bh = row / N;
    const int64_t off =
        ((bh / H) * sb + (bh % H) * sh + (int64_t)n * sn + (int64_t)part * kElems) / kElems;
    const uint4 x = a[off], y = b[off];
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (BF16) {
        const float d0 = __uint_as_float(xs[w] << 16) - __uint_as_float(ys[w] << 16);
        const float d1 =
            __uint_as_float(xs[w] & 0xffff0000u) - __uint_as_float(ys[w] & 0xffff0000u);
        m = max(m, max(__float_as_uint(fabsf(d0)), __float_as_uint(fabsf(d1))));
      } else {
        m = max(m, __float_as_uint(fabsf(__uint_as_float(xs[w]) - __uint_as_float(ys[w]))));
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  __shared__ uint32_t s_max[4];
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax(result, max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3])));
}

}  // namespace

hipError_t launch_mask_fill_zero(uint32_t* mask, size_t words, hipStream_t stream) {
  if (words == 0) return hipSuccess;
  size_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  void* args[] = {&mask, &words};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mask_fill_zero), dim3((unsigned)blocks),
                         dim3(256), args, 0, stream);
}

size_t plan_workspace_bytes(int64_t n_tiles) {
  return ((size_t)n_tiles * 4 + 255) / 256 * 256 + ((size_t)n_tiles * 2 + 255) / 256 * 256;
}

hipError_t launch_plan(const uint32_t* mask, int n_tiles, int Tq, int W, int Tk, int descending,
                       int tail_max, void* workspace, hipStream_t stream) {
  if (n_tiles == 0) return hipSuccess;
  uint32_t* perm = static_cast<uint32_t*>(workspace);
  uint16_t* count = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(workspace) +
                                                ((size_t)n_tiles * 4 + 255) / 256 * 256);
  void* cargs[] = {&mask, &n_tiles, &W, &Tk, &count};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&plan_count),
                                 dim3((unsigned)((n_tiles + 255) / 256)), dim3(256), cargs, 0,
                                 stream);
  if (e != hipSuccess) return e;
  const uint16_t* ccount = count;
  void* args[] = {&ccount, &n_tiles, &Tq, &Tk, &descending, &tail_max, &perm};
  return hipLaunchKernel(reinterpret_cast<const void*>(&plan_order), dim3(1),
                         dim3(kPlanThreads), args, 0, stream);
}

hipError_t launch_output_max_abs_diff(const void* a, const void* b, bool bf16, int B, int H,
                                      int N, int D, int64_t sb, int64_t sh, int64_t sn,
                                      float* result, hipStream_t stream) {
  uint32_t* res = reinterpret_cast<uint32_t*>(result);
  hipError_t e = launch_mask_fill_zero(res, 1, stream);
  if (e != hipSuccess) return e;
  int per_row = D / (bf16 ? 8 : 4);
  int64_t chunks = (int64_t)B * H * N * per_row;
  if (chunks == 0) return hipSuccess;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  const uint4* pa = static_cast<const uint4*>(a);
  const uint4* pb = static_cast<const uint4*>(b);
  void* args[] = {&pa, &pb, &chunks, &per_row, &H, &N, &sb, &sh, &sn, &res};
  const void* fn = bf16 ? reinterpret_cast<const void*>(&output_max_abs_diff<true>)
                        : reinterpret_cast<const void*>(&output_max_abs_diff<false>);
  return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(256), args, 0, stream);
}

hipError_t launch_mask_popcount(const uint32_t* mask, uint32_t* counts, int heads_total, int Tq,
                                int Tk, int W, hipStream_t stream) {
  if (heads_total == 0) return hipSuccess;
  void* args[] = {&mask, &counts, &Tq, &Tk, &W};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mask_popcount), dim3((unsigned)heads_total),
                         dim3(256), args, 0, stream);
}

}  // namespace lite_attn
