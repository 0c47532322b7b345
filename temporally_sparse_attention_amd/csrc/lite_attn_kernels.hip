// gfx950 (CDNA4) kernels of the LiteAttention step: tiled softmax attention with the QK-Skip
// test inside the online-softmax pipeline and a persistent per-(b, h, query tile, key tile)
// skip bitmask.
//
// Method: "LiteAttention: Temporal Sparse Attention for Diffusion Transformers", page 1
// "Core Concept" (QK-Skip: a tile whose local maximum score is far below the cumulative
// maximum is flagged, and the flag persists across denoising steps) and "Architecture
// Overview" (bitmask, skip logic inside the FlashAttention softmax pipeline).
//
// Work decomposition. A workgroup owns one query tile (b, h, i) at a time and is the only reader
// and writer of that tile's mask row, so the mask needs no atomics. The grid is persistent:
// workgroups take tiles from a queue, one atomic add per tile. Each 64-lane wave owns 32 query
// rows. Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: the
// accumulator then holds one query per lane (lane % 32) and 16 keys per register group, so the
// row maximum and row sum of the online softmax are in-lane reductions plus a single swap
// between the two half-waves (v_permlane32_swap). The PV product is likewise computed
// transposed, O^T += V^T P^T, which takes P straight from the score registers (converted to
// bf16) as the B operand; V stays row-major in LDS and the A operand is read with
// ds_read_b64_tr_b16, which transposes as it reads. The key order
// inside a 16-key MFMA step is permuted identically on both operands, which leaves the
// contraction unchanged.
//
// The QK-Skip vote needs nothing beyond the online softmax: the tile's row maximum mt is
// already computed for the rescale, and the running maximum m is the softmax state. A wave
// votes "keep" when any of its valid rows has (mt - m) * scale >= log_eps (or NaN). Each wave
// collects its votes as scalar bits by position in the visiting list; after the tile loop the
// workgroup ORs them, and a visited tile is flagged when no wave voted keep. (With in-step skip
// the votes go to an LDS bitset at once, since later tiles of the same step read them.)
//
// Skipped tiles cost nothing: the mask row is turned into a compact visiting list in LDS
// before any K/V load, and the K/V pipeline only ever fetches listed tiles.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "lite_attn_internal.h"

namespace lite_attn {

// Tile queues of persistent launches, kQueueSlots pairs (next tile, finished workgroups) per
// device. Zero at load; every persistent launch leaves its pair at zero when it ends.
__device__ uint32_t g_tile_queues[2 * kQueueSlots];

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BK = kTileK;

// ---------------------------------------------------------------------------------------
// small helpers
// ---------------------------------------------------------------------------------------

// Bits of mask word w that correspond to real key tiles (< Tk).
__device__ __forceinline__ uint32_t valid_bits(int w, int Tk) {
  const int rem = Tk - 32 * w;
  return rem >= 32 ? 0xffffffffu : (rem <= 0 ? 0u : ((1u << rem) - 1u));
}

// Bits of word w for key tiles j < jp (the exempt columns of a dense prefix).
__device__ __forceinline__ uint32_t low_bits(int w, int jp) {
  const int rem = jp - 32 * w;
  return rem >= 32 ? 0xffffffffu : (rem <= 0 ? 0u : ((1u << rem) - 1u));
}

// IEEE 754-2019 maximum: a NaN operand gives NaN (v_maximum3_f32 on gfx950). Row maxima use it,
// so that a NaN score makes the row's maximum, and with it the QK-Skip margin, NaN: such a tile
// is never flagged.
__device__ __forceinline__ float nanmax(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// Value of x in the other half-wave (lane ^ 32) combined with x by max / sum.
__device__ __forceinline__ float halves_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return nanmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wave 0's share of a mask row: lane l holds words 2l and 2l+1 (clamped into the row, W >= 1,
// so that both loads are always in flight together; W <= 128). Other waves load nothing.
__device__ __forceinline__ void load_mask_words(const uint32_t* mrow, int W, uint32_t& r0,
                                                uint32_t& r1) {
  if (threadIdx.x < 64) {
    r0 = mrow[min(2 * (int)threadIdx.x, W - 1)];
    r1 = mrow[min(2 * (int)threadIdx.x + 1, W - 1)];
  }
}

// Turn a mask row (its words as load_mask_words holds them) into the list of key tiles to
// visit, in traversal order. Runs on wave 0, which also keeps the row's words in `old` for the
// mask update at the end of the tile; every thread clears the keep bitset. Ends with a
// workgroup barrier; returns the list length.
template <int NT>
__device__ int build_visit_list(uint32_t r0, uint32_t r1, int W, int Tk, bool descending,
                                uint16_t* list, uint32_t* keep, uint32_t* old, int* s_count) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int lane = tid;
    const int w0 = 2 * lane, w1 = 2 * lane + 1;
    if (w0 < W) old[w0] = r0;
    if (w1 < W) old[w1] = r1;
    uint32_t b0 = w0 < W ? (~r0 & valid_bits(w0, Tk)) : 0u;
    uint32_t b1 = w1 < W ? (~r1 & valid_bits(w1, Tk)) : 0u;
    const int cnt = __popc(b0) + __popc(b1);
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    const int total = __shfl(incl, 63, 64);
    int pos = incl - cnt;
    while (b0) {
      const int bit = __builtin_ctz(b0);
      b0 &= b0 - 1u;
      list[descending ? total - 1 - pos : pos] = (uint16_t)(32 * w0 + bit);
      ++pos;
    }
    while (b1) {
      const int bit = __builtin_ctz(b1);
      b1 &= b1 - 1u;
      list[descending ? total - 1 - pos : pos] = (uint16_t)(32 * w1 + bit);
      ++pos;
    }
    if (lane == 0) *s_count = total;
  }
  for (int w = tid; w < W; w += NT) keep[w] = 0u;
  __syncthreads();
  return *s_count;
}

// Fold this step's flags into the mask row: flags = visited & ~keep & ~exempt. `old` holds the
// row as it was at the start of the tile (only this workgroup writes the row).
template <int NT>
__device__ void write_mask_row(uint32_t* mrow, int W, int Tk, const uint32_t* old,
                               const uint32_t* keep, bool row_exempt, int exempt_cols) {
  if (row_exempt) return;
  for (int w = threadIdx.x; w < W; w += NT) {
    const uint32_t visited = ~old[w] & valid_bits(w, Tk);
    const uint32_t flags = visited & ~keep[w] & ~low_bits(w, exempt_cols);
    if (flags) mrow[w] = old[w] | flags;
  }
}

// Divergence-triggered refresh (LiteAttention, page 1 "Core Concept": the mask is updated only
// when the attention pattern diverges significantly; "Architecture Overview": decisions carry
// forward unless the attention distribution shifts). The statistic of the query tile is the
// mean over its valid rows of the running row maximum m (raw scores; times `scale` gives
// scaled units), taken after the tile loop. With no reference yet (NaN) it becomes the
// reference; when it moves by more than `delta` (or the move is NaN) the reference is dropped
// and the mask row is cleared instead of updated. Every thread calls this after the final
// barrier of the tile loop; returns true when the row is to be cleared. Each wave's lanes 0..31
// hold its 32 rows (lanes 32..63 hold copies), so wave sums are added in wave order: the
// statistic is the same on every run.
template <int NW>
__device__ bool refresh_decision(float m_run, bool row_valid, int valid_rows, float scale,
                                 float delta, float* stat_slot, float* s_part, int* s_clear) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float v = (lane < 32 && row_valid) ? m_run : 0.f;
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  if (lane == 0) s_part[wave] = v;
  __syncthreads();
  if (tid == 0) {
    float total = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) total += s_part[w];
    const float stat = total / (float)valid_rows * scale;
    const float ref = *stat_slot;
    int clear = 0;
    if (ref != ref) {
      *stat_slot = stat;
    } else if (!(fabsf(stat - ref) <= delta)) {
      *stat_slot = __builtin_nanf("");
      clear = 1;
    }
    *s_clear = clear;
  }
  __syncthreads();
  return *s_clear != 0;
}

// Clears the valid bits of a mask row (reserved bits stay as they are: zero).
template <int NT>
__device__ void clear_mask_row(uint32_t* mrow, int W, int Tk, const uint32_t* old) {
  for (int w = threadIdx.x; w < W; w += NT) mrow[w] = old[w] & ~valid_bits(w, Tk);
}

// ---------------------------------------------------------------------------------------
// bf16 kernel: MFMA 32x32x16 bf16, software-pipelined across key tiles; K/V streamed straight
// into LDS (double-buffered) with buffer loads; one workgroup barrier per visited tile.
// ---------------------------------------------------------------------------------------
//
// Work split. A workgroup owns one query tile (tile_q = 32 * NW rows) and runs NW waves; wave w
// owns query rows 32w .. 32w+31 and every key of every visited tile.
//
// Pipelining. A wave overlaps its own MFMAs with independent VALU work well, but within one
// tile the softmax depends on the scores and the PV product on the softmax. So iteration n
// works on two tiles at once:
//   phase 1: exponentials and bf16 weights P(n) (VALU)  ||  S(n+1) = K(n+1) Q^T (MFMA)
//   phase 2: O += V(n)^T P(n)^T (MFMA)                   ||  row maxima of S(n+1) (VALU)
//   between: QK-Skip vote and the lazy rescale for tile n+1 (short, branchy, rare work).
// K runs one tile ahead of V: during iteration n the workgroup reads K(n+1) and V(n) and loads
// K(n+2) and V(n+1) into the other stages.
//
// LDS layouts (bf16, row-major [64 keys][D], rows padded):
//  K rows are D*2 + 16 bytes apart: the S^T operand read has 32 lanes reading one 16-byte
//  column chunk of 32 consecutive rows, and the 16-byte skew puts every 8 consecutive rows on
//  distinct banks.
//  V rows are D*2 + 32 bytes apart. The V^T operand is read with ds_read_b64_tr_b16: each
//  16-lane group reads 4 consecutive rows x 32 bytes and receives them transposed (lane i gets
//  column i of the 4 rows); the 32-byte skew spreads the 4 row segments over the banks.
//  Both keep every operand address a per-lane base plus a compile-time offset.
//  The tiles are written by buffer_load_dwordx4 ... lds: each instruction deposits 64 lanes x
//  16 bytes contiguously, so each 16-byte LDS slot is filled by the lane whose source offset is
//  the matching (row, chunk) of global memory; padding slots read an out-of-range offset and
//  receive zeros without touching memory. Keys >= N lie outside the buffer range and read as
//  zeros too.
template <int D>
struct Bf16TileGeom {
  static constexpr int CH = D / 8;           // 16-byte chunks of one K or V row
  static constexpr int KCH = CH + 1;         // padded K row, in chunks
  static constexpr int VCH = CH + 2;         // padded V row, in chunks
  static constexpr int KROW = KCH * 16;      // bytes
  static constexpr int VROW = VCH * 16;
  static constexpr int K_BYTES = BK * KROW;
  static constexpr int V_BYTES = BK * VROW;
};

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr uint32_t kOobOffset = 0x7ffffff0u;   // beyond every buffer range used here

// Device-only helpers and kernel bodies below use AMDGPU buffer-resource types that the host
// compilation pass cannot represent; the host pass only needs the kernels' launch stubs.
#if defined(__HIP_DEVICE_COMPILE__)
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource (4 SGPRs) over [base, base + bytes): stride 0, so reads at offsets
// >= bytes return zero.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from the buffer at byte offset voff straight into LDS: lane l's data lands
// at lds_a + lds_b + 16 * l. Issued as inline assembly so that the compiler does not track
// these loads as LDS writes: the kernel orders them itself (each wave waits for its own loads
// with s_waitcnt vmcnt(0) before the workgroup barrier that precedes any read of the stage),
// and the compiler would otherwise make unrelated LDS accesses wait for every load in flight.
// The LDS address is summed into M0 inside the block (a per-wave base plus a constant), which
// keeps the many loop-invariant addresses out of scalar registers. The instruction has no
// register result, and M0 is declared clobbered.
__device__ __forceinline__ void lds_dma16(const i32x4& rsrc, uint32_t lds_a, uint32_t lds_b,
                                          uint32_t voff, uint32_t soff) {
  asm volatile(
      "s_add_u32 m0, %0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %2, %3, %4 offen lds"
      :
      : "s"(lds_a), "s"(lds_b), "v"(voff), "s"(rsrc), "s"(soff)
      : "memory", "m0", "scc");
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}
#endif

// The launch parameters as the kernel received them, read through scalar loads.
typedef const FwdParams __attribute__((address_space(4))) ArgParams;

// Tile position of queue entry w (persistent launches without a schedule). The dense-prefix
// query tiles (P per head) never skip: they are the longest, and go first, head by head, so
// that none of them starts last. The other tiles follow in the direction of the step's key
// traversal (measured: +3% on a descending step with 39% of tiles skipped, neutral elsewhere).
// With a schedule, the entry is the position in the schedule.
template <int NW>
__device__ __forceinline__ uint32_t queue_position(ArgParams& p, uint32_t w) {
  if (p.perm != nullptr) return w;
  const uint32_t n_tiles = (uint32_t)(p.B * p.H * p.Tq);
  const uint32_t Tq = (uint32_t)p.Tq;
  const uint32_t P = min(Tq, (uint32_t)((p.dense_prefix + NW * 32 - 1) / (NW * 32)));
  const uint32_t n_pre = (uint32_t)(p.B * p.H) * P;
  if (w < n_pre) return (w / P) * Tq + w % P;
  uint32_t r = w - n_pre;                        // among the B*H*(Tq-P) other tiles
  if (p.descending) r = n_tiles - n_pre - 1u - r;
  return (r / (Tq - P)) * Tq + P + r % (Tq - P);
}

// What a query tile needs before its first K/V load: the wave's Q rows as MFMA B operands
// (lane holds features 16c + 8*half .. +7 of query row l32, for every 16-feature step c) and,
// on wave 0, its share of the tile's mask row; both are loaded together, so that the two
// memory latencies overlap.
template <int D>
struct TileInputs {
  bf16x8 qf[D / 16];
  uint32_t m0, m1;
};

template <int D, int NW>
__device__ __forceinline__ void load_tile_inputs(ArgParams& p, uint32_t pos, TileInputs<D>& in) {
  const uint32_t tile = p.perm ? p.perm[pos] : pos;
  const int i = (int)(tile % (uint32_t)p.Tq);
  const int bh = (int)(tile / (uint32_t)p.Tq);
  const int b = bh / p.H, h = bh % p.H;
  const __bf16* qh = static_cast<const __bf16*>(p.q) + (int64_t)b * p.sb + (int64_t)h * p.sh;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) & (NW - 1);
  const int qrow = i * NW * 32 + wave * 32 + (lane & 31);
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    if (qrow < p.N) {
      in.qf[c] = *reinterpret_cast<const bf16x8*>(qh + (int64_t)qrow * p.sn + 16 * c +
                                                  8 * (lane >> 5));
    } else {
      in.qf[c] = bf16x8{};
    }
  }
  load_mask_words(p.mask + (size_t)tile * p.W, p.W, in.m0, in.m1);
}

// One query tile. `args` is the address of the kernel's argument segment (the FwdParams), `w_in`
// the tile's position (in the schedule when there is one), `in` its inputs, already loaded.
// Inlined into the out-of-line drivers below, which the kernel calls (one instantiation per
// configuration, so both drivers share its LDS arrays; s_next is a constant at each call site).
// With s_next (persistent launches), thread 0 takes the next queue entry when the tile loop
// ends and publishes it through *s_next; the tile returns that entry, the same value in every
// thread (>= B*H*Tq: the queue is empty). Without it, returns 0. Measured alternatives: taking
// the entry when the tile starts was 3-5% slower on sparse steps (a reserved tile waits for its
// workgroup while others go idle), and loading the next tile's Q rows before this tile's
// epilogue was 7-9% slower (Q registers carried from one tile to the next cost the tile loop
// its pinned MFMA/VALU interleave).
template <int D, int NW, bool INSTEP>
__device__ __forceinline__ uint32_t bf16_tile_body(uint64_t args, uint32_t w_in,
                                                   TileInputs<D>& in, uint32_t* s_next) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t a_lo = __builtin_amdgcn_readfirstlane((uint32_t)args);
  const uint32_t a_hi = __builtin_amdgcn_readfirstlane((uint32_t)(args >> 32));
  ArgParams& p = *(ArgParams*)(((uint64_t)a_hi << 32) | a_lo);
  const uint32_t w = __builtin_amdgcn_readfirstlane(w_in);
  using G = Bf16TileGeom<D>;
  constexpr int NT = NW * 64;
  constexpr int BQ = NW * 32;

  // One LDS object per stage: every operand read and every tile load names its stage
  // statically (the tile loop is unrolled by two), so the compiler can tell that the loads
  // filling one stage never alias the reads of the other and needs no wait between them.
  __shared__ __attribute__((aligned(16))) unsigned char s_k0[G::K_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char s_k1[G::K_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char s_v0[G::V_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char s_v1[G::V_BYTES];
  __shared__ uint16_t s_list[kMaxTilesK + 8];   // +8: the loop reads a few entries ahead
  __shared__ uint32_t s_keep[kMaxWords];
  __shared__ uint64_t s_wkeep[NW][kMaxTilesK / 64];   // per-wave keep votes by list position
  __shared__ uint32_t s_old[kMaxWords];                // the mask row at the start of the tile
  __shared__ int s_count;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (NW - 1);   // scalar
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // Position = logical tile (b * H + h) * Tq + i, unless a schedule permutes them.
  const uint32_t tile = p.perm ? p.perm[w] : w;
  const int i = (int)(tile % (uint32_t)p.Tq);
  const int bh = (int)(tile / (uint32_t)p.Tq);
  const int b = bh / p.H, h = bh % p.H;
  const int64_t head_off = (int64_t)b * p.sb + (int64_t)h * p.sh;
  const __bf16* __restrict__ kh = static_cast<const __bf16*>(p.k) + head_off;
  const __bf16* __restrict__ vh = static_cast<const __bf16*>(p.v) + head_off;
  __bf16* __restrict__ oh = static_cast<__bf16*>(p.out) + head_off;
  uint32_t* mrow = p.mask + (size_t)tile * p.W;
  const int N = p.N;
  const int64_t sn = p.sn;
  const uint32_t row_bytes = (uint32_t)sn * 2u;

  const int qrow = i * BQ + wave * 32 + l32;
  const bool row_valid = qrow < N;
  bf16x8 (&qf)[D / 16] = in.qf;

  const int cnt = build_visit_list<NT>(in.m0, in.m1, p.W, p.Tk, p.descending != 0, s_list,
                                       s_keep, s_old, &s_count);

  // Consume Q here: the compiler then waits for these loads once, before the tile loop, rather
  // than at the loop's first MFMA on every iteration (where the wait would also cover the K/V
  // tile loads in flight).
#pragma unroll
  for (int c = 0; c < D / 16; ++c) asm volatile("" ::"v"(qf[c]));

  // Per-lane source offsets of this wave's share of the tile loads (loop invariant). Load
  // instruction x (64 lanes) fills the 16-byte slots [64x, 64x + 64) of a tile; instructions
  // are dealt round-robin to the waves.
  constexpr int KLOADS = (G::KCH + NW - 1) / NW;
  constexpr int VLOADS = (G::VCH + NW - 1) / NW;
  uint32_t koff[KLOADS], voff[VLOADS];
#pragma unroll
  for (int n = 0; n < KLOADS; ++n) {
    const int slot = 64 * (wave + NW * n) + lane;
    const int row = slot / G::KCH, ch = slot % G::KCH;
    koff[n] = ch < G::CH ? (uint32_t)row * row_bytes + 16u * ch : kOobOffset;
  }
#pragma unroll
  for (int n = 0; n < VLOADS; ++n) {
    const int slot = 64 * (wave + NW * n) + lane;
    const int row = slot / G::VCH, ch = slot % G::VCH;
    voff[n] = ch < G::CH ? (uint32_t)row * row_bytes + 16u * ch : kOobOffset;
  }
  const uint32_t wave1k = 1024u * wave;   // this wave's first 1 KB slot of a stage
  // One buffer resource per tensor covers the head's N rows, built once per query tile: rows
  // >= N of the ragged last tile lie past its end and read as zeros, and a tile load only adds
  // the tile's first row as a scalar offset (the head's span is below 2^31 bytes, checked when
  // the handle is created, so no offset wraps).
  const uint32_t head_bytes = (uint32_t)(N - 1) * row_bytes + D * 2;
  const i32x4 rk = make_rsrc(kh, head_bytes);
  const i32x4 rv = make_rsrc(vh, head_bytes);
  auto issue_k = [&](int j, unsigned char* dst) {
    const uint32_t soff = (uint32_t)(j * BK) * row_bytes;
    const uint32_t base = lds_address(dst);
#pragma unroll
    for (int n = 0; n < KLOADS; ++n) {
      const int x = wave + NW * n;
      if (KLOADS * NW == G::KCH || x < G::KCH) lds_dma16(rk, wave1k, base + NW * n * 1024, koff[n], soff);
    }
  };
  auto issue_v = [&](int j, unsigned char* dst) {
    const uint32_t soff = (uint32_t)(j * BK) * row_bytes;
    const uint32_t base = lds_address(dst);
#pragma unroll
    for (int n = 0; n < VLOADS; ++n) {
      const int x = wave + NW * n;
      if (VLOADS * NW == G::VCH || x < G::VCH) lds_dma16(rv, wave1k, base + NW * n * 1024, voff[n], soff);
    }
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};

  float m_run = -INFINITY;   // running row maximum of raw scores (the QK-Skip reference)
  float m_ref = -INFINITY;   // exponent reference of the accumulators (lags m_run by < 2^8)
  float l_run = 0.f;         // this lane's partial row sum
  const float c2 = p.scale_log2;
  const float inv_c2 = 1.f / c2;
  // In a register rather than a literal: the row-sum v_dot2 then encodes in 4 bytes instead of 8
  // (measured +1% on the 75600-token workload, from its sparse steps).
  bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  asm volatile("" : "+v"(ones));

  // Software pipeline. Iteration n of the tile loop overlaps the matrix work of one tile with
  // the vector work of another, so that a wave keeps the MFMA pipe busy while it computes its
  // own softmax:
  //   phase A: MFMAs of S^T for tile n+1  ||  exponentials, bf16 packing, row sums of tile n
  //   phase B: MFMAs of O^T += V^T P^T for tile n  ||  scaling and row maxima of tile n+1
  // Stages: K(n+1) and V(n) are resident during iteration n; K(n+2) and V(n+1) are loaded into
  // the other stages meanwhile (the stages they overwrite were last read in iteration n-1,
  // which the barrier at the top of the iteration has closed).

  // Operand reads. K operand for key block kb, feature step c: key row 32kb + l32, chunk
  // 2c + half. V^T operand for feature block db and 16-key step kc: two transposed 4-row reads
  // at key rows 16kc + 4*half (+8), columns 32db + 16*(g16 & 1) + 4*(lane & 3) of each 16-lane
  // group g16.
  const int k_rd = l32 * G::KROW + 16 * half;
  const int g16 = lane >> 4, gi = lane & 15;
  const int v_rd = (4 * half + (gi >> 2)) * G::VROW + 2 * (16 * (g16 & 1) + 4 * (gi & 3));
  auto kread = [&](const unsigned char* kst, int t) {   // t -> key block t & 1, feature step t >> 1
    return *reinterpret_cast<const bf16x8*>(kst + k_rd + (t & 1) * 32 * G::KROW + 32 * (t >> 1));
  };
  auto vread = [&](const unsigned char* vst, int t) {   // t -> feature block t % (D/32), keys t / (D/32)
    const int db = t % (D / 32), kc = t / (D / 32);
    const unsigned char* base = vst + v_rd + kc * 16 * G::VROW + db * 64;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)base);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(base + 8 * G::VROW));
    const bf16x4 lo4 = __builtin_bit_cast(bf16x4, lo), hi4 = __builtin_bit_cast(bf16x4, hi);
    bf16x8 av;
    av[0] = lo4[0]; av[1] = lo4[1]; av[2] = lo4[2]; av[3] = lo4[3];
    av[4] = hi4[0]; av[5] = hi4[1]; av[6] = hi4[2]; av[7] = hi4[3];
    return av;
  };
  constexpr int RING = 4;   // operand reads in flight ahead of their MFMA

  // S^T = K Q^T for keys 32kb + 8(r/4) + 4*half + (r%4) of a tile, query l32 (lane). The 16
  // MFMAs alternate between the two key blocks. No scheduling directives: callers interleave.
  auto qk_mfma = [&](const unsigned char* kst, f32x16 (&sc)[2]) {
    bf16x8 kr[RING];
#pragma unroll
    for (int t = 0; t < RING; ++t) kr[t] = kread(kst, t);
    sc[0] = f32x16{};
    sc[1] = f32x16{};
#pragma unroll
    for (int t = 0; t < D / 8; ++t) {
      sc[t & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[t % RING], qf[t >> 1], sc[t & 1], 0, 0, 0);
      if (t + RING < D / 8) kr[t % RING] = kread(kst, t + RING);
    }
  };
  // O^T += V^T P^T: lane holds query l32 and features 32db + 8(r/4) + 4*half + (r%4).
  // The same with the first RING operands already read (early V reads, see phase_a_sched_v).
  auto pv_mfma_pre = [&](const unsigned char* vst, const bf16x8 (&pb)[4], bf16x8 (&vr)[RING]) {
#pragma unroll
    for (int t = 0; t < D / 8; ++t) {
      const int db = t % (D / 32), kc = t / (D / 32);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[t % RING], pb[kc], o[db], 0, 0, 0);
      if (t + RING < D / 8) vr[t % RING] = vread(vst, t + RING);
    }
  };
  auto pv_mfma = [&](const unsigned char* vst, const bf16x8 (&pb)[4]) {
    bf16x8 vr[RING];
#pragma unroll
    for (int t = 0; t < RING; ++t) vr[t] = vread(vst, t);
#pragma unroll
    for (int t = 0; t < D / 8; ++t) {
      const int db = t % (D / 32), kc = t / (D / 32);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[t % RING], pb[kc], o[db], 0, 0, 0);
      if (t + RING < D / 8) vr[t % RING] = vread(vst, t + RING);
    }
  };
  // Keys >= N of the ragged last tile do not exist: their scores become -inf.
  auto mask_ragged = [&](int j, f32x16 (&sc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (j * BK + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3) >= N) sc[kb][r] = -INFINITY;
  };
  // Scores to exp2 units relative to the exponent reference, in place (t = s * c2 - m_ref * c2),
  // and the tile's row maximum in raw units. The maximum is taken on the results of the
  // arithmetic, which needs no NaN quieting (taking it on the raw MFMA results would cost one
  // extra instruction per score); the raw maximum is recovered from it. Returns the maximum in
  // exp2 units through tm.
  auto scale_max = [&](f32x16 (&s)[2], float nb, float& tm) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = fmaf(s[kb][r], c2, nb);
    // two chains of three-input maxima (v_maximum3_f32): 16 instructions for 32 scores
    float tm0 = nanmax(nanmax(s[0][0], s[1][0]), s[0][2]);
    float tm1 = nanmax(nanmax(s[0][1], s[1][1]), s[1][2]);
#pragma unroll
    for (int r = 3; r < 16; r += 2) {
      tm0 = nanmax(nanmax(tm0, s[0][r]), s[1][r]);
      if (r + 1 < 16) tm1 = nanmax(nanmax(tm1, s[0][r + 1]), s[1][r + 1]);
    }
    tm = halves_max(nanmax(tm0, tm1));
    return (tm - nb) * inv_c2;
  };
  // The ragged last key tile, after scale_max: keys >= N get -inf and the maxima are taken
  // again over the remaining keys.
  auto ragged_fix = [&](int j, f32x16 (&s)[2], float nb, float& tm) {
    mask_ragged(j, s);
    float tm0 = nanmax(nanmax(s[0][0], s[1][0]), s[0][2]);
    float tm1 = nanmax(nanmax(s[0][1], s[1][1]), s[1][2]);
#pragma unroll
    for (int r = 3; r < 16; r += 2) {
      tm0 = nanmax(nanmax(tm0, s[0][r]), s[1][r]);
      if (r + 1 < 16) tm1 = nanmax(nanmax(tm1, s[0][r + 1]), s[1][r + 1]);
    }
    tm = halves_max(nanmax(tm0, tm1));
    return (tm - nb) * inv_c2;
  };
  // P as bf16 B operands (16-key step kc: registers 8(kc%2) .. +7 of t[kc/2]) and the row sum
  // over the same rounded weights (v_dot2 with ones, two partial sums).
  auto exp_pack = [&](const f32x16 (&t)[2], bf16x8 (&pb)[4]) {
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x2 pr = {__builtin_amdgcn_exp2f(t[kc >> 1][8 * (kc & 1) + 2 * e]),
                          __builtin_amdgcn_exp2f(t[kc >> 1][8 * (kc & 1) + 2 * e + 1])};
        const bf16x2 pk = __builtin_convertvector(pr, bf16x2);
        w[e] = __builtin_bit_cast(uint32_t, pk);
        if (e & 1) ps1 = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, ps1, false);
        else ps0 = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, ps0, false);
      }
      pb[kc] = __builtin_bit_cast(bf16x8, w);
    }
    return ps0 + ps1;
  };
  // Folds the scaled scores s of the tile just scored into the running maximum and, when some
  // row's maximum exceeds the exponent reference by more than 2^8 in exp2 units (or there is
  // no reference yet), moves the reference: exponentials then stay <= 256 and the common case
  // skips the accumulator rescale. `live` is false for the dummy tile after the last one.
  auto fold_max = [&](f32x16 (&s)[2], float nb, float tm, float mt, bool live) {
    if (!live) return;   // the dummy tile after the last one holds stale scores
    m_run = nanmax(m_run, mt);
    if (__ballot(m_ref == -INFINITY || tm > 8.f) != 0ull) {
      const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_ref - m_run) * c2);
      const float shift = -m_run * c2 - nb;
      m_ref = m_run;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] += shift;
    }
  };

  // One iteration: tile n (key tile j, scaled scores in tc, row maximum mt and the running
  // maximum before it mp) is finished, and tile n+1 (key tile j1, raw scores into tn) is
  // scored. j2 is the key tile at position n+2 (loaded here). kst: stage holding K(n+1);
  // kfree: stage to receive K(n+2); vst: stage holding V(n); vfree: stage to receive V(n+1).
  // QK-Skip vote for a tile against the running maximum of the tiles visited before it (mp):
  // the wave keeps the tile if any of its valid rows is not far enough below (a NaN margin
  // keeps); the workgroup's keep bits are OR-ed in LDS.
  auto vote = [&](int j, float mt, float mp) {
    const float diff = (mt - mp) * p.scale;
    const bool below = !row_valid || diff < p.log_eps;
    if (__ballot(!below) != 0ull) {
      if (lane == 0) atomicOr(&s_keep[j >> 5], 1u << (j & 31));
    }
  };
  // Without in-step skip nobody needs a tile's votes before the end, so each wave collects its
  // keep votes as bits of a scalar register indexed by list position, and stores the register
  // to LDS every 64 positions; the bits are combined into the keep bitset after the loop.
  uint64_t kmask = 0ull;
  auto vote_batched = [&](int n, float mt, float mp) {
    const float diff = (mt - mp) * p.scale;
    const bool below = !row_valid || diff < p.log_eps;
    if (__ballot(!below) != 0ull) kmask |= 1ull << (n & 63);
    if ((n & 63) == 63 || n == cnt - 1) {
      if (lane == 0) s_wkeep[wave][n >> 6] = kmask;
      kmask = 0ull;
    }
  };
  const bool row_exempt = i * BQ < p.dense_prefix;
  const int exempt_cols = (p.dense_prefix + BK - 1) / BK;

  // Vector slots per MFMA group. At D = 64 each MFMA carries about twice the softmax work of one
  // at D = 128 (8 vector instructions rather than 4); with four slots, phase B's scaling and
  // maxima trailed the last PV MFMA (measured +1.5% with eight).
  constexpr int VSLOT = D == 64 ? 8 : 4;
  auto phase_a_sched = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, RING, 0);    // K operand reads
    __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);       // VALU / transcendental
#pragma unroll
    for (int t = 0; t < D / 8; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (t + RING < D / 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, VSLOT, 0);
    }
  };
  // Early V reads (D = 128): V(n) is resident from the iteration's barrier on, so the first RING
  // V^T operand reads of phase B take the slots of the last QK MFMAs of phase A, which read no
  // K operand, and phase B starts with an MFMA instead of waiting for its reads (measured +0.6%
  // at D = 128, -1% at D = 64).
  auto phase_a_sched_v = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, RING, 0);    // K operand reads
    __builtin_amdgcn_sched_group_barrier(0x402, 6, 0);       // VALU / transcendental
#pragma unroll
    for (int t = 0; t < D / 8; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (t + RING < D / 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // K reads
      else __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                    // then V reads
      __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);
    }
  };
  auto phase_b_sched_v = [&]() {
#pragma unroll
    for (int t = 0; t < D / 8; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (t + RING < D / 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      if (t >= 1) __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);
    }
  };
  auto phase_b_sched = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * RING, 0);   // V operand reads
#pragma unroll
    for (int t = 0; t < D / 8; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (t + RING < D / 8) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      if (t >= 1) __builtin_amdgcn_sched_group_barrier(0x402, VSLOT, 0);
    }
  };

  auto iteration = [&](int n, int j, int j1, int j2, f32x16 (&tc)[2], f32x16 (&tn)[2],
                       float& mt, float& mp, const unsigned char* kst, unsigned char* kfree,
                       const unsigned char* vst, unsigned char* vfree) {
    // Tile n's vote needs only its row maximum and the running maximum before it. It is cast
    // here, ahead of the pipelined body, so that its branch (the store of the vote register
    // every 64 positions) does not split the body either.
    if constexpr (!INSTEP) vote_batched(n, mt, mp);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's loads have landed
    __syncthreads();                                      // everyone's; iteration n-1 is done
    if (n + 2 < cnt) issue_k(j2, kfree);
    if (n + 1 < cnt) issue_v(j1, vfree);
    const bool live = n + 1 < cnt;

    // With in-step skip, tile n's votes were cast when it was scored (previous iteration) and
    // the barrier above has closed them: a flagged tile gets no exponentials and no PV.
    bool skip = false;
    if constexpr (INSTEP) {
      const uint32_t kw = __builtin_amdgcn_readfirstlane(s_keep[j >> 5]);
      skip = !((kw >> (j & 31)) & 1u) && !row_exempt && j >= exempt_cols;
    }

    float nb, tm, mt1;
    if (!skip) {
      // phase A. After the last tile, K(n+1) is a stale stage: its scores are never used.
      bf16x8 pb[4];
      if constexpr (!INSTEP && D == 128) {
        qk_mfma(kst, tn);
        l_run += exp_pack(tc, pb);
        bf16x8 vr[RING];
#pragma unroll
        for (int t = 0; t < RING; ++t) vr[t] = vread(vst, t);
        phase_a_sched_v();
        // phase B
        nb = m_ref == -INFINITY ? 0.f : -m_ref * c2;   // exponent reference for tile n+1
        pv_mfma_pre(vst, pb, vr);
        mt1 = scale_max(tn, nb, tm);
        phase_b_sched_v();
      } else {
        qk_mfma(kst, tn);
        l_run += exp_pack(tc, pb);
        phase_a_sched();
        // In-step skip masks the ragged tile between the phases: it has more live registers,
        // and in the whole-body form below (tile n's exponentials kept in phase A) it spills.
        if constexpr (INSTEP) {
          if (live && (j1 + 1) * BK > N) mask_ragged(j1, tn);
        }
        // phase B
        nb = m_ref == -INFINITY ? 0.f : -m_ref * c2;   // exponent reference for tile n+1
        pv_mfma(vst, pb);
        mt1 = scale_max(tn, nb, tm);
        phase_b_sched();
      }
      // The ragged last key tile is fixed up after phase B rather than masked between the two
      // phases: a branch there would split the body into two basic blocks, and the compiler
      // would then move tile n's exponentials out of phase A. The empty asm keeps the maxima
      // computed in phase B.
      if constexpr (!INSTEP) {
        asm volatile("" : "+v"(mt1), "+v"(tm));
        if (live && (j1 + 1) * BK > N) mt1 = ragged_fix(j1, tn, nb, tm);
      }
    } else {
      qk_mfma(kst, tn);
      __builtin_amdgcn_sched_group_barrier(0x100, RING, 0);
#pragma unroll
      for (int t = 0; t < D / 8; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (t + RING < D / 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if (live && (j1 + 1) * BK > N) mask_ragged(j1, tn);
      nb = m_ref == -INFINITY ? 0.f : -m_ref * c2;
      mt1 = scale_max(tn, nb, tm);
    }
    mp = m_run;
    mt = mt1;
    if constexpr (INSTEP) {
      if (live) vote(j1, mt1, mp);
    }
    fold_max(tn, nb, tm, mt1, live);
  };

  // Prologue: load K(0), V(0), K(1); score tile 0.
  f32x16 ta[2], tb[2];
  float mt = -INFINITY, mp = -INFINITY;
  int j0 = cnt > 0 ? __builtin_amdgcn_readfirstlane(s_list[0]) : 0;
  int j1 = cnt > 1 ? __builtin_amdgcn_readfirstlane(s_list[1]) : 0;
  int j2 = cnt > 2 ? __builtin_amdgcn_readfirstlane(s_list[2]) : 0;
  if (cnt > 0) {
    issue_k(j0, s_k0);
    issue_v(j0, s_v0);
    if (cnt > 1) issue_k(j1, s_k1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    qk_mfma(s_k0, ta);
    if ((j0 + 1) * BK > N) mask_ragged(j0, ta);
    const float nb = 0.f;
    float tm;
    mt = scale_max(ta, nb, tm);
    mp = m_run;
    if constexpr (INSTEP) vote(j0, mt, mp);
    fold_max(ta, nb, tm, mt, true);
  }
  // Main loop, unrolled by two so that every stage is named statically. The list entries two
  // positions ahead are read early so that tile indices are in scalar registers.
  // List entries are read into vector registers one iteration before they are needed, so
  // that the LDS latency of the read is hidden (entries past cnt are read but never used).
  int jv3 = s_list[3];
  for (int n = 0; n < cnt; n += 2) {
    const int jv4 = s_list[n + 4];
    iteration(n, j0, j1, j2, ta, tb, mt, mp, s_k1, s_k0, s_v0, s_v1);
    const int j3 = __builtin_amdgcn_readfirstlane(jv3);
    if (n + 1 < cnt) {
      const int jv5 = s_list[n + 5];
      iteration(n + 1, j1, j2, j3, tb, ta, mt, mp, s_k0, s_k1, s_v1, s_v0);
      j0 = j2;
      j1 = j3;
      j2 = __builtin_amdgcn_readfirstlane(jv4);
      jv3 = jv5;
    }
  }
  // The next queue entry is taken as the tile loop ends: its latency overlaps the epilogue, and
  // the queue still hands each tile to the first workgroup that is nearly free.
  uint32_t next = 0u;
  if (s_next != nullptr && threadIdx.x == 0)
    next = __hip_atomic_fetch_add(&p.queue[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if constexpr (!INSTEP) {
    // a visited tile is kept when any wave voted keep at its list position
    for (int pos = tid; pos < cnt; pos += NT) {
      uint64_t any = 0ull;
#pragma unroll
      for (int w = 0; w < NW; ++w) any |= s_wkeep[w][pos >> 6];
      if ((any >> (pos & 63)) & 1ull) {
        const int jj = s_list[pos];
        atomicOr(&s_keep[jj >> 5], 1u << (jj & 31));
      }
    }
    __syncthreads();
  }

  // Epilogue: normalise and store this wave's rows.
  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_valid) {
    __bf16* orow = oh + (int64_t)qrow * sn;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[db][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * db + 8 * g + 4 * half) = w;
      }
  }

  bool clear = false;
  if (p.stats) {
    __shared__ float s_part[NW];
    __shared__ int s_clear;
    clear = refresh_decision<NW>(m_run, row_valid, min(BQ, N - i * BQ), p.scale,
                                 p.refresh_delta, p.stats + tile, s_part, &s_clear);
  }
  if (clear) clear_mask_row<NT>(mrow, p.W, p.Tk, s_old);
  else write_mask_row<NT>(mrow, p.W, p.Tk, s_old, s_keep, row_exempt, exempt_cols);
  if (s_next == nullptr) return 0u;
  if (threadIdx.x == 0) *s_next = next;
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*s_next);
#else
  return 0u;
#endif  // __HIP_DEVICE_COMPILE__
}

// The drivers are out-of-line functions rather than code in the kernel: there, the kernel's own
// argument loads stay in scalar registers across the tile, and inlined into the kernel the tile
// needed more scalar registers than there are (the spills undid its instruction schedule).

// One tile at position w_in (one workgroup per tile).
template <int D, int NW, bool INSTEP>
__device__ __attribute__((noinline)) void bf16_tile(uint64_t args, uint32_t w_in) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)args);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(args >> 32));
  ArgParams& p = *(ArgParams*)(((uint64_t)hi << 32) | lo);
  TileInputs<D> in;
  load_tile_inputs<D, NW>(p, __builtin_amdgcn_readfirstlane(w_in), in);
  bf16_tile_body<D, NW, INSTEP>(args, w_in, in, nullptr);
#endif
}

// Tiles from the queue until it runs out. The loop lives inside the out-of-line function, so the
// callee-saved registers are saved and restored once per workgroup rather than once per tile
// (which cost about 8 us per tile, 38% of the cost of a tile with one key tile to visit). The
// argument address passes through an empty asm at the top of every iteration, so that nothing
// loaded through it is held in registers from one tile to the next. Each tile takes the next
// queue entry while it runs (queue_position gives the order).
template <int D, int NW, bool INSTEP>
__device__ __attribute__((noinline)) void bf16_tiles(uint64_t args) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ uint32_t s_next;
  uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)args);
  uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(args >> 32));
  {
    ArgParams& p = *(ArgParams*)(((uint64_t)hi << 32) | lo);
    if (threadIdx.x == 0)
      s_next = __hip_atomic_fetch_add(&p.queue[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
  }
  uint32_t w = __builtin_amdgcn_readfirstlane(s_next);
  for (;;) {
    asm volatile("" : "+s"(lo), "+s"(hi));
    ArgParams& p = *(ArgParams*)(((uint64_t)hi << 32) | lo);
    if (w >= (uint32_t)(p.B * p.H * p.Tq)) break;   // the same value in every thread
    const uint32_t pos = queue_position<NW>(p, w);
    TileInputs<D> in;
    load_tile_inputs<D, NW>(p, pos, in);
    w = bf16_tile_body<D, NW, INSTEP>(((uint64_t)hi << 32) | lo, pos, in, &s_next);
    __syncthreads();           // LDS and s_next are reused by the next tile
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// At D = 128 and tile_q 64 the tile runs one wave per SIMD at 256 VGPRs; inlined into the queue
// loop it lost its pinned MFMA/VALU interleave, so that configuration calls the one-tile driver
// once per tile, with no prefetch.
template <int D, int NW, bool INSTEP>
__device__ __attribute__((noinline)) void bf16_tiles_calls(uint64_t args) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ uint32_t s_next;
  for (;;) {
    uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)args);
    uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(args >> 32));
    asm volatile("" : "+s"(lo), "+s"(hi));
    ArgParams& p = *(ArgParams*)(((uint64_t)hi << 32) | lo);
    if (threadIdx.x == 0)
      s_next = __hip_atomic_fetch_add(&p.queue[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const uint32_t w = s_next;
    if (w >= (uint32_t)(p.B * p.H * p.Tq)) break;   // the same value in every thread
    bf16_tile<D, NW, INSTEP>(((uint64_t)hi << 32) | lo, queue_position<NW>(p, w));
    __syncthreads();           // LDS and s_next are reused by the next tile
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// bf16 attention step. Without a queue, workgroup b takes the tile at position b. With one, the
// grid is sized to the workgroups the device holds at once and each workgroup takes positions
// from the queue until none is left: a workgroup that finishes a short tile starts the next
// one at once. (With one workgroup per tile, the dispatcher deals the workgroups of an XCD to
// its shader engines in a fixed rotation, so when tile lengths differ, as they do once tiles
// are skipped, free slots wait for their turn.) The last workgroup to finish puts the queue
// back to zero for the next launch on its stream.
template <int D, int NW, bool INSTEP>
__global__ void __launch_bounds__(NW * 64, 2) lite_attn_fwd_bf16(FwdParams p) {
  const uint64_t args = (uint64_t)__builtin_amdgcn_kernarg_segment_ptr();
  if (p.queue == nullptr) {
    bf16_tile<D, NW, INSTEP>(args, blockIdx.x);
    return;
  }
  if constexpr (D == 128 && NW == 2) bf16_tiles_calls<D, NW, INSTEP>(args);
  else bf16_tiles<D, NW, INSTEP>(args);
  // Every workgroup has taken its last position before it counts itself finished, so the last
  // one to finish can reset the queue.
  if (threadIdx.x == 0) {
    const uint32_t done =
        __hip_atomic_fetch_add(&p.queue[1], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == gridDim.x - 1) {
      __hip_atomic_store(&p.queue[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&p.queue[1], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------------------
// fp32 kernel: MFMA 32x32x2 f32, single-buffered (the fp32 workload is small).
// ---------------------------------------------------------------------------------------
template <int D, int NW, bool INSTEP>
__global__ void __launch_bounds__(NW * 64) lite_attn_fwd_f32(FwdParams p) {
  constexpr int NT = NW * 64;
  constexpr int BQ = NW * 32;
  constexpr int KP = D + 1;          // padded K row (conflict-free column reads)
  constexpr int VP = D + 4;
  constexpr int CH = D / 4;          // 16-byte chunks per row

  __shared__ float s_k[BK * KP];
  __shared__ float s_v[BK * VP];
  __shared__ uint16_t s_list[kMaxTilesK];
  __shared__ uint32_t s_keep[kMaxWords];
  __shared__ int s_count;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const uint32_t tile = p.perm ? p.perm[blockIdx.x] : blockIdx.x;   // (b * H + h) * Tq + i
  const int i = (int)(tile % (uint32_t)p.Tq);
  const int bh = (int)(tile / (uint32_t)p.Tq);
  const int b = bh / p.H, h = bh % p.H;
  const int64_t head_off = (int64_t)b * p.sb + (int64_t)h * p.sh;
  const float* __restrict__ qh = static_cast<const float*>(p.q) + head_off;
  const float* __restrict__ kh = static_cast<const float*>(p.k) + head_off;
  const float* __restrict__ vh = static_cast<const float*>(p.v) + head_off;
  float* __restrict__ oh = static_cast<float*>(p.out) + head_off;
  uint32_t* mrow = p.mask + (size_t)tile * p.W;
  const int N = p.N;
  const int64_t sn = p.sn;

  __shared__ uint32_t s_old[kMaxWords];
  uint32_t r0 = 0u, r1 = 0u;
  load_mask_words(mrow, p.W, r0, r1);
  const int cnt = build_visit_list<NT>(r0, r1, p.W, p.Tk, p.descending != 0, s_list, s_keep,
                                       s_old, &s_count);

  const int qrow = i * BQ + wave * 32 + l32;
  const bool row_valid = qrow < N;
  float qf[D / 2];  // lane holds features 2c + half of query row l32
#pragma unroll
  for (int c = 0; c < D / 2; ++c) qf[c] = row_valid ? qh[(int64_t)qrow * sn + 2 * c + half] : 0.f;

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  const float c2 = p.scale_log2;

  for (int n = 0; n < cnt; ++n) {
    const int j = s_list[n];
    const int key0 = j * BK;
    __syncthreads();  // previous tile fully consumed
    for (int ch = tid; ch < BK * CH; ch += NT) {
      const int row = ch / CH, cc = ch % CH;
      const int key = key0 + row;
      f32x4 kx = f32x4{0.f, 0.f, 0.f, 0.f}, vx = f32x4{0.f, 0.f, 0.f, 0.f};
      if (key < N) {
        kx = *reinterpret_cast<const f32x4*>(kh + (int64_t)key * sn + 4 * cc);
        vx = *reinterpret_cast<const f32x4*>(vh + (int64_t)key * sn + 4 * cc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s_k[row * KP + 4 * cc + e] = kx[e];
        s_v[row * VP + 4 * cc + e] = vx[e];
      }
    }
    __syncthreads();

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const int row = 32 * kb + l32;
#pragma unroll
      for (int c = 0; c < D / 2; ++c)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(s_k[row * KP + 2 * c + half], qf[c], s[kb],
                                                     0, 0, 0);
    }
    if ((j + 1) * BK > N) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key >= N) s[kb][r] = -INFINITY;
        }
    }
    float mt = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = nanmax(mt, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = nanmax(mt, s[1][r]);
    mt = halves_max(mt);

    const float diff = (mt - m_run) * p.scale;
    const bool below = !row_valid || (diff < p.log_eps);
    if (__ballot(!below) != 0ull) {
      if (lane == 0) atomicOr(&s_keep[j >> 5], 1u << (j & 31));
    }
    if constexpr (INSTEP) {
      // the workgroup's votes on this tile are complete after the barrier; a flagged tile
      // (which lies below the running maximum, so m is unchanged) is left out of this output
      __syncthreads();
      const uint32_t kw = __builtin_amdgcn_readfirstlane(s_keep[j >> 5]);
      if (!((kw >> (j & 31)) & 1u) && !(i * BQ < p.dense_prefix) &&
          j >= (p.dense_prefix + BK - 1) / BK)
        continue;
    }

    const float m_new = nanmax(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
    const float nb = -m_new * c2;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c2, nb));
        s[kb][r] = e;
        psum += e;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= alpha;

    // O^T += V^T P^T, two keys per MFMA: lane half 0 contributes key 32kb+8(r/4)+(r%4),
    // half 1 the key 4 above it; each lane's P value for that key is its own register r.
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(s_v[key * VP + 32 * db + l32], s[kb][r],
                                                       o[db], 0, 0, 0);
        }
  }
  __syncthreads();

  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_valid) {
    float* orow = oh + (int64_t)qrow * sn;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = o[db][4 * g + e] * inv;
        *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * g + 4 * half) = w;
      }
  }
  const int exempt_cols = (p.dense_prefix + BK - 1) / BK;
  bool clear = false;
  if (p.stats) {
    __shared__ float s_part[NW];
    __shared__ int s_clear;
    clear = refresh_decision<NW>(m_run, row_valid, min(BQ, N - i * BQ), p.scale,
                                 p.refresh_delta, p.stats + tile, s_part, &s_clear);
  }
  if (clear) clear_mask_row<NT>(mrow, p.W, p.Tk, s_old);
  else write_mask_row<NT>(mrow, p.W, p.Tk, s_old, s_keep, i * BQ < p.dense_prefix, exempt_cols);
}

// hipLaunchKernel reports the status of this launch only (hipGetLastError would also return
// errors left behind by other HIP users in the process).
template <int D, int NW, bool INSTEP>
hipError_t launch_bf16(const FwdParams& p, hipStream_t stream, unsigned* grid_out) {
  const unsigned tiles = (unsigned)((int64_t)p.B * p.H * p.Tq);
  unsigned grid = tiles;
  if (p.queue != nullptr) {
    // workgroups per compute unit at this kernel's register and LDS use (two)
    static const int per_cu = [] {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
              &n, reinterpret_cast<const void*>(&lite_attn_fwd_bf16<D, NW, INSTEP>), NW * 64,
              0) != hipSuccess)
        n = 0;
      return n;
    }();
    const int64_t resident = (int64_t)(per_cu > 0 ? per_cu : 1) * (p.n_cu > 0 ? p.n_cu : 1);
    if (resident < (int64_t)grid) grid = (unsigned)resident;
  }
  *grid_out = grid;
  FwdParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&lite_attn_fwd_bf16<D, NW, INSTEP>),
                         dim3(grid), dim3(NW * 64), args, 0, stream);
}

template <int D, int NW, bool INSTEP>
hipError_t launch_f32(const FwdParams& p, hipStream_t stream, unsigned* grid_out) {
  const unsigned grid = (unsigned)((int64_t)p.B * p.H * p.Tq);
  *grid_out = grid;
  FwdParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&lite_attn_fwd_f32<D, NW, INSTEP>),
                         dim3(grid), dim3(NW * 64), args, 0, stream);
}

template <bool INSTEP>
FwdLauncher pick_launcher(int dtype, int head_dim, int tile_q) {
  if (dtype == 0) {
    if (head_dim == 128 && tile_q == 128) return &launch_bf16<128, 4, INSTEP>;
    if (head_dim == 128 && tile_q == 64) return &launch_bf16<128, 2, INSTEP>;
    if (head_dim == 64 && tile_q == 128) return &launch_bf16<64, 4, INSTEP>;
    if (head_dim == 64 && tile_q == 64) return &launch_bf16<64, 2, INSTEP>;
  } else if (dtype == 1) {
    if (head_dim == 128 && tile_q == 128) return &launch_f32<128, 4, INSTEP>;
    if (head_dim == 128 && tile_q == 64) return &launch_f32<128, 2, INSTEP>;
    if (head_dim == 64 && tile_q == 128) return &launch_f32<64, 4, INSTEP>;
    if (head_dim == 64 && tile_q == 64) return &launch_f32<64, 2, INSTEP>;
  }
  return nullptr;
}

}  // namespace

FwdLauncher get_fwd_launcher(int dtype, int head_dim, int tile_q, bool in_step_skip) {
  return in_step_skip ? pick_launcher<true>(dtype, head_dim, tile_q)
                      : pick_launcher<false>(dtype, head_dim, tile_q);
}

hipError_t tile_queue_address(int slot, uint32_t** out) {
  *out = nullptr;
  if (slot < 0 || slot >= kQueueSlots) return hipErrorInvalidValue;
  void* base = nullptr;
  const hipError_t e = hipGetSymbolAddress(&base, HIP_SYMBOL(g_tile_queues));
  if (e != hipSuccess) return e;
  *out = static_cast<uint32_t*>(base) + 2 * slot;
  return hipSuccess;
}

}  // namespace lite_attn
