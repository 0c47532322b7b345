// gfx950 (CDNA4) kernels of the LiteAttention step: tiled softmax attention with the QK-Skip
// test inside the online-softmax pipeline and a persistent per-(b, h, query tile, key tile)
// skip bitmask.
//
// Method: "LiteAttention: Temporal Sparse Attention for Diffusion Transformers", page 1
// "Core Concept" (QK-Skip: a tile whose local maximum score is far below the cumulative
// maximum is flagged, and the flag persists across denoising steps) and "Architecture
// Overview" (bitmask, skip logic inside the FlashAttention softmax pipeline).
//
// Work decomposition. One workgroup owns one query tile (b, h, i) and is the only reader and
// writer of that tile's mask row, so no global atomics are needed. Each 64-lane wave owns 32
// query rows. Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
// the accumulator then holds one query per lane (lane % 32) and 16 keys per register group,
// so the row maximum and row sum of the online softmax are in-lane reductions plus a single
// swap between the two half-waves (v_permlane32_swap). The PV product is likewise computed
// transposed, O^T += V^T P^T, which takes P straight from the score registers (converted to
// bf16) as the B operand; V is stored transposed in LDS so that the A operand is one 16-byte
// LDS read per lane. The key order inside a 16-key MFMA step is permuted identically on both
// operands, which leaves the contraction unchanged.
//
// The QK-Skip vote needs nothing beyond the online softmax: the tile's row maximum mt is
// already computed for the rescale, and the running maximum m is the softmax state. A wave
// votes "keep" when any of its valid rows has (mt - m) * scale >= log_eps (or NaN); the votes
// of the workgroup's waves are OR-ed into an LDS bitset, and the tile is flagged at the end
// when no wave voted keep.
//
// Skipped tiles cost nothing: the mask row is turned into a compact visiting list in LDS
// before any K/V load, and the K/V pipeline only ever fetches listed tiles.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "lite_attn_internal.h"

namespace lite_attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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

// Workgroups are dispatched to the 8 XCDs round-robin by block index. Remap so that each
// XCD receives a contiguous range of logical tiles: consecutive query tiles of one head then
// run on the same XCD and share its L2 for the K/V stream.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t n) {
  const uint32_t per = n / 8u, rem = n % 8u, xcd = bid % 8u, loc = bid / 8u;
  return xcd < rem ? xcd * (per + 1u) + loc : rem * (per + 1u) + (xcd - rem) * per + loc;
}

// Value of x in the other half-wave (lane ^ 32) combined with x by max / sum.
__device__ __forceinline__ float halves_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Turn mask row `mrow` (W words) into the list of key tiles to visit, in traversal order.
// Runs on wave 0 (each lane owns words 2*lane and 2*lane+1, W <= 128); also clears the keep
// bitset. Ends with a workgroup barrier; returns the list length.
template <int NT>
__device__ int build_visit_list(const uint32_t* mrow, int W, int Tk, bool descending,
                                uint16_t* list, uint32_t* keep, int* s_count) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int lane = tid;
    const int w0 = 2 * lane, w1 = 2 * lane + 1;
    uint32_t b0 = w0 < W ? (~mrow[w0] & valid_bits(w0, Tk)) : 0u;
    uint32_t b1 = w1 < W ? (~mrow[w1] & valid_bits(w1, Tk)) : 0u;
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

// Fold this step's flags into the mask row: flags = visited & ~keep & ~exempt.
template <int NT>
__device__ void write_mask_row(uint32_t* mrow, int W, int Tk, const uint32_t* keep,
                               bool row_exempt, int exempt_cols) {
  if (row_exempt) return;
  for (int w = threadIdx.x; w < W; w += NT) {
    const uint32_t old = mrow[w];
    const uint32_t visited = ~old & valid_bits(w, Tk);
    const uint32_t flags = visited & ~keep[w] & ~low_bits(w, exempt_cols);
    if (flags) mrow[w] = old | flags;
  }
}

// ---------------------------------------------------------------------------------------
// bf16 kernel: MFMA 32x32x16 bf16, K/V double-buffered in LDS, one barrier per tile.
// ---------------------------------------------------------------------------------------

// LDS layouts (bf16 elements):
//  K tile  [64 keys][D]: 16-byte chunk c of key row r is stored at chunk c ^ (r & 7), which
//          makes both the coalesced row-wise writes and the 32-rows-one-column operand reads
//          bank-conflict free.
//  V^T tile [D][64 keys]: row d holds the 64 keys of feature d. Within each 16-key group the
//          keys are stored in MFMA operand order (bits 2 and 3 of the key index swapped), so a
//          lane's 8 operand keys are one 16-byte chunk; chunk c of row d is stored at
//          c ^ ((d ^ (d >> 3)) & 7), which spreads both the transposing 8-byte writes and the
//          16-byte operand reads over all banks.
__device__ __forceinline__ int k_lds_off(int row, int chunk, int D) {
  return row * D + ((chunk ^ (row & 7)) << 3);
}
__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }

template <int D, int NW>
__global__ void __launch_bounds__(NW * 64, 2) lite_attn_fwd_bf16(FwdParams p) {
  constexpr int NT = NW * 64;
  constexpr int BQ = NW * 32;
  constexpr int KCH = D / 8;                          // 16-byte chunks per K row
  constexpr int KLD = (BK * KCH) / NT;                // K chunks per thread per tile
  constexpr int VUNITS = (BK / 4) * (D / 8);          // (4 keys x 8 features) units per tile
  constexpr int VLD = (VUNITS + NT - 1) / NT;         // units per thread per tile
  static_assert((BK * KCH) % NT == 0, "K tile must split evenly over the workgroup");

  __shared__ __attribute__((aligned(16))) __bf16 s_k[2][BK * D];
  __shared__ __attribute__((aligned(16))) __bf16 s_vt[2][D * BK];
  __shared__ uint16_t s_list[kMaxTilesK];
  __shared__ uint32_t s_keep[kMaxWords];
  __shared__ int s_count;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const uint32_t tile = xcd_remap(blockIdx.x, gridDim.x);  // = (b * H + h) * Tq + i
  const int i = (int)(tile % (uint32_t)p.Tq);
  const int bh = (int)(tile / (uint32_t)p.Tq);
  const int b = bh / p.H, h = bh % p.H;
  const int64_t head_off = (int64_t)b * p.sb + (int64_t)h * p.sh;
  const __bf16* __restrict__ qh = static_cast<const __bf16*>(p.q) + head_off;
  const __bf16* __restrict__ kh = static_cast<const __bf16*>(p.k) + head_off;
  const __bf16* __restrict__ vh = static_cast<const __bf16*>(p.v) + head_off;
  __bf16* __restrict__ oh = static_cast<__bf16*>(p.out) + head_off;
  uint32_t* mrow = p.mask + (size_t)tile * p.W;
  const int N = p.N;
  const int64_t sn = p.sn;

  const int cnt = build_visit_list<NT>(mrow, p.W, p.Tk, p.descending != 0, s_list, s_keep,
                                       &s_count);

  // Q rows of this wave as MFMA B operands: lane holds features 16c + 8*half .. +7 of query
  // row l32 for every 16-feature step c.
  const int qrow = i * BQ + wave * 32 + l32;
  const bool row_valid = qrow < N;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    if (row_valid) {
      qf[c] = *reinterpret_cast<const bf16x8*>(qh + (int64_t)qrow * sn + 16 * c + 8 * half);
    } else {
      qf[c] = bf16x8{};
    }
  }

  // ---- K/V pipeline: global -> registers (prefetch) -> LDS ----
  u32x4 kreg[KLD];
  u32x4 vreg[VLD][4];
  auto load_kv = [&](int j) {
    const int key0 = j * BK;
#pragma unroll
    for (int x = 0; x < KLD; ++x) {
      const int ch = tid + NT * x;
      const int row = ch / KCH, cc = ch % KCH;
      const int key = key0 + row;
      kreg[x] = key < N ? *reinterpret_cast<const u32x4*>(kh + (int64_t)key * sn + cc * 8)
                        : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int x = 0; x < VLD; ++x) {
      const int u = tid + NT * x;
      if (VUNITS % NT == 0 || u < VUNITS) {
        const int kg = u / (D / 8), dg = u % (D / 8);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int key = key0 + 4 * kg + kk;
          vreg[x][kk] = key < N ? *reinterpret_cast<const u32x4*>(vh + (int64_t)key * sn + dg * 8)
                                : u32x4{0u, 0u, 0u, 0u};
        }
      }
    }
  };
  auto store_kv = [&](int buf) {
#pragma unroll
    for (int x = 0; x < KLD; ++x) {
      const int ch = tid + NT * x;
      const int row = ch / KCH, cc = ch % KCH;
      *reinterpret_cast<u32x4*>(&s_k[buf][k_lds_off(row, cc, D)]) = kreg[x];
    }
#pragma unroll
    for (int x = 0; x < VLD; ++x) {
      const int u = tid + NT * x;
      if (VUNITS % NT == 0 || u < VUNITS) {
        const int kg = u / (D / 8), dg = u % (D / 8);
        const int g4 = kg & 3;                       // 4-key group inside a 16-key group
        const int pos = 16 * (kg >> 2) + 8 * (g4 & 1) + 4 * (g4 >> 1);  // operand order
        const int lc = pos >> 3, hf = (pos >> 2) & 1;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const int sh = 16 * (m & 1);
          const uint32_t e0 = (vreg[x][0][m >> 1] >> sh) & 0xffffu;
          const uint32_t e1 = (vreg[x][1][m >> 1] >> sh) & 0xffffu;
          const uint32_t e2 = (vreg[x][2][m >> 1] >> sh) & 0xffffu;
          const uint32_t e3 = (vreg[x][3][m >> 1] >> sh) & 0xffffu;
          const int d = 8 * dg + m;
          const int off = d * BK + ((lc ^ vt_swz(d)) << 3) + 4 * hf;
          *reinterpret_cast<u32x2*>(&s_vt[buf][off]) = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
        }
      }
    }
  };

  float m_run = -INFINITY;   // running row maximum (raw scores)
  float l_run = 0.f;         // this lane's partial row sum (its 32 keys of every tile)
  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};

  const float c2 = p.scale_log2;
  if (cnt > 0) {
    load_kv(s_list[0]);
    store_kv(0);
    if (cnt > 1) load_kv(s_list[1]);
    __syncthreads();
  }

  for (int n = 0; n < cnt; ++n) {
    const int j = s_list[n];
    const int buf = n & 1;
    if (n + 1 < cnt) store_kv(buf ^ 1);
    if (n + 2 < cnt) load_kv(s_list[n + 2]);

    // S^T = K Q^T for keys [32kb, 32kb+32) of the tile: lane holds query l32 and keys
    // 32kb + 8(r/4) + 4*half + (r%4) in register r.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const int row = 32 * kb + l32;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(&s_k[buf][k_lds_off(row, 2 * c + half, D)]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s[kb], 0, 0, 0);
      }
    }

    // Ragged last tile: keys >= N do not exist.
    if ((j + 1) * BK > N) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j * BK + 32 * kb + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key >= N) s[kb][r] = -INFINITY;
        }
    }

    // Row maximum of the tile.
    float mt = s[0][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[1][r]);
    mt = halves_max(mt);

    // QK-Skip vote: keep the tile if any valid row's local max is not far enough below the
    // running max (a NaN difference keeps it too).
    const float diff = (mt - m_run) * p.scale;
    const bool below = !row_valid || (diff < p.log_eps);
    if (__ballot(!below) != 0ull) {
      if (lane == 0) atomicOr(&s_keep[j >> 5], 1u << (j & 31));
    }

    // Online softmax update (base 2: exp(x*scale) = exp2(x*scale*log2 e)).
    const float m_new = fmaxf(m_run, mt);
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

    // P as bf16 B operands: 16-key step kc uses registers 8(kc%2) .. +7 of s[kc/2].
    bf16x8 pb[4];
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int m = 0; m < 8; ++m) pb[kc][m] = (__bf16)s[kc >> 1][8 * (kc & 1) + m];

    // O^T += V^T P^T: lane holds query l32 and features 32db + 8(r/4) + 4*half + (r%4).
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int d = 32 * db + l32;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(
            &s_vt[buf][d * BK + (((2 * kc + half) ^ vt_swz(d)) << 3)]);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kc], o[db], 0, 0, 0);
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

  const int exempt_cols = (p.dense_prefix + BK - 1) / BK;
  write_mask_row<NT>(mrow, p.W, p.Tk, s_keep, i * BQ < p.dense_prefix, exempt_cols);
}

// ---------------------------------------------------------------------------------------
// fp32 kernel: MFMA 32x32x2 f32, single-buffered (the fp32 workload is small).
// ---------------------------------------------------------------------------------------
template <int D, int NW>
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

  const uint32_t tile = xcd_remap(blockIdx.x, gridDim.x);
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

  const int cnt = build_visit_list<NT>(mrow, p.W, p.Tk, p.descending != 0, s_list, s_keep,
                                       &s_count);

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
    for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[0][r]);
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[1][r]);
    mt = halves_max(mt);

    const float diff = (mt - m_run) * p.scale;
    const bool below = !row_valid || (diff < p.log_eps);
    if (__ballot(!below) != 0ull) {
      if (lane == 0) atomicOr(&s_keep[j >> 5], 1u << (j & 31));
    }

    const float m_new = fmaxf(m_run, mt);
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
  write_mask_row<NT>(mrow, p.W, p.Tk, s_keep, i * BQ < p.dense_prefix, exempt_cols);
}

// ---------------------------------------------------------------------------------------
// mask bookkeeping kernels
// ---------------------------------------------------------------------------------------
__global__ void __launch_bounds__(256) mask_fill_zero(uint32_t* mask, size_t words) {
  for (size_t w = (size_t)blockIdx.x * blockDim.x + threadIdx.x; w < words;
       w += (size_t)gridDim.x * blockDim.x)
    mask[w] = 0u;
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

// hipLaunchKernel reports the status of this launch only (hipGetLastError would also return
// errors left behind by other HIP users in the process).
template <int D, int NW>
hipError_t launch_bf16(const FwdParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)p.B * p.H * p.Tq);
  FwdParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&lite_attn_fwd_bf16<D, NW>), dim3(grid),
                         dim3(NW * 64), args, 0, stream);
}

template <int D, int NW>
hipError_t launch_f32(const FwdParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)((int64_t)p.B * p.H * p.Tq);
  FwdParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&lite_attn_fwd_f32<D, NW>), dim3(grid),
                         dim3(NW * 64), args, 0, stream);
}

}  // namespace

FwdLauncher get_fwd_launcher(int dtype, int head_dim, int tile_q) {
  if (dtype == 0) {
    if (head_dim == 128 && tile_q == 128) return &launch_bf16<128, 4>;
    if (head_dim == 128 && tile_q == 64) return &launch_bf16<128, 2>;
    if (head_dim == 64 && tile_q == 128) return &launch_bf16<64, 4>;
    if (head_dim == 64 && tile_q == 64) return &launch_bf16<64, 2>;
  } else if (dtype == 1) {
    if (head_dim == 128 && tile_q == 128) return &launch_f32<128, 4>;
    if (head_dim == 128 && tile_q == 64) return &launch_f32<128, 2>;
    if (head_dim == 64 && tile_q == 128) return &launch_f32<64, 4>;
    if (head_dim == 64 && tile_q == 64) return &launch_f32<64, 2>;
  }
  return nullptr;
}

hipError_t launch_mask_fill_zero(uint32_t* mask, size_t words, hipStream_t stream) {
  if (words == 0) return hipSuccess;
  size_t blocks = (words + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  void* args[] = {&mask, &words};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mask_fill_zero), dim3((unsigned)blocks),
                         dim3(256), args, 0, stream);
}

hipError_t launch_mask_popcount(const uint32_t* mask, uint32_t* counts, int heads_total, int Tq,
                                int Tk, int W, hipStream_t stream) {
  if (heads_total == 0) return hipSuccess;
  void* args[] = {&mask, &counts, &Tq, &Tk, &W};
  return hipLaunchKernel(reinterpret_cast<const void*>(&mask_popcount), dim3((unsigned)heads_total),
                         dim3(256), args, 0, stream);
}

}  // namespace lite_attn
