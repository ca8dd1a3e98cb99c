// Internal definitions shared by the MoE HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// ------------------------------------------------------------------ bf16
// bfloat16 is carried as its 16 bit pattern (uint16_t).
__device__ __forceinline__ float bf2f(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// float -> bf16, round to nearest, ties to even: the hardware conversion
// (v_cvt_pk_bf16_f32), which gives the same bits as rounding the float's
// bit pattern (adding 0x7FFF plus the kept lsb, then shifting) for every
// input that is not a NaN, subnormals and infinities included.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// two floats -> packed bf16x2 (lo in bits 0..15)
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint16_t f2bf(float f) {
  return static_cast<uint16_t>(pack_bf2(f, 0.0f));
}

// ------------------------------------------------------------------ storage traits
// St<float> / St<uint16_t>: element type of the activation/weight storage.
template <typename T> struct St;
template <> struct St<float> {
  static constexpr int kVec = 4;  // elements per 16-byte vector
  __device__ static __forceinline__ float to_f(float v) { return v; }
  __device__ static __forceinline__ float from_f(float v) { return v; }
  // unpack one 16-byte vector into kVec floats
  __device__ static __forceinline__ void unpack(const u32x4& u, float* o) {
    o[0] = __uint_as_float(u.x); o[1] = __uint_as_float(u.y);
    o[2] = __uint_as_float(u.z); o[3] = __uint_as_float(u.w);
  }
  __device__ static __forceinline__ u32x4 pack(const float* o) {
    return u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]),
                 __float_as_uint(o[2]), __float_as_uint(o[3])};
  }
};
template <> struct St<uint16_t> {
  static constexpr int kVec = 8;
  __device__ static __forceinline__ float to_f(uint16_t v) { return bf2f(v); }
  __device__ static __forceinline__ uint16_t from_f(float v) { return f2bf(v); }
  __device__ static __forceinline__ void unpack(const u32x4& u, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(u[i] << 16);
      o[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  }
  __device__ static __forceinline__ u32x4 pack(const float* o) {
    return u32x4{pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]),
                 pack_bf2(o[4], o[5]), pack_bf2(o[6], o[7])};
  }
};

// ------------------------------------------------------------------ GELU (tanh form)
// gelu(a) = 0.5 a (1 + tanh u), u = sqrt(2/pi) (a + 0.044715 a^3).  Since
// 0.5 (1 + tanh u) = s = 1 / (1 + e^{-2u}), gelu(a) = a s with
// e^{-2u} = 2^t, t = a (K1 + K2 a^2): a hardware exp2 and reciprocal and
// five other operations per element (about half the work of evaluating tanh
// as 1 - 2 / (e^{2u} + 1)).  s saturates to 0 and 1 (2^t overflowing to inf
// gives 0).
constexpr float kGeluK1 = -2.302208198144325f;   // -2 sqrt(2/pi) / ln 2
constexpr float kGeluK2 = -0.1029432395800235f;  // kGeluK1 * 0.044715
__device__ __forceinline__ float gelu_sig(float a) {
  const float t = a * fmaf(kGeluK2, a * a, kGeluK1);
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
}
__device__ __forceinline__ float gelu_tanh(float a) { return a * gelu_sig(a); }
// d gelu / da = 0.5 (1 + tanh u) + 0.5 a (1 - tanh^2 u) sqrt(2/pi) (1 + 3*0.044715 a^2)
//             = s + a s (1 - s) 2 sqrt(2/pi) (1 + 0.134145 a^2)
__device__ __forceinline__ float gelu_tanh_grad(float a) {
  const float s = gelu_sig(a);
  const float p = a * fmaf(0.21406444881780076f, a * a, 1.5957691216057308f);
  return fmaf(p, fmaf(-s, s, s), s);
}

// ------------------------------------------------------------------ wave helpers
// Wave reductions: lanes exchanged within each row of 16 by DPP (quad
// swaps at distance 1 and 2, then the half-row and row mirrors), which
// leaves every lane of a row holding the row's result, then the four rows'
// results read out with readlane and combined in row order.  Every lane
// returns the same value.  (A shuffle would go through the LDS crossbar:
// six dependent round trips per reduction.)
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(x)));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i of 8 <-> 7 - i
constexpr int kDppMirror = 0x140;      // lane i of 16 <-> 15 - i
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  v += dpp_f<kDppMirror>(v);
  return ((readlane_f(v, 0) + readlane_f(v, 16)) + readlane_f(v, 32)) + readlane_f(v, 48);
}
// The same sum by an xor butterfly of shuffles (every lane gets the sum).
// In the memory-bound gathers the shuffles' latency hides behind the row
// loads, and this form measured faster there than the DPP one above
// (c4_large combine backward 477 vs 469 us per launch).
__device__ __forceinline__ float wave_sum_xor(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)),
               fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
  const uint64_t u = __double_as_longlong(x);
  const uint32_t lo = (uint32_t)dpp_i<CTRL>((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)dpp_i<CTRL>((int)(uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double readlane_d(double v, int l) {
  const uint64_t u = __double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}
__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_d<kDppXor1>(v);
  v += dpp_d<kDppXor2>(v);
  v += dpp_d<kDppHalfMirror>(v);
  v += dpp_d<kDppMirror>(v);
  return ((readlane_d(v, 0) + readlane_d(v, 16)) + readlane_d(v, 32)) + readlane_d(v, 48);
}

// Exclusive scan of v over a block of 256 threads (4 waves); *total gets
// the block's sum.  Every thread of the block must call it; s_wave is 4
// ints of shared memory.
__device__ __forceinline__ int block_exclusive_scan_256(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  __syncthreads();  // s_wave may still be read by an earlier call
  if (lane == 63) s_wave[w] = incl;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (i < w) base += s_wave[i];
  *total = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
  return base + incl - v;
}

// The M-tile prefix of the grouped row GEMMs: tiles[e] = sum over e' < e of
// ceil(m_e' / BM), tiles[E] = the total, with thread e of a 256-thread block
// holding m = m_e (0 for e >= E; E <= 256).  Every thread of the block calls
// it (it synchronises).
__device__ __forceinline__ void block_tile_prefix(int m, int E, int BM, int32_t* tiles,
                                                  int* s_wave) {
  const int e = threadIdx.x;
  int tot;
  const int ex = block_exclusive_scan_256((m + BM - 1) / BM, s_wave, &tot);
  if (e < E) tiles[e] = ex;
  if (e == 0) tiles[E] = tot;
}

// The split plan of the expert weight-gradient GEMMs (dW1, dW2: a
// reduction over each expert's m_e rows, te output tiles per expert).
// Thread e of a 256-thread block holds m = m_e (0 for e >= E; E <= 256);
// every thread calls it (it synchronises).  With R = sum m_e and
// Kc = max(256, ceil(R te / 512)) rounded up to 32, an expert with more than
// 2 Kc rows is split into ceil(m_e / Kc) parts of about equal rows, so that
// no single tile's reduction is long against the chip's share of the work
// (about 512 part-tiles of Kc rows or more in all).  The work units
// (parts x tiles, expert-major) are then cut into 8 contiguous ranges of
// about equal work, one per XCD, a unit weighing its rows plus kKragUnitRows
// for its prologue and epilogue; with few units per XCD a cut close to an
// expert boundary moves onto it.  Written:
//   plan[e]          first work unit of expert e (units = parts x te)
//   plan[E]          number of units
//   plan[E+1+e]      first fp32 partial slab of expert e (split experts only)
//   plan[2E+1]       number of slabs
//   plan[2E+2]       Kc
//   plan[2E+3+x]     first unit of XCD x (x = 0..8; plan[2E+11] = units)
constexpr int kKragUnitRows = 128;
inline int krag_plan_ints(int E) { return 3 * E + 12; }
__device__ __forceinline__ void block_krag_plan(int m, int E, int te, int32_t* plan,
                                                int* s_wave) {
  __shared__ double s_wsum[4];
  const int e = threadIdx.x;
  int R;
  (void)block_exclusive_scan_256(m, s_wave, &R);
  // integer quantities below 2^53 are exact in double, whose division is
  // cheaper here than a 64-bit integer one
  int kc = (int)ceil((double)R * te / 512.0);
  kc = (kc + 31) / 32 * 32;
  if (kc < 256) kc = 256;
  const int parts = (e < E && m > 2 * kc) ? (int)ceil((double)m / kc) : 1;
  int tot_u, tot_s;
  const int ex_u = block_exclusive_scan_256(e < E ? parts * te : 0, s_wave, &tot_u);
  const int ex_s = block_exclusive_scan_256(e < E && parts > 1 ? parts : 0, s_wave, &tot_s);
  if (e < E) {
    plan[e] = ex_u;
    plan[E + 1 + e] = ex_s;
  }
  if (e == 0) {
    plan[E] = tot_u;
    plan[2 * E + 1] = tot_s;
    plan[2 * E + 2] = kc;
  }
  // work of one of this expert's units (its parts have equal rows but the
  // last), and of all its units; their exclusive scan
  const int rows = parts > 1 ? ((m + parts - 1) / parts + 31) / 32 * 32 : m;
  const double wu = (double)(rows + kKragUnitRows);
  const double we = e < E ? wu * parts * te : 0.0;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double incl = we;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  __syncthreads();
  if (lane == 63) s_wsum[w] = incl;
  __syncthreads();
  double base = 0.0;
  for (int i = 0; i < w; ++i) base += s_wsum[i];
  const double W = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
  const double pre = base + incl - we;
  // XCD x starts at the unit holding work x W / 8: the expert whose work
  // interval holds that point writes it.  With few units per XCD (under 256
  // on average, a handful of rounds of tiles) the cut moves to the nearer
  // end of that expert when this shifts it by at most W / 32 (a quarter of
  // an XCD's share): an XCD then serves whole experts from its L2, and a
  // layer of near-equal experts keeps the same number of tiles on every XCD
  // (a cut inside an expert there adds a round of tiles to one XCD).
  if (e < E) {
    const bool snap = tot_u < 8 * 256;
    for (int x = 1; x < 8; ++x) {
      const double target = floor(W * x / 8.0);
      if (target >= pre && target < pre + we) {
        int cut = ex_u + (int)floor((target - pre) / wu);
        const double slack = W / 32.0;
        if (snap && target - pre <= slack && target - pre <= pre + we - target) cut = ex_u;
        else if (snap && pre + we - target <= slack) cut = ex_u + parts * te;
        plan[2 * E + 3 + x] = cut;
      }
    }
  }
  if (e == 0) {
    plan[2 * E + 3] = 0;
    plan[2 * E + 11] = tot_u;
  }
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ------------------------------------------------------------------ workspace
// One workspace buffer serves every entry point; each region is 256-byte
// aligned.  Regions:
//   wrT      [Epad, d] s        router weights transposed, zero rows >= E
//   zf       [T, Epad] f32      fast router logits x Wr (no bias); then the
//                               canonical logits of the rescoring worklist
//   wl_*                        router rescoring worklist: count, tokens [T],
//                               candidate counts [T], candidates [T, Epad]
//   gpart                       fp32 partial tiles of the grouped GEMMs'
//                               split-K tail (bf16 storage)
//   perm_blk [nblk_perm, E] i32 per-block expert histograms / bases
//   tiles    [E+1] i32          grouped-GEMM M-tile prefix per expert
//   dz       [T, E] f32         router logit gradient (float storage)
//   dzb      [T, 2*Ep] bf16     dz split into bf16 high and low parts
//   wrp      [d, 2*Ep] bf16     Wr twice side by side, zero padded (bf16)
//   dwr_part [nchunk, d, Nw] f32 per-token-chunk partial sums of x^T dz
//   db_part  [E, nblk_dz] f32   per-block partial sums of dz
//   dgate    [T, k] f32         combine-backward gate gradient
//   dYp, dA, dXp                backward row gradients (Rmax rows, s)
//   dxe      [T, d] f32         unpermute-sum of dXp (router backward)
//   rA, rH   [Rmax, f] s        A and H of the recomputation mode
//   kplan    [3E+12] i32        split plan of the weight-gradient GEMMs
//   kslab    [slabs, d, f] f32  their fp32 partial sums (split experts)
struct WsLayout {
  size_t wrT, zf, wl_count, wl_tok, wl_n, wl_e, gpart, perm_blk, tiles, aux_part, dz, dzb, wrp,
      dwr_part, db_part, dgate, dYp, dA, dXp, dxe, rA, rH, kplan, kslab, total;
  int nblk_perm;
  int nblk_aux;
  int nblk_dz;
  int dwr_chunks, dwr_chunk, dwr_n;
};

constexpr int kPermTokens = 256;  // tokens per permute block
// fp32 partial tiles of the grouped GEMM's split-K tail: at most one tile
// per CU (256) of up to 256 x 256
constexpr size_t kGemmPartFloats = (size_t)256 * 256 * 256;
constexpr int kDzTokens = 16;     // tokens per router-backward dz block
constexpr int kAuxTokens = 32;    // tokens per block of the balancing-loss column sums

inline int64_t rows_max(const moe_cfg& c) {
  const int64_t tk = c.T * c.k;
  // no limit, or one that keeps every assignment (this test first also
  // keeps C * E below 2^44, so the product cannot overflow)
  if (c.capacity < 0 || c.capacity >= tk) return tk;
  const int64_t ec = c.capacity * (int64_t)c.E;
  return tk < ec ? tk : ec;
}

// Block tile of the expert weight-gradient GEMMs (bf16): 256 x 256 when
// the experts are not small (at least 512 rows each on average) and the
// problem has a full round of such tiles for the chip, else 128 x 128
inline int krag_tile(const moe_cfg& c) {
  const bool small = rows_max(c) < 512 * (int64_t)c.E;
  const int64_t big = (int64_t)c.E * ceil_div(c.d, 256) * ceil_div(c.f, 256);
  return (!small && big >= 256) ? 256 : 128;
}
// output tiles per expert of the weight-gradient GEMMs
inline int64_t krag_te(const moe_cfg& c) {
  const int b = krag_tile(c);
  return ceil_div(c.d, b) * ceil_div(c.f, b);
}
// fp32 partial slabs (d x f floats each) the split plan can need: split
// experts hold at most 1.5 R / Kc <= 768 / te slabs (Kc >= R te / 512)
inline int64_t krag_slabs_max(const moe_cfg& c) {
  if (c.dtype != MOE_BF16) return 0;
  return ceil_div(768, krag_te(c)) + 2;
}

// experts padded to 32, 64, 128 or 256 (whole 32-wide MFMA tiles) in the router
inline int route_epad(int E) {
  const int nt = (E + 31) / 32;
  return 32 * (nt <= 1 ? 1 : nt <= 2 ? 2 : nt <= 4 ? 4 : 8);
}
// Block tile of the router's fast-logit GEMM (bf16): the experts in one or
// two N tiles, 128-row M tiles when that gives a full round for the chip
inline void route_tile(const moe_cfg& c, int& bm, int& bn) {
  const int Epad = route_epad(c.E);
  bn = Epad <= 64 ? 64 : 128;
  bm = ceil_div(c.T, 128) * ceil_div(Epad, bn) >= 256 ? 128 : 64;
}
// K parts of that GEMM (1, 2 or 4): each writes its own fp32 partial
// logits, summed in part order by the select kernel.  Parts are added while
// the launch stays within two blocks per CU and each part keeps at least
// four whole K tiles of 32.
inline int route_ksplit(const moe_cfg& c) {
  if (c.dtype != MOE_BF16 || c.T <= 0) return 1;
  int bm, bn;
  route_tile(c, bm, bn);
  const int64_t tiles = ceil_div(c.T, bm) * ceil_div(route_epad(c.E), bn);
  int ks = 1;
  while (ks < 4 && tiles * ks * 2 <= 512 && c.d % (32 * ks * 2) == 0 && c.d / (ks * 2) >= 4 * 32)
    ks *= 2;
  return ks;
}
// experts padded to a multiple of 8 (16-byte bf16 rows) in the router backward
inline int bwd_ep(int E) { return (E + 7) / 8 * 8; }

inline size_t elem_bytes(const moe_cfg& c) { return c.dtype == MOE_BF16 ? 2 : 4; }

inline WsLayout ws_layout(const moe_cfg& c) {
  WsLayout L{};
  const size_t s = elem_bytes(c);
  const int64_t Rmax = rows_max(c);
  const int64_t T1 = c.T > 0 ? c.T : 1;
  // permute blocks: over T tokens, or k T virtual tokens for slot priority
  L.nblk_perm = (int)ceil_div((c.flags & MOE_FLAG_SLOT_PRIORITY) ? T1 * c.k : T1, kPermTokens);
  L.nblk_dz = (int)ceil_div(T1, kDzTokens);
  L.nblk_aux = (int)ceil_div(T1, kAuxTokens);
  // dWr = x^T dz as a k-ragged GEMM over uniform token chunks: enough chunks
  // for ~1024 blocks of 128 x 128 output tiles, at least 256 tokens each
  const bool bf = c.dtype == MOE_BF16;
  L.dwr_n = bf ? 2 * bwd_ep(c.E) : c.E;
  const int64_t tiles = ceil_div(c.d, bf ? 128 : 64) * ceil_div(L.dwr_n, bf ? 128 : 64);
  int64_t nch = ceil_div(1024, tiles);
  const int64_t cap = ceil_div(T1, 256);
  if (nch > cap) nch = cap;
  if (nch < 1) nch = 1;
  L.dwr_chunk = (int)(ceil_div(ceil_div(T1, nch), 64) * 64);
  L.dwr_chunks = (int)ceil_div(T1, L.dwr_chunk);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes, 256);
    return o;
  };
  L.wrT = take((size_t)route_epad(c.E) * c.d * s);
  L.zf = take((size_t)route_ksplit(c) * c.T * route_epad(c.E) * 4);
  L.wl_count = take(4);
  L.wl_tok = take((size_t)c.T * 4);
  L.wl_n = take((size_t)c.T * 4);
  L.wl_e = take((size_t)c.T * route_epad(c.E) * 4);
  L.gpart = take(c.dtype == MOE_BF16 ? kGemmPartFloats * 4 : 0);
  L.perm_blk = take((size_t)L.nblk_perm * c.E * 4);
  L.tiles = take((size_t)(c.E + 1) * 4 * 4);
  L.aux_part = take((size_t)L.nblk_aux * c.E * 4);
  L.dz = take(bf ? 0 : (size_t)c.T * c.E * 4);
  L.dzb = take(bf ? (size_t)c.T * 2 * bwd_ep(c.E) * 2 : 0);
  L.wrp = take(bf ? (size_t)c.d * 2 * bwd_ep(c.E) * 2 : 0);
  L.dwr_part = take((size_t)L.dwr_chunks * c.d * L.dwr_n * 4);
  L.db_part = take((size_t)L.nblk_dz * c.E * 4);
  L.dgate = take((size_t)c.T * c.k * 4);
  L.dYp = take((size_t)Rmax * c.d * s);
  L.dA = take((size_t)Rmax * c.f * s);
  L.dXp = take((size_t)Rmax * c.d * s);
  L.dxe = take((size_t)c.T * c.d * 4);
  // A and H of the recomputation mode (kept in the workspace, not saved)
  const bool rec = (c.flags & MOE_FLAG_RECOMPUTE) != 0;
  L.rA = take(rec ? (size_t)Rmax * c.f * s : 0);
  L.rH = take(rec ? (size_t)Rmax * c.f * s : 0);
  // split plan and fp32 partial slabs of the weight-gradient GEMMs
  L.kplan = take((size_t)krag_plan_ints(c.E) * 4);
  L.kslab = take((size_t)krag_slabs_max(c) * c.d * c.f * 4);
  L.total = off;
  return L;
}

template <typename P>
inline P* ws_ptr(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

// ------------------------------------------------------------------ launch + timing
// The caller's kernel timing (moe_cfg.probe): event records around the
// launches of the probed kernel
inline void prof_begin(const moe_cfg& c, int kid, hipStream_t s) {
  moe_probe* p = c.probe;
  if (p && p->kernel_id == kid && p->count < p->capacity)
    (void)hipEventRecord(static_cast<hipEvent_t>(p->begin[p->count]), s);
}
inline void prof_end(const moe_cfg& c, int kid, hipStream_t s) {
  moe_probe* p = c.probe;
  if (p && p->kernel_id == kid && p->count < p->capacity) {
    (void)hipEventRecord(static_cast<hipEvent_t>(p->end[p->count]), s);
    p->count++;
  }
}
void note_launch_error(int kernel_id, hipError_t e);

// Launch, then check that launch (a failed event record of the probe shows
// up here too).  Entry points clear any error state left by earlier,
// unrelated HIP calls of the process before their first launch.  Both
// macros need the launch's moe_cfg in scope as `c`.
// A launch that the probe does not time.
#define MOE_LAUNCH_NP(kid, ...)                                       \
  do {                                                                \
    __VA_ARGS__;                                                      \
    hipError_t e_ = hipGetLastError();                                \
    if (e_ != hipSuccess) {                                           \
      ::moe::note_launch_error((kid), e_);                            \
      return MOE_ERR_LAUNCH;                                          \
    }                                                                 \
  } while (0)

#define MOE_LAUNCH(kid, stream, ...)                                  \
  do {                                                                \
    ::moe::prof_begin(c, (kid), (stream));                            \
    __VA_ARGS__;                                                      \
    ::moe::prof_end(c, (kid), (stream));                              \
    hipError_t e_ = hipGetLastError();                                \
    if (e_ != hipSuccess) {                                           \
      ::moe::note_launch_error((kid), e_);                            \
      return MOE_ERR_LAUNCH;                                          \
    }                                                                 \
  } while (0)

// ------------------------------------------------------------------ launchers
// (each validates nothing: the C-ABI layer in api.hip has done that)
int launch_route(const moe_cfg& c, const void* x, const void* Wr, const float* b,
                 float* probs, int32_t* idx, float* gate, void* ws, hipStream_t s);
int launch_route_aux(const moe_cfg& c, const float* probs, const int32_t* counts,
                     const int32_t* offsets, float* aux, void* ws, hipStream_t s);
// M tile of the grouped row GEMMs (their tile schedule is built for it)
int ffn_row_tile(const moe_cfg& c);
// tiles (nullable): also write the grouped GEMMs' M-tile prefix for the kept
// rows, so that the layer forward needs no schedule kernel
int launch_permute(const moe_cfg& c, const void* x, const int32_t* idx,
                   int32_t* counts, int32_t* offsets, int32_t* row_of,
                   int32_t* src_of, void* x_perm, void* ws, hipStream_t s,
                   int32_t* tiles = nullptr);
// the same with its scratch (per-block histograms) in a fixed device array
// of permute_noalloc_scratch_max() bytes; MOE_ERR_WORKSPACE when the cfg
// needs more
size_t permute_noalloc_scratch_bytes(const moe_cfg& c);
size_t permute_noalloc_scratch_max();
int launch_permute_noalloc(const moe_cfg& c, const void* x, const int32_t* idx,
                           int32_t* counts, int32_t* offsets, int32_t* row_of,
                           int32_t* src_of, void* x_perm, hipStream_t s);
// have_tiles: the workspace already holds the M-tile prefix for offsets
// (written by the permute or the combine backward), so no schedule kernel
int launch_ffn_fwd(const moe_cfg& c, const void* x_perm, const int32_t* offsets,
                   const void* W1, const void* W2, void* A, void* H, void* Y,
                   void* ws, hipStream_t s, bool have_tiles = false);
int launch_ffn_bwd(const moe_cfg& c, const void* x_perm, const int32_t* offsets,
                   const void* W1, const void* W2, const void* A, const void* H,
                   const void* dYp, void* dXp, void* dW1, void* dW2, void* ws,
                   hipStream_t s, bool have_tiles = false);
// x, gate and dOut feed the identity fallback of dropped assignments
// (MOE_FLAG_DROP_IDENTITY) and are unused otherwise.
int launch_combine(const moe_cfg& c, const void* Y, const int32_t* row_of,
                   const float* gate, const void* x, void* out, hipStream_t s);
// offsets and tiles (nullable): also write the grouped GEMMs' M-tile prefix
// (and, plan non-null, the weight-gradient split plan)
int launch_combine_bwd(const moe_cfg& c, const void* dOut, const void* Y,
                       const int32_t* row_of, const float* gate, const void* x, void* dYp,
                       float* dgate, hipStream_t s, const int32_t* offsets = nullptr,
                       int32_t* tiles = nullptr, int32_t* plan = nullptr);
int launch_unpermute_bwd(const moe_cfg& c, const void* dXp, const int32_t* row_of,
                         const float* gate, const void* dOut, float* dXe, hipStream_t s,
                         int kernel_id = MOE_KERNEL_UNPERMUTE_BWD);
// dX = dXe + dz Wr^T: dXe is the caller's fp32 unpermute-sum, or (dXe NULL)
// gathered from dXp, row_of and, under the identity fallback, gate and dOut
int launch_route_bwd(const moe_cfg& c, const void* x, const void* Wr,
                     const float* probs, const int32_t* idx, const int32_t* row_of,
                     const int32_t* counts, const float* gate, const void* dOut,
                     const float* dgate, const void* dXp, const float* dXe, void* dX,
                     void* dWr, float* db, void* ws, hipStream_t s);

}  // namespace moe
