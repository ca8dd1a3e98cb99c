// Grouped expert GEMMs over ragged per-expert segments (F3, F4, B4, B3).
// Every local expert runs on the rows routed to it as one grouped GEMM
// rather than one small GEMM per expert ("GPU expert parallel", section
// "The step timeline").  The per-expert segments are [offsets[e],
// offsets[e+1]) and live on the device only; tile lists are derived on the
// device.
//
// Two problem shapes:
//   ROW  (forward and input-gradient GEMMs): C_e[m_e, N] = A_e[m_e, K] B_e
//        with A_e the expert's rows (K contiguous) and B_e the expert's
//        weight, stored either [K][N] (N contiguous: x W1, H W2) or [N][K]
//        (K contiguous: dYp W2^T, dA W1^T).
//   KRAG (weight gradients): C_e[M, N] = A_e^T B_e over the expert's m_e
//        rows, A_e [m_e][M] and B_e [m_e][N] both row-major, i.e. the
//        reduction runs over a ragged K = m_e (H^T dYp, x_perm^T dA).
//        Experts with m_e = 0 get a zero matrix.
//
// bf16 kernels (gfx950), fp32 accumulation, K tiles of 32 held in a ring of
// LDS stages filled straight from HBM by global_load_lds_dwordx4:
//   gemm_pp_kernel: row GEMMs on 256 x 256 tiles, eight waves in two groups
//     that alternate between reading a K tile's fragments and issuing its
//     v_mfma_f32_16x16x32_bf16 (four stages);
//   gemm_bf16_kernel: four waves in 2 x 2 with v_mfma_f32_32x32x16_bf16 on
//     128 x 128, 128 x 256 (wide expert row GEMMs) or 256 x 256 tiles (the
//     weight gradients, the router's GEMMs, row GEMMs not on 256-row
//     tiles); four stages for 256 x 256, else three.  Operands keep their HBM orientation in LDS:
// K-contiguous tiles with an XOR swizzle, read as 16-byte fragments;
// M/N-contiguous tiles read with the transposing ds_read_b64_tr_b16.  Tiles
// are ordered so that the blocks resident on one XCD (block id mod 8) work
// on a compact group of output tiles, which keeps their operand panels in
// that XCD's L2; the last, partial round of row-GEMM tiles is split along K
// and summed by a fixup kernel in part order.  The epilogue is staged
// through LDS for 16-byte row stores.
#include "gemm.h"

namespace moe {

// M tiles per traversal group: 4 for 128 x 128 tiles, 2 for 256 x 256
// (the 32 tiles resident on one XCD then span fewer distinct operand panels)
template <int BM>
constexpr int group_m() { return BM >= 256 ? 2 : 4; }
constexpr int BK_ALL = 32;  // K tile of the bf16 kernels

namespace {

// Block -> output tile.  Block ids are dealt round-robin to the 8 XCDs;
// give each XCD a contiguous range of logical tiles, then walk that range
// in groups of group_m M-tiles with M fastest (compact 2-D groups).
__device__ __forceinline__ bool xcd_logical(int ntotal, int& lid) {
  const int per = (ntotal + 7) >> 3;
  const int bid = blockIdx.x;
  const int local = bid >> 3, xcd = bid & 7;
  if (local >= per) return false;
  lid = xcd * per + local;
  return lid < ntotal;
}
template <int kGroupM>
__device__ __forceinline__ void group_mn(int lid, int num_m, int ntn, int& mt, int& nt) {
  const int per_group = kGroupM * ntn;
  const int g = lid / per_group;
  const int first = g * kGroupM;
  const int gsz = min(num_m - first, kGroupM);
  const int in = lid - g * per_group;
  mt = first + in % gsz;
  nt = in / gsz;
}

struct Tile {
  int e, m0, n0, M, K;
  int64_t row0;  // ROW: first row of the expert; KRAG: first K row
  int kofs;      // split-K part: first K element of the part (0 otherwise)
  int slab;      // KRAG split part: its fp32 partial slab (-1 otherwise)
  int64_t coff;  // ROW K part of a ksplit problem: offset of its output (0 otherwise)
};

// Number of output tiles (and of M tiles for ROW).  ROW problems with a
// schedule load it into s_tiles (block-wide, synchronising).
template <int MODE, int BM>
__device__ __forceinline__ int tile_count(const GemmArgs& g, int* s_tiles, int& num_m) {
  if constexpr (MODE == MODE_ROW) {
    if (!g.offsets) {
      num_m = (g.M + BM - 1) / BM;
    } else {
      for (int i = threadIdx.x; i <= g.E; i += blockDim.x) s_tiles[i] = g.tiles[i];
      __syncthreads();
      num_m = s_tiles[g.E];
    }
    return num_m * g.ntn;
  } else {
    num_m = g.ntm;
    if (g.kplan != nullptr) {  // the split plan's work units
      for (int i = threadIdx.x; i <= g.E; i += blockDim.x) s_tiles[i] = g.kplan[i];
      __syncthreads();
      return s_tiles[g.E];
    }
    return g.E * g.ntm * g.ntn;
  }
}

// Logical tile lid -> tile.
template <int MODE, int BM, int BN>
__device__ __forceinline__ void tile_of(const GemmArgs& g, const int* s_tiles, int num_m, int lid,
                                        Tile& t) {
  t.kofs = 0;
  t.slab = -1;
  t.coff = 0;
  if constexpr (MODE == MODE_ROW) {
    int mt, nt;
    group_mn<group_m<BM>()>(lid, num_m, g.ntn, mt, nt);
    if (!g.offsets) {  // one group of g.M rows
      t.e = 0;
      t.row0 = 0;
      t.M = g.M;
      t.m0 = mt * BM;
    } else {
      int lo = 0, hi = g.E - 1;  // last e with s_tiles[e] <= mt
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_tiles[mid] <= mt) lo = mid; else hi = mid - 1;
      }
      t.e = lo;
      t.row0 = g.offsets[lo];
      t.M = g.offsets[lo + 1] - (int)t.row0;
      t.m0 = (mt - s_tiles[lo]) * BM;
    }
    t.n0 = nt * BN;
    t.K = g.K;
  } else if (g.kplan != nullptr) {
    // unit lid of the split plan: expert, part, then the part's tile
    const int te = g.ntm * g.ntn;
    int lo = 0, hi = g.E - 1;  // last e with s_tiles[e] <= lid
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_tiles[mid] <= lid) lo = mid; else hi = mid - 1;
    }
    t.e = lo;
    const int u = lid - s_tiles[lo];
    const int parts = (s_tiles[lo + 1] - s_tiles[lo]) / te;
    const int part = u / te;
    int mt, nt;
    group_mn<group_m<BM>()>(u - part * te, g.ntm, g.ntn, mt, nt);
    const int64_t r0 = g.offsets[t.e];
    const int m = g.offsets[t.e + 1] - (int)r0;
    t.row0 = r0;
    t.K = m;
    if (parts > 1) {
      // parts of equal rows, rounded up to whole K tiles
      const int chunk = ((m + parts - 1) / parts + BK_ALL - 1) / BK_ALL * BK_ALL;
      const int k0 = min(part * chunk, m);
      t.row0 = r0 + k0;
      t.K = min(chunk, m - k0);
      t.slab = g.kplan[g.E + 1 + t.e] + part;
    }
    t.M = g.M;
    t.m0 = mt * BM;
    t.n0 = nt * BN;
  } else {
    const int per_e = g.ntm * g.ntn;
    t.e = lid / per_e;
    int mt, nt;
    group_mn<group_m<BM>()>(lid - t.e * per_e, g.ntm, g.ntn, mt, nt);
    if (g.offsets) {
      t.row0 = g.offsets[t.e];
      t.K = g.offsets[t.e + 1] - (int)t.row0;
    } else {  // uniform groups of g.chunk rows out of g.K
      t.row0 = (int64_t)t.e * g.chunk;
      t.K = min(g.chunk, g.K - (int)t.row0);
    }
    t.M = g.M;
    t.m0 = mt * BM;
    t.n0 = nt * BN;
  }
}

// Split-K tail of ROW problems.  Tiles run in full rounds of one tile per
// CU (g.slots = 256); the rem tiles of the last, partial round are each
// split into sp parts along K (sp = slots / rem, at most the number of K
// tiles; no split below 3 parts), so that every CU ends with about the same
// share of work.  The parts
// write fp32 partial tiles that gemm_fixup_kernel sums in part order.
struct Split {
  int full, rem, sp;
};
template <int MODE>
__device__ __forceinline__ Split split_of(const GemmArgs& g, int ntotal) {
  Split p{ntotal, 0, 1};
  if constexpr (MODE == MODE_ROW) {
    if (g.part != nullptr && g.slots > 0) {
      const int full = ntotal / g.slots * g.slots;
      const int rem = ntotal - full;
      const int nkt = (g.K + BK_ALL - 1) / BK_ALL;
      int sp = rem > 0 ? g.slots / rem : 1;
      if (sp > nkt) sp = nkt;
      // halves do not repay the partial-tile traffic and the fixup
      if (sp >= 3) p = Split{full, rem, sp};
    }
  }
  return p;
}

// This block's work: a whole tile (part < 0) or one K part of a tail tile.
// Whole tiles take the first block ids and the parts the ids after them,
// each range dealt XCD-contiguously, so that with blocks dispatched in id
// order every CU receives the same mix of whole tiles and parts.
template <int MODE, int BM, int BN>
__device__ __forceinline__ bool decode_work(const GemmArgs& g, int* s_tiles, Tile& t, int& part,
                                            int& pid) {
  int num_m;
  const int ntotal = tile_count<MODE, BM>(g, s_tiles, num_m);
  part = -1;
  pid = 0;
  if constexpr (MODE == MODE_ROW) {
    if (g.ksplit > 1) {  // K parts of a one-group problem, a tile's parts adjacent
      int u;
      if (!xcd_logical(ntotal * g.ksplit, u)) return false;
      tile_of<MODE, BM, BN>(g, s_tiles, num_m, u / g.ksplit, t);
      const int kp = g.K / g.ksplit, kpart = u % g.ksplit;
      t.kofs = kpart * kp;
      t.K = kp;
      t.coff = kpart * g.c_kstride;
      return true;
    }
  }
  const Split sp = split_of<MODE>(g, ntotal);
  const int per_full = (sp.full + 7) >> 3;
  const int bid = blockIdx.x;
  int lid;
  if (bid < 8 * per_full) {
    lid = (bid & 7) * per_full + (bid >> 3);
    if (lid >= sp.full) return false;
  } else {
    const int nparts = sp.rem * sp.sp;
    const int per_part = (nparts + 7) >> 3;
    const int b2 = bid - 8 * per_full;
    if ((b2 >> 3) >= per_part) return false;
    const int u = (b2 & 7) * per_part + (b2 >> 3);
    if (u >= nparts) return false;
    lid = sp.full + u / sp.sp;
    part = u % sp.sp;
    pid = u;
  }
  tile_of<MODE, BM, BN>(g, s_tiles, num_m, lid, t);
  if (part >= 0) {
    const int nkt = (t.K + BK_ALL - 1) / BK_ALL;
    const int per = (nkt + sp.sp - 1) / sp.sp;
    const int kb = min(part * per, nkt), ke = min(kb + per, nkt);
    t.kofs = kb * BK_ALL;
    t.K = min(t.K, ke * BK_ALL) - t.kofs;  // may be 0: the part writes zeros
  }
  return true;
}

// 16-byte store that no later kernel of the step reads soon: non-temporal,
// so that it does not push the next kernel's inputs out of the caches
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Epilogue of 8 consecutive outputs of one row at element offset o.  NT:
// the output is stored non-temporally (weight gradients).  The GELU
// epilogue's pre-activation A (read again only in the backward) and the
// fp32-add epilogue's output (the router's dX, a final output) always are.
template <int EPI, bool NT = false>
__device__ __forceinline__ void epi_write8(const GemmArgs& g, int64_t o, float (&v8)[8],
                                           const u32x4* pre = nullptr) {
  if constexpr (EPI == EPI_F32) {
    float* C = static_cast<float*>(g.C) + o;
    *reinterpret_cast<f32x4*>(C) = *reinterpret_cast<const f32x4*>(v8);
    *reinterpret_cast<f32x4*>(C + 4) = *reinterpret_cast<const f32x4*>(v8 + 4);
  } else if constexpr (EPI == EPI_STORE) {
    if constexpr (NT) st16_nt(static_cast<uint16_t*>(g.C) + o, St<uint16_t>::pack(v8));
    else st16(static_cast<uint16_t*>(g.C) + o, St<uint16_t>::pack(v8));
  } else if constexpr (EPI == EPI_GELU) {
    const u32x4 ab = St<uint16_t>::pack(v8);
    if (g.C != nullptr) st16_nt(static_cast<uint16_t*>(g.C) + o, ab);  // NULL: H only
    float a8[8];
    St<uint16_t>::unpack(ab, a8);
#pragma unroll
    for (int q = 0; q < 8; ++q) a8[q] = gelu_tanh(a8[q]);
    st16(static_cast<uint16_t*>(g.C2) + o, St<uint16_t>::pack(a8));
  } else if constexpr (EPI == EPI_ADDF32) {
    // pre: the 32 bytes of the addend, loaded ahead by the caller
    const float* ad = static_cast<const float*>(g.Aux) + o;
    const f32x4 a0 = pre ? __builtin_bit_cast(f32x4, pre[0]) : *reinterpret_cast<const f32x4*>(ad);
    const f32x4 a1 =
        pre ? __builtin_bit_cast(f32x4, pre[1]) : *reinterpret_cast<const f32x4*>(ad + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v8[q] += a0[q];
      v8[q + 4] += a1[q];
    }
    st16_nt(static_cast<uint16_t*>(g.C) + o, St<uint16_t>::pack(v8));
  } else {
    float x8[8];
    // pre: the same 16 bytes, loaded ahead by the caller
    St<uint16_t>::unpack(pre ? *pre : ld16(static_cast<const uint16_t*>(g.Aux) + o), x8);
#pragma unroll
    for (int q = 0; q < 8; ++q) v8[q] *= gelu_tanh_grad(x8[q]);
    st16(static_cast<uint16_t*>(g.C) + o, St<uint16_t>::pack(v8));
  }
}

// Non-split problems (KRAG, fp32 storage): one block per tile.
template <int MODE, int BM, int BN>
__device__ __forceinline__ bool decode_tile(const GemmArgs& g, int* s_tiles, Tile& t) {
  int num_m;
  const int ntotal = tile_count<MODE, BM>(g, s_tiles, num_m);
  int lid;
  if (!xcd_logical(ntotal, lid)) return false;
  tile_of<MODE, BM, BN>(g, s_tiles, num_m, lid, t);
  return true;
}

// ------------------------------------------------------------------ bf16 MFMA kernel
// Main loop: a ring of kStages LDS stages of BK = 32.  Full K tiles travel
// from HBM straight into LDS (global_load_lds_dwordx4: each lane's 16 bytes
// land at M0 + 16 * lane), so each lane picks the global chunk that belongs
// at its LDS slot; a stage is waited for with the vector-memory counter of
// the loads issued after it.  Operands keep their HBM orientation in LDS:
//   KC (K contiguous) tile [rows][32]: 16-byte chunk q of a row stored at
//      chunk q ^ ((row >> KSW) & 3); MFMA fragments are plain 16-byte reads.
//      The shift follows the fragment shape (measured with the LDS
//      bank-conflict counter): KSW = 2 leaves the 32x32x16 fragments (32
//      rows x one chunk) conflict-free and gives the 16x16x32 ones (16 rows
//      x four chunks) four conflict cycles per read; KSW = 1 is the reverse.
//   MN (M or N contiguous) tile [32][R]: chunk c of k-row k stored at chunk
//      c ^ mn_swz(k); fragments come from two ds_read_b64_tr_b16, which
//      transpose 4 x 4 blocks of 16-bit elements across each 16-lane group.
//      The XOR spreads the four k-rows of one such read, and two reads 8
//      k-rows apart (the 16-lane groups of a 16 x 16 x 32 fragment), over
//      distinct banks.
// Rows (KC) or column chunks (MN) past the tile's M or N edge are clamped
// to the last valid one; they only feed outputs that are never stored.  A
// final partial K tile goes through registers with zero fill.
constexpr int BK = BK_ALL;
// stages of the ring: 4 for the 256 x 256 tile (1 block per CU); 3 for
// smaller tiles, so that three blocks of 128 x 128 (or two of 128 x 256)
// fit a CU's LDS
template <int BM, int BN>
constexpr int ring_stages() { return BM * BN >= 256 * 256 ? 4 : 3; }

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s* lds_v4s_ptr;

template <int KSW>
__device__ __forceinline__ int kc_off(int row, int q) {
  return row * BK + ((q ^ ((row >> KSW) & 3)) << 3);
}
__device__ __forceinline__ int mn_swz(int k) { return ((k & 3) << 2) ^ (((k >> 3) & 1) << 1); }
template <int R>
__device__ __forceinline__ int mn_off(int k, int m) {
  return k * R + (((m >> 3) ^ mn_swz(k)) << 3) + (m & 7);
}

// One operand tile of R rows (M or N extent) per stage; KSW: the shift of
// the K-contiguous layout's swizzle (2 for 32x32x16 fragments, 1 for
// 16x16x32 ones).
template <bool KC, int R, int KSW = 2>
struct Operand {
  static_assert(KC || R >= 128, "MN swizzle needs at least 16 chunks per k-row");
  static constexpr int kChunks = R * BK / 8;      // 16-byte chunks per stage
  static constexpr int kLoads = kChunks / 256;    // 1 KB wave loads per wave
  static constexpr int kElems = R * BK;
  const uint16_t* base;
  int64_t src[kLoads];  // element offsets of this lane's chunks, K tile 0
  int64_t kstep;        // element offset of one K tile
  int ld, mn0, lim;

  __device__ __forceinline__ void init(const uint16_t* b, int ld_, int mn0_, int lim_, int w,
                                       int lane) {
    base = b;
    ld = ld_;
    mn0 = mn0_;
    lim = lim_;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int p = (w * kLoads + j) * kWave + lane;  // physical chunk of the stage
      if constexpr (KC) {
        const int row = p >> 2, q = (p & 3) ^ ((row >> KSW) & 3);
        src[j] = (int64_t)min(mn0 + row, lim - 1) * ld + q * 8;
      } else {
        const int k = p / (R / 8), c = (p % (R / 8)) ^ mn_swz(k);
        src[j] = (int64_t)k * ld + min(mn0 + c * 8, lim - 8);
      }
    }
    kstep = KC ? (int64_t)BK : (int64_t)BK * ld;
  }
  // direct HBM -> LDS copy of K tile kt into the stage at LDS byte address lds
  __device__ __forceinline__ void issue(int kt, uint32_t lds, uint32_t wslot) const {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const uint32_t dst = lds + (wslot * kLoads + j) * 1024u;
      const uint16_t* gp = base + src[j] + (int64_t)kt * kstep;
      asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                   :: "v"(gp), "s"(dst) : "memory", "m0");
    }
  }
  // Partial K tile [k0, klim) through registers, zero outside, in two
  // halves, so that all of a thread's loads (both operands') are in flight
  // together before the first store: every chunk is loaded from an address
  // clamped into the operand (its own when it is inside; k0 < klim holds
  // for a partial tile), so that no load is predicated away, and bit i of
  // `in` says whether chunk i is inside; the store half writes zeros for
  // the chunks outside.  (Loaded and stored one chunk at a time, each load
  // waited for alone, the partial tile of the weight gradients, whose K is
  // an expert's ragged row count, cost about 2.5% of their time.)
  static constexpr int kTail = kChunks / 256;  // chunks per thread
  __device__ __forceinline__ void tail_load(int k0, int klim, u32x4 (&v)[kTail],
                                            uint32_t& in) const {
    in = 0;
#pragma unroll
    for (int i = 0; i < kTail; ++i) {
      const int c = threadIdx.x + i * 256;
      int64_t at;
      if constexpr (KC) {
        const int row = c >> 2, q = c & 3;
        const int gr = mn0 + row, gk = k0 + q * 8;
        in |= (uint32_t)(gr < lim && gk < klim) << i;
        at = (int64_t)min(gr, lim - 1) * ld + (gk < klim ? gk : k0);
      } else {
        const int k = c / (R / 8), cc = c % (R / 8);
        const int gk = k0 + k, gm = mn0 + cc * 8;
        in |= (uint32_t)(gk < klim && gm < lim) << i;
        at = (int64_t)min(gk, klim - 1) * ld + min(gm, lim - 8);
      }
      v[i] = ld16(base + at);
    }
  }
  __device__ __forceinline__ void tail_store(uint16_t* s, const u32x4 (&v)[kTail],
                                             uint32_t in) const {
#pragma unroll
    for (int i = 0; i < kTail; ++i) {
      const int c = threadIdx.x + i * 256;
      const u32x4 x = ((in >> i) & 1u) ? v[i] : u32x4{0, 0, 0, 0};
      if constexpr (KC)
        *reinterpret_cast<u32x4*>(s + kc_off<KSW>(c >> 2, c & 3)) = x;
      else
        *reinterpret_cast<u32x4*>(s + mn_off<R>(c / (R / 8), (c % (R / 8)) * 8)) = x;
    }
  }
  // MFMA 32x32x16 fragment of the 32 rows starting at mb, k sub-step kk:
  // lane l gets the 8 k values 8 (l / 32) .. +7 of row mb + l % 32
  __device__ __forceinline__ bf16x8 frag(const uint16_t* s, int mb, int kk, int lane) const {
    if constexpr (KC) {
      return *reinterpret_cast<const bf16x8*>(s + kc_off<KSW>(mb + (lane & 31), kk * 2 + (lane >> 5)));
    } else {
      const int G = lane >> 4, a4 = (lane >> 2) & 3, b4 = lane & 3;
      const int m = mb + (G & 1) * 16 + 4 * b4;
      const int k = kk * 16 + (G >> 1) * 8 + a4;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(s + mn_off<R>(k, m)));
      const v4s hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(s + mn_off<R>(k + 4, m)));
      const v8s both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      return __builtin_bit_cast(bf16x8, both);
    }
  }
  // MFMA 16x16x32 fragment of the 16 rows starting at mb (the whole K tile):
  // lane l gets the 8 k values 8 (l / 16) .. +7 of row mb + l % 16
  __device__ __forceinline__ bf16x8 frag16(const uint16_t* s, int mb, int lane) const {
    if constexpr (KC) {
      return *reinterpret_cast<const bf16x8*>(s + kc_off<KSW>(mb + (lane & 15), lane >> 4));
    } else {
      const int G = lane >> 4, a4 = (lane >> 2) & 3, b4 = lane & 3;
      const int m = mb + 4 * b4, k = G * 8 + a4;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(s + mn_off<R>(k, m)));
      const v4s hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(s + mn_off<R>(k + 4, m)));
      const v8s both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      return __builtin_bit_cast(bf16x8, both);
    }
  }
};

// Epilogue of one wave's TM x TN blocks of 32 x 32 outputs whose origin in
// the block tile is row wr0, column wc0: through LDS, TNP column blocks at a
// time.  The accumulators are 32 x 32 MFMA tiles (f32x16: D[i][j] in lane
// j + 32*((i/4)%2), register (i%4) + 4*(i/8)) or 16 x 16 ones (f32x4, two
// by two per block: D[i][j] in lane j + 16*(i/4), register i%4).  The wave
// stages 32 rows x 32 TNP columns in `stage`, then every lane handles 8
// consecutive columns of a row with 16-byte loads and stores.  Every thread
// of the block calls it with the same trip counts (it synchronises).
template <int MODE, int EPI, int BM, int BN, int TM, int TN, int TNP, typename Acc, int TMA,
          int TNA>
__device__ __forceinline__ void tile_epilogue(const GemmArgs& g, const Tile& t, int part, int pid,
                                              Acc (&acc)[TMA][TNA], float* stage, int wr0,
                                              int wc0) {
  constexpr int MF = sizeof(Acc) == sizeof(f32x16) ? 32 : 16;  // MFMA tile edge
  static_assert(sizeof(Acc) == sizeof(f32x16) || sizeof(Acc) == sizeof(f32x4), "accumulator");
  static_assert(TMA * MF == TM * 32 && TNA * MF == TN * 32, "accumulator tiles");
  constexpr int PW = TNP * 32;      // staged columns per pass
  constexpr int SP = PW + 4;        // staging row stride (floats)
  constexpr int LPR = PW / 8;       // lanes per staged row
  constexpr int RPP = kWave / LPR;  // rows per pass
  const int lane = threadIdx.x & 63;
  const int h = lane >> 5, r = lane & 31;
  int64_t cbase;
  if constexpr (MODE == MODE_ROW) cbase = t.row0 * g.ldc + t.coff;
  else cbase = (int64_t)t.e * g.c_estride;
  float* ptile = part >= 0 ? g.part + (int64_t)pid * BM * BN : nullptr;
  // KRAG split part: fp32 partial sums into the part's [M][N] slab
  float* pslab = nullptr;
  if constexpr (MODE == MODE_KRAG) {
    if (t.slab >= 0) pslab = g.kslab + (int64_t)t.slab * g.M * g.N;
  }
  // GELU backward and fp32 add: the auxiliary input of a pass (the bf16
  // pre-activation, 16 bytes per row and lane; the fp32 addend, 32 bytes)
  // is loaded before the pass's staging, so that a lane's loads are in
  // flight together; where the registers allow (the GELU backward, and the
  // fp32 add on 128 x 128 tiles) every pass's is loaded before the first.
  constexpr bool kPre = EPI == EPI_DGELU || EPI == EPI_ADDF32;
  constexpr int kPreV = EPI == EPI_ADDF32 ? 2 : 1;  // 16-byte vectors per row
  constexpr int kNP = TN / TNP;                      // passes per row block
  constexpr bool kHoist = kPre && (EPI == EPI_DGELU || BM * BN <= 128 * 128);
  u32x4 pa[kHoist ? TM * kNP : 1][kPre ? 32 / RPP : 1][kPreV];
  auto load_aux = [&](int slot, int i, int jp) {
#pragma unroll
    for (int p = 0; p < 32 / RPP; ++p) {
      const int row = t.m0 + wr0 + i * 32 + p * RPP + lane / LPR;
      const int col = t.n0 + wc0 + jp * TNP * 32 + (lane % LPR) * 8;
      const bool ok = row < t.M && col < g.N;
      const int64_t o = cbase + (int64_t)row * g.ldc + col;
#pragma unroll
      for (int u = 0; u < kPreV; ++u) {
        if constexpr (EPI == EPI_DGELU)
          pa[slot][p][u] = ok ? ld16(static_cast<const uint16_t*>(g.Aux) + o) : u32x4{0, 0, 0, 0};
        else
          pa[slot][p][u] =
              ok ? ld16(static_cast<const float*>(g.Aux) + o + 4 * u) : u32x4{0, 0, 0, 0};
      }
    }
  };
  if constexpr (kHoist) {
    if (ptile == nullptr) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jp = 0; jp < kNP; ++jp) load_aux(i * kNP + jp, i, jp);
    }
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j0 = 0; j0 < TN; j0 += TNP) {
      if constexpr (kPre && !kHoist) {
        if (ptile == nullptr) load_aux(0, i, j0 / TNP);
      }
      if constexpr (MF == 32) {
#pragma unroll
        for (int j = 0; j < TNP; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            stage[(8 * (v >> 2) + 4 * h + (v & 3)) * SP + j * 32 + r] = acc[i][j0 + j][v];
      } else {
#pragma unroll
        for (int j = 0; j < 2 * TNP; ++j)
#pragma unroll
          for (int ri = 0; ri < 2; ++ri)
#pragma unroll
            for (int v = 0; v < 4; ++v)
              stage[(ri * 16 + 4 * (lane >> 4) + v) * SP + j * 16 + (lane & 15)] =
                  acc[2 * i + ri][2 * j0 + j][v];
      }
      __syncthreads();
#pragma unroll
      for (int p = 0; p < 32 / RPP; ++p) {
        const int rl = p * RPP + lane / LPR, cl = (lane % LPR) * 8;
        float v8[8];
        *reinterpret_cast<f32x4*>(v8) = *reinterpret_cast<const f32x4*>(stage + rl * SP + cl);
        *reinterpret_cast<f32x4*>(v8 + 4) =
            *reinterpret_cast<const f32x4*>(stage + rl * SP + cl + 4);
        const int tr = wr0 + i * 32 + rl, tc = wc0 + j0 * 32 + cl;  // in the tile
        if (ptile) {  // split part: the whole fp32 tile, unmasked
          float* q = ptile + tr * BN + tc;
          *reinterpret_cast<f32x4*>(q) = *reinterpret_cast<const f32x4*>(v8);
          *reinterpret_cast<f32x4*>(q + 4) = *reinterpret_cast<const f32x4*>(v8 + 4);
        } else if (pslab) {
          const int row = t.m0 + tr, col = t.n0 + tc;
          if (row < g.M && col < g.N) {
            float* q = pslab + (int64_t)row * g.N + col;
            *reinterpret_cast<f32x4*>(q) = *reinterpret_cast<const f32x4*>(v8);
            *reinterpret_cast<f32x4*>(q + 4) = *reinterpret_cast<const f32x4*>(v8 + 4);
          }
        } else {
          const int row = t.m0 + tr, col = t.n0 + tc;
          if (row < t.M && col < g.N)
            epi_write8<EPI, MODE == MODE_KRAG>(g, cbase + (int64_t)row * g.ldc + col, v8,
                                               kPre ? pa[kHoist ? i * kNP + j0 / TNP : 0][p]
                                                    : nullptr);
        }
      }
      __syncthreads();
    }
  }
}

// LDS of one block: the operand ring, reused as the epilogue staging area
template <int MODE, bool B_KC, int BM, int BN>
constexpr int smem_elems() {
  return ring_stages<BM, BN>() *
         (Operand<MODE == MODE_ROW, BM>::kElems + Operand<(MODE == MODE_ROW) && B_KC, BN>::kElems);
}

// One output tile (or split part) t: main loop and epilogue.  Every thread
// of the block calls it; it ends with a barrier, so the block may go on to
// another tile.
template <int MODE, bool B_KC, int EPI, int BM, int BN>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, const Tile& t, int part, int pid,
                                          uint16_t* smem) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr bool A_KC = (MODE == MODE_ROW);
  constexpr bool BKC = (MODE == MODE_ROW) && B_KC;
  using OpA = Operand<A_KC, BM>;
  using OpB = Operand<BKC, BN>;
  constexpr int kStageElems = OpA::kElems + OpB::kElems;
  constexpr int kStages = ring_stages<BM, BN>();
  constexpr int kSmemBytes = smem_elems<MODE, B_KC, BM, BN>() * 2;

  // operand origins, advanced to the first K element of a split part
  const uint16_t* A = static_cast<const uint16_t*>(g.A) + t.row0 * g.lda + t.kofs;
  const uint16_t* B;
  if constexpr (MODE == MODE_ROW)
    B = static_cast<const uint16_t*>(g.B) + (int64_t)t.e * g.b_estride +
        (BKC ? (int64_t)t.kofs : (int64_t)t.kofs * g.ldb);
  else
    B = static_cast<const uint16_t*>(g.B) + t.row0 * g.ldb;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;

  OpA opa;
  OpB opb;
  opa.init(A, g.lda, t.m0, t.M, w, lane);
  opb.init(B, g.ldb, t.n0, g.N, w, lane);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)(smem));
  const uint32_t wslot = __builtin_amdgcn_readfirstlane((uint32_t)w);
  auto issue = [&](int kt) {
    const uint32_t sa = lds0 + (uint32_t)(kt % kStages) * kStageElems * 2u;
    opa.issue(kt, sa, wslot);
    opb.issue(kt, sa + OpA::kElems * 2u, wslot);
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  // Fragments are double-buffered in registers: the MFMAs of one 16-wide k
  // step run on set c while the fragments of the next k step (possibly in
  // the next stage) are read into set c ^ 1, one read after each MFMA.
  bf16x8 fa[2][TM], fb[2][TN];
  auto ring = [&](int kt) { return smem + (kt % kStages) * kStageElems; };
  auto load_frags = [&](int c, const uint16_t* st, int kk) {
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[c][i] = opa.frag(st, wm * WM + i * 32, kk, lane);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[c][j] = opb.frag(st + OpA::kElems, wn * WN + j * 32, kk, lane);
  };
  auto read_frag = [&](int c, const uint16_t* nst, int nkk, int f) {
    if (f < TM) fa[c][f] = opa.frag(nst, wm * WM + f * 32, nkk, lane);
    else fb[c][f - TM] = opb.frag(nst + OpA::kElems, wn * WN + (f - TM) * 32, nkk, lane);
  };
  auto step = [&](int c, const uint16_t* nst, int nkk) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][i], fb[c][j], acc[i][j], 0, 0, 0);
        // fragment q after MFMA q; the last MFMA is followed by any rest
        const int q = i * TN + j;
#pragma unroll
        for (int f = 0; f < TM + TN; ++f)
          if (f == q || (q == TM * TN - 1 && f > q)) read_frag(c ^ 1, nst, nkk, f);
        __builtin_amdgcn_sched_barrier(0);
      }
  };

  // K tiles: nfull full tiles copied straight into LDS, then at most one
  // partial tile written through registers.  The ring holds kStages tiles;
  // tile kt + kStages is issued into tile kt's stage once every wave has
  // read all of tile kt's fragments (the barrier inside iteration kt).
  constexpr int kPer = OpA::kLoads + OpB::kLoads;  // loads per wave per tile
  constexpr int KS = BK / 16;                      // k steps per tile
  const int nfull = t.K / BK;
  const int ntile = nfull + (t.K % BK != 0 ? 1 : 0);
  auto write_tail = [&](int kt) {  // both operands' loads first, then the stores
    u32x4 va[OpA::kTail], vb[OpB::kTail];
    uint32_t ia, ib;
    opa.tail_load(kt * BK, t.K, va, ia);
    opb.tail_load(kt * BK, t.K, vb, ib);
    opa.tail_store(ring(kt), va, ia);
    opb.tail_store(ring(kt) + OpA::kElems, vb, ib);
  };
  if (ntile > 0) {
#pragma unroll
    for (int s0 = 0; s0 < kStages; ++s0)
      if (s0 < nfull) issue(s0);
    if (nfull >= kStages)
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"((kStages - 1) * kPer) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (nfull == 0) write_tail(0);
    __syncthreads();
    load_frags(0, ring(0), 0);
  }
  for (int kt = 0; kt < ntile; ++kt) {
    const uint16_t* st = ring(kt);
#pragma unroll
    for (int kk = 0; kk < KS - 1; ++kk) step(kk & 1, st, kk + 1);
    const bool more = kt + 1 < ntile;
    if (more) {
      if (kt + 1 < nfull) {
        // tile kt+1 has landed once at most the tiles issued after it
        // (up to kStages - 2) are outstanding
        if (kt + kStages - 1 < nfull)
          asm volatile("s_waitcnt vmcnt(%0)" :: "n"((kStages - 2) * kPer) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      } else {
        // tile kt+1 is the partial one; its stage was last read in
        // iteration kt+1-kStages and receives no copy
        write_tail(kt + 1);
      }
      __syncthreads();
      if (kt + kStages < nfull) issue(kt + kStages);
    }
    // after the last tile the reads below re-read this tile (unused)
    step((KS - 1) & 1, more ? ring(kt + 1) : st, 0);
    if constexpr (((KS - 1) & 1) == 0) {
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[0][i] = fa[1][i];
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[0][j] = fb[1][j];
    }
  }
  __syncthreads();  // the staging below overwrites the ring

  static_assert(4 * 32 * (WN + 4) * 4 <= kSmemBytes, "staging does not fit");
  tile_epilogue<MODE, EPI, BM, BN, TM, TN, TN>(g, t, part, pid, acc,
                                               reinterpret_cast<float*>(smem) + w * 32 * (WN + 4),
                                               wm * WM, wn * WN);
}

// Weight gradients on 128 x 128 tiles (short, skewed reductions: most of a
// tile's time is its prologue and epilogue) are held to three waves per
// SIMD, three blocks per CU, so that a block's fixed costs overlap the
// others' MFMAs; unconstrained they took 172 registers, two blocks per CU.
template <int MODE, int BM, int BN>
constexpr int gemm_waves_per_simd() {
  return MODE == MODE_KRAG && BM * BN <= 128 * 128 ? 3 : 1;
}

template <int MODE, bool B_KC, int EPI, int BM, int BN>
__global__ __launch_bounds__(256) __attribute__((
    amdgpu_waves_per_eu(gemm_waves_per_simd<MODE, BM, BN>()))) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __align__(16) uint16_t smem[smem_elems<MODE, B_KC, BM, BN>()];
  __shared__ int s_tiles[257];
  if constexpr (MODE == MODE_KRAG) {
    if (g.kplan != nullptr) {
      // Split plan: XCD x (block id mod 8) walks the work-balanced unit range
      // [plan[2E+3+x], plan[2E+4+x]) with its blocks in turn.
      int num_m;
      (void)tile_count<MODE, BM>(g, s_tiles, num_m);
      const int x = blockIdx.x & 7;
      const int first = g.kplan[2 * g.E + 3 + x], last = g.kplan[2 * g.E + 4 + x];
      const int step = (int)(gridDim.x >> 3);
      for (int lid = first + (int)(blockIdx.x >> 3); lid < last; lid += step) {
        Tile t;
        tile_of<MODE, BM, BN>(g, s_tiles, num_m, lid, t);
        gemm_tile<MODE, B_KC, EPI, BM, BN>(g, t, -1, 0, smem);
      }
      return;
    }
  }
  Tile t;
  int part, pid;
  if (!decode_work<MODE, BM, BN>(g, s_tiles, t, part, pid)) return;
  if constexpr (MODE == MODE_ROW) {
    if (t.m0 >= t.M) return;
  }
  gemm_tile<MODE, B_KC, EPI, BM, BN>(g, t, part, pid, smem);
}

// ------------------------------------------------------------------ ping-pong kernel
// 256 x 256 tiles with eight waves, two per SIMD, in two groups of four
// (waves 0-3 and 4-7; waves w and w + 4 share a SIMD).  Wave (group g,
// q = w % 4) owns rows 128 (q / 2) + 64 g .. +64 and columns 128 (q % 2) ..
// +128 of the tile: 4 x 8 MFMA tiles of 16 x 16, one 16x16x32 MFMA each per
// K tile.  (Only one wave of a SIMD issues MFMAs at a time; in that regime
// the 16x16x32 form, accumulating in VGPRs, keeps the matrix core busier
// than 32x32x16.)  The K tiles pass through the same four-stage LDS ring as
// gemm_tile; group 0 copies their A parts and group 1 their B parts.  Both
// groups run the same sequence of phases, one phase apart, with a block
// barrier after every phase:
//   group 0: read K tile 0's fragments, MFMAs of tile 0, read tile 1, ...
//   group 1: (nothing), read tile 0, MFMAs of tile 0, read tile 1, ...
// so on every SIMD one wave issues MFMAs while the other reads its next
// fragments and issues its copies into the ring stage the previous tile
// freed.  Stage j is read by group 0 in phase 2j and by group 1 in phase
// 2j + 1; tile j + 4 goes into it in phases 2j + 2 (A) and 2j + 3 (B).
constexpr int kPPStages = 4;

template <int MODE, bool B_KC, int EPI>
__device__ __forceinline__ void gemm_tile_pp(const GemmArgs& g, const Tile& t, int part, int pid,
                                             uint16_t* smem) {
  constexpr int BM = 256, BN = 256, TM = 2, TN = 4;  // 32 x 32 blocks of the wave tile
  constexpr int FM = 4, FN = 8;                      // 16 x 16 MFMA tiles of the wave tile
  constexpr bool A_KC = (MODE == MODE_ROW);
  constexpr bool BKC = (MODE == MODE_ROW) && B_KC;
  using OpA = Operand<A_KC, BM, 1>;
  using OpB = Operand<BKC, BN, 1>;
  constexpr int kStageElems = OpA::kElems + OpB::kElems;
  constexpr int S = kPPStages;
  constexpr int kPer = OpA::kLoads + OpB::kLoads;  // loads per group-0 wave per tile

  const uint16_t* A = static_cast<const uint16_t*>(g.A) + t.row0 * g.lda + t.kofs;
  const uint16_t* B;
  if constexpr (MODE == MODE_ROW)
    B = static_cast<const uint16_t*>(g.B) + (int64_t)t.e * g.b_estride +
        (BKC ? (int64_t)t.kofs : (int64_t)t.kofs * g.ldb);
  else
    B = static_cast<const uint16_t*>(g.B) + t.row0 * g.ldb;

  const int lane = threadIdx.x & 63;
  // wave-uniform (scalar) indices: the group decides which branch a wave takes
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = w >> 2, q = w & 3;
  const int wr0 = (q >> 1) * 128 + grp * 64, wc0 = (q & 1) * 128;
  OpA opa;
  OpB opb;
  opa.init(A, g.lda, t.m0, t.M, q, lane);
  opb.init(B, g.ldb, t.n0, g.N, q, lane);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)(smem));
  const uint32_t wslot = __builtin_amdgcn_readfirstlane((uint32_t)q);
  auto ring = [&](int kt) { return smem + (kt % S) * kStageElems; };
  // group 0 copies the A part of every K tile, group 1 the B part
  static_assert(OpA::kLoads == OpB::kLoads, "both groups wait with the same counts");
  constexpr int kP = OpA::kLoads;  // copies per wave per K tile
  auto issue = [&](int kt) {
    const uint32_t sa = lds0 + (uint32_t)(kt % S) * kStageElems * 2u;
    if (grp == 0) opa.issue(kt, sa, wslot);
    else opb.issue(kt, sa + OpA::kElems * 2u, wslot);
  };
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{};
  bf16x8 fa[FM], fb[FN];  // fragments of one K tile
  auto read_frags = [&](const uint16_t* st) {
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = opa.frag16(st, wr0 + i * 16, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = opb.frag16(st + OpA::kElems, wc0 + j * 16, lane);
  };
  auto mfmas = [&]() {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
  };
  // Waits until this wave's copies of K tile j have landed, given that its
  // last copies issued are of tile min(last, nfull - 1).  K is a whole
  // number of K tiles here (the launcher's condition), so every tile is
  // copied straight into LDS.
  const int nfull = t.K / BK;
  const int ntile = nfull;
  auto wait_tile = [&](int j, int last) {
    const int newer = min(last, nfull - 1) - j;
    if (newer >= 3)
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"(3 * kP) : "memory");
    else if (newer == 2)
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * kP) : "memory");
    else if (newer == 1)
      asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kP) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  if (ntile > 0) {
#pragma unroll
    for (int s0 = 0; s0 < S; ++s0)
      if (s0 < nfull) issue(s0);
    wait_tile(0, S - 1);
  }
  __syncthreads();
  // Both groups run the same loop; group 1 starts one barrier later (and
  // group 0 ends with one more), so that its fragment reads of tile j meet
  // group 0's MFMAs of tile j.  s_barrier counts arrivals, whatever the
  // barrier instruction a wave arrives at, and the branches are uniform per
  // wave.  Tile j's stage is free once both groups have read it, i.e. from
  // group 0's read phase of tile j + 1 on; each group copies its part of
  // tile j + S in its read phase of tile j + 1.  Tile j + 1 is read next by
  // group 0, so both groups wait for their parts of it before the barrier
  // that opens that phase: group 1 at the end of its read phase of tile j,
  // group 0 at the end of its MFMA phase of tile j.
  if (grp == 1) __syncthreads();
  for (int j = 0; j < ntile; ++j) {
    // the copies first: they have the longer way to go
    if (j >= 1 && j - 1 + S < nfull) issue(j - 1 + S);
    read_frags(ring(j));
    if (grp == 1 && j + 1 < nfull) wait_tile(j + 1, j + S - 1);
    __syncthreads();
    mfmas();
    if (grp == 0 && j + 1 < nfull) wait_tile(j + 1, j + S - 1);
    __syncthreads();
  }
  if (grp == 0) __syncthreads();
  static_assert(8 * 32 * (64 + 4) * 4 <= S * kStageElems * 2, "staging does not fit");
  tile_epilogue<MODE, EPI, BM, BN, TM, TN, 2>(g, t, part, pid, acc,
                                              reinterpret_cast<float*>(smem) + w * 32 * (64 + 4),
                                              wr0, wc0);
}

// Row GEMMs (MODE_ROW) whose K is a multiple of the K tile.
template <int MODE, bool B_KC, int EPI>
__global__ __launch_bounds__(512) void gemm_pp_kernel(GemmArgs g) {
  static_assert(MODE == MODE_ROW, "row GEMMs only");
  constexpr int BM = 256, BN = 256;
  __shared__ __align__(16) uint16_t smem[smem_elems<MODE, B_KC, BM, BN>()];
  __shared__ int s_tiles[257];
  Tile t;
  int part, pid;
  if (!decode_work<MODE, BM, BN>(g, s_tiles, t, part, pid)) return;
  if (t.m0 >= t.M) return;
  gemm_tile_pp<MODE, B_KC, EPI>(g, t, part, pid, smem);
}

// Sums the split-K parts of the tail tiles (in part order) and applies the
// epilogue; a no-op when the problem had no split tail.
template <int EPI, int BM, int BN>
__global__ __launch_bounds__(256) void gemm_fixup_kernel(GemmArgs g) {
  __shared__ int s_tiles[257];
  int num_m;
  const int ntotal = tile_count<MODE_ROW, BM>(g, s_tiles, num_m);
  const Split sp = split_of<MODE_ROW>(g, ntotal);
  if (sp.sp <= 1) return;
  constexpr int CPR = BN / 8;  // 8-column chunks per tile row
  const int64_t items = (int64_t)sp.rem * BM * CPR;
  for (int64_t it = blockIdx.x * 256 + threadIdx.x; it < items; it += (int64_t)gridDim.x * 256) {
    const int i = (int)(it / (BM * CPR));
    const int in = (int)(it - (int64_t)i * BM * CPR);
    const int tr = in / CPR, tc = (in % CPR) * 8;
    Tile t;
    tile_of<MODE_ROW, BM, BN>(g, s_tiles, num_m, sp.full + i, t);
    const int row = t.m0 + tr, col = t.n0 + tc;
    if (row >= t.M || col >= g.N) continue;
    float v8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const float* q = g.part + ((int64_t)i * sp.sp) * BM * BN + tr * BN + tc;
    // in part order; unrolled so that several parts' loads are in flight
#pragma unroll 4
    for (int p = 0; p < sp.sp; ++p, q += BM * BN) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(q);
      const f32x4 b = *reinterpret_cast<const f32x4*>(q + 4);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        v8[u] += a[u];
        v8[u + 4] += b[u];
      }
    }
    epi_write8<EPI>(g, t.row0 * g.ldc + (int64_t)row * g.ldc + col, v8);
  }
}

// Sums the fp32 partial slabs of the split experts of a weight-gradient
// GEMM in part order and stores the bf16 result (non-temporally, like the
// unsplit tiles); experts that were not split are skipped.
__global__ __launch_bounds__(256) void gemm_krag_fixup_kernel(GemmArgs g) {
  // the plan's unit prefix and first slabs, read once into LDS (one
  // dependent global load per expert would serialise E round trips)
  __shared__ int s_units[257], s_slab[256];
  __shared__ int s_any;
  const int32_t* plan = g.kplan;
  const int E = g.E;
  const int te = g.ntm * g.ntn;
  if (threadIdx.x == 0) s_any = 0;
  __syncthreads();
  for (int i = threadIdx.x; i <= E; i += blockDim.x) s_units[i] = plan[i];
  for (int i = threadIdx.x; i < E; i += blockDim.x) s_slab[i] = plan[E + 1 + i];
  __syncthreads();
  for (int i = threadIdx.x; i < E; i += blockDim.x)
    if (s_units[i + 1] - s_units[i] > te) s_any = 1;
  __syncthreads();
  if (s_any == 0) return;  // no expert was split
  const int64_t chunks = (int64_t)g.M * (g.N / 8);
  for (int e = 0; e < E; ++e) {
    const int parts = (s_units[e + 1] - s_units[e]) / te;
    if (parts <= 1) continue;
    const float* s0 = g.kslab + (int64_t)s_slab[e] * g.M * g.N;
    for (int64_t it = blockIdx.x * 256 + threadIdx.x; it < chunks;
         it += (int64_t)gridDim.x * 256) {
      const int64_t row = it / (g.N / 8);
      const int col = (int)(it - row * (g.N / 8)) * 8;
      float v8[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      const float* q = s0 + row * g.N + col;
#pragma unroll 4
      for (int p = 0; p < parts; ++p, q += (int64_t)g.M * g.N) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(q);
        const f32x4 b = *reinterpret_cast<const f32x4*>(q + 4);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          v8[u] += a[u];
          v8[u + 4] += b[u];
        }
      }
      epi_write8<EPI_STORE, true>(g, (int64_t)e * g.c_estride + row * g.ldc + col, v8);
    }
  }
}

// ------------------------------------------------------------------ fp32 VALU kernel
// Plain LDS-tiled fp32 GEMM with the same problem decode and epilogues,
// used for float storage (64 x 64 tile, 4 x 4 outputs per thread).
template <int MODE, bool B_KC, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  constexpr int BM = 64, BN = 64, BKF = 16;
  __shared__ float sA[BKF][BM + 1];
  __shared__ float sB[BKF][BN + 1];
  __shared__ int s_tiles[257];
  Tile t;
  if (!decode_tile<MODE, BM, BN>(g, s_tiles, t)) return;
  if constexpr (MODE == MODE_ROW) {
    if (t.m0 >= t.M) return;
  }
  const float* A = static_cast<const float*>(g.A) + t.row0 * g.lda;
  const float* B;
  if constexpr (MODE == MODE_ROW) B = static_cast<const float*>(g.B) + (int64_t)t.e * g.b_estride;
  else B = static_cast<const float*>(g.B) + t.row0 * g.ldb;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < t.K; k0 += BKF) {
    for (int i = threadIdx.x; i < BM * BKF; i += 256) {
      const int kk = i % BKF, m = i / BKF;  // A element (m, k)
      const int gm = t.m0 + m, gk = k0 + kk;
      float v = 0.0f;
      if (gm < t.M && gk < t.K) {
        if constexpr (MODE == MODE_ROW) v = A[(int64_t)gm * g.lda + gk];
        else v = A[(int64_t)gk * g.lda + gm];
      }
      sA[kk][m] = v;
    }
    for (int i = threadIdx.x; i < BN * BKF; i += 256) {
      const int kk = i % BKF, n = i / BKF;
      const int gn = t.n0 + n, gk = k0 + kk;
      float v = 0.0f;
      if (gn < g.N && gk < t.K) {
        if constexpr (MODE == MODE_ROW && B_KC) v = B[(int64_t)gn * g.ldb + gk];
        else v = B[(int64_t)gk * g.ldb + gn];
      }
      sB[kk][n] = v;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKF; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
  float* C = static_cast<float*>(g.C);
  float* C2 = static_cast<float*>(g.C2);
  const float* Aux = static_cast<const float*>(g.Aux);
  int64_t cbase;
  if constexpr (MODE == MODE_ROW) cbase = t.row0 * g.ldc;
  else cbase = (int64_t)t.e * g.c_estride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = t.m0 + ty * 4 + i;
    if (row >= t.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = t.n0 + tx * 4 + j;
      if (col >= g.N) continue;
      const int64_t o = cbase + (int64_t)row * g.ldc + col;
      if constexpr (EPI == EPI_STORE || EPI == EPI_F32) C[o] = acc[i][j];
      else if constexpr (EPI == EPI_ADDF32) C[o] = acc[i][j] + Aux[o];
      else if constexpr (EPI == EPI_GELU) {
        if (C != nullptr) C[o] = acc[i][j];
        C2[o] = gelu_tanh(acc[i][j]);
      }
      else C[o] = acc[i][j] * gelu_tanh_grad(Aux[o]);
    }
  }
}

// tiles[e] = sum_{e' < e} ceil(m_e' / BM); tiles[E] = number of M tiles
// (one thread per expert, E <= 256, block scan)
// and, when plan is given, the split plan of the weight-gradient GEMMs
__global__ __launch_bounds__(256) void gemm_schedule_kernel(const int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ tiles, int E,
                                                            int BM, int32_t* __restrict__ plan,
                                                            int te) {
  __shared__ int s_wave[4];
  const int e = threadIdx.x;
  const int m = e < E ? offsets[e + 1] - offsets[e] : 0;
  block_tile_prefix(m, E, BM, tiles, s_wave);
  if (plan != nullptr) block_krag_plan(m, E, te, plan, s_wave);
}

constexpr int kFM = 64, kFN = 64;    // fp32 block tile
// 256 x 256 tiles on the eight-wave ping-pong kernel (gemm_pp_kernel)
constexpr bool kPingPong = true;
// epilogues of the expert GEMMs, the only ones that take 128 x 256 tiles
template <int EPI>
constexpr bool kWideRow() { return EPI == EPI_STORE || EPI == EPI_GELU || EPI == EPI_DGELU; }

// bf16 block tile: 256 x 256 (4 waves of 128 x 128) when the problem has at
// least one full round of such tiles for the chip, else 128 x 128.
inline bool use_big_tile(const moe_cfg& c, int mode, int M, int N, int E) {
  if (c.dtype != MOE_BF16) return false;
  int64_t tiles;
  if (mode == MODE_ROW) tiles = (ceil_div(rows_max(c), 256) + E) * ceil_div(N, 256);
  else tiles = (int64_t)E * ceil_div(M, 256) * ceil_div(N, 256);
  return tiles >= 256;
}
// M tile of the ROW GEMMs of a layer (the schedule is built for it).
// 256 x 256 tiles run on the eight-wave kernel, about 1.45x the 128 x 128
// tiles' rate per flop; a 256-row tile pads an expert by 128 rows on
// average against 64, so it wins from about 80 rows per expert on average.
// Below 128 rows per expert, and when an expert GEMM is narrower than one
// 256-wide tile, the layer keeps 128 x 128 tiles.
inline int row_bm(const moe_cfg& c) {
  if (c.dtype != MOE_BF16) return kFM;
  if (rows_max(c) < 128 * (int64_t)c.E) return 128;
  const int nmin = c.d < c.f ? c.d : c.f;
  if (nmin < 256) return 128;
  return use_big_tile(c, MODE_ROW, 0, nmin, c.E) ? 256 : 128;
}

inline int grid8(int64_t n) { return (int)((n + 7) / 8 * 8); }

// Upper bound of M tiles of a ROW problem: sum_e ceil(m_e/BM) <= Rmax/BM + E
inline int64_t row_mtiles_bound(const moe_cfg& c, int BM) {
  return ceil_div(rows_max(c), BM) + c.E;
}

// A one-group problem's tile count is known here: whether split_of would
// split its tail (256 slots), so that a problem without a split launches no
// fixup kernel.
inline bool one_group_splits(int M, int BM, int ntn, int K) {
  const int64_t ntotal = ceil_div(M, BM) * ntn;
  const int64_t rem = ntotal % 256;
  if (rem == 0) return false;
  const int64_t nkt = ceil_div(K, BK_ALL);
  const int64_t sp = std::min<int64_t>(256 / rem, nkt);
  return sp >= 3;
}

template <int MODE, bool B_KC, int EPI>
int run_gemm(int kid, const moe_cfg& c, GemmArgs g, hipStream_t s) {
  const bool bf = c.dtype == MOE_BF16;
  int BM, BN;
  if (!bf) {
    BM = kFM;
    BN = kFN;
  } else if constexpr (MODE == MODE_ROW) {
    // one-group problems choose freely; grouped ones follow the schedule
    BM = g.offsets ? row_bm(c) : (use_big_tile(c, MODE_KRAG, g.M, g.N, 1) ? 256 : 128);
    BN = BM;
    // expert GEMMs on 128-row tiles, N >= 1024, take 128 x 256 tiles: two blocks
    // per CU instead of three, a third less LDS traffic per flop
    if (kWideRow<EPI>() && g.offsets && BM == 128 && g.N >= 1024) BN = 256;
    if constexpr (B_KC && (EPI == EPI_F32 || EPI == EPI_ADDF32)) {
      if (!g.offsets && g.bm) BM = g.bm;
      if (!g.offsets && g.bn) BN = g.bn;
    }
  } else {
    // expert weight gradients (per-expert offsets) follow krag_tile, whose
    // tile count the split plan was built for
    BM = BN = g.offsets != nullptr ? krag_tile(c)
                                   : (use_big_tile(c, MODE_KRAG, g.M, g.N, g.E) ? 256 : 128);
  }
  g.ntn = (int)ceil_div(g.N, BN);
  int64_t nblk;
  if constexpr (MODE == MODE_ROW) {
    nblk = g.offsets ? row_mtiles_bound(c, BM) * g.ntn : ceil_div(g.M, BM) * g.ntn;
    if (g.ksplit > 1) {
      // K parts: one-group bf16 problems with an fp32 epilogue and whole K
      // tiles per part only; they replace the split-K tail
      if (!bf || g.offsets || EPI != EPI_F32 || g.K % (BK_ALL * g.ksplit) != 0)
        return MOE_ERR_ARG;
      nblk *= g.ksplit;
      g.part = nullptr;
    }
  } else {
    g.ntm = (int)ceil_div(g.M, BM);
    nblk = (int64_t)g.E * g.ntm * g.ntn;
    // the split plan adds at most R / Kc <= 512 / te parts' worth of tiles
    if (g.kplan != nullptr) nblk += 512 + g.ntm * g.ntn;
  }
  if (nblk == 0) return MOE_OK;
  if constexpr (MODE == MODE_ROW) {
    // split-K tail for the bf16 kernels: whole tiles, then up to one block
    // per CU for the parts
    if (bf && g.part != nullptr && (BM == 256 || BM == 128) && (BN == BM || BN == 2 * BM) &&
        (g.offsets || one_group_splits(g.M, BM, g.ntn, g.K))) {
      g.slots = 256;  // CUs
      nblk = grid8(nblk) + g.slots;
    } else {
      g.part = nullptr;
      g.slots = 0;
    }
  }
  const int grid = grid8(nblk);
  if (!bf) {
    MOE_LAUNCH(kid, s, gemm_f32_kernel<MODE, B_KC, EPI><<<grid, 256, 0, s>>>(g));
    return MOE_OK;
  }
  if constexpr (MODE == MODE_ROW && B_KC && EPI == EPI_F32) {
    if (BM == 64 && BN == 64)
      MOE_LAUNCH(kid, s, gemm_bf16_kernel<MODE, B_KC, EPI, 64, 64><<<grid, 256, 0, s>>>(g));
    else if (BM == 64 && BN == 128)
      MOE_LAUNCH(kid, s, gemm_bf16_kernel<MODE, B_KC, EPI, 64, 128><<<grid, 256, 0, s>>>(g));
    else if (BM == 128 && BN == 64)
      MOE_LAUNCH(kid, s, gemm_bf16_kernel<MODE, B_KC, EPI, 128, 64><<<grid, 256, 0, s>>>(g));
    else
      MOE_LAUNCH(kid, s, gemm_bf16_kernel<MODE, B_KC, EPI, 128, 128><<<grid, 256, 0, s>>>(g));
    return MOE_OK;
  }
  if constexpr (MODE == MODE_ROW) {
    if (g.part != nullptr) {
      // the fixup is timed under its own id, so that a probe of the GEMM
      // times the main kernel alone; grid-stride over the split tiles'
      // 8-column chunks, few blocks, so that a problem whose tail was not
      // split pays little for the launch
      const int fgrid = (int)std::min<int64_t>(ceil_div((int64_t)g.slots * BM * BN / 8, 256), 512);
      if (BM == 256) {
        if (kPingPong && g.K % BK_ALL == 0)
          MOE_LAUNCH(kid, s, gemm_pp_kernel<MODE, B_KC, EPI><<<grid, 512, 0, s>>>(g));
        else
          MOE_LAUNCH(kid, s, gemm_bf16_kernel<MODE, B_KC, EPI, 256, 256><<<grid, 256, 0, s>>>(g));
        MOE_LAUNCH(MOE_KERNEL_GEMM_FIXUP, s,
                   gemm_fixup_kernel<EPI, 256, 256><<<fgrid, 256, 0, s>>>(g));
      } else {
        if constexpr (kWideRow<EPI>()) {
          if (BN == 256) {
            MOE_LAUNCH(kid, s,
                       gemm_bf16_kernel<MODE, B_KC, EPI, 128, 256><<<grid, 256, 0, s>>>(g));
            MOE_LAUNCH(MOE_KERNEL_GEMM_FIXUP, s,
                       gemm_fixup_kernel<EPI, 128, 256><<<fgrid, 256, 0, s>>>(g));
            return MOE_OK;
          }
        }
        MOE_LAUNCH(kid, s, gemm_bf16_kernel<MODE, B_KC, EPI, 128, 128><<<grid, 256, 0, s>>>(g));
        MOE_LAUNCH(MOE_KERNEL_GEMM_FIXUP, s,
                   gemm_fixup_kernel<EPI, 128, 128><<<fgrid, 256, 0, s>>>(g));
      }
      return MOE_OK;
    }
  }
  if constexpr (MODE == MODE_ROW && kWideRow<EPI>()) {
    if (BM == 128 && BN == 256) {
      MOE_LAUNCH(kid, s, gemm_bf16_kernel<MODE_ROW, B_KC, EPI, 128, 256><<<grid, 256, 0, s>>>(g));
      return MOE_OK;
    }
  }
  if (MODE == MODE_ROW && BM == 256 && kPingPong && g.K % BK_ALL == 0)
    MOE_LAUNCH(kid, s, gemm_pp_kernel<MODE_ROW, B_KC, EPI><<<grid, 512, 0, s>>>(g));
  else if (BM == 256)
    MOE_LAUNCH(kid, s, gemm_bf16_kernel<MODE, B_KC, EPI, 256, 256><<<grid, 256, 0, s>>>(g));
  else
    MOE_LAUNCH(kid, s, gemm_bf16_kernel<MODE, B_KC, EPI, 128, 128><<<grid, 256, 0, s>>>(g));
  if constexpr (MODE == MODE_KRAG && EPI == EPI_STORE) {
    // the split experts' slabs, summed in part order (a no-op without splits)
    if (g.kplan != nullptr)
      MOE_LAUNCH(MOE_KERNEL_GEMM_FIXUP, s, gemm_krag_fixup_kernel<<<1024, 256, 0, s>>>(g));
  }
  return MOE_OK;
}

int schedule(const moe_cfg& c, const int32_t* offsets, int32_t* tiles, hipStream_t s,
             int32_t* plan = nullptr) {
  MOE_LAUNCH(MOE_KERNEL_SCHEDULE, s,
             gemm_schedule_kernel<<<1, 256, 0, s>>>(offsets, tiles, c.E, row_bm(c), plan,
                                                    (int)krag_te(c)));
  return MOE_OK;
}

}  // namespace

int launch_gemm_schedule(const moe_cfg& c, const int32_t* offsets, int32_t* tiles,
                         hipStream_t s) {
  return schedule(c, offsets, tiles, s);
}

int ffn_row_tile(const moe_cfg& c) { return row_bm(c); }

int launch_gemm(int kid, int mode, bool b_kc, int epi, const moe_cfg& c, GemmArgs g,
                hipStream_t s) {
  if (mode == MODE_ROW && !b_kc && epi == EPI_GELU)
    return run_gemm<MODE_ROW, false, EPI_GELU>(kid, c, g, s);
  if (mode == MODE_ROW && !b_kc && epi == EPI_STORE)
    return run_gemm<MODE_ROW, false, EPI_STORE>(kid, c, g, s);
  if (mode == MODE_ROW && b_kc && epi == EPI_DGELU)
    return run_gemm<MODE_ROW, true, EPI_DGELU>(kid, c, g, s);
  if (mode == MODE_ROW && b_kc && epi == EPI_STORE)
    return run_gemm<MODE_ROW, true, EPI_STORE>(kid, c, g, s);
  if (mode == MODE_KRAG && !b_kc && epi == EPI_STORE)
    return run_gemm<MODE_KRAG, false, EPI_STORE>(kid, c, g, s);
  if (mode == MODE_KRAG && !b_kc && epi == EPI_F32)
    return run_gemm<MODE_KRAG, false, EPI_F32>(kid, c, g, s);
  if (mode == MODE_ROW && b_kc && epi == EPI_ADDF32)
    return run_gemm<MODE_ROW, true, EPI_ADDF32>(kid, c, g, s);
  if (mode == MODE_ROW && b_kc && epi == EPI_F32)
    return run_gemm<MODE_ROW, true, EPI_F32>(kid, c, g, s);
  return MOE_ERR_UNIMPLEMENTED;
}

int launch_ffn_fwd(const moe_cfg& c, const void* x_perm, const int32_t* offsets,
                   const void* W1, const void* W2, void* A, void* H, void* Y, void* ws,
                   hipStream_t s, bool have_tiles) {
  if (rows_max(c) == 0) return MOE_OK;
  const WsLayout L = ws_layout(c);
  int32_t* tiles = ws_ptr<int32_t>(ws, L.tiles);
  int rc = have_tiles ? MOE_OK : schedule(c, offsets, tiles, s);
  if (rc != MOE_OK) return rc;
  const bool rec = (c.flags & MOE_FLAG_RECOMPUTE) != 0;
  if (rec) {
    A = nullptr;  // not kept
    H = ws_ptr<void>(ws, L.rH);
  }
  GemmArgs g{};
  g.offsets = offsets;
  g.tiles = tiles;
  g.E = c.E;
  g.part = ws_ptr<float>(ws, L.gpart);
  // A = x_perm W1 ; H = gelu(A)
  g.A = x_perm; g.B = W1; g.C = A; g.C2 = H;
  g.N = c.f; g.K = c.d; g.lda = c.d; g.ldb = c.f; g.ldc = c.f;
  g.b_estride = (int64_t)c.d * c.f;
  rc = run_gemm<MODE_ROW, false, EPI_GELU>(MOE_KERNEL_GEMM_UP, c, g, s);
  if (rc != MOE_OK) return rc;
  // Y = H W2
  g.A = H; g.B = W2; g.C = Y; g.C2 = nullptr;
  g.N = c.d; g.K = c.f; g.lda = c.f; g.ldb = c.d; g.ldc = c.d;
  g.b_estride = (int64_t)c.f * c.d;
  return run_gemm<MODE_ROW, false, EPI_STORE>(MOE_KERNEL_GEMM_DOWN, c, g, s);
}

int launch_ffn_bwd(const moe_cfg& c, const void* x_perm, const int32_t* offsets,
                   const void* W1, const void* W2, const void* A, const void* H,
                   const void* dYp, void* dXp, void* dW1, void* dW2, void* ws,
                   hipStream_t s, bool have_tiles) {
  const WsLayout L = ws_layout(c);
  int32_t* tiles = ws_ptr<int32_t>(ws, L.tiles);
  // split plan of the weight-gradient GEMMs (bf16), built with the tiles
  int32_t* plan = c.dtype == MOE_BF16 ? ws_ptr<int32_t>(ws, L.kplan) : nullptr;
  void* dA = ws_ptr<void>(ws, L.dA);
  int rc;
  GemmArgs g{};
  g.offsets = offsets;
  g.tiles = tiles;
  g.E = c.E;
  g.part = ws_ptr<float>(ws, L.gpart);
  if (rows_max(c) > 0) {
    rc = have_tiles ? MOE_OK : schedule(c, offsets, tiles, s, plan);
    if (rc != MOE_OK) return rc;
    if (c.flags & MOE_FLAG_RECOMPUTE) {
      // recompute A and H exactly as the forward does (same kernel, inputs
      // and tile schedule: bitwise the forward's values)
      void* rA = ws_ptr<void>(ws, L.rA);
      void* rH = ws_ptr<void>(ws, L.rH);
      g.A = x_perm; g.B = W1; g.C = rA; g.C2 = rH;
      g.N = c.f; g.K = c.d; g.lda = c.d; g.ldb = c.f; g.ldc = c.f;
      g.b_estride = (int64_t)c.d * c.f;
      rc = run_gemm<MODE_ROW, false, EPI_GELU>(MOE_KERNEL_GEMM_RECOMPUTE, c, g, s);
      if (rc != MOE_OK) return rc;
      g.C2 = nullptr;
      A = rA;
      H = rH;
    }
  }
  const bool rows = rows_max(c) > 0;
  // dA = (dYp W2^T) * gelu'(A): B = W2[e] as [N=f][K=d]
  auto gemm_dh = [&]() {
    GemmArgs h = g;
    h.A = dYp; h.B = W2; h.C = dA; h.Aux = A;
    h.N = c.f; h.K = c.d; h.lda = c.d; h.ldb = c.d; h.ldc = c.f;
    h.b_estride = (int64_t)c.f * c.d;
    return run_gemm<MODE_ROW, true, EPI_DGELU>(MOE_KERNEL_GEMM_DH, c, h, s);
  };
  // dXp = dA W1^T: B = W1[e] as [N=d][K=f]
  auto gemm_dx = [&]() {
    GemmArgs h = g;
    h.A = dA; h.B = W1; h.C = dXp;
    h.N = c.d; h.K = c.f; h.lda = c.f; h.ldb = c.f; h.ldc = c.d;
    h.b_estride = (int64_t)c.d * c.f;
    return run_gemm<MODE_ROW, true, EPI_STORE>(MOE_KERNEL_GEMM_DX, c, h, s);
  };
  // dW2[e] = H_e^T dYp_e : M = f, N = d
  // without rows the plan was never built: every expert is empty, nothing
  // to split
  const int32_t* kplan = rows_max(c) > 0 ? plan : nullptr;
  auto gemm_dw2 = [&]() {
    GemmArgs h = g;
    h.part = nullptr;
    h.kplan = kplan;
    h.kslab = ws_ptr<float>(ws, L.kslab);
    h.A = H; h.B = dYp; h.C = dW2;
    h.M = c.f; h.N = c.d; h.lda = c.f; h.ldb = c.d; h.ldc = c.d;
    h.c_estride = (int64_t)c.f * c.d;
    return run_gemm<MODE_KRAG, false, EPI_STORE>(MOE_KERNEL_GEMM_DW2, c, h, s);
  };
  // dW1[e] = x_perm_e^T dA_e : M = d, N = f
  auto gemm_dw1 = [&]() {
    GemmArgs h = g;
    h.part = nullptr;
    h.kplan = kplan;
    h.kslab = ws_ptr<float>(ws, L.kslab);
    h.A = x_perm; h.B = dA; h.C = dW1;
    h.M = c.d; h.N = c.f; h.lda = c.d; h.ldb = c.f; h.ldc = c.f;
    h.c_estride = (int64_t)c.d * c.f;
    return run_gemm<MODE_KRAG, false, EPI_STORE>(MOE_KERNEL_GEMM_DW1, c, h, s);
  };
  // Each GEMM runs right after the one that wrote its largest input, so
  // that input is still in the memory-side cache: dW2 after the combine
  // backward (dYp), dW1 after dH (dA), dX after dW1 (dA again).
  if ((rc = gemm_dw2()) != MOE_OK) return rc;
  if (rows && (rc = gemm_dh()) != MOE_OK) return rc;
  if ((rc = gemm_dw1()) != MOE_OK) return rc;
  if (rows && (rc = gemm_dx()) != MOE_OK) return rc;
  return MOE_OK;
}

}  // namespace moe
