// Permute with capacity drop (F2): per-expert histogram, exclusive scan of
// the kept counts, stable scatter in token order, and the row copy
// x -> x_perm.  Under MOE_FLAG_SLOT_PRIORITY the walk is slot-major, (j, t)
// in lexicographic order: the same kernels then run over k*T virtual tokens
// v = j T + t with one assignment each, so ranks, drops and row order all
// follow the slot-major walk.  Routed tokens are laid out contiguously per expert ("GPU
// expert parallel", section "The step timeline"); assignments beyond the
// capacity are dropped (distributed-training tutorial, "The Capacity
// Factor"), the later tokens first.
//
// Determinism: atomics are used only to count (order-independent) and to
// OR lane bits into 64-bit LDS masks; every position comes from scans and
// popcounts in token order.
#include <mutex>

#include "common.h"

namespace moe {

// Scratch of moe_permute_noalloc: the per-block expert histograms, in a
// fixed device array instead of the caller's workspace.  Host code must
// not use the array's name as a device address: its address on each device
// comes from hipGetSymbolAddress (noalloc_scratch below).
constexpr size_t kNoallocScratchInts = (size_t)1 << 20;  // 4 MiB
static __device__ __align__(256) int32_t scratch[kNoallocScratchInts];

namespace {

constexpr int kPW = kPermTokens / kWave;  // waves per permute block

// The walk: virtual token v, its slot jv < kv; returns the flat assignment
// index t * k + j.  Token-major: v = t, kv = k.  Slot-major: v = j T + t, kv = 1.
struct Walk {
  int64_t T, Tv;
  int k, kv;
  bool slot;
  __device__ __forceinline__ int64_t flat(int64_t v, int jv) const {
    if (slot) {
      const int64_t j = v / T;
      return (v - j * T) * k + j;
    }
    return v * k + jv;
  }
};
static_assert(kPermTokens == 256, "the scatter kernel's offset scan is a 256-thread scan");

// per-block expert histogram: blk[b][e] = #assignments of block b to e
__global__ __launch_bounds__(kPermTokens) void permute_count_kernel(
    const int32_t* __restrict__ idx, int32_t* __restrict__ blk, Walk wk, int E) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int64_t v = (int64_t)blockIdx.x * kPermTokens + threadIdx.x;
  if (v < wk.Tv)
    for (int j = 0; j < wk.kv; ++j) {
      const int e = idx[wk.flat(v, j)];
      if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
    }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x)
    blk[(int64_t)blockIdx.x * E + e] = hist[e];
}

// Column scan over blocks, one block per expert: blk[b][e] becomes block b's
// first position among the assignments to e, and counts[e] their total.
// With no token blocks it writes zero offsets instead (the scatter kernel,
// which writes them otherwise, is not launched).
__global__ __launch_bounds__(256) void permute_scan_kernel(
    int32_t* __restrict__ blk, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int nblk, int E) {
  __shared__ int s_wave[4];
  const int e = blockIdx.x;
  if (nblk == 0) {
    if (threadIdx.x == 0) {
      counts[e] = 0;
      offsets[e] = 0;
      if (e == 0) offsets[E] = 0;
    }
    return;
  }
  int carry = 0;
  for (int b0 = 0; b0 < nblk; b0 += 256) {
    const int b = b0 + threadIdx.x;
    const int v = b < nblk ? blk[(int64_t)b * E + e] : 0;
    int tot;
    const int ex = block_exclusive_scan_256(v, s_wave, &tot);
    if (b < nblk) blk[(int64_t)b * E + e] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) counts[e] = carry;
}

// Rank every assignment among the assignments to the same expert in token
// order, drop beyond capacity, and write the maps.
__global__ __launch_bounds__(kPermTokens) void permute_scatter_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ blk,
    const int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_of, int32_t* __restrict__ src_of, Walk wk, int E, int64_t cap,
    int32_t* __restrict__ tiles, int BM) {
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned long long* mask = reinterpret_cast<unsigned long long*>(smem);  // [kPW][E]
  int32_t* wbase = reinterpret_cast<int32_t*>(mask + kPW * E);            // [kPW][E]
  int32_t* s_off = wbase + kPW * E;                                       // [E]
  __shared__ int s_wave[4];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t v = (int64_t)blockIdx.x * kPermTokens + threadIdx.x;
  const bool valid = v < wk.Tv;

  // offsets = exclusive scan of min(counts, C) (E <= 256, one per thread);
  // block 0 publishes them
  {
    const int e = threadIdx.x;
    int kept = 0;
    if (e < E) {
      const int32_t cnt = counts[e];
      kept = (cap >= 0 && cnt > cap) ? (int32_t)cap : cnt;
    }
    int tot;
    const int ex = block_exclusive_scan_256(kept, s_wave, &tot);
    if (e < E) s_off[e] = ex;
    if (blockIdx.x == 0) {
      if (e < E) offsets[e] = ex;
      if (e == 0) offsets[E] = tot;
      // and the grouped GEMMs' M-tile prefix of the kept rows (uniform branch)
      if (tiles != nullptr) block_tile_prefix(kept, E, BM, tiles, s_wave);
    }
  }

  for (int i = threadIdx.x; i < kPW * E; i += blockDim.x) mask[i] = 0ull;
  __syncthreads();
  if (valid)
    for (int j = 0; j < wk.kv; ++j) {
      const int e = idx[wk.flat(v, j)];
      if ((unsigned)e < (unsigned)E) atomicOr(&mask[w * E + e], 1ull << lane);
    }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int32_t run = 0;
    for (int ww = 0; ww < kPW; ++ww) {
      wbase[ww * E + e] = run;
      run += __popcll(mask[ww * E + e]);
    }
  }
  __syncthreads();
  if (valid) {
    const unsigned long long lt = (1ull << lane) - 1ull;
    for (int j = 0; j < wk.kv; ++j) {
      const int64_t a = wk.flat(v, j);
      const int e = idx[a];
      if ((unsigned)e >= (unsigned)E) {  // outside the contract: treat as dropped
        row_of[a] = -1;
        continue;
      }
      const int64_t pos = (int64_t)blk[(int64_t)blockIdx.x * E + e] + wbase[w * E + e] +
                          __popcll(mask[w * E + e] & lt);
      int32_t row = -1;
      if (cap < 0 || pos < cap) {
        row = (int32_t)(s_off[e] + pos);
        src_of[row] = (int32_t)a;
      }
      row_of[a] = row;
    }
  }
}

// x_perm[row_of[t,j]] = x[t]: one wave per token reads the row once (up to
// kCopyVec 16-byte vectors per lane in flight) and writes every kept copy.
// x is read non-temporally, so that it does not push the copies, which the
// up-projection reads next, out of the memory-side cache.
constexpr int kCopyVec = 4;
template <typename T>
__global__ __launch_bounds__(256) void permute_copy_kernel(
    const T* __restrict__ x, const int32_t* __restrict__ row_of, T* __restrict__ x_perm,
    int64_t T_, int d, int k) {
  constexpr int V = St<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int nch = d / V;
  for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < T_;
       t += (int64_t)gridDim.x * 4) {
    const T* src = x + t * (int64_t)d;
    for (int c0 = 0; c0 < nch; c0 += kWave * kCopyVec) {
      u32x4 v[kCopyVec];
#pragma unroll
      for (int q = 0; q < kCopyVec; ++q) {
        const int c = c0 + q * kWave + lane;
        if (c < nch) v[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + c * V));
      }
      for (int j = 0; j < k; ++j) {
        const int32_t row = row_of[t * k + j];
        if (row < 0) continue;
        T* dst = x_perm + (int64_t)row * d;
#pragma unroll
        for (int q = 0; q < kCopyVec; ++q) {
          const int c = c0 + q * kWave + lane;
          if (c < nch) st16(dst + c * V, v[q]);
        }
      }
    }
  }
}

}  // namespace

namespace {

int permute_with(const moe_cfg& c, const void* x, const int32_t* idx, int32_t* counts,
                 int32_t* offsets, int32_t* row_of, int32_t* src_of, void* x_perm,
                 int32_t* blk, hipStream_t s, int32_t* tiles) {
  Walk wk;
  wk.T = c.T;
  wk.k = c.k;
  wk.slot = (c.flags & MOE_FLAG_SLOT_PRIORITY) != 0;
  wk.Tv = wk.slot ? c.T * c.k : c.T;
  wk.kv = wk.slot ? 1 : c.k;
  const int nblk = c.T > 0 ? (int)ceil_div(wk.Tv, kPermTokens) : 0;  // L.nblk_perm
  if (nblk > 0)
    MOE_LAUNCH(MOE_KERNEL_PERMUTE_COUNT, s,
               permute_count_kernel<<<nblk, kPermTokens, c.E * 4, s>>>(idx, blk, wk, c.E));
  MOE_LAUNCH(MOE_KERNEL_PERMUTE_SCAN, s,
             permute_scan_kernel<<<c.E, 256, 0, s>>>(blk, counts, offsets, nblk, c.E));
  if (nblk > 0) {
    const size_t sm = (size_t)kPW * c.E * 8 + (size_t)kPW * c.E * 4 + (size_t)c.E * 4;
    MOE_LAUNCH(MOE_KERNEL_PERMUTE_SCATTER, s,
               permute_scatter_kernel<<<nblk, kPermTokens, sm, s>>>(
                   idx, blk, counts, offsets, row_of, src_of, wk, c.E, c.capacity, tiles,
                   ffn_row_tile(c)));
    const int g = (int)std::min<int64_t>(ceil_div(c.T, 4), 65536);
    if (c.dtype == MOE_BF16)
      MOE_LAUNCH(MOE_KERNEL_PERMUTE_COPY, s,
                 permute_copy_kernel<uint16_t><<<g, 256, 0, s>>>(
                     static_cast<const uint16_t*>(x), row_of,
                     static_cast<uint16_t*>(x_perm), c.T, c.d, c.k));
    else
      MOE_LAUNCH(MOE_KERNEL_PERMUTE_COPY, s,
                 permute_copy_kernel<float><<<g, 256, 0, s>>>(
                     static_cast<const float*>(x), row_of, static_cast<float*>(x_perm),
                     c.T, c.d, c.k));
  }
  return MOE_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device and kept (the array lives as long as the process)
constexpr int kMaxDevices = 64;
int32_t* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

int noalloc_scratch(int32_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    note_launch_error(MOE_KERNEL_PERMUTE_COUNT, e);
    return MOE_ERR_LAUNCH;
  }
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNIMPLEMENTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      note_launch_error(MOE_KERNEL_PERMUTE_COUNT, e != hipSuccess ? e : hipErrorInvalidSymbol);
      return MOE_ERR_LAUNCH;
    }
    g_scratch[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

int launch_permute(const moe_cfg& c, const void* x, const int32_t* idx,
                   int32_t* counts, int32_t* offsets, int32_t* row_of,
                   int32_t* src_of, void* x_perm, void* ws, hipStream_t s, int32_t* tiles) {
  const WsLayout L = ws_layout(c);
  return permute_with(c, x, idx, counts, offsets, row_of, src_of, x_perm,
                      ws_ptr<int32_t>(ws, L.perm_blk), s, tiles);
}

size_t permute_noalloc_scratch_bytes(const moe_cfg& c) {
  return (size_t)ws_layout(c).nblk_perm * c.E * 4;
}

size_t permute_noalloc_scratch_max() { return kNoallocScratchInts * 4; }

int launch_permute_noalloc(const moe_cfg& c, const void* x, const int32_t* idx,
                           int32_t* counts, int32_t* offsets, int32_t* row_of,
                           int32_t* src_of, void* x_perm, hipStream_t s) {
  if (permute_noalloc_scratch_bytes(c) > permute_noalloc_scratch_max())
    return MOE_ERR_WORKSPACE;
  int32_t* blk = nullptr;
  const int rc = noalloc_scratch(&blk);
  if (rc != MOE_OK) return rc;
  // every histogram entry is written by the count kernel before it is read:
  // nothing left by an earlier call needs clearing
  return permute_with(c, x, idx, counts, offsets, row_of, src_of, x_perm, blk, s, nullptr);
}

}  // namespace moe
