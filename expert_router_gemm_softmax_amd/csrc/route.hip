// Router forward (F1): logits z = x Wr + b, softmax over all experts,
// top-k in the order (z descending, expert ascending), gates = chosen
// probabilities.  Expert-parallel MoE layer, "GPU expert parallel"
// (aicassindra.com), sections "The step timeline" and "Sharded by expert,
// replicated everywhere else" (router decisions must agree on every rank).
//
// Decision rule.  The decision is defined on the canonical logit
// z = RN_fp32(sum_i x_i Wr_ie + b_e) with the sum in fp64.  The fast path
// computes zf with fp32 accumulation; with |zf - z| < tau/2 for every
// expert, two experts whose fast logits differ by at least tau are in the
// same order canonically.  Cutting the fast top-(k+1) wherever neighbours
// differ by at least tau splits it into clusters that keep their order
// canonically; only inside a cluster of two or more can the order change.
// An expert below rank k can enter the top-k only through the cluster of
// rank k, and only if no cut separates rank k from rank k - 1 and its zf
// lies within tau of the (k+1)-th value (any expert further below has k+1
// experts canonically above it).  If there is no cluster of two, the fast
// order is the canonical one; otherwise the members of those clusters that
// reach an output rank are rescored in fp64 and each cluster's output ranks
// go to its canonically best members.
//
// Two kernels after the logits.  The fast logits x Wr come from the grouped
// GEMM (one group of T rows, the transposed router weights as a
// K-contiguous operand, fp32 epilogue into [T, Epad] workspace matrices):
// the router is a skinny GEMM whose cost is reading x once.  When its tiles
// alone would leave CUs idle, K is cut into 2 or 4 parts, each block writing
// one part's partial logits.  The select kernel takes four tokens per wave,
// one per row of 16 lanes (lanes across experts): the parts' sum, softmax
// statistics, top-(k+1), coalesced writes of probabilities, experts and
// gates, and the worklist of uncertain tokens; the rescoring kernel then
// certifies those tokens in fp64, one per wave.
// Gates are the chosen probabilities, or (MOE_FLAG_RENORM) those divided by
// their sum taken in selection order; both kernels form them the same way.
#include "gemm.h"

#include <float.h>

namespace moe {

int launch_transpose_wr(const moe_cfg& c, const void* Wr, void* wrT, int* wl_count,
                        hipStream_t s);

namespace {

struct RouteWorklist {
  int* count;  // number of uncertain tokens
  int* tok;    // [T] their token indices
  int* n;      // [T] their candidate counts
  int* e;      // [T, Epad] their candidates, ascending: expert | lo << 16 |
               // hi << 24, [lo, hi] the output ranks of the candidate's cluster
};

// wrT[e][i] = Wr[i][e] for e < E, zero rows for E <= e < Epad.
template <typename T>
__global__ void transpose_wr_kernel(const T* __restrict__ Wr, T* __restrict__ wrT,
                                    int d, int E, int Epad, int* __restrict__ wl_count) {
  if (wl_count && blockIdx.x == 0 && threadIdx.x == 0) *wl_count = 0;
  const int64_t n = (int64_t)Epad * d;
  for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < n;
       o += (int64_t)gridDim.x * blockDim.x) {
    const int e = (int)(o / d), i = (int)(o - (int64_t)e * d);
    wrT[o] = e < E ? Wr[(int64_t)i * E + e] : T(0);
  }
}

// Wave argmax over (value, expert) pairs: larger value first, lower
// expert on equal values (-0 == +0).  Conditions here and at the callers
// are combined with bitwise operators, which evaluate every operand, so the
// compiler emits compares and selects rather than branches.
__device__ __forceinline__ bool route_better(float v, int e, float w, int f) {
  return (v > w) | ((v == w) & (e < f));
}
// The wave's best (v, e) under route_better, in every lane: DPP exchanges
// within each row of 16, then the four row winners compared in row order
// (route_better is a strict total order, so the pairing does not matter).
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& e) {
  const float w = dpp_f<CTRL>(v);
  const int f = dpp_i<CTRL>(e);
  if (route_better(w, f, v, e)) {
    v = w;
    e = f;
  }
}
__device__ __forceinline__ void wave_argmax(float& v, int& e) {
  argmax_step<kDppXor1>(v, e);
  argmax_step<kDppXor2>(v, e);
  argmax_step<kDppHalfMirror>(v, e);
  argmax_step<kDppMirror>(v, e);
  float bv = readlane_f(v, 0);
  int be = __builtin_amdgcn_readlane(e, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float w = readlane_f(v, 16 * r);
    const int f = __builtin_amdgcn_readlane(e, 16 * r);
    if (route_better(w, f, bv, be)) {
      bv = w;
      be = f;
    }
  }
  v = bv;
  e = be;
}

// Row reductions: the same DPP exchanges as the wave reductions, stopped
// after the row of 16 lanes, so that each row (one token) gets its own
// result in all of its lanes.  Every lane of a row combines the same values
// in the same pairing (a + b and b + a are equal), so they agree bitwise.
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  return fmaxf(v, dpp_f<kDppMirror>(v));
}
__device__ __forceinline__ float row_sum(float v) {
  v += dpp_f<kDppXor1>(v);
  v += dpp_f<kDppXor2>(v);
  v += dpp_f<kDppHalfMirror>(v);
  return v + dpp_f<kDppMirror>(v);
}
__device__ __forceinline__ void row_argmax(float& v, int& e) {
  argmax_step<kDppXor1>(v, e);
  argmax_step<kDppXor2>(v, e);
  argmax_step<kDppHalfMirror>(v, e);
  argmax_step<kDppMirror>(v, e);
}

// Select: four tokens per wave, one per row of 16 lanes; lane s of a row
// holds the V = Epad / 16 consecutive experts s V .. s V + V - 1 (16- or
// 8-byte loads of the logits).  Softmax statistics by row reductions; the
// top-(k+1) by k+1 rounds of a row argmax, the round's expert and its
// probability (from the lane that owns it) kept by lane j % 16 of the row
// for choice j.  Tokens whose adjacent top-(k+1) gaps fall below tau go to
// the rescoring worklist with the members of their uncertain clusters
// (ascending experts, each with its cluster's output ranks), and their
// experts and gates written here are provisional for those ranks.  The
// token loop is uniform over the wave (rows past T
// compute on zeros and store nothing), so every DPP exchange runs with all
// lanes active.
template <int V>
__global__ __launch_bounds__(256) void route_kernel(
    const float* __restrict__ zf, int ks, const float* __restrict__ bias, float* __restrict__ probs,
    int32_t* __restrict__ idx_out, float* __restrict__ gate_out, int* __restrict__ wl_count,
    int* __restrict__ wl_tok, int* __restrict__ wl_n, int* __restrict__ wl_e, int64_t T_,
    int E, int Epad, int k, float tau, bool renorm) {
  static_assert(V == 2 || V == 4 || V == 8 || V == 16, "experts per lane");
  const int lane = threadIdx.x & 63;
  const int sub = lane & 15, row0 = lane & 48;
  const int e0 = sub * V;
  float bz[V];
#pragma unroll
  for (int i = 0; i < V; ++i) bz[i] = (e0 + i < E && bias) ? bias[e0 + i] : 0.0f;
  // probs rows as vectors when E fills the lanes and probs is aligned to them
  const bool vec = E == Epad && reinterpret_cast<uintptr_t>(probs) % (V == 2 ? 8 : 16) == 0;
  const int64_t nw = (int64_t)gridDim.x * 4;
  for (int64_t tb = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4; tb < T_; tb += nw * 4) {
    const int64_t t = tb + (lane >> 4);
    const bool live = t < T_;
    float z[V];
    if (live) {
      // the K parts' partial logits, summed in part order
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if (p >= ks) break;
        const float* zr = zf + ((int64_t)p * T_ + t) * Epad + e0;
        float a[V];
        if constexpr (V == 2) {
          const f32x2_t v2 = *reinterpret_cast<const f32x2_t*>(zr);
          a[0] = v2[0];
          a[1] = v2[1];
        } else {
#pragma unroll
          for (int u = 0; u < V / 4; ++u) {
            const f32x4 v4 = *reinterpret_cast<const f32x4*>(zr + 4 * u);
#pragma unroll
            for (int q = 0; q < 4; ++q) a[4 * u + q] = v4[q];
          }
        }
#pragma unroll
        for (int i = 0; i < V; ++i) z[i] = p == 0 ? a[i] : z[i] + a[i];
      }
    }
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      z[i] = e0 + i < E ? (live ? z[i] + bz[i] : 0.0f) : -INFINITY;
      m = fmaxf(m, z[i]);
    }
    m = row_max(m);
    float ps[V], sum = 0.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      ps[i] = e0 + i < E ? expf(z[i] - m) : 0.0f;
      sum += ps[i];
    }
    sum = row_sum(sum);
#pragma unroll
    for (int i = 0; i < V; ++i) ps[i] = ps[i] / sum;
    if (live) {
      float* pr = probs + t * E + e0;
      if (vec) {  // whole rows of V: vector stores (t E + e0 is a multiple of V)
        if constexpr (V == 2) {
          *reinterpret_cast<f32x2_t*>(pr) = f32x2_t{ps[0], ps[1]};
        } else {
#pragma unroll
          for (int u = 0; u < V / 4; ++u)
            *reinterpret_cast<f32x4*>(pr + 4 * u) =
                f32x4{ps[4 * u], ps[4 * u + 1], ps[4 * u + 2], ps[4 * u + 3]};
        }
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i)
          if (e0 + i < E) pr[i] = ps[i];
      }
    }
    // top-(k+1): taken experts are marked per slot by their owner lane
    const int nsel = E > k ? k + 1 : k;
    uint32_t taken = 0;
    float vsel_prev = 0.0f, vk = -INFINITY;
    int ek = 0;
    bool flag = false;
    uint64_t cuts = 0;  // bit r: v_{r-1} - v_r >= tau (ranks 1 .. k)
    float S = 0.0f;
    float psel0 = 0.0f, psel1 = 0.0f;  // lane s: choices s and s + 16
    int esel0 = 0, esel1 = 0;
    for (int j = 0; j < nsel; ++j) {
      float v = -INFINITY;
      int e = 0x7fffffff;
      // this lane's best untaken expert
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const bool ok = (e0 + i < E) & !((taken >> i) & 1u) & route_better(z[i], e0 + i, v, e);
        v = ok ? z[i] : v;
        e = ok ? e0 + i : e;
      }
      row_argmax(v, e);
      const int o = e - e0;  // the winner's slot in its owner lane
      if ((unsigned)o < (unsigned)V) taken |= 1u << o;
      if (j > 0) {
        if (vsel_prev - v < tau) flag = true;
        else cuts |= 1ull << j;
      }
      vsel_prev = v;
      if (j < k) {
        float pown = 0.0f;
#pragma unroll
        for (int i = 0; i < V; ++i)
          if (i == o) pown = ps[i];
        const float pe = __shfl(pown, row0 | (e / V), kWave);
        S += pe;
        if (j < 16) {
          if (sub == j) {
            psel0 = pe;
            esel0 = e;
          }
        } else if (sub == j - 16) {
          psel1 = pe;
          esel1 = e;
        }
      } else {
        vk = v;
        ek = e;
      }
    }
    if (nsel == k) cuts |= 1ull << k;  // no (k+1)-th expert: nothing below rank k - 1 competes
    if (live) {
      if (sub < k) {
        idx_out[t * k + sub] = esel0;
        gate_out[t * k + sub] = renorm ? psel0 / S : psel0;
      }
      if (sub + 16 < k) {
        idx_out[t * k + sub + 16] = esel1;
        gate_out[t * k + sub + 16] = renorm ? psel1 / S : psel1;
      }
    }
    if (flag && live) {  // uniform over the row
      // Cuts split ranks 0 .. k into clusters; members of different
      // clusters keep their fast order canonically.  The candidates are the
      // members of clusters of two or more that reach an output rank (< k),
      // each with that cluster's output ranks [lo, hi]; the unranked
      // experts within tau of v_k join the last cluster when no cut
      // separates rank k from rank k - 1.
      int rk[V];
#pragma unroll
      for (int i = 0; i < V; ++i) rk[i] = -1;
      for (int r = 0; r < nsel; ++r) {
        const int er = r < k ? __shfl(r < 16 ? esel0 : esel1, row0 | (r & 15), kWave) : ek;
#pragma unroll
        for (int i = 0; i < V; ++i)
          if (e0 + i == er) rk[i] = r;
      }
      const float thr = E > k ? vk - tau : -INFINITY;
      const bool open_end = !((cuts >> k) & 1ull);
      uint32_t in = 0;
      int ent[V];
#pragma unroll
      for (int i = 0; i < V; ++i) {
        ent[i] = 0;
        int r = rk[i];
        bool cand = true;
        if (r < 0) {  // unranked: a candidate only within tau of v_k and with no cut at k
          cand = open_end && e0 + i < E && z[i] >= thr;
          r = k;
        }
        // cluster of rank r: from the last cut at or below r to the rank
        // before the first cut above it
        const uint64_t upto = (2ull << r) - 1ull;
        const uint64_t below = cuts & upto, above = cuts & ~upto;
        const int lo = below ? 63 - __clzll((long long)below) : 0;
        const int hf = above ? __ffsll((long long)above) - 2 : nsel - 1;
        if (cand && hf > lo && lo < k) {
          in |= 1u << i;
          ent[i] = (e0 + i) | (lo << 16) | (min(hf, k - 1) << 24);
        }
      }
      // this lane's first position among the row's candidates (ascending
      // experts): inclusive scan of the counts over the row, minus its own
      const int cnt = __popc(in);
      int incl = cnt;
#pragma unroll
      for (int dlt = 1; dlt < 16; dlt <<= 1) {
        const int up = __shfl_up(incl, dlt, 16);
        if (sub >= dlt) incl += up;
      }
      const int n = __shfl(incl, row0 | 15, kWave);
      int slot = 0;
      if (sub == 0) slot = atomicAdd(wl_count, 1);
      slot = __shfl(slot, row0, kWave);
      int pos = incl - cnt;
#pragma unroll
      for (int i = 0; i < V; ++i)
        if ((in >> i) & 1u) wl_e[(int64_t)slot * Epad + pos++] = ent[i];
      if (sub == 0) {
        wl_tok[slot] = (int)t;
        wl_n[slot] = n;
      }
    }
  }
}

constexpr int kRescoreGroup = 4;  // candidates rescored together

// Canonical rescoring of the worklist: one wave per uncertain token.  Each
// candidate's logit is RN_fp32(fp64 sum of x_i Wr_ie + b_e), four
// candidates at a time with all their 16-byte loads in flight; lane u % 64
// keeps candidate u.  Each candidate carries its cluster's output ranks
// [lo, hi]; rank r inside some cluster goes to the best (z descending,
// expert ascending) of that cluster's candidates not yet placed, by wave
// argmax, and every other rank keeps the select kernel's expert.  The
// token's experts and gates are then written again in full (the gate
// renormalisation sums the final choices in rank order).
template <typename T>
__global__ __launch_bounds__(256) void route_rescore_kernel(
    const int* __restrict__ wl_count, const int* __restrict__ wl_tok,
    const int* __restrict__ wl_n, const int* __restrict__ wl_e, const T* __restrict__ x, const T* __restrict__ wrT, const float* __restrict__ bias,
    const float* __restrict__ probs, int32_t* __restrict__ idx_out,
    float* __restrict__ gate_out, int d, int E, int Epad, int k, bool renorm) {
  constexpr int V = St<T>::kVec;
  constexpr int CPL = 4;  // 16-byte chunks per lane per pass
  const int lane = threadIdx.x & 63;
  const int count = *wl_count;
  const int nch = d / V;
  for (int slot = blockIdx.x * 4 + (threadIdx.x >> 6); slot < count; slot += gridDim.x * 4) {
    const int64_t t = wl_tok[slot];
    const int n = wl_n[slot];
    const int* cand = wl_e + (int64_t)slot * Epad;
    float cz[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // candidate lane + 64 i, canonical z
    const T* xr = x + t * d;
    for (int c0 = 0; c0 < n; c0 += kRescoreGroup) {
      const T* wr[kRescoreGroup];
      int ec[kRescoreGroup];
#pragma unroll
      for (int q = 0; q < kRescoreGroup; ++q) {
        ec[q] = cand[c0 + q < n ? c0 + q : c0] & 0xffff;
        wr[q] = wrT + (int64_t)ec[q] * d;
      }
      double acc[kRescoreGroup];
#pragma unroll
      for (int q = 0; q < kRescoreGroup; ++q) acc[q] = 0.0;
      for (int g = lane; g < nch; g += CPL * kWave) {
        u32x4 xv[CPL], wv[kRescoreGroup][CPL];
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
          const int c = g + u * kWave;
          if (c < nch) {
            xv[u] = ld16(xr + c * V);
#pragma unroll
            for (int q = 0; q < kRescoreGroup; ++q) wv[q][u] = ld16(wr[q] + c * V);
          }
        }
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
          if (g + u * kWave >= nch) continue;
          float xf[V];
          St<T>::unpack(xv[u], xf);
#pragma unroll
          for (int q = 0; q < kRescoreGroup; ++q) {
            float wf[V];
            St<T>::unpack(wv[q][u], wf);
#pragma unroll
            for (int i = 0; i < V; ++i) acc[q] += (double)xf[i] * (double)wf[i];
          }
        }
      }
#pragma unroll
      for (int q = 0; q < kRescoreGroup; ++q) {
        const double sum = wave_sum_d(acc[q]);
        const int u = c0 + q;  // lane u % 64 keeps candidate u in slot u / 64
        if (u < n && (u & 63) == lane) {
          const float zc = (float)(sum + (double)(bias ? bias[ec[q]] : 0.0f));
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i == (u >> 6)) cz[i] = zc;
        }
      }
    }
    // candidates' experts and cluster ranks; the ranks some cluster covers
    int ce[4], lo[4], hi[4];
    uint32_t cov = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = lane + kWave * i;
      const int en = u < n ? cand[u] : 0;
      ce[i] = u < n ? (en & 0xffff) : 0x7fffffff;
      lo[i] = u < n ? (en >> 16) & 0xff : 1;
      hi[i] = u < n ? (en >> 24) & 0xff : 0;
      if (u < n) cov |= (2u << hi[i]) - (1u << lo[i]);  // ranks lo .. hi (hi <= 31)
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cov |= (uint32_t)__shfl_xor((int)cov, o, kWave);
    const int eprov = lane < k ? idx_out[t * k + lane] : 0;  // the select kernel's experts
    float pv[4];  // the token's probabilities, expert lane + 64 i in slot i
#pragma unroll
    for (int i = 0; i < 4; ++i) pv[i] = lane + kWave * i < E ? probs[t * E + lane + kWave * i] : 0.0f;
    uint32_t taken = 0;
    float psel = 0.0f, S = 0.0f;  // lane j: probability of the j-th choice
    int esel = 0;
    for (int j = 0; j < k; ++j) {
      int e;
      if ((cov >> j) & 1u) {
        float v = -INFINITY;
        e = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = (lo[i] <= j) & (j <= hi[i]) & !((taken >> i) & 1u) &
                          route_better(cz[i], ce[i], v, e);
          v = ok ? cz[i] : v;
          e = ok ? ce[i] : e;
        }
        wave_argmax(v, e);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (ce[i] == e && !((taken >> i) & 1u)) taken |= 1u << i;
      } else {
        e = __builtin_amdgcn_readlane(eprov, j);
      }
      // e is wave-uniform: its probability from the lane that holds it
      const float pq = (e >> 6) == 0 ? pv[0] : (e >> 6) == 1 ? pv[1] : (e >> 6) == 2 ? pv[2] : pv[3];
      const float pe = readlane_f(pq, e & 63);
      S += pe;
      if (lane == j) {
        psel = pe;
        esel = e;
      }
    }
    if (lane < k) {
      idx_out[t * k + lane] = esel;
      gate_out[t * k + lane] = renorm ? psel / S : psel;
    }
  }
}

template <typename T>
int launch_route_t(const moe_cfg& c, const T* x, const T* Wr, const float* b, float* probs,
                   int32_t* idx, float* gate, T* wrT, float* zf, const RouteWorklist& wl,
                   hipStream_t s) {
  const int Epad = route_epad(c.E);
  const bool renorm = (c.flags & MOE_FLAG_RENORM) != 0;
  int rc = launch_transpose_wr(c, Wr, wrT, wl.count, s);
  if (rc != MOE_OK) return rc;
  // zf = x wrT^T: one group of T rows, N = Epad, K = d
  GemmArgs g{};
  g.E = 1;
  g.M = (int)c.T;
  g.N = Epad;
  g.K = c.d;
  g.A = x;
  g.lda = c.d;
  g.B = wrT;
  g.ldb = c.d;
  g.C = zf;
  g.ldc = Epad;
  route_tile(c, g.bm, g.bn);
  const int ks = route_ksplit(c);
  g.ksplit = ks;
  g.c_kstride = c.T * (int64_t)Epad;
  rc = launch_gemm(MOE_KERNEL_ROUTE_LOGITS, MODE_ROW, true, EPI_F32, c, g, s);
  if (rc != MOE_OK) return rc;
  const float tau = c.route_margin > 0.0f ? c.route_margin : 1e-3f;
  // four tokens per wave, sixteen per block
  const int grid = (int)std::min<int64_t>(ceil_div(c.T, 16), 16384);
#define MOE_ROUTE_SELECT(V)                                                                 \
  MOE_LAUNCH(MOE_KERNEL_ROUTE, s,                                                           \
             route_kernel<V><<<grid, 256, 0, s>>>(zf, ks, b, probs, idx, gate, wl.count,     \
                                                  wl.tok, wl.n, wl.e, c.T, c.E, Epad, c.k, tau, \
                                                  renorm))
  if (Epad == 32)
    MOE_ROUTE_SELECT(2);
  else if (Epad == 64)
    MOE_ROUTE_SELECT(4);
  else if (Epad == 128)
    MOE_ROUTE_SELECT(8);
  else
    MOE_ROUTE_SELECT(16);
#undef MOE_ROUTE_SELECT
  const int rgrid = (int)std::min<int64_t>(ceil_div(c.T, 4), 2048);
  MOE_LAUNCH(MOE_KERNEL_ROUTE, s,
             route_rescore_kernel<T><<<rgrid, 256, 0, s>>>(
                 wl.count, wl.tok, wl.n, wl.e, x, wrT, b, probs, idx, gate, c.d, c.E,
                 Epad, c.k, renorm));
  return MOE_OK;
}

}  // namespace

int launch_transpose_wr(const moe_cfg& c, const void* Wr, void* wrT, int* wl_count,
                        hipStream_t s) {
  const int Epad = route_epad(c.E);
  const int64_t n = (int64_t)Epad * c.d;
  const int tgrid = (int)std::min<int64_t>(ceil_div(n, 256), 4096);
  if (c.dtype == MOE_BF16)
    MOE_LAUNCH(MOE_KERNEL_ROUTE_PREP, s,
               transpose_wr_kernel<uint16_t><<<tgrid, 256, 0, s>>>(
                   static_cast<const uint16_t*>(Wr), static_cast<uint16_t*>(wrT), c.d, c.E,
                   Epad, wl_count));
  else
    MOE_LAUNCH(MOE_KERNEL_ROUTE_PREP, s,
               transpose_wr_kernel<float><<<tgrid, 256, 0, s>>>(
                   static_cast<const float*>(Wr), static_cast<float*>(wrT), c.d, c.E, Epad,
                   wl_count));
  return MOE_OK;
}

int launch_route(const moe_cfg& c, const void* x, const void* Wr, const float* b,
                 float* probs, int32_t* idx, float* gate, void* ws, hipStream_t s) {
  if (c.T == 0) return MOE_OK;
  const WsLayout L = ws_layout(c);
  RouteWorklist wl;
  wl.count = ws_ptr<int>(ws, L.wl_count);
  wl.tok = ws_ptr<int>(ws, L.wl_tok);
  wl.n = ws_ptr<int>(ws, L.wl_n);
  wl.e = ws_ptr<int>(ws, L.wl_e);
  float* zf = ws_ptr<float>(ws, L.zf);
  if (c.dtype == MOE_FP32)
    return launch_route_t<float>(c, static_cast<const float*>(x), static_cast<const float*>(Wr), b,
                           probs, idx, gate, ws_ptr<float>(ws, L.wrT), zf, wl, s);
  return launch_route_t<uint16_t>(c, static_cast<const uint16_t*>(x),
                            static_cast<const uint16_t*>(Wr), b, probs, idx, gate,
                            ws_ptr<uint16_t>(ws, L.wrT), zf, wl, s);
}

}  // namespace moe
