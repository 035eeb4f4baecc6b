// Routing kernels of the MoE layer for gfx950: router logits in one fixed fp32
// summation order, top-k selection with routing weights, and the grouping of
// tokens by expert (counts, offsets, permutation, inverse positions, tile list)
// in two multi-block passes that synchronise only at kernel boundaries.
//
// The routing semantics (top-k, softmax or sigmoid renormalised over the
// selected experts) come from the checkpoint and are never altered (ro99/strata
// README, list of enforced rules).  Grouping tokens by expert lets every
// selected expert's packed bytes stream once per forward, the per-layer
// read-once principle of the yibie/strata-mlx README ("What it is", prompts
// read a layer at a time).
#include "moe_common.h"

namespace strata {

// ---------------------------------------------------------------------------
// Router logits.  One wave computes a TT x TE block of logits.  Lane L owns
// inputs h = (c*64 + L)*8 + v (one 16-byte load of 8 bf16 per chunk c) and
// accumulates them in increasing (c, v) with a fused multiply-add starting
// from +0; the 64 lane partials are then folded with offsets 32, 16, 8, 4, 2,
// 1 (p[L] += p[L + o]) and lane 0 holds the logit; the bias is added last.
// That order is part of the layer's definition so that the top-k decision is
// reproducible bit for bit.  When x16 is given (int4 layers, whose expert
// GEMMs run in fp16) the waves of the first expert block also write the fp16
// copy of their token rows (bf16 -> fp16 is exact in the fp16 range).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// p[L] += p[L + o] for o = 32, 16 (cross-row lane permutes) then 8, 4, 2, 1
// (DPP row shifts inside 16-lane rows); lane 0 ends with the canonical sum.
template <int CTRL>
__device__ __forceinline__ float dpp_row_shl(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf,
                                                               0xf, true));
}
__device__ __forceinline__ float fold_to_lane0(float p) {
  p = p + __shfl_down(p, 32, 64);
  p = p + __shfl_down(p, 16, 64);
  p = p + dpp_row_shl<0x108>(p);
  p = p + dpp_row_shl<0x104>(p);
  p = p + dpp_row_shl<0x102>(p);
  p = p + dpp_row_shl<0x101>(p);
  return p;
}

template <int TT, int TE>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ logits,
                                                            uint16_t* __restrict__ x16, int T, int E,
                                                            int H) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int neb = (E + TE - 1) / TE;
  const int t0 = (wave / neb) * TT, e0 = (wave % neb) * TE;
  if (t0 >= T) return;
  float acc[TT][TE];
#pragma unroll
  for (int a = 0; a < TT; ++a)
#pragma unroll
    for (int b = 0; b < TE; ++b) acc[a][b] = 0.0f;
  const int C = H >> 9;
  for (int c = 0; c < C; ++c) {
    const int off = (c * 64 + lane) * 8;
    uint4 xv[TT], wv[TE];
#pragma unroll
    for (int a = 0; a < TT; ++a) {
      const int t = min(t0 + a, T - 1);
      xv[a] = *reinterpret_cast<const uint4*>(x + (size_t)t * H + off);
    }
#pragma unroll
    for (int b = 0; b < TE; ++b) {
      const int e = min(e0 + b, E - 1);
      wv[b] = *reinterpret_cast<const uint4*>(wr + (size_t)e * H + off);
    }
    if (x16 && e0 == 0) {
#pragma unroll
      for (int a = 0; a < TT; ++a) {
        if (t0 + a < T) {
          uint4 hv;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t w = (&xv[a].x)[q];
            const _Float16 lo = (_Float16)bf16_lo(w), hi = (_Float16)bf16_hi(w);
            (&hv.x)[q] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                         ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
          }
          *reinterpret_cast<uint4*>(x16 + (size_t)(t0 + a) * H + off) = hv;
        }
      }
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) {
#pragma unroll
      for (int a = 0; a < TT; ++a) {
        const uint32_t xw = (&xv[a].x)[v >> 1];
        const float xf = (v & 1) ? bf16_hi(xw) : bf16_lo(xw);
#pragma unroll
        for (int b = 0; b < TE; ++b) {
          const uint32_t ww = (&wv[b].x)[v >> 1];
          const float wf = (v & 1) ? bf16_hi(ww) : bf16_lo(ww);
          acc[a][b] = __builtin_fmaf(xf, wf, acc[a][b]);
        }
      }
    }
  }
#pragma unroll
  for (int a = 0; a < TT; ++a)
#pragma unroll
    for (int b = 0; b < TE; ++b) acc[a][b] = fold_to_lane0(acc[a][b]);
  if (lane == 0) {
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
      for (int b = 0; b < TE; ++b) {
        const int t = t0 + a, e = e0 + b;
        if (t < T && e < E) logits[(size_t)t * E + e] = bias ? acc[a][b] + bias[e] : acc[a][b];
      }
  }
}


// ---------------------------------------------------------------------------
// Router logits for many tokens: one wave computes an 8 x 8 block (64 logits).
// Each lane accumulates its inputs exactly as above; the 64 lane partials of
// every logit are then transposed through LDS so that lane j holds the 64
// partials of logit j and folds them in registers with the same pairing
// (q[i] += q[i + o] for o = 32..1), which costs 63 adds per lane for all 64
// logits instead of 64 cross-lane folds.
// ---------------------------------------------------------------------------
constexpr int kRbTT = 8, kRbTE = 8, kRbPitch = 68;

__global__ __launch_bounds__(256) void router_block_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr,
                                                          const float* __restrict__ bias,
                                                          float* __restrict__ logits,
                                                          uint16_t* __restrict__ x16, int T, int E,
                                                          int H) {
  __shared__ __attribute__((aligned(16))) float red[4][64 * kRbPitch];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wave = blockIdx.x * 4 + w;
  const int neb = (E + kRbTE - 1) / kRbTE;
  const int t0 = (wave / neb) * kRbTT, e0 = (wave % neb) * kRbTE;
  const bool active = t0 < T;
  float acc[kRbTT][kRbTE];
#pragma unroll
  for (int a = 0; a < kRbTT; ++a)
#pragma unroll
    for (int b = 0; b < kRbTE; ++b) acc[a][b] = 0.0f;
  const int C = H >> 9;
  for (int c = 0; c < C && active; ++c) {
    const int off = (c * 64 + lane) * 8;
    uint4 xv[kRbTT], wv[kRbTE];
#pragma unroll
    for (int a = 0; a < kRbTT; ++a)
      xv[a] = *reinterpret_cast<const uint4*>(x + (size_t)min(t0 + a, T - 1) * H + off);
#pragma unroll
    for (int b = 0; b < kRbTE; ++b)
      wv[b] = *reinterpret_cast<const uint4*>(wr + (size_t)min(e0 + b, E - 1) * H + off);
    if (x16 && e0 == 0) {
#pragma unroll
      for (int a = 0; a < kRbTT; ++a) {
        if (t0 + a < T) {
          uint4 hv;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t wd = (&xv[a].x)[q];
            const _Float16 lo = (_Float16)bf16_lo(wd), hi = (_Float16)bf16_hi(wd);
            (&hv.x)[q] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                         ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
          }
          *reinterpret_cast<uint4*>(x16 + (size_t)(t0 + a) * H + off) = hv;
        }
      }
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      float xf[kRbTT];
#pragma unroll
      for (int a = 0; a < kRbTT; ++a) {
        const uint32_t xw = (&xv[a].x)[v >> 1];
        xf[a] = (v & 1) ? bf16_hi(xw) : bf16_lo(xw);
      }
#pragma unroll
      for (int b = 0; b < kRbTE; ++b) {
        const uint32_t ww = (&wv[b].x)[v >> 1];
        const float wf = (v & 1) ? bf16_hi(ww) : bf16_lo(ww);
#pragma unroll
        for (int a = 0; a < kRbTT; ++a) acc[a][b] = __builtin_fmaf(xf[a], wf, acc[a][b]);
      }
    }
  }
  // transpose: partial of logit j = a*8 + b from lane L goes to red[j][L]
  float* rw = red[w];
#pragma unroll
  for (int a = 0; a < kRbTT; ++a)
#pragma unroll
    for (int b = 0; b < kRbTE; ++b) rw[(a * kRbTE + b) * kRbPitch + lane] = acc[a][b];
  __syncthreads();
  float q[64];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 v = *reinterpret_cast<const float4*>(&rw[lane * kRbPitch + 4 * i]);
    q[4 * i + 0] = v.x;
    q[4 * i + 1] = v.y;
    q[4 * i + 2] = v.z;
    q[4 * i + 3] = v.w;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
    for (int i = 0; i < o; ++i) q[i] = q[i] + q[i + o];
  const int t = t0 + lane / kRbTE, e = e0 + lane % kRbTE;
  if (active && t < T && e < E) logits[(size_t)t * E + e] = bias ? q[0] + bias[e] : q[0];
}

// ---------------------------------------------------------------------------
// Top-k + routing weights (one wave per token), and the first half of the
// grouping by expert.  Selection is by (logit descending, expert id ascending)
// with IEEE comparison, so -0 and +0 tie.  Weights: softmax over the selected
// logits, exp(l_j - l_0) / sum, or sigmoid(l_j) / sum of the selected
// sigmoids; the sum runs j = 0..k-1.  The rank pass takes tokens in blocks of
// 64: each selected (token, expert) sets the token's bit in a 64-bit LDS mask
// of that expert; the block writes its per-expert histogram and, for every
// entry, the number of earlier tokens of the block that chose the same expert
// (its rank inside the block).  Integer work only: independent of ordering.
// ---------------------------------------------------------------------------
constexpr int kPermMaxE = 1024;
constexpr int kRouteBlock = 64;      // tokens per routing block

template <int CTRL>
__device__ __forceinline__ int dpp_mov(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}
// keep the better of (v, e) and its partner lane's under the DPP pattern CTRL
__device__ __forceinline__ void best_of_impl(float& v, int& e, float ov, int oe) {
  if (ov > v || (ov == v && oe < e)) {
    v = ov;
    e = oe;
  }
}
#define best_of(v, e, CTRL)                                                               \
  best_of_impl(v, e, __builtin_bit_cast(float, dpp_mov<CTRL>(__builtin_bit_cast(int, v))), \
               dpp_mov<CTRL>(e))

// Lanes r < k end with the r-th selected (logit, expert) of token t.  JPL =
// logits per lane (E <= 64 * JPL); the per-round scan is branch-free.
template <int JPL>
__device__ __forceinline__ void topk_token(const float* __restrict__ logits, int t, int E, int k,
                                           int lane, float& my_v, int& my_e) {
  float vals[JPL];
#pragma unroll
  for (int j = 0; j < JPL; ++j) {
    const int e = lane + 64 * j;
    const float v = logits[(size_t)t * E + min(e, E - 1)];
    vals[j] = (e < E) ? v : -INFINITY;
  }
  uint32_t taken = 0;
  my_v = 0.0f;
  my_e = 0;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < JPL; ++j) {
      const int e = lane + 64 * j;
      const bool ok = (e < E) && !((taken >> j) & 1u);
      const float v = ok ? vals[j] : -INFINITY;
      const int ee = ok ? e : 0x7fffffff;
      const bool better = v > bv || (v == bv && ee < be);
      bv = better ? v : bv;
      be = better ? ee : be;
    }
    // (value desc, id asc) is a strict total order, so any reduction tree
    // finds the same winner: quad swaps, half-row and row mirrors (DPP) give
    // every lane its row's best, then the four rows are compared.
    best_of(bv, be, 0xB1);   // lanes xor 1
    best_of(bv, be, 0x4E);   // lanes xor 2
    best_of(bv, be, 0x141);  // half-row mirror
    best_of(bv, be, 0x140);  // row mirror
    float cv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), 0));
    int ce = __builtin_amdgcn_readlane(be, 0);
#pragma unroll
    for (int row = 1; row < 4; ++row) {
      const float ov =
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), row * 16));
      const int oe = __builtin_amdgcn_readlane(be, row * 16);
      if (ov > cv || (ov == cv && oe < ce)) {
        cv = ov;
        ce = oe;
      }
    }
    if ((ce & 63) == lane) taken |= 1u << (ce >> 6);
    if (lane == r) {
      my_v = cv;
      my_e = ce;
    }
  }
}

// Weights of one token from its selected logits (lanes r < k hold pick r).
__device__ __forceinline__ float topk_weight(float my_v, int k, int router, int lane) {
  const float v0 = __shfl(my_v, 0, 64);
  float z = 0.0f;
  if (lane < k) z = (router == R_SOFTMAX) ? __expf(my_v - v0) : 1.0f / (1.0f + __expf(-my_v));
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum += __shfl(z, j, 64);
  return z / sum;
}

// one wave per token, 4 tokens per workgroup
template <int JPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int router, int32_t* __restrict__ idx,
                                                   float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float my_v;
  int my_e;
  topk_token<JPL>(logits, t, E, k, lane, my_v, my_e);
  const float wt = topk_weight(my_v, k, router, lane);
  if (lane < k) {
    idx[(size_t)t * k + lane] = my_e;
    w[(size_t)t * k + lane] = wt;
  }
}

// exclusive scan over up to 1024 values held one per thread of a 1024-thread
// workgroup; returns the thread's prefix and the total
__device__ __forceinline__ int block_scan1024(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(inc, o, 64);
    if (lane >= o) inc += n;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  int wbase = 0, tot = 0;
#pragma unroll
  for (int w2 = 0; w2 < 16; ++w2) {
    const int x = wave_tot[w2];
    if (w2 < wave) wbase += x;
    tot += x;
  }
  total = tot;
  __syncthreads();
  return wbase + inc - v;
}

// Writes counts, offsets, the tile list (ascending expert, then the shared
// expert) and the distinct-expert counter from per-expert totals held one per
// thread of a 1024-thread workgroup (E <= 1024).
// Tiles are emitted heaviest first so that persistent workgroups, which take
// items in list order, finish together: the shared expert's tiles (all T rows,
// mostly full), then the routed tiles grouped by their number of 32-row column
// tiles (4, 3, 2, 1), experts ascending inside a group.  Tiles cover disjoint
// rows, so their order changes no result.  With one tile per expert (decode)
// the order is simply by expert.
__device__ __forceinline__ void emit_counts_and_tiles(int c, int o, int total, int T, int k, int E,
                                                      int S, int tile_rows, int shared_slot,
                                                      int* wave_tot, int32_t* counts,
                                                      int32_t* offsets, Tile* tiles,
                                                      int32_t* n_tiles,
                                                      unsigned long long* distinct_total) {
  const int e = threadIdx.x;
  const bool used = e < E && c > 0;
  const int nt = used ? (c + tile_rows - 1) / tile_rows : 0;
  const int TK = T * k;
  const int nsh = S ? (T + tile_rows - 1) / tile_rows : 0;
  int ntot;
  const int to = block_scan1024(nt, wave_tot, ntot);
  int nd_tot;
  (void)block_scan1024(used ? 1 : 0, wave_tot, nd_tot);
  auto put = [&](int at, int ex, int slot, int row_begin, int nrows, int first, int count) {
    Tile tl;
    tl.expert = ex;
    tl.slot = slot;
    tl.row_begin = row_begin;
    tl.nrows = nrows;
    tl.group_first = first;
    tl.group_count = count;
    tiles[at] = tl;
  };
  for (int i = e; i < nsh; i += 1024)
    put(i, E, shared_slot, TK + i * tile_rows, min(tile_rows, T - i * tile_rows), 0, nsh);
  if (tile_rows > kPrefillTM) {  // one tile per expert
    if (used) put(nsh + to, e, e, o, c, nsh + to, 1);
  } else {
    // column tiles of each tile: full tiles have tile_rows / 32, the last one
    // ceil(rem / 32); group g = column tiles, g = 4 first
    const int full = c / tile_rows, rem = c - full * tile_rows;
    const int last_g = rem ? (rem + 31) / 32 : 0;
    const int gfull = tile_rows / 32;
    int base = nsh;
    for (int g = gfull; g >= 1; --g) {
      const int mine = (g == gfull ? full : 0) + (last_g == g ? 1 : 0);
      int tot;
      const int at = block_scan1024(used ? mine : 0, wave_tot, tot);
      if (used && mine > 0) {
        int j = 0;
        if (g == gfull)
          for (; j < full; ++j) put(base + at + j, e, e, o + j * tile_rows, tile_rows, base + at, mine);
        if (last_g == g) put(base + at + j, e, e, o + full * tile_rows, rem, base + at, mine);
      }
      base += tot;
    }
  }
  if (e < E) {
    counts[e] = c;
    offsets[e] = o;
  }
  if (e == 0) {
    offsets[E] = total;
    n_tiles[0] = ntot + nsh;
    atomicAdd(distinct_total, (unsigned long long)nd_tot);  // no return value: nothing waits for it
  }
}

// Per 64-token block: histogram over experts and each entry's rank inside the
// block, from 64-bit LDS masks (bit = token of the block).
__global__ __launch_bounds__(1024) void rank_kernel(const int32_t* __restrict__ idx, int T, int E, int k,
                                                    int32_t* __restrict__ rank_in_block,
                                                    int32_t* __restrict__ hist) {
  __shared__ unsigned long long mask[kPermMaxE];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += 1024) mask[e] = 0ull;
  __syncthreads();
  const int tb = blockIdx.x * kRouteBlock;
  const int n = min(kRouteBlock, T - tb) * k;
  for (int i = tid; i < n; i += 1024) atomicOr(&mask[idx[(size_t)tb * k + i]], 1ull << (i / k));
  __syncthreads();
  for (int e = tid; e < E; e += 1024) hist[(size_t)blockIdx.x * E + e] = __popcll(mask[e]);
  for (int i = tid; i < n; i += 1024) {
    const int tl = i / k;
    const unsigned long long below = (tl == 0) ? 0ull : (~0ull >> (64 - tl));
    rank_in_block[(size_t)tb * k + i] = __popcll(mask[idx[(size_t)tb * k + i]] & below);
  }
}

// ---------------------------------------------------------------------------
// Permute (one 1024-thread workgroup per block of 64 tokens).  Every workgroup
// reads all per-block histograms (G = 1024 / E threads per expert, each
// summing every G-th block) to get, per expert, its total and its entries in
// earlier blocks; a scan of the totals gives the expert offsets.  Token t's
// entry for expert e lands at offset[e] + entries of e in earlier blocks +
// its rank inside the block, i.e. tokens ascending inside each expert
// segment; pos is the inverse map.  Shared-expert rows are the identity after
// the routed rows.  Workgroup 0 also writes counts, offsets and the tile list.
// No workgroup waits for another: the histograms are complete when the pass
// starts.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void permute_kernel(const int32_t* __restrict__ idx,
                                                       const int32_t* __restrict__ rank_in_block,
                                                       const int32_t* __restrict__ hist, int T, int E,
                                                       int k, int S, int tile_rows, int shared_slot,
                                                       int32_t* __restrict__ counts,
                                                       int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ perm,
                                                       int32_t* __restrict__ pos, Tile* __restrict__ tiles,
                                                       int32_t* __restrict__ n_tiles,
                                                       unsigned long long* __restrict__ distinct_total) {
  __shared__ int tot_s[kPermMaxE];
  __shared__ int pre_s[kPermMaxE];
  __shared__ int wave_tot[16];
  const int tid = threadIdx.x, b = blockIdx.x, nb = gridDim.x;
  for (int e = tid; e < E; e += 1024) tot_s[e] = pre_s[e] = 0;
  __syncthreads();
  const int G = 1024 / E;  // E <= kPermMaxE = 1024
  if (tid < G * E) {
    const int e = tid % E, g = tid / E;
    int tot = 0, pre = 0;
    int bb = g;
    for (; bb + 3 * G < nb; bb += 4 * G) {
      const int h0 = hist[(size_t)bb * E + e], h1 = hist[(size_t)(bb + G) * E + e];
      const int h2 = hist[(size_t)(bb + 2 * G) * E + e], h3 = hist[(size_t)(bb + 3 * G) * E + e];
      tot += h0 + h1 + h2 + h3;
      pre += (bb < b ? h0 : 0) + (bb + G < b ? h1 : 0) + (bb + 2 * G < b ? h2 : 0) + (bb + 3 * G < b ? h3 : 0);
    }
    for (; bb < nb; bb += G) {
      const int h = hist[(size_t)bb * E + e];
      tot += h;
      pre += bb < b ? h : 0;
    }
    atomicAdd(&tot_s[e], tot);
    atomicAdd(&pre_s[e], pre);
  }
  __syncthreads();
  const int c = tid < E ? tot_s[tid] : 0;
  int total;
  const int o = block_scan1024(c, wave_tot, total);
  if (tid < E) pre_s[tid] += o;
  __syncthreads();
  const int tb = b * kRouteBlock;
  const int n = min(kRouteBlock, T - tb) * k;
  for (int i = tid; i < n; i += 1024) {
    const size_t q = (size_t)tb * k + i;
    const int p = pre_s[idx[q]] + rank_in_block[q];
    perm[p] = tb + i / k;
    pos[q] = p;
  }
  if (S && tid < min(kRouteBlock, T - tb)) perm[T * k + tb + tid] = tb + tid;
  if (b == 0)
    emit_counts_and_tiles(c, o, total, T, k, E, S, tile_rows, shared_slot, wave_tot, counts, offsets,
                          tiles, n_tiles, distinct_total);
}

// ---------------------------------------------------------------------------
// Whole routing of a small batch (T <= 16) in one 1024-thread workgroup: top-k
// (wave w takes token w), then the same masks, offsets, permutation and tile
// list as the multi-block passes.
// ---------------------------------------------------------------------------
constexpr int kSmallT = 16;

template <int JPL>
__global__ __launch_bounds__(1024) void route_small_kernel(
    const float* __restrict__ logits, int T, int E, int k, int router, int S, int tile_rows,
    int shared_slot, int32_t* __restrict__ idx, float* __restrict__ w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ pos,
    Tile* __restrict__ tiles, int32_t* __restrict__ n_tiles,
    unsigned long long* __restrict__ distinct_total) {
  __shared__ unsigned int mask[kPermMaxE];  // bit = token (T <= 16)
  __shared__ int off[kPermMaxE];
  __shared__ int sel[kSmallT * 32];
  __shared__ int wave_tot[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += 1024) mask[e] = 0u;
  __syncthreads();
  if (wave < T) {
    float my_v;
    int my_e;
    topk_token<JPL>(logits, wave, E, k, lane, my_v, my_e);
    const float wt = topk_weight(my_v, k, router, lane);
    if (lane < k) {
      idx[wave * k + lane] = my_e;
      w[wave * k + lane] = wt;
      sel[wave * k + lane] = my_e;
      atomicOr(&mask[my_e], 1u << wave);
    }
  }
  __syncthreads();
  const int c = (tid < E) ? __popc(mask[tid]) : 0;
  int total;
  const int o = block_scan1024(c, wave_tot, total);
  if (tid < E) off[tid] = o;
  __syncthreads();
  const int TK = T * k;
  for (int i = tid; i < TK; i += 1024) {
    const int t = i / k, e = sel[i];
    const int p = off[e] + __popc(mask[e] & ((1u << t) - 1u));
    perm[p] = t;
    pos[i] = p;
  }
  if (S && tid < T) perm[TK + tid] = tid;
  emit_counts_and_tiles(c, o, total, T, k, E, S, tile_rows, shared_slot, wave_tot, counts, offsets,
                        tiles, n_tiles, distinct_total);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_router(const uint16_t* x, const uint16_t* wr, const float* bias, float* logits,
                         uint16_t* x16, int T, int E, int H, hipStream_t s) {
  // 8 x 8 blocks when they still give the GPU thousands of waves, else one
  // logit per wave (small T or few experts)
  const int blocked_waves = ((T + kRbTT - 1) / kRbTT) * ((E + kRbTE - 1) / kRbTE);
  if (blocked_waves >= 2048) {
    launch_k(router_block_kernel, dim3((blocked_waves + 3) / 4), dim3(256), 0, s, x, wr, bias, logits, x16, T, E, H);
  } else {
    const int waves = T * E;
    launch_k(router_logits_kernel<1, 1>, dim3((waves + 3) / 4), dim3(256), 0, s, x, wr, bias, logits, x16, T, E, H);
  }
  return hipGetLastError();
}

template <int JPL>
static void launch_route_jpl(const float* logits, int T, int E, int k, int router, int S, int tile_rows,
                             int shared_slot, int32_t* idx, float* w, int32_t* rank_in_block,
                             int32_t* hist, int32_t* counts, int32_t* offsets,
                             int32_t* perm, int32_t* pos, Tile* tiles, int32_t* n_tiles,
                             unsigned long long* distinct_total, hipStream_t s) {
  if (T <= kSmallT) {
    route_small_kernel<JPL><<<1, 1024, 0, s>>>(logits, T, E, k, router, S, tile_rows, shared_slot, idx,
                                               w, counts, offsets, perm, pos, tiles, n_tiles,
                                               distinct_total);
    return;
  }
  const int nblk = (T + kRouteBlock - 1) / kRouteBlock;
  topk_kernel<JPL><<<(T + 3) / 4, 256, 0, s>>>(logits, T, E, k, router, idx, w);
  rank_kernel<<<nblk, 1024, 0, s>>>(idx, T, E, k, rank_in_block, hist);
  permute_kernel<<<nblk, 1024, 0, s>>>(idx, rank_in_block, hist, T, E, k, S, tile_rows, shared_slot, counts,
                                       offsets, perm, pos, tiles, n_tiles, distinct_total);
}

hipError_t launch_route(const float* logits, int T, int E, int k, int router, int S, int tile_rows,
                        int shared_slot, int32_t* idx, float* w, int32_t* rank_in_block, int32_t* hist,
                        int32_t* counts, int32_t* offsets, int32_t* perm,
                        int32_t* pos, Tile* tiles, int32_t* n_tiles, unsigned long long* distinct_total,
                        hipStream_t s) {
#define STRATA_ROUTE(J)                                                                             \
  launch_route_jpl<J>(logits, T, E, k, router, S, tile_rows, shared_slot, idx, w, rank_in_block, hist, \
                      counts, offsets, perm, pos, tiles, n_tiles, distinct_total, s)
  if (E <= 64)
    STRATA_ROUTE(1);
  else if (E <= 128)
    STRATA_ROUTE(2);
  else if (E <= 256)
    STRATA_ROUTE(4);
  else if (E <= 512)
    STRATA_ROUTE(8);
  else
    STRATA_ROUTE(16);
#undef STRATA_ROUTE
  return hipGetLastError();
}

}  // namespace strata
