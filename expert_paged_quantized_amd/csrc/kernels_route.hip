// Routing kernels of the MoE layer for gfx950: router logits in one fixed fp32
// summation order, top-k selection with routing weights, and the grouping of
// tokens by expert (counts, offsets, permutation, inverse positions, tile list).
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
  for (int o = 32; o >= 1; o >>= 1) {
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
      for (int b = 0; b < TE; ++b) acc[a][b] = acc[a][b] + __shfl_down(acc[a][b], o, 64);
  }
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
// Top-k + routing weights: one wave per token.  Selection is by (logit
// descending, expert id ascending) with IEEE comparison, so -0 and +0 tie.
// Weights: softmax over the selected logits, exp(l_j - l_0) / sum, or
// sigmoid(l_j) / sum of the selected sigmoids; the sum runs j = 0..k-1.
// ---------------------------------------------------------------------------
constexpr int kTopkMaxPerLane = 16;  // E <= 1024

__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int router, int32_t* __restrict__ idx,
                                                   float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float vals[kTopkMaxPerLane];
#pragma unroll
  for (int j = 0; j < kTopkMaxPerLane; ++j) {
    const int e = lane + 64 * j;
    vals[j] = (e < E) ? logits[(size_t)t * E + e] : -INFINITY;
  }
  uint32_t taken = 0;
  float my_v = 0.0f;
  int my_e = 0;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < kTopkMaxPerLane; ++j) {
      const int e = lane + 64 * j;
      if (e < E && !((taken >> j) & 1u)) {
        const float v = vals[j];
        if (v > bv || (v == bv && e < be)) {
          bv = v;
          be = e;
        }
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (ov > bv || (ov == bv && oe < be)) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & 63) == lane) taken |= 1u << (be >> 6);
    if (lane == r) {
      my_v = bv;
      my_e = be;
    }
  }
  const float v0 = __shfl(my_v, 0, 64);
  float z = 0.0f;
  if (lane < k) z = (router == R_SOFTMAX) ? __expf(my_v - v0) : 1.0f / (1.0f + __expf(-my_v));
  float sum = 0.0f;
  for (int j = 0; j < k; ++j) sum += __shfl(z, j, 64);
  if (lane < k) {
    idx[(size_t)t * k + lane] = my_e;
    w[(size_t)t * k + lane] = z / sum;
  }
}

// ---------------------------------------------------------------------------
// Permute: a single 1024-thread workgroup.
//   counts[e]    LDS histogram of idx (integer atomics: order-free)
//   offsets      exclusive prefix sum over experts
//   perm, pos    stable ranks: token t's entry for expert e lands at
//                offsets[e] + #{t' < t : e in idx[t']}.  Tokens are swept in
//                chunks of NW*64; in a chunk every wave sets bit `lane` of a
//                64-bit LDS mask per expert, and the rank is the running count
//                of earlier chunks + popcounts of earlier waves' masks + the
//                popcount of lower lanes in the own mask.
//   shared rows  perm[T*k + t] = t for the shared expert
//   tiles        per expert ceil(count / tile_rows) tiles in ascending expert
//                id, then the shared expert's tiles; slot = expert id (this
//                list serves the all-resident case).
// ---------------------------------------------------------------------------
constexpr int kPermThreads = 1024;
constexpr int kPermMaxE = 1024;
constexpr int kPermMaskWords = 4096;  // NW * E <= 4096 64-bit masks (32 KB)

__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(inc, o, 64);
    if (lane >= o) inc += n;
  }
  if (lane == 63) wave_tot[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int nw = kPermThreads / 64;
    int s = (lane < nw) ? wave_tot[lane] : 0;
    int si = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int n = __shfl_up(si, o, 64);
      if (lane >= o) si += n;
    }
    if (lane < nw) wave_tot[lane] = si - s;  // exclusive per wave
    if (lane == nw - 1) wave_tot[nw] = si;   // grand total
  }
  __syncthreads();
  const int r = inc - v + wave_tot[wave];
  total = wave_tot[kPermThreads / 64];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, int S, int tile_rows, int shared_slot,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ pos, Tile* __restrict__ tiles, int32_t* __restrict__ n_tiles,
    unsigned long long* __restrict__ distinct_total) {
  __shared__ int cnt[kPermMaxE];
  __shared__ int off[kPermMaxE + 1];
  __shared__ int run[kPermMaxE];
  __shared__ int toff[kPermMaxE + 1];
  __shared__ int wave_tot[kPermThreads / 64 + 1];
  __shared__ unsigned long long masks[kPermMaskWords];
  __shared__ int n_distinct;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < E) {
    cnt[tid] = 0;
    run[tid] = 0;
  }
  if (tid == 0) n_distinct = 0;
  __syncthreads();
  const int TK = T * k;
  for (int i = tid; i < TK; i += kPermThreads) atomicAdd(&cnt[idx[i]], 1);
  __syncthreads();
  const int c = (tid < E) ? cnt[tid] : 0;
  int total;
  const int o = block_exclusive_scan(c, wave_tot, total);
  const int nt = (c > 0) ? (c + tile_rows - 1) / tile_rows : 0;
  int ntot;
  const int to = block_exclusive_scan(nt, wave_tot, ntot);
  if (tid < E) {
    off[tid] = o;
    toff[tid] = to;
    counts[tid] = c;
    offsets[tid] = o;
    if (c > 0) atomicAdd(&n_distinct, 1);
  }
  if (tid == 0) {
    off[E] = total;
    toff[E] = ntot;
    offsets[E] = total;
  }
  __syncthreads();

  // stable ranks
  int nw = kPermMaskWords / E;
  nw = nw < 1 ? 1 : (nw > kPermThreads / 64 ? kPermThreads / 64 : nw);
  for (int base = 0; base < T; base += nw * 64) {
    for (int i = tid; i < nw * E; i += kPermThreads) masks[i] = 0ull;
    __syncthreads();
    const int t = base + wave * 64 + lane;
    const bool act = wave < nw && t < T;
    if (act)
      for (int j = 0; j < k; ++j) atomicOr(&masks[wave * E + idx[(size_t)t * k + j]], 1ull << lane);
    __syncthreads();
    if (act) {
      const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      for (int j = 0; j < k; ++j) {
        const int e = idx[(size_t)t * k + j];
        int r = run[e];
        for (int w2 = 0; w2 < wave; ++w2) r += __popcll(masks[w2 * E + e]);
        r += __popcll(masks[wave * E + e] & below);
        const int p = off[e] + r;
        perm[p] = t;
        pos[(size_t)t * k + j] = p;
      }
    }
    __syncthreads();
    if (tid < E) {
      int add = 0;
      for (int w2 = 0; w2 < nw; ++w2) add += __popcll(masks[w2 * E + tid]);
      run[tid] += add;
    }
    __syncthreads();
  }

  if (S)
    for (int t = tid; t < T; t += kPermThreads) perm[TK + t] = t;

  if (tid < E && c > 0) {
    for (int i = 0; i < nt; ++i) {
      Tile tl;
      tl.expert = tid;
      tl.slot = tid;
      tl.row_begin = o + i * tile_rows;
      tl.nrows = min(tile_rows, c - i * tile_rows);
      tl.group_first = to;
      tl.group_count = nt;
      tiles[to + i] = tl;
    }
  }
  const int nsh = S ? (T + tile_rows - 1) / tile_rows : 0;
  for (int i = tid; i < nsh; i += kPermThreads) {
    Tile tl;
    tl.expert = E;
    tl.slot = shared_slot;
    tl.row_begin = TK + i * tile_rows;
    tl.nrows = min(tile_rows, T - i * tile_rows);
    tl.group_first = ntot;
    tl.group_count = nsh;
    tiles[ntot + i] = tl;
  }
  if (tid == 0) {
    n_tiles[0] = ntot + nsh;
    distinct_total[0] += (unsigned long long)n_distinct;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_router(const uint16_t* x, const uint16_t* wr, const float* bias, float* logits,
                         uint16_t* x16, int T, int E, int H, hipStream_t s) {
  if (T <= 8) {
    const int waves = T * E;
    router_logits_kernel<1, 1><<<(waves + 3) / 4, 256, 0, s>>>(x, wr, bias, logits, x16, T, E, H);
  } else {
    const int waves = ((T + 3) / 4) * ((E + 3) / 4);
    router_logits_kernel<4, 4><<<(waves + 3) / 4, 256, 0, s>>>(x, wr, bias, logits, x16, T, E, H);
  }
  return hipGetLastError();
}

hipError_t launch_topk(const float* logits, int T, int E, int k, int router, int32_t* idx,
                       float* w, hipStream_t s) {
  topk_kernel<<<(T + 3) / 4, 256, 0, s>>>(logits, T, E, k, router, idx, w);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int S, int tile_rows,
                          int shared_slot, int32_t* counts, int32_t* offsets, int32_t* perm,
                          int32_t* pos, Tile* tiles, int32_t* n_tiles,
                          unsigned long long* distinct_total, hipStream_t s) {
  permute_kernel<<<1, kPermThreads, 0, s>>>(idx, T, k, E, S, tile_rows, shared_slot, counts,
                                            offsets, perm, pos, tiles, n_tiles, distinct_total);
  return hipGetLastError();
}

}  // namespace strata
