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
// reproducible bit for bit.  wr has E rows: the Eo routed experts' rows, then,
// for a layer with a shared-expert gate, the gate row, whose fp32 logit goes
// to gate_out[t] (no bias).
//
// When x16 is given (int4 and NVFP4 layers, whose expert GEMMs take fp16
// operands) the waves also write each token's row scaled into the fp16 range:
// x * 2^-e with e = floor(log2 max|x|) - 14, so the row's largest magnitude
// lands in [2^14, 2^15) whatever the bf16 input (bf16 reaches 2^128, fp16
// only 65504), and e goes to xexp[t] for the GEMM epilogues to undo in fp32.
// Every wave of a token block tracks the rows' largest magnitudes while it
// streams them for its logits, then converts its own share of the rows'
// 16-byte pieces (the wave of expert block b takes pieces b, b + nb, ...), so
// no wave pays a whole extra pass.  The scaling is exact except for elements
// below 2^-32 of the row's largest, which round to fp16's 2^-24 grid.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Running max of the magnitudes of a word of two bf16 values, compared as
// their 15-bit magnitude patterns (for non-negative floats the bit order is
// the numeric order).
__device__ __forceinline__ uint32_t amax_bits(uint32_t am, uint32_t w) {
  return max(am, max(w & 0x7fffu, (w >> 16) & 0x7fffu));
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
  return v;
}
// floor(log2 of the magnitude with bf16 bits `am`) - 14; 0 for a zero row.
// Exponent field 0 is a subnormal m * 2^-133.
__device__ __forceinline__ int token_exponent(uint32_t am) {
  if (am == 0) return 0;
  const int ef = (int)(am >> 7);
  const int fl = ef ? ef - 127 : (31 - __clz(am)) - 133;
  return fl - 14;
}
// Two bf16 values times 2^ne (exact in fp32), rounded to fp16 (nearest-even).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2_scaled(uint32_t w, int ne) {
  const _Float16 lo = (_Float16)__builtin_amdgcn_ldexpf(bf16_lo(w), ne);
  const _Float16 hi = (_Float16)__builtin_amdgcn_ldexpf(bf16_hi(w), ne);
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}
// The scaled fp16 copy of tokens t0 .. t0 + NT - 1 (< T): from the rows'
// running magnitude maxima (per lane), this wave (share `part` of `nparts`)
// converts the 16-byte pieces part, part + nparts, ... of the NT rows; share
// 0 also writes the exponents.
template <int NT>
__device__ __forceinline__ void write_scaled_rows(const uint16_t* __restrict__ x, uint16_t* __restrict__ x16,
                                                  int32_t* __restrict__ xexp, const uint32_t (&am)[NT], int t0,
                                                  int T, int H, int lane, int part, int nparts) {
  int ex[NT];
#pragma unroll
  for (int a = 0; a < NT; ++a) ex[a] = token_exponent(wave_max(am[a]));
  const int pieces = NT * (H >> 3);  // 8 values per piece
  for (int q = part + nparts * lane; q < pieces; q += nparts * 64) {
    const int a = q / (H >> 3), off = (q - a * (H >> 3)) * 8;
    if (t0 + a >= T) continue;
    int e = ex[0];
#pragma unroll
    for (int i = 1; i < NT; ++i) e = (a == i) ? ex[i] : e;
    const uint4 xv = *reinterpret_cast<const uint4*>(x + (size_t)(t0 + a) * H + off);
    uint4 hv;
#pragma unroll
    for (int w = 0; w < 4; ++w) (&hv.x)[w] = bf16x2_to_f16x2_scaled((&xv.x)[w], -e);
    *reinterpret_cast<uint4*>(x16 + (size_t)(t0 + a) * H + off) = hv;
  }
  if (part == 0 && lane == 0) {
#pragma unroll
    for (int a = 0; a < NT; ++a)
      if (t0 + a < T) xexp[t0 + a] = ex[a];
  }
}

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

// One wave's TT x TE logits (wave index `wave` of the launch).  COHERENT:
// the logits are stored at device scope (through to memory), for a
// workgroup of the same launch on another XCD to read them.
template <int TT, int TE, bool COHERENT>
__device__ __forceinline__ void router_logits_wave(int wave, const uint16_t* __restrict__ x,
                                                   const uint16_t* __restrict__ wr,
                                                   const float* __restrict__ bias,
                                                   float* __restrict__ logits, uint16_t* __restrict__ x16,
                                                   int32_t* __restrict__ xexp, float* __restrict__ gate_out,
                                                   int T, int E, int Eo, int H) {
  const int lane = threadIdx.x & 63;
  const int neb = (E + TE - 1) / TE;
  const int t0 = (wave / neb) * TT, e0 = (wave % neb) * TE;
  if (t0 >= T) return;
  const bool copy = x16 != nullptr;  // the waves write the scaled fp16 rows
  uint32_t am[TT];
  float acc[TT][TE];
#pragma unroll
  for (int a = 0; a < TT; ++a) {
    am[a] = 0;
#pragma unroll
    for (int b = 0; b < TE; ++b) acc[a][b] = 0.0f;
  }
  const int C = H >> 9;
  // Chunks in rounds of up to four (H is a multiple of 512): a round's loads
  // are all issued before its first multiply waits; the sums still run chunk
  // by chunk, in order.  Loads past C re-read chunk C - 1 and are not used.
  constexpr int RC = 4;
  for (int c0 = 0; c0 < C; c0 += RC) {
    uint4 xv[RC][TT], wv[RC][TE];
#pragma unroll
    for (int u = 0; u < RC; ++u) {
      const int off = (min(c0 + u, C - 1) * 64 + lane) * 8;
#pragma unroll
      for (int a = 0; a < TT; ++a) {
        const int t = min(t0 + a, T - 1);
        xv[u][a] = *reinterpret_cast<const uint4*>(x + (size_t)t * H + off);
      }
#pragma unroll
      for (int b = 0; b < TE; ++b) {
        const int e = min(e0 + b, E - 1);
        wv[u][b] = *reinterpret_cast<const uint4*>(wr + (size_t)e * H + off);
      }
    }
#pragma unroll
    for (int u = 0; u < RC; ++u) {
      if (c0 + u >= C) break;
      if (copy) {
#pragma unroll
        for (int a = 0; a < TT; ++a)
#pragma unroll
          for (int q = 0; q < 4; ++q) am[a] = amax_bits(am[a], (&xv[u][a].x)[q]);
      }
#pragma unroll
      for (int v = 0; v < 8; ++v) {
#pragma unroll
        for (int a = 0; a < TT; ++a) {
          const uint32_t xw = (&xv[u][a].x)[v >> 1];
          const float xf = (v & 1) ? bf16_hi(xw) : bf16_lo(xw);
#pragma unroll
          for (int b = 0; b < TE; ++b) {
            const uint32_t ww = (&wv[u][b].x)[v >> 1];
            const float wf = (v & 1) ? bf16_hi(ww) : bf16_lo(ww);
            acc[a][b] = __builtin_fmaf(xf, wf, acc[a][b]);
          }
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
        if (t < T && e < Eo) {
          const float l = bias ? acc[a][b] + bias[e] : acc[a][b];
          if constexpr (COHERENT)
            __hip_atomic_store(&logits[(size_t)t * Eo + e], l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          else
            logits[(size_t)t * Eo + e] = l;
        } else if (t < T && e < E) {
          gate_out[t] = acc[a][b];  // the shared-expert gate row
        }
      }
  }
  if (copy) write_scaled_rows<TT>(x, x16, xexp, am, t0, T, H, lane, wave % neb, neb);
}

template <int TT, int TE>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            float* __restrict__ logits,
                                                            uint16_t* __restrict__ x16,
                                                            int32_t* __restrict__ xexp,
                                                            float* __restrict__ gate_out, int T, int E,
                                                            int Eo, int H) {
  router_logits_wave<TT, TE, false>(blockIdx.x * 4 + (threadIdx.x >> 6), x, wr, bias, logits, x16, xexp, gate_out,
                                    T, E, Eo, H);
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
                                                          uint16_t* __restrict__ x16,
                                                          int32_t* __restrict__ xexp,
                                                          float* __restrict__ gate_out, int T, int E,
                                                          int Eo, int H) {
  __shared__ __attribute__((aligned(16))) float red[4][64 * kRbPitch];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wave = blockIdx.x * 4 + w;
  const int neb = (E + kRbTE - 1) / kRbTE;
  const int t0 = (wave / neb) * kRbTT, e0 = (wave % neb) * kRbTE;
  const bool active = t0 < T;
  const bool copy = active && x16;  // the waves write the scaled fp16 rows
  uint32_t am[kRbTT];
  float acc[kRbTT][kRbTE];
#pragma unroll
  for (int a = 0; a < kRbTT; ++a) {
    am[a] = 0;
#pragma unroll
    for (int b = 0; b < kRbTE; ++b) acc[a][b] = 0.0f;
  }
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
    if (copy) {
#pragma unroll
      for (int a = 0; a < kRbTT; ++a)
#pragma unroll
        for (int q = 0; q < 4; ++q) am[a] = amax_bits(am[a], (&xv[a].x)[q]);
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
  if (active && t < T && e < Eo) logits[(size_t)t * Eo + e] = bias ? q[0] + bias[e] : q[0];
  else if (active && t < T && e < E) gate_out[t] = q[0];  // the shared-expert gate row
  if (copy) write_scaled_rows<kRbTT>(x, x16, xexp, am, t0, T, H, lane, wave % neb, neb);
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
// COHERENT: the logits were stored at device scope by other workgroups of
// the same launch and are loaded at device scope (from memory, not from a
// possibly stale line of this XCD's L2).
template <bool COHERENT>
__device__ __forceinline__ float load_logit(const float* p) {
  if constexpr (COHERENT)
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    return *p;
}

// taken_out (optional): bit j of lane l set when expert l + 64 j was picked.
template <int JPL, bool COHERENT = false>
__device__ __forceinline__ void topk_token(const float* __restrict__ logits, int t, int E, int k,
                                           int lane, float& my_v, int& my_e, uint32_t* taken_out = nullptr) {
  float vals[JPL];
#pragma unroll
  for (int j = 0; j < JPL; ++j) {
    const int e = lane + 64 * j;
    const float v = load_logit<COHERENT>(&logits[(size_t)t * E + min(e, E - 1)]);
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
  if (taken_out) *taken_out = taken;
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

// exclusive scan over up to 1024 values held one per thread of a 1024-thread
// workgroup; returns the thread's prefix and the total
// inclusive prefix sum over the wave: row shifts 1, 2, 4, 8 inside each
// 16-lane row (lanes shifted in from outside the row add 0), then the row
// totals broadcast forward (lane 15 into row 1, 47 into row 3; lane 31 into
// rows 2 and 3)
template <int CTRL, int ROWS, int BANKS>
__device__ __forceinline__ int dpp_add(int v) {
  return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, BANKS, true);
}
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  v = dpp_add<0x111, 0xf, 0xf>(v);  // row_shr:1
  v = dpp_add<0x112, 0xf, 0xf>(v);  // row_shr:2
  v = dpp_add<0x114, 0xf, 0xf>(v);  // row_shr:4
  v = dpp_add<0x118, 0xf, 0xf>(v);  // row_shr:8
  v = dpp_add<0x142, 0xa, 0xf>(v);  // row_bcast:15
  v = dpp_add<0x143, 0xc, 0xf>(v);  // row_bcast:31
  return v;
}

__device__ __forceinline__ int block_scan1024(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_inclusive_scan(v);
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
// pre_used (>= 0 only with one tile per expert): this thread's exclusive
// prefix of used experts and, in pre_total, their number, when the caller
// has scanned them already (then nt = used and both scans below are that one).
__device__ __forceinline__ void emit_counts_and_tiles(int c, int o, int total, int T, int k, int E,
                                                      int S, int tile_rows, int shared_slot,
                                                      int* wave_tot, int32_t* counts,
                                                      int32_t* offsets, Tile* tiles,
                                                      int32_t* n_tiles,
                                                      unsigned long long* distinct_total,
                                                      int pre_used = -1, int pre_total = 0) {
  const int e = threadIdx.x;
  const bool used = e < E && c > 0;
  const int nt = used ? (c + tile_rows - 1) / tile_rows : 0;
  const int TK = T * k;
  const int nsh = S ? (T + tile_rows - 1) / tile_rows : 0;
  int ntot, nd_tot, to;
  if (pre_used >= 0) {
    to = pre_used;
    ntot = nd_tot = pre_total;
  } else {
    to = block_scan1024(nt, wave_tot, ntot);
    (void)block_scan1024(used ? 1 : 0, wave_tot, nd_tot);
  }
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
  } else if (tile_rows < 32) {  // decode: tiles of at most tile_rows rows, by expert
    if (used)
      for (int j = 0; j < nt; ++j)
        put(nsh + to + j, e, e, o + j * tile_rows, min(tile_rows, c - j * tile_rows), nsh + to, nt);
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
// Small batches search each token's k-th largest key in one wave
// (topk_by_threshold), token t in wave t.
// One token's grouping in one wave (route_one_token) when its top-k takes at
// most this many (pick, logit-per-lane) steps (top-2 of 8 experts: ~0.9 us
// sooner than the workgroup path).
constexpr int kOneWaveSteps = 4;  // largest k * JPL

// Selection key of a logit of expert e: larger is better.  The fp32 order
// (with -0 == +0: adding +0 maps -0 to +0) in the high word, the complement
// of the id in the low word, so equal logits rank the lower id first.
__device__ __forceinline__ uint64_t select_key(float l, int e) {
  const uint32_t u = __float_as_uint(l + 0.0f);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)~(uint32_t)e;
}

// One token with one tile per expert (a one-token decode forward): the whole
// grouping in one wave, with no LDS and no workgroup barrier.  The picks are
// the one-wave top-k's (value descending, equal values to the lower id).
// With one token every picked expert holds exactly one row, so a pick's
// position in the expert-major grouping is the number of picks with a lower
// id, and counts, offsets, perm, pos and the tile list (the shared expert's
// tile, then one tile per picked expert by ascending id) follow from the k
// picks alone; they are the values the workgroup path below computes.
template <int JPL, bool COHERENT>
__device__ __forceinline__ void route_one_token(
    const float* __restrict__ logits, int E, int k, int router, int S, int shared_slot,
    int32_t* __restrict__ idx, float* __restrict__ w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ pos,
    Tile* __restrict__ tiles, int32_t* __restrict__ n_tiles, unsigned long long* __restrict__ distinct_total) {
  const int lane = threadIdx.x & 63;
  float my_v;
  int my_e;
  uint32_t taken;
  topk_token<JPL, COHERENT>(logits, 0, E, k, lane, my_v, my_e, &taken);
  const float wt = topk_weight(my_v, k, router, lane);
  // counts and offsets of experts lane + 64 j: the picks below an id are
  // those of the earlier 64-expert groups plus this group's lower lanes
  int below = 0;
#pragma unroll
  for (int j = 0; j < JPL; ++j) {
    const int e = lane + 64 * j;
    const int c = (taken >> j) & 1;
    const int inc = wave_inclusive_scan(c);
    if (e < E) {
      counts[e] = c;
      offsets[e] = below + inc - c;
    }
    below += __builtin_amdgcn_readlane(inc, 63);
  }
  int r = 0;  // pick `lane`'s position: the picks with a lower id
  for (int j = 0; j < k; ++j) r += __builtin_amdgcn_readlane(my_e, j) < my_e ? 1 : 0;
  const int nsh = S ? 1 : 0;
  if (lane < k) {
    idx[lane] = my_e;
    w[lane] = wt;
    perm[r] = 0;
    pos[lane] = r;
    Tile tl;
    tl.expert = my_e;
    tl.slot = my_e;
    tl.row_begin = r;
    tl.nrows = 1;
    tl.group_first = nsh + r;
    tl.group_count = 1;
    tiles[nsh + r] = tl;
  }
  if (lane == 0) {
    offsets[E] = k;
    if (S) {
      perm[k] = 0;
      Tile tl;
      tl.expert = E;
      tl.slot = shared_slot;
      tl.row_begin = k;
      tl.nrows = 1;
      tl.group_first = 0;
      tl.group_count = 1;
      tiles[0] = tl;
    }
    n_tiles[0] = k + nsh;
    atomicAdd(distinct_total, (unsigned long long)k);
  }
}

// Lanes r < k end with the r-th selected (logit, expert) of token t in
// select_key's order (value descending, -0 == +0, equal values to the lower
// id), found without k dependent rounds: a bitwise search for an fp32
// order o that at least k of the token's keys reach (one wave-wide ballot
// count per bit; the largest such o, unless exactly k reach one on the
// way), and, when more keys sit at o than are still needed, the same search
// over their ids; the k keys above that threshold
// are gathered in `lds` (k entries of this wave's own) and each is placed by
// counting the picks above it.  Slots past E hold order 0 and ids >= E, so
// they rank below every expert.
template <int JPL, bool COHERENT>
__device__ __forceinline__ void topk_by_threshold(const float* __restrict__ logits, int t, int E, int k,
                                                  int lane, float& my_v, int& my_e, uint64_t* lds) {
  constexpr int kIdBits = 6 + (JPL >= 2) + (JPL >= 4) + (JPL >= 8) + (JPL >= 16);  // ids < 64 * JPL
  uint32_t ord[JPL];
#pragma unroll
  for (int j = 0; j < JPL; ++j) {
    const int e = lane + 64 * j;
    const float v = load_logit<COHERENT>(&logits[(size_t)t * E + min(e, E - 1)]);
    ord[j] = (e < E) ? (uint32_t)(select_key(v, e) >> 32) : 0u;
  }
  // count(ord >= o) >= k holds throughout; once exactly k keys reach o they
  // are the top k (the next key lies below o), and the search stops there
  uint32_t o = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = o | (1u << b);
    int n = 0;
#pragma unroll
    for (int j = 0; j < JPL; ++j) n += __popcll(__ballot(ord[j] >= c));
    if (n >= k) {
      o = c;
      if (n == k) break;
    }
  }
  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int j = 0; j < JPL; ++j) {
    n_gt += __popcll(__ballot(ord[j] > o));
    n_eq += __popcll(__ballot(ord[j] == o));
  }
  const int need = k - n_gt;  // 1 .. n_eq keys at o, lowest ids first
  int x = 64 * JPL - 1;       // the largest id taken at o
  if (n_eq > need) {
    x = 0;  // the largest x with fewer than `need` keys at o below it
    for (int b = kIdBits - 1; b >= 0; --b) {
      const int c = x | (1 << b);
      int n = 0;
#pragma unroll
      for (int j = 0; j < JPL; ++j) n += __popcll(__ballot(ord[j] == o && lane + 64 * j < c));
      if (n < need) x = c;
    }
  }
  uint32_t pick = 0;
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < JPL; ++j) {
    const bool p = ord[j] > o || (ord[j] == o && lane + 64 * j <= x);
    pick |= (p ? 1u : 0u) << j;
    cnt += p ? 1 : 0;
  }
  int at = wave_inclusive_scan(cnt) - cnt;  // k picks in all
#pragma unroll
  for (int j = 0; j < JPL; ++j)
    if ((pick >> j) & 1u) lds[at++] = ((uint64_t)ord[j] << 32) | (uint32_t)~(uint32_t)(lane + 64 * j);
  __threadfence_block();
  __builtin_amdgcn_wave_barrier();
  const uint64_t key = lane < k ? lds[lane] : 0ull;
  int r = 0;  // picks above this one
  for (int j = 0; j < k; ++j) {
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(key >> 32), j);
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)key, j);
    r += (((uint64_t)hi << 32) | lo) > key ? 1 : 0;
  }
  if (lane < k) lds[r] = key;
  __threadfence_block();
  __builtin_amdgcn_wave_barrier();
  my_v = 0.0f;
  my_e = 0;
  if (lane < k) {
    const uint64_t q = lds[lane];
    const uint32_t oq = (uint32_t)(q >> 32);
    my_v = __uint_as_float((oq & 0x80000000u) ? (oq & 0x7fffffffu) : ~oq);
    my_e = (int)~(uint32_t)q;
  }
}

// Top-k and weights of a long batch: one wave per token, 4 tokens per
// workgroup; k rounds of one-wave picks when the top-k is short (at most
// kOneWaveSteps pick x logit-per-lane steps), else the threshold search.
template <int JPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int k, int router, int32_t* __restrict__ idx,
                                                   float* __restrict__ w) {
  __shared__ uint64_t sel[4 * 32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  float my_v;
  int my_e;
  if (k * JPL <= kOneWaveSteps)
    topk_token<JPL>(logits, t, E, k, lane, my_v, my_e);
  else
    topk_by_threshold<JPL, false>(logits, t, E, k, lane, my_v, my_e, sel + wave * 32);
  const float wt = topk_weight(my_v, k, router, lane);
  if (lane < k) {
    idx[(size_t)t * k + lane] = my_e;
    w[(size_t)t * k + lane] = wt;
  }
}

template <int JPL, bool COHERENT>
__device__ __forceinline__ void route_small_body(
    const float* __restrict__ logits, int T, int E, int k, int router, int S, int tile_rows,
    int shared_slot, int32_t* __restrict__ idx, float* __restrict__ w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ pos,
    Tile* __restrict__ tiles, int32_t* __restrict__ n_tiles,
    unsigned long long* __restrict__ distinct_total) {
  __shared__ unsigned int mask[kPermMaxE];  // bit = token (T <= 16)
  __shared__ int off[kPermMaxE];
  __shared__ int sel[kSmallT * 32];
  __shared__ uint64_t keys[kSmallT * 32];  // threshold search: 32 per token's wave
  __shared__ int wave_tot[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (T == 1 && tile_rows > kPrefillTM && k * JPL <= kOneWaveSteps) {
    if (wave == 0)
      route_one_token<JPL, COHERENT>(logits, E, k, router, S, shared_slot, idx, w, counts, offsets, perm, pos,
                                     tiles, n_tiles, distinct_total);
    return;
  }
  for (int e = tid; e < E; e += 1024) mask[e] = 0u;
  __syncthreads();
  if (wave < T) {
    float my_v;
    int my_e;
    topk_by_threshold<JPL, COHERENT>(logits, wave, E, k, lane, my_v, my_e, keys + wave * 32);
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
  int total, o, pre_used = -1, n_used = 0;
  if (tile_rows > kPrefillTM) {
    // one tile per expert: the offsets and the used-expert prefix in one
    // scan (counts in the low 16 bits: T * k <= 16 * 32; used in the high)
    int tot2;
    const int o2 = block_scan1024(c | ((c > 0 ? 1 : 0) << 16), wave_tot, tot2);
    o = o2 & 0xffff;
    pre_used = o2 >> 16;
    total = tot2 & 0xffff;
    n_used = tot2 >> 16;
  } else {
    o = block_scan1024(c, wave_tot, total);
  }
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
                        tiles, n_tiles, distinct_total, pre_used, n_used);
}

// ---------------------------------------------------------------------------
// Router and small-batch routing in one launch (T <= 16): 1024-thread
// workgroups whose first four waves each compute the logits of the router's
// one-logit-per-wave layout (so the launch spreads the router bytes over as
// many CUs as the four-wave router kernel does), stored at device scope.
// Each workgroup then counts itself in `arrive` (device scope, after its
// stores are acknowledged); the workgroup that arrives last resets the
// counter for the next launch and runs the whole routing on the logits,
// loaded at device scope.  No workgroup waits for another.
// ---------------------------------------------------------------------------
template <int JPL>
__global__ __launch_bounds__(1024) void route_decode_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, const float* __restrict__ bias,
    float* __restrict__ logits, uint16_t* __restrict__ x16, int32_t* __restrict__ xexp,
    float* __restrict__ gate_out, int Eall, int H, uint32_t* __restrict__ arrive, int T, int E, int k,
    int router, int S, int tile_rows, int shared_slot, int32_t* __restrict__ idx, float* __restrict__ w,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
    int32_t* __restrict__ pos, Tile* __restrict__ tiles, int32_t* __restrict__ n_tiles,
    unsigned long long* __restrict__ distinct_total) {
  __shared__ int is_last;
  const int wave = threadIdx.x >> 6;
  if (wave < 4)
    router_logits_wave<1, 1, true>(blockIdx.x * 4 + wave, x, wr, bias, logits, x16, xexp, gate_out, T, Eall, E,
                                   H);
  // the stores of this wave are acknowledged at device scope
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t n = __hip_atomic_fetch_add(arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    is_last = n + 1 == gridDim.x;
    if (is_last) __hip_atomic_store(arrive, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!is_last) return;
  route_small_body<JPL, true>(logits, T, E, k, router, S, tile_rows, shared_slot, idx, w, counts, offsets,
                              perm, pos, tiles, n_tiles, distinct_total);
}

template <int JPL>
__global__ __launch_bounds__(1024) void route_small_kernel(
    const float* __restrict__ logits, int T, int E, int k, int router, int S, int tile_rows,
    int shared_slot, int32_t* __restrict__ idx, float* __restrict__ w, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ pos,
    Tile* __restrict__ tiles, int32_t* __restrict__ n_tiles,
    unsigned long long* __restrict__ distinct_total) {
  route_small_body<JPL, false>(logits, T, E, k, router, S, tile_rows, shared_slot, idx, w, counts, offsets, perm,
                               pos, tiles, n_tiles, distinct_total);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_router(const uint16_t* x, const uint16_t* wr, const float* bias, float* logits,
                         uint16_t* x16, int32_t* xexp, float* gate_out, int T, int E, int Eo, int H,
                         hipStream_t s) {
  // 8 x 8 blocks when they still give the GPU thousands of waves, else one
  // logit per wave (small T or few experts)
  const int blocked_waves = ((T + kRbTT - 1) / kRbTT) * ((E + kRbTE - 1) / kRbTE);
  if (blocked_waves >= 2048) {
    launch_k(router_block_kernel, dim3((blocked_waves + 3) / 4), dim3(256), 0, s, x, wr, bias, logits, x16,
             xexp, gate_out, T, E, Eo, H);
  } else {
    const int waves = T * E;
    launch_k(router_logits_kernel<1, 1>, dim3((waves + 3) / 4), dim3(256), 0, s, x, wr, bias, logits, x16,
             xexp, gate_out, T, E, Eo, H);
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

template <int JPL>
static void launch_route_decode_jpl(const uint16_t* x, const uint16_t* wr, const float* bias, float* logits,
                                    uint16_t* x16, int32_t* xexp, float* gate_out, int Eall, int H,
                                    uint32_t* arrive, int T, int E, int k, int router, int S, int tile_rows,
                                    int shared_slot, int32_t* idx, float* w, int32_t* counts, int32_t* offsets,
                                    int32_t* perm, int32_t* pos, Tile* tiles, int32_t* n_tiles,
                                    unsigned long long* distinct_total, hipStream_t s) {
  const int waves = T * Eall;  // one logit per router wave, four router waves per workgroup
  launch_k(route_decode_kernel<JPL>, dim3((waves + 3) / 4), dim3(1024), 0, s, x, wr, bias, logits, x16, xexp,
           gate_out, Eall, H, arrive, T, E, k, router, S, tile_rows, shared_slot, idx, w, counts, offsets, perm,
           pos, tiles, n_tiles, distinct_total);
}

// The fused launch holds one 1024-thread workgroup per four logits; beyond
// 256 workgroups (T * E > 1024) the two launches take less time.
bool route_decode_fits(int T, int Eall) { return T >= 1 && T <= kSmallT && T * Eall <= 1024; }

hipError_t launch_route_decode(const uint16_t* x, const uint16_t* wr, const float* bias, float* logits,
                               uint16_t* x16, int32_t* xexp, float* gate_out, int Eall, int H, uint32_t* arrive,
                               int T, int E, int k, int router, int S, int tile_rows, int shared_slot,
                               int32_t* idx, float* w, int32_t* counts, int32_t* offsets, int32_t* perm,
                               int32_t* pos, Tile* tiles, int32_t* n_tiles, unsigned long long* distinct_total,
                               hipStream_t s) {
#define STRATA_RD(J)                                                                                        \
  launch_route_decode_jpl<J>(x, wr, bias, logits, x16, xexp, gate_out, Eall, H, arrive, T, E, k, router, S, \
                             tile_rows, shared_slot, idx, w, counts, offsets, perm, pos, tiles, n_tiles,     \
                             distinct_total, s)
  if (E <= 64)
    STRATA_RD(1);
  else if (E <= 128)
    STRATA_RD(2);
  else if (E <= 256)
    STRATA_RD(4);
  else if (E <= 512)
    STRATA_RD(8);
  else
    STRATA_RD(16);
#undef STRATA_RD
  return hipGetLastError();
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
