// Expert kernels of the MoE layer for gfx950: grouped SwiGLU FFN computed
// straight from 4-bit packed weights on the MFMA units, and the weighted
// combine.
//
// Weights stay 4-bit in HBM and are decoded in registers into MFMA operands,
// never into a wider resident copy (ro99/strata README: precision paragraph,
// and the SM86 kernel paragraph, whose register-fed decode into matrix-core
// operands is the prior art here; its prepack into operand order is a pure
// byte permutation, as is the tile order used below).  One weight layout
// serves both the decode kernel (T <= 8 tokens, split-K over a workgroup's
// waves) and the prefill kernel (token tiles of 128 rows staged in LDS), as
// the same README does with one layout for M=1 decode and M=128 pages.
//
// MFMA used: v_mfma_f32_32x32x16_{f16,bf16}.  The weight tile is the A
// operand (32 output rows x 16 inputs), the tokens are the B operand (16
// inputs x 32 tokens); lane l holds A row l%32 / B column l%32 and inputs
// 8*(l/32)..+7 of the step; the accumulator holds 16 rows per lane: row
// (i/4)*8 + (l/32)*4 + i%4, column l%32.  Each lane's 16-byte code chunk holds
// inputs 32*(l/32)..+31 of its row, 8 per MFMA step, and the activations are
// read with the same mapping, so the reduction covers each input exactly once.
//
// int4 group-64 affine weights are decoded to fp16 (w = s*q + b, one fp16
// rounding; s and b are admitted only if exact in fp16) and the activations
// arrive as fp16 (the router kernel writes that copy of x; exact in range).
// MXFP4 weights are decoded to bf16 with the gfx950 scaled FP4 conversion
// (exact: an E2M1 value times a power of two).  Accumulation is fp32 throughout; nothing uses float atomics,
// so every expert's result depends only on its own rows and weights.
#include <type_traits>

#include "moe_common.h"

namespace strata {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <class To, class From>
__device__ __forceinline__ To bitcast(const From& f) {
  static_assert(sizeof(To) == sizeof(From), "size");
  return __builtin_bit_cast(To, f);
}

// Loads through global-address-space pointers: the expert records are reached
// through a pointer table, and a generic (flat) load would also count against
// the LDS wait counter, serialising weight prefetches with LDS reads.
typedef const __attribute__((address_space(1))) u32x4 g_u32x4;
typedef const __attribute__((address_space(1))) uint32_t g_u32;
typedef const __attribute__((address_space(1))) uint8_t g_u8;
__device__ __forceinline__ u32x4 ld16(const void* p) { return *(g_u32x4*)(p); }
__device__ __forceinline__ uint32_t ld4(const void* p) { return *(g_u32*)(p); }
__device__ __forceinline__ uint32_t ld1(const void* p) { return *(g_u8*)(p); }

// (a & b) | c in one instruction (the compiler splits it when b, c are literals)
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// One MFMA step (8 inputs) of a decoded int4 chunk: word `st` of the 16-byte
// chunk.  Nibble n of the word holds input k0 k2 k4 k6 k1 k3 k5 k7 (n = 0..7),
// so the low nibbles of bytes 0 and 2 are (k0, k1) and their high nibbles
// (k2, k3); after a shift by 8 the same masks give (k4, k5) and (k6, k7).  A
// low nibble OR 0x6400 is the fp16 1024 + q, a high nibble (bits 4..7) OR
// 0x5400 is the fp16 64 + q; subtracting 1024 or 64 gives q exactly and one
// fp16 fma gives s*q + b.
__device__ __forceinline__ u32x4 dequant_int4_step(uint32_t w, f16x2 s2, f16x2 b2) {
  const uint32_t m_lo = 0x000F000Fu, m_hi = 0x00F000F0u, mag_lo = 0x64006400u, mag_hi = 0x54005400u;
  const f16x2 k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
  const f16x2 k64 = {(_Float16)64.0f, (_Float16)64.0f};
  const uint32_t w8 = w >> 8;
  const f16x2 h0 = bitcast<f16x2>(and_or(w, m_lo, mag_lo)) - k1024;
  const f16x2 h1 = bitcast<f16x2>(and_or(w, m_hi, mag_hi)) - k64;
  const f16x2 h2 = bitcast<f16x2>(and_or(w8, m_lo, mag_lo)) - k1024;
  const f16x2 h3 = bitcast<f16x2>(and_or(w8, m_hi, mag_hi)) - k64;
  u32x4 a;
  a[0] = bitcast<uint32_t>(__builtin_elementwise_fma(h0, s2, b2));
  a[1] = bitcast<uint32_t>(__builtin_elementwise_fma(h1, s2, b2));
  a[2] = bitcast<uint32_t>(__builtin_elementwise_fma(h2, s2, b2));
  a[3] = bitcast<uint32_t>(__builtin_elementwise_fma(h3, s2, b2));
  return a;
}

__device__ __forceinline__ u32x4 dequant_fp4_step(uint32_t w, float scale) {
  u32x4 a;
  a[0] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  a[1] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  a[2] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  a[3] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return a;
}

// Per-chunk decode parameters: fp16 (scale, bias) pairs for int4, the fp32
// power of two for MXFP4.
template <int QF>
struct ChunkScale {
  f16x2 s2, b2;
  float scale;
  __device__ __forceinline__ explicit ChunkScale(uint32_t sc) {
    if constexpr (QF == Q_INT4) {
      const _Float16 s = (_Float16)__uint_as_float(sc << 16);
      const _Float16 b = (_Float16)__uint_as_float(sc & 0xffff0000u);
      s2 = f16x2{s, s};
      b2 = f16x2{b, b};
      scale = 0.0f;
    } else {
      scale = __uint_as_float(sc << 23);
    }
  }
  __device__ __forceinline__ u32x4 step(uint32_t w) const {
    if constexpr (QF == Q_INT4)
      return dequant_int4_step(w, s2, b2);
    else
      return dequant_fp4_step(w, scale);
  }
};

template <int QF>
__device__ __forceinline__ void dequant(const u32x4& c, uint32_t sc, u32x4 (&a)[4]) {
  const ChunkScale<QF> cs(sc);
#pragma unroll
  for (int st = 0; st < 4; ++st) a[st] = cs.step(c[st]);
}

template <int QF>
__device__ __forceinline__ f32x16 mfma(const u32x4& a, const u32x4& b, const f32x16& c) {
  if constexpr (QF == Q_INT4)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<f16x8>(a), bitcast<f16x8>(b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8>(a), bitcast<bf16x8>(b), c, 0, 0,
                                                   0);
}

// scale bytes per weight tile and the lane's offset inside it
template <int QF>
struct ScaleLayout {
  static constexpr int kTileBytes = (QF == Q_INT4) ? 128 : 64;
  __device__ static int lane_off(int lane) { return (QF == Q_INT4) ? (lane & 31) * 4 : lane; }
  __device__ static uint32_t load(const uint8_t* p) {
    if constexpr (QF == Q_INT4)
      return ld4(p);
    else
      return ld1(p);
  }
};

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

template <int QF>
__device__ __forceinline__ uint16_t to_h_elem(float f) {
  if constexpr (QF == Q_INT4)
    return bitcast<uint16_t>((_Float16)f);
  else
    return f32_to_bf16_rne(f);
}

// ---------------------------------------------------------------------------
// Decode kernel: one workgroup of 8 waves per (tile, 32-row weight tile).  The
// waves split the K-blocks of the row tile in contiguous ranges, each streams
// its 1 KB code chunks (plus scales) with up to 4 blocks in flight, the tokens
// (<= 8) read their activations straight from global memory, and the partial
// sums are added in LDS in wave order 0..7 before the epilogue.
// ---------------------------------------------------------------------------
constexpr int kDecWaves = 8;

template <int QF, bool GATE_UP>
__global__ __launch_bounds__(512) void moe_decode_kernel(GemmArgs p) {
  using SL = ScaleLayout<QF>;
  __shared__ float red[kDecWaves][kDecodeMaxT][32];
  const int nrt = p.N >> 5;
  const int tile_i = blockIdx.x / nrt, rt = blockIdx.x % nrt;
  const int n_tiles = p.n_tiles_dev ? p.n_tiles_dev[0] : p.n_tiles;
  if (tile_i >= n_tiles) return;
  const Tile t = p.tiles[tile_i];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int KB = p.K >> 6;
  const int kb0 = wave * KB / kDecWaves, kb1 = (wave + 1) * KB / kDecWaves;
  const uint8_t* rec = p.slot_ptr[t.slot];
  const uint8_t* codes = rec + p.off_codes + (int64_t)rt * KB * kTileCodeBytes + lane * 16;
  const uint8_t* scales = rec + p.off_scales + (int64_t)rt * KB * SL::kTileBytes + SL::lane_off(lane);
  const int m = lane & 31;
  const bool valid = m < t.nrows;
  int64_t arow = 0;
  if (valid) arow = p.gather ? p.gather[t.row_begin + m] : (t.row_begin + m);
  const uint16_t* act = reinterpret_cast<const uint16_t*>(p.act) + arow * p.K + 32 * (lane >> 5);

  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;

  for (int kb = kb0; kb < kb1; kb += 4) {
    const int nb = min(4, kb1 - kb);
    u32x4 wq[4], xa[4][4];
    uint32_t ws[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u < nb) {
        wq[u] = ld16(codes + (int64_t)(kb + u) * kTileCodeBytes);
        ws[u] = SL::load(scales + (int64_t)(kb + u) * SL::kTileBytes);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (u < nb && valid) v = ld16(act + (kb + u) * 64 + 8 * st);
        xa[u][st] = v;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (u < nb) {
        u32x4 a[4];
        dequant<QF>(wq[u], ws[u], a);
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          acc = mfma<QF>(a[st], xa[u][st], acc);
        }
      }
    }
  }

  if (valid && m < kDecodeMaxT) {
#pragma unroll
    for (int i = 0; i < 16; ++i) red[wave][m][(i >> 2) * 8 + (lane >> 5) * 4 + (i & 3)] = acc[i];
  }
  __syncthreads();
  const int tid = threadIdx.x;
  if constexpr (GATE_UP) {
    const int mm = tid >> 4, n = tid & 15;
    if (mm < t.nrows) {
      float g = 0.0f, u = 0.0f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        g += red[w][mm][n];
        u += red[w][mm][n + 16];
      }
      uint16_t* h = reinterpret_cast<uint16_t*>(p.out);
      h[(int64_t)(t.row_begin + mm) * p.out_ld + rt * 16 + n] = to_h_elem<QF>(silu(g) * u);
    }
  } else {
    const int mm = tid >> 5, r = tid & 31;
    if (mm < t.nrows) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) s += red[w][mm][r];
      float* o = reinterpret_cast<float*>(p.out);
      o[(int64_t)(t.row_begin + mm) * p.out_ld + rt * 32 + r] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill kernel: persistent workgroups of 4 waves, two per CU.  A work item is
// (tile of up to 128 token rows of one expert, block of 8 weight row-tiles =
// 256 outputs).  Wave w owns row tiles 2w, 2w+1 of the block (64 outputs) and
// all of the tile's tokens (NCT column tiles of 32, a template parameter so the
// K loop has no branches).  Per K-block of 64 inputs the workgroup stages
// the activation tile in LDS (two buffers, rows padded to 144 bytes) while
// each wave decodes its weight chunks straight from global memory into MFMA
// operands.  Software pipeline: weights and activations are loaded two
// K-blocks ahead into register rings; activations are written to the other
// LDS buffer one K-block ahead.  Loads never branch: padding rows read a valid
// row of the tile and row tiles past N re-read the last row tile; those
// results are computed and not stored.
// ---------------------------------------------------------------------------
constexpr int kPreThreads = 256;
constexpr int kPreRowTilesPerWave = 2;
constexpr int kPreRowTilesPerItem = 8;
// LDS row: 64 16-bit inputs (32 u32) padded to 36 u32 (144 B), so 16
// consecutive rows start in 16 different 16-byte bank groups and both the
// staging writes (one row per lane) and the MFMA operand reads (one row per
// lane) are free of bank conflicts.
constexpr int kRowU32 = 36;

template <int QF, bool GATE_UP, int NCT, int WD>
__device__ __forceinline__ void prefill_item(const GemmArgs& p, const Tile& t, int nb,
                                             uint32_t (*lds)[kPrefillTM * kRowU32]) {
  using SL = ScaleLayout<QF>;
  constexpr int RTW = kPreRowTilesPerWave;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nrt = p.N >> 5;
  const int KB = p.K >> 6;
  // staging: 8 consecutive lanes read one 128-byte activation row, so each
  // load instruction covers 32 whole rows; chunk sc of rows q*32 + sr0, only
  // for the NCT*32 rows the tile uses
  const int sc = threadIdx.x & 7, sr0 = threadIdx.x >> 3;
  const int rt0 = nb * kPreRowTilesPerItem + wave * RTW;

  // staging sources: rows past the tile's end re-read its first row
  const uint16_t* s_src[NCT];
#pragma unroll
  for (int q = 0; q < NCT; ++q) {
    const int r = q * 32 + sr0;
    const int srow = (r < t.nrows) ? r : 0;
    const int64_t gr = p.gather ? p.gather[t.row_begin + srow] : (t.row_begin + srow);
    s_src[q] = reinterpret_cast<const uint16_t*>(p.act) + gr * p.K + sc * 8;
  }

  const uint8_t* rec = p.slot_ptr[t.slot];
  const uint8_t* codes[RTW];
  const uint8_t* scs[RTW];
#pragma unroll
  for (int r = 0; r < RTW; ++r) {
    const int rtl = min(rt0 + r, nrt - 1);
    codes[r] = rec + p.off_codes + (int64_t)rtl * KB * kTileCodeBytes + lane * 16;
    scs[r] = rec + p.off_scales + (int64_t)rtl * KB * SL::kTileBytes + SL::lane_off(lane);
  }

  f32x16 acc[RTW][NCT];
#pragma unroll
  for (int a = 0; a < RTW; ++a)
#pragma unroll
    for (int b = 0; b < NCT; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  u32x4 sv[2][NCT];        // activation chunks of two K-blocks in flight
  u32x4 wq[WD][RTW];       // weight ring: K-block kb lives in slot kb % WD
  uint32_t ws[WD][RTW];

  auto stage_load = [&](u32x4(&v)[NCT], int kb) {
    kb = min(kb, KB - 1);
#pragma unroll
    for (int q = 0; q < NCT; ++q) v[q] = ld16(s_src[q] + kb * 64);
  };
  auto stage_store = [&](const u32x4(&v)[NCT], int buf) {
#pragma unroll
    for (int q = 0; q < NCT; ++q)
      *reinterpret_cast<u32x4*>(&lds[buf][(q * 32 + sr0) * kRowU32 + sc * 4]) = v[q];
  };
  auto w_load = [&](u32x4(&q4)[RTW], uint32_t(&s4)[RTW], int kb) {
    kb = min(kb, KB - 1);
#pragma unroll
    for (int r = 0; r < RTW; ++r) {
      q4[r] = ld16(codes[r] + (int64_t)kb * kTileCodeBytes);
      s4[r] = SL::load(scs[r] + (int64_t)kb * SL::kTileBytes);
    }
  };
  auto compute = [&](int buf, const u32x4(&q4)[RTW], const uint32_t(&s4)[RTW]) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int c = 4 * (lane >> 5) + st;
      u32x4 b[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int mrow = ct * 32 + (lane & 31);
        b[ct] = *reinterpret_cast<const u32x4*>(&lds[buf][mrow * kRowU32 + c * 4]);
      }
#pragma unroll
      for (int r = 0; r < RTW; ++r) {
        const u32x4 a = ChunkScale<QF>(s4[r]).step(q4[r][st]);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[r][ct] = mfma<QF>(a, b[ct], acc[r][ct]);
      }
    }
  };
  // One K-block: store activation kb+1 into the other LDS buffer, load
  // activation kb+3 into the freed registers and weights kb+WD into the freed
  // ring slot, compute K-block kb.  D = kb % WD and the buffer parity are
  // compile-time, so every register index is static.
  auto one_step = [&](int kb, auto dc) {
    constexpr int D = decltype(dc)::value;
    constexpr int BUF = D & 1;
    stage_store(sv[BUF ^ 1], BUF ^ 1);
    stage_load(sv[BUF ^ 1], kb + 3);
    u32x4 q4[RTW];
    uint32_t s4[RTW];
#pragma unroll
    for (int r = 0; r < RTW; ++r) {
      q4[r] = wq[D][r];
      s4[r] = ws[D][r];
    }
    w_load(wq[D], ws[D], kb + WD);
    compute(BUF, q4, s4);
    __syncthreads();
  };

  // prologue: activation 0 in LDS, activations 1 and 2 and weights 0..WD-1 in flight
  stage_load(sv[0], 0);
  stage_load(sv[1], 1);
#pragma unroll
  for (int d = 0; d < WD; ++d) w_load(wq[d], ws[d], d);
  stage_store(sv[0], 0);
  stage_load(sv[0], 2);
  __syncthreads();

  int kb = 0;
  for (; kb + WD <= KB; kb += WD) {
    one_step(kb + 0, std::integral_constant<int, 0>{});
    one_step(kb + 1, std::integral_constant<int, 1>{});
    if constexpr (WD == 4) {
      one_step(kb + 2, std::integral_constant<int, 2>{});
      one_step(kb + 3, std::integral_constant<int, 3>{});
    }
  }
  // tail (KB not a multiple of WD): slots 0.. hold K-blocks kb..
  if (kb + 0 < KB) one_step(kb + 0, std::integral_constant<int, 0>{});
  if (kb + 1 < KB) one_step(kb + 1, std::integral_constant<int, 1>{});
  if constexpr (WD == 4) {
    if (kb + 2 < KB) one_step(kb + 2, std::integral_constant<int, 2>{});
  }

  // epilogue
#pragma unroll
  for (int r = 0; r < RTW; ++r) {
    const int rt = rt0 + r;
    if (rt >= nrt) continue;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int mm = ct * 32 + (lane & 31);
      if (mm >= t.nrows) continue;
      const int64_t row = t.row_begin + mm;
      if constexpr (GATE_UP) {
        uint16_t* h = reinterpret_cast<uint16_t*>(p.out) + row * p.out_ld + rt * 16;
#pragma unroll
        for (int g4 = 0; g4 < 2; ++g4) {
          uint16_t v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int i = g4 * 4 + q;
            v[q] = to_h_elem<QF>(silu(acc[r][ct][i]) * acc[r][ct][i + 8]);
          }
          const uint2 pk = {(uint32_t)v[0] | ((uint32_t)v[1] << 16),
                            (uint32_t)v[2] | ((uint32_t)v[3] << 16)};
          *reinterpret_cast<uint2*>(h + g4 * 8 + (lane >> 5) * 4) = pk;
        }
      } else {
        float* o = reinterpret_cast<float*>(p.out) + row * p.out_ld + rt * 32;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 v = {acc[r][ct][g4 * 4 + 0], acc[r][ct][g4 * 4 + 1], acc[r][ct][g4 * 4 + 2],
                            acc[r][ct][g4 * 4 + 3]};
          *reinterpret_cast<float4*>(o + g4 * 8 + (lane >> 5) * 4) = v;
        }
      }
    }
  }
}

template <int QF, bool GATE_UP>
__global__ __launch_bounds__(kPreThreads, 2) void moe_prefill_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[2][kPrefillTM * kRowU32];
  const int nrt = p.N >> 5;
  const int n_nb = (nrt + kPreRowTilesPerItem - 1) / kPreRowTilesPerItem;
  const int n_tiles = p.n_tiles_dev ? p.n_tiles_dev[0] : p.n_tiles;
  const int n_items = n_tiles * n_nb;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const Tile t = p.tiles[item / n_nb];
    const int nb = item % n_nb;
    switch ((t.nrows + 31) >> 5) {
      case 1: prefill_item<QF, GATE_UP, 1, 4>(p, t, nb, lds); break;
      case 2: prefill_item<QF, GATE_UP, 2, 4>(p, t, nb, lds); break;
      case 3: prefill_item<QF, GATE_UP, 3, 2>(p, t, nb, lds); break;
      default: prefill_item<QF, GATE_UP, 4, 2>(p, t, nb, lds); break;
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Combine: y[t] = sum_j w[t,j] * o[pos[t,j]] (j ascending) + o[shared row of t],
// fp32, rounded to bf16 (nearest-even).  One workgroup per token.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o,
                                                      const int32_t* __restrict__ pos,
                                                      const float* __restrict__ w, int k, int H,
                                                      int shared_row0, uint16_t* __restrict__ y) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x * 4; c < H; c += 1024) {
    float4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < k; ++j) {
      const float wj = w[(size_t)t * k + j];
      const float4 v = *reinterpret_cast<const float4*>(o + (size_t)pos[(size_t)t * k + j] * H + c);
      acc.x = __builtin_fmaf(wj, v.x, acc.x);
      acc.y = __builtin_fmaf(wj, v.y, acc.y);
      acc.z = __builtin_fmaf(wj, v.z, acc.z);
      acc.w = __builtin_fmaf(wj, v.w, acc.w);
    }
    if (shared_row0 >= 0) {
      const float4 v = *reinterpret_cast<const float4*>(o + (size_t)(shared_row0 + t) * H + c);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const uint2 pk = {(uint32_t)f32_to_bf16_rne(acc.x) | ((uint32_t)f32_to_bf16_rne(acc.y) << 16),
                      (uint32_t)f32_to_bf16_rne(acc.z) | ((uint32_t)f32_to_bf16_rne(acc.w) << 16)};
    *reinterpret_cast<uint2*>(y + (size_t)t * H + c) = pk;
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_expert_gemm(const GemmArgs& a, int quant, bool gate_up, bool decode, int grid,
                              hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (decode) {
    if (quant == Q_INT4) {
      if (gate_up)
        moe_decode_kernel<Q_INT4, true><<<grid, 512, 0, s>>>(a);
      else
        moe_decode_kernel<Q_INT4, false><<<grid, 512, 0, s>>>(a);
    } else {
      if (gate_up)
        moe_decode_kernel<Q_MXFP4, true><<<grid, 512, 0, s>>>(a);
      else
        moe_decode_kernel<Q_MXFP4, false><<<grid, 512, 0, s>>>(a);
    }
  } else {
    if (quant == Q_INT4) {
      if (gate_up)
        moe_prefill_kernel<Q_INT4, true><<<grid, kPreThreads, 0, s>>>(a);
      else
        moe_prefill_kernel<Q_INT4, false><<<grid, kPreThreads, 0, s>>>(a);
    } else {
      if (gate_up)
        moe_prefill_kernel<Q_MXFP4, true><<<grid, kPreThreads, 0, s>>>(a);
      else
        moe_prefill_kernel<Q_MXFP4, false><<<grid, kPreThreads, 0, s>>>(a);
    }
  }
  return hipGetLastError();
}

hipError_t launch_combine(const float* o, const int32_t* pos, const float* w, int T, int k, int H,
                          int shared_row0, uint16_t* y, hipStream_t s) {
  combine_kernel<<<T, 256, 0, s>>>(o, pos, w, k, H, shared_row0, y);
  return hipGetLastError();
}

}  // namespace strata
