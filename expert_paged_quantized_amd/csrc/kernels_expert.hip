// Expert kernels of the MoE layer for gfx950: grouped SwiGLU FFN computed
// straight from 4-bit packed weights (on the MFMA units for prefill and 5..8
// decode tokens, on the VALU dot units for 1..4), and the weighted combine.
//
// Weights stay 4-bit in HBM and are decoded in registers into MFMA or dot
// operands, never into a wider resident copy (ro99/strata README: precision
// paragraph, and the SM86 kernel paragraph, whose register-fed decode into
// matrix-core operands is the prior art here; its prepack into operand order
// is a pure byte permutation, as is the tile order used below).  One weight
// layout serves the decode kernels (T <= 8 tokens: a 32-row tile per group of
// waves, K split across the waves of one workgroup and added in LDS in a fixed
// order) and the prefill kernel (token tiles of 128 rows staged in LDS), as
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
// int4 affine weights are decoded to fp16 (w' = s'*q + b', one fp16 rounding,
// where s', b' are the checkpoint's bf16 scale and bias times one power of
// two 2^-c per matrix, chosen at load so that both are exact in fp16 and no
// decoded weight exceeds 2^15) and the activations arrive as fp16 scaled per
// token by 2^-xexp[t] (the router kernel writes that copy of x).  The GEMM
// epilogues undo both powers of two in fp32, and the SwiGLU output h is
// stored scaled by a further 2^-(xexp[t] + c_h), with c_h fixed per expert
// from its weights so that |h| stays below 2^14 for any bf16 x: the fp16
// operands never overflow.  NVFP4 takes the same route (its decoded weights
// are exact in fp16).  MXFP4 weights are decoded to bf16 with the gfx950
// scaled FP4 conversion (exact: an E2M1 value times a power of two) and run
// on the bf16 input and a bf16 h, which have fp32's exponent range.
// Accumulation is fp32 throughout; nothing uses float atomics, so every
// expert's result depends only on its own rows and weights.
#include <algorithm>
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
typedef const __attribute__((address_space(1))) uint16_t g_u16;
typedef const __attribute__((address_space(1))) float g_f32;
__device__ __forceinline__ u32x4 ld16(const void* p) { return *(g_u32x4*)(p); }
__device__ __forceinline__ uint32_t ld4(const void* p) { return *(g_u32*)(p); }
__device__ __forceinline__ uint32_t ld1(const void* p) { return *(g_u8*)(p); }
__device__ __forceinline__ uint32_t ld2(const void* p) { return *(g_u16*)(p); }
// Streaming (non-temporal) variants for weights read once per launch: they
// do not displace cached data, and measured streaming reads reach about 7 TB/s
// this way against about 5 TB/s with ordinary loads.
__device__ __forceinline__ u32x4 ld16_nt(const void* p) { return __builtin_nontemporal_load((g_u32x4*)(p)); }
__device__ __forceinline__ uint32_t ld4_nt(const void* p) { return __builtin_nontemporal_load((g_u32*)(p)); }
__device__ __forceinline__ uint32_t ld1_nt(const void* p) { return __builtin_nontemporal_load((g_u8*)(p)); }
__device__ __forceinline__ uint32_t ld2_nt(const void* p) { return __builtin_nontemporal_load((g_u16*)(p)); }

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
// fp16 fma gives s'*q + b' (the matrix's rescaled scale and bias).
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

// OCP FP8 E4M3 byte -> fp32 (exact): sign bit 7, exponent bits 6..3 (bias 7),
// mantissa bits 2..0, exponent 0 subnormal (m * 2^-9).  NaN bytes never reach
// a kernel (admission refuses them).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u, sgn = (b & 0x80u) << 24;
  const float nrm = __uint_as_float(sgn | ((e + 120u) << 23) | (m << 20));
  const float sub = __uint_as_float(__float_as_uint((float)m * 0.001953125f) | sgn);
  return e ? nrm : sub;
}

// One MFMA step (8 inputs) of an NVFP4 chunk: the E2M1 codes converted with a
// unit scale (exact in fp16), times the fp16 E4M3 block scale (exact: at most
// 6 significant bits, magnitudes 2^-10 .. 2688).
__device__ __forceinline__ u32x4 dequant_nvfp4_step(uint32_t w, f16x2 sc) {
  u32x4 a;
  a[0] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sc);
  a[1] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sc);
  a[2] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sc);
  a[3] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sc);
  return a;
}

// Per-chunk decode parameters: fp16 (scale, bias) pairs for int4 (the scale
// word holds fp16 s' in its low half and b' in its high half), the fp32
// power of two for MXFP4, the fp16 scales of the chunk's two 16-input blocks
// for NVFP4 (words 0-1 and 2-3 of the chunk).
template <int QF>
struct ChunkScale {
  f16x2 s2, b2;
  float scale;
  __device__ __forceinline__ explicit ChunkScale(uint32_t sc) {
    if constexpr (QF == Q_INT4) {
      const f16x2 sb = bitcast<f16x2>(sc);
      s2 = __builtin_shufflevector(sb, sb, 0, 0);
      b2 = __builtin_shufflevector(sb, sb, 1, 1);
      scale = 0.0f;
    } else if constexpr (QF == Q_NVFP4) {
      // both block scales in one register: (first 16 inputs, second 16)
      s2 = f16x2{(_Float16)e4m3_to_f32(sc & 0xffu), (_Float16)e4m3_to_f32(sc >> 8)};
      b2 = s2;
      scale = 0.0f;
    } else {
      scale = __uint_as_float(sc << 23);
    }
  }
  __device__ __forceinline__ u32x4 step(uint32_t w, int st) const {
    if constexpr (QF == Q_INT4)
      return dequant_int4_step(w, s2, b2);
    else if constexpr (QF == Q_NVFP4)
      return dequant_nvfp4_step(w, st < 2 ? __builtin_shufflevector(s2, s2, 0, 0)
                                          : __builtin_shufflevector(s2, s2, 1, 1));
    else
      return dequant_fp4_step(w, scale);
  }
};

template <int QF>
__device__ __forceinline__ void dequant(const u32x4& c, uint32_t sc, u32x4 (&a)[4]) {
  const ChunkScale<QF> cs(sc);
#pragma unroll
  for (int st = 0; st < 4; ++st) a[st] = cs.step(c[st], st);
}

// fp32 matrix scales of this GEMM (NVFP4: gate and up, or down in .x), else 1.
template <int QF>
__device__ __forceinline__ float2 matrix_scales(const GemmArgs& p, const uint8_t* rec) {
  if constexpr (QF == Q_NVFP4) {
    const g_f32* g = (const g_f32*)(rec + p.off_gscale);
    return float2{g[0], g[1]};
  } else {
    return float2{1.0f, 1.0f};
  }
}

template <int QF>
__device__ __forceinline__ f32x16 mfma(const u32x4& a, const u32x4& b, const f32x16& c) {
  if constexpr (QF != Q_MXFP4)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(bitcast<f16x8>(a), bitcast<f16x8>(b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(bitcast<bf16x8>(a), bitcast<bf16x8>(b), c, 0, 0,
                                                   0);
}

// scale bytes per scale block and the lane's offset inside it
template <int QF>
struct ScaleLayout {
  static constexpr int kTileBytes = (QF == Q_MXFP4) ? 64 : 128;
  __device__ static int lane_off(int lane) {
    if constexpr (QF == Q_INT4) return (lane & 31) * 4;
    else if constexpr (QF == Q_NVFP4) return lane * 2;
    else return lane;
  }
  __device__ static uint32_t load(const uint8_t* p) {
    if constexpr (QF == Q_INT4) return ld4(p);
    else if constexpr (QF == Q_NVFP4) return ld2(p);
    else return ld1(p);
  }
  __device__ static uint32_t load_nt(const uint8_t* p) {
    if constexpr (QF == Q_INT4) return ld4_nt(p);
    else if constexpr (QF == Q_NVFP4) return ld2_nt(p);
    else return ld1_nt(p);
  }
};

// silu(g) = g / (1 + e^-g) with the hardware reciprocal (1 ulp) in place of an
// IEEE division (about ten instructions): the result is rounded to 16 bits
// right after, and g = -inf.. +inf still give -0 .. g.
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

template <int QF>
__device__ __forceinline__ uint16_t to_h_elem(float f) {
  if constexpr (QF != Q_MXFP4)
    return bitcast<uint16_t>((_Float16)f);
  else
    return f32_to_bf16_rne(f);
}

// Epilogue exponents of one output column (a row of the permuted space) of
// expert `expert`, for the fp16 formats; all zero for MXFP4.  Gate+up: the
// gate accumulator times 2^g is g itself, the up accumulator times 2^u is u
// times the h row's 2^-(2 xexp[t] + c_h).  Down: the accumulator times 2^o.
struct ColExp {
  int g, u, o;
};
template <int QF, bool GATE_UP>
__device__ __forceinline__ ColExp col_exp(const GemmArgs& p, int expert, int64_t row) {
  ColExp r{0, 0, 0};
  if constexpr (QF != Q_MXFP4) {
    const int et = p.xexp[p.tok_of_row[row]];
    const int32_t* we = p.wexp + expert * kWexpCount;
    if constexpr (GATE_UP) {
      r.g = et + we[kWexpGate];
      r.u = we[kWexpUp] - et - we[kWexpH];
    } else {
      r.o = 2 * et + we[kWexpH] + we[kWexpDown];
    }
  }
  return r;
}
// The same exponents in two steps, for the prefill epilogue: the expert's
// weight exponents (and each column's token) can be loaded before the K
// loop, leaving one dependent load (the token's exponent) for after it.
// Integer sums, so the split changes no value.
struct ColExpPre {
  int wa, wb;  // gate+up: gate and up - h exponents; down: h + down
};
template <int QF, bool GATE_UP>
__device__ __forceinline__ ColExpPre col_exp_pre(const GemmArgs& p, int expert) {
  ColExpPre r{0, 0};
  if constexpr (QF != Q_MXFP4) {
    const int32_t* we = p.wexp + expert * kWexpCount;
    if constexpr (GATE_UP) {
      r.wa = we[kWexpGate];
      r.wb = we[kWexpUp] - we[kWexpH];
    } else {
      r.wa = we[kWexpH] + we[kWexpDown];
    }
  }
  return r;
}
template <int QF, bool GATE_UP>
__device__ __forceinline__ ColExp col_exp_post(const GemmArgs& p, const ColExpPre& q, int tok) {
  ColExp r{0, 0, 0};
  if constexpr (QF != Q_MXFP4) {
    const int et = p.xexp[tok];
    if constexpr (GATE_UP) {
      r.g = et + q.wa;
      r.u = q.wb - et;
    } else {
      r.o = 2 * et + q.wa;
    }
  }
  return r;
}
__device__ __forceinline__ float pow2_scale(float v, int e) { return __builtin_amdgcn_ldexpf(v, e); }

// The stored h element from the gate and up accumulators (gs: NVFP4 matrix
// scales, else 1).
template <int QF>
__device__ __forceinline__ uint16_t h_elem(float ag, float au, float2 gs, const ColExp& ce) {
  if constexpr (QF == Q_MXFP4)
    return to_h_elem<QF>(silu(ag) * au);
  else
    return to_h_elem<QF>(silu(pow2_scale(ag * gs.x, ce.g)) * pow2_scale(au * gs.y, ce.u));
}
// One element of o from the down accumulator.
template <int QF>
__device__ __forceinline__ float o_elem(float acc, float gsx, const ColExp& ce) {
  if constexpr (QF == Q_MXFP4)
    return acc;
  else
    return pow2_scale(acc * gsx, ce.o);
}

// ---------------------------------------------------------------------------
// MFMA decode kernel (T <= 8 tokens; used where the dot-product kernel's
// staged token rows would not fit its LDS).  Workgroup = 8 waves = R row tiles (32
// weight rows each) of one expert x S K-splits, R*S = 8.  K is walked in
// chunks of S*8 K-blocks; in a chunk, wave (r, s) takes the 8 consecutive
// blocks s*8..s*8+7 of row tile r.  The token rows of a chunk are staged in
// LDS once for all eight waves, their loads issued a whole chunk ahead.  Each
// wave streams its 1 KB code chunks (and scales) through an 8-deep register
// ring: a slot is decoded, then refilled with the block of the next chunk, so
// eight blocks stay in flight.  Every load address is clamped rather than
// branched around, keeping the loop straight-line so the wait counters track
// each slot (and the activation loads, issued a chunk before their use)
// exactly.  At the end the S partial sums of a row tile are added in LDS in
// split order 0..S-1, then the epilogue runs.  S is fixed per layer shape
// (capped by LDS at 8 tokens), never by the tiles of a launch.
// ---------------------------------------------------------------------------
constexpr int kDecWaves = 8;
constexpr int kDecDepth = 8;

// Epilogue of one wave's 32-row tile rt for the token columns n < nrows.
template <int QF, bool GATE_UP>
__device__ __forceinline__ void decode_store(const GemmArgs& p, const Tile& t, int rt, int lane,
                                             const f32x16& acc, float2 gs) {
  const int n = lane & 31;
  if (n >= t.nrows) return;
  const int64_t row = t.row_begin + n;
  const ColExp ce = col_exp<QF, GATE_UP>(p, t.expert, row);
  if constexpr (GATE_UP) {
    uint16_t* h = reinterpret_cast<uint16_t*>(p.out) + row * p.out_ld + rt * 16;
#pragma unroll
    for (int g4 = 0; g4 < 2; ++g4) {
      uint16_t v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = g4 * 4 + q;
        v[q] = h_elem<QF>(acc[i], acc[i + 8], gs, ce);
      }
      const uint2 pk = {(uint32_t)v[0] | ((uint32_t)v[1] << 16), (uint32_t)v[2] | ((uint32_t)v[3] << 16)};
      *reinterpret_cast<uint2*>(h + g4 * 8 + (lane >> 5) * 4) = pk;
    }
  } else {
    float* o = reinterpret_cast<float*>(p.out) + row * p.out_ld + rt * 32;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const float4 v = {o_elem<QF>(acc[g4 * 4 + 0], gs.x, ce), o_elem<QF>(acc[g4 * 4 + 1], gs.x, ce),
                        o_elem<QF>(acc[g4 * 4 + 2], gs.x, ce), o_elem<QF>(acc[g4 * 4 + 3], gs.x, ce)};
      *reinterpret_cast<float4*>(o + g4 * 8 + (lane >> 5) * 4) = v;
    }
  }
}

// NP = 16-byte activation pieces each thread stages per chunk:
// ceil(T * S * 64 / 512) for the launch's token count T (>= every tile's
// rows), with T * S <= 32.
template <int QF, bool GATE_UP, int NP>
__global__ __launch_bounds__(kDecWaves * 64) void moe_decode_kernel(GemmArgs p, int log2S) {
  extern __shared__ __attribute__((aligned(16))) uint32_t xs[];
  using SL = ScaleLayout<QF>;
  const int S = 1 << log2S, R = kDecWaves >> log2S;
  const int nrt = p.N >> 5;
  const int nrg = (nrt + R - 1) / R;
  const int rg = blockIdx.x % nrg, tile_i = blockIdx.x / nrg;
  const int n_tiles = p.n_tiles_dev ? p.n_tiles_dev[0] : p.n_tiles;
  if (tile_i >= n_tiles) return;  // the whole workgroup leaves together
  const Tile t = p.tiles[tile_i];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sw = wave & (S - 1);           // this wave's split
  const int rt = rg * R + (wave >> log2S);
  const int rtc = min(rt, nrt - 1);
  const int KB = p.K >> 6;
  const int cb = S * kDecDepth;             // K-blocks per chunk
  const int nc = (KB + cb - 1) / cb;
  const int row_u32 = cb * 32 + 4;          // staged row: cb*64 16-bit inputs + 16 B pad

  const uint8_t* rec = p.slot_ptr[t.slot];
  const uint8_t* codes = rec + p.off_codes + (int64_t)rtc * KB * kTileCodeBytes + lane * 16;
  const uint8_t* scales =
      rec + p.off_scales + (int64_t)rtc * (KB >> p.sshift) * SL::kTileBytes + SL::lane_off(lane);

  // staging pieces (the tile's own rows only): piece pc = tid + 512*j ->
  // token row pc >> (log2S + 6), 16-byte column pc & (S*64 - 1) of the
  // chunk; columns past K re-read the row's last piece (staged, never used)
  const int pieces = t.nrows << (log2S + 6);
  const uint16_t* xrow[NP];
  int xcol[NP], xdst[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    const int q = tid + j * kDecWaves * 64;
    const int pc = min(q, pieces - 1);
    const int r = pc >> (log2S + 6), c = pc & ((S << 6) - 1);
    const int64_t ar = p.gather ? p.gather[t.row_begin + r] : (t.row_begin + r);
    xrow[j] = reinterpret_cast<const uint16_t*>(p.act) + ar * p.K;
    xcol[j] = c * 8;
    xdst[j] = (q < pieces) ? r * row_u32 + c * 4 : -1;
  }
  auto x_load = [&](u32x4(&v)[NP], int cc) {
#pragma unroll
    for (int j = 0; j < NP; ++j) v[j] = ld16(xrow[j] + min(cc * cb * 64 + xcol[j], p.K - 8));
  };
  auto x_store = [&](const u32x4(&v)[NP]) {
#pragma unroll
    for (int j = 0; j < NP; ++j)
      if (xdst[j] >= 0) *reinterpret_cast<u32x4*>(&xs[xdst[j]]) = v[j];
  };

  // weight ring prologue: slot j holds block sw*8 + j of chunk 0
  u32x4 wq[kDecDepth];
  uint32_t ws[kDecDepth];
#pragma unroll
  for (int j = 0; j < kDecDepth; ++j) {
    const int kb = min(sw * kDecDepth + j, KB - 1);
    wq[j] = ld16_nt(codes + (int64_t)kb * kTileCodeBytes);
    ws[j] = SL::load_nt(scales + (int64_t)(kb >> p.sshift) * SL::kTileBytes);
  }
  u32x4 xv[NP];
  x_load(xv, 0);
  x_store(xv);
  x_load(xv, 1);  // chunk 1 in flight during chunk 0
  __syncthreads();

  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
  const uint32_t* brow = xs + min(lane & 31, t.nrows - 1) * row_u32 + sw * (kDecDepth * 32) + (lane >> 5) * 16;

  for (int cc = 0; cc < nc; ++cc) {
    const int kbase = cc * cb + sw * kDecDepth;
#pragma unroll
    for (int j = 0; j < kDecDepth; ++j) {
      // decode slot j first so its registers are free for the refill (the
      // refill then reuses them in place and nothing is copied at the loop
      // edge, which would wait for every load in flight)
      u32x4 a[4];
      dequant<QF>(wq[j], ws[j], a);
      asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3])::"memory");
      const int kn = min(kbase + cb + j, KB - 1);
      wq[j] = ld16_nt(codes + (int64_t)kn * kTileCodeBytes);
      ws[j] = SL::load_nt(scales + (int64_t)(kn >> p.sshift) * SL::kTileBytes);
      if (kbase + j < KB) {
        const uint32_t* bp = brow + j * 32;
#pragma unroll
        for (int st = 0; st < 4; ++st)
          acc = mfma<QF>(a[st], *reinterpret_cast<const u32x4*>(bp + st * 4), acc);
      }
    }
    __syncthreads();  // chunk cc fully read
    x_store(xv);      // chunk cc+1 (past the end: unused)
    x_load(xv, cc + 2);
    __syncthreads();
  }

  // add the S partial sums of each row tile in split order (LDS reused)
  float* red = reinterpret_cast<float*>(xs);
  const int n = lane & 31;
  if (sw > 0 && n < t.nrows) {
    float* d = red + ((wave * kDecodeMaxT + n) * 32) + (lane >> 5) * 4;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4)
      *reinterpret_cast<float4*>(d + g4 * 8) =
          float4{acc[g4 * 4 + 0], acc[g4 * 4 + 1], acc[g4 * 4 + 2], acc[g4 * 4 + 3]};
  }
  __syncthreads();
  if (sw == 0 && rt < nrt) {
    if (n < t.nrows) {
      for (int s2 = 1; s2 < S; ++s2) {
        const float* d = red + (((wave + s2) * kDecodeMaxT + n) * 32) + (lane >> 5) * 4;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 v = *reinterpret_cast<const float4*>(d + g4 * 8);
          acc[g4 * 4 + 0] += v.x;
          acc[g4 * 4 + 1] += v.y;
          acc[g4 * 4 + 2] += v.z;
          acc[g4 * 4 + 3] += v.w;
        }
      }
    }
    decode_store<QF, GATE_UP>(p, t, rt, lane, acc, matrix_scales<QF>(p, rec));
  }
}


// ---------------------------------------------------------------------------
// Dot-product decode kernel (T <= 8 tokens; above 4 the tiles hold at most 4
// rows, so a tile never has more than 4).  At a handful of tokens the
// 32-column MFMA wastes most of its work and its issue time adds to the
// decode time, so the contraction runs on the VALU dot units instead:
//   int4:  an AND leaves a code pair as fp16 denormals (q * 2^-24 for the low
//          nibbles, q * 2^-20 for the high ones, exact), v_dot2_f32_f16
//          multiplies them with the scaled fp16 activations, and the group's
//          affine parameters are applied once per 32 inputs in fp32:
//          s' * sum(x q) + b' * sum(x), with sum(x) staged alongside the
//          activations.  No weight is rounded to 16 bits on this path.
//   MXFP4: the gfx950 FP4 conversion (unit scale) gives exact bf16 pairs,
//          v_dot2_f32_bf16 contracts them, and the E8M0 power of two scales
//          the 32-input group sum.
//   NVFP4: the same conversion to fp16 pairs, v_dot2_f32_f16 against the fp16
//          activations, each 16-input block sum times its E4M3 scale, the
//          matrix scale applied to the final sums.
// Workgroup = S waves on one 32-row weight tile, wave s streaming the
// contiguous K-blocks [s*KB/S, (s+1)*KB/S) of it; lane l owns tile row l%32
// and inputs 32*(l/32)..+31 of each block (the prepacked layout: one 16-byte
// code chunk, one affine or E8M0 group).  The token rows (all of K) are
// staged in LDS once; weights stream through a register ring (16, 12 or 8 deep),
// each slot unpacked before it is refilled in place.  The halves of a row are
// added lane l + lane l+32, then the S partial sums in wave order, then the
// epilogue.
// ---------------------------------------------------------------------------
// weight ring depth: registers at 1024 threads per workgroup are capped at
// 128 per lane, and every token adds accumulators and activation operands
// Weight ring depth (K-blocks in flight per wave) by token rows: one row
// holds 14 blocks, or 16 when every wave's K range is a multiple of 16 (one
// round then loads each block once).  At 16 the int4 and MXFP4 code fits the
// 128 registers of a 1,024-thread launch with no spill (int4 with its paired
// scale words); NVFP4 at 16 still spills a few registers.
constexpr int dot_depth(int tt, bool d16) { return tt == 1 ? (d16 ? 16 : 14) : (tt == 2 ? 12 : 8); }

// Token rows of a dot-decode unit into registers: thread tid loads the
// 16-byte pieces tid + j * nthr (j < NPR) of each of the TT rows; rows past
// nrows re-read the last row and pieces past the row re-read its last piece.
template <int TT, int NPR>
__device__ __forceinline__ void dot_load_rows(const GemmArgs& p, const Tile& t, int tid, int nthr,
                                              u32x4 (&v)[TT][NPR]) {
  const int pr = p.K >> 3;  // 16-byte pieces per row
#pragma unroll
  for (int r = 0; r < TT; ++r) {
    const int rr = min(r, t.nrows - 1);
    const int64_t ar = p.gather ? p.gather[t.row_begin + rr] : (t.row_begin + rr);
    const uint16_t* src = reinterpret_cast<const uint16_t*>(p.act) + ar * p.K;
#pragma unroll
    for (int j = 0; j < NPR; ++j) {
      v[r][j] = ld16(src + min(tid + j * nthr, pr - 1) * 8);
    }
  }
}

// Stages the token rows in LDS (row r at xs + r * row_u32); for int4 also the
// sums of each 32 inputs (xsum[r][K/32]), four consecutive 8-input pieces per
// quad of threads, added in a fixed tree.
template <int QF, int TT, int NPR>
__device__ __forceinline__ void dot_store_rows(const u32x4 (&v)[TT][NPR], uint32_t* xs, int row_u32,
                                               float* xsum, int tid, int nthr, int K) {
  const int pr = K >> 3;
#pragma unroll
  for (int r = 0; r < TT; ++r) {
#pragma unroll
    for (int j = 0; j < NPR; ++j) {
      const int c = tid + j * nthr;
      if (c < pr) *reinterpret_cast<u32x4*>(&xs[r * row_u32 + c * 4]) = v[r][j];
      if constexpr (QF == Q_INT4) {
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
        float sum = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) sum = __builtin_amdgcn_fdot2(bitcast<f16x2>(v[r][j][q]), one, sum, false);
        // quad (xor 1, then xor 2) sum in a fixed tree; nthr is a multiple
        // of 64 and pr of 8, so a quad never straddles rows
        sum += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, sum), 0xB1, 0xF, 0xF, false));
        sum += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, sum), 0x4E, 0xF, 0xF, false));
        if (c < pr && (c & 3) == 0) xsum[r * (K >> 5) + (c >> 2)] = sum;
      }
    }
  }
}

// Scale words a wave's ring holds for DEPTH K-blocks.  int4: one register
// per two consecutive K-blocks.  Lanes l and l + 32 contract the same weight
// row (l % 32), so both halves of a wave would load the same 32 scale words;
// instead lanes 0-31 hold K-block 2i's words and lanes 32-63 K-block 2i+1's,
// and a lane swap (v_permlane32_swap) gives every lane both.  MXFP4 and NVFP4
// scale bytes differ per lane: one register per K-block.
constexpr int ring_scales(int qf, int depth) { return qf == Q_INT4 ? depth / 2 : depth; }

// Weight ring prologue: slot j holds K-block kb0 + j.  Slots past the wave's
// K range (never contracted) load the same 16 bytes in every lane instead, one
// small request rather than a second copy of a 1 KB block: the address is
// selected, not branched around, so the wait counts stay exact.
template <int QF, int DEPTH>
__device__ __forceinline__ void dot_prologue(u32x4 (&wq)[DEPTH], uint32_t (&ws)[ring_scales(QF, DEPTH)],
                                             const uint8_t* codes, const uint8_t* scales, const uint8_t* codes0,
                                             const uint8_t* scales0, int kb0, int nkb, int sshift, int lane) {
  using SL = ScaleLayout<QF>;
#pragma unroll
  for (int j = 0; j < DEPTH; ++j) {
    const bool in = j < nkb;
    wq[j] = ld16_nt(in ? codes + (int64_t)j * kTileCodeBytes : codes0);
    if constexpr (QF == Q_INT4) {
      if (j % 2 == 0) {
        const int kb = j + (lane >> 5);  // this half's K-block of the pair
        ws[j / 2] = SL::load_nt(kb < nkb ? scales + (int64_t)((kb0 + kb) >> sshift) * SL::kTileBytes : scales0);
      }
    } else {
      ws[j] = SL::load_nt(in ? scales + (int64_t)((kb0 + j) >> sshift) * SL::kTileBytes : scales0);
    }
  }
}

// The K loop of one wave: K-blocks kb0 .. kb0 + nkb - 1 of its row tile against
// the staged token rows; each ring slot is unpacked, refilled in place, then
// contracted.  acc[r] = this lane's partial sum for token r (row lane % 32,
// inputs of half lane / 32).
template <int QF, int TT, int DEPTH>
__device__ __forceinline__ void dot_contract(u32x4 (&wq)[DEPTH], uint32_t (&ws)[ring_scales(QF, DEPTH)],
                                             const uint8_t* codes,
                                             const uint8_t* scales, const uint8_t* codes0,
                                             const uint8_t* scales0, int kb0, int nkb, int sshift,
                                             const uint32_t* xs, int row_u32, const float* xsum, int K,
                                             int lane, float (&acc)[TT]) {
  using SL = ScaleLayout<QF>;
  const int h = lane >> 5;
  const uint32_t* xl = xs + (kb0 * 32 + h * 16);  // this lane's 32 inputs of block kb0, row 0
  const float* xsl = xsum + kb0 * 2 + h;
  // One round of DEPTH slots from K-block i; RF: refill each slot with the
  // K-block DEPTH later (past the K range: the one small request of the
  // prologue).  The last round refills nothing, so every block of the wave's
  // K range is loaded exactly once.
  auto round = [&](int i, auto rf) {
    constexpr bool RF = decltype(rf)::value;
    uint32_t sc_lo = 0, sc_hi = 0;  // int4: the current pair's scale words
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      const int kbl = i + j;
      const int kn = kbl + DEPTH;
      const bool kn_in = kn < nkb;
      if constexpr (QF == Q_INT4) {
        uint32_t m[4][4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          const uint32_t w = wq[j][st], w8 = w >> 8;
          m[st][0] = w & 0x000F000Fu;   // (k0, k1) * 2^-24
          m[st][1] = w & 0x00F000F0u;   // (k2, k3) * 2^-20
          m[st][2] = w8 & 0x000F000Fu;  // (k4, k5) * 2^-24
          m[st][3] = w8 & 0x00F000F0u;  // (k6, k7) * 2^-20
        }
        // the pair's words: K-block j (lanes 0-31's) and j + 1 (lanes 32-63's)
        // in every lane, taken at the even slot, which frees the register
        if (j % 2 == 0) {
          const auto sw = __builtin_amdgcn_permlane32_swap(ws[j / 2], ws[j / 2], false, false);
          sc_lo = sw[0];
          sc_hi = sw[1];
        }
        const f16x2 sbh = bitcast<f16x2>(j % 2 == 0 ? sc_lo : sc_hi);  // (s', b') in fp16
        float s = (float)sbh[0], b = (float)sbh[1];
        asm volatile("" : "+v"(m[0][0]), "+v"(m[0][1]), "+v"(m[0][2]), "+v"(m[0][3]), "+v"(m[1][0]),
                     "+v"(m[1][1]), "+v"(m[1][2]), "+v"(m[1][3]), "+v"(m[2][0]), "+v"(m[2][1]),
                     "+v"(m[2][2]), "+v"(m[2][3]), "+v"(m[3][0]), "+v"(m[3][1]), "+v"(m[3][2]),
                     "+v"(m[3][3]), "+v"(s), "+v"(b), "+v"(sc_hi)::"memory");
        if constexpr (RF) {
          wq[j] = ld16_nt(kn_in ? codes + (int64_t)kn * kTileCodeBytes : codes0);
          if (j % 2 == 0) {
            const int kh = kn + (lane >> 5);  // this half's K-block of the next pair
            ws[j / 2] = SL::load_nt(kh < nkb ? scales + (int64_t)((kb0 + kh) >> sshift) * SL::kTileBytes : scales0);
          }
        }
        if (kbl < nkb) {
          float xsv[TT];  // sum(x) of the group: read first, used last
#pragma unroll
          for (int r = 0; r < TT; ++r) xsv[r] = xsl[r * (K >> 5) + kbl * 2];
#pragma unroll
          for (int r = 0; r < TT; ++r) {
            const uint32_t* xr = xl + r * row_u32 + kbl * 32;
            float lo = 0.0f, hi = 0.0f;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
              const u32x4 x = *reinterpret_cast<const u32x4*>(xr + st * 4);
              lo = __builtin_amdgcn_fdot2(bitcast<f16x2>(m[st][0]), bitcast<f16x2>(x[0]), lo, false);
              hi = __builtin_amdgcn_fdot2(bitcast<f16x2>(m[st][1]), bitcast<f16x2>(x[1]), hi, false);
              lo = __builtin_amdgcn_fdot2(bitcast<f16x2>(m[st][2]), bitcast<f16x2>(x[2]), lo, false);
              hi = __builtin_amdgcn_fdot2(bitcast<f16x2>(m[st][3]), bitcast<f16x2>(x[3]), hi, false);
            }
            const float xq = __builtin_fmaf(lo, 16.0f, hi) * 1048576.0f;  // sum(x q)
            acc[r] = __builtin_fmaf(s, xq, acc[r]);
            acc[r] = __builtin_fmaf(b, xsv[r], acc[r]);
          }
        }
      } else if constexpr (QF == Q_NVFP4) {
        // E2M1 codes converted with a unit scale (exact in fp16); the chunk's
        // two 16-input blocks (words 0-1, 2-3) get their E4M3 scales in fp32
        u32x4 m[4];
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int st = 0; st < 4; ++st) m[st] = dequant_nvfp4_step(wq[j][st], one);
        float s0 = e4m3_to_f32(ws[j] & 0xffu), s1 = e4m3_to_f32(ws[j] >> 8);
        asm volatile("" : "+v"(m[0]), "+v"(m[1]), "+v"(m[2]), "+v"(m[3]), "+v"(s0), "+v"(s1)::"memory");
        if constexpr (RF) {
          wq[j] = ld16_nt(kn_in ? codes + (int64_t)kn * kTileCodeBytes : codes0);
          ws[j] = SL::load_nt(kn_in ? scales + (int64_t)((kb0 + kn) >> sshift) * SL::kTileBytes : scales0);
        }
        if (kbl < nkb) {
#pragma unroll
          for (int r = 0; r < TT; ++r) {
            const uint32_t* xr = xl + r * row_u32 + kbl * 32;
            float d0 = 0.0f, d1 = 0.0f;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
              const u32x4 x = *reinterpret_cast<const u32x4*>(xr + st * 4);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if (st < 2)
                  d0 = __builtin_amdgcn_fdot2(bitcast<f16x2>(m[st][e]), bitcast<f16x2>(x[e]), d0, false);
                else
                  d1 = __builtin_amdgcn_fdot2(bitcast<f16x2>(m[st][e]), bitcast<f16x2>(x[e]), d1, false);
              }
            }
            acc[r] = __builtin_fmaf(s0, d0, acc[r]);
            acc[r] = __builtin_fmaf(s1, d1, acc[r]);
          }
        }
      } else {
        u32x4 m[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) m[st] = dequant_fp4_step(wq[j][st], 1.0f);
        float scale = __uint_as_float(ws[j] << 23);
        asm volatile("" : "+v"(m[0]), "+v"(m[1]), "+v"(m[2]), "+v"(m[3]), "+v"(scale)::"memory");
        if constexpr (RF) {
          wq[j] = ld16_nt(kn_in ? codes + (int64_t)kn * kTileCodeBytes : codes0);
          ws[j] = SL::load_nt(kn_in ? scales + (int64_t)((kb0 + kn) >> sshift) * SL::kTileBytes : scales0);
        }
        if (kbl < nkb) {
#pragma unroll
          for (int r = 0; r < TT; ++r) {
            const uint32_t* xr = xl + r * row_u32 + kbl * 32;
            float d = 0.0f;
#pragma unroll
            for (int st = 0; st < 4; ++st) {
              const u32x4 x = *reinterpret_cast<const u32x4*>(xr + st * 4);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                d = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(m[st][e]), bitcast<bf16x2>(x[e]), d, false);
            }
            acc[r] = __builtin_fmaf(scale, d, acc[r]);
          }
        }
      }
    }
  };
  int i = 0;
  for (; i + DEPTH < nkb; i += DEPTH) round(i, std::true_type{});
  round(i, std::false_type{});
}

// One dot-decode unit: row tile rt of tile t, contracted by the S waves of
// the workgroup (this wave is split sw, streaming the contiguous K-blocks
// [sw*KB/S, (sw+1)*KB/S)).  Every thread of the workgroup stages the token
// rows.  The halves of a row are added lane l + lane l+32, then the S
// partial sums in split order, then the epilogue.
template <int QF, bool GATE_UP, int TT, int NPR, bool D16>
__device__ __forceinline__ void dot_unit(const GemmArgs& p, const Tile& t, int rt, int S, int sw, uint32_t* xs) {
  using SL = ScaleLayout<QF>;
  constexpr int DEPTH = dot_depth(TT, D16);
  const int tid = threadIdx.x, lane = tid & 63, nthr = blockDim.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = p.K, KB = K >> 6;
  const int kb0 = sw * KB / S, kb1 = (sw + 1) * KB / S, nkb = kb1 - kb0;
  const int row_u32 = K / 2 + 4;                              // staged row: K 16-bit inputs + 16 B pad
  float* xsum = reinterpret_cast<float*>(xs + TT * row_u32);  // [TT][K/32] (int4)

  const uint8_t* rec = p.slot_ptr[t.slot];
  const uint8_t* codes = rec + p.off_codes + ((int64_t)rt * KB + kb0) * kTileCodeBytes + lane * 16;
  // scale block of (absolute) k-block kb0 + kb is (kb0 + kb) >> sshift
  const uint8_t* scales =
      rec + p.off_scales + (int64_t)rt * (KB >> p.sshift) * SL::kTileBytes + SL::lane_off(lane);

  // activation loads first: waiting for them later leaves the weight loads
  // issued after them in flight
  u32x4 v[TT][NPR];
  dot_load_rows<TT, NPR>(p, t, tid, nthr, v);
  asm volatile("" ::: "memory");
  u32x4 wq[DEPTH];
  uint32_t ws[ring_scales(QF, DEPTH)];
  const uint8_t* codes0 = codes - lane * 16;         // the K range's first 16 bytes, every lane
  const uint8_t* scales0 = scales - SL::lane_off(lane);
  dot_prologue<QF, DEPTH>(wq, ws, codes, scales, codes0, scales0, kb0, nkb, p.sshift, lane);
  dot_store_rows<QF, TT, NPR>(v, xs, row_u32, xsum, tid, nthr, K);
  __syncthreads();

  float acc[TT];
#pragma unroll
  for (int r = 0; r < TT; ++r) acc[r] = 0.0f;
  dot_contract<QF, TT, DEPTH>(wq, ws, codes, scales, codes0, scales0, kb0, nkb, p.sshift, xs, row_u32, xsum, K,
                              lane, acc);

  // halves: lane l (< 32) adds lane l+32; then the S waves in order
  __syncthreads();  // staging area reused below
  float* red = reinterpret_cast<float*>(xs);  // [waves][TT][32]
#pragma unroll
  for (int r = 0; r < TT; ++r) {
    const float other = __shfl_down(acc[r], 32);
    if (lane < 32) red[(wave * TT + r) * 32 + lane] = acc[r] + other;
  }
  __syncthreads();
  const float2 gs = matrix_scales<QF>(p, rec);  // NVFP4 matrix scales, else 1
  for (int q = tid; q < TT * 32; q += nthr) {
    const int n = q >> 5, row = q & 31;  // (token, row)
    if (n >= t.nrows) continue;
    const ColExp ce = col_exp<QF, GATE_UP>(p, t.expert, t.row_begin + n);
    if constexpr (GATE_UP) {
      if (row >= 16) continue;
      float g = red[n * 32 + row], u = red[n * 32 + row + 16];
      for (int w = 1; w < S; ++w) {
        g += red[(w * TT + n) * 32 + row];
        u += red[(w * TT + n) * 32 + row + 16];
      }
      uint16_t* hp = reinterpret_cast<uint16_t*>(p.out);
      hp[(int64_t)(t.row_begin + n) * p.out_ld + rt * 16 + row] = h_elem<QF>(g, u, gs, ce);
    } else {
      float o = red[n * 32 + row];
      for (int w = 1; w < S; ++w) o += red[(w * TT + n) * 32 + row];
      reinterpret_cast<float*>(p.out)[(int64_t)(t.row_begin + n) * p.out_ld + rt * 32 + row] =
          o_elem<QF>(o, gs.x, ce);
    }
  }
}

// TT: the most token rows a tile of the launch can have (1, 2 or 4; the LDS
// is sized for it).  Each workgroup contracts as many rows as its own tile
// has, rounded up to 1, 2 or 4: with several tokens most experts still hold
// one of them, and a 1-row tile then stages, reads and multiplies one row
// instead of four.  A token's sums do not depend on the rows beside it.
template <int QF, bool GATE_UP, int TT, int NPR, bool D16>
__global__ __launch_bounds__(1024) void moe_decode_dot_kernel(GemmArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint32_t xs[];
  const int S = blockDim.x >> 6;
  const int nrt = p.N >> 5;
  const int rt = blockIdx.x % nrt, tile_i = blockIdx.x / nrt;
  const int n_tiles = p.n_tiles_dev ? p.n_tiles_dev[0] : p.n_tiles;
  if (tile_i >= n_tiles) return;  // the whole workgroup leaves together
  const Tile t = p.tiles[tile_i];
  // wave-uniform in scalar registers: the K range, its bounds checks and the
  // ring's branches are then scalar
  const int sw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if constexpr (TT >= 4) {
    if (t.nrows > 2) {
      dot_unit<QF, GATE_UP, 4, NPR, D16>(p, t, rt, S, sw, xs);
      return;
    }
  }
  if constexpr (TT >= 2) {
    if (t.nrows > 1) {
      dot_unit<QF, GATE_UP, 2, NPR, D16>(p, t, rt, S, sw, xs);
      return;
    }
  }
  dot_unit<QF, GATE_UP, 1, NPR, D16>(p, t, rt, S, sw, xs);
}

// ---------------------------------------------------------------------------
// Prefill kernel: persistent workgroups of 4 waves, two per CU.  A work item is
// (tile of up to 128 token rows of one expert, block of 8 weight row-tiles =
// 256 outputs, range of K when the down GEMM splits K).  Wave w owns row tiles
// 2w, 2w+1 of the block (64 outputs) and all of the tile's tokens (NCT column
// tiles of 32, a template parameter so the K loop has no branches).
//
// Every global load is a 16- or 4-byte LDS-DMA load (global memory straight
// into LDS, no registers) into a ring of stages, issued S - 1 K-blocks ahead:
// per K-block the tile's activations (shared by the four waves) and each
// wave's own weight codes and scales.  A stage holds NCT * 4 KB of
// activations and 9 KB of weights, so the 75 KB of a workgroup hold 3 stages
// of a full token tile but 4 (2 column tiles) or 5 (1) of a small one: the
// items of small experts, which stream a whole weight block for a few rows,
// keep more of it in flight.  The only vector-memory
// operations in the K loop are those DMA loads, so the wait before a K-block
// is a fixed count of them.  One barrier per K-block: after it the K-block's
// stage is complete for all waves and the stage read in the previous K-block
// is free for the next DMA.  Inside a K-block the B operands and decoded
// weights of the next MFMA step are read and decoded while the current step's
// MFMAs run.  Loads never branch: padding rows read a valid row of the tile,
// row tiles past N re-read the last row tile and K-blocks past the end
// re-read the last one; those results are not stored.
// ---------------------------------------------------------------------------
constexpr int kPreThreads = 256;
constexpr int kPreRowTilesPerWave = 2;
constexpr int kPreRowTilesPerItem = 8;
constexpr int kPreLdsBytes = 3 * 25 * 1024;  // per workgroup; two workgroups per CU
// Activation rows in LDS: 64 16-bit inputs = 128 bytes = 8 chunks of 16
// bytes, unpadded.  Chunk c of row r sits in slot c ^ f(r),
// f(r) = (r ^ (r >> 3)) & 7, so the 8 (or 16) consecutive rows that one
// ds_read_b128 pass serves fall in distinct 16-byte bank groups whether the
// LDS has 32 or 64 banks.
constexpr int kRowBytes = 128;
constexpr int kWaveWBytes = 2 * kTileCodeBytes + 256;       // codes of 2 row tiles + their scales
// activation bytes, stage bytes and stages of an item with NCT column tiles
// (every stage starts at a multiple of 1 KB, so the row swizzle below keeps
// its bank pattern in every stage)
constexpr int pre_act_bytes(int nct) { return nct * 32 * kRowBytes; }
constexpr int pre_stage_bytes(int nct) { return pre_act_bytes(nct) + 4 * kWaveWBytes; }
constexpr int pre_stages(int nct) { return kPreLdsBytes / pre_stage_bytes(nct) < 5 ? kPreLdsBytes / pre_stage_bytes(nct) : 5; }
static_assert(pre_stages(4) == 3 && pre_stages(3) == 3 && pre_stages(2) == 4 && pre_stages(1) == 5, "stages");
static_assert(pre_stage_bytes(1) % 1024 == 0 && pre_stage_bytes(2) % 1024 == 0 && pre_stage_bytes(3) % 1024 == 0 &&
                  pre_stage_bytes(4) % 1024 == 0,
              "stage alignment");

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt on vmcnt only (expcnt and lgkmcnt left at their maximum)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}
// wait until at most n * PER loads are in flight, n in [0, NMAX] wave-uniform
template <int PER, int NMAX>
__device__ __forceinline__ void wait_vm_groups(int n) {
  if constexpr (NMAX <= 0) {
    wait_vm<0>();
  } else {
    if (n >= NMAX) wait_vm<NMAX * PER>();
    else wait_vm_groups<PER, NMAX - 1>(n);
  }
}


// a row tile's scale word for this lane, from the tile's scale bytes in LDS
template <int QF>
__device__ __forceinline__ uint32_t lds_scale(const uint8_t* tile, int lane) {
  if constexpr (QF == Q_INT4)
    return *reinterpret_cast<const uint32_t*>(tile + (lane & 31) * 4);
  else if constexpr (QF == Q_NVFP4)
    return *reinterpret_cast<const uint16_t*>(tile + lane * 2);
  else
    return tile[lane];
}

// LDS-DMA loads of 16 and 4 bytes per lane: lane l's bytes land at
// lds + l * size (lds wave-uniform, in M0).  They are written as inline asm
// (with a memory clobber, so no memory access moves across them) because the
// compiler cannot tell a DMA into one stage from a read of another and would
// wait for every DMA before each LDS read; the waits for these loads are the
// explicit vmcnt waits of the K loop.  The asm has no register outputs.
__device__ __forceinline__ void dma16(const void* g, const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)lds);
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma4(const void* g, const void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)lds);
  asm volatile("global_load_lds_dword %0, off" : : "v"(g), "{m0}"(m0) : "memory");
}

template <int QF, bool GATE_UP, int NCT>
__device__ __forceinline__ void prefill_item(const GemmArgs& p, const Tile& t, int nb, int ks, uint8_t* lds) {
  constexpr int S = pre_stages(NCT);
  constexpr int SB = pre_stage_bytes(NCT);
  constexpr int kActBytes = pre_act_bytes(NCT);
  auto stage = [&](auto stc) -> uint8_t* { return lds + decltype(stc)::value * SB; };
  using SL = ScaleLayout<QF>;
  constexpr int RTW = kPreRowTilesPerWave;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nrt = p.N >> 5;
  // this item's K range: k-blocks [kb0, kb0 + KB) (the whole K unless split)
  const int KB = (p.K >> 6) / p.ksplit;
  const int kb0 = ks * KB;
  const int rt0 = nb * kPreRowTilesPerItem + wave * RTW;

  // Activation DMA: load q of wave w fills rows 8j .. 8j+7 (j = 4q + w) of
  // the stage, 1 KB: lane l writes slot l & 7 of row 8j + (l >> 3), which
  // holds chunk (l & 7) ^ f(row) of that row.  Rows past the tile's end
  // re-read the tile's first row.
  const uint16_t* a_src[NCT];
#pragma unroll
  for (int q = 0; q < NCT; ++q) {
    const int j = 4 * q + wave;
    const int r = 8 * j + (lane >> 3);
    const int chunk = (lane & 7) ^ (lane >> 3) ^ (j & 7);
    const int srow = (r < t.nrows) ? r : 0;
    const int64_t gr = p.gather ? p.gather[t.row_begin + srow] : (t.row_begin + srow);
    a_src[q] = reinterpret_cast<const uint16_t*>(p.act) + gr * p.K + kb0 * 64 + chunk * 8;
  }
  // Weight DMA: row tile r's 1 KB code chunk (lane l: bytes 16l..16l+15) and
  // one dword per lane of the two row tiles' scale bytes: int4 and NVFP4
  // (128 bytes per tile) lanes 0-31 tile 0, 32-63 tile 1; MXFP4 (64 bytes)
  // lanes 0-15 tile 0, 16-31 tile 1, 32-63 repeat 0-31.
  const uint8_t* rec = p.slot_ptr[t.slot];
  const int kbt = p.K >> 6;  // k-blocks per row tile in the record
  const uint8_t* c_src[RTW];
#pragma unroll
  for (int r = 0; r < RTW; ++r) {
    const int rtl = min(rt0 + r, nrt - 1);
    c_src[r] = rec + p.off_codes + ((int64_t)rtl * kbt + kb0) * kTileCodeBytes + lane * 16;
  }
  const uint8_t* sc_src;
  {
    constexpr int TB = SL::kTileBytes;  // 128 or 64
    const int r = (TB == 128) ? (lane >> 5) : ((lane >> 4) & 1);
    const int off = (TB == 128) ? (lane & 31) * 4 : (lane & 15) * 4;
    const int rtl = min(rt0 + r, nrt - 1);
    // kb0 is a multiple of the scale block (1 << sshift k-blocks)
    sc_src = rec + p.off_scales + ((int64_t)rtl * (kbt >> p.sshift) + (kb0 >> p.sshift)) * TB + off;
  }
  // B-operand reads: lane reads row ct*32 + (lane & 31), chunk 4*(lane >> 5) + st
  const int key = (lane & 7) ^ ((lane >> 3) & 3);
  const int rd_base = (lane & 31) * kRowBytes;
  const int rd_hi = (lane >> 5) ^ (key >> 2);

  f32x16 acc[RTW][NCT];
#pragma unroll
  for (int a = 0; a < RTW; ++a)
#pragma unroll
    for (int b = 0; b < NCT; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  auto dma = [&](auto stc, int kb) {
    uint8_t* st = stage(stc);
    kb = min(kb, KB - 1);
#pragma unroll
    for (int q = 0; q < NCT; ++q) dma16(a_src[q] + kb * 64, st + (4 * q + wave) * 8 * kRowBytes);
    uint8_t* wst = st + kActBytes + wave * kWaveWBytes;
#pragma unroll
    for (int r = 0; r < RTW; ++r) dma16(c_src[r] + (int64_t)kb * kTileCodeBytes, wst + r * kTileCodeBytes);
    dma4(sc_src + (int64_t)(kb >> p.sshift) * SL::kTileBytes, wst + RTW * kTileCodeBytes);
  };
  // One K-block from stage ST; `issue` (the DMA of a later K-block) runs
  // once the first LDS reads are in flight.
  auto compute = [&](auto stc, auto&& issue) {
    const uint8_t* st = stage(stc);
    const uint8_t* wst = st + kActBytes + wave * kWaveWBytes;
    auto read_b = [&](int stp, u32x4(&b)[NCT]) {
      const int slot_lo = (stp ^ key) & 3;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const int slot = slot_lo | ((rd_hi ^ (ct & 1)) << 2);
        b[ct] = *reinterpret_cast<const u32x4*>(st + ct * 32 * kRowBytes + rd_base + slot * 16);
      }
    };
    u32x4 q4[RTW];
    uint32_t s4[RTW];
#pragma unroll
    for (int r = 0; r < RTW; ++r) {
      q4[r] = *reinterpret_cast<const u32x4*>(wst + r * kTileCodeBytes + lane * 16);
      s4[r] = lds_scale<QF>(wst + RTW * kTileCodeBytes + r * SL::kTileBytes, lane);
    }
    u32x4 b0[NCT];
    read_b(0, b0);
    issue();
    u32x4 a[RTW];
#pragma unroll
    for (int r = 0; r < RTW; ++r) a[r] = ChunkScale<QF>(s4[r]).step(q4[r][0], 0);
#pragma unroll
    for (int stp = 0; stp < 4; ++stp) {
      u32x4 b[NCT];
      if (stp == 0) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) b[ct] = b0[ct];
      } else {
        read_b(stp, b);
      }
      u32x4 an[RTW];
      if (stp < 3) {
#pragma unroll
        for (int r = 0; r < RTW; ++r) an[r] = ChunkScale<QF>(s4[r]).step(q4[r][stp + 1], stp + 1);
      }
#pragma unroll
      for (int r = 0; r < RTW; ++r)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) acc[r][ct] = mfma<QF>(a[r], b[ct], acc[r][ct]);
      if (stp < 3) {
#pragma unroll
        for (int r = 0; r < RTW; ++r) a[r] = an[r];
      }
    }
  };
  // Step kb: wait for this wave's DMA of K-block kb (the loads of the
  // K-blocks after it, up to S - 2 of them, may still be in flight), barrier
  // (every wave's DMA of kb is in LDS; every wave is done with stage kb - 1),
  // compute K-block kb, issuing the DMA of K-block kb + S - 1 into stage
  // kb - 1 after its first reads.  No DMA is issued past the last K-block;
  // the waits of the last steps count only the loads that were issued.
  constexpr int kPerStep = NCT + RTW + 1;
  static_assert((S - 2) * kPerStep < 64, "vmcnt range");
  auto one_step = [&](int kb, auto uc) {
    constexpr int U = decltype(uc)::value;  // kb % S
    wait_vm_groups<kPerStep, S - 2>(KB - 1 - kb);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    compute(std::integral_constant<int, U>{}, [&] {
      if (kb + S - 1 < KB) dma(std::integral_constant<int, (U + S - 1) % S>{}, kb + S - 1);
    });
    __builtin_amdgcn_sched_barrier(0);
  };

  // Epilogue operands, loaded ahead of the K loop (older than every DMA, so
  // the loop's counted waits cover them): each column's token, the expert's
  // weight exponents and the NVFP4 matrix scales.  The epilogue then waits
  // for one dependent load (the tokens' exponents), not for a chain of loads
  // per row tile and column tile, each behind the h stores before it (the
  // memory counter counts stores too).
  int tok[NCT] = {};
  if constexpr (QF != Q_MXFP4) {
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int mm = min(ct * 32 + (lane & 31), t.nrows - 1);  // columns past the tile: a valid row
      tok[ct] = p.tok_of_row[t.row_begin + mm];
    }
  }
  const ColExpPre cpre = col_exp_pre<QF, GATE_UP>(p, t.expert);
  const float2 gs = matrix_scales<QF>(p, rec);

  [&]<int... I>(std::integer_sequence<int, I...>) {
    ((I < KB ? dma(std::integral_constant<int, I>{}, I) : void()), ...);
  }(std::make_integer_sequence<int, S - 1>{});
  int kb = 0;
  for (; kb + S <= KB; kb += S) {
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (one_step(kb + I, std::integral_constant<int, I>{}), ...);
    }(std::make_integer_sequence<int, S>{});
  }
  [&]<int... I>(std::integer_sequence<int, I...>) {
    ((kb + I < KB ? one_step(kb + I, std::integral_constant<int, I>{}) : void()), ...);
  }(std::make_integer_sequence<int, S - 1>{});
  // no DMA may still be writing LDS when the next item starts
  wait_vm<0>();

  // epilogue (NVFP4: times the fp32 matrix scales)
  ColExp ce_ct[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) ce_ct[ct] = col_exp_post<QF, GATE_UP>(p, cpre, tok[ct]);
#pragma unroll
  for (int r = 0; r < RTW; ++r) {
    const int rt = rt0 + r;
    if (rt >= nrt) continue;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int mm = ct * 32 + (lane & 31);
      if (mm >= t.nrows) continue;
      const int64_t row = t.row_begin + mm;
      const ColExp& ce = ce_ct[ct];
      if constexpr (GATE_UP) {
        uint16_t* h = reinterpret_cast<uint16_t*>(p.out) + row * p.out_ld + rt * 16;
#pragma unroll
        for (int g4 = 0; g4 < 2; ++g4) {
          uint16_t v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int i = g4 * 4 + q;
            v[q] = h_elem<QF>(acc[r][ct][i], acc[r][ct][i + 8], gs, ce);
          }
          const uint2 pk = {(uint32_t)v[0] | ((uint32_t)v[1] << 16),
                            (uint32_t)v[2] | ((uint32_t)v[3] << 16)};
          *reinterpret_cast<uint2*>(h + g4 * 8 + (lane >> 5) * 4) = pk;
        }
      } else {
        float* o = reinterpret_cast<float*>(p.out) + ks * p.split_stride + row * p.out_ld + rt * 32;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 v = {o_elem<QF>(acc[r][ct][g4 * 4 + 0], gs.x, ce), o_elem<QF>(acc[r][ct][g4 * 4 + 1], gs.x, ce),
                            o_elem<QF>(acc[r][ct][g4 * 4 + 2], gs.x, ce), o_elem<QF>(acc[r][ct][g4 * 4 + 3], gs.x, ce)};
          *reinterpret_cast<float4*>(o + g4 * 8 + (lane >> 5) * 4) = v;
        }
      }
    }
  }
}

template <int QF, bool GATE_UP>
__global__ __launch_bounds__(kPreThreads, 2) void moe_prefill_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kPreLdsBytes];
  const int nrt = p.N >> 5;
  const int n_nb = (nrt + kPreRowTilesPerItem - 1) / kPreRowTilesPerItem;
  const int n_tiles = p.n_tiles_dev ? p.n_tiles_dev[0] : p.n_tiles;
  const int per_tile = n_nb * p.ksplit;
  const int n_items = n_tiles * per_tile;
  // Consecutive workgroups are dispatched to the 8 XCDs in turn, so those
  // with equal blockIdx % 8 share an XCD and its L2.  With few items per
  // tile (at most 16 row blocks and K ranges) the tiles of the list are dealt
  // to the XCDs in a snake order (0..7, 7..0, ...), which keeps the work of
  // the XCDs even under the heaviest-first list, and all the items of a tile
  // (which read the same activations) run on the same XCD, about at the same
  // time: each XCD's workgroups take its items in turn.  With more (a wide
  // expert: its row blocks are the bulk of the bytes) the items go out in
  // list order, which puts the same row block of an expert's consecutive
  // tiles on one XCD when per_tile is a multiple of 8; so do launches with
  // no more items than workgroups (one item each, whatever the XCD).
  const int G = gridDim.x;
  const bool by_xcd = G % 8 == 0 && G > 8 && per_tile <= 16 && n_items > G;
  const int x = blockIdx.x & 7, gx = by_xcd ? G >> 3 : G;
  const int n_local = by_xcd ? ((n_tiles + 7) >> 3) * per_tile : n_items;  // XCD: rounds of 8 tiles
  for (int i = by_xcd ? (blockIdx.x >> 3) : blockIdx.x; i < n_local; i += gx) {
    int item = i;
    if (by_xcd) {
      const int r = (i / per_tile);  // this XCD's r-th tile: list tile 8r + x or 8r + 7 - x
      const int tl = 8 * r + ((r & 1) ? 7 - x : x);
      if (tl >= n_tiles) continue;
      item = tl * per_tile + i % per_tile;
    }
    const Tile t = p.tiles[item / per_tile];
    const int rem = item % per_tile;
    const int nb = rem / p.ksplit, ks = rem % p.ksplit;
    switch ((t.nrows + 31) >> 5) {
      case 1: prefill_item<QF, GATE_UP, 1>(p, t, nb, ks, lds); break;
      case 2: prefill_item<QF, GATE_UP, 2>(p, t, nb, ks, lds); break;
      case 3: prefill_item<QF, GATE_UP, 3>(p, t, nb, ks, lds); break;
      default: prefill_item<QF, GATE_UP, 4>(p, t, nb, ks, lds); break;
    }
    __syncthreads();
  }
}

#ifndef STRATA_DECODE_UNIT
// ---------------------------------------------------------------------------
// Page-in: copies whole records (b.stride bytes each) from the pinned host
// store, read through its device mapping, into device slots.  The work is cut
// into 4 KB chunks (a workgroup's 256 lanes x 16 bytes); each of 64
// workgroups keeps four chunks of loads in flight (1 MB in all), which runs
// the host link at its full rate.  The kernel stays at 28 VGPRs so that one
// of its waves fits on a SIMD beside two prefill waves (2 x 232 or 2 x 240 of
// 512): with eight chunks in flight it needed 52, and the CUs it ran on then
// held one prefill workgroup instead of two, which delayed part of the
// persistent prefill grid (2-4% longer paged steps on the larger layers).
// Host reads are non-temporal.
// ---------------------------------------------------------------------------
constexpr int kPageThreads = 256;
constexpr int kPageUnroll = 4;
constexpr int kPageGrid = 64;

__global__ __launch_bounds__(kPageThreads) void page_in_kernel(PageBatch b) {
  const int per_rec = (int)((b.stride + 4095) >> 12);  // chunks per record
  const int total = per_rec * b.n;
  for (int c0 = blockIdx.x * kPageUnroll; c0 < total; c0 += gridDim.x * kPageUnroll) {
    u32x4 v[kPageUnroll];
#pragma unroll
    for (int u = 0; u < kPageUnroll; ++u) {
      const int c = c0 + u;
      const int r = c / per_rec;
      const int64_t off = (int64_t)(c - r * per_rec) * 4096 + threadIdx.x * 16;
      if (c < total && off < b.stride) v[u] = ld16_nt(b.src + (int64_t)b.expert[r] * b.stride + off);
    }
#pragma unroll
    for (int u = 0; u < kPageUnroll; ++u) {
      const int c = c0 + u;
      const int r = c / per_rec;
      const int64_t off = (int64_t)(c - r * per_rec) * 4096 + threadIdx.x * 16;
      if (c < total && off < b.stride) *reinterpret_cast<u32x4*>(b.slot_ptr[b.slot[r]] + off) = v[u];
    }
  }
}

hipError_t launch_page_in(const PageBatch& b, hipStream_t s) {
  if (b.n <= 0) return hipSuccess;
  const int per_rec = (int)((b.stride + 4095) >> 12);
  const int grid = std::min(kPageGrid, (per_rec * b.n + kPageUnroll - 1) / kPageUnroll);
  page_in_kernel<<<grid, kPageThreads, 0, s>>>(b);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine: y[t] = sum_j w[t,j] * o[pos[t,j]] (j ascending) + g_t o[shared row of t],
// fp32, rounded to bf16 (nearest-even); g_t = sigmoid(gate logit of t) for a
// layer with a shared-expert gate, else 1 (added without a multiply).  One workgroup per (token, block of
// 1024 columns); each thread owns 4 consecutive columns.  With a K-split
// prefill down GEMM each o row is the sum of its partial planes, in plane
// order, before it is weighted.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float4 o_row(const float* __restrict__ o, size_t at, int ksplit,
                                        int64_t stride) {
  float4 v = *reinterpret_cast<const float4*>(o + at);
  for (int s = 1; s < ksplit; ++s) {
    const float4 q = *reinterpret_cast<const float4*>(o + s * stride + at);
    v.x += q.x;
    v.y += q.y;
    v.z += q.z;
    v.w += q.w;
  }
  return v;
}

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o,
                                                      const int32_t* __restrict__ pos,
                                                      const float* __restrict__ w, int k, int H,
                                                      int shared_row0, int ksplit, int64_t stride,
                                                      const float* __restrict__ gate,
                                                      uint16_t* __restrict__ y) {
  const int t = blockIdx.x;
  // the shared expert's weight: sigmoid of its gate logit, or 1 without a gate
  const float gw = gate ? __builtin_amdgcn_rcpf(1.0f + __expf(-gate[t])) : 1.0f;
  // workgroup (t, blockIdx.y) takes column blocks of 1024, gridDim.y apart
  for (int c = blockIdx.y * 1024 + threadIdx.x * 4; c < H; c += gridDim.y * 1024) {
    float4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    // experts in rounds of eight: a round's rows are all requested before
    // the first is added (in the order j = 0, 1, ...; slots past k re-read
    // the last row and are not added)
    constexpr int RJ = 8;
    for (int j0 = 0; j0 < k; j0 += RJ) {
      float wj[RJ];
      float4 v[RJ];
#pragma unroll
      for (int u = 0; u < RJ; ++u) {
        const int j = min(j0 + u, k - 1);
        wj[u] = w[(size_t)t * k + j];
        v[u] = o_row(o, (size_t)pos[(size_t)t * k + j] * H + c, ksplit, stride);
      }
#pragma unroll
      for (int u = 0; u < RJ; ++u) {
        if (j0 + u >= k) break;
        acc.x = __builtin_fmaf(wj[u], v[u].x, acc.x);
        acc.y = __builtin_fmaf(wj[u], v[u].y, acc.y);
        acc.z = __builtin_fmaf(wj[u], v[u].z, acc.z);
        acc.w = __builtin_fmaf(wj[u], v[u].w, acc.w);
      }
    }
    if (shared_row0 >= 0) {
      const float4 v = o_row(o, (size_t)(shared_row0 + t) * H + c, ksplit, stride);
      if (gate) {
        acc.x = __builtin_fmaf(gw, v.x, acc.x);
        acc.y = __builtin_fmaf(gw, v.y, acc.y);
        acc.z = __builtin_fmaf(gw, v.z, acc.z);
        acc.w = __builtin_fmaf(gw, v.w, acc.w);
      } else {
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
      }
    }
    const uint2 pk = {(uint32_t)f32_to_bf16_rne(acc.x) | ((uint32_t)f32_to_bf16_rne(acc.y) << 16),
                      (uint32_t)f32_to_bf16_rne(acc.z) | ((uint32_t)f32_to_bf16_rne(acc.w) << 16)};
    *reinterpret_cast<uint2*>(y + (size_t)t * H + c) = pk;
  }
}

#endif  // !STRATA_DECODE_UNIT

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
// Dispatch over the quant family and gate+up / down at run time.
template <template <int, bool> class L, class... A>
static void by_format(int quant, bool gate_up, A&&... args) {
  if (quant == Q_INT4) {
    if (gate_up) L<Q_INT4, true>::run(args...); else L<Q_INT4, false>::run(args...);
  } else if (quant == Q_NVFP4) {
    if (gate_up) L<Q_NVFP4, true>::run(args...); else L<Q_NVFP4, false>::run(args...);
  } else {
    if (gate_up) L<Q_MXFP4, true>::run(args...); else L<Q_MXFP4, false>::run(args...);
  }
}

#ifdef STRATA_DECODE_UNIT
template <int QF, bool GATE_UP>
static void launch_decode(const GemmArgs& a, int T, int log2S, int grid, hipStream_t s) {
  const int S = 1 << log2S;
  const size_t lds = std::max<size_t>((size_t)T * (S * kDecDepth * 128 + 16),
                                      (size_t)kDecWaves * kDecodeMaxT * 32 * 4);
  const int np = (T * S * 64 + kDecWaves * 64 - 1) / (kDecWaves * 64);
  if (np <= 1)
    launch_k(moe_decode_kernel<QF, GATE_UP, 1>, dim3(grid), dim3(kDecWaves * 64), lds, s, a, log2S);
  else if (np <= 2)
    launch_k(moe_decode_kernel<QF, GATE_UP, 2>, dim3(grid), dim3(kDecWaves * 64), lds, s, a, log2S);
  else
    launch_k(moe_decode_kernel<QF, GATE_UP, 4>, dim3(grid), dim3(kDecWaves * 64), lds, s, a, log2S);
}

// Decode split: waves per row tile, log2.  Enough waves for about 16 per CU
// at one token (k + S expert tiles), at least 4 K-blocks per wave, and at
// most 8 splits; 8 tokens allow at most 4 (LDS and staging registers).
// Depends only on the layer shape and the token count.
int decode_log2_splits(int N, int K, int tiles_per_token, int T) {
  const int KB = K / 64, units = tiles_per_token * (N / 32);
  int l = 0;
  while (l < 3 && (units << (l + 1)) <= 4096 && KB / (2 << l) >= 4) ++l;
  while (T * (1 << l) > 32) --l;
  return l;
}

int decode_grid(int N, int log2S, int n_tiles) {
  const int R = kDecWaves >> log2S;
  return n_tiles * ((N / 32 + R - 1) / R);
}

// Dot decode eligibility and split for an N x K weight at T tokens: waves per
// row tile (1..16), 16-byte staging pieces per thread per row (<= 4), and the
// LDS the staged rows need (<= 64 KB).  Returns 0 if the MFMA kernel is to be
// used instead.  Depends only on the layer shape and T.  The split doubles
// while each wave keeps a full ring of 16 K-blocks and the launch stays within
// 8,192 waves, or, up to 4 splits, while each wave keeps 8 K-blocks and the
// launch stays within 4,096 waves (small layers: shorter serial K loops).
int decode_dot_waves(int N, int K, int quant, int tiles_per_token, int T) {
  if (T > kDecodeMaxT) return 0;  // above 4 tokens the tiles hold at most 4 rows
  const int TT = T <= 1 ? 1 : (T <= 2 ? 2 : 4);
  const int KB = K / 64, units = tiles_per_token * (N / 32);
  int S = 1;
  while (S < 16) {
    const int per_wave = KB / (2 * S), waves = units * 2 * S;
    const bool full_ring = per_wave >= 16 && waves <= 8192;
    const bool short_loop = per_wave >= 8 && waves <= 4096 && 2 * S <= 4;
    if (!full_ring && !short_loop) break;
    S *= 2;
  }
  while (S < 16 && (K / 8 + 64 * S - 1) / (64 * S) > 4) S *= 2;
  if ((K / 8 + 64 * S - 1) / (64 * S) > 4) return 0;
  const size_t lds = (size_t)TT * (K * 2 + 16) + (quant == Q_INT4 ? (size_t)TT * (K / 32) * 4 : 0);
  if (lds > 64 * 1024) return 0;
  return S;
}

template <int QF, bool GATE_UP, int TT, bool D16>
static void launch_dot_d(const GemmArgs& a, int S, int grid, size_t lds, hipStream_t s) {
  const int npr = (a.K / 8 + 64 * S - 1) / (64 * S);
  if (npr <= 1)
    launch_k(moe_decode_dot_kernel<QF, GATE_UP, TT, 1, D16>, dim3(grid), dim3(64 * S), lds, s, a);
  else if (npr <= 2)
    launch_k(moe_decode_dot_kernel<QF, GATE_UP, TT, 2, D16>, dim3(grid), dim3(64 * S), lds, s, a);
  else
    launch_k(moe_decode_dot_kernel<QF, GATE_UP, TT, 4, D16>, dim3(grid), dim3(64 * S), lds, s, a);
}

// true when every wave's K range (split sw of S: blocks sw*KB/S .. (sw+1)*KB/S - 1)
// is a nonzero multiple of 16 K-blocks
static bool ranges_of_16(int KB, int S) {
  for (int sw = 0; sw < S; ++sw) {
    const int n = (sw + 1) * KB / S - sw * KB / S;
    if (n == 0 || n % 16) return false;
  }
  return true;
}

template <int QF, bool GATE_UP, int TT>
static void launch_dot_tt(const GemmArgs& a, int S, int grid, size_t lds, hipStream_t s) {
  if (ranges_of_16(a.K / 64, S))
    launch_dot_d<QF, GATE_UP, TT, true>(a, S, grid, lds, s);
  else
    launch_dot_d<QF, GATE_UP, TT, false>(a, S, grid, lds, s);
}

template <int QF, bool GATE_UP>
static void launch_dot(const GemmArgs& a, int T, int S, int n_tiles, hipStream_t s) {
  const int TT = T <= 1 ? 1 : (T <= 2 ? 2 : 4);
  size_t lds = (size_t)TT * (a.K * 2 + 16) + (QF == Q_INT4 ? (size_t)TT * (a.K / 32) * 4 : 0);
  lds = std::max(lds, (size_t)S * TT * 32 * 4);
  const int grid = n_tiles * (a.N / 32);
  if (TT == 1)
    launch_dot_tt<QF, GATE_UP, 1>(a, S, grid, lds, s);
  else if (TT == 2)
    launch_dot_tt<QF, GATE_UP, 2>(a, S, grid, lds, s);
  else
    launch_dot_tt<QF, GATE_UP, 4>(a, S, grid, lds, s);
}

template <int QF, bool GU>
struct DotL {
  static void run(const GemmArgs& a, int T, int S, int n_tiles, hipStream_t s) { launch_dot<QF, GU>(a, T, S, n_tiles, s); }
};
template <int QF, bool GU>
struct DecL {
  static void run(const GemmArgs& a, int T, int log2S, int grid, hipStream_t s) {
    launch_decode<QF, GU>(a, T, log2S, grid, s);
  }
};
hipError_t launch_decode_dot(const GemmArgs& a, int quant, bool gate_up, int T, int S, int n_tiles,
                             hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  by_format<DotL>(quant, gate_up, a, T, S, n_tiles, s);
  return hipGetLastError();
}

hipError_t launch_decode_mfma(const GemmArgs& a, int quant, bool gate_up, int T, int log2S, int grid,
                              hipStream_t s) {
  by_format<DecL>(quant, gate_up, a, T, log2S, grid, s);
  return hipGetLastError();
}
#else   // the main unit: prefill, page-in, combine
hipError_t launch_decode_mfma(const GemmArgs& a, int quant, bool gate_up, int T, int log2S, int grid,
                              hipStream_t s);

template <int QF, bool GU>
struct PreL {
  static void run(const GemmArgs& a, int grid, hipStream_t s) {
    launch_k(moe_prefill_kernel<QF, GU>, dim3(grid), dim3(kPreThreads), 0, s, a);
  }
};

hipError_t launch_expert_gemm(const GemmArgs& a, int quant, bool gate_up, bool decode, int T, int log2S,
                              int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (decode) return launch_decode_mfma(a, quant, gate_up, T, log2S, grid, s);
  by_format<PreL>(quant, gate_up, a, grid, s);
  return hipGetLastError();
}

hipError_t launch_combine(const float* o, const int32_t* pos, const float* w, int T, int k, int H,
                          int shared_row0, int ksplit, int64_t stride, const float* gate, uint16_t* y,
                          hipStream_t s) {
  // one workgroup per (token, 1024 columns): a decode token's columns are
  // read in parallel rather than in dependent rounds of one workgroup
  launch_k(combine_kernel, dim3(T, (H + 1023) / 1024), dim3(256), 0, s, o, pos, w, k, H, shared_row0, ksplit,
           stride, gate, y);
  return hipGetLastError();
}
#endif  // STRATA_DECODE_UNIT

}  // namespace strata
