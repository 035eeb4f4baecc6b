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
// are converted bf16 -> fp16 (exact in range).  MXFP4 weights are decoded to
// bf16 with the gfx950 scaled FP4 conversion (exact: an E2M1 value times a
// power of two).  Accumulation is fp32 throughout; nothing uses float atomics,
// so every expert's result depends only on its own rows and weights.
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

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// --- decode of one 16-byte code chunk into four MFMA A operands ------------
// int4: the prepack stores each 32-bit word's nibbles as k0 k2 k4 k6 k1 k3 k5 k7
// (low to high), so (w >> 4j) & 0x000F000F holds the pair (k_2j, k_2j+1) in the
// two fp16 halves; OR-ing 0x6400 makes them 1024 + q exactly; subtracting 1024
// gives q, and one fp16 fma gives s*q + b.
__device__ __forceinline__ void dequant_int4(const u32x4& c, uint32_t sb, u32x4 (&a)[4]) {
  const _Float16 s = (_Float16)__uint_as_float(sb << 16);
  const _Float16 b = (_Float16)__uint_as_float(sb & 0xffff0000u);
  const f16x2 s2 = {s, s}, b2 = {b, b};
  const f16x2 k1024 = {(_Float16)1024.0f, (_Float16)1024.0f};
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const uint32_t w = c[st];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = ((w >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
      f16x2 h = bitcast<f16x2>(v) - k1024;
      h = __builtin_elementwise_fma(h, s2, b2);
      a[st][j] = bitcast<uint32_t>(h);
    }
  }
}

// MXFP4: byte i of a word holds elements 2i (low nibble) and 2i+1; the scale
// is the E8M0 exponent as an fp32 power of two.
__device__ __forceinline__ void dequant_fp4(const u32x4& c, uint32_t e8m0, u32x4 (&a)[4]) {
  const float scale = __uint_as_float(e8m0 << 23);
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const uint32_t w = c[st];
    a[st][0] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
    a[st][1] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
    a[st][2] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
    a[st][3] = bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  }
}

template <int QF>
__device__ __forceinline__ void dequant(const u32x4& c, uint32_t sc, u32x4 (&a)[4]) {
  if constexpr (QF == Q_INT4)
    dequant_int4(c, sc, a);
  else
    dequant_fp4(c, sc, a);
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
      return *reinterpret_cast<const uint32_t*>(p);
    else
      return *p;
  }
};

// bf16x8 -> f16x8 (exact for |x| in the fp16 normal range)
__device__ __forceinline__ u32x4 bf16_to_f16_8(const u32x4& v) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = {(_Float16)__uint_as_float(v[i] << 16),
                     (_Float16)__uint_as_float(v[i] & 0xffff0000u)};
    r[i] = bitcast<uint32_t>(h);
  }
  return r;
}

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
  constexpr bool kCvt = (QF == Q_INT4) && GATE_UP;
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
          const u32x4 b = kCvt ? bf16_to_f16_8(xa[u][st]) : xa[u][st];
          acc = mfma<QF>(a[st], b, acc);
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
// Prefill kernel: persistent workgroups of 4 waves.  A work item is (tile of up
// to 128 token rows of one expert, block of 8 weight row-tiles = 256 outputs).
// Wave w owns row tiles 2w, 2w+1 of the block and all 128 tokens (4 column
// tiles, skipped beyond the tile's rows).  Per K-block of 64 inputs the
// workgroup stages the 128 x 64 activation tile in LDS (double buffered,
// 16-byte chunks XOR-swizzled by row) while each wave decodes its weight
// chunks straight from global memory into MFMA operands.
// ---------------------------------------------------------------------------
constexpr int kPreThreads = 256;
constexpr int kPreRowTilesPerWave = 2;
constexpr int kPreRowTilesPerItem = 8;

template <int QF, bool GATE_UP>
__global__ __launch_bounds__(kPreThreads, 2) void moe_prefill_kernel(GemmArgs p) {
  using SL = ScaleLayout<QF>;
  constexpr bool kCvt = (QF == Q_INT4) && GATE_UP;
  constexpr int kRowU32 = kTileK / 2;  // 64 16-bit elements = 32 u32 per LDS row
  __shared__ __attribute__((aligned(16))) uint32_t lds[2][kPrefillTM * kRowU32];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nrt = p.N >> 5;
  const int n_nb = (nrt + kPreRowTilesPerItem - 1) / kPreRowTilesPerItem;
  const int n_tiles = p.n_tiles_dev ? p.n_tiles_dev[0] : p.n_tiles;
  const int n_items = n_tiles * n_nb;
  const int KB = p.K >> 6;
  const int sr = threadIdx.x >> 1, sh = threadIdx.x & 1;  // staging row / half

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const Tile t = p.tiles[item / n_nb];
    const int nb = item % n_nb;
    const int n_ct = (t.nrows + 31) >> 5;
    const int rtA = nb * kPreRowTilesPerItem + wave * kPreRowTilesPerWave;
    const bool okA = rtA < nrt, okB = rtA + 1 < nrt;

    const bool s_valid = sr < t.nrows;
    int64_t s_row = 0;
    if (s_valid) s_row = p.gather ? p.gather[t.row_begin + sr] : (t.row_begin + sr);
    const uint16_t* s_src = reinterpret_cast<const uint16_t*>(p.act) + s_row * p.K + sh * 32;

    const uint8_t* rec = p.slot_ptr[t.slot];
    const uint8_t* codesA = rec + p.off_codes + (int64_t)rtA * KB * kTileCodeBytes + lane * 16;
    const uint8_t* codesB = codesA + (int64_t)KB * kTileCodeBytes;
    const uint8_t* scA = rec + p.off_scales + (int64_t)rtA * KB * SL::kTileBytes + SL::lane_off(lane);
    const uint8_t* scB = scA + (int64_t)KB * SL::kTileBytes;

    f32x16 acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

    u32x4 sv[4];
    auto stage_load = [&](int kb) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (s_valid) v = ld16(s_src + kb * 64 + q * 8);
        sv[q] = v;
      }
    };
    auto stage_store = [&](int buf) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = sh * 4 + q;
        const int pc = c ^ (sr & 7);
        const u32x4 v = kCvt ? bf16_to_f16_8(sv[q]) : sv[q];
        *reinterpret_cast<u32x4*>(&lds[buf][sr * kRowU32 + pc * 4]) = v;
      }
    };
    u32x4 wA = {0u, 0u, 0u, 0u}, wB = {0u, 0u, 0u, 0u};
    uint32_t sA = 0, sB = 0;
    auto w_load = [&](int kb) {
      if (okA) {
        wA = ld16(codesA + (int64_t)kb * kTileCodeBytes);
        sA = SL::load(scA + (int64_t)kb * SL::kTileBytes);
      }
      if (okB) {
        wB = ld16(codesB + (int64_t)kb * kTileCodeBytes);
        sB = SL::load(scB + (int64_t)kb * SL::kTileBytes);
      }
    };

    stage_load(0);
    w_load(0);
    stage_store(0);
    __syncthreads();

    for (int kb = 0; kb < KB; ++kb) {
      const int cur = kb & 1;
      u32x4 aA[4], aB[4];
      if (okA) dequant<QF>(wA, sA, aA);
      if (okB) dequant<QF>(wB, sB, aB);
      if (kb + 1 < KB) {
        stage_load(kb + 1);
        w_load(kb + 1);
      }
      if (okA) {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          if (ct < n_ct) {
            const int mrow = ct * 32 + (lane & 31);
#pragma unroll
            for (int st = 0; st < 4; ++st) {
              const int c = 4 * (lane >> 5) + st;
              const u32x4 b =
                  *reinterpret_cast<const u32x4*>(&lds[cur][mrow * kRowU32 + ((c ^ (mrow & 7)) * 4)]);
              acc[0][ct] = mfma<QF>(aA[st], b, acc[0][ct]);
              if (okB) acc[1][ct] = mfma<QF>(aB[st], b, acc[1][ct]);
            }
          }
        }
      }
      if (kb + 1 < KB) stage_store(cur ^ 1);
      __syncthreads();
    }

    // epilogue
#pragma unroll
    for (int which = 0; which < 2; ++which) {
      const int rt = rtA + which;
      if (rt >= nrt) continue;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const int mm = ct * 32 + (lane & 31);
        if (ct >= n_ct || mm >= t.nrows) continue;
        const int64_t row = t.row_begin + mm;
        if constexpr (GATE_UP) {
          uint16_t* h = reinterpret_cast<uint16_t*>(p.out) + row * p.out_ld + rt * 16;
#pragma unroll
          for (int g4 = 0; g4 < 2; ++g4) {
            uint16_t v[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int i = g4 * 4 + q;
              v[q] = to_h_elem<QF>(silu(acc[which][ct][i]) * acc[which][ct][i + 8]);
            }
            const uint2 pk = {(uint32_t)v[0] | ((uint32_t)v[1] << 16),
                              (uint32_t)v[2] | ((uint32_t)v[3] << 16)};
            *reinterpret_cast<uint2*>(h + g4 * 8 + (lane >> 5) * 4) = pk;
          }
        } else {
          float* o = reinterpret_cast<float*>(p.out) + row * p.out_ld + rt * 32;
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const float4 v = {acc[which][ct][g4 * 4 + 0], acc[which][ct][g4 * 4 + 1],
                              acc[which][ct][g4 * 4 + 2], acc[which][ct][g4 * 4 + 3]};
            *reinterpret_cast<float4*>(o + g4 * 8 + (lane >> 5) * 4) = v;
          }
        }
      }
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
