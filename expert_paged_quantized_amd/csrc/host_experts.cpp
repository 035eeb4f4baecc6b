// Host-core expert computation for hybrid decode forwards (see host_experts.h).
//
// Reads the prepacked record layout of moe_common.h:
//   w1 = gate and up, [F/16 row tiles][H/64 k-blocks], a tile = 16 gate rows
//        then the same 16 up rows; w2 = down, [H/32 row tiles][F/64 k-blocks];
//   a k-block of a tile is 1024 code bytes: lane l (0..63) holds tile row
//        l % 32, inputs 32 * (l / 32) .. + 31 of the block (a "chunk");
//   int4: nibble n of each 32-bit word holds input {0,2,4,6,1,3,5,7}[n] of the
//        word's 8; scales per (row, scale block) a u32 of fp16 s' | fp16 b'
//        << 16, the checkpoint's values times 2^-c of the matrix;
//   MXFP4 / NVFP4: element 2i in the low nibble of byte i (as stored); MXFP4
//        one E8M0 byte per (half, row), NVFP4 two E4M3 bytes per (half, row)
//        and three fp32 matrix scales (gate, up, down) at the record's end.
// A chunk's 16 low nibbles and 16 high nibbles are decoded in byte order, and
// each token's activations are permuted once per forward into that order, so
// the inner loops are straight multiply-adds over 16-element runs.
#include "host_experts.h"

#include <string.h>

#include <chrono>
#include <cmath>

namespace strata {

// ---------------------------------------------------------------------------
// pool
// ---------------------------------------------------------------------------
HostPool::HostPool(int threads) {
  for (int i = 1; i < threads; ++i) workers_.emplace_back([this] { loop(); });
}

HostPool::~HostPool() {
  {
    std::lock_guard<std::mutex> lk(mu_);
    stop_ = true;
    gen_.fetch_add(1, std::memory_order_release);
  }
  cv_.notify_all();
  for (auto& t : workers_) t.join();
}

void HostPool::work(Task& t) {
  for (;;) {
    const int i = t.next.fetch_add(1, std::memory_order_acq_rel);
    if (i >= t.n) break;
    (*t.fn)(i);
    t.done.fetch_add(1, std::memory_order_acq_rel);
  }
}

void HostPool::run(int n, const std::function<void(int)>& fn) {
  if (n <= 0) return;
  Task t;
  t.fn = &fn;
  t.n = n;
  {
    std::lock_guard<std::mutex> lk(mu_);
    task_ = &t;
    gen_.fetch_add(1, std::memory_order_release);
  }
  cv_.notify_all();
  work(t);
  while (t.done.load(std::memory_order_acquire) < n) std::this_thread::yield();
  {
    std::lock_guard<std::mutex> lk(mu_);
    task_ = nullptr;
  }
  // threads that joined the task have all left it before it goes out of scope
  while (t.users.load(std::memory_order_acquire) != 0) std::this_thread::yield();
}

void HostPool::loop() {
  uint64_t seen = gen_.load(std::memory_order_acquire);
  for (;;) {
    const auto t0 = std::chrono::steady_clock::now();
    uint64_t g;
    while ((g = gen_.load(std::memory_order_acquire)) == seen) {
      if (std::chrono::steady_clock::now() - t0 > std::chrono::microseconds(300)) {
        std::unique_lock<std::mutex> lk(mu_);
        cv_.wait(lk, [&] { return gen_.load(std::memory_order_acquire) != seen; });
      }
    }
    seen = g;
    Task* t;
    {
      std::lock_guard<std::mutex> lk(mu_);
      if (stop_) return;
      t = task_;
      if (t) t->users.fetch_add(1, std::memory_order_acq_rel);
    }
    if (t) {
      work(*t);
      t->users.fetch_sub(1, std::memory_order_acq_rel);
    }
  }
}

// ---------------------------------------------------------------------------
// dot products of tile rows with the permuted activations
// ---------------------------------------------------------------------------
namespace {

inline float f16_bits(uint16_t b) {
  _Float16 v;
  memcpy(&v, &b, 2);
  return (float)v;
}

// OCP FP8 E4M3 values of all 256 bytes (NaN bytes were refused at
// admission): sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0,
// exponent 0 being m * 2^-9.
struct E4M3Table {
  float v[256];
  E4M3Table() {
    for (int b = 0; b < 256; ++b) {
      const int ex = (b >> 3) & 15, man = b & 7;
      const float mag = ex ? std::ldexp(1.0f + man / 8.0f, ex - 7) : std::ldexp((float)man, -9);
      v[b] = (b & 0x80) ? -mag : mag;
    }
  }
};
const E4M3Table kE4M3;

inline float pow2(int e) {  // 2^e for an E8M0 exponent, e in -126..127
  const uint32_t bits = uint32_t(e + 127) << 23;
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

// E2M1 value of a 4-bit code (sign bit 3, exponent bits 2..1 with bias 1,
// mantissa bit 0), built from its bits.
inline float e2m1(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const uint32_t mag = e ? ((e + 126u) << 23) | (m << 22) : (m ? 0x3F000000u : 0u);
  const uint32_t bits = mag | ((c & 8u) << 28);
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

struct Mat {
  const uint8_t* codes;
  const uint8_t* scales;
  int KB;  // k-blocks per row tile
  int c;   // int4: the stored scales and biases are the checkpoint's times 2^-c
};

// Input index (0..31 inside a chunk) of the d-th decoded value: d < 16 are
// the low nibbles of bytes 0..15, d >= 16 the high nibbles.
inline int chunk_input(int qf, int d) {
  const int byte = d & 15, hi = d >> 4;
  if (qf == Q_INT4) {  // byte j of word wi: nibbles 2j (low), 2j + 1 (high)
    static const int pos[8] = {0, 2, 4, 6, 1, 3, 5, 7};
    return 8 * (byte >> 2) + pos[2 * (byte & 3) + hi];
  }
  return 2 * byte + hi;
}

typedef float v8f __attribute__((vector_size(32)));
typedef int32_t v8i __attribute__((vector_size(32)));
typedef uint8_t v8u8 __attribute__((vector_size(8)));

inline v8f load8(const float* p) {
  v8f v;
  memcpy(&v, p, sizeof v);
  return v;
}

// E2M1 codes (low 4 bits of each lane) to their values, from the bits.
inline v8f e2m1_vec(v8i c) {
  const v8i e = (c >> 1) & 3, m = c & 1;
  const v8i nz = (v8i)(e != 0);  // a vector compare gives all ones (-1) where true
  const v8i mag = (nz & (((e + 126) << 23) | (m << 22))) | (~nz & (m * 0x3F000000));
  const v8i bits = mag | ((c & 8) << 28);
  v8f f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

// The 32 weights of one chunk, as 4 vectors in decode order (low nibbles of
// bytes 0..7, of 8..15, then the high nibbles): int4 as plain q, FP4 as E2M1
// values.
template <int QF>
inline void decode_codes(const uint8_t* ch, v8f (&q)[4]) {
  v8u8 b[2];
  memcpy(&b[0], ch, 8);
  memcpy(&b[1], ch + 8, 8);
  for (int i = 0; i < 2; ++i) {
    const v8u8 lo = b[i] & (uint8_t)15, hi = b[i] >> (uint8_t)4;
    if (QF == Q_INT4) {
      q[i] = __builtin_convertvector(lo, v8f);
      q[2 + i] = __builtin_convertvector(hi, v8f);
    } else {
      q[i] = e2m1_vec(__builtin_convertvector(lo, v8i));
      q[2 + i] = e2m1_vec(__builtin_convertvector(hi, v8i));
    }
  }
}

// out[t][r] for the 32 rows r of row tile rt: sum over K of w[r][k] x[t][k],
// with xp the activations permuted per chunk (xp[t][kb][half][32] in decode
// order) and xs the per-chunk sums of x (int4 biases).  Each (row, token)
// sums in 8 lanes in a fixed order, then adds the lanes in order.
template <int QF>
__attribute__((always_inline)) inline void tile_rows(int sshift, const Mat& m, int rt, const float* xp,
                                                     const float* xs, int ntok, int KB, float* out) {
  constexpr int kMaxTok = 8;
  for (int r = 0; r < 32; ++r) {
    v8f acc[kMaxTok];
    float bsum[kMaxTok];
    for (int t = 0; t < ntok; ++t) {
      bsum[t] = 0.0f;
      acc[t] = v8f{};
    }
    for (int kb = 0; kb < KB; ++kb) {
      for (int half = 0; half < 2; ++half) {
        const int lane = half * 32 + r;
        v8f q[4];
        decode_codes<QF>(m.codes + ((size_t)rt * m.KB + kb) * kTileCodeBytes + lane * 16, q);
        float s0, s1 = 0.0f, b = 0.0f;
        if (QF == Q_INT4) {
          // s', b' in the matrix's scaled domain; the row's sum is scaled by
          // 2^c once at the end
          uint32_t sc;
          memcpy(&sc, m.scales + ((size_t)rt * (m.KB >> sshift) + (kb >> sshift)) * 128 + r * 4, 4);
          s0 = f16_bits((uint16_t)(sc & 0xffff));
          b = f16_bits((uint16_t)(sc >> 16));
        } else if (QF == Q_MXFP4) {
          s0 = pow2((int)m.scales[((size_t)rt * m.KB + kb) * 64 + lane] - 127);
        } else {
          const uint8_t* sb = m.scales + ((size_t)rt * m.KB + kb) * 128 + lane * 2;
          s0 = kE4M3.v[sb[0]];
          s1 = kE4M3.v[sb[1]];
        }
        for (int t = 0; t < ntok; ++t) {
          const float* x = xp + (((size_t)t * KB + kb) * 2 + half) * 32;
          const v8f x0 = load8(x), x1 = load8(x + 8), x2 = load8(x + 16), x3 = load8(x + 24);
          if (QF == Q_NVFP4) {
            // bytes 0..7 hold inputs 0..15 (first E4M3 block), 8..15 the rest
            const v8f p0 = q[0] * x0 + q[2] * x2, p1 = q[1] * x1 + q[3] * x3;
            acc[t] += s0 * p0 + s1 * p1;
          } else {
            const v8f p = ((q[0] * x0 + q[1] * x1) + q[2] * x2) + q[3] * x3;
            acc[t] += s0 * p;
            if (QF == Q_INT4) bsum[t] += b * xs[((size_t)t * KB + kb) * 2 + half];
          }
        }
      }
    }
    for (int t = 0; t < ntok; ++t) {
      float v = 0.0f;
      for (int j = 0; j < 8; ++j) v += acc[t][j];
      v += bsum[t];
      out[t * 32 + r] = QF == Q_INT4 ? std::ldexp(v, m.c) : v;
    }
  }
}

template <int QF>
__attribute__((target("avx2,fma,f16c"))) void tile_rows_avx2(int sshift, const Mat& m, int rt, const float* xp,
                                                        const float* xs, int ntok, int KB, float* out) {
  tile_rows<QF>(sshift, m, rt, xp, xs, ntok, KB, out);
}
template <int QF>
void tile_rows_base(int sshift, const Mat& m, int rt, const float* xp, const float* xs, int ntok, int KB,
                    float* out) {
  tile_rows<QF>(sshift, m, rt, xp, xs, ntok, KB, out);
}

void tile_dot(int qf, int sshift, const Mat& m, int rt, const float* xp, const float* xs, int ntok, int KB,
              float* out) {
  static const bool avx2 =
      __builtin_cpu_supports("avx2") && __builtin_cpu_supports("fma") && __builtin_cpu_supports("f16c");
  if (qf == Q_INT4)
    (avx2 ? tile_rows_avx2<Q_INT4> : tile_rows_base<Q_INT4>)(sshift, m, rt, xp, xs, ntok, KB, out);
  else if (qf == Q_MXFP4)
    (avx2 ? tile_rows_avx2<Q_MXFP4> : tile_rows_base<Q_MXFP4>)(sshift, m, rt, xp, xs, ntok, KB, out);
  else
    (avx2 ? tile_rows_avx2<Q_NVFP4> : tile_rows_base<Q_NVFP4>)(sshift, m, rt, xp, xs, ntok, KB, out);
}

// Activations of ntok tokens (K inputs each) in chunk decode order, and the
// sum of each chunk's 32 inputs (summed in input order).
void permute_rows(int qf, const float* x, int ntok, int K, float* xp, float* xs) {
  const int KB = K / kTileK;
  int pos[32];
  for (int d = 0; d < 32; ++d) pos[d] = chunk_input(qf, d);
  for (int t = 0; t < ntok; ++t)
    for (int kb = 0; kb < KB; ++kb)
      for (int half = 0; half < 2; ++half) {
        const float* src = x + (size_t)t * K + kb * kTileK + half * 32;
        float* dst = xp + (((size_t)t * KB + kb) * 2 + half) * 32;
        float sum = 0.0f;
        for (int d = 0; d < 32; ++d) {
          dst[d] = src[pos[d]];
          sum += src[d];
        }
        xs[((size_t)t * KB + kb) * 2 + half] = sum;
      }
}

}  // namespace

void host_experts_run(HostPool& pool, const std::vector<HostJob>& jobs, int H, int F, int qf, int sshift,
                      const RecordLayout& lay, float* hbuf) {
  const int nj = (int)jobs.size();
  std::vector<int> hoff(nj + 1, 0);  // rows of h (and tokens) per job
  for (int j = 0; j < nj; ++j) hoff[j + 1] = hoff[j] + jobs[j].ntok;
  const int rows = hoff[nj];
  const int t1 = F / 16, t2 = H / 32;  // row tiles of w1, w2
  const int KB1 = H / kTileK, KB2 = F / kTileK;
  std::vector<float> xp((size_t)rows * H), xs((size_t)rows * KB1 * 2);
  std::vector<float> hp((size_t)rows * F), hs((size_t)rows * KB2 * 2);
  for (int j = 0; j < nj; ++j)
    permute_rows(qf, jobs[j].x, jobs[j].ntok, H, xp.data() + (size_t)hoff[j] * H,
                 xs.data() + (size_t)hoff[j] * KB1 * 2);

  auto gscale = [&](const HostJob& jb, int i) {
    if (qf != Q_NVFP4) return 1.0f;
    float g[3];
    memcpy(g, jb.rec + lay.gscale, sizeof g);
    return g[i];
  };

  // gate + up: unit = (job, w1 tile) -> 16 outputs of h per token.  A w1 tile
  // mixes gate rows (0..15) and up rows (16..31): int4 decodes each with its
  // own matrix's power of two (two passes when they differ).
  pool.run(nj * t1, [&](int u) {
    const int j = u / t1, rt = u % t1;
    const HostJob& jb = jobs[j];
    const float* x = xp.data() + (size_t)hoff[j] * H;
    const float* s = xs.data() + (size_t)hoff[j] * KB1 * 2;
    Mat mg{jb.rec + lay.w1_codes, jb.rec + lay.w1_scales, KB1, jb.wexp[kWexpGate]};
    float dg[8 * 32], du[8 * 32];
    tile_dot(qf, sshift, mg, rt, x, s, jb.ntok, KB1, dg);
    const float* up = dg;
    if (qf == Q_INT4 && jb.wexp[kWexpUp] != mg.c) {
      Mat mu = mg;
      mu.c = jb.wexp[kWexpUp];
      tile_dot(qf, sshift, mu, rt, x, s, jb.ntok, KB1, du);
      up = du;
    }
    const float gg = gscale(jb, 0), gu = gscale(jb, 1);
    for (int t = 0; t < jb.ntok; ++t)
      for (int r = 0; r < 16; ++r) {
        const float g = dg[t * 32 + r] * gg, v = up[t * 32 + 16 + r] * gu;
        hbuf[((size_t)hoff[j] + t) * F + rt * 16 + r] = g / (1.0f + std::exp(-g)) * v;
      }
  });
  for (int j = 0; j < nj; ++j)
    permute_rows(qf, hbuf + (size_t)hoff[j] * F, jobs[j].ntok, F, hp.data() + (size_t)hoff[j] * F,
                 hs.data() + (size_t)hoff[j] * KB2 * 2);
  // down: unit = (job, w2 tile) -> 32 outputs of o per token
  pool.run(nj * t2, [&](int u) {
    const int j = u / t2, rt = u % t2;
    const HostJob& jb = jobs[j];
    Mat md{jb.rec + lay.w2_codes, jb.rec + lay.w2_scales, KB2, jb.wexp[kWexpDown]};
    float d[8 * 32];
    tile_dot(qf, sshift, md, rt, hp.data() + (size_t)hoff[j] * F, hs.data() + (size_t)hoff[j] * KB2 * 2,
             jb.ntok, KB2, d);
    const float gd = gscale(jb, 2);
    for (int t = 0; t < jb.ntok; ++t)
      for (int r = 0; r < 32; ++r) jb.o[(size_t)t * H + rt * 32 + r] = d[t * 32 + r] * gd;
  });
}

}  // namespace strata
