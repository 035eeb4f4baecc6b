// Host runtime and C ABI of the routed 4-bit MoE layer (see include/strata_moe.h).
//
// Create validates and admits the checkpoint, prepacks every routed expert
// once into a pinned host store (a byte permutation into the kernels' tile
// order: same byte count, no wider copy; ro99/strata README, SM86 kernel and
// precision paragraphs), allocates the HBM slot pool for the budget
// ("Documentation" page, Signature) plus the resident shared expert and router
// ("Strata, Explained", section 2: routers and shared experts live in GPU
// memory next to a cache of routed experts), and preloads slots.
//
// Forward enqueues router -> top-k -> permute, then the expert GEMMs and the
// combine.  With every expert resident the whole forward stays on the device.
// With a smaller budget the per-expert counts come back to the host once, the
// residency manager decides hits, misses and waves, and misses are copied from
// the pinned store into their slots.  A prefill pages on the copy streams
// (kCopyStreams of them, masked to kPageCUs CUs) while each wave runs its hit
// experts on the paged compute stream, and a wave's pages wait only for the
// compute of the wave that last read their slots; a decode forward pages on
// the caller's stream, in wave order.  After a forward the policy may page
// experts ahead of need (prefetch); the next forward waits for those pages.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <sched.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <type_traits>
#include <cmath>
#include <chrono>
#include <cstdio>
#include <string>
#include <thread>
#include <vector>

#include "../../include/strata_moe.h"
#include "moe_common.h"
#include "host_experts.h"
#include "residency.h"

namespace strata {
hipError_t launch_router(const uint16_t*, const uint16_t*, const float*, float*, uint16_t*, int32_t*, float*,
                         int, int, int, int, hipStream_t);
hipError_t launch_route(const float*, int, int, int, int, int, int, int, int32_t*, float*, int32_t*,
                        int32_t*, int32_t*, int32_t*, int32_t*, int32_t*, Tile*, int32_t*,
                        unsigned long long*, hipStream_t);
bool route_decode_fits(int T, int Eall);
hipError_t launch_route_decode(const uint16_t*, const uint16_t*, const float*, float*, uint16_t*, int32_t*, float*,
                               int, int, uint32_t*, int, int, int, int, int, int, int, int32_t*, float*, int32_t*,
                               int32_t*, int32_t*, int32_t*, Tile*, int32_t*, unsigned long long*, hipStream_t);
hipError_t launch_expert_gemm(const GemmArgs&, int, bool, bool, int, int, int, hipStream_t);
hipError_t launch_page_in(const PageBatch&, hipStream_t);
int decode_log2_splits(int N, int K, int tiles_per_token, int T);
int decode_grid(int N, int log2S, int n_tiles);
uint64_t read_probe_bytes(uint64_t bytes);
hipError_t launch_read_probe(const void* p, uint64_t bytes, uint32_t* out, hipStream_t s);
int decode_dot_waves(int N, int K, int quant, int tiles_per_token, int T);
hipError_t launch_decode_dot(const GemmArgs& a, int quant, bool gate_up, int T, int S, int n_tiles, hipStream_t s);
hipError_t launch_combine(const float*, const int32_t*, const float*, int, int, int, int, int, int64_t,
                          const float*, uint16_t*, hipStream_t);
uint64_t scratch_bytes();
hipError_t scratch_init(int device);
void* scratch_ptr(int device);
}  // namespace strata

using namespace strata;

// ---------------------------------------------------------------------------
// error state
// ---------------------------------------------------------------------------
static thread_local std::string g_err;

static strata_status fail(strata_status st, const std::string& msg) {
  g_err = msg;
  return st;
}

static const char* fault_env() {
  const char* f = getenv("STRATA_FAULT");
  return f ? f : "";
}
static bool fault(const char* what) { return strcmp(fault_env(), what) == 0; }

#define HIP_CHECK(expr)                                                                      \
  do {                                                                                       \
    hipError_t _e = (expr);                                                                  \
    if (_e != hipSuccess) return fail(STRATA_E_HIP, std::string(#expr) + ": " + hipGetErrorString(_e)); \
  } while (0)

// ---------------------------------------------------------------------------
// handle
// ---------------------------------------------------------------------------
struct TimingRec {
  int cls;
  hipEvent_t a, b;
};

namespace strata {
thread_local KernelTimer g_ktimer;
}  // namespace strata

#ifndef STRATA_COPY_STREAMS
#define STRATA_COPY_STREAMS 2
#endif
// Side streams the expert pages are copied on (all at the default priority).
// A budgeted forward uses the caller's stream, the paged compute stream and
// these: four streams, the hardware queues HIP gives a process by default.
constexpr int kCopyStreams = STRATA_COPY_STREAMS;
// CUs set aside for the page-in kernel of a budgeted layer (the copy streams'
// CU mask); its expert GEMMs run on an internal stream masked to the others.
// The runtime deals CU-mask bits round-robin over the XCDs, so the first 16
// bits are two CUs of each of the 8 XCDs.
constexpr int kPageCUs = 16;
// Tokens per host expert the host kernels take (hybrid_rows at most this).
constexpr int kHostMaxRows = 8;

// Device buffers of one forward, carved from one block of device memory: the
// handle's own (sized for max_tokens at create) or, for the no-allocation
// entry point, the library's static scratch (sized for the call's T).  Every
// forward writes each element before it reads it, so nothing here needs
// clearing between forwards.
struct Workspace {
  float* logits = nullptr;      // [T, E]
  int32_t* idx = nullptr;       // [T, k]
  float* w = nullptr;           // [T, k]
  int32_t* counts = nullptr;    // [E]
  int32_t* offsets = nullptr;   // [E + 1]
  int32_t* perm = nullptr;      // [max_rows]: routed rows, then the shared rows
  int32_t* pos = nullptr;       // [T, k]
  int32_t* rank = nullptr;      // [T, k]: rank inside its 64-token block
  int32_t* hist = nullptr;      // [ceil(T / 64), E]
  Tile* tiles_dev = nullptr;    // tile list built by the routing kernels
  Tile* tiles_host = nullptr;   // tile lists built by the residency manager
  int32_t* ntiles = nullptr;
  void* hbuf = nullptr;         // h [max_rows, F], 16-bit
  float* o = nullptr;           // [ksplit][max_rows, H]
  uint16_t* x16 = nullptr;      // fp16 formats: the scaled fp16 copy of x [T, H]
  int32_t* xexp = nullptr;      // fp16 formats: its per-token exponents [T]
  float* gate = nullptr;        // shared-expert gate logits [T] (gated layers)
  size_t max_rows = 0, max_tiles = 0;
};

struct strata_moe {
  int H = 0, F = 0, E = 0, k = 0, S = 0, quant = 0, router = 0, policy = 0, budget = 0;
  int sshift = 0;  // scale block of k-block kb is kb >> sshift (int4 group-128: 1)
  int ksplit = 1;  // prefill down: partial-sum planes of o
  int max_tokens = 0, device = 0;
  RecordLayout lay{};
  size_t slot_stride = 0;
  bool f16 = false;    // int4 / NVFP4: fp16 GEMMs on the scaled fp16 copy of x
  bool gated = false;  // the shared expert is weighted by sigmoid(x . w_s)

  uint8_t* host_store = nullptr;  // pinned, E records at slot_stride
  const uint8_t* host_dev = nullptr;  // the same store's device address (read by the page-in kernel)
  uint8_t* d_pool = nullptr;      // budget * slot_stride
  uint8_t* d_shared = nullptr;    // slot_stride
  uint16_t* d_router_w = nullptr;
  float* d_router_bias = nullptr;
  uint8_t** d_slot_ptr = nullptr;  // budget + 1 entries
  std::vector<uint8_t*> h_slot_ptr;

  Workspace ws;                // per-forward buffers for max_tokens (one allocation)
  uint8_t* d_ws = nullptr;
  unsigned long long* d_distinct = nullptr;  // distinct experts used, summed over forwards
  int32_t* d_wexp = nullptr;   // per expert (+ shared): kWexpCount rescaling exponents
  std::vector<int32_t> wexp;   // host copy of the same

  int32_t* h_counts = nullptr;  // pinned
  Tile* h_tiles = nullptr;      // pinned
  // hybrid forwards: the host pool and pinned staging of the tokens, their
  // grouping and the host-computed output rows (decode: kDecodeMaxT tokens;
  // with hybrid_rows, prefill: max_tokens tokens, at most E * hybrid_rows
  // host rows)
  bool hybrid = false;
  int hybrid_rows = 0;          // hybrid prefill: row limit of a host expert (0: none)
  HostPool* pool = nullptr;
  int32_t* h_perm = nullptr;    // pinned [tokens * k]
  uint16_t* h_x = nullptr;      // pinned bf16 [tokens, H]
  float* h_o = nullptr;         // pinned fp32 [host rows, H]
  hipEvent_t ev_hx = nullptr;   // perm and x of a hybrid prefill have reached the host
  std::vector<float> h_xf, h_hbuf;
  uint64_t host_ns = 0;         // wall time of the host expert computations
  hipStream_t copy_streams[kCopyStreams] = {};
  // Budgeted layers: the expert GEMMs of a paged forward run on pstream, whose
  // CU mask excludes the copy streams' CUs (a page-in workgroup's host reads
  // stall the memory path of the CU it shares: expert GEMM launches beside it
  // took 3-6x longer).  ev_pfork orders pstream after the forward's routing
  // on the caller's stream, ev_pjoin the combine after pstream.  Null when
  // the split is not in use (all experts resident, or the masks were refused).
  hipStream_t pstream = nullptr;
  hipEvent_t ev_pfork = nullptr, ev_pjoin = nullptr;
  hipEvent_t ev_fwd_done = nullptr;
  hipEvent_t ev_counts = nullptr;  // the token counts have reached h_counts
  bool fwd_recorded = false;
  std::vector<hipEvent_t> ev_copied;  // [wave][copy stream]
  std::vector<hipEvent_t> ev_wave_done;
  // pages made ahead of need (prefetch, profile loads): the last one on each
  // copy stream; the next forward orders its copies and compute after them
  hipEvent_t ev_ahead[kCopyStreams] = {};
  bool ahead_used[kCopyStreams] = {};
  bool ahead_pending = false;

  ResidencyManager rm;
  int decay_shift = 0, prefetch = 0;
  int pager = STRATA_PAGER_KERNEL;  // the paging engine in use
  uint64_t forwards = 0;
  bool poisoned = false;

  bool timing = false;
  std::vector<TimingRec> trecs;
  std::vector<hipEvent_t> ev_pool;
  double t_ms[STRATA_K_COUNT] = {};
  uint64_t t_launch[STRATA_K_COUNT] = {};
};

// ---------------------------------------------------------------------------
// validation / admission (pure host; runs before any HIP call)
// ---------------------------------------------------------------------------
static float bf16_float(uint16_t bf) {
  const uint32_t u = uint32_t(bf) << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// OCP FP8 E4M3 byte (NaN bytes refused at admission): sign bit 7, exponent
// bits 6..3 with bias 7, mantissa bits 2..0; exponent 0 is m * 2^-9.
static double e4m3_float(uint8_t byte) {
  const int ex = (byte >> 3) & 15, man = byte & 7;
  const double mag = ex ? std::ldexp(1.0 + man / 8.0, ex - 7) : std::ldexp((double)man, -9);
  return (byte & 0x80) ? -mag : mag;
}

// int4 scale and bias re-encoding.  The kernels compute int4 layers in fp16,
// whose exponent range (2^-24 .. 65504) is far narrower than bf16's, so every
// matrix (gate, up or down of one expert) gets one power of two 2^-c: its
// scales and biases are stored as the fp16 numbers s * 2^-c, b * 2^-c, which
// must be exact (lowest set bit at or above 2^-24), and no decoded weight
// s' q + b' may exceed 2^15 in magnitude (15 |s'| + |b'| <= 2^15).  Of the
// exponents that satisfy both, the smallest is taken: it puts the largest
// decoded weight in (2^14, 2^15], as far above fp16's subnormal range as the
// matrix allows.  A matrix whose values span more than fp16 holds exactly
// under one c is refused (E_UNSUPPORTED), a NaN or infinite scale or bias
// fails admission (E_BAD_SCALE).  The epilogues multiply the results by
// 2^c again, so the weights the layer computes with are the checkpoint's.
static strata_status int4_matrix_exponent(const uint16_t* s, const uint16_t* b, size_t n, const char* name,
                                          int* c_out) {
  int c_max = 1 << 20;  // every value's lowest set bit, + 24
  double m = 0.0;       // max 15 |s| + |b|
  for (size_t i = 0; i < n; ++i) {
    for (uint16_t v : {s[i], b[i]}) {
      const int ef = (v >> 7) & 0xff, man = v & 0x7f;
      if (ef == 255) return fail(STRATA_E_BAD_SCALE, std::string(name) + ": int4 scale or bias is not a finite number");
      if (ef == 0 && man == 0) continue;
      // value = sig * 2^(q0): normal sig = 1.man (8 bits) at q0 = ef - 134,
      // subnormal sig = man at q0 = -133
      const int sig = ef ? (man | 0x80) : man;
      const int q0 = ef ? ef - 134 : -133;
      c_max = std::min(c_max, q0 + __builtin_ctz(sig) + 24);
    }
    m = std::max(m, 15.0 * std::fabs((double)bf16_float(s[i])) + std::fabs((double)bf16_float(b[i])));
  }
  if (m == 0.0) {
    *c_out = 0;
    return STRATA_OK;
  }
  int e;
  const double f = std::frexp(m, &e);  // m = f 2^e, f in [0.5, 1)
  const int c_min = (f == 0.5 ? e - 1 : e) - 15;  // smallest c with m <= 2^(15 + c)
  if (c_min > c_max)
    return fail(STRATA_E_UNSUPPORTED, std::string(name) +
                                          ": int4 scales and biases span more than fp16 holds exactly under one "
                                          "power-of-two rescaling (2^-24 .. 2^15)");
  *c_out = c_min;
  return STRATA_OK;
}

// What the host needs to know about a weight format.
struct FormatInfo {
  int kq;       // kernel dequant family (QFormat)
  int group;    // inputs per scale
  bool affine;  // int4: bf16 scale and bias per group
  bool f16;     // the kernels compute in fp16 (and read the fp16 copy of x)
  int sshift;   // scale block of k-block kb is kb >> sshift
};

static bool format_of(int quant, FormatInfo& f) {
  switch (quant) {
    case STRATA_Q_INT4_G64_AFFINE_BF16: f = {Q_INT4, 64, true, true, 0}; return true;
    case STRATA_Q_INT4_G128_AFFINE_BF16: f = {Q_INT4, 128, true, true, 1}; return true;
    case STRATA_Q_MXFP4_E2M1_E8M0_G32: f = {Q_MXFP4, 32, false, false, 0}; return true;
    case STRATA_Q_NVFP4_E2M1_E4M3_G16: f = {Q_NVFP4, 16, false, true, 0}; return true;
    default: return false;
  }
}

// Residency arguments shared by create and the dry-run planner.
static strata_status check_residency(int E, int budget, int policy, int decay_shift, int prefetch,
                                     const uint64_t* profile) {
  if (policy != STRATA_P_LRU && policy != STRATA_P_LFU && policy != STRATA_P_WARM)
    return fail(STRATA_E_INVALID, "unknown policy");
  if (budget < 1 || budget > E) return fail(STRATA_E_INVALID, "expert_budget must be in [1, num_experts]");
  if (policy == STRATA_P_WARM && (decay_shift < 1 || decay_shift > 24))
    return fail(STRATA_E_INVALID, "WARM needs decay_shift in [1, 24]");
  if (policy != STRATA_P_WARM && decay_shift != 0)
    return fail(STRATA_E_INVALID, "decay_shift applies to WARM only");
  if (prefetch < 0 || prefetch > budget) return fail(STRATA_E_INVALID, "prefetch must be in [0, budget]");
  if (profile)
    for (int e = 0; e < E; ++e)
      if (profile[e] > ResidencyManager::kMaxScore) return fail(STRATA_E_INVALID, "profile score above 2^62");
  return STRATA_OK;
}

static int rm_policy(int policy) {
  return policy == STRATA_P_WARM ? ResidencyManager::kWARM
                                 : policy == STRATA_P_LFU ? ResidencyManager::kLFU : ResidencyManager::kLRU;
}

static strata_status validate(const strata_moe_desc* d) {
  if (!d) return fail(STRATA_E_INVALID, "desc is NULL");
  if (d->hidden <= 0 || d->ffn <= 0 || d->num_experts <= 0 || d->top_k <= 0 || d->max_tokens <= 0)
    return fail(STRATA_E_INVALID, "sizes must be positive");
  if (d->num_experts > 1024) return fail(STRATA_E_UNSUPPORTED, "num_experts > 1024");
  if (d->top_k > d->num_experts) return fail(STRATA_E_INVALID, "top_k > num_experts");
  if (d->top_k > 32) return fail(STRATA_E_UNSUPPORTED, "top_k > 32");
  if (d->num_shared != 0 && d->num_shared != 1) return fail(STRATA_E_UNSUPPORTED, "num_shared must be 0 or 1");
  FormatInfo fi;
  if (!format_of(d->quant, fi)) return fail(STRATA_E_INVALID, "unknown quant");
  if (d->router != STRATA_R_SOFTMAX_TOPK_RENORM && d->router != STRATA_R_SIGMOID_TOPK_RENORM)
    return fail(STRATA_E_INVALID, "unknown router");
  if (d->pager != STRATA_PAGER_AUTO && d->pager != STRATA_PAGER_KERNEL && d->pager != STRATA_PAGER_DMA)
    return fail(STRATA_E_INVALID, "unknown pager");
  if (strata_status st = check_residency(d->num_experts, d->expert_budget, d->policy, d->decay_shift,
                                         d->prefetch, d->expert_profile))
    return st;
  if (d->hybrid != 0 && d->hybrid != 1) return fail(STRATA_E_INVALID, "hybrid must be 0 or 1");
  if (d->host_threads < 0) return fail(STRATA_E_INVALID, "host_threads must be >= 0");
  if (d->hybrid_rows < 0 || d->hybrid_rows > kHostMaxRows)
    return fail(STRATA_E_INVALID, "hybrid_rows must be in [0, 8]");
  if (d->hybrid_rows > 0 && d->hybrid != 1) return fail(STRATA_E_INVALID, "hybrid_rows needs hybrid = 1");
  if (d->max_tokens > (1 << 20)) return fail(STRATA_E_UNSUPPORTED, "max_tokens > 2^20");
  if (d->hidden % 512) return fail(STRATA_E_UNSUPPORTED, "hidden must be a multiple of 512");
  if (d->ffn % 64) return fail(STRATA_E_UNSUPPORTED, "ffn must be a multiple of 64");
  if (d->ffn % fi.group) return fail(STRATA_E_UNSUPPORTED, "ffn must be a multiple of the quant group");
  if (!d->router_w) return fail(STRATA_E_INVALID, "router_w is NULL");
  const bool int4 = fi.affine, nvfp4 = fi.kq == Q_NVFP4;
  auto chk = [&](const strata_qmat& m, const char* name) -> strata_status {
    if (!m.codes || !m.scales) return fail(STRATA_E_INVALID, std::string(name) + ": codes/scales NULL");
    if (int4 && !m.biases) return fail(STRATA_E_INVALID, std::string(name) + ": int4 needs biases");
    if (!int4 && m.biases) return fail(STRATA_E_INVALID, std::string(name) + ": MXFP4/NVFP4 take no biases");
    if (nvfp4 && !m.global_scale) return fail(STRATA_E_INVALID, std::string(name) + ": NVFP4 needs global_scale");
    if (!nvfp4 && m.global_scale)
      return fail(STRATA_E_INVALID, std::string(name) + ": global_scale is for NVFP4 only");
    return STRATA_OK;
  };
  strata_status st;
  if ((st = chk(d->gate, "gate")) || (st = chk(d->up, "up")) || (st = chk(d->down, "down"))) return st;
  if (d->num_shared) {
    if ((st = chk(d->sh_gate, "sh_gate")) || (st = chk(d->sh_up, "sh_up")) || (st = chk(d->sh_down, "sh_down")))
      return st;
  } else if (d->sh_gate.codes || d->sh_up.codes || d->sh_down.codes) {
    return fail(STRATA_E_INVALID, "shared expert weights given with num_shared = 0");
  } else if (d->shared_gate_w) {
    return fail(STRATA_E_INVALID, "shared_gate_w given with num_shared = 0");
  }
  // admission of scales
  const size_t H = d->hidden, F = d->ffn;
  auto admit = [&](const strata_qmat& m, size_t n_exp, size_t rows, size_t cols, const char* name) -> strata_status {
    if (int4) {
      const size_t n = rows * (cols / fi.group);  // per expert
      for (size_t e = 0; e < n_exp; ++e) {
        int c;
        if (strata_status st2 = int4_matrix_exponent((const uint16_t*)m.scales + e * n,
                                                     (const uint16_t*)m.biases + e * n, n, name, &c))
          return st2;
      }
    } else if (nvfp4) {
      const size_t n = n_exp * rows * (cols / 16);
      const uint8_t* s = (const uint8_t*)m.scales;
      for (size_t i = 0; i < n; ++i)
        if ((s[i] & 0x7F) == 0x7F)
          return fail(STRATA_E_BAD_SCALE, std::string(name) + ": E4M3 scale byte is NaN at index " +
                                              std::to_string(i));
      for (size_t e = 0; e < n_exp; ++e) {
        const float g = m.global_scale[e];
        if (!(g > 0.0f) || g == __builtin_inff())
          return fail(STRATA_E_BAD_SCALE, std::string(name) + ": NVFP4 matrix scale not finite and > 0");
      }
    } else {
      const size_t n = n_exp * rows * (cols / 32);
      const uint8_t* s = (const uint8_t*)m.scales;
      for (size_t i = 0; i < n; ++i)
        if (s[i] == 0 || s[i] == 255)
          return fail(STRATA_E_BAD_SCALE, std::string(name) + ": E8M0 scale byte 0 or 255 at index " +
                                              std::to_string(i));
    }
    return STRATA_OK;
  };
  const size_t E = d->num_experts;
  if ((st = admit(d->gate, E, F, H, "gate")) || (st = admit(d->up, E, F, H, "up")) ||
      (st = admit(d->down, E, H, F, "down")))
    return st;
  if (d->num_shared) {
    if ((st = admit(d->sh_gate, 1, F, H, "sh_gate")) || (st = admit(d->sh_up, 1, F, H, "sh_up")) ||
        (st = admit(d->sh_down, 1, H, F, "sh_down")))
      return st;
  }
  return STRATA_OK;
}

// ---------------------------------------------------------------------------
// prepack: one expert's gate/up/down into the tile-order record
// ---------------------------------------------------------------------------
// int4 word nibble order k0 k2 k4 k6 k1 k3 k5 k7 (low to high); see the kernel.
static inline uint32_t int4_word_perm(uint32_t w) {
  uint32_t r = 0;
  for (int j = 0; j < 4; ++j) {
    r |= ((w >> (8 * j)) & 0xFu) << (4 * j);            // k_2j  -> nibble j
    r |= ((w >> (8 * j + 4)) & 0xFu) << (4 * (j + 4));  // k_2j+1 -> nibble j+4
  }
  return r;
}

struct MatView {
  const uint8_t* codes;   // [rows, cols/2]
  const uint8_t* scales;  // int4: bf16 [rows, cols/G]; MXFP4: u8 [rows, cols/32]; NVFP4: u8 [rows, cols/16]
  const uint8_t* biases;  // int4: bf16 [rows, cols/G]
  float gscale;           // NVFP4 matrix scale
  int c = 0;              // int4: scales and biases are stored times 2^-c (fp16)
};

static MatView view(const strata_qmat& m, size_t e, size_t rows, size_t cols, const FormatInfo& fi) {
  MatView v;
  v.codes = (const uint8_t*)m.codes + e * rows * (cols / 2);
  const size_t per = rows * (cols / fi.group);
  v.scales = (const uint8_t*)m.scales + e * per * (fi.affine ? 2 : 1);
  v.biases = fi.affine ? (const uint8_t*)m.biases + e * per * 2 : nullptr;
  v.gscale = m.global_scale ? m.global_scale[e] : 0.0f;
  return v;
}

// Packs the tiles of one matrix.  `row_of(rt, r)` maps tile row r of row tile
// rt to a (source matrix, row) pair.
template <class RowOf>
static void pack_matrix(uint8_t* codes_dst, uint8_t* scales_dst, int n_rt, int K, const FormatInfo& fi,
                        RowOf row_of) {
  const int KB = K / 64;
  for (int rt = 0; rt < n_rt; ++rt) {
    for (int kb = 0; kb < KB; ++kb) {
      uint8_t* cd = codes_dst + ((size_t)rt * KB + kb) * kTileCodeBytes;
      for (int l = 0; l < 64; ++l) {
        const int r = l & 31, h = l >> 5;
        const MatView* mv;
        int row;
        row_of(rt, r, mv, row);
        const uint8_t* src = mv->codes + (size_t)row * (K / 2) + (kb * 64 + h * 32) / 2;
        uint8_t* dst = cd + l * 16;
        if (fi.affine) {
          for (int wi = 0; wi < 4; ++wi) {
            uint32_t w;
            memcpy(&w, src + 4 * wi, 4);
            w = int4_word_perm(w);
            memcpy(dst + 4 * wi, &w, 4);
          }
        } else {
          memcpy(dst, src, 16);
        }
      }
      if (fi.affine) {
        if (kb & ((1 << fi.sshift) - 1)) continue;  // one block per 2^sshift k-blocks
        const int nsb = KB >> fi.sshift, sblk = kb >> fi.sshift;
        uint8_t* sd = scales_dst + ((size_t)rt * nsb + sblk) * 128;
        for (int r = 0; r < 32; ++r) {
          const MatView* mv;
          int row;
          row_of(rt, r, mv, row);
          const size_t gi = (size_t)row * nsb + sblk;
          uint16_t sc, b;
          memcpy(&sc, mv->scales + gi * 2, 2);
          memcpy(&b, mv->biases + gi * 2, 2);
          // exact by admission (int4_matrix_exponent)
          const _Float16 s16 = (_Float16)std::ldexp(bf16_float(sc), -mv->c);
          const _Float16 b16 = (_Float16)std::ldexp(bf16_float(b), -mv->c);
          uint16_t sbits, bbits;
          memcpy(&sbits, &s16, 2);
          memcpy(&bbits, &b16, 2);
          const uint32_t u = uint32_t(sbits) | (uint32_t(bbits) << 16);
          memcpy(sd + r * 4, &u, 4);
        }
      } else if (fi.kq == Q_NVFP4) {
        uint8_t* sd = scales_dst + ((size_t)rt * KB + kb) * 128;
        for (int l = 0; l < 64; ++l) {
          const int r = l & 31, h = l >> 5;
          const MatView* mv;
          int row;
          row_of(rt, r, mv, row);
          const uint8_t* src = mv->scales + (size_t)row * (K / 16) + kb * 4 + h * 2;
          sd[(h * 32 + r) * 2 + 0] = src[0];
          sd[(h * 32 + r) * 2 + 1] = src[1];
        }
      } else {
        uint8_t* sd = scales_dst + ((size_t)rt * KB + kb) * 64;
        for (int l = 0; l < 64; ++l) {
          const int r = l & 31, h = l >> 5;
          const MatView* mv;
          int row;
          row_of(rt, r, mv, row);
          sd[l] = mv->scales[(size_t)row * (K / 32) + kb * 2 + h];
        }
      }
    }
  }
}

// Sum of |w| along each row of one matrix, the largest over its rows (fp64;
// int4 and NVFP4, the formats the kernels compute in fp16).  Bounds the
// matrix's output: |W x| <= this * max|x|.
static double max_row_l1(const MatView& v, int rows, int cols, const FormatInfo& fi) {
  static const double e2m1_mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
  double best = 0.0;
  const int G = fi.group, ng = cols / G;
  for (int r = 0; r < rows; ++r) {
    const uint8_t* c = v.codes + (size_t)r * (cols / 2);
    double sum = 0.0;
    for (int g = 0; g < ng; ++g) {
      double tab[16];
      if (fi.affine) {
        uint16_t sb, bb;
        memcpy(&sb, v.scales + ((size_t)r * ng + g) * 2, 2);
        memcpy(&bb, v.biases + ((size_t)r * ng + g) * 2, 2);
        const double sv = bf16_float(sb), bv = bf16_float(bb);
        for (int q = 0; q < 16; ++q) tab[q] = std::fabs(sv * q + bv);
      } else {  // NVFP4: |e2m1| * |E4M3 block scale| * matrix scale
        const double sc = std::fabs(e4m3_float(v.scales[(size_t)r * ng + g])) * v.gscale;
        for (int q = 0; q < 16; ++q) tab[q] = e2m1_mag[q & 7] * sc;
      }
      for (int k = g * G; k < (g + 1) * G; k += 2) {
        const uint8_t byte = c[k / 2];
        sum += tab[byte & 15] + tab[byte >> 4];
      }
    }
    best = std::max(best, sum);
  }
  return best;
}

// Rescaling exponents of one expert (kWexp* order).  The h exponent c_h makes
// the stored h row of token t, h * 2^-(2 xexp[t] + c_h), stay below 2^14:
// the fp16 x row is below 2^15, so |g| <= 2^(xexp[t] + 15) A_g and likewise
// |u|, and |h| = |silu(g) u| <= |g| |u| (A = largest row sum of |w|).
static void expert_exponents(const strata_qmat& g, const strata_qmat& u, const strata_qmat& d, size_t e, int H,
                             int F, const FormatInfo& fi, int32_t* out) {
  for (int i = 0; i < kWexpCount; ++i) out[i] = 0;
  if (!fi.f16) return;  // MXFP4: bf16 operands, nothing to rescale
  if (fi.affine) {
    const size_t ng = H / fi.group, nd = F / fi.group;
    int c;
    (void)int4_matrix_exponent((const uint16_t*)g.scales + e * F * ng, (const uint16_t*)g.biases + e * F * ng,
                               F * ng, "gate", &c);  // admitted: cannot fail
    out[kWexpGate] = c;
    (void)int4_matrix_exponent((const uint16_t*)u.scales + e * F * ng, (const uint16_t*)u.biases + e * F * ng,
                               F * ng, "up", &c);
    out[kWexpUp] = c;
    (void)int4_matrix_exponent((const uint16_t*)d.scales + e * H * nd, (const uint16_t*)d.biases + e * H * nd,
                               H * nd, "down", &c);
    out[kWexpDown] = c;
  }
  const double ag = max_row_l1(view(g, e, F, H, fi), F, H, fi);
  const double au = max_row_l1(view(u, e, F, H, fi), F, H, fi);
  if (ag > 0.0 && au > 0.0) out[kWexpH] = (int)std::ceil(std::log2(ag) + std::log2(au)) + 16;
}

static void pack_expert(uint8_t* rec, const RecordLayout& lay, const strata_qmat& g,
                        const strata_qmat& u, const strata_qmat& d, size_t e, int H, int F,
                        const FormatInfo& fi, const int32_t* wexp) {
  MatView vg = view(g, e, F, H, fi), vu = view(u, e, F, H, fi), vd = view(d, e, H, F, fi);
  vg.c = wexp[kWexpGate];
  vu.c = wexp[kWexpUp];
  vd.c = wexp[kWexpDown];
  // w1: tile rt = gate rows 16rt..+15 then up rows 16rt..+15
  pack_matrix(rec + lay.w1_codes, rec + lay.w1_scales, F / 16, H, fi,
              [&](int rt, int r, const MatView*& mv, int& row) {
                mv = (r < 16) ? &vg : &vu;
                row = rt * 16 + (r & 15);
              });
  pack_matrix(rec + lay.w2_codes, rec + lay.w2_scales, H / 32, F, fi,
              [&](int rt, int r, const MatView*& mv, int& row) {
                mv = &vd;
                row = rt * 32 + r;
              });
  if (fi.kq == Q_NVFP4) {
    const float gs[3] = {vg.gscale, vu.gscale, vd.gscale};
    memcpy(rec + lay.gscale, gs, sizeof gs);
  }
}

// ---------------------------------------------------------------------------
// create / destroy
// ---------------------------------------------------------------------------
static void release(strata_moe* h) {
  if (!h) return;
  if (h->device >= 0) (void)hipSetDevice(h->device);
  for (auto cs : h->copy_streams)
    if (cs) (void)hipStreamSynchronize(cs);
  (void)hipDeviceSynchronize();
  for (auto& r : h->trecs) {
    h->ev_pool.push_back(r.a);
    h->ev_pool.push_back(r.b);
  }
  for (auto e : h->ev_pool) (void)hipEventDestroy(e);
  for (auto e : h->ev_copied) (void)hipEventDestroy(e);
  for (auto e : h->ev_wave_done) (void)hipEventDestroy(e);
  for (auto e : h->ev_ahead)
    if (e) (void)hipEventDestroy(e);
  if (h->ev_fwd_done) (void)hipEventDestroy(h->ev_fwd_done);
  if (h->ev_counts) (void)hipEventDestroy(h->ev_counts);
  if (h->ev_hx) (void)hipEventDestroy(h->ev_hx);
  for (auto cs : h->copy_streams)
    if (cs) (void)hipStreamDestroy(cs);
  if (h->pstream) (void)hipStreamDestroy(h->pstream);
  if (h->ev_pfork) (void)hipEventDestroy(h->ev_pfork);
  if (h->ev_pjoin) (void)hipEventDestroy(h->ev_pjoin);
  void* dev[] = {h->d_pool, h->d_shared, h->d_router_w, h->d_router_bias, h->d_slot_ptr,
                 h->d_ws, h->d_distinct, h->d_wexp};
  for (void* p : dev)
    if (p) (void)hipFree(p);
  if (h->host_store) (void)hipHostFree(h->host_store);
  if (h->h_counts) (void)hipHostFree(h->h_counts);
  if (h->h_tiles) (void)hipHostFree(h->h_tiles);
  delete h->pool;
  for (void* p : {(void*)h->h_perm, (void*)h->h_x, (void*)h->h_o})
    if (p) (void)hipHostFree(p);
  delete h;
}

template <class T>
static strata_status dev_alloc(T** p, size_t bytes) {
  if (fault("devalloc")) return fail(STRATA_E_NOMEM, "hipMalloc failed (injected fault)");
  bytes = std::max<size_t>(bytes, 256);
  hipError_t e = hipMalloc((void**)p, bytes);
  if (e != hipSuccess) {
    *p = nullptr;
    (void)hipGetLastError();
    return fail(STRATA_E_NOMEM, std::string("hipMalloc(") + std::to_string(bytes) + "): " + hipGetErrorString(e));
  }
  return STRATA_OK;
}

template <class T>
static strata_status host_alloc(T** p, size_t bytes) {
  if (fault("hostalloc")) return fail(STRATA_E_NOMEM, "hipHostMalloc failed (injected fault)");
  hipError_t e = hipHostMalloc((void**)p, std::max<size_t>(bytes, 64), hipHostMallocDefault);
  if (e != hipSuccess) {
    *p = nullptr;
    (void)hipGetLastError();
    return fail(STRATA_E_NOMEM, std::string("hipHostMalloc(") + std::to_string(bytes) + "): " + hipGetErrorString(e));
  }
  return STRATA_OK;
}

static int prefill_ksplit(int K, int sshift);

// Lays out the workspace of layer h for T tokens at `base` (nullptr: only
// sizes it); every buffer starts on a 256-byte boundary.  Returns the bytes.
static uint64_t carve(const strata_moe* h, size_t T, uint8_t* base, Workspace* ws) {
  const size_t TK = T * h->k;
  ws->max_rows = TK + (h->S ? T : 0);
  // prefill tiles, or decode tiles of at most 4 rows (each expert's count
  // rounded up to 4: at most one more tile per expert than TK / 4)
  ws->max_tiles = TK / kPrefillTM + std::min<size_t>(h->E, TK) + (T + kPrefillTM - 1) / kPrefillTM + 4 +
                  std::min<size_t>(T, kDecodeMaxT) * h->k / 4 + 2;
  uint64_t at = 0;
  auto take = [&](auto*& p, size_t bytes) {
    using P = std::remove_reference_t<decltype(p)>;
    p = base ? reinterpret_cast<P>(base + at) : nullptr;
    at += (std::max<size_t>(bytes, 1) + 255) & ~size_t(255);
  };
  take(ws->logits, T * h->E * 4);
  take(ws->idx, TK * 4);
  take(ws->w, TK * 4);
  take(ws->counts, size_t(h->E) * 4);
  take(ws->offsets, size_t(h->E + 1) * 4);
  take(ws->perm, ws->max_rows * 4);
  take(ws->pos, TK * 4);
  take(ws->rank, TK * 4);
  take(ws->hist, ((T + 63) / 64) * size_t(h->E) * 4);
  take(ws->tiles_dev, ws->max_tiles * sizeof(Tile));
  take(ws->tiles_host, ws->max_tiles * sizeof(Tile));
  take(ws->ntiles, 4);
  take(ws->hbuf, ws->max_rows * h->F * 2);
  take(ws->o, ws->max_rows * h->H * 4 * h->ksplit);
  if (h->f16) {
    take(ws->x16, T * h->H * 2);
    take(ws->xexp, T * 4);
  } else {
    ws->x16 = nullptr;
    ws->xexp = nullptr;
  }
  if (h->gated)
    take(ws->gate, T * 4);
  else
    ws->gate = nullptr;
  return at;
}

static strata_status create_impl(const strata_moe_desc* d, strata_moe* h) {
  h->H = d->hidden;
  h->F = d->ffn;
  h->E = d->num_experts;
  h->k = d->top_k;
  h->S = d->num_shared;
  FormatInfo fi;
  (void)format_of(d->quant, fi);  // validated
  h->quant = fi.kq;
  h->sshift = fi.sshift;
  h->ksplit = prefill_ksplit(h->F, h->sshift);
  h->router = d->router == STRATA_R_SOFTMAX_TOPK_RENORM ? R_SOFTMAX : R_SIGMOID;
  h->policy = d->policy;
  h->decay_shift = d->decay_shift;
  h->prefetch = d->prefetch;
  h->budget = d->expert_budget;
  h->max_tokens = d->max_tokens;
  h->lay = RecordLayout::make(h->H, h->F, h->quant, h->sshift);
  h->slot_stride = (size_t(h->lay.bytes) + 255) & ~size_t(255);
  // paging engine: the kernel for records up to 8 MiB, the DMA engines above
  h->pager = d->pager != STRATA_PAGER_AUTO ? d->pager
                                          : (h->slot_stride <= (size_t(8) << 20) ? STRATA_PAGER_KERNEL : STRATA_PAGER_DMA);

  int dev = d->device;
  if (dev < 0) HIP_CHECK(hipGetDevice(&dev));
  h->device = dev;
  HIP_CHECK(hipSetDevice(dev));
  // this device's copy of the static scratch (no-allocation forwards)
  HIP_CHECK(scratch_init(dev));

  // pinned host store, prepacked in parallel over experts
  strata_status st;
  const size_t rec = h->lay.bytes;
  // records sit at the slot stride (256-byte aligned) in the pinned store too,
  // so every page is an aligned copy
  if ((st = host_alloc(&h->host_store, h->slot_stride * h->E))) return st;
  {
    void* dp = nullptr;
    HIP_CHECK(hipHostGetDevicePointer(&dp, h->host_store, 0));
    h->host_dev = static_cast<const uint8_t*>(dp);
  }
  // rescaling exponents of every expert (fp16 formats), then the prepack
  h->wexp.assign(size_t(h->E + 1) * kWexpCount, 0);
  {
    unsigned nth = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    std::vector<std::thread> th;
    for (unsigned t = 0; t < nth; ++t)
      th.emplace_back([&, t]() {
        for (int e = t; e < h->E; e += nth) {
          int32_t* we = h->wexp.data() + size_t(e) * kWexpCount;
          expert_exponents(d->gate, d->up, d->down, e, h->H, h->F, fi, we);
          pack_expert(h->host_store + h->slot_stride * e, h->lay, d->gate, d->up, d->down, e, h->H, h->F, fi, we);
        }
      });
    for (auto& t : th) t.join();
  }
  if (h->S) expert_exponents(d->sh_gate, d->sh_up, d->sh_down, 0, h->H, h->F, fi, h->wexp.data() + size_t(h->E) * kWexpCount);

  // device: slot pool, shared expert, router, slot pointer table
  if ((st = dev_alloc(&h->d_pool, h->slot_stride * h->budget))) return st;
  if (h->S) {
    if ((st = dev_alloc(&h->d_shared, h->slot_stride))) return st;
    std::vector<uint8_t> tmp(rec);
    pack_expert(tmp.data(), h->lay, d->sh_gate, d->sh_up, d->sh_down, 0, h->H, h->F, fi,
                h->wexp.data() + size_t(h->E) * kWexpCount);
    HIP_CHECK(hipMemcpy(h->d_shared, tmp.data(), rec, hipMemcpyHostToDevice));
  }
  // router rows, then the shared-expert gate row of a gated layer
  h->gated = d->shared_gate_w != nullptr;
  if ((st = dev_alloc(&h->d_router_w, size_t(h->E + h->gated) * h->H * 2))) return st;
  HIP_CHECK(hipMemcpy(h->d_router_w, d->router_w, size_t(h->E) * h->H * 2, hipMemcpyHostToDevice));
  if (h->gated)
    HIP_CHECK(hipMemcpy(h->d_router_w + size_t(h->E) * h->H, d->shared_gate_w, size_t(h->H) * 2,
                        hipMemcpyHostToDevice));
  if ((st = dev_alloc(&h->d_wexp, h->wexp.size() * 4))) return st;
  HIP_CHECK(hipMemcpy(h->d_wexp, h->wexp.data(), h->wexp.size() * 4, hipMemcpyHostToDevice));
  if (d->router_bias) {
    if ((st = dev_alloc(&h->d_router_bias, size_t(h->E) * 4))) return st;
    HIP_CHECK(hipMemcpy(h->d_router_bias, d->router_bias, size_t(h->E) * 4, hipMemcpyHostToDevice));
  }
  h->h_slot_ptr.resize(h->budget + 1);
  for (int s = 0; s < h->budget; ++s) h->h_slot_ptr[s] = h->d_pool + h->slot_stride * s;
  h->h_slot_ptr[h->budget] = h->d_shared ? h->d_shared : h->d_pool;
  if ((st = dev_alloc(&h->d_slot_ptr, sizeof(uint8_t*) * (h->budget + 1)))) return st;
  HIP_CHECK(hipMemcpy(h->d_slot_ptr, h->h_slot_ptr.data(), sizeof(uint8_t*) * (h->budget + 1),
                      hipMemcpyHostToDevice));

  // workspace for max_tokens
  h->f16 = fi.f16;
  if ((st = dev_alloc(&h->d_ws, carve(h, h->max_tokens, nullptr, &h->ws)))) return st;
  (void)carve(h, h->max_tokens, h->d_ws, &h->ws);
  if ((st = dev_alloc(&h->d_distinct, 64))) return st;
  HIP_CHECK(hipMemset(h->d_distinct, 0, 64));
  if ((st = host_alloc(&h->h_counts, size_t(h->E) * 4))) return st;
  h->hybrid = d->hybrid != 0;
  h->hybrid_rows = h->hybrid ? d->hybrid_rows : 0;
  if (h->hybrid) {
    const size_t toks = h->hybrid_rows > 0 ? std::max<size_t>(kDecodeMaxT, h->max_tokens) : size_t(kDecodeMaxT);
    const size_t rows = std::max(size_t(kDecodeMaxT) * h->k,
                                 std::min(toks * h->k, size_t(h->E) * size_t(h->hybrid_rows)));
    if ((st = host_alloc(&h->h_perm, toks * h->k * 4)) || (st = host_alloc(&h->h_x, toks * h->H * 2)) ||
        (st = host_alloc(&h->h_o, rows * h->H * 4)))
      return st;
    HIP_CHECK(hipEventCreateWithFlags(&h->ev_hx, hipEventDisableTiming));
    h->h_xf.resize(rows * h->H);
    h->h_hbuf.resize(rows * h->F);
    int nth = d->host_threads;
    if (nth <= 0) {
      cpu_set_t set;
      nth = sched_getaffinity(0, sizeof set, &set) == 0 ? CPU_COUNT(&set) : 1;
    }
    h->pool = new HostPool(std::max(1, std::min(nth, 256)));
  }
  if ((st = host_alloc(&h->h_tiles, h->ws.max_tiles * sizeof(Tile)))) return st;

  // copy streams: on a budgeted layer with enough CUs, masked to kPageCUs
  // CUs with the paged compute stream on the rest; plain streams otherwise
  // (also if the runtime refuses the masks)
  {
    int ncu = 0;
    HIP_CHECK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, h->device));
    bool split = h->budget < h->E && ncu >= 8 * kPageCUs;
    if (split) {
      std::vector<uint32_t> mc((ncu + 31) / 32, 0u), mp((ncu + 31) / 32, 0u);
      for (int i = 0; i < ncu; ++i) (i < kPageCUs ? mc : mp)[i / 32] |= 1u << (i % 32);
      for (auto& cs : h->copy_streams)
        if (split && hipExtStreamCreateWithCUMask(&cs, (uint32_t)mc.size(), mc.data()) != hipSuccess) split = false;
      if (split && hipExtStreamCreateWithCUMask(&h->pstream, (uint32_t)mp.size(), mp.data()) != hipSuccess)
        split = false;
      if (!split) {
        (void)hipGetLastError();
        for (auto& cs : h->copy_streams)
          if (cs) {
            (void)hipStreamDestroy(cs);
            cs = nullptr;
          }
        if (h->pstream) (void)hipStreamDestroy(h->pstream);
        h->pstream = nullptr;
      }
    }
    if (split) {
      HIP_CHECK(hipEventCreateWithFlags(&h->ev_pfork, hipEventDisableTiming));
      HIP_CHECK(hipEventCreateWithFlags(&h->ev_pjoin, hipEventDisableTiming));
    } else {
      for (auto& cs : h->copy_streams) HIP_CHECK(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
    }
  }
  HIP_CHECK(hipEventCreateWithFlags(&h->ev_fwd_done, hipEventDisableTiming));
  HIP_CHECK(hipEventCreateWithFlags(&h->ev_counts, hipEventDisableTiming));
  for (auto& e : h->ev_ahead) HIP_CHECK(hipEventCreateWithFlags(&e, hipEventDisableTiming));

  // preload: experts 0..budget-1 in slots 0..budget-1, or the profile's
  // hottest experts
  h->rm.init(h->E, h->budget, rm_policy(h->policy), d->decay_shift, d->prefetch, rec);
  if (d->expert_profile) {
    std::vector<PlanEntry> pages;
    h->rm.load_profile(d->expert_profile, false, pages);
  }
  for (int s = 0; s < h->budget; ++s)
    HIP_CHECK(hipMemcpy(h->h_slot_ptr[s], h->host_store + h->slot_stride * h->rm.expert_in(s), rec,
                        hipMemcpyHostToDevice));
  HIP_CHECK(hipDeviceSynchronize());
  return STRATA_OK;
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
static hipEvent_t pool_event(strata_moe* h) {
  if (!h->ev_pool.empty()) {
    hipEvent_t e = h->ev_pool.back();
    h->ev_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Times one step of a forward.  Single-kernel steps get the events attached to
// the kernel's own dispatch (its start and end); the routing group, several
// kernels, is bracketed by events recorded on the stream around it.
template <class Fn>
static hipError_t timed(strata_moe* h, int cls, hipStream_t s, Fn&& fn) {
  if (!h->timing) return fn();
  hipEvent_t a = pool_event(h), b = pool_event(h);
  if (!a || !b) return hipErrorOutOfMemory;
  hipError_t e;
  if (cls == STRATA_K_GROUP) {
    e = hipEventRecord(a, s);
    if (e != hipSuccess) return e;
    e = fn();
    if (e != hipSuccess) return e;
    e = hipEventRecord(b, s);
  } else {
    strata::g_ktimer = {a, b, false};
    e = fn();
    const bool used = strata::g_ktimer.used;
    strata::g_ktimer = {};
    if (!used) {  // nothing was launched (empty range): no record
      h->ev_pool.push_back(a);
      h->ev_pool.push_back(b);
      return e;
    }
  }
  h->trecs.push_back({cls, a, b});
  return e;
}

static GemmArgs gemm_args(strata_moe* h, const Workspace& ws, bool gate_up, const void* x, const Tile* tiles,
                          const int32_t* n_dev, int n_tiles) {
  GemmArgs a;
  a.act = gate_up ? (ws.x16 ? (const void*)ws.x16 : x) : ws.hbuf;
  a.gather = gate_up ? ws.perm : nullptr;
  a.tiles = tiles;
  a.n_tiles_dev = n_dev;
  a.n_tiles = n_tiles;
  a.slot_ptr = h->d_slot_ptr;
  a.off_codes = gate_up ? h->lay.w1_codes : h->lay.w2_codes;
  a.off_scales = gate_up ? h->lay.w1_scales : h->lay.w2_scales;
  a.N = gate_up ? 2 * h->F : h->H;
  a.K = gate_up ? h->H : h->F;
  a.out = gate_up ? ws.hbuf : (void*)ws.o;
  a.out_ld = gate_up ? h->F : h->H;
  a.sshift = h->sshift;
  a.off_gscale = h->quant == Q_NVFP4 ? h->lay.gscale + (gate_up ? 0 : 8) : -1;
  a.ksplit = 1;
  a.split_stride = 0;
  a.tok_of_row = ws.perm;
  a.xexp = ws.xexp;
  a.wexp = h->d_wexp;
  return a;
}

// Prefill down GEMMs with a long reduction (K = F of many k-blocks) split K
// into equal ranges, each its own work item writing a partial-sum plane; the
// combine adds the planes in order.  Long-K experts then give the GPU
// several times more work items (a handful of experts with F = 14336 would
// otherwise leave most CUs idle).  Depends on the layer shape only, so every
// forward of a layer (paged or not) sums in the same order.
static int prefill_ksplit(int K, int sshift) {
  const int KB = K >> 6;
  for (int s : {4, 2})
    if (KB >= 48 * s && KB % (s << sshift) == 0) return s;
  return 1;
}

// Persistent prefill grid: at most two workgroups per CU; a multiple of 8
// (the XCD count) above 8, so the kernel can give each XCD its own runs of
// items.
static int prefill_grid(int items) {
  int g = std::max(1, std::min(items, 512));
  return g > 8 ? (g & ~7) : g;
}

// Runs gate+up then down over a tile range.  n_dev != nullptr: the count lives
// on the device and `n_tiles` is only an upper bound.
static hipError_t run_experts(strata_moe* h, const Workspace& ws, const void* x, const Tile* tiles,
                              const int32_t* n_dev, int n_tiles, bool decode, int T, hipStream_t s) {
  if (n_tiles <= 0) return hipSuccess;
  for (int pass = 0; pass < 2; ++pass) {
    const bool gate_up = pass == 0;
    GemmArgs a = gemm_args(h, ws, gate_up, x, tiles, n_dev, n_tiles);
    const int nrt = a.N / 32;
    int grid;
    int log2S = 0;
    const int dot_s = decode ? decode_dot_waves(a.N, a.K, h->quant, h->k + h->S, T) : 0;
    if (dot_s > 0) {
      const int cls = gate_up ? STRATA_K_DEC_UP : STRATA_K_DEC_DOWN;
      hipError_t e = timed(h, cls, s, [&]() { return launch_decode_dot(a, h->quant, gate_up, T, dot_s, n_tiles, s); });
      if (e != hipSuccess) return e;
      continue;
    }
    if (decode) {
      log2S = decode_log2_splits(a.N, a.K, h->k + h->S, T);
      grid = decode_grid(a.N, log2S, n_tiles);
    } else {
      if (!gate_up) {
        a.ksplit = h->ksplit;
        a.split_stride = int64_t(ws.max_rows) * h->H;
      }
      grid = prefill_grid(n_tiles * ((nrt + 7) / 8) * a.ksplit);
    }
    const int cls = decode ? (gate_up ? STRATA_K_DEC_UP : STRATA_K_DEC_DOWN)
                           : (gate_up ? STRATA_K_PRE_UP : STRATA_K_PRE_DOWN);
    hipError_t e = timed(h, cls, s, [&]() { return launch_expert_gemm(a, h->quant, gate_up, decode, T, log2S, grid, s); });
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

static void add_tiles(strata_moe* h, int expert, int slot, int row_begin, int count, int tile_rows,
                      int& n) {
  const int tr = std::min(tile_rows, std::max(count, 1));
  const int first = n, nt = (count + tr - 1) / tr;
  for (int r = 0; r < count; r += tr) {
    Tile t;
    t.expert = expert;
    t.slot = slot;
    t.row_begin = row_begin + r;
    t.nrows = std::min(tr, count - r);
    t.group_first = first;
    t.group_count = nt;
    h->h_tiles[n++] = t;
  }
}

// Waits for `ev` on the host: polls for up to about 2 ms (the token counts
// usually arrive within tens of microseconds, and a blocking wait adds its
// own wake-up latency to every paged forward), then blocks.
static hipError_t wait_spin(hipEvent_t ev) {
  const auto t0 = std::chrono::steady_clock::now();
  for (;;) {
    const hipError_t e = hipEventQuery(ev);
    if (e != hipErrorNotReady) return e;
    if (std::chrono::steady_clock::now() - t0 > std::chrono::microseconds(2000)) return hipEventSynchronize(ev);
  }
}

// Copies `pages` from the pinned store into their slots on the copy streams
// (round-robin), after `after` (the compute that last read those slots), and
// marks them pending for the next forward.
static hipError_t page_ahead(strata_moe* h, const std::vector<PlanEntry>& pages, hipEvent_t after) {
  const size_t rec = h->lay.bytes;
  bool waited[kCopyStreams] = {};
  int c = 0;
  for (const PlanEntry& p : pages) {
    hipStream_t cs = h->copy_streams[c];
    if (!waited[c]) {
      waited[c] = true;
      hipError_t e = after ? hipStreamWaitEvent(cs, after, 0) : hipSuccess;
      // an earlier batch of pages on another stream may target the same slot
      for (int i = 0; i < kCopyStreams && e == hipSuccess; ++i)
        if (i != c && h->ahead_used[i]) e = hipStreamWaitEvent(cs, h->ev_ahead[i], 0);
      if (e != hipSuccess) return e;
    }
    hipError_t e = hipMemcpyAsync(h->h_slot_ptr[p.slot], h->host_store + h->slot_stride * p.expert, rec,
                                  hipMemcpyHostToDevice, cs);
    if (e != hipSuccess) return e;
    c = (c + 1) % kCopyStreams;
  }
  for (int i = 0; i < kCopyStreams; ++i) {
    if (!waited[i]) continue;
    hipError_t e = hipEventRecord(h->ev_ahead[i], h->copy_streams[i]);
    if (e != hipSuccess) return e;
    h->ahead_used[i] = true;
  }
  h->ahead_pending = true;
  return hipSuccess;
}

// Waits, on the compute stream and on every copy stream, for the pages made
// ahead of this forward (prefetch, profile loads).
static hipError_t wait_ahead(strata_moe* h, hipStream_t s) {
  if (!h->ahead_pending) return hipSuccess;
  for (int i = 0; i < kCopyStreams; ++i) {
    if (!h->ahead_used[i]) continue;
    hipError_t e = hipStreamWaitEvent(s, h->ev_ahead[i], 0);
    for (int c = 0; c < kCopyStreams && e == hipSuccess; ++c)
      if (c != i) e = hipStreamWaitEvent(h->copy_streams[c], h->ev_ahead[i], 0);
    if (e != hipSuccess) return e;
    h->ahead_used[i] = false;
  }
  h->ahead_pending = false;
  return hipSuccess;
}

// Computes the experts `host` on the host threads for their tokens (rows
// off[e] .. off[e] + count of the grouping; token ids in h_perm, bf16 rows in
// h_x, both on the host already) and copies their output rows into o on
// stream s: plane 0 gets the rows, planes 1 .. planes-1 (a K-split down GEMM's
// partial sums) get zeros, so the combine's plane sum is the host result.
static strata_status host_experts_to_o(strata_moe* h, const Workspace& ws, const std::vector<int32_t>& host,
                                       const std::vector<int32_t>& off, int planes, hipStream_t s) {
  std::vector<HostJob> jobs;
  int row = 0;
  for (int32_t e : host) {
    const int c = h->h_counts[e];
    for (int i = 0; i < c; ++i) {
      const int t = h->h_perm[off[e] + i];
      const uint16_t* src = h->h_x + size_t(t) * h->H;
      float* dst = h->h_xf.data() + size_t(row + i) * h->H;
      for (int k = 0; k < h->H; ++k) {
        const uint32_t u = uint32_t(src[k]) << 16;
        memcpy(&dst[k], &u, 4);
      }
    }
    jobs.push_back({h->host_store + h->slot_stride * e, h->wexp.data() + size_t(e) * kWexpCount, c,
                    h->h_xf.data() + size_t(row) * h->H, h->h_o + size_t(row) * h->H});
    row += c;
  }
  const auto t0 = std::chrono::steady_clock::now();
  host_experts_run(*h->pool, jobs, h->H, h->F, h->quant, h->sshift, h->lay, h->h_hbuf.data());
  h->host_ns +=
      (uint64_t)std::chrono::duration_cast<std::chrono::nanoseconds>(std::chrono::steady_clock::now() - t0).count();
  row = 0;
  const int64_t plane = int64_t(ws.max_rows) * h->H;
  for (int32_t e : host) {
    const int c = h->h_counts[e];
    HIP_CHECK(hipMemcpyAsync(ws.o + size_t(off[e]) * h->H, h->h_o + size_t(row) * h->H, size_t(c) * h->H * 4,
                             hipMemcpyHostToDevice, s));
    for (int p = 1; p < planes; ++p)
      HIP_CHECK(hipMemsetAsync(ws.o + p * plane + size_t(off[e]) * h->H, 0, size_t(c) * h->H * 4, s));
    row += c;
  }
  return STRATA_OK;
}

// Decode forward of a hybrid layer, after routing: the resident experts run
// on the GPU while the host threads compute the others from the pinned store;
// their output rows are then copied into o for the combine.  The tokens,
// their grouping and the counts reach the host with one wait.
static strata_status forward_hybrid(strata_moe* h, const Workspace& ws, const void* x, int T, hipStream_t s) {
  const int TK = T * h->k;
  HIP_CHECK(hipMemcpyAsync(h->h_counts, ws.counts, size_t(h->E) * 4, hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipMemcpyAsync(h->h_perm, ws.perm, size_t(TK) * 4, hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipMemcpyAsync(h->h_x, x, size_t(T) * h->H * 2, hipMemcpyDeviceToHost, s));
  HIP_CHECK(hipEventRecord(h->ev_counts, s));
  HIP_CHECK(wait_spin(h->ev_counts));
  std::vector<int32_t> needed, off(h->E + 1, 0);
  for (int e = 0; e < h->E; ++e) {
    off[e + 1] = off[e] + h->h_counts[e];
    if (h->h_counts[e] > 0) needed.push_back(e);
  }
  if (off[h->E] != TK) return fail(STRATA_E_HIP, "token counts do not add up to T*k");
  std::vector<PlanEntry> hits, ahead;
  std::vector<int32_t> host;
  h->rm.forward_hybrid(needed, hits, host, ahead);
  // GPU: the hits and the shared expert, one launch set
  int n = 0;
  const int tr = decode_tile_rows(T);
  for (const PlanEntry& p : hits) add_tiles(h, p.expert, p.slot, off[p.expert], h->h_counts[p.expert], tr, n);
  if (h->S) add_tiles(h, h->E, h->budget, TK, T, tr, n);
  if ((size_t)n > ws.max_tiles) return fail(STRATA_E_HIP, "tile list overflow");
  if (n > 0)
    HIP_CHECK(hipMemcpyAsync(ws.tiles_host, h->h_tiles, size_t(n) * sizeof(Tile), hipMemcpyHostToDevice, s));
  if (h->ev_wave_done.empty()) {
    hipEvent_t b;
    HIP_CHECK(hipEventCreateWithFlags(&b, hipEventDisableTiming));
    h->ev_wave_done.push_back(b);
    for (int c = 0; c < kCopyStreams; ++c) {
      hipEvent_t a;
      HIP_CHECK(hipEventCreateWithFlags(&a, hipEventDisableTiming));
      h->ev_copied.push_back(a);
    }
  }
  HIP_CHECK(wait_ahead(h, s));
  HIP_CHECK(run_experts(h, ws, x, ws.tiles_host, nullptr, n, true, T, s));
  HIP_CHECK(hipEventRecord(h->ev_wave_done[0], s));
  // host: the other experts, for their tokens (rows off[e] .. of the grouping)
  if (!host.empty()) {
    strata_status hs = host_experts_to_o(h, ws, host, off, 1, s);
    if (hs) return hs;
  }
  if (!ahead.empty()) HIP_CHECK(page_ahead(h, ahead, h->ev_wave_done[0]));
  return STRATA_OK;
}

static strata_status forward_impl(strata_moe* h, const Workspace& ws, const void* x, int T, void* y,
                                  hipStream_t s, const strata_route_dbg* dbg) {
  const bool decode = T <= kDecodeMaxT;
  const int TK = T * h->k;
  // under stream capture only kernels may be enqueued: an all-resident
  // forward is nothing else (the caller orders replays against other forwards)
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  HIP_CHECK(hipStreamIsCapturing(s, &cap));
  const bool capturing = cap != hipStreamCaptureStatusNone;
  if (capturing && h->budget != h->E)
    return fail(STRATA_E_UNSUPPORTED, "a budgeted forward decides its pages on the host and cannot be captured");
  if (capturing && h->timing) return fail(STRATA_E_UNSUPPORTED, "kernel timing cannot be captured");
  if (h->fwd_recorded && !capturing) HIP_CHECK(hipStreamWaitEvent(s, h->ev_fwd_done, 0));

  const int tile_rows = decode ? decode_tile_rows(T) : kPrefillTM;
  if (route_decode_fits(T, h->E + h->gated)) {
    // router and routing in one launch (its last workgroup routes); the
    // arrival counter is the word after the distinct-expert total
    HIP_CHECK(timed(h, STRATA_K_ROUTER, s, [&]() {
      return launch_route_decode((const uint16_t*)x, h->d_router_w, h->d_router_bias, ws.logits, ws.x16, ws.xexp,
                                 ws.gate, h->E + h->gated, h->H, reinterpret_cast<uint32_t*>(h->d_distinct + 1), T,
                                 h->E, h->k, h->router, h->S, tile_rows, h->budget, ws.idx, ws.w, ws.counts,
                                 ws.offsets, ws.perm, ws.pos, ws.tiles_dev, ws.ntiles, h->d_distinct, s);
    }));
  } else {
    HIP_CHECK(timed(h, STRATA_K_ROUTER, s, [&]() {
      return launch_router((const uint16_t*)x, h->d_router_w, h->d_router_bias, ws.logits, ws.x16, ws.xexp,
                           ws.gate, T, h->E + h->gated, h->E, h->H, s);
    }));
    HIP_CHECK(timed(h, STRATA_K_GROUP, s, [&]() {
      return launch_route(ws.logits, T, h->E, h->k, h->router, h->S, tile_rows, h->budget, ws.idx,
                          ws.w, ws.rank, ws.hist, ws.counts, ws.offsets,
                          ws.perm, ws.pos, ws.tiles_dev, ws.ntiles, h->d_distinct, s);
    }));
  }

  if (h->budget == h->E) {
    const int ub = decode ? (T > 4 ? std::min(h->E, TK) + TK / 4 + h->S * ((T + 3) / 4) : std::min(h->E, TK) + h->S)
                          : TK / kPrefillTM + std::min(h->E, TK) + (h->S ? (T + kPrefillTM - 1) / kPrefillTM : 0);
    HIP_CHECK(run_experts(h, ws, x, ws.tiles_dev, ws.ntiles, ub, decode, T, s));
    h->rm.forwards++;
    h->rm.waves++;
  } else if (h->hybrid && decode) {
    strata_status hs = forward_hybrid(h, ws, x, T, s);
    if (hs) return hs;
  } else {
    // hybrid prefill: the tokens and their grouping follow the counts to the
    // host, for the experts the host will compute
    const bool hprefill = h->hybrid && h->hybrid_rows > 0 && !decode;
    HIP_CHECK(hipMemcpyAsync(h->h_counts, ws.counts, size_t(h->E) * 4, hipMemcpyDeviceToHost, s));
    HIP_CHECK(hipEventRecord(h->ev_counts, s));
    if (hprefill) {
      HIP_CHECK(hipMemcpyAsync(h->h_perm, ws.perm, size_t(TK) * 4, hipMemcpyDeviceToHost, s));
      HIP_CHECK(hipMemcpyAsync(h->h_x, x, size_t(T) * h->H * 2, hipMemcpyDeviceToHost, s));
      HIP_CHECK(hipEventRecord(h->ev_hx, s));
    }
    HIP_CHECK(wait_spin(h->ev_counts));
    std::vector<int32_t> needed;
    std::vector<int32_t> off(h->E + 1, 0);
    for (int e = 0; e < h->E; ++e) {
      off[e + 1] = off[e] + h->h_counts[e];
      if (h->h_counts[e] > 0) needed.push_back(e);
    }
    if (off[h->E] != TK) return fail(STRATA_E_HIP, "token counts do not add up to T*k");
    std::vector<std::vector<PlanEntry>> plan;
    std::vector<PlanEntry> ahead;
    std::vector<int32_t> host;  // hybrid prefill: experts the host computes
    h->rm.forward(needed, plan, ahead, h->h_counts, hprefill ? h->hybrid_rows : 0, hprefill ? &host : nullptr);
    // tile lists: per wave [hits (+ shared in wave 0)] [paged]
    if (plan.empty()) plan.emplace_back();  // every needed expert on the host: the shared expert's wave
    const int nw = (int)plan.size();
    std::vector<int> hb(nw), he(nw), pe(nw);
    int n = 0;
    for (int w = 0; w < nw; ++w) {
      hb[w] = n;
      for (const PlanEntry& p : plan[w])
        if (!p.paged) add_tiles(h, p.expert, p.slot, off[p.expert], h->h_counts[p.expert], tile_rows, n);
      if (w == 0 && h->S) add_tiles(h, h->E, h->budget, TK, T, tile_rows, n);
      he[w] = n;
      for (const PlanEntry& p : plan[w])
        if (p.paged) add_tiles(h, p.expert, p.slot, off[p.expert], h->h_counts[p.expert], tile_rows, n);
      pe[w] = n;
    }
    if ((size_t)n > ws.max_tiles) return fail(STRATA_E_HIP, "tile list overflow");
    // group indices are relative to the first tile of each launch's range;
    // prefill ranges then run heaviest tiles first (more 32-row column tiles
    // first, list order otherwise), as the device-built list does
    for (int w = 0; w < nw; ++w) {
      for (int i = hb[w]; i < he[w]; ++i) h->h_tiles[i].group_first -= hb[w];
      for (int i = he[w]; i < pe[w]; ++i) h->h_tiles[i].group_first -= he[w];
      if (!decode) {
        auto heavier = [](const Tile& a, const Tile& b) { return (a.nrows + 31) / 32 > (b.nrows + 31) / 32; };
        std::stable_sort(h->h_tiles + hb[w], h->h_tiles + he[w], heavier);
        std::stable_sort(h->h_tiles + he[w], h->h_tiles + pe[w], heavier);
      }
    }
    HIP_CHECK(hipMemcpyAsync(ws.tiles_host, h->h_tiles, size_t(n) * sizeof(Tile), hipMemcpyHostToDevice, s));
    while ((int)h->ev_wave_done.size() < nw) {
      hipEvent_t b;
      HIP_CHECK(hipEventCreateWithFlags(&b, hipEventDisableTiming));
      h->ev_wave_done.push_back(b);
      for (int c = 0; c < kCopyStreams; ++c) {
        hipEvent_t a;
        HIP_CHECK(hipEventCreateWithFlags(&a, hipEventDisableTiming));
        h->ev_copied.push_back(a);
      }
    }
    // The expert GEMMs of this forward run on the paged compute stream ps
    // (after the routing on s; the combine on s waits for them below), except
    // in a decode forward, which runs on s itself, its page-in kernels too
    // (inline_pages), in wave order: nothing of it then runs beside a page-in
    // workgroup, the page-in spreads over every CU, and the token's dependent
    // chain has no cross-queue wait (a fork, a join and the waits for the
    // copy streams cost more than the overlap of the pages with the hit
    // experts' compute that a decode forward gives up).  With the DMA-engine
    // pager a decode forward with pages keeps the split.
    int n_pages = 0;
    for (const auto& pw : plan)
      for (const PlanEntry& p : pw) n_pages += p.paged ? 1 : 0;
    const bool inline_pages = decode && h->pager == STRATA_PAGER_KERNEL;
    hipStream_t ps = (h->pstream && !(decode && (n_pages == 0 || inline_pages))) ? h->pstream : s;
    if (ps != s) {
      HIP_CHECK(hipEventRecord(h->ev_pfork, s));
      HIP_CHECK(hipStreamWaitEvent(ps, h->ev_pfork, 0));
    }
    // Pages made ahead of this forward (prefetch, profile load) land before
    // its compute reads the slots and before any copy of it overwrites one.
    HIP_CHECK(wait_ahead(h, ps));
    // A wave's misses go out first the pages that overwrite slots no compute
    // of this forward still reads, then per wave whose compute must finish
    // first (the latest wave of this forward that read a slot being
    // overwritten; never the current or the previous wave: pages overlap a
    // wave's compute).  Page-in kernel: one launch per group of pages that
    // wait for the same wave, groups round-robin over the copy streams, so a
    // group that waits does not hold back the next.  DMA engines: one copy
    // per record, round-robin over the copy streams.
    int rr = 0;  // the round-robin runs on across waves
    for (int w = 0; w < nw; ++w) {
      const bool any_paged = pe[w] > he[w];
      bool used[kCopyStreams] = {};
      if (any_paged) {
        std::vector<const PlanEntry*> pages;
        for (const PlanEntry& p : plan[w])
          if (p.paged) pages.push_back(&p);
        std::stable_sort(pages.begin(), pages.end(),
                         [](const PlanEntry* a, const PlanEntry* b) { return a->after_wave < b->after_wave; });
        if (h->pager == STRATA_PAGER_KERNEL) {
          for (size_t g0 = 0; g0 < pages.size();) {
            size_t g1 = g0;
            while (g1 < pages.size() && pages[g1]->after_wave == pages[g0]->after_wave &&
                   int(g1 - g0) < kPageJobs)
              ++g1;
            if (fault("h2d")) return fail(STRATA_E_HIP, "page-in launch failed (injected fault)");
            // inline: enqueued on s after every earlier wave's compute, so
            // a page needs no event to wait for the wave it follows
            const int c = inline_pages ? 0 : rr++ % kCopyStreams;
            hipStream_t cs = inline_pages ? ps : h->copy_streams[c];
            if (!inline_pages) used[c] = true;
            if (pages[g0]->after_wave >= 0 && !inline_pages)
              HIP_CHECK(hipStreamWaitEvent(cs, h->ev_wave_done[pages[g0]->after_wave], 0));
            PageBatch b;
            b.src = h->host_dev;
            b.stride = int64_t(h->slot_stride);
            b.slot_ptr = h->d_slot_ptr;
            b.n = int(g1 - g0);
            for (size_t i = g0; i < g1; ++i) {
              b.expert[i - g0] = pages[i]->expert;
              b.slot[i - g0] = pages[i]->slot;
            }
            HIP_CHECK(launch_page_in(b, cs));
            g0 = g1;
          }
        } else {
          // one copy per record, dealt round-robin over the copy streams (so
          // one record's setup overlaps another's transfer); each stream waits
          // for a wave's compute just before its first page that needs it
          const size_t rec = h->lay.bytes;
          int waited[kCopyStreams];
          std::fill(waited, waited + kCopyStreams, -1);
          for (const PlanEntry* p : pages) {
            if (fault("h2d")) return fail(STRATA_E_HIP, "hipMemcpyAsync H2D failed (injected fault)");
            const int c = rr++ % kCopyStreams;
            used[c] = true;
            if (p->after_wave > waited[c]) {
              HIP_CHECK(hipStreamWaitEvent(h->copy_streams[c], h->ev_wave_done[p->after_wave], 0));
              waited[c] = p->after_wave;
            }
            HIP_CHECK(hipMemcpyAsync(h->h_slot_ptr[p->slot], h->host_store + h->slot_stride * p->expert, rec,
                                     hipMemcpyHostToDevice, h->copy_streams[c]));
          }
        }
        for (int i = 0; i < kCopyStreams; ++i)
          if (used[i]) HIP_CHECK(hipEventRecord(h->ev_copied[w * kCopyStreams + i], h->copy_streams[i]));
      }
      HIP_CHECK(run_experts(h, ws, x, ws.tiles_host + hb[w], nullptr, he[w] - hb[w], decode, T, ps));
      if (any_paged) {
        for (int i = 0; i < kCopyStreams; ++i)
          if (used[i]) HIP_CHECK(hipStreamWaitEvent(ps, h->ev_copied[w * kCopyStreams + i], 0));
        HIP_CHECK(run_experts(h, ws, x, ws.tiles_host + he[w], nullptr, pe[w] - he[w], decode, T, ps));
      }
      HIP_CHECK(hipEventRecord(h->ev_wave_done[w], ps));
    }
    // the policy's pages ahead of need, once this forward's experts are done
    if (!ahead.empty()) HIP_CHECK(page_ahead(h, ahead, h->ev_wave_done[nw - 1]));
    if (ps != s) {
      HIP_CHECK(hipEventRecord(h->ev_pjoin, ps));
      HIP_CHECK(hipStreamWaitEvent(s, h->ev_pjoin, 0));
    }
    // hybrid prefill: the host computes its experts while the GPU runs the
    // waves enqueued above; their rows reach o before the combine
    if (!host.empty()) {
      HIP_CHECK(wait_spin(h->ev_hx));
      strata_status hs = host_experts_to_o(h, ws, host, off, h->ksplit, s);
      if (hs) return hs;
    }
  }

  HIP_CHECK(timed(h, STRATA_K_COMBINE, s, [&]() {
    return launch_combine(ws.o, ws.pos, ws.w, T, h->k, h->H, h->S ? TK : -1, decode ? 1 : h->ksplit,
                          int64_t(ws.max_rows) * h->H, ws.gate, (uint16_t*)y, s);
  }));

  if (dbg) {
    auto cp = [&](void* dst, const void* src, size_t bytes) -> hipError_t {
      return dst ? hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s) : hipSuccess;
    };
    HIP_CHECK(cp(dbg->logits, ws.logits, size_t(T) * h->E * 4));
    HIP_CHECK(cp(dbg->topk_idx, ws.idx, size_t(TK) * 4));
    HIP_CHECK(cp(dbg->topk_w, ws.w, size_t(TK) * 4));
    HIP_CHECK(cp(dbg->counts, ws.counts, size_t(h->E) * 4));
    HIP_CHECK(cp(dbg->offsets, ws.offsets, size_t(h->E + 1) * 4));
    HIP_CHECK(cp(dbg->perm, ws.perm, size_t(TK) * 4));
  }
  if (!capturing) {
    HIP_CHECK(hipEventRecord(h->ev_fwd_done, s));
    h->fwd_recorded = true;
  }
  if (getenv("STRATA_LOG")) {
    fprintf(stderr, "[strata] T=%d forwards=%llu hits=%llu misses=%llu waves=%llu bytes_h2d=%llu\n", T,
            (unsigned long long)h->rm.forwards, (unsigned long long)h->rm.hits,
            (unsigned long long)h->rm.misses, (unsigned long long)h->rm.waves,
            (unsigned long long)h->rm.bytes_h2d);
  }
  return STRATA_OK;
}

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

strata_status strata_moe_create(const strata_moe_desc* desc, strata_moe** out) {
  if (!out) return fail(STRATA_E_INVALID, "out is NULL");
  *out = nullptr;
  strata_status st = validate(desc);
  if (st) return st;
  strata_moe* h = new strata_moe();
  h->device = -1;
  st = create_impl(desc, h);
  if (st) {
    std::string msg = g_err;
    release(h);
    g_err = msg;
    return st;
  }
  g_err.clear();
  *out = h;
  return STRATA_OK;
}

strata_status strata_moe_forward(strata_moe* h, const void* x, int32_t T, void* y, void* stream,
                                 const strata_route_dbg* dbg) {
  if (!h) return fail(STRATA_E_INVALID, "handle is NULL");
  if (h->poisoned) return fail(STRATA_E_POISONED, "handle poisoned by an earlier HIP failure");
  if (T < 0 || T > h->max_tokens) return fail(STRATA_E_INVALID, "T out of range [0, max_tokens]");
  if (T == 0) return STRATA_OK;
  if (!x || !y) return fail(STRATA_E_INVALID, "x or y is NULL");
  const uintptr_t xa = (uintptr_t)x, ya = (uintptr_t)y, nb = (uintptr_t)T * h->H * 2;
  if (xa < ya + nb && ya < xa + nb) return fail(STRATA_E_INVALID, "x and y overlap");
  if ((xa | ya) & 15) return fail(STRATA_E_INVALID, "x and y must be 16-byte aligned");
  int cur = -1;
  if (hipGetDevice(&cur) == hipSuccess && cur != h->device) (void)hipSetDevice(h->device);
  strata_status st = forward_impl(h, h->ws, x, T, y, (hipStream_t)stream, dbg);
  if (cur >= 0 && cur != h->device) (void)hipSetDevice(cur);
  if (st == STRATA_E_HIP) h->poisoned = true;
  return st;
}

strata_status strata_moe_forward_noalloc(strata_moe* h, const void* x, int32_t T, void* y, void* stream,
                                         const strata_route_dbg* dbg) {
  if (!h) return fail(STRATA_E_INVALID, "handle is NULL");
  if (h->poisoned) return fail(STRATA_E_POISONED, "handle poisoned by an earlier HIP failure");
  if (T < 0 || T > h->max_tokens) return fail(STRATA_E_INVALID, "T out of range [0, max_tokens]");
  if (h->budget != h->E)
    return fail(STRATA_E_UNSUPPORTED, "no-allocation forwards need every expert resident (budget == E): "
                                      "a budgeted forward plans its pages in host memory it allocates");
  if (h->timing) return fail(STRATA_E_UNSUPPORTED, "kernel timing creates events; turn it off");
  if (T == 0) return STRATA_OK;
  if (!x || !y) return fail(STRATA_E_INVALID, "x or y is NULL");
  const uintptr_t xa = (uintptr_t)x, ya = (uintptr_t)y, nb = (uintptr_t)T * h->H * 2;
  if (xa < ya + nb && ya < xa + nb) return fail(STRATA_E_INVALID, "x and y overlap");
  if ((xa | ya) & 15) return fail(STRATA_E_INVALID, "x and y must be 16-byte aligned");
  Workspace ws;
  const uint64_t need = carve(h, T, nullptr, &ws);
  if (need > scratch_bytes()) {
    int lo = 0, hi = T;  // largest T whose workspace fits
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      Workspace tmp;
      if (carve(h, mid, nullptr, &tmp) <= scratch_bytes()) lo = mid; else hi = mid - 1;
    }
    return fail(STRATA_E_INVALID, "T = " + std::to_string(T) + " needs " + std::to_string(need) +
                                      " bytes of workspace; the static scratch holds " +
                                      std::to_string(scratch_bytes()) + " (at most " + std::to_string(lo) +
                                      " tokens of this layer)");
  }
  void* base = scratch_ptr(h->device);  // looked up at create, never the array's host stand-in
  if (!base) return fail(STRATA_E_HIP, "static scratch was not set up on this device");
  (void)carve(h, T, static_cast<uint8_t*>(base), &ws);
  int cur = -1;
  if (hipGetDevice(&cur) == hipSuccess && cur != h->device) (void)hipSetDevice(h->device);
  strata_status st = forward_impl(h, ws, x, T, y, (hipStream_t)stream, dbg);
  if (cur >= 0 && cur != h->device) (void)hipSetDevice(cur);
  if (st == STRATA_E_HIP) h->poisoned = true;
  return st;
}

strata_status strata_expert_cache_stats(const strata_moe* h, strata_cache_stats* out) {
  if (!h || !out) return fail(STRATA_E_INVALID, "NULL argument");
  memset(out, 0, sizeof(*out));
  out->forwards = h->rm.forwards;
  out->hits = h->rm.hits;
  out->misses = h->rm.misses;
  out->evictions = h->rm.evictions;
  out->bytes_h2d = h->rm.bytes_h2d;
  out->waves = h->rm.waves;
  if (h->budget == h->E && h->rm.forwards > 0) {
    unsigned long long d = 0;
    HIP_CHECK(hipSetDevice(h->device));
    HIP_CHECK(hipDeviceSynchronize());
    HIP_CHECK(hipMemcpy(&d, h->d_distinct, 8, hipMemcpyDeviceToHost));
    out->hits = d;
  }
  out->budget = h->budget;
  out->resident = h->rm.resident();
  out->policy = h->policy;
  out->decay_shift = h->decay_shift;
  out->expert_bytes = h->lay.bytes;
  out->resident_bytes = uint64_t(out->resident) * h->lay.bytes;
  out->prefetched = h->rm.prefetched;
  out->prefetch_hits = h->rm.prefetch_hits;
  out->prefetch = h->prefetch;
  out->pager = h->pager;
  out->host_experts = h->rm.host_experts;
  out->host_ns = h->host_ns;
  return STRATA_OK;
}

strata_status strata_expert_profile_save(const strata_moe* h, uint64_t* scores, int32_t num_experts) {
  if (!h || !scores) return fail(STRATA_E_INVALID, "NULL argument");
  if (num_experts != h->E) return fail(STRATA_E_INVALID, "num_experts does not match the layer");
  const std::vector<uint64_t>& sc = h->rm.scores();
  std::copy(sc.begin(), sc.end(), scores);
  return STRATA_OK;
}

strata_status strata_expert_profile_load(strata_moe* h, const uint64_t* scores, int32_t num_experts) {
  if (!h || !scores) return fail(STRATA_E_INVALID, "NULL argument");
  if (h->poisoned) return fail(STRATA_E_POISONED, "handle poisoned by an earlier HIP failure");
  if (num_experts != h->E) return fail(STRATA_E_INVALID, "num_experts does not match the layer");
  for (int e = 0; e < h->E; ++e)
    if (scores[e] > ResidencyManager::kMaxScore) return fail(STRATA_E_INVALID, "profile score above 2^62");
  hipError_t err = hipSetDevice(h->device);
  std::vector<PlanEntry> pages;
  h->rm.load_profile(scores, true, pages);
  if (err == hipSuccess && !pages.empty())
    err = page_ahead(h, pages, h->fwd_recorded ? h->ev_fwd_done : nullptr);
  if (err != hipSuccess) {
    h->poisoned = true;
    return fail(STRATA_E_HIP, std::string("profile load: ") + hipGetErrorString(err));
  }
  return STRATA_OK;
}

strata_status strata_moe_memory(const strata_moe* h, strata_memory_info* out) {
  if (!h || !out) return fail(STRATA_E_INVALID, "NULL argument");
  memset(out, 0, sizeof(*out));
  out->slot_pool = uint64_t(h->slot_stride) * h->budget;
  out->shared = h->S ? h->slot_stride : 0;
  out->router = uint64_t(h->E + h->gated) * h->H * 2 + (h->d_router_bias ? uint64_t(h->E) * 4 : 0) +
                uint64_t(sizeof(uint8_t*)) * (h->budget + 1) + uint64_t(h->wexp.size()) * 4;
  Workspace lay;
  out->workspace = carve(h, h->max_tokens, nullptr, &lay);
  out->device_total = out->slot_pool + out->shared + out->router + out->workspace;
  out->host_store = uint64_t(h->slot_stride) * h->E;
  return STRATA_OK;
}

strata_status strata_moe_set_timing(strata_moe* h, int32_t enable) {
  if (!h) return fail(STRATA_E_INVALID, "handle is NULL");
  h->timing = enable != 0;
  return STRATA_OK;
}

strata_status strata_moe_timing(strata_moe* h, strata_timing* out) {
  if (!h || !out) return fail(STRATA_E_INVALID, "NULL argument");
  HIP_CHECK(hipSetDevice(h->device));
  for (auto& r : h->trecs) {
    HIP_CHECK(hipEventSynchronize(r.b));
    float ms = 0.0f;
    HIP_CHECK(hipEventElapsedTime(&ms, r.a, r.b));
    h->t_ms[r.cls] += ms;
    h->t_launch[r.cls] += 1;
    h->ev_pool.push_back(r.a);
    h->ev_pool.push_back(r.b);
  }
  h->trecs.clear();
  memset(out, 0, sizeof(*out));
  for (int c = 0; c < STRATA_K_COUNT; ++c) {
    out->ms[c] = h->t_ms[c];
    out->launches[c] = h->t_launch[c];
    h->t_ms[c] = 0.0;
    h->t_launch[c] = 0;
  }
  return STRATA_OK;
}

void strata_moe_destroy(strata_moe* h) { release(h); }

const char* strata_last_error(void) { return g_err.c_str(); }

strata_status strata_measure_h2d(int32_t device, uint64_t bytes, int32_t iters, double* gbps) {
  if (!gbps || bytes == 0 || iters < 1) return fail(STRATA_E_INVALID, "bad arguments");
  *gbps = 0.0;
  if (device < 0) HIP_CHECK(hipGetDevice(&device));
  HIP_CHECK(hipSetDevice(device));
  void* hbuf = nullptr;
  void* dbuf = nullptr;
  strata_status st = host_alloc(&hbuf, bytes);
  if (st) return st;
  if (hipMalloc(&dbuf, bytes) != hipSuccess) {
    (void)hipGetLastError();
    (void)hipHostFree(hbuf);
    return fail(STRATA_E_NOMEM, "hipMalloc failed");
  }
  memset(hbuf, 1, bytes);
  hipStream_t s = nullptr;
  hipEvent_t a = nullptr, b = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  if (e == hipSuccess) e = hipMemcpyAsync(dbuf, hbuf, bytes, hipMemcpyHostToDevice, s);  // warm
  if (e == hipSuccess) e = hipEventRecord(a, s);
  for (int i = 0; i < iters && e == hipSuccess; ++i)
    e = hipMemcpyAsync(dbuf, hbuf, bytes, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipEventRecord(b, s);
  if (e == hipSuccess) e = hipEventSynchronize(b);
  float ms = 0.0f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
  if (a) (void)hipEventDestroy(a);
  if (b) (void)hipEventDestroy(b);
  if (s) (void)hipStreamDestroy(s);
  (void)hipFree(dbuf);
  (void)hipHostFree(hbuf);
  if (e != hipSuccess) return fail(STRATA_E_HIP, std::string("h2d probe: ") + hipGetErrorString(e));
  *gbps = double(bytes) * iters / (ms * 1e-3) / 1e9;
  return STRATA_OK;
}

strata_status strata_measure_hbm_read(int32_t device, uint64_t bytes, int32_t iters, double* gbps) {
  if (!gbps || bytes < (uint64_t(64) << 20) || iters < 1) return fail(STRATA_E_INVALID, "bad arguments");
  *gbps = 0.0;
  if (device < 0) HIP_CHECK(hipGetDevice(&device));
  HIP_CHECK(hipSetDevice(device));
  void* dbuf = nullptr;
  const uint64_t flag_off = (bytes + 255) & ~uint64_t(255);
  if (hipMalloc(&dbuf, flag_off + 256) != hipSuccess) {
    (void)hipGetLastError();
    return fail(STRATA_E_NOMEM, "hipMalloc failed");
  }
  uint32_t* flag = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(dbuf) + flag_off);
  hipStream_t s = nullptr;
  hipEvent_t a = nullptr, b = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  if (e == hipSuccess) e = hipMemsetAsync(dbuf, 0x11, flag_off + 256, s);
  if (e == hipSuccess) e = launch_read_probe(dbuf, bytes, flag, s);  // warm-up pass
  float best = 0.0f;
  for (int i = 0; i < iters && e == hipSuccess; ++i) {
    e = hipEventRecord(a, s);
    if (e == hipSuccess) e = launch_read_probe(dbuf, bytes, flag, s);
    if (e == hipSuccess) e = hipEventRecord(b, s);
    if (e == hipSuccess) e = hipEventSynchronize(b);
    float ms = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
    if (e == hipSuccess && (best == 0.0f || ms < best)) best = ms;
  }
  if (a) (void)hipEventDestroy(a);
  if (b) (void)hipEventDestroy(b);
  if (s) (void)hipStreamDestroy(s);
  (void)hipFree(dbuf);
  if (e != hipSuccess) return fail(STRATA_E_HIP, std::string("read probe: ") + hipGetErrorString(e));
  *gbps = double(read_probe_bytes(bytes)) / (best * 1e-3) / 1e9;
  return STRATA_OK;
}

strata_status strata_residency_replay(int32_t num_experts, int32_t budget, int32_t policy,
                                      int32_t decay_shift, int32_t prefetch, const uint64_t* profile,
                                      uint64_t expert_bytes, int32_t n_forwards,
                                      const int32_t* needed_len, const int32_t* needed_flat,
                                      const int32_t* hybrid_flags, const int32_t* needed_rows,
                                      int32_t host_rows, int32_t* plan_slots, uint64_t* scores_out,
                                      strata_cache_stats* out) {
  if (!out || n_forwards < 0 || (n_forwards > 0 && (!needed_len || !needed_flat)))
    return fail(STRATA_E_INVALID, "NULL argument or negative count");
  if (host_rows < 0 || host_rows > kHostMaxRows || (host_rows > 0 && !needed_rows))
    return fail(STRATA_E_INVALID, "host_rows must be in [0, 8], with needed_rows");
  if (num_experts < 1 || num_experts > (1 << 20)) return fail(STRATA_E_INVALID, "num_experts out of range");
  if (strata_status st = check_residency(num_experts, budget, policy, decay_shift, prefetch, profile)) return st;
  ResidencyManager rm;
  rm.init(num_experts, budget, rm_policy(policy), decay_shift, prefetch, expert_bytes);
  std::vector<PlanEntry> ahead;
  if (profile) rm.load_profile(profile, false, ahead);
  size_t pos = 0, out_pos = 0;
  std::vector<std::vector<PlanEntry>> plan;
  std::vector<int32_t> rows(host_rows > 0 ? num_experts : 0), host;
  for (int32_t f = 0; f < n_forwards; ++f) {
    if (needed_len[f] < 0) return fail(STRATA_E_INVALID, "negative needed_len");
    std::vector<int32_t> nd(needed_flat + pos, needed_flat + pos + needed_len[f]);
    for (int32_t e : nd)
      if (e < 0 || e >= num_experts) return fail(STRATA_E_INVALID, "expert id out of range");
    if (host_rows > 0) {  // rows of each needed expert, at its first occurrence
      std::fill(rows.begin(), rows.end(), -1);
      for (int32_t j = 0; j < needed_len[f]; ++j) {
        const int32_t e = needed_flat[pos + j], r = needed_rows[pos + j];
        if (r < 1) return fail(STRATA_E_INVALID, "needed_rows entries must be >= 1");
        if (rows[e] < 0) rows[e] = r;
      }
    }
    pos += needed_len[f];
    std::sort(nd.begin(), nd.end());
    nd.erase(std::unique(nd.begin(), nd.end()), nd.end());
    if (hybrid_flags && hybrid_flags[f]) {
      std::vector<PlanEntry> hit_list;
      std::vector<int32_t> host;
      rm.forward_hybrid(nd, hit_list, host, ahead);
      size_t hi = 0;
      for (int32_t e : nd) {  // ascending: the hit's slot, or -1 for a host expert
        const bool hit = hi < hit_list.size() && hit_list[hi].expert == e;
        if (plan_slots) plan_slots[out_pos] = hit ? hit_list[hi].slot : -1;
        hi += hit;
        ++out_pos;
      }
    } else {
      // a hybrid prefill (host_rows > 0): its run order, then its host
      // experts ascending with slot -1
      rm.forward(nd, plan, ahead, rows.data(), host_rows, host_rows > 0 ? &host : nullptr);
      for (auto& w : plan)
        for (auto& p : w) {
          if (plan_slots) plan_slots[out_pos] = p.slot;
          ++out_pos;
        }
      if (host_rows > 0)
        for (size_t i = 0; i < host.size(); ++i) {
          if (plan_slots) plan_slots[out_pos] = -1;
          ++out_pos;
        }
    }
    // duplicates collapse: keep the output aligned with needed_len
    out_pos += (size_t)needed_len[f] - nd.size();
  }
  memset(out, 0, sizeof(*out));
  out->forwards = rm.forwards;
  out->hits = rm.hits;
  out->misses = rm.misses;
  out->evictions = rm.evictions;
  out->bytes_h2d = rm.bytes_h2d;
  out->waves = rm.waves;
  out->budget = budget;
  out->resident = rm.resident();
  out->policy = policy;
  out->decay_shift = decay_shift;
  out->expert_bytes = expert_bytes;
  out->resident_bytes = uint64_t(rm.resident()) * expert_bytes;
  out->prefetched = rm.prefetched;
  out->prefetch_hits = rm.prefetch_hits;
  out->prefetch = prefetch;
  out->pager = 0;
  out->host_experts = rm.host_experts;
  if (scores_out) std::copy(rm.scores().begin(), rm.scores().end(), scores_out);
  return STRATA_OK;
}

}  // extern "C"
